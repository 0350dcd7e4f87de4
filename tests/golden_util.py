"""Reader for the small text fixtures under tests/golden/ (key = value lines, # comments)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    """Returns {key: [value-strings, ...]} with repeated keys collected in order."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out.setdefault(key, []).append(val)
    return out


def ints(s):
    return [int(x) for x in s.split()]
