"""Benchmark of the MI355X dense GEMM: one step = one C = alpha * A x B through the C ABI.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only NAME]
                [--copy-calib-mib N]
python bench.py --ingest-pmc FETCH_CSV WRITE_CSV --only NAME --command "..."   (CPU only)

Headline: BF16 M = N = K = 4096, uniform[-1, 1] operands resident in HBM, FP32 accumulate, bf16
output, grouped-M (G = 8) tile mapping, persistent scheduler.  The JSON line's "secondary" block
carries the other workloads (FP8 e4m3 8192^3 with per-tensor scales, the 4096 x 14336 x 4096 MLP
shape, the 512 x 512 x 65536 Stream-K case, 256^3) timed the same way.  Progress goes to stderr;
stdout holds exactly one JSON line.

HBM traffic: two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over
`bench.py --only NAME --copy-calib-mib N`, which after the GEMM launches copies N MiB device to
device with the runtime's plain copy kernel.  --ingest-pmc scales each GEMM counter by
known copy bytes / the same counter on that copy, and writes the per-launch figure, keyed by a
hash of the kernel sources, to profiles/hbm_traffic.json.txt; the JSON line's roofline.traffic
uses it only while the sources still match.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "e4m3": 5000.0}   # MI355X dense MFMA, published
HBM_PEAK_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# The device code: the kernels and the scheduler they run.  A counter record stays valid while
# these are unchanged; the planner (gemm.hip) only picks among them.
DEVICE_SOURCES = ("gemm_kernel.h", "sched.h")


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_design_amd", "csrc")
    for name in DEVICE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "hbm_traffic.json.txt")
PEAK_CLOCK_MHZ = 2400.0  # the engine clock the published MFMA peaks assume
# below this mean shader clock the sampled metrics tables were taken while the GPU idled (these
# kernels hold 1.7 - 2.4 GHz; an idle MI355X drops to a few hundred MHz)
BUSY_CLOCK_FLOOR_MHZ = 1000.0


class BoardSampler:
    """Reads the GPU's shader clock (mean over its XCDs), socket power and energy counter through
    the amdsmi library in a background thread.  The board's metrics table behind these values is
    refreshed about once a second (its timestamp and the energy counter step together), so only
    refreshes that happen while the kernel under test runs back to back tell anything: a run
    keeps its kernel busy for over a second after the clock ramp, and stop() uses the tables
    first seen from then on -- the clock as their mean, the power as the energy counter's
    increase between the first and last of them over their timestamps (or the table's own power
    reading when only one refresh fell in the window).  Without amdsmi, or if the GPU cannot be
    matched to torch's device 0 by PCI address, it records nothing (fields None)."""

    def __init__(self, torch):
        self.handle = None
        self.samples = []
        self._stop = None
        try:
            import amdsmi
            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            props = torch.cuda.get_device_properties(0)
            want = (int(props.pci_domain_id), int(props.pci_bus_id), int(props.pci_device_id))
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.handle = h
            if self.handle is None:
                log(f"board sampler: no amdsmi GPU at PCI {want}; clock and power not recorded")
        except Exception as e:  # amdsmi missing or not permitted: measure without it
            log(f"board sampler unavailable ({type(e).__name__}: {e})")

    def read(self):
        """(host time s, table timestamp ns, mean shader clock MHz over the XCDs, socket power
        W, energy J)."""
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        e = self.amdsmi.amdsmi_get_energy_count(self.handle)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and
                0 < c < 10000]
        pw = m.get("current_socket_power")
        return (time.perf_counter(), int(e["timestamp"]),
                sum(clks) / len(clks) if clks else None,
                float(pw) if isinstance(pw, (int, float)) and pw < 100000 else None,
                e["energy_accumulator"] * e["counter_resolution"] * 1e-6)

    def start(self):
        import threading
        self.samples = []
        if self.handle is None:
            return
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    self.samples.append(self.read())
                except Exception:
                    return
                self._stop.wait(0.01)
        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()

    def stop(self, since=0.0):
        """Stops sampling; returns {"clock_mhz", "clock_mhz_min_max", "power_w", "refreshes"}
        from the metrics tables first seen at or after host time `since`."""
        if self._stop is not None:
            self._stop.set()
            self._thread.join()
            self._stop = None
        seen, tables = set(), []
        for t, ts, clk, pw, en in self.samples:
            if ts in seen:
                continue
            seen.add(ts)
            if t >= since:
                tables.append((ts, clk, pw, en))
        clk = [c for _, c, _, _ in tables if c is not None]
        if clk and sum(clk) / len(clk) < BUSY_CLOCK_FLOOR_MHZ:
            # tables refreshed while the GPU idled (as when a tracer holds the launches back and
            # the refreshes miss the busy stretches): they tell nothing about the kernel
            log(f"board sampler: mean clock {sum(clk) / len(clk):.0f} MHz over {len(tables)} "
                f"refreshes is an idle reading; clock and power not recorded")
            return {"clock_mhz": None, "clock_mhz_min_max": None, "power_w": None,
                    "refreshes": len(tables)}
        power = None
        if len(tables) >= 2 and tables[-1][0] > tables[0][0]:
            power = (tables[-1][3] - tables[0][3]) / ((tables[-1][0] - tables[0][0]) * 1e-9)
        elif tables and tables[0][2] is not None:
            power = tables[0][2]
        return {"clock_mhz": round(sum(clk) / len(clk), 1) if clk else None,
                "clock_mhz_min_max": [min(clk), max(clk)] if clk else None,
                "power_w": round(power, 1) if power else None,
                "refreshes": len(tables)}


def _read_counter_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _gemm_and_copy(rows, counter):
    """Per-dispatch counter values (KiB) of the GEMM kernel and of the calibration copies (the
    copy-kernel dispatches after the last GEMM dispatch)."""
    rows = [r for r in rows if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    gemm = [r for r in rows if "gemm_kernel" in r["Kernel_Name"]]
    if not gemm:
        raise SystemExit(f"no gemm_kernel dispatch with {counter}")
    last = max(int(r["Dispatch_Id"]) for r in gemm)
    copy = [r for r in rows if int(r["Dispatch_Id"]) > last and "copyBuffer" in r["Kernel_Name"]]
    if not copy:
        raise SystemExit(f"no calibration copy dispatch with {counter} after the GEMMs")
    return [float(r["Counter_Value"]) for r in gemm], [float(r["Counter_Value"]) for r in copy]


def ingest_pmc(fetch_csv, write_csv, name, command, copy_mib):
    import statistics
    wl = RUNS[name][0]
    fg, fc = _gemm_and_copy(_read_counter_csv(fetch_csv), "FETCH_SIZE")
    wg, wc = _gemm_and_copy(_read_counter_csv(write_csv), "WRITE_SIZE")
    known = copy_mib * 1024.0  # KiB read and KiB written by one copy
    f_factor = known / statistics.median(fc)
    w_factor = known / statistics.median(wc)
    fetch = statistics.median(fg) * 1024.0 * f_factor
    write = statistics.median(wg) * 1024.0 * w_factor
    data = {}
    if os.path.exists(TRAFFIC_PATH):
        with open(TRAFFIC_PATH) as f:
            data = json.loads(f.read().strip().splitlines()[-1])
    data[wl] = {"run": name, "source_hash": source_hash(), "bytes_per_launch": round(fetch + write),
                "fetch_bytes": round(fetch), "write_bytes": round(write),
                "fetch_kib_raw_median": statistics.median(fg),
                "write_kib_raw_median": statistics.median(wg),
                "copy_mib": copy_mib, "copy_fetch_factor": round(f_factor, 5),
                "copy_write_factor": round(w_factor, 5), "gemm_dispatches": len(fg),
                "command": command}
    with open(TRAFFIC_PATH, "w") as f:
        f.write("# HBM bytes per GEMM launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a "
                "plain device copy of known size; written by bench.py --ingest-pmc\n")
        f.write(json.dumps(data, sort_keys=True) + "\n")
    print(json.dumps(data[wl]))


def summarize_trace(path, last):
    """Kernel-trace summary (rocprofv3 --kernel-trace CSV): per GEMM kernel, its resources and the
    duration of its last `last` dispatches (the timed ones), for the profiles/ summaries."""
    import statistics
    rows = _read_counter_csv(path)
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(r)
    for name, rs in sorted(by.items(), key=lambda kv: -len(kv[1])):
        rs.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        tail = d[-last:] if last else d
        r0 = rs[-1]
        print(f"kernel: {name}")
        print(f"  grid {r0.get('Grid_Size', r0.get('Grid_Size_X'))} work-items, workgroup "
              f"{r0.get('Workgroup_Size', r0.get('Workgroup_Size_X'))}, LDS "
              f"{r0.get('LDS_Block_Size')} B, arch VGPR {r0.get('VGPR_Count')}, AGPR "
              f"{r0.get('Accum_VGPR_Count')}, SGPR {r0.get('SGPR_Count')}, scratch "
              f"{r0.get('Scratch_Size')}")
        print(f"  dispatches {len(d)}; over the last {len(tail)}: mean {statistics.mean(tail):.1f} us, "
              f"median {statistics.median(tail):.1f}, min {min(tail):.1f}, max {max(tail):.1f}; "
              f"over all: mean {statistics.mean(d):.1f} us")


def summarize_pmc(path):
    """Counter summary (rocprofv3 --pmc CSV): per counter, the median over the GEMM dispatches
    (summed over the counter's instances within a dispatch), with the dispatch duration."""
    import statistics
    rows = [r for r in _read_counter_csv(path) if "gemm_kernel" in r["Kernel_Name"]]
    per = {}
    dur = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        per.setdefault(d, {}).setdefault(r["Counter_Name"], 0.0)
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    names = sorted({n for v in per.values() for n in v})
    print(f"GEMM dispatches {len(per)}; median duration {statistics.median(dur.values()):.1f} us")
    for n in names:
        print(f"  {n:28s} {statistics.median(v[n] for v in per.values()):.4g}")


def copy_calibration(torch, mib, reps=3):
    """Plain device-to-device copies of `mib` MiB (the runtime's copy kernel), for counter
    calibration."""
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
        torch.cuda.synchronize()
    log(f"copy calibration: {reps} x {mib} MiB device copies")


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources; else None."""
    path = TRAFFIC_PATH
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.loads(f.read().strip().splitlines()[-1])
    except Exception:
        return None
    entry = data.get(workload)
    if not entry or entry.get("source_hash") != source_hash():
        return None
    return entry.get("bytes_per_launch")


# name, workload key, mapping, group, sched, tile, out, workers[, bk[, variant[, epilogue[,
# Stream-K groups]]]]
# variant: "chain" = Stream-K lock-chain fixup; "coop" / "pp" / "wide" = the cooperative /
# ping-pong / wide-wave kernel instead of the default for data-parallel
# 256 x 256 tiles (the wide-wave kernel).  epilogue: the fused operations, {"bias": "row" |
# "col", "act": "relu" | "gelu" | "silu", "amax": True}; out "e4m3" quantises the output.
# Stream-K groups: 0 / 1 = one pool of units over the band, up to 8.
RUNS = {
    "bf16_4096": ("bf16_4096", "grouped_m", 8, "persistent", 0, "bf16", 0),
    "bf16_4096_coop": ("bf16_4096", "grouped_m", 8, "persistent", 256, "bf16", 0, 0, "coop"),
    "bf16_4096_linear": ("bf16_4096", "linear_n", 1, "persistent", 0, "bf16", 0),
    "bf16_4096_t128": ("bf16_4096", "grouped_m", 8, "persistent", 128, "bf16", 0),
    "fp8_8192": ("fp8_8192", "grouped_m", 16, "persistent", 0, "bf16", 0),
    "fp8_8192_coop": ("fp8_8192", "grouped_m", 16, "persistent", 256, "bf16", 0, 0, "coop"),
    "bf16_4096_pp": ("bf16_4096", "grouped_m", 8, "persistent", 256, "bf16", 0, 0, "pp"),
    "fp8_8192_pp": ("fp8_8192", "grouped_m", 16, "persistent", 256, "bf16", 0, 0, "pp"),
    "bf16_mlp_up_pp": ("bf16_mlp_up", "grouped_m", 8, "persistent", 256, "bf16", 0, 0, "pp"),
    "bf16_mlp_up": ("bf16_mlp_up", "grouped_m", 8, "auto", 0, "bf16", 0),
    "bf16_mlp_up_t256": ("bf16_mlp_up", "grouped_m", 8, "persistent", 256, "bf16", 0),
    "bf16_streamk": ("bf16_streamk", "linear_n", 1, "streamk", 128, "f32", 256),
    "bf16_streamk_chain": ("bf16_streamk", "linear_n", 1, "streamk", 128, "f32", 256, 0,
                           "chain"),
    "bf16_256": ("bf16_256", "linear_n", 1, "static", 128, "f32", 0),
    # the other mapping families: 2D blocking (the planner's box: the 32 tiles an XCD runs at a
    # time as a 4 x 8 box) and Morton
    "bf16_4096_blocked": ("bf16_4096", "blocked", 0, "persistent", 0, "bf16", 0),
    "fp8_8192_blocked": ("fp8_8192", "blocked", 0, "persistent", 0, "bf16", 0),
    "bf16_mlp_up_blocked": ("bf16_mlp_up", "blocked", 0, "persistent", 0, "bf16", 0),
    "fp8_8192_morton": ("fp8_8192", "morton", 1, "persistent", 0, "bf16", 0),
    "bf16_mlp_up_morton": ("bf16_mlp_up", "morton", 1, "persistent", 0, "bf16", 0),
    # fused epilogues: the MLP up-projection with its bias and GELU; an FP8 layer whose output
    # is quantised back to e4m3 with amax tracking
    "bf16_mlp_up_bias_gelu": ("bf16_mlp_up", "grouped_m", 8, "auto", 0, "bf16", 0, 0, "",
                              {"bias": "col", "act": "gelu"}),
    # ... and with a bf16 source matrix S added first (Z = Acc + S, then the bias and GELU)
    "bf16_mlp_up_source_bias_gelu": ("bf16_mlp_up", "grouped_m", 8, "auto", 0, "bf16", 0, 0, "",
                                     {"source": "bf16", "beta": 1.0, "bias": "col",
                                      "act": "gelu"}),
    "fp8_8192_e4m3_amax": ("fp8_8192", "grouped_m", 16, "persistent", 0, "e4m3", 0, 0, "",
                           {"amax": True}),
}


def run_flags(name, dg):
    """GEMM_FLAG_* bits of a RUNS entry's variant."""
    variant = RUNS[name][8] if len(RUNS[name]) > 8 else ""
    return {"": 0, "chain": dg.GEMM_FLAG_STREAMK_CHAIN, "pp": dg.GEMM_FLAG_PINGPONG,
            "coop": dg.GEMM_FLAG_COOPERATIVE,
            "wide": dg.GEMM_FLAG_WIDE}[variant]


def workload_operands(wl_name, torch, gi, cache):
    """The workload's operands on the host (gemm_inputs) and resident in HBM, cached by name."""
    if wl_name not in cache:
        import numpy as np
        t0 = time.time()
        op = gi.make_workload(wl_name)
        dev = torch.device("cuda:0")
        if op.dtype == "bf16":
            A = torch.from_numpy(op.A.view(np.int16)).to(dev)
            B = torch.from_numpy(op.B.view(np.int16)).to(dev)
        else:
            A = torch.from_numpy(op.A).to(dev)
            B = torch.from_numpy(op.B).to(dev)
        sa = torch.tensor([op.scale_a], dtype=torch.float32, device=dev)
        sb = torch.tensor([op.scale_b], dtype=torch.float32, device=dev)
        cache[wl_name] = (op, A, B, sa, sb)
        log(f"{wl_name}: inputs generated and resident in HBM ({time.time() - t0:.1f} s)")
    return cache[wl_name]


def setup_run(name, torch, dg, gi, cache):
    """The launch configuration of a RUNS entry, as the benchmark times it and the full-size
    tests check it: the plan, the output and workspace buffers, and the fused epilogue's device
    operands.  Returns a dict; run["launch"](stream) enqueues one GEMM (into run["C"], or into
    the buffer given as out_buf)."""
    wl_name, mapping, group, sched, tile, out, workers = RUNS[name][:7]
    bk = RUNS[name][7] if len(RUNS[name]) > 7 else 0
    epi_spec = RUNS[name][9] if len(RUNS[name]) > 9 else {}
    sk_groups = RUNS[name][10] if len(RUNS[name]) > 10 else 0
    flags = run_flags(name, dg)
    wl = gi.WORKLOADS[wl_name]
    op, A, B, sa, sb = workload_operands(wl_name, torch, gi, cache)
    epi = dg.ACTIVATIONS[epi_spec.get("act")]
    epi |= {None: 0, "row": dg.GEMM_EPI_BIAS_ROW, "col": dg.GEMM_EPI_BIAS_COL}[
        epi_spec.get("bias")]
    epi |= dg.GEMM_EPI_AMAX if epi_spec.get("amax") else 0
    src_kind = epi_spec.get("source")
    epi |= {None: 0, "f32": dg.GEMM_EPI_SOURCE_F32, "bf16": dg.GEMM_EPI_SOURCE_BF16}[src_kind]
    desc = dg.make_desc(op.M, op.N, op.K,
                        dg.GEMM_BF16 if op.dtype == "bf16" else dg.GEMM_FP8_E4M3,
                        dg.OUT_DTYPES[out], dg.MAPPINGS[mapping],
                        group, dg.SCHEDS[sched], workers, tile, tile, bk, flags, epilogue=epi,
                        sk_groups=sk_groups)
    plan = dg.Plan(desc)
    C = torch.empty((op.M, op.N), device=A.device,
                    dtype={"bf16": torch.bfloat16, "f32": torch.float32, "e4m3": torch.uint8}[out])
    ws = None
    if plan.workspace_bytes:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=A.device)
    bias = amax = scale_d = bias_host = None
    epi_bytes = 0  # bytes the epilogue reads besides A and B (bias, source)
    if epi_spec.get("bias"):
        n = op.M if epi_spec["bias"] == "row" else op.N
        bias_host = gi.make_vector(n, seed=wl.seed + 7)
        bias = torch.from_numpy(bias_host).to(A.device)
        epi_bytes = 4 * n
    if epi_spec.get("amax"):
        amax = torch.zeros(1, dtype=torch.float32, device=A.device)
    source = source_host = None
    beta = float(epi_spec.get("beta", 0.0))
    if src_kind:  # a seeded N(0, 1) matrix, held in the source's element type
        v = gi.make_vector(op.M * op.N, seed=wl.seed + 13).reshape(op.M, op.N)
        t = torch.from_numpy(v)
        if src_kind == "bf16":
            t = t.to(torch.bfloat16)
        source = t.to(A.device)
        source_host = t.float().numpy()
        epi_bytes += t.numel() * t.element_size()
    if out == "e4m3":  # the output's dequantisation scale: N(0, 1) operands give |C| up to
        # about 4 sqrt(K), mapped onto the format's 448
        scale_d = torch.tensor([4.0 * op.K ** 0.5 / 448.0], dtype=torch.float32,
                               device=A.device)

    def launch(stream=None, out_buf=None):
        plan.run(A, B, C if out_buf is None else out_buf, sa, sb, ws, stream, bias=bias,
                 scale_d=scale_d, amax=amax, source=source, beta=beta)
    return {"name": name, "workload": wl_name, "op": op, "plan": plan, "C": C, "ws": ws,
            "out": out, "epi": epi_spec, "bias": bias, "bias_host": bias_host, "amax": amax,
            "source_host": source_host, "beta": beta,
            "scale_d": scale_d, "epi_bytes": epi_bytes, "mapping": mapping, "sched": sched,
            "launch": launch}


def time_run(name, steps, warmup, torch, dg, gi, cache, settle_ms=0.0, batches=10, batch=50,
             sampler=None):
    """Times one RUNS entry.  Returns a dict with the contract's wall-clock figures over exactly
    `steps` launches (ms_per_step, tflops) and the kernel time as the median of `batches`
    event-timed batches of `batch` launches (kernel_us, kernel_tflops), with the shader clock
    and socket power sampled during the batches."""
    import statistics
    run = setup_run(name, torch, dg, gi, cache)
    op, plan, out, epi_spec = run["op"], run["plan"], run["out"], run["epi"]
    wl_name, mapping, sched, epi_bytes = run["workload"], run["mapping"], run["sched"], \
        run["epi_bytes"]
    A = cache[wl_name][1]
    stream = torch.cuda.current_stream()

    def launch():
        run["launch"](stream)
    # Warmup: at least `warmup` launches and at least `settle_ms` of back-to-back launches, so the
    # GPU's clock has left its ramp (it climbs for a few hundred ms under a sustained MFMA load).
    if sampler is not None:
        sampler.start()
    n_warm, t_w = 0, time.perf_counter()
    since = t_w + min(0.4 * settle_ms * 1e-3, 0.4)  # past the clock's ramp
    while True:
        for _ in range(max(1, warmup) if n_warm == 0 else 50):
            launch()
            n_warm += 1
        torch.cuda.synchronize()
        if n_warm >= warmup and (time.perf_counter() - t_w) * 1e3 >= settle_ms:
            break
    # The contract's timed region: exactly `steps` launches, synchronised on both sides.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        launch()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The kernel time: `batches` batches of `batch` back-to-back launches, each bracketed by HIP
    # events recorded on the launch stream; the median batch over its launch count.  Clock and
    # power are sampled meanwhile.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(batches)]
    for e0, e1 in ev:
        e0.record(stream)
        for _ in range(batch):
            launch()
        e1.record(stream)
    torch.cuda.synchronize()
    board = sampler.stop(since) if sampler is not None else {
        "clock_mhz": None, "clock_mhz_min_max": None, "power_w": None, "refreshes": 0}
    batch_us = sorted(e0.elapsed_time(e1) * 1e3 / batch for e0, e1 in ev)
    dev_ms = statistics.median(batch_us) * 1e-3
    flops = 2.0 * op.M * op.N * op.K
    info = plan.info
    res = {
        "workload": wl_name, "M": op.M, "N": op.N, "K": op.K, "dtype": op.dtype, "out": out,
        "tile": [info.bm, info.bn, info.bk], "stages": info.stages, "mapping": mapping,
        "kernel": dg.KERNEL_NAMES[info.kernel],
        "group": info.group, "group_n": info.group_n, "sched": sched, "grid": info.grid,
        "sk_groups": info.sk_groups,
        "epilogue": epi_spec,
        "dp_tiles": info.dp_tiles, "sk_tiles": info.sk_tiles, "warmup_launches": n_warm,
        "ms_per_step": wall * 1e3 / steps, "kernel_us": dev_ms * 1e3,
        "tflops": flops / (wall / steps) / 1e12, "kernel_tflops": flops / (dev_ms * 1e-3) / 1e12,
        "batches": batches, "batch": batch,
        "batch_us_min_median_max": [round(batch_us[0], 2), round(dev_ms * 1e3, 2),
                                    round(batch_us[-1], 2)],
        "clock_mhz": board["clock_mhz"], "clock_mhz_min_max": board["clock_mhz_min_max"],
        "power_w": board["power_w"], "board_refreshes": board["refreshes"],
    }
    res["frac_of_peak"] = res["kernel_tflops"] / PEAK_TFLOPS[op.dtype]
    # against the peak at the clock the chip held: CUs x FLOP/clk/CU x f_measured
    res["frac_clock_adjusted"] = (res["frac_of_peak"] * PEAK_CLOCK_MHZ / board["clock_mhz"]
                                  if board["clock_mhz"] else None)
    alg_bytes = (op.A.nbytes + op.B.nbytes + epi_bytes +
                 op.M * op.N * {"bf16": 2, "f32": 4, "e4m3": 1}[out])
    res["alg_bytes"] = alg_bytes
    res["hbm_gbs_alg"] = alg_bytes / (dev_ms * 1e-3) / 1e9
    clk = (f", {board['clock_mhz']:.0f} MHz, {board['power_w']:.0f} W"
           if board["clock_mhz"] and board["power_w"] else "")
    log(f"{name}: {res['kernel_us']:.1f} us/launch, {res['kernel_tflops']:.1f} TFLOP/s "
        f"({100 * res['frac_of_peak']:.1f}% of {PEAK_TFLOPS[op.dtype]:.0f}), grid {info.grid}, "
        f"tile {info.bm}x{info.bn}x{info.bk}, {res['kernel']}{clk}")
    return res


def cpu_baseline(gi, budget_s=12.0):
    """The oracle as it stands, timed on the host's cores over the bf16 4096^3 workload: the
    whole product (all rows) when it takes less than the budget, repeated until about
    `budget_s` seconds of CPU work have run (a row block of it on a slower host)."""
    import numpy as np
    import oracle
    op = gi.make_workload("bf16_4096")
    threads = oracle.default_threads()
    A = np.ascontiguousarray(op.A).reshape(-1)
    rows = 64
    t0 = time.perf_counter()
    oracle.gemm_ref(rows, op.N, op.K, oracle.BF16, A[: rows * op.K], op.B, threads=threads)
    t_probe = time.perf_counter() - t0
    rows = int(min(op.M, max(64, rows * budget_s / max(t_probe, 1e-3))))
    rows -= rows % 64 or 0
    rows = max(rows, 64)
    reps, dt = 0, 0.0
    while dt < 0.8 * budget_s or reps == 0:
        t0 = time.perf_counter()
        oracle.gemm_ref(rows, op.N, op.K, oracle.BF16, A[: rows * op.K], op.B, threads=threads)
        dt += time.perf_counter() - t0
        reps += 1
    tflops = 2.0 * rows * op.N * op.K * reps / dt / 1e12
    log(f"cpu baseline: oracle on {rows} x {op.N} x {op.K}, {reps} times, in {dt:.1f} s with "
        f"{threads} threads -> {tflops * 1e3:.2f} GFLOP/s")
    host = os.cpu_count() or 0
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = host
    log(f"cpu baseline: host has {host} cores ({usable} usable by this process; nproc)")
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "host_cores": host,
            "host_cores_usable": usable, "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the bf16 4096^3 product (all 4096 columns, full K), "
                      f"{reps} times, fp64 sequential dot products, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=1500.0,
                    help="minimum duration of the untimed warmup per run: the GPU clock settles "
                         "and the board's metrics table (refreshed about once a second) is read "
                         "under load")
    ap.add_argument("--batches", type=int, default=10,
                    help="event-timed batches per run for the kernel time (median batch)")
    ap.add_argument("--batch", type=int, default=50, help="launches per timed batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", default=None, help="time just this run (see RUNS)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the runs, copy this many MiB device to device (counter calibration)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--command", default="", help="with --ingest-pmc: the profiling command")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print a kernel-trace summary (CPU only); --last N timed dispatches")
    ap.add_argument("--summarize-pmc", metavar="COUNTER_CSV",
                    help="print a counter summary (CPU only)")
    ap.add_argument("--last", type=int, default=0)
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.last)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.only or "bf16_4096",
                   args.command, args.copy_calib_mib or 1024)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for {args.gpus}); sharding "
              "across GPUs is a design note, not an implemented path.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import dense_gemm_design_amd as dg
    import gemm_inputs as gi
    dg.load()  # fails loudly if the HIP library is not built

    cache = {}
    sampler = BoardSampler(torch)
    timing = dict(batches=args.batches, batch=args.batch, sampler=sampler)
    if args.only:
        res = time_run(args.only, args.steps, args.warmup, torch, dg, gi, cache, args.settle_ms,
                       **timing)
        if args.copy_calib_mib:
            copy_calibration(torch, args.copy_calib_mib)
        print(json.dumps(res), flush=True)
        return

    head = time_run("bf16_4096", args.steps, args.warmup, torch, dg, gi, cache, args.settle_ms,
                    **timing)
    secondary = {}
    if not args.no_secondary:
        for name in ("bf16_4096_pp", "bf16_4096_coop", "bf16_4096_linear", "bf16_4096_t128",
                     "bf16_4096_blocked", "fp8_8192_pp", "fp8_8192_e4m3_amax", "fp8_8192_blocked",
                     "fp8_8192_morton", "fp8_8192", "bf16_mlp_up_bias_gelu",
                     "bf16_mlp_up_source_bias_gelu", "bf16_mlp_up",
                     "bf16_mlp_up_t256",
                     "bf16_streamk", "bf16_256"):
            steps = max(10, args.steps // (4 if name.startswith("fp8_8192") else 1))
            r = time_run(name, steps, max(2, args.warmup // 2), torch, dg, gi, cache,
                         args.settle_ms, **timing)
            secondary[name] = {k: r[k] for k in ("kernel_us", "kernel_tflops", "frac_of_peak",
                                                 "frac_clock_adjusted", "clock_mhz", "power_w",
                                                 "batch_us_min_median_max",
                                                 "hbm_gbs_alg", "tile", "grid", "mapping",
                                                 "sched", "kernel", "out", "epilogue",
                                                 "group", "group_n")}
            if name in cache:
                del cache[name]
    cache.clear()
    torch.cuda.empty_cache()

    flops = 2.0 * head["M"] * head["N"] * head["K"]
    achieved = flops / (head["kernel_us"] * 1e-6) / 1e12
    line = {
        "metric": "GEMM TFLOPS and % of MI355X MFMA peak, bf16 4096^3 and fp8 8192^3",
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 gemm M=N=K=4096, uniform[-1,1], fp32 accumulate, bf16 out",
                   "M": 4096, "N": 4096, "K": 4096, "tile": head["tile"],
                   "mapping": "grouped_m", "group": 8, "sched": "persistent",
                   "grid": head["grid"], "kernel": head["kernel"],
                   "warmup_launches": head["warmup_launches"],
                   "settle_ms": args.settle_ms},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": measured_traffic("bf16_4096"),
                     "kernel_us": round(head["kernel_us"], 2),
                     "timing": f"median of {args.batches} batches of {args.batch} launches, HIP "
                               "events on the launch stream",
                     "clock_mhz": head["clock_mhz"], "power_w": head["power_w"],
                     "peak_at_clock": (round(PEAK_TFLOPS["bf16"] * head["clock_mhz"] /
                                             PEAK_CLOCK_MHZ, 1) if head["clock_mhz"] else None),
                     "frac_clock_adjusted": (round(head["frac_clock_adjusted"], 4)
                                             if head["frac_clock_adjusted"] else None)},
        "secondary": secondary,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(gi)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
