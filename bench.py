"""Benchmark: tiled, software-pipelined GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--variant k=v,...]

A step is one C = A x B of the workload (default bf16 M = N = K = 4096,
N(0,1) operands rounded to bf16, fp32 output) through the C ABI, with A, B
and C already resident in HBM.  Prints ONE JSON line with the throughput, a
roofline record for the kernel (achieved vs MI355X dense peak, from HIP
events on the launch stream) and the CPU oracle's rate on a bounded sample of
the same workload.

Extra modes (not used by the default run):
    --ladder     the ablation ladder of the workload's type, one change per rung
                 (TFLOP/s, gain over the rung it changes, bit identity with the
                 default plan; --ladder-summary writes the table)
    --late-barrier  the default kernel against its late-barrier twin, in sustained
                 bursts with each one's shader clock (the power-cap measurement)
    --c-stores   the default plan under each C store policy (auto / streaming / plain)
    --variants   time every compiled variant of the workload's type
    --sweep      the bf16 shape sweep: the 128x128x32 tile with the register-
                 staged loader (2 slots) and the direct loader (1-4 slots), and
                 the default plan per shape, timed by HIP-graph replay
                 (--sweep-summary writes the heatmap)
    --lds-probe  LDS read throughput of ds_read_b32 / b64 / b128 / b64_tr_b16
    --mfma-probe matrix-core rate and clock for bf16 / int8 operand bits
                 (the workloads' random operands, all ones, all zeros)
    --cold       per-launch kernel time with the caches cold: a 512 MiB buffer is
                 written before every launch, evicting L2 and MALL (one JSON line)
    --soak S     run the workload's GEMM, then the matrix-core probe on random
                 operands of its type, back to back for S seconds each while
                 sampling socket power and shader clocks (amd-smi)
    --gpus N     N > 1 exits: this path runs on one GPU
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s or TOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2500.0, "i8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# timed regions whose launches take less than this (ms each when launched one
# by one from Python, about the host's own launch path) are re-timed as one
# HIP-graph replay of the same steps.  Longer kernels stay eager: replaying
# graph nodes costs a few microseconds per kernel (bf16 512x4096x4096: 31.0
# us per launch replayed against 26.5 eager).
GRAPH_BELOW_MS = 0.02
METRIC = "GEMM TFLOPS (TOPS int8) and % of MI355X MFMA peak, bf16 M=N=K=4096"


def parse_variant(text, lib):
    if not text:
        return None
    v = lib.Variant()
    for kv in text.split(","):
        k, val = kv.split("=")
        setattr(v, k.strip(), int(val))
    return v


def algorithmic_bytes(w):
    from tiled_software_pipelined_amd import metrics
    return metrics.algorithmic_bytes(w.M, w.N, w.K, {"f32": 4, "bf16": 2, "i8": 1}[w.dtype], 4)


def time_plan(lib, torch, w, A, B, C, variant, steps, warmup):
    """Per-launch kernel durations (ms) from HIP events on the launch stream,
    plus the wall time of the whole timed region."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        lib.gemm(A, B, out=C, variant=variant)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        lib.gemm(A, B, out=C, variant=variant)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return per, wall


def time_region(lib, torch, A, B, C, variant, steps, warmup):
    """The timed region of the headline run: `steps` launches back to back
    on the launch stream with nothing between them, bracketed by a
    synchronisation and a HIP event on each side.  Returns the mean launch
    duration from the two events (ms) and the wall time of the region (s).
    (Events around every launch would put their own commands between the
    kernels and slow the region down.)"""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        lib.gemm(A, B, out=C, variant=variant)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        lib.gemm(A, B, out=C, variant=variant)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_region_graph(lib, torch, A, B, C, variant, steps):
    """The timed region as one HIP-graph replay of `steps` launches, for
    kernels shorter than the host's launch path (a few microseconds): the
    same bracketing (synchronisation and a HIP event on each side) with no
    host work between the launches.  Returns (mean ms per launch from the
    events, wall seconds, whether the replay reproduced the eager C)."""
    lib.gemm(A, B, out=C, variant=variant)
    torch.cuda.synchronize()
    eager = C.clone()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(steps):
            lib.gemm(A, B, out=C, variant=variant)
    graph.replay()  # warm
    torch.cuda.synchronize()
    C.zero_()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    same = bool(torch.equal(C, eager))
    del graph
    return e0.elapsed_time(e1) / steps, wall, same


def time_graph(lib, torch, A, B, C, variant, per_graph=20, replays=10):
    """Per-launch time (ms) from replaying a HIP graph of `per_graph`
    launches: no host work inside the timed interval, so short kernels are
    timed at the GPU's own cadence rather than the launch path's.  Returns
    (median ms per launch, whether every replay reproduced the eager C)."""
    lib.gemm(A, B, out=C, variant=variant)
    torch.cuda.synchronize()
    eager = C.clone()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(per_graph):
            lib.gemm(A, B, out=C, variant=variant)
    same = True
    per = []
    for _ in range(replays):
        C.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / per_graph)
        same = same and bool(torch.equal(C, eager))
    del graph
    return statistics.median(per), same


def cpu_model():
    """The host CPU's model name (Linux), or an empty string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(w, A_cpu, B_cpu, budget_s=12.0):
    """The oracle (fp64 / int64 triple loop, OpenMP) on a row sample of the
    same operands: blocks of rows are taken, passing over A again from its
    first row when the whole product has been done, until about `budget_s`
    of CPU work.  Products of at most 2 GFLOP are also timed whole on one
    thread (`single_thread_s`)."""
    import numpy as np

    import oracle
    from tiled_software_pipelined_amd import inputs
    Bo = inputs.as_oracle_array(B_cpu)
    rows = 8
    t = 0.0
    done_rows = 0
    total_t = 0.0
    start = 0
    while True:
        n = min(rows, w.M - start)
        Ao = inputs.as_oracle_array(A_cpu[start:start + n])
        t0 = time.perf_counter()
        oracle.gemm(Ao, Bo, w.dtype)
        t = time.perf_counter() - t0
        done_rows += n
        start = (start + n) % w.M
        total_t += t
        if total_t >= budget_s:
            break
        left = budget_s - total_t
        rows = int(max(8, min(w.M, rows * min(4.0, left / max(t, 1e-3)))))
    flops = 2.0 * done_rows * w.N * w.K
    passes = done_rows / w.M
    sample = ("%.2f passes over all %d rows of A" % (passes, w.M) if passes >= 1 else
              "first %d of %d rows of A" % (done_rows, w.M))
    rec = {"value": flops / total_t / 1e12, "unit": "TFLOPS" if w.dtype != "i8" else "TOPS",
           "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
           "sample": "%s times all of B (%s %dx%dx%d), %.1f s" % (sample, w.dtype, w.M, w.N, w.K, total_t)}
    if 2.0 * w.M * w.N * w.K <= 2e9:
        threads = oracle.num_threads()
        oracle.set_num_threads(1)
        try:
            Ao = inputs.as_oracle_array(A_cpu)
            t0 = time.perf_counter()
            oracle.gemm(Ao, Bo, w.dtype)
            rec["single_thread_s"] = round(time.perf_counter() - t0, 4)
        finally:
            oracle.set_num_threads(threads)
    return rec


def lds_probe(torch, lib, workgroups=2048, reps=2048, rounds=8, launches=3):
    """LDS read throughput per instruction form and address pattern, timed
    round-robin.  Each workgroup of 256 threads reads 64 bytes per thread per
    iteration: pattern "linear" is conflict-free for every width (the forms
    differ by instruction alone), "swizzled" reads 16-byte pieces of
    256-byte rows whose chunks are XOR-permuted by the row index."""
    out = torch.empty(workgroups * lib.LDS_PROBE_THREADS, dtype=torch.int32, device="cuda:0")
    nbytes = workgroups * lib.LDS_PROBE_THREADS * 64 * reps
    cases = [(k, p) for p in range(2) for k in range(4)]
    times = {c: [] for c in cases}
    for k, p in cases:
        lib.lds_read_probe(k, p, 16, out)  # warm-up
    torch.cuda.synchronize()
    for _ in range(rounds):
        for k, p in cases:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(launches)]
            for e0, e1 in ev:
                e0.record()
                lib.lds_read_probe(k, p, reps, out)
                e1.record()
            torch.cuda.synchronize()
            times[(k, p)] += [e0.elapsed_time(e1) for e0, e1 in ev]
    for k, p in cases:
        ms = statistics.median(times[(k, p)])
        tbs = nbytes / (ms * 1e-3) / 1e12
        print(json.dumps({"mode": "lds_probe", "instruction": lib.LDS_PROBE_KINDS[k],
                          "pattern": lib.LDS_PROBE_PATTERNS[p], "workgroups": workgroups, "reps": reps,
                          "bytes": nbytes, "median_ms": round(ms, 4), "TB_per_s": round(tbs, 2),
                          "bytes_per_clk_per_cu_at_2p4GHz": round(tbs * 1e12 / 256 / 2.4e9, 1)}), flush=True)


def mfma_ceiling(torch, lib, dtype, source, reps=None, workgroups=256, launches=3):
    """The rate probe (no memory traffic) on operand bits drawn as `source`:
    "random" = the GEMM workloads' distribution (bf16 N(0,1), int8 uniform,
    fp32 uniform[-1, 1)), "ones", "zeros".  bf16 / int8: the matrix
    instruction, one wave per SIMD, 16 independent accumulators; fp32:
    v_fmac_f32, with `workgroups` / 256 x 4 waves per SIMD.  Returns
    (TFLOP/s or TOP/s, mean clock in GHz from the shader-clock / real-time
    tick ratio, median ms)."""
    from tiled_software_pipelined_amd import inputs
    kind = lib.RATE_PROBE_KINDS.index(dtype)
    nbytes = workgroups * lib.RATE_PROBE_THREADS * 8 * 16
    if source == "random":
        kinds = {"bf16": ("bf16_normal", 2), "i8": ("i8_uniform", 1), "f32": ("f32_uniform", 4),
                 "bf16_lds": ("bf16_normal", 2), "bf16_lds_dma": ("bf16_normal", 2)}
        kname, esz = kinds[dtype]
        ops = inputs.operand(kname, nbytes // esz // 2048, 2048, 77 + kind)
    else:
        tdt = {"i8": torch.int8, "f32": torch.float32}.get(dtype, torch.bfloat16)
        esz = {"i8": 1, "f32": 4}.get(dtype, 2)
        ops = torch.full((nbytes // esz,), 1 if source == "ones" else 0, dtype=tdt)
    ops = ops.contiguous().view(-1).to("cuda:0")
    out = torch.empty(workgroups * lib.RATE_PROBE_THREADS, dtype=torch.int32, device="cuda:0")
    clocks = torch.empty(2 * workgroups, dtype=torch.int64, device="cuda:0")
    per_iter = float(lib.RATE_PROBE_OPS_PER_INST[dtype]) * 16 * 4 * workgroups  # ops per loop iteration
    # about 20 ms per launch at the datasheet peak
    reps = reps or max(1, int(20e-3 * PEAK_TFLOPS[dtype[:4] if dtype.startswith("bf16") else dtype] * 1e12 / per_iter))
    lib.mfma_rate_probe(kind, max(1, reps // 10), ops, out, clocks)
    torch.cuda.synchronize()
    ms, ghz = [], []
    for _ in range(launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lib.mfma_rate_probe(kind, reps, ops, out, clocks)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        c = clocks.view(-1, 2).double().cpu()
        ghz.append(float((c[:, 0] / c[:, 1]).mean()) * 0.1)
    med = statistics.median(ms)
    return per_iter * reps / (med * 1e-3) / 1e12, statistics.median(ghz), med


# waves per SIMD of the fp32 rate probe and the workgroups that give them
F32_PROBE_WAVES = {4: 1024, 8: 2048}


class PowerSampler:
    """Samples socket power (W) and the per-XCD shader clocks (MHz) with
    amd-smi in a child process every `period` seconds while active."""

    def __init__(self, period=0.25):
        import shutil
        import threading
        self.exe = shutil.which("amd-smi")
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)

    def _one(self):
        import subprocess
        r = subprocess.run([self.exe, "metric", "-p", "-c", "--json"], capture_output=True, text=True, timeout=10)
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        watts = float(g["power"]["socket_power"]["value"])
        clocks = [float(v["clk"]["value"]) for k, v in sorted(g["clock"].items()) if k.startswith("gfx_")]
        return watts, clocks

    def _loop(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._one())
            except Exception:  # noqa: BLE001 - a missing or failing tool leaves no sample
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self.exe:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.exe:
            self._thread.join()

    def summary(self, skip=2):
        s = self.samples[skip:] if len(self.samples) > skip + 2 else self.samples
        if not s:
            return None
        watts = statistics.mean(w for w, _ in s)
        per_xcd = [statistics.mean(c[i] for _, c in s) for i in range(len(s[0][1]))]
        return {"socket_w": round(watts, 1), "gfx_mhz_per_xcd": [round(c) for c in per_xcd],
                "gfx_mhz_mean": round(statistics.mean(per_xcd)), "samples": len(s)}


def soak(torch, lib, w, A, B, C, seconds):
    """The default plan back to back for `seconds`, then the matrix-core
    probe on random operands of the workload's type for as long, each with
    power and clock samples: energy per operation of the GEMM against the
    same chip's energy per operation of the matrix cores alone."""
    lines = []
    with PowerSampler() as ps:
        n = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(200):
                lib.gemm(A, B, out=C)
            torch.cuda.synchronize()
            n += 200
        dt = time.perf_counter() - t0
    rate = w.flops * n / dt / 1e12
    lines.append({"mode": "soak", "what": "gemm " + w.name, "launches": n, "seconds": round(dt, 2),
                  "rate": round(rate, 1), "power": ps.summary()})
    if w.dtype in ("bf16", "i8"):
        with PowerSampler() as ps:
            t0 = time.perf_counter()
            reps = 0
            while time.perf_counter() - t0 < seconds:
                r, ghz, ms = mfma_ceiling(torch, lib, w.dtype, "random", launches=3)
                reps += 1
        lines.append({"mode": "soak", "what": "matrix-core probe, random %s operands" % w.dtype,
                      "rate": round(r, 1), "clock_ghz": round(ghz, 3), "power": ps.summary()})
    for rec in lines:
        p = rec.get("power")
        if p:
            rec["pj_per_op"] = round(p["socket_w"] / (rec["rate"] * 1e12) * 1e12, 3)
        print(json.dumps(rec), flush=True)


def cold_timing(torch, lib, w, A, B, C, variant, launches=30):
    """Kernel time per launch with cold caches: before each launch a 512 MiB
    buffer is filled (more than the 256 MB MALL and the 8 x 4 MB of L2), so
    A and B start in HBM; HIP events bracket the GEMM alone."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(20):
        lib.gemm(A, B, out=C, variant=variant)
    per = []
    for _ in range(launches):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lib.gemm(A, B, out=C, variant=variant)
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    ms = statistics.median(per)
    print(json.dumps({"mode": "cold", "workload": w.name, "launches": launches, "median_ms": round(ms, 5),
                      "min_ms": round(min(per), 5), "rate": round(w.flops / ms / 1e9, 1),
                      "unit": "TOP/s" if w.dtype == "i8" else "TFLOP/s"}), flush=True)


NOMINAL_GHZ = 2.4      # the shader clock the datasheet peaks assume
CLOCKED_LAUNCHES = 20


def clocked_rate(torch, lib, plan, A, B, C, variant):
    """Clock readings of the plan's tiled kernel over a few launches through
    gemm_run_clocked, or None when the plan has none to clock or the run
    repacks operands (the clocked entry runs the plan as gemm_run does).
    Returns a dict: mean shader clock (GHz), per XCD (workgroup w runs on
    XCD w mod 8) its mean clock and the time from the launch's first
    workgroup start to that XCD's last end, and the split of the launch into
    K loop and C write-back (per-workgroup means, and the time from the
    first start to the last K-loop end vs to the last end)."""
    slots = plan.clock_slots()
    if slots == 0 or (variant is None and plan.workspace_bytes(A.data_ptr(), B.data_ptr()) > 0):
        return None
    clocks = torch.zeros(CLOCKED_LAUNCHES * slots, dtype=torch.int64, device=A.device)
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(CLOCKED_LAUNCHES):
        plan.run_clocked_ptr(A.data_ptr(), B.data_ptr(), C.data_ptr(), clocks.data_ptr() + 8 * i * slots, slots,
                             stream)
    torch.cuda.synchronize()
    nv = lib.CLOCK_VALUES
    # the buffer is sized for the largest grid among the plan's kernels (a
    # fallback for unaligned rows may use a smaller tile); the operands here
    # are the plan's own, so its main kernel ran and only its grid's rows
    # were written
    grid = plan.info().grid
    c = clocks.cpu().numpy().view("uint64").reshape(CLOCKED_LAUNCHES, -1, nv)[:, :grid]
    if not (c[:, :, 1] > 0).all():
        raise RuntimeError("clocked run: a workgroup of the grid wrote no clock values")
    ghz = lib.clock_ghz(c)
    wg = c.shape[1]
    xcd = [lib.clock_ghz(c[:, x::8]) if x < wg else None for x in range(8)]
    start = c[:, :, 1].min(axis=1).astype("int64")
    span_us = [float(((c[:, x::8, 5].max(axis=1).astype("int64") - start) * 0.01).mean()) if x < wg else None
               for x in range(8)]
    loop_us, store_us = lib.clock_split_us(c)
    last_loop = float(((c[:, :, 3].max(axis=1).astype("int64") - start) * 0.01).mean())
    last_end = float(((c[:, :, 5].max(axis=1).astype("int64") - start) * 0.01).mean())
    return {"ghz": ghz, "xcd_ghz": xcd, "xcd_last_end_us": span_us,
            "wg_loop_us": float(loop_us.mean()), "wg_store_us": float(store_us.mean()),
            "last_loop_end_us": last_loop, "last_end_us": last_end}


def env_record(torch, lib, dev):
    """Where the line was measured: device, runtime versions, library
    version and the hash of the kernel sources it was built from."""
    from tiled_software_pipelined_amd import provenance
    p = torch.cuda.get_device_properties(dev)
    return {"device": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__, "libtgemm": lib.version(),
            "kernel_sources": provenance.source_hash()}


def _round_robin(torch, lib, w, A, B, C, variants, steps, slow):
    """Median / p10 per-launch ms of every variant, timed round-robin (a few
    launches of each per round, many rounds) so that clock and thermal drift
    spreads over all of them.  `slow`: indices timed once per round and only
    in the first two rounds."""
    rounds = max(4, steps // 3)
    times = {i: [] for i in range(len(variants))}
    for v in variants:  # warm every kernel once
        lib.gemm(A, B, out=C, variant=v)
    torch.cuda.synchronize()
    for r in range(rounds):
        for i, v in enumerate(variants):
            if i in slow and r >= 2:
                continue
            per, _ = time_plan(lib, torch, w, A, B, C, v, 1 if i in slow else 3, 0)
            times[i] += per
    out = []
    for i in range(len(variants)):
        t = sorted(times[i])
        out.append((t[len(t) // 2], t[len(t) // 10], len(t)))
    return out


def run_ladder(torch, lib, w, A, B, C, args):
    """The ablation ladder of the workload's type (tiled_software_pipelined_amd
    .ladders): every rung timed round-robin, then one JSON line per rung with
    TFLOP/s, the gain over the rung it changes one thing of, and whether its
    C is the same bit for bit as the default plan's (every matrix-core rung
    and every fp32 rung accumulates each output in increasing k; the oracle
    check of every rung at this size is tests/test_ladder_gpu.py).  With
    --ladder-summary PATH also a Markdown table."""
    from tiled_software_pipelined_amd import ladders
    code = {"f32": lib.F32, "bf16": lib.BF16, "i8": lib.I8}[w.dtype]
    rungs = list(ladders.LADDERS[w.dtype])
    variants = []
    for r in rungs:
        variants.append(None if r.fields is None else lib.Variant(**r.fields))
    labels = [r.label for r in rungs]
    if w.dtype != "f32":
        # the default plan under each workgroup order
        for grp in (lib.ORDER_ROW_MAJOR, 1, 2, 4, 8):
            dv = lib.plan_for(w.M, w.N, w.K, code, w.K, w.N, w.N).info().variant
            dv.wg_group = grp
            variants.append(dv)
            rungs.append(ladders.Rung("R8g%d" % grp, "default plan, workgroup order %s" % (
                "row-major" if grp < 0 else "XCD-aware, groups of %d tile rows" % grp), dv.as_dict(),
                base="R8"))
            labels.append(rungs[-1].label)
    ref = torch.empty_like(C)
    lib.gemm(A, B, out=ref)
    torch.cuda.synchronize()
    same = []
    for v in variants:
        C.fill_(-7)
        lib.gemm(A, B, out=C, variant=v)
        torch.cuda.synchronize()
        same.append(bool(torch.equal(C, ref)))
        if not same[-1]:
            d = (C.double() - ref.double()).abs().max().item()
            same[-1] = "max |diff| %.3g" % d
    slow = {i for i, v in enumerate(variants) if v is not None and v.kernel == lib.KERNEL_NAIVE}
    timing = _round_robin(torch, lib, w, A, B, C, variants, args.steps, slow)
    unit = "TOP/s" if w.dtype == "i8" else "TFLOP/s"
    lines = []
    for i, r in enumerate(rungs):
        ms, p10, n = timing[i]
        tf = w.flops / ms / 1e9
        b = ladders.base_of(rungs, i)
        gain = None if b is None else 100.0 * (timing[b][0] / ms - 1.0)
        kname = lib.plan_for(w.M, w.N, w.K, code, w.K, w.N, w.N, variants[i]).name
        rec = {"mode": "ladder", "workload": w.name, "rung": r.label, "change": r.change, "kernel": kname,
               "median_ms": round(ms, 5), "p10_ms": round(p10, 5), "launches": n, "rate": round(tf, 1),
               "unit": unit, "frac_peak": round(tf / PEAK_TFLOPS[w.dtype], 4),
               "base": None if b is None else rungs[b].label,
               "gain_vs_base_pct": None if gain is None else round(gain, 1),
               "same_bits_as_default": same[i]}
        lines.append(rec)
        print(json.dumps(rec), flush=True)
    if args.ladder_summary:
        write_ladder_summary(args, w, lines, unit)


def write_ladder_summary(args, w, lines, unit):
    import torch
    from tiled_software_pipelined_amd import lib
    hdr = ["# Ablation ladder: %s GEMM M=%d N=%d K=%d" % (w.dtype, w.M, w.N, w.K), "",
           "Command: `python bench.py --workload %s --ladder --steps %d --ladder-summary %s`" % (
               w.name, args.steps, args.ladder_summary), "",
           "Device: %s (%s), libtgemm %s.  Every rung timed round-robin in one process (median of the "
           "per-launch HIP-event times); `gain` is against the rung in `base`, which differs from it in one "
           "thing; `same bits` compares C with the default plan's bit for bit (each rung's C is also checked "
           "against the CPU oracle at this size by tests/test_ladder_gpu.py)." % (
               torch.cuda.get_device_properties(0).name, getattr(torch.cuda.get_device_properties(0),
                                                                 "gcnArchName", ""), lib.version()), "",
           "| rung | change | kernel | median us | %s | %% of peak | base | gain | same bits |" % unit,
           "|---|---|---|---|---|---|---|---|---|"]
    for r in lines:
        hdr.append("| %s | %s | `%s` | %.1f | %.1f | %.1f | %s | %s | %s |" % (
            r["rung"], r["change"], r["kernel"], r["median_ms"] * 1e3, r["rate"], 100 * r["frac_peak"],
            r["base"] or "", "" if r["gain_vs_base_pct"] is None else "%+.1f %%" % r["gain_vs_base_pct"],
            "yes" if r["same_bits_as_default"] is True else r["same_bits_as_default"]))
    os.makedirs(os.path.dirname(os.path.abspath(args.ladder_summary)), exist_ok=True)
    with open(args.ladder_summary, "w") as f:
        f.write("\n".join(hdr) + "\n")


def run_variants(torch, lib, w, A, B, C, args):
    """Every compiled variant of the workload's type, timed round-robin (one
    JSON line each)."""
    code = {"f32": lib.F32, "bf16": lib.BF16, "i8": lib.I8}[w.dtype]
    variants = lib.variants(code)
    slow = {i for i, v in enumerate(variants) if v.kernel == lib.KERNEL_NAIVE}
    timing = _round_robin(torch, lib, w, A, B, C, variants, args.steps, slow)
    for i, v in enumerate(variants):
        ms, p10, n = timing[i]
        print(json.dumps({"mode": "variants", "workload": w.name,
                          "kernel": lib.plan_for(w.M, w.N, w.K, code, w.K, w.N, w.N, v).name,
                          "median_ms": ms, "p10_ms": p10, "launches": n, "rate": w.flops / ms / 1e9,
                          "frac_peak": w.flops / ms / 1e9 / PEAK_TFLOPS[w.dtype]}), flush=True)


def run_late_barrier(torch, lib, w, A, B, C, args, rounds=6, settle=500, timed=300):
    """The workload's default kernel against its twin with the slice's
    barrier half-way through the last K step (copy_sched LATE: the cores idle
    longer there, everything else the same).  Each is timed in sustained
    bursts, since the shader clock follows the power drawn over many
    milliseconds: `settle` launches, then `timed` launches between two HIP
    events, then clocked launches for the kernel's own shader clock; the two
    alternate for `rounds` rounds.  One JSON line per burst, then one summary
    line per kernel (medians) with whether the two wrote the same bits."""
    code = {"f32": lib.F32, "bf16": lib.BF16, "i8": lib.I8}[w.dtype]
    kinds = [("default", None), ("late barrier", lib.Variant(kernel=lib.KERNEL_TILED, copy_sched=lib.COPY_LATE))]
    outs = []
    for _, v in kinds:
        C.fill_(-7)
        lib.gemm(A, B, out=C, variant=v)
        torch.cuda.synchronize()
        outs.append(C.clone())
    same = bool(torch.equal(outs[0], outs[1]))
    del outs
    stream = torch.cuda.current_stream()
    res = {label: {"us": [], "ghz": []} for label, _ in kinds}
    names = {}
    for r in range(rounds):
        for label, v in kinds:
            plan = lib.plan_for(w.M, w.N, w.K, code, w.K, w.N, w.N, v)
            names[label] = plan.name
            for _ in range(settle):
                lib.gemm(A, B, out=C, variant=v)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(timed):
                lib.gemm(A, B, out=C, variant=v)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / timed
            clk = clocked_rate(torch, lib, plan, A, B, C, v)
            res[label]["us"].append(us)
            res[label]["ghz"].append(clk["ghz"])
            print(json.dumps({"mode": "late_barrier", "workload": w.name, "round": r, "kernel": plan.name,
                              "us": round(us, 2), "ghz": round(clk["ghz"], 3)}), flush=True)
    for label, _ in kinds:
        us = sorted(res[label]["us"])[len(res[label]["us"]) // 2]
        ghz = sorted(res[label]["ghz"])[len(res[label]["ghz"]) // 2]
        print(json.dumps({"mode": "late_barrier_summary", "workload": w.name, "kernel": names[label],
                          "median_us": round(us, 2), "median_ghz": round(ghz, 3),
                          "rate": round(w.flops / us / 1e6, 1), "rate_per_ghz": round(w.flops / us / 1e6 / ghz, 1),
                          "same_bits_as_default": same, "rounds": rounds, "settle": settle, "timed": timed}),
              flush=True)


def run_c_stores(torch, lib, w, A, B, C, per_graph=20, rounds=15):
    """The workload's default plan under each C store policy (AUTO, STREAM,
    PLAIN: tgemm_set_c_store_policy), each captured as one HIP graph of
    `per_graph` launches (the policy is read when a run is enqueued) and
    replayed round-robin `rounds` times.  One JSON line per policy: the
    median per-launch time, and whether its C equals AUTO's bit for bit."""
    policies = [("auto", lib.C_STORES_AUTO), ("stream", lib.C_STORES_STREAM), ("plain", lib.C_STORES_PLAIN)]
    graphs, outs = {}, {}
    try:
        for label, pol in policies:
            lib.set_c_store_policy(pol)
            C.fill_(-7)
            lib.gemm(A, B, out=C)
            torch.cuda.synchronize()
            outs[label] = C.clone()
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for _ in range(per_graph):
                        lib.gemm(A, B, out=C)
            graphs[label] = g
    finally:
        lib.set_c_store_policy(lib.C_STORES_AUTO)
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()
    times = {label: [] for label in graphs}
    for _ in range(rounds):
        for label, g in graphs.items():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            times[label].append(e0.elapsed_time(e1) * 1e3 / per_graph)
    kname = lib.plan_for(w.M, w.N, w.K, {"f32": lib.F32, "bf16": lib.BF16, "i8": lib.I8}[w.dtype],
                         w.K, w.N, w.N).name
    for label, t in times.items():
        t.sort()
        print(json.dumps({"mode": "c_stores", "workload": w.name, "kernel": kname, "policy": label,
                          "median_us": round(t[len(t) // 2], 2), "min_us": round(t[0], 2),
                          "same_bits_as_auto": bool(torch.equal(outs[label], outs["auto"]))}), flush=True)


SWEEP_VARIANTS = [  # (label, loader, stages) on the 128 x 128 x 32 tile, then the default plan
    ("direct_s1", 2, 1), ("vgpr_s2", 1, 2), ("direct_s2", 2, 2), ("direct_s3", 2, 3), ("direct_s4", 2, 4),
    ("default", None, None)]


def run_sweep(torch, lib, dev, args, rounds=3):
    """The bf16 shape sweep: every sweep shape x (the 128 x 128 x 32 tile
    with the register-staged loader at 2 slots and the direct loader at 1 to
    4 slots, and the default plan).  Per-launch times come from HIP-graph
    replay (the smallest shapes run for a few microseconds, less than the
    host's launch path), interleaved over the variants `rounds` times; the
    median is reported.  Each variant's C must equal the default plan's bit
    for bit (the oracle check of every cell is tests/test_fullsize_gpu.py).
    With --sweep-summary PATH also a Markdown heatmap."""
    from tiled_software_pipelined_amd import inputs, metrics
    vs = []
    for label, loader, st in SWEEP_VARIANTS:
        v = None if loader is None else lib.Variant(
            kernel=lib.KERNEL_TILED, tile_m=128, tile_n=128, tile_k=32, stages=st, loader=loader,
            lds_layout=lib.LDS_XOR, waves_m=2, waves_n=2)
        vs.append((label, v))
    cells = []
    for name, sw in inputs.workloads().items():
        if not name.startswith("bf16_sweep"):
            continue
        a, b = sw.operands()
        a, b = a.to(dev), b.to(dev)
        c = torch.empty((sw.M, sw.N), dtype=torch.float32, device=dev)
        ref = torch.empty_like(c)
        lib.gemm(a, b, out=ref)
        torch.cuda.synchronize()
        ideal_ms = 1e3 * metrics.roofline_time(sw.M, sw.N, sw.K, 2, 4, PEAK_TFLOPS["bf16"] * 1e12,
                                               PEAK_HBM_GBS * 1e9)
        times = {label: [] for label, _ in vs}
        for _ in range(rounds):
            for label, v in vs:
                ms, same = time_graph(lib, torch, a, b, c, v)
                if not same:
                    raise RuntimeError("graph replay of %s (%s) did not reproduce the eager result" % (name, label))
                if not torch.equal(c, ref):
                    raise RuntimeError("%s (%s) differs from the default plan's C" % (name, label))
                times[label].append(ms)
        for label, v in vs:
            ms = statistics.median(times[label])
            rec = {"mode": "sweep", "workload": name, "M": sw.M, "N": sw.N, "K": sw.K, "plan": label,
                   "kernel": lib.plan_for(sw.M, sw.N, sw.K, lib.BF16, sw.K, sw.N, sw.N, v).name,
                   "median_ms": ms, "tflops": sw.flops / ms / 1e9, "frac_peak": sw.flops / ms / 1e9 / PEAK_TFLOPS["bf16"],
                   "frac_roofline": ideal_ms / ms, "ideal_ms": ideal_ms, "same_bits_as_default": True}
            cells.append(rec)
            print(json.dumps(rec), flush=True)
        del a, b, c, ref
    if args.sweep_summary:
        write_sweep_summary(args, cells)


def write_sweep_summary(args, cells):
    import torch
    from tiled_software_pipelined_amd import lib
    labels = [l for l, _, _ in SWEEP_VARIANTS]
    shapes = []
    for c in cells:
        if (c["M"], c["K"]) not in shapes:
            shapes.append((c["M"], c["K"]))
    get = {(c["M"], c["K"], c["plan"]): c for c in cells}
    out = ["# bf16 shape sweep by loader and ring depth", "",
           "Command: `python bench.py --sweep --sweep-summary %s`" % args.sweep_summary, "",
           "Device: %s, libtgemm %s.  TFLOP/s per cell from HIP-graph replay (20 launches per replay, median "
           "of 3 interleaved rounds).  The 128 x 128 x 32 tile with the register-staged loader at 2 slots "
           "(`vgpr_s2`) and the direct global->LDS loader at 1 to 4 slots, and the default plan.  Every "
           "cell's C equals the default plan's bit for bit; tests/test_fullsize_gpu.py checks every cell "
           "against the oracle.  `async gain` = vgpr_s2 time / direct_s2 time - 1 (the same ring depth, "
           "the copy alone changed); `best direct` = the fastest direct ring depth against vgpr_s2.  "
           "%% roofline = max(2MNK / 2.5 PF, algorithmic bytes / 8 TB/s) / time." % (
               torch.cuda.get_device_properties(0).name, lib.version()), "",
           "| M=N | K | " + " | ".join(labels) + " | default kernel | default % roofline | async gain | "
           "best direct vs vgpr_s2 |",
           "|---|---|" + "---|" * len(labels) + "---|---|---|---|"]
    for mn, k in shapes:
        row = [str(mn), str(k)] + ["%.1f" % get[(mn, k, l)]["tflops"] for l in labels]
        d = get[(mn, k, "default")]
        vg = get[(mn, k, "vgpr_s2")]["median_ms"]
        d2 = get[(mn, k, "direct_s2")]["median_ms"]
        best = min(get[(mn, k, l)]["median_ms"] for l in ("direct_s2", "direct_s3", "direct_s4"))
        row += ["`%s`" % d["kernel"], "%.1f" % (100 * d["frac_roofline"]), "%+.1f %%" % (100 * (vg / d2 - 1)),
                "%+.1f %%" % (100 * (vg / best - 1))]
        out.append("| " + " | ".join(row) + " |")
    os.makedirs(os.path.dirname(os.path.abspath(args.sweep_summary)), exist_ok=True)
    with open(args.sweep_summary, "w") as f:
        f.write("\n".join(out) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the shader clock takes tens of milliseconds of load to ramp up from idle
    # (the first 50 launches of bf16 4096^3 average 134 us, later ones 115)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="bf16_4096")
    ap.add_argument("--variant", default="")
    ap.add_argument("--ladder", action="store_true",
                    help="the ablation ladder of the workload's type (one JSON line per rung)")
    ap.add_argument("--ladder-summary", default="", metavar="PATH",
                    help="with --ladder: also write the rung table as Markdown to PATH")
    ap.add_argument("--variants", action="store_true",
                    help="time every compiled variant of the workload's type")
    ap.add_argument("--c-stores", action="store_true",
                    help="the default plan under each C store policy (auto, streaming, plain), timed by "
                         "HIP-graph replay (one JSON line per policy)")
    ap.add_argument("--late-barrier", action="store_true",
                    help="the default kernel against its twin with the slice's barrier later in the last K "
                         "step, each timed in sustained bursts with its shader clock (one JSON line per burst)")
    ap.add_argument("--sweep", action="store_true",
                    help="the bf16 shape sweep by loader and ring depth (one JSON line per cell)")
    ap.add_argument("--sweep-summary", default="", metavar="PATH",
                    help="with --sweep: also write the heatmap as Markdown to PATH")
    ap.add_argument("--lds-probe", action="store_true",
                    help="time the LDS read-path probe: the same bytes through ds_read_b32 / b64 / "
                         "b128 / b64_tr_b16 (one JSON line per instruction form)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="matrix-core rate and clock for bf16 / int8 with random, all-ones and all-zero "
                         "operand bits (one JSON line each)")
    ap.add_argument("--cold", action="store_true",
                    help="per-launch kernel time with L2 and MALL evicted before every launch")
    ap.add_argument("--soak", type=float, default=0.0, metavar="S",
                    help="GEMM and matrix-core probe back to back for S seconds each, with socket "
                         "power and shader clocks sampled by amd-smi")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-mix-probe", action="store_true",
                    help="skip the data-movement ceiling probes of the bf16 line")
    ap.add_argument("--probe-last", action="store_true",
                    help="run the ceiling probe after the timed region instead of before the warmup "
                         "(the timed region then starts from whatever clock state the warmup leaves)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (a reference for the HBM "
                         "byte counters when profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this GEMM path runs on one GPU only (--gpus %d requested); "
              "sharding across GPUs is not built" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from tiled_software_pipelined_amd import inputs, lib, metrics

    if args.lds_probe:
        lds_probe(torch, lib)
        return
    if args.mfma_probe:
        cases = [(dt, src, 256, 1) for dt in ("bf16", "i8") for src in ("random", "ones", "zeros")]
        cases += [("f32", src, wgs, w) for src in ("random", "ones") for w, wgs in F32_PROBE_WAVES.items()]
        # the default bf16 kernel's matrix stream at its 2 waves per SIMD:
        # bare, + its LDS fragment reads, + its direct copies (random operands)
        cases += [(dt, "random", 512, 2) for dt in ("bf16", "bf16_lds", "bf16_lds_dma")]
        for dt, src, wgs, waves in cases:
            rate, ghz, ms = mfma_ceiling(torch, lib, dt, src, workgroups=wgs)
            peak = PEAK_TFLOPS["bf16" if dt.startswith("bf16") else dt]
            print(json.dumps({"mode": "mfma_probe", "dtype": dt, "operands": src, "waves_per_simd": waves,
                              "rate": round(rate, 1), "unit": "TOP/s" if dt == "i8" else "TFLOP/s",
                              "frac_peak": round(rate / peak, 4), "clock_ghz": round(ghz, 3),
                              "median_ms": round(ms, 3)}), flush=True)
        return

    w = inputs.workloads()[args.workload]
    dev = torch.device("cuda:0")
    A_cpu, B_cpu = w.operands()
    A = A_cpu.to(dev)
    B = B_cpu.to(dev)
    out_dtype = torch.int32 if w.dtype == "i8" else torch.float32
    C = torch.empty((w.M, w.N), dtype=out_dtype, device=dev)
    torch.cuda.synchronize()

    if args.ladder:
        run_ladder(torch, lib, w, A, B, C, args)
    if args.variants:
        run_variants(torch, lib, w, A, B, C, args)
    if args.late_barrier:
        run_late_barrier(torch, lib, w, A, B, C, args)
        return
    if args.c_stores:
        run_c_stores(torch, lib, w, A, B, C)
        return
    if args.sweep:
        run_sweep(torch, lib, dev, args)

    if args.soak:
        soak(torch, lib, w, A, B, C, args.soak)
        return
    if args.cold:
        cold_timing(torch, lib, w, A, B, C, parse_variant(args.variant, lib))
        return

    if args.calib_copy:
        nbytes = args.calib_copy << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    variant = parse_variant(args.variant, lib)
    ceiling = None
    # bound by HBM rather than the arithmetic (the roofline's time for the
    # algorithmic bytes exceeds that for the flops): the thin products
    esz = {"f32": 4, "bf16": 2, "i8": 1}[w.dtype]
    hbm_bytes = metrics.algorithmic_bytes(w.M, w.N, w.K, esz, 4)
    hbm_bound = hbm_bytes / (PEAK_HBM_GBS * 1e9) > w.flops / (PEAK_TFLOPS[w.dtype] * 1e12)
    if not args.calib_copy and not args.probe_last and not hbm_bound:
        # The rate the arithmetic units sustain on this machine for the
        # workload's operand distribution with no memory traffic at all (the
        # power budget lowers the clock below nominal for random operands;
        # the fp32 rate grows with the waves per SIMD, 8 at most).  Measured
        # before the warmup steps: it also brings the shader clock out of its
        # idle state, which otherwise takes tens of milliseconds of load, so
        # that a short warmup does not leave the timed region on a ramping
        # clock.
        ceiling = mfma_ceiling(torch, lib, w.dtype, "random",
                               workgroups=256 if w.dtype != "f32" else F32_PROBE_WAVES[8])
    kernel_ms, wall = time_region(lib, torch, A, B, C, variant, args.steps, args.warmup)
    timing_mode = "eager"
    eager_ms = kernel_ms
    if kernel_ms < GRAPH_BELOW_MS:
        # launched one by one from here the GPU waits on the host between
        # kernels: time the same steps as one graph replay instead
        kernel_ms, wall, same = time_region_graph(lib, torch, A, B, C, variant, args.steps)
        if not same:
            raise RuntimeError("graph replay did not reproduce the eager result")
        timing_mode = "hip_graph"
    # after the timed region, one pass with a pair of events around every
    # launch: the per-launch distribution (median, min, max) of that pass
    per, _ = time_plan(lib, torch, w, A, B, C, variant, args.steps, 0)
    per_sorted = sorted(per)
    code = {"f32": lib.F32, "bf16": lib.BF16, "i8": lib.I8}[w.dtype]
    plan = lib.plan_for(w.M, w.N, w.K, code, w.K, w.N, w.N, variant)
    ms_step = wall * 1e3 / args.steps
    value = metrics.tflops(w.M, w.N, w.K, wall / args.steps)
    achieved = metrics.tflops(w.M, w.N, w.K, kernel_ms * 1e-3)
    peak = PEAK_TFLOPS[w.dtype]
    # HBM bytes per launch measured by the counter layer on these exact
    # kernel sources (profiles/*.md); null when none matches
    from tiled_software_pipelined_amd import provenance
    # the kernel that ran (the repacked plan's when operand rows were misaligned)
    kname = plan.kernel_for(A.data_ptr(), B.data_ptr(), workspace=variant is None)
    prof = provenance.find_profile(kname, w.name)
    traffic = None
    if prof and prof.get("traffic_bytes") not in (None, "null"):
        traffic = int(float(prof["traffic_bytes"]))
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS" if w.dtype == "i8" else "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": "%s GEMM M=%d N=%d K=%d" % (w.dtype, w.M, w.N, w.K),
                   "operands": w.kind, "seed": w.seed, "kernel": kname,
                   "grid": plan.info().grid, "frac_of_peak": round(value / peak, 4)},
        "roofline": {"bound": "mfma" if w.dtype != "f32" else "alu", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s" if w.dtype != "i8" else "TOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "algorithmic_bytes": hbm_bytes,
                     "traffic_unit": "bytes per launch between L2 and the memory fabric (FETCH_SIZE + "
                                     "WRITE_SIZE, copy-scaled): L2-miss bytes, which the 256 MB MALL may serve "
                                     "without reaching HBM",
                     "traffic_source": prof["path"] if prof else None,
                     "kernel_ms_mean": round(kernel_ms, 5),
                     "timing_mode": timing_mode, "eager_kernel_ms_mean": round(eager_ms, 5),
                     "per_launch_ms": {"median": round(per_sorted[len(per_sorted) // 2], 5),
                                       "min": round(per_sorted[0], 5), "max": round(per_sorted[-1], 5),
                                       "launches": len(per_sorted)},
                     "timing": "kernel_ms_mean (used for achieved): HIP events on the launch stream at the two "
                               "ends of the timed region / steps (timing_mode hip_graph: the steps replayed as one "
                               "HIP graph, for launches shorter than the host's launch path; eager_kernel_ms_mean "
                               "is the one-by-one figure); per_launch_ms: one further pass of the same "
                               "number of launches with a pair of events around each launch (the events add "
                               "their own commands between kernels, so these are slightly longer)"},
        "cpu_baseline": None,
        "env": env_record(torch, lib, dev),
    }
    if hbm_bound:
        # one read of A and B and one write of C per launch at the HBM peak
        gbps = hbm_bytes / (kernel_ms * 1e-3) / 1e9
        rec["roofline"].update({"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(gbps / PEAK_HBM_GBS, 4)})
    clk = clocked_rate(torch, lib, plan, A, B, C, variant)
    if clk is not None:
        at_clock = peak * clk["ghz"] / NOMINAL_GHZ
        rec["roofline"]["clock"] = {
            "ghz": round(clk["ghz"], 3), "peak_at_clock": round(at_clock, 1),
            "frac": round(achieved / at_clock, 4),
            "xcd_ghz": [round(x, 3) if x is not None else None for x in clk["xcd_ghz"]],
            "xcd_last_end_us": [round(x, 2) if x is not None else None for x in clk["xcd_last_end_us"]],
            "wg_loop_us": round(clk["wg_loop_us"], 2), "wg_store_us": round(clk["wg_store_us"], 2),
            "last_loop_end_us": round(clk["last_loop_end_us"], 2), "last_end_us": round(clk["last_end_us"], 2),
            "source": "s_memtime / s_memrealtime of every workgroup (start, end of its K loop, end) over %d "
                      "launches right after the timed region; peak scaled from %.1f GHz; per XCD (workgroup "
                      "mod 8): mean clock and time from the launch's first workgroup start to that XCD's last "
                      "end; wg_loop_us / wg_store_us: per-workgroup means of K loop and C write-back; "
                      "last_loop_end_us / last_end_us: from the first start to the last K-loop end / last "
                      "end" % (CLOCKED_LAUNCHES, NOMINAL_GHZ)}
    if not args.calib_copy and not hbm_bound:
        if ceiling is None:
            ceiling = mfma_ceiling(torch, lib, w.dtype, "random",
                                   workgroups=256 if w.dtype != "f32" else F32_PROBE_WAVES[8])
        rate, ghz, _ = ceiling
        unit = "matrix-core" if w.dtype != "f32" else "v_fmac_f32 (8 waves per SIMD)"
        rec["roofline"]["measured_ceiling"] = {
            "value": round(rate, 1), "clock_ghz": round(ghz, 3), "frac": round(achieved / rate, 4),
            "source": "%s rate probe, random %s operands, no memory traffic; run %s the warmup steps" % (
                unit, w.dtype, "after the timed region" if args.probe_last else "before")}
    if w.dtype == "bf16" and not args.calib_copy and not args.no_mix_probe and not hbm_bound:
        # the same matrix stream with the default kernel's on-chip data
        # movement and nothing else (no barrier, no C store): what the power
        # budget leaves once the LDS fragment reads and the direct copies are
        # paid for (the rate probe's kinds 3 and 4, 2 waves per SIMD)
        lds, ghz_l, _ = mfma_ceiling(torch, lib, "bf16_lds", "random", workgroups=512)
        mix, ghz_m, _ = mfma_ceiling(torch, lib, "bf16_lds_dma", "random", workgroups=512)
        bare, ghz_b, _ = mfma_ceiling(torch, lib, "bf16", "random", workgroups=512)
        rec["roofline"]["data_movement_ceiling"] = {
            "bare_2w": round(bare, 1), "bare_2w_ghz": round(ghz_b, 3),
            "with_lds_reads": round(lds, 1), "with_lds_reads_ghz": round(ghz_l, 3),
            "with_lds_reads_and_copies": round(mix, 1), "with_lds_reads_and_copies_ghz": round(ghz_m, 3),
            "frac": round(achieved / mix, 4),
            "source": "rate probe kinds 0 / 3 / 4 at 2 waves per SIMD, random bf16 operands: the default "
                      "kernel's matrix stream bare, with its LDS fragment reads, and with its direct "
                      "global->LDS copies as well; run after the timed region"}
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, A_cpu, B_cpu)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
