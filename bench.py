"""Benchmark of the INT8 linear layer on one MI355X.

A step is one pass of the whole layer over one batch already resident in
HBM: per-row (or tensor-wide) quantisation of x, then the int8 GEMM with
the fused dequant epilogue writing bf16.  Inputs are synthetic and seeded
(the recipe of the minimal reproduction in comfy-kitchen issue #136).

Prints ONE JSON line.  value = 2*m*n*k per step / wall time per step
(TOPS, whole layer); the GEMM kernel's own rate, measured with HIP events
on the launch stream around each GEMM launch in the timed region, is the
roofline's `achieved`.  The CPU oracle, timed on a bounded sample of rows of
the same workload, is reported as cpu_baseline.  After the timed steps the
GEMM runs back to back for --telemetry-seconds while amd-smi samples the
engine clock of each XCD and the socket power (`telemetry`).

`configs` holds every workload the layer is measured on (the headline one
included): its tile, the GEMM's median / mean launch time with TOPS and the
fraction of the dense INT8 peak from the median, the quantisation's rate,
and the oracle timed for at least a second on a row sample of it.
`roofline.mfma_alone` is the int8 matrix cores' rate with nothing else to
do (ck_mfma_ceiling mode 0: random operands in registers, products only) on
the same board, the most its power limit allows; `roofline.mfma_lds_alone`
adds the LDS reads of the operand fragments a GEMM main loop makes (mode 1)
and no global memory traffic.  `frac_of_mfma_alone` and
`frac_of_mfma_lds_alone` are the GEMM's rate over them.
`quantize.ceiling` compares the quantisation with a streaming kernel that
has its traffic and no arithmetic (ck_hbm_stream, the best of a small sweep
of its launch shape) on the same activations, both on their own and in the
step's position (right after the GEMM).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0     # MI355X dense INT8 matrix-core peak (published)
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak (published)
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E peak (published)
KERNEL_SRC = os.path.join(ROOT, "int8_weight_quantized_amd", "csrc", "ck_int8.hip")

# HBM traffic of one GEMM launch, from rocprofv3 --pmc FETCH_SIZE and
# --pmc WRITE_SIZE runs of this script (KiB per dispatch), each scaled by what
# the same counter reads for a plain 1 GiB device copy (--copy-calibration).
# Valid only for the kernel source it was measured on (sha256 below); any
# change to the source makes the reported traffic null until re-measured.
MEASURED_TRAFFIC = {
    "80666x28672x5376 per-row+bias": {
        "source_sha256": "6f47f398d586cde4ae3e3446fc4b9ec6217992d488f79cc1062086decf294143",
        "tile": 13, "group_m": 4,
        "fetch_bytes": 19760938330,   # FETCH_SIZE 9649107.31 KiB x 1.99996 (copy calibration)
        "write_bytes": 5967791328,    # WRITE_SIZE 5827921.22 KiB x 1.00000
    },
}

PAGES_A6000_TOPS = {        # the pages' own number for the same workload (context)
    "80666x28672x5376 per-row+bias": 2.0 * 80666 * 28672 * 5376 / 122.8e-3 / 1e12,
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4,
                    help="index into the workload list (default: 80666x28672x5376)")
    ap.add_argument("--tile", type=int, default=-1)
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--telemetry-seconds", type=float, default=3.0,
                    help="after the timed steps, issue the GEMM back to back this long while "
                         "sampling clocks and power with amd-smi (0: skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the CPU oracle sample (0: skip)")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the headline workload (no `configs` entries for the others)")
    ap.add_argument("--config-cpu-seconds", type=float, default=1.5,
                    help="oracle time per non-headline workload in `configs` (0: skip)")
    ap.add_argument("--rotation", type=str, default="",
                    help="comma-separated block sizes: also time the rotated per-row "
                         "quantisation of the workload's x for each; extra lines go to stderr")
    ap.add_argument("--dequant", action="store_true",
                    help="also time the dequant-on-the-fly (bf16) path on the workload; "
                         "an extra line goes to stderr")
    ap.add_argument("--decode", type=str, default="",
                    help="comma-separated row counts m: also time ck_int8_layer on m rows of the "
                         "workload's n x k weight, one kernel against the two kernels "
                         "(quantisation + GEMM), and the dequant-on-the-fly path on the same "
                         "rows; extra lines go to stderr")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times "
                         "(reference for the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def kernel_sha256():
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def measured_traffic(workload, tile, group_m):
    t = MEASURED_TRAFFIC.get(workload)
    if not t or t["source_sha256"] != kernel_sha256() or t["tile"] != tile or t["group_m"] != group_m:
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def gemm_kernel_name(r):
    """The GEMM kernel that ran: tile 13 runs its persistent kernel when k is
    a multiple of 128 and there are more tiles than compute units, otherwise
    the direct-to-LDS kernel of tile 12."""
    tiles = -(-r["m"] // r["bm"]) * -(-r["n"] // r["bn"])
    if r["tile"] == 13 and r["k"] % 128 == 0 and tiles > 256:
        return "gemm_persist_kernel"
    return "gemm_dma_kernel"


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "repeats": 3}), flush=True)


def sample_telemetry(run, seconds):
    """Engine clock per XCD and socket power while `run` (one GEMM launch)
    is issued back to back for about `seconds`: `amd-smi metric --power
    --clock --json` in a child process, sampled repeatedly after a 0.5 s
    ramp.  None when amd-smi is missing or returns nothing usable."""
    import shutil
    import statistics
    import subprocess
    import threading
    import torch
    exe = shutil.which("amd-smi")
    if exe is None or seconds <= 0:
        return None
    samples = []
    stop = threading.Event()

    def sampler():
        time.sleep(0.5)
        while not stop.is_set():
            try:
                res = subprocess.run([exe, "metric", "--power", "--clock", "--json"],
                                     capture_output=True, text=True, timeout=30)
                gpu = json.loads(res.stdout)["gpu_data"][0]
                clk = [gpu["clock"][f"gfx_{i}"]["clk"]["value"] for i in range(8)
                       if f"gfx_{i}" in gpu["clock"]]
                samples.append((float(gpu["power"]["socket_power"]["value"]),
                                [float(c) for c in clk]))
            except (OSError, ValueError, KeyError, IndexError, TypeError,
                    subprocess.SubprocessError):
                return

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            run()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=60)
    if not samples:
        return None
    nx = min(len(c) for _, c in samples)
    return {"tool": "amd-smi metric --power --clock --json", "samples": len(samples),
            "seconds": seconds,
            "socket_power_w": statistics.median(p for p, _ in samples),
            "gfx_clock_mhz_per_xcd": [statistics.median(c[i] for _, c in samples)
                                      for i in range(nx)]}


def _median_ms(launch, stream, steps, warmup, between=None):
    """Median HIP-event time of `launch` on `stream`; `between` (the GEMM,
    when given) runs after each timed launch, so the timed kernel starts
    where the quantisation starts in a step."""
    import torch
    for _ in range(warmup):
        launch()
        if between:
            between()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        launch()
        e1.record(stream)
        if between:
            between()
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) for e0, e1 in evs)[(steps - 1) // 2]


def kernel_ms(launch, stream, n=20, warmup=3):
    """HIP-event durations (ms, sorted) of `launch` issued n times back to
    back behind a GPU sleep, so that the host has enqueued every launch
    before the GPU reaches it: no host gap falls inside an interval.  For
    short kernels the Python host issues launches more slowly than the GPU
    runs them, and intervals in the step loop then include that gap."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda._sleep(int(5e6))
    for e0, e1 in evs:
        e0.record(stream)
        launch()
        e1.record(stream)
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) for e0, e1 in evs)


def queued_ms(step, stream, n=200, warmup=10):
    """Mean wall time (ms) of `step` issued n times back to back behind a GPU
    sleep: the host enqueues every step before the GPU reaches the first, so
    no host time falls between them (HIP events only around the whole run,
    none per step)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e7))
    e0.record(stream)
    for _ in range(n):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def mfma_ceiling(mode, reps=3, iters=100000):
    """Rate of ck_mfma_ceiling in `mode` (0: the int8 matrix cores with
    nothing else to do, 16 independent 32 x 32 x 32 products per wave and
    iteration on random register operands; 1: the same with every
    fragment read from LDS), about 60-80 ms per launch so that the board
    settles at its power limit; median of `reps` launches after one."""
    import torch
    import int8_weight_quantized_amd as ck
    dev = torch.device("cuda:0")
    out = torch.empty((256 * 512,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ms = _median_ms(lambda: ck.ck_mfma_ceiling(iters, mode, out.data_ptr(), 1, stream.cuda_stream),
                    stream, reps, 1)
    ops = 2.0 * 256 * 8 * 16 * iters * 32768      # blocks, waves, products, MACs
    return {"kernel": "mfma_ceiling_kernel<%d>" % mode, "iters": iters, "ms_median": ms,
            "tops": ops / (ms * 1e-3) / 1e12}


def stream_ceiling(x, q, steps, warmup, quantize, gemm):
    """The quantisation against ck_hbm_stream (its reads and writes,
    streamed, without its arithmetic) over the same x -> q.  The streaming
    kernel's launch shape is the best of a small sweep, run on its own; then
    both kernels are timed on their own (back to back) and in the step's
    position (each launch followed by the GEMM, as the quantisation is in a
    step, where the GEMM before it has left the clock lowered and the
    caches full of its output)."""
    import torch
    import int8_weight_quantized_amd as ck
    stream = torch.cuda.current_stream(x.device)
    sh = stream.cuda_stream
    chunks = x.numel() // 8
    nbytes = 16.0 * chunks + 8.0 * chunks
    sweep = []
    for unroll in (2, 4, 8):
        for per_cu in (2, 4, 8, 16):
            blocks = 256 * per_cu
            ms = _median_ms(lambda: ck.ck_hbm_stream(x.data_ptr(), chunks, q.data_ptr(), blocks,
                                                      unroll, sh), stream, steps, warmup)
            sweep.append((nbytes / (ms * 1e-3) / 1e9, unroll, blocks))
    gbps, unroll, blocks = max(sweep)

    def hbm():
        ck.ck_hbm_stream(x.data_ptr(), chunks, q.data_ptr(), blocks, unroll, sh)

    res = {"kernel": "hbm_stream_kernel", "unroll": unroll, "blocks": blocks, "bytes": nbytes}
    for name, fn in (("stream", hbm), ("quantize", quantize)):
        alone = _median_ms(fn, stream, steps, warmup)
        in_step = _median_ms(fn, stream, max(10, steps // 2), 2, between=gemm)
        res[f"{name}_alone_us"] = alone * 1e3
        res[f"{name}_alone_GBps"] = nbytes / (alone * 1e-3) / 1e9
        res[f"{name}_in_step_us"] = in_step * 1e3
        res[f"{name}_in_step_GBps"] = nbytes / (in_step * 1e-3) / 1e9
    quantize()                       # leave the codes in q
    torch.cuda.synchronize()
    return res


def time_workload(idx, steps, warmup, tile=-1, group_m=0, telemetry_s=0.0, quantize_ceiling=False):
    import torch
    import int8_weight_quantized_amd as ck
    from int8_weight_quantized_amd import synth

    wl = synth.WORKLOADS[idx]
    m, n, k, mode = wl["m"], wl["n"], wl["k"], wl["mode"]
    dev = torch.device("cuda:0")
    x, w, ws, b = synth.make_inputs(m, n, k, mode=mode, bias=wl["bias"],
                                    seed=synth.workload_seed(idx), device=dev)
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    xs = torch.empty((m if mode == "row" else 1,), dtype=torch.float32, device=dev)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    ck_mode = ck.CK_SCALE_ROW if mode == "row" else ck.CK_SCALE_TENSOR
    bias_ptr = 0 if b is None else b.data_ptr()
    if tile < 0:
        from int8_weight_quantized_amd import tile_table
        tile_table.ensure_loaded(dev)             # the measured table, as the layer uses it
        tile_id, bm, bn, g = ck.ck_int8_select_tile(m, n, k)
    else:
        tile_id = tile
        bm, bn, _ = ck.ck_int8_tile_info(tile)
        g = 8
    if group_m > 0:
        g = group_m
    sh = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ck.ck_quantize_int8_rowwise(x.data_ptr(), m, k, k, q.data_ptr(), k, xs.data_ptr(),
                                    ck_mode, sh)
        if ev is not None:
            ev[1].record(stream)
        ck.ck_int8_linear_tiled(q.data_ptr(), k, xs.data_ptr(), ck_mode, w.data_ptr(), k,
                                ws.data_ptr(), ck_mode, bias_ptr, out.data_ptr(), n, m, n, k,
                                tile_id, g, sh)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    qz_ms = [e[0].elapsed_time(e[1]) for e in evs]
    gm_ms = [e[1].elapsed_time(e[2]) for e in evs]
    qz_sorted = sorted(qz_ms)
    ops = 2.0 * m * n * k
    qz_bytes = 2.0 * m * k + 1.0 * m * k + 4.0 * (m if mode == "row" else 1)
    gm_sorted = sorted(gm_ms)
    res = {
        "workload": wl["name"], "m": m, "n": n, "k": k, "mode": mode, "bias": wl["bias"],
        "tile": tile_id, "bm": bm, "bn": bn, "group_m": g,
        "wall_ms_per_step": wall * 1e3 / steps,
        "gemm_ms": sum(gm_ms) / steps,
        "gemm_ms_p20": gm_sorted[int(0.2 * (steps - 1))],
        "gemm_ms_p50": gm_sorted[int(0.5 * (steps - 1))],
        "gemm_ms_p80": gm_sorted[int(0.8 * (steps - 1))],
        "quantize_ms": sum(qz_ms) / steps,
        "quantize_ms_p50": qz_sorted[int(0.5 * (steps - 1))],
        "ops": ops, "quantize_bytes": qz_bytes,
    }
    res["gemm_tops"] = ops / (res["gemm_ms"] * 1e-3) / 1e12
    res["gemm_frac_of_peak"] = res["gemm_tops"] / INT8_PEAK_TOPS
    res["quantize_gbps"] = qz_bytes / (res["quantize_ms"] * 1e-3) / 1e9
    res["step_tops"] = ops / (res["wall_ms_per_step"] * 1e-3) / 1e12
    # algorithmic bytes of the GEMM: q + W + scales + bias + bf16 out
    res["gemm_bytes"] = (m * k + n * k + 4.0 * (m + n) + (2.0 * n if wl["bias"] else 0)
                         + 2.0 * m * n)

    def gemm():
        ck.ck_int8_linear_tiled(q.data_ptr(), k, xs.data_ptr(), ck_mode, w.data_ptr(), k,
                                ws.data_ptr(), ck_mode, bias_ptr, out.data_ptr(), n, m, n, k,
                                tile_id, g, sh)

    def quantize_only():
        ck.ck_quantize_int8_rowwise(x.data_ptr(), m, k, k, q.data_ptr(), k, xs.data_ptr(), ck_mode, sh)

    kg = kernel_ms(gemm, stream)
    kq = kernel_ms(quantize_only, stream)
    # the step issued back to back without per-step events (the timed loop
    # above records three events per step, which for the small workloads
    # costs more host time than the GPU spends on the step)
    res["step_ms_queued"] = queued_ms(step, stream, n=max(20, min(200, int(200.0 / max(res["wall_ms_per_step"], 1e-3)))))
    res["gemm_kernel_ms_median"] = kg[(len(kg) - 1) // 2]
    res["gemm_kernel_ms_mean"] = sum(kg) / len(kg)
    res["quantize_kernel_ms_median"] = kq[(len(kq) - 1) // 2]
    res["telemetry"] = sample_telemetry(gemm, telemetry_s)
    if quantize_ceiling:
        def quantize():
            ck.ck_quantize_int8_rowwise(x.data_ptr(), m, k, k, q.data_ptr(), k, xs.data_ptr(),
                                        ck_mode, sh)
        res["quantize_ceiling"] = stream_ceiling(x, q, steps, warmup, quantize, gemm)
    del x, w, ws, b, q, xs, out
    torch.cuda.empty_cache()
    return res


def time_dequant(idx, steps, warmup):
    """The dequant-on-the-fly path (bf16 x times the int8 weight dequantised
    to bf16 on its way into LDS, on the bf16 matrix cores) on the same
    workload: one launch per step, HIP events on its launch stream."""
    import torch
    import int8_weight_quantized_amd as ck
    from int8_weight_quantized_amd import synth

    wl = synth.WORKLOADS[idx]
    m, n, k = wl["m"], wl["n"], wl["k"]
    dev = torch.device("cuda:0")
    x, w, ws, b = synth.make_inputs(m, n, k, mode=wl["mode"], bias=wl["bias"],
                                    seed=synth.workload_seed(idx), device=dev)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    w_mode = ck.CK_SCALE_ROW if ws.numel() == n else ck.CK_SCALE_TENSOR
    bias_ptr = 0 if b is None else b.data_ptr()

    def call():
        ck.ck_int8_linear_dequant(x.data_ptr(), k, w.data_ptr(), k, ws.data_ptr(), w_mode,
                                  bias_ptr, out.data_ptr(), n, ck.CK_OUT_BF16, m, n, k, sh)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    mean = sum(ms) / steps
    flops = 2.0 * m * n * k
    tiles = -(-m // 256) * -(-n // 256)
    res = {"workload": wl["name"], "path": "dequant (bf16 MFMA)", "steps": steps,
           "kernel": "gemm_dq_persist_kernel" if tiles > 256 else "gemm_dq_kernel",
           "ms": mean, "ms_p20": ms[int(0.2 * (steps - 1))], "ms_p80": ms[int(0.8 * (steps - 1))],
           "tflops": flops / (mean * 1e-3) / 1e12}
    res["frac_of_bf16_peak"] = res["tflops"] / BF16_PEAK_TFLOPS
    del x, w, ws, b, out
    torch.cuda.empty_cache()
    return res


def time_rotation(idx, block, steps, warmup):
    """Quantisation of the workload's x after the online Hadamard rotation of
    block size `block`: per row (one launch per step) and tensor-wide (the
    amax pass and the code pass per step), HIP events on the launch stream."""
    import torch
    import int8_weight_quantized_amd as ck
    from int8_weight_quantized_amd import synth

    wl = synth.WORKLOADS[idx]
    m, k = wl["m"], wl["k"]
    dev = torch.device("cuda:0")
    x, _, _, _ = synth.make_inputs(m, 1, k, mode="row", seed=synth.workload_seed(idx), device=dev)
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    s = torch.empty((m,), dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream(dev).cuda_stream
    stream = torch.cuda.current_stream(dev)

    def timed(mode):
        def call():
            ck.ck_quantize_int8_rotated(x.data_ptr(), m, k, k, block, q.data_ptr(), k, s.data_ptr(),
                                        mode, sh)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for e0, e1 in evs:
            e0.record(stream)
            call()
            e1.record(stream)
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)

    us = timed(ck.CK_SCALE_ROW)
    ut = timed(ck.CK_SCALE_TENSOR)
    mean = sum(us) / steps
    nbytes = 3.0 * m * k + 4.0 * m
    del x, q, s
    torch.cuda.empty_cache()
    return {"workload": f"{m}x{k} activations of {wl['name']}", "path": "rotated quantisation",
            "block": block, "steps": steps, "us": mean, "us_p20": us[int(0.2 * (steps - 1))],
            "us_p80": us[int(0.8 * (steps - 1))], "rate_GBps": nbytes / (mean * 1e-6) / 1e9,
            "tensor_us": sum(ut) / steps, "tensor_us_p20": ut[int(0.2 * (steps - 1))],
            "tensor_us_p80": ut[int(0.8 * (steps - 1))]}


def time_decode(idx, m, reps=200):
    """The whole layer (ck_int8_layer) on m rows of the workload's weight,
    per call with the launches queued back to back behind a GPU sleep (so
    no host gap falls inside), once as one kernel (fused=1) and once as
    the quantisation kernel + the GEMM (fused=0); outputs compared.  Then
    the dequant-on-the-fly path (ck_int8_linear_dequant) on the same x and
    weight, timed the same way."""
    import torch
    import int8_weight_quantized_amd as ck
    from int8_weight_quantized_amd import synth

    wl = synth.WORKLOADS[idx]
    n, k = wl["n"], wl["k"]
    dev = torch.device("cuda:0")
    x, w, ws, b = synth.make_inputs(m, n, k, mode="row", bias=wl["bias"],
                                    seed=synth.workload_seed(idx) + m, device=dev)
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    xs = torch.empty((m,), dtype=torch.float32, device=dev)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    bias = 0 if b is None else b.data_ptr()
    res, outs = {"workload": f"{m}x{n}x{k} (weight of {wl['name']})", "path": "ck_int8_layer"}, {}
    for fused in (1, 0):
        def call():
            ck.ck_int8_layer(x.data_ptr(), k, q.data_ptr(), k, xs.data_ptr(), ck.CK_SCALE_ROW,
                             w.data_ptr(), k, ws.data_ptr(), ck.CK_SCALE_ROW, bias, out.data_ptr(),
                             n, ck.CK_OUT_BF16, m, n, k, fused, stream.cuda_stream)
        for _ in range(20):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(2e7))
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res["one_kernel_us" if fused else "two_kernels_us"] = us
        outs[fused] = out.clone()
    res["speedup"] = res["two_kernels_us"] / res["one_kernel_us"]
    res["identical"] = bool(torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)))
    res["weight_GBps_one_kernel"] = n * k / (res["one_kernel_us"] * 1e-6) / 1e9

    # the dequant-on-the-fly (W8A16) path on the same rows and weight
    def call_dq():
        ck.ck_int8_linear_dequant(x.data_ptr(), k, w.data_ptr(), k, ws.data_ptr(), ck.CK_SCALE_ROW,
                                  bias, out.data_ptr(), n, ck.CK_OUT_BF16, m, n, k, stream.cuda_stream)
    for _ in range(20):
        call_dq()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e7))
    e0.record(stream)
    for _ in range(reps):
        call_dq()
    e1.record(stream)
    torch.cuda.synchronize()
    res["dequant_us"] = e0.elapsed_time(e1) * 1e3 / reps
    res["weight_GBps_dequant"] = n * k / (res["dequant_us"] * 1e-6) / 1e9
    del x, w, ws, b, q, xs, out, outs
    torch.cuda.empty_cache()
    return res


def cpu_baseline(idx, target_s):
    """The oracle (quantise + integer product + epilogue) on a bounded row
    sample of the same workload, on this host's cores."""
    import numpy as np
    import torch
    import oracle
    from int8_weight_quantized_amd import synth

    wl = synth.WORKLOADS[idx]
    m, n, k, mode = wl["m"], wl["n"], wl["k"], wl["mode"]
    x, w, ws, b = synth.make_inputs(m, n, k, mode=mode, bias=wl["bias"],
                                    seed=synth.workload_seed(idx), device="cuda:0")
    w_h = w.cpu().numpy()
    ws_h = ws.cpu().numpy()
    b_h = None if b is None else b.view(torch.int16).cpu().numpy().view(np.uint16)

    def run(rows):
        xb = x[:rows].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        if mode == "row":
            qo, so = oracle.quantize_rowwise(xb)
        else:
            qo, so = oracle.quantize_tensorwise(xb)
        oracle.linear(qo, so, w_h, ws_h, b_h)
        return time.perf_counter() - t0

    rows = min(m, 8)
    dt = run(rows)
    rows = max(min(m, 8), min(m, int(rows * target_s / max(dt, 1e-3))))
    reps, dt = 0, 0.0
    while reps == 0 or dt < target_s:          # the whole of a small workload, repeated
        dt += run(rows)
        reps += 1
    what = "tensor-wide scale of the sample" if mode == "tensor" else "per-row scales"
    return {"value": 2.0 * rows * n * k * reps / dt / 1e12, "unit": "TOPS",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {rows} of {m} rows x all {n} columns, k={k}"
                      f"{f', {reps} runs' if reps > 1 else ''} (quantise with {what}"
                      f" + int32 product + epilogue), {dt:.1f} s"}


def config_entry(r, cpu):
    """One workload's figures for the `configs` object.  gemm_ms_* and
    quantize_us_step are HIP-event times inside the timed steps; TOPS,
    the fraction of peak and the quantisation rate come from the kernels'
    median durations issued back to back (kernel_ms), which for the short
    workloads leave out the host's launch gaps."""
    tops = r["ops"] / (r["gemm_kernel_ms_median"] * 1e-3) / 1e12
    return {"workload": r["workload"], "tile": r["tile"], "block": f"{r['bm']}x{r['bn']}",
            "group_m": r["group_m"], "gemm_kernel": gemm_kernel_name(r),
            "gemm_kernel_ms_median": r["gemm_kernel_ms_median"],
            "gemm_kernel_ms_mean": r["gemm_kernel_ms_mean"],
            "gemm_ms_median": r["gemm_ms_p50"], "gemm_ms_mean": r["gemm_ms"],
            "gemm_ms_p20": r["gemm_ms_p20"], "gemm_ms_p80": r["gemm_ms_p80"],
            "gemm_tops": tops, "frac": tops / INT8_PEAK_TOPS,
            "quantize_us_median": r["quantize_kernel_ms_median"] * 1e3,
            "quantize_GBps": r["quantize_bytes"] / (r["quantize_kernel_ms_median"] * 1e-3) / 1e9,
            "quantize_us_step": r["quantize_ms_p50"] * 1e3,
            "step_ms": r["wall_ms_per_step"], "step_tops": r["step_tops"],
            "step_ms_queued": r["step_ms_queued"],
            "step_tops_queued": r["ops"] / (r["step_ms_queued"] * 1e-3) / 1e12,
            "cpu_baseline": cpu}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU only; there is no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    import int8_weight_quantized_amd as ck
    ck.lib()

    from int8_weight_quantized_amd import synth
    configs = {}
    if not args.no_configs:
        for i in range(len(synth.WORKLOADS)):
            if i == args.workload:
                continue
            # at least 20 timed steps after 10 warm-ups: the shorter workloads'
            # GEMM times spread by several percent from step to step
            r = time_workload(i, max(20, args.steps), 10)
            cpu = (cpu_baseline(i, args.config_cpu_seconds)
                   if args.config_cpu_seconds > 0 else None)
            configs[f"c{i}"] = config_entry(r, cpu)
            print(json.dumps({"config": f"c{i}", **configs[f"c{i}"]}), file=sys.stderr, flush=True)

    if args.dequant:
        d = time_dequant(args.workload, args.steps, args.warmup)
        print(json.dumps({"extra": d}), file=sys.stderr, flush=True)
    for blk in [int(v) for v in args.rotation.split(",") if v]:
        d = time_rotation(args.workload, blk, args.steps, args.warmup)
        print(json.dumps({"extra": d}), file=sys.stderr, flush=True)
    for rows in [int(v) for v in args.decode.split(",") if v]:
        d = time_decode(args.workload, rows)
        print(json.dumps({"extra": d}), file=sys.stderr, flush=True)

    r = time_workload(args.workload, args.steps, args.warmup, args.tile, args.group_m,
                      telemetry_s=args.telemetry_seconds, quantize_ceiling=True)
    wl = synth.WORKLOADS[args.workload]
    base = PAGES_A6000_TOPS.get(wl["name"])
    cpu = cpu_baseline(args.workload, args.cpu_seconds) if args.cpu_seconds > 0 else None
    configs[f"c{args.workload}"] = config_entry(r, cpu)
    mc = mfma_ceiling(0)
    ml = mfma_ceiling(1)
    configs = {key: configs[key] for key in sorted(configs)}
    qc = r["quantize_ceiling"]
    qz_gbps = r["quantize_bytes"] / (r["quantize_ms_p50"] * 1e-3) / 1e9
    line = {
        "metric": "INT8 GEMM TOPS (+% of MI355X INT8 MFMA peak) at "
                  f"{r['m']}x{r['n']}x{r['k']}",
        "value": r["step_tops"],
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["wall_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (r["step_tops"] / base) if base else None,
        "vs_baseline_basis": ("value / 202.5 TOPS, the rate derived from the pages' 122.8 ms "
                              "for this workload on an RTX A6000 (other hardware: context)"
                              if base else None),
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl["name"], "m": r["m"], "n": r["n"], "k": r["k"],
                   "x_scale": "per-row" if r["mode"] == "row" else "tensor",
                   "w_scale": "per-column" if r["mode"] == "row" else "tensor",
                   "bias": r["bias"], "out": "bf16", "tile": r["tile"],
                   "block": f"{r['bm']}x{r['bn']}", "group_m": r["group_m"],
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": r["gemm_tops"], "peak": INT8_PEAK_TOPS,
                     "unit": "TOPS", "frac": r["gemm_tops"] / INT8_PEAK_TOPS,
                     "traffic": measured_traffic(wl["name"], r["tile"], r["group_m"]),
                     "traffic_unit": "bytes per launch",
                     "kernel": gemm_kernel_name(r) + " (int8 GEMM + fused epilogue)",
                     "gemm_ms": r["gemm_ms"], "gemm_ms_p20": r["gemm_ms_p20"],
                     "gemm_ms_p50": r["gemm_ms_p50"], "gemm_ms_p80": r["gemm_ms_p80"],
                     "gemm_kernel_ms_median_back_to_back": r["gemm_kernel_ms_median"],
                     "mfma_alone": mc,
                     "frac_of_mfma_alone": r["gemm_tops"] / mc["tops"],
                     "mfma_lds_alone": ml,
                     "frac_of_mfma_lds_alone": r["gemm_tops"] / ml["tops"]},
        "telemetry": r["telemetry"],
        "quantize": {"ms": r["quantize_ms"], "us_median": r["quantize_ms_p50"] * 1e3,
                     "GBps": qz_gbps, "frac_hbm": qz_gbps / HBM_PEAK_GBPS,
                     "ceiling": qc,
                     "frac_ceiling_in_step": qc["quantize_in_step_GBps"] / qc["stream_in_step_GBps"],
                     "frac_ceiling_alone": qc["quantize_alone_GBps"] / qc["stream_alone_GBps"]},
        "gemm_tops": r["gemm_tops"],
        "configs": configs,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
