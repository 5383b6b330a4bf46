"""Sweep tool for the measured tile table (PR #142, "What this does", item
2: benchmark every configuration on the shapes you care about and write a
JSON table that the layer consults before its heuristic).

    python -m int8_weight_quantized_amd.tune --out table.json 80666x28672x5376 274x2048x2048 ...

For each m x n x k (bf16 output, per-row scales, bias, synthetic inputs of
int8_weight_quantized_amd.synth) it times every compiled tile at group_m 4,
then the three fastest tiles at group_m 1, 2, 4 and 8, with HIP events on
the current stream, and records the fastest configuration next to the
heuristic's own time.  A configuration replaces the heuristic's only when it
is faster by more than --min-gain (default 2 %, above the run-to-run noise);
otherwise the entry keeps the heuristic's choice.  The table is stamped with
the device architecture; the loader ignores it on any other.  A timing is
the median over 3 batches of the mean of --reps back-to-back launches,
after --warmup launches.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys


def _time_us(fn, warmup: int, reps: int) -> float:
    import torch
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / reps)
    return statistics.median(times)


def sweep_shape(m: int, n: int, k: int, warmup: int, reps: int, min_gain: float = 0.02,
                log=print) -> dict:
    import torch
    import int8_weight_quantized_amd as ck
    from int8_weight_quantized_amd import synth
    dev = torch.device("cuda:0")
    x, w, ws, b = synth.make_inputs(m, n, k, bias=True, seed=1, device=dev)
    w = ck.pad_rows(w)
    q, xs = ck.quantize_int8_rowwise(x)
    del x
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

    def run(tile, group):
        return lambda: ck.int8_linear_q(q, xs, w, ws, b, out=out, tile=tile, group_m=group)

    h_tile, _, _, h_group = ck.ck_int8_select_tile(m, n, k)
    timings = {}
    for tile in range(ck.CK_NUM_TILES):
        timings[(tile, 4)] = _time_us(run(tile, 4), warmup, reps)
    best3 = sorted(range(ck.CK_NUM_TILES), key=lambda t: timings[(t, 4)])[:3]
    for tile in best3:
        for group in (1, 2, 8):
            timings[(tile, group)] = _time_us(run(tile, group), warmup, reps)
    (tile, group), us = min(timings.items(), key=lambda kv: kv[1])
    heur = timings.get((h_tile, h_group))
    if heur is None:
        heur = _time_us(run(h_tile, h_group), warmup, reps)
        timings[(h_tile, h_group)] = heur
    if us > heur * (1.0 - min_gain):                   # within the noise: keep the heuristic
        tile, group, us = h_tile, h_group, heur
    entry = {"m": m, "n": n, "k": k, "tile": tile, "group_m": group, "us": round(us, 2),
             "tops": round(2.0 * m * n * k / us / 1e6, 1),
             "heuristic": [h_tile, h_group], "heuristic_us": round(heur, 2),
             "timings": {f"{t}/{g}": round(v, 2) for (t, g), v in sorted(timings.items())}}
    log(json.dumps({kk: entry[kk] for kk in ("m", "n", "k", "tile", "group_m", "us", "tops",
                                             "heuristic", "heuristic_us")}))
    del q, w, out
    torch.cuda.empty_cache()
    return entry


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("shapes", nargs="+", help="m x n x k, e.g. 80666x28672x5376")
    ap.add_argument("--out", required=True)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--min-gain", type=float, default=0.02)
    a = ap.parse_args(argv)
    import int8_weight_quantized_amd as ck
    from int8_weight_quantized_amd import tile_table
    os.environ["CK_INT8_TILE_TABLE"] = "off"          # time the library's own choices
    arch = tile_table.device_arch()
    ck.ck_int8_table_clear()
    entries = []
    for spec in a.shapes:
        m, n, k = (int(v) for v in spec.lower().split("x"))
        entries.append(sweep_shape(m, n, k, a.warmup, a.reps, a.min_gain,
                                   log=lambda s: print(s, flush=True)))
    table = {"arch": arch, "abi": ck.CK_ABI_VERSION,
             "note": "bf16 output, per-row scales, bias; HIP-event timings in us",
             "min_gain": a.min_gain,
             "entries": entries}
    with open(a.out, "w") as fh:
        json.dump(table, fh, indent=1)
        fh.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
