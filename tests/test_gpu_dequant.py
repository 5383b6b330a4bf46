"""The dequant-on-the-fly path (#278, "Suggested fix": the int8 weight
dequantised to the 16-bit compute type on the fly, bf16 matrix cores, x not
quantised), HIP path vs the CPU oracle.

The hardware sums the exact fp32 products in fp32 in an order of its own,
so the bar is the accumulation bound rather than bit equality: for every
output, |got - (S + bias)| <= k * 2^-24 * A + 2^-23 |S + bias| + 1 ulp of the
output type, with S and A = sum |x * wdq| from the oracle (the fp32 bias
add and the final rounding account for the last two terms).  The tests
also report how many outputs are bit-identical to the oracle's rounding of
the exact sum."""
import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import bits16, cuda_device

pytestmark = pytest.mark.gpu


def _values(arr, out_dtype):
    if out_dtype == "fp32":
        return arr.astype(np.float64)
    if out_dtype == "fp16":
        return arr.view(np.float16).astype(np.float64)
    return oracle.bf16_to_f32(arr).astype(np.float64)


def _ulp(v, out_dtype):
    mant, emin = {"bf16": (7, -126), "fp16": (10, -14), "fp32": (23, -126)}[out_dtype]
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** emin)))
    return np.exp2(e - mant)


def _check(m, n, k, out_dtype, bias, mode="row", seed=0):
    import torch
    dev = cuda_device()
    x, w, ws, b = synth.make_inputs(m, n, k, mode=mode, bias=bias, seed=seed, device=dev)
    w = ck.pad_rows(w)
    bt = None if b is None else b.to({"bf16": torch.bfloat16, "fp16": torch.float16,
                                      "fp32": torch.float32}[out_dtype])
    out = ck.int8_linear_dequant(x, w, ws, bt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    bo = None if bt is None else (bt.cpu().numpy() if out_dtype == "fp32" else bits16(bt))
    ref, s, a = oracle.linear_dequant(bits16(x), w.cpu().numpy(), ws.cpu().numpy(), bo, out_dtype)
    got = out.cpu().numpy() if out_dtype == "fp32" else bits16(out)
    g = _values(got, out_dtype)
    exact = s + (0.0 if bo is None else _values(bo, out_dtype)[None, :])
    tol = k * 2.0 ** -24 * a + 2.0 ** -23 * np.abs(exact) + _ulp(np.maximum(np.abs(exact), np.abs(g)), out_dtype)
    bad = np.abs(g - exact) > tol
    assert not bad.any(), (f"{bad.sum()} outputs outside the bound; worst excess "
                           f"{float(np.max(np.abs(g - exact) - tol))}")
    same = float(np.mean(got.view(np.uint32 if out_dtype == "fp32" else np.uint16) ==
                         ref.view(np.uint32 if out_dtype == "fp32" else np.uint16)))
    return same


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("m,n,k,bias", [(300, 520, 2048, True), (257, 255, 1000, False),
                                        (1, 40, 64, True), (64, 96, 8, True), (33, 70, 4104, False)])
def test_dequant_small_blocks(out_dtype, m, n, k, bias):
    same = _check(m, n, k, out_dtype, bias, seed=m + k)
    assert same > (0.9 if out_dtype != "fp32" else 0.0), same


# Up to 64 rows run the few-row kernel: 32 columns per block, K split over
# 8 or 4 waves by the number of column blocks (n under 8192: 8; 16,424 and
# 28,672: 4), one, two, four or eight x loads
# per chunk (up to 8, 16, 32 or 64 rows).  Ragged columns, K tails of 8 to
# 56 elements (x rows are contiguous here, so k is a multiple of 8; the
# strided test below has a tail of 28), K shorter than one 64-element
# chunk, fewer chunks than waves, 16, 17, 24, 32, 33, 48 and 64 rows.
@pytest.mark.parametrize("out_dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("m,n,k,bias", [(1, 4160, 5376, True), (2, 130, 24, False), (7, 70, 40, True),
                                        (5, 300, 1000, True), (16, 16424, 4104, False),
                                        (3, 16424, 4104, True), (12, 28672, 2048, True),
                                        (2, 28672, 1000, False), (1, 28672, 5376, True),
                                        (16, 28672, 96, True), (9, 4096, 4160, False),
                                        (24, 28672, 2048, True), (32, 16424, 1000, False),
                                        (17, 300, 4104, True), (33, 28672, 1000, True),
                                        (48, 16424, 2048, False), (64, 300, 4104, True)])
def test_dequant_few_rows(out_dtype, m, n, k, bias):
    same = _check(m, n, k, out_dtype, bias, seed=m * 3 + k)
    assert same > (0.9 if out_dtype != "fp32" else 0.0), same


@pytest.mark.parametrize("n", [1000, 28672])
def test_dequant_few_rows_path_strides_and_tensor_scale(n, capfd):
    """m <= 64 logs the few-row kernel and m = 65 does not; x rows wider
    than k, W rows padded past k with nonzero bytes and output rows wider
    than n give the same bits as buffers padded with zeros and leave the
    output padding alone (8 waves a block with n = 1000, 4 with
    n = 28672); a tensor-wide scale stays inside the bound."""
    import torch
    dev = cuda_device()
    _check(3, 500, 704, "bf16", True, mode="tensor", seed=21)
    ck.ck_int8_set_path_log(True)
    try:
        kk = 160 if n == 1000 else 192           # the log has one line per shape
        for m, nn in ((64, 96), (65, 96), (1, 28672)):
            x, w, ws, _ = synth.make_inputs(m, nn, kk, seed=m, device=dev)
            capfd.readouterr()
            ck.int8_linear_dequant(x, w, ws)
            torch.cuda.synchronize()
            err = capfd.readouterr().err
            line = [l for l in err.splitlines() if f"gemm_dequant {m}x{nn}x{kk} " in l]
            assert line and (("few rows" in line[0]) == (m <= 64)), err
    finally:
        ck.ck_int8_set_path_log(False)
    m, k = 9, 1500
    xw, w, ws, b = synth.make_inputs(m, n, k + 44, bias=True, seed=5, device=dev)
    x = xw[:, :k]                                          # row stride 1544 elements
    wpad = torch.full((n, 1520), 5, dtype=torch.int8, device=dev)
    wpad[:, :k] = w[:, :k]
    wv = wpad[:, :k]                                       # bytes 1500 .. 1503 of each row are 5
    ofull = torch.full((m, n + 24), 7.0, dtype=torch.bfloat16, device=dev)
    out = ofull[:, :n]
    ck.int8_linear_dequant(x, wv, ws, b, out=out)
    xz = torch.zeros((m, 1504), dtype=torch.bfloat16, device=dev)   # zeros past k
    xz[:, :k] = x
    ref = ck.int8_linear_dequant(xz[:, :k], ck.pad_rows(w[:, :k].contiguous()), ws, b)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert bool((ofull[:, n:] == 7.0).all())
    ro, s, a = oracle.linear_dequant(bits16(x.contiguous()), w[:, :k].cpu().numpy(), ws.cpu().numpy(),
                                     bits16(b), "bf16")
    g = _values(bits16(out), "bf16")
    exact = s + _values(bits16(b), "bf16")[None, :]
    tol = k * 2.0 ** -24 * a + 2.0 ** -23 * np.abs(exact) + _ulp(np.maximum(np.abs(exact), np.abs(g)), "bf16")
    assert not (np.abs(g - exact) > tol).any()


@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_dequant_large_blocks_ragged(out_dtype):
    """17 x 16 tiles of 256 x 256 (the large-block kernel), ragged m, K tail."""
    same = _check(4100, 4096, 200, out_dtype, True, seed=3)
    assert same > (0.9 if out_dtype == "bf16" else 0.0), same


def test_dequant_tensor_scale_and_k_zero():
    import torch
    _check(200, 300, 768, "bf16", True, mode="tensor", seed=4)
    dev = cuda_device()
    x = torch.empty((5, 0), dtype=torch.bfloat16, device=dev)
    w = torch.empty((24, 0), dtype=torch.int8, device=dev)
    b = (torch.arange(24, device=dev, dtype=torch.float32) * 0.25 - 2).to(torch.bfloat16)
    out = ck.int8_linear_dequant(x, w, torch.ones(24, device=dev), b)
    torch.cuda.synchronize()
    assert torch.equal(out, b.expand(5, 24))


def test_dequant_beats_int8_layer_accuracy():
    """x unquantised: closer to x (w * ws)^T than the int8 layer."""
    import torch
    dev = cuda_device()
    m, n, k = 512, 768, 2048
    x, w, ws, _ = synth.make_inputs(m, n, k, seed=8, device=dev)
    ref = x.double() @ (w.double() * ws.double()[:, None]).t()
    dq = ck.int8_linear_dequant(x, w, ws)
    i8 = ck.int8_linear(x, w, ws)
    e_dq = float((dq.double() - ref).norm() / ref.norm())
    e_8 = float((i8.double() - ref).norm() / ref.norm())
    assert e_dq < 0.005 and e_dq < 0.6 * e_8, (e_dq, e_8)


def test_dequant_persistent_walk_and_shared_counters():
    """19 x 18 = 342 tiles: one block per CU claims tiles (the counters of the
    stream, which the int8 persistent GEMM on the same stream also uses).
    fp16 output with bias against the oracle's bound, then dequant and int8
    launches interleaved on one stream and on two, each dequant result the
    same bits as the first."""
    import torch
    same = _check(4700, 4568, 320, "fp16", True, seed=12)
    assert same > 0.9, same
    dev = cuda_device()
    m, n, k = 4700, 4568, 320
    x, w, ws, b = synth.make_inputs(m, n, k, bias=True, seed=13, device=dev)
    ref = ck.int8_linear_dequant(x, w, ws, b)
    q, xs = ck.quantize_int8_rowwise(x)
    ref8 = ck.int8_linear_q(q, xs, w, ws, b, tile=12)
    outs = []
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for st in (None, None, s1, s2):
        with torch.cuda.stream(st if st is not None else torch.cuda.current_stream()):
            outs.append((ck.int8_linear_dequant(x, w, ws, b), ck.int8_linear_q(q, xs, w, ws, b, tile=13)))
    torch.cuda.synchronize()
    for i, (od, o8) in enumerate(outs):
        assert torch.equal(od.view(torch.int16), ref.view(torch.int16)), i
        assert torch.equal(o8.view(torch.int16), ref8.view(torch.int16)), i


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16"])
def test_dequant_output_layouts_agree(out_dtype):
    """16-bit outputs of interior tiles with 16-byte aligned rows go through
    an LDS-staged epilogue (whole row segments); rows that are only 8-byte
    aligned, or not aligned at all, are stored from the accumulators.  One
    product (persistent 256x256 blocks, edge tiles on both sides) written
    to a contiguous output, to one with rows 4 elements longer and to one
    with rows 1 element longer gives the same bits, leaves the padding
    alone, and stays inside the accumulation bound."""
    import torch
    dev = cuda_device()
    m, n, k = 4136, 4104, 256
    _check(m, n, k, out_dtype, True, seed=77)
    x, w, ws, b = synth.make_inputs(m, n, k, bias=True, seed=77, device=dev)
    w = ck.pad_rows(w)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[out_dtype]
    bt = b.to(tdt)
    ref = ck.int8_linear_dequant(x, w, ws, bt, out_dtype=out_dtype)
    for pad in (4, 1):
        buf = torch.full((m, n + pad), 7.0, dtype=tdt, device=dev)
        out = buf[:, :n]
        ck.int8_linear_dequant(x, w, ws, bt, out=out, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), pad
        assert bool((buf[:, n:] == 7.0).all()), pad


def _dequant_rows(m, n, k, seed):
    """About 80-125 output rows: the first and last 8, +-4 around every 32-bit
    wrap boundary inside m, the first 32 rows holding elements past 2^31, and
    64 seeded uniform rows (the fp64 oracle takes ~0.1 s per row here)."""
    rows = set(range(8)) | set(range(m - 8, m))
    for r in synth.boundary_rows(m, n, k).values():
        if r < m:
            rows.update(range(max(0, r - 4), min(m, r + 4)))
    r31 = synth.boundary_rows(m, n, k)["out_elem_2^31"]
    if r31 < m:
        rows.update(range(r31, min(m, r31 + 32)))
    rows.update(int(v) for v in np.random.default_rng(seed).integers(0, m, size=64))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("idx", [2, 3, 4], ids=[synth.WORKLOADS[i]["name"].replace(" ", "_")
                                               for i in (2, 3, 4)])
def test_dequant_workload_sampled(idx):
    """The dequant path at the three large workloads' full size, in the launch
    bench.py --dequant times (persistent 256x256 blocks, bf16 out), on
    sampled rows (all n columns), rows past 2^31 output elements included:
    every sampled output inside the accumulation bound."""
    import torch
    dev = cuda_device()
    wl = synth.WORKLOADS[idx]
    m, n, k = wl["m"], wl["n"], wl["k"]
    print(f"\n[{wl['name']}] dequant path", flush=True)
    x, w, ws, b = synth.make_inputs(m, n, k, mode=wl["mode"], bias=wl["bias"],
                                    seed=synth.workload_seed(idx), device=dev)
    out = ck.int8_linear_dequant(x, w, ws, b)
    torch.cuda.synchronize()
    rows = _dequant_rows(m, n, k, seed=idx)
    r31 = synth.boundary_rows(m, n, k)["out_elem_2^31"]
    assert r31 >= m or rows.max() >= r31
    ridx = torch.from_numpy(rows).to(dev)
    bo = None if b is None else bits16(b)
    ref, s, a = oracle.linear_dequant(bits16(x.index_select(0, ridx)), w.cpu().numpy(),
                                      ws.cpu().numpy(), bo, "bf16")
    got = bits16(out.index_select(0, ridx))
    g = _values(got, "bf16")
    exact = s + (0.0 if bo is None else _values(bo, "bf16")[None, :])
    tol = k * 2.0 ** -24 * a + 2.0 ** -23 * np.abs(exact) + _ulp(np.maximum(np.abs(exact), np.abs(g)), "bf16")
    bad = np.abs(g - exact) > tol
    assert not bad.any(), f"{bad.sum()} of {bad.size} sampled outputs outside the bound"
    same = float(np.mean(got == ref))
    print(f"[{wl['name']}] {rows.size} rows x {n}: inside the bound, {100 * same:.3f}% equal to the "
          f"rounded exact sum", flush=True)

