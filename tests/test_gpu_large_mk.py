"""Inputs past 2^31 elements: m = 400,500 rows of k = 5376, against n = 5376.

Issue #136 ("INT8 GEMM kernels index the output in int32 ..."), section
"Minimal reproduction", measured-boundary table, row n = 5376: the first
failing m is 400,500 at k = 5376.  There m*n = m*k = 2.153e9 > 2^31, so
besides the output the int8 codes (2.15 GB) and the bf16 activations
(4.3 GB, byte offsets past 2^32) are addressed past the 32-bit range; issue
#280 ("INT8 linears on sm_121 ..."), section "Kernel used", names the M*K
wrap as well.  The launch configuration is the heuristic's (the persistent
tile-13 kernel, for the bf16 output and for the int32 accumulators).

Checked against the oracle on >= 4096 sampled rows, all n columns each:
rows 0..63, the last two row tiles, +-64 rows around every 32-bit wrap of a
q, x or output byte / element offset (rows 199,728 and 399,457), every row
holding an output element at or past 2^31 (399,457 to the end), and seeded
uniform rows.  Per-row quantisation: codes, scales and int32 accumulators
bit-exact, bf16 within 1 ulp.  Tensor-wide quantisation of the same x: the
scale and the sampled rows' codes bit-exact (the oracle takes the amax over
all 2.15e9 values), and the layer with that scale within 1 ulp.  ConvRot
per-row quantisation (blocks of 16 and 128) of the same x: codes and scales
bit-exact on the sampled rows.  The dequant-on-the-fly layer on the same x
and W (its persistent kernel, x read as bf16 past 2^32 bytes): about 180
rows around the wraps and past 2^31 output elements inside the fp32
accumulation bound."""
import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import assert_bf16_within_1ulp, bits16, cuda_device

pytestmark = pytest.mark.gpu

M, N, K = 400500, 5376, 5376
SEED = 20261202 + 16 * 7


def _say(msg):
    print(f"[m*k past 2^31, {M}x{N}x{K}] {msg}", flush=True)


@pytest.fixture(scope="module")
def inputs():
    import torch
    dev = cuda_device()
    _say("generating inputs")
    x, w, ws, _ = synth.make_inputs_chunked(M, N, K, mode="row", bias=False, seed=SEED, device=dev)
    rows = synth.sample_rows(M, N, K, count=4096, seed=7)
    b = synth.boundary_rows(M, N, K)
    assert b["q_byte_2^31"] < M and b["x_byte_2^32"] < M and b["out_elem_2^31"] < M
    assert set(range(b["out_elem_2^31"], M)) <= set(rows.tolist())
    for name in ("q_byte_2^31", "x_byte_2^31", "x_byte_2^32"):
        r = b[name]
        assert set(range(r - 64, min(M, r + 64))) <= set(rows.tolist()), name
    ridx = torch.from_numpy(rows).to(dev)
    yield dict(x=x, w=w, ws=ws, rows=rows, ridx=ridx, w_h=w.cpu().numpy(), ws_h=ws.cpu().numpy())
    del x, w, ws
    torch.cuda.empty_cache()


def test_per_row_layer_and_accumulators(inputs, capfd):
    import torch
    x, w, ws, rows, ridx = (inputs[k] for k in ("x", "w", "ws", "rows", "ridx"))
    ck.ck_int8_set_path_log(True)
    try:
        capfd.readouterr()
        _say("per-row quantisation, bf16 layer, int32 accumulators")
        q, xs = ck.quantize_int8_rowwise(x)
        out = ck.int8_linear_q(q, xs, w, ws)
        acc = ck.int8_gemm_i32(q, w)
        torch.cuda.synchronize()
        err = capfd.readouterr().err
    finally:
        ck.ck_int8_set_path_log(False)
    gemm = [l for l in err.splitlines() if f" gemm {M}x{N}x{K} " in l]
    assert any("out=bf16" in l and "persistent" in l for l in gemm), gemm
    assert any("out=int32" in l and "persistent" in l for l in gemm), gemm

    _say(f"checking {rows.size} rows")
    q_o, s_o = oracle.quantize_rowwise(bits16(x.index_select(0, ridx)))
    np.testing.assert_array_equal(xs.index_select(0, ridx).cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.index_select(0, ridx).cpu().numpy(), q_o)
    acc_o = oracle.gemm_i32(q_o, inputs["w_h"])
    np.testing.assert_array_equal(acc.index_select(0, ridx).cpu().numpy(), acc_o)
    del acc
    out_o = oracle.epilogue(acc_o, s_o, inputs["ws_h"], None)
    exact = assert_bf16_within_1ulp(bits16(out.index_select(0, ridx)), out_o, "per-row")
    _say(f"codes, scales, accumulators bit-exact; bf16 {100 * exact:.4f}% bit-identical")
    del q, xs, out
    torch.cuda.empty_cache()


def test_tensorwise_quantisation_and_layer(inputs):
    import torch
    x, w, ws, rows, ridx = (inputs[k] for k in ("x", "w", "ws", "rows", "ridx"))
    _say("tensor-wide quantisation and the layer with that scale")
    q, xs = ck.quantize_int8_rowwise(x, mode="tensor")
    out = ck.int8_linear_q(q, xs, w, ws)
    torch.cuda.synchronize()
    _say("oracle amax over every value of x")
    q_o, s_o = oracle.quantize_tensorwise(bits16(x))
    q_o = q_o[rows]
    np.testing.assert_array_equal(xs.cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.index_select(0, ridx).cpu().numpy(), q_o)
    out_o = oracle.linear(q_o, s_o, inputs["w_h"], inputs["ws_h"], None)
    exact = assert_bf16_within_1ulp(bits16(out.index_select(0, ridx)), out_o, "tensor-wide")
    _say(f"scale and codes bit-exact; bf16 {100 * exact:.4f}% bit-identical")
    del q, xs, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("block", [16, 128])
def test_rotated_quantisation(inputs, block):
    """ConvRot per-row quantisation (x H, block-diagonal Hadamard) with x and
    q byte offsets past 2^31 and 2^32: codes and scales of the sampled rows
    bit-exact."""
    import torch
    x, rows, ridx = (inputs[k] for k in ("x", "rows", "ridx"))
    _say(f"rotated per-row quantisation, block {block}")
    q, xs = ck.quantize_int8_rotated(x, block)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_rotated(bits16(x.index_select(0, ridx)), block)
    np.testing.assert_array_equal(xs.index_select(0, ridx).cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.index_select(0, ridx).cpu().numpy(), q_o)
    _say(f"block {block}: codes and scales of {rows.size} rows bit-exact")
    del q, xs
    torch.cuda.empty_cache()


def test_dequant_layer(inputs, capfd):
    """The dequant-on-the-fly layer (bf16 x times W dequantised in the
    kernel) at the same size, in its persistent launch: every sampled
    output inside the fp32 accumulation bound |got - S| <= k 2^-24 A +
    2^-23 |S| + 1 bf16 ulp (S, A from the oracle)."""
    import torch
    x, w, ws = (inputs[k] for k in ("x", "w", "ws"))
    ck.ck_int8_set_path_log(True)
    try:
        capfd.readouterr()
        _say("dequant-on-the-fly layer")
        out = ck.int8_linear_dequant(x, w, ws)
        torch.cuda.synchronize()
        err = capfd.readouterr().err
    finally:
        ck.ck_int8_set_path_log(False)
    assert any("persistent" in l for l in err.splitlines() if f"{M}x{N}x{K}" in l), err
    b = synth.boundary_rows(M, N, K)
    sel = set(range(8)) | set(range(M - 8, M))
    for r in b.values():
        if r < M:
            sel.update(range(max(0, r - 8), min(M, r + 8)))
    sel.update(range(b["out_elem_2^31"], b["out_elem_2^31"] + 32))
    sel.update(int(v) for v in np.random.default_rng(11).integers(0, M, size=64))
    rows = np.array(sorted(sel), dtype=np.int64)
    ridx = torch.from_numpy(rows).to(x.device)
    _say(f"checking {rows.size} rows of the dequant layer")
    ref, s_o, a_o = oracle.linear_dequant(bits16(x.index_select(0, ridx)), inputs["w_h"],
                                          inputs["ws_h"], None, "bf16")
    got = bits16(out.index_select(0, ridx))
    g = oracle.bf16_to_f32(got).astype(np.float64)
    e = np.floor(np.log2(np.maximum(np.maximum(np.abs(s_o), np.abs(g)), 2.0 ** -126)))
    tol = K * 2.0 ** -24 * a_o + 2.0 ** -23 * np.abs(s_o) + np.exp2(e - 7)
    bad = np.abs(g - s_o) > tol
    assert not bad.any(), f"{bad.sum()} of {bad.size} sampled outputs outside the bound"
    _say(f"{rows.size} rows inside the bound, {100 * float(np.mean(got == ref)):.3f}% equal "
         "to the oracle's rounding")
    del out
    torch.cuda.empty_cache()
