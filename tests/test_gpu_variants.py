"""HIP path vs the CPU oracle for the layer's variants: fp16 and fp32
outputs (#280 "Exactness": the audit's output types), K that is not a
multiple of 16 (zero-padded K tail) and activation rows at any alignment.

Codes, scales and int32 accumulators bit-exact; floating outputs within 1
ulp of their type (and, with the same fp32 operation chain, bit-identical).
Every call goes through the C ABI (libck_int8.so)."""
import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import assert_within_1ulp, bits16, cuda_device

pytestmark = pytest.mark.gpu


def _host(t):
    """Output tensor -> numpy in the oracle's representation."""
    import torch
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return bits16(t)


def _bias_for(b_bf16, out_dtype):
    """The workload's bias in the output's type."""
    import torch
    if b_bf16 is None:
        return None
    return b_bf16.to({"bf16": torch.bfloat16, "fp16": torch.float16,
                      "fp32": torch.float32}[out_dtype])


def _oracle_bias(b, out_dtype):
    if b is None:
        return None
    return b.cpu().numpy() if out_dtype == "fp32" else bits16(b)


def _check(q, xs, w, ws, b, out_dtype, tile, what):
    import torch
    out = ck.int8_linear_q(q, xs, w, ws, b, tile=tile, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(), ws.cpu().numpy(),
                        _oracle_bias(b, out_dtype), out_dtype)
    return assert_within_1ulp(_host(out), ref, what)


# ---------------------------------------------------------------- output types

@pytest.mark.parametrize("out_dtype", ["fp16", "fp32"])
@pytest.mark.parametrize("tile", range(ck.CK_NUM_TILES))
def test_linear_out_dtype_all_tiles(out_dtype, tile):
    dev = cuda_device()
    m, n, k = 300, 520, 2064
    x, w, ws, b = synth.make_inputs(m, n, k, bias=True, seed=77 + tile, device=dev)
    q, xs = ck.quantize_int8_rowwise(x)
    exact = _check(q, xs, w, ws, _bias_for(b, out_dtype), out_dtype, tile,
                   f"{out_dtype} tile {tile}")
    assert exact == 1.0, exact


@pytest.mark.parametrize("out_dtype", ["fp16", "fp32"])
@pytest.mark.parametrize("x_mode,w_mode,bias", [("tensor", "tensor", False),
                                                ("row", "tensor", True),
                                                ("tensor", "row", False)])
def test_linear_out_dtype_scale_modes(out_dtype, x_mode, w_mode, bias):
    dev = cuda_device()
    m, n, k = 257, 700, 1024
    x, w, ws, b = synth.make_inputs(m, n, k, mode=w_mode, bias=bias, seed=5, device=dev)
    q, xs = ck.quantize_int8_rowwise(x, mode=x_mode)
    assert _check(q, xs, w, ws, _bias_for(b, out_dtype), out_dtype, -1, out_dtype) == 1.0


@pytest.mark.parametrize("tile", [3, 7, 12])
def test_fp16_output_range_subnormal_to_overflow(tile):
    """Outputs from fp16 subnormals (< 2^-14) through the largest finite
    value to overflow (>= 65520 becomes infinity), with exact ties."""
    import torch
    dev = cuda_device()
    m, n, k = 64, 256, 32
    q = torch.ones((m, k), dtype=torch.int8, device=dev)
    q[1::2] = -1
    wv = (torch.arange(n, device=dev) % 61 - 30).to(torch.int8)
    w = wv[:, None].repeat(1, k).contiguous()                   # acc = +-32 * wv
    ws = torch.exp2(torch.linspace(-34.0, 12.0, n, device=dev)).float()
    xs = torch.linspace(0.5, 2.0, m, device=dev).float()
    out = ck.int8_linear_q(q, xs, w, ws, None, tile=tile, out_dtype="fp16")
    torch.cuda.synchronize()
    ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(), ws.cpu().numpy(),
                        None, "fp16")
    got = bits16(out)
    np.testing.assert_array_equal(got, ref)
    mag = ref & 0x7FFF
    assert (mag == 0x7C00).any() and ((mag > 0) & (mag < 0x0400)).any()


# ---------------------------------------------------------------- K tail

def _padded(rows, k, lo, hi, g, dev, fill):
    """int8 [rows, k] view into [rows, k rounded up to 16] storage whose
    padding bytes hold `fill` (garbage the GEMM must ignore)."""
    import torch
    kp = (k + 15) // 16 * 16
    buf = torch.full((rows, kp), fill, dtype=torch.int8, device=dev)
    buf[:, :k] = torch.randint(lo, hi, (rows, k), generator=g, device=dev, dtype=torch.int8)
    return buf[:, :k]


KS = [1, 7, 15, 17, 40, 100, 127, 129, 200, 2055, 4100]


@pytest.mark.parametrize("tile", [-1, 2, 3, 7, 11, 12])
@pytest.mark.parametrize("k", KS)
def test_gemm_i32_any_k_with_garbage_padding(tile, k):
    import torch
    dev = cuda_device()
    m, n = 130, 290
    g = torch.Generator(device=dev).manual_seed(k * 31 + tile)
    q = _padded(m, k, -127, 128, g, dev, fill=-128)
    w = _padded(n, k, -128, 128, g, dev, fill=127)
    acc = ck.int8_gemm_i32(q, w, tile=tile)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(),
                                  oracle.gemm_i32(q.cpu().numpy(), w.cpu().numpy()))


@pytest.mark.parametrize("out_dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("k", [9, 104, 5000])
def test_linear_any_k_end_to_end(out_dtype, k):
    """bf16 x with any k: quantise (element kernel when rows are not 16-byte
    aligned), pad the weight rows once, then the fused layer."""
    import torch
    dev = cuda_device()
    m, n = 333, 515
    x, w, ws, b = synth.make_inputs(m, n, k, bias=True, seed=k, device=dev)
    wp = ck.pad_rows(w)
    assert wp.stride(0) % 16 == 0 and torch.equal(wp, w)
    bias = _bias_for(b, out_dtype)
    out = ck.int8_linear(x, wp, ws, bias, out_dtype=out_dtype)
    torch.cuda.synchronize()
    q_o, s_o, ref = oracle.int8_linear(bits16(x), w.cpu().numpy(), ws.cpu().numpy(),
                                       _oracle_bias(bias, out_dtype), out_dtype=out_dtype)
    assert assert_within_1ulp(_host(out), ref, f"k={k} {out_dtype}") == 1.0


def test_linear_rejects_unpadded_weight_rows():
    import torch
    dev = cuda_device()
    x = torch.ones((4, 24), dtype=torch.bfloat16, device=dev)
    w = torch.ones((8, 24), dtype=torch.int8, device=dev)          # rows 24 bytes apart
    with pytest.raises(ck.CKError) as e:
        ck.int8_linear(x, w, torch.ones(8, device=dev))
    assert e.value.status == ck.CK_ERR_UNSUPPORTED


# ---------------------------------------------------------------- unaligned quantise

@pytest.mark.parametrize("mode", ["row", "tensor"])
@pytest.mark.parametrize("k,off", [(31, 1), (4099, 3), (20001, 5)])
def test_quantize_unaligned_rows(mode, k, off):
    """x rows starting at odd element offsets (not 16-byte aligned) and q
    rows at odd byte strides: the element-wise kernels."""
    import torch
    dev = cuda_device()
    m = 37
    xf, _, _, _ = synth.make_inputs(m, 1, k + off + 2, seed=k, device=dev)
    x = xf[:, off:off + k]
    qf = torch.full((m, k + 3), 55, dtype=torch.int8, device=dev)
    q = qf[:, 1:k + 1]
    s = torch.empty(m if mode == "row" else 1, dtype=torch.float32, device=dev)
    ck.quantize_int8_rowwise(x, mode=mode, q=q, scale=s)
    torch.cuda.synchronize()
    fn = oracle.quantize_rowwise if mode == "row" else oracle.quantize_tensorwise
    q_o, s_o = fn(bits16(x))
    np.testing.assert_array_equal(s.cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    assert bool((qf[:, 0] == 55).all() and (qf[:, k + 1:] == 55).all())
