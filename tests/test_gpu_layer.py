"""The whole layer in one call (ck_int8_layer), HIP path vs the CPU oracle.

Issue #280, "Kernel used": activations quantised per row (or per tensor),
then the int8 GEMM with the dequant epilogue.  For few rows the library
runs both steps as one kernel: every 64 x 64 block quantises its own rows
into LDS with the quantisation kernel's arithmetic.  Checked on ragged
shapes (partial row and column tiles, one row, rows past a 64-row tile),
both scale modes, bias, and the three output types:
- q and x_scale that the call leaves: bit-exact against the oracle;
- out within 1 ulp of the oracle's, and bit-identical to the two-kernel
  path (quantisation kernel + GEMM) on the same inputs;
- the path log names the one-kernel path where it was asked for, and the
  library's own choice takes it for m <= 2."""
import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import assert_within_1ulp, bits16, cuda_device

pytestmark = pytest.mark.gpu

_TORCH_OUT = {"bf16": "bfloat16", "fp16": "float16", "fp32": "float32"}


def _host(t):
    import torch
    return t.cpu().numpy() if t.dtype == torch.float32 else bits16(t)


def _run(x, w, ws, b, mode, out_dtype, fused):
    import torch
    m, k = x.shape
    q = torch.full((m, (k + 15) // 16 * 16), 99, dtype=torch.int8, device=x.device)[:, :k]
    xs = torch.full((m if mode == "row" else 1,), -1.0, dtype=torch.float32, device=x.device)
    out = ck.int8_linear(x, w, ws, b, mode=mode, out_dtype=out_dtype, fused=fused, q=q, x_scale=xs)
    torch.cuda.synchronize()
    return q, xs, out


def _case(m, n, k, mode, out_dtype, bias, seed, capfd=None):
    import torch
    dev = cuda_device()
    print(f"\n[layer {m}x{n}x{k} {mode} {out_dtype} bias={bias}]", flush=True)
    x, w, ws, b = synth.make_inputs(m, n, k, mode=mode, bias=bias, seed=seed, device=dev)
    if b is not None:
        b = b.to(getattr(torch, _TORCH_OUT[out_dtype]))
    ck.ck_int8_set_path_log(True)
    try:
        if capfd is not None:
            capfd.readouterr()
        q1, s1, o1 = _run(x, w, ws, b, mode, out_dtype, fused=1)
        err = capfd.readouterr().err if capfd is not None else ""
    finally:
        ck.ck_int8_set_path_log(False)
    if capfd is not None:
        assert any(f"layer {m}x{n}x{k} " in l and "one kernel" in l for l in err.splitlines()), err
    q0, s0, o0 = _run(x, w, ws, b, mode, out_dtype, fused=0)
    bo = None if b is None else _host(b)
    q_o, s_o, out_o = oracle.int8_linear(bits16(x), w.cpu().numpy(), ws.cpu().numpy(), bo, mode,
                                         out_dtype)
    np.testing.assert_array_equal(q1.cpu().numpy(), q_o)
    np.testing.assert_array_equal(s1.cpu().numpy(), s_o)
    np.testing.assert_array_equal(q0.cpu().numpy(), q_o)
    np.testing.assert_array_equal(s0.cpu().numpy(), s_o)
    exact = assert_within_1ulp(_host(o1), out_o, f"one kernel {m}x{n}x{k}")
    wide = np.uint32 if out_dtype == "fp32" else np.uint16
    assert np.array_equal(_host(o1).view(wide), _host(o0).view(wide)), "one kernel != two kernels"
    return exact


@pytest.mark.parametrize("m,n,k", [(1, 40, 64), (1, 4160, 5376), (7, 129, 128), (16, 2048, 2048),
                                   (33, 70, 2048), (64, 520, 1024), (65, 200, 192),
                                   (130, 96, 256), (274, 2048, 2048)])
def test_layer_one_kernel_per_row(m, n, k, capfd):
    _case(m, n, k, "row", "bf16", bias=(m % 2 == 0), seed=m * 7 + n, capfd=capfd)


@pytest.mark.parametrize("m,n,k", [(1, 300, 640), (5, 64, 64), (32, 1000, 2048), (16, 130, 5376)])
def test_layer_one_kernel_tensor(m, n, k, capfd):
    _case(m, n, k, "tensor", "bf16", bias=True, seed=m + n, capfd=capfd)


@pytest.mark.parametrize("out_dtype", ["fp16", "fp32"])
@pytest.mark.parametrize("mode", ["row", "tensor"])
def test_layer_one_kernel_out_types(out_dtype, mode):
    _case(21, 333, 1088, mode, out_dtype, bias=True, seed=5)


def test_layer_longest_rows_in_lds():
    """Near the LDS limit of the one-kernel path (16,896 + 128 r rounded up
    to 256 + r k <= 163,840 bytes, r = min(m, 64)): 64 rows at k = 2112
    (160,256 bytes, with a second, partial row tile), 17 rows at k = 8448
    (162,816), one row at k = 131,072, and a tensor-wide scale over 2 rows
    at k = 65,536."""
    _case(70, 300, 2112, "row", "bf16", bias=False, seed=3)
    _case(17, 70, 8448, "row", "bf16", bias=True, seed=4)
    _case(1, 70, 131072, "row", "bf16", bias=True, seed=6)
    _case(2, 200, 65536, "tensor", "bf16", bias=True, seed=5)


def test_layer_library_choice(capfd):
    """fused=-1: one kernel for m <= 2, the two kernels above (both match
    the oracle, checked in _case through fused=1/0)."""
    import torch
    dev = cuda_device()
    ck.ck_int8_set_path_log(True)
    try:
        for m in (1, 2, 3, 64):
            x, w, ws, _ = synth.make_inputs(m, 256, 512, seed=m, device=dev)
            capfd.readouterr()
            out = ck.int8_linear(x, w, ws)
            torch.cuda.synchronize()
            err = capfd.readouterr().err
            one = any(f"layer {m}x256x512 " in l and "one kernel" in l for l in err.splitlines())
            assert one == (m <= 2), (m, err)
            q_o, s_o, out_o = oracle.int8_linear(bits16(x), w.cpu().numpy(), ws.cpu().numpy())
            assert_within_1ulp(bits16(out), out_o, f"library choice m={m}")
    finally:
        ck.ck_int8_set_path_log(False)


def test_layer_unsupported_one_kernel_raises_before_launch():
    """fused=1 on layouts the one-kernel path does not take: CK_ERR_UNSUPPORTED,
    nothing written; fused=-1 on the same inputs runs the two kernels."""
    import torch
    dev = cuda_device()
    for m, k, mode in ((8, 200, "row"), (65, 128, "tensor"), (64, 2176, "row"), (17, 8512, "row")):
        x, w, ws, _ = synth.make_inputs(m, 96, k, mode=mode, seed=k, device=dev)
        w = ck.pad_rows(w)
        out = torch.full((m, 96), 7.0, dtype=torch.bfloat16, device=dev)
        with pytest.raises(ck.CKError) as e:
            ck.int8_linear(x, w, ws, mode=mode, out=out, fused=1)
        assert e.value.status == ck.CK_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
        out = ck.int8_linear(x, w, ws, mode=mode, fused=-1)
        torch.cuda.synchronize()
        q_o, s_o, out_o = oracle.int8_linear(bits16(x), w.cpu().numpy(), ws.cpu().numpy(), None, mode)
        assert_within_1ulp(bits16(out), out_o, f"fallback {m}x{k} {mode}")
