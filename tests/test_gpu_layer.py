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


# 1 x 64 and 1 x 192 have fewer K stages than the four weight stages the
# prologue issues; 1 x 8192 and 2 x 4096 hold 1024 chunks of 8 values, four
# per thread; 65 and 130 rows end in a partial row tile.
@pytest.mark.parametrize("m,n,k", [(1, 40, 64), (1, 64, 192), (1, 4160, 5376), (1, 200, 8192),
                                   (2, 130, 4096), (7, 129, 128), (16, 2048, 2048),
                                   (33, 70, 2048), (64, 520, 1024), (65, 200, 192),
                                   (130, 96, 256), (274, 2048, 2048)])
def test_layer_one_kernel_per_row(m, n, k, capfd):
    _case(m, n, k, "row", "bf16", bias=(m % 2 == 0), seed=m * 7 + n, capfd=capfd)


@pytest.mark.parametrize("m,n,k", [(1, 300, 640), (5, 64, 64), (2, 96, 4096), (32, 1000, 2048),
                                   (16, 130, 5376)])
def test_layer_one_kernel_tensor(m, n, k, capfd):
    _case(m, n, k, "tensor", "bf16", bias=True, seed=m + n, capfd=capfd)


@pytest.mark.parametrize("out_dtype", ["fp16", "fp32"])
@pytest.mark.parametrize("mode", ["row", "tensor"])
def test_layer_one_kernel_out_types(out_dtype, mode):
    _case(21, 333, 1088, mode, out_dtype, bias=True, seed=5)


def test_layer_longest_rows_in_lds():
    """Near the LDS limit of the one-kernel path (17,408 + 128 r rounded up
    to 256 + r k <= 163,840 bytes, r = min(m, 64)): 64 rows at k = 2112
    (160,768 bytes, with a second, partial row tile), 17 rows at k = 8448
    (163,328), one row at k = 131,072, and a tensor-wide scale over 2 rows
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


def test_layer_one_kernel_strided_buffers():
    """x rows 256 elements apart inside a wider tensor, q rows padded to 16
    bytes past k, out rows wider than n: q, x_scale and out as the oracle's,
    and the bytes past each row untouched."""
    import torch
    dev = cuda_device()
    m, n, k = 2, 1000, 1792
    xw, w, ws, b = synth.make_inputs(m, n, k + 256, mode="row", bias=True, seed=8, device=dev)
    x = xw[:, :k]
    w = w[:, :k].contiguous()
    qfull = torch.full((m, k + 16), 99, dtype=torch.int8, device=dev)
    q = qfull[:, :k]
    xs = torch.empty((m,), dtype=torch.float32, device=dev)
    ofull = torch.full((m, n + 24), 7.0, dtype=torch.bfloat16, device=dev)
    out = ofull[:, :n]
    ck.int8_linear(x, w, ws, b, out=out, fused=1, q=q, x_scale=xs)
    torch.cuda.synchronize()
    q_o, s_o, out_o = oracle.int8_linear(bits16(x), w.cpu().numpy(), ws.cpu().numpy(), bits16(b))
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    np.testing.assert_array_equal(xs.cpu().numpy(), s_o)
    assert_within_1ulp(bits16(out), out_o, "strided one kernel")
    assert bool((qfull[:, k:] == 99).all()) and bool((ofull[:, n:] == 7.0).all())


def test_layer_one_kernel_graph_capture_and_two_streams():
    """The one-kernel layer keeps no state between calls: captured into a
    graph and replayed three times between eager calls on other data, and
    issued on two streams at once, every result is the oracle's."""
    import torch
    dev = cuda_device()
    m, n, k = 1, 4096, 4096
    x, w, ws, _ = synth.make_inputs(m, n, k, seed=21, device=dev)
    y = (x.float() * -3.0).to(torch.bfloat16)
    _, _, ox = oracle.int8_linear(bits16(x), w.cpu().numpy(), ws.cpu().numpy())
    _, _, oy = oracle.int8_linear(bits16(y), w.cpu().numpy(), ws.cpu().numpy())
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    xs = torch.empty((m,), dtype=torch.float32, device=dev)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ck.int8_linear(x, w, ws, out=out, fused=1, q=q, x_scale=xs)       # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ck.int8_linear(x, w, ws, out=out, fused=1, q=q, x_scale=xs)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        oy_got = ck.int8_linear(y, w, ws, fused=1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_within_1ulp(bits16(out), ox, f"replay {rep}")
        assert_within_1ulp(bits16(oy_got), oy, f"eager {rep}")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(4):
        for st, t in ((s1, x), (s2, y)):
            with torch.cuda.stream(st):
                outs.append(ck.int8_linear(t, w, ws, fused=1))
    torch.cuda.synchronize()
    for j, o in enumerate(outs):
        assert_within_1ulp(bits16(o), ox if j % 2 == 0 else oy, f"two streams {j}")
