"""ck_int8_linear_noalloc, the entry point for callers that cannot allocate:
ck_int8_linear_ex's arguments and kernels, with the persistent kernel's
tile-claim counters in the library's fixed per-device scratch array
instead of a per-stream slot.  Through the C ABI: two calls in a row, the
second on a smaller input, both on the persistent kernel (so the second
finds the first call's leftovers in the shared array), each bit-identical
to ck_int8_linear_ex on the same inputs and within 1 ulp of the oracle;
then the call captured into a graph and replayed between eager calls of
both entry points."""
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import assert_bf16_within_1ulp, bits16, cuda_device

pytestmark = pytest.mark.gpu


def _inputs(m, n, k, seed):
    dev = cuda_device()
    x, w, ws, b = synth.make_inputs(m, n, k, mode="row", bias=True, seed=seed, device=dev)
    q, xs = ck.quantize_int8_rowwise(x)
    return q, xs, w, ws, b


def _noalloc(q, xs, w, ws, b, out, stream):
    m, k = q.shape
    n = w.shape[0]
    ck.ck_int8_linear_noalloc(q.data_ptr(), q.stride(0), xs.data_ptr(), ck.CK_SCALE_ROW,
                              w.data_ptr(), w.stride(0), ws.data_ptr(), ck.CK_SCALE_ROW,
                              b.data_ptr(), out.data_ptr(), out.stride(0), ck.CK_OUT_BF16,
                              m, n, k, -1, 0, stream)


def _ex(q, xs, w, ws, b, out, stream):
    m, k = q.shape
    n = w.shape[0]
    ck.ck_int8_linear_ex(q.data_ptr(), q.stride(0), xs.data_ptr(), ck.CK_SCALE_ROW,
                         w.data_ptr(), w.stride(0), ws.data_ptr(), ck.CK_SCALE_ROW,
                         b.data_ptr(), out.data_ptr(), out.stride(0), ck.CK_OUT_BF16,
                         m, n, k, -1, 0, stream)


def test_noalloc_two_calls_match_linear_ex(capfd):
    import torch
    stream = torch.cuda.current_stream(cuda_device()).cuda_stream
    ck.ck_int8_set_path_log(True)
    try:
        # 19 x 18 = 342 tiles, then 18 x 18 = 324: both above 256, persistent
        for m, n, k, seed in ((4700, 4568, 384, 71), (4400, 4400, 256, 72)):
            print(f"\n[noalloc {m}x{n}x{k}]", flush=True)
            q, xs, w, ws, b = _inputs(m, n, k, seed)
            ref = torch.empty((m, n), dtype=torch.bfloat16, device=q.device)
            out = torch.full((m, n), 3.0, dtype=torch.bfloat16, device=q.device)
            capfd.readouterr()
            _ex(q, xs, w, ws, b, ref, stream)
            _noalloc(q, xs, w, ws, b, out, stream)
            torch.cuda.synchronize()
            err = capfd.readouterr().err
            lines = [l for l in err.splitlines() if f" gemm {m}x{n}x{k} " in l]
            assert any("persistent" in l and "counters=scratch" in l for l in lines), lines
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
            want = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(),
                                 ws.cpu().numpy(), bits16(b))
            assert_bf16_within_1ulp(bits16(out), want, f"noalloc {m}x{n}x{k}")
    finally:
        ck.ck_int8_set_path_log(False)


def test_noalloc_under_graph_capture():
    """The captured call (scratch clear + persistent GEMM) replayed three
    times, with eager calls of both entry points on other data in between;
    every replay equals ck_int8_linear_ex's result."""
    import torch
    dev = cuda_device()
    m, n, k = 4700, 4568, 256
    q, xs, w, ws, b = _inputs(m, n, k, 81)
    q2, xs2, w2, ws2, b2 = _inputs(4400, 4400, 128, 82)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ref = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _ex(q, xs, w, ws, b, ref, stream)
    ref2 = torch.empty((4400, 4400), dtype=torch.bfloat16, device=dev)
    _ex(q2, xs2, w2, ws2, b2, ref2, stream)
    out = torch.empty_like(ref)
    out2 = torch.empty_like(ref2)
    out3 = torch.empty_like(ref2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _noalloc(q, xs, w, ws, b, out, side.cuda_stream)             # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _noalloc(q, xs, w, ws, b, out, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        out2.zero_()
        out3.zero_()
        _noalloc(q2, xs2, w2, ws2, b2, out2, stream)
        _ex(q2, xs2, w2, ws2, b2, out3, stream)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        assert torch.equal(out2.view(torch.int16), ref2.view(torch.int16)), rep
        assert torch.equal(out3.view(torch.int16), ref2.view(torch.int16)), rep
