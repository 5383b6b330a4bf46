"""Past 1024 streams on a device no counters are left for a new stream: the
persistent GEMM then runs tile 12's one-block-per-tile kernel and the
tensor-wide quantisation its four-launch chain (scale[0] as the amax cell),
with the same results (the header's allocation convention).  The streams
are plain HIP streams (default priority), created here so that each call
sees a new handle.  The test uses up the process's counters, so it is
collected last."""
import ctypes

import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import bits16, cuda_device

pytestmark = pytest.mark.gpu

N_STREAMS = 1100


def _hip():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    return hip


def test_counter_pool_exhausted(capfd):
    import torch
    dev = cuda_device()
    hip = _hip()
    m, k = 67, 264
    x, _, _, _ = synth.make_inputs(m, 1, k, mode="tensor", seed=91, device=dev)
    q_o, s_o = oracle.quantize_tensorwise(bits16(x))
    bufs = [(torch.empty((m, k), dtype=torch.int8, device=dev),
             torch.empty(1, dtype=torch.float32, device=dev)) for _ in range(N_STREAMS)]
    gm, gn, gk = 4608, 4352, 128                    # 18 x 17 = 306 tiles: persistent when it can
    gx, gw, gws, gb = synth.make_inputs(gm, gn, gk, mode="row", bias=True, seed=92, device=dev)
    gq, gxs = ck.quantize_int8_rowwise(gx)
    gref = ck.int8_linear_q(gq, gxs, gw, gws, gb, tile=12)
    gout = torch.empty_like(gref)
    torch.cuda.synchronize()
    handles = []
    ck.ck_int8_set_path_log(True)
    try:
        for _ in range(N_STREAMS):
            h = ctypes.c_void_p()
            assert hip.hipStreamCreate(ctypes.byref(h)) == 0
            handles.append(h.value)
        capfd.readouterr()
        for h, (q, s) in zip(handles, bufs):
            ck.ck_quantize_int8_rowwise(x.data_ptr(), m, k, k, q.data_ptr(), k, s.data_ptr(),
                                        ck.CK_SCALE_TENSOR, h)
        ck.ck_int8_linear_tiled(gq.data_ptr(), gq.stride(0), gxs.data_ptr(), ck.CK_SCALE_ROW,
                                gw.data_ptr(), gw.stride(0), gws.data_ptr(), ck.CK_SCALE_ROW,
                                gb.data_ptr(), gout.data_ptr(), gn, gm, gn, gk, 13, 4, handles[-1])
        for h in handles:
            assert hip.hipStreamSynchronize(h) == 0
        err = capfd.readouterr().err
    finally:
        ck.ck_int8_set_path_log(False)
        for h in handles:
            hip.hipStreamDestroy(h)
    for q, s in bufs:
        np.testing.assert_array_equal(s.cpu().numpy(), s_o)
        np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    assert torch.equal(gout.view(torch.int16), gref.view(torch.int16))
    quant = [l for l in err.splitlines() if f" quantize {m}x{k} " in l]
    assert any("amax=two launches" in l for l in quant), quant
    assert any("amax=four launches" in l for l in quant), quant
    gemm = [l for l in err.splitlines() if f" gemm {gm}x{gn}x{gk} " in l]
    assert gemm and all("persistent" not in l for l in gemm), gemm
