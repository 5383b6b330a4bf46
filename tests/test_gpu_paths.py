"""Path logging, the forced tile and the measured tile table on real
launches (PR #142, "What this does", items 1-3): each launch logs the
kernel that ran once per unique shape, a forced or tabled tile is the one
that runs, and the results stay those of the oracle."""
import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import assert_bf16_within_1ulp, bits16, cuda_device

pytestmark = pytest.mark.gpu


def _run(m, n, k, seed, **kw):
    import torch
    dev = cuda_device()
    x, w, ws, b = synth.make_inputs(m, n, k, bias=True, seed=seed, device=dev)
    q, xs = ck.quantize_int8_rowwise(x)
    out = ck.int8_linear_q(q, xs, w, ws, b, **kw)
    torch.cuda.synchronize()
    ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(), ws.cpu().numpy(),
                        bits16(b))
    assert assert_bf16_within_1ulp(bits16(out), ref) == 1.0


def _lines(text):
    return [l for l in text.splitlines() if l.startswith("ck_int8 path:")]


def test_path_log_forced_tile_and_table(capfd):
    cuda_device()
    forced_before = ck.ck_int8_forced_tile()
    ck.ck_int8_set_path_log(True)
    try:
        capfd.readouterr()
        _run(300, 520, 2064, 1)
        _run(300, 520, 2064, 2)                       # same shape: no second line
        lines = _lines(capfd.readouterr().err)
        gemm = [l for l in lines if " gemm 300x520x2064 " in l]
        quant = [l for l in lines if " quantize 300x2064 " in l]
        assert len(gemm) == 1 and len(quant) == 1, lines
        t, _, _, g = ck.ck_int8_select_tile(300, 520, 2064)
        assert f"tile={t} " in gemm[0] and "out=bf16" in gemm[0] and "K tail 16 bytes" in gemm[0]
        assert "source=heuristic" in gemm[0] or "source=table" in gemm[0]

        ck.ck_int8_set_forced_tile(7)                 # register-staged 64x64
        _run(300, 520, 2064, 3)
        gemm = [l for l in _lines(capfd.readouterr().err) if " gemm 300x520x2064 " in l]
        assert len(gemm) == 1 and "tile=7 " in gemm[0] and "source=forced" in gemm[0]
        assert "register-staged" in gemm[0]
        ck.ck_int8_set_forced_tile(-1)

        ck.ck_int8_table_set(300, 520, 2064, 1, 2)    # 256x128, group 2
        _run(300, 520, 2064, 4)
        gemm = [l for l in _lines(capfd.readouterr().err) if " gemm 300x520x2064 " in l]
        assert len(gemm) == 1 and "tile=1 " in gemm[0] and "group_m=2" in gemm[0]
        assert "source=table" in gemm[0]
        _run(300, 520, 2064, 5, tile=2)               # an explicit tile wins over the table
        gemm = [l for l in _lines(capfd.readouterr().err) if " gemm 300x520x2064 " in l]
        assert len(gemm) == 1 and "tile=2 " in gemm[0] and "source=argument" in gemm[0]
    finally:
        ck.ck_int8_table_set(300, 520, 2064, -1, 0)
        ck.ck_int8_set_forced_tile(forced_before)
        ck.ck_int8_set_path_log(False)


@pytest.mark.parametrize("chunks,blocks,unroll", [(1, 1, 1), (1000003, 512, 4), (65536, 4096, 8),
                                                  (70001, 256, 2)])
def test_hbm_stream_writes_the_xor_of_each_chunks_halves(chunks, blocks, unroll):
    """The measurement kernel behind the quantisation's ceiling touches
    every chunk exactly once: word j of the output is the xor of 32-bit
    words j and j + 2 of input chunk j."""
    import torch
    dev = cuda_device()
    g = torch.Generator(device=dev).manual_seed(chunks)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (chunks, 4), generator=g, device=dev, dtype=torch.int32)
    dst = torch.full((chunks, 2), 7, dtype=torch.int32, device=dev)
    ck.ck_hbm_stream(src.data_ptr(), chunks, dst.data_ptr(), blocks, unroll,
                     torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(dst, torch.stack([src[:, 0] ^ src[:, 2], src[:, 1] ^ src[:, 3]], 1))
