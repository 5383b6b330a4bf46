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


def _mfma_ceiling_model(iters, seed):
    """The per-lane checksums ck_mfma_ceiling defines, in numpy: a 32 x 32 x
    32 int8 product D = A B of one wave takes A[m][k] from byte k % 16 of
    the first operand in lane m + 32 (k // 16) and B[k][n] from byte k % 16
    of the second operand in lane n + 32 (k // 16) (any order of k inside
    the instruction gives the same integer sums), and returns D[m][n] in
    lane n + 32 ((m % 8) // 4), register 4 (m // 8) + m % 4."""
    u32 = np.uint32
    t = np.arange(512, dtype=np.uint64)
    l = ((t * 2654435761) & 0xFFFFFFFF).astype(u32) ^ u32(seed)

    def ops(mul, xor, add, mul2, i):
        return np.stack([(l.astype(np.uint64) * (i + mul)) & 0xFFFFFFFF,
                         (l ^ u32(xor * i)).astype(np.uint64),
                         (l.astype(np.uint64) + add * i) & 0xFFFFFFFF,
                         (l.astype(np.uint64) * mul2 + i) & 0xFFFFFFFF], 1).astype(u32)

    a = [ops(1, 77, 911, 3, i) for i in range(4)]
    b = [ops(5, 131, 313, 7, j) for j in range(2)]
    acc = np.zeros((8, 512, 16), np.int64)
    m = np.arange(32)
    lane_of = (np.arange(32)[None, :] + 32 * ((m[:, None] % 8) // 4))      # [m, n]
    reg_of = np.broadcast_to((4 * (m // 8) + m % 4)[:, None], (32, 32))
    for _ in range(iters):
        for i in range(4):
            for j in range(2):
                for w in range(8):
                    src0 = b[j][64 * w:64 * w + 64].view(np.int8).reshape(64, 16).astype(np.int64)
                    src1 = a[i][64 * w:64 * w + 64].view(np.int8).reshape(64, 16).astype(np.int64)
                    A = np.concatenate([src0[:32], src0[32:]], 1)           # [m, 32 k]
                    B = np.concatenate([src1[:32], src1[32:]], 1)           # [n, 32 k]
                    D = A @ B.T                                             # [m, n]
                    acc[2 * i + j, 64 * w + lane_of, reg_of] += D
        a = [((x.astype(np.uint64) * 1103515245 + 12345) & 0xFFFFFFFF).astype(u32) for x in a]
        b = [((x.astype(np.uint64) * 1103515245 + 12345) & 0xFFFFFFFF).astype(u32) for x in b]
    acc32 = (acc & 0xFFFFFFFF).astype(np.uint32)
    return np.bitwise_xor.reduce(acc32.transpose(1, 0, 2).reshape(512, -1), axis=1).view(np.int32)


@pytest.mark.parametrize("iters,seed", [(0, 0), (1, 0), (3, 12345)])
def test_mfma_ceiling_checksums(iters, seed):
    """The matrix-core measurement kernel computes what its header says:
    every block's 512 lane checksums equal the numpy model's."""
    import torch
    dev = cuda_device()
    out = torch.full((256 * 512,), 7, dtype=torch.int32, device=dev)
    ck.ck_mfma_ceiling(iters, out.data_ptr(), seed, torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    got = out.view(256, 512).cpu().numpy()
    want = _mfma_ceiling_model(iters, seed)
    assert (got == want[None, :]).all()
