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


def _lowbias32(x):
    """C. Wellons' 32-bit integer hash ("Prospecting for hash functions"),
    on a numpy uint64 array holding 32-bit values."""
    m = 0xFFFFFFFF
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & m
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & m
    return x ^ (x >> 16)


def _mfma_slice_products(seed):
    """D[s, t, m, n]: the 8 products (t = 2i + j) one half-step with slice s
    adds to one wave's accumulator tiles, in numpy int64.  A 32 x 32 x 32
    int8 product D = A B takes A[m][k] from byte k % 16 of the first operand
    in lane m + 32 (k // 16) and B[k][n] from byte k % 16 of the second in
    lane n + 32 (k // 16) (any order of k inside the instruction gives the
    same integer sums)."""
    words = _lowbias32(np.arange(12288, dtype=np.uint64) + 12288 * seed).astype(np.uint32)
    frags = words.reshape(8, 6, 64, 4)                      # slice, fragment, lane, word
    D = np.zeros((8, 8, 32, 32), np.int64)
    for s in range(8):
        for i in range(4):
            for j in range(2):
                src0 = frags[s, 4 + j].view(np.int8).reshape(64, 16).astype(np.int64)
                src1 = frags[s, i].view(np.int8).reshape(64, 16).astype(np.int64)
                A = np.concatenate([src0[:32], src0[32:]], 1)   # [m, 32 k]
                B = np.concatenate([src1[:32], src1[32:]], 1)   # [n, 32 k]
                D[s, 2 * i + j] = A @ B.T
    return D


def _mfma_ceiling_model(iters, mode, seed):
    """The 512 per-lane checksums ck_mfma_ceiling defines (every block and
    every wave computes the same).  Integer sums do not depend on the order
    of the products, so each slice's products enter as many times as the
    launch uses the slice.  D[m][n] sits in lane n + 32 ((m % 8) // 4),
    register 4 (m // 8) + m % 4."""
    D = _mfma_slice_products(seed)
    if mode == 0:
        uses = np.array([iters, iters] + [0] * 6, np.int64)
    else:
        q = 2 * iters                                       # half-steps
        uses = np.array([(q - s + 7) // 8 for s in range(8)], np.int64)
    acc = np.einsum("s,stmn->tmn", uses, D)                 # [tile, m, n]
    m = np.arange(32)
    lane_of = np.arange(32)[None, :] + 32 * ((m[:, None] % 8) // 4)
    reg_of = np.broadcast_to((4 * (m // 8) + m % 4)[:, None], (32, 32))
    lanes = np.zeros((64, 8, 16), np.int64)
    lanes[lane_of, :, reg_of] = acc.transpose(1, 2, 0)
    acc32 = (lanes & 0xFFFFFFFF).astype(np.uint32)
    per_lane = np.bitwise_xor.reduce(acc32.reshape(64, -1), axis=1).view(np.int32)
    return np.tile(per_lane, 8)


@pytest.mark.parametrize("iters,mode,seed", [(0, 0, 0), (1, 0, 0), (3, 0, 12345), (0, 1, 0),
                                             (1, 1, 0), (3, 1, 7), (13, 1, 12345),
                                             (100000, 0, 1), (100000, 1, 1)])
def test_mfma_ceiling_checksums(iters, mode, seed):
    """The matrix-core measurement kernel computes what its header says:
    every block's 512 lane checksums equal the numpy model's, in both modes,
    at the iteration count bench.py times (wrapping int32 sums)."""
    import torch
    dev = cuda_device()
    out = torch.full((256 * 512,), 7, dtype=torch.int32, device=dev)
    ck.ck_mfma_ceiling(iters, mode, out.data_ptr(), seed, torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    got = out.view(256, 512).cpu().numpy()
    want = _mfma_ceiling_model(iters, mode, seed)
    assert (got == want[None, :]).all()
