"""ConvRot online rotation (#278, "Suggested fix": x_rot = x H with the
weight stored as W H^T), HIP path vs the CPU oracle: codes and scales
bit-exact, the fused layer on rotated operands within 1 bf16 ulp.
Every call goes through the C ABI (libck_int8.so)."""
import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import assert_bf16_within_1ulp, bits16, cuda_device

pytestmark = pytest.mark.gpu


def _to_dev(xb, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16).copy()).to(dev).view(torch.bfloat16)


def _rotated_pair(x, block, mode="row"):
    import torch
    q, s = ck.quantize_int8_rotated(x, block, mode=mode)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_rotated(bits16(x), block, mode)
    np.testing.assert_array_equal(s.cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)


# Row lengths 5376 and 6144 (11 and 12 chunks of 512) and 4104 (9 chunks,
# the last one 8 elements long) run on the 12-chunk register kernel, 8192 on
# the 16-chunk one, 20480 re-reads what 16 chunks do not hold.
CASES = [(b, m, k) for b in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)
         for (m, k) in ((5, 512), (33, 5376), (17, 6144), (7, 8192), (3, 20480), (64, 1024))
         if k % b == 0] + [(8, 64, 136), (16, 9, 2064), (8, 11, 4104)]


@pytest.mark.parametrize("block,m,k", CASES)
def test_quantize_rotated_bit_exact(block, m, k):
    dev = cuda_device()
    x, _, _, _ = synth.make_inputs(m, 1, k, seed=block * 7 + k, device=dev)
    _rotated_pair(x, block)


@pytest.mark.parametrize("block,m,k", [(128, 40, 5376), (64, 12, 6144), (512, 9, 20480), (4, 300, 64)])
def test_quantize_rotated_tensorwise(block, m, k):
    dev = cuda_device()
    x, _, _, _ = synth.make_inputs(m, 1, k, mode="tensor", seed=k + 1, device=dev)
    _rotated_pair(x, block, mode="tensor")


def test_quantize_rotated_wide_dynamic_range_and_zero_rows():
    """Values spread over 2^-20 .. 2^10 (the butterfly sums round), outlier
    channels, and all-zero rows (scale 0, codes 0)."""
    dev = cuda_device()
    rng = np.random.default_rng(31)
    m, k = 24, 4096
    f = (rng.standard_normal((m, k)) * np.exp2(rng.integers(-20, 10, (m, k)))).astype(np.float32)
    f[:, rng.choice(k, 16, replace=False)] *= 300.0
    f[5] = 0.0
    xb = (f.view(np.uint32) >> 16).astype(np.uint16)
    for block in (32, 256, 512):
        _rotated_pair(_to_dev(xb, dev), block)


@pytest.mark.parametrize("amax", [1.0, 127.0, 0.001953125, 1.5 * 2.0 ** -100, 2.0 ** 120])
def test_quantize_rotated_block1_every_bf16_value(amax):
    """block = 1 leaves x unchanged (r = 1), so the fp32 code path of the
    rotated kernel meets every finite bf16 value under several scales."""
    dev = cuda_device()
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(b)
    a_bits = np.uint16(np.float32(amax).view(np.uint32) >> 16)
    vals = b[np.isfinite(f) & (np.abs(f) <= amax)]
    row = np.concatenate([[a_bits], vals])
    row = np.concatenate([row, np.zeros((-row.size) % 16, np.uint16)])
    _rotated_pair(_to_dev(row[None, :], dev), 1)


@pytest.mark.parametrize("tile", [-1, 3, 12])
def test_rotated_layer_end_to_end(tile):
    """x with outlier channels, W_rot = W H^T (= W H, H symmetric)
    quantised per row by the same rotated quantisation: the fused layer on
    the rotated codes matches the oracle and lands within 2 % of x W^T,
    well under the unrotated layer's error."""
    import torch
    dev = cuda_device()
    m, n, k, block = 300, 520, 2048, 128
    g = torch.Generator(device=dev).manual_seed(9)
    xf = torch.randn((m, k), generator=g, device=dev)
    xf[:, torch.randperm(k, generator=g, device=dev)[:16]] *= 60.0
    x = xf.to(torch.bfloat16)
    w = torch.randn((n, k), generator=g, device=dev, dtype=torch.float64) * 0.02
    wq, ws = ck.quantize_int8_rotated(w.to(torch.bfloat16), block)
    wq_o, ws_o = oracle.quantize_rotated(bits16(w.to(torch.bfloat16)), block, "row")
    np.testing.assert_array_equal(wq.cpu().numpy(), wq_o)
    np.testing.assert_array_equal(ws.cpu().numpy(), ws_o)
    q, xs = ck.quantize_int8_rotated(x, block)
    out = ck.int8_linear_q(q, xs, wq, ws, tile=tile)
    torch.cuda.synchronize()
    ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), wq.cpu().numpy(), ws.cpu().numpy())
    assert assert_bf16_within_1ulp(bits16(out), ref, "rotated layer") == 1.0
    exact = x.double() @ w.t()
    err = float((out.double() - exact).norm() / exact.norm())
    wq0, ws0 = ck.quantize_int8_rowwise(w.to(torch.bfloat16))
    plain = ck.int8_linear(x, wq0, ws0)
    err0 = float((plain.double() - exact).norm() / exact.norm())
    assert err < 0.02 and err < 0.5 * err0, (err, err0)


def test_rotated_tensorwise_eager_and_under_graph_capture(capfd):
    """Tensor-wide rotated quantisation: eager calls take two launches
    through the stream's alternating amax cells (which the plain tensor-wide
    quantisation shares), graph capture the four-launch chain with scale[0]
    as the cell.  Three replays between eager rotated and plain calls on
    other data each give the oracle's codes and scale."""
    import torch
    dev = cuda_device()
    m, k, block = 40, 2048, 128
    x, _, _, _ = synth.make_inputs(m, 1, k, seed=61, device=dev)
    y = (x.float() * 0.5).to(torch.bfloat16)
    q_o, s_o = oracle.quantize_rotated(bits16(x), block, "tensor")
    qy_o, sy_o = oracle.quantize_rotated(bits16(y), block, "tensor")
    qp_o, sp_o = oracle.quantize_tensorwise(bits16(y))
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    s = torch.empty(1, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ck.quantize_int8_rotated(x, block, mode="tensor", q=q, scale=s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ck.ck_int8_set_path_log(True)
    try:
        capfd.readouterr()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            ck.quantize_int8_rotated(x, block, mode="tensor", q=q, scale=s)
        torch.cuda.synchronize()
        for rep in range(3):
            q.zero_()
            s.zero_()
            qy, sy = ck.quantize_int8_rotated(y, block, mode="tensor")
            qp, sp = ck.quantize_int8_rowwise(y, mode="tensor")
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for got, want in ((s, s_o), (q, q_o), (sy, sy_o), (qy, qy_o), (sp, sp_o), (qp, qp_o)):
                np.testing.assert_array_equal(got.cpu().numpy(), want)
        lines = [l for l in capfd.readouterr().err.splitlines() if f" quantize {m}x{k} " in l]
    finally:
        ck.ck_int8_set_path_log(False)
    assert any("rotation" in l and "amax=four launches" in l for l in lines), lines
    assert any("rotation" in l and "amax=two launches" in l for l in lines), lines


@pytest.mark.parametrize("block", [16, 128])
def test_rotated_quantize_full_size_sampled(block):
    """Per-row rotated quantisation of the 80666 x 5376 activations (the
    largest workload's x): codes and scales of 200 sampled rows (the first
    and last 32, and seeded uniform rows) bit-exact against the oracle."""
    import torch
    dev = cuda_device()
    wl = synth.WORKLOADS[4]
    m, k = wl["m"], wl["k"]
    x, _, _, _ = synth.make_inputs(m, 1, k, seed=synth.workload_seed(4), device=dev)
    q, s = ck.quantize_int8_rotated(x, block)
    torch.cuda.synchronize()
    rows = set(range(32)) | set(range(m - 32, m))
    rows.update(int(v) for v in np.random.default_rng(block).integers(0, m, size=136))
    rows = np.array(sorted(rows), dtype=np.int64)
    ridx = torch.from_numpy(rows).to(dev)
    q_o, s_o = oracle.quantize_rotated(bits16(x.index_select(0, ridx)), block, "row")
    np.testing.assert_array_equal(s.index_select(0, ridx).cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.index_select(0, ridx).cpu().numpy(), q_o)

