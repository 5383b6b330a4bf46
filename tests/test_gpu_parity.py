"""HIP path vs the CPU oracle, element by element, on small and ragged shapes.

Codes, scales and int32 accumulators must be bit-exact; bf16 outputs within
1 bf16 ulp.  Every call goes through the C ABI (libck_int8.so)."""
import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import assert_bf16_within_1ulp, bits16, cuda_device

pytestmark = pytest.mark.gpu


def _inputs(m, n, k, mode="row", bias=False, seed=0):
    dev = cuda_device()
    return synth.make_inputs(m, n, k, mode=mode, bias=bias, seed=seed, device=dev)


# ---------------------------------------------------------------- quantise

@pytest.mark.parametrize("m,k", [(1, 16), (5, 2056), (274, 2048), (64, 8192), (9, 8200),
                                 (3, 20000), (130, 5376)])
def test_quantize_rowwise_bit_exact(m, k):
    import torch
    x, _, _, _ = _inputs(m, 1, k, seed=m + k)
    q, s = ck.quantize_int8_rowwise(x)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_rowwise(bits16(x))
    np.testing.assert_array_equal(s.cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)


def test_quantize_rowwise_strided_and_ragged():
    """k not a multiple of 8 (element tail) with padded rows in x and q."""
    import torch
    dev = cuda_device()
    m, k, ld = 33, 4100, 4104
    xfull, _, _, _ = synth.make_inputs(m, 1, ld, seed=3, device=dev)
    x = xfull[:, :k]
    qfull = torch.full((m, ld), 99, dtype=torch.int8, device=dev)
    q = qfull[:, :k]
    s = torch.empty(m, dtype=torch.float32, device=dev)
    ck.quantize_int8_rowwise(x, q=q, scale=s)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_rowwise(bits16(x))
    np.testing.assert_array_equal(s.cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    assert bool((qfull[:, k:] == 99).all()), "padding of q was written"


@pytest.mark.parametrize("m,k,ld", [(33, 1001, 1008), (5000, 260, 264), (2, 8195, 8200),
                                    (300, 16390, 16392)])
def test_quantize_tensorwise_strided_tail(m, k, ld):
    """Tensor-wide scale over rows whose stride is a multiple of 8 but whose
    length is not (the element tail after the 16-byte loads): one pass of 4
    or 16 chunks per lane, two passes (rows past 8192 elements), and more
    rows than one sweep of the grid (5000 > 256 blocks x 8 waves)."""
    import torch
    dev = cuda_device()
    xfull, _, _, _ = synth.make_inputs(m, 1, ld, mode="tensor", seed=m + k, device=dev)
    x = xfull[:, :k]
    qfull = torch.full((m, ld), 99, dtype=torch.int8, device=dev)
    q = qfull[:, :k]
    s = torch.empty(1, dtype=torch.float32, device=dev)
    ck.quantize_int8_rowwise(x, mode="tensor", q=q, scale=s)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_tensorwise(bits16(x))
    np.testing.assert_array_equal(s.cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    assert bool((qfull[:, k:] == 99).all()), "padding of q was written"


@pytest.mark.parametrize("m,k", [(7, 96), (4096, 4096), (3, 10008)])
def test_quantize_tensorwise_bit_exact(m, k):
    import torch
    x, _, _, _ = _inputs(m, 1, k, mode="tensor", seed=m * 3 + k)
    q, s = ck.quantize_int8_rowwise(x, mode="tensor")
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_tensorwise(bits16(x))
    np.testing.assert_array_equal(s.cpu().numpy(), s_o)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)


@pytest.mark.parametrize("amax", [1.0, 3.0, 5.5, 127.0, 448.0, 0.001953125,
                                  1.25 * 2.0 ** 127, 1.5 * 2.0 ** -100, 2.0 ** -130,
                                  2.0 ** -120, 2.0 ** 120])
def test_quantize_every_bf16_value(amax):
    """Every finite bf16 x with |x| <= amax, as one long row and as rows of
    4096 (each led by amax), against the oracle."""
    import torch
    dev = cuda_device()
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(b)
    a_bits = np.uint16(np.float32(amax).view(np.uint32) >> 16)
    vals = b[np.isfinite(f) & (np.abs(f) <= amax)]
    row = np.concatenate([[a_bits], vals])
    pad = (-row.size) % 16
    row = np.concatenate([row, np.zeros(pad, np.uint16)])
    for xb in (row[None, :], None):
        if xb is None:
            if row.size < 4095:
                continue
            r = row[: (row.size // 4095) * 4095].reshape(-1, 4095)
            xb = np.concatenate([np.full((r.shape[0], 1), a_bits, np.uint16), r], axis=1)
        xt = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        q, s = ck.quantize_int8_rowwise(xt)
        torch.cuda.synchronize()
        q_o, s_o = oracle.quantize_rowwise(xb)
        np.testing.assert_array_equal(s.cpu().numpy(), s_o)
        np.testing.assert_array_equal(q.cpu().numpy(), q_o)


def test_quantize_zero_rows():
    import torch
    dev = cuda_device()
    x = torch.zeros((6, 64), dtype=torch.bfloat16, device=dev)
    x[2, 5] = 1.5
    q, s = ck.quantize_int8_rowwise(x)
    torch.cuda.synchronize()
    assert s.cpu().tolist()[0] == 0.0 and s.cpu().tolist()[3] == 0.0
    assert int(q[2, 5]) == 127 and int(q.abs().sum()) == 127
    qt, st = ck.quantize_int8_rowwise(torch.zeros((3, 32), dtype=torch.bfloat16, device=dev),
                                      mode="tensor")
    torch.cuda.synchronize()
    assert float(st[0]) == 0.0 and int(qt.abs().sum()) == 0


# ---------------------------------------------------------------- int32 GEMM

SHAPES = [(1, 1, 16), (64, 64, 64), (300, 520, 2064), (257, 255, 1024), (37, 700, 80),
          (513, 129, 4096)]


@pytest.mark.parametrize("tile", range(ck.CK_NUM_TILES))
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_i32_bit_exact(tile, m, n, k):
    import torch
    dev = cuda_device()
    g = torch.Generator(device=dev).manual_seed(m * 7 + n * 3 + k + tile)
    q = torch.randint(-127, 128, (m, k), generator=g, device=dev, dtype=torch.int8)
    w = torch.randint(-128, 128, (n, k), generator=g, device=dev, dtype=torch.int8)
    acc = ck.int8_gemm_i32(q, w, tile=tile)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), oracle.gemm_i32(q.cpu().numpy(), w.cpu().numpy()))


@pytest.mark.parametrize("tile", [0, 3])
def test_gemm_i32_extreme_magnitude(tile):
    """Largest |acc| the int32 accumulator must hold: k * 127 * 128."""
    import torch
    dev = cuda_device()
    k = 132096
    q = torch.full((40, k), -127, dtype=torch.int8, device=dev)
    w = torch.full((33, k), -128, dtype=torch.int8, device=dev)
    w[1::2] = 127
    acc = ck.int8_gemm_i32(q, w, tile=tile)
    torch.cuda.synchronize()
    a = acc.cpu().numpy().astype(np.int64)
    assert np.all(a[:, 0::2] == k * 127 * 128)
    assert np.all(a[:, 1::2] == -k * 127 * 127)


def test_gemm_i32_strided_operands():
    import torch
    dev = cuda_device()
    m, n, k = 70, 90, 320
    g = torch.Generator(device=dev).manual_seed(5)
    qf = torch.randint(-127, 128, (m, k + 48), generator=g, device=dev, dtype=torch.int8)
    wf = torch.randint(-128, 128, (n, k + 16), generator=g, device=dev, dtype=torch.int8)
    q, w = qf[:, :k], wf[:, :k]
    outf = torch.full((m, n + 4), 7, dtype=torch.int32, device=dev)
    ck.int8_gemm_i32(q, w, out=outf[:, :n])
    torch.cuda.synchronize()
    ref = oracle.gemm_i32(q.cpu().numpy(), w.cpu().numpy())
    np.testing.assert_array_equal(outf[:, :n].cpu().numpy(), ref)
    assert bool((outf[:, n:] == 7).all())


# ---------------------------------------------------------------- fused linear

def _check_linear(m, n, k, tile, bias, x_mode, w_mode, seed):
    import torch
    x, w, ws, b = _inputs(m, n, k, mode=w_mode, bias=bias, seed=seed)
    q, xs = ck.quantize_int8_rowwise(x, mode=x_mode)
    out = ck.int8_linear_q(q, xs, w, ws, b, tile=tile)
    torch.cuda.synchronize()
    xb = bits16(x)
    q_o, s_o = (oracle.quantize_rowwise if x_mode == "row" else oracle.quantize_tensorwise)(xb)
    np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    np.testing.assert_array_equal(xs.cpu().numpy(), s_o)
    ref = oracle.linear(q_o, s_o, w.cpu().numpy(), ws.cpu().numpy(),
                        None if b is None else bits16(b))
    return assert_bf16_within_1ulp(bits16(out), ref, f"{m}x{n}x{k} tile {tile}")


@pytest.mark.parametrize("tile", range(ck.CK_NUM_TILES))
@pytest.mark.parametrize("m,n,k,bias", [(300, 520, 2064, True), (257, 255, 1024, False),
                                        (1, 40, 64, True), (520, 1030, 512, True)])
def test_linear_per_row(tile, m, n, k, bias):
    exact = _check_linear(m, n, k, tile, bias, "row", "row", seed=m + n + k)
    assert exact == 1.0, f"bit-identical fraction {exact}"


@pytest.mark.parametrize("tile", [11, 12, 13])
def test_linear_more_tiles_than_cus(tile):
    """17 x 17 = 289 block tiles of 256 x 256, more than one per compute unit,
    with a ragged last row and column of tiles, checked in full."""
    exact = _check_linear(4133, 4155, 384, tile, True, "row", "row", seed=4133)
    assert exact == 1.0, f"bit-identical fraction {exact}"


@pytest.mark.parametrize("x_mode,w_mode", [("tensor", "tensor"), ("row", "tensor"),
                                           ("tensor", "row")])
def test_linear_scale_modes(x_mode, w_mode):
    exact = _check_linear(200, 300, 768, -1, True, x_mode, w_mode, seed=11)
    assert exact == 1.0


def test_linear_k_zero_gives_bias():
    import torch
    dev = cuda_device()
    m, n = 5, 24
    q = torch.empty((m, 0), dtype=torch.int8, device=dev)
    w = torch.empty((n, 0), dtype=torch.int8, device=dev)
    xs = torch.ones(m, device=dev)
    ws = torch.ones(n, device=dev)
    b = (torch.arange(n, device=dev, dtype=torch.float32) * 0.25 - 2).to(torch.bfloat16)
    out = ck.int8_linear_q(q, xs, w, ws, b)
    out0 = ck.int8_linear_q(q, xs, w, ws, None)
    torch.cuda.synchronize()
    assert torch.equal(out, b.expand(m, n))
    assert bool((out0 == 0).all())


def test_linear_empty_is_noop():
    import torch
    dev = cuda_device()
    w = torch.zeros((8, 64), dtype=torch.int8, device=dev)
    q = torch.zeros((0, 64), dtype=torch.int8, device=dev)
    out = ck.int8_linear_q(q, torch.ones(1, device=dev), w, torch.ones(8, device=dev))
    assert out.shape == (0, 8)


def test_linear_strided_output_and_odd_n():
    """ldo > n and n not a multiple of 4 (element-wise stores)."""
    import torch
    dev = cuda_device()
    m, n, k = 130, 37, 256
    x, w, ws, b = synth.make_inputs(m, n, k, bias=True, seed=21, device=dev)
    q, xs = ck.quantize_int8_rowwise(x)
    for ldo in (37, 40, 45):
        full = torch.full((m, ldo), 3.0, dtype=torch.bfloat16, device=dev)
        ck.int8_linear_q(q, xs, w, ws, b, out=full[:, :n])
        torch.cuda.synchronize()
        ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(),
                            ws.cpu().numpy(), bits16(b))
        assert assert_bf16_within_1ulp(bits16(full[:, :n]), ref) == 1.0
        assert bool((full[:, n:] == 3.0).all())


def test_linear_end_to_end_error_about_one_percent():
    """Issue #136, "Measured boundary": ~1 % against a bf16 reference."""
    import torch
    x, w, ws, b = _inputs(256, 512, 2048, seed=99)
    out = ck.int8_linear(x, w, ws)
    ref = x.float() @ (w.float() * ws[:, None]).t()
    rel = float((out.float() - ref).norm() / ref.norm())
    assert 0.005 < rel < 0.012, rel


def test_quantize_tensorwise_repeated_and_two_streams():
    """The tensor-wide amax goes through one of two cells of the stream's
    counter block, alternating from call to call (each call clears the cell
    the next one uses).  Consecutive calls with different data (the second
    one with a smaller amax), and calls on two streams at once, each give the
    oracle's codes and scale."""
    import torch
    dev = cuda_device()
    xs = []
    for seed, gain in ((21, 4.0), (22, 0.25), (23, 1.0)):
        x, _, _, _ = _inputs(1000, 1, 3000, mode="tensor", seed=seed)
        xs.append((x.float() * gain).to(torch.bfloat16))
    refs = [oracle.quantize_tensorwise(bits16(x)) for x in xs]
    for x, (q_o, s_o) in zip(xs, refs):
        q, s = ck.quantize_int8_rowwise(x, mode="tensor")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(s.cpu().numpy(), s_o)
        np.testing.assert_array_equal(q.cpu().numpy(), q_o)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(2):
        for st, x in zip((s1, s2, s1), xs):
            with torch.cuda.stream(st):
                outs.append(ck.quantize_int8_rowwise(x, mode="tensor"))
    torch.cuda.synchronize()
    for j, (q, s) in enumerate(outs):
        q_o, s_o = refs[j % 3]
        np.testing.assert_array_equal(s.cpu().numpy(), s_o)
        np.testing.assert_array_equal(q.cpu().numpy(), q_o)


def test_quantize_tensorwise_under_graph_capture(capfd):
    """Under graph capture the tensor-wide quantisation takes the four-launch
    chain, with scale[0] as its amax cell (no stream counters in a graph).
    Eager calls take the two-launch chain.  Three replays, each after an
    eager call on other data on the default stream (which flips that
    stream's amax cells), give the oracle's codes and scale, and so do the
    eager calls."""
    import torch
    dev = cuda_device()
    x, _, _, _ = _inputs(777, 1, 2056, mode="tensor", seed=41)
    y = (x.float() * 3.0).to(torch.bfloat16)
    q_o, s_o = oracle.quantize_tensorwise(bits16(x))
    qy_o, sy_o = oracle.quantize_tensorwise(bits16(y))
    q = torch.empty(x.shape, dtype=torch.int8, device=dev)
    s = torch.empty(1, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ck.quantize_int8_rowwise(x, mode="tensor", q=q, scale=s)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ck.ck_int8_set_path_log(True)
    try:
        capfd.readouterr()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            ck.quantize_int8_rowwise(x, mode="tensor", q=q, scale=s)
        torch.cuda.synchronize()
        for rep in range(3):
            q.zero_()
            s.zero_()
            qy, sy = ck.quantize_int8_rowwise(y, mode="tensor")
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(s.cpu().numpy(), s_o)
            np.testing.assert_array_equal(q.cpu().numpy(), q_o)
            np.testing.assert_array_equal(sy.cpu().numpy(), sy_o)
            np.testing.assert_array_equal(qy.cpu().numpy(), qy_o)
        lines = [l for l in capfd.readouterr().err.splitlines() if " quantize 777x2056 " in l]
    finally:
        ck.ck_int8_set_path_log(False)
    assert any("amax=four launches" in l for l in lines), lines
    assert any("amax=two launches" in l for l in lines), lines


def test_quantize_tensorwise_threads_sharing_a_stream():
    """Host threads that quantise tensor-wide on one stream at the same time
    share that stream's two amax cells; the cell is chosen under a lock held
    across both launches of a call, so every call still gets the oracle's
    codes and scale.  (ctypes releases the GIL, so the calls overlap in the
    library.)"""
    import threading
    import torch
    cuda_device()
    xs = []
    for seed, gain in ((51, 1.0), (52, 8.0), (53, 0.125), (54, 2.0)):
        x, _, _, _ = _inputs(300, 1, 1040, mode="tensor", seed=seed)
        xs.append((x.float() * gain).to(torch.bfloat16))
    refs = [oracle.quantize_tensorwise(bits16(x)) for x in xs]
    stream = torch.cuda.current_stream()
    results = [[] for _ in xs]
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(stream):
                for _ in range(25):
                    results[i].append(ck.quantize_int8_rowwise(xs[i], mode="tensor"))
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(xs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (q_o, s_o) in enumerate(refs):
        assert len(results[i]) == 25
        for q, s in results[i]:
            np.testing.assert_array_equal(s.cpu().numpy(), s_o)
            np.testing.assert_array_equal(q.cpu().numpy(), q_o)

