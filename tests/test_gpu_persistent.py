"""Tile 13, the persistent form of tile 12, against the oracle: one block per
compute unit walks several 256 x 256 output tiles, so the tests use more
tiles than compute units (256), ragged last tiles, both 16-bit output types,
both scale modes, with and without a bias, and K of one, two and three
128-byte stages.  The same arithmetic as every other tile ("Exactness" of
the output types): bit-identical results are expected, within 1 ulp is the
bar.  Calls go through the C ABI (libck_int8.so)."""
import numpy as np
import pytest

import int8_weight_quantized_amd as ck
from int8_weight_quantized_amd import synth
import oracle
from tests.gpu_util import assert_within_1ulp, bits16, cuda_device

pytestmark = pytest.mark.gpu

TILE = 13


def _inputs(m, n, k, out_dtype, x_mode, w_mode, bias, seed):
    import torch
    dev = cuda_device()
    x, w, ws, b = synth.make_inputs(m, n, k, mode=w_mode, bias=bias, seed=seed, device=dev)
    q, xs = ck.quantize_int8_rowwise(x, mode=x_mode)
    if b is not None:
        b = b.to(torch.float16 if out_dtype == "fp16" else torch.bfloat16)
    return q, xs, w, ws, b


@pytest.mark.parametrize("out_dtype,x_mode,w_mode,bias,k", [
    ("bf16", "row", "row", True, 256),
    ("fp16", "row", "row", True, 128),
    ("bf16", "tensor", "tensor", False, 384),
    ("fp16", "row", "tensor", False, 256),
    ("bf16", "tensor", "row", True, 128),
])
def test_persistent_walk_matches_oracle(out_dtype, x_mode, w_mode, bias, k):
    """19 x 18 = 342 tiles on 256 blocks (blocks 0..85 take a second tile);
    the last row of tiles has 92 rows and the last column 216 columns."""
    import torch
    m, n = 4700, 4568
    q, xs, w, ws, b = _inputs(m, n, k, out_dtype, x_mode, w_mode, bias, seed=m + k)
    out = ck.int8_linear_q(q, xs, w, ws, b, tile=TILE, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(), ws.cpu().numpy(),
                        None if b is None else bits16(b), out_dtype)
    exact = assert_within_1ulp(bits16(out), ref, f"{out_dtype} {x_mode}/{w_mode} k={k}")
    assert exact == 1.0, exact


def test_persistent_odd_width_and_strided_output():
    """n odd inside a wider output buffer (ldo > n): element stores on every
    row; the columns past n keep their contents."""
    import torch
    m, n, k, ldo = 4133, 4155, 384, 4160
    q, xs, w, ws, b = _inputs(m, n, k, "bf16", "row", "row", True, seed=9)
    buf = torch.full((m, ldo), 7.0, dtype=torch.bfloat16, device=q.device)
    out = buf[:, :n]
    ck.int8_linear_q(q, xs, w, ws, b, out=out, tile=TILE)
    torch.cuda.synchronize()
    ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(), ws.cpu().numpy(),
                        bits16(b))
    assert assert_within_1ulp(bits16(out), ref, "odd n") == 1.0
    assert bool((buf[:, n:] == 7.0).all())


def test_persistent_equals_tile12_at_full_size_sampled():
    """80666 x 28672 x 5376 with bias (outputs past 2^31 elements): tile 13
    and tile 12 give the same bits everywhere, and sampled rows agree with
    the oracle row by row."""
    import torch
    m, n, k = 80666, 28672, 5376
    q, xs, w, ws, b = _inputs(m, n, k, "bf16", "row", "row", True, seed=4)
    out13 = ck.int8_linear_q(q, xs, w, ws, b, tile=TILE)
    out12 = ck.int8_linear_q(q, xs, w, ws, b, tile=12)
    torch.cuda.synchronize()
    assert torch.equal(out13.view(torch.int16), out12.view(torch.int16))
    del out12
    rows = np.array([0, 1, 255, 256, 40000, 74899, m - 92, m - 1])   # row 74899 on: past 2^31
    wh, wsh, bh = w.cpu().numpy(), ws.cpu().numpy(), bits16(b)
    idx = torch.as_tensor(rows, device=q.device)
    qh, xsh = q[idx].cpu().numpy(), xs[idx].cpu().numpy()
    got = bits16(out13[idx])
    ref = oracle.linear(qh, xsh, wh, wsh, bh)
    assert assert_within_1ulp(got, ref, "sampled rows") == 1.0


def test_persistent_path_log(capfd):
    """With more tiles than compute units and k a multiple of 128 the log
    names the persistent kernel; otherwise tile 13 runs tile 12's kernel."""
    import torch
    cuda_device()
    ck.ck_int8_set_path_log(True)
    try:
        capfd.readouterr()
        for m, n, k in ((4352, 4352, 256), (4352, 4352, 272), (512, 512, 256)):
            q, xs, w, ws, b = _inputs(m, n, k, "bf16", "row", "row", True, seed=k)
            ck.int8_linear_q(q, xs, w, ws, b, tile=TILE)
        torch.cuda.synchronize()
        lines = [l for l in capfd.readouterr().err.splitlines() if " gemm " in l]
        by = {l.split(" gemm ")[1].split()[0]: l for l in lines}
        assert "persistent" in by["4352x4352x256"] and "blocks=256" in by["4352x4352x256"]
        assert "persistent" not in by["4352x4352x272"]
        assert "persistent" not in by["512x512x256"]
    finally:
        ck.ck_int8_set_path_log(False)


def test_persistent_back_to_back_and_two_streams():
    """Launches of different sizes back to back on one stream, then two at
    once on two streams: each stream's tile counters start from zero every
    time, so every launch covers all its tiles exactly once (same bits as
    tile 12, and the oracle on one of them)."""
    import torch
    dev = cuda_device()
    shapes = [(4700, 4568, 256), (2600, 8000, 128), (4133, 4400, 384)]
    cases = []
    for i, (m, n, k) in enumerate(shapes):
        q, xs, w, ws, b = _inputs(m, n, k, "bf16", "row", "row", True, seed=100 + i)
        ref12 = ck.int8_linear_q(q, xs, w, ws, b, tile=12)
        cases.append((q, xs, w, ws, b, ref12))
    for _ in range(2):
        for q, xs, w, ws, b, ref12 in cases:
            out = ck.int8_linear_q(q, xs, w, ws, b, tile=TILE)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref12.view(torch.int16))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for st, (q, xs, w, ws, b, _) in zip((s1, s2, s1), cases):
            with torch.cuda.stream(st):
                outs.append(ck.int8_linear_q(q, xs, w, ws, b, tile=TILE))
    torch.cuda.synchronize()
    for j, out in enumerate(outs):
        assert torch.equal(out.view(torch.int16), cases[j % 3][5].view(torch.int16)), j
    q, xs, w, ws, b, _ = cases[1]
    ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(), ws.cpu().numpy(),
                        bits16(b))
    assert assert_within_1ulp(bits16(outs[1]), ref, "second stream") == 1.0


def test_persistent_longest_k_sampled():
    """K = 132096 (the largest the int32 accumulator allows at full code
    magnitude), 342 tiles: 1032 K stages per tile on the persistent kernel.
    Codes of extreme magnitude in the first rows put the accumulators at
    k * 127 * 128; the whole output equals tile 12's, and sampled rows the
    oracle's."""
    import torch
    dev = cuda_device()
    m, n, k = 4700, 4568, 132096
    g = torch.Generator(device=dev).manual_seed(7)
    q = torch.randint(-127, 128, (m, k), generator=g, device=dev, dtype=torch.int8)
    w = torch.randint(-128, 128, (n, k), generator=g, device=dev, dtype=torch.int8)
    q[:2] = -127
    w[:3] = -128
    xs = torch.rand(m, generator=g, device=dev) * 1e-6 + 1e-7
    ws = torch.rand(n, generator=g, device=dev) * 1e-3 + 1e-4
    b = (torch.rand(n, generator=g, device=dev) - 0.5).to(torch.bfloat16)
    out13 = ck.int8_linear_q(q, xs, w, ws, b, tile=TILE)
    out12 = ck.int8_linear_q(q, xs, w, ws, b, tile=12)
    torch.cuda.synchronize()
    assert torch.equal(out13.view(torch.int16), out12.view(torch.int16))
    rows = np.array([0, 1, 2, 2047, m - 1])
    idx = torch.as_tensor(rows, device=dev)
    ref = oracle.linear(q[idx].cpu().numpy(), xs[idx].cpu().numpy(), w.cpu().numpy(),
                        ws.cpu().numpy(), bits16(b))
    assert assert_within_1ulp(bits16(out13[idx]), ref, "k=132096") == 1.0


def test_persistent_tile_under_graph_capture():
    """Under graph capture tile 13 runs tile 12's kernel (no shared tile
    counters in a graph).  Three replays, with eager persistent launches on
    the default stream in between, each checked against the eager result."""
    import torch
    dev = cuda_device()
    m, n, k = 4700, 4568, 256
    q, xs, w, ws, b = _inputs(m, n, k, "bf16", "row", "row", True, seed=31)
    ref = ck.int8_linear_q(q, xs, w, ws, b, tile=12)
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ck.int8_linear_q(q, xs, w, ws, b, out=out, tile=TILE)      # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ck.int8_linear_q(q, xs, w, ws, b, out=out, tile=TILE)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        eager = ck.int8_linear_q(q, xs, w, ws, b, tile=TILE)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        assert torch.equal(eager.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.parametrize("k", [128, 384, 5376])
def test_persistent_int32_accumulators(k, capfd):
    """ck_int8_gemm_i32 at tile 13 runs the persistent kernel's tile walk
    and main loop with an int32 epilogue: every accumulator of a ragged
    342-tile shape equals the oracle's exact sum, into a wider buffer whose
    extra columns keep their contents, and the path log names the
    persistent kernel."""
    import torch
    m, n, ldacc = 4700, 4568, 4576
    dev = cuda_device()
    x, w, _, _ = synth.make_inputs(m, n, k, mode="row", seed=k + 3, device=dev)
    q, _ = ck.quantize_int8_rowwise(x)
    buf = torch.full((m, ldacc), -5, dtype=torch.int32, device=dev)
    ck.ck_int8_set_path_log(True)
    try:
        capfd.readouterr()
        ck.int8_gemm_i32(q, w, tile=TILE, out=buf[:, :n])
        torch.cuda.synchronize()
        err = capfd.readouterr().err
    finally:
        ck.ck_int8_set_path_log(False)
    assert any(f"gemm {m}x{n}x{k} out=int32 tile=13" in l and "persistent" in l
               for l in err.splitlines()), err
    np.testing.assert_array_equal(buf[:, :n].cpu().numpy(),
                                  oracle.gemm_i32(q.cpu().numpy(), w.cpu().numpy()))
    assert bool((buf[:, n:] == -5).all())


def test_int32_accumulators_off_the_persistent_path():
    """k not a multiple of 128 (tile 13 then runs tile 12's kernel, with a
    K tail) and too few tiles for the persistent kernel: still exact."""
    import torch
    dev = cuda_device()
    for m, n, k in ((4700, 4568, 200), (700, 900, 256)):
        x, w, _, _ = synth.make_inputs(m, n, k, mode="row", seed=m + k, device=dev)
        w = ck.pad_rows(w)                    # rows 16 bytes apart for k = 200
        q, _ = ck.quantize_int8_rowwise(x)
        acc = ck.int8_gemm_i32(q, w, tile=TILE)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(),
                                      oracle.gemm_i32(q.cpu().numpy(), w.cpu().numpy()))


@pytest.mark.parametrize("tile", [3, 12, 13])
def test_group_larger_than_the_row_tiles(tile):
    """A launch-order group of 2^31 - 1 row tiles is clamped to the row
    tiles there are; the results are the oracle's."""
    import torch
    m, n, k = 4700, 4568, 256
    q, xs, w, ws, b = _inputs(m, n, k, "bf16", "row", "row", True, seed=31)
    out = ck.int8_linear_q(q, xs, w, ws, b, tile=tile, group_m=2 ** 31 - 1)
    torch.cuda.synchronize()
    ref = oracle.linear(q.cpu().numpy(), xs.cpu().numpy(), w.cpu().numpy(), ws.cpu().numpy(),
                        bits16(b))
    assert assert_within_1ulp(bits16(out), ref, f"tile {tile} group 2^31-1") == 1.0
