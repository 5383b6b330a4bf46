"""Seeded synthetic inputs and output-row sampling for the INT8 linear layer.

This module holds no step of the layer's arithmetic.  It only draws the
inputs (the recipe of the minimal reproduction in comfy-kitchen issue #136,
section "Minimal reproduction": x ~ randn in bf16, W ~ randint(-127, 127) in
int8, w_scale ~ rand * 0.01 in fp32) and chooses which output rows a
checker looks at.  Both the HIP path's tests and the CPU oracle's tests take
their inputs from here; neither side's arithmetic lives here.
"""
from __future__ import annotations

import numpy as np

TWO31 = 2 ** 31

# The five workloads the layer is measured and checked on.  Shapes are
# (m tokens, n output features, k input features).  "row": one x scale per
# token row and one w scale per output column; "tensor": one scale for all of
# x and one for all of W.
WORKLOADS = [
    dict(name="274x2048x2048 per-row", m=274, n=2048, k=2048, mode="row", bias=False),
    dict(name="4096x4096x4096 tensorwise", m=4096, n=4096, k=4096, mode="tensor", bias=False),
    dict(name="25900x16384x4096 per-row+bias", m=25900, n=16384, k=4096, mode="row", bias=True),
    dict(name="99900x21504x5376 per-row", m=99900, n=21504, k=5376, mode="row", bias=False),
    dict(name="80666x28672x5376 per-row+bias", m=80666, n=28672, k=5376, mode="row", bias=True),
]

SEED_BASE = 20261202


def workload_seed(index: int) -> int:
    return SEED_BASE + 16 * index


def make_inputs(m, n, k, mode="row", bias=False, seed=0, device="cpu"):
    """Draw (x bf16 [m,k], w int8 [n,k], w_scale fp32 [n] or [1], bias bf16 [n] or None).

    Draw order is fixed: x, W, w_scale, bias.  Torch tensors on `device`."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn((m, k), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    w = torch.randint(-127, 127, (n, k), generator=g, device=device, dtype=torch.int8)
    ns = n if mode == "row" else 1
    w_scale = torch.rand((ns,), generator=g, device=device, dtype=torch.float32) * 0.01
    b = None
    if bias:
        b = (torch.randn((n,), generator=g, device=device, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    return x, w, w_scale, b


def make_inputs_chunked(m, n, k, mode="row", bias=False, seed=0, device="cuda", chunk_rows=8192):
    """Same recipe as make_inputs but x is drawn in row chunks, so that a
    multi-GB x never needs a multi-GB fp32 temporary.  Chunk c of x is drawn
    from its own generator seeded with seed + 1 + c."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    w = torch.randint(-127, 127, (n, k), generator=g, device=device, dtype=torch.int8)
    ns = n if mode == "row" else 1
    w_scale = torch.rand((ns,), generator=g, device=device, dtype=torch.float32) * 0.01
    b = None
    if bias:
        b = (torch.randn((n,), generator=g, device=device, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    x = torch.empty((m, k), device=device, dtype=torch.bfloat16)
    for c, r0 in enumerate(range(0, m, chunk_rows)):
        r1 = min(m, r0 + chunk_rows)
        gc = torch.Generator(device=device)
        gc.manual_seed(int(seed) + 1 + c)
        x[r0:r1] = torch.randn((r1 - r0, k), generator=gc, device=device,
                               dtype=torch.float32).to(torch.bfloat16)
    return x, w, w_scale, b


def boundary_rows(m: int, n: int, k: int):
    """First rows at which 32-bit offsets would wrap.

    Returns a dict name -> first row index r such that some element of row r
    lies at or past the limit:
      out_elem_2^31  : element offset r*n + c >= 2^31 (the int32 law of
                       issue #136, section "Summary");
      out_byte_2^31/2^32 : bf16 output byte offsets;
      q_byte_2^31/2^32   : int8 activation byte offsets (m*k);
      x_byte_2^31/2^32   : bf16 activation byte offsets."""
    def first_row(limit, row_len):
        # smallest r with r*row_len + (row_len - 1) >= limit
        return limit // row_len

    return {
        "out_elem_2^31": first_row(TWO31, n),
        "out_byte_2^31": first_row(TWO31, 2 * n),
        "out_byte_2^32": first_row(2 * TWO31, 2 * n),
        "q_byte_2^31": first_row(TWO31, k),
        "q_byte_2^32": first_row(2 * TWO31, k),
        "x_byte_2^31": first_row(TWO31, 2 * k),
        "x_byte_2^32": first_row(2 * TWO31, 2 * k),
    }


def sample_rows(m: int, n: int, k: int, count: int = 4096, seed: int = 0,
                tile: int = 256, window: int = 64, min_random: int = 1024):
    """Sorted unique output rows for a sampled check of an [m, n] result.

    Always includes rows 0..window-1, the last two row tiles, +-window rows
    around each 32-bit wrap boundary that falls inside m, and every row from
    the first row holding an element at or past 2^31 to the end.  Seeded
    uniform rows then fill the set up to `count` rows, and at least
    `min_random` of them are added in any case (all rows if m <= count)."""
    if m <= count:
        return np.arange(m, dtype=np.int64)
    rows = set(range(min(window, m)))
    rows.update(range(max(0, m - 2 * tile), m))
    b = boundary_rows(m, n, k)
    for r in b.values():
        if r < m:
            rows.update(range(max(0, r - window), min(m, r + window)))
    r31 = b["out_elem_2^31"]
    if r31 < m:
        rows.update(range(max(0, r31 - 1), m))
    rng = np.random.default_rng(seed)
    target = max(count, len(rows) + min_random)
    while len(rows) < target:
        rows.update(int(v) for v in rng.integers(0, m, size=target - len(rows)))
    return np.array(sorted(rows), dtype=np.int64)
