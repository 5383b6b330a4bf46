"""The C ABI on the host: the library loads, exports what include/ck_int8.h
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import os
import re

import pytest

import int8_weight_quantized_amd as ck

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "ck_int8.h")
P = 4096          # a stand-in device address: validation never dereferences it


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(ck_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("ck_quantize_int8_rowwise", "ck_int8_linear", "ck_int8_gemm_i32",
              "ck_status_string", "ck_last_error"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = ck.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(ck.EXPORTED) == declared_functions()


def test_abi_version_and_status_strings():
    assert ck.lib().ck_abi_version() == ck.CK_ABI_VERSION
    assert ck.ck_status_string(0) == "CK_OK"
    assert ck.ck_status_string(2) == "CK_ERR_UNSUPPORTED"
    assert ck.ck_status_string(99) == "CK_ERR_UNKNOWN"


def _linear(**kw):
    a = dict(q=P, ldq=64, x_scale=P, x_mode=1, w=P, ldw=64, w_scale=P, w_mode=1, bias=0,
             out=P, ldo=32, m=16, n=32, k=64)
    a.update(kw)
    return ck.lib().ck_int8_linear(a["q"], a["ldq"], a["x_scale"], a["x_mode"], a["w"],
                                   a["ldw"], a["w_scale"], a["w_mode"], a["bias"], a["out"],
                                   a["ldo"], a["m"], a["n"], a["k"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), ck.CK_ERR_INVALID_ARG),
    (dict(w=0), ck.CK_ERR_INVALID_ARG),
    (dict(out=0), ck.CK_ERR_INVALID_ARG),
    (dict(x_scale=0), ck.CK_ERR_INVALID_ARG),
    (dict(m=-1), ck.CK_ERR_INVALID_ARG),
    (dict(k=-16), ck.CK_ERR_INVALID_ARG),
    (dict(ldq=48), ck.CK_ERR_INVALID_ARG),
    (dict(ldo=31), ck.CK_ERR_INVALID_ARG),
    (dict(x_mode=7), ck.CK_ERR_INVALID_ARG),
    (dict(k=40, ldq=48, ldw=48), ck.CK_ERR_HIP),           # any k, with 16-byte rows
    (dict(k=40, ldq=40, ldw=48), ck.CK_ERR_UNSUPPORTED),   # q rows not 16 bytes apart
    (dict(k=132112, ldq=132112, ldw=132112), ck.CK_ERR_UNSUPPORTED),
    (dict(ldq=72), ck.CK_ERR_UNSUPPORTED),
    (dict(q=P + 8), ck.CK_ERR_UNSUPPORTED),
    (dict(m=0), ck.CK_OK),
    (dict(n=0, out=0), ck.CK_OK),
    (dict(k=0, q=0, w=0), ck.CK_ERR_HIP),   # nothing to read: validation passes
])
def test_linear_validation(kw, status):
    import torch
    if status == ck.CK_ERR_HIP and torch.cuda.is_available():
        pytest.skip("needs the no-GPU host")
    assert _linear(**kw) == status
    if status != ck.CK_OK:
        assert ck.ck_last_error() != ""


def test_tiled_rejects_unknown_tile():
    L = ck.lib()
    r = L.ck_int8_linear_tiled(P, 64, P, 1, P, 64, P, 1, 0, P, 32, 16, 32, 64, ck.CK_NUM_TILES, 0, 0)
    assert r == ck.CK_ERR_INVALID_ARG
    r = L.ck_int8_linear_tiled(P, 64, P, 1, P, 64, P, 1, 0, P, 32, 16, 32, 64, 0, -2, 0)
    assert r == ck.CK_ERR_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    ((P, 4, 64, 64, P, 64, P, 5), ck.CK_ERR_INVALID_ARG),     # bad mode
    ((P, 4, 64, 64, P, 64, 0, 1), ck.CK_ERR_INVALID_ARG),     # NULL scale
    ((0, 4, 64, 64, P, 64, P, 1), ck.CK_ERR_INVALID_ARG),     # NULL x
    ((P, 4, 64, 60, P, 64, P, 1), ck.CK_ERR_INVALID_ARG),     # ldx < k
    ((P + 1, 4, 64, 64, P, 64, P, 1), ck.CK_ERR_UNSUPPORTED), # x not 2-byte aligned
    ((P, 4, 64, 68, P, 64, P, 1), ck.CK_ERR_HIP),             # any ldx (element kernel)
    ((P + 2, 4, 64, 64, P, 64, P, 1), ck.CK_ERR_HIP),         # x rows not 16-byte aligned
    ((P, 4, 64, 64, P + 4, 64, P, 1), ck.CK_ERR_HIP),         # q rows not 8-byte aligned
    ((P, 4, 61, 61, P, 61, P, 1), ck.CK_ERR_HIP),             # odd k
    ((P, 0, 64, 64, P, 64, P, 1), ck.CK_OK),                  # empty, per row
])
def test_quantize_validation(args, status):
    import torch
    if status == ck.CK_ERR_HIP and torch.cuda.is_available():
        pytest.skip("needs the no-GPU host")
    assert ck.lib().ck_quantize_int8_rowwise(*args, 0) == status


@pytest.mark.parametrize("args,status", [
    ((P, 4, 64, 64, 3, P, 64, P, 1), ck.CK_ERR_INVALID_ARG),     # block not a power of two
    ((P, 4, 64, 64, 1024, P, 64, P, 1), ck.CK_ERR_INVALID_ARG),  # block > 512
    ((P, 4, 96, 96, 64, P, 96, P, 1), ck.CK_ERR_INVALID_ARG),    # k % block
    ((P, 4, 36, 40, 4, P, 40, P, 1), ck.CK_ERR_UNSUPPORTED),     # k % 8
    ((P, 4, 64, 68, 16, P, 64, P, 1), ck.CK_ERR_UNSUPPORTED),    # x rows not 16-byte aligned
    ((P, 4, 64, 64, 16, P + 4, 64, P, 1), ck.CK_ERR_UNSUPPORTED),  # q rows not 8-byte aligned
    ((P, 4, 64, 64, 16, P, 64, P, 9), ck.CK_ERR_INVALID_ARG),    # bad mode
    ((P, 0, 64, 64, 16, P, 64, P, 1), ck.CK_OK),
    ((P, 4, 64, 64, 16, P, 64, P, 1), ck.CK_ERR_HIP),
])
def test_quantize_rotated_validation(args, status):
    import torch
    if status == ck.CK_ERR_HIP and torch.cuda.is_available():
        pytest.skip("needs the no-GPU host")
    assert ck.lib().ck_quantize_int8_rotated(*args, 0) == status


@pytest.mark.parametrize("args,status", [
    # x, ldx, w, ldw, w_scale, w_mode, bias, out, ldo, out_dtype, m, n, k
    ((P, 64, P, 64, P, 1, 0, P, 32, 0, 16, 32, 64), ck.CK_ERR_HIP),
    ((P, 64, P, 64, P, 1, 0, P, 32, 4, 16, 32, 64), ck.CK_ERR_INVALID_ARG),   # out_dtype
    ((P, 64, P, 64, P, 3, 0, P, 32, 0, 16, 32, 64), ck.CK_ERR_INVALID_ARG),   # w_mode
    ((0, 64, P, 64, P, 1, 0, P, 32, 0, 16, 32, 64), ck.CK_ERR_INVALID_ARG),   # NULL x
    ((P, 60, P, 64, P, 1, 0, P, 32, 0, 16, 32, 64), ck.CK_ERR_INVALID_ARG),   # ldx < k
    ((P, 68, P, 64, P, 1, 0, P, 32, 0, 16, 32, 64), ck.CK_ERR_UNSUPPORTED),   # ldx % 8
    ((P, 64, P, 72, P, 1, 0, P, 32, 0, 16, 32, 64), ck.CK_ERR_UNSUPPORTED),   # ldw % 16
    ((P, 64, P, 64, P, 1, 0, P + 2, 32, 2, 16, 32, 64), ck.CK_ERR_UNSUPPORTED),  # fp32 out
    ((P, 64, P, 64, P, 1, 0, P, 32, 0, 0, 32, 64), ck.CK_OK),
    ((0, 0, 0, 0, P, 1, 0, P, 32, 0, 16, 32, 0), ck.CK_ERR_HIP),             # k = 0
    ((P, 1 << 24, P, 64, P, 1, 0, P, 32, 0, 16, 32, 64), ck.CK_ERR_UNSUPPORTED),   # x lane offsets
    ((P, 64, P, 1 << 26, P, 1, 0, P, 32, 0, 64, 32, 64), ck.CK_ERR_UNSUPPORTED),   # W lane offsets
    ((P, 64, P, 1 << 25, P, 1, 0, P, 32, 0, 65, 32, 64), ck.CK_ERR_UNSUPPORTED),   # W tile offsets
])
def test_linear_dequant_validation(args, status):
    import torch
    if status == ck.CK_ERR_HIP and torch.cuda.is_available():
        pytest.skip("needs the no-GPU host")
    assert ck.lib().ck_int8_linear_dequant(*args, 0) == status


def _linear_ex(**kw):
    a = dict(q=P, ldq=64, x_scale=P, x_mode=1, w=P, ldw=64, w_scale=P, w_mode=1, bias=0,
             out=P, ldo=32, out_dtype=ck.CK_OUT_FP32, m=16, n=32, k=64, tile=-1, group_m=0)
    a.update(kw)
    return ck.lib().ck_int8_linear_ex(*a.values(), 0)


@pytest.mark.parametrize("kw,status", [
    (dict(out_dtype=3), ck.CK_ERR_INVALID_ARG),
    (dict(out_dtype=-1), ck.CK_ERR_INVALID_ARG),
    (dict(out=P + 2), ck.CK_ERR_UNSUPPORTED),                  # fp32 out needs 4-byte alignment
    (dict(bias=P + 2), ck.CK_ERR_UNSUPPORTED),
    (dict(out=P + 2, out_dtype=ck.CK_OUT_FP16), ck.CK_ERR_HIP),
    (dict(tile=ck.CK_NUM_TILES), ck.CK_ERR_INVALID_ARG),
    (dict(m=0), ck.CK_OK),
    (dict(), ck.CK_ERR_HIP),
])
def test_linear_ex_validation(kw, status):
    import torch
    if status == ck.CK_ERR_HIP and torch.cuda.is_available():
        pytest.skip("needs the no-GPU host")
    assert _linear_ex(**kw) == status


def _layer(**kw):
    a = dict(x=P, ldx=64, q=P, ldq=64, x_scale=P, x_mode=1, w=P, ldw=64, w_scale=P, w_mode=1,
             bias=0, out=P, ldo=32, out_dtype=ck.CK_OUT_BF16, m=16, n=32, k=64, fused=-1)
    a.update(kw)
    return ck.lib().ck_int8_layer(*a.values(), 0)


@pytest.mark.parametrize("kw,status", [
    (dict(fused=2), ck.CK_ERR_INVALID_ARG),
    (dict(fused=-2), ck.CK_ERR_INVALID_ARG),
    (dict(out_dtype=3), ck.CK_ERR_INVALID_ARG),
    (dict(x_mode=5), ck.CK_ERR_INVALID_ARG),
    (dict(w_mode=-1), ck.CK_ERR_INVALID_ARG),
    (dict(x=0), ck.CK_ERR_INVALID_ARG),
    (dict(q=0), ck.CK_ERR_INVALID_ARG),
    (dict(x_scale=0), ck.CK_ERR_INVALID_ARG),
    (dict(w_scale=0), ck.CK_ERR_INVALID_ARG),
    (dict(ldx=60), ck.CK_ERR_INVALID_ARG),
    (dict(ldq=72), ck.CK_ERR_UNSUPPORTED),                     # q rows 16 bytes apart
    (dict(x=P + 1), ck.CK_ERR_UNSUPPORTED),                    # misaligned x
    (dict(out=P + 2, out_dtype=ck.CK_OUT_FP32), ck.CK_ERR_UNSUPPORTED),
    (dict(k=200, ldx=208, ldq=208, ldw=208, fused=1), ck.CK_ERR_UNSUPPORTED),   # k % 64
    (dict(m=65, x_mode=0, fused=1), ck.CK_ERR_UNSUPPORTED),    # tensor scale, two row tiles
    (dict(m=64, k=4096, ldx=4096, ldq=4096, ldw=4096, fused=1), ck.CK_ERR_UNSUPPORTED),  # LDS
    (dict(ldx=68, fused=1), ck.CK_ERR_UNSUPPORTED),            # x rows not 16-byte aligned
    (dict(k=200, ldx=208, ldq=208, ldw=208), ck.CK_ERR_HIP),    # falls back to two kernels
    (dict(fused=1), ck.CK_ERR_HIP),
    (dict(fused=0), ck.CK_ERR_HIP),
    (dict(), ck.CK_ERR_HIP),
    (dict(m=0), ck.CK_OK),
])
def test_layer_validation(kw, status):
    """Every argument of both steps is checked before anything is launched
    (no GPU here: a call that passes the checks reaches the device check)."""
    import torch
    if status == ck.CK_ERR_HIP and torch.cuda.is_available():
        pytest.skip("needs the no-GPU host")
    assert _layer(**kw) == status


def test_gemm_i32_validation():
    L = ck.lib()
    assert L.ck_int8_gemm_i32(P, 64, P, 64, P, 32, 16, 32, 64, ck.CK_NUM_TILES, 0) == ck.CK_ERR_INVALID_ARG
    assert L.ck_int8_gemm_i32(P, 64, 0, 64, P, 32, 16, 32, 64, -1, 0) == ck.CK_ERR_INVALID_ARG
    assert L.ck_int8_gemm_i32(P, 64, P, 64, P, 32, 0, 32, 64, -1, 0) == ck.CK_OK


def test_binding_raises_ckerror():
    with pytest.raises(ck.CKError) as e:
        ck.ck_int8_linear(0, 64, P, 1, P, 64, P, 1, 0, P, 32, 16, 32, 64)
    assert e.value.status == ck.CK_ERR_INVALID_ARG


def test_tile_heuristic_and_info():
    assert ck.ck_int8_tile_info(0)[:2] == (256, 256)
    for t in range(ck.CK_NUM_TILES):
        bm, bn, th = ck.ck_int8_tile_info(t)
        assert bm % 32 == 0 and bn % 32 == 0 and th % 64 == 0
    with pytest.raises(ck.CKError):
        ck.ck_int8_tile_info(ck.CK_NUM_TILES)
    # large-M shapes fill 256 CUs with the largest tile
    for m, n, k in ((80666, 28672, 5376), (99900, 21504, 5376), (25900, 16384, 4096)):
        t, bm, bn, g = ck.ck_int8_select_tile(m, n, k)
        assert (bm, bn) == (256, 256) and g >= 1
        assert -(-m // bm) * -(-n // bn) >= 256
    t, bm, bn, g = ck.ck_int8_select_tile(274, 2048, 2048)
    assert -(-274 // bm) * -(-2048 // bn) >= 64
    # more 256 x 256 tiles than compute units: the persistent tile; exactly
    # one per compute unit: its one-tile-per-block form
    ck.ck_int8_table_clear()
    assert ck.ck_int8_select_tile(80666, 28672, 5376)[0] == 13
    assert ck.ck_int8_select_tile(4096, 4096, 4096)[0] == 12


def test_valid_call_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _linear() in (ck.CK_ERR_HIP, ck.CK_ERR_WRONG_ARCH)
    assert ck.ck_last_error() != ""


# ---------------------------------------------------------------- tile table, forced tile, path log

def test_tile_table_drives_select_tile():
    ck.ck_int8_table_clear()
    try:
        shape = (1000, 3000, 512)
        h = ck.ck_int8_select_tile(*shape)
        ck.ck_int8_table_set(*shape, 7, 2)
        assert ck.ck_int8_table_size() == 1
        t, bm, bn, g = ck.ck_int8_select_tile(*shape)
        assert (t, g) == (7, 2) and (bm, bn) == ck.ck_int8_tile_info(7)[:2]
        assert ck.ck_int8_select_tile(1000, 3000, 528) == ck.ck_int8_select_tile(1000, 3000, 528)
        ck.ck_int8_table_set(*shape, -1, 0)                 # remove
        assert ck.ck_int8_table_size() == 0 and ck.ck_int8_select_tile(*shape) == h
        for bad in ((ck.CK_NUM_TILES, 1), (-2, 1), (3, 0)):
            with pytest.raises(ck.CKError):
                ck.ck_int8_table_set(*shape, *bad)
    finally:
        ck.ck_int8_table_clear()


def test_forced_tile_wins_over_table_and_heuristic():
    ck.ck_int8_table_clear()
    before = ck.ck_int8_forced_tile()
    try:
        ck.ck_int8_table_set(512, 512, 512, 1, 4)
        ck.ck_int8_set_forced_tile(5)
        assert ck.ck_int8_forced_tile() == 5
        assert ck.ck_int8_select_tile(512, 512, 512)[0] == 5
        assert ck.ck_int8_select_tile(80666, 28672, 5376)[0] == 5
        with pytest.raises(ck.CKError):
            ck.ck_int8_set_forced_tile(ck.CK_NUM_TILES)
    finally:
        ck.ck_int8_set_forced_tile(before)
        ck.ck_int8_table_clear()


def test_environment_sets_initial_forced_tile_and_log():
    import subprocess
    import sys
    code = ("import int8_weight_quantized_amd as ck; "
            "print(ck.ck_int8_forced_tile(), ck.ck_int8_select_tile(80666, 28672, 5376)[0])")
    env = dict(os.environ, CK_INT8_FORCE_TILE="9")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["9", "9"]
    env["CK_INT8_FORCE_TILE"] = "99"                        # out of range: ignored
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.stdout.split()[0] == "-1"


def test_table_file_is_gated_by_architecture(tmp_path):
    import json
    from int8_weight_quantized_amd import tile_table
    ck.ck_int8_table_clear()
    try:
        p = tmp_path / "t.json"
        p.write_text(json.dumps({"arch": "gfx950", "entries": [
            {"m": 7, "n": 9, "k": 32, "tile": 3, "group_m": 1}]}))
        assert tile_table.load(str(p), "gfx942") == 0 and ck.ck_int8_table_size() == 0
        assert tile_table.load(str(p), "gfx950") == 1
        assert ck.ck_int8_select_tile(7, 9, 32)[0] == 3
    finally:
        ck.ck_int8_table_clear()


def test_packaged_table_is_valid():
    import json
    from int8_weight_quantized_amd import tile_table
    path = tile_table.default_path("gfx950")
    if not os.path.exists(path):
        pytest.skip("no packaged table")
    t = json.load(open(path))
    assert t["arch"] == "gfx950" and t["entries"]
    for e in t["entries"]:
        assert 0 <= e["tile"] < ck.CK_NUM_TILES and e["group_m"] >= 1
        assert e["us"] <= e["heuristic_us"] * 1.0001


@pytest.fixture
def host_checks(monkeypatch):
    """Run the binding's argument checks on CPU tensors: the device type is
    switched to "cpu" and every library entry the helpers call is replaced
    by one that fails the test, so a check that lets a bad argument through
    shows up as a launch."""
    import torch

    class Launched(Exception):
        pass

    def launched(*a, **k):
        raise Launched()

    monkeypatch.setattr(ck, "_DEVICE_TYPE", "cpu")
    monkeypatch.setattr(ck, "_stream", lambda t: 0)
    for f in ("ck_int8_linear_ex", "ck_int8_linear_dequant", "ck_int8_gemm_i32",
              "ck_quantize_int8_rowwise", "ck_quantize_int8_rotated", "ck_int8_layer"):
        monkeypatch.setattr(ck, f, launched)
    m, n, k = 8, 16, 32
    t = dict(q=torch.zeros((m, k), dtype=torch.int8), w=torch.zeros((n, k), dtype=torch.int8),
             xs=torch.ones(m), ws=torch.ones(n), x=torch.zeros((m, k), dtype=torch.bfloat16),
             bias=torch.zeros(n, dtype=torch.bfloat16))
    return Launched, t


def test_binding_accepts_valid_arguments(host_checks):
    Launched, t = host_checks
    with pytest.raises(Launched):
        ck.int8_linear_q(t["q"], t["xs"], t["w"], t["ws"], t["bias"])
    with pytest.raises(Launched):
        ck.int8_linear_q(t["q"], t["xs"][:1], t["w"], t["ws"][:1])      # tensor-wide scales
    with pytest.raises(Launched):
        ck.int8_linear_dequant(t["x"], t["w"], t["ws"], t["bias"])
    with pytest.raises(Launched):
        ck.int8_gemm_i32(t["q"], t["w"])
    with pytest.raises(Launched):
        ck.int8_linear(t["x"], t["w"], t["ws"], t["bias"])
    with pytest.raises(Launched):
        ck.int8_linear(t["x"], t["w"], t["ws"][:1], mode="tensor", q=t["q"].clone(),
                       x_scale=t["xs"][:1].clone(), fused=1)
    with pytest.raises(Launched):
        ck.quantize_int8_rowwise(t["x"], q=t["q"].clone(), scale=t["xs"].clone())
    with pytest.raises(Launched):
        ck.quantize_int8_rotated(t["x"], 8, mode="tensor", scale=t["xs"][:1].clone())


def _bad_linear_args(torch, t):
    q, w, xs, ws, bias = t["q"], t["w"], t["xs"], t["ws"], t["bias"]
    return [
        (TypeError, dict(x_scale=xs.half())),                        # fp16 scale
        (TypeError, dict(w_scale=ws.to(torch.bfloat16))),            # bf16 scale
        (TypeError, dict(x_scale=xs.double())),
        (ValueError, dict(x_scale=torch.ones(2 * xs.numel())[::2])),  # strided scale
        (ValueError, dict(x_scale=torch.ones(3))),                   # neither 1 nor m
        (ValueError, dict(w_scale=torch.ones((ws.numel(), 1)))),      # not 1-D
        (ValueError, dict(w=torch.zeros((w.shape[0], w.shape[1] + 16), dtype=torch.int8))),
        (TypeError, dict(w=w.to(torch.int16))),
        (TypeError, dict(bias=bias.float())),                        # wrong bias type
        (ValueError, dict(bias=torch.zeros(3, dtype=torch.bfloat16))),
        (ValueError, dict(out=torch.empty((q.shape[0], w.shape[0] + 1), dtype=torch.bfloat16))),
        (TypeError, dict(out=torch.empty((q.shape[0], w.shape[0]), dtype=torch.float16))),
        (TypeError, dict(q=q.to(torch.uint8))),
    ]


def test_binding_rejects_bad_linear_arguments(host_checks):
    import torch
    Launched, t = host_checks
    for exc, kw in _bad_linear_args(torch, t):
        a = dict(q=t["q"], x_scale=t["xs"], w=t["w"], w_scale=t["ws"], bias=t["bias"], out=None)
        a.update(kw)
        with pytest.raises(exc):
            ck.int8_linear_q(a["q"], a["x_scale"], a["w"], a["w_scale"], a["bias"], out=a["out"])


def test_binding_rejects_bad_layer_arguments(host_checks):
    """int8_linear (one ck_int8_layer call) checks x, w, scales, bias, q,
    x_scale and out before the call."""
    import torch
    Launched, t = host_checks
    cases = [
        (TypeError, dict(x=t["x"].float())),
        (ValueError, dict(w=torch.zeros((16, 48), dtype=torch.int8))),          # k mismatch
        (TypeError, dict(w_scale=t["ws"].half())),
        (ValueError, dict(w_scale=torch.ones(5))),
        (TypeError, dict(bias=t["bias"].float())),
        (ValueError, dict(q=torch.zeros((8, 16), dtype=torch.int8))),
        (TypeError, dict(x_scale=t["xs"].double())),
        (ValueError, dict(x_scale=torch.ones(3))),                              # per-row needs m
        (ValueError, dict(out=torch.empty((8, 15), dtype=torch.bfloat16))),
        (TypeError, dict(out=torch.empty((8, 16), dtype=torch.float32))),       # bf16 out
        (TypeError, dict(w_scale=torch.ones(16, device="meta"))),
    ]
    for exc, kw in cases:
        a = dict(x=t["x"], w=t["w"], w_scale=t["ws"], bias=t["bias"], q=None, x_scale=None, out=None)
        a.update(kw)
        with pytest.raises(exc):
            ck.int8_linear(a["x"], a["w"], a["w_scale"], a["bias"], q=a["q"], x_scale=a["x_scale"],
                           out=a["out"])
    with pytest.raises(ValueError):
        ck.int8_linear(t["x"], t["w"], t["ws"], mode="rows")


def test_binding_rejects_operands_on_other_devices(host_checks):
    """A scale, weight, bias or output on another device than q is rejected
    (a host address handed to a kernel would fault the GPU).  Here the
    "other device" is the meta device, which the checks treat as foreign."""
    import torch
    Launched, t = host_checks
    meta = dict(x_scale=torch.ones(8, device="meta"), w_scale=torch.ones(16, device="meta"),
                bias=torch.zeros(16, dtype=torch.bfloat16, device="meta"),
                w=torch.zeros((16, 32), dtype=torch.int8, device="meta"))
    for name, v in meta.items():
        a = dict(q=t["q"], x_scale=t["xs"], w=t["w"], w_scale=t["ws"], bias=t["bias"])
        a[name] = v
        with pytest.raises(TypeError):
            ck.int8_linear_q(a["q"], a["x_scale"], a["w"], a["w_scale"], a["bias"])


def test_binding_rejects_bad_gemm_dequant_and_quantize_arguments(host_checks):
    import torch
    Launched, t = host_checks
    w_wide = torch.zeros((16, 48), dtype=torch.int8)
    with pytest.raises(ValueError):
        ck.int8_gemm_i32(t["q"], w_wide)                          # k mismatch
    with pytest.raises(TypeError):
        ck.int8_gemm_i32(t["q"], t["w"], out=torch.empty((8, 16), dtype=torch.float32))
    with pytest.raises(ValueError):
        ck.int8_gemm_i32(t["q"], t["w"], out=torch.empty((8, 15), dtype=torch.int32))
    with pytest.raises(ValueError):
        ck.int8_linear_dequant(t["x"], w_wide, t["ws"])
    with pytest.raises(TypeError):
        ck.int8_linear_dequant(t["x"], t["w"], t["ws"].half())
    with pytest.raises(ValueError):
        ck.int8_linear_dequant(t["x"], t["w"], torch.ones(5))
    with pytest.raises(TypeError):
        ck.quantize_int8_rowwise(t["x"], scale=t["xs"].half())
    with pytest.raises(ValueError):
        ck.quantize_int8_rowwise(t["x"], scale=torch.ones(3))      # per-row needs m
    with pytest.raises(ValueError):
        ck.quantize_int8_rowwise(t["x"], mode="tensor", scale=t["xs"].clone())   # needs 1
    with pytest.raises(ValueError):
        ck.quantize_int8_rowwise(t["x"], q=torch.zeros((8, 16), dtype=torch.int8))
    with pytest.raises(TypeError):
        ck.quantize_int8_rowwise(t["x"], q=torch.zeros((8, 32), dtype=torch.uint8))
    with pytest.raises(ValueError):
        ck.quantize_int8_rowwise(t["x"], mode="rows")
    with pytest.raises(TypeError):
        ck.quantize_int8_rotated(t["x"], 8, scale=t["xs"].double())


@pytest.mark.parametrize("args,status", [
    # src, chunks, dst, blocks, unroll
    ((P, 0, P, 8, 4), ck.CK_OK),
    ((P, -1, P, 8, 4), ck.CK_ERR_INVALID_ARG),
    ((0, 64, P, 8, 4), ck.CK_ERR_INVALID_ARG),
    ((P, 64, P, 0, 4), ck.CK_ERR_INVALID_ARG),
    ((P, 64, P, 8, 3), ck.CK_ERR_INVALID_ARG),
    ((P + 8, 64, P, 8, 4), ck.CK_ERR_UNSUPPORTED),
    ((P, 64, P + 4, 8, 4), ck.CK_ERR_UNSUPPORTED),
    ((P, 64, P, 8, 4), ck.CK_ERR_HIP),
])
def test_hbm_stream_validation(args, status):
    import torch
    if status == ck.CK_ERR_HIP and torch.cuda.is_available():
        pytest.skip("needs the no-GPU host")
    assert ck.lib().ck_hbm_stream(*args, 0) == status


@pytest.mark.parametrize("args,status", [
    ((-1, 0, P, 0), ck.CK_ERR_INVALID_ARG),
    ((10, 2, P, 0), ck.CK_ERR_INVALID_ARG),
    ((10, -1, P, 0), ck.CK_ERR_INVALID_ARG),
    ((10, 1, 0, 0), ck.CK_ERR_INVALID_ARG),
    ((10, 0, P + 2, 0), ck.CK_ERR_UNSUPPORTED),
    ((10, 0, P, 0), ck.CK_ERR_HIP),
    ((10, 1, P, 0), ck.CK_ERR_HIP),
])
def test_mfma_ceiling_validation(args, status):
    import torch
    if status == ck.CK_ERR_HIP and torch.cuda.is_available():
        pytest.skip("needs the no-GPU host")
    assert ck.lib().ck_mfma_ceiling(*args, 0) == status
