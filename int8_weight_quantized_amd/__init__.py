"""MI355X (gfx950) INT8 linear layer: Python binding of libck_int8.so.

The functions named ``ck_*`` mirror the C ABI in include/ck_int8.h one to
one: they take device addresses (ints) and sizes, call the library through
ctypes, and raise CKError on any status other than CK_OK.  The tensor-level
helpers (``quantize_int8_rowwise``, ``int8_linear``, ...) only allocate the
outputs with torch and pass pointers and the current stream; every step of
the layer runs in the library's HIP kernels.  There is no other code path:
if the library is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libck_int8.so")

CK_OK = 0
CK_ERR_INVALID_ARG = 1
CK_ERR_UNSUPPORTED = 2
CK_ERR_HIP = 3
CK_ERR_WRONG_ARCH = 4

CK_SCALE_TENSOR = 0
CK_SCALE_ROW = 1

CK_OUT_BF16 = 0
CK_OUT_FP16 = 1
CK_OUT_FP32 = 2

CK_MAX_K = 132104
CK_NUM_TILES = 14
CK_ABI_VERSION = 11

EXPORTED = (
    "ck_quantize_int8_rowwise", "ck_quantize_int8_rotated", "ck_int8_linear",
    "ck_int8_linear_tiled", "ck_int8_linear_ex", "ck_int8_linear_noalloc", "ck_int8_layer", "ck_int8_linear_dequant", "ck_int8_gemm_i32", "ck_int8_select_tile", "ck_int8_tile_info",
    "ck_hbm_stream", "ck_mfma_ceiling", "ck_status_string", "ck_last_error", "ck_abi_version",
    "ck_int8_table_set", "ck_int8_table_clear", "ck_int8_table_size",
    "ck_int8_set_forced_tile", "ck_int8_forced_tile", "ck_int8_set_path_log",
)


class CKError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {_status_name(status)}: {detail}")


_lib = None


def _status_name(s: int) -> str:
    names = {0: "CK_OK", 1: "CK_ERR_INVALID_ARG", 2: "CK_ERR_UNSUPPORTED",
             3: "CK_ERR_HIP", 4: "CK_ERR_WRONG_ARCH"}
    return names.get(s, f"status {s}")


def lib():
    """The loaded libck_int8.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m int8_weight_quantized_amd.build` "
            "(or __graft_entry__.build()) first. There is no fallback path.")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    pi = ctypes.POINTER(ctypes.c_int)
    L.ck_quantize_int8_rowwise.argtypes = [p, i64, i64, i64, p, i64, p, ci, p]
    L.ck_quantize_int8_rotated.argtypes = [p, i64, i64, i64, i64, p, i64, p, ci, p]
    L.ck_int8_linear.argtypes = [p, i64, p, ci, p, i64, p, ci, p, p, i64, i64, i64, i64, p]
    L.ck_int8_linear_tiled.argtypes = [p, i64, p, ci, p, i64, p, ci, p, p, i64, i64, i64, i64,
                                       ci, ci, p]
    L.ck_int8_linear_ex.argtypes = [p, i64, p, ci, p, i64, p, ci, p, p, i64, ci, i64, i64, i64,
                                    ci, ci, p]
    L.ck_int8_linear_noalloc.argtypes = [p, i64, p, ci, p, i64, p, ci, p, p, i64, ci, i64, i64,
                                         i64, ci, ci, p]
    L.ck_int8_layer.argtypes = [p, i64, p, i64, p, ci, p, i64, p, ci, p, p, i64, ci, i64, i64, i64,
                                ci, p]
    L.ck_int8_linear_dequant.argtypes = [p, i64, p, i64, p, ci, p, p, i64, ci, i64, i64, i64, p]
    L.ck_int8_gemm_i32.argtypes = [p, i64, p, i64, p, i64, i64, i64, i64, ci, p]
    L.ck_hbm_stream.argtypes = [p, i64, p, ci, ci, p]
    L.ck_hbm_stream.restype = ci
    L.ck_mfma_ceiling.argtypes = [i64, ci, p, ctypes.c_uint32, p]
    L.ck_mfma_ceiling.restype = ci
    L.ck_int8_select_tile.argtypes = [i64, i64, i64, pi, pi, pi, pi]
    L.ck_int8_tile_info.argtypes = [ci, pi, pi, pi]
    for f in ("ck_quantize_int8_rowwise", "ck_quantize_int8_rotated", "ck_int8_linear", "ck_int8_linear_tiled",
              "ck_int8_linear_ex", "ck_int8_linear_noalloc", "ck_int8_layer", "ck_int8_linear_dequant", "ck_int8_gemm_i32", "ck_int8_select_tile", "ck_int8_tile_info"):
        getattr(L, f).restype = ci
    L.ck_int8_table_set.argtypes = [i64, i64, i64, ci, ci]
    L.ck_int8_table_set.restype = ci
    L.ck_int8_table_clear.argtypes = []
    L.ck_int8_table_clear.restype = ci
    L.ck_int8_table_size.argtypes = []
    L.ck_int8_table_size.restype = i64
    L.ck_int8_set_forced_tile.argtypes = [ci]
    L.ck_int8_set_forced_tile.restype = ci
    L.ck_int8_forced_tile.argtypes = []
    L.ck_int8_forced_tile.restype = ci
    L.ck_int8_set_path_log.argtypes = [ci]
    L.ck_int8_set_path_log.restype = ci
    L.ck_status_string.argtypes = [ci]
    L.ck_status_string.restype = ctypes.c_char_p
    L.ck_last_error.argtypes = []
    L.ck_last_error.restype = ctypes.c_char_p
    L.ck_abi_version.argtypes = []
    L.ck_abi_version.restype = ci
    if L.ck_abi_version() != CK_ABI_VERSION:
        raise ImportError("libck_int8.so ABI version does not match the binding")
    _lib = L
    return L


def _check(status: int, func: str):
    if status != CK_OK:
        raise CKError(status, func, lib().ck_last_error().decode())


# ---------------------------------------------------------------- C ABI mirror

def ck_quantize_int8_rowwise(x, m, k, ldx, q, ldq, scale, mode, stream=0):
    _check(lib().ck_quantize_int8_rowwise(x, m, k, ldx, q, ldq, scale, mode, stream),
           "ck_quantize_int8_rowwise")


def ck_quantize_int8_rotated(x, m, k, ldx, block, q, ldq, scale, mode, stream=0):
    _check(lib().ck_quantize_int8_rotated(x, m, k, ldx, block, q, ldq, scale, mode, stream),
           "ck_quantize_int8_rotated")


def ck_int8_linear(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                   m, n, k, stream=0):
    _check(lib().ck_int8_linear(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias,
                                out, ldo, m, n, k, stream), "ck_int8_linear")


def ck_int8_linear_tiled(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                         m, n, k, tile, group_m, stream=0):
    _check(lib().ck_int8_linear_tiled(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias,
                                      out, ldo, m, n, k, tile, group_m, stream),
           "ck_int8_linear_tiled")


def ck_int8_linear_ex(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                      out_dtype, m, n, k, tile=-1, group_m=0, stream=0):
    _check(lib().ck_int8_linear_ex(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias,
                                   out, ldo, out_dtype, m, n, k, tile, group_m, stream),
           "ck_int8_linear_ex")


def ck_int8_linear_noalloc(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                           out_dtype, m, n, k, tile=-1, group_m=0, stream=0):
    _check(lib().ck_int8_linear_noalloc(q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias,
                                        out, ldo, out_dtype, m, n, k, tile, group_m, stream),
           "ck_int8_linear_noalloc")


def ck_int8_layer(x, ldx, q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias, out, ldo,
                  out_dtype, m, n, k, fused=-1, stream=0):
    _check(lib().ck_int8_layer(x, ldx, q, ldq, x_scale, x_mode, w, ldw, w_scale, w_mode, bias,
                               out, ldo, out_dtype, m, n, k, fused, stream), "ck_int8_layer")


def ck_int8_linear_dequant(x, ldx, w, ldw, w_scale, w_mode, bias, out, ldo, out_dtype,
                           m, n, k, stream=0):
    _check(lib().ck_int8_linear_dequant(x, ldx, w, ldw, w_scale, w_mode, bias, out, ldo,
                                        out_dtype, m, n, k, stream), "ck_int8_linear_dequant")


def ck_int8_gemm_i32(q, ldq, w, ldw, acc, ldacc, m, n, k, tile=-1, stream=0):
    _check(lib().ck_int8_gemm_i32(q, ldq, w, ldw, acc, ldacc, m, n, k, tile, stream),
           "ck_int8_gemm_i32")


def ck_hbm_stream(src, chunks, dst, blocks, unroll, stream=0):
    _check(lib().ck_hbm_stream(src, chunks, dst, blocks, unroll, stream), "ck_hbm_stream")


def ck_mfma_ceiling(iters, mode, out, seed=0, stream=0):
    _check(lib().ck_mfma_ceiling(iters, mode, out, seed, stream), "ck_mfma_ceiling")


def ck_int8_select_tile(m, n, k):
    """-> (tile, bm, bn, group_m) the heuristic picks for the shape."""
    t, bm, bn, g = (ctypes.c_int() for _ in range(4))
    _check(lib().ck_int8_select_tile(m, n, k, ctypes.byref(t), ctypes.byref(bm),
                                     ctypes.byref(bn), ctypes.byref(g)), "ck_int8_select_tile")
    return t.value, bm.value, bn.value, g.value


def ck_int8_tile_info(tile):
    """-> (bm, bn, threads) of compiled tile configuration `tile`."""
    bm, bn, th = (ctypes.c_int() for _ in range(3))
    _check(lib().ck_int8_tile_info(tile, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(th)),
           "ck_int8_tile_info")
    return bm.value, bn.value, th.value


def ck_int8_table_set(m, n, k, tile, group_m):
    _check(lib().ck_int8_table_set(m, n, k, tile, group_m), "ck_int8_table_set")


def ck_int8_table_clear():
    _check(lib().ck_int8_table_clear(), "ck_int8_table_clear")


def ck_int8_table_size() -> int:
    return int(lib().ck_int8_table_size())


def ck_int8_set_forced_tile(tile: int):
    _check(lib().ck_int8_set_forced_tile(tile), "ck_int8_set_forced_tile")


def ck_int8_forced_tile() -> int:
    return int(lib().ck_int8_forced_tile())


def ck_int8_set_path_log(on: bool):
    _check(lib().ck_int8_set_path_log(1 if on else 0), "ck_int8_set_path_log")


def ck_status_string(s: int) -> str:
    return lib().ck_status_string(s).decode()


def ck_last_error() -> str:
    return lib().ck_last_error().decode()


# ---------------------------------------------------------------- torch helpers

def _stream(t):
    import torch
    from . import tile_table
    tile_table.ensure_loaded(t.device)
    return torch.cuda.current_stream(t.device).cuda_stream


def _mode(mode: str) -> int:
    if mode == "row":
        return CK_SCALE_ROW
    if mode == "tensor":
        return CK_SCALE_TENSOR
    raise ValueError(f"mode must be 'row' or 'tensor', not {mode!r}")


# Device type every tensor handed to the library must live on.  (The CPU
# tests of this module's argument checks set it to "cpu".)
_DEVICE_TYPE = "cuda"


def _need(t, dtype, name, device=None):
    """t is a `dtype` tensor on the GPU (on `device`, when given) with unit
    stride in its last dimension.  Raises TypeError / ValueError before any
    pointer reaches the library: a host tensor's address would make the
    kernels read host memory, and a wrong dtype or stride silently wrong
    values."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device.type != _DEVICE_TYPE:
        raise TypeError(f"{name} must be a {dtype} {_DEVICE_TYPE} tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if t.dim() >= 1 and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")


def _need_matrix(t, dtype, name, shape, device=None):
    """A 2-D `dtype` tensor of the given shape (rows may be strided)."""
    _need(t, dtype, name, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need_vector(t, dtype, name, sizes, device=None):
    """A contiguous 1-D `dtype` tensor whose length is one of `sizes`."""
    _need(t, dtype, name, device)
    if t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-D tensor")
    if t.numel() not in sizes:
        raise ValueError(f"{name} has {t.numel()} values, expected one of {sorted(set(sizes))}")


def _pad16(k: int) -> int:
    return (k + 15) // 16 * 16


def pad_rows(w):
    """An int8 [n, k] tensor as a view whose rows start 16 bytes apart:
    returns w itself when k is a multiple of 16 and w is contiguous, else a
    copy into zero-filled [n, k rounded up to 16] storage, viewed as [n, k].
    The GEMM reads operand rows in 16-byte chunks, so weights whose k is not
    a multiple of 16 are stored this way once, when they are loaded."""
    import torch
    _need(w, torch.int8, "w")
    n, k = w.shape
    if w.is_contiguous() and k % 16 == 0 and w.data_ptr() % 16 == 0:
        return w
    buf = torch.zeros((n, _pad16(k)), dtype=torch.int8, device=w.device)
    buf[:, :k].copy_(w)
    return buf[:, :k]


def quantize_int8_rowwise(x, mode: str = "row", q=None, scale=None):
    """x bf16 [m, k] -> (q int8 [m, k], scale fp32 [m] or [1]).

    A q allocated here has rows 16 bytes apart (its storage is padded when
    k is not a multiple of 16), as the GEMM needs."""
    import torch
    code = _mode(mode)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, k]")
    m, k = x.shape
    ns = m if mode == "row" else 1
    if q is None:
        q = torch.empty((m, _pad16(k)), dtype=torch.int8, device=x.device)[:, :k]
    else:
        _need_matrix(q, torch.int8, "q", (m, k), x.device)
    if scale is None:
        scale = torch.empty((ns,), dtype=torch.float32, device=x.device)
    else:
        _need_vector(scale, torch.float32, "scale", (ns,), x.device)
    ck_quantize_int8_rowwise(x.data_ptr(), m, k, x.stride(0), q.data_ptr(), q.stride(0),
                             scale.data_ptr(), code, _stream(x))
    return q, scale


def quantize_int8_rotated(x, block: int, mode: str = "row", q=None, scale=None):
    """ConvRot activations: x bf16 [m, k] -> codes and scales of x H, with H
    the block-diagonal normalised Hadamard matrix of order `block`.

    The same call prepares the weight: W_rot = W H^T = W H (H is symmetric)
    rotates each row of W [n, k] exactly as an activation row, so
    quantize_int8_rotated(W, block) gives W_rot's int8 codes and per-row
    scales, and the layer on the rotated codes computes x W^T."""
    import torch
    code = _mode(mode)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, k]")
    m, k = x.shape
    ns = m if mode == "row" else 1
    if q is None:
        q = torch.empty((m, _pad16(k)), dtype=torch.int8, device=x.device)[:, :k]
    else:
        _need_matrix(q, torch.int8, "q", (m, k), x.device)
    if scale is None:
        scale = torch.empty((ns,), dtype=torch.float32, device=x.device)
    else:
        _need_vector(scale, torch.float32, "scale", (ns,), x.device)
    ck_quantize_int8_rotated(x.data_ptr(), m, k, x.stride(0), block, q.data_ptr(), q.stride(0),
                             scale.data_ptr(), code, _stream(x))
    return q, scale


_OUT = {"bf16": CK_OUT_BF16, "fp16": CK_OUT_FP16, "fp32": CK_OUT_FP32}


def _out_dtype(name):
    import torch
    torch_dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    if name not in _OUT:
        raise ValueError(f"out_dtype must be 'bf16', 'fp16' or 'fp32', not {name!r}")
    return _OUT[name], torch_dt[name]


def int8_linear_q(q, x_scale, w, w_scale, bias=None, out=None, tile: int = -1,
                  group_m: int = 0, out_dtype: str = "bf16"):
    """Steps 2 + 3 on already-quantised activations -> [m, n] of out_dtype
    ("bf16", "fp16" or "fp32"; a given bias has that type too).

    x_scale has m values (per row) or 1 (tensor); w_scale n values or 1."""
    import torch
    code, tdt = _out_dtype(out_dtype)
    _need(q, torch.int8, "q")
    if q.dim() != 2 or w.dim() != 2:
        raise ValueError("q and w must be 2-D")
    dev = q.device
    _need(w, torch.int8, "w", dev)
    m, k = q.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("q and w disagree on k")
    _need_vector(x_scale, torch.float32, "x_scale", (1, m), dev)
    _need_vector(w_scale, torch.float32, "w_scale", (1, n), dev)
    x_mode = CK_SCALE_ROW if x_scale.numel() == m and m != 1 else CK_SCALE_TENSOR
    w_mode = CK_SCALE_ROW if w_scale.numel() == n and n != 1 else CK_SCALE_TENSOR
    if bias is not None:
        _need_vector(bias, tdt, "bias", (n,), dev)
    if out is None:
        out = torch.empty((m, n), dtype=tdt, device=dev)
    else:
        _need_matrix(out, tdt, "out", (m, n), dev)
    b = 0 if bias is None else bias.data_ptr()
    ck_int8_linear_ex(q.data_ptr(), q.stride(0), x_scale.data_ptr(), x_mode,
                      w.data_ptr(), w.stride(0), w_scale.data_ptr(), w_mode, b,
                      out.data_ptr(), out.stride(0), code, m, n, k, tile, group_m, _stream(q))
    return out


def int8_linear(x, w, w_scale, bias=None, mode: str = "row", out=None,
                out_dtype: str = "bf16", fused: int = -1, q=None, x_scale=None):
    """The whole layer: bf16 x [m, k], int8 w [n, k], fp32 w_scale -> [m, n]
    of out_dtype.  w rows must start 16 bytes apart (see pad_rows).

    One call of ck_int8_layer: quantisation then the GEMM, as one kernel for
    few rows (fused=-1 lets the library choose, 0 forces two kernels, 1 one
    kernel).  The codes and scales land in q and x_scale when given."""
    import torch
    code, tdt = _out_dtype(out_dtype)
    xm = _mode(mode)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x and w must be 2-D")
    dev = x.device
    _need(w, torch.int8, "w", dev)
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("x and w disagree on k")
    _need_vector(w_scale, torch.float32, "w_scale", (1, n), dev)
    w_mode = CK_SCALE_ROW if w_scale.numel() == n and n != 1 else CK_SCALE_TENSOR
    ns = m if mode == "row" else 1
    if q is None:
        q = torch.empty((m, _pad16(k)), dtype=torch.int8, device=dev)[:, :k]
    else:
        _need_matrix(q, torch.int8, "q", (m, k), dev)
    if x_scale is None:
        x_scale = torch.empty((ns,), dtype=torch.float32, device=dev)
    else:
        _need_vector(x_scale, torch.float32, "x_scale", (ns,), dev)
    if bias is not None:
        _need_vector(bias, tdt, "bias", (n,), dev)
    if out is None:
        out = torch.empty((m, n), dtype=tdt, device=dev)
    else:
        _need_matrix(out, tdt, "out", (m, n), dev)
    b = 0 if bias is None else bias.data_ptr()
    ck_int8_layer(x.data_ptr(), x.stride(0), q.data_ptr(), q.stride(0), x_scale.data_ptr(), xm,
                  w.data_ptr(), w.stride(0), w_scale.data_ptr(), w_mode, b, out.data_ptr(),
                  out.stride(0), code, m, n, k, fused, _stream(x))
    return out


def int8_linear_dequant(x, w, w_scale, bias=None, out=None, out_dtype: str = "bf16"):
    """Dequant-on-the-fly layer: bf16 x [m, k] times the int8 weight [n, k]
    dequantised to bf16 (w * w_scale) inside the kernel, on bf16 matrix
    cores; x is not quantised.  -> [m, n] of out_dtype."""
    import torch
    code, tdt = _out_dtype(out_dtype)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x and w must be 2-D")
    dev = x.device
    _need(w, torch.int8, "w", dev)
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("x and w disagree on k")
    _need_vector(w_scale, torch.float32, "w_scale", (1, n), dev)
    w_mode = CK_SCALE_ROW if w_scale.numel() == n and n != 1 else CK_SCALE_TENSOR
    if bias is not None:
        _need_vector(bias, tdt, "bias", (n,), dev)
    if out is None:
        out = torch.empty((m, n), dtype=tdt, device=dev)
    else:
        _need_matrix(out, tdt, "out", (m, n), dev)
    b = 0 if bias is None else bias.data_ptr()
    ck_int8_linear_dequant(x.data_ptr(), x.stride(0), w.data_ptr(), w.stride(0), w_scale.data_ptr(),
                           w_mode, b, out.data_ptr(), out.stride(0), code, m, n, k, _stream(x))
    return out


def int8_gemm_i32(q, w, tile: int = -1, out=None):
    """int32 accumulators acc[m, n] = q . w^T (checking aid)."""
    import torch
    _need(q, torch.int8, "q")
    if q.dim() != 2 or w.dim() != 2:
        raise ValueError("q and w must be 2-D")
    dev = q.device
    _need(w, torch.int8, "w", dev)
    m, k = q.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("q and w disagree on k")
    if out is None:
        out = torch.empty((m, n), dtype=torch.int32, device=dev)
    else:
        _need_matrix(out, torch.int32, "out", (m, n), dev)
    ck_int8_gemm_i32(q.data_ptr(), q.stride(0), w.data_ptr(), w.stride(0), out.data_ptr(),
                     out.stride(0), m, n, k, tile, _stream(q))
    return out
