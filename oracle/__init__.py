"""CPU oracle for the INT8 linear layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product package
``int8_weight_quantized_amd`` never imports it, and it imports nothing from
there: the two share no code.

The arithmetic lives in ``ck_oracle.c`` (plain C, built with gcc); this module
only marshals numpy arrays into it.  bf16 tensors travel as ``uint16`` bit
patterns.  See the header of ``ck_oracle.c`` for what each step computes and
which passage of the comfy-kitchen pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ck_oracle.c")
_LIB_AVX2 = os.path.join(_HERE, "libck_oracle.so")
_LIB_GENERIC = os.path.join(_HERE, "libck_oracle_generic.so")

# -ffp-contract=off: every epilogue operation is one fp32 rounding (no FMA).
# Two builds of the same source: one that lets gcc auto-vectorise the integer
# dot products with AVX2, and a baseline x86-64 one for hosts without AVX2.
_COMMON = ["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", _SRC, "-lm"]
BUILD_CMDS = [
    _COMMON[:1] + ["-O3", "-march=x86-64-v3"] + _COMMON[1:] + ["-o", _LIB_AVX2],
    _COMMON[:1] + ["-O2"] + _COMMON[1:] + ["-o", _LIB_GENERIC],
]

_lib = None


def build() -> str:
    """Compile the oracle library with gcc; returns the path this host loads."""
    for cmd in BUILD_CMDS:
        subprocess.run(cmd, check=True)
    return _lib_path()


def _host_has_avx2() -> bool:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("flags"):
                    f = line.split()
                    return "avx2" in f and "fma" in f and "bmi2" in f
    except OSError:
        pass
    return False


def _lib_path() -> str:
    return _LIB_AVX2 if _host_has_avx2() else _LIB_GENERIC


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _lib_path()
    if not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.ck_oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.ck_oracle_bf16_to_f32.restype = ctypes.c_float
    lib.ck_oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.ck_oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.ck_oracle_f32_to_bf16_array.argtypes = [p, p, i64]
    lib.ck_oracle_f32_to_bf16_array.restype = None
    for name in ("ck_oracle_quantize_rowwise", "ck_oracle_quantize_tensorwise"):
        f = getattr(lib, name)
        f.argtypes = [p, i64, i64, i64, p, i64, p]
        f.restype = None
    lib.ck_oracle_gemm_i32.argtypes = [p, i64, p, i64, p, i64, i64, i64, i64]
    lib.ck_oracle_gemm_i32.restype = ci
    lib.ck_oracle_epilogue.argtypes = [p, i64, p, ci, p, ci, p, p, i64, i64, i64]
    lib.ck_oracle_epilogue.restype = None
    lib.ck_oracle_linear.argtypes = [p, i64, p, ci, p, i64, p, ci, p, p, i64,
                                     i64, i64, i64]
    lib.ck_oracle_linear.restype = ci
    lib.ck_oracle_f32_to_f16_array.argtypes = [p, p, i64]
    lib.ck_oracle_f32_to_f16_array.restype = None
    lib.ck_oracle_f16_to_f32_array.argtypes = [p, p, i64]
    lib.ck_oracle_f16_to_f32_array.restype = None
    lib.ck_oracle_epilogue_ex.argtypes = [p, i64, p, ci, p, ci, p, p, i64, i64, i64, ci]
    lib.ck_oracle_epilogue_ex.restype = None
    lib.ck_oracle_linear_ex.argtypes = [p, i64, p, ci, p, i64, p, ci, p, p, i64,
                                        i64, i64, i64, ci]
    lib.ck_oracle_linear_ex.restype = ci
    lib.ck_oracle_rot_scale.argtypes = [i64]
    lib.ck_oracle_rot_scale.restype = ctypes.c_float
    lib.ck_oracle_rotate.argtypes = [p, i64, i64, i64, i64, p]
    lib.ck_oracle_rotate.restype = None
    for name in ("ck_oracle_quantize_rowwise_f32", "ck_oracle_quantize_tensorwise_f32"):
        f = getattr(lib, name)
        f.argtypes = [p, i64, i64, i64, p, i64, p]
        f.restype = None
    lib.ck_oracle_dequant_weight.argtypes = [p, i64, i64, i64, p, ci, p]
    lib.ck_oracle_dequant_weight.restype = None
    lib.ck_oracle_linear_dequant.argtypes = [p, i64, p, p, p, i64, i64, i64, i64, ci, p, p]
    lib.ck_oracle_linear_dequant.restype = None
    lib.ck_oracle_num_threads.argtypes = []
    lib.ck_oracle_num_threads.restype = ci
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use."""
    return int(_load().ck_oracle_num_threads())


def bf16_to_f32(b):
    """Widen bf16 bit patterns (uint16) to float32, exactly."""
    b = _c(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f):
    """Round float32 values to bf16 bit patterns (nearest, ties to even)."""
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().ck_oracle_f32_to_bf16_array(_ptr(f), _ptr(out), f.size)
    return out


def f32_to_f16(f):
    """Round float32 values to fp16 bit patterns (nearest, ties to even)."""
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().ck_oracle_f32_to_f16_array(_ptr(f), _ptr(out), f.size)
    return out


def f16_to_f32(h):
    """Widen fp16 bit patterns (uint16) to float32, exactly."""
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().ck_oracle_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


# Output types of the epilogue: bf16 and fp16 travel as uint16 bit patterns,
# fp32 as float32.  The bias, when given, has the output's type.
_OUT = {"bf16": (0, np.uint16), "fp16": (1, np.uint16), "fp32": (2, np.float32)}


def quantize_rowwise(x_bf16):
    """x: uint16 [m, k] bf16 bits -> (q int8 [m, k], scale float32 [m])."""
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    s = np.empty((m,), np.float32)
    _load().ck_oracle_quantize_rowwise(_ptr(x), m, k, k, _ptr(q), k, _ptr(s))
    return q, s


def quantize_tensorwise(x_bf16):
    """x: uint16 [m, k] bf16 bits -> (q int8 [m, k], scale float32 [1])."""
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    s = np.empty((1,), np.float32)
    _load().ck_oracle_quantize_tensorwise(_ptr(x), m, k, k, _ptr(q), k, _ptr(s))
    return q, s


def rot_scale(b: int) -> float:
    """fl(1/sqrt(b)), the scale applied after the butterflies."""
    return float(_load().ck_oracle_rot_scale(b))


def rotate(x_bf16, block: int):
    """x_rot = x H for the block-diagonal normalised Hadamard H of order
    `block` (fp32 result [m, k]; k a multiple of block)."""
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    assert block >= 1 and block & (block - 1) == 0 and k % block == 0
    out = np.empty((m, k), np.float32)
    _load().ck_oracle_rotate(_ptr(x), m, k, k, block, _ptr(out))
    return out


def quantize_f32(x_f32, mode="row"):
    """Quantise fp32 rows (per row or tensor-wide) -> (q int8, scale)."""
    x = _c(x_f32, np.float32)
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    s = np.empty((m if mode == "row" else 1,), np.float32)
    fn = (_load().ck_oracle_quantize_rowwise_f32 if mode == "row"
          else _load().ck_oracle_quantize_tensorwise_f32)
    fn(_ptr(x), m, k, k, _ptr(q), k, _ptr(s))
    return q, s


def quantize_rotated(x_bf16, block: int, mode="row"):
    """Step 0 + step 1: quantise x H -> (q int8 [m, k], scale)."""
    return quantize_f32(rotate(x_bf16, block), mode)


def gemm_i32(q, w):
    """Exact int32 accumulators acc[m, n] = q[m, k] . w[n, k]^T.

    Raises OverflowError if any accumulator does not fit in int32."""
    q = _c(q, np.int8)
    w = _c(w, np.int8)
    m, k = q.shape
    n, k2 = w.shape
    assert k == k2
    acc = np.empty((m, n), np.int32)
    rc = _load().ck_oracle_gemm_i32(_ptr(q), k, _ptr(w), k, _ptr(acc), n, m, n, k)
    if rc != 0:
        raise OverflowError("int32 accumulator overflow")
    return acc


def epilogue(acc, xs, ws, bias=None, out_dtype="bf16"):
    """out[m, n] = round_out(((fp32(acc) * xs) * ws) + bias).

    out_dtype "bf16" / "fp16" give uint16 bit patterns, "fp32" float32."""
    code, odt = _OUT[out_dtype]
    acc = _c(acc, np.int32)
    m, n = acc.shape
    xs = _c(np.atleast_1d(xs), np.float32)
    ws = _c(np.atleast_1d(ws), np.float32)
    b = None if bias is None else _c(bias, odt)
    out = np.empty((m, n), odt)
    assert xs.size in (1, m) and ws.size in (1, n)
    _load().ck_oracle_epilogue_ex(_ptr(acc), n, _ptr(xs), int(xs.size == m),
                                  _ptr(ws), int(ws.size == n), _ptr(b),
                                  _ptr(out), n, m, n, code)
    return out


def linear(q, xs, w, ws, bias=None, out_dtype="bf16"):
    """Steps 2+3 element by element: out[m, n] of the output type.

    xs is [m] (per row) or [1] (tensor); ws is [n] (per column) or [1]."""
    code, odt = _OUT[out_dtype]
    q = _c(q, np.int8)
    w = _c(w, np.int8)
    m, k = q.shape
    n, k2 = w.shape
    assert k == k2
    xs = _c(np.atleast_1d(xs), np.float32)
    ws = _c(np.atleast_1d(ws), np.float32)
    assert xs.size in (1, m) and ws.size in (1, n)
    b = None if bias is None else _c(bias, odt)
    out = np.empty((m, n), odt)
    rc = _load().ck_oracle_linear_ex(_ptr(q), k, _ptr(xs), int(xs.size == m),
                                     _ptr(w), k, _ptr(ws), int(ws.size == n),
                                     _ptr(b), _ptr(out), n, m, n, k, code)
    if rc != 0:
        raise OverflowError("int32 accumulator overflow")
    return out


def dequant_weight(w, ws):
    """bf16 bits wdq[n, k] = bf16(fp32(w) * ws[j]) (ws [n] or [1])."""
    w = _c(w, np.int8)
    n, k = w.shape
    ws = _c(np.atleast_1d(ws), np.float32)
    assert ws.size in (1, n)
    out = np.empty((n, k), np.uint16)
    _load().ck_oracle_dequant_weight(_ptr(w), n, k, k, _ptr(ws), int(ws.size == n), _ptr(out))
    return out


def linear_dequant(x_bf16, w, ws, bias=None, out_dtype="bf16"):
    """The dequant-on-the-fly layer: (out, S, A) where out = round_out(fl32(S)
    + bias), S = sum_t x * wdq as fl32 (float64 array), A = sum_t |x * wdq|."""
    code, odt = _OUT[out_dtype]
    x = _c(x_bf16, np.uint16)
    m, k = x.shape
    wdq = dequant_weight(w, ws)
    n = wdq.shape[0]
    assert wdq.shape[1] == k
    b = None if bias is None else _c(bias, odt)
    out = np.empty((m, n), odt)
    s = np.empty((m, n), np.float64)
    a = np.empty((m, n), np.float64)
    _load().ck_oracle_linear_dequant(_ptr(x), k, _ptr(wdq), _ptr(b), _ptr(out), n, m, n, k,
                                     code, _ptr(s), _ptr(a))
    return out, s, a


def int8_linear(x_bf16, w, ws, bias=None, mode="row", out_dtype="bf16"):
    """The whole layer: quantise x, then integer product and epilogue.

    Returns (q, x_scale, out)."""
    if mode == "row":
        q, s = quantize_rowwise(x_bf16)
    elif mode == "tensor":
        q, s = quantize_tensorwise(x_bf16)
    else:
        raise ValueError(mode)
    return q, s, linear(q, s, w, ws, bias, out_dtype)
