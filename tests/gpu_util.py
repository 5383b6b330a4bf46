"""Helpers for the GPU parity tests: device checks and bit-level comparisons."""
import numpy as np
import pytest


def cuda_device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bits16(t):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ordered(bits):
    """bf16 bit patterns -> integers whose difference counts bf16 ulps
    (+0 and -0 both map to 0)."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_diff(a_bits, b_bits):
    return np.abs(ordered(a_bits) - ordered(b_bits))


def assert_bf16_within_1ulp(got_bits, ref_bits, what=""):
    """The bar for bf16 outputs: at most 1 bf16 ulp apart (relative 2^-8).
    Returns the fraction that is bit-identical."""
    assert got_bits.shape == ref_bits.shape
    d = ulp_diff(got_bits, ref_bits)
    worst = int(d.max()) if d.size else 0
    if worst > 1:
        i = np.unravel_index(int(d.argmax()), d.shape)
        raise AssertionError(f"{what}: {worst} ulp at {i}: got {got_bits[i]:#06x} "
                             f"want {ref_bits[i]:#06x}; {(d > 1).sum()} elements > 1 ulp")
    return float((d == 0).mean()) if d.size else 1.0


def ordered32(f):
    """float32 values -> integers whose difference counts float32 ulps."""
    b = np.ascontiguousarray(f, np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


def assert_within_1ulp(got, ref, what=""):
    """The bar for floating outputs of any type: uint16 arrays hold bf16 or
    fp16 bit patterns, float32 arrays fp32 values; at most 1 ulp of that
    type apart.  Returns the fraction that is bit-identical."""
    if got.dtype == np.uint16:
        return assert_bf16_within_1ulp(got, ref, what)
    assert got.shape == ref.shape and got.dtype == np.float32 == ref.dtype
    d = np.abs(ordered32(got) - ordered32(ref))
    worst = int(d.max()) if d.size else 0
    if worst > 1:
        i = np.unravel_index(int(d.argmax()), d.shape)
        raise AssertionError(f"{what}: {worst} ulp at {i}: got {got[i]!r} want {ref[i]!r}")
    return float((d == 0).mean()) if d.size else 1.0
