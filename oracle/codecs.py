"""Storage codecs of the compressed cache (oracle side, test infrastructure).

bf16   upper 16 bits of an IEEE fp32; encoding rounds fp64 -> fp32 -> bf16,
       each round-to-nearest-even.  Decoding is exact.
fp16   IEEE binary16 (numpy float16); used for the int4 group scales.
int4   symmetric per-group-of-32 quantisation (the LowRAM-Q composition of
       the LowRAM review's comparison table): codes in [-7, 7],
       scale = fp16(absmax / 7), code = clamp(rint(x / scale)) with
       round-half-even, a zero group gets scale 0 and zero codes.  Two codes
       per byte, the even element in the low nibble, two's complement.
       Dequantised value = float(code) * float(scale).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- bf16 --
def bf16_encode(x) -> np.ndarray:
    """fp64/fp32 values -> bf16 bit patterns (uint16), RNE at each narrowing."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    # round to nearest even on the 16 dropped bits
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    return bf16_decode(bf16_encode(x))


# ---------------------------------------------------------------- fp16 --
def fp16_encode(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_decode(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- int4 --
INT4_GROUP = 32
INT4_QMAX = 7


def int4_encode(x):
    """Quantise the last axis in groups of 32.

    Returns (packed uint8 [..., n/2], scale bits uint16 [..., n/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % INT4_GROUP:
        raise ValueError("last axis must be a multiple of 32")
    g = x.reshape(x.shape[:-1] + (n // INT4_GROUP, INT4_GROUP))
    absmax = np.max(np.abs(g), axis=-1)
    scale_bits = fp16_encode(absmax / INT4_QMAX)
    scale = fp16_decode(scale_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(scale[..., None] > 0, np.rint(g / scale[..., None]), 0.0)
    q = np.clip(q, -INT4_QMAX, INT4_QMAX).astype(np.int8).reshape(x.shape)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return packed, scale_bits


def int4_codes(packed) -> np.ndarray:
    """Unpack two's-complement nibbles (even element = low nibble) to int8."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int8)
    hi = (p >> 4).astype(np.int8)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def int4_decode(packed, scale_bits) -> np.ndarray:
    """Dequantise: float(code) * float(scale) per group of 32, fp64."""
    q = int4_codes(packed).astype(np.float64)
    s = fp16_decode(scale_bits)
    n = q.shape[-1]
    g = q.reshape(q.shape[:-1] + (n // INT4_GROUP, INT4_GROUP))
    return (g * s[..., None]).reshape(q.shape)
