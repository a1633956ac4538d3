"""Exact decoders: code -> real value (float64), written from the format definitions.

Test infrastructure only (see ``oracle/__init__.py``).

* Integer weights (the announcement's "Unified quantization representation"
  section names bit width, sign and zero point as the parameters of a weight
  format): two's complement INT-b, plain UINT-b.
* Zero-exponent floats e0mN (announcement, section "Quantization support"): a
  sign bit and N magnitude bits, one unit per magnitude LSB, so e0m7 covers
  exactly the integers -127..127, the same set as INT8 without -128.
* e2m1 (MXFP4 element), e8m0 (MX shared scale): OCP Microscaling Formats v1.0,
  section 5.3 / 5.4.
* e4m3: OCP 8-bit Floating Point (OFP8) "E4M3" -- bias 7, no infinities, the
  all-ones exponent+mantissa pattern is NaN, largest finite 448.
* bf16: the upper 16 bits of an IEEE binary32.

Every decoder computes from the bit fields; nothing here is a lookup table.
"""
from __future__ import annotations

import numpy as np


def unpack_bitstream(packed: np.ndarray, bits: int, count: int) -> np.ndarray:
    """Read ``count`` b-bit codes per row from an LSB-first bitstream (last axis bytes).

    Code i occupies stream bits ``[bits*i, bits*i + bits)``; stream bit j is bit
    ``j % 8`` of byte ``j // 8``.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    if bits == 4:
        # two codes per byte: even k in the low nibble, odd k in the high nibble
        out = np.empty(lead + (2 * packed.shape[-1],), dtype=np.int64)
        out[..., 0::2] = packed & 15
        out[..., 1::2] = packed >> 4
        return out[..., :count]
    flat = packed.reshape(-1, packed.shape[-1])
    out = np.zeros((flat.shape[0], count), dtype=np.int64)
    for j in range(bits):
        pos = np.arange(count, dtype=np.int64) * bits + j
        byte = flat[:, pos // 8].astype(np.int64)
        out |= ((byte >> (pos % 8)) & 1) << j
    return out.reshape(*lead, count)


def decode_int(codes, bits: int) -> np.ndarray:
    """Two's complement INT-b: c - 2^b when the sign bit is set."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c >= (1 << (bits - 1)), c - (1 << bits), c).astype(np.float64)


def decode_uint(codes) -> np.ndarray:
    return np.asarray(codes, dtype=np.int64).astype(np.float64)


def decode_e0m(codes, bits: int) -> np.ndarray:
    """e0m(b-1): sign = bit b-1, magnitude = low b-1 bits (integer units); -0 == 0."""
    c = np.asarray(codes, dtype=np.int64)
    mag = c & ((1 << (bits - 1)) - 1)
    sign = (c >> (bits - 1)) & 1
    return np.where(sign == 1, -mag, mag).astype(np.float64)


def decode_e2m1(codes) -> np.ndarray:
    """OCP e2m1: bias 1; exponent 0 is subnormal (m * 0.5); no Inf/NaN."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return np.where(s == 1, -mag, mag)


def decode_e4m3(codes) -> np.ndarray:
    """OCP E4M3: bias 7; exponent 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.exp2(-6.0) * (m / 8.0), np.exp2(e - 7.0) * (1.0 + m / 8.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def decode_e8m0(codes) -> np.ndarray:
    """OCP E8M0 scale: 2^(c-127) for c in 0..254; 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)
