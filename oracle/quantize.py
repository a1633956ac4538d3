"""Reference activation quantization and MoE output stage -- TEST INFRASTRUCTURE.

Only ``tests/``, the smoke check and the CPU-baseline leg of ``bench.py`` use
this module (see ``oracle/__init__.py``); the library never does.

* bf16 -> MXFP8 (announcement, section "Choosing the activation type": a
  deployment may override the checkpoint's activation type, e.g. MXFP8 for the
  MoE layers, so bf16 activations are quantized at run time before the W4A8
  GEMM).  The conversion follows the OCP Microscaling Formats v1.0 rule
  (section 6.3): per block of 32 consecutive values along K, the shared scale
  is X = 2^(floor(log2(max |V_i|)) - emax_elem), emax_elem = 8 for e4m3; each
  element is V_i / X rounded to the nearest e4m3 value, ties to the even
  code, with magnitudes beyond the largest finite value (448) saturated to it.
  The scale's e8m0 code is log2(X) + 127, clamped to 0..254; an all-zero block
  has X = 1.  Rounding keeps the input's sign, so a negative value that rounds
  to zero gives the code 0x80 (e4m3 -0).
  Written here as a search over the 127 non-negative finite e4m3 values, which
  are decoded from their bit fields by ``formats.decode_e4m3``.
* bf16 -> MXFP4 (announcement, section "W8A8 / W4A8 / W4A4": MXFP4 on both
  operands).  The same OCP rule with e2m1 elements: emax_elem = 2 (the largest
  e2m1 value is 6 = 1.5 * 2^2), elements rounded to the nearest of the eight
  non-negative e2m1 values, ties to the even code, saturated at 6, sign kept
  (a negative value that rounds to zero gives code 0x8).  Codes are returned
  one per element; ``pack_e2m1`` puts two per byte, element 2i in the low
  nibble of byte i.
* bf16 -> FP8 with fp32 scales (announcement, section "End to end": W4A8
  serving with per-token FP8 activations; section "W8A8 / W4A8 / W4A4": FP8
  with block-wise scaling).  The pages name the granularity only, so the rule
  is the plain one, in fp32 arithmetic: per block (a whole row for per-token
  scaling, 128 consecutive values of a row for block scaling) with largest
  magnitude a, the scale is s = fl32(a / 448) (448 = the largest e4m3 value;
  s = 1 for an all-zero block), and each element is e4m3 of fl32(v / s),
  nearest with ties to the even code, saturated at 448, sign kept.  fl32 is
  IEEE binary32 division, rounded to nearest-even.
* MoE output stage (announcement, section "Shared CUDA components": scaling
  and bias additions can be fused into the output stage; MoE layers route each
  token to top-k experts):
  - SiLU-gated product of the fused gate/up projection:
    h[r, j] = silu(g[r, j]) * g[r, I + j], silu(v) = v / (1 + e^-v),
    for j < I where the fused row holds the gate half then the up half.
  - Weighted combine of the top-k expert outputs of each token:
    out[t, n] = sum_j w[t, j] * y[t*topk + j, n] (+ bias[n]).
  Both in float64.
"""
from __future__ import annotations

import numpy as np

from . import formats as F

E4M3_EMAX = 8          # largest e4m3 binade: 448 = 1.75 * 2^8
_E4M3_MAX_CODE = 0x7E  # 448


def _e4m3_table():
    """Non-negative finite e4m3 values in increasing code order (codes 0x00..0x7E)."""
    codes = np.arange(_E4M3_MAX_CODE + 1, dtype=np.int64)
    return codes, F.decode_e4m3(codes)


def mx_block_exponent(amax: np.ndarray, emax_elem: int = E4M3_EMAX) -> np.ndarray:
    """floor(log2(amax)) - emax_elem clamped to [-127, 127]; 0 for amax == 0.

    floor(log2 a) is read off frexp exactly: a = f * 2^e with f in [0.5, 1)."""
    a = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    x = np.clip(e.astype(np.int64) - 1 - emax_elem, -127, 127)
    return np.where(a > 0, x, 0)


def e4m3_nearest(v: np.ndarray) -> np.ndarray:
    """e4m3 code of each real v: nearest finite value, ties to the even code,
    |v| > 448 saturated to 448, sign taken from v (including -0.0)."""
    v = np.asarray(v, dtype=np.float64)
    codes, vals = _e4m3_table()
    a = np.minimum(np.abs(v), vals[-1])
    hi = np.searchsorted(vals, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    mag = np.where(a == vals[hi], codes[hi], np.where(pick_hi, codes[hi], codes[lo]))
    sign = np.signbit(v).astype(np.int64)
    return ((sign << 7) | mag).astype(np.uint8)


def quantize_mxfp8(x: np.ndarray):
    """MXFP8 quantization of real rows [rows, K] (K % 32 == 0) along K.

    Returns (codes uint8 [rows, K] e4m3, scales uint8 [rows, K/32] e8m0)."""
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    blk = x.reshape(rows, k // 32, 32)
    e = mx_block_exponent(np.abs(blk).max(axis=-1))
    scaled = blk * np.exp2(-e.astype(np.float64))[..., None]   # exact: power-of-two scale
    codes = e4m3_nearest(scaled).reshape(rows, k)
    return codes, (e + 127).astype(np.uint8)


def quantize_mxfp8_bf16(x_bits: np.ndarray):
    """quantize_mxfp8 of bf16 bit patterns (uint16 [rows, K])."""
    return quantize_mxfp8(F.decode_bf16(x_bits))


def dequantize_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Real values of MXFP8 rows: e4m3(code) * 2^(scale - 127), blocks of 32."""
    v = F.decode_e4m3(codes)
    s = F.decode_e8m0(scales)
    return v * np.repeat(s, 32, axis=-1)


E2M1_EMAX = 2          # largest e2m1 binade: 6 = 1.5 * 2^2


def e2m1_nearest(v: np.ndarray) -> np.ndarray:
    """e2m1 code of each real v: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to
    the even code, |v| > 6 saturated to 6, sign (bit 3) taken from v
    (including -0.0)."""
    v = np.asarray(v, dtype=np.float64)
    codes = np.arange(8, dtype=np.int64)
    vals = F.decode_e2m1(codes)                          # increasing with the code
    a = np.minimum(np.abs(v), vals[-1])
    d = np.abs(a[..., None] - vals)                      # distance to every value
    best = d.min(axis=-1, keepdims=True)
    tied = d == best                                      # one or two nearest codes
    even = tied & (codes % 2 == 0)
    mag = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(tied, axis=-1))
    sign = np.signbit(v).astype(np.int64)
    return ((sign << 3) | mag).astype(np.uint8)


def quantize_mxfp4(x: np.ndarray):
    """MXFP4 quantization of real rows [rows, K] (K % 32 == 0) along K.

    Returns (codes uint8 [rows, K], one e2m1 code per element,
    scales uint8 [rows, K/32] e8m0)."""
    x = np.asarray(x, dtype=np.float64)
    rows, k = x.shape
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    blk = x.reshape(rows, k // 32, 32)
    e = mx_block_exponent(np.abs(blk).max(axis=-1), E2M1_EMAX)
    scaled = blk * np.exp2(-e.astype(np.float64))[..., None]   # exact: power-of-two scale
    codes = e2m1_nearest(scaled).reshape(rows, k)
    return codes, (e + 127).astype(np.uint8)


def quantize_mxfp4_bf16(x_bits: np.ndarray):
    """quantize_mxfp4 of bf16 bit patterns (uint16 [rows, K])."""
    return quantize_mxfp4(F.decode_bf16(x_bits))


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte along the last axis: element 2i in the low
    nibble of byte i, element 2i + 1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def dequantize_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Real values of MXFP4 rows (one code per element): e2m1(code) *
    2^(scale - 127), blocks of 32."""
    v = F.decode_e2m1(codes)
    s = F.decode_e8m0(scales)
    return v * np.repeat(s, 32, axis=-1)


E4M3_MAX = 448.0


def quantize_fp8(x: np.ndarray, block: int | None = None):
    """FP8 quantization of rows [rows, K] of fp32-representable reals.

    block = None: one scale per row (per token); block = B: one scale per B
    consecutive values (the last block of a row may be shorter).  Returns
    (codes uint8 [rows, K] e4m3, scales float32 [rows] or [rows, ceil(K/B)])."""
    x = np.asarray(x, dtype=np.float64)
    x32 = x.astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), x, equal_nan=True):
        raise ValueError("inputs must be exact in fp32")
    rows, k = x.shape
    b = k if block is None else block
    nb = -(-k // b)
    xp = np.zeros((rows, nb * b), np.float32)
    xp[:, :k] = x32
    blk = xp.reshape(rows, nb, b)
    amax = np.abs(blk).max(axis=-1)                                   # exact
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)              # IEEE fp32 division
    s = np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)
    q = (blk / s[..., None]).astype(np.float32)                       # IEEE fp32 division
    # keep -0.0 of negative zeros: the division preserves the sign
    codes = e4m3_nearest(q.astype(np.float64)).reshape(rows, nb * b)[:, :k]
    return codes, (s[:, 0] if block is None else s)


def quantize_fp8_bf16(x_bits: np.ndarray, block: int | None = None):
    """quantize_fp8 of bf16 bit patterns (uint16 [rows, K])."""
    return quantize_fp8(F.decode_bf16(x_bits), block)


def silu(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def silu_mul(gu: np.ndarray, inter: int) -> np.ndarray:
    """h[r, j] = silu(gu[r, j]) * gu[r, inter + j] for j < inter (float64)."""
    gu = np.asarray(gu, dtype=np.float64)
    return silu(gu[:, :inter]) * gu[:, inter:2 * inter]


def moe_combine(y: np.ndarray, topk_weights: np.ndarray, topk: int,
                bias: np.ndarray | None = None) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y[t*topk + j] (+ bias), float64 [T, N]."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float64)
    t = w.shape[0]
    out = (y.reshape(t, topk, -1) * w[:, :, None]).sum(axis=1)
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    return out
