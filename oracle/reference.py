"""Plain reference of the quantized GEMM: decode -> dequantize -> float64 GEMM.

Test infrastructure only (see ``oracle/__init__.py``).

What is computed (readings of the Humming pages, listed with reasons in the
design notes):

* The announcement's section "Shared CUDA components" says dequantization and
  scaling are part of the kernel's computation, and the English benchmark page,
  section "H100 group-32 W4A8", says the fused kernel and the QDQ baseline
  (dequantize, then a plain GEMM) were all numerically correct.  So the
  reference is the QDQ form written out: decode every code exactly,
  dequantize, and multiply in float64.
* Dequantized weight (A16 formats): the exact real ``(q - z) * s``, with q the
  decoded code, z the group's zero point (0 for symmetric formats) and s the
  group's bf16 scale, groups running along K.  No rounding is applied: the
  product of a <=5-bit integer and a bf16 is exact in binary32 and in float64.
* MXFP4 weights and MXFP8 activations: ``e2m1(c) * 2^(e-127)`` and
  ``e4m3(a) * 2^(ea-127)``, one e8m0 scale per 32 consecutive K elements.
* More WnA16 weights (announcement, section "WnA16": integer and
  floating-point weights from 1 to 8 bits share the dequantize-and-compute
  path): INT-b / UINT-b for b in 1, 2, 3, 4, 8 (two's complement / plain with
  a zero point), the zero-exponent formats e0m3 / e0m7 (section
  "Quantization support": sign and magnitude, the values of INT4 without -8
  and of INT8 without -128) and e4m3 weights, each with a bf16 scale per
  group: ``(q - z) * s`` as above.
* Per-token FP8 activations (section "End to end": W4A8 serving with FP8
  activations scaled per token): ``e4m3(a) * s_row`` with one fp32 scale per
  row.
* W8A8 FP8 with block-wise scaling (section "W8A8 / W4A8 / W4A4"): e4m3
  weights with one fp32 scale per 128 x 128 block of W (128 output rows by
  128 K), e4m3 activations with one fp32 scale per row and 128 K.
* Y = Xdq @ Wdq^T summed in float64.
* MoE (announcement, "WnA16" section: tokens spread over experts with
  per-expert load): pair p = t*topk + j goes to expert topk_ids[t, j]; its output
  row is the dense product of its input row with that expert's weights.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import formats as F

W_INT4, W_UINT4, W_INT3, W_UINT3, W_MXFP4 = 0, 1, 2, 3, 4
W_INT8, W_UINT8, W_INT2, W_UINT2, W_INT1, W_UINT1, W_E0M3, W_E0M7, W_FP8 = 5, 6, 7, 8, 9, 10, 11, 12, 13
A_BF16, A_MXFP8, A_MXFP4, A_FP8_TOKEN, A_FP8_BLOCK = 0, 1, 2, 3, 4
_BITS = {W_INT4: 4, W_UINT4: 4, W_INT3: 3, W_UINT3: 3, W_MXFP4: 4, W_INT8: 8, W_UINT8: 8, W_INT2: 2,
         W_UINT2: 2, W_INT1: 1, W_UINT1: 1, W_E0M3: 4, W_E0M7: 8, W_FP8: 8}
_SIGNED_INT = (W_INT4, W_INT3, W_INT8, W_INT2, W_INT1)
_UNSIGNED_INT = (W_UINT4, W_UINT3, W_UINT8, W_UINT2, W_UINT1)
FP8_BLOCK = 128   # W8A8: weight scales per 128 x 128 block, activation scales per 128 along K


# ----------------------------------------------------------------------------
# dequantization
# ----------------------------------------------------------------------------

def weight_values(wtype: int, codes_packed: np.ndarray, k: int) -> np.ndarray:
    """Decoded weight codes (before scaling) as float64 [..., N, K]."""
    bits = _BITS[wtype]
    c = F.unpack_bitstream(codes_packed, bits, k)
    if wtype in _SIGNED_INT:
        return F.decode_int(c, bits)
    if wtype in _UNSIGNED_INT:
        return F.decode_uint(c)
    if wtype in (W_E0M3, W_E0M7):
        return F.decode_e0m(c, bits)
    if wtype == W_FP8:
        return F.decode_e4m3(c)
    return F.decode_e2m1(c)


def dequant_weights(wtype: int, codes_packed: np.ndarray, scales: np.ndarray,
                    zeros: np.ndarray | None, k: int, group: int) -> np.ndarray:
    """Wdq [..., N, K] float64.

    A16 formats: (q - z) * s[n, k // group], s a bf16 pattern.  MXFP4: e2m1 *
    2^(e - 127) with group 32.
    """
    v = weight_values(wtype, codes_packed, k)
    if wtype == W_MXFP4:
        assert group == 32
        s = F.decode_e8m0(scales)
    else:
        s = F.decode_bf16(scales)
        if zeros is not None:
            v = v - np.repeat(np.asarray(zeros, dtype=np.float64), group, axis=-1)
    return v * np.repeat(s, group, axis=-1)


def dequant_weights_fp8_block(codes: np.ndarray, scales: np.ndarray, n: int, k: int) -> np.ndarray:
    """W8A8 weights Wdq [..., N, K] float64: e4m3 codes (one byte per
    element, [..., N, K]) times the fp32 scale of their 128 x 128 block,
    scales [..., ceil(N / 128), ceil(K / 128)]."""
    v = F.decode_e4m3(np.asarray(codes)[..., :n, :k])
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    s = np.repeat(np.repeat(s, FP8_BLOCK, axis=-2), FP8_BLOCK, axis=-1)[..., :n, :k]
    return v * s


def dequant_activations(atype: int, x: np.ndarray, x_scales: np.ndarray | None,
                        k: int) -> np.ndarray:
    """Xdq [rows, K] float64: bf16 patterns; e4m3 codes times e8m0 per-32
    scales (MXFP8); e4m3 codes times one fp32 scale per row (per-token FP8,
    x_scales [rows]) or per row and 128 K (block FP8, x_scales [rows,
    ceil(K / 128)])."""
    if atype == A_BF16:
        return F.decode_bf16(x)[..., :k]
    v = F.decode_e4m3(np.asarray(x)[..., :k])
    if atype == A_FP8_TOKEN:
        return v * np.asarray(x_scales, dtype=np.float32).astype(np.float64)[..., None]
    if atype == A_FP8_BLOCK:
        s = np.asarray(x_scales, dtype=np.float32).astype(np.float64)
        return v * np.repeat(s, FP8_BLOCK, axis=-1)[..., :k]
    return v * np.repeat(F.decode_e8m0(x_scales), 32, axis=-1)


# ----------------------------------------------------------------------------
# GEMM
# ----------------------------------------------------------------------------

def gemm(xdq: np.ndarray, wdq: np.ndarray) -> np.ndarray:
    """Y = X @ W^T in float64 (numpy's float64 matmul)."""
    return np.matmul(np.asarray(xdq, np.float64), np.asarray(wdq, np.float64).T)


def gemm_exact(xdq: np.ndarray, wdq: np.ndarray) -> list:
    """Exact rational Y = X @ W^T by brute force (tiny shapes only)."""
    m, k = xdq.shape
    n = wdq.shape[0]
    xf = [[Fraction(float(xdq[i, j])) for j in range(k)] for i in range(m)]
    wf = [[Fraction(float(wdq[i, j])) for j in range(k)] for i in range(n)]
    return [[sum((xf[i][j] * wf[o][j] for j in range(k)), Fraction(0)) for o in range(n)]
            for i in range(m)]


def qg_gemm(wtype: int, codes_packed, scales, zeros, n: int, k: int, group: int,
            atype: int, x, x_scales=None) -> np.ndarray:
    """Dense reference: Y[M, N] float64 from standard-format inputs (W8A8
    block FP8: ``codes_packed`` one e4m3 byte per element, ``scales`` fp32
    per 128 x 128 block)."""
    if atype == A_FP8_BLOCK:
        wdq = dequant_weights_fp8_block(codes_packed, scales, n, k)
    else:
        wdq = dequant_weights(wtype, codes_packed, scales, zeros, k, group)
    assert wdq.shape == (n, k)
    xdq = dequant_activations(atype, x, x_scales, k)
    return gemm(xdq, wdq)


# ----------------------------------------------------------------------------
# MoE
# ----------------------------------------------------------------------------

def moe_counts(topk_ids: np.ndarray, experts: int) -> np.ndarray:
    """Rows routed to each expert."""
    return np.bincount(np.asarray(topk_ids).reshape(-1), minlength=experts).astype(np.int64)


def moe_offsets(topk_ids: np.ndarray, experts: int) -> np.ndarray:
    """Exclusive prefix sum of the per-expert counts, length E + 1."""
    c = moe_counts(topk_ids, experts)
    return np.concatenate([[0], np.cumsum(c)]).astype(np.int64)


def moe_sorted_pairs(topk_ids: np.ndarray, experts: int) -> np.ndarray:
    """One valid expert-sorted order of the pair ids p = t*topk + j (stable)."""
    e = np.asarray(topk_ids).reshape(-1)
    return np.argsort(e, kind="stable").astype(np.int64)


def moe_gemm(expert_weights, x_rows: np.ndarray, topk_ids: np.ndarray,
             rows_by_token: bool) -> np.ndarray:
    """Grouped reference, output rows indexed by pair id.

    ``expert_weights(e)`` returns Wdq[e] (float64 [N, K]); ``x_rows`` is the
    dequantized input: [T, K] when ``rows_by_token`` (row of pair p is token
    p // topk) or [P, K] indexed by pair.
    """
    t, topk = topk_ids.shape
    flat = np.asarray(topk_ids).reshape(-1)
    p_total = t * topk
    y = None
    for e in np.unique(flat):
        pairs = np.nonzero(flat == e)[0]
        rows = pairs // topk if rows_by_token else pairs
        ye = gemm(x_rows[rows], expert_weights(int(e)))
        if y is None:
            y = np.zeros((p_total, ye.shape[1]), dtype=np.float64)
        y[pairs] = ye
    return y


# ----------------------------------------------------------------------------
# comparison
# ----------------------------------------------------------------------------

def round_bf16(y: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest-even bf16 value, as float64.

    bf16 keeps 8 significant bits and binary32's exponent range, so below the
    smallest normal 2^-126 its spacing stays 2^-133 (subnormals).  Values past
    the largest finite bf16 are not expected here."""
    y = np.asarray(y, dtype=np.float64)
    m, e = np.frexp(y)          # y = m * 2^e, 0.5 <= |m| < 1
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))  # 8 significant bits, subnormal floor
    return np.where(y == 0, 0.0, np.rint(y / quantum) * quantum)


def normwise_error(y: np.ndarray, yref: np.ndarray) -> float:
    """max |Y - Yref| / max |Yref| (0 when both are zero)."""
    y = np.asarray(y, dtype=np.float64)
    yref = np.asarray(yref, dtype=np.float64)
    den = np.max(np.abs(yref)) if yref.size else 0.0
    num = np.max(np.abs(y - yref)) if yref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
