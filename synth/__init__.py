"""Seeded synthetic inputs for the quantized GEMM, in the standard (unpacked) format.

This module is shared by the tests, the smoke check and the benchmark.  It only
*draws* inputs: codes, scales, zero points, activations and router choices.  It
holds none of the GEMM arithmetic (no decoding of codes to values, no
dequantization, no matrix product); the oracle and the HIP library each do that
on their own.

Standard format (the layout every producer hands to ``qg_preprocess``):

* weight codes ``[E][N][K]`` row-major, each row an LSB-first bitstream of
  b-bit codes (code k occupies bits ``[b*k, b*k+b)`` of the row);
* scales ``[E][N][K/g]``: bf16 bit patterns (uint16) or e8m0 codes (uint8);
* zero points ``[E][N][K/g]`` uint8 in ``0 .. 2^b-1`` (asymmetric formats only);
* activations ``[rows][K]``: bf16 bit patterns, or e4m3 codes with e8m0
  scales ``[rows][K/32]``.

The value distributions follow the workloads quoted on the Humming pages'
"H100 group-32 W4A8" and "SM80 single-request decode" sections and the
announcement's "WnA16" / "W8A8 / W4A8 / W4A4" sections: group-wise INT4/INT3
weights with bf16 scales, MXFP4 weights, bf16 or MXFP8 activations.
"""
from __future__ import annotations

import numpy as np

# Weight-type names shared with the C header (values match ``qg_wtype``).
W_INT4, W_UINT4, W_INT3, W_UINT3, W_MXFP4 = 0, 1, 2, 3, 4
W_INT8, W_UINT8, W_INT2, W_UINT2, W_INT1, W_UINT1, W_E0M3, W_E0M7, W_FP8 = 5, 6, 7, 8, 9, 10, 11, 12, 13
WTYPE_BITS = {W_INT4: 4, W_UINT4: 4, W_INT3: 3, W_UINT3: 3, W_MXFP4: 4, W_INT8: 8, W_UINT8: 8, W_INT2: 2,
              W_UINT2: 2, W_INT1: 1, W_UINT1: 1, W_E0M3: 4, W_E0M7: 8, W_FP8: 8}
WTYPE_HAS_ZP = {w: w in (W_UINT4, W_UINT3, W_UINT8, W_UINT2, W_UINT1) for w in WTYPE_BITS}


def rng(seed: int, *stream: int) -> np.random.Generator:
    """A numpy generator keyed by (seed, *stream) so parts can be regenerated alone."""
    return np.random.default_rng([int(seed), *[int(s) for s in stream]])


# ----------------------------------------------------------------------------
# bit-level helpers (layout only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even) and return the bit patterns.

    Used to draw bf16 activations and scales; NaN is not expected in inputs.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack b-bit codes (last axis = K) into an LSB-first bitstream of bytes per row."""
    codes = np.asarray(codes, dtype=np.uint8)
    k = codes.shape[-1]
    assert (k * bits) % 8 == 0, "row must fill whole bytes"
    lead = codes.shape[:-1]
    c = codes.reshape(-1, k)
    # bit j of code i -> stream bit i*bits + j
    bitplanes = ((c[:, :, None] >> np.arange(bits, dtype=np.uint8)) & 1).astype(np.uint8)
    stream = bitplanes.reshape(c.shape[0], k * bits)
    packed = np.packbits(stream, axis=1, bitorder="little")
    return packed.reshape(*lead, k * bits // 8)


# ----------------------------------------------------------------------------
# group-wise integer weights (A16 paths)
# ----------------------------------------------------------------------------

def scales_bf16(r: np.random.Generator, shape, sigma: float = 0.02) -> np.ndarray:
    """bf16(|N(0, sigma)|) bit patterns."""
    return f32_to_bf16_bits(np.abs(r.normal(0.0, sigma, size=shape)).astype(np.float32))


def int_weights(r: np.random.Generator, n: int, k: int, wtype: int, group: int,
                experts: int | None = None):
    """Draw group-wise integer weights in the standard format.

    Signed types draw codes uniformly over the full two's-complement range
    ([-8, 7] for INT4, [-4, 3] for INT3) and have no zero point.  Unsigned
    types draw codes and zero points uniformly over ``0 .. 2^b-1``.
    Returns ``(codes_packed, scales_bits, zeros_or_None, raw_codes)``.
    """
    bits = WTYPE_BITS[wtype]
    lead = (n,) if experts is None else (experts, n)
    assert k % group == 0
    if wtype == W_FP8:
        # e4m3 codes of N(0, 1) values (finite: NaN codes never drawn)
        raw = _encode_e4m3(np.copysign(_round_to_grid(np.abs(r.normal(0.0, 1.0, size=lead + (k,))), "e4m3"),
                                       r.choice([-1.0, 1.0], size=lead + (k,))))
    else:
        raw = r.integers(0, 1 << bits, size=lead + (k,), dtype=np.uint8)  # code bits
    sc = scales_bf16(r, lead + (k // group,))
    zp = None
    if WTYPE_HAS_ZP[wtype]:
        zp = r.integers(0, 1 << bits, size=lead + (k // group,), dtype=np.uint8)
    return pack_codes(raw, bits), sc, zp, raw


def fp8_block_weights(r: np.random.Generator, n: int, k: int, experts: int | None = None,
                      sigma: float = 0.02):
    """W8A8 weights: e4m3 codes [.., N, K] (one byte per element) of N(0,
    sigma^2) values over fp32 scales, one per 128 x 128 block
    ([.., ceil(N/128), ceil(K/128)]): each block's scale is its largest
    magnitude / 448 (1 for an all-zero block), the codes the nearest-even
    e4m3 of value / scale."""
    lead = (n,) if experts is None else (experts, n)
    w = r.normal(0.0, sigma, size=lead + (k,))
    nb, kb = -(-n // 128), -(-k // 128)
    wp = np.zeros(lead[:-1] + (nb * 128, kb * 128))
    wp[..., :n, :k] = w
    blk = wp.reshape(lead[:-1] + (nb, 128, kb, 128))
    amax = np.abs(blk).max(axis=(-3, -1))
    sc = np.where(amax > 0, amax / _E4M3_MAX, 1.0).astype(np.float32)
    full = np.repeat(np.repeat(sc.astype(np.float64), 128, axis=-2), 128, axis=-1)
    v = wp / full
    codes = _encode_e4m3(np.copysign(_round_to_grid(np.abs(v), "e4m3"), v))[..., :n, :k]
    return np.ascontiguousarray(codes), sc


def fp8_activations(r: np.random.Generator, m: int, k: int, block: int | None, sigma: float = 1.0):
    """e4m3 activations [m, k] over fp32 scales, one per row (block None) or
    per row and ``block`` values: scale = block max / 448, codes nearest-even."""
    x = r.normal(0.0, sigma, size=(m, k))
    b = k if block is None else block
    nb = -(-k // b)
    xp = np.zeros((m, nb * b))
    xp[:, :k] = x
    amax = np.abs(xp.reshape(m, nb, b)).max(axis=-1)
    sc = np.where(amax > 0, amax / _E4M3_MAX, 1.0).astype(np.float32)
    v = xp / np.repeat(sc.astype(np.float64), b, axis=-1)
    codes = _encode_e4m3(np.copysign(_round_to_grid(np.abs(v), "e4m3"), v))[:, :k]
    return np.ascontiguousarray(codes), (sc[:, 0] if block is None else sc)


def int4_weights_packed(r: np.random.Generator, n: int, k: int, wtype: int, group: int):
    """Large 4-bit weights drawn directly in packed form.

    Uniform random bytes are exactly a stream of i.i.d. uniform 4-bit codes, so
    this has the distribution of :func:`int_weights` without the per-code
    packing cost.  Returns ``(codes_packed, scales_bits, zeros_or_None)``.
    """
    assert WTYPE_BITS[wtype] == 4 and wtype != W_MXFP4 and k % group == 0
    codes = r.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    sc = scales_bf16(r, (n, k // group))
    zp = r.integers(0, 16, size=(n, k // group), dtype=np.uint8) if WTYPE_HAS_ZP[wtype] else None
    return codes, sc, zp


def x_bf16(r: np.random.Generator, m: int, k: int, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of N(0, sigma) activations, shape [m, k]."""
    return f32_to_bf16_bits(r.normal(0.0, sigma, size=(m, k)).astype(np.float32))


# ----------------------------------------------------------------------------
# MX encoding (input synthesis for the MXFP4 x MXFP8 path)
#
# OCP Microscaling Formats (MX) v1.0, section 6.3 (conversion): the shared
# exponent of a 32-element block is floor(log2(amax)) - emax_elem, and every
# element is rounded to nearest-even on its own grid, saturating at the
# format's largest finite magnitude.  An all-zero block gets scale 2^0.
# ----------------------------------------------------------------------------

_E4M3_MAX, _E2M1_MAX = 448.0, 6.0
_EMAX = {"e4m3": 8, "e2m1": 2}


def _round_to_grid(a: np.ndarray, fmt: str) -> np.ndarray:
    """Round non-negative reals to the nearest-even point of the e4m3 / e2m1 grid."""
    if fmt == "e4m3":
        min_normal_exp, mbits, vmax = -6, 3, _E4M3_MAX
    else:
        min_normal_exp, mbits, vmax = 0, 1, _E2M1_MAX
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, min_normal_exp)
    quantum = np.exp2(e - mbits)
    q = np.rint(a / quantum) * quantum  # np.rint rounds half to even
    return np.minimum(q, vmax)


def _encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Bit pattern of grid values (already representable) in OCP e4m3."""
    s = np.signbit(v).astype(np.uint8)
    a = np.abs(v)
    sub = a < 2.0 ** -6
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, a)))
    exp_field = np.where(sub, 0, e + 7).astype(np.int64)
    man = np.where(sub, a / 2.0 ** -9, (a / np.exp2(e) - 1.0) * 8.0)
    man = np.rint(man).astype(np.int64)
    return ((s.astype(np.int64) << 7) | (exp_field << 3) | man).astype(np.uint8)


def _encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Bit pattern of grid values (already representable) in OCP e2m1 (bit 3 = sign)."""
    s = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    sub = a < 1.0
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(sub, 1.0, a)))
    exp_field = np.where(sub, 0, e + 1).astype(np.int64)
    man = np.where(sub, a / 0.5, (a / np.exp2(e) - 1.0) * 2.0)
    man = np.rint(man).astype(np.int64)
    return ((s << 3) | (exp_field << 1) | man).astype(np.uint8)


def mx_quantize(x: np.ndarray, fmt: str):
    """MX-quantize real values along the last axis (blocks of 32).

    Returns ``(codes uint8 [..., K], scales uint8 [..., K/32])``; e2m1 codes are
    one per byte (use :func:`pack_codes` with 4 bits for the standard format).
    """
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1]
    assert k % 32 == 0
    blk = x.reshape(*x.shape[:-1], k // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - _EMAX[fmt]
    e = np.where(amax > 0, e, 0.0)
    e = np.clip(e, -127, 127)
    scaled = blk / np.exp2(e)[..., None]
    q = np.copysign(_round_to_grid(np.abs(scaled), fmt), scaled)
    codes = _encode_e4m3(q) if fmt == "e4m3" else _encode_e2m1(q)
    return codes.reshape(x.shape).astype(np.uint8), (e + 127).astype(np.uint8)


def mx_weights(r: np.random.Generator, n: int, k: int, sigma: float = 0.02,
               experts: int | None = None):
    """MXFP4 weights: OCP-quantized N(0, sigma^2), one e8m0 scale per 32 along K.

    Returns ``(codes_packed [.., N, K/2], scales [.., N, K/32], raw_codes)``.
    """
    lead = (n,) if experts is None else (experts, n)
    w = r.normal(0.0, sigma, size=lead + (k,))
    codes, sc = mx_quantize(w, "e2m1")
    return pack_codes(codes, 4), sc, codes


def mx_activations(r: np.random.Generator, m: int, k: int, sigma: float = 1.0):
    """MXFP8 activations: e4m3 codes [m, k] and e8m0 scales [m, k/32] of N(0, sigma^2)."""
    return mx_quantize(r.normal(0.0, sigma, size=(m, k)), "e4m3")


# ----------------------------------------------------------------------------
# MoE routing (input synthesis: the router is upstream of the grouped GEMM)
# ----------------------------------------------------------------------------

def zipf_bias(r: np.random.Generator, experts: int, a: float = 1.1) -> np.ndarray:
    """Per-expert logit bias -a*ln(rank), ranks a seeded permutation of 1..E.

    Adding a*ln-rank to the logits makes expert popularity fall off like a Zipf
    law with exponent ``a`` (the skewed per-expert load the announcement's
    "WnA16" section describes for MoE).
    """
    ranks = r.permutation(experts) + 1
    return -a * np.log(ranks.astype(np.float64))


def route(r: np.random.Generator, tokens: int, experts: int, topk: int,
          a: float = 1.1) -> np.ndarray:
    """top-k expert ids [tokens, topk] (int32) from N(0,1) logits plus a Zipf bias.

    Ties go to the lower expert index (a stable sort of -logits)."""
    bias = zipf_bias(r, experts, a)
    logits = r.normal(0.0, 1.0, size=(tokens, experts)) + bias[None, :]
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :topk].astype(np.int32)
