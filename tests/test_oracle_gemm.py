"""Pins for the oracle's dequantization, GEMM and MoE reference.

Chosen so a plausible slip (nibble order, zero-point sign, group index, a
transposed operand, a dropped term, a wrong expert) fails at least one test:
exact rational brute force, integer-GEMM special cases, closed forms, one-hot
probes at group boundaries and invariants of the routing sort.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import formats as F

BF16_ONE = 0x3F80


def _x_small_ints(r, m, k, lo=-3, hi=4):
    vals = r.integers(lo, hi, size=(m, k)).astype(np.float32)
    return synth.f32_to_bf16_bits(vals), vals.astype(np.float64)


A16_WTYPES = [oracle.W_INT4, oracle.W_UINT4, oracle.W_INT3, oracle.W_UINT3, oracle.W_INT8, oracle.W_UINT8,
              oracle.W_INT2, oracle.W_UINT2, oracle.W_INT1, oracle.W_UINT1, oracle.W_E0M3, oracle.W_E0M7,
              oracle.W_FP8]
INT_WTYPES = [oracle.W_INT4, oracle.W_UINT4, oracle.W_INT3, oracle.W_UINT3, oracle.W_INT8, oracle.W_UINT8,
              oracle.W_INT2, oracle.W_UINT2, oracle.W_INT1, oracle.W_UINT1]


@pytest.mark.parametrize("wtype", A16_WTYPES)
def test_fraction_bruteforce_equals_fp64_a16(wtype):
    r = np.random.default_rng(100 + wtype)
    m, n, k, g = 3, 5, 64, 32
    codes, sc, zp, _ = synth.int_weights(r, n, k, wtype, g)
    x = synth.x_bf16(r, m, k)
    y = oracle.qg_gemm(wtype, codes, sc, zp, n, k, g, oracle.A_BF16, x)
    xdq = oracle.dequant_activations(oracle.A_BF16, x, None, k)
    wdq = oracle.dequant_weights(wtype, codes, sc, zp, k, g)
    exact = oracle.gemm_exact(xdq, wdq)
    for i in range(m):
        for j in range(n):
            bound = 64 * 2.0 ** -52 * float(np.abs(xdq[i]) @ np.abs(wdq[j]))
            assert abs(Fraction(float(y[i, j])) - exact[i][j]) <= Fraction(bound)


def test_fraction_bruteforce_equals_fp64_mx():
    r = np.random.default_rng(200)
    m, n, k = 4, 6, 64
    wc, ws, _ = synth.mx_weights(r, n, k)
    xc, xs = synth.mx_activations(r, m, k)
    y = oracle.qg_gemm(oracle.W_MXFP4, wc, ws, None, n, k, 32, oracle.A_MXFP8, xc, xs)
    xdq = oracle.dequant_activations(oracle.A_MXFP8, xc, xs, k)
    wdq = oracle.dequant_weights(oracle.W_MXFP4, wc, ws, None, k, 32)
    exact = oracle.gemm_exact(xdq, wdq)
    for i in range(m):
        for j in range(n):
            assert Fraction(float(y[i, j])) == exact[i][j]  # dyadic, short span: exact


@pytest.mark.parametrize("wtype", INT_WTYPES)
def test_unit_scales_reduce_to_integer_gemm(wtype):
    """All scales 1.0 -> an integer GEMM, checked with numpy int64 on raw codes."""
    r = np.random.default_rng(300 + wtype)
    m, n, k, g = 4, 8, 256, 128
    codes, sc, zp, raw = synth.int_weights(r, n, k, wtype, g)
    sc = np.full_like(sc, BF16_ONE)
    xb, xv = _x_small_ints(r, m, k)
    y = oracle.qg_gemm(wtype, codes, sc, zp, n, k, g, oracle.A_BF16, xb)
    bits = synth.WTYPE_BITS[wtype]
    w = raw.astype(np.int64)
    if synth.WTYPE_HAS_ZP[wtype]:
        w = w - np.repeat(zp.astype(np.int64), g, axis=1)
    else:  # two's complement via int8 shift pair
        sh = 8 - bits
        w = ((raw << sh).view(np.int8) >> sh).astype(np.int64)
    ref = xv.astype(np.int64) @ w.T
    assert np.array_equal(y, ref.astype(np.float64))


@pytest.mark.parametrize("wtype,bits", [(oracle.W_E0M3, 4), (oracle.W_E0M7, 8)])
def test_e0m_unit_scales_reduce_to_integer_gemm(wtype, bits):
    """Announcement, "Quantization support": e0m codes are sign + magnitude in
    integer units.  With unit scales the GEMM is an integer GEMM on
    v = c for c < 2^(b-1) and v = 2^(b-1) - c otherwise (the magnitude
    negated), written here without bit masks."""
    r = np.random.default_rng(310 + wtype)
    m, n, k, g = 3, 6, 256, 64
    codes, sc, zp, raw = synth.int_weights(r, n, k, wtype, g)
    assert zp is None
    sc = np.full_like(sc, BF16_ONE)
    xb, xv = _x_small_ints(r, m, k)
    y = oracle.qg_gemm(wtype, codes, sc, None, n, k, g, oracle.A_BF16, xb)
    half = 1 << (bits - 1)
    raw = raw.astype(np.int64)
    w = np.where(raw < half, raw, half - raw)
    assert np.array_equal(y, (xv.astype(np.int64) @ w.T).astype(np.float64))


def test_fp8_weights_unit_scales_reduce_to_value_table_gemm():
    """e4m3 weights with bf16 scale 1.0: a GEMM on torch's e4m3 values."""
    r = np.random.default_rng(320)
    m, n, k, g = 3, 5, 128, 32
    codes, sc, _, raw = synth.int_weights(r, n, k, oracle.W_FP8, g)
    assert np.array_equal(codes, raw)            # 8-bit codes: one byte each
    sc = np.full_like(sc, BF16_ONE)
    xb, xv = _x_small_ints(r, m, k)
    y = oracle.qg_gemm(oracle.W_FP8, codes, sc, None, n, k, g, oracle.A_BF16, xb)
    wv = torch.from_numpy(raw.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(y, xv @ wv.T)


def test_fp8_block_closed_form():
    """W8A8 (announcement, "W8A8 / W4A8 / W4A4": FP8 with block-wise
    scaling): all codes 1.0 (0x38), activation scales 2^a[r, kb], weight
    scales 2^b[nb, kb] -> Y[r, n] = sum_kb 128 * 2^(a[r, kb] + b[n // 128, kb]).
    N = 200 has a partial second block of rows, K = 384 three blocks; a
    swapped block index or a per-column (not per-128-rows) weight scale fails."""
    m, n, k = 3, 200, 384
    a = np.array([[0, 1, 2], [3, -1, 0], [2, 2, -3]])
    b = np.array([[1, 0, -2], [0, 4, 1]])
    x = np.full((m, k), 0x38, np.uint8)
    w = np.full((n, k), 0x38, np.uint8)
    xs = np.exp2(a).astype(np.float32)
    ws = np.exp2(b).astype(np.float32)
    y = oracle.qg_gemm(oracle.W_FP8, w, ws, None, n, k, 128, oracle.A_FP8_BLOCK, x, xs)
    for r_ in range(m):
        for j in range(n):
            assert y[r_, j] == sum(128 * 2.0 ** (a[r_, kb] + b[j // 128, kb]) for kb in range(3))


def test_fp8_block_fraction_bruteforce_and_orientation():
    """Random W8A8 operands at distinct M, N, K: float64 equals the exact
    rational sum of e4m3(a) s_a[r, k // 128] e4m3(w) s_w[n // 128, k // 128]
    term by term."""
    r = synth.rng(0, 7)
    m, n, k = 2, 130, 256
    wc, ws = synth.fp8_block_weights(r, n, k)
    xc, xs = synth.fp8_activations(r, m, k, 128)
    y = oracle.qg_gemm(oracle.W_FP8, wc, ws, None, n, k, 128, oracle.A_FP8_BLOCK, xc, xs)
    e4 = {c: Fraction(float(v)) for c, v in enumerate(
        torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().tolist()) if v == v}
    for i in range(m):
        for j in (0, 1, 127, 128, 129):
            terms = [e4[int(xc[i, kk])] * Fraction(float(xs[i, kk // 128])) * e4[int(wc[j, kk])] *
                     Fraction(float(ws[j // 128, kk // 128])) for kk in range(k)]
            # float64 summation error: at most k ulps of the sum of magnitudes
            bound = k * Fraction(2) ** -52 * sum(abs(t) for t in terms)
            assert abs(Fraction(float(y[i, j])) - sum(terms)) <= bound


def test_per_token_fp8_w4a8_fraction_bruteforce():
    """MXFP4 weights x per-token FP8 activations (announcement, "End to
    end"): Y[r, n] = s_r * sum_k e4m3(a[r, k]) * e2m1(w[n, k]) 2^(e[n, k // 32] - 127),
    exactly (a one-scale row check catches a scale applied per column)."""
    r = synth.rng(0, 8)
    m, n, k = 3, 4, 64
    wc, wsc, wraw = synth.mx_weights(r, n, k)
    xc, xs = synth.fp8_activations(r, m, k, None)
    y = oracle.qg_gemm(oracle.W_MXFP4, wc, wsc, None, n, k, 32, oracle.A_FP8_TOKEN, xc, xs)
    e4 = torch.from_numpy(xc.copy()).view(torch.float8_e4m3fn).double().numpy()
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(float(e4[i, kk])) * Fraction(float(F.decode_e2m1(wraw[j, kk]))) *
                        Fraction(2) ** (int(wsc[j, kk // 32]) - 127) for kk in range(k))
            assert Fraction(float(y[i, j])) == Fraction(float(xs[i])) * exact


def test_closed_form_constant_codes_zero_point_and_groups():
    """Constant code c, zero point z, scale 2^g per group, X = ones:
    Y = sum_g 2^g * g_size * (c - z).  Catches a flipped zero-point sign or a
    wrong group index."""
    n, k, g = 3, 512, 128
    c, z = 11, 4
    raw = np.full((n, k), c, np.uint8)
    codes = synth.pack_codes(raw, 4)
    groups = k // g
    sc = np.tile(synth.f32_to_bf16_bits(np.exp2(np.arange(groups)).astype(np.float32)), (n, 1))
    zp = np.full((n, groups), z, np.uint8)
    x = np.full((2, k), BF16_ONE, np.uint16)
    y = oracle.qg_gemm(oracle.W_UINT4, codes, sc, zp, n, k, g, oracle.A_BF16, x)
    expect = sum(2.0 ** j * g * (c - z) for j in range(groups))
    assert np.all(y == expect)


def test_one_hot_rows_pick_single_weights_at_group_edges():
    """X = e_k returns column k of Wdq, i.e. (q - z) * s[n, k // g]."""
    r = np.random.default_rng(400)
    n, k, g = 4, 256, 32
    codes, sc, zp, raw = synth.int_weights(r, n, k, oracle.W_UINT4, g)
    ks = [0, 31, 32, 63, 64, 127, 128, 255]
    x = np.zeros((len(ks), k), np.uint16)
    for i, kk in enumerate(ks):
        x[i, kk] = BF16_ONE
    y = oracle.qg_gemm(oracle.W_UINT4, codes, sc, zp, n, k, g, oracle.A_BF16, x)
    s = F.decode_bf16(sc)
    for i, kk in enumerate(ks):
        for j in range(n):
            assert y[i, j] == (int(raw[j, kk]) - int(zp[j, kk // g])) * s[j, kk // g]


def test_transposed_operands_are_detected():
    """Y[m, n] = sum_k X[m, k] W[n, k] with every dimension distinct."""
    r = np.random.default_rng(500)
    m, n, k, g = 2, 3, 32, 32
    codes, sc, zp, raw = synth.int_weights(r, n, k, oracle.W_INT4, g)
    xb, xv = _x_small_ints(r, m, k)
    y = oracle.qg_gemm(oracle.W_INT4, codes, sc, zp, n, k, g, oracle.A_BF16, xb)
    s = F.decode_bf16(sc)
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                q = int(raw[j, kk])
                q = q - 16 if q >= 8 else q
                acc += xv[i, kk] * q * s[j, kk // g]
            assert y[i, j] == pytest.approx(acc, rel=1e-14, abs=1e-14)


def test_linearity_in_x():
    r = np.random.default_rng(600)
    n, k, g = 8, 256, 128
    codes, sc, zp, _ = synth.int_weights(r, n, k, oracle.W_UINT4, g)
    xa, va = _x_small_ints(r, 3, k)
    xb, vb = _x_small_ints(r, 3, k)
    xs = synth.f32_to_bf16_bits((va + vb).astype(np.float32))
    ya = oracle.qg_gemm(oracle.W_UINT4, codes, sc, zp, n, k, g, oracle.A_BF16, xa)
    yb = oracle.qg_gemm(oracle.W_UINT4, codes, sc, zp, n, k, g, oracle.A_BF16, xb)
    ys = oracle.qg_gemm(oracle.W_UINT4, codes, sc, zp, n, k, g, oracle.A_BF16, xs)
    assert np.allclose(ys, ya + yb, rtol=0, atol=1e-9 * np.abs(ys).max())


def test_mx_unit_scales_reduce_to_value_table_gemm():
    """Every scale code 127 -> a GEMM on e4m3 (torch) and e2m1 (OCP table) values."""
    r = np.random.default_rng(700)
    m, n, k = 3, 4, 64
    wraw = r.integers(0, 16, size=(n, k), dtype=np.uint8)
    xraw = r.integers(0, 256, size=(m, k), dtype=np.uint8)
    xraw[(xraw & 0x7F) == 0x7F] = 0x38  # no NaN codes
    ws = np.full((n, k // 32), 127, np.uint8)
    xs = np.full((m, k // 32), 127, np.uint8)
    y = oracle.qg_gemm(oracle.W_MXFP4, synth.pack_codes(wraw, 4), ws, None, n, k, 32,
                       oracle.A_MXFP8, xraw, xs)
    e2m1 = {}
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                e2m1[int(c, 16)] = float(v)
    wv = np.vectorize(e2m1.get)(wraw).astype(np.float64)
    xv = torch.from_numpy(xraw).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(y, xv @ wv.T)


def test_mx_block_scale_applies_per_32():
    r = np.random.default_rng(800)
    m, n, k = 2, 3, 128
    wc, ws, _ = synth.mx_weights(r, n, k)
    xc, xs = synth.mx_activations(r, m, k)
    y0 = oracle.qg_gemm(oracle.W_MXFP4, wc, ws, None, n, k, 32, oracle.A_MXFP8, xc, xs)
    ws2 = ws.copy()
    ws2[:, 2] += 1  # doubles block 2 of every weight row
    y1 = oracle.qg_gemm(oracle.W_MXFP4, wc, ws2, None, n, k, 32, oracle.A_MXFP8, xc, xs)
    xdq = oracle.dequant_activations(oracle.A_MXFP8, xc, xs, k)
    wdq = oracle.dequant_weights(oracle.W_MXFP4, wc, ws, None, k, 32)
    blk = xdq[:, 64:96] @ wdq[:, 64:96].T
    assert np.allclose(y1 - y0, blk, rtol=0, atol=1e-12)


def test_moe_sort_invariants():
    r = synth.rng(0, 1)
    t, e, topk = 300, 64, 8
    ids = synth.route(r, t, e, topk)
    assert ids.shape == (t, topk)
    assert all(len(set(row)) == topk for row in ids.tolist())  # distinct experts per token
    counts = oracle.moe_counts(ids, e)
    offs = oracle.moe_offsets(ids, e)
    assert counts.sum() == t * topk and offs[-1] == t * topk
    assert np.all(np.diff(offs) >= 0)
    order = oracle.moe_sorted_pairs(ids, e)
    flat = ids.reshape(-1)
    assert sorted(order.tolist()) == list(range(t * topk))
    for ex in range(e):
        seg = order[offs[ex]:offs[ex + 1]]
        assert set(seg.tolist()) == set(np.nonzero(flat == ex)[0].tolist())
    # Zipf bias skews the load
    assert counts.max() > 4 * np.median(counts[counts > 0])


def test_moe_gemm_matches_per_pair_products_and_permutes_with_tokens():
    r = synth.rng(0, 2)
    t, e, topk, n, k, g = 12, 6, 2, 8, 64, 32
    ids = synth.route(r, t, e, topk)
    codes, sc, zp, _ = synth.int_weights(r, n, k, oracle.W_UINT4, g, experts=e)
    wdq = [oracle.dequant_weights(oracle.W_UINT4, codes[i], sc[i], zp[i], k, g) for i in range(e)]
    xb, xv = _x_small_ints(r, t, k)
    y = oracle.moe_gemm(lambda i: wdq[i], xv, ids, rows_by_token=True)
    assert y.shape == (t * topk, n)
    for p in range(t * topk):
        ex = ids[p // topk, p % topk]
        assert np.array_equal(y[p], wdq[ex] @ xv[p // topk])
    perm = r.permutation(t)
    y2 = oracle.moe_gemm(lambda i: wdq[i], xv[perm], ids[perm], rows_by_token=True)
    pair_perm = (perm[:, None] * topk + np.arange(topk)).reshape(-1)
    assert np.array_equal(y2, y[pair_perm])
    # rows by pair: the down projection reads row p of H
    h = np.repeat(xv, topk, axis=0)
    y3 = oracle.moe_gemm(lambda i: wdq[i], h, ids, rows_by_token=False)
    assert np.array_equal(y3, y)


def test_round_bf16_and_normwise_error():
    r = np.random.default_rng(1)
    y = r.normal(0, 100, 5000).astype(np.float32).astype(np.float64)
    got = oracle.round_bf16(y)
    lib = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, lib)
    # binary32 subnormals and the normal/subnormal boundary, every tie case
    bits = np.concatenate([r.integers(1, 0x00800000, 3000, dtype=np.uint32),
                           r.integers(0x00700000, 0x00900000, 2000, dtype=np.uint32),
                           np.arange(0x00007FF0, 0x00008010, dtype=np.uint32)])
    bits = np.concatenate([bits, bits | 0x80000000])
    ys = bits.view(np.float32)
    got = oracle.round_bf16(ys.astype(np.float64))
    lib = torch.from_numpy(ys.copy()).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, lib)
    assert oracle.normwise_error(np.array([1.0, 2.0]), np.array([1.0, 2.5])) == pytest.approx(0.2)
    assert oracle.normwise_error(np.zeros(3), np.zeros(3)) == 0.0
