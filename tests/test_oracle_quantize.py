"""Pins of the oracle's MXFP8 / MXFP4 quantizers and MoE output stage (CPU only).

Each pin ties ``oracle.quantize`` to something other than itself: hand-worked
cases of the OCP MX conversion rule, an exact round trip of representable
blocks, a brute-force nearest-value search over every finite e4m3 / e2m1
value, the input generator's independent quantizer (grid-step arithmetic),
closed forms of SiLU and torch's float64 SiLU.
"""
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import quantize as Q
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp8_quantize_cases.txt")
GOLDEN4 = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_quantize_cases.txt")


def _cases(path=GOLDEN):
    out = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, vals, scale, codes = [p.strip() for p in line.split("|")]
        x = np.zeros(32)
        c = np.zeros(32, dtype=np.uint8)
        for tok in vals.split():
            i, v = tok.split("=")
            x[int(i)] = float(v)
        for tok in codes.split():
            i, v = tok.split("=")
            c[int(i)] = int(v, 16)
        out.append((name, x, int(scale), c))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0])
def test_hand_worked_cases(case):
    _, x, scale, codes = case
    c, s = Q.quantize_mxfp8(x[None, :])
    assert int(s[0, 0]) == scale
    np.testing.assert_array_equal(c[0], codes)


def test_representable_blocks_round_trip():
    # blocks made of e4m3 values times 2^E, with one element in the top binade
    # [256, 448]: the scale rule must give back E and every code exactly
    r = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    codes = r.choice(finite, size=(400, 32)).astype(np.uint8)
    top = r.integers(0x78, 0x7F, size=400)
    pos = r.integers(0, 32, size=400)
    codes[np.arange(400), pos] = (top | (r.integers(0, 2, size=400) << 7)).astype(np.uint8)
    e = r.integers(-119, 112, size=400)
    x = F.decode_e4m3(codes) * np.exp2(e.astype(np.float64))[:, None]
    c, s = Q.quantize_mxfp8(x.reshape(100, 128))
    np.testing.assert_array_equal(s.reshape(400), (e + 127).astype(np.uint8))
    # -0 codes stay -0 (sign kept); compare exactly
    np.testing.assert_array_equal(c.reshape(400, 32), codes)


def test_nearest_by_brute_force():
    r = np.random.default_rng(12)
    v = np.concatenate([r.normal(0, 60, 3000), r.uniform(-500, 500, 3000),
                        r.normal(0, 0.01, 2000)])
    codes = Q.e4m3_nearest(v)
    allc = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    allv = F.decode_e4m3(allc)
    got = F.decode_e4m3(codes.astype(np.int64))
    clipped = np.clip(v, -448, 448)
    dist = np.abs(allv[None, :] - clipped[:, None])
    best = dist.min(axis=1)
    np.testing.assert_array_equal(np.abs(got - clipped), best)
    # ties: the chosen code is even among the nearest ones
    nearest = dist == best[:, None]
    ties = nearest.sum(axis=1) > 1
    tie_codes = codes[ties] & 0x7F
    nz = np.abs(got[ties]) > 0
    assert np.all(tie_codes[nz] % 2 == 0)
    # sign kept
    assert np.all(((codes >> 7) & 1) == np.signbit(v))


def test_midpoints_go_to_even():
    # midpoints between consecutive non-negative e4m3 values
    vals = F.decode_e4m3(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    c = Q.e4m3_nearest(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(c, expect.astype(np.uint8))


def test_scale_rule_invariant():
    r = np.random.default_rng(13)
    x = r.normal(0, 1, size=(64, 256)) * np.exp2(r.integers(-40, 40, size=(64, 1)))
    _, s = Q.quantize_mxfp8(x)
    amax = np.abs(x.reshape(64, 8, 32)).max(axis=-1)
    ratio = amax / np.exp2(s.astype(np.float64) - 127)
    assert np.all((ratio >= 256) & (ratio < 512))


def test_agrees_with_grid_step_quantizer():
    # the input generator quantizes by grid-step arithmetic (rint(a / step));
    # the oracle searches the value table: two independent routes
    import synth
    r = np.random.default_rng(14)
    xb = synth.x_bf16(r, 96, 512)
    xv = F.decode_bf16(xb)
    c1, s1 = Q.quantize_mxfp8(xv)
    c2, s2 = synth.mx_quantize(xv, "e4m3")
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


def test_dequantized_error_bounds():
    r = np.random.default_rng(15)
    x = r.normal(0, 3, size=(16, 512))
    c, s = Q.quantize_mxfp8(x)
    d = Q.dequantize_mxfp8(c, s)
    # in units of the block scale X the largest step is 32 (binade [256, 512)),
    # so unsaturated values err by <= 16 X; values in (448 X, 512 X) saturate
    # to 448 X and err by < 64 X
    xs = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=-1)
    sat = np.abs(x) > 448 * xs
    assert np.all(np.abs(d - x)[~sat] <= 16 * xs[~sat])
    assert np.all(np.abs(d - x)[sat] < 64 * xs[sat])
    # and within 2^-4 relative for unsaturated values in the normal range
    big = (np.abs(x) >= 2.0 ** -6 * xs) & ~sat
    assert np.all(np.abs(d - x)[big] <= 2.0 ** -4 * np.abs(x)[big])


@pytest.mark.parametrize("case", _cases(GOLDEN4), ids=lambda c: c[0])
def test_mxfp4_hand_worked_cases(case):
    _, x, scale, codes = case
    c, s = Q.quantize_mxfp4(x[None, :])
    assert int(s[0, 0]) == scale
    np.testing.assert_array_equal(c[0], codes)


def test_mxfp4_representable_blocks_round_trip():
    # e2m1 values times 2^E with one element of magnitude 4 or 6 (the top
    # binade [4, 8)): the scale rule gives back E and every code exactly
    r = np.random.default_rng(16)
    codes = r.integers(0, 16, size=(400, 32)).astype(np.uint8)
    pos = r.integers(0, 32, size=400)
    codes[np.arange(400), pos] = (r.integers(6, 8, size=400) | (r.integers(0, 2, size=400) << 3)).astype(np.uint8)
    e = r.integers(-125, 126, size=400)
    x = F.decode_e2m1(codes) * np.exp2(e.astype(np.float64))[:, None]
    c, s = Q.quantize_mxfp4(x.reshape(100, 128))
    np.testing.assert_array_equal(s.reshape(400), (e + 127).astype(np.uint8))
    np.testing.assert_array_equal(c.reshape(400, 32), codes)   # -0 stays 0x8


def test_e2m1_nearest_by_brute_force_and_midpoints():
    r = np.random.default_rng(17)
    v = np.concatenate([r.normal(0, 2, 4000), r.uniform(-8, 8, 4000)])
    codes = Q.e2m1_nearest(v)
    allv = F.decode_e2m1(np.arange(16))
    got = F.decode_e2m1(codes.astype(np.int64))
    clipped = np.clip(v, -6, 6)
    best = np.abs(allv[None, :] - clipped[:, None]).min(axis=1)
    np.testing.assert_array_equal(np.abs(got - clipped), best)
    assert np.all(((codes >> 3) & 1) == np.signbit(v))
    # the midpoints between consecutive non-negative values go to the even code
    vals = F.decode_e2m1(np.arange(8))
    mids = (vals[:-1] + vals[1:]) / 2
    lo = np.arange(7)
    np.testing.assert_array_equal(Q.e2m1_nearest(mids), np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))


def test_mxfp4_agrees_with_grid_step_quantizer_and_bounds():
    import synth
    r = np.random.default_rng(18)
    xb = synth.x_bf16(r, 64, 512)
    xv = F.decode_bf16(xb)
    c1, s1 = Q.quantize_mxfp4_bf16(xb)
    c2, s2 = synth.mx_quantize(xv, "e2m1")
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)
    # scale rule: the block maximum lies in [4 X, 8 X)
    amax = np.abs(xv.reshape(64, 16, 32)).max(axis=-1)
    ratio = amax / F.decode_e8m0(s1)
    assert np.all((ratio >= 4) & (ratio < 8))
    # error: half the largest step (2 X) where unsaturated, < 2 X above 6 X
    d = Q.dequantize_mxfp4(c1, s1)
    xs = np.repeat(F.decode_e8m0(s1), 32, axis=-1)
    sat = np.abs(xv) > 6 * xs
    assert np.all(np.abs(d - xv)[~sat] <= 1 * xs[~sat])
    assert np.all(np.abs(d - xv)[sat] < 2 * xs[sat])
    # packing: element 2i in the low nibble of byte i
    p = Q.pack_e2m1(c1)
    np.testing.assert_array_equal(p, synth.pack_codes(c1, 4))


def test_silu_closed_forms():
    torch = pytest.importorskip("torch")
    v = np.linspace(-30, 30, 1001)
    s = Q.silu(v)
    assert Q.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - Q.silu(-v), v, rtol=0, atol=1e-12)  # silu(v) - silu(-v) = v
    np.testing.assert_allclose(s, torch.nn.functional.silu(torch.from_numpy(v)).numpy(),
                               rtol=1e-15, atol=1e-300)
    gu = np.concatenate([v[None, :], np.full((1, 1001), 2.0)], axis=1)
    np.testing.assert_array_equal(Q.silu_mul(gu, 1001)[0], 2.0 * s)


def test_combine_cases():
    y = np.arange(12, dtype=np.float64).reshape(6, 2)   # 3 tokens, topk 2
    w = np.array([[1.0, 0.0], [0.5, 0.5], [2.0, -1.0]])
    out = Q.moe_combine(y, w, 2)
    np.testing.assert_array_equal(out, [[0, 1], [(4 + 6) / 2, (5 + 7) / 2], [2 * 8 - 10, 2 * 9 - 11]])
    out_b = Q.moe_combine(y, w, 2, bias=np.array([1.0, -1.0]))
    np.testing.assert_array_equal(out_b, out + [[1, -1]])
    # topk = 1 with unit weights is the identity
    np.testing.assert_array_equal(Q.moe_combine(y, np.ones((6, 1)), 1), y)


# ---------------------------------------------------------------------------
# FP8 with fp32 scales (per token, per 128 values)
# ---------------------------------------------------------------------------

GOLDEN_FP8 = os.path.join(os.path.dirname(__file__), "golden", "fp8_quantize_cases.txt")


def _fp8_cases():
    out = []
    for line in open(GOLDEN_FP8):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, vals, scale, codes = [p.strip() for p in line.split("|")]
        x = np.zeros(8)
        c = np.zeros(8, dtype=np.uint8)
        for tok in vals.split():
            i, v = tok.split("=")
            x[int(i)] = float(v)
        for tok in codes.split():
            i, v = tok.split("=")
            c[int(i)] = int(v, 16)
        out.append((name, x, float(scale), c))
    return out


@pytest.mark.parametrize("case", _fp8_cases(), ids=lambda c: c[0])
def test_fp8_hand_worked_cases(case):
    _, x, scale, codes = case
    c, s = Q.quantize_fp8(x[None, :])
    assert s.dtype == np.float32 and float(s[0]) == scale
    np.testing.assert_array_equal(c[0], codes)


def _torch_fp8(x, block):
    """The same rule through torch's fp32 arithmetic and its e4m3 cast."""
    import torch
    t = torch.from_numpy(np.asarray(x, np.float32))
    rows, k = t.shape
    b = k if block is None else block
    nb = -(-k // b)
    tp = torch.zeros((rows, nb * b), dtype=torch.float32)
    tp[:, :k] = t
    blk = tp.view(rows, nb, b)
    amax = blk.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / s[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(rows, nb * b)[:, :k]
    return q.numpy(), (s[:, 0] if block is None else s).numpy()


@pytest.mark.parametrize("block", [None, 128])
def test_fp8_matches_torch_route(block):
    """Random bf16 rows over a wide range of magnitudes, K not a multiple of
    the block: codes and scales equal torch's fp32 division and e4m3 cast."""
    r = np.random.default_rng(21)
    x = r.normal(0, 1, size=(64, 320)) * np.exp2(r.integers(-20, 20, size=(64, 1)))
    x[3] = 0.0
    x[5, :130] = 0.0
    xb = synth.f32_to_bf16_bits(x.astype(np.float32))
    c, s = Q.quantize_fp8_bf16(xb, block)
    ct, st = _torch_fp8(F.decode_bf16(xb), block)
    np.testing.assert_array_equal(s, st)
    np.testing.assert_array_equal(c, ct)


def test_fp8_round_trip_of_representable_rows():
    """Rows of e4m3 values times 2^E with one element at +-448: the scale is
    exactly 2^E and every code comes back."""
    r = np.random.default_rng(22)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    codes = r.choice(finite, size=(200, 64)).astype(np.uint8)
    codes[np.arange(200), r.integers(0, 64, size=200)] = r.choice([0x7E, 0xFE], size=200)
    e = r.integers(-100, 100, size=200)
    x = F.decode_e4m3(codes) * np.exp2(e.astype(np.float64))[:, None]
    c, s = Q.quantize_fp8(x)
    np.testing.assert_array_equal(s, np.exp2(e).astype(np.float32))
    # +-0 codes come back as +-0 (0x00 / 0x80)
    np.testing.assert_array_equal(c, codes)


def test_fp8_block_scales_are_per_128():
    """Block scaling equals per-token scaling of each 128-value slice."""
    r = np.random.default_rng(23)
    x = synth.f32_to_bf16_bits(r.normal(0, 1, size=(5, 384)).astype(np.float32))
    c, s = Q.quantize_fp8_bf16(x, 128)
    assert s.shape == (5, 3)
    for kb in range(3):
        ck, sk = Q.quantize_fp8_bf16(x[:, 128 * kb:128 * kb + 128])
        np.testing.assert_array_equal(c[:, 128 * kb:128 * kb + 128], ck)
        np.testing.assert_array_equal(s[:, kb], sk)
