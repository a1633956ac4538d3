"""Pins for the oracle's format decoders and for the input generators' encoders.

Each decoder is checked against something other than itself: torch's own
float8 / bfloat16 dtypes, the OCP value tables in ``tests/golden/``, numpy's bit
unpacking, and the e0m7 identity the Humming announcement states in its
"Quantization support" section.
"""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def _same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


def test_e2m1_matches_ocp_table():
    rows = _read_table("e2m1_ocp_mx_v1.txt")
    assert len(rows) == 16
    codes = np.array([c for c, _ in rows])
    got = F.decode_e2m1(codes)
    assert _same(got, [v for _, v in rows])
    assert sorted(set(np.abs(got).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    # sign is bit 3
    assert np.all(np.signbit(got[8:]) | (got[8:] == 0))


def test_e4m3_matches_torch_and_ocp_table():
    codes = np.arange(256)
    got = F.decode_e4m3(codes)
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert _same(got, lib)
    for c, v in _read_table("e4m3_ocp_ofp8.txt"):
        assert _same(got[c], v), hex(c)
    finite = got[np.isfinite(got)]
    assert finite.size == 254
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert got[0x01] == 2.0 ** -9
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"


def test_e8m0_matches_torch():
    codes = np.arange(256)
    got = F.decode_e8m0(codes)
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert _same(got, lib)
    assert got[127] == 1.0 and got[128] == 2.0 and got[0] == 2.0 ** -127
    assert np.isnan(got[255])


def test_bf16_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = F.decode_bf16(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert _same(got, lib)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_int_decode_matches_sign_extension(bits):
    c = np.arange(1 << bits)
    got = F.decode_int(c, bits)
    # sign-extend through an int8 shift pair (a different route than the decoder)
    sh = 8 - bits
    ref = ((c.astype(np.uint8) << sh).view(np.int8) >> sh).astype(np.float64)
    assert np.array_equal(got, ref)
    assert got.min() == -(1 << (bits - 1)) and got.max() == (1 << (bits - 1)) - 1


def test_e0m7_identity_with_int8_without_minus_128():
    """Announcement, "Quantization support": e0m7 values are the integers -127..127,
    the same set as INT8 without -128."""
    e0 = F.decode_e0m(np.arange(256), 8)
    assert set(e0.tolist()) == set(range(-127, 128))
    assert e0[0x00] == 0 and e0[0x80] == 0  # +0 and -0
    int8 = F.decode_int(np.arange(256), 8)
    for c in range(256):
        if c == 0x80:
            continue
        assert int8[c] in set(e0.tolist())
        match = np.nonzero(e0 == int8[c])[0]
        assert match.size >= 1
    # same for e0m3 vs INT4 without -8
    e03 = F.decode_e0m(np.arange(16), 4)
    assert set(e03.tolist()) == set(range(-7, 8))
    int4 = F.decode_int(np.arange(16), 4)
    assert set(int4.tolist()) - set(e03.tolist()) == {-8.0}


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_unpack_bitstream_matches_numpy_unpackbits(bits):
    r = np.random.default_rng(7)
    k = 96
    packed = r.integers(0, 256, size=(5, k * bits // 8), dtype=np.uint8)
    got = F.unpack_bitstream(packed, bits, k)
    stream = np.unpackbits(packed, axis=1, bitorder="little").astype(np.int64)
    ref = (stream.reshape(5, k, bits) << np.arange(bits)).sum(axis=2)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_pack_codes_roundtrip(bits):
    r = np.random.default_rng(3)
    codes = r.integers(0, 1 << bits, size=(4, 7, 256), dtype=np.uint8)
    packed = synth.pack_codes(codes, bits)
    assert packed.shape == (4, 7, 256 * bits // 8)
    assert np.array_equal(F.unpack_bitstream(packed, bits, 256), codes)
    # LSB-first: code 0 sits in the low bits of byte 0
    one = np.zeros((1, 8), np.uint8)
    one[0, 0] = 5
    assert synth.pack_codes(one, 4)[0, 0] == 5


def test_bf16_rounding_of_generator_matches_torch():
    r = np.random.default_rng(11)
    x = (r.normal(0, 1, 100000) * np.exp2(r.integers(-30, 30, 100000))).astype(np.float32)
    got = synth.f32_to_bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, lib)


def test_mx_e4m3_rounding_matches_torch():
    """The generator's e4m3 element rounding equals torch's float8_e4m3fn cast in range."""
    r = np.random.default_rng(5)
    v = r.uniform(-440, 440, 20000) * np.exp2(r.integers(-12, 1, 20000))
    v = v.astype(np.float32).astype(np.float64)  # both sides round the same float32 values
    q = np.copysign(synth._round_to_grid(np.abs(v), "e4m3"), v)
    codes = synth._encode_e4m3(q)
    lib = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, lib)
    assert np.array_equal(F.decode_e4m3(codes), q)


def test_mx_quantize_blocks():
    r = np.random.default_rng(9)
    x = r.normal(0, 1, size=(6, 128))
    x[1, 32:64] = 0.0
    for fmt, dec, vmax in (("e4m3", F.decode_e4m3, 448.0), ("e2m1", F.decode_e2m1, 6.0)):
        codes, sc = synth.mx_quantize(x, fmt)
        assert codes.shape == x.shape and sc.shape == (6, 4)
        assert sc[1, 1] == 127  # all-zero block -> 2^0
        val = dec(codes) * np.repeat(F.decode_e8m0(sc), 32, axis=1)
        blk = np.abs(x).reshape(6, 4, 32).max(axis=2)
        emax = 8 if fmt == "e4m3" else 2
        for i in range(6):
            for b in range(4):
                if blk[i, b] == 0:
                    continue
                e = math.floor(math.log2(blk[i, b])) - emax
                assert sc[i, b] == e + 127
        # every element is within half a quantum of the grid, or saturated
        scale = np.repeat(F.decode_e8m0(sc), 32, axis=1)
        err = np.abs(val - x) / scale
        a = np.abs(x) / scale
        mbits = 3 if fmt == "e4m3" else 1
        minexp = -6 if fmt == "e4m3" else 0
        with np.errstate(divide="ignore"):
            quantum = np.exp2(np.maximum(np.floor(np.log2(np.where(a > 0, a, 1))), minexp) - mbits)
        ok = (err <= quantum / 2 + 1e-12) | (np.abs(dec(codes)) == vmax)
        assert ok.all()
