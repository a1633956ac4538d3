"""Host-side tests of the C ABI (no GPU needed).

* libqg.so loads and exports every entry point ``include/qg.h`` declares;
* descriptor validation returns the documented status codes;
* the host repack writes the packed layout its header comment describes
  (read back here by an independent decoder of that layout);
* argument errors in qg_gemm / qg_moe_gemm / qg_moe_sort come back as status
  codes before anything is launched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_gemm_qg_amd as qg
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "qg.h")).read()
    declared = set(re.findall(r"^(?:qg_status|const char \*|int32_t|void)\s*(qg_\w+)\(", hdr, re.M))
    assert declared == set(qg.EXPORTS)
    lib = ctypes.CDLL(qg.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def _desc(**kw):
    base = dict(wtype=qg.W_INT4, n=256, k=512, group_size=128)
    base.update(kw)
    return qg.layer_desc(base.pop("wtype"), base.pop("n"), base.pop("k"), base.pop("group_size"),
                         **base)


@pytest.mark.parametrize("kw,status", [
    (dict(k=500), qg.QG_ERR_SHAPE),                      # K % 32
    (dict(k=480, group_size=128), qg.QG_ERR_SHAPE),      # K % group
    (dict(n=0), qg.QG_ERR_SHAPE),
    (dict(group_size=256, k=512), qg.QG_ERR_UNSUPPORTED),
    (dict(atype=qg.A_MXFP8), qg.QG_ERR_UNSUPPORTED),     # INT4 x MXFP8: no kernel
    (dict(wtype=qg.W_MXFP4, group_size=64, atype=qg.A_BF16), qg.QG_ERR_UNSUPPORTED),
    (dict(wtype=qg.W_MXFP4, group_size=128), qg.QG_ERR_UNSUPPORTED),
    (dict(stype=qg.S_E8M0), qg.QG_ERR_UNSUPPORTED),
    (dict(wtype=14), qg.QG_ERR_INVALID_ARGUMENT),
    (dict(atype=5), qg.QG_ERR_INVALID_ARGUMENT),
    (dict(stype=3), qg.QG_ERR_INVALID_ARGUMENT),
    (dict(wtype=qg.W_INT8, stype=qg.S_E8M0), qg.QG_ERR_UNSUPPORTED),
    (dict(wtype=qg.W_INT2, atype=qg.A_FP8_TOKEN), qg.QG_ERR_UNSUPPORTED),
    (dict(atype=qg.A_FP8_BLOCK), qg.QG_ERR_UNSUPPORTED),               # INT4 x block FP8: no kernel
    (dict(wtype=qg.W_FP8, atype=qg.A_FP8_BLOCK, group_size=64), qg.QG_ERR_UNSUPPORTED),   # W8A8: 128
    (dict(wtype=qg.W_FP8, atype=qg.A_FP8_BLOCK, stype=qg.S_BF16), qg.QG_ERR_UNSUPPORTED),  # W8A8: fp32 scales
    (dict(wtype=qg.W_FP8, atype=qg.A_FP8_TOKEN), qg.QG_ERR_UNSUPPORTED),
    (dict(wtype=qg.W_MXFP4, group_size=32, atype=qg.A_FP8_BLOCK), qg.QG_ERR_UNSUPPORTED),
    (dict(atype=qg.A_MXFP4), qg.QG_ERR_UNSUPPORTED),     # INT4 x MXFP4: no kernel
    (dict(wtype=qg.W_MXFP4, group_size=32, atype=qg.A_MXFP4, k=544), qg.QG_ERR_UNSUPPORTED),  # W4A4: K % 128
])
def test_descriptor_validation(kw, status):
    with pytest.raises(qg.QGError) as e:
        qg.packed_size(_desc(**kw))
    assert e.value.status == status


def test_bad_abi_version():
    d = _desc()
    d.abi_version = 99
    with pytest.raises(qg.QGError) as e:
        qg.packed_size(d)
    assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT


BITS = {qg.W_INT4: 4, qg.W_UINT4: 4, qg.W_INT3: 3, qg.W_UINT3: 3, qg.W_MXFP4: 4, qg.W_INT8: 8, qg.W_UINT8: 8,
        qg.W_INT2: 2, qg.W_UINT2: 2, qg.W_INT1: 1, qg.W_UINT1: 1, qg.W_E0M3: 4, qg.W_E0M7: 8, qg.W_FP8: 8}
ZP_TYPES = (qg.W_UINT4, qg.W_UINT3, qg.W_UINT8, qg.W_UINT2, qg.W_UINT1)


def _layout(d):
    n_tiles = -(-d.n // 16)
    k_blocks = -(-d.k // 128)
    gpad = -(-(k_blocks * 128 // d.group_size) // 32) * 32
    kb_pad = -(-k_blocks // 4) * 4
    bits = BITS[d.wtype]
    mx = d.wtype == qg.W_MXFP4 and d.atype != qg.A_BF16
    f8 = d.atype == qg.A_FP8_BLOCK
    zp = d.wtype in ZP_TYPES
    bb = 256 * bits
    codes = n_tiles * k_blocks * bb
    al = lambda v: -(-v // 256) * 256  # noqa: E731
    s_off = al(codes)
    s_bytes = n_tiles * 16 * 4 * kb_pad if mx else n_tiles * kb_pad * 4 if f8 else n_tiles * 16 * gpad * 2
    end = s_off + s_bytes
    z_off = 0
    if zp:
        z_off = al(end)
        end = z_off + (n_tiles * 16 * gpad if bits == 8 else n_tiles * 16 * (gpad // 8) * 4)
    return dict(n_tiles=n_tiles, k_blocks=k_blocks, gpad=gpad, kb_pad=kb_pad, bits=bits, mx=mx, f8=f8,
                zp=zp, bb=bb, s_off=s_off, z_off=z_off, stride=al(end))


def test_packed_size_formula():
    for d in (_desc(), _desc(wtype=qg.W_UINT4, n=14336, k=4096),
              _desc(wtype=qg.W_INT3, n=40, k=640, group_size=32),
              _desc(wtype=qg.W_MXFP4, n=1280, k=640, group_size=32, num_experts=3),
              _desc(wtype=qg.W_UINT8, n=200, k=640, group_size=64),
              _desc(wtype=qg.W_UINT2, n=40, k=384, group_size=32, num_experts=2),
              _desc(wtype=qg.W_INT1, n=17, k=256),
              _desc(wtype=qg.W_FP8, n=300, k=512, atype=qg.A_FP8_BLOCK),
              _desc(wtype=qg.W_MXFP4, n=64, k=256, group_size=32, atype=qg.A_FP8_TOKEN)):
        assert qg.packed_size(d) == _layout(d)["stride"] * d.num_experts


def _slot(e):
    return e // 2 + 4 * (e % 2)


def _unpack_packed(d, buf):
    """Independent reader of the packed layout -> (codes[n,k] standard values,
    scales[n,g], zeros[n,g] or None) for expert 0."""
    L = _layout(d)
    n, k = d.n, d.k
    codes = np.zeros((n, k), np.int64)
    for nn in range(n):
        t, ln = divmod(nn, 16)
        for kk in range(k):
            kb, r = divmod(kk, 128)
            blk = (t * L["k_blocks"] + kb) * L["bb"]
            if L["mx"]:
                q, e = divmod(r, 32)
                byte = buf[blk + (ln + 16 * q) * 16 + e // 2]
                codes[nn, kk] = (byte >> (4 * (e % 2))) & 15
                continue
            if L["f8"]:
                half, rr = divmod(r, 64)
                q, i = divmod(rr, 16)
                codes[nn, kk] = buf[blk + (ln + 16 * q) * 32 + 16 * half + i]
                continue
            j, rr = divmod(r, 32)
            q, e = divmod(rr, 8)
            lane = ln + 16 * q
            if L["bits"] in (8, 2, 1):
                nb = L["bits"]
                base = blk + lane * 4 * nb
                if nb == 8:
                    u = buf[base + 8 * j + e]
                else:
                    word, slot = (j // 2, 4 * (j % 2) + e // 2 + 8 * (e % 2)) if nb == 2 else \
                        (0, 4 * j + e // 2 + 16 * (e % 2))
                    w = int.from_bytes(bytes(buf[base + 4 * word: base + 4 * word + 4]), "little")
                    u = (w >> (nb * slot)) & ((1 << nb) - 1)
                half_v = 1 << (nb - 1)
                if d.wtype in (qg.W_INT8, qg.W_INT2, qg.W_INT1):
                    u ^= half_v                       # back to the two's complement code
                elif d.wtype == qg.W_E0M7:
                    u = int(u) - half_v               # the value (checked against the e0m decode)
                codes[nn, kk] = u
                continue
            if L["bits"] == 4:
                w = int.from_bytes(bytes(buf[blk + lane * 16 + 4 * j: blk + lane * 16 + 4 * j + 4]), "little")
                u = (w >> (4 * _slot(e))) & 15
                codes[nn, kk] = u ^ 8 if d.wtype == qg.W_INT4 else u - 8 if d.wtype == qg.W_E0M3 else u
            else:
                ws = [int.from_bytes(bytes(buf[blk + lane * 12 + 4 * b: blk + lane * 12 + 4 * b + 4]), "little")
                      for b in range(3)]
                if j < 3:
                    u = (ws[j] >> (4 * _slot(e))) & 7
                else:
                    u = sum(((ws[b] >> (4 * _slot(e) + 3)) & 1) << b for b in range(3))
                codes[nn, kk] = u ^ 4 if d.wtype == qg.W_INT3 else u
    G = k // d.group_size
    if L["f8"]:
        f = np.frombuffer(bytes(buf[L["s_off"]:L["s_off"] + L["n_tiles"] * L["kb_pad"] * 4]), np.float32)
        return codes, f.reshape(L["n_tiles"], L["kb_pad"]), None
    if L["mx"]:
        sc = np.zeros((n, k // 32), np.int64)
        for nn in range(n):
            for i in range(k // 32):
                kb, q = divmod(i, 4)
                unit = (nn // 16) * (L["kb_pad"] // 4) + kb // 4
                sc[nn, i] = buf[L["s_off"] + unit * 256 + ((nn % 16) * 4 + q) * 4 + kb % 4]
        return codes, sc, None
    s16 = np.frombuffer(bytes(buf[L["s_off"]:L["s_off"] + d.n * L["gpad"] * 2]), np.uint16)
    sc = s16.reshape(d.n, L["gpad"])[:, :G].astype(np.int64)
    zp = None
    if L["zp"] and L["bits"] == 8:
        zb = np.frombuffer(bytes(buf[L["z_off"]:L["z_off"] + d.n * L["gpad"]]), np.uint8)
        zp = zb.reshape(d.n, L["gpad"])[:, :G].astype(np.int64)
    elif L["zp"]:
        words = np.frombuffer(bytes(buf[L["z_off"]:L["z_off"] + d.n * L["gpad"] // 2]), np.uint32)
        words = words.reshape(d.n, L["gpad"] // 8).astype(np.int64)
        zp = np.array([[(words[nn, g // 8] >> (4 * (g % 8))) & 15 for g in range(G)]
                       for nn in range(d.n)])
    return codes, sc, zp


@pytest.mark.parametrize("wtype,n,k,g", [
    (qg.W_INT4, 40, 256, 128), (qg.W_UINT4, 33, 640, 64), (qg.W_INT3, 20, 384, 128),
    (qg.W_UINT3, 16, 256, 32), (qg.W_MXFP4, 24, 640, 32), (qg.W_INT8, 20, 384, 128),
    (qg.W_UINT8, 18, 256, 64), (qg.W_INT2, 33, 384, 32), (qg.W_UINT2, 16, 256, 128),
    (qg.W_INT1, 21, 256, 64), (qg.W_UINT1, 16, 384, 32), (qg.W_E0M3, 17, 256, 128),
    (qg.W_E0M7, 19, 256, 64), (qg.W_FP8, 20, 256, 32)])
def test_repack_roundtrip(wtype, n, k, g):
    r = synth.rng(42, wtype)
    d = qg.layer_desc(wtype, n, k, g)
    if wtype == qg.W_MXFP4:
        codes, sc, raw = synth.mx_weights(r, n, k)
        zp = None
    else:
        codes, sc, zp, raw = synth.int_weights(r, n, k, wtype, g)
    buf = np.zeros(qg.packed_size(d), np.uint8)
    qg.repack_host(d, codes, sc, zp, buf)
    got_c, got_s, got_z = _unpack_packed(d, buf)
    want = raw.astype(np.int64)
    if wtype in (qg.W_E0M3, qg.W_E0M7):
        # sign and magnitude, written out without the oracle: the packed code holds the value
        half = 1 << (synth.WTYPE_BITS[wtype] - 1)
        want = np.where(want < half, want, half - want)
    assert np.array_equal(got_c, want)
    assert np.array_equal(got_s, sc.astype(np.int64))
    if zp is not None:
        assert np.array_equal(got_z, zp.astype(np.int64))
    # padding beyond N is zero
    L = _layout(d)
    assert not buf[L["stride"]:].any()


def test_repack_roundtrip_w8a8():
    r = synth.rng(43, 1)
    n, k = 300, 384
    d = qg.layer_desc(qg.W_FP8, n, k, 128, atype=qg.A_FP8_BLOCK)
    codes, sc = synth.fp8_block_weights(r, n, k)
    buf = np.zeros(qg.packed_size(d), np.uint8)
    qg.repack_host(d, codes, sc, None, buf)
    got_c, got_s, _ = _unpack_packed(d, buf)
    assert np.array_equal(got_c, codes.astype(np.int64))
    L = _layout(d)
    for t in range(L["n_tiles"]):
        assert np.array_equal(got_s[t, :L["k_blocks"]], sc[16 * t // 128])
        assert not got_s[t, L["k_blocks"]:].any()


def test_repack_selected_experts_only():
    r = synth.rng(1, 1)
    d = qg.layer_desc(qg.W_INT4, 32, 256, 128, num_experts=3)
    codes, sc, zp, raw = synth.int_weights(r, 32, 256, qg.W_INT4, 128, experts=1)
    buf = np.zeros(qg.packed_size(d), np.uint8)
    qg.repack_host(d, codes, sc, None, buf, expert_begin=2, expert_count=1)
    stride = _layout(d)["stride"]
    assert not buf[:2 * stride].any() and buf[2 * stride:].any()
    with pytest.raises(qg.QGError) as e:
        qg.repack_host(d, codes, sc, None, buf, expert_begin=2, expert_count=2)
    assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT
    with pytest.raises(qg.QGError) as e:
        qg.repack_host(d, codes, sc, None, buf[:100])
    assert e.value.status == qg.QG_ERR_BUFFER_TOO_SMALL


FAKE_DEV = 1 << 40  # 256-aligned address that is never dereferenced


def _bound(desc):
    return qg.weight_bind(desc, FAKE_DEV, qg.packed_size(desc))


def test_gemm_argument_errors_before_launch():
    w = _bound(qg.layer_desc(qg.W_UINT4, 256, 512, 128))
    S = 0  # null stream: never used because validation fails first
    # m == 0 is a no-op
    qg.gemm(w, None, None, 0, 512, None, qg.O_BF16, 256, stream=S)
    cases = [
        (dict(x=None), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(otype=7), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(ldx=100), qg.QG_ERR_SHAPE),
        (dict(ldy=10), qg.QG_ERR_SHAPE),
        (dict(x=FAKE_DEV + 2), qg.QG_ERR_ALIGNMENT),
        (dict(ldx=516), qg.QG_ERR_ALIGNMENT),
        (dict(m=-1), qg.QG_ERR_INVALID_ARGUMENT),
    ]
    for kw, status in cases:
        a = dict(x=FAKE_DEV, m=4, ldx=512, y=FAKE_DEV, otype=qg.O_BF16, ldy=256)
        a.update(kw)
        with pytest.raises(qg.QGError) as e:
            qg.gemm(w, a["x"], None, a["m"], a["ldx"], a["y"], a["otype"], a["ldy"], stream=S)
        assert e.value.status == status, kw
    bad = qg.Weight.from_buffer_copy(w)
    bad.layout_version = 7
    with pytest.raises(qg.QGError) as e:
        qg.gemm(bad, FAKE_DEV, None, 4, 512, FAKE_DEV, qg.O_BF16, 256, stream=S)
    assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT
    mx = _bound(qg.layer_desc(qg.W_MXFP4, 256, 512, 32))
    with pytest.raises(qg.QGError) as e:  # MXFP8 activations need their scales
        qg.gemm(mx, FAKE_DEV, None, 4, 512, FAKE_DEV, qg.O_BF16, 256, stream=S)
    assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT


def test_moe_argument_errors_before_launch():
    w = _bound(qg.layer_desc(qg.W_INT4, 256, 512, 128, num_experts=8))
    S = 0
    qg.moe_gemm(w, FAKE_DEV, None, qg.ROWS_BY_TOKEN, FAKE_DEV, FAKE_DEV, 0, 2, FAKE_DEV,
                qg.O_BF16, qg.ROWS_BY_PAIR, stream=S)  # no tokens: no-op
    with pytest.raises(qg.QGError) as e:
        qg.moe_gemm(w, FAKE_DEV, None, qg.ROWS_BY_TOKEN, FAKE_DEV, FAKE_DEV, 4, 2, FAKE_DEV,
                    qg.O_BF16, qg.ROWS_BY_TOKEN, stream=S)  # y by token is not a mode
    assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT
    with pytest.raises(qg.QGError) as e:
        qg.moe_gemm(w, FAKE_DEV, None, qg.ROWS_BY_TOKEN, None, FAKE_DEV, 4, 2, FAKE_DEV,
                    qg.O_BF16, qg.ROWS_BY_PAIR, stream=S)
    assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT
    assert qg.moe_workspace_size(w, 64, 8) >= 9 * 4
    with pytest.raises(qg.QGError) as e:
        qg.moe_sort(FAKE_DEV, 4, 2, 8, FAKE_DEV, FAKE_DEV, FAKE_DEV, 8, stream=S)
    assert e.value.status == qg.QG_ERR_BUFFER_TOO_SMALL
    with pytest.raises(qg.QGError) as e:
        qg.moe_sort(FAKE_DEV, 4, 0, 8, FAKE_DEV, FAKE_DEV, FAKE_DEV, 256, stream=S)
    assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT


def test_dispatch_table_covers_k():
    for wt, n, k, g in [(qg.W_UINT4, 14336, 4096, 128), (qg.W_UINT4, 4096, 14336, 128),
                        (qg.W_INT3, 4096, 14336, 128), (qg.W_INT4, 256, 512, 128),
                        (qg.W_INT4, 4096, 14336, 32), (qg.W_MXFP4, 3072, 4096, 32),
                        (qg.W_MXFP4, 4096, 640, 32)]:
        w = _bound(qg.layer_desc(wt, n, k, g))
        for m in (1, 4, 16, 64, 4096):
            s = qg.describe_dispatch(w, m)
            if "tiled" in s:  # LDS-tiled large-M paths: loop over all of K
                assert m >= 128 and k % 128 == 0, s
                assert ("mx_" in s) == (wt == qg.W_MXFP4), s
                if wt != qg.W_MXFP4:  # the group row sums of X live behind the counter prefix
                    assert qg.gemm_workspace_size(w, m) >= 65536 + (k // g) * m * 4
                continue
            if "decode_wide" in s:  # K slices of KR blocks, W column tiles per workgroup
                assert wt != qg.W_MXFP4 and 2 <= m <= 16 and k % 512 == 0, s
                KR, W, S = (int(v) for v in re.findall(r"=(\d+)", s))
                kb = -(-k // 128)
                assert S == -(-kb // KR) and 1 <= W <= 16, s
                if S > 1:  # arrival counters (prefix) and partials live in the workspace
                    assert qg.gemm_workspace_size(w, m) >= 65536 + S * -(-n // (16 * W)) * W * 256 * 4
                continue
            if "decode" in s:  # activations in LDS, one workgroup over all of K (or of a split)
                assert wt != qg.W_MXFP4 and m <= 16 and k % 512 == 0, s
                vals = [int(v) for v in re.findall(r"=(\d+)", s)]
                T, KR, W = vals[:3]
                S = vals[3] if len(vals) > 3 else 1
                assert W * KR * S >= -(-k // 128) and 1 <= W <= 16, s
                if S > 1:  # arrival counters (prefix) and partials live in the workspace
                    assert (S - 1) * W * KR < -(-k // 128) and (W * KR) % 4 == 0, s
                    assert qg.gemm_workspace_size(w, m) >= 65536 + S * -(-n // (16 * T)) * T * 256 * 4
                continue
            # skinny: the waves of all splits cover K in P passes, none empty
            vals = [int(v) for v in re.findall(r"=(\d+)", s)]
            T, KR, W, S = vals[:4]
            P = vals[4] if len(vals) > 4 else 1
            span, kb = W * KR * S, -(-k // 128)
            assert span * P >= kb and span * (P - 1) < kb, s
            assert 1 <= W <= 16
    # a split-K layout (long K over too few column tiles to fill the CUs)
    # asks for a workspace
    w = _bound(qg.layer_desc(qg.W_INT4, 1024, 14336, 32))
    assert "splits=2" in qg.describe_dispatch(w, 1)
    assert qg.gemm_workspace_size(w, 1) > 0
    assert "splits" not in qg.describe_dispatch(_bound(qg.layer_desc(qg.W_UINT4, 4096, 14336, 128)), 1)
    assert qg.gemm_workspace_size(_bound(qg.layer_desc(qg.W_UINT4, 14336, 4096, 128)), 1) == 0


def test_decode_four_tiles_when_rows_fill_lds():
    """Rows that fill more than half of a CU's LDS leave one two-tile decode
    workgroup per CU: where that needs more rounds of resident workgroups than
    four tiles per workgroup, the four-tile instance runs (14336 x 4096 from
    10 rows; 28672 x 4096, whose two-tile form exceeds one round already at 4
    rows); one row keeps one tile per workgroup."""
    def t_of(n, k, m):
        s = qg.describe_dispatch(_bound(qg.layer_desc(qg.W_UINT4, n, k, 128)), m)
        assert s.startswith("a16_decode T="), s
        return int(re.search(r"T=(\d+)", s).group(1)), int(re.search(r"KR=(\d+)", s).group(1))
    assert t_of(14336, 4096, 1) == (1, 8)
    for m in (2, 4, 8, 9):
        assert t_of(14336, 4096, m) == (2, 4), m
    for m in (10, 12, 16):
        assert t_of(14336, 4096, m) == (4, 4), m
    for m in (4, 8, 16):
        assert t_of(28672, 4096, m) == (4, 4), m


def test_decode_int3_one_row_two_tiles():
    """INT3 at one row: two n-tiles of 8 blocks per wave while that leaves 200
    to 512 workgroups, one n-tile otherwise; other formats one n-tile."""
    def t_kr(wt, n, k):
        s = qg.describe_dispatch(_bound(qg.layer_desc(wt, n, k, 128)), 1)
        return tuple(int(v) for v in re.findall(r"(?:T|KR)=(\d+)", s))
    assert t_kr(qg.W_INT3, 14336, 4096) == (2, 8)
    assert t_kr(qg.W_INT3, 8192, 8192) == (2, 8)
    assert t_kr(qg.W_INT3, 28672, 4096) == (1, 8)
    assert t_kr(qg.W_INT3, 4096, 14336) == (1, 8)
    for wt in (qg.W_UINT3, qg.W_INT4, qg.W_UINT4):
        assert t_kr(wt, 14336, 4096) == (1, 8), wt


def test_binding_maps_a_single_hip_runtime():
    """libqg must share the caller's (torch's) HIP runtime: one libamdhip64 mapped."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import quantized_gemm_qg_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "1"


def test_moe_dispatch_covers_configured_shapes():
    """The grouped kernel keeps K in one workgroup: every configured expert
    shape (gate_up and down of both MoE configurations) is covered by up to
    4 waves of 2 blocks looping over K: four n-tiles per wave for the
    integer formats, two for MXFP8 activations (four on 2 waves over K <=
    1024 from 64 pairs)."""
    for wt, n, k, g, e in [(qg.W_INT4, 4096, 7168, 128, 256), (qg.W_INT4, 7168, 2048, 128, 256),
                           (qg.W_MXFP4, 1280, 4096, 32, 128), (qg.W_MXFP4, 4096, 640, 32, 128)]:
        w = _bound(qg.layer_desc(wt, n, k, g, num_experts=e))
        for pairs in (8, 512, 4096, 32768):
            s = qg.describe_dispatch(w, pairs)
            vals = [int(v) for v in re.findall(r"=(\d+)", s)]
            T, KR, W, S = vals[:4]
            P = vals[4] if len(vals) > 4 else 1
            kb = -(-k // 128)
            assert S == 1 and W * KR * P >= kb and W * KR * (P - 1) < kb and W <= 16, s
            if wt == qg.W_INT4:
                assert (T, KR, W) == (4, 2, 4), s
            elif kb <= 8 and pairs >= 64:  # MX down projection (K = 640)
                assert (T, KR, W) == (4, 2, 2), s
            else:
                assert (T, KR, W) == (2, 2, min(4, -(-kb // 2))), s


def test_library_has_no_undefined_internal_symbols():
    """Every kernel and launcher of the library is defined in libqg.so itself
    (an uninstantiated kernel template would leave an undefined qg:: symbol)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", qg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert not [l for l in out.splitlines() if "_ZN2qg" in l], out


def test_activation_entry_points_validate_before_launch():
    S = 0
    # no-ops
    qg.quantize_mxfp8(None, 0, 64, 64, None, 64, None, stream=S)
    qg.silu_mul(None, qg.O_BF16, 0, 64, 128, None, qg.A_BF16, 64, stream=S)
    qg.moe_combine(None, qg.O_BF16, 64, None, 0, 2, 64, None, None, qg.O_BF16, 64, stream=S)
    F = FAKE_DEV
    q_cases = [
        (dict(k=48), qg.QG_ERR_SHAPE),                  # K % 32
        (dict(ldx=32), qg.QG_ERR_SHAPE),                # ldx < K
        (dict(ldq=32), qg.QG_ERR_SHAPE),
        (dict(x=None), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(qs=None), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(x=F + 8), qg.QG_ERR_ALIGNMENT),
        (dict(ldx=68), qg.QG_ERR_ALIGNMENT),
        (dict(q=F + 4), qg.QG_ERR_ALIGNMENT),
        (dict(rows=-1), qg.QG_ERR_INVALID_ARGUMENT),
    ]
    for kw, status in q_cases:
        a = dict(x=F, rows=4, k=64, ldx=64, q=F, ldq=64, qs=F)
        a.update(kw)
        with pytest.raises(qg.QGError) as e:
            qg.quantize_mxfp8(a["x"], a["rows"], a["k"], a["ldx"], a["q"], a["ldq"], a["qs"], stream=S)
        assert e.value.status == status, kw
    s_cases = [
        (dict(inter=36), qg.QG_ERR_SHAPE),               # bf16 output needs inter % 8
        (dict(inter=40, ht=qg.A_MXFP8), qg.QG_ERR_SHAPE),  # MXFP8 output needs inter % 32
        (dict(ldgu=100), qg.QG_ERR_SHAPE),               # ldgu < 2 inter
        (dict(gt=5), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(ht=qg.A_MXFP8), qg.QG_ERR_INVALID_ARGUMENT),  # scales missing
        (dict(gu=F + 4), qg.QG_ERR_ALIGNMENT),
        (dict(h=F + 8), qg.QG_ERR_ALIGNMENT),
    ]
    for kw, status in s_cases:
        a = dict(gu=F, gt=qg.O_BF16, rows=4, inter=64, ldgu=128, h=F, ht=qg.A_BF16, ldh=64, hs=None)
        a.update(kw)
        with pytest.raises(qg.QGError) as e:
            qg.silu_mul(a["gu"], a["gt"], a["rows"], a["inter"], a["ldgu"], a["h"], a["ht"], a["ldh"], a["hs"],
                        stream=S)
        assert e.value.status == status, kw
    c_cases = [
        (dict(n=60), qg.QG_ERR_SHAPE),
        (dict(topk=0), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(w=None), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(yt=3), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(bias=F + 2), qg.QG_ERR_ALIGNMENT),
        (dict(out=F + 8), qg.QG_ERR_ALIGNMENT),
        (dict(ldout=32), qg.QG_ERR_SHAPE),
    ]
    for kw, status in c_cases:
        a = dict(y=F, yt=qg.O_BF16, ldy=64, w=F, t=4, topk=2, n=64, bias=None, out=F, ot=qg.O_BF16, ldout=64)
        a.update(kw)
        with pytest.raises(qg.QGError) as e:
            qg.moe_combine(a["y"], a["yt"], a["ldy"], a["w"], a["t"], a["topk"], a["n"], a["bias"], a["out"],
                           a["ot"], a["ldout"], stream=S)
        assert e.value.status == status, kw


def test_gemm_ex_flags_validated():
    w = _bound(qg.layer_desc(qg.W_INT4, 256, 512, 128))
    for bad in (2, 0x80000000):
        with pytest.raises(qg.QGError) as e:
            qg.gemm_workspace_size_ex(w, 4, bad)
        assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT
        with pytest.raises(qg.QGError) as e:
            qg.gemm_ex(w, FAKE_DEV, None, 4, 512, FAKE_DEV, qg.O_BF16, 256, None, 0, bad, stream=0)
        assert e.value.status == qg.QG_ERR_INVALID_ARGUMENT
    # the invariant option sizes the large-M kernel's workspace at any M
    assert qg.gemm_workspace_size_ex(w, 1, qg.GEMM_BATCH_INVARIANT) > 0
    assert qg.gemm_workspace_size_ex(w, 1, 0) == qg.gemm_workspace_size(w, 1)


def test_autotune_validates_before_launch():
    w = _bound(qg.layer_desc(qg.W_UINT4, 256, 512, 128))
    need = qg.gemm_autotune_workspace_size(w, 4)
    assert need >= 16384
    cases = [
        (dict(reps=0), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(reps=65), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(m=0), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(x=None), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(ws=None), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(ws_bytes=100), qg.QG_ERR_BUFFER_TOO_SMALL),
        (dict(ws=FAKE_DEV + 16), qg.QG_ERR_ALIGNMENT),
        (dict(flush=FAKE_DEV + 4, flush_bytes=1 << 20), qg.QG_ERR_ALIGNMENT),
        (dict(ldx=100), qg.QG_ERR_SHAPE),
    ]
    for kw, status in cases:
        a = dict(x=FAKE_DEV, m=4, ldx=512, y=FAKE_DEV, ws=FAKE_DEV, ws_bytes=need, flush=None, flush_bytes=0, reps=3)
        a.update(kw)
        with pytest.raises(qg.QGError) as e:
            qg.gemm_autotune(w, a["x"], None, a["m"], a["ldx"], a["y"], qg.O_BF16, 256, a["ws"], a["ws_bytes"],
                             a["flush"], a["flush_bytes"], a["reps"], stream=0)
        assert e.value.status == status, kw
    qg.autotune_reset()


def test_repack_fp4_bf16_layout():
    """MXFP4 weights for bf16 activations: e2m1 codes in the 4-bit integer
    lane order with standard nibble order, e8m0 scales stored as bf16 powers
    of two (read back here by an independent decoder of that layout)."""
    n, k = 40, 384
    desc = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=qg.A_BF16)
    codes_std, sc, raw = synth.mx_weights(synth.rng(3, 1), n, k)
    sc = sc.copy()
    sc[0, 0], sc[1, 1] = 0, 255  # the subnormal and NaN codes
    dst = np.zeros(qg.packed_size(desc), np.uint8)
    qg.repack_host(desc, codes_std, sc, None, dst)
    w = _bound(desc)
    kbs, gp = w.k_blocks, w.groups_padded
    for nn in range(n):
        t, ln = divmod(nn, 16)
        for kk in range(k):
            kb, r = divmod(kk, 128)
            j, q, e = r // 32, (r % 32) // 8, kk % 8
            lane = ln + 16 * q
            off = (t * kbs + kb) * 1024 + lane * 16 + 4 * j
            dword = int.from_bytes(dst[off:off + 4].tobytes(), "little")
            assert (dword >> (4 * e)) & 15 == raw[nn, kk], (nn, kk)
    s16 = dst[w.scales_offset:w.scales_offset + w.n_tiles * 16 * gp * 2].view(np.uint16).reshape(-1, gp)
    for nn in range(n):
        for g in range(k // 32):
            c = int(sc[nn, g])
            expect = 0x0040 if c == 0 else 0x7FC0 if c == 255 else c << 7
            assert s16[nn, g] == expect, (nn, g)


def test_w4a4_host_logic():
    d = qg.layer_desc(qg.W_MXFP4, 256, 512, 32, atype=qg.A_MXFP4)
    # the weight layout is the W4A8 one
    assert qg.packed_size(d) == qg.packed_size(qg.layer_desc(qg.W_MXFP4, 256, 512, 32))
    w = _bound(d)
    # from 128 rows the MX tiled kernel (its scales scratch in the
    # workspace); below, the MX skinny kernel (e2m1 fragments widened to e4m3
    # in registers), with the W4A8 layer's workspace
    w8 = _bound(qg.layer_desc(qg.W_MXFP4, 256, 512, 32))
    for m in (1, 7, 127):
        assert qg.describe_dispatch(w, m).startswith("mx_skinny"), m
        assert qg.describe_dispatch(w, m) == qg.describe_dispatch(w8, m)
        assert qg.gemm_workspace_size(w, m) == qg.gemm_workspace_size(w8, m)
    for m in (128, 130, 4096):
        assert qg.describe_dispatch(w, m).startswith("mx_tiled"), m
        assert qg.gemm_workspace_size(w, m) > 0
    # the batch-invariant option keeps the tiled kernel at every M (its
    # scales scratch covers rows padded to 256 either way)
    assert qg.gemm_workspace_size_ex(w, 1, qg.GEMM_BATCH_INVARIANT) == qg.gemm_workspace_size(w, 256)
    F, S = FAKE_DEV, 0
    cases = [
        (dict(ldx=513), qg.QG_ERR_ALIGNMENT),      # odd: half a byte per row
        (dict(ldx=528), qg.QG_ERR_ALIGNMENT),      # 264-byte rows
        (dict(ldx=500), qg.QG_ERR_SHAPE),
        (dict(xs=None), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(m=1 << 24, ldx=512), qg.QG_ERR_UNSUPPORTED),  # 4 GiB of e2m1 rows
    ]
    for kw, status in cases:
        a = dict(m=4, ldx=512, xs=F)
        a.update(kw)
        with pytest.raises(qg.QGError) as e:
            qg.gemm(w, F, a["xs"], a["m"], a["ldx"], F, qg.O_BF16, 256, F, 1 << 40, stream=S)
        assert e.value.status == status, kw
    # MXFP8 rows spanning 4 GiB are refused too (32-bit activation offsets)
    w8k = _bound(qg.layer_desc(qg.W_MXFP4, 256, 1024, 32))
    with pytest.raises(qg.QGError) as e:
        qg.gemm(w8k, F, F, 1 << 22, 1024, F, qg.O_BF16, 256, F, 1 << 40, stream=S)
    assert e.value.status == qg.QG_ERR_UNSUPPORTED
    # W4A4 MoE: W4A8's kernel choices and workspace, on e2m1 rows
    dm4 = qg.layer_desc(qg.W_MXFP4, 256, 512, 32, atype=qg.A_MXFP4, num_experts=8)
    dm8 = qg.layer_desc(qg.W_MXFP4, 256, 512, 32, num_experts=8)
    assert qg.packed_size(dm4) == qg.packed_size(dm8)
    for t, topk in ((1, 1), (16, 2), (300, 8)):
        assert qg.moe_workspace_size(_bound(dm4), t, topk) == qg.moe_workspace_size(_bound(dm8), t, topk)
    # quantizer validation
    qg.quantize_mxfp4(None, 0, 64, 64, None, 64, None, stream=S)
    q_cases = [
        (dict(k=48), qg.QG_ERR_SHAPE),
        (dict(ldq=32), qg.QG_ERR_SHAPE),
        (dict(qs=None), qg.QG_ERR_INVALID_ARGUMENT),
        (dict(q=F + 2), qg.QG_ERR_ALIGNMENT),
        (dict(ldq=68), qg.QG_ERR_ALIGNMENT),
        (dict(x=F + 8), qg.QG_ERR_ALIGNMENT),
    ]
    for kw, status in q_cases:
        a = dict(x=F, rows=4, k=64, ldx=64, q=F, ldq=64, qs=F)
        a.update(kw)
        with pytest.raises(qg.QGError) as e:
            qg.quantize_mxfp4(a["x"], a["rows"], a["k"], a["ldx"], a["q"], a["ldq"], a["qs"], stream=S)
        assert e.value.status == status, kw


def test_long_k_dispatch_loops_inside_the_workgroup():
    """K past one pass of a workgroup's waves (MoE: 16 waves x 4 blocks = 8192)
    is served by looping over K, never rejected: the MoE dispatch at K = 14336
    and a dense layer whose split-K counters would not fit the workspace's
    counter prefix."""
    for wt, g in ((qg.W_INT4, 128), (qg.W_MXFP4, 32)):
        w = _bound(qg.layer_desc(wt, 256, 14336, g, num_experts=32))
        for pairs in (8, 16, 200):
            s = qg.describe_dispatch(w, pairs)
            T, KR, W, S, P = (int(v) for v in re.findall(r"=(\d+)", s))
            assert S == 1 and W <= 16 and W * KR * P >= 112 and W * KR * (P - 1) < 112, s
        assert qg.moe_workspace_size(w, 4096, 8) > 0
    # K % 128 != 0 (no large-M kernel), long K, many rows: no cross-workgroup
    # split (its counters would exceed the 64 KiB prefix), the workgroups loop
    w = _bound(qg.layer_desc(qg.W_INT4, 14336, 14336 + 32, 32))
    s = qg.describe_dispatch(w, 4096)
    assert "splits=1 passes=" in s, s
    assert qg.gemm_workspace_size(w, 4096) == 0
    # and at 16 rows the split is kept (16 x 896 / T counters fit)
    assert "splits=1" not in qg.describe_dispatch(w, 16)


def test_overrides_through_the_library():
    """Experiment overrides are set through qg_set_override (the environment is
    read once per process), and clearing them restores the heuristics."""
    w = _bound(qg.layer_desc(qg.W_UINT4, 4096, 14336, 128))
    base = qg.describe_dispatch(w, 1)
    assert base.startswith("a16_decode")
    try:
        qg.set_override("QG_DECODE", "0")
        assert qg.describe_dispatch(w, 1).startswith("a16_skinny")
        qg.set_override("QG_DECODE", "2,8")
        assert qg.describe_dispatch(w, 1).startswith("a16_decode T=2 KR=8")
        qg.set_override("QG_DECODE", None)
        assert qg.describe_dispatch(w, 1) == base
        qg.set_override("QG_TUNE", "1,2,8,2")
        assert qg.describe_dispatch(w, 4) == "a16_skinny T=1 KR=2 W=8 splits=2 passes=4"
        with pytest.raises(qg.QGError):
            qg.set_override("QG_NOT_A_KNOB", "1")
    finally:
        qg.clear_overrides()
    assert qg.describe_dispatch(w, 1) == base



def test_noalloc_validates_before_any_device_call():
    """qg_gemm_noalloc: m == 0 is a no-op, and a call whose kernels would need
    more scratch than the static array holds is refused before any device
    call (host logic only)."""
    w = _bound(qg.layer_desc(qg.W_INT4, 1024, 14336, 128))
    qg.gemm_noalloc(w, None, None, 0, 14336, None, qg.O_BF16, 1024, stream=0)
    assert qg.gemm_workspace_size(w, 32768) > qg.NOALLOC_SCRATCH_BYTES
    with pytest.raises(qg.QGError) as e:
        qg.gemm_noalloc(w, FAKE_DEV, None, 32768, 14336, FAKE_DEV, qg.O_BF16, 1024, stream=0)
    assert e.value.status == qg.QG_ERR_BUFFER_TOO_SMALL


def test_skinny_two_passes_from_two_row_tiles():
    """Dense launches over K >= 4096 with two or more 16-row tiles (W8A8 from
    9 rows): every wave walks its K range in two passes, the waves per
    workgroup capped by the rows; one pass at one tile, and for the grouped
    (MoE) and batch-invariant launches."""
    def parse(wt, n, k, g, m, atype=None):
        s = qg.describe_dispatch(_bound(qg.layer_desc(wt, n, k, g, atype=atype)), m)
        vals = [int(v) for v in re.findall(r"=(\d+)", s)]
        return s, vals
    for wt, g, atype, lo, caps in [
            (qg.W_INT4, 128, None, 17, {24: 8, 64: 8, 128: 4}),
            (qg.W_MXFP4, 32, None, 17, {24: 16, 64: 8, 200: 4}),
            (qg.W_MXFP4, 32, qg.A_FP8_TOKEN, 17, {32: 16, 48: 8, 128: 4}),
            (qg.W_FP8, 128, qg.A_FP8_BLOCK, 9, {9: 8, 16: 8, 32: 16})]:
        for m, cap in caps.items():
            s, v = parse(wt, 4096, 14336, g, m, atype)
            assert "skinny" in s and s.endswith("passes=2"), (wt, m, s)
            T, KR, W, S, P = v
            per = -(-(-(-112 // KR)) // 2)  # half of the waves along K (K blocks of 128)
            assert W <= cap and W * S >= per and W * (S - 1) < per, (wt, m, s)
        if wt in (qg.W_INT4,):  # (W8A8 and MX take two passes at few rows too)
            s, _ = parse(wt, 4096, 14336, g, lo - 1, atype)
            assert "passes" not in s, (wt, s)
    # few-row rules: one row of MX activations, (2, 2) in two passes of <= 8
    # waves; beyond 16384 columns four tiles from one row; elsewhere one pass
    assert parse(qg.W_MXFP4, 14336, 4096, 32, 1, qg.A_FP8_TOKEN)[0] == \
        "mx_skinny T=2 KR=2 W=8 splits=1 passes=2"
    assert parse(qg.W_MXFP4, 4096, 14336, 32, 1)[0] == "mx_skinny T=2 KR=2 W=7 splits=4 passes=2"
    assert parse(qg.W_MXFP4, 28672, 4096, 32, 4)[0] == "mx_skinny T=4 KR=2 W=8 splits=1 passes=2"
    assert parse(qg.W_MXFP4, 14336, 4096, 32, 4)[0] == "mx_skinny T=4 KR=2 W=16 splits=1"
    assert "passes" not in parse(qg.W_MXFP4, 4096, 14336, 32, 16)[0]
    assert "passes" not in parse(qg.W_MXFP4, 4096, 2048, 32, 1)[0]
    assert parse(qg.W_MXFP4, 8192, 8192, 32, 1)[0] == "mx_skinny T=2 KR=4 W=16 splits=1"
    # UINT4 (zero points) up to 32 rows: two n-tiles per wave, then four
    assert parse(qg.W_UINT4, 14336, 4096, 128, 24)[0] == "a16_skinny T=2 KR=2 W=8 splits=1 passes=2"
    assert parse(qg.W_UINT4, 14336, 4096, 128, 33)[0].startswith("a16_skinny T=4")
    assert parse(qg.W_INT4, 14336, 4096, 128, 24)[0].startswith("a16_skinny T=4")
    # K below 4096: one pass
    assert "passes" not in parse(qg.W_INT4, 4096, 2048, 128, 64)[0]
    # 1-, 2-, 8-bit integers keep one pass
    assert "passes" not in parse(qg.W_UINT8, 4096, 14336, 128, 64)[0]


def test_tiled_needs_enough_column_tiles_below_256_rows():
    """Integer formats take the tiled kernel from 128 rows (128 x 128 tiles)
    where N gives 96 or more 128-column tiles; MX (not W8A8) below 256 rows
    over K >= 4096 needs 32 or more column tiles."""
    def d(wt, n, k, g, m, atype=None):
        return qg.describe_dispatch(_bound(qg.layer_desc(wt, n, k, g, atype=atype)), m)
    assert d(qg.W_INT4, 14336, 4096, 128, 128) == "a16_tiled BM=128 BN=128"
    assert "skinny" in d(qg.W_INT4, 8192, 8192, 128, 128)
    assert d(qg.W_INT4, 8192, 8192, 128, 192) == "a16_tiled BM=128 BN=128"
    assert "skinny" in d(qg.W_INT4, 4096, 14336, 128, 255)
    assert "skinny" in d(qg.W_INT4, 14336, 4096, 128, 127)
    assert "tiled" in d(qg.W_INT4, 8192, 8192, 128, 256)
    assert "skinny" in d(qg.W_MXFP4, 4096, 14336, 32, 128)
    assert "skinny" in d(qg.W_MXFP4, 4096, 14336, 32, 255)
    assert "tiled" in d(qg.W_MXFP4, 4096, 14336, 32, 256)
    assert "tiled" in d(qg.W_MXFP4, 8192, 8192, 32, 128)
    assert "tiled" in d(qg.W_MXFP4, 136, 896, 32, 130)
    assert "tiled" in d(qg.W_FP8, 4096, 14336, 128, 128, qg.A_FP8_BLOCK)


def test_decode_wide_slices_by_k():
    """Rows too long for LDS over all of K take the wide decode in K slices
    of 16 blocks, or of 8 where K has at most 64 blocks (4 slices of 16 would
    leave one workgroup per CU)."""
    def d(n, k, m):
        return qg.describe_dispatch(_bound(qg.layer_desc(qg.W_INT4, n, k, 128)), m)
    assert d(4096, 14336, 16) == "a16_decode_wide KR=16 W=8 splits=7"
    assert d(8192, 8192, 16) == "a16_decode_wide KR=8 W=8 splits=8"
    assert d(4096, 8192, 12) == "a16_decode_wide KR=8 W=8 splits=8"
    assert d(14336, 4096, 16).startswith("a16_decode T=")


def test_tiled_shape_by_rounds_and_area():
    """The larger tile (256 rows; integer formats 128 x 256) from 256 rows
    only where its rounds of 256 CUs times its area do not exceed the
    128-row tile's (taken 15 % dearer for MX and W8A8, 40 % for the integer
    formats); explicit tile overrides keep 256-row tiles from 256 rows."""
    def d(wt, n, k, g, m, atype=None):
        return qg.describe_dispatch(_bound(qg.layer_desc(wt, n, k, g, atype=atype)), m)
    tok, f8 = qg.A_FP8_TOKEN, qg.A_FP8_BLOCK
    # few tiles: 128-row tiles double the workgroups
    assert d(qg.W_MXFP4, 4096, 14336, 32, 512, tok) == "mx_tiled BM=128 BN=192"
    assert d(qg.W_FP8, 8192, 8192, 128, 512, f8) == "f8_tiled BM=128 BN=128"
    assert d(qg.W_INT4, 8192, 8192, 128, 512) == "a16_tiled BM=128 BN=128"
    assert d(qg.W_MXFP4, 4096, 14336, 32, 512, qg.A_MXFP4) == "mx_tiled BM=128 BN=192"
    # many tiles (M = 4096): the larger tile
    assert d(qg.W_MXFP4, 14336, 4096, 32, 4096, tok) == "mx_tiled BM=256 BN=224"
    assert d(qg.W_MXFP4, 3072, 4096, 32, 4096) == "mx_tiled BM=256 BN=192"
    assert d(qg.W_FP8, 14336, 4096, 128, 4096, f8) == "f8_tiled BM=256 BN=128"
    assert d(qg.W_INT4, 3072, 4096, 128, 4096) == "a16_tiled BM=128 BN=256"
    assert d(qg.W_INT4, 14336, 4096, 128, 4096) == "a16_tiled BM=128 BN=256"
    # (W8A8 3072 x 4096: three rounds of 128-row tiles beat two of 256)
    assert d(qg.W_FP8, 3072, 4096, 128, 4096, f8) == "f8_tiled BM=128 BN=128"
    # integer formats from 256 to 383 rows over K >= 4096 and few columns:
    # the skinny kernel's two passes; over K < 4096 the tiled kernel
    assert "skinny" in d(qg.W_INT4, 3072, 4096, 128, 256)
    assert "skinny" in d(qg.W_INT4, 4096, 14336, 128, 383)
    assert "tiled" in d(qg.W_INT4, 4096, 14336, 128, 384)
    assert "tiled" in d(qg.W_INT4, 200, 640, 128, 300)
    try:
        qg.set_override("QG_MX_BN", "256")
        assert d(qg.W_MXFP4, 128, 1024, 32, 256) == "mx_tiled BM=256 BN=256"
        qg.set_override("QG_MX_BN", None)
        qg.set_override("QG_A16_BN", "256")
        assert d(qg.W_UINT4, 128, 1024, 128, 256) == "a16_tiled BM=128 BN=256"
    finally:
        qg.set_override("QG_MX_BN", None)
        qg.set_override("QG_A16_BN", None)


def test_w8a8_few_rows_long_k_splits():
    """W8A8 up to 8 rows over K of 16 or more waves of 4 blocks: two K
    passes where N gives 128 column blocks, else beyond 16 waves 4 waves per
    split, at most 8 splits; K below 16 waves keeps one workgroup."""
    def d(n, k, m):
        return qg.describe_dispatch(_bound(qg.layer_desc(qg.W_FP8, n, k, 128, atype=qg.A_FP8_BLOCK)), m)
    for m in (1, 4, 8):
        assert d(4096, 14336, m) == "f8_skinny T=1 KR=4 W=7 splits=2 passes=2"
        assert d(1024, 28672, m) == "f8_skinny T=1 KR=4 W=7 splits=8"
        assert d(8192, 8192, m) == "f8_skinny T=1 KR=4 W=8 splits=1 passes=2"
        # (K of 4096 to 8191: 2 blocks in two passes of 8 waves)
        assert d(14336, 4096, m) == "f8_skinny T=1 KR=2 W=8 splits=1 passes=2"
        assert d(4096, 2048, m) == "f8_skinny T=1 KR=4 W=4 splits=1"


def test_moe_integer_formats_below_256_pairs_all_skinny():
    """4- and 3-bit integer and MXFP8-activation MoE layers below 256 pairs
    put every expert on the skinny kernel's 4-wave launch (a hot expert's
    64+ rows included); from 256 pairs the tiled and small-tile split."""
    w = _bound(qg.layer_desc(qg.W_INT4, 4096, 7168, 128, num_experts=256))
    for t in (1, 16, 31):
        assert qg.describe_moe_dispatch(w, t, 8).endswith("for every expert"), t
    assert "a16_tiled BM=128" in qg.describe_moe_dispatch(w, 32, 8)
    mx = _bound(qg.layer_desc(qg.W_MXFP4, 1280, 4096, 32, num_experts=128))
    assert qg.describe_moe_dispatch(mx, 16, 8).endswith("for every expert")
    assert "mx_tiled BM=128" in qg.describe_moe_dispatch(mx, 32, 8)
    try:  # an explicit threshold still applies
        qg.set_override("QG_MOE_TILED_MIN", "64")
        assert "a16_tiled BM=128" in qg.describe_moe_dispatch(w, 16, 8)
    finally:
        qg.set_override("QG_MOE_TILED_MIN", None)


def test_moe_w8a8_long_k_four_waves():
    """W8A8 grouped skinny launches over K > 1024 loop over K on 4 waves:
    (1, 4) below 64 pairs, (2, 2) from 64; K <= 1024 keeps the dense rule."""
    up = _bound(qg.layer_desc(qg.W_FP8, 1280, 4096, 128, atype=qg.A_FP8_BLOCK, num_experts=128))
    assert qg.describe_dispatch(up, 8) == "f8_skinny T=1 KR=4 W=4 splits=1 passes=2"
    assert qg.describe_dispatch(up, 128) == "f8_skinny T=2 KR=2 W=4 splits=1 passes=4"
    down = _bound(qg.layer_desc(qg.W_FP8, 4096, 640, 128, atype=qg.A_FP8_BLOCK, num_experts=128))
    assert qg.describe_dispatch(down, 128) == "f8_skinny T=2 KR=2 W=3 splits=1"


def test_moe_fp4_bf16_four_tiles_four_waves():
    """MXFP4 x bf16 grouped skinny launches take the integer formats' form:
    four n-tiles of 2 blocks on 4 waves, looping over K."""
    w = _bound(qg.layer_desc(qg.W_MXFP4, 4096, 7168, 32, atype=qg.A_BF16, num_experts=256))
    for pairs in (8, 128):
        assert qg.describe_dispatch(w, pairs) == "a16_skinny T=4 KR=2 W=4 splits=1 passes=7"
