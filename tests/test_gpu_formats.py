"""GPU parity of the further weight and activation formats through the C ABI:
1-, 2- and 8-bit integer weights, e0m3 / e0m7 and e4m3 weights with bf16
activations (the announcement's "WnA16" and "Quantization support"
sections), MXFP4 weights with per-token FP8 activations (section "End to
end"), W8A8 FP8 with block scales (section "W8A8 / W4A8 / W4A4") and the
FP8 activation quantizer, each against the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import mx_mfma_model as MM
import oracle
import quantized_gemm_qg_amd as qg
import synth
from gpu_harness import (TOL_BF16, TOL_F32, Acts, Layer, assert_bf16_is_rne, check_mx_f32, err, moe_mx_forms, mx_codes,
                         require_gpu, run_gemm, to_dev)
from oracle import quantize as Q

pytestmark = pytest.mark.gpu

A16_EXT = [qg.W_INT8, qg.W_UINT8, qg.W_INT2, qg.W_UINT2, qg.W_INT1, qg.W_UINT1, qg.W_E0M3, qg.W_E0M7, qg.W_FP8]
# (N, K, group, M values): decode-kernel shapes (K % 512 == 0), a ragged N with
# group 64, group 32 with a K that is not a multiple of 512
SHAPES = [(256, 1024, 128, (1, 3, 16)), (200, 640, 64, (1, 37)), (96, 384, 32, (5, 300))]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check_a16(layer, m, seed):
    acts = Acts(False, m, layer.k, seed=seed)
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {}
    for otype, tol in ((qg.O_BF16, TOL_BF16), (qg.O_F32, TOL_F32)):
        y = ys[otype] = run_gemm(layer, acts, m, otype)
        e = err(y, yref)
        print(f"  M={m} otype={otype} err={e:.3e} ({qg.describe_dispatch(layer.w, m)})", flush=True)
        assert torch.isfinite(y.float()).all()
        assert e <= tol, (otype, e)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"N{s[0]}_K{s[1]}_g{s[2]}")
@pytest.mark.parametrize("wtype", A16_EXT)
def test_wna16_formats_dense(wtype, shape):
    n, k, g, ms = shape
    print(f"wtype={wtype} N={n} K={k} g={g}", flush=True)
    layer = Layer(wtype, n, k, g, seed=50 + wtype)
    for m in ms:
        _check_a16(layer, m, seed=60 + m)


@pytest.mark.parametrize("m", [8, 20])
@pytest.mark.parametrize("wtype", A16_EXT)
def test_wna16_identity_rows_are_exact(wtype, m):
    """X rows = unit vectors at group edges: each fp32 output row is a column
    of the dequantized weight, exactly ((q - z) * s is exact in fp32)."""
    n, k, g = 64, 1024, 64
    layer = Layer(wtype, n, k, g, seed=70 + wtype)
    cols = [(37 * i + 63 * (i % 2)) % k for i in range(m)]
    bits = np.zeros((m, k), np.uint16)
    for i, c in enumerate(cols):
        bits[i, c] = 0x3F80
    acts = Acts(False, m, k, values=bits)
    y = run_gemm(layer, acts, m, qg.O_F32).cpu().numpy().astype(np.float64)
    wdq = layer.wdq()
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], wdq[:, c]), (i, c, qg.describe_dispatch(layer.w, m))


def test_wna16_dispatch():
    """Decode kernel at M = 1 when K % 512 == 0; the skinny kernel at large M
    (no tiled kernel for these formats) except e0m3, which is stored as INT4
    and takes the integer tiled kernel."""
    for wtype in A16_EXT:
        layer = Layer(wtype, 128, 1024, 128, seed=1)
        assert "decode" in qg.describe_dispatch(layer.w, 1), wtype
        big = qg.describe_dispatch(layer.w, 512)
        assert ("tiled" in big) == (wtype == qg.W_E0M3), (wtype, big)


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("wtype", A16_EXT)
def test_wna16_decode_wide(override, wtype, group):
    """The wide decode form (column tiles along the workgroup's waves, K in
    slices): N = 200 (a partial last column group), K = 2560 (20 k-blocks:
    three slices of 8, the last half full, or two of 16, the last short);
    16-block slices only below 8-bit codes."""
    layer = Layer(wtype, 200, 2560, group, seed=90 + wtype + group)
    bits8 = wtype in (qg.W_INT8, qg.W_UINT8, qg.W_E0M7, qg.W_FP8)
    for tune in ("8,8", "8,16", "5,8"):
        override("QG_DECODE_WIDE", tune)
        for m in (2, 16):
            d = qg.describe_dispatch(layer.w, m)
            if tune == "8,16" and (bits8 or group == 32):  # (g32: 64 scales per slice, 96 per row)
                assert "a16_decode_wide" not in d, d
                continue
            assert "a16_decode_wide" in d, (tune, m, d)
            _check_a16(layer, m, seed=95 + m)


def test_wna16_long_k_decode_split():
    """INT8 and INT2 at the long-K decode shape (N = 4096, K = 14336, M = 1)."""
    for wtype in (qg.W_INT8, qg.W_UINT2):
        layer = Layer(wtype, 4096, 14336, 128, seed=80 + wtype)
        print(f"wtype={wtype}: {qg.describe_dispatch(layer.w, 1)}", flush=True)
        _check_a16(layer, 1, seed=81)
        layer.drop_wdq()


# ---------------------------------------------------------------------------
# MoE with the new A16 formats
# ---------------------------------------------------------------------------

def _moe(layer, acts, ids, x_rows, otype):
    """qg_moe_sort then qg_moe_gemm (rows by pair); layer: .w, .n, .experts."""
    t, topk = ids.shape
    e = layer.experts
    d_ids = to_dev(ids.astype(np.int32))
    sorted_ids = torch.full((t * topk,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.empty(e + 1, dtype=torch.int32, device="cuda")
    ws_bytes = qg.moe_workspace_size(layer.w, t, topk)
    ws = torch.full((max(ws_bytes, 1),), 0x5A, dtype=torch.uint8, device="cuda")
    qg.moe_sort(d_ids, t, topk, e, sorted_ids, offsets, ws, ws_bytes)
    y = torch.zeros((t * topk, layer.n), dtype=torch.float32 if otype == qg.O_F32 else torch.bfloat16,
                    device="cuda")
    qg.moe_gemm(layer.w, acts.x, acts.xs, x_rows, sorted_ids, offsets, t, topk, y, otype, qg.ROWS_BY_PAIR,
                ws, ws_bytes)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("wtype", [qg.W_INT8, qg.W_UINT2, qg.W_INT1, qg.W_FP8, qg.W_E0M3])
def test_wna16_formats_moe(wtype):
    t, e, topk, n, k, g = 40, 8, 2, 96, 512, 128
    ids = synth.route(synth.rng(3, wtype), t, e, topk)
    layer = Layer(wtype, n, k, g, seed=4, experts=e)
    acts = Acts(False, t, k, seed=5)
    ref = oracle.moe_gemm(layer.wdq, acts.xdq, ids, rows_by_token=True)
    yb = _moe(layer, acts, ids, qg.ROWS_BY_TOKEN, qg.O_BF16)
    yf = _moe(layer, acts, ids, qg.ROWS_BY_TOKEN, qg.O_F32)
    eb, ef = oracle.normwise_error(yb, ref), oracle.normwise_error(yf, ref)
    print(f"  wtype={wtype} bf16 err {eb:.3e} fp32 err {ef:.3e}", flush=True)
    assert eb <= TOL_BF16 and ef <= TOL_F32
    assert np.array_equal(yb, oracle.round_bf16(yf))


# ---------------------------------------------------------------------------
# W4A8 with per-token FP8 activations
# ---------------------------------------------------------------------------

class TokActs:
    """e4m3 activations with one fp32 scale per row."""

    def __init__(self, m, k, seed):
        self.codes, self.scales = synth.fp8_activations(synth.rng(seed, 9), m, k, None)
        self.xdq = oracle.dequant_activations(oracle.A_FP8_TOKEN, self.codes, self.scales, k)
        self.x = to_dev(self.codes)
        self.xs = to_dev(self.scales)


def _tok_model(layer, acts, rows, cols, dispatch):
    """fp32 outputs the kernel must produce: the block-scaled MFMA model with
    unit activation block scales, times the row's scale in fp32."""
    wc, ws = mx_codes(layer)
    ones = np.full((len(rows), layer.k // 32), 127, np.uint8)
    part = MM.predict(acts.codes[rows], ones, wc[cols], ws[cols], "e4m3", dispatch)
    return (part * acts.scales[rows][:, None].astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("m", [1, 16, 100, 128, 300])
@pytest.mark.parametrize("nk", [(512, 1024), (200, 640)])
def test_w4a8_per_token_dense(m, nk):
    """Below 128 rows the MX skinny kernel, from 128 rows the MX tiled kernel
    (256-row tiles from 256 rows; 300 rows leave a ragged second tile), each
    with unit activation block scales and the row scale on the output."""
    n, k = nk
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=90, atype=qg.A_FP8_TOKEN)
    acts = TokActs(m, k, seed=91 + m)
    disp = qg.describe_dispatch(layer.w, m)
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        ys[otype] = run_gemm(layer, acts, m, otype)
        print(f"  M={m} N={n} K={k} otype={otype} err={err(ys[otype], yref):.3e} ({disp})", flush=True)
    assert err(ys[qg.O_BF16], yref) <= TOL_BF16
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    assert ("mx_tiled" in disp) == (m >= 128), disp
    rows = np.arange(m)
    cols = np.arange(n)
    want = _tok_model(layer, acts, rows, cols, disp)
    got = ys[qg.O_F32].cpu().numpy()
    diff = got != want
    ulps = np.abs(got[diff].astype(np.float64) - want[diff]) / np.spacing(np.abs(want[diff]))
    print(f"  fp32 == model on {got.size - int(diff.sum())} of {got.size}", flush=True)
    assert int(diff.sum()) <= max(1, got.size // 1000) and np.all(ulps <= 1.0)


@pytest.mark.parametrize("t,k", [(33, 512), (300, 512), (300, 640)])
def test_w4a8_per_token_moe(t, k):
    """33 tokens x top-4 (132 pairs, every expert on the skinny kernel) and
    300 x top-4 (1200 pairs over 8 experts: the 128-row tiles of the MX tiled
    kernel), at K = 512 and 640."""
    e, topk, n = 8, 4, 128
    ids = synth.route(synth.rng(6, 1), t, e, topk)
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=7, experts=e, atype=qg.A_FP8_TOKEN)
    acts = TokActs(t, k, seed=8)
    ref = oracle.moe_gemm(layer.wdq, acts.xdq, ids, rows_by_token=True)
    yb = _moe(layer, acts, ids, qg.ROWS_BY_TOKEN, qg.O_BF16)
    yf = _moe(layer, acts, ids, qg.ROWS_BY_TOKEN, qg.O_F32)
    eb, ef = oracle.normwise_error(yb, ref), oracle.normwise_error(yf, ref)
    print(f"  bf16 err {eb:.3e} fp32 err {ef:.3e}", flush=True)
    assert eb <= TOL_BF16
    assert np.array_equal(yb, oracle.round_bf16(yf))
    # fp32 rows against the model, expert by expert (one of the kernel forms
    # the MoE dispatch names for this pair count)
    flat = ids.reshape(-1)
    forms = moe_mx_forms(layer, flat.size)
    print(f"  MoE dispatch: {qg.describe_moe_dispatch(layer.w, t, topk)}", flush=True)
    for ex in np.unique(flat):
        pairs = np.nonzero(flat == ex)[0]
        wc, ws = mx_codes(layer, int(ex))
        ones = np.full((pairs.size, k // 32), 127, np.uint8)
        got = yf[pairs].astype(np.float32)
        diffs = []
        for disp in forms:
            part = MM.predict(acts.codes[pairs // topk], ones, wc, ws, "e4m3", disp)
            want = (part * acts.scales[pairs // topk][:, None].astype(np.float32)).astype(np.float32)
            diffs.append(int((got != want).sum()))
        assert min(diffs) <= max(1, got.size // 1000), (ex, forms, diffs)


# ---------------------------------------------------------------------------
# W8A8 FP8 with block scales
# ---------------------------------------------------------------------------

class W8A8:
    def __init__(self, n, k, seed, experts=1):
        self.n, self.k, self.experts = n, k, experts
        self.desc = qg.layer_desc(qg.W_FP8, n, k, 128, atype=qg.A_FP8_BLOCK, num_experts=experts)
        self.buf = torch.empty(qg.packed_size(self.desc), dtype=torch.uint8, device="cuda")
        self.std = []
        for e in range(experts):
            codes, sc = synth.fp8_block_weights(synth.rng(seed, 300 + e), n, k)
            self.std.append((codes, sc))
            self.w = qg.preprocess(self.desc, codes, sc, None, self.buf, expert_begin=e, expert_count=1)

    def wdq(self, e=0):
        codes, sc = self.std[e]
        return oracle.dequant_weights_fp8_block(codes, sc, self.n, self.k)

    def col_scales(self, e=0):
        return self.std[e][1][np.arange(self.n) // 128]


class BlockActs:
    def __init__(self, m, k, seed):
        self.codes, self.scales = synth.fp8_activations(synth.rng(seed, 10), m, k, 128)
        self.xdq = oracle.dequant_activations(oracle.A_FP8_BLOCK, self.codes, self.scales, k)
        self.x = to_dev(self.codes)
        self.xs = to_dev(self.scales)


def _check_w8a8_f32(y, layer, acts, rows, disp, e=0, ref=None):
    """fp32 outputs within the W8A8 error bound of the exact product and, for
    a skinny-kernel launch, equal to the instruction model of its wave layout
    (tests/mx_mfma_model.py: the block-scaled MFMA rules with both operands
    e4m3, each step's partial scaled by an fp32 fma), with the allowance of
    assert_mx_f32: at most 1 in 1000 outputs one ulp apart."""
    wc, _ = layer.std[e]
    wcol = layer.col_scales(e)
    exact = oracle.gemm(acts.xdq[rows], layer.wdq(e)) if ref is None else ref
    bound = MM.w8a8_error_bound(acts.codes[rows], acts.scales[rows], wc, wcol)
    dev = np.abs(np.asarray(y, np.float64) - exact)
    assert np.all(dev <= bound), (float((dev / np.maximum(bound, 1e-300)).max()), disp)
    if "skinny" in disp or "tiled" in disp:
        import re
        v = dict(re.findall(r"(\w+)=(\d+)", disp))
        if "tiled" in disp:  # one chain over every K step in order
            kr, waves, splits = layer.k // 128, 1, 1
        else:
            kr, waves, splits = int(v["KR"]), int(v["W"]), int(v.get("splits", 1))
        pred = MM.gemm_w8a8(acts.codes[rows], acts.scales[rows], wc, wcol, kr, waves, splits)
        got = np.asarray(y, np.float32)
        diff = pred != got
        ulps = np.abs(got[diff].astype(np.float64) - pred[diff]) / np.spacing(np.abs(pred[diff]))
        print(f"  fp32 within the bound; equal to the instruction model on {pred.size - int(diff.sum())} of "
              f"{pred.size}", flush=True)
        assert int(diff.sum()) <= max(1, pred.size // 1000) and np.all(ulps <= 1.0), (int(diff.sum()), disp)


@pytest.mark.parametrize("m", [1, 16, 64, 128, 300])
@pytest.mark.parametrize("nk", [(512, 1024), (200, 640), (136, 384), (72, 128)])
def test_w8a8_dense(m, nk):
    """Below 128 rows the skinny kernel; from 128 rows the tiled kernel's
    W8A8 form (128 x 128 tiles, 256 x 128 from 256 rows; 300 rows leave a
    ragged tile, N = 200 a ragged column tile, K = 640 five steps, K = 384
    three, K = 128 one; N = 136 and 72 end inside a 16-column tile)."""
    n, k = nk
    layer = W8A8(n, k, seed=100)
    acts = BlockActs(m, k, seed=101 + m)
    disp = qg.describe_dispatch(layer.w, m)
    assert ("f8_tiled" in disp) == (m >= 128), disp
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        ys[otype] = run_gemm(layer, acts, m, otype)
        print(f"  M={m} N={n} K={k} otype={otype} err={err(ys[otype], yref):.3e} ({disp})", flush=True)
    assert err(ys[qg.O_BF16], yref) <= TOL_BF16
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    _check_w8a8_f32(ys[qg.O_F32].cpu().numpy(), layer, acts, np.arange(m), disp, ref=yref)


def test_w8a8_tiled_right_edge_inside_padded_rows():
    """The W8A8 tiled form (transposed epilogue) with N = 102 inside rows of
    ldy = 104: the last chunk of each row is written byte by byte, the padding
    columns keep their values, the valid ones meet the W8A8 bounds."""
    from test_gpu_dense import gemm_padded_rows
    m, n, k, ldy = 256, 102, 512, 104
    layer = W8A8(n, k, seed=103)
    acts = BlockActs(m, k, seed=104)
    disp = qg.describe_dispatch(layer.w, m)
    assert "f8_tiled" in disp, disp
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        y = gemm_padded_rows(layer, acts, m, otype, ldy)
        assert (y[:, n:] == 7.0).all(), otype
        ys[otype] = y[:, :n].contiguous()
    assert err(ys[qg.O_BF16], yref) <= TOL_BF16
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    _check_w8a8_f32(ys[qg.O_F32].cpu().numpy(), layer, acts, np.arange(m), disp, ref=yref)


@pytest.mark.parametrize("m", [40, 100])
def test_tiled_below_128_rows(m):
    """Wide layers run the MX and W8A8 tiled forms from a few dozen rows (one
    partial 128-row tile): W8A8 at N = 8192, MXFP8 and per-token W4A8 at
    N = 12288, each against the oracle and its instruction model."""
    k = 256
    # W8A8
    layer = W8A8(8192, k, seed=107)
    acts = BlockActs(m, k, seed=108)
    disp = qg.describe_dispatch(layer.w, m)
    assert "f8_tiled" in disp, disp
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {o: run_gemm(layer, acts, m, o) for o in (qg.O_BF16, qg.O_F32)}
    assert err(ys[qg.O_BF16], yref) <= TOL_BF16
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    _check_w8a8_f32(ys[qg.O_F32].cpu().numpy(), layer, acts, np.arange(m), disp, ref=yref)
    # per-token FP8 W4A8
    n = 12288
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=109, atype=qg.A_FP8_TOKEN)
    acts = TokActs(m, k, seed=110)
    disp = qg.describe_dispatch(layer.w, m)
    assert "mx_tiled" in disp, disp
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {o: run_gemm(layer, acts, m, o) for o in (qg.O_BF16, qg.O_F32)}
    assert err(ys[qg.O_BF16], yref) <= TOL_BF16
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    want = _tok_model(layer, acts, np.arange(m), np.arange(n), disp)
    got = ys[qg.O_F32].cpu().numpy()
    diff = got != want
    ulps = np.abs(got[diff].astype(np.float64) - want[diff]) / np.spacing(np.abs(want[diff]))
    assert int(diff.sum()) <= max(1, got.size // 1000) and np.all(ulps <= 1.0)
    # MXFP4 x MXFP8
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=111)
    acts = Acts(True, m, k, seed=112)
    disp = qg.describe_dispatch(layer.w, m)
    assert "mx_tiled" in disp, disp
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {o: run_gemm(layer, acts, m, o) for o in (qg.O_BF16, qg.O_F32)}
    assert err(ys[qg.O_BF16], yref) <= TOL_BF16
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    check_mx_f32(layer, acts, m, ys[qg.O_F32])


@pytest.mark.parametrize("m", [8, 136])
def test_w8a8_identity_rows_are_exact(m):
    """Unit activations (e4m3 1.0, scale 1) at block edges: each fp32 row is a
    column of the dequantized weight, e4m3(w) * sw[n // 128][k // 128], rounded
    once to fp32 (the step's exact partial times its scale; every other step
    adds an exact zero).  8 rows: the skinny kernel; 136: the tiled kernel."""
    n, k = 160, 512
    layer = W8A8(n, k, seed=102)
    cols = [[0, 127, 128, 255, 256, 383, 384, 511][i % 8] for i in range(m)]
    codes = np.zeros((m, k), np.uint8)
    for i, c in enumerate(cols):
        codes[i, c] = 0x38
    acts = BlockActs(m, k, seed=1)
    acts.codes, acts.scales = codes, np.ones((m, k // 128), np.float32)
    acts.x, acts.xs = to_dev(codes), to_dev(acts.scales)
    y = run_gemm(layer, acts, m, qg.O_F32).cpu().numpy().astype(np.float64)
    wdq = layer.wdq()
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], wdq[:, c].astype(np.float32).astype(np.float64)), (i, c)


@pytest.mark.parametrize("t,k", [(40, 512), (300, 512), (300, 640)])
def test_w8a8_moe(t, k):
    """40 tokens x top-2 (80 pairs: the skinny kernel) and 300 x top-2 (600
    pairs: 128-row tiles for experts with >= 64 rows, 64-row tiles below);
    K = 640 is five K steps (the weight-scale ring's second group holds one
    step)."""
    e, topk, n = 8, 2, 256
    ids = synth.route(synth.rng(11, 1), t, e, topk)
    layer = W8A8(n, k, seed=12, experts=e)
    acts = BlockActs(t, k, seed=13)
    ref = oracle.moe_gemm(layer.wdq, acts.xdq, ids, rows_by_token=True)
    yb = _moe(layer, acts, ids, qg.ROWS_BY_TOKEN, qg.O_BF16)
    yf = _moe(layer, acts, ids, qg.ROWS_BY_TOKEN, qg.O_F32)
    eb, ef = oracle.normwise_error(yb, ref), oracle.normwise_error(yf, ref)
    print(f"  bf16 err {eb:.3e} fp32 err {ef:.3e}", flush=True)
    assert eb <= TOL_BF16
    assert np.array_equal(yb, oracle.round_bf16(yf))
    print(f"  MoE dispatch: {qg.describe_moe_dispatch(layer.w, t, topk)}", flush=True)
    flat = ids.reshape(-1)
    for ex in np.unique(flat):
        pairs = np.nonzero(flat == ex)[0]
        _check_w8a8_f32(yf[pairs], layer, acts, pairs // topk, "moe", e=int(ex), ref=ref[pairs])


# ---------------------------------------------------------------------------
# FP8 activation quantizer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block", [0, 128])
@pytest.mark.parametrize("rows,k", [(1, 4096), (37, 7168), (5, 200), (300, 640)])
def test_quantize_fp8_bit_exact(block, rows, k):
    r = synth.rng(20, rows, k)
    x = r.normal(0, 1, size=(rows, k)) * np.exp2(r.integers(-30, 30, size=(rows, 1)))
    x[0, : k // 3] = 0.0
    if rows > 2:
        x[2] = 0.0                      # an all-zero row
        x[1, 5] = -0.0
    xb = synth.f32_to_bf16_bits(x.astype(np.float32))
    ldq = -(-k // 16) * 16
    q = torch.full((rows, ldq), 0xEE, dtype=torch.uint8, device="cuda")
    ns = 1 if block == 0 else -(-k // 128)
    qs = torch.full((rows, ns), -7.0, dtype=torch.float32, device="cuda")
    qg.quantize_fp8(to_dev(xb), rows, k, k, block, q, ldq, qs)
    torch.cuda.synchronize()
    c, s = Q.quantize_fp8_bf16(xb, None if block == 0 else 128)
    got_c = q.cpu().numpy()[:, :k]
    got_s = qs.cpu().numpy()
    assert np.array_equal(got_s.reshape(s.shape), s)
    bad = np.argwhere(got_c != c)
    assert bad.shape[0] == 0, (bad[:5].tolist(), got_c[tuple(bad[0])], c[tuple(bad[0])])
    assert (q.cpu().numpy()[:, k:] == 0xEE).all()   # nothing written past k


def test_w4a8_per_token_end_to_end():
    """bf16 X -> qg_quantize_fp8 (per token) -> the per-token W4A8 GEMM,
    against the oracle's quantizer and GEMM."""
    m, n, k = 24, 384, 1024
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=30, atype=qg.A_FP8_TOKEN)
    xb = synth.x_bf16(synth.rng(31, 1), m, k)
    q = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    qs = torch.empty((m,), dtype=torch.float32, device="cuda")
    qg.quantize_fp8(to_dev(xb), m, k, k, 0, q, k, qs)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    ws_bytes = qg.gemm_workspace_size(layer.w, m)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    qg.gemm(layer.w, q, qs, m, k, y, qg.O_F32, n, ws, ws_bytes)
    torch.cuda.synchronize()
    c, s = Q.quantize_fp8_bf16(xb, None)
    assert np.array_equal(q.cpu().numpy(), c)
    yref = oracle.gemm(oracle.dequant_activations(oracle.A_FP8_TOKEN, c, s, k), layer.wdq())
    e = err(y, yref)
    print(f"  end-to-end fp32 err {e:.3e}", flush=True)
    assert e <= 1e-4   # the block-scaled instruction's truncation (checked bit for bit above)
