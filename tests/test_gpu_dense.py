"""GPU parity of the dense path (qg_gemm through the C ABI) against the CPU oracle.

Tolerances (normwise max |Y - Yref| / max |Yref|): 2e-2 for bf16 outputs and
1e-5 for the fp32 accumulators (QG_O_F32) of the integer formats; 3e-5 for the
MXFP4 x MXFP8 accumulators, whose scaled MFMA sums each step in a fixed-point
window (see gpu_harness).  Dequantized weights are checked bit-exactly through
one-hot activation rows.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qg_amd as qg
import synth
from gpu_harness import TOL_BF16, TOL_F32, Acts, Layer, assert_bf16_is_rne, check_mx_f32, err, require_gpu, run_gemm

pytestmark = pytest.mark.gpu

A16 = [qg.W_INT4, qg.W_UINT4, qg.W_INT3, qg.W_UINT3]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check(layer, acts, m, rows=None):
    """bf16 outputs against the oracle (normwise); fp32 outputs against the
    oracle (integer formats: normwise) or, for MX layers, bit for bit
    against the block-scaled MFMA model (the normwise error is printed); the
    bf16 output against RNE of the fp32 one (bit for bit)."""
    ys = {}
    for otype, tol in ((qg.O_BF16, TOL_BF16), (qg.O_F32, TOL_F32)):
        y = ys[otype] = run_gemm(layer, acts, m, otype)
        if rows is None:
            yref = oracle.gemm(acts.xdq, layer.wdq())
            e = err(y, yref)
        else:
            yref = oracle.gemm(acts.xdq[rows], layer.wdq())
            e = oracle.normwise_error(y[rows].float().cpu().numpy().astype(np.float64), yref)
        print(f"  otype={otype} err={e:.3e}", flush=True)
        assert torch.isfinite(y.float()).all()
        if otype == qg.O_F32 and layer.mx:
            check_mx_f32(layer, acts, m, y, rows=rows)
        else:
            assert e <= tol, (otype, e)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])


def test_tiny_w4a16_config():
    """M=16, N=256, K=512, symmetric INT4 group 128, bf16 activations."""
    layer = Layer(qg.W_INT4, 256, 512, 128, seed=0)
    _check(layer, Acts(False, 16, 512, seed=0), 16)


@pytest.mark.parametrize("wtype", A16)
@pytest.mark.parametrize("group", [32, 64, 128])
def test_a16_formats_and_groups(wtype, group):
    layer = Layer(wtype, 96, 768, group, seed=wtype * 10 + group)
    for m in (1, 5, 16):
        _check(layer, Acts(False, m, 768, seed=m), m)


@pytest.mark.parametrize("wtype", A16 + [qg.W_MXFP4])
def test_identity_rows_give_exact_dequantized_weights(wtype):
    """One-hot X rows return Wdq[:, k] exactly in the fp32 output."""
    n, k = 40, 640
    g = 32 if wtype == qg.W_MXFP4 else 128
    layer = Layer(wtype, n, k, g, seed=5)
    wdq = layer.wdq()
    ks = [0, 1, 7, 8, 31, 32, 95, 96, 127, 128, 255, 256, 383, 511, 512, 639]
    m = len(ks)
    if wtype == qg.W_MXFP4:
        codes = np.zeros((m, k), np.uint8)
        for i, kk in enumerate(ks):
            codes[i, kk] = 0x38  # e4m3 1.0
        acts = Acts(True, m, k, values=(codes, np.full((m, k // 32), 127, np.uint8)))
    else:
        bits = np.zeros((m, k), np.uint16)
        for i, kk in enumerate(ks):
            bits[i, kk] = 0x3F80
        acts = Acts(False, m, k, values=bits)
    y = run_gemm(layer, acts, m, qg.O_F32).cpu().numpy()
    for i, kk in enumerate(ks):
        assert np.array_equal(y[i].astype(np.float64), wdq[:, kk]), kk


@pytest.mark.parametrize("m", [1, 2, 15, 17, 33, 64])
def test_ragged_shapes(m):
    """N not a multiple of 16, K = 640 (five 128-blocks), several row tiles."""
    layer = Layer(qg.W_UINT4, 72, 640, 64, seed=m)
    _check(layer, Acts(False, m, 640, seed=m), m)
    mxl = Layer(qg.W_MXFP4, 40, 640, 32, seed=m)
    _check(mxl, Acts(True, m, 640, seed=m), m)


def test_split_k_path_matches(override):
    """K split across workgroups: one zero-filled workspace serves consecutive
    calls with different split counts (the counters reset themselves)."""
    layer = Layer(qg.W_UINT4, 64, 4096, 128, seed=3)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    for m in (16, 3):
        acts = Acts(False, m, 4096, seed=3)
        ref = oracle.gemm(acts.xdq, layer.wdq())
        for tune in ("1,2,4,4", "1,1,2,16", "2,2,4,4", "4,2,8,2", "1,4,1,8"):
            override("QG_TUNE", tune)
            assert int(qg.describe_dispatch(layer.w, m).split("splits=")[1].split()[0]) > 1
            need = qg.gemm_workspace_size(layer.w, m)
            assert 0 < need <= ws.numel()
            for _ in range(2):
                y = torch.empty((m, 64), dtype=torch.float32, device="cuda")
                qg.gemm(layer.w, acts.x, None, m, 4096, y, qg.O_F32, 64, ws, ws.numel())
                torch.cuda.synchronize()
                assert err(y, ref) <= TOL_F32, tune
            assert int(ws[:4 * 64].view(torch.int32).abs().sum()) == 0  # counters back at zero


def test_tuning_variants_agree(override):
    layer = Layer(qg.W_INT3, 64, 2048, 128, seed=4)
    acts = Acts(False, 7, 2048, seed=4)
    ref = oracle.gemm(acts.xdq, layer.wdq())
    for tune in ("1,1,16,1", "1,2,8,1", "1,4,4,1", "2,4,4,1", "2,1,16,1", "1,8,2,1"):
        override("QG_TUNE", tune)
        y = run_gemm(layer, acts, 7, qg.O_F32)
        assert err(y, ref) <= TOL_F32, tune


def test_mx_small_and_medium_m():
    layer = Layer(qg.W_MXFP4, 1280, 4096, 32, seed=9)
    for m in (1, 16, 100):
        _check(layer, Acts(True, m, 4096, seed=m), m)


def test_zero_rows_is_noop():
    layer = Layer(qg.W_INT4, 64, 256, 128)
    y = torch.full((1, 64), 7.0, device="cuda")
    qg.gemm(layer.w, torch.empty(256, dtype=torch.int16, device="cuda"), None, 0, 256, y,
            qg.O_F32, 64)
    torch.cuda.synchronize()
    assert (y == 7.0).all()


def gemm_padded_rows(layer, acts, m, otype, ldy, fill=7.0):
    """One qg_gemm into rows of ldy >= N elements pre-filled with `fill`;
    returns the [m, ldy] output."""
    dt = torch.float32 if otype == qg.O_F32 else torch.bfloat16
    y = torch.full((m, ldy), fill, dtype=dt, device="cuda")
    ws_bytes = qg.gemm_workspace_size(layer.w, m)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    qg.gemm(layer.w, acts.x, acts.xs, m, layer.k, y, otype, ldy, ws, ws_bytes)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("wtype", [qg.W_INT4, qg.W_MXFP4])
def test_tiled_right_edge_inside_padded_rows(wtype):
    """N = 102 ends inside the last 16-byte chunk of a row (bf16: 6 of its 8
    elements, fp32: 2 of 4), which the tiled kernels' epilogue writes byte by
    byte; rows of ldy = 104 keep every row start 16-byte aligned.  The valid
    columns match the oracle, the two padding columns keep their values."""
    m, n, k, ldy = 256, 102, 512, 104
    layer = Layer(wtype, n, k, 32 if wtype == qg.W_MXFP4 else 128, seed=81)
    acts = Acts(wtype == qg.W_MXFP4, m, k, seed=82)
    disp = qg.describe_dispatch(layer.w, m)
    assert "tiled" in disp, disp
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        y = gemm_padded_rows(layer, acts, m, otype, ldy)
        assert (y[:, n:] == 7.0).all(), otype
        ys[otype] = y[:, :n].contiguous()
        print(f"  {disp} otype={otype} err={err(ys[otype], yref):.3e}", flush=True)
    assert err(ys[qg.O_BF16], yref) <= TOL_BF16
    if layer.mx:
        check_mx_f32(layer, acts, m, ys[qg.O_F32])
    else:
        assert err(ys[qg.O_F32], yref) <= TOL_F32
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])


# ---------------------------------------------------------------------------
# full-size decode shapes (dense W4A16, memory bound): every element compared
# ---------------------------------------------------------------------------

DECODE_SHAPES = [(14336, 4096), (4096, 14336)]


@pytest.mark.parametrize("wtype", [qg.W_UINT4, qg.W_INT3])
@pytest.mark.parametrize("nk", DECODE_SHAPES)
def test_decode_full_size(wtype, nk):
    n, k = nk
    print(f"decode wtype={wtype} N={n} K={k}", flush=True)
    layer = Layer(wtype, n, k, 128, seed=11)
    for m in (1, 4, 8, 10, 16):
        _check(layer, Acts(False, m, k, seed=20 + m), m)


@pytest.mark.parametrize("nk", [(3072, 4096), (14336, 4096)])
def test_w4a8_mx_full_size_sampled_rows(nk):
    """(4096, N, 4096) MXFP4 x MXFP8: all outputs computed, 96 sampled rows
    compared against the oracle (the oracle computes those rows only)."""
    n, k = nk
    m = 4096
    print(f"mx M={m} N={n} K={k}", flush=True)
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=13)
    acts = Acts(True, m, k, seed=13)
    rows = np.sort(synth.rng(0, 99).choice(m, 96, replace=False))
    rows[0], rows[-1] = 0, m - 1
    _check(layer, acts, m, rows=rows)


@pytest.mark.parametrize("bn", ["256", "224", "192"])
@pytest.mark.parametrize("m,n,k", [(256, 128, 1024), (300, 200, 640), (777, 1040, 4096)])
def test_mx_tiled_large_m_ragged(override, m, n, k, bn):
    """The LDS-tiled MX kernel (M >= 256) with partial row and column tiles,
    at each tile width (224 and 192 columns split their blocks unevenly over
    the 8 waves)."""
    override("QG_MX_BN", bn)
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=m)
    assert f"tiled BM=256 BN={bn}" in qg.describe_dispatch(layer.w, m)
    _check(layer, Acts(True, m, k, seed=m), m)


@pytest.mark.parametrize("m", [256, 130])
@pytest.mark.parametrize("k", [128, 256, 384, 896])
def test_mx_tiled_short_k(m, k):
    """1, 2, 3 and 7 K steps through the tiled MX kernel (256- and 128-row
    tiles): its K loop runs four steps per trip (the weight-scale byte select
    is an instruction field), so every remainder of the step count by 4 is
    exercised."""
    layer = Layer(qg.W_MXFP4, 136, k, 32, seed=k + m)
    assert "mx_tiled" in qg.describe_dispatch(layer.w, m)
    _check(layer, Acts(True, m, k, seed=k), m)


@pytest.mark.parametrize("m,n,k", [(300, 200, 1024), (256, 448, 4096)])
def test_mx_tiled_unaligned_activation_scales(m, n, k):
    """K % 512 == 0 with the activation scales at a 4-byte (not 16-byte)
    aligned address: the tiled kernel falls back from its scale ring to the
    scales regrouped by K step.  Checked against the oracle, and against the
    same call on aligned scales bit for bit."""
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=k + n)
    acts = Acts(True, m, k, seed=m + 5)
    assert "mx_tiled" in qg.describe_dispatch(layer.w, m)
    y_al = run_gemm(layer, acts, m, qg.O_F32)
    buf = torch.zeros(acts.xs.numel() + 16, dtype=torch.uint8, device="cuda")
    view = buf[4:4 + acts.xs.numel()].view(acts.xs.shape)
    view.copy_(acts.xs)
    assert view.data_ptr() % 16 == 4
    acts.xs = view
    y_un = run_gemm(layer, acts, m, qg.O_F32)
    assert torch.equal(y_al, y_un)
    check_mx_f32(layer, acts, m, y_un)


def test_mx_tiled_identity_rows_exact():
    n, k, m = 64, 640, 256
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=21)
    wdq = layer.wdq()
    codes = np.zeros((m, k), np.uint8)
    codes[np.arange(m), np.arange(m) * 2 % k] = 0x38
    acts = Acts(True, m, k, values=(codes, np.full((m, k // 32), 127, np.uint8)))
    y = run_gemm(layer, acts, m, qg.O_F32).cpu().numpy()
    for i in range(m):
        assert np.array_equal(y[i].astype(np.float64), wdq[:, (2 * i) % k]), i


# ---------------------------------------------------------------------------
# LDS-tiled bf16-MFMA kernel for the integer formats (M >= 256)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tile", ["256x128", "128x128", "128x256"])
@pytest.mark.parametrize("wtype", A16)
@pytest.mark.parametrize("group", [32, 64, 128])
def test_a16_tiled_formats_and_groups(override, tile, wtype, group):
    """Every integer format and group size through the tiled kernel at each
    tile shape, with a partial row tile and a partial column tile (N = 200 is
    not a multiple of the 128- or 256-column tile)."""
    bm, bn = tile.split("x")
    override("QG_TILED_BM", bm)
    override("QG_A16_BN", bn)
    layer = Layer(wtype, 200, 640, group, seed=wtype * 10 + group)
    m = 300
    assert f"a16_tiled BM={bm} BN={bn}" in qg.describe_dispatch(layer.w, m)
    _check(layer, Acts(False, m, 640, seed=m + group), m)


@pytest.mark.parametrize("bn", ["128", "256"])
@pytest.mark.parametrize("m,n,k", [(256, 128, 1024), (512, 72, 128), (777, 1040, 4096)])
def test_a16_tiled_ragged(override, m, n, k, bn):
    override("QG_A16_BN", bn)
    layer = Layer(qg.W_UINT4, n, k, 128, seed=m)
    assert f"a16_tiled BM={256 if bn == '128' else 128} BN={bn}" in qg.describe_dispatch(layer.w, m)
    _check(layer, Acts(False, m, k, seed=m), m)


@pytest.mark.parametrize("wtype", A16)
def test_a16_tiled_identity_rows_exact(wtype):
    """One-hot X rows through the tiled kernel return Wdq[:, k] bit-exactly."""
    n, k, m = 136, 640, 320
    layer = Layer(wtype, n, k, 64, seed=23)
    wdq = layer.wdq()
    bits = np.zeros((m, k), np.uint16)
    cols = (np.arange(m) * 2 + 1) % k
    bits[np.arange(m), cols] = 0x3F80
    acts = Acts(False, m, k, values=bits)
    assert "a16_tiled" in qg.describe_dispatch(layer.w, m)
    y = run_gemm(layer, acts, m, qg.O_F32).cpu().numpy()
    for i in range(m):
        assert np.array_equal(y[i].astype(np.float64), wdq[:, cols[i]]), i


@pytest.mark.parametrize("nk", [(14336, 4096), (4096, 14336)])
def test_w4a16_large_m_full_size_sampled_rows(nk):
    """(4096, N, K) symmetric INT4, group 128: all outputs computed, 64 sampled
    rows compared against the oracle."""
    n, k = nk
    m = 4096
    print(f"w4a16 M={m} N={n} K={k}", flush=True)
    layer = Layer(qg.W_INT4, n, k, 128, seed=17)
    acts = Acts(False, m, k, seed=17)
    rows = np.sort(synth.rng(0, 98).choice(m, 64, replace=False))
    rows[0], rows[-1] = 0, m - 1
    assert "a16_tiled" in qg.describe_dispatch(layer.w, m)
    _check(layer, acts, m, rows=rows)


# ---------------------------------------------------------------------------
# dense decode kernel (integer formats, M <= 16, K % 512 == 0, rows in LDS)
# ---------------------------------------------------------------------------

# "T,KR" or "T,KR,splits" (split K across workgroups)
DECODE_VARIANTS = {128: ["4,2", "2,4", "4,4", "1,4", "1,8", "2,8", "1,4,2", "1,4,3", "1,8,2", "2,4,2", "4,4,2"],
                   64: ["4,2", "2,4", "2,4,2"],
                   32: ["1,4", "1,8", "1,4,2", "1,8,2"]}


@pytest.mark.parametrize("wtype", A16)
@pytest.mark.parametrize("group", [32, 64, 128])
def test_decode_kernel_variants(override, wtype, group):
    """Every compiled (T, KR) of the decode kernel, with and without a K
    split; N = 200 leaves a partial n-tile block, K = 1536 (12 blocks) a
    partial last wave for KR = 8 and a short last split."""
    layer = Layer(wtype, 200, 1536, group, seed=wtype * 10 + group + 1)
    for tune in DECODE_VARIANTS[group]:
        override("QG_DECODE", tune)
        for m in (1, 3, 16):
            assert "a16_decode" in qg.describe_dispatch(layer.w, m), (tune, m)
            print(f"  decode {tune} m={m}", flush=True)
            _check(layer, Acts(False, m, 1536, seed=m + group), m)


def test_decode_split_k_reuses_workspace(override):
    """Split-K decode: the per-tile arrival counters return to zero, so one
    workspace (zero-filled once) serves consecutive calls."""
    override("QG_DECODE", "1,4,2")
    n, k = 200, 2048
    layer = Layer(qg.W_UINT4, n, k, 128, seed=77)
    m = 1
    assert "splits=2" in qg.describe_dispatch(layer.w, m)
    ws_bytes = qg.gemm_workspace_size(layer.w, m)
    assert ws_bytes > 0
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    wdq = layer.wdq()
    for call in range(3):
        acts = Acts(False, m, k, seed=100 + call)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        qg.gemm(layer.w, acts.x, None, m, k, y, qg.O_F32, n, ws, ws_bytes)
        torch.cuda.synchronize()
        e = err(y, oracle.gemm(acts.xdq, wdq))
        print(f"  call {call} err={e:.3e}", flush=True)
        assert e <= TOL_F32, (call, e)


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("wtype", A16)
def test_decode_kernel_identity_rows_exact(override, wtype, group):
    override("QG_DECODE", "1,8")  # 16 rows: past the default row limit
    n, k = 72, 1024
    layer = Layer(wtype, n, k, group, seed=31)
    wdq = layer.wdq()
    ks = [0, 1, 31, 32, 127, 128, 255, 511, 512, 513, 767, 896, 1000, 1023, 300, 700]
    m = len(ks)
    bits = np.zeros((m, k), np.uint16)
    for i, kk in enumerate(ks):
        bits[i, kk] = 0x3F80
    acts = Acts(False, m, k, values=bits)
    assert "a16_decode" in qg.describe_dispatch(layer.w, m)
    y = run_gemm(layer, acts, m, qg.O_F32).cpu().numpy()
    for i, kk in enumerate(ks):
        assert np.array_equal(y[i].astype(np.float64), wdq[:, kk]), kk


# wide decode form: "W,KR" = column tiles (waves) per workgroup, k-blocks per
# K slice
WIDE_VARIANTS = ["8,8", "8,16", "16,8", "3,16"]


@pytest.mark.parametrize("wtype", A16)
@pytest.mark.parametrize("group", [32, 128])
def test_decode_wide_variants(override, wtype, group):
    """The wide decode form.  N = 200 is 13 n-tiles (a partial last column
    group, a ragged last tile); K = 2560 is 20 k-blocks (KR = 8: three slices,
    the last half full; KR = 16: two, the last short), K = 1024 one slice at
    KR = 8 (direct stores), K = 4096 two full slices at KR = 16.  Rows 2, 7
    and 16."""
    for k in (2560, 1024, 4096):
        layer = Layer(wtype, 200, k, group, seed=wtype * 7 + group + k)
        for tune in WIDE_VARIANTS:
            override("QG_DECODE_WIDE", tune)
            for m in (2, 7, 16):
                d = qg.describe_dispatch(layer.w, m)
                if tune.endswith(",16") and group == 32 and k != 4096:
                    # a slice's 64 group scales must divide the row's padded
                    # groups (32 at K = 1024, 96 at K = 2560)
                    assert "a16_decode_wide" not in d, d
                    continue
                assert "a16_decode_wide" in d, (tune, m, d)
                print(f"  wide {tune} k={k} m={m}: {d}", flush=True)
                _check(layer, Acts(False, m, k, seed=m + group + k), m)


def test_decode_wide_split_reuses_workspace(override):
    """Wide form over several K slices: the per-group arrival counters return
    to zero, so one workspace (zero-filled once) serves consecutive calls of
    different row counts."""
    override("QG_DECODE_WIDE", "8,8")
    n, k = 200, 3072
    layer = Layer(qg.W_UINT4, n, k, 128, seed=78)
    wdq = layer.wdq()
    ws_bytes = max(qg.gemm_workspace_size(layer.w, m) for m in (16, 5))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    for call, m in enumerate((16, 5, 16)):
        assert "splits=3" in qg.describe_dispatch(layer.w, m)
        acts = Acts(False, m, k, seed=200 + call)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        qg.gemm(layer.w, acts.x, None, m, k, y, qg.O_F32, n, ws, ws_bytes)
        torch.cuda.synchronize()
        e = err(y, oracle.gemm(acts.xdq, wdq))
        print(f"  call {call} m={m} err={e:.3e}", flush=True)
        assert e <= TOL_F32, (call, e)


# ---------------------------------------------------------------------------
# one workspace shared by calls of different kernels, layers and M
# ---------------------------------------------------------------------------

def _gemm_ws(layer, acts, m, ws, otype=qg.O_F32):
    need = qg.gemm_workspace_size(layer.w, m)
    assert need <= ws.numel(), (need, ws.numel())
    y = torch.empty((m, layer.n), dtype=torch.float32 if otype == qg.O_F32 else torch.bfloat16, device="cuda")
    qg.gemm(layer.w, acts.x, acts.xs, m, layer.k, y, otype, layer.n, ws, ws.numel())
    torch.cuda.synchronize()
    return y


def test_workspace_shared_by_prefill_and_split_decode(override):
    """The headline layer (UINT4 + zero points, g128, N = 4096, K = 14336):
    M = 4096 runs the tiled kernel (group row sums written to the workspace's
    scratch), then M = 1 runs the decode kernel split in two along K (forced:
    the heuristic keeps this shape in one workgroup per tile) on the same
    workspace (its arrival counters sit in the workspace's counter prefix),
    then both once more.  Every result against the oracle; the counters end
    at zero."""
    override("QG_DECODE", "1,8,2")
    n, k = 4096, 14336
    layer = Layer(qg.W_UINT4, n, k, 128, seed=81)
    assert "a16_tiled" in qg.describe_dispatch(layer.w, 4096)
    assert "splits=2" in qg.describe_dispatch(layer.w, 1), qg.describe_dispatch(layer.w, 1)
    ws = torch.zeros(max(qg.gemm_workspace_size(layer.w, 4096), qg.gemm_workspace_size(layer.w, 1)),
                     dtype=torch.uint8, device="cuda")
    big = Acts(False, 4096, k, seed=82)
    rows = np.array([0, 1, 777, 2048, 4095])
    ref_big = oracle.gemm(big.xdq[rows], layer.wdq())
    for rnd in range(2):
        y = _gemm_ws(layer, big, 4096, ws)
        e = oracle.normwise_error(y[rows].cpu().numpy().astype(np.float64), ref_big)
        print(f"  round {rnd} M=4096 err={e:.3e}", flush=True)
        assert e <= TOL_F32
        for seed in (83, 84):
            small = Acts(False, 1, k, seed=seed + rnd)
            y = _gemm_ws(layer, small, 1, ws)
            e = err(y, oracle.gemm(small.xdq, layer.wdq()))
            print(f"  round {rnd} M=1 err={e:.3e}", flush=True)
            assert e <= TOL_F32
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


def test_workspace_shared_by_mx_tiled_scratch_and_split_skinny():
    """An MX layer with K % 512 != 0: the tiled kernel (M = 256) first regroups
    the activation scales by K step into the workspace's scratch; the skinny
    kernel at M = 1 then splits K across workgroups on the same workspace, and
    another layer's split call follows."""
    k = 8320  # 65 K steps of 128
    a = Layer(qg.W_MXFP4, 512, k, 32, seed=85)
    b = Layer(qg.W_MXFP4, 1040, k, 32, seed=86)
    assert "mx_tiled" in qg.describe_dispatch(a.w, 256)
    for L in (a, b):
        assert int(qg.describe_dispatch(L.w, 1).split("splits=")[1].split()[0]) > 1, qg.describe_dispatch(L.w, 1)
    need = max(qg.gemm_workspace_size(L.w, m) for L in (a, b) for m in (1, 256))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rnd in range(2):
        for L, m in ((a, 256), (a, 1), (b, 1), (b, 256), (a, 1)):
            acts = Acts(True, m, k, seed=87 + m + rnd)
            y = _gemm_ws(L, acts, m, ws)
            print(f"  N={L.n} M={m} err={err(y, oracle.gemm(acts.xdq, L.wdq())):.3e}", flush=True)
            check_mx_f32(L, acts, m, y)
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


def test_skinny_loops_over_long_k(override):
    """K beyond one pass of the workgroup (W * KR * splits < K blocks): the
    workgroups loop over K.  Integer and MX formats, dense."""
    for wtype, g, mx in ((qg.W_UINT4, 128, False), (qg.W_INT3, 64, False), (qg.W_MXFP4, 32, True)):
        layer = Layer(wtype, 80, 5120, g, seed=88)
        override("QG_TUNE", "2,2,4,1")  # 8 of 40 K blocks per pass: five passes
        m = 19
        assert "W=4 splits=1" in qg.describe_dispatch(layer.w, m)
        _check(layer, Acts(mx, m, 5120, seed=89), m)


@pytest.mark.parametrize("mnk", [(21, 200, 1024), (64, 512, 1024)])
@pytest.mark.parametrize("atype", ["mxfp8", "mxfp4"])
def test_mx_skinny_every_variant(override, atype, mnk):
    """Every compiled (T, KR) of the MX skinny kernel, with one wave per
    block up to 8 waves and a cross-workgroup split, for MXFP8 and MXFP4
    (widened in registers) activations."""
    from test_gpu_w4a4 import A4, check_a4
    m, n, k = mnk
    a4 = atype == "mxfp4"
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=90, atype=qg.A_MXFP4 if a4 else None)
    acts = A4(m, k, seed=91) if a4 else Acts(True, m, k, seed=91)
    bad = []
    for T in (1, 2, 4):
        for KR in (1, 2, 4):
            if T * KR > 8 or (T, KR) == (4, 4):
                continue
            for W, S in ((8 // KR, 1), (max(1, 4 // KR), 2), (1, 8 // KR)):
                tune = f"{T},{KR},{W},{S}"
                override("QG_TUNE", tune)
                print(f"  {atype} {tune}: {qg.describe_dispatch(layer.w, m)}", flush=True)
                try:
                    if a4:
                        check_a4(layer, acts, m)
                    else:
                        _check(layer, acts, m)
                except AssertionError as e:
                    bad.append((tune, str(e)[:120]))
    assert not bad, bad
