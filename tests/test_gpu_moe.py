"""GPU parity of the MoE path: qg_moe_sort (routing sort) and qg_moe_gemm
(grouped GEMM) through the C ABI, against the oracle's sort invariants and its
per-expert dense products."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qg_amd as qg
import synth
from gpu_harness import TOL_BF16, TOL_F32, Acts, Layer, assert_bf16_is_rne, check_moe_mx_f32, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def sort_on_gpu(ids: np.ndarray, experts: int, layer: Layer):
    t, topk = ids.shape
    d_ids = to_dev(ids.astype(np.int32))
    sorted_ids = torch.full((max(t * topk, 1),), -1, dtype=torch.int32, device="cuda")
    offsets = torch.empty(experts + 1, dtype=torch.int32, device="cuda")
    ws_bytes = qg.moe_workspace_size(layer.w, t, topk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    qg.moe_sort(d_ids, t, topk, experts, sorted_ids, offsets, ws, ws_bytes)
    torch.cuda.synchronize()
    return sorted_ids, offsets


def check_sort(ids, experts, sorted_ids, offsets):
    offs = offsets.cpu().numpy().astype(np.int64)
    assert np.array_equal(offs, oracle.moe_offsets(ids, experts))
    s = sorted_ids.cpu().numpy()[: ids.size]
    flat = ids.reshape(-1)
    for e in range(experts):
        seg = s[offs[e]:offs[e + 1]]
        assert set(seg.tolist()) == set(np.nonzero(flat == e)[0].tolist())


def run_moe(layer, acts, sorted_ids, offsets, t, topk, x_rows, y_rows, otype):
    p = t * topk
    y = torch.zeros((p, layer.n), dtype=torch.float32 if otype == qg.O_F32 else torch.bfloat16,
                    device="cuda")
    ws_bytes = qg.moe_workspace_size(layer.w, t, topk)
    ws = torch.full((max(ws_bytes, 1),), 0x5A, dtype=torch.uint8, device="cuda")  # contents must not matter
    qg.moe_gemm(layer.w, acts.x, acts.xs, x_rows, sorted_ids, offsets, t, topk, y, otype, y_rows,
                ws, ws_bytes)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def check_f32(layer, acts, ids, y, ref, x_rows, y_rows, sorted_ids=None):
    """An fp32 grouped-GEMM output: integer formats within TOL_F32 of the
    oracle (normwise); MX layers bit for bit against the block-scaled MFMA
    model, expert by expert (the normwise error is printed)."""
    e = oracle.normwise_error(y, ref)
    print(f"  fp32 normwise err {e:.3e}", flush=True)
    if layer.mx:
        check_moe_mx_f32(layer, acts.codes, acts.scales, "e4m3", ids, y, x_rows, y_rows, sorted_ids)
    else:
        assert e <= TOL_F32, e


def moe_reference(layer, xdq, ids, by_token, verbose=False):
    def wdq(e):
        if verbose:
            print(f"    oracle expert {e}", flush=True)
        return layer.wdq(e)
    return oracle.moe_gemm(wdq, xdq, ids, rows_by_token=by_token)


# environment per split of the experts between kernels
SPLITS = {
    "skinny": {"QG_MOE_TILED_MIN": "0"},   # every expert on the skinny kernel
    "tiled": {"QG_MOE_TILED_MIN": "1"},    # every expert with a row on 128-row tiles
    "tiled_bn128": {"QG_MOE_TILED_MIN": "1", "QG_A16_BN": "128"},  # the same, 128-column tiles
    "tiled_mx_bn256": {"QG_MOE_TILED_MIN": "1", "QG_MOE_MX_BN": "256"},  # MX: 256-column tiles
    "mixed": {"QG_MOE_TILED_MIN": "12", "QG_MOE_SMALL": "1"},  # >= 12 rows: 128-row tiles; fewer: small tiles
    "mixed_skinny": {"QG_MOE_TILED_MIN": "12", "QG_MOE_SMALL": "0"},  # fewer: skinny kernel
    "small": {"QG_MOE_TILED_MIN": "1000", "QG_MOE_SMALL": "1"},  # every expert on 64-row small tiles
    "small32": {"QG_MOE_TILED_MIN": "1000", "QG_MOE_SMALL": "1", "QG_MOE_SMALL_BM": "32"},  # 32-row (integer formats)
}


@pytest.mark.parametrize("split", list(SPLITS))
@pytest.mark.parametrize("wtype", [qg.W_INT4, qg.W_UINT4, qg.W_INT3, qg.W_UINT3, qg.W_MXFP4])
def test_moe_small_all_row_modes(override, wtype, split):
    """All row modes, with the experts split between the kernels by row count
    (128-row tiles, 64-row small tiles, the skinny kernel)."""
    if wtype == qg.W_MXFP4 and split in ("tiled_bn128", "small32"):
        pytest.skip("same dispatch as another split for MXFP4")
    if wtype != qg.W_MXFP4 and split == "tiled_mx_bn256":
        pytest.skip("same dispatch as the tiled split for the integer formats")
    for var, val in SPLITS[split].items():
        override(var, val)
    t, e, topk, n, k = 37, 16, 4, 80, 640
    g = 32 if wtype == qg.W_MXFP4 else 128
    ids = synth.route(synth.rng(1, wtype), t, e, topk)
    layer = Layer(wtype, n, k, g, seed=2, experts=e)
    sorted_ids, offsets = sort_on_gpu(ids, e, layer)
    check_sort(ids, e, sorted_ids, offsets)
    mx = wtype == qg.W_MXFP4
    # gate/up style: rows by token
    acts = Acts(mx, t, k, seed=3)
    ref = moe_reference(layer, acts.xdq, ids, True)
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        ys[otype] = run_moe(layer, acts, sorted_ids, offsets, t, topk, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR, otype)
    assert oracle.normwise_error(ys[qg.O_BF16], ref) <= TOL_BF16
    check_f32(layer, acts, ids, ys[qg.O_F32], ref, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    # down style: rows by pair, output in sorted order
    h = Acts(mx, t * topk, k, seed=4)
    ref_pair = moe_reference(layer, h.xdq, ids, False)
    y = run_moe(layer, h, sorted_ids, offsets, t, topk, qg.ROWS_BY_PAIR, qg.ROWS_SORTED, qg.O_F32)
    s = sorted_ids.cpu().numpy()
    check_f32(layer, h, ids, y, ref_pair[s], qg.ROWS_BY_PAIR, qg.ROWS_SORTED, sorted_ids)
    # sorted input rows
    hs = Acts(mx, t * topk, k, seed=4)
    y = run_moe(layer, hs, sorted_ids, offsets, t, topk, qg.ROWS_SORTED, qg.ROWS_BY_PAIR, qg.O_F32)
    # pair s[i] reads H row i
    inv = np.empty_like(s)
    inv[s] = np.arange(s.size)
    ref2 = np.stack([hs.xdq[inv[p]] @ layer.wdq(int(ids.reshape(-1)[p])).T for p in range(t * topk)])
    check_f32(layer, hs, ids, y, ref2, qg.ROWS_SORTED, qg.ROWS_BY_PAIR, sorted_ids)


def test_moe_empty_and_single_row_experts():
    e, topk, n, k = 8, 2, 48, 256
    ids = np.array([[0, 7], [0, 7], [0, 3], [0, 7]], np.int32)  # experts 1,2,4,5,6 empty; 3 has one row
    t = ids.shape[0]
    layer = Layer(qg.W_UINT4, n, k, 128, seed=6, experts=e)
    sorted_ids, offsets = sort_on_gpu(ids, e, layer)
    check_sort(ids, e, sorted_ids, offsets)
    acts = Acts(False, t, k, seed=7)
    y = run_moe(layer, acts, sorted_ids, offsets, t, topk, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR, qg.O_F32)
    assert oracle.normwise_error(y, moe_reference(layer, acts.xdq, ids, True)) <= TOL_F32


def test_moe_sort_zero_tokens_and_out_of_range_ids():
    layer = Layer(qg.W_INT4, 32, 256, 128, experts=4)
    ids = np.zeros((0, 2), np.int32)
    _, offsets = sort_on_gpu(ids, 4, layer)
    assert (offsets.cpu().numpy() == 0).all()
    ids = np.array([[0, 9], [-1, 2]], np.int32)
    sorted_ids, offsets = sort_on_gpu(ids, 4, layer)
    offs = offsets.cpu().numpy()
    assert offs.tolist() == [0, 1, 1, 2, 2]
    assert sorted(sorted_ids.cpu().numpy()[:2].tolist()) == [0, 3]


def _expert_sample(ids, n=8):
    """The most and the least loaded experts and some in between."""
    counts = np.bincount(np.asarray(ids).ravel())
    act = np.nonzero(counts)[0]
    order = act[np.argsort(-counts[act], kind="stable")]
    return np.unique(np.concatenate([order[:3], order[-3:], order[np.linspace(0, order.size - 1, n - 6).astype(int)]]))


def _moe_full(wtype, experts, topk, n1, k1, n2, k2, tokens, seed):
    """gate_up (rows by token) and down (rows by pair) at full expert shapes;
    only the experts the router picks get weights (others are never read)."""
    g = 32 if wtype == qg.W_MXFP4 else 128
    mx = wtype == qg.W_MXFP4
    ids = synth.route(synth.rng(seed, 1), tokens, experts, topk)
    active = np.unique(ids)
    print(f"moe wtype={wtype} E={experts} T={tokens} active={active.size}", flush=True)
    up = Layer(wtype, n1, k1, g, seed=seed, experts=experts, active=active)
    print("  gate_up weights ready", flush=True)
    sorted_ids, offsets = sort_on_gpu(ids, experts, up)
    check_sort(ids, experts, sorted_ids, offsets)
    x = Acts(mx, tokens, k1, seed=seed + 1)
    ref = moe_reference(up, x.xdq, ids, True, verbose=True)
    ys = {o: run_moe(up, x, sorted_ids, offsets, tokens, topk, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR, o)
          for o in (qg.O_BF16, qg.O_F32)}
    e1 = [oracle.normwise_error(ys[o], ref) for o in (qg.O_BF16, qg.O_F32)]
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    if mx:
        check_moe_mx_f32(up, x.codes, x.scales, "e4m3", ids, ys[qg.O_F32], qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR,
                         experts=_expert_sample(ids))
    up.drop_wdq()
    del up, ref
    down = Layer(wtype, n2, k2, g, seed=seed + 7, experts=experts, active=active)
    print("  down weights ready", flush=True)
    h = Acts(mx, tokens * topk, k2, seed=seed + 2)
    ref = moe_reference(down, h.xdq, ids, False, verbose=True)
    ys = {o: run_moe(down, h, sorted_ids, offsets, tokens, topk, qg.ROWS_BY_PAIR, qg.ROWS_BY_PAIR, o)
          for o in (qg.O_BF16, qg.O_F32)}
    e2 = [oracle.normwise_error(ys[o], ref) for o in (qg.O_BF16, qg.O_F32)]
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    if mx:
        check_moe_mx_f32(down, h.codes, h.scales, "e4m3", ids, ys[qg.O_F32], qg.ROWS_BY_PAIR, qg.ROWS_BY_PAIR,
                         experts=_expert_sample(ids))
    print(f"  gate_up err bf16/fp32={e1[0]:.3e}/{e1[1]:.3e} down err={e2[0]:.3e}/{e2[1]:.3e}", flush=True)
    assert e1[0] <= TOL_BF16 and e2[0] <= TOL_BF16
    if not mx:
        assert e1[1] <= TOL_F32 and e2[1] <= TOL_F32


def test_moe_w4a16_256_experts_t64():
    _moe_full(qg.W_INT4, 256, 8, 4096, 7168, 7168, 2048, 64, seed=40)


@pytest.mark.parametrize("tokens", [1, 16, 64, 512])
def test_moe_w4a8_128_experts_padding_shape(tokens):
    """(T = 16: 128 pairs, every expert on the grouped skinny kernel, gate_up
    looping over K, the K = 640 down projection on four n-tiles of 2 waves.)"""
    _moe_full(qg.W_MXFP4, 128, 8, 1280, 4096, 4096, 640, tokens, seed=50)


def test_moe_w4a16_256_experts_t16():
    """128 pairs: every expert on the grouped skinny kernel (four n-tiles of
    2 blocks on 4 waves, looping over K = 7168 and K = 2048)."""
    _moe_full(qg.W_INT4, 256, 8, 4096, 7168, 7168, 2048, 16, seed=41)


@pytest.mark.parametrize("wtype", [qg.W_INT4, qg.W_UINT4, qg.W_MXFP4])
def test_moe_tiled_multi_tile_experts(wtype):
    """Skewed routing over 8 experts with hundreds of rows each: experts span
    several 128-row tiles with a partial last tile; small experts take the
    small-tile form (the default split at 1024 pairs).  N = 200 leaves a
    partial column tile."""
    t, e, topk, n, k = 512, 8, 2, 200, 1024
    g = 32 if wtype == qg.W_MXFP4 else 64
    mx = wtype == qg.W_MXFP4
    ids = synth.route(synth.rng(3, wtype), t, e, topk)
    counts = np.bincount(ids.ravel(), minlength=e)
    assert counts.max() > 256 and counts.min() < 64, counts
    layer = Layer(wtype, n, k, g, seed=9, experts=e)
    sorted_ids, offsets = sort_on_gpu(ids, e, layer)
    acts = Acts(mx, t, k, seed=10)
    ref = moe_reference(layer, acts.xdq, ids, True)
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        ys[otype] = run_moe(layer, acts, sorted_ids, offsets, t, topk, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR, otype)
    assert oracle.normwise_error(ys[qg.O_BF16], ref) <= TOL_BF16
    check_f32(layer, acts, ids, ys[qg.O_F32], ref, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    h = Acts(mx, t * topk, k, seed=11)
    y = run_moe(layer, h, sorted_ids, offsets, t, topk, qg.ROWS_BY_PAIR, qg.ROWS_SORTED, qg.O_F32)
    s = sorted_ids.cpu().numpy()
    check_f32(layer, h, ids, y, moe_reference(layer, h.xdq, ids, False)[s], qg.ROWS_BY_PAIR, qg.ROWS_SORTED,
              sorted_ids)


def _moe_sampled(wtype, experts, topk, n, k, tokens, seed, by_token, n_experts_checked=12, atype=None,
                 make_acts=None):
    """Full-size grouped GEMM; the oracle checks every pair of a sample of
    experts (the largest, the smallest and some in between).  atype /
    make_acts(rows, k, seed): another activation type and its inputs."""
    g = 32 if wtype == qg.W_MXFP4 else 128
    mx = wtype == qg.W_MXFP4
    ids = synth.route(synth.rng(seed, 1), tokens, experts, topk)
    counts = np.bincount(ids.ravel(), minlength=experts)
    active = np.nonzero(counts)[0]
    order = active[np.argsort(-counts[active], kind="stable")]
    pick = np.unique(np.concatenate([order[:4], order[-4:],
                                     order[np.linspace(0, order.size - 1, n_experts_checked - 8).astype(int)]]))
    print(f"moe wtype={wtype} E={experts} T={tokens} N={n} K={k} active={active.size} "
          f"max rows={counts.max()} checked experts={pick.tolist()}", flush=True)
    layer = Layer(wtype, n, k, g, seed=seed, experts=experts, active=active, atype=atype)
    sorted_ids, offsets = sort_on_gpu(ids, experts, layer)
    rows = tokens if by_token else tokens * topk
    acts = make_acts(rows, k, seed + 1) if make_acts else Acts(mx, rows, k, seed=seed + 1)
    y = run_moe(layer, acts, sorted_ids, offsets, tokens, topk,
                qg.ROWS_BY_TOKEN if by_token else qg.ROWS_BY_PAIR, qg.ROWS_BY_PAIR, qg.O_BF16)
    flat = ids.reshape(-1)
    worst = 0.0
    for e in pick:
        pairs = np.nonzero(flat == e)[0]
        xr = acts.xdq[pairs // topk if by_token else pairs]
        ref = oracle.gemm(xr, layer.wdq(int(e)))
        layer.drop_wdq()
        err = oracle.normwise_error(y[pairs], ref)
        worst = max(worst, err)
        assert err <= TOL_BF16, (e, err)
    print(f"  worst err={worst:.3e}", flush=True)


def test_moe_w4a16_256_experts_t4096_gate_up_sampled():
    _moe_sampled(qg.W_INT4, 256, 8, 4096, 7168, 4096, seed=60, by_token=True)


def test_moe_w4a16_256_experts_t4096_down_sampled():
    _moe_sampled(qg.W_INT4, 256, 8, 7168, 2048, 4096, seed=61, by_token=False)


@pytest.mark.parametrize("nk,by_token", [((1280, 4096), True), ((4096, 640), False)])
def test_moe_w4a8_128_experts_t4096_sampled(nk, by_token):
    _moe_sampled(qg.W_MXFP4, 128, 8, nk[0], nk[1], 4096, seed=62, by_token=by_token)


@pytest.mark.parametrize("tokens,topk", [(4, 4), (64, 4), (4096, 2)])
@pytest.mark.parametrize("wtype", [qg.W_INT4, qg.W_MXFP4])
def test_moe_long_k(tokens, topk, wtype):
    """K = 14336 (a down projection of a 14336-wide expert): few tokens run the
    skinny kernel, whose workgroups then loop over K; 64 tokens the small
    tiles; 4096 tokens the 128-row tiles and the small tiles.  Every pair
    against the oracle, bf16 and fp32 outputs."""
    experts, n, k = 32, 256, 14336
    g = 32 if wtype == qg.W_MXFP4 else 128
    mx = wtype == qg.W_MXFP4
    ids = synth.route(synth.rng(70, tokens), tokens, experts, topk)
    layer = Layer(wtype, n, k, g, seed=71, experts=experts, active=np.unique(ids))
    print(f"  T={tokens} dispatch {qg.describe_dispatch(layer.w, tokens * topk)}", flush=True)
    sorted_ids, offsets = sort_on_gpu(ids, experts, layer)
    h = Acts(mx, tokens * topk, k, seed=72)
    ref = moe_reference(layer, h.xdq, ids, False)
    ys = {o: run_moe(layer, h, sorted_ids, offsets, tokens, topk, qg.ROWS_BY_PAIR, qg.ROWS_BY_PAIR, o)
          for o in (qg.O_BF16, qg.O_F32)}
    e = [oracle.normwise_error(ys[o], ref) for o in (qg.O_BF16, qg.O_F32)]
    print(f"  err bf16 {e[0]:.3e} fp32 {e[1]:.3e}", flush=True)
    assert e[0] <= TOL_BF16
    if mx:
        check_moe_mx_f32(layer, h.codes, h.scales, "e4m3", ids, ys[qg.O_F32], qg.ROWS_BY_PAIR, qg.ROWS_BY_PAIR,
                         experts=_expert_sample(ids))
    else:
        assert e[1] <= TOL_F32
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
