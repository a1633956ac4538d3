"""GPU parity of W4A4 (MXFP4 weights x MXFP4 activations, the announcement's
"W8A8 / W4A8 / W4A4" section) and of the bf16 -> MXFP4 quantizer, through the
C ABI, against the CPU oracle.

* qg_quantize_mxfp4: codes and scales are integer results, compared bit for
  bit with the oracle (packed two per byte) over every finite bf16 pattern,
  over blocks whose maxima walk every scale exponent of the bf16 range, and
  on N(0, 1) rows with padded leading dimensions.
* qg_gemm on W4A4 layers: below 128 rows the MX skinny kernel, which widens
  each e2m1 fragment exactly to e4m3 in registers, from 128 the MX tiled
  kernel on e2m1 operands;
  ragged N, K % 512 != 0 (scales regrouped by K step) and
  == 0 (scale ring), padded rows, unaligned scales; bf16 output within
  TOL_BF16 of the float64 product of the exact operands, fp32 output bit
  for bit equal to the block-scaled MFMA model (tests/mx_mfma_model.py).
* Batch invariance, the autotuner's choice, and the quantize -> GEMM chain.
* W4A4 MoE (W4A8's dispatch on e2m1 rows: the tiled kernel's e2m1 form,
  its 64-row small tiles, the skinny kernel's in-register widening) in every
  row mode and every split of the experts between kernels.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qg_amd as qg
import synth
from gpu_harness import TOL_BF16, Layer, assert_bf16_is_rne, check_moe_mx_f32, check_mx_f32, require_gpu, to_dev
from oracle import formats as F
from oracle import quantize as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def gpu_quantize4(xbits: np.ndarray, ldx=None, ldq=None):
    rows, k = xbits.shape
    ldx = ldx or k
    ldq = ldq or k
    xpad = np.zeros((rows, ldx), dtype=np.uint16)
    xpad[:, :k] = xbits
    q = torch.full((rows, ldq // 2), 0xAA, dtype=torch.uint8, device="cuda")
    qs = torch.full((rows, k // 32), 0xAA, dtype=torch.uint8, device="cuda")
    qg.quantize_mxfp4(to_dev(xpad), rows, k, ldx, q, ldq, qs)
    torch.cuda.synchronize()
    qn = q.cpu().numpy()
    assert np.all(qn[:, k // 2:] == 0xAA)  # padding bytes untouched
    return qn[:, :k // 2], qs.cpu().numpy()


def check_quantize4(xbits, **kw):
    c, s = gpu_quantize4(xbits, **kw)
    rc, rs = Q.quantize_mxfp4_bf16(xbits)
    rp = Q.pack_e2m1(rc)
    assert np.array_equal(s, rs), np.nonzero(s != rs)
    bad = np.nonzero(c != rp)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], c[bad][:5], rp[bad][:5])


def test_quantize4_every_finite_bf16_pattern():
    pats = np.arange(65536, dtype=np.uint32)
    finite = pats[((pats >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    x = np.random.default_rng(41).permutation(finite)
    x = x[: (x.size // 512) * 512].reshape(-1, 512)
    print(f"  {x.size} patterns in {x.shape[0]} rows", flush=True)
    check_quantize4(x)


def test_quantize4_every_scale_exponent():
    # block maximum 2^(E + 2) for every E the bf16 range gives (the -127 clamp
    # included); the other 31 values within 5 binades below it (every e2m1
    # magnitude, midpoints and values that round to zero)
    r = np.random.default_rng(42)
    rows = []
    for ef in range(1, 255):
        lo = max(ef - 5, 0)
        e = r.integers(lo, ef + 1, size=(64, 32))
        m = r.integers(0, 128, size=(64, 32))
        m = np.where(e == ef, 0, m)  # stay <= the maximum
        blk = ((r.integers(0, 2, size=(64, 32)) << 15) | (e << 7) | m).astype(np.uint32)
        blk[:, r.integers(0, 32)] = ef << 7
        rows.append(blk.reshape(8, 256))
    sub = r.integers(0, 128, size=(64, 256)).astype(np.uint32) | (r.integers(0, 2, size=(64, 256)) << 15)
    rows.append(sub)
    check_quantize4(np.concatenate(rows).astype(np.uint16))
    z = np.zeros((4, 64), dtype=np.uint16)
    z[1, :] = 0x8000
    check_quantize4(z)


@pytest.mark.parametrize("rows,k,ldx,ldq", [(1, 32, None, None), (3, 96, 104, 112), (37, 4096, None, 4160),
                                            (4096, 4096, None, None)])
def test_quantize4_normal_rows(rows, k, ldx, ldq):
    r = synth.rng(43, rows)
    check_quantize4(synth.x_bf16(r, rows, k), ldx=ldx, ldq=ldq)


class A4:
    """MXFP4 activations (from N(0, 1)): packed codes, scales, exact values."""

    def __init__(self, m, k, seed, ldx=None):
        r = synth.rng(seed, 44)
        codes, self.scales = synth.mx_quantize(r.normal(0.0, 1.0, size=(m, k)), "e2m1")
        self.codes, self.a4 = codes, True
        self.xdq = Q.dequantize_mxfp4(codes, self.scales)
        ldx = ldx or k
        packed = np.zeros((m, ldx // 2), dtype=np.uint8)
        packed[:, :k // 2] = Q.pack_e2m1(codes)
        self.ldx = ldx
        self.x = to_dev(packed)
        self.xs = to_dev(self.scales)


def a4_layer(n, k, seed):
    return Layer(qg.W_MXFP4, n, k, 32, seed=seed, atype=qg.A_MXFP4)


def run_a4(layer, acts, m, otype, flags=0):
    y = torch.empty((m, layer.n), dtype=torch.float32 if otype == qg.O_F32 else torch.bfloat16, device="cuda")
    ws_bytes = qg.gemm_workspace_size_ex(layer.w, m, flags)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    qg.gemm_ex(layer.w, acts.x, acts.xs, m, acts.ldx, y, otype, layer.n, ws, ws_bytes, flags)
    torch.cuda.synchronize()
    return y


def check_a4(layer, acts, m, flags=0):
    """bf16 output against the oracle (normwise), fp32 output bit for bit
    against the block-scaled MFMA model, bf16 == RNE(fp32)."""
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        y = ys[otype] = run_a4(layer, acts, m, otype, flags)
        e = oracle.normwise_error(y.float().cpu().numpy().astype(np.float64), yref)
        print(f"  m={m} n={layer.n} k={layer.k} otype={otype} err={e:.3e}", flush=True)
        assert torch.isfinite(y.float()).all()
        if otype == qg.O_BF16:
            assert e <= TOL_BF16, (otype, e)
        elif not flags:
            check_mx_f32(layer, acts, m, y)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])


@pytest.mark.parametrize("m,n,k", [(1, 256, 512), (7, 136, 384), (33, 300, 1024), (127, 512, 2048),
                                   (1, 4096, 14336), (4, 14336, 4096), (130, 300, 1024), (300, 1000, 2048),
                                   (513, 448, 640), (256, 512, 4096)])
def test_w4a4_gemm(m, n, k):
    """Below 128 rows the MX skinny kernel widens the e2m1 fragments to e4m3
    in registers (long K: split over workgroups); from 128 the tiled kernel
    takes the e2m1 operands directly."""
    layer = a4_layer(n, k, seed=m + n)
    assert qg.describe_dispatch(layer.w, m).startswith("mx_skinny" if m < 128 else "mx_tiled")
    check_a4(layer, A4(m, k, seed=m + k), m)


def test_w4a4_skinny_padded_rows_repeat_calls():
    """Padded e2m1 rows through the skinny kernel, two calls on one
    workspace (its split-K counters must be left at zero), then a smaller M."""
    n, k = 512, 8192
    layer = a4_layer(n, k, seed=53)
    ws_bytes = qg.gemm_workspace_size(layer.w, 16)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    print(f"  dispatch {qg.describe_dispatch(layer.w, 16)}", flush=True)
    for m in (16, 16, 3):
        acts = A4(m, k, seed=54 + m, ldx=k + 96)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        qg.gemm(layer.w, acts.x, acts.xs, m, acts.ldx, y, qg.O_F32, n, ws, ws_bytes)
        torch.cuda.synchronize()
        e = oracle.normwise_error(y.cpu().numpy().astype(np.float64), oracle.gemm(acts.xdq, layer.wdq()))
        print(f"  m={m} err={e:.3e}", flush=True)
        check_mx_f32(layer, acts, m, y)


@pytest.mark.parametrize("m,k", [(300, 128), (300, 256), (130, 384), (257, 896)])
def test_w4a4_short_k(m, k):
    """1, 2, 3 and 7 K steps (every remainder of the step count by 4 of the
    kernel's four-step loop), 256- and 128-row tiles."""
    check_a4(a4_layer(136, k, seed=k), A4(m, k, seed=k + 1), m)


def test_w4a4_padded_rows_and_unaligned_scales():
    m, n, k = 300, 200, 1024
    layer = a4_layer(n, k, seed=45)
    acts = A4(m, k, seed=46, ldx=k + 64)
    check_a4(layer, acts, m)
    y_al = run_a4(layer, acts, m, qg.O_F32)
    buf = torch.zeros(acts.xs.numel() + 16, dtype=torch.uint8, device="cuda")
    view = buf[4:4 + acts.xs.numel()].view(acts.xs.shape)
    view.copy_(acts.xs)
    assert view.data_ptr() % 16 == 4
    acts.xs = view
    y_un = run_a4(layer, acts, m, qg.O_F32)
    assert torch.equal(y_al, y_un)


def test_w4a4_batch_invariant():
    n, k = 384, 1024
    layer = a4_layer(n, k, seed=47)
    big = A4(300, k, seed=48)
    y_big = run_a4(layer, big, 300, qg.O_F32, qg.GEMM_BATCH_INVARIANT)
    for m, rows in ((1, [0]), (17, list(range(17)))):
        small = A4(m, k, seed=48)
        small.x, small.xs = big.x[:m].contiguous(), big.xs[:m].contiguous()
        y = run_a4(layer, small, m, qg.O_F32, qg.GEMM_BATCH_INVARIANT)
        assert torch.equal(y, y_big[rows]), m


def test_w4a4_autotune():
    """The tuner times the MX tiled kernel and the skinny kernel; whichever
    it keeps serves the next calls, within parity."""
    m, n, k = 64, 512, 1024
    layer = a4_layer(n, k, seed=49)
    acts = A4(m, k, seed=50)
    qg.autotune_reset()
    try:
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ws_bytes = qg.gemm_autotune_workspace_size(layer.w, m)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        desc, us = qg.gemm_autotune(layer.w, acts.x, acts.xs, m, k, y, qg.O_BF16, n, ws, ws_bytes, reps=3)
        print(f"  chose {desc} ({us:.2f} us)", flush=True)
        assert desc.startswith(("mx_tiled", "mx_skinny")) and us > 0
        assert qg.describe_dispatch(layer.w, m) == desc
        check_a4(layer, acts, m)
    finally:
        qg.autotune_reset()


def test_quantize4_then_w4a4_gemm():
    m, n, k = 300, 512, 1024
    xb = synth.x_bf16(synth.rng(51, 0), m, k)
    c, s = gpu_quantize4(xb)
    layer = a4_layer(n, k, seed=52)
    rc, rs = Q.quantize_mxfp4_bf16(xb)   # the oracle's codes
    xdq = Q.dequantize_mxfp4(rc, rs)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws_bytes = qg.gemm_workspace_size(layer.w, m)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    qg.gemm(layer.w, to_dev(c), to_dev(s), m, k, y, qg.O_BF16, n, ws, ws_bytes)
    torch.cuda.synchronize()
    e = oracle.normwise_error(y.float().cpu().numpy().astype(np.float64), oracle.gemm(xdq, layer.wdq()))
    print(f"  quantize -> W4A4 err {e:.3e}", flush=True)
    assert e <= TOL_BF16
    # MX error of the activations themselves against the bf16 product (e2m1
    # keeps about one significant bit: a loose sanity bound, not a parity one)
    e_q = oracle.normwise_error(y.float().cpu().numpy().astype(np.float64),
                                oracle.gemm(F.decode_bf16(xb), layer.wdq()))
    assert e_q < 0.5


# ---------------------------------------------------------------------------
# W4A4 MoE: W4A8's dispatch on e2m1 rows (every split of the experts between
# the tiled kernel, its small tiles and the skinny kernel)
# ---------------------------------------------------------------------------

def _moe_a4_layer(n, k, experts, seed):
    return Layer(qg.W_MXFP4, n, k, 32, seed=seed, experts=experts, atype=qg.A_MXFP4)


@pytest.mark.parametrize("split", ["skinny", "tiled", "tiled_4waves", "mixed", "mixed_skinny", "small"])
def test_w4a4_moe_all_row_modes(override, split):
    from test_gpu_moe import SPLITS, moe_reference, run_moe, sort_on_gpu
    env = dict(SPLITS["tiled"], QG_MX_WAVES="4") if split == "tiled_4waves" else SPLITS[split]
    for var, val in env.items():
        override(var, val)
    t, e, topk, n, k = 37, 16, 4, 80, 640
    ids = synth.route(synth.rng(60, 0), t, e, topk)
    layer = _moe_a4_layer(n, k, e, seed=61)
    sorted_ids, offsets = sort_on_gpu(ids, e, layer)
    acts = A4(t, k, seed=62)
    ref = moe_reference(layer, acts.xdq, ids, True)
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        y = ys[otype] = run_moe(layer, acts, sorted_ids, offsets, t, topk, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR, otype)
        err = oracle.normwise_error(y, ref)
        print(f"  {split} by-token otype={otype} err={err:.3e}", flush=True)
        if otype == qg.O_BF16:
            assert err <= TOL_BF16
    check_moe_mx_f32(layer, acts.codes, acts.scales, "e2m1", ids, ys[qg.O_F32], qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])
    h = A4(t * topk, k, seed=63)
    y = run_moe(layer, h, sorted_ids, offsets, t, topk, qg.ROWS_BY_PAIR, qg.ROWS_SORTED, qg.O_F32)
    check_moe_mx_f32(layer, h.codes, h.scales, "e2m1", ids, y, qg.ROWS_BY_PAIR, qg.ROWS_SORTED, sorted_ids)
    y = run_moe(layer, h, sorted_ids, offsets, t, topk, qg.ROWS_SORTED, qg.ROWS_BY_PAIR, qg.O_F32)
    check_moe_mx_f32(layer, h.codes, h.scales, "e2m1", ids, y, qg.ROWS_SORTED, qg.ROWS_BY_PAIR, sorted_ids)


def test_w4a4_moe_multi_tile_experts():
    """Skewed routing, experts over several 128-row tiles (tiled kernel) and
    small ones (small tiles), N = 200 with a partial column tile."""
    from test_gpu_moe import moe_reference, run_moe, sort_on_gpu
    t, e, topk, n, k = 512, 8, 2, 200, 1024
    ids = synth.route(synth.rng(64, 0), t, e, topk)
    layer = _moe_a4_layer(n, k, e, seed=65)
    sorted_ids, offsets = sort_on_gpu(ids, e, layer)
    acts = A4(t, k, seed=66)
    ref = moe_reference(layer, acts.xdq, ids, True)
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        y = ys[otype] = run_moe(layer, acts, sorted_ids, offsets, t, topk, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR, otype)
        err = oracle.normwise_error(y, ref)
        print(f"  multi-tile otype={otype} err={err:.3e}", flush=True)
        if otype == qg.O_BF16:
            assert err <= TOL_BF16
    check_moe_mx_f32(layer, acts.codes, acts.scales, "e2m1", ids, ys[qg.O_F32], qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])


@pytest.mark.parametrize("nk", [(3072, 4096), (14336, 4096)])
def test_w4a4_full_size_sampled_rows(nk):
    """(4096, N, 4096) W4A4 at the benchmarked sizes, in the benchmarked
    launch: every output computed, 96 sampled rows (first and last included)
    against the oracle, which computes those rows only."""
    n, k = nk
    m = 4096
    print(f"w4a4 M={m} N={n} K={k}", flush=True)
    layer = a4_layer(n, k, seed=13)
    acts = A4(m, k, seed=13)
    assert qg.describe_dispatch(layer.w, m).startswith("mx_tiled BM=256")
    rows = np.sort(synth.rng(0, 98).choice(m, 96, replace=False))
    rows[0], rows[-1] = 0, m - 1
    yref = oracle.gemm(acts.xdq[rows], layer.wdq())
    ys = {}
    for otype in (qg.O_BF16, qg.O_F32):
        y = ys[otype] = run_a4(layer, acts, m, otype)
        e = oracle.normwise_error(y[rows].float().cpu().numpy().astype(np.float64), yref)
        print(f"  otype={otype} err={e:.3e}", flush=True)
        assert torch.isfinite(y.float()).all()
        if otype == qg.O_BF16:
            assert e <= TOL_BF16
        else:
            check_mx_f32(layer, acts, m, y, rows=rows[:48])
    assert_bf16_is_rne(ys[qg.O_BF16][rows], ys[qg.O_F32][rows])


@pytest.mark.parametrize("env", [{"QG_MX_BN": "256"}, {"QG_MX_BN": "224"}, {"QG_MX_BN": "192"},
                                 {"QG_MX_WAVES": "4"}], ids=lambda e: "-".join(f"{k}={v}" for k, v in e.items()))
@pytest.mark.parametrize("m,n,k", [(256, 128, 1024), (300, 200, 640), (777, 1040, 4096)])
def test_w4a4_tiled_ragged_every_shape(override, env, m, n, k):
    """Every compiled form of the e2m1-operand tiled kernel (256-, 224- and
    192-column tiles with 8 waves; 256 with 4) on partial row and column
    tiles."""
    for var, val in env.items():
        override(var, val)
    layer = a4_layer(n, k, seed=m + 1)
    bn = env.get("QG_MX_BN", "256")
    assert f"mx_tiled BM=256 BN={bn}" == qg.describe_dispatch(layer.w, m)
    check_a4(layer, A4(m, k, seed=m + 2), m)


@pytest.mark.parametrize("nk,by_token", [((1280, 4096), True), ((4096, 640), False)])
def test_w4a4_moe_128_experts_t4096_sampled(nk, by_token):
    """The benchmarked W4A4 MoE layer (E = 128, top-8, T = 4096; gate_up by
    token, down by pair) at full size: every pair of a sample of experts
    against the oracle."""
    from test_gpu_moe import _moe_sampled
    _moe_sampled(qg.W_MXFP4, 128, 8, nk[0], nk[1], 4096, seed=63, by_token=by_token, atype=qg.A_MXFP4,
                 make_acts=lambda rows, k, seed: A4(rows, k, seed))
