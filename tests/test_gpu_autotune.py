"""GPU tests of the dense autotune (qg_gemm_autotune): the fastest candidate
is recorded for its (layer, M bucket), later qg_gemm calls in that bucket run
it and still match the oracle, other buckets keep the heuristics, and
qg_autotune_reset restores them.  The table is process-wide, so every test
resets it when it ends."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qg_amd as qg
from gpu_harness import TOL_BF16, TOL_F32, Acts, Layer, check_mx_f32, err, require_gpu, run_gemm

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    qg.autotune_reset()
    yield
    qg.autotune_reset()


def tune(layer, acts, m, flush=None, reps=4):
    y = torch.empty((m, layer.n), dtype=torch.bfloat16, device="cuda")
    wsb = qg.gemm_autotune_workspace_size(layer.w, m)
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device="cuda")  # contents must not matter
    fb = 0 if flush is None else flush.numel()
    chosen, us = qg.gemm_autotune(layer.w, acts.x, acts.xs, m, layer.k, y, qg.O_BF16, layer.n, ws, wsb,
                                  flush, fb, reps)
    torch.cuda.synchronize()
    return chosen, us


@pytest.mark.parametrize("wtype,n,k,g,m", [(qg.W_UINT4, 4096, 14336, 128, 1), (qg.W_INT3, 2048, 4096, 128, 4),
                                           (qg.W_MXFP4, 1024, 2048, 32, 200), (qg.W_INT4, 512, 1024, 64, 300)])
def test_autotune_records_and_dispatches(wtype, n, k, g, m):
    layer = Layer(wtype, n, k, g, seed=41)
    acts = Acts(wtype == qg.W_MXFP4, m, k, seed=42)
    other_m = 2000 if m < 1000 else 1
    before_other = qg.describe_dispatch(layer.w, other_m)
    flush = torch.empty(320 << 20, dtype=torch.uint8, device="cuda") if m == 1 else None
    chosen, us = tune(layer, acts, m, flush)
    print(f"  {wtype} N={n} K={k} M={m}: heuristic -> tuned {chosen} ({us:.2f} us)", flush=True)
    assert us > 0
    assert qg.describe_dispatch(layer.w, m) == chosen
    assert qg.describe_dispatch(layer.w, other_m) == before_other  # another M bucket keeps the heuristics
    for otype, tol in ((qg.O_BF16, TOL_BF16), (qg.O_F32, TOL_F32)):
        y = run_gemm(layer, acts, m, otype)
        e = err(y, oracle.gemm(acts.xdq, layer.wdq()))
        if otype == qg.O_F32 and layer.mx:
            check_mx_f32(layer, acts, m, y)   # the tuned variant's own accumulation
        else:
            assert e <= tol, (otype, e)
    qg.autotune_reset()
    assert qg.describe_dispatch(layer.w, other_m) == before_other


def test_autotune_entry_serves_its_bucket_only_when_valid():
    # a decode-kernel entry tuned at M = 1 (bucket "1") is not used for M = 2
    # (bucket "2-4"); tuning M = 3 gives that bucket its own entry
    layer = Layer(qg.W_UINT4, 4096, 4096, 128, seed=43)
    acts = Acts(False, 4, 4096, seed=44)
    h2 = qg.describe_dispatch(layer.w, 2)
    a1 = Acts(False, 1, 4096, seed=45)
    c1, _ = tune(layer, a1, 1)
    assert qg.describe_dispatch(layer.w, 1) == c1
    assert qg.describe_dispatch(layer.w, 2) == h2
    c3, _ = tune(layer, acts, 3)
    assert qg.describe_dispatch(layer.w, 2) == c3 and qg.describe_dispatch(layer.w, 4) == c3
    y = run_gemm(layer, acts, 4, qg.O_F32)
    assert err(y, oracle.gemm(acts.xdq, layer.wdq())) <= TOL_F32


def test_batch_invariant_ignores_the_table():
    layer = Layer(qg.W_INT4, 384, 1024, 128, seed=46)
    acts = Acts(False, 64, 1024, seed=47)

    def inv():
        y = torch.empty((64, 384), dtype=torch.float32, device="cuda")
        wsb = qg.gemm_workspace_size_ex(layer.w, 64, qg.GEMM_BATCH_INVARIANT)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        qg.gemm_ex(layer.w, acts.x, None, 64, 1024, y, qg.O_F32, 384, ws, wsb, qg.GEMM_BATCH_INVARIANT)
        torch.cuda.synchronize()
        return y.cpu()
    before = inv()
    tune(layer, acts, 64)
    assert torch.equal(inv(), before)


def test_autotune_entries_are_per_activation_type():
    """Two MXFP4 layers of one shape, one with MXFP8 and one with bf16
    activations: tuning one leaves the other on its heuristics."""
    n, k, m = 1024, 2048, 200
    a8 = Layer(qg.W_MXFP4, n, k, 32, seed=48)
    a16 = Layer(qg.W_MXFP4, n, k, 32, seed=48, atype=qg.A_BF16)
    h16 = qg.describe_dispatch(a16.w, m)
    chosen, _ = tune(a8, Acts(True, m, k, seed=49), m)
    assert qg.describe_dispatch(a8.w, m) == chosen
    assert qg.describe_dispatch(a16.w, m) == h16
    acts = Acts(False, m, k, seed=50)
    y = run_gemm(a16, acts, m, qg.O_F32)
    assert err(y, oracle.gemm(acts.xdq, a16.wdq())) <= TOL_F32


# ---------------------------------------------------------------------------
# MoE autotune (qg_moe_autotune)
# ---------------------------------------------------------------------------

def _moe_inputs(wtype, t, e, topk, n, k, seed):
    import synth
    from test_gpu_moe import sort_on_gpu
    g = 32 if wtype == qg.W_MXFP4 else 128
    ids = synth.route(synth.rng(seed, wtype), t, e, topk)
    layer = Layer(wtype, n, k, g, seed=seed + 1, experts=e)
    sorted_ids, offsets = sort_on_gpu(ids, e, layer)
    acts = Acts(wtype == qg.W_MXFP4, t, k, seed=seed + 2)
    return ids, layer, sorted_ids, offsets, acts


@pytest.mark.parametrize("wtype", [qg.W_UINT4, qg.W_MXFP4])
def test_moe_autotune_records_and_dispatches(wtype):
    """The tuned plan is the one qg_describe_moe_dispatch then names for the
    pair-count bucket, qg_moe_gemm runs it against the oracle (MX: bit for
    bit against the MFMA model of the plan's kernels), another bucket keeps
    the heuristic, and qg_autotune_reset restores it."""
    from test_gpu_moe import check_f32, run_moe
    t, e, topk, n, k = 300, 8, 2, 256, 1024
    ids, layer, sorted_ids, offsets, acts = _moe_inputs(wtype, t, e, topk, n, k, seed=70)
    heur = qg.describe_moe_dispatch(layer.w, t, topk)
    other = qg.describe_moe_dispatch(layer.w, 3, topk)
    y = torch.empty((t * topk, n), dtype=torch.bfloat16, device="cuda")
    wsb = qg.moe_autotune_workspace_size(layer.w, t, topk)
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device="cuda")  # contents must not matter
    flush = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    chosen, us = qg.moe_autotune(layer.w, acts.x, acts.xs, qg.ROWS_BY_TOKEN, sorted_ids, offsets, t, topk, y,
                                 qg.O_BF16, qg.ROWS_BY_PAIR, ws, wsb, flush, flush.numel(), 3)
    torch.cuda.synchronize()
    print(f"  heuristic: {heur}\n  chosen: {chosen} ({us:.1f} us)", flush=True)
    assert us > 0
    assert qg.describe_moe_dispatch(layer.w, t, topk) == chosen
    assert qg.describe_moe_dispatch(layer.w, 3, topk) == other  # another bucket
    ref = oracle.moe_gemm(layer.wdq, acts.xdq, ids, rows_by_token=True)
    ys = {o: run_moe(layer, acts, sorted_ids, offsets, t, topk, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR, o)
          for o in (qg.O_BF16, qg.O_F32)}
    assert oracle.normwise_error(ys[qg.O_BF16], ref) <= TOL_BF16
    check_f32(layer, acts, ids, ys[qg.O_F32], ref, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR)
    qg.autotune_reset()
    assert qg.describe_moe_dispatch(layer.w, t, topk) == heur


def test_moe_autotune_every_candidate_is_correct():
    """Each plan the tuner may pick, forced through the overrides, matches the
    oracle (the candidates are the same kernel forms)."""
    t, e, topk, n, k = 200, 8, 2, 128, 512
    ids, layer, sorted_ids, offsets, acts = _moe_inputs(qg.W_MXFP4, t, e, topk, n, k, seed=80)
    _every_plan(layer, acts, ids, sorted_ids, offsets, t, topk, ("128", "256"))


def test_moe_autotune_every_candidate_is_correct_integer():
    """The same for an integer format (the small tiles compute the group row
    sums of X themselves when no 128-row tile runs)."""
    t, e, topk, n, k = 200, 8, 2, 128, 512
    ids, layer, sorted_ids, offsets, acts = _moe_inputs(qg.W_UINT4, t, e, topk, n, k, seed=81)
    _every_plan(layer, acts, ids, sorted_ids, offsets, t, topk, ("128",))


def _every_plan(layer, acts, ids, sorted_ids, offsets, t, topk, bns):
    from test_gpu_moe import check_f32, run_moe
    ref = oracle.moe_gemm(layer.wdq, acts.xdq, ids, rows_by_token=True)
    for r in ("0", "16", "128", "1073741824"):  # (the last: every expert on the small tiles)
        for small in ("0", "1"):
            for bn in bns:
                qg.clear_overrides()
                qg.set_override("QG_MOE_TILED_MIN", r)
                qg.set_override("QG_MOE_SMALL", small)
                qg.set_override("QG_MOE_MX_BN", bn)
                print(f"  {qg.describe_moe_dispatch(layer.w, t, topk)}", flush=True)
                y = run_moe(layer, acts, sorted_ids, offsets, t, topk, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR, qg.O_F32)
                check_f32(layer, acts, ids, y, ref, qg.ROWS_BY_TOKEN, qg.ROWS_BY_PAIR)
    qg.clear_overrides()
