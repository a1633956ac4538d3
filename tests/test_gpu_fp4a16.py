"""GPU parity of MXFP4 weights x bf16 activations (e2m1 codes, e8m0 scale per
32 along K, bf16 activations) through the C ABI against the CPU oracle.

The kernels turn each code into the exact bf16 value e2m1 x 2^(e - 127) and
run the bf16 MFMA on it, so the fp32 accumulators meet the integer formats'
1e-5 normwise bound and one-hot rows return the dequantized weights bit for
bit."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qg_amd as qg
import synth
from gpu_harness import TOL_BF16, TOL_F32, Acts, assert_bf16_is_rne, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class Fp4Layer:
    def __init__(self, n, k, seed, experts=1):
        self.n, self.k, self.experts = n, k, experts
        self.desc = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=qg.A_BF16, num_experts=experts)
        self.buf = torch.empty(qg.packed_size(self.desc), dtype=torch.uint8, device="cuda")
        self.std = []
        for e in range(experts):
            codes, sc, _ = synth.mx_weights(synth.rng(seed, 500 + e), n, k)
            self.std.append((codes, sc))
            self.w = qg.preprocess(self.desc, codes, sc, None, self.buf, expert_begin=e, expert_count=1)

    def wdq(self, e=0):
        codes, sc = self.std[e]
        return oracle.dequant_weights(qg.W_MXFP4, codes, sc, None, self.k, 32)


def run(layer, x, m, otype):
    y = torch.empty((m, layer.n), dtype=torch.float32 if otype == qg.O_F32 else torch.bfloat16, device="cuda")
    wsb = qg.gemm_workspace_size(layer.w, m)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    qg.gemm(layer.w, x, None, m, layer.k, y, otype, layer.n, ws, wsb)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,n,k", [(16, 256, 512), (1, 200, 640), (37, 136, 544), (300, 264, 1024),
                                   (4, 4096, 14336), (1, 14336, 4096), (8, 264, 1536), (3, 72, 512)])
def test_fp4_bf16_dense(m, n, k):
    layer = Fp4Layer(n, k, seed=m + n)
    acts = Acts(False, m, k, seed=k)
    print(f"  M={m} N={n} K={k}: {qg.describe_dispatch(layer.w, m)}", flush=True)
    expect = ("a16_tiled" if m >= 256 and k % 128 == 0 else
              "a16_decode" if m <= 16 and k % 512 == 0 else "a16_skinny")
    assert expect in qg.describe_dispatch(layer.w, m)
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {}
    for otype, tol in ((qg.O_BF16, TOL_BF16), (qg.O_F32, TOL_F32)):
        e = oracle.normwise_error(ys.setdefault(otype, run(layer, acts.x, m, otype)), yref)
        assert e <= tol, (otype, e)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])


def test_fp4_bf16_identity_rows_exact():
    n, k, m = 136, 640, 16
    layer = Fp4Layer(n, k, seed=5)
    wdq = layer.wdq()
    for c0 in range(0, k, 16 * 8):
        bits = np.zeros((m, k), np.uint16)
        cols = c0 + np.arange(m) * 7 % 128
        bits[np.arange(m), cols] = 0x3F80
        y = run(layer, to_dev(bits), m, qg.O_F32)
        for i in range(m):
            ref = wdq[:, cols[i]]
            bad = np.nonzero(y[i] != ref)[0]
            assert bad.size == 0, (c0, i, bad.size, bad[:4].tolist(), y[i][bad[:4]].tolist(), ref[bad[:4]].tolist(),
                                   float(np.max(np.abs(y[i] - ref))))


@pytest.mark.parametrize("t,env", [(40, {}), (256, {}), (256, {"QG_MOE_TILED_MIN": "1"}),
                                   (256, {"QG_MOE_TILED_MIN": "0"}),
                                   (256, {"QG_MOE_TILED_MIN": "1000", "QG_MOE_SMALL": "1"}),
                                   (256, {"QG_MOE_TILED_MIN": "1000", "QG_MOE_SMALL": "1", "QG_MOE_SMALL_BM": "32"})])
def test_fp4_bf16_moe(override, t, env):
    """Grouped MXFP4 x bf16: few tokens (skinny kernel), a skewed batch whose
    large experts take the 128-row tiled kernel and the rest the 64-row small
    tiles, every expert on 128-row tiles, none on tiles, and every expert on
    64- or 32-row small tiles."""
    for key, val in env.items():
        override(key, val)
    experts, topk, n, k = 8, 2, 256, 512
    layer = Fp4Layer(n, k, seed=7, experts=experts)
    r = synth.rng(8, 0)
    ids = synth.route(r, t, experts, topk)
    acts = Acts(False, t, k, seed=9)
    d_ids = to_dev(ids.astype(np.int32))
    sorted_ids = torch.empty(t * topk, dtype=torch.int32, device="cuda")
    offsets = torch.empty(experts + 1, dtype=torch.int32, device="cuda")
    wsb = qg.moe_workspace_size(layer.w, t, topk)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    qg.moe_sort(d_ids, t, topk, experts, sorted_ids, offsets, ws, wsb)
    y = torch.empty((t * topk, n), dtype=torch.float32, device="cuda")
    qg.moe_gemm(layer.w, acts.x, None, qg.ROWS_BY_TOKEN, sorted_ids, offsets, t, topk, y, qg.O_F32,
                qg.ROWS_BY_PAIR, ws, wsb)
    torch.cuda.synchronize()
    yref = oracle.moe_gemm(layer.wdq, acts.xdq, ids, rows_by_token=True)
    e = oracle.normwise_error(y.cpu().numpy().astype(np.float64), yref)
    assert e <= TOL_F32, e


@pytest.mark.parametrize("tile", ["128x256", "256x128", "128x128"])
def test_fp4_bf16_tiled_shapes(override, tile):
    """The LDS-tiled kernel (M >= 256) at each dense tile shape, with partial
    row and column tiles."""
    bm, bn = tile.split("x")
    override("QG_TILED_BM", bm)
    override("QG_A16_BN", bn)
    m, n, k = 300, 200, 640
    layer = Fp4Layer(n, k, seed=11)
    assert f"a16_tiled BM={bm} BN={bn}" in qg.describe_dispatch(layer.w, m)
    acts = Acts(False, m, k, seed=12)
    yref = oracle.gemm(acts.xdq, layer.wdq())
    ys = {}
    for otype, tol in ((qg.O_BF16, TOL_BF16), (qg.O_F32, TOL_F32)):
        e = oracle.normwise_error(ys.setdefault(otype, run(layer, acts.x, m, otype)), yref)
        assert e <= tol, (otype, e)
    assert_bf16_is_rne(ys[qg.O_BF16], ys[qg.O_F32])


def test_fp4_bf16_tiled_identity_rows_exact():
    n, k, m = 136, 640, 320
    layer = Fp4Layer(n, k, seed=13)
    wdq = layer.wdq()
    bits = np.zeros((m, k), np.uint16)
    cols = (np.arange(m) * 2 + 1) % k
    bits[np.arange(m), cols] = 0x3F80
    assert "a16_tiled" in qg.describe_dispatch(layer.w, m)
    y = run(layer, to_dev(bits), m, qg.O_F32)
    for i in range(m):
        assert np.array_equal(y[i], wdq[:, cols[i]]), i


def test_fp4_bf16_batch_invariant_rows():
    n, k, mfull = 264, 1024, 300
    layer = Fp4Layer(n, k, seed=15)
    acts = Acts(False, mfull, k, seed=16)

    def inv(rows):
        x = acts.x.index_select(0, torch.as_tensor(rows, device="cuda")).contiguous()
        y = torch.empty((len(rows), n), dtype=torch.float32, device="cuda")
        wsb = qg.gemm_workspace_size_ex(layer.w, len(rows), qg.GEMM_BATCH_INVARIANT)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        qg.gemm_ex(layer.w, x, None, len(rows), k, y, qg.O_F32, n, ws, wsb, qg.GEMM_BATCH_INVARIANT)
        torch.cuda.synchronize()
        return y.cpu()
    full = inv(list(range(mfull)))
    assert oracle.normwise_error(full.numpy().astype(np.float64), oracle.gemm(acts.xdq, layer.wdq())) <= TOL_F32
    for m in (1, 5, 64, 257):
        rows = list(range(3, 3 + m))
        assert torch.equal(inv(rows).view(torch.int32), full[rows].view(torch.int32)), m


@pytest.mark.parametrize("decode", ["1,8", "1,4", "1,8,2"])
def test_fp4_bf16_decode_identity_rows_exact(override, decode):
    """One-hot rows through the decode kernel (activations in LDS; with and
    without a K split) return the dequantized weights bit for bit."""
    override("QG_DECODE", decode)
    n, k, m = 72, 2048, 8
    layer = Fp4Layer(n, k, seed=17)
    assert "a16_decode" in qg.describe_dispatch(layer.w, m)
    wdq = layer.wdq()
    for c0 in range(0, k, 512):
        bits = np.zeros((m, k), np.uint16)
        cols = c0 + (np.arange(m) * 37) % 512
        bits[np.arange(m), cols] = 0x3F80
        wsb = qg.gemm_workspace_size(layer.w, m)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        qg.gemm(layer.w, to_dev(bits), None, m, k, y, qg.O_F32, n, ws, wsb)
        torch.cuda.synchronize()
        y = y.cpu().numpy().astype(np.float64)
        for i in range(m):
            assert np.array_equal(y[i], wdq[:, cols[i]]), (c0, i)
