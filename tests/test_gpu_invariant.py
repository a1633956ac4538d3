"""GPU tests of the batch-invariant compute option (qg_gemm_ex with
QG_GEMM_BATCH_INVARIANT): each output row must be bit-identical whatever the
number of rows in the call, and the result must still match the oracle
(normwise 2e-2 bf16, 1e-5 / 3e-5 fp32 as for qg_gemm)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qg_amd as qg
from gpu_harness import TOL_BF16, TOL_F32, Acts, Layer, assert_mx_f32, mx_codes, require_gpu

pytestmark = pytest.mark.gpu
INV = qg.GEMM_BATCH_INVARIANT


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def run(layer, acts, rows, otype, flags):
    m = len(rows)
    idx = torch.as_tensor(rows, device="cuda")
    x = acts.x.index_select(0, idx).contiguous()
    xs = acts.xs.index_select(0, idx).contiguous() if acts.xs is not None else None
    y = torch.empty((m, layer.n), dtype=torch.float32 if otype == qg.O_F32 else torch.bfloat16, device="cuda")
    wsb = qg.gemm_workspace_size_ex(layer.w, m, flags)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    qg.gemm_ex(layer.w, x, xs, m, layer.k, y, otype, layer.n, ws, wsb, flags)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("wtype,k,g", [(qg.W_INT4, 1024, 128), (qg.W_UINT4, 1024, 128), (qg.W_INT3, 1024, 128),
                                       (qg.W_UINT3, 512, 64), (qg.W_MXFP4, 1024, 32), (qg.W_MXFP4, 4096, 32),
                                       (qg.W_MXFP4, 1152, 32), (qg.W_UINT4, 1056, 32), (qg.W_MXFP4, 1056, 32)])
def test_rows_do_not_depend_on_m(wtype, k, g):
    n, mfull = 384, 300
    layer = Layer(wtype, n, k, g, seed=31)
    acts = Acts(wtype == qg.W_MXFP4, mfull, k, seed=32)
    for otype in (qg.O_F32, qg.O_BF16):
        full = run(layer, acts, list(range(mfull)), otype, INV)
        yref = oracle.gemm(acts.xdq, layer.wdq())
        e = oracle.normwise_error(full.float().cpu().numpy().astype(np.float64), yref)
        if otype == qg.O_F32 and layer.mx:
            wc, wsc = mx_codes(layer)
            assert_mx_f32(full, acts.codes, acts.scales, wc, wsc, "e4m3", [qg.describe_dispatch(layer.w, mfull, INV)],
                          what="batch-invariant")
        else:
            assert e <= (TOL_F32 if otype == qg.O_F32 else TOL_BF16), e
        fb = full.view(torch.int32 if otype == qg.O_F32 else torch.int16).cpu()
        r = np.random.default_rng(33)
        for m in (1, 3, 16, 17, 64, 129, 255, 256):
            rows = sorted(r.choice(mfull, size=m, replace=False).tolist())
            part = run(layer, acts, rows, otype, INV)
            pb = part.view(torch.int32 if otype == qg.O_F32 else torch.int16).cpu()
            assert torch.equal(pb, fb[rows]), (m, otype)
    print(f"  {qg.describe_dispatch(layer.w, 1)} by default at M=1; invariant rows identical", flush=True)
