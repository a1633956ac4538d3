"""qg_gemm_noalloc (qg_gemm with the library's static device scratch instead of
a caller workspace) against qg_gemm, through the C ABI.

Two calls in a row on one device share the static array, the second with a
smaller input: a large-M call whose tiled kernel writes its pre-pass results
into the scratch, then a decode call that splits K across workgroups (arrival
counters and partial tiles in the scratch).  Outputs must equal qg_gemm's bit
for bit (same kernels, same reduction order)."""
import numpy as np
import pytest
import torch

import quantized_gemm_qg_amd as qg
from gpu_harness import Acts, Layer, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _both(layer, acts, m, otype):
    dt = torch.float32 if otype == qg.O_F32 else torch.bfloat16
    y_ws = torch.empty((m, layer.n), dtype=dt, device="cuda")
    wsb = qg.gemm_workspace_size(layer.w, m)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    qg.gemm(layer.w, acts.x, acts.xs, m, layer.k, y_ws, otype, layer.n, ws, wsb)
    y_na = torch.full((m, layer.n), float("nan"), dtype=dt, device="cuda")
    qg.gemm_noalloc(layer.w, acts.x, acts.xs, m, layer.k, y_na, otype, layer.n)
    torch.cuda.synchronize()
    return y_ws, y_na, wsb


# (1024 x 14336: 400 rows take the tiled kernel (group row sums in the
# scratch), 200 rows the skinny kernel's K splits (partials, 6 MB), one row
# the decode kernel's K split in two (64 column tiles))
@pytest.mark.parametrize("wtype,n,k,g,ms", [(qg.W_UINT4, 1024, 14336, 128, (400, 200, 1)),
                                           (qg.W_MXFP4, 512, 8320, 32, (256, 1))])
def test_noalloc_matches_gemm_on_consecutive_calls(wtype, n, k, g, ms):
    layer = Layer(wtype, n, k, g, seed=95)
    mx = wtype == qg.W_MXFP4
    for rnd in range(2):
        for m in ms:
            disp = qg.describe_dispatch(layer.w, m)
            acts = Acts(mx, m, k, seed=96 + m + rnd)
            for otype in (qg.O_F32, qg.O_BF16):
                y_ws, y_na, wsb = _both(layer, acts, m, otype)
                print(f"  round {rnd} M={m} {disp} otype={otype} scratch {wsb} B", flush=True)
                assert wsb > 0  # the call does use scratch
                assert torch.equal(y_ws.view(torch.int16 if otype == qg.O_BF16 else torch.int32),
                                   y_na.view(torch.int16 if otype == qg.O_BF16 else torch.int32)), (m, otype)


def test_noalloc_rejects_calls_beyond_its_scratch():
    layer = Layer(qg.W_INT4, 1024, 14336, 128, seed=97)
    # the tiled kernel's group row sums at 32768 rows: 112 x 32768 x 4 B
    need = qg.gemm_workspace_size(layer.w, 32768)
    assert need > qg.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((32768, 14336), dtype=torch.int16, device="cuda")
    y = torch.empty((32768, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qg.QGError) as e:
        qg.gemm_noalloc(layer.w, x, None, 32768, 14336, y, qg.O_BF16, 1024)
    assert e.value.status == qg.QG_ERR_BUFFER_TOO_SMALL
