"""GPU parity of the activation-side entry points (qg_quantize_mxfp8,
qg_silu_mul, qg_moe_combine) against the CPU oracle, through the C ABI.

* MXFP8 codes and scales are integer results: compared bit-exactly, over every
  finite bf16 pattern, over blocks whose maxima walk every scale exponent the
  bf16 range produces, and on N(0, 1) rows at the W4A8 GEMM shape.
* SiLU-gated products (fp32 arithmetic, bf16 output): elementwise within one
  bf16 rounding plus fp32 exp error (2^-8 relative), and normwise <= 2e-2.
  The MXFP8 form is checked against the oracle's product within the bf16
  rounding plus the e4m3 step of its block, and bit-exactly against the
  oracle's quantization of the bf16 form.
* Combine: fp32 output normwise <= 1e-5; bf16 output <= 2e-2 normwise and one
  bf16 rounding elementwise.
* A small MoE layer chained through the library (quantize -> gate_up ->
  SiLU-gated product -> down -> combine) against the oracle's chain.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_qg_amd as qg
import synth
from gpu_harness import TOL_BF16, TOL_F32, Acts, Layer, require_gpu, to_dev
from oracle import formats as F
from oracle import quantize as Q

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def gpu_quantize(xbits: np.ndarray, ldx=None, ldq=None, qs_off=0):
    rows, k = xbits.shape
    ldx = ldx or k
    ldq = ldq or k
    xpad = np.zeros((rows, ldx), dtype=np.uint16)
    xpad[:, :k] = xbits
    x = to_dev(xpad)
    q = torch.full((rows, ldq), 0xAA, dtype=torch.uint8, device="cuda")
    # qs_off places the scale array at an odd or 2-byte offset; the bytes
    # around it must stay untouched
    qbuf = torch.full((rows * (k // 32) + 2 * qs_off,), 0xAA, dtype=torch.uint8, device="cuda")
    qs = qbuf[qs_off:qs_off + rows * (k // 32)].view(rows, k // 32)
    qg.quantize_mxfp8(x, rows, k, ldx, q, ldq, qs)
    torch.cuda.synchronize()
    qn = q.cpu().numpy()
    assert np.all(qn[:, k:] == 0xAA)  # padding columns untouched
    qb = qbuf.cpu().numpy()
    assert np.all(qb[:qs_off] == 0xAA) and np.all(qb[qs_off + rows * (k // 32):] == 0xAA)
    return qn[:, :k], qs.cpu().numpy()


def check_quantize(xbits, **kw):
    c, s = gpu_quantize(xbits, **kw)
    rc, rs = Q.quantize_mxfp8_bf16(xbits)
    bad = np.nonzero(c != rc)
    assert np.array_equal(s, rs), np.nonzero(s != rs)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], xbits[bad][:5], c[bad][:5], rc[bad][:5])


def test_quantize_every_finite_bf16_pattern():
    pats = np.arange(65536, dtype=np.uint32)
    finite = pats[((pats >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    r = np.random.default_rng(21)
    x = r.permutation(finite)
    x = x[: (x.size // 512) * 512].reshape(-1, 512)
    print(f"  {x.size} patterns in {x.shape[0]} rows", flush=True)
    check_quantize(x)


def test_quantize_every_scale_exponent():
    # block maximum 2^(E + 8) for every E the bf16 range gives (-127 clamp
    # included), the other 31 values random patterns within 12 binades below
    # it (e4m3 normals, subnormals, ties and values that round to zero)
    r = np.random.default_rng(22)
    rows = []
    for ef in range(1, 255):                      # exponent field of the maximum
        blk = np.empty((64, 32), dtype=np.uint32)
        lo = max(ef - 12, 0)
        e = r.integers(lo, ef + 1, size=(64, 32))
        m = r.integers(0, 128, size=(64, 32))
        m = np.where(e == ef, np.minimum(m, 0), m)  # stay <= the maximum
        blk[:] = (r.integers(0, 2, size=(64, 32)) << 15) | (e << 7) | m
        blk[:, r.integers(0, 32)] = ef << 7
        rows.append(blk.reshape(8, 256))
    # blocks whose maximum is a bf16 subnormal (scale clamped at 2^-127)
    sub = r.integers(0, 128, size=(64, 256)).astype(np.uint32) | (r.integers(0, 2, size=(64, 256)) << 15)
    rows.append(sub)
    x = np.concatenate(rows).astype(np.uint16)
    check_quantize(x)
    # all-zero and signed-zero blocks
    z = np.zeros((4, 64), dtype=np.uint16)
    z[1, :] = 0x8000
    check_quantize(z)


@pytest.mark.parametrize("rows,k,ldx,ldq,qs_off", [(1, 32, None, None, 0), (3, 96, 104, 104, 0),
                                                   (37, 4096, None, 4112, 0), (4096, 4096, None, None, 0),
                                                   (5, 1024, None, None, 1), (9, 1536, None, None, 2)])
def test_quantize_normal_rows(rows, k, ldx, ldq, qs_off):
    r = synth.rng(23, rows)
    check_quantize(synth.x_bf16(r, rows, k), ldx=ldx, ldq=ldq, qs_off=qs_off)


def test_quantize_then_w4a8_gemm():
    m, n, k = 300, 512, 1024
    r = synth.rng(24, 0)
    xb = synth.x_bf16(r, m, k)
    c, s = gpu_quantize(xb)
    layer = Layer(qg.W_MXFP4, n, k, 32, seed=24)
    acts = Acts(True, m, k, values=Q.quantize_mxfp8_bf16(xb))  # the oracle's codes
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws_bytes = qg.gemm_workspace_size(layer.w, m)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    qg.gemm(layer.w, to_dev(c), to_dev(s), m, k, y, qg.O_BF16, n, ws, ws_bytes)
    torch.cuda.synchronize()
    yref = oracle.gemm(acts.xdq, layer.wdq())
    e = oracle.normwise_error(y.float().cpu().numpy().astype(np.float64), yref)
    print(f"  quantize -> W4A8 err {e:.3e}", flush=True)
    assert e <= TOL_BF16


def _gu(rows, inter, f32, seed):
    r = synth.rng(seed, 3)
    v = r.normal(0.0, 2.0, size=(rows, 2 * inter))
    if f32:
        return v.astype(np.float32), v.astype(np.float32).astype(np.float64)
    b = synth.f32_to_bf16_bits(v.astype(np.float32))
    return b, F.decode_bf16(b)


def _silu_gpu(gu_host, f32, rows, inter, mx, ldgu=None):
    ldgu = ldgu or 2 * inter
    if ldgu != 2 * inter:
        pad = np.zeros((rows, ldgu), dtype=gu_host.dtype)
        pad[:, :2 * inter] = gu_host
        gu_host = pad
    gu = to_dev(gu_host)
    if mx:
        h = torch.empty((rows, inter), dtype=torch.uint8, device="cuda")
        hs = torch.empty((rows, inter // 32), dtype=torch.uint8, device="cuda")
    else:
        h = torch.empty((rows, inter), dtype=torch.bfloat16, device="cuda")
        hs = None
    qg.silu_mul(gu, qg.O_F32 if f32 else qg.O_BF16, rows, inter, ldgu, h, qg.A_MXFP8 if mx else qg.A_BF16,
                inter, hs)
    torch.cuda.synchronize()
    if mx:
        return h.cpu().numpy(), hs.cpu().numpy()
    return h.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("rows,inter,ldgu", [(1, 8, None), (7, 40, 96), (512, 2048, None)])
def test_silu_mul_bf16(f32, rows, inter, ldgu):
    g, gv = _gu(rows, inter, f32, 25 + rows)
    h = _silu_gpu(g, f32, rows, inter, False, ldgu)
    ref = Q.silu_mul(gv, inter)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-37
    worst = np.max(np.abs(h - ref) - bound)
    assert worst <= 0, worst
    assert oracle.normwise_error(h, ref) <= TOL_BF16


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("rows,inter", [(256, 640), (96, 2048)])
def test_silu_mul_mxfp8(f32, rows, inter):
    g, gv = _gu(rows, inter, f32, 26)
    c, s = _silu_gpu(g, f32, rows, inter, True)
    deq = Q.dequantize_mxfp8(c, s)
    ref = Q.silu_mul(gv, inter)
    X = np.repeat(F.decode_e8m0(s), 32, axis=-1)
    # bf16 rounding of the product (<= 2^-8 relative with the fp32 exp), then
    # the e4m3 step of the block (<= 16 X, < 64 X where it saturates)
    assert np.all(np.abs(deq - ref) <= 2.0 ** -8 * np.abs(ref) + 64 * X)
    amax = np.abs(ref.reshape(rows, -1, 32)).max(axis=-1)
    ratio = amax / F.decode_e8m0(s)
    assert np.all((ratio >= 255) & (ratio < 513))  # the scale rule, up to the bf16 rounding of the maximum
    # (no normwise 2e-2 bound here: an e4m3 element alone errs by up to 2^-4
    # of its value, 1/8 where the block maximum saturates)
    # the MXFP8 form is the bf16 form quantized
    hb = _silu_gpu(g, f32, rows, inter, False)
    hbits = synth.f32_to_bf16_bits(hb.astype(np.float32))
    rc, rs = Q.quantize_mxfp8_bf16(hbits)
    assert np.array_equal(c, rc) and np.array_equal(s, rs)


@pytest.mark.parametrize("y_f32,out_f32,bias", [(False, False, False), (False, True, True), (True, True, False),
                                                (True, False, True)])
@pytest.mark.parametrize("tokens,topk,n", [(1, 1, 8), (5, 3, 40), (256, 8, 7168)])
def test_moe_combine(y_f32, out_f32, bias, tokens, topk, n):
    r = synth.rng(27, tokens)
    yv = r.normal(0, 1, size=(tokens * topk, n)).astype(np.float32)
    if y_f32:
        yh, yref = yv, yv.astype(np.float64)
    else:
        yh = synth.f32_to_bf16_bits(yv)
        yref = F.decode_bf16(yh)
    w = r.dirichlet(np.ones(topk), size=tokens).astype(np.float32)
    b = synth.f32_to_bf16_bits(r.normal(0, 0.1, size=n).astype(np.float32)) if bias else None
    out = torch.empty((tokens, n), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    qg.moe_combine(to_dev(yh), qg.O_F32 if y_f32 else qg.O_BF16, n, to_dev(w), tokens, topk, n,
                   None if b is None else to_dev(b), out, qg.O_F32 if out_f32 else qg.O_BF16, n)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    ref = Q.moe_combine(yref, w.astype(np.float64), topk, None if b is None else F.decode_bf16(b))
    mag = (np.abs(yref).reshape(tokens, topk, n) * w[:, :, None]).sum(axis=1) + (0 if b is None else 0.1)
    fp32_slack = 2.0 ** -20 * mag
    if out_f32:
        assert np.all(np.abs(o - ref) <= fp32_slack)
        assert oracle.normwise_error(o, ref) <= TOL_F32
    else:
        assert np.all(np.abs(o - ref) <= 2.0 ** -8 * np.abs(ref) + fp32_slack)
        assert oracle.normwise_error(o, ref) <= TOL_BF16


def _sort(ids, experts, layer):
    t, topk = ids.shape
    sorted_ids = torch.full((t * topk,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.empty(experts + 1, dtype=torch.int32, device="cuda")
    ws_bytes = qg.moe_workspace_size(layer.w, t, topk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    qg.moe_sort(to_dev(ids.astype(np.int32)), t, topk, experts, sorted_ids, offsets, ws, ws_bytes)
    return sorted_ids, offsets


def _moe(layer, x, xs, x_rows, sorted_ids, offsets, t, topk, otype=qg.O_BF16):
    y = torch.empty((t * topk, layer.n), dtype=torch.float32 if otype == qg.O_F32 else torch.bfloat16,
                    device="cuda")
    ws_bytes = qg.moe_workspace_size(layer.w, t, topk)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    qg.moe_gemm(layer.w, x, xs, x_rows, sorted_ids, offsets, t, topk, y, otype, qg.ROWS_BY_PAIR, ws, ws_bytes)
    return y


@pytest.mark.parametrize("mx", [False, True])
def test_moe_layer_chain(mx):
    """x (bf16) -> [MXFP8] -> gate_up -> SiLU-gated product [-> MXFP8] -> down -> combine."""
    experts, topk, t, hidden, inter = 8, 2, 96, 512, 256
    wt = qg.W_MXFP4 if mx else qg.W_INT4
    g = 32 if mx else 128
    w13 = Layer(wt, 2 * inter, hidden, g, seed=28, experts=experts)
    w2 = Layer(wt, hidden, inter, g, seed=29, experts=experts)
    r = synth.rng(30, 0)
    xb = synth.x_bf16(r, t, hidden)
    ids = synth.route(r, t, experts, topk)
    wts = r.dirichlet(np.ones(topk), size=t).astype(np.float32)
    sorted_ids, offsets = _sort(ids, experts, w13)
    if mx:
        xq = torch.empty((t, hidden), dtype=torch.uint8, device="cuda")
        xs = torch.empty((t, hidden // 32), dtype=torch.uint8, device="cuda")
        qg.quantize_mxfp8(to_dev(xb), t, hidden, hidden, xq, hidden, xs)
        gu = _moe(w13, xq, xs, qg.ROWS_BY_TOKEN, sorted_ids, offsets, t, topk, qg.O_F32)
        h = torch.empty((t * topk, inter), dtype=torch.uint8, device="cuda")
        hs = torch.empty((t * topk, inter // 32), dtype=torch.uint8, device="cuda")
        qg.silu_mul(gu, qg.O_F32, t * topk, inter, 2 * inter, h, qg.A_MXFP8, inter, hs)
    else:
        gu = _moe(w13, to_dev(xb), None, qg.ROWS_BY_TOKEN, sorted_ids, offsets, t, topk, qg.O_F32)
        h = torch.empty((t * topk, inter), dtype=torch.bfloat16, device="cuda")
        hs = None
        qg.silu_mul(gu, qg.O_F32, t * topk, inter, 2 * inter, h, qg.A_BF16, inter)
    y = _moe(w2, h, hs, qg.ROWS_BY_PAIR, sorted_ids, offsets, t, topk, qg.O_F32)
    out = torch.empty((t, hidden), dtype=torch.bfloat16, device="cuda")
    qg.moe_combine(y, qg.O_F32, hidden, to_dev(wts), t, topk, hidden, None, out, qg.O_BF16, hidden)
    torch.cuda.synchronize()
    # oracle chain in float64
    xv = F.decode_bf16(xb)
    if mx:
        xv = Q.dequantize_mxfp8(*Q.quantize_mxfp8(xv))
    gref = oracle.moe_gemm(w13.wdq, xv, ids, rows_by_token=True)
    # H as the library hands it to the down projection: rounded to bf16, then
    # (MX) quantized; computed here from the oracle's exact gate_up output
    href = oracle.round_bf16(Q.silu_mul(gref, inter))
    if mx:
        href = Q.dequantize_mxfp8(*Q.quantize_mxfp8(href))
    yref = oracle.moe_gemm(w2.wdq, href, ids, rows_by_token=False)
    ref = Q.moe_combine(yref, wts.astype(np.float64), topk)
    e = oracle.normwise_error(out.float().cpu().numpy().astype(np.float64), ref)
    print(f"  MoE chain ({'MX' if mx else 'INT4'}) err {e:.3e}", flush=True)
    assert e <= TOL_BF16
