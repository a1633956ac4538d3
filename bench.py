"""Benchmark of the quantized GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]

Primary workload (the metric's "weight GB/s at M=1 decode"): dense W4A16
decode -- asymmetric INT4 with uint4 zero points, group 128, bf16 scales, bf16
N(0,1) activations, M = 1.  One step = the two decode GEMMs of an MLP block,
(N, K) = (14336, 4096) then (4096, 14336), one qg_gemm launch each.  Weights
are resident in HBM before timing; consecutive steps read different copies
of the weights (8 rotating copies, 488 MB > the 256 MB MALL), as a decode
pass over distinct layers would.

value = algorithmic weight bytes per step (codes at 0.5 B/weight + bf16 scales
+ 4-bit zero points, unpadded) / step time.

roofline: the dominant kernel's algorithmic bytes per launch / its average
launch duration, from HIP events around a run of back-to-back launches of that
kernel alone on the launch stream.

Unless --quick, the line also carries the other configurations ("extra"):
INT3 and M = 4 / 16 decode, the W4A8 MXFP4 x MXFP8 GEMM at M = 4096, the
activation-side kernels (bf16 -> MXFP8 quantization, the W4A8 GEMM fed from
bf16, the MoE SiLU-gated product and top-k combine), and the MoE grouped
configurations (gate_up + down latency, the routing sort apart).
MoE weights are random bytes written straight into the packed layout on the
device (uniform codes, |N(0, 0.02)| bf16 or e8m0 scales near 2^-7): the kernels
read the same bytes a preprocessed checkpoint would give, and multi-GB expert
sets are ready in seconds; parity tests go through qg_preprocess instead.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0, "fp4": 10100.0}
METRIC = "TFLOPS at M=4096 (W4A16, W4A8-MXFP4) + weight GB/s at M=1 decode, 1 GPU"
ROTATE = 8
MALL_BYTES = 256 << 20
WARM_MS = 50.0  # minimum untimed back-to-back work before each timed configuration


def weight_bytes(n: int, k: int, bits: int, group: int, zp: bool, scale_bytes: int = 2) -> int:
    """Algorithmic bytes of one weight matrix: codes + scales + zero points."""
    g = n * (k // group)
    return n * k * bits // 8 + g * scale_bytes + (g // 2 if zp else 0)


class DenseWeights:
    """`copies` packed copies of one seeded weight matrix on the device."""

    def __init__(self, qg, synth, torch, wtype, n, k, group, seed, copies=ROTATE):
        self.n, self.k, self.group, self.wtype = n, k, group, wtype
        r = synth.rng(seed, 1)
        if wtype == qg.W_MXFP4:
            codes, sc, _ = synth.mx_weights(r, n, k)
            zp = None
        elif wtype in (qg.W_INT4, qg.W_UINT4):
            codes, sc, zp = synth.int4_weights_packed(r, n, k, wtype, group)
        else:
            codes, sc, zp, _ = synth.int_weights(r, n, k, wtype, group)
        self.std = (codes, sc, zp)
        desc = qg.layer_desc(wtype, n, k, group)
        size = qg.packed_size(desc)
        self.bytes = weight_bytes(n, k, synth.WTYPE_BITS[wtype], group, zp is not None,
                                  1 if wtype == qg.W_MXFP4 else 2)
        if copies is None:  # cold: the rotation spans twice the MALL
            copies = max(2, -(-2 * MALL_BYTES // self.bytes))
        # one host repack; the other copies are device copies of the packed bytes
        first = torch.empty(size, dtype=torch.uint8, device="cuda")
        self.bufs, self.ws = [first], [qg.preprocess(desc, codes, sc, zp, first)]
        for _ in range(copies - 1):
            b = first.clone()
            self.ws.append(qg.weight_bind(desc, b, size))
            self.bufs.append(b)


def make_x(qg, synth, torch, mx, m, k, seed):
    r = synth.rng(seed, 2)
    if mx:
        c, s = synth.mx_activations(r, m, k)
        return torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(), (c, s)
    b = synth.x_bf16(r, m, k)
    return torch.from_numpy(b.view(np.int16)).cuda(), None, b


def timed(torch, launch, iters, warmup, warm_ms=WARM_MS):
    """Mean ms per call of `launch(i)` over `iters` back-to-back calls, HIP
    events at both ends on the current stream.  Untimed first: `warmup` calls,
    then more until at least `warm_ms` of back-to-back work has run (the GPU's
    clocks take about 25 ms of sustained load to settle; the first
    milliseconds run up to 15 % slower)."""
    t0 = time.perf_counter()
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    i = warmup
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(8):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(iters):
        launch(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def dense_launcher(qg, torch, wts, x, xs, m):
    y = torch.empty((m, wts.n), dtype=torch.bfloat16, device="cuda")
    ws_bytes = qg.gemm_workspace_size(wts.ws[0], m)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    n = len(wts.ws)
    return lambda i: qg.gemm(wts.ws[i % n], x, xs, m, wts.k, y, qg.O_BF16, wts.n, ws, ws_bytes, stream)


# ---------------------------------------------------------------------------
# MoE configurations
# ---------------------------------------------------------------------------

def fill_packed_random(qg, torch, w, buf, gen):
    """Random valid content written straight into a packed weight buffer."""
    d = w.desc
    E, n, k = d.num_experts, d.n, d.k
    v = buf.view(E, w.expert_stride)
    block = {3: 768, 4: 1024, 8: 2048}[8 if d.wtype == qg.W_FP8 else 3 if d.wtype in (qg.W_INT3, qg.W_UINT3) else 4]
    codes_bytes = w.n_tiles * w.k_blocks * block
    for e0 in range(0, E, 16):  # bounded temporaries
        e1 = min(E, e0 + 16)
        c = torch.randint(0, 256, (e1 - e0, codes_bytes), dtype=torch.uint8, device="cuda", generator=gen)
        if d.wtype == qg.W_FP8:  # no e4m3 NaN codes (S.1111.111)
            c[(c & 0x7F) == 0x7F] -= 1
        v[e0:e1, :codes_bytes] = c
    n_pad = w.n_tiles * 16
    so = w.scales_offset
    if d.wtype == qg.W_FP8:
        # W8A8: fp32 block scales [n_tile][kb_pad] near 2e-2 / 448
        kb_pad = -(-w.k_blocks // 4) * 4
        sc = torch.rand((E, w.n_tiles * kb_pad), device="cuda", generator=gen) * 4e-5 + 2e-5
        v[:, so:so + w.n_tiles * kb_pad * 4] = sc.view(torch.uint8).view(E, -1)
    elif d.wtype == qg.W_MXFP4 and d.atype == qg.A_BF16:
        # bf16 powers of two 2^(e - 127), e near 120, in the integer formats' scale layout
        gp, G = w.groups_padded, k // 32
        s16 = v[:, so:so + n_pad * gp * 2].clone().view(torch.int16).view(E, n_pad, gp)
        e8 = torch.randint(118, 123, (E, n, G), dtype=torch.int16, device="cuda", generator=gen)
        s16[:, :n, :G] = e8 << 7
        v[:, so:so + n_pad * gp * 2] = s16.view(E, -1).view(torch.uint8)
    elif d.wtype == qg.W_MXFP4:
        kb_pad = -(-w.k_blocks // 4) * 4
        sc = v[:, so:so + n_pad * 4 * kb_pad].view(E, n_pad, 4, kb_pad)
        sc[:, :n, :, :k // 128] = torch.randint(118, 123, (E, n, 4, k // 128), dtype=torch.uint8,
                                                device="cuda", generator=gen)
        if k % 128:
            sc[:, :n, :(k % 128) // 32, k // 128] = 120
    else:
        gp, G = w.groups_padded, k // d.group_size
        s16 = v[:, so:so + n_pad * gp * 2].clone().view(torch.int16).view(E, n_pad, gp)
        vals = (torch.randn((E, n, G), device="cuda", generator=gen) * 0.02).abs()
        s16[:, :n, :G] = vals.to(torch.bfloat16).view(torch.int16)
        v[:, so:so + n_pad * gp * 2] = s16.view(E, -1).view(torch.uint8)
        if d.wtype in (qg.W_UINT4, qg.W_UINT3):
            zo = w.zeros_offset
            zw = v[:, zo:zo + n_pad * gp // 2].view(E, n_pad, gp // 2)
            zw[:, :n, :G // 2] = torch.randint(0, 256, (E, n, G // 2), dtype=torch.uint8, device="cuda",
                                               generator=gen)


class MoELayer:
    def __init__(self, qg, torch, wtype, experts, n, k, copies, gen, atype=None):
        g = 32 if wtype == qg.W_MXFP4 else 128
        desc = qg.layer_desc(wtype, n, k, g, num_experts=experts, atype=atype)
        size = qg.packed_size(desc)
        self.n, self.k, self.ws = n, k, []
        self.bufs = []
        for _ in range(copies):
            b = torch.zeros(size, dtype=torch.uint8, device="cuda")
            w = qg.weight_bind(desc, b, size)
            fill_packed_random(qg, torch, w, b, gen)
            self.ws.append(w)
            self.bufs.append(b)


def mx_acts_device(torch, rows, k, gen):
    """MXFP8 activations quantized on the device from N(0,1): per-32 e8m0
    exponent floor(log2 amax) - 8, elements rounded to e4m3 (saturating)."""
    x = torch.randn((rows, k // 32, 32), device="cuda", generator=gen)
    amax = x.abs().amax(dim=2).clamp_min(2.0 ** -100)
    e = torch.floor(torch.log2(amax)) - 8
    q = (x / torch.exp2(e)[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).view(rows, k).contiguous(), (e + 127).to(torch.uint8).contiguous()


def moe_dispatch(qg, w, ids, experts):
    """The library's MoE dispatch rule for this routing, with the number of
    experts on each side of its row threshold."""
    import re
    rule = qg.describe_moe_dispatch(w, ids.shape[0], ids.shape[1])
    m = re.search(r">= (\d+) rows", rule)
    if not m:
        return rule
    counts = np.bincount(ids.ravel(), minlength=experts)
    thr = int(m.group(1))
    return f"{rule} ({int((counts >= thr).sum())} / {int(((counts > 0) & (counts < thr)).sum())} experts)"


def fp8_acts_device(torch, rows, k, block, gen):
    """e4m3 activations from N(0, 1) with fp32 scales per row (block None) or
    per row and 128 K (values near the range a per-block amax / 448 gives)."""
    q = torch.randn((rows, k), device="cuda", generator=gen).to(torch.float8_e4m3fn)
    cols = 1 if block is None else k // block
    s = torch.rand((rows, cols), device="cuda", generator=gen) * 4e-3 + 6e-3
    return q.view(torch.uint8).contiguous(), (s[:, 0] if block is None else s).contiguous()


def bench_moe(qg, synth, torch, name, wtype, experts, topk, n1, k1, n2, k2, tokens, iters, atype=None, tune=False):
    """gate_up + down of one MoE layer (T tokens, top-k routing).  tune: run
    qg_moe_autotune on both GEMMs first (cold caches), time the tuned plans,
    and reset the table afterwards."""
    fp4 = wtype == qg.W_MXFP4 and atype == qg.A_BF16  # MXFP4 weights x bf16 activations
    tok = atype == qg.A_FP8_TOKEN                       # MXFP4 weights x per-token FP8
    f8 = wtype == qg.W_FP8                              # W8A8 block FP8
    mx = wtype == qg.W_MXFP4 and not fp4 and not tok
    g = 32 if wtype == qg.W_MXFP4 else 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    ids = synth.route(synth.rng(7, tokens), tokens, experts, topk)
    active = int(np.unique(ids).size)
    p = tokens * topk
    sb = 1 if wtype == qg.W_MXFP4 else 2
    if f8:
        touched = active * (n1 * k1 + n2 * k2 + 4 * (-(-n1 // 128) * (k1 // 128) + -(-n2 // 128) * (k2 // 128)))
    else:
        touched = active * (weight_bytes(n1, k1, 4, g, False, sb) + weight_bytes(n2, k2, 4, g, False, sb))
    copies = int(min(16, max(1, -(-2 * MALL_BYTES // touched))))
    up = MoELayer(qg, torch, wtype, experts, n1, k1, copies, gen, atype)
    down = MoELayer(qg, torch, wtype, experts, n2, k2, copies, gen, atype)
    d_ids = torch.from_numpy(ids).cuda()
    sorted_ids = torch.empty(p, dtype=torch.int32, device="cuda")
    offsets = torch.empty(experts + 1, dtype=torch.int32, device="cuda")
    wsb = qg.moe_workspace_size(up.ws[0], tokens, topk)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    t_sort = timed(torch, lambda i: qg.moe_sort(d_ids, tokens, topk, experts, sorted_ids, offsets,
                                                ws, wsb, stream), iters, 3)
    if tok or f8:
        x, xs = fp8_acts_device(torch, tokens, k1, 128 if f8 else None, gen)
        h, hs = fp8_acts_device(torch, p, k2, 128 if f8 else None, gen)
    elif mx:
        x, xs = mx_acts_device(torch, tokens, k1, gen)
        h, hs = mx_acts_device(torch, p, k2, gen)
        if atype == qg.A_MXFP4:  # two e2m1 codes per byte
            x, h = x[:, :k1 // 2].contiguous(), h[:, :k2 // 2].contiguous()
    else:
        x = torch.randn((tokens, k1), device="cuda", generator=gen).to(torch.bfloat16)
        h = torch.randn((p, k2), device="cuda", generator=gen).to(torch.bfloat16)
        xs = hs = None
    y1 = torch.empty((p, n1), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((p, n2), dtype=torch.bfloat16, device="cuda")
    chosen = None
    if tune:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        chosen = []
        for L, xx, xxs, xr, yy in ((up, x, xs, qg.ROWS_BY_TOKEN, y1), (down, h, hs, qg.ROWS_BY_PAIR, y2)):
            wsb_t = qg.moe_autotune_workspace_size(L.ws[0], tokens, topk)
            wst = torch.empty(wsb_t, dtype=torch.uint8, device="cuda")
            c, _ = qg.moe_autotune(L.ws[0], xx, xxs, xr, sorted_ids, offsets, tokens, topk, yy, qg.O_BF16,
                                   qg.ROWS_BY_PAIR, wst, wsb_t, flush, flush.numel(), 3)
            chosen.append(c)
            del wst
        del flush
    gws = max(qg.moe_workspace_size(up.ws[0], tokens, topk), qg.moe_workspace_size(down.ws[0], tokens, topk))
    gw = torch.empty(max(gws, 1), dtype=torch.uint8, device="cuda")
    t_up = timed(torch, lambda i: qg.moe_gemm(up.ws[i % copies], x, xs, qg.ROWS_BY_TOKEN, sorted_ids,
                                              offsets, tokens, topk, y1, qg.O_BF16, qg.ROWS_BY_PAIR,
                                              gw, gws, stream), iters, 2)
    t_dn = timed(torch, lambda i: qg.moe_gemm(down.ws[i % copies], h, hs, qg.ROWS_BY_PAIR, sorted_ids,
                                              offsets, tokens, topk, y2, qg.O_BF16, qg.ROWS_BY_PAIR,
                                              gw, gws, stream), iters, 2)
    t = t_up + t_dn
    flops = 2.0 * p * (n1 * k1 + n2 * k2)
    tflops = flops / (t * 1e-3) / 1e12
    gbs = touched / (t * 1e-3) / 1e9
    peak = PEAK_TFLOPS["fp8" if (mx or tok or f8) else "bf16"]
    out = {"tokens": tokens, "active_experts": active, "weight_copies": copies,
           "gate_up_us": round(t_up * 1e3, 2), "down_us": round(t_dn * 1e3, 2),
           "sort_us": round(t_sort * 1e3, 2), "TFLOPS": round(tflops, 2),
           "weight_GBs": round(gbs, 1), "mfma_frac": round(tflops / peak, 4),
           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "dispatch": moe_dispatch(qg, up.ws[0], ids, experts)}
    if tune:
        out["tuned_plans"] = chosen
        qg.autotune_reset()
    del up, down
    torch.cuda.empty_cache()
    print(f"[bench] {name} T={tokens}: {out}", file=sys.stderr, flush=True)
    return out


def bench_stream_ceiling(qg, torch, nbytes=30507008):
    """Plain qg_stream_read of one decode GEMM's weight bytes (30.5 MB), the
    buffers rotating over twice the MALL: the practical single-launch read
    rate that bounds the decode kernels."""
    copies = max(2, -(-2 * MALL_BYTES // nbytes))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(16384, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    t = timed(torch, lambda i: qg.stream_read(bufs[i % copies], nbytes, sink, stream), 200, 20)
    out = {"bytes": nbytes, "us": round(t * 1e3, 2), "GBs": round(nbytes / (t * 1e-3) / 1e9, 1),
           "hbm_frac": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "copies": copies}
    print(f"[bench] stream-read ceiling: {out}", file=sys.stderr, flush=True)
    del bufs
    return out


def bench_moe_large(qg, synth, torch):
    """The MoE configurations at T = 4096 only (for profiling)."""
    return {
        "w4a16_E256_top8_T4096": bench_moe(qg, synth, torch, "moe_w4a16", qg.W_INT4, 256, 8, 4096, 7168, 7168,
                                           2048, 4096, iters=5),
        "w4a8_E128_top8_T4096": bench_moe(qg, synth, torch, "moe_w4a8", qg.W_MXFP4, 128, 8, 1280, 4096, 4096,
                                          640, 4096, iters=5),
    }


def bench_moe_tuned(qg, synth, torch):
    """The W4A16 and W4A8 MoE layers after qg_moe_autotune of both GEMMs."""
    out = {"w4a16_E256_top8_T4096_autotuned": bench_moe(
        qg, synth, torch, "moe_w4a16 tuned", qg.W_INT4, 256, 8, 4096, 7168, 7168, 2048, 4096, iters=5, tune=True)}
    for tokens in (64, 4096):
        out[f"w4a8_E128_top8_T{tokens}_autotuned"] = bench_moe(
            qg, synth, torch, "moe_w4a8 tuned", qg.W_MXFP4, 128, 8, 1280, 4096, 4096, 640, tokens,
            iters=5 if tokens > 512 else 30, tune=True)
    return out


def bench_moe_formats(qg, synth, torch):
    """W8A8 block FP8 and MXFP4 x per-token FP8 on the E = 128 top-8 MoE
    layer (gate_up 1280 x 4096, down 4096 x 640 per expert), T = 1 .. 4096."""
    out = {}
    for tokens in (1, 64, 512, 4096):
        out[f"w8a8_block_fp8_E128_top8_T{tokens}"] = bench_moe(
            qg, synth, torch, "moe_w8a8", qg.W_FP8, 128, 8, 1280, 4096, 4096, 640, tokens,
            iters=5 if tokens > 512 else 30, atype=qg.A_FP8_BLOCK)
        out[f"w4a8_fp8_token_E128_top8_T{tokens}"] = bench_moe(
            qg, synth, torch, "moe_w4a8_token", qg.W_MXFP4, 128, 8, 1280, 4096, 4096, 640, tokens,
            iters=5 if tokens > 512 else 30, atype=qg.A_FP8_TOKEN)
    return out


def cpu_baseline(oracle, shapes, budget_s=15.0):
    """The oracle (decode codes -> dequantize -> float64 GEMM) on host cores,
    on the same decode work, repeated until ~budget_s; weight GB/s."""
    cores = len(os.sched_getaffinity(0))
    done_bytes, t0, reps = 0, time.perf_counter(), 0
    while True:
        for (wtype, codes, sc, zp, n, k, g, xb, nbytes) in shapes:
            oracle.qg_gemm(wtype, codes, sc, zp, n, k, g, oracle.A_BF16, xb)
            done_bytes += nbytes
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(done_bytes / el / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} repetitions of the M=1 decode step (both (N,K) shapes, "
                      f"{2 * reps} GEMMs), {el:.1f} s wall on the host"}


# HBM traffic of the dominant decode kernel, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE passes scaled by the same counters on a copy of known size (see
# the traffic summary under profiles/).  Used only while the kernel sources
# still hash to what was measured.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_w4a16_m1_hbm_traffic.md")
KERNEL_SOURCES = ["qg_kernels.hip", "qg_wave.h", "qg_device.h", "qg_internal.h", "qg_formats.hip"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_gemm_qg_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(n: int, k: int):
    """Bytes per launch of the M = 1 decode GEMM (n, k) recorded for the
    current kernel sources (`traffic_bytes_per_launch_{n}x{k}:`), else None."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    key = f"traffic_bytes_per_launch_{n}x{k}:"
    for line in text.splitlines():
        for kk in ("source_hash:", key):
            if line.strip().startswith(kk):
                vals[kk] = line.split(":", 1)[1].strip().strip("`")
    if vals.get("source_hash:") != kernel_source_hash() or key not in vals:
        return None
    return int(vals[key])


def pmc_workload(qg, synth, torch):
    """A short run for rocprofv3 counter passes: qg_stream_copy of 256 MiB
    (three launches, the calibration), then the two M = 1 decode GEMMs of the
    headline step (dense W4A16 UINT4 + zp, (N, K) = (4096, 14336) then
    (14336, 4096)) 20 times each on rotating weight copies, then the 16-row
    decode GEMMs (UINT4 + zp and INT3, both decode shapes) 20 times each."""
    n_copy = 256 << 20
    src = torch.empty(n_copy, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n_copy, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        qg.stream_copy(dst, src, n_copy, stream)
    torch.cuda.synchronize()
    del src, dst
    print(f"pmc workload: copy {n_copy} B x3, source hash {kernel_source_hash()}", flush=True)
    for n, k in ((4096, 14336), (14336, 4096)):
        L = DenseWeights(qg, synth, torch, qg.W_UINT4, n, k, 128, seed=1)
        x, _, _ = make_x(qg, synth, torch, False, 1, k, seed=11)
        f = dense_launcher(qg, torch, L, x, None, 1)
        for i in range(20):
            f(i)
        torch.cuda.synchronize()
        print(f"pmc workload: decode N={n} K={k} M=1 x20 ({L.bytes} algorithmic bytes per launch): "
              f"{qg.describe_dispatch(L.ws[0], 1)}", flush=True)
        del L
    for wtype, name in ((qg.W_UINT4, "uint4_zp"), (qg.W_INT3, "int3")):
        for i, (n, k) in enumerate([(14336, 4096), (4096, 14336)]):
            L = DenseWeights(qg, synth, torch, wtype, n, k, 128, seed=30 + i)
            x, _, _ = make_x(qg, synth, torch, False, 16, k, seed=56)
            f = dense_launcher(qg, torch, L, x, None, 16)
            for j in range(20):
                f(j)
            torch.cuda.synchronize()
            print(f"pmc workload: decode {name} N={n} K={k} M=16 x20 ({L.bytes} algorithmic weight bytes, "
                  f"{16 * k * 2} activation bytes, {16 * n * 2} output bytes per launch): "
                  f"{qg.describe_dispatch(L.ws[0], 16)}", flush=True)
            del L


def bench_decode_rows(qg, synth, torch, shapes, layers=None):
    """Dense W4A16 decode (UINT4 + zp and INT3, group 128) at M = 1, 4, 8, 16
    on both decode shapes: per-GEMM time, weight GB/s and the M / M=1 time
    ratio.  `layers`: the UINT4 weights already on the device, if any."""
    out = {}
    for wtype, name in ((qg.W_UINT4, "uint4_zp"), (qg.W_INT3, "int3")):
        for i, (n, k) in enumerate(shapes):
            L = (layers[i] if wtype == qg.W_UINT4 and layers is not None
                 else DenseWeights(qg, synth, torch, wtype, n, k, 128, seed=(0 if wtype == qg.W_UINT4 else 30) + i))
            t1 = None
            for mm in (1, 4, 8, 16):
                x, _, _ = make_x(qg, synth, torch, False, mm, k, seed=40 + mm)
                t = timed(torch, dense_launcher(qg, torch, L, x, None, mm), 100, 10)
                t1 = t if mm == 1 else t1
                out[f"decode_{name}_M{mm}_N{n}_K{k}"] = {
                    "us": round(t * 1e3, 2), "weight_GBs": round(L.bytes / (t * 1e-3) / 1e9, 1),
                    "hbm_frac": round(L.bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "vs_M1": round(t / t1, 3), "dispatch": qg.describe_dispatch(L.ws[0], mm)}
            del L
        print(f"[bench] decode rows {name} done", file=sys.stderr, flush=True)
    return out


def bench_formats(qg, synth, torch, shapes):
    """The further weight and activation formats at the decode shapes: WnA16
    integer and e4m3 weights (group 128, bf16 activations) at M = 1 and 16;
    W8A8 block FP8 and MXFP4 x per-token FP8 at M = 1, 16 and 256 (both on
    the skinny kernel).  Weight bytes per GEMM / time, and TFLOPS."""
    out = {}
    stream = torch.cuda.current_stream().cuda_stream

    def run(name, ws, x, xs, m, n, k, nbytes):
        y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        wsb = qg.gemm_workspace_size(ws[0], m)
        wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        t = timed(torch, lambda j: qg.gemm(ws[j % len(ws)], x, xs, m, k, y, qg.O_BF16, n, wsp, wsb, stream),
                  100, 10)
        out[name] = {"us": round(t * 1e3, 2), "weight_GBs": round(nbytes / (t * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "TFLOPS": round(2.0 * m * n * k / (t * 1e-3) / 1e12, 2),
                     "dispatch": qg.describe_dispatch(ws[0], m)}

    for wtype, name in ((qg.W_INT8, "int8"), (qg.W_UINT2, "uint2_zp"), (qg.W_INT1, "int1"), (qg.W_FP8, "e4m3")):
        for i, (n, k) in enumerate(shapes):
            L = DenseWeights(qg, synth, torch, wtype, n, k, 128, seed=90 + i)
            for mm in (1, 16):
                x, _, _ = make_x(qg, synth, torch, False, mm, k, seed=40 + mm)
                run(f"{name}_bf16_M{mm}_N{n}_K{k}", L.ws, x, None, mm, n, k, L.bytes)
            del L
        print(f"[bench] formats {name} done", file=sys.stderr, flush=True)
    for i, (n, k) in enumerate(shapes):
        # W8A8: e4m3 weights, fp32 scale per 128 x 128 block; e4m3 activations,
        # fp32 scale per row and 128 K
        codes, sc = synth.fp8_block_weights(synth.rng(95 + i, 1), n, k)
        desc = qg.layer_desc(qg.W_FP8, n, k, 128, atype=qg.A_FP8_BLOCK)
        first = torch.empty(qg.packed_size(desc), dtype=torch.uint8, device="cuda")
        bufs, ws = [first], [qg.preprocess(desc, codes, sc, None, first)]
        for _ in range(ROTATE - 1):
            bufs.append(first.clone())
            ws.append(qg.weight_bind(desc, bufs[-1], first.numel()))
        nbytes = n * k + sc.size * 4
        for mm in (1, 16, 256):
            c, s_ = synth.fp8_activations(synth.rng(96, mm), mm, k, 128)
            run(f"w8a8_block_fp8_M{mm}_N{n}_K{k}", ws, torch.from_numpy(c).cuda(), torch.from_numpy(s_).cuda(),
                mm, n, k, nbytes)
        del bufs, ws
        # MXFP4 weights x FP8 activations with one fp32 scale per row
        mc, msc, _ = synth.mx_weights(synth.rng(97 + i, 1), n, k)
        desc = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=qg.A_FP8_TOKEN)
        first = torch.empty(qg.packed_size(desc), dtype=torch.uint8, device="cuda")
        bufs, ws = [first], [qg.preprocess(desc, mc, msc, None, first)]
        for _ in range(ROTATE - 1):
            bufs.append(first.clone())
            ws.append(qg.weight_bind(desc, bufs[-1], first.numel()))
        nbytes = weight_bytes(n, k, 4, 32, False, 1)
        for mm in (1, 16, 256):
            c, s_ = synth.fp8_activations(synth.rng(98, mm), mm, k, None)
            run(f"w4a8_fp8_token_M{mm}_N{n}_K{k}", ws, torch.from_numpy(c).cuda(), torch.from_numpy(s_).cuda(),
                mm, n, k, nbytes)
        del bufs, ws
    print(f"[bench] formats W8A8 / per-token W4A8 done", file=sys.stderr, flush=True)
    return out


def cold_copies(qg, torch, desc, codes, sc, nbytes):
    """Packed copies of one weight whose rotation spans twice the MALL (each
    launch reads its weights from HBM): one host repack, device copies."""
    copies = max(2, -(-2 * MALL_BYTES // nbytes))
    first = torch.empty(qg.packed_size(desc), dtype=torch.uint8, device="cuda")
    bufs, wts = [first], [qg.preprocess(desc, codes, sc, None, first)]
    for _ in range(copies - 1):
        b = first.clone()
        bufs.append(b)
        wts.append(qg.weight_bind(desc, b, b.numel()))
    return bufs, wts


def bench_large_m(qg, synth, torch):
    """W4A16 INT4 (g128) and W4A8 MXFP4 x MXFP8 dense GEMMs at M = 4096:
    TFLOPS against the bf16 / fp8 dense MFMA peaks.  Weights rotate over
    copies spanning twice the MALL, so every launch reads them from HBM."""
    extra = {}
    for n, k in ((14336, 4096), (4096, 14336)):
        L = DenseWeights(qg, synth, torch, qg.W_INT4, n, k, 128, seed=60, copies=None)
        x, _, _ = make_x(qg, synth, torch, False, 4096, k, seed=61)
        t = timed(torch, dense_launcher(qg, torch, L, x, None, 4096), 40, 10)
        fl = 2.0 * 4096 * n * k
        extra[f"w4a16_int4_M4096_N{n}_K{k}"] = {
            "us": round(t * 1e3, 1), "TFLOPS": round(fl / (t * 1e-3) / 1e12, 2),
            "bf16_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
            "dispatch": qg.describe_dispatch(L.ws[0], 4096)}
        print(f"[bench] extra w4a16 N={n} K={k}: {extra[f'w4a16_int4_M4096_N{n}_K{k}']}", file=sys.stderr, flush=True)
        del L
    # MXFP4 weights x bf16 activations (tiled kernel, exact bf16 operands)
    n, k = 14336, 4096
    codes, sc, _ = synth.mx_weights(synth.rng(80, 1), n, k)
    desc = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=qg.A_BF16)
    bufs, wts = cold_copies(qg, torch, desc, codes, sc, weight_bytes(n, k, 4, 32, False, 1))
    nw = len(wts)
    x, _, _ = make_x(qg, synth, torch, False, 4096, k, seed=81)
    y = torch.empty((4096, n), dtype=torch.bfloat16, device="cuda")
    wsb = qg.gemm_workspace_size(wts[0], 4096)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    t = timed(torch, lambda i: qg.gemm(wts[i % nw], x, None, 4096, k, y, qg.O_BF16, n, ws, wsb, stream), 40, 10)
    fl = 2.0 * 4096 * n * k
    extra[f"mxfp4_bf16_M4096_N{n}_K{k}"] = {
        "us": round(t * 1e3, 1), "TFLOPS": round(fl / (t * 1e-3) / 1e12, 2),
        "bf16_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
        "dispatch": qg.describe_dispatch(wts[0], 4096)}
    print(f"[bench] extra mxfp4 x bf16: {extra[f'mxfp4_bf16_M4096_N{n}_K{k}']}", file=sys.stderr, flush=True)
    del bufs, wts
    for n in (3072, 14336):
        L = DenseWeights(qg, synth, torch, qg.W_MXFP4, n, 4096, 32, seed=50, copies=None)
        x, xsc, _ = make_x(qg, synth, torch, True, 4096, 4096, seed=51)
        t = timed(torch, dense_launcher(qg, torch, L, x, xsc, 4096), 100, 20)
        fl = 2.0 * 4096 * n * 4096
        extra[f"w4a8_mx_M4096_N{n}_K4096"] = {
            "us": round(t * 1e3, 1), "TFLOPS": round(fl / (t * 1e-3) / 1e12, 2),
            "fp8_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
            "dispatch": qg.describe_dispatch(L.ws[0], 4096)}
        print(f"[bench] extra mx N={n}: {extra[f'w4a8_mx_M4096_N{n}_K4096']}", file=sys.stderr, flush=True)
        del L
    # W4A4: MXFP4 weights x MXFP4 activations (the same MX tiled kernel with
    # e2m1 A operands; fp4 dense MFMA peak)
    for n in (3072, 14336):
        k = 4096
        codes, sc, _ = synth.mx_weights(synth.rng(82, n), n, k)
        desc = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=qg.A_MXFP4)
        bufs, wts = cold_copies(qg, torch, desc, codes, sc, weight_bytes(n, k, 4, 32, False, 1))
        nw = len(wts)
        xc = torch.randint(0, 256, (4096, k // 2), dtype=torch.uint8, device="cuda")
        xs = torch.randint(118, 128, (4096, k // 32), dtype=torch.uint8, device="cuda")
        y = torch.empty((4096, n), dtype=torch.bfloat16, device="cuda")
        wsb = qg.gemm_workspace_size(wts[0], 4096)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        t = timed(torch, lambda i: qg.gemm(wts[i % nw], xc, xs, 4096, k, y, qg.O_BF16, n, ws, wsb, stream), 100, 20)
        fl = 2.0 * 4096 * n * k
        extra[f"w4a4_mx_M4096_N{n}_K{k}"] = {
            "us": round(t * 1e3, 1), "TFLOPS": round(fl / (t * 1e-3) / 1e12, 2),
            "fp4_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_TFLOPS["fp4"], 4),
            "dispatch": qg.describe_dispatch(wts[0], 4096)}
        print(f"[bench] extra w4a4 N={n}: {extra[f'w4a4_mx_M4096_N{n}_K{k}']}", file=sys.stderr, flush=True)
        del bufs, wts
    # W8A8 block FP8 and MXFP4 x per-token FP8 on the tiled kernel (fp8 peak)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(83)
    stream = torch.cuda.current_stream().cuda_stream
    for n in (3072, 14336):
        k = 4096
        for name, atype in (("w8a8_block_fp8", qg.A_FP8_BLOCK), ("w4a8_fp8_token", qg.A_FP8_TOKEN)):
            if atype == qg.A_FP8_BLOCK:
                codes, sc = synth.fp8_block_weights(synth.rng(84, n), n, k)
                desc = qg.layer_desc(qg.W_FP8, n, k, 128, atype=atype)
                nbytes = n * k + sc.size * 4
            else:
                codes, sc, _ = synth.mx_weights(synth.rng(85, n), n, k)
                desc = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=atype)
                nbytes = weight_bytes(n, k, 4, 32, False, 1)
            bufs, wts = cold_copies(qg, torch, desc, codes, sc, nbytes)
            nw = len(wts)
            xc, xs = fp8_acts_device(torch, 4096, k, 128 if atype == qg.A_FP8_BLOCK else None, gen)
            y = torch.empty((4096, n), dtype=torch.bfloat16, device="cuda")
            wsb = qg.gemm_workspace_size(wts[0], 4096)
            ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
            t = timed(torch, lambda i: qg.gemm(wts[i % nw], xc, xs, 4096, k, y, qg.O_BF16, n, ws, wsb, stream),
                      100, 20)
            fl = 2.0 * 4096 * n * k
            key = f"{name}_M4096_N{n}_K{k}"
            extra[key] = {"us": round(t * 1e3, 1), "TFLOPS": round(fl / (t * 1e-3) / 1e12, 2),
                          "fp8_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
                          "dispatch": qg.describe_dispatch(wts[0], 4096)}
            print(f"[bench] extra {key}: {extra[key]}", file=sys.stderr, flush=True)
            del bufs, wts
    return extra


def bench_act(qg, synth, torch):
    """Activation-side kernels at the hot path's shapes (HBM-bound; algorithmic
    bytes read + written per call / time), and the W4A8 / W4A4 GEMMs fed from
    bf16 activations (quantize + GEMM).  Inputs rotate over copies totalling more
    than twice the MALL so each call reads from HBM."""
    extra = {}
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)

    def copies_for(nbytes):
        return int(min(16, max(1, -(-2 * MALL_BYTES // nbytes))))

    def record(name, t, nbytes, **kw):
        gbs = nbytes / (t * 1e-3) / 1e9
        extra[name] = {"us": round(t * 1e3, 2), "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                       "bytes": int(nbytes), **kw}
        print(f"[bench] {name}: {extra[name]}", file=sys.stderr, flush=True)

    # bf16 -> MXFP8, M = 4096, K = 4096 (the W4A8 GEMM's activations)
    m, k = 4096, 4096
    nc = copies_for(m * k * 2)
    xs = [torch.randn((m, k), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(nc)]
    q = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    qs = torch.empty((m, k // 32), dtype=torch.uint8, device="cuda")
    t = timed(torch, lambda i: qg.quantize_mxfp8(xs[i % nc], m, k, k, q, k, qs, stream), 100, 10)
    record("quantize_mxfp8_M4096_K4096", t, m * k * 3 + m * k // 32)
    # W4A8 from bf16 activations: quantize, then the MXFP4 x MXFP8 GEMM
    n = 14336
    L = DenseWeights(qg, synth, torch, qg.W_MXFP4, n, k, 32, seed=50, copies=2)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    wsb = qg.gemm_workspace_size(L.ws[0], m)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")

    def qgemm(i):
        qg.quantize_mxfp8(xs[i % nc], m, k, k, q, k, qs, stream)
        qg.gemm(L.ws[i % 2], q, qs, m, k, y, qg.O_BF16, n, ws, wsb, stream)
    t = timed(torch, qgemm, 50, 10)
    fl = 2.0 * m * n * k
    extra[f"w4a8_from_bf16_M{m}_N{n}_K{k}"] = {
        "us": round(t * 1e3, 1), "TFLOPS": round(fl / (t * 1e-3) / 1e12, 2),
        "fp8_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
        "steps": "qg_quantize_mxfp8 + qg_gemm"}
    print(f"[bench] w4a8 from bf16: {extra[f'w4a8_from_bf16_M{m}_N{n}_K{k}']}", file=sys.stderr, flush=True)
    del L
    # bf16 -> MXFP4 (2 B read, 1/2 + 1/32 B written per value), then W4A4
    q4 = torch.empty((m, k // 2), dtype=torch.uint8, device="cuda")
    t = timed(torch, lambda i: qg.quantize_mxfp4(xs[i % nc], m, k, k, q4, k, qs, stream), 100, 10)
    record("quantize_mxfp4_M4096_K4096", t, m * k * 2 + m * k // 2 + m * k // 32)
    codes, sc, _ = synth.mx_weights(synth.rng(50, 1), n, k)
    desc4 = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=qg.A_MXFP4)
    bufs4 = [torch.empty(qg.packed_size(desc4), dtype=torch.uint8, device="cuda") for _ in range(2)]
    w4 = [qg.preprocess(desc4, codes, sc, None, b) for b in bufs4]
    wsb4 = qg.gemm_workspace_size(w4[0], m)
    ws4 = torch.zeros(max(wsb4, 1), dtype=torch.uint8, device="cuda")

    def qgemm4(i):
        qg.quantize_mxfp4(xs[i % nc], m, k, k, q4, k, qs, stream)
        qg.gemm(w4[i % 2], q4, qs, m, k, y, qg.O_BF16, n, ws4, wsb4, stream)
    t = timed(torch, qgemm4, 50, 10)
    extra[f"w4a4_from_bf16_M{m}_N{n}_K{k}"] = {
        "us": round(t * 1e3, 1), "TFLOPS": round(fl / (t * 1e-3) / 1e12, 2),
        "fp4_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_TFLOPS["fp4"], 4),
        "steps": "qg_quantize_mxfp4 + qg_gemm"}
    print(f"[bench] w4a4 from bf16: {extra[f'w4a4_from_bf16_M{m}_N{n}_K{k}']}", file=sys.stderr, flush=True)
    del bufs4, w4, xs
    # SiLU-gated product between gate_up and down at T = 4096, top-8 (32768 pairs)
    p = 4096 * 8
    for inter, mx in ((2048, False), (640, True)):
        nc = copies_for(p * 2 * inter * 2)
        gus = [torch.randn((p, 2 * inter), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(nc)]
        h = torch.empty((p, inter), dtype=torch.uint8 if mx else torch.bfloat16, device="cuda")
        hs = torch.empty((p, inter // 32), dtype=torch.uint8, device="cuda") if mx else None
        ht = qg.A_MXFP8 if mx else qg.A_BF16
        t = timed(torch, lambda i: qg.silu_mul(gus[i % nc], qg.O_BF16, p, inter, 2 * inter, h, ht, inter, hs,
                                               stream), 50, 5)
        out_bytes = p * inter + p * inter // 32 if mx else p * inter * 2
        record(f"silu_mul_P{p}_I{inter}_{'mxfp8' if mx else 'bf16'}", t, p * 2 * inter * 2 + out_bytes)
        del gus, h, hs
    # weighted top-8 combine of the down projection's rows, T = 4096, N = 7168
    tokens, topk, n = 4096, 8, 7168
    nc = copies_for(tokens * topk * n * 2)
    ys = [torch.randn((tokens * topk, n), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(nc)]
    w = torch.rand((tokens, topk), device="cuda", generator=gen)
    o = torch.empty((tokens, n), dtype=torch.bfloat16, device="cuda")
    t = timed(torch, lambda i: qg.moe_combine(ys[i % nc], qg.O_BF16, n, w, tokens, topk, n, None, o, qg.O_BF16, n,
                                              stream), 50, 5)
    record(f"moe_combine_T{tokens}_top{topk}_N{n}", t, tokens * topk * (n * 2 + 4) + tokens * n * 2)
    del ys
    torch.cuda.empty_cache()
    return extra


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 2500 decode steps are about 50 ms of back-to-back work: the clocks settle
    ap.add_argument("--warmup", type=int, default=2500)
    ap.add_argument("--quick", action="store_true", help="primary decode workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--large-m", action="store_true",
                    help="only the M=4096 dense GEMMs (for profiling the tiled kernels)")
    ap.add_argument("--act", action="store_true",
                    help="only the activation-side kernels (quantizer, SiLU-gated product, combine)")
    ap.add_argument("--moe", action="store_true",
                    help="only the MoE configurations at T=4096 (for profiling the grouped kernels)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only the plain stream-read ceiling at one decode GEMM's weight bytes")
    ap.add_argument("--moe-tuned", action="store_true",
                    help="only the MoE configurations after qg_moe_autotune")
    ap.add_argument("--moe-formats", action="store_true",
                    help="only the W8A8 and per-token W4A8 MoE configurations")
    ap.add_argument("--formats", action="store_true",
                    help="only the further formats (WnA16 integer / e4m3 weights, W8A8, per-token W4A8)")
    ap.add_argument("--decode-rows", action="store_true",
                    help="only the dense W4A16 decode GEMMs at M = 1, 4, 8, 16 (UINT4 + zp and INT3)")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="only run the copy calibration + decode kernel for rocprofv3 counter passes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the quantized GEMM path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_gemm_qg_amd as qg
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.pmc_workload:
        pmc_workload(qg, synth, torch)
        return
    if args.large_m:
        print(json.dumps(bench_large_m(qg, synth, torch)), flush=True)
        return
    if args.act:
        print(json.dumps(bench_act(qg, synth, torch)), flush=True)
        return
    if args.moe:
        print(json.dumps(bench_moe_large(qg, synth, torch)), flush=True)
        return
    if args.moe_formats:
        print(json.dumps(bench_moe_formats(qg, synth, torch)), flush=True)
        return
    if args.moe_tuned:
        print(json.dumps(bench_moe_tuned(qg, synth, torch)), flush=True)
        return
    if args.ceiling:
        print(json.dumps(bench_stream_ceiling(qg, torch)), flush=True)
        return
    shapes = [(14336, 4096), (4096, 14336)]
    if args.decode_rows:
        print(json.dumps(bench_decode_rows(qg, synth, torch, shapes)), flush=True)
        return
    if args.formats:
        print(json.dumps(bench_formats(qg, synth, torch, shapes)), flush=True)
        return

    print(f"[bench] preparing decode weights {shapes} x{ROTATE} copies", file=sys.stderr, flush=True)
    layers = [DenseWeights(qg, synth, torch, qg.W_UINT4, n, k, 128, seed=i) for i, (n, k) in enumerate(shapes)]
    xs = [make_x(qg, synth, torch, False, 1, k, seed=10 + i) for i, (_, k) in enumerate(shapes)]
    launchers = [dense_launcher(qg, torch, L, x, None, 1) for L, (x, _, _) in zip(layers, xs)]

    def step(i):
        for f in launchers:
            f(i)

    # per-kernel average launch durations (each kernel alone, back to back,
    # after at least 50 ms of its own launches); measured first, so the
    # step below also starts on settled clocks
    per_kernel_ms = [timed(torch, f, args.steps, 5) for f in launchers]
    # timed region: K steps bracketed by a synchronize and events on both sides
    ms_step = timed(torch, step, args.steps, args.warmup, warm_ms=0)  # exactly W warmup steps
    step_bytes = sum(L.bytes for L in layers)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dom = int(np.argmax(per_kernel_ms))
    achieved = layers[dom].bytes / (per_kernel_ms[dom] * 1e-3) / 1e9
    print(f"[bench] decode step {ms_step * 1e3:.2f} us, {value:.0f} GB/s", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 weights, bf16 MFMA, f32 accumulate",
        "data": "synthetic (seeded); weights resident in HBM, 8 rotating copies",
        "config": {
            "workload": "dense W4A16 decode: UINT4 + uint4 zero point, group 128, bf16 scales, "
                        "bf16 activations, M=1, (N,K)=(14336,4096) then (4096,14336)",
            "m": 1, "shapes": shapes, "group": 128, "weight_bytes_per_step": step_bytes,
            "dispatch": [qg.describe_dispatch(L.ws[0], 1) for L in layers],
        },
        "per_kernel_us": [round(t * 1e3, 3) for t in per_kernel_ms],
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(layers[dom].n, layers[dom].k),
            "kernel": f"{qg.describe_dispatch(layers[dom].ws[0], 1)}: dense W4A16 N={layers[dom].n} "
                      f"K={layers[dom].k} M=1",
            "bytes_per_launch": layers[dom].bytes,
        },
    }

    if not args.quick:
        extra = {}
        # the same decode step after qg_gemm_autotune of both GEMMs (candidates
        # timed from cold caches: a 512 MiB read before every timed launch)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        tuned = []
        for L, (x, _, _) in zip(layers, xs):
            y = torch.empty((1, L.n), dtype=torch.bfloat16, device="cuda")
            wsb = qg.gemm_autotune_workspace_size(L.ws[0], 1)
            wst = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            tuned.append(qg.gemm_autotune(L.ws[0], x, None, 1, L.k, y, qg.O_BF16, L.n, wst, wsb, flush, flush.numel(), 10))
        del flush
        launchers_t = [dense_launcher(qg, torch, L, x, None, 1) for L, (x, _, _) in zip(layers, xs)]
        ms_t = timed(torch, lambda i: [f(i) for f in launchers_t], args.steps, args.warmup)
        extra["decode_step_autotuned"] = {
            "us": round(ms_t * 1e3, 2), "weight_GBs": round(step_bytes / (ms_t * 1e-3) / 1e9, 1),
            "hbm_frac": round(step_bytes / (ms_t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "dispatch": [t[0] for t in tuned], "cold_cache_us": [round(t[1], 2) for t in tuned]}
        print(f"[bench] autotuned decode step: {extra['decode_step_autotuned']}", file=sys.stderr, flush=True)
        qg.autotune_reset()
        extra.update(bench_decode_rows(qg, synth, torch, shapes, layers))
        extra["formats"] = bench_formats(qg, synth, torch, shapes)
        # MXFP4 weights x bf16 activations at the decode shapes
        for i, (n, k) in enumerate(shapes):
            r = synth.rng(70 + i, 1)
            codes, sc, _ = synth.mx_weights(r, n, k)
            desc = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=qg.A_BF16)
            size = qg.packed_size(desc)
            bufs = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(ROTATE)]
            wts = [qg.preprocess(desc, codes, sc, None, b) for b in bufs]
            wbytes = weight_bytes(n, k, 4, 32, False, 1)
            for mm in (1, 16):
                x, _, _ = make_x(qg, synth, torch, False, mm, k, seed=40 + mm)
                y = torch.empty((mm, n), dtype=torch.bfloat16, device="cuda")
                wsb = qg.gemm_workspace_size(wts[0], mm)
                wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
                stream = torch.cuda.current_stream().cuda_stream
                t = timed(torch, lambda j: qg.gemm(wts[j % ROTATE], x, None, mm, k, y, qg.O_BF16, n, wsp, wsb, stream),
                          100, 10)
                extra[f"mxfp4_bf16_M{mm}_N{n}_K{k}"] = {
                    "us": round(t * 1e3, 2), "weight_GBs": round(wbytes / (t * 1e-3) / 1e9, 1),
                    "hbm_frac": round(wbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "dispatch": qg.describe_dispatch(wts[0], mm)}
            del bufs, wts
        print(f"[bench] extra MXFP4 x bf16 decode done", file=sys.stderr, flush=True)
        # MXFP4 weights x MX activations at the decode shapes: W4A8 (MXFP8) and
        # W4A4 (MXFP4) on the MX skinny kernel, which widens W4A4's e2m1
        # activation fragments to e4m3 in registers (one launch per GEMM)
        for i, (n, k) in enumerate(shapes):
            codes, sc, _ = synth.mx_weights(synth.rng(70 + i, 1), n, k)
            wbytes = weight_bytes(n, k, 4, 32, False, 1)
            for atype, name in ((qg.A_MXFP8, "w4a8_mx"), (qg.A_MXFP4, "w4a4_mx")):
                desc = qg.layer_desc(qg.W_MXFP4, n, k, 32, atype=atype)
                bufs = [torch.empty(qg.packed_size(desc), dtype=torch.uint8, device="cuda") for _ in range(ROTATE)]
                wts = [qg.preprocess(desc, codes, sc, None, b) for b in bufs]
                for mm in (1, 16):
                    xb = k if atype == qg.A_MXFP8 else k // 2
                    xm = torch.randint(0, 256, (mm, xb), dtype=torch.uint8, device="cuda")
                    xms = torch.randint(118, 128, (mm, k // 32), dtype=torch.uint8, device="cuda")
                    y = torch.empty((mm, n), dtype=torch.bfloat16, device="cuda")
                    wsb = qg.gemm_workspace_size(wts[0], mm)
                    wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
                    stream = torch.cuda.current_stream().cuda_stream
                    t = timed(torch, lambda j: qg.gemm(wts[j % ROTATE], xm, xms, mm, k, y, qg.O_BF16, n, wsp, wsb,
                                                        stream), 100, 10)
                    extra[f"{name}_M{mm}_N{n}_K{k}"] = {
                        "us": round(t * 1e3, 2), "weight_GBs": round(wbytes / (t * 1e-3) / 1e9, 1),
                        "hbm_frac": round(wbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "dispatch": qg.describe_dispatch(wts[0], mm)}
                del bufs, wts
        print(f"[bench] extra MX-activation decode done", file=sys.stderr, flush=True)
        # the batch-invariant compute option at decode sizes (one kernel for every M)
        for i, (n, k) in enumerate(shapes):
            L = layers[i]
            for mm in (1, 16):
                x, _, _ = make_x(qg, synth, torch, False, mm, k, seed=40 + mm)
                y = torch.empty((mm, n), dtype=torch.bfloat16, device="cuda")
                wsb = qg.gemm_workspace_size_ex(L.ws[0], mm, qg.GEMM_BATCH_INVARIANT)
                wsp = torch.zeros(max(wsb, 1), dtype=torch.uint8, device="cuda")
                stream = torch.cuda.current_stream().cuda_stream
                t = timed(torch, lambda j: qg.gemm_ex(L.ws[j % len(L.ws)], x, None, mm, k, y, qg.O_BF16, n, wsp, wsb,
                                                      qg.GEMM_BATCH_INVARIANT, stream), 100, 10)
                extra[f"batch_invariant_uint4_zp_M{mm}_N{n}_K{k}"] = {
                    "us": round(t * 1e3, 2), "weight_GBs": round(L.bytes / (t * 1e-3) / 1e9, 1),
                    "hbm_frac": round(L.bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] extra batch-invariant decode done", file=sys.stderr, flush=True)
        extra["stream_read_ceiling"] = bench_stream_ceiling(qg, torch)
        extra.update(bench_large_m(qg, synth, torch))
        extra["activation"] = bench_act(qg, synth, torch)
        moe = {}
        for tokens in (64, 4096):
            moe[f"w4a16_E256_top8_T{tokens}"] = bench_moe(
                qg, synth, torch, "moe_w4a16", qg.W_INT4, 256, 8, 4096, 7168, 7168, 2048, tokens,
                iters=5 if tokens > 64 else 30)
        for tokens in (64, 4096):
            moe[f"w4a16_mxfp4_E256_top8_T{tokens}"] = bench_moe(
                qg, synth, torch, "moe_w4a16_mxfp4", qg.W_MXFP4, 256, 8, 4096, 7168, 7168, 2048, tokens,
                iters=5 if tokens > 64 else 30, atype=qg.A_BF16)
        for tokens in (1, 64, 512, 4096):
            moe[f"w4a8_E128_top8_T{tokens}"] = bench_moe(
                qg, synth, torch, "moe_w4a8", qg.W_MXFP4, 128, 8, 1280, 4096, 4096, 640, tokens,
                iters=5 if tokens > 512 else 30)
        for tokens in (64, 4096):
            moe[f"w4a4_E128_top8_T{tokens}"] = bench_moe(
                qg, synth, torch, "moe_w4a4", qg.W_MXFP4, 128, 8, 1280, 4096, 4096, 640, tokens,
                iters=5 if tokens > 512 else 30, atype=qg.A_MXFP4)
        moe.update(bench_moe_formats(qg, synth, torch))
        moe.update(bench_moe_tuned(qg, synth, torch))
        extra["moe"] = moe
        out["extra"] = extra

    if not args.no_cpu:
        import oracle
        sample = []
        for L, (_, _, xb) in zip(layers, xs):
            codes, sc, zp = L.std
            sample.append((qg.W_UINT4, codes, sc, zp, L.n, L.k, 128, xb, L.bytes))
        out["cpu_baseline"] = cpu_baseline(oracle, sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
