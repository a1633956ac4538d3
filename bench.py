"""Benchmark of the quantized GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--extra]

Primary workload (the metric's "weight GB/s at M=1 decode"): dense W4A16
decode, asymmetric INT4 with uint4 zero points, group 128, bf16 scales, bf16
N(0,1) activations, M = 1.  One step = the two decode GEMMs of an MLP block,
(N, K) = (14336, 4096) and (4096, 14336), each one qg_gemm launch.  Weights are
resident in HBM before timing; every step reads a different copy of the
weights (8 rotating copies, 488 MB > 256 MB MALL + L2), so each launch streams
its weights from HBM as a decode step over distinct layers would.

value = algorithmic weight bytes (packed codes at 0.5 B/weight + bf16 scales +
4-bit zero points, unpadded) per step / step time.

The JSON line also carries the roofline of the dominant kernel (per-launch HIP
events on the launch stream, averaged over the timed steps), the CPU oracle
timed on a bounded sample (rank 0 only), and with --extra the other decode
shapes/formats, the W4A8 MXFP4 x MXFP8 GEMM at M = 4096 and MoE grouped runs.
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
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "TFLOPS at M=4096 (W4A16, W4A8-MXFP4) + weight GB/s at M=1 decode, 1 GPU"
ROTATE = 8


def weight_bytes(n: int, k: int, bits: int, group: int, zp: bool, scale_bytes: int = 2) -> int:
    """Algorithmic bytes of one weight matrix: codes + scales + zero points."""
    g = n * (k // group)
    return n * k * bits // 8 + g * scale_bytes + (g // 2 if zp else 0)


class DenseWeights:
    """ROTATE packed copies of one seeded weight matrix on the device."""

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
        self.bufs, self.ws = [], []
        for _ in range(copies):
            b = torch.empty(size, dtype=torch.uint8, device="cuda")
            self.ws.append(qg.preprocess(desc, codes, sc, zp, b))
            self.bufs.append(b)
        bits = 3 if wtype in (qg.W_INT3, qg.W_UINT3) else 4
        self.bytes = weight_bytes(n, k, bits, group, zp is not None, 1 if wtype == qg.W_MXFP4 else 2)


def make_x(qg, synth, torch, mx, m, k, seed):
    r = synth.rng(seed, 2)
    if mx:
        c, s = synth.mx_activations(r, m, k)
        return torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(), (c, s)
    b = synth.x_bf16(r, m, k)
    return torch.from_numpy(b.view(np.int16)).cuda(), None, b


def time_dense(qg, torch, wts, x, xs, m, steps, warmup, otype=None):
    """Times `steps` launches rotating over the weight copies; returns mean ms per launch."""
    otype = qg.O_BF16 if otype is None else otype
    y = torch.empty((m, wts.n), dtype=torch.bfloat16, device="cuda")
    ws_bytes = qg.gemm_workspace_size(wts.ws[0], m)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        qg.gemm(wts.ws[i % len(wts.ws)], x, xs, m, wts.k, y, otype, wts.n, ws, ws_bytes, stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        qg.gemm(wts.ws[i % len(wts.ws)], x, xs, m, wts.k, y, otype, wts.n, ws, ws_bytes, stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


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
            "sample": f"{reps} repetitions of the M=1 decode step (both (N,K) shapes), "
                      f"{el:.1f} s of CPU time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--extra", action="store_true", help="also time the other configurations")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_gemm_qg_amd as qg
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    shapes = [(14336, 4096), (4096, 14336)]
    print(f"[bench] preparing decode weights {shapes} x{ROTATE} copies", file=sys.stderr, flush=True)
    layers = [DenseWeights(qg, synth, torch, qg.W_UINT4, n, k, 128, seed=i) for i, (n, k) in enumerate(shapes)]
    xs = [make_x(qg, synth, torch, False, 1, k, seed=10 + i) for i, (_, k) in enumerate(shapes)]
    m = 1
    stream = torch.cuda.current_stream()
    ys = [torch.empty((m, L.n), dtype=torch.bfloat16, device="cuda") for L in layers]
    wsb = [qg.gemm_workspace_size(L.ws[0], m) for L in layers]
    wsp = [torch.zeros(max(b, 1), dtype=torch.uint8, device="cuda") for b in wsb]
    for i in range(args.warmup):
        for j, (L, (x, _, _), y) in enumerate(zip(layers, xs, ys)):
            qg.gemm(L.ws[i % ROTATE], x, None, m, L.k, y, qg.O_BF16, L.n, wsp[j], wsb[j], stream)
    torch.cuda.synchronize()
    # timed region: K steps; per-launch events on the launch stream
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in layers] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        for j, (L, (x, _, _), y) in enumerate(zip(layers, xs, ys)):
            ev[s][j][0].record(stream)
            qg.gemm(L.ws[s % ROTATE], x, None, m, L.k, y, qg.O_BF16, L.n, wsp[j], wsb[j], stream)
            ev[s][j][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    per_kernel_ms = [float(np.mean([ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(args.steps)]))
                     for j in range(len(layers))]
    step_bytes = sum(L.bytes for L in layers)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    dom = int(np.argmax(per_kernel_ms))
    achieved = layers[dom].bytes / (per_kernel_ms[dom] * 1e-3) / 1e9
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
        "dtype": "u4 codes, bf16 MFMA, f32 accumulate",
        "data": "synthetic (seeded), weights resident in HBM, 8 rotating copies",
        "config": {
            "workload": "dense W4A16 decode: UINT4 + uint4 zero point, group 128, bf16 scales, "
                        "M=1, (N,K)=(14336,4096) then (4096,14336)",
            "m": 1, "shapes": shapes, "group": 128, "weight_bytes_per_step": step_bytes,
            "dispatch": [qg.describe_dispatch(L.ws[0], 1) for L in layers],
        },
        "per_kernel_us": [round(t * 1e3, 3) for t in per_kernel_ms],
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": f"skinny_kernel (dense W4A16, N={layers[dom].n}, K={layers[dom].k}, M=1)",
        },
    }

    if args.extra:
        extra = {}
        for wtype, name in ((qg.W_UINT4, "uint4_zp"), (qg.W_INT3, "int3")):
            for i, (n, k) in enumerate(shapes):
                L = layers[i] if wtype == qg.W_UINT4 else DenseWeights(qg, synth, torch, wtype, n, k, 128, seed=30 + i)
                for mm in (1, 4, 16):
                    x, _, _ = make_x(qg, synth, torch, False, mm, k, seed=40 + mm)
                    t = time_dense(qg, torch, L, x, None, mm, 100, 10)
                    extra[f"decode_{name}_M{mm}_N{n}_K{k}"] = {
                        "us": round(t * 1e3, 2), "weight_GBs": round(L.bytes / (t * 1e-3) / 1e9, 1),
                        "hbm_frac": round(L.bytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
                print(f"[bench] extra {name} {n}x{k} done", file=sys.stderr, flush=True)
        for n in (3072, 14336):
            L = DenseWeights(qg, synth, torch, qg.W_MXFP4, n, 4096, 32, seed=50, copies=2)
            x, xsc, _ = make_x(qg, synth, torch, True, 4096, 4096, seed=51)
            t = time_dense(qg, torch, L, x, xsc, 4096, 10, 2)
            fl = 2.0 * 4096 * n * 4096
            extra[f"w4a8_mx_M4096_N{n}_K4096"] = {
                "us": round(t * 1e3, 1), "TFLOPS": round(fl / (t * 1e-3) / 1e12, 1),
                "fp8_frac": round(fl / (t * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)}
            print(f"[bench] extra mx N={n} done", file=sys.stderr, flush=True)
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
