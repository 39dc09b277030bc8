#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

A step is one call of nvfp4_moe_grouped_gemm -- route, quantize x, grouped
gate_up GEMM + SwiGLU, quantize h, grouped down GEMM, router-weighted combine
-- on the 384-expert layer share (top-8, hidden 7168, expert intermediate
2048) at a prefill batch of 16384 tokens, with experts that start as MXFP4
and were remapped to NVFP4.  All inputs are resident in HBM before timing.

Prints ONE JSON line (rank 0).  Besides the headline TFLOP/s it carries
  roofline      the dominant kernel (grouped gate_up GEMM) timed with HIP
                events on its own stream, against the f16 MFMA peak it runs
                on (fractions of the FP8 and FP4 peaks are given too);
  cpu_baseline  the CPU oracle on a bounded sample of the same workload;
  breakdown     the other hot-path rows (quantize, remap, KV cache, dense
                MLP, 512-expert MoE, decode MoE) measured on their configs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0   # MI355X dense f16/bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_moe384_T16384.json")
# sources that shape the grouped gate_up launch (kernels, tile plan, class dispatch)
GEMM_SOURCES = ["precision_moe_gemm_amd/csrc/gemm.h", "precision_moe_gemm_amd/csrc/common.h",
                "precision_moe_gemm_amd/csrc/moe.h", "precision_moe_gemm_amd/csrc/libnvfp4.hip"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the breakdown of other rows")
    ap.add_argument("--profile-copy", action="store_true",
                    help="also launch a 1 GiB plain copy (counter calibration)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the 384-expert decode rows (for profiling); prints their JSON")
    return ap.parse_args()


def source_hash():
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(launch_units):
    """HBM bytes per gate_up launch from the committed rocprofv3 counter runs,
    or None when they are missing or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t.get("bytes_per_launch")


def time_loop(fn, iters, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.stderr.write("bench.py: multi-GPU runs are not part of this build (one GPU only)\n")
        sys.exit(2)

    import numpy as np
    import torch

    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import synth, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.decode_only:
        print(json.dumps({"decode_rows": decode_rows(dev, stream, 10)}))
        return
    cfg = synth.C4_PREFILL
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I

    log(f"building {E} MXFP4-origin experts (H={H}, I={I}) and routing T={T}")
    t0 = time.time()
    W = workloads.build_moe_weights(cfg, dev)
    x = cfg.x(dev)
    ids, w = workloads.routing(cfg, dev)
    from precision_moe_gemm_amd import _lib
    ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE, T, k, E, H, I), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    def step():
        nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2, out=out, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    err = nv.nvfp4_get_error()
    if err != 0:
        raise RuntimeError(f"device error {err} during warmup")
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    ms = time_loop(step, args.steps, stream)
    torch.cuda.synchronize()
    flops = 2.0 * T * k * 3 * H * I
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"MoE prefill: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")

    # ---- dominant kernel: the grouped gate_up GEMM, timed on its stream ----
    xq = nv.nvfp4_quantize(x)
    perm, offsets, inv = nv.nvfp4_moe_route(ids, E)
    route_ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE_ROUTE, T, k, E, H, I), dtype=torch.uint8, device=dev)
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    hmax = torch.zeros(1, dtype=torch.int32, device=dev)
    counts = (offsets[1:] - offsets[:-1]).cpu().numpy()
    import ctypes
    lib = _lib.load()
    xc, wc = xq.c(), W.w13.c()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def gate_up():
        lib.nvfp4_moe_gate_up(ctypes.byref(xc), ctypes.c_void_p(perm.data_ptr()),
                              ctypes.c_void_p(offsets.data_ptr()), T, k, E, ctypes.byref(wc),
                              ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(hmax.data_ptr()),
                              ctypes.c_void_p(route_ws.data_ptr()), route_ws.numel(), sptr)

    for _ in range(2):
        gate_up()
    gu_ms = time_loop(gate_up, max(5, args.steps), stream)
    gu_flops = 2.0 * T * k * (2 * I) * H
    gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    traffic = load_traffic(1)  # HBM bytes per gate_up call, from the committed counter runs
    roofline = {
        "bound": "mfma", "achieved": round(gu_tflops, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(gu_tflops / PEAK_F16_TFLOPS, 4), "traffic": traffic,
        "kernel": "grouped gate_up GEMM + SwiGLU, one nvfp4_moe_gate_up call: tile plan, then "
                  "256-row and 128-row gemm_rtile_kernel classes (codes staged by LDS DMA, "
                  "decoded by each wave into f16 MFMA 32x32x16 operands) and the 16-row "
                  "gemm_stream_kernel class (f16 MFMA 16x16x32); power-of-two weight-scale "
                  "variants (MXFP4-origin experts)",
        "launch_ms": round(gu_ms, 4),
        "algorithmic_flops_per_launch": gu_flops,
        "frac_of_fp8_peak": round(gu_tflops / PEAK_FP8_TFLOPS, 4),
        "frac_of_fp4_peak": round(gu_tflops / PEAK_FP4_TFLOPS, 4),
        "peak_basis": "NVFP4 (E4M3 scale per 16) has no exact mapping onto gfx950's block-32 "
                      "E8M0 scaled MFMA; operands are decoded exactly to f16 and run on the "
                      "f16 MFMA path (2.5 PFLOP/s dense)",
    }
    log(f"gate_up: {gu_ms:.3f} ms/launch, {gu_tflops:.1f} TFLOP/s")

    result = {
        "metric": "W4A4 MoE grouped-GEMM TFLOP/s (NVFP4, 384 experts top-8, prefill 16384 tokens)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 w4a4 (e2m1 x e4m3 decoded to f16, f16 MFMA, fp32 accumulate)",
        "data": "synthetic (seeded N(0,0.02) MXFP4-origin experts, N(0,1) activations, "
                "Zipf(1.1)-biased top-8 routing)",
        "config": {"workload": "moe-384e-top8-h7168-i2048-prefill-T16384", "experts": E,
                   "top_k": k, "hidden": H, "intermediate": I, "tokens": T,
                   "expert_origin": "mxfp4 remapped to nvfp4",
                   "max_tokens_per_expert": int(counts.max()),
                   "experts_touched": int((counts > 0).sum())},
        "roofline": roofline,
    }

    # ---- the same layer with calibrated (static) globals: the gate_up
    # epilogue encodes h to NVFP4 itself (no bf16 h, no h quantize pass) ----
    static_res = None
    if not args.no_extras:
        gh = float(np.uint32(hmax.item()).view(np.float32)) / 2688.0
        sg = torch.tensor([float(xq.global_[0].item()), gh], dtype=torch.float32, device=dev)

        def step_static():
            nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2, static_in_globals=sg, out=out, ws=ws)

        step_static()
        sms = time_loop(step_static, max(5, args.steps), stream)
        log(f"MoE prefill, static globals: {sms:.3f} ms/step")
        static_res = {"ms": round(sms, 4), "TFLOPs": round(flops / (sms * 1e-3) / 1e12, 2),
                      "globals": "G_x, G_h = amax/2688 of this input (calibrated); h encoded in the "
                                 "gate_up epilogue"}
    # ---- CPU oracle baseline on a bounded sample -------------------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, x, ids, perm, offsets)
    # ---- other hot-path rows ------------------------------------------------
    if not args.no_extras:
        del W, ws, h, route_ws, out
        torch.cuda.empty_cache()
        result["breakdown"] = breakdown(args)
        result["breakdown"]["moe_384e_prefill_static_globals"] = static_res
    if args.profile_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    print(json.dumps(result), flush=True)


def cpu_baseline(cfg, x, ids, perm, offsets):
    """The oracle (single-threaded C, as it stands) on 32 (token, slot) pairs
    of the most-loaded expert: quantize their x rows, gate_up + SwiGLU,
    quantize h, down.  Expert weights are prepared by the oracle untimed."""
    import numpy as np
    import oracle
    from precision_moe_gemm_amd import synth
    H, I, k = cfg.H, cfg.I, cfg.k
    off = offsets.cpu().numpy()
    e = int(np.argmax(off[1:] - off[:-1]))
    n = min(32, int(off[e + 1] - off[e]))
    rows = np.arange(off[e], off[e] + n)
    pairs = perm.cpu().numpy()[rows]
    toks = pairs // k
    log(f"cpu baseline: preparing expert {e} weights with the oracle")
    w13 = oracle.mxfp4_to_nvfp4(*oracle.mxfp4_encode(synth.bits(cfg.w13(e, "cuda"))))
    w2 = oracle.mxfp4_to_nvfp4(*oracle.mxfp4_encode(synth.bits(cfg.w2(e, "cuda"))))
    xs = np.ascontiguousarray(synth.bits(x[torch_index(toks)]))
    gx = oracle.global_from_amax(float(x.float().abs().max().item()))
    ex13 = oracle.Experts(w13.packed[None], w13.scales[None], np.array([w13.G], np.float32))
    ex2 = oracle.Experts(w2.packed[None], w2.scales[None], np.array([w2.G], np.float32))
    log(f"cpu baseline: timing {n} pairs")
    t0 = time.perf_counter()
    xq = oracle.quantize(xs, static_G=gx)
    lperm = np.arange(n, dtype=np.int32)          # sample row i is pair i (k = 1 view)
    loff = np.array([0, n], np.int32)
    h = oracle.moe_gate_up(xq, lperm, loff, 1, ex13, np.arange(n))
    hq = oracle.quantize(h)
    oracle.moe_down(hq, loff, ex2, np.arange(n))
    dt = time.perf_counter() - t0
    flops = 2.0 * n * 3 * H * I
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"{n} (token, slot) pairs of expert {e} (the most loaded): x-row quantize, "
                      f"exact int64 gate_up + SwiGLU, h quantize, exact down; weights prepared "
                      f"by the oracle outside the timed region; single-threaded C"}


def torch_index(a):
    import torch
    return torch.from_numpy(a).to("cuda")


def decode_rows(dev, st, it):
    """The 384-expert decode batch (T=64): fused layer with dynamic and with
    calibrated globals, the W4A16 layer, and the MXFP4 -> NVFP4 remap of its
    w13 weights; each timed with HIP events."""
    import numpy as np
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib, synth, workloads
    res = {}

    def gbs(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    c4 = synth.C4_DECODE
    log("breakdown: 384-expert decode + remap")
    W = workloads.build_moe_weights(c4, dev, keep_mx=True)
    x = c4.x(dev)
    ids, wt = workloads.routing(c4, dev)
    ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE, c4.T, c4.k, c4.E, c4.H, c4.I), dtype=torch.uint8, device=dev)
    out = torch.empty((c4.T, c4.H), dtype=torch.bfloat16, device=dev)
    f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, W.w13, W.w2, out=out, ws=ws)
    f()
    ms = time_loop(f, it, st)
    touched = np.unique(ids.cpu().numpy())
    wbytes = len(touched) * 3 * c4.H * c4.I * 0.5625
    res["moe_384e_top8_decode_T64"] = {"ms": round(ms, 4), "experts_touched": int(len(touched)),
                                       "touched_weight_GBps": gbs(wbytes, ms),
                                       "frac_hbm": round(gbs(wbytes, ms) / PEAK_HBM_GBS, 4)}
    # calibrated globals (from one dynamic staged pass): h encoded in the epilogue
    xq4 = nv.nvfp4_quantize(x)
    perm4, off4, _ = nv.nvfp4_moe_route(ids, c4.E)
    _, hmax4 = nv.nvfp4_moe_gate_up(xq4, perm4, off4, c4.k, W.w13)
    sg4 = torch.tensor([float(xq4.global_[0].item()),
                        float(np.uint32(hmax4.item()).view(np.float32)) / 2688.0],
                       dtype=torch.float32, device=dev)
    f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, W.w13, W.w2, static_in_globals=sg4, out=out, ws=ws)
    f()
    ms = time_loop(f, it, st)
    res["moe_384e_top8_decode_T64_static_globals"] = {"ms": round(ms, 4), "touched_weight_GBps": gbs(wbytes, ms),
                                                      "frac_hbm": round(gbs(wbytes, ms) / PEAK_HBM_GBS, 4)}
    # the same experts as W4A16 (bf16 activations, no activation quantization)
    f = lambda: nv.nvfp4_moe_w4a16(x, ids, wt, W.w13, W.w2, out=out, ws=ws)
    f()
    ms = time_loop(f, it, st)
    res["moe_384e_top8_w4a16_decode_T64"] = {"ms": round(ms, 4), "touched_weight_GBps": gbs(wbytes, ms),
                                             "frac_hbm": round(gbs(wbytes, ms) / PEAK_HBM_GBS, 4)}
    # the same MXFP4 experts as an MX-native W4A8 layer (MXFP8 activations)
    (m13, e13), (m2, e2) = W.mx13, W.mx2
    mws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MX_MOE, c4.T, c4.k, c4.E, c4.H, c4.I), dtype=torch.uint8,
                      device=dev)
    f = lambda: nv.mx_moe_w4a8(x, ids, wt, m13, e13, m2, e2, out=out, ws=mws)
    f()
    ms = time_loop(f, it, st)
    mx_bytes = len(touched) * 3 * c4.H * c4.I * (0.5 + 1 / 32)
    res["moe_384e_top8_mx_w4a8_decode_T64"] = {"ms": round(ms, 4), "touched_weight_GBps": gbs(mx_bytes, ms),
                                               "frac_hbm": round(gbs(mx_bytes, ms) / PEAK_HBM_GBS, 4),
                                               "bytes_basis": "touched MXFP4 experts: 0.5 + 1/32 B/elem"}
    del mws
    p13, s13 = W.mx13
    dst = nv.NVFP4Tensor.empty(2 * c4.I, c4.H, c4.E, dev)
    rws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_REMAP, c4.E, 0, 0, 2 * c4.I, c4.H), dtype=torch.uint8, device=dev)
    f = lambda: nv.mxfp4_to_nvfp4(p13, s13, 2 * c4.I, c4.H, c4.E, out=dst, ws=rws)
    f()
    ms = time_loop(f, 3, st)
    nel = c4.E * 2 * c4.I * c4.H
    res["remap_w13_384x4096x7168"] = {"ms": round(ms, 4), "GBps": gbs(nel * (0.5 + 1 / 32 + 0.5 + 1 / 16), ms),
                                      "bytes_basis": "0.5+1/32 B/elem read, 0.5+1/16 B/elem written",
                                      "frac_hbm": round(gbs(nel * 1.09375, ms) / PEAK_HBM_GBS, 4)}
    del W, ws, out, dst, rws
    torch.cuda.empty_cache()

    return res


def breakdown(args):
    """Other hot-path rows on their own configs (each timed with HIP events)."""
    import ctypes
    import numpy as np
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib, synth, workloads
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    res = {}
    it = 10

    def gbs(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    # dense MLP weights (27B class): static quantize and dense MLP as a 1-expert MoE
    c2 = synth.C2
    log("breakdown: dense MLP 5120/17408")
    w13b = c2.w13(dev)
    n13 = w13b.numel()
    g = torch.tensor([0.01], device=dev)
    q = nv.nvfp4_quantize(w13b, static_global=g)
    qws = torch.empty(4096, dtype=torch.uint8, device=dev)
    ms_s = time_loop(lambda: nv.nvfp4_quantize(w13b, static_global=g, out=q), it, st)
    ms_d = time_loop(lambda: nv.nvfp4_quantize(w13b, out=q, ws=qws), it, st)
    res["quantize_weight_34816x5120"] = {
        "static_ms": round(ms_s, 4), "static_GBps": gbs(2.5625 * n13, ms_s),
        "dynamic_ms": round(ms_d, 4), "dynamic_GBps": gbs(4.5625 * n13, ms_d),
        "bytes_basis": "static 2.5625 B/elem (bf16 read + codes + scales); dynamic 4.5625 B/elem "
                       "(+ the amax pass)", "frac_hbm_static": round(gbs(2.5625 * n13, ms_s) / PEAK_HBM_GBS, 3)}
    del q
    mlp = workloads.build_dense_mlp(c2, dev)
    del w13b
    for M in c2.Ms:
        x = c2.x(M, dev)
        ids = torch.zeros((M, 1), dtype=torch.int32, device=dev)
        wt = torch.ones((M, 1), dtype=torch.float32, device=dev)
        ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE, M, 1, 1, c2.H, c2.I), dtype=torch.uint8, device=dev)
        out = torch.empty((M, c2.H), dtype=torch.bfloat16, device=dev)
        f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, mlp.w13, mlp.w2, out=out, ws=ws)
        f()
        ms = time_loop(f, it, st)
        flops = 2.0 * M * 3 * c2.H * c2.I
        wbytes = 3 * c2.H * c2.I * 0.5625
        res[f"dense_mlp_M{M}"] = {"ms": round(ms, 4), "TFLOPs": round(flops / ms / 1e9, 2),
                                  "weight_GBps": gbs(wbytes, ms),
                                  "frac_f16_peak": round(flops / ms / 1e9 / PEAK_F16_TFLOPS, 4),
                                  "frac_hbm_weights": round(gbs(wbytes, ms) / PEAK_HBM_GBS, 4)}
        log(f"breakdown: dense MLP M={M}: {ms:.3f} ms")
    del mlp
    torch.cuda.empty_cache()

    # MX-native W4A8 (MXFP8 activations x MXFP4 weights) on the 8192 x 4096 x
    # 7168 GEMM, and the MXFP8 activation encode
    log("breakdown: MX W4A8 GEMM")
    Mm, Nm, Km = 8192, 4096, 7168
    xa = synth.normal_bf16((Mm, Km), 1.0, (860, Mm, Km), dev)
    wm = synth.normal_bf16((Nm, Km), 0.02, (861, Nm, Km), dev)
    q8, q8e = nv.mxfp8_quantize(xa)
    wp4, we4 = nv.mxfp4_quantize(wm)
    del wm
    cm = torch.empty((Mm, Nm), dtype=torch.bfloat16, device=dev)
    f = lambda: nv.mx_gemm_w4a8(q8, q8e, wp4, we4, out=cm)
    f()
    ms = time_loop(f, it, st)
    ms_q = time_loop(lambda: nv.mxfp8_quantize(xa), it, st)
    tf = 2.0 * Mm * Nm * Km / ms / 1e9
    res["mx_w4a8_gemm_8192x4096x7168"] = {
        "ms": round(ms, 4), "TFLOPs": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
        "frac_f16_peak": round(tf / PEAK_F16_TFLOPS, 4),
        "mxfp8_quantize_ms": round(ms_q, 4), "mxfp8_quantize_GBps": gbs(Mm * Km * (2 + 1 + 1 / 32), ms_q),
        "quantize_bytes_basis": "2 B/elem bf16 read + 1 B E4M3 + 1/32 B scale written"}
    del xa, q8, q8e, wp4, we4, cm
    torch.cuda.empty_cache()

    # 512-expert top-10 MoE
    c3 = synth.C3
    log("breakdown: 512-expert MoE")
    W = workloads.build_moe_weights(c3, dev)
    x = c3.x(dev)
    ids, wt = workloads.routing(c3, dev)
    ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE, c3.T, c3.k, c3.E, c3.H, c3.I), dtype=torch.uint8, device=dev)
    out = torch.empty((c3.T, c3.H), dtype=torch.bfloat16, device=dev)
    f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, W.w13, W.w2, out=out, ws=ws)
    f()
    ms = time_loop(f, it, st)
    flops = 2.0 * c3.T * c3.k * 3 * c3.H * c3.I
    wbytes = c3.E * 3 * c3.H * c3.I * 0.5625
    res["moe_512e_top10_T4096"] = {"ms": round(ms, 4), "TFLOPs": round(flops / ms / 1e9, 2),
                                   "weight_GBps": gbs(wbytes, ms)}
    del W, ws, out
    torch.cuda.empty_cache()

    res.update(decode_rows(dev, st, it))

    # MX-native W4A8 layer on the 384-expert prefill batch (MXFP4 experts,
    # MXFP8 activations on the scaled FP8 x FP4 MFMA)
    cp = synth.C4_PREFILL
    log("breakdown: MX W4A8 MoE prefill")
    Wm = workloads.build_moe_weights(cp, dev, keep_mx=True)
    del Wm.w13, Wm.w2
    (m13, e13), (m2, e2) = Wm.mx13, Wm.mx2
    xm = cp.x(dev)
    idm, wtm = workloads.routing(cp, dev)
    mws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MX_MOE, cp.T, cp.k, cp.E, cp.H, cp.I), dtype=torch.uint8,
                      device=dev)
    outm = torch.empty((cp.T, cp.H), dtype=torch.bfloat16, device=dev)
    f = lambda: nv.mx_moe_w4a8(xm, idm, wtm, m13, e13, m2, e2, out=outm, ws=mws)
    f()
    ms = time_loop(f, 5, st)
    flops = 2.0 * cp.T * cp.k * 3 * cp.H * cp.I
    res["moe_384e_top8_mx_w4a8_prefill_T16384"] = {
        "ms": round(ms, 4), "TFLOPs": round(flops / ms / 1e9, 1), "frac_fp8_peak": round(flops / ms / 1e9 / PEAK_FP8_TFLOPS, 4),
        "frac_f16_peak": round(flops / ms / 1e9 / PEAK_F16_TFLOPS, 4)}
    del Wm, mws, outm, xm
    torch.cuda.empty_cache()

    # KV cache 262144 x 4 x 256
    c5 = synth.C5
    log("breakdown: n-gram table gather-dequant")
    # one of the 128 shards of a 20M-row x 2560 NVFP4 n-gram table; 16384 lookups
    V, D, n = 20000000 // 128, 2560, 16384
    tab = nv.NVFP4Tensor.empty(V, D, 1, dev)
    for r0 in range(0, V, 16384):
        r1 = min(V, r0 + 16384)
        blk = synth.normal_bf16((r1 - r0, D), 0.05, (740, r0), dev)
        nv.nvfp4_quantize(blk, static_global=torch.tensor([0.05 * 5 / 2688], device=dev),
                          out=nv.NVFP4Tensor(tab.packed[:, r0:r1], tab.scales[:, r0:r1], tab.global_, r1 - r0, D, 1))
    tab.global_.fill_(0.05 * 5 / 2688)
    gids = torch.randint(0, V, (n,), dtype=torch.int32, device=dev, generator=torch.Generator(device=dev).manual_seed(741))
    gout = torch.empty((n, D), dtype=torch.bfloat16, device=dev)
    lib = _lib.load()
    tcs = tab.c()
    f = lambda: lib.nvfp4_gather_dequantize(ctypes.byref(tcs), ctypes.c_void_p(gids.data_ptr()), n,
                                            ctypes.c_void_p(gout.data_ptr()), _lib.BF16, ctypes.c_void_p(st.cuda_stream))
    f()
    ms = time_loop(f, it, st)
    gb = n * D * (0.5625 + 2)
    res["gather_dequant_ngram_shard_156250x2560_n16384"] = {
        "ms": round(ms, 4), "GBps": gbs(gb, ms), "bytes_basis": "0.5625 B/elem read (codes + scales of the looked-up rows) + 2 B/elem bf16 written",
        "frac_hbm": round(gbs(gb, ms) / PEAK_HBM_GBS, 4)}
    del tab, gout, gids
    torch.cuda.empty_cache()

    log("breakdown: KV cache")
    kk, vv = c5.k(dev), c5.v(dev)
    kc = nv.NVFP4Tensor.empty(c5.tokens * c5.heads, c5.dim, 1, dev)
    vc = nv.NVFP4Tensor.empty(c5.tokens * c5.heads, c5.dim, 1, dev)
    kc.global_.fill_(float(kk.float().abs().max()) / 2688)
    vc.global_.fill_(float(vv.float().abs().max()) / 2688)

    def write_all():
        for c0 in range(0, c5.tokens, c5.chunk):
            nv.nvfp4_kv_quant(kk[c0:c0 + c5.chunk], vv[c0:c0 + c5.chunk], c0, kc, vc, c5.heads)

    write_all()
    ms_w = time_loop(write_all, 3, st)
    # the same 128 chunk writes replayed from a captured HIP graph, as a
    # serving loop issues them (no host overhead per chunk)
    side = torch.cuda.Stream()
    side.wait_stream(st)
    with torch.cuda.stream(side):
        write_all()
    st.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        write_all()
    graph.replay()
    ms_wg = time_loop(graph.replay, 5, st)
    ms_w1 = time_loop(lambda: nv.nvfp4_kv_quant(kk, vv, 0, kc, vc, c5.heads), it, st)
    ko = torch.empty((c5.tokens, c5.heads, c5.dim), dtype=torch.bfloat16, device=dev)
    ms_r = time_loop(lambda: nv.nvfp4_kv_dequant(kc, vc, c5.heads, 0, c5.tokens, torch.bfloat16), it, st)
    nel = 2 * c5.tokens * c5.heads * c5.dim
    res["kv_262144x4x256"] = {"write_128_chunks_ms": round(ms_w, 4), "write_chunked_GBps": gbs(2.5625 * nel, ms_w),
                              "write_128_chunks_graph_ms": round(ms_wg, 4),
                              "write_chunked_graph_GBps": gbs(2.5625 * nel, ms_wg),
                              "write_single_call_ms": round(ms_w1, 4),
                              "write_single_GBps": gbs(2.5625 * nel, ms_w1),
                              "read_ms": round(ms_r, 4), "read_GBps": gbs(2.5625 * nel, ms_r),
                              "frac_hbm_read": round(gbs(2.5625 * nel, ms_r) / PEAK_HBM_GBS, 4)}
    return res


if __name__ == "__main__":
    main()
