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
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, at
                one thread and on all the host cores it may use, plus
                full-tensor timings of the quantize, dequantize, remap and KV
                oracles;
  breakdown     the other hot-path rows (quantize, remap, KV cache, dense
                MLP, 512-expert MoE, decode MoE, ...) on their own configs,
                each with its bound (hbm or mfma), its lower bound t_min and
                frac = t_min / measured time.  Bandwidth-bound rows read a
                512 MB buffer before every timed iteration, so they start
                with no operand in L2 or the last-level cache.

--only <group> runs one group of rows and prints their JSON (for rocprofv3).
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
FLUSH_BYTES = 512 << 20    # larger than the 256 MB last-level cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_moe384_T16384.json")
# sources that shape the grouped gate_up launch (kernels, tile plan, class dispatch)
GEMM_SOURCES = ["precision_moe_gemm_amd/csrc/gemm.h", "precision_moe_gemm_amd/csrc/common.h",
                "precision_moe_gemm_amd/csrc/moe.h", "precision_moe_gemm_amd/csrc/libnvfp4.hip"]
GROUPS = ("prefill", "gate_up", "quantize", "mlp", "mx", "c3", "decode", "mx_prefill", "gather", "kv", "ceiling")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the breakdown of other rows")
    ap.add_argument("--only", choices=GROUPS, help="run one group of rows only (profiling)")
    ap.add_argument("--iters", type=int, default=10, help="timed iterations per breakdown row")
    ap.add_argument("--profile-copy", action="store_true",
                    help="also launch a 1 GiB plain copy (counter calibration)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the gate_up traffic summary from two rocprofv3 --pmc runs (FETCH_SIZE, "
                         "WRITE_SIZE) of --only gate_up --profile-copy, then exit (no GPU use)")
    return ap.parse_args()


# kernels of one nvfp4_moe_gate_up call on the 384-expert prefill layer
TRAFFIC_KERNELS = {"moe_plan_kernel": r"moe_plan_kernel",
                   "gemm_rtile_kernel<256,256,1,true>": r"gemm_rtile_kernel<256, 256, 1, true>",
                   "gemm_rtile_kernel<128,256,1,true>": r"gemm_rtile_kernel<128, 256, 1, true>",
                   "gemm_stream_kernel<1,true,false,16>": r"gemm_stream_kernel<1, true, false, 16>"}


def _pmc_per_dispatch(d, counter):
    """Mean per dispatch of `counter` (summed over its instances) for every
    kernel in the rocprofv3 counter CSV under directory d; the copyBuffer
    dispatches are kept apart (largest one)."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out, copy = {}, 0.0
    for name, short in TRAFFIC_KERNELS.items():
        vals = [v for (k, _), v in per.items() if short in k]
        if vals:
            out[name] = sum(vals) / len(vals)
    copies = [v for (k, _), v in per.items() if "copyBuffer" in k]
    copy = max(copies) if copies else 0.0
    return out, copy


def write_traffic(fetch_dir, write_dir):
    fetch, fcopy = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write, wcopy = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    if not fcopy or not wcopy:
        raise SystemExit("the 1 GiB calibration copy (--profile-copy) is missing from the counter runs")
    gib = 1 << 30
    ff, wf = gib / (fcopy * 1024), gib / (wcopy * 1024)
    fb = sum(fetch.values()) * 1024 * ff
    wb = sum(write.values()) * 1024 * wf
    cmd = ("cd /tmp && TMPDIR=/tmp timeout -s KILL 150 rocprofv3 --pmc {c} --kernel-include-regex "
           "'gemm_rtile_kernel|gemm_stream|moe_plan|copyBuffer' --output-format csv -d {d} -o p -- "
           "python3 $R/bench.py --only gate_up --steps 2 --warmup 1 --profile-copy")
    t = {"what": "HBM traffic of one grouped gate_up call (nvfp4_moe_gate_up) of the 384-expert top-8 layer at "
                 "T=16384: tile plan + 256-row and 128-row register-decode tile kernels and the 16-row streaming "
                 "kernel (power-of-two weight-scale variants)",
         "commands": [cmd.format(c="FETCH_SIZE", d=fetch_dir), cmd.format(c="WRITE_SIZE", d=write_dir),
                      f"python3 $R/bench.py --write-traffic {fetch_dir} {write_dir}"],
         "fetch_kib_per_dispatch": {k: round(v, 1) for k, v in fetch.items()},
         "write_kib_per_dispatch": {k: round(v, 1) for k, v in write.items()},
         "calibration": {"kernel": "__amd_rocclr_copyBuffer, the 1 GiB copy of --profile-copy (largest dispatch)",
                         "bytes_read": gib, "bytes_written": gib, "fetch_kib": fcopy, "write_kib": wcopy,
                         "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
         "fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
         "bytes_per_launch": int(fb + wb),
         "algorithmic_bytes_per_launch_note": "minimum: gathered x rows 131072 x 7168 x 0.5625 B + touched "
                                              "experts' w13 225 x 4096 x 7168 x 0.5625 B + h 131072 x 2048 x 2 B "
                                              "= 4.77e9 B",
         "source_hash": source_hash(), "sources": GEMM_SOURCES}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    print(json.dumps({"bytes_per_launch": t["bytes_per_launch"], "file": TRAFFIC_FILE}))


def source_hash():
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
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


class Timer:
    """HIP-event timing on one stream.  With flush=True every iteration first
    reads a 512 MB buffer (outside the timed region), so the operands of the
    timed call come from HBM, not from L2 or the last-level cache."""

    def __init__(self, stream, device):
        import torch
        self.torch = torch
        self.stream = stream
        self.flushbuf = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=device)

    def __call__(self, fn, iters, flush=False):
        torch = self.torch
        if not flush:
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record(self.stream)
            for _ in range(iters):
                fn()
            end.record(self.stream)
            end.synchronize()
            return start.elapsed_time(end) / iters
        evs = []
        for _ in range(iters):
            self.flushbuf.amax()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            fn()
            b.record(self.stream)
            evs.append((a, b))
        evs[-1][1].synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / iters


def row(ms, nbytes=None, flops=None, peak_tflops=PEAK_F16_TFLOPS, **extra):
    """One breakdown row: the lower bound t_min = max(bytes / 8 TB/s, flops /
    MFMA peak), its bound and frac = t_min / ms."""
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e6) if nbytes else 0.0
    t_mma = flops / (peak_tflops * 1e9) if flops else 0.0
    t_min = max(t_hbm, t_mma)
    d = {"ms": round(ms, 4), "bound": "hbm" if t_hbm >= t_mma else "mfma", "t_min_ms": round(t_min, 4),
         "frac": round(t_min / ms, 4)}
    if nbytes:
        d["GBps"] = round(nbytes / ms / 1e6, 1)
    if flops:
        d["TFLOPs"] = round(flops / ms / 1e9, 2)
        d["mfma_peak_TFLOPs"] = peak_tflops
    d.update(extra)
    return d


def cpu_threads():
    """Host threads this process may use (the GPU machine's share is 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.stderr.write("bench.py: multi-GPU runs are not part of this build (one GPU only)\n")
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    timer = Timer(stream, dev)
    if args.profile_copy:
        # a plain 1 GiB copy: its FETCH_SIZE / WRITE_SIZE readings calibrate
        # the counters against known bytes
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.only and args.only not in ("prefill", "gate_up"):
        print(json.dumps(breakdown(args, timer, only=args.only)))
        return
    result, ctx = headline(args, timer, dev, stream)
    if args.only:
        print(json.dumps(result), flush=True)
        return
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ctx)
    if not args.no_extras:
        static_res, tiled_res = ctx.pop("static_res"), ctx.pop("tiled_res")
        ctx.clear()
        torch.cuda.empty_cache()
        result["breakdown"] = breakdown(args, timer)
        result["breakdown"]["moe_384e_prefill_static_globals"] = static_res
        result["breakdown"]["moe_384e_prefill_tiled_scales"] = tiled_res
    print(json.dumps(result), flush=True)


def headline(args, timer, dev, stream):
    import ctypes

    import numpy as np
    import torch

    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib, synth, workloads

    cfg = synth.C4_PREFILL
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    log(f"building {E} MXFP4-origin experts (H={H}, I={I}) and routing T={T}")
    t0 = time.time()
    W = workloads.build_moe_weights(cfg, dev)
    x = cfg.x(dev)
    ids, w = workloads.routing(cfg, dev)
    ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE, T, k, E, H, I), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    flops = 2.0 * T * k * 3 * H * I
    result = {}
    ms = None
    if args.only != "gate_up":
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
        ms = timer(step, args.steps)
        torch.cuda.synchronize()
        log(f"MoE prefill: {ms:.3f} ms/step, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")

    # ---- dominant kernel: the grouped gate_up GEMM, timed on its stream ----
    xq = nv.nvfp4_quantize(x)
    perm, offsets, inv = nv.nvfp4_moe_route(ids, E)
    route_ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE_ROUTE, T, k, E, H, I), dtype=torch.uint8, device=dev)
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    hmax = torch.zeros(1, dtype=torch.int32, device=dev)
    counts = (offsets[1:] - offsets[:-1]).cpu().numpy()
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
    gu_ms = timer(gate_up, max(5, args.steps))
    gu_flops = 2.0 * T * k * (2 * I) * H
    gu_tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    log(f"gate_up: {gu_ms:.3f} ms/launch, {gu_tflops:.1f} TFLOP/s")
    roofline = {
        "bound": "mfma", "achieved": round(gu_tflops, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(gu_tflops / PEAK_F16_TFLOPS, 4), "traffic": load_traffic(),
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
                      "f16 MFMA path (2.5 PFLOP/s dense), whose ceiling is half the FP8 and a "
                      "quarter of the FP4 peak",
        "fp4_fp8_target_met": bool(gu_tflops / PEAK_FP8_TFLOPS >= 0.5),
    }
    if args.only == "gate_up":
        return {"gate_up_ms": round(gu_ms, 4), "TFLOPs": round(gu_tflops, 2)}, {}
    result = {
        "metric": "W4A4 MoE grouped-GEMM TFLOP/s (NVFP4, 384 experts top-8, prefill 16384 tokens)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
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
        "layer_frac_f16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
    }
    if args.only == "prefill":
        return result, {}
    # ---- the same layer with calibrated (static) globals: the gate_up
    # epilogue encodes h to NVFP4 itself (no bf16 h, no h quantize pass) ----
    static_res = None
    if not args.no_extras:
        gh = float(np.uint32(hmax.item()).view(np.float32)) / 2688.0
        sg = torch.tensor([float(xq.global_[0].item()), gh], dtype=torch.float32, device=dev)

        def step_static():
            nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2, static_in_globals=sg, out=out, ws=ws)

        step_static()
        sms = timer(step_static, max(5, args.steps))
        log(f"MoE prefill, static globals: {sms:.3f} ms/step")
        static_res = row(sms, flops=flops, globals="G_x, G_h = amax/2688 of this input (calibrated); h "
                                                   "encoded in the gate_up epilogue")
    # ---- the same layer with the experts' scale bytes in the 128-row tiled
    # order (prepared once, outside the timed region) ----
    tiled_res = None
    if not args.no_extras:
        w13t, w2t = nv.nvfp4_tile_scales(W.w13), nv.nvfp4_tile_scales(W.w2)

        def step_tiled():
            nv.nvfp4_moe_grouped_gemm(x, ids, w, w13t, w2t, out=out, ws=ws)

        step_tiled()
        tms = timer(step_tiled, max(5, args.steps))
        log(f"MoE prefill, tiled weight scales: {tms:.3f} ms/step")
        tiled_res = row(tms, flops=flops, weights="scale bytes in the 128-row tiled order")
        del w13t, w2t
    ctx = dict(cfg=cfg, x=x, perm=perm, offsets=offsets, static_res=static_res, tiled_res=tiled_res)
    return result, ctx


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def _pool_time(fn, jobs, threads):
    """Wall time of fn over jobs on `threads` host threads (the oracle's C
    calls release the GIL); returns (seconds, results)."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    if threads == 1:
        res = [fn(j) for j in jobs]
    else:
        with ThreadPoolExecutor(threads) as pool:
            res = list(pool.map(fn, jobs))
    return time.perf_counter() - t0, res


def cpu_baseline(ctx):
    """The oracle as it stands (plain C, one call per job) on the GPU machine's
    host: the headline layer on (token, slot) pairs of the most-loaded
    expert at one thread and on every allowed core (the harness spreads
    pairs over threads; the oracle itself is single-threaded), and
    full-tensor timings of the quantize, dequantize, remap and KV oracles."""
    import numpy as np
    import oracle
    from precision_moe_gemm_amd import synth
    cfg, x, perm, offsets = ctx["cfg"], ctx["x"], ctx["perm"], ctx["offsets"]
    H, I, k = cfg.H, cfg.I, cfg.k
    nthr = cpu_threads()
    off = offsets.cpu().numpy()
    e = int(np.argmax(off[1:] - off[:-1]))
    n1, nall = 24, 8 * nthr
    pairs = perm.cpu().numpy()[off[e]:off[e] + nall]
    toks = pairs // k
    log(f"cpu baseline: preparing expert {e} weights with the oracle ({nthr} threads)")
    w13 = oracle.mxfp4_to_nvfp4(*oracle.mxfp4_encode(synth.bits(cfg.w13(e, "cuda"))))
    w2 = oracle.mxfp4_to_nvfp4(*oracle.mxfp4_encode(synth.bits(cfg.w2(e, "cuda"))))
    xs_all = synth.bits(x[_dev_index(toks)])
    gx = oracle.global_from_amax(float(x.float().abs().max().item()))
    ex13 = oracle.Experts(w13.packed[None], w13.scales[None], np.array([w13.G], np.float32))
    ex2 = oracle.Experts(w2.packed[None], w2.scales[None], np.array([w2.G], np.float32))
    gh = np.float32(1.0)

    def layer(rows):
        # x-row quantize, exact gate_up + SwiGLU, h quantize (static G_h), exact down
        n = rows.size
        xq = oracle.quantize(np.ascontiguousarray(xs_all[rows]), static_G=gx)
        lperm = np.arange(n, dtype=np.int32)      # sample row i is pair i (k = 1 view)
        loff = np.array([0, n], np.int32)
        hh = oracle.moe_gate_up(xq, lperm, loff, 1, ex13, np.arange(n))
        hq = oracle.quantize(hh, static_G=gh)
        oracle.moe_down(hq, loff, ex2, np.arange(n))
        return n

    log(f"cpu baseline: layer, {n1} pairs on 1 thread, {nall} on {nthr}")
    t1, _ = _pool_time(layer, [np.arange(n1)], 1)
    tall, _ = _pool_time(layer, [np.arange(i, i + 4) for i in range(0, nall, 4)], nthr)
    fl = 2.0 * 3 * H * I
    out = {"value": round(fl * nall / tall / 1e12, 6), "unit": "TFLOP/s", "cores": nthr, "kind": "oracle",
           "seconds": round(tall, 2),
           "sample": f"{nall} (token, slot) pairs of expert {e} (the most loaded): x-row quantize, exact "
                     f"int64 gate_up + SwiGLU, h quantize, exact down, 4 pairs per oracle call spread over "
                     f"{nthr} threads; weights prepared by the oracle outside the timed region",
           "single_thread": {"value": round(fl * n1 / t1 / 1e12, 6), "unit": "TFLOP/s", "seconds": round(t1, 2),
                             "sample": f"{n1} pairs in one call"},
           "nproc": os.cpu_count(), "threads_allowed": nthr, "cpu_model": cpu_model()}
    out["full_tensor"] = cpu_full_tensors(nthr)
    return out


def cpu_full_tensors(nthr):
    """Oracle quantize / dequantize / remap / KV on full tensors of the
    workloads: all-core (row chunks over threads, the global computed over
    the whole tensor first) and one thread on a slice (rows are independent
    given the global), in elements per second."""
    import numpy as np
    import oracle
    from precision_moe_gemm_amd import synth
    res = {}

    def rate(nel, sec):
        return round(nel / sec / 1e6, 2)

    def chunks(R, n):
        step = max(1, (R + n - 1) // n)
        return [(r, min(R, r + step)) for r in range(0, R, step)]

    # quantize / dequantize: the 27B gate_up weight, 34816 x 5120
    log("cpu baseline: full-tensor quantize / dequantize (34816 x 5120)")
    w = synth.bits(synth.C2.w13("cuda"))
    R, K = w.shape
    G = oracle.global_from_amax(oracle.amax_bf16(w))
    jobs = chunks(R, 4 * nthr)
    q = lambda rr: oracle.quantize(np.ascontiguousarray(w[rr[0]:rr[1]]), static_G=G)
    tq, parts = _pool_time(q, jobs, nthr)
    s1 = R // 32
    tq1, _ = _pool_time(q, [(0, s1)], 1)
    res["quantize_34816x5120"] = {"Melem_per_s_all_cores": rate(R * K, tq), "seconds_all_cores": round(tq, 2),
                                  "Melem_per_s_1_thread": rate(s1 * K, tq1),
                                  "one_thread_sample": f"{s1} rows"}
    dq = lambda p: oracle.dequantize(p)
    td, _ = _pool_time(dq, parts, nthr)
    td1, _ = _pool_time(dq, [parts[0].rows(0, min(s1, parts[0].shape[0]))], 1)
    res["dequantize_34816x5120"] = {"Melem_per_s_all_cores": rate(R * K, td), "seconds_all_cores": round(td, 2),
                                    "Melem_per_s_1_thread": rate(min(s1, parts[0].shape[0]) * K, td1)}
    del w, parts
    # remap: one expert's fused [w1; w3] of the 384-expert layer (one tensor,
    # one global: a single oracle call)
    log("cpu baseline: full-tensor remap (4096 x 7168)")
    c4 = synth.C4_PREFILL
    mp, me = oracle.mxfp4_encode(synth.bits(c4.w13(0, "cuda")))
    tr, _ = _pool_time(lambda a: oracle.mxfp4_to_nvfp4(*a), [(mp, me)], 1)
    res["remap_4096x7168"] = {"Melem_per_s_1_thread": rate(mp.size * 2, tr), "seconds": round(tr, 2),
                              "note": "one tensor is one oracle call (its global spans the tensor): one thread"}
    # KV cache: the whole K tensor (262144 x 4 x 256) written and read
    log("cpu baseline: full-tensor KV write / read (262144 x 4 x 256)")
    c5 = synth.C5
    kb = synth.bits(c5.k("cuda")).reshape(c5.tokens * c5.heads, c5.dim)
    Gk = oracle.global_from_amax(oracle.amax_bf16(kb))
    jobs = chunks(kb.shape[0], 4 * nthr)
    qk = lambda rr: oracle.quantize(np.ascontiguousarray(kb[rr[0]:rr[1]]), static_G=Gk)
    tk, parts = _pool_time(qk, jobs, nthr)
    ck = c5.chunk * c5.heads
    tk1, _ = _pool_time(qk, [(0, ck)], 1)
    tkr, _ = _pool_time(dq, parts, nthr)
    nel = kb.size
    res["kv_write_K_262144x4x256"] = {"Melem_per_s_all_cores": rate(nel, tk), "seconds_all_cores": round(tk, 2),
                                      "Melem_per_s_1_thread": rate(ck * c5.dim, tk1),
                                      "one_thread_sample": "one 2048-token chunk"}
    res["kv_read_K_262144x4x256"] = {"Melem_per_s_all_cores": rate(nel, tkr), "seconds_all_cores": round(tkr, 2)}
    return res


def _dev_index(a):
    import torch
    return torch.from_numpy(a).to("cuda")


# ---------------------------------------------------------------------------
# other rows
# ---------------------------------------------------------------------------

def breakdown(args, timer, only=None):
    """Other hot-path rows on their own configs, each timed with HIP events."""
    import torch
    res = {}
    it = args.iters
    groups = [only] if only else ["quantize", "mlp", "mx", "c3", "decode", "mx_prefill", "gather", "kv", "ceiling"]
    for gname in groups:
        res.update(ROWS[gname](timer, it))
        torch.cuda.empty_cache()
    return res


def rows_quantize(timer, it):
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import synth
    dev = torch.device("cuda:0")
    log("breakdown: weight quantize 34816 x 5120")
    w13b = synth.C2.w13(dev)
    n = w13b.numel()
    g = torch.tensor([0.01], device=dev)
    q = nv.nvfp4_quantize(w13b, static_global=g)
    qws = torch.empty(4096, dtype=torch.uint8, device=dev)
    ms_s = timer(lambda: nv.nvfp4_quantize(w13b, static_global=g, out=q), it, flush=True)
    ms_d = timer(lambda: nv.nvfp4_quantize(w13b, out=q, ws=qws), it, flush=True)
    return {"quantize_static_34816x5120": row(ms_s, 2.5625 * n, bytes_basis="bf16 read + codes + scales, "
                                                                            "2.5625 B/elem"),
            "quantize_dynamic_34816x5120": row(ms_d, 4.5625 * n, bytes_basis="amax pass + encode pass, "
                                                                             "4.5625 B/elem")}


def rows_mlp(timer, it):
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib, synth, workloads
    dev = torch.device("cuda:0")
    c2 = synth.C2
    log("breakdown: dense MLP 5120/17408 as one expert")
    mlp = workloads.build_dense_mlp(c2, dev)
    mlp_t = workloads.MoEWeights(nv.nvfp4_tile_scales(mlp.w13), nv.nvfp4_tile_scales(mlp.w2))
    res = {}
    for M in c2.Ms:
        x = c2.x(M, dev)
        ids = torch.zeros((M, 1), dtype=torch.int32, device=dev)
        wt = torch.ones((M, 1), dtype=torch.float32, device=dev)
        ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE, M, 1, 1, c2.H, c2.I), dtype=torch.uint8, device=dev)
        out = torch.empty((M, c2.H), dtype=torch.bfloat16, device=dev)
        f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, mlp.w13, mlp.w2, out=out, ws=ws)
        f()
        flops = 2.0 * M * 3 * c2.H * c2.I
        wbytes = 3 * c2.H * c2.I * 0.5625
        if M <= 32:
            ms = timer(f, it, flush=True)
            res[f"dense_mlp_M{M}"] = row(ms, wbytes, flops, bytes_basis="NVFP4 weights, 0.5625 B/elem")
            # weight scale bytes in the 128-row tiled order
            ft = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, mlp_t.w13, mlp_t.w2, out=out, ws=ws)
            ft()
            res[f"dense_mlp_M{M}_tiled_scales"] = row(timer(ft, it, flush=True), wbytes, flops,
                                                      bytes_basis="NVFP4 weights, 0.5625 B/elem")
        else:
            ms = timer(f, it)
            res[f"dense_mlp_M{M}"] = row(ms, None, flops)
        log(f"breakdown: dense MLP M={M}: {ms:.3f} ms")
    return res


def rows_mx(timer, it):
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import synth
    dev = torch.device("cuda:0")
    log("breakdown: MX W4A8 GEMM 8192 x 4096 x 7168")
    Mm, Nm, Km = 8192, 4096, 7168
    xa = synth.normal_bf16((Mm, Km), 1.0, (860, Mm, Km), dev)
    wm = synth.normal_bf16((Nm, Km), 0.02, (861, Nm, Km), dev)
    q8, q8e = nv.mxfp8_quantize(xa)
    wp4, we4 = nv.mxfp4_quantize(wm)
    cm = torch.empty((Mm, Nm), dtype=torch.bfloat16, device=dev)
    f = lambda: nv.mx_gemm_w4a8(q8, q8e, wp4, we4, out=cm)
    f()
    ms = timer(f, it)
    ms_q = timer(lambda: nv.mxfp8_quantize(xa), it, flush=True)
    return {"mx_w4a8_gemm_8192x4096x7168": row(ms, None, 2.0 * Mm * Nm * Km, PEAK_FP8_TFLOPS,
                                               note="fp8 x fp4 scaled MFMA: FP8 peak"),
            "mxfp8_quantize_8192x7168": row(ms_q, Mm * Km * (2 + 1 + 1 / 32),
                                            bytes_basis="bf16 read + E4M3 + 1/32 B scale written")}


def rows_c3(timer, it):
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib, synth, workloads
    dev = torch.device("cuda:0")
    c3 = synth.C3
    log("breakdown: 512-expert MoE")
    W = workloads.build_moe_weights(c3, dev)
    x = c3.x(dev)
    ids, wt = workloads.routing(c3, dev)
    ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE, c3.T, c3.k, c3.E, c3.H, c3.I), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((c3.T, c3.H), dtype=torch.bfloat16, device=dev)
    f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, W.w13, W.w2, out=out, ws=ws)
    f()
    ms = timer(f, it, flush=True)
    flops = 2.0 * c3.T * c3.k * 3 * c3.H * c3.I
    wbytes = c3.E * 3 * c3.H * c3.I * 0.5625
    w13t, w2t = nv.nvfp4_tile_scales(W.w13), nv.nvfp4_tile_scales(W.w2)
    f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, w13t, w2t, out=out, ws=ws)
    f()
    mst = timer(f, it, flush=True)
    return {"moe_512e_top10_T4096": row(ms, wbytes, flops, bytes_basis="all 512 experts' NVFP4 weights"),
            "moe_512e_top10_T4096_tiled_scales": row(mst, wbytes, flops,
                                                     bytes_basis="all 512 experts' NVFP4 weights")}


def rows_decode(timer, it):
    """The 384-expert decode batch (T=64): fused layer with dynamic and with
    calibrated globals, the W4A16 and MX W4A8 layers on the same experts, and
    the MXFP4 -> NVFP4 remap of the 384 experts' w13."""
    import numpy as np
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib, synth, workloads
    dev = torch.device("cuda:0")
    res = {}
    c4 = synth.C4_DECODE
    log("breakdown: 384-expert decode + remap")
    W = workloads.build_moe_weights(c4, dev, keep_mx=True)
    x = c4.x(dev)
    ids, wt = workloads.routing(c4, dev)
    ws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MOE, c4.T, c4.k, c4.E, c4.H, c4.I), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((c4.T, c4.H), dtype=torch.bfloat16, device=dev)
    touched = np.unique(ids.cpu().numpy())
    wbytes = len(touched) * 3 * c4.H * c4.I * 0.5625
    basis = f"NVFP4 weights of the {len(touched)} touched experts, 0.5625 B/elem"
    f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, W.w13, W.w2, out=out, ws=ws)
    f()
    res["moe_384e_top8_decode_T64"] = row(timer(f, it, flush=True), wbytes, bytes_basis=basis,
                                          experts_touched=int(len(touched)))
    # the same experts with their scale bytes in the 128-row tiled order
    # (prepared once, outside the timed region)
    w13t, w2t = nv.nvfp4_tile_scales(W.w13), nv.nvfp4_tile_scales(W.w2)
    f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, w13t, w2t, out=out, ws=ws)
    f()
    res["moe_384e_top8_decode_T64_tiled_scales"] = row(timer(f, it, flush=True), wbytes, bytes_basis=basis)
    # calibrated globals (from one dynamic staged pass): h encoded in the epilogue
    xq4 = nv.nvfp4_quantize(x)
    perm4, off4, _ = nv.nvfp4_moe_route(ids, c4.E)
    _, hmax4 = nv.nvfp4_moe_gate_up(xq4, perm4, off4, c4.k, W.w13)
    sg4 = torch.tensor([float(xq4.global_[0].item()),
                        float(np.uint32(hmax4.item()).view(np.float32)) / 2688.0],
                       dtype=torch.float32, device=dev)
    f = lambda: nv.nvfp4_moe_grouped_gemm(x, ids, wt, W.w13, W.w2, static_in_globals=sg4, out=out, ws=ws)
    f()
    res["moe_384e_top8_decode_T64_static_globals"] = row(timer(f, it, flush=True), wbytes, bytes_basis=basis)
    f = lambda: nv.nvfp4_moe_w4a16(x, ids, wt, W.w13, W.w2, out=out, ws=ws)
    f()
    res["moe_384e_top8_w4a16_decode_T64"] = row(timer(f, it, flush=True), wbytes, bytes_basis=basis)
    f = lambda: nv.nvfp4_moe_w4a16(x, ids, wt, w13t, w2t, out=out, ws=ws)
    f()
    res["moe_384e_top8_w4a16_decode_T64_tiled_scales"] = row(timer(f, it, flush=True), wbytes, bytes_basis=basis)
    del w13t, w2t
    (m13, e13), (m2, e2) = W.mx13, W.mx2
    mws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_MX_MOE, c4.T, c4.k, c4.E, c4.H, c4.I), dtype=torch.uint8,
                      device=dev)
    f = lambda: nv.mx_moe_w4a8(x, ids, wt, m13, e13, m2, e2, out=out, ws=mws)
    f()
    mx_bytes = len(touched) * 3 * c4.H * c4.I * (0.5 + 1 / 32)
    res["moe_384e_top8_mx_w4a8_decode_T64"] = row(timer(f, it, flush=True), mx_bytes,
                                                  bytes_basis="touched MXFP4 experts: 0.5 + 1/32 B/elem")
    del mws
    p13, s13 = W.mx13
    dst = nv.NVFP4Tensor.empty(2 * c4.I, c4.H, c4.E, dev)
    rws = torch.empty(nv.nvfp4_workspace_size(_lib.OP_REMAP, c4.E, 0, 0, 2 * c4.I, c4.H), dtype=torch.uint8,
                      device=dev)
    f = lambda: nv.mxfp4_to_nvfp4(p13, s13, 2 * c4.I, c4.H, c4.E, out=dst, ws=rws)
    f()
    nel = c4.E * 2 * c4.I * c4.H
    res["remap_w13_384x4096x7168"] = row(timer(f, 3, flush=True), nel * 1.09375,
                                         bytes_basis="0.5+1/32 B/elem read, 0.5+1/16 B/elem written")
    return res


def rows_mx_prefill(timer, it):
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib, synth, workloads
    dev = torch.device("cuda:0")
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
    ms = timer(f, 5)
    flops = 2.0 * cp.T * cp.k * 3 * cp.H * cp.I
    return {"moe_384e_top8_mx_w4a8_prefill_T16384": row(ms, None, flops, PEAK_FP8_TFLOPS,
                                                        note="fp8 x fp4 scaled MFMA: FP8 peak",
                                                        frac_f16_peak=round(flops / ms / 1e9 / PEAK_F16_TFLOPS, 4))}


def rows_gather(timer, it):
    import ctypes
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import _lib, synth
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    log("breakdown: n-gram table gather-dequant")
    # one of the 128 shards of a 20M-row x 2560 NVFP4 n-gram table; 16384 lookups
    V, D, n = 20000000 // 128, 2560, 16384
    tab = nv.NVFP4Tensor.empty(V, D, 1, dev)
    gt = torch.tensor([0.05 * 5 / 2688], device=dev)
    for r0 in range(0, V, 16384):
        r1 = min(V, r0 + 16384)
        blk = synth.normal_bf16((r1 - r0, D), 0.05, (740, r0), dev)
        nv.nvfp4_quantize(blk, static_global=gt,
                          out=nv.NVFP4Tensor(tab.packed[:, r0:r1], tab.scales[:, r0:r1], tab.global_, r1 - r0, D, 1))
    tab.global_.fill_(0.05 * 5 / 2688)
    gids = torch.randint(0, V, (n,), dtype=torch.int32, device=dev,
                         generator=torch.Generator(device=dev).manual_seed(741))
    gout = torch.empty((n, D), dtype=torch.bfloat16, device=dev)
    lib = _lib.load()
    tcs = tab.c()
    f = lambda: lib.nvfp4_gather_dequantize(ctypes.byref(tcs), ctypes.c_void_p(gids.data_ptr()), n,
                                            ctypes.c_void_p(gout.data_ptr()), _lib.BF16,
                                            ctypes.c_void_p(st.cuda_stream))
    f()
    ms = timer(f, it, flush=True)
    return {"gather_dequant_ngram_shard_156250x2560_n16384": row(
        ms, n * D * (0.5625 + 2), bytes_basis="0.5625 B/elem read (codes + scales of the looked-up rows) + "
                                              "2 B/elem bf16 written")}


def rows_kv(timer, it):
    import torch
    import precision_moe_gemm_amd as nv
    from precision_moe_gemm_amd import synth
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    c5 = synth.C5
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
    ms_w = timer(write_all, 3, flush=True)
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
    ms_wg = timer(graph.replay, 5, flush=True)
    ms_w1 = timer(lambda: nv.nvfp4_kv_quant(kk, vv, 0, kc, vc, c5.heads), it, flush=True)
    ko = torch.empty((c5.tokens, c5.heads, c5.dim), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    ms_r = timer(lambda: nv.nvfp4_kv_dequant(kc, vc, c5.heads, 0, c5.tokens, torch.bfloat16, k_out=ko, v_out=vo),
                 it, flush=True)
    nel = 2 * c5.tokens * c5.heads * c5.dim
    basis = "K and V: bf16 read + codes + scales written (2.5625 B/elem)"
    return {"kv_write_128_chunks_eager": row(ms_w, 2.5625 * nel, bytes_basis=basis),
            "kv_write_128_chunks_graph": row(ms_wg, 2.5625 * nel, bytes_basis=basis),
            "kv_write_single_call": row(ms_w1, 2.5625 * nel, bytes_basis=basis),
            "kv_read_full": row(ms_r, 2.5625 * nel, bytes_basis="K and V: codes + scales read, bf16 written "
                                                                "(2.5625 B/elem)")}


def rows_ceiling(timer, it):
    """Context, not hot-path rows: the read rate this GPU reaches on the
    streaming GEMM's access patterns (csrc/probe/hbm_read.hip), over 778 MB of
    weight-shaped rows (53 experts x 4096 rows x 3584 B, the decode batch's
    touched gate_up codes) plus their 97 MB of scale bytes, a 512 MB flush
    between passes."""
    import ctypes
    import torch
    from precision_moe_gemm_amd import build
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    if not os.path.exists(build.PROBE_LIB):
        raise SystemExit(f"{build.PROBE_LIB} not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(build.PROBE_LIB)
    lib.hbm_read_probe.restype = ctypes.c_int
    lib.hbm_read_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    log("breakdown: HBM read ceiling of the streaming access patterns")
    rows, rb = 53 * 4096, 3584
    w = torch.zeros(rows * rb, dtype=torch.uint8, device=dev)
    sc = torch.zeros(rows * rb // 8, dtype=torch.uint8, device=dev)
    grid = 768  # the streaming GEMM's resident grid (3 workgroups per CU)
    out = torch.empty(grid * 256, dtype=torch.int32, device=dev)
    res = {}
    for name, lanes, rbytes, with_sc, sc_tiled in (("contiguous_16KB_per_stage", 256, 4096, False, 0),
                                                   ("weight_tiles_128rows_x128B", 8, rb, False, 0),
                                                   ("weight_tiles_plus_row_scales_16B", 8, rb, True, 0),
                                                   ("weight_tiles_plus_tiled_scales_2KB", 8, rb, True, 1)):
        n = w.numel() // rbytes
        n -= n % (128 if lanes == 8 else 4)
        nbytes = n * rbytes + (n * rbytes // 8 if with_sc else 0)
        args = (lanes, ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(sc.data_ptr() if with_sc else None), sc_tiled,
                n, rbytes, grid, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.cuda_stream))
        rc = lib.hbm_read_probe(*args)
        if rc != 0:
            raise SystemExit(f"hbm_read_probe({name}) failed: {rc}")
        ms = timer(lambda: lib.hbm_read_probe(*args), it, flush=True)
        res[f"hbm_read_{name}"] = row(ms, nbytes, bytes_basis=f"{nbytes / 1e6:.0f} MB read once")
        log(f"breakdown: read {name}: {nbytes / ms / 1e9:.2f} TB/s")
    return res


ROWS = {"quantize": rows_quantize, "mlp": rows_mlp, "mx": rows_mx, "c3": rows_c3, "decode": rows_decode,
        "mx_prefill": rows_mx_prefill, "gather": rows_gather, "kv": rows_kv, "ceiling": rows_ceiling}


if __name__ == "__main__":
    main()
