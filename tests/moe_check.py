"""Staged oracle check of a routed-expert layer on chosen (token, slot) rows.

Test infrastructure.  The layer runs on the GPU stage by stage (quantize x,
route, gate_up + SwiGLU, quantize h, down, combine); the oracle recomputes
each stage for the chosen list positions from the GPU's inputs to that
stage, following the staged protocol:

  1. x and every expert weight the rows touch: bytes bit-exact vs oracle Q;
  2. route: perm / offsets / inv bit-exact;
  3. h: max|h - R| / max|R| <= 1e-3 + 2^-8 (bf16 output), and element by
     element over |R| >= 1e-2 max|R| within 1e-3 + one bf16 ulp (2^-7);
  4. G_h == amax(h_gpu) / 2688 and hq == oracle Q(h_gpu) bit-exact;
  5. y from the GPU's hq: 1e-3 (max-normalised and element-wise);
  6. out: the oracle combine of the GPU's y on sampled tokens, and the oracle
     down + combine on a few tokens;
  7. the fused entry point equals the staged one.

Each expert's rows form a one-expert sub-problem (offsets [0, n], the
expert's weights only), so a 384-expert layer never needs all experts on the
host.  The oracle's C calls release the GIL, so experts run on a thread pool.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import precision_moe_gemm_amd as nv
from precision_moe_gemm_amd import synth, workloads
from tests.gpu_util import (BF16_HALF_ULP, BF16_ULP, GEMM_TOL, bf16_to_f64, elem_rel_err, rel_err, step,
                            tensor_bf16_to_f64, u8)

DEV = "cuda"


def workers() -> int:
    # the GPU machine's CPU share is 16 threads
    return max(1, min(16, os.cpu_count() or 1))


def tile_class_rows(offsets, T):
    """Host replay of the grouped tile plan (for choosing rows only): for each
    expert, its full 256-row tiles and the class of its remainder (256-row
    tile for > 128 rows, 128-row tile for 65-128, 16-row streaming tiles for
    <= 64).  Batches of at most 64 tokens put every row in streaming tiles.
    Returns {class: [(expert, first_row, last_row_exclusive)]}."""
    out = {"full256": [], "part256": [], "t128": [], "stream": []}
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        n = hi - lo
        if n == 0:
            continue
        if T <= 64:
            out["stream"].append((e, lo, hi))
            continue
        nf, r = n // 256, n % 256
        for i in range(nf):
            out["full256"].append((e, lo + 256 * i, lo + 256 * i + 256))
        if r:
            c = "part256" if r > 128 else "t128" if r > 64 else "stream"
            out[c].append((e, lo + 256 * nf, hi))
    return out


def stratified_rows(offsets, T, rng, per_class=4, random_rows=24):
    """List positions covering every tile class: the most loaded expert's
    first, middle and last 256-row tiles (first, interior and last rows) and
    its remainder, the first/middle/last row of up to `per_class` tiles of
    each other class (every 128-row tile when there are few), and random rows."""
    cls = tile_class_rows(offsets, T)
    counts = np.diff(offsets)
    heavy = int(np.argmax(counts))
    rows = []
    full = [t for t in cls["full256"] if t[0] == heavy]
    if full:
        for t in (full[0], full[len(full) // 2], full[-1]):
            rows += [t[1], t[1] + 1, t[1] + 127, t[1] + 128, t[2] - 1]
    for name in ("part256", "t128", "stream"):
        tiles = cls[name]
        heavy_t = [t for t in tiles if t[0] == heavy]
        others = [t for t in tiles if t[0] != heavy]
        take = others if (name == "t128" and len(others) <= 24) else \
            [others[i] for i in rng.choice(len(others), min(per_class, len(others)), replace=False)] if others else []
        for t in heavy_t + take:
            n = t[2] - t[1]
            if name == "stream" and n <= 16:
                rows += list(range(t[1], t[2]))
            else:
                rows += [t[1], t[1] + n // 2, t[2] - 1]
    npairs = int(offsets[-1])
    rows += list(rng.choice(npairs, min(random_rows, npairs), replace=False))
    rows = np.unique(np.asarray(rows, np.int64))
    return rows, cls


def class_counts(rows, offsets, T):
    cls = tile_class_rows(offsets, T)
    found = {}
    for name, tiles in cls.items():
        c = 0
        for (_, lo, hi) in tiles:
            c += int(np.count_nonzero((rows >= lo) & (rows < hi)))
        found[name] = (c, len(tiles))
    return found


def run_staged(x, ids, w, W, cfg):
    T, k, E = cfg.T, cfg.k, cfg.E
    xq = nv.nvfp4_quantize(x)
    perm, offsets, inv = nv.nvfp4_moe_route(ids, E)
    h, hmax = nv.nvfp4_moe_gate_up(xq, perm, offsets, k, W.w13)
    hq = nv.nvfp4_quantize(h)
    y = nv.nvfp4_moe_down(hq, offsets, T, k, W.w2)
    out = nv.nvfp4_moe_combine(y, inv, w)
    torch.cuda.synchronize()
    return dict(xq=xq, perm=perm, offsets=offsets, inv=inv, h=h, hmax=hmax, hq=hq, y=y, out=out)


class ExpertOracle:
    """Oracle NVFP4 weights of chosen experts, each checked bit-exact against
    the GPU's copy.  The bf16 sources are drawn on the device (the device
    generator is the one the GPU weights came from) and copied to the host in
    the calling thread; the oracle encodes run on the pool."""

    def __init__(self, cfg, W, pool):
        self.cfg, self.W, self.pool = cfg, W, pool
        self.w13, self.w2 = {}, {}

    def _encode(self, src):
        if self.cfg.mx:
            return oracle.mxfp4_to_nvfp4(*oracle.mxfp4_encode(src))
        return oracle.quantize(src)

    def _job(self, which, e, src, gp, gs, gg):
        ref = self._encode(src)
        np.testing.assert_array_equal(gs, ref.scales, err_msg=f"{which} expert {e} scale bytes")
        np.testing.assert_array_equal(gp, ref.packed, err_msg=f"{which} expert {e} codes")
        assert np.float32(gg) == ref.G, (which, e, gg, ref.G)
        return ref

    def need(self, experts, which=("w13", "w2")):
        futs = []
        for e in sorted(set(int(e) for e in experts)):
            for wh in which:
                store = self.w13 if wh == "w13" else self.w2
                if e in store:
                    continue
                if wh == "w13":
                    src = synth.bits(self.cfg.w13(e, DEV))
                    gt = workloads.expert_view(self.W.w13, e)
                else:
                    src = synth.bits(self.cfg.w2(e, DEV))
                    gt = workloads.expert_view(self.W.w2, e)
                gp, gs, gg = u8(gt.packed)[0], u8(gt.scales)[0], float(gt.global_.item())
                futs.append((store, e, self.pool.submit(self._job, wh, e, src, gp, gs, gg)))
        for store, e, f in futs:
            store[e] = f.result()

    @staticmethod
    def one(t):
        return oracle.Experts(t.packed[None], t.scales[None], np.array([t.G], np.float32))


def _by_expert(rows, offsets):
    ex = np.searchsorted(offsets, rows, side="right") - 1
    return {int(e): rows[ex == e] for e in np.unique(ex)}


def _jobs(groups, chunk=4):
    """(expert, rows) jobs of at most `chunk` rows, so one heavy expert still
    spreads over the pool."""
    return [(e, q[i:i + chunk]) for e, q in groups.items() for i in range(0, q.size, chunk)]


def quantize_rows_parallel(bits2d, G, pool, chunk=1024):
    """Oracle Q of every row with a given global (rows are independent given
    G), in row chunks on the pool; returns (packed, scales)."""
    R = bits2d.shape[0]
    parts = list(pool.map(lambda r0: oracle.quantize(np.ascontiguousarray(bits2d[r0:r0 + chunk]), static_G=G),
                          range(0, R, chunk)))
    return np.concatenate([p.packed for p in parts]), np.concatenate([p.scales for p in parts])


def check_moe_rows(cfg, rows=None, sample_tokens=8, full_tokens=2, seed=0, fused="exact", W=None,
                   full_h_check=True):
    """Run the staged protocol on list positions `rows` (None: every row, or a
    stratified sample when given the string "stratified").  Returns the GPU
    stages and a report dict."""
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    step(f"moe build E={E} k={k} H={H} I={I} T={T} mx={cfg.mx}")
    if W is None:
        W = workloads.build_moe_weights(cfg, DEV)
    x = cfg.x(DEV)
    ids, w = workloads.routing(cfg, DEV)
    step("moe staged run")
    g = run_staged(x, ids, w, W, cfg)
    assert nv.nvfp4_get_error() == 0
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    rng = np.random.default_rng(seed)
    report = {}
    with ThreadPoolExecutor(workers()) as pool:
        # 1. x bit-exact (every row), with the oracle's dynamic global
        xb = synth.bits(x)
        Gx = oracle.global_from_amax(oracle.amax_bf16(xb))
        xp, xs = quantize_rows_parallel(xb, Gx, pool)
        assert np.float32(g["xq"].global_.item()) == np.float32(Gx)
        np.testing.assert_array_equal(u8(g["xq"].scales)[0], xs)
        np.testing.assert_array_equal(u8(g["xq"].packed)[0], xp)
        xo = oracle.NVFP4(xp, xs, Gx)
        # 2. route bit-exact
        perm, offsets, inv = oracle.moe_route(ids_np, E)
        np.testing.assert_array_equal(g["perm"].cpu().numpy(), perm)
        np.testing.assert_array_equal(g["offsets"].cpu().numpy(), offsets)
        np.testing.assert_array_equal(g["inv"].cpu().numpy(), inv)
        npairs = int(offsets[-1])
        if rows is None:
            rows = np.arange(npairs, dtype=np.int64)
        elif isinstance(rows, str):
            rows, _ = stratified_rows(offsets, T, rng)
        rows = np.asarray(rows, np.int64)
        report["rows"] = int(rows.size)
        report["classes"] = class_counts(rows, offsets, T)
        print(f"checked rows {rows.size} of {npairs}; per tile class (rows, tiles): {report['classes']}")
        groups = _by_expert(rows, offsets)
        eo = ExpertOracle(cfg, W, pool)
        step(f"oracle weights of {len(groups)} experts")
        eo.need(groups.keys())
        # 3. h on the chosen rows: one-expert sub-problems
        rows_t = torch.from_numpy(rows).to(DEV)
        h_rows = synth.bits(g["h"].index_select(0, rows_t).cpu())

        def gate_up_job(job):
            e, q = job
            sub_perm = np.ascontiguousarray(perm[q])
            offs = np.array([0, q.size], np.int32)
            return oracle.moe_gate_up(xo, sub_perm, offs, k, ExpertOracle.one(eo.w13[e]),
                                      np.arange(q.size, dtype=np.int64))

        step("oracle gate_up rows")
        h_ref = np.zeros((rows.size, I), np.uint16)
        pos = {int(r): i for i, r in enumerate(rows)}
        jobs = _jobs(groups)
        for (e, q), part in zip(jobs, pool.map(gate_up_job, jobs)):
            h_ref[[pos[int(r)] for r in q]] = part
        got, ref = bf16_to_f64(h_rows), bf16_to_f64(h_ref)
        err_h, eerr_h = rel_err(got, ref), elem_rel_err(got, ref)
        report.update(h_rel=err_h, h_elem_rel=eerr_h)
        print(f"h rel err {err_h:.3e} (element-wise {eerr_h:.3e})")
        assert err_h <= GEMM_TOL + BF16_HALF_ULP
        assert eerr_h <= GEMM_TOL + BF16_ULP
        # 4. G_h and hq bit-exact vs oracle Q(h_gpu)
        h_all = synth.bits(g["h"].cpu())
        # |x| orders as its bf16 bits with the sign cleared (finite values)
        amax_bits = np.uint32(int((h_all & 0x7FFF).max()) << 16)
        amax_h = float(amax_bits.view(np.float32))
        assert np.uint32(g["hmax"].item()) == amax_bits
        Gh = oracle.global_from_amax(amax_h)
        assert np.float32(g["hq"].global_.item()) == np.float32(Gh)
        hq_rows = rows if not full_h_check else np.arange(npairs, dtype=np.int64)
        step(f"oracle quantize of h on {hq_rows.size} rows")
        hp, hs = quantize_rows_parallel(np.ascontiguousarray(h_all[hq_rows]), Gh, pool)
        gp, gs = u8(g["hq"].packed)[0], u8(g["hq"].scales)[0]
        np.testing.assert_array_equal(gs[hq_rows], hs)
        np.testing.assert_array_equal(gp[hq_rows], hp)
        del h_all
        hq_o = oracle.NVFP4(gp, gs, np.float32(g["hq"].global_.item()))

        # 5. y on the chosen rows from the GPU's hq
        def down_job(job):
            e, q = job
            sub = oracle.NVFP4(np.ascontiguousarray(hq_o.packed[q]), np.ascontiguousarray(hq_o.scales[q]), hq_o.G)
            offs = np.array([0, q.size], np.int32)
            return oracle.moe_down(sub, offs, ExpertOracle.one(eo.w2[e]), np.arange(q.size, dtype=np.int64))

        step("oracle down rows")
        y_ref = np.zeros((rows.size, H))
        for (e, q), part in zip(jobs, pool.map(down_job, jobs)):
            y_ref[[pos[int(r)] for r in q]] = part
        y_rows = g["y"].index_select(0, rows_t).cpu().numpy()
        err_y, eerr_y = rel_err(y_rows, y_ref), elem_rel_err(y_rows, y_ref)
        report.update(y_rel=err_y, y_elem_rel=eerr_y)
        print(f"y rel err {err_y:.3e} (element-wise {eerr_y:.3e})")
        assert err_y <= GEMM_TOL
        assert eerr_y <= GEMM_TOL
        # 6a. combine of the GPU's y on sampled tokens (all k slots each)
        toks = np.unique(np.r_[rng.choice(T, min(sample_tokens, T), replace=False), 0, T - 1])
        slot_rows = inv.reshape(T, k)[toks].ravel()
        sr_t = torch.from_numpy(slot_rows.astype(np.int64)).to(DEV)
        y_slots = g["y"].index_select(0, sr_t).cpu().numpy().astype(np.float64)
        inv_sub = np.arange(toks.size * k, dtype=np.int32)
        out_ref = oracle.moe_combine(y_slots, inv_sub, np.ascontiguousarray(w_np[toks]))
        got_o, ref_o = tensor_bf16_to_f64(g["out"])[toks], bf16_to_f64(out_ref)
        err_c = rel_err(got_o, ref_o)
        report["combine_rel"] = err_c
        print(f"combine (GPU y) rel err {err_c:.3e}")
        assert err_c <= GEMM_TOL + BF16_HALF_ULP
        # 6b. oracle down + combine on a few whole tokens
        ft = toks[:full_tokens]
        fr = inv.reshape(T, k)[ft].ravel()
        fgroups = _by_expert(np.asarray(fr, np.int64), offsets)
        eo.need(fgroups.keys(), which=("w2",))
        y_tok = np.zeros((fr.size, H))
        fpos = {int(r): i for i, r in enumerate(fr)}
        fjobs = _jobs(fgroups)
        for (e, q), part in zip(fjobs, pool.map(down_job, fjobs)):
            y_tok[[fpos[int(r)] for r in q]] = part
        out_tok = oracle.moe_combine(y_tok, np.arange(fr.size, dtype=np.int32), np.ascontiguousarray(w_np[ft]))
        err_o = rel_err(tensor_bf16_to_f64(g["out"])[ft], bf16_to_f64(out_tok))
        report["out_rel"] = err_o
        print(f"out rel err {err_o:.3e}")
        assert err_o <= GEMM_TOL + BF16_HALF_ULP
    # 7. fused == staged
    if fused:
        step("moe fused run")
        out = nv.nvfp4_moe_grouped_gemm(x, ids, w, W.w13, W.w2)
        torch.cuda.synchronize()
        if fused == "exact":
            assert torch.equal(out, g["out"])
        else:
            err_f = rel_err(tensor_bf16_to_f64(out), tensor_bf16_to_f64(g["out"]))
            print(f"fused vs staged rel err {err_f:.3e}")
            assert err_f <= GEMM_TOL + BF16_HALF_ULP
        assert nv.nvfp4_get_error() == 0
    return g, W, report
