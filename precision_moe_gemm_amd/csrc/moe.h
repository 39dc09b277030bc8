// moe.h -- routed-expert plumbing around the grouped W4A4 GEMMs (page
// "Qwen3.8-Flash-Next-NVFP4": routed experts with top-k routing and fused
// gate_up / down projections; page "DeepSeek-V4.1-Flash-NVFP4", section 三:
// experts w1, w3, w2).
//
// route: the T*k (token, slot) pairs p = t*k + j are listed expert by expert
// and, inside an expert, in increasing p (a stable counting sort):
//   1. per-chunk histograms (chunks of kRouteChunk pairs),
//   2. per-expert scans turn them into per-chunk bases, then expert offsets,
//   3. per-chunk stable scatter: a pair's rank among equal ids earlier in its
//      chunk, plus its chunk base.
// combine: out[t] = sum_j w[t,j] * y[inv[t*k+j]] in fp32, j ascending, one
// thread per 8 output columns; no atomics, so results are run-to-run
// identical.
#pragma once
#include "common.h"

namespace nvfp4 {

constexpr int kRouteChunk = 256;
constexpr int kMaxExperts = 4096;

// 1. hist[c][e] = pairs of chunk c routed to e.  Out-of-range ids raise the
// sticky range error and are dropped.
__global__ void __launch_bounds__(kRouteChunk)
route_hist_kernel(const int32_t* __restrict__ ids, int64_t npairs, int E, int32_t* __restrict__ hist)
{
    extern __shared__ int32_t cnt[];  // [E]
    for (int i = threadIdx.x; i < E; i += blockDim.x)
        cnt[i] = 0;
    __syncthreads();
    const int64_t p = (int64_t)blockIdx.x * kRouteChunk + threadIdx.x;
    if (p < npairs) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else
            raise_error(NVFP4_ERR_RANGE);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += blockDim.x)
        hist[(int64_t)blockIdx.x * E + i] = cnt[i];
}

// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024, a
// multiple of 64): .x = the exclusive prefix, .y = the block total.
struct ScanResult {
    int32_t prefix, total;
};
NVFP4_DEV ScanResult block_exclusive_scan(int32_t v, int32_t* lds16)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += o;
    }
    __syncthreads();
    if (lane == 63)
        lds16[wid] = incl;
    __syncthreads();
    int32_t base = 0, all = 0;
    const int nw = blockDim.x >> 6;
    for (int w = 0; w < nw; w++) {
        base += w < wid ? lds16[w] : 0;
        all += lds16[w];
    }
    return ScanResult{base + incl - v, all};
}

// 2a. One workgroup per expert e: exclusive scan of hist[.][e] over chunks
// into base[.][e]; tot[e] = pairs routed to e.
__global__ void __launch_bounds__(256)
route_expert_scan_kernel(const int32_t* __restrict__ hist, int64_t nchunks, int E,
                         int32_t* __restrict__ base, int32_t* __restrict__ tot)
{
    __shared__ int32_t lds16[16];
    const int e = blockIdx.x;
    const int64_t per = (nchunks + blockDim.x - 1) / blockDim.x;
    const int64_t c0 = threadIdx.x * per;
    int32_t local = 0;
    for (int64_t c = c0; c < c0 + per && c < nchunks; c++)
        local += hist[c * E + e];
    const ScanResult sr = block_exclusive_scan(local, lds16);
    const int32_t total = sr.total;
    int32_t run = sr.prefix;
    for (int64_t c = c0; c < c0 + per && c < nchunks; c++) {
        const int32_t v = hist[c * E + e];
        base[c * E + e] = run;
        run += v;
    }
    if (threadIdx.x == 0)
        tot[e] = total;
}

// 2b. One workgroup: offsets[e] = exclusive scan of tot, offsets[E] = total;
// also zeroes `zero_word` (the h max word of the fused MoE) when given.
__global__ void __launch_bounds__(1024)
route_offsets_kernel(const int32_t* __restrict__ tot, int E, int32_t* __restrict__ offsets,
                     uint32_t* zero_word)
{
    __shared__ int32_t lds16[16];
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per;
    int32_t local = 0;
    for (int e = e0; e < e0 + per && e < E; e++)
        local += tot[e];
    const ScanResult sr = block_exclusive_scan(local, lds16);
    const int32_t total = sr.total;
    int32_t run = sr.prefix;
    for (int e = e0; e < e0 + per && e < E; e++) {
        offsets[e] = run;
        run += tot[e];
    }
    if (threadIdx.x == 0) {
        offsets[E] = total;
        if (zero_word)
            *zero_word = 0;
    }
}

// 3. Stable scatter of chunk c.
__global__ void __launch_bounds__(kRouteChunk)
route_scatter_kernel(const int32_t* __restrict__ ids, int64_t npairs, int E,
                     const int32_t* __restrict__ base, const int32_t* __restrict__ offsets,
                     int32_t* __restrict__ perm, int32_t* __restrict__ inv)
{
    __shared__ int32_t sid[kRouteChunk];
    const int64_t p = (int64_t)blockIdx.x * kRouteChunk + threadIdx.x;
    const int32_t e = p < npairs ? ids[p] : -1;
    sid[threadIdx.x] = e;
    __syncthreads();
    if (p >= npairs)
        return;
    if (e < 0 || e >= E) {
        inv[p] = -1;
        return;
    }
    int32_t rank = 0;
    for (int i = 0; i < (int)threadIdx.x; i++)
        rank += sid[i] == e;
    const int32_t q = offsets[e] + base[(int64_t)blockIdx.x * E + e] + rank;
    perm[q] = (int32_t)p;
    inv[p] = q;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

// m-tile prefix for a grouped GEMM with BM-row tiles:
// tile_off[e] = sum_{e' < e} ceil(count_e' / BM).  One workgroup.
__global__ void __launch_bounds__(1024)
tile_offsets_kernel(const int32_t* __restrict__ offsets, int E, int bm, int32_t* __restrict__ tile_off)
{
    __shared__ int32_t lds16[16];
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per;
    int32_t local = 0;
    for (int e = e0; e < e0 + per && e < E; e++)
        local += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
    const ScanResult sr = block_exclusive_scan(local, lds16);
    const int32_t total = sr.total;
    int32_t run = sr.prefix;
    for (int e = e0; e < e0 + per && e < E; e++) {
        tile_off[e] = run;
        run += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
    }
    if (threadIdx.x == 0)
        tile_off[E] = total;
}

// Tile plan of a grouped projection.  Each expert's rows are cut into full
// 256-row tiles plus one remainder of r = rows % 256 rows, and the remainder
// goes to the smallest tile class that holds it, so that little MFMA work is
// spent on padding rows when the tokens per expert are skewed:
//   class 0: 256-row tiles (the full tiles, and remainders r > 128)
//   class 1: 128-row tiles (64 < r <= 128)
//   class 2: `small_bm`-row tiles (r <= 64; small_bm is 16, 32 or 64)
// With `all_small`, every expert's rows go to class 2 instead.
// For class c, plan + 3 c (E + 1) holds tile_off[E + 1] (exclusive prefix of
// the class's tiles per expert), then row_base[E + 1] and row_lim[E + 1]:
// tile i of expert e covers rows [row_base[e] + i bm, min(+bm, row_lim[e])).
constexpr int kPlanClasses = 3;
constexpr int kPlanSmall = 2;  // the small-tile class

// Class C's share of expert rows [lo, hi): its tile count, row base and row
// limit (scalars, so the callers' unrolled class loops stay in registers).
struct ClassPlan {
    int32_t tiles, base, lim;
};
template <int C>
NVFP4_DEV ClassPlan plan_class(int32_t lo, int32_t hi, int small_bm, int all_small)
{
    if (all_small) {
        // every row in small tiles (K-split streaming projections)
        if (C == kPlanSmall)
            return ClassPlan{(hi - lo + small_bm - 1) / small_bm, lo, hi};
        return ClassPlan{0, lo, lo};
    }
    const int32_t rows = hi - lo, nf = rows >> 8, r = rows & 255;
    const int32_t tail = lo + (nf << 8);
    const int c = r > 128 ? 0 : r > 64 ? 1 : kPlanSmall;
    if (C == 0)
        return ClassPlan{nf + (c == 0 && r > 0 ? 1 : 0), lo, c == 0 ? hi : tail};
    if (C == kPlanSmall)
        return ClassPlan{c == kPlanSmall ? (r + small_bm - 1) / small_bm : 0, tail, c == kPlanSmall ? hi : tail};
    return ClassPlan{c == C ? 1 : 0, tail, c == C ? hi : tail};
}

// The plan of all experts by one workgroup of 1024 threads; offs[e] and
// offs[e + 1] bound expert e's rows (offs may be in LDS).
NVFP4_DEV void plan_block(const int32_t* offs, int E, int small_bm, int all_small, int32_t* plan,
                          int32_t* lds16)
{
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = threadIdx.x * per;
    int32_t cnt0 = 0, cnt1 = 0, cnt2 = 0;
    for (int e = e0; e < e0 + per && e < E; e++) {
        const int32_t lo = offs[e], hi = offs[e + 1];
        cnt0 += plan_class<0>(lo, hi, small_bm, all_small).tiles;
        cnt1 += plan_class<1>(lo, hi, small_bm, all_small).tiles;
        cnt2 += plan_class<2>(lo, hi, small_bm, all_small).tiles;
    }
    // when every row takes small tiles the other classes are empty: their
    // counts are zero in every thread, so their scans are skipped
    const ScanResult zero{0, 0};
    const ScanResult s0 = all_small ? zero : block_exclusive_scan(cnt0, lds16);
    const ScanResult s1 = all_small ? zero : block_exclusive_scan(cnt1, lds16);
    const ScanResult s2 = block_exclusive_scan(cnt2, lds16);
    int32_t run0 = s0.prefix, run1 = s1.prefix, run2 = s2.prefix;
    auto put = [&](int c, int e, const ClassPlan& cp, int32_t& run) {
        int32_t* pc = plan + 3 * c * (E + 1);
        pc[e] = run;
        pc[(E + 1) + e] = cp.base;
        pc[2 * (E + 1) + e] = cp.lim;
        run += cp.tiles;
    };
    for (int e = e0; e < e0 + per && e < E; e++) {
        const int32_t lo = offs[e], hi = offs[e + 1];
        put(0, e, plan_class<0>(lo, hi, small_bm, all_small), run0);
        put(1, e, plan_class<1>(lo, hi, small_bm, all_small), run1);
        put(2, e, plan_class<2>(lo, hi, small_bm, all_small), run2);
    }
    if (threadIdx.x == 0) {
        plan[E] = s0.total;
        plan[3 * (E + 1) + E] = s1.total;
        plan[6 * (E + 1) + E] = s2.total;
    }
}

__global__ void __launch_bounds__(1024)
moe_plan_kernel(const int32_t* __restrict__ offsets, int E, int small_bm, int all_small,
                int32_t* __restrict__ plan)
{
    __shared__ int32_t lds16[16];
    plan_block(offsets, E, small_bm, all_small, plan, lds16);
}

// Routing of a small batch (at most kRouteSmall pairs) in one workgroup, with
// the result of the chunked route above: counts in LDS, one scan, and each
// pair's rank among the earlier pairs with the same id.  Optionally also
// writes the tile plans of the two grouped projections (plan_gu, plan_dn)
// and zeroes `zero_word`, so a small layer needs one launch for all of it.
constexpr int kRouteSmall = 1024;

NVFP4_DEV void route_small_block(const int32_t* __restrict__ ids, int npairs, int E, int32_t* __restrict__ offsets,
                                 int32_t* __restrict__ perm, int32_t* __restrict__ inv, uint32_t* zero_word,
                                 int32_t* plan_gu, int small_bm_gu, int all_small_gu, int32_t* plan_dn,
                                 int small_bm_dn, int all_small_dn)
{
    __shared__ __attribute__((aligned(16))) int32_t sid[kRouteSmall];
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t lds16[16];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x)
        off[e] = 0;
    int32_t my = -1;
    if (tid < npairs) {
        my = ids[tid];
        if (my < 0 || my >= E) {
            raise_error(NVFP4_ERR_RANGE);
            my = -1;
        }
    }
    sid[tid] = my;
    __syncthreads();
    if (my >= 0)
        atomicAdd(&off[my], 1);
    __syncthreads();
    // counts -> exclusive offsets, in place
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int e0 = tid * per;
    int32_t local = 0;
    for (int e = e0; e < e0 + per && e < E; e++)
        local += off[e];
    const ScanResult sr = block_exclusive_scan(local, lds16);
    const int32_t total = sr.total;
    int32_t run = sr.prefix;
    for (int e = e0; e < e0 + per && e < E; e++) {
        const int32_t c = off[e];
        off[e] = run;
        offsets[e] = run;
        run += c;
    }
    if (tid == 0) {
        off[E] = total;
        offsets[E] = total;
        if (zero_word)
            *zero_word = 0;
    }
    __syncthreads();
    if (tid < npairs) {
        if (my < 0) {
            inv[tid] = -1;
        } else {
            // earlier pairs with the same id: 16 ids per step, four
            // 16-byte LDS reads in flight
            int32_t rank = 0;
            const int4* s4 = (const int4*)sid;
            const int full = tid >> 4;
            for (int q = 0; q < full; q++) {
                int4 v[4];
#pragma unroll
                for (int u = 0; u < 4; u++)
                    v[u] = s4[4 * q + u];
#pragma unroll
                for (int u = 0; u < 4; u++)
                    rank += (v[u].x == my) + (v[u].y == my) + (v[u].z == my) + (v[u].w == my);
            }
            for (int i = full << 4; i < tid; i++)
                rank += sid[i] == my;
            const int32_t q = off[my] + rank;
            perm[q] = tid;
            inv[tid] = q;
        }
    }
    if (plan_gu)
        plan_block(off, E, small_bm_gu, all_small_gu, plan_gu, lds16);
    if (plan_dn)
        plan_block(off, E, small_bm_dn, all_small_dn, plan_dn, lds16);
}

__global__ void __launch_bounds__(1024)
route_small_kernel(const int32_t* __restrict__ ids, int npairs, int E, int32_t* __restrict__ offsets,
                   int32_t* __restrict__ perm, int32_t* __restrict__ inv, uint32_t* zero_word,
                   int32_t* plan_gu, int small_bm_gu, int all_small_gu, int32_t* plan_dn, int small_bm_dn,
                   int all_small_dn)
{
    route_small_block(ids, npairs, E, offsets, perm, inv, zero_word, plan_gu, small_bm_gu, all_small_gu, plan_dn,
                      small_bm_dn, all_small_dn);
}

// Sum over the `planes` partial planes (`plane` floats apart) of the four
// floats at p, added in plane order; the loads of four planes are in flight
// together.  y is read exactly once: nontemporal loads (the 384-expert
// prefill's combine of 3.76 GB: 783 -> 702 us).
NVFP4_DEV float4_t sum_planes(const float* p, int planes, int64_t plane)
{
    float4_t v = __builtin_nontemporal_load((const float4_t*)p);
    for (int sp = 1; sp < planes; sp += 4) {
        float4_t x[4];
#pragma unroll
        for (int u = 0; u < 4; u++)
            x[u] = sp + u < planes ? __builtin_nontemporal_load((const float4_t*)(p + (sp + u) * plane))
                                   : (float4_t){0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; u++)
            if (sp + u < planes)
                v += x[u];
    }
    return v;
}

// out[t, 4c..4c+4) = bf16(sum_j w[t,j] * y[inv[t*k+j], 4c..4c+4)), j in
// ascending order, where y is the sum (in plane order) of `planes` partial
// planes `plane` floats apart.  A workgroup takes one token at a time (its
// slot rows and weights read once, with scalar loads) and one slice of the
// columns (blockIdx.y of col_split; several slices when the tokens alone
// cannot fill the chip); each thread takes 4 columns per step and issues
// the loads of all k slot rows together.
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ inv,
               const float* __restrict__ w, int64_t T, int k, int64_t H, int planes, int64_t plane,
               int col_split, u32x2* __restrict__ out)
{
    const int64_t groups = H / 4;
    const int64_t per = (groups + col_split - 1) / col_split;
    const int64_t g0 = (int64_t)blockIdx.y * per;
    const int64_t g1 = g0 + per < groups ? g0 + per : groups;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        for (int64_t g = g0 + threadIdx.x; g < g1; g += blockDim.x) {
            float4_t acc = {0, 0, 0, 0};
            for (int j0 = 0; j0 < k; j0 += 8) {
                int32_t q[8];
                float wt[8];
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const bool in = j0 + u < k;
                    q[u] = in ? const_load(inv, t * k + j0 + u) : -1;
                    wt[u] = in ? const_load(w, t * k + j0 + u) : 0.0f;
                }
                float4_t v[8];
#pragma unroll
                for (int u = 0; u < 8; u++)
                    v[u] = q[u] >= 0 ? sum_planes(y + (int64_t)q[u] * H + 4 * g, planes, plane)
                                     : (float4_t){0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    if (q[u] >= 0) {
                        acc.x += wt[u] * v[u].x;
                        acc.y += wt[u] * v[u].y;
                        acc.z += wt[u] * v[u].z;
                        acc.w += wt[u] * v[u].w;
                    }
                }
            }
            out[t * groups + g] = (u32x2){pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
        }
    }
}

}  // namespace nvfp4
