// libnvfp4.hip -- the C ABI of include/nvfp4.h: argument validation,
// workspace layout and kernel dispatch.  One translation unit so that every
// kernel shares the per-device sticky error word.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "common.h"
#include "gemm.h"
#include "moe.h"
#include "mx.h"
#include "mx8.h"
#include "quant.h"

#ifndef NVFP4_BUILD_STAMP
#define NVFP4_BUILD_STAMP "unstamped"
#endif

using namespace nvfp4;

namespace {

inline hipStream_t S(void* s) { return (hipStream_t)s; }

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline nvfp4_status launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_DEVICE;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// number of 256-thread blocks for a grid-stride kernel that wants `work` threads (capped)
// grid for a grid-stride streaming kernel over `work` items of 256 threads
inline unsigned stream_grid(int64_t work, int64_t cap = 8192)
{
    int64_t g = ceil_div(work, 256);
    if (g < 1)
        g = 1;
    return (unsigned)std::min<int64_t>(g, cap);
}

// Router-weighted combine of `planes` planes of y into bf16 out [T, H]: one
// workgroup per token and column slice; small batches split the columns so
// that about 2048 workgroups run.
void launch_combine(const float* y, const int32_t* inv, const float* w, int64_t T, int k, int64_t H, int planes,
                    int64_t plane, void* out, hipStream_t st)
{
    const int64_t groups = H / 4;
    if (T <= 0 || groups <= 0)
        return;
    int64_t split = std::max<int64_t>(1, std::min<int64_t>(ceil_div(2048, T), ceil_div(groups, 64)));
    const unsigned gx = (unsigned)std::min<int64_t>(T, 65535);
    combine_kernel<<<dim3(gx, (unsigned)split), 256, 0, st>>>(y, inv, w, T, k, H, planes, plane, (int)split,
                                                              (u32x2*)out);
}

// An empty tensor (rows or cols 0) may carry null code/scale pointers.
// Tensor argument checks.  Scale bytes in the 128-row tiled order
// (NVFP4_TILED_SCALES) are taken only where `tiled_ok` (GEMM weight
// operands), and only with whole 128-row, 256-column tiles.
nvfp4_status check_tensor(const nvfp4_tensor* t, bool need_global = true, bool tiled_ok = false)
{
    if (!t || (need_global && !t->global))
        return NVFP4_ERR_INVALID_ARG;
    const bool empty = t->rows == 0 || t->cols == 0;
    if (!empty && (!t->packed || !t->scales))
        return NVFP4_ERR_INVALID_ARG;
    if (t->rows < 0 || t->cols < 0 || t->batch < 1 || t->cols % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!aligned(t->packed, 16) || !aligned(t->scales, 4) || (t->global && !aligned(t->global, 4)))
        return NVFP4_ERR_INVALID_ARG;
    if (t->flags & NVFP4_TILED_SCALES) {
        if (!tiled_ok)
            return NVFP4_ERR_UNSUPPORTED;
        if (t->rows % 128 != 0 || t->cols % 256 != 0)
            return NVFP4_ERR_SHAPE;
        if (!aligned(t->scales, 16))
            return NVFP4_ERR_INVALID_ARG;
    }
    return NVFP4_OK;
}

// ---------------------------------------------------------------- checks
// The data-check switch (nvfp4_set_checks): its start value comes from the
// NVFP4_CHECK environment variable when the library is loaded, else from the
// NVFP4_CHECK build flag.
#ifndef NVFP4_CHECK
#define NVFP4_CHECK 0
#endif
int checks_initial()
{
    const char* e = getenv("NVFP4_CHECK");
    if (e && *e)
        return atoi(e) != 0;
    return NVFP4_CHECK != 0;
}
std::atomic<int> g_checks{checks_initial()};
bool checks_on() { return g_checks.load(std::memory_order_relaxed) != 0; }

void check_bf16(const void* x, int64_t rows, int64_t cols, int64_t ld, hipStream_t st)
{
    if (rows > 0 && cols > 0)
        check_bf16_kernel<<<stream_grid(rows * cols, 2048), kQuantThreads, 0, st>>>((const uint16_t*)x, rows, cols,
                                                                                     ld);
}

void check_globals(const float* g, int64_t n, hipStream_t st)
{
    if (g && n > 0)
        check_globals_kernel<<<1, 64, 0, st>>>(g, n);
}

// scale bytes and globals of validated tensors (null entries skipped)
nvfp4_status check_tensors_data(std::initializer_list<const nvfp4_tensor*> ts, hipStream_t st)
{
    for (const nvfp4_tensor* t : ts) {
        if (!t)
            continue;
        const int64_t n = t->batch * t->rows * (t->cols / 16);
        if (n > 0)
            check_scales_kernel<<<stream_grid(n, 2048), kQuantThreads, 0, st>>>(t->scales, n);
        check_globals(t->global, t->batch, st);
    }
    return launch_status();
}

nvfp4_status check_tensor_data(const nvfp4_tensor* t, hipStream_t st) { return check_tensors_data({t}, st); }

// ---------------------------------------------------------------- quantize
// Launch the block quantizer for up to two tensors sharing a shape.
nvfp4_status launch_quantize(QuantArgs a, int ntensors, hipStream_t st)
{
    const int64_t nblk = a.rows * a.blocks_per_row;
    if (nblk == 0)
        return NVFP4_OK;
    // 8 half-blocks per thread per trip; 2 when that leaves under 4
    // workgroups per CU (a KV-cache chunk)
    const int64_t wg8 = ceil_div(2 * nblk, 8 * kQuantThreads) * ntensors;
    if (wg8 < 1024) {
        dim3 grid(stream_grid(ceil_div(2 * nblk, 2), 4096), ntensors);
        quantize_kernel<2><<<grid, kQuantThreads, 0, st>>>(a);
    } else {
        dim3 grid(stream_grid(ceil_div(2 * nblk, 8), 4096), ntensors);
        quantize_kernel<8><<<grid, kQuantThreads, 0, st>>>(a);
    }
    return launch_status();
}

// With src == kGlobalPartials and pre_parts > 0, the partial maxima were
// already written (pre_parts of them, by route_small_amax_kernel).
nvfp4_status quantize_impl(const void* x, int64_t rows, int64_t cols, int64_t ld, int src,
                           const void* gsrc, const nvfp4_tensor* out, int64_t row_off,
                           uint32_t* partials, hipStream_t st, int pre_parts = 0)
{
    QuantArgs a{};
    a.x[0] = (const u32x4*)x;
    a.packed[0] = (u32x2*)out->packed;
    a.scales[0] = out->scales;
    a.global_out[0] = out->global;
    a.row_off[0] = row_off;
    a.rows = rows;
    a.blocks_per_row = cols / 16;
    a.ld_chunks = ld / 8;
    a.nparts = 0;
    if (src == kGlobalPartials && pre_parts > 0) {
        a.gsrc[0] = partials;
        a.nparts = pre_parts;
    } else if (src == kGlobalPartials) {
        const int64_t chunks = rows * (cols / 8);
        const unsigned parts = stream_grid(chunks, kAmaxParts);
        amax_partials_kernel<<<parts, kQuantThreads, 0, st>>>((const u32x4*)x, rows, cols / 8, ld / 8, partials);
        nvfp4_status s = launch_status();
        if (s != NVFP4_OK)
            return s;
        a.gsrc[0] = partials;
        a.nparts = (int)parts;
    } else {
        a.gsrc[0] = gsrc;
    }
    a.src[0] = src;
    if (rows == 0) {
        // still publish G (1 for an empty dynamic tensor, or the static value)
        a.rows = 1;
        a.blocks_per_row = 0;
        quantize_kernel<8><<<dim3(1, 1), kQuantThreads, 0, st>>>(a);
        return launch_status();
    }
    return launch_quantize(a, 1, st);
}

// ---------------------------------------------------------------- GEMM
template <int BM, int BN, int WM, int WN, int MODE, bool RAG = false>
nvfp4_status launch_gemm(GemmArgs p, int64_t m_tiles_ub, hipStream_t st)
{
    p.m_tiles = m_tiles_ub;
    int64_t blocks = m_tiles_ub * p.n_tiles;
    if (blocks == 0)
        return NVFP4_OK;
    blocks = ceil_div(blocks, 8) * 8;
    if (blocks > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    gemm_kernel<BM, BN, WM, WN, MODE, RAG><<<(unsigned)blocks, WM * WN * 64, 0, st>>>(p);
    return launch_status();
}

template <int BM, int BN, int MODE>
nvfp4_status launch_tile(GemmArgs p, int64_t m_tiles_ub, hipStream_t st)
{
    if (p.w_tiled && p.K % 256 != 0)
        return NVFP4_ERR_UNSUPPORTED;  // (tiled scales come with K % 256 == 0)
    p.m_tiles = m_tiles_ub;
    int64_t blocks = m_tiles_ub * p.n_tiles;
    if (blocks == 0)
        return NVFP4_OK;
    blocks = ceil_div(blocks, 8) * 8;
    if (blocks > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    if (p.K >= 256 && p.K % 256 == 0) {
        if (p.w_pow2)
            gemm_rtile_kernel<BM, BN, MODE, true><<<(unsigned)blocks, 256, 0, st>>>(p);
        else
            gemm_rtile_kernel<BM, BN, MODE, false><<<(unsigned)blocks, 256, 0, st>>>(p);
    } else if (p.w_pow2) {
        gemm_tile_kernel<BM, BN, MODE, true><<<(unsigned)blocks, 256, 0, st>>>(p);
    } else {
        gemm_tile_kernel<BM, BN, MODE, false><<<(unsigned)blocks, 256, 0, st>>>(p);
    }
    return launch_status();
}

// The register-decode tile kernel alone, general weight scales (K a
// multiple of 256).
template <int BM, int BN, int MODE>
nvfp4_status launch_rtile_general(GemmArgs p, int64_t m_tiles_ub, hipStream_t st)
{
    p.m_tiles = m_tiles_ub;
    int64_t blocks = m_tiles_ub * p.n_tiles;
    if (blocks == 0)
        return NVFP4_OK;
    blocks = ceil_div(blocks, 8) * 8;
    if (blocks > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    gemm_rtile_kernel<BM, BN, MODE, false><<<(unsigned)blocks, 256, 0, st>>>(p);
    return launch_status();
}

// The weight-streaming kernel serves A operands of at most 32 rows per
// expert (on average; tiles of 16 or 32 rows) when K is a multiple of its
// 256-element stage.
bool use_stream_gemm(int64_t rows_avg, int64_t K) { return rows_avg <= 2 * kSkBM && K > 0 && K % kSkBK == 0; }

// Rows of a dense weight-streaming tile: 32 when A has more than 16 rows
// (each W tile is then read once for all of them), else 16.
int stream_bm(int64_t rows) { return rows > kSkBM ? 2 * kSkBM : kSkBM; }
// Workgroups the chip holds at once of the bm-row streaming kernel
// (3 per CU with 16-row tiles, 2 with 32-row tiles, 256 CUs).
int64_t stream_slots(int bm) { return bm == kSkBM ? 768 : 512; }

// K split of the dense weight-streaming GEMM: at most one workgroup per
// resident slot, at least four stages per split, partials <= 32 MiB.
// K split of `tiles` streaming work items over `slots` resident workgroups,
// at most smax ways: the split that minimises the finishing time, counted
// as rounds of items (ceil(tiles * s / slots)) times the item length (1 / s),
// the smaller split on a tie.  A persistent grid finishes when its busiest
// workgroup does, so 272 tiles on 512 slots take one full item unsplit, two
// half items split in two, but two thirds of an item split in three.
int64_t balanced_split(int64_t tiles, int64_t slots, int64_t smax)
{
    if (tiles <= 0 || tiles >= slots * 2 / 3 || smax <= 1)
        return 1;
    int64_t best = 1;
    double best_t = (double)ceil_div(tiles, slots);
    for (int64_t s = 2; s <= smax; s++) {
        const double t = (double)ceil_div(tiles * s, slots) / (double)s;
        if (t < best_t - 1e-9) {
            best = s;
            best_t = t;
        }
    }
    return best;
}

int gemm_ksplit(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || !use_stream_gemm(M, K))
        return 1;
    const int64_t base = ceil_div(M, stream_bm(M)) * ceil_div(N, kSkBN);
    int64_t smax = std::min<int64_t>(K / kSkBK / 4, ((int64_t)32 << 20) / (M * N * 4));
    smax = std::min<int64_t>(smax, stream_slots(stream_bm(M)));
    return (int)balanced_split(base, stream_slots(stream_bm(M)), smax);
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K)
{
    const int s = gemm_ksplit(M, N, K);
    return s > 1 ? align256((size_t)s * M * N * sizeof(float)) : 0;
}

// Workgroups of a weight-streaming kernel that the current device holds at
// once, rounded down to a multiple of 8 (one query per kernel and device).
// The per-device cache is atomic (relaxed): threads that race on a first
// call each compute the same value and store it.
template <int MODE, bool P2, bool A16, int BM>
int64_t stream_resident()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        dev = 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm_stream_kernel<MODE, P2, A16, BM>, kSkThreads, 0) !=
                hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 8;
        v = std::max(8, per_cu * cus / 8 * 8);
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int MODE, bool P2, bool A16, int BM>
void launch_stream_kernel(const GemmArgs& p, int64_t items, hipStream_t st)
{
    // a resident grid (multiple of 8) that walks the items
    const int64_t blocks = std::min(ceil_div(items, 8) * 8, stream_resident<MODE, P2, A16, BM>());
    gemm_stream_kernel<MODE, P2, A16, BM><<<(unsigned)blocks, kSkThreads, 0, st>>>(p);
}

template <int MODE, int BM>
void launch_stream_variant(const GemmArgs& p, int64_t items, hipStream_t st)
{
    if (p.a_bf16 && p.w_pow2)
        launch_stream_kernel<MODE, true, true, BM>(p, items, st);
    else if (p.a_bf16)
        launch_stream_kernel<MODE, false, true, BM>(p, items, st);
    else if (p.w_pow2)
        launch_stream_kernel<MODE, true, false, BM>(p, items, st);
    else
        launch_stream_kernel<MODE, false, false, BM>(p, items, st);
}

// Weight-streaming GEMM over m_tiles_ub (an upper bound when grouped) A tiles
// of bm (16 or 32) rows.
template <int MODE>
nvfp4_status launch_stream_gemm(GemmArgs p, int64_t m_tiles_ub, int bm, hipStream_t st)
{
    p.m_tiles = m_tiles_ub;
    const int64_t items = m_tiles_ub * p.n_tiles * p.ksplit;
    if (items == 0)
        return NVFP4_OK;
    // every K split holds at least one stage; item indices fit 31 bits
    if (items > 0x7FFFFFFF || p.ksplit < 1 || p.ksplit > p.K / kSkBK)
        return NVFP4_ERR_SHAPE;
    if (bm == 2 * kSkBM)
        launch_stream_variant<MODE, 2 * kSkBM>(p, items, st);
    else if (bm == kSkBM)
        launch_stream_variant<MODE, kSkBM>(p, items, st);
    else
        return NVFP4_ERR_SHAPE;
    nvfp4_status s = launch_status();
    if (s != NVFP4_OK || p.ksplit <= 1 || MODE == kModeDown)
        return s;  // grouped down: the combine adds the planes
    if (MODE == kModeGateUp) {
        // (at most 256 workgroups: each adds one same-address atomic)
        const int64_t cnt = p.M * p.N;
        const unsigned rb = (unsigned)std::max<int64_t>(1, std::min<int64_t>(256, ceil_div(cnt, 256)));
        swiglu_reduce_kernel<<<rb, 256, 0, st>>>(p.partial, p.ksplit, p.M, p.N, (uint16_t*)p.out, p.h_amax,
                                                 p.hq_global, p.hq_packed, p.hq_scales);
        return launch_status();
    }
    const int64_t count = p.M * p.N;
    const unsigned rb = (unsigned)std::min<int64_t>(2048, ceil_div(count, 256));
    splitk_reduce_kernel<<<rb, 256, 0, st>>>(p.partial, p.ksplit, count, p.out, p.out_bf16);
    return launch_status();
}

// Dense GEMM tile configurations (BM, BN, waves), chosen by the rows of A.
nvfp4_status dispatch_dense(GemmArgs p, hipStream_t st)
{
    if (p.ksplit < 1)
        p.ksplit = 1;
    if (p.a_bf16 || use_stream_gemm(p.M, p.K)) {
        // (W4A16 runs the weight-streaming kernel at every M)
        p.n_tiles = ceil_div(p.N, kSkBN);
        const int bm = stream_bm(p.M);
        return launch_stream_gemm<kModeDense>(p, ceil_div(p.M, bm), bm, st);
    }
    p.ksplit = 1;
    p.n_tiles = ceil_div(p.N, 256);
    if (p.K % kBK != 0) {
        // K a multiple of 16 only: the register-decode kernel with ragged loads
        if (p.M > 32)
            return launch_gemm<64, 256, 1, 4, kModeDense, true>(p, ceil_div(p.M, 64), st);
        return launch_gemm<32, 256, 1, 4, kModeDense, true>(p, ceil_div(p.M, 32), st);
    }
    if (p.M >= 256)
        return launch_tile<256, 256, kModeDense>(p, ceil_div(p.M, 256), st);
    if (p.M >= 96)
        return launch_tile<128, 256, kModeDense>(p, ceil_div(p.M, 128), st);
    if (p.M > 32)
        return launch_gemm<64, 256, 1, 4, kModeDense>(p, ceil_div(p.M, 64), st);
    return launch_gemm<32, 256, 1, 4, kModeDense>(p, ceil_div(p.M, 32), st);
}

// A grouped projection whose K is not a multiple of the 64-element stage, or
// a gate_up projection whose N (= I) is not a multiple of its 128-column
// tile, runs every row in 32-row tiles of the register-decode kernel (ragged
// K loads, columns past N masked).
bool grouped_ragged(int mode, int64_t K, int64_t N)
{
    return K % kBK != 0 || (mode == kModeGateUp && N % 128 != 0);
}

// Rows of the small tiles of a grouped projection with reduction length K
// over `rows` (token, slot) pairs and E experts: 32-row tiles of the
// register-decode kernel when K is not a multiple of the streaming stage;
// else streaming tiles of 32 rows when every row takes them and the experts
// average at least 32 rows (a dense MLP run as one expert: each W tile is
// then read once), and of 16 rows otherwise.  (Measured: 32-row streaming
// tiles run slower for the remainders next to the 128- and 256-row tiles and
// for skewed decode batches, where most experts hold a few rows.)
int grouped_small_bm(int64_t K, int all_small, int64_t rows, int32_t experts, bool ragged = false)
{
    if (ragged || K % kSkBK != 0)
        return 32;
    return (all_small && rows >= 2 * kSkBM * (int64_t)experts) ? 2 * kSkBM : kSkBM;
}

// K split of the grouped down projection of a tiny batch (a dense MLP run as
// a one-expert layer, or a handful of tokens over few experts): every tile is
// a weight-streaming tile and split s writes its scaled partial sums to plane
// s of y, which the combine adds in split order.
// Upper bound of the bm-row tiles the np pairs of a small batch fill: np/bm
// full tiles plus at most one partial tile per other non-empty expert.
int64_t small_tiles_est(int64_t np, int32_t E, int bm) { return std::min<int64_t>(np, ceil_div(np, bm) + E - 1); }

int moe_down_ksplit(int64_t T, int32_t k, int32_t E, int64_t H, int64_t I)
{
    const int64_t np = T * k;
    if (np <= 0 || np > 256 || I % kSkBK != 0)
        return 1;
    const int bm = grouped_small_bm(I, 1, np, E);
    const int64_t tiles = small_tiles_est(np, E, bm) * ceil_div(H, kSkBN);
    int64_t smax = std::min<int64_t>(I / kSkBK / 4, ((int64_t)64 << 20) / (np * H * 4));
    smax = std::min<int64_t>(smax, stream_slots(bm));
    return (int)balanced_split(tiles, stream_slots(bm), smax);
}

// K split of the fused gate_up projection of a tiny batch (as the down
// projection): when the streaming tiles cannot fill the chip, split s writes
// scaled partial gate and up sums to plane s and swiglu_reduce_kernel adds
// the planes in order before the SwiGLU.  One wave of workgroups at most
// (3 per CU), at least four 256-element stages per split.
int moe_gate_ksplit(int64_t T, int32_t k, int32_t E, int64_t H, int64_t I)
{
    const int64_t np = T * k;
    if (np <= 0 || np > 256 || H % kSkBK != 0 || grouped_ragged(kModeGateUp, H, I))
        return 1;
    const int bm = grouped_small_bm(H, 1, np, E);
    const int64_t tiles = small_tiles_est(np, E, bm) * ceil_div(I, kSkBN / 2);
    // the partial gate and up planes stay within 16 MB
    int64_t smax = std::min<int64_t>(H / kSkBK / 4, ((int64_t)16 << 20) / (np * 2 * I * 4));
    smax = std::min<int64_t>(smax, stream_slots(bm));
    return (int)balanced_split(tiles, stream_slots(bm), smax);
}

// Grouped projections: plan the tiles of every class on the device, then
// launch each class (largest tiles first).  With p.ksplit > 1 (down only)
// every tile is a 16-row streaming tile.

// All rows of a grouped projection take 16-row weight-streaming tiles when
// the down projection is K-split, or when the batch has at most 64 tokens:
// top-k routing sends a token to an expert at most once, so no expert can
// fill a 128- or 256-row tile and those launches would be empty.  (Any ids
// still come out right: small tiles cover every row of every expert.)
int grouped_all_small(int64_t T, int64_t K, int ksplit, bool ragged = false)
{
    if (ragged)
        return 1;
    if (K % kSkBK != 0)
        return 0;
    return (ksplit > 1 || T <= 64) ? 1 : 0;
}

template <int MODE>
nvfp4_status dispatch_grouped(GemmArgs p, const int32_t* offsets, int64_t total_rows, int experts,
                              int all_small, int32_t* plan, bool plan_ready, hipStream_t st)
{
    const bool ragged = grouped_ragged(MODE, p.K, p.N);
    const bool stream_ok = !ragged && p.K % kSkBK == 0;
    if (p.a_bf16 && !stream_ok)
        return NVFP4_ERR_UNSUPPORTED;
    if (p.ksplit < 1 || !stream_ok)
        p.ksplit = 1;
    if (p.ksplit > 1 || p.a_bf16 || ragged)
        all_small = 1;  // the split planes cover every row; W4A16 streams every tile
    const int small_bm = grouped_small_bm(p.K, all_small, total_rows, experts, ragged);
    nvfp4_status s = NVFP4_OK;
    if (!plan_ready) {
        moe_plan_kernel<<<1, 1024, 0, st>>>(offsets, experts, small_bm, all_small, plan);
        s = launch_status();
        if (s != NVFP4_OK)
            return s;
    }
    const int64_t E1 = experts + 1;
    auto cls = [&](int c) {
        GemmArgs q = p;
        q.tile_off = plan + 3 * c * E1;
        q.row_base = q.tile_off + E1;
        q.row_lim = q.tile_off + 2 * E1;
        return q;
    };
    const int64_t big_cols = MODE == kModeGateUp ? 128 : 256;
    // class 0 needs an expert with more than 128 rows, class 1 one with more
    // than 64: skip launches that cannot have work
    if (!all_small && total_rows > 128) {
        GemmArgs q = cls(0);
        q.ksplit = 1;
        q.n_tiles = ceil_div(p.N, big_cols);
        s = launch_tile<256, 256, MODE>(q, total_rows / 128 + 1, st);
        if (s != NVFP4_OK)
            return s;
    }
    if (!all_small && total_rows > 64) {
        GemmArgs q = cls(1);
        q.ksplit = 1;
        const int64_t m1 = std::min<int64_t>(experts, total_rows / 65 + 1);
        if (!p.w_pow2 && p.K % 256 == 0) {
            // general weight scales: the decode of both operands keeps the
            // VALU as busy as the MFMA, and 128-column tiles (72 KB of LDS,
            // 188 registers) run two workgroups per CU, so one wave's decode
            // issues while the other's MFMA runs
            q.n_tiles = ceil_div(p.N, big_cols / 2);
            s = launch_rtile_general<128, 128, MODE>(q, m1, st);
        } else {
            q.n_tiles = ceil_div(p.N, big_cols);
            s = launch_tile<128, 256, MODE>(q, m1, st);
        }
        if (s != NVFP4_OK)
            return s;
    }
    GemmArgs q = cls(kPlanSmall);
    // small class: every tile holds at least one row; at most 64 rows per expert
    // (4 tiles of 16 or 2 of 32) unless all rows take small tiles, then at
    // most one partial tile per non-empty expert
    const int64_t m_small =
        all_small ? std::min<int64_t>(total_rows, total_rows / small_bm + std::min<int64_t>(experts, total_rows))
                  : std::min<int64_t>((int64_t)experts * 4, total_rows);
    if (stream_ok) {
        q.n_tiles = ceil_div(p.N, MODE == kModeGateUp ? kSkBN / 2 : kSkBN);
        return launch_stream_gemm<MODE>(q, m_small, small_bm, st);
    }
    q.ksplit = 1;
    q.n_tiles = ceil_div(p.N, big_cols);
    if (p.K % kBK != 0)
        return launch_gemm<32, 256, 1, 4, MODE, true>(q, m_small, st);
    return launch_gemm<32, 256, 1, 4, MODE>(q, m_small, st);
}

// ---------------------------------------------------------------- MoE ws
struct RouteLayout {
    size_t hist, base, tot, offsets, plan_gu, plan_dn, end;
};

RouteLayout route_layout(int64_t npairs, int32_t E)
{
    RouteLayout L{};
    const int64_t nchunks = std::max<int64_t>(1, ceil_div(npairs, kRouteChunk));
    size_t o = 0;
    L.hist = o; o = align256(o + sizeof(int32_t) * nchunks * E);
    L.base = o; o = align256(o + sizeof(int32_t) * nchunks * E);
    L.tot = o; o = align256(o + sizeof(int32_t) * E);
    L.offsets = o; o = align256(o + sizeof(int32_t) * (E + 1));
    L.plan_gu = o; o = align256(o + sizeof(int32_t) * 3 * kPlanClasses * (E + 1));
    L.plan_dn = o; o = align256(o + sizeof(int32_t) * 3 * kPlanClasses * (E + 1));
    L.end = o;
    return L;
}

struct MoeLayout {
    RouteLayout r;
    size_t perm, inv, xparts, xq_p, xq_s, gx, gpart, h, hmax, hq_p, hq_s, gh, y, end;
};

MoeLayout moe_layout(int64_t T, int32_t k, int32_t E, int64_t H, int64_t I)
{
    MoeLayout L{};
    const int64_t np = T * k;
    L.r = route_layout(np, E);
    size_t o = L.r.end;
    L.perm = o; o = align256(o + sizeof(int32_t) * np);
    L.inv = o; o = align256(o + sizeof(int32_t) * np);
    L.xparts = o; o = align256(o + sizeof(uint32_t) * kAmaxParts);
    L.xq_p = o; o = align256(o + (size_t)(T * H / 2));
    L.xq_s = o; o = align256(o + (size_t)(T * H / 16));
    L.gx = o; o = align256(o + sizeof(float));
    const int gs = moe_gate_ksplit(T, k, E, H, I);
    L.gpart = o; o = align256(o + (gs > 1 ? sizeof(float) * (size_t)(np * 2 * I) * gs : 0));
    L.h = o; o = align256(o + sizeof(uint16_t) * (size_t)(np * I));
    L.hmax = o; o = align256(o + sizeof(uint32_t));
    L.hq_p = o; o = align256(o + (size_t)(np * I / 2));
    L.hq_s = o; o = align256(o + (size_t)(np * I / 16));
    L.gh = o; o = align256(o + sizeof(float));
    L.y = o; o = align256(o + sizeof(float) * (size_t)(np * H) * moe_down_ksplit(T, k, E, H, I));
    L.end = o;
    return L;
}

template <typename T>
inline T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

// Route the T*k pairs.  Small batches take one workgroup, which can also
// write the two tile plans (plan_gu / plan_dn non-null) for the fused layer.
nvfp4_status route_impl(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* perm,
                        int32_t* offsets, int32_t* inv, void* ws, const RouteLayout& L,
                        uint32_t* zero_word, hipStream_t st, int32_t* plan_gu = nullptr,
                        int small_bm_gu = 0, int all_small_gu = 0, int32_t* plan_dn = nullptr,
                        int small_bm_dn = 0, int all_small_dn = 0)
{
    const int64_t np = T * k;
    if (np <= kRouteSmall) {
        route_small_kernel<<<1, 1024, 0, st>>>(ids, (int)np, E, offsets, perm, inv, zero_word, plan_gu,
                                               small_bm_gu, all_small_gu, plan_dn, small_bm_dn, all_small_dn);
        return launch_status();
    }
    if (plan_gu || plan_dn)
        return NVFP4_ERR_INVALID_ARG;  // plans come from the small route only
    const int64_t nchunks = ceil_div(np, kRouteChunk);
    if (np > 0) {
        route_hist_kernel<<<(unsigned)nchunks, kRouteChunk, sizeof(int32_t) * E, st>>>(
            ids, np, E, at<int32_t>(ws, L.hist));
        route_expert_scan_kernel<<<(unsigned)E, 256, 0, st>>>(
            at<int32_t>(ws, L.hist), nchunks, E, at<int32_t>(ws, L.base), at<int32_t>(ws, L.tot));
    } else {
        // no pairs: every expert is empty
        fill_i32_kernel<<<stream_grid(E), 256, 0, st>>>(at<int32_t>(ws, L.tot), E, 0);
    }
    route_offsets_kernel<<<1, 1024, 0, st>>>(at<int32_t>(ws, L.tot), E, offsets, zero_word);
    if (np > 0)
        route_scatter_kernel<<<(unsigned)nchunks, kRouteChunk, 0, st>>>(
            ids, np, E, at<int32_t>(ws, L.base), offsets, perm, inv);
    return launch_status();
}

}  // namespace

// ======================================================================== ABI

// ---------------------------------------------------------------- MX MoE
// Workspace of mx_moe_w4a8: routing, one tile plan (both projections share
// the expert offsets), MXFP8 x, h (bf16), MXFP8 h, y (fp32).
struct MxMoeLayout {
    RouteLayout r;
    size_t perm, inv, plan, xq, xs, h, hmax, hq, hs, y, end;
};

MxMoeLayout mx_moe_layout(int64_t T, int32_t k, int32_t E, int64_t H, int64_t I)
{
    MxMoeLayout L{};
    const int64_t np = T * k;
    L.r = route_layout(np, E);
    size_t o = L.r.end;
    L.perm = o; o = align256(o + sizeof(int32_t) * np);
    L.inv = o; o = align256(o + sizeof(int32_t) * np);
    L.plan = o; o = align256(o + sizeof(int32_t) * 3 * kPlanClasses * (E + 1));
    L.xq = o; o = align256(o + (size_t)(T * H));
    L.xs = o; o = align256(o + (size_t)(T * H / 32));
    L.h = o; o = align256(o + sizeof(uint16_t) * (size_t)(np * I));
    L.hmax = o; o = align256(o + sizeof(uint32_t));
    L.hq = o; o = align256(o + (size_t)(np * I));
    L.hs = o; o = align256(o + (size_t)(np * I / 32));
    L.y = o; o = align256(o + sizeof(float) * (size_t)(np * H));
    L.end = o;
    return L;
}

template <int BM, int MODE>
nvfp4_status launch_mx_grouped_class(MxArgs q, int64_t m_tiles_ub, hipStream_t st)
{
    q.m_tiles = m_tiles_ub;
    const int64_t blocks = ceil_div(m_tiles_ub * q.n_tiles, 8) * 8;
    if (blocks == 0)
        return NVFP4_OK;
    if (blocks > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    mx_w4a8_kernel<BM, 256, MODE><<<(unsigned)blocks, 256, 0, st>>>(q);
    return launch_status();
}

// Tile plan of the MX layer: 64-row small tiles; with at most 64 tokens
// every row takes them (top-k sends a token to an expert at most once, so
// no expert could fill a larger tile; any ids are still covered).
int mx_all_small(int64_t T) { return T <= 64 ? 1 : 0; }

// Rows of the MX layer's small tiles: 32-row weight-streaming tiles when
// every row takes small tiles and both projections' K (H, and I) are
// multiples of the 256-element stage (H always is), else 64-row tiles of the
// tile kernel.  One plan serves both projections.
int mx_small_bm(int64_t T, int64_t I) { return (mx_all_small(T) && I % kMsBK == 0) ? kMsBM : 64; }

// Workgroups of the MX streaming kernel the device holds at once (a multiple
// of 8; one query per mode and device, cached as stream_resident caches).
template <int MODE, bool SC4>
int64_t mx_stream_resident()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        dev = 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mx_stream_kernel<MODE, SC4>, 256, 0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 8;
        v = std::max(8, per_cu * cus / 8 * 8);
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// The 32-row weight-streaming class of an MX projection: items of (A tile,
// 64 h columns (gate_up) or 128 W rows), a resident grid.
template <int MODE>
nvfp4_status launch_mx_stream(MxArgs q, int64_t m_tiles_ub, hipStream_t st)
{
    if (q.K % kMsBK != 0)
        return NVFP4_ERR_SHAPE;
    q.m_tiles = m_tiles_ub;
    q.n_tiles = ceil_div(q.N, MODE == kModeGateUp ? 64 : kMsBN);
    const int64_t items = m_tiles_ub * q.n_tiles;
    if (items == 0)
        return NVFP4_OK;
    if (items > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    // scale bytes of four stages per request when every item holds whole
    // four-stage chunks and the scale arrays are 16-byte aligned
    const bool sc4 = q.K % (4 * kMsBK) == 0 && (((uintptr_t)q.w_sc | (uintptr_t)q.a_sc) & 15) == 0;
    if (sc4) {
        const int64_t blocks = std::min(ceil_div(items, 8) * 8, mx_stream_resident<MODE, true>());
        mx_stream_kernel<MODE, true><<<(unsigned)blocks, 256, 0, st>>>(q);
    } else {
        const int64_t blocks = std::min(ceil_div(items, 8) * 8, mx_stream_resident<MODE, false>());
        mx_stream_kernel<MODE, false><<<(unsigned)blocks, 256, 0, st>>>(q);
    }
    return launch_status();
}

// One grouped MX projection over the plan's classes: 256-row tiles, one
// 128-row tile for a remainder of 65-128 rows, one 64-row tile for at most 64
// (only the last when every row takes small tiles; then 32-row streaming
// tiles instead when K allows, as mx_small_bm decides for the plan).
template <int MODE>
nvfp4_status mx_grouped(MxArgs p, const int32_t* plan, int64_t T, int64_t total_rows, int32_t E, hipStream_t st)
{
    const int64_t E1 = E + 1;
    p.n_tiles = ceil_div(p.N, MODE == kModeGateUp ? 128 : 256);
    auto cls = [&](int c) {
        MxArgs q = p;
        q.tile_off = plan + 3 * c * E1;
        q.row_base = q.tile_off + E1;
        q.row_lim = q.tile_off + 2 * E1;
        return q;
    };
    nvfp4_status s = NVFP4_OK;
    const int64_t I = MODE == kModeGateUp ? p.N : p.K;
    if (mx_small_bm(T, I) == kMsBM)
        return launch_mx_stream<MODE>(cls(kPlanSmall), total_rows / kMsBM + std::min<int64_t>(E, total_rows), st);
    if (mx_all_small(T))
        return launch_mx_grouped_class<64, MODE>(cls(kPlanSmall), total_rows / 64 + std::min<int64_t>(E, total_rows), st);
    if (total_rows > 128)
        s = launch_mx_grouped_class<256, MODE>(cls(0), total_rows / 128 + 1, st);
    if (s == NVFP4_OK && total_rows > 64)
        s = launch_mx_grouped_class<128, MODE>(cls(1), std::min<int64_t>(E, total_rows / 65 + 1), st);
    if (s == NVFP4_OK)
        s = launch_mx_grouped_class<64, MODE>(cls(kPlanSmall), std::min<int64_t>(E, total_rows), st);
    return s;
}

// The two MX projections of a routed-expert layer over a tile plan that is
// computed here (plan_ready false) or was already written.
nvfp4_status mx_moe_gate_up_impl(const uint8_t* xq, const uint8_t* xe, const int32_t* perm, const int32_t* offsets,
                                 int64_t T, int32_t k, int32_t E, int64_t H, int64_t I, const uint8_t* w13,
                                 const uint8_t* w13e, void* h, uint32_t* h_amax, int32_t* plan, bool plan_ready,
                                 hipStream_t st)
{
    if (!plan_ready) {
        moe_plan_kernel<<<1, 1024, 0, st>>>(offsets, E, mx_small_bm(T, I), mx_all_small(T), plan);
        nvfp4_status s = launch_status();
        if (s != NVFP4_OK)
            return s;
    }
    MxArgs p{};
    p.a = xq;
    p.a_sc = xe;
    p.w = w13;
    p.w_sc = w13e;
    p.M = T * k;
    p.N = I;
    p.K = H;
    p.perm = perm;
    p.topk = k;
    p.experts = E;
    p.out = h;
    p.h_amax = h_amax;
    return mx_grouped<kModeGateUp>(p, plan, T, T * k, E, st);
}

nvfp4_status mx_moe_down_impl(const uint8_t* hq, const uint8_t* he, const int32_t* offsets, int64_t T, int32_t k,
                              int32_t E, int64_t H, int64_t I, const uint8_t* w2, const uint8_t* w2e, float* y,
                              int32_t* plan, bool plan_ready, hipStream_t st)
{
    if (!plan_ready) {
        moe_plan_kernel<<<1, 1024, 0, st>>>(offsets, E, mx_small_bm(T, I), mx_all_small(T), plan);
        nvfp4_status s = launch_status();
        if (s != NVFP4_OK)
            return s;
    }
    MxArgs q{};
    q.a = hq;
    q.a_sc = he;
    q.w = w2;
    q.w_sc = w2e;
    q.M = T * k;
    q.N = H;
    q.K = I;
    q.topk = k;
    q.experts = E;
    q.out = y;
    return mx_grouped<kModeDown>(q, plan, T, T * k, E, st);
}

nvfp4_status mx_moe_check(int64_t T, int32_t k, int32_t E, int64_t H, int64_t I)
{
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || T * k > 0x7FFFFFFF || H < 0 || I < 0)
        return NVFP4_ERR_SHAPE;
    if (H % 256 != 0 || I % 128 != 0)
        return NVFP4_ERR_UNSUPPORTED;
    return NVFP4_OK;
}

// ---------------------------------------------------------------- scratch
// Library-owned device scratch for the allocation-free MoE entry point
// (nvfp4_moe_grouped_gemm_noalloc): one array per GPU, held from the first
// use of the library on that GPU until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// for the device symbol): it takes the device address from
// hipGetSymbolAddress once per device, with that device current, and uses
// only that address.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, or null with the
// failing status in *st.
void* scratch_address(nvfp4_status* st)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = NVFP4_ERR_DEVICE;
        return nullptr;
    }
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr)
        return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        *st = NVFP4_ERR_DEVICE;
        return nullptr;
    }
    // threads racing on the first call obtain the same address
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    return ptr;
}
}  // namespace

extern "C" {

const char* nvfp4_status_string(int32_t s)
{
    switch (s) {
    case (int32_t)NVFP4_OK: return "ok";
    case (int32_t)NVFP4_ERR_INVALID_ARG: return "invalid argument";
    case (int32_t)NVFP4_ERR_SHAPE: return "invalid shape";
    case (int32_t)NVFP4_ERR_RANGE: return "value out of range";
    case (int32_t)NVFP4_ERR_WORKSPACE: return "workspace too small";
    case (int32_t)NVFP4_ERR_DEVICE: return "HIP device error";
    case (int32_t)NVFP4_ERR_UNSUPPORTED: return "unsupported by this build";
    case (int32_t)NVFP4_ERR_DATA: return "invalid data (non-finite input, bad block scale or global)";
    }
    return "unknown status";
}

const char* nvfp4_build_stamp(void) { return NVFP4_BUILD_STAMP; }

int nvfp4_set_checks(int on) { return g_checks.exchange(on != 0 ? 1 : 0, std::memory_order_relaxed); }

void nvfp4_recipe(int32_t out[6])
{
    if (!out)
        return;
    out[0] = 16;   // block size
    out[1] = 2;    // E2M1 exponent bits
    out[2] = 1;    // E2M1 mantissa bits
    out[3] = 4;    // E4M3 exponent bits
    out[4] = 3;    // E4M3 mantissa bits
    out[5] = 450;  // effective bits x 100: (16*4 + 8) / 16
}

size_t nvfp4_workspace_size(int op, int64_t T, int32_t k, int32_t E, int64_t H, int64_t I)
{
    switch (op) {
    case NVFP4_OP_QUANTIZE:
        return sizeof(uint32_t) * kAmaxParts;
    case NVFP4_OP_REMAP: {
        const int64_t batch = T < 1 ? 1 : T;
        const int64_t blocks = H * (I / 32);
        return align256((size_t)(batch * blocks)) + 2 * align256(sizeof(int) * kRemapParts * batch);
    }
    case NVFP4_OP_GEMM:
        // T = M (A rows), H = K, I = N (W rows)
        if (T <= 0 || H <= 0 || I <= 0)
            return 0;
        return gemm_ws_bytes(T, I, H);
    case NVFP4_OP_MOE:
        if (T < 0 || k < 1 || E < 1)
            return 0;
        return moe_layout(T, k, E, H, I).end;
    case NVFP4_OP_MOE_ROUTE:
        if (T < 0 || k < 1 || E < 1)
            return 0;
        return route_layout(T * k, E).end;
    case NVFP4_OP_MX_MOE:
        if (T < 0 || k < 1 || E < 1)
            return 0;
        return mx_moe_layout(T, k, E, H, I).end;
    }
    return 0;
}

nvfp4_status nvfp4_get_error(void* stream)
{
    if (hipStreamSynchronize(S(stream)) != hipSuccess)
        return NVFP4_ERR_DEVICE;
    unsigned v = 0, zero = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_nvfp4_error), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess)
        return NVFP4_ERR_DEVICE;
    if (v != 0 && hipMemcpyToSymbol(HIP_SYMBOL(g_nvfp4_error), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) != hipSuccess)
        return NVFP4_ERR_DEVICE;
    return (nvfp4_status)v;
}

static nvfp4_status quantize_unchecked(const void* x, int64_t rows, int64_t cols, int64_t ld,
                            const float* static_global, const nvfp4_tensor* out, void* ws,
                            size_t ws_bytes, void* stream)
{
    nvfp4_status s = check_tensor(out);
    if (s != NVFP4_OK)
        return s;
    if ((!x && rows * cols != 0) || !aligned(x, 16))
        return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0 || cols % 16 != 0 || ld < cols || ld % 8 != 0)
        return NVFP4_ERR_SHAPE;
    if (out->rows != rows || out->cols != cols || out->batch != 1)
        return NVFP4_ERR_SHAPE;
    if (static_global) {
        if (!aligned(static_global, 4))
            return NVFP4_ERR_INVALID_ARG;
        return quantize_impl(x, rows, cols, ld, kGlobalStatic, static_global, out, 0, nullptr, S(stream));
    }
    if (!ws || !aligned(ws, 4))
        return NVFP4_ERR_INVALID_ARG;
    if (ws_bytes < nvfp4_workspace_size(NVFP4_OP_QUANTIZE, 0, 0, 0, 0, 0))
        return NVFP4_ERR_WORKSPACE;
    return quantize_impl(x, rows, cols, ld, kGlobalPartials, nullptr, out, 0, (uint32_t*)ws, S(stream));
}

nvfp4_status nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld,
                            const float* static_global, const nvfp4_tensor* out, void* ws,
                            size_t ws_bytes, void* stream)
{
    nvfp4_status s = quantize_unchecked(x, rows, cols, ld, static_global, out, ws, ws_bytes, stream);
    if (s == NVFP4_OK && checks_on()) {
        check_bf16(x, rows, cols, ld, S(stream));
        if (static_global)
            check_globals(static_global, 1, S(stream));
        s = launch_status();
    }
    return s;
}

static nvfp4_status dequantize_unchecked(const nvfp4_tensor* in, void* out, int32_t dtype, void* stream)
{
    nvfp4_status s = check_tensor(in);
    if (s != NVFP4_OK)
        return s;
    if (!out || !aligned(out, 16))
        return NVFP4_ERR_INVALID_ARG;
    if (dtype != NVFP4_F32 && dtype != NVFP4_BF16)
        return NVFP4_ERR_INVALID_ARG;
    const int64_t bpr = in->cols / 16;
    const int64_t nblk = in->batch * in->rows * bpr;
    if (nblk == 0 || in->rows == 0)
        return NVFP4_OK;
    const unsigned grid = stream_grid(ceil_div(2 * nblk, 8), 8192);  // 8 half-blocks per thread per trip
    if (dtype == NVFP4_BF16)
        dequantize_kernel<true><<<grid, kQuantThreads, 0, S(stream)>>>(
            (const uint32_t*)in->packed, in->scales, in->global, nblk, in->rows * bpr, 0, out);
    else
        dequantize_kernel<false><<<grid, kQuantThreads, 0, S(stream)>>>(
            (const uint32_t*)in->packed, in->scales, in->global, nblk, in->rows * bpr, 0, out);
    return launch_status();
}

nvfp4_status nvfp4_dequantize(const nvfp4_tensor* in, void* out, int32_t dtype, void* stream)
{
    nvfp4_status s = dequantize_unchecked(in, out, dtype, stream);
    if (s == NVFP4_OK && checks_on())
        s = check_tensor_data(in, S(stream));
    return s;
}

static nvfp4_status gather_dequantize_unchecked(const nvfp4_tensor* table, const int32_t* ids, int64_t n, void* out,
                                     int32_t dtype, void* stream)
{
    nvfp4_status s = check_tensor(table);
    if (s != NVFP4_OK)
        return s;
    if (table->batch != 1)
        return NVFP4_ERR_SHAPE;
    if (n < 0)
        return NVFP4_ERR_SHAPE;
    if (n == 0 || table->cols == 0)
        return NVFP4_OK;
    if (!ids || !out || !aligned(out, 16) || !aligned(ids, 4))
        return NVFP4_ERR_INVALID_ARG;
    if (dtype != NVFP4_F32 && dtype != NVFP4_BF16)
        return NVFP4_ERR_INVALID_ARG;
    const int64_t hpr = table->cols / 8;
    if (n * hpr >= ((int64_t)1 << 32) - 4 * kQuantThreads)
        return NVFP4_ERR_UNSUPPORTED;
    const unsigned grid = stream_grid(ceil_div(n * hpr, 4), 8192);  // 4 row slices of 8 per thread
    if (dtype == NVFP4_BF16)
        gather_dequant_kernel<true><<<grid, kQuantThreads, 0, S(stream)>>>(
            (const uint32_t*)table->packed, table->scales, table->global, ids, (uint32_t)n, table->rows,
            (uint32_t)hpr, out);
    else
        gather_dequant_kernel<false><<<grid, kQuantThreads, 0, S(stream)>>>(
            (const uint32_t*)table->packed, table->scales, table->global, ids, (uint32_t)n, table->rows,
            (uint32_t)hpr, out);
    return launch_status();
}

nvfp4_status nvfp4_gather_dequantize(const nvfp4_tensor* table, const int32_t* ids, int64_t n, void* out,
                                     int32_t dtype, void* stream)
{
    nvfp4_status s = gather_dequantize_unchecked(table, ids, n, out, dtype, stream);
    if (s == NVFP4_OK && checks_on())
        s = check_tensor_data(table, S(stream));
    return s;
}

nvfp4_status nvfp4_tile_scales(const nvfp4_tensor* in, uint8_t* scales_out, void* stream)
{
    nvfp4_status s = check_tensor(in, false);
    if (s != NVFP4_OK)
        return s == NVFP4_ERR_UNSUPPORTED ? NVFP4_ERR_INVALID_ARG : s;  // (already tiled)
    if (in->rows % 128 != 0 || in->cols % 256 != 0)
        return NVFP4_ERR_SHAPE;
    const int64_t bytes = in->batch * in->rows * (in->cols / 16);
    if (bytes == 0)
        return NVFP4_OK;
    if (!scales_out || !aligned(scales_out, 16) || !aligned(in->scales, 16))
        return NVFP4_ERR_INVALID_ARG;
    const uint8_t *a = in->scales, *b = scales_out;
    if (a < b + bytes && b < a + bytes)
        return NVFP4_ERR_INVALID_ARG;  // the runs move: no in-place tiling
    const int64_t n = bytes / 16;
    tile_scales_kernel<<<stream_grid(n, 8192), 256, 0, S(stream)>>>((const u32x4*)in->scales, (u32x4*)scales_out,
                                                                     in->rows, in->cols / 256, n);
    return launch_status();
}

nvfp4_status mxfp4_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* packed,
                            uint8_t* e8m0, void* stream)
{
    if (!x || !packed || !e8m0 || !aligned(x, 16) || !aligned(packed, 16))
        return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0 || cols % 32 != 0 || ld < cols || ld % 8 != 0)
        return NVFP4_ERR_SHAPE;
    const int64_t bpr = cols / 32;
    const int64_t nblk = rows * bpr;
    if (nblk == 0)
        return NVFP4_OK;
    mxfp4_encode_kernel<<<stream_grid(nblk, 8192), kMxThreads, 0, S(stream)>>>(
        (const u32x4*)x, rows, bpr, ld / 8, (u32x4*)packed, e8m0);
    return launch_status();
}

nvfp4_status mxfp4_to_nvfp4(const uint8_t* mx_packed, const uint8_t* e8m0, int64_t rows, int64_t cols,
                            int64_t batch, const nvfp4_tensor* out, void* ws, size_t ws_bytes,
                            void* stream)
{
    nvfp4_status s = check_tensor(out);
    if (s != NVFP4_OK)
        return s;
    if (!mx_packed || !e8m0 || !aligned(mx_packed, 16) || !ws || !aligned(ws, 4))
        return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0 || cols % 32 != 0 || batch < 1)
        return NVFP4_ERR_SHAPE;
    if (out->rows != rows || out->cols != cols || out->batch != batch)
        return NVFP4_ERR_SHAPE;
    if (ws_bytes < nvfp4_workspace_size(NVFP4_OP_REMAP, batch, 0, 0, rows, cols))
        return NVFP4_ERR_WORKSPACE;
    if (batch > 65535)
        return NVFP4_ERR_UNSUPPORTED;
    const int64_t per_mat = rows * (cols / 32);
    uint8_t* flags = (uint8_t*)ws;
    int* pmax = at<int>(ws, align256((size_t)(batch * per_mat)));
    int* pmin = pmax + align256(sizeof(int) * kRemapParts * batch) / sizeof(int);
    const unsigned parts = (unsigned)std::max<int64_t>(1, std::min<int64_t>(kRemapParts, ceil_div(per_mat, 256)));
    u32x4* dst = (out->packed == mx_packed) ? nullptr : (u32x4*)out->packed;
    remap_scan_kernel<<<dim3(parts, (unsigned)batch), kMxThreads, 0, S(stream)>>>(
        (const u32x4*)mx_packed, e8m0, per_mat, dst, flags, pmax, pmin);
    s = launch_status();
    if (s != NVFP4_OK)
        return s;
    // 16 blocks per thread when every 16-block group is 16-byte aligned
    const int vec16 = per_mat % 16 == 0 && aligned(e8m0, 16) && aligned(out->scales, 16) && aligned(ws, 16);
    const int64_t items = vec16 ? per_mat / 16 : per_mat;
    // at most 32 workgroups per matrix: each reduces the matrix's partial
    // exponent ranges once and then walks several groups
    const unsigned parts2 = (unsigned)std::max<int64_t>(1, std::min<int64_t>(32, ceil_div(items, 256)));
    remap_scales_kernel<<<dim3(parts2, (unsigned)batch), kMxThreads, 0, S(stream)>>>(
        e8m0, flags, per_mat, pmax, pmin, (int)parts, (uint16_t*)out->scales, out->global, vec16);
    return launch_status();
}

static nvfp4_status gemm_unchecked(const nvfp4_tensor* A, const nvfp4_tensor* W, void* C, int32_t dtype,
                        void* ws, size_t ws_bytes, void* stream)
{
    nvfp4_status s = check_tensor(A);
    if (s == NVFP4_OK)
        s = check_tensor(W, true, true);
    if (s != NVFP4_OK)
        return s;
    if (!C || (dtype != NVFP4_F32 && dtype != NVFP4_BF16))
        return NVFP4_ERR_INVALID_ARG;
    if (A->cols != W->cols || A->batch != 1 || W->batch != 1)
        return NVFP4_ERR_SHAPE;
    if (A->rows == 0 || W->rows == 0)
        return NVFP4_OK;
    if (A->cols == 0)
        return NVFP4_ERR_UNSUPPORTED;
    GemmArgs p{};
    p.a_packed = A->packed;
    p.a_scales = A->scales;
    p.a_global = A->global;
    p.w_packed = W->packed;
    p.w_scales = W->scales;
    p.w_global = W->global;
    p.w_pow2 = (W->flags & NVFP4_POW2_SCALES) != 0;
    p.w_tiled = (W->flags & NVFP4_TILED_SCALES) != 0;
    p.K = A->cols;
    p.M = A->rows;
    p.N = W->rows;
    p.experts = 1;
    p.out = C;
    p.out_bf16 = dtype == NVFP4_BF16;
    p.ksplit = 1;
    const int ksplit = gemm_ksplit(p.M, p.N, p.K);
    if (ksplit > 1 && ws) {
        if (!aligned(ws, 256))
            return NVFP4_ERR_INVALID_ARG;
        if (ws_bytes < gemm_ws_bytes(p.M, p.N, p.K))
            return NVFP4_ERR_WORKSPACE;
        p.ksplit = ksplit;
        p.partial = (float*)ws;
    }
    return dispatch_dense(p, S(stream));
}

nvfp4_status nvfp4_gemm(const nvfp4_tensor* A, const nvfp4_tensor* W, void* C, int32_t dtype,
                        void* ws, size_t ws_bytes, void* stream)
{
    nvfp4_status s = gemm_unchecked(A, W, C, dtype, ws, ws_bytes, stream);
    if (s == NVFP4_OK && checks_on())
        s = check_tensors_data({A, W}, S(stream));
    return s;
}

static nvfp4_status gemm_w4a16_unchecked(const void* a, int64_t M, int64_t K, int64_t lda, const nvfp4_tensor* W,
                              void* C, int32_t dtype, void* ws, size_t ws_bytes, void* stream)
{
    nvfp4_status s = check_tensor(W, true, true);
    if (s != NVFP4_OK)
        return s;
    if (!C || (dtype != NVFP4_F32 && dtype != NVFP4_BF16))
        return NVFP4_ERR_INVALID_ARG;
    if (M < 0 || K < 0 || lda < K || W->cols != K || W->batch != 1)
        return NVFP4_ERR_SHAPE;
    if (M == 0 || W->rows == 0)
        return NVFP4_OK;
    if (K == 0 || K % kSkBK != 0)
        return NVFP4_ERR_UNSUPPORTED;
    if (!a || !aligned(a, 16) || lda % 8 != 0)
        return NVFP4_ERR_INVALID_ARG;
    GemmArgs p{};
    p.a_bf16 = (const uint16_t*)a;
    p.lda = lda;
    p.w_packed = W->packed;
    p.w_scales = W->scales;
    p.w_global = W->global;
    p.w_pow2 = (W->flags & NVFP4_POW2_SCALES) != 0;
    p.w_tiled = (W->flags & NVFP4_TILED_SCALES) != 0;
    p.K = K;
    p.M = M;
    p.N = W->rows;
    p.experts = 1;
    p.out = C;
    p.out_bf16 = dtype == NVFP4_BF16;
    p.ksplit = 1;
    const int ksplit = gemm_ksplit(p.M, p.N, p.K);
    if (ksplit > 1 && ws) {
        if (!aligned(ws, 256))
            return NVFP4_ERR_INVALID_ARG;
        if (ws_bytes < gemm_ws_bytes(p.M, p.N, p.K))
            return NVFP4_ERR_WORKSPACE;
        p.ksplit = ksplit;
        p.partial = (float*)ws;
    }
    return dispatch_dense(p, S(stream));
}

nvfp4_status nvfp4_gemm_w4a16(const void* a, int64_t M, int64_t K, int64_t lda, const nvfp4_tensor* W,
                              void* C, int32_t dtype, void* ws, size_t ws_bytes, void* stream)
{
    nvfp4_status s = gemm_w4a16_unchecked(a, M, K, lda, W, C, dtype, ws, ws_bytes, stream);
    if (s == NVFP4_OK && checks_on()) {
        check_bf16(a, M, K, lda, S(stream));
        s = check_tensors_data({W}, S(stream));
    }
    return s;
}

nvfp4_status mxfp8_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* fp8, uint8_t* e8m0,
                            void* stream)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0 || ld < cols || ld % 8 != 0)
        return NVFP4_ERR_SHAPE;
    const int64_t nblk = rows * (cols / 32);
    if (nblk == 0)
        return NVFP4_OK;
    if (!x || !fp8 || !e8m0 || !aligned(x, 16) || !aligned(fp8, 16))
        return NVFP4_ERR_INVALID_ARG;
    // 4 chunks of 8 elements per thread per trip
    mxfp8_encode_kernel<4><<<stream_grid(ceil_div(4 * nblk, 4), 8192), kMx8Threads, 0, S(stream)>>>(
        (const u32x4*)x, rows, cols / 32, ld / 8, (u32x2*)fp8, e8m0);
    return launch_status();
}

nvfp4_status mx_gemm_w4a8(const uint8_t* a, const uint8_t* a_e8m0, int64_t M, int64_t K, const uint8_t* w,
                          const uint8_t* w_e8m0, int64_t N, void* C, int32_t dtype, void* stream)
{
    if (M < 0 || N < 0 || K < 0)
        return NVFP4_ERR_SHAPE;
    if (dtype != NVFP4_F32 && dtype != NVFP4_BF16)
        return NVFP4_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return NVFP4_OK;
    if (K == 0 || K % kMxGrpK != 0)
        return NVFP4_ERR_UNSUPPORTED;
    if (!a || !a_e8m0 || !w || !w_e8m0 || !C || !aligned(a, 16) || !aligned(w, 16) || !aligned(a_e8m0, 4) ||
        !aligned(w_e8m0, 4))
        return NVFP4_ERR_INVALID_ARG;
    MxArgs p{};
    p.a = a;
    p.a_sc = a_e8m0;
    p.w = w;
    p.w_sc = w_e8m0;
    p.M = M;
    p.N = N;
    p.K = K;
    p.out = C;
    p.out_bf16 = dtype == NVFP4_BF16;
    p.n_tiles = ceil_div(N, 256);
    hipStream_t st = S(stream);
    if (M >= 256) {
        p.m_tiles = ceil_div(M, 256);
        const int64_t blocks = ceil_div(p.m_tiles * p.n_tiles, 8) * 8;
        if (blocks > 0x7FFFFFFF)
            return NVFP4_ERR_SHAPE;
        mx_w4a8_kernel<256, 256, kModeDense><<<(unsigned)blocks, 256, 0, st>>>(p);
    } else {
        p.m_tiles = ceil_div(M, 128);
        const int64_t blocks = ceil_div(p.m_tiles * p.n_tiles, 8) * 8;
        mx_w4a8_kernel<128, 256, kModeDense><<<(unsigned)blocks, 256, 0, st>>>(p);
    }
    return launch_status();
}

nvfp4_status mx_moe_gate_up(const uint8_t* x_fp8, const uint8_t* x_e8m0, const int32_t* perm,
                            const int32_t* offsets, int64_t T, int32_t k, int32_t E, int64_t H, int64_t I,
                            const uint8_t* w13, const uint8_t* w13_e8m0, void* h_bf16, uint32_t* h_amax, void* ws,
                            size_t ws_bytes, void* stream)
{
    nvfp4_status s = mx_moe_check(T, k, E, H, I);
    if (s != NVFP4_OK)
        return s;
    if (T == 0 || I == 0)
        return NVFP4_OK;
    if (!x_fp8 || !x_e8m0 || !perm || !offsets || !w13 || !w13_e8m0 || !h_bf16 || !h_amax || !ws ||
        !aligned(x_fp8, 16) || !aligned(w13, 16) || !aligned(x_e8m0, 4) || !aligned(w13_e8m0, 4) ||
        !aligned(h_bf16, 16) || !aligned(ws, 256))
        return NVFP4_ERR_INVALID_ARG;
    const RouteLayout L = route_layout(T * k, E);
    if (ws_bytes < L.end)
        return NVFP4_ERR_WORKSPACE;
    return mx_moe_gate_up_impl(x_fp8, x_e8m0, perm, offsets, T, k, E, H, I, w13, w13_e8m0, h_bf16, h_amax,
                               at<int32_t>(ws, L.plan_gu), false, S(stream));
}

nvfp4_status mx_moe_down(const uint8_t* h_fp8, const uint8_t* h_e8m0, const int32_t* offsets, int64_t T, int32_t k,
                         int32_t E, int64_t H, int64_t I, const uint8_t* w2, const uint8_t* w2_e8m0, float* y,
                         void* ws, size_t ws_bytes, void* stream)
{
    nvfp4_status s = mx_moe_check(T, k, E, H, I);
    if (s != NVFP4_OK)
        return s;
    if (T == 0 || H == 0)
        return NVFP4_OK;
    if (!h_fp8 || !h_e8m0 || !offsets || !w2 || !w2_e8m0 || !y || !ws || !aligned(h_fp8, 16) || !aligned(w2, 16) ||
        !aligned(h_e8m0, 4) || !aligned(w2_e8m0, 4) || !aligned(y, 16) || !aligned(ws, 256))
        return NVFP4_ERR_INVALID_ARG;
    const RouteLayout L = route_layout(T * k, E);
    if (ws_bytes < L.end)
        return NVFP4_ERR_WORKSPACE;
    return mx_moe_down_impl(h_fp8, h_e8m0, offsets, T, k, E, H, I, w2, w2_e8m0, y, at<int32_t>(ws, L.plan_dn),
                            false, S(stream));
}

nvfp4_status mx_moe_w4a8(const void* x, const int32_t* ids, const float* w, int64_t T, int32_t k, int32_t E,
                         int64_t H, int64_t I, const uint8_t* w13, const uint8_t* w13_e8m0, const uint8_t* w2,
                         const uint8_t* w2_e8m0, void* out, void* ws, size_t ws_bytes, void* stream)
{
    nvfp4_status s = mx_moe_check(T, k, E, H, I);
    if (s != NVFP4_OK)
        return s;
    if (T == 0 || H == 0)
        return NVFP4_OK;
    if (!x || !ids || !w || !w13 || !w13_e8m0 || !w2 || !w2_e8m0 || !out || !ws || !aligned(x, 16) ||
        !aligned(out, 16) || !aligned(ws, 256) || !aligned(w13, 16) || !aligned(w2, 16) || !aligned(w13_e8m0, 4) ||
        !aligned(w2_e8m0, 4))
        return NVFP4_ERR_INVALID_ARG;
    const MxMoeLayout L = mx_moe_layout(T, k, E, H, I);
    if (ws_bytes < L.end)
        return NVFP4_ERR_WORKSPACE;
    hipStream_t st = S(stream);
    const int64_t np = T * k;
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* inv = at<int32_t>(ws, L.inv);
    int32_t* offsets = at<int32_t>(ws, L.r.offsets);
    int32_t* plan = at<int32_t>(ws, L.plan);
    uint32_t* hmax = at<uint32_t>(ws, L.hmax);
    // 1. route (also zeroes the h max word); one tile plan serves both
    // projections, written by the route's workgroup when the batch is small
    if (np <= kRouteSmall) {
        if ((s = route_impl(ids, T, k, E, perm, offsets, inv, ws, L.r, hmax, st, plan, mx_small_bm(T, I),
                            mx_all_small(T))) != NVFP4_OK)
            return s;
    } else {
        if ((s = route_impl(ids, T, k, E, perm, offsets, inv, ws, L.r, hmax, st)) != NVFP4_OK)
            return s;
        moe_plan_kernel<<<1, 1024, 0, st>>>(offsets, E, mx_small_bm(T, I), mx_all_small(T), plan);
        if ((s = launch_status()) != NVFP4_OK)
            return s;
    }
    // 2. x -> MXFP8 (token order)
    if ((s = mxfp8_quantize(x, T, H, H, at<uint8_t>(ws, L.xq), at<uint8_t>(ws, L.xs), stream)) != NVFP4_OK)
        return s;
    // 3. gate_up + SwiGLU (h bf16, list order)
    if ((s = mx_moe_gate_up_impl(at<uint8_t>(ws, L.xq), at<uint8_t>(ws, L.xs), perm, offsets, T, k, E, H, I, w13,
                                 w13_e8m0, at<void>(ws, L.h), hmax, plan, true, st)) != NVFP4_OK)
        return s;
    // 4. h -> MXFP8 (list order)
    if ((s = mxfp8_quantize(at<void>(ws, L.h), np, I, I, at<uint8_t>(ws, L.hq), at<uint8_t>(ws, L.hs), stream)) !=
        NVFP4_OK)
        return s;
    // 5. down (y fp32, list order)
    if ((s = mx_moe_down_impl(at<uint8_t>(ws, L.hq), at<uint8_t>(ws, L.hs), offsets, T, k, E, H, I, w2, w2_e8m0,
                              at<float>(ws, L.y), plan, true, st)) != NVFP4_OK)
        return s;
    // 6. router-weighted combine
    launch_combine(at<float>(ws, L.y), inv, w, T, k, H, 1, 0, out, st);
    return launch_status();
}

nvfp4_status nvfp4_moe_route(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* perm,
                             int32_t* offsets, int32_t* inv, void* ws, size_t ws_bytes, void* stream)
{
    if (!ids || !perm || !offsets || !inv || !ws || !aligned(ws, 256))
        return NVFP4_ERR_INVALID_ARG;
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || T * k > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    const RouteLayout L = route_layout(T * k, E);
    if (ws_bytes < L.end)
        return NVFP4_ERR_WORKSPACE;
    return route_impl(ids, T, k, E, perm, offsets, inv, ws, L, nullptr, S(stream));
}

static nvfp4_status check_experts(const nvfp4_tensor* w13, const nvfp4_tensor* w2, int32_t E,
                                  int64_t* H, int64_t* I)
{
    nvfp4_status s = NVFP4_OK;
    if (w13) {
        s = check_tensor(w13, true, true);
        if (s != NVFP4_OK)
            return s;
        if (w13->batch != E || w13->rows % 2 != 0)
            return NVFP4_ERR_SHAPE;
        *H = w13->cols;
        *I = w13->rows / 2;
    }
    if (w2) {
        s = check_tensor(w2, true, true);
        if (s != NVFP4_OK)
            return s;
        if (w2->batch != E)
            return NVFP4_ERR_SHAPE;
        if (w13 && (w2->rows != *H || w2->cols != *I))
            return NVFP4_ERR_SHAPE;
        *H = w2->rows;
        *I = w2->cols;
    }
    return NVFP4_OK;
}

static nvfp4_status moe_gate_up_impl(const nvfp4_tensor* xq, const int32_t* perm, const int32_t* offsets,
                                     int64_t T, int32_t k, int32_t E, const nvfp4_tensor* w13, void* h,
                                     uint32_t* h_amax, void* ws, size_t ws_bytes, bool plan_ready,
                                     hipStream_t st, int ksplit = 1, float* gpart = nullptr,
                                     const float* hq_global = nullptr, const nvfp4_tensor* hq = nullptr)
{
    int64_t H = 0, I = 0;
    nvfp4_status s = check_experts(w13, nullptr, E, &H, &I);
    if (s == NVFP4_OK)
        s = check_tensor(xq);
    if (s != NVFP4_OK)
        return s;
    if (!perm || !offsets || !ws || !aligned(ws, 256))
        return NVFP4_ERR_INVALID_ARG;
    if (hq_global) {
        // h encoded in the epilogue: hq rows are list positions
        if (!hq || !hq->packed || !hq->scales || !aligned(hq_global, 4) || !aligned(hq->packed, 4))
            return NVFP4_ERR_INVALID_ARG;
    } else if (!h || !h_amax) {
        return NVFP4_ERR_INVALID_ARG;
    }
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || xq->rows != T || xq->cols != H || xq->batch != 1)
        return NVFP4_ERR_SHAPE;
    if (H % 16 != 0 || I % 16 != 0 || H == 0 || I == 0)
        return NVFP4_ERR_SHAPE;
    const RouteLayout L = route_layout(T * k, E);
    if (ws_bytes < L.end)
        return NVFP4_ERR_WORKSPACE;
    if (T == 0)
        return NVFP4_OK;
    GemmArgs p{};
    p.a_packed = xq->packed;
    p.a_scales = xq->scales;
    p.a_global = xq->global;
    p.w_packed = w13->packed;
    p.w_scales = w13->scales;
    p.w_global = w13->global;
    p.w_pow2 = (w13->flags & NVFP4_POW2_SCALES) != 0;
    p.w_tiled = (w13->flags & NVFP4_TILED_SCALES) != 0;
    p.K = H;
    p.N = I;
    p.perm = perm;
    p.topk = k;
    p.experts = E;
    if (hq_global && (hq->rows != T * k || hq->cols != I || hq->batch != 1))
        return NVFP4_ERR_SHAPE;
    p.out = h;
    p.h_amax = h_amax;
    p.hq_global = hq_global;
    p.hq_packed = hq_global ? hq->packed : nullptr;
    p.hq_scales = hq_global ? hq->scales : nullptr;
    p.M = T * k;
    p.ksplit = gpart ? ksplit : 1;
    p.partial = gpart;
    return dispatch_grouped<kModeGateUp>(p, offsets, T * k, E,
                                         grouped_all_small(T, H, p.ksplit, grouped_ragged(kModeGateUp, H, I)),
                                         at<int32_t>(ws, L.plan_gu), plan_ready, st);
}

static nvfp4_status moe_gate_up_unchecked(const nvfp4_tensor* xq, const int32_t* perm, const int32_t* offsets,
                               int64_t T, int32_t k, int32_t E, const nvfp4_tensor* w13, void* h,
                               uint32_t* h_amax, void* ws, size_t ws_bytes, void* stream)
{
    return moe_gate_up_impl(xq, perm, offsets, T, k, E, w13, h, h_amax, ws, ws_bytes, false, S(stream));
}

nvfp4_status nvfp4_moe_gate_up(const nvfp4_tensor* xq, const int32_t* perm, const int32_t* offsets,
                               int64_t T, int32_t k, int32_t E, const nvfp4_tensor* w13, void* h,
                               uint32_t* h_amax, void* ws, size_t ws_bytes, void* stream)
{
    nvfp4_status s = moe_gate_up_unchecked(xq, perm, offsets, T, k, E, w13, h, h_amax, ws, ws_bytes, stream);
    if (s == NVFP4_OK && checks_on())
        s = check_tensors_data({xq, w13}, S(stream));
    return s;
}

static nvfp4_status moe_gate_up_q_unchecked(const nvfp4_tensor* xq, const int32_t* perm, const int32_t* offsets,
                                 int64_t T, int32_t k, int32_t E, const nvfp4_tensor* w13,
                                 const float* h_global, const nvfp4_tensor* hq, void* ws, size_t ws_bytes,
                                 void* stream)
{
    if (!h_global)
        return NVFP4_ERR_INVALID_ARG;
    return moe_gate_up_impl(xq, perm, offsets, T, k, E, w13, nullptr, nullptr, ws, ws_bytes, false, S(stream),
                            1, nullptr, h_global, hq);
}

nvfp4_status nvfp4_moe_gate_up_q(const nvfp4_tensor* xq, const int32_t* perm, const int32_t* offsets,
                                 int64_t T, int32_t k, int32_t E, const nvfp4_tensor* w13,
                                 const float* h_global, const nvfp4_tensor* hq, void* ws, size_t ws_bytes,
                                 void* stream)
{
    nvfp4_status s = moe_gate_up_q_unchecked(xq, perm, offsets, T, k, E, w13, h_global, hq, ws, ws_bytes, stream);
    if (s == NVFP4_OK && checks_on()) {
        check_globals(h_global, 1, S(stream));
        s = check_tensors_data({xq, w13}, S(stream));
    }
    return s;
}

static nvfp4_status moe_down_impl(const nvfp4_tensor* hq, const int32_t* offsets, int64_t T, int32_t k,
                                  int32_t E, const nvfp4_tensor* w2, float* y, int ksplit, void* ws,
                                  size_t ws_bytes, bool plan_ready, hipStream_t st)
{
    int64_t H = 0, I = 0;
    nvfp4_status s = check_experts(nullptr, w2, E, &H, &I);
    if (s == NVFP4_OK)
        s = check_tensor(hq);
    if (s != NVFP4_OK)
        return s;
    if (!offsets || !y || !ws || !aligned(ws, 256))
        return NVFP4_ERR_INVALID_ARG;
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || hq->rows != T * k || hq->cols != I || hq->batch != 1)
        return NVFP4_ERR_SHAPE;
    if (H % 16 != 0 || I % 16 != 0 || H == 0 || I == 0)
        return NVFP4_ERR_SHAPE;
    const RouteLayout L = route_layout(T * k, E);
    if (ws_bytes < L.end)
        return NVFP4_ERR_WORKSPACE;
    if (T == 0)
        return NVFP4_OK;
    GemmArgs p{};
    p.a_packed = hq->packed;
    p.a_scales = hq->scales;
    p.a_global = hq->global;
    p.w_packed = w2->packed;
    p.w_scales = w2->scales;
    p.w_global = w2->global;
    p.w_pow2 = (w2->flags & NVFP4_POW2_SCALES) != 0;
    p.w_tiled = (w2->flags & NVFP4_TILED_SCALES) != 0;
    p.K = I;
    p.N = H;
    p.M = T * k;
    p.topk = k;
    p.experts = E;
    p.out = y;
    p.ksplit = ksplit;
    p.partial = y;
    return dispatch_grouped<kModeDown>(p, offsets, T * k, E,
                                       grouped_all_small(T, I, ksplit, grouped_ragged(kModeDown, I, H)),
                                       at<int32_t>(ws, L.plan_dn), plan_ready, st);
}

static nvfp4_status moe_down_unchecked(const nvfp4_tensor* hq, const int32_t* offsets, int64_t T, int32_t k,
                            int32_t E, const nvfp4_tensor* w2, float* y, void* ws, size_t ws_bytes,
                            void* stream)
{
    return moe_down_impl(hq, offsets, T, k, E, w2, y, 1, ws, ws_bytes, false, S(stream));
}

nvfp4_status nvfp4_moe_down(const nvfp4_tensor* hq, const int32_t* offsets, int64_t T, int32_t k,
                            int32_t E, const nvfp4_tensor* w2, float* y, void* ws, size_t ws_bytes,
                            void* stream)
{
    nvfp4_status s = moe_down_unchecked(hq, offsets, T, k, E, w2, y, ws, ws_bytes, stream);
    if (s == NVFP4_OK && checks_on())
        s = check_tensors_data({hq, w2}, S(stream));
    return s;
}

nvfp4_status nvfp4_moe_combine(const float* y, const int32_t* inv, const float* w, int64_t T, int32_t k,
                               int64_t H, void* out, void* stream)
{
    if (T < 0 || k < 1 || H < 0 || H % 8 != 0)
        return NVFP4_ERR_SHAPE;
    if (T == 0 || H == 0)
        return NVFP4_OK;
    if (!y || !inv || !w || !out || !aligned(y, 16) || !aligned(out, 8))
        return NVFP4_ERR_INVALID_ARG;
    launch_combine(y, inv, w, T, k, H, 1, 0, out, S(stream));
    return launch_status();
}

static nvfp4_status moe_grouped_gemm_impl(const void* x, const int32_t* ids, const float* w, int64_t T,
                                          int32_t k, int32_t E, const nvfp4_tensor* w13,
                                          const nvfp4_tensor* w2, const float* static_in_globals, void* out,
                                          void* ws, size_t ws_bytes, void* stream)
{
    int64_t H = 0, I = 0;
    nvfp4_status s = check_experts(w13, w2, E, &H, &I);
    if (s != NVFP4_OK)
        return s;
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || T * k > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    if (H % 16 != 0 || I % 16 != 0 || H == 0 || I == 0)
        return NVFP4_ERR_SHAPE;
    if (T == 0)
        return NVFP4_OK;
    if (!x || !ids || !w || !out || !ws || !aligned(x, 16) || !aligned(out, 16) || !aligned(ws, 256))
        return NVFP4_ERR_INVALID_ARG;
    const MoeLayout L = moe_layout(T, k, E, H, I);
    if (ws_bytes < L.end)
        return NVFP4_ERR_WORKSPACE;
    hipStream_t st = S(stream);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* inv = at<int32_t>(ws, L.inv);
    int32_t* offsets = at<int32_t>(ws, L.r.offsets);
    uint32_t* hmax = at<uint32_t>(ws, L.hmax);
    // 1. route (also zeroes the h max word); a small batch routes in one
    // workgroup that also plans both projections' tiles
    const int ksplit = moe_down_ksplit(T, k, E, H, I);
    const int gsplit = moe_gate_ksplit(T, k, E, H, I);
    const bool small = T * k <= kRouteSmall;
    const bool rag_gu = grouped_ragged(kModeGateUp, H, I), rag_dn = grouped_ragged(kModeDown, I, H);
    const int small_gu = grouped_all_small(T, H, gsplit, rag_gu), small_dn = grouped_all_small(T, I, ksplit, rag_dn);
    nvfp4_tensor xq{at<uint8_t>(ws, L.xq_p), at<uint8_t>(ws, L.xq_s), at<float>(ws, L.gx), T, H, 1};
    int pre_parts = 0;  // partial maxima of x written by the routing launch
    // a batch of at most kQuantSmall elements is quantized whole by that launch
    const bool xq_fused = small && !static_in_globals && T * H <= kQuantSmall;
    if (small && !static_in_globals) {
        // one launch: routing and both tile plans in block 0, the first pass
        // of x's dynamic global (or all of x's quantize) in the others
        pre_parts = xq_fused ? 1 : (int)std::max<int64_t>(1, std::min<int64_t>(kAmaxParts, ceil_div(T * (H / 8), 1024)));
        route_small_amax_kernel<<<1 + pre_parts, 1024, 0, st>>>(
            ids, (int)(T * k), E, offsets, perm, inv, hmax, at<int32_t>(ws, L.r.plan_gu),
            grouped_small_bm(H, small_gu, T * k, E, rag_gu), small_gu, at<int32_t>(ws, L.r.plan_dn),
            grouped_small_bm(I, small_dn, T * k, E, rag_dn), small_dn, (const u32x4*)x, T, H / 8, H / 8,
            at<uint32_t>(ws, L.xparts), xq_fused ? (uint32_t*)xq.packed : nullptr, xq_fused ? xq.scales : nullptr,
            xq_fused ? xq.global : nullptr);
        s = launch_status();
    } else if (small) {
        s = route_impl(ids, T, k, E, perm, offsets, inv, ws, L.r, hmax, st, at<int32_t>(ws, L.r.plan_gu),
                       grouped_small_bm(H, small_gu, T * k, E, rag_gu), small_gu, at<int32_t>(ws, L.r.plan_dn),
                       grouped_small_bm(I, small_dn, T * k, E, rag_dn), small_dn);
    } else {
        s = route_impl(ids, T, k, E, perm, offsets, inv, ws, L.r, hmax, st);
    }
    if (s != NVFP4_OK)
        return s;
    // 2. quantize x once (unless the routing launch did)
    if (static_in_globals)
        s = quantize_impl(x, T, H, H, kGlobalStatic, static_in_globals, &xq, 0, nullptr, st);
    else if (!xq_fused)
        s = quantize_impl(x, T, H, H, kGlobalPartials, nullptr, &xq, 0, at<uint32_t>(ws, L.xparts), st,
                          pre_parts);
    if (s != NVFP4_OK)
        return s;
    // 3. gate_up + SwiGLU; with a static G_h the epilogue encodes h to NVFP4
    // directly (no bf16 h, no max, no separate quantize)
    void* h = at<void>(ws, L.h);
    nvfp4_tensor hq{at<uint8_t>(ws, L.hq_p), at<uint8_t>(ws, L.hq_s), at<float>(ws, L.gh), T * k, I, 1};
    if (static_in_globals)
        hq.global = (float*)(static_in_globals + 1);
    s = moe_gate_up_impl(&xq, perm, offsets, T, k, E, w13, h, hmax, ws, L.r.end, small, st, gsplit,
                         gsplit > 1 ? at<float>(ws, L.gpart) : nullptr,
                         static_in_globals ? static_in_globals + 1 : nullptr, &hq);
    if (s != NVFP4_OK)
        return s;
    // 4. quantize h over all T*k rows (dynamic G_h from the max word)
    if (!static_in_globals) {
        s = quantize_impl(h, T * k, I, I, kGlobalAmaxWord, hmax, &hq, 0, nullptr, st);
        if (s != NVFP4_OK)
            return s;
    }
    // 5. down (K split into planes of y for tiny batches)
    float* y = at<float>(ws, L.y);
    s = moe_down_impl(&hq, offsets, T, k, E, w2, y, ksplit, ws, L.r.end, small, st);
    if (s != NVFP4_OK)
        return s;
    // 6. combine (adds the planes of y in order)
    if (!w || H % 8 != 0)
        return NVFP4_ERR_SHAPE;
    launch_combine(y, inv, w, T, k, H, ksplit, T * k * H, out, st);
    return launch_status();
}

nvfp4_status nvfp4_moe_grouped_gemm(const void* x, const int32_t* ids, const float* w, int64_t T,
                                    int32_t k, int32_t E, const nvfp4_tensor* w13,
                                    const nvfp4_tensor* w2, const float* static_in_globals, void* out,
                                    void* ws, size_t ws_bytes, void* stream)
{
    nvfp4_status s =
        moe_grouped_gemm_impl(x, ids, w, T, k, E, w13, w2, static_in_globals, out, ws, ws_bytes, stream);
    if (s == NVFP4_OK && checks_on() && T > 0) {
        check_bf16(x, T, w13->cols, w13->cols, S(stream));
        if (static_in_globals)
            check_globals(static_in_globals, 2, S(stream));
        s = check_tensors_data({w13, w2}, S(stream));
    }
    return s;
}

static nvfp4_status moe_w4a16_unchecked(const void* x, const int32_t* ids, const float* w, int64_t T, int32_t k,
                             int32_t E, const nvfp4_tensor* w13, const nvfp4_tensor* w2, void* out, void* ws,
                             size_t ws_bytes, void* stream)
{
    int64_t H = 0, I = 0;
    nvfp4_status s = check_experts(w13, w2, E, &H, &I);
    if (s != NVFP4_OK)
        return s;
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || T * k > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    if (H % kSkBK != 0 || I % kSkBK != 0 || H % 8 != 0)
        return NVFP4_ERR_UNSUPPORTED;
    if (T == 0)
        return NVFP4_OK;
    if (!x || !ids || !w || !out || !ws || !aligned(x, 16) || !aligned(out, 16) || !aligned(ws, 256))
        return NVFP4_ERR_INVALID_ARG;
    const MoeLayout L = moe_layout(T, k, E, H, I);
    if (ws_bytes < L.end)
        return NVFP4_ERR_WORKSPACE;
    hipStream_t st = S(stream);
    int32_t* perm = at<int32_t>(ws, L.perm);
    int32_t* inv = at<int32_t>(ws, L.inv);
    int32_t* offsets = at<int32_t>(ws, L.r.offsets);
    uint32_t* hmax = at<uint32_t>(ws, L.hmax);
    // 1. route; every tile of both projections is a 16-row streaming tile
    const int ksplit = moe_down_ksplit(T, k, E, H, I);
    const int gsplit = moe_gate_ksplit(T, k, E, H, I);
    const bool small = T * k <= kRouteSmall;
    if (small)
        s = route_impl(ids, T, k, E, perm, offsets, inv, ws, L.r, hmax, st, at<int32_t>(ws, L.r.plan_gu),
                       grouped_small_bm(H, 1, T * k, E), 1, at<int32_t>(ws, L.r.plan_dn),
                       grouped_small_bm(I, 1, T * k, E), 1);
    else
        s = route_impl(ids, T, k, E, perm, offsets, inv, ws, L.r, hmax, st);
    if (s != NVFP4_OK)
        return s;
    // 2. gate_up + SwiGLU from the bf16 rows of x (h bf16, list order)
    GemmArgs p{};
    p.a_bf16 = (const uint16_t*)x;
    p.lda = H;
    p.w_packed = w13->packed;
    p.w_scales = w13->scales;
    p.w_global = w13->global;
    p.w_pow2 = (w13->flags & NVFP4_POW2_SCALES) != 0;
    p.w_tiled = (w13->flags & NVFP4_TILED_SCALES) != 0;
    p.K = H;
    p.N = I;
    p.M = T * k;
    p.perm = perm;
    p.topk = k;
    p.experts = E;
    p.out = at<void>(ws, L.h);
    p.h_amax = hmax;
    p.ksplit = gsplit;
    p.partial = gsplit > 1 ? at<float>(ws, L.gpart) : nullptr;
    s = dispatch_grouped<kModeGateUp>(p, offsets, T * k, E, 1, at<int32_t>(ws, L.r.plan_gu), small, st);
    if (s != NVFP4_OK)
        return s;
    // 3. down from the bf16 h rows (K split into planes of y for tiny batches)
    float* y = at<float>(ws, L.y);
    GemmArgs q{};
    q.a_bf16 = at<const uint16_t>(ws, L.h);
    q.lda = I;
    q.w_packed = w2->packed;
    q.w_scales = w2->scales;
    q.w_global = w2->global;
    q.w_pow2 = (w2->flags & NVFP4_POW2_SCALES) != 0;
    q.w_tiled = (w2->flags & NVFP4_TILED_SCALES) != 0;
    q.K = I;
    q.N = H;
    q.M = T * k;
    q.topk = k;
    q.experts = E;
    q.out = y;
    q.ksplit = ksplit;
    q.partial = y;
    s = dispatch_grouped<kModeDown>(q, offsets, T * k, E, 1, at<int32_t>(ws, L.r.plan_dn), small, st);
    if (s != NVFP4_OK)
        return s;
    // 4. combine (adds the planes of y in order)
    launch_combine(y, inv, w, T, k, H, ksplit, T * k * H, out, st);
    return launch_status();
}

size_t nvfp4_noalloc_scratch_bytes(void) { return kScratchBytes; }

nvfp4_status nvfp4_moe_grouped_gemm_noalloc(const void* x, const int32_t* ids, const float* w, int64_t T,
                                            int32_t k, int32_t E, const nvfp4_tensor* w13,
                                            const nvfp4_tensor* w2, const float* static_in_globals,
                                            void* out, void* stream)
{
    int64_t H = 0, I = 0;
    nvfp4_status s = check_experts(w13, w2, E, &H, &I);
    if (s != NVFP4_OK)
        return s;
    if (T < 0 || k < 1 || E < 1 || E > kMaxExperts || T * k > 0x7FFFFFFF)
        return NVFP4_ERR_SHAPE;
    if (H % 16 != 0 || I % 16 != 0 || H == 0 || I == 0)
        return NVFP4_ERR_SHAPE;
    if (T == 0)
        return NVFP4_OK;
    // the workspace of this layer must fit the scratch array
    if (moe_layout(T, k, E, H, I).end > kScratchBytes)
        return NVFP4_ERR_WORKSPACE;
    void* ws = scratch_address(&s);
    if (!ws)
        return s;
    s = moe_grouped_gemm_impl(x, ids, w, T, k, E, w13, w2, static_in_globals, out, ws, kScratchBytes, stream);
    if (s == NVFP4_OK && checks_on()) {
        check_bf16(x, T, H, H, S(stream));
        if (static_in_globals)
            check_globals(static_in_globals, 2, S(stream));
        s = check_tensors_data({w13, w2}, S(stream));
    }
    return s;
}

nvfp4_status nvfp4_moe_w4a16(const void* x, const int32_t* ids, const float* w, int64_t T, int32_t k,
                             int32_t E, const nvfp4_tensor* w13, const nvfp4_tensor* w2, void* out, void* ws,
                             size_t ws_bytes, void* stream)
{
    nvfp4_status s = moe_w4a16_unchecked(x, ids, w, T, k, E, w13, w2, out, ws, ws_bytes, stream);
    if (s == NVFP4_OK && checks_on() && T > 0) {
        check_bf16(x, T, w13->cols, w13->cols, S(stream));
        s = check_tensors_data({w13, w2}, S(stream));
    }
    return s;
}

nvfp4_status nvfp4_kv_quant(const void* k, const void* v, int64_t n, int64_t heads, int64_t tok_offset,
                            const nvfp4_tensor* k_cache, const nvfp4_tensor* v_cache, void* stream)
{
    const void* src[2] = {k, v};
    const nvfp4_tensor* dst[2] = {k_cache, v_cache};
    QuantArgs a{};
    int nt = 0;
    int64_t D = -1;
    if (n < 0 || heads < 1 || tok_offset < 0)
        return NVFP4_ERR_SHAPE;
    for (int j = 0; j < 2; j++) {
        if (!src[j])
            continue;
        nvfp4_status s = check_tensor(dst[j]);
        if (s != NVFP4_OK)
            return s;
        if (!aligned(src[j], 16))
            return NVFP4_ERR_INVALID_ARG;
        if (dst[j]->batch != 1 || dst[j]->rows % heads != 0 || (D >= 0 && dst[j]->cols != D))
            return NVFP4_ERR_SHAPE;
        D = dst[j]->cols;
        if (D % 16 != 0 || (tok_offset + n) * heads > dst[j]->rows)
            return NVFP4_ERR_SHAPE;
        a.x[nt] = (const u32x4*)src[j];
        a.packed[nt] = (u32x2*)dst[j]->packed;
        a.scales[nt] = dst[j]->scales;
        a.global_out[nt] = nullptr;
        a.gsrc[nt] = dst[j]->global;
        a.src[nt] = kGlobalStatic;
        a.row_off[nt] = tok_offset * heads;
        nt++;
    }
    if (nt == 0 || n == 0)
        return NVFP4_OK;
    a.rows = n * heads;
    a.blocks_per_row = D / 16;
    a.ld_chunks = D / 8;
    return launch_quantize(a, nt, S(stream));
}

static nvfp4_status kv_dequant_unchecked(const nvfp4_tensor* k_cache, const nvfp4_tensor* v_cache, int64_t heads,
                              int64_t tok_begin, int64_t n, void* k_out, void* v_out, int32_t dtype,
                              void* stream)
{
    const nvfp4_tensor* src[2] = {k_cache, v_cache};
    void* dst[2] = {k_out, v_out};
    if (n < 0 || heads < 1 || tok_begin < 0)
        return NVFP4_ERR_SHAPE;
    if (dtype != NVFP4_F32 && dtype != NVFP4_BF16)
        return NVFP4_ERR_INVALID_ARG;
    for (int j = 0; j < 2; j++) {
        if (!dst[j])
            continue;
        nvfp4_status s = check_tensor(src[j]);
        if (s != NVFP4_OK)
            return s;
        if (!aligned(dst[j], 16))
            return NVFP4_ERR_INVALID_ARG;
        if (src[j]->batch != 1 || src[j]->rows % heads != 0 || (tok_begin + n) * heads > src[j]->rows)
            return NVFP4_ERR_SHAPE;
    }
    for (int j = 0; j < 2; j++) {
        if (!dst[j] || n == 0)
            continue;
        const int64_t bpr = src[j]->cols / 16;
        const int64_t nblk = n * heads * bpr;
        const unsigned grid = stream_grid(ceil_div(2 * nblk, 8), 8192);
        if (dtype == NVFP4_BF16)
            dequantize_kernel<true><<<grid, kQuantThreads, 0, S(stream)>>>(
                (const uint32_t*)src[j]->packed, src[j]->scales, src[j]->global, nblk, src[j]->rows * bpr,
                tok_begin * heads * bpr, dst[j]);
        else
            dequantize_kernel<false><<<grid, kQuantThreads, 0, S(stream)>>>(
                (const uint32_t*)src[j]->packed, src[j]->scales, src[j]->global, nblk, src[j]->rows * bpr,
                tok_begin * heads * bpr, dst[j]);
        nvfp4_status s = launch_status();
        if (s != NVFP4_OK)
            return s;
    }
    return NVFP4_OK;
}

nvfp4_status nvfp4_kv_dequant(const nvfp4_tensor* k_cache, const nvfp4_tensor* v_cache, int64_t heads,
                              int64_t tok_begin, int64_t n, void* k_out, void* v_out, int32_t dtype,
                              void* stream)
{
    nvfp4_status s = kv_dequant_unchecked(k_cache, v_cache, heads, tok_begin, n, k_out, v_out, dtype, stream);
    if (s == NVFP4_OK && checks_on())
        s = check_tensors_data({k_out ? k_cache : nullptr, v_out ? v_cache : nullptr}, S(stream));
    return s;
}

nvfp4_status nvfp4_audit_scales(const nvfp4_tensor* t, int64_t* counts, void* stream)
{
    nvfp4_status s = check_tensor(t, false, true);
    if (s != NVFP4_OK)
        return s;
    if (!counts || !aligned(counts, 8))
        return NVFP4_ERR_INVALID_ARG;
    const int64_t n = t->batch * t->rows * (t->cols / 16);
    zero_u64_kernel<<<1, 64, 0, S(stream)>>>((unsigned long long*)counts, 4);
    if (n > 0)
        audit_kernel<<<stream_grid(n, 1024), kQuantThreads, 0, S(stream)>>>(t->scales, n,
                                                                             (unsigned long long*)counts);
    return launch_status();
}

}  // extern "C"
