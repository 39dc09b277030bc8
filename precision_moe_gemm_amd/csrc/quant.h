// quant.h -- NVFP4 quantize / dequantize, KV-cache write/read and the scale
// audit (page "Qwen3.8-Flash-Next-NVFP4", section 核心: level-1 E4M3 scale per
// 16 elements along the last dimension, level-2 FP32 tensor scale, dynamic
// activations; section 证据链: scale audit; page "Qwen3.8-2.4T-A95B-NVFP4":
// NVFP4 KV cache).
//
// All of these are HBM-bound streaming kernels.  One thread owns one
// 16-element block: two 16-byte loads of bf16 (a wave reads 2 KiB
// contiguous), one 8-byte store of codes and one scale byte.
#pragma once
#include "common.h"

namespace nvfp4 {

constexpr int kQuantThreads = 256;
constexpr int kAmaxParts = 1024;  // partial maxima of the dynamic-global pass

// Where a quantize launch takes its global scale from.
enum GlobalSource : int {
    kGlobalStatic = 0,   // gsrc points at a device float
    kGlobalPartials = 1, // gsrc points at `nparts` partial maxima (float bits)
    kGlobalAmaxWord = 2  // gsrc points at one uint32 max |x| (float bits)
};

// ---- pass 1 of a dynamic global: partial max |x| per workgroup ----------
// x is viewed as rows x (cols/8) chunks of 16 bytes.  The pass walks the
// tensor from its end to its start with ordinary (cached) loads, so that
// when the encode pass then walks it from the start, its first part (up to
// the size of the last-level cache) is still cached.
__global__ void __launch_bounds__(kQuantThreads)
amax_partials_kernel(const u32x4* __restrict__ x, int64_t rows, int64_t chunks_per_row,
                     int64_t ld_chunks, uint32_t* __restrict__ partials)
{
    __shared__ uint32_t red[16];
    const int64_t total = rows * chunks_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t m = 0;
    if (ld_chunks == chunks_per_row) {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
            uint32_t a = absmax_bits8(x[total - 1 - i]);
            m = m > a ? m : a;
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
            const int64_t ir = total - 1 - i;
            int64_t r = ir / chunks_per_row, c = ir - r * chunks_per_row;
            uint32_t a = absmax_bits8(x[r * ld_chunks + c]);
            m = m > a ? m : a;
        }
    }
    m = block_max_u32(m, red);
    if (threadIdx.x == 0)
        partials[blockIdx.x] = m << 16;  // bf16 magnitude bits -> float bits
}

// Dynamic-global quantize of a whole small tensor (at most kQuantSmall
// elements, nhalf = elements / 8 half-blocks) by one workgroup of 1024
// threads: thread t holds half-blocks t + 1024 u in v[u] (any value past the
// end) and m_local, the largest magnitude bits among its valid ones.  The
// workgroup max gives the global (written to gout), and every half-block is
// encoded as quantize_kernel encodes it: lanes 2j and 2j + 1 hold the two
// halves of one block.
constexpr int kQuantSmall = 65536;
constexpr int kQsU = kQuantSmall / 8 / 1024;  // half-blocks per thread

NVFP4_DEV void encode_small_block(const u32x4 (&v)[kQsU], uint32_t m_local, int64_t nhalf,
                                  uint32_t* __restrict__ packed, uint8_t* __restrict__ scales, float* gout,
                                  uint32_t* red)
{
    const uint32_t m = block_max_u32(m_local, red);
    const float G = global_from_amax(__uint_as_float(m << 16));
    if (threadIdx.x == 0)
        *gout = G;
    const float six_g = 6.0f * G;
#pragma unroll
    for (int u = 0; u < kQsU; u++) {
        const int64_t h = (int64_t)u * 1024 + threadIdx.x;
        uint32_t am = absmax_bits8(v[u]);
        const uint32_t other = (uint32_t)__shfl_xor((int)am, 1, 64);
        am = am > other ? am : other;
        uint32_t sc;
        const float r = block_scale(am, G, six_g, &sc);
        const uint32_t code = encode_half(v[u], r);
        if (h < nhalf) {
            packed[h] = code;
            if ((h & 1) == 0)
                scales[h >> 1] = (uint8_t)sc;
        }
    }
}

// The routing of a small batch (block 0, one workgroup: route_small_block)
// and the first pass of the activations' dynamic global (blocks 1..P: the
// partial max |x| of a P-way split, as amax_partials_kernel) are
// independent, so one launch of 1 + P workgroups serves both.  With xq_packed
// non-null (then P = 1 and rows * chunks_per_row <= kQuantSmall / 8), block 1
// quantizes all of x itself: codes to xq_packed, scale bytes to xq_scales,
// the global to xq_gout.
__global__ void __launch_bounds__(1024)
route_small_amax_kernel(const int32_t* __restrict__ ids, int npairs, int E, int32_t* __restrict__ offsets,
                        int32_t* __restrict__ perm, int32_t* __restrict__ inv, uint32_t* zero_word,
                        int32_t* plan_gu, int small_bm_gu, int all_small_gu, int32_t* plan_dn, int small_bm_dn,
                        int all_small_dn, const u32x4* __restrict__ x, int64_t rows, int64_t chunks_per_row,
                        int64_t ld_chunks, uint32_t* __restrict__ partials, uint32_t* __restrict__ xq_packed,
                        uint8_t* __restrict__ xq_scales, float* xq_gout)
{
    if (blockIdx.x == 0) {
        route_small_block(ids, npairs, E, offsets, perm, inv, zero_word, plan_gu, small_bm_gu, all_small_gu,
                          plan_dn, small_bm_dn, all_small_dn);
        return;
    }
    __shared__ uint32_t red[16];
    if (xq_packed) {
        const int64_t nhalf = rows * chunks_per_row;
        u32x4 v[kQsU];
        uint32_t m = 0;
#pragma unroll
        for (int u = 0; u < kQsU; u++) {
            const int64_t h = (int64_t)u * 1024 + threadIdx.x;
            v[u] = (u32x4){0, 0, 0, 0};
            if (h < nhalf) {
                const int64_t r = h / chunks_per_row, c = h - r * chunks_per_row;
                v[u] = x[r * ld_chunks + c];
                const uint32_t a = absmax_bits8(v[u]);
                m = m > a ? m : a;
            }
        }
        encode_small_block(v, m, nhalf, xq_packed, xq_scales, xq_gout, red);
        return;
    }
    const int64_t total = rows * chunks_per_row;
    const int64_t stride = (int64_t)(gridDim.x - 1) * blockDim.x;
    uint32_t m = 0;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / chunks_per_row, c = i - r * chunks_per_row;
        const uint32_t a = absmax_bits8(x[r * ld_chunks + c]);
        m = m > a ? m : a;
    }
    m = block_max_u32(m, red);
    if (threadIdx.x == 0)
        partials[blockIdx.x - 1] = m << 16;  // bf16 magnitude bits -> float bits
}

// Global scale of a quantize launch (identical in every thread).
NVFP4_DEV float load_global(int src, const void* gsrc, int nparts, uint32_t* lds16)
{
    if (src == kGlobalStatic)
        return *(const float*)gsrc;
    uint32_t m = 0;
    if (src == kGlobalPartials) {
        const uint32_t* p = (const uint32_t*)gsrc;
        for (int i = threadIdx.x; i < nparts; i += blockDim.x)
            m = m > p[i] ? m : p[i];
        m = block_max_u32(m, lds16);
    } else {
        m = *(const uint32_t*)gsrc;
    }
    return global_from_amax(__uint_as_float(m));
}

// ---- pass 2: block quantize ---------------------------------------------
// Up to two independent tensors per launch (blockIdx.y), used by the KV
// cache to write K and V together.  Rows of tensor j start at output row
// row_off[j].  blocks_per_row = cols / 16.
struct QuantArgs {
    const u32x4* x[2];
    u32x2* packed[2];       // [rows_out, cols/2] as u32x2 (16 codes)
    uint8_t* scales[2];     // [rows_out, cols/16]
    float* global_out[2];   // may be null
    const void* gsrc[2];
    int src[2];
    int64_t row_off[2];
    int64_t rows, blocks_per_row, ld_chunks;  // ld in 16-byte chunks
    int nparts;
};

template <int kQU>
__global__ void __launch_bounds__(kQuantThreads)
quantize_kernel(QuantArgs a)
{
    __shared__ uint32_t red[16];
    const int j = blockIdx.y;
    const int64_t bpr = a.blocks_per_row;
    const int64_t nhalf = 2 * a.rows * bpr;
    const u32x4* __restrict__ x = a.x[j];
    uint32_t* __restrict__ packed = (uint32_t*)(a.packed[j] + a.row_off[j] * bpr);
    uint8_t* __restrict__ scales = a.scales[j] + a.row_off[j] * bpr;
    const bool flat = a.ld_chunks == 2 * bpr;
    // work item = half a block (8 elements, one 16-byte chunk): lanes 2j and
    // 2j+1 hold the two halves of a block and share its max with one lane
    // swap, so loads and code stores are contiguous per instruction.  A
    // workgroup takes kQU * 256 consecutive half-blocks per trip, all loads
    // issued first (kQU = 8; 2 for launches too small to fill the chip, so
    // that four times as many waves share the work).
    constexpr int64_t kChunk = (int64_t)kQU * kQuantThreads;
    u32x4 v[kQU];
    auto load_trip = [&](int64_t base) {
#pragma unroll
        for (int u = 0; u < kQU; u++) {
            int64_t h = base + u * kQuantThreads + threadIdx.x;
            h = h < nhalf ? h : nhalf - 1;
            int64_t src = h;
            if (!flat) {
                const int64_t b = h >> 1, r = b / bpr;
                src = r * a.ld_chunks + 2 * (b - r * bpr) + (h & 1);
            }
            v[u] = __builtin_nontemporal_load(x + src);  // read once
        }
    };
    int64_t base = (int64_t)blockIdx.x * kChunk;
    // the first trip's data is requested before the global scale, so the two
    // memory latencies overlap (this matters for small writes such as a KV chunk)
    if (base < nhalf)
        load_trip(base);
    const float G = load_global(a.src[j], a.gsrc[j], a.nparts, red);
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.global_out[j])
        *a.global_out[j] = G;
    const float six_g = 6.0f * G;
    for (; base < nhalf; base += (int64_t)gridDim.x * kChunk) {
#pragma unroll
        for (int u = 0; u < kQU; u++) {
            const int64_t h = base + u * kQuantThreads + threadIdx.x;
            uint32_t am = absmax_bits8(v[u]);
            const uint32_t other = (uint32_t)__shfl_xor((int)am, 1, 64);
            am = am > other ? am : other;
            uint32_t sc;
            const float r = block_scale(am, G, six_g, &sc);
            const uint32_t code = encode_half(v[u], r);
            if (h < nhalf) {
                packed[h] = code;
                if ((h & 1) == 0)
                    scales[h >> 1] = (uint8_t)sc;
            }
        }
        const int64_t next = base + (int64_t)gridDim.x * kChunk;
        if (next < nhalf)
            load_trip(next);
    }
}

// ---- dequantize ------------------------------------------------------------
// v = (e2m1 * s) * G in fp32; bf16 output rounds that value to nearest even.
// Block gb = b + blk_off belongs to batch matrix gb / blocks_per_batch, whose
// global applies.
template <bool kBf16>
__global__ void __launch_bounds__(kQuantThreads)
dequantize_kernel(const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
                  const float* __restrict__ globals, int64_t nblk, int64_t blocks_per_batch,
                  int64_t blk_off, void* __restrict__ out)
{
    // one matrix (the common case): one global, no per-block division
    const bool single = blk_off + nblk <= blocks_per_batch;
    const float G0 = globals[0];
    // work item = half a block (8 codes, one code dword): lanes 2j and 2j+1
    // take the two halves of a block, so every store instruction writes
    // contiguous output.  A workgroup takes kDqUnroll * 256 consecutive
    // half-blocks per trip, all loads issued first.
    constexpr int kDqUnroll = 8;
    constexpr int64_t kChunk = (int64_t)kDqUnroll * kQuantThreads;
    const int64_t nhalf = 2 * nblk;
    for (int64_t base = (int64_t)blockIdx.x * kChunk; base < nhalf; base += (int64_t)gridDim.x * kChunk) {
        uint32_t c[kDqUnroll], sb[kDqUnroll];
#pragma unroll
        for (int u = 0; u < kDqUnroll; u++) {
            const int64_t hb = base + u * kQuantThreads + threadIdx.x;
            const int64_t gh = (hb < nhalf ? hb : nhalf - 1) + 2 * blk_off;
            c[u] = packed[gh];
            sb[u] = scales[gh >> 1];
        }
#pragma unroll
        for (int u = 0; u < kDqUnroll; u++) {
            const int64_t hb = base + u * kQuantThreads + threadIdx.x;
            if (hb >= nhalf)
                break;
            const float G = single ? G0 : globals[((hb >> 1) + blk_off) / blocks_per_batch];
            const float sc = e4m3_decode(sb[u]);
            const float2_t q[4] = {FP4_TO_F32X2(c[u], 0), FP4_TO_F32X2(c[u], 1), FP4_TO_F32X2(c[u], 2),
                                   FP4_TO_F32X2(c[u], 3)};
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[2 * i] = (q[i].x * sc) * G;
                v[2 * i + 1] = (q[i].y * sc) * G;
            }
            // the output is written once and not read back here: nontemporal
            // stores (measured +4% on the KV read)
            if (kBf16) {
                __builtin_nontemporal_store((u32x4){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
                                            (u32x4*)out + hb);
            } else {
                float4_t* o = (float4_t*)out + 2 * hb;
                __builtin_nontemporal_store((float4_t){v[0], v[1], v[2], v[3]}, o);
                __builtin_nontemporal_store((float4_t){v[4], v[5], v[6], v[7]}, o + 1);
            }
        }
    }
}

// ---- row gather-dequantize (embedding tables) -------------------------------
// out[i] = dequantize(table row ids[i]) for i < n, rows of `hpr` half-blocks
// (cols / 8); the same value rule as dequantize_kernel.  An id outside
// [0, rows) gives a zero output row and raises NVFP4_ERR_RANGE.  Work item
// = one output half-block; four per thread per trip, loads first.  Plain
// stores: on the n-gram shard lookup they measured 4% faster than
// nontemporal ones (the reverse of the contiguous dequantize).
template <bool kBf16>
__global__ void __launch_bounds__(kQuantThreads)
gather_dequant_kernel(const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
                      const float* __restrict__ global, const int32_t* __restrict__ ids, uint32_t n,
                      int64_t rows, uint32_t hpr, void* __restrict__ out)
{
    constexpr int kU = 4;
    const float G = *global;
    const uint32_t nhalf = n * hpr;
    const uint32_t chunk = kU * kQuantThreads;
    for (uint32_t base = blockIdx.x * chunk; base < nhalf; base += gridDim.x * chunk) {
        uint32_t c[kU], sb[kU];
        bool ok[kU];
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const uint32_t hb = base + u * kQuantThreads + threadIdx.x;
            const uint32_t i = (hb < nhalf ? hb : nhalf - 1) / hpr;
            const uint32_t j = (hb < nhalf ? hb : nhalf - 1) - i * hpr;
            const int32_t id = ids[i];
            ok[u] = id >= 0 && id < rows;
            const int64_t src = (int64_t)(ok[u] ? id : 0) * hpr + j;
            c[u] = packed[src];
            sb[u] = scales[src >> 1];
            if (!ok[u] && hb < nhalf && j == 0)
                raise_error(NVFP4_ERR_RANGE);
        }
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const uint32_t hb = base + u * kQuantThreads + threadIdx.x;
            if (hb >= nhalf)
                break;
            const float sc = ok[u] ? e4m3_decode(sb[u]) : 0.0f;
            const float2_t q[4] = {FP4_TO_F32X2(c[u], 0), FP4_TO_F32X2(c[u], 1), FP4_TO_F32X2(c[u], 2),
                                   FP4_TO_F32X2(c[u], 3)};
            float v[8];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                v[2 * t] = ok[u] ? (q[t].x * sc) * G : 0.0f;
                v[2 * t + 1] = ok[u] ? (q[t].y * sc) * G : 0.0f;
            }
            if (kBf16) {
                *((u32x4*)out + hb) = (u32x4){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
            } else {
                float4_t* o = (float4_t*)out + 2 * (int64_t)hb;
                o[0] = (float4_t){v[0], v[1], v[2], v[3]};
                o[1] = (float4_t){v[4], v[5], v[6], v[7]};
            }
        }
    }
}

// ---- scale audit: counts of {all, NaN pattern, zero/negative, 448} ---------
__global__ void __launch_bounds__(kQuantThreads)
audit_kernel(const uint8_t* __restrict__ scales, int64_t n, unsigned long long* __restrict__ counts)
{
    __shared__ unsigned long long c[3];
    if (threadIdx.x < 3)
        c[threadIdx.x] = 0;
    __syncthreads();
    unsigned long long nan = 0, nonpos = 0, mx = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint8_t s = scales[i];
        nan += (s & 0x7F) == 0x7F;
        nonpos += (s == 0) | ((s & 0x80) != 0);
        mx += s == 0x7E;
    }
    atomicAdd(&c[0], nan);
    atomicAdd(&c[1], nonpos);
    atomicAdd(&c[2], mx);
    __syncthreads();
    if (threadIdx.x < 3)
        atomicAdd(&counts[1 + threadIdx.x], c[threadIdx.x]);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        atomicAdd(&counts[0], (unsigned long long)n);
}

// ---- optional data checks// ---- optional data checks (nvfp4_set_checks): raise NVFP4_ERR_DATA ---------
// E4M3 scale bytes: a NaN pattern (0x7F, 0xFF) or a set sign bit.
__global__ void __launch_bounds__(kQuantThreads)
check_scales_kernel(const uint8_t* __restrict__ s, int64_t n)
{
    bool bad = false;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint8_t b = s[i];
        bad |= (b & 0x80) != 0 || (b & 0x7F) == 0x7F;
    }
    if (bad)
        raise_error(NVFP4_ERR_DATA);
}

// fp32 globals: each finite and positive.
__global__ void check_globals_kernel(const float* __restrict__ g, int64_t n)
{
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const float v = g[i];
        if (!(v > 0.0f) || __builtin_isinf(v))
            raise_error(NVFP4_ERR_DATA);
    }
}

// bf16 rows [rows, cols] with row stride ld: every value finite.
__global__ void __launch_bounds__(kQuantThreads)
check_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld)
{
    bool bad = false;
    const int64_t total = rows * cols;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / cols, c = i - r * cols;
        bad |= (x[r * ld + c] & 0x7F80u) == 0x7F80u;
    }
    if (bad)
        raise_error(NVFP4_ERR_DATA);
}

__global__ void zero_u64_kernel(unsigned long long* p, int n)
{
    if ((int)threadIdx.x < n)
        p[threadIdx.x] = 0;
}

// Scale bytes, row-major [batch][rows][chunks * 16] -> the 128-row tiled
// order [batch][rows/128][chunks][128][16] (chunks = K / 256): output run o
// (16 bytes) takes input run (m, 128 t + rr, c) for o = ((m * rows/128 + t) *
// chunks + c) * 128 + rr, so the writes are contiguous.
__global__ void __launch_bounds__(256)
tile_scales_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out, int64_t rows, int64_t chunks, int64_t n)
{
    const int64_t tiles = rows / 128;
    for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < n; o += (int64_t)gridDim.x * 256) {
        const int64_t rr = o & 127, q = o >> 7;
        const int64_t c = q % chunks, mt = q / chunks;
        const int64_t t = mt % tiles, m = mt / tiles;
        out[o] = in[(m * rows + 128 * t + rr) * chunks + c];
    }
}

}  // namespace nvfp4
