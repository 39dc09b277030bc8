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
// x is viewed as rows x (cols/8) chunks of 16 bytes.
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
            uint32_t a = absmax_bits8(__builtin_nontemporal_load(x + i));
            m = m > a ? m : a;
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
            int64_t r = i / chunks_per_row, c = i - r * chunks_per_row;
            uint32_t a = absmax_bits8(x[r * ld_chunks + c]);
            m = m > a ? m : a;
        }
    }
    m = block_max_u32(m, red);
    if (threadIdx.x == 0)
        partials[blockIdx.x] = m << 16;  // bf16 magnitude bits -> float bits
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

// Encode one 16-element block held as two u32x4 of bf16 bits.
// Returns the two code dwords; *scale_out gets the E4M3 byte.
NVFP4_DEV u32x2 encode_block(u32x4 lo, u32x4 hi, float G, float six_g, uint32_t* scale_out)
{
    uint32_t am = absmax_bits8(lo);
    uint32_t am2 = absmax_bits8(hi);
    am = am > am2 ? am : am2;
    const float ab = __uint_as_float(am << 16);
    const float s_real = ab / six_g;
    const uint32_t sc = e4m3_encode(s_real);
    *scale_out = sc;
    const float s = e4m3_decode(sc);
    float r = 0.0f;                       // scale 0: every code becomes +-0
    if (sc != 0) {
        const float p = s * G;
        r = 1.0f / p;
    }
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    float y[16];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        y[2 * i] = bf16_lo(w[i]) * r;
        y[2 * i + 1] = bf16_hi(w[i]) * r;
    }
    if (__builtin_isinf(r)) {
        // s * G underflowed: x * inf is +-inf (code 6) except 0 * inf, which
        // is taken as a zero code with the sign of x.
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
            y[2 * i] = a == 0.0f ? a : y[2 * i];
            y[2 * i + 1] = b == 0.0f ? b : y[2 * i + 1];
        }
    }
    uint32_t c0 = 0, c1 = 0;
    c0 = FP4_PACK2(c0, y[0], y[1], 0);
    c0 = FP4_PACK2(c0, y[2], y[3], 1);
    c0 = FP4_PACK2(c0, y[4], y[5], 2);
    c0 = FP4_PACK2(c0, y[6], y[7], 3);
    c1 = FP4_PACK2(c1, y[8], y[9], 0);
    c1 = FP4_PACK2(c1, y[10], y[11], 1);
    c1 = FP4_PACK2(c1, y[12], y[13], 2);
    c1 = FP4_PACK2(c1, y[14], y[15], 3);
    return (u32x2){c0, c1};
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

__global__ void __launch_bounds__(kQuantThreads)
quantize_kernel(QuantArgs a)
{
    __shared__ uint32_t red[16];
    const int j = blockIdx.y;
    const float G = load_global(a.src[j], a.gsrc[j], a.nparts, red);
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.global_out[j])
        *a.global_out[j] = G;
    const float six_g = 6.0f * G;
    const int64_t nblk = a.rows * a.blocks_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const u32x4* __restrict__ x = a.x[j];
    u32x2* __restrict__ packed = a.packed[j] + a.row_off[j] * a.blocks_per_row;
    uint8_t* __restrict__ scales = a.scales[j] + a.row_off[j] * a.blocks_per_row;
    const bool flat = a.ld_chunks == 2 * a.blocks_per_row;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
        int64_t src;
        if (flat) {
            src = 2 * b;
        } else {
            int64_t r = b / a.blocks_per_row;
            src = r * a.ld_chunks + 2 * (b - r * a.blocks_per_row);
        }
        const u32x4 lo = __builtin_nontemporal_load(x + src);
        const u32x4 hi = __builtin_nontemporal_load(x + src + 1);
        uint32_t sc;
        const u32x2 codes = encode_block(lo, hi, G, six_g, &sc);
        packed[b] = codes;
        scales[b] = (uint8_t)sc;
    }
}

// ---- dequantize ------------------------------------------------------------
// v = (e2m1 * s) * G in fp32; bf16 output rounds that value to nearest even.
// rows_per_batch selects the global of each row's batch matrix.
template <bool kBf16>
__global__ void __launch_bounds__(kQuantThreads)
dequantize_kernel(const u32x2* __restrict__ packed, const uint8_t* __restrict__ scales,
                  const float* __restrict__ globals, int64_t nblk, int64_t blocks_per_row,
                  int64_t rows_per_batch, int64_t row_off, void* __restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
        const int64_t gb = b + row_off * blocks_per_row;
        const float G = globals[(gb / blocks_per_row) / rows_per_batch];
        const u32x2 c = packed[gb];
        const float s = e4m3_decode(scales[gb]);
        float2_t q[8] = {FP4_TO_F32X2(c.x, 0), FP4_TO_F32X2(c.x, 1), FP4_TO_F32X2(c.x, 2),
                         FP4_TO_F32X2(c.x, 3), FP4_TO_F32X2(c.y, 0), FP4_TO_F32X2(c.y, 1),
                         FP4_TO_F32X2(c.y, 2), FP4_TO_F32X2(c.y, 3)};
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            v[2 * i] = (q[i].x * s) * G;
            v[2 * i + 1] = (q[i].y * s) * G;
        }
        if (kBf16) {
            u32x4* o = (u32x4*)out + 2 * b;
            o[0] = (u32x4){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
            o[1] = (u32x4){pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]),
                              pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15])};
        } else {
            float4_t* o = (float4_t*)out + 4 * b;
#pragma unroll
            for (int i = 0; i < 4; i++)
                o[i] = (float4_t){v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
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

__global__ void zero_u64_kernel(unsigned long long* p, int n)
{
    if ((int)threadIdx.x < n)
        p[threadIdx.x] = 0;
}

}  // namespace nvfp4
