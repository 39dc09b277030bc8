// common.h -- device helpers shared by the libnvfp4 kernels (gfx950 only).
//
// Format facts used here: E2M1 codes (page "DeepSeek-V4.1-Flash-NVFP4",
// section 二), E4M3 block scales with maximum 448 (page
// "Qwen3.8-Flash-Next-NVFP4", sections 核心 and 证据链).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define NVFP4_DEV __device__ __forceinline__

// Sticky data-dependent error word of this device (0 = none).  Kernels raise
// an error with atomicCAS so the first one wins.
__device__ unsigned int g_nvfp4_error;

// Load from a table that no kernel in flight writes (produced by an earlier
// launch, or an input): through the constant address space, so that a
// uniform index becomes a scalar load, counted apart from the vector loads
// in flight.
template <class T>
NVFP4_DEV T const_load(const T* ptr, int64_t i)
{
    typedef const __attribute__((address_space(4))) T* cptr;
    return ((cptr)(uintptr_t)ptr)[i];
}

NVFP4_DEV void raise_error(unsigned code)
{
    atomicCAS(&g_nvfp4_error, 0u, code);
}

// ---------------------------------------------------------------- bf16 ----

NVFP4_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
NVFP4_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Nearest-even bf16 of an fp32 (the gfx950 conversion rounds to nearest even).
NVFP4_DEV uint16_t f32_to_bf16(float f)
{
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

NVFP4_DEV uint32_t pack_bf16x2(float lo, float hi)
{
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// max over the 8 bf16 magnitudes (bit patterns, sign cleared) in 16 bytes.
// Non-negative finite floats order like their bit patterns.
NVFP4_DEV uint32_t absmax_bits8(u32x4 v)
{
    ushort2_t a = __builtin_bit_cast(ushort2_t, v.x & 0x7FFF7FFFu);
    ushort2_t b = __builtin_bit_cast(ushort2_t, v.y & 0x7FFF7FFFu);
    ushort2_t c = __builtin_bit_cast(ushort2_t, v.z & 0x7FFF7FFFu);
    ushort2_t d = __builtin_bit_cast(ushort2_t, v.w & 0x7FFF7FFFu);
    ushort2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                            __builtin_elementwise_max(c, d));
    return m.x > m.y ? m.x : m.y;
}

// ---------------------------------------------------------------- E4M3 ----

// Nearest-even E4M3 code (0x00..0x7E) of s >= 0; s >= 448 (and +inf)
// saturates to 0x7E.
NVFP4_DEV uint32_t e4m3_encode(float s)
{
    if (!(s < 448.0f))
        return 0x7Eu;
    if (s < 0.015625f) {
        // subnormal range: value m * 2^-9, m = round-half-even(s * 2^9);
        // the product is exact and m = 8 is the code of 2^-6.
        return (uint32_t)__builtin_rintf(s * 512.0f);
    }
    uint32_t u = __float_as_uint(s);
    uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);  // round mantissa to 3 bits, ties even
    return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
}

// fp32 value of an E4M3 code in 0x00..0x7E.
NVFP4_DEV float e4m3_decode(uint32_t c)
{
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 0)
        return (float)m * 0.001953125f;  // m * 2^-9, exact
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// -------------------------------------------------------------- E2M1 ------

// Two fp32 values -> byte `sel` of `old`: low nibble from a, high nibble
// from b, nearest-even on the E2M1 grid, saturating at +-6, sign kept (also
// for zero).  The hardware conversion with unit scale was checked against
// that rule over every non-NaN fp32 input.
#define FP4_PACK2(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// byte `sel` of `src` (two E2M1 codes) -> two f16 values (exact, sign kept).
#define FP4_TO_F16X2(src, sel) __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((src), 1.0f, (sel))
// byte `sel` of `src` (two E2M1 codes) -> two f32 values (exact).
#define FP4_TO_F32X2(src, sel) __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((src), 1.0f, (sel))

// Scale of one 16-element block from its bf16 magnitude bits `am` (the
// block amax): *sc gets the E4M3 byte, the return value is the reciprocal
// r = 1 / (s * G) the codes are taken with (0 when s = 0).
NVFP4_DEV float block_scale(uint32_t am, float G, float six_g, uint32_t* sc)
{
    const float ab = __uint_as_float(am << 16);
    const float s_real = ab / six_g;
    *sc = e4m3_encode(s_real);
    const float s = e4m3_decode(*sc);
    float r = 0.0f;                       // scale 0: every code becomes +-0
    if (*sc != 0) {
        const float p = s * G;
        r = 1.0f / p;
    }
    return r;
}

// Eight bf16 values (one u32x4) times r -> eight E2M1 codes (one dword,
// element 2j in the low nibble of byte j).
NVFP4_DEV uint32_t encode_half(u32x4 v, float r)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float y[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        y[2 * i] = bf16_lo(w[i]) * r;
        y[2 * i + 1] = bf16_hi(w[i]) * r;
    }
    if (__builtin_isinf(r)) {
        // s * G underflowed: x * inf is +-inf (code 6) except 0 * inf, which
        // is taken as a zero code with the sign of x.
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
            y[2 * i] = a == 0.0f ? a : y[2 * i];
            y[2 * i + 1] = b == 0.0f ? b : y[2 * i + 1];
        }
    }
    uint32_t c = 0;
    c = FP4_PACK2(c, y[0], y[1], 0);
    c = FP4_PACK2(c, y[2], y[3], 1);
    c = FP4_PACK2(c, y[4], y[5], 2);
    c = FP4_PACK2(c, y[6], y[7], 3);
    return c;
}

// The value of lane (l ^ M) for lane l, within each group of 32 lanes
// (ds_swizzle bit mode: the pattern is an immediate, no lane address).
template <int M>
NVFP4_DEV uint32_t swz_xor(uint32_t v)
{
    static_assert(M > 0 && M < 32, "xor within 32 lanes");
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));
}
NVFP4_DEV uint32_t umax_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// One NVFP4 block held by 16 consecutive lanes (lane 16 q + p holds
// element p, as bf16 bits in the low half of hb), encoded as nvfp4_quantize
// encodes it: the block max over the 16 lanes, block_scale, codes of x * r
// (with the same zero rule for an infinite r).  Every lane gets the scale
// byte; lanes with p = 0 and p = 8 get the dword of codes of elements
// [0, 8) and [8, 16).  All 64 lanes must execute it.
NVFP4_DEV void encode_block16(uint32_t hb, float G, float six_g, uint32_t* sc, uint32_t* codes)
{
    uint32_t am = hb & 0x7FFFu;
    am = umax_u32(am, swz_xor<1>(am));
    am = umax_u32(am, swz_xor<2>(am));
    am = umax_u32(am, swz_xor<4>(am));
    am = umax_u32(am, swz_xor<8>(am));
    const float r = block_scale(am, G, six_g, sc);
    const float x = __uint_as_float(hb << 16);
    float y = x * r;
    if (__builtin_isinf(r) && x == 0.0f)
        y = x;
    const float yo = __uint_as_float(swz_xor<1>(__float_as_uint(y)));
    const int p = threadIdx.x & 15;
    // even lanes: elements p (low nibble) and p + 1 of byte p / 2
    const uint32_t b = FP4_PACK2(0u, y, yo, 0) & 0xFFu;
    uint32_t w = b << (8 * ((p >> 1) & 3));
    w |= swz_xor<2>(w);
    w |= swz_xor<4>(w);
    *codes = w;
}

// ------------------------------------------------------------ reductions --

NVFP4_DEV uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = __shfl_xor(v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

NVFP4_DEV int wave_max_i32(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        int o = __shfl_xor(v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

NVFP4_DEV int wave_min_i32(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        int o = __shfl_xor(v, off, 64);
        v = v < o ? v : o;
    }
    return v;
}

// Block-wide max of a uint32 (blockDim.x a multiple of 64, <= 1024);
// result valid in every thread.
NVFP4_DEV uint32_t block_max_u32(uint32_t v, uint32_t* lds16)
{
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0)
        lds16[wid] = v;
    __syncthreads();
    const int nw = blockDim.x >> 6;
    uint32_t r = 0;
    for (int i = 0; i < nw; i++)
        r = r > lds16[i] ? r : lds16[i];
    return r;
}

// G from a tensor maximum: amax / (6 * 448), or 1 for an all-zero tensor.
NVFP4_DEV float global_from_amax(float amax)
{
    return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
