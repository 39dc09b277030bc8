// mx.h -- MXFP4 encode and the lossless MXFP4 -> NVFP4 remap (page
// "DeepSeek-V4.1-Flash-NVFP4": section 二, MXFP4 = 32-element blocks with a
// power-of-two UE8M0 scale, NVFP4 = 16-element blocks with E4M3 scales;
// sections 一/四/六: every MXFP4 weight block remaps to NVFP4 without loss).
//
// The remap is integer work: the E2M1 codes are kept, each UE8M0 exponent e
// becomes the E4M3 power of two 2^(e - e_max + 8) and the tensor global
// becomes 2^(e_max - 8).  Two passes per matrix: (1) read codes + exponent
// bytes, copy the codes, record which 32-blocks hold a non-zero code and
// reduce max/min exponent over them; (2) write the scale bytes.
#pragma once
#include "common.h"

namespace nvfp4 {

constexpr int kMxThreads = 256;
constexpr int kRemapParts = 64;  // partial reductions per matrix
constexpr int kNoExp = -100000;  // "no non-zero block" marker

// ---- MXFP4 encode: one thread per 32-element block ----------------------
__global__ void __launch_bounds__(kMxThreads)
mxfp4_encode_kernel(const u32x4* __restrict__ x, int64_t rows, int64_t blocks_per_row,
                    int64_t ld_chunks, u32x4* __restrict__ packed, uint8_t* __restrict__ e8m0)
{
    const int64_t nblk = rows * blocks_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
        const int64_t r = b / blocks_per_row;
        const u32x4* src = x + r * ld_chunks + 4 * (b - r * blocks_per_row);
        u32x4 v[4];
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[i] = __builtin_nontemporal_load(src + i);
            uint32_t a = absmax_bits8(v[i]);
            am = am > a ? am : a;
        }
        const float amax = __uint_as_float(am << 16);
        int e = 0;
        float scale = 0.0f;  // an all-zero block: codes +-0, scale byte 0
        uint32_t byte = 0;
        if (amax > 0.0f) {
            // amax = f * 2^p with f in [0.5, 1): floor(log2 amax) = p - 1;
            // the shared exponent is that minus 2 (the exponent of 6.0)
            e = __builtin_amdgcn_frexp_expf(amax) - 3;
            e = e < -127 ? -127 : (e > 127 ? 127 : e);
            byte = (uint32_t)(e + 127);
            scale = 1.0f;
        }
        u32x4 out;
        uint32_t* o = (uint32_t*)&out;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            uint32_t c = 0;
            // |x| / 2^e is exact wherever it can reach a code boundary
            c = FP4_PACK2(c, __builtin_ldexpf(bf16_lo(w[0]), -e) * scale, __builtin_ldexpf(bf16_hi(w[0]), -e) * scale, 0);
            c = FP4_PACK2(c, __builtin_ldexpf(bf16_lo(w[1]), -e) * scale, __builtin_ldexpf(bf16_hi(w[1]), -e) * scale, 1);
            c = FP4_PACK2(c, __builtin_ldexpf(bf16_lo(w[2]), -e) * scale, __builtin_ldexpf(bf16_hi(w[2]), -e) * scale, 2);
            c = FP4_PACK2(c, __builtin_ldexpf(bf16_lo(w[3]), -e) * scale, __builtin_ldexpf(bf16_hi(w[3]), -e) * scale, 3);
            o[i] = c;
        }
        packed[b] = out;
        e8m0[b] = (uint8_t)byte;
    }
}

// ---- remap pass 1: copy codes, flag non-zero blocks, exponent window ------
// grid = (kRemapParts, batch).  mats: blocks32_per_mat 32-blocks each.
__global__ void __launch_bounds__(kMxThreads)
remap_scan_kernel(const u32x4* __restrict__ mx, const uint8_t* __restrict__ e8m0,
                  int64_t blocks_per_mat, u32x4* __restrict__ out_packed,
                  uint8_t* __restrict__ nz_flags, int* __restrict__ part_max,
                  int* __restrict__ part_min)
{
    __shared__ int smax[16], smin[16];
    const int64_t mat = blockIdx.y;
    const u32x4* src = mx + mat * blocks_per_mat;
    const uint8_t* ex = e8m0 + mat * blocks_per_mat;
    u32x4* dst = out_packed ? out_packed + mat * blocks_per_mat : nullptr;
    uint8_t* flags = nz_flags + mat * blocks_per_mat;
    int emax = kNoExp, emin = -kNoExp;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < blocks_per_mat; b += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + b);
        if (dst)
            __builtin_nontemporal_store(v, dst + b);
        const bool nz = ((v.x | v.y | v.z | v.w) & 0x77777777u) != 0;
        flags[b] = nz;
        if (nz) {
            const int e = (int)ex[b] - 127;
            if (e == 128) {
                raise_error(NVFP4_ERR_RANGE);  // NaN scale byte on a non-zero block
            } else {
                emax = emax > e ? emax : e;
                emin = emin < e ? emin : e;
            }
        }
    }
    emax = wave_max_i32(emax);
    emin = wave_min_i32(emin);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) {
        smax[wid] = emax;
        smin[wid] = emin;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < (int)(blockDim.x >> 6); i++) {
            emax = emax > smax[i] ? emax : smax[i];
            emin = emin < smin[i] ? emin : smin[i];
        }
        emax = emax > smax[0] ? emax : smax[0];
        emin = emin < smin[0] ? emin : smin[0];
        part_max[mat * gridDim.x + blockIdx.x] = emax;
        part_min[mat * gridDim.x + blockIdx.x] = emin;
    }
}

// ---- remap pass 2: scale bytes and the global -----------------------------
__global__ void __launch_bounds__(kMxThreads)
remap_scales_kernel(const uint8_t* __restrict__ e8m0, const uint8_t* __restrict__ nz_flags,
                    int64_t blocks_per_mat, const int* __restrict__ part_max,
                    const int* __restrict__ part_min, int nparts,
                    uint16_t* __restrict__ scales, float* __restrict__ globals)
{
    const int64_t mat = blockIdx.y;
    int emax = kNoExp, emin = -kNoExp;
    for (int i = 0; i < nparts; i++) {
        const int a = part_max[mat * nparts + i], b = part_min[mat * nparts + i];
        emax = emax > a ? emax : a;
        emin = emin < b ? emin : b;
    }
    const bool any = emax != kNoExp;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        globals[mat] = any ? __builtin_ldexpf(1.0f, emax - 8) : 1.0f;
        if (any && emax - emin > 17)
            raise_error(NVFP4_ERR_RANGE);
    }
    const uint8_t* ex = e8m0 + mat * blocks_per_mat;
    const uint8_t* flags = nz_flags + mat * blocks_per_mat;
    uint16_t* sc = scales + mat * blocks_per_mat;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < blocks_per_mat; b += stride) {
        uint32_t code = 0x01;  // zero block
        if (flags[b]) {
            const int d = ((int)ex[b] - 127) - emax + 8;  // in [-9, 8] when in range
            if (ex[b] == 255 || d < -9)
                code = 0;      // cannot be represented: scale 0, error raised above
            else if (d < -6)
                code = 1u << (d + 9);           // subnormal E4M3 powers of two
            else
                code = (uint32_t)(d + 7) << 3;  // normal E4M3 2^d
        }
        sc[b] = (uint16_t)(code | (code << 8));
    }
}

}  // namespace nvfp4
