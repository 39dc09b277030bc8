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

// E4M3 byte for the block with E8M0 byte `eb` (2^(eb-127)) relative to the
// window top emax: 2^((eb-127) - emax + 8), or 0x01 for an all-zero block
// (flag 0), or 0 for a scale out of range (the error is raised elsewhere).
NVFP4_DEV uint32_t remap_scale_code(uint32_t eb, uint32_t flag, int emax)
{
    if (!flag)
        return 0x01;
    const int d = ((int)eb - 127) - emax + 8;  // in [-9, 8] when in range
    if (eb == 255 || d < -9)
        return 0;
    if (d < -6)
        return 1u << (d + 9);           // subnormal E4M3 powers of two
    return (uint32_t)(d + 7) << 3;      // normal E4M3 2^d
}

// ---- remap pass 2: scale bytes and the global -----------------------------
__global__ void __launch_bounds__(kMxThreads)
remap_scales_kernel(const uint8_t* __restrict__ e8m0, const uint8_t* __restrict__ nz_flags,
                    int64_t blocks_per_mat, const int* __restrict__ part_max,
                    const int* __restrict__ part_min, int nparts,
                    uint16_t* __restrict__ scales, float* __restrict__ globals, int vec16)
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
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (vec16) {
        // 16 blocks per thread: 16 exponent bytes and 16 flags in, 32 scale bytes out
        const int64_t groups = blocks_per_mat >> 4;
        for (int64_t gi = first; gi < groups; gi += stride) {
            const int64_t b = gi << 4;
            const u32x4 ew = *(const u32x4*)(ex + b);
            const u32x4 fw = *(const u32x4*)(flags + b);
            uint32_t o[8];
#pragma unroll
            for (int w = 0; w < 4; w++) {
                const uint32_t e4 = w == 0 ? ew.x : w == 1 ? ew.y : w == 2 ? ew.z : ew.w;
                const uint32_t f4 = w == 0 ? fw.x : w == 1 ? fw.y : w == 2 ? fw.z : fw.w;
                uint32_t c[4];
#pragma unroll
                for (int j = 0; j < 4; j++)
                    c[j] = remap_scale_code((e4 >> (8 * j)) & 0xFF, (f4 >> (8 * j)) & 0xFF, emax);
                o[2 * w] = (c[0] | (c[0] << 8)) | ((c[1] | (c[1] << 8)) << 16);
                o[2 * w + 1] = (c[2] | (c[2] << 8)) | ((c[3] | (c[3] << 8)) << 16);
            }
            u32x4* d = (u32x4*)(sc + b);
            d[0] = (u32x4){o[0], o[1], o[2], o[3]};
            d[1] = (u32x4){o[4], o[5], o[6], o[7]};
        }
        return;
    }
    for (int64_t b = first; b < blocks_per_mat; b += stride) {
        const uint32_t code = remap_scale_code(ex[b], flags[b], emax);
        sc[b] = (uint16_t)(code | (code << 8));
    }
}

}  // namespace nvfp4
