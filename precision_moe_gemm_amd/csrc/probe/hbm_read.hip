// Achievable HBM read rate for the access patterns of the weight-streaming
// GEMM, as a measurement aid for the roofline (not part of libnvfp4).
//
// A matrix of `rows` rows of `row_bytes` bytes is read in tiles of R rows by
// a resident grid: each stage of a tile takes L * 16 contiguous bytes of every
// tile row (L lanes of 16 bytes per row, 4 loads per thread per stage, 16 KB
// per workgroup and stage), three stages in flight per workgroup.  Every
// loaded word is folded into an XOR that one store per thread keeps alive.
//   L = 256 with 4096-byte rows: 16 KB contiguous per stage (a plain stream)
//   L = 8: 128 rows x 128 bytes per stage (the streaming GEMM's code loads)
// With `scales` non-null the 128-row tiles also read 16 scale bytes of every
// row per stage from a [rows, row_bytes / 8] array (its scale-byte loads):
// row-major (16 bytes of each of 128 rows), or in the 128-row tiled order
// (one 2 KB run per tile and stage).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int L>
__global__ void __launch_bounds__(256)
read_kernel(const uint8_t* __restrict__ w, const uint8_t* __restrict__ sc, int sc_tiled, int ntiles, int nst,
            int64_t row_bytes, uint32_t* __restrict__ out)
{
    constexpr int RP = 256 / L;  // rows per load instruction round
    constexpr int R = 4 * RP;    // rows per tile
    const int tid = threadIdx.x;
    const int prow = tid / L, pc = tid % L;
    const int tile0 = blockIdx.x;
    if (tile0 >= ntiles)
        return;
    const int total = ((ntiles - 1 - tile0) / (int)gridDim.x + 1) * nst;
    const int64_t sc_bytes = row_bytes / 8;
    int ltile = tile0, ls = 0;
    u32x4 r[3][4], s[3];
    auto load = [&](u32x4 (&dst)[4], u32x4& sdst) {
        const uint8_t* base = w + ((int64_t)ltile * R + prow) * row_bytes + (int64_t)ls * L * 16 + pc * 16;
#pragma unroll
        for (int j = 0; j < 4; j++)
            dst[j] = *(const u32x4*)(base + (int64_t)j * RP * row_bytes);
        if (sc && tid < R)
            sdst = sc_tiled ? *(const u32x4*)(sc + ((int64_t)ltile * nst + ls) * 2048 + tid * 16)
                            : *(const u32x4*)(sc + ((int64_t)ltile * R + tid) * sc_bytes + (int64_t)ls * 16);
        if (++ls == nst) {
            // next tile of this workgroup; past the last, reread the last stage
            ls = 0;
            ltile += gridDim.x;
            if (ltile >= ntiles) {
                ltile -= gridDim.x;
                ls = nst - 1;
            }
        }
    };
    u32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < 3; d++) {
        s[d] = (u32x4){0, 0, 0, 0};
        load(r[d], s[d]);
    }
    int done = 0;
    while (done + 3 <= total) {
#pragma unroll
        for (int d = 0; d < 3; d++) {
            acc ^= r[d][0] ^ r[d][1] ^ r[d][2] ^ r[d][3] ^ s[d];
            // consume a set before refilling it, so three stay in flight
            __builtin_amdgcn_sched_barrier(0);
            load(r[d], s[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
        done += 3;
    }
#pragma unroll
    for (int d = 0; d < 3; d++)
        if (done + d < total)
            acc ^= r[d][0] ^ r[d][1] ^ r[d][2] ^ r[d][3] ^ s[d];
    out[(int64_t)blockIdx.x * 256 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

// Launch one read pass on `stream`.  lanes_per_row is 8 (128-row tiles) or
// 256 (4-row tiles of whole 4096-byte rows); rows * row_bytes bytes at w; sc
// null or rows * row_bytes / 8 bytes (lanes_per_row 8 only), in the tiled
// order when sc_tiled is non-zero; out holds grid *
// 256 words.  Returns 0, or -1 for a shape the kernel does not take (rows not
// a whole number of tiles, row_bytes not a whole number of stages, grid
// outside [8, 4096]), or the HIP error of the launch.
extern "C" int hbm_read_probe(int lanes_per_row, const void* w, const void* sc, int sc_tiled, int64_t rows,
                              int64_t row_bytes, int grid, void* out, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    if (grid < 8 || grid > 4096 || rows <= 0 || row_bytes <= 0 || !w || !out)
        return -1;
    if (lanes_per_row == 8) {
        if (rows % 128 != 0 || row_bytes % 128 != 0 || row_bytes % 8 != 0)
            return -1;
        read_kernel<8><<<grid, 256, 0, st>>>((const uint8_t*)w, (const uint8_t*)sc, sc_tiled, (int)(rows / 128),
                                             (int)(row_bytes / 128), row_bytes, (uint32_t*)out);
    } else if (lanes_per_row == 256) {
        if (rows % 4 != 0 || row_bytes != 4096 || sc)
            return -1;
        read_kernel<256><<<grid, 256, 0, st>>>((const uint8_t*)w, nullptr, 0, (int)(rows / 4), 1, row_bytes,
                                               (uint32_t*)out);
    } else {
        return -1;
    }
    return (int)hipGetLastError();
}
