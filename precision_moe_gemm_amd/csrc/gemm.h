// gemm.h -- W4A4 NVFP4 GEMM mainloop for gfx950, shared by the dense GEMM
// and the grouped MoE projections.
//
// What is computed (page "Qwen3.8-Flash-Next-NVFP4", section 核心: W4A4, both
// operands NVFP4; page "DeepSeek-V4.1-Flash-NVFP4", section 二: block scales
// applied inside the accumulation):
//   C[m, n] = G_A * G_W * sum_k (q*s)(A[m,k]) * (q*s)(W[n,k])
//
// Mapping onto CDNA4.  gfx950's scaled FP4 MFMA takes one power-of-two scale
// per 32 elements, NVFP4 needs an E4M3 scale (3 mantissa bits) per 16, so
// NVFP4 does not map onto it.  Instead every element is decoded to f16: the
// E2M1 value q (1 cvt per 2 elements, exact) times the E4M3 scale s (one
// packed f16 multiply per 2 elements).  q*s has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in f16, the MFMA products are
// exact in fp32 and only the fp32 summation rounds.
//
// Tiling.  A workgroup of WM x WN waves owns a BM x BN output tile and walks
// K in stages of 128 elements.  Each stage stages the *packed* operands in
// LDS (64 bytes of codes + 8 scale bytes per row, double-buffered), so LDS
// traffic is a quarter of an f16 tile.  Each wave reads its fragments'
// codes from LDS, decodes them in registers and issues
// v_mfma_f32_32x32x16_f16.  Inside a stage the K order is permuted: the two
// 32-lane halves of a wave hold elements [0, 64) and [64, 128) of the stage
// and step through them 8 at a time; A and W use the same permutation, which
// leaves the sum unchanged and lets every lane read 16 contiguous bytes.
#pragma once
#include "common.h"

namespace nvfp4 {

constexpr int kBK = 128;          // K elements per stage
constexpr int kRowBytes = kBK / 2; // packed bytes per row per stage
constexpr int kRowScales = kBK / 16;

enum GemmMode : int {
    kModeDense = 0,   // C = acc * G_A * G_W  (fp32 or bf16 output)
    kModeGateUp = 1,  // h = bf16(silu(g) * u), max |h| -> atomic word
    kModeDown = 2     // y = acc * G_A * G_W[e] (fp32)
};

struct GemmArgs {
    // A operand: NVFP4 rows; row r of the tile maps to an A row (see below)
    const uint8_t* a_packed;
    const uint8_t* a_scales;
    const float* a_global;
    // W operand: `experts` stacked [N_w, K] matrices
    const uint8_t* w_packed;
    const uint8_t* w_scales;
    const float* w_global;    // [experts]
    int64_t K;
    int64_t M;                // dense: rows of A
    int64_t N;                // output columns (dense/down: rows of W; gate_up: I)
    int64_t n_tiles;          // output column tiles
    int64_t m_tiles;          // dense: m tiles; grouped: upper bound
    // grouped: list positions of expert e are [offsets[e], offsets[e+1])
    const int32_t* offsets;
    const int32_t* tile_off;  // [experts+1] prefix of m tiles per expert
    const int32_t* perm;      // gate_up: list position -> t*k + j
    int32_t topk;
    int32_t experts;
    void* out;                // dense: C; gate_up: h bf16 [T*k, I]; down: y fp32
    int out_bf16;             // dense only
    uint32_t* h_amax;         // gate_up only
};

NVFP4_DEV int lds_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// Eight E2M1 codes (one dword) times one f16 scale -> the MFMA operand.
NVFP4_DEV half8_t decode8(uint32_t codes, _Float16 s)
{
    const half2_t ss = {s, s};
    const half2_t h0 = FP4_TO_F16X2(codes, 0) * ss;
    const half2_t h1 = FP4_TO_F16X2(codes, 1) * ss;
    const half2_t h2 = FP4_TO_F16X2(codes, 2) * ss;
    const half2_t h3 = FP4_TO_F16X2(codes, 3) * ss;
    return (half8_t){h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

// Two E4M3 bytes (byte 2*sel and 2*sel+1 of `w`) -> two f16 scales (exact).
template <int kSel>
NVFP4_DEV half2_t scales2(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kSel != 0);
}

NVFP4_DEV float silu_f(float g)
{
    return g / (1.0f + __expf(-g));
}

template <int BM, int BN, int WM, int WN, int MODE>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(GemmArgs p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 fragments per wave
    constexpr int ROWS = BM + BN;
    constexpr int CPT = (ROWS * 4 + NT - 1) / NT;  // 16-byte code chunks per thread per stage
    constexpr int SPT = (ROWS + NT - 1) / NT;   // scale rows per thread per stage
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 fragment");
    static_assert(MODE != kModeGateUp || FN % 2 == 0, "gate_up pairs gate and up fragments");
    static_assert(NT % 4 == 0, "four threads per staged row");

    __shared__ __attribute__((aligned(16))) uint8_t lds_codes[2][ROWS * kRowBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds_scales[2][ROWS * kRowScales];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / WN, wave_n = wave % WN;

    // ---- tile assignment (XCD-aware: consecutive ids go round-robin over 8
    // XCDs, so give each XCD a contiguous range of logical tiles) ----------
    const int64_t nblocks = (int64_t)gridDim.x;
    int64_t bid = blockIdx.x;
    if ((nblocks & 7) == 0)
        bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
    const int64_t mt = bid / p.n_tiles;
    const int64_t nt = bid - mt * p.n_tiles;

    int e = 0;
    int64_t row_begin, row_end;  // A-side rows of this tile (list positions or rows)
    if (MODE == kModeDense) {
        if (mt >= p.m_tiles)
            return;
        row_begin = mt * BM;
        row_end = row_begin + BM < p.M ? row_begin + BM : p.M;
    } else {
        if (mt >= p.tile_off[p.experts])
            return;
        int lo = 0, hi = p.experts - 1;  // largest e with tile_off[e] <= mt
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.tile_off[mid] <= mt)
                lo = mid;
            else
                hi = mid - 1;
        }
        e = lo;
        row_begin = p.offsets[e] + (mt - p.tile_off[e]) * BM;
        const int64_t eend = p.offsets[e + 1];
        row_end = row_begin + BM < eend ? row_begin + BM : eend;
    }

    const int64_t K = p.K;
    const int64_t kpb = K / 2, kpsb = K / 16;  // packed / scale bytes per row
    const int64_t w_rows = (MODE == kModeGateUp) ? 2 * p.N : p.N;
    const uint8_t* wp = p.w_packed + (int64_t)e * w_rows * kpb;
    const uint8_t* ws = p.w_scales + (int64_t)e * w_rows * kpsb;

    // ---- global source rows of this thread's staging chunks --------------
    auto a_row_of = [&](int r) -> int64_t {
        int64_t q = row_begin + r;
        if (q >= row_end)
            q = row_begin;  // padding rows repeat a valid row; never stored
        if (MODE == kModeGateUp)
            return p.perm[q] / p.topk;
        return q;
    };
    auto w_row_of = [&](int r) -> int64_t {
        if (MODE == kModeGateUp) {
            const int wn = r / TN, rr = r % TN;
            const int64_t base = nt * (BN / 2) + wn * (TN / 2);
            const int64_t i = rr < TN / 2 ? base + rr : base + (rr - TN / 2);
            return rr < TN / 2 ? i : p.N + i;
        }
        int64_t n = nt * BN + r;
        return n < p.N ? n : p.N - 1;
    };

    const uint8_t* csrc[CPT];
    int cdst[CPT];
    const int cchunk = tid & 3;
#pragma unroll
    for (int i = 0; i < CPT; i++) {
        int row = (tid >> 2) + i * (NT / 4);
        if (row >= ROWS)
            row = ROWS - 1;  // surplus chunk of the last pass: reload a real row
        if (row < BM)
            csrc[i] = p.a_packed + a_row_of(row) * kpb + cchunk * 16;
        else
            csrc[i] = wp + w_row_of(row - BM) * kpb + cchunk * 16;
        cdst[i] = row * kRowBytes + 16 * (cchunk ^ lds_swz(row));
    }
    const uint8_t* ssrc[SPT];
#pragma unroll
    for (int i = 0; i < SPT; i++) {
        const int row = tid + i * NT;
        const int rr = row < ROWS ? row : 0;
        if (rr < BM)
            ssrc[i] = p.a_scales + a_row_of(rr) * kpsb;
        else
            ssrc[i] = ws + w_row_of(rr - BM) * kpsb;
    }

    u32x4 creg[CPT];
    u32x2 sreg[SPT];
    auto load_stage = [&](int64_t s) {
#pragma unroll
        for (int i = 0; i < CPT; i++)
            creg[i] = *(const u32x4*)(csrc[i] + s * kRowBytes);
#pragma unroll
        for (int i = 0; i < SPT; i++)
            if (tid + i * NT < ROWS)
                sreg[i] = *(const u32x2*)(ssrc[i] + s * kRowScales);
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; i++)
            *(u32x4*)(&lds_codes[buf][cdst[i]]) = creg[i];
#pragma unroll
        for (int i = 0; i < SPT; i++)
            if (tid + i * NT < ROWS)
                *(u32x2*)(&lds_scales[buf][(tid + i * NT) * kRowScales]) = sreg[i];
    };

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            acc[i][j] = (float16_t){};

    const int frow = lane & 31;  // fragment row of this lane
    const int g = lane >> 5;     // K half of this lane
    const int64_t nstages = K / kBK;

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int64_t s = 0; s < nstages; s++) {
        const int buf = (int)(s & 1);
        if (s + 1 < nstages)
            load_stage(s + 1);

        const uint8_t* lc = lds_codes[buf];
        const uint8_t* lsc = lds_scales[buf];
        uint32_t sa[FM], sw[FN];
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int row = wave_m * TM + i * 32 + frow;
            sa[i] = *(const uint32_t*)(lsc + row * kRowScales + 4 * g);
        }
#pragma unroll
        for (int j = 0; j < FN; j++) {
            const int row = BM + wave_n * TN + j * 32 + frow;
            sw[j] = *(const uint32_t*)(lsc + row * kRowScales + 4 * g);
        }
#pragma unroll
        for (int t = 0; t < 2; t++) {
            u32x4 ca[FM], cw[FN];
            half2_t sca[FM], scw[FN];
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const int row = wave_m * TM + i * 32 + frow;
                ca[i] = *(const u32x4*)(lc + row * kRowBytes + 16 * ((2 * g + t) ^ lds_swz(row)));
                sca[i] = t == 0 ? scales2<0>(sa[i]) : scales2<1>(sa[i]);
            }
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int row = BM + wave_n * TN + j * 32 + frow;
                cw[j] = *(const u32x4*)(lc + row * kRowBytes + 16 * ((2 * g + t) ^ lds_swz(row)));
                scw[j] = t == 0 ? scales2<0>(sw[j]) : scales2<1>(sw[j]);
            }
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                half8_t fa[FM], fw[FN];
#pragma unroll
                for (int i = 0; i < FM; i++)
                    fa[i] = decode8(ca[i][kk], kk < 2 ? sca[i].x : sca[i].y);
#pragma unroll
                for (int j = 0; j < FN; j++)
                    fw[j] = decode8(cw[j][kk], kk < 2 ? scw[j].x : scw[j].y);
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int j = 0; j < FN; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fw[j], acc[i][j], 0, 0, 0);
            }
        }
        if (s + 1 < nstages)
            store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue --------------------------------------------------------
    const float ga = *p.a_global;
    const float gw = p.w_global[e];
    const float gscale = ga * gw;
    const int ncol = lane & 31;
    const int rsub = 4 * (lane >> 5);

    if (MODE == kModeGateUp) {
        uint16_t* h = (uint16_t*)p.out;
        uint32_t hmax = 0;
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int j = 0; j < FN / 2; j++) {
                const int64_t col = nt * (BN / 2) + wave_n * (TN / 2) + j * 32 + ncol;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t q = row_begin + wave_m * TM + i * 32 + (r & 3) + 8 * (r >> 2) + rsub;
                    const float gg = acc[i][j][r] * gscale;
                    const float uu = acc[i][j + FN / 2][r] * gscale;
                    const uint16_t hb = f32_to_bf16(silu_f(gg) * uu);
                    if (q < row_end) {
                        h[q * p.N + col] = hb;
                        const uint32_t mag = hb & 0x7FFFu;
                        hmax = hmax > mag ? hmax : mag;
                    }
                }
            }
        }
        hmax = wave_max_u32(hmax);
        if (lane == 0 && hmax != 0)
            atomicMax(p.h_amax, hmax << 16);
    } else {
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const int64_t col = nt * BN + wave_n * TN + j * 32 + ncol;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t q = row_begin + wave_m * TM + i * 32 + (r & 3) + 8 * (r >> 2) + rsub;
                    if (q < row_end && col < p.N) {
                        const float v = acc[i][j][r] * gscale;
                        if (MODE == kModeDense && p.out_bf16)
                            ((uint16_t*)p.out)[q * p.N + col] = f32_to_bf16(v);
                        else
                            ((float*)p.out)[q * p.N + col] = v;
                    }
                }
            }
        }
    }
}

}  // namespace nvfp4
