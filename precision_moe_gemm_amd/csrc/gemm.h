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
// NVFP4 does not map onto it.  Every element is decoded to f16 instead: the
// fp4->f16 conversion instruction (full VALU rate, 2 codes per instruction,
// unit scale) gives each E2M1 value q exactly, and one packed f16 multiply by
// the E4M3 scale s gives q*s exactly (at most 6 significant bits, magnitude
// in [2^-10, 2688], inside the f16 normal range).  Products are exact in fp32,
// only the fp32 summation rounds, and the epilogue multiplies by G_A * G_W.
//
// Tiling.  A workgroup of 4 waves (WM x WN) owns a BM x BN output tile and
// walks K in stages of 64.  Each element of a stage is decoded once per
// workgroup: thread t loads the packed codes and scale bytes of one A row and
// one W row (registers, prefetched a stage ahead), decodes them and writes
// f16 into a double-buffered LDS tile (rows of 128 bytes, 16-byte chunks
// XOR-swizzled by row so fragment reads and decode writes are free of bank
// conflicts).  Waves read MFMA fragments (8 f16 per lane) from the current
// tile and issue v_mfma_f32_32x32x16_f16 while decoding the next stage.
#pragma once
#include <utility>

#include "common.h"

namespace nvfp4 {

constexpr int kBK = 64;             // K elements per stage
constexpr int kRowF16Bytes = kBK * 2;  // f16 bytes per tile row per stage
constexpr int kStageCodeBytes = kBK / 2;
constexpr int kStageScaleBytes = kBK / 16;

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
    // grouped: tile i of expert e covers list positions
    // [row_base[e] + i BM, min(+BM, row_lim[e])), i < tile_off[e+1] - tile_off[e]
    const int32_t* tile_off;  // [experts+1] prefix of m tiles per expert
    const int32_t* row_base;  // [experts]
    const int32_t* row_lim;   // [experts]
    const int32_t* perm;      // gate_up: list position -> t*k + j
    int32_t topk;
    int32_t experts;
    void* out;                // dense: C; gate_up: h bf16 [T*k, I]; down: y fp32
    int out_bf16;             // dense only
    uint32_t* h_amax;         // gate_up only
    // weight-streaming kernel (dense and down modes): K split over `ksplit`
    // workgroups whose scaled fp32 sums go to partial[ksplit][M][N]
    // (ksplit > 1 only; M = rows of the output)
    int32_t ksplit;
    float* partial;
    // every W block scale is a power of two (or zero): the scale is folded
    // into the fp4 -> f16 conversion
    int32_t w_pow2;
    // W scale bytes in the 128-row tiled order (NVFP4_TILED_SCALES; then
    // the W row count % 128 == 0 and K % 256 == 0)
    int32_t w_tiled;
    // gate_up with a static G_h (non-null): h is encoded to NVFP4 in the
    // epilogue (codes [rows, N/2], scale bytes [rows, N/16]) instead of being
    // written as bf16 with its max
    const float* hq_global;
    uint8_t* hq_packed;
    uint8_t* hq_scales;
    // W4A16 (weight-streaming kernel only): the A operand is bf16 rows of
    // `lda` elements instead of NVFP4 (a_packed / a_scales / a_global unused)
    const uint16_t* a_bf16;
    int64_t lda;
};

// 16-byte chunk slot of chunk c in tile row r (8 chunks per row).
NVFP4_DEV int chunk_slot(int r, int c) { return c ^ ((r ^ (r >> 1)) & 7); }

// The 16 scale bytes of W row `row` (of its matrix) for the first 256
// elements of K; those of the next 256 follow `w_scale_step` bytes on.
// Row-major: row * K/16, step 16.  Tiled (NVFP4_TILED_SCALES): the 128-row
// tile's 2 KB runs, one per 256 elements of K, step 2048.
NVFP4_DEV const uint8_t* w_scale_row(const uint8_t* wsc, int64_t row, int64_t K, bool tiled)
{
    if (!tiled)
        return wsc + row * (K / 16);
    return wsc + ((row >> 7) * (K / 256) * 128 + (row & 127)) * 16;
}
NVFP4_DEV int64_t w_scale_step(bool tiled) { return tiled ? 2048 : 16; }

// Two E4M3 bytes (byte 2*sel and 2*sel+1 of `w`) -> two f16 scales (exact).
template <int kSel>
NVFP4_DEV half2_t scales2(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kSel != 0);
}

// Decode 8 codes (one dword, element 2j in the low nibble of byte j) times
// one f16 scale into a 16-byte f16 chunk.
NVFP4_DEV u32x4 decode_chunk(uint32_t codes, _Float16 s)
{
    const half2_t ss = {s, s};
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss);
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss);
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss);
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss);
    return r;
}

// 8 codes times a power-of-two (or zero) scale s: the conversion applies
// 2^exponent(s) exactly, so q * s needs no separate multiply.
NVFP4_DEV u32x4 decode_chunk_p2(uint32_t codes, float s)
{
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, s, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, s, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, s, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, s, 3));
    return r;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 8 codes times an fp32 block scale s into 8 bf16 (16 bytes): q -> fp32,
// one multiply each (exact: q * s has at most 6 significant bits), bf16.
NVFP4_DEV u32x4 decode_chunk_bf16(uint32_t codes, float s)
{
    const float2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const float2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const float2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const float2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    return (u32x4){pack_bf16x2(q0.x * s, q0.y * s), pack_bf16x2(q1.x * s, q1.y * s),
                   pack_bf16x2(q2.x * s, q2.y * s), pack_bf16x2(q3.x * s, q3.y * s)};
}

// 8 codes times a power-of-two (or zero) scale s into 8 bf16: the
// conversion applies 2^exponent(s) exactly.
NVFP4_DEV u32x4 decode_chunk_bf16_p2(uint32_t codes, float s)
{
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, s, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, s, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, s, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, s, 3));
    return r;
}

// Work item of this workgroup, or -1.  Workgroups are dispatched to the 8
// XCDs round-robin by id, so XCD (id % 8) takes a contiguous eighth of the
// `items` real work items (neighbouring tiles share operands through that
// XCD's L2).  The grid may hold more workgroups than items (grouped launches
// size it by an upper bound): the surplus exits here, on every XCD alike.
NVFP4_DEV int64_t xcd_item(int64_t items)
{
    const int64_t per = (items + 7) >> 3;
    const int64_t j = (int64_t)(blockIdx.x >> 3);
    const int64_t it = (int64_t)(blockIdx.x & 7) * per + j;
    return (j < per && it < items) ? it : -1;
}

template <int V>
struct IntC {
    static constexpr int value = V;
};

// f(IntC<0>{}), ..., f(IntC<N-1>{}) in order
template <class F, int... I>
NVFP4_DEV void static_for_impl(F&& f, std::integer_sequence<int, I...>)
{
    (f(IntC<I>{}), ...);
}
template <int N, class F>
NVFP4_DEV void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// g * sigmoid(g) in fp32 with the hardware exponential and reciprocal
// (about 1 ulp each, far below the bf16 rounding of h that follows)
NVFP4_DEV float silu_f(float g)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Output tile of a prefill-class workgroup: expert, A-side rows
// [row_begin, row_end) (rows of A, or list positions when grouped) and the
// column tile.  False for surplus workgroups.
struct TileCoord {
    int e;
    int64_t row_begin, row_end, nt;
};
template <int BM, int MODE>
NVFP4_DEV bool tile_coord(const GemmArgs& p, TileCoord& tc)
{
    // XCD-aware: consecutive ids go round-robin over 8 XCDs, so each XCD
    // takes a contiguous range of logical tiles
    const int64_t m_act = MODE == kModeDense ? p.m_tiles : p.tile_off[p.experts];
    const int64_t bid = xcd_item(m_act * p.n_tiles);
    if (bid < 0)
        return false;
    // Order of the logical tiles: bands of GM = 4 A tiles, and inside a band
    // groups of GN (8, 7 or 4) W tiles with the A tile varying fastest.  The
    // 32 tiles resident on an XCD at once then read about 4 A and 8 W tiles
    // instead of 2 A and 16 (A tile fastest over all W tiles): the 384-expert
    // prefill's 256-row class fetched 4.2 instead of 5.6 GB through L2.
    const int64_t nt_all = p.n_tiles;
    const int64_t GN = nt_all % 8 == 0 ? 8 : nt_all % 7 == 0 ? 7 : nt_all % 4 == 0 ? 4 : nt_all;
    constexpr int64_t GM = 4;
    const int64_t band = bid / (GM * nt_all), r = bid - band * GM * nt_all;
    const int64_t gm = m_act - band * GM < GM ? m_act - band * GM : GM;
    const int64_t ng = r / (gm * GN), q = r - ng * gm * GN;
    const int64_t mt = band * GM + q % gm;
    tc.nt = ng * GN + q / gm;
    tc.e = 0;
    if (MODE == kModeDense) {
        if (mt >= p.m_tiles)
            return false;
        tc.row_begin = mt * BM;
        tc.row_end = tc.row_begin + BM < p.M ? tc.row_begin + BM : p.M;
    } else {
        if (mt >= p.tile_off[p.experts])
            return false;
        int lo = 0, hi = p.experts - 1;  // largest e with tile_off[e] <= mt
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.tile_off[mid] <= mt)
                lo = mid;
            else
                hi = mid - 1;
        }
        tc.e = lo;
        tc.row_begin = p.row_base[lo] + (mt - p.tile_off[lo]) * BM;
        const int64_t eend = p.row_lim[lo];
        tc.row_end = tc.row_begin + BM < eend ? tc.row_begin + BM : eend;
    }
    return true;
}

// Row of A that tile row r reads (padding rows repeat a valid row and are
// never stored); gate_up gathers token rows through the permutation.
template <int MODE>
NVFP4_DEV int64_t tile_a_row(const GemmArgs& p, const TileCoord& tc, int r)
{
    int64_t q = tc.row_begin + r;
    if (q >= tc.row_end)
        q = tc.row_begin;
    if (MODE == kModeGateUp)
        return p.perm[q] / p.topk;
    return q;
}

// Row of W (within the expert) that W-tile row r reads.  For gate_up, wave
// column group wn holds TN/2 gate rows then the matching TN/2 up rows, so a
// lane's gate and up accumulators cover the same output column.
template <int BN, int TN, int MODE>
NVFP4_DEV int64_t tile_w_row(const GemmArgs& p, const TileCoord& tc, int r)
{
    if (MODE == kModeGateUp) {
        // columns past N (a last tile of an N that is not a multiple of the
        // tile) reread column N - 1 of the same half and are never stored
        const int wn = r / TN, rr = r % TN;
        const int64_t base = tc.nt * (BN / 2) + wn * (TN / 2);
        int64_t c = base + (rr < TN / 2 ? rr : rr - TN / 2);
        c = c < p.N ? c : p.N - 1;
        return rr < TN / 2 ? c : p.N + c;
    }
    const int64_t n = tc.nt * BN + r;
    return n < p.N ? n : p.N - 1;
}

// Epilogue of a 32x32-fragment wave tile: lane holds column lane % 32 and
// rows (i % 4) + 8 (i / 4) + 4 (lane / 32) of each fragment.
template <int BN, int WM, int WN, int TM, int TN, int FM, int FN, int MODE>
NVFP4_DEV void store_tile(const GemmArgs& p, const TileCoord& tc, float16_t (&acc)[FM][FN], int wave_m,
                          int wave_n, int lane, uint8_t* lds)
{
    const float gscale = *p.a_global * p.w_global[tc.e];
    const int ncol = lane & 31;
    const int rsub = 4 * (lane >> 5);
    const int64_t wrow0 = tc.row_begin + wave_m * TM;  // first output row of this wave
    const int rows_left = (int)(tc.row_end - wrow0);
    const int ld = (int)p.N;
    if (MODE == kModeGateUp && p.hq_global) {
        // h straight to NVFP4 through LDS (free once the mainloop is done),
        // one wave row at a time: the waves of that row put their bf16 h
        // [TM, BN/2] in LDS, then every thread encodes whole 16-element
        // blocks as the quantize kernel does
        constexpr int HC = BN / 2;  // h columns of the tile
        uint16_t* hs = (uint16_t*)lds;
        const float Gh = *p.hq_global, six = 6.0f * Gh;
        const int64_t hcol0 = tc.nt * HC;
#pragma unroll 1
        for (int pm = 0; pm < WM; pm++) {
            __syncthreads();
            if (wave_m == pm) {
#pragma unroll
                for (int i = 0; i < FM; i++) {
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int rr = i * 32 + (r & 3) + 8 * (r >> 2) + rsub;
#pragma unroll
                        for (int j = 0; j < FN / 2; j++) {
                            const float gg = acc[i][j][r] * gscale;
                            const float uu = acc[i][j + FN / 2][r] * gscale;
                            hs[rr * HC + wave_n * (TN / 2) + j * 32 + ncol] = f32_to_bf16(silu_f(gg) * uu);
                        }
                    }
                }
            }
            __syncthreads();
            for (int b = threadIdx.x; b < TM * (HC / 16); b += blockDim.x) {
                const int row = b / (HC / 16), bc = b - row * (HC / 16);
                const int64_t grow = tc.row_begin + pm * TM + row;
                if (grow < tc.row_end && hcol0 + 16 * bc < p.N) {
                    const u32x4 v0 = *(const u32x4*)(hs + row * HC + 16 * bc);
                    const u32x4 v1 = *(const u32x4*)(hs + row * HC + 16 * bc + 8);
                    const uint32_t a0 = absmax_bits8(v0), a1 = absmax_bits8(v1);
                    uint32_t sc;
                    const float rcp = block_scale(a0 > a1 ? a0 : a1, Gh, six, &sc);
                    const int64_t col = hcol0 + 16 * bc;
                    *(u32x2*)(p.hq_packed + grow * (p.N / 2) + col / 2) =
                        (u32x2){encode_half(v0, rcp), encode_half(v1, rcp)};
                    p.hq_scales[grow * (p.N / 16) + col / 16] = (uint8_t)sc;
                }
            }
        }
    } else if (MODE == kModeGateUp) {
        const int64_t col0 = tc.nt * (BN / 2) + wave_n * (TN / 2) + ncol;
        uint16_t* h = (uint16_t*)p.out + wrow0 * p.N + col0;
        uint32_t hmax = 0;
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int rr = i * 32 + (r & 3) + 8 * (r >> 2) + rsub;
                if (rr < rows_left) {
#pragma unroll
                    for (int j = 0; j < FN / 2; j++) {
                        if (col0 + j * 32 >= p.N)
                            continue;
                        const float gg = acc[i][j][r] * gscale;
                        const float uu = acc[i][j + FN / 2][r] * gscale;
                        const uint16_t hb = f32_to_bf16(silu_f(gg) * uu);
                        h[rr * ld + j * 32] = hb;
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
        const int64_t col0 = tc.nt * BN + wave_n * TN + ncol;
        const bool bf16_out = MODE == kModeDense && p.out_bf16;
        float* of = (float*)p.out + wrow0 * p.N + col0;
        uint16_t* ob = (uint16_t*)p.out + wrow0 * p.N + col0;
#pragma unroll
        for (int i = 0; i < FM; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int rr = i * 32 + (r & 3) + 8 * (r >> 2) + rsub;
                if (rr < rows_left) {
#pragma unroll
                    for (int j = 0; j < FN; j++) {
                        if (col0 + j * 32 < p.N) {
                            const float v = acc[i][j][r] * gscale;
                            if (bf16_out)
                                ob[rr * ld + j * 32] = f32_to_bf16(v);
                            else
                                of[rr * ld + j * 32] = v;
                        }
                    }
                }
            }
        }
    }
}

// RAG: K is a multiple of 16 but not of 64.  Rows then start on 8-byte
// (codes) and 1-byte (scales) boundaries, so codes are loaded 8 bytes (one
// 16-element block) at a time and scale bytes one at a time, and the last,
// partial stage reads only its valid blocks: the rest of it is zero codes
// with zero scales, which add nothing to the sums.
template <int BM, int BN, int WM, int WN, int MODE, bool RAG = false>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_kernel(GemmArgs p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 fragments per wave
    constexpr int ROWS = BM + BN;               // tile rows: A rows, then W rows
    constexpr int RPT = (ROWS + NT - 1) / NT;   // rows decoded per thread per stage
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 fragment");
    static_assert(MODE != kModeGateUp || FN % 2 == 0, "gate_up pairs gate and up fragments");

    // f16 operand tiles: A rows and W rows, 128 bytes per row per stage,
    // written one stage ahead (ring of 2)
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kRowF16Bytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds_w[2][BN * kRowF16Bytes];
    // scale bytes: each decoded row's 16 bytes for a group of 4 stages are
    // fetched in one request and parked here, dword q of slot (i, tid) at
    // [buf][q][i * NT + tid]; only the thread that parked them reads them
    __shared__ uint32_t lds_sc[2][4][NT * RPT];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / WN, wave_n = wave % WN;

    TileCoord tc;
    if (!tile_coord<BM, MODE>(p, tc))
        return;
    const int e = tc.e;

    const int64_t K = p.K;
    const int64_t kpb = K / 2, kpsb = K / 16;  // packed / scale bytes per row
    const int64_t w_rows = (MODE == kModeGateUp) ? 2 * p.N : p.N;
    const uint8_t* wp = p.w_packed + (int64_t)e * w_rows * kpb;
    const uint8_t* wsc = p.w_scales + (int64_t)e * w_rows * kpsb;
    auto a_row_of = [&](int r) -> int64_t { return tile_a_row<MODE>(p, tc, r); };
    auto w_row_of = [&](int r) -> int64_t { return tile_w_row<BN, TN, MODE>(p, tc, r); };

    // ---- rows this thread decodes from packed codes ----------------------
    const uint8_t* csrc[RPT];
    const uint8_t* ssrc[RPT];
    int64_t sstep[RPT];  // scale bytes from one group of 4 stages to the next
    int drow[RPT];
#pragma unroll
    for (int i = 0; i < RPT; i++) {
        int row = tid + i * NT;
        if (row >= ROWS)
            row = ROWS - 1;  // surplus thread of the last pass: decodes the last row again
        drow[i] = row;
        if (row < BM) {
            const int64_t ar = a_row_of(row);
            csrc[i] = p.a_packed + ar * kpb;
            ssrc[i] = p.a_scales + ar * kpsb;
            sstep[i] = 16;
        } else {
            const int64_t wr = w_row_of(row - BM);
            csrc[i] = wp + wr * kpb;
            // (tiled W scales come with K % 256 == 0: whole groups, no RAG)
            ssrc[i] = w_scale_row(wsc, wr, K, p.w_tiled);
            sstep[i] = w_scale_step(p.w_tiled);
        }
    }
    u32x4 creg[2][RPT][2];
    const int64_t nstages = RAG ? (K + kBK - 1) / kBK : K / kBK;
    auto load_stage = [&](int st, int set) {
        if (RAG) {
            // valid code bytes of this stage: 32, or 8/16/24 in the last one
            const int64_t vb = kpb - (int64_t)st * kStageCodeBytes;
#pragma unroll
            for (int i = 0; i < RPT; i++) {
                const uint8_t* c = csrc[i] + (int64_t)st * kStageCodeBytes;
                u32x2 v[4];
#pragma unroll
                for (int q = 0; q < 4; q++)
                    v[q] = 8 * q < vb ? *(const u32x2*)(c + 8 * q) : (u32x2){0, 0};
                creg[set][i][0] = (u32x4){v[0].x, v[0].y, v[1].x, v[1].y};
                creg[set][i][1] = (u32x4){v[2].x, v[2].y, v[3].x, v[3].y};
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const u32x4* c = (const u32x4*)(csrc[i] + st * kStageCodeBytes);
            creg[set][i][0] = c[0];
            creg[set][i][1] = c[1];
        }
    };
    // scale dwords of stages [4 G, 4 G + 4): one 16-byte load per row, or,
    // for a last group that is not whole, one clamped dword per stage
    // (ragged K: byte loads, zero past the row's kpsb bytes)
    u32x4 tsc[RPT];
    auto load_scales = [&](int64_t grp) {
        const int64_t st0 = 4 * grp;
        if (RAG) {
            const int64_t last = nstages - 1;
#pragma unroll
            for (int i = 0; i < RPT; i++) {
                uint32_t d[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int64_t b0 = (st0 + j < last ? st0 + j : last) * kStageScaleBytes;
                    uint32_t w = 0;
#pragma unroll
                    for (int b = 0; b < 4; b++)
                        w |= (b0 + b < kpsb ? (uint32_t)ssrc[i][b0 + b] : 0u) << (8 * b);
                    d[j] = w;
                }
                tsc[i] = (u32x4){d[0], d[1], d[2], d[3]};
            }
            return;
        }
        if (st0 + 4 <= nstages) {
#pragma unroll
            for (int i = 0; i < RPT; i++)
                tsc[i] = *(const u32x4*)(ssrc[i] + grp * sstep[i]);
        } else {
            const int64_t last = nstages - 1;
#pragma unroll
            for (int i = 0; i < RPT; i++) {
                tsc[i].x = *(const uint32_t*)(ssrc[i] + (st0 < last ? st0 : last) * kStageScaleBytes);
                tsc[i].y = *(const uint32_t*)(ssrc[i] + (st0 + 1 < last ? st0 + 1 : last) * kStageScaleBytes);
                tsc[i].z = *(const uint32_t*)(ssrc[i] + (st0 + 2 < last ? st0 + 2 : last) * kStageScaleBytes);
                tsc[i].w = *(const uint32_t*)(ssrc[i] + (st0 + 3 < last ? st0 + 3 : last) * kStageScaleBytes);
            }
        }
    };
    auto park_scales = [&](int buf) {
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            lds_sc[buf][0][i * NT + tid] = tsc[i].x;
            lds_sc[buf][1][i * NT + tid] = tsc[i].y;
            lds_sc[buf][2][i * NT + tid] = tsc[i].z;
            lds_sc[buf][3][i * NT + tid] = tsc[i].w;
        }
    };
    uint32_t scw[RPT];  // scale dwords of the stage being decoded
    auto read_scales = [&](int64_t st) {
#pragma unroll
        for (int i = 0; i < RPT; i++)
            scw[i] = lds_sc[(st >> 2) & 1][st & 3][i * NT + tid];
    };
    // decode part q (of 4: the 16-element block q) of the stage in register
    // set `set` into tile buffer `buf`
    auto decode_part = [&](int set, int buf, int part) {
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const uint32_t sw = scw[i];
            const half2_t s2 = part < 2 ? scales2<0>(sw) : scales2<1>(sw);
            const _Float16 sc = (part & 1) ? s2.y : s2.x;
            const u32x4 cv = creg[set][i][part >> 1];
            const uint32_t c0 = (part & 1) ? cv.z : cv.x;
            const uint32_t c1 = (part & 1) ? cv.w : cv.y;
            const int r = drow[i];
            uint8_t* rowp = r < BM ? &lds_a[buf][r * kRowF16Bytes] : &lds_w[buf][(r - BM) * kRowF16Bytes];
            *(u32x4*)(rowp + 16 * chunk_slot(r, 2 * part)) = decode_chunk(c0, sc);
            *(u32x4*)(rowp + 16 * chunk_slot(r, 2 * part + 1)) = decode_chunk(c1, sc);
        }
    };

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            acc[i][j] = (float16_t){};

    const int frow = lane & 31;  // fragment row of this lane
    const int g = lane >> 5;     // which 8 of the 16 K-elements of an MFMA step
    int aoff[FM], woff[FN];      // byte offset of this lane's fragment rows
#pragma unroll
    for (int i = 0; i < FM; i++)
        aoff[i] = (wave_m * TM + i * 32 + frow) * kRowF16Bytes;
#pragma unroll
    for (int j = 0; j < FN; j++)
        woff[j] = (wave_n * TN + j * 32 + frow) * kRowF16Bytes;
    // the chunk slot depends on the row only through (row ^ row >> 1) & 7,
    // the same for every fragment of this lane (rows differ by 32)
    const int sw_a = ((wave_m * TM + frow) ^ ((wave_m * TM + frow) >> 1)) & 7;
    const int sw_w = ((BM + wave_n * TN + frow) ^ ((BM + wave_n * TN + frow) >> 1)) & 7;

    half8_t fa[2][FM], fw[2][FN];
    auto read_frags = [&](const uint8_t* ta, const uint8_t* tw, int kk, int slot) {
#pragma unroll
        for (int i = 0; i < FM; i++)
            fa[slot][i] = *(const half8_t*)(ta + aoff[i] + 16 * ((2 * kk + g) ^ sw_a));
#pragma unroll
        for (int j = 0; j < FN; j++)
            fw[slot][j] = *(const half8_t*)(tw + woff[j] + 16 * ((2 * kk + g) ^ sw_w));
    };

    // prologue: scales of stages 0..3 parked, stage 0 decoded into buffers
    // 0, packed stage 1 in registers
    load_scales(0);
    park_scales(0);
    load_stage(0, 0);
    read_scales(0);
#pragma unroll
    for (int q = 0; q < 4; q++)
        decode_part(0, 0, q);
    load_stage(nstages > 1 ? 1 : 0, 1);
    __syncthreads();
    read_frags(lds_a[0], lds_w[0], 0, 0);

    // one stage: MFMAs on buffers CUR (stage s) interleaved with decoding
    // the packed stage s+1 (register set CUR ^ 1) into buffers CUR ^ 1.
    // Q = s mod 4 and CUR = Q mod 2 are compile-time constants, so every
    // register set stays in fixed registers.
    auto stage = [&](int64_t s, auto q_tag) {
        constexpr int Q = decltype(q_tag)::value;
        constexpr int cur = Q & 1, nxt = cur ^ 1;
        // refill the register set stage s used (decoded last iteration);
        // past the end reload the last stage (harmless, never decoded)
        load_stage(s + 2 < nstages ? s + 2 : nstages - 1, cur);
        if (Q == 2)
            load_scales((s + 2) >> 2);  // the group that starts at stage s+2
        // issue those loads first: they have the whole stage to land
        __builtin_amdgcn_sched_group_barrier(0x020, Q == 2 ? 3 * RPT : 2 * RPT, 0);  // VMEM read
        if (Q == 3)
            park_scales(((s + 1) >> 2) & 1);  // its buffer was last read four stages ago
        read_scales(s + 1);
        const uint8_t* ta = lds_a[cur];
        const uint8_t* tw = lds_w[cur];
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            const int sl = kk & 1;
            // fragments of the next k-step first, fenced so the scheduler
            // cannot sink them next to their use; the last k-step reads the
            // first fragments of stage s+1 (complete since the barrier)
            if (kk < 3)
                read_frags(ta, tw, kk + 1, sl ^ 1);
            else
                read_frags(lds_a[nxt], lds_w[nxt], 0, sl ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[sl][i], fw[sl][j], acc[i][j], 0, 0, 0);
            // the next stage is decoded during the first three k-steps (the
            // last stage decodes stale registers into a buffer nobody reads)
            if (kk < 2)
                decode_part(nxt, nxt, kk);
            if (kk == 2) {
                decode_part(nxt, nxt, 2);
                decode_part(nxt, nxt, 3);
            }
            // interleave the decode VALU work and its stores between MFMAs
            if (kk < 2) {
#pragma unroll
                for (int m = 0; m < FM * FN; m++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);      // VALU
                    if (m % 4 == 3)
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
                }
            } else if (kk == 2) {
#pragma unroll
                for (int m = 0; m < FM * FN; m++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);      // VALU
                    if (m % 2 == 1)
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // stage s+1 is fully written and stage s's last fragments are in
            // registers: one barrier, then the last k-step's MFMAs cover the
            // latency of the first reads of stage s+1
            if (kk == 2)
                __syncthreads();
        }
    };
    int64_t s = 0;
    for (; s + 3 < nstages; s += 4) {
        stage(s, IntC<0>{});
        stage(s + 1, IntC<1>{});
        stage(s + 2, IntC<2>{});
        stage(s + 3, IntC<3>{});
    }
    if (s < nstages)
        stage(s, IntC<0>{});
    if (s + 1 < nstages)
        stage(s + 1, IntC<1>{});
    if (s + 2 < nstages)
        stage(s + 2, IntC<2>{});

    store_tile<BN, WM, WN, TM, TN, FM, FN, MODE>(p, tc, acc, wave_m, wave_n, lane, &lds_w[0][0]);
}

// ---------------------------------------------------------------------------
// Prefill mainloop with coalesced, direct-to-LDS code loads.
//
// Same tiles, MFMA and decode-once scheme as gemm_kernel (4 waves of
// 128 x 128, v_mfma_f32_32x32x16_f16 on f16 LDS tiles), with the packed codes
// moved by the LDS DMA path instead of through registers: a workgroup copies
// the codes of a 128-element group of K for all its tile rows (64 bytes per
// row, four lanes per row, 16 rows per instruction) straight into an LDS
// staging buffer, two groups ahead of use.  Each f16 stage covers 32 K
// elements; during stage s every thread reads its rows' 16 code bytes of
// stage s+1 from the staging buffer, decodes them with their block scales
// (held in registers, 16 bytes per row per 256 elements) and writes the f16
// tile of stage s+1, while the waves run the two k-steps of stage s.  One
// barrier per stage, placed between the two k-steps so the first fragments
// of the next stage are read under the second k-step's MFMAs.
// ---------------------------------------------------------------------------
constexpr int kTFK = 32;             // K elements per f16 stage
constexpr int kTFRow = kTFK * 2;     // f16 bytes per tile row per stage
constexpr int kTGRow = 64;           // packed bytes per row per group (4 stages)
constexpr int kTSRow = 16;           // scale bytes per row per scale group (8 stages)

// Byte offset of 16-byte chunk c (of 4) of the 64-byte row r in an f16
// tile or in the packed staging.  Rows are paired into 128-byte lines
// (line r / 2 holds chunk c of row r in slot 4 (r % 2) + c) and the 8 slots
// of line q are XOR-swizzled by (q ^ q / 2) mod 8: measured free of bank
// conflicts both for reads and writes of 64 consecutive rows at one chunk
// (staging reads, decode writes) and for MFMA fragment reads (32 rows, two
// chunks); the plain 64-byte-row layouts measured were not.
NVFP4_DEV int tline_sw(int r) { return ((r >> 1) ^ (r >> 2)) & 7; }
NVFP4_DEV int tpos(int r, int c) { return 64 * (r & ~1) + 16 * ((4 * (r & 1) + c) ^ tline_sw(r)); }

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
NVFP4_DEV void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// wait until all of this wave's LDS operations are complete
NVFP4_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then s_barrier.  __syncthreads() would also wait for the LDS DMA
// copies in flight (they count as LDS writes), which must stay in flight
// across stages; their completion is awaited explicitly with wait_vm.
NVFP4_DEV void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int BM, int BN, int MODE, bool P2>
__global__ void __launch_bounds__(256)
gemm_tile_kernel(GemmArgs p)
{
    constexpr int WM = 2, WN = 2, NW = 4, NT = 256;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int NJ = (ROWS + 16 * NW - 1) / (16 * NW);  // staging copies per wave per group
    constexpr int SROWS = NJ * NW * 16;                    // staged rows (>= ROWS)
    constexpr int RPT = (ROWS + NT - 1) / NT;              // rows decoded per thread per stage
    static_assert(BM % 32 == 0 && BN % 64 == 0, "tile shape");
    static_assert(MODE != kModeGateUp || FN % 2 == 0, "gate_up pairs gate and up fragments");

    __shared__ __attribute__((aligned(16))) uint8_t lds_f[2][ROWS * kTFRow];  // f16 tiles
    // packed codes of groups with even / odd index (separate arrays, so the
    // compiler sees that reading one does not wait for copies into the other)
    __shared__ __attribute__((aligned(16))) uint8_t lds_p0[SROWS * kTGRow];
    __shared__ __attribute__((aligned(16))) uint8_t lds_p1[SROWS * kTGRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;

    TileCoord tc;
    if (!tile_coord<BM, MODE>(p, tc))
        return;
    const int e = tc.e;
    const int64_t K = p.K;
    const int64_t kpb = K / 2, kpsb = K / 16;  // packed / scale bytes per row
    const int64_t w_rows = (MODE == kModeGateUp) ? 2 * p.N : p.N;
    const uint8_t* wp = p.w_packed + (int64_t)e * w_rows * kpb;
    const uint8_t* wsc = p.w_scales + (int64_t)e * w_rows * kpsb;
    auto matrix_row = [&](int r) -> int64_t {
        return r < BM ? tile_a_row<MODE>(p, tc, r) : tile_w_row<BN, TN, MODE>(p, tc, r - BM);
    };

    const int64_t nst = K / kTFK;      // f16 stages (even: K % 64 == 0)
    const int64_t ngr = (nst + 3) >> 2;  // packed groups
    const int64_t nsg = (nst + 7) >> 3;  // scale groups

    // ---- staging copies: copy j of this wave fills LDS bytes
    // [1024 (NJ wave + j), +1024), lane l writing 16 bytes at 16 l, which is
    // line q = 8 (NJ wave + j) + l / 8, slot l % 8: the lane copies the
    // (row, chunk) that tpos places there.  The 8 lanes of a line cover the
    // 64 bytes of both its rows, so each copy reads 16 whole row segments.
    int32_t srow[NJ];
    int scq[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        const int q = 8 * (NJ * wave + j) + (lane >> 3);
        const int hc = (lane & 7) ^ ((q ^ (q >> 1)) & 7);  // 4 (r % 2) + c
        int r = 2 * q + (hc >> 2);
        if (r >= ROWS)
            r = ROWS - 1;
        srow[j] = (int32_t)matrix_row(r);
        scq[j] = hc & 3;
    }
    // copies [J0, J1) of group G into staging buffer BUF
    auto issue_group = [&](int64_t G, auto buf_tag, auto j0_tag, auto j1_tag) {
        constexpr int BUF = decltype(buf_tag)::value;
        constexpr int J0 = decltype(j0_tag)::value, J1 = decltype(j1_tag)::value;
        const int64_t cb = G * kTGRow;
        const int cvalid = (int)((kpb - cb) >> 4);  // whole chunks left in the row (>= 2)
        uint8_t* dst = BUF ? lds_p1 : lds_p0;
#pragma unroll
        for (int j = J0; j < J1; j++) {
            const bool is_a = 16 * (NJ * wave + j) < BM;  // uniform per copy
            const int c = scq[j] < cvalid ? scq[j] : cvalid - 1;
            const uint8_t* src = (is_a ? p.a_packed : wp) + (int64_t)srow[j] * kpb + cb + 16 * c;
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)(dst + (NJ * wave + j) * 1024), 16,
                                             0, 0);
        }
    };

    // ---- rows this thread decodes, and their scale bytes (16 per row per
    // scale group, in registers: the current group and the next)
    int drow[RPT];
    const uint8_t* ssrc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; i++) {
        int r = tid + i * NT;
        if (r >= ROWS)
            r = ROWS - 1;  // surplus thread: decodes the last row again
        drow[i] = r;
        const int64_t mr = matrix_row(r);
        ssrc[i] = (r < BM ? p.a_scales : wsc) + mr * kpsb;
    }
    u32x4 sc_cur[RPT], sc_nxt[RPT];
    auto load_scales = [&](int64_t SG, u32x4 (&dst)[RPT]) {
        const int64_t sb = SG * kTSRow;
        if (sb + kTSRow <= kpsb) {
#pragma unroll
            for (int i = 0; i < RPT; i++)
                dst[i] = *(const u32x4*)(ssrc[i] + sb);
        } else {
            // last group of a K that is not a multiple of 256: clamp dwords
            const int64_t last = (kpsb >> 2) - 1;
            const int64_t d0 = sb >> 2;
#pragma unroll
            for (int i = 0; i < RPT; i++) {
                const uint32_t* q = (const uint32_t*)ssrc[i];
                dst[i].x = q[d0 < last ? d0 : last];
                dst[i].y = q[d0 + 1 < last ? d0 + 1 : last];
                dst[i].z = q[d0 + 2 < last ? d0 + 2 : last];
                dst[i].w = q[d0 + 3 < last ? d0 + 3 : last];
            }
        }
    };

    // decode f16 stage with index T (mod 8) of its scale group from the
    // staged codes into f16 buffer FB
    u32x4 dcodes[RPT];
    auto stage_codes = [&](auto t_tag) {
        constexpr int T = decltype(t_tag)::value;
        const uint8_t* src = ((T >> 2) & 1) ? lds_p1 : lds_p0;
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int r = drow[i];
            dcodes[i] = *(const u32x4*)(src + tpos(r, T & 3));
        }
    };
    auto decode_stage = [&](auto t_tag, const u32x4 (&sc)[RPT]) {
        constexpr int T = decltype(t_tag)::value;
        uint8_t* dst = lds_f[T & 1];
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int r = drow[i];
            const uint32_t sw = (T >> 1) == 0 ? sc[i].x : (T >> 1) == 1 ? sc[i].y : (T >> 1) == 2 ? sc[i].z : sc[i].w;
            if (P2 && i * NT >= BM) {
                // rows of this pass are all W rows: power-of-two scales
                const float s0 = __builtin_amdgcn_cvt_f32_fp8(sw, 2 * (T & 1));
                const float s1 = __builtin_amdgcn_cvt_f32_fp8(sw, 2 * (T & 1) + 1);
                *(u32x4*)(dst + tpos(r, 0)) = decode_chunk_p2(dcodes[i].x, s0);
                *(u32x4*)(dst + tpos(r, 1)) = decode_chunk_p2(dcodes[i].y, s0);
                *(u32x4*)(dst + tpos(r, 2)) = decode_chunk_p2(dcodes[i].z, s1);
                *(u32x4*)(dst + tpos(r, 3)) = decode_chunk_p2(dcodes[i].w, s1);
            } else {
                const half2_t s2 = (T & 1) ? scales2<1>(sw) : scales2<0>(sw);
                *(u32x4*)(dst + tpos(r, 0)) = decode_chunk(dcodes[i].x, s2.x);
                *(u32x4*)(dst + tpos(r, 1)) = decode_chunk(dcodes[i].y, s2.x);
                *(u32x4*)(dst + tpos(r, 2)) = decode_chunk(dcodes[i].z, s2.y);
                *(u32x4*)(dst + tpos(r, 3)) = decode_chunk(dcodes[i].w, s2.y);
            }
        }
    };

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            acc[i][j] = (float16_t){};

    const int frow = lane & 31;  // fragment row of this lane
    const int g = lane >> 5;     // which 8 of the 16 K-elements of an MFMA step
    // fragment rows of a lane differ by multiples of 32, which keeps the
    // line swizzle and the row parity: one slot base per operand
    const int ra = wave_m * TM + frow, rw = BM + wave_n * TN + frow;
    const int aoff = 64 * (ra & ~1), woff = 64 * (rw & ~1);
    const int ha = 4 * (ra & 1) + g, hw = 4 * (rw & 1) + g;
    const int sw_a = tline_sw(ra), sw_w = tline_sw(rw);
    half8_t fa[2][FM], fw[2][FN];
    auto read_frags = [&](const uint8_t* t, int kk, int slot) {
#pragma unroll
        for (int i = 0; i < FM; i++)
            fa[slot][i] = *(const half8_t*)(t + aoff + 2048 * i + 16 * ((ha + 2 * kk) ^ sw_a));
#pragma unroll
        for (int j = 0; j < FN; j++)
            fw[slot][j] = *(const half8_t*)(t + woff + 2048 * j + 16 * ((hw + 2 * kk) ^ sw_w));
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[slot][i], fw[slot][j], acc[i][j], 0, 0, 0);
    };

    // ---- prologue: scale groups 0 and 1 in registers, code groups 0 and 1
    // staged, stage 0 decoded
    load_scales(0, sc_cur);
    load_scales(nsg > 1 ? 1 : 0, sc_nxt);
    issue_group(0, IntC<0>{}, IntC<0>{}, IntC<NJ>{});
    issue_group(ngr > 1 ? 1 : 0, IntC<1>{}, IntC<0>{}, IntC<NJ>{});
    wait_vm<0>();
    __syncthreads();
    stage_codes(IntC<0>{});
    decode_stage(IntC<0>{}, sc_cur);
    stage_codes(IntC<1>{});
    __syncthreads();
    read_frags(lds_f[0], 0, 0);

    // ---- stage s, T = s mod 8 (compile time): k-step 0 (fragments read
    // last stage) with the decode of stage s+1, barrier, k-step 1 with the
    // first fragment reads of stage s+1
    auto stage = [&](int64_t s, auto t_tag) {
        constexpr int T = decltype(t_tag)::value;
        constexpr int CUR = T & 1;
        constexpr int TN1 = (T + 1) & 7;  // stage s+1 mod 8
        // Group G + 2 is copied into the staging buffer of group G (free
        // from stage 4 G + 3 on) during stages 4 G + 3 .. 4 G + 5, three
        // copies per stage spread between the MFMAs so the address unit never
        // backs up, and awaited at stage 4 G + 6.  Past the last group the
        // copies repeat the last group into the free buffer (harmless), which
        // keeps the stage straight-line code.
        constexpr bool CP = T != 2 && T != 6;
        constexpr int PH = (T + 5) & 3;  // 0, 1, 2 for T = 3, 4, 5 (and 7, 0, 1)
        constexpr int BUF = (T >= 3 && T <= 5) ? 0 : 1;
        // copies [C0, C1) go between the first k-step's MFMAs, [C1, C2)
        // between the second's (the first stage of a window: all three in
        // its second k-step, which has no decode work)
        constexpr int C0 = 3 * PH < NJ ? 3 * PH : NJ;
        constexpr int C1 = PH == 0 ? C0 : (3 * PH + 1 < NJ ? 3 * PH + 1 : NJ);
        constexpr int C2 = 3 * PH + 3 < NJ ? 3 * PH + 3 : NJ;
        int64_t G2 = ((s + 1) >> 2) + 1;
        G2 = G2 < ngr ? G2 : ngr - 1;
        if (T == 4) {
            // scales of the next group: the previous one moved in at T == 0
            if ((s >> 3) + 1 < nsg)
                load_scales((s >> 3) + 1, sc_nxt);
        }
        read_frags(lds_f[CUR], 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(0);
        if (T == 7)
            decode_stage(IntC<TN1>{}, sc_nxt);
        else
            decode_stage(IntC<TN1>{}, sc_cur);
        if (CP && C1 > C0)
            issue_group(G2, IntC<BUF>{}, IntC<C0>{}, IntC<C1>{});
#pragma unroll
        for (int m = 0; m < FM * FN; m++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);      // VALU
            if (m % 2 == 1)
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
            if (CP && C1 > C0 && m == 7)
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (copy)
        }
        __builtin_amdgcn_sched_barrier(0);
        if (T == 2 || T == 6)
            wait_vm<0>();  // the next group's codes (copied 3 stages ago) and scales
        wait_lgkm0();      // (tells the compiler the barrier's wait happened)
        lds_barrier();
        // the codes stage s+1 decodes (stage s+2, visible since this
        // barrier) and the first fragments of stage s+1
        stage_codes(IntC<(T + 2) & 7>{});
        read_frags(lds_f[CUR ^ 1], 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(1);
        if (CP && C2 > C1)
            issue_group(G2, IntC<BUF>{}, IntC<C1>{}, IntC<C2>{});
        if (CP && C2 - C1 == 3) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (copy)
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        } else if (CP && C2 - C1 == 2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
        } else if (CP && C2 - C1 == 1) {
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // those reads have landed under the MFMAs: retire them so the next
        // stage starts with an empty LDS counter and decodes without a wait
        wait_lgkm0();
        if (T == 7) {
#pragma unroll
            for (int i = 0; i < RPT; i++)
                sc_cur[i] = sc_nxt[i];
        }
    };
    // The loop body runs stages 3..10 mod 8: its back edge follows the wait
    // at T == 2, where no copy is in flight, so the compiler's wait
    // bookkeeping stays exact around the loop.
    stage(0, IntC<0>{});
    stage(1, IntC<1>{});
    if (nst > 2)
        stage(2, IntC<2>{});
    wait_vm<0>();  // no-op after stage 2; keeps the wait bookkeeping exact on both paths
    int64_t s = 3;
    for (; s + 8 <= nst; s += 8) {
        stage(s, IntC<3>{});
        stage(s + 1, IntC<4>{});
        stage(s + 2, IntC<5>{});
        stage(s + 3, IntC<6>{});
        stage(s + 4, IntC<7>{});
        stage(s + 5, IntC<0>{});
        stage(s + 6, IntC<1>{});
        stage(s + 7, IntC<2>{});
    }
    if (s < nst)
        stage(s, IntC<3>{});
    if (s + 1 < nst)
        stage(s + 1, IntC<4>{});
    if (s + 2 < nst)
        stage(s + 2, IntC<5>{});
    if (s + 3 < nst)
        stage(s + 3, IntC<6>{});
    if (s + 4 < nst)
        stage(s + 4, IntC<7>{});
    if (s + 5 < nst)
        stage(s + 5, IntC<0>{});
    if (s + 6 < nst)
        stage(s + 6, IntC<1>{});
    store_tile<BN, WM, WN, TM, TN, FM, FN, MODE>(p, tc, acc, wave_m, wave_n, lane, &lds_f[0][0]);
}

// Epilogue of gemm_rtile_kernel, whose MFMAs take the W fragment as the
// first operand: acc[i][j] is the transposed 32x32 fragment, lane l holding
// output row 32 i + l % 32 of the wave tile and, in element 4 q + t, output
// column 32 j + 8 q + 4 (l / 32) + t.  Each pass stages up to 128 bytes of
// every wave row in this wave's own LDS region (TM rows; 16-byte slot s of row
// r at slot s ^ (r % 8)) and writes whole 16-byte pieces: 8 lanes per row, 8
// rows per store instruction (gate_up with 64-column wave tiles: 4 lanes per
// row of 32 h columns, 16 rows).  The output is not read again by this
// launch: nontemporal stores, so that a round's output (4-8 MB per XCD)
// does not push out the operand lines the resident tiles share in L2
// (384-expert prefill: down 3108 -> 2985 us, gate_up 5159 -> 5115 us).
template <int BN, int TM, int TN, int FM, int FN, int MODE>
NVFP4_DEV void store_tile_t(const GemmArgs& p, const TileCoord& tc, const float16_t (&acc)[FM][FN], int wave_m,
                            int wave_n, int lane, uint8_t* stg)
{
    const float gscale = *p.a_global * p.w_global[tc.e];
    const int mrow = lane & 31, g = lane >> 5;
    const int64_t wrow0 = tc.row_begin + wave_m * TM;  // first output row of this wave
    const int rows_left = (int)(tc.row_end - wrow0);
    const int64_t N = p.N;
    auto slot = [&](int r, int s) { return stg + r * 128 + 16 * (s ^ (r & 7)); };
    const int rl = lane >> 3, sl = lane & 7;  // read-back: row 8 k + rl, slot sl
    auto staged = [&]() {
        // LDS operations of a wave complete in order; the fence keeps the
        // compiler from moving the reads of other lanes' data above the writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    if constexpr (MODE == kModeGateUp) {
        // h = silu(gate) * up, bf16: TN / 2 columns (64 or 32: 128 or 64
        // bytes) per wave row
        constexpr int HS = TN / 16;  // 16-byte slots of h per wave row (64 or 32 columns)
        static_assert(HS == 8 || HS == 4, "one pass holds the wave's h columns");
        const int64_t hcol0 = tc.nt * (BN / 2) + wave_n * (TN / 2);
        uint32_t hmax = 0;
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const bool rv = 32 * i + mrow < rows_left;
#pragma unroll
            for (int j = 0; j < FN / 2; j++) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    uint32_t hb[4];
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        const float gg = acc[i][j][4 * q + t] * gscale;
                        const float uu = acc[i][j + FN / 2][4 * q + t] * gscale;
                        hb[t] = f32_to_bf16(silu_f(gg) * uu);
                        const uint32_t mag = rv ? (hb[t] & 0x7FFFu) : 0u;
                        hmax = hmax > mag ? hmax : mag;
                    }
                    // columns 32 j + 8 q + 4 g + t: bytes 64 j + 16 q + 8 g
                    *(u32x2*)(slot(32 * i + mrow, 4 * j + q) + 8 * g) = (u32x2){hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
                }
            }
        }
        staged();
        if (p.hq_global) {
            // h straight to NVFP4: each lane encodes whole 16-element blocks
            // (row b / 4, columns 16 (b % 4)) as the quantize kernel does
            const float Gh = *p.hq_global, six = 6.0f * Gh;
            for (int b = lane; b < TM * (HS / 2); b += 64) {
                const int r = b / (HS / 2), c16 = b % (HS / 2);
                if (r < rows_left) {
                    const u32x4 v0 = *(const u32x4*)slot(r, 2 * c16);
                    const u32x4 v1 = *(const u32x4*)slot(r, 2 * c16 + 1);
                    const uint32_t a0 = absmax_bits8(v0), a1 = absmax_bits8(v1);
                    uint32_t sc;
                    const float rcp = block_scale(a0 > a1 ? a0 : a1, Gh, six, &sc);
                    const int64_t grow = wrow0 + r, col = hcol0 + 16 * c16;
                    *(u32x2*)(p.hq_packed + grow * (N / 2) + col / 2) =
                        (u32x2){encode_half(v0, rcp), encode_half(v1, rcp)};
                    p.hq_scales[grow * (N / 16) + col / 16] = (uint8_t)sc;
                }
            }
        } else {
            uint16_t* h = (uint16_t*)p.out;
            constexpr int RPI = 64 / HS;  // rows per store instruction
            const int hr = lane / HS, hs = lane % HS;
#pragma unroll
            for (int k = 0; k < TM / RPI; k++) {
                const int r = RPI * k + hr;
                if (r < rows_left)
                    __builtin_nontemporal_store(*(const u32x4*)slot(r, hs),
                                                (u32x4*)(h + (wrow0 + r) * N + hcol0 + 8 * hs));
            }
            // one atomic per workgroup: the four waves meet in LDS first
            __shared__ uint32_t red[16];
            hmax = block_max_u32(hmax, red);
            if (threadIdx.x == 0 && hmax != 0)
                atomicMax(p.h_amax, hmax << 16);
        }
    } else {
        const bool bf16_out = MODE == kModeDense && p.out_bf16;
        const int64_t colw = tc.nt * BN + wave_n * TN;  // first output column of the wave
        if (bf16_out) {
            // passes over pairs of W fragments: 64 columns = 128 bytes per row
            const bool vec = N % 8 == 0 && ((uintptr_t)p.out & 15) == 0;
            uint16_t* ob = (uint16_t*)p.out;
#pragma unroll
            for (int jp = 0; jp < FN / 2; jp++) {
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int jj = 0; jj < 2; jj++)
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const float16_t& a = acc[i][2 * jp + jj];
                            const uint32_t b0 = f32_to_bf16(a[4 * q] * gscale), b1 = f32_to_bf16(a[4 * q + 1] * gscale);
                            const uint32_t b2 = f32_to_bf16(a[4 * q + 2] * gscale), b3 = f32_to_bf16(a[4 * q + 3] * gscale);
                            *(u32x2*)(slot(32 * i + mrow, 4 * jj + q) + 8 * g) = (u32x2){b0 | (b1 << 16), b2 | (b3 << 16)};
                        }
                staged();
#pragma unroll
                for (int k = 0; k < TM / 8; k++) {
                    const int r = 8 * k + rl;
                    const int64_t col = colw + 64 * jp + 8 * sl;
                    if (r < rows_left && col < N) {
                        const u32x4 v = *(const u32x4*)slot(r, sl);
                        uint16_t* dst = ob + (wrow0 + r) * N + col;
                        if (vec) {
                            __builtin_nontemporal_store(v, (u32x4*)dst);
                        } else {
                            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                            for (int t = 0; t < 8; t++)
                                if (col + t < N)
                                    dst[t] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
                        }
                    }
                }
                staged();
            }
        } else {
            // fp32: one pass per W fragment, 32 columns = 128 bytes per row
            const bool vec = N % 4 == 0 && ((uintptr_t)p.out & 15) == 0;
            float* of = (float*)p.out;
#pragma unroll
            for (int j = 0; j < FN; j++) {
#pragma unroll
                for (int i = 0; i < FM; i++)
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const float16_t& a = acc[i][j];
                        *(float4_t*)slot(32 * i + mrow, 2 * q + g) =
                            (float4_t){a[4 * q] * gscale, a[4 * q + 1] * gscale, a[4 * q + 2] * gscale,
                                       a[4 * q + 3] * gscale};
                    }
                staged();
#pragma unroll
                for (int k = 0; k < TM / 8; k++) {
                    const int r = 8 * k + rl;
                    const int64_t col = colw + 32 * j + 4 * sl;
                    if (r < rows_left && col < N) {
                        const float4_t v = *(const float4_t*)slot(r, sl);
                        float* dst = of + (wrow0 + r) * N + col;
                        if (vec) {
                            __builtin_nontemporal_store(v, (float4_t*)dst);
                        } else {
#pragma unroll
                            for (int t = 0; t < 4; t++)
                                if (col + t < N)
                                    dst[t] = v[t];
                        }
                    }
                }
                staged();
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill mainloop with register decode (K a multiple of 256).
//
// Same tiles, waves and MFMA as gemm_tile_kernel, but no f16 tile in LDS:
// every wave reads the packed codes of its own fragment rows from the LDS
// staging and decodes them straight into MFMA operand registers.  Measured
// on one wave per SIMD: a 16-byte LDS write stalls the issuing wave's MFMA
// stream by about 35 cycles when VALU work is interleaved, while up to four
// conversions per 32x32x16 MFMA issue in its shadow for free.  Decoding per
// wave repeats each row's decode on the two waves that share it, which stays
// within that budget, and removes the f16 writes, the f16 fragment reads and
// three of every four barriers.
//
// K is walked in groups of 128 elements.  Inside a group the K order of the
// MFMA is permuted identically for A and W: lane half g (lane / 32) of
// k-step j (0..7) takes the 8 elements of dword j % 4 of 16-byte chunk
// g + 2 (j / 4) of the row's 64 code bytes, so each lane reads one chunk per
// row per four k-steps, and those 32 elements share two scale bytes.  Codes
// are copied by the LDS DMA path into four group buffers (layout tpos), two
// groups ahead; the scale bytes of a pair of groups (16 per row) go to two
// pair buffers.  One barrier per group, after its fourth k-step, publishes
// the next group's staging (each wave first waits for its own copies) and
// frees the buffer that the group after next is copied into.  Every buffer
// is its own LDS array so that reads from one never wait for copies into
// another.
// ---------------------------------------------------------------------------
constexpr int kRGrpK = 128;  // K elements per group

// true when f maps 0..n-1 onto 0..n-1 one to one
template <class F>
constexpr bool rt_is_perm(F f, int n)
{
    for (int v = 0; v < n; v++) {
        int hits = 0;
        for (int x = 0; x < n; x++)
            hits += f(x) == v;
        if (hits != 1)
            return false;
    }
    return true;
}

template <int BM, int BN, int MODE, bool P2>
__global__ void __launch_bounds__(256)
gemm_rtile_kernel(GemmArgs p)
{
    constexpr int WM = 2, WN = 2, NW = 4;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int NJ = (ROWS + 16 * NW - 1) / (16 * NW);  // code copies per wave per group
    constexpr int SROWS = NJ * NW * 16;                    // staged code rows (>= ROWS)
    constexpr int NS = (ROWS + 64 * NW - 1) / (64 * NW);   // scale copies per wave per group pair
    constexpr int SSROWS = NS * NW * 64;                   // staged scale rows (>= ROWS)
    constexpr int CB = SROWS * kTGRow;                     // bytes per code buffer
    static_assert(BM % 64 == 0 && BN % 64 == 0 && NJ % 2 == 0, "tile shape");
    static_assert(MODE != kModeGateUp || FN % 2 == 0, "gate_up pairs gate and up fragments");

    __shared__ __attribute__((aligned(16))) uint8_t lds_c0[CB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_c1[CB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_c2[CB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_c3[CB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_s0[SSROWS * 16];
    __shared__ __attribute__((aligned(16))) uint8_t lds_s1[SSROWS * 16];
    auto cbuf = [&](auto b_tag) -> uint8_t* {
        constexpr int B = decltype(b_tag)::value & 3;
        return B == 0 ? lds_c0 : B == 1 ? lds_c1 : B == 2 ? lds_c2 : lds_c3;
    };
    auto sbuf = [&](auto b_tag) -> uint8_t* { return (decltype(b_tag)::value & 1) ? lds_s1 : lds_s0; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;

    TileCoord tc;
    if (!tile_coord<BM, MODE>(p, tc))
        return;
    const int e = tc.e;
    const int64_t K = p.K;
    const int64_t kpb = K / 2, kpsb = K / 16;  // packed / scale bytes per row
    const int64_t w_rows = (MODE == kModeGateUp) ? 2 * p.N : p.N;
    const uint8_t* wp = p.w_packed + (int64_t)e * w_rows * kpb;
    const uint8_t* wsc = p.w_scales + (int64_t)e * w_rows * kpsb;
    auto matrix_row = [&](int r) -> int64_t {
        return r < BM ? tile_a_row<MODE>(p, tc, r) : tile_w_row<BN, TN, MODE>(p, tc, r - BM);
    };
    const int64_t ngr = K / kRGrpK;  // even
    const int64_t npr = ngr / 2;

    // ---- code copies: copy j of this wave fills bytes [1024 (NJ wave + j),
    // +1024) of a group buffer, lane l the 16 bytes at 16 l: line
    // q = 8 (NJ wave + j) + l / 8, slot l % 8, i.e. the (row, chunk) that tpos
    // places there
    int32_t srow[NJ];
    int scq[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        const int q = 8 * (NJ * wave + j) + (lane >> 3);
        const int hc = (lane & 7) ^ ((q ^ (q >> 1)) & 7);  // 4 (r % 2) + c
        int r = 2 * q + (hc >> 2);
        if (r >= ROWS)
            r = ROWS - 1;
        srow[j] = (int32_t)matrix_row(r);
        scq[j] = hc & 3;
    }
    // ---- scale copies: copy j of this wave fills 16-byte row slots
    // [64 (NS wave + j), +64) of a pair buffer with the 16 scale bytes of a
    // pair of groups (slots past the last row repeat it)
    // (a copy's 64 rows are all A rows or all W rows: BM % 64 == 0)
    const uint8_t* ssrc[NS];
    int64_t sstep[NS];  // scale bytes from one group pair to the next
#pragma unroll
    for (int j = 0; j < NS; j++) {
        int r = 64 * (NS * wave + j) + lane;
        if (r >= ROWS)
            r = ROWS - 1;
        ssrc[j] = r < BM ? p.a_scales + matrix_row(r) * kpsb : w_scale_row(wsc, matrix_row(r), K, p.w_tiled);
        sstep[j] = r < BM ? 16 : w_scale_step(p.w_tiled);
    }
    // copies [J0, J1) of the codes of group G (clamped to the last) into buffer B
    auto issue_codes = [&](int64_t G, auto b_tag, auto j0_tag, auto j1_tag) {
        constexpr int J0 = decltype(j0_tag)::value, J1 = decltype(j1_tag)::value;
        const int64_t cb = (G < ngr ? G : ngr - 1) * kTGRow;
        uint8_t* dst = cbuf(b_tag);
#pragma unroll
        for (int j = J0; j < J1; j++) {
            const bool is_a = 16 * (NJ * wave + j) < BM;  // uniform per copy
            const uint8_t* src = (is_a ? p.a_packed : wp) + (int64_t)srow[j] * kpb + cb + 16 * scq[j];
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)(dst + (NJ * wave + j) * 1024), 16,
                                             0, 0);
        }
    };
    // the scale copies of group pair Q (clamped to the last) into pair buffer B
    auto issue_scales = [&](int64_t Q, auto b_tag) {
        const int64_t q = Q < npr ? Q : npr - 1;
        uint8_t* dst = sbuf(b_tag);
#pragma unroll
        for (int j = 0; j < NS; j++)
            __builtin_amdgcn_global_load_lds((const void*)(ssrc[j] + q * sstep[j]),
                                             (lds_ptr_t)(dst + (NS * wave + j) * 1024), 16, 0, 0);
    };

    // ---- this lane's fragment rows: A rows ra + 32 i, W rows rw + 32 j.
    // They differ by multiples of 32, which keeps the line swizzle and the
    // row parity, so one chunk offset per half serves all of them.
    const int frow = lane & 31;
    const int g = lane >> 5;
    const int ra = wave_m * TM + frow, rw = BM + wave_n * TN + frow;
    const int lsw = tline_sw(frow), par = frow & 1;
    const int aoff0 = 64 * (ra & ~1) + 16 * ((4 * par + g) ^ lsw);
    const int aoff1 = 64 * (ra & ~1) + 16 * ((4 * par + g + 2) ^ lsw);
    const int woff0 = 64 * (rw & ~1) + 16 * ((4 * par + g) ^ lsw);
    const int woff1 = 64 * (rw & ~1) + 16 * ((4 * par + g + 2) ^ lsw);
    const uint32_t sshift = 16 * g;  // this lane's two scale bytes of a chunk

    u32x4 cA[FM], cW[FN];  // codes, chunk g of the group (k-steps 0-3)
    u32x4 hA[FM], hW[FN];  // codes, chunk g + 2 (k-steps 4-7)
    u32x2 sA[FM], sW[FN];  // scale bytes of the group (8 per row)
    u32x2 nA[FM], nW[FN];  // ... of the next group
    half2_t vA[FM];        // f16 scales of the two blocks of the current chunk
    half2_t vWh[FN];       // (W, general scales)
    float vW0[FN], vW1[FN];  // (W, power-of-two scales: the conversion's operand)
    uint32_t oa[2][FM][4], ow[2][FN][4];  // MFMA operands (8 f16 each), two sets

    // MFMA slot m of a k-step is followed by decode units [U0(m), U0(m+1)):
    // unit u decodes half u % 2 (4 of the 8 f16) of operand row u / 2, rows
    // taken A, W, A, W, ... then the remaining W rows
    constexpr int NM = FM * FN, NU = 2 * (FM + FN);
    constexpr auto unit_row = [](int rho) { return rho < 2 * FM ? ((rho & 1) ? FM + (rho >> 1) : (rho >> 1)) : rho; };
    static_assert(rt_is_perm(unit_row, FM + FN), "decode units cover every operand row once");

    // scale values of half H of a group for row R (A rows 0..FM-1, then W)
    auto prep_row = [&](auto h_tag, auto r_tag, const u32x2 (&ba)[FM], const u32x2 (&bw)[FN]) {
        constexpr int H = decltype(h_tag)::value, R = decltype(r_tag)::value;
        if constexpr (R < FM) {
            vA[R] = scales2<0>((H ? ba[R].y : ba[R].x) >> sshift);
        } else {
            constexpr int J = R - FM;
            const uint32_t w = (H ? bw[J].y : bw[J].x) >> sshift;
            if (P2) {
                vW0[J] = __builtin_amdgcn_cvt_f32_fp8(w, 0);
                vW1[J] = __builtin_amdgcn_cvt_f32_fp8(w, 1);
            } else {
                vWh[J] = scales2<0>(w);
            }
        }
    };
    // decode unit U of k-step KS into operand set S
    auto decode_unit = [&](auto ks_tag, auto s_tag, auto u_tag) {
        constexpr int KS = decltype(ks_tag)::value & 7, S = decltype(s_tag)::value, U = decltype(u_tag)::value;
        constexpr int R = unit_row(U >> 1), HF = U & 1, D = KS & 3;
        if constexpr (R < FM) {
            const u32x4 c = KS < 4 ? cA[R] : hA[R];
            const uint32_t cw = D == 0 ? c.x : D == 1 ? c.y : D == 2 ? c.z : c.w;
            const _Float16 sc = (D >> 1) ? vA[R].y : vA[R].x;
            const half2_t ss = {sc, sc};
            oa[S][R][2 * HF] =
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2 * HF) * ss);
            oa[S][R][2 * HF + 1] =
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2 * HF + 1) * ss);
        } else {
            constexpr int J = R - FM;
            const u32x4 c = KS < 4 ? cW[J] : hW[J];
            const uint32_t cw = D == 0 ? c.x : D == 1 ? c.y : D == 2 ? c.z : c.w;
            if (P2) {
                const float sc = (D >> 1) ? vW1[J] : vW0[J];
                ow[S][J][2 * HF] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 2 * HF));
                ow[S][J][2 * HF + 1] =
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 2 * HF + 1));
            } else {
                const _Float16 sc = (D >> 1) ? vWh[J].y : vWh[J].x;
                const half2_t ss = {sc, sc};
                ow[S][J][2 * HF] =
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2 * HF) * ss);
                ow[S][J][2 * HF + 1] =
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2 * HF + 1) * ss);
            }
        }
    };
    auto operand = [](const uint32_t (&o)[4]) { return __builtin_bit_cast(half8_t, (u32x4){o[0], o[1], o[2], o[3]}); };

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            acc[i][j] = (float16_t){};

    // One k-step: MFMA slot m of operand set S, then the decode units of
    // slot m for k-step KN into set S ^ 1 (preceded, at a row's first unit,
    // by that row's scale values of half PH when PH >= 0: half 1 from this
    // group's bytes, half 0 from the next group's), then extra(m) (LDS reads
    // or copies placed at that slot).  The fences keep this order.
    auto kstep = [&](auto s_tag, auto kn_tag, auto ph_tag, auto&& extra) {
        constexpr int S = decltype(s_tag)::value, PH = decltype(ph_tag)::value;
        static_for<NM>([&](auto m_tag) {
            constexpr int m = decltype(m_tag)::value;
            constexpr int i = m / FN, j = m % FN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(operand(ow[S][j]), operand(oa[S][i]), acc[i][j], 0, 0, 0);
            static_for<(m + 1) * NU / NM - m * NU / NM>([&](auto k_tag) {
                constexpr int U = m * NU / NM + decltype(k_tag)::value;
                if constexpr (PH >= 0 && (U & 1) == 0) {
                    if constexpr (PH == 1)
                        prep_row(IntC<1>{}, IntC<unit_row(U >> 1)>{}, sA, sW);
                    else
                        prep_row(IntC<0>{}, IntC<unit_row(U >> 1)>{}, nA, nW);
                }
                decode_unit(kn_tag, IntC<S ^ 1>{}, IntC<U>{});
            });
            extra(m_tag);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto none = [](auto) {};

    // ---- prologue: group 0 and scale pair 0 staged (group 1 in flight),
    // group 0 read, the first half of the copies of group 2 and scale pair 1
    // issued, the operands of k-step 0 decoded
    issue_codes(0, IntC<0>{}, IntC<0>{}, IntC<NJ>{});
    issue_scales(0, IntC<0>{});
    issue_codes(1, IntC<1>{}, IntC<0>{}, IntC<NJ>{});
    wait_vm<NJ>();  // group 0 and scale pair 0 (group 1 is awaited at the first barrier)
    lds_barrier();
#pragma unroll
    for (int i = 0; i < FM; i++)
        cA[i] = *(const u32x4*)(lds_c0 + aoff0 + 2048 * i);
#pragma unroll
    for (int j = 0; j < FN; j++)
        cW[j] = *(const u32x4*)(lds_c0 + woff0 + 2048 * j);
#pragma unroll
    for (int i = 0; i < FM; i++)
        nA[i] = *(const u32x2*)(lds_s0 + 16 * (ra + 32 * i));
#pragma unroll
    for (int j = 0; j < FN; j++)
        nW[j] = *(const u32x2*)(lds_s0 + 16 * (rw + 32 * j));
    issue_codes(2, IntC<2>{}, IntC<0>{}, IntC<NJ / 2>{});
    issue_scales(1, IntC<1>{});
    static_for<NU>([&](auto u_tag) {
        constexpr int U = decltype(u_tag)::value;
        if constexpr ((U & 1) == 0)
            prep_row(IntC<0>{}, IntC<unit_row(U >> 1)>{}, nA, nW);
        decode_unit(IntC<0>{}, IntC<0>{}, u_tag);
    });
#pragma unroll
    for (int i = 0; i < FM; i++)
        sA[i] = nA[i];
#pragma unroll
    for (int j = 0; j < FN; j++)
        sW[j] = nW[j];
    __builtin_amdgcn_sched_barrier(0);

    // ---- group G with T = G mod 4 (compile time): buffers, copy targets and
    // wait counts follow from T
    constexpr int NH = NJ / 2;
    constexpr int CPS = NM / 2;  // the slot that carries a k-step's copies
    auto group = [&](int64_t G, auto t_tag) {
        constexpr int T = decltype(t_tag)::value;
        constexpr int T1 = (T + 1) & 3;
        const uint8_t* cb = cbuf(IntC<T>{});
        const uint8_t* cb1 = cbuf(IntC<T1>{});
        const uint8_t* sb1 = sbuf(IntC<(T1 >> 1)>{}) + 8 * (T1 & 1);
        // copies [CK(q), CK(q+1)) of a half window go with its k-step q of 4
#define RT_CK(q) (((q) * NH) / 4)
        // k-step 0, with the reads of the chunk g + 2 codes of this group
        kstep(IntC<0>{}, IntC<1>{}, IntC<-1>{}, [&](auto m_tag) {
            constexpr int m = decltype(m_tag)::value;
            if constexpr (m < FM)
                hA[m] = *(const u32x4*)(cb + aoff1 + 2048 * m);
            else if constexpr (m < FM + FN)
                hW[m - FM] = *(const u32x4*)(cb + woff1 + 2048 * (m - FM));
            if constexpr (m == CPS)
                issue_codes(G + 2, IntC<(T + 2) & 3>{}, IntC<NH + RT_CK(0)>{}, IntC<NH + RT_CK(1)>{});
        });
        kstep(IntC<1>{}, IntC<2>{}, IntC<-1>{}, [&](auto m_tag) {
            if constexpr (decltype(m_tag)::value == CPS)
                issue_codes(G + 2, IntC<(T + 2) & 3>{}, IntC<NH + RT_CK(1)>{}, IntC<NH + RT_CK(2)>{});
        });
        kstep(IntC<0>{}, IntC<3>{}, IntC<-1>{}, [&](auto m_tag) {
            if constexpr (decltype(m_tag)::value == CPS)
                issue_codes(G + 2, IntC<(T + 2) & 3>{}, IntC<NH + RT_CK(2)>{}, IntC<NH + RT_CK(3)>{});
        });
        kstep(IntC<1>{}, IntC<4>{}, IntC<1>{}, [&](auto m_tag) {
            if constexpr (decltype(m_tag)::value == CPS)
                issue_codes(G + 2, IntC<(T + 2) & 3>{}, IntC<NH + RT_CK(3)>{}, IntC<NJ>{});
        });
        // group G + 1 was copied a whole window ago; the copies of group G + 2
        // (and, for even G, of scale pair G / 2 + 1) may stay in flight
        wait_vm<NJ + ((T & 1) == 0 ? NS : 0)>();
        wait_lgkm0();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // k-step 4, with the reads of group G + 1 (chunk g, scales) and the
        // first copies of group G + 3 (and, for odd G, scale pair (G + 3) / 2)
        kstep(IntC<0>{}, IntC<5>{}, IntC<-1>{}, [&](auto m_tag) {
            constexpr int m = decltype(m_tag)::value;
            constexpr int q = m / 2;
            if constexpr ((m & 1) == 0 && q < FM)
                cA[q] = *(const u32x4*)(cb1 + aoff0 + 2048 * q);
            else if constexpr ((m & 1) == 0 && q < FM + FN)
                cW[q - FM] = *(const u32x4*)(cb1 + woff0 + 2048 * (q - FM));
            if constexpr ((m & 1) == 1 && q < FM)
                nA[q] = *(const u32x2*)(sb1 + 16 * (ra + 32 * q));
            else if constexpr ((m & 1) == 1 && q < FM + FN)
                nW[q - FM] = *(const u32x2*)(sb1 + 16 * (rw + 32 * (q - FM)));
            if constexpr (m == CPS)
                issue_codes(G + 3, IntC<(T + 3) & 3>{}, IntC<RT_CK(0)>{}, IntC<RT_CK(1)>{});
            if constexpr (m == CPS + 1 && (T & 1))
                issue_scales((G + 3) >> 1, IntC<(((T + 3) >> 1) & 1)>{});
        });
        if constexpr (2 * (FM + FN) > NM) {
            // rows left over when a k-step has fewer slots than reads
#pragma unroll
            for (int q = NM / 2; q < FM + FN; q++) {
                if (q < FM) {
                    cA[q] = *(const u32x4*)(cb1 + aoff0 + 2048 * q);
                    nA[q] = *(const u32x2*)(sb1 + 16 * (ra + 32 * q));
                } else {
                    cW[q - FM] = *(const u32x4*)(cb1 + woff0 + 2048 * (q - FM));
                    nW[q - FM] = *(const u32x2*)(sb1 + 16 * (rw + 32 * (q - FM)));
                }
            }
        }
        kstep(IntC<1>{}, IntC<6>{}, IntC<-1>{}, [&](auto m_tag) {
            if constexpr (decltype(m_tag)::value == CPS)
                issue_codes(G + 3, IntC<(T + 3) & 3>{}, IntC<RT_CK(1)>{}, IntC<RT_CK(2)>{});
        });
        kstep(IntC<0>{}, IntC<7>{}, IntC<-1>{}, [&](auto m_tag) {
            if constexpr (decltype(m_tag)::value == CPS)
                issue_codes(G + 3, IntC<(T + 3) & 3>{}, IntC<RT_CK(2)>{}, IntC<RT_CK(3)>{});
        });
        // k-step 7 decodes k-step 0 of group G + 1 (past the end: unused)
        kstep(IntC<1>{}, IntC<0>{}, IntC<0>{}, [&](auto m_tag) {
            if constexpr (decltype(m_tag)::value == CPS)
                issue_codes(G + 3, IntC<(T + 3) & 3>{}, IntC<RT_CK(3)>{}, IntC<NH>{});
        });
#undef RT_CK
#pragma unroll
        for (int i = 0; i < FM; i++)
            sA[i] = nA[i];
#pragma unroll
        for (int j = 0; j < FN; j++)
            sW[j] = nW[j];
    };
    (void)none;
    int64_t G = 0;
    for (; G + 4 <= ngr; G += 4) {
        group(G, IntC<0>{});
        group(G + 1, IntC<1>{});
        group(G + 2, IntC<2>{});
        group(G + 3, IntC<3>{});
    }
    if (G < ngr) {
        group(G, IntC<0>{});
        group(G + 1, IntC<1>{});
    }
    // copies past the end are still in flight into the buffers; after the
    // barrier every wave stages its output in its own part of two buffers
    wait_vm<0>();
    __syncthreads();
    static_assert(2 * TM * 128 <= CB, "two waves' output staging fits one code buffer");
    store_tile_t<BN, TM, TN, FM, FN, MODE>(p, tc, acc, wave_m, wave_n, lane,
                                           (wave < 2 ? lds_c0 : lds_c1) + (wave & 1) * TM * 128);
}

}  // namespace nvfp4

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Weight-streaming W4A4 GEMM for few A rows (decode batches: 16 A rows per
// tile).
//
// With few A rows the GEMM is bound by reading the 4-bit weights, so each
// weight byte is read from HBM once, in whole 128-byte lines, and decoded
// once.  A workgroup of 4 waves owns 128 W rows (32 per wave, as two 16-row
// fragments of v_mfma_f32_16x16x32_f16) and walks K in stages of 256
// elements.  Each thread loads 16-byte pieces so that 8 consecutive lanes
// cover one row's 128 bytes of a stage; the pieces sit in registers two
// stages ahead, then go to a swizzled LDS tile from which every lane reads
// the codes of its own row.  The few A rows are decoded once per workgroup
// into an f16 LDS tile.  Inside a stage the K order is permuted the same way
// for both operands: k-step kk = 4 q + d (q < 2, d < 4) gives lane group
// kg = lane / 16 the stage elements [128 q + 32 kg + 8 d, +8).  When the
// tiles alone cannot fill the chip, K is split over several workgroups and a
// second kernel adds their partial sums in a fixed order.
//
// The grid is persistent: as many workgroups as the chip holds at once, each
// walking a list of (tile, K split) items with one register pipeline that
// runs on from the last stages of one item into the first of the next, so
// that the weight stream never waits for a new workgroup to start.  Item
// set-up reads its tables (tile offsets, list positions) with scalar loads,
// which are counted apart from the vector loads in flight.
// ---------------------------------------------------------------------------
constexpr int kSkBK = 256;               // K elements per stage
constexpr int kSkRowF16 = kSkBK * 2;     // f16 A-tile bytes per row per stage
constexpr int kSkBM = 16;                // A rows per tile
constexpr int kSkBN = 128;               // W rows per workgroup
constexpr int kSkThreads = 256;

// 16-byte slot of piece c (of 8) in W tile row r: rows r and r + 1 fall in
// different halves of the banks, and the 8 even (odd) rows of a 16-row
// fragment get 8 different slots, so a 16-lane read phase is conflict free.
NVFP4_DEV int sk_wslot(int r, int c) { return c ^ ((r >> 1) & 7); }
// 16-byte slot of f16 chunk c (of 32) in A tile row r
NVFP4_DEV int sk_aslot(int r, int c) { return c ^ (r & 15); }

template <int MODE, bool P2, bool A16, int SBM>
__global__ void __launch_bounds__(kSkThreads)
gemm_stream_kernel(GemmArgs p)
{
    static_assert(SBM == 16 || SBM == 32, "16- or 32-row A tiles");
    constexpr int BM = SBM, BN = kSkBN;
    constexpr int NA = BM / 16;           // A fragments (MFMA 16 x 16 x 32 rows) per tile
    constexpr bool kAllA = BM == 32;      // every thread loads a piece of the A tile
    __shared__ __attribute__((aligned(16))) uint8_t lds_w[2][BN * 128];        // codes, 2 x 16 KiB
    __shared__ __attribute__((aligned(16))) uint8_t lds_ws[2][BN * 16];        // scales, 2 x 2 KiB
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kSkRowF16];  // f16 A, 2 x 8 KiB

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int fr = lane & 15, kg = lane >> 4;

    // ---- work items (A tile, K split, W tile), the A tile varying fastest.
    // The grid is resident (a multiple of 8, at most what the chip holds) and
    // each workgroup walks its items with one load pipeline that runs on from
    // one item into the next.  XCD x (workgroups x, x + 8, ...) owns a
    // contiguous eighth of the items, so the tiles that share W rows run
    // together on one XCD and share its L2; within the XCD the items are
    // dealt round-robin to its workgroups.  (Item counts stay below 2^31.)
    const int m_act = MODE == kModeDense ? (int)p.m_tiles : const_load(p.tile_off, p.experts);
    const int items = m_act * (int)p.n_tiles * p.ksplit;
    const int per = (items + 7) >> 3;
    const int x_begin = (int)(blockIdx.x & 7) * per;
    const int x_end = x_begin + per < items ? x_begin + per : items;
    if (x_begin >= x_end)
        return;
    const int active = (int)(gridDim.x >> 3), slot = (int)(blockIdx.x >> 3);
    if (x_begin + slot >= x_end)
        return;

    const int64_t K = p.K;
    const int64_t kpb = K / 2, kpsb = K / 16;
    const int nst_all = (int)(K / kSkBK);
    const int64_t w_rows = (MODE == kModeGateUp) ? 2 * p.N : p.N;
    const int64_t ws_step = w_scale_step(p.w_tiled);  // W scale bytes per stage

    // item -> expert, A-side rows [row_begin, row_end), W tile, K split and
    // its stages [st0, st0 + nst)
    struct Item {
        int64_t row_begin, row_end, nt;
        int e, ks, st0, nst;
    };
    auto item_of = [&](int it) {
        Item t;
        const uint32_t u = (uint32_t)it, ma = (uint32_t)m_act, sp = (uint32_t)p.ksplit;
        const int mt = (int)(u % ma);
        const uint32_t rest = u / ma;
        t.ks = (int)(rest % sp);
        t.nt = rest / sp;
        t.e = 0;
        if (MODE == kModeDense) {
            t.row_begin = mt * BM;
            t.row_end = t.row_begin + BM < p.M ? t.row_begin + BM : p.M;
        } else {
            int lo = 0, hi = p.experts - 1;  // largest e with tile_off[e] <= mt
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (const_load(p.tile_off, mid) <= mt)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            t.e = lo;
            t.row_begin = const_load(p.row_base, lo) + (mt - const_load(p.tile_off, lo)) * BM;
            const int64_t eend = const_load(p.row_lim, lo);
            t.row_end = t.row_begin + BM < eend ? t.row_begin + BM : eend;
        }
        t.st0 = nst_all * t.ks / p.ksplit;
        t.nst = nst_all * (t.ks + 1) / p.ksplit - t.st0;
        return t;
    };
    // stages of item it (its K split's share of the nst_all stages)
    auto item_nst = [&](int it) {
        const int ks = (int)(((uint32_t)it / (uint32_t)m_act) % (uint32_t)p.ksplit);
        return nst_all * (ks + 1) / p.ksplit - nst_all * ks / p.ksplit;
    };

    // ---- this thread's loads: W code pieces j (tile row 32 j + tid / 8,
    // piece tid % 8), a W scale row (threads < 128) and an A piece (A row
    // tid / 8 % BM, piece tid % 8): with 16-row tiles the threads >= 128
    // load the A tile, with 32-row tiles every thread does --------------
    const int pc = tid & 7;
    const bool loads_scales = tid < 128;
    const bool loads_a = kAllA || tid >= 128;
    const int arow = (tid >> 3) & (BM - 1);
    int wdst[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int r = 32 * j + (tid >> 3);
        wdst[j] = r * 128 + 16 * sk_wslot(r, pc);
    }
    const uint8_t* wsrc[4];
    const uint8_t* xsrc;    // 16-row tiles: W scale row or A piece; 32-row tiles: A piece
    const uint8_t* ssrc;    // 32-row tiles: W scale row
    const uint8_t* ysrc;
    const uint16_t* bsrc;  // W4A16: A row as bf16, this thread's 32 elements (64 bytes) of a stage
    // point the loads at stage 0 of item t
    auto setup_loads = [&](const Item& t) {
        // the thread index passes through an empty asm statement, so that
        // what is derived from it is formed here, once per item, rather than
        // hoisted out of the stage loop into registers held throughout
        int th = tid;
        asm volatile("" : "+v"(th));
        const int pc = th & 7, arow = (th >> 3) & (BM - 1);
        const bool loads_scales = th < 128;
        const uint8_t* wp = p.w_packed + (int64_t)t.e * w_rows * kpb;
        const uint8_t* wsc = p.w_scales + (int64_t)t.e * w_rows * kpsb;
        // tile row r -> W row.  Wave w's fragment f is tile rows 32 w + 16 f +
        // [0, 16); in gate_up mode fragment 0 holds gate rows and fragment 1
        // the matching up rows.
        auto w_row_of = [&](int r) -> int64_t {
            if (MODE == kModeGateUp) {
                const int64_t c = t.nt * (BN / 2) + 16 * (r >> 5) + (r & 15);
                return ((r >> 4) & 1) == 0 ? c : p.N + c;
            }
            const int64_t n = t.nt * BN + r;
            return n < p.N ? n : p.N - 1;  // ragged last tile: reread a valid row, never stored
        };
#pragma unroll
        for (int j = 0; j < 4; j++)
            wsrc[j] = wp + w_row_of(32 * j + (th >> 3)) * kpb + t.st0 * (kSkBK / 2) + 16 * pc;
        int64_t ar = t.row_begin + arow;
        if (ar >= t.row_end)
            ar = t.row_begin;  // padding rows repeat a valid row; never stored
        if (MODE == kModeGateUp) {
            // the tile's 16 list positions -> tokens: uniform (scalar) loads,
            // each lane keeping the one of its own row
            int32_t pv = 0;
#pragma unroll
            for (int i = 0; i < BM; i++) {
                const int64_t q = t.row_begin + i < t.row_end ? t.row_begin + i : t.row_begin;
                const int32_t v = const_load(p.perm, q);
                pv = arow == i ? v : pv;
            }
            ar = pv / p.topk;
        }
        const uint8_t* wsrow = w_scale_row(wsc, w_row_of(th & 127), K, p.w_tiled) + t.st0 * ws_step;
        const uint8_t* apiece = p.a_packed + ar * kpb + t.st0 * (kSkBK / 2) + 16 * pc;
        xsrc = (!kAllA && loads_scales) ? wsrow : apiece;
        ssrc = wsrow;
        ysrc = p.a_scales + ar * kpsb + t.st0 * (kSkBK / 16) + 2 * pc;
        bsrc = A16 ? p.a_bf16 + ar * p.lda + t.st0 * kSkBK + 32 * pc : nullptr;
    };

    u32x4 wreg[3][4];
    u32x4 xreg[3];
    u32x4 sreg[3];  // 32-row tiles: W scales (threads < 128)
    uint32_t yreg[3];
    u32x4 breg[3][4];
    auto load_stage = [&](int64_t st, int set) {
        if (kAllA) {
            if (loads_scales)
                sreg[set] = *(const u32x4*)(ssrc + st * ws_step);
            if (A16) {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    breg[set][i] = *(const u32x4*)(bsrc + st * kSkBK + 8 * i);
            } else {
                xreg[set] = *(const u32x4*)(xsrc + st * (kSkBK / 2));
                yreg[set] = *(const uint16_t*)(ysrc + st * (kSkBK / 16));
            }
        } else if (A16 && !loads_scales) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                breg[set][i] = *(const u32x4*)(bsrc + st * kSkBK + 8 * i);
        } else {
            const int64_t xo = loads_scales ? st * ws_step : st * (kSkBK / 2);
            xreg[set] = *(const u32x4*)(xsrc + xo);
            if (!A16 && !loads_scales)
                yreg[set] = *(const uint16_t*)(ysrc + st * (kSkBK / 16));
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
            wreg[set][j] = *(const u32x4*)(wsrc[j] + st * (kSkBK / 2));
    };
    // registers of a stage -> LDS buffer b (A decoded to f16 on the way)
    auto store_stage = [&](int set, int b) {
#pragma unroll
        for (int j = 0; j < 4; j++)
            *(u32x4*)(&lds_w[b][wdst[j]]) = wreg[set][j];
        if (loads_scales)
            *(u32x4*)(&lds_ws[b][16 * tid]) = kAllA ? sreg[set] : xreg[set];
        if (loads_a && A16) {
            uint8_t* rowp = &lds_a[b][arow * kSkRowF16];
#pragma unroll
            for (int i = 0; i < 4; i++)
                *(u32x4*)(rowp + 16 * sk_aslot(arow, 4 * pc + i)) = breg[set][i];
        } else if (loads_a) {
            const half2_t s2 = scales2<0>(yreg[set]);
            uint8_t* rowp = &lds_a[b][arow * kSkRowF16];
            const u32x4 cv = xreg[set];
            *(u32x4*)(rowp + 16 * sk_aslot(arow, 4 * pc + 0)) = decode_chunk(cv.x, s2.x);
            *(u32x4*)(rowp + 16 * sk_aslot(arow, 4 * pc + 1)) = decode_chunk(cv.y, s2.x);
            *(u32x4*)(rowp + 16 * sk_aslot(arow, 4 * pc + 2)) = decode_chunk(cv.z, s2.y);
            *(u32x4*)(rowp + 16 * sk_aslot(arow, 4 * pc + 3)) = decode_chunk(cv.w, s2.y);
        }
    };

    typedef float float4_t __attribute__((ext_vector_type(4)));
    float4_t acc[2][NA];  // [W fragment][A fragment]
#pragma unroll
    for (int f = 0; f < 2; f++)
#pragma unroll
        for (int a = 0; a < NA; a++)
            acc[f][a] = (float4_t){};

    auto compute = [&](int b) {
        const uint8_t* ta = lds_a[b] + fr * kSkRowF16;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            u32x4 piece[2];
            half2_t s2[2];
            float sf[2][2];
#pragma unroll
            for (int f = 0; f < 2; f++) {
                const int r = 32 * wave + 16 * f + fr;
                piece[f] = *(const u32x4*)(&lds_w[b][r * 128 + 16 * sk_wslot(r, 4 * q + kg)]);
                // blocks 8 q + 2 kg + {0, 1} of the stage
                const uint32_t sb = *(const uint16_t*)(&lds_ws[b][r * 16 + 8 * q + 2 * kg]);
                if (P2) {
                    sf[f][0] = __builtin_amdgcn_cvt_f32_fp8(sb, 0);
                    sf[f][1] = __builtin_amdgcn_cvt_f32_fp8(sb, 1);
                } else {
                    s2[f] = scales2<0>(sb);
                }
            }
#pragma unroll
            for (int d = 0; d < 4; d++) {
                u32x4 fa[NA];
#pragma unroll
                for (int a = 0; a < NA; a++)
                    fa[a] = *(const u32x4*)(ta + 16 * a * kSkRowF16 + 16 * sk_aslot(16 * a + fr, 16 * q + 4 * kg + d));
#pragma unroll
                for (int f = 0; f < 2; f++) {
                    const u32x4 pv = piece[f];
                    const uint32_t codes = d == 0 ? pv.x : d == 1 ? pv.y : d == 2 ? pv.z : pv.w;
                    if constexpr (A16) {
                        // bf16 operands; the scale as fp32 (general scales:
                        // the fp8 byte pair converted exactly)
                        const float sc = P2 ? sf[f][d >> 1] : (float)(d < 2 ? s2[f].x : s2[f].y);
                        const u32x4 dv = P2 ? decode_chunk_bf16_p2(codes, sc) : decode_chunk_bf16(codes, sc);
#pragma unroll
                        for (int a = 0; a < NA; a++)
                            acc[f][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, fa[a]), __builtin_bit_cast(bf16x8_t, dv), acc[f][a], 0, 0, 0);
                    } else {
                        const u32x4 dv = P2 ? decode_chunk_p2(codes, sf[f][d >> 1])
                                            : decode_chunk(codes, d < 2 ? s2[f].x : s2[f].y);
#pragma unroll
                        for (int a = 0; a < NA; a++)
                            acc[f][a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(half8_t, fa[a]), __builtin_bit_cast(half8_t, dv), acc[f][a], 0, 0, 0);
                    }
                }
            }
        }
    };

    // ---- epilogue of item t: lane holds output rows 16 a + 4 kg + i (A
    // fragment a), column fr of each W fragment -------------------------------
    uint32_t hmax = 0;  // gate_up with bf16 h: max |h| bits seen by this lane
    auto epilogue = [&](const Item& t) {
        // (lane index made opaque as in setup_loads)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int fr = ln & 15, kg = ln >> 4;
        const float gscale = (A16 ? 1.0f : const_load(p.a_global, 0)) * const_load(p.w_global, t.e);
        const int rows_left = (int)(t.row_end - t.row_begin);
        if (MODE == kModeGateUp && p.ksplit > 1) {
            // K split: scaled partial gate and up sums to plane ks, rows of
            // 2N (gate columns, then up columns); swiglu_reduce_kernel finishes
            const int64_t col = t.nt * (BN / 2) + 16 * wave + fr;
            float* part = p.partial + (int64_t)t.ks * p.M * 2 * p.N;
#pragma unroll
            for (int a = 0; a < NA; a++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int m = 16 * a + 4 * kg + i;
                    if (m < rows_left) {
                        const int64_t o = (t.row_begin + m) * 2 * p.N + col;
                        part[o] = acc[0][a][i] * gscale;
                        part[o + p.N] = acc[1][a][i] * gscale;
                    }
                }
        } else if (MODE == kModeGateUp && p.hq_global) {
            // h straight to NVFP4: the 16 lanes of a k-group hold the 16
            // columns of one block of row 4 kg + i
            const int64_t col = t.nt * (BN / 2) + 16 * wave + fr;
            const float Gh = const_load(p.hq_global, 0), six = 6.0f * Gh;
#pragma unroll
            for (int a = 0; a < NA; a++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int m = 16 * a + 4 * kg + i;
                    const float gg = acc[0][a][i] * gscale;
                    const float uu = acc[1][a][i] * gscale;
                    const uint32_t hb = f32_to_bf16(silu_f(gg) * uu);
                    uint32_t sc, codes;
                    encode_block16(hb, Gh, six, &sc, &codes);
                    if (m < rows_left) {
                        const int64_t row = t.row_begin + m;
                        if ((fr & 7) == 0)
                            *(uint32_t*)(p.hq_packed + row * (p.N / 2) + (col >> 1)) = codes;
                        if (fr == 0)
                            p.hq_scales[row * (p.N / 16) + (col >> 4)] = (uint8_t)sc;
                    }
                }
        } else if (MODE == kModeGateUp) {
            // h as bf16; its max magnitude is kept per lane over the items
            // and goes to the atomic word once, after the last item
            const int64_t col = t.nt * (BN / 2) + 16 * wave + fr;
            uint16_t* h = (uint16_t*)p.out + t.row_begin * p.N + col;
#pragma unroll
            for (int a = 0; a < NA; a++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int m = 16 * a + 4 * kg + i;
                    if (m < rows_left) {
                        const float gg = acc[0][a][i] * gscale;
                        const float uu = acc[1][a][i] * gscale;
                        const uint16_t hb = f32_to_bf16(silu_f(gg) * uu);
                        h[(int64_t)m * p.N] = hb;
                        const uint32_t mag = hb & 0x7FFFu;
                        hmax = hmax > mag ? hmax : mag;
                    }
                }
        } else {
            // K split: split ks writes its scaled partial sums to plane ks
            const bool split = p.ksplit > 1;
            const bool bf16_out = MODE == kModeDense && p.out_bf16;
            float* part = split ? p.partial + (int64_t)t.ks * p.M * p.N : nullptr;
#pragma unroll
            for (int f = 0; f < 2; f++) {
                const int64_t col = t.nt * BN + 32 * wave + 16 * f + fr;
                if (col < p.N) {
#pragma unroll
                    for (int a = 0; a < NA; a++)
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int m = 16 * a + 4 * kg + i;
                            if (m < rows_left) {
                                const int64_t o = (t.row_begin + m) * p.N + col;
                                if (split)
                                    part[o] = acc[f][a][i] * gscale;
                                else if (bf16_out)
                                    ((uint16_t*)p.out)[o] = f32_to_bf16(acc[f][a][i] * gscale);
                                else
                                    ((float*)p.out)[o] = acc[f][a][i] * gscale;
                            }
                        }
                }
            }
        }
    };

    // ---- load cursor: runs three stages ahead of the compute cursor over
    // the same item sequence; past the last item it rereads that item's last
    // stage (never computed) ------------------------------------------------
    int l_it = x_begin + slot, l_s = 0, l_nst;
    {
        const Item t = item_of(l_it);
        setup_loads(t);
        l_nst = t.nst;
    }
    auto load_next = [&](int set) {
        load_stage(l_s, set);
        if (++l_s == l_nst) {
            if (l_it + active < x_end) {
                l_it += active;
                const Item t = item_of(l_it);
                setup_loads(t);
                l_s = 0;
                l_nst = t.nst;
            } else {
                l_s = l_nst - 1;
            }
        }
    };

    // ---- pipeline: registers hold stages g+2 and g+3 in flight while stage
    // g+1 goes to LDS and stage g is computed; one barrier per stage -------
    int c_it = x_begin + slot, c_s = 0, c_nst = item_nst(c_it);
    int total = 0;  // stages this workgroup computes
    for (int it = c_it; it < x_end; it += active)
        total += item_nst(it);
    load_next(0);
    load_next(1);
    load_next(2);
    store_stage(0, 0);
    __syncthreads();
    int g = 0;  // stages computed so far; its parity picks the LDS buffer
    auto iter = [&](auto set_tag) {
        constexpr int cur = decltype(set_tag)::value;  // register set of stage g (and g+3)
        constexpr int nxt = (cur + 1) % 3;              // register set of stage g+1
        store_stage(nxt, (g + 1) & 1);
        load_next(cur);
        compute(g & 1);
        __syncthreads();
        g++;
        if (++c_s == c_nst) {
            epilogue(item_of(c_it));
#pragma unroll
            for (int f = 0; f < 2; f++)
#pragma unroll
                for (int a = 0; a < NA; a++)
                    acc[f][a] = (float4_t){};
            c_it += active;
            c_nst = item_nst(c_it);
            c_s = 0;
        }
    };
    while (g + 3 <= total) {
        iter(IntC<0>{});
        iter(IntC<1>{});
        iter(IntC<2>{});
    }
    if (g < total)
        iter(IntC<0>{});
    if (g < total)
        iter(IntC<1>{});
    if (MODE == kModeGateUp && p.ksplit == 1 && !p.hq_global) {
        // one atomic per workgroup (the waves meet in the idle scale staging):
        // all workgroups finish together, and same-address atomics serialize
        hmax = block_max_u32(hmax, (uint32_t*)lds_ws[0]);
        if (tid == 0 && hmax != 0)
            atomicMax(p.h_amax, hmax << 16);
    }
    wait_vm<0>();  // the rereads past the last item
}

// K-split gate_up: h[r, c] = bf16(silu(g) * u) with g, u the sums in split
// order of the scaled partials (plane s: rows of 2N floats, gate then up);
// max |h| to the atomic word as the unsplit epilogue does.
// With a static G_h (hq_global non-null) h is encoded to NVFP4 instead:
// 16 consecutive threads hold one block (N % 16 == 0).
__global__ void __launch_bounds__(256)
swiglu_reduce_kernel(const float* __restrict__ partial, int ksplit, int64_t rows, int64_t N,
                     uint16_t* __restrict__ h, uint32_t* h_amax, const float* hq_global,
                     uint8_t* __restrict__ hq_packed, uint8_t* __restrict__ hq_scales)
{
    const int64_t count = rows * N;
    const int64_t plane = rows * 2 * N;
    const float Gh = hq_global ? *hq_global : 1.0f, six = 6.0f * Gh;
    uint32_t hmax = 0;
    if (!hq_global && N % 4 == 0 && count < ((int64_t)1 << 31)) {
        // bf16 h: four consecutive columns per thread (16-byte loads, the
        // planes' loads four at a time, added in the same split order)
        const uint32_t n4 = (uint32_t)(N / 4), count4 = (uint32_t)(count / 4);
        for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < count4; i += gridDim.x * blockDim.x) {
            const uint32_t r = i / n4, c = 4 * (i - r * n4);
            const float* g = partial + (int64_t)r * 2 * N + c;
            float4_t gg = *(const float4_t*)g, uu = *(const float4_t*)(g + N);
            for (int s0 = 1; s0 < ksplit; s0 += 4) {
                float4_t xg[4], xu[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const bool in = s0 + u < ksplit;
                    xg[u] = in ? *(const float4_t*)(g + (int64_t)(s0 + u) * plane) : (float4_t){0, 0, 0, 0};
                    xu[u] = in ? *(const float4_t*)(g + (int64_t)(s0 + u) * plane + N) : (float4_t){0, 0, 0, 0};
                }
#pragma unroll
                for (int u = 0; u < 4; u++)
                    if (s0 + u < ksplit) {
                        gg += xg[u];
                        uu += xu[u];
                    }
            }
            uint32_t hb[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                hb[t] = f32_to_bf16(silu_f(gg[t]) * uu[t]);
                const uint32_t mag = hb[t] & 0x7FFFu;
                hmax = hmax > mag ? hmax : mag;
            }
            *(u32x2*)(h + (int64_t)r * N + c) = (u32x2){hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
        }
    } else
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / N, c = i - r * N;
        const float* g = partial + r * 2 * N + c;
        float gg = g[0], uu = g[N];
        for (int s = 1; s < ksplit; s++) {
            gg += g[(int64_t)s * plane];
            uu += g[(int64_t)s * plane + N];
        }
        const uint16_t hb = f32_to_bf16(silu_f(gg) * uu);
        if (hq_global) {
            uint32_t sc, codes;
            encode_block16(hb, Gh, six, &sc, &codes);
            if ((i & 7) == 0)
                *(uint32_t*)(hq_packed + (i >> 1)) = codes;
            if ((i & 15) == 0)
                hq_scales[i >> 4] = (uint8_t)sc;
            continue;
        }
        h[i] = hb;
        const uint32_t mag = hb & 0x7FFFu;
        hmax = hmax > mag ? hmax : mag;
    }
    if (hq_global)
        return;
    // one atomic per workgroup: same-address atomics serialize
    __shared__ uint32_t red[16];
    hmax = block_max_u32(hmax, red);
    if (threadIdx.x == 0 && hmax != 0)
        atomicMax(h_amax, hmax << 16);
}

// Sum the scaled K-split partials in split order and store fp32 or bf16.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ partial, int ksplit, int64_t count, void* out, int out_bf16)
{
    if (count % 4 == 0 && ((uintptr_t)out & (out_bf16 ? 7 : 15)) == 0) {
        // four consecutive outputs per thread, the planes' loads four at a
        // time, added in split order
        for (int64_t i = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x); i < count;
             i += 4 * (int64_t)gridDim.x * blockDim.x) {
            float4_t v = *(const float4_t*)(partial + i);
            for (int s0 = 1; s0 < ksplit; s0 += 4) {
                float4_t x[4];
#pragma unroll
                for (int u = 0; u < 4; u++)
                    x[u] = s0 + u < ksplit ? *(const float4_t*)(partial + (int64_t)(s0 + u) * count + i)
                                           : (float4_t){0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < 4; u++)
                    if (s0 + u < ksplit)
                        v += x[u];
            }
            if (out_bf16)
                *(u32x2*)((uint16_t*)out + i) = (u32x2){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            else
                *(float4_t*)((float*)out + i) = v;
        }
        return;
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = partial[i];
        for (int s = 1; s < ksplit; s++)
            v += partial[(int64_t)s * count + i];
        if (out_bf16)
            ((uint16_t*)out)[i] = f32_to_bf16(v);
        else
            ((float*)out)[i] = v;
    }
}

}  // namespace nvfp4
