// mx8.h -- MX-native W4A8: MXFP8 activations x MXFP4 weights on the scaled
// MFMA (page "DeepSeek-V4.1-Flash-NVFP4", section 二: the reference FP8 x FP4
// GEMM quantizes activations in blocks and weights in 32-element blocks with
// power-of-two scales and applies the block scales inside the accumulation).
//
// Both operands carry one UE8M0 scale per 32 elements along K, which is
// exactly what v_mfma_scale_f32_32x32x64_f8f6f4 applies, so the operands go
// from LDS to the MFMA without any decode.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (A = E4M3 bytes in the
// first operand, B = E2M1 nibbles in the second; measured with a probe that
// fitted random inputs): lane l supplies row (or column) l % 32 and the
// scale byte of K-block l / 32 (32 elements each) for both operands; the
// fp4 operand holds K-block l / 32 as 32 nibbles in order (element 2j in the
// low nibble of byte j, 16 bytes); the fp8 operand holds 16 elements of each
// block: bytes 0-15 are K [16 (l/32), +16) of block 0 and bytes 16-31 the
// same range of block 1 (the same per-type layout holds with the operands in
// either position).  Output: lane l holds column l % 32 (of the second
// operand) and rows (i % 4) + 8 (i / 4) + 4 (l / 32) (of the first) of the
// 32x32 fragment.  The instruction's
// internal sum is not exact fp32 (about 6e-5 relative on random 64-element
// steps), far inside the GEMM tolerance.
#pragma once
#include "common.h"
#include "gemm.h"

namespace nvfp4 {

typedef int v8i_t __attribute__((ext_vector_type(8)));

// unit global scale for the shared dense epilogue (MX operands carry only
// block scales)
__device__ const float kMxOne = 1.0f;

// ---- MXFP8 encode: one thread per 32-element block -----------------------
// Block scale 2^e with e the smallest integer such that amax <= 448 * 2^e
// (no element saturates), clamped to the UE8M0 range [-127, 127]; an
// all-zero block takes e = 0.  Elements x * 2^-e rounded to E4M3 (nearest,
// ties to even).  Output: fp8 bytes [rows, cols], scale bytes
// [rows, cols / 32] (e + 127).
constexpr int kMx8Threads = 256;

NVFP4_DEV int mx8_exponent(uint32_t amax_bits16)
{
    if (amax_bits16 == 0)
        return 0;
    // amax = s * 2^E with s in [1, 2): the smallest e is E - 8, plus one when
    // s > 1.75 (448 = 1.75 * 2^8)
    float a = __builtin_bit_cast(float, amax_bits16 << 16);
    int shift = 0;
    if (a < 0x1p-100f) {  // bf16 subnormal range: normalise exactly first
        a *= 0x1p64f;
        shift = 64;
    }
    const uint32_t u = __builtin_bit_cast(uint32_t, a);
    const int E = (int)((u >> 23) & 255) - 127 - shift;
    int e = E - 8 + ((u & 0x7FFFFF) > 0x600000 ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__global__ void __launch_bounds__(kMx8Threads)
mxfp8_encode_kernel(const u32x4* __restrict__ x, int64_t rows, int64_t blocks_per_row, int64_t ld_chunks,
                    u32x4* __restrict__ out, uint8_t* __restrict__ e8m0)
{
    const int64_t nblk = rows * blocks_per_row;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
        const int64_t r = b / blocks_per_row;
        const u32x4* src = x + r * ld_chunks + 4 * (b - r * blocks_per_row);
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            v[i] = __builtin_nontemporal_load(src + i);
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t m = absmax_bits8(v[i]);
            am = am > m ? am : m;
        }
        const int e = mx8_exponent(am);
        const float inv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);  // 2^-e (e in [-127, 127])
        // 2^-e for e = -127 is 2^127: representable; e = 127 gives 2^-127, a
        // subnormal fp32 whose exponent field is 0: build it from two factors
        const float inv_lo = e == 127 ? 0x1p-64f : 1.0f;
        const float inv_hi = e == 127 ? 0x1p-63f : inv;
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const float f0 = __builtin_bit_cast(float, w[2 * h] << 16) * inv_hi * inv_lo;
                const float f1 = __builtin_bit_cast(float, w[2 * h] & 0xFFFF0000u) * inv_hi * inv_lo;
                const float f2 = __builtin_bit_cast(float, w[2 * h + 1] << 16) * inv_hi * inv_lo;
                const float f3 = __builtin_bit_cast(float, w[2 * h + 1] & 0xFFFF0000u) * inv_hi * inv_lo;
                uint32_t p = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
                p = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, p, true);
                o[2 * i + h] = p;
            }
        }
        out[2 * b] = (u32x4){o[0], o[1], o[2], o[3]};
        out[2 * b + 1] = (u32x4){o[4], o[5], o[6], o[7]};
        e8m0[b] = (uint8_t)(e + 127);
    }
}

// ---- W4A8 GEMM: C[M, N] = sum over 32-blocks b of 2^(ea[m,b] + ew[n,b]) *
// sum_{k in b} a[m, k] * w[n, k] ----------------------------------------------
struct MxArgs {
    const uint8_t* a;      // E4M3 [M, K]
    const uint8_t* a_sc;   // UE8M0 [M, K/32]
    const uint8_t* w;      // E2M1 packed [experts][N_w, K/2]
    const uint8_t* w_sc;   // UE8M0 [experts][N_w, K/32]
    int64_t M, N, K;       // gate_up: N = I (W holds 2I rows: gate, then up)
    int64_t m_tiles, n_tiles;
    void* out;             // dense: [M, N] fp32 or bf16; gate_up: h bf16; down: y fp32
    int out_bf16;
    // grouped projections: the tile plan of one class, as GemmArgs has it
    const int32_t* tile_off;
    const int32_t* row_base;
    const int32_t* row_lim;
    const int32_t* perm;   // gate_up: list position -> t*k + j
    int32_t topk;
    int32_t experts;
    uint32_t* h_amax;      // gate_up: max |h| bits (atomic)
};

constexpr int kMxGrpK = 128;  // K elements per staged group (two MFMA k-steps)

// Tile BM x BN, 4 waves of (BM/2) x (BN/2), v_mfma_scale_f32_32x32x64_f8f6f4.
// Per 128-element group of K the workgroup copies its A rows (128 bytes
// each, 16-byte chunk c of row r at slot c ^ (r % 8)) and W rows (64 bytes,
// paired-row layout tpos) into one of three buffers with the LDS DMA path,
// two groups ahead; the scale bytes (4 per row per group, one dword) are
// loaded straight into registers one group ahead.  One barrier per group.
template <int BM, int BN, int MODE>
__global__ void __launch_bounds__(256)
mx_w4a8_kernel(MxArgs p)
{
    constexpr int WM = 2, WN = 2, NW = 4;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int NJA = BM * 128 / 1024 / NW;  // A copies per wave per group
    constexpr int NJW = BN * 64 / 1024 / NW;   // W copies per wave per group
    constexpr int AB = BM * 128, WB = BN * 64;
    static_assert(BM % 64 == 0 && BN % 64 == 0 && NJA >= 1 && NJW >= 1, "tile shape");
    __shared__ __attribute__((aligned(16))) uint8_t lds_a0[AB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a1[AB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_a2[AB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_w0[WB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_w1[WB];
    __shared__ __attribute__((aligned(16))) uint8_t lds_w2[WB];
    auto abuf = [&](auto t) -> uint8_t* {
        constexpr int B = decltype(t)::value % 3;
        return B == 0 ? lds_a0 : B == 1 ? lds_a1 : lds_a2;
    };
    auto wbuf = [&](auto t) -> uint8_t* {
        constexpr int B = decltype(t)::value % 3;
        return B == 0 ? lds_w0 : B == 1 ? lds_w1 : lds_w2;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave / WN, wave_n = wave % WN;
    // tile coordinates, A rows and W rows through the grouped-GEMM helpers
    // (dense: the plain tiling); MX operands carry no global scale
    GemmArgs g{};
    g.a_global = &kMxOne;
    g.w_global = &kMxOne;
    g.M = p.M;
    g.N = p.N;
    g.K = p.K;
    g.m_tiles = p.m_tiles;
    g.n_tiles = p.n_tiles;
    g.tile_off = p.tile_off;
    g.row_base = p.row_base;
    g.row_lim = p.row_lim;
    g.perm = p.perm;
    g.topk = p.topk;
    g.experts = p.experts;
    g.out = p.out;
    g.out_bf16 = p.out_bf16;
    g.h_amax = p.h_amax;
    g.ksplit = 1;
    TileCoord tc;
    if (!tile_coord<BM, MODE>(g, tc))
        return;
    const int64_t K = p.K, kb = K / 32, kpb = K / 2;
    const int64_t ngr = K / kMxGrpK;
    const int64_t w_rows = MODE == kModeGateUp ? 2 * p.N : p.N;
    const uint8_t* wexp = p.w + (int64_t)tc.e * w_rows * kpb;
    const uint8_t* wsexp = p.w_sc + (int64_t)tc.e * w_rows * kb;
    auto arow = [&](int r) -> int64_t { return tile_a_row<MODE>(g, tc, r); };
    auto wrow = [&](int r) -> int64_t { return tile_w_row<BN, TN, MODE>(g, tc, r); };

    // copy sources: A copy j covers rows 8 (NJA wave + j) + lane / 8, lane
    // slot lane % 8 holding chunk (lane % 8) ^ (row % 8); W copy j as the
    // paired-row layout of gemm_rtile_kernel
    const uint8_t* asrc[NJA];
#pragma unroll
    for (int j = 0; j < NJA; j++) {
        const int r = 8 * (NJA * wave + j) + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        asrc[j] = p.a + arow(r) * K + 16 * c;
    }
    const uint8_t* wsrc[NJW];
#pragma unroll
    for (int j = 0; j < NJW; j++) {
        const int q = 8 * (NJW * wave + j) + (lane >> 3);
        const int hc = (lane & 7) ^ ((q ^ (q >> 1)) & 7);
        const int r = 2 * q + (hc >> 2);
        wsrc[j] = wexp + wrow(r) * kpb + 16 * (hc & 3);
    }
    auto issue = [&](int64_t G, auto t) {
        const int64_t g = G < ngr ? G : ngr - 1;
        uint8_t* da = abuf(t);
        uint8_t* dw = wbuf(t);
#pragma unroll
        for (int j = 0; j < NJA; j++)
            __builtin_amdgcn_global_load_lds((const void*)(asrc[j] + g * kMxGrpK), (lds_ptr_t)(da + (NJA * wave + j) * 1024),
                                             16, 0, 0);
#pragma unroll
        for (int j = 0; j < NJW; j++)
            __builtin_amdgcn_global_load_lds((const void*)(wsrc[j] + g * (kMxGrpK / 2)),
                                             (lds_ptr_t)(dw + (NJW * wave + j) * 1024), 16, 0, 0);
    };

    // fragment rows of this lane and their scale sources
    const int fr = lane & 31, q = lane >> 5;
    const int ra = wave_m * TM + fr, rw = wave_n * TN + fr;
    const int lsw = tline_sw(fr), par = fr & 1;
    const uint8_t* asc[FM];
    const uint8_t* wsc[FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
        asc[i] = p.a_sc + arow(ra + 32 * i) * kb;
#pragma unroll
    for (int j = 0; j < FN; j++)
        wsc[j] = wsexp + wrow(rw + 32 * j) * kb;
    uint32_t sa[FM], sw[FN], na[FM], nw[FN];
    auto load_scales = [&](int64_t G, uint32_t (&da)[FM], uint32_t (&dw)[FN]) {
        const int64_t g = G < ngr ? G : ngr - 1;
#pragma unroll
        for (int i = 0; i < FM; i++)
            da[i] = *(const uint32_t*)(asc[i] + 4 * g);
#pragma unroll
        for (int j = 0; j < FN; j++)
            dw[j] = *(const uint32_t*)(wsc[j] + 4 * g);
    };
    // this lane's blocks (q, 2 + q) of a group in bytes 0 and 2 (shifted
    // only when used, so the loads stay in flight)
    auto take_scales = [&]() {
#pragma unroll
        for (int i = 0; i < FM; i++)
            sa[i] = na[i] >> (8 * q);
#pragma unroll
        for (int j = 0; j < FN; j++)
            sw[j] = nw[j] >> (8 * q);
    };

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
            acc[i][j] = (float16_t){};

    // fragments of k-step S (of 2) of group buffer T into set D
    v8i_t fa[2][FM];
    u32x4 fw[2][FN];
    auto read_frags = [&](auto t, auto s_tag, auto d_tag) {
        constexpr int S = decltype(s_tag)::value, D = decltype(d_tag)::value;
        const uint8_t* ba = abuf(t);
        const uint8_t* bw = wbuf(t);
#pragma unroll
        for (int i = 0; i < FM; i++) {
            const int r = ra + 32 * i;
            const u32x4 lo = *(const u32x4*)(ba + r * 128 + 16 * ((4 * S + q) ^ (r & 7)));
            const u32x4 hi = *(const u32x4*)(ba + r * 128 + 16 * ((4 * S + 2 + q) ^ (r & 7)));
            fa[D][i] = (v8i_t){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < FN; j++)
            fw[D][j] = *(const u32x4*)(bw + 64 * (rw & ~1) + 2048 * j + 16 * ((4 * par + 2 * S + q) ^ lsw));
    };
    // the MFMAs of k-step S from set D: the weight fragment goes first, so
    // each lane accumulates one output row and runs of four columns
    auto mfmas = [&](auto s_tag, auto d_tag) {
        constexpr int S = decltype(s_tag)::value, D = decltype(d_tag)::value;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++) {
                const u32x4 w = fw[D][j];
                const v8i_t wv = (v8i_t){(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, fa[D][i], acc[i][j], 4, 0, 2 * S,
                                                                            (int)sw[j], 2 * S, (int)sa[i]);
            }
    };

    // prologue: groups 0 and 1 staged, scales and k-step 0 fragments of
    // group 0 in registers
    load_scales(0, na, nw);
    issue(0, IntC<0>{});
    issue(1, IntC<1>{});
    wait_vm<0>();
    __syncthreads();
    take_scales();
    read_frags(IntC<0>{}, IntC<0>{}, IntC<0>{});
    constexpr int NC = NJA + NJW;
    // group G (T = G mod 3): scales of G + 1 and the copies of group G + 2
    // (into the buffer group G - 1 used, free since the last barrier), then
    // k-step 0 with the reads of k-step 1, the barrier that publishes group
    // G + 1, k-step 1 with the reads of group G + 1's first fragments
    auto group = [&](int64_t G, auto t) {
        constexpr int T = decltype(t)::value;
        load_scales(G + 1, na, nw);
        issue(G + 2, IntC<(T + 2) % 3>{});
        __builtin_amdgcn_sched_barrier(0);
        mfmas(IntC<0>{}, IntC<0>{});
        read_frags(IntC<T>{}, IntC<1>{}, IntC<1>{});
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<NC>();  // group G + 1 and its scales (the copies of G + 2 may stay in flight)
        wait_lgkm0();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        mfmas(IntC<1>{}, IntC<1>{});
        read_frags(IntC<(T + 1) % 3>{}, IntC<0>{}, IntC<0>{});  // past the end: unused
        __builtin_amdgcn_sched_barrier(0);
        take_scales();
        __builtin_amdgcn_sched_barrier(0);
    };
    int64_t G = 0;
    for (; G + 3 <= ngr; G += 3) {
        group(G, IntC<0>{});
        group(G + 1, IntC<1>{});
        group(G + 2, IntC<2>{});
    }
    if (G < ngr)
        group(G, IntC<0>{});
    if (G + 1 < ngr)
        group(G + 1, IntC<1>{});
    wait_vm<0>();
    __syncthreads();

    // epilogue: the output tile staged per wave in the A buffers (free now)
    // and written as 16-byte pieces (gate_up: SwiGLU, h bf16 and its max;
    // the scale of every expert is 1)
    tc.e = 0;
    static_assert(2 * TM * 128 <= AB, "two waves' output staging fits one A buffer");
    store_tile_t<BN, TM, TN, FM, FN, MODE>(g, tc, acc, wave_m, wave_n, lane,
                                           (wave < 2 ? lds_a0 : lds_a1) + (wave & 1) * TM * 128);
}

}  // namespace nvfp4
