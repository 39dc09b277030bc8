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

// ---- MXFP8 encode: four lanes per 32-element block ------------------------
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

// Work item = 8 elements (one 16-byte bf16 chunk, one 8-byte fp8 output):
// consecutive lanes take consecutive chunks, so loads and stores are whole
// lines per instruction, and the 4 lanes of a 32-element block share its
// max with two lane swaps.  kU items per thread per trip, loads first.
template <int kU>
__global__ void __launch_bounds__(kMx8Threads)
mxfp8_encode_kernel(const u32x4* __restrict__ x, int64_t rows, int64_t blocks_per_row, int64_t ld_chunks,
                    u32x2* __restrict__ out, uint8_t* __restrict__ e8m0)
{
    const int64_t cpr = 4 * blocks_per_row;  // 8-element chunks per row
    const int64_t nq = rows * cpr;
    const bool flat = ld_chunks == cpr;
    constexpr int64_t kChunk = (int64_t)kU * kMx8Threads;
    for (int64_t base = (int64_t)blockIdx.x * kChunk; base < nq; base += (int64_t)gridDim.x * kChunk) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; u++) {
            int64_t h = base + u * kMx8Threads + threadIdx.x;
            h = h < nq ? h : nq - 1;
            int64_t src = h;
            if (!flat) {
                const int64_t r = h / cpr;
                src = r * ld_chunks + (h - r * cpr);
            }
            v[u] = __builtin_nontemporal_load(x + src);
        }
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int64_t h = base + u * kMx8Threads + threadIdx.x;
            uint32_t am = absmax_bits8(v[u]);
            uint32_t o = (uint32_t)__shfl_xor((int)am, 1, 64);
            am = am > o ? am : o;
            o = (uint32_t)__shfl_xor((int)am, 2, 64);
            am = am > o ? am : o;
            const int e = mx8_exponent(am);
            const float inv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);  // 2^-e (e in [-127, 127])
            // 2^-e for e = -127 is 2^127: representable; e = 127 gives 2^-127, a
            // subnormal fp32 whose exponent field is 0: build it from two factors
            const float inv_lo = e == 127 ? 0x1p-64f : 1.0f;
            const float inv_hi = e == 127 ? 0x1p-63f : inv;
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            uint32_t q[2];
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                const float f0 = __builtin_bit_cast(float, w[2 * hh] << 16) * inv_hi * inv_lo;
                const float f1 = __builtin_bit_cast(float, w[2 * hh] & 0xFFFF0000u) * inv_hi * inv_lo;
                const float f2 = __builtin_bit_cast(float, w[2 * hh + 1] << 16) * inv_hi * inv_lo;
                const float f3 = __builtin_bit_cast(float, w[2 * hh + 1] & 0xFFFF0000u) * inv_hi * inv_lo;
                uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
                pk = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, pk, true);
                q[hh] = pk;
            }
            if (h < nq) {
                out[h] = (u32x2){q[0], q[1]};
                if ((h & 3) == 0)
                    e8m0[h >> 2] = (uint8_t)(e + 127);
            }
        }
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
    // scale dwords of three groups in rotation (set G mod 3 holds group G's),
    // so that a set is read only a group after its loads were issued
    uint32_t sa[FM], sw[FN], ra3[3][FM], rw3[3][FN];
    auto load_scales = [&](int64_t G, uint32_t (&da)[FM], uint32_t (&dw)[FN]) {
        const int64_t g = G < ngr ? G : ngr - 1;
#pragma unroll
        for (int i = 0; i < FM; i++)
            da[i] = *(const uint32_t*)(asc[i] + 4 * g);
#pragma unroll
        for (int j = 0; j < FN; j++)
            dw[j] = *(const uint32_t*)(wsc[j] + 4 * g);
    };
    // this lane's blocks (q, 2 + q) of a group in bytes 0 and 2, from set U
    auto take_scales = [&](auto u_tag) {
        constexpr int U = decltype(u_tag)::value % 3;
#pragma unroll
        for (int i = 0; i < FM; i++)
            sa[i] = ra3[U][i] >> (8 * q);
#pragma unroll
        for (int j = 0; j < FN; j++)
            sw[j] = rw3[U][j] >> (8 * q);
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

    // prologue: groups 0 and 1 staged, the scales of groups 0 and 1 loaded,
    // k-step 0 fragments of group 0 read
    load_scales(0, ra3[0], rw3[0]);
    load_scales(1, ra3[1], rw3[1]);
    issue(0, IntC<0>{});
    issue(1, IntC<1>{});
    wait_vm<0>();
    __syncthreads();
    take_scales(IntC<0>{});
    read_frags(IntC<0>{}, IntC<0>{}, IntC<0>{});
    constexpr int NC = NJA + NJW;
    // group G (T = G mod 3): the scales and the copies of group G + 2 (into
    // the buffer group G - 1 used, free since the last barrier), then k-step
    // 0 with the reads of k-step 1, the barrier that publishes group G + 1,
    // k-step 1 with the reads of group G + 1's first fragments.  The scales
    // of G + 1 were loaded a group earlier, so the wait before the barrier
    // leaves both the scale loads and the copies of G + 2 in flight.
    auto group = [&](int64_t G, auto t) {
        constexpr int T = decltype(t)::value;
        load_scales(G + 2, ra3[(T + 2) % 3], rw3[(T + 2) % 3]);
        issue(G + 2, IntC<(T + 2) % 3>{});
        __builtin_amdgcn_sched_barrier(0);
        mfmas(IntC<0>{}, IntC<0>{});
        read_frags(IntC<T>{}, IntC<1>{}, IntC<1>{});
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<NC + FM + FN>();  // group G + 1 (the scales and copies of G + 2 may stay in flight)
        wait_lgkm0();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        mfmas(IntC<1>{}, IntC<1>{});
        read_frags(IntC<(T + 1) % 3>{}, IntC<0>{}, IntC<0>{});  // past the end: unused
        __builtin_amdgcn_sched_barrier(0);
        take_scales(IntC<T + 1>{});
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

// ---------------------------------------------------------------------------
// Weight-streaming W4A8 for decode batches (at most 32 rows per A tile).
//
// The structure of the NVFP4 weight-streaming kernel (gemm_stream_kernel):
// a resident grid whose workgroups walk (A tile, W tile) items with one
// register pipeline three 256-element stages deep, each stage staged in LDS
// behind one barrier; but no decode: the scaled MFMA (32x32x64, E2M1 x E4M3
// with one E8M0 scale per 32 elements of each operand) reads both operands
// from LDS as stored.  A workgroup owns 128 W rows, one 32-row fragment per
// wave, and up to 32 A rows.  Per stage each thread loads 4 pieces of W
// codes (8 lanes per 128-byte row segment), 2 pieces of A (16 lanes per
// 256-byte row segment) and, for 128 + 32 threads, the 8 scale bytes of a W
// or A row.  In gate_up mode the rows of a fragment alternate four gate and
// four up rows of the same 16 output columns: the MFMA puts rows 8 j + 4 q +
// [0, 4) of the weight fragment in lane half q, so lane l holds gate and
// lane l + 32 up of the same (token, column) and one lane swap forms h.
// ---------------------------------------------------------------------------
constexpr int kMsBK = 256;   // K elements per stage
constexpr int kMsBN = 128;   // W rows per workgroup
constexpr int kMsBM = 32;    // A rows per tile

//
// Scale bytes (SC4 = false): each of threads 0-159 loads its row's 8 bytes
// of a stage.  SC4 (stages per item a multiple of 4, K % 1024 == 0, 16-byte
// aligned scale arrays): the 32 bytes of four stages in one request (inside
// one cache line), carried in the register set of the chunk's first stage
// and stored, at that stage's LDS store, into one of two chunk buffers
// (chunk parity) that the next four stages' MFMAs read.  Items hold whole
// chunks, so chunk c is global stages [4 c, 4 c + 4) of the workgroup's walk.
template <int MODE, bool SC4>
__global__ void __launch_bounds__(256)
mx_stream_kernel(MxArgs p)
{
    constexpr int SCW = SC4 ? 8 : 2;  // u32 scale words per row in one scale buffer
    __shared__ __attribute__((aligned(16))) uint8_t lds_w[2][kMsBN * 128];  // E2M1 codes, 2 x 16 KB
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kMsBM * 256];  // E4M3, 2 x 8 KB
    __shared__ __attribute__((aligned(16))) uint32_t lds_sw[2][kMsBN * SCW];  // W scale bytes, 4 * SCW per row
    __shared__ __attribute__((aligned(16))) uint32_t lds_sa[2][kMsBM * SCW];  // A scale bytes, 4 * SCW per row

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 5, fr = lane & 31;

    // ---- items (A tile fastest), dealt as gemm_stream_kernel deals them:
    // XCD x owns a contiguous eighth, round-robin over its workgroups
    const int m_act = const_load(p.tile_off, p.experts);
    const int items = m_act * (int)p.n_tiles;
    const int per = (items + 7) >> 3;
    const int x_begin = (int)(blockIdx.x & 7) * per;
    const int x_end = x_begin + per < items ? x_begin + per : items;
    if (x_begin >= x_end)
        return;
    const int active = (int)(gridDim.x >> 3), slot = (int)(blockIdx.x >> 3);
    if (x_begin + slot >= x_end)
        return;

    const int64_t K = p.K, kpb = K / 2, kb = K / 32;
    const int nst = (int)(K / kMsBK);
    const int64_t w_rows = MODE == kModeGateUp ? 2 * p.N : p.N;

    struct Item {
        int64_t row_begin, row_end, nt;
        int e;
    };
    auto item_of = [&](int it) {
        Item t;
        const int mt = (int)((uint32_t)it % (uint32_t)m_act);
        t.nt = (int)((uint32_t)it / (uint32_t)m_act);
        int lo = 0, hi = p.experts - 1;  // largest e with tile_off[e] <= mt
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (const_load(p.tile_off, mid) <= mt)
                lo = mid;
            else
                hi = mid - 1;
        }
        t.e = lo;
        t.row_begin = const_load(p.row_base, lo) + (int64_t)(mt - const_load(p.tile_off, lo)) * kMsBM;
        const int64_t eend = const_load(p.row_lim, lo);
        t.row_end = t.row_begin + kMsBM < eend ? t.row_begin + kMsBM : eend;
        return t;
    };
    // W row (within the expert) of tile row r (wave r / 32, fragment row
    // r % 32); gate_up: fragment row rho holds column 16 wave + (rho % 4) +
    // 4 (rho / 8), from the gate half when (rho / 4) is even, else the up half
    auto w_row_of = [&](const Item& t, int r) -> int64_t {
        if (MODE == kModeGateUp) {
            const int rho = r & 31;
            const int64_t c = t.nt * 64 + 16 * (r >> 5) + (rho & 3) + 4 * (rho >> 3);
            return ((rho >> 2) & 1) ? p.N + c : c;
        }
        const int64_t n = t.nt * kMsBN + r;
        return n < p.N ? n : p.N - 1;  // (a ragged last tile rereads a valid row, never stored)
    };

    // ---- this thread's loads: W pieces j (tile row 32 j + tid / 8, piece
    // tid % 8), A pieces j (tile row 16 j + tid / 16, piece tid % 16), and
    // the scale bytes of W row tid (tid < 128) or A row tid - 128
    const uint8_t* wsrc[4];
    const uint8_t* asrc[2];
    const uint8_t* ssrc;
    auto setup_loads = [&](const Item& t) {
        int th = tid;
        asm volatile("" : "+v"(th));  // formed here, once per item (see gemm_stream_kernel)
        const uint8_t* wp = p.w + (int64_t)t.e * w_rows * kpb;
        const uint8_t* wsc = p.w_sc + (int64_t)t.e * w_rows * kb;
#pragma unroll
        for (int j = 0; j < 4; j++)
            wsrc[j] = wp + w_row_of(t, 32 * j + (th >> 3)) * kpb + 16 * (th & 7);
        auto a_row = [&](int r) -> int64_t {
            int64_t q_ = t.row_begin + r;
            if (q_ >= t.row_end)
                q_ = t.row_begin;  // padding rows repeat a valid row; never stored
            if (MODE == kModeGateUp)
                return const_load(p.perm, q_) / p.topk;
            return q_;
        };
#pragma unroll
        for (int j = 0; j < 2; j++)
            asrc[j] = p.a + a_row(16 * j + (th >> 4)) * K + 16 * (th & 15);
        ssrc = th < kMsBN ? wsc + w_row_of(t, th) * kb : p.a_sc + a_row((th - kMsBN) & 31) * kb;
    };

    u32x4 wreg[3][4], areg[3][2];
    u32x2 sreg[3];            // (!SC4) a stage's 8 scale bytes
    u32x4 slo[3], shi[3];     // (SC4) a chunk's 32 scale bytes, in its first stage's set
    const bool loads_sc = tid < kMsBN + kMsBM;
    auto load_stage = [&](int st, int set) {
#pragma unroll
        for (int j = 0; j < 4; j++)
            wreg[set][j] = *(const u32x4*)(wsrc[j] + (int64_t)st * (kMsBK / 2));
#pragma unroll
        for (int j = 0; j < 2; j++)
            areg[set][j] = *(const u32x4*)(asrc[j] + (int64_t)st * kMsBK);
        if (SC4) {
            if (loads_sc && (st & 3) == 0) {
                const u32x4* src = (const u32x4*)(ssrc + (int64_t)st * (kMsBK / 32));
                slo[set] = src[0];
                shi[set] = src[1];
            }
        } else if (loads_sc) {
            sreg[set] = *(const u32x2*)(ssrc + (int64_t)st * (kMsBK / 32));
        }
    };
    // LDS store of the register set of global stage gs into stage buffer b
    auto store_stage = [&](int set, int b, int gs) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int r = 32 * j + (tid >> 3);
            *(u32x4*)(&lds_w[b][r * 128 + 16 * sk_wslot(r, tid & 7)]) = wreg[set][j];
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int r = 16 * j + (tid >> 4);
            *(u32x4*)(&lds_a[b][r * 256 + 16 * ((tid & 15) ^ (r & 15))]) = areg[set][j];
        }
        if (SC4) {
            if ((gs & 3) == 0) {
                const int cb = (gs >> 2) & 1;
                if (tid < kMsBN) {
                    *(u32x4*)(&lds_sw[cb][8 * tid]) = slo[set];
                    *(u32x4*)(&lds_sw[cb][8 * tid + 4]) = shi[set];
                } else if (loads_sc) {
                    *(u32x4*)(&lds_sa[cb][8 * (tid - kMsBN)]) = slo[set];
                    *(u32x4*)(&lds_sa[cb][8 * (tid - kMsBN) + 4]) = shi[set];
                }
            }
        } else if (tid < kMsBN) {
            *(u32x2*)(&lds_sw[b][2 * tid]) = sreg[set];
        } else if (loads_sc) {
            *(u32x2*)(&lds_sa[b][2 * (tid - kMsBN)]) = sreg[set];
        }
    };

    float16_t acc = (float16_t){};
    // k-steps S = 0..3 of the stage in buffer b: the wave's W fragment row
    // fr of block 2 S + q (16 bytes of codes) and A row fr's elements
    // [16 q, +16) of blocks 2 S and 2 S + 1; scale byte 2 S + q of each row
    auto compute = [&](int b, int gs) {
        const int rw = 32 * wave + fr;
        const uint32_t* swr = SC4 ? &lds_sw[(gs >> 2) & 1][8 * rw + 2 * (gs & 3)] : &lds_sw[b][2 * rw];
        const uint32_t* sar = SC4 ? &lds_sa[(gs >> 2) & 1][8 * fr + 2 * (gs & 3)] : &lds_sa[b][2 * fr];
#pragma unroll
        for (int S = 0; S < 4; S++) {
            const u32x4 w = *(const u32x4*)(&lds_w[b][rw * 128 + 16 * sk_wslot(rw, 2 * S + q)]);
            const u32x4 lo = *(const u32x4*)(&lds_a[b][fr * 256 + 16 * ((4 * S + q) ^ (fr & 15))]);
            const u32x4 hi = *(const u32x4*)(&lds_a[b][fr * 256 + 16 * ((4 * S + 2 + q) ^ (fr & 15))]);
            const uint32_t sw = swr[S >> 1] >> (8 * q), sa = sar[S >> 1] >> (8 * q);
            const v8i_t wv = (v8i_t){(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
            const v8i_t av = (v8i_t){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                                     (int)hi.w};
            if (S & 1)
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc, 4, 0, 2, (int)sw, 2, (int)sa);
            else
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc, 4, 0, 0, (int)sw, 0, (int)sa);
        }
    };

    // ---- epilogue of item t: lane l holds token row fr and, in element i,
    // fragment row (i % 4) + 8 (i / 4) + 4 q ---------------------------------
    uint32_t hmax = 0;
    auto epilogue = [&](const Item& t) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int fr_ = ln & 31, q_ = ln >> 5;
        const int rows_left = (int)(t.row_end - t.row_begin);
        const int64_t row = t.row_begin + fr_;
        if (MODE == kModeGateUp) {
            // lane half 0: gate, half 1: up, of columns 16 wave + i
            float up[16];
#pragma unroll
            for (int i = 0; i < 16; i++)
                up[i] = __shfl_xor(acc[i], 32, 64);
            if (q_ == 0 && fr_ < rows_left) {
                uint32_t hv[8];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const uint32_t h0 = f32_to_bf16(silu_f(acc[2 * i]) * up[2 * i]);
                    const uint32_t h1 = f32_to_bf16(silu_f(acc[2 * i + 1]) * up[2 * i + 1]);
                    hv[i] = h0 | (h1 << 16);
                    const uint32_t m0 = h0 & 0x7FFFu, m1 = h1 & 0x7FFFu;
                    hmax = hmax > m0 ? hmax : m0;
                    hmax = hmax > m1 ? hmax : m1;
                }
                uint16_t* h = (uint16_t*)p.out + row * p.N + t.nt * 64 + 16 * wave;
                *(u32x4*)h = (u32x4){hv[0], hv[1], hv[2], hv[3]};
                *(u32x4*)(h + 8) = (u32x4){hv[4], hv[5], hv[6], hv[7]};
            }
        } else if (fr_ < rows_left) {
            // columns 32 wave + 8 j + 4 q + [0, 4)
            const int64_t col0 = t.nt * kMsBN + 32 * wave + 4 * q_;
            float* y = (float*)p.out + row * p.N + col0;
#pragma unroll
            for (int j = 0; j < 4; j++)
                if (col0 + 8 * j < p.N)
                    *(float4_t*)(y + 8 * j) = (float4_t){acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
        }
    };

    // ---- load cursor three stages ahead of the compute cursor; past the
    // last item it rereads that item's last stage (never computed) -------------
    int l_it = x_begin + slot, l_s = 0;
    setup_loads(item_of(l_it));
    auto load_next = [&](int set) {
        load_stage(l_s, set);
        if (++l_s == nst) {
            if (l_it + active < x_end) {
                l_it += active;
                setup_loads(item_of(l_it));
                l_s = 0;
            } else {
                l_s = nst - 1;
            }
        }
    };
    int c_it = x_begin + slot, c_s = 0;
    int total = 0;
    for (int it = c_it; it < x_end; it += active)
        total += nst;
    load_next(0);
    load_next(1);
    load_next(2);
    store_stage(0, 0, 0);
    __syncthreads();
    int g = 0;
    auto iter = [&](auto set_tag) {
        constexpr int cur = decltype(set_tag)::value;
        constexpr int nxt = (cur + 1) % 3;
        store_stage(nxt, (g + 1) & 1, g + 1);
        load_next(cur);
        compute(g & 1, g);
        __syncthreads();
        g++;
        if (++c_s == nst) {
            epilogue(item_of(c_it));
            acc = (float16_t){};
            c_it += active;
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
    if (MODE == kModeGateUp) {
        hmax = block_max_u32(hmax, &lds_sw[0][0]);
        if (tid == 0 && hmax != 0)
            atomicMax(p.h_amax, hmax << 16);
    }
    wait_vm<0>();  // the rereads past the last item
}

}  // namespace nvfp4
