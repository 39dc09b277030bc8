/*
 * nvfp4.h -- C ABI of libnvfp4: NVFP4 W4A4 quantization and the quantized
 * GEMMs it feeds, for AMD Instinct MI355X (gfx950).
 *
 * NVFP4 format (page "Qwen3.8-Flash-Next-NVFP4", section 核心: W4A4 two-level
 * scaling; page "DeepSeek-V4.1-Flash-NVFP4", section 二: E2M1 table and
 * packing).  A tensor of R x K values (K a multiple of 16, blocks of 16
 * contiguous elements along the last dimension) is stored as:
 *   packed  uint8 [R, K/2]   E2M1 codes (1 sign, 2 exponent, 1 mantissa
 *                            bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6),
 *                            element 2j in the low nibble of byte j
 *   scales  uint8 [R, K/16]  one FP8 E4M3 (bias 7, max 448) block scale per
 *                            16 elements, row-major (weights may also
 *                            be given in 128-row tiles: NVFP4_TILED_SCALES)
 *   global  float [1]        one FP32 per-tensor scale
 * and value = (e2m1 * scale) * global, i.e. 4.5 bits per element.  The three
 * buffers map onto a checkpoint's weight / weight_scale / weight_scale_2
 * tensors (page "Qwen3.8-27B-NVFP4", section 2).
 *
 * Conventions for every entry point:
 *   - All pointers are device pointers unless marked "host".  The caller owns
 *     every buffer; the library allocates no device memory.  Scratch memory
 *     is passed as (ws, ws_bytes); nvfp4_workspace_size() gives its size.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on that stream and never synchronizes the host, except
 *     nvfp4_get_error().  Global scales live in device memory, so dynamic
 *     scales never visit the host.
 *   - A tensor with no elements may pass null data pointers.
 *   - bf16 inputs must start on a 16-byte boundary and have a row stride
 *     (ld, in elements) that is a multiple of 8; packed buffers must be
 *     16-byte aligned and scale buffers 4-byte aligned.
 *   - Shape and argument errors are found on the host and returned before
 *     any launch.  Data-dependent errors (remap exponent spread, expert id
 *     out of range) set a sticky per-device error word that
 *     nvfp4_get_error() reads and clears.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified output.
 *   - The only host state is a per-device cache of occupancy queries,
 *     written with relaxed atomics (every thread computes the same value);
 *     calls on different streams may run concurrently as long as their
 *     buffers do not overlap.
 *
 * Arithmetic (bit-exact contract).  Quantization follows these fp32 steps,
 * each IEEE round-to-nearest-even, no fused multiply-add:
 *   G      = amax / 2688           (dynamic; 2688 = 6 * 448)  or a static G
 *   s_real = a_b / (6 * G)         a_b = max |x| over the 16-element block
 *   s      = E4M3 nearest-even to s_real, saturating at 448
 *   y      = x * (1 / (s * G))     (the reciprocal once per block)
 *   code   = E2M1 nearest-even to |y|, saturating at 6; sign = sign of x
 * A block whose scale rounds to 0 stores zero codes.  An all-zero tensor
 * gets G = 1.  Dequantization is v = (e2m1 * s) * G in fp32.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_INVALID_ARG = 1, /* null pointer, bad alignment, bad enum      */
    NVFP4_ERR_SHAPE = 2,       /* a size that breaks the layout rules        */
    NVFP4_ERR_RANGE = 3,       /* data outside what the format can hold      */
    NVFP4_ERR_WORKSPACE = 4,   /* ws too small                               */
    NVFP4_ERR_DEVICE = 5,      /* a HIP runtime error (launch, no device)    */
    NVFP4_ERR_UNSUPPORTED = 6, /* a valid request this build does not handle */
    NVFP4_ERR_DATA = 7         /* (checks on) non-finite input, NaN or negative
                                  block scale, global not finite and positive */
} nvfp4_status;

/* Output element types.  Entry points take them as int32_t, so that any value
 * a C caller passes is well defined to check (others: NVFP4_ERR_INVALID_ARG). */
typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;

/* One NVFP4 tensor, or `batch` tensors of the same shape stacked
 * contiguously (experts): packed [batch, rows, cols/2], scales
 * [batch, rows, cols/16], global [batch]. */
typedef struct {
    uint8_t* packed;
    uint8_t* scales;
    float* global;
    int64_t rows;
    int64_t cols;   /* multiple of 16 */
    int64_t batch;  /* >= 1 */
    uint32_t flags; /* NVFP4_POW2_SCALES or 0 (see below) */
} nvfp4_tensor;

/* nvfp4_tensor.flags: every block scale is a power of two (or zero).  The
 * library only reads it; the caller sets it on the output of
 * mxfp4_to_nvfp4 (whose scales are 2^k or zero by construction) and clears
 * it for tensors from nvfp4_quantize.  When a GEMM's weight operand carries
 * it, the weight block scale is folded into the fp4 -> f16 conversion
 * (which applies a power-of-two factor exactly) instead of a separate
 * multiply; the product is the same.  Setting it on a tensor with other
 * scales gives wrong results. */
#define NVFP4_POW2_SCALES 1u

/* nvfp4_tensor.flags: the scale bytes are stored in 128-row tiles instead of
 * row-major (set by nvfp4_tile_scales; the values, codes and globals are the
 * same).  For rows % 128 == 0 and cols % 256 == 0 only: scale byte b of row
 * r of matrix m (b < cols/16) is at
 *     m * rows * cols/16 + ((r/128 * cols/256 + b/16) * 128 + r%128) * 16 + b%16
 * so the 16 bytes that 256 consecutive elements of each of 128 rows use are
 * one contiguous 2 KB run.  A GEMM that streams a weight tile of 128 rows
 * then reads its scales in whole cache lines instead of a 16-byte piece per
 * row and stage.  This storage order is the library's own; the pages fix
 * the scale (one E4M3 per 16 elements along the last dimension), not where
 * it lives.  Accepted for the weight operand of nvfp4_gemm,
 * nvfp4_gemm_w4a16 and the NVFP4 MoE entry points (w13, w2); every other
 * tensor argument with this flag is refused (NVFP4_ERR_UNSUPPORTED), as is
 * a tiled tensor whose shape breaks the rule above (NVFP4_ERR_SHAPE). */
#define NVFP4_TILED_SCALES 2u

/* Operations for nvfp4_workspace_size(). */
enum {
    NVFP4_OP_QUANTIZE = 0, /* nvfp4_quantize                       */
    NVFP4_OP_REMAP = 1,    /* mxfp4_to_nvfp4 (T = batch)           */
    NVFP4_OP_GEMM = 2,     /* nvfp4_gemm                            */
    NVFP4_OP_MOE = 3,      /* nvfp4_moe_grouped_gemm                */
    NVFP4_OP_MOE_ROUTE = 4, /* nvfp4_moe_route / the staged GEMMs   */
    NVFP4_OP_MX_MOE = 5     /* mx_moe_w4a8                          */
};

/* Bytes of `ws` an operation needs.  Unused arguments may be 0:
 *   QUANTIZE: none.  REMAP: T = batch, H = rows, I = cols.
 *   GEMM: T = M (rows of A), H = K, I = N (rows of W); non-zero only for
 *         few-row shapes whose K is split over several workgroups.
 *   MOE, MOE_ROUTE: T tokens, k slots, E experts, H hidden, I intermediate. */
size_t nvfp4_workspace_size(int op, int64_t T, int32_t k, int32_t E, int64_t H, int64_t I);

/*
 * Quantize a bf16 matrix x [rows, cols] (row stride ld elements) to NVFP4
 * (page "Qwen3.8-Flash-Next-NVFP4", section 核心: level-1 E4M3 block scale
 * per 16 along the last dimension, level-2 FP32 tensor scale; weights
 * quantized once offline, activations per call).
 *   static_global: device float[1] holding G, or NULL for the dynamic
 *                  G = amax(x) / 2688 (computed on the device).
 *   out:           host struct; out->rows == rows, out->cols == cols,
 *                  out->batch == 1; G is written to out->global[0].
 *   ws:            nvfp4_workspace_size(NVFP4_OP_QUANTIZE) bytes (dynamic
 *                  only; may be NULL with a static global).
 * Errors: NVFP4_ERR_SHAPE if cols % 16 != 0 or ld < cols; INVALID_ARG for
 * null or misaligned pointers; WORKSPACE if ws is too small.
 */
nvfp4_status nvfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld,
                            const float* static_global, const nvfp4_tensor* out,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Dequantize an NVFP4 tensor (all batch matrices) to out [batch*rows, cols]
 * in fp32 or bf16 (nearest-even from the fp32 value (e2m1*s)*G)
 * (page "DeepSeek-V4.1-Flash-NVFP4", section 二: value = code x block scale
 * x tensor scale).
 */
nvfp4_status nvfp4_dequantize(const nvfp4_tensor* in, void* out, int32_t dtype, void* stream);

/*
 * Row gather-dequantize for NVFP4 embedding tables (page
 * "Qwen3.8-Flash-Next-FP4-Local", section 2.1: the n-gram embedding table
 * stored as NVFP4 with 16-element groups, rows of 2560 looked up per
 * token): out[i] = dequantize(table row ids[i]) for i < n, out
 * [n, cols] fp32 or bf16 with nvfp4_dequantize's value rule.  table: batch
 * 1 (one shard, one global); ids: int32 [n] on the device.  An id outside
 * [0, rows) gives a zero row and the sticky NVFP4_ERR_RANGE (the call itself
 * returns OK).  n * cols / 8 must stay below 2^32 (else UNSUPPORTED).
 */
nvfp4_status nvfp4_gather_dequantize(const nvfp4_tensor* table, const int32_t* ids, int64_t n,
                                     void* out, int32_t dtype, void* stream);

/* Tile the scale bytes of `in` (row-major: flags without NVFP4_TILED_SCALES)
 * into the 128-row order of NVFP4_TILED_SCALES, writing all
 * in->batch * rows * cols/16 bytes to scales_out (device, caller-owned, 16-byte
 * aligned, not overlapping in->scales).  The caller then describes the
 * tensor with in->packed, scales_out, in->global and flags |
 * NVFP4_TILED_SCALES.  For weights, done once when they are loaded.  Errors:
 * NVFP4_ERR_SHAPE unless rows % 128 == 0 and cols % 256 == 0;
 * NVFP4_ERR_INVALID_ARG for null or misaligned pointers or a tiled input. */
nvfp4_status nvfp4_tile_scales(const nvfp4_tensor* in, uint8_t* scales_out, void* stream);

/*
 * MXFP4 encode (OCP MX: blocks of 32 along the last dimension, UE8M0 scale
 * 2^(floor(log2 amax) - 2), E2M1 nearest-even codes saturating at 6; an
 * all-zero block stores scale byte 0) of a bf16 matrix [rows, cols].
 * cols % 32 == 0.  Outputs: packed [rows, cols/2], e8m0 [rows, cols/32].
 * This produces the MXFP4 checkpoints that mxfp4_to_nvfp4 consumes (page
 * "DeepSeek-V4.1-Flash-NVFP4", section 二, MXFP4 column of the table).
 */
nvfp4_status mxfp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld,
                            uint8_t* packed, uint8_t* e8m0, void* stream);

/*
 * Lossless MXFP4 -> NVFP4 remap (page "DeepSeek-V4.1-Flash-NVFP4", sections
 * 一, 二 and 四: block-wise remap that keeps every dequantized value).
 * Input: `batch` stacked MXFP4 matrices: mx_packed [batch, rows, cols/2],
 * e8m0 [batch, rows, cols/32]; cols % 32 == 0.  For each matrix:
 *   e_max = largest block exponent over blocks with a non-zero code
 *   G     = 2^(e_max - 8)
 *   both 16-halves of a non-zero block get the E4M3 scale 2^(e - e_max + 8)
 *   zero blocks get scale byte 0x01; a matrix with no non-zero block G = 1
 *   codes are copied unchanged (out->packed may equal mx_packed: then no
 *   copy is made).
 * A matrix whose non-zero block exponents spread over more than 17 octaves
 * cannot be held by E4M3 block scales: its out-of-range blocks get scale 0
 * and the sticky error NVFP4_ERR_RANGE is raised (see nvfp4_get_error).
 * A 0xFF (NaN) scale byte is treated the same way.
 * ws: nvfp4_workspace_size(NVFP4_OP_REMAP, batch, 0, 0, rows, cols) bytes.
 */
nvfp4_status mxfp4_to_nvfp4(const uint8_t* mx_packed, const uint8_t* e8m0,
                            int64_t rows, int64_t cols, int64_t batch,
                            const nvfp4_tensor* out, void* ws, size_t ws_bytes, void* stream);

/*
 * W4A4 GEMM (page "Qwen3.8-Flash-Next-NVFP4", section 核心: weights and
 * activations both NVFP4; page "DeepSeek-V4.1-Flash-NVFP4", section 二:
 * block scales applied inside the accumulation):
 *   C[m, n] = G_A * G_W * sum_k (e2m1*s)(A[m,k]) * (e2m1*s)(W[n,k])
 * A: [M, K] (batch 1), W: [N, K] (batch 1); C: [M, N] row-major, fp32 or
 * bf16.  Products are exact; the sum is accumulated in fp32.
 * K % 16 == 0 (a K that is not a multiple of 64 runs a slower kernel that
 * reads the last, partial 64-element stage block by block).
 * ws: nvfp4_workspace_size(NVFP4_OP_GEMM, M, 0, 0, K, N) bytes, 256-byte
 *     aligned, holding the fp32 partial sums of few-row shapes whose K is
 *     split over several workgroups (they are added in a fixed order, so
 *     results are reproducible).  NULL (or a size of 0) is allowed: the
 *     GEMM then runs unsplit, slower for such shapes.  A non-NULL ws that is
 *     smaller than required gives NVFP4_ERR_WORKSPACE.
 */
nvfp4_status nvfp4_gemm(const nvfp4_tensor* A, const nvfp4_tensor* W, void* C, int32_t dtype,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * MXFP8 activation encode for the MX-native W4A8 GEMM (page
 * "DeepSeek-V4.1-Flash-NVFP4", section 二: the reference FP8 x FP4 GEMM
 * quantizes activations in blocks with power-of-two scales).  Per block of
 * 32 elements along a row: scale 2^e, e the smallest integer with
 * amax <= 448 * 2^e (so no element saturates), clamped to [-127, 127]; an
 * all-zero block takes e = 0.  Elements x * 2^-e rounded to E4M3 (nearest,
 * ties to even; -0 keeps its sign).  x: bf16 [rows, cols] with row stride ld
 * (elements, ld % 8 == 0, 16-byte aligned); fp8: E4M3 bytes [rows, cols]
 * (16-byte aligned); e8m0: UE8M0 bytes [rows, cols / 32] (e + 127).
 * cols % 32 == 0.  Inputs must be finite.
 */
nvfp4_status mxfp8_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld, uint8_t* fp8,
                            uint8_t* e8m0, void* stream);

/*
 * MX-native W4A8 GEMM (page "DeepSeek-V4.1-Flash-NVFP4", section 二: MXFP4
 * weights, FP8 activations, the power-of-two block scales applied inside the
 * accumulation; the routed experts are MXFP4 in the original checkpoint):
 *   C[m, n] = sum over 32-element blocks b of K of
 *             2^(ea[m,b] - 127) * 2^(ew[n,b] - 127) * sum_{k in b} a[m,k] * w[n,k]
 * a: E4M3 [M, K] and a_e8m0 [M, K/32] (as from mxfp8_quantize); w: MXFP4
 * codes [N, K/2] (element 2j in the low nibble of byte j) and w_e8m0
 * [N, K/32] (as from mxfp4_quantize); C: [M, N] row-major, fp32 or bf16.
 * Runs on the scaled FP8 x FP4 MFMA with no decode (its internal sum is
 * not exact fp32: about 6e-5 relative per 64-element step).  K % 128 == 0
 * on this build (else NVFP4_ERR_UNSUPPORTED); a and w 16-byte aligned,
 * the scale arrays 4-byte aligned.
 */
nvfp4_status mx_gemm_w4a8(const uint8_t* a_fp8, const uint8_t* a_e8m0, int64_t M, int64_t K,
                          const uint8_t* w_packed, const uint8_t* w_e8m0, int64_t N, void* C, int32_t dtype,
                          void* stream);

/*
 * MX-native W4A8 routed-expert layer (page "DeepSeek-V4.1-Flash-NVFP4",
 * section 二: MXFP4 expert weights with FP8 activations; the layer as the
 * NVFP4 one, page "Qwen3.8-Flash-Next-NVFP4", section 核心):
 *   1. route the T x k (token, slot) pairs by expert (as nvfp4_moe_route);
 *   2. x (bf16 [T, H]) -> MXFP8 (as mxfp8_quantize);
 *   3. per pair (t, j) with e = ids[t, j]: g || u = the MX GEMM of x row t
 *      with w13[e] (gate rows 0..I-1, up rows I..2I-1), h = bf16(silu(g) u);
 *   4. h -> MXFP8 (as mxfp8_quantize, rows in list order);
 *   5. y = the MX GEMM of the h row with w2[e] (fp32);
 *   6. out[t] = bf16(sum_j w[t, j] y[t, j]), j ascending, in fp32.
 * w13: MXFP4 codes [E, 2I, H/2] and UE8M0 scales [E, 2I, H/32]; w2: codes
 * [E, H, I/2] and scales [E, H, I/32] (as from mxfp4_quantize per expert).
 * ids int32 [T, k] in [0, E) (others raise NVFP4_ERR_RANGE and the pair
 * is dropped); w fp32 [T, k]; out bf16 [T, H] (16-byte aligned).
 * H % 256 == 0 and I % 128 == 0 on this build (else NVFP4_ERR_UNSUPPORTED).
 * ws: nvfp4_workspace_size(NVFP4_OP_MX_MOE, T, k, E, H, I) bytes, 256-byte
 * aligned, caller-owned; too small gives NVFP4_ERR_WORKSPACE.
 */
/*
 * The two projections of mx_moe_w4a8 on their own (steps 3 and 5 there), for
 * staged use and parity tests, with perm / offsets as from nvfp4_moe_route:
 *   mx_moe_gate_up: x MXFP8 [T, H] (E4M3 codes, UE8M0 [T, H/32]) -> h bf16
 *     [T*k, I] in list order; max |h| as float bits goes to *h_amax by
 *     atomic max (the caller zeroes it first).
 *   mx_moe_down: h MXFP8 [T*k, I] in list order -> y fp32 [T*k, H].
 * Shapes, alignment and errors as mx_moe_w4a8; ws: as nvfp4_moe_route.
 */
nvfp4_status mx_moe_gate_up(const uint8_t* x_fp8, const uint8_t* x_e8m0, const int32_t* perm,
                            const int32_t* offsets, int64_t T, int32_t k, int32_t E, int64_t H, int64_t I,
                            const uint8_t* w13_packed, const uint8_t* w13_e8m0, void* h_bf16, uint32_t* h_amax,
                            void* ws, size_t ws_bytes, void* stream);
nvfp4_status mx_moe_down(const uint8_t* h_fp8, const uint8_t* h_e8m0, const int32_t* offsets, int64_t T, int32_t k,
                         int32_t E, int64_t H, int64_t I, const uint8_t* w2_packed, const uint8_t* w2_e8m0,
                         float* y, void* ws, size_t ws_bytes, void* stream);

nvfp4_status mx_moe_w4a8(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, int64_t T, int32_t k,
                         int32_t E, int64_t H, int64_t I, const uint8_t* w13_packed, const uint8_t* w13_e8m0,
                         const uint8_t* w2_packed, const uint8_t* w2_e8m0, void* out_bf16, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * W4A16 GEMM (page "Qwen3.8-Flash-Next-FP4-Local", section 3.2: routed
 * experts of the MTP head keep their activations in BF16 and only the
 * weights in NVFP4):
 *   C[m, n] = G_W * sum_k A[m, k] * (e2m1*s)(W[n, k])
 * A: bf16 [M, K] with row stride lda (elements, lda >= K, lda % 8 == 0,
 * 16-byte aligned); W: [N, K] (batch 1); C: [M, N] row-major, fp32 or bf16.
 * The weights are decoded exactly to bf16 and multiplied on the bf16 MFMA
 * path: products are exact, the sum is accumulated in fp32.  Every M runs
 * the weight-streaming kernel (16 rows of A per tile): the format serves
 * decode-sized batches.  K % 256 == 0 on this build (else
 * NVFP4_ERR_UNSUPPORTED).  ws: as nvfp4_gemm (nvfp4_workspace_size
 * (NVFP4_OP_GEMM, M, 0, 0, K, N) bytes, or NULL).
 */
nvfp4_status nvfp4_gemm_w4a16(const void* a_bf16, int64_t M, int64_t K, int64_t lda, const nvfp4_tensor* W,
                              void* C, int32_t dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * W4A16 routed-expert MoE layer (page "Qwen3.8-Flash-Next-FP4-Local",
 * section 3.2: W4A16_NVFP4 MTP experts): as nvfp4_moe_grouped_gemm without
 * the activation quantization: route, gate_up from the bf16 rows of x
 * (g || u = x[t] W13[e]^T, h = silu(g) * u rounded to bf16), down from the
 * bf16 h rows (y = h W2[e]^T, fp32), combine out[t] = sum_j topk_w[t, j]
 * y[t, j] (j in order) rounded to bf16.  Arguments and ws as
 * nvfp4_moe_grouped_gemm (nvfp4_workspace_size(NVFP4_OP_MOE, ...)).
 * H % 256 == 0 and I % 256 == 0 on this build (else NVFP4_ERR_UNSUPPORTED).
 */
nvfp4_status nvfp4_moe_w4a16(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, int64_t T,
                             int32_t k, int32_t E, const nvfp4_tensor* w13, const nvfp4_tensor* w2,
                             void* out_bf16, void* ws, size_t ws_bytes, void* stream);

/*
 * Routed-expert MoE layer with NVFP4 experts (page "Qwen3.8-Flash-Next-NVFP4":
 * routed experts with fused gate_up / down projections, top-k routing; page
 * "DeepSeek-V4.1-Flash-NVFP4", section 三: experts w1, w3, w2):
 *   1. route: stable token-by-expert permutation of the T*k (token, slot)
 *      pairs (nvfp4_moe_route);
 *   2. quantize x [T, H] once (dynamic G_x, or static_in_globals[0]);
 *   3. gate_up: for each pair (t, j) with expert e = topk_ids[t, j],
 *      g || u = xq[t] W13[e]^T (W13[e] is [2I, H]: rows [0, I) gate (w1),
 *      rows [I, 2I) up (w3)), h = silu(g) * u rounded to bf16;
 *   4. quantize h over all T*k rows (dynamic G_h = amax(h)/2688, or
 *      static_in_globals[1]: then step 3's epilogue encodes h to NVFP4
 *      directly, as nvfp4_moe_gate_up_q, with the same bytes);
 *   5. down: y = hq W2[e]^T (W2[e] is [H, I]), fp32;
 *   6. combine: out[t] = sum_j topk_w[t, j] * y[t, j] (j in order, fp32),
 *      rounded to bf16.
 * topk_ids int32 [T, k] in [0, E) (others raise the sticky RANGE error and
 * the pair is dropped); topk_w fp32 [T, k]; x bf16 [T, H] contiguous;
 * w13: batch E, rows 2I, cols H; w2: batch E, rows H, cols I;
 * static_in_globals: device float[2] or NULL; out bf16 [T, H].
 * H % 16 == 0 and I % 16 == 0 (else NVFP4_ERR_SHAPE); H % 64 != 0 or
 * I % 128 != 0 runs every row in slower 32-row tiles.
 * ws: nvfp4_workspace_size(NVFP4_OP_MOE, T, k, E, H, I) bytes.
 */
nvfp4_status nvfp4_moe_grouped_gemm(const void* x_bf16, const int32_t* topk_ids,
                                    const float* topk_w, int64_t T, int32_t k, int32_t E,
                                    const nvfp4_tensor* w13, const nvfp4_tensor* w2,
                                    const float* static_in_globals, void* out_bf16,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * nvfp4_moe_grouped_gemm without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus ws), same
 * kernels and bit-identical output; the workspace is a library-owned device
 * array of nvfp4_noalloc_scratch_bytes() bytes (32 MiB) per GPU, held from
 * the library's first use on that GPU until the process ends.  A layer whose
 * workspace (nvfp4_workspace_size(NVFP4_OP_MOE, ...)) exceeds it gives
 * NVFP4_ERR_WORKSPACE before any launch (decode-sized batches fit: the
 * 384-expert T = 64 layer needs 18 MB).  No call allocates or frees.  Every
 * call on a GPU shares that GPU's array, which keeps the previous call's
 * contents (nothing in it needs to start at zero): calls that overlap in
 * time on one GPU -- on different streams or from different host threads --
 * race and give undefined results.
 */
nvfp4_status nvfp4_moe_grouped_gemm_noalloc(const void* x_bf16, const int32_t* topk_ids,
                                            const float* topk_w, int64_t T, int32_t k, int32_t E,
                                            const nvfp4_tensor* w13, const nvfp4_tensor* w2,
                                            const float* static_in_globals, void* out_bf16, void* stream);

/* Host: bytes of the per-GPU scratch array of nvfp4_moe_grouped_gemm_noalloc. */
size_t nvfp4_noalloc_scratch_bytes(void);

/* ---- staged MoE entry points (the steps of nvfp4_moe_grouped_gemm) ---- */

/*
 * Token-by-expert permutation: pairs p = t*k + j listed expert by expert,
 * increasing p within an expert.  perm int32 [T*k] (list position -> p),
 * offsets int32 [E+1] (first list position of each expert, offsets[E] =
 * number of valid pairs), inv int32 [T*k] (p -> list position, -1 for a
 * dropped pair).  ws: nvfp4_workspace_size(NVFP4_OP_MOE_ROUTE, T, k, E, 0, 0).
 */
nvfp4_status nvfp4_moe_route(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                             int32_t* perm, int32_t* offsets, int32_t* inv,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * gate_up + SwiGLU for every listed pair: h[q] = bf16(silu(g) * u) with
 * g || u = xq[perm[q] / k] W13[e]^T, e the expert owning list position q.
 * xq: NVFP4 [T, H]; h: bf16 [T*k, I] in list order.  h_amax: device uint32
 * that receives max |h| as float bits via atomic max (the caller zeroes it
 * first).  ws: as nvfp4_moe_route.
 */
nvfp4_status nvfp4_moe_gate_up(const nvfp4_tensor* xq, const int32_t* perm,
                               const int32_t* offsets, int64_t T, int32_t k, int32_t E,
                               const nvfp4_tensor* w13, void* h_bf16, uint32_t* h_amax,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * gate_up + SwiGLU with the NVFP4 encode of h fused into the epilogue, for a
 * calibrated (static) activation global G_h, as the checkpoints' per-layer
 * input scales allow (page "Qwen3.8-Flash-Next-NVFP4", section 核心: static
 * activation scales calibrated from the max; page "Qwen3.8-27B-NVFP4",
 * section 2: input_scale in the checkpoint).  hq receives the bytes that
 * nvfp4_quantize(h, static_global = h_global) would give for the h of
 * nvfp4_moe_gate_up: codes [T*k, I/2] and scales [T*k, I/16] in list
 * order; no bf16 h is written and no max is taken.  h_global: device
 * float[1]; hq: rows T*k, cols I, batch 1 (hq->global is not written; point
 * it at h_global for nvfp4_moe_down).  ws: as nvfp4_moe_route.
 */
nvfp4_status nvfp4_moe_gate_up_q(const nvfp4_tensor* xq, const int32_t* perm,
                                 const int32_t* offsets, int64_t T, int32_t k, int32_t E,
                                 const nvfp4_tensor* w13, const float* h_global,
                                 const nvfp4_tensor* hq, void* ws, size_t ws_bytes, void* stream);

/*
 * down projection for every listed pair: y[q] = hq[q] W2[e]^T (fp32
 * [T*k, H], list order).  hq: NVFP4 [T*k, I].  ws: as nvfp4_moe_route.
 */
nvfp4_status nvfp4_moe_down(const nvfp4_tensor* hq, const int32_t* offsets, int64_t T,
                            int32_t k, int32_t E, const nvfp4_tensor* w2, float* y,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Router-weighted combine: out[t] = bf16(sum_{j=0..k-1} w[t,j] * y[inv[t*k+j]])
 * in fp32, j ascending; pairs with inv = -1 are skipped.
 */
nvfp4_status nvfp4_moe_combine(const float* y, const int32_t* inv, const float* topk_w,
                               int64_t T, int32_t k, int64_t H, void* out_bf16, void* stream);

/*
 * NVFP4 KV cache (page "Qwen3.8-2.4T-A95B-NVFP4": K and V stored at about 4
 * bits; 4 KV heads x 256 head_dim per token).  A cache tensor holds rows
 * (token, head) x head_dim columns: rows = capacity_tokens * heads, batch 1,
 * and its global[0] is the static per-tensor G set by the caller before the
 * first write.  kv_quant quantizes n tokens of k and v (bf16 [n, heads,
 * head_dim], contiguous) with those globals and stores them at token offset
 * tok_offset, in one launch.  Either of k/v may be NULL to skip it.
 */
nvfp4_status nvfp4_kv_quant(const void* k_bf16, const void* v_bf16, int64_t n, int64_t heads,
                            int64_t tok_offset, const nvfp4_tensor* k_cache,
                            const nvfp4_tensor* v_cache, void* stream);

/* Dequantize tokens [tok_begin, tok_begin + n) of the caches to k_out, v_out
 * ([n, heads, head_dim], fp32 or bf16); either may be NULL to skip it. */
nvfp4_status nvfp4_kv_dequant(const nvfp4_tensor* k_cache, const nvfp4_tensor* v_cache,
                              int64_t heads, int64_t tok_begin, int64_t n, void* k_out,
                              void* v_out, int32_t dtype, void* stream);

/*
 * Scale audit (page "Qwen3.8-Flash-Next-NVFP4", section 证据链: every block
 * scale finite and positive, maximum 448).  counts_out: device int64[4] =
 * {scale bytes, non-finite (NaN pattern), non-positive (zero or negative),
 * equal to 448}, over all batch matrices; overwritten.
 */
nvfp4_status nvfp4_audit_scales(const nvfp4_tensor* t, int64_t* counts_out, void* stream);

/* Synchronize `stream`, then read and clear the sticky device error word of
 * the current device: NVFP4_OK or the first data-dependent error raised
 * since the last call. */
nvfp4_status nvfp4_get_error(void* stream);

/* Static description of a status code (any int32_t; unknown codes give
 * "unknown status"). */
const char* nvfp4_status_string(int32_t s);

/* Format constants, host: block size 16, E2M1 exponent/mantissa bits 2/1,
 * E4M3 exponent/mantissa bits 4/3, effective bits x 100 (450). */
void nvfp4_recipe(int32_t out[6]);

/* Data checks (the release audit of page "Qwen3.8-Flash-Next-NVFP4", section
 * 证据链, applied to every call): while on, the quantize, dequantize, GEMM
 * and routed-expert entry points first launch checks of their operands --
 * bf16 inputs finite, every E4M3 block scale neither a NaN pattern nor
 * negative, every fp32 global finite and positive -- that raise the sticky
 * NVFP4_ERR_DATA (read with nvfp4_get_error); the computation still runs.
 * Expert ids are always checked (NVFP4_ERR_RANGE).  Off by default; on when
 * the library was built with -DNVFP4_CHECK=1 or the environment variable
 * NVFP4_CHECK is 1 when the library is loaded.  Host: sets the switch for
 * the process (on != 0), returns the previous setting. */
int nvfp4_set_checks(int on);

/* Host: a hash of the sources and flags this library was built from (16 hex
 * digits, static storage).  Loaders compare it with their source tree and
 * refuse a stale build. */
const char* nvfp4_build_stamp(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
