/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for the NVFP4 W4A4 hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (libnvfp4 and its Python binding) never links, imports or calls it, and it
 * shares no code, header or table with the HIP kernels.
 *
 * Sources (the five web pages on NVFP4 checkpoints):
 *   [FlashNext]  "Qwen3.8-Flash-Next-NVFP4", section "核心: W4A4 双级缩放机制拆解"
 *                (level-1 block scale, level-2 global scale, 4.5 bits, A4 dynamic)
 *                and section "证据链" (scale audit, max scale 448).
 *   [DSV41]      "DeepSeek-V4.1-Flash-NVFP4", section 二 (E2M1 magnitudes, two
 *                codes per byte, MXFP4 vs NVFP4 table), sections 一/四/六
 *                (lossless block-wise MXFP4 -> NVFP4 remap).
 *   [A95B]       "Qwen3.8-2.4T-A95B-NVFP4" (NVFP4 KV cache, 4 KV heads x 256).
 *   [27B]        "Qwen3.8-27B-NVFP4", section 2 (NVFP4 MLP, hidden 5120 /
 *                intermediate 17408; weight / weight_scale / weight_scale_2).
 *   [Local]      "Qwen3.8-Flash-Next-FP4-Local", section 3.2 (W4A16 NVFP4
 *                MTP experts: NVFP4 weights, BF16 activations).
 *
 * Arithmetic rules.  Every float operation is one IEEE binary32 operation,
 * correctly rounded to nearest-even; the file must be built with
 * -ffp-contract=off (no fused multiply-add) and without fast-math.  Where
 * the pages leave an order of operations open, the order used here is the
 * stated reading (each function documents it).  Codecs are brute-force
 * nearest-value searches over enumerated value tables.
 *
 * Return codes: 0 ok, 1 invalid argument, 2 shape, 3 range.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_INVALID 1
#define ORC_SHAPE 2
#define ORC_RANGE 3

/* ------------------------------------------------------------------------ */
/* Value tables                                                             */
/* ------------------------------------------------------------------------ */

/* The eight non-negative E2M1 magnitudes, in code order 0..7 ([DSV41] §二).
 * Bit 3 of a 4-bit code is the sign. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(uint8_t nibble)
{
    double m = E2M1_MAG[nibble & 7];
    return (nibble & 8) ? -m : m;
}

/* FP8 E4M3 ("scale_bits [4,3]" in [FlashNext] §核心): sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals for exponent field 0, no
 * infinities, and S.1111.111 is NaN.  The largest finite value is 448, the
 * maximum the scale audit of [FlashNext] reports. */
double orc_e4m3_value(uint8_t byte)
{
    int sign = byte >> 7;
    int e = (byte >> 3) & 15;
    int m = byte & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);            /* (m/8) * 2^(1-7) */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* UE8M0 (the MXFP4 block scale of [DSV41] §二): 2^(byte-127); 0xFF is NaN. */
double orc_e8m0_value(uint8_t byte)
{
    if (byte == 0xFF)
        return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* bf16 bits -> float (exact: bf16 is the upper half of a binary32). */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Value of a non-negative bf16 magnitude pattern in 0x0000..0x7F80; the
 * infinity pattern is given the value 2^128 (the next power of two past the
 * largest finite bf16), which is where IEEE rounding places the overflow
 * threshold. */
static double bf16_mag_value(uint32_t bits)
{
    if (bits >= 0x7F80)
        return ldexp(1.0, 128);
    return (double)bf16_to_float((uint16_t)bits);
}

/* Round a double to bf16: nearest value, ties to the even pattern, overflow
 * to infinity.  Binary search for the largest finite magnitude pattern not
 * above |v|, then pick the nearer of it and its successor. */
uint16_t orc_bf16_from_double(double v)
{
    uint32_t lo = 0, hi = 0x7F7F, mid, pick;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v), dlo, dhi;
    if (isnan(v))
        return 0x7FC0;
    if (a >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80);
    while (lo < hi) { /* invariant: value(lo) <= a */
        mid = (lo + hi + 1) / 2;
        if (bf16_mag_value(mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    dlo = a - bf16_mag_value(lo);
    dhi = bf16_mag_value(lo + 1) - a;
    if (dlo < dhi || (dlo == dhi && (lo & 1) == 0))
        pick = lo;
    else
        pick = lo + 1;
    return (uint16_t)(sign | pick);
}

/* ------------------------------------------------------------------------ */
/* Codecs: brute-force nearest search                                       */
/* ------------------------------------------------------------------------ */

/* Nearest non-negative finite E4M3 value (codes 0x00..0x7E) to s >= 0.
 * Equidistant candidates: the even code wins (round half to even on the
 * 3-bit mantissa).  s >= 448 saturates to 0x7E. */
uint8_t orc_e4m3_encode(float s)
{
    int c, best = 0;
    double bd = INFINITY;
    if (s >= 448.0f)
        return 0x7E;
    for (c = 0; c <= 0x7E; c++) {
        double d = fabs((double)s - orc_e4m3_value((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)best;
}

/* Nearest E2M1 magnitude code (0..7) to a >= 0.  Equidistant candidates:
 * the even code wins; a > 6 saturates to code 7 (6.0).  A NaN (only
 * produced by 0 * inf, see orc_quantize) gives code 0. */
uint8_t orc_e2m1_encode(float a)
{
    int c, best = 0;
    double bd = INFINITY;
    if (isnan(a))
        return 0;
    if (a > 6.0f)
        return 7;
    for (c = 0; c < 8; c++) {
        double d = fabs((double)a - E2M1_MAG[c]);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)best;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 quantize / dequantize                                              */
/* ------------------------------------------------------------------------ */

/* Per-tensor global from the tensor maximum: G = amax / (6 * 448) so that the
 * largest block scale lands on the E4M3 maximum ([FlashNext] §核心 level 2;
 * 6 is the largest E2M1 magnitude, 448 the largest E4M3 value).  An all-zero
 * tensor gets G = 1. */
float orc_global_from_amax(float amax)
{
    return amax > 0.0f ? amax / 2688.0f : 1.0f;
}

/* max |x| over an R x K bf16 matrix with row stride ld (exact). */
float orc_amax_bf16(const uint16_t* x, int64_t R, int64_t K, int64_t ld)
{
    float amax = 0.0f;
    int64_t r, k;
    for (r = 0; r < R; r++)
        for (k = 0; k < K; k++) {
            float a = fabsf(bf16_to_float(x[r * ld + k]));
            if (a > amax)
                amax = a;
        }
    return amax;
}

/*
 * NVFP4 quantization of an R x K bf16 matrix (row stride ld elements).
 * Blocks are 16 contiguous elements along the last dimension ([FlashNext]
 * §核心 level 1).  For every block b of row r:
 *   a_b    = max |x| over the block                       (exact)
 *   s_real = a_b / (6 * G)            (one fp32 multiply, then one divide)
 *   s      = nearest E4M3 to s_real, stored as the scale byte
 *   if s == 0: every code is 0 (sign kept)
 *   else     : r = 1 / (s * G)        (fp32 multiply, then divide)
 *              code_i = nearest E2M1 magnitude to |x_i * r|
 *   nibble_i = signbit(x_i) << 3 | code_i ; element 2j -> low nibble of byte j
 * G is static_G[0] when static_G != NULL, else the dynamic global of
 * orc_global_from_amax().  Outputs: packed [R, K/2], scales [R, K/16], G.
 */
int orc_quantize(const uint16_t* x, int64_t R, int64_t K, int64_t ld,
                 const float* static_G, uint8_t* packed, uint8_t* scales,
                 float* G_out)
{
    int64_t r, b, i;
    float G, six_g;
    if (K % 16 != 0 || R < 0 || K < 0 || ld < K)
        return ORC_SHAPE;
    for (r = 0; r < R; r++)
        for (i = 0; i < K; i++)
            if (!isfinite(bf16_to_float(x[r * ld + i])))
                return ORC_INVALID;
    if (static_G) {
        G = static_G[0];
        if (!(G > 0.0f) || !isfinite(G))
            return ORC_INVALID;
    } else {
        G = orc_global_from_amax(orc_amax_bf16(x, R, K, ld));
    }
    *G_out = G;
    six_g = 6.0f * G;
    for (r = 0; r < R; r++) {
        for (b = 0; b < K / 16; b++) {
            const uint16_t* xb = x + r * ld + b * 16;
            float ab = 0.0f, s_real, s, rinv = 0.0f;
            uint8_t sbyte, nib[16];
            for (i = 0; i < 16; i++) {
                float a = fabsf(bf16_to_float(xb[i]));
                if (a > ab)
                    ab = a;
            }
            s_real = ab / six_g;
            sbyte = orc_e4m3_encode(s_real);
            s = (float)orc_e4m3_value(sbyte);
            if (sbyte != 0) {
                float p = s * G;
                rinv = 1.0f / p;
            }
            for (i = 0; i < 16; i++) {
                float xv = bf16_to_float(xb[i]);
                uint8_t code = 0;
                if (sbyte != 0) {
                    float y = xv * rinv;
                    code = orc_e2m1_encode(fabsf(y));
                }
                nib[i] = (uint8_t)((signbit(xv) ? 8 : 0) | code);
            }
            scales[r * (K / 16) + b] = sbyte;
            for (i = 0; i < 8; i++)
                packed[r * (K / 2) + b * 8 + i] =
                    (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
        }
    }
    return ORC_OK;
}

/* Dequantize: v = (e2m1(code) * s) * G in fp32 (the first product is exact).
 * out_f32 [R, K] row-major; out_bf16 (optional) gets the same values
 * rounded to nearest-even bf16. */
int orc_dequantize(const uint8_t* packed, const uint8_t* scales, float G,
                   int64_t R, int64_t K, float* out_f32, uint16_t* out_bf16)
{
    int64_t r, k;
    if (K % 16 != 0)
        return ORC_SHAPE;
    for (r = 0; r < R; r++)
        for (k = 0; k < K; k++) {
            uint8_t byte = packed[r * (K / 2) + k / 2];
            uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
            float q = (float)orc_e2m1_value(nib);
            float s = (float)orc_e4m3_value(scales[r * (K / 16) + k / 16]);
            float qs = q * s;
            float v = qs * G;
            if (out_f32)
                out_f32[r * K + k] = v;
            if (out_bf16)
                out_bf16[r * K + k] = orc_bf16_from_double((double)v);
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Exact W4A4 GEMM                                                          */
/* ------------------------------------------------------------------------ */

/* Integer image of one dequantized element without its global:
 *   (2 * e2m1(code)) * (2^9 * s)
 * 2*e2m1 is an integer in [-12, 12]; 2^9 * s is an integer in [0, 229376]
 * for every finite E4M3 s, so the product is an exact integer < 2^22. */
static int64_t int_unit(uint8_t nibble, uint8_t sbyte)
{
    double q2 = 2.0 * orc_e2m1_value(nibble);
    double s9 = ldexp(orc_e4m3_value(sbyte), 9);
    return (int64_t)q2 * (int64_t)s9;
}

static void unpack_row_int(const uint8_t* packed, const uint8_t* scales,
                           int64_t row, int64_t K, int64_t* out)
{
    int64_t k;
    for (k = 0; k < K; k++) {
        uint8_t byte = packed[row * (K / 2) + k / 2];
        uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
        out[k] = int_unit(nib, scales[row * (K / 16) + k / 16]);
    }
}

/*
 * Exact W4A4 product of two NVFP4 operands (W4A4 of [FlashNext] §核心, per-block
 * scales applied inside the sum as in [DSV41] §二):
 *   C[m, n] = Ga * Gw * sum_k deq0(A[m,k]) * deq0(W[n,k])
 * where deq0 is the dequantized element without its global.  The sum is an
 * int64 sum of the integer images (|sum| < 2^59 for K <= 2^15) scaled by
 * 2^-20, then by Ga * Gw in double: the exact result rounded once to double.
 * A rows are taken from a_rows[i] (i < n_a); W rows from w_rows[j] (j < n_w).
 * W is [.., K] row-major, i.e. C = A * W^T.  C is [n_a, n_w] row-major.
 */
int orc_gemm_rows(const uint8_t* Ap, const uint8_t* As, float Ga,
                  const int64_t* a_rows, int64_t n_a,
                  const uint8_t* Wp, const uint8_t* Ws, float Gw,
                  const int64_t* w_rows, int64_t n_w, int64_t K, double* C)
{
    int64_t i, j, k;
    int64_t *ai, *wi;
    double scale;
    if (K % 16 != 0 || K > 32768)
        return ORC_SHAPE;
    ai = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
    wi = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1) *
                          (size_t)(n_w > 0 ? n_w : 1));
    if (!ai || !wi) {
        free(ai);
        free(wi);
        return ORC_INVALID;
    }
    for (j = 0; j < n_w; j++)
        unpack_row_int(Wp, Ws, w_rows[j], K, wi + j * K);
    scale = ldexp(1.0, -20) * (double)Ga * (double)Gw;
    for (i = 0; i < n_a; i++) {
        unpack_row_int(Ap, As, a_rows[i], K, ai);
        for (j = 0; j < n_w; j++) {
            const int64_t* w = wi + j * K;
            int64_t acc = 0;
            for (k = 0; k < K; k++)
                acc += ai[k] * w[k];
            C[i * n_w + j] = (double)acc * scale;
        }
    }
    free(ai);
    free(wi);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 (OCP MX, block 32, UE8M0) and the lossless remap                   */
/* ------------------------------------------------------------------------ */

/*
 * MXFP4 encode ([DSV41] §二 table: block 32, power-of-two UE8M0 scale),
 * following the OCP MX rule: the block's shared exponent is
 * floor(log2(amax)) - 2 (2 = exponent of the largest E2M1 magnitude),
 * clamped to the UE8M0 range, and each element is the nearest E2M1
 * magnitude to |x| / 2^e (ties to even, saturating at 6).  An all-zero block
 * stores scale byte 0 and zero codes.  Sign nibble bit = signbit(x).
 */
int orc_mxfp4_encode(const uint16_t* x, int64_t R, int64_t K, int64_t ld,
                     uint8_t* packed, uint8_t* e8m0)
{
    int64_t r, b, i;
    if (K % 32 != 0 || ld < K)
        return ORC_SHAPE;
    for (r = 0; r < R; r++) {
        for (b = 0; b < K / 32; b++) {
            const uint16_t* xb = x + r * ld + b * 32;
            float amax = 0.0f;
            int e = 0, p;
            uint8_t nib[32];
            for (i = 0; i < 32; i++) {
                float a = fabsf(bf16_to_float(xb[i]));
                if (!isfinite(a))
                    return ORC_INVALID;
                if (a > amax)
                    amax = a;
            }
            if (amax > 0.0f) {
                (void)frexp((double)amax, &p); /* amax = f * 2^p, f in [0.5,1) */
                e = (p - 1) - 2;
                if (e < -127)
                    e = -127;
                if (e > 127)
                    e = 127;
                e8m0[r * (K / 32) + b] = (uint8_t)(e + 127);
            } else {
                e8m0[r * (K / 32) + b] = 0;
            }
            for (i = 0; i < 32; i++) {
                float xv = bf16_to_float(xb[i]);
                uint8_t code = 0;
                if (amax > 0.0f) {
                    /* |x| / 2^e is exact and below 8 (or below 2^-124 * 2^127
                     * when the exponent was clamped), so the float is exact */
                    double y = ldexp(fabs((double)xv), -e);
                    code = orc_e2m1_encode((float)y);
                }
                nib[i] = (uint8_t)((signbit(xv) ? 8 : 0) | code);
            }
            for (i = 0; i < 16; i++)
                packed[r * (K / 2) + b * 16 + i] =
                    (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
        }
    }
    return ORC_OK;
}

/* MXFP4 dequantize: v = e2m1(code) * 2^(byte-127) in fp32. */
int orc_mxfp4_dequantize(const uint8_t* packed, const uint8_t* e8m0,
                         int64_t R, int64_t K, float* out)
{
    int64_t r, k;
    if (K % 32 != 0)
        return ORC_SHAPE;
    for (r = 0; r < R; r++)
        for (k = 0; k < K; k++) {
            uint8_t byte = packed[r * (K / 2) + k / 2];
            uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
            double v = orc_e2m1_value(nib) *
                       orc_e8m0_value(e8m0[r * (K / 32) + k / 32]);
            out[r * K + k] = (float)v;
        }
    return ORC_OK;
}

/*
 * Lossless MXFP4 -> NVFP4 remap of one R x K tensor ([DSV41] §一, §二, §四).
 * The E2M1 codes are kept byte for byte.  Every MX block scale 2^e becomes
 * G * s with G a power of two shared by the tensor and s an E4M3 power of
 * two, so the dequantized value of every element is unchanged.
 *   e_max = the largest exponent over blocks with a non-zero code
 *   G     = 2^(e_max - 8)      (the largest block maps to s = 256, the
 *                              largest power of two that E4M3 holds)
 *   s     = 2^(e - e_max + 8) for both 16-element halves of a non-zero
 *           block; it must be >= 2^-9 (smallest E4M3), i.e. the tensor's
 *           exponents may spread over at most 17 octaves, else ORC_RANGE
 *   zero blocks (all codes +-0) get scale byte 0x01; a tensor with no
 *   non-zero block gets G = 1.
 * A NaN scale byte (0xFF) gives ORC_INVALID.
 */
int orc_mxfp4_to_nvfp4(const uint8_t* mx_packed, const uint8_t* e8m0,
                       int64_t R, int64_t K, uint8_t* packed,
                       uint8_t* scales, float* G_out)
{
    int64_t r, b, i;
    int have = 0, e_max = -1000;
    if (K % 32 != 0)
        return ORC_SHAPE;
    for (r = 0; r < R; r++)
        for (b = 0; b < K / 32; b++) {
            const uint8_t* pb = mx_packed + r * (K / 2) + b * 16;
            int nz = 0;
            uint8_t sb = e8m0[r * (K / 32) + b];
            if (sb == 0xFF)
                return ORC_INVALID;
            for (i = 0; i < 16; i++)
                if ((pb[i] & 0x77) != 0)
                    nz = 1;
            if (nz) {
                int e = (int)sb - 127;
                have = 1;
                if (e > e_max)
                    e_max = e;
            }
        }
    if (!have) {
        *G_out = 1.0f;
    } else {
        *G_out = (float)ldexp(1.0, e_max - 8);
    }
    for (r = 0; r < R; r++)
        for (b = 0; b < K / 32; b++) {
            const uint8_t* pb = mx_packed + r * (K / 2) + b * 16;
            int nz = 0;
            uint8_t out_byte = 0x01;
            for (i = 0; i < 16; i++)
                if ((pb[i] & 0x77) != 0)
                    nz = 1;
            if (nz) {
                int d = ((int)e8m0[r * (K / 32) + b] - 127) - e_max + 8;
                if (d < -9)
                    return ORC_RANGE;
                out_byte = orc_e4m3_encode((float)ldexp(1.0, d));
            }
            scales[r * (K / 16) + 2 * b] = out_byte;
            scales[r * (K / 16) + 2 * b + 1] = out_byte;
        }
    memcpy(packed, mx_packed, (size_t)(R * (K / 2)));
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* MoE routed experts                                                       */
/* ------------------------------------------------------------------------ */

/*
 * Token-by-expert permutation for top-k routing ([FlashNext]: 512 routed
 * experts, top-10).  The T*k (token, slot) pairs, numbered p = t*k + j, are
 * listed expert by expert, and inside one expert in increasing p (a stable
 * sort by expert id):
 *   perm[q]     = p of the q-th listed pair
 *   offsets[e]  = first q of expert e, offsets[E] = T*k
 *   inv[p]      = q
 * Ids outside [0, E) give ORC_RANGE.
 */
int orc_moe_route(const int32_t* ids, int64_t T, int32_t k, int32_t E,
                  int32_t* perm, int32_t* offsets, int32_t* inv)
{
    int64_t p, q = 0, n = T * (int64_t)k;
    int32_t e;
    for (p = 0; p < n; p++)
        if (ids[p] < 0 || ids[p] >= E)
            return ORC_RANGE;
    for (e = 0; e < E; e++) {
        offsets[e] = (int32_t)q;
        for (p = 0; p < n; p++)
            if (ids[p] == e) {
                perm[q] = (int32_t)p;
                inv[p] = (int32_t)q;
                q++;
            }
    }
    offsets[E] = (int32_t)q;
    return ORC_OK;
}

static double silu(double z)
{
    return z / (1.0 + exp(-z));
}

/*
 * gate_up projection + SwiGLU for listed pairs.  For each requested list
 * position q (rows[i]), with token t = perm[q] / k and expert e (the e with
 * offsets[e] <= q < offsets[e+1]):
 *   g = exact W4A4 row product of xq[t] with W13[e] rows [0, I)    (gate)
 *   u = same with W13[e] rows [I, 2I)                              (up)
 *   h = silu(g) * u  in double, rounded to nearest-even bf16
 * xq: NVFP4 [T, H] with global Gx.  W13: E stacked NVFP4 [2I, H] matrices
 * (packed [E, 2I, H/2], scales [E, 2I, H/16]) with globals G13[E].
 * h_out: [n_rows, I] bf16 bits.
 */
int orc_moe_gate_up(const uint8_t* xp, const uint8_t* xs, float Gx,
                    const int32_t* perm, const int32_t* offsets, int32_t k,
                    int32_t E, const uint8_t* w13p, const uint8_t* w13s,
                    const float* G13, int64_t H, int64_t I,
                    const int64_t* rows, int64_t n_rows, uint16_t* h_out)
{
    int64_t i, n, *w_rows, a_row;
    double* gu;
    int rc = ORC_OK;
    if (H % 16 != 0)
        return ORC_SHAPE;
    w_rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(2 * I));
    gu = (double*)malloc(sizeof(double) * (size_t)(2 * I));
    if (!w_rows || !gu) {
        free(w_rows);
        free(gu);
        return ORC_INVALID;
    }
    for (n = 0; n < 2 * I; n++)
        w_rows[n] = n;
    for (i = 0; i < n_rows && rc == ORC_OK; i++) {
        int64_t q = rows[i];
        int32_t e = 0;
        while (e < E && !(offsets[e] <= q && q < offsets[e + 1]))
            e++;
        if (e == E) {
            rc = ORC_RANGE;
            break;
        }
        a_row = perm[q] / k;
        rc = orc_gemm_rows(xp, xs, Gx, &a_row, 1,
                           w13p + (size_t)e * (size_t)(2 * I) * (size_t)(H / 2),
                           w13s + (size_t)e * (size_t)(2 * I) * (size_t)(H / 16),
                           G13[e], w_rows, 2 * I, H, gu);
        for (n = 0; n < I; n++)
            h_out[i * I + n] = orc_bf16_from_double(silu(gu[n]) * gu[I + n]);
    }
    free(w_rows);
    free(gu);
    return rc;
}

/*
 * down projection for listed pairs: y[i] = exact W4A4 row product of hq row
 * rows[i] (hq is in list order, NVFP4 [T*k, I], global Gh) with W2[e]
 * ([H, I] per expert, globals G2[E]).  y_out: [n_rows, H] double.
 */
int orc_moe_down(const uint8_t* hp, const uint8_t* hs, float Gh,
                 const int32_t* offsets, int32_t E, const uint8_t* w2p,
                 const uint8_t* w2s, const float* G2, int64_t H, int64_t I,
                 const int64_t* rows, int64_t n_rows, double* y_out)
{
    int64_t i, n, *w_rows;
    int rc = ORC_OK;
    if (I % 16 != 0)
        return ORC_SHAPE;
    w_rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)H);
    if (!w_rows)
        return ORC_INVALID;
    for (n = 0; n < H; n++)
        w_rows[n] = n;
    for (i = 0; i < n_rows && rc == ORC_OK; i++) {
        int64_t q = rows[i];
        int32_t e = 0;
        while (e < E && !(offsets[e] <= q && q < offsets[e + 1]))
            e++;
        if (e == E) {
            rc = ORC_RANGE;
            break;
        }
        rc = orc_gemm_rows(hp, hs, Gh, &q, 1,
                           w2p + (size_t)e * (size_t)H * (size_t)(I / 2),
                           w2s + (size_t)e * (size_t)H * (size_t)(I / 16),
                           G2[e], w_rows, H, I, y_out + i * H);
    }
    free(w_rows);
    return rc;
}

/*
 * Router-weighted combine: out[t, n] = sum over slots j = 0..k-1 (in that
 * order) of w[t, j] * y[inv[t*k + j], n], in double, rounded to bf16.
 * y: [T*k, H] double in list order.
 */
int orc_moe_combine(const double* y, const int32_t* inv, const float* w,
                    int64_t T, int32_t k, int64_t H, uint16_t* out)
{
    int64_t t, n;
    int32_t j;
    for (t = 0; t < T; t++)
        for (n = 0; n < H; n++) {
            double acc = 0.0;
            for (j = 0; j < k; j++)
                acc += (double)w[t * k + j] * y[(int64_t)inv[t * k + j] * H + n];
            out[t * H + n] = orc_bf16_from_double(acc);
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* W4A16: bf16 activations x NVFP4 weights                                   */
/* ------------------------------------------------------------------------ */

/* Dequantized weight element without its global, as a double (exact). */
static double deq0_value(const uint8_t* packed, const uint8_t* scales, int64_t row, int64_t K, int64_t k)
{
    uint8_t byte = packed[row * (K / 2) + k / 2];
    uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
    return orc_e2m1_value(nib) * orc_e4m3_value(scales[row * (K / 16) + k / 16]);
}

/*
 * W4A16 product ("Qwen3.8-Flash-Next-FP4-Local", section 3.2: NVFP4 weights,
 * BF16 activations):
 *   C[i, j] = Gw * sum_k A[a_rows[i], k] * deq0(W[w_rows[j], k])
 * A: bf16 bits, row stride lda.  Every product is exact in double (8 + 6
 * significant bits); the sum is a compensated (Neumaier) double sum, within
 * a few ulps of the exact sum, then multiplied by Gw.  C is [n_a, n_w].
 */
int orc_gemm_w4a16_rows(const uint16_t* A, int64_t lda, const int64_t* a_rows, int64_t n_a,
                        const uint8_t* Wp, const uint8_t* Ws, float Gw,
                        const int64_t* w_rows, int64_t n_w, int64_t K, double* C)
{
    int64_t i, j, k;
    double* wv;
    if (K % 16 != 0 || lda < K)
        return ORC_SHAPE;
    wv = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)(n_w > 0 ? n_w : 1));
    if (!wv)
        return ORC_INVALID;
    for (j = 0; j < n_w; j++)
        for (k = 0; k < K; k++)
            wv[j * K + k] = deq0_value(Wp, Ws, w_rows[j], K, k);
    for (i = 0; i < n_a; i++) {
        const uint16_t* a = A + a_rows[i] * lda;
        for (j = 0; j < n_w; j++) {
            double sum = 0.0, comp = 0.0;
            for (k = 0; k < K; k++) {
                double p = (double)bf16_to_float(a[k]) * wv[j * K + k];
                double t = sum + p;
                if (fabs(sum) >= fabs(p))
                    comp += (sum - t) + p;
                else
                    comp += (p - t) + sum;
                sum = t;
            }
            C[i * n_w + j] = (sum + comp) * (double)Gw;
        }
    }
    free(wv);
    return ORC_OK;
}

/*
 * W4A16 gate_up + SwiGLU for listed pairs: as orc_moe_gate_up with the
 * token's bf16 row x[perm[q] / k] in place of its NVFP4 row.  x: [T, H]
 * bf16 bits.  h_out: [n_rows, I] bf16 bits.
 */
int orc_moe_w4a16_gate_up(const uint16_t* x, const int32_t* perm, const int32_t* offsets, int32_t k,
                          int32_t E, const uint8_t* w13p, const uint8_t* w13s, const float* G13,
                          int64_t H, int64_t I, const int64_t* rows, int64_t n_rows, uint16_t* h_out)
{
    int64_t i, n, *w_rows, a_row;
    double* gu;
    int rc = ORC_OK;
    if (H % 16 != 0)
        return ORC_SHAPE;
    w_rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(2 * I));
    gu = (double*)malloc(sizeof(double) * (size_t)(2 * I));
    if (!w_rows || !gu) {
        free(w_rows);
        free(gu);
        return ORC_INVALID;
    }
    for (n = 0; n < 2 * I; n++)
        w_rows[n] = n;
    for (i = 0; i < n_rows && rc == ORC_OK; i++) {
        int64_t q = rows[i];
        int32_t e = 0;
        while (e < E && !(offsets[e] <= q && q < offsets[e + 1]))
            e++;
        if (e == E) {
            rc = ORC_RANGE;
            break;
        }
        a_row = perm[q] / k;
        rc = orc_gemm_w4a16_rows(x, H, &a_row, 1, w13p + (size_t)e * (size_t)(2 * I) * (size_t)(H / 2),
                                 w13s + (size_t)e * (size_t)(2 * I) * (size_t)(H / 16), G13[e], w_rows, 2 * I,
                                 H, gu);
        for (n = 0; n < I; n++)
            h_out[i * I + n] = orc_bf16_from_double(silu(gu[n]) * gu[I + n]);
    }
    free(w_rows);
    free(gu);
    return rc;
}

/*
 * W4A16 down projection for listed pairs: y[i] = W4A16 row product of the
 * bf16 h row rows[i] (h in list order, [T*k, I]) with W2[e].  y_out:
 * [n_rows, H] double.
 */
int orc_moe_w4a16_down(const uint16_t* h, const int32_t* offsets, int32_t E, const uint8_t* w2p,
                       const uint8_t* w2s, const float* G2, int64_t H, int64_t I, const int64_t* rows,
                       int64_t n_rows, double* y_out)
{
    int64_t i, n, *w_rows;
    int rc = ORC_OK;
    if (I % 16 != 0)
        return ORC_SHAPE;
    w_rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)H);
    if (!w_rows)
        return ORC_INVALID;
    for (n = 0; n < H; n++)
        w_rows[n] = n;
    for (i = 0; i < n_rows && rc == ORC_OK; i++) {
        int64_t q = rows[i];
        int32_t e = 0;
        while (e < E && !(offsets[e] <= q && q < offsets[e + 1]))
            e++;
        if (e == E) {
            rc = ORC_RANGE;
            break;
        }
        rc = orc_gemm_w4a16_rows(h, I, &q, 1, w2p + (size_t)e * (size_t)H * (size_t)(I / 2),
                                 w2s + (size_t)e * (size_t)H * (size_t)(I / 16), G2[e], w_rows, H, I,
                                 y_out + i * H);
    }
    free(w_rows);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* MX-native W4A8: MXFP8 activations x MXFP4 weights                         */
/* ------------------------------------------------------------------------ */

/*
 * MXFP8 encode of a bf16 matrix ([DSV41] §二: the reference FP8 x FP4 GEMM
 * quantizes activations in blocks with power-of-two scales; the reading
 * taken: blocks of 32 along the row, UE8M0 scale 2^e with e the smallest
 * integer such that amax <= 448 * 2^e (no element saturates), clamped to
 * [-127, 127], e = 0 for an all-zero block).  Element: the nearest E4M3
 * magnitude to |x| * 2^-e (brute-force search, ties to the even code),
 * sign bit = signbit(x).  out: [R, K] E4M3 bytes; e8m0: [R, K/32] (e + 127).
 */
int orc_mxfp8_encode(const uint16_t* x, int64_t R, int64_t K, int64_t ld, uint8_t* out, uint8_t* e8m0)
{
    int64_t r, b, j;
    if (K % 32 != 0 || ld < K)
        return ORC_SHAPE;
    for (r = 0; r < R; r++)
        for (b = 0; b < K / 32; b++) {
            const uint16_t* xb = x + r * ld + 32 * b;
            double amax = 0.0;
            int e = 0;
            for (j = 0; j < 32; j++) {
                double a = fabs((double)bf16_to_float(xb[j]));
                if (a > amax)
                    amax = a;
            }
            if (amax > 0.0) {
                e = -127;
                while (e < 127 && amax > 448.0 * ldexp(1.0, e))
                    e++;
            }
            e8m0[r * (K / 32) + b] = (uint8_t)(e + 127);
            for (j = 0; j < 32; j++) {
                float v = bf16_to_float(xb[j]);
                float y = (float)ldexp(fabs((double)v), -e);
                uint8_t c = orc_e4m3_encode(y);
                out[r * K + 32 * b + j] = (uint8_t)(c | (signbit(v) ? 0x80 : 0));
            }
        }
    return ORC_OK;
}

/* Value of an E8M0 byte (2^(b - 127)); byte 255 (NaN) is an error for the
 * caller to avoid. */
static double e8m0_pow(uint8_t b)
{
    return ldexp(1.0, (int)b - 127);
}

/*
 * MX-native W4A8 product ([DSV41] §二: FP8 activations, MXFP4 weights, block
 * scales applied inside the accumulation):
 *   C[i, j] = sum over 32-blocks b of 2^(ea - 127) 2^(ew - 127)
 *             * sum_{k in b} e4m3(A[a_rows[i], k]) * e2m1(W[w_rows[j], k])
 * Each block sum is an exact int64 sum of the integer images
 * (2^9 * e4m3) * (2 * e2m1), scaled exactly by 2^(ea + ew - 264); the block
 * terms are added in double with compensated summation.  A: [.., K] E4M3
 * with Ae [.., K/32]; W: packed [.., K/2] with We [.., K/32].  C: [n_a, n_w].
 */
int orc_mx_gemm_w4a8_rows(const uint8_t* A, const uint8_t* Ae, const int64_t* a_rows, int64_t n_a,
                          const uint8_t* Wp, const uint8_t* We, const int64_t* w_rows, int64_t n_w, int64_t K,
                          double* C)
{
    int64_t i, j, b, k;
    if (K % 32 != 0)
        return ORC_SHAPE;
    for (i = 0; i < n_a; i++)
        for (j = 0; j < n_w; j++) {
            const uint8_t* a = A + a_rows[i] * K;
            const uint8_t* w = Wp + w_rows[j] * (K / 2);
            double sum = 0.0, comp = 0.0;
            for (b = 0; b < K / 32; b++) {
                uint8_t ea = Ae[a_rows[i] * (K / 32) + b], ew = We[w_rows[j] * (K / 32) + b];
                int64_t acc = 0;
                double t, p;
                if (ea == 255 || ew == 255)
                    return ORC_RANGE;
                for (k = 32 * b; k < 32 * b + 32; k++) {
                    uint8_t byte = w[k / 2];
                    uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 15);
                    int64_t ai = (int64_t)ldexp(orc_e4m3_value(a[k]), 9);
                    int64_t wi = (int64_t)(2.0 * orc_e2m1_value(nib));
                    acc += ai * wi;
                }
                p = ldexp((double)acc, -10) * e8m0_pow(ea) * e8m0_pow(ew);
                t = sum + p;
                if (fabs(sum) >= fabs(p))
                    comp += (sum - t) + p;
                else
                    comp += (p - t) + sum;
                sum = t;
            }
            C[i * n_w + j] = sum + comp;
        }
    return ORC_OK;
}

/*
 * MX-native W4A8 routed-expert projections (page "DeepSeek-V4.1-Flash-NVFP4",
 * section 二: MXFP4 expert weights with FP8 activations), for listed pairs,
 * in the same steps as orc_moe_gate_up / orc_moe_down with the MX row
 * product of orc_mx_gemm_w4a8_rows in place of the NVFP4 one:
 *   gate_up: for list position q (rows[i]), token t = perm[q] / k, expert e
 *     (offsets[e] <= q < offsets[e+1]): g, u = the MX products of x row t
 *     with W13[e] rows [0, I) and [I, 2I); h = bf16(silu(g) * u) (double
 *     SwiGLU, nearest-even).  x: E4M3 [T, H] + UE8M0 [T, H/32]; W13: codes
 *     [E, 2I, H/2] + UE8M0 [E, 2I, H/32].  h_out: [n_rows, I] bf16 bits.
 *   down: y[i] = the MX products of hq row rows[i] (list order, E4M3
 *     [T*k, I] + UE8M0 [T*k, I/32]) with W2[e] ([E, H, I/2] + [E, H, I/32]).
 *     y_out: [n_rows, H] double.
 */
static int orc_expert_of(const int32_t* offsets, int32_t E, int64_t q)
{
    int32_t e = 0;
    while (e < E && !(offsets[e] <= q && q < offsets[e + 1]))
        e++;
    return e;
}

int orc_mx_moe_gate_up(const uint8_t* xq, const uint8_t* xe, const int32_t* perm, const int32_t* offsets,
                       int32_t k, int32_t E, const uint8_t* w13p, const uint8_t* w13e, int64_t H, int64_t I,
                       const int64_t* rows, int64_t n_rows, uint16_t* h_out)
{
    int64_t i, n, *w_rows;
    double* gu;
    int rc = ORC_OK;
    if (H % 32 != 0)
        return ORC_SHAPE;
    w_rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(2 * I));
    gu = (double*)malloc(sizeof(double) * (size_t)(2 * I));
    if (!w_rows || !gu) {
        free(w_rows);
        free(gu);
        return ORC_INVALID;
    }
    for (n = 0; n < 2 * I; n++)
        w_rows[n] = n;
    for (i = 0; i < n_rows && rc == ORC_OK; i++) {
        const int64_t q = rows[i];
        const int32_t e = orc_expert_of(offsets, E, q);
        int64_t a_row;
        if (e == E) {
            rc = ORC_RANGE;
            break;
        }
        a_row = perm[q] / k;
        rc = orc_mx_gemm_w4a8_rows(xq, xe, &a_row, 1, w13p + (size_t)e * (size_t)(2 * I) * (size_t)(H / 2),
                                   w13e + (size_t)e * (size_t)(2 * I) * (size_t)(H / 32), w_rows, 2 * I, H, gu);
        for (n = 0; n < I; n++)
            h_out[i * I + n] = orc_bf16_from_double(silu(gu[n]) * gu[I + n]);
    }
    free(w_rows);
    free(gu);
    return rc;
}

int orc_mx_moe_down(const uint8_t* hq, const uint8_t* he, const int32_t* offsets, int32_t E, const uint8_t* w2p,
                    const uint8_t* w2e, int64_t H, int64_t I, const int64_t* rows, int64_t n_rows, double* y_out)
{
    int64_t i, n, *w_rows;
    int rc = ORC_OK;
    if (I % 32 != 0)
        return ORC_SHAPE;
    w_rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)H);
    if (!w_rows)
        return ORC_INVALID;
    for (n = 0; n < H; n++)
        w_rows[n] = n;
    for (i = 0; i < n_rows && rc == ORC_OK; i++) {
        const int64_t q = rows[i];
        const int32_t e = orc_expert_of(offsets, E, q);
        if (e == E) {
            rc = ORC_RANGE;
            break;
        }
        rc = orc_mx_gemm_w4a8_rows(hq, he, &q, 1, w2p + (size_t)e * (size_t)H * (size_t)(I / 2),
                                   w2e + (size_t)e * (size_t)H * (size_t)(I / 32), w_rows, H, I, y_out + i * H);
    }
    free(w_rows);
    return rc;
}
