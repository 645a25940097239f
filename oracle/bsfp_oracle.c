/*
 * bsfp_oracle.c -- plain, slow, obviously correct CPU oracle for the
 * block-scaled 4-bit quantized matmul path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP library; both sides receive the same seeded inputs and nothing else.
 *
 * Build: C99, -O2 -ffp-contract=off, no -ffast-math (every fp32 operation is a
 * single correctly rounded IEEE operation, no FMA contraction, no excess
 * precision).  fp32 is used where the method takes a rounding decision (the
 * converter the pages name, cvt.rn.satfinite.e2m1x2.f32, takes fp32 inputs:
 * "perf(cuda): enable hardware NVFP4/MXFP4 conversion on Blackwell builds",
 * Problem / Background); fp64 is used for the matmul reference.
 *
 * Codecs are built by enumeration from the format definitions (OCP
 * Microscaling Formats (MX) v1.0: FP4 E2M1, FP8 E4M3, E8M0 scale), and
 * encoding is a nearest-value search over the enumerated grid, not bit tricks.
 *
 * Readings taken where the pages are silent (each marked [R] below):
 *   R1  E2M1 rounding is nearest, ties to the even code; |v| >= 6 saturates.
 *   R2  a negative value that rounds to zero keeps its sign (code 8).
 *   R3  E4M3 block scale: nearest finite, ties to even code, > 448 -> 448.
 *   R4  NVFP4: g = amax/(448*6); sf = bamax/(6*g); S = E4M3(sf);
 *       d = E4M3(S)*g; codes = E2M1(x * (1/d)).  d == 0 -> S = 0, codes 0.
 *   R5  MXFP4: shared exponent e = floor(log2 bamax) - 2 (OCP MX rule),
 *       clamped to [-127,127]; bamax == 0 -> e = -127, codes 0.
 *   R6  affine: sb = bf16((max-min)/15), bb = bf16(min), q = clamp(rint((x -
 *       bb) * (1/sb)), 0, 15); sb == 0 -> q = 0.
 *   R7  packing: low nibble first, 8 codes per little-endian uint32.
 *   R8  dequant: NVFP4 bf16((E2M1*E4M3)*g); MXFP4 bf16(E2M1*2^e); affine
 *       bf16(fma(sb, q, bb)).
 *   R17 MXFP8 (OCP MX v1.0, E4M3 elements): shared exponent e =
 *       floor(log2 bamax) - 8 (448 = 1.75 * 2^8), clamped to [-127, 127];
 *       bamax == 0 -> e = -127; elements E4M3(x * 2^-e) nearest even,
 *       saturating at 448, sign bit kept; 4 codes per uint32, byte k mod 4.
 *   R18 affine b-bit, group G in {32, 64, 128}: R6 with 2^b - 1 in place of
 *       15; b = 8 packs 4 codes per uint32, byte k mod 4.
 *   R15  stochastic rounding (the USE_SR variant of the 4-bit quantizer; the
 *       pages give no rounding rule or random-bit contract): scales as in
 *       R4/R5; an element |v| strictly between grid magnitudes lo < hi
 *       becomes hi when u < p, else lo, with p = (|v| - lo) / (hi - lo) and
 *       u = (r >> 8) * 2^-24 for the element's caller-supplied 32-bit r;
 *       both are exact in fp32.  Grid values stay, |v| >= 6 saturates, the
 *       sign bit follows v.  E[E2M1(v)] = v up to 2^-24 of the spacing.
 *
 * Parity status: the codecs, packing, the exact-reproduction cases, the
 * invariants and the matmul are pinned by the not-gpu test suite (closed
 * forms, library decoders, hand-worked fixtures, brute force).  The choice of
 * formula itself in R4, R5 and R6 is parity unpinned beyond those
 * properties: the pages print no quantizer arithmetic and no worked values.
 */
#include "bsfp_oracle.h"

#include <math.h>
#include <string.h>

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ======================================================================== */
/* bf16                                                                      */
/* ======================================================================== */

float bo_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Nearest bf16 to f; on a tie, the candidate with the even significand.  The
 * two candidates are the truncation of f toward zero and the next bf16 away
 * from zero; distances are compared exactly in fp64. */
uint16_t bo_bf16_from_f32(float f)
{
    uint32_t u = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x40);
    uint16_t lo = (uint16_t)(u >> 16);
    if ((u & 0xFFFFu) == 0) return lo;
    uint16_t hi = (uint16_t)(lo + 1); /* next magnitude, same sign */
    double dl = fabs((double)f - (double)bo_bf16_to_f32(lo));
    double dh = fabs((double)f - (double)bo_bf16_to_f32(hi));
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1) ? hi : lo;
}

/* Nearest bf16 to a double (single rounding), ties to even significand. */
uint16_t bo_bf16_from_f64(double d)
{
    if (isnan(d)) return 0x7FC0;
    if (d == 0.0) return signbit(d) ? 0x8000 : 0x0000;
    /* (float)d is within one bf16 step of the answer; search its neighbours. */
    float t = (float)d;
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    uint16_t mag0 = (uint16_t)((bits_from_f32(t) >> 16) & 0x7FFF);
    int best = -1;
    double bd = INFINITY;
    for (int dm = -1; dm <= 1; ++dm) {
        int mag = (int)mag0 + dm;
        if (mag < 0 || mag > 0x7F80) continue; /* 0x7F80 = inf */
        double v = (double)bo_bf16_to_f32((uint16_t)(sign | mag));
        double dist = fabs(d - v);
        if (best < 0 || dist < bd || (dist == bd && (mag & 1) == 0)) {
            best = mag;
            bd = dist;
        }
    }
    return (uint16_t)(sign | best);
}

void bo_bf16_from_f32_array(const float* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bo_bf16_from_f32(v[i]);
}
void bo_bf16_from_f64_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bo_bf16_from_f64(v[i]);
}
void bo_bf16_to_f64_array(const uint16_t* x, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (double)bo_bf16_to_f32(x[i]);
}

/* ======================================================================== */
/* E2M1 (FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit.                 */
/* ======================================================================== */

/* Definition: e == 0 -> subnormal m * 2^-1; else 2^(e-1) * (1 + m/2). */
double bo_e2m1_decode(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m * 0.5, e - 1);
    return s ? -mag : mag;
}

/* [R1][R2] Nearest of the 8 magnitudes, ties to the even code, saturating at
 * the largest magnitude (6, the pages' F4E2M1_MAX in "mlx 0.30.7.3 ->
 * 0.30.7.6", qqmm_utils.cu hunk); the sign bit follows the sign of v. */
int bo_e2m1_encode(float v)
{
    double a = fabs((double)v);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(a - bo_e2m1_decode(c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    /* satfinite: every magnitude at or beyond the largest grid value is code
     * 7 (for very large |v| the fp64 distances to 4 and 6 would tie). */
    if (a >= 6.0) best = 7;
    return best | (signbit(v) ? 8 : 0);
}

/* [R15] Stochastic rounding to E2M1 with the random word r. */
int bo_e2m1_encode_sr(float v, uint32_t r)
{
    const int sign = signbit(v) ? 8 : 0;
    const float a = fabsf(v);
    if (!(a < 6.0f)) return 7 | sign; /* saturate (NaN too) */
    int lo = 0; /* largest grid magnitude <= a */
    for (int c = 1; c < 8; ++c)
        if (bo_e2m1_decode(c) <= (double)a) lo = c;
    const float flo = (float)bo_e2m1_decode(lo);
    if (flo == a) return lo | sign;
    const float fhi = (float)bo_e2m1_decode(lo + 1);
    const float p = (a - flo) / (fhi - flo); /* exact: Sterbenz, power-of-two divisor */
    const float u = (float)(r >> 8) * 0x1p-24f;
    return (u < p ? lo + 1 : lo) | sign;
}

void bo_e2m1_encode_array(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)bo_e2m1_encode(v[i]);
}

/* ======================================================================== */
/* E4M3 (OCP E4M3FN): bias 7, no infinities, S.1111.111 is NaN, max 448.    */
/* ======================================================================== */

double bo_e4m3_decode(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = m * ldexp(1.0, -9);          /* subnormal: m/8 * 2^-6 */
    else        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* [R3] s >= 0: nearest of the 127 finite non-negative codes, ties to the even
 * code; anything above 448 (the pages' F8E4M3_MAX) saturates to 448. */
int bo_e4m3_encode(float s)
{
    double a = (double)s;
    if (!(a <= 448.0)) return 0x7E;
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(a - bo_e4m3_decode(c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return best;
}

void bo_e4m3_encode_array(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)bo_e4m3_encode(v[i]);
}

/* ======================================================================== */
/* E8M0: code c -> 2^(c-127); 0xFF is NaN and never produced.                */
/* ======================================================================== */

double bo_e8m0_decode(int code)
{
    if ((code & 0xFF) == 0xFF) return NAN;
    return ldexp(1.0, (code & 0xFF) - 127);
}

/* ======================================================================== */
/* amax, global scale, alpha                                                  */
/* ======================================================================== */

/* max |x| over the tensor; exact and independent of order. */
float bo_amax(const uint16_t* x, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(bo_bf16_to_f32(x[i]));
        if (a > m) m = a;
    }
    return m;
}

/* The NVFP4 per-tensor global scale g = amax / (448 * 6): the MLX form of the
 * scale is m * 2688 = amax ("mlx: opt-in dense GEMM for nvfp4 prefill",
 * global-scale representation discussion), so the checkpoint multiplier is
 * m = amax / 2688, with 448 and 6 the E4M3 and E2M1 maxima ("mlx 0.30.7.3 ->
 * 0.30.7.6", qqmm_utils.cu, compute_qqmm_pointers). */
float bo_nvfp4_global_scale(float amax)
{
    const float max_product = 448.0f * 6.0f; /* exact: 2688 */
    return amax / max_product;
}

/* alpha = g_x * g_w in fp32.  The pages compute alpha as amax_x * amax_w /
 * (448*6)^2 ("mlx 0.30.7.3 -> 0.30.7.6", qqmm_utils.cu, compute_qqmm_pointers
 * and create_nvfp4_scalars); with g = amax/2688 that is g_x * g_w, equal up to
 * fp32 rounding. */
float bo_alpha(float g_x, float g_w) { return g_x * g_w; }

/* ======================================================================== */
/* packing [R7]                                                               */
/* ======================================================================== */

static void put_code(uint32_t* row_words, int64_t k, int code)
{
    row_words[k / 8] |= (uint32_t)(code & 0xF) << (4 * (k % 8));
}
static int get_code(const uint32_t* row_words, int64_t k)
{
    return (int)((row_words[k / 8] >> (4 * (k % 8))) & 0xF);
}

/* ======================================================================== */
/* NVFP4 quantize [R4]                                                        */
/* ======================================================================== */

/* One 16-element group of one row: block amax, E4M3 block scale relative to
 * the global scale, then each element multiplied by the reciprocal of the
 * decoded block scale and converted to E2M1 ("perf(cuda): enable hardware
 * NVFP4/MXFP4 conversion on Blackwell builds", Current Behavior: the
 * scale-then-convert helpers; "mlx 0.30.7.3 -> 0.30.7.6", quantized.h,
 * fp_quantize with a global scale). */
static void quantize_nvfp4(const uint16_t* x, int64_t rows, int64_t cols,
                           int use_global, const float* g_given,
                           uint32_t* codes, uint8_t* scales,
                           float* g_out, float* amax_out, const uint32_t* rbits)
{
    const int G = 16;
    float g = 1.0f;
    if (use_global) {
        if (g_given) {
            g = *g_given;
        } else {
            float amax = bo_amax(x, rows * cols);
            if (amax_out) *amax_out = amax;
            g = bo_nvfp4_global_scale(amax);
        }
    }
    if (g_out) *g_out = g;
    const int64_t words = cols / 8, groups = cols / G;
    memset(codes, 0, (size_t)(rows * words) * sizeof(uint32_t));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        uint32_t* cr = codes + r * words;
        for (int64_t b = 0; b < groups; ++b) {
            float bamax = 0.0f;
            for (int i = 0; i < G; ++i) {
                float a = fabsf(bo_bf16_to_f32(xr[b * G + i]));
                if (a > bamax) bamax = a;
            }
            int S = 0;
            float d = 0.0f;
            if (g != 0.0f) {
                float six_g = 6.0f * g;
                float sf = bamax / six_g;
                S = bo_e4m3_encode(sf);
                d = (float)bo_e4m3_decode(S) * g;
            }
            if (d == 0.0f) {
                scales[r * groups + b] = 0; /* zero rule: scale 0, codes 0 */
                continue;
            }
            scales[r * groups + b] = (uint8_t)S;
            float inv = 1.0f / d;
            for (int i = 0; i < G; ++i) {
                float v = bo_bf16_to_f32(xr[b * G + i]) * inv;
                int c = rbits ? bo_e2m1_encode_sr(v, rbits[r * cols + b * G + i])
                              : bo_e2m1_encode(v);
                put_code(cr, b * G + i, c);
            }
        }
    }
}

void bo_quantize_nvfp4(const uint16_t* x, int64_t rows, int64_t cols,
                       int use_global, const float* g_given,
                       uint32_t* codes, uint8_t* scales,
                       float* g_out, float* amax_out)
{
    quantize_nvfp4(x, rows, cols, use_global, g_given, codes, scales, g_out, amax_out, NULL);
}

/* [R15] NVFP4 with stochastically rounded codes; rbits [rows, cols]. */
void bo_quantize_nvfp4_sr(const uint16_t* x, int64_t rows, int64_t cols,
                          int use_global, const float* g_given, const uint32_t* rbits,
                          uint32_t* codes, uint8_t* scales,
                          float* g_out, float* amax_out)
{
    quantize_nvfp4(x, rows, cols, use_global, g_given, codes, scales, g_out, amax_out, rbits);
}

/* ======================================================================== */
/* MXFP4 quantize [R5]                                                        */
/* ======================================================================== */

/* floor(log2(a)) for finite a > 0, exactly (frexp: a = f * 2^ex, f in
 * [0.5, 1)). */
static int floor_log2(double a)
{
    int ex;
    (void)frexp(a, &ex);
    return ex - 1;
}

/* One 32-element group: power-of-two (E8M0) shared scale from the group
 * amax, elements scaled exactly by 2^-e and converted to E2M1 (the MX arm of
 * the same bits == 4 quantizer, "perf(cuda): enable hardware NVFP4/MXFP4
 * conversion on Blackwell builds", Current Behavior, use_mx_scale). */
static void quantize_mxfp4(const uint16_t* x, int64_t rows, int64_t cols,
                           uint32_t* codes, uint8_t* scales, const uint32_t* rbits)
{
    const int G = 32;
    const int emax_e2m1 = 2; /* largest E2M1 magnitude 6 = 1.5 * 2^2 */
    const int64_t words = cols / 8, groups = cols / G;
    memset(codes, 0, (size_t)(rows * words) * sizeof(uint32_t));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        uint32_t* cr = codes + r * words;
        for (int64_t b = 0; b < groups; ++b) {
            float bamax = 0.0f;
            for (int i = 0; i < G; ++i) {
                float a = fabsf(bo_bf16_to_f32(xr[b * G + i]));
                if (a > bamax) bamax = a;
            }
            int e = (bamax == 0.0f) ? -127 : floor_log2((double)bamax) - emax_e2m1;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
            scales[r * groups + b] = (uint8_t)(e + 127);
            for (int i = 0; i < G; ++i) {
                float v = ldexpf(bo_bf16_to_f32(xr[b * G + i]), -e);
                int c = rbits ? bo_e2m1_encode_sr(v, rbits[r * cols + b * G + i])
                              : bo_e2m1_encode(v);
                put_code(cr, b * G + i, c);
            }
        }
    }
}

void bo_quantize_mxfp4(const uint16_t* x, int64_t rows, int64_t cols,
                       uint32_t* codes, uint8_t* scales)
{
    quantize_mxfp4(x, rows, cols, codes, scales, NULL);
}

/* [R15] MXFP4 with stochastically rounded codes; rbits [rows, cols]. */
void bo_quantize_mxfp4_sr(const uint16_t* x, int64_t rows, int64_t cols,
                          const uint32_t* rbits, uint32_t* codes, uint8_t* scales)
{
    quantize_mxfp4(x, rows, cols, codes, scales, rbits);
}

/* ======================================================================== */
/* affine 4-bit quantize [R6]                                                 */
/* ======================================================================== */

/* One 64-element group: asymmetric min/max, codes computed from the stored
 * (bf16) scale and bias so that dequantization reproduces what was encoded
 * (affine 4-bit group 64 with a scale and a bias per group: "epic: NVIDIA
 * Volta (sm_70) inference acceleration program", Baseline; "mlx 0.30.7.3 ->
 * 0.30.7.6", quantized.cpp, affine_quantize(w, wq, scales, biases, ...)). */
void bo_quantize_affine(const uint16_t* x, int64_t rows, int64_t cols,
                        uint32_t* codes, uint16_t* scales, uint16_t* biases)
{
    const int G = 64;
    const int64_t words = cols / 8, groups = cols / G;
    memset(codes, 0, (size_t)(rows * words) * sizeof(uint32_t));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        uint32_t* cr = codes + r * words;
        for (int64_t b = 0; b < groups; ++b) {
            float mn = bo_bf16_to_f32(xr[b * G]), mx = mn;
            for (int i = 1; i < G; ++i) {
                float v = bo_bf16_to_f32(xr[b * G + i]);
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            float range = mx - mn;
            float step = range / 15.0f;
            uint16_t sb = bo_bf16_from_f32(step);
            uint16_t bb = bo_bf16_from_f32(mn);
            scales[r * groups + b] = sb;
            biases[r * groups + b] = bb;
            float s = bo_bf16_to_f32(sb), bias = bo_bf16_to_f32(bb);
            float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
            for (int i = 0; i < G; ++i) {
                float t = (bo_bf16_to_f32(xr[b * G + i]) - bias) * inv;
                float q = nearbyintf(t); /* round to nearest, ties to even */
                if (q < 0.0f) q = 0.0f;
                if (q > 15.0f) q = 15.0f;
                put_code(cr, b * G + i, (int)q);
            }
        }
    }
}

/* ======================================================================== */
/* format variants [R17][R18]: generic b-bit packing                          */
/* ======================================================================== */

static void put_code_b(uint32_t* row_words, int64_t k, int code, int bits)
{
    const int64_t per = 32 / bits;
    row_words[k / per] |= (uint32_t)code << (bits * (k % per));
}

static int get_code_b(const uint32_t* row_words, int64_t k, int bits)
{
    const int64_t per = 32 / bits;
    return (int)((row_words[k / per] >> (bits * (k % per))) & ((1u << bits) - 1u));
}

/* Signed E4M3: sign bit 0x80, magnitude nearest even, > 448 -> 448. */
static int e4m3_encode_signed(float v)
{
    return bo_e4m3_encode(fabsf(v)) | (signbit(v) ? 0x80 : 0);
}

static double e4m3_decode_signed(int c)
{
    double m = bo_e4m3_decode(c & 0x7F);
    return (c & 0x80) ? -m : m;
}

/* [R18] affine b-bit quantize with group G: min/max per group, step
 * bf16((max - min) / (2^b - 1)), bias bf16(min), codes from the stored
 * scale and bias. */
void bo_quantize_affine_g(const uint16_t* x, int64_t rows, int64_t cols, int bits, int G,
                          uint32_t* codes, uint16_t* scales, uint16_t* biases)
{
    const float qmax = (float)((1 << bits) - 1);
    const int64_t words = cols * bits / 32, groups = cols / G;
    memset(codes, 0, (size_t)(rows * words) * sizeof(uint32_t));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        uint32_t* cr = codes + r * words;
        for (int64_t b = 0; b < groups; ++b) {
            float mn = bo_bf16_to_f32(xr[b * G]), mx = mn;
            for (int i = 1; i < G; ++i) {
                float v = bo_bf16_to_f32(xr[b * G + i]);
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            float step = (mx - mn) / qmax;
            uint16_t sb = bo_bf16_from_f32(step);
            uint16_t bb = bo_bf16_from_f32(mn);
            scales[r * groups + b] = sb;
            biases[r * groups + b] = bb;
            float s = bo_bf16_to_f32(sb), bias = bo_bf16_to_f32(bb);
            float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
            for (int i = 0; i < G; ++i) {
                float t = (bo_bf16_to_f32(xr[b * G + i]) - bias) * inv;
                float q = nearbyintf(t);
                if (q < 0.0f) q = 0.0f;
                if (q > qmax) q = qmax;
                put_code_b(cr, b * G + i, (int)q, bits);
            }
        }
    }
}

/* [R17] MXFP8: one E8M0 exponent per 32 elements, E4M3 elements. */
void bo_quantize_mxfp8(const uint16_t* x, int64_t rows, int64_t cols,
                       uint32_t* codes, uint8_t* scales)
{
    const int G = 32;
    const int emax_e4m3 = 8; /* largest E4M3 magnitude 448 = 1.75 * 2^8 */
    const int64_t words = cols / 4, groups = cols / G;
    memset(codes, 0, (size_t)(rows * words) * sizeof(uint32_t));
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + r * cols;
        uint32_t* cr = codes + r * words;
        for (int64_t b = 0; b < groups; ++b) {
            float bamax = 0.0f;
            for (int i = 0; i < G; ++i) {
                float a = fabsf(bo_bf16_to_f32(xr[b * G + i]));
                if (a > bamax) bamax = a;
            }
            int e = (bamax == 0.0f) ? -127 : floor_log2((double)bamax) - emax_e4m3;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
            scales[r * groups + b] = (uint8_t)(e + 127);
            for (int i = 0; i < G; ++i) {
                float v = ldexpf(bo_bf16_to_f32(xr[b * G + i]), -e);
                put_code_b(cr, b * G + i, e4m3_encode_signed(v), 8);
            }
        }
    }
}

/* Format variants to bf16 [R8]: affine bf16(fma(s, q, b)); MXFP8
 * bf16(E4M3 * 2^e) with the product in fp32.  mode 0 affine, 3 MXFP8. */
void bo_dequantize_g(int mode, int bits, int G, const uint32_t* codes, const void* scales,
                     const uint16_t* biases, int64_t rows, int64_t cols, uint16_t* out)
{
    const int64_t words = cols * bits / 32, groups = cols / G;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            int c = get_code_b(codes + r * words, k, bits);
            if (mode == 0) {
                const uint16_t* s16 = (const uint16_t*)scales;
                float s = bo_bf16_to_f32(s16[r * groups + k / G]);
                float b = bo_bf16_to_f32(biases[r * groups + k / G]);
                out[r * cols + k] = bo_bf16_from_f32(fmaf(s, (float)c, b));
            } else {
                const uint8_t* s8 = (const uint8_t*)scales;
                float t = (float)(e4m3_decode_signed(c) * bo_e8m0_decode(s8[r * groups + k / G]));
                out[r * cols + k] = bo_bf16_from_f32(t);
            }
        }
}

/* Exact real values (fp64) of the format variants. */
void bo_dequant_exact_g(int mode, int bits, int G, const uint32_t* codes, const void* scales,
                        const uint16_t* biases, int64_t rows, int64_t cols, double* out)
{
    const int64_t words = cols * bits / 32, groups = cols / G;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            int c = get_code_b(codes + r * words, k, bits);
            if (mode == 0) {
                const uint16_t* s16 = (const uint16_t*)scales;
                double s = bo_bf16_to_f32(s16[r * groups + k / G]);
                double b = bo_bf16_to_f32(biases[r * groups + k / G]);
                out[r * cols + k] = s * c + b;
            } else {
                const uint8_t* s8 = (const uint8_t*)scales;
                out[r * cols + k] = e4m3_decode_signed(c) * bo_e8m0_decode(s8[r * groups + k / G]);
            }
        }
}

/* ======================================================================== */
/* dequantize to bf16 [R8]                                                    */
/* ======================================================================== */

/* ("mlx 0.30.7.3 -> 0.30.7.6", quantized.cpp, fast::Quantize::eval_gpu:
 * fp_dequantize with an optional NVFP4 global scale.) */
void bo_dequantize_nvfp4(const uint32_t* codes, const uint8_t* scales,
                         const float* g, int64_t rows, int64_t cols,
                         uint16_t* out)
{
    const int64_t words = cols / 8, groups = cols / 16;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            double e = bo_e2m1_decode(get_code(codes + r * words, k));
            double S = bo_e4m3_decode(scales[r * groups + k / 16]);
            float t = (float)(e * S); /* exact: at most 6 significant bits */
            if (g) t = t * (*g);
            out[r * cols + k] = bo_bf16_from_f32(t);
        }
}

void bo_dequantize_mxfp4(const uint32_t* codes, const uint8_t* scales,
                         int64_t rows, int64_t cols, uint16_t* out)
{
    const int64_t words = cols / 8, groups = cols / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            double e = bo_e2m1_decode(get_code(codes + r * words, k));
            double S = bo_e8m0_decode(scales[r * groups + k / 32]);
            out[r * cols + k] = bo_bf16_from_f32((float)(e * S));
        }
}

void bo_dequantize_affine(const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, int64_t rows, int64_t cols,
                          uint16_t* out)
{
    const int64_t words = cols / 8, groups = cols / 64;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            float q = (float)get_code(codes + r * words, k);
            float s = bo_bf16_to_f32(scales[r * groups + k / 64]);
            float b = bo_bf16_to_f32(biases[r * groups + k / 64]);
            out[r * cols + k] = bo_bf16_from_f32(fmaf(s, q, b));
        }
}

/* ======================================================================== */
/* exact dequantized operands (fp64)                                         */
/* ======================================================================== */

void bo_dequant_exact(int mode, const uint32_t* codes, const void* scales,
                      const uint16_t* biases, const float* g,
                      int64_t rows, int64_t cols, double* out)
{
    const int64_t words = cols / 8;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            int c = get_code(codes + r * words, k);
            double v;
            if (mode == 0) {
                const uint16_t* s16 = (const uint16_t*)scales;
                double s = bo_bf16_to_f32(s16[r * (cols / 64) + k / 64]);
                double b = bo_bf16_to_f32(biases[r * (cols / 64) + k / 64]);
                v = s * c + b;
            } else if (mode == 1) {
                const uint8_t* s8 = (const uint8_t*)scales;
                v = bo_e2m1_decode(c) * bo_e8m0_decode(s8[r * (cols / 32) + k / 32]);
            } else {
                const uint8_t* s8 = (const uint8_t*)scales;
                v = bo_e2m1_decode(c) * bo_e4m3_decode(s8[r * (cols / 16) + k / 16]);
                if (g) v *= (double)(*g);
            }
            out[r * cols + k] = v;
        }
}

/* ======================================================================== */
/* matmul: y = scale * A . B^T in fp64 (B holds W's rows, the pages' MLX     */
/* "transposed" weight layout: "mlx 0.30.7.3 -> 0.30.7.6", qqmm.cpp,         */
/* QQMatmul::eval_gpu, w_transposed = true)                                   */
/* ======================================================================== */

void bo_matmul_f64(const double* A, const double* B, int64_t M, int64_t N,
                   int64_t K, double scale, double* y, double* denom)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = A[m * K + k] * B[n * K + k];
                s += p;
                sa += fabs(p);
            }
            if (y) y[m * N + n] = scale * s;
            if (denom) denom[m * N + n] = fabs(scale) * sa;
        }
}

void bo_matmul_f64_pairs(const double* A_rows, const double* B_rows, int64_t K,
                         const int64_t* ai, const int64_t* bi, int64_t count,
                         double scale, double* y, double* denom)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const double* a = A_rows + ai[t] * K;
        const double* b = B_rows + bi[t] * K;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = a[k] * b[k];
            s += p;
            sa += fabs(p);
        }
        if (y) y[t] = scale * s;
        if (denom) denom[t] = fabs(scale) * sa;
    }
}
