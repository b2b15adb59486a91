/*
 * fp4q_oracle.c -- CPU oracle for block-scaled FP4 quantize / dequantize.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, single-threaded
 * statement of what the quantize-dequantize path computes.  Only tests/,
 * the smoke check in __graft_entry__.py and the cpu_baseline leg of bench.py
 * load it; the library under microscaling_fp4_block_fp4q_amd/ never does, and
 * the two share no source, header, table or helper.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared.
 * On x86-64 every `float` operation below is one IEEE-754 binary32 operation
 * rounded to nearest-even (SSE2, FLT_EVAL_METHOD == 0, no contraction), so
 * the fp32 operation sequence written here IS the specification that the
 * GPU path has to reproduce bit for bit.  fp64 appears only where it is
 * exact (grid distances, format decoding, narrowing conversions).
 *
 * Sources (page title, then section on that page):
 *  [MR-GPTQ]  "Bridging the Gap Between Promise and Performance for
 *             Microscaling FP4 Quantization" -- technical summary, section 1
 *             (MXFP4 = E8M0 power-of-two block scale; NVFP4 = block of 16),
 *             section 2.1/2.2 (block-wise Hadamard rotation, MSE-optimised
 *             scales per group).
 *  [FINER]    "Finer is Better (with the Right Scaling)" -- method, part 1
 *             (numerical study: OCP E2M1 elements, E4M3 scale factors, block
 *             sizes 4/8/16/32) and part 2 (scaling strategies: abs-max,
 *             prevent-zero, 4-over-6, brute-force search, hierarchical
 *             per-tensor-then-per-block scaling); key findings (region A
 *             underflow, region B clipping at 6.0).
 *  [FOCUS]    "FOCUS: FP4 Optimization via Coupled-Relaxation and
 *             Dual-Granularity Scaling" -- method 1 (scale learning with a
 *             straight-through estimator), method 2 (CRS: S_q = S_dq * c_i,
 *             c_i in FP16 initialised to 1), method 3 (DGS: sub-blocks of e.g.
 *             8 inside each hardware block, W_k quantized with
 *             Q(W_k / (S_dq * c_k)), S_dq shared by the block), method 4
 *             (only FP4 weights and S_dq are deployed).
 *
 * The pages never spell out the quantizer Q, the scale formulas, the
 * global-scale constant, rounding or tie rules.  Where they are silent this
 * file takes the plainest reading (OCP formats, round-half-to-even, abs-max
 * mapped onto the largest element 6.0, global scale = tensor abs-max /
 * (6 * 448)); every such reading is listed in the design notes.
 *
 * Parity pins: every function here is checked by tests/test_oracle_*.py
 * against something other than itself (exact rational arithmetic, torch's
 * float8/bfloat16/float16 casts, scipy's Hadamard matrix, closed forms,
 * brute force, finite differences).  One reading has nothing to pin it:
 * the exponent bias 15 of the UE5M3 scale format, which no page states
 * ("parity unpinned" for that bias; its rounding, saturation and use in
 * every strategy are pinned like E4M3's).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
enum { SF_E8M0 = 0, SF_E4M3 = 1, SF_UE5M3 = 2 };
enum { ST_ABSMAX = 0, ST_PREVENT_ZERO = 1, ST_FOUR_OVER_SIX = 2, ST_BRUTE_FORCE = 3, ST_GIVEN = 4 };
enum { GM_NONE = 0, GM_TENSOR_AMAX = 1, GM_USER = 2, GM_SEARCH = 3 };

/* Candidate shrink factors of the per-tensor scale search: rho_j = 1 - j/64,
 * j = 0 .. SEARCH_CANDIDATES - 1 (exact in fp32). */
#define SEARCH_CANDIDATES 32

#define E4M3_NAN_CODE 0x7F
#define UE5M3_NAN_CODE 0xFF
#define E8M0_NAN_CODE 0xFF
#define QNAN_BITS 0x7FC00000u

static float f32_of_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_of_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
static float canonical_nan(int negative) { return f32_of_bits(QNAN_BITS | (negative ? 0x80000000u : 0u)); }

/* ------------------------------------------------------------------------ */
/* Element and scale formats                                                 */
/* ------------------------------------------------------------------------ */

/* OCP E2M1 magnitudes, indexed by the 3-bit magnitude code (bit 0 is the
 * mantissa bit, so an even code has an even mantissa). */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Q of [FOCUS] method 3 / round-to-nearest of [FINER] part 1: the E2M1
 * magnitude code nearest to |u|; a tie goes to the even code; anything past
 * 6 saturates to 6; NaN gives 0.  Plain nearest-of-eight search. */
int oracle_e2m1_mag(float u)
{
    if (isnan(u)) return 0;
    double a = fabs((double)u);
    if (a > 6.0) return 7;                   /* saturation (also for inf) */
    int best = 0;
    double best_d = a;                       /* distance to magnitude 0 */
    for (int m = 1; m < 8; ++m) {
        double d = fabs(a - E2M1_MAG[m]);    /* exact: a <= 6 is an fp32 value */
        if (d < best_d || (d == best_d && (m & 1) == 0)) { best = m; best_d = d; }
    }
    return best;
}

double oracle_e2m1_value(int mag) { return E2M1_MAG[mag & 7]; }

/* OCP E4M3 (the "FN" variant: bias 7, no infinities, 0x7F is NaN, max 448).
 * Used as an unsigned block scale, so bit 7 of a stored code is ignored. */
double oracle_e4m3_decode(int code)
{
    code &= 0x7F;
    if (code == E4M3_NAN_CODE) return NAN;
    int e = code >> 3, m = code & 7;
    if (e == 0) return m * ldexp(1.0, -9);               /* subnormal */
    return (1.0 + m / 8.0) * ldexp(1.0, e - 7);
}

/* Round v >= 0 to the nearest finite E4M3 value, ties to the even code,
 * saturating at 448 (satfinite); NaN -> the NaN code.  Plain search over the
 * 127 finite codes. */
int oracle_e4m3_encode(float v)
{
    if (isnan(v)) return E4M3_NAN_CODE;
    double a = fabs((double)v);
    if (a >= 448.0) return 0x7E;
    int best = 0;
    double best_d = a;
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - oracle_e4m3_decode(c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) { best = c; best_d = d; }
    }
    return best;
}

/* E8M0: 2^(code-127), code 0xFF is NaN, there is no zero. */
double oracle_e8m0_decode(int code)
{
    code &= 0xFF;
    if (code == E8M0_NAN_CODE) return NAN;
    return ldexp(1.0, code - 127);
}

/* UE5M3: the unsigned wide-exponent scale format the Finer-is-Better page
 * (key findings and significance) sets against E4M3 + hierarchical scaling
 * + 4-over-6.  The page gives no encoding; reading: 5 exponent bits with
 * bias 15, 3 mantissa bits, subnormals m * 2^-17, no infinities, 0xFF NaN,
 * so the largest value is 0xFE = 1.75 * 2^16.  (The bias is a reading with
 * nothing on the page to pin it: parity unpinned for the bias.) */
double oracle_ue5m3_decode(int code)
{
    code &= 0xFF;
    if (code == UE5M3_NAN_CODE) return NAN;
    int e = code >> 3, m = code & 7;
    if (e == 0) return m * ldexp(1.0, -17);
    return (1.0 + m / 8.0) * ldexp(1.0, e - 15);
}

/* Round v >= 0 to the nearest finite UE5M3 value, ties to the even code,
 * saturating at the largest value; NaN -> the NaN code.  Plain search over
 * the 255 finite codes. */
int oracle_ue5m3_encode(float v)
{
    if (isnan(v)) return UE5M3_NAN_CODE;
    double a = fabs((double)v);
    double top = oracle_ue5m3_decode(0xFE);
    if (a >= top) return 0xFE;
    int best = 0;
    double best_d = a;
    for (int c = 1; c <= 0xFE; ++c) {
        double d = fabs(a - oracle_ue5m3_decode(c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) { best = c; best_d = d; }
    }
    return best;
}

/* MXFP4 abs-max scale ([MR-GPTQ] section 1: power-of-two rounding of the
 * scale): the largest power of two 2^k with 2^k * 4 <= a_b, i.e.
 * k = floor(log2 a_b) - 2 (the exponent of 6.0 = 1.5 * 2^2), so a_b / 2^k
 * lies in [4, 8) and the block maximum clips at 6.  Codes are clamped to
 * [0, 254]; a zero or tiny block gets code 0. */
int oracle_e8m0_absmax_code(float a_b)
{
    if (!(a_b >= ldexp(1.0, -124))) return 0;      /* zero, subnormal, tiny */
    int e;
    frexp((double)a_b, &e);                        /* a_b in [2^(e-1), 2^e) */
    int code = (e - 1) - 2 + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
    return code;
}

/* ------------------------------------------------------------------------ */
/* Element types                                                             */
/* ------------------------------------------------------------------------ */

float oracle_bf16_to_f32(uint16_t h) { return f32_of_bits((uint32_t)h << 16); }

float oracle_f16_to_f32(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = m * ldexp(1.0, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = (1024 + m) * ldexp(1.0, e - 25);
    return (float)(s ? -v : v);
}

/* Round-half-to-even of a non-negative double that is an exact multiple of
 * 1/2 or finer (the defaults of nearbyint are round-to-nearest-even). */
static double rne(double q) { return nearbyint(q); }

/* fp32 -> bf16, round-half-to-even, NaN -> quiet NaN with the same sign. */
uint16_t oracle_bf16_from_f32(float f)
{
    uint16_t sign = (bits_of_f32(f) >> 16) & 0x8000;
    if (isnan(f)) return sign | 0x7FC0;
    double a = fabs((double)f);
    /* largest finite bf16 is (2 - 2^-7) * 2^127; at or past the midpoint to
     * the next binade the value rounds to infinity (ties go to even = inf) */
    if (a >= (2.0 - ldexp(1.0, -8)) * ldexp(1.0, 127)) return sign | 0x7F80;
    if (a < ldexp(1.0, -126)) {                   /* subnormal spacing 2^-133 */
        double m = rne(ldexp(a, 133));
        return sign | (uint16_t)m;
    }
    int e;
    frexp(a, &e);
    int E = e - 1;                                /* a in [2^E, 2^(E+1)) */
    double m = rne(ldexp(a, 7 - E));              /* in [128, 256] */
    return sign | (uint16_t)(((E + 127) << 7) + ((int)m - 128));
}

/* fp32 -> fp16, round-half-to-even, overflow -> inf, NaN -> quiet NaN. */
uint16_t oracle_f16_from_f32(float f)
{
    uint16_t sign = (bits_of_f32(f) >> 16) & 0x8000;
    if (isnan(f)) return sign | 0x7E00;
    double a = fabs((double)f);
    if (a >= 65520.0) return sign | 0x7C00;       /* 65504 + half ulp -> inf */
    if (a < ldexp(1.0, -14)) {                    /* subnormal spacing 2^-24 */
        double m = rne(ldexp(a, 24));
        return sign | (uint16_t)m;
    }
    int e;
    frexp(a, &e);
    int E = e - 1;
    double m = rne(ldexp(a, 10 - E));             /* in [1024, 2048] */
    return sign | (uint16_t)(((E + 15) << 10) + ((int)m - 1024));
}

static float load_elem(const void* base, int dt, int64_t idx)
{
    if (dt == DT_F32) return ((const float*)base)[idx];
    if (dt == DT_BF16) return oracle_bf16_to_f32(((const uint16_t*)base)[idx]);
    return oracle_f16_to_f32(((const uint16_t*)base)[idx]);
}

static void store_elem(void* base, int dt, int64_t idx, float v)
{
    if (dt == DT_F32) ((float*)base)[idx] = v;
    else if (dt == DT_BF16) ((uint16_t*)base)[idx] = oracle_bf16_from_f32(v);
    else ((uint16_t*)base)[idx] = oracle_f16_from_f32(v);
}

/* ------------------------------------------------------------------------ */
/* Block-wise Hadamard rotation ([MR-GPTQ] sections 2.1, 2.2)                */
/* ------------------------------------------------------------------------ */

/* fl(1 / sqrt(n)) for the normalised transform. */
float oracle_hadamard_coef(int n) { return (float)(1.0 / sqrt((double)n)); }

/* In-place normalised Walsh-Hadamard transform of one segment of n = 2^k
 * values, Sylvester (natural) order: radix-2 butterflies with stride
 * h = 1, 2, 4, ..., n/2, each pair (a, b) -> (a + b, a - b) in fp32, then one
 * multiplication of every output by fl(1/sqrt(n)). */
void oracle_fwht(float* v, int n)
{
    for (int h = 1; h < n; h <<= 1)
        for (int i = 0; i < n; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    float c = oracle_hadamard_coef(n);
    for (int i = 0; i < n; ++i) v[i] = v[i] * c;
}

/* ------------------------------------------------------------------------ */
/* One block: encode, dequantize, error                                      */
/* ------------------------------------------------------------------------ */

/* Balanced binary tree sum in index order: sum(v[0:n]) =
 * sum(v[0:n/2]) + sum(v[n/2:n]); n is a power of two. */
float oracle_tree_sum(const float* v, int n)
{
    if (n == 1) return v[0];
    float left = oracle_tree_sum(v, n / 2);
    float right = oracle_tree_sum(v + n / 2, n / 2);
    return left + right;
}

/* A block scale is usable when it is a number, finite and not negative;
 * anything else turns the block into a NaN block. */
static int scale_usable(float S) { return !isnan(S) && !isinf(S) && !(S < 0.0f); }

/* Effective scale S = fl(dec(code) * g); the decoded value is exact in fp32. */
static float effective_scale(int fmt, int code, float g)
{
    double d = (fmt == SF_E8M0) ? oracle_e8m0_decode(code)
             : (fmt == SF_E4M3) ? oracle_e4m3_decode(code) : oracle_ue5m3_decode(code);
    return (float)d * g;
}

/* Quantize one element y at scale S (usable): magnitude code, sign, and the
 * fp32 dequantized value  (-1)^sign * fl(grid[mag] * S). */
static int encode_elem(float y, float S, float* yhat)
{
    float u = (S == 0.0f) ? 0.0f : y / S;
    int mag = oracle_e2m1_mag(u);
    int neg = signbit(y) ? 1 : 0;
    float v = (float)E2M1_MAG[mag] * S;
    *yhat = copysignf(v, neg ? -1.0f : 1.0f);
    return (neg << 3) | mag;
}

/* Sum of squared errors of one block of B values quantized at scale S:
 * d_i = fl(y_i - yhat_i), e_i = fl(d_i * d_i), tree sum of e. */
float oracle_block_sse(const float* y, int B, float S)
{
    float e[32];
    if (!scale_usable(S)) return canonical_nan(0);
    for (int i = 0; i < B; ++i) {
        float yh;
        encode_elem(y[i], S, &yh);
        float d = y[i] - yh;
        e[i] = d * d;
    }
    return oracle_tree_sum(e, B);
}

/* Block abs-max as the largest |bit pattern| (exact, order-free; NaN and inf
 * order above every finite value). */
static uint32_t block_amax_bits(const float* y, int n)
{
    uint32_t m = 0;
    for (int i = 0; i < n; ++i) {
        uint32_t b = bits_of_f32(y[i]) & 0x7FFFFFFFu;
        if (b > m) m = b;
    }
    return m;
}

/* Scale-factor selection for one block ([FINER] part 2).  Returns the code.
 * g is the per-tensor scale (1 when there is none). */
static int choose_scale(int fmt, int strategy, const float* y, int B, float g, int given)
{
    if (strategy == ST_GIVEN) return (fmt == SF_E4M3) ? (given & 0x7F) : given;
    uint32_t ab_bits = block_amax_bits(y, B);
    float a_b = f32_of_bits(ab_bits);
    int nan_code = (fmt == SF_E8M0) ? E8M0_NAN_CODE : (fmt == SF_E4M3) ? E4M3_NAN_CODE : UE5M3_NAN_CODE;
    if (ab_bits >= 0x7F800000u || isnan(g) || isinf(g)) return nan_code;

    if (fmt == SF_E8M0) {
        if (strategy == ST_BRUTE_FORCE) {
            int best = -1;
            float best_sse = 0.0f;
            for (int c = 0; c <= 254; ++c) {
                float sse = oracle_block_sse(y, B, effective_scale(fmt, c, g));
                if (best < 0 || sse < best_sse) { best = c; best_sse = sse; }
            }
            return best;
        }
        /* abs-max; prevent-zero is the same rule since E8M0 has no zero */
        return oracle_e8m0_absmax_code(a_b);
    }

    /* E4M3 (and UE5M3): abs-max maps the block maximum onto 6 = the largest
     * E2M1 value, rounded to the nearest scale value. */
    int (*encode)(float) = (fmt == SF_E4M3) ? oracle_e4m3_encode : oracle_ue5m3_encode;
    int top_code = (fmt == SF_E4M3) ? 0x7E : 0xFE;
    float six_g = 6.0f * g;
    int s6 = encode(a_b / six_g);
    switch (strategy) {
    case ST_ABSMAX:
        return s6;
    case ST_PREVENT_ZERO:                 /* clip to the smallest nonzero scale */
        return s6 < 1 ? 1 : s6;
    case ST_FOUR_OVER_SIX: {              /* map the maximum to 6 or to 4 */
        float four_g = 4.0f * g;
        int s4 = encode(a_b / four_g);
        float sse6 = oracle_block_sse(y, B, effective_scale(fmt, s6, g));
        float sse4 = oracle_block_sse(y, B, effective_scale(fmt, s4, g));
        return (sse4 < sse6) ? s4 : s6;  /* equal error keeps the smaller code */
    }
    case ST_BRUTE_FORCE: {                /* every positive finite scale */
        int best = -1;
        float best_sse = 0.0f;
        for (int c = 1; c <= top_code; ++c) {
            float sse = oracle_block_sse(y, B, effective_scale(fmt, c, g));
            if (best < 0 || sse < best_sse) { best = c; best_sse = sse; }
        }
        return best;
    }
    }
    return nan_code;
}

/* ------------------------------------------------------------------------ */
/* Tensor-level entry points                                                 */
/* ------------------------------------------------------------------------ */

/* Widen a [rows, cols] tensor with row stride ld to a dense fp32 copy and
 * rotate each contiguous segment of H values when H != 0.  A NaN the
 * rotation produces is taken as the positive quiet NaN: IEEE 754 does not
 * fix the sign of a NaN that arithmetic returns, and that sign would reach
 * the sign bit of the element's code. */
static float* widen_and_rotate(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld, int H)
{
    float* y = (float*)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
    if (!y) return NULL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) y[r * cols + c] = load_elem(x, dt, r * ld + c);
    if (H > 0) {
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = 0; c < cols; c += H) oracle_fwht(y + r * cols + c, H);
        for (int64_t i = 0; i < rows * cols; ++i)
            if (isnan(y[i])) y[i] = canonical_nan(0);
    }
    return y;
}

/* Hierarchical scaling ([FINER] part 2): per-tensor scale
 * g = fl(amax_t / (6 * 448)) so that the tensor maximum lands on the
 * largest E2M1 value times the largest E4M3 value; g = 1 for a tensor whose
 * quotient is zero; NaN when the tensor holds a NaN or an infinity. */
float oracle_global_scale(const float* y, int64_t n)
{
    uint32_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b = bits_of_f32(y[i]) & 0x7FFFFFFFu;
        if (b > m) m = b;
    }
    if (m >= 0x7F800000u) return canonical_nan(0);
    float g = f32_of_bits(m) / 2688.0f;
    return (g == 0.0f) ? 1.0f : g;
}

/* Per-tensor scale of a whole [rows, cols] tensor (rotated first when
 * H != 0), as the hierarchical mode computes it; lets a test quantize a
 * sample of rows with the scale of the full tensor. */
float oracle_tensor_global_scale(const void* x, int x_dt, int64_t rows, int64_t cols, int64_t ld_x, int H)
{
    float* y = widen_and_rotate(x, x_dt, rows, cols, ld_x, H);
    if (!y) return canonical_nan(0);
    float g = oracle_global_scale(y, rows * cols);
    free(y);
    return g;
}

/* fp64 balanced binary tree over v[0:n] zero-padded to len (a power of two
 * >= n): sum(v[0:len]) = sum(v[0:len/2]) + sum(v[len/2:len]). */
static double tree_sum_f64_padded(const double* v, int64_t n, int64_t len)
{
    if (n <= 0) return 0.0;
    if (len == 1) return v[0];
    int64_t half = len / 2;
    double left = tree_sum_f64_padded(v, n < half ? n : half, half);
    double right = tree_sum_f64_padded(v + half, n - half, half);
    return left + right;
}

/* MSE-optimised per-tensor scale ([MR-GPTQ] section 2.2: scale grids chosen
 * for minimum MSE per tensor; [FINER] part 2 names optimal scale selection as
 * open).  Starting from the hierarchical scale g0 of the (rotated) tensor,
 * candidates g_j = fl(g0 * rho_j) shrink it so that the largest blocks clip
 * in exchange for finer scales elsewhere; each candidate quantizes every
 * block with the inner strategy (E4M3 scales) and scores the tensor by the
 * fp64 tree sum (over all blocks in row-major order, zero-padded to a power
 * of two) of the fp32 block SSEs.  The smallest total wins, ties to the
 * smallest j (the least shrink).  totals (optional) receives the
 * SEARCH_CANDIDATES sums.  A tensor with NaN or infinity gives g = NaN. */
static float search_global_scale(int strategy, int B, const float* y, int64_t rows, int64_t cols,
                                 double* totals)
{
    float g0 = oracle_global_scale(y, rows * cols);
    int64_t nblk = rows * (cols / B), len = 1;
    while (len < nblk) len <<= 1;
    double* sse = (double*)malloc(sizeof(double) * (size_t)(nblk > 0 ? nblk : 1));
    if (!sse) return canonical_nan(0);
    int best = 0;
    double best_total = 0.0;
    for (int j = 0; j < SEARCH_CANDIDATES; ++j) {
        float g = g0 * (float)(1.0 - j / 64.0);
        for (int64_t b = 0; b < nblk; ++b) {
            const float* yb = y + b * B;            /* blocks are consecutive in row-major order */
            int code = choose_scale(SF_E4M3, strategy, yb, B, g, 0);
            float S = (code == E4M3_NAN_CODE) ? canonical_nan(0) : effective_scale(SF_E4M3, code, g);
            sse[b] = (double)oracle_block_sse(yb, B, S);
        }
        double total = tree_sum_f64_padded(sse, nblk, len);
        if (totals) totals[j] = total;
        if (j == 0 || total < best_total || (isnan(best_total) && !isnan(total))) {
            best = j;
            best_total = total;
        }
    }
    free(sse);
    return g0 * (float)(1.0 - best / 64.0);
}

/* The searched per-tensor scale of x and, optionally, the candidates'
 * totals; lets tests check the search on its own. */
float oracle_global_scale_search(int strategy, int B, int H, const void* x, int x_dt, int64_t rows,
                                 int64_t cols, int64_t ld_x, double* totals)
{
    float* y = widen_and_rotate(x, x_dt, rows, cols, ld_x, H);
    if (!y) return canonical_nan(0);
    float g = search_global_scale(strategy, B, y, rows, cols, totals);
    free(y);
    return g;
}

/* Quantize a [rows, cols] tensor in blocks of B along each row.
 * Outputs (each may be NULL): packed codes [rows, cols/2] (low nibble = even
 * column), scales [rows, cols/B] (input when strategy is GIVEN), g_out,
 * dequantized values [rows, ld_dq] of type dq_dt, per-block MSE and SSE
 * [rows, cols/B].  Returns 0, or -1 on an argument it does not handle. */
int oracle_quantize(int fmt, int B, int strategy, int global_mode, float user_g, int H,
                    const void* x, int x_dt, int64_t rows, int64_t cols, int64_t ld_x,
                    uint8_t* codes, uint8_t* scales, float* g_out,
                    void* dq, int dq_dt, int64_t ld_dq, float* mse, float* sse_out)
{
    if (B != 4 && B != 8 && B != 16 && B != 32) return -1;
    if (H != 0 && H != 16 && H != 32) return -1;
    if (cols % B || (H && cols % H) || cols % 2) return -1;
    if (fmt == SF_E8M0 && (global_mode != GM_NONE || strategy == ST_FOUR_OVER_SIX)) return -1;
    if (fmt == SF_UE5M3 && global_mode != GM_NONE && global_mode != GM_USER) return -1;
    if (strategy == ST_GIVEN && (!scales || global_mode == GM_SEARCH)) return -1;

    float* y = widen_and_rotate(x, x_dt, rows, cols, ld_x, H);
    if (!y) return -1;

    float g = 1.0f;
    if (global_mode == GM_USER) g = user_g;
    else if (global_mode == GM_TENSOR_AMAX) g = oracle_global_scale(y, rows * cols);
    else if (global_mode == GM_SEARCH) g = search_global_scale(strategy, B, y, rows, cols, NULL);
    if (g_out) *g_out = g;

    int64_t nb = cols / B;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < nb; ++j) {
            const float* yb = y + r * cols + j * B;
            int given = (strategy == ST_GIVEN) ? scales[r * nb + j] : 0;
            int code = choose_scale(fmt, strategy, yb, B, g, given);
            if (scales && strategy != ST_GIVEN) scales[r * nb + j] = (uint8_t)code;

            int nan_code = (fmt == SF_E8M0) ? E8M0_NAN_CODE : (fmt == SF_E4M3) ? E4M3_NAN_CODE : UE5M3_NAN_CODE;
            float S = (code == nan_code) ? canonical_nan(0) : effective_scale(fmt, code, g);
            int usable = scale_usable(S);

            float e[32];
            for (int i = 0; i < B; ++i) {
                float yi = yb[i], yh;
                int q;
                if (usable) {
                    q = encode_elem(yi, S, &yh);
                } else {
                    q = signbit(yi) ? 8 : 0;
                    yh = canonical_nan(signbit(yi));
                }
                float d = yi - yh;
                e[i] = d * d;
                int64_t col = j * B + i;
                if (codes) {
                    uint8_t* byte = codes + r * (cols / 2) + col / 2;
                    if ((col & 1) == 0) *byte = (uint8_t)q;
                    else *byte = (uint8_t)(*byte | (q << 4));
                }
                if (dq) store_elem(dq, dq_dt, r * ld_dq + col, yh);
            }
            float sse = usable ? oracle_tree_sum(e, B) : canonical_nan(0);
            if (isnan(sse)) sse = canonical_nan(0);
            if (sse_out) sse_out[r * nb + j] = sse;
            if (mse) {
                float m = sse / (float)B;
                mse[r * nb + j] = isnan(m) ? canonical_nan(0) : m;
            }
        }
    }
    free(y);
    return 0;
}

/* Decode one stored code at scale S (usable or not). */
static float decode_elem(int q, float S)
{
    int neg = (q >> 3) & 1;
    if (!scale_usable(S)) return canonical_nan(neg);
    float v = (float)E2M1_MAG[q & 7] * S;
    return copysignf(v, neg ? -1.0f : 1.0f);
}

static float stored_scale(int fmt, int code, float g)
{
    if (fmt == SF_E4M3) code &= 0x7F;
    int nan_code = (fmt == SF_E8M0) ? E8M0_NAN_CODE : (fmt == SF_E4M3) ? E4M3_NAN_CODE : UE5M3_NAN_CODE;
    if (code == nan_code) return canonical_nan(0);
    return effective_scale(fmt, code, g);
}

/* Dequantize packed codes + scales (+ g) to [rows, ld_out] values. */
int oracle_dequantize(int fmt, int B, const uint8_t* codes, const uint8_t* scales, float g,
                      int64_t rows, int64_t cols, void* out, int out_dt, int64_t ld_out)
{
    if (B != 4 && B != 8 && B != 16 && B != 32) return -1;
    if (cols % B || cols % 2) return -1;
    int64_t nb = cols / B;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            int q = (c & 1) ? (byte >> 4) : (byte & 15);
            float S = stored_scale(fmt, scales[r * nb + c / B], g);
            store_elem(out, out_dt, r * ld_out + c, decode_elem(q, S));
        }
    return 0;
}

/* Per-block MSE of x (rotated when H != 0) against stored codes + scales. */
int oracle_block_mse(int fmt, int B, int H, const void* x, int x_dt, int64_t rows, int64_t cols,
                     int64_t ld_x, const uint8_t* codes, const uint8_t* scales, float g, float* mse)
{
    if (B != 4 && B != 8 && B != 16 && B != 32) return -1;
    if (cols % B || (H && cols % H) || cols % 2) return -1;
    float* y = widen_and_rotate(x, x_dt, rows, cols, ld_x, H);
    if (!y) return -1;
    int64_t nb = cols / B;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < nb; ++j) {
            float S = stored_scale(fmt, scales[r * nb + j], g);
            float e[32];
            for (int i = 0; i < B; ++i) {
                int64_t c = j * B + i;
                uint8_t byte = codes[r * (cols / 2) + c / 2];
                int q = (c & 1) ? (byte >> 4) : (byte & 15);
                float d = y[r * cols + c] - decode_elem(q, S);
                e[i] = d * d;
            }
            float m = oracle_tree_sum(e, B) / (float)B;
            mse[r * nb + j] = isnan(m) ? canonical_nan(0) : m;
        }
    free(y);
    return 0;
}

/* Codebook occupancy ([TORQ] section 2.B: the codeword usage whose collapse
 * onto the smallest codes the method measures against the uniform
 * distribution): counts[c] = number of nibbles equal to c, c = 0..15, in
 * packed codes [rows, cols/2] (sign bit 3, E2M1 magnitude bits 0-2). */
int oracle_code_histogram(const uint8_t* codes, int64_t rows, int64_t cols, uint64_t* counts)
{
    if (cols % 2) return -1;
    for (int c = 0; c < 16; ++c) counts[c] = 0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) {
            uint8_t byte = codes[r * (cols / 2) + j / 2];
            int q = (j & 1) ? (byte >> 4) : (byte & 15);
            counts[q] += 1;
        }
    return 0;
}

/* FP4 GEMM on MXFP4 operands ([MR-GPTQ] section 2.3: the QuTLASS kernels
 * multiply the packed FP4 weights and activations with their block scales):
 * C[m][n] = sum over k of dq(A)[m][k] * dq(B)[n][k], with dq the MXFP4 decode
 * (E2M1 grid value times 2^(scale-127) of the 32-element block, NaN for
 * scale 0xFF).  A codes [M, K/2] + scales [M, K/32], B likewise [N, ...];
 * products and sum in fp64 (every product of two decoded values is exact in
 * fp64, so C is the exact dot product rounded once per addition). */
int oracle_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                      const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, double* c)
{
    if (K % 32) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                uint8_t ab = a_codes[m * (K / 2) + k / 2], bb = b_codes[n * (K / 2) + k / 2];
                int qa = (k & 1) ? (ab >> 4) : (ab & 15), qb = (k & 1) ? (bb >> 4) : (bb & 15);
                double sa = oracle_e8m0_decode(a_scales[m * (K / 32) + k / 32]);
                double sb = oracle_e8m0_decode(b_scales[n * (K / 32) + k / 32]);
                double va = ((qa & 8) ? -1.0 : 1.0) * E2M1_MAG[qa & 7] * sa;
                double vb = ((qb & 8) ? -1.0 : 1.0) * E2M1_MAG[qb & 7] * sb;
                acc += va * vb;
            }
            c[m * N + n] = acc;
        }
    return 0;
}

/* FP4 GEMM on NVFP4 operands ([MR-GPTQ] section 2.3: QuTLASS multiplies
 * both MXFP4 and NVFP4 operands): C[m][n] = sum over k of dq(A)[m][k] *
 * dq(B)[n][k], with dq the NVFP4 decode that oracle_dequantize applies: the
 * E2M1 grid value times S = fl(dec(scale) * g) of its 16-element block
 * (E4M3 scale, per-tensor g of that operand), rounded to fp32 (NaN for
 * scale 0x7F).  A codes [M, K/2] + scales [M, K/16], B likewise [N, ...];
 * products and sum in fp64 (the decoded values are fp32, so every product
 * is exact in fp64 and C is the exact dot product rounded once per
 * addition). */
int oracle_nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, float g_a, const uint8_t* b_codes,
                      const uint8_t* b_scales, float g_b, int64_t M, int64_t N, int64_t K, double* c)
{
    if (K % 16) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                uint8_t ab = a_codes[m * (K / 2) + k / 2], bb = b_codes[n * (K / 2) + k / 2];
                int qa = (k & 1) ? (ab >> 4) : (ab & 15), qb = (k & 1) ? (bb >> 4) : (bb & 15);
                float sa = stored_scale(SF_E4M3, a_scales[m * (K / 16) + k / 16], g_a);
                float sb = stored_scale(SF_E4M3, b_scales[n * (K / 16) + k / 16], g_b);
                acc += (double)decode_elem(qa, sa) * (double)decode_elem(qb, sb);
            }
            c[m * N + n] = acc;
        }
    return 0;
}

/* FOCUS relaxed fake-quant forward ([FOCUS] methods 2-3): per sub-block k of
 * K values, S_q = fl(S_dq * c_k) with c_k an FP16 coefficient; the element
 * is encoded with u = fl(W / S_q) (0 when S_q is 0) and dequantized with the
 * hardware scale alone: What = (-1)^sign * fl(grid[mag] * S_dq).  Codes, when
 * requested, are the deployable FP4 weights of method 4. */
int oracle_relaxed_fwd(int fmt, int B, const void* w, int w_dt, int64_t rows, int64_t cols,
                       int64_t ld_w, const uint8_t* scales, float g, const uint16_t* c_f16, int K,
                       void* w_hat, int out_dt, int64_t ld_out, uint8_t* codes)
{
    if (B != 4 && B != 8 && B != 16 && B != 32) return -1;
    if (K < 1 || B % K || cols % B || cols % 2) return -1;
    int64_t nb = cols / B, nk = cols / K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float S_dq = stored_scale(fmt, scales[r * nb + c / B], g);
            float c_k = oracle_f16_to_f32(c_f16[r * nk + c / K]);
            float S_q = S_dq * c_k;
            float W = load_elem(w, w_dt, r * ld_w + c);
            float wh;
            int q;
            if (scale_usable(S_dq) && scale_usable(S_q)) {
                float u = (S_q == 0.0f) ? 0.0f : W / S_q;
                int mag = oracle_e2m1_mag(u);
                int neg = signbit(W) ? 1 : 0;
                wh = copysignf((float)E2M1_MAG[mag] * S_dq, neg ? -1.0f : 1.0f);
                q = (neg << 3) | mag;
            } else {
                q = signbit(W) ? 8 : 0;
                wh = canonical_nan(signbit(W));
            }
            store_elem(w_hat, out_dt, r * ld_out + c, wh);
            if (codes) {
                uint8_t* byte = codes + r * (cols / 2) + c / 2;
                if ((c & 1) == 0) *byte = (uint8_t)q;
                else *byte = (uint8_t)(*byte | (q << 4));
            }
        }
    return 0;
}

/* Straight-through backward to c_k ([FOCUS] method 1: scales are learned
 * through Q with the STE).  Q is replaced by the clip to [-6, 6], so inside
 * the clip range dWhat_i/dc_k = S_dq * d(W_i/(S_dq c_k))/dc_k = -W_i / c_k^2
 * and 0 outside:  dL/dc_k = fl(-A_k / fl(c_k * c_k)) with
 * A_k = tree sum over the sub-block of [S_q > 0 and |u_i| <= 6] * fl(G_i * W_i). */
int oracle_relaxed_bwd(int fmt, int B, const void* w, int w_dt, int64_t rows, int64_t cols,
                       int64_t ld_w, const uint8_t* scales, float g, const uint16_t* c_f16, int K,
                       const void* grad, int g_dt, int64_t ld_g, float* grad_c)
{
    if (B != 4 && B != 8 && B != 16 && B != 32) return -1;
    if (K < 1 || B % K || cols % B || cols % 2) return -1;
    int64_t nb = cols / B, nk = cols / K;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < nk; ++k) {
            int64_t c0 = k * K;
            float S_dq = stored_scale(fmt, scales[r * nb + c0 / B], g);
            float c_k = oracle_f16_to_f32(c_f16[r * nk + k]);
            float S_q = S_dq * c_k;
            float out;
            if (scale_usable(S_dq) && scale_usable(S_q)) {
                float t[32];
                for (int i = 0; i < K; ++i) {
                    float W = load_elem(w, w_dt, r * ld_w + c0 + i);
                    float G = load_elem(grad, g_dt, r * ld_g + c0 + i);
                    int inside = 0;
                    if (S_q > 0.0f) {
                        float u = W / S_q;
                        inside = fabsf(u) <= 6.0f;
                    }
                    t[i] = inside ? G * W : 0.0f;
                }
                float A = oracle_tree_sum(t, K);
                float cc = c_k * c_k;
                out = -A / cc;
            } else {
                out = canonical_nan(0);
            }
            grad_c[r * nk + k] = isnan(out) ? canonical_nan(0) : out;
        }
    return 0;
}
