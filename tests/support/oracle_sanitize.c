/* Driver that runs every entry point of the CPU oracle (oracle/fp4q_oracle.c)
 * over small seeded tensors, every format / block / strategy / global mode /
 * rotation / element type (invalid combinations included: the oracle must
 * refuse them cleanly), with special values (NaN, infinities, signed zeros,
 * subnormals, values on E2M1 grid points and bin boundaries), and prints one
 * FNV-1a hash per output buffer.
 *
 * tests/test_oracle_sanitizers.py builds it twice against the oracle source,
 * once plainly and once with AddressSanitizer + UndefinedBehaviorSanitizer
 * (no recovery, leak detection on), and requires both to exit cleanly with
 * identical hashes.  The plain build computes what the pinned oracle
 * computes; identical hashes show the sanitized run took the same paths.
 * The inputs come from a counter-based generator (splitmix64); nothing here
 * performs the method's arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle entry points (oracle/fp4q_oracle.c) */
int oracle_e2m1_mag(float u);
double oracle_e2m1_value(int mag);
double oracle_e4m3_decode(int code);
int oracle_e4m3_encode(float v);
double oracle_e8m0_decode(int code);
double oracle_ue5m3_decode(int code);
int oracle_ue5m3_encode(float v);
int oracle_e8m0_absmax_code(float a_b);
float oracle_bf16_to_f32(uint16_t h);
float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_bf16_from_f32(float f);
uint16_t oracle_f16_from_f32(float f);
float oracle_hadamard_coef(int n);
void oracle_fwht(float* v, int n);
float oracle_tree_sum(const float* v, int n);
float oracle_block_sse(const float* y, int B, float S);
float oracle_global_scale(const float* y, int64_t n);
float oracle_tensor_global_scale(const void* x, int x_dt, int64_t rows, int64_t cols, int64_t ld_x, int H);
float oracle_global_scale_search(int strategy, int B, int H, const void* x, int x_dt, int64_t rows,
                                 int64_t cols, int64_t ld_x, double* totals);
int oracle_quantize(int fmt, int B, int strategy, int global_mode, float user_g, int H, const void* x, int x_dt,
                    int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes, uint8_t* scales, float* g_out,
                    void* dq, int dq_dt, int64_t ld_dq, float* mse, float* sse_out);
int oracle_dequantize(int fmt, int B, const uint8_t* codes, const uint8_t* scales, float g, int64_t rows,
                      int64_t cols, void* out, int out_dt, int64_t ld_out);
int oracle_block_mse(int fmt, int B, int H, const void* x, int x_dt, int64_t rows, int64_t cols, int64_t ld_x,
                     const uint8_t* codes, const uint8_t* scales, float g, float* mse);
int oracle_code_histogram(const uint8_t* codes, int64_t rows, int64_t cols, uint64_t* counts);
int oracle_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                      const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, double* c);
int oracle_relaxed_fwd(int fmt, int B, const void* w, int w_dt, int64_t rows, int64_t cols, int64_t ld_w,
                       const uint8_t* scales, float g, const uint16_t* c_f16, int K, void* w_hat, int out_dt,
                       int64_t ld_out, uint8_t* codes);
int oracle_relaxed_bwd(int fmt, int B, const void* w, int w_dt, int64_t rows, int64_t cols, int64_t ld_w,
                       const uint8_t* scales, float g, const uint16_t* c_f16, int K, const void* grad, int g_dt,
                       int64_t ld_g, float* grad_c);

static uint64_t hash_bytes(const void* p, size_t n) {
    const unsigned char* b = (const unsigned char*)p;
    uint64_t h = 1469598103934665603ull;
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 1099511628211ull;
    return h;
}

static void emit(const char* what, int a, int b, int c, int d, int e, int f, const void* p, size_t n) {
    printf("%s %d %d %d %d %d %d %016llx\n", what, a, b, c, d, e, f, (unsigned long long)hash_bytes(p, n));
}

static uint64_t splitmix(uint64_t* s) {
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static float uniform(uint64_t* s) { return (float)((splitmix(s) >> 40) * 0x1p-24); }

/* roughly normal: sum of four uniforms, centred */
static float gaussish(uint64_t* s) { return (uniform(s) + uniform(s) + uniform(s) + uniform(s) - 2.0f) * 1.7f; }

static float special(int k, uint64_t* s) {
    static const float grid[] = {0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f, 0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    switch (k % 9) {
    case 0: return NAN;
    case 1: return -INFINITY;
    case 2: return INFINITY;
    case 3: return -0.0f;
    case 4: return 0x1p-140f;                              /* subnormal */
    case 5: return -grid[splitmix(s) % 14];
    case 6: return 3.0e38f;
    case 7: return grid[splitmix(s) % 14] * 0x1p-20f;
    default: return gaussish(s) * 1.0e-4f;
    }
}

/* kind 0: finite gaussian; 1: gaussian with specials sprinkled in; 2: tiny */
static void fill(float* v, int64_t n, int kind, uint64_t seed) {
    uint64_t s = seed;
    for (int64_t i = 0; i < n; ++i) {
        float x = gaussish(&s);
        if (kind == 1 && splitmix(&s) % 7 == 0) x = special((int)(splitmix(&s) % 1000), &s);
        if (kind == 2) x *= 1.0e-4f;
        v[i] = x;
    }
}

/* the same values in the element type dt (bf16 / fp16 as bit patterns) */
static void* typed(const float* v, int64_t n, int dt) {
    if (dt == 0) {
        float* o = (float*)malloc((size_t)n * 4);
        memcpy(o, v, (size_t)n * 4);
        return o;
    }
    uint16_t* o = (uint16_t*)malloc((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i) o[i] = dt == 1 ? oracle_bf16_from_f32(v[i]) : oracle_f16_from_f32(v[i]);
    return o;
}

static size_t esize(int dt) { return dt == 0 ? 4 : 2; }

static void scalar_functions(void) {
    uint32_t acc[8] = {0};
    for (int c = 0; c < 256; ++c) {
        double a = oracle_e4m3_decode(c), b = oracle_e8m0_decode(c), u = oracle_ue5m3_decode(c);
        acc[0] = acc[0] * 31u + (uint32_t)oracle_e4m3_encode((float)a);
        acc[1] = acc[1] * 31u + (uint32_t)oracle_ue5m3_encode((float)u);
        acc[2] = acc[2] * 31u + (uint32_t)(isnan(b) ? 7 : (int)(b > 1.0));
    }
    for (int k = 0; k < 8; ++k) acc[3] = acc[3] * 31u + (uint32_t)(oracle_e2m1_value(k) * 2.0);
    uint64_t s = 42;
    for (int i = 0; i < 20000; ++i) {
        float f = i % 3 == 0 ? special(i, &s) : gaussish(&s) * 10.0f;
        uint16_t hb = oracle_bf16_from_f32(f), hf = oracle_f16_from_f32(f);
        float rb = oracle_bf16_to_f32(hb), rf = oracle_f16_to_f32(hf);
        uint32_t bb, bf;
        memcpy(&bb, &rb, 4);
        memcpy(&bf, &rf, 4);
        acc[4] = acc[4] * 31u + hb + bb;
        acc[5] = acc[5] * 31u + hf + bf;
        acc[6] = acc[6] * 31u + (uint32_t)oracle_e2m1_mag(fabsf(f)) + (uint32_t)oracle_e4m3_encode(fabsf(f)) +
                 (uint32_t)oracle_ue5m3_encode(fabsf(f)) + (uint32_t)oracle_e8m0_absmax_code(fabsf(f));
    }
    for (int n = 1; n <= 32; n <<= 1) {
        float v[32];
        fill(v, n, 0, (uint64_t)n);
        if (n >= 2) oracle_fwht(v, n);
        float t = oracle_tree_sum(v, n), c = oracle_hadamard_coef(n), e = oracle_block_sse(v, n, 0.5f);
        uint32_t bt, bc, be;
        memcpy(&bt, &t, 4);
        memcpy(&bc, &c, 4);
        memcpy(&be, &e, 4);
        acc[7] = acc[7] * 31u + bt + bc + be;
    }
    emit("scalars", 0, 0, 0, 0, 0, 0, acc, sizeof acc);
}

int main(void) {
    scalar_functions();
    const int64_t rows = 3, cols = 64, ld = 72;     /* row stride beyond cols */
    const int64_t n = rows * ld;
    float* v = (float*)malloc((size_t)n * 4);
    const int blocks[4] = {4, 8, 16, 32};
    const int hs[3] = {0, 16, 32};

    for (int kind = 0; kind < 3; ++kind) {
        fill(v, n, kind, 1000u + (uint64_t)kind);
        for (int dt = 0; dt < 3; ++dt) {
            void* x = typed(v, n, dt);
            for (int H = 0; H < 3; ++H) {
                const float tg = oracle_tensor_global_scale(x, dt, rows, cols, ld, hs[H]);
                emit("tensor_g", kind, dt, hs[H], 0, 0, 0, &tg, 4);
            }
            for (int fmt = 0; fmt < 3; ++fmt)
                for (int bi = 0; bi < 4; ++bi)
                    for (int st = 0; st < 5; ++st)
                        for (int gm = 0; gm < 4; ++gm)
                            for (int hi = 0; hi < 3; ++hi) {
                                const int B = blocks[bi], H = hs[hi];
                                if (gm == 3 && (kind != 0 || dt != 0 || (st == 3 && B < 16))) continue;
                                const int64_t nb = cols / B;
                                const int dq_dt = (fmt + bi + st) % 3;
                                uint8_t* codes = (uint8_t*)calloc((size_t)(rows * cols / 2), 1);
                                uint8_t* scales = (uint8_t*)calloc((size_t)(rows * nb), 1);
                                void* dq = calloc((size_t)(rows * ld), esize(dq_dt));
                                float* mse = (float*)calloc((size_t)(rows * nb), 4);
                                float* sse = (float*)calloc((size_t)(rows * nb), 4);
                                float g = 0.0f;
                                if (st == 4) {        /* GIVEN: scales of every code value, NaN code included */
                                    for (int64_t i = 0; i < rows * nb; ++i) scales[i] = (uint8_t)(i * 37 + 3);
                                }
                                const float user_g = fmt == 2 ? 0.25f : 0.0078125f;
                                const int rc = oracle_quantize(fmt, B, st, gm, user_g, H, x, dt, rows, cols, ld,
                                                               codes, scales, &g, dq, dq_dt, ld, mse, sse);
                                printf("quant %d %d %d %d %d %d %d rc=%d\n", kind, dt, fmt, B, st, gm, H, rc);
                                if (rc == 0) {
                                    emit("codes", kind, dt, fmt, B, st, gm * 100 + H, codes, (size_t)(rows * cols / 2));
                                    emit("scales", kind, dt, fmt, B, st, gm * 100 + H, scales, (size_t)(rows * nb));
                                    emit("g", kind, dt, fmt, B, st, gm * 100 + H, &g, 4);
                                    emit("dq", kind, dt, fmt, B, st, gm * 100 + H, dq, (size_t)(rows * ld) * esize(dq_dt));
                                    emit("mse", kind, dt, fmt, B, st, gm * 100 + H, mse, (size_t)(rows * nb) * 4);
                                    emit("sse", kind, dt, fmt, B, st, gm * 100 + H, sse, (size_t)(rows * nb) * 4);
                                    /* decode and re-score what was written */
                                    const float gd = fmt == 0 ? 1.0f : g;
                                    void* out = calloc((size_t)(rows * ld), esize(dq_dt));
                                    oracle_dequantize(fmt, B, codes, scales, gd, rows, cols, out, dq_dt, ld);
                                    emit("dequant", kind, dt, fmt, B, st, gm * 100 + H, out,
                                         (size_t)(rows * ld) * esize(dq_dt));
                                    float* m2 = (float*)calloc((size_t)(rows * nb), 4);
                                    oracle_block_mse(fmt, B, H, x, dt, rows, cols, ld, codes, scales, gd, m2);
                                    emit("block_mse", kind, dt, fmt, B, st, gm * 100 + H, m2, (size_t)(rows * nb) * 4);
                                    uint64_t counts[16] = {0};
                                    oracle_code_histogram(codes, rows, cols, counts);
                                    emit("hist", kind, dt, fmt, B, st, gm * 100 + H, counts, sizeof counts);
                                    free(out);
                                    free(m2);
                                }
                                free(codes);
                                free(scales);
                                free(dq);
                                free(mse);
                                free(sse);
                            }
            /* per-tensor search on its own, with its candidate totals */
            for (int st = 0; st < 4; ++st) {
                if (st == 3 && kind != 0) continue;
                double totals[32];
                memset(totals, 0, sizeof totals);
                const float gs = oracle_global_scale_search(st, 16, 0, x, dt, rows, cols, ld, totals);
                emit("search", kind, dt, st, 0, 0, 0, totals, sizeof totals);
                emit("search_g", kind, dt, st, 0, 0, 0, &gs, 4);
            }
            /* FOCUS relaxed forward / backward on scales picked by abs-max */
            for (int fmt = 0; fmt < 2; ++fmt)
                for (int bi = 1; bi < 4; ++bi)
                    for (int K = 4; K <= blocks[bi]; K <<= 1) {
                        const int B = blocks[bi];
                        const int64_t nb = cols / B, nk = cols / K;
                        uint8_t* scales = (uint8_t*)calloc((size_t)(rows * nb), 1);
                        uint8_t* codes = (uint8_t*)calloc((size_t)(rows * cols / 2), 1);
                        float g = 1.0f;
                        oracle_quantize(fmt, B, 0, fmt == 1 ? 1 : 0, 1.0f, 0, x, dt, rows, cols, ld, codes, scales,
                                        &g, NULL, 0, cols, NULL, NULL);
                        uint16_t* c16 = (uint16_t*)malloc((size_t)(rows * nk) * 2);
                        uint64_t s = 77;
                        for (int64_t i = 0; i < rows * nk; ++i)
                            c16[i] = oracle_f16_from_f32(0.8f + 0.45f * uniform(&s));
                        if (kind == 1) c16[0] = 0;                       /* S_q == 0 */
                        const int out_dt = (B + K) % 3;
                        void* wh = calloc((size_t)(rows * ld), esize(out_dt));
                        uint8_t* fc = (uint8_t*)calloc((size_t)(rows * cols / 2), 1);
                        const float gf = fmt == 0 ? 1.0f : g;
                        const int rf = oracle_relaxed_fwd(fmt, B, x, dt, rows, cols, ld, scales, gf, c16, K, wh,
                                                          out_dt, ld, fc);
                        emit("focus_fwd", kind, dt, fmt, B, K, rf, wh, (size_t)(rows * ld) * esize(out_dt));
                        emit("focus_codes", kind, dt, fmt, B, K, rf, fc, (size_t)(rows * cols / 2));
                        float* gv = (float*)malloc((size_t)n * 4);
                        fill(gv, n, 0, 555u + (uint64_t)K);
                        void* gt = typed(gv, n, (dt + 1) % 3);
                        float* gc = (float*)calloc((size_t)(rows * nk), 4);
                        const int rb = oracle_relaxed_bwd(fmt, B, x, dt, rows, cols, ld, scales, gf, c16, K, gt,
                                                          (dt + 1) % 3, ld, gc);
                        emit("focus_bwd", kind, dt, fmt, B, K, rb, gc, (size_t)(rows * nk) * 4);
                        free(scales);
                        free(codes);
                        free(c16);
                        free(wh);
                        free(fc);
                        free(gv);
                        free(gt);
                        free(gc);
                    }
            free(x);
        }
    }

    /* MXFP4 GEMM: K = 64 and 96 */
    for (int64_t K = 64; K <= 96; K += 32) {
        const int64_t M = 3, N = 5;
        float* a = (float*)malloc((size_t)(M * K) * 4);
        float* b = (float*)malloc((size_t)(N * K) * 4);
        fill(a, M * K, 1, 9u);
        fill(b, N * K, 0, 10u);
        uint8_t *ac = (uint8_t*)calloc((size_t)(M * K / 2), 1), *as = (uint8_t*)calloc((size_t)(M * K / 32), 1);
        uint8_t *bc = (uint8_t*)calloc((size_t)(N * K / 2), 1), *bs = (uint8_t*)calloc((size_t)(N * K / 32), 1);
        oracle_quantize(0, 32, 0, 0, 1.0f, 0, a, 0, M, K, K, ac, as, NULL, NULL, 0, K, NULL, NULL);
        oracle_quantize(0, 32, 0, 0, 1.0f, 0, b, 0, N, K, K, bc, bs, NULL, NULL, 0, K, NULL, NULL);
        double c[15];
        const int rg = oracle_mxfp4_gemm(ac, as, bc, bs, M, N, K, c);
        emit("gemm", (int)K, rg, 0, 0, 0, 0, c, sizeof c);
        free(a);
        free(b);
        free(ac);
        free(as);
        free(bc);
        free(bs);
    }
    free(v);
    return 0;
}
