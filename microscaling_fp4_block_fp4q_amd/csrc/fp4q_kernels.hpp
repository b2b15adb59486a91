// fp4q_kernels.hpp -- gfx950 kernels of the block-scaled FP4 path and the
// host launchers that pick their template instantiation.
//
// Work mapping: one lane owns one "unit" -- U contiguous values of a row,
// U = max(block, rotation size, 16 bytes of input) -- so a block, its
// rotation segment and its squared-error tree live in that lane's registers
// and no cross-lane traffic is needed.  A 256-thread workgroup walks the
// units grid-stride; lanes of a wave own neighbouring units, so a wave
// covers one contiguous stretch of the tensor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.hpp"

namespace fp4q_dev {

constexpr int kThreads = 256;
constexpr int kAmaxBlocks = 1024;   // partial abs-max results of the pre-pass

template <int... Is> struct ISeq {};
template <int N, int... Is> struct MakeISeq : MakeISeq<N - 1, N - 1, Is...> {};
template <int... Is> struct MakeISeq<0, Is...> { using type = ISeq<Is...>; };
template <int I> struct IC { static constexpr int value = I; };
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, ISeq<Is...>) { (f(IC<Is>{}), ...); }
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl(f, typename MakeISeq<N>::type{}); }

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <class InT, int B, int H>
constexpr int unit_elems() { return cmax(cmax(B, H), 16 / ElemSize<InT>::value); }

// ---------------------------------------------------------------------------
// Argument blocks (plain data, passed by value)
// ---------------------------------------------------------------------------

struct QuantArgs {
    const void* x;
    int64_t ld_x;
    int64_t cols;
    int64_t units;          // rows * cols / U
    int64_t units_per_row;  // cols / U
    int contiguous;         // ld_x == cols and (no dequant or ld_dq == cols)
    uint8_t* codes;         // [rows, cols/2] or null
    uint8_t* scales;        // [rows, cols/B]: output, or input for GIVEN
    float* g_out;           // or null
    void* dq;               // or null
    int64_t ld_dq;
    int dq_dt;
    float* mse;             // [rows, cols/B] or null
    float* sse;             // [rows, cols/B] or null
    const uint32_t* amax_partials;
    int n_partials;
    int global_mode;
    float user_g;
    int prevent_zero;
};

struct AmaxArgs {
    const void* x;
    int64_t ld_x;
    int64_t units;
    int64_t units_per_row;
    int contiguous;
    uint32_t* partials;     // [gridDim.x]
};

struct DequantArgs {
    const uint8_t* codes;
    const uint8_t* scales;
    const float* g_dev;     // or null (g = 1)
    int scale_fmt;
    int64_t cols;
    int64_t units;
    int64_t units_per_row;
    void* out;
    int64_t ld_out;
    int out_dt;
};

struct MseArgs {
    const void* x;
    int64_t ld_x;
    int64_t cols;
    int64_t units;
    int64_t units_per_row;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* g_dev;
    int scale_fmt;
    float* mse;
};

struct RelaxedArgs {
    const void* w;
    int64_t ld_w;
    int64_t cols;
    int64_t units;
    int64_t units_per_row;
    const uint8_t* scales;
    const float* g_dev;
    int scale_fmt;
    const uint16_t* c;      // [rows, cols/K] fp16 bits
    void* w_hat;            // fwd output
    int64_t ld_out;
    int out_dt;
    uint8_t* codes;         // fwd, or null
    const void* grad;       // bwd input
    int64_t ld_g;
    int g_dt;
    float* grad_c;          // bwd output [rows, cols/K]
};

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

__device__ __forceinline__ uint32_t workgroup_max_u32(uint32_t v) {
    __shared__ uint32_t s_part[kThreads / 64];
    v = wave_max_u32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s_part[wave] = v;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) m = max(m, s_part[i]);
    __syncthreads();
    return m;
}

// A scale usable for encoding: a number, finite, not negative.
__device__ __forceinline__ bool scale_usable(float S) { return S >= 0.0f && S < __builtin_inff(); }

// (-1)^sign(of s) |v|
__device__ __forceinline__ float with_sign_of(float v, float s) {
    return as_f((as_u(v) & 0x7FFFFFFFu) | (as_u(s) & 0x80000000u));
}

__device__ __forceinline__ float canonical_nan_like(float s) { return as_f(kQNaN | (as_u(s) & 0x80000000u)); }

// Per-tensor scale g of hierarchical scaling ("Finer is Better (with the
// Right Scaling)", method part 2): NONE -> 1, USER -> given, TENSOR_AMAX ->
// fl(amax / (6 * 448)), 1 when that is 0, NaN when amax is not finite.
// Every thread of the workgroup must call it.
__device__ __forceinline__ float workgroup_global_scale(const QuantArgs& p) {
    if (p.global_mode == GM_NONE) return 1.0f;
    if (p.global_mode == GM_USER) return p.user_g;
    uint32_t m = 0;
    for (int i = threadIdx.x; i < p.n_partials; i += kThreads) m = max(m, p.amax_partials[i]);
    m = workgroup_max_u32(m);
    if (m >= 0x7F800000u) return as_f(kQNaN);
    float g = as_f(m) / 2688.0f;
    return g == 0.0f ? 1.0f : g;
}

__device__ __forceinline__ float read_g(const float* g_dev) { return g_dev ? *g_dev : 1.0f; }

// Element offset of unit u in a [rows, ld] tensor whose rows hold upr units.
template <int U>
__device__ __forceinline__ int64_t unit_offset(int64_t u, int64_t upr, int64_t ld, bool contiguous) {
    if (contiguous) return u * U;
    int64_t row = u / upr;
    return row * ld + (u - row * upr) * U;
}

// ---------------------------------------------------------------------------
// Encoding of one block at one scale
// ---------------------------------------------------------------------------

// Quantize y[OFF, OFF+B) at scale S (usable; invS = 1/S exactly for E8M0):
// r[i] receives the E2M1 grid value of |y_i| / S; returns the block SSE.
// For a power-of-two E8M0 scale, |y| * 2^-k is exactly the IEEE quotient
// fl(|y| / 2^k); E4M3 scales use the correctly rounded division.
// NAN_GUARD: elements may be NaN (caller-given scales), which encode as 0.
template <int SF, int B, int OFF, bool NAN_GUARD, int U>
__device__ __forceinline__ float encode_block(const float (&y)[U], float S, float invS, float (&r)[B]) {
    float e[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
        const float a = fabsf(y[OFF + i]);
        float u;
        if constexpr (SF == SF_E8M0) u = a * invS;
        else u = (S > 0.0f) ? a / S : 0.0f;
        float rr = e2m1_round(u);
        if constexpr (NAN_GUARD) rr = (a == a) ? rr : 0.0f;
        r[i] = rr;
        const float d = a - rr * S;       // |y| - fl(grid * S): same magnitude as y - yhat
        e[i] = d * d;
    }
    return tree_sum<B>(e);
}

// Scale selection + encoding of block number BI of a unit.
template <int SF, int ST, int B, int BI, int U>
__device__ __forceinline__ void quant_block(const float (&y)[U], float g, float six_g, float four_g,
                                            int prevent_zero, uint32_t given, uint32_t (&code)[U],
                                            float (&dq)[U], uint32_t& scale_code, float& sse) {
    constexpr int OFF = BI * B;
    uint32_t sc;
    bool nan_block;
    float S = 0.0f, invS = 0.0f;
    float r[B];

    if constexpr (ST == ST_GIVEN) {
        if constexpr (SF == SF_E8M0) {
            sc = given & 0xFFu;
            nan_block = sc == kE8M0NaN;
            S = e8m0_value(sc);
            invS = e8m0_inverse(sc);
        } else {
            sc = given & 0x7Fu;
            S = e4m3_value(sc) * g;
            nan_block = sc == kE4M3NaN || !scale_usable(S);
        }
        if (!nan_block) sse = encode_block<SF, B, OFF, true>(y, S, invS, r);
    } else {
        uint32_t ab = 0;
#pragma unroll
        for (int i = 0; i < B; ++i) ab = max(ab, as_u(y[OFF + i]) & 0x7FFFFFFFu);
        const float a_b = as_f(ab);
        nan_block = ab >= 0x7F800000u || !(g < __builtin_inff());   // also catches NaN g
        if (!nan_block) {
            if constexpr (SF == SF_E8M0) {
                if constexpr (ST == ST_BRUTE_FORCE) {
                    float best = __builtin_inff();
                    uint32_t bc = 0;
#pragma unroll 1
                    for (uint32_t c = 0; c <= 254u; ++c) {
                        float rc[B];
                        float s = encode_block<SF, B, OFF, false>(y, e8m0_value(c), e8m0_inverse(c), rc);
                        if (s < best) { best = s; bc = c; }
                    }
                    sc = bc;
                } else {
                    sc = e8m0_absmax_code(ab);
                }
                S = e8m0_value(sc);
                invS = e8m0_inverse(sc);
                sse = encode_block<SF, B, OFF, false>(y, S, invS, r);
            } else {
                const uint32_t s6 = e4m3_encode(a_b / six_g);
                if constexpr (ST == ST_ABSMAX) {
                    sc = (prevent_zero && s6 == 0u) ? 1u : s6;
                    S = e4m3_value(sc) * g;
                    sse = encode_block<SF, B, OFF, false>(y, S, 0.0f, r);
                } else if constexpr (ST == ST_FOUR_OVER_SIX) {
                    const uint32_t s4 = e4m3_encode(a_b / four_g);
                    const float S6 = e4m3_value(s6) * g, S4 = e4m3_value(s4) * g;
                    float r4[B];
                    const float e6 = encode_block<SF, B, OFF, false>(y, S6, 0.0f, r);
                    const float e4 = encode_block<SF, B, OFF, false>(y, S4, 0.0f, r4);
                    const bool take4 = e4 < e6;   // equal error keeps the smaller code s6
                    sc = take4 ? s4 : s6;
                    S = take4 ? S4 : S6;
                    sse = take4 ? e4 : e6;
#pragma unroll
                    for (int i = 0; i < B; ++i) r[i] = take4 ? r4[i] : r[i];
                } else {   // brute force over the 126 positive finite E4M3 scales
                    float best = __builtin_inff();
                    uint32_t bc = 1;
#pragma unroll 1
                    for (uint32_t c = 1; c <= 0x7Eu; ++c) {
                        float rc[B];
                        float s = encode_block<SF, B, OFF, false>(y, e4m3_value(c) * g, 0.0f, rc);
                        if (s < best) { best = s; bc = c; }
                    }
                    sc = bc;
                    S = e4m3_value(sc) * g;
                    sse = encode_block<SF, B, OFF, false>(y, S, 0.0f, r);
                }
            }
        } else {
            sc = SF == SF_E8M0 ? kE8M0NaN : kE4M3NaN;
        }
    }

    scale_code = sc;
    if (nan_block) {
        sse = as_f(kQNaN);
#pragma unroll
        for (int i = 0; i < B; ++i) {
            code[OFF + i] = (as_u(y[OFF + i]) >> 31) << 3;
            dq[OFF + i] = canonical_nan_like(y[OFF + i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < B; ++i) {
            code[OFF + i] = ((as_u(y[OFF + i]) >> 31) << 3) | e2m1_code_of(r[i]);
            dq[OFF + i] = with_sign_of(r[i] * S, y[OFF + i]);
        }
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// Partial per-tensor abs-max (of the rotated values when H != 0) for
// hierarchical scaling.  One result per workgroup in p.partials.
template <class InT, int H>
__global__ __launch_bounds__(kThreads) void k_amax(AmaxArgs p) {
    constexpr int U = unit_elems<InT, 1, H>();
    constexpr int UNROLL = 4;
    const InT* x = reinterpret_cast<const InT*>(p.x);
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t u0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; u0 < p.units; u0 += stride * UNROLL) {
        float y[UNROLL][U];
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
            const int64_t u = u0 + k * stride;
            if (u < p.units) {
                load_elems<InT, U>(x + unit_offset<U>(u, p.units_per_row, p.ld_x, p.contiguous), y[k]);
            } else {
#pragma unroll
                for (int i = 0; i < U; ++i) y[k][i] = 0.0f;
            }
        }
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
            if constexpr (H > 0) fwht_segments<H, U>(y[k]);
#pragma unroll
            for (int i = 0; i < U; ++i) m = max(m, as_u(y[k][i]) & 0x7FFFFFFFu);
        }
    }
    m = workgroup_max_u32(m);
    if (threadIdx.x == 0) p.partials[blockIdx.x] = m;
}

// Quantize: scale selection, encode, pack, dequantize, block error.
template <class InT, int B, int H, int SF, int ST>
__global__ __launch_bounds__(kThreads) void k_quant(QuantArgs p) {
    constexpr int U = unit_elems<InT, B, H>();
    constexpr int NB = U / B;
    const InT* x = reinterpret_cast<const InT*>(p.x);

    const float g = workgroup_global_scale(p);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.g_out) *p.g_out = g;
    const float six_g = 6.0f * g, four_g = 4.0f * g;

    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < p.units; u += stride) {
        const int64_t xo = unit_offset<U>(u, p.units_per_row, p.ld_x, p.contiguous);
        float y[U];
        load_elems<InT, U>(x + xo, y);
        if constexpr (H > 0) fwht_segments<H, U>(y);

        uint32_t given[NB];
        if constexpr (ST == ST_GIVEN) {
#pragma unroll
            for (int b = 0; b < NB; ++b) given[b] = p.scales[u * NB + b];
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) given[b] = 0;
        }

        uint32_t code[U];
        float dq[U];
        uint32_t sc[NB];
        float sse[NB];
        static_for<NB>([&](auto bi) {
            constexpr int b = decltype(bi)::value;
            quant_block<SF, ST, B, b>(y, g, six_g, four_g, p.prevent_zero, given[b], code, dq, sc[b], sse[b]);
        });

        if (p.codes) store_codes<U>(p.codes + u * (U / 2), code);
        if constexpr (ST != ST_GIVEN) {
#pragma unroll
            for (int b = 0; b < NB; ++b) p.scales[u * NB + b] = (uint8_t)sc[b];
        }
        if (p.dq) {
            const int64_t dqo = unit_offset<U>(u, p.units_per_row, p.ld_dq, p.contiguous);
            store_elems_rt<U>(p.dq, p.dq_dt, dqo, dq);
        }
        if (p.sse) {
#pragma unroll
            for (int b = 0; b < NB; ++b) p.sse[u * NB + b] = sse[b];
        }
        if (p.mse) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float m = sse[b] * (1.0f / (float)B);   // exact: B is a power of two
                p.mse[u * NB + b] = (m == m) ? m : as_f(kQNaN);
            }
        }
    }
}

// Dequantize codes + scales.
template <int B>
__global__ __launch_bounds__(kThreads) void k_dequant(DequantArgs p) {
    constexpr int U = cmax(B, 4);
    constexpr int NB = U / B;
    const float g = read_g(p.g_dev);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < p.units; u += stride) {
        uint32_t c[U];
        load_codes<U>(p.codes + u * (U / 2), c);
        float v[U];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t code = p.scales[u * NB + b];
            float S;
            bool nan_block;
            if (p.scale_fmt == SF_E8M0) {
                nan_block = code == kE8M0NaN;
                S = e8m0_value(code);
            } else {
                const uint32_t c7 = code & 0x7Fu;
                S = e4m3_value(c7) * g;
                nan_block = c7 == kE4M3NaN || !scale_usable(S);
            }
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const uint32_t q = c[b * B + i];
                const float sgn = as_f((q & 8u) << 28);
                v[b * B + i] = nan_block ? canonical_nan_like(sgn) : with_sign_of(e2m1_value(q) * S, sgn);
            }
        }
        store_elems_rt<U>(p.out, p.out_dt, unit_offset<U>(u, p.units_per_row, p.ld_out, false), v);
    }
}

// Per-block MSE of (rotated) x against stored codes + scales.
template <class InT, int B, int H>
__global__ __launch_bounds__(kThreads) void k_block_mse(MseArgs p) {
    constexpr int U = unit_elems<InT, B, H>();
    constexpr int NB = U / B;
    const InT* x = reinterpret_cast<const InT*>(p.x);
    const float g = read_g(p.g_dev);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < p.units; u += stride) {
        float y[U];
        load_elems<InT, U>(x + unit_offset<U>(u, p.units_per_row, p.ld_x, false), y);
        if constexpr (H > 0) fwht_segments<H, U>(y);
        uint32_t c[U];
        load_codes<U>(p.codes + u * (U / 2), c);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t code = p.scales[u * NB + b];
            float S;
            bool nan_block;
            if (p.scale_fmt == SF_E8M0) {
                nan_block = code == kE8M0NaN;
                S = e8m0_value(code);
            } else {
                const uint32_t c7 = code & 0x7Fu;
                S = e4m3_value(c7) * g;
                nan_block = c7 == kE4M3NaN || !scale_usable(S);
            }
            float e[B];
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const uint32_t q = c[b * B + i];
                const float yh = with_sign_of(e2m1_value(q) * S, as_f((q & 8u) << 28));
                const float d = y[b * B + i] - yh;
                e[i] = d * d;
            }
            const float m = tree_sum<B>(e) * (1.0f / (float)B);
            p.mse[u * NB + b] = (nan_block || m != m) ? as_f(kQNaN) : m;
        }
    }
}

// Scale of block `code` for the FOCUS kernels.
__device__ __forceinline__ float stored_scale(int fmt, uint32_t code, float g, bool& usable) {
    if (fmt == SF_E8M0) {
        usable = code != kE8M0NaN;
        return e8m0_value(code);
    }
    const uint32_t c7 = code & 0x7Fu;
    const float S = e4m3_value(c7) * g;
    usable = c7 != kE4M3NaN && scale_usable(S);
    return S;
}

__device__ __forceinline__ float f16_value(uint16_t h) { return f16_bits_to_f32(h); }

// FOCUS relaxed fake-quant forward (FOCUS page, methods 2-3):
// S_q = fl(S_dq c_k), u = fl(|W| / S_q), What = (-1)^s fl(grid * S_dq).
template <class InT, int B, int K>
__global__ __launch_bounds__(kThreads) void k_relaxed_fwd(RelaxedArgs p) {
    constexpr int U = unit_elems<InT, B, 0>();
    constexpr int NB = U / B;
    const InT* w = reinterpret_cast<const InT*>(p.w);
    const float g = read_g(p.g_dev);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t nk = p.cols / K;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < p.units; u += stride) {
        const int64_t row = u / p.units_per_row;
        const int64_t col0 = (u - row * p.units_per_row) * U;
        float y[U];
        load_elems<InT, U>(w + row * p.ld_w + col0, y);
        uint32_t code[U];
        float wh[U];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            bool ok_dq;
            const float S_dq = stored_scale(p.scale_fmt, p.scales[u * NB + b], g, ok_dq);
#pragma unroll
            for (int k = 0; k < B / K; ++k) {
                const float c_k = f16_value(p.c[row * nk + (col0 + b * B) / K + k]);
                const float S_q = S_dq * c_k;
                const bool ok = ok_dq && scale_usable(S_q);
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    const int j = b * B + k * K + i;
                    const float a = fabsf(y[j]);
                    const float u_ = (S_q > 0.0f) ? a / S_q : 0.0f;
                    float rr = e2m1_round(u_);
                    rr = (a == a) ? rr : 0.0f;
                    const uint32_t s = (as_u(y[j]) >> 31) << 3;
                    code[j] = ok ? (s | e2m1_code_of(rr)) : s;
                    wh[j] = ok ? with_sign_of(rr * S_dq, y[j]) : canonical_nan_like(y[j]);
                }
            }
        }
        store_elems_rt<U>(p.w_hat, p.out_dt, row * p.ld_out + col0, wh);
        if (p.codes) store_codes<U>(p.codes + u * (U / 2), code);
    }
}

// Straight-through backward to c_k (FOCUS page, method 1):
// grad_c = fl(-A / fl(c c)), A = tree sum of [S_q > 0, |u| <= 6] fl(G W).
template <class InT, int B, int K>
__global__ __launch_bounds__(kThreads) void k_relaxed_bwd(RelaxedArgs p) {
    constexpr int U = unit_elems<InT, B, 0>();
    constexpr int NB = U / B;
    const InT* w = reinterpret_cast<const InT*>(p.w);
    const float g = read_g(p.g_dev);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t nk = p.cols / K;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < p.units; u += stride) {
        const int64_t row = u / p.units_per_row;
        const int64_t col0 = (u - row * p.units_per_row) * U;
        float y[U], G[U];
        load_elems<InT, U>(w + row * p.ld_w + col0, y);
        load_elems_rt<U>(p.grad, p.g_dt, row * p.ld_g + col0, G);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            bool ok_dq;
            const float S_dq = stored_scale(p.scale_fmt, p.scales[u * NB + b], g, ok_dq);
#pragma unroll
            for (int k = 0; k < B / K; ++k) {
                const int64_t ci = row * nk + (col0 + b * B) / K + k;
                const float c_k = f16_value(p.c[ci]);
                const float S_q = S_dq * c_k;
                const bool ok = ok_dq && scale_usable(S_q);
                float t[K];
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    const int j = b * B + k * K + i;
                    bool inside = false;
                    if (S_q > 0.0f) inside = fabsf(y[j]) / S_q <= 6.0f;
                    t[i] = inside ? G[j] * y[j] : 0.0f;
                }
                const float A = tree_sum<K>(t);
                const float out = -A / (c_k * c_k);
                p.grad_c[ci] = (ok && out == out) ? out : as_f(kQNaN);
            }
        }
    }
}

}  // namespace fp4q_dev
