// fp4q_device.hpp -- device building blocks of the gfx950 FP4 quantizer.
//
// Arithmetic contract (shared with nothing: the CPU oracle is a separate
// implementation of the same definitions):
//  * every float operation is one IEEE binary32 operation rounded to
//    nearest-even (hipcc -ffp-contract=off, correctly rounded division,
//    fp32 denormals kept);
//  * E2M1 elements, OCP E4M3 / E8M0 block scales ("Finer is Better (with
//    the Right Scaling)", method part 1; MR-GPTQ page, technical summary
//    section 1);
//  * u = fl(y / S), rounded half-to-even onto {0, .5, 1, 1.5, 2, 3, 4, 6}
//    with saturation; dequantized value (-1)^s fl(grid * S); block error
//    = balanced-tree fp32 sum of fl(d * d), d = fl(y - yhat).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q_dev {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
enum : int { SF_E8M0 = 0, SF_E4M3 = 1, SF_UE5M3 = 2 };
enum : int { ST_ABSMAX = 0, ST_PREVENT_ZERO = 1, ST_FOUR_OVER_SIX = 2, ST_BRUTE_FORCE = 3, ST_GIVEN = 4 };
// Per-tensor scale modes of the kernels; GM_DEVICE reads g from device
// memory (the searched scale).
enum : int { GM_NONE = 0, GM_TENSOR_AMAX = 1, GM_USER = 2, GM_DEVICE = 3 };

constexpr uint32_t kQNaN = 0x7FC00000u;
constexpr uint32_t kE4M3NaN = 0x7Fu;
constexpr uint32_t kE8M0NaN = 0xFFu;
constexpr uint32_t kUE5M3NaN = 0xFFu;

__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }

// ---------------------------------------------------------------------------
// E2M1 rounding
// ---------------------------------------------------------------------------

// Round u >= 0 (may be +inf, must not be NaN) half-to-even onto the E2M1
// magnitudes, saturating at 6; returns the grid value itself as fp32.
//
// Within a binade of u the E2M1 grid spacing is 2^k with
// k = clamp(floor(log2 u) - 1, -1, 2) (0.5 below 2, then 1, then 2).
// Adding C = 1.5 * 2^(23+k) puts u + C in C's binade, whose ulp is 2^k, so
// the fp32 addition rounds u half-to-even to a multiple of 2^k ("even" =
// multiple of 2^(k+1), exactly the E2M1 tie rule); subtracting C is exact.
// Anything from 8 up (k clamped at 2) lands on >= 8 and the final min
// saturates it to 6, as does +inf.  Six VALU operations, no division.
__device__ __forceinline__ float e2m1_round(float u) {
    uint32_t be = as_u(u) >> 23;                         // biased exponent of u
    uint32_t ce = min(max(be + 22u, 149u), 152u);        // biased exponent of C
    float C = as_f((ce << 23) | 0x00400000u);
    float t = u + C;
    float r = t - C;
    return fminf(r, 6.0f);
}

// Magnitude code 0..7 of a grid value r (0, .5, 1, 1.5, 2, 3, 4, 6):
// r >= 1 has bits >> 22 = 252 + code; 0.5 is 252, 0 is 0.
__device__ __forceinline__ uint32_t e2m1_code_of(float r) {
    uint32_t h = as_u(r) >> 22;
    return h >= 254u ? h - 252u : (h == 252u ? 1u : 0u);
}

// Grid value of a magnitude code.
__device__ __forceinline__ float e2m1_value(uint32_t mag) {
    mag &= 7u;
    return mag >= 2u ? as_f((mag + 252u) << 22) : (mag == 1u ? 0.5f : 0.0f);
}

// ---------------------------------------------------------------------------
// Scale formats
// ---------------------------------------------------------------------------

// Unsigned OCP E4M3 value of code 0..0x7E: (1 + m/8) 2^(e-7), or m 2^-9 for e = 0.
__device__ __forceinline__ float e4m3_value(uint32_t code) {
    uint32_t e = code >> 3, m = code & 7u;
    return e ? as_f(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// Nearest E4M3 code of v >= 0 (may be +inf, not NaN), ties to the even
// code, satfinite at 448 (0x7E).  v * 2^(3-e) is an exact scaling that puts
// the three mantissa bits in front of the binary point (subnormals share
// e = -6), rint rounds half-to-even, and a carry into the next binade falls
// out of the code arithmetic.  Saturation is a minimum (448 itself encodes
// to 0x7E, and the minimum of a NaN and 448 is 448), so there is no branch.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    v = fminf(v, 448.0f);
    int e = max((int)(as_u(v) >> 23) - 127, -6);
    float q = __builtin_ldexpf(v, 3 - e);
    float r = __builtin_rintf(q);
    return (uint32_t)((e + 7) * 8 - 8) + (uint32_t)r;
}

// UE5M3, the unsigned wide-exponent scale of the Finer-is-Better page (key
// findings), read as 5 exponent bits with bias 15 and 3 mantissa bits:
// (1 + m/8) 2^(e-15), or m 2^-17 for e = 0; codes 0..0xFE, 0xFF is NaN.
__device__ __forceinline__ float ue5m3_value(uint32_t code) {
    uint32_t e = code >> 3, m = code & 7u;
    return e ? as_f(((e + 112u) << 23) | (m << 20)) : (float)m * 0x1p-17f;
}

// Nearest UE5M3 code of v >= 0 (may be +inf, not NaN), ties to the even
// code, saturating at 0xFE = 1.75 * 2^16; the same exact scaling and
// half-to-even rint as e4m3_encode, with subnormals sharing e = -14.
__device__ __forceinline__ uint32_t ue5m3_encode(float v) {
    v = fminf(v, 114688.0f);                       // saturation as in e4m3_encode
    int e = max((int)(as_u(v) >> 23) - 127, -14);
    float q = __builtin_ldexpf(v, 3 - e);
    float r = __builtin_rintf(q);
    return (uint32_t)((e + 15) * 8 - 8) + (uint32_t)r;
}

// The non-power-of-two scale formats (E4M3, UE5M3) behind one interface.
template <int SF>
__device__ __forceinline__ float scale_value(uint32_t code) {
    if constexpr (SF == SF_E4M3) return e4m3_value(code);
    else return ue5m3_value(code);
}
template <int SF>
__device__ __forceinline__ uint32_t scale_encode(float v) {
    if constexpr (SF == SF_E4M3) return e4m3_encode(v);
    else return ue5m3_encode(v);
}
template <int SF>
constexpr uint32_t scale_nan() { return SF == SF_E8M0 ? kE8M0NaN : (SF == SF_E4M3 ? kE4M3NaN : kUE5M3NaN); }
// Bits of a stored code that carry the scale (E4M3 scales are unsigned: bit 7 is ignored).
template <int SF>
constexpr uint32_t scale_code_mask() { return SF == SF_E4M3 ? 0x7Fu : 0xFFu; }
// Largest finite code.
template <int SF>
constexpr uint32_t scale_top() { return SF == SF_E4M3 ? 0x7Eu : 0xFEu; }

// E8M0 scale 2^(code-127) and its exact reciprocal 2^(127-code), code 0..254
// (2^-127 is the fp32 subnormal 0x00400000).
__device__ __forceinline__ float e8m0_value(uint32_t code) {
    return code ? as_f(code << 23) : as_f(0x00400000u);
}
__device__ __forceinline__ float e8m0_inverse(uint32_t code) {
    return code < 254u ? as_f((254u - code) << 23) : as_f(0x00400000u);
}

// MXFP4 abs-max scale: 2^(floor(log2 a_b) - 2), code = biased exponent - 2,
// clamped at 0 (zero, subnormal and a_b < 2^-124 give 0).  a_b finite.
__device__ __forceinline__ uint32_t e8m0_absmax_code(uint32_t ab_bits) {
    int c = (int)(ab_bits >> 23) - 2;
    return c > 0 ? (uint32_t)c : 0u;
}

// ---------------------------------------------------------------------------
// Element loads / stores.  bf16 and fp16 travel as 16-bit patterns.
// ---------------------------------------------------------------------------

struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

template <class T> struct ElemSize;
template <> struct ElemSize<float> { static constexpr int value = 4; };
template <> struct ElemSize<bf16_t> { static constexpr int value = 2; };
template <> struct ElemSize<f16_t> { static constexpr int value = 2; };

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Load N contiguous elements (N * size a multiple of 16 bytes, 16-byte aligned).
template <class T, int N>
__device__ __forceinline__ void load_elems(const T* __restrict__ p, float (&y)[N]) {
    if constexpr (ElemSize<T>::value == 4) {
        const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            float4 v = q[i];
            y[4 * i + 0] = v.x; y[4 * i + 1] = v.y; y[4 * i + 2] = v.z; y[4 * i + 3] = v.w;
        }
    } else {
        const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int i = 0; i < N / 8; ++i) {
            uint4 v = q[i];
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (sizeof(T) == 2 && __is_same(T, bf16_t)) {
                    y[8 * i + 2 * k] = as_f(w[k] << 16);
                    y[8 * i + 2 * k + 1] = as_f(w[k] & 0xFFFF0000u);
                } else {
                    y[8 * i + 2 * k] = f16_bits_to_f32(w[k] & 0xFFFFu);
                    y[8 * i + 2 * k + 1] = f16_bits_to_f32(w[k] >> 16);
                }
            }
        }
    }
}

// Runtime-typed load of N elements, N * size >= 16 bytes not required
// (used for the gradient operand whose dtype is a runtime argument).
template <int N>
__device__ __forceinline__ void load_elems_rt(const void* __restrict__ base, int dt, int64_t off,
                                              float (&y)[N]) {
    if (dt == DT_F32) {
        const float* p = reinterpret_cast<const float*>(base) + off;
        if constexpr (N % 4 == 0) {
            load_elems<float, N>(p, y);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) y[i] = p[i];
        }
    } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + off;
        if constexpr (N % 8 == 0) {
            if (dt == DT_BF16) load_elems<bf16_t, N>(reinterpret_cast<const bf16_t*>(p), y);
            else load_elems<f16_t, N>(reinterpret_cast<const f16_t*>(p), y);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i)
                y[i] = dt == DT_BF16 ? as_f((uint32_t)p[i] << 16) : f16_bits_to_f32(p[i]);
        }
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round two fp32 values half-to-even to bf16 / fp16 and pack them.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t v = {a, b};
    bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    f32x2_t v = {a, b};
    f16x2_t h = __builtin_convertvector(v, f16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// Streaming stores for the outputs that are written once, never read back
// by the kernel, and large next to its input: dequantized tensors (as large
// as the input) and per-block errors.  Non-temporal, so they do not evict
// the input tensors from L2 and the last-level cache.  Only for stores
// where a wave writes whole contiguous lines (partial-line non-temporal
// writes are slow).  Codes and scales, which the next operation
// (dequantize, GEMM) reads, are stored normally.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
    u32x4_t w;
    w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_stream(uint2* p, uint2 v) {
    u32x2_t w;
    w.x = v.x; w.y = v.y;
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void store_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }

// N consecutive fp32 values (N = 1, 2, 4 or 8; p aligned to 4 N bytes) as
// streaming stores, so that lanes writing neighbouring runs fill whole lines.
template <int N>
__device__ __forceinline__ void store_stream_f32(float* p, const float (&v)[N]) {
    if constexpr (N == 1) {
        store_stream(p, v[0]);
    } else if constexpr (N == 2) {
        store_stream(reinterpret_cast<uint2*>(p), make_uint2(as_u(v[0]), as_u(v[1])));
    } else {
        static_assert(N % 4 == 0, "runs of 1, 2 or a multiple of 4 values");
#pragma unroll
        for (int i = 0; i < N / 4; ++i)
            store_stream(reinterpret_cast<uint4*>(p) + i,
                         make_uint4(as_u(v[4 * i]), as_u(v[4 * i + 1]), as_u(v[4 * i + 2]), as_u(v[4 * i + 3])));
    }
}

// Store N fp32 values as dtype dt at base + off (elements); N * size is a
// multiple of 8 bytes and the address is aligned to that.
template <int N>
__device__ __forceinline__ void store_elems_rt(void* __restrict__ base, int dt, int64_t off,
                                               const float (&v)[N]) {
    if (dt == DT_F32) {
        float* p = reinterpret_cast<float*>(base) + off;
#pragma unroll
        for (int i = 0; i < N / 4; ++i)
            reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        if constexpr (N % 4 == 2)
            reinterpret_cast<float2*>(p)[N / 2 - 1] = make_float2(v[N - 2], v[N - 1]);
    } else {
        uint16_t* p = reinterpret_cast<uint16_t*>(base) + off;
        uint32_t w[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
            w[i] = dt == DT_BF16 ? pack_bf16x2(v[2 * i], v[2 * i + 1]) : pack_f16x2(v[2 * i], v[2 * i + 1]);
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int i = 0; i < N / 8; ++i)
                reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
        } else if constexpr (N % 4 == 0) {
#pragma unroll
            for (int i = 0; i < N / 4; ++i) reinterpret_cast<uint2*>(p)[i] = make_uint2(w[2 * i], w[2 * i + 1]);
        } else {
#pragma unroll
            for (int i = 0; i < N / 2; ++i) reinterpret_cast<uint32_t*>(p)[i] = w[i];
        }
    }
}

// Store N/2 packed code bytes (N nibbles, even element in the low nibble).
template <int N>
__device__ __forceinline__ void store_codes(uint8_t* __restrict__ p, const uint32_t (&c)[N]) {
    constexpr int NB = N / 2;
    uint32_t w[(NB + 3) / 4];
#pragma unroll
    for (int i = 0; i < (NB + 3) / 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) w[i / 8] |= (c[i] & 15u) << (4 * (i % 8));
    if constexpr (NB == 16) {
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (NB == 8) {
        *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else if constexpr (NB == 4) {
        *reinterpret_cast<uint32_t*>(p) = w[0];
    } else {
        static_assert(NB == 2, "unit of 4 elements");
        *reinterpret_cast<uint16_t*>(p) = (uint16_t)w[0];
    }
}

// Load N nibbles.
template <int N>
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ p, uint32_t (&c)[N]) {
    constexpr int NB = N / 2;
    uint32_t w[(NB + 3) / 4];
    if constexpr (NB == 16) {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (NB == 8) {
        uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x; w[1] = v.y;
    } else if constexpr (NB == 4) {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
        w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) c[i] = (w[i / 8] >> (4 * (i % 8))) & 15u;
}

// ---------------------------------------------------------------------------
// Reductions inside a lane
// ---------------------------------------------------------------------------

// Balanced binary tree sum in index order over v[OFF, OFF+N).
template <int N, int OFF = 0, class T, int M>
__device__ __forceinline__ T tree_sum(const T (&v)[M]) {
    if constexpr (N == 1) {
        return v[OFF];
    } else {
        T l = tree_sum<N / 2, OFF>(v);
        T r = tree_sum<N / 2, OFF + N / 2>(v);
        return l + r;
    }
}

// ---------------------------------------------------------------------------
// Block-wise normalised Walsh-Hadamard transform in registers (MR-GPTQ page,
// sections 2.1-2.3): Sylvester order, radix-2 butterflies with stride
// h = 1, 2, ..., H/2, then one multiplication by fl(1/sqrt(H)).  A NaN the
// transform produces leaves as the positive quiet NaN: IEEE 754 leaves the
// sign of an arithmetic NaN open (gfx950's subtraction flips it where x86's
// keeps it), and the sign of a NaN element reaches its code nibble.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float rotated_nan_canonical(float v) { return v == v ? v : as_f(kQNaN); }

template <int H>
__device__ __forceinline__ constexpr float hadamard_coef() {
    static_assert(H == 16 || H == 32, "rotation size");
    return H == 16 ? 0.25f : 0x1.6a09e6p-3f;   // fl(1/sqrt(32)) = 0x3E3504F3
}

template <int H, int U>
__device__ __forceinline__ void fwht_segments(float (&y)[U]) {
    static_assert(U % H == 0, "unit holds whole segments");
#pragma unroll
    for (int s = 0; s < U / H; ++s) {
#pragma unroll
        for (int h = 1; h < H; h <<= 1) {
#pragma unroll
            for (int i = 0; i < H; ++i) {
                if ((i & h) == 0) {
                    float a = y[s * H + i], b = y[s * H + i + h];
                    y[s * H + i] = a + b;
                    y[s * H + i + h] = a - b;
                }
            }
        }
    }
    constexpr float c = hadamard_coef<H>();
#pragma unroll
    for (int i = 0; i < U; ++i) y[i] = rotated_nan_canonical(y[i] * c);
}

}  // namespace fp4q_dev
