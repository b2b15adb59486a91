// probes.hip -- measurement probes behind the roofline ceilings the
// benchmark reports (libfp4q_probe.so, loaded only by bench.py --probe).
// They are not part of the quantize-dequantize path.
//
//   int fp4q_probe_stream(int kind, const void* src, void* dst, int64_t n16,
//                         int grid, void* stream);
//       HBM streams over n16 16-byte chunks, grid-stride, consecutive lanes on
//       consecutive chunks.  kind 0 / 4 / 5 read src with 4 / 8 / 16 loads
//       in flight per lane, 6 with 8 non-temporal loads (each lane's xor-fold
//       goes to dst, which holds grid * 256 words); 1 writes dst with
//       streaming stores, 7 with plain stores; 2 / 8 copy src to dst (4 / 8
//       loads in flight, streaming stores), 3 with plain stores.  Returns 0,
//       or -1 for a bad argument or launch.
//
//   int fp4q_probe_valu(int kind, int iters, int grid, float* out,
//                       void* stream);
//       VALU issue rate: every lane runs 16 independent dependency chains for
//       iters iterations and writes one float to out[global thread index]
//       (out holds grid * 256 floats).  kind 0: v_add_f32; 1: v_mul_f32;
//       2: v_fma_f32; 3: integer add / xor / shift; 4: fp32 min / max / add;
//       5: the candidate evaluation of the brute-force scale search (division-
//       free quotient at a scale read from LDS, E2M1 rounding, dequantized
//       product, difference, square, balanced-tree sum over a block of 16);
//       6: the same with the rounding by the hardware FP4 pair converts.
//       The executed instruction count comes from the SQ_INSTS_VALU counter.
//
//   int fp4q_probe_fp4_convert(unsigned long long* mismatches, void* stream);
//       Every non-NaN fp32 bit pattern u (2^32 - 2^24 values) through the
//       gfx950 pair converts fp32 -> FP4 (E2M1, scale 1) and back, against
//       the round-half-to-even E2M1 rounding with saturation at 6 that the
//       library computes with ordinary arithmetic: mismatches[0] counts
//       nibbles (sign and magnitude) that differ, mismatches[1] decoded
//       values whose bits differ.  mismatches[2] must be zeroed by the caller
//       (it receives the number of patterns checked).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.hpp"

using namespace fp4q_dev;

namespace {

constexpr int kThreads = 256;

template <int UNROLL, bool NT>
__global__ __launch_bounds__(kThreads) void k_read(const uint4* __restrict__ src, int64_t n, uint32_t* dst) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
            if constexpr (NT) {
                const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i + k * stride));
                v[k] = make_uint4(w.x, w.y, w.z, w.w);
            } else {
                v[k] = src[i + k * stride];
            }
        }
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < n; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    dst[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <bool STREAM>
__global__ __launch_bounds__(kThreads) void k_write(uint4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const uint32_t t = threadIdx.x;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const uint4 v = make_uint4(t, t + 1u, t + 2u, (uint32_t)i);
        if constexpr (STREAM) store_stream(dst + i, v);
        else dst[i] = v;
    }
}

template <int UNROLL, bool STREAM>
__global__ __launch_bounds__(kThreads) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) v[k] = src[i + k * stride];
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) {
            if constexpr (STREAM) store_stream(dst + i + k * stride, v[k]);
            else dst[i + k * stride] = v[k];
        }
    }
    for (; i < n; i += stride) {
        if constexpr (STREAM) store_stream(dst + i, src[i]);
        else dst[i] = src[i];
    }
}

constexpr int kChains = 16;

template <int KIND>
__global__ __launch_bounds__(kThreads) void k_valu(int iters, float* out) {
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = 1.0f + (float)((gid + c) & 7) * 0.125f;
    if constexpr (KIND <= 2) {
        const float a = 1.0f + (float)(gid & 1) * 0x1p-20f, b = 0x1p-30f * (float)(threadIdx.x & 3);
#pragma unroll 1
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                if constexpr (KIND == 0) x[c] = x[c] + b;
                else if constexpr (KIND == 1) x[c] = x[c] * a;
                else x[c] = __builtin_fmaf(x[c], a, b);
            }
        }
    } else if constexpr (KIND == 3) {
        uint32_t u[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) u[c] = as_u(x[c]);
        const uint32_t k = (uint32_t)gid | 1u;
#pragma unroll 1
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) u[c] = ((u[c] + k) ^ (u[c] >> 3));
        }
#pragma unroll
        for (int c = 0; c < kChains; ++c) x[c] = as_f(u[c] & 0x3FFFFFFFu);
    } else if constexpr (KIND == 4) {
        const float lo = 0.5f + (float)(gid & 3), hi = 6.0f + (float)(gid & 1), d = 0x1p-20f;
#pragma unroll 1
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) x[c] = fminf(fmaxf(x[c], lo), hi) + d;
        }
    } else if constexpr (KIND == 6) {
        // the same evaluation with the E2M1 rounding done by the hardware FP4
        // pair converts (fp32 -> FP4 -> fp32)
        __shared__ float2 s_tab[128];
        if (threadIdx.x < 128) {
            const float S = 0.0625f + 0.015625f * (float)threadIdx.x;
            s_tab[threadIdx.x] = make_float2(S, 1.0f / S);
        }
        __syncthreads();
        float acc = 0.0f;
#pragma unroll 1
        for (int it = 0; it < iters; ++it) {
            const float2 sr = s_tab[it & 127];
            float q[kChains], e[kChains];
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                const float a = x[c];
                const float q0 = a * sr.y;
                const float rr = __builtin_fmaf(-q0, sr.x, a);
                q[c] = __builtin_fmaf(rr, sr.y, q0);
            }
#pragma unroll
            for (int c = 0; c < kChains; c += 2) {
                const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[c], q[c + 1], 1.0f, 0);
                const auto g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float d = x[c + h] - g2[h] * sr.x;
                    e[c + h] = d * d;
                }
            }
            acc = fminf(acc, tree_sum<kChains>(e));
        }
        x[0] += acc;
    } else {
        // the brute-force candidate evaluation: a block of 16 values at scale
        // S_it (one LDS broadcast per candidate), as the search kernels run it
        __shared__ float2 s_tab[128];
        if (threadIdx.x < 128) {
            const float S = 0.0625f + 0.015625f * (float)threadIdx.x;
            s_tab[threadIdx.x] = make_float2(S, 1.0f / S);
        }
        __syncthreads();
        float acc = 0.0f;
#pragma unroll 1
        for (int it = 0; it < iters; ++it) {
            const float2 sr = s_tab[it & 127];
            float e[kChains];
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                const float a = x[c];
                const float q0 = a * sr.y;
                const float rr = __builtin_fmaf(-q0, sr.x, a);
                const float q = __builtin_fmaf(rr, sr.y, q0);
                const float r = e2m1_round(q);
                const float d = a - r * sr.x;
                e[c] = d * d;
            }
            acc = fminf(acc, tree_sum<kChains>(e));
        }
        x[0] += acc;
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[gid] = s;
}

// Exhaustive check of the hardware FP4 pair convert, 2^32 patterns: each
// thread takes 64 consecutive patterns (32 pairs).
__global__ __launch_bounds__(kThreads) void k_fp4_convert(unsigned long long* mismatches) {
    const uint64_t base = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * 64u;
    unsigned long long bad_code = 0, bad_value = 0, checked = 0;
    for (int k = 0; k < 64; k += 2) {
        const uint32_t b0 = (uint32_t)(base + k), b1 = b0 + 1u;
        const float u0 = as_f(b0), u1 = as_f(b1);
        const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, u0, u1, 1.0f, 0);
        const auto back = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(hw, 1.0f, 0);
        const float uu[2] = {u0, u1};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float u = uu[e];
            if (u != u) continue;
            const float r = e2m1_round(fabsf(u));
            const uint32_t want = ((as_u(u) >> 31) << 3) | e2m1_code_of(r);
            const uint32_t got = (hw >> (4 * e)) & 15u;
            const float want_v = as_f(as_u(r) | (as_u(u) & 0x80000000u));
            bad_code += got != want;
            bad_value += as_u(back[e]) != as_u(want_v);
            ++checked;
        }
    }
    if (bad_code) atomicAdd(&mismatches[0], bad_code);
    if (bad_value) atomicAdd(&mismatches[1], bad_value);
    atomicAdd(&mismatches[2], checked);
}

// The gfx950 scaled converts FP4 -> bf16 and FP4 -> fp16 (which the NVFP4
// GEMM dequantizes its operands with): every byte of two nibbles, at each of
// the four byte positions of the source dword, for the power-of-two part
// P_c = 2^(max(e, 1) - 7) of every E4M3 block scale code c = (e, m), c =
// 0..126, against the exact product of the E2M1 value and P_c.  The same
// converts given the full scale value dec(c) are counted too: they apply
// only its exponent (as an E8M0 scale would be), which is why the GEMM
// multiplies the scale's mantissa in separately.  counts: [0] bf16 values
// that differ (+0 and -0 equal), [1] bf16 bit patterns that differ, [2], [3]
// the same for fp16, [4] values checked, [5] fp16 values that differ from
// the exact product when the full dec(c) is passed.
typedef __bf16 probe_bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 probe_f16x2 __attribute__((ext_vector_type(2)));

template <int POS>
__device__ __forceinline__ void scaled_convert_pos(uint32_t byte, float P, float S, unsigned long long (&bad)[6]) {
    const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const uint32_t src = (0xA5C3E1F7u & ~(0xFFu << (8 * POS))) | (byte << (8 * POS));
    const probe_bf16x2 hb = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, P, POS);
    const probe_f16x2 hh = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, P, POS);
    const probe_f16x2 hs = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, S, POS);
    const uint32_t gb = __builtin_bit_cast(uint32_t, hb), gh = __builtin_bit_cast(uint32_t, hh);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t nib = (byte >> (4 * h)) & 15u;
        const float mag = grid[nib & 7u], sgn = nib & 8u ? -1.0f : 1.0f;
        const float want = sgn * mag * P, want_s = sgn * mag * S;
        const uint32_t wb = as_u(want) >> 16;
        const uint32_t wh = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)want);
        const uint32_t xb = (gb >> (16 * h)) & 0xFFFFu, xh = (gh >> (16 * h)) & 0xFFFFu;
        bad[0] += as_f(xb << 16) != want;
        bad[1] += xb != wb;
        bad[2] += (float)__builtin_bit_cast(_Float16, (uint16_t)xh) != want;
        bad[3] += xh != wh;
        bad[4] += 1;
        bad[5] += (float)hs[h] != want_s;
    }
}

__global__ __launch_bounds__(256) void k_fp4_scaled_convert(unsigned long long* counts) {
    const uint32_t code = blockIdx.x, byte = threadIdx.x;
    const uint32_t e = code >> 3, m = code & 7u;
    const float S = e == 0u ? (float)m * 0x1p-9f : __builtin_ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
    const float P = __builtin_ldexpf(1.0f, (int)(e > 0u ? e : 1u) - 7);
    unsigned long long bad[6] = {0, 0, 0, 0, 0, 0};
    scaled_convert_pos<0>(byte, P, S, bad);
    scaled_convert_pos<1>(byte, P, S, bad);
    scaled_convert_pos<2>(byte, P, S, bad);
    scaled_convert_pos<3>(byte, P, S, bad);
#pragma unroll
    for (int i = 0; i < 6; ++i)
        if (bad[i]) atomicAdd(&counts[i], bad[i]);
}

template <int KIND>
hipError_t launch_valu(int iters, int grid, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_valu<KIND>, dim3(grid), dim3(kThreads), 0, s, iters, out);
    return hipGetLastError();
}

}  // namespace

extern "C" {

int fp4q_probe_stream(int kind, const void* src, void* dst, int64_t n16, int grid, void* stream) {
    if (n16 <= 0 || grid <= 0 || !dst || (kind != 1 && kind != 7 && !src)) return -1;
    hipStream_t s = (hipStream_t)stream;
    const uint4* in = reinterpret_cast<const uint4*>(src);
    uint4* out = reinterpret_cast<uint4*>(dst);
    uint32_t* words = reinterpret_cast<uint32_t*>(dst);
    switch (kind) {
    case 0: hipLaunchKernelGGL((k_read<4, false>), dim3(grid), dim3(kThreads), 0, s, in, n16, words); break;
    case 1: hipLaunchKernelGGL(k_write<true>, dim3(grid), dim3(kThreads), 0, s, out, n16); break;
    case 2: hipLaunchKernelGGL((k_copy<4, true>), dim3(grid), dim3(kThreads), 0, s, in, out, n16); break;
    case 3: hipLaunchKernelGGL((k_copy<4, false>), dim3(grid), dim3(kThreads), 0, s, in, out, n16); break;
    case 4: hipLaunchKernelGGL((k_read<8, false>), dim3(grid), dim3(kThreads), 0, s, in, n16, words); break;
    case 5: hipLaunchKernelGGL((k_read<16, false>), dim3(grid), dim3(kThreads), 0, s, in, n16, words); break;
    case 6: hipLaunchKernelGGL((k_read<8, true>), dim3(grid), dim3(kThreads), 0, s, in, n16, words); break;
    case 7: hipLaunchKernelGGL(k_write<false>, dim3(grid), dim3(kThreads), 0, s, out, n16); break;
    case 8: hipLaunchKernelGGL((k_copy<8, true>), dim3(grid), dim3(kThreads), 0, s, in, out, n16); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int fp4q_probe_fp4_convert(unsigned long long* mismatches, void* stream) {
    if (!mismatches) return -1;
    const uint64_t threads = (1ull << 32) / 64u;
    hipLaunchKernelGGL(k_fp4_convert, dim3((unsigned)(threads / kThreads)), dim3(kThreads), 0, (hipStream_t)stream,
                       mismatches);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int fp4q_probe_fp4_scaled_convert(unsigned long long* counts, void* stream) {
    if (!counts) return -1;
    hipLaunchKernelGGL(k_fp4_scaled_convert, dim3(127), dim3(256), 0, (hipStream_t)stream, counts);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int fp4q_probe_valu(int kind, int iters, int grid, float* out, void* stream) {
    if (iters <= 0 || grid <= 0 || !out) return -1;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (kind) {
    case 0: e = launch_valu<0>(iters, grid, out, s); break;
    case 1: e = launch_valu<1>(iters, grid, out, s); break;
    case 2: e = launch_valu<2>(iters, grid, out, s); break;
    case 3: e = launch_valu<3>(iters, grid, out, s); break;
    case 4: e = launch_valu<4>(iters, grid, out, s); break;
    case 5: e = launch_valu<5>(iters, grid, out, s); break;
    case 6: e = launch_valu<6>(iters, grid, out, s); break;
    default: return -1;
    }
    return e == hipSuccess ? 0 : -1;
}

}  // extern "C"
