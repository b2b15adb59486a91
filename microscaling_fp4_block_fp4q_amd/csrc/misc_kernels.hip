// misc_kernels.hip -- launchers of the per-tensor abs-max pre-pass,
// dequantize, block MSE and FOCUS relaxed forward / backward kernels; the
// reduction and pick steps of the per-tensor scale search; the code
// histogram.
#include "fp4q_launch.hpp"

namespace fp4q_dev {

__global__ void k_write_g(float* g_dev, float g) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *g_dev = g;
}

hipError_t launch_write_g(float* g_dev, float g, hipStream_t s) {
    hipLaunchKernelGGL(k_write_g, dim3(1), dim3(64), 0, s, g_dev, g);
    return hipGetLastError();
}

// One level of the candidates' fp64 trees: out[j][k] = tree of
// in[j][512 k .. 512 k + 511], entries at or past n counting as 0.
// Grid (ceil(n / 512), kSearchCandidates).
__global__ __launch_bounds__(kThreads) void k_tree_reduce_f64(const double* in, int64_t n, int64_t in_stride,
                                                              double* out, int64_t out_stride) {
    __shared__ double s[kThreads];
    const double* src = in + (int64_t)blockIdx.y * in_stride;
    const int64_t i0 = (int64_t)blockIdx.x * (2 * kThreads) + 2 * threadIdx.x;
    const double a = i0 < n ? src[i0] : 0.0;
    const double b = i0 + 1 < n ? src[i0 + 1] : 0.0;
    s[threadIdx.x] = a + b;
    __syncthreads();
    for (int w = kThreads / 2; w >= 1; w >>= 1) {
        double v = 0.0;
        if ((int)threadIdx.x < w) v = s[2 * threadIdx.x] + s[2 * threadIdx.x + 1];
        __syncthreads();
        if ((int)threadIdx.x < w) s[threadIdx.x] = v;
        __syncthreads();
    }
    if (threadIdx.x == 0) out[(int64_t)blockIdx.y * out_stride + blockIdx.x] = s[0];
}

// The winning candidate: smallest total (a NaN total never wins over a
// number), ties to the smallest j; writes g = fl(g0 (1 - j/64)).
__global__ __launch_bounds__(kThreads) void k_gsearch_pick(const double* totals, int64_t stride,
                                                           const uint32_t* amax_partials, int n_partials,
                                                           float* g_dev) {
    const float g0 = workgroup_amax_scale(amax_partials, n_partials);
    if (threadIdx.x == 0) {
        int best = 0;
        double bt = totals[0];
        for (int j = 1; j < kSearchCandidates; ++j) {
            const double t = totals[j * stride];
            if (t < bt || (bt != bt && t == t)) {
                best = j;
                bt = t;
            }
        }
        *g_dev = g0 * search_factor(best);
    }
}

hipError_t launch_tree_reduce_f64(const double* in, int64_t n, int64_t in_stride, double* out, int64_t out_stride,
                                  hipStream_t s) {
    const int64_t groups = (n + 2 * kThreads - 1) / (2 * kThreads);
    hipLaunchKernelGGL(k_tree_reduce_f64, dim3((unsigned)groups, kSearchCandidates), dim3(kThreads), 0, s, in, n,
                       in_stride, out, out_stride);
    return hipGetLastError();
}

hipError_t launch_gsearch_pick(const double* totals, int64_t stride, const uint32_t* amax_partials, int n_partials,
                               float* g_dev, hipStream_t s) {
    hipLaunchKernelGGL(k_gsearch_pick, dim3(1), dim3(kThreads), 0, s, totals, stride, amax_partials, n_partials,
                       g_dev);
    return hipGetLastError();
}

// Codebook occupancy (TORQ page, section 2.B: codeword usage): counts of the
// 16 nibble codes, added to the caller's counts.  Each lane adds into its own
// LDS bins (bin-major, so the lanes of a wave hit distinct banks), the
// workgroup sums them, and one 64-bit atomic add per code and workgroup
// reaches global memory.

__device__ __forceinline__ void hist_word(uint32_t* h, uint32_t w) {
#pragma unroll
    for (int k = 0; k < 8; ++k) atomicAdd(&h[((w >> (4 * k)) & 15u) * kThreads], 1u);
}

__global__ __launch_bounds__(kThreads) void k_code_hist(const uint8_t* codes, int64_t nbytes,
                                                        unsigned long long* counts) {
    __shared__ uint32_t s_h[16 * kThreads];
    __shared__ uint32_t s_part[kThreads];
    for (int i = threadIdx.x; i < 16 * kThreads; i += kThreads) s_h[i] = 0u;
    __syncthreads();
    uint32_t* h = s_h + threadIdx.x;
    const int64_t nvec = nbytes / 16;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const uint4* src = reinterpret_cast<const uint4*>(codes);
    for (int64_t v = t0; v < nvec; v += stride) {
        const uint4 w = src[v];
        hist_word(h, w.x);
        hist_word(h, w.y);
        hist_word(h, w.z);
        hist_word(h, w.w);
    }
    for (int64_t b = nvec * 16 + t0; b < nbytes; b += stride) {
        const uint32_t byte = codes[b];
        atomicAdd(&h[(byte & 15u) * kThreads], 1u);
        atomicAdd(&h[(byte >> 4) * kThreads], 1u);
    }
    __syncthreads();
    // thread t sums code t & 15 over lanes 16 (t >> 4) .. 16 (t >> 4) + 15
    const int code = threadIdx.x & 15, seg = threadIdx.x >> 4;
    uint32_t part = 0;
#pragma unroll
    for (int l = 0; l < 16; ++l) part += s_h[code * kThreads + seg * 16 + l];
    s_part[threadIdx.x] = part;
    __syncthreads();
    if (threadIdx.x < 16) {
        unsigned long long total = 0;
        for (int sgm = 0; sgm < kThreads / 16; ++sgm) total += s_part[sgm * 16 + threadIdx.x];
        if (total) atomicAdd(&counts[threadIdx.x], total);
    }
}

hipError_t launch_code_hist(const uint8_t* codes, int64_t nbytes, unsigned long long* counts, int grid,
                            hipStream_t s) {
    if (nbytes > 0) {
        const int cap = resident_workgroups<k_code_hist>();
        hipLaunchKernelGGL(k_code_hist, dim3(grid < cap ? grid : cap), dim3(kThreads), 0, s, codes, nbytes, counts);
    }
    return hipGetLastError();
}

// The pre-pass always runs kAmaxBlocks workgroups (one partial each); a.units
// counts 16-byte chunks.
template <class InT>
static hipError_t amax_h(const AmaxArgs& a, int H, int grid, hipStream_t s) {
    constexpr int R = stream_rounds<InT>();
    switch (H) {
    case 0: hipLaunchKernelGGL((k_amax_stream<InT, 0, R>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_amax_stream<InT, 16, R>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_amax_stream<InT, 32, R>), dim3(grid), dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_amax(const AmaxArgs& a, int x_dt, int H, int grid, hipStream_t s) {
    switch (x_dt) {
    case DT_F32: return amax_h<float>(a, H, grid, s);
    case DT_BF16: return amax_h<bf16_t>(a, H, grid, s);
    case DT_F16: return amax_h<f16_t>(a, H, grid, s);
    }
    return hipErrorInvalidValue;
}

// Grid of a chunk-per-lane kernel: R chunks per lane per trip, at most the
// resident workgroups (launch_resident caps it).
template <int R>
static int stream_grid(int64_t units) {
    const int64_t per_wg = (int64_t)kThreads * R;
    const int64_t g = (units + per_wg - 1) / per_wg;
    return (int)(g < 1 ? 1 : (g > (1 << 20) ? (1 << 20) : g));
}

constexpr int kDqRounds = 4;

// a.units counts chunks of 16 bytes of output.
template <int OE>
static hipError_t dequant_b(const DequantArgs& a, int B, hipStream_t s) {
    const int grid = stream_grid<kDqRounds>(a.units);
    switch (B) {
    case 4: return launch_resident<k_dq_stream<4, OE, kDqRounds>>(a, grid, s);
    case 8: return launch_resident<k_dq_stream<8, OE, kDqRounds>>(a, grid, s);
    case 16: return launch_resident<k_dq_stream<16, OE, kDqRounds>>(a, grid, s);
    case 32: return launch_resident<k_dq_stream<32, OE, kDqRounds>>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_dequant(const DequantArgs& a, int B, int out_es, int grid, hipStream_t s) {
    (void)grid;
    return out_es == 4 ? dequant_b<4>(a, B, s) : dequant_b<2>(a, B, s);
}

// a.units counts 16-byte chunks of x.
template <class InT, int B>
static hipError_t mse_h(const MseArgs& a, int H, hipStream_t s) {
    constexpr int R = stream_rounds<InT>();
    const int grid = stream_grid<R>(a.units);
    switch (H) {
    case 0: return launch_resident<k_mse_stream<InT, B, 0, R>>(a, grid, s);
    case 16: return launch_resident<k_mse_stream<InT, B, 16, R>>(a, grid, s);
    case 32: return launch_resident<k_mse_stream<InT, B, 32, R>>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class InT>
static hipError_t mse_b(const MseArgs& a, int B, int H, hipStream_t s) {
    switch (B) {
    case 4: return mse_h<InT, 4>(a, H, s);
    case 8: return mse_h<InT, 8>(a, H, s);
    case 16: return mse_h<InT, 16>(a, H, s);
    case 32: return mse_h<InT, 32>(a, H, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_block_mse(const MseArgs& a, int x_dt, int B, int H, int grid, hipStream_t s) {
    (void)grid;
    switch (x_dt) {
    case DT_F32: return mse_b<float>(a, B, H, s);
    case DT_BF16: return mse_b<bf16_t>(a, B, H, s);
    case DT_F16: return mse_b<f16_t>(a, B, H, s);
    }
    return hipErrorInvalidValue;
}

// a.units counts 16-byte chunks of W.
template <bool BWD, class InT, int B, int K>
static hipError_t relaxed_launch(const RelaxedArgs& a, hipStream_t s) {
    if constexpr (K <= B) {
        constexpr int R = stream_rounds<InT>();
        const int grid = stream_grid<R>(a.units);
        if constexpr (BWD) return launch_resident<k_relaxed_bwd_stream<InT, B, K, R>>(a, grid, s);
        else return launch_resident<k_relaxed_fwd_stream<InT, B, K, R>>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <bool BWD, class InT, int B>
static hipError_t relaxed_k(const RelaxedArgs& a, int K, hipStream_t s) {
    switch (K) {
    case 4: return relaxed_launch<BWD, InT, B, 4>(a, s);
    case 8: return relaxed_launch<BWD, InT, B, 8>(a, s);
    case 16: return relaxed_launch<BWD, InT, B, 16>(a, s);
    case 32: return relaxed_launch<BWD, InT, B, 32>(a, s);
    }
    return hipErrorInvalidValue;
}

template <bool BWD, class InT>
static hipError_t relaxed_b(const RelaxedArgs& a, int B, int K, hipStream_t s) {
    switch (B) {
    case 4: return relaxed_k<BWD, InT, 4>(a, K, s);
    case 8: return relaxed_k<BWD, InT, 8>(a, K, s);
    case 16: return relaxed_k<BWD, InT, 16>(a, K, s);
    case 32: return relaxed_k<BWD, InT, 32>(a, K, s);
    }
    return hipErrorInvalidValue;
}

template <bool BWD>
static hipError_t relaxed_dt(const RelaxedArgs& a, int w_dt, int B, int K, hipStream_t s) {
    switch (w_dt) {
    case DT_F32: return relaxed_b<BWD, float>(a, B, K, s);
    case DT_BF16: return relaxed_b<BWD, bf16_t>(a, B, K, s);
    case DT_F16: return relaxed_b<BWD, f16_t>(a, B, K, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_relaxed_fwd(const RelaxedArgs& a, int w_dt, int B, int K, int grid, hipStream_t s) {
    (void)grid;
    return relaxed_dt<false>(a, w_dt, B, K, s);
}

hipError_t launch_relaxed_bwd(const RelaxedArgs& a, int w_dt, int B, int K, int grid, hipStream_t s) {
    (void)grid;
    return relaxed_dt<true>(a, w_dt, B, K, s);
}

}  // namespace fp4q_dev
