// misc_kernels.hip -- launchers of the per-tensor abs-max pre-pass,
// dequantize, block MSE and FOCUS relaxed forward / backward kernels.
#include "fp4q_launch.hpp"

namespace fp4q_dev {

__global__ void k_write_g(float* g_dev, float g) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *g_dev = g;
}

hipError_t launch_write_g(float* g_dev, float g, hipStream_t s) {
    hipLaunchKernelGGL(k_write_g, dim3(1), dim3(64), 0, s, g_dev, g);
    return hipGetLastError();
}

template <class InT>
static hipError_t amax_h(const AmaxArgs& a, int H, int grid, hipStream_t s) {
    switch (H) {
    case 0: hipLaunchKernelGGL((k_amax<InT, 0>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_amax<InT, 16>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_amax<InT, 32>), dim3(grid), dim3(kThreads), 0, s, a); break;
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

template <int DU>
static hipError_t dequant_b(const DequantArgs& a, int B, int grid, hipStream_t s) {
    switch (B) {
    case 4: return launch_resident<k_dequant<4, DU>>(a, grid, s);
    case 8: return launch_resident<k_dequant<8, DU>>(a, grid, s);
    case 16: return launch_resident<k_dequant<16, DU>>(a, grid, s);
    case 32: return launch_resident<k_dequant<32, DU>>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_dequant(const DequantArgs& a, int B, int DU, int grid, hipStream_t s) {
    return DU == 8 ? dequant_b<8>(a, B, grid, s) : dequant_b<4>(a, B, grid, s);
}

template <class InT, int B>
static hipError_t mse_h(const MseArgs& a, int H, int grid, hipStream_t s) {
    switch (H) {
    case 0: return launch_resident<k_block_mse<InT, B, 0>>(a, grid, s);
    case 16: return launch_resident<k_block_mse<InT, B, 16>>(a, grid, s);
    case 32: return launch_resident<k_block_mse<InT, B, 32>>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class InT>
static hipError_t mse_b(const MseArgs& a, int B, int H, int grid, hipStream_t s) {
    switch (B) {
    case 4: return mse_h<InT, 4>(a, H, grid, s);
    case 8: return mse_h<InT, 8>(a, H, grid, s);
    case 16: return mse_h<InT, 16>(a, H, grid, s);
    case 32: return mse_h<InT, 32>(a, H, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_block_mse(const MseArgs& a, int x_dt, int B, int H, int grid, hipStream_t s) {
    switch (x_dt) {
    case DT_F32: return mse_b<float>(a, B, H, grid, s);
    case DT_BF16: return mse_b<bf16_t>(a, B, H, grid, s);
    case DT_F16: return mse_b<f16_t>(a, B, H, grid, s);
    }
    return hipErrorInvalidValue;
}

template <bool BWD, class InT, int B, int K>
static hipError_t relaxed_launch(const RelaxedArgs& a, int grid, hipStream_t s) {
    if constexpr (K <= B) {
        if constexpr (BWD) return launch_resident<k_relaxed_bwd<InT, B, K>>(a, grid, s);
        else return launch_resident<k_relaxed_fwd<InT, B, K>>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <bool BWD, class InT, int B>
static hipError_t relaxed_k(const RelaxedArgs& a, int K, int grid, hipStream_t s) {
    switch (K) {
    case 4: return relaxed_launch<BWD, InT, B, 4>(a, grid, s);
    case 8: return relaxed_launch<BWD, InT, B, 8>(a, grid, s);
    case 16: return relaxed_launch<BWD, InT, B, 16>(a, grid, s);
    case 32: return relaxed_launch<BWD, InT, B, 32>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <bool BWD, class InT>
static hipError_t relaxed_b(const RelaxedArgs& a, int B, int K, int grid, hipStream_t s) {
    switch (B) {
    case 4: return relaxed_k<BWD, InT, 4>(a, K, grid, s);
    case 8: return relaxed_k<BWD, InT, 8>(a, K, grid, s);
    case 16: return relaxed_k<BWD, InT, 16>(a, K, grid, s);
    case 32: return relaxed_k<BWD, InT, 32>(a, K, grid, s);
    }
    return hipErrorInvalidValue;
}

template <bool BWD>
static hipError_t relaxed_dt(const RelaxedArgs& a, int w_dt, int B, int K, int grid, hipStream_t s) {
    switch (w_dt) {
    case DT_F32: return relaxed_b<BWD, float>(a, B, K, grid, s);
    case DT_BF16: return relaxed_b<BWD, bf16_t>(a, B, K, grid, s);
    case DT_F16: return relaxed_b<BWD, f16_t>(a, B, K, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_relaxed_fwd(const RelaxedArgs& a, int w_dt, int B, int K, int grid, hipStream_t s) {
    return relaxed_dt<false>(a, w_dt, B, K, grid, s);
}

hipError_t launch_relaxed_bwd(const RelaxedArgs& a, int w_dt, int B, int K, int grid, hipStream_t s) {
    return relaxed_dt<true>(a, w_dt, B, K, grid, s);
}

}  // namespace fp4q_dev
