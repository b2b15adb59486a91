// fp4q_launch.hpp -- host-side launch entry points of the kernel
// translation units (internal to libfp4q.so).
#pragma once

#include <hip/hip_runtime.h>

#include "fp4q_kernels.hpp"
#include "fp4q_stream.hpp"

namespace fp4q_dev {

// Quantize launch for one input dtype (fp32 / bf16 / fp16 translation units).
hipError_t launch_quant_f32(const QuantArgs& a, int B, int H, int sf, int st, int grid, hipStream_t s);
hipError_t launch_quant_bf16(const QuantArgs& a, int B, int H, int sf, int st, int grid, hipStream_t s);
hipError_t launch_quant_f16(const QuantArgs& a, int B, int H, int sf, int st, int grid, hipStream_t s);

// Per-tensor scale search for one input dtype; st is ST_ABSMAX (with
// a.prevent_zero) or ST_FOUR_OVER_SIX.
hipError_t launch_gsearch_f32(const GSearchArgs& a, int B, int H, int st, int grid, hipStream_t s);
hipError_t launch_gsearch_bf16(const GSearchArgs& a, int B, int H, int st, int grid, hipStream_t s);
hipError_t launch_gsearch_f16(const GSearchArgs& a, int B, int H, int st, int grid, hipStream_t s);
hipError_t launch_tree_reduce_f64(const double* in, int64_t n, int64_t in_stride, double* out, int64_t out_stride,
                                  hipStream_t s);
hipError_t launch_gsearch_pick(const double* totals, int64_t stride, const uint32_t* amax_partials, int n_partials,
                               float* g_dev, hipStream_t s);

size_t mxfp4_gemm_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_mxfp4_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs, int64_t M,
                             int64_t N, int64_t K, void* c, int c_dt, int64_t ldc, void* workspace, hipStream_t s);
size_t nvfp4_gemm_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_nvfp4_gemm(const uint8_t* a, const uint8_t* as, const float* ga, const uint8_t* b,
                             const uint8_t* bs, const float* gb, int64_t M, int64_t N, int64_t K, void* c, int c_dt,
                             int64_t ldc, void* workspace, hipStream_t s);
hipError_t launch_code_hist(const uint8_t* codes, int64_t nbytes, unsigned long long* counts, int grid,
                            hipStream_t s);
hipError_t launch_amax(const AmaxArgs& a, int x_dt, int H, int grid, hipStream_t s);
hipError_t launch_write_g(float* g_dev, float g, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, int B, int out_es, int grid, hipStream_t s);
hipError_t launch_block_mse(const MseArgs& a, int x_dt, int B, int H, int grid, hipStream_t s);
hipError_t launch_relaxed_fwd(const RelaxedArgs& a, int w_dt, int B, int K, int grid, hipStream_t s);
hipError_t launch_relaxed_bwd(const RelaxedArgs& a, int w_dt, int B, int K, int grid, hipStream_t s);

// Workgroups of KERNEL that the device holds at once (occupancy from its
// registers and LDS, at most MAX_PER_CU per compute unit when given, times
// the compute units), computed on first use.  Grid-stride kernels are
// launched with at most this many workgroups, so every workgroup is
// resident from the start and the tiles are spread evenly (a second,
// partial round of long-running workgroups would leave most compute units
// idle at the end).
template <auto KERNEL, int MAX_PER_CU = 0>
int resident_workgroups() {
    static const int n = [] {
        int per_cu = 0, dev = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERNEL, kThreads, 0) != hipSuccess) per_cu = 1;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 256;
        if (MAX_PER_CU > 0 && per_cu > MAX_PER_CU) per_cu = MAX_PER_CU;
        return (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    }();
    return n;
}

template <auto KERNEL, int MAX_PER_CU = 0, class Args>
hipError_t launch_resident(const Args& a, int grid, hipStream_t s) {
    const int cap = resident_workgroups<KERNEL, MAX_PER_CU>();
    hipLaunchKernelGGL(KERNEL, dim3(grid < cap ? grid : cap), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// Workgroups per compute unit of the brute-force kernels: B = 4 fits seven
// by registers and LDS, but runs 6 % faster with six (measured on 4096 x 4096
// fp32); larger blocks hold at most five anyway.
constexpr int kBfMaxWorkgroupsPerCU = 6;

// Template dispatch over block size, rotation size, scale format and
// strategy.  The streaming kernel takes a.units in 16-byte chunks and sizes
// its grid itself (R chunks per lane per trip, at most the resident
// workgroups); brute force takes units of unit_elems values.
template <class InT, int B, int H, int SF, int ST>
hipError_t launch_quant_t(const QuantArgs& a, int grid, hipStream_t s) {
    if constexpr (ST == ST_BRUTE_FORCE) {
        if (a.counts) return launch_resident<k_quant_bf<InT, B, H, SF, true>, kBfMaxWorkgroupsPerCU>(a, grid, s);
        return launch_resident<k_quant_bf<InT, B, H, SF, false>, kBfMaxWorkgroupsPerCU>(a, grid, s);
    } else {
        constexpr int R = stream_rounds<InT>();
        const int64_t per_wg = (int64_t)kThreads * R;
        const int64_t g = (a.units + per_wg - 1) / per_wg;
        return launch_resident<k_qstream<InT, B, H, SF, ST, R>>(a, (int)(g < 1 ? 1 : (g > (1 << 20) ? (1 << 20) : g)), s);
    }
}

template <class InT, int B, int H, int SF>
hipError_t dispatch_quant_st(const QuantArgs& a, int st, int grid, hipStream_t s) {
    switch (st) {
    case ST_ABSMAX:
    case ST_PREVENT_ZERO:
        return launch_quant_t<InT, B, H, SF, ST_ABSMAX>(a, grid, s);
    case ST_FOUR_OVER_SIX:
        if constexpr (SF != SF_E8M0) return launch_quant_t<InT, B, H, SF, ST_FOUR_OVER_SIX>(a, grid, s);
        return hipErrorInvalidValue;
    case ST_BRUTE_FORCE:
        return launch_quant_t<InT, B, H, SF, ST_BRUTE_FORCE>(a, grid, s);
    case ST_GIVEN:
        return launch_quant_t<InT, B, H, SF, ST_GIVEN>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class InT, int B, int H>
hipError_t dispatch_quant_sf(const QuantArgs& a, int sf, int st, int grid, hipStream_t s) {
    switch (sf) {
    case SF_E8M0: return dispatch_quant_st<InT, B, H, SF_E8M0>(a, st, grid, s);
    case SF_E4M3: return dispatch_quant_st<InT, B, H, SF_E4M3>(a, st, grid, s);
    case SF_UE5M3: return dispatch_quant_st<InT, B, H, SF_UE5M3>(a, st, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class InT, int B>
hipError_t dispatch_quant_h(const QuantArgs& a, int H, int sf, int st, int grid, hipStream_t s) {
    switch (H) {
    case 0: return dispatch_quant_sf<InT, B, 0>(a, sf, st, grid, s);
    case 16: return dispatch_quant_sf<InT, B, 16>(a, sf, st, grid, s);
    case 32: return dispatch_quant_sf<InT, B, 32>(a, sf, st, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class InT>
hipError_t dispatch_quant(const QuantArgs& a, int B, int H, int sf, int st, int grid, hipStream_t s) {
    switch (B) {
    case 4: return dispatch_quant_h<InT, 4>(a, H, sf, st, grid, s);
    case 8: return dispatch_quant_h<InT, 8>(a, H, sf, st, grid, s);
    case 16: return dispatch_quant_h<InT, 16>(a, H, sf, st, grid, s);
    case 32: return dispatch_quant_h<InT, 32>(a, H, sf, st, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class InT, int B, int H>
hipError_t dispatch_gsearch_st(const GSearchArgs& a, int st, int grid, hipStream_t s) {
    if (st == ST_FOUR_OVER_SIX) return launch_resident<k_gsearch<InT, B, H, ST_FOUR_OVER_SIX>>(a, grid, s);
    if (st == ST_BRUTE_FORCE) return launch_resident<k_gsearch_bf<InT, B, H>, kBfMaxWorkgroupsPerCU>(a, grid, s);
    return launch_resident<k_gsearch<InT, B, H, ST_ABSMAX>>(a, grid, s);
}

template <class InT, int B>
hipError_t dispatch_gsearch_h(const GSearchArgs& a, int H, int st, int grid, hipStream_t s) {
    switch (H) {
    case 0: return dispatch_gsearch_st<InT, B, 0>(a, st, grid, s);
    case 16: return dispatch_gsearch_st<InT, B, 16>(a, st, grid, s);
    case 32: return dispatch_gsearch_st<InT, B, 32>(a, st, grid, s);
    }
    return hipErrorInvalidValue;
}

template <class InT>
hipError_t dispatch_gsearch(const GSearchArgs& a, int B, int H, int st, int grid, hipStream_t s) {
    switch (B) {
    case 4: return dispatch_gsearch_h<InT, 4>(a, H, st, grid, s);
    case 8: return dispatch_gsearch_h<InT, 8>(a, H, st, grid, s);
    case 16: return dispatch_gsearch_h<InT, 16>(a, H, st, grid, s);
    case 32: return dispatch_gsearch_h<InT, 32>(a, H, st, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace fp4q_dev
