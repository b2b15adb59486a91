// quant_f32.hip -- quantize kernels for f32 input (one translation unit per
// input dtype so the instantiations compile in parallel).
#include "fp4q_launch.hpp"

namespace fp4q_dev {

hipError_t launch_quant_f32(const QuantArgs& a, int B, int H, int sf, int st, int grid, hipStream_t s) {
    return dispatch_quant<float>(a, B, H, sf, st, grid, s);
}

hipError_t launch_gsearch_f32(const GSearchArgs& a, int B, int H, int st, int grid, hipStream_t s) {
    return dispatch_gsearch<float>(a, B, H, st, grid, s);
}

}  // namespace fp4q_dev
