// fp4q_api.hip -- the C ABI of include/fp4q.h: synchronous argument
// validation on the host, then kernel launches on the caller's stream.
// Nothing here allocates, synchronises or keeps state.
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fp4q.h"
#include <algorithm>
#include <mutex>

#include "fp4q_launch.hpp"

using namespace fp4q_dev;

static_assert(FP4Q_COUNT_REPLICAS == kCountReplicas, "rows of the fused code counts");

// Workspace of fp4q_quantize_noalloc: one copy per device, held until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol); it takes the device address that
// hipGetSymbolAddress returns for the device in use.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxGrid = 1 << 20;   // workgroups of a grid-stride launch (further capped by residency)

int elem_size(int dt) { return dt == FP4Q_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == FP4Q_F32 || dt == FP4Q_BF16 || dt == FP4Q_F16; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int grid_for(int64_t units) {
    int64_t g = (units + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    return (int)(g < kMaxGrid ? g : kMaxGrid);
}

// Checks of the configuration shared by every call.
fp4q_status check_config(const fp4q_config* cfg) {
    if (!cfg || cfg->struct_size != sizeof(fp4q_config)) return FP4Q_ERR_INVALID_ARG;
    if (cfg->scale_fmt != FP4Q_SCALE_E8M0 && cfg->scale_fmt != FP4Q_SCALE_E4M3 &&
        cfg->scale_fmt != FP4Q_SCALE_UE5M3)
        return FP4Q_ERR_INVALID_ARG;
    if (cfg->strategy < FP4Q_ABSMAX || cfg->strategy > FP4Q_GIVEN) return FP4Q_ERR_INVALID_ARG;
    if (cfg->global_mode < FP4Q_GLOBAL_NONE || cfg->global_mode > FP4Q_GLOBAL_SEARCH) return FP4Q_ERR_INVALID_ARG;
    if (cfg->hadamard < 0) return FP4Q_ERR_INVALID_ARG;
    if (cfg->block != 4 && cfg->block != 8 && cfg->block != 16 && cfg->block != 32) return FP4Q_ERR_SHAPE;
    if (cfg->hadamard != 0 && cfg->hadamard != 16 && cfg->hadamard != 32) return FP4Q_ERR_UNSUPPORTED;
    if (cfg->scale_fmt == FP4Q_SCALE_E8M0 &&
        (cfg->global_mode != FP4Q_GLOBAL_NONE || cfg->strategy == FP4Q_FOUR_OVER_SIX))
        return FP4Q_ERR_UNSUPPORTED;
    if (cfg->scale_fmt == FP4Q_SCALE_UE5M3 &&
        (cfg->global_mode == FP4Q_GLOBAL_TENSOR_AMAX || cfg->global_mode == FP4Q_GLOBAL_SEARCH))
        return FP4Q_ERR_UNSUPPORTED;
    if (cfg->global_mode == FP4Q_GLOBAL_SEARCH && cfg->strategy == FP4Q_GIVEN) return FP4Q_ERR_UNSUPPORTED;
    if (cfg->global_mode == FP4Q_GLOBAL_USER) {
        const double g = cfg->global_scale;
        if (!(g >= FLT_MIN) || !(448.0 * g < FLT_MAX)) return FP4Q_ERR_INVALID_ARG;
    }
    return FP4Q_OK;
}

// A [rows, ld] tensor operand of element type dt.
fp4q_status check_tensor(const void* p, int dt, int64_t rows, int64_t cols, int64_t ld) {
    if (!p) return FP4Q_ERR_INVALID_ARG;
    if (!dtype_ok(dt)) return FP4Q_ERR_INVALID_ARG;
    if (ld < cols) return FP4Q_ERR_SHAPE;
    (void)rows;
    const int es = elem_size(dt);
    if (!aligned16(p) || (ld * es) % 16 != 0 || (cols * es) % 16 != 0) return FP4Q_ERR_ALIGNMENT;
    return FP4Q_OK;
}

fp4q_status check_dims(int64_t rows, int64_t cols, int block, int H) {
    if (rows < 0 || cols < 0) return FP4Q_ERR_INVALID_ARG;
    if (cols > 0 && rows > INT64_MAX / 64 / cols) return FP4Q_ERR_INVALID_ARG;
    if (cols % block != 0) return FP4Q_ERR_SHAPE;
    if (H && cols % H != 0) return FP4Q_ERR_SHAPE;
    return FP4Q_OK;
}

fp4q_status check_buffer(const void* p) {
    if (!p) return FP4Q_ERR_INVALID_ARG;
    return aligned16(p) ? FP4Q_OK : FP4Q_ERR_ALIGNMENT;
}

fp4q_status device_status(hipError_t e) { return e == hipSuccess ? FP4Q_OK : FP4Q_ERR_DEVICE; }

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream), looked up once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

fp4q_status scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return FP4Q_ERR_DEVICE;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return FP4Q_ERR_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return FP4Q_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return FP4Q_ERR_DEVICE;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return FP4Q_ERR_DEVICE;
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !ptr) return FP4Q_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FP4Q_OK;
}

int unit_of(int x_dt, int block, int H) {
    int u = 16 / elem_size(x_dt);
    if (block > u) u = block;
    if (H > u) u = H;
    return u;
}

// Workspace of the per-tensor scale search: abs-max partials, then the
// candidates' per-tile sums, then one reduction level's sums.
constexpr size_t kAmaxBytes = (size_t)kAmaxBlocks * sizeof(uint32_t);

int64_t search_tiles(int64_t rows, int64_t cols, int U) { return (rows * cols / U + kTileUnits - 1) / kTileUnits; }

size_t search_workspace_bytes(int64_t tiles) {
    const int64_t level = (tiles + 2 * kThreads - 1) / (2 * kThreads);
    return kAmaxBytes + (size_t)kSearchCandidates * sizeof(double) * (size_t)(tiles + level);
}

#define FP4Q_TRY(expr)                           \
    do {                                         \
        fp4q_status st_ = (expr);                \
        if (st_ != FP4Q_OK) return st_;          \
    } while (0)

// Shared body of fp4q_quantize and fp4q_scale_search.
// from_scratch: the workspace is the static scratch (fp4q_quantize_noalloc),
// looked up after every argument check.  counts: code occupancy to add to
// (fp4q_quantize_histogram), checked by the caller.
fp4q_status run_quant(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows, int64_t cols,
                      int64_t ld_x, uint8_t* codes, uint8_t* scales, float* g_dev, void* dequant,
                      int dq_dt, int64_t ld_dq, float* mse, float* sse, void* workspace,
                      void* stream, bool from_scratch = false, unsigned long long* counts = nullptr) {
    const int B = cfg->block, H = cfg->hadamard;
    FP4Q_TRY(check_dims(rows, cols, B, H));
    const bool need_g = cfg->global_mode != FP4Q_GLOBAL_NONE;
    if (need_g && !g_dev) return FP4Q_ERR_INVALID_ARG;
    if (g_dev && ((uintptr_t)g_dev & 3u)) return FP4Q_ERR_ALIGNMENT;
    hipStream_t s = (hipStream_t)stream;
    if (rows == 0 || cols == 0) {
        // nothing is read or written except g (1 for an empty tensor, or the user's)
        if (!dtype_ok(x_dt) || (dequant && !dtype_ok(dq_dt))) return FP4Q_ERR_INVALID_ARG;
        const float g_fixed = cfg->global_mode == FP4Q_GLOBAL_USER ? cfg->global_scale : 1.0f;
        if (g_dev) return device_status(launch_write_g(g_dev, g_fixed, s));
        return FP4Q_OK;
    }
    FP4Q_TRY(check_tensor(x, x_dt, rows, cols, ld_x));
    FP4Q_TRY(check_buffer(scales));
    if (codes) FP4Q_TRY(check_buffer(codes));
    if (dequant) FP4Q_TRY(check_tensor(dequant, dq_dt, rows, cols, ld_dq));
    if (mse) FP4Q_TRY(check_buffer(mse));
    if (sse) FP4Q_TRY(check_buffer(sse));
    const bool search = cfg->global_mode == FP4Q_GLOBAL_SEARCH;
    const bool tamax = cfg->global_mode == FP4Q_GLOBAL_TENSOR_AMAX || search;
    if (tamax && from_scratch) FP4Q_TRY(scratch_address(s, &workspace));
    if (tamax) FP4Q_TRY(check_buffer(workspace));

    if (tamax) {
        const int U = 16 / elem_size(x_dt);       // the pre-pass walks 16-byte chunks
        AmaxArgs aa{};
        aa.x = x;
        aa.ld_x = ld_x;
        aa.units = rows * cols / U;
        aa.units_per_row = cols / U;
        aa.contiguous = ld_x == cols;
        aa.partials = reinterpret_cast<uint32_t*>(workspace);
        FP4Q_TRY(device_status(launch_amax(aa, x_dt, H, kAmaxBlocks, s)));
    }

    if (search) {
        const int U = unit_of(x_dt, B, H);
        GSearchArgs ga{};
        ga.x = x;
        ga.ld_x = ld_x;
        ga.units = rows * cols / U;
        ga.units_per_row = cols / U;
        ga.contiguous = ld_x == cols;
        ga.amax_partials = reinterpret_cast<const uint32_t*>(workspace);
        ga.n_partials = kAmaxBlocks;
        ga.prevent_zero = cfg->strategy == FP4Q_PREVENT_ZERO;
        ga.ntiles = search_tiles(rows, cols, U);
        double* level0 = reinterpret_cast<double*>(reinterpret_cast<char*>(workspace) + kAmaxBytes);
        double* level1 = level0 + (size_t)kSearchCandidates * ga.ntiles;
        ga.partials = level0;
        const int st = cfg->strategy == FP4Q_FOUR_OVER_SIX ? ST_FOUR_OVER_SIX
                       : cfg->strategy == FP4Q_BRUTE_FORCE ? ST_BRUTE_FORCE
                                                           : ST_ABSMAX;
        const int grid = grid_for(ga.units);
        hipError_t e;
        switch (x_dt) {
        case FP4Q_F32: e = launch_gsearch_f32(ga, B, H, st, grid, s); break;
        case FP4Q_BF16: e = launch_gsearch_bf16(ga, B, H, st, grid, s); break;
        default: e = launch_gsearch_f16(ga, B, H, st, grid, s); break;
        }
        FP4Q_TRY(device_status(e));
        // tiles -> groups of 512 -> ... -> one total per candidate, alternating buffers
        const double* src = level0;
        int64_t n = ga.ntiles, stride = ga.ntiles;
        while (n > 1) {
            const int64_t m = (n + 2 * kThreads - 1) / (2 * kThreads);
            double* dst = src == level0 ? level1 : level0;
            FP4Q_TRY(device_status(launch_tree_reduce_f64(src, n, stride, dst, m, s)));
            src = dst;
            n = m;
            stride = m;
        }
        FP4Q_TRY(device_status(launch_gsearch_pick(src, stride, ga.amax_partials, kAmaxBlocks, g_dev, s)));
    }

    // brute force works in units of unit_of() values, the streaming kernel in
    // 16-byte chunks
    const int U = cfg->strategy == FP4Q_BRUTE_FORCE ? unit_of(x_dt, B, H) : 16 / elem_size(x_dt);
    QuantArgs qa{};
    qa.x = x;
    qa.ld_x = ld_x;
    qa.cols = cols;
    qa.units = rows * cols / U;
    qa.units_per_row = cols / U;
    qa.contiguous = ld_x == cols && (!dequant || ld_dq == cols);
    qa.codes = codes;
    qa.scales = scales;
    qa.g_out = g_dev;
    qa.dq = dequant;
    qa.ld_dq = ld_dq;
    qa.dq_dt = dq_dt;
    qa.mse = mse;
    qa.sse = sse;
    qa.amax_partials = reinterpret_cast<const uint32_t*>(workspace);
    qa.n_partials = tamax ? kAmaxBlocks : 0;
    qa.global_mode = search ? GM_DEVICE : cfg->global_mode;
    qa.user_g = cfg->global_scale;
    qa.g_in = g_dev;
    if (search) qa.g_out = nullptr;      // g_dev already holds the searched scale
    qa.prevent_zero = cfg->strategy == FP4Q_PREVENT_ZERO;
    qa.counts = counts;
    const int grid = grid_for(qa.units);
    hipError_t e;
    switch (x_dt) {
    case FP4Q_F32: e = launch_quant_f32(qa, B, H, cfg->scale_fmt, cfg->strategy, grid, s); break;
    case FP4Q_BF16: e = launch_quant_bf16(qa, B, H, cfg->scale_fmt, cfg->strategy, grid, s); break;
    default: e = launch_quant_f16(qa, B, H, cfg->scale_fmt, cfg->strategy, grid, s); break;
    }
    return device_status(e);
}

// g_dev of the calls that read a scale: must be NULL for E8M0.
fp4q_status check_g_in(const fp4q_config* cfg, const float* g_dev) {
    if (g_dev && cfg->scale_fmt == FP4Q_SCALE_E8M0) return FP4Q_ERR_UNSUPPORTED;
    if (g_dev && ((uintptr_t)g_dev & 3u)) return FP4Q_ERR_ALIGNMENT;
    return FP4Q_OK;
}

}  // namespace

extern "C" {

int fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

const char* fp4q_status_string(int status) {
    switch (status) {
    case FP4Q_OK: return "ok";
    case FP4Q_ERR_INVALID_ARG: return "invalid argument";
    case FP4Q_ERR_UNSUPPORTED: return "unsupported combination";
    case FP4Q_ERR_SHAPE: return "shape does not tile into blocks";
    case FP4Q_ERR_ALIGNMENT: return "pointer or row pitch not 16-byte aligned";
    case FP4Q_ERR_DEVICE: return "device launch failed";
    case FP4Q_ERR_TOO_LARGE: return "workspace needed exceeds the library's static scratch";
    }
    return "unknown status";
}

size_t fp4q_workspace_bytes(const fp4q_config* cfg, int64_t rows, int64_t cols) {
    if (!cfg) return 0;
    if (cfg->global_mode == FP4Q_GLOBAL_SEARCH) {
        // the most units any input type gives: fp32, U = max(4, block, hadamard)
        const int U = unit_of(FP4Q_F32, cfg->block > 0 ? cfg->block : 1, cfg->hadamard > 0 ? cfg->hadamard : 0);
        return search_workspace_bytes(rows > 0 && cols > 0 ? search_tiles(rows, cols, U) : 0);
    }
    return cfg->global_mode == FP4Q_GLOBAL_TENSOR_AMAX ? kAmaxBytes : 0;
}

fp4q_status fp4q_quantize(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows, int64_t cols,
                          int64_t ld_x, uint8_t* codes, uint8_t* scales, float* g_dev, void* dequant,
                          int dq_dt, int64_t ld_dq, float* block_mse, void* workspace, void* stream) {
    FP4Q_TRY(check_config(cfg));
    if (!codes && rows > 0 && cols > 0) return FP4Q_ERR_INVALID_ARG;
    return run_quant(cfg, x, x_dt, rows, cols, ld_x, codes, scales, g_dev, dequant, dq_dt, ld_dq,
                     block_mse, nullptr, workspace, stream);
}

fp4q_status fp4q_quantize_noalloc(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows, int64_t cols,
                                  int64_t ld_x, uint8_t* codes, uint8_t* scales, float* g_dev, void* dequant,
                                  int dq_dt, int64_t ld_dq, float* block_mse, void* stream) {
    FP4Q_TRY(check_config(cfg));
    if (!codes && rows > 0 && cols > 0) return FP4Q_ERR_INVALID_ARG;
    if (fp4q_workspace_bytes(cfg, rows, cols) > kNoAllocScratchBytes) return FP4Q_ERR_TOO_LARGE;
    return run_quant(cfg, x, x_dt, rows, cols, ld_x, codes, scales, g_dev, dequant, dq_dt, ld_dq, block_mse,
                     nullptr, nullptr, stream, true);
}

fp4q_status fp4q_quantize_histogram(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows,
                                    int64_t cols, int64_t ld_x, uint8_t* codes, uint8_t* scales, float* g_dev,
                                    void* dequant, int dq_dt, int64_t ld_dq, float* block_mse, uint64_t* counts,
                                    void* workspace, void* stream) {
    FP4Q_TRY(check_config(cfg));
    if (!counts) return FP4Q_ERR_INVALID_ARG;
    if ((uintptr_t)counts & 7u) return FP4Q_ERR_ALIGNMENT;
    if (!codes && rows > 0 && cols > 0) return FP4Q_ERR_INVALID_ARG;
    return run_quant(cfg, x, x_dt, rows, cols, ld_x, codes, scales, g_dev, dequant, dq_dt, ld_dq, block_mse,
                     nullptr, workspace, stream, false, reinterpret_cast<unsigned long long*>(counts));
}

fp4q_status fp4q_scale_search(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows,
                              int64_t cols, int64_t ld_x, uint8_t* scales, float* g_dev,
                              float* best_sse, void* workspace, void* stream) {
    FP4Q_TRY(check_config(cfg));
    if (cfg->strategy == FP4Q_GIVEN) return FP4Q_ERR_INVALID_ARG;
    return run_quant(cfg, x, x_dt, rows, cols, ld_x, nullptr, scales, g_dev, nullptr, FP4Q_F32, cols,
                     nullptr, best_sse, workspace, stream);
}

fp4q_status fp4q_dequantize(const fp4q_config* cfg, const uint8_t* codes, const uint8_t* scales,
                            const float* g_dev, int64_t rows, int64_t cols, void* out, int out_dt,
                            int64_t ld_out, void* stream) {
    FP4Q_TRY(check_config(cfg));
    const int B = cfg->block;
    FP4Q_TRY(check_dims(rows, cols, B, 0));
    FP4Q_TRY(check_g_in(cfg, g_dev));
    if (rows == 0 || cols == 0) return dtype_ok(out_dt) ? FP4Q_OK : FP4Q_ERR_INVALID_ARG;
    FP4Q_TRY(check_buffer(codes));
    FP4Q_TRY(check_buffer(scales));
    FP4Q_TRY(check_tensor(out, out_dt, rows, cols, ld_out));
    const int oes = elem_size(out_dt);
    const int DU = 16 / oes;                  // output values per 16-byte chunk
    DequantArgs a{};
    a.codes = codes;
    a.scales = scales;
    a.g_dev = g_dev;
    a.scale_fmt = cfg->scale_fmt;
    a.cols = cols;
    a.units = rows * cols / DU;
    a.units_per_row = cols / DU;
    a.out = out;
    a.ld_out = ld_out;
    a.out_dt = out_dt;
    return device_status(launch_dequant(a, B, oes, grid_for(a.units), (hipStream_t)stream));
}

fp4q_status fp4q_block_mse(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows, int64_t cols,
                           int64_t ld_x, const uint8_t* codes, const uint8_t* scales,
                           const float* g_dev, float* block_mse, void* stream) {
    FP4Q_TRY(check_config(cfg));
    const int B = cfg->block, H = cfg->hadamard;
    FP4Q_TRY(check_dims(rows, cols, B, H));
    FP4Q_TRY(check_g_in(cfg, g_dev));
    if (rows == 0 || cols == 0) return dtype_ok(x_dt) ? FP4Q_OK : FP4Q_ERR_INVALID_ARG;
    FP4Q_TRY(check_tensor(x, x_dt, rows, cols, ld_x));
    FP4Q_TRY(check_buffer(codes));
    FP4Q_TRY(check_buffer(scales));
    FP4Q_TRY(check_buffer(block_mse));
    const int U = 16 / elem_size(x_dt);       // 16-byte chunks of x
    MseArgs a{};
    a.x = x;
    a.ld_x = ld_x;
    a.cols = cols;
    a.units = rows * cols / U;
    a.units_per_row = cols / U;
    a.codes = codes;
    a.scales = scales;
    a.g_dev = g_dev;
    a.scale_fmt = cfg->scale_fmt;
    a.mse = block_mse;
    return device_status(launch_block_mse(a, x_dt, B, H, grid_for(a.units), (hipStream_t)stream));
}

static fp4q_status check_relaxed(const fp4q_config* cfg, const void* w, int w_dt, int64_t rows,
                                 int64_t cols, int64_t ld_w, const uint8_t* scales, const float* g_dev,
                                 const uint16_t* c_f16, int32_t sub_block) {
    FP4Q_TRY(check_config(cfg));
    if (cfg->hadamard != 0) return FP4Q_ERR_UNSUPPORTED;
    const int B = cfg->block;
    if (sub_block != 4 && sub_block != 8 && sub_block != 16 && sub_block != 32) return FP4Q_ERR_SHAPE;
    if (B % sub_block != 0) return FP4Q_ERR_SHAPE;
    FP4Q_TRY(check_dims(rows, cols, B, 0));
    FP4Q_TRY(check_g_in(cfg, g_dev));
    if (rows == 0 || cols == 0) return dtype_ok(w_dt) ? FP4Q_OK : FP4Q_ERR_INVALID_ARG;
    FP4Q_TRY(check_tensor(w, w_dt, rows, cols, ld_w));
    FP4Q_TRY(check_buffer(scales));
    FP4Q_TRY(check_buffer(c_f16));
    return FP4Q_OK;
}

fp4q_status fp4q_relaxed_fakequant_fwd(const fp4q_config* cfg, const void* w, int w_dt, int64_t rows,
                                       int64_t cols, int64_t ld_w, const uint8_t* scales,
                                       const float* g_dev, const uint16_t* c_f16, int32_t sub_block,
                                       void* w_hat, int out_dt, int64_t ld_out, uint8_t* codes,
                                       void* stream) {
    FP4Q_TRY(check_relaxed(cfg, w, w_dt, rows, cols, ld_w, scales, g_dev, c_f16, sub_block));
    if (rows == 0 || cols == 0) return dtype_ok(out_dt) ? FP4Q_OK : FP4Q_ERR_INVALID_ARG;
    FP4Q_TRY(check_tensor(w_hat, out_dt, rows, cols, ld_out));
    if (codes) FP4Q_TRY(check_buffer(codes));
    const int U = 16 / elem_size(w_dt);       // 16-byte chunks of W
    RelaxedArgs a{};
    a.w = w;
    a.ld_w = ld_w;
    a.cols = cols;
    a.units = rows * cols / U;
    a.units_per_row = cols / U;
    a.scales = scales;
    a.g_dev = g_dev;
    a.scale_fmt = cfg->scale_fmt;
    a.c = c_f16;
    a.w_hat = w_hat;
    a.ld_out = ld_out;
    a.out_dt = out_dt;
    a.codes = codes;
    return device_status(
        launch_relaxed_fwd(a, w_dt, cfg->block, sub_block, grid_for(a.units), (hipStream_t)stream));
}

fp4q_status fp4q_relaxed_fakequant_bwd(const fp4q_config* cfg, const void* w, int w_dt, int64_t rows,
                                       int64_t cols, int64_t ld_w, const uint8_t* scales,
                                       const float* g_dev, const uint16_t* c_f16, int32_t sub_block,
                                       const void* grad_out, int g_dt, int64_t ld_g, float* grad_c,
                                       void* stream) {
    FP4Q_TRY(check_relaxed(cfg, w, w_dt, rows, cols, ld_w, scales, g_dev, c_f16, sub_block));
    if (rows == 0 || cols == 0) return dtype_ok(g_dt) ? FP4Q_OK : FP4Q_ERR_INVALID_ARG;
    FP4Q_TRY(check_tensor(grad_out, g_dt, rows, cols, ld_g));
    FP4Q_TRY(check_buffer(grad_c));
    const int U = 16 / elem_size(w_dt);       // 16-byte chunks of W
    RelaxedArgs a{};
    a.w = w;
    a.ld_w = ld_w;
    a.cols = cols;
    a.units = rows * cols / U;
    a.units_per_row = cols / U;
    a.scales = scales;
    a.g_dev = g_dev;
    a.scale_fmt = cfg->scale_fmt;
    a.c = c_f16;
    a.grad = grad_out;
    a.ld_g = ld_g;
    a.g_dt = g_dt;
    a.grad_c = grad_c;
    return device_status(
        launch_relaxed_bwd(a, w_dt, cfg->block, sub_block, grid_for(a.units), (hipStream_t)stream));
}

fp4q_status fp4q_code_histogram(const uint8_t* codes, int64_t rows, int64_t cols, uint64_t* counts,
                                void* stream) {
    if (!counts || rows < 0 || cols < 0) return FP4Q_ERR_INVALID_ARG;
    if ((uintptr_t)counts & 7u) return FP4Q_ERR_ALIGNMENT;
    if (cols % 2 != 0) return FP4Q_ERR_SHAPE;
    const int64_t nbytes = rows * (cols / 2);
    if (nbytes > 0) FP4Q_TRY(check_buffer(codes));
    // few workgroups, each walking many 16-byte chunks: every workgroup ends with one
    // 64-bit atomic per code on the same 128 bytes, which serialise in the cache
    const int64_t chunks = (nbytes + 15) / 16;
    const int grid = (int)std::min<int64_t>(std::max<int64_t>((chunks + 2047) / 2048, 1), 256);
    return device_status(launch_code_hist(codes, nbytes, reinterpret_cast<unsigned long long*>(counts), grid,
                                          (hipStream_t)stream));
}

size_t fp4q_mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0) return 0;
    return mxfp4_gemm_workspace(M, N, K);
}

fp4q_status fp4q_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                            const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c, int c_dt,
                            int64_t ldc, void* workspace, void* stream) {
    if (M < 0 || N < 0 || K < 0) return FP4Q_ERR_INVALID_ARG;
    if (c_dt != FP4Q_F32 && c_dt != FP4Q_BF16) return FP4Q_ERR_INVALID_ARG;
    if (K % 32 != 0) return FP4Q_ERR_SHAPE;
    if (M == 0 || N == 0) return FP4Q_OK;
    if (K == 0 || ldc < N) return FP4Q_ERR_SHAPE;
    const uint64_t kp = (uint64_t)(K + 255) / 256 * 256;      // K as the matrix cores run it
    if ((uint64_t)M * (kp / 2) >= (1ull << 32) || (uint64_t)N * (kp / 2) >= (1ull << 32)) return FP4Q_ERR_SHAPE;
    if (!c || !a_codes || !a_scales || !b_codes || !b_scales || !workspace) return FP4Q_ERR_INVALID_ARG;
    if (!aligned16(c) || (ldc * elem_size(c_dt)) % 16 != 0) return FP4Q_ERR_ALIGNMENT;
    if (!aligned16(a_codes) || !aligned16(b_codes) || ((uintptr_t)a_scales & 3u) || ((uintptr_t)b_scales & 3u) ||
        ((uintptr_t)workspace & 255u))
        return FP4Q_ERR_ALIGNMENT;
    return device_status(launch_mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, c, c_dt, ldc, workspace,
                                           (hipStream_t)stream));
}

size_t fp4q_nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return 0;
    return nvfp4_gemm_workspace(M, N, K);
}

fp4q_status fp4q_nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g,
                            const uint8_t* b_codes, const uint8_t* b_scales, const float* b_g, int64_t M, int64_t N,
                            int64_t K, void* c, int c_dt, int64_t ldc, void* workspace, void* stream) {
    if (M < 0 || N < 0 || K < 0) return FP4Q_ERR_INVALID_ARG;
    if (c_dt != FP4Q_F32 && c_dt != FP4Q_BF16) return FP4Q_ERR_INVALID_ARG;
    if (K % 16 != 0) return FP4Q_ERR_SHAPE;
    if (M == 0 || N == 0) return FP4Q_OK;
    if (K == 0 || ldc < N) return FP4Q_ERR_SHAPE;
    const uint64_t kp = (uint64_t)(K + 255) / 256 * 256;      // K as the matrix cores run it
    if ((uint64_t)M * (kp / 2) >= (1ull << 32) || (uint64_t)N * (kp / 2) >= (1ull << 32)) return FP4Q_ERR_SHAPE;
    if (!c || !a_codes || !a_scales || !b_codes || !b_scales || !workspace) return FP4Q_ERR_INVALID_ARG;
    if (!aligned16(c) || (ldc * elem_size(c_dt)) % 16 != 0) return FP4Q_ERR_ALIGNMENT;
    if (!aligned16(a_codes) || !aligned16(b_codes) || ((uintptr_t)a_scales & 3u) || ((uintptr_t)b_scales & 3u) ||
        ((uintptr_t)workspace & 255u) || ((uintptr_t)a_g & 3u) || ((uintptr_t)b_g & 3u))
        return FP4Q_ERR_ALIGNMENT;
    return device_status(launch_nvfp4_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, M, N, K, c, c_dt, ldc,
                                           workspace, (hipStream_t)stream));
}

}  // extern "C"
