// gemm.hip -- FP4 GEMM on MXFP4 operands with gfx950's block-scaled MFMA
// (the FP4 matrix products of the MR-GPTQ page, section 2.3, which its
// QuTLASS kernels run on Blackwell; here on CDNA4 matrix cores).
//
// C[M, N] = dq(A) dq(B)^T with A codes [M, K/2] + E8M0 scales [M, K/32] and
// B codes [N, K/2] + scales [N, K/32]: exactly the layouts fp4q_quantize
// writes for {E8M0, block 32}.  v_mfma_scale_f32_16x16x128_f8f6f4 with both
// operands in E2M1 multiplies a 16 x 128 A fragment by a 16 x 128 B fragment
// and applies one E8M0 scale per operand lane: lane l holds row l % 16 and the
// 32 consecutive K values of block l / 16, which is the 16 contiguous code
// bytes of that row and block, and its block's scale byte.  The result lane l
// holds column l % 16 of rows 4 (l / 16) .. 4 (l / 16) + 3.
//
// Tiling: a workgroup of 4 waves computes a 256 x 256 tile of C, each wave a
// 128 x 128 quarter (8 x 8 MFMA fragments, 256 fp32 accumulators per lane,
// which the compiler keeps in the accumulation registers).  K advances 128
// at a time; each K slice (256 rows x 64 code bytes of A and of B, and their
// scale words) goes straight from global memory into LDS with the direct
// loads, 4 slices deep, so three slices are loading while the MFMAs consume
// the fourth.  In LDS the fragments lie in the order the MFMA lanes read
// them, so every fragment read is one linear, conflict-free 1 KB read.
#include "fp4q_launch.hpp"

namespace fp4q_dev {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGemmTileM = 256;
constexpr int kGemmTileN = 256;
constexpr int kGemmK = 128;                      // K per step: 4 scale blocks
constexpr int kGemmRowBytes = kGemmK / 2;        // code bytes of one row per step

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* as;
    const uint8_t* b;
    const uint8_t* bs;
    int64_t M, N, K;
    void* c;
    int c_dt;
    int64_t ldc;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ v8i frag_of(const uint4 v) {
    v8i f = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    return f;
}

// Tile order: workgroups go round-robin to the 8 XCDs (blockIdx % 8), each
// with its own L2.  Give XCD x a contiguous run of tiles, and walk tiles in
// groups of 8 tile rows, so the 32 compute units of one XCD share few A and
// B panels.
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, int& tm, int& tn) {
    const int ntiles = p.tiles_m * p.tiles_n;
    const int per_xcd = (ntiles + 7) / 8;
    const int bid = blockIdx.x;
    int t = (bid % 8) * per_xcd + bid / 8;
    if (t >= ntiles) t = bid;                    // the uneven tail keeps the plain order
    constexpr int G = 8;
    const int in_group = G * p.tiles_n;
    const int first_m = (t / in_group) * G;
    const int gsize = min(G, p.tiles_m - first_m);
    tm = first_m + (t % in_group) % gsize;
    tn = (t % in_group) / gsize;
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kGemmStages = 4;                   // K slices in flight
constexpr int kFragBytes = 64 * 16;              // one MFMA operand fragment
constexpr int kSliceBytes = 16 * kFragBytes;     // 256 rows x 64 code bytes
// Direct global -> LDS loads each wave issues per slice: 4 A fragments,
// 4 B fragments, one A-scale and one B-scale dword per lane.
constexpr int kDmaPerSlice = 10;

// Wait until at most n of this wave's direct loads are outstanding (the
// compiler's own waits would wait for all of them), then a workgroup barrier
// without the fence of __syncthreads (the fence would also drain them).
template <int N>
__device__ __forceinline__ void gemm_wait_barrier() {
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    __builtin_amdgcn_s_barrier();
}

// Issue the direct loads of K slice ks into LDS stage buffers.  LDS holds
// fragments in the order the MFMA reads them: fragment f (rows 16 f .. 16 f
// + 15 of the slice) at f * 1024, lane l's 16 bytes (row 16 f + l % 16, K
// block l / 16) at + 16 l, so a fragment read is one linear 1 KB ds_read.
// Scales: row-major words (the 4 K-block scale bytes of a row).  Rows past
// the matrix read its last row; their results are not stored.
__device__ __forceinline__ void gemm_issue(const GemmArgs& p, int64_t m0, int64_t n0, int ks, uint8_t* sa,
                                           uint8_t* sb, uint32_t* ssa, uint32_t* ssb, int wave, int lane) {
    const int64_t kbytes = p.K / 2, kscales = p.K / 32;
    const int64_t koff = (int64_t)ks * kGemmRowBytes + (lane >> 4) * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int f = wave * 4 + q;
        const int r = 16 * f + (lane & 15);
        const int64_t ra = min<int64_t>(m0 + r, p.M - 1), rb = min<int64_t>(n0 + r, p.N - 1);
        __builtin_amdgcn_global_load_lds((const void*)(p.a + ra * kbytes + koff), (lds_void_ptr)(sa + f * kFragBytes),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(p.b + rb * kbytes + koff), (lds_void_ptr)(sb + f * kFragBytes),
                                         16, 0, 0);
    }
    const int r = wave * 64 + lane;
    const int64_t ra = min<int64_t>(m0 + r, p.M - 1), rb = min<int64_t>(n0 + r, p.N - 1);
    __builtin_amdgcn_global_load_lds((const void*)(p.as + ra * kscales + (int64_t)ks * 4),
                                     (lds_void_ptr)(ssa + wave * 64), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(p.bs + rb * kscales + (int64_t)ks * 4),
                                     (lds_void_ptr)(ssb + wave * 64), 4, 0, 0);
}

// One K slice in LDS.  Four of them, as four separate objects: the compiler
// tracks the direct loads per LDS object, so reading one stage does not make
// it wait for the loads still filling the others.
struct GemmSlice {
    uint8_t a[kSliceBytes];
    uint8_t b[kSliceBytes];
    uint32_t as[kGemmTileM];
    uint32_t bs[kGemmTileN];
};
__shared__ __attribute__((aligned(1024))) GemmSlice g_slice0;
__shared__ __attribute__((aligned(1024))) GemmSlice g_slice1;
__shared__ __attribute__((aligned(1024))) GemmSlice g_slice2;
__shared__ __attribute__((aligned(1024))) GemmSlice g_slice3;

template <int S>
__device__ __forceinline__ GemmSlice& gemm_slice() {
    if constexpr (S == 0) return g_slice0;
    else if constexpr (S == 1) return g_slice1;
    else if constexpr (S == 2) return g_slice2;
    else return g_slice3;
}

template <int S>
__device__ __forceinline__ void gemm_issue_slice(const GemmArgs& p, int64_t m0, int64_t n0, int ks, int wave,
                                                 int lane) {
    GemmSlice& sl = gemm_slice<S>();
    gemm_issue(p, m0, n0, ks, sl.a, sl.b, sl.as, sl.bs, wave, lane);
}

// One K step on stage S (slice ks): wait for it, refill the stage the
// previous step used with slice ks + 3, and run the 64 MFMAs of this wave.
// The refill is issued on every step, also past the last slice (it then
// reloads the last slice into a stage nobody reads again): with the direct
// loads outside any branch, the compiler knows which stage each pending load
// fills and adds no wait of its own before the fragment reads.
template <int S>
__device__ __forceinline__ void gemm_step(const GemmArgs& p, int64_t m0, int64_t n0, int ks, int nk, int wave,
                                          int lane, int wm, int wn, v4f (&acc)[8][8]) {
    gemm_wait_barrier<2 * kDmaPerSlice>();
    gemm_issue_slice<(S + kGemmStages - 1) % kGemmStages>(p, m0, n0, min(ks + kGemmStages - 1, nk - 1), wave, lane);
    if (ks >= nk) return;
    const GemmSlice& sl = gemm_slice<S>();
    const int fr = lane & 15, kb = lane >> 4;    // fragment row and K block of this lane
    v8i bf[8];
    int bsc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int f = wn * 8 + j;
        bf[j] = frag_of(*reinterpret_cast<const uint4*>(&sl.b[f * kFragBytes + lane * 16]));
        bsc[j] = (int)((sl.bs[16 * f + fr] >> (8 * kb)) & 0xFFu);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int f = wm * 8 + i;
        const v8i af = frag_of(*reinterpret_cast<const uint4*>(&sl.a[f * kFragBytes + lane * 16]));
        const int asc = (int)((sl.as[16 * f + fr] >> (8 * kb)) & 0xFFu);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 4, 4, 0, asc, 0, bsc[j]);
    }
}

__global__ __launch_bounds__(256, 1) void k_mxfp4_gemm(GemmArgs p) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    gemm_tile(p, tm, tn);
    const int64_t m0 = (int64_t)tm * kGemmTileM, n0 = (int64_t)tn * kGemmTileN;
    const int nk = (int)(p.K / kGemmK);

    v4f acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // slices 0 .. 2 in flight before the first step (a short K reloads its last slice)
    gemm_issue_slice<0>(p, m0, n0, 0, wave, lane);
    gemm_issue_slice<1>(p, m0, n0, min(1, nk - 1), wave, lane);
    gemm_issue_slice<2>(p, m0, n0, min(2, nk - 1), wave, lane);
#pragma unroll 1
    for (int ks = 0; ks < nk; ks += kGemmStages) {
        gemm_step<0>(p, m0, n0, ks, nk, wave, lane, wm, wn, acc);
        gemm_step<1>(p, m0, n0, ks + 1, nk, wave, lane, wm, wn, acc);
        gemm_step<2>(p, m0, n0, ks + 2, nk, wave, lane, wm, wn, acc);
        gemm_step<3>(p, m0, n0, ks + 3, nk, wave, lane, wm, wn, acc);
    }
    gemm_wait_barrier<0>();                      // no direct load outlives the kernel

    // result lane l holds column l % 16 of rows 4 (l / 16) .. + 3 of each fragment
    const int fr = lane & 15, kb = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t col = n0 + wn * 128 + 16 * j + fr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 128 + 16 * i + 4 * kb + r;
                if (row < p.M && col < p.N) {
                    if (p.c_dt == DT_F32) reinterpret_cast<float*>(p.c)[row * p.ldc + col] = acc[i][j][r];
                    else reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + col] =
                        (uint16_t)(pack_bf16x2(acc[i][j][r], 0.0f) & 0xFFFFu);
                }
            }
        }
}

hipError_t launch_mxfp4_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs, int64_t M,
                             int64_t N, int64_t K, void* c, int c_dt, int64_t ldc, hipStream_t s) {
    GemmArgs p{};
    p.a = a;
    p.as = as;
    p.b = b;
    p.bs = bs;
    p.M = M;
    p.N = N;
    p.K = K;
    p.c = c;
    p.c_dt = c_dt;
    p.ldc = ldc;
    p.tiles_m = (int)((M + kGemmTileM - 1) / kGemmTileM);
    p.tiles_n = (int)((N + kGemmTileN - 1) / kGemmTileN);
    hipLaunchKernelGGL(k_mxfp4_gemm, dim3((unsigned)p.tiles_m * p.tiles_n), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace fp4q_dev
