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
// 128 x 128 quarter (8 x 8 MFMA fragments, 256 fp32 accumulators per lane).
// K advances 128 at a time: the A and B slices (256 rows x 64 bytes each) and
// their scale words go global -> registers -> LDS, double-buffered, so the
// next slice's loads are in flight while the MFMAs of the current one run.
// LDS rows are padded to 80 bytes, which makes the 16-byte fragment reads of
// 16 consecutive rows conflict-free.
#include "fp4q_launch.hpp"

namespace fp4q_dev {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGemmTileM = 256;
constexpr int kGemmTileN = 256;
constexpr int kGemmK = 128;                      // K per step: 4 scale blocks
constexpr int kGemmRowBytes = kGemmK / 2;        // code bytes of one row per step
constexpr int kGemmLdsRow = kGemmRowBytes + 16;  // padded LDS row

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

__global__ __launch_bounds__(256, 1) void k_mxfp4_gemm(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][kGemmTileM * kGemmLdsRow];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][kGemmTileN * kGemmLdsRow];
    __shared__ uint32_t sAs[2][kGemmTileM];    // the 4 scale bytes of a row's K step
    __shared__ uint32_t sBs[2][kGemmTileN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
    const int64_t m0 = (int64_t)tm * kGemmTileM, n0 = (int64_t)tn * kGemmTileN;
    const int64_t kbytes = p.K / 2, kscales = p.K / 32;
    const int nk = (int)(p.K / kGemmK);

    // staging registers: 4 chunks of 16 bytes of A and of B, one scale word each
    uint4 ra[4], rb[4];
    uint32_t rsa, rsb;
    auto load_stage = [&](int ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, row = c >> 2, part = c & 3;
            // rows past the matrix read its last row; their results are not stored
            const int64_t ga = min<int64_t>(m0 + row, p.M - 1), gb = min<int64_t>(n0 + row, p.N - 1);
            ra[i] = *reinterpret_cast<const uint4*>(p.a + ga * kbytes + (int64_t)ks * kGemmRowBytes + part * 16);
            rb[i] = *reinterpret_cast<const uint4*>(p.b + gb * kbytes + (int64_t)ks * kGemmRowBytes + part * 16);
        }
        const int64_t ga = min<int64_t>(m0 + tid, p.M - 1), gb = min<int64_t>(n0 + tid, p.N - 1);
        rsa = *reinterpret_cast<const uint32_t*>(p.as + ga * kscales + (int64_t)ks * 4);
        rsb = *reinterpret_cast<const uint32_t*>(p.bs + gb * kscales + (int64_t)ks * 4);
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i, row = c >> 2, part = c & 3;
            *reinterpret_cast<uint4*>(&sA[buf][row * kGemmLdsRow + part * 16]) = ra[i];
            *reinterpret_cast<uint4*>(&sB[buf][row * kGemmLdsRow + part * 16]) = rb[i];
        }
        sAs[buf][tid] = rsa;
        sBs[buf][tid] = rsb;
    };

    v4f acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int fr = lane & 15, kb = lane >> 4;    // fragment row and K block of this lane
    load_stage(0);
    store_stage(0);
    __syncthreads();
#pragma unroll 1
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) load_stage(ks + 1);
        v8i bf[8];
        int bsc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = wn * 128 + 16 * j + fr;
            bf[j] = frag_of(*reinterpret_cast<const uint4*>(&sB[buf][col * kGemmLdsRow + kb * 16]));
            bsc[j] = (int)((sBs[buf][col] >> (8 * kb)) & 0xFFu);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = wm * 128 + 16 * i + fr;
            const v8i af = frag_of(*reinterpret_cast<const uint4*>(&sA[buf][row * kGemmLdsRow + kb * 16]));
            const int asc = (int)((sAs[buf][row] >> (8 * kb)) & 0xFFu);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 4, 4, 0, asc, 0,
                                                                             bsc[j]);
        }
        if (ks + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // result lane l holds column l % 16 of rows 4 (l / 16) .. + 3 of each fragment
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
