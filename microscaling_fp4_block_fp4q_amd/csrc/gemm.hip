// gemm.hip -- FP4 GEMM on MXFP4 operands with gfx950's block-scaled MFMA
// (the FP4 matrix products of the MR-GPTQ page, section 2.3, which its
// QuTLASS kernels run on Blackwell; here on CDNA4 matrix cores).
//
// C[M, N] = dq(A) dq(B)^T with A codes [M, K/2] + E8M0 scales [M, K/32] and
// B codes [N, K/2] + scales [N, K/32]: the layouts fp4q_quantize writes for
// {E8M0, block 32}.
//
// Matrix core: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1
// (a rate probe on gfx950: 8.6 PFLOP/s for this shape with E2M1 operands,
// 4.6 for the 16 x 16 x 128 one, which runs E2M1 at the E4M3 rate).
// Operand lane l holds row l % 32 of a 32-row fragment and the 32 K values
// of K block l / 32 of the 64-wide K substep (16 code bytes), and a scale
// dword whose byte op_sel is that block's scale.
// The result lane l holds column l % 32 of the second operand's rows and
// rows 8 (r / 4) + 4 (l / 32) + r % 4 of the first's.  B goes first, so a
// lane ends up with one row of C and 4 consecutive columns per r / 4.
//
// Tiling: a workgroup of 4 waves computes a 256 x 256 tile of C, each wave a
// 128 x 128 quarter (4 x 4 fragments, 256 fp32 accumulators per lane in the
// accumulation registers).  K advances 256 per step.  A step's codes (256
// rows x 128 bytes of A and of B) go straight from global memory into one of
// two LDS stages with the direct loads, each load reading 8 whole 128-byte
// rows; the next step's load runs while the current step computes.  Within a
// row the eight 16-byte chunks are stored XOR-swizzled by the row pair, so
// both the direct-load writes and the fragment reads are free of bank
// conflicts (a 16-byte read serves 16 lanes at a time from the 64 banks,
// i.e. two 128-byte rows).
//
// Scales: a small pass first rewrites each operand's [rows, K/32] scale bytes
// into the per-lane dwords the MFMA takes (for fragment f, step t, lane l:
// the scales of K blocks 8 t + 2 h + l / 32 of row 32 f + l % 32, h = 0..3),
// so each step's scales are one coalesced 256-byte load per fragment.
//
// Epilogue: the accumulators go through LDS (per wave, a 32-row block at a
// time) and leave as 16-byte stores of whole row pieces.
#include "fp4q_launch.hpp"

namespace fp4q_dev {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kGemmTile = 256;                   // tile rows of A and of B
constexpr int kGemmStepK = 256;                  // K per step: 8 scale blocks
constexpr int kGemmRowBytes = kGemmStepK / 2;    // code bytes of a row per step
constexpr int kGemmOperandBytes = kGemmTile * kGemmRowBytes;   // 32 KB
constexpr int kGemmDmaPerOperand = kGemmOperandBytes / 1024 / 4;  // direct loads per wave

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* b;
    const uint32_t* sa;                          // shuffled scale dwords
    const uint32_t* sb;
    int64_t M, N, K;
    void* c;
    int c_dt;
    int64_t ldc;
    int tiles_m, tiles_n;
    int steps;                                   // K / 256
    int frags_a, frags_b;                        // ceil(M / 32), ceil(N / 32)
};

// ---------------------------------------------------------------------------
// Scale shuffle: out[(f * T + t) * 64 + l] = scale bytes of K blocks
// 8 t + l / 32 + {0, 2, 4, 6} of row 32 f + l % 32 (byte h = block
// 8 t + 2 h + l / 32); rows past the matrix get 127 (2^0).
// ---------------------------------------------------------------------------
__global__ void k_gemm_shuffle_scales(const uint8_t* __restrict__ s, int64_t rows, int64_t kblocks, int steps,
                                      int64_t total, uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int l = (int)(i & 63);
    const int64_t ft = i >> 6;
    const int t = (int)(ft % steps);
    const int64_t row = (ft / steps) * 32 + (l & 31);
    uint32_t w = 0x7F7F7F7Fu;
    if (row < rows) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(s + row * kblocks + 8 * t);
        const uint32_t lo = p[0], hi = p[1];     // blocks 8 t .. 8 t + 7
        // bytes l / 32 and 2 + l / 32 of lo, then of hi
        w = __builtin_amdgcn_perm(hi, lo, (l >> 5) ? 0x07050301u : 0x06040200u);
    }
    out[i] = w;
}

// Tile order: workgroups go round-robin to the 8 XCDs (blockIdx % 8), each
// with its own L2.  XCD x runs the workgroups x, x + 8, ...: ntiles / 8 of
// them, one more for x < ntiles % 8; give it that many consecutive tiles,
// starting after the runs of the XCDs before it (a bijection onto the
// tiles).  Tiles are numbered in groups of 8 tile rows, so the 32 compute
// units of one XCD share few A and B panels.
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, int& tm, int& tn) {
    const int ntiles = p.tiles_m * p.tiles_n;
    const int bid = blockIdx.x, x = bid % 8, q = ntiles / 8, r = ntiles % 8;
    const int t = x * q + min(x, r) + bid / 8;
    constexpr int G = 8;
    const int in_group = G * p.tiles_n;
    const int first_m = (t / in_group) * G;
    const int gsize = min(G, p.tiles_m - first_m);
    tm = first_m + (t % in_group) % gsize;
    tn = (t % in_group) / gsize;
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// and all its LDS reads have completed, then a workgroup barrier, fenced for
// the compiler only: __syncthreads' fence would also wait for every load.
// The compiler does not know that the barrier is what makes the other waves'
// direct loads visible, so the empty asm statements keep it from moving
// memory accesses across.
template <int N>
__device__ __forceinline__ void gemm_wait_barrier() {
    static_assert(N < 64, "vmcnt field");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One step's codes.  Two stages, as two separate objects: the compiler tracks
// the direct loads per LDS object, so reading one stage does not make it wait
// for the loads still filling the other.  Row r's chunk c (16 bytes, K block
// c of the step) sits at r * 128 + 16 (c ^ (r / 2 % 8)).
struct GemmStage {
    uint8_t a[kGemmOperandBytes];
    uint8_t b[kGemmOperandBytes];
};
__shared__ __attribute__((aligned(1024))) GemmStage g_stage0;
__shared__ __attribute__((aligned(1024))) GemmStage g_stage1;

template <int S>
__device__ __forceinline__ GemmStage& gemm_stage() {
    if constexpr (S == 0) return g_stage0;
    else return g_stage1;
}

// Per-lane state fixed for the whole K loop.
struct GemmLane {
    __amdgpu_buffer_rsrc_t ra, rb;               // buffer descriptors of the A and B codes
    uint32_t oa[kGemmDmaPerOperand], ob[kGemmDmaPerOperand];   // direct-load byte offsets in them
    const uint32_t* sa;                          // scale dwords of this wave's first A fragment, step 0
    const uint32_t* sb;
};

// Direct load q of wave w covers tile rows 8 (8 w + q) .. + 7, 1 KB of LDS:
// lane l writes 16 bytes at + 16 l, i.e. row 8 (8 w + q) + l / 8, slot l % 8,
// which holds chunk (l % 8) ^ (row / 2 % 8) - the 8 lanes of a row read its
// whole 128 bytes.  Rows past the matrix read its last row (results not
// stored).
__device__ __forceinline__ GemmLane gemm_lane(const GemmArgs& p, int64_t m0, int64_t n0, int wave, int lane,
                                              int wm, int wn) {
    const int64_t kbytes = p.K / 2;
    const int sub = lane >> 3;
    GemmLane L;
    // raw buffers (stride 0) over the code arrays; sizes are below 2^32
    // bytes, and every offset below stays inside them
    L.ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.a, (short)0, (int)(uint32_t)(p.M * kbytes), 0x00020000);
    L.rb = __builtin_amdgcn_make_buffer_rsrc((void*)p.b, (short)0, (int)(uint32_t)(p.N * kbytes), 0x00020000);
#pragma unroll
    for (int q = 0; q < kGemmDmaPerOperand; ++q) {
        const int r = 8 * (kGemmDmaPerOperand * wave + q) + sub;
        const int chunk = (lane & 7) ^ ((r >> 1) & 7);
        L.oa[q] = (uint32_t)(min<int64_t>(m0 + r, p.M - 1) * kbytes + 16 * chunk);
        L.ob[q] = (uint32_t)(min<int64_t>(n0 + r, p.N - 1) * kbytes + 16 * chunk);
    }
    L.sa = p.sa + (int64_t)((m0 + 128 * wm) / 32) * p.steps * 64 + lane;
    L.sb = p.sb + (int64_t)((n0 + 128 * wn) / 32) * p.steps * 64 + lane;
    return L;
}

// The 8 scale dwords of one step for this wave: 4 A fragments, 4 B
// fragments (fragments past the matrix take its last one).
struct GemmScales {
    int a[4], b[4];
};

// Issue step t's direct loads of the codes into stage S: buffer loads with
// the per-lane offset fixed for the loop and the step's K offset in a scalar
// register, so a load needs no address arithmetic of its own.
template <int S, int Q0 = 0, int Q1 = kGemmDmaPerOperand>
__device__ __forceinline__ void gemm_issue_codes(const GemmLane& L, int t, int wave) {
    GemmStage& st = gemm_stage<S>();
    const uint32_t koff = (uint32_t)t * kGemmRowBytes;
#pragma unroll
    for (int q = Q0; q < Q1; ++q) {
        const int j = kGemmDmaPerOperand * wave + q;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(L.ra, (lds_void_ptr)(st.a + j * 1024), 16, L.oa[q], koff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rb, (lds_void_ptr)(st.b + j * 1024), 16, L.ob[q], koff, 0, 0);
    }
}

// Load step t's scale dwords into sc.
__device__ __forceinline__ void gemm_issue_scales(const GemmArgs& p, const GemmLane& L, int t, int64_t fa0,
                                                  int64_t fb0, GemmScales& sc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t fa = min<int64_t>(fa0 + i, p.frags_a - 1) - fa0;
        const int64_t fb = min<int64_t>(fb0 + i, p.frags_b - 1) - fb0;
        sc.a[i] = (int)L.sa[(fa * p.steps + t) * 64];
        sc.b[i] = (int)L.sb[(fb * p.steps + t) * 64];
    }
}

// One 16-byte fragment read from LDS as a single vector load, widened to the
// 8-dword operand (E2M1 uses the low 4 dwords).
__device__ __forceinline__ v8i frag_at(const uint8_t* p) {
    const v4i v = *reinterpret_cast<const v4i*>(p);
    v8i f = {v.x, v.y, v.z, v.w, 0, 0, 0, 0};
    return f;
}

// Fragments of one K substep h: A rows 128 wm + 32 i + l % 32, B rows
// 128 wn + 32 j + l % 32, chunk 2 h + l / 32.
struct GemmFrags {
    v8i a[4], b[4];
};

template <int S>
__device__ __forceinline__ void gemm_read(GemmFrags& fr, int h, int lane, int wm, int wn) {
    const GemmStage& st = gemm_stage<S>();
    const int r = lane & 31;
    const int slot = (2 * h + (lane >> 5)) ^ ((r >> 1) & 7);
    const int off = r * kGemmRowBytes + 16 * slot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fr.a[i] = frag_at(st.a + ((128 * wm + 32 * i) * kGemmRowBytes + off));
        fr.b[i] = frag_at(st.b + ((128 * wn + 32 * i) * kGemmRowBytes + off));
    }
}

template <int H>
__device__ __forceinline__ void gemm_mfma(const GemmFrags& fr, const GemmScales& sc, v16f (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr.b[j], fr.a[i], acc[i][j], 4, 4, H,
                                                                        sc.b[j], H, sc.a[i]);
}

// Scheduling: one wave per SIMD cannot run ahead of its matrix pipe (an MFMA
// issues only once the previous one is under way), so loads placed after a
// run of MFMAs would show their latency in full.  The group barriers below
// put one fragment read (DS) or direct load (VMEM) after each MFMA.
template <int NREAD>
__device__ __forceinline__ void gemm_sched_reads() {
#pragma unroll
    for (int k = 0; k < NREAD; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16 - NREAD, 0);
}

constexpr int kHalfDma = kGemmDmaPerOperand / 2;

// Step t on stage S with scales sc; f0 holds substep 0's fragments (read
// during the previous step).  Substeps 0..2 each read the next substep's
// fragments while their MFMAs run; substep 0 also issues the second half of
// step t + 1's direct loads (into the other stage, free since the previous
// barrier).  Then wait for step t + 1's loads and this wave's reads, pass the
// barrier (every wave is done with stage S and step t + 1 is in LDS), and
// during substep 3 issue the first half of step t + 2's loads into stage S
// and read step t + 1's substep-0 fragments into f0; last, step t + 2's
// scales into sc.  Spreading the direct loads over two substeps keeps the
// four waves, which leave the barrier together, from queueing 64 loads at
// once.  The loads run on every step, also past the last one (they then
// reload the last step), so they stay outside any branch and the compiler
// adds no wait of its own before the fragment reads.
template <int S>
__device__ __forceinline__ void gemm_step(const GemmArgs& p, const GemmLane& L, int t, int wave, int lane, int wm,
                                          int wn, int64_t fa0, int64_t fb0, GemmScales& sc, GemmFrags& f0,
                                          v16f (&acc)[4][4]) {
    GemmFrags f1;
    // substep 0: the second half of step t + 1's direct loads into the other stage
    gemm_issue_codes<S ^ 1, kHalfDma, kGemmDmaPerOperand>(L, min(t + 1, p.steps - 1), wave);
    gemm_read<S>(f1, 1, lane, wm, wn);
    gemm_mfma<0>(f0, sc, acc);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // direct load
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    gemm_read<S>(f0, 2, lane, wm, wn);
    gemm_mfma<1>(f1, sc, acc);
    gemm_sched_reads<8>();
    __builtin_amdgcn_sched_barrier(0);
    gemm_read<S>(f1, 3, lane, wm, wn);
    gemm_mfma<2>(f0, sc, acc);
    gemm_sched_reads<8>();
    __builtin_amdgcn_sched_barrier(0);
    gemm_wait_barrier<0>();
    gemm_issue_codes<S, 0, kHalfDma>(L, min(t + 2, p.steps - 1), wave);
    gemm_read<S ^ 1>(f0, 0, lane, wm, wn);
    gemm_mfma<3>(f1, sc, acc);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // direct load
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    gemm_issue_scales(p, L, min(t + 2, p.steps - 1), fa0, fb0, sc);
    __builtin_amdgcn_sched_barrier(0);
}

// Store a wave's 128 x 128 quarter (rows r0.., columns c0.. of C) through
// its own LDS region, 32 rows at a time.  Lane l holds row 32 i + l % 32 and
// columns 32 j + 8 g + 4 (l / 32) + 0..3 in acc[i][j][4 g ..].  In LDS the
// 16-byte chunks of a row are XOR-swizzled by the row.
template <class T>
__device__ __forceinline__ void gemm_store(const GemmArgs& p, const v16f (&acc)[4][4], uint8_t* buf, int64_t r0,
                                           int64_t c0, int lane, bool full) {
    constexpr int kVals = 16 / sizeof(T);        // values per 16-byte chunk
    constexpr int kRowChunks = 128 / kVals;      // chunks per 128-column row
    constexpr int kRowBytes = 128 * sizeof(T);
    constexpr int kRowsPerPass = 64 / kRowChunks;
    const int rr = lane & 31, hi = lane >> 5;
    T* c = reinterpret_cast<T*>(p.c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * j + 8 * g + 4 * hi;           // first of the lane's 4 columns
                const int chunk = col / kVals, part = col % kVals;
                uint8_t* dst = buf + rr * kRowBytes + 16 * (chunk ^ (rr % kRowChunks)) + part * (int)sizeof(T);
                if constexpr (sizeof(T) == 4) {
                    *reinterpret_cast<v4i*>(dst) = v4i{__float_as_int(acc[i][j][4 * g]),
                                                       __float_as_int(acc[i][j][4 * g + 1]),
                                                       __float_as_int(acc[i][j][4 * g + 2]),
                                                       __float_as_int(acc[i][j][4 * g + 3])};
                } else {
                    *reinterpret_cast<v2i*>(dst) =
                        v2i{(int)pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                            (int)pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
                }
            }
        // all reads of the block first, then the stores: one wait for LDS
        constexpr int kPasses = 32 / kRowsPerPass;
        v4i v[kPasses];
#pragma unroll
        for (int pass = 0; pass < kPasses; ++pass) {
            const int row = kRowsPerPass * pass + lane / kRowChunks, q = lane % kRowChunks;
            v[pass] = *reinterpret_cast<const v4i*>(buf + row * kRowBytes + 16 * (q ^ (row % kRowChunks)));
        }
#pragma unroll
        for (int pass = 0; pass < kPasses; ++pass) {
            const int row = kRowsPerPass * pass + lane / kRowChunks, q = lane % kRowChunks;
            const int64_t grow = r0 + 32 * i + row, gcol = c0 + q * kVals;
            T* out = c + grow * p.ldc + gcol;
            if (full || (grow < p.M && gcol + kVals <= p.N)) {
                *reinterpret_cast<v4i*>(out) = v[pass];
            } else if (grow < p.M) {
                const T* e = reinterpret_cast<const T*>(&v[pass]);
                for (int k = 0; k < kVals; ++k)
                    if (gcol + k < p.N) out[k] = e[k];
            }
        }
    }
}

// PARITY = steps % 2: an odd step count runs its first step ahead of the
// pairs, so the loop body is a whole number of stage pairs.
template <int PARITY>
__global__ __launch_bounds__(256, 1) void k_mxfp4_gemm(GemmArgs p) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS addresses in scalars
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    gemm_tile(p, tm, tn);
    const int64_t m0 = (int64_t)tm * kGemmTile, n0 = (int64_t)tn * kGemmTile;
    const int64_t fa0 = (m0 + 128 * wm) / 32, fb0 = (n0 + 128 * wn) / 32;
    const int nt = p.steps;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    // step 0 and the first half of step 1 in flight (a single step reloads
    // itself), wait for step 0
    const GemmLane L = gemm_lane(p, m0, n0, wave, lane, wm, wn);
    GemmScales s0, s1;
    gemm_issue_codes<0>(L, 0, wave);
    gemm_issue_scales(p, L, 0, fa0, fb0, s0);
    __builtin_amdgcn_sched_barrier(0);           // keep step 0's loads ahead of the wait count
    gemm_issue_codes<1, 0, kHalfDma>(L, min(1, nt - 1), wave);
    gemm_issue_scales(p, L, min(1, nt - 1), fa0, fb0, s1);
    __builtin_amdgcn_sched_barrier(0);
    gemm_wait_barrier<kGemmDmaPerOperand + 8>();    // all but step 1's half and its 8 scale loads
    GemmFrags f0;
    gemm_read<0>(f0, 0, lane, wm, wn);
    if constexpr (PARITY == 1) {
        gemm_step<0>(p, L, 0, wave, lane, wm, wn, fa0, fb0, s0, f0, acc);
#pragma unroll 1
        for (int t = 1; t < nt; t += 2) {
            gemm_step<1>(p, L, t, wave, lane, wm, wn, fa0, fb0, s1, f0, acc);
            gemm_step<0>(p, L, t + 1, wave, lane, wm, wn, fa0, fb0, s0, f0, acc);
        }
    } else {
#pragma unroll 1
        for (int t = 0; t < nt; t += 2) {
            gemm_step<0>(p, L, t, wave, lane, wm, wn, fa0, fb0, s0, f0, acc);
            gemm_step<1>(p, L, t + 1, wave, lane, wm, wn, fa0, fb0, s1, f0, acc);
        }
    }
    // The last step waited for every load it issued but one step's worth,
    // and re-issued loads past the end: drain them before reusing stage 0.
    gemm_wait_barrier<0>();
    uint8_t* buf = reinterpret_cast<uint8_t*>(&g_stage0) + wave * (32 * 128 * 4);
    const int64_t r0 = m0 + 128 * wm, c0 = n0 + 128 * wn;
    const bool full = m0 + kGemmTile <= p.M && n0 + kGemmTile <= p.N;
    if (p.c_dt == DT_F32) gemm_store<float>(p, acc, buf, r0, c0, lane, full);
    else gemm_store<uint16_t>(p, acc, buf, r0, c0, lane, full);
}

// ---------------------------------------------------------------------------
// NVFP4 operands: E4M3 block scales per 16 values and a per-tensor scale g
// per operand (the NVFP4 matrix products QuTLASS runs, MR-GPTQ page,
// section 2.3).  gfx950's block-scaled matrix cores take only power-of-two
// scales per 32 values, so this kernel decodes each operand to fp16 and
// runs the fp16 matrix cores (v_mfma_f32_32x32x16_f16): a value is
// grid * dec(s), E2M1 value times E4M3 scale, which has at most six
// significant bits and lies in [2^-10, 2688], so fp16 holds it exactly and
// every product is exact in the fp32 accumulation; g_a g_b multiplies the
// result once.  The decode: the scaled FP4 -> fp16 convert with the
// power-of-two part P = 2^(max(e, 1) - 7) of the scale (the convert applies
// only a scale's exponent), then one packed fp16 multiply by the mantissa
// part mu = dec(s) / P (1 + m / 8, or m / 8 for the subnormal codes; NaN
// for code 0x7F).  P and mu of all 128 codes sit in an LDS table.
//
// Codes are staged exactly as in the MXFP4 kernel (same tiles, stages,
// direct loads, XOR swizzle and fragment reads).  A lane's 16-byte
// fragment chunk holds 32 K values (two 16-value scale blocks); each of its
// four dwords (8 values) is the lane's part of one 32 x 32 x 16 product,
// the same dword of A and of B in the same product, so the products sum
// matching K indices (the K order inside a step is permuted alike for both
// operands, which leaves the dot product's terms unchanged).
//
// Scales: a pass rewrites each operand's [rows, K/16] scale bytes so that a
// lane loads, per fragment and step, the 8 scale bytes of its chunks' blocks
// (byte 2 h + j: block 4 h + 2 (l / 32) + j of the step) in one 8-byte load.
// ---------------------------------------------------------------------------

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

struct NvGemmArgs {
    GemmArgs g;                                  // sa / sb: the rearranged scale bytes (as uint2)
    const float* ga;                             // per-tensor scales (device scalars; null: 1)
    const float* gb;
};

// out[(f * T + t) * 64 + l] = the 8 scale bytes of lane l of fragment f at
// step t: byte 2 h + j = block 16 t + 4 h + 2 (l / 32) + j of row
// 32 f + l % 32; rows past the matrix get code 0x38 (1.0).
__global__ void k_gemm_shuffle_scales_nv(const uint8_t* __restrict__ s, int64_t rows, int64_t kblocks, int steps,
                                         int64_t total, uint2* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int l = (int)(i & 63);
    const int64_t ft = i >> 6;
    const int t = (int)(ft % steps);
    const int64_t row = (ft / steps) * 32 + (l & 31);
    uint2 w = make_uint2(0x38383838u, 0x38383838u);
    if (row < rows) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(s + row * kblocks + 16 * t);
        const uint32_t q0 = p[0], q1 = p[1], q2 = p[2], q3 = p[3];   // blocks 4 h .. 4 h + 3 in q_h
        const uint32_t sel = (l >> 5) ? 0x07060302u : 0x05040100u;  // bytes 2 (l / 32) + {0, 1} of each
        w = make_uint2(__builtin_amdgcn_perm(q1, q0, sel), __builtin_amdgcn_perm(q3, q2, sel));
    }
    out[i] = w;
}

// Decode table entry of E4M3 code c = (e, m): P's fp32 bits (low 16 bits
// zero) with mu's fp16 bits in the low half.
__device__ __forceinline__ uint32_t nv_table_entry(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    const uint32_t p_bits = ((e > 0u ? e : 1u) + 120u) << 23;
    const float mu = (float)(e > 0u ? 8u + m : m) * 0.125f;
    uint32_t mu_bits = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)mu);
    if (c == 0x7Fu) mu_bits = 0x7E00u;           // NaN scale: every value NaN
    return p_bits | mu_bits;
}

__shared__ uint32_t g_nv_table[128];

// The fp16 operand of one 32 x 32 x 16 product: dword d of a fragment chunk
// (8 codes, byte k = values 2 k and 2 k + 1) decoded with table entry w.
__device__ __forceinline__ v8h nv_operand(uint32_t d, uint32_t w) {
    const float P = __builtin_bit_cast(float, w & 0xFFFF0000u);
    const v2h mu = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(w, w, 0x01000100u));
    const v2h x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, P, 0) * mu;
    const v2h x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, P, 1) * mu;
    const v2h x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, P, 2) * mu;
    const v2h x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, P, 3) * mu;
    return v8h{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
}

struct NvScales {
    uint2 a[4], b[4];
};

__device__ __forceinline__ void nv_issue_scales(const GemmArgs& p, const uint2* sa, const uint2* sb, int t,
                                                int64_t fa0, int64_t fb0, NvScales& sc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t fa = min<int64_t>(fa0 + i, p.frags_a - 1) - fa0;
        const int64_t fb = min<int64_t>(fb0 + i, p.frags_b - 1) - fb0;
        sc.a[i] = sa[(fa * p.steps + t) * 64];
        sc.b[i] = sb[(fb * p.steps + t) * 64];
    }
}

// Table entry of scale byte 2 h + j of a lane's 8 bytes.
template <int H, int J>
__device__ __forceinline__ uint32_t nv_entry(const uint2& b) {
    constexpr int k = 2 * H + J;
    const uint32_t w = k < 4 ? b.x : b.y;
    return g_nv_table[(w >> (8 * (k & 3))) & 0x7Fu];
}

// A substep's fragment chunks (16 bytes each, no widening).
struct NvFrags {
    v4i a[4], b[4];
};

template <int S>
__device__ __forceinline__ void nv_read(NvFrags& fr, int h, int lane, int wm, int wn) {
    const GemmStage& st = gemm_stage<S>();
    const int r = lane & 31;
    const int slot = (2 * h + (lane >> 5)) ^ ((r >> 1) & 7);
    const int off = r * kGemmRowBytes + 16 * slot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fr.a[i] = *reinterpret_cast<const v4i*>(st.a + ((128 * wm + 32 * i) * kGemmRowBytes + off));
        fr.b[i] = *reinterpret_cast<const v4i*>(st.b + ((128 * wn + 32 * i) * kGemmRowBytes + off));
    }
}

// The fp16 operands of dword d of every fragment chunk.
struct NvOps {
    v8h a[4], b[4];
};

__device__ __forceinline__ void nv_convert(const NvFrags& fr, int d, const uint32_t (&ea)[4], const uint32_t (&eb)[4],
                                           NvOps& o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o.a[i] = nv_operand((uint32_t)fr.a[i][d], ea[i]);
        o.b[i] = nv_operand((uint32_t)fr.b[i][d], eb[i]);
    }
}

// Substep H on fragments fr with scales sc: on entry o holds the operands
// of dword 0; each dword's 16 products run while the next dword's operands
// are decoded, the last while dword 0 of the next substep's fragments frn
// (at substep HN, scales scn) is; on return o holds those.  One product,
// then five decode instructions.
template <int H, int HN>
__device__ __forceinline__ void nv_substep(const NvFrags& fr, const NvScales& sc, const NvFrags& frn,
                                           const NvScales& scn, NvOps& o, v16f (&acc)[4][4]) {
    uint32_t ea0[4], ea1[4], eb0[4], eb1[4], na[4], nb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ea0[i] = nv_entry<H, 0>(sc.a[i]);
        eb0[i] = nv_entry<H, 0>(sc.b[i]);
        ea1[i] = nv_entry<H, 1>(sc.a[i]);
        eb1[i] = nv_entry<H, 1>(sc.b[i]);
        na[i] = nv_entry<HN, 0>(scn.a[i]);
        nb[i] = nv_entry<HN, 0>(scn.b[i]);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        NvOps n;
        if (d == 0) nv_convert(fr, 1, ea0, eb0, n);
        else if (d == 1) nv_convert(fr, 2, ea1, eb1, n);
        else if (d == 2) nv_convert(fr, 3, ea1, eb1, n);
        else nv_convert(frn, 0, na, nb, n);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.b[j], o.a[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // VALU
        }
        o = n;
    }
}

// One step, staged as gemm_step (the same direct loads, fragment reads and
// barrier), with the fp16 products of each substep.  o holds the operands
// of dword 0 of substep 0 (decoded during the previous step).
template <int S>
__device__ __forceinline__ void nv_step(const GemmArgs& p, const GemmLane& L, const uint2* sa, const uint2* sb,
                                        int t, int wave, int lane, int wm, int wn, int64_t fa0, int64_t fb0,
                                        NvScales& sc, const NvScales& sc_next, NvFrags& f0, NvOps& o,
                                        v16f (&acc)[4][4]) {
    NvFrags f1;
    gemm_issue_codes<S ^ 1, kHalfDma, kGemmDmaPerOperand>(L, min(t + 1, p.steps - 1), wave);
    nv_read<S>(f1, 1, lane, wm, wn);
    nv_substep<0, 1>(f0, sc, f1, sc, o, acc);
    nv_read<S>(f0, 2, lane, wm, wn);
    nv_substep<1, 2>(f1, sc, f0, sc, o, acc);
    nv_read<S>(f1, 3, lane, wm, wn);
    nv_substep<2, 3>(f0, sc, f1, sc, o, acc);
    __builtin_amdgcn_sched_barrier(0);
    gemm_wait_barrier<0>();
    gemm_issue_codes<S, 0, kHalfDma>(L, min(t + 2, p.steps - 1), wave);
    nv_read<S ^ 1>(f0, 0, lane, wm, wn);
    nv_substep<3, 0>(f1, sc, f0, sc_next, o, acc);
    __builtin_amdgcn_sched_barrier(0);
    nv_issue_scales(p, sa, sb, min(t + 2, p.steps - 1), fa0, fb0, sc);
    __builtin_amdgcn_sched_barrier(0);
}

template <int PARITY>
__global__ __launch_bounds__(256, 1) void k_nvfp4_gemm(NvGemmArgs q) {
    const GemmArgs& p = q.g;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    if (tid < 128) g_nv_table[tid] = nv_table_entry((uint32_t)tid);
    int tm, tn;
    gemm_tile(p, tm, tn);
    const int64_t m0 = (int64_t)tm * kGemmTile, n0 = (int64_t)tn * kGemmTile;
    const int64_t fa0 = (m0 + 128 * wm) / 32, fb0 = (n0 + 128 * wn) / 32;
    const int nt = p.steps;
    const uint2* sa = reinterpret_cast<const uint2*>(p.sa) + fa0 * nt * 64 + lane;
    const uint2* sb = reinterpret_cast<const uint2*>(p.sb) + fb0 * nt * 64 + lane;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    const GemmLane L = gemm_lane(p, m0, n0, wave, lane, wm, wn);
    NvScales s0, s1;
    gemm_issue_codes<0>(L, 0, wave);
    nv_issue_scales(p, sa, sb, 0, fa0, fb0, s0);
    __builtin_amdgcn_sched_barrier(0);
    gemm_issue_codes<1, 0, kHalfDma>(L, min(1, nt - 1), wave);
    nv_issue_scales(p, sa, sb, min(1, nt - 1), fa0, fb0, s1);
    __builtin_amdgcn_sched_barrier(0);
    gemm_wait_barrier<kGemmDmaPerOperand + 8>();    // all but step 1's half and its 8 scale loads (also the table)
    NvFrags f0;
    nv_read<0>(f0, 0, lane, wm, wn);
    NvOps o;
    {
        uint32_t ea[4], eb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ea[i] = nv_entry<0, 0>(s0.a[i]);
            eb[i] = nv_entry<0, 0>(s0.b[i]);
        }
        nv_convert(f0, 0, ea, eb, o);
    }
    // the step after the last reloads the last step (never used); its
    // scales then are those of the last step, which the loads hold anyway
    if constexpr (PARITY == 1) {
        nv_step<0>(p, L, sa, sb, 0, wave, lane, wm, wn, fa0, fb0, s0, s1, f0, o, acc);
#pragma unroll 1
        for (int t = 1; t < nt; t += 2) {
            nv_step<1>(p, L, sa, sb, t, wave, lane, wm, wn, fa0, fb0, s1, s0, f0, o, acc);
            nv_step<0>(p, L, sa, sb, t + 1, wave, lane, wm, wn, fa0, fb0, s0, s1, f0, o, acc);
        }
    } else {
#pragma unroll 1
        for (int t = 0; t < nt; t += 2) {
            nv_step<0>(p, L, sa, sb, t, wave, lane, wm, wn, fa0, fb0, s0, s1, f0, o, acc);
            nv_step<1>(p, L, sa, sb, t + 1, wave, lane, wm, wn, fa0, fb0, s1, s0, f0, o, acc);
        }
    }
    gemm_wait_barrier<0>();
    const float gg = (q.ga ? *q.ga : 1.0f) * (q.gb ? *q.gb : 1.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] *= gg;
    uint8_t* buf = reinterpret_cast<uint8_t*>(&g_stage0) + wave * (32 * 128 * 4);
    const int64_t r0 = m0 + 128 * wm, c0 = n0 + 128 * wn;
    const bool full = m0 + kGemmTile <= p.M && n0 + kGemmTile <= p.N;
    if (p.c_dt == DT_F32) gemm_store<float>(p, acc, buf, r0, c0, lane, full);
    else gemm_store<uint16_t>(p, acc, buf, r0, c0, lane, full);
}

// Copy of an NVFP4 operand with K padded to Kp: block j of a row (16
// values: 8 code bytes and one scale byte) copied for j < K / 16, code 0
// (+0) with scale 0x38 (1.0) past it.  One lane per block.
__global__ void k_gemm_pad_nv(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows,
                              int64_t kb, int64_t kbp, uint8_t* __restrict__ pcodes, uint8_t* __restrict__ pscales) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * kbp) return;
    const int64_t r = i / kbp, j = i - r * kbp;
    uint2 v = make_uint2(0u, 0u);
    uint8_t sc = 0x38;
    if (j < kb) {
        v = *reinterpret_cast<const uint2*>(codes + (r * kb + j) * 8);
        sc = scales[r * kb + j];
    }
    *reinterpret_cast<uint2*>(pcodes + i * 8) = v;
    pscales[i] = sc;
}

// Copy of an operand with K padded to Kp (a multiple of the K-step): block
// j of a row (32 values: 16 code bytes and one scale byte) is copied for
// j < K / 32, and the padding holds code 0 (+0, which adds exactly 0 to
// every product whatever its scale) with scale 1.  One lane per block.
__global__ void k_gemm_pad(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows,
                           int64_t kb, int64_t kbp, uint8_t* __restrict__ pcodes, uint8_t* __restrict__ pscales) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * kbp) return;
    const int64_t r = i / kbp, j = i - r * kbp;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    uint8_t sc = 127;
    if (j < kb) {
        v = *reinterpret_cast<const uint4*>(codes + (r * kb + j) * 16);
        sc = scales[r * kb + j];
    }
    *reinterpret_cast<uint4*>(pcodes + i * 16) = v;
    pscales[i] = sc;
}

namespace {

constexpr int64_t round256(int64_t n) { return (n + 255) / 256 * 256; }

// Bytes of the rearranged scales of both operands for K a multiple of the K-step.
size_t shuffled_scales_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t steps = K / kGemmStepK;
    const auto part = [&](int64_t rows) { return (size_t)round256(((rows + 31) / 32) * steps * 256); };
    return part(M) + part(N);
}

hipError_t launch_mxfp4_gemm_padded_k(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                      int64_t M, int64_t N, int64_t K, void* c, int c_dt, int64_t ldc, void* workspace,
                                      hipStream_t s);

}  // namespace

size_t mxfp4_gemm_workspace(int64_t M, int64_t N, int64_t K) {
    if (K % kGemmStepK == 0) return shuffled_scales_bytes(M, N, K);
    // K padded to the K-step: both operands copied, then the rearranged scales
    const int64_t Kp = (K + kGemmStepK - 1) / kGemmStepK * kGemmStepK;
    return shuffled_scales_bytes(M, N, Kp) + (size_t)(round256(M * Kp / 2) + round256(N * Kp / 2) +
                                                      round256(M * Kp / 32) + round256(N * Kp / 32));
}

hipError_t launch_mxfp4_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs, int64_t M,
                             int64_t N, int64_t K, void* c, int c_dt, int64_t ldc, void* workspace, hipStream_t s) {
    if (K % kGemmStepK != 0) return launch_mxfp4_gemm_padded_k(a, as, b, bs, M, N, K, c, c_dt, ldc, workspace, s);
    GemmArgs p{};
    p.a = a;
    p.b = b;
    p.M = M;
    p.N = N;
    p.K = K;
    p.c = c;
    p.c_dt = c_dt;
    p.ldc = ldc;
    p.tiles_m = (int)((M + kGemmTile - 1) / kGemmTile);
    p.tiles_n = (int)((N + kGemmTile - 1) / kGemmTile);
    p.steps = (int)(K / kGemmStepK);
    p.frags_a = (int)((M + 31) / 32);
    p.frags_b = (int)((N + 31) / 32);
    const size_t wa = ((size_t)p.frags_a * p.steps * 256 + 255) / 256 * 256;
    uint32_t* sa = reinterpret_cast<uint32_t*>(workspace);
    uint32_t* sb = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(workspace) + wa);
    const int64_t ta = (int64_t)p.frags_a * p.steps * 64, tb = (int64_t)p.frags_b * p.steps * 64;
    hipLaunchKernelGGL(k_gemm_shuffle_scales, dim3((unsigned)((ta + 255) / 256)), dim3(256), 0, s, as, M, K / 32,
                       p.steps, ta, sa);
    hipLaunchKernelGGL(k_gemm_shuffle_scales, dim3((unsigned)((tb + 255) / 256)), dim3(256), 0, s, bs, N, K / 32,
                       p.steps, tb, sb);
    p.sa = sa;
    p.sb = sb;
    const dim3 grid((unsigned)p.tiles_m * p.tiles_n), block(256);
    if (p.steps % 2) hipLaunchKernelGGL(k_mxfp4_gemm<1>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(k_mxfp4_gemm<0>, grid, block, 0, s, p);
    return hipGetLastError();
}

namespace {

hipError_t launch_mxfp4_gemm_padded_k(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                      int64_t M, int64_t N, int64_t K, void* c, int c_dt, int64_t ldc, void* workspace,
                                      hipStream_t s) {
    const int64_t Kp = (K + kGemmStepK - 1) / kGemmStepK * kGemmStepK;
    uint8_t* w = reinterpret_cast<uint8_t*>(workspace) + shuffled_scales_bytes(M, N, Kp);
    uint8_t* pa = w;
    uint8_t* pb = pa + round256(M * Kp / 2);
    uint8_t* pas = pb + round256(N * Kp / 2);
    uint8_t* pbs = pas + round256(M * Kp / 32);
    const int64_t kb = K / 32, kbp = Kp / 32;
    const auto pad = [&](const uint8_t* codes, const uint8_t* scales, int64_t rows, uint8_t* pc, uint8_t* ps) {
        const int64_t n = rows * kbp;
        hipLaunchKernelGGL(k_gemm_pad, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, scales, rows, kb,
                           kbp, pc, ps);
    };
    pad(a, as, M, pa, pas);
    pad(b, bs, N, pb, pbs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_mxfp4_gemm(pa, pas, pb, pbs, M, N, Kp, c, c_dt, ldc, workspace, s);
}

// Bytes of the rearranged NVFP4 scales of both operands (K a multiple of the K-step).
size_t shuffled_scales_bytes_nv(int64_t M, int64_t N, int64_t K) {
    const int64_t steps = K / kGemmStepK;
    const auto part = [&](int64_t rows) { return (size_t)round256(((rows + 31) / 32) * steps * 512); };
    return part(M) + part(N);
}

}  // namespace

size_t nvfp4_gemm_workspace(int64_t M, int64_t N, int64_t K) {
    if (K % kGemmStepK == 0) return shuffled_scales_bytes_nv(M, N, K);
    const int64_t Kp = (K + kGemmStepK - 1) / kGemmStepK * kGemmStepK;
    return shuffled_scales_bytes_nv(M, N, Kp) + (size_t)(round256(M * Kp / 2) + round256(N * Kp / 2) +
                                                         round256(M * Kp / 16) + round256(N * Kp / 16));
}

hipError_t launch_nvfp4_gemm(const uint8_t* a, const uint8_t* as, const float* ga, const uint8_t* b,
                             const uint8_t* bs, const float* gb, int64_t M, int64_t N, int64_t K, void* c, int c_dt,
                             int64_t ldc, void* workspace, hipStream_t s) {
    if (K % kGemmStepK != 0) {
        // pad K to the K-step: copies of both operands after the rearranged scales
        const int64_t Kp = (K + kGemmStepK - 1) / kGemmStepK * kGemmStepK;
        uint8_t* w = reinterpret_cast<uint8_t*>(workspace) + shuffled_scales_bytes_nv(M, N, Kp);
        uint8_t* pa = w;
        uint8_t* pb = pa + round256(M * Kp / 2);
        uint8_t* pas = pb + round256(N * Kp / 2);
        uint8_t* pbs = pas + round256(M * Kp / 16);
        const int64_t kb = K / 16, kbp = Kp / 16;
        const auto pad = [&](const uint8_t* codes, const uint8_t* scales, int64_t rows, uint8_t* pc, uint8_t* ps) {
            const int64_t n = rows * kbp;
            hipLaunchKernelGGL(k_gemm_pad_nv, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, scales, rows,
                               kb, kbp, pc, ps);
        };
        pad(a, as, M, pa, pas);
        pad(b, bs, N, pb, pbs);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_nvfp4_gemm(pa, pas, ga, pb, pbs, gb, M, N, Kp, c, c_dt, ldc, workspace, s);
    }
    NvGemmArgs q{};
    GemmArgs& p = q.g;
    p.a = a;
    p.b = b;
    p.M = M;
    p.N = N;
    p.K = K;
    p.c = c;
    p.c_dt = c_dt;
    p.ldc = ldc;
    p.tiles_m = (int)((M + kGemmTile - 1) / kGemmTile);
    p.tiles_n = (int)((N + kGemmTile - 1) / kGemmTile);
    p.steps = (int)(K / kGemmStepK);
    p.frags_a = (int)((M + 31) / 32);
    p.frags_b = (int)((N + 31) / 32);
    const size_t wa = ((size_t)p.frags_a * p.steps * 512 + 255) / 256 * 256;
    uint2* sa = reinterpret_cast<uint2*>(workspace);
    uint2* sb = reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(workspace) + wa);
    const int64_t ta = (int64_t)p.frags_a * p.steps * 64, tb = (int64_t)p.frags_b * p.steps * 64;
    hipLaunchKernelGGL(k_gemm_shuffle_scales_nv, dim3((unsigned)((ta + 255) / 256)), dim3(256), 0, s, as, M, K / 16,
                       p.steps, ta, sa);
    hipLaunchKernelGGL(k_gemm_shuffle_scales_nv, dim3((unsigned)((tb + 255) / 256)), dim3(256), 0, s, bs, N, K / 16,
                       p.steps, tb, sb);
    p.sa = reinterpret_cast<const uint32_t*>(sa);
    p.sb = reinterpret_cast<const uint32_t*>(sb);
    q.ga = ga;
    q.gb = gb;
    const dim3 grid((unsigned)p.tiles_m * p.tiles_n), block(256);
    if (p.steps % 2) hipLaunchKernelGGL(k_nvfp4_gemm<1>, grid, block, 0, s, q);
    else hipLaunchKernelGGL(k_nvfp4_gemm<0>, grid, block, 0, s, q);
    return hipGetLastError();
}

}  // namespace fp4q_dev
