/*
 * fp4q.h -- C ABI of the MI355X (gfx950) block-scaled FP4 quantize /
 * dequantize library (libfp4q.so).
 *
 * What the calls compute comes from these pages (title -- section):
 *  - "Bridging the Gap Between Promise and Performance for Microscaling FP4
 *    Quantization", technical summary section 1 (MXFP4: power-of-two E8M0
 *    block scale; NVFP4: blocks of 16) and 2.1-2.3 (block-wise Hadamard
 *    rotation of weights and of activations on the fly; scales optimised
 *    for MSE per group).
 *  - "Finer is Better (with the Right Scaling)", method part 1 (OCP E2M1
 *    elements, E4M3 scale factors, blocks of 4/8/16/32) and part 2 (scale
 *    strategies abs-max, prevent-zero, 4-over-6, brute-force search,
 *    hierarchical per-tensor-then-per-block scaling).
 *  - "FOCUS: FP4 Optimization via Coupled-Relaxation and Dual-Granularity
 *    Scaling", method 1 (STE scale learning), 2 (CRS: S_q = S_dq * c_i with
 *    FP16 c_i), 3 (DGS: one c_k per sub-block, W_k -> Q(W_k / (S_dq c_k)),
 *    S_dq shared by the block), 4 (deploy FP4 codes and S_dq only).
 *
 * Conventions shared by every call
 *  - A tensor is [rows, cols] row-major with a row stride `ld` in ELEMENTS
 *    (ld >= cols).  Blocks are `block` contiguous values along a row (the
 *    GEMM reduction dimension of a [out, in] weight, the hidden dimension of
 *    a [tokens, hidden] activation), starting at column 0.
 *  - codes:  [rows, cols/2] bytes, dense; byte j of a row holds element 2j in
 *            its low nibble and element 2j+1 in its high nibble; a nibble is
 *            sign (bit 3) and E2M1 magnitude code 0..7 for
 *            {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *  - scales: [rows, cols/block] bytes, dense, row-major; E8M0 (value
 *            2^(code-127), 0xFF = NaN), unsigned OCP E4M3 (bit 7 ignored,
 *            0x7F = NaN, largest 448) or UE5M3 (below).
 *  - g:      the per-tensor fp32 scale of hierarchical scaling; the
 *            effective block scale is S = fl(decode(code) * g).  For E8M0
 *            there is no g (it is 1); UE5M3 takes g from NONE or USER only.
 *  - Every buffer is device memory the caller allocated (the library
 *    allocates nothing and keeps no state; the one exception is the static
 *    scratch array of fp4q_quantize_noalloc).  Base pointers must be 16-byte
 *    aligned, and ld * element_size must be a multiple of 16 bytes, as must
 *    cols * element_size.  Element types: fp32, bf16, fp16.
 *  - `stream` is a hipStream_t (NULL = the default stream).  A call only
 *    validates its arguments and enqueues kernels; it never synchronises.
 *    Outputs are valid once the stream reaches that point.
 *  - Arguments are checked on the host before anything is launched; a bad
 *    argument returns an error code and enqueues nothing.  A failed launch
 *    returns FP4Q_ERR_DEVICE.  Errors never abort or throw.
 *  - NaN or infinity inside a block whose scale the library chooses makes
 *    that block a NaN block: NaN scale code, zero-magnitude codes carrying
 *    the element signs, NaN dequantized values (0x7FC00000 with the element
 *    sign), NaN MSE.  A scale that decodes to NaN, infinity or a negative
 *    value (possible with a caller's g) gives a NaN block as well.  With a
 *    rotation, every NaN the rotation produces counts as positive (IEEE 754
 *    leaves the sign of a NaN returned by arithmetic unspecified).
 *  - Results are deterministic and independent of the launch shape.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 8

typedef enum {
    FP4Q_OK = 0,
    FP4Q_ERR_INVALID_ARG = 1, /* null required pointer, bad enum, bad user scale */
    FP4Q_ERR_UNSUPPORTED = 2, /* combination the formats do not define, or SEARCH
                                 with GIVEN */
    FP4Q_ERR_SHAPE = 3,       /* block / rotation / sub-block does not tile the row */
    FP4Q_ERR_ALIGNMENT = 4,   /* base pointer or row pitch not 16-byte aligned */
    FP4Q_ERR_DEVICE = 5,      /* the HIP runtime refused a launch */
    FP4Q_ERR_TOO_LARGE = 6    /* fp4q_quantize_noalloc: the workspace this call needs
                                 exceeds the library's static scratch */
} fp4q_status;

typedef enum { FP4Q_F32 = 0, FP4Q_BF16 = 1, FP4Q_F16 = 2 } fp4q_dtype;

/* Block scale formats.  UE5M3 is the unsigned wide-exponent scale the
 * "Finer is Better" page compares with E4M3 + hierarchical scaling +
 * 4-over-6 (key findings); the page gives no encoding, so this library reads
 * it as 5 exponent bits with bias 15 and 3 mantissa bits: (1 + m/8) 2^(e-15),
 * subnormals m 2^-17, largest 0xFE = 114688, 0xFF = NaN, no infinities,
 * round-half-to-even with saturation.  It needs no per-tensor scale: global
 * modes NONE and USER. */
typedef enum { FP4Q_SCALE_E8M0 = 0, FP4Q_SCALE_E4M3 = 1, FP4Q_SCALE_UE5M3 = 2 } fp4q_scale_fmt;

/* Scale strategies ("Finer is Better (with the Right Scaling)", method
 * part 2).  ABSMAX maps the block abs-max onto 6 and rounds the scale to the
 * format (E8M0: the power of two 2^(floor(log2 amax) - 2)); PREVENT_ZERO is
 * ABSMAX with an E4M3 code of 0 raised to the smallest nonzero code;
 * FOUR_OVER_SIX keeps whichever of the map-to-6 and map-to-4 scales gives
 * the lower block squared error (E4M3, UE5M3); BRUTE_FORCE tries every
 * positive finite scale (126 E4M3 codes, 255 E8M0 codes, 254 UE5M3 codes)
 * and keeps the lowest squared error, ties to the smaller code; GIVEN reads
 * the scales. */
typedef enum {
    FP4Q_ABSMAX = 0,
    FP4Q_PREVENT_ZERO = 1,
    FP4Q_FOUR_OVER_SIX = 2,
    FP4Q_BRUTE_FORCE = 3,
    FP4Q_GIVEN = 4
} fp4q_strategy;

/* Per-tensor scale g (hierarchical scaling, same page, method part 2):
 * NONE -> g = 1; TENSOR_AMAX -> g = fl(amax(|x|) / 2688) over the whole
 * (rotated) tensor, 2688 = 6 * 448, and g = 1 when that is 0, NaN when the
 * tensor holds NaN or infinity; USER -> g = global_scale.  TENSOR_AMAX and
 * SEARCH: E4M3 only; USER: E4M3 and UE5M3.
 * SEARCH (per-tensor scale chosen for minimum MSE, MR-GPTQ page, section
 * 2.2): with g0 the TENSOR_AMAX scale, the candidates g_j = fl(g0 (1 - j/64)),
 * j = 0..31, are each scored by the fp64 balanced-tree sum, over all blocks
 * in row-major order (zero-padded to a power of two), of the fp32 block SSE
 * under the configured strategy; the smallest total wins, ties to the
 * smallest j.  Strategies ABSMAX, PREVENT_ZERO, FOUR_OVER_SIX and
 * BRUTE_FORCE (each block at its exhaustive-argmin scale for every
 * candidate: 32 brute-force searches of the tensor). */
typedef enum {
    FP4Q_GLOBAL_NONE = 0,
    FP4Q_GLOBAL_TENSOR_AMAX = 1,
    FP4Q_GLOBAL_USER = 2,
    FP4Q_GLOBAL_SEARCH = 3
} fp4q_global;

typedef struct {
    uint32_t struct_size;  /* sizeof(fp4q_config) */
    int32_t scale_fmt;     /* fp4q_scale_fmt */
    int32_t block;         /* 4, 8, 16 or 32 */
    int32_t strategy;      /* fp4q_strategy */
    int32_t global_mode;   /* fp4q_global */
    float global_scale;    /* used only by FP4Q_GLOBAL_USER: finite, >= FLT_MIN, 448*g < FLT_MAX */
    int32_t hadamard;      /* 0 (none), 16 or 32: normalised Walsh-Hadamard on each
                              aligned segment of that many values before quantizing */
} fp4q_config;

/* MXFP4 = {E8M0, 32, ABSMAX, NONE}; NVFP4 = {E4M3, 16, ABSMAX or FOUR_OVER_SIX, TENSOR_AMAX}. */

int fp4q_abi_version(void);
const char* fp4q_status_string(int status);

/* Bytes of caller-provided device workspace `fp4q_quantize` and
 * `fp4q_scale_search` need for this configuration and shape (0 when none):
 * room for the per-tensor abs-max partial results of TENSOR_AMAX, and for
 * SEARCH also the candidates' partial sums (about 32 * 8 bytes per 64 * 4
 * elements).  Returns 0 for a NULL config. */
size_t fp4q_workspace_bytes(const fp4q_config* cfg, int64_t rows, int64_t cols);

/* Quantize x [rows, cols] (type x_dt, row stride ld_x) into packed E2M1
 * codes and block scales.
 *   codes      [rows, cols/2]      required output
 *   scales     [rows, cols/block]  required; output, or input for GIVEN
 *   g_dev      1 fp32              output of the g used; required for
 *                                  TENSOR_AMAX, USER and SEARCH, optional
 *                                  for NONE (then 1.0 is written when
 *                                  non-NULL)
 *   dequant    [rows, ld_dq]       optional output (type dq_dt): the fp32
 *                                  dequantized value (-1)^s fl(grid * S),
 *                                  rounded half-to-even to bf16 / fp16
 *   block_mse  [rows, cols/block]  optional output: fl(SSE / block), SSE the
 *                                  balanced-tree fp32 sum of fl(d*d),
 *                                  d = fl(y - yhat)
 *   workspace  fp4q_workspace_bytes(...) bytes of device memory, or NULL
 *              when that is 0.
 * With hadamard != 0 the rotated values are quantized and dequant / MSE are
 * in the rotated domain. */
fp4q_status fp4q_quantize(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows,
                          int64_t cols, int64_t ld_x, uint8_t* codes, uint8_t* scales,
                          float* g_dev, void* dequant, int dq_dt, int64_t ld_dq,
                          float* block_mse, void* workspace, void* stream);

/* fp4q_quantize that also counts the codes it writes: the codebook
 * occupancy of the TORQ page, section 2.B (how evenly the 16 FP4 codewords
 * are used; their collapse onto the smallest magnitudes is what it
 * measures), fused into the quantize kernels instead of a second pass over
 * the codes.  counts [FP4Q_COUNT_REPLICAS][16] device uint64, dense,
 * ACCUMULATED: the number of written nibbles equal to c (sign bit 3, E2M1
 * magnitude bits 0-2), NaN blocks included (their nibbles carry only the
 * sign), is added to column c, split over the rows in a way that depends
 * on the launch; the occupancy of code c is the sum of column c.  The rows
 * spread the kernels' final atomic additions over separate 128-byte lines
 * (128-byte alignment keeps each row on one line): additions from many
 * workgroups to one line serialise.  Zero counts before the first call.
 * The codes, scales, g, dequant and MSE are those fp4q_quantize writes.
 * counts is required (FP4Q_ERR_INVALID_ARG) and 8-byte aligned
 * (FP4Q_ERR_ALIGNMENT); every other argument as for fp4q_quantize.  The
 * column sums are integers, exact whatever the order of the additions. */
#define FP4Q_COUNT_REPLICAS 64
fp4q_status fp4q_quantize_histogram(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows,
                                    int64_t cols, int64_t ld_x, uint8_t* codes, uint8_t* scales,
                                    float* g_dev, void* dequant, int dq_dt, int64_t ld_dq,
                                    float* block_mse, uint64_t* counts, void* workspace,
                                    void* stream);

/* fp4q_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and errors, without `workspace`.  The workspace
 * lives in a static device array of 16 MiB inside the library (one per GPU,
 * held until the process ends); a call never calls hipMalloc, hipFree or any
 * allocating routine.  A configuration and shape whose fp4q_workspace_bytes
 * exceeds 16 MiB (only GLOBAL_SEARCH on tensors of more than about 4 M
 * 16-value units) returns FP4Q_ERR_TOO_LARGE and enqueues nothing.  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (other streams, other host threads) race and must be ordered by the
 * caller.  Nothing in the array needs to start at zero (each call writes
 * every entry it reads). */
fp4q_status fp4q_quantize_noalloc(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows,
                                  int64_t cols, int64_t ld_x, uint8_t* codes, uint8_t* scales,
                                  float* g_dev, void* dequant, int dq_dt, int64_t ld_dq,
                                  float* block_mse, void* stream);

/* Dequantize codes + scales to out [rows, ld_out] (type out_dt):
 * (-1)^s fl(grid[mag] * S) with S = fl(decode(scale) * g); g is read from
 * g_dev (device fp32) or is 1 when g_dev is NULL; g_dev must be NULL for
 * E8M0.  Values stay in the rotated domain when the codes came from a
 * rotated tensor (cfg->hadamard is not used here). */
fp4q_status fp4q_dequantize(const fp4q_config* cfg, const uint8_t* codes, const uint8_t* scales,
                            const float* g_dev, int64_t rows, int64_t cols, void* out,
                            int out_dt, int64_t ld_out, void* stream);

/* Per-block MSE [rows, cols/block] of x (rotated first when cfg->hadamard
 * != 0) against the values that codes + scales (+ g_dev) decode to. */
fp4q_status fp4q_block_mse(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows,
                           int64_t cols, int64_t ld_x, const uint8_t* codes,
                           const uint8_t* scales, const float* g_dev, float* block_mse,
                           void* stream);

/* Scale selection alone ("MSE-optimised grid" per group of the MR-GPTQ
 * page, section 2.2; brute force of the Finer-is-Better page): writes the
 * block scales the configured strategy (not GIVEN) picks, g_dev as in
 * fp4q_quantize, and optionally best_sse [rows, cols/block], the fp32 tree
 * SSE of each block at its chosen scale. */
fp4q_status fp4q_scale_search(const fp4q_config* cfg, const void* x, int x_dt, int64_t rows,
                              int64_t cols, int64_t ld_x, uint8_t* scales, float* g_dev,
                              float* best_sse, void* workspace, void* stream);

/* FOCUS relaxed fake-quant forward (FOCUS page, methods 2-3): with S_dq
 * from scales + g_dev (g_dev NULL -> 1) and c_k the fp16 coefficient of
 * sub-block k (c_f16 [rows, cols/sub_block], dense),
 *   S_q = fl(S_dq * c_k),  u = fl(W / S_q) (0 when S_q == 0),
 *   What = (-1)^sign(W) fl(grid[RNE_E2M1(|u|)] * S_dq).
 * w_hat [rows, ld_out] of type out_dt; codes [rows, cols/2] optional (the
 * deployable FP4 weights, method 4).  sub_block in {4, 8, 16, 32}, dividing
 * block.  cfg->strategy and cfg->global_mode are not used; hadamard must be 0
 * (FOCUS applies no rotation, method 4). */
fp4q_status fp4q_relaxed_fakequant_fwd(const fp4q_config* cfg, const void* w, int w_dt,
                                       int64_t rows, int64_t cols, int64_t ld_w,
                                       const uint8_t* scales, const float* g_dev,
                                       const uint16_t* c_f16, int32_t sub_block, void* w_hat,
                                       int out_dt, int64_t ld_out, uint8_t* codes, void* stream);

/* Straight-through backward of the forward above to c (FOCUS page, method
 * 1): Q is replaced by the clip to [-6, 6], so
 *   grad_c[k] = fl(-A_k / fl(c_k * c_k)),
 *   A_k = tree sum over the sub-block of [S_q > 0 and |u_i| <= 6] * fl(G_i * W_i),
 * with G = grad_out [rows, ld_g] of type g_dt (dL/dWhat).  grad_c
 * [rows, cols/sub_block] fp32; NaN sub-blocks give NaN (0x7FC00000). */
fp4q_status fp4q_relaxed_fakequant_bwd(const fp4q_config* cfg, const void* w, int w_dt,
                                       int64_t rows, int64_t cols, int64_t ld_w,
                                       const uint8_t* scales, const float* g_dev,
                                       const uint16_t* c_f16, int32_t sub_block,
                                       const void* grad_out, int g_dt, int64_t ld_g,
                                       float* grad_c, void* stream);

/* Codebook occupancy of packed codes (TORQ page, section 2.B: the usage of
 * the FP4 codewords, whose collapse onto the smallest codes the method
 * measures against the uniform distribution).  counts [16] device uint64,
 * ACCUMULATED: counts[c] += number of nibbles equal to c (sign bit 3, E2M1
 * magnitude bits 0-2) in codes [rows, cols/2], dense; zero counts before
 * the first call (several tensors can share one count).  cols must be even
 * (FP4Q_ERR_SHAPE); codes 16-byte aligned, counts 8-byte aligned
 * (FP4Q_ERR_ALIGNMENT); an empty tensor adds nothing. */
fp4q_status fp4q_code_histogram(const uint8_t* codes, int64_t rows, int64_t cols, uint64_t* counts,
                                void* stream);

/* FP4 GEMM on MXFP4 operands (the FP4 matrix products of the MR-GPTQ page,
 * section 2.3, run on gfx950's block-scaled matrix cores):
 *   C[m][n] = sum_k dq(A)[m][k] * dq(B)[n][k]
 * with dq the MXFP4 decode (E2M1 value times 2^(scale-127) of its 32-element
 * block).  A codes [M, K/2] + E8M0 scales [M, K/32] and B codes [N, K/2] +
 * scales [N, K/32], dense: the layouts fp4q_quantize writes for {E8M0, 32}
 * (B is the [out, in] weight, A the [tokens, in] activation).  C [M, ldc] of
 * type c_dt (FP4Q_F32 or FP4Q_BF16, rounded half-to-even), ldc >= N.
 * Accumulation is fp32 inside the matrix cores, in an order of its own.
 * workspace: fp4q_mxfp4_gemm_workspace_bytes(M, N, K) bytes of device
 * memory, 256-byte aligned, owned by the caller (the scales rearranged for
 * the matrix cores go there, and the padded operand copies described below;
 * its contents need no initialisation and are dead after the call).  K must be a positive multiple of 32 (one scale
 * block) and M * Kp / 2, N * Kp / 2 below 2^32, Kp = K rounded up to a
 * multiple of 256 (FP4Q_ERR_SHAPE).  When K is not a multiple of 256 both
 * operands are first copied into the workspace with K padded to Kp (zero
 * codes, which add exactly 0); codes and C 16-byte aligned,
 * ldc * element size a multiple of 16, scales 4-byte aligned, workspace
 * 256-byte aligned (FP4Q_ERR_ALIGNMENT). */
size_t fp4q_mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
fp4q_status fp4q_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                            const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c, int c_dt,
                            int64_t ldc, void* workspace, void* stream);

/* FP4 GEMM on NVFP4 operands (the MR-GPTQ page, section 2.3: QuTLASS runs
 * the FP4 matrix products on MXFP4 and on NVFP4 operands):
 *   C[m][n] = sum_k dq(A)[m][k] * dq(B)[n][k]
 * with dq the NVFP4 decode that fp4q_dequantize applies for {E4M3, 16}: the
 * E2M1 value times fl(dec(scale) * g) of its 16-element block (NaN for
 * scale 0x7F).  A codes [M, K/2] + E4M3 scales [M, K/16] with per-tensor
 * scale *a_g, B likewise with *b_g (device fp32 scalars as fp4q_quantize
 * writes them; NULL means 1): the layouts fp4q_quantize writes for
 * {E4M3, 16}.  C [M, ldc] of type c_dt (FP4Q_F32 or FP4Q_BF16, rounded
 * half-to-even), ldc >= N.  gfx950's block-scaled matrix cores take only
 * power-of-two scales per 32 values, so the operands are decoded to fp16
 * (grid value times dec(scale), exact) and multiplied on the fp16 matrix
 * cores with fp32 accumulation in an order of their own; the result is then
 * multiplied by fl(g_a g_b), so it differs from the definition by the
 * accumulation order and a few roundings of g (relative 2^-22 of the sum
 * of |products|).  workspace: fp4q_nvfp4_gemm_workspace_bytes(M, N, K)
 * bytes, 256-byte aligned, owned by the caller (rearranged scales, and
 * padded operand copies when K is not a multiple of 256; no initialisation
 * needed, dead after the call).  K must be a positive multiple of 16 and
 * M * Kp / 2, N * Kp / 2 below 2^32, Kp = K rounded up to a multiple of 256
 * (FP4Q_ERR_SHAPE); codes and C 16-byte aligned, ldc * element size a
 * multiple of 16, scales 4-byte aligned, workspace 256-byte aligned
 * (FP4Q_ERR_ALIGNMENT). */
size_t fp4q_nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
fp4q_status fp4q_nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g,
                            const uint8_t* b_codes, const uint8_t* b_scales, const float* b_g, int64_t M, int64_t N,
                            int64_t K, void* c, int c_dt, int64_t ldc, void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
