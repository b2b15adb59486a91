// fp4q_kernels.hpp -- gfx950 kernels of the block-scaled FP4 path and the
// host launchers that pick their template instantiation.
//
// Work mapping: one lane owns one "unit" -- U contiguous values of a row,
// U = max(block, rotation size, 16 bytes of input) -- so a block, its
// rotation segment and its squared-error tree live in that lane's registers
// and no cross-lane traffic is needed.  A 256-thread workgroup walks the
// units grid-stride; lanes of a wave own neighbouring units, so a wave
// covers one contiguous stretch of the tensor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4q_device.hpp"

namespace fp4q_dev {

constexpr int kThreads = 256;
constexpr int kAmaxBlocks = 1024;   // partial abs-max results of the pre-pass
constexpr int kSearchCandidates = 32;   // per-tensor scale candidates g0 * (1 - j/64)

template <int... Is> struct ISeq {};
template <int N, int... Is> struct MakeISeq : MakeISeq<N - 1, N - 1, Is...> {};
template <int... Is> struct MakeISeq<0, Is...> { using type = ISeq<Is...>; };
template <int I> struct IC { static constexpr int value = I; };
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, ISeq<Is...>) { (f(IC<Is>{}), ...); }
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl(f, typename MakeISeq<N>::type{}); }

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <class InT, int B, int H>
constexpr int unit_elems() { return cmax(cmax(B, H), 16 / ElemSize<InT>::value); }

// ---------------------------------------------------------------------------
// Argument blocks (plain data, passed by value)
// ---------------------------------------------------------------------------

struct QuantArgs {
    const void* x;
    int64_t ld_x;
    int64_t cols;
    int64_t units;          // rows * cols / U
    int64_t units_per_row;  // cols / U
    int contiguous;         // ld_x == cols and (no dequant or ld_dq == cols)
    uint8_t* codes;         // [rows, cols/2] or null
    uint8_t* scales;        // [rows, cols/B]: output, or input for GIVEN
    float* g_out;           // or null
    void* dq;               // or null
    int64_t ld_dq;
    int dq_dt;
    float* mse;             // [rows, cols/B] or null
    float* sse;             // [rows, cols/B] or null
    const uint32_t* amax_partials;
    int n_partials;
    int global_mode;
    float user_g;
    const float* g_in;      // GM_DEVICE: the scale to use
    int prevent_zero;
    unsigned long long* counts;   // [16] code occupancy to add to, or null
};

// Per-tensor scale search: block SSE totals of every candidate, per tile.
struct GSearchArgs {
    const void* x;
    int64_t ld_x;
    int64_t units;
    int64_t units_per_row;
    int contiguous;
    const uint32_t* amax_partials;
    int n_partials;
    int prevent_zero;
    double* partials;       // [kSearchCandidates][ntiles]
    int64_t ntiles;
};

struct AmaxArgs {
    const void* x;
    int64_t ld_x;
    int64_t units;
    int64_t units_per_row;
    int contiguous;
    uint32_t* partials;     // [gridDim.x]
};

struct DequantArgs {
    const uint8_t* codes;
    const uint8_t* scales;
    const float* g_dev;     // or null (g = 1)
    int scale_fmt;
    int64_t cols;
    int64_t units;
    int64_t units_per_row;
    void* out;
    int64_t ld_out;
    int out_dt;
};

struct MseArgs {
    const void* x;
    int64_t ld_x;
    int64_t cols;
    int64_t units;
    int64_t units_per_row;
    const uint8_t* codes;
    const uint8_t* scales;
    const float* g_dev;
    int scale_fmt;
    float* mse;
};

struct RelaxedArgs {
    const void* w;
    int64_t ld_w;
    int64_t cols;
    int64_t units;
    int64_t units_per_row;
    const uint8_t* scales;
    const float* g_dev;
    int scale_fmt;
    const uint16_t* c;      // [rows, cols/K] fp16 bits
    void* w_hat;            // fwd output
    int64_t ld_out;
    int out_dt;
    uint8_t* codes;         // fwd, or null
    const void* grad;       // bwd input
    int64_t ld_g;
    int g_dt;
    float* grad_c;          // bwd output [rows, cols/K]
};

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

__device__ __forceinline__ uint32_t workgroup_max_u32(uint32_t v) {
    __shared__ uint32_t s_part[kThreads / 64];
    v = wave_max_u32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s_part[wave] = v;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) m = max(m, s_part[i]);
    __syncthreads();
    return m;
}

// A scale usable for encoding: a number, finite, not negative.
__device__ __forceinline__ bool scale_usable(float S) { return S >= 0.0f && S < __builtin_inff(); }

// (-1)^sign(of s) |v|
__device__ __forceinline__ float with_sign_of(float v, float s) {
    return as_f((as_u(v) & 0x7FFFFFFFu) | (as_u(s) & 0x80000000u));
}

__device__ __forceinline__ float canonical_nan_like(float s) { return as_f(kQNaN | (as_u(s) & 0x80000000u)); }

// Per-tensor scale g of hierarchical scaling ("Finer is Better (with the
// Right Scaling)", method part 2): NONE -> 1, USER -> given, TENSOR_AMAX ->
// fl(amax / (6 * 448)), 1 when that is 0, NaN when amax is not finite.
// Every thread of the workgroup must call it.
__device__ __forceinline__ float workgroup_amax_scale(const uint32_t* partials, int n) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < n; i += kThreads) m = max(m, partials[i]);
    m = workgroup_max_u32(m);
    if (m >= 0x7F800000u) return as_f(kQNaN);
    float g = as_f(m) / 2688.0f;
    return g == 0.0f ? 1.0f : g;
}

__device__ __forceinline__ float workgroup_global_scale(const QuantArgs& p) {
    if (p.global_mode == GM_NONE) return 1.0f;
    if (p.global_mode == GM_USER) return p.user_g;
    if (p.global_mode == GM_DEVICE) return *p.g_in;
    return workgroup_amax_scale(p.amax_partials, p.n_partials);
}

// Shrink factor of search candidate j: 1 - j/64 (exact in fp32).
__device__ __forceinline__ float search_factor(int j) { return 1.0f - (float)j * 0.015625f; }

__device__ __forceinline__ float read_g(const float* g_dev) { return g_dev ? *g_dev : 1.0f; }

// Element offset of unit u in a [rows, ld] tensor whose rows hold upr units.
template <int U>
__device__ __forceinline__ int64_t unit_offset(int64_t u, int64_t upr, int64_t ld, bool contiguous) {
    if (contiguous) return u * U;
    int64_t row = u / upr;
    return row * ld + (u - row * upr) * U;
}

// ---------------------------------------------------------------------------
// Code occupancy counted while quantizing (TORQ page, section 2.B: how often
// each of the 16 FP4 codewords is used).  Counters are private per thread
// while a kernel runs; each workgroup adds its 16 totals, once, at the end,
// to one of kCountReplicas rows of the caller's 64-bit counts (row =
// workgroup index mod kCountReplicas).  Atomic additions from many
// workgroups to one 128-byte line serialise at several ns each; with every
// workgroup on the same line the resident grid's final additions took
// longer than a whole quantize call, spread over 64 lines they overlap.
// ---------------------------------------------------------------------------

constexpr int kCountReplicas = 64;   // rows of 16 counts (FP4Q_COUNT_REPLICAS)

// Adds to cnt[v], for every v, the number of the eight nibbles of w equal to
// v.  Bit j of every nibble is sliced out to bit 4k of b[j]; the mask of the
// nibbles equal to v is the AND of four slices or their complements (shared
// as two pair products), and one popcount adds it.
__device__ __forceinline__ void count_nibbles(uint32_t w, uint32_t (&cnt)[16]) {
    constexpr uint32_t M = 0x11111111u;
    uint32_t b[4], nb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        b[j] = (w >> j) & M;
        nb[j] = b[j] ^ M;
    }
    const uint32_t lo[4] = {nb[1] & nb[0], nb[1] & b[0], b[1] & nb[0], b[1] & b[0]};   // bits 1..0 = v & 3
    const uint32_t hi[4] = {nb[3] & nb[2], nb[3] & b[2], b[3] & nb[2], b[3] & b[2]};   // bits 3..2 = v >> 2
#pragma unroll
    for (int v = 0; v < 16; ++v) cnt[v] += (uint32_t)__popc(hi[v >> 2] & lo[v & 3]);
}

// Adds the workgroup's totals of one code per thread to its row of counts:
// thread t holds part (its partial count of code t & 15).  Every thread of
// the workgroup calls it; one 64-bit atomic per nonzero code per workgroup.
__device__ __forceinline__ void add_code_counts(uint32_t part, unsigned long long* counts) {
    __shared__ unsigned long long s_part[kThreads / 64][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned long long v = part;
    v += __shfl_xor(v, 16, 64);                   // the four lanes of a wave with the same code
    v += __shfl_xor(v, 32, 64);
    if (lane < 16) s_part[wave][lane] = v;
    __syncthreads();
    if (threadIdx.x < 16) {
        unsigned long long total = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) total += s_part[w][threadIdx.x];
        if (total) atomicAdd(&counts[(blockIdx.x % kCountReplicas) * 16 + threadIdx.x], total);
    }
}

// Workgroup flush of 16 per-thread register counters (cnt[v] of every
// thread): thread t first gathers code t & 15 from the 16 threads of its
// group of 16 lanes.
__device__ __forceinline__ void flush_code_counts(const uint32_t (&cnt)[16], unsigned long long* counts) {
    const int lane = threadIdx.x & 63;
    uint32_t part = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        // sum of cnt[v] over the 16 lanes of this lane's group; lane v of the group keeps it
        uint32_t c = cnt[v];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) c += (uint32_t)__shfl_xor((int)c, o, 64);
        part = (lane & 15) == v ? c : part;
    }
    add_code_counts(part, counts);
}

// ---------------------------------------------------------------------------
// Encoding of one block at one scale
// ---------------------------------------------------------------------------

// Scales for which the division-free quotient below is exact (see
// quotient()): R = fl(1/S) is then a normal number and so is every residual.
__device__ __forceinline__ bool fast_quotient_range(float S) { return S >= 0x1p-100f && S <= 0x1p100f; }

// fl(a / S) for a >= 0.  E8M0: S is a power of two and R = 1/S exactly, so
// the product is the correctly rounded quotient.  E4M3 with FAST: R =
// fl(1/S); q0 = fl(a R) is within two ulps, the FMA residual a - q0 S is
// exact, and one FMA correction gives the correctly rounded quotient (the
// classic reciprocal-refinement argument; checked exhaustively for every
// fp32 scale mantissa at every E2M1 bin boundary and at 6, the clip bound).
// Otherwise the IEEE division (0 for S == 0).
template <int SF, bool FAST>
__device__ __forceinline__ float quotient(float a, float S, float R) {
    if constexpr (SF == SF_E8M0) {
        return a * R;
    } else if constexpr (FAST) {
        const float q0 = a * R;
        const float rr = __builtin_fmaf(-q0, S, a);
        return __builtin_fmaf(rr, R, q0);
    } else {
        return (S > 0.0f) ? a / S : 0.0f;
    }
}

// Quantize y[OFF, OFF+B) at scale S (usable; R as for quotient()): r[i]
// receives the E2M1 grid value of |y_i| / S; returns the block SSE.
// NAN_GUARD: elements may be NaN (caller-given scales), which encode as 0.
template <int SF, int B, int OFF, bool NAN_GUARD, bool FAST, int U>
__device__ __forceinline__ float encode_block(const float (&y)[U], float S, float R, float (&r)[B]) {
    float e[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
        const float a = fabsf(y[OFF + i]);
        float rr = e2m1_round(quotient<SF, FAST>(a, S, R));
        if constexpr (NAN_GUARD) rr = (a == a) ? rr : 0.0f;
        r[i] = rr;
        const float d = a - rr * S;       // |y| - fl(grid * S): same magnitude as y - yhat
        e[i] = d * d;
    }
    return tree_sum<B>(e);
}

// encode_block at a scale chosen per lane that need not be a power of two
// (E4M3 or UE5M3 times g): division-free when S is in range, IEEE division
// otherwise (extreme g).  A zero scale with finite elements also takes the
// division-free path with R = 0, which yields the quotient 0 that a zero
// scale defines (q0 = 0, residual a, correction 0).
template <int B, int OFF, bool NAN_GUARD, int U>
__device__ __forceinline__ float encode_block_at(const float (&y)[U], float S, float (&r)[B]) {
    const bool zero = !NAN_GUARD && S == 0.0f;
    if (fast_quotient_range(S) || zero)
        return encode_block<SF_E4M3, B, OFF, NAN_GUARD, true>(y, S, zero ? 0.0f : 1.0f / S, r);
    return encode_block<SF_E4M3, B, OFF, NAN_GUARD, false>(y, S, 0.0f, r);
}

// Candidate scales of the brute-force search, one table per workgroup.
// Entry c holds, for the scale S_c of code c (E4M3: fl(dec(c) g), c = 1..126;
// E8M0: 2^(c-127), c = 0..254):
//   sr = (S_c, R_c), R_c = fl(1/S_c) when the division-free quotient applies
//   (exact 2^(127-c) for E8M0);  t0 = T0_c, the largest fp32 a with
//   fl(a / S_c) <= 0.25 (a that encodes to zero);  six = fl(6 S_c), the value
//   a saturated element dequantizes to.
struct BfTable {
    static constexpr int kPad = 8;   // entries past the last code, read by padded work items
    float2 sr[256 + kPad];           // (S_c, R_c)
    float t0[256];                   // T0_c
    float six[256];                  // fl(6 S_c)
    bool fast;                       // every candidate in the division-free range
};

// Largest fp32 a with a / S <= 0.25 + 2^-26 (the rounding boundary above
// 0.25, which itself rounds down to 0.25): the product is exact in double
// and is rounded toward zero to fp32.
__device__ __forceinline__ float zero_bin_limit(float S) {
    const double p = (0.25 + 0x1p-26) * (double)S;
    float t = (float)p;
    if ((double)t > p) t = as_f(as_u(t) - 1u);
    return t;
}

template <int SF>
__device__ __forceinline__ void fill_bf_table(BfTable& t, float g) {
    constexpr uint32_t N = SF == SF_E8M0 ? 255u : scale_top<SF>() + 1u;
    for (uint32_t c = threadIdx.x; c < N; c += kThreads) {
        float S, R;
        if constexpr (SF == SF_E8M0) {
            S = e8m0_value(c);
            R = e8m0_inverse(c);
        } else {
            S = scale_value<SF>(c) * g;
            R = fast_quotient_range(S) ? 1.0f / S : 0.0f;
        }
        t.sr[c] = make_float2(S, R);
        t.t0[c] = zero_bin_limit(S);
        t.six[c] = 6.0f * S;
    }
    // codes past the last one, read by work items padded to a whole number
    // of candidates: a NaN scale gives a NaN SSE, which packs above every
    // real candidate and so never wins
    for (uint32_t c = N + threadIdx.x; c < 256u + BfTable::kPad; c += kThreads)
        t.sr[c] = make_float2(__builtin_nanf(""), __builtin_nanf(""));
    if (threadIdx.x == 0)
        t.fast = SF == SF_E8M0 || (fast_quotient_range(scale_value<SF>(1u) * g) &&
                                   fast_quotient_range(scale_value<SF>(scale_top<SF>()) * g));
    __syncthreads();
}

// Exact brute-force search ("Finer is Better (with the Right Scaling)",
// method part 2: the scale with the least block MSE among all representable
// ones; ties to the smaller code) by branch and bound.  Every code outside
// the window [c_lo, c_hi) provably has a larger fp32 tree SSE than the best
// of the two start codes, so the minimum over the start codes and the window
// is the exhaustive argmin:
//  * upper side: an element with a <= T0_c encodes to 0 at scale c and adds
//    exactly fl(a*a) to the tree.  With scales in the division-free range
//    (S_c normal, so H_c = S_c / 2 is the exact dequantized value of grid
//    point 0.5), an element with T0_c < a <= H_c encodes to 0.5 (its
//    quotient lies in (0.25, 0.5]) and adds exactly fl((H_c - a)^2).  Both
//    terms only grow with c: (H_c - a)^2 grows with S_c, and where the
//    element enters the zero bin (a <= T0_c, so S_c < 4a before) it
//    becomes fl(a*a) >= fl((H_c - a)^2).  So the tree over these terms (0
//    for every other element) is a lower bound of SSE_c (fp32 addition is
//    monotone) that only grows with c; codes from the first one whose bound
//    exceeds the best are skipped, and once every element encodes to 0
//    (a_max <= T0_c) all larger codes tie with c, so nothing above c can
//    win;
//  * lower side: while fl(6 S_c) <= a_max the block maximum saturates and
//    contributes fl((a_max - fl(6 S_c))^2) <= SSE_c, which shrinks as c
//    grows; codes below the first one whose term is <= best are skipped.
// Both window ends come from binary searches (the predicates are monotone).
// Returns the best start candidate packed as (SSE bits << 32) | code: for
// non-negative floats the bit patterns order like the values, so the
// smallest packed value is the smallest SSE, ties to the smallest code.
__device__ __forceinline__ unsigned long long pack_candidate(float sse, uint32_t code) {
    return ((unsigned long long)as_u(sse) << 32) | code;
}

// First index in [lo, hi) where the monotone predicate (false ... true)
// holds, or hi.  Starts at a guess and doubles its step outwards, so a good
// guess costs two or three predicate evaluations; then bisects the bracket.
template <class Pred>
__device__ __forceinline__ uint32_t first_true_from(uint32_t lo, uint32_t hi, uint32_t guess, Pred pred) {
    if (lo >= hi) return hi;
    guess = guess < lo ? lo : (guess >= hi ? hi - 1 : guess);
    uint32_t a, b;                        // pred(a - 1) false (or a == lo), pred(b) true (or b == hi)
    if (pred(guess)) {
        b = guess;
        uint32_t step = 1;
        a = lo;
#pragma unroll 1
        while (b > lo) {
            const uint32_t c = b - lo > step ? b - step : lo;
            if (!pred(c)) { a = c + 1; break; }
            b = c;
            step <<= 1;
        }
    } else {
        a = guess + 1;
        uint32_t step = 1;
        b = hi;
#pragma unroll 1
        while (a < hi) {
            const uint32_t c = hi - a > step ? a + step - 1 : hi - 1;
            if (pred(c)) { b = c; break; }
            a = c + 1;
            step <<= 1;
        }
    }
#pragma unroll 1
    while (a < b) {
        const uint32_t mid = (a + b) >> 1;
        if (pred(mid)) b = mid; else a = mid + 1;
    }
    return a;
}

// first_true_from for an answer expected within 2^L - 1 codes above lo: one
// evaluation at lo + 2^L - 1 confirms that, then L bisection steps with a
// fixed trip count find it, so the lanes of a wave stay in step.  An answer
// further up continues with the general search.
template <int L, class Pred>
__device__ __forceinline__ uint32_t first_true_up(uint32_t lo, uint32_t hi, Pred pred) {
    constexpr uint32_t span = (1u << L) - 1u;
    if (lo >= hi) return hi;
    uint32_t cap;                         // the answer lies in [lo, cap] (cap == hi: none)
    if (hi - lo > span) {
        cap = lo + span;
        if (!pred(cap)) return first_true_from(cap + 1u, hi, cap + 1u, pred);
    } else {
        cap = hi;
    }
    uint32_t pos = lo;
#pragma unroll
    for (int st = L - 1; st >= 0; --st) {
        const uint32_t probe = pos + (1u << st) - 1u;
        if (probe < cap && !pred(probe)) pos += 1u << st;
    }
    return pos;
}

// The mirror image: an answer expected within 2^L - 1 codes below hi.
template <int L, class Pred>
__device__ __forceinline__ uint32_t first_true_down(uint32_t lo, uint32_t hi, Pred pred) {
    constexpr uint32_t span = (1u << L) - 1u;
    if (lo >= hi) return hi;
    uint32_t base = lo;                   // the answer lies in [base, hi] (hi: none)
    if (hi - lo > span) {
        base = hi - span;
        if (pred(base - 1u)) return first_true_from(lo, base, base - 1u, pred);
    }
    uint32_t pos = base;
#pragma unroll
    for (int st = L - 1; st >= 0; --st) {
        const uint32_t probe = pos + (1u << st) - 1u;
        if (probe < hi && !pred(probe)) pos += 1u << st;
    }
    return pos;
}

template <int SF, int B, int OFF, bool FAST, int U>
__device__ __forceinline__ unsigned long long bf_window(const float (&y)[U], float a_b, uint32_t c_first,
                                                        uint32_t c_second, const BfTable& t, uint32_t& c_lo,
                                                        uint32_t& c_hi) {
    constexpr uint32_t CLO = SF == SF_E8M0 ? 0u : 1u;           // candidate codes [CLO, CEND)
    constexpr uint32_t CEND = SF == SF_E8M0 ? 255u : scale_top<SF>() + 1u;
    // Window ends are searched within 2^L codes of the start: 4 binades of
    // an 8-code-per-binade format above, 2 below; E8M0 codes are binades.
    constexpr int L_UP = SF == SF_E8M0 ? 3 : 5;
    constexpr int L_DOWN = SF == SF_E8M0 ? 2 : 4;
    // the half-bin term needs exact halves of the scales (normal S_c)
    constexpr bool HALF_BIN = FAST;
    // every element encodes to zero at the smallest scale: all codes tie
    if (a_b <= t.t0[CLO]) {
        c_lo = c_hi = CLO;
        return pack_candidate(0.0f, CLO);   // callers recompute the SSE at the winning code
    }
    float rc[B];
    const float2 e1 = t.sr[c_first], e2 = t.sr[c_second];
    unsigned long long best = pack_candidate(encode_block<SF, B, OFF, false, FAST>(y, e1.x, e1.y, rc), c_first);
    if (c_second != c_first) {
        const unsigned long long b2 =
            pack_candidate(encode_block<SF, B, OFF, false, FAST>(y, e2.x, e2.y, rc), c_second);
        best = b2 < best ? b2 : best;
    }
    const float best0 = as_f((uint32_t)(best >> 32));
    const uint32_t c_best = (uint32_t)(best & 0xFFFFFFFFull);

    // upper end: first code past c_best whose bound exceeds best0, or whose
    // every element encodes to zero (that code is still evaluated)
    float a[B], sq[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
        a[i] = fabsf(y[OFF + i]);
        sq[i] = a[i] * a[i];
    }
    auto stop_up = [&](uint32_t c) {
        const float T0 = t.t0[c];
        float z[B];
        if constexpr (HALF_BIN) {
            // min(fl(max(H - a, 0)^2), fl(a^2)) per element: the exact term
            // of the lower half of the 0.5 bin, of the zero bin (there
            // a <= S/4, so the second square is the smaller, except in the
            // rounding sliver just above S/4 where the first one is still a
            // lower bound), and 0 above H.  It grows with S_c, so the bound
            // keeps its monotonicity without a bin test.
            const float H = 0.5f * t.sr[c].x;
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const float d = fmaxf(H - a[i], 0.0f);
                z[i] = fminf(d * d, sq[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < B; ++i) z[i] = a[i] <= T0 ? sq[i] : 0.0f;
        }
        return tree_sum<B>(z) > best0 || a_b <= T0;
    };
    c_hi = first_true_up<L_UP>(c_best + 1u, CEND, stop_up);
    if (c_hi < CEND && a_b <= t.t0[c_hi]) ++c_hi;

    // lower end: below c_star the block maximum saturates (fl(6 S) <= a_max) and
    // contributes (a_max - fl(6 S))^2; skip the codes where that exceeds best0
    const uint32_t c_star = first_true_from(CLO, CEND, c_first, [&](uint32_t c) { return t.six[c] > a_b; });
    c_lo = first_true_down<L_DOWN>(CLO, c_star, [&](uint32_t c) {
        const float d = a_b - t.six[c];
        return d * d <= best0;
    });
    return best;
}

// Scale selection + encoding of block number BI of a unit.
constexpr int code_words(int U) { return (U + 7) / 8; }

// Pack the codes of block OFF/B into the unit's code words and hand its
// dequantized values (fp32) to emit(off, values), four at a time.
template <int B, int OFF, int U, class Emit>
__device__ __forceinline__ void finish_block(const float (&y)[U], const float (&r)[B], float S, bool nan_block,
                                             uint32_t (&cw)[code_words(U)], Emit&& emit) {
#pragma unroll
    for (int i0 = 0; i0 < B; i0 += 4) {
        float dq4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + k;
            const uint32_t sgn = as_u(y[OFF + i]) >> 31;
            uint32_t nib;
            if (nan_block) {
                nib = sgn << 3;
                dq4[k] = canonical_nan_like(y[OFF + i]);
            } else {
                nib = (sgn << 3) | e2m1_code_of(r[i]);
                dq4[k] = with_sign_of(r[i] * S, y[OFF + i]);
            }
            cw[(OFF + i) / 8] |= nib << (4 * ((OFF + i) % 8));
        }
        emit(OFF + i0, dq4);
    }
}

template <int SF, int ST, int B, int BI, int U, class Emit>
__device__ __forceinline__ void quant_block(const float (&y)[U], float g, float six_g, float four_g,
                                            int prevent_zero, uint32_t given, uint32_t (&cw)[code_words(U)],
                                            Emit&& emit, uint32_t& scale_code, float& sse) {
    constexpr int OFF = BI * B;
    uint32_t sc;
    bool nan_block;
    float S = 0.0f;
    float r[B];

    if constexpr (ST == ST_GIVEN) {
        if constexpr (SF == SF_E8M0) {
            sc = given & 0xFFu;
            nan_block = sc == kE8M0NaN;
            S = e8m0_value(sc);
            if (!nan_block) sse = encode_block<SF, B, OFF, true, true>(y, S, e8m0_inverse(sc), r);
        } else {
            sc = given & scale_code_mask<SF>();
            S = scale_value<SF>(sc) * g;
            nan_block = sc == scale_nan<SF>() || !scale_usable(S);
            if (!nan_block) sse = encode_block_at<B, OFF, true>(y, S, r);
        }
    } else {
        uint32_t ab = 0;
#pragma unroll
        for (int i = 0; i < B; ++i) ab = max(ab, as_u(y[OFF + i]) & 0x7FFFFFFFu);
        const float a_b = as_f(ab);
        nan_block = ab >= 0x7F800000u || !(g < __builtin_inff());   // also catches NaN g
        if (!nan_block) {
            if constexpr (SF == SF_E8M0) {
                sc = e8m0_absmax_code(ab);
                S = e8m0_value(sc);
                sse = encode_block<SF, B, OFF, false, true>(y, S, e8m0_inverse(sc), r);
            } else {
                const uint32_t s6 = scale_encode<SF>(a_b / six_g);
                if constexpr (ST == ST_ABSMAX) {
                    sc = (prevent_zero && s6 == 0u) ? 1u : s6;
                    S = scale_value<SF>(sc) * g;
                    sse = encode_block_at<B, OFF, false>(y, S, r);
                } else {
                    static_assert(ST == ST_FOUR_OVER_SIX, "brute force has its own kernel");
                    const uint32_t s4 = scale_encode<SF>(a_b / four_g);
                    const float S6 = scale_value<SF>(s6) * g, S4 = scale_value<SF>(s4) * g;
                    float r4[B];
                    const float e6 = encode_block_at<B, OFF, false>(y, S6, r);
                    const float e4 = encode_block_at<B, OFF, false>(y, S4, r4);
                    const bool take4 = e4 < e6;   // equal error keeps the smaller code s6
                    sc = take4 ? s4 : s6;
                    S = take4 ? S4 : S6;
                    sse = take4 ? e4 : e6;
#pragma unroll
                    for (int i = 0; i < B; ++i) r[i] = take4 ? r4[i] : r[i];
                }
            }
        } else {
            sc = scale_nan<SF>();
        }
    }

    scale_code = sc;
    if (nan_block) sse = as_f(kQNaN);
    finish_block<B, OFF>(y, r, S, nan_block, cw, emit);
}

// ---------------------------------------------------------------------------
// Coalesced tile I/O through LDS.  A wave owns a tile of 64 consecutive
// units of a contiguous tensor.  Global memory is touched 16 bytes per lane
// with consecutive lanes on consecutive addresses; LDS re-distributes the
// bytes so that each lane holds its own unit.  Units sit in LDS slots padded
// by 16 bytes, which spreads the 16-byte reads of 16 consecutive lanes over
// all banks.  Only the owning wave touches its LDS region, so a wave-level
// compiler barrier orders the exchange.
// ---------------------------------------------------------------------------

constexpr int kTileUnits = 64;

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bytes of one unit's LDS slot: U values of at most 4 bytes plus padding.
template <int U>
constexpr int slot_bytes() { return U * 4 + 16; }

// Load the tile's input (nvalid units of U elements of type T starting at
// base) and return this lane's unit widened to fp32.
template <class T, int U>
__device__ __forceinline__ void tile_load(const T* __restrict__ base, int nvalid, char* lds, int lane,
                                          float (&y)[U]) {
    constexpr int ES = ElemSize<T>::value;
    constexpr int C = U * ES / 16;                   // 16-byte chunks per unit
    constexpr int SLOT = slot_bytes<U>();
    const int nchunks = nvalid * C;
    const uint4* src = reinterpret_cast<const uint4*>(base);
#pragma unroll
    for (int k = 0; k < C; ++k) {
        const int j = k * 64 + lane;
        if (j < nchunks) {
            const uint4 v = src[j];
            *reinterpret_cast<uint4*>(lds + (j / C) * SLOT + (j % C) * 16) = v;
        }
    }
    wave_sync_lds();
    load_elems<T, U>(reinterpret_cast<const T*>(lds + lane * SLOT), y);
    wave_sync_lds();
}

// Copy a tile of nvalid units whose values (type of size EO) sit in the
// lanes' LDS slots to out_base, 16 coalesced bytes per lane, as streaming
// stores.
template <int U, int EO>
__device__ __forceinline__ void tile_flush_t(void* __restrict__ out_base, int nvalid, const char* lds, int lane) {
    constexpr int UB = U * EO;                 // bytes of one unit
    constexpr int SLOT = slot_bytes<U>();
    uint4* dst = reinterpret_cast<uint4*>(out_base);
    wave_sync_lds();
    if constexpr (UB >= 16) {
        constexpr int C = UB / 16;
        const int nchunks = nvalid * C;
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const int j = k * 64 + lane;
            if (j < nchunks) store_stream(dst + j, *reinterpret_cast<const uint4*>(lds + (j / C) * SLOT + (j % C) * 16));
        }
    } else {
        static_assert(UB == 8, "units of 4 two-byte values");
        const int nchunks = nvalid / 2;        // pairs of units
        if (lane < nchunks) {
            const uint2 a = *reinterpret_cast<const uint2*>(lds + (2 * lane) * SLOT);
            const uint2 b = *reinterpret_cast<const uint2*>(lds + (2 * lane + 1) * SLOT);
            store_stream(dst + lane, make_uint4(a.x, a.y, b.x, b.y));
        }
        if ((nvalid & 1) && lane == nvalid - 1)
            store_stream(reinterpret_cast<uint2*>(out_base) + lane, *reinterpret_cast<const uint2*>(lds + lane * SLOT));
    }
    wave_sync_lds();
}

template <int U>
__device__ __forceinline__ void tile_flush(void* __restrict__ out_base, int dt, int nvalid, const char* lds, int lane) {
    if (dt == DT_F32) tile_flush_t<U, 4>(out_base, nvalid, lds, lane);
    else tile_flush_t<U, 2>(out_base, nvalid, lds, lane);
}

// Store U/2 packed code bytes from code words.
template <int U>
__device__ __forceinline__ void store_code_words(uint8_t* __restrict__ p, const uint32_t (&cw)[code_words(U)]) {
    if constexpr (U == 32) *reinterpret_cast<uint4*>(p) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    else if constexpr (U == 16) *reinterpret_cast<uint2*>(p) = make_uint2(cw[0], cw[1]);
    else if constexpr (U == 8) *reinterpret_cast<uint32_t*>(p) = cw[0];
    else *reinterpret_cast<uint16_t*>(p) = (uint16_t)cw[0];
}

// Destination of a unit's dequantized values: the lane's LDS slot when the
// tile is flushed coalesced afterwards (contiguous tensors), else the strided
// output itself.  Kept as two pointers so that each store keeps its address
// space.
template <int U>
struct DqSink {
    char* slot;          // LDS slot, or null
    void* out;           // global output, or null
    int64_t off;         // element offset of the unit in out
    int dt;
    bool direct;         // contiguous fp32 units of 4: one streaming 16-byte store per lane
    __device__ __forceinline__ void operator()(int o, const float (&v)[4]) const {
        if (slot) {
            store_elems_rt<4>(slot, dt, o, v);
        } else if (out) {
            if (direct) store_stream_f32<4>(reinterpret_cast<float*>(out) + off + o, v);
            else store_elems_rt<4>(out, dt, off + o, v);
        }
    }
};

// Contiguous tensors whose unit is exactly 16 bytes need no LDS exchange:
// lane l's unit is already the l-th 16-byte piece of the tile.  For the
// input that holds for units of 4 fp32 or 8 16-bit values, for the fp32
// dequantized output for units of 4.
template <class InT, int U>
constexpr bool bf_direct_input() { return U * ElemSize<InT>::value == 16; }
template <int U, class P>
__device__ __forceinline__ bool bf_direct_dq(const P& p) { return U == 4 && p.contiguous && p.dq_dt == DT_F32; }

template <int U, class P>
__device__ __forceinline__ DqSink<U> dq_sink(const P& p, char* lds, int lane, int64_t u, bool active) {
    if (!p.dq) return {nullptr, nullptr, 0, 0, false};
    const bool direct = bf_direct_dq<U>(p);
    if (p.contiguous && !direct) return {lds + lane * slot_bytes<U>(), nullptr, 0, p.dq_dt, false};
    if (!active) return {nullptr, nullptr, 0, 0, false};
    return {nullptr, p.dq, unit_offset<U>(u, p.units_per_row, p.ld_dq, p.contiguous), p.dq_dt, direct};
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Per-tensor scale search (MR-GPTQ page, section 2.2: scales chosen per
// tensor for minimum MSE).  Candidate g_j = fl(g0 (1 - j/64)); its score is
// the fp64 balanced tree over all blocks (row-major, zero-padded to a power
// of two) of the fp32 block SSE the strategy reaches at g_j.  A tile's 64 x NB
// blocks are an aligned subtree: each lane sums its NB blocks as a tree, the
// wave combines lanes with an xor butterfly (pairs of neighbours first, so the
// same tree), and lane 0 stores the tile's subtree sum; k_tree_reduce_f64
// then combines tiles 512 at a time, again as aligned subtrees.
// ---------------------------------------------------------------------------

// fp32 SSE of block BI at scale factor g under abs-max (prevent-zero) or
// 4-over-6, as quant_block chooses and scores it; NaN for a NaN block.
template <int ST, int B, int BI, int U>
__device__ __forceinline__ float block_score(const float (&y)[U], uint32_t ab, float g, float six_g, float four_g,
                                             int prevent_zero) {
    constexpr int OFF = BI * B;
    if (ab >= 0x7F800000u || !(g < __builtin_inff())) return as_f(kQNaN);
    const float a_b = as_f(ab);
    const uint32_t s6 = e4m3_encode(a_b / six_g);
    float r[B];
    if constexpr (ST == ST_ABSMAX) {
        const uint32_t sc = (prevent_zero && s6 == 0u) ? 1u : s6;
        return encode_block_at<B, OFF, false>(y, e4m3_value(sc) * g, r);
    } else {
        static_assert(ST == ST_FOUR_OVER_SIX, "abs-max, prevent-zero or 4-over-6");
        const uint32_t s4 = e4m3_encode(a_b / four_g);
        const float e6 = encode_block_at<B, OFF, false>(y, e4m3_value(s6) * g, r);
        const float e4 = encode_block_at<B, OFF, false>(y, e4m3_value(s4) * g, r);
        return e4 < e6 ? e4 : e6;
    }
}

template <class InT, int B, int H, int ST>
__global__ __launch_bounds__(kThreads) void k_gsearch(GSearchArgs p) {
    constexpr int U = unit_elems<InT, B, H>();
    constexpr int NB = U / B;
    __shared__ __attribute__((aligned(16))) char s_tiles[kThreads / 64][kTileUnits * slot_bytes<U>()];
    const InT* x = reinterpret_cast<const InT*>(p.x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    char* lds = s_tiles[wave];
    const float g0 = workgroup_amax_scale(p.amax_partials, p.n_partials);

    const int64_t ntiles = (p.units + kTileUnits - 1) / kTileUnits;
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave; t < ntiles; t += tstride) {
        const int64_t u0 = t * kTileUnits;
        const int nvalid = (int)min<int64_t>(kTileUnits, p.units - u0);
        const int64_t u = u0 + lane;
        const bool active = lane < nvalid;
        float y[U];
        if (p.contiguous) {
            tile_load<InT, U>(x + u0 * U, nvalid, lds, lane, y);
        } else if (active) {
            load_elems<InT, U>(x + unit_offset<U>(u, p.units_per_row, p.ld_x, false), y);
        } else {
#pragma unroll
            for (int i = 0; i < U; ++i) y[i] = 0.0f;
        }
        if constexpr (H > 0) fwht_segments<H, U>(y);
        uint32_t ab[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            ab[b] = 0;
#pragma unroll
            for (int i = 0; i < B; ++i) ab[b] = max(ab[b], as_u(y[b * B + i]) & 0x7FFFFFFFu);
        }
#pragma unroll 1
        for (int j = 0; j < kSearchCandidates; ++j) {
            const float g = g0 * search_factor(j);
            const float six_g = 6.0f * g, four_g = 4.0f * g;
            double e[NB];
            static_for<NB>([&](auto bi) {
                constexpr int b = decltype(bi)::value;
                e[b] = (double)block_score<ST, B, b>(y, ab[b], g, six_g, four_g, p.prevent_zero);
            });
            double s = active ? tree_sum<NB>(e) : 0.0;      // lanes past the tensor are padding
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) s = s + __shfl_xor(s, o, 64);
            if (lane == 0) p.partials[j * p.ntiles + t] = s;
        }
    }
}

// Outputs of one tile: codes, scales, SSE and MSE from the lanes' registers;
// the dequantized values, already in the LDS slots for contiguous tensors,
// are flushed coalesced.
template <int B, int U>
__device__ __forceinline__ void store_unit_outputs(const QuantArgs& p, int64_t u0, int nvalid, int lane,
                                                   const char* lds, const uint32_t (&cw)[code_words(U)],
                                                   const uint32_t (&sc)[U / B], const float (&sse)[U / B],
                                                   bool write_scales) {
    constexpr int NB = U / B;
    const int64_t u = u0 + lane;
    if (lane < nvalid) {
        if (p.codes) store_code_words<U>(p.codes + u * (U / 2), cw);
        if (write_scales) {
#pragma unroll
            for (int b = 0; b < NB; ++b) p.scales[u * NB + b] = (uint8_t)sc[b];
        }
        if (p.sse) store_stream_f32<NB>(p.sse + u * NB, sse);
        if (p.mse) {
            float m[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float v = sse[b] * (1.0f / (float)B);   // exact: B is a power of two
                m[b] = (v == v) ? v : as_f(kQNaN);
            }
            store_stream_f32<NB>(p.mse + u * NB, m);
        }
    }
    if (p.dq && p.contiguous && !bf_direct_dq<U>(p)) {
        const int eo = p.dq_dt == DT_F32 ? 4 : 2;
        tile_flush<U>(reinterpret_cast<char*>(p.dq) + u0 * U * eo, p.dq_dt, nvalid, lds, lane);
    }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = (uint32_t)__shfl_up((int)v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// LDS of one wave of the brute-force kernels: the tile's fp32 values (one
// padded slot per lane), each block's best candidate, and the work list.
template <int U, int B>
struct BfWaveLds {
    static constexpr int NBLK = kTileUnits * (U / B);
    static constexpr int NMASK = B <= 8 ? NBLK : 1;   // candidate masks (bf_search_tile_mask)
    char tile[kTileUnits * slot_bytes<U>()];
    unsigned long long best[NBLK];
    uint32_t start[NBLK + 1];
    uint8_t clo[NBLK];
    unsigned long long mask[NMASK];
    uint8_t mbase[NMASK];
    uint8_t movf[NMASK];
};

// Brute-force search of one tile (exhaustive argmin, computed as branch and
// bound).  Each lane publishes its (rotated) fp32 values y in LDS and finds,
// for each of its blocks, the best of two start scales and the window of
// codes that can still beat it (bf_window).  The windows of all blocks of the
// tile form one work list that the 64 lanes split evenly: a work item is K
// consecutive codes of one block (K = 16 / B for small blocks, which gives a
// lane independent candidates to interleave; a window is padded to whole
// items).  A lane walks its slice, evaluates the items with the block's
// values read from LDS, and merges its per-block minimum into an LDS 64-bit
// atomic minimum over (SSE bits, code).  FAST: every candidate scale is in
// the division-free range (BfTable::fast; the choice is a template
// parameter so that no per-candidate branch is left for the compiler to
// speculate both ways).  On return W.best[lane * NB + b]
// holds the winning code of each finite block in its low word (its high
// word is the SSE the search saw, 0 for a block whose elements all encode
// to zero at every scale), and nan_blk[b] flags blocks with a NaN or
// infinite value or a non-finite g.  Idle lanes (active false) must hold
// zeros in y.
template <int SF, int B, int U, bool FAST>
__device__ __forceinline__ void bf_search_tile(const float (&y)[U], bool active, float g, float inv_six_g,
                                               float inv_four_g, const BfTable& s_bf, BfWaveLds<U, B>& W, int lane,
                                               bool (&nan_blk)[U / B]) {
    constexpr int NB = U / B;
    constexpr int SLOT = slot_bytes<U>();
    constexpr int NBLK = kTileUnits * NB;
    constexpr uint32_t CEND = SF == SF_E8M0 ? 255u : scale_top<SF>() + 1u;
    constexpr int K = B >= 16 ? 1 : 16 / B;       // candidates of one block per work item
    // an item reads codes c0 .. c0 + K - 1 with c0 < CEND
    static_assert(CEND + K - 1 <= 256 + BfTable::kPad, "items read past the table");

    // publish the fp32 values of this lane's unit
#pragma unroll
    for (int i = 0; i < U / 4; ++i)
        reinterpret_cast<float4*>(W.tile + lane * SLOT)[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);

    // start candidates and windows of this lane's blocks
    uint32_t n[NB], clo[NB];
    static_for<NB>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        uint32_t ab = 0;
#pragma unroll
        for (int i = 0; i < B; ++i) ab = max(ab, as_u(y[b * B + i]) & 0x7FFFFFFFu);
        nan_blk[b] = ab >= 0x7F800000u || !(g < __builtin_inff());
        n[b] = 0;
        clo[b] = 0;
        unsigned long long best = ~0ull;
        if (!nan_blk[b] && active) {
            const float a_b = as_f(ab);
            uint32_t c1, c2;
            if constexpr (SF == SF_E8M0) {
                c1 = e8m0_absmax_code(ab);
                c2 = c1 < 254u ? c1 + 1u : c1;
            } else {
                const uint32_t s6 = scale_encode<SF>(a_b * inv_six_g), s4 = scale_encode<SF>(a_b * inv_four_g);
                c1 = s6 > 0u ? s6 : 1u;
                c2 = s4 > 0u ? s4 : 1u;
            }
            uint32_t lo, hi;
            best = bf_window<SF, B, b * B, FAST>(y, a_b, c1, c2, s_bf, lo, hi);
            clo[b] = lo;
            n[b] = hi > lo ? (hi - lo + K - 1) / K : 0u;     // work items of K codes
        }
        W.best[lane * NB + b] = best;
    });

    // one work list for the tile
    uint32_t mine = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) mine += n[b];
    const uint32_t incl = wave_inclusive_sum(mine, lane);
    const uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
    uint32_t run = incl - mine;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        W.start[lane * NB + b] = run;
        W.clo[lane * NB + b] = (uint8_t)clo[b];
        run += n[b];
    }
    if (lane == 63) W.start[NBLK] = total;
    wave_sync_lds();

    const uint32_t j0 = (uint32_t)(((uint64_t)total * lane) >> 6);
    const uint32_t j1 = (uint32_t)(((uint64_t)total * (lane + 1)) >> 6);
    if (j0 < j1) {
        // block k containing item j0: the largest k with start[k] <= j0
        uint32_t lo = 0, hi = NBLK;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if (W.start[mid] <= j0) lo = mid; else hi = mid - 1;
        }
        uint32_t k = lo;
        auto load_block = [&](uint32_t kk, float (&dst)[B]) {
            const float4* src = reinterpret_cast<const float4*>(W.tile + (kk / NB) * SLOT + (kk % NB) * B * 4);
#pragma unroll
            for (int i = 0; i < B / 4; ++i) {
                const float4 v = src[i];
                dst[4 * i] = v.x; dst[4 * i + 1] = v.y; dst[4 * i + 2] = v.z; dst[4 * i + 3] = v.w;
            }
        };
        float yb[B];
        load_block(k, yb);
        uint32_t k_begin = W.start[k], k_end = W.start[k + 1], k_clo = W.clo[k];
        unsigned long long local = ~0ull;
#pragma unroll 1
        for (uint32_t j = j0; j < j1; ++j) {
            while (j >= k_end) {
                atomicMin(&W.best[k], local);
                local = ~0ull;
                ++k;
                k_begin = k_end;
                k_end = W.start[k + 1];
                k_clo = W.clo[k];
                if (j < k_end) load_block(k, yb);
            }
            // K consecutive codes of block k.  The last item of a window may run
            // past its end: those codes are real candidates (more candidates
            // cannot change the argmin) or table padding (NaN SSE)
            const uint32_t c0 = k_clo + K * (j - k_begin);
            float2 es[K];
#pragma unroll
            for (int q = 0; q < K; ++q) es[q] = s_bf.sr[c0 + q];
#pragma unroll
            for (int q = 0; q < K; ++q) {
                const uint32_t c = c0 + q;
                const float2 e = es[q];
                float rc[B];
                const float sse = encode_block<SF, B, 0, false, FAST>(yb, e.x, e.y, rc);
                const unsigned long long cand = pack_candidate(sse, c);
                local = cand < local ? cand : local;
            }
        }
        atomicMin(&W.best[k], local);
    }
    wave_sync_lds();
}

// ---------------------------------------------------------------------------
// Brute force for blocks of 4 with E4M3 scales in the division-free range:
// candidate masks instead of the window.  Each element's squared error is
// one term of the block's tree sum, and a tree sum of non-negative terms is
// at least each term, so a code c can only reach SSE_c <= tau (tau = the
// best start SSE) if every element's own error e_i(c) <= tau.  For an
// element a the computed error (a - fl(r S))^2 with r on the E2M1 grid is at
// most tau only if |a - r S| <= delta, delta = sqrt(tau) plus the rounding
// of the product, difference and square, for some grid value r in {6, 4,
// 3, 2, 1.5, 1, 0.5} (r = 0 needs a <= delta).  So the admissible scales of
// a are the union of the intervals S in [(a - delta) / r, (a + delta) / r]:
// in E4M3 codes of S / g, the r = 6 interval and its doublings (r = 3, 1.5)
// and the r = 4 interval and its doublings (r = 2, 1, 0.5), where doubling a
// value adds 8 to a normal code (and about doubles a subnormal one; those
// bounds are widened by a code).  The candidates of a block are the codes
// admissible for both its largest and its second largest element, minus the
// two start codes already evaluated; every other code has SSE > tau and
// cannot win.  Masks are 64 codes wide from the lowest admissible code of
// the largest element; codes of its intervals above that frame (possible
// only for a very large tau) are all kept as candidates.
// ---------------------------------------------------------------------------

// E4M3 codes of a scale value u (in units of g) in the normal range (u >=
// 2^-6, code 8 up): the smallest code with a value >= u and the largest
// with a value <= u, from the fp32 bits ((e + 7) << 3 | top mantissa bits).
// Below 2^-6 they return 0 and 8, bounds that contain every subnormal code;
// far above 448 or for an infinite u they return codes past 126.
__device__ __forceinline__ int e4m3_code_ceil(float u) {
    return u < 0x1p-6f ? 0 : (int)((as_u(u) + 0xFFFFFu) >> 20) - 960;
}
__device__ __forceinline__ int e4m3_code_floor(float u) {
    return u < 0x1p-6f ? 8 : (int)(as_u(u) >> 20) - 960;
}

// The same with the subnormal codes m 2^-9 (m = 1..7) resolved.
__device__ __forceinline__ int e4m3_code_ceil_sub(float u) {
    if (u >= 0x1p-6f) return e4m3_code_ceil(u);
    return u > 0.0f ? (int)__builtin_ceilf(u * 512.0f) : 0;
}
__device__ __forceinline__ int e4m3_code_floor_sub(float u) {
    if (u >= 0x1p-6f) return e4m3_code_floor(u);
    return u > 0.0f ? (int)(u * 512.0f) : -1;
}

// A bound on the code of twice a code's value: + 8 for normal codes; below
// code 8 (value m 2^-9) twice the value is code 2m, so the bounds widen by
// one code to stay on the safe side.
__device__ __forceinline__ int doubled_lo(int l) { return min(2 * l - 1, l + 8); }
__device__ __forceinline__ int doubled_hi(int h) { return min(2 * h + 1, h + 8); }

// Bits 0 .. w (nothing for w < 0, all for w >= 63).
__device__ __forceinline__ unsigned long long low_bits(int w) {
    return w < 0 ? 0ull : (~0ull >> (63 - (w < 63 ? w : 63)));
}

// Bits [l - base, h - base] of a 64-code frame (nothing when empty).
__device__ __forceinline__ unsigned long long frame_bits(int l, int h, int base) {
    int lo = l - base, hi = h - base;
    lo = lo < 0 ? 0 : lo;
    hi = hi > 63 ? 63 : hi;
    return lo <= hi ? ((~0ull >> (63 - (hi - lo))) << lo) : 0ull;
}

// Admissible codes of one element a, as a pattern relative to its lowest
// admissible code l6 (the r = 6 bound): the r = 6 and r = 4 intervals and
// their doublings, 8 codes apart.  inv6 / inv4 are fl(1 / fl(6 g)) and
// fl(1 / fl(4 g)) times (1 -+ 2^-18) for the lower / upper bounds (margin
// for the rounding of the bounds themselves).  When the r = 6 interval
// reaches below code 8 the doubling is not a shift by 8: then every code
// between the lowest and the highest bound is kept.  top receives the
// highest admissible code (the r = 0.5 end), and sat is set when admissible
// codes may lie past bit 63 of the pattern.
__device__ __forceinline__ unsigned long long element_pattern(float a, float delta, float inv6_lo, float inv6_hi,
                                                              float inv4_lo, float inv4_hi, int& l6, int& top,
                                                              bool& sat) {
    const float lo = a - delta, hi = a + delta;
    l6 = e4m3_code_ceil(lo * inv6_lo);
    const int h6 = e4m3_code_floor(hi * inv6_hi);
    const int l4 = e4m3_code_ceil(lo * inv4_lo);
    const int h4 = e4m3_code_floor(hi * inv4_hi);
    const unsigned long long p6 = low_bits(h6 - l6);
    const int d46 = l4 - l6;                                        // 4 to 6 for normal codes (ratio 1.5)
    const unsigned long long p4 = low_bits(h4 - l4) << (d46 < 63 ? d46 : 63);
    const unsigned long long q = p6 | p4;
    unsigned long long pat = q | (q << 8) | (q << 16) | (p4 << 24);
    top = h4 + 24;
    if (l6 < 8) {
        // subnormal codes involved (rare, and a few codes only): every code
        // from the r = 6 lower bound to the r = 0.5 upper bound
        l6 = e4m3_code_ceil_sub(lo * inv6_lo);
        top = doubled_hi(doubled_hi(doubled_hi(e4m3_code_floor_sub(hi * inv4_hi))));
        pat = low_bits(top - l6);
    }
    sat = top - l6 > 63;
    return pat;
}

// A pattern of codes relative to code l (bit i = code l + i) moved into the
// frame from base; when sat, the pattern may continue past its bit 63 and
// the frame bits it would reach are kept.
__device__ __forceinline__ unsigned long long place_pattern(unsigned long long pat, int l, bool sat, int base) {
    const int sh = l - base;
    if (sh >= 0) return sh < 64 ? pat << sh : 0ull;
    unsigned long long m = sh > -64 ? pat >> -sh : 0ull;
    if (sat) m |= sh > -64 ? ~0ull << (64 + sh) : ~0ull;
    return m;
}

// Blocks of 4: the masks alone (no window).  Blocks of 8: the window of
// bf_window (its bounds on the zero bin and the saturated maximum cut what
// two elements cannot) intersected with the masks.
template <int U, int B>
__device__ __forceinline__ void bf_search_tile_mask(const float (&y)[U], bool active, float g, float inv_six_g,
                                                    float inv_four_g, const BfTable& s_bf, BfWaveLds<U, B>& W,
                                                    int lane, bool (&nan_blk)[U / B]) {
    static_assert(B == 4 || B == 8, "candidate masks for blocks of 4 and 8");
    constexpr int NB = U / B;
    constexpr int SLOT = slot_bytes<U>();
    constexpr int NBLK = kTileUnits * NB;
    constexpr int TOP = (int)scale_top<SF_E4M3>();
    const float inv6_lo = inv_six_g * (1.0f - 0x1p-18f), inv6_hi = inv_six_g * (1.0f + 0x1p-18f);
    const float inv4_lo = inv_four_g * (1.0f - 0x1p-18f), inv4_hi = inv_four_g * (1.0f + 0x1p-18f);

#pragma unroll
    for (int i = 0; i < U / 4; ++i)
        reinterpret_cast<float4*>(W.tile + lane * SLOT)[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);

    uint32_t n[NB];
    static_for<NB>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        // largest and second largest magnitude (integer compare of |y| bits)
        uint32_t ab = 0, a2b = 0;
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const uint32_t v = as_u(y[b * B + i]) & 0x7FFFFFFFu;
            a2b = max(a2b, min(ab, v));
            ab = max(ab, v);
        }
        nan_blk[b] = ab >= 0x7F800000u || !(g < __builtin_inff());
        n[b] = 0;
        unsigned long long best = ~0ull, mask = 0ull;
        int base = 0, ovf = 0;
        if (!nan_blk[b] && active) {
            const float a_b = as_f(ab);
            const uint32_t s6 = scale_encode<SF_E4M3>(a_b * inv_six_g), s4 = scale_encode<SF_E4M3>(a_b * inv_four_g);
            const uint32_t c1 = s6 > 0u ? s6 : 1u, c2 = s4 > 0u ? s4 : 1u;
            int wlo = 1, whi = TOP;                  // candidate codes [wlo, whi]
            bool none = false;
            if constexpr (B == 4) {
                if (a_b <= s_bf.t0[1]) {
                    best = pack_candidate(0.0f, 1u);    // every element encodes to 0 at every code: all tie
                    none = true;
                } else {
                    float rc[B];
                    const float2 e1 = s_bf.sr[c1], e2 = s_bf.sr[c2];
                    best = pack_candidate(encode_block<SF_E4M3, B, b * B, false, true>(y, e1.x, e1.y, rc), c1);
                    if (c2 != c1) {
                        const unsigned long long b2 =
                            pack_candidate(encode_block<SF_E4M3, B, b * B, false, true>(y, e2.x, e2.y, rc), c2);
                        best = b2 < best ? b2 : best;
                    }
                }
            } else {
                uint32_t lo, hi;
                best = bf_window<SF_E4M3, B, b * B, true>(y, a_b, c1, c2, s_bf, lo, hi);
                wlo = (int)lo;
                whi = (int)hi - 1;
                none = hi <= lo;
            }
            if (!none) {
                const float tau = as_f((uint32_t)(best >> 32));
                // sqrt with a relative margin far above its error, the
                // rounding of product, difference and square (relative to
                // a), and the square's underflow
                const float delta = __builtin_amdgcn_sqrtf(tau) * (1.0f + 0x1p-16f) + a_b * 0x1p-20f + 0x1p-70f;
                int top;
                if (B == 8 && whi - wlo < 7) {
                    // a short window: masks would cost more than the evaluations they save
                    base = wlo;
                    mask = ~0ull;
                    top = whi;
                } else if (tau < __builtin_inff() && a_b > delta) {
                    int l1, l2, top2;
                    bool sat1, sat2;
                    const unsigned long long p1 =
                        element_pattern(a_b, delta, inv6_lo, inv6_hi, inv4_lo, inv4_hi, l1, top, sat1);
                    const float a2 = as_f(a2b);
                    const unsigned long long p2 =
                        element_pattern(a2, delta, inv6_lo, inv6_hi, inv4_lo, inv4_hi, l2, top2, sat2);
                    // frame from the largest element's lowest admissible
                    // code (blocks of 4) or from the window's start
                    if constexpr (B == 4) {
                        base = l1;
                        mask = p1;
                    } else {
                        base = wlo > l1 ? wlo : l1;
                        mask = place_pattern(p1, l1, sat1, base);
                    }
                    mask &= a2 > delta ? place_pattern(p2, l2, sat2, base) : ~0ull;
                    top = top < whi ? top : whi;
                } else {
                    // The largest element may encode to zero within tau (or
                    // tau is infinite).  From the first code at which every
                    // element encodes to zero (S >= 4 a_b is enough) all
                    // larger codes tie with it, so the candidates are the
                    // codes of the window up to a bound on that code.
                    int up = whi;
                    if (tau < __builtin_inff()) {
                        const int z = e4m3_code_ceil_sub(a_b * inv_four_g * 16.0f * (1.0f + 0x1p-18f));
                        up = z < up ? z : up;
                    }
                    base = wlo;
                    mask = ~0ull;
                    top = up;
                }
                // codes wlo .. min(top, whi) only, and not the two starts
                if (base < wlo) mask &= wlo - base < 64 ? ~0ull << (wlo - base) : 0ull;
                top = top < whi ? top : whi;
                mask = top < base ? 0ull : mask & low_bits(top - base);
                if (base == 0) mask &= ~1ull;
                const int d1 = (int)c1 - base, d2 = (int)c2 - base;
                if (d1 >= 0 && d1 <= 63) mask &= ~(1ull << d1);
                if (d2 >= 0 && d2 <= 63) mask &= ~(1ull << d2);
                ovf = top - (base + 63) > 0 ? top - (base + 63) : 0;
                n[b] = (uint32_t)__popcll(mask) + (uint32_t)ovf;
            }
        }
        W.best[lane * NB + b] = best;
        W.mask[lane * NB + b] = mask;
        W.mbase[lane * NB + b] = (uint8_t)base;
        W.movf[lane * NB + b] = (uint8_t)ovf;
    });

    uint32_t mine = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) mine += n[b];
    const uint32_t incl = wave_inclusive_sum(mine, lane);
    const uint32_t total = (uint32_t)__shfl((int)incl, 63, 64);
    uint32_t run = incl - mine;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        W.start[lane * NB + b] = run;
        run += n[b];
    }
    if (lane == 63) W.start[NBLK] = total;
    wave_sync_lds();

    const uint32_t j0 = (uint32_t)(((uint64_t)total * lane) >> 6);
    const uint32_t j1 = (uint32_t)(((uint64_t)total * (lane + 1)) >> 6);
    if (j0 < j1) {
        uint32_t lo = 0, hi = NBLK;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if (W.start[mid] <= j0) lo = mid; else hi = mid - 1;
        }
        // cursor over the candidates: block k (values yk, mask m from bit
        // base, then ovf codes from base + 64), survivor index range k_end
        uint32_t k = lo;
        float yk[B];
        unsigned long long m;
        int base, ovf_pos;
        auto load_block = [&](uint32_t kk) {
            const float4* src = reinterpret_cast<const float4*>(W.tile + (kk / NB) * SLOT + (kk % NB) * B * 4);
#pragma unroll
            for (int i = 0; i < B / 4; ++i) {
                const float4 v = src[i];
                yk[4 * i] = v.x; yk[4 * i + 1] = v.y; yk[4 * i + 2] = v.z; yk[4 * i + 3] = v.w;
            }
            m = W.mask[kk];
            base = W.mbase[kk];
            ovf_pos = 0;
        };
        load_block(k);
        uint32_t k_end = W.start[k + 1];
        {
            // skip the candidates of block k before j0
            uint32_t t = j0 - W.start[k];
            const uint32_t pc = (uint32_t)__popcll(m);
            if (t >= pc) {
                ovf_pos = (int)(t - pc);
                m = 0ull;
            } else {
#pragma unroll 1
                for (; t > 0; --t) m &= m - 1ull;
            }
        }
        // candidate j: its block, code and values
        auto next = [&](uint32_t j, uint32_t& kk, uint32_t& c, float (&v)[B]) {
            while (j >= k_end) {
                ++k;
                k_end = W.start[k + 1];
                if (j < k_end) load_block(k);
            }
            if (m) {
                c = (uint32_t)(base + __builtin_ctzll(m));
                m &= m - 1ull;
            } else {
                c = (uint32_t)(base + 64 + ovf_pos);
                ++ovf_pos;
            }
            kk = k;
#pragma unroll
            for (int i = 0; i < B; ++i) v[i] = yk[i];
        };
        // two independent candidates per step (the second repeats the first
        // at an odd end)
#pragma unroll 1
        for (uint32_t j = j0; j < j1; j += 2) {
            uint32_t ka, ca, kb, cb;
            float va[B], vb[B];
            next(j, ka, ca, va);
            const bool two = j + 1 < j1;
            if (two) {
                next(j + 1, kb, cb, vb);
            } else {
                kb = ka; cb = ca;
#pragma unroll
                for (int i = 0; i < B; ++i) vb[i] = va[i];
            }
            const float2 ea = s_bf.sr[ca], eb = s_bf.sr[cb];
            float ra[B], rb[B];
            const float sa = encode_block<SF_E4M3, B, 0, false, true>(va, ea.x, ea.y, ra);
            const float sb = encode_block<SF_E4M3, B, 0, false, true>(vb, eb.x, eb.y, rb);
            atomicMin(&W.best[ka], pack_candidate(sa, ca));
            atomicMin(&W.best[kb], pack_candidate(sb, cb));
        }
    }
    wave_sync_lds();
}

// SSE of block BI of a unit at the winning code c of a brute-force search,
// computed as the quantizer computes it (r receives the grid values).
template <int SF, int B, int BI, int U>
__device__ __forceinline__ float bf_block_sse(const float (&y)[U], uint32_t c, const BfTable& s_bf, float (&r)[B],
                                              float& S) {
    constexpr int OFF = BI * B;
    if constexpr (SF == SF_E8M0) {
        S = e8m0_value(c);
        return encode_block<SF, B, OFF, false, true>(y, S, e8m0_inverse(c), r);
    } else {
        S = s_bf.sr[c].x;
        return encode_block_at<B, OFF, false>(y, S, r);
    }
}

// Tile load for the brute-force kernels: contiguous tensors through the
// wave's LDS slots (units of 16 bytes straight into the lanes), strided
// ones unit by unit; rotated when H != 0; idle lanes hold zeros (they
// contribute empty windows).
template <class InT, int U, int H, class P>
__device__ __forceinline__ void bf_load_tile(const P& p, int64_t u0, int nvalid, int lane, char* lds, float (&y)[U]) {
    const InT* x = reinterpret_cast<const InT*>(p.x);
    const int64_t u = u0 + lane;
    const bool active = lane < nvalid;
    if (p.contiguous && !bf_direct_input<InT, U>()) {
        tile_load<InT, U>(x + u0 * U, nvalid, lds, lane, y);
    } else if (active) {
        load_elems<InT, U>(x + unit_offset<U>(u, p.units_per_row, p.ld_x, p.contiguous), y);
    } else {
#pragma unroll
        for (int i = 0; i < U; ++i) y[i] = 0.0f;
    }
    if constexpr (H > 0) fwht_segments<H, U>(y);
    if (!active) {
#pragma unroll
        for (int i = 0; i < U; ++i) y[i] = 0.0f;
    }
}

// Brute-force quantize: bf_search_tile per tile, then every lane encodes its
// blocks at the winning codes and stores the outputs.  CNT: also count the
// written codes into p.counts (register counters per thread).
template <class InT, int B, int H, int SF, bool CNT>
__global__ __launch_bounds__(kThreads) void k_quant_bf(QuantArgs p) {
    constexpr int U = unit_elems<InT, B, H>();
    constexpr int NB = U / B;
    constexpr uint32_t CEND = SF == SF_E8M0 ? 255u : scale_top<SF>() + 1u;
    __shared__ __attribute__((aligned(16))) BfWaveLds<U, B> s_w[kThreads / 64];
    __shared__ BfTable s_bf;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    BfWaveLds<U, B>& W = s_w[wave];

    const float g = workgroup_global_scale(p);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.g_out) *p.g_out = g;
    // start codes only need to be near the abs-max and map-to-4 scales (any
    // start gives the same result), so reciprocals replace the divisions
    const float inv_six_g = 1.0f / (6.0f * g), inv_four_g = 1.0f / (4.0f * g);
    fill_bf_table<SF>(s_bf, g);
    const bool fast = s_bf.fast;

    const int64_t ntiles = (p.units + kTileUnits - 1) / kTileUnits;
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);
    // Units of 32 values run two waves per SIMD, too few to hide a tile
    // load: each lane loads its own unit of the wave's next tile before
    // searching the current one (measured 6-7 % faster; no gain for smaller
    // units, which run more waves).
    constexpr bool PREFETCH = U >= 32;
    const InT* x = reinterpret_cast<const InT*>(p.x);
    float ynext[U];                       // unused without PREFETCH
    auto fetch = [&](int64_t tt) {
        const int64_t uu = tt * kTileUnits + lane;
        if (tt < ntiles && uu < p.units) {
            load_elems<InT, U>(x + unit_offset<U>(uu, p.units_per_row, p.ld_x, p.contiguous), ynext);
        } else {
#pragma unroll
            for (int i = 0; i < U; ++i) ynext[i] = 0.0f;
        }
    };
    uint32_t cnt[16];                     // code occupancy of this thread (CNT)
#pragma unroll
    for (int v = 0; v < 16; ++v) cnt[v] = 0u;
    // units of 4 values fill half a code word: two tiles' words are counted together
    uint32_t pend = 0u;
    bool have_pend = false;
    if constexpr (PREFETCH) fetch((int64_t)blockIdx.x * (kThreads / 64) + wave);
    for (int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave; t < ntiles; t += tstride) {
        const int64_t u0 = t * kTileUnits;
        const int nvalid = (int)min<int64_t>(kTileUnits, p.units - u0);
        const int64_t u = u0 + lane;
        const bool active = lane < nvalid;

        float y[U];
        if constexpr (PREFETCH) {
#pragma unroll
            for (int i = 0; i < U; ++i) y[i] = ynext[i];
            fetch(t + tstride);
            if constexpr (H > 0) fwht_segments<H, U>(y);
            if (!active) {
#pragma unroll
                for (int i = 0; i < U; ++i) y[i] = 0.0f;   // idle lanes contribute empty windows
            }
        } else {
            bf_load_tile<InT, U, H>(p, u0, nvalid, lane, W.tile, y);
        }
        bool nan_blk[NB];
        if constexpr ((B == 4 || B == 8) && SF == SF_E4M3) {
            if (fast) bf_search_tile_mask<U, B>(y, active, g, inv_six_g, inv_four_g, s_bf, W, lane, nan_blk);
            else bf_search_tile<SF, B, U, false>(y, active, g, inv_six_g, inv_four_g, s_bf, W, lane, nan_blk);
        } else {
            if (fast) bf_search_tile<SF, B, U, true>(y, active, g, inv_six_g, inv_four_g, s_bf, W, lane, nan_blk);
            else bf_search_tile<SF, B, U, false>(y, active, g, inv_six_g, inv_four_g, s_bf, W, lane, nan_blk);
        }

        // encode every block at its winning code
        uint32_t cw[code_words(U)];
#pragma unroll
        for (int i = 0; i < code_words(U); ++i) cw[i] = 0;
        const DqSink<U> sink = dq_sink<U>(p, W.tile, lane, u, active);
        uint32_t sc[NB];
        float sse[NB];
        static_for<NB>([&](auto bi) {
            constexpr int b = decltype(bi)::value;
            float r[B];
            float S = 0.0f;
            if (nan_blk[b]) {
                sc[b] = scale_nan<SF>();
                sse[b] = as_f(kQNaN);
#pragma unroll
                for (int i = 0; i < B; ++i) r[i] = 0.0f;
            } else {
                const uint32_t c = (uint32_t)(W.best[lane * NB + b] & 0xFFFFFFFFull) % CEND;
                sc[b] = c;
                sse[b] = bf_block_sse<SF, B, b>(y, c, s_bf, r, S);
            }
            finish_block<B, b * B>(y, r, S, nan_blk[b], cw, sink);
        });
        store_unit_outputs<B, U>(p, u0, nvalid, lane, W.tile, cw, sc, sse, true);
        if constexpr (CNT) {
            if (active) {
                if constexpr (U == 4) {
                    if (have_pend) count_nibbles(pend | (cw[0] << 16), cnt);
                    pend = cw[0];
                    have_pend = !have_pend;
                } else {
                    static_assert(U % 8 == 0, "units of 4 or of whole code words");
#pragma unroll
                    for (int i = 0; i < code_words(U); ++i) count_nibbles(cw[i], cnt);
                }
            }
        }
    }
    if constexpr (CNT) {
        if (have_pend) {
            count_nibbles(pend, cnt);
            cnt[0] -= 4u;                     // the empty high half of the word
        }
        flush_code_counts(cnt, p.counts);
    }
}

// Per-tensor scale search with the brute-force block search inside: for each
// candidate g_j (one table fill per candidate, shared by the workgroup) every
// tile runs bf_search_tile and scores its blocks at their winning codes; the
// per-tile fp64 sums go to the same partials as k_gsearch.
template <class InT, int B, int H>
__global__ __launch_bounds__(kThreads) void k_gsearch_bf(GSearchArgs p) {
    constexpr int U = unit_elems<InT, B, H>();
    constexpr int NB = U / B;
    constexpr uint32_t CEND = scale_top<SF_E4M3>() + 1u;
    __shared__ __attribute__((aligned(16))) BfWaveLds<U, B> s_w[kThreads / 64];
    __shared__ BfTable s_bf;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    BfWaveLds<U, B>& W = s_w[wave];
    const float g0 = workgroup_amax_scale(p.amax_partials, p.n_partials);

    const int64_t ntiles = (p.units + kTileUnits - 1) / kTileUnits;
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);
#pragma unroll 1
    for (int j = 0; j < kSearchCandidates; ++j) {
        const float g = g0 * search_factor(j);
        const float inv_six_g = 1.0f / (6.0f * g), inv_four_g = 1.0f / (4.0f * g);
        fill_bf_table<SF_E4M3>(s_bf, g);
        const bool fast = s_bf.fast;
        for (int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave; t < ntiles; t += tstride) {
            const int64_t u0 = t * kTileUnits;
            const int nvalid = (int)min<int64_t>(kTileUnits, p.units - u0);
            const bool active = lane < nvalid;
            float y[U];
            bf_load_tile<InT, U, H>(p, u0, nvalid, lane, W.tile, y);
            bool nan_blk[NB];
            if constexpr (B == 4 || B == 8) {
                if (fast) bf_search_tile_mask<U, B>(y, active, g, inv_six_g, inv_four_g, s_bf, W, lane, nan_blk);
                else bf_search_tile<SF_E4M3, B, U, false>(y, active, g, inv_six_g, inv_four_g, s_bf, W, lane, nan_blk);
            } else {
                if (fast) bf_search_tile<SF_E4M3, B, U, true>(y, active, g, inv_six_g, inv_four_g, s_bf, W, lane, nan_blk);
                else bf_search_tile<SF_E4M3, B, U, false>(y, active, g, inv_six_g, inv_four_g, s_bf, W, lane, nan_blk);
            }
            double e[NB];
            static_for<NB>([&](auto bi) {
                constexpr int b = decltype(bi)::value;
                float r[B], S;
                const uint32_t c = (uint32_t)(W.best[lane * NB + b] & 0xFFFFFFFFull) % CEND;
                e[b] = nan_blk[b] ? (double)as_f(kQNaN) : (double)bf_block_sse<SF_E4M3, B, b>(y, c, s_bf, r, S);
            });
            double s = active ? tree_sum<NB>(e) : 0.0;      // lanes past the tensor are padding
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) s = s + __shfl_xor(s, o, 64);
            if (lane == 0) p.partials[j * p.ntiles + t] = s;
            wave_sync_lds();                                  // W is reused by the next tile
        }
        __syncthreads();                                      // every wave is done with this table
    }
}

// Scale of a stored block code (runtime format) times g; usable is false
// for the NaN code and for scales that are NaN, infinite or negative.
__device__ __forceinline__ float stored_scale(int fmt, uint32_t code, float g, bool& usable) {
    if (fmt == SF_E8M0) {
        usable = code != kE8M0NaN;
        return e8m0_value(code);
    }
    if (fmt == SF_E4M3) {
        const uint32_t c7 = code & 0x7Fu;
        const float S = e4m3_value(c7) * g;
        usable = c7 != kE4M3NaN && scale_usable(S);
        return S;
    }
    const float S = ue5m3_value(code) * g;
    usable = code != kUE5M3NaN && scale_usable(S);
    return S;
}

}  // namespace fp4q_dev
