// fp4q_stream.hpp -- the streaming kernels of the path (scale choice by
// abs-max, prevent-zero, 4-over-6 or given codes; the per-tensor abs-max
// pre-pass) laid out for coalesced HBM traffic on gfx950.
//
// Work mapping: lane l of a wave owns one 16-byte chunk of the input (4 fp32
// or 8 bf16 / fp16 values), and consecutive lanes own consecutive chunks, so
// every load and every store of a wave covers whole contiguous cache lines.
// A block of B values (or a rotation segment of H values) wider than one
// chunk spans B / E neighbouring lanes, aligned to that lane count; its
// abs-max, its squared-error tree and the cross-chunk stages of the
// Walsh-Hadamard transform are exchanged between those lanes with DPP row
// moves.  The exchange reproduces the per-block arithmetic exactly: the
// abs-max is an integer max, the squared-error tree pairs neighbouring
// lanes first (the balanced binary tree in index order), and each
// butterfly keeps its operand order.  Each wave handles R chunks per lane
// per trip (R * 1 KiB of input), all loaded before any is processed.
#pragma once

#include "fp4q_kernels.hpp"

namespace fp4q_dev {

// ---------------------------------------------------------------------------
// Lane exchange inside aligned groups of 2, 4 or 8 lanes: the value of lane
// l ^ M.  DPP row moves (quad_perm, row_half_mirror): no LDS traffic.
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
    static_assert(M == 1 || M == 2 || M == 4, "partners within groups of 8 lanes");
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    } else {
        // row_half_mirror gives lane l ^ 7 (within 8); quad_perm [3,2,1,0] then ^ 3
        const int t = __builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, false);
    }
}

template <int M>
__device__ __forceinline__ float lane_xor_f32(float v) { return as_f(lane_xor_u32<M>(as_u(v))); }

// Integer max over an aligned group of L lanes (every lane gets it).
template <int L>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    if constexpr (L >= 2) v = max(v, lane_xor_u32<1>(v));
    if constexpr (L >= 4) v = max(v, lane_xor_u32<2>(v));
    if constexpr (L >= 8) v = max(v, lane_xor_u32<4>(v));
    return v;
}

// Balanced-tree sum of the lanes' partial sums over an aligned group of L
// lanes: neighbours first, then pairs of pairs (every lane gets the total;
// each addition is commutative, so both partners hold the same bits).
template <int L>
__device__ __forceinline__ float group_tree_sum(float v) {
    if constexpr (L >= 2) v = v + lane_xor_f32<1>(v);
    if constexpr (L >= 4) v = v + lane_xor_f32<2>(v);
    if constexpr (L >= 8) v = v + lane_xor_f32<4>(v);
    return v;
}

// Block-wise normalised Walsh-Hadamard transform of segments of H values
// spread over H / E lanes (MR-GPTQ page, sections 2.1-2.3): the stages with
// stride h < E run inside the lane, the stages with h >= E pair lane l with
// lane l ^ (h / E).  The lower element of a pair becomes fl(a + b), the
// upper fl(a - b), a the lower and b the upper value, as in the in-lane
// stages.  Across lanes both are one addition: the lower lane adds its
// partner's b to its a, the upper lane adds its partner's a to -b (IEEE
// defines a - b as a + (-b), signed zeros included).  With SCALE every value
// is then multiplied once by fl(1 / sqrt(H)); without it the caller applies
// that factor (the abs-max pre-pass scales only its maximum, which gives
// the same bits because rounding is monotone).  NaN signs are left as the
// arithmetic makes them: the quantizer canonicalises the elements of a NaN
// block, the only place where the sign of a NaN reaches an output.
template <int H, int E, bool SCALE = true>
__device__ __forceinline__ void fwht_chunk(float (&y)[E], int lane) {
    static_assert(H % E == 0 && H / E <= 8, "segments of 1 to 8 chunks");
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
            if ((i & h) == 0) {
                const float a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
        }
    }
    static_for<3>([&](auto si) {
        constexpr int m = 1 << decltype(si)::value;     // lane distance of this stage
        if constexpr (m < H / E) {
            const uint32_t flip = (lane & m) ? 0x80000000u : 0u;
#pragma unroll
            for (int i = 0; i < E; ++i) y[i] = lane_xor_f32<m>(y[i]) + as_f(as_u(y[i]) ^ flip);
        }
    });
    if constexpr (SCALE) {
        constexpr float c = hadamard_coef<H>();
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] *= c;
    }
}

// ---------------------------------------------------------------------------
// Scale table of one call for the formats whose scales are not powers of
// two (E4M3, UE5M3), filled once per workgroup: entry c holds S_c =
// fl(dec(c) g) and R_c = fl(1 / S_c) when S_c is in the division-free range
// (else NaN: that scale takes the IEEE division per element).  With it a
// block's encode needs no division.
// ---------------------------------------------------------------------------
struct ScaleTab {
    float2 sr[256];
};

template <int SF>
__device__ __forceinline__ void fill_scale_tab(ScaleTab& t, float g) {
    for (uint32_t c = threadIdx.x; c < 256u; c += kThreads) {
        float S = __builtin_nanf(""), R = __builtin_nanf("");
        if (c <= scale_top<SF>()) {
            S = scale_value<SF>(c) * g;
            if (fast_quotient_range(S)) R = 1.0f / S;
        }
        t.sr[c] = make_float2(S, R);
    }
    __syncthreads();
}

// fl(a / d) for the block scale code, a = the block abs-max, d = fl(M g)
// with Rd = fl(1 / d) computed once per call (valid when d lies in
// [2^-60, 2^60]): the same reciprocal refinement as the element quotient
// (checked exhaustively around every grid point and midpoint of the 3-bit
// mantissa scale formats).  Quotients below 2^-20 or above 2^20 round to the
// smallest or the saturated code whatever their last bits, so the first
// product stands for them (and keeps the residual clear of underflow); the
// refinement is computed either way and the choice is a select.
__device__ __forceinline__ float block_quotient(float a, float d, float Rd) {
    const float q0 = a * Rd;
    const float rr = __builtin_fmaf(-q0, d, a);
    const float q1 = __builtin_fmaf(rr, Rd, q0);
    return (q0 >= 0x1p-20f && q0 <= 0x1p20f) ? q1 : q0;
}

// Per-call constants of the scale choice.
struct ScaleCtx {
    float g, six_g, four_g, r6, r4;
    bool div_fast;                // six_g and four_g in [2^-60, 2^60]
    const ScaleTab* tab;          // E4M3 / UE5M3
};

template <int SF>
__device__ __forceinline__ uint32_t scale_code_of(float a_b, float d, float Rd, bool div_fast) {
    return scale_encode<SF>(div_fast ? block_quotient(a_b, d, Rd) : a_b / d);
}

// ---------------------------------------------------------------------------
// Element encode with the gfx950 FP4 pair converts.  The signed quotient
// fl(y / S) goes through v_cvt_scalef32_pk_fp4_f32 (scale 1), which rounds
// half-to-even onto the E2M1 grid with saturation at 6 and writes the two
// nibbles (sign and magnitude) straight into their byte of the chunk's code
// word; v_cvt_scalef32_pk_f32_fp4 returns the signed grid values, whose
// product with S is the dequantized value.  Both converts agree bit for bit
// with the arithmetic rounding of e2m1_round on every non-NaN fp32 input.
// ---------------------------------------------------------------------------

// Quotient modes: E8M0 (S a power of two, fl(y R) exact), FAST (reciprocal
// refinement with R = fl(1/S)), SLOW (IEEE division, 0 for S = 0).
enum : int { QM_E8M0 = 0, QM_FAST = 1, QM_SLOW = 2 };

// Signed fl(y / S) carrying y's sign bit (also on zero quotients); with
// NAN_GUARD a NaN y gives a zero of y's sign (magnitude code 0).
template <int QM, bool NAN_GUARD>
__device__ __forceinline__ float signed_quotient(float y, float S, float R) {
    float q;
    if constexpr (QM == QM_E8M0) {
        q = y * R;
    } else {
        const float a = fabsf(y);
        float qa;
        if constexpr (QM == QM_FAST) {
            const float q0 = a * R;
            const float rr = __builtin_fmaf(-q0, S, a);
            qa = __builtin_fmaf(rr, R, q0);
        } else {
            qa = (S > 0.0f) ? a / S : 0.0f;
        }
        q = with_sign_of(qa, y);
    }
    if constexpr (NAN_GUARD) q = (y == y) ? q : with_sign_of(0.0f, y);
    return q;
}

// Encode y[OFF, OFF + BL) at scale S: the nibbles go to bytes OFF/2 ... of
// *cw (which must hold zeros there), p receives the signed dequantized
// values fl(grid * S); returns the tree SSE of these BL values.
template <int QM, int BL, int OFF, bool NAN_GUARD, int E>
__device__ __forceinline__ float encode_hw(const float (&y)[E], float S, float R, uint32_t& cw, float (&p)[E]) {
    static_assert(BL % 2 == 0 && OFF % 2 == 0, "whole pairs");
    float q[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) q[i] = signed_quotient<QM, NAN_GUARD>(y[OFF + i], S, R);
    static_for<BL / 2>([&](auto ki) {
        constexpr int k = decltype(ki)::value;
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, q[2 * k], q[2 * k + 1], 1.0f, OFF / 2 + k);
    });
    float e[BL];
    static_for<BL / 2>([&](auto ki) {
        constexpr int k = decltype(ki)::value;
        const auto g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, OFF / 2 + k);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int i = 2 * k + h;
            p[OFF + i] = g2[h] * S;
            const float d = y[OFF + i] - p[OFF + i];
            e[i] = d * d;
        }
    });
    return tree_sum<BL>(e);
}

// encode_hw at a table scale (S, R): division-free when R is a number (or,
// for finite elements, when S is 0: the quotient 0), else the IEEE division.
template <int BL, int OFF, bool NAN_GUARD, int E>
__device__ __forceinline__ float encode_hw_tab(const float (&y)[E], float S, float R, uint32_t& cw, float (&p)[E]) {
    const bool zero = !NAN_GUARD && S == 0.0f;
    if (R == R || zero) return encode_hw<QM_FAST, BL, OFF, NAN_GUARD>(y, S, zero ? 0.0f : R, cw, p);
    return encode_hw<QM_SLOW, BL, OFF, NAN_GUARD>(y, S, 0.0f, cw, p);
}

// The nibbles (sign only) and values (NaN with the sign) of a NaN block part.
// ROT: the values come from the rotation, whose NaNs count as the positive
// quiet NaN (IEEE 754 leaves the sign of an arithmetic NaN open, gfx950's
// subtraction flips it where x86's keeps it, and here it reaches the code).
template <int BL, int OFF, bool ROT, int E>
__device__ __forceinline__ void nan_block_hw(const float (&y)[E], uint32_t& cw, float (&p)[E]) {
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const float v = ROT ? rotated_nan_canonical(y[OFF + i]) : y[OFF + i];
        cw |= (as_u(v) >> 31) << (4 * (OFF + i) + 3);
        p[OFF + i] = canonical_nan_like(v);
    }
}

// ---------------------------------------------------------------------------
// Scale choice and encoding of the blocks one chunk touches.  BL = values of
// a block inside this lane (min(B, E)), LB = lanes a block spans; the chunk
// holds E / BL (partial) blocks.  Outputs: the chunk's code word (E
// nibbles), the dequantized values p, each block's scale code and SSE
// (whole block, every lane of it).  ROT: y comes from the rotation, whose
// NaNs count as the positive quiet NaN.
// ---------------------------------------------------------------------------
template <int SF, int ST, int B, int E, bool ROT>
__device__ __forceinline__ void quant_chunk(const float (&y)[E], const ScaleCtx& cx, int prevent_zero,
                                            const uint32_t (&given)[(E + B - 1) / B], uint32_t& cw, float (&p)[E],
                                            uint32_t (&sc)[(E + B - 1) / B], float (&sse)[(E + B - 1) / B]) {
    constexpr int BL = B < E ? B : E;
    constexpr int LB = B / BL;
    constexpr int NB = E / BL;
    cw = 0;
    static_for<NB>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        constexpr int OFF = b * BL;
        float e = 0.0f;
        uint32_t code = 0;
        bool nanb;
        if constexpr (ST == ST_GIVEN) {
            // a NaN element encodes as a zero of its sign here, so a rotated
            // NaN takes its canonical (positive) sign first
            float yc[E];
#pragma unroll
            for (int i = 0; i < E; ++i) yc[i] = ROT ? rotated_nan_canonical(y[i]) : y[i];
            if constexpr (SF == SF_E8M0) {
                code = given[b] & 0xFFu;
                nanb = code == kE8M0NaN;
                if (!nanb) e = encode_hw<QM_E8M0, BL, OFF, true>(yc, e8m0_value(code), e8m0_inverse(code), cw, p);
            } else {
                code = given[b] & scale_code_mask<SF>();
                const float2 sr = cx.tab->sr[code];
                nanb = code == scale_nan<SF>() || !scale_usable(sr.x);
                if (!nanb) e = encode_hw_tab<BL, OFF, true>(yc, sr.x, sr.y, cw, p);
            }
            // a caller-given scale needs no cross-lane choice; the SSE still
            // sums over the whole block
            e = group_tree_sum<LB>(e);
        } else {
            uint32_t ab = 0;
#pragma unroll
            for (int i = 0; i < BL; ++i) ab = max(ab, as_u(y[OFF + i]) & 0x7FFFFFFFu);
            ab = group_max_u32<LB>(ab);
            const float a_b = as_f(ab);
            nanb = ab >= 0x7F800000u || !(cx.g < __builtin_inff());   // also catches NaN g
            if (!nanb) {
                if constexpr (SF == SF_E8M0) {
                    code = e8m0_absmax_code(ab);
                    e = group_tree_sum<LB>(
                        encode_hw<QM_E8M0, BL, OFF, false>(y, e8m0_value(code), e8m0_inverse(code), cw, p));
                } else {
                    const uint32_t s6 = scale_code_of<SF>(a_b, cx.six_g, cx.r6, cx.div_fast);
                    if constexpr (ST == ST_ABSMAX) {
                        code = (prevent_zero && s6 == 0u) ? 1u : s6;
                        const float2 sr = cx.tab->sr[code];
                        e = group_tree_sum<LB>(encode_hw_tab<BL, OFF, false>(y, sr.x, sr.y, cw, p));
                    } else {
                        static_assert(ST == ST_FOUR_OVER_SIX, "brute force has its own kernel");
                        const uint32_t s4 = scale_code_of<SF>(a_b, cx.four_g, cx.r4, cx.div_fast);
                        const float2 sr6 = cx.tab->sr[s6], sr4 = cx.tab->sr[s4];
                        uint32_t cw6 = 0, cw4 = 0;
                        float p4[E];
                        const float e6 = group_tree_sum<LB>(encode_hw_tab<BL, OFF, false>(y, sr6.x, sr6.y, cw6, p));
                        const float e4 = group_tree_sum<LB>(encode_hw_tab<BL, OFF, false>(y, sr4.x, sr4.y, cw4, p4));
                        const bool take4 = e4 < e6;   // equal error keeps the smaller code s6
                        code = take4 ? s4 : s6;
                        e = take4 ? e4 : e6;
                        cw |= take4 ? cw4 : cw6;
#pragma unroll
                        for (int i = 0; i < BL; ++i) p[OFF + i] = take4 ? p4[OFF + i] : p[OFF + i];
                    }
                }
            } else {
                code = scale_nan<SF>();
            }
        }
        if (nanb) {
            nan_block_hw<BL, OFF, ROT>(y, cw, p);
            e = as_f(kQNaN);
        }
        sc[b] = code;
        sse[b] = e;
    });
}

// The choice and encoding of quant_chunk for abs-max, prevent-zero and
// 4-over-6 without a branch, for calls whose every candidate scale has a
// division-free quotient (E8M0, or E4M3 / UE5M3 with g in the range that
// keeps every table scale there: the usual case): the scale-code quotient
// by its reciprocal refinement, the element quotient by the table's
// reciprocal (0 for the zero scale; such a block holds finite values only),
// saturation by a minimum.  A NaN block is encoded like any other here;
// nanb reports it and fix_nan_blocks rewrites its outputs afterwards, so
// the work of every chunk of a trip is one straight run of instructions
// that the compiler can interleave.  Same results as quant_chunk.
template <int SF, int ST, int B, int E>
__device__ __forceinline__ void quant_chunk_fast(const float (&y)[E], const ScaleCtx& cx, int prevent_zero,
                                                 uint32_t& cw, float (&p)[E], uint32_t (&sc)[(E + B - 1) / B],
                                                 float (&sse)[(E + B - 1) / B], bool (&nanb)[(E + B - 1) / B]) {
    static_assert(ST == ST_ABSMAX || ST == ST_FOUR_OVER_SIX, "scale choice from the block abs-max");
    constexpr int BL = B < E ? B : E;
    constexpr int LB = B / BL;
    constexpr int NB = E / BL;
    cw = 0;
    static_for<NB>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        constexpr int OFF = b * BL;
        uint32_t ab = 0;
#pragma unroll
        for (int i = 0; i < BL; ++i) ab = max(ab, as_u(y[OFF + i]) & 0x7FFFFFFFu);
        ab = group_max_u32<LB>(ab);
        const float a_b = as_f(ab);
        nanb[b] = ab >= 0x7F800000u || !(cx.g < __builtin_inff());
        uint32_t code;
        float e;
        if constexpr (SF == SF_E8M0) {
            code = e8m0_absmax_code(ab);
            e = group_tree_sum<LB>(
                encode_hw<QM_E8M0, BL, OFF, false>(y, e8m0_value(code), e8m0_inverse(code), cw, p));
        } else {
            const uint32_t s6 = scale_encode<SF>(block_quotient(a_b, cx.six_g, cx.r6));
            if constexpr (ST == ST_ABSMAX) {
                code = (prevent_zero && s6 == 0u) ? 1u : s6;
                const float2 sr = cx.tab->sr[code];
                e = group_tree_sum<LB>(
                    encode_hw<QM_FAST, BL, OFF, false>(y, sr.x, sr.x == 0.0f ? 0.0f : sr.y, cw, p));
            } else {
                const uint32_t s4 = scale_encode<SF>(block_quotient(a_b, cx.four_g, cx.r4));
                const float2 sr6 = cx.tab->sr[s6], sr4 = cx.tab->sr[s4];
                uint32_t cw6 = 0, cw4 = 0;
                float p4[E];
                const float e6 = group_tree_sum<LB>(
                    encode_hw<QM_FAST, BL, OFF, false>(y, sr6.x, sr6.x == 0.0f ? 0.0f : sr6.y, cw6, p));
                const float e4 = group_tree_sum<LB>(
                    encode_hw<QM_FAST, BL, OFF, false>(y, sr4.x, sr4.x == 0.0f ? 0.0f : sr4.y, cw4, p4));
                const bool take4 = e4 < e6;   // equal error keeps the smaller code s6
                code = take4 ? s4 : s6;
                e = take4 ? e4 : e6;
                cw |= take4 ? cw4 : cw6;
#pragma unroll
                for (int i = 0; i < BL; ++i) p[OFF + i] = take4 ? p4[OFF + i] : p[OFF + i];
            }
        }
        sc[b] = code;
        sse[b] = e;
    });
}

// The outputs of the NaN blocks of a chunk that quant_chunk_fast encoded as
// numbers: the nibbles carry the sign only, the values are NaN with the
// sign (the rotation's NaNs count as the positive quiet NaN), the error is
// NaN and the scale the NaN code.
template <int SF, int B, int E, bool ROT>
__device__ __forceinline__ void fix_nan_blocks(const float (&y)[E], const bool (&nanb)[(E + B - 1) / B],
                                               uint32_t& cw, float (&p)[E], uint32_t (&sc)[(E + B - 1) / B],
                                               float (&sse)[(E + B - 1) / B]) {
    constexpr int BL = B < E ? B : E;
    constexpr int NB = E / BL;
    static_for<NB>([&](auto bi) {
        constexpr int b = decltype(bi)::value;
        constexpr int OFF = b * BL;
        constexpr uint32_t m = 4 * BL >= 32 ? 0xFFFFFFFFu : ((1u << (4 * BL)) - 1u) << (4 * OFF);
        if (nanb[b]) {
            cw &= ~m;
            nan_block_hw<BL, OFF, ROT>(y, cw, p);
            sse[b] = as_f(kQNaN);
            sc[b] = scale_nan<SF>();
        }
    });
}

// Chunk index -> element offset in a [rows, ld] tensor with cpr chunks of E
// values per row.
template <int E>
__device__ __forceinline__ int64_t chunk_offset(int64_t j, int64_t cpr, int64_t ld, bool contiguous) {
    if (contiguous) return j * E;
    const int64_t row = j / cpr;
    return row * ld + (j - row * cpr) * E;
}

// Load one 16-byte chunk as raw words (zeros past the end).
__device__ __forceinline__ uint4 load_chunk(const void* base, int64_t elem_off, int es, bool valid) {
    if (!valid) return make_uint4(0u, 0u, 0u, 0u);
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + elem_off * es);
}

template <class InT, int E>
__device__ __forceinline__ void widen_chunk(const uint4& w, float (&y)[E]) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
    if constexpr (ElemSize<InT>::value == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = as_f(v[i]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (__is_same(InT, bf16_t)) {
                y[2 * k] = as_f(v[k] << 16);
                y[2 * k + 1] = as_f(v[k] & 0xFFFF0000u);
            } else {
                y[2 * k] = f16_bits_to_f32(v[k] & 0xFFFFu);
                y[2 * k + 1] = f16_bits_to_f32(v[k] >> 16);
            }
        }
    }
}

// Store a chunk's E dequantized values as dtype dt at element offset off,
// streaming (each wave writes whole contiguous lines: 64 lanes x 8 or 16
// bytes per store).
template <int E>
__device__ __forceinline__ void store_dq_chunk(void* base, int dt, int64_t off, const float (&v)[E]) {
    if (dt == DT_F32) {
        uint4* q = reinterpret_cast<uint4*>(reinterpret_cast<float*>(base) + off);
#pragma unroll
        for (int i = 0; i < E / 4; ++i)
            store_stream(q + i, make_uint4(as_u(v[4 * i]), as_u(v[4 * i + 1]), as_u(v[4 * i + 2]), as_u(v[4 * i + 3])));
    } else {
        uint32_t w[E / 2];
#pragma unroll
        for (int i = 0; i < E / 2; ++i)
            w[i] = dt == DT_BF16 ? pack_bf16x2(v[2 * i], v[2 * i + 1]) : pack_f16x2(v[2 * i], v[2 * i + 1]);
        uint16_t* q = reinterpret_cast<uint16_t*>(base) + off;
        if constexpr (E == 8) store_stream(reinterpret_cast<uint4*>(q), make_uint4(w[0], w[1], w[2], w[3]));
        else store_stream(reinterpret_cast<uint2*>(q), make_uint2(w[0], w[1]));
    }
}

// E nibbles (E / 2 bytes) of packed codes at dense element index e0.
template <int E>
__device__ __forceinline__ uint32_t load_code_word(const uint8_t* codes, int64_t e0) {
    if constexpr (E == 4) return *reinterpret_cast<const uint16_t*>(codes + e0 / 2);
    else return *reinterpret_cast<const uint32_t*>(codes + e0 / 2);
}

template <int E>
__device__ __forceinline__ void store_code_word(uint8_t* codes, int64_t e0, uint32_t cw) {
    if constexpr (E == 4) *reinterpret_cast<uint16_t*>(codes + e0 / 2) = (uint16_t)cw;
    else *reinterpret_cast<uint32_t*>(codes + e0 / 2) = cw;
}

// Chunks per lane per trip: enough 16-byte loads in flight per wave.
template <class InT>
constexpr int stream_rounds() { return 2; }

// Streaming quantize: scale selection by abs-max / prevent-zero / 4-over-6 /
// given codes, encode, pack, dequantize, block error.
//
// The next trip's loads are issued before the current trip is processed.
// Loads never sit behind a branch (past the end they re-read the last chunk,
// whose values are discarded), and the trips whose chunks are all inside the
// tensor store without a per-lane test, so the compiler can count the memory
// operations in flight and wait only for the ones a value needs.  Every lane
// of a block stores the block's scale and error (the same value to the same
// address), which keeps those stores unconditional too.
//
// With p.counts the written codes are also counted: 16 counters per thread
// in LDS (code n of thread t at n * kThreads + t, so a wave's increments
// fall on distinct banks), one LDS add per code, summed per workgroup at
// the end.  The 16 KiB this takes leave the occupancy unchanged (eight
// workgroups per compute unit still fit).
template <class InT, int B, int H, int SF, int ST, int R>
__global__ __launch_bounds__(kThreads) void k_qstream(QuantArgs p) {
    constexpr int ES = ElemSize<InT>::value;
    constexpr int E = 16 / ES;                    // values per chunk
    constexpr int BL = B < E ? B : E;
    constexpr int NB = E / BL;                    // (partial) blocks per chunk
    static_assert(ST != ST_BRUTE_FORCE, "brute force runs in k_quant_bf");

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float g = workgroup_global_scale(p);
    if (blockIdx.x == 0 && threadIdx.x == 0 && p.g_out) *p.g_out = g;
    ScaleCtx cx;
    cx.g = g;
    cx.six_g = 6.0f * g;
    cx.four_g = 4.0f * g;
    cx.div_fast = cx.six_g >= 0x1p-60f && cx.six_g <= 0x1p60f && cx.four_g >= 0x1p-60f && cx.four_g <= 0x1p60f;
    cx.r6 = cx.div_fast ? 1.0f / cx.six_g : 0.0f;
    cx.r4 = cx.div_fast ? 1.0f / cx.four_g : 0.0f;
    cx.tab = nullptr;
    if constexpr (SF != SF_E8M0) {
        __shared__ ScaleTab s_tab;
        fill_scale_tab<SF>(s_tab, g);
        cx.tab = &s_tab;
    }

    __shared__ uint32_t s_bins[16 * kThreads];
    const bool counting = p.counts != nullptr;
    uint32_t* bins = s_bins + threadIdx.x;        // only this thread touches them until the end
    if (counting) {
#pragma unroll
        for (int v = 0; v < 16; ++v) bins[v * kThreads] = 0u;
    }

    const int64_t nchunks = p.units;              // rows * cols / E (>= 1)
    const int64_t cpr = p.units_per_row;          // chunks per row
    const bool in_contig = p.ld_x == p.cols;
    const bool dq_contig = p.ld_dq == p.cols;
    const int64_t per_trip = (int64_t)kTileUnits * R;
    const int64_t ntrips = (nchunks + per_trip - 1) / per_trip;
    const int64_t nfull = nchunks / per_trip;     // trips with every chunk inside
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);

    struct Trip {
        uint4 raw[R];
        uint32_t given[R][NB];
    };
    auto fetch = [&](int64_t tt, Trip& d) {
        const int64_t jb = tt * per_trip + lane;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            int64_t j = jb + k * kTileUnits;
            j = j < nchunks ? j : nchunks - 1;
            d.raw[k] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.x) +
                                                        chunk_offset<E>(j, cpr, p.ld_x, in_contig) * ES);
            if constexpr (ST == ST_GIVEN) {
#pragma unroll
                for (int b = 0; b < NB; ++b) d.given[k][b] = p.scales[j * E / B + b];
            }
        }
    };
    // the outputs of chunk j
    auto store_chunk = [&](int64_t j, uint32_t cw, const float (&dq)[E], const uint32_t (&sc)[NB],
                           const float (&sse)[NB]) {
        const int64_t e0 = j * E;                     // dense element index of the chunk
        if (p.codes) store_code_word<E>(p.codes, e0, cw);
        if (counting) {
#pragma unroll
            for (int i = 0; i < E; ++i) atomicAdd(&bins[((cw >> (4 * i)) & 15u) * kThreads], 1u);
        }
        if (p.dq) store_dq_chunk<E>(p.dq, p.dq_dt, chunk_offset<E>(j, cpr, p.ld_dq, dq_contig), dq);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int64_t bi = e0 / B + b;
            if constexpr (ST != ST_GIVEN) p.scales[bi] = (uint8_t)sc[b];
            if (p.sse) p.sse[bi] = sse[b];
            if (p.mse) {
                const float m = sse[b] * (1.0f / (float)B);   // exact: B is a power of two
                p.mse[bi] = (m == m) ? m : as_f(kQNaN);
            }
        }
    };
    auto process = [&](const Trip& d, int64_t tt, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        const int64_t j0 = tt * per_trip + lane;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = j0 + k * kTileUnits;
            float y[E];
            widen_chunk<InT, E>(d.raw[k], y);
            if constexpr (H > 0) fwht_chunk<H, E>(y, lane);
            uint32_t given[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) given[b] = ST == ST_GIVEN ? d.given[k][b] : 0u;

            uint32_t cw, sc[NB];
            float dq[E], sse[NB];
            quant_chunk<SF, ST, B, E, (H > 0)>(y, cx, p.prevent_zero, given, cw, dq, sc, sse);
            if (!FULL && j >= nchunks) continue;
            store_chunk(j, cw, dq, sc, sse);
        }
    };
    // every chunk of the trip through quant_chunk_fast, then the NaN blocks
    // (rare: one wave-level test; their values are widened and rotated
    // again from the loaded words), then the stores
    auto process_fast = [&](const Trip& d, int64_t tt, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        const int64_t j0 = tt * per_trip + lane;
        float dq[R][E], sse[R][NB];
        uint32_t cw[R], sc[R][NB];
        bool nb[R][NB];
        bool any_nan = false;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            float y[E];
            widen_chunk<InT, E>(d.raw[k], y);
            if constexpr (H > 0) fwht_chunk<H, E>(y, lane);
            if constexpr (ST == ST_ABSMAX || ST == ST_FOUR_OVER_SIX)
                quant_chunk_fast<SF, ST, B, E>(y, cx, p.prevent_zero, cw[k], dq[k], sc[k], sse[k], nb[k]);
#pragma unroll
            for (int b = 0; b < NB; ++b) any_nan |= nb[k][b];
        }
        if (any_nan) {
#pragma unroll
            for (int k = 0; k < R; ++k) {
                float y[E];
                widen_chunk<InT, E>(d.raw[k], y);
                if constexpr (H > 0) fwht_chunk<H, E>(y, lane);
                fix_nan_blocks<SF, B, E, (H > 0)>(y, nb[k], cw[k], dq[k], sc[k], sse[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = j0 + k * kTileUnits;
            if (!FULL && j >= nchunks) continue;
            store_chunk(j, cw[k], dq[k], sc[k], sse[k]);
        }
    };
    auto run = [&](auto& proc) {
        int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave;
        if (t < ntrips) {
            Trip cur;
            fetch(t, cur);
            for (; t < nfull; t += tstride) {
                Trip nxt;
                fetch(t + tstride, nxt);
                proc(cur, t, IC<1>{});
                cur = nxt;
            }
            if (t < ntrips) proc(cur, t, IC<0>{});    // the last, partial trip
        }
    };
    // the branch-free path serves abs-max, prevent-zero and 4-over-6 when
    // every candidate scale has a division-free quotient (16-bit inputs with
    // the 32-point rotation keep the chunk-by-chunk path: there the larger
    // register footprint of the interleaved trip measured 5-8 % slower)
    if constexpr ((ST == ST_ABSMAX || ST == ST_FOUR_OVER_SIX) && !(ES == 2 && H == 32)) {
        bool fast = true;
        if constexpr (SF != SF_E8M0)
            fast = cx.div_fast && fast_quotient_range(scale_value<SF>(1u) * g) &&
                   fast_quotient_range(scale_value<SF>(scale_top<SF>()) * g);
        if (fast) run(process_fast);
        else run(process);
    } else {
        run(process);
    }
    if (counting) {
        // thread t gathers code t & 15 from the 16 threads of its group of 16
        __syncthreads();
        const int code = threadIdx.x & 15, seg = threadIdx.x >> 4;
        uint32_t part = 0;
#pragma unroll
        for (int l = 0; l < 16; ++l) part += s_bins[code * kThreads + seg * 16 + l];
        add_code_counts(part, p.counts);
    }
}

// Partial per-tensor abs-max (of the rotated values when H != 0) for
// hierarchical scaling: one result per workgroup in p.partials.
template <class InT, int H, int R>
__global__ __launch_bounds__(kThreads) void k_amax_stream(AmaxArgs p) {
    constexpr int ES = ElemSize<InT>::value;
    constexpr int E = 16 / ES;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nchunks = p.units;
    const bool contig = p.contiguous != 0;
    const int64_t per_trip = (int64_t)kTileUnits * R;
    const int64_t ntrips = (nchunks + per_trip - 1) / per_trip;
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);
    auto fetch = [&](int64_t tt, uint4 (&dst)[R]) {
        const int64_t jb = tt * per_trip + lane;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = jb + k * kTileUnits;
            dst[k] = load_chunk(p.x, chunk_offset<E>(j, p.units_per_row, p.ld_x, contig), ES, j < nchunks);
        }
    };
    uint32_t m = 0;
    int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    uint4 raw[R];
    fetch(t, raw);
    for (; t < ntrips; t += tstride) {
        uint4 nxt[R];
        fetch(t + tstride, nxt);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            float y[E];
            widen_chunk<InT, E>(raw[k], y);
            if constexpr (H > 0) fwht_chunk<H, E, false>(y, lane);
#pragma unroll
            for (int i = 0; i < E; ++i) m = max(m, as_u(y[i]) & 0x7FFFFFFFu);
        }
#pragma unroll
        for (int k = 0; k < R; ++k) raw[k] = nxt[k];
    }
    // the rotation's factor fl(1 / sqrt(H)), applied to the maximum only:
    // rounding is monotone, so fl(c max |v|) = max fl(c |v|); an infinite
    // or NaN maximum stays one, which is all the per-tensor scale reads
    if constexpr (H > 0) {
        if (m < 0x7F800000u) m = as_u(as_f(m) * hadamard_coef<H>());
    }
    m = workgroup_max_u32(m);
    if (threadIdx.x == 0) p.partials[blockIdx.x] = m;
}

// ---------------------------------------------------------------------------
// Stand-alone dequantize, block MSE and the FOCUS relaxed quantizer, with the
// same chunk-per-lane layout.  Codes, scales, c and the per-block outputs are
// dense, so their index follows from a chunk's dense element index e0; only
// the row-strided tensors (x / W, G, the dequantized output, W_hat) need the
// row of the chunk.
// ---------------------------------------------------------------------------

// N values of a runtime-typed operand (fp32, bf16 or fp16) at element offset
// off, 16-byte aligned pieces: N * size is 8, 16 or 32 bytes.
template <int N>
__device__ __forceinline__ void load_rt_chunk(const void* base, int dt, int64_t off, float (&v)[N]) {
    if (dt == DT_F32) {
        const uint4* q = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + off);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const uint4 w = q[i];
            v[4 * i] = as_f(w.x); v[4 * i + 1] = as_f(w.y); v[4 * i + 2] = as_f(w.z); v[4 * i + 3] = as_f(w.w);
        }
    } else {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(base) + off;
        uint32_t w[N / 2];
        if constexpr (N == 8) {
            const uint4 t = *reinterpret_cast<const uint4*>(q);
            w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
        } else {
            static_assert(N == 4, "chunks of 4 or 8 values");
            const uint2 t = *reinterpret_cast<const uint2*>(q);
            w[0] = t.x; w[1] = t.y;
        }
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            if (dt == DT_BF16) {
                v[2 * k] = as_f(w[k] << 16);
                v[2 * k + 1] = as_f(w[k] & 0xFFFF0000u);
            } else {
                v[2 * k] = f16_bits_to_f32(w[k] & 0xFFFFu);
                v[2 * k + 1] = f16_bits_to_f32(w[k] >> 16);
            }
        }
    }
}

// Dequantize codes + scales: E = 16 / OE output values of OE bytes per lane.
template <int B, int OE, int R>
__global__ __launch_bounds__(kThreads) void k_dq_stream(DequantArgs p) {
    constexpr int E = 16 / OE;
    constexpr int BL = B < E ? B : E;
    constexpr int NB = E / BL;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float g = read_g(p.g_dev);
    const int64_t nchunks = p.units, cpr = p.units_per_row;
    const bool contig = p.ld_out == p.cols;
    const int64_t per_trip = (int64_t)kTileUnits * R;
    const int64_t ntrips = (nchunks + per_trip - 1) / per_trip;
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);
    struct Trip {
        uint32_t cw[R], scb[R][NB];
    };
    auto fetch = [&](int64_t tt, Trip& d) {
        const int64_t jb = tt * per_trip + lane;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = jb + k * kTileUnits;
            const bool valid = j < nchunks;
            d.cw[k] = valid ? load_code_word<E>(p.codes, j * E) : 0u;
#pragma unroll
            for (int b = 0; b < NB; ++b) d.scb[k][b] = valid ? p.scales[j * E / B + b] : 0u;
        }
    };
    int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    Trip cur;
    fetch(t, cur);
    for (; t < ntrips; t += tstride) {
        const int64_t j0 = t * per_trip + lane;
        Trip nxt;
        fetch(t + tstride, nxt);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = j0 + k * kTileUnits;
            if (j >= nchunks) continue;
            float S[NB];
            bool nanb[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                bool usable;
                S[b] = stored_scale(p.scale_fmt, cur.scb[k][b], g, usable);
                nanb[b] = !usable;
            }
            // signed grid values of the nibbles (hardware FP4 pair convert)
            float v[E];
            static_for<E / 2>([&](auto ki) {
                constexpr int kk = decltype(ki)::value;
                const auto g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cur.cw[k], 1.0f, kk);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i = 2 * kk + h;
                    const int b = i / BL;
                    v[i] = nanb[b] ? canonical_nan_like(g2[h]) : g2[h] * S[b];
                }
            });
            store_dq_chunk<E>(p.out, p.out_dt, chunk_offset<E>(j, cpr, p.ld_out, contig), v);
        }
        cur = nxt;
    }
}

// Per-block MSE of (rotated) x against stored codes + scales.
template <class InT, int B, int H, int R>
__global__ __launch_bounds__(kThreads) void k_mse_stream(MseArgs p) {
    constexpr int ES = ElemSize<InT>::value;
    constexpr int E = 16 / ES;
    constexpr int BL = B < E ? B : E;
    constexpr int NB = E / BL;
    constexpr int LB = B / BL;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float g = read_g(p.g_dev);
    const int64_t nchunks = p.units, cpr = p.units_per_row;
    const bool contig = p.ld_x == p.cols;
    const int64_t per_trip = (int64_t)kTileUnits * R;
    const int64_t ntrips = (nchunks + per_trip - 1) / per_trip;
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);
    struct Trip {
        uint4 raw[R];
        uint32_t cw[R], scb[R][NB];
    };
    auto fetch = [&](int64_t tt, Trip& d) {
        const int64_t jb = tt * per_trip + lane;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = jb + k * kTileUnits;
            const bool valid = j < nchunks;
            d.raw[k] = load_chunk(p.x, chunk_offset<E>(j, cpr, p.ld_x, contig), ES, valid);
            d.cw[k] = valid ? load_code_word<E>(p.codes, j * E) : 0u;
#pragma unroll
            for (int b = 0; b < NB; ++b) d.scb[k][b] = valid ? p.scales[j * E / B + b] : 0u;
        }
    };
    int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    Trip cur;
    fetch(t, cur);
    for (; t < ntrips; t += tstride) {
        const int64_t j0 = t * per_trip + lane;
        Trip nxt;
        fetch(t + tstride, nxt);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = j0 + k * kTileUnits;
            float y[E];
            widen_chunk<InT, E>(cur.raw[k], y);
            if constexpr (H > 0) fwht_chunk<H, E>(y, lane);
            // signed grid values of the nibbles (hardware FP4 pair convert)
            float gv[E];
            static_for<E / 2>([&](auto ki) {
                constexpr int kk = decltype(ki)::value;
                const auto g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cur.cw[k], 1.0f, kk);
                gv[2 * kk] = g2[0];
                gv[2 * kk + 1] = g2[1];
            });
            float mse[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                bool usable;
                const float S = stored_scale(p.scale_fmt, cur.scb[k][b], g, usable);
                float e[BL];
#pragma unroll
                for (int i = 0; i < BL; ++i) {
                    const float d = y[b * BL + i] - gv[b * BL + i] * S;
                    e[i] = d * d;
                }
                const float m = group_tree_sum<LB>(tree_sum<BL>(e)) * (1.0f / (float)B);
                mse[b] = (!usable || m != m) ? as_f(kQNaN) : m;
            }
            if (j < nchunks && (lane & (LB - 1)) == 0) {
#pragma unroll
                for (int b = 0; b < NB; ++b) p.mse[j * E / B + b] = mse[b];
            }
        }
        cur = nxt;
    }
}

// FOCUS relaxed fake-quant forward (FOCUS page, methods 2-3):
// S_q = fl(S_dq c_k), u = fl(|W| / S_q), What = (-1)^s fl(grid * S_dq).
template <class InT, int B, int K, int R>
__global__ __launch_bounds__(kThreads) void k_relaxed_fwd_stream(RelaxedArgs p) {
    constexpr int ES = ElemSize<InT>::value;
    constexpr int E = 16 / ES;
    constexpr int KL = K < E ? K : E;             // values of a sub-block in this lane
    constexpr int NK = E / KL;                    // sub-blocks (or parts) per chunk
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float g = read_g(p.g_dev);
    const int64_t nchunks = p.units, cpr = p.units_per_row;
    const bool w_contig = p.ld_w == p.cols, o_contig = p.ld_out == p.cols;
    const int64_t per_trip = (int64_t)kTileUnits * R;
    const int64_t ntrips = (nchunks + per_trip - 1) / per_trip;
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);
    struct Trip {
        uint4 raw[R];
        uint32_t ck[R][NK], scb[R][NK];
    };
    auto fetch = [&](int64_t tt, Trip& d) {
        const int64_t jb = tt * per_trip + lane;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = jb + k * kTileUnits;
            const bool valid = j < nchunks;
            d.raw[k] = load_chunk(p.w, chunk_offset<E>(j, cpr, p.ld_w, w_contig), ES, valid);
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                const int64_t e = j * E + q * KL;     // first value of this sub-block part
                d.ck[k][q] = valid ? p.c[e / K] : 0u;
                d.scb[k][q] = valid ? p.scales[e / B] : 0u;
            }
        }
    };
    int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    Trip cur;
    fetch(t, cur);
    for (; t < ntrips; t += tstride) {
        const int64_t j0 = t * per_trip + lane;
        Trip nxt;
        fetch(t + tstride, nxt);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = j0 + k * kTileUnits;
            if (j >= nchunks) continue;
            float y[E];
            widen_chunk<InT, E>(cur.raw[k], y);
            float S_dq[NK], S_q[NK], R_q[NK];
            bool ok[NK], fast[NK];
            bool all_fast = true;
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                bool ok_dq;
                S_dq[q] = stored_scale(p.scale_fmt, cur.scb[k][q], g, ok_dq);
                S_q[q] = S_dq[q] * f16_bits_to_f32(cur.ck[k][q]);
                ok[q] = ok_dq && scale_usable(S_q[q]);
                fast[q] = fast_quotient_range(S_q[q]);
                R_q[q] = fast[q] ? 1.0f / S_q[q] : 0.0f;
                all_fast = all_fast && fast[q];
            }
            uint32_t cw = 0;
            float wh[E];
            // codes from the quotient by S_q (division-free for every part, or
            // per part the quotient its scale allows: one uniform branch per
            // chunk), What = grid * S_dq; a NaN W keeps magnitude code 0
            auto encode = [&](auto all_fast_c) {
                float qv[E];
#pragma unroll
                for (int q = 0; q < NK; ++q) {
#pragma unroll
                    for (int i = 0; i < KL; ++i) {
                        const int n = q * KL + i;
                        if constexpr (decltype(all_fast_c)::value)
                            qv[n] = signed_quotient<QM_FAST, true>(y[n], S_q[q], R_q[q]);
                        else
                            qv[n] = fast[q] ? signed_quotient<QM_FAST, true>(y[n], S_q[q], R_q[q])
                                            : signed_quotient<QM_SLOW, true>(y[n], S_q[q], 0.0f);
                    }
                }
                static_for<E / 2>([&](auto ki) {
                    constexpr int kk = decltype(ki)::value;
                    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, qv[2 * kk], qv[2 * kk + 1], 1.0f, kk);
                });
            };
            if (all_fast) encode(IC<1>{});
            else encode(IC<0>{});
            static_for<E / 2>([&](auto ki) {
                constexpr int kk = decltype(ki)::value;
                const auto g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, kk);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int n = 2 * kk + h;
                    const int q = n / KL;
                    wh[n] = ok[q] ? g2[h] * S_dq[q] : canonical_nan_like(y[n]);
                }
            });
            // sub-blocks without a usable scale: sign-only nibbles
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                if (!ok[q]) {
                    const uint32_t mask = ((KL == 8 ? 0xFFFFFFFFu : ((1u << (4 * KL)) - 1u)) << (4 * q * KL));
                    uint32_t sg = 0;
#pragma unroll
                    for (int i = 0; i < KL; ++i) sg |= (as_u(y[q * KL + i]) >> 31) << (4 * (q * KL + i) + 3);
                    cw = (cw & ~mask) | sg;
                }
            }
            store_dq_chunk<E>(p.w_hat, p.out_dt, chunk_offset<E>(j, cpr, p.ld_out, o_contig), wh);
            if (p.codes) store_code_word<E>(p.codes, j * E, cw);
        }
        cur = nxt;
    }
}

// Straight-through backward to c_k (FOCUS page, method 1):
// grad_c = fl(-A / fl(c c)), A = tree sum of [S_q > 0, |u| <= 6] fl(G W).
template <class InT, int B, int K, int R>
__global__ __launch_bounds__(kThreads) void k_relaxed_bwd_stream(RelaxedArgs p) {
    constexpr int ES = ElemSize<InT>::value;
    constexpr int E = 16 / ES;
    constexpr int KL = K < E ? K : E;
    constexpr int NK = E / KL;
    constexpr int LK = K / KL;                    // lanes a sub-block spans
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float g = read_g(p.g_dev);
    const int64_t nchunks = p.units, cpr = p.units_per_row;
    const bool w_contig = p.ld_w == p.cols, g_contig = p.ld_g == p.cols;
    const int64_t per_trip = (int64_t)kTileUnits * R;
    const int64_t ntrips = (nchunks + per_trip - 1) / per_trip;
    const int64_t tstride = (int64_t)gridDim.x * (kThreads / 64);
    struct Trip {
        uint4 raw[R];
        float G[R][E];
        uint32_t ck[R][NK], scb[R][NK];
    };
    auto fetch = [&](int64_t tt, Trip& d) {
        const int64_t jb = tt * per_trip + lane;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = jb + k * kTileUnits;
            const bool valid = j < nchunks;
            d.raw[k] = load_chunk(p.w, chunk_offset<E>(j, cpr, p.ld_w, w_contig), ES, valid);
            if (valid) {
                load_rt_chunk<E>(p.grad, p.g_dt, chunk_offset<E>(j, cpr, p.ld_g, g_contig), d.G[k]);
            } else {
#pragma unroll
                for (int i = 0; i < E; ++i) d.G[k][i] = 0.0f;
            }
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                const int64_t e = j * E + q * KL;
                d.ck[k][q] = valid ? p.c[e / K] : 0u;
                d.scb[k][q] = valid ? p.scales[e / B] : 0u;
            }
        }
    };
    int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    Trip cur;
    fetch(t, cur);
    for (; t < ntrips; t += tstride) {
        const int64_t j0 = t * per_trip + lane;
        Trip nxt;
        fetch(t + tstride, nxt);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = j0 + k * kTileUnits;
            float y[E];
            widen_chunk<InT, E>(cur.raw[k], y);
            float c_k[NK], S_q[NK], R_q[NK];
            bool okq[NK], fast[NK];
            bool all_fast = true;
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                bool ok_dq;
                const float S_dq = stored_scale(p.scale_fmt, cur.scb[k][q], g, ok_dq);
                c_k[q] = f16_bits_to_f32(cur.ck[k][q]);
                S_q[q] = S_dq * c_k[q];
                okq[q] = ok_dq && scale_usable(S_q[q]);
                fast[q] = fast_quotient_range(S_q[q]);
                R_q[q] = fast[q] ? 1.0f / S_q[q] : 0.0f;
                all_fast = all_fast && fast[q];
            }
            float part[NK];
            auto terms = [&](auto all_fast_c) {
#pragma unroll
                for (int q = 0; q < NK; ++q) {
                    float tt[KL];
#pragma unroll
                    for (int i = 0; i < KL; ++i) {
                        const int n = q * KL + i;
                        const float a = fabsf(y[n]);
                        float u;
                        if constexpr (decltype(all_fast_c)::value) u = quotient<SF_E4M3, true>(a, S_q[q], R_q[q]);
                        else u = fast[q] ? quotient<SF_E4M3, true>(a, S_q[q], R_q[q])
                                         : quotient<SF_E4M3, false>(a, S_q[q], 0.0f);
                        const bool inside = (S_q[q] > 0.0f) && (u <= 6.0f);
                        tt[i] = inside ? cur.G[k][n] * y[n] : 0.0f;
                    }
                    part[q] = tree_sum<KL>(tt);
                }
            };
            if (all_fast) terms(IC<1>{});
            else terms(IC<0>{});
            float out[NK];
#pragma unroll
            for (int q = 0; q < NK; ++q) {
                const float A = group_tree_sum<LK>(part[q]);
                out[q] = -A / (c_k[q] * c_k[q]);
            }
            if (j < nchunks && (lane & (LK - 1)) == 0) {
#pragma unroll
                for (int q = 0; q < NK; ++q) {
                    const int64_t ci = (j * E + q * KL) / K;
                    p.grad_c[ci] = (okq[q] && out[q] == out[q]) ? out[q] : as_f(kQNaN);
                }
            }
        }
        cur = nxt;
    }
}

}  // namespace fp4q_dev
