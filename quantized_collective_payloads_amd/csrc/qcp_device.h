// qcp_device.h -- device-side building blocks of the gfx950 payload kernels.
//
// Everything here is written for CDNA4 wave64: cross-lane reductions use DPP
// (quad_perm, row_half_mirror, row_mirror) inside a row of 16 lanes and
// ds_swizzle across 32 lanes; 16-byte global loads/stores; hardware fp8/bf16/fp16
// conversions of gfx950; v_perm_b32 byte gathers for packing.  Floating point
// follows IEEE binary32: the library is built with -ffp-contract=off and fp32
// denormals enabled, and every fused multiply-add below is written out.  (It is
// also built without NaN semantics: inputs are finite by contract, which lets
// max/max3 take |x| operands without canonicalization.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace qcp {

enum DType : int { F16 = 1, BF16 = 2, F32 = 3 };
enum Fmt : int { INT2 = 2, INT4 = 4, INT6 = 6, INT8 = 8, E4M3 = 0x43 };

template <int FMT> struct fmt_traits {
    static constexpr int bits = FMT;
    static constexpr float qmax = (float)((1 << (FMT - 1)) - 1);
};
template <> struct fmt_traits<E4M3> {
    static constexpr int bits = 8;
    static constexpr float qmax = 448.0f;
};

template <int XT> struct dtype_traits { static constexpr int bytes = 2; };
template <> struct dtype_traits<F32> { static constexpr int bytes = 4; };

// unrolled loops over compile-time indices
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// cross-lane max inside aligned groups of GL lanes (GL a power of two <= 64);
// every lane of the group receives the group's maximum.  Operates on the bit
// patterns of non-negative floats, whose unsigned order is their numeric order.
// All 64 lanes must be active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

template <int GL>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    if constexpr (GL >= 2) v = max(v, dpp_u32<0xB1>(v));     // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (GL >= 4) v = max(v, dpp_u32<0x4E>(v));     // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (GL >= 8) v = max(v, dpp_u32<0x141>(v));    // row_half_mirror: 8-lane max
    if constexpr (GL >= 16) v = max(v, dpp_u32<0x140>(v));   // row_mirror: 16-lane max
    if constexpr (GL >= 32)                                  // swizzle xor 16 within 32 lanes
        v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
    if constexpr (GL >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// ---------------------------------------------------------------------------
// streaming (non-temporal) 16-byte global accesses, for data a kernel reads or
// writes exactly once.  The hint keeps such lines from being retained in the
// caches: on MI355X a kernel whose 16-bit output is written this way no longer
// leaves hundreds of MB dirty in the Infinity Cache for the next kernel to
// write back (measured: INT2 unpack of 235M elements 77 us back to back, against
// 103 us with ordinary stores).  Results are unchanged; only cache policy is.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void *p) {
    u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream16(void *p, uint4 v) {
    u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (u32x4_t *)p);
}

// ---------------------------------------------------------------------------
// exact binary32 quotients
// ---------------------------------------------------------------------------
// For positive s and r = RN(1/s), with no underflow or overflow in between:
//   y0 = RN(x*r) is within two ulps of x/s;
//   y1 = RN(y0 + RN(x - y0*s)*r) is then within one ulp (faithful);
//   with y1 faithful the residual x - y1*s is exact in one fma, and
//   RN(y1 + (x - y1*s)*r) = RN(x/s)            (P. Markstein, IBM J. R&D 34(1), 1990).
// Five VALU operations instead of the ~11 of an IEEE division.  It is used for
// element quotients when the block scale lies in [2^-64, 2^64] (quotients small
// enough for the residual to underflow round to code 0 / E4M3 +-0 either way),
// and for the block scale itself (absmax / qmax, r = RN(1/qmax) a constant)
// under the same range condition on the result.
constexpr float kFastScaleMin = 5.42101086e-20f;   // 2^-64
constexpr float kFastScaleMax = 1.84467441e+19f;   // 2^64

// The residual is formed as e = y*s - x and applied as y - e*r (negations are free
// source modifiers): by the symmetry of round-to-nearest these are the same
// values as x - y*s and y + (x - y*s)*r, but a zero result keeps x's sign (for
// x = -0, -0*r = -0, and every correction adds another -0), which the E4M3 code
// of a signed zero needs.
__device__ __forceinline__ float quot_fast(float x, float s, float r) {
    float y = x * r;
    float e = __builtin_fmaf(y, s, -x);
    y = __builtin_fmaf(-e, r, y);
    e = __builtin_fmaf(y, s, -x);
    return __builtin_fmaf(-e, r, y);
}

__device__ __forceinline__ bool scale_in_fast_range(float s) {
    return s == 0.0f || (s >= kFastScaleMin && s <= kFastScaleMax);
}

// RN(1/s) for s in [2^-64, 2^64]: the hardware reciprocal approximation plus one
// Newton correction, y + y*(1 - s*y) with the residual in one fma.  This equals
// the IEEE quotient 1/s for every s in that range -- checked exhaustively on
// gfx950 over all 2^23 significands of each of its 128 binades (the
// hardware self-test under tests/hw).  Three VALU operations instead of ~11.
__device__ __forceinline__ float recip_fast(float s) {
    float y = __builtin_amdgcn_rcpf(s);
    float e = __builtin_fmaf(-s, y, 1.0f);
    return __builtin_fmaf(e, y, y);
}

// Block scale and its reciprocal.  `fast` reports whether quot_fast() is exact
// for this block's element quotients; when it is not (tiny or huge blocks),
// callers divide with IEEE '/'.  r is 0 for a zero block (every code is 0 then).
template <int FMT> struct BlockScale {
    float s, r;
    bool fast;
};

template <int FMT>
__device__ __forceinline__ BlockScale<FMT> block_scale(float absmax) {
    constexpr float qm = fmt_traits<FMT>::qmax;
    constexpr float rq = 1.0f / qm;                     // RN(1/qmax), folded at compile time
    BlockScale<FMT> b;
    float s = quot_fast(absmax, qm, rq);
    bool fast = scale_in_fast_range(s);
    if (!__all(fast)) {                                 // rare, wave-uniform: IEEE division
        s = fast ? s : absmax / qm;
        fast = scale_in_fast_range(s);    // a subnormal absmax can still give s = 0
    }
    b.s = s;
    b.fast = fast;
    b.r = (s == 0.0f || !fast) ? 0.0f : recip_fast(s);
    return b;
}

// ---------------------------------------------------------------------------
// codes as "magic" floats: t = RN(q + 1.5*2^23).  For |q| < 2^22 the addition
// rounds q to an integer, ties to even, and the low bits of t's bit pattern
// are that integer in two's complement -- the code field, ready to pack.  In
// the fast range |q| <= qmax*(1 + 2^-22), so round(q) never exceeds qmax and
// needs no clamp; the slow path clamps first.
// ---------------------------------------------------------------------------
constexpr float kMagic = 12582912.0f;               // 1.5 * 2^23

template <int FMT, bool FAST>
__device__ __forceinline__ uint32_t int_code_bits(float x, const BlockScale<FMT> &b) {
    if constexpr (FAST) {
        return __float_as_uint(quot_fast(x, b.s, b.r) + kMagic);
    } else {
        constexpr float qm = fmt_traits<FMT>::qmax;
        float q = b.fast ? quot_fast(x, b.s, b.r) : x / b.s;
        q = __builtin_amdgcn_fmed3f(__builtin_rintf(q), -qm, qm);
        return __float_as_uint(q + kMagic);
    }
}

// INT codes from two products that bracket the quotient, for blocks in the
// fast range.  With r = RN(1/s) and r_lo, r_hi = RN(r*(1 -+ 2^-21)), the exact
// products x*r_lo and x*r_hi enclose fl(x/s): each of r, r_lo, r_hi is within
// 2^-24 (relative) of what it rounds, so x*r_lo is at most
// (x/s)*(1 - 2^-21 + 2^-23) in magnitude on one side and x*r_hi at least
// (x/s)*(1 + 2^-21 - 2^-23) on the other, while fl(x/s) is within
// (x/s)*2^-24 of x/s (or, for |x/s| below the normal range, everything rounds
// to 0).  Rounding to integers is monotone, so when
// t_lo = RN(x*r_lo + 1.5*2^23) and t_hi = RN(x*r_hi + 1.5*2^23) (one fma each,
// the product held exactly) agree, fl(x/s) rounds to the same integer, ties
// included.  The caller ors t_lo ^ t_hi over its elements into `diff` (one
// v_bitop3 per element)
// and recomputes the codes with the exact quotient when it is nonzero: when an
// integer + 1/2 falls inside the bracket, about qmax*2^-20 of the elements for
// quotients spread evenly.  Three operations per element against six for
// quot_fast + t.  (A block of zeros has r = 0: every code is 0, diff stays 0.)
struct RecipBracket {
    float lo, hi;
};

__device__ __forceinline__ RecipBracket recip_bracket(float r) {
    return RecipBracket{__builtin_fmaf(r, -0x1p-21f, r), __builtin_fmaf(r, 0x1p-21f, r)};
}

__device__ __forceinline__ uint32_t int_code_bits_bracket(float x, RecipBracket rb, uint32_t &diff) {
    const uint32_t a = __float_as_uint(__builtin_fmaf(x, rb.lo, kMagic));
    const uint32_t b = __float_as_uint(__builtin_fmaf(x, rb.hi, kMagic));
    // diff | (a ^ b) as one v_bitop3 (truth table 0xf6 over diff, a, b); written
    // out as C, the compiler turns the or-of-xors into one compare per element
    diff = __builtin_amdgcn_bitop3_b32(diff, a, b, 0xf6);
    return a;
}

template <int FMT, bool FAST>
__device__ __forceinline__ float e4m3_quotient(float x, const BlockScale<FMT> &b) {
    if constexpr (FAST) {
        return quot_fast(x, b.s, b.r);                         // keeps the sign of zero
    } else {
        const float q = b.fast ? quot_fast(x, b.s, b.r) : x / b.s;   // IEEE '/' does too
        return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
    }
}

// ---------------------------------------------------------------------------
// 16-bit <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

template <int XT>
__device__ __forceinline__ float widen_lo(uint32_t w) {
    if constexpr (XT == BF16) return bf16_lo(w); else return f16_lo(w);
}
template <int XT>
__device__ __forceinline__ float widen_hi(uint32_t w) {
    if constexpr (XT == BF16) return bf16_hi(w); else return f16_hi(w);
}

// round-to-nearest-even fp32 -> 16-bit pair packed in one dword (lo, hi)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int YT>
__device__ __forceinline__ uint32_t narrow2(float a, float b) {
    f32x2_t v = {a, b};
    if constexpr (YT == BF16) {
        bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
        return __builtin_bit_cast(uint32_t, h);
    } else {
        f16x2_t h = __builtin_convertvector(v, f16x2_t);
        return __builtin_bit_cast(uint32_t, h);
    }
}

// bf16 round trips of two values: fp32 -> nearest bf16 -> fp32 (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ void round_bf16x2(float &a, float &b) {
    uint32_t h = narrow2<BF16>(a, b);
    a = bf16_lo(h);
    b = bf16_hi(h);
}

// ---------------------------------------------------------------------------
// E4M3 (OCP E4M3FN on gfx950)
// ---------------------------------------------------------------------------
// four quotients -> four E4M3 codes in one dword (byte i = code of q_i), round to
// nearest even; callers pass |q| <= 448 plus at most two ulps (e4m3_quotient).
__device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
    return (uint32_t)w;
}

template <int BYTE>
__device__ __forceinline__ float e4m3_value(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8((int)w, BYTE);
}

// ---------------------------------------------------------------------------
// one-instruction code -> float conversions through SDWA byte selects (both
// checked on gfx950 over every byte/nibble pattern by the hardware self-test):
//   v_cvt_f32_i32 with sext(BYTE_k):   float((int8_t) byte k)
//   v_cvt_off_f32_i4 with BYTE_k:      (signed low nibble of byte k) / 16
// Written as plain code: the compiler folds the byte select into the SDWA
// operand (one instruction each, as the gfx950 assembly shows), and, unlike
// inline asm, sees the instructions, so it needs no conservative hazard waits
// around them.  The high nibbles of a word come from the same selects on the
// word rotated right by 4 (a rotate, not a shift, so that the compiler does not
// turn shift-and-select back into a bit-field extract per nibble).
// ---------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ float cvt_sbyte(uint32_t w) {
    return (float)(int32_t)(int8_t)(w >> (8 * K));
}

template <int K>
__device__ __forceinline__ float cvt_nibble_16th(uint32_t w) {
    if constexpr (K == 3) return __builtin_amdgcn_cvt_off_f32_i4((int)(w >> 24));
    else return __builtin_amdgcn_cvt_off_f32_i4((int)((w >> (8 * K)) & 0xffu));
}

// w rotated right by 4 bits: byte k's low nibble is nibble 2k+1 of w
__device__ __forceinline__ uint32_t odd_nibbles(uint32_t w) { return __builtin_amdgcn_alignbit(w, w, 4); }

// ---------------------------------------------------------------------------
// packing the codes of 8 consecutive elements (one "vector"); LSB-first fields
// ---------------------------------------------------------------------------
struct Packed8 {       // up to 8 bytes: lo = bytes 0..3, hi = bytes 4..7
    uint32_t lo, hi;
};

// low bytes of four dwords -> one dword (v_perm_b32 byte gathers)
__device__ __forceinline__ uint32_t gather_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                     uint32_t b3) {
    uint32_t p01 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);   // [b0.0, b1.0, 0, 0]
    uint32_t p23 = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);   // [b2.0, b3.0, 0, 0]
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);         // [b0.0, b1.0, b2.0, b3.0]
}

// t[i]: magic-float bit patterns whose low bits are code i (two's complement)
template <int FMT>
__device__ __forceinline__ Packed8 pack8_codes(const uint32_t (&t)[8]) {
    Packed8 p;
    if constexpr (FMT == INT8) {
        p.lo = gather_low_bytes(t[0], t[1], t[2], t[3]);
        p.hi = gather_low_bytes(t[4], t[5], t[6], t[7]);
    } else if constexpr (FMT == INT4) {
        uint32_t ev = gather_low_bytes(t[0], t[2], t[4], t[6]);
        uint32_t od = gather_low_bytes(t[1], t[3], t[5], t[7]);
        p.lo = ((od << 4) & 0xf0f0f0f0u) | (ev & 0x0f0f0f0fu);
        p.hi = 0;
    } else if constexpr (FMT == INT2) {
        // fields f_i = low 2 bits of t_i.  Gather four codes' low bytes, keep
        // their fields (f_i at bit 8i), then fold: x | x >> 6 brings f1 next to
        // f0 and f3 next to f2, x | x >> 12 brings f2 f3 down to bits 4..7, so
        // the low byte is f0 | f1 << 2 | f2 << 4 | f3 << 6.  About two
        // operations per code against three for a shift-and-or per field.
        auto fold4 = [](uint32_t x) {
            x &= 0x03030303u;
            x |= x >> 6;
            return x | (x >> 12);
        };
        const uint32_t a = fold4(gather_low_bytes(t[0], t[1], t[2], t[3]));
        const uint32_t b = fold4(gather_low_bytes(t[4], t[5], t[6], t[7]));
        p.lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);     // [a.0, b.0, 0, 0]
        p.hi = 0;
    } else {  // INT6: 48 bits
        uint32_t lo = 0;
#pragma unroll
        for (int i = 0; i < 5; i++) lo |= (t[i] & 0x3fu) << (6 * i);
        lo |= (t[5] & 0x3u) << 30;
        uint32_t hi = ((t[5] >> 2) & 0xfu) | ((t[6] & 0x3fu) << 4) | ((t[7] & 0x3fu) << 10);
        p.lo = lo;
        p.hi = hi;
    }
    return p;
}

// quantize 8 widened values with their block's scale -> packed codes
template <int FMT, bool FAST>
__device__ __forceinline__ Packed8 quantize8(const float (&x)[8], const BlockScale<FMT> &b) {
    Packed8 p;
    if constexpr (FMT == E4M3) {
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; i++) q[i] = e4m3_quotient<FMT, FAST>(x[i], b);
        p.lo = e4m3_pack4(q[0], q[1], q[2], q[3]);
        p.hi = e4m3_pack4(q[4], q[5], q[6], q[7]);
    } else {
        uint32_t t[8];
#pragma unroll
        for (int i = 0; i < 8; i++) t[i] = int_code_bits<FMT, FAST>(x[i], b);
        p = pack8_codes<FMT>(t);
    }
    if (b.s == 0.0f) { p.lo = 0; p.hi = 0; }   // a block of zeros: every code is 0
    return p;
}

// quantize8<FMT, true> for INT formats through int_code_bits_bracket: the same
// codes while diff stays 0.
template <int FMT>
__device__ __forceinline__ Packed8 quantize8_bracket(const float (&x)[8], RecipBracket rb,
                                                     uint32_t &diff) {
    static_assert(FMT != E4M3, "INT formats only");
    uint32_t t[8];
#pragma unroll
    for (int i = 0; i < 8; i++) t[i] = int_code_bits_bracket(x[i], rb, diff);
    return pack8_codes<FMT>(t);
}

// signed field i (0..7) of a vector's packed codes -> float
template <int FMT, int I>
__device__ __forceinline__ float field_value(const Packed8 &p) {
    if constexpr (FMT == INT8) {
        return cvt_sbyte<I & 3>(I < 4 ? p.lo : p.hi);
    } else if constexpr (FMT == INT4) {
        return (float)(((int32_t)(p.lo << (28 - 4 * I))) >> 28);
    } else if constexpr (FMT == INT2) {
        return (float)(((int32_t)(p.lo << (30 - 2 * I))) >> 30);
    } else {  // INT6: bits [6I, 6I+6) of the 48-bit (hi:lo)
        constexpr int bit = 6 * I;
        uint32_t v;
        if constexpr (bit + 6 <= 32) v = p.lo << (26 - bit);
        else if constexpr (bit >= 32) v = p.hi << (26 - (bit - 32));
        else v = __builtin_amdgcn_alignbit(p.hi, p.lo, bit) << 26;
        return (float)(((int32_t)v) >> 26);
    }
}

// bytes that 8 codes occupy
template <int FMT> constexpr int vec_bytes() { return fmt_traits<FMT>::bits; }

}  // namespace qcp
