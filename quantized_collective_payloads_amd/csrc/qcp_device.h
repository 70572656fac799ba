// qcp_device.h -- device-side building blocks of the gfx950 payload kernels.
//
// Everything here is written for CDNA4 wave64: cross-lane reductions use DPP
// (quad_perm, row_half_mirror, row_mirror) inside a row of 16 lanes and
// ds_swizzle across 32 lanes; 16-byte global loads/stores; hardware fp8/bf16/fp16
// conversions of gfx950.  Floating point follows IEEE binary32 exactly: the
// library is built with -ffp-contract=off and fp32 denormals enabled, and every
// fused multiply-add below is written out.
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
// exact binary32 quotient
// ---------------------------------------------------------------------------
// The scale s of a block is positive; r = RN(1/s) is computed once per block by
// an IEEE division.  For s in [2^-64, 2^64]:
//   y0 = RN(x*r) is within two ulps of x/s;
//   y1 = RN(y0 + RN(x - y0*s)*r) is then within one ulp (faithful);
//   with y1 faithful the residual x - y1*s is exact in one fma, and
//   RN(y1 + (x - y1*s)*r) = RN(x/s)            (P. Markstein, IBM J. R&D 34(1), 1990)
// as long as nothing underflows; quotients small enough for the residual to
// underflow round to code 0 / E4M3 +-0 either way.  Five VALU operations instead
// of the ~12 of a full IEEE division.  Other scales take quot_ieee().
constexpr float kFastScaleMin = 5.42101086e-20f;   // 2^-64
constexpr float kFastScaleMax = 1.84467441e+19f;   // 2^64

__device__ __forceinline__ float quot_fast(float x, float s, float r) {
    float y = x * r;
    float e = __builtin_fmaf(-y, s, x);
    y = __builtin_fmaf(e, r, y);
    e = __builtin_fmaf(-y, s, x);
    return __builtin_fmaf(e, r, y);
}

__device__ __forceinline__ float quot_ieee(float x, float s) { return x / s; }

__device__ __forceinline__ bool scale_is_fast(float s) {
    return s == 0.0f || (s >= kFastScaleMin && s <= kFastScaleMax);
}

// INT code of a quotient: round half to even, clamp to [-qmax, qmax].
template <int FMT>
__device__ __forceinline__ int int_code(float q) {
    constexpr float qm = fmt_traits<FMT>::qmax;
    float c = __builtin_rintf(q);
    c = __builtin_amdgcn_fmed3f(c, -qm, qm);
    return (int)c;
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

// bf16 round trip of one value: fp32 -> nearest bf16 -> fp32
__device__ __forceinline__ float round_bf16(float a) {
    f32x2_t v = {a, a};
    bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    return __uint_as_float(__builtin_bit_cast(uint32_t, h) << 16);
}

// the 16-bit pattern of |max| over the halves of a dword (pk_max on u16 lanes)
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax16_acc(uint32_t acc, uint32_t w) {
    u16x2_t a = __builtin_bit_cast(u16x2_t, acc);
    u16x2_t b = __builtin_bit_cast(u16x2_t, w & 0x7fff7fffu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// fp32 bit pattern of the larger half of a packed absmax
template <int XT>
__device__ __forceinline__ uint32_t absmax16_to_f32bits(uint32_t acc) {
    uint32_t h = max(acc & 0xffffu, acc >> 16);
    if constexpr (XT == BF16) return h << 16;
    else return __float_as_uint((float)__builtin_bit_cast(_Float16, (unsigned short)h));
}

// ---------------------------------------------------------------------------
// E4M3 (OCP E4M3FN on gfx950)
// ---------------------------------------------------------------------------
// four quotients -> four E4M3 codes in one dword (byte i = code of q_i),
// round to nearest even; |q| never exceeds 448 by more than rounding here.
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
// packing 8 codes (one vector) into b bits each; layout LSB-first
// ---------------------------------------------------------------------------
struct Packed8 {       // up to 8 bytes: lo = bytes 0..3, hi = bytes 4..7
    uint32_t lo, hi;
};

template <int FMT>
__device__ __forceinline__ Packed8 pack8_int(const int (&c)[8]) {
    Packed8 p;
    if constexpr (FMT == INT8) {
        p.lo = (uint32_t)(c[0] & 0xff) | ((uint32_t)(c[1] & 0xff) << 8) |
               ((uint32_t)(c[2] & 0xff) << 16) | ((uint32_t)c[3] << 24);
        p.hi = (uint32_t)(c[4] & 0xff) | ((uint32_t)(c[5] & 0xff) << 8) |
               ((uint32_t)(c[6] & 0xff) << 16) | ((uint32_t)c[7] << 24);
    } else if constexpr (FMT == INT4) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) w |= (uint32_t)(c[i] & 0xf) << (4 * i);
        p.lo = w;
        p.hi = 0;
    } else if constexpr (FMT == INT2) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) w |= (uint32_t)(c[i] & 0x3) << (2 * i);
        p.lo = w;
        p.hi = 0;
    } else {  // INT6: 48 bits
        uint32_t lo = 0;
#pragma unroll
        for (int i = 0; i < 5; i++) lo |= (uint32_t)(c[i] & 0x3f) << (6 * i);
        lo |= (uint32_t)(c[5] & 0x3) << 30;
        uint32_t hi = ((uint32_t)(c[5] & 0x3f) >> 2) | ((uint32_t)(c[6] & 0x3f) << 4) |
                      ((uint32_t)(c[7] & 0x3f) << 10);
        p.lo = lo;
        p.hi = hi;
    }
    return p;
}

// signed field i (0..7) of a vector's packed codes -> float
template <int FMT>
__device__ __forceinline__ float field_value(const Packed8 &p, int i) {
    if constexpr (FMT == INT8) {
        uint32_t w = i < 4 ? p.lo : p.hi;
        return (float)(((int32_t)(w << (24 - 8 * (i & 3)))) >> 24);
    } else if constexpr (FMT == INT4) {
        return (float)(((int32_t)(p.lo << (28 - 4 * i))) >> 28);
    } else if constexpr (FMT == INT2) {
        return (float)(((int32_t)(p.lo << (30 - 2 * i))) >> 30);
    } else {
        uint64_t w = (uint64_t)p.lo | ((uint64_t)p.hi << 32);
        return (float)(((int64_t)(w << (58 - 6 * i))) >> 58);
    }
}

// bytes that 8 codes occupy
template <int FMT> constexpr int vec_bytes() { return fmt_traits<FMT>::bits; }

}  // namespace qcp
