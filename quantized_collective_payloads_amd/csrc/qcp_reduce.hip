// qcp_reduce.hip -- fused N-slice dequantize -> fp32 sum -> requantize, and the
// in-place FP8 main-gradient accumulate.
//
// Method: [ZPP] "Quantized LLM Training at Scale with ZeRO++", sections "QGZ
// keeps reductions in full precision while sending quantized gradients" and
// "The implementation combines kernel fusion with communication overlap" (the
// intra-node dequantization and reduction are fused with the next hop's
// quantization to cut global-memory traffic).  [AGOQ] "AGoQ ...", Section 2.B
// QuanGrad: "Local Accumulation" and step 2 "Local Reduce" of the
// precision-preserved all-reduce.
//
// Layout: the N slices a rank receives sit in one HBM allocation, slice j at
// codes_in + j*stride, its scales at scales_in + j*scale_stride, exactly as an
// all-to-all would leave them.  Blocks restart at each slice.
//
// Geometry of the reduce: a lane owns "chunks" of CPL consecutive elements whose
// codes are one 16-byte load (INT4, INT8, E4M3: 32/16/16 codes), 8 bytes (INT2,
// 32 codes) or 12 bytes (INT6, 16 codes).  A block of G elements is G/CPL
// chunks over GL <= 16 lanes, U chunks per lane.  For each slice in order a lane
// loads its chunks and one scale and runs acc = fmaf(value, scale, acc) on CPL*U
// fp32 accumulators that never leave registers; then the block absmax is a DPP
// max over the GL lanes, and the sums are quantized and packed in registers and
// stored as whole dwords.  Each output byte has one writer; no LDS, no atomics.
#include "qcp_device.h"
#include "qcp_launch.h"

namespace qcp {

template <int FMT> struct chunk_traits {
    static constexpr int CPL = (FMT == INT2 || FMT == INT4) ? 32 : 16;   // codes per chunk
};

template <int FIN, int G> struct rgeom {
    static constexpr int CPL = chunk_traits<FIN>::CPL;
    static constexpr int C = G / CPL;                        // chunks per block
    static constexpr int U = C > 16 ? C / 16 : 1;            // chunks per lane
    static constexpr int GL = C / U;                         // lanes per block (<= 16)
    static constexpr int BPW = 64 / GL;                      // blocks per wave
    static_assert(GL * U * CPL == G && GL <= 16, "reduce geometry");
};

// number of 32-bit words that n codes of format FMT occupy (n*b a multiple of 32)
template <int FMT, int N> constexpr int words_of() { return N * fmt_traits<FMT>::bits / 32; }

// ---- word-level I/O (whole, 4-byte-aligned dwords) ----
// three dwords with 4-byte alignment (one global_load/store_dwordx3); HIP's
// uint3 is not used because its storage may be padded to 16 bytes.
struct alignas(4) words3 { uint32_t a, b, c; };

template <int NW>
__device__ __forceinline__ void load_words(const uint8_t *p, uint32_t (&w)[NW]) {
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 4) {
            uint4 v = *(const uint4 *)(p + 4 * i);
            w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
        }
    } else if constexpr (NW == 3) {
        words3 v = *(const words3 *)p;
        w[0] = v.a; w[1] = v.b; w[2] = v.c;
    } else if constexpr (NW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 2) {
            uint2 v = *(const uint2 *)(p + 4 * i);
            w[i] = v.x; w[i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; i++) w[i] = *(const uint32_t *)(p + 4 * i);
    }
}

// the same, for data read exactly once (streaming hint on 16-byte loads)
template <int NW>
__device__ __forceinline__ void load_words_stream(const uint8_t *p, uint32_t (&w)[NW]) {
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 4) {
            uint4 v = load_stream16(p + 4 * i);
            w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
        }
    } else {
        load_words<NW>(p, w);
    }
}

template <int NW>
__device__ __forceinline__ void store_words_stream(uint8_t *p, const uint32_t (&w)[NW]) {
    static_assert(NW % 4 == 0, "16-byte units");
#pragma unroll
    for (int i = 0; i < NW; i += 4) store_stream16(p + 4 * i, make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]));
}

template <int NW>
__device__ __forceinline__ void load_words_tail(const uint8_t *p, uint32_t (&w)[NW],
                                                int64_t valid) {
#pragma unroll
    for (int i = 0; i < NW; i++) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; b++)
            if (4 * i + b < valid) v |= (uint32_t)p[4 * i + b] << (8 * b);
        w[i] = v;
    }
}

template <int NW>
__device__ __forceinline__ void store_words(uint8_t *p, const uint32_t (&w)[NW]) {
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 4) *(uint4 *)(p + 4 * i) = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
    } else if constexpr (NW == 3) {
        *(words3 *)p = words3{w[0], w[1], w[2]};
    } else if constexpr (NW == 6) {
        *(words3 *)p = words3{w[0], w[1], w[2]};
        *(words3 *)(p + 12) = words3{w[3], w[4], w[5]};
    } else if constexpr (NW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NW; i += 2) *(uint2 *)(p + 4 * i) = make_uint2(w[i], w[i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < NW; i++) *(uint32_t *)(p + 4 * i) = w[i];
    }
}

template <int NW>
__device__ __forceinline__ void store_words_tail(uint8_t *p, const uint32_t (&w)[NW],
                                                 int64_t valid) {
#pragma unroll
    for (int i = 0; i < NW; i++)
#pragma unroll
        for (int b = 0; b < 4; b++)
            if (4 * i + b < valid) p[4 * i + b] = (uint8_t)(w[i] >> (8 * b));
}

// ---- code i of a chunk held in words -> float (I is a compile-time index) ----
template <int FMT, int I, int NW>
__device__ __forceinline__ float chunk_value(const uint32_t (&w)[NW]) {
    if constexpr (FMT == E4M3) {
        return e4m3_value<I % 4>(w[I / 4]);
    } else if constexpr (FMT == INT8) {
        return cvt_sbyte<I % 4>(w[I / 4]);
    } else {
        constexpr int b = fmt_traits<FMT>::bits;
        constexpr int bit = b * I, wi = bit / 32, off = bit % 32;
        uint32_t v;
        if constexpr (off + b <= 32) {
            v = w[wi] >> off;
        } else {
            v = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off);
        }
        return (float)(((int32_t)(v << (32 - b))) >> (32 - b));
    }
}

template <int FMT, int I, int NW>
__device__ __forceinline__ void chunk_put(uint32_t (&w)[NW], uint32_t field) {
    constexpr int b = fmt_traits<FMT>::bits;
    constexpr int bit = b * I, wi = bit / 32, off = bit % 32;
    w[wi] |= field << off;
    if constexpr (off + b > 32) w[wi + 1] |= field >> (32 - off);
}

// place the packed codes of the g-th group of 8 values into a chunk's words
template <int FMT, int g, int NW>
__device__ __forceinline__ void place_group(uint32_t (&w)[NW], const Packed8 &p) {
    if constexpr (FMT == INT8 || FMT == E4M3) {
        w[2 * g] = p.lo;
        w[2 * g + 1] = p.hi;
    } else if constexpr (FMT == INT4) {
        w[g] = p.lo;
    } else if constexpr (FMT == INT2) {
        if constexpr (g % 2 == 0) w[g / 2] = p.lo;
        else w[g / 2] |= p.lo << 16;
    } else {  // INT6: two groups = 96 bits = 3 words
        constexpr int w0 = 3 * (g / 2);
        if constexpr (g % 2 == 0) {
            w[w0] = p.lo;
            w[w0 + 1] = p.hi;
        } else {
            w[w0 + 1] |= p.lo << 16;
            w[w0 + 2] = (p.lo >> 16) | (p.hi << 16);
        }
    }
}

// quantize CPL values of a chunk into the words of format FOUT
template <int FOUT, int CPL, bool FAST>
__device__ __forceinline__ void quantize_chunk(const float (&v)[CPL], const BlockScale<FOUT> &b,
                                               uint32_t (&w)[words_of<FOUT, CPL>()]) {
    static_for<CPL / 8>([&](auto GI) {
        constexpr int g = decltype(GI)::value;
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; i++) x[i] = v[8 * g + i];
        place_group<FOUT, g>(w, quantize8<FOUT, FAST>(x, b));
    });
}

// the same through quantize8_bracket (INT formats, fast range): equal to
// quantize_chunk<FOUT, CPL, true> while diff stays 0
template <int FOUT, int CPL>
__device__ __forceinline__ void quantize_chunk_bracket(const float (&v)[CPL], RecipBracket rb,
                                                       uint32_t (&w)[words_of<FOUT, CPL>()],
                                                       uint32_t &diff) {
    static_for<CPL / 8>([&](auto GI) {
        constexpr int g = decltype(GI)::value;
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; i++) x[i] = v[8 * g + i];
        place_group<FOUT, g>(w, quantize8_bracket<FOUT>(x, rb, diff));
    });
}

// codes of a chunk in the fast range, by the shortest exact route.  Used by the
// 8-slice INT4 reduce, which is bound by its VALU issue rate.  (In the
// encoders and the general reduce, whose waves wait on memory latency rather
// than on the VALU, the extra branch measured slower.)
template <int FOUT, int CPL>
__device__ __forceinline__ void quantize_chunk_fast(const float (&v)[CPL], const BlockScale<FOUT> &b,
                                                    uint32_t (&w)[words_of<FOUT, CPL>()]) {
    if constexpr (FOUT == E4M3) {
        quantize_chunk<FOUT, CPL, true>(v, b, w);
    } else {
        uint32_t diff = 0;
        quantize_chunk_bracket<FOUT, CPL>(v, recip_bracket(b.r), w, diff);
        if (diff != 0) quantize_chunk<FOUT, CPL, true>(v, b, w);
    }
}

// INT4 input, fast form: v_cvt_off_f32_i4 turns a nibble into code/16 in one
// instruction (even nibbles from the word, odd ones from the word rotated
// right by 4), and with s16 = 16*s (exact: a power-of-two scaling that stays
// finite) fmaf(code/16, s16, acc) == fmaf(code, s, acc) bit for bit.
constexpr float kScaleX16Max = 1.06338240e+37f;   // 2^123: 16*s stays finite

// ---- the reduce kernel ----

// acc[i] = fmaf(value(c_i), s, acc[i]) for the CPL codes of one chunk, in
// slice order.  INT4 input decodes through code/16: FAST16 multiplies it by
// s16 = 16*s; otherwise (16*s would overflow) it is scaled back to the code
// first (exact), one more multiply per element with the same register use.
template <int FIN, int CPL, bool FAST16, int NW>
__device__ __forceinline__ void accumulate_chunk(const uint32_t (&w)[NW], float s, float s16,
                                                 float (&acc)[CPL]) {
    if constexpr (FIN == INT4) {
#pragma unroll
        for (int d = 0; d < NW; d++) {
            const uint32_t hi = odd_nibbles(w[d]);
            static_for<4>([&](auto K) {
                constexpr int k = decltype(K)::value;
                float v0 = cvt_nibble_16th<k>(w[d]), v1 = cvt_nibble_16th<k>(hi);
                if constexpr (FAST16) {
                    acc[8 * d + 2 * k] = __builtin_fmaf(v0, s16, acc[8 * d + 2 * k]);
                    acc[8 * d + 2 * k + 1] = __builtin_fmaf(v1, s16, acc[8 * d + 2 * k + 1]);
                } else {
                    acc[8 * d + 2 * k] = __builtin_fmaf(v0 * 16.0f, s, acc[8 * d + 2 * k]);
                    acc[8 * d + 2 * k + 1] = __builtin_fmaf(v1 * 16.0f, s, acc[8 * d + 2 * k + 1]);
                }
            });
        }
    } else {
        static_for<CPL>([&](auto I) {
            constexpr int i = decltype(I)::value;
            acc[i] = __builtin_fmaf(chunk_value<FIN, i>(w), s, acc[i]);
        });
    }
}

// General form for one wave: the BPW blocks kw, kw+1, ... (any slice count; the
// short last block and lanes past the end take guarded paths).
template <int FIN, int FOUT, int G>
__device__ __forceinline__ void reduce_blocks(
    const uint8_t *__restrict__ codes_in, int64_t slice_stride, const float *__restrict__ scales_in,
    int64_t scale_stride, int n_slices, int64_t L, int64_t nb, int64_t kw,
    uint8_t *__restrict__ codes_out, float *__restrict__ scales_out, float *__restrict__ sum_out) {
    using Gm = rgeom<FIN, G>;
    constexpr int CPL = Gm::CPL, U = Gm::U, GL = Gm::GL;
    constexpr int NWI = words_of<FIN, CPL>();
    constexpr int NWO = words_of<FOUT, CPL>();
    constexpr int BIN = fmt_traits<FIN>::bits, BOUT = fmt_traits<FOUT>::bits;
    const int lane = lane_id();
    const int gi = lane / GL, li = lane % GL;
    const int64_t k = kw + gi;
    const bool active = k < nb;
    const int64_t base = k * G;
    const bool full = active && base + G <= L;

    float acc[U][CPL];
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < CPL; i++) acc[u][i] = -0.0f;

    // Slices go in batches of up to B = 8: all loads of a batch are issued
    // before any of it is accumulated (8 x 16 bytes in flight per lane), then
    // the FMAs run in slice order.  Fast form: every block of the wave is full
    // (no guards), and for INT4 input no slice scale is so large that 16*s
    // overflows (the code/16 decode).
    constexpr int B = 8;
    bool fast = full;
    if constexpr (FIN == INT4) {
        for (int j0 = 0; j0 < n_slices; j0 += B) {
            float sc[B];
#pragma unroll
            for (int jj = 0; jj < B; jj++)
                sc[jj] = (active && j0 + jj < n_slices) ? scales_in[(int64_t)(j0 + jj) * scale_stride + k] : 0.0f;
#pragma unroll
            for (int jj = 0; jj < B; jj++) fast = fast && sc[jj] <= kScaleX16Max;
        }
    }
    if (__all(fast)) {
        const uint8_t *src = codes_in + (base + (int64_t)li * CPL) * BIN / 8;
        const float *sp = scales_in + k;
        for (int j0 = 0; j0 < n_slices; j0 += B) {
            uint32_t w[B][U][NWI];
            float sc[B];
#pragma unroll
            for (int jj = 0; jj < B; jj++) {
                if (j0 + jj < n_slices) {
                    const uint8_t *sj = src + (int64_t)(j0 + jj) * slice_stride;
                    sc[jj] = sp[(int64_t)(j0 + jj) * scale_stride];
#pragma unroll
                    for (int u = 0; u < U; u++) load_words_stream<NWI>(sj + (int64_t)u * GL * CPL * BIN / 8, w[jj][u]);
                }
            }
#pragma unroll
            for (int jj = 0; jj < B; jj++) {
                if (j0 + jj < n_slices) {
#pragma unroll
                    for (int u = 0; u < U; u++)
                        accumulate_chunk<FIN, CPL, true>(w[jj][u], sc[jj], sc[jj] * 16.0f, acc[u]);
                }
            }
        }
    } else {
        const int64_t in_bytes = (L * BIN + 7) / 8;
        for (int j0 = 0; j0 < n_slices; j0 += B) {
            uint32_t w[B][U][NWI];
            float sc[B];
#pragma unroll
            for (int jj = 0; jj < B; jj++) {
                if (j0 + jj < n_slices) {
                    const uint8_t *sj = codes_in + (int64_t)(j0 + jj) * slice_stride;
                    sc[jj] = active ? scales_in[(int64_t)(j0 + jj) * scale_stride + k] : 0.0f;
#pragma unroll
                    for (int u = 0; u < U; u++) {
                        const int64_t off = (base + (int64_t)(u * GL + li) * CPL) * BIN / 8;
                        if (full) load_words<NWI>(sj + off, w[jj][u]);
                        else if (active) load_words_tail<NWI>(sj + off, w[jj][u], in_bytes - off);
                        else {
#pragma unroll
                            for (int i = 0; i < NWI; i++) w[jj][u][i] = 0;
                        }
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < B; jj++) {
                if (j0 + jj < n_slices) {
#pragma unroll
                    for (int u = 0; u < U; u++) accumulate_chunk<FIN, CPL, false>(w[jj][u], sc[jj], sc[jj], acc[u]);
                }
            }
        }
    }
    if (!full) {   // elements past the end of the slice do not count
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int i = 0; i < CPL; i++)
                if (!active || base + (int64_t)(u * GL + li) * CPL + i >= L) acc[u][i] = 0.0f;
    }

    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < CPL; i++) m = __builtin_fmaxf(m, __builtin_fabsf(acc[u][i]));
    const float a = __uint_as_float(group_max_u32<GL>(__float_as_uint(m)));
    const BlockScale<FOUT> b = block_scale<FOUT>(a);
    const bool all_fast = __all(b.fast);
    if (!active) return;
    const int64_t out_bytes = (L * BOUT + 7) / 8;

#pragma unroll
    for (int u = 0; u < U; u++) {
        int64_t e0 = base + (int64_t)(u * GL + li) * CPL;
        uint32_t w[NWO];
        if (all_fast) quantize_chunk<FOUT, CPL, true>(acc[u], b, w);
        else quantize_chunk<FOUT, CPL, false>(acc[u], b, w);
        int64_t off = e0 * BOUT / 8;
        if (full) {
            if constexpr (NWO % 4 == 0) store_words_stream<NWO>(codes_out + off, w);
            else store_words<NWO>(codes_out + off, w);
        } else if (e0 < L) {
            store_words_tail<NWO>(codes_out + off, w, out_bytes - off);
        }
        if (sum_out) {
            if (full) {
#pragma unroll
                for (int i = 0; i < CPL; i += 4)
                    *(float4 *)(sum_out + e0 + i) =
                        make_float4(acc[u][i], acc[u][i + 1], acc[u][i + 2], acc[u][i + 3]);
            } else {
#pragma unroll
                for (int i = 0; i < CPL; i++)
                    if (e0 + i < L) sum_out[e0 + i] = acc[u][i];
            }
        }
    }
    if (li == 0) scales_out[k] = b.s;
}

template <int FIN, int FOUT, int G>
__global__ __launch_bounds__(kThreads) void k_reduce(
    const uint8_t *__restrict__ codes_in, int64_t slice_stride, const float *__restrict__ scales_in,
    int64_t scale_stride, int n_slices, int64_t L, int64_t nb, uint8_t *__restrict__ codes_out,
    float *__restrict__ scales_out, float *__restrict__ sum_out) {
    const int64_t wave = wave_id();
    reduce_blocks<FIN, FOUT, G>(codes_in, slice_stride, scales_in, scale_stride, n_slices, L, nb,
                                wave * rgeom<FIN, G>::BPW, codes_out, scales_out, sum_out);
}

// ---- INT4 input, exactly 8 slices, no fp32 sums ----
// A lane owns 16 consecutive elements of a block (8 bytes of INT4 codes per
// slice), a block of G elements is spread over G/16 lanes, and a wave's group
// is the 64*16 = 1024 elements of 1024/G consecutive blocks.  Wave v takes
// groups v, v + W, v + 2W, ...; the slices are two halves, P = slices 0..3
// and Q = slices 4..7, and a wave accumulates P while Q's loads are in flight
// and, when it has a next group, loads that group's P while it accumulates Q.
// The launch gives every group its own wave (W >= number of groups), so each
// wave runs the loop once with all 8 slices' loads issued first, and the
// hardware starts a new wave as soon as one ends: that measured faster than 7
// persistent waves per SIMD walking the groups (3-4 us on 8 slices of 62.5M
// elements, 17% on 8 slices of 5e8).  Used without the optional fp32 sums only.
//
// Why 16 elements per lane: the decode (v_cvt_off_f32_i4) and the fmas, which
// share the scale register, never dual-issue, so every element costs two
// issue slots, and the kernel needs enough resident waves to cover each
// other's memory and dependency waits.  With 16 elements per lane the codes
// of 8 slices and the sums fit in 64 VGPRs: 8 waves per SIMD.  (32 elements
// per lane needs about 100 VGPRs, 4 waves per SIMD, and measured slower; an
// LDS-staged variant, global_load_lds into two 8 KB stages per wave, measured
// slower too: its LDS footprint caps occupancy.)

constexpr int kI4x8Slices = 8;
constexpr int kI4x8CPL = 16;                // elements per lane per slice
constexpr int kI4x8WavesPerSimd = 8;        // register budget: 64 VGPRs

template <int G> struct i4x8geom {
    static constexpr int CPL = kI4x8CPL;
    static constexpr int GL = G / CPL;     // lanes per block (2 .. 64)
    static constexpr int BPW = 64 / GL;    // blocks per group
    static_assert(GL * CPL == G && GL <= 64, "int4 x 8 geometry");
};

template <int FIN, int G> struct i4x8_ok {
    static constexpr bool value = FIN == INT4;
};

typedef unsigned int u32x2v_t __attribute__((ext_vector_type(2)));

template <int FIN, int FOUT, int G>
__global__ __launch_bounds__(kThreads, kI4x8WavesPerSimd) void k_reduce_int4x8(
    const uint8_t *__restrict__ codes_in, int64_t slice_stride, const float *__restrict__ scales_in,
    int64_t scale_stride, int64_t L, int64_t nb, int64_t W, uint8_t *__restrict__ codes_out,
    float *__restrict__ scales_out) {
    using Gm = i4x8geom<G>;
    constexpr int CPL = Gm::CPL, GL = Gm::GL, BPW = Gm::BPW;
    constexpr int NWO = words_of<FOUT, CPL>();
    constexpr int BIN = fmt_traits<FIN>::bits, BOUT = fmt_traits<FOUT>::bits;
    constexpr int64_t GBI = (int64_t)BPW * G * BIN / 8, GBO = (int64_t)BPW * G * BOUT / 8;
    static_assert(i4x8_ok<FIN, G>::value && CPL * BIN == 64, "one 8-byte INT4 chunk per lane");
    const int lane = lane_id();
    const int gi = lane / GL, li = lane % GL;
    // The group index is wave-uniform and lives in scalar registers: every
    // address below is a scalar base (slice, group) plus a constant per-lane
    // offset, so the loop spends no vector instructions on addressing.
    const int lin8 = lane;                                   // lane's 8-byte unit in a group
    const int lout = lane * CPL * BOUT / 8;                  // lane's output bytes in a group
    const int64_t ngroups = (L / G) / BPW;                   // groups of full blocks
    // Wave numbering.  Wave v takes groups v, v + W, v + 2W, ...  A 128-byte
    // line of scales holds 32 blocks: 16 groups.  Work-groups are dealt
    // round-robin to the 8 XCDs, each with its own L2, so in launch order the
    // 16 groups of a line sit on 4 XCDs and the line is fetched 4 times (12 MB,
    // 4% of the reads).  Within each run of 32 work-groups (128 groups, 4 per
    // XCD), work-group b = 8r + x (XCD x) therefore takes the groups
    // 128(r/4) + 16x + 4(r%4) .. +3: each XCD gets whole lines, and the 32
    // work-groups still cover one contiguous window, as in launch order (a
    // renumbering that gave each XCD one long contiguous range measured 2.5 us
    // slower).  Any bijection is correct; work-groups past the last full run of
    // 32 keep their launch-order number.
    int64_t g;
    {
        const int nwg = (int)(W / kWavesPerGroup);
        const int b = (int)__builtin_amdgcn_workgroup_id_x();
        int vb = b;
        if (b < nwg - nwg % 32) {
            const int x = b % 8, r = b / 8;
            vb = 32 * (r / 4) + 4 * x + (r % 4);
        }
        g = (int64_t)vb * kWavesPerGroup +
            __builtin_amdgcn_readfirstlane((int)(__builtin_amdgcn_workitem_id_x() >> 6));
    }

    // half h of group grp: slices 4h .. 4h+3
    auto load_half = [&](int64_t grp, int h, uint32_t (&w)[4][2], float (&sc)[4]) {
        // slice 4h of the group, then one slice stride at a time (scalar adds)
        const uint8_t *cb = codes_in + grp * GBI + 4 * h * slice_stride;
        const float *sb = scales_in + grp * BPW + 4 * h * scale_stride;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            sc[j] = sb[gi];
            const u32x2v_t v = __builtin_nontemporal_load((const u32x2v_t *)cb + lin8);
            w[j][0] = v.x; w[j][1] = v.y;
            cb += slice_stride;
            sb += scale_stride;
        }
    };
    // the code/16 decode needs every scale of the half <= 2^123 (wave-uniform)
    auto scales_ok = [&](const float (&sc)[4]) {
        const uint32_t m = max(max(__float_as_uint(sc[0]), __float_as_uint(sc[1])),
                               max(__float_as_uint(sc[2]), __float_as_uint(sc[3])));
        return __all(m <= __float_as_uint(kScaleX16Max));
    };
    auto absmax = [&](const float (&acc)[CPL]) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; i++) m = __builtin_fmaxf(m, __builtin_fabsf(acc[i]));
        return __uint_as_float(group_max_u32<GL>(__float_as_uint(m)));
    };
    auto finish = [&](int64_t grp, const uint32_t (&wo)[NWO], float s) {
        uint8_t *ob = codes_out + grp * GBO + lout;
        if constexpr (NWO == 2) {
            const u32x2v_t v = {wo[0], wo[1]};
            __builtin_nontemporal_store(v, (u32x2v_t *)ob);
        } else if constexpr (NWO % 4 == 0) {
            store_words_stream<NWO>(ob, wo);
        } else {
            store_words<NWO>(ob, wo);
        }
        if (li == 0) scales_out[grp * BPW + gi] = s;
    };
    // One slice's 16 decoded operands at a time.  Left free, the scheduler
    // decodes a whole half ahead of its multiply-adds, which does not fit the
    // register budget; this empty asm makes the next slice's code words depend
    // on the current sums, so a slice is decoded only after the previous one's
    // multiply-adds.
    auto after_sums = [&](uint32_t (&w)[2], const float (&a)[CPL]) {
        static_assert(CPL == 16, "one statement of 16 sums");
        asm volatile("" : "+v"(w[0]), "+v"(w[1])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]),
                       "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]),
                       "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15]));
    };
    // Any group with exact arithmetic and guards: decode (code, s) with no
    // bound on s, guarded quotients, and the slice end honoured.  A chunk that
    // straddles the end is read as its whole aligned 8 bytes (an aligned 8-byte
    // load stays in the memory page of its first byte, which lies in the slice)
    // and the bytes past the end are cleared in registers.
    auto exact_group = [&](int64_t grp) {
        const int64_t k = grp * BPW + gi;
        const bool active = k < nb;
        const int64_t e0 = k * G + (int64_t)li * CPL;
        const int64_t off = e0 * BIN / 8, valid = (L * BIN + 7) / 8 - off;
        const bool any = active && valid > 0;
        uint32_t keep[2];
#pragma unroll
        for (int d = 0; d < 2; d++) {
            const int64_t v = valid - 4 * d;
            keep[d] = v >= 4 ? 0xffffffffu : v <= 0 ? 0u : (1u << (8 * v)) - 1u;
        }
        float acc[CPL];
#pragma unroll
        for (int i = 0; i < CPL; i++) acc[i] = -0.0f;
#pragma unroll
        for (int j = 0; j < kI4x8Slices; j++) {
            const float sc = active ? scales_in[(int64_t)j * scale_stride + k] : 0.0f;
            uint32_t w[2] = {0u, 0u};
            if (any) load_words<2>(codes_in + (int64_t)j * slice_stride + off, w);
#pragma unroll
            for (int d = 0; d < 2; d++) w[d] &= keep[d];
            accumulate_chunk<FIN, CPL, false>(w, sc, sc, acc);
        }
#pragma unroll
        for (int i = 0; i < CPL; i++)
            if (e0 + i >= L) acc[i] = 0.0f;               // past the end: not part of the block
        const BlockScale<FOUT> bs = block_scale<FOUT>(absmax(acc));
        uint32_t wo[NWO];
        quantize_chunk<FOUT, CPL, false>(acc, bs, wo);
        if (!active) return;
        const int64_t o = e0 * BOUT / 8;
        if (e0 + CPL <= L) store_words<NWO>(codes_out + o, wo);
        else if (e0 < L) store_words_tail<NWO>(codes_out + o, wo, (L * BOUT + 7) / 8 - o);
        if (li == 0) scales_out[k] = bs.s;
    };

    // The inner loop assumes the common case: every scale of the group <= 2^123
    // and an output scale in the fast-quotient range.  A group that breaks
    // either leaves it as xg and is redone from memory with the exact form;
    // keeping the rare forms out of the loop keeps its register count down.
    // The short last group (blocks past the full groups), if any, is the grid's
    // last wave's job.
    uint32_t P[4][2], Q[4][2];
    float sp[4], sq[4];
    int64_t xg = (ngroups * BPW < nb && g == W - 1) ? ngroups : -1;
    while (true) {
        if (xg >= 0) exact_group(xg);                    // xg and g are wave-uniform
        if (g >= ngroups) return;
        xg = -1;
        load_half(g, 0, P, sp);
        while (true) {
            load_half(g, 1, Q, sq);
            const int64_t g1 = g + W;
            if (!scales_ok(sp)) {
                xg = g;
                g = g1;
                break;
            }
            float acc[CPL];
#pragma unroll
            for (int i = 0; i < CPL; i++) acc[i] = -0.0f;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                accumulate_chunk<FIN, CPL, true>(P[j], sp[j], sp[j] * 16.0f, acc);
                if (j < 3) after_sums(P[j + 1], acc);
            }
            // The first half's sums are needed here (the asm takes them), so
            // the compiler cannot sink those multiply-adds past the next scale
            // check with their decoded operands live across it.
            after_sums(Q[0], acc);
            const bool more = g1 < ngroups;
            if (more) load_half(g1, 0, P, sp);
            if (!scales_ok(sq)) {
                xg = g;
                g = g1;
                break;
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                accumulate_chunk<FIN, CPL, true>(Q[j], sq[j], sq[j] * 16.0f, acc);
                if (j < 3) after_sums(Q[j + 1], acc);
            }
            const BlockScale<FOUT> bs = block_scale<FOUT>(absmax(acc));
            if (!__all(bs.fast)) {
                xg = g;
                g = g1;
                break;
            }
            uint32_t wo[NWO];
            quantize_chunk_fast<FOUT, CPL>(acc, bs, wo);
            finish(g, wo, bs.s);
            if (!more) return;
            g = g1;
        }
    }
}

// ---- FP8 accumulate kernel ----
// A lane owns chunks of 16 elements: 16 E4M3 bytes (one 16-byte load) and 16
// gradient values (two 16-byte loads of bf16/fp16, four of fp32).

template <int G> struct ageom {
    static constexpr int CPL = 16;
    static constexpr int C = G / CPL;
    static constexpr int U = C > 16 ? C / 16 : 1;
    static constexpr int GL = C / U;
    static constexpr int BPW = 64 / GL;
    static_assert(GL * U * CPL == G && GL <= 16, "accumulate geometry");
};

template <int GT>
__device__ __forceinline__ void load_grad16(const void *g, int64_t e0, bool full, int64_t n,
                                            float (&out)[16]) {
    if (full) {
        if constexpr (GT == F32) {
            const float *p = (const float *)g + e0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                uint4 v = load_stream16(p + 4 * i);
                out[4 * i] = __uint_as_float(v.x); out[4 * i + 1] = __uint_as_float(v.y);
                out[4 * i + 2] = __uint_as_float(v.z); out[4 * i + 3] = __uint_as_float(v.w);
            }
        } else {
            const uint16_t *p = (const uint16_t *)g + e0;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                uint4 v = load_stream16(p + 8 * i);
                uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    out[8 * i + 2 * t] = widen_lo<GT>(d[t]);
                    out[8 * i + 2 * t + 1] = widen_hi<GT>(d[t]);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            bool ok = e0 + i < n;
            if constexpr (GT == F32) {
                out[i] = ok ? ((const float *)g)[e0 + i] : 0.0f;
            } else {
                uint32_t h = ok ? ((const uint16_t *)g)[e0 + i] : 0u;
                out[i] = widen_lo<GT>(h);
            }
        }
    }
}

template <int GT, int G>
__global__ __launch_bounds__(kThreads) void k_accum(uint8_t *__restrict__ st_codes,
                                                    float *__restrict__ st_scales,
                                                    const void *__restrict__ grad, int64_t n,
                                                    int64_t nb) {
    using Gm = ageom<G>;
    constexpr int U = Gm::U, GL = Gm::GL, BPW = Gm::BPW;
    const int lane = lane_id();
    const int gi = lane / GL, li = lane % GL;
    const int64_t wave = wave_id();
    const int64_t k = wave * BPW + gi;
    const bool active = k < nb;
    const int64_t base = k * G;
    const bool full = active && base + G <= n;

    float t[U][16];
    if (active) {
        const float s_old = st_scales[k];
#pragma unroll
        for (int u = 0; u < U; u++) {
            int64_t e0 = base + (int64_t)(u * GL + li) * 16;
            uint32_t w[4];
            if (full) load_words_stream<4>(st_codes + e0, w);
            else load_words_tail<4>(st_codes + e0, w, n - e0);
            float g[16];
            load_grad16<GT>(grad, e0, full, n, g);
            float d[16];
            static_for<16>([&](auto I) {
                constexpr int i = decltype(I)::value;
                d[i] = chunk_value<E4M3, i>(w) * s_old;
            });
#pragma unroll
            for (int i = 0; i < 16; i += 2) round_bf16x2(d[i], d[i + 1]);
#pragma unroll
            for (int i = 0; i < 16; i++) t[u][i] = d[i] + g[i];
#pragma unroll
            for (int i = 0; i < 16; i += 2) round_bf16x2(t[u][i], t[u][i + 1]);
            if (!full) {
#pragma unroll
                for (int i = 0; i < 16; i++)
                    if (e0 + i >= n) t[u][i] = 0.0f;
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int i = 0; i < 16; i++) t[u][i] = 0.0f;
    }

    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < 16; i++) m = __builtin_fmaxf(m, __builtin_fabsf(t[u][i]));
    const float a = __uint_as_float(group_max_u32<GL>(__float_as_uint(m)));
    const BlockScale<E4M3> b = block_scale<E4M3>(a);
    const bool all_fast = __all(b.fast);
    if (!active) return;

#pragma unroll
    for (int u = 0; u < U; u++) {
        int64_t e0 = base + (int64_t)(u * GL + li) * 16;
        uint32_t w[4];
        if (all_fast) quantize_chunk<E4M3, 16, true>(t[u], b, w);
        else quantize_chunk<E4M3, 16, false>(t[u], b, w);
        if (full) store_words_stream<4>(st_codes + e0, w);
        else if (e0 < n) store_words_tail<4>(st_codes + e0, w, n - e0);
    }
    if (li == 0) st_scales[k] = b.s;
}

// ---- dispatch ----

#define QCP_FOR_G(G_, CALL)                                  \
    switch (G_) {                                            \
    case 32: { constexpr int GG = 32; return CALL; }         \
    case 64: { constexpr int GG = 64; return CALL; }         \
    case 128: { constexpr int GG = 128; return CALL; }       \
    case 256: { constexpr int GG = 256; return CALL; }       \
    case 512: { constexpr int GG = 512; return CALL; }       \
    case 1024: { constexpr int GG = 1024; return CALL; }     \
    default: return hipErrorInvalidValue;                    \
    }


template <int FIN, int FOUT, int G>
static hipError_t run_reduce(const uint8_t *ci, int64_t ss, const float *si, int64_t sst, int N,
                             int64_t L, uint8_t *co, float *so, float *sum, hipStream_t st) {
    using Gm = rgeom<FIN, G>;
    const int64_t nb = (L + G - 1) / G;
    const int64_t groups = (nb + Gm::BPW - 1) / Gm::BPW;
    if constexpr (i4x8_ok<FIN, G>::value) {
        if (N == kI4x8Slices && sum == nullptr) {
            const int64_t waves = (nb + i4x8geom<G>::BPW - 1) / i4x8geom<G>::BPW;   // one per group
            const unsigned grid = grid_for_waves(waves);
            hipLaunchKernelGGL((k_reduce_int4x8<FIN, FOUT, G>), dim3(grid), dim3(kThreads), 0, st, ci,
                               ss, si, sst, L, nb, (int64_t)grid * kWavesPerGroup, co, so);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_reduce<FIN, FOUT, G>), dim3(grid_for_waves(groups)), dim3(kThreads), 0,
                       st, ci, ss, si, sst, N, L, nb, co, so, sum);
    return hipGetLastError();
}

template <int FIN, int FOUT>
static hipError_t red_g(const uint8_t *ci, int64_t ss, const float *si, int64_t sst, int N,
                        int64_t L, int G, uint8_t *co, float *so, float *sum, hipStream_t st) {
    QCP_FOR_G(G, (run_reduce<FIN, FOUT, GG>(ci, ss, si, sst, N, L, co, so, sum, st)))
}

template <int FIN>
static hipError_t red_o(const uint8_t *ci, int64_t ss, const float *si, int64_t sst, int N,
                        int64_t L, int G, int fout, uint8_t *co, float *so, float *sum,
                        hipStream_t st) {
    switch (fout) {
    case INT2: return red_g<FIN, INT2>(ci, ss, si, sst, N, L, G, co, so, sum, st);
    case INT4: return red_g<FIN, INT4>(ci, ss, si, sst, N, L, G, co, so, sum, st);
    case INT6: return red_g<FIN, INT6>(ci, ss, si, sst, N, L, G, co, so, sum, st);
    case INT8: return red_g<FIN, INT8>(ci, ss, si, sst, N, L, G, co, so, sum, st);
    case E4M3: return red_g<FIN, E4M3>(ci, ss, si, sst, N, L, G, co, so, sum, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce(const uint8_t *codes_in, int64_t slice_stride, const float *scales_in,
                         int64_t scale_stride, int n_slices, int64_t L, int G, int fmt_in,
                         int fmt_out, uint8_t *codes_out, float *scales_out, float *sum_out,
                         hipStream_t st) {
    switch (fmt_in) {
    case INT2: return red_o<INT2>(codes_in, slice_stride, scales_in, scale_stride, n_slices, L, G, fmt_out, codes_out, scales_out, sum_out, st);
    case INT4: return red_o<INT4>(codes_in, slice_stride, scales_in, scale_stride, n_slices, L, G, fmt_out, codes_out, scales_out, sum_out, st);
    case INT6: return red_o<INT6>(codes_in, slice_stride, scales_in, scale_stride, n_slices, L, G, fmt_out, codes_out, scales_out, sum_out, st);
    case INT8: return red_o<INT8>(codes_in, slice_stride, scales_in, scale_stride, n_slices, L, G, fmt_out, codes_out, scales_out, sum_out, st);
    case E4M3: return red_o<E4M3>(codes_in, slice_stride, scales_in, scale_stride, n_slices, L, G, fmt_out, codes_out, scales_out, sum_out, st);
    default: return hipErrorInvalidValue;
    }
}

template <int GT, int G>
static hipError_t run_accum(uint8_t *c, float *s, const void *g, int64_t n, hipStream_t st) {
    int64_t nb = (n + G - 1) / G;
    int64_t waves = (nb + ageom<G>::BPW - 1) / ageom<G>::BPW;
    hipLaunchKernelGGL((k_accum<GT, G>), dim3(grid_for_waves(waves)), dim3(kThreads), 0, st, c, s,
                       g, n, nb);
    return hipGetLastError();
}

template <int GT>
static hipError_t acc_g(uint8_t *c, float *s, const void *g, int64_t n, int G, hipStream_t st) {
    QCP_FOR_G(G, (run_accum<GT, GG>(c, s, g, n, st)))
}

hipError_t launch_accum(uint8_t *state_codes, float *state_scales, const void *grad, int gt,
                        int64_t n, int G, hipStream_t st) {
    switch (gt) {
    case F16: return acc_g<F16>(state_codes, state_scales, grad, n, G, st);
    case BF16: return acc_g<BF16>(state_codes, state_scales, grad, n, G, st);
    case F32: return acc_g<F32>(state_codes, state_scales, grad, n, G, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qcp
