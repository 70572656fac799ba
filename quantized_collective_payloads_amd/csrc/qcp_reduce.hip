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

// unrolled loops over compile-time indices
template <int N, class F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// quantize CPL values of a chunk into words of format FOUT
template <int FOUT, int CPL, bool ALL_FAST>
__device__ __forceinline__ void quantize_chunk(const float (&v)[CPL], float s, float r, bool fast,
                                               uint32_t (&w)[words_of<FOUT, CPL>()]) {
    constexpr int NW = words_of<FOUT, CPL>();
#pragma unroll
    for (int i = 0; i < NW; i++) w[i] = 0;
    if constexpr (FOUT == E4M3) {
#pragma unroll
        for (int i = 0; i < CPL; i += 4) {
            float q[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                float x = v[i + t];
                float qq = ALL_FAST ? quot_fast(x, s, r) : (fast ? quot_fast(x, s, r) : quot_ieee(x, s));
                q[t] = __builtin_copysignf(qq, x);
            }
            w[i / 4] = e4m3_pack4(q[0], q[1], q[2], q[3]);
        }
    } else {
        static_for<CPL>([&](auto I) {
            constexpr int i = decltype(I)::value;
            float x = v[i];
            float q = ALL_FAST ? quot_fast(x, s, r) : (fast ? quot_fast(x, s, r) : quot_ieee(x, s));
            uint32_t f = (uint32_t)int_code<FOUT>(q) & ((1u << fmt_traits<FOUT>::bits) - 1u);
            chunk_put<FOUT, i>(w, f);
        });
    }
    if (s == 0.0f) {
#pragma unroll
        for (int i = 0; i < NW; i++) w[i] = 0;
    }
}

// ---- the reduce kernel ----

template <int FIN, int FOUT, int G>
__global__ __launch_bounds__(kThreads) void k_reduce(
    const uint8_t *__restrict__ codes_in, int64_t slice_stride, const float *__restrict__ scales_in,
    int64_t scale_stride, int n_slices, int64_t L, int64_t nb, uint8_t *__restrict__ codes_out,
    float *__restrict__ scales_out, float *__restrict__ sum_out) {
    using Gm = rgeom<FIN, G>;
    constexpr int CPL = Gm::CPL, U = Gm::U, GL = Gm::GL, BPW = Gm::BPW;
    constexpr int NWI = words_of<FIN, CPL>();
    constexpr int NWO = words_of<FOUT, CPL>();
    constexpr int BIN = fmt_traits<FIN>::bits, BOUT = fmt_traits<FOUT>::bits;
    constexpr float QMAX = fmt_traits<FOUT>::qmax;
    const int lane = threadIdx.x & 63;
    const int gi = lane / GL, li = lane % GL;
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
    const int64_t k = wave * BPW + gi;
    const bool active = k < nb;
    const int64_t base = k * G;
    const bool full = active && base + G <= L;
    const int64_t in_bytes = (L * BIN + 7) / 8;

    float acc[U][CPL];
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < CPL; i++) acc[u][i] = -0.0f;

    if (active) {
        for (int j = 0; j < n_slices; j++) {
            const uint8_t *src = codes_in + (int64_t)j * slice_stride;
            const float s = scales_in[(int64_t)j * scale_stride + k];
            uint32_t w[U][NWI];
#pragma unroll
            for (int u = 0; u < U; u++) {
                int64_t e0 = base + (int64_t)(u * GL + li) * CPL;
                int64_t off = e0 * BIN / 8;
                if (full) load_words<NWI>(src + off, w[u]);
                else load_words_tail<NWI>(src + off, w[u], in_bytes - off);
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                static_for<CPL>([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    acc[u][i] = __builtin_fmaf(chunk_value<FIN, i>(w[u]), s, acc[u][i]);
                });
            }
        }
        if (!full) {   // elements past the end of the slice do not count
#pragma unroll
            for (int u = 0; u < U; u++)
#pragma unroll
                for (int i = 0; i < CPL; i++)
                    if (base + (int64_t)(u * GL + li) * CPL + i >= L) acc[u][i] = 0.0f;
        }
    }

    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < CPL; i++) m = max(m, __float_as_uint(acc[u][i]) & 0x7fffffffu);
    const float a = __uint_as_float(group_max_u32<GL>(m));
    const float s = a / QMAX;
    const bool fast = scale_is_fast(s);
    const float r = (s == 0.0f || !fast) ? 0.0f : 1.0f / s;
    const bool all_fast = __all(fast);
    if (!active) return;
    const int64_t out_bytes = (L * BOUT + 7) / 8;

#pragma unroll
    for (int u = 0; u < U; u++) {
        int64_t e0 = base + (int64_t)(u * GL + li) * CPL;
        uint32_t w[NWO];
        if (all_fast) quantize_chunk<FOUT, CPL, true>(acc[u], s, r, true, w);
        else quantize_chunk<FOUT, CPL, false>(acc[u], s, r, fast, w);
        int64_t off = e0 * BOUT / 8;
        if (full) {
            store_words<NWO>(codes_out + off, w);
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
    if (li == 0) scales_out[k] = s;
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
            const float4 *p = (const float4 *)((const float *)g + e0);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float4 v = p[i];
                out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
            }
        } else {
            const uint4 *p = (const uint4 *)((const uint16_t *)g + e0);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                uint4 v = p[i];
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
    const int lane = threadIdx.x & 63;
    const int gi = lane / GL, li = lane % GL;
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
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
            if (full) load_words<4>(st_codes + e0, w);
            else load_words_tail<4>(st_codes + e0, w, n - e0);
            float g[16];
            load_grad16<GT>(grad, e0, full, n, g);
            static_for<16>([&](auto I) {
                constexpr int i = decltype(I)::value;
                float d = round_bf16(chunk_value<E4M3, i>(w) * s_old);
                t[u][i] = round_bf16(d + g[i]);
            });
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

    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < 16; i++) m = max(m, __float_as_uint(t[u][i]) & 0x7fffffffu);
    const float a = __uint_as_float(group_max_u32<GL>(m));
    const float s = a / 448.0f;
    const bool fast = scale_is_fast(s);
    const float r = (s == 0.0f || !fast) ? 0.0f : 1.0f / s;
    const bool all_fast = __all(fast);
    if (!active) return;

#pragma unroll
    for (int u = 0; u < U; u++) {
        int64_t e0 = base + (int64_t)(u * GL + li) * 16;
        uint32_t w[4];
        if (all_fast) quantize_chunk<E4M3, 16, true>(t[u], s, r, true, w);
        else quantize_chunk<E4M3, 16, false>(t[u], s, r, fast, w);
        if (full) store_words<4>(st_codes + e0, w);
        else if (e0 < n) store_words_tail<4>(st_codes + e0, w, n - e0);
    }
    if (li == 0) st_scales[k] = s;
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
    int64_t nb = (L + G - 1) / G;
    int64_t waves = (nb + rgeom<FIN, G>::BPW - 1) / rgeom<FIN, G>::BPW;
    hipLaunchKernelGGL((k_reduce<FIN, FOUT, G>), dim3(grid_for_waves(waves)), dim3(kThreads), 0,
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
