// qcp_codec.hip -- blockwise quantize+pack and unpack+dequantize kernels.
//
// Method: [ZPP] "Quantized LLM Training at Scale with ZeRO++", section
// "Blockwise weight quantization cuts forward-gather traffic in half" (qwZ:
// per-block 8-bit codes for the forward all-gather, 16-bit values after it);
// [AQV] "Aquavit ..." review, Section 5.1 / Table 1 / Eq. 6 (b in {2,4,6,8},
// one 32-bit scale per block of G so bpw = b + 32/G) and Section 5.2 (fused
// sub-byte packing).  [AGOQ] Section 2.B for the E4M3 variant.
//
// Geometry.  A "vector" is 8 consecutive elements: 16 bytes of fp16/bf16
// input (one global_load_dwordx4), 32 bytes of fp32.  A block of G elements
// has G/8 vectors, spread over GL lanes with U vectors per lane:
//     G                        32  64  128  256  512  1024
//     GL (INT2/INT6 encoders)   4   8    8    8   16    32
//     U                         1   1    2    4    4     4
//     GL (INT8/E4M3 encoders)   4   8   16   16   16    32
//     U                         1   1    1    2    4     4
//     GL (INT4 encoders, all    4   8   16   32   32    32
//         decoders)
//     U                         1   1    1    1    2     4
// Vector u of lane li of a block is vector u*GL + li, so each load instruction
// reads GL*16 contiguous bytes per block (>= one 64/128-byte line) and a wave
// covers 64/GL whole blocks.  The block absmax is a per-lane max followed by a
// DPP/ds_swizzle max over the GL lanes; no LDS, no barrier, no atomics.  The
// last block may be short: its lanes take a guarded element-wise path.
#include "qcp_device.h"
#include "qcp_launch.h"

namespace qcp {

// MINGL: the fewest lanes a block is spread over when it has that many
// vectors (fewer vectors per lane, more lanes per block).
template <int G, int MINGL = 8> struct geom {
    static constexpr int VPB = G / 8;
    static constexpr int U = (VPB / MINGL) < 1 ? 1 : ((VPB / MINGL) > 4 ? 4 : VPB / MINGL);
    static constexpr int GL = VPB / U;
    static constexpr int BPW = 64 / GL;
    // Groups of BPW blocks per wave.  With one vector per lane a group is only
    // 1 KB of 16-bit data per wave, too little in flight to cover the memory
    // latency; such a wave issues the loads of four groups before it converts
    // any (encoders and decoders alike).
    static constexpr int PW = U == 1 ? 4 : 1;
    // A decoder's wave reads little (its codes) and writes a lot, and cannot
    // start writing before its codes arrive, so each wave's life includes one
    // full read latency; when the codes come from HBM rather than from the
    // memory-side cache (e.g. after an unrelated 1 GiB read) that latency
    // doubles.  Decoders therefore take two groups per wave also where a lane
    // holds two or more vectors, both groups' loads issued first: from a cold
    // cache 2-8 us faster per kernel, the same within noise in the step (four
    // groups: between the two).
    static constexpr int PWD = U == 1 ? 4 : 2;
    static_assert(GL * U * 8 == G && GL <= 64, "block geometry");
};

// Encoder geometry.  An INT4 lane stores 4 bytes of codes per vector, so with
// 8 lanes per block each store instruction writes 32-byte pieces, eight per
// wave, each in its own cache line; spread over 32 lanes, a block's store
// instruction writes one whole 128-byte line.  INT8/E4M3 lanes store 8 bytes
// per vector and take 16 lanes per block for the same reason.  Measured:
// INT4 G=256 packing of 234.9M bf16 values 2-5 us faster, the INT4 G=512 qgZ
// sender over a 5e8-element bucket ~10 us, INT8 G=256 quantization of 218M
// values ~3 us; 32 lanes for INT8 were no faster than 8.  INT2 and INT6 keep
// 8 lanes per block (16 for INT6 measured slower).
template <int FMT, int G>
using egeom = geom<G, FMT == INT4 ? 32 : ((FMT == INT8 || FMT == E4M3) ? 16 : 8)>;

// Decoder geometry: at least 32 lanes per block, so that each 16-byte output
// store instruction writes 512 contiguous bytes of a block.  Against 8 lanes
// per block: the INT8 G=256 dequantize of 218M values ~1 us faster in the
// step and ~2.5 us from a cold cache, the INT6 G=128 unpack of 234.9M values
// ~3.5 us cold; the other decoders unchanged (64 lanes at G=1024 were slower).
template <int G> using dgeom = geom<G, 32>;

// waves for nb blocks at BPW blocks per group and PW groups per wave
template <class Gm, int PW> inline int64_t codec_waves(int64_t nb) {
    const int64_t groups = (nb + Gm::BPW - 1) / Gm::BPW;
    return (groups + PW - 1) / PW;
}

// ---- packed-code I/O for one vector (element offset e0, a multiple of 8) ----

// A8: the codes of a vector are 8-byte aligned (separate code arrays); in the
// interleaved record layout they are only 4-byte aligned and go as dwords.
// Code accesses are 2-8 bytes per lane, several per cache line across the
// wave's instructions: they go through the caches normally (a streaming hint
// here measured slower -- lines are fetched again between the instructions).
template <class T> __device__ __forceinline__ void st_once(void *p, T v) { *(T *)p = v; }
template <class T> __device__ __forceinline__ T ld_once(const void *p) { return *(const T *)p; }

template <int FMT, bool A8 = true>
__device__ __forceinline__ void store_vec_codes(uint8_t *codes, int64_t e0, Packed8 p) {
    if constexpr ((FMT == INT8 || FMT == E4M3) && !A8) {
        st_once<uint32_t>(codes + e0, p.lo);
        st_once<uint32_t>(codes + e0 + 4, p.hi);
    } else if constexpr (FMT == INT8 || FMT == E4M3) {
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        u32x2_t w = {p.lo, p.hi};
        st_once<u32x2_t>(codes + e0, w);
    } else if constexpr (FMT == INT4) {
        st_once<uint32_t>(codes + e0 / 2, p.lo);
    } else if constexpr (FMT == INT2) {
        st_once<uint16_t>(codes + e0 / 4, (uint16_t)p.lo);
    } else {  // INT6: 6 bytes at 6*(e0/8); 4-byte aligned when e0/8 is even
        int64_t v = e0 / 8, off = 6 * v;
        if ((v & 1) == 0) {
            st_once<uint32_t>(codes + off, p.lo);
            st_once<uint16_t>(codes + off + 4, (uint16_t)p.hi);
        } else {
            st_once<uint16_t>(codes + off, (uint16_t)p.lo);
            st_once<uint32_t>(codes + off + 2, (p.lo >> 16) | (p.hi << 16));
        }
    }
}

template <int FMT, bool A8 = true>
__device__ __forceinline__ Packed8 load_vec_codes(const uint8_t *codes, int64_t e0) {
    Packed8 p;
    if constexpr ((FMT == INT8 || FMT == E4M3) && !A8) {
        p.lo = ld_once<uint32_t>(codes + e0);
        p.hi = ld_once<uint32_t>(codes + e0 + 4);
    } else if constexpr (FMT == INT8 || FMT == E4M3) {
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        u32x2_t w = ld_once<u32x2_t>(codes + e0);
        p.lo = w.x;
        p.hi = w.y;
    } else if constexpr (FMT == INT4) {
        p.lo = ld_once<uint32_t>(codes + e0 / 2);
        p.hi = 0;
    } else if constexpr (FMT == INT2) {
        p.lo = ld_once<uint16_t>(codes + e0 / 4);
        p.hi = 0;
    } else {
        int64_t v = e0 / 8, off = 6 * v;
        if ((v & 1) == 0) {
            p.lo = ld_once<uint32_t>(codes + off);
            p.hi = ld_once<uint16_t>(codes + off + 4);
        } else {
            uint32_t a = ld_once<uint16_t>(codes + off);
            uint32_t b = ld_once<uint32_t>(codes + off + 2);
            p.lo = a | (b << 16);
            p.hi = b >> 16;
        }
    }
    return p;
}

// byte offset of a vector's codes and their count
template <int FMT> __device__ __forceinline__ int64_t vec_code_offset(int64_t e0) {
    return e0 / 8 * vec_bytes<FMT>();
}

// guarded byte-wise versions for the short last block
template <int FMT>
__device__ __forceinline__ void store_vec_codes_tail(uint8_t *codes, int64_t e0, Packed8 p,
                                                     int64_t total_bytes) {
    int64_t off = vec_code_offset<FMT>(e0);
#pragma unroll
    for (int j = 0; j < vec_bytes<FMT>(); j++) {
        uint32_t w = j < 4 ? p.lo : p.hi;
        if (off + j < total_bytes) codes[off + j] = (uint8_t)(w >> (8 * (j & 3)));
    }
}

template <int FMT>
__device__ __forceinline__ Packed8 load_vec_codes_tail(const uint8_t *codes, int64_t e0,
                                                       int64_t total_bytes) {
    Packed8 p{0, 0};
    int64_t off = vec_code_offset<FMT>(e0);
#pragma unroll
    for (int j = 0; j < vec_bytes<FMT>(); j++) {
        uint32_t byte = off + j < total_bytes ? codes[off + j] : 0u;
        if (j < 4) p.lo |= byte << (8 * j); else p.hi |= byte << (8 * (j - 4));
    }
    return p;
}

// ---- INT6 vectors are 6 bytes: adjacent lanes (vectors 2m, 2m+1) form one
// 12-byte, 4-byte-aligned unit that the even lane stores / both lanes load ----

// even lane: its own 6 bytes + the odd neighbour's (via DPP quad_perm [1,1,3,3])
__device__ __forceinline__ void int6_pair_words(Packed8 p, uint32_t (&w)[3]) {
    uint32_t nlo = dpp_u32<0xF5>(p.lo), nhi = dpp_u32<0xF5>(p.hi);
    w[0] = p.lo;
    w[1] = (p.hi & 0xffffu) | (nlo << 16);
    w[2] = (nlo >> 16) | (nhi << 16);
}

// both lanes of a pair load its 12 bytes and take their half
__device__ __forceinline__ Packed8 int6_pair_load(const uint8_t *codes, int64_t e0) {
    int64_t v = e0 / 8;
    bool odd = v & 1;
    const uint8_t *w = codes + 6 * (v & ~(int64_t)1);
    uint32_t w0 = ld_once<uint32_t>(w), w1 = ld_once<uint32_t>(w + 4), w2 = ld_once<uint32_t>(w + 8);
    Packed8 p;
    p.lo = odd ? __builtin_amdgcn_alignbit(w2, w1, 16) : w0;
    p.hi = odd ? (w2 >> 16) : (w1 & 0xffffu);
    return p;
}

// ---- payload layouts: where block k's codes and scale live ----

// Codes and scales in two arrays: block k's codes at codes + k*G*b/8 (the
// stream of the whole tensor), its scale at scales[k].
template <int FMT, int G> struct SplitLayout {
    uint8_t *codes;
    float *scales;
    static constexpr bool kA8 = true;
    __device__ uint8_t *block(int64_t k) const { return codes + k * (G * fmt_traits<FMT>::bits / 8); }
    __device__ float *scale(int64_t k) const { return scales + k; }
};

// Metadata interleaving ([AQV] Section 5.2): one record per block, the fp32
// scale then the block's codes, records back to back (4 + G*b/8 bytes each,
// a multiple of 4, so every record and its codes are 4-byte aligned).
template <int FMT, int G> struct RecordLayout {
    uint8_t *records;
    static constexpr bool kA8 = false;
    static constexpr int64_t kRecord = 4 + G * fmt_traits<FMT>::bits / 8;
    __device__ uint8_t *block(int64_t k) const { return records + k * kRecord + 4; }
    __device__ float *scale(int64_t k) const { return (float *)(records + k * kRecord); }
};

// ---- encode kernels ----

// Where element e of the tensor being quantized lives in the input: the
// identity for a plain quantize, the qgZ tensor-slice reordering for the fused
// sender.  For both, the 8 elements of a vector are contiguous in the input.
struct LinearSrc {
    __device__ int64_t operator()(int64_t e) const { return e; }
};

// Slice j of the reordered bucket is chunks b*N + j (b = 0..K-1, C elements
// each) in node order, so its element e is element (e mod C) of chunk
// (e / C)*N + j.  e / C comes from a double-precision estimate and one exact
// integer correction (the estimate is off by at most one).  C is a multiple
// of 8, so a vector never straddles two chunks.
struct ReorderSrc {
    int64_t C, N, j;
    double inv_c;
    __device__ int64_t operator()(int64_t e) const {
        int64_t b = (int64_t)((double)e * inv_c);
        int64_t r = e - b * C;
        if (r < 0) { b--; r += C; }
        else if (r >= C) { b++; r -= C; }
        return (b * N + j) * C + r;
    }
};

// the U vectors of a lane in block k (base = k*G) as floats: 16-byte streaming
// loads when the block is full, element by element (zeros past n) otherwise
template <int XT, class Gm, class Src>
__device__ __forceinline__ void load_block_vectors(const void *__restrict__ xv, int64_t n,
                                                   int64_t base, int li, bool active, bool full,
                                                   Src src, float (&xf)[Gm::U][8]) {
    constexpr int U = Gm::U, GL = Gm::GL;
    constexpr int DW = dtype_traits<XT>::bytes * 2;       // dwords per vector: 4 (16-bit) or 8
    if (full) {
        const uint32_t *x = (const uint32_t *)xv;
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t e0 = src(base + (int64_t)(u * GL + li) * 8);
            uint32_t raw[DW];
#pragma unroll
            for (int d = 0; d < DW; d += 4) {
                uint4 w = load_stream16(x + e0 * DW / 8 + d);
                raw[d] = w.x; raw[d + 1] = w.y; raw[d + 2] = w.z; raw[d + 3] = w.w;
            }
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if constexpr (XT == F32) xf[u][i] = __uint_as_float(raw[i]);
                else xf[u][i] = (i & 1) ? widen_hi<XT>(raw[i / 2]) : widen_lo<XT>(raw[i / 2]);
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; u++) {
            int64_t e0 = base + (int64_t)(u * GL + li) * 8;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                int64_t e = e0 + i;
                bool ok = active && e < n;
                if constexpr (XT == F32) {
                    xf[u][i] = ok ? ((const float *)xv)[src(e)] : 0.0f;
                } else {
                    uint32_t h = ok ? ((const uint16_t *)xv)[src(e)] : 0u;
                    xf[u][i] = widen_lo<XT>(h);
                }
            }
        }
    }
}

// block absmax, scale and codes of block k from the lane's loaded vectors
template <int FMT, int G, class Gm, class Out>
__device__ __forceinline__ void encode_loaded(int64_t n, int64_t k, int li, bool active, bool full,
                                              Out out, const float (&xf)[Gm::U][8]) {
    constexpr int U = Gm::U, GL = Gm::GL;
    const int64_t base = k * G;
    // block absmax: per-lane max of |x|, then across the block's GL lanes
    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < 8; i++) m = __builtin_fmaxf(m, __builtin_fabsf(xf[u][i]));
    const float a = __uint_as_float(group_max_u32<GL>(__float_as_uint(m)));
    const BlockScale<FMT> b = block_scale<FMT>(a);
    const bool all_fast = __all(b.fast);
    // this block's code bytes (fewer in the short last block); vector offsets
    // below are relative to the block's first element
    const int64_t block_bytes = ((n - base < G ? n - base : G) * fmt_traits<FMT>::bits + 7) / 8;
    uint8_t *const codes = out.block(k);

#pragma unroll
    for (int u = 0; u < U; u++) {
        Packed8 p = all_fast ? quantize8<FMT, true>(xf[u], b) : quantize8<FMT, false>(xf[u], b);
        const int64_t el = (int64_t)(u * GL + li) * 8;
        if constexpr (FMT == INT6) {
            uint32_t w[3];
            int6_pair_words(p, w);                   // all lanes take part in the DPP
            if (full) {
                if ((li & 1) == 0) {
                    uint8_t *o = codes + 6 * (el / 8);
                    st_once<uint32_t>(o, w[0]);
                    st_once<uint32_t>(o + 4, w[1]);
                    st_once<uint32_t>(o + 8, w[2]);
                }
            } else if (active && base + el < n) {
                store_vec_codes_tail<FMT>(codes, el, p, block_bytes);
            }
        } else {
            if (full) store_vec_codes<FMT, Out::kA8>(codes, el, p);
            else if (active && base + el < n) store_vec_codes_tail<FMT>(codes, el, p, block_bytes);
        }
    }
    if (active && li == 0) *out.scale(k) = b.s;
}

// Wave `wave` encodes groups PW*wave ... PW*wave + PW-1 of BPW blocks each.
// When they are all full (wave-uniform), every load is issued before any block
// is quantized; otherwise (the tensor's last groups) one group at a time.
template <int XT, int FMT, int G, class Src, class Out>
__device__ __forceinline__ void encode_blocks(const void *__restrict__ xv, int64_t n, int64_t nb,
                                              int64_t wave, Out out, Src src) {
    using Gm = egeom<FMT, G>;
    constexpr int U = Gm::U, GL = Gm::GL, BPW = Gm::BPW, PW = Gm::PW;
    const int lane = lane_id();
    const int gi = lane / GL, li = lane % GL;
    const int64_t g0 = wave * PW;
    if constexpr (PW > 1) {
        if ((g0 + PW) * BPW * G <= n) {
            float xf[PW][U][8];
#pragma unroll
            for (int p = 0; p < PW; p++)
                load_block_vectors<XT, Gm>(xv, n, ((g0 + p) * BPW + gi) * G, li, true, true, src, xf[p]);
#pragma unroll
            for (int p = 0; p < PW; p++)
                encode_loaded<FMT, G, Gm>(n, (g0 + p) * BPW + gi, li, true, true, out, xf[p]);
            return;
        }
    }
#pragma unroll
    for (int p = 0; p < PW; p++) {
        const int64_t k = (g0 + p) * BPW + gi;
        const bool active = k < nb;
        const bool full = active && k * G + G <= n;
        float xf[U][8];
        load_block_vectors<XT, Gm>(xv, n, k * G, li, active, full, src, xf);
        encode_loaded<FMT, G, Gm>(n, k, li, active, full, out, xf);
    }
}

template <int XT, int FMT, int G>
__global__ __launch_bounds__(kThreads) void k_encode(const void *__restrict__ xv, int64_t n,
                                                     int64_t nb, uint8_t *__restrict__ codes,
                                                     float *__restrict__ scales) {
    const int64_t wave = wave_id();
    encode_blocks<XT, FMT, G>(xv, n, nb, wave, SplitLayout<FMT, G>{codes, scales}, LinearSrc{});
}

// Aquavit payload with interleaved metadata: records[k] = [scale][codes].
template <int XT, int FMT, int G>
__global__ __launch_bounds__(kThreads) void k_encode_records(const void *__restrict__ xv,
                                                             int64_t n, int64_t nb,
                                                             uint8_t *__restrict__ records) {
    const int64_t wave = wave_id();
    encode_blocks<XT, FMT, G>(xv, n, nb, wave, RecordLayout<FMT, G>{records}, LinearSrc{});
}

// qgZ sender: tensor-slice reordering fused with the quantization of the N
// slices ([ZPP] "Tensor-slice reordering fixes incorrect gradient placement";
// "The implementation combines kernel fusion with communication overlap").
// The work-group y index is the slice; each slice is blocked on its own.
template <int XT, int FMT, int G>
__global__ __launch_bounds__(kThreads) void k_encode_reorder(
    const void *__restrict__ xv, int64_t slice_len, int64_t nb, int64_t C, int64_t N, double inv_c,
    uint8_t *__restrict__ codes, int64_t slice_stride, float *__restrict__ scales,
    int64_t scale_stride) {
    const int64_t j = group_y();
    const int64_t wave = wave_id();
    encode_blocks<XT, FMT, G>(xv, slice_len, nb, wave,
                              SplitLayout<FMT, G>{codes + j * slice_stride, scales + j * scale_stride},
                              ReorderSrc{C, N, j, inv_c});
}

// ---- decode kernel ----

// the 8 values of one vector of codes: fl(code * s)
template <int FMT>
__device__ __forceinline__ void decode_vector(const Packed8 &p, float s, float (&y)[8]) {
    if constexpr (FMT == E4M3) {
        y[0] = e4m3_value<0>(p.lo) * s; y[1] = e4m3_value<1>(p.lo) * s;
        y[2] = e4m3_value<2>(p.lo) * s; y[3] = e4m3_value<3>(p.lo) * s;
        y[4] = e4m3_value<0>(p.hi) * s; y[5] = e4m3_value<1>(p.hi) * s;
        y[6] = e4m3_value<2>(p.hi) * s; y[7] = e4m3_value<3>(p.hi) * s;
    } else {
        static_for<8>([&](auto I) {
            constexpr int i = decltype(I)::value;
            y[i] = field_value<FMT, i>(p) * s;
        });
    }
}

// 8 outputs at element e0 (a whole vector inside the tensor), streamed
template <int YT>
__device__ __forceinline__ void store_vector(void *__restrict__ yv, int64_t e0, const float (&y)[8]) {
    if constexpr (YT == F32) {
        float *o = (float *)yv + e0;
        store_stream16(o, make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]),
                                     __float_as_uint(y[2]), __float_as_uint(y[3])));
        store_stream16(o + 4, make_uint4(__float_as_uint(y[4]), __float_as_uint(y[5]),
                                         __float_as_uint(y[6]), __float_as_uint(y[7])));
    } else {
        store_stream16((uint16_t *)yv + e0,
                       make_uint4(narrow2<YT>(y[0], y[1]), narrow2<YT>(y[2], y[3]),
                                  narrow2<YT>(y[4], y[5]), narrow2<YT>(y[6], y[7])));
    }
}

// group `grp` (BPW blocks) of a wave, any block: the short last block and lanes
// past the end take guarded loads and stores
template <int FMT, int YT, int G, class In>
__device__ __forceinline__ void decode_group(In in, int64_t n, int64_t nb, int64_t grp,
                                             void *__restrict__ yv) {
    using Gm = dgeom<G>;
    constexpr int U = Gm::U, GL = Gm::GL, BPW = Gm::BPW;
    const int lane = lane_id();
    const int gi = lane / GL, li = lane % GL;
    const int64_t k = grp * BPW + gi;
    if (k >= nb) return;                       // no cross-lane work in this kernel
    const int64_t base = k * G;
    const bool full = base + G <= n;
    const float s = *in.scale(k);
    const int64_t block_bytes = ((n - base < G ? n - base : G) * fmt_traits<FMT>::bits + 7) / 8;
    const uint8_t *const codes = in.block(k);

#pragma unroll
    for (int u = 0; u < U; u++) {
        const int64_t el = (int64_t)(u * GL + li) * 8;
        const int64_t e0 = base + el;
        if (!full && e0 >= n) continue;
        Packed8 p;
        if (!full) p = load_vec_codes_tail<FMT>(codes, el, block_bytes);
        else if constexpr (FMT == INT6) p = int6_pair_load(codes, el);
        else p = load_vec_codes<FMT, In::kA8>(codes, el);
        float y[8];
        decode_vector<FMT>(p, s, y);
        if (full) {
            store_vector<YT>(yv, e0, y);
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                if (e0 + i >= n) break;
                if constexpr (YT == F32) {
                    ((float *)yv)[e0 + i] = y[i];
                } else {
                    ((uint16_t *)yv)[e0 + i] = (uint16_t)narrow2<YT>(y[i], 0.0f);
                }
            }
        }
    }
}

// Wave `wave` decodes groups PW*wave ... PW*wave + PW-1.  When they are all
// full (wave-uniform), every code and scale load is issued before any block is
// decoded; otherwise one group at a time.
template <int FMT, int YT, int G, class In>
__device__ __forceinline__ void decode_blocks(In in, int64_t n, int64_t nb, int64_t wave,
                                              void *__restrict__ yv) {
    using Gm = dgeom<G>;
    constexpr int U = Gm::U, GL = Gm::GL, BPW = Gm::BPW, PW = Gm::PWD;
    const int64_t g0 = wave * PW;
    if constexpr (PW > 1) {
        if ((g0 + PW) * BPW * G <= n) {
            const int lane = lane_id();
            const int gi = lane / GL, li = lane % GL;
            float s[PW];
            Packed8 p[PW][U];
#pragma unroll
            for (int q = 0; q < PW; q++) {
                const int64_t k = (g0 + q) * BPW + gi;
                s[q] = *in.scale(k);
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const int64_t el = (int64_t)(u * GL + li) * 8;
                    if constexpr (FMT == INT6) p[q][u] = int6_pair_load(in.block(k), el);
                    else p[q][u] = load_vec_codes<FMT, In::kA8>(in.block(k), el);
                }
            }
#pragma unroll
            for (int q = 0; q < PW; q++) {
                const int64_t k = (g0 + q) * BPW + gi;
#pragma unroll
                for (int u = 0; u < U; u++) {
                    float y[8];
                    decode_vector<FMT>(p[q][u], s[q], y);
                    store_vector<YT>(yv, k * G + (int64_t)(u * GL + li) * 8, y);
                }
            }
            return;
        }
    }
#pragma unroll
    for (int q = 0; q < PW; q++) decode_group<FMT, YT, G>(in, n, nb, g0 + q, yv);
}

template <int FMT, int YT, int G>
__global__ __launch_bounds__(kThreads) void k_decode(const uint8_t *__restrict__ codes,
                                                     const float *__restrict__ scales, int64_t n,
                                                     int64_t nb, void *__restrict__ yv) {
    const int64_t wave = wave_id();
    decode_blocks<FMT, YT, G>(SplitLayout<FMT, G>{(uint8_t *)codes, (float *)scales}, n, nb,
                              wave, yv);
}

template <int FMT, int YT, int G>
__global__ __launch_bounds__(kThreads) void k_decode_records(const uint8_t *__restrict__ records,
                                                             int64_t n, int64_t nb,
                                                             void *__restrict__ yv) {
    const int64_t wave = wave_id();
    decode_blocks<FMT, YT, G>(RecordLayout<FMT, G>{(uint8_t *)records}, n, nb, wave, yv);
}

// ---- dispatch ----

template <int XT, int FMT, int G>
static hipError_t run_encode(const void *x, int64_t n, uint8_t *codes, float *scales,
                             hipStream_t st) {
    const int64_t nb = (n + G - 1) / G;
    hipLaunchKernelGGL((k_encode<XT, FMT, G>), dim3(grid_for_waves(codec_waves<egeom<FMT, G>, egeom<FMT, G>::PW>(nb))), dim3(kThreads), 0, st,
                       x, n, nb, codes, scales);
    return hipGetLastError();
}

template <int FMT, int YT, int G>
static hipError_t run_decode(const uint8_t *codes, const float *scales, int64_t n, void *y,
                             hipStream_t st) {
    const int64_t nb = (n + G - 1) / G;
    hipLaunchKernelGGL((k_decode<FMT, YT, G>), dim3(grid_for_waves(codec_waves<dgeom<G>, dgeom<G>::PWD>(nb))), dim3(kThreads), 0, st,
                       codes, scales, n, nb, y);
    return hipGetLastError();
}

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

template <int XT, int FMT>
static hipError_t enc_g(const void *x, int64_t n, int G, uint8_t *c, float *s, hipStream_t st) {
    QCP_FOR_G(G, (run_encode<XT, FMT, GG>(x, n, c, s, st)))
}

template <int XT>
static hipError_t enc_f(const void *x, int64_t n, int G, int fmt, uint8_t *c, float *s,
                        hipStream_t st) {
    switch (fmt) {
    case INT2: return enc_g<XT, INT2>(x, n, G, c, s, st);
    case INT4: return enc_g<XT, INT4>(x, n, G, c, s, st);
    case INT6: return enc_g<XT, INT6>(x, n, G, c, s, st);
    case INT8: return enc_g<XT, INT8>(x, n, G, c, s, st);
    case E4M3: return enc_g<XT, E4M3>(x, n, G, c, s, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_encode(const void *x, int xt, int64_t n, int G, int fmt, uint8_t *codes,
                         float *scales, hipStream_t st) {
    switch (xt) {
    case F16: return enc_f<F16>(x, n, G, fmt, codes, scales, st);
    case BF16: return enc_f<BF16>(x, n, G, fmt, codes, scales, st);
    case F32: return enc_f<F32>(x, n, G, fmt, codes, scales, st);
    default: return hipErrorInvalidValue;
    }
}

template <int XT, int FMT, int G>
static hipError_t run_encode_records(const void *x, int64_t n, uint8_t *records, hipStream_t st) {
    const int64_t nb = (n + G - 1) / G;
    hipLaunchKernelGGL((k_encode_records<XT, FMT, G>), dim3(grid_for_waves(codec_waves<egeom<FMT, G>, egeom<FMT, G>::PW>(nb))), dim3(kThreads),
                       0, st, x, n, nb, records);
    return hipGetLastError();
}

template <int FMT, int YT, int G>
static hipError_t run_decode_records(const uint8_t *records, int64_t n, void *y, hipStream_t st) {
    const int64_t nb = (n + G - 1) / G;
    hipLaunchKernelGGL((k_decode_records<FMT, YT, G>), dim3(grid_for_waves(codec_waves<dgeom<G>, dgeom<G>::PWD>(nb))), dim3(kThreads),
                       0, st, records, n, nb, y);
    return hipGetLastError();
}

template <int XT, int FMT>
static hipError_t encrec_g(const void *x, int64_t n, int G, uint8_t *r, hipStream_t st) {
    QCP_FOR_G(G, (run_encode_records<XT, FMT, GG>(x, n, r, st)))
}

template <int XT>
static hipError_t encrec_b(const void *x, int64_t n, int G, int b, uint8_t *r, hipStream_t st) {
    switch (b) {
    case INT2: return encrec_g<XT, INT2>(x, n, G, r, st);
    case INT4: return encrec_g<XT, INT4>(x, n, G, r, st);
    case INT6: return encrec_g<XT, INT6>(x, n, G, r, st);
    case INT8: return encrec_g<XT, INT8>(x, n, G, r, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_encode_records(const void *x, int xt, int64_t n, int G, int b, uint8_t *records,
                                 hipStream_t st) {
    switch (xt) {
    case F16: return encrec_b<F16>(x, n, G, b, records, st);
    case BF16: return encrec_b<BF16>(x, n, G, b, records, st);
    case F32: return encrec_b<F32>(x, n, G, b, records, st);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT, int YT>
static hipError_t decrec_g(const uint8_t *r, int64_t n, int G, void *y, hipStream_t st) {
    QCP_FOR_G(G, (run_decode_records<FMT, YT, GG>(r, n, y, st)))
}

template <int FMT>
static hipError_t decrec_y(const uint8_t *r, int64_t n, int G, void *y, int yt, hipStream_t st) {
    switch (yt) {
    case F16: return decrec_g<FMT, F16>(r, n, G, y, st);
    case BF16: return decrec_g<FMT, BF16>(r, n, G, y, st);
    case F32: return decrec_g<FMT, F32>(r, n, G, y, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_records(const uint8_t *records, int64_t n, int G, int b, void *y, int yt,
                                 hipStream_t st) {
    switch (b) {
    case INT2: return decrec_y<INT2>(records, n, G, y, yt, st);
    case INT4: return decrec_y<INT4>(records, n, G, y, yt, st);
    case INT6: return decrec_y<INT6>(records, n, G, y, yt, st);
    case INT8: return decrec_y<INT8>(records, n, G, y, yt, st);
    default: return hipErrorInvalidValue;
    }
}

template <int XT, int FMT, int G>
static hipError_t run_encode_reorder(const void *x, int64_t n, int K, int N, uint8_t *codes,
                                     int64_t slice_stride, float *scales, int64_t scale_stride,
                                     hipStream_t st) {
    const int64_t L = n / N, C = L / K;
    const int64_t nb = (L + G - 1) / G;
    hipLaunchKernelGGL((k_encode_reorder<XT, FMT, G>), dim3(grid_for_waves(codec_waves<egeom<FMT, G>, egeom<FMT, G>::PW>(nb)), N),
                       dim3(kThreads), 0, st, x, L, nb, C, (int64_t)N, 1.0 / (double)C, codes,
                       slice_stride, scales, scale_stride);
    return hipGetLastError();
}

template <int XT, int FMT>
static hipError_t encr_g(const void *x, int64_t n, int K, int N, int G, uint8_t *c, int64_t cs,
                         float *s, int64_t ss, hipStream_t st) {
    QCP_FOR_G(G, (run_encode_reorder<XT, FMT, GG>(x, n, K, N, c, cs, s, ss, st)))
}

template <int XT>
static hipError_t encr_f(const void *x, int64_t n, int K, int N, int G, int fmt, uint8_t *c,
                         int64_t cs, float *s, int64_t ss, hipStream_t st) {
    switch (fmt) {
    case INT2: return encr_g<XT, INT2>(x, n, K, N, G, c, cs, s, ss, st);
    case INT4: return encr_g<XT, INT4>(x, n, K, N, G, c, cs, s, ss, st);
    case INT6: return encr_g<XT, INT6>(x, n, K, N, G, c, cs, s, ss, st);
    case INT8: return encr_g<XT, INT8>(x, n, K, N, G, c, cs, s, ss, st);
    case E4M3: return encr_g<XT, E4M3>(x, n, K, N, G, c, cs, s, ss, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_encode_reorder(const void *x, int xt, int64_t n, int n_nodes,
                                 int gpus_per_node, int G, int fmt, uint8_t *codes,
                                 int64_t slice_stride, float *scales, int64_t scale_stride,
                                 hipStream_t st) {
    switch (xt) {
    case F16: return encr_f<F16>(x, n, n_nodes, gpus_per_node, G, fmt, codes, slice_stride, scales, scale_stride, st);
    case BF16: return encr_f<BF16>(x, n, n_nodes, gpus_per_node, G, fmt, codes, slice_stride, scales, scale_stride, st);
    case F32: return encr_f<F32>(x, n, n_nodes, gpus_per_node, G, fmt, codes, slice_stride, scales, scale_stride, st);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT, int YT>
static hipError_t dec_g(const uint8_t *c, const float *s, int64_t n, int G, void *y,
                        hipStream_t st) {
    QCP_FOR_G(G, (run_decode<FMT, YT, GG>(c, s, n, y, st)))
}

template <int FMT>
static hipError_t dec_y(const uint8_t *c, const float *s, int64_t n, int G, void *y, int yt,
                        hipStream_t st) {
    switch (yt) {
    case F16: return dec_g<FMT, F16>(c, s, n, G, y, st);
    case BF16: return dec_g<FMT, BF16>(c, s, n, G, y, st);
    case F32: return dec_g<FMT, F32>(c, s, n, G, y, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const uint8_t *codes, const float *scales, int fmt, int64_t n, int G,
                         void *y, int yt, hipStream_t st) {
    switch (fmt) {
    case INT2: return dec_y<INT2>(codes, scales, n, G, y, yt, st);
    case INT4: return dec_y<INT4>(codes, scales, n, G, y, yt, st);
    case INT6: return dec_y<INT6>(codes, scales, n, G, y, yt, st);
    case INT8: return dec_y<INT8>(codes, scales, n, G, y, yt, st);
    case E4M3: return dec_y<E4M3>(codes, scales, n, G, y, yt, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qcp
