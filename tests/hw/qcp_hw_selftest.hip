// Hardware self-test of the arithmetic shortcuts the library kernels rely on
// (test infrastructure, not part of the library).  Each check compares a
// shortcut from qcp_device.h with the operation it stands in for, computed on
// the same GPU with IEEE-exact instructions, over every input where that is
// feasible:
//   recip_fast(s) == 1/s         every s in [2^-64, 2^64]          (2^30 values)
//   block_scale<F>(a).s == a/qmax, .r == 1/s
//                                every finite a >= 0, each format  (2^31 values)
//   quot_fast(x, s, 1/s) == x/s  hashed sample, s in [2^-64, 2^64], |x/s| < 2^9;
//                                below |x| = 2^-100 only the sign and |q| < 2^-10
//                                (code 0 / E4M3 zero either way) are required
//   cvt_sbyte<k>, cvt_nibble_16th<k>   every byte value at every byte position
// Every kernel covers its index space exactly: all lanes of every wave active
// (block_scale uses wave-wide votes), one result slot per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qcp_device.h"

using namespace qcp;

namespace {

constexpr int kPerLane = 64;            // values per lane
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t mix32(uint32_t h) {     // murmur3 finalizer
    h ^= h >> 16; h *= 0x85ebca6bu; h ^= h >> 13; h *= 0xc2b2ae35u; h ^= h >> 16;
    return h;
}

// one result per wave: number of failing values and the first one (bits)
__device__ __forceinline__ void wave_report(uint32_t bad, uint32_t bad_bits, uint32_t *count,
                                            uint32_t *example) {
    const int lane = threadIdx.x & 63;
    const uint64_t wave = ((uint64_t)__builtin_amdgcn_workgroup_id_x() * kThreads + threadIdx.x) >> 6;
    uint32_t total = bad;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) total += __shfl_xor(total, o);
    const uint64_t m = __ballot(bad != 0);
    const int first = m ? __builtin_ctzll(m) : 0;
    const uint32_t ex = __shfl(bad_bits, first);
    if (lane == 0) {
        count[wave] = total;
        example[wave] = ex;
    }
}

__global__ __launch_bounds__(kThreads) void k_recip(uint32_t *count, uint32_t *example) {
    const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t bad = 0, bad_bits = 0;
    for (int i = 0; i < kPerLane; i++) {
        const uint32_t j = (uint32_t)(t * kPerLane + i);            // < 2^30
        const uint32_t bits = ((63u + (j >> 23)) << 23) | (j & 0x7fffffu);   // 2^-64 .. 2^64 - ulp
        const float s = __uint_as_float(bits);
        const float got = recip_fast(s), want = 1.0f / s;
        if (__float_as_uint(got) != __float_as_uint(want)) {
            if (!bad) bad_bits = bits;
            bad++;
        }
    }
    wave_report(bad, bad_bits, count, example);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_block_scale(uint32_t *count, uint32_t *example) {
    const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    constexpr float qm = fmt_traits<FMT>::qmax;
    uint32_t bad = 0, bad_bits = 0;
    for (int i = 0; i < kPerLane; i++) {
        const uint32_t bits = (uint32_t)(t * kPerLane + i);          // 0 .. 0x7f7fffff
        const float a = __uint_as_float(bits);
        const BlockScale<FMT> b = block_scale<FMT>(a);
        const float s = a / qm;
        bool ok = __float_as_uint(b.s) == __float_as_uint(s) && b.fast == scale_in_fast_range(s);
        if (b.fast && s != 0.0f) ok = ok && __float_as_uint(b.r) == __float_as_uint(1.0f / s);
        if (!ok) {
            if (!bad) bad_bits = bits;
            bad++;
        }
    }
    wave_report(bad, bad_bits, count, example);
}

__global__ __launch_bounds__(kThreads) void k_quot(uint32_t seed, uint32_t *count, uint32_t *example) {
    const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t bad = 0, bad_bits = 0;
    for (int i = 0; i < kPerLane; i++) {
        const uint32_t c = (uint32_t)(t * kPerLane + i);
        const uint32_t h1 = mix32(c ^ seed), h2 = mix32(c * 0x9e3779b9u + seed);
        // s: any significand, exponent 2^-64 .. 2^63;  q: |q| in [2^-40, 2^9)
        const float s = __uint_as_float(((63u + (h1 >> 25)) << 23) | (h2 & 0x7fffffu));
        const float q = __uint_as_float(((87u + (h2 >> 23) % 49u) << 23) | (h1 & 0x7fffffu));
        float x = q * s;                       // a representable numerator near q*s
        if (h1 & 0x1000000u) x = -x;
        const float got = quot_fast(x, s, recip_fast(s)), want = x / s;
        bool ok;
        if (__builtin_fabsf(x) >= 7.88860905e-31f)          // 2^-100: exact
            ok = __float_as_uint(got) == __float_as_uint(want);
        else                                                // both round to a zero code
            ok = (__float_as_uint(got) >> 31) == (__float_as_uint(want) >> 31) &&
                 __builtin_fabsf(got) < 0.0009765625f && __builtin_fabsf(want) < 0.0009765625f;
        if (!ok) {
            if (!bad) bad_bits = c;
            bad++;
        }
    }
    wave_report(bad, bad_bits, count, example);
}

__global__ void k_sdwa(float *out) {
    const int t = threadIdx.x + blockIdx.x * blockDim.x;     // 0 .. 1023
    const int k = t >> 8, v = t & 255;
    const uint32_t w = (0x5a5a5a5au & ~(0xffu << (8 * k))) | ((uint32_t)v << (8 * k));
    float a, b;
    switch (k) {
        case 0: a = cvt_sbyte<0>(w); b = cvt_nibble_16th<0>(w); break;
        case 1: a = cvt_sbyte<1>(w); b = cvt_nibble_16th<1>(w); break;
        case 2: a = cvt_sbyte<2>(w); b = cvt_nibble_16th<2>(w); break;
        default: a = cvt_sbyte<3>(w); b = cvt_nibble_16th<3>(w); break;
    }
    out[2 * t] = a;
    out[2 * t + 1] = b;
}

// element-wise values for a host cross-check of the GPU's own reference operations
__global__ void k_values(const float *x, const float *s, int n, float *q_ieee, float *q_fast,
                         float *r_ieee, float *r_fast) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    q_ieee[i] = x[i] / s[i];
    q_fast[i] = quot_fast(x[i], s[i], recip_fast(s[i]));
    r_ieee[i] = 1.0f / s[i];
    r_fast[i] = recip_fast(s[i]);
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

// slots: 2^30 / 64 / 64 = 262144 waves
int64_t hw_recip_slots(void) { return ((int64_t)1 << 30) / kPerLane / 64; }

int hw_recip_exhaustive(uint32_t *count, uint32_t *example, void *stream) {
    const int64_t threads = ((int64_t)1 << 30) / kPerLane;
    hipLaunchKernelGGL(k_recip, dim3((unsigned)(threads / kThreads)), dim3(kThreads), 0,
                       (hipStream_t)stream, count, example);
    return status(hipGetLastError());
}

// slots: 0x7f800000 / 64 / 64 = 522240 waves
int64_t hw_block_scale_slots(void) { return (int64_t)0x7f800000 / kPerLane / 64; }

int hw_block_scale_exhaustive(int fmt, uint32_t *count, uint32_t *example, void *stream) {
    const int64_t threads = (int64_t)0x7f800000 / kPerLane;     // 33,423,360 = 130,560 x 256
    const dim3 grid((unsigned)(threads / kThreads)), block(kThreads);
    hipStream_t st = (hipStream_t)stream;
    switch (fmt) {
        case INT2: hipLaunchKernelGGL(k_block_scale<INT2>, grid, block, 0, st, count, example); break;
        case INT4: hipLaunchKernelGGL(k_block_scale<INT4>, grid, block, 0, st, count, example); break;
        case INT6: hipLaunchKernelGGL(k_block_scale<INT6>, grid, block, 0, st, count, example); break;
        case INT8: hipLaunchKernelGGL(k_block_scale<INT8>, grid, block, 0, st, count, example); break;
        case E4M3: hipLaunchKernelGGL(k_block_scale<E4M3>, grid, block, 0, st, count, example); break;
        default: return -1;
    }
    return status(hipGetLastError());
}

// `waves` result slots, 64 * 64 * waves sampled pairs
int hw_quot_sample(uint32_t seed, int64_t waves, uint32_t *count, uint32_t *example, void *stream) {
    if (waves <= 0 || waves % 4 != 0 || waves > ((int64_t)1 << 24)) return -1;
    hipLaunchKernelGGL(k_quot, dim3((unsigned)(waves / 4)), dim3(kThreads), 0, (hipStream_t)stream,
                       seed, count, example);
    return status(hipGetLastError());
}

// out: 2048 floats; out[2t], out[2t+1] for byte position t>>8 holding value t&255
int hw_sdwa(float *out, void *stream) {
    hipLaunchKernelGGL(k_sdwa, dim3(4), dim3(256), 0, (hipStream_t)stream, out);
    return status(hipGetLastError());
}

int hw_values(const float *x, const float *s, int n, float *q_ieee, float *q_fast, float *r_ieee,
              float *r_fast, void *stream) {
    if (n <= 0) return n == 0 ? 0 : -1;
    hipLaunchKernelGGL(k_values, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                       x, s, n, q_ieee, q_fast, r_ieee, r_fast);
    return status(hipGetLastError());
}

}  // extern "C"
