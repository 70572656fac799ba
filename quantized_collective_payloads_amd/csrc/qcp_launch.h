// qcp_launch.h -- internal launchers behind the C-ABI (one per kernel family).
// Arguments are already validated by the caller (qcp_api.hip); each launcher
// picks the template instance for (dtype, format, G) and enqueues it on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qcp {

// blockwise quantize + pack: x[n] of dtype xt -> codes (fmt), scales
hipError_t launch_encode(const void *x, int xt, int64_t n, int G, int fmt, uint8_t *codes,
                         float *scales, hipStream_t st);

// qgZ sender: tensor-slice reordering of x[n] (n_nodes x gpus_per_node chunks)
// fused with the quantization of the gpus_per_node slices it produces
hipError_t launch_encode_reorder(const void *x, int xt, int64_t n, int n_nodes,
                                 int gpus_per_node, int G, int fmt, uint8_t *codes,
                                 int64_t slice_stride, float *scales, int64_t scale_stride,
                                 hipStream_t st);

// sub-byte pack / unpack with interleaved metadata: one record per block,
// [fp32 scale][G*b/8 code bytes]
hipError_t launch_encode_records(const void *x, int xt, int64_t n, int G, int b, uint8_t *records,
                                 hipStream_t st);
hipError_t launch_decode_records(const uint8_t *records, int64_t n, int G, int b, void *y, int yt,
                                 hipStream_t st);

// unpack + dequantize: codes (fmt), scales -> y[n] of dtype yt
hipError_t launch_decode(const uint8_t *codes, const float *scales, int fmt, int64_t n, int G,
                         void *y, int yt, hipStream_t st);

// N-slice dequantize -> fp32 fmaf chain -> requantize
hipError_t launch_reduce(const uint8_t *codes_in, int64_t slice_stride, const float *scales_in,
                         int64_t scale_stride, int n_slices, int64_t L, int G, int fmt_in,
                         int fmt_out, uint8_t *codes_out, float *scales_out, float *sum_out,
                         hipStream_t st);

// in-place FP8 main-gradient accumulate
hipError_t launch_accum(uint8_t *state_codes, float *state_scales, const void *grad, int gt,
                        int64_t n, int G, hipStream_t st);

// workgroups of 4 waves; each kernel derives its wave index from the
// work-group and work-item ids
constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / 64;

// Work-item and work-group ids read through the compiler builtins.  (HIP's
// threadIdx / blockIdx / gridDim go through device-library functions that are
// compiled with different floating-point attributes than this library, so
// they are not inlined: every kernel would start with two function calls.)
__device__ __forceinline__ int lane_id() { return (int)(__builtin_amdgcn_workitem_id_x() & 63u); }
__device__ __forceinline__ int64_t wave_id() {
    return (int64_t)__builtin_amdgcn_workgroup_id_x() * kWavesPerGroup +
           (__builtin_amdgcn_workitem_id_x() >> 6);
}
__device__ __forceinline__ int64_t group_y() { return (int64_t)__builtin_amdgcn_workgroup_id_y(); }

// Work-groups per launch: a dispatch holds at most 2^32 - 1 work-items.  The
// entry points reject element counts whose grid would exceed this (QCP_EINVAL)
// before any launch; grid_for_waves returns 0 -- a launch the runtime refuses --
// should a grid still be too large.
constexpr int64_t kMaxGroups = ((int64_t)1 << 32) / kThreads - 1;

inline unsigned grid_for_waves(int64_t waves) {
    const int64_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
    return groups <= kMaxGroups ? (unsigned)groups : 0u;
}

}  // namespace qcp
