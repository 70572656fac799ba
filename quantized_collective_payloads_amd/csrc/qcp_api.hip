// qcp_api.hip -- the extern "C" entry points declared in include/qcp.h.
//
// Each entry point validates its arguments on the host (pure checks: no HIP
// call is made for a rejected call or for n == 0), then enqueues one kernel on
// the caller's stream and maps a launch error to QCP_EHIP.  Nothing is
// allocated and no state is kept between calls.
#include <stdint.h>

#include "qcp.h"
#include "qcp_launch.h"

namespace {

// Largest element count (per tensor, or per slice of a reduce) any entry point
// accepts.  A dispatch holds at most 2^32 - 1 work-items, i.e. kMaxGroups
// work-groups of 256; every kernel gives a work-group at least 4096 elements
// (4 waves, each at least 64 lanes x 16 codes), so kMaxGroups * 4096 elements
// always fit in one launch.  That is 2^36 - 4096 elements: 137 GB of bf16 input.
constexpr int64_t kMaxElems = qcp::kMaxGroups * 4096;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool valid_g(int32_t G) { return G >= 32 && G <= 1024 && (G & (G - 1)) == 0; }
bool valid_dtype(int t) { return t == QCP_F16 || t == QCP_BF16 || t == QCP_F32; }
bool valid_fmt(int f) {
    return f == QCP_INT2 || f == QCP_INT4 || f == QCP_INT6 || f == QCP_INT8 || f == QCP_E4M3;
}
int fmt_bits(int f) { return f == QCP_E4M3 ? 8 : f; }
int64_t dtype_bytes(int t) { return t == QCP_F32 ? 4 : 2; }
int64_t code_bytes(int64_t n, int fmt) { return (n * fmt_bits(fmt) + 7) / 8; }
int64_t n_blocks(int64_t n, int32_t G) { return (n + G - 1) / G; }

// do [a, a+na) and [b, b+nb) intersect?
bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return na > 0 && nb > 0 && a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int status_of(hipError_t e) { return e == hipSuccess ? QCP_OK : QCP_EHIP; }

int check_common(int64_t n, int32_t G) {
    if (n < 0 || n > kMaxElems) return QCP_EINVAL;
    if (!valid_g(G)) return QCP_EINVAL;
    return QCP_OK;
}

}  // namespace

extern "C" {

int quantize_blockwise(const void *x, int xt, int64_t n, int32_t G, int fmt, void *codes,
                       float *scales, void *stream) {
    int rc = check_common(n, G);
    if (rc != QCP_OK) return rc;
    if (!valid_dtype(xt) || !valid_fmt(fmt)) return QCP_EINVAL;
    if (n == 0) return QCP_OK;
    if (!x || !codes || !scales) return QCP_EINVAL;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return QCP_EALIGN;
    int64_t xb = n * dtype_bytes(xt), cb = code_bytes(n, fmt), sb = 4 * n_blocks(n, G);
    if (overlap(x, xb, codes, cb) || overlap(x, xb, scales, sb) || overlap(codes, cb, scales, sb))
        return QCP_EINVAL;
    return status_of(qcp::launch_encode(x, xt, n, G, fmt, (uint8_t *)codes, scales,
                                        (hipStream_t)stream));
}

int reorder_quantize(const void *x, int xt, int64_t n, int32_t n_nodes, int32_t gpus_per_node,
                     int32_t G, int fmt, void *codes, int64_t slice_stride_bytes, float *scales,
                     int64_t scale_stride, void *stream) {
    int rc = check_common(n, G);
    if (rc != QCP_OK) return rc;
    if (!valid_dtype(xt) || !valid_fmt(fmt)) return QCP_EINVAL;
    if (n_nodes < 1 || n_nodes > 65536 || gpus_per_node < 1 || gpus_per_node > 64) return QCP_EINVAL;
    const int64_t W = (int64_t)n_nodes * gpus_per_node;
    if (n % W != 0 || (n / W) % 8 != 0) return QCP_EINVAL;
    if (n == 0) return QCP_OK;
    if (!x || !codes || !scales) return QCP_EINVAL;
    const int64_t L = n / gpus_per_node, cb = code_bytes(L, fmt), nb = n_blocks(L, G);
    if (slice_stride_bytes < cb || scale_stride < nb) return QCP_EINVAL;
    if (slice_stride_bytes % 16 != 0 || scale_stride % 4 != 0) return QCP_EALIGN;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return QCP_EALIGN;
    const int64_t xb = n * dtype_bytes(xt);
    const int64_t ob = (int64_t)(gpus_per_node - 1) * slice_stride_bytes + cb;
    const int64_t sb = 4 * ((int64_t)(gpus_per_node - 1) * scale_stride + nb);
    if (overlap(x, xb, codes, ob) || overlap(x, xb, scales, sb) || overlap(codes, ob, scales, sb))
        return QCP_EINVAL;
    return status_of(qcp::launch_encode_reorder(x, xt, n, n_nodes, gpus_per_node, G, fmt,
                                                (uint8_t *)codes, slice_stride_bytes, scales,
                                                scale_stride, (hipStream_t)stream));
}

int dequantize_blockwise(const void *codes, const float *scales, int fmt, int64_t n, int32_t G,
                         void *y, int yt, void *stream) {
    int rc = check_common(n, G);
    if (rc != QCP_OK) return rc;
    if (!valid_dtype(yt) || !valid_fmt(fmt)) return QCP_EINVAL;
    if (n == 0) return QCP_OK;
    if (!codes || !scales || !y) return QCP_EINVAL;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(y)) return QCP_EALIGN;
    int64_t yb = n * dtype_bytes(yt), cb = code_bytes(n, fmt), sb = 4 * n_blocks(n, G);
    if (overlap(y, yb, codes, cb) || overlap(y, yb, scales, sb)) return QCP_EINVAL;
    return status_of(qcp::launch_decode((const uint8_t *)codes, scales, fmt, n, G, y, yt,
                                        (hipStream_t)stream));
}

int pack_subbyte(const void *x, int xt, int64_t n, int32_t b, int32_t G, uint8_t *packed,
                 float *scales, void *stream) {
    if (b != 2 && b != 4 && b != 6 && b != 8) return QCP_EINVAL;
    return quantize_blockwise(x, xt, n, G, b, packed, scales, stream);
}

int unpack_subbyte(const uint8_t *packed, const float *scales, int64_t n, int32_t b, int32_t G,
                   void *y, int yt, void *stream) {
    if (b != 2 && b != 4 && b != 6 && b != 8) return QCP_EINVAL;
    return dequantize_blockwise(packed, scales, b, n, G, y, yt, stream);
}

int pack_subbyte_records(const void *x, int xt, int64_t n, int32_t b, int32_t G,
                         uint8_t *records, void *stream) {
    int rc = check_common(n, G);
    if (rc != QCP_OK) return rc;
    if (!valid_dtype(xt) || (b != 2 && b != 4 && b != 6 && b != 8)) return QCP_EINVAL;
    if (n == 0) return QCP_OK;
    if (!x || !records) return QCP_EINVAL;
    if (!aligned16(x) || !aligned16(records)) return QCP_EALIGN;
    if (overlap(x, n * dtype_bytes(xt), records, qcp_payload_bytes(n, b, G))) return QCP_EINVAL;
    return status_of(qcp::launch_encode_records(x, xt, n, G, b, records, (hipStream_t)stream));
}

int unpack_subbyte_records(const uint8_t *records, int64_t n, int32_t b, int32_t G, void *y,
                           int yt, void *stream) {
    int rc = check_common(n, G);
    if (rc != QCP_OK) return rc;
    if (!valid_dtype(yt) || (b != 2 && b != 4 && b != 6 && b != 8)) return QCP_EINVAL;
    if (n == 0) return QCP_OK;
    if (!records || !y) return QCP_EINVAL;
    if (!aligned16(records) || !aligned16(y)) return QCP_EALIGN;
    if (overlap(y, n * dtype_bytes(yt), records, qcp_payload_bytes(n, b, G))) return QCP_EINVAL;
    return status_of(qcp::launch_decode_records(records, n, G, b, y, yt, (hipStream_t)stream));
}

int dequant_reduce_requant(const void *codes_in, int64_t in_slice_stride_bytes,
                           const float *scales_in, int64_t in_scale_stride, int32_t n_slices,
                           int64_t slice_len, int32_t G, int fmt_in, int fmt_out,
                           void *codes_out, float *scales_out, float *sum_out, void *stream) {
    int rc = check_common(slice_len, G);
    if (rc != QCP_OK) return rc;
    if (!valid_fmt(fmt_in) || !valid_fmt(fmt_out)) return QCP_EINVAL;
    if (n_slices < 1 || n_slices > 64) return QCP_EINVAL;
    if (slice_len == 0) return QCP_OK;
    if (!codes_in || !scales_in || !codes_out || !scales_out) return QCP_EINVAL;
    int64_t in_cb = code_bytes(slice_len, fmt_in), nb = n_blocks(slice_len, G);
    if (in_slice_stride_bytes < in_cb || in_scale_stride < nb) return QCP_EINVAL;
    if (in_slice_stride_bytes % 16 != 0 || in_scale_stride % 4 != 0) return QCP_EALIGN;
    if (!aligned16(codes_in) || !aligned16(scales_in) || !aligned16(codes_out) ||
        !aligned16(scales_out) || (sum_out && !aligned16(sum_out)))
        return QCP_EALIGN;
    int64_t in_b = (int64_t)(n_slices - 1) * in_slice_stride_bytes + in_cb;
    int64_t in_sb = 4 * ((int64_t)(n_slices - 1) * in_scale_stride + nb);
    int64_t out_cb = code_bytes(slice_len, fmt_out), out_sb = 4 * nb, sum_b = 4 * slice_len;
    const void *outs[3] = {codes_out, scales_out, sum_out};
    int64_t out_len[3] = {out_cb, out_sb, sum_out ? sum_b : 0};
    for (int i = 0; i < 3; i++) {
        if (overlap(outs[i], out_len[i], codes_in, in_b) ||
            overlap(outs[i], out_len[i], scales_in, in_sb))
            return QCP_EINVAL;
        for (int j = i + 1; j < 3; j++)
            if (overlap(outs[i], out_len[i], outs[j], out_len[j])) return QCP_EINVAL;
    }
    return status_of(qcp::launch_reduce((const uint8_t *)codes_in, in_slice_stride_bytes,
                                        scales_in, in_scale_stride, n_slices, slice_len, G,
                                        fmt_in, fmt_out, (uint8_t *)codes_out, scales_out,
                                        sum_out, (hipStream_t)stream));
}

int fp8_accum_requant(uint8_t *state_codes, float *state_scales, const void *grad, int gt,
                      int64_t n, int32_t G, void *stream) {
    int rc = check_common(n, G);
    if (rc != QCP_OK) return rc;
    if (!valid_dtype(gt)) return QCP_EINVAL;
    if (n == 0) return QCP_OK;
    if (!state_codes || !state_scales || !grad) return QCP_EINVAL;
    if (!aligned16(state_codes) || !aligned16(state_scales) || !aligned16(grad)) return QCP_EALIGN;
    int64_t cb = n, sb = 4 * n_blocks(n, G), gb = n * dtype_bytes(gt);
    if (overlap(state_codes, cb, state_scales, sb) || overlap(grad, gb, state_codes, cb) ||
        overlap(grad, gb, state_scales, sb))
        return QCP_EINVAL;
    return status_of(qcp::launch_accum(state_codes, state_scales, grad, gt, n, G,
                                       (hipStream_t)stream));
}

int64_t qcp_payload_bytes(int64_t n, int32_t bits, int32_t G) {
    if (n < 0 || G < 1 || bits < 1 || bits > 32) return -1;
    return (n * bits + 7) / 8 + 4 * ((n + G - 1) / G);
}

double qcp_aquavit_target(int64_t t, int64_t T, double a, double c) {
    if (T <= 0 || t < 0 || t > T) return -1.0;
    return 8.0 - 6.0 / (a + c * (double)t / (double)T);   // (c*t)/T, left to right
}

int qcp_aquavit_level(int64_t t, int64_t T, double a, double c, int32_t *b, int32_t *G) {
    if (T <= 0 || t < 0 || t > T || !b || !G) return QCP_EINVAL;
    const double want = qcp_aquavit_target(t, T, a, c);
    // levels b + 32/G in increasing bpw: within each b, G from 1024 down to 32
    double best = 0.0;
    bool have = false;
    for (int32_t bb = 2; bb <= 8; bb += 2) {
        for (int32_t gg = 1024; gg >= 32; gg /= 2) {
            const double level = bb + 32.0 / gg;
            const double d = level > want ? level - want : want - level;
            // strictly closer wins; on a tie the earlier (smaller) level stays
            if (!have || d < best) {
                best = d;
                *b = bb;
                *G = gg;
                have = true;
            }
        }
    }
    return QCP_OK;
}

const char *qcp_strerror(int status) {
    switch (status) {
    case QCP_OK: return "success";
    case QCP_EINVAL: return "invalid argument (size, block size, bit width, format, dtype, stride, null or overlapping buffer)";
    case QCP_EALIGN: return "pointer or stride not aligned to 16 bytes";
    case QCP_EUNSUPPORTED: return "unsupported combination";
    case QCP_EHIP: return "HIP runtime error at kernel launch";
    default: return "unknown status";
    }
}

const char *qcp_version(void) { return "0.2.0"; }

int64_t qcp_max_elements(void) { return kMaxElems; }

}  // extern "C"
