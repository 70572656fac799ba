/*
 * qcp.h -- quantized collective payloads: the C-ABI of libqcp.so.
 *
 * The data-parallel hot path of quantized ZeRO-3 communication, on one
 * gfx950 (MI355X) GPU: the kernels that sit on either side of the collectives
 * (quantize before an all-gather or all-to-all, dequantize or reduce after it).
 *
 * Sources (web pages, cited by title and section):
 *  [ZPP]  "Quantized LLM Training at Scale with ZeRO++" (talk summary):
 *         "Blockwise weight quantization cuts forward-gather traffic in half" (qwZ),
 *         "QGZ keeps reductions in full precision while sending quantized gradients",
 *         "The implementation combines kernel fusion with communication overlap" (qgZ).
 *  [AQV]  "Aquavit: Ascending Quantization for Communication-Efficient Vast-Scale
 *         Distributed Training" (review): granularity modulation, bpw = b + 32/G
 *         (Eq. 6, Table 1), b in {2,4,6,8}, sub-byte packing kernels (Section 5.2).
 *  [AGOQ] "AGoQ: Activation and Gradient Quantization for Memory-Efficient
 *         Distributed Training of LLMs", Section 2.B (QuanGrad): local accumulation
 *         of FP8 gradients, and the local-reduce step of the precision-preserved
 *         all-reduce.
 *
 * Conventions shared by every entry point
 *  - Pointers are device pointers (HBM), except where a comment says otherwise.
 *    The caller allocates and frees every buffer; the library allocates nothing,
 *    keeps no pointer after returning and holds no mutable global state.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call
 *    enqueues its kernel(s) on `stream` and returns without synchronizing; the
 *    status reports argument validation and launch errors only.
 *  - Element types (qcp_dtype): fp16, bf16, fp32.  A payload format (qcp_fmt) is
 *    INT2/INT4/INT6/INT8 (symmetric two's-complement codes in [-qmax, qmax],
 *    qmax = 2^(b-1)-1) or E4M3 (OCP E4M3FN, largest finite value 448).
 *  - Blocks: element i of a tensor (or of one slice) belongs to block i / G; the
 *    last block may be short.  Each block has one fp32 scale s = absmax / qmax
 *    (IEEE division; a block of zeros has s = +0 and all codes 0).
 *  - Codes: q = IEEE fp32 quotient x / s; INT code = round-half-even(q) clamped
 *    to [-qmax, qmax]; E4M3 code = nearest E4M3FN value to q, ties to even
 *    mantissa (sign of zero kept, NaN never produced).
 *  - Code layout: an LSB-first bitstream; element i occupies bits [b*i, b*i+b)
 *    and bit 8j+t of the stream is bit t of byte j.  So INT8 and E4M3 are one
 *    byte per code, INT4 puts the even element in the low nibble, INT6 packs 4
 *    codes in 3 bytes.  The stream is ceil(n*b/8) bytes, zero-padded at the end.
 *    Scales are a separate fp32 array of ceil(n/G) entries.
 *  - Preconditions: 0 <= n <= qcp_max_elements() (n == 0 is a no-op returning
 *    QCP_OK; for a reduce, n is the slice length); G a power of two in
 *    [32, 1024]; every pointer non-null and 16-byte aligned when there is work;
 *    inputs finite (non-finite inputs give unspecified codes, never a fault);
 *    outputs do not overlap inputs (except the in-place state of
 *    fp8_accum_requant) and do not overlap each other.
 *  - Results are a pure function of the inputs: no atomics, a fixed order of
 *    summation, byte-identical on every run.
 */
#ifndef QCP_H
#define QCP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QCP_OK = 0,
    QCP_EINVAL = -1,        /* bad size, G, b, format, dtype, stride, null or overlapping pointer */
    QCP_EALIGN = -2,        /* a pointer or stride is not a multiple of 16 bytes */
    QCP_EUNSUPPORTED = -3,  /* a combination this library does not implement */
    QCP_EHIP = -4           /* the HIP runtime reported an error at launch */
} qcp_status;

typedef enum { QCP_F16 = 1, QCP_BF16 = 2, QCP_F32 = 3 } qcp_dtype;

typedef enum { QCP_INT2 = 2, QCP_INT4 = 4, QCP_INT6 = 6, QCP_INT8 = 8, QCP_E4M3 = 0x43 } qcp_fmt;

/*
 * Blockwise quantize [ZPP qwZ: per-block 8-bit weight quantization of the
 * forward all-gather payload; AGOQ: per-block E4M3].
 *   x       n elements of type xt
 *   codes   out: ceil(n*b/8) bytes in format fmt (b = 8 for INT8/E4M3)
 *   scales  out: ceil(n/G) fp32
 * Any qcp_fmt is accepted; INT8 is the qwZ payload, E4M3 the FP8 one.
 */
int quantize_blockwise(const void *x, int xt, int64_t n, int32_t G, int fmt,
                       void *codes, float *scales, void *stream);

/*
 * Blockwise dequantize [ZPP qwZ: the gathered 8-bit payload becomes 16-bit
 * values again before compute]:  y_i = cast(fl(value(code_i) * s_{i/G})) with
 * one round-to-nearest-even cast to yt (fp32 output is the product itself).
 *   codes   ceil(n*b/8) bytes;  scales ceil(n/G) fp32;  y out: n elements of yt
 */
int dequantize_blockwise(const void *codes, const float *scales, int fmt, int64_t n,
                         int32_t G, void *y, int yt, void *stream);

/*
 * Sub-byte pack [AQV granularity modulation, Section 5.1-5.2]: fused blockwise
 * quantize + pack to b bits, b in {2,4,6,8}; identical to
 * quantize_blockwise(fmt = b).  Payload = ceil(n*b/8) + 4*ceil(n/G) bytes, so
 * bpw = b + 32/G when G divides n.
 */
int pack_subbyte(const void *x, int xt, int64_t n, int32_t b, int32_t G,
                 uint8_t *packed, float *scales, void *stream);

/* Sub-byte unpack + dequantize [AQV]: identical to dequantize_blockwise(fmt = b). */
int unpack_subbyte(const uint8_t *packed, const float *scales, int64_t n, int32_t b,
                   int32_t G, void *y, int yt, void *stream);

/*
 * Fused dequantize -> fp32 sum over N slices -> requantize.
 * [ZPP qgZ: the slices one rank receives from its N peers after the all-to-all
 * are dequantized, reduced in full precision and requantized for the next hop,
 * in one kernel.  AGOQ precision-preserved all-reduce, step 2 "Local Reduce":
 * dequantize received FP8 to FP32, sum, requantize to FP8.]
 *   codes_in   slice j (j = 0..n_slices-1) starts at codes_in + j*in_slice_stride_bytes
 *              and holds slice_len codes in fmt_in (ceil(slice_len*b_in/8) bytes)
 *   scales_in  slice j's ceil(slice_len/G) scales start at scales_in + j*in_scale_stride
 *   For each element i:  acc = -0.0;  acc = fmaf(value(c_ji), s_j[i/G], acc) for
 *   j = 0..n_slices-1 in order;  sum_i = acc.
 *   The sums are quantized blockwise with the same G in fmt_out:
 *   codes_out  ceil(slice_len*b_out/8) bytes;  scales_out ceil(slice_len/G) fp32
 *   sum_out    nullable; if given, slice_len fp32 sums
 *   1 <= n_slices <= 64; in_slice_stride_bytes is a multiple of 16 and at least
 *   one slice's code bytes; in_scale_stride (in floats) is a multiple of 4 and
 *   at least ceil(slice_len/G).
 */
int dequant_reduce_requant(const void *codes_in, int64_t in_slice_stride_bytes,
                           const float *scales_in, int64_t in_scale_stride,
                           int32_t n_slices, int64_t slice_len, int32_t G,
                           int fmt_in, int fmt_out, void *codes_out, float *scales_out,
                           float *sum_out, void *stream);

/*
 * Sub-byte pack / unpack with interleaved metadata [AQV Section 5.2, metadata
 * interleaving]: the payload of n elements at b bits with block size G as one
 * record per block, records back to back:
 *   record k = [fp32 scale s_k (4 bytes)][codes of block k, LSB-first b-bit
 *              fields: G*b/8 bytes, ceil(len*b/8) for the short last block]
 * so record k starts at byte k*(4 + G*b/8) and the whole stream has exactly
 * qcp_payload_bytes(n, b, G) bytes.  Codes and scales are those of
 * pack_subbyte / unpack_subbyte; only the layout differs.
 *   records   output of pack / input of unpack, 16-byte aligned.
 * Errors: as pack_subbyte / unpack_subbyte.
 */
int pack_subbyte_records(const void *x, int xt, int64_t n, int32_t b, int32_t G,
                         uint8_t *records, void *stream);
int unpack_subbyte_records(const uint8_t *records, int64_t n, int32_t b, int32_t G, void *y,
                           int yt, void *stream);

/*
 * Aquavit ascending precision schedule [AQV key idea, Section 5.1, Table 1]:
 * the target bits per weight at step t of T is 8 - 6/(a + c*t/T) ((a, c) =
 * (0.9, 5) on the pages); qcp_aquavit_level writes the granularity-modulation
 * level (b in {2,4,6,8}, G in {32, ..., 1024}) whose b + 32/G is nearest the
 * target (ties: the smaller b + 32/G).  From t = 0 to t = T this runs from
 * 2-bit/G=1024 (2.03 bpw) to 6-bit/G=32 (7.00 bpw).  Host only.
 * qcp_aquavit_target returns -1 and qcp_aquavit_level QCP_EINVAL unless
 * 0 <= t <= T and T > 0 (and b, G non-null).
 */
double qcp_aquavit_target(int64_t t, int64_t T, double a, double c);
int qcp_aquavit_level(int64_t t, int64_t T, double a, double c, int32_t *b, int32_t *G);

/*
 * qgZ sender: tensor-slice reordering fused with the quantization of the
 * intra-node all-to-all's send slices [ZPP "Tensor-slice reordering fixes
 * incorrect gradient placement"; "The implementation combines kernel fusion
 * with communication overlap": reordering fused with intra-node quantization].
 *   x               one rank's gradient bucket, n elements of type xt; it is
 *                   W = n_nodes*gpus_per_node chunks of C = n/W elements, chunk
 *                   c being the part global rank c (node c/N, GPU c%N) owns
 *                   after the reduce-scatter (N = gpus_per_node, K = n_nodes)
 *   codes, scales   N slices: slice j holds chunks b*N + j for b = 0..K-1 in
 *                   node order (L = n/N elements), quantized blockwise in fmt
 *                   with blocks restarting at each slice.  Its codes start at
 *                   codes + j*slice_stride_bytes (ceil(L*b/8) bytes), its
 *                   ceil(L/G) scales at scales + j*scale_stride.
 * With this order, after the intra-node reduce (dequant_reduce_requant on the
 * N received slices) and the inter-node exchange, every rank holds its own
 * chunk.  Equivalent to reordering x and calling quantize_blockwise on each
 * slice.  Preconditions beyond the shared ones: 1 <= n_nodes <= 65536,
 * 1 <= gpus_per_node <= 64, n divisible by W with C a multiple of 8;
 * slice_stride_bytes a multiple of 16 and >= ceil(L*b/8); scale_stride a
 * multiple of 4 and >= ceil(L/G).  Errors: QCP_EINVAL, QCP_EALIGN, QCP_EHIP.
 */
int reorder_quantize(const void *x, int xt, int64_t n, int32_t n_nodes, int32_t gpus_per_node,
                     int32_t G, int fmt, void *codes, int64_t slice_stride_bytes, float *scales,
                     int64_t scale_stride, void *stream);

/*
 * FP8 main-gradient accumulation, in place [AGOQ QuanGrad "Local Accumulation":
 * dequantize the FP8 main gradient to 16 bits, add the micro-batch gradient,
 * requantize the sum to FP8]:
 *   d_i = bf16(fl(value(e_i) * s_{i/G}));  t_i = bf16(fl(d_i + g_i));
 *   (state_codes, state_scales) <- E4M3 blockwise quantization of t.
 *   state_codes  n E4M3 bytes (read and overwritten)
 *   state_scales ceil(n/G) fp32 (read and overwritten)
 *   grad         n elements of type gt
 * The all-zero state (codes 0x00, scales +0) is the empty accumulator.
 */
int fp8_accum_requant(uint8_t *state_codes, float *state_scales, const void *grad, int gt,
                      int64_t n, int32_t G, void *stream);

/* Payload bytes of n codes at `bits` bits with one fp32 scale per G elements:
 * ceil(n*bits/8) + 4*ceil(n/G); -1 for invalid arguments.  Host only. */
int64_t qcp_payload_bytes(int64_t n, int32_t bits, int32_t G);

/* Static, human-readable text for a qcp_status value.  Host only. */
const char *qcp_strerror(int status);

/* Library version as "major.minor.patch".  Host only. */
const char *qcp_version(void);

/* Largest element count an entry point accepts (per tensor, or per slice of a
 * reduce): 2^36 - 4096, the most one kernel launch covers (a dispatch holds at
 * most 2^32 - 1 work-items).  Larger counts return QCP_EINVAL without a
 * launch; split such payloads into several calls.  Host only. */
int64_t qcp_max_elements(void);

#ifdef __cplusplus
}
#endif

#endif /* QCP_H */
