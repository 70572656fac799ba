/*
 * qcp_oracle.c -- CPU oracle for blockwise quantization of ZeRO-3
 * communication payloads.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
 * benchmark's CPU-baseline leg are the only code allowed to load this library.
 * The product (the HIP library and its Python binding) never calls, links or
 * includes anything from here, and this file includes nothing from the product.
 *
 * What it is: a plain, scalar, single-threaded restatement of what the method
 * computes, written for a reader who checks it against the pages by eye.  It is
 * deliberately slow.  Arithmetic is IEEE-754 binary32, round-to-nearest-even,
 * gradual underflow, no contraction: the build uses -O2 -fno-fast-math
 * -ffp-contract=off, and a fused multiply-add happens only where fmaf() is
 * written.  Conversions to and from binary16, bfloat16 and OCP E4M3 are written
 * here from the format definitions (in double precision, where every step is
 * exact), not taken from any library.
 *
 * Sources (web pages; cited by title and section):
 *  [ZPP]   "Quantized LLM Training at Scale with ZeRO++" (talk summary), sections
 *          "Blockwise weight quantization cuts forward-gather traffic in half",
 *          "QGZ keeps reductions in full precision while sending quantized
 *          gradients", "Two-hop communication prevents QGZ traffic from
 *          multiplying across GPUs", "The implementation combines kernel fusion
 *          with communication overlap".
 *  [AQV]   "Aquavit: Ascending Quantization for Communication-Efficient
 *          Vast-Scale Distributed Training" (review), 1-minute summary
 *          (granularity modulation), key idea (b in {2,4,6,8}, G 1024 -> 32,
 *          Table 1), glossary "Granularity modulation / effective bpw" (Eq. 6).
 *  [AGOQ]  "AGoQ: Activation and Gradient Quantization for Memory-Efficient
 *          Distributed Training of LLMs", section 2.B "Precision-Preserved
 *          Gradient Quantization (QuanGrad)": "Local Accumulation" and
 *          "Precision-Preserved All-Reduce", step 2 "Local Reduce".
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes):
 *  - symmetric absmax scaling, one binary32 scale per block of G elements, no
 *    zero point; s = fl(absmax / qmax), qmax = 2^(b-1)-1 (INT) or 448 (E4M3);
 *  - INT code = clamp(round-half-even(fl(x / s)), -qmax, qmax), a true IEEE
 *    division; a block whose absmax is 0 gets s = +0 and all codes 0;
 *  - E4M3 code = OCP E4M3FN value nearest fl(x / s), ties to even mantissa,
 *    saturating at +-448, sign of zero kept, NaN never produced;
 *  - the last block of a tensor (or of a slice) may be short; blocking restarts
 *    at every slice of a reduce input;
 *  - INT b codes are b-bit two's-complement fields in an LSB-first bitstream
 *    (element i occupies stream bits [b*i, b*i+b), stream bit 8j+t is bit t of
 *    byte j), zero-padded at the end only;
 *  - dequantize = fl(float(code) * s), then one round-to-nearest-even cast;
 *  - the N-slice reduce is an fmaf chain in slice order starting from -0.0;
 *  - FP8 accumulate rounds to bfloat16 after the dequantize and after the add.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* element types and payload formats (numeric values are this file's own) */
enum { O_F16 = 1, O_BF16 = 2, O_F32 = 3 };
enum { O_INT2 = 2, O_INT4 = 4, O_INT6 = 6, O_INT8 = 8, O_E4M3 = 0x43 };

#define O_OK 0
#define O_BAD (-1)

/* ------------------------------------------------------------------------ */
/* Number formats, written from their definitions.                          */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* binary16: sign, 5-bit biased exponent (bias 15), 10-bit fraction. */
static float f16_value(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* 2^-14 * m/1024 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + m, e - 25);          /* 2^(e-15) * (1 + m/1024) */
    return (float)(sign ? -v : v);
}

/* bfloat16 is the upper half of a binary32 bit pattern. */
static float bf16_value(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* Nearest binary16 to v, ties to even; |v| >= 65520 (max + half ulp) -> inf. */
static uint16_t f16_round(float v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs((double)v);
    int e;
    if (isnan(v)) return sign | 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        e = -14;                                /* subnormal binade, spacing 2^-24 */
    } else {
        frexp(a, &e);                           /* a in [2^(e-1), 2^e) */
        e -= 1;                                 /* a in [2^e, 2^(e+1)) */
    }
    double m = nearbyint(ldexp(a, 10 - e));     /* units of 2^(e-10), ties even */
    if (e == -14 && m < 1024.0) return sign | (uint16_t)m;
    if (m >= 2048.0) { m /= 2.0; e += 1; }      /* carry into the next binade */
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* Nearest bfloat16 to v, ties to even.  The two candidates are v truncated to
 * 16 bits and the next bfloat16 away from zero; above the largest finite value
 * the next one is 2^128, which encodes as infinity. */
static uint16_t bf16_round(float v) {
    uint32_t u = f32_to_bits(v);
    if (isnan(v)) return (uint16_t)((u >> 16) | 0x40);
    if (isinf(v)) return (uint16_t)(u >> 16);
    uint32_t lo = u & 0xffff0000u;
    uint32_t hi = lo + 0x10000u;
    double dv = fabs((double)v);
    double dlo = fabs((double)bits_to_f32(lo));
    double dhi = ((hi & 0x7fffffffu) == 0x7f800000u) ? ldexp(1.0, 128)
                                                      : fabs((double)bits_to_f32(hi));
    double below = dv - dlo, above = dhi - dv;
    if (below < above) return (uint16_t)(lo >> 16);
    if (above < below) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

/* OCP E4M3FN: sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent 0 is
 * subnormal (2^-6 * m/8); S.1111.111 is NaN; largest finite value 448. */
static float e4m3_value(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + m, e - 10);             /* 2^(e-7) * (1 + m/8) */
    return (float)(sign ? -v : v);
}

/* Nearest E4M3FN value to q, ties to even mantissa, saturating to +-448.
 * Inputs are finite by contract, so a NaN quotient has no specified code; it
 * saturates here (a defined result, where converting NaN to an integer below
 * would be undefined behaviour in C). */
static uint8_t e4m3_round(float q) {
    uint8_t sign = signbit(q) ? 0x80 : 0;
    double a = fabs((double)q);
    int e;
    if (!(a < 448.0)) return sign | 0x7e;
    if (a < ldexp(1.0, -6)) {
        e = -6;                                 /* subnormal binade, spacing 2^-9 */
    } else {
        frexp(a, &e);
        e -= 1;                                 /* a in [2^e, 2^(e+1)) */
    }
    double m = nearbyint(ldexp(a, 3 - e));      /* units of 2^(e-3), ties even */
    if (e == -6 && m < 8.0) return sign | (uint8_t)m;
    if (m >= 16.0) { m /= 2.0; e += 1; }
    if (e > 8 || (e == 8 && m > 14.0)) return sign | 0x7e;
    return sign | (uint8_t)(((e + 7) << 3) | ((int)m - 8));
}

static float load_elem(const void *x, int dt, int64_t i) {
    switch (dt) {
    case O_F32: return ((const float *)x)[i];
    case O_F16: return f16_value(((const uint16_t *)x)[i]);
    default:    return bf16_value(((const uint16_t *)x)[i]);
    }
}

static void store_elem(void *y, int dt, int64_t i, float v) {
    switch (dt) {
    case O_F32: ((float *)y)[i] = v; break;
    case O_F16: ((uint16_t *)y)[i] = f16_round(v); break;
    default:    ((uint16_t *)y)[i] = bf16_round(v); break;
    }
}

static int dtype_ok(int dt) { return dt == O_F16 || dt == O_BF16 || dt == O_F32; }
static int fmt_ok(int f) {
    return f == O_INT2 || f == O_INT4 || f == O_INT6 || f == O_INT8 || f == O_E4M3;
}
static int g_ok(int32_t G) { return G >= 1 && G <= (1 << 20); }

/* bits per code and the largest code magnitude of a payload format */
static int fmt_bits(int f) { return f == O_E4M3 ? 8 : f; }
static float fmt_qmax(int f) { return f == O_E4M3 ? 448.0f : (float)((1 << (f - 1)) - 1); }

/* ------------------------------------------------------------------------ */
/* The steps of the method.                                                 */
/* ------------------------------------------------------------------------ */

/* Block absmax [ZPP blockwise weight quantization]: exact max of |x_i|. */
static float block_absmax(const float *v, int64_t len) {
    float a = 0.0f;
    for (int64_t i = 0; i < len; i++)
        if (fabsf(v[i]) > a) a = fabsf(v[i]);
    return a;
}

/* One binary32 scale per block [AQV Eq. 6: 32 metadata bits per block]. */
static float block_scale(float absmax, int fmt) { return absmax / fmt_qmax(fmt); }

/* Signed integer code [ZPP blockwise 8-bit; AQV b in {2,4,6,8}]. */
static int int_code(float x, float s, int fmt) {
    float qmax = fmt_qmax(fmt);
    if (s == 0.0f) return 0;
    float q = x / s;
    float c = nearbyintf(q);
    if (!(c <= qmax)) c = qmax;      /* a NaN quotient (non-finite input, no */
    if (c < -qmax) c = -qmax;        /* specified code) takes qmax, not UB */
    return (int)c;
}

/* FP8 code [AGOQ QuanGrad: FP8 gradients, block scaled]. */
static uint8_t e4m3_code(float x, float s) {
    if (s == 0.0f) return 0x00;
    return e4m3_round(x / s);
}

/* Write field `f` (low b bits) as element i of an LSB-first bitstream. */
static void put_field(uint8_t *stream, int64_t i, int b, uint32_t f) {
    for (int t = 0; t < b; t++) {
        int64_t bit = (int64_t)b * i + t;
        if ((f >> t) & 1u) stream[bit >> 3] |= (uint8_t)(1u << (bit & 7));
    }
}

static uint32_t get_field(const uint8_t *stream, int64_t i, int b) {
    uint32_t f = 0;
    for (int t = 0; t < b; t++) {
        int64_t bit = (int64_t)b * i + t;
        f |= (uint32_t)((stream[bit >> 3] >> (bit & 7)) & 1u) << t;
    }
    return f;
}

/* Decoded code value (before scaling): a two's-complement field or E4M3. */
static float code_value(const uint8_t *stream, int64_t i, int fmt) {
    if (fmt == O_E4M3) return e4m3_value(stream[i]);
    int b = fmt;
    int32_t f = (int32_t)get_field(stream, i, b);
    if (f & (1 << (b - 1))) f -= (1 << b);
    return (float)f;
}

/* Payload bytes: ceil(n*b/8) code bytes plus one binary32 scale per block
 * [AQV Eq. 6: bpw = b + 32/G]. */
int64_t oracle_payload_bytes(int64_t n, int32_t bits, int32_t G) {
    if (n < 0 || G < 1 || bits < 1) return -1;
    return (n * bits + 7) / 8 + 4 * ((n + G - 1) / G);
}

/* Quantize the float values v[0..n) blockwise into `codes` (a stream of
 * ceil(n*b/8) bytes, zeroed here first) and scales[0..ceil(n/G)). */
static void quantize_values(const float *v, int64_t n, int32_t G, int fmt,
                            uint8_t *codes, float *scales) {
    int b = fmt_bits(fmt);
    memset(codes, 0, (size_t)((n * b + 7) / 8));
    for (int64_t k = 0; k * G < n; k++) {
        int64_t lo = k * G, len = (n - lo < G) ? n - lo : G;
        float s = block_scale(block_absmax(v + lo, len), fmt);
        scales[k] = s;
        for (int64_t i = lo; i < lo + len; i++) {
            if (fmt == O_E4M3)
                codes[i] = e4m3_code(v[i], s);
            else
                put_field(codes, i, b, (uint32_t)int_code(v[i], s, fmt) & ((1u << b) - 1u));
        }
    }
}

static float *widen_all(const void *x, int dt, int64_t n) {
    float *v = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!v) return NULL;
    for (int64_t i = 0; i < n; i++) v[i] = load_elem(x, dt, i);
    return v;
}

/* qwZ quantize (INT8) or FP8 quantize (E4M3) of a 16/32-bit tensor. */
int oracle_quantize_blockwise(const void *x, int xt, int64_t n, int32_t G, int fmt,
                              void *codes, float *scales) {
    if (n < 0 || !dtype_ok(xt) || !g_ok(G) || !fmt_ok(fmt)) return O_BAD;
    if (n == 0) return O_OK;
    float *v = widen_all(x, xt, n);
    if (!v) return O_BAD;
    quantize_values(v, n, G, fmt, (uint8_t *)codes, scales);
    free(v);
    return O_OK;
}

/* Aquavit sub-byte pack: the same blockwise quantizer at b in {2,4,6,8}. */
int oracle_pack_subbyte(const void *x, int xt, int64_t n, int32_t b, int32_t G,
                        uint8_t *packed, float *scales) {
    if (b != 2 && b != 4 && b != 6 && b != 8) return O_BAD;
    return oracle_quantize_blockwise(x, xt, n, G, b, packed, scales);
}

/* Dequantize [ZPP: 8-bit values travel, the receiver computes in 16 bits]:
 * y_i = cast(fl(value(c_i) * s_k)). */
int oracle_dequantize_blockwise(const void *codes, const float *scales, int fmt,
                                int64_t n, int32_t G, void *y, int yt) {
    if (n < 0 || !dtype_ok(yt) || !g_ok(G) || !fmt_ok(fmt)) return O_BAD;
    for (int64_t i = 0; i < n; i++) {
        float c = code_value((const uint8_t *)codes, i, fmt);
        store_elem(y, yt, i, c * scales[i / G]);
    }
    return O_OK;
}

int oracle_unpack_subbyte(const uint8_t *packed, const float *scales, int64_t n,
                          int32_t b, int32_t G, void *y, int yt) {
    if (b != 2 && b != 4 && b != 6 && b != 8) return O_BAD;
    return oracle_dequantize_blockwise(packed, scales, b, n, G, y, yt);
}

/* qgZ fused dequantize -> full-precision sum -> requantize [ZPP: QGZ keeps
 * reductions in full precision; kernel fusion of intra-node dequantization and
 * reduction with inter-node quantization], and AGoQ step 2 "Local Reduce"
 * [AGOQ: dequantize received FP8 to FP32, sum, requantize to FP8].
 *
 * Slice j (j = 0..N-1) holds slice_len codes at codes_in + j*stride bytes and
 * its own block scales at scales_in + j*scale_stride.  For every element i:
 *   acc = -0.0;  for j in 0..N-1:  acc = fmaf(value(c_ji), s_j[i/G], acc)
 * The sums are then quantized blockwise (same G) in fmt_out. */
int oracle_dequant_reduce_requant(const void *codes_in, int64_t in_slice_stride_bytes,
                                  const float *scales_in, int64_t in_scale_stride,
                                  int32_t n_slices, int64_t slice_len, int32_t G,
                                  int fmt_in, int fmt_out, void *codes_out,
                                  float *scales_out, float *sum_out) {
    if (slice_len < 0 || n_slices < 1 || !g_ok(G) || !fmt_ok(fmt_in) || !fmt_ok(fmt_out))
        return O_BAD;
    if (slice_len == 0) return O_OK;
    float *sum = (float *)malloc((size_t)slice_len * sizeof(float));
    if (!sum) return O_BAD;
    for (int64_t i = 0; i < slice_len; i++) {
        float acc = -0.0f;
        for (int32_t j = 0; j < n_slices; j++) {
            const uint8_t *slice = (const uint8_t *)codes_in + (int64_t)j * in_slice_stride_bytes;
            float s = scales_in[(int64_t)j * in_scale_stride + i / G];
            acc = fmaf(code_value(slice, i, fmt_in), s, acc);
        }
        sum[i] = acc;
    }
    quantize_values(sum, slice_len, G, fmt_out, (uint8_t *)codes_out, scales_out);
    if (sum_out) memcpy(sum_out, sum, (size_t)slice_len * sizeof(float));
    free(sum);
    return O_OK;
}

/* AGoQ local accumulation [AGOQ QuanGrad "Local Accumulation": dequantize the
 * FP8 main gradient to 16 bits, add the new micro-batch gradient, requantize
 * the sum to FP8], in place on (state_codes, state_scales):
 *   d_i = bf16(fl(value(e_i) * s_k));  t_i = bf16(fl(d_i + g_i));
 *   state <- E4M3 blockwise quantization of t. */
int oracle_fp8_accum_requant(uint8_t *state_codes, float *state_scales,
                             const void *grad, int gt, int64_t n, int32_t G) {
    if (n < 0 || !dtype_ok(gt) || !g_ok(G)) return O_BAD;
    if (n == 0) return O_OK;
    float *t = (float *)malloc((size_t)n * sizeof(float));
    if (!t) return O_BAD;
    for (int64_t i = 0; i < n; i++) {
        float d = bf16_value(bf16_round(e4m3_value(state_codes[i]) * state_scales[i / G]));
        t[i] = bf16_value(bf16_round(d + load_elem(grad, gt, i)));
    }
    quantize_values(t, n, G, O_E4M3, state_codes, state_scales);
    free(t);
    return O_OK;
}

/* qgZ tensor-slice reordering [ZPP: "Tensor-slice reordering fixes incorrect
 * gradient placement"; fused with the intra-node quantization per "The
 * implementation combines kernel fusion with communication overlap"].
 *
 * A rank's bucket of n elements is W = K*N chunks of C = n/W elements (K nodes,
 * N GPUs per node); chunk c is the part global rank c = node*N + gpu owns after
 * the reduce-scatter.  In the two-hop protocol [ZPP: "Two-hop communication
 * ..."] the intra-node all-to-all hands slice j of every local GPU to local GPU
 * j, which reduces them and then sends, to GPU j of each node b, the piece that
 * rank b*N + j owns.  So slice j must hold the chunks b*N + j for b = 0..K-1, in
 * node order:   y[j*K*C + b*C + i] = x[(b*N + j)*C + i].
 * Reading: the pages show the reordering only by example; this is the
 * permutation that makes the two hops deliver chunk c to rank c (pinned by a
 * simulation of the two hops on virtual ranks). */
int oracle_reorder_slices(const void *x, int xt, int64_t n, int32_t n_nodes,
                          int32_t gpus_per_node, void *y) {
    if (n < 0 || !dtype_ok(xt) || n_nodes < 1 || gpus_per_node < 1) return O_BAD;
    int64_t W = (int64_t)n_nodes * gpus_per_node;
    if (n % W != 0) return O_BAD;
    int64_t C = n / W, esz = xt == O_F32 ? 4 : 2;
    for (int64_t j = 0; j < gpus_per_node; j++)
        for (int64_t b = 0; b < n_nodes; b++)
            memcpy((uint8_t *)y + (j * n_nodes * C + b * C) * esz,
                   (const uint8_t *)x + ((b * gpus_per_node + j) * C) * esz, (size_t)(C * esz));
    return O_OK;
}

/* The sender side of qgZ: reorder, then quantize each of the N slices on its
 * own (blocks restart at each slice).  Slice j's codes go to
 * codes + j*slice_stride_bytes, its scales to scales + j*scale_stride. */
int oracle_reorder_quantize(const void *x, int xt, int64_t n, int32_t n_nodes,
                            int32_t gpus_per_node, int32_t G, int fmt, void *codes,
                            int64_t slice_stride_bytes, float *scales, int64_t scale_stride) {
    if (n < 0 || !dtype_ok(xt) || !g_ok(G) || !fmt_ok(fmt) || n_nodes < 1 || gpus_per_node < 1)
        return O_BAD;
    int64_t W = (int64_t)n_nodes * gpus_per_node;
    if (n % W != 0) return O_BAD;
    if (n == 0) return O_OK;
    int64_t L = n / gpus_per_node, esz = xt == O_F32 ? 4 : 2;
    uint8_t *y = (uint8_t *)malloc((size_t)(n * esz));
    if (!y) return O_BAD;
    int rc = oracle_reorder_slices(x, xt, n, n_nodes, gpus_per_node, y);
    for (int64_t j = 0; rc == O_OK && j < gpus_per_node; j++)
        rc = oracle_quantize_blockwise(y + j * L * esz, xt, L, G, fmt,
                                       (uint8_t *)codes + j * slice_stride_bytes,
                                       scales + j * scale_stride);
    free(y);
    return rc;
}

/* Aquavit ascending precision schedule [AQV: key idea, Section 5.1 -- the
 * target effective bits per weight rise as bpw(t) = 8 - 6/(a + c*t/T), with
 * (a, c) = (0.9, 5) by default; granularity modulation realizes a target with
 * b in {2,4,6,8} and a block size G, bpw = b + 32/G (Eq. 6, Table 1), G from
 * 1024 down to 32].  Reading: the level used at step t is the (b, G) whose
 * b + 32/G is nearest to bpw(t) among b in {2,4,6,8}, G in {32, 64, ..., 1024};
 * on a tie the smaller bpw (fewer bytes) wins. */
double oracle_aquavit_target(int64_t t, int64_t T, double a, double c) {
    return 8.0 - 6.0 / (a + c * (double)t / (double)T);
}

int oracle_aquavit_level(int64_t t, int64_t T, double a, double c, int32_t *b_out,
                         int32_t *G_out) {
    if (T <= 0 || t < 0 || t > T) return O_BAD;
    double target = oracle_aquavit_target(t, T, a, c);
    double best_d = 1e300, best_bpw = 0.0;
    for (int b = 2; b <= 8; b += 2) {
        for (int G = 32; G <= 1024; G *= 2) {
            double bpw = b + 32.0 / G;
            double d = fabs(bpw - target);
            if (d < best_d || (d == best_d && bpw < best_bpw)) {
                best_d = d;
                best_bpw = bpw;
                *b_out = b;
                *G_out = G;
            }
        }
    }
    return O_OK;
}

/* Metadata interleaving [AQV Section 5.2]: the payload as one record per
 * block -- the block's fp32 scale (4 bytes, little-endian) followed by the
 * block's own b-bit code stream (ceil(len*b/8) bytes, LSB-first as above) --
 * records back to back.  Reading: scale first, no padding, so the stream has
 * exactly payload_bytes(n, b, G) bytes, the same as codes and scales apart. */
int oracle_pack_records(const void *x, int xt, int64_t n, int32_t b, int32_t G,
                        uint8_t *records) {
    if (n < 0 || (b != 2 && b != 4 && b != 6 && b != 8) || !g_ok(G) || (G * b) % 8) return O_BAD;
    if (n == 0) return O_OK;
    int64_t nb = (n + G - 1) / G, cb = (n * b + 7) / 8;
    uint8_t *codes = (uint8_t *)malloc((size_t)cb);
    float *scales = (float *)malloc((size_t)nb * sizeof(float));
    int rc = (codes && scales) ? oracle_pack_subbyte(x, xt, n, b, G, codes, scales) : O_BAD;
    for (int64_t k = 0; rc == O_OK && k < nb; k++) {
        int64_t len = (n - k * G < G) ? n - k * G : G;
        uint8_t *rec = records + k * (4 + (int64_t)G * b / 8);
        memcpy(rec, &scales[k], 4);
        memcpy(rec + 4, codes + k * (int64_t)G * b / 8, (size_t)((len * b + 7) / 8));
    }
    free(codes);
    free(scales);
    return rc;
}

int oracle_unpack_records(const uint8_t *records, int64_t n, int32_t b, int32_t G, void *y,
                          int yt) {
    if (n < 0 || (b != 2 && b != 4 && b != 6 && b != 8) || !g_ok(G) || (G * b) % 8) return O_BAD;
    if (n == 0) return O_OK;
    int64_t nb = (n + G - 1) / G, cb = (n * b + 7) / 8;
    uint8_t *codes = (uint8_t *)calloc((size_t)cb, 1);
    float *scales = (float *)malloc((size_t)nb * sizeof(float));
    int rc = (codes && scales) ? O_OK : O_BAD;
    for (int64_t k = 0; rc == O_OK && k < nb; k++) {
        int64_t len = (n - k * G < G) ? n - k * G : G;
        const uint8_t *rec = records + k * (4 + (int64_t)G * b / 8);
        memcpy(&scales[k], rec, 4);
        memcpy(codes + k * (int64_t)G * b / 8, rec + 4, (size_t)((len * b + 7) / 8));
    }
    if (rc == O_OK) rc = oracle_unpack_subbyte(codes, scales, n, b, G, y, yt);
    free(codes);
    free(scales);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Format conversions exposed for pinning the oracle's own converters.      */
/* ------------------------------------------------------------------------ */

void oracle_f32_to_f16(const float *x, int64_t n, uint16_t *y) {
    for (int64_t i = 0; i < n; i++) y[i] = f16_round(x[i]);
}
void oracle_f32_to_bf16(const float *x, int64_t n, uint16_t *y) {
    for (int64_t i = 0; i < n; i++) y[i] = bf16_round(x[i]);
}
void oracle_f16_to_f32(const uint16_t *x, int64_t n, float *y) {
    for (int64_t i = 0; i < n; i++) y[i] = f16_value(x[i]);
}
void oracle_f32_to_e4m3(const float *x, int64_t n, uint8_t *y) {
    for (int64_t i = 0; i < n; i++) y[i] = e4m3_round(x[i]);
}
void oracle_e4m3_to_f32(const uint8_t *x, int64_t n, float *y) {
    for (int64_t i = 0; i < n; i++) y[i] = e4m3_value(x[i]);
}
