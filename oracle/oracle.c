/*
 * oracle.c -- plain, slow, fp64 CPU reference for the fused QK / KV
 * RMSNorm + RoPE (+ cache) operators.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header, table or helper with the HIP
 * kernels.
 *
 * Sources (cited by page title and section):
 *   [qkv_cte]  "Kernel reference: qkv_cte -- Wan2.2 additions to the NKI Library
 *              QKV CTE MXFP8 projection", Design section 1 (across-heads QK
 *              RMSNorm, steps a-c) and section 2 (bundled rotate-half RoPE,
 *              its `out = ...` expression and the lane pairing (i, i+d/2)).
 *   [CP]       "Context Parallelism in vLLM Omni Neuron", the WanSelfAttention
 *              forward listing (norm_q / norm_k before the rotary embedding)
 *              and "Distributed Normalization".
 *   [KVRNRC]   "KvRmsNormRopeCache" (CANN ops-transformer), section
 *              "function description -> formulas" (1) RmsNorm, (2) interleaveRope,
 *              (3) quantisation, (4) scatter, (5) raw outputs; the parameter
 *              table; the constraint tables for cache_mode / index.
 *
 * Everything is evaluated in IEEE double on the exactly decoded inputs and
 * rounded once at the end. Where the pages leave a point open, the reading
 * taken is stated at the function that depends on it.
 *
 * Every function here is pinned by tests/test_oracle_pins.py against closed
 * forms, hand cases, library special cases and an independent pure-Python
 * brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* storage type codes used by the oracle's own wrapper (oracle/__init__.py) */
enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2, ORC_F16 = 3, ORC_INT8 = 4, ORC_E4M3FN = 5, ORC_E5M2 = 6 };
enum { ORC_NORM = 0, ORC_PA_BNSD = 1, ORC_PA_BLK_BNSD = 2 };

/* ------------------------------------------------------------------------ */
/* Format definitions: decode (exact) and encode (round to nearest, ties to  */
/* even, written from the format definitions with frexp/ldexp/nearbyint).   */
/* ------------------------------------------------------------------------ */

/* bfloat16 = the upper 16 bits of an IEEE binary32 */
static double dec_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits */
static double dec_f16(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1024.0 + m, e - 25);
    return s ? -v : v;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa; no inf; S.1111.111 is NaN */
static double dec_e4m3fn(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(8.0 + m, e - 10);
    return s ? -v : v;
}

/* OCP FP8 E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa; IEEE-like: exponent
 * 31 holds inf (mantissa 0) and NaN */
static double dec_e5m2(uint8_t c) {
    int s = c >> 7, e = (c >> 2) & 31, m = c & 3;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -16);
    else v = ldexp(4.0 + m, e - 17);
    return s ? -v : v;
}

/*
 * Round |x| to a binary format with `p` significant bits, minimum normal
 * exponent `emin` (value 2^emin) and subnormals spaced 2^(emin-p+1):
 * the quantum of the binade that holds |x| is 2^(E-p+1), E = floor(log2|x|),
 * floored at the subnormal quantum. nearbyint rounds half to even in the
 * default rounding mode.
 */
static double round_to_format(double a, int p, int emin) {
    if (a == 0.0) return 0.0;
    int e;
    frexp(a, &e);              /* a = m * 2^e, m in [0.5, 1) -> E = e - 1 */
    int E = e - 1;
    if (E < emin) E = emin;
    double q = ldexp(1.0, E - p + 1);
    return nearbyint(a / q) * q;
}

static uint16_t enc_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    double a = fabs(x);
    double r = round_to_format(a, 8, -126);
    uint16_t s = signbit(x) ? 0x8000 : 0;
    /* largest finite bf16 is (2 - 2^-7) * 2^127; a value rounding past it is inf */
    if (r > ldexp(255.0, 120)) return s | 0x7F80;
    float f = (float)r;        /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return s | (uint16_t)(u >> 16);
}

static uint16_t enc_f16(double x) {
    if (isnan(x)) return 0x7E00;
    double a = fabs(x);
    double r = round_to_format(a, 11, -14);
    uint16_t s = signbit(x) ? 0x8000 : 0;
    if (r > 65504.0) return s | 0x7C00;
    if (r < ldexp(1.0, -14)) return s | (uint16_t)(r / ldexp(1.0, -24));  /* subnormal field */
    int e;
    double m = frexp(r, &e);   /* r = m * 2^e, m in [0.5,1) */
    int E = e - 1;
    uint16_t mant = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
    return s | (uint16_t)((E + 15) << 10) | mant;
}

/* saturating E4M3FN encoder: |x| at or above the largest finite (448) -> 448 */
static uint8_t enc_e4m3fn(double x) {
    if (isnan(x)) return 0x7F;
    uint8_t s = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0) return s | 0x7E;
    double r = round_to_format(a, 4, -6);
    if (r >= 448.0) return s | 0x7E;
    if (r < ldexp(1.0, -6)) return s | (uint8_t)(r / ldexp(1.0, -9));   /* subnormal field */
    int e;
    double m = frexp(r, &e);
    int E = e - 1;
    uint8_t mant = (uint8_t)((m * 2.0 - 1.0) * 8.0);
    return s | (uint8_t)((E + 7) << 3) | mant;
}

/* saturating E5M2 encoder: |x| at or above the largest finite (57344) -> 57344 */
static uint8_t enc_e5m2(double x) {
    if (isnan(x)) return 0x7F;
    uint8_t s = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 57344.0) return s | 0x7B;
    double r = round_to_format(a, 3, -14);
    if (r >= 57344.0) return s | 0x7B;
    if (r < ldexp(1.0, -14)) return s | (uint8_t)(r / ldexp(1.0, -16));  /* subnormal field */
    int e;
    double m = frexp(r, &e);
    int E = e - 1;
    uint8_t mant = (uint8_t)((m * 2.0 - 1.0) * 4.0);
    return s | (uint8_t)((E + 15) << 2) | mant;
}

static double load(int dtype, const void *p, int64_t i) {
    switch (dtype) {
    case ORC_F64: return ((const double *)p)[i];
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_BF16: return dec_bf16(((const uint16_t *)p)[i]);
    case ORC_F16: return dec_f16(((const uint16_t *)p)[i]);
    case ORC_INT8: return (double)((const int8_t *)p)[i];
    case ORC_E4M3FN: return dec_e4m3fn(((const uint8_t *)p)[i]);
    case ORC_E5M2: return dec_e5m2(((const uint8_t *)p)[i]);
    }
    return NAN;
}

/* Round once from the exact value to the storage type (RNE). */
static void store(int dtype, void *p, int64_t i, double v) {
    switch (dtype) {
    case ORC_F64: ((double *)p)[i] = v; break;
    case ORC_F32: ((float *)p)[i] = (float)v; break;     /* IEEE cast: RNE */
    case ORC_BF16: ((uint16_t *)p)[i] = enc_bf16(v); break;
    case ORC_F16: ((uint16_t *)p)[i] = enc_f16(v); break;
    default: break;
    }
}

/* exported codec entry points (pinned by the codebook tests) */
void oracle_decode(int dtype, const void *src, double *dst, int64_t n) {
    for (int64_t i = 0; i < n; i++) dst[i] = load(dtype, src, i);
}

void oracle_encode(int dtype, const double *src, void *dst, int64_t n) {
    for (int64_t i = 0; i < n; i++) {
        if (dtype == ORC_E4M3FN) ((uint8_t *)dst)[i] = enc_e4m3fn(src[i]);
        else if (dtype == ORC_E5M2) ((uint8_t *)dst)[i] = enc_e5m2(src[i]);
        else store(dtype, dst, i, src[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* (a) across-heads RMSNorm + rotate-half RoPE                               */
/* ------------------------------------------------------------------------ */

/*
 * One segment (all heads of Q, or all heads of K) of one token.
 *
 * [qkv_cte] section 1: one RMS over the whole segment of n_heads*d_head
 * channels (step b: inv_rms = 1/sqrt(sum(x^2)/(n_heads*d_head*tp) + eps);
 * with all heads resident tp = 1 and the sum is this segment's own), then the
 * per-channel segment-wide gamma (step c). When the heads are split over tp
 * ranks, step a gives each rank the sum over its own heads, step b adds the
 * ranks' sums, and step c applies with the added sum and the whole segment's
 * channel count: `given_ss` / `channels` are that sum and count.
 * [qkv_cte] "Upstream behavior" and section 1: the upstream qk-norm is per
 * head instead -- each head's d_head slice normalised by its own RMS, with a
 * per-head [d_head] gamma shared by every head (`per_head`).
 * [CP] forward listing: the norm runs before the rotary embedding.
 * [qkv_cte] section 2: rotate-half RoPE per head, lanes i and i+d/2 paired,
 * out = y*cos + [-y_hi, y_lo]*sin with cos/sin indexed by the output lane
 * and shared by every head of the token. Folding inv_rms into the cos/sin
 * products is an evaluation order, not a different result, so the
 * definition is written here as norm-then-rotate.
 */
static void qk_segment(int64_t nh, int64_t d, int dtype, const void *x, int64_t x0,
                       const void *gamma, const void *cs, const void *sn, int64_t r0,
                       double eps, int apply_norm, int apply_rope, int per_head,
                       const double *given_ss, double channels, double *y, double *out) {
    int64_t C = nh * d, h2 = d / 2;
    if (!apply_norm) {
        for (int64_t c = 0; c < C; c++) y[c] = load(dtype, x, x0 + c);
    } else if (per_head) {
        for (int64_t h = 0; h < nh; h++) {
            double ss = 0.0;
            for (int64_t i = 0; i < d; i++) {
                double v = load(dtype, x, x0 + h * d + i);
                ss += v * v;
            }
            double inv_rms = 1.0 / sqrt(ss / (double)d + eps);
            for (int64_t i = 0; i < d; i++)
                y[h * d + i] = load(dtype, x, x0 + h * d + i) * inv_rms * load(dtype, gamma, i);
        }
    } else {
        double ss = 0.0;
        if (given_ss) {
            ss = *given_ss;
        } else {
            for (int64_t c = 0; c < C; c++) {
                double v = load(dtype, x, x0 + c);
                ss += v * v;
            }
        }
        double inv_rms = 1.0 / sqrt(ss / (channels > 0 ? channels : (double)C) + eps);
        for (int64_t c = 0; c < C; c++)
            y[c] = load(dtype, x, x0 + c) * inv_rms * load(dtype, gamma, c);
    }
    for (int64_t h = 0; h < nh; h++) {
        const double *yh = y + h * d;
        double *oh = out + h * d;
        for (int64_t i = 0; i < d; i++) {
            if (!apply_rope) {
                oh[i] = yh[i];
                continue;
            }
            double rot = (i < h2) ? -yh[i + h2] : yh[i - h2];    /* [-y_hi, y_lo] */
            oh[i] = yh[i] * load(dtype, cs, r0 + i) + rot * load(dtype, sn, r0 + i);
        }
    }
}

/*
 * q: [T, n_q*d], k: [T, n_k*d] (NULL when n_k == 0), contiguous rows; gammas
 * [n*d] (across heads) or [d] (per head); cos/sin [T, d]. q_sumsq/k_sumsq [T]
 * (or NULL): sums of squares to use instead of this call's own (the apply
 * step of a split over ranks), with q_channels/k_channels the whole
 * segment's channel count (<= 0: n*d). Writes q_out/k_out in `dtype` (rounded
 * once) and, if given, the exact results q_val/k_val. Returns 0, or -1 on bad
 * dimensions.
 */
int oracle_qk_norm_rope(int64_t T, int64_t n_q, int64_t n_k, int64_t d, int dtype,
                        const void *q, const void *k, const void *q_gamma,
                        const void *k_gamma, const void *cs, const void *sn, double eps,
                        int apply_norm, int apply_rope, int per_head,
                        const double *q_sumsq, const double *k_sumsq, double q_channels,
                        double k_channels, void *q_out, void *k_out, double *q_val,
                        double *k_val, int nthreads) {
    if (T < 0 || n_q < 1 || n_k < 0 || d < 2 || (d & 1)) return -1;
    if (per_head && (q_sumsq || k_sumsq)) return -1;
    int64_t cq = n_q * d, ck = n_k * d;
    int64_t cmax = cq > ck ? cq : ck;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
    {
        double *y = (double *)malloc(sizeof(double) * cmax);
        double *o = (double *)malloc(sizeof(double) * cmax);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; t++) {
            for (int seg = 0; seg < 2; seg++) {
                int64_t nh = seg == 0 ? n_q : n_k;
                if (nh == 0) continue;
                int64_t C = nh * d;
                const void *x = seg == 0 ? q : k;
                const void *g = seg == 0 ? q_gamma : k_gamma;
                const double *given = seg == 0 ? q_sumsq : k_sumsq;
                double channels = seg == 0 ? q_channels : k_channels;
                void *dst = seg == 0 ? q_out : k_out;
                double *val = seg == 0 ? q_val : k_val;
                qk_segment(nh, d, dtype, x, t * C, g, cs, sn, t * d, eps, apply_norm,
                           apply_rope, per_head, given ? given + t : NULL, channels, y, o);
                for (int64_t c = 0; c < C; c++) {
                    if (dst) store(dtype, dst, t * C + c, o[c]);
                    if (val) val[t * C + c] = o[c];
                }
            }
        }
        free(y);
        free(o);
    }
    return 0;
}

/* The across-heads operator with every head on one device (tp = 1). */
int oracle_qk_norm_rope_across_heads(int64_t T, int64_t n_q, int64_t n_k, int64_t d,
                                     int dtype, const void *q, const void *k,
                                     const void *q_gamma, const void *k_gamma,
                                     const void *cs, const void *sn, double eps,
                                     int apply_norm, int apply_rope, void *q_out,
                                     void *k_out, double *q_val, double *k_val,
                                     int nthreads) {
    return oracle_qk_norm_rope(T, n_q, n_k, d, dtype, q, k, q_gamma, k_gamma, cs, sn, eps,
                               apply_norm, apply_rope, 0, NULL, NULL, 0.0, 0.0, q_out, k_out,
                               q_val, k_val, nthreads);
}

/*
 * [qkv_cte] section 1, step a: each token's sum of x^2 over one segment of
 * n*d channels, x: [T, n*d] contiguous. Writes sumsq[T].
 */
int oracle_qk_sumsq(int64_t T, int64_t n, int64_t d, int dtype, const void *x,
                    double *sumsq) {
    if (T < 0 || n < 1 || d < 1) return -1;
    for (int64_t t = 0; t < T; t++) {
        double ss = 0.0;
        for (int64_t c = 0; c < n * d; c++) {
            double v = load(dtype, x, t * n * d + c);
            ss += v * v;
        }
        sumsq[t] = ss;
    }
    return 0;
}

/*
 * [qkv_cte] "Upstream behavior" and "Interface": the projection that produces
 * Q|K|V, O[S, I] = A[S, H] @ W[H, I] (+ bias), with the ROW_MX dequantisation
 * of the same page (a per-row activation scale and a per-output-channel weight
 * scale) when the operands are FP8 codes:
 *   O[s, i] = (sum_h A[s, h] * W[i, h]) * a_scale[s] * w_scale[i] + bias[i].
 * W is passed as [I, H] (one row per output channel, the layout of a linear
 * layer's weight). A scale or the bias may be NULL (1 and 0). The sum is
 * evaluated in fp64 over h in order; O is rounded once to out_dtype and, if
 * o_val is given, also returned exactly. Returns 0, or -1 on bad sizes.
 */
int oracle_linear(int64_t S, int64_t H, int64_t I, int a_dtype, const void *A, int w_dtype,
                  const void *W, const void *bias, int bias_dtype, const double *a_scale,
                  const double *w_scale, int out_dtype, void *O, double *o_val, int nthreads) {
    if (S < 0 || H < 1 || I < 1) return -1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t s = 0; s < S; s++) {
        for (int64_t i = 0; i < I; i++) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; h++)
                acc += load(a_dtype, A, s * H + h) * load(w_dtype, W, i * H + h);
            if (a_scale) acc *= a_scale[s];
            if (w_scale) acc *= w_scale[i];
            if (bias) acc += load(bias_dtype, bias, i);
            if (O) store(out_dtype, O, s * I + i, acc);
            if (o_val) o_val[s * I + i] = acc;
        }
    }
    return 0;
}

/* E8M0 (OCP Microscaling shared scale): an unsigned biased exponent, value
 * 2^(e - 127); 255 is NaN. */
static double dec_e8m0(uint8_t e) {
    return e == 255 ? NAN : ldexp(1.0, (int)e - 127);
}

/*
 * [qkv_cte] "Upstream behavior" names MXFP8 among the projection's
 * quantisation modes without defining it; read as the OCP Microscaling (MX)
 * format: FP8 E4M3 elements in blocks of 32 consecutive values along the
 * contraction axis, each block with one E8M0 scale, element value = code *
 * 2^(e - 127). For the projection both operands are MX along H:
 *   O[s, i] = (sum_h A[s, h] * X(a_bs[s, h / 32]) * W[i, h] * X(w_bs[i, h / 32]))
 *             * a_scale[s] * w_scale[i] + bias[i],
 * a_bs [S, H/32] and w_bs [I, H/32] E8M0 bytes (row strides a_bs_stride,
 * w_bs_stride), the ROW_MX scales optional (NULL = 1) as in oracle_linear.
 * H must be a multiple of 32. Evaluated in fp64 over h in order; O rounded
 * once to out_dtype; o_val (if given) the exact value. Returns 0 or -1.
 */
int oracle_linear_mx(int64_t S, int64_t H, int64_t I, const void *A, const void *W, const uint8_t *a_bs,
                     int64_t a_bs_stride, const uint8_t *w_bs, int64_t w_bs_stride, const void *bias,
                     int bias_dtype, const double *a_scale, const double *w_scale, int out_dtype, void *O,
                     double *o_val, int nthreads) {
    if (S < 0 || H < 32 || H % 32 || I < 1 || a_bs_stride < H / 32 || w_bs_stride < H / 32) return -1;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t s = 0; s < S; s++) {
        for (int64_t i = 0; i < I; i++) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; h++) {
                double a = load(ORC_E4M3FN, A, s * H + h) * dec_e8m0(a_bs[s * a_bs_stride + h / 32]);
                double w = load(ORC_E4M3FN, W, i * H + h) * dec_e8m0(w_bs[i * w_bs_stride + h / 32]);
                acc += a * w;
            }
            if (a_scale) acc *= a_scale[s];
            if (w_scale) acc *= w_scale[i];
            if (bias) acc += load(bias_dtype, bias, i);
            if (O) store(out_dtype, O, s * I + i, acc);
            if (o_val) o_val[s * I + i] = acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* (b) KvRmsNormRopeCache                                                     */
/* ------------------------------------------------------------------------ */

/*
 * [KVRNRC] formula (3): x*scale if a scale is given, then +offset if an
 * offset is given; with any quantisation the value is rounded (half to even,
 * as torch.round does) and clamped to [-128, 127] for INT8. For FLOAT8E4M3FN
 * and FLOAT8E5M2 the pages give no separate formula; the value is cast to the
 * format with round to nearest even, saturating at its largest finite value
 * (+-448, +-57344). Every decision is taken on the exact t, with no
 * intermediate rounding: formula (3) has none.
 * Returns t (the exact pre-rounding value) and writes the code.
 */
static double quantise(int cdtype, void *cache, int64_t pos, double x,
                       const double *scale, const double *offset, int64_t qi) {
    double t = x;
    if (scale) t = t * scale[qi];
    if (offset) t = t + offset[qi];
    if (cdtype == ORC_INT8) {
        double r = nearbyint(t);
        if (r < -128.0) r = -128.0;
        if (r > 127.0) r = 127.0;
        ((int8_t *)cache)[pos] = (int8_t)r;
    } else if (cdtype == ORC_E4M3FN) {
        ((uint8_t *)cache)[pos] = enc_e4m3fn(t);
    } else if (cdtype == ORC_E5M2) {
        ((uint8_t *)cache)[pos] = enc_e5m2(t);
    } else {
        store(cdtype, cache, pos, t);
    }
    return t;
}

/*
 * Dimensions (the parameter table and the V1/V2 scenario table of [KVRNRC]):
 *   kv [B, N, S, Dkv]; V1 (v == NULL): rms over kv[..., :rms_size], RoPE on the
 *   raw kv[..., rms_size:] (rope_size = Dkv - rms_size wide).
 *   V2 (v != NULL, [B, N, S, Dv]): rms over all of kv (rms_size = Dkv), RoPE on
 *   the first rope_size normed values, which are overwritten.
 *   gamma [rms_size]; cos/sin [B, N, rope_S, rope_size], rope_S == S (or 1:
 *   the S-axis broadcast the constraint tables allow).
 *   index: Norm [B, S] rows of batch b's cache slab, in [-1, Scache);
 *          PA_BNSD [B*S] global slots in [-1, block_num*block_size);
 *          PA_BLK_BNSD [B*ceil(S/block_size)]: the starting slot of each run
 *          of block_size consecutive tokens of a batch; token s of batch b
 *          goes to slot index[b*ceil(S/bs) + s/bs] + s%bs.
 *   Caches: Norm [B, N, Scache, D]; PA_BNSD and PA_BLK_BNSD
 *   [block_num, block_size, N, D] (the shape the cache/index table gives).
 *   k width Dk_out = rope_size (V1) or Dkv (V2); ckv width Dc = rms_size (V1)
 *   or Dv (V2).
 *   k_scale/k_offset [N, Dk_out], v_scale/v_offset [N, Dc] fp64 or NULL (the
 *   wrapper broadcasts [1], [D], [1, D] to [N, D]).
 *   index == -1, or a slot outside the cache: the token writes no cache row
 *   (the pages allow -1 without saying what it does; skipping the token's
 *   cache rows is the plainest reading, and the raw outputs are still written).
 * Outputs: caches updated in place; k_rope/c_kv (if out_kv) in in_dtype;
 * optional exact values: k_x/c_x (the values fed to Quant) and k_t/c_t (the
 * values right before rounding, = x*scale+offset, or x without quantisation).
 * Returns 0, or -1 on bad dimensions.
 */
int oracle_kv_rmsnorm_rope_cache(
    int64_t B, int64_t N, int64_t S, int64_t Dkv, int64_t rms_size, int64_t rope_size,
    int64_t Dv, int in_dtype, const void *kv, const void *v, const void *gamma,
    const void *cs, const void *sn, int64_t rope_S, const int64_t *index,
    int cache_mode, int64_t cache_dim0, int64_t block_size, int k_dtype,
    int ckv_dtype, void *k_cache, void *ckv_cache, const double *k_scale,
    const double *k_offset, const double *v_scale, const double *v_offset,
    double eps, int out_kv, void *k_rope, void *c_kv, double *k_x, double *c_x,
    double *k_t, double *c_t, int nthreads) {
    int v2 = v != NULL;
    if (B < 1 || N < 1 || S < 1 || rope_size < 2 || (rope_size & 1)) return -1;
    if (!v2 && rms_size + rope_size != Dkv) return -1;
    if (v2 && (rms_size != Dkv || rope_size > Dkv || Dv < 1)) return -1;
    if (rope_S != S && rope_S != 1) return -1;
    if (cache_mode != ORC_NORM && block_size < 1) return -1;
    int64_t Dk_out = v2 ? Dkv : rope_size;
    int64_t Dc = v2 ? Dv : rms_size;
    int64_t half = rope_size / 2;
    if (nthreads < 1) nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        double *y = (double *)malloc(sizeof(double) * rms_size);
        double *rope_out = (double *)malloc(sizeof(double) * Dk_out);
        double *c_src = (double *)malloc(sizeof(double) * Dc);
        double *z = (double *)malloc(sizeof(double) * rope_size);
#pragma omp for schedule(static)
        for (int64_t row = 0; row < B * N * S; row++) {
            int64_t b = row / (N * S), n = (row / S) % N, s = row % S;
            int64_t kv0 = row * Dkv;

            /* (1) RmsNorm over the first rms_size values of the kv row */
            double ss = 0.0;
            for (int64_t i = 0; i < rms_size; i++) {
                double xi = load(in_dtype, kv, kv0 + i);
                ss += xi * xi;
            }
            double rms = sqrt(ss / (double)rms_size + eps);
            for (int64_t i = 0; i < rms_size; i++)
                y[i] = load(in_dtype, kv, kv0 + i) / rms * load(in_dtype, gamma, i);

            /* (2) interleaveRope: the input is the raw tail (V1) or the first
             * rope_size normed values (V2); x1 = even lanes, x2 = odd lanes,
             * out = cat(x1, x2)*cos + cat(-x2, x1)*sin, cos/sin indexed by the
             * output lane. */
            for (int64_t i = 0; i < rope_size; i++)
                z[i] = v2 ? y[i] : load(in_dtype, kv, kv0 + rms_size + i);
            int64_t r0 = ((b * N + n) * rope_S + (rope_S == 1 ? 0 : s)) * rope_size;
            for (int64_t j = 0; j < rope_size; j++) {
                double p1 = j < half ? z[2 * j] : z[2 * (j - half) + 1];
                double p2 = j < half ? -z[2 * j + 1] : z[2 * (j - half)];
                rope_out[j] = p1 * load(in_dtype, cs, r0 + j) + p2 * load(in_dtype, sn, r0 + j);
            }
            /* V2: rope_out = concat(y_rope, RmsNorm(x)[rope_size:]) */
            for (int64_t j = rope_size; j < Dk_out; j++) rope_out[j] = y[j];

            /* what goes to the ckv cache: RmsNorm(x) (V1) or v_optional (V2) */
            for (int64_t i = 0; i < Dc; i++)
                c_src[i] = v2 ? load(in_dtype, v, row * Dv + i) : y[i];

            /* (4) scatter slot for token (b, s): Norm's index is [B, S] and
             * PA_BNSD's is [B*S], the same flat position b*S + s; PA_BLK_BNSD
             * holds one starting slot per block_size tokens of a batch */
            int64_t slot, capacity;
            if (cache_mode == ORC_PA_BLK_BNSD) {
                int64_t nblk = (S + block_size - 1) / block_size;
                int64_t start = index[b * nblk + s / block_size];
                slot = start < 0 ? -1 : start + s % block_size;
            } else {
                slot = index[b * S + s];
            }
            capacity = cache_mode == ORC_NORM ? cache_dim0 : cache_dim0 * block_size;
            int64_t krow = -1, crow = -1;   /* first element of the cache row */
            if (slot >= 0 && slot < capacity) {
                if (cache_mode == ORC_NORM) {
                    int64_t r = (b * N + n) * cache_dim0 + slot;      /* [B, N, Scache, D] */
                    krow = r * Dk_out;
                    crow = r * Dc;
                } else {
                    int64_t blk = slot / block_size, off = slot % block_size;
                    int64_t r = (blk * block_size + off) * N + n;     /* [blocks, bs, N, D] */
                    krow = r * Dk_out;
                    crow = r * Dc;
                }
            }
            int kq = k_scale != NULL, cq = v_scale != NULL;
            for (int64_t j = 0; j < Dk_out; j++) {
                double t = rope_out[j];
                if (kq) {
                    t = t * k_scale[n * Dk_out + j];
                    if (k_offset) t = t + k_offset[n * Dk_out + j];
                }
                if (krow >= 0)
                    quantise(k_dtype, k_cache, krow + j, rope_out[j], kq ? k_scale : NULL,
                             kq ? k_offset : NULL, n * Dk_out + j);
                if (k_x) k_x[row * Dk_out + j] = rope_out[j];
                if (k_t) k_t[row * Dk_out + j] = t;
                /* (5) raw outputs */
                if (out_kv && k_rope) store(in_dtype, k_rope, row * Dk_out + j, rope_out[j]);
            }
            for (int64_t i = 0; i < Dc; i++) {
                double t = c_src[i];
                if (cq) {
                    t = t * v_scale[n * Dc + i];
                    if (v_offset) t = t + v_offset[n * Dc + i];
                }
                if (crow >= 0)
                    quantise(ckv_dtype, ckv_cache, crow + i, c_src[i], cq ? v_scale : NULL,
                             cq ? v_offset : NULL, n * Dc + i);
                if (c_x) c_x[row * Dc + i] = c_src[i];
                if (c_t) c_t[row * Dc + i] = t;
                if (out_kv && c_kv) store(in_dtype, c_kv, row * Dc + i, c_src[i]);
            }
        }
        free(y);
        free(rope_out);
        free(c_src);
        free(z);
    }
    return 0;
}
