/*
 * qknr.h -- C ABI of the fused QK / KV RMSNorm + RoPE (+ KV-cache scatter)
 * library for AMD Instinct MI355X (gfx950).
 *
 * Operators, each one kernel launch on the caller's HIP stream:
 *
 *   qknr_qk_norm_rope_across_heads  -- per-token RMSNorm over the whole Q
 *       segment (and, separately, the whole K segment) of n_heads*d_head
 *       channels, segment-wide gamma, then rotate-half RoPE per head with the
 *       inverse RMS folded into the rotation; V is never read or written.
 *       Defined by "Kernel reference: qkv_cte -- Wan2.2 additions to the NKI
 *       Library QKV CTE MXFP8 projection", Design section 1 (across-heads QK
 *       RMSNorm, steps a-c, here with every head on one GPU) and section 2
 *       (bundled rotate-half RoPE), and by the WanSelfAttention forward of
 *       "Context Parallelism in vLLM Omni Neuron" (norm before rotary).
 *   qknr_qk_sumsq_across_heads / qknr_qk_apply_across_heads  -- the same
 *       operator when a segment's heads are split over ranks: step a (sums of
 *       squares over this rank's heads) and step c (apply with the sums added
 *       over every rank); the caller adds the sums in between (all-reduce).
 *   qknr_qk_norm_rope_per_head  -- the upstream per-head qk-norm the same page
 *       contrasts with ("Upstream behavior"): one RMS per head, [d_head] gamma.
 *   qknr_interleaved_to_rotate_half  -- the offline lane permutation that turns
 *       an interleaved-pair checkpoint (weights, bias, gamma, cos/sin) into the
 *       rotate-half layout the kernels use (qkv_cte Design section 2).
 *   qknr_qkv_projection  -- the QKV projection GEMM (matrix cores) with step a
 *       of the across-heads norm in its epilogue (qkv_cte Design section 1).
 *
 *   qknr_kv_rmsnorm_rope_cache  -- the MLA operator of the CANN page
 *       "KvRmsNormRopeCache": RmsNorm (formula 1), interleaveRope (formula 2),
 *       static quantisation (formula 3), index scatter into k_cache/ckv_cache
 *       (formula 4) and optional raw outputs k_rope/c_kv (formula 5), with the
 *       parameter table and the constraint tables of that page.
 *
 * Conventions for every call:
 *   - Status: 0 OK; 1 INVALID_ARGUMENT (a constraint of the pages or of this
 *     ABI is violated; nothing is launched); 2 UNSUPPORTED (legal on the pages
 *     but not built here, e.g. FRACTAL_NZ cache layouts, HiFloat8); 3
 *     DEVICE_ERROR (the HIP runtime reported an error at launch).
 *     qknr_last_error() returns a message for the last non-zero status on the
 *     calling thread. Nothing throws or aborts across the ABI.
 *   - Ownership: every tensor pointer is device memory owned by the caller.
 *     The library never allocates, frees or keeps a pointer after returning,
 *     and uses no workspace.
 *   - Asynchrony: work is enqueued on `stream` (NULL = the null stream) and
 *     the call returns without synchronising.
 *   - Layouts are given as element strides (not bytes); the innermost
 *     (channel) dimension is always contiguous.
 *   - Data values are not checked on the device: inf/nan inputs are outside
 *     the operators' domain, and out-of-range or duplicate cache indices are
 *     undefined behaviour (the KvRmsNormRopeCache constraint tables), except
 *     that index -1 means "no cache write" for that token.
 *   - Determinism: no atomics; every output element has exactly one writer
 *     and every reduction runs in a fixed order, so results are bit-identical
 *     from run to run.
 */
#ifndef QKNR_H
#define QKNR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKNR_ABI_VERSION 3

/* status codes */
#define QKNR_OK 0
#define QKNR_INVALID_ARGUMENT 1
#define QKNR_UNSUPPORTED 2
#define QKNR_DEVICE_ERROR 3

/* element types */
#define QKNR_F32 0
#define QKNR_BF16 1
#define QKNR_F16 2
#define QKNR_INT8 3
#define QKNR_FP8_E4M3FN 4
#define QKNR_FP8_E5M2 5

/* cache modes (KvRmsNormRopeCache, cache_mode attribute) */
#define QKNR_CACHE_NORM 0      /* "Norm": [Bkv, N, Scache, D], index [Bkv, Skv] */
#define QKNR_CACHE_PA_BNSD 1   /* "PA" / "PA_BNSD": [block_num, block_size, N, D], index [Bkv*Skv] */
#define QKNR_CACHE_PA_BLK_BNSD 2 /* "PA_BLK_BNSD": PA_BNSD's layout, index [Bkv*ceil(Skv/block_size)]
                                    of block starting slots */

/* shapes of a quantisation parameter (constraint table for k_rope_scale etc.) */
#define QKNR_QSHAPE_SCALAR 0       /* [1]                 */
#define QKNR_QSHAPE_CHANNEL 1      /* [D] or [1, D]       */
#define QKNR_QSHAPE_HEAD_CHANNEL 2 /* [N, D], row-major   */

/*
 * (a) Across-heads QK RMSNorm + rotate-half RoPE.
 *
 * Token (b, s) of Q has channel c = h*d_head + i at
 *   q_in[b*in_batch_stride + s*in_token_stride + h*in_head_stride + i]
 * and K likewise from k_in (the same strides). With a BSD [B, S, I] projection
 * output (Q at channel 0, K at n_q_heads*d_head, V after), pass
 * q_in = base, k_in = base + n_q_heads*d_head, token stride I, head stride
 * d_head; an NBSd [n_heads, B, S, d_head] layout is head stride B*S*d_head,
 * batch stride S*d_head, token stride d_head. Outputs use the out_* strides
 * and may alias the inputs exactly (in place); V is never touched.
 *
 * Per token and segment (Q: n = n_q_heads; K: n = n_k_heads):
 *   r   = 1 / sqrt( sum_c x_c^2 / (n*d_head) + eps )                 (apply_norm)
 *   y_c = x_c * gamma_c                                              (apply_norm)
 *   out[h, i]        = r*(y[h,i]*cos[i]        - y[h,i+d/2]*sin[i])          i < d/2
 *   out[h, i+d/2]    = r*(y[h,i+d/2]*cos[i+d/2] + y[h,i]*sin[i+d/2])        (apply_rope)
 * with cos/sin[b, s, :] read at
 *   cos[b*rope_batch_stride + s*rope_token_stride + i] (batch stride 0 = shared table).
 * Without apply_norm, r = 1 and gamma is not read; without apply_rope the
 * output is r*y. Arithmetic is fp32; results are rounded once (RNE) to `dtype`.
 *
 * Arguments:
 *   dtype            QKNR_F32, QKNR_BF16 or QKNR_F16: Q/K in and out, gammas, cos, sin.
 *   batch, seq       B, S >= 0 (zero tokens is a no-op).
 *   n_q_heads >= 1, n_k_heads >= 0 (0: a Q-only projection; K pointers ignored).
 *   head_dim         even, 2..1024.
 *   q_gamma [n_q_heads*head_dim], k_gamma [n_k_heads*head_dim] (segment-wide gammas).
 *   eps              added to the mean of squares inside the square root.
 *   q_norm_channels, k_norm_channels   0, except in qknr_qk_apply_across_heads
 *       (the channel count of the whole segment over every rank).
 *   sumsq_parts      0, except in qknr_qk_apply_across_heads (partial sums per
 *       token and segment, see there).
 */
typedef struct qknr_qk_args {
    int32_t dtype;
    int32_t n_q_heads;
    int32_t n_k_heads;
    int32_t head_dim;
    int64_t batch;
    int64_t seq;
    const void *q_in;
    const void *k_in;
    void *q_out;
    void *k_out;
    int64_t in_batch_stride;
    int64_t in_token_stride;
    int64_t in_head_stride;
    int64_t out_batch_stride;
    int64_t out_token_stride;
    int64_t out_head_stride;
    const void *q_gamma;
    const void *k_gamma;
    const void *cos;
    const void *sin;
    int64_t rope_batch_stride;
    int64_t rope_token_stride;
    float eps;
    int32_t apply_norm;
    int32_t apply_rope;
    int32_t sumsq_parts;
    int64_t q_norm_channels;
    int64_t k_norm_channels;
} qknr_qk_args;

int32_t qknr_qk_norm_rope_across_heads(const qknr_qk_args *args, hipStream_t stream);

/* Host-only validation of (a)'s arguments: the same checks the launch call
 * makes, without touching a device. Returns a status code. */
int32_t qknr_qk_validate(const qknr_qk_args *args);

/*
 * (a) split over ranks, step a ("Kernel reference: qkv_cte", Design section 1:
 * each rank accumulates sum(x^2) of its own heads for every token).
 *   sumsq[seg*B*S + b*S + s] = sum over this call's heads and channels of x^2
 * for seg 0 = Q and seg 1 = K (K only when n_k_heads > 0), fp32, written by the
 * call; sumsq is a caller-owned device array of (n_k_heads > 0 ? 2 : 1)*B*S
 * floats, 4-byte aligned. Only q_in/k_in, the input strides, dtype and the
 * sizes of `args` are read (gammas, tables, outputs, apply_* are ignored).
 * The caller then adds the arrays of all ranks (an all-reduce; on one GPU, the
 * array itself) before step c.
 */
int32_t qknr_qk_sumsq_across_heads(const qknr_qk_args *args, float *sumsq, hipStream_t stream);

/*
 * (a) split over ranks, step c: as qknr_qk_norm_rope_across_heads on this
 * rank's heads, but with
 *   r = 1 / sqrt( sumsq[seg*B*S + b*S + s] / norm_channels + eps )
 * where sumsq holds the sums added over every rank (layout of step a) and
 * norm_channels = args->q_norm_channels (Q) / k_norm_channels (K), the
 * channel count of the whole segment (n_heads*d_head*tp, below 2^24); 0 means
 * this call's own n*d_head. apply_norm must be 1.
 * With args->sumsq_parts = P > 1 the sum of a token's segment is itself the
 * sum of P partial sums laid out [seg][B*S][P]
 *   sum = sumsq[(seg*B*S + t)*P + 0] + ... + sumsq[(seg*B*S + t)*P + P-1]
 * added in a fixed order (a pairwise tree; the same bits on every run), e.g.
 * the per-tile sums qknr_qkv_projection writes; 0 or 1 means one sum (the
 * layout of step a).
 */
int32_t qknr_qk_apply_across_heads(const qknr_qk_args *args, const float *sumsq, hipStream_t stream);

/*
 * (a) per head: as qknr_qk_norm_rope_across_heads, but with one RMS per
 * (token, head) over head_dim channels,
 *   r_h = 1 / sqrt( sum_i x[h,i]^2 / head_dim + eps ),   y[h,i] = x[h,i]*gamma_i,
 * and q_gamma, k_gamma of head_dim elements shared by every head (the per-head
 * [1, d_head] gamma of the upstream qk-norm, qkv_cte "Upstream behavior").
 */
int32_t qknr_qk_norm_rope_per_head(const qknr_qk_args *args, hipStream_t stream);

/*
 * Interleaved-pair -> rotate-half lane permutation (qkv_cte Design section 2:
 * an interleaved checkpoint is converted once, offline, by permuting the Q/K
 * weights, bias, gamma and cos/sin caches).
 *
 * The tensor is viewed as [outer, axis_len, inner] (row-major, contiguous,
 * `elem_bytes`-byte elements). Along the middle axis, the n_heads blocks of
 * head_dim indices starting at `first` are permuted:
 *   dst[o, first + h*d + j, :] = src[o, first + h*d + (j < d/2 ? 2j : 2(j - d/2) + 1), :]
 * (inverse = 1 applies the inverse permutation); every other index is copied.
 * Examples: a fused QKV weight [H, I] -> outer H, axis I, inner 1, first 0,
 * n_heads = n_q + n_k (V's blocks stay); an MX weight [H/4, I, 4] -> inner 4;
 * interleaved cos/sin tables [S, d] (each angle at lanes 2j and 2j+1) -> outer S,
 * axis d, n_heads 1, giving rotate-half tables.
 * src and dst are caller-owned device memory and must not overlap.
 */
typedef struct qknr_permute_args {
    int32_t elem_bytes;     /* 1, 2, 4 or 8 */
    int32_t inverse;        /* 0: interleaved -> rotate-half; 1: rotate-half -> interleaved */
    int64_t outer;          /* >= 0 */
    int64_t axis_len;       /* >= 1 */
    int64_t inner;          /* >= 1 elements per axis index */
    int64_t first;          /* >= 0 */
    int64_t n_heads;        /* >= 0; first + n_heads*head_dim <= axis_len */
    int64_t head_dim;       /* even, >= 2 */
    const void *src;
    void *dst;
} qknr_permute_args;

int32_t qknr_interleaved_to_rotate_half(const qknr_permute_args *args, hipStream_t stream);

/* qknr_proj_args.scale_mode */
#define QKNR_PROJ_SCALE_ROW 0   /* a_scale / w_scale per row / per output channel (ROW_MX), or none */
#define QKNR_PROJ_SCALE_MX32 1  /* OCP MX block scales: one E8M0 byte per 32 values of K, on a and w */

/*
 * The QKV projection with step a of the across-heads norm fused into its
 * epilogue ("Kernel reference: qkv_cte": "Upstream behavior" for
 * O[S, I] = A[S, H] @ W + bias with I = (n_q + 2*n_kv)*d_head and the
 * MXFP8 / ROW_MX quantisation modes, Design section 1 step a for sum(x^2)
 * accumulated as the output tiles are copied out). On matrix cores (bf16 or
 * FP8 E4M3 operands, fp32 accumulation):
 *   out[m, n] = RNE_bf16( sum_k A[m, k] * W[n, k] * a_scale[m] * w_scale[n] + bias[n] )
 * where, with scale_mode QKNR_PROJ_SCALE_MX32 (MXFP8, the OCP Microscaling
 * format), A[m, k] = a[m, k] * 2^(a_block_scale[m, k/32] - 127) and
 * W[n, k] = w[n, k] * 2^(w_block_scale[n, k/32] - 127); otherwise A = a and
 * W = w. A NULL a_scale / w_scale is 1 (bf16 operands normally have none;
 * FP8 operands with a per-row activation scale and a per-output-channel
 * weight scale are the page's ROW_MX mode; MXFP8 usually has none).
 * for m < rows, n < out_features, and, when q_cols > 0, for every 128-column
 * tile of the Q columns [0, q_cols) and of the K columns [q_cols, q_cols +
 * k_cols), the per-row sum of the squares of the stored (rounded) values:
 *   sumsq[(seg*rows + m)*P + part],  P = q_cols / 128, seg 0 = Q, 1 = K.
 * qknr_qk_apply_across_heads with sumsq_parts = P then finishes the norm and
 * RoPE on the Q and K columns of `out` (steps b-c, with the sums of all
 * ranks when the heads are split).
 *
 * Arguments:
 *   dtype            QKNR_BF16 or QKNR_FP8_E4M3FN: the type of a and w; bias
 *       and out are bf16 in both cases.
 *   scale_mode       QKNR_PROJ_SCALE_ROW, or QKNR_PROJ_SCALE_MX32 (FP8 only).
 *   rows, in_features, out_features   M = B*S >= 0, K = H (a multiple of 128
 *       bytes: 64 bf16 or 128 FP8 values), N = I (multiple of 128).
 *   a [rows, in_features] with row stride a_row_stride; w [out_features,
 *       in_features] (a linear layer's weight) with row stride w_row_stride;
 *       bias [out_features] or NULL; out [rows, out_features] with row stride
 *       out_row_stride. Strides are elements and multiples of 16 bytes
 *       (a_row_stride and w_row_stride at most 4 MiB in bytes); pointers
 *       16-byte aligned. out must not overlap a, w or bias.
 *   a_scale [rows], w_scale [out_features]   fp32 or NULL.
 *   q_cols, k_cols   multiples of 128 with q_cols + k_cols <= out_features;
 *       k_cols is 0 or q_cols. q_cols = 0: no sums (sumsq ignored).
 *   sumsq            fp32 [(k_cols ? 2 : 1) * P * rows], 4-byte aligned.
 *   a_block_scale [rows, in_features/32], w_block_scale [out_features,
 *       in_features/32]   E8M0 bytes (MX32 only; NULL otherwise), row strides
 *       a_block_scale_stride / w_block_scale_stride in bytes, multiples of 4
 *       and >= in_features/32; pointers 4-byte aligned. The code 255 (NaN)
 *       is not supported (the result is unspecified).
 * Errors: INVALID_ARGUMENT for a violated rule above (nothing launched),
 * UNSUPPORTED for an operand type or scale mode that is not built, or a row
 * stride beyond the limits above.
 */
typedef struct qknr_proj_args {
    int32_t dtype;
    int32_t scale_mode;
    int64_t rows;
    int64_t in_features;
    int64_t out_features;
    const void *a;
    int64_t a_row_stride;
    const void *w;
    int64_t w_row_stride;
    const void *bias;
    void *out;
    int64_t out_row_stride;
    int64_t q_cols;
    int64_t k_cols;
    float *sumsq;
    const float *a_scale;
    const float *w_scale;
    const uint8_t *a_block_scale;
    int64_t a_block_scale_stride;
    const uint8_t *w_block_scale;
    int64_t w_block_scale_stride;
} qknr_proj_args;

int32_t qknr_qkv_projection(const qknr_proj_args *args, hipStream_t stream);

/*
 * (b) KvRmsNormRopeCache.
 *
 * Rows are (b, n, s) with b < batch (Bkv), n < heads (N), s < seq (Skv).
 *   V1 (v_optional == NULL): kv rows are [rms_size | rope_size] (Dv | Dk);
 *       y = RmsNorm(kv[:rms_size]) * gamma; rope_out = interleaveRope(kv[rms_size:]);
 *       k_cache <- Quant(rope_out), ckv_cache <- Quant(y). heads must be 1.
 *   V2 (v_optional != NULL): kv rows are rms_size = kv_dim wide;
 *       y = RmsNorm(kv) * gamma; rope_out = [interleaveRope(y[:rope_size]) | y[rope_size:]];
 *       k_cache <- Quant(rope_out), ckv_cache <- Quant(v_optional row).
 *       heads in {1, 2, 4, 8}.
 *   RmsNorm: x / sqrt(mean(x^2) + eps) * gamma.
 *   interleaveRope(z): out[j] = z[2j]*cos[j] - z[2j+1]*sin[j],
 *       out[j+R/2] = z[2j+1]*cos[j+R/2] + z[2j]*sin[j+R/2], j < R/2 (the even
 *       lanes' results first, then the odd lanes'; cos/sin indexed by output lane).
 *   Quant (per cache): t = x*scale (+offset); INT8: round half to even, clamp to
 *       [-128, 127]; FP8_E4M3FN / FP8_E5M2: round to nearest even, saturate at
 *       the largest finite value (+-448 / +-57344);
 *       cache dtype == dtype: round the value to dtype (no scale/offset allowed).
 *       Rounding decisions are taken on the fp32 value of t.
 *   Scatter: NORM: row index[b*Skv + s] (index is [Bkv, Skv]) inside batch b:
 *       k_cache[b*kc_stride0 + n*kc_stride2 + row*kc_stride1];
 *       PA_BNSD: slot = index[b*Skv + s] (index is [Bkv*Skv]):
 *       k_cache[(slot/block_size)*kc_stride0 + (slot%block_size)*kc_stride1 + n*kc_stride2];
 *       PA_BLK_BNSD: the tokens of batch b form runs of block_size (the last
 *       may be shorter); run j fills consecutive slots from its starting slot
 *       index[b*ceil(Skv/block_size) + j] (the cache/index constraint table
 *       gives one entry per block of tokens, the block's starting offset), so
 *       token s goes to slot index[b*ceil(Skv/bs) + s/bs] + s%bs, addressed as
 *       in PA_BNSD. Starts need not be multiples of block_size.
 *       The ckv cache is addressed likewise with the ckv strides. index -1: no
 *       cache write (PA_BLK_BNSD: for the whole run); a slot outside the cache
 *       (undefined on the page) writes nothing.
 *   Raw outputs (is_output_kv): k_rope[b,n,s,:] = rope_out and
 *       c_kv[b,n,s,:] = y (V1) or v_optional row (V2), in `dtype`, unquantised.
 *
 * Widths: k rows are k_dim = rope_size (V1) or kv_dim (V2) wide; ckv rows are
 * c_dim = rms_size (V1) or v_dim (V2) wide.
 *
 * Arguments:
 *   dtype            QKNR_BF16 or QKNR_F16: kv, gamma, cos, sin, v_optional, k_rope, c_kv.
 *   batch, heads, seq    Bkv, N, Skv >= 1 (empty tensors are not allowed).
 *   kv_dim, rms_size, rope_size, v_dim   see above; rope_size even.
 *   kv_strides[3], v_strides[3], rope_strides[3], k_rope_strides[3],
 *   c_kv_strides[3]: element strides of the (b, n, s) axes; the channel axis is
 *       contiguous. rope_strides[2] == 0 is the S-axis broadcast (Srope = 1).
 *       Every stride is below 2^32 elements (QKNR_UNSUPPORTED otherwise).
 *   index            int64 device array (see Scatter): Bkv*Skv entries (NORM,
 *       PA_BNSD) or Bkv*ceil(Skv/block_size) (PA_BLK_BNSD).
 *   cache_mode       QKNR_CACHE_NORM, QKNR_CACHE_PA_BNSD or QKNR_CACHE_PA_BLK_BNSD.
 *   cache_rows       NORM: Scache (>= Skv). Paged: block_num (>= floor(Skv/bs)*Bkv).
 *   block_size       paged: > 1 and block_size*sizeof(cache element) a multiple of 32.
 *   k_cache_dtype, ckv_cache_dtype   dtype, QKNR_INT8, QKNR_FP8_E4M3FN or QKNR_FP8_E5M2.
 *   k_cache_strides[3], ckv_cache_strides[3]: element strides of the cache's
 *       leading axes: NORM (batch, row, head); paged (block, slot in block,
 *       head). The channel axis is contiguous. Below 2^32 elements.
 *   k_scale, k_offset, v_scale, v_offset   fp32 device arrays or NULL; the
 *       *_qshape fields give their shapes (QKNR_QSHAPE_*). A scale is required
 *       exactly when the cache dtype differs from dtype; an offset needs its
 *       scale. V1 allows SCALAR/CHANNEL shapes, V2 HEAD_CHANNEL.
 *   eps              default on the page 1e-5.
 *   is_output_kv     1: write k_rope and c_kv (effective in the paged modes,
 *       and in NORM only for V2 with quantisation; ignored elsewhere).
 */
typedef struct qknr_kv_args {
    int32_t dtype;
    int32_t heads;
    int64_t batch;
    int64_t seq;
    int32_t kv_dim;
    int32_t rms_size;
    int32_t rope_size;
    int32_t v_dim;
    const void *kv;
    const void *v_optional;
    const void *gamma;
    const void *cos;
    const void *sin;
    int64_t kv_strides[3];
    int64_t v_strides[3];
    int64_t rope_strides[3];
    const int64_t *index;
    int32_t cache_mode;
    int32_t block_size;
    int64_t cache_rows;
    void *k_cache;
    void *ckv_cache;
    int32_t k_cache_dtype;
    int32_t ckv_cache_dtype;
    int64_t k_cache_strides[3];
    int64_t ckv_cache_strides[3];
    const float *k_scale;
    const float *k_offset;
    const float *v_scale;
    const float *v_offset;
    int32_t k_qshape;
    int32_t v_qshape;
    float eps;
    int32_t is_output_kv;
    void *k_rope;
    void *c_kv;
    int64_t k_rope_strides[3];
    int64_t c_kv_strides[3];
} qknr_kv_args;

int32_t qknr_kv_rmsnorm_rope_cache(const qknr_kv_args *args, hipStream_t stream);

/* Host-only validation of (b)'s arguments (no device access). */
int32_t qknr_kv_validate(const qknr_kv_args *args);

/* Message for the last non-zero status returned on the calling thread
 * (empty string if none). The pointer stays valid until the next call on
 * this thread. */
const char *qknr_last_error(void);

/* QKNR_ABI_VERSION of the loaded library. */
int32_t qknr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QKNR_H */
