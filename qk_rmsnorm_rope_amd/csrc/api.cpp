// api.cpp -- the extern "C" entry points declared in include/qknr.h: argument
// validation (host only), vector-width selection and kernel dispatch.
//
// Validation follows the constraint sections of the "KvRmsNormRopeCache" page
// (dtype equalities, the scale/offset legality table, cache/index shapes,
// block_size alignment, V1/V2 head counts, no empty tensors, is_output_kv
// validity) and the argument list of the qkv_cte page's interface (segment
// widths, gammas, rotate-half tables).
#include <cstdarg>
#include <cstdint>
#include <climits>
#include <cstdio>
#include <string>
#include <utility>

#include "qknr.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int32_t ok() {
    return QKNR_OK;
}

int elem_size(int32_t dtype) {
    switch (dtype) {
    case QKNR_F32: return 4;
    case QKNR_BF16: case QKNR_F16: return 2;
    case QKNR_INT8: case QKNR_FP8_E4M3FN: case QKNR_FP8_E5M2: return 1;
    }
    return 0;
}

bool aligned(const void *p, int bytes) {
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) % (uintptr_t)bytes) == 0;
}

// ---------------------------------------------------------------- (a)

struct QkPlan {
    qknr::QkParams p;
    int elem_type;
    int vec;
};

// mode: qknr::QkMode (which entry point); sumsq: step a's output / step c's input.
int32_t qk_check(const qknr_qk_args *a, int mode, const float *sumsq, QkPlan *out) {
    if (!a) return fail(QKNR_INVALID_ARGUMENT, "args is NULL");
    const bool sums_only = mode == qknr::QK_SUMSQ;
    if (a->dtype != QKNR_F32 && a->dtype != QKNR_BF16 && a->dtype != QKNR_F16)
        return fail(QKNR_INVALID_ARGUMENT, "dtype must be QKNR_F32, QKNR_BF16 or QKNR_F16 (got %d)", a->dtype);
    if (a->n_q_heads < 1) return fail(QKNR_INVALID_ARGUMENT, "n_q_heads must be >= 1");
    if (a->n_k_heads < 0) return fail(QKNR_INVALID_ARGUMENT, "n_k_heads must be >= 0");
    if (a->head_dim < 2 || (a->head_dim & 1))
        return fail(QKNR_INVALID_ARGUMENT, "head_dim must be even and >= 2 (rotate-half pairs i, i+d/2)");
    if (a->batch < 0 || a->seq < 0) return fail(QKNR_INVALID_ARGUMENT, "batch and seq must be >= 0");
    if (!(a->eps >= 0.0f) || a->eps == __builtin_inff())
        return fail(QKNR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    const int64_t tokens = a->batch * a->seq;
    const bool has_k = a->n_k_heads > 0;
    const bool use_norm = !sums_only && a->apply_norm, use_rope = !sums_only && a->apply_rope;
    if (mode == qknr::QK_APPLY && !a->apply_norm)
        return fail(QKNR_INVALID_ARGUMENT, "the apply pass of a split norm needs apply_norm = 1");
    if (tokens > 0) {
        if (!a->q_in || (!sums_only && !a->q_out))
            return fail(QKNR_INVALID_ARGUMENT, "q_in and q_out are required");
        if (has_k && (!a->k_in || (!sums_only && !a->k_out)))
            return fail(QKNR_INVALID_ARGUMENT, "k_in and k_out are required when n_k_heads > 0");
        if (use_norm && (!a->q_gamma || (has_k && !a->k_gamma)))
            return fail(QKNR_INVALID_ARGUMENT, "apply_norm needs q_gamma (and k_gamma when n_k_heads > 0)");
        if (use_rope && (!a->cos || !a->sin))
            return fail(QKNR_INVALID_ARGUMENT, "apply_rope needs cos and sin");
        if ((mode == qknr::QK_SUMSQ || mode == qknr::QK_APPLY) && !sumsq)
            return fail(QKNR_INVALID_ARGUMENT, "sumsq is required");
        if (!aligned(sumsq, 4)) return fail(QKNR_INVALID_ARGUMENT, "sumsq must be 4-byte aligned");
    }
    // total channel counts belong to the apply pass; elsewhere 0 (or the call's own count)
    const int64_t own_q = (int64_t)a->n_q_heads * a->head_dim, own_k = (int64_t)a->n_k_heads * a->head_dim;
    const int64_t q_total = a->q_norm_channels ? a->q_norm_channels : own_q;
    const int64_t k_total = a->k_norm_channels ? a->k_norm_channels : own_k;
    if (mode != qknr::QK_APPLY && (q_total != own_q || (has_k && k_total != own_k)))
        return fail(QKNR_INVALID_ARGUMENT, "q_norm_channels/k_norm_channels are for the apply pass only (else 0)");
    if (a->sumsq_parts < 0 || (mode != qknr::QK_APPLY && a->sumsq_parts > 1) || a->sumsq_parts > 65536)
        return fail(QKNR_INVALID_ARGUMENT, "sumsq_parts is 0 or 1 except in the apply pass (at most 65536)");
    if (q_total < own_q || (has_k && k_total < own_k) || q_total >= (1LL << 24) || k_total >= (1LL << 24))
        return fail(QKNR_INVALID_ARGUMENT,
                    "norm channel counts must cover this call's heads and stay below 2^24");
    if (a->in_batch_stride < 0 || a->in_token_stride < 0 || a->out_batch_stride < 0 ||
        a->out_token_stride < 0 || a->rope_batch_stride < 0 || a->rope_token_stride < 0)
        return fail(QKNR_INVALID_ARGUMENT, "strides must be >= 0");
    if (a->in_head_stride < a->head_dim || (!sums_only && a->out_head_stride < a->head_dim))
        return fail(QKNR_INVALID_ARGUMENT, "head strides must be >= head_dim (heads may not overlap)");
    const bool q_alias = !sums_only && a->q_out == a->q_in, k_alias = !sums_only && has_k && a->k_out == a->k_in;
    if ((q_alias || k_alias) && (a->in_batch_stride != a->out_batch_stride ||
                                 a->in_token_stride != a->out_token_stride ||
                                 a->in_head_stride != a->out_head_stride))
        return fail(QKNR_INVALID_ARGUMENT, "in-place use needs identical input and output strides");

    const int es = elem_size(a->dtype);
    const int half = a->head_dim / 2;
    const void *ptrs[] = {a->q_in, sums_only ? nullptr : a->q_out, has_k ? a->k_in : nullptr,
                          (has_k && !sums_only) ? a->k_out : nullptr,
                          use_norm ? a->q_gamma : nullptr,
                          (use_norm && has_k) ? a->k_gamma : nullptr,
                          use_rope ? a->cos : nullptr, use_rope ? a->sin : nullptr};
    const int64_t strides[] = {a->in_batch_stride, a->in_token_stride, a->in_head_stride,
                               sums_only ? 0 : a->out_batch_stride, sums_only ? 0 : a->out_token_stride,
                               sums_only ? 0 : a->out_head_stride,
                               use_rope ? a->rope_batch_stride : 0,
                               use_rope ? a->rope_token_stride : 0};
    auto fits = [&](int vec) {
        if (half % vec) return false;
        for (const void *p : ptrs)
            if (!aligned(p, vec * es)) return false;
        for (int64_t s : strides)
            if (s % vec) return false;
        return true;
    };
    const int wide = 16 / es, narrow = 4 / es;
    int vec = fits(wide) ? wide : (fits(narrow) ? narrow : 0);
    if (!vec)
        return fail(QKNR_UNSUPPORTED, "pointers/strides are not aligned to 4 bytes for this dtype");

    // 32-bit index ranges used inside the kernel
    const int64_t max_heads = a->n_q_heads > a->n_k_heads ? a->n_q_heads : a->n_k_heads;
    const int64_t span_in = ((max_heads - 1) * a->in_head_stride + a->head_dim) * es;
    const int64_t span_out = sums_only ? 0 : ((max_heads - 1) * a->out_head_stride + a->head_dim) * es;
    if (mode == qknr::QK_APPLY && a->sumsq_parts > 1 &&
        (int64_t)a->sumsq_parts * (has_k ? 2 : 1) * (tokens > 0 ? tokens : 1) >= (1LL << 40))
        return fail(QKNR_INVALID_ARGUMENT, "sumsq array too large");
    if (tokens >= (1LL << 31) || span_in >= (1LL << 32) || span_out >= (1LL << 32))
        return fail(QKNR_UNSUPPORTED, "more than 2^31 tokens, or one token's heads span 4 GiB or more");

    QkPlan plan;
    qknr::QkParams &p = plan.p;
    p = qknr::QkParams{};
    p.q_in = a->q_in; p.k_in = a->k_in; p.q_out = a->q_out; p.k_out = a->k_out;
    p.q_gamma = a->q_gamma; p.k_gamma = a->k_gamma; p.cos = a->cos; p.sin = a->sin;
    p.tokens = (uint32_t)tokens;
    p.seq = (uint32_t)(a->seq > 0 ? a->seq : 1);
    p.seq_div = qknr::make_fastdiv(p.seq);
    p.in_batch_stride = a->in_batch_stride; p.in_token_stride = a->in_token_stride;
    p.in_head_stride = (uint32_t)a->in_head_stride;
    p.out_batch_stride = a->out_batch_stride; p.out_token_stride = a->out_token_stride;
    p.out_head_stride = (uint32_t)a->out_head_stride;
    p.rope_batch_stride = a->rope_batch_stride; p.rope_token_stride = a->rope_token_stride;
    p.n_q = a->n_q_heads; p.n_k = a->n_k_heads; p.head_dim = a->head_dim;
    p.segs = has_k ? 2 : 1;
    p.apply_norm = use_norm ? 1 : 0; p.apply_rope = use_rope ? 1 : 0;
    p.q_channels = (float)q_total;
    p.k_channels = (float)(has_k ? k_total : a->head_dim);
    p.eps = a->eps;
    p.sumsq = const_cast<float *>(sumsq);
    p.sum_parts = a->sumsq_parts > 1 ? a->sumsq_parts : 1;
    int J = qknr::qk_plan(p, vec);
    if (J < 0 && vec == wide && fits(narrow)) {
        vec = narrow;
        J = qknr::qk_plan(p, vec);
    }
    if (J < 0)
        return fail(QKNR_UNSUPPORTED, "head_dim %d with %d heads exceeds one block's register plan",
                    a->head_dim, (int)max_heads);
    plan.elem_type = a->dtype == QKNR_F32 ? 0 : (a->dtype == QKNR_BF16 ? 1 : 2);
    plan.vec = vec;
    if (out) *out = plan;
    return ok();
}

// ---------------------------------------------------------------- (b)

struct KvPlan {
    qknr::KvParams p;
    int elem_type;
    int vec;
    bool v2;
};

int32_t cache_code(int32_t cache_dtype, int32_t dtype, const char *which, int32_t *code) {
    if (cache_dtype == dtype) { *code = qknr::CODE_SAME; return QKNR_OK; }
    if (cache_dtype == QKNR_INT8) { *code = qknr::CODE_INT8; return QKNR_OK; }
    if (cache_dtype == QKNR_FP8_E4M3FN) { *code = qknr::CODE_E4M3FN; return QKNR_OK; }
    if (cache_dtype == QKNR_FP8_E5M2) { *code = qknr::CODE_E5M2; return QKNR_OK; }
    if (cache_dtype == QKNR_F32 || cache_dtype == QKNR_BF16 || cache_dtype == QKNR_F16)
        return fail(QKNR_INVALID_ARGUMENT, "%s: an unquantised cache must have the kv dtype", which);
    return fail(QKNR_UNSUPPORTED, "%s: cache dtype %d is not built (INT8, FP8_E4M3FN and FP8_E5M2 are)", which,
                cache_dtype);
}

int32_t kv_check(const qknr_kv_args *a, KvPlan *out) {
    if (!a) return fail(QKNR_INVALID_ARGUMENT, "args is NULL");
    if (a->dtype != QKNR_BF16 && a->dtype != QKNR_F16)
        return fail(QKNR_INVALID_ARGUMENT, "dtype must be QKNR_BF16 or QKNR_F16 (got %d)", a->dtype);
    if (a->batch < 1 || a->heads < 1 || a->seq < 1)
        return fail(QKNR_INVALID_ARGUMENT, "empty tensors are not supported (batch, heads, seq >= 1)");
    if (!a->kv || !a->gamma || !a->cos || !a->sin || !a->index || !a->k_cache || !a->ckv_cache)
        return fail(QKNR_INVALID_ARGUMENT, "kv, gamma, cos, sin, index, k_cache and ckv_cache are required");
    if (a->rope_size < 2 || (a->rope_size & 1))
        return fail(QKNR_INVALID_ARGUMENT, "rope_size must be even and >= 2");
    if (a->rms_size < 1) return fail(QKNR_INVALID_ARGUMENT, "rms_size must be >= 1");
    if (!(a->eps >= 0.0f) || a->eps == __builtin_inff())
        return fail(QKNR_INVALID_ARGUMENT, "epsilon must be finite and >= 0");
    const bool v2 = a->v_optional != nullptr;
    int32_t k_dim, c_dim;
    if (!v2) {
        if (a->heads != 1) return fail(QKNR_INVALID_ARGUMENT, "V1 (merged kv) supports N = 1 only");
        if (a->kv_dim != a->rms_size + a->rope_size)
            return fail(QKNR_INVALID_ARGUMENT, "V1: kv_dim must equal rms_size + rope_size");
        k_dim = a->rope_size;
        c_dim = a->rms_size;
    } else {
        if (a->heads != 1 && a->heads != 2 && a->heads != 4 && a->heads != 8)
            return fail(QKNR_INVALID_ARGUMENT, "V2 (split k/v) supports N in {1, 2, 4, 8}");
        if (a->rms_size != a->kv_dim) return fail(QKNR_INVALID_ARGUMENT, "V2: rms_size must equal kv_dim");
        if (a->rope_size > a->kv_dim) return fail(QKNR_INVALID_ARGUMENT, "V2: rope_size must be <= kv_dim");
        if (a->v_dim < 1) return fail(QKNR_INVALID_ARGUMENT, "V2: v_dim must be >= 1");
        k_dim = a->kv_dim;
        c_dim = a->v_dim;
    }

    int32_t k_code, c_code, rc;
    if ((rc = cache_code(a->k_cache_dtype, a->dtype, "k_cache", &k_code)) != QKNR_OK) return rc;
    if ((rc = cache_code(a->ckv_cache_dtype, a->dtype, "ckv_cache", &c_code)) != QKNR_OK) return rc;
    // scale/offset legality table: no scale + no offset -> cache has the kv dtype;
    // offset without scale is illegal; a quantised cache needs its scale.
    if (a->k_offset && !a->k_scale) return fail(QKNR_INVALID_ARGUMENT, "k_offset given without k_scale");
    if (a->v_offset && !a->v_scale) return fail(QKNR_INVALID_ARGUMENT, "v_offset given without v_scale");
    if (k_code == qknr::CODE_SAME && (a->k_scale || a->k_offset))
        return fail(QKNR_INVALID_ARGUMENT, "k_cache is unquantised (kv dtype): k_scale/k_offset must be NULL");
    if (c_code == qknr::CODE_SAME && (a->v_scale || a->v_offset))
        return fail(QKNR_INVALID_ARGUMENT, "ckv_cache is unquantised (kv dtype): v_scale/v_offset must be NULL");
    if (k_code != qknr::CODE_SAME && !a->k_scale)
        return fail(QKNR_INVALID_ARGUMENT, "a quantised k_cache needs k_scale");
    if (c_code != qknr::CODE_SAME && !a->v_scale)
        return fail(QKNR_INVALID_ARGUMENT, "a quantised ckv_cache needs v_scale");
    const bool k_quant = k_code != qknr::CODE_SAME, c_quant = c_code != qknr::CODE_SAME;
    for (int which = 0; which < 2; which++) {
        const bool q = which == 0 ? k_quant : c_quant;
        const int32_t shape = which == 0 ? a->k_qshape : a->v_qshape;
        if (!q) continue;
        if (!v2 && shape != QKNR_QSHAPE_SCALAR && shape != QKNR_QSHAPE_CHANNEL)
            return fail(QKNR_INVALID_ARGUMENT, "V1 quantisation parameters are [1], [D] or [1, D]");
        if (v2 && shape != QKNR_QSHAPE_HEAD_CHANNEL)
            return fail(QKNR_INVALID_ARGUMENT, "V2 quantisation parameters are [N, D]");
    }

    // cache modes and index ranges
    int64_t capacity;
    if (a->cache_mode == QKNR_CACHE_NORM) {
        if (a->cache_rows < a->seq) return fail(QKNR_INVALID_ARGUMENT, "Norm cache: Scache must be >= Skv");
        capacity = a->cache_rows;
    } else if (a->cache_mode == QKNR_CACHE_PA_BNSD || a->cache_mode == QKNR_CACHE_PA_BLK_BNSD) {
        if (a->block_size <= 1) return fail(QKNR_INVALID_ARGUMENT, "paged cache: block_size must be > 1");
        const int kb = k_quant ? 1 : elem_size(a->dtype), cb = c_quant ? 1 : elem_size(a->dtype);
        if (((int64_t)a->block_size * kb) % 32 || ((int64_t)a->block_size * cb) % 32)
            return fail(QKNR_INVALID_ARGUMENT,
                        "paged cache: block_size must be 32-byte aligned for each cache dtype");
        if (a->cache_rows < (a->seq / a->block_size) * a->batch)
            return fail(QKNR_INVALID_ARGUMENT, "paged cache: block_num must be >= floor(Skv/block_size)*Bkv");
        capacity = a->cache_rows * (int64_t)a->block_size;
    } else {
        return fail(QKNR_UNSUPPORTED, "cache_mode %d is not built (Norm, PA/PA_BNSD and PA_BLK_BNSD are)",
                    a->cache_mode);
    }

    // S-axis broadcast of cos/sin (Srope = 1): allowed for Norm and for an
    // unquantised paged cache
    const bool s_bcast = a->rope_strides[2] == 0 && a->seq > 1;
    const bool paged = a->cache_mode != QKNR_CACHE_NORM;
    if (s_bcast && paged && (k_quant || c_quant))
        return fail(QKNR_INVALID_ARGUMENT, "S-axis broadcast of cos/sin is not allowed with quantised paged caches");

    // is_output_kv: effective for paged caches, and for Norm only in V2 with quantisation
    const bool out_kv = a->is_output_kv &&
                        (paged || (v2 && (k_quant || c_quant)));
    if (out_kv && (!a->k_rope || !a->c_kv))
        return fail(QKNR_INVALID_ARGUMENT, "is_output_kv needs k_rope and c_kv");

    const int64_t kStride32 = 1LL << 32;
    for (int i = 0; i < 3; i++) {
        if (a->kv_strides[i] < 0 || a->rope_strides[i] < 0 || (v2 && a->v_strides[i] < 0) ||
            a->k_cache_strides[i] < 0 || a->ckv_cache_strides[i] < 0 ||
            (out_kv && (a->k_rope_strides[i] < 0 || a->c_kv_strides[i] < 0)))
            return fail(QKNR_INVALID_ARGUMENT, "strides must be >= 0");
        if (a->kv_strides[i] >= kStride32 || a->rope_strides[i] >= kStride32 || (v2 && a->v_strides[i] >= kStride32) ||
            a->k_cache_strides[i] >= kStride32 || a->ckv_cache_strides[i] >= kStride32 ||
            (out_kv && (a->k_rope_strides[i] >= kStride32 || a->c_kv_strides[i] >= kStride32)))
            return fail(QKNR_UNSUPPORTED, "strides must be < 2^32 elements");
    }

    // vector width: 8 elements (16-byte accesses) or 4 (8-byte)
    const int es = elem_size(a->dtype);
    auto fits = [&](int vec) {
        const int h = vec / 2;
        if (a->rms_size % vec || a->rope_size % vec || (v2 && a->v_dim % vec)) return false;
        const void *full[] = {a->kv, v2 ? a->v_optional : nullptr, a->gamma, out_kv ? a->c_kv : nullptr};
        for (const void *p : full)
            if (!aligned(p, vec * es)) return false;
        if (!aligned(a->cos, h * es) || !aligned(a->sin, h * es)) return false;
        // k rows take half-chunk stores (the rotated part); V2 k rows also take
        // whole chunks (the unrotated normed part)
        const int kw = v2 ? vec : h;
        if (out_kv && !aligned(a->k_rope, kw * es)) return false;
        const int kb = k_quant ? 1 : es, cb = c_quant ? 1 : es;
        if (!aligned(a->k_cache, kw * kb) || !aligned(a->ckv_cache, vec * cb)) return false;
        const float *qp[] = {a->k_scale, a->k_offset, a->v_scale, a->v_offset};
        for (const float *p : qp)
            if (!aligned(p, 16)) return false;
        for (int i = 0; i < 3; i++) {
            if (a->kv_strides[i] % vec || (v2 && a->v_strides[i] % vec) || a->rope_strides[i] % h ||
                a->k_cache_strides[i] % kw || a->ckv_cache_strides[i] % vec ||
                (out_kv && (a->k_rope_strides[i] % kw || a->c_kv_strides[i] % vec)))
                return false;
        }
        return true;
    };
    const int vec = fits(8) ? 8 : (fits(4) ? 4 : 0);
    if (!vec)
        return fail(QKNR_UNSUPPORTED,
                    "sizes, pointers or strides are not multiples of 4 elements (8-byte accesses)");

    KvPlan plan;
    qknr::KvParams &p = plan.p;
    p = qknr::KvParams{};
    p.kv = a->kv; p.v = a->v_optional; p.gamma = a->gamma; p.cos = a->cos; p.sin = a->sin;
    p.index = a->index; p.k_cache = a->k_cache; p.ckv_cache = a->ckv_cache;
    p.k_scale = a->k_scale; p.k_offset = a->k_offset; p.v_scale = a->v_scale; p.v_offset = a->v_offset;
    p.k_rope = a->k_rope; p.c_kv = a->c_kv;
    const int64_t rows = a->batch * a->heads * a->seq;
    if (rows >= (1LL << 31) || capacity >= (1LL << 31) || a->batch * a->seq >= (1LL << 31))
        return fail(QKNR_UNSUPPORTED, "more than 2^31 rows, tokens or cache slots in one call");
    p.rows = (uint32_t)rows;
    p.seq = (uint32_t)a->seq;
    p.seq_div = qknr::make_fastdiv(p.seq);
    p.heads_div = qknr::make_fastdiv((uint32_t)a->heads);
    p.block_div = qknr::make_fastdiv((uint32_t)(a->cache_mode == QKNR_CACHE_NORM ? 1 : a->block_size));
    p.stream_rope = s_bcast ? 0 : 1;
    // strides checked above to be in [0, 2^32) where they are used; unused ones are 0
    auto u32 = [](int64_t v) { return (uint32_t)(v >= 0 && v < (1LL << 32) ? v : 0); };
    p.kv_b = u32(a->kv_strides[0]); p.kv_n = u32(a->kv_strides[1]); p.kv_s = u32(a->kv_strides[2]);
    if (v2) { p.v_b = u32(a->v_strides[0]); p.v_n = u32(a->v_strides[1]); p.v_s = u32(a->v_strides[2]); }
    p.rope_b = u32(a->rope_strides[0]); p.rope_n = u32(a->rope_strides[1]); p.rope_s = u32(a->rope_strides[2]);
    if (out_kv) {
        p.kr_b = u32(a->k_rope_strides[0]); p.kr_n = u32(a->k_rope_strides[1]); p.kr_s = u32(a->k_rope_strides[2]);
        p.ck_b = u32(a->c_kv_strides[0]); p.ck_n = u32(a->c_kv_strides[1]); p.ck_s = u32(a->c_kv_strides[2]);
    }
    p.kc0 = u32(a->k_cache_strides[0]); p.kc1 = u32(a->k_cache_strides[1]); p.kc2 = u32(a->k_cache_strides[2]);
    p.cc0 = u32(a->ckv_cache_strides[0]); p.cc1 = u32(a->ckv_cache_strides[1]); p.cc2 = u32(a->ckv_cache_strides[2]);
    p.capacity = capacity;
    p.heads = a->heads;
    p.mode = a->cache_mode;     // 0 Norm, 1 PA_BNSD, 2 PA_BLK_BNSD
    p.runs = a->cache_mode == QKNR_CACHE_PA_BLK_BNSD
                 ? (uint32_t)((a->seq + a->block_size - 1) / a->block_size) : 0;
    p.block_size = a->cache_mode == QKNR_CACHE_NORM ? 1 : a->block_size;
    p.rms_size = a->rms_size; p.rope_size = a->rope_size; p.half_rope = a->rope_size / 2;
    p.k_dim = k_dim; p.c_dim = c_dim;
    p.k_code = k_code; p.c_code = c_code;
    p.k_qshape = a->k_qshape; p.v_qshape = a->v_qshape;
    p.out_kv = out_kv ? 1 : 0;
    p.eps = a->eps;
    int ca = 0, cb = 0;
    if (qknr::kv_plan(p, vec, v2, ca, cb) != 0)
        return fail(QKNR_UNSUPPORTED, "row too wide for one block's register plan");
    plan.elem_type = a->dtype == QKNR_BF16 ? 1 : 2;
    plan.vec = vec;
    plan.v2 = v2;
    if (out) *out = plan;
    return ok();
}

}  // namespace

extern "C" {

int32_t qknr_qk_validate(const qknr_qk_args *args) {
    return qk_check(args, qknr::QK_ACROSS, nullptr, nullptr);
}

static int32_t qk_run(const qknr_qk_args *args, int mode, const float *sumsq, hipStream_t stream) {
    QkPlan plan;
    int32_t rc = qk_check(args, mode, sumsq, &plan);
    if (rc != QKNR_OK) return rc;
    hipError_t e = qknr::qk_launch(plan.p, plan.elem_type, plan.vec, mode, stream);
    if (e != hipSuccess) return fail(QKNR_DEVICE_ERROR, "launch failed: %s", hipGetErrorString(e));
    return QKNR_OK;
}

int32_t qknr_qk_norm_rope_across_heads(const qknr_qk_args *args, hipStream_t stream) {
    return qk_run(args, qknr::QK_ACROSS, nullptr, stream);
}

int32_t qknr_qk_sumsq_across_heads(const qknr_qk_args *args, float *sumsq, hipStream_t stream) {
    return qk_run(args, qknr::QK_SUMSQ, sumsq, stream);
}

int32_t qknr_qk_apply_across_heads(const qknr_qk_args *args, const float *sumsq, hipStream_t stream) {
    return qk_run(args, qknr::QK_APPLY, sumsq, stream);
}

int32_t qknr_qk_norm_rope_per_head(const qknr_qk_args *args, hipStream_t stream) {
    return qk_run(args, qknr::QK_PER_HEAD, nullptr, stream);
}

int32_t qknr_qkv_projection(const qknr_proj_args *a, hipStream_t stream) {
    if (!a) return fail(QKNR_INVALID_ARGUMENT, "args is NULL");
    if (a->dtype != QKNR_BF16 && a->dtype != QKNR_FP8_E4M3FN)
        return fail(QKNR_UNSUPPORTED, "the projection is built for QKNR_BF16 and QKNR_FP8_E4M3FN operands");
    const bool fp8 = a->dtype == QKNR_FP8_E4M3FN;
    const int eb = fp8 ? 1 : 2;
    if (a->scale_mode != QKNR_PROJ_SCALE_ROW && a->scale_mode != QKNR_PROJ_SCALE_MX32)
        return fail(QKNR_UNSUPPORTED, "scale_mode %d is not built (QKNR_PROJ_SCALE_ROW, QKNR_PROJ_SCALE_MX32 are)",
                    a->scale_mode);
    const bool mx = a->scale_mode == QKNR_PROJ_SCALE_MX32;
    if (mx && !fp8) return fail(QKNR_INVALID_ARGUMENT, "MX block scales need FP8 operands (QKNR_FP8_E4M3FN)");
    if (!mx && (a->a_block_scale || a->w_block_scale))
        return fail(QKNR_INVALID_ARGUMENT, "block scales are given only with scale_mode QKNR_PROJ_SCALE_MX32");
    if (a->rows < 0 || a->in_features < 1 || a->out_features < 1)
        return fail(QKNR_INVALID_ARGUMENT, "rows >= 0, in_features >= 1, out_features >= 1");
    if ((a->in_features * eb) % 128 || a->out_features % 128)
        return fail(QKNR_UNSUPPORTED, "in_features must be a multiple of 128 bytes and out_features of 128");
    if (a->q_cols < 0 || a->k_cols < 0 || a->q_cols % 128 || a->k_cols % 128 ||
        a->q_cols + a->k_cols > a->out_features || (a->k_cols && a->k_cols != a->q_cols) ||
        (a->k_cols && !a->q_cols))
        return fail(QKNR_INVALID_ARGUMENT,
                    "q_cols, k_cols: multiples of 128, k_cols 0 or q_cols, q_cols + k_cols <= out_features");
    if (a->a_row_stride < a->in_features || a->w_row_stride < a->in_features ||
        a->out_row_stride < a->out_features)
        return fail(QKNR_INVALID_ARGUMENT, "row strides must cover a row");
    if ((a->a_row_stride * eb) % 16 || (a->w_row_stride * eb) % 16 || a->out_row_stride % 8)
        return fail(QKNR_UNSUPPORTED, "row strides must be multiples of 16 bytes");
    if (a->a_row_stride * eb > (4LL << 20) || a->w_row_stride * eb > (4LL << 20))
        return fail(QKNR_UNSUPPORTED, "a and w row strides above 4 MiB (tile copies use 32-bit offsets)");
    const int64_t blocks = a->in_features / 32;        // MX blocks per row (in_features is a multiple of 128)
    if (mx && (a->a_block_scale_stride < blocks || a->w_block_scale_stride < blocks ||
               a->a_block_scale_stride % 4 || a->w_block_scale_stride % 4))
        return fail(QKNR_INVALID_ARGUMENT,
                    "block-scale row strides must be >= in_features/32 bytes and multiples of 4");
    if (a->rows == 0) return ok();
    if (mx && (!a->a_block_scale || !a->w_block_scale || !aligned(a->a_block_scale, 4) ||
               !aligned(a->w_block_scale, 4)))
        return fail(QKNR_INVALID_ARGUMENT, "MX mode needs a_block_scale and w_block_scale, 4-byte aligned");
    if (!a->a || !a->w || !a->out) return fail(QKNR_INVALID_ARGUMENT, "a, w and out are required");
    if (!aligned(a->a, 16) || !aligned(a->w, 16) || !aligned(a->out, 16) || !aligned(a->bias, 2) ||
        !aligned(a->a_scale, 4) || !aligned(a->w_scale, 4))
        return fail(QKNR_UNSUPPORTED, "a, w and out must be 16-byte aligned (bias 2, scales 4)");
    if (a->q_cols && (!a->sumsq || !aligned(a->sumsq, 4)))
        return fail(QKNR_INVALID_ARGUMENT, "sumsq (4-byte aligned) is required when q_cols > 0");
    if (a->rows >= (1LL << 31) || a->out_features >= (1LL << 31) || a->in_features >= (1LL << 31))
        return fail(QKNR_UNSUPPORTED, "sizes of 2^31 or more");
    const int64_t tiles = ((a->rows + 255) / 256) * (a->out_features / 128);
    if (tiles >= (1LL << 31)) return fail(QKNR_UNSUPPORTED, "more than 2^31 tiles");
    auto span = [](const void *p, int64_t rows, int64_t stride, int64_t cols, int bytes) {
        const uintptr_t b = reinterpret_cast<uintptr_t>(p);
        return std::pair<uintptr_t, uintptr_t>(b, b + (uintptr_t)(((rows - 1) * stride + cols) * bytes));
    };
    const auto o = span(a->out, a->rows, a->out_row_stride, a->out_features, 2);
    const std::pair<uintptr_t, uintptr_t> none(0, 0);
    const std::pair<uintptr_t, uintptr_t> ins[] = {
        span(a->a, a->rows, a->a_row_stride, a->in_features, eb),
        span(a->w, a->out_features, a->w_row_stride, a->in_features, eb),
        a->bias ? span(a->bias, 1, 0, a->out_features, 2) : none,
        a->a_scale ? span(a->a_scale, 1, 0, a->rows, 4) : none,
        a->w_scale ? span(a->w_scale, 1, 0, a->out_features, 4) : none,
        mx ? span(a->a_block_scale, a->rows, a->a_block_scale_stride, blocks, 1) : none,
        mx ? span(a->w_block_scale, a->out_features, a->w_block_scale_stride, blocks, 1) : none};
    for (const auto &r : ins)
        if (r.first < o.second && o.first < r.second) return fail(QKNR_INVALID_ARGUMENT, "out overlaps an input");
    qknr::ProjParams p{};
    p.a = a->a; p.w = a->w; p.bias = a->bias; p.o = a->out; p.sumsq = a->sumsq;
    p.a_scale = a->a_scale; p.w_scale = a->w_scale;
    p.m = a->rows; p.n = a->out_features; p.k = a->in_features;
    p.lda = a->a_row_stride; p.ldw = a->w_row_stride; p.ldo = a->out_row_stride;
    p.q_cols = a->q_cols; p.k_cols = a->k_cols; p.parts = a->q_cols / 128;
    if (mx) {
        p.a_bs = a->a_block_scale; p.w_bs = a->w_block_scale;
        p.lda_bs = a->a_block_scale_stride; p.ldw_bs = a->w_block_scale_stride;
    }
    hipError_t e = qknr::proj_launch(p, fp8, stream);
    if (e != hipSuccess) return fail(QKNR_DEVICE_ERROR, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int32_t qknr_interleaved_to_rotate_half(const qknr_permute_args *a, hipStream_t stream) {
    if (!a) return fail(QKNR_INVALID_ARGUMENT, "args is NULL");
    if (a->elem_bytes != 1 && a->elem_bytes != 2 && a->elem_bytes != 4 && a->elem_bytes != 8)
        return fail(QKNR_INVALID_ARGUMENT, "elem_bytes must be 1, 2, 4 or 8");
    if (a->outer < 0 || a->axis_len < 1 || a->inner < 1 || a->first < 0 || a->n_heads < 0)
        return fail(QKNR_INVALID_ARGUMENT, "outer >= 0, axis_len >= 1, inner >= 1, first >= 0, n_heads >= 0");
    if (a->head_dim < 2 || (a->head_dim & 1)) return fail(QKNR_INVALID_ARGUMENT, "head_dim must be even and >= 2");
    if (a->first > a->axis_len || a->n_heads > (a->axis_len - a->first) / a->head_dim)
        return fail(QKNR_INVALID_ARGUMENT, "first + n_heads*head_dim exceeds axis_len");
    if (a->inner > (1LL << 40) || a->axis_len > (1LL << 40))
        return fail(QKNR_INVALID_ARGUMENT, "tensor too large");
    const int64_t index_bytes = a->inner * a->elem_bytes;
    if (a->outer && a->axis_len * index_bytes > (INT64_MAX / 2) / a->outer)
        return fail(QKNR_INVALID_ARGUMENT, "tensor too large");
    const int64_t bytes = a->outer * a->axis_len * index_bytes;
    if (bytes == 0) return ok();
    if (!a->src || !a->dst) return fail(QKNR_INVALID_ARGUMENT, "src and dst are required");
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(a->src), d0 = reinterpret_cast<uintptr_t>(a->dst);
    if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes)
        return fail(QKNR_INVALID_ARGUMENT, "src and dst overlap");
    int unit = 16;
    while (unit > 1 && (index_bytes % unit || !aligned(a->src, unit) || !aligned(a->dst, unit))) unit /= 2;
    qknr::PermuteParams p;
    p.src = a->src;
    p.dst = a->dst;
    p.outer = (uint64_t)a->outer;
    p.axis_len = (uint64_t)a->axis_len;
    p.units_per_index = (uint64_t)(index_bytes / unit);
    p.first = (uint64_t)a->first;
    p.n_heads = (uint64_t)a->n_heads;
    p.head_dim = (uint64_t)a->head_dim;
    p.inverse = a->inverse ? 1 : 0;
    hipError_t e = qknr::permute_launch(p, unit, stream);
    if (e != hipSuccess) return fail(QKNR_DEVICE_ERROR, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

int32_t qknr_kv_validate(const qknr_kv_args *args) {
    return kv_check(args, nullptr);
}

int32_t qknr_kv_rmsnorm_rope_cache(const qknr_kv_args *args, hipStream_t stream) {
    KvPlan plan;
    int32_t rc = kv_check(args, &plan);
    if (rc != QKNR_OK) return rc;
    hipError_t e = qknr::kv_launch(plan.p, plan.elem_type, plan.vec, plan.v2, stream);
    if (e != hipSuccess) return fail(QKNR_DEVICE_ERROR, "launch failed: %s", hipGetErrorString(e));
    return QKNR_OK;
}

const char *qknr_last_error(void) {
    return g_last_error.c_str();
}

int32_t qknr_version(void) {
    return QKNR_ABI_VERSION;
}

}  // extern "C"
