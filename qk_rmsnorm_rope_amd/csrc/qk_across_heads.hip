// qk_across_heads.hip -- across-heads QK RMSNorm + rotate-half RoPE for gfx950.
//
// The operation is the one the "Kernel reference: qkv_cte" page describes in
// Design section 1 (one RMS per token over the whole Q segment and the whole
// K segment, segment-wide gamma, steps a-c) and section 2 (rotate-half RoPE on
// the same pass, inv_rms folded into the cos/sin products), with every head on
// one GPU so step b's all-reduce disappears (tp = 1).
//
// MI355X design (not the Trainium one): the pass is HBM-bound (about 2 flops
// per byte), so the kernel is one read and one write of Q|K:
//   * one wavefront per token (W = 1) or W waves per token for very wide
//     segments; each lane owns the chunk pair (i, i + d/2) of J heads, so the
//     rotate-half partner of every element is in the same lane and no
//     cross-lane shuffle is needed;
//   * lane k of every head group reads the same cos/sin chunks, so each lane
//     loads its cos/sin once per token and reuses it for all its heads and
//     for both segments;
//   * 16-byte loads and stores (8 bf16 or 4 fp32 per access); consecutive
//     lanes cover whole 128-byte lines;
//   * the sum of squares is fp32 in registers, reduced across the wave with
//     DPP (no LDS), across waves through LDS when W > 1;
//   * inv_rms is multiplied into cos and sin once per lane
//     (r*cos, r*sin), so the per-element work is
//     y = x*gamma; out = y*rc - y_partner*rs.
#include "device_common.h"
#include "launch.h"

namespace qknr {

template <typename T, int VEC, int J>
__global__ __launch_bounds__(256) void qk_across_heads_kernel(QkParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;                 // 0..3
    const int W = p.waves_per_token;                   // 1, 2 or 4
    const int token_in_block = wave / W;
    const int wave_in_token = wave - token_in_block * W;
    const int64_t t = (int64_t)blockIdx.x * (4 / W) + token_in_block;
    const bool token_ok = t < p.tokens;

    const int kc = p.chunks_per_half;                  // d/2 / VEC
    const int hpw = p.heads_per_step;                  // 64 / kc
    const int k = lane % kc;
    const int hsub = lane / kc;
    const bool lane_ok = token_ok && hsub < hpw;
    const int half = p.half;

    int64_t b = 0, s = 0;
    if (token_ok) { b = t / p.seq; s = t - b * p.seq; }
    const int64_t in_base = b * p.in_batch_stride + s * p.in_token_stride;
    const int64_t out_base = b * p.out_batch_stride + s * p.out_token_stride;
    const int64_t rope_base = b * p.rope_batch_stride + s * p.rope_token_stride;

    const T *qi = reinterpret_cast<const T *>(p.q_in);
    const T *ki = reinterpret_cast<const T *>(p.k_in);

    // Raw (packed) chunks of this lane's heads: (lo, hi) = lanes [kVEC, kVEC+VEC)
    // and their rotate-half partners d/2 further on.
    Chunk<T, VEC> qlo[J], qhi[J], klo[J], khi[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int h = (j * W + wave_in_token) * hpw + hsub;
        const int64_t off = in_base + (int64_t)h * p.in_head_stride + k * VEC;
        if (lane_ok && h < p.n_q) {
            qlo[j].load(qi + off);
            qhi[j].load(qi + off + half);
        } else {
            qlo[j].zero();
            qhi[j].zero();
        }
        if (lane_ok && h < p.n_k) {
            klo[j].load(ki + off);
            khi[j].load(ki + off + half);
        } else {
            klo[j].zero();
            khi[j].zero();
        }
    }

    Chunk<T, VEC> c_lo, c_hi, s_lo, s_hi;
    const bool rope = p.apply_rope != 0;
    if (rope && lane_ok) {
        const T *cs = reinterpret_cast<const T *>(p.cos) + rope_base + k * VEC;
        const T *sn = reinterpret_cast<const T *>(p.sin) + rope_base + k * VEC;
        c_lo.load(cs);
        c_hi.load(cs + half);
        s_lo.load(sn);
        s_hi.load(sn + half);
    }

    float rq = 1.0f, rk = 1.0f;
    if (p.apply_norm) {
        float sq = 0.0f, sk = 0.0f;
#pragma unroll
        for (int j = 0; j < J; j++) {
            sq = qhi[j].sumsq(qlo[j].sumsq(sq));
            sk = khi[j].sumsq(klo[j].sumsq(sk));
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        if (W > 1) {
            __shared__ float part[4][2];
            if (lane == 0) { part[wave][0] = sq; part[wave][1] = sk; }
            __syncthreads();
            sq = 0.0f;
            sk = 0.0f;
            for (int w = 0; w < W; w++) {                 // fixed order: deterministic
                sq += part[token_in_block * W + w][0];
                sk += part[token_in_block * W + w][1];
            }
        }
        rq = rsqrtf(sq / p.q_channels + p.eps);
        rk = rsqrtf(sk / p.k_channels + p.eps);
    }
    if (!lane_ok) return;

    // inv_rms folded into the rotation coefficients, one set per segment:
    //   out_lo = y_lo*(r*cos_lo) - y_hi*(r*sin_lo),  out_hi = y_hi*(r*cos_hi) + y_lo*(r*sin_hi)
    float qc_lo[VEC], qc_hi[VEC], qs_lo[VEC], qs_hi[VEC];
    float kc_lo[VEC], kc_hi[VEC], ks_lo[VEC], ks_hi[VEC];
    {
        float clo[VEC], chi[VEC], slo[VEC], shi[VEC];
        if (rope) {
            c_lo.decode(clo); c_hi.decode(chi); s_lo.decode(slo); s_hi.decode(shi);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; e++) { clo[e] = 1.0f; chi[e] = 1.0f; slo[e] = 0.0f; shi[e] = 0.0f; }
        }
#pragma unroll
        for (int e = 0; e < VEC; e++) {
            qc_lo[e] = rq * clo[e]; qc_hi[e] = rq * chi[e]; qs_lo[e] = rq * slo[e]; qs_hi[e] = rq * shi[e];
            kc_lo[e] = rk * clo[e]; kc_hi[e] = rk * chi[e]; ks_lo[e] = rk * slo[e]; ks_hi[e] = rk * shi[e];
        }
    }

    T *qo = reinterpret_cast<T *>(p.q_out);
    T *ko = reinterpret_cast<T *>(p.k_out);
    const T *qg = reinterpret_cast<const T *>(p.q_gamma);
    const T *kg = reinterpret_cast<const T *>(p.k_gamma);
    const bool norm = p.apply_norm != 0;

#pragma unroll
    for (int j = 0; j < J; j++) {
        const int h = (j * W + wave_in_token) * hpw + hsub;
        const int64_t off = out_base + (int64_t)h * p.out_head_stride + k * VEC;
        const int64_t goff = (int64_t)h * p.head_dim + k * VEC;
#pragma unroll
        for (int seg = 0; seg < 2; seg++) {
            const int nh = seg == 0 ? p.n_q : p.n_k;
            if (h >= nh) continue;
            const T *g = seg == 0 ? qg : kg;
            T *o = seg == 0 ? qo : ko;
            const float *cl = seg == 0 ? qc_lo : kc_lo;
            const float *ch = seg == 0 ? qc_hi : kc_hi;
            const float *sl = seg == 0 ? qs_lo : ks_lo;
            const float *sh = seg == 0 ? qs_hi : ks_hi;
            float xlo[VEC], xhi[VEC], glo[VEC], ghi[VEC], olo[VEC], ohi[VEC];
            (seg == 0 ? qlo[j] : klo[j]).decode(xlo);
            (seg == 0 ? qhi[j] : khi[j]).decode(xhi);
            if (norm) {
                load_vec<T, VEC>(g + goff, glo);
                load_vec<T, VEC>(g + goff + half, ghi);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; e++) { glo[e] = 1.0f; ghi[e] = 1.0f; }
            }
#pragma unroll
            for (int e = 0; e < VEC; e++) {
                const float ylo = xlo[e] * glo[e];
                const float yhi = xhi[e] * ghi[e];
                olo[e] = fmaf(ylo, cl[e], -(yhi * sl[e]));
                ohi[e] = fmaf(yhi, ch[e], ylo * sh[e]);
            }
            store_vec<T, VEC>(o + off, olo);
            store_vec<T, VEC>(o + off + half, ohi);
        }
    }
}

// ---------------------------------------------------------------------------
// launcher: picks VEC (16-byte or scalar access), W and J
// ---------------------------------------------------------------------------

template <typename T, int VEC>
static hipError_t launch_vec(const QkParams &p, int J, hipStream_t stream) {
    const int tokens_per_block = 4 / p.waves_per_token;
    const int64_t blocks = (p.tokens + tokens_per_block - 1) / tokens_per_block;
    dim3 grid((unsigned)blocks), block(256);
#define QKNR_CASE(JJ) \
    case JJ: hipLaunchKernelGGL((qk_across_heads_kernel<T, VEC, JJ>), grid, block, 0, stream, p); break;
    switch (J) {
        QKNR_CASE(1) QKNR_CASE(2) QKNR_CASE(3) QKNR_CASE(4) QKNR_CASE(5) QKNR_CASE(6) QKNR_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef QKNR_CASE
    return hipGetLastError();
}

static int round_up_j(int j) {
    if (j <= 6) return j;
    if (j <= 8) return 8;
    return -1;
}

// Geometry only (host side, no device access): fills chunks_per_half,
// heads_per_step, waves_per_token and returns J (> 0), or -1 if the shape does
// not fit the register budget of one 256-thread block.
int qk_plan(QkParams &p, int vec) {
    const int half = p.head_dim / 2;
    if (half % vec) return -1;
    const int kc = half / vec;
    if (kc > 64) return -1;
    const int hpw = 64 / kc;
    const int heads = p.n_q > p.n_k ? p.n_q : p.n_k;
    for (int W = 1; W <= 4; W *= 2) {
        int J = (heads + hpw * W - 1) / (hpw * W);
        J = round_up_j(J);
        if (J > 0) {
            p.half = half;
            p.chunks_per_half = kc;
            p.heads_per_step = hpw;
            p.waves_per_token = W;
            return J;
        }
    }
    return -1;
}

hipError_t qk_launch(QkParams &p, int elem_type, int vec, hipStream_t stream) {
    const int J = qk_plan(p, vec);
    if (J < 0) return hipErrorInvalidValue;
    if (p.tokens == 0) return hipSuccess;
    switch (elem_type) {
    case 0:  // f32: 16-byte chunks, or single elements
        return vec == 4 ? launch_vec<float, 4>(p, J, stream) : launch_vec<float, 1>(p, J, stream);
    case 1:  // bf16: 16-byte chunks, or pairs
        return vec == 8 ? launch_vec<bf16_t, 8>(p, J, stream) : launch_vec<bf16_t, 2>(p, J, stream);
    case 2:  // f16
        return vec == 8 ? launch_vec<f16_t, 8>(p, J, stream) : launch_vec<f16_t, 2>(p, J, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qknr
