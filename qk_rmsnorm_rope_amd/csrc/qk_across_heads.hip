// qk_across_heads.hip -- across-heads QK RMSNorm + rotate-half RoPE for gfx950.
//
// The operation is the one the "Kernel reference: qkv_cte" page describes in
// Design section 1 (one RMS per token over the whole Q segment and the whole
// K segment, segment-wide gamma, steps a-c) and section 2 (rotate-half RoPE on
// the same pass, inv_rms folded into the cos/sin products), with every head on
// one GPU so step b's all-reduce disappears (tp = 1).
//
// MI355X design (not the Trainium one): the pass is HBM-bound (about 2 flops
// per byte), so the kernel is exactly one read and one write of Q|K:
//   * one wavefront per (token, segment) unit -- the Q segment and the K
//     segment of a token are independent reductions, so splitting them halves
//     the registers a wave holds and doubles the waves in flight; very wide
//     segments use W = 2 or 4 waves per unit, joined through LDS;
//   * each lane owns the chunk pair (i, i + d/2) of J heads, so the
//     rotate-half partner of every element is in the same lane: no shuffles;
//   * lane k of every head group reads the same cos/sin chunks, so each lane
//     loads its cos/sin once per unit and reuses them for all its heads;
//   * 16-byte non-temporal loads and stores for Q/K (read once, written once),
//     ordinary cached loads for the reused gammas and position tables; the
//     gammas of all of a lane's heads are requested with the data, so their
//     latency hides under the HBM latency;
//   * addresses are a wave-uniform 64-bit base (scalar registers) plus a
//     32-bit per-lane offset, and the head geometry is a compile-time constant
//     for the usual head sizes, so address arithmetic costs few VGPRs;
//   * the sum of squares is fp32 (v_dot2 on packed 16-bit pairs), reduced with
//     DPP inside the wave, and inv_rms is folded into cos/sin once per lane:
//     per element y = x*gamma; out = y*(r*cos) -/+ y_partner*(r*sin).
#include "device_common.h"
#include "launch.h"

#ifndef QKNR_QK_STREAMING
#define QKNR_QK_STREAMING 1   // non-temporal Q/K loads and stores
#endif

namespace qknr {

template <typename T, int VEC>
__device__ __forceinline__ void load_stream(Chunk<T, VEC> &c, const T *p) {
#if QKNR_QK_STREAMING
    c.load_nt(p);
#else
    c.load(p);
#endif
}

template <typename T, int VEC>
__device__ __forceinline__ void store_stream(T *p, const float *v) {
#if QKNR_QK_STREAMING
    store_vec_nt<T, VEC>(p, v);
#else
    store_vec<T, VEC>(p, v);
#endif
}

// KC: chunks per half head known at compile time (0: read p.chunks_per_half).
template <typename T, int VEC, int KC, int J>
__global__ __launch_bounds__(256) void qk_across_heads_kernel(QkParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0..3, wave-uniform
    const int W = p.waves_per_unit;
    const int unit_in_block = wave / W;
    const int wave_in_unit = wave - unit_in_block * W;
    const uint32_t unit = blockIdx.x * (uint32_t)(4 / W) + unit_in_block;
    const uint32_t t = p.segs == 2 ? unit >> 1 : unit;
    const int seg = p.segs == 2 ? (int)(unit & 1u) : 0;
    const bool unit_ok = t < p.tokens;
    if (W == 1 && !unit_ok) return;                     // no barrier follows when W == 1

    const int kc = KC ? KC : p.chunks_per_half;
    const int hpw = 64 / kc;                            // heads covered by one wave step
    const int half = kc * VEC;
    const int k = lane % kc;
    const int hsub = lane / kc;
    const bool lane_ok = unit_ok && hsub < hpw;

    uint32_t b = 0, s = 0;
    if (unit_ok) {
        b = fastdiv(t, p.seq_div);
        s = t - b * p.seq;
    }
    const int nh = seg ? p.n_k : p.n_q;
    const T *x = reinterpret_cast<const T *>(seg ? p.k_in : p.q_in) + b * p.in_batch_stride +
                 s * p.in_token_stride;
    // per-lane byte offset inside the token (32-bit; checked on the host)
    const uint32_t lane_in = ((uint32_t)hsub * p.in_head_stride + (uint32_t)(k * VEC)) * (uint32_t)sizeof(T);

    Chunk<T, VEC> lo[J], hi[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int hb = (j * W + wave_in_unit) * hpw;    // first head of this step (uniform)
        const char *xj = reinterpret_cast<const char *>(x + (uint64_t)hb * p.in_head_stride) + lane_in;
        if (lane_ok && hb + hsub < nh) {
            load_stream<T, VEC>(lo[j], reinterpret_cast<const T *>(xj));
            load_stream<T, VEC>(hi[j], reinterpret_cast<const T *>(xj) + half);
        } else {
            lo[j].zero();
            hi[j].zero();
        }
    }

    // Gammas of all J heads are requested together with the data: their cached
    // (L2) latency then overlaps the HBM latency instead of serialising one
    // round trip per head in the apply loop.
    const T *g = reinterpret_cast<const T *>(seg ? p.k_gamma : p.q_gamma);
    const uint32_t lane_g = (uint32_t)(hsub * p.head_dim + k * VEC) * (uint32_t)sizeof(T);
    const bool norm = p.apply_norm != 0;
    Chunk<T, VEC> glo[J], ghi[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int hb = (j * W + wave_in_unit) * hpw;
        if (norm && lane_ok && hb + hsub < nh) {
            const T *gj = reinterpret_cast<const T *>(reinterpret_cast<const char *>(g + (uint64_t)hb * p.head_dim) +
                                                      lane_g);
            glo[j].load(gj);
            ghi[j].load(gj + half);
        } else {
            glo[j].zero();
            ghi[j].zero();
        }
    }

    Chunk<T, VEC> c_lo, c_hi, s_lo, s_hi;
    const bool rope = p.apply_rope != 0;
    if (rope && lane_ok) {
        const int64_t rb = b * p.rope_batch_stride + s * p.rope_token_stride + k * VEC;
        const T *cs = reinterpret_cast<const T *>(p.cos) + rb;
        const T *sn = reinterpret_cast<const T *>(p.sin) + rb;
        c_lo.load(cs);
        c_hi.load(cs + half);
        s_lo.load(sn);
        s_hi.load(sn + half);
    }

    float r = 1.0f;
    if (p.apply_norm) {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < J; j++) ss = hi[j].sumsq(lo[j].sumsq(ss));
        ss = wave_sum(ss);
        if (W > 1) {
            __shared__ float part[4];
            if (lane == 0) part[wave] = ss;
            __syncthreads();
            ss = 0.0f;
            for (int w = 0; w < W; w++) ss += part[unit_in_block * W + w];   // fixed order
        }
        r = rsqrtf(ss / (seg ? p.k_channels : p.q_channels) + p.eps);
    }
    if (!lane_ok) return;

    // inv_rms folded into the rotation coefficients
    float rc_lo[VEC], rc_hi[VEC], rs_lo[VEC], rs_hi[VEC];
    if (rope) {
        c_lo.decode(rc_lo);
        c_hi.decode(rc_hi);
        s_lo.decode(rs_lo);
        s_hi.decode(rs_hi);
#pragma unroll
        for (int e = 0; e < VEC; e++) { rc_lo[e] *= r; rc_hi[e] *= r; rs_lo[e] *= r; rs_hi[e] *= r; }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; e++) { rc_lo[e] = r; rc_hi[e] = r; rs_lo[e] = 0.0f; rs_hi[e] = 0.0f; }
    }

    T *o = reinterpret_cast<T *>(seg ? p.k_out : p.q_out) + b * p.out_batch_stride + s * p.out_token_stride;
    const uint32_t lane_out = ((uint32_t)hsub * p.out_head_stride + (uint32_t)(k * VEC)) * (uint32_t)sizeof(T);

#pragma unroll
    for (int j = 0; j < J; j++) {
        const int hb = (j * W + wave_in_unit) * hpw;
        if (hb + hsub >= nh) continue;
        float xl[VEC], xh[VEC], gl[VEC], gh[VEC], ol[VEC], oh[VEC];
        lo[j].decode(xl);
        hi[j].decode(xh);
        if (norm) {
            glo[j].decode(gl);
            ghi[j].decode(gh);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; e++) { gl[e] = 1.0f; gh[e] = 1.0f; }
        }
#pragma unroll
        for (int e = 0; e < VEC; e++) {
            const float yl = xl[e] * gl[e];
            const float yh = xh[e] * gh[e];
            ol[e] = fmaf(yl, rc_lo[e], -(yh * rs_lo[e]));
            oh[e] = fmaf(yh, rc_hi[e], yl * rs_hi[e]);
        }
        T *oj = reinterpret_cast<T *>(reinterpret_cast<char *>(o + (uint64_t)hb * p.out_head_stride) + lane_out);
        store_stream<T, VEC>(oj, ol);
        store_stream<T, VEC>(oj + half, oh);
    }
}

// ---------------------------------------------------------------------------
// launcher: picks the head-geometry specialisation, W and J
// ---------------------------------------------------------------------------

template <typename T, int VEC, int KC>
static hipError_t launch_kc(const QkParams &p, int J, hipStream_t stream) {
    const uint32_t units = p.tokens * (uint32_t)p.segs;
    const uint32_t per_block = 4 / p.waves_per_unit;
    dim3 grid((units + per_block - 1) / per_block), block(256);
#define QKNR_CASE(JJ) \
    case JJ: hipLaunchKernelGGL((qk_across_heads_kernel<T, VEC, KC, JJ>), grid, block, 0, stream, p); break;
    switch (J) {
        QKNR_CASE(1) QKNR_CASE(2) QKNR_CASE(3) QKNR_CASE(4) QKNR_CASE(5) QKNR_CASE(6) QKNR_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef QKNR_CASE
    return hipGetLastError();
}

template <typename T, int VEC>
static hipError_t launch_vec(const QkParams &p, int J, hipStream_t stream) {
    switch (p.chunks_per_half) {
    case 4: return launch_kc<T, VEC, 4>(p, J, stream);
    case 8: return launch_kc<T, VEC, 8>(p, J, stream);
    case 16: return launch_kc<T, VEC, 16>(p, J, stream);
    default: return launch_kc<T, VEC, 0>(p, J, stream);
    }
}

static int round_up_j(int j) {
    if (j <= 6) return j;
    if (j <= 8) return 8;
    return -1;
}

int qk_plan(QkParams &p, int vec) {
    const int half = p.head_dim / 2;
    if (half % vec) return -1;
    const int kc = half / vec;
    if (kc > 64) return -1;
    const int hpw = 64 / kc;
    const int heads = p.n_q > p.n_k ? p.n_q : p.n_k;
    for (int W = 1; W <= 4; W *= 2) {
        const int J = round_up_j((heads + hpw * W - 1) / (hpw * W));
        if (J > 0) {
            p.half = half;
            p.chunks_per_half = kc;
            p.heads_per_step = hpw;
            p.waves_per_unit = W;
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
        return vec == 4 ? launch_vec<float, 4>(p, J, stream) : launch_kc<float, 1, 0>(p, J, stream);
    case 1:  // bf16: 16-byte chunks, or pairs
        return vec == 8 ? launch_vec<bf16_t, 8>(p, J, stream) : launch_kc<bf16_t, 2, 0>(p, J, stream);
    case 2:  // f16
        return vec == 8 ? launch_vec<f16_t, 8>(p, J, stream) : launch_kc<f16_t, 2, 0>(p, J, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qknr
