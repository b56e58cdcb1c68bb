// qk_kernel.h -- the QK RMSNorm + rotate-half RoPE kernel for gfx950, in the
// four forms of QkMode (launch.h). Each form is instantiated by its own
// translation unit: qk_across_heads.hip, qk_per_head.hip, qk_split.hip.
//
// The operation is the one the "Kernel reference: qkv_cte" page describes in
// Design section 1 (one RMS per token over the whole Q segment and the whole
// K segment, segment-wide gamma, steps a-c) and section 2 (rotate-half RoPE on
// the same pass, inv_rms folded into the cos/sin products). With every head on
// one GPU step b's all-reduce disappears (QK_ACROSS); with the heads split over
// ranks, step a is QK_SUMSQ and step c is QK_APPLY, the caller adding the
// ranks' sums in between. QK_PER_HEAD is the upstream per-head qk-norm the
// page contrasts it with ("Upstream behavior").
//
// MI355X design (not the Trainium one): the pass is HBM-bound (about 2 flops
// per byte), so the kernel is exactly one read and one write of Q|K:
//   * one wavefront per (token, segment) unit -- the Q segment and the K
//     segment of a token are independent reductions, so splitting them halves
//     the registers a wave holds and doubles the waves in flight; very wide
//     segments use W = 2 or 4 waves per unit, joined through LDS;
//   * each lane owns the chunk pair (i, i + d/2) of J heads, so the
//     rotate-half partner of every element is in the same lane: no shuffles;
//     the kc lanes of one head are consecutive, so a per-head sum is a
//     kc-lane group reduction;
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
//     per element y = x*gamma; out = y*(r*cos) -/+ y_partner*(r*sin). Per
//     head, r differs between a lane's heads and is folded into gamma instead.
#pragma once

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

// Sum of v over the kc consecutive lanes of one head (lanes hsub*kc ..
// hsub*kc + kc - 1); every lane of the group gets the same bits. Power-of-two
// groups reduce with DPP; other widths add the group's values in lane order
// through ds_bpermute. Must be called with the whole wave active.
__device__ __forceinline__ float head_sum(float v, int kc, int lane) {
    switch (kc) {
    case 1: return v;
    case 2: return v + dpp_quad_xor1(v);
    case 4: return group_sum<4>(v);
    case 8: return group_sum<8>(v);
    case 16: return group_sum<16>(v);
    case 32: return group_sum<32>(v);
    case 64: return group_sum<64>(v);
    default: {
        const int base = (lane / kc) * kc;
        float acc = 0.0f;
        for (int i = 0; i < kc; i++)
            acc += __int_as_float(__builtin_amdgcn_ds_bpermute(((base + i) & 63) << 2, __float_as_int(v)));
        return acc;
    }
    }
}

// KC: chunks per half head known at compile time (0: read p.chunks_per_half).
template <typename T, int VEC, int KC, int J, int MODE>
__global__ __launch_bounds__(256) void qk_kernel(QkParams p) {
    constexpr bool kApply = MODE != QK_SUMSQ;     // writes Q/K
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

    // Gammas are requested together with the data: their cached (L2) latency
    // then overlaps the HBM latency instead of serialising one round trip per
    // head in the apply loop. Across heads each head has its own slice of the
    // segment-wide gamma; per head one [head_dim] gamma serves every head.
    const T *g = reinterpret_cast<const T *>(seg ? p.k_gamma : p.q_gamma);
    const bool norm = p.apply_norm != 0;
    constexpr int JG = MODE == QK_PER_HEAD ? 1 : (kApply ? J : 0);
    Chunk<T, VEC> glo[JG > 0 ? JG : 1], ghi[JG > 0 ? JG : 1];
    if constexpr (MODE == QK_PER_HEAD) {
        if (norm && lane_ok) {
            glo[0].load(g + k * VEC);
            ghi[0].load(g + k * VEC + half);
        } else {
            glo[0].zero();
            ghi[0].zero();
        }
    } else if constexpr (kApply) {
        const uint32_t lane_g = (uint32_t)(hsub * p.head_dim + k * VEC) * (uint32_t)sizeof(T);
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int hb = (j * W + wave_in_unit) * hpw;
            if (norm && lane_ok && hb + hsub < nh) {
                const T *gj = reinterpret_cast<const T *>(
                    reinterpret_cast<const char *>(g + (uint64_t)hb * p.head_dim) + lane_g);
                glo[j].load(gj);
                ghi[j].load(gj + half);
            } else {
                glo[j].zero();
                ghi[j].zero();
            }
        }
    }

    Chunk<T, VEC> c_lo, c_hi, s_lo, s_hi;
    const bool rope = p.apply_rope != 0;
    if (kApply && rope && lane_ok) {
        const int64_t rb = b * p.rope_batch_stride + s * p.rope_token_stride + k * VEC;
        const T *cs = reinterpret_cast<const T *>(p.cos) + rb;
        const T *sn = reinterpret_cast<const T *>(p.sin) + rb;
        c_lo.load(cs);
        c_hi.load(cs + half);
        s_lo.load(sn);
        s_hi.load(sn + half);
    }

    float r = 1.0f;          // QK_ACROSS / QK_APPLY: the segment's inverse RMS
    float rh[J];             // QK_PER_HEAD: one inverse RMS per head of the lane
#pragma unroll
    for (int j = 0; j < J; j++) rh[j] = 1.0f;
    if constexpr (MODE == QK_ACROSS || MODE == QK_SUMSQ) {
        if (MODE == QK_SUMSQ || norm) {
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
            if constexpr (MODE == QK_SUMSQ) {
                // one vector store per unit, by lane 0 of its first wave
                if (unit_ok && wave_in_unit == 0 && lane == 0) p.sumsq[(uint32_t)seg * p.tokens + t] = ss;
                return;
            }
            r = rsqrtf(ss / (seg ? p.k_channels : p.q_channels) + p.eps);
        }
    } else if constexpr (MODE == QK_APPLY) {
        if (norm && unit_ok) {
            // the token's partial sums (one per projection tile; one in all when
            // the ranks' sums were already added) are contiguous: lane i loads
            // part i, and a fixed DPP tree adds them (the whole wave is active)
            const float *sp = p.sumsq + ((uint64_t)seg * p.tokens + t) * (uint32_t)p.sum_parts;
            float ss = 0.0f;
            for (int i0 = 0; i0 < p.sum_parts; i0 += 64) {
                const float v = i0 + lane < p.sum_parts ? sp[i0 + lane] : 0.0f;
                ss += wave_sum(v);
            }
            r = rsqrtf(ss / (seg ? p.k_channels : p.q_channels) + p.eps);
        }
    } else {   // QK_PER_HEAD
        if (norm) {
#pragma unroll
            for (int j = 0; j < J; j++) {
                const float ss = head_sum(hi[j].sumsq(lo[j].sumsq(0.0f)), kc, lane);
                rh[j] = rsqrtf(ss / (float)p.head_dim + p.eps);
            }
        }
    }
    if constexpr (kApply) {
        if (!lane_ok) return;

        // inv_rms folded into the rotation coefficients (per head: r = 1 here)
        float rc_lo[VEC], rc_hi[VEC], rs_lo[VEC], rs_hi[VEC];
        if (rope) {
            c_lo.decode(rc_lo);
            c_hi.decode(rc_hi);
            s_lo.decode(rs_lo);
            s_hi.decode(rs_hi);
            if (MODE != QK_PER_HEAD) {
#pragma unroll
                for (int e = 0; e < VEC; e++) { rc_lo[e] *= r; rc_hi[e] *= r; rs_lo[e] *= r; rs_hi[e] *= r; }
            }
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
                constexpr int JJ = MODE == QK_PER_HEAD ? 0 : 1;
                glo[JJ * j].decode(gl);
                ghi[JJ * j].decode(gh);
                if (MODE == QK_PER_HEAD) {
#pragma unroll
                    for (int e = 0; e < VEC; e++) { gl[e] *= rh[j]; gh[e] *= rh[j]; }
                }
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
}

// ---------------------------------------------------------------------------
// launch helpers: the head-geometry specialisation and J
// ---------------------------------------------------------------------------

template <typename T, int VEC, int KC, int MODE>
static hipError_t qk_launch_kc(const QkParams &p, int J, hipStream_t stream) {
    const uint32_t units = p.tokens * (uint32_t)p.segs;
    const uint32_t per_block = 4 / p.waves_per_unit;
    dim3 grid((units + per_block - 1) / per_block), block(256);
#define QKNR_CASE(JJ) \
    case JJ: hipLaunchKernelGGL((qk_kernel<T, VEC, KC, JJ, MODE>), grid, block, 0, stream, p); break;
    switch (J) {
        QKNR_CASE(1) QKNR_CASE(2) QKNR_CASE(3) QKNR_CASE(4) QKNR_CASE(5) QKNR_CASE(6) QKNR_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef QKNR_CASE
    return hipGetLastError();
}

template <typename T, int VEC, int MODE>
static hipError_t qk_launch_vec(const QkParams &p, int J, hipStream_t stream) {
    switch (p.chunks_per_half) {
    case 4: return qk_launch_kc<T, VEC, 4, MODE>(p, J, stream);
    case 8: return qk_launch_kc<T, VEC, 8, MODE>(p, J, stream);
    case 16: return qk_launch_kc<T, VEC, 16, MODE>(p, J, stream);
    default: return qk_launch_kc<T, VEC, 0, MODE>(p, J, stream);
    }
}

// elem_type: 0 f32 (16-byte chunks, or single elements), 1 bf16 and 2 f16
// (16-byte chunks, or pairs).
template <int MODE>
static hipError_t qk_launch_mode(const QkParams &p, int elem_type, int vec, int J, hipStream_t stream) {
    switch (elem_type) {
    case 0: return vec == 4 ? qk_launch_vec<float, 4, MODE>(p, J, stream) : qk_launch_kc<float, 1, 0, MODE>(p, J, stream);
    case 1: return vec == 8 ? qk_launch_vec<bf16_t, 8, MODE>(p, J, stream) : qk_launch_kc<bf16_t, 2, 0, MODE>(p, J, stream);
    case 2: return vec == 8 ? qk_launch_vec<f16_t, 8, MODE>(p, J, stream) : qk_launch_kc<f16_t, 2, 0, MODE>(p, J, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace qknr
