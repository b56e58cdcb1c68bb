// kv_rmsnorm_rope_cache.hip -- the KvRmsNormRopeCache operator for gfx950.
//
// Computes, per (b, n, s) row, the CANN page's formulas: (1) RmsNorm over the
// first rms_size values, (2) interleaveRope (V1: on the raw tail; V2: on the
// first rope_size normed values, which it replaces), (3) static quantisation
// per cache, (4) scatter of the k and ckv rows to the slot index(b, s) of a
// Norm or paged (PA_BNSD) cache, (5) optional raw outputs k_rope / c_kv.
//
// MI355X design: the operator is HBM-bound, so each row is read once and every
// output row is written once, in one pass:
//   * a group of G lanes (8..64, a power of two) owns one row; 64/G rows per
//     wavefront, 256/G per block. Lane l of a group owns the 8-element chunks
//     l, l+G, l+2G, ... of the row (16-byte loads of bf16/f16);
//   * the sum of squares reduces inside the group with DPP / ds_swizzle (no
//     LDS, no barrier); the result is bit-identical in every lane of the group;
//   * an interleaved input chunk (pairs 2j, 2j+1) produces half a chunk of the
//     even-lane outputs (positions j) and half a chunk of the odd-lane outputs
//     (positions j + R/2), so the rotation needs no data exchange between
//     lanes: each lane writes two half-chunks;
//   * quantisation (int8 RNE + clamp, or FP8 E4M3FN RNE saturating) is fused
//     into the stores; each cache row is written by whole-chunk vector stores
//     to its slot, so there are no atomics and each output byte has one writer;
//   * an index of -1 (or, defensively, outside the cache) writes no cache row;
//   * data read once (kv, v, per-row cos/sin) moves with non-temporal loads;
//     k_rope / c_kv and cache rows made of whole 128-byte lines with
//     non-temporal stores; cache rows that cover lines only in part (e.g. 192-
//     or 64-byte int8 rows) with ordinary stores, so that neighbouring rows
//     written by other waves merge in L2 before they reach HBM; gamma and the
//     quantisation parameters, reused by every row, stay cached;
//   * row -> (b, n, s) and slot -> (block, offset) use multiply-high division
//     by the invariant sizes instead of 64-bit divides.
#include "device_common.h"
#include "launch.h"

namespace qknr {

// Store N codes (one byte each) at p (naturally aligned).
template <int N>
__device__ __forceinline__ void store_codes(void *p, const uint32_t *code, bool nt) {
    if constexpr (N >= 4) {
        constexpr int W = N / 4;
        Words<W> r;
#pragma unroll
        for (int i = 0; i < W; i++)
            r.w[i] = code[4 * i] | (code[4 * i + 1] << 8) | (code[4 * i + 2] << 16) | (code[4 * i + 3] << 24);
        if (nt) store_words_nt<W>(p, r); else store_words<W>(p, r);
    } else if constexpr (N == 2) {
        *reinterpret_cast<uint16_t *>(p) = (uint16_t)(code[0] | (code[1] << 8));
    } else {
        *reinterpret_cast<uint8_t *>(p) = (uint8_t)code[0];
    }
}

// N consecutive fp32 quantisation parameters starting at channel c of head n.
template <int N>
__device__ __forceinline__ void load_qparam(const float *p, int shape, int n, int width, int c, float *out) {
    if (shape == QS_SCALAR) {
        const float v = p[0];
#pragma unroll
        for (int i = 0; i < N; i++) out[i] = v;
        return;
    }
    const float *q = p + (shape == QS_HEAD_CHANNEL ? (int64_t)n * width : 0) + c;
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; i++) {
            float4 v = reinterpret_cast<const float4 *>(q)[i];
            out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
        }
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; i++) {
            float2 v = reinterpret_cast<const float2 *>(q)[i];
            out[2 * i] = v.x; out[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) out[i] = q[i];
    }
}

// Write N values of one cache row starting at channel c: quantised (int8 /
// E4M3FN, t = x*scale (+offset) in fp32 with one rounding) or rounded to T.
template <typename T, int N>
__device__ __forceinline__ void put_cache(void *row, int code, int c, const float *x,
                                          const float *scale, const float *offset, int qshape,
                                          int n, int width, bool nt) {
    if (code == CODE_SAME) {
        if (nt) store_vec_nt<T, N>(reinterpret_cast<T *>(row) + c, x);
        else store_vec<T, N>(reinterpret_cast<T *>(row) + c, x);
        return;
    }
    float sc[N], of[N];
    load_qparam<N>(scale, qshape, n, width, c, sc);
    if (offset) {
        load_qparam<N>(offset, qshape, n, width, c, of);
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) of[i] = 0.0f;
    }
    uint32_t q[N];
    if (code == CODE_INT8) {
#pragma unroll
        for (int i = 0; i < N; i++) q[i] = enc_int8(fmaf(x[i], sc[i], of[i]));
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) q[i] = enc_e4m3fn(fmaf(x[i], sc[i], of[i]));
    }
    store_codes<N>(reinterpret_cast<uint8_t *>(row) + c, q, nt);
}

__device__ __forceinline__ float row_sum(float v, int G) {
    switch (G) {
    case 8: return group_sum<8>(v);
    case 16: return group_sum<16>(v);
    case 32: return group_sum<32>(v);
    default: return group_sum<64>(v);
    }
}

// Interleave RoPE of one input chunk (VEC elements = VEC/2 pairs starting at
// pair j0): the even-lane results go to positions j0.., the odd-lane results
// to half_rope + j0.. .
template <typename T, int VEC>
__device__ __forceinline__ void rope_chunk(const float *z, const T *cs, const T *sn, int j0, int half,
                                           bool streaming, float *o1, float *o2) {
    constexpr int H = VEC / 2;
    float c1[H], c2[H], s1[H], s2[H];
    Chunk<T, H> a, b2, c, d;
    if (streaming) {
        a.load_nt(cs + j0); b2.load_nt(cs + half + j0); c.load_nt(sn + j0); d.load_nt(sn + half + j0);
    } else {
        a.load(cs + j0); b2.load(cs + half + j0); c.load(sn + j0); d.load(sn + half + j0);
    }
    a.decode(c1); b2.decode(c2); c.decode(s1); d.decode(s2);
#pragma unroll
    for (int m = 0; m < H; m++) {
        o1[m] = fmaf(z[2 * m], c1[m], -(z[2 * m + 1] * s1[m]));
        o2[m] = fmaf(z[2 * m + 1], c2[m], z[2 * m] * s2[m]);
    }
}

// The occupancy hint (at least 6 waves per SIMD, 4 for the widest rows) keeps register use low enough
// for many rows in flight; the planner's shapes fit without spilling.
template <typename T, int VEC, bool V2, int CR, int CX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CR >= 4 ? 4 : 6, 8))) void kv_rmsnorm_rope_cache_kernel(
    KvParams p) {
    const int G = p.lanes_per_row;
    const int gl = threadIdx.x & (G - 1);
    const uint32_t row = blockIdx.x * (uint32_t)(256 / G) + threadIdx.x / (uint32_t)G;
    const bool row_ok = row < p.rows;

    uint32_t b = 0, n = 0, s = 0;
    if (row_ok) {
        const uint32_t bn = fastdiv(row, p.seq_div);
        s = row - bn * p.seq;
        b = fastdiv(bn, p.heads_div);
        n = bn - b * (uint32_t)p.heads;
    }
    const T *kv = reinterpret_cast<const T *>(p.kv) + b * p.kv_b + n * p.kv_n + s * p.kv_s;

    // ---- loads: rms chunks, then the raw rope tail (V1) or the v row (V2)
    Chunk<T, VEC> x[CR], z[CX];
#pragma unroll
    for (int i = 0; i < CR; i++) {
        const int c = gl + i * G;
        if (row_ok && c < p.nr) x[i].load_nt(kv + c * VEC); else x[i].zero();
    }
    const T *zrow = V2 ? reinterpret_cast<const T *>(p.v) + b * p.v_b + n * p.v_n + s * p.v_s
                       : kv + p.rms_size;
#pragma unroll
    for (int i = 0; i < CX; i++) {
        const int c = gl + i * G;
        if (row_ok && c < p.nx) z[i].load_nt(zrow + c * VEC); else z[i].zero();
    }
    const int64_t slot = row_ok ? p.index[(uint64_t)b * p.seq + s] : -1;

    // ---- (1) RmsNorm statistic over rms_size values, reduced over the group
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < CR; i++) ss = x[i].sumsq(ss);
    ss = row_sum(ss, G);
    const float inv_rms = rsqrtf(ss / (float)p.rms_size + p.eps);
    if (!row_ok) return;

    // ---- destinations
    const bool to_cache = slot >= 0 && slot < p.capacity;
    uint8_t *krow = nullptr, *crow = nullptr;
    if (to_cache) {
        int64_t ko, co;
        if (p.mode == 0) {
            ko = b * p.kc0 + slot * p.kc1 + n * p.kc2;
            co = b * p.cc0 + slot * p.cc1 + n * p.cc2;
        } else {
            const uint32_t blk = fastdiv((uint32_t)slot, p.block_div);     // slot < capacity < 2^31
            const uint32_t off = (uint32_t)slot - blk * (uint32_t)p.block_size;
            ko = blk * p.kc0 + off * p.kc1 + n * p.kc2;
            co = blk * p.cc0 + off * p.cc1 + n * p.cc2;
        }
        const int kbytes = p.k_code == CODE_SAME ? (int)sizeof(T) : 1;
        const int cbytes = p.c_code == CODE_SAME ? (int)sizeof(T) : 1;
        krow = reinterpret_cast<uint8_t *>(p.k_cache) + ko * kbytes;
        crow = reinterpret_cast<uint8_t *>(p.ckv_cache) + co * cbytes;
    }
    const bool out_kv = p.out_kv != 0;
    T *k_rope = out_kv ? reinterpret_cast<T *>(p.k_rope) + b * p.kr_b + n * p.kr_n + s * p.kr_s : nullptr;
    T *c_kv = out_kv ? reinterpret_cast<T *>(p.c_kv) + b * p.ck_b + n * p.ck_n + s * p.ck_s : nullptr;
    const T *gamma = reinterpret_cast<const T *>(p.gamma);
    const T *cs = reinterpret_cast<const T *>(p.cos) + b * p.rope_b + n * p.rope_n + s * p.rope_s;
    const T *sn = reinterpret_cast<const T *>(p.sin) + b * p.rope_b + n * p.rope_n + s * p.rope_s;
    constexpr int H = VEC / 2;
    const bool stream_rope = p.stream_rope != 0;
    const bool k_nt = p.k_rows_whole_lines != 0, c_nt = p.c_rows_whole_lines != 0;

    // ---- normed chunks: y = x * inv_rms * gamma
#pragma unroll
    for (int i = 0; i < CR; i++) {
        const int c = gl + i * G;
        if (c >= p.nr) continue;
        float xv[VEC], g[VEC], y[VEC];
        x[i].decode(xv);
        load_vec<T, VEC>(gamma + c * VEC, g);
#pragma unroll
        for (int e = 0; e < VEC; e++) y[e] = xv[e] * inv_rms * g[e];
        if constexpr (!V2) {
            // V1: the normed row goes to the ckv cache and c_kv
            if (to_cache)
                put_cache<T, VEC>(crow, p.c_code, c * VEC, y, p.v_scale, p.v_offset, p.v_qshape, (int)n, p.c_dim, c_nt);
            if (out_kv) store_vec_nt<T, VEC>(c_kv + c * VEC, y);
        } else {
            if (c < p.n_rope_chunks) {
                // V2: rotate the first rope_size normed values in place
                float o1[H], o2[H];
                const int j0 = c * H;
                rope_chunk<T, VEC>(y, cs, sn, j0, p.half_rope, stream_rope, o1, o2);
                if (to_cache) {
                    put_cache<T, H>(krow, p.k_code, j0, o1, p.k_scale, p.k_offset, p.k_qshape, (int)n, p.k_dim, k_nt);
                    put_cache<T, H>(krow, p.k_code, p.half_rope + j0, o2, p.k_scale, p.k_offset, p.k_qshape,
                                    (int)n, p.k_dim, k_nt);
                }
                if (out_kv) {
                    store_vec_nt<T, H>(k_rope + j0, o1);
                    store_vec_nt<T, H>(k_rope + p.half_rope + j0, o2);
                }
            } else {
                if (to_cache)
                    put_cache<T, VEC>(krow, p.k_code, c * VEC, y, p.k_scale, p.k_offset, p.k_qshape, (int)n, p.k_dim, k_nt);
                if (out_kv) store_vec_nt<T, VEC>(k_rope + c * VEC, y);
            }
        }
    }

    // ---- second part of the row: V1 raw rope tail -> k; V2 v row -> ckv
#pragma unroll
    for (int i = 0; i < CX; i++) {
        const int c = gl + i * G;
        if (c >= p.nx) continue;
        if constexpr (!V2) {
            float zv[VEC], o1[H], o2[H];
            z[i].decode(zv);
            const int j0 = c * H;
            rope_chunk<T, VEC>(zv, cs, sn, j0, p.half_rope, stream_rope, o1, o2);
            if (to_cache) {
                put_cache<T, H>(krow, p.k_code, j0, o1, p.k_scale, p.k_offset, p.k_qshape, (int)n, p.k_dim, k_nt);
                put_cache<T, H>(krow, p.k_code, p.half_rope + j0, o2, p.k_scale, p.k_offset, p.k_qshape, (int)n,
                                p.k_dim, k_nt);
            }
            if (out_kv) {
                store_vec_nt<T, H>(k_rope + j0, o1);
                store_vec_nt<T, H>(k_rope + p.half_rope + j0, o2);
            }
        } else {
            // V2: v_optional goes to the ckv cache (quantised or copied) and to c_kv unchanged
            if (to_cache) {
                if (p.c_code == CODE_SAME) {
                    if (c_nt) {
                        z[i].store_nt(reinterpret_cast<T *>(crow) + c * VEC);
                    } else {
                        Words<Chunk<T, VEC>::kWords> rw;
#pragma unroll
                        for (int q = 0; q < Chunk<T, VEC>::kWords; q++) rw.w[q] = z[i].w[q];
                        store_words<Chunk<T, VEC>::kWords>(reinterpret_cast<T *>(crow) + c * VEC, rw);
                    }
                } else {
                    float zv[VEC];
                    z[i].decode(zv);
                    put_cache<T, VEC>(crow, p.c_code, c * VEC, zv, p.v_scale, p.v_offset, p.v_qshape, (int)n,
                                      p.c_dim, c_nt);
                }
            }
            if (out_kv) z[i].store_nt(c_kv + c * VEC);
        }
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------

static int round_slots(int c, const int *allowed, int n_allowed) {
    for (int i = 0; i < n_allowed; i++)
        if (c <= allowed[i]) return allowed[i];
    return -1;
}

static const int kCR[] = {1, 2, 3, 4};
static const int kCX[] = {1, 2};

// Lane-group size: the smallest G whose register slots hold the row (fewest
// lanes per row, most rows per wave), unless that leaves fewer than 2048
// wavefronts (two per SIMD on 256 CUs); then larger groups spread few rows
// over more waves (a decode batch of 512 rows runs on 512 waves at G = 64).
int kv_plan(KvParams &p, int vec, bool v2, int &cr, int &cx) {
    p.nr = p.rms_size / vec;
    p.nx = (v2 ? p.c_dim : p.rope_size) / vec;
    p.n_rope_chunks = v2 ? p.rope_size / vec : 0;
    int found = -1;
    for (int G = 8; G <= 64; G *= 2) {
        int r = round_slots((p.nr + G - 1) / G, kCR, 4);
        int x = round_slots((p.nx + G - 1) / G, kCX, 2);
        if (r > 0 && x > 0) {
            p.lanes_per_row = G;
            cr = r;
            cx = x;
            found = 0;
            if ((uint64_t)p.rows * (uint64_t)G >= 2048ull * 64ull) return 0;
        }
    }
    return found;
}

template <typename T, int VEC, bool V2>
static hipError_t launch_t(const KvParams &p, int cr, int cx, hipStream_t stream) {
    const uint32_t rows_per_block = 256 / p.lanes_per_row;
    const uint32_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
    dim3 grid((unsigned)blocks), block(256);
#define QKNR_KV(CRV, CXV)                                                                              \
    if (cr == CRV && cx == CXV) {                                                                      \
        hipLaunchKernelGGL((kv_rmsnorm_rope_cache_kernel<T, VEC, V2, CRV, CXV>), grid, block, 0, stream, p); \
        return hipGetLastError();                                                                      \
    }
    QKNR_KV(1, 1) QKNR_KV(2, 1) QKNR_KV(3, 1) QKNR_KV(4, 1)
    QKNR_KV(1, 2) QKNR_KV(2, 2) QKNR_KV(3, 2) QKNR_KV(4, 2)
#undef QKNR_KV
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_elem(const KvParams &p, int vec, bool v2, int cr, int cx, hipStream_t stream) {
    if (vec == 8) return v2 ? launch_t<T, 8, true>(p, cr, cx, stream) : launch_t<T, 8, false>(p, cr, cx, stream);
    return v2 ? launch_t<T, 4, true>(p, cr, cx, stream) : launch_t<T, 4, false>(p, cr, cx, stream);
}

hipError_t kv_launch(KvParams &p, int elem_type, int vec, bool v2, hipStream_t stream) {
    int cr = 0, cx = 0;
    if (kv_plan(p, vec, v2, cr, cx) != 0) return hipErrorInvalidValue;
    if (p.rows == 0) return hipSuccess;
    if (elem_type == 1) return launch_elem<bf16_t>(p, vec, v2, cr, cx, stream);
    if (elem_type == 2) return launch_elem<f16_t>(p, vec, v2, cr, cx, stream);
    return hipErrorInvalidValue;
}

}  // namespace qknr
