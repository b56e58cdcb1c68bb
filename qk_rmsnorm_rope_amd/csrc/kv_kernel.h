// kv_kernel.h -- the KvRmsNormRopeCache kernel for gfx950 (device code and
// its launch templates), included by the two translation units that
// instantiate it: kv_rmsnorm_rope_cache.hip (bf16, planner, entry) and
// kv_rmsnorm_rope_cache_f16.hip (f16).
//
// Computes, per (b, n, s) row, the CANN page's formulas: (1) RmsNorm over the
// first rms_size values, (2) interleaveRope (V1: on the raw tail; V2: on the
// first rope_size normed values, which it replaces), (3) static quantisation
// per cache (int8, FP8 E4M3FN or E5M2), (4) scatter of the k and ckv rows to
// the slot of token (b, s) in a Norm or paged cache (PA_BNSD: one index entry
// per token; PA_BLK_BNSD: one starting slot per run of block_size tokens),
// (5) optional raw outputs k_rope / c_kv.
//
// MI355X design: the operator is HBM-bound, so each row is read once and every
// output row is written once, in one pass:
//   * each row splits into two independent parts with their own waves (blocks
//     are typed): part A is the normed part (V1: RmsNorm of kv[:Dv] -> ckv
//     cache and c_kv; V2: RmsNorm of kv, RoPE on its head -> k cache and
//     k_rope), part B the other (V1: RoPE of the raw kv[Dv:] -> k cache and
//     k_rope; V2: v_optional -> ckv cache and c_kv). Splitting halves the
//     registers a wave holds and leaves part B without any reduction;
//   * in each part a group of G lanes (8..64, a power of two) owns one row; 64/G
//     rows per wavefront, 256/G per block. Lane l of a group owns the 8-element
//     chunks l, l+G, l+2G, ... of its part (16-byte loads of bf16/f16);
//   * the sum of squares reduces inside the group with DPP / ds_swizzle (no
//     LDS, no barrier); the result is bit-identical in every lane of the group;
//   * an interleaved input chunk (pairs 2j, 2j+1) produces half a chunk of the
//     even-lane outputs (positions j) and half a chunk of the odd-lane outputs
//     (positions j + R/2), so the rotation needs no data exchange between
//     lanes: each lane writes two half-chunks;
//   * quantisation (int8 RNE + clamp, or FP8 E4M3FN / E5M2 RNE saturating) is fused
//     into the stores; there are no atomics and each output byte has one writer;
//     each part is specialised (one dispatch per block) on the encoding of the
//     cache it writes;
//   * when a wave holds several rows, quantised caches use two per-wave LDS
//     regions: the wave's per-head (or per-channel) scale/offset rows, loaded
//     once per wave instead of per lane and chunk, and the wave's rows of
//     codes, written out in 16-byte pieces so that whole lines leave in one
//     request (WaveParams, WaveCodes below);
//   * an index of -1 (or, defensively, outside the cache) writes no cache row;
//   * data read once (kv, v, per-row cos/sin) moves with non-temporal loads;
//     k_rope / c_kv (contiguous) with non-temporal stores; cache rows (at
//     random slots) with ordinary stores, which measured faster for every
//     row width here: rows that cover lines only in part (the 192-byte int8
//     rows) merge with their neighbours in L2 before they reach HBM; gamma,
//     reused by every row, stays cached;
//   * row -> (b, n, s) and slot -> (block, offset) use multiply-high division
//     by the invariant sizes instead of 64-bit divides; kernel fields are read
//     from the kernel-argument segment where they are used;
//   * gamma and the cos/sin of rotated chunks are requested together with the
//     row data, so their latency overlaps the HBM latency.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace qknr {

// Per-wave LDS regions (launch-time size: 4 waves x lds_wave_bytes): staged
// quantisation parameters, then staged codes (WaveParams, WaveCodes). Every
// access to them goes through LDS-typed pointers (kv_lds_at).
extern __shared__ float4 kv_lds[];

__device__ __forceinline__ lds_u8 *kv_lds_at(uint32_t byte_off) {
    return (lds_u8 *)kv_lds + byte_off;
}

// N codes (byte 0 of each word) packed into N/4 words.
template <int W>
__device__ __forceinline__ Words<W> pack_codes(const uint32_t *code) {
    Words<W> r;
#pragma unroll
    for (int i = 0; i < W; i++) r.w[i] = pack_bytes4(code[4 * i], code[4 * i + 1], code[4 * i + 2], code[4 * i + 3]);
    return r;
}

// Store N codes at p in global memory (naturally aligned).
template <int N>
__device__ __forceinline__ void store_codes(void *p, const uint32_t *code) {
    if constexpr (N >= 4) {
        store_words<N / 4>(p, pack_codes<N / 4>(code));
    } else {
        static_assert(N == 2, "2, 4 or 8 codes");
        *reinterpret_cast<uint16_t *>(p) = (uint16_t)pack_bytes2(code[0], code[1]);
    }
}

// Store N codes into the wave's LDS staging at byte offset `off` of kv_lds.
template <int N>
__device__ __forceinline__ void stage_codes(uint32_t off, const uint32_t *code) {
    if constexpr (N >= 4) {
        lds_store_words<N / 4>(kv_lds_at(off), pack_codes<N / 4>(code));
    } else {
        static_assert(N == 2, "2, 4 or 8 codes");
        *reinterpret_cast<lds_u16 *>(kv_lds_at(off)) = (uint16_t)pack_bytes2(code[0], code[1]);
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
    const float *q = p + (shape == QS_HEAD_CHANNEL ? n * width : 0) + c;
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; i++) {
            float4 v = reinterpret_cast<const float4 *>(q)[i];
            out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
        }
    } else {
        static_assert(N % 2 == 0, "even parameter counts");
#pragma unroll
        for (int i = 0; i < N / 2; i++) {
            float2 v = reinterpret_cast<const float2 *>(q)[i];
            out[2 * i] = v.x; out[2 * i + 1] = v.y;
        }
    }
}

// One destination row (a cache row and its quantisation parameters); the
// encoding is a template parameter of the code that writes it.
struct CacheRow {
    uint8_t *row;            // nullptr: no cache write for this token
    int32_t stage;           // >= 0: quantised codes go to kv_lds at this byte offset (the wave's copy of the row)
    int64_t off;             // byte offset of row in its cache (-1: none)
    const float *scale, *offset;
    int qshape, n, width;
};

// The scale and offset of N consecutive channels from c. An absent offset is
// -0, so that fmaf(x, scale, offset) is exactly x*scale, signed zeros included.
template <int N>
struct QuantParams {
    float sc[N], of[N];
    // from a wave's staged copy [scale[width] | offset[width]] at byte offset
    // wp of kv_lds (see WaveParams); c and width are multiples of 4 for N >= 4,
    // of 2 for N == 2
    __device__ __forceinline__ void load_lds(uint32_t wp, int width, int c) {
        const lds_u8 *s = kv_lds_at(wp + 4u * (uint32_t)c);
        const lds_u8 *o = kv_lds_at(wp + 4u * (uint32_t)(width + c));
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int i = 0; i < N; i += 4) {
                const Words<4> a = lds_load_words<4>(s + 4 * i), b = lds_load_words<4>(o + 4 * i);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    sc[i + e] = __uint_as_float(a.w[e]);
                    of[i + e] = __uint_as_float(b.w[e]);
                }
            }
        } else {
            static_assert(N == 2, "2, 4 or 8 parameters");
            const Words<2> a = lds_load_words<2>(s), b = lds_load_words<2>(o);
            sc[0] = __uint_as_float(a.w[0]); sc[1] = __uint_as_float(a.w[1]);
            of[0] = __uint_as_float(b.w[0]); of[1] = __uint_as_float(b.w[1]);
        }
    }
    __device__ __forceinline__ void load(const float *scale, const float *offset, int qshape, int n, int width,
                                         int c) {
        load_qparam<N>(scale, qshape, n, width, c, sc);
        if (offset) {
            load_qparam<N>(offset, qshape, n, width, c, of);
        } else {
#pragma unroll
            for (int i = 0; i < N; i++) of[i] = -0.0f;   // fmaf(x, s, -0) == x*s, signed zeros included
        }
    }
};

template <int CODE>
__device__ __forceinline__ uint32_t encode(float t) {
    if constexpr (CODE == CODE_INT8) return enc_int8(t);
    else if constexpr (CODE == CODE_E4M3FN) return enc_e4m3fn(t);
    else return enc_e5m2(t);
}

// Write N quantised values starting at channel c (t = x*scale (+offset) in
// fp32 with one rounding), parameters already loaded.
template <int CODE, int N>
__device__ __forceinline__ void put_codes(const CacheRow &d, int c, const float *x, const QuantParams<N> &qp) {
    uint32_t q[N];
#pragma unroll
    for (int i = 0; i < N; i++) q[i] = encode<CODE>(fmaf(x[i], qp.sc[i], qp.of[i]));
    if (d.stage >= 0) stage_codes<N>((uint32_t)(d.stage + c), q);
    else store_codes<N>(d.row + c, q);
}

// Write N values starting at channel c: quantised, or rounded to T.
template <typename T, int CODE, int N>
__device__ __forceinline__ void put_cache(const CacheRow &d, int c, const float *x) {
    if constexpr (CODE == CODE_SAME) {
        store_vec<T, N>(reinterpret_cast<T *>(d.row) + c, x);
    } else {
        QuantParams<N> qp;
        qp.load(d.scale, d.offset, d.qshape, d.n, d.width, c);
        put_codes<CODE, N>(d, c, x, qp);
    }
}

__device__ __forceinline__ float row_sum(float v, int G) {
    switch (G) {
    case 8: return group_sum<8>(v);
    case 16: return group_sum<16>(v);
    case 32: return group_sum<32>(v);
    default: return group_sum<64>(v);
    }
}

// cos/sin of one interleaved input chunk (VEC elements = H = VEC/2 pairs
// starting at pair j0): the even-lane results go to positions j0.., the
// odd-lane results to half + j0.. .
template <typename T, int H>
struct RopeCoef {
    Chunk<T, H> c1, c2, s1, s2;
    __device__ __forceinline__ void load(const T *cs, const T *sn, int j0, int half, bool streaming) {
        if (streaming) {
            c1.load_nt(cs + j0); c2.load_nt(cs + half + j0); s1.load_nt(sn + j0); s2.load_nt(sn + half + j0);
        } else {
            c1.load(cs + j0); c2.load(cs + half + j0); s1.load(sn + j0); s2.load(sn + half + j0);
        }
    }
    // o1[m] = z[2m] cos[j0+m] - z[2m+1] sin[j0+m]; o2[m] = z[2m+1] cos[h+j0+m] + z[2m] sin[h+j0+m]
    __device__ __forceinline__ void apply(const float *z, float *o1, float *o2) const {
        float a[H], b[H], c[H], d[H];
        c1.decode(a); c2.decode(b); s1.decode(c); s2.decode(d);
#pragma unroll
        for (int m = 0; m < H; m++) {
            o1[m] = fmaf(z[2 * m], a[m], -(z[2 * m + 1] * c[m]));
            o2[m] = fmaf(z[2 * m + 1], b[m], z[2 * m] * d[m]);
        }
    }
};

struct RowPos {
    uint32_t b, n, s;
    bool ok;
};

// Position of row index `row`; ok is false past the last row.
__device__ __forceinline__ RowPos row_pos(const KvParams &p, uint32_t row) {
    RowPos r{0, 0, 0, row < p.rows};
    if (r.ok) {
        const uint32_t bn = fastdiv(row, p.seq_div);
        r.s = row - bn * p.seq;
        r.b = fastdiv(bn, p.heads_div);
        r.n = bn - r.b * (uint32_t)p.heads;
    }
    return r;
}

// Row `blk * 256/G + tid/G` of the part whose lane groups are G = 2^shift wide.
__device__ __forceinline__ RowPos row_pos(const KvParams &p, uint32_t blk, int shift) {
    const uint32_t row = (blk << (8 - shift)) + (threadIdx.x >> shift);
    RowPos r{0, 0, 0, row < p.rows};
    if (r.ok) {
        const uint32_t bn = fastdiv(row, p.seq_div);
        r.s = row - bn * p.seq;
        r.b = fastdiv(bn, p.heads_div);
        r.n = bn - r.b * (uint32_t)p.heads;
    }
    return r;
}

// Per-channel quantisation parameters shared by every row of a wavefront,
// staged once per wave in its own LDS region as [scale[width] | offset[width]]
// (offset -0 if absent): one 16-byte load per lane instead of the parameters
// of every chunk of every row through the vector cache, where they would
// compete with the row data. Used when a wave holds several rows (G < 64),
// the parameters are per channel or per head and channel, 8*width <=
// lds_param_bytes (<= 2 KB), and every row of the wave has the same head
// (checked from its first and last row). Only the
// wave writes and reads its region, and LDS accesses of one wave complete in
// order, so no barrier is needed. (At most kWaveParamFloats per wave.)
struct WaveParams {
    float4 v[2];      // staged 16-byte pieces of this lane (lane, lane + 64)
    uint32_t wp;      // byte offset of the wave's region in kv_lds
    bool on;

    // The head of the wave's rows, the decision, and the loads (issued first,
    // so that the data loads behind them do not wait for them).
    __device__ __forceinline__ void load(const KvParams &p, uint32_t blk, int shift, const float *scale,
                                         const float *offset, int qshape, int width, int rsteps = 1) {
        const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        wp = wave * (uint32_t)p.lds_wave_bytes;
        // the wave's rows: (64 / G) consecutive rows in each of rsteps steps 256 / G apart
        const uint32_t first = blk * ((uint32_t)rsteps << (8 - shift)) + (wave << (6 - shift));
        // (a wave of one row, G = 64, reads each parameter once anyway)
        on = shift < 6 && qshape != QS_SCALAR && 8 * width <= p.lds_param_bytes && first < p.rows;
        if (!on) return;
        const uint32_t last = min(first + ((uint32_t)(rsteps - 1) << (8 - shift)) + (64u >> shift) - 1u, p.rows - 1u);
        const uint32_t bn = fastdiv(first, p.seq_div);
        if (p.heads > 1 && qshape == QS_HEAD_CHANNEL && fastdiv(last, p.seq_div) != bn) {
            on = false;
            return;
        }
        const uint32_t n = bn - fastdiv(bn, p.heads_div) * (uint32_t)p.heads;
        const uint64_t base = qshape == QS_HEAD_CHANNEL ? (uint64_t)n * (uint32_t)width : 0;
        const int q4 = width >> 2;
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int q = lane + 64 * j;
            if (q < q4) v[j] = reinterpret_cast<const float4 *>(scale + base)[q];
            else if (q < 2 * q4) v[j] = offset ? reinterpret_cast<const float4 *>(offset + base)[q - q4]
                                               : make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
        }
    }
    __device__ __forceinline__ void store(int width) const {
        if (!on) return;
        const int q4 = width >> 2;
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int q = lane + 64 * j;
            if (q < 2 * q4) {
                Words<4> w;
                w.w[0] = __float_as_uint(v[j].x); w.w[1] = __float_as_uint(v[j].y);
                w.w[2] = __float_as_uint(v[j].z); w.w[3] = __float_as_uint(v[j].w);
                lds_store_words<4>(kv_lds_at(wp + 16u * (uint32_t)q), w);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
};

// Quantised codes of the wave's rows staged in LDS (after the parameters,
// rows of `width` bytes packed back to back) and written out in 16-byte
// pieces: lane q takes pieces q and q + 64, so the 8..64 lanes of a row store
// it contiguously, and whole 128-byte lines leave in one request instead of
// the 4- and 8-byte pieces of the lanes' own chunks. The destination row of a
// piece comes from the lane that computed the row (ds_bpermute), so every
// lane of the wave takes part in the flush. Used when a wave holds several
// rows, the row width is a multiple of 16 bytes and the planner allowed it for
// the part (a cache whose base and strides are 16-byte multiples).
struct WaveCodes {
    uint32_t buf;     // byte offset of the wave's staged rows in kv_lds
    int width;        // bytes per row
    bool on;

    __device__ __forceinline__ void init(const KvParams &p, bool allowed, int shift, int width_bytes,
                                         int rsteps = 1) {
        const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        buf = wave * (uint32_t)p.lds_wave_bytes + (uint32_t)p.lds_param_bytes;
        width = width_bytes;
        on = allowed && shift < 6 && (width_bytes & 15) == 0 && rsteps * (64 >> shift) * width_bytes <= p.lds_code_bytes &&
             rsteps * (64 >> shift) * (width_bytes >> 4) <= 128;   // flush() moves at most two pieces per lane
    }
    // byte offset in kv_lds of this lane's row of step k in the staging buffer
    __device__ __forceinline__ int32_t row_buf(int shift, int k = 0) const {
        return (int32_t)(buf + (uint32_t)(k * (64 >> shift) + ((threadIdx.x & 63) >> shift)) * (uint32_t)width);
    }
    // cache: the cache's base; off[k]: this lane's row offset in it for step k
    // (-1: none). Executed by every lane.
    template <int R>
    __device__ __forceinline__ void flush(int shift, uint8_t *cache, const int64_t *off) const {
        __builtin_amdgcn_wave_barrier();
        const int ppr = width >> 4;                    // pieces per row
        const int rpw = 64 >> shift;                   // rows per wave and step
        const int pieces = R * rpw * ppr;              // <= 128
        const float inv_ppr = 1.0f / (float)ppr;
        const int lane = threadIdx.x & 63;
        const lds_u8 *staged = kv_lds_at(buf);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int q = lane + 64 * j;
            // q / ppr for q < 128: (q + 0.5) / ppr is at least 0.5 / ppr from an integer
            const int rs = q < pieces ? (int)(((float)q + 0.5f) * inv_ppr) : 0;
            const int kstep = rs / rpw, rw = rs - kstep * rpw;
            const int src = (rw << shift) << 2;
            int64_t o = -1;
#pragma unroll
            for (int k = 0; k < R; k++) {
                const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(uint64_t)off[k]);
                const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)((uint64_t)off[k] >> 32));
                if (k == kstep) o = (int64_t)(((uint64_t)hi << 32) | lo);
            }
            if (q < pieces && o >= 0) {
                const Words<4> v = lds_load_words<4>(staged + q * 16);
                store_words<4>(cache + o + (q - rs * ppr) * 16, v);
            }
        }
    }
};

// Element offset b*sb + n*sn + s*ss (32-bit strides, 64-bit sum).
__device__ __forceinline__ uint64_t row_off(const RowPos &r, uint32_t sb, uint32_t sn, uint32_t ss) {
    return (uint64_t)r.b * sb + (uint64_t)r.n * sn + (uint64_t)r.s * ss;
}

// The cache slot of token (b, s), or -1. Norm and PA_BNSD: index[b*S + s].
// PA_BLK_BNSD: the run s / block_size of batch b starts at index[b*runs + run]
// and the token takes the slot s % block_size places after that start.
__device__ __forceinline__ int64_t token_slot(const KvParams &p, const RowPos &r) {
    if (!r.ok) return -1;
    if (p.mode != 2) return p.index[(uint64_t)r.b * p.seq + r.s];
    const uint32_t run = fastdiv(r.s, p.block_div);
    const int64_t start = p.index[(uint64_t)r.b * p.runs + run];
    return start < 0 ? -1 : start + (int64_t)(r.s - run * (uint32_t)p.block_size);
}

// The cache row of token (b, s), head n, for the k cache (is_k) or the ckv
// cache; `eb` is the cache's element size in bytes.
__device__ __forceinline__ CacheRow cache_row(const KvParams &p, bool is_k, int eb, int64_t slot, const RowPos &r) {
    CacheRow d;
    d.scale = is_k ? p.k_scale : p.v_scale;
    d.offset = is_k ? p.k_offset : p.v_offset;
    d.qshape = is_k ? p.k_qshape : p.v_qshape;
    d.n = (int)r.n;
    d.width = is_k ? p.k_dim : p.c_dim;
    d.row = nullptr;
    d.stage = -1;
    d.off = -1;
    if (slot >= 0 && slot < p.capacity) {
        const uint32_t s0 = is_k ? p.kc0 : p.cc0, s1 = is_k ? p.kc1 : p.cc1, s2 = is_k ? p.kc2 : p.cc2;
        uint64_t off;
        if (p.mode == 0) {
            off = (uint64_t)r.b * s0 + (uint64_t)(uint32_t)slot * s1 + (uint64_t)r.n * s2;
        } else {
            const uint32_t blk = fastdiv((uint32_t)slot, p.block_div);     // slot < capacity < 2^31
            const uint32_t in_blk = (uint32_t)slot - blk * (uint32_t)p.block_size;
            off = (uint64_t)blk * s0 + (uint64_t)in_blk * s1 + (uint64_t)r.n * s2;
        }
        d.off = (int64_t)(off * (uint32_t)eb);
        d.row = reinterpret_cast<uint8_t *>(is_k ? p.k_cache : p.ckv_cache) + d.off;
    }
    return d;
}

// Part A: the normed part of a row. V1: y = RmsNorm(kv[:Dv]) -> ckv cache,
// c_kv. V2: y = RmsNorm(kv); the first rope_size values rotated -> k cache,
// k_rope (the planner keeps every rotated chunk in slot 0). CODE: the
// encoding of that cache. Each lane takes R rows, 256/G apart, whose loads
// are all issued before any is used; gamma serves all of them.
template <typename T, int VEC, bool V2, int CA, int CODE, int R>
__device__ __forceinline__ void part_a(const KvParams &p, uint32_t blk) {
    constexpr int H = VEC / 2;
    constexpr bool kQuant = CODE != CODE_SAME;
    const int shift = p.ga_shift;
    const int G = 1 << shift;
    const int gl = threadIdx.x & (G - 1);
    const uint32_t row0 = blk * ((uint32_t)R << (8 - shift)) + (threadIdx.x >> shift);
    const T *gamma = reinterpret_cast<const T *>(p.gamma);

    // Quantisation parameters of the cache this part writes (V1: ckv, V2: k):
    // staged per wave in LDS where possible; else V1's ([1] or [Dc], the same
    // for every row) are requested with the data when they fit in registers
    // and V2's are loaded at the store.
    const int qwidth = V2 ? p.k_dim : p.c_dim;
    WaveParams wpar;
    wpar.on = false;
    if constexpr (kQuant)
        wpar.load(p, blk, shift, V2 ? p.k_scale : p.v_scale, V2 ? p.k_offset : p.v_offset,
                  V2 ? p.k_qshape : p.v_qshape, qwidth, R);
    constexpr bool kPreT = !V2 && kQuant && CA == 1 && R == 1;
    const bool kPre = kPreT && !wpar.on;
    RowPos r[R];
    Chunk<T, VEC> x[R][CA], gm[CA];
    RopeCoef<T, H> rc[V2 ? R : 1];
    QuantParams<VEC> qp[kPreT ? CA : 1];
#pragma unroll
    for (int k = 0; k < R; k++) {
        r[k] = row_pos(p, row0 + ((uint32_t)k << (8 - shift)));
        const T *kv = reinterpret_cast<const T *>(p.kv) + row_off(r[k], p.kv_b, p.kv_n, p.kv_s);
#pragma unroll
        for (int i = 0; i < CA; i++) {
            const int c = gl + i * G;
            if (r[k].ok && c < p.nr) {
                x[k][i].load_nt(kv + c * VEC);
                if (k == 0) gm[i].load(gamma + c * VEC);
                if constexpr (kPreT)
                    if (k == 0 && kPre) qp[i].load(p.v_scale, p.v_offset, p.v_qshape, (int)r[k].n, p.c_dim, c * VEC);
            } else {
                x[k][i].zero();
            }
        }
        if constexpr (V2) {
            if (r[k].ok && gl < p.n_rope_chunks) {
                const uint64_t ro = row_off(r[k], p.rope_b, p.rope_n, p.rope_s);
                rc[k].load(reinterpret_cast<const T *>(p.cos) + ro, reinterpret_cast<const T *>(p.sin) + ro, gl * H,
                           p.half_rope, p.stream_rope != 0);
            }
        }
    }
    int64_t slot[R];
#pragma unroll
    for (int k = 0; k < R; k++) slot[k] = token_slot(p, r[k]);
    if constexpr (kQuant) wpar.store(qwidth);

    // (1) RmsNorm statistic over rms_size values, reduced over the group
    float inv_rms[R];
#pragma unroll
    for (int k = 0; k < R; k++) {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < CA; i++) ss = x[k][i].sumsq(ss);
        ss = row_sum(ss, G);
        inv_rms[k] = rsqrtf(ss / (float)p.rms_size + p.eps);
    }

    WaveCodes wc;
    wc.on = false;
    if constexpr (kQuant) wc.init(p, p.stage_a != 0, shift, qwidth, R);
    const bool out_kv = p.out_kv != 0;
    int64_t offs[R];
#pragma unroll
    for (int k = 0; k < R; k++) {
        CacheRow d = cache_row(p, V2, kQuant ? 1 : (int)sizeof(T), slot[k], r[k]);
        offs[k] = d.off;
        if (kQuant && wc.on) d.stage = wc.row_buf(shift, k);
        T *raw = nullptr;   // c_kv (V1) or k_rope (V2)
        if (out_kv && r[k].ok)
            raw = V2 ? reinterpret_cast<T *>(p.k_rope) + row_off(r[k], p.kr_b, p.kr_n, p.kr_s)
                     : reinterpret_cast<T *>(p.c_kv) + row_off(r[k], p.ck_b, p.ck_n, p.ck_s);
#pragma unroll
        for (int i = 0; i < CA; i++) {
            const int c = gl + i * G;
            if (!r[k].ok || c >= p.nr) continue;
            float xv[VEC], g[VEC], y[VEC];
            x[k][i].decode(xv);
            gm[i].decode(g);
#pragma unroll
            for (int e = 0; e < VEC; e++) y[e] = xv[e] * inv_rms[k] * g[e];
            if (V2 && i == 0 && c < p.n_rope_chunks) {
                // (2) interleaveRope on the normed head: rope_out replaces y there
                float o1[H], o2[H];
                const int j0 = c * H;
                rc[V2 ? k : 0].apply(y, o1, o2);
                if (d.row) {
                    if (kQuant && wpar.on) {
                        QuantParams<H> q1, q2;
                        q1.load_lds(wpar.wp, qwidth, j0);
                        q2.load_lds(wpar.wp, qwidth, p.half_rope + j0);
                        put_codes<CODE, H>(d, j0, o1, q1);
                        put_codes<CODE, H>(d, p.half_rope + j0, o2, q2);
                    } else {
                        put_cache<T, CODE, H>(d, j0, o1);
                        put_cache<T, CODE, H>(d, p.half_rope + j0, o2);
                    }
                }
                if (out_kv) {
                    store_vec_nt<T, H>(raw + j0, o1);
                    store_vec_nt<T, H>(raw + p.half_rope + j0, o2);
                }
            } else {
                if (d.row) {
                    if (kQuant && wpar.on) {
                        QuantParams<VEC> ql;
                        ql.load_lds(wpar.wp, qwidth, c * VEC);
                        put_codes<CODE, VEC>(d, c * VEC, y, ql);
                    } else if (kPre) {
                        put_codes<CODE, VEC>(d, c * VEC, y, qp[i]);
                    } else {
                        put_cache<T, CODE, VEC>(d, c * VEC, y);
                    }
                }
                if (out_kv) store_vec_nt<T, VEC>(raw + c * VEC, y);
            }
        }
    }
    if constexpr (kQuant)
        if (wc.on) wc.flush<R>(shift, reinterpret_cast<uint8_t *>(V2 ? p.k_cache : p.ckv_cache), offs);
}

// Part B: V1: interleaveRope of the raw kv[Dv:] -> k cache, k_rope.
//         V2: v_optional -> ckv cache (quantised or copied), c_kv (copied).
// CODE: the encoding of that cache. Each lane takes R rows, 256/G apart, whose
// loads are all issued before any is used.
template <typename T, int VEC, bool V2, int CB, int CODE, int R>
__device__ __forceinline__ void part_b(const KvParams &p, uint32_t blk) {
    constexpr int H = VEC / 2;
    constexpr bool kQuant = CODE != CODE_SAME;
    constexpr bool kQuantV = V2 && kQuant;              // V2 quantised ckv
    constexpr bool kPreKT = !V2 && kQuant && CB == 1 && R == 1;
    const int shift = p.gb_shift;
    const int G = 1 << shift;
    const int gl = threadIdx.x & (G - 1);
    const uint32_t row0 = blk * ((uint32_t)R << (8 - shift)) + (threadIdx.x >> shift);

    // Quantisation parameters of the cache this part writes (V1: k, V2: ckv):
    // staged per wave in LDS where possible; else requested with the data
    // (one row per lane) or loaded at the store.
    const int qwidth = V2 ? p.c_dim : p.k_dim;
    WaveParams wpar;
    wpar.on = false;
    if constexpr (kQuant)
        wpar.load(p, blk, shift, V2 ? p.v_scale : p.k_scale, V2 ? p.v_offset : p.k_offset,
                  V2 ? p.v_qshape : p.k_qshape, qwidth, R);
    const bool kPreV = kQuantV && R == 1 && !wpar.on;
    const bool kPreK = kPreKT && !wpar.on;

    RowPos r[R];
    Chunk<T, VEC> z[R][CB];
    RopeCoef<T, H> rc[V2 ? 1 : R][V2 ? 1 : CB];
    QuantParams<VEC> qp[(kQuantV && R == 1) ? CB : 1];
    QuantParams<H> qk1[kPreKT ? CB : 1], qk2[kPreKT ? CB : 1];
#pragma unroll
    for (int k = 0; k < R; k++) {
        r[k] = row_pos(p, row0 + ((uint32_t)k << (8 - shift)));
        const T *src = V2 ? reinterpret_cast<const T *>(p.v) + row_off(r[k], p.v_b, p.v_n, p.v_s)
                          : reinterpret_cast<const T *>(p.kv) + row_off(r[k], p.kv_b, p.kv_n, p.kv_s) + p.rms_size;
        const uint64_t ro = row_off(r[k], p.rope_b, p.rope_n, p.rope_s);
        const T *cs = reinterpret_cast<const T *>(p.cos) + ro;
        const T *sn = reinterpret_cast<const T *>(p.sin) + ro;
#pragma unroll
        for (int i = 0; i < CB; i++) {
            const int c = gl + i * G;
            if (r[k].ok && c < p.nx) {
                z[k][i].load_nt(src + c * VEC);
                if constexpr (!V2) rc[k][i].load(cs, sn, c * H, p.half_rope, p.stream_rope != 0);
                if constexpr (kQuantV && R == 1)
                    if (kPreV) qp[i].load(p.v_scale, p.v_offset, p.v_qshape, (int)r[k].n, p.c_dim, c * VEC);
                if constexpr (kPreKT) {
                    if (kPreK) {
                        qk1[i].load(p.k_scale, p.k_offset, p.k_qshape, (int)r[k].n, p.k_dim, c * H);
                        qk2[i].load(p.k_scale, p.k_offset, p.k_qshape, (int)r[k].n, p.k_dim, p.half_rope + c * H);
                    }
                }
            } else {
                z[k][i].zero();
            }
        }
    }
    int64_t slot[R];
#pragma unroll
    for (int k = 0; k < R; k++) slot[k] = token_slot(p, r[k]);
    if constexpr (kQuant) wpar.store(qwidth);

    WaveCodes wc;
    wc.on = false;
    if constexpr (kQuant) wc.init(p, p.stage_b != 0, shift, qwidth, R);
    const bool out_kv = p.out_kv != 0;
    int64_t offs[R];
#pragma unroll
    for (int k = 0; k < R; k++) {
        CacheRow d = cache_row(p, !V2, CODE == CODE_SAME ? (int)sizeof(T) : 1, slot[k], r[k]);
        offs[k] = d.off;
        if (kQuant && wc.on) d.stage = wc.row_buf(shift, k);
        T *raw = nullptr;   // k_rope (V1) or c_kv (V2)
        if (out_kv && r[k].ok)
            raw = V2 ? reinterpret_cast<T *>(p.c_kv) + row_off(r[k], p.ck_b, p.ck_n, p.ck_s)
                     : reinterpret_cast<T *>(p.k_rope) + row_off(r[k], p.kr_b, p.kr_n, p.kr_s);
#pragma unroll
        for (int i = 0; i < CB; i++) {
            const int c = gl + i * G;
            if (!r[k].ok || c >= p.nx) continue;
            if constexpr (!V2) {
                float zv[VEC], o1[H], o2[H];
                z[k][i].decode(zv);
                const int j0 = c * H;
                rc[k][i].apply(zv, o1, o2);
                if (d.row) {
                    if (kQuant && wpar.on) {
                        QuantParams<H> q1, q2;
                        q1.load_lds(wpar.wp, qwidth, j0);
                        q2.load_lds(wpar.wp, qwidth, p.half_rope + j0);
                        put_codes<CODE, H>(d, j0, o1, q1);
                        put_codes<CODE, H>(d, p.half_rope + j0, o2, q2);
                    } else if (kPreK) {
                        put_codes<CODE, H>(d, j0, o1, qk1[i]);
                        put_codes<CODE, H>(d, p.half_rope + j0, o2, qk2[i]);
                    } else {
                        put_cache<T, CODE, H>(d, j0, o1);
                        put_cache<T, CODE, H>(d, p.half_rope + j0, o2);
                    }
                }
                if (out_kv) {
                    store_vec_nt<T, H>(raw + j0, o1);
                    store_vec_nt<T, H>(raw + p.half_rope + j0, o2);
                }
            } else {
                if (d.row) {
                    if constexpr (CODE == CODE_SAME) {
                        T *dst = reinterpret_cast<T *>(d.row) + c * VEC;
                        Words<Chunk<T, VEC>::kWords> rw;
#pragma unroll
                        for (int q = 0; q < Chunk<T, VEC>::kWords; q++) rw.w[q] = z[k][i].w[q];
                        store_words<Chunk<T, VEC>::kWords>(dst, rw);
                    } else {
                        float zv[VEC];
                        z[k][i].decode(zv);
                        if (wpar.on) {
                            QuantParams<VEC> ql;
                            ql.load_lds(wpar.wp, qwidth, c * VEC);
                            put_codes<CODE, VEC>(d, c * VEC, zv, ql);
                        } else if (kPreV) {
                            put_codes<CODE, VEC>(d, c * VEC, zv, qp[i]);
                        } else {
                            put_cache<T, CODE, VEC>(d, c * VEC, zv);
                        }
                    }
                }
                if (out_kv) z[k][i].store_nt(raw + c * VEC);
            }
        }
    }
    if constexpr (kQuant)
        if (wc.on) wc.flush<R>(shift, reinterpret_cast<uint8_t *>(V2 ? p.ckv_cache : p.k_cache), offs);
}

// V2: blocks [0, blocks_a) run part A, the rest part B; V1 the other way
// round. Each part dispatches once
// on the encoding of the cache it writes, so the per-chunk code is
// specialised. RA, RB: rows per lane in part A and part B. The occupancy hint
// keeps register use low enough for many rows in flight (lower for the widest
// rows, for two V2 value chunks and for two rows per lane, so that no
// instantiation spills).
constexpr int kv_waves(int ca, int cb, bool v2, int ra, int rb) {
    return ra == 2 ? 4 : (ca >= 4 ? 6 : ((ca == 3 || (v2 && cb == 2) || rb == 2) ? 7 : 8));
}

template <typename T, int VEC, bool V2, int CA, int CB, int RA, int RB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kv_waves(CA, CB, V2, RA, RB), 8))) void kv_rmsnorm_rope_cache_kernel(
    KvParams params) {
    // Read the fields where they are used, from the kernel-argument segment
    // (scalar loads), rather than all at entry: the entry loads of a struct
    // this wide stay live across both parts and spill.
    (void)params;
    const KvParams &p = *(const KvParams *)__builtin_amdgcn_kernarg_segment_ptr();
    // V1: part B's blocks first (its rows are short and latency-bound; started
    // early they overlap part A's stream instead of forming the tail);
    // V2: part A's first (measured: V1 prefill -2.6 %, V2 split +9 % the other way)
    constexpr bool kBFirst = !V2;
    const uint32_t first_blocks = kBFirst ? p.blocks_b : p.blocks_a;
    if (kBFirst ? blockIdx.x >= first_blocks : blockIdx.x < first_blocks) {
        const uint32_t blk = kBFirst ? blockIdx.x - first_blocks : blockIdx.x;
        switch (V2 ? p.k_code : p.c_code) {
        case CODE_INT8: part_a<T, VEC, V2, CA, CODE_INT8, RA>(p, blk); break;
        case CODE_E4M3FN: part_a<T, VEC, V2, CA, CODE_E4M3FN, RA>(p, blk); break;
        case CODE_E5M2: part_a<T, VEC, V2, CA, CODE_E5M2, RA>(p, blk); break;
        default: part_a<T, VEC, V2, CA, CODE_SAME, RA>(p, blk); break;
        }
    } else {
        const uint32_t blk = kBFirst ? blockIdx.x : blockIdx.x - first_blocks;
        switch (V2 ? p.c_code : p.k_code) {
        case CODE_INT8: part_b<T, VEC, V2, CB, CODE_INT8, RB>(p, blk); break;
        case CODE_E4M3FN: part_b<T, VEC, V2, CB, CODE_E4M3FN, RB>(p, blk); break;
        case CODE_E5M2: part_b<T, VEC, V2, CB, CODE_E5M2, RB>(p, blk); break;
        default: part_b<T, VEC, V2, CB, CODE_SAME, RB>(p, blk); break;
        }
    }
}

// ---------------------------------------------------------------------------
// launch templates (the kernel instantiations of one element type per translation unit)
// ---------------------------------------------------------------------------

template <typename T, int VEC, bool V2>
inline hipError_t launch_t(const KvParams &p, int ca, int cb, hipStream_t stream) {
    dim3 grid(p.blocks_a + p.blocks_b), block(256);
#define QKNR_KV(CAV, CBV, RAV, RBV)                                                                       \
    if (ca == CAV && cb == CBV && p.ra == RAV && p.rb == RBV) {                                           \
        hipLaunchKernelGGL((kv_rmsnorm_rope_cache_kernel<T, VEC, V2, CAV, CBV, RAV, RBV>), grid, block,    \
                           4u * (uint32_t)p.lds_wave_bytes, stream, p);                                   \
        return hipGetLastError();                                                                         \
    }
    QKNR_KV(1, 1, 1, 1) QKNR_KV(2, 1, 1, 1) QKNR_KV(3, 1, 1, 1) QKNR_KV(4, 1, 1, 1)
    QKNR_KV(1, 2, 1, 1) QKNR_KV(2, 2, 1, 1) QKNR_KV(3, 2, 1, 1) QKNR_KV(4, 2, 1, 1)
    if constexpr (VEC == 8) {
        QKNR_KV(1, 1, 1, 2) QKNR_KV(2, 1, 1, 2) QKNR_KV(3, 1, 1, 2) QKNR_KV(4, 1, 1, 2)
        if constexpr (V2) {
            QKNR_KV(1, 2, 1, 2) QKNR_KV(2, 2, 1, 2) QKNR_KV(3, 2, 1, 2) QKNR_KV(4, 2, 1, 2)
        } else {
            QKNR_KV(1, 1, 2, 2) QKNR_KV(2, 1, 2, 2) QKNR_KV(3, 1, 2, 2) QKNR_KV(4, 1, 2, 2)
        }
    }
#undef QKNR_KV
    return hipErrorInvalidValue;
}

template <typename T>
inline hipError_t launch_elem(const KvParams &p, int vec, bool v2, int ca, int cb, hipStream_t stream) {
    if (vec == 8) return v2 ? launch_t<T, 8, true>(p, ca, cb, stream) : launch_t<T, 8, false>(p, ca, cb, stream);
    return v2 ? launch_t<T, 4, true>(p, ca, cb, stream) : launch_t<T, 4, false>(p, ca, cb, stream);
}

}  // namespace qknr
