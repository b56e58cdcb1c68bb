// launch.h -- flat kernel parameter blocks and launcher entry points shared by
// the C-ABI layer (api.cpp) and the two kernels. Host and device code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qknr {

// Unsigned 32-bit division by a runtime-invariant divisor d >= 1 with a
// multiply-high and two shifts: for l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (t + ((n - t) >> 1)) >> (l - 1)
// with t = mulhi(n, m) (the round-up method of Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994); d = 1 uses
// m = 0 and zero shifts. Exact for every n < 2^32.
struct FastDiv {
    uint32_t d, m, sh1, sh2;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f{d, 0u, 0u, 0u};
    if (d <= 1) return f;
    uint32_t l = 0;
    while ((1ull << l) < d) l++;
    f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    f.sh1 = 1;
    f.sh2 = l - 1;
    return f;
}

__host__ __device__ inline uint32_t fastdiv(uint32_t n, const FastDiv &f) {
#ifdef __HIP_DEVICE_COMPILE__
    const uint32_t t = __umulhi(n, f.m);
#else
    const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
#endif
    return (t + ((n - t) >> f.sh1)) >> f.sh2;
}

// (a) QK RMSNorm + rotate-half RoPE. The kernel has four forms:
//   QK_ACROSS    one RMS per (token, segment) over all its heads, then RoPE;
//   QK_PER_HEAD  one RMS per (token, head), gamma [head_dim] shared by heads;
//   QK_SUMSQ     first pass of a split over ranks: each (token, segment)'s sum
//                of squares over this call's heads -> sumsq[seg*tokens + t];
//   QK_APPLY     second pass: RMS from sumsq (the sum over every rank) and
//                q_channels / k_channels (the whole segment), then as QK_ACROSS.
enum QkMode : int32_t { QK_ACROSS = 0, QK_PER_HEAD = 1, QK_SUMSQ = 2, QK_APPLY = 3 };

struct QkParams {
    const void *q_in;
    const void *k_in;
    void *q_out;
    void *k_out;
    const void *q_gamma;
    const void *k_gamma;
    const void *cos;
    const void *sin;
    int64_t in_batch_stride, in_token_stride;
    int64_t out_batch_stride, out_token_stride;
    int64_t rope_batch_stride, rope_token_stride;
    uint32_t tokens;           // B*S (< 2^31)
    uint32_t seq;
    FastDiv seq_div;           // token -> (b, s)
    uint32_t in_head_stride, out_head_stride;   // elements; head offsets fit 32 bits
    int32_t n_q, n_k, head_dim, half;
    int32_t chunks_per_half;   // half / VEC
    int32_t heads_per_step;    // 64 / chunks_per_half
    int32_t waves_per_unit;    // W: waves sharing one (token, segment), 1, 2 or 4
    int32_t segs;              // 2 with a K segment, 1 for Q only
    int32_t apply_norm, apply_rope;
    float q_channels, k_channels, eps;   // RMS denominators (QK_PER_HEAD: head_dim)
    float *sumsq;              // QK_SUMSQ output [segs, tokens] / QK_APPLY input [segs, tokens, sum_parts]
    int32_t sum_parts;         // QK_APPLY: partial sums per token and segment, added in order
};

// Fills the lane geometry of p for chunk width `vec`; returns J > 0 or -1.
int qk_plan(QkParams &p, int vec);
// elem_type: 0 f32, 1 bf16, 2 f16. vec: 16-byte chunk width, or the narrow fallback.
hipError_t qk_launch(QkParams &p, int elem_type, int vec, int mode, hipStream_t stream);
// One translation unit per form (compiled in parallel); J from qk_plan.
hipError_t qk_launch_across(const QkParams &p, int elem_type, int vec, int J, hipStream_t stream);
hipError_t qk_launch_per_head(const QkParams &p, int elem_type, int vec, int J, hipStream_t stream);
hipError_t qk_launch_split(const QkParams &p, int elem_type, int vec, int J, int mode, hipStream_t stream);

// Interleaved-pair -> rotate-half lane permutation of a tensor viewed as
// [outer, axis_len, inner]: along the axis, n_heads blocks of head_dim starting
// at `first` are permuted (inverse: back); every other index is copied.
struct PermuteParams {
    const void *src;
    void *dst;
    uint64_t outer, axis_len, units_per_index;   // units of `unit` bytes per axis index
    uint64_t first, n_heads, head_dim;
    int32_t inverse;
};
// unit: bytes moved per access (1, 2, 4, 8 or 16), dividing the bytes per index.
hipError_t permute_launch(const PermuteParams &p, int unit, hipStream_t stream);

// QKV projection O[m, n] = sum_k A[m, k] W[n, k] (* a_scale[m] * w_scale[n])
// + bias[n] (bf16 or FP8 E4M3 operands, the FP8 ones optionally with MX block
// scales along k, fp32 accumulation, bf16 bias and
// output) with per-row partial sums of squares of the Q columns
// [0, q_cols) and the K columns [q_cols, q_cols + k_cols) of each 128-column
// tile: sumsq[(seg*m + row)*parts + part], parts = q_cols / 128.
struct ProjParams {
    const void *a;             // [m, k], row stride lda
    const void *w;             // [n, k], row stride ldw
    const void *bias;          // [n] bf16 or nullptr
    const float *a_scale;      // [m] or nullptr (per-row dequantisation)
    const float *w_scale;      // [n] or nullptr (per-channel dequantisation)
    void *o;                   // [m, n], row stride ldo
    float *sumsq;
    int64_t m, n, k, lda, ldw, ldo;
    int64_t q_cols, k_cols, parts;
    uint32_t tiles_m, tiles_n; // set by the launcher
    // MXFP8: E8M0 scale bytes, one per 32 values of k ([m, k/32] and [n, k/32],
    // row strides in bytes, multiples of 4); nullptr: no block scales
    const uint8_t *a_bs, *w_bs;
    int64_t lda_bs, ldw_bs;
};
// n a multiple of 128, k of 128 bytes; leading dimensions multiples of 16 bytes.
hipError_t proj_launch(ProjParams &p, bool fp8, hipStream_t stream);

// (b) KvRmsNormRopeCache
enum CacheCode : int32_t { CODE_SAME = 0, CODE_INT8 = 1, CODE_E4M3FN = 2, CODE_E5M2 = 3 };
enum QShape : int32_t { QS_SCALAR = 0, QS_CHANNEL = 1, QS_HEAD_CHANNEL = 2 };

struct KvParams {
    const void *kv;
    const void *v;
    const void *gamma;
    const void *cos;
    const void *sin;
    const int64_t *index;
    void *k_cache;
    void *ckv_cache;
    const float *k_scale, *k_offset, *v_scale, *v_offset;
    void *k_rope;
    void *c_kv;
    uint32_t rows;             // B*N*S (< 2^31)
    uint32_t seq;
    FastDiv seq_div, heads_div, block_div;   // row -> (b, n, s); slot -> (block, offset)
    // strides in elements, each < 2^32 (offsets are summed in 64 bits)
    uint32_t kv_b, kv_n, kv_s;
    uint32_t v_b, v_n, v_s;
    uint32_t rope_b, rope_n, rope_s;
    uint32_t kr_b, kr_n, kr_s; // k_rope strides
    uint32_t ck_b, ck_n, ck_s; // c_kv strides
    uint32_t kc0, kc1, kc2;    // k_cache strides (NORM: batch,row,head; PA: block,slot,head)
    uint32_t cc0, cc1, cc2;    // ckv_cache strides
    int64_t capacity;          // NORM: Scache; PA: block_num*block_size
    int32_t heads;
    int32_t mode;              // 0 NORM, 1 PA_BNSD, 2 PA_BLK_BNSD
    uint32_t runs;             // PA_BLK_BNSD: index entries per batch, ceil(seq / block_size)
    int32_t block_size;
    int32_t rms_size, rope_size, half_rope;
    int32_t k_dim, c_dim;      // widths of the k and ckv rows
    int32_t nr;                // part A chunks per row (the normed part)
    int32_t nx;                // part B chunks per row (V1: raw rope tail; V2: v row)
    int32_t n_rope_chunks;     // V2: rope_size / VEC (normed chunks that are rotated)
    int32_t ga, gb;            // lanes per row in part A / part B: 8, 16, 32 or 64
    int32_t ga_shift, gb_shift; // log2 of ga, gb
    int32_t ra, rb;            // rows per lane in part A / part B (1 or 2)
    int32_t lds_param_bytes, lds_code_bytes, lds_wave_bytes;   // per-wave LDS: staged parameters, staged codes
    int32_t stage_a, stage_b;  // the part's cache rows may leave as staged 16-byte pieces (see kv_plan)
    uint32_t blocks_a, blocks_b;   // blocks of part A, then of part B
    int32_t k_code, c_code;    // CacheCode
    int32_t k_qshape, v_qshape;
    int32_t out_kv;
    int32_t stream_rope;       // cos/sin read once (no S-axis broadcast): streaming loads
    float eps;
};

// Staged quantisation parameters of one wave: at most 512 floats (2 KB, two
// 16-byte pieces per lane), [scale[width] | offset[width]].
constexpr int kWaveParamFloats = 512;

// Lane geometry of the two row parts and their register slots; returns 0 and
// sets ca/cb, or -1 if a row is too wide.
int kv_plan(KvParams &p, int vec, bool v2, int &ca, int &cb);
// elem_type: 1 bf16, 2 f16. vec: 8 or 4.
hipError_t kv_launch(KvParams &p, int elem_type, int vec, bool v2, hipStream_t stream);
// The kernel instantiations of one element type (one translation unit each).
hipError_t kv_launch_bf16(const KvParams &p, int vec, bool v2, int ca, int cb, hipStream_t stream);
hipError_t kv_launch_f16(const KvParams &p, int vec, bool v2, int ca, int cb, hipStream_t stream);

}  // namespace qknr
