// qkv_proj.hip -- the QKV projection with step a of the across-heads norm in
// its epilogue, for gfx950 matrix cores, with bf16 operands or FP8 E4M3
// operands with per-row / per-channel dequantisation scales (ROW_MX) and/or
// MX block scales (MXFP8: one E8M0 scale per 32 values along k, the OCP
// Microscaling format).
//
// "Kernel reference: qkv_cte" describes the projection O[S, I] = A[S, H] @ W +
// bias that produces Q|K|V ("Upstream behavior") and, for the across-heads
// norm, accumulates each token's sum(x^2) over the Q and the K segment while
// the finished output tile is copied out (Design section 1, step a), so that
// only the apply pass (step c) re-reads Q and K. Here the copy-out is the
// GEMM epilogue: each output tile's Q or K columns add one partial sum per row
// to a [segment][part][row] array, and the apply kernel adds the parts.
//
// MI355X design:
//   * 256 x 256 output tile per workgroup of 8 waves (2 x 4), each wave
//     128 x 64 = 4 x 2 tiles of 32 x 32 MFMAs with fp32 accumulators:
//     v_mfma_f32_32x32x16_bf16, or for FP8 v_mfma_scale_f32_32x32x64_f8f6f4,
//     whose per-lane scale operands carry the MX block scales (a substep's
//     64 k values are two MX blocks; lane l passes the scale of row l % 32's
//     block l / 32, and each lane holds 16 values of each block, the layout
//     the instruction requires), or unit scales for ROW_MX (whose scales are
//     applied in the epilogue);
//     the block scales of a tile's rows move global -> LDS with the tiles, in
//     groups of four k steps one group ahead (coalesced 16-byte row pieces,
//     rows rotated in LDS so that each lane's ds_read of its row's 4-byte
//     word is conflict-free), and each lane shifts its block's byte down;
//     a k step is one 128-byte row per operand row (64 bf16 or 128 FP8
//     values), so both types share the LDS tiling below;
//   * both operands are K-contiguous (W is [I, H], a linear layer's weight), so
//     every MFMA operand is one 16-byte LDS read;
//   * tiles move global -> LDS with global_load_lds_dwordx4 (no registers):
//     each wave instruction fills 8 rows of 128 bytes, and a 16-byte chunk c
//     of row r sits in slot c ^ ((r >> 1) & 7), so the fragment reads of 16
//     consecutive rows hit 16 disjoint bank groups; two k-step buffers (128 KB)
//     let the next step's loads run under the current step's MFMAs, with one
//     barrier per k step;
//   * workgroups go round-robin over the 8 XCDs; each XCD takes a contiguous
//     range of tiles ordered in groups of 8 row-tiles, row-tile fastest, so
//     the ~32 workgroups running together on one XCD cover 8 row-tiles x 4
//     column-tiles and read each k step of 12 tiles through its L2 instead
//     of 32 (measured: L2 misses 6.5x the compulsory bytes, against 16x when
//     the XCDs share one row-tile each); the weight (157 MB) fits the MALL;
//   * epilogue: bias, RNE to bf16, the tile staged through LDS and written
//     with 16-byte stores, the sums of squares taken from the rounded values
//     (the values the apply pass reads back) with 16-lane DPP reductions, one
//     per 128-column half of the tile.
#include "device_common.h"
#include "launch.h"

namespace qknr {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256;
constexpr int ROW_BYTES = 128;                      // one k step of one tile row, in bytes
constexpr int WAVES_M = 2, WAVES_N = 4;             // wave grid of a workgroup (two per SIMD)
constexpr int THREADS = 64 * WAVES_M * WAVES_N;
constexpr int NWAVES = WAVES_M * WAVES_N;
constexpr int MT = BM / WAVES_M / 32, NT = BN / WAVES_N / 32;   // 32x32 MFMA tiles per wave
constexpr int LOADS = (BM / 8) / NWAVES;            // LDS-DMA instructions per wave per operand and k step
constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;  // one k step of A and W tiles (64 KB)
constexpr int LDC_S = BN + 8;                       // LDS row stride of the staged output tile (elements)
constexpr int GROUP_M = 8;
constexpr int LDS_BYTES_AB = 2 * STAGE_BYTES;       // two k-step buffers: 128 KB
constexpr int LDS_BYTES_C = BM * LDC_S * 2 + BM * 4;   // 132 KB output tile + the row scales
// MX block scales: groups of 4 k steps (16 scale bytes per tile row and
// operand), two group buffers after the tile buffers
constexpr int MX_GROUP = 4;                          // k steps per scale group
constexpr int MX_OPERAND_BYTES = BM * MX_GROUP * 4;  // one group of one operand's 256 rows: 4 KB
constexpr int MX_BYTES = 2 * 2 * MX_OPERAND_BYTES;   // two groups x (A, W): 16 KB
constexpr int lds_bytes(bool mx) {
    const int ab = LDS_BYTES_AB + (mx ? MX_BYTES : 0);
    return ab > LDS_BYTES_C ? ab : LDS_BYTES_C;
}
static_assert(BM == BN, "one scale-group layout for both operands");

// Word index of (tile row r, k step j of the group) in a group buffer: rows of
// four words, rotated by r / 8, so that the 32 rows of one MFMA tile read at
// one k step fall in 32 distinct banks (r = 8a + b -> bank 4b + (j + a) % 4).
__device__ __forceinline__ int mx_word(int r, int j) { return r * MX_GROUP + ((j + (r >> 3)) & (MX_GROUP - 1)); }

struct alignas(16) U4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ void st_global16(void *p, const U4 &v) { *reinterpret_cast<U4 *>(p) = v; }
__device__ __forceinline__ U4 ld_lds16(const void *p) { return *reinterpret_cast<const U4 *>(p); }

// LDS slot of logical 16-byte chunk c (0..7) of tile row r (rows of 128 bytes):
// 16 consecutive rows of one chunk land in 16 distinct 4-bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// Sum of squares of the 8 bf16 values of a 16-byte chunk (fp32).
__device__ __forceinline__ float sumsq8(const U4 &v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float a = lo_bf16(w[i]), b = hi_bf16(w[i]);
        s = fmaf(a, a, s);
        s = fmaf(b, b, s);
    }
    return s;
}

// One MFMA operand of substep kk of a k step: the lane's 16 (bf16) or 32
// (FP8) bytes of tile row `row`; lanes l and l + 32 hold the two halves of the
// substep's k range (any split works as long as A and W use the same one,
// except that MX block scales need the FP8 split below).
template <bool FP8>
struct Frag;

template <>
struct Frag<false> {
    bf16x8_t v;
    __device__ __forceinline__ void read(const uint8_t *tile, int row, int kk, int half) {
        v = __builtin_bit_cast(bf16x8_t, ld_lds16(tile + row * ROW_BYTES + swz(row, kk * 2 + half) * 16));
    }
};

// FP8: the 64 k values of substep kk are blocks 2kk and 2kk + 1 of 32 (one MX
// block each). The scaled 32x32x64 MFMA counts bytes 0-15 of every lane in
// its first k block and bytes 16-31 in its second, and takes the first block's
// scale from lane r and the second's from lane r + 32 (measured on gfx950 with
// in-bounds probes: one 1.0 at each byte of lane 0 and of lane 32 under a
// doubled second-block scale). So lane half h holds 16 values of each block:
// chunk 4kk + h (block 2kk, its values 16h..16h+15) and chunk 4kk + 2 + h
// (block 2kk + 1, likewise), and lane r + 32h passes the scale of block 2kk + h.
template <>
struct Frag<true> {
    i32x8_t v;
    __device__ __forceinline__ void read(const uint8_t *tile, int row, int kk, int half) {
        const int c = kk * 4 + half;
        const U4 lo = ld_lds16(tile + row * ROW_BYTES + swz(row, c) * 16);
        const U4 hi = ld_lds16(tile + row * ROW_BYTES + swz(row, c + 2) * 16);
        v = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
};

__device__ __forceinline__ f32x16_t mfma(const Frag<false> &a, const Frag<false> &b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma(const Frag<true> &a, const Frag<true> &b, f32x16_t c) {
    // both operands FP8 E4M3 (format 0), block scales 2^(127 - 127) = 1
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, b.v, c, 0, 0, 0, 127, 0, 127);
}
// FP8 E4M3 operands with per-lane E8M0 block scales (byte 0 of sa / sb)
__device__ __forceinline__ f32x16_t mfma_mx(const Frag<true> &a, const Frag<true> &b, f32x16_t c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, b.v, c, 0, 0, 0, sa, 0, sb);
}

template <bool FP8, bool MX>
__global__ __launch_bounds__(THREADS) void qkv_proj_kernel(ProjParams p) {
    static_assert(FP8 || !MX, "MX block scales come with FP8 operands");
    constexpr int EB = FP8 ? 1 : 2;                 // operand bytes per element
    constexpr int KSUB = FP8 ? 2 : 4;               // MFMA substeps per 128-byte k step
    __shared__ __attribute__((aligned(16))) uint8_t lds[lds_bytes(MX)];

    // tile order: a contiguous range of logical tiles per XCD (workgroup i runs on
    // XCD i % 8), grouped by GROUP_M row-tiles
    const uint32_t per_xcd = gridDim.x / 8;
    const uint32_t lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (lid >= p.tiles_m * p.tiles_n) return;
    const uint32_t in_group = GROUP_M * p.tiles_n;
    const uint32_t first_m = (lid / in_group) * GROUP_M;
    const uint32_t gm = min((uint32_t)GROUP_M, p.tiles_m - first_m);
    const uint32_t tile_m = first_m + (lid % in_group) % gm;
    const uint32_t tile_n = (lid % in_group) / gm;
    const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // LDS-DMA sources: wave `wave`, instruction j fills tile rows 8*(LOADS*wave + j) .. +7
    // of A, then the same rows of W; lane l -> row + l/8, slot l%8, holding logical
    // chunk swz(row, l%8).
    const uint8_t *a_src[LOADS], *w_src[LOADS];
    {
        const int slot = lane & 7;
#pragma unroll
        for (int j = 0; j < LOADS; j++) {
            const int row = 8 * (LOADS * wave + j) + (lane >> 3);
            const int c = swz(row, slot);
            int64_t ra = m0 + row;
            if (ra >= p.m) ra = p.m - 1;             // rows past M: any valid data, never stored
            int64_t rw = n0 + row;
            if (rw >= p.n) rw = p.n - 1;             // columns past N (a final half tile)
            a_src[j] = reinterpret_cast<const uint8_t *>(p.a) + (ra * p.lda) * EB + c * 16;
            w_src[j] = reinterpret_cast<const uint8_t *>(p.w) + (rw * p.ldw) * EB + c * 16;
        }
    }
    auto issue_loads = [&](int ks, int buf) {
        uint8_t *as = lds + buf * STAGE_BYTES;
        uint8_t *bs = as + BM * ROW_BYTES;
        const int64_t k0 = (int64_t)ks * ROW_BYTES;
#pragma unroll
        for (int j = 0; j < LOADS; j++)
            __builtin_amdgcn_global_load_lds(a_src[j] + k0, as + (LOADS * wave + j) * 8 * ROW_BYTES, 16, 0, 0);
#pragma unroll
        for (int j = 0; j < LOADS; j++)
            __builtin_amdgcn_global_load_lds(w_src[j] + k0, bs + (LOADS * wave + j) * 8 * ROW_BYTES, 16, 0, 0);
    };

    f32x16_t acc[MT][NT];
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[mi][ni][r] = 0.0f;

    // fragment rows: lane holds row (l % 32) of a 32-row tile and half (l / 32) of a substep's k
    const int fr = lane & 31, fc = lane >> 5;
    const int ksteps = (int)(p.k * EB / ROW_BYTES);

    // MX: the block scales move global -> LDS with the tiles, one group of
    // MX_GROUP k steps at a time (the 4-byte word of one k step holds the scales
    // of its four 32-value blocks; row r's words of a group are 16 contiguous
    // bytes), one group ahead, into the group buffer g & 1 at word mx_word(r, j).
    // Each of the 8 waves copies 2 x 64 words per operand and group: copy i
    // covers rows 16i .. 16i + 15, lane L row 16i + L/4 and, so that lane L
    // lands on word 64i + L, k step j = (L % 4 - r / 8) % 4. k steps past the
    // last (a partial last group) copy nothing. In substep kk lane half fc
    // passes the scale of block 2*kk + fc (see Frag<true>).
    const uint8_t *mx_src[MX ? 4 : 1];
    int mx_j[MX ? 4 : 1];
    if constexpr (MX) {
        const int lane_r = lane >> 2;
#pragma unroll
        for (int c = 0; c < 4; c++) {              // copies 0,1: A rows of copy 2*wave + c; 2,3: W rows
            const bool is_w = c >= 2;
            const int r = 16 * (2 * wave + (c & 1)) + lane_r;
            mx_j[c] = ((lane & 3) - (r >> 3)) & (MX_GROUP - 1);
            int64_t gr = (is_w ? n0 : m0) + r;
            const int64_t lim = is_w ? p.n : p.m;
            if (gr >= lim) gr = lim - 1;           // rows past M or N: any valid row, never stored
            mx_src[c] = (is_w ? p.w_bs + gr * p.ldw_bs : p.a_bs + gr * p.lda_bs) + 4 * mx_j[c];
        }
    }
    auto issue_scales = [&](int g) {
        if constexpr (MX) {
            uint8_t *dst = lds + LDS_BYTES_AB + (g & 1) * 2 * MX_OPERAND_BYTES;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int copy = 2 * wave + (c & 1);
                if (g * MX_GROUP + mx_j[c] < ksteps)
                    __builtin_amdgcn_global_load_lds(mx_src[c] + 4 * MX_GROUP * g,
                                                     dst + (c >= 2 ? MX_OPERAND_BYTES : 0) + copy * 256, 4, 0, 0);
            }
        }
    };

    issue_loads(0, 0);
    issue_scales(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ks++) {
        const int buf = ks & 1;
        if (ks + 1 < ksteps) issue_loads(ks + 1, buf ^ 1);
        uint32_t asw[MX ? MT : 1], wsw[MX ? NT : 1];   // this k step's scale words of the lane's rows
        if constexpr (MX) {
            const int g = ks / MX_GROUP, j = ks % MX_GROUP;
            if (j == 0 && (g + 1) * MX_GROUP < ksteps) issue_scales(g + 1);
            const uint32_t *sw = reinterpret_cast<const uint32_t *>(lds + LDS_BYTES_AB + (g & 1) * 2 * MX_OPERAND_BYTES);
#pragma unroll
            for (int mi = 0; mi < MT; mi++) asw[mi] = sw[mx_word(wm * (MT * 32) + mi * 32 + fr, j)];
#pragma unroll
            for (int ni = 0; ni < NT; ni++) wsw[ni] = sw[BM * MX_GROUP + mx_word(wn * (NT * 32) + ni * 32 + fr, j)];
        }
        const uint8_t *as = lds + buf * STAGE_BYTES;
        const uint8_t *bs = as + BM * ROW_BYTES;
#pragma unroll
        for (int kk = 0; kk < KSUB; kk++) {
            Frag<FP8> af[MT], bfr[NT];
#pragma unroll
            for (int mi = 0; mi < MT; mi++) af[mi].read(as, wm * (MT * 32) + mi * 32 + fr, kk, fc);
#pragma unroll
            for (int ni = 0; ni < NT; ni++) bfr[ni].read(bs, wn * (NT * 32) + ni * 32 + fr, kk, fc);
            if constexpr (MX) {
                const int sh = 8 * (2 * kk + fc);
                int sa[MT], sb[NT];
#pragma unroll
                for (int mi = 0; mi < MT; mi++) sa[mi] = (int)(asw[mi] >> sh);
#pragma unroll
                for (int ni = 0; ni < NT; ni++) sb[ni] = (int)(wsw[ni] >> sh);
#pragma unroll
                for (int mi = 0; mi < MT; mi++)
#pragma unroll
                    for (int ni = 0; ni < NT; ni++)
                        acc[mi][ni] = mfma_mx(af[mi], bfr[ni], acc[mi][ni], sa[mi], sb[ni]);
            } else {
#pragma unroll
                for (int mi = 0; mi < MT; mi++)
#pragma unroll
                    for (int ni = 0; ni < NT; ni++) acc[mi][ni] = mfma(af[mi], bfr[ni], acc[mi][ni]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);            // this wave's loads of the next step have landed
        __syncthreads();                          // ... everyone's, and no wave still reads `buf`
    }

    // epilogue 1: scales, bias, round to bf16, stage the 256 x 256 tile in LDS
    uint16_t *Cs = reinterpret_cast<uint16_t *>(lds);           // [BM][LDC_S]
    float *row_scale = reinterpret_cast<float *>(lds + BM * LDC_S * 2);
    if (p.a_scale && t < BM) {
        int64_t r = m0 + t;
        if (r >= p.m) r = p.m - 1;
        row_scale[t] = p.a_scale[r];
    }
    __syncthreads();
    const uint16_t *bias = reinterpret_cast<const uint16_t *>(p.bias);
#pragma unroll
    for (int ni = 0; ni < NT; ni++) {
        const int col = wn * (NT * 32) + ni * 32 + fr;
        const bool col_in = n0 + col < p.n;
        float bv = 0.0f, cs = 1.0f;
        if (bias && col_in) bv = __uint_as_float((uint32_t)bias[n0 + col] << 16);
        if (p.w_scale && col_in) cs = p.w_scale[n0 + col];
#pragma unroll
        for (int mi = 0; mi < MT; mi++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = wm * (MT * 32) + mi * 32 + fc * 4 + (r >> 2) * 8 + (r & 3);
                float v = acc[mi][ni][r];
                if (p.a_scale) v *= row_scale[row];
                if (p.w_scale) v *= cs;
                const uint32_t packed = pack_bf16(v + bv, 0.0f);
                Cs[row * LDC_S + col] = (uint16_t)(packed & 0xFFFFu);
            }
        }
    }
    __syncthreads();

    // epilogue 2: 16-byte coalesced stores (32 lanes per 512-byte row) and the
    // per-row sums of squares of each 128-column half that lies in Q or K
    const int half = (lane >> 4) & 1;             // lanes 0-15: columns 0..127, 16-31: 128..255
    const int64_t hc0 = n0 + half * 128;
    int seg = -1;
    int64_t part = 0;
    if (hc0 < p.q_cols) {
        seg = 0;
        part = hc0 / 128;
    } else if (hc0 >= p.q_cols && hc0 < p.q_cols + p.k_cols) {
        seg = 1;
        part = (hc0 - p.q_cols) / 128;
    }
    const bool col_ok = hc0 < p.n;
    uint16_t *o_base = reinterpret_cast<uint16_t *>(p.o);
    const int cr = t >> 5, cc = t & 31;
    constexpr int ROWS_PER_PASS = THREADS / 32;
#pragma unroll 4
    for (int j = 0; j < BM / ROWS_PER_PASS; j++) {
        const int row = cr + ROWS_PER_PASS * j;
        const U4 v = ld_lds16(Cs + row * LDC_S + cc * 8);
        const bool ok = m0 + row < p.m;
        if (ok && col_ok) st_global16(o_base + (m0 + row) * p.ldo + n0 + cc * 8, v);
        const float ss = group_sum<16>(sumsq8(v));
        if (seg >= 0 && ok && (cc & 15) == 0) p.sumsq[((int64_t)seg * p.m + m0 + row) * p.parts + part] = ss;
    }
}

}  // namespace

hipError_t proj_launch(ProjParams &p, bool fp8, hipStream_t stream) {
    p.tiles_m = (uint32_t)((p.m + BM - 1) / BM);
    p.tiles_n = (uint32_t)((p.n + BN - 1) / BN);
    const uint64_t tiles = (uint64_t)p.tiles_m * p.tiles_n;
    if (tiles == 0) return hipSuccess;
    const uint64_t grid = (tiles + 7) / 8 * 8;          // a whole number of tiles per XCD
    if (fp8 && p.a_bs)
        hipLaunchKernelGGL((qkv_proj_kernel<true, true>), dim3((uint32_t)grid), dim3(THREADS), 0, stream, p);
    else if (fp8)
        hipLaunchKernelGGL((qkv_proj_kernel<true, false>), dim3((uint32_t)grid), dim3(THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((qkv_proj_kernel<false, false>), dim3((uint32_t)grid), dim3(THREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace qknr
