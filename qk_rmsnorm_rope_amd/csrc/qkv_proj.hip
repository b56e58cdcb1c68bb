// qkv_proj.hip -- the QKV projection with step a of the across-heads norm in
// its epilogue, for gfx950 matrix cores.
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
//     128 x 64 = 4 x 2 tiles of v_mfma_f32_32x32x16_bf16 (fp32 accumulators):
//     128 flops per byte staged, so the L2 -> LDS stream stays well below the
//     L2 bandwidth at the matrix cores' rate;
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
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WAVES_M = 2, WAVES_N = 4;             // wave grid of a workgroup (two per SIMD)
constexpr int THREADS = 64 * WAVES_M * WAVES_N;
constexpr int NWAVES = WAVES_M * WAVES_N;
constexpr int MT = BM / WAVES_M / 32, NT = BN / WAVES_N / 32;   // 32x32 MFMA tiles per wave
constexpr int LOADS = (BM / 8) / NWAVES;            // LDS-DMA instructions per wave per operand and k step
constexpr int STAGE_ELEMS = (BM + BN) * BK;         // one k step of A and W tiles (64 KB)
constexpr int LDC_S = BN + 8;                       // LDS row stride of the staged output tile
constexpr int GROUP_M = 8;
constexpr int LDS_BYTES_AB = 2 * STAGE_ELEMS * 2;   // two k-step buffers: 128 KB
constexpr int LDS_BYTES_C = BM * LDC_S * 2;         // 132 KB
constexpr int LDS_BYTES = LDS_BYTES_AB > LDS_BYTES_C ? LDS_BYTES_AB : LDS_BYTES_C;

struct alignas(16) U4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ void st_global16(void *p, const U4 &v) { *reinterpret_cast<U4 *>(p) = v; }
__device__ __forceinline__ U4 ld_lds16(const uint16_t *p) { return *reinterpret_cast<const U4 *>(p); }
__device__ __forceinline__ bf16x8_t as_bf16x8(const U4 &v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS slot of logical 16-byte chunk c (0..7) of tile row r (rows of 128 bytes).
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

__global__ __launch_bounds__(THREADS) void qkv_proj_bf16_kernel(ProjParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_BYTES / 2];

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

    // LDS-DMA sources: wave `wave`, instruction j fills tile rows 8*(4*wave + j) .. +7
    // (A rows for j < 4 of the A pass, W rows in the W pass); lane l -> row + l/8,
    // slot l%8, holding logical chunk swz(row, l%8).
    const uint16_t *a_src[LOADS], *w_src[LOADS];
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
            a_src[j] = reinterpret_cast<const uint16_t *>(p.a) + ra * p.lda + c * 8;
            w_src[j] = reinterpret_cast<const uint16_t *>(p.w) + rw * p.ldw + c * 8;
        }
    }
    auto issue_loads = [&](int ks, int buf) {
        uint16_t *as = lds + buf * STAGE_ELEMS;
        uint16_t *bs = as + BM * BK;
        const int64_t k0 = (int64_t)ks * BK;
#pragma unroll
        for (int j = 0; j < LOADS; j++)
            __builtin_amdgcn_global_load_lds(a_src[j] + k0, as + (LOADS * wave + j) * 8 * BK, 16, 0, 0);
#pragma unroll
        for (int j = 0; j < LOADS; j++)
            __builtin_amdgcn_global_load_lds(w_src[j] + k0, bs + (LOADS * wave + j) * 8 * BK, 16, 0, 0);
    };

    f32x16_t acc[MT][NT];
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[mi][ni][r] = 0.0f;

    // fragment rows: lane holds row (l % 32) of a 32-row tile and k chunk (l / 32) of a 16-k substep
    const int fr = lane & 31, fc = lane >> 5;
    const int ksteps = (int)(p.k / BK);
    issue_loads(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ks++) {
        const int buf = ks & 1;
        if (ks + 1 < ksteps) issue_loads(ks + 1, buf ^ 1);
        const uint16_t *as = lds + buf * STAGE_ELEMS;
        const uint16_t *bs = as + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            const int c = kk * 2 + fc;                // logical 16-byte chunk of this substep
            bf16x8_t af[MT], bfr[NT];
#pragma unroll
            for (int mi = 0; mi < MT; mi++) {
                const int row = wm * (MT * 32) + mi * 32 + fr;
                af[mi] = as_bf16x8(ld_lds16(as + row * BK + swz(row, c) * 8));
            }
#pragma unroll
            for (int ni = 0; ni < NT; ni++) {
                const int row = wn * (NT * 32) + ni * 32 + fr;
                bfr[ni] = as_bf16x8(ld_lds16(bs + row * BK + swz(row, c) * 8));
            }
#pragma unroll
            for (int mi = 0; mi < MT; mi++)
#pragma unroll
                for (int ni = 0; ni < NT; ni++)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);            // this wave's loads of the next step have landed
        __syncthreads();                          // ... everyone's, and no wave still reads `buf`
    }

    // epilogue 1: bias, round to bf16, stage the 256 x 256 tile in LDS
    uint16_t *Cs = lds;                           // [BM][LDC_S]
    const uint16_t *bias = reinterpret_cast<const uint16_t *>(p.bias);
#pragma unroll
    for (int ni = 0; ni < NT; ni++) {
        const int col = wn * (NT * 32) + ni * 32 + fr;
        float bv = 0.0f;
        if (bias && n0 + col < p.n) bv = __uint_as_float((uint32_t)bias[n0 + col] << 16);
#pragma unroll
        for (int mi = 0; mi < MT; mi++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = wm * (MT * 32) + mi * 32 + fc * 4 + (r >> 2) * 8 + (r & 3);
                const uint32_t packed = pack_bf16(acc[mi][ni][r] + bv, 0.0f);
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

hipError_t proj_launch(ProjParams &p, hipStream_t stream) {
    p.tiles_m = (uint32_t)((p.m + BM - 1) / BM);
    p.tiles_n = (uint32_t)((p.n + BN - 1) / BN);
    const uint64_t tiles = (uint64_t)p.tiles_m * p.tiles_n;
    if (tiles == 0) return hipSuccess;
    const uint64_t grid = (tiles + 7) / 8 * 8;          // a whole number of tiles per XCD
    hipLaunchKernelGGL(qkv_proj_bf16_kernel, dim3((uint32_t)grid), dim3(THREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace qknr
