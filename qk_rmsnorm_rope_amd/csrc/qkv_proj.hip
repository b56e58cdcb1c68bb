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
//   * 256 x 128 output tile per workgroup of 4 waves (2 x 2), each wave
//     128 x 64 = 4 x 2 tiles of v_mfma_f32_32x32x16_bf16 (fp32 accumulators);
//     k steps of 64, A and W tiles staged in LDS with rows padded to 144 bytes
//     so that the 16-byte fragment reads of 16 lanes hit disjoint banks;
//   * both operands are K-contiguous (W is [I, H], a linear layer's weight), so
//     every MFMA operand is one 16-byte LDS read;
//   * the next k step's tiles are loaded into registers while the current one
//     is multiplied (two workgroups per CU overlap each other's barriers);
//   * tiles are ordered in groups of 8 row-tiles and each XCD (workgroups go
//     round-robin over the 8 XCDs) takes a contiguous range of them, so the
//     workgroups running together on one XCD share A rows and W columns in
//     its L2; the whole weight (157 MB for Wan2.2) stays in the 256 MB MALL;
//   * epilogue: bias, RNE to bf16, the tile staged through LDS and written
//     with 16-byte stores, the sums of squares taken from the rounded values
//     (the values the apply pass reads back) with a 16-lane DPP reduction.
#include "device_common.h"
#include "launch.h"

namespace qknr {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int LDA_S = BK + 8;       // LDS row stride of the A / W tiles (elements): 144 bytes
constexpr int LDC_S = BN + 8;       // LDS row stride of the staged output tile: 272 bytes
constexpr int GROUP_M = 8;
constexpr int LDS_BYTES_AB = (BM + BN) * LDA_S * 2;
constexpr int LDS_BYTES_C = BM * LDC_S * 2;
constexpr int LDS_BYTES = LDS_BYTES_AB > LDS_BYTES_C ? LDS_BYTES_AB : LDS_BYTES_C;

struct alignas(16) U4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 ld_global16(const void *p) { return *reinterpret_cast<const U4 *>(p); }
__device__ __forceinline__ void st_global16(void *p, const U4 &v) { *reinterpret_cast<U4 *>(p) = v; }
__device__ __forceinline__ U4 ld_lds16(const uint16_t *p) { return *reinterpret_cast<const U4 *>(p); }
__device__ __forceinline__ void st_lds16(uint16_t *p, const U4 &v) { *reinterpret_cast<U4 *>(p) = v; }

__device__ __forceinline__ bf16x8_t as_bf16x8(const U4 &v) { return __builtin_bit_cast(bf16x8_t, v); }

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

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void qkv_proj_bf16_kernel(ProjParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_BYTES / 2];
    uint16_t *As = lds;                       // [BM][LDA_S]
    uint16_t *Bs = lds + BM * LDA_S;          // [BN][LDA_S] (rows are output channels)

    // tile order: a contiguous range of logical tiles per XCD, grouped by GROUP_M row-tiles
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
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // global -> register tile loads: 8 A chunks and 4 W chunks of 16 bytes per thread
    const int lr = t >> 3, lc = t & 7;        // row (plus 32*j) and 16-byte chunk within the k step
    const uint16_t *a_base = reinterpret_cast<const uint16_t *>(p.a);
    const uint16_t *w_base = reinterpret_cast<const uint16_t *>(p.w);
    U4 ra[8], rb[4];
    auto load_tiles = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int64_t row = m0 + lr + 32 * j;
            if (row < p.m) ra[j] = ld_global16(a_base + row * p.lda + k0 + lc * 8);
            else ra[j] = U4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t col = n0 + lr + 32 * j;      // always < n: n is a multiple of BN
            rb[j] = ld_global16(w_base + col * p.ldw + k0 + lc * 8);
        }
    };
    auto store_tiles = [&]() {
#pragma unroll
        for (int j = 0; j < 8; j++) st_lds16(As + (lr + 32 * j) * LDA_S + lc * 8, ra[j]);
#pragma unroll
        for (int j = 0; j < 4; j++) st_lds16(Bs + (lr + 32 * j) * LDA_S + lc * 8, rb[j]);
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; mi++)
#pragma unroll
        for (int ni = 0; ni < 2; ni++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[mi][ni][r] = 0.0f;

    // fragment addresses: lane holds row (l % 32) of a 32-row tile and k (l / 32)*8 .. +7
    const int fr = lane & 31, fk = (lane >> 5) * 8;
    const uint16_t *a_frag = As + (wm * 128 + fr) * LDA_S + fk;
    const uint16_t *b_frag = Bs + (wn * 64 + fr) * LDA_S + fk;

    const int ksteps = (int)(p.k / BK);
    load_tiles(0);
    store_tiles();
    __syncthreads();
    for (int ks = 0; ks < ksteps; ks++) {
        if (ks + 1 < ksteps) load_tiles((int64_t)(ks + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            bf16x8_t af[4], bfr[2];
#pragma unroll
            for (int mi = 0; mi < 4; mi++) af[mi] = as_bf16x8(ld_lds16(a_frag + mi * 32 * LDA_S + kk * 16));
#pragma unroll
            for (int ni = 0; ni < 2; ni++) bfr[ni] = as_bf16x8(ld_lds16(b_frag + ni * 32 * LDA_S + kk * 16));
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
#pragma unroll
                for (int ni = 0; ni < 2; ni++)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
        __syncthreads();                      // every wave is done with this k step's tiles
        if (ks + 1 < ksteps) {
            store_tiles();
            __syncthreads();
        }
    }

    // epilogue 1: bias, round to bf16, stage the 256 x 128 tile in LDS
    uint16_t *Cs = lds;                       // [BM][LDC_S]
    const uint16_t *bias = reinterpret_cast<const uint16_t *>(p.bias);
#pragma unroll
    for (int ni = 0; ni < 2; ni++) {
        const int col = wn * 64 + ni * 32 + fr;
        const float bv = bias ? __uint_as_float((uint32_t)bias[n0 + col] << 16) : 0.0f;
#pragma unroll
        for (int mi = 0; mi < 4; mi++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = wm * 128 + mi * 32 + (lane >> 5) * 4 + (r >> 2) * 8 + (r & 3);
                const uint32_t packed = pack_bf16(acc[mi][ni][r] + bv, 0.0f);
                Cs[row * LDC_S + col] = (uint16_t)(packed & 0xFFFFu);
            }
        }
    }
    __syncthreads();

    // epilogue 2: 16-byte coalesced stores (16 lanes per 256-byte row) and the
    // per-row sums of squares of a Q or K tile
    int seg = -1;
    int64_t part = 0;
    if (p.q_cols > 0 && n0 < p.q_cols) {
        seg = 0;
        part = n0 / BN;
    } else if (p.k_cols > 0 && n0 >= p.q_cols && n0 < p.q_cols + p.k_cols) {
        seg = 1;
        part = (n0 - p.q_cols) / BN;
    }
    uint16_t *o_base = reinterpret_cast<uint16_t *>(p.o);
    const int cr = t >> 4, cc = t & 15;
#pragma unroll 4
    for (int j = 0; j < BM / 16; j++) {
        const int row = cr + 16 * j;
        const U4 v = ld_lds16(Cs + row * LDC_S + cc * 8);
        const bool ok = m0 + row < p.m;
        if (ok) st_global16(o_base + (m0 + row) * p.ldo + n0 + cc * 8, v);
        if (seg >= 0) {
            const float ss = group_sum<16>(sumsq8(v));
            if (ok && cc == 0) p.sumsq[((int64_t)seg * p.parts + part) * p.m + m0 + row] = ss;
        }
    }
}

}  // namespace

hipError_t proj_launch(ProjParams &p, hipStream_t stream) {
    p.tiles_m = (uint32_t)((p.m + BM - 1) / BM);
    p.tiles_n = (uint32_t)(p.n / BN);
    const uint64_t tiles = (uint64_t)p.tiles_m * p.tiles_n;
    if (tiles == 0) return hipSuccess;
    const uint64_t grid = (tiles + 7) / 8 * 8;          // a whole number of tiles per XCD
    hipLaunchKernelGGL(qkv_proj_bf16_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace qknr
