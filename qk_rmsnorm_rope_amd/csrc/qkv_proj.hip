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
// GEMM epilogue: each 128-column part of an output tile that lies in Q or K
// writes one partial sum per row to a [segment][row][part] array (token-major,
// so the apply kernel loads a row's parts together and adds them).
//
// MI355X design:
//   * 256 x 384 (bf16, FP8 ROW_MX) or 256 x 256 (MXFP8) output tile per
//     workgroup of 8 waves (2 x 4), each wave 128 x 96 = 4 x 3 or 128 x 64 =
//     4 x 2 tiles of 32 x 32 MFMAs with fp32 accumulators (the wider tile moves
//     a fifth fewer LDS and copy bytes per flop; its 192 accumulators fill most
//     of the registers two waves per SIMD leave, so FP8's wider fragments are
//     read two A fragments at a time beside the substep's W fragments; MXFP8's
//     block scales need LDS the wider tile's two 80 KB k-step buffers leave no
//     room for):
//     v_mfma_f32_32x32x16_bf16 (on the 384-wide bf16 tile v_mfma_f32_16x16x32_bf16,
//     8 x 6 per wave, the W fragments of a substep held and four A fragments in
//     flight: 3 % faster, bit-identical), or for FP8 v_mfma_scale_f32_32x32x64_f8f6f4,
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
//   * tiles move global -> LDS with buffer_load_dwordx4 ... lds (no
//     registers; a buffer resource per tile, so each copy's address is a
//     32-bit lane offset fixed for the tile plus the k step in a scalar
//     register: 8 % faster than 64-bit per-lane addresses on the bf16 tile):
//     each wave instruction fills 8 rows of 128 bytes, and a 16-byte chunk c
//     of row r sits in slot c ^ ((r >> 1) & 7), so the fragment reads of 16
//     consecutive rows hit 16 disjoint bank groups; two k-step buffers (160 KB
//     for the 384-wide tile, 128 KB plus the block scales for MXFP8) let the
//     next step's loads run under the current step's MFMAs, with one barrier
//     per k step; with FP8 operands the four waves of one half issue the
//     copies of both waves on their SIMD, so that the other keeps the matrix
//     core busy meanwhile;
//   * workgroups go round-robin over the 8 XCDs; each XCD takes a contiguous
//     range of tiles ordered in groups of 4 row-tiles, row-tile fastest, so
//     the ~32 workgroups running together on one XCD cover 4 row-tiles x 8
//     column-tiles and share each k step of them through its L2. The weight
//     (157 MB bf16) stays in the MALL while A streams from HBM, so narrow
//     groups (each A row-tile re-read by few waves of column-tiles, the
//     weight re-read from the MALL more often) are fastest: measured on
//     Wan2.2 with this kernel, groups of 2 / 3 / 4 / 5 / 6 row-tiles take
//     9.03 / 9.10-9.18 / 8.97-9.02 / 9.16-9.29 / 9.27-9.30 ms (bf16),
//     4.61-4.62 / 4.61-4.62 / 4.53-4.58 / 4.57-4.58 / 4.61 ms (FP8) and
//     5.11 / 5.05-5.09 / 5.01-5.05 / 5.46-5.48 / 5.36-5.41 ms (MXFP8);
//   * the MFMAs take W as the first operand (they compute the transposed
//     tile), so each lane's accumulators hold four consecutive output columns
//     of one row per 8-column group: the epilogue applies scales and bias
//     from LDS copies (loaded before the k loop), rounds to bf16 and stages
//     the tile through LDS with 8-byte writes (in two passes of half of every
//     wave's rows for the 384-wide tile), then reads it out part by part
//     (each 16-lane group a fixed row offset, so the addresses are constants)
//     with 16-byte stores, and takes the sums of squares from the rounded
//     values (the values the apply pass reads back) with v_dot2 on bf16 pairs
//     and 16-lane DPP reductions, one per 128-column part of a row. With the
//     accumulators in the other layout (one column,
//     four rows per lane) the staging took 2-byte writes and the packing
//     per-element scale selects: measured on Wan2.2, this layout makes the
//     projection 2-3 % faster with bit-identical outputs.
#include "device_common.h"
#include "launch.h"

namespace qknr {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 256;
constexpr int ROW_BYTES = 128;                      // one k step of one tile row, in bytes
constexpr int WAVES_M = 2, WAVES_N = 4;             // wave grid of a workgroup (two per SIMD)
constexpr int THREADS = 64 * WAVES_M * WAVES_N;
constexpr int NWAVES = WAVES_M * WAVES_N;
constexpr int MT = BM / WAVES_M / 32;               // 32x32 MFMA tiles per wave along M
constexpr int LOADS = (BM / 8) / NWAVES;            // LDS-DMA instructions per wave and k step for A
constexpr int GROUP_M = 4;
// The block tile is BM x BN, BN = 256 (wave tiles 128 x 64) or 384 (128 x 96: a
// fifth fewer LDS and copy bytes per flop; the accumulators then fill most of
// the registers two waves per SIMD leave).
template <int BN>
struct Tile {
    static constexpr int NT = BN / WAVES_N / 32;            // 32x32 MFMA tiles per wave along N
    static constexpr int LOADS_W = (BN / 8) / NWAVES;       // LDS-DMA instructions per wave and k step for W
    static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;   // one k step of A and W: 64 or 80 KB
    static constexpr int LDS_BYTES_AB = 2 * STAGE_BYTES;    // two k-step buffers: 128 or 160 KB
    static constexpr int LDC_S = BN + 8;                    // LDS row stride of the staged output (elements)
    static constexpr int PASSES = BN == 256 ? 1 : 2;        // output staged in row halves when it would not fit
    static constexpr int ROWS_PER_PASS = BM / PASSES;
    // staged rows + per-column bias and scale + per-row scale (fp32)
    static constexpr int LDS_BYTES_C = ROWS_PER_PASS * LDC_S * 2 + (2 * BN + BM) * 4;
};
constexpr int LDS_BYTES_AB = Tile<256>::LDS_BYTES_AB;     // the MX path's tile buffers (BN = 256)
constexpr int STAGE_BYTES = Tile<256>::STAGE_BYTES;
constexpr int LDS_BYTES_C = Tile<256>::LDS_BYTES_C;
// MX block scales: groups of 4 k steps (16 scale bytes per tile row and
// operand), two group buffers after the tile buffers
constexpr int MX_GROUP = 4;                          // k steps per scale group
constexpr int MX_OPERAND_BYTES = BM * MX_GROUP * 4;  // one group of one operand's 256 rows: 4 KB
constexpr int MX_BYTES = 2 * 2 * MX_OPERAND_BYTES;   // two groups x (A, W): 16 KB
template <int BN>
constexpr int lds_bytes(bool mx) {
    const int ab = Tile<BN>::LDS_BYTES_AB + (mx ? MX_BYTES : 0);
    return ab > Tile<BN>::LDS_BYTES_C ? ab : Tile<BN>::LDS_BYTES_C;
}
static_assert(lds_bytes<384>(false) <= 160 * 1024 && lds_bytes<256>(true) <= 160 * 1024, "LDS of one CU");

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
__host__ __device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// Tile copies read through a buffer resource based at the tile's first row:
// the lane's 32-bit offset (row * pitch + the place of its 16-byte chunk) and
// the k step's byte offset in a scalar register; the LDS destination of a
// wave's copy is 64 consecutive 16-byte pieces.
struct TileRsrc {
    __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ TileRsrc tile_rsrc(const void *base, int64_t bytes) {
    return TileRsrc{__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000)};
}
__device__ __forceinline__ void copy16_to_lds(const TileRsrc &t, uint8_t *lds_dst, uint32_t lane_offset,
                                              int k_offset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(t.r, (lds_u8 *)lds_dst, 16, lane_offset, k_offset, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const TileRsrc &t, uint8_t *lds_dst, uint32_t lane_offset,
                                             int k_offset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(t.r, (lds_u8 *)lds_dst, 4, lane_offset, k_offset, 0, 0);
}
// Lane offset of one 16-byte piece of a tile copy: tile row `row` (rows at or
// past `rows` read the last valid row: any valid data, never stored), row
// pitch `pitch` bytes, the logical chunk that lands in LDS slot `slot`.
__device__ __forceinline__ uint32_t tile_offset(int row, int rows, int64_t pitch, int slot) {
    return (uint32_t)((int64_t)min(row, rows - 1) * pitch + swz(row, slot) * 16);
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

template <bool FP8, bool MX, int BN>
__global__ __launch_bounds__(THREADS) void qkv_proj_kernel(ProjParams p) {
    static_assert(FP8 || !MX, "MX block scales come with FP8 operands");
    static_assert(!MX || BN == 256, "the MX scale groups are laid out for 256-wide tiles");
    using TL = Tile<BN>;
    constexpr int NT = TL::NT, LOADS_W = TL::LOADS_W, STAGE_BYTES = TL::STAGE_BYTES, LDC_S = TL::LDC_S;
    constexpr int LDS_BYTES_AB = TL::LDS_BYTES_AB;
    constexpr int EB = FP8 ? 1 : 2;                 // operand bytes per element
    constexpr int KSUB = FP8 ? 2 : 4;               // MFMA substeps per 128-byte k step
    __shared__ __attribute__((aligned(16))) uint8_t lds[lds_bytes<BN>(MX)];

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

    // LDS-DMA: copy j of wave `wave` fills tile rows 8*(L*wave + j) .. +7 of an
    // operand (L = LOADS for A, LOADS_W for W); lane l -> row + l/8, LDS slot l%8,
    // holding logical chunk swz(row, l%8). The offsets are set once per tile; a
    // k step only moves the scalar offset.
    const int slot = lane & 7;
    const int64_t a_pitch = p.lda * EB, w_pitch = p.ldw * EB;
    const int a_rows = (int)min((int64_t)BM, p.m - m0), w_rows = (int)min((int64_t)BN, p.n - n0);
    const TileRsrc ra = tile_rsrc(reinterpret_cast<const uint8_t *>(p.a) + m0 * a_pitch,
                                  (int64_t)(a_rows - 1) * a_pitch + p.k * EB);
    const TileRsrc rw = tile_rsrc(reinterpret_cast<const uint8_t *>(p.w) + n0 * w_pitch,
                                  (int64_t)(w_rows - 1) * w_pitch + p.k * EB);
    uint32_t a_off[LOADS], w_off[LOADS_W];
#pragma unroll
    for (int j = 0; j < LOADS; j++) a_off[j] = tile_offset(8 * (LOADS * wave + j) + (lane >> 3), a_rows, a_pitch, slot);
#pragma unroll
    for (int j = 0; j < LOADS_W; j++)
        w_off[j] = tile_offset(8 * (LOADS_W * wave + j) + (lane >> 3), w_rows, w_pitch, slot);
    auto issue_loads = [&](int ks, int buf) {
        uint8_t *as = lds + buf * STAGE_BYTES;
        uint8_t *bs = as + BM * ROW_BYTES;
        const int k0 = ks * ROW_BYTES;
#pragma unroll
        for (int j = 0; j < LOADS; j++) copy16_to_lds(ra, as + (LOADS * wave + j) * 8 * ROW_BYTES, a_off[j], k0);
#pragma unroll
        for (int j = 0; j < LOADS_W; j++) copy16_to_lds(rw, bs + (LOADS_W * wave + j) * 8 * ROW_BYTES, w_off[j], k0);
    };
    // FP8 operands: in the k loop, wave w < 4 also issues the copies of wave
    // w + 4, which shares its SIMD, so that one of the two keeps the matrix core
    // busy while the other's copies queue (Wan2.2: MXFP8 -4 %, FP8 ROW_MX -1 %;
    // bf16 +1 %, so it keeps one share per wave). The partner's rows lie 32 L
    // rows further; rows past the tile's valid ones read the last valid row's
    // last chunk (in bounds for every k step, never stored). With row pitches
    // of at most 4 MiB the sums stay below 2^32 (at most 575 rows of pitch).
    constexpr bool PAIR_COPY = FP8;
    [[maybe_unused]] const bool copier = !PAIR_COPY || wave < NWAVES / 2;
    const uint32_t pair_a = (uint32_t)(8 * LOADS * (NWAVES / 2) * a_pitch);
    const uint32_t pair_w = (uint32_t)(8 * LOADS_W * (NWAVES / 2) * w_pitch);
    const uint32_t last_a = (uint32_t)((int64_t)(a_rows - 1) * a_pitch + ROW_BYTES - 16);
    const uint32_t last_w = (uint32_t)((int64_t)(w_rows - 1) * w_pitch + ROW_BYTES - 16);
    auto issue_pair_loads = [&](int ks, int buf) {
        uint8_t *as = lds + buf * STAGE_BYTES;
        uint8_t *bs = as + BM * ROW_BYTES;
        const int k0 = ks * ROW_BYTES;
        const int pw = wave + NWAVES / 2;
        uint32_t da = pair_a, dw = pair_w, ma = last_a, mw = last_w;
        asm volatile("" : "+s"(da), "+s"(dw), "+s"(ma), "+s"(mw));   // partner offsets formed here, not held
#pragma unroll
        for (int j = 0; j < LOADS; j++) copy16_to_lds(ra, as + (LOADS * wave + j) * 8 * ROW_BYTES, a_off[j], k0);
#pragma unroll
        for (int j = 0; j < LOADS; j++)
            copy16_to_lds(ra, as + (LOADS * pw + j) * 8 * ROW_BYTES, min(a_off[j] + da, ma), k0);
#pragma unroll
        for (int j = 0; j < LOADS_W; j++) copy16_to_lds(rw, bs + (LOADS_W * wave + j) * 8 * ROW_BYTES, w_off[j], k0);
#pragma unroll
        for (int j = 0; j < LOADS_W; j++)
            copy16_to_lds(rw, bs + (LOADS_W * pw + j) * 8 * ROW_BYTES, min(w_off[j] + dw, mw), k0);
    };

    // bf16 on the 384-wide tile: 16 x 16 x 32 MFMAs, 8 x 6 of them per wave (the
    // same 128 x 96 wave tile; 3 % faster than 32 x 32 x 16 on Wan2.2, bit-identical)
    constexpr bool M16 = !FP8 && BN == 384;
    f32x16_t acc[M16 ? 1 : MT][M16 ? 1 : NT];
    f32x4_t acc16[M16 ? 8 : 1][M16 ? 6 : 1];
    if constexpr (M16) {
#pragma unroll
        for (int mi = 0; mi < 8; mi++)
#pragma unroll
            for (int ni = 0; ni < 6; ni++) acc16[mi][ni] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
#pragma unroll
    for (int mi = 0; mi < MT; mi++)
#pragma unroll
        for (int ni = 0; ni < NT; ni++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[mi][ni][r] = 0.0f;
    }

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
    uint32_t mx_off[MX ? 4 : 1];
    int mx_j[MX ? 4 : 1];
    TileRsrc mx_ra{}, mx_rw{};
    if constexpr (MX) {
        // one buffer resource per operand's scale rows of the tile, like the
        // tile copies; lane offset row * stride + the word's place, the group's
        // 16 bytes as the scalar offset
        const int64_t blocks = p.k / 32;                      // scale bytes per row in use
        mx_ra = tile_rsrc(p.a_bs + m0 * p.lda_bs, (int64_t)(a_rows - 1) * p.lda_bs + blocks);
        mx_rw = tile_rsrc(p.w_bs + n0 * p.ldw_bs, (int64_t)(w_rows - 1) * p.ldw_bs + blocks);
        const int lane_r = lane >> 2;
#pragma unroll
        for (int c = 0; c < 4; c++) {              // copies 0,1: A rows of copy 2*wave + c; 2,3: W rows
            const bool is_w = c >= 2;
            const int r = 16 * (2 * wave + (c & 1)) + lane_r;
            mx_j[c] = ((lane & 3) - (r >> 3)) & (MX_GROUP - 1);
            // rows past M or N read the last valid row: any valid data, never stored
            const int rc = min(r, (is_w ? w_rows : a_rows) - 1);
            mx_off[c] = (uint32_t)(rc * (is_w ? p.ldw_bs : p.lda_bs) + 4 * mx_j[c]);
        }
    }
    auto issue_scales = [&](int g) {
        if constexpr (MX) {
            uint8_t *dst = lds + LDS_BYTES_AB + (g & 1) * 2 * MX_OPERAND_BYTES;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int copy = 2 * wave + (c & 1);
                if (g * MX_GROUP + mx_j[c] < ksteps)
                    copy4_to_lds(c >= 2 ? mx_rw : mx_ra, dst + (c >= 2 ? MX_OPERAND_BYTES : 0) + copy * 256,
                                 mx_off[c], 4 * MX_GROUP * g);
            }
        }
    };

    // the epilogue's per-column bias and channel scale (thread t: column t) and
    // per-row scale (thread t: row t), loaded now so that their latency is not
    // paid after the k loop
    float pre_b = 0.0f, pre_w = 1.0f, pre_a = 1.0f;
    if (t < BN && n0 + t < p.n) {
        if (p.bias) pre_b = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p.bias)[n0 + t] << 16);
        if (p.w_scale) pre_w = p.w_scale[n0 + t];
    }
    if (t < BM && p.a_scale) pre_a = p.a_scale[min(m0 + t, p.m - 1)];
    issue_loads(0, 0);
    issue_scales(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ks++) {
        const int buf = ks & 1;
        if constexpr (PAIR_COPY) {
            if (ks + 1 < ksteps && copier) issue_pair_loads(ks + 1, buf ^ 1);
        } else if (ks + 1 < ksteps) {
            issue_loads(ks + 1, buf ^ 1);
        }
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
        // LLVM's small-GEMM interleave of the fragment reads with the MFMAs
        // (measured on Wan2.2: bf16 -4 %, MXFP8 -1 %, FP8 level)
        __builtin_amdgcn_iglp_opt(0);
      if constexpr (M16) {
        // 16 x 16 x 32 MFMAs: lane l holds row l % 16 of a 16-row fragment and
        // the 8 k values of chunk 4 kk + l / 16 (any k split common to A and W)
        const int r16 = lane & 15, c16 = lane >> 4;
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            bf16x8_t b16[6];
#pragma unroll
            for (int ni = 0; ni < 6; ni++) {
                const int row = wn * 96 + ni * 16 + r16;
                b16[ni] = __builtin_bit_cast(bf16x8_t, ld_lds16(bs + row * ROW_BYTES + swz(row, kk * 4 + c16) * 16));
            }
            // A fragments read three row blocks ahead of their MFMAs (four in flight)
            auto rda = [&](int mi) {
                const int row = wm * 128 + mi * 16 + r16;
                return __builtin_bit_cast(bf16x8_t, ld_lds16(as + row * ROW_BYTES + swz(row, kk * 4 + c16) * 16));
            };
            bf16x8_t a0 = rda(0), a1 = rda(1), a2 = rda(2), a3;
#pragma unroll
            for (int mi = 0; mi < 8; mi++) {
                if (mi + 3 < 8) a3 = rda(mi + 3);
#pragma unroll
                for (int ni = 0; ni < 6; ni++)
                    acc16[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b16[ni], a0, acc16[mi][ni], 0, 0, 0);
                a0 = a1;
                a1 = a2;
                a2 = a3;
            }
        }
      } else if constexpr (FP8 && !MX && BN == 384) {
        // FP8 fragments are twice as wide: with the W fragments of a substep held,
        // the A fragments go two at a time, the next row block's read under the
        // current one's MFMAs (one A fragment at a time left the read latency
        // exposed: this order is 3.5 % faster on Wan2.2)
#pragma unroll
        for (int kk = 0; kk < KSUB; kk++) {
            Frag<FP8> bfr[NT];
#pragma unroll
            for (int ni = 0; ni < NT; ni++) bfr[ni].read(bs, wn * (NT * 32) + ni * 32 + fr, kk, fc);
            Frag<FP8> a_cur, a_next;
            a_cur.read(as, wm * (MT * 32) + fr, kk, fc);
#pragma unroll
            for (int mi = 0; mi < MT; mi++) {
                if (mi + 1 < MT) a_next.read(as, wm * (MT * 32) + (mi + 1) * 32 + fr, kk, fc);
#pragma unroll
                for (int ni = 0; ni < NT; ni++) acc[mi][ni] = mfma(bfr[ni], a_cur, acc[mi][ni]);
                a_cur = a_next;
            }
        }
      } else
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
                        acc[mi][ni] = mfma_mx(bfr[ni], af[mi], acc[mi][ni], sb[ni], sa[mi]);
            } else {
#pragma unroll
                for (int mi = 0; mi < MT; mi++)
#pragma unroll
                    for (int ni = 0; ni < NT; ni++) acc[mi][ni] = mfma(bfr[ni], af[mi], acc[mi][ni]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);            // this wave's loads of the next step have landed
        __syncthreads();                          // ... everyone's, and no wave still reads `buf`
    }

    // epilogue. The MFMAs above take W as the first operand, so each lane's
    // accumulators hold, for one row (token) m, four consecutive output columns
    // 8i + 4(lane / 32) + 0..3 of each 32-column tile (i = 0..3). Scales, bias,
    // RNE to bf16 in registers; the tile is staged in LDS with 8-byte writes
    // (in two passes of half the rows of every wave when it would not fit),
    // then written with 16-byte coalesced stores, 16 lanes per 128-column part
    // of a row, with that part's sum of the squares of the stored values when
    // it lies in Q or K.
    constexpr int PASSES = TL::PASSES, RPP = TL::ROWS_PER_PASS, PARTS = BN / 128;
    constexpr int MT_PASS = MT / PASSES, WROWS = MT_PASS * 32;   // a wave's rows per pass
    uint8_t *Cs = lds;                                            // [RPP][LDC_S] bf16
    float *col_bias = reinterpret_cast<float *>(lds + RPP * LDC_S * 2);
    float *col_scale = col_bias + BN;
    float *row_scale = col_scale + BN;
    if (t < BN) {
        col_bias[t] = pre_b;
        col_scale[t] = pre_w;
    }
    if (t < BM) row_scale[t] = pre_a;
    __syncthreads();
    const bool scaled = p.a_scale || p.w_scale;
    const int g16 = t >> 4, l16 = t & 15;
    // read-out: per 128-column part of the tile, its place in the output, and
    // the segment (Q: 0, K: 1, none: -1) and part index of its sums
    const int rows_in = (int)min((int64_t)BM, p.m - m0);
    uint16_t *o_lane = reinterpret_cast<uint16_t *>(p.o) + (m0 + g16) * p.ldo + n0 + l16 * 8;
    float *const sq_q = p.sumsq + m0 * p.parts, *const sq_k = p.sumsq + (p.m + m0) * p.parts;
    int part_seg[PARTS], part_idx[PARTS];
    bool part_in[PARTS];
#pragma unroll
    for (int q = 0; q < PARTS; q++) {
        const int64_t c0 = n0 + q * 128;
        part_in[q] = c0 < p.n;
        part_seg[q] = c0 < p.q_cols ? 0 : (c0 < p.q_cols + p.k_cols ? 1 : -1);
        part_idx[q] = (int)(part_seg[q] == 0 ? c0 / 128 : (c0 - p.q_cols) / 128);
    }
#pragma unroll
    for (int pass = 0; pass < PASSES; pass++) {
        if (pass > 0) __syncthreads();              // the previous pass's rows are read out
      if constexpr (M16) {
        // lane: token row 16 mi + l % 16 of the wave, columns 16 ni + 4 (l / 16) + 0..3
        const int r16 = lane & 15, c16 = lane >> 4;
#pragma unroll
        for (int ni = 0; ni < 6; ni++) {
            const int cb = wn * 96 + ni * 16 + 4 * c16;
            const U4 b4 = ld_lds16(col_bias + cb);
            const float bv[4] = {__uint_as_float(b4.x), __uint_as_float(b4.y), __uint_as_float(b4.z), __uint_as_float(b4.w)};
            float ws[4] = {1.0f, 1.0f, 1.0f, 1.0f};
            if (scaled) {
                const U4 w4 = ld_lds16(col_scale + cb);
                ws[0] = __uint_as_float(w4.x); ws[1] = __uint_as_float(w4.y);
                ws[2] = __uint_as_float(w4.z); ws[3] = __uint_as_float(w4.w);
            }
#pragma unroll
            for (int mh = 0; mh < 4; mh++) {
                const int mi = pass * 4 + mh;
                const int srow = wm * WROWS + mh * 16 + r16;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; r++) v[r] = acc16[mi][ni][r];
                if (scaled) {
                    const float as = row_scale[wm * 128 + mi * 16 + r16];
#pragma unroll
                    for (int r = 0; r < 4; r++) v[r] = v[r] * as * ws[r];
                }
                const uint32_t lo = pack_bf16(v[0] + bv[0], v[1] + bv[1]);
                const uint32_t hi = pack_bf16(v[2] + bv[2], v[3] + bv[3]);
                *reinterpret_cast<uint2 *>(Cs + srow * (LDC_S * 2) + cb * 2) = make_uint2(lo, hi);
            }
        }
      } else
#pragma unroll
        for (int ni = 0; ni < NT; ni++) {
            const int cb = wn * (NT * 32) + ni * 32 + 4 * fc;       // + 8i: the lane's 4 columns
            float bv[16], ws[16];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const U4 b4 = ld_lds16(col_bias + cb + 8 * i);
                bv[4 * i] = __uint_as_float(b4.x);
                bv[4 * i + 1] = __uint_as_float(b4.y);
                bv[4 * i + 2] = __uint_as_float(b4.z);
                bv[4 * i + 3] = __uint_as_float(b4.w);
            }
            if (scaled) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const U4 w4 = ld_lds16(col_scale + cb + 8 * i);
                    ws[4 * i] = __uint_as_float(w4.x);
                    ws[4 * i + 1] = __uint_as_float(w4.y);
                    ws[4 * i + 2] = __uint_as_float(w4.z);
                    ws[4 * i + 3] = __uint_as_float(w4.w);
                }
            }
#pragma unroll
            for (int mh = 0; mh < MT_PASS; mh++) {
                const int mi = pass * MT_PASS + mh;
                const int srow = wm * WROWS + mh * 32 + fr;            // staged row
                float v[16];
#pragma unroll
                for (int r = 0; r < 16; r++) v[r] = acc[mi][ni][r];
                if (scaled) {
                    const float as = row_scale[wm * (MT * 32) + mi * 32 + fr];
#pragma unroll
                    for (int r = 0; r < 16; r++) v[r] = v[r] * as * ws[r];
                }
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const uint32_t lo = pack_bf16(v[4 * i] + bv[4 * i], v[4 * i + 1] + bv[4 * i + 1]);
                    const uint32_t hi = pack_bf16(v[4 * i + 2] + bv[4 * i + 2], v[4 * i + 3] + bv[4 * i + 3]);
                    *reinterpret_cast<uint2 *>(Cs + srow * (LDC_S * 2) + (cb + 8 * i) * 2) = make_uint2(lo, hi);
                }
            }
        }
        __syncthreads();
        // read-out, part by part: the 32 groups of 16 lanes take staged rows
        // g16, g16 + 32, ..., so that each lane's row offset is fixed and the
        // part, the rest of the row and the LDS offset are known at compile time
        constexpr int RGROUPS = THREADS / 16, RITERS = RPP / RGROUPS;
        static_assert(RPP % RGROUPS == 0 && WROWS % RGROUPS == 0, "whole read-out iterations");
        const uint8_t *cs_lane = Cs + g16 * (LDC_S * 2) + l16 * 16;
#pragma unroll
        for (int q = 0; q < PARTS; q++) {
#pragma unroll
            for (int it = 0; it < RITERS; it++) {
                // staged row g16 + 32 it is tile row r0 + g16
                const int r0 = (it * RGROUPS / WROWS) * (MT * 32) + pass * WROWS + (it * RGROUPS) % WROWS;
                const U4 v = ld_lds16(cs_lane + it * RGROUPS * (LDC_S * 2) + q * 256);
                const int row = r0 + g16;
                const bool ok = row < rows_in;
                if (ok && part_in[q]) st_global16(o_lane + (int64_t)r0 * p.ldo + q * 128, v);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                const float ss = group_sum<16>(sumsq_bf16_words<8>(w, 0.0f));
                if (part_seg[q] >= 0 && ok && l16 == 0)
                    (part_seg[q] ? sq_k : sq_q)[(int64_t)row * p.parts + part_idx[q]] = ss;
            }
        }
    }
}

}  // namespace

hipError_t proj_launch(ProjParams &p, bool fp8, hipStream_t stream) {
    // bf16 and FP8 ROW_MX operands: 256 x 384 tiles; MXFP8 (whose block scales
    // also take LDS): 256 x 256
    const int bn = (fp8 && p.a_bs) ? 256 : 384;
    p.tiles_m = (uint32_t)((p.m + BM - 1) / BM);
    p.tiles_n = (uint32_t)((p.n + bn - 1) / bn);
    const uint64_t tiles = (uint64_t)p.tiles_m * p.tiles_n;
    if (tiles == 0) return hipSuccess;
    const uint64_t grid = (tiles + 7) / 8 * 8;          // a whole number of tiles per XCD
    if (fp8 && p.a_bs)
        hipLaunchKernelGGL((qkv_proj_kernel<true, true, 256>), dim3((uint32_t)grid), dim3(THREADS), 0, stream, p);
    else if (fp8)
        hipLaunchKernelGGL((qkv_proj_kernel<true, false, 384>), dim3((uint32_t)grid), dim3(THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((qkv_proj_kernel<false, false, 384>), dim3((uint32_t)grid), dim3(THREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace qknr
