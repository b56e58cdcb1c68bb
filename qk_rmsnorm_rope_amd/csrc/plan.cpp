// plan.cpp -- host-only launch planning for the two operators: the lane
// geometry of the QK kernel and of the KV kernel (groups of lanes per row,
// register slots, rows per lane, per-wave LDS staging), and the dispatch from
// a plan to the kernel instantiations in the .hip units. No device code: the
// host layer (api.cpp and this file) also builds with a plain host compiler,
// for the sanitizer run of the tests.
#include "launch.h"

namespace qknr {

// ---------------------------------------------------------------------------
// (a) QK RMSNorm + rotate-half RoPE
// ---------------------------------------------------------------------------

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

hipError_t qk_launch(QkParams &p, int elem_type, int vec, int mode, hipStream_t stream) {
    const int J = qk_plan(p, vec);
    if (J < 0) return hipErrorInvalidValue;
    if (p.tokens == 0) return hipSuccess;
    switch (mode) {
    case QK_ACROSS: return qk_launch_across(p, elem_type, vec, J, stream);
    case QK_PER_HEAD: return qk_launch_per_head(p, elem_type, vec, J, stream);
    case QK_SUMSQ:
    case QK_APPLY: return qk_launch_split(p, elem_type, vec, J, mode, stream);
    }
    return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------
// (b) KvRmsNormRopeCache
// ---------------------------------------------------------------------------

static int round_slots(int c, const int *allowed, int n_allowed) {
    for (int i = 0; i < n_allowed; i++)
        if (c <= allowed[i]) return allowed[i];
    return -1;
}

static const int kCA[] = {1, 2, 3, 4};
static const int kCB[] = {1, 2};

// Lane-group size of one part: the smallest G whose register slots hold the
// part (fewest lanes per row, most rows per wave), unless that leaves fewer
// than 2048 wavefronts (two per SIMD on 256 CUs); then larger groups spread few
// rows over more waves (a decode batch of 512 rows runs on 512 waves at G = 64).
static int pick_group(uint32_t rows, int chunks, const int *allowed, int n_allowed, int min_g, int &slots) {
    int found = -1;
    for (int G = 8; G <= 64; G *= 2) {
        if (G < min_g) continue;
        const int k = round_slots((chunks + G - 1) / G, allowed, n_allowed);
        if (k > 0) {
            found = G;
            slots = k;
            if ((uint64_t)rows * (uint64_t)G >= 2048ull * 64ull) break;
        }
    }
    return found;
}

int kv_plan(KvParams &p, int vec, bool v2, int &ca, int &cb) {
    p.nr = p.rms_size / vec;
    p.nx = (v2 ? p.c_dim : p.rope_size) / vec;
    p.n_rope_chunks = v2 ? p.rope_size / vec : 0;
    // V2: rotated chunks 0..n_rope_chunks-1 must all sit in slot 0 (G >= their count)
    const int ga = pick_group(p.rows, p.nr, kCA, 4, v2 ? p.n_rope_chunks : 8, ca);
    const int gb = pick_group(p.rows, p.nx, kCB, 2, 8, cb);
    if (ga < 0 || gb < 0) return -1;
    p.ga = ga;
    p.gb = gb;
    p.ga_shift = __builtin_ctz((unsigned)ga);
    p.gb_shift = __builtin_ctz((unsigned)gb);
    // part B: two rows per lane (both rows' loads issued before either is
    // used) when the part keeps at least 2048 waves that way; its short rows
    // are latency-bound with one (16-byte chunks only; not for V1's two-chunk
    // rope tails, whose coefficients would not fit)
    p.rb = (vec == 8 && (v2 || cb == 1) && (uint64_t)p.rows * (uint64_t)gb >= 2ull * 2048ull * 64ull) ? 2 : 1;
    // part A: two rows per lane as well in V1 (at four waves per SIMD: its rows
    // of 512 normed values hold more registers); V2's part A measured no faster
    p.ra = (!v2 && p.rb == 2 && (uint64_t)p.rows * (uint64_t)ga >= 2ull * 2048ull * 64ull) ? 2 : 1;
    // per-wave LDS: staged quantisation parameters (2*width floats of the
    // widest quantised cache with per-channel parameters that fits 2 KB), then
    // staged codes (the rows of a wave, for rows whose width in bytes is a
    // multiple of 16)
    {
        int w = 0;
        if (p.k_code != CODE_SAME && p.k_qshape != QS_SCALAR && 2 * p.k_dim <= kWaveParamFloats) w = p.k_dim;
        if (p.c_code != CODE_SAME && p.v_qshape != QS_SCALAR && 2 * p.c_dim <= kWaveParamFloats && p.c_dim > w)
            w = p.c_dim;
        p.lds_param_bytes = 8 * w;
        // part A writes the k cache (V2) or the ckv cache (V1); part B the other
        // Staged rows leave as 16-byte stores at the row's own address, so the
        // cache base and its strides (bytes; quantised elements are one byte)
        // must be multiples of 16; other layouts keep the lanes' own stores.
        const auto lines16 = [](const void *base, uint32_t s0, uint32_t s1, uint32_t s2) {
            return (reinterpret_cast<uintptr_t>(base) & 15u) == 0 && (s0 & 15u) == 0 && (s1 & 15u) == 0 &&
                   (s2 & 15u) == 0;
        };
        const bool k16 = lines16(p.k_cache, p.kc0, p.kc1, p.kc2), c16 = lines16(p.ckv_cache, p.cc0, p.cc1, p.cc2);
        const int wa = v2 ? p.k_dim : p.c_dim, ca_code = v2 ? p.k_code : p.c_code;
        const int wb = v2 ? p.c_dim : p.k_dim, cb_code = v2 ? p.c_code : p.k_code;
        const bool a16 = v2 ? k16 : c16, b16 = v2 ? c16 : k16;
        const int need_a = p.ra * (64 / ga) * wa, need_b = p.rb * (64 / gb) * wb;
        // wider staged rows than 2 KB per wave fall back to direct stores
        p.stage_a = ca_code != CODE_SAME && ga < 64 && wa % 16 == 0 && a16 && need_a <= 2048;
        p.stage_b = cb_code != CODE_SAME && gb < 64 && wb % 16 == 0 && b16 && need_b <= 2048;
        int cbytes = 0;
        if (p.stage_a) cbytes = need_a;
        if (p.stage_b && need_b > cbytes) cbytes = need_b;
        p.lds_code_bytes = cbytes;
        p.lds_wave_bytes = p.lds_param_bytes + p.lds_code_bytes;
    }
    p.blocks_a = (p.rows + (p.ra * 256 / ga) - 1) / (p.ra * 256 / ga);
    p.blocks_b = (p.rows + (p.rb * 256 / gb) - 1) / (p.rb * 256 / gb);
    if ((uint64_t)p.blocks_a + p.blocks_b >= (1ull << 31)) return -1;
    return 0;
}

hipError_t kv_launch(KvParams &p, int elem_type, int vec, bool v2, hipStream_t stream) {
    int ca = 0, cb = 0;
    if (kv_plan(p, vec, v2, ca, cb) != 0) return hipErrorInvalidValue;
    if (p.rows == 0) return hipSuccess;
    if (elem_type == 1) return kv_launch_bf16(p, vec, v2, ca, cb, stream);
    if (elem_type == 2) return kv_launch_f16(p, vec, v2, ca, cb, stream);
    return hipErrorInvalidValue;
}

}  // namespace qknr
