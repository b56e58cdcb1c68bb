// stub_launch.cpp -- launchers for a host-only build of the ABI layer
// (api.cpp + plan.cpp) used by the sanitizer run of the tests: they launch
// nothing and return hipErrorNoDevice, after checking that the plan they were
// given is one the kernels can run (a grid that covers every row exactly,
// lane groups and register slots of the built shapes, per-wave LDS within
// the block's budget, staged code rows only on 16-byte cache layouts).
// A violated invariant aborts, which the sanitizer run reports as a failure.
#include <cstdio>
#include <cstdlib>

#include "launch.h"

namespace {

void require(bool ok, const char *what) {
    if (!ok) {
        std::fprintf(stderr, "plan invariant violated: %s\n", what);
        std::abort();
    }
}

bool pow2_group(int g, int shift) {
    return (g == 8 || g == 16 || g == 32 || g == 64) && (1 << shift) == g;
}

// blocks of rows_per_block cover `rows` with no empty block
void covers(uint32_t blocks, uint32_t rows_per_block, uint32_t rows, const char *what) {
    require(rows_per_block > 0, what);
    require((uint64_t)blocks * rows_per_block >= rows, what);
    require(blocks == 0 || (uint64_t)(blocks - 1) * rows_per_block < rows, what);
}

bool lines16(const void *base, uint32_t s0, uint32_t s1, uint32_t s2) {
    return (reinterpret_cast<uintptr_t>(base) & 15u) == 0 && ((s0 | s1 | s2) & 15u) == 0;
}

void check_kv(const qknr::KvParams &p, int vec, int ca, int cb) {
    require(vec == 8 || vec == 4, "kv: chunk width");
    require(pow2_group(p.ga, p.ga_shift) && pow2_group(p.gb, p.gb_shift), "kv: lane groups");
    require(ca >= 1 && ca <= 4 && cb >= 1 && cb <= 2, "kv: register slots");
    require((int64_t)ca * p.ga >= p.nr && (int64_t)cb * p.gb >= p.nx, "kv: slots hold the row");
    require(p.ra >= 1 && p.ra <= 2 && p.rb >= 1 && p.rb <= 2, "kv: rows per lane");
    covers(p.blocks_a, (uint32_t)(p.ra * 256 / p.ga), p.rows, "kv: part A grid");
    covers(p.blocks_b, (uint32_t)(p.rb * 256 / p.gb), p.rows, "kv: part B grid");
    require(p.lds_wave_bytes == p.lds_param_bytes + p.lds_code_bytes, "kv: LDS regions");
    require(p.lds_param_bytes <= 4 * qknr::kWaveParamFloats && p.lds_code_bytes <= 2048, "kv: LDS per wave");
    require(4 * p.lds_wave_bytes <= 65536, "kv: LDS per block");
    require(p.n_rope_chunks <= p.ga, "kv: V2 rotated chunks sit in slot 0");
    const bool v2 = p.v != nullptr;
    const void *cache_a = v2 ? p.k_cache : p.ckv_cache, *cache_b = v2 ? p.ckv_cache : p.k_cache;
    if (p.stage_a)
        require(lines16(cache_a, v2 ? p.kc0 : p.cc0, v2 ? p.kc1 : p.cc1, v2 ? p.kc2 : p.cc2) &&
                    p.lds_code_bytes >= p.ra * (64 / p.ga) * (v2 ? p.k_dim : p.c_dim),
                "kv: part A staging");
    if (p.stage_b)
        require(lines16(cache_b, v2 ? p.cc0 : p.kc0, v2 ? p.cc1 : p.kc1, v2 ? p.cc2 : p.kc2) &&
                    p.lds_code_bytes >= p.rb * (64 / p.gb) * (v2 ? p.c_dim : p.k_dim),
                "kv: part B staging");
}

void check_qk(const qknr::QkParams &p, int vec, int J) {
    require(J >= 1 && J <= 8, "qk: heads per lane");
    require(p.chunks_per_half * vec == p.half && p.half * 2 == p.head_dim, "qk: chunks of a half head");
    require(p.heads_per_step * p.chunks_per_half <= 64, "qk: one step's lanes");
    require(p.waves_per_unit == 1 || p.waves_per_unit == 2 || p.waves_per_unit == 4, "qk: waves per unit");
    const int heads = p.n_q > p.n_k ? p.n_q : p.n_k;
    require((int64_t)p.heads_per_step * p.waves_per_unit * J >= heads, "qk: every head has a lane");
}

}  // namespace

namespace qknr {

hipError_t qk_launch_across(const QkParams &p, int, int vec, int J, hipStream_t) {
    check_qk(p, vec, J);
    return hipErrorNoDevice;
}
hipError_t qk_launch_per_head(const QkParams &p, int, int vec, int J, hipStream_t) {
    check_qk(p, vec, J);
    return hipErrorNoDevice;
}
hipError_t qk_launch_split(const QkParams &p, int, int vec, int J, int, hipStream_t) {
    check_qk(p, vec, J);
    return hipErrorNoDevice;
}
hipError_t kv_launch_bf16(const KvParams &p, int vec, bool, int ca, int cb, hipStream_t) {
    check_kv(p, vec, ca, cb);
    return hipErrorNoDevice;
}
hipError_t kv_launch_f16(const KvParams &p, int vec, bool, int ca, int cb, hipStream_t) {
    check_kv(p, vec, ca, cb);
    return hipErrorNoDevice;
}
hipError_t permute_launch(const PermuteParams &, int unit, hipStream_t) {
    require(unit == 1 || unit == 2 || unit == 4 || unit == 8 || unit == 16, "permute: access width");
    return hipErrorNoDevice;
}
hipError_t proj_launch(ProjParams &p, bool, hipStream_t) {
    require(p.n % 128 == 0 && p.m >= 1, "projection: tile shape");
    return hipErrorNoDevice;
}

}  // namespace qknr
