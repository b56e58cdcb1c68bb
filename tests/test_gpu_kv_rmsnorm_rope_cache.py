"""GPU parity of qknr_kv_rmsnorm_rope_cache against the fp64 oracle.

Cases: the three MLA workloads at their full sizes (V1 prefill into bf16 paged
caches with k_rope/c_kv; V1 decode into int8 / fp8-e4m3fn Norm caches of 8192
rows, plus the same with k scales large enough to exercise rounding and
clamping; V2 split mode with asymmetric int8 per-head parameters, with and
without k_rope/c_kv) and variants at reduced size: index -1 entries, several
tokens per batch in a Norm cache, fp16 inputs, fp8 ckv in V2, scalar and
[1, D] scale shapes, S-axis broadcast of cos/sin, the 8-byte access path, and
determinism; FP8 E5M2 caches (with and without saturation) and PA_BLK_BNSD
block-start indexing (full V1 prefill size; ragged runs; starts off block
boundaries; runs marked -1); quantised rows where a wavefront's rows share one
head (parameters staged per wave) and where they straddle two heads. Untouched
cache rows must keep their pre-filled bytes exactly.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import check_kv, run_gpu_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import qk_rmsnorm_rope_amd as lib
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


def test_mla_v1_prefill_full(Q):
    d = W.make_kv_cache(W.MLA_V1_PREFILL, device="cuda")
    rep, _ = check_kv(Q, d, "v1-prefill")
    print(rep)


def test_mla_v1_prefill_pa_blk_full(Q):
    """The V1 prefill workload with block-start indexing: 256 runs of 128 tokens."""
    d = W.make_kv_cache(W.MLA_V1_PREFILL, device="cuda", cache_mode=W.PA_BLK_BNSD)
    assert d["index"].numel() == 8 * 32
    rep, _ = check_kv(Q, d, "v1-prefill-pablk")
    print(rep)


def test_e5m2_saturation_exercised(Q):
    """Scales of 1e4..5e4 push |t| past 57344: saturated codes must match."""
    cfg, over = VARIANTS["v1_e5m2_saturating"]
    d = W.make_kv_cache(cfg, device="cuda", **over)
    rep, r = check_kv(Q, d, "e5m2-sat")
    assert (np.abs(r["c_t"]) > 57344).any() and (np.abs(r["k_t"]) > 57344).any()
    print(rep)


def test_mla_v1_decode_quant_full(Q):
    d = W.make_kv_cache(W.MLA_V1_DECODE_QUANT, device="cuda")
    rep, r = check_kv(Q, d, "v1-decode", big_cache=True)
    print(rep)


def test_mla_v1_decode_quant_large_k_scale(Q):
    """k scale ~U(20, 100): k codes span the int8 range and clamp."""
    d = W.make_kv_cache(W.MLA_V1_DECODE_QUANT, device="cuda", k_scale=(20.0, 100.0, "D"))
    rep, r = check_kv(Q, d, "v1-decode-bigscale", big_cache=True)
    codes = np.rint(np.clip(r["k_t"], -128, 127))
    assert (np.abs(codes) == 127).sum() + (codes == -128).sum() > 0, "clamping not exercised"
    assert len(np.unique(codes)) > 100
    print(rep)


@pytest.mark.parametrize("out_kv", [False, True])
def test_mla_v2_split_full(Q, out_kv):
    d = W.make_kv_cache(W.MLA_V2_SPLIT, device="cuda", is_output_kv=out_kv)
    rep, _ = check_kv(Q, d, f"v2-split-outkv{int(out_kv)}")
    print(rep)


VARIANTS = {
    "v1_pa_invalid_index": (W.MLA_V1_PREFILL, dict(seq=300, block_num=24, invalid_every=7)),
    "v1_norm_multi_token": (W.MLA_V1_DECODE_QUANT, dict(batch=5, seq=37, cache_rows=64, index_kind="perm",
                                                        rope_pos="seq", invalid_every=11)),
    "v1_norm_bf16_caches": (W.MLA_V1_DECODE_QUANT, dict(batch=9, seq=3, cache_rows=16, index_kind="perm",
                                                        k_cache_dtype=torch.bfloat16,
                                                        ckv_cache_dtype=torch.bfloat16, k_scale=None,
                                                        v_scale=None, rope_pos="seq")),
    "v1_fp16": (W.MLA_V1_PREFILL, dict(seq=130, block_num=12, dtype=torch.float16,
                                       k_cache_dtype=torch.float16, ckv_cache_dtype=torch.float16)),
    "v1_scalar_scale_pa": (W.MLA_V1_PREFILL, dict(seq=96, block_num=8, k_cache_dtype=torch.int8,
                                                  ckv_cache_dtype=torch.int8, k_scale=(20.0, 40.0, "1"),
                                                  v_scale=(20.0, 40.0, "1D"), is_output_kv=True)),
    "v1_e4m3_both": (W.MLA_V1_PREFILL, dict(seq=64, block_num=8, k_cache_dtype=torch.float8_e4m3fn,
                                            ckv_cache_dtype=torch.float8_e4m3fn, k_scale=(50.0, 400.0, "D"),
                                            v_scale=(0.5, 2.0, "D"))),
    "v2_e4m3_ckv": (W.MLA_V2_SPLIT, dict(batch=2, seq=256, block_num=8, ckv_cache_dtype=torch.float8_e4m3fn,
                                         v_offset=None, v_scale=(1.0, 8.0, "ND"), is_output_kv=True)),
    "v2_bf16_caches_n4": (W.MLA_V2_SPLIT, dict(batch=3, heads=4, seq=100, block_num=8,
                                               k_cache_dtype=torch.bfloat16, ckv_cache_dtype=torch.bfloat16,
                                               k_scale=None, k_offset=None, v_scale=None, v_offset=None,
                                               is_output_kv=True)),
    "v2_norm_quant_outkv": (W.MLA_V2_SPLIT, dict(batch=2, heads=2, seq=40, cache_mode=W.NORM, cache_rows=64,
                                                 is_output_kv=True, invalid_every=5)),
    "v2_symmetric_n1": (W.MLA_V2_SPLIT, dict(batch=4, heads=1, seq=128, block_num=8, k_offset=None,
                                             v_offset=None)),
    "v1_e5m2_norm": (W.MLA_V1_DECODE_QUANT, dict(batch=9, seq=3, cache_rows=16, index_kind="perm",
                                                 k_cache_dtype=torch.float8_e5m2,
                                                 ckv_cache_dtype=torch.float8_e5m2, k_scale=(20.0, 100.0, "D"),
                                                 rope_pos="seq")),
    "v1_e5m2_saturating": (W.MLA_V1_PREFILL, dict(seq=64, block_num=8, k_cache_dtype=torch.float8_e5m2,
                                                  ckv_cache_dtype=torch.float8_e5m2, k_scale=(1e4, 5e4, "D"),
                                                  v_scale=(1e4, 5e4, "1D"))),
    "v1_pablk_ragged": (W.MLA_V1_PREFILL, dict(cache_mode=W.PA_BLK_BNSD, seq=300, block_num=24,
                                               invalid_every=5)),
    "v1_pablk_unaligned_int8": (W.MLA_V1_PREFILL, dict(cache_mode=W.PA_BLK_BNSD, batch=3, seq=200, block_num=16,
                                                       index_kind="blocks_unaligned", k_cache_dtype=torch.int8,
                                                       ckv_cache_dtype=torch.int8, k_scale=(20.0, 40.0, "D"),
                                                       v_scale=(20.0, 40.0, "D"))),
    "v2_pablk_unaligned_e5m2": (W.MLA_V2_SPLIT, dict(cache_mode=W.PA_BLK_BNSD, batch=2, seq=200, block_num=16,
                                                     index_kind="blocks_unaligned",
                                                     ckv_cache_dtype=torch.float8_e5m2, v_offset=None,
                                                     v_scale=(1.0, 8.0, "ND"), is_output_kv=True)),
    # 8 rows per wavefront (16496 rows) with S = 1031: waves that straddle two
    # heads load their per-head parameters per lane, the others share them
    "v2_waves_straddle_heads": (W.MLA_V2_SPLIT, dict(batch=2, heads=8, seq=1031, block_num=20, is_output_kv=True)),
    # V1 with per-channel int8 parameters at 16800 rows: several rows per wave
    "v1_channel_int8_many_rows": (W.MLA_V1_PREFILL, dict(batch=8, seq=2100, block_num=140, k_cache_dtype=torch.int8,
                                                         ckv_cache_dtype=torch.int8, k_scale=(20.0, 40.0, "D"),
                                                         v_scale=(20.0, 40.0, "1D"))),
    # two rows per lane in part B (>= 32768 rows at 8 lanes per row): V2 with waves that
    # straddle two heads (S = 2061), V1 with int8 / FP8 caches
    "v2_two_rows_per_lane_straddle": (W.MLA_V2_SPLIT, dict(batch=2, heads=8, seq=2061, block_num=40,
                                                           is_output_kv=True)),
    "v1_quant_two_rows_per_lane": (W.MLA_V1_PREFILL, dict(batch=8, seq=4100, block_num=260,
                                                          k_cache_dtype=torch.int8,
                                                          ckv_cache_dtype=torch.float8_e4m3fn,
                                                          k_scale=(20.0, 40.0, "D"), v_scale=(1.0, 8.0, "1D"))),
    # FP8 codes staged per wave (16384 rows, 8 per wavefront): E5M2 in V2, E4M3FN in V1
    "v2_e5m2_both_staged": (W.MLA_V2_SPLIT, dict(batch=2, heads=8, seq=1024, block_num=16,
                                                 k_cache_dtype=torch.float8_e5m2, ckv_cache_dtype=torch.float8_e5m2,
                                                 k_scale=(1.0, 8.0, "ND"), v_scale=(1.0, 8.0, "ND"),
                                                 v_offset=None)),
    "v1_e4m3_both_many_rows": (W.MLA_V1_PREFILL, dict(batch=8, seq=2048, block_num=128,
                                                      k_cache_dtype=torch.float8_e4m3fn,
                                                      ckv_cache_dtype=torch.float8_e4m3fn, k_scale=(1.0, 8.0, "D"),
                                                      v_scale=(1.0, 8.0, "1D"))),
    "v2_pablk_bf16_n2": (W.MLA_V2_SPLIT, dict(cache_mode=W.PA_BLK_BNSD, batch=3, heads=2, seq=129, block_num=12,
                                              k_cache_dtype=torch.bfloat16, ckv_cache_dtype=torch.bfloat16,
                                              k_scale=None, k_offset=None, v_scale=None, v_offset=None,
                                              invalid_every=4)),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variants(Q, name):
    cfg, over = VARIANTS[name]
    d = W.make_kv_cache(cfg, device="cuda", **over)
    rep, _ = check_kv(Q, d, name)
    print(name, rep)


def test_pa_blk_run_past_the_cache_end(Q):
    """A run that starts 3 slots before the end of the cache writes 3 rows; the
    other 125 tokens of the run write nothing."""
    d = W.make_kv_cache(W.MLA_V1_PREFILL, device="cuda", cache_mode=W.PA_BLK_BNSD, batch=2, seq=256, block_num=8)
    d["index"].copy_(torch.tensor([0, 256, 512, 8 * 128 - 3], dtype=torch.int64))
    rep, _ = check_kv(Q, d, "pablk-past-end")
    print(rep)


def test_s_axis_broadcast_cos_sin(Q):
    """cos/sin [B, N, 1, rope] shared by every position (Norm cache)."""
    d = W.make_kv_cache(W.MLA_V1_DECODE_QUANT, device="cuda", batch=4, seq=20, cache_rows=32,
                        index_kind="perm", rope_pos="seq")
    d["cos"] = d["cos"][:, :, 5:6].contiguous()
    d["sin"] = d["sin"][:, :, 5:6].contiguous()
    rep, _ = check_kv(Q, d, "s-broadcast")
    print(rep)


def test_narrow_access_path(Q):
    """rms_size 12 (not a multiple of 8): the 4-element (8-byte) path."""
    d = W.make_kv_cache(W.MLA_V1_PREFILL, device="cuda", seq=64, block_num=8, kv_dim=12 + 16, rms_size=12,
                        rope_size=16, is_output_kv=True)
    rep, _ = check_kv(Q, d, "narrow")
    print(rep)


def test_deterministic(Q):
    d1 = W.make_kv_cache(W.MLA_V2_SPLIT, device="cuda", batch=2, seq=512, block_num=16)
    d2 = W.make_kv_cache(W.MLA_V2_SPLIT, device="cuda", batch=2, seq=512, block_num=16)
    run_gpu_kv(Q, d1)
    run_gpu_kv(Q, d2)
    torch.cuda.synchronize()
    assert torch.equal(d1["k_cache"], d2["k_cache"]) and torch.equal(d1["ckv_cache"], d2["ckv_cache"])


def test_prepared_call_matches_direct_call(Q):
    """The prepared launcher (arguments marshalled once) writes what a direct call writes."""
    d1 = W.make_kv_cache(W.MLA_V1_PREFILL, device="cuda", seq=256, block_num=16)
    d2 = W.make_kv_cache(W.MLA_V1_PREFILL, device="cuda", seq=256, block_num=16)
    run_gpu_kv(Q, d1)
    cfg = d2["cfg"]
    launch = Q.prepare_kv_rmsnorm_rope_cache(d2["kv"], d2["gamma"], d2["cos"], d2["sin"], d2["index"],
                                             d2["k_cache"], d2["ckv_cache"], cache_mode="PA_BNSD",
                                             epsilon=cfg.eps, is_output_kv=True, k_rope=d2["k_rope"],
                                             c_kv=d2["c_kv"])
    launch()
    launch()                                         # idempotent: same inputs, same slots
    torch.cuda.synchronize()
    for key in ("k_cache", "ckv_cache", "k_rope", "c_kv"):
        assert torch.equal(d1[key].view(torch.int16), d2[key].view(torch.int16)), key
