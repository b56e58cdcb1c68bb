"""Seeded input generators: determinism, shapes, and the algorithmic byte
counts each workload's roofline is priced on (CPU only)."""
import torch

import workloads as W


def test_wan_latent_grid():
    grid, s = W.math_check()
    assert grid == (21, 45, 80) and s == 75600 == W.WAN22_SELF_ATTN.seq


def test_across_heads_inputs_deterministic_and_shaped():
    a = W.make_across_heads(W.TINY_ACROSS_HEADS)
    b = W.make_across_heads(W.TINY_ACROSS_HEADS)
    assert torch.equal(a["qkv"], b["qkv"]) and torch.equal(a["cos"], b["cos"])
    assert a["qkv"].shape == (1, 64, 512) and a["qkv"].dtype == torch.float32
    assert a["cos"].shape == (1, 64, 64)
    g = a["q_gamma"]
    assert g.shape == (256,) and float(g.min()) >= 0.5 and float(g.max()) <= 1.5
    # rotate-half layout: lanes i and i+d/2 share the angle
    assert torch.equal(a["cos"][..., :32], a["cos"][..., 32:])


def test_wan_table_small_grid():
    c, s = W.wan_3d_table(2, 3, 4, d=128)
    assert c.shape == (24, 128)
    # token 0 sits at (0,0,0): every angle is 0
    assert torch.all(c[0] == 1) and torch.all(s[0] == 0)
    # token 1 is (t=0, h=0, w=1): only the w pairs (last 21 of 64) rotate
    assert torch.all(s[1, :43] == 0) and torch.all(s[1, 43:64] != 0)
    # token 4 is (0, 1, 0): only the h pairs rotate
    assert torch.all(s[4, :22] == 0) and torch.all(s[4, 22:43] != 0) and torch.all(s[4, 43:64] == 0)


def test_kv_inputs_shapes_and_index():
    d = W.make_kv_cache(W.MLA_V1_PREFILL, seq=256, block_num=20)
    assert d["kv"].shape == (8, 1, 256, 576)
    assert d["k_cache"].shape == (20, 128, 1, 64) and d["ckv_cache"].shape == (20, 128, 1, 512)
    idx = d["index"]
    assert idx.shape == (2048,) and len(set(idx.tolist())) == 2048 and int(idx.max()) < 2560
    d4 = W.make_kv_cache(W.MLA_V1_DECODE_QUANT, batch=16, cache_rows=64)
    assert d4["index"].shape == (16, 1) and len(set(d4["index"].ravel().tolist())) == 16
    assert d4["k_cache"].dtype == torch.int8 and d4["ckv_cache"].dtype == torch.float8_e4m3fn
    assert d4["k_scale"].shape == (64,) and d4["v_scale"].shape == (512,)
    d5 = W.make_kv_cache(W.MLA_V2_SPLIT, batch=2, seq=256, block_num=8)
    assert d5["v"].shape == (2, 8, 256, 128) and d5["k_scale"].shape == (8, 192)
    assert d5["k_cache"].shape == (8, 128, 8, 192)


def test_algorithmic_bytes_match_the_roofline_tables():
    assert W.algorithmic_bytes_across_heads(W.WAN22_SELF_ATTN) == 3_135_303_680
    assert W.algorithmic_bytes_across_heads(W.TINY_ACROSS_HEADS) == 4 * (64 * (2 * 512 + 128) + 512)
    assert W.algorithmic_bytes_kv_cache(W.MLA_V1_PREFILL) == 121_897_984
    assert W.algorithmic_bytes_kv_cache(W.MLA_V1_DECODE_QUANT) == 1_023_232
    assert W.algorithmic_bytes_kv_cache(W.MLA_V2_SPLIT) == 319_050_112
