"""HIP-graph capture of the library's launches.

Each case captures prepared launches (arguments marshalled once) into one
graph, then replays it several times; between replays the test writes new
input values with ordinary eager copies and synchronises. Every replay must
write exactly what the same launches write eagerly on a second set of buffers
holding the same inputs (same kernels, so the bytes must be identical). The
cases cover the KV operator's decode shape (one row per wavefront), its V2
shape with several rows per wavefront (the per-wave LDS staging, whose size
is part of the captured launch), the across-heads operator, and the
projection followed by the apply pass (two kernels in one graph).
"""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def Q():
    import qk_rmsnorm_rope_amd as lib
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


def _capture(make):
    """Warm up on a side stream, then capture `make(stream)()` into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    side = make(s)
    side()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        make(torch.cuda.current_stream())()
    torch.cuda.synchronize()
    return g


def _clone(d):
    return {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _kv_make(Q, d):
    cfg = d["cfg"]
    mode = {W.NORM: "Norm", W.PA_BNSD: "PA_BNSD", W.PA_BLK_BNSD: "PA_BLK_BNSD"}[cfg.cache_mode]

    def make(stream=None):
        return Q.prepare_kv_rmsnorm_rope_cache(
            d["kv"], d["gamma"], d["cos"], d["sin"], d["index"], d["k_cache"], d["ckv_cache"],
            k_rope_scale=d["k_scale"], k_rope_offset=d["k_offset"], c_kv_scale=d["v_scale"],
            c_kv_offset=d["v_offset"], v=d["v"], epsilon=cfg.eps, cache_mode=mode,
            is_output_kv=cfg.is_output_kv, k_rope=d["k_rope"], c_kv=d["c_kv"], stream=stream)
    return make


def _same(a, b, what):
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), what


def _kv_case(Q, cfg, over, new_index):
    g_d = W.make_kv_cache(cfg, device="cuda", **over)
    e_d = _clone(g_d)
    graph = _capture(_kv_make(Q, g_d))   # the warm-up wrote g_d's outputs once
    eager = _kv_make(Q, e_d)()
    eager()                               # the same first write on e_d
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(77)
    for r in range(REPLAYS):
        kv = torch.randn(g_d["kv"].shape, generator=gen, device="cuda").to(g_d["kv"].dtype)
        g_d["kv"].copy_(kv)
        e_d["kv"].copy_(kv)
        if g_d["v"] is not None:
            v = torch.randn(g_d["v"].shape, generator=gen, device="cuda").to(g_d["v"].dtype)
            g_d["v"].copy_(v)
            e_d["v"].copy_(v)
        idx = new_index(r).reshape(g_d["index"].shape)
        g_d["index"].copy_(idx)
        e_d["index"].copy_(idx)
        torch.cuda.synchronize()
        graph.replay()
        eager()
        torch.cuda.synchronize()
        for name in ("k_cache", "ckv_cache", "k_rope", "c_kv"):
            if g_d.get(name) is not None:
                _same(g_d[name], e_d[name], f"replay {r}: {name}")


def test_kv_decode_graph_replays(Q):
    """V1 decode into int8 / FP8 Norm caches, a new index (distinct rows) per replay."""
    over = dict(batch=64, cache_rows=256)
    gen = torch.Generator().manual_seed(5)

    def new_index(r):
        return torch.randperm(256, generator=gen)[:64].to("cuda")
    _kv_case(Q, W.MLA_V1_DECODE_QUANT, over, new_index)


def test_kv_v2_staged_graph_replays(Q):
    """V2 split with 16496 rows (8 rows per wavefront: parameters and codes
    staged in LDS) into int8 paged caches, with k_rope / c_kv."""
    over = dict(batch=2, heads=8, seq=1031, block_num=20, is_output_kv=True)
    gen = torch.Generator().manual_seed(6)

    def new_index(r):
        return torch.randperm(20 * 128, generator=gen)[:2 * 1031].to("cuda")
    _kv_case(Q, W.MLA_V2_SPLIT, over, new_index)


def test_across_heads_graph_replays(Q):
    """Across-heads norm + RoPE, Wan2.2 width, 300 tokens, out of place."""
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=300)
    qkv = d["qkv"]
    nq, nk, hd = 40, 40, 128
    q = qkv[..., : nq * hd].unflatten(-1, (nq, hd))
    k = qkv[..., nq * hd: (nq + nk) * hd].unflatten(-1, (nk, hd))
    outs = {w: torch.zeros_like(qkv) for w in ("graph", "eager")}

    def make_for(which):
        o = outs[which]
        qo = o[..., : nq * hd].unflatten(-1, (nq, hd))
        ko = o[..., nq * hd: (nq + nk) * hd].unflatten(-1, (nk, hd))

        def make(stream=None):
            return Q.prepare_qk_norm_rope_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"],
                                                       eps=d["eps"], q_out=qo, k_out=ko,
                                                       stream=stream)
        return make
    graph = _capture(make_for("graph"))
    eager = make_for("eager")()
    gen = torch.Generator(device="cuda").manual_seed(8)
    for r in range(REPLAYS):
        qkv.copy_(torch.randn(qkv.shape, generator=gen, device="cuda").to(qkv.dtype))
        torch.cuda.synchronize()
        graph.replay()
        eager()
        torch.cuda.synchronize()
        _same(outs["graph"], outs["eager"], f"replay {r}")


@pytest.mark.parametrize("operands", ["bf16", "fp8", "mxfp8"])
def test_projection_then_apply_graph_replays(Q, operands):
    """QKV projection with sums, then the apply pass, captured as one graph
    (Wan2.2 width, 300 tokens); bf16 operands, FP8 with row / channel scales
    (a kernel that spills two registers per lane to the private segment,
    which every replay needs too) and MXFP8 with block scales."""
    cfg = {"bf16": W.WAN22_QKV_PROJ, "fp8": W.WAN22_QKV_PROJ_FP8, "mxfp8": W.WAN22_QKV_PROJ_MXFP8}[operands]
    d = W.make_qkv_projection(cfg, device="cuda", seq=300)
    S, nq, nk, hd = 300, 40, 40, 128
    bufs = {w: (torch.zeros(S, d["out_features"], dtype=torch.bfloat16, device="cuda"),
                torch.zeros(2, S, 40, dtype=torch.float32, device="cuda")) for w in ("graph", "eager")}

    def make_for(which):
        out, sums = bufs[which]
        q = out[:, : nq * hd].unflatten(-1, (nq, hd)).unsqueeze(0)
        k = out[:, nq * hd: (nq + nk) * hd].unflatten(-1, (nk, hd)).unsqueeze(0)

        def make(stream=None):
            if operands == "fp8":
                proj = Q.prepare_qkv_projection(d["a8"], d["w8"], d["bias"], out=out, q_cols=5120, k_cols=5120,
                                                sumsq=sums, a_scale=d["a_scale"], w_scale=d["w_scale"],
                                                stream=stream)
            elif operands == "mxfp8":
                proj = Q.prepare_qkv_projection(d["a8"], d["w8"], d["bias"], out=out, q_cols=5120, k_cols=5120,
                                                sumsq=sums, a_block_scale=d["a_bs"], w_block_scale=d["w_bs"],
                                                stream=stream)
            else:
                proj = Q.prepare_qkv_projection(d["a"], d["w"], d["bias"], out=out, q_cols=5120, k_cols=5120,
                                                sumsq=sums, stream=stream)
            apply = Q.prepare_qk_apply_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], sums,
                                                    eps=d["eps"], q_norm_channels=0, stream=stream)

            def both():
                proj()
                apply()
            return both
        return make
    graph = _capture(make_for("graph"))
    eager = make_for("eager")()
    gen = torch.Generator(device="cuda").manual_seed(9)
    for r in range(REPLAYS):
        if operands != "bf16":    # new codes and row scales, written eagerly (rows rotated)
            codes = d["a8"].view(torch.uint8)
            codes.copy_(codes.roll(r + 1, 0))
            row_scales = d["a_scale"] if operands == "fp8" else d["a_bs"]
            row_scales.copy_(row_scales.roll(r + 1, 0))
        else:
            d["a"].copy_(torch.randn(d["a"].shape, generator=gen, device="cuda").to(d["a"].dtype))
        torch.cuda.synchronize()
        graph.replay()
        eager()
        torch.cuda.synchronize()
        _same(bufs["graph"][0], bufs["eager"][0], f"replay {r}: out")
        _same(bufs["graph"][1], bufs["eager"][1], f"replay {r}: sums")
