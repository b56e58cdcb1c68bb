"""Seeded random shapes for qknr_kv_rmsnorm_rope_cache against the fp64 oracle.

The hand-picked cases elsewhere pin the benchmark workloads and each code path
on purpose; these 40 cases draw the operator's free parameters at random, so
that combinations nobody picked also meet the parity bar: V1 or V2 (N in
{1, 2, 4, 8}), widths (rms 128-512, rope 16-64, v 64-256; V2 kv 64-256),
bf16 or fp16, each cache unquantised, int8 (with or without offsets), FP8
E4M3FN or E5M2 (some with scales that saturate), every parameter shape the
version allows, Norm / PA_BNSD / PA_BLK_BNSD caches with block sizes 32-128,
skipped tokens (index -1), k_rope / c_kv where they take effect, row-padded
inputs and outputs (16- and 8-byte access paths), cache rows padded by 8 or 16
bytes (the padding must stay untouched), cos/sin shared over S, and from one
row to 40,000 rows (so the launch planner's choices -- lanes per row, rows per
lane, staged parameters and codes, waves that straddle heads -- vary too).

Every drawn case is a legal call: the CPU test below checks that host
validation accepts each one (no GPU needed), so the GPU test never skips.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import LIB_MODE, check_kv, padded_cache

N_CASES = 40


def _draw(i):
    """The workload overrides of case i (a base config and keyword overrides)."""
    rng = np.random.default_rng(7000 + i)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    v2 = bool(rng.random() < 0.5)
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float16
    if v2:
        heads = pick([1, 2, 4, 8])
        kv_dim = pick([64, 128, 192, 256])
        rope = pick([r for r in (16, 32, 64) if r <= kv_dim])
        rms, v_dim = kv_dim, pick([64, 128, 256])
        dk, dc = kv_dim, v_dim
    else:
        heads, v_dim = 1, 0
        rms, rope = pick([128, 256, 512]), pick([16, 32, 64])
        kv_dim = rms + rope
        dk, dc = rope, rms

    size = rng.random()
    batch = int(rng.integers(1, 5))
    if size < 0.4:
        seq = int(rng.integers(1, 65))
    elif size < 0.8:
        seq = int(rng.integers(65, 1500))
    else:                                    # 16k-40k rows
        seq = int(rng.integers(16000, 40000)) // (batch * heads) + 1

    def cache(width):
        kind = pick(["same", "same", "int8", "int8", "e4m3", "e5m2"])
        if kind == "same":
            return dtype, None, None
        shape = "ND" if v2 else pick(["1", "D", "1D"])
        if kind == "int8":
            lo, hi = pick([(0.5, 4.0), (20.0, 40.0)])
            offset = (-16.0, 16.0, shape) if rng.random() < 0.5 else None
            return torch.int8, (lo, hi, shape), offset
        if kind == "e4m3":
            lo, hi = pick([(1.0, 8.0), (50.0, 400.0)])
            return torch.float8_e4m3fn, (lo, hi, shape), None
        lo, hi = pick([(1.0, 8.0), (1e4, 5e4)])
        return torch.float8_e5m2, (lo, hi, shape), None

    k_dt, k_scale, k_offset = cache(dk)
    c_dt, v_scale, v_offset = cache(dc)
    quant = k_scale is not None or v_scale is not None

    mode = pick([W.NORM, W.PA_BNSD, W.PA_BLK_BNSD])
    over = dict(batch=batch, heads=heads, seq=seq, kv_dim=kv_dim, rms_size=rms, rope_size=rope, v_dim=v_dim,
                dtype=dtype, cache_mode=mode, k_cache_dtype=k_dt, ckv_cache_dtype=c_dt, k_scale=k_scale,
                k_offset=k_offset, v_scale=v_scale, v_offset=v_offset, rope_pos="seq",
                invalid_every=pick([0, 0, 3, 7, 50]), seed=7000 + i)
    if mode == W.NORM:
        over.update(cache_rows=seq + int(rng.integers(0, 64)), index_kind="perm", block_size=0, block_num=0)
    else:
        bs = pick([32, 64, 128])
        runs = batch * -(-seq // bs)
        if mode == W.PA_BLK_BNSD:
            unaligned = bool(rng.random() < 0.5)
            over.update(index_kind="blocks_unaligned" if unaligned else "perm",
                        block_size=bs, block_num=(2 * runs if unaligned else runs) + int(rng.integers(0, 8)))
        else:
            over.update(index_kind="perm", block_size=bs, block_num=runs + int(rng.integers(0, 8)))
    # k_rope / c_kv take effect for paged caches, and for Norm only in V2 with a quantised cache
    over["is_output_kv"] = bool(rng.random() < 0.5) and (mode != W.NORM or (v2 and quant))
    base = W.MLA_V2_SPLIT if v2 else W.MLA_V1_PREFILL
    # layout of the inputs and raw outputs: rows padded by 8 elements (16-byte accesses
    # stay legal) or by 4 (the 8-byte access path), and one cos/sin row shared by every
    # position (allowed for Norm caches and unquantised paged caches)
    lay = dict(pad=pick([0, 0, 8, 4]), out_pad=pick([0, 0, 8]),
               s_bcast=bool(rng.random() < 0.2) and (mode == W.NORM or not quant) and seq > 1,
               s_pos=int(rng.integers(0, seq)))
    # cache rows padded by 8 bytes (quantised rows then leave by the lanes' own
    # stores: staged 16-byte pieces need 16-byte rows) or by 16 (staging stays on)
    lay["cache_pad"] = pick([0, 0, 0, 8, 16])
    return base, over, lay


def _relayout(d, lay):
    """The same values in the drawn layout: kv and v as views into row-padded
    buffers, cos/sin of one position broadcast over S, k_rope / c_kv as views
    into row-padded outputs."""
    def padded(t, pad):
        if t is None or not pad:
            return t
        full = torch.zeros(*t.shape[:-1], t.shape[-1] + pad, dtype=t.dtype, device=t.device)
        view = full[..., : t.shape[-1]]
        view.copy_(t)
        return view
    d["kv"] = padded(d["kv"], lay["pad"])
    d["v"] = padded(d["v"], lay["pad"])
    if lay["s_bcast"]:
        s0 = lay["s_pos"]
        d["cos"] = d["cos"][:, :, s0:s0 + 1].contiguous()
        d["sin"] = d["sin"][:, :, s0:s0 + 1].contiguous()
    d["k_rope"] = padded(d["k_rope"], lay["out_pad"])
    d["c_kv"] = padded(d["c_kv"], lay["out_pad"])
    if lay.get("cache_pad"):
        for name in ("k_cache", "ckv_cache"):
            d[name], d[name + "_full"] = padded_cache(d[name], lay["cache_pad"], d["cfg"].seed)
    return d


def _describe(base, over, lay):
    keys = ("batch", "heads", "seq", "kv_dim", "rope_size", "v_dim", "cache_mode", "block_size", "k_cache_dtype",
            "ckv_cache_dtype", "invalid_every", "is_output_kv")
    return base.name + " " + " ".join(f"{k}={over[k]}" for k in keys) + f" layout={lay}"


def _args(Q, d):
    cfg = d["cfg"]
    return Q.kv_args(d["kv"], d["gamma"], d["cos"], d["sin"], d["index"], d["k_cache"], d["ckv_cache"],
                     k_rope_scale=d["k_scale"], k_rope_offset=d["k_offset"], c_kv_scale=d["v_scale"],
                     c_kv_offset=d["v_offset"], v=d["v"], epsilon=cfg.eps, cache_mode=LIB_MODE[cfg.cache_mode],
                     is_output_kv=cfg.is_output_kv, k_rope=d["k_rope"], c_kv=d["c_kv"])


def test_random_cases_are_legal_calls():
    """Host validation accepts every drawn case (CPU tensors; nothing runs on a GPU)."""
    import qk_rmsnorm_rope_amd as Q
    for i in range(N_CASES):
        base, over, lay = _draw(i)
        d = _relayout(W.make_kv_cache(base, device="cpu", **over), lay)
        code = Q.kv_validate(_args(Q, d))
        assert code == 0, f"case {i} ({_describe(base, over, lay)}): {Q.last_error()}"


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    import qk_rmsnorm_rope_amd as Q
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    base, over, lay = _draw(i)
    print(f"case {i}: {_describe(base, over, lay)}", flush=True)
    d = _relayout(W.make_kv_cache(base, device="cuda", **over), lay)
    assert Q.kv_validate(_args(Q, d)) == 0, Q.last_error()
    rep, _ = check_kv(Q, d, f"random-{i}")
    print(rep)
