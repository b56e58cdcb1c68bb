"""Helpers for the GPU parity tests: host copies of device tensors, the
tolerance rules, and runners that feed one seeded workload to both the HIP
library and the fp64 oracle.

Tolerances (stated by the operator's specification of this build):
* bf16 / f16 outputs: |gpu - ref| <= 8e-3*|ref| + 1e-3, ref = the oracle's
  exact value;
* fp32 outputs: the same bar, plus |gpu - ref| <= 1e-5*(1 + |ref|) (about 150
  fp32 ulps at unit scale: the GPU sums 256..5120 squares in fp32 and uses a
  1-ulp rsqrt; the oracle is exact);
* INT8 codes: equal, or one apart where the oracle's pre-rounding value t lies
  within 1e-3 of a .5 boundary;
* FP8 E4M3FN / E5M2 codes: equal, or adjacent where t lies within 1e-3 of the
  code spacing from the midpoint between the two values;
* cache bytes the operator must not write, and scatter positions: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

ORC = {torch.float32: oracle.F32, torch.bfloat16: oracle.BF16, torch.float16: oracle.F16,
       torch.int8: oracle.INT8, torch.float8_e4m3fn: oracle.E4M3FN, torch.float8_e5m2: oracle.E5M2}
_FP8 = {torch.float8_e4m3fn: oracle.E4M3FN, torch.float8_e5m2: oracle.E5M2}


def host(t):
    """Storage bits of a tensor as a host numpy array (16-bit floats as uint16)."""
    if t is None:
        return None
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in _FP8:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def values(t):
    return t.detach().float().double().cpu().numpy()


def check_float(gpu, ref, what, fp32=False):
    """gpu: torch tensor of outputs; ref: exact oracle values (same shape)."""
    g = values(gpu).reshape(ref.shape)
    err = np.abs(g - ref)
    bound = 8e-3 * np.abs(ref) + 1e-3
    bad = ~(err <= bound)
    if bad.any():
        i = np.argmax(np.where(bad, err - bound, -np.inf))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside 8e-3|ref|+1e-3; "
                             f"worst at flat {i}: gpu {g.flat[i]!r} ref {ref.flat[i]!r}")
    if fp32:
        tight = err <= 1e-5 * (1 + np.abs(ref))
        assert tight.all(), f"{what}: fp32 error above 1e-5(1+|ref|): max {err.max()}"
    rel = float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0
    return rel


def check_dot(gpu, ref, mag, k, what):
    """Outputs of a k-term dot product rounded to bf16: the bf16 bar plus the
    classical worst-case bound for recursive fp32 summation, k * 2^-24 times
    the sum of the magnitudes of the terms (`mag` = sum_k |a_k w_k|, scaled as
    the output is). The matrix cores' FP8 dot product adds its 64-term blocks
    in an order of its own, so the exact fp64 value is off by up to that much
    before the output rounding."""
    g = values(gpu).reshape(ref.shape)
    err = np.abs(g - ref)
    bound = 8e-3 * np.abs(ref) + 1e-3 + k * 2.0 ** -24 * mag
    bad = ~(err <= bound)
    if bad.any():
        i = np.argmax(np.where(bad, err - bound, -np.inf))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the dot-product bound; worst at "
                             f"flat {i}: gpu {g.flat[i]!r} ref {ref.flat[i]!r} term magnitude {mag.flat[i]!r}")
    return float((err / np.maximum(mag, 1e-30)).max()) if err.size else 0.0


def check_int8(gpu_codes, ref_codes, t, what):
    g = np.asarray(gpu_codes, np.int64).reshape(ref_codes.shape)
    r = np.asarray(ref_codes, np.int64)
    diff = g != r
    if diff.any():
        frac = np.abs(t - (np.floor(t) + 0.5))
        ok = (np.abs(g - r) == 1) & (frac <= 1e-3)
        bad = diff & ~ok
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            raise AssertionError(f"{what}: {int(bad.sum())} int8 codes differ outside the tie window; "
                                 f"first at {i}: gpu {g.flat[i]} ref {r.flat[i]} t {t.flat[i]!r}")
    return int(diff.sum())


def check_fp8(gpu_codes, ref_codes, t, what, fmt=oracle.E4M3FN):
    """FP8 codes of format `fmt` (oracle.E4M3FN or oracle.E5M2)."""
    g = np.asarray(gpu_codes, np.uint8).reshape(ref_codes.shape)
    r = np.asarray(ref_codes, np.uint8)
    diff = g != r
    if diff.any():
        gv = oracle.decode(fmt, g[diff])
        rv = oracle.decode(fmt, r[diff])
        tt = np.asarray(t, np.float64)[diff]
        spacing = np.abs(gv - rv)
        mid = (gv + rv) / 2
        # adjacent: no representable value strictly between them
        adjacent = np.array([_adjacent(a, b, fmt) for a, b in zip(g[diff], r[diff])])
        ok = adjacent & (np.abs(tt - mid) <= 1e-3 * spacing)
        if not ok.all():
            j = int(np.flatnonzero(~ok)[0])
            raise AssertionError(f"{what}: {int((~ok).sum())} fp8 codes differ outside the tie window; "
                                 f"gpu {gv[j]} ref {rv[j]} t {tt[j]!r}")
    return int(diff.sum())



def _adjacent(a, b, fmt=oracle.E4M3FN):
    va, vb = oracle.decode(fmt, np.array([a, b], np.uint8))
    lo, hi = min(va, vb), max(va, vb)
    allv = oracle.decode(fmt, np.arange(256, dtype=np.uint8))
    allv = allv[np.isfinite(allv)]
    return not np.any((allv > lo) & (allv < hi))


# ---------------------------------------------------------------- (a)

def qk_views(d, with_v=False):
    """Q and K views [B, S, N, d] of the BSD buffer of a workload dict."""
    qkv = d["qkv"]
    nq, nk, hd = d["n_q_heads"], d["n_k_heads"], d["head_dim"]
    q = qkv[..., : nq * hd].unflatten(-1, (nq, hd))
    k = qkv[..., nq * hd: (nq + nk) * hd].unflatten(-1, (nk, hd)) if nk else None
    return q, k


def oracle_qk(q, k, d, tokens=None, **kw):
    """Oracle of (a) for the tokens (flat b*S+s indices, None = all)."""
    B, S, nq, hd = q.shape
    T = B * S
    qf = q.reshape(T, nq * hd)
    kf = k.reshape(T, k.shape[2] * hd) if k is not None else None
    cos = d["cos"].expand(B, S, hd).reshape(T, hd)
    sin = d["sin"].expand(B, S, hd).reshape(T, hd)
    if tokens is not None:
        idx = torch.as_tensor(tokens, device=q.device)
        qf, cos, sin = qf[idx], cos[idx], sin[idx]
        kf = kf[idx] if kf is not None else None
    return oracle.qk_norm_rope_across_heads(
        host(qf), host(kf), host(d["q_gamma"]), host(d["k_gamma"]), host(cos), host(sin), d["eps"],
        nq, k.shape[2] if k is not None else 0, hd, ORC[q.dtype], **kw)


# ---------------------------------------------------------------- (b)

def cache_rows(d):
    """Flat cache row (of [rows, D]) written by each (b, n, s), -1 if none.

    Norm [B, N, Scache, D]: (b*N + n)*Scache + index[b, s];
    PA_BNSD [block_num, block_size, N, D]: slot*N + n with slot = index[b*S + s];
    PA_BLK_BNSD: the same with slot = index[b, s // bs] + s % bs (one starting
    slot per run of bs tokens). A slot outside the cache writes nothing.
    """
    cfg = d["cfg"]
    B, N, S = cfg.batch, cfg.heads, cfg.seq
    n = np.arange(N).reshape(1, N, 1)
    if cfg.cache_mode == "pa_blk_bnsd":
        bs = cfg.block_size
        starts = d["index"].cpu().numpy().reshape(B, -1).astype(np.int64)
        s = np.arange(S)
        st = starts[:, s // bs]
        slot = np.where(st >= 0, st + s % bs, -1).reshape(B, 1, S)
    else:
        slot = d["index"].cpu().numpy().reshape(B, 1, S).astype(np.int64)
    if cfg.cache_mode == "norm":
        capacity = cfg.cache_rows
        rows = (np.arange(B).reshape(B, 1, 1) * N + n) * cfg.cache_rows + slot
    else:
        capacity = cfg.block_num * cfg.block_size
        rows = slot * N + n
    return np.where((slot >= 0) & (slot < capacity), rows, -1)


def run_oracle_kv(d, inplace_zero_caches=False):
    cfg = d["cfg"]
    k_cache = d["k_cache"]
    c_cache = d["ckv_cache"]
    if inplace_zero_caches:
        kh = np.zeros(tuple(k_cache.shape), oracle.STORAGE[ORC[k_cache.dtype]])
        ch = np.zeros(tuple(c_cache.shape), oracle.STORAGE[ORC[c_cache.dtype]])
    else:
        kh, ch = host(k_cache), host(c_cache)
    np32 = lambda t: None if t is None else t.cpu().numpy()
    return oracle.kv_rmsnorm_rope_cache(
        host(d["kv"]), host(d["v"]), host(d["gamma"]), host(d["cos"]), host(d["sin"]),
        d["index"].cpu().numpy(), kh, ch, rms_size=cfg.rms_size, rope_size=cfg.rope_size,
        eps=cfg.eps, cache_mode=_ORC_MODE[cfg.cache_mode],
        in_dtype=ORC[cfg.dtype], k_dtype=ORC[k_cache.dtype], ckv_dtype=ORC[c_cache.dtype],
        block_size=cfg.block_size, k_scale=np32(d["k_scale"]), k_offset=np32(d["k_offset"]),
        v_scale=np32(d["v_scale"]), v_offset=np32(d["v_offset"]), is_output_kv=cfg.is_output_kv,
        copy_caches=not inplace_zero_caches)


_ORC_MODE = {"norm": oracle.NORM, "pa_bnsd": oracle.PA_BNSD, "pa_blk_bnsd": oracle.PA_BLK_BNSD}
LIB_MODE = {"norm": "Norm", "pa_bnsd": "PA_BNSD", "pa_blk_bnsd": "PA_BLK_BNSD"}


def run_gpu_kv(Q, d):
    cfg = d["cfg"]
    mode = LIB_MODE[cfg.cache_mode]
    return Q.kv_rmsnorm_rope_cache(
        d["kv"], d["gamma"], d["cos"], d["sin"], d["index"], d["k_cache"], d["ckv_cache"],
        k_rope_scale=d["k_scale"], k_rope_offset=d["k_offset"], c_kv_scale=d["v_scale"],
        c_kv_offset=d["v_offset"], v=d["v"], epsilon=cfg.eps, cache_mode=mode,
        is_output_kv=cfg.is_output_kv, k_rope=d["k_rope"], c_kv=d["c_kv"])


def padded_cache(cache, pad_bytes, seed):
    """The cache's values in a buffer whose rows are pad_bytes longer (the
    padding filled with seeded random bytes); returns (view, full buffer)."""
    pad = pad_bytes // cache.element_size()
    g = torch.Generator(device=cache.device).manual_seed(seed + 31)
    full_shape = tuple(cache.shape[:-1]) + (cache.shape[-1] + pad,)
    raw = torch.randint(0, 256, full_shape[:-1] + (full_shape[-1] * cache.element_size(),), generator=g,
                        device=cache.device, dtype=torch.uint8)
    full = raw.view(cache.dtype)
    view = full[..., : cache.shape[-1]]
    view.copy_(cache)
    return view, full


def check_kv(Q, d, what, big_cache=False):
    """Run the HIP operator and the oracle on workload d and compare:
    untouched cache rows bit-exact, written rows within the code/float rules,
    k_rope / c_kv within the float rule, and the padding of row-padded caches
    (d["k_cache_full"], d["ckv_cache_full"]) untouched. Returns a small report
    dict."""
    cfg = d["cfg"]
    k_pre, c_pre = d["k_cache"].clone(), d["ckv_cache"].clone()
    pads = {n: d[n + "_full"][..., d[n].shape[-1]:].clone() for n in ("k_cache", "ckv_cache") if n + "_full" in d}
    run_gpu_kv(Q, d)
    torch.cuda.synchronize()
    for n, before in pads.items():
        after = d[n + "_full"][..., d[n].shape[-1]:]
        assert torch.equal(after.view(torch.uint8) if after.element_size() == 1 else after.view(torch.int16),
                           before.view(torch.uint8) if before.element_size() == 1 else before.view(torch.int16)), \
            f"{what}/{n}: the row padding was written"
    r = run_oracle_kv(d, inplace_zero_caches=big_cache)
    rows = cache_rows(d)                          # [B, N, S]
    valid = rows >= 0
    flat = rows[valid]
    assert len(np.unique(flat)) == len(flat), "workload has duplicate slots"
    report = {}
    for name, cache, pre, t, x, ref_cache in (
            ("k_cache", d["k_cache"], k_pre, r["k_t"], r["k_x"], r["k_cache"]),
            ("ckv_cache", d["ckv_cache"], c_pre, r["c_t"], r["c_x"], r["ckv_cache"])):
        width = cache.shape[-1]
        g2 = cache.reshape(-1, width)
        p2 = pre.reshape(-1, width)
        bytes_now = g2.view(torch.uint8) if cache.element_size() == 1 else g2.view(torch.int16)
        bytes_pre = p2.view(torch.uint8) if cache.element_size() == 1 else p2.view(torch.int16)
        changed = (bytes_now != bytes_pre).any(-1)
        mask = torch.zeros(g2.shape[0], dtype=torch.bool, device=cache.device)
        mask[torch.as_tensor(flat, device=cache.device)] = True
        stray = changed & ~mask
        assert not bool(stray.any()), f"{what}/{name}: {int(stray.sum())} rows written outside the index set"
        got = g2[torch.as_tensor(flat, device=cache.device)]
        ref_rows = ref_cache.reshape(-1, width)[flat]
        tv = t[valid]
        xv = x[valid]
        if cache.dtype == torch.int8:
            report[name + "_pm1"] = check_int8(host(got), ref_rows, tv, f"{what}/{name}")
        elif cache.dtype in _FP8:
            report[name + "_adjacent"] = check_fp8(host(got), ref_rows, tv, f"{what}/{name}", _FP8[cache.dtype])
        else:
            report[name + "_rel"] = check_float(got, xv, f"{what}/{name}")
    if cfg.is_output_kv and d["k_rope"] is not None:
        report["k_rope_rel"] = check_float(d["k_rope"], r["k_x"], f"{what}/k_rope")
        report["c_kv_rel"] = check_float(d["c_kv"], r["c_x"], f"{what}/c_kv")
        # An unquantised cache row is the same rounding of the same value as
        # the raw output row: the two must agree bit for bit.
        vmask = torch.as_tensor(valid, device=d["kv"].device)
        for name, cache, out in (("k_cache", d["k_cache"], d["k_rope"]), ("ckv_cache", d["ckv_cache"], d["c_kv"])):
            if cache.dtype != out.dtype:
                continue
            width = cache.shape[-1]
            got = cache.reshape(-1, width)[torch.as_tensor(flat, device=cache.device)]
            raw = out.reshape(B_N_S(cfg) + (width,))[vmask]
            same = got.view(torch.int16) == raw.view(torch.int16)
            assert bool(same.all()), (f"{what}/{name}: {int((~same).sum())} cache elements differ from "
                                      f"the raw output row's bits")
        report["cache_equals_raw_rows"] = True
    return report, r


def B_N_S(cfg):
    return (cfg.batch, cfg.heads, cfg.seq)
