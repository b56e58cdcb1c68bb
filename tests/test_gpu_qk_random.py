"""Seeded random shapes for the QK operator's forms against the fp64 oracle.

30 cases draw the form (across heads, per head, or the two-pass split over
2-4 head shards composed back), the element type (bf16, fp16, fp32), the head
size (64, 96, 128, 256), the head counts (1-64 Q heads, 0 to as many K heads,
so Q-only and grouped K), batch and sequence (1-700 tokens per batch), in or out
of place, a cos/sin table shared by the batch or one per batch, the layout of Q
and K (the BSD projection buffer, separate NBSd tensors, or heads padded by 8 or
4 elements: the 16- and 8-byte access paths), and (for the single-pass forms)
norm-only or rope-only calls. The launch choices that follow
from them -- chunks per half head, heads per lane, 1/2/4 waves per unit -- vary
with the draw. A CPU test checks that host validation accepts every drawn
case, so the GPU test never skips.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import check_float, qk_views
from tests.test_gpu_qk_forms import _oracle

N_CASES = 30


def _draw(i):
    rng = np.random.default_rng(8000 + i)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    form = pick(["across", "across", "per_head", "split"])
    dtype = pick([torch.bfloat16, torch.bfloat16, torch.float16, torch.float32])
    hd = pick([64, 96, 128, 256])
    if form == "split":
        tp = pick([2, 3, 4])
        nq = tp * int(rng.integers(1, 17))
        nk = tp * int(rng.integers(1, nq // tp + 1))
    else:
        tp = 1
        nq = int(rng.integers(1, 65))
        nk = pick([0, nq, max(1, nq // int(rng.integers(1, 9)))])
    batch, seq = int(rng.integers(1, 4)), int(rng.integers(1, 701))
    norm, rope = True, True
    if form != "split" and rng.random() < 0.2:
        norm, rope = pick([(True, False), (False, True)])
    c = dict(form=form, dtype=dtype, head_dim=hd, n_q=nq, n_k=nk, tp=tp, batch=batch, seq=seq,
             in_place=bool(rng.random() < 0.5), shared_table=bool(rng.random() < 0.3), norm=norm, rope=rope,
             eps=pick([1e-6, 1e-5]), seed=8000 + i)
    # memory layout of Q and K (and of the outputs): the BSD projection buffer, separate
    # NBSd tensors viewed as [B, S, N, d], or heads padded by 8 or 4 elements
    c["layout"] = pick(["bsd", "bsd", "nbsd", "pad8", "pad4"])
    if c["layout"] == "pad4" and nq * hd > 4096:
        c["layout"] = "pad8"      # 8-byte accesses hold fewer heads per block: wide segments are unsupported
    return c


def _views(d, c, buf_like=None):
    """Q and K views [B, S, N, d] in the case's layout holding the values of
    the workload's BSD buffer (or, with buf_like, fresh storage of that layout
    filled with 5.0, for outputs)."""
    q0, k0 = qk_views(d)
    lay = c["layout"]
    B, S, nq, hd = q0.shape
    nk = k0.shape[2] if k0 is not None else 0
    dev, dt = q0.device, q0.dtype
    if lay == "bsd":
        if buf_like is None:
            return q0, k0
        return qk_views(dict(d, qkv=torch.full_like(d["qkv"], 5.0)))
    if lay == "nbsd":
        q = torch.full((nq, B, S, hd), 5.0, dtype=dt, device=dev).permute(1, 2, 0, 3)
        k = torch.full((nk, B, S, hd), 5.0, dtype=dt, device=dev).permute(1, 2, 0, 3) if nk else None
    else:
        pad = 8 if lay == "pad8" else 4
        buf = torch.full((B, S, nq + nk, hd + pad), 5.0, dtype=dt, device=dev)
        q = buf[:, :, :nq, :hd]
        k = buf[:, :, nq:, :hd] if nk else None
    if buf_like is None:
        q.copy_(q0)
        if nk:
            k.copy_(k0)
    return q, k


def _split(Q, q, k, oq, ok_, qg, kg, cos, sin, eps, tp):
    """The two passes over tp head shards of q/k, writing shard views of oq/ok_
    (Q and K outputs share one buffer, and so their strides), the shards' sums
    added in between as an all-reduce would."""
    nq, nk, d = q.shape[2], k.shape[2], q.shape[3]
    lq, lk = nq // tp, nk // tp
    shard = lambda t, r, n: t[:, :, r * n:(r + 1) * n]
    sums = [Q.qk_sumsq_across_heads(shard(q, r, lq), shard(k, r, lk)) for r in range(tp)]
    total = torch.stack(sums).sum(0)
    for r in range(tp):
        Q.qk_apply_across_heads(shard(q, r, lq), shard(k, r, lk), qg[r * lq * d:(r + 1) * lq * d],
                                kg[r * lk * d:(r + 1) * lk * d], cos, sin, total, eps=eps, q_norm_channels=nq * d,
                                k_norm_channels=nk * d, q_out=shard(oq, r, lq), k_out=shard(ok_, r, lk))
    torch.cuda.synchronize()


def _inputs(c, device):
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device=device, batch=c["batch"], seq=c["seq"], n_q_heads=c["n_q"],
                            n_k_heads=c["n_k"], head_dim=c["head_dim"], dtype=c["dtype"], table="1d",
                            eps=c["eps"], seed=c["seed"])
    if c["shared_table"]:
        d["cos"], d["sin"] = d["cos"][:1], d["sin"][:1]
    hd = c["head_dim"]
    if c["form"] == "per_head":
        g = torch.Generator(device=device).manual_seed(c["seed"])
        d["q_gamma"] = (torch.rand(hd, generator=g, device=device) + 0.5).to(c["dtype"])
        d["k_gamma"] = (torch.rand(hd, generator=g, device=device) + 0.5).to(c["dtype"]) if c["n_k"] else None
    return d


def _host_args(Q, i):
    """Case i's argument struct on CPU tensors (a split case: its first shard),
    with the tensors it points into."""
    c = _draw(i)
    d = _inputs(c, "cpu")
    q, k = _views(d, c)
    if c["form"] == "split":
        lq, lk = c["n_q"] // c["tp"], c["n_k"] // c["tp"]
        q, k = q[:, :, :lq], k[:, :, :lk]
        d["q_gamma"], d["k_gamma"] = d["q_gamma"][: lq * c["head_dim"]], d["k_gamma"][: lk * c["head_dim"]]
    a = Q.qk_args(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], eps=c["eps"],
                  apply_norm=c["norm"], apply_rope=c["rope"], per_head=c["form"] == "per_head")
    return c, a, (d, q, k)


def host_call_status(Q, i):
    """Status of case i's entry point called on CPU tensors (no GPU: past
    validation and planning the launch itself fails)."""
    import ctypes
    c, a, keep = _host_args(Q, i)
    if c["form"] == "split":
        sums = torch.empty(2, c["batch"] * c["seq"], dtype=torch.float32)
        return Q._lib.qknr_qk_sumsq_across_heads(ctypes.byref(a), ctypes.c_void_p(sums.data_ptr()), None)
    fn = Q._lib.qknr_qk_norm_rope_per_head if c["form"] == "per_head" else Q._lib.qknr_qk_norm_rope_across_heads
    return fn(ctypes.byref(a), None)


def test_random_qk_cases_are_legal_calls():
    """Host validation accepts every drawn case (CPU tensors; nothing runs on a GPU)."""
    import qk_rmsnorm_rope_amd as Q
    for i in range(N_CASES):
        c, a, keep = _host_args(Q, i)
        assert Q.qk_validate(a) == 0, f"case {i} ({c}): {Q.last_error()}"


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_qk_case(i):
    import qk_rmsnorm_rope_amd as Q
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = _draw(i)
    print(f"case {i}: {c}", flush=True)
    d = _inputs(c, "cuda")
    q, k = _views(d, c)
    qi = q.clone()
    ki = k.clone() if k is not None else None
    fp32 = c["dtype"] == torch.float32
    if c["form"] == "split":
        oq, ok_ = _views(d, c, buf_like=True)
        _split(Q, q, k, oq, ok_, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], c["eps"], c["tp"])
        rq, rk = _oracle(qi, ki, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], c["eps"])
    else:
        if c["in_place"]:
            oq, ok_ = q, k
        else:
            oq, ok_ = _views(d, c, buf_like=True)
        call = Q.qk_norm_rope_per_head if c["form"] == "per_head" else Q.qk_norm_rope_across_heads
        cos, sin = (d["cos"], d["sin"]) if c["rope"] else (None, None)
        call(q, k, d["q_gamma"], d["k_gamma"], cos, sin, eps=c["eps"], q_out=oq,
             k_out=ok_ if k is not None else None, apply_norm=c["norm"], apply_rope=c["rope"])
        torch.cuda.synchronize()
        rq, rk = _oracle(qi, ki, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], c["eps"],
                         per_head=c["form"] == "per_head", apply_norm=c["norm"], apply_rope=c["rope"])
        if not c["in_place"]:
            assert torch.equal(q, qi), "an out-of-place call modified its input"
    check_float(oq, rq.reshape(oq.shape), f"case {i}/q", fp32=fp32)
    if k is not None:
        check_float(ok_, rk.reshape(ok_.shape), f"case {i}/k", fp32=fp32)
