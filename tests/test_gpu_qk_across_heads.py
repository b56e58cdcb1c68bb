"""GPU parity of qknr_qk_norm_rope_across_heads against the fp64 oracle.

Cases: the tiny fp32 workload in full; the Wan2.2-shaped workload at reduced S
(several blocks and a ragged tail, V present and checked untouched, in and out
of place) and at its full S = 75600 in the launch configuration the benchmark
times (sampled tokens vs the oracle, plus determinism); layout and shape
variants (Q-only, grouped K heads, NBSd strides, many heads -> several waves
per token, head_dim 64/256, fp16, the narrow 4-byte access path, no norm / no
rope, a shared cos/sin table over a batch of 3) and zero tokens.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import check_float, host, oracle_qk, qk_views

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import qk_rmsnorm_rope_amd as lib
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


def _run(Q, d, q, k, q_out=None, k_out=None, **kw):
    Q.qk_norm_rope_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], eps=d["eps"],
                                q_out=q_out, k_out=k_out, **kw)
    torch.cuda.synchronize()


def test_tiny_fp32_full(Q):
    d = W.make_across_heads(W.TINY_ACROSS_HEADS, device="cuda")
    q, k = qk_views(d)
    q_out, k_out = torch.empty_like(q), torch.empty_like(k)
    _run(Q, d, q, k, q_out, k_out)
    _, _, qv, kv = oracle_qk(q, k, d)
    rq = check_float(q_out, qv.reshape(q.shape), "tiny/q", fp32=True)
    rk = check_float(k_out, kv.reshape(k.shape), "tiny/k", fp32=True)
    print(f"tiny fp32 max rel err q {rq:.3g} k {rk:.3g}")


@pytest.mark.parametrize("in_place", [False, True])
def test_wan_reduced_with_v_untouched(Q, in_place):
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=1237, with_v=True)
    qkv_in = d["qkv"].clone()
    q, k = qk_views(d)
    if in_place:
        _run(Q, d, q, k)
        out = d["qkv"]
    else:
        out = torch.full_like(d["qkv"], 7.0)
        oq, ok_ = qk_views(dict(d, qkv=out))
        _run(Q, d, q, k, oq, ok_)
        assert torch.equal(d["qkv"], qkv_in), "out-of-place call modified its input"
    cq = 40 * 128
    # V (after Q|K) is never read or written
    if in_place:
        assert torch.equal(out[..., 2 * cq:], qkv_in[..., 2 * cq:])
    else:
        assert bool((out[..., 2 * cq:] == 7.0).all())
    qi, ki = qk_views(dict(d, qkv=qkv_in))
    _, _, qv, kv = oracle_qk(qi, ki, d)
    oq, ok_ = qk_views(dict(d, qkv=out))
    check_float(oq, qv.reshape(oq.shape), "wan-reduced/q")
    check_float(ok_, kv.reshape(ok_.shape), "wan-reduced/k")


def test_wan_full_size_every_token_and_deterministic(Q):
    """S = 75600, Q|K buffer [1, S, 10240] bf16, out of place -- the benchmark's
    launch; every element of Q and K against the oracle (in token chunks)."""
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda")
    q, k = qk_views(d)
    out1 = torch.empty_like(d["qkv"])
    o1q, o1k = qk_views(dict(d, qkv=out1))
    _run(Q, d, q, k, o1q, o1k)
    T = 75600
    for t0 in range(0, T, 8192):
        tokens = np.arange(t0, min(T, t0 + 8192))
        _, _, qv, kv = oracle_qk(q, k, d, tokens=tokens)
        idx = torch.as_tensor(tokens, device="cuda")
        check_float(o1q.reshape(T, -1)[idx], qv, f"wan-full/q tokens {t0}..")
        check_float(o1k.reshape(T, -1)[idx], kv, f"wan-full/k tokens {t0}..")
    assert bool(torch.isfinite(out1.float()).all())
    out2 = torch.empty_like(d["qkv"])
    o2q, o2k = qk_views(dict(d, qkv=out2))
    _run(Q, d, q, k, o2q, o2k)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "two runs differ"


VARIANTS = {
    "q_only": dict(n_k_heads=0),
    "gqa_8q_2k": dict(n_q_heads=8, n_k_heads=2),
    "many_heads_two_waves": dict(n_q_heads=96, n_k_heads=96),
    "many_heads_four_waves": dict(n_q_heads=200, n_k_heads=64),
    "head_dim_64": dict(head_dim=64, n_q_heads=16, n_k_heads=16),
    "head_dim_256": dict(head_dim=256, n_q_heads=8, n_k_heads=8),
    "head_dim_96": dict(head_dim=96, n_q_heads=6, n_k_heads=6),
    "fp16": dict(dtype=torch.float16),
    "fp32_d128": dict(dtype=torch.float32, n_q_heads=12, n_k_heads=12),
    "batch3": dict(batch=3),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variants(Q, name):
    over = dict(seq=203, table="1d")
    over.update(VARIANTS[name])
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", **over)
    if name == "batch3":
        d["cos"], d["sin"] = d["cos"][:1], d["sin"][:1]       # one table shared by the batch
    q, k = qk_views(d)
    qi, ki = q.clone(), (k.clone() if k is not None else None)
    _run(Q, d, q, k)                                           # in place
    _, _, qv, kv = oracle_qk(qi, ki, d)
    fp32 = d["qkv"].dtype == torch.float32
    check_float(q, qv.reshape(q.shape), f"{name}/q", fp32=fp32)
    if k is not None:
        check_float(k, kv.reshape(k.shape), f"{name}/k", fp32=fp32)


def test_nbsd_layout(Q):
    """Q and K in [n_heads, B, S, d] buffers (the head-major NBSd layout)."""
    B, S, N, hd = 2, 77, 8, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    qn = torch.randn(N, B, S, hd, generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn(N, B, S, hd, generator=g, device="cuda").to(torch.bfloat16)
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", batch=B, seq=S, n_q_heads=N, n_k_heads=N,
                            table="1d")
    q, k = qn.permute(1, 2, 0, 3), kn.permute(1, 2, 0, 3)
    qo, ko = torch.empty_like(qn).permute(1, 2, 0, 3), torch.empty_like(kn).permute(1, 2, 0, 3)
    _run(Q, d, q, k, qo, ko)
    _, _, qv, kv = oracle_qk(q.contiguous(), k.contiguous(), d)
    check_float(qo, qv.reshape(q.shape), "nbsd/q")
    check_float(ko, kv.reshape(k.shape), "nbsd/k")


@pytest.mark.parametrize("norm, rope", [(False, True), (True, False)])
def test_norm_or_rope_only(Q, norm, rope):
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=129, n_q_heads=4, n_k_heads=4, table="1d")
    q, k = qk_views(d)
    qi, ki = q.clone(), k.clone()
    _run(Q, d, q, k, apply_norm=norm, apply_rope=rope)
    _, _, qv, kv = oracle_qk(qi, ki, d, apply_norm=norm, apply_rope=rope)
    check_float(q, qv.reshape(q.shape), "flags/q")
    check_float(k, kv.reshape(k.shape), "flags/k")


def test_narrow_access_path(Q):
    """Q|K start 4 bytes past a 16-byte boundary: the 2-element access path."""
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=65, n_q_heads=4, n_k_heads=4, table="1d")
    B, S = 1, 65
    buf = torch.zeros(B, S, 2 + 8 * 128, dtype=torch.bfloat16, device="cuda")
    buf[..., 2:] = d["qkv"]
    q = buf[..., 2: 2 + 512].unflatten(-1, (4, 128))
    k = buf[..., 2 + 512:].unflatten(-1, (4, 128))
    qi, ki = q.clone(), k.clone()
    a = Q.qk_args(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], eps=d["eps"])
    assert Q.qk_validate(a) == Q.OK
    _run(Q, d, q, k)
    _, _, qv, kv = oracle_qk(qi, ki, d)
    check_float(q, qv.reshape(q.shape), "narrow/q")
    check_float(k, kv.reshape(k.shape), "narrow/k")
    assert bool((buf[..., :2] == 0).all())


def test_zero_tokens_is_a_noop(Q):
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=4, n_q_heads=2, n_k_heads=2, table="1d")
    q, k = qk_views(d)
    Q.qk_norm_rope_across_heads(q[:, :0], k[:, :0], d["q_gamma"], d["k_gamma"], d["cos"][:, :0], d["sin"][:, :0],
                                eps=1e-6)
    torch.cuda.synchronize()


def test_prepared_call_matches_direct_call(Q):
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=333, table="1d")
    q, k = qk_views(d)
    o1, o2 = torch.empty_like(d["qkv"]), torch.empty_like(d["qkv"])
    q1, k1 = qk_views(dict(d, qkv=o1))
    q2, k2 = qk_views(dict(d, qkv=o2))
    _run(Q, d, q, k, q1, k1)
    launch = Q.prepare_qk_norm_rope_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"],
                                                 eps=d["eps"], q_out=q2, k_out=k2)
    launch()
    torch.cuda.synchronize()
    assert torch.equal(q1.reshape(-1).view(torch.int16), q2.reshape(-1).view(torch.int16))
    assert torch.equal(k1.reshape(-1).view(torch.int16), k2.reshape(-1).view(torch.int16))
