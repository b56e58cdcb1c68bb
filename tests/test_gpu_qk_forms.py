"""GPU parity of the other forms of the QK operator against the fp64 oracle.

* per head (qknr_qk_norm_rope_per_head): the Wan2.2 head geometry at reduced S
  (several blocks, ragged tail), head_dim 64 / 96 (a 6-lane head: the
  non-power-of-two group sum) / 128 / 256, fp16, fp32, Q only, many heads (2 and
  4 waves per unit), the 4-byte access path, no RoPE;
* split over ranks (qknr_qk_sumsq_across_heads, then the caller's sum, then
  qknr_qk_apply_across_heads): the 40 Wan heads over tp = 2, 4, 5 shards at
  reduced S and tp = 4 at the full S = 75600 on sampled tokens -- the composed
  result must match the oracle's single-device operator; the sums themselves
  against the oracle's fp64 sums; sums of all heads fed back with the call's own
  channel count reproduce the fused kernel bit for bit;
* the interleaved -> rotate-half permutation: a fused QKV weight (V block
  untouched), an MX-style [H/4, I, 4] fp8 weight, interleaved cos/sin tables,
  6-byte inner blocks, the inverse; bit-exact against the oracle's index
  arithmetic. And end to end: an interleaved-lane model converted on the GPU
  and run through the rotate-half kernel equals the oracle's interleaved RoPE
  in permuted lane order.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import ORC, check_float, host, qk_views

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import qk_rmsnorm_rope_amd as lib
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


def _oracle(q, k, qg, kg, cos, sin, eps, **kw):
    """Oracle on [B, S, n, d] tensors (any strides), cos/sin [B or 1, S, d]."""
    B, S, nq, d = q.shape
    nk = k.shape[2] if k is not None else 0
    dt = ORC[q.dtype]
    flat = lambda t: host(t.contiguous().reshape(B * S, -1))
    cs = cos.expand(B, S, d).reshape(B * S, d)
    sn = sin.expand(B, S, d).reshape(B * S, d)
    return oracle.qk_norm_rope(flat(q), flat(k) if nk else None, host(qg), host(kg) if nk else None,
                               host(cs), host(sn), eps, nq, nk, d, dt, **kw)[2:]


def _per_head_inputs(seq=203, nq=40, nk=40, d=128, dtype=torch.bfloat16, seed=11):
    d_ = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=seq, n_q_heads=nq, n_k_heads=nk,
                             head_dim=d, dtype=dtype, table="1d")
    g = torch.Generator(device="cuda").manual_seed(seed)
    qg = (torch.rand(d, generator=g, device="cuda") + 0.5).to(dtype)
    kg = (torch.rand(d, generator=g, device="cuda") + 0.5).to(dtype)
    return d_, qg, kg


PER_HEAD = {
    "wan_d128": dict(),
    "d64": dict(d=64, nq=16, nk=16),
    "d96_six_lane_heads": dict(d=96, nq=12, nk=12),
    "d256": dict(d=256, nq=8, nk=8),
    "fp16": dict(dtype=torch.float16),
    "fp32": dict(dtype=torch.float32, nq=12, nk=12),
    "q_only": dict(nk=0),
    "two_waves": dict(nq=96, nk=96),
    "four_waves": dict(nq=200, nk=64),
}


@pytest.mark.parametrize("name", sorted(PER_HEAD))
def test_per_head(Q, name):
    d, qg, kg = _per_head_inputs(**PER_HEAD[name])
    q, k = qk_views(d)
    out = torch.full_like(d["qkv"], 3.0)
    oq, ok_ = qk_views(dict(d, qkv=out))
    Q.qk_norm_rope_per_head(q, k, qg, kg if k is not None else None, d["cos"], d["sin"], eps=d["eps"],
                            q_out=oq, k_out=ok_)
    torch.cuda.synchronize()
    rq, rk = _oracle(q, k, qg, kg, d["cos"], d["sin"], d["eps"], per_head=True)
    fp32 = q.dtype == torch.float32
    check_float(oq, rq.reshape(oq.shape), f"{name}/q", fp32=fp32)
    if k is not None:
        check_float(ok_, rk.reshape(ok_.shape), f"{name}/k", fp32=fp32)


def test_per_head_narrow_path_and_no_rope(Q):
    """Q|K 4 bytes past a 16-byte boundary (2-element chunks: 32-lane heads)."""
    d, qg, kg = _per_head_inputs(seq=65, nq=4, nk=4)
    buf = torch.zeros(1, 65, 2 + 8 * 128, dtype=torch.bfloat16, device="cuda")
    buf[..., 2:] = d["qkv"]
    q = buf[..., 2: 2 + 512].unflatten(-1, (4, 128))
    k = buf[..., 2 + 512:].unflatten(-1, (4, 128))
    qi, ki = q.clone(), k.clone()
    Q.qk_norm_rope_per_head(q, k, qg, kg, d["cos"], d["sin"], eps=d["eps"])
    torch.cuda.synchronize()
    rq, rk = _oracle(qi, ki, qg, kg, d["cos"], d["sin"], d["eps"], per_head=True)
    check_float(q, rq.reshape(q.shape), "narrow/q")
    check_float(k, rk.reshape(k.shape), "narrow/k")
    q2, k2 = qi.clone(), ki.clone()
    Q.qk_norm_rope_per_head(q2, k2, qg, kg, None, None, eps=d["eps"], apply_rope=False)
    torch.cuda.synchronize()
    rq, rk = _oracle(qi, ki, qg, kg, d["cos"], d["sin"], d["eps"], per_head=True, apply_rope=False)
    check_float(q2, rq.reshape(q.shape), "norope/q")
    check_float(k2, rk.reshape(k.shape), "norope/k")


def _split(Q, q, k, qg, kg, cos, sin, eps, tp):
    """Run the two passes on tp head shards of q/k (views), adding the sums."""
    nq, nk, d = q.shape[2], k.shape[2], q.shape[3]
    lq, lk = nq // tp, nk // tp
    shards = [(q[:, :, r * lq:(r + 1) * lq], k[:, :, r * lk:(r + 1) * lk],
               qg[r * lq * d:(r + 1) * lq * d], kg[r * lk * d:(r + 1) * lk * d]) for r in range(tp)]
    sums = [Q.qk_sumsq_across_heads(sq, sk) for sq, sk, _, _ in shards]
    total = torch.stack(sums).sum(0)           # stands in for the all-reduce over the ranks
    outs = []
    for sq, sk, gq, gk in shards:
        oq, ok_ = torch.empty_like(sq), torch.empty_like(sk)
        Q.qk_apply_across_heads(sq, sk, gq, gk, cos, sin, total, eps=eps, q_norm_channels=nq * d,
                                k_norm_channels=nk * d, q_out=oq, k_out=ok_)
        outs.append((oq, ok_))
    torch.cuda.synchronize()
    return sums, total, torch.cat([o[0] for o in outs], 2), torch.cat([o[1] for o in outs], 2)


@pytest.mark.parametrize("tp", [2, 4, 5])
def test_split_over_ranks_matches_the_single_device_operator(Q, tp):
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=1237)
    q, k = qk_views(d)
    sums, total, oq, ok_ = _split(Q, q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], d["eps"], tp)
    rq, rk = _oracle(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], d["eps"])
    check_float(oq, rq.reshape(oq.shape), f"tp{tp}/q")
    check_float(ok_, rk.reshape(ok_.shape), f"tp{tp}/k")
    # each shard's sums against the oracle's fp64 sums (fp32 accumulation of 1280..2560 squares)
    T = q.shape[0] * q.shape[1]
    lq = 40 // tp
    for r, s in enumerate(sums):
        xs = host(q[:, :, r * lq:(r + 1) * lq].contiguous().reshape(T, -1))
        ref = oracle.qk_sumsq(xs, lq, 128, oracle.BF16)
        np.testing.assert_allclose(s[0].cpu().double().numpy(), ref, rtol=2e-5)


def test_split_full_size_every_token(Q):
    """tp = 4 shards of the 40 + 40 heads at S = 75600; every token against the
    single-device oracle (in token chunks)."""
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda")
    q, k = qk_views(d)
    _, _, oq, ok_ = _split(Q, q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], d["eps"], 4)
    T = 75600
    for t0 in range(0, T, 8192):
        tokens = np.arange(t0, min(T, t0 + 8192))
        idx = torch.as_tensor(tokens, device="cuda")
        sel = lambda t: t.reshape(T, *t.shape[2:])[idx].unsqueeze(0)
        rq, rk = _oracle(sel(q), sel(k), d["q_gamma"], d["k_gamma"], sel(d["cos"]), sel(d["sin"]), d["eps"])
        check_float(sel(oq), rq.reshape(1, len(tokens), 40, 128), f"full/q tokens {t0}..")
        check_float(sel(ok_), rk.reshape(1, len(tokens), 40, 128), f"full/k tokens {t0}..")


def test_sums_of_all_heads_reproduce_the_fused_kernel_bitwise(Q):
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=777)
    q, k = qk_views(d)
    f = torch.empty_like(d["qkv"])
    fq, fk = qk_views(dict(d, qkv=f))
    Q.qk_norm_rope_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], eps=d["eps"],
                                q_out=fq, k_out=fk)
    s = Q.qk_sumsq_across_heads(q, k)
    a = torch.empty_like(d["qkv"])
    aq, ak = qk_views(dict(d, qkv=a))
    Q.qk_apply_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], s, eps=d["eps"],
                            q_norm_channels=0, q_out=aq, k_out=ak)
    torch.cuda.synchronize()
    assert torch.equal(f.view(torch.int16), a.view(torch.int16))


def test_split_q_only_and_zero_tokens(Q):
    d = W.make_across_heads(W.WAN22_SELF_ATTN, device="cuda", seq=99, n_k_heads=0, table="1d")
    q, _ = qk_views(d)
    s = Q.qk_sumsq_across_heads(q)
    assert tuple(s.shape) == (1, 99)
    out = torch.empty_like(q)
    Q.qk_apply_across_heads(q, None, d["q_gamma"], None, d["cos"], d["sin"], s, eps=d["eps"],
                            q_norm_channels=40 * 128, q_out=out)
    torch.cuda.synchronize()
    rq, _ = _oracle(q, None, d["q_gamma"], None, d["cos"], d["sin"], d["eps"])
    check_float(out, rq.reshape(out.shape), "q-only")
    e = Q.qk_sumsq_across_heads(q[:, :0])
    torch.cuda.synchronize()
    assert e.numel() == 0


def _perm_ref(t, head_dim, dim, first, n_heads, inverse=False):
    a = t.cpu().view(torch.uint8 if t.element_size() == 1 else
                     {2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]).numpy()
    return oracle.interleaved_to_rotate_half(a, head_dim, axis=dim, first=first, n_heads=n_heads,
                                             inverse=inverse)


def _bits(t):
    return t.cpu().view(torch.uint8 if t.element_size() == 1 else
                        {2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]).numpy()


@pytest.mark.parametrize("case", ["qkv_weight", "mx_weight", "tables_fp32", "inner6", "bias_inverse"])
def test_permutation_bit_exact(Q, case):
    g = torch.Generator(device="cuda").manual_seed(31)
    if case == "qkv_weight":          # [H, (40 + 2*40)*128] bf16: Q and K blocks, V untouched
        t = torch.randn(64, 120 * 128, generator=g, device="cuda").to(torch.bfloat16)
        kw = dict(head_dim=128, dim=1, first=0, n_heads=80)
    elif case == "mx_weight":         # [H/4, I, 4] fp8 codes
        t = torch.randint(0, 256, (16, 24 * 64, 4), generator=g, device="cuda", dtype=torch.uint8)
        t = t.view(torch.float8_e4m3fn)
        kw = dict(head_dim=64, dim=1, first=0, n_heads=16)
    elif case == "tables_fp32":       # interleaved cos table [S, d]
        th = torch.rand(300, 64, generator=g, device="cuda", dtype=torch.float64)
        t = th.repeat_interleave(2, dim=1).cos().float()
        kw = dict(head_dim=128, dim=-1, first=0, n_heads=1)
    elif case == "inner6":            # 6-byte inner blocks (2-byte accesses), blocks start at 3
        t = torch.randn(5, 3 + 4 * 16 + 5, 3, generator=g, device="cuda").to(torch.float16)
        kw = dict(head_dim=16, dim=1, first=3, n_heads=4)
    else:                             # a bias [I], permuted and back
        t = torch.randn(80 * 128, generator=g, device="cuda").to(torch.bfloat16)
        kw = dict(head_dim=128, dim=0, first=0, n_heads=80)
    out = Q.interleaved_to_rotate_half(t, kw["head_dim"], dim=kw["dim"], first=kw["first"], n_heads=kw["n_heads"])
    back = Q.interleaved_to_rotate_half(out, kw["head_dim"], dim=kw["dim"], first=kw["first"],
                                        n_heads=kw["n_heads"], inverse=True)
    torch.cuda.synchronize()
    ref = _perm_ref(t, kw["head_dim"], kw["dim"], kw["first"], kw["n_heads"])
    np.testing.assert_array_equal(_bits(out), ref)
    np.testing.assert_array_equal(_bits(back), _bits(t))
    if case == "tables_fp32":         # the converted table is a rotate-half table
        o = out.cpu()
        assert torch.equal(o[:, :64], o[:, 64:])


def test_interleaved_model_converted_on_gpu_runs_on_the_rotate_half_kernel(Q):
    """q, k in interleaved lane order with interleaved tables and gammas: after
    the GPU conversion, the across-heads kernel's output equals the oracle's
    interleaved-pair RoPE (complex rotation of lanes 2j, 2j+1) in rotate-half
    lane order."""
    S, nh, dh = 129, 8, 128
    g = torch.Generator(device="cuda").manual_seed(41)
    q = torch.randn(1, S, nh, dh, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, S, nh, dh, generator=g, device="cuda").to(torch.bfloat16)
    gq = (torch.rand(nh * dh, generator=g, device="cuda") + 0.5).to(torch.bfloat16)
    gk = (torch.rand(nh * dh, generator=g, device="cuda") + 0.5).to(torch.bfloat16)
    th = torch.rand(S, dh // 2, generator=g, device="cuda", dtype=torch.float64) * 6 - 3
    cos_i = th.cos().repeat_interleave(2, dim=1).to(torch.bfloat16).unsqueeze(0)   # [1, S, d] interleaved
    sin_i = th.sin().repeat_interleave(2, dim=1).to(torch.bfloat16).unsqueeze(0)
    P = lambda t, n, dim=-1: Q.interleaved_to_rotate_half(t, dh, dim=dim, n_heads=n)
    qp, kp = P(q, 1), P(k, 1)            # per head: the last dim is one head
    gqp, gkp, cp, sp = P(gq, nh), P(gk, nh), P(cos_i, 1), P(sin_i, 1)
    Q.qk_norm_rope_across_heads(qp, kp, gqp, gkp, cp, sp, eps=1e-6)
    torch.cuda.synchronize()
    # oracle: across-heads norm without rotation, then the interleaved complex rotation, then permute
    ident_c = torch.ones(1, S, dh, dtype=torch.bfloat16, device="cuda")
    ident_s = torch.zeros(1, S, dh, dtype=torch.bfloat16, device="cuda")
    yq, yk = _oracle(q, k, gq, gk, ident_c, ident_s, 1e-6, apply_rope=False)
    cs = cos_i[0].double().cpu().numpy()[:, 0::2]
    sn = sin_i[0].double().cpu().numpy()[:, 0::2]
    rot = cs + 1j * sn                                              # the bf16 table values as a complex factor

    def inter(y):
        z = (y.reshape(S, nh, dh // 2, 2) @ np.array([1, 1j])) * rot[:, None, :]
        return np.stack([z.real, z.imag], -1).reshape(S, nh, dh)
    for name, y, got in (("q", yq, qp), ("k", yk, kp)):
        ref = oracle.interleaved_to_rotate_half(inter(y), dh, axis=-1, n_heads=1)
        check_float(got, ref.reshape(got.shape), f"converted/{name}")
