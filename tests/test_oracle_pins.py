"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: the pages' formulas
worked by hand (tests/golden/*.json, each with its citation), closed forms of
RMSNorm and RoPE, library special cases (torch's fp64 rms_norm, complex
multiplication, torch's and numpy's RNE casts), exhaustive format codebooks,
and an independent pure-Python brute force (tests/brute.py) on tiny inputs.
"""
import json
import math
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _across(x, gamma, cos, sin, nh, d, eps, norm=True, rope=True):
    """Run the oracle on fp64 storage (F64 keeps the exact values)."""
    T = x.shape[0]
    _, _, qv, _ = oracle.qk_norm_rope_across_heads(
        np.asarray(x, np.float64).reshape(T, nh * d), None,
        np.asarray(gamma, np.float64), None, np.asarray(cos, np.float64).reshape(T, d),
        np.asarray(sin, np.float64).reshape(T, d), eps, nh, 0, d, oracle.F64,
        apply_norm=norm, apply_rope=rope, nthreads=1)
    return qv


# ---------------------------------------------------------------- (a) hand cases

def test_across_heads_golden_hand_cases():
    for c in _golden("across_heads_hand.json")["cases"]:
        nh, d = c["n_heads"], c["d"]
        out = _across(np.array([c["x"]], float), c["gamma"], [c["cos"]], [c["sin"]], nh, d, c["eps"])
        np.testing.assert_allclose(out[0], c["out"], rtol=0, atol=1e-14)


def test_across_heads_rms_closed_form():
    # gamma = 1, cos = 1, sin = 0: the output row's RMS is 1/sqrt(1 + eps/ms)
    rng = np.random.default_rng(0)
    for eps in (0.0, 1e-6, 0.3, 2.0):
        nh, d = 5, 8
        x = rng.standard_normal((7, nh * d)) * rng.uniform(0.1, 3.0, (7, 1))
        out = _across(x, np.ones(nh * d), np.ones((7, d)), np.zeros((7, d)), nh, d, eps)
        ms = (x ** 2).mean(axis=1)
        rms_out = np.sqrt((out ** 2).mean(axis=1))
        np.testing.assert_allclose(rms_out, 1 / np.sqrt(1 + eps / ms), rtol=1e-13)


def test_across_heads_one_statistic_for_all_heads():
    # heads of very different scale keep their ratio: the statistic spans heads
    nh, d = 4, 6
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, nh * d))
    x[:, :d] *= 100.0
    out = _across(x, np.ones(nh * d), np.ones((3, d)), np.zeros((3, d)), nh, d, 0.0)
    np.testing.assert_allclose(out / x, np.broadcast_to(out[:, :1] / x[:, :1], x.shape), rtol=1e-12)


def test_across_heads_matches_torch_rms_norm_and_complex_rotation():
    # Library special case: torch's fp64 rms_norm over the whole segment, then
    # rotate-half RoPE written as complex multiplication (y_i + i*y_{i+d/2}) e^{i*theta}
    # with the standard table cos_i = cos_{i+d/2}.
    rng = np.random.default_rng(2)
    T, nh, d, eps = 9, 3, 16, 1e-5
    x = rng.standard_normal((T, nh * d))
    g = rng.uniform(0.5, 1.5, nh * d)
    theta = rng.uniform(-4, 4, (T, d // 2))
    cos = np.cos(np.concatenate([theta, theta], 1))
    sin = np.sin(np.concatenate([theta, theta], 1))
    out = _across(x, g, cos, sin, nh, d, eps)
    y = torch.nn.functional.rms_norm(torch.from_numpy(x), [nh * d], torch.from_numpy(g), eps)
    y = y.reshape(T, nh, d)
    z = torch.complex(y[..., : d // 2], y[..., d // 2:]) * torch.polar(
        torch.ones(T, 1, d // 2, dtype=torch.float64), torch.from_numpy(theta)[:, None, :])
    ref = torch.cat([z.real, z.imag], -1).reshape(T, nh * d).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_across_heads_identity_and_pair_norms():
    rng = np.random.default_rng(3)
    T, nh, d, eps = 5, 2, 8, 1e-6
    x = rng.standard_normal((T, nh * d))
    g = rng.uniform(0.5, 1.5, nh * d)
    normed = _across(x, g, np.ones((T, d)), np.zeros((T, d)), nh, d, eps)
    # cos = 1, sin = 0 leaves the normed input unchanged
    no_rope = _across(x, g, np.zeros((T, d)), np.zeros((T, d)), nh, d, eps, rope=False)
    np.testing.assert_allclose(normed, no_rope, rtol=1e-15)
    # rotation preserves |(y_i, y_{i+d/2})| when cos_i = cos_{i+d/2} and cos^2 + sin^2 = 1
    th = rng.uniform(-3, 3, (T, d // 2))
    out = _across(x, g, np.cos(np.hstack([th, th])), np.sin(np.hstack([th, th])), nh, d, eps)
    a, b = normed.reshape(T, nh, 2, d // 2), out.reshape(T, nh, 2, d // 2)
    np.testing.assert_allclose((b ** 2).sum(2), (a ** 2).sum(2), rtol=1e-12)


def test_across_heads_rotate_half_equals_permuted_interleaved():
    # The caller's offline conversion: interleaved-lane RoPE (pairs 2j, 2j+1,
    # complex form) on x equals rotate-half RoPE on the permuted lanes.
    rng = np.random.default_rng(4)
    T, nh, d = 4, 3, 8
    x = rng.standard_normal((T, nh * d))
    th = rng.uniform(-3, 3, (T, d // 2))
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    xp = x.reshape(T, nh, d)[:, :, perm].reshape(T, nh * d)
    out = _across(xp, np.ones(nh * d), np.cos(np.hstack([th, th])), np.sin(np.hstack([th, th])),
                  nh, d, 0.0, norm=False)
    z = (x.reshape(T, nh, d // 2, 2) @ np.array([1, 1j])) * np.exp(1j * th)[:, None, :]
    inter = np.stack([z.real, z.imag], -1).reshape(T, nh, d)     # interleaved output lanes
    np.testing.assert_allclose(out.reshape(T, nh, d), inter[:, :, perm], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- (a) per head, split, permutation

def _qk(x, g, cos, sin, nh, d, eps, **kw):
    qv = oracle.qk_norm_rope(np.asarray(x, np.float64), None, np.asarray(g, np.float64), None,
                             np.asarray(cos, np.float64), np.asarray(sin, np.float64), eps, nh, 0, d,
                             oracle.F64, nthreads=1, **kw)[2]
    return qv


def test_per_head_golden_hand_cases():
    for c in _golden("across_heads_hand.json")["per_head_cases"]:
        out = _qk([c["x"]], c["gamma"], [c["cos"]], [c["sin"]], c["n_heads"], c["d"], c["eps"], per_head=True)
        np.testing.assert_allclose(out[0], c["out"], rtol=0, atol=1e-14)


def test_per_head_matches_torch_rms_norm_per_head_and_complex_rotation():
    rng = np.random.default_rng(12)
    T, nh, d, eps = 7, 4, 16, 1e-6
    x = rng.standard_normal((T, nh * d)) * rng.uniform(0.1, 10, (1, nh * d))
    g = rng.uniform(0.5, 1.5, d)
    theta = rng.uniform(-4, 4, (T, d // 2))
    out = _qk(x, g, np.cos(np.hstack([theta, theta])), np.sin(np.hstack([theta, theta])), nh, d, eps,
              per_head=True)
    y = torch.nn.functional.rms_norm(torch.from_numpy(x).reshape(T, nh, d), [d], torch.from_numpy(g), eps)
    z = torch.complex(y[..., : d // 2], y[..., d // 2:]) * torch.polar(
        torch.ones(T, 1, d // 2, dtype=torch.float64), torch.from_numpy(theta)[:, None, :])
    ref = torch.cat([z.real, z.imag], -1).reshape(T, nh * d).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_per_head_closed_form_and_one_head_equals_across():
    rng = np.random.default_rng(13)
    T, nh, d, eps = 5, 3, 8, 0.25
    x = rng.standard_normal((T, nh * d)) * rng.uniform(0.1, 5, (T, nh * d))
    out = _qk(x, np.ones(d), np.ones((T, d)), np.zeros((T, d)), nh, d, eps, per_head=True)
    ms = (x.reshape(T, nh, d) ** 2).mean(-1)
    rms_out = np.sqrt((out.reshape(T, nh, d) ** 2).mean(-1))
    np.testing.assert_allclose(rms_out, 1 / np.sqrt(1 + eps / ms), rtol=1e-13)
    x1 = x[:, :d]
    g1 = rng.uniform(0.5, 1.5, d)
    th = rng.uniform(-3, 3, (T, d))
    a = _qk(x1, g1, np.cos(th), np.sin(th), 1, d, eps, per_head=True)
    b = _qk(x1, g1, np.cos(th), np.sin(th), 1, d, eps)
    np.testing.assert_allclose(a, b, rtol=1e-15, atol=0)


def test_sumsq_brute_force_and_rms_identity():
    rng = np.random.default_rng(14)
    T, nh, d, eps = 6, 3, 4, 1e-3
    x = rng.standard_normal((T, nh * d))
    ss = oracle.qk_sumsq(x, nh, d, oracle.F64)
    for t in range(T):
        assert abs(ss[t] - sum(v * v for v in x[t].tolist())) <= 1e-13 * ss[t]
    # with gamma = 1, cos = 1, sin = 0 the fused operator scales x by 1/sqrt(ss/C + eps)
    out = _qk(x, np.ones(nh * d), np.ones((T, d)), np.zeros((T, d)), nh, d, eps)
    inv = out[:, 0] / x[:, 0]
    np.testing.assert_allclose(inv, 1 / np.sqrt(ss / (nh * d) + eps), rtol=1e-13)


@pytest.mark.parametrize("tp", [2, 4, 5])
def test_split_over_ranks_reproduces_the_fused_operator(tp):
    """Steps a-c of the page with the heads split over tp ranks: each rank's
    sum over its own heads, the sums added (the all-reduce), each rank applying
    with the total over n_heads*d*tp channels -- equals every head on one
    device."""
    rng = np.random.default_rng(20 + tp)
    T, nh, d, eps = 5, 20, 8, 1e-6
    q = rng.standard_normal((T, nh * d))
    k = rng.standard_normal((T, nh * d)) * 3
    gq, gk = rng.uniform(0.5, 1.5, nh * d), rng.uniform(0.5, 1.5, nh * d)
    th = rng.uniform(-3, 3, (T, d // 2))
    cos, sin = np.cos(np.hstack([th, th])), np.sin(np.hstack([th, th]))
    full_q, full_k = oracle.qk_norm_rope(q, k, gq, gk, cos, sin, eps, nh, nh, d, oracle.F64, nthreads=1)[2:]
    lh = nh // tp
    sl = [slice(r * lh * d, (r + 1) * lh * d) for r in range(tp)]
    sq = sum(oracle.qk_sumsq(np.ascontiguousarray(q[:, s]), lh, d, oracle.F64) for s in sl)
    sk = sum(oracle.qk_sumsq(np.ascontiguousarray(k[:, s]), lh, d, oracle.F64) for s in sl)
    for s in sl:
        oq, ok_ = oracle.qk_norm_rope(np.ascontiguousarray(q[:, s]), np.ascontiguousarray(k[:, s]), gq[s], gk[s],
                                      cos, sin, eps, lh, lh, d, oracle.F64, q_sumsq=sq, k_sumsq=sk,
                                      q_channels=nh * d, k_channels=nh * d, nthreads=1)[2:]
        np.testing.assert_allclose(oq, full_q[:, s], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(ok_, full_k[:, s], rtol=1e-13, atol=1e-15)
    # a rank that used only its own sum would be wrong
    own = oracle.qk_norm_rope(np.ascontiguousarray(q[:, sl[0]]), None, gq[sl[0]], None, cos, sin, eps, lh, 0,
                              d, oracle.F64, nthreads=1)[2]
    assert not np.allclose(own, full_q[:, sl[0]], rtol=1e-6)


def test_permutation_closed_form_inverse_and_untouched_lanes():
    np.testing.assert_array_equal(oracle.rotate_half_permutation(8), [0, 2, 4, 6, 1, 3, 5, 7])
    a = np.arange(3 * 26).reshape(3, 26)
    p = oracle.interleaved_to_rotate_half(a, 6, axis=1, first=5, n_heads=3)
    np.testing.assert_array_equal(p[:, :5], a[:, :5])
    np.testing.assert_array_equal(p[:, 23:], a[:, 23:])
    np.testing.assert_array_equal(p[0, 5:23], [5, 7, 9, 6, 8, 10, 11, 13, 15, 12, 14, 16, 17, 19, 21, 18, 20, 22])
    back = oracle.interleaved_to_rotate_half(p, 6, axis=1, first=5, n_heads=3, inverse=True)
    np.testing.assert_array_equal(back, a)
    # a weight [H, I]: permuting output columns permutes the projection's outputs
    rng = np.random.default_rng(15)
    x, w = rng.standard_normal((4, 7)), rng.standard_normal((7, 24))
    wp = oracle.interleaved_to_rotate_half(w, 8, axis=1, first=0, n_heads=2)   # Q|K blocks, V (last 8) untouched
    np.testing.assert_allclose(x @ wp, oracle.interleaved_to_rotate_half(x @ w, 8, first=0, n_heads=2), rtol=1e-13)
    np.testing.assert_array_equal(wp[:, 16:], w[:, 16:])


def test_permutation_makes_rotate_half_equal_interleaved_rope_and_keeps_scores():
    """The offline conversion of [qkv_cte] Design section 2: with q, k, the
    interleaved cos/sin tables (each angle at lanes 2j and 2j+1) and gammas
    permuted, rotate-half RoPE gives the permuted interleaved result, and the
    attention scores q.k per head do not change."""
    rng = np.random.default_rng(16)
    T, nh, d, eps = 5, 3, 8, 1e-6
    q, k = rng.standard_normal((T, nh * d)), rng.standard_normal((T, nh * d))
    gq, gk = rng.uniform(0.5, 1.5, nh * d), rng.uniform(0.5, 1.5, nh * d)
    th = rng.uniform(-3, 3, (T, d // 2))
    cos_i, sin_i = np.repeat(np.cos(th), 2, axis=1), np.repeat(np.sin(th), 2, axis=1)   # interleaved tables

    def interleaved(x, g):
        y = _qk(x, g, np.ones((T, d)), np.zeros((T, d)), nh, d, eps)   # across-heads norm, no rotation
        z = (y.reshape(T, nh, d // 2, 2) @ np.array([1, 1j])) * np.exp(1j * th)[:, None, :]
        return np.stack([z.real, z.imag], -1).reshape(T, nh * d)

    P = lambda a, n=nh: oracle.interleaved_to_rotate_half(a, d, n_heads=n)
    rq = oracle.qk_norm_rope(P(q), P(k), P(gq), P(gk), P(cos_i, 1), P(sin_i, 1), eps, nh, nh, d, oracle.F64,
                             nthreads=1)
    iq, ik = interleaved(q, gq), interleaved(k, gk)
    np.testing.assert_allclose(rq[2], P(iq), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rq[3], P(ik), rtol=1e-12, atol=1e-14)
    s_int = np.einsum("thd,uhd->htu", iq.reshape(T, nh, d), ik.reshape(T, nh, d))
    s_rh = np.einsum("thd,uhd->htu", rq[2].reshape(T, nh, d), rq[3].reshape(T, nh, d))
    np.testing.assert_allclose(s_rh, s_int, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- the projection

def test_linear_golden_hand_cases():
    for c in _golden("linear_hand.json")["cases"]:
        _, v = oracle.linear(np.array(c["A"], float), np.array(c["W"], float), oracle.F64,
                             bias=None if c["bias"] is None else np.array(c["bias"], float),
                             a_scale=c["a_scale"], w_scale=c["w_scale"], nthreads=1)
        np.testing.assert_allclose(v, c["out"], rtol=1e-15, atol=1e-15)


def test_linear_matches_numpy_matmul_and_brute_force():
    rng = np.random.default_rng(30)
    S, H, I = 9, 37, 13
    a = torch.from_numpy(rng.standard_normal((S, H))).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((I, H)) / 6).to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal(I)).to(torch.bfloat16)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    out, v = oracle.linear(bits(a), bits(w), oracle.BF16, bias=bits(b), out_dtype=oracle.BF16, nthreads=2)
    ref = a.double().numpy() @ w.double().numpy().T + b.double().numpy()      # library matmul
    np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-12)
    ad, wd, bd = a.double().tolist(), w.double().tolist(), b.double().tolist()
    for s_ in range(S):
        for i in range(I):
            brute_v = sum(ad[s_][h] * wd[i][h] for h in range(H)) + bd[i]
            assert abs(v[s_, i] - brute_v) <= 1e-12 * (1 + abs(brute_v))
            assert out[s_, i] == brute.encode_nearest("bf16", brute_v)


def test_linear_fp8_row_scaled_and_identity_weight():
    rng = np.random.default_rng(31)
    S, H, I = 5, 16, 7
    ac = rng.integers(0, 256, (S, H)).astype(np.uint8)
    wc = rng.integers(0, 256, (I, H)).astype(np.uint8)
    ac[(ac & 0x7F) == 0x7F] = 0                       # no NaN codes
    wc[(wc & 0x7F) == 0x7F] = 0
    asc, wsc = rng.uniform(0.01, 0.1, S), rng.uniform(0.01, 0.1, I)
    _, v = oracle.linear(ac, wc, oracle.E4M3FN, a_scale=asc, w_scale=wsc, nthreads=1)
    av, wv = oracle.decode(oracle.E4M3FN, ac), oracle.decode(oracle.E4M3FN, wc)
    np.testing.assert_allclose(v, (av @ wv.T) * asc[:, None] * wsc[None, :], rtol=1e-12, atol=1e-12)
    # identity weight plus bias returns the input plus bias exactly
    x = rng.standard_normal((4, 6))
    bias = rng.standard_normal(6)
    _, v = oracle.linear(x, np.eye(6), oracle.F64, bias=bias, nthreads=1)
    np.testing.assert_array_equal(v, x + bias)


def test_linear_mx_golden_hand_cases():
    g = _golden("linear_mx_hand.json")
    for c in g["cases"]:
        bias = None if c["bias"] is None else np.array(c["bias"], np.float64)
        _, v = oracle.linear_mx(np.array(g["A"], np.uint8), np.array(g["W"], np.uint8),
                                np.array(g["a_block_scale"], np.uint8), np.array(g["w_block_scale"], np.uint8),
                                bias=bias, bias_dtype=oracle.F64, a_scale=c["a_scale"], w_scale=c["w_scale"],
                                nthreads=1)
        np.testing.assert_array_equal(v, c["out"])


def _mx_operands(rng, S, H, I):
    ac = rng.integers(0, 256, (S, H)).astype(np.uint8)
    wc = rng.integers(0, 256, (I, H)).astype(np.uint8)
    ac[(ac & 0x7F) == 0x7F] = 0                       # no NaN codes
    wc[(wc & 0x7F) == 0x7F] = 0
    abs_ = rng.integers(110, 140, (S, H // 32)).astype(np.uint8)
    wbs = rng.integers(110, 140, (I, H // 32)).astype(np.uint8)
    return ac, wc, abs_, wbs


def test_linear_mx_matches_dequantised_matmul():
    """Library special case: decode the codes with torch's E4M3 cast, expand
    each block scale over its 32 values with numpy (2.0 ** (e - 127)), then a
    plain fp64 matmul."""
    rng = np.random.default_rng(32)
    S, H, I = 7, 160, 11
    ac, wc, abs_, wbs = _mx_operands(rng, S, H, I)
    asc, wsc = rng.uniform(0.5, 2, S), rng.uniform(0.5, 2, I)
    bias = rng.standard_normal(I)
    _, v = oracle.linear_mx(ac, wc, abs_, wbs, bias=bias, bias_dtype=oracle.F64, a_scale=asc, w_scale=wsc,
                            nthreads=2)
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    ad = dec(ac) * np.repeat(2.0 ** (abs_.astype(np.float64) - 127), 32, axis=1)
    wd = dec(wc) * np.repeat(2.0 ** (wbs.astype(np.float64) - 127), 32, axis=1)
    ref = (ad @ wd.T) * asc[:, None] * wsc[None, :] + bias
    np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_linear_mx_block_exponent_closed_form():
    """Raising one block's E8M0 exponent by one doubles exactly that block's
    share of the sum: the output moves by the block's own partial dot product
    (computed from the oracle with every other block's codes zeroed)."""
    rng = np.random.default_rng(33)
    S, H, I = 3, 128, 4
    ac, wc, abs_, wbs = _mx_operands(rng, S, H, I)
    _, v0 = oracle.linear_mx(ac, wc, abs_, wbs, nthreads=1)
    for blk in range(H // 32):
        only = np.zeros_like(ac)
        only[:, blk * 32:(blk + 1) * 32] = ac[:, blk * 32:(blk + 1) * 32]
        _, part = oracle.linear_mx(only, wc, abs_, wbs, nthreads=1)
        bumped = abs_.copy()
        bumped[:, blk] += 1
        _, v1 = oracle.linear_mx(ac, wc, bumped, wbs, nthreads=1)
        # (fp64 rounding of the two sums: a few ulps of their magnitudes)
        tol = 1e-13 * (np.abs(v0).max() + np.abs(v1).max())
        np.testing.assert_allclose(v1 - v0, part, rtol=0, atol=tol)
        wb = wbs.copy()
        wb[:, blk] += 1
        _, v2 = oracle.linear_mx(ac, wc, abs_, wb, nthreads=1)
        np.testing.assert_allclose(v2 - v0, part, rtol=0, atol=1e-13 * (np.abs(v0).max() + np.abs(v2).max()))
        assert np.abs(part).max() > 1e3 * tol        # the moved share is far above the rounding


def test_linear_mx_brute_force_tiny():
    rng = np.random.default_rng(34)
    S, H, I = 2, 64, 3
    ac, wc, abs_, wbs = _mx_operands(rng, S, H, I)
    bias = torch.from_numpy(rng.standard_normal(I)).to(torch.bfloat16)
    bbits = bias.view(torch.int16).numpy().view(np.uint16)
    out, v = oracle.linear_mx(ac, wc, abs_, wbs, bias=bbits, bias_dtype=oracle.BF16, out_dtype=oracle.BF16,
                              nthreads=1)
    for s_ in range(S):
        for i in range(I):
            acc = 0.0
            for h in range(H):
                acc += (brute.e4m3fn_value(int(ac[s_, h])) * 2.0 ** (int(abs_[s_, h // 32]) - 127) *
                        brute.e4m3fn_value(int(wc[i, h])) * 2.0 ** (int(wbs[i, h // 32]) - 127))
            acc += brute.bf16_value(int(bbits[i]))
            assert abs(v[s_, i] - acc) <= 1e-12 * (1 + abs(acc))
            assert out[s_, i] == brute.encode_nearest("bf16", acc)


def test_across_heads_brute_force_tiny():
    rng = np.random.default_rng(5)
    for (T, nq, nk, d, norm, rope) in [(3, 2, 2, 4, 1, 1), (2, 3, 1, 6, 1, 1), (2, 1, 0, 2, 1, 1),
                                      (2, 2, 2, 8, 0, 1), (2, 2, 3, 4, 1, 0)]:
        q = rng.standard_normal((T, nq * d)).astype(np.float32)
        k = rng.standard_normal((T, nk * d)).astype(np.float32) if nk else None
        gq = rng.uniform(0.5, 1.5, nq * d).astype(np.float32)
        gk = rng.uniform(0.5, 1.5, nk * d).astype(np.float32) if nk else None
        cos = rng.uniform(-1, 1, (T, d)).astype(np.float32)   # deliberately cos_i != cos_{i+d/2}
        sin = rng.uniform(-1, 1, (T, d)).astype(np.float32)
        qo, ko, qv, kv = oracle.qk_norm_rope_across_heads(
            q, k, gq, gk, cos, sin, 1e-3, nq, nk, d, oracle.F32, norm, rope, nthreads=2)
        for t in range(T):
            ref = brute.across_heads([float(v) for v in q[t]], [float(v) for v in gq], cos[t].tolist(),
                                     sin[t].tolist(), nq, d, 1e-3, norm, rope)
            np.testing.assert_allclose(qv[t], ref, rtol=1e-13, atol=1e-15)
            np.testing.assert_array_equal(qo[t], np.array([brute.to_fp32(r) for r in ref], np.float32))
            if nk:
                ref = brute.across_heads([float(v) for v in k[t]], [float(v) for v in gk], cos[t].tolist(),
                                         sin[t].tolist(), nk, d, 1e-3, norm, rope)
                np.testing.assert_allclose(kv[t], ref, rtol=1e-13, atol=1e-15)


def test_across_heads_bf16_output_is_rne_of_exact_value():
    rng = np.random.default_rng(6)
    T, nh, d = 6, 2, 8
    x = torch.randn(T, nh * d, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    g = torch.rand(nh * d).add(0.5).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    th = rng.uniform(-3, 3, (T, d // 2))
    cs = torch.from_numpy(np.cos(np.hstack([th, th]))).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    sn = torch.from_numpy(np.sin(np.hstack([th, th]))).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    qo, _, qv, _ = oracle.qk_norm_rope_across_heads(bits, None, g, None, cs, sn, 1e-6, nh, 0, d, oracle.BF16)
    assert qo.dtype == np.uint16
    expect = [brute.encode_nearest("bf16", float(v)) for v in qv.ravel()]
    np.testing.assert_array_equal(qo.ravel(), np.array(expect, np.uint16))


# ---------------------------------------------------------------- formats

def test_bf16_encoder_matches_torch_for_fp32_inputs():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 3.0e38, -3.0e38, 1e-40, -1e-42]]).astype(np.float32)
    ours = oracle.encode(oracle.BF16, v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_encoder_rounds_once_from_double():
    # 1 + 2^-8 is the midpoint of bf16 1 and 1 + 2^-7 -> even (1.0); a hair above
    # must round up even though fp32 rounding first would land on the midpoint.
    one = 0x3F80
    assert oracle.encode(oracle.BF16, [1 + 2 ** -8])[0] == one
    assert oracle.encode(oracle.BF16, [1 + 2 ** -8 + 2 ** -40])[0] == one + 1
    assert oracle.encode(oracle.BF16, [1 + 3 * 2 ** -8])[0] == one + 2     # tie -> even code
    for x in [1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8 + 2 ** -40), 3.0e-39, 1e300]:
        assert oracle.encode(oracle.BF16, [x])[0] == brute.encode_nearest("bf16", x)


def test_bf16_decode_exhaustive():
    codes = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(oracle.BF16, codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_f16_codec_matches_numpy():
    rng = np.random.default_rng(8)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        [65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -25, 3 * 2.0 ** -26, -0.0]])
    np.testing.assert_array_equal(oracle.encode(oracle.F16, v), v.astype(np.float16).view(np.uint16))
    codes = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours, ref = oracle.decode(oracle.F16, codes), codes.view(np.float16).astype(np.float64)
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_e4m3fn_codebook_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(oracle.E4M3FN, codes)
    for c in range(256):
        bv = brute.e4m3fn_value(c)
        if math.isnan(bv):
            assert math.isnan(vals[c]) and c in (0x7F, 0xFF)
            continue
        assert vals[c] == bv
        assert oracle.encode(oracle.E4M3FN, [bv])[0] == c
    # every midpoint between neighbours goes to the even code; just off it goes nearest
    finite = sorted(brute.e4m3fn_value(c) for c in range(0, 0x7F))
    for lo, hi in zip(finite[:-1], finite[1:]):
        mid = (lo + hi) / 2
        for x in (mid, math.nextafter(mid, 0), math.nextafter(mid, 1e9), -mid):
            assert oracle.encode(oracle.E4M3FN, [x])[0] == brute.encode_nearest("e4m3fn", x, saturate=True), x
    # torch's cast is a library RNE cast below the saturation point
    rng = np.random.default_rng(9)
    t = rng.uniform(-447, 447, 20000) * 10.0 ** rng.integers(-4, 1, 20000)
    ref = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.encode(oracle.E4M3FN, t.astype(np.float32).astype(np.float64)), ref)


def test_e5m2_codebook_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(oracle.E5M2, codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    for c in range(256):
        bv = brute.e5m2_value(c)
        if math.isnan(bv):
            assert math.isnan(vals[c]) and math.isnan(ref[c])
            continue
        assert vals[c] == bv == ref[c], c
        if math.isfinite(bv):
            assert oracle.encode(oracle.E5M2, [bv])[0] == c
    # inf and values past the largest finite saturate (57344 = 0x7B)
    assert oracle.encode(oracle.E5M2, [math.inf])[0] == 0x7B
    assert oracle.encode(oracle.E5M2, [-1e30])[0] == 0xFB
    finite = sorted(brute.e5m2_value(c) for c in range(0, 0x7C))
    for lo, hi in zip(finite[:-1], finite[1:]):
        mid = (lo + hi) / 2
        for x in (mid, math.nextafter(mid, 0), math.nextafter(mid, 1e9), -mid):
            assert oracle.encode(oracle.E5M2, [x])[0] == brute.encode_nearest("e5m2", x, saturate=True), x
    # torch's cast is a library RNE cast below the saturation point
    rng = np.random.default_rng(10)
    t = rng.uniform(-57343, 57343, 20000) * 10.0 ** rng.integers(-8, 1, 20000)
    ref = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.encode(oracle.E5M2, t.astype(np.float32).astype(np.float64)), ref)


def test_quant_golden_hand_cases():
    g = _golden("quant_hand.json")
    for c in g["int8"]:
        res = _run_single_quant(c["x"], c["scale"], c["offset"], oracle.INT8)
        assert int(res) == c["code"], c
        code, _ = brute.quant_code(c["x"], c["scale"], c["offset"], "int8")
        assert code == c["code"]
    for c in g["e4m3fn"]:
        assert oracle.encode(oracle.E4M3FN, [c["t"]])[0] == c["code"], c
        assert brute.encode_nearest("e4m3fn", c["t"], saturate=True) == c["code"]
    for c in g["e5m2"]:
        assert oracle.encode(oracle.E5M2, [c["t"]])[0] == c["code"], c
        assert brute.encode_nearest("e5m2", c["t"], saturate=True) == c["code"], c


def _run_single_quant(x, scale, offset, kdtype):
    # V2 row of width 2 whose rope part is empty is not allowed (rope >= 2), so
    # use a V1 row: rms part = [1,1], rope part = [x, 0] with cos=[1,1], sin=0:
    # rope_out[0] = x exactly, and the k cache code of lane 0 is Quant(x).
    kv = np.array([1.0, 1.0, x, 0.0]).reshape(1, 1, 1, 4)
    one = np.ones(2)
    cos = np.ones((1, 1, 1, 2))
    sin = np.zeros((1, 1, 1, 2))
    kc = np.zeros((1, 1, 1, 2), np.int8)
    cc = np.zeros((1, 1, 1, 2), np.float64)
    r = oracle.kv_rmsnorm_rope_cache(
        kv, None, one, cos, sin, np.array([[0]], np.int64), kc, cc, rms_size=2, rope_size=2,
        eps=0.0, cache_mode=oracle.NORM, in_dtype=oracle.F64, k_dtype=kdtype, ckv_dtype=oracle.F64,
        k_scale=np.array([scale]) if scale is not None else None,
        k_offset=np.array([offset]) if offset is not None else None, nthreads=1)
    return r["k_cache"].ravel()[0]


# ---------------------------------------------------------------- (b) hand cases

def _kv_v1_run(z, cos, sin):
    R = len(z)
    kv = np.concatenate([[1.0, 1.0], z]).reshape(1, 1, 1, 2 + R)
    r = oracle.kv_rmsnorm_rope_cache(
        kv, None, np.ones(2), np.array(cos, float).reshape(1, 1, 1, R),
        np.array(sin, float).reshape(1, 1, 1, R), np.array([[0]], np.int64),
        np.zeros((1, 1, 1, R)), np.zeros((1, 1, 1, 2)), rms_size=2, rope_size=R, eps=0.0,
        cache_mode=oracle.NORM, in_dtype=oracle.F64, k_dtype=oracle.F64, ckv_dtype=oracle.F64,
        is_output_kv=True, nthreads=1)
    return r


def test_interleave_rope_golden_hand_cases():
    for c in _golden("interleave_rope_hand.json")["cases"]:
        r = _kv_v1_run(c["z"], c["cos"], c["sin"])
        np.testing.assert_array_equal(r["k_x"].ravel(), c["out"])
        np.testing.assert_array_equal(r["k_cache"].ravel(), c["out"])
        np.testing.assert_array_equal(r["k_rope"].ravel(), c["out"])
        assert brute.interleave_rope(c["z"], c["cos"], c["sin"]) == c["out"]


def test_interleave_rope_is_rotate_half_of_even_odd_permutation_and_complex():
    rng = np.random.default_rng(10)
    R = 16
    z = rng.standard_normal(R)
    th = rng.uniform(-3, 3, R // 2)
    cos, sin = np.cos(np.hstack([th, th])), np.sin(np.hstack([th, th]))
    out = _kv_v1_run(z, cos, sin)["k_x"].ravel()
    pz = np.concatenate([z[0::2], z[1::2]])
    rot = np.concatenate([-pz[R // 2:], pz[: R // 2]])
    np.testing.assert_allclose(out, pz * cos + rot * sin, rtol=1e-14, atol=1e-15)
    w = (z[0::2] + 1j * z[1::2]) * np.exp(1j * th)
    np.testing.assert_allclose(out, np.concatenate([w.real, w.imag]), rtol=1e-13, atol=1e-15)
    # cos = 1, sin = 0 gives the even/odd permutation of z, not z itself
    np.testing.assert_array_equal(_kv_v1_run(z, np.ones(R), np.zeros(R))["k_x"].ravel(), pz)


def test_kv_rmsnorm_matches_torch_rms_norm_closed_form():
    rng = np.random.default_rng(11)
    D, R, eps = 12, 4, 1e-5
    kv = rng.standard_normal((2, 1, 3, D + R))
    g = rng.uniform(0.5, 1.5, D)
    r = oracle.kv_rmsnorm_rope_cache(
        kv, None, g, np.ones((2, 1, 3, R)), np.zeros((2, 1, 3, R)),
        np.array([[0, 1, 2], [2, 1, 0]], np.int64), np.zeros((2, 1, 3, R)), np.zeros((2, 1, 3, D)),
        rms_size=D, rope_size=R, eps=eps, cache_mode=oracle.NORM, in_dtype=oracle.F64,
        k_dtype=oracle.F64, ckv_dtype=oracle.F64, nthreads=1)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(kv[..., :D]), [D], torch.from_numpy(g), eps).numpy()
    np.testing.assert_allclose(r["c_x"], ref, rtol=1e-13)
    # gamma = 1: RMS of the normed row is 1/sqrt(1 + eps/ms)
    r1 = oracle.kv_rmsnorm_rope_cache(
        kv, None, np.ones(D), np.ones((2, 1, 3, R)), np.zeros((2, 1, 3, R)),
        np.array([[0, 1, 2], [2, 1, 0]], np.int64), np.zeros((2, 1, 3, R)), np.zeros((2, 1, 3, D)),
        rms_size=D, rope_size=R, eps=0.5, cache_mode=oracle.NORM, in_dtype=oracle.F64,
        k_dtype=oracle.F64, ckv_dtype=oracle.F64, nthreads=1)
    ms = (kv[..., :D] ** 2).mean(-1)
    np.testing.assert_allclose(np.sqrt((r1["c_x"] ** 2).mean(-1)), 1 / np.sqrt(1 + 0.5 / ms), rtol=1e-13)


def test_scatter_golden_norm_and_pa():
    g = _golden("scatter_hand.json")
    # Norm
    c = g["norm"]
    B, S, N, Sc, R = c["B"], c["S"], c["N"], c["Scache"], 2
    kv = np.arange(B * N * S * (2 + R), dtype=float).reshape(B, N, S, 2 + R) + 1.0
    pre_k = np.full((B, N, Sc, R), -7.0)
    pre_c = np.full((B, N, Sc, 2), -7.0)
    r = oracle.kv_rmsnorm_rope_cache(
        kv, None, np.ones(2), np.ones((B, N, S, R)), np.zeros((B, N, S, R)),
        np.array(c["index"], np.int64), pre_k, pre_c, rms_size=2, rope_size=R, eps=0.0,
        cache_mode=oracle.NORM, in_dtype=oracle.F64, k_dtype=oracle.F64, ckv_dtype=oracle.F64, nthreads=1)
    written = set()
    for b, s, n, row in c["written"]:
        written.add((b, n, row))
        np.testing.assert_array_equal(r["k_cache"][b, n, row], r["k_x"][b, n, s])
        np.testing.assert_array_equal(r["ckv_cache"][b, n, row], r["c_x"][b, n, s])
    for b in range(B):
        for n in range(N):
            for row in range(Sc):
                if (b, n, row) not in written:
                    assert (r["k_cache"][b, n, row] == -7).all() and (r["ckv_cache"][b, n, row] == -7).all()
    # PA_BNSD
    c = g["pa_bnsd"]
    B, S, N, bs, nb = c["B"], c["S"], c["N"], c["block_size"], c["block_num"]
    kv = np.arange(B * N * S * (2 + R), dtype=float).reshape(B, N, S, 2 + R) + 1.0
    pre_k = np.full((nb, bs, N, R), -7.0)
    pre_c = np.full((nb, bs, N, 2), -7.0)
    r = oracle.kv_rmsnorm_rope_cache(
        kv, None, np.ones(2), np.ones((B, N, S, R)), np.zeros((B, N, S, R)),
        np.array(c["index"], np.int64), pre_k, pre_c, rms_size=2, rope_size=R, eps=0.0,
        cache_mode=oracle.PA_BNSD, in_dtype=oracle.F64, k_dtype=oracle.F64, ckv_dtype=oracle.F64,
        block_size=bs, nthreads=1)
    written = set()
    for b, s, n, blk, off in c["written"]:
        written.add((blk, off, n))
        np.testing.assert_array_equal(r["k_cache"][blk, off, n], r["k_x"][b, n, s])
        np.testing.assert_array_equal(r["ckv_cache"][blk, off, n], r["c_x"][b, n, s])
    untouched = [(i, j, n) for i in range(nb) for j in range(bs) for n in range(N) if (i, j, n) not in written]
    for i, j, n in untouched:
        assert (r["k_cache"][i, j, n] == -7).all() and (r["ckv_cache"][i, j, n] == -7).all()


@pytest.mark.parametrize("key", ["pa_blk_bnsd", "pa_blk_bnsd_unaligned"])
def test_scatter_golden_pa_blk(key):
    c = _golden("scatter_hand.json")[key]
    B, S, N, bs, nb, R = c["B"], c["S"], c["N"], c["block_size"], c["block_num"], 2
    kv = np.arange(B * N * S * (2 + R), dtype=float).reshape(B, N, S, 2 + R) + 1.0
    pre_k = np.full((nb, bs, N, R), -7.0)
    pre_c = np.full((nb, bs, N, 2), -7.0)
    r = oracle.kv_rmsnorm_rope_cache(
        kv, None, np.ones(2), np.ones((B, N, S, R)), np.zeros((B, N, S, R)),
        np.array(c["index"], np.int64), pre_k, pre_c, rms_size=2, rope_size=R, eps=0.0,
        cache_mode=oracle.PA_BLK_BNSD, in_dtype=oracle.F64, k_dtype=oracle.F64, ckv_dtype=oracle.F64,
        block_size=bs, nthreads=1)
    written = set()
    for b, s, n, blk, off in c["written"]:
        written.add((blk, off, n))
        np.testing.assert_array_equal(r["k_cache"][blk, off, n], r["k_x"][b, n, s])
        np.testing.assert_array_equal(r["ckv_cache"][blk, off, n], r["c_x"][b, n, s])
    for i in range(nb):
        for j in range(bs):
            for n in range(N):
                if (i, j, n) not in written:
                    assert (r["k_cache"][i, j, n] == -7).all() and (r["ckv_cache"][i, j, n] == -7).all()


def test_pa_blk_with_block_size_one_is_pa_bnsd():
    """With runs of one token the block starts are per-token slots: PA_BLK_BNSD
    reduces to PA_BNSD (a special case the constraint table's two rows share)."""
    B, N, S, R = 2, 1, 3, 2
    kv = np.random.default_rng(3).standard_normal((B, N, S, 2 + R))
    idx = np.array([4, -1, 0, 5, 2, 1], np.int64)
    outs = []
    for mode in (oracle.PA_BNSD, oracle.PA_BLK_BNSD):
        outs.append(oracle.kv_rmsnorm_rope_cache(
            kv, None, np.ones(2), np.ones((B, N, S, R)), np.zeros((B, N, S, R)), idx,
            np.zeros((6, 1, N, R)), np.zeros((6, 1, N, 2)), rms_size=2, rope_size=R, eps=1e-6,
            cache_mode=mode, in_dtype=oracle.F64, k_dtype=oracle.F64, ckv_dtype=oracle.F64,
            block_size=1, nthreads=1))
    np.testing.assert_array_equal(outs[0]["k_cache"], outs[1]["k_cache"])
    np.testing.assert_array_equal(outs[0]["ckv_cache"], outs[1]["ckv_cache"])


def test_kv_slot_past_the_cache_writes_nothing():
    """Each cache is the leading part of a larger buffer; the rest is a guard
    region that a write past the cache would land in."""
    kv = np.ones((1, 1, 2, 4))
    for mode, idx, buf_shape in ((oracle.NORM, [[3, 0]], (2, 1, 3, 2)), (oracle.PA_BNSD, [6, 1], (4, 2, 1, 2))):
        kbuf, cbuf = np.full(buf_shape, 5.0), np.full(buf_shape, 5.0)
        oracle.kv_rmsnorm_rope_cache(
            kv, None, np.ones(2), np.ones((1, 1, 2, 2)), np.zeros((1, 1, 2, 2)), np.array(idx, np.int64),
            kbuf[:buf_shape[0] - 1], cbuf[:buf_shape[0] - 1], rms_size=2, rope_size=2, eps=0.0,
            cache_mode=mode, in_dtype=oracle.F64, k_dtype=oracle.F64, ckv_dtype=oracle.F64,
            block_size=0 if mode == oracle.NORM else 2, nthreads=1, copy_caches=False)
        assert (kbuf[-1] == 5).all() and (cbuf[-1] == 5).all(), "wrote past the cache"
        assert (kbuf != 5).sum() == 2 and (cbuf != 5).sum() == 2     # only the in-range token


# ---------------------------------------------------------------- (b) brute force

def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype in (torch.bfloat16, torch.float16) else t.numpy()


KV_CASES = [
    # (name, V2?, mode, k fmt, ckv fmt, k quant (scale kind, offset?), v quant, out_kv)
    ("v1_pa_bf16_out", False, "pa", "bf16", "bf16", None, None, True),
    ("v1_norm_int8_e4m3", False, "norm", "int8", "e4m3fn", ("D", False), ("D", False), False),
    ("v1_pa_int8_scalar", False, "pa", "int8", "int8", ("1", False), ("1D", False), True),
    ("v2_pa_int8_asym", True, "pa", "int8", "int8", ("ND", True), ("ND", True), True),
    ("v2_norm_bf16", True, "norm", "bf16", "bf16", None, None, True),
    ("v2_pa_mixed", True, "pa", "e4m3fn", "bf16", ("ND", True), None, False),
    ("v1_pablk_e5m2", False, "pablk", "e5m2", "e5m2", ("D", False), ("1D", False), True),
    ("v2_pablk_e5m2_int8", True, "pablk", "int8", "e5m2", ("ND", True), ("ND", False), True),
    ("v1_norm_e5m2", False, "norm", "e5m2", "e4m3fn", ("1", False), ("D", False), False),
]

_FMT = {"bf16": oracle.BF16, "int8": oracle.INT8, "e4m3fn": oracle.E4M3FN, "e5m2": oracle.E5M2}
_NP = {"bf16": np.uint16, "int8": np.int8, "e4m3fn": np.uint8, "e5m2": np.uint8}
_MODE = {"norm": oracle.NORM, "pa": oracle.PA_BNSD, "pablk": oracle.PA_BLK_BNSD}


@pytest.mark.parametrize("case", KV_CASES, ids=[c[0] for c in KV_CASES])
def test_kv_brute_force_tiny(case):
    name, v2, mode, kf, cf, kq, vq, out_kv = case
    g = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    B, N, S = 2, (2 if v2 else 1), 3
    R = 4
    Dkv = 10 if v2 else 8 + R
    rms = Dkv if v2 else 8
    Dv = 6 if v2 else 0
    kv = torch.randn(B, N, S, Dkv, generator=g).to(torch.bfloat16)
    v = torch.randn(B, N, S, Dv, generator=g).to(torch.bfloat16) if v2 else None
    gamma = (torch.rand(rms, generator=g) + 0.5).to(torch.bfloat16)
    th = torch.rand(B, N, S, R // 2, generator=g, dtype=torch.float64) * 6 - 3
    cos = torch.cat([th.cos(), th.cos()], -1).to(torch.bfloat16)
    sin = torch.cat([th.sin(), th.sin()], -1).to(torch.bfloat16)
    dk, dc = (Dkv, Dv) if v2 else (R, rms)

    def qp(spec, width):
        if spec is None:
            return None, None
        kind, off = spec
        shape = {"1": (1,), "D": (width,), "1D": (1, width), "ND": (N, width)}[kind]
        sc = (torch.rand(shape, generator=g) * 30 + 2).numpy().astype(np.float32)
        of = (torch.rand(shape, generator=g) * 20 - 10).numpy().astype(np.float32) if off else None
        return sc, of

    ks, ko = qp(kq, dk)
    vs, vo = qp(vq, dc)
    if mode == "norm":
        Sc = 5
        index = np.array([[4, -1, 0], [1, 4, 2]], np.int64)
        k_cache = np.random.default_rng(1).integers(0, 200, (B, N, Sc, dk)).astype(_NP[kf])
        c_cache = np.random.default_rng(2).integers(0, 200, (B, N, Sc, dc)).astype(_NP[cf])
        bs = 0
    elif mode == "pablk":
        bs, nb = 2, 4
        index = np.array([6, 0, -1, 3], np.int64)     # runs {0,1}, {2} of each batch
        k_cache = np.random.default_rng(1).integers(0, 200, (nb, bs, N, dk)).astype(_NP[kf])
        c_cache = np.random.default_rng(2).integers(0, 200, (nb, bs, N, dc)).astype(_NP[cf])
    else:
        bs, nb = 2, 4
        index = np.array([7, 0, -1, 3, 4, 1], np.int64)
        k_cache = np.random.default_rng(1).integers(0, 200, (nb, bs, N, dk)).astype(_NP[kf])
        c_cache = np.random.default_rng(2).integers(0, 200, (nb, bs, N, dc)).astype(_NP[cf])
    r = oracle.kv_rmsnorm_rope_cache(
        _bits(kv), _bits(v) if v2 else None, _bits(gamma), _bits(cos), _bits(sin), index,
        k_cache, c_cache, rms_size=rms, rope_size=R, eps=1e-5,
        cache_mode=_MODE[mode], in_dtype=oracle.BF16,
        k_dtype=_FMT[kf], ckv_dtype=_FMT[cf], block_size=bs, k_scale=ks, k_offset=ko,
        v_scale=vs, v_offset=vo, is_output_kv=out_kv, nthreads=2)

    def at(p, n, c):
        if p is None:
            return None
        a = np.asarray(p, np.float64)
        if a.ndim == 2:
            a = a[n if a.shape[0] > 1 else 0]
        return float(a[c] if a.size > 1 else a[0])

    kvd = kv.double().numpy()
    vd = v.double().numpy() if v2 else None
    gd = gamma.double().tolist()
    cd, sd = cos.double().numpy(), sin.double().numpy()
    exp_k = k_cache.copy()
    exp_c = c_cache.copy()
    for b in range(B):
        for n in range(N):
            for s in range(S):
                rope_out, csrc = brute.kv_row(kvd[b, n, s].tolist(), vd[b, n, s].tolist() if v2 else None,
                                              gd, cd[b, n, s].tolist(), sd[b, n, s].tolist(), rms, R, 1e-5)
                np.testing.assert_allclose(r["k_x"][b, n, s], rope_out, rtol=1e-13, atol=1e-15)
                np.testing.assert_allclose(r["c_x"][b, n, s], csrc, rtol=1e-13, atol=1e-15)
                slot = brute.token_slot(mode, index.tolist(), b, s, S, bs)
                if out_kv:
                    assert r["k_rope"][b, n, s].tolist() == [brute.encode_nearest("bf16", x) for x in rope_out]
                    assert r["c_kv"][b, n, s].tolist() == [brute.encode_nearest("bf16", x) for x in csrc]
                if slot is None:
                    continue
                row = brute.cache_row_address(mode, b, n, slot, N, 5, bs)
                krow = [brute.quant_code(x, at(ks, n, j), at(ko, n, j), kf)[0] for j, x in enumerate(rope_out)]
                crow = [brute.quant_code(x, at(vs, n, i), at(vo, n, i), cf)[0] for i, x in enumerate(csrc)]
                exp_k.reshape(-1, dk)[row] = np.array(krow).astype(np.int64).astype(exp_k.dtype)
                exp_c.reshape(-1, dc)[row] = np.array(crow).astype(np.int64).astype(exp_c.dtype)
    np.testing.assert_array_equal(r["k_cache"], exp_k)
    np.testing.assert_array_equal(r["ckv_cache"], exp_c)
    if not out_kv:
        assert r["k_rope"] is None and r["c_kv"] is None


def test_kv_index_minus_one_writes_nothing_but_outputs():
    kv = np.ones((1, 1, 2, 6))
    r = oracle.kv_rmsnorm_rope_cache(
        kv, None, np.ones(4), np.ones((1, 1, 2, 2)), np.zeros((1, 1, 2, 2)), np.array([-1, -1], np.int64),
        np.full((2, 2, 1, 2), 5.0), np.full((2, 2, 1, 4), 5.0), rms_size=4, rope_size=2, eps=0.0,
        cache_mode=oracle.PA_BNSD, in_dtype=oracle.F64, k_dtype=oracle.F64, ckv_dtype=oracle.F64,
        block_size=2, is_output_kv=True, nthreads=1)
    assert (r["k_cache"] == 5).all() and (r["ckv_cache"] == 5).all()
    np.testing.assert_array_equal(r["c_kv"], np.ones((1, 1, 2, 4)))


def test_oracle_rejects_bad_dims():
    with pytest.raises(ValueError):
        oracle.qk_norm_rope_across_heads(np.zeros((1, 3)), None, np.zeros(3), None, np.zeros((1, 3)),
                                         np.zeros((1, 3)), 0.0, 1, 0, 3, oracle.F64)
