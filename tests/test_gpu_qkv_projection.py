"""GPU parity of qknr_qkv_projection (the QKV GEMM with step a of the
across-heads norm in its epilogue) and of the projection -> apply path.

Cases: a small ragged case (300 rows: two row-tiles, the second partial;
3 column tiles: Q, K and V) with bias; no bias and no sums; FP8 E4M3 operands
with ROW_MX scales (and without scales); MXFP8 operands (one E8M0 scale per
32 values of hidden on both operands; alone and with ROW_MX scales as well,
blocks whose scales span 2^-20..2^20, an all-zero block); the Wan2.2 width
(hidden 5120 -> 15360 columns, 40 + 40 + 40 heads) at 1000 rows with sampled
rows against the oracle, the per-tile sums against fp64 sums of the stored
outputs, and the projection -> apply path against the oracle's across-heads
operator on the stored Q|K; the full S = 75600 case on sampled rows; two runs
bit-identical -- the last two with bf16, FP8 ROW_MX and MXFP8 operands; 16
seeded random shapes (1-1500 rows, hidden up to 1024 bf16 / 2048 FP8 values,
1-4 Q heads with as many or fewer K heads, with or without bias, sums over
Q and K, Q only, or none) and 8 more with MXFP8 operands.

The projection's outputs are checked against the oracle's exact fp64 values
at the bf16 bar; the sums against fp64 sums of the kernel's own stored bf16
outputs (the values the apply pass reads), so each check has one rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import check_dot, check_float, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    import qk_rmsnorm_rope_amd as lib
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return lib


def _codes(t):
    return t.view(torch.uint8).cpu().numpy()


def _oracle_rows(d, rows, with_bias=True, row_scales=False):
    bias = host(d["bias"]) if with_bias else None
    if d["cfg"].operands == "mxfp8":
        sc = dict(a_scale=d["a_scale"].cpu().numpy()[rows], w_scale=d["w_scale"].cpu().numpy()) if row_scales else {}
        _, v = oracle.linear_mx(_codes(d["a8"])[rows], _codes(d["w8"]), d["a_bs"].cpu().numpy()[rows],
                                d["w_bs"].cpu().numpy(), bias=bias, bias_dtype=oracle.BF16, **sc)
        return v
    if d["cfg"].operands == "fp8":
        a8 = d["a8"][torch.as_tensor(rows, device=d["a8"].device)].view(torch.uint8).cpu().numpy()
        _, v = oracle.linear(a8, d["w8"].view(torch.uint8).cpu().numpy(), oracle.E4M3FN, bias=bias,
                             bias_dtype=oracle.BF16, a_scale=d["a_scale"].cpu().numpy()[rows],
                             w_scale=d["w_scale"].cpu().numpy())
        return v
    _, v = oracle.linear(host(d["a"][rows]), host(d["w"]), oracle.BF16, bias=bias)
    return v


def _fp8_magnitude(d, rows, scaled=True):
    """sum_k |a_k w_k| of the FP8 operands (times the scales), per output."""
    a = np.abs(oracle.decode(oracle.E4M3FN, d["a8"].view(torch.uint8).cpu().numpy()[rows]))
    w = np.abs(oracle.decode(oracle.E4M3FN, d["w8"].view(torch.uint8).cpu().numpy()))
    if d["cfg"].operands == "mxfp8":      # each value times its block's scale
        a = a * np.repeat(2.0 ** (d["a_bs"].cpu().numpy()[rows].astype(np.float64) - 127), 32, axis=1)
        w = w * np.repeat(2.0 ** (d["w_bs"].cpu().numpy().astype(np.float64) - 127), 32, axis=1)
        scaled = scaled and "a_scale" in d
    mag = a @ w.T
    if scaled:
        mag *= d["a_scale"].cpu().double().numpy()[rows][:, None] * d["w_scale"].cpu().double().numpy()[None, :]
    return mag


def _check_out(d, got, rows, what):
    ref = _oracle_rows(d, rows)
    if d["cfg"].operands in ("fp8", "mxfp8"):
        check_dot(got, ref, _fp8_magnitude(d, rows), d["cfg"].hidden, what)
    else:
        check_float(got, ref, what)


def _project(Q, d, **kw):
    if d["cfg"].operands == "mxfp8":
        return Q.qkv_projection(d["a8"], d["w8"], d["bias"], a_block_scale=d["a_bs"], w_block_scale=d["w_bs"], **kw)
    if d["cfg"].operands == "fp8":
        return Q.qkv_projection(d["a8"], d["w8"], d["bias"], a_scale=d["a_scale"], w_scale=d["w_scale"], **kw)
    return Q.qkv_projection(d["a"], d["w"], d["bias"], **kw)


def _check_sums(out, sumsq, q_cols, k_cols, what):
    o = out.float().double().cpu().numpy()
    parts = q_cols // 128
    got = sumsq.cpu().double().numpy().reshape(-1, out.shape[0], parts).transpose(0, 2, 1)
    for seg, c0 in ((0, 0), (1, q_cols)):
        if seg == 1 and not k_cols:
            continue
        for p in range(parts):
            ref = (o[:, c0 + p * 128: c0 + (p + 1) * 128] ** 2).sum(1)
            np.testing.assert_allclose(got[seg, p], ref, rtol=1e-5, atol=1e-6, err_msg=f"{what} seg {seg} part {p}")


def _small(seq=300, hidden=256, heads=1, seed=5):
    return W.make_qkv_projection(W.WAN22_QKV_PROJ, device="cuda", seq=seq, hidden=hidden, n_q_heads=heads,
                                 n_k_heads=heads, seed=seed)


def test_small_ragged_with_bias_and_sums(Q):
    d = _small()
    out, s = Q.qkv_projection(d["a"], d["w"], d["bias"], q_cols=128, k_cols=128)
    torch.cuda.synchronize()
    rows = np.arange(300)
    check_float(out, _oracle_rows(d, rows), "small/out")
    _check_sums(out, s, 128, 128, "small")


def test_no_bias_no_sums_and_q_only_sums(Q):
    d = _small(seq=77, hidden=192, heads=2, seed=6)
    out, s = Q.qkv_projection(d["a"], d["w"], None)
    torch.cuda.synchronize()
    assert s is None
    check_float(out, _oracle_rows(d, np.arange(77), with_bias=False), "nobias/out")
    out2, s2 = Q.qkv_projection(d["a"], d["w"], d["bias"], q_cols=256)
    torch.cuda.synchronize()
    assert tuple(s2.shape) == (1, 77, 2)
    _check_sums(out2, s2, 256, 0, "q-only")


def test_fp8_small_ragged_with_scales(Q):
    """FP8 E4M3 operands (K = 256 values = 2 k steps of 128 bytes), per-row and
    per-channel scales, bias, 300 rows."""
    d = W.make_qkv_projection(W.WAN22_QKV_PROJ_FP8, device="cuda", seq=300, hidden=256, n_q_heads=1,
                              n_k_heads=1, seed=8)
    out, s = _project(Q, d, q_cols=128, k_cols=128)
    torch.cuda.synchronize()
    _check_out(d, out, np.arange(300), "fp8-small/out")
    _check_sums(out, s, 128, 128, "fp8-small")
    # without scales the codes are multiplied as they are (sums of up to 256 products of +-448)
    o2, _ = Q.qkv_projection(d["a8"], d["w8"], None)
    torch.cuda.synchronize()
    _, v = oracle.linear(d["a8"].view(torch.uint8).cpu().numpy(), d["w8"].view(torch.uint8).cpu().numpy(),
                         oracle.E4M3FN)
    check_dot(o2, v, _fp8_magnitude(d, np.arange(300), scaled=False), 256, "fp8-small/unscaled")


def test_mxfp8_small_ragged_alone_and_with_row_scales(Q):
    """MXFP8 operands (K = 384 values = 3 k steps, 12 blocks), 300 rows, bias,
    sums; block scales pushed to span 2^-20..2^20 and one all-zero block;
    then the same codes with ROW_MX scales on top of the block scales."""
    d = W.make_qkv_projection(W.WAN22_QKV_PROJ_MXFP8, device="cuda", seq=300, hidden=384, n_q_heads=1,
                              n_k_heads=1, seed=12)
    g = torch.Generator(device="cuda").manual_seed(12)
    d["a_bs"] = (d["a_bs"].int() + torch.randint(-10, 11, d["a_bs"].shape, generator=g, device="cuda")).to(torch.uint8)
    d["w_bs"] = (d["w_bs"].int() + torch.randint(-10, 11, d["w_bs"].shape, generator=g, device="cuda")).to(torch.uint8)
    d["a8"].view(torch.uint8)[7, 64:96] = 0                      # an all-zero block
    out, s = _project(Q, d, q_cols=128, k_cols=128)
    torch.cuda.synchronize()
    rows = np.arange(300)
    _check_out(d, out, rows, "mx-small/out")
    _check_sums(out, s, 128, 128, "mx-small")
    d["a_scale"] = torch.rand(300, generator=g, device="cuda") + 0.5
    d["w_scale"] = torch.rand(384, generator=g, device="cuda") + 0.5
    o2, _ = Q.qkv_projection(d["a8"], d["w8"], d["bias"], a_block_scale=d["a_bs"], w_block_scale=d["w_bs"],
                             a_scale=d["a_scale"], w_scale=d["w_scale"])
    torch.cuda.synchronize()
    check_dot(o2, _oracle_rows(d, rows, row_scales=True), _fp8_magnitude(d, rows), 384, "mx-small/row-scaled")


def test_bf16_with_row_and_channel_scales(Q):
    """bf16 operands with ROW_MX scales (both, either alone), 300 rows (a ragged
    row tile): the epilogue's scaled path. Unit scales must give the unscaled
    output bit for bit (x * 1 * 1 = x in fp32)."""
    d = _small(seq=300, hidden=256, heads=1, seed=15)
    g = torch.Generator(device="cuda").manual_seed(15)
    asc = torch.rand(300, generator=g, device="cuda") + 0.5
    wsc = torch.rand(384, generator=g, device="cuda") + 0.5
    rows = np.arange(300)
    a_h, w_h, b_h = host(d["a"]), host(d["w"]), host(d["bias"])
    for name, sa, sw in (("both", asc, wsc), ("row", asc, None), ("channel", None, wsc)):
        out, s = Q.qkv_projection(d["a"], d["w"], d["bias"], a_scale=sa, w_scale=sw, q_cols=128, k_cols=128)
        torch.cuda.synchronize()
        _, ref = oracle.linear(a_h, w_h, oracle.BF16, bias=b_h, bias_dtype=oracle.BF16,
                               a_scale=None if sa is None else sa.cpu().numpy(),
                               w_scale=None if sw is None else sw.cpu().numpy())
        check_float(out, ref, f"bf16-scaled-{name}/out")
        _check_sums(out, s, 128, 128, f"bf16-scaled-{name}")
    plain, _ = Q.qkv_projection(d["a"], d["w"], d["bias"])
    ones, _ = Q.qkv_projection(d["a"], d["w"], d["bias"], a_scale=torch.ones_like(asc), w_scale=torch.ones_like(wsc))
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), ones.view(torch.int16))


def test_strided_operands_and_output(Q):
    """Row strides larger than the rows: a slice of a wider activation buffer
    and an output written into a wider buffer."""
    d = _small(seq=130, hidden=128, heads=1, seed=7)
    wide = torch.zeros(130, 128 + 64, dtype=torch.bfloat16, device="cuda")
    wide[:, 32:160] = d["a"]
    a = wide[:, 32:160]
    big = torch.full((130, 384 + 128), 7.0, dtype=torch.bfloat16, device="cuda")
    o = big[:, 64:448]
    Q.qkv_projection(a, d["w"], d["bias"], out=o)
    torch.cuda.synchronize()
    check_float(o, _oracle_rows(d, np.arange(130)), "strided/out")
    assert bool((big[:, :64] == 7.0).all()) and bool((big[:, 448:] == 7.0).all())


@pytest.mark.parametrize("mode", ["bf16", "fp8", "mxfp8"])
def test_row_pitch_at_the_limit(Q, mode):
    """A and W with row pitches of exactly 4 MiB (the largest the entry point
    accepts): the tile copies' 32-bit lane offsets then reach ~1.5 GiB within a
    tile, and with FP8 operands the copies a wave issues for its SIMD partner
    (rows 128 or 192 further) ~2.3 GiB before their clamp. 300 rows (a partial
    second row-tile), 384 output columns (a partial tile of the 256-wide MXFP8
    kernel)."""
    cfg = {"bf16": W.WAN22_QKV_PROJ, "fp8": W.WAN22_QKV_PROJ_FP8, "mxfp8": W.WAN22_QKV_PROJ_MXFP8}[mode]
    fp8 = mode != "bf16"
    d = W.make_qkv_projection(cfg, device="cuda", seq=300, hidden=256, n_q_heads=1, n_k_heads=1, seed=19)
    a_src, w_src = (d["a8"], d["w8"]) if fp8 else (d["a"], d["w"])
    pitch = (4 << 20) // a_src.element_size()
    a = torch.empty_strided(tuple(a_src.shape), (pitch, 1), dtype=a_src.dtype, device="cuda")
    w = torch.empty_strided(tuple(w_src.shape), (pitch, 1), dtype=w_src.dtype, device="cuda")
    a.copy_(a_src)
    w.copy_(w_src)
    if mode == "fp8":
        sc = dict(a_scale=d["a_scale"], w_scale=d["w_scale"])
    elif mode == "mxfp8":
        sc = dict(a_block_scale=d["a_bs"], w_block_scale=d["w_bs"])
    else:
        sc = {}
    out, s = Q.qkv_projection(a, w, d["bias"], q_cols=128, k_cols=128, **sc)
    torch.cuda.synchronize()
    _check_out(d, out, np.arange(300), f"pitch-limit/{mode}")
    _check_sums(out, s, 128, 128, "pitch-limit")
    del a, w
    torch.cuda.empty_cache()


_WAN_CFG = {"bf16": W.WAN22_QKV_PROJ, "fp8_row_mx": W.WAN22_QKV_PROJ_FP8, "mxfp8": W.WAN22_QKV_PROJ_MXFP8}


def _wan(seq, mode="bf16"):
    return W.make_qkv_projection(_WAN_CFG[mode], device="cuda", seq=seq)


def _apply(Q, d, out, s):
    nq, nk, hd = 40, 40, 128
    q = out[:, : nq * hd].unflatten(-1, (nq, hd)).unsqueeze(0)
    k = out[:, nq * hd: (nq + nk) * hd].unflatten(-1, (nk, hd)).unsqueeze(0)
    qi, ki = q.clone(), k.clone()
    Q.qk_apply_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], s, eps=d["eps"],
                            q_norm_channels=0)
    torch.cuda.synchronize()
    return qi, ki, q, k


@pytest.mark.parametrize("mode", sorted(_WAN_CFG))
def test_wan_width_projection_sums_and_apply(Q, mode):
    S = 1000
    d = _wan(S, mode)
    out, s = _project(Q, d, q_cols=5120, k_cols=5120)
    torch.cuda.synchronize()
    assert tuple(s.shape) == (2, S, 40)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(S - 8, S),
                                     np.random.default_rng(3).choice(S, 48, replace=False)]))
    _check_out(d, out[torch.as_tensor(rows, device="cuda")], rows, "wan1000/out")
    _check_sums(out, s, 5120, 5120, "wan1000")
    qi, ki, q, k = _apply(Q, d, out, s)
    T = S
    _, _, rq, rk = oracle.qk_norm_rope_across_heads(
        host(qi.reshape(T, -1)), host(ki.reshape(T, -1)), host(d["q_gamma"]), host(d["k_gamma"]),
        host(d["cos"][0]), host(d["sin"][0]), d["eps"], 40, 40, 128, oracle.BF16)
    check_float(q, rq.reshape(q.shape), "wan1000/apply-q")
    check_float(k, rk.reshape(k.shape), "wan1000/apply-k")
    # V columns are the projection's, untouched by the apply pass
    ref = _oracle_rows(d, rows)[:, 10240:]
    got = out[torch.as_tensor(rows, device="cuda"), 10240:]
    if mode != "bf16":
        check_dot(got, ref, _fp8_magnitude(d, rows)[:, 10240:], 5120, "wan1000/v")
    else:
        check_float(got, ref, "wan1000/v")


@pytest.mark.parametrize("mode", sorted(_WAN_CFG))
def test_wan_full_size_sampled_and_deterministic(Q, mode):
    S = 75600
    d = _wan(S, mode)
    out, s = _project(Q, d, q_cols=5120, k_cols=5120)
    out2 = torch.empty_like(out)
    s2 = torch.empty_like(s)
    _project(Q, d, out=out2, q_cols=5120, k_cols=5120, sumsq=s2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(s, s2)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(S - 4, S),
                                     np.random.default_rng(4).choice(S, 24, replace=False)]))
    idx = torch.as_tensor(rows, device="cuda")
    _check_out(d, out[idx], rows, "full/out")
    o = out[idx].float().double().cpu().numpy()
    got = s[:, idx, :].cpu().double().numpy()
    for seg, c0 in ((0, 0), (1, 5120)):
        ref = (o[:, c0: c0 + 5120] ** 2).reshape(len(rows), 40, 128).sum(-1)
        np.testing.assert_allclose(got[seg], ref, rtol=1e-5, atol=1e-6)


def _draw_proj(i):
    """Seeded random projection shapes: rows 1-1500 (ragged 256-row tiles),
    hidden 128-1024 bf16 values (or 128-2048 FP8), 1-4 Q heads and as many or
    fewer K heads of 128, bias or not, sums over Q and K, Q only, or none."""
    rng = np.random.default_rng(9100 + i)
    fp8 = bool(rng.random() < 0.4)
    step = 128 if fp8 else 64                     # one 128-byte k step
    hidden = step * int(rng.integers(2, 17))
    nq = int(rng.integers(1, 5))
    nk = int(rng.choice([nq, max(1, nq - 1), 1]))
    sums = str(rng.choice(["qk", "q", "none"])) if nk == nq else str(rng.choice(["q", "none"]))
    return dict(fp8=fp8, seq=int(rng.integers(1, 1501)), hidden=hidden, n_q=nq, n_k=nk,
                bias=bool(rng.random() < 0.7), sums=sums, seed=9100 + i)


@pytest.mark.parametrize("i", range(16))
def test_random_projection_shapes(Q, i):
    c = _draw_proj(i)
    print(f"case {i}: {c}", flush=True)
    cfg = W.WAN22_QKV_PROJ_FP8 if c["fp8"] else W.WAN22_QKV_PROJ
    d = W.make_qkv_projection(cfg, device="cuda", seq=c["seq"], hidden=c["hidden"], n_q_heads=c["n_q"],
                              n_k_heads=c["n_k"], seed=c["seed"])
    q_cols = 128 * c["n_q"] if c["sums"] != "none" else 0
    k_cols = 128 * c["n_k"] if c["sums"] == "qk" else 0
    if not c["bias"]:
        d["bias"] = None
    out, s = _project(Q, d, q_cols=q_cols, k_cols=k_cols)
    torch.cuda.synchronize()
    rows = np.arange(c["seq"])
    ref = _oracle_rows(d, rows, with_bias=c["bias"])
    if c["fp8"]:
        check_dot(out, ref, _fp8_magnitude(d, rows), c["hidden"], f"random-{i}/out")
    else:
        check_float(out, ref, f"random-{i}/out")
    if q_cols:
        _check_sums(out, s, q_cols, k_cols, f"random-{i}")
    else:
        assert s is None


def _draw_mx(i):
    """Seeded random MXFP8 shapes: rows 1-1500, hidden 128-2048 FP8 values,
    1-4 Q heads and as many or fewer K heads, bias or not, sums or not."""
    rng = np.random.default_rng(9300 + i)
    nq = int(rng.integers(1, 5))
    nk = int(rng.choice([nq, max(1, nq - 1), 1]))
    return dict(seq=int(rng.integers(1, 1501)), hidden=128 * int(rng.integers(1, 17)), n_q=nq, n_k=nk,
                bias=bool(rng.random() < 0.7), sums=nk == nq and bool(rng.random() < 0.7), seed=9300 + i)


@pytest.mark.parametrize("i", range(8))
def test_random_mxfp8_shapes(Q, i):
    c = _draw_mx(i)
    print(f"mx case {i}: {c}", flush=True)
    d = W.make_qkv_projection(W.WAN22_QKV_PROJ_MXFP8, device="cuda", seq=c["seq"], hidden=c["hidden"],
                              n_q_heads=c["n_q"], n_k_heads=c["n_k"], seed=c["seed"])
    if not c["bias"]:
        d["bias"] = None
    q_cols, k_cols = (128 * c["n_q"], 128 * c["n_k"]) if c["sums"] else (0, 0)
    out, s = _project(Q, d, q_cols=q_cols, k_cols=k_cols)
    torch.cuda.synchronize()
    rows = np.arange(c["seq"])
    check_dot(out, _oracle_rows(d, rows, with_bias=c["bias"]), _fp8_magnitude(d, rows), c["hidden"],
              f"mx-random-{i}/out")
    if q_cols:
        _check_sums(out, s, q_cols, k_cols, f"mx-random-{i}")
