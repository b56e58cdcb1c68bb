"""Exact pin of the kernel's cache encoders, through the operator.

The parity bar elsewhere allows an int8 code one apart, or an FP8 code one
step apart, where the value lies within 1e-3 of a rounding boundary, and
random inputs almost never land on one. Here every input is a boundary: with a
unit scale and no offset, t is the input value itself on both sides (formula
(3) of the KvRmsNormRopeCache page: x*scale, then + offset when one is given),
so the cache bytes must equal the oracle's codes bit for bit.

Values (exactly representable in the input dtype, drawn from the format
definitions, not from either implementation):
* INT8 (round half to even, then clamp to [-128, 127]): every k + 0.5 for
  k = -131..130, every integer in that range, the input-ulp neighbours of
  each tie, and values far past the clamp;
* FP8 E4M3FN / E5M2 (OCP, round to nearest even, saturating at 448 / 57344):
  every finite code value, every midpoint between adjacent values (subnormal
  ones included), the input-ulp neighbours of each midpoint, the saturation
  edges 448 / 464 and 57344 / 61440 and values beyond them, and signed zeros
  (-0 * 1 is -0: code 0x80).

Paths: V2's v_optional -> ckv cache (part B of V2) and V1's raw rope tail ->
k cache with cos = 1, sin = 0 (part B of V1: the rotation then returns its
inputs exactly), each at 16 rows (one row per wavefront, direct stores) and at
40,000 rows (several rows per wavefront, codes staged per wave in LDS).

A CPU test checks the oracle at the same values against numpy's
round-half-even and torch's FP8 casts.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import check_kv, host

FMT = {"int8": torch.int8, "e4m3fn": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
ORC_FMT = {"e4m3fn": oracle.E4M3FN, "e5m2": oracle.E5M2}


def _representable(x, dtype):
    """The values of x (fp64) that the 16-bit dtype holds exactly."""
    x = np.asarray(x, np.float64)
    back = torch.from_numpy(x).to(dtype).double().numpy()
    return x[back == x]


def _neighbours(x, dtype):
    """Each value's next representable values down and up in the 16-bit dtype."""
    t = torch.from_numpy(np.asarray(x, np.float64)).to(dtype)
    bits = t.view(torch.int16).numpy().view(np.uint16).astype(np.int64)
    mag = bits & 0x7FFF
    out = []
    for step in (-1, 1):
        m = mag + step
        keep = (m > 0) & (m < 0x7C00 if dtype == torch.float16 else m < 0x7F80)
        nb = ((bits & 0x8000) | m)[keep].astype(np.uint16)
        out.append(torch.from_numpy(nb.view(np.int16)).view(dtype).double().numpy())
    return np.concatenate(out)


def _codebook(fmt):
    """Finite values of an FP8 format, decoded by torch."""
    v = torch.arange(256, dtype=torch.uint8).view(FMT[fmt]).double().numpy()
    return np.unique(v[np.isfinite(v)])


def boundary_values(fmt, dtype):
    """The boundary inputs of one cache encoding, as fp64 values exact in dtype
    (signed zeros kept)."""
    if fmt == "int8":
        k = np.arange(-131, 131, dtype=np.float64)
        ties = k + 0.5
        vals = np.concatenate([ties, k, _neighbours(_representable(ties, dtype), dtype),
                               [-1e4, -1000.0, -300.0, -200.0, -129.0, 129.0, 200.0, 300.0, 1000.0, 1e4]])
    else:
        book = _codebook(fmt)
        mids = (book[:-1] + book[1:]) / 2
        top = 448.0 if fmt == "e4m3fn" else 57344.0
        nxt = 464.0 if fmt == "e4m3fn" else 61440.0      # half a step past the largest finite value
        edges = np.array([top, nxt, (top + nxt) / 2, 2 * nxt, 3 * top])
        edges = np.concatenate([edges, -edges])
        vals = np.concatenate([book, mids, _neighbours(_representable(mids, dtype), dtype), edges,
                               _neighbours(_representable(edges, dtype), dtype)])
    vals = _representable(vals, dtype)
    return np.concatenate([vals, [0.0, -0.0]])


def _fill(vals, count):
    """count values cycling through vals (with a shift each period, so that a
    value meets different lanes and chunk positions)."""
    n = len(vals)
    idx = (np.arange(count) + np.arange(count) // n) % n
    return vals[idx]


def make_case(path, fmt, dtype, rows, device):
    """A workload whose quantised cache sees exactly the boundary values."""
    vals = boundary_values(fmt, dtype)
    one = (1.0, 1.0, "ND" if path == "v2" else "D")
    if path == "v2":
        over = dict(batch=1, heads=2, seq=rows // 2, dtype=dtype, k_cache_dtype=dtype, ckv_cache_dtype=FMT[fmt],
                    k_scale=None, k_offset=None, v_scale=one, v_offset=None, block_size=128,
                    block_num=-(-(rows // 2) // 128) + 2, is_output_kv=False, seed=9100)
        d = W.make_kv_cache(W.MLA_V2_SPLIT, device=device, **over)
        v = _fill(vals, d["v"].numel())
        d["v"].copy_(torch.from_numpy(v).to(dtype).reshape(d["v"].shape))
        return d, vals
    over = dict(batch=1, heads=1, seq=rows, dtype=dtype, k_cache_dtype=FMT[fmt], ckv_cache_dtype=dtype,
                k_scale=one, k_offset=None, v_scale=None, v_offset=None, block_size=128,
                block_num=-(-rows // 128) + 2, is_output_kv=False, seed=9200)
    d = W.make_kv_cache(W.MLA_V1_PREFILL, device=device, **over)
    tail = d["kv"][..., 512:]
    tail.copy_(torch.from_numpy(_fill(vals, tail.numel())).to(dtype).reshape(tail.shape))
    d["cos"].fill_(1.0)
    d["sin"].fill_(0.0)
    return d, vals


CASES = [(path, fmt, dt) for path in ("v2", "v1") for fmt in ("int8", "e4m3fn", "e5m2")
         for dt in (torch.bfloat16, torch.float16)]


def _ids(c):
    return f"{c[0]}-{c[1]}-{str(c[2]).split('.')[-1]}"


def test_boundary_values_cover_every_tie():
    """The value sets hold what the pins need (CPU): every int8 tie in f16,
    every FP8 midpoint and code, both saturation edges, signed zeros."""
    v = boundary_values("int8", torch.float16)
    assert set(np.arange(-131, 131) + 0.5) <= set(v)
    for fmt in ("e4m3fn", "e5m2"):
        book = _codebook(fmt)
        v = boundary_values(fmt, torch.bfloat16)
        assert set(book) <= set(v) and set((book[:-1] + book[1:]) / 2) <= set(v)
        assert {448.0, 464.0} <= set(v) if fmt == "e4m3fn" else {57344.0, 61440.0} <= set(v)
        assert np.signbit(v[v == 0]).any() and (~np.signbit(v[v == 0])).any()


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_oracle_codes_at_boundaries(case):
    """The oracle's codes at the boundary values, through the whole operator
    (CPU): int8 equals numpy's round-half-even then clip; FP8 equals torch's
    cast below the largest finite value and saturates at or above it."""
    path, fmt, dtype = case
    d, _ = make_case(path, fmt, dtype, 16, "cpu")
    r = _run_oracle(d)
    name = "ckv_cache" if path == "v2" else "k_cache"
    tkey, ckey = ("c_t", "ckv_cache") if path == "v2" else ("k_t", "k_cache")
    t = r[tkey].reshape(-1)
    codes = r[ckey].reshape(-1, d[name].shape[-1])[_written_rows(d)].reshape(-1)
    src = (d["v"] if path == "v2" else _deinterleave(d["kv"][..., 512:])).double().numpy().reshape(-1)
    np.testing.assert_array_equal(t, src)
    if path == "v2":   # (V1's rotation gives z0*1 - z1*0, which is +0 for z0 = -0 and z1 < 0)
        assert np.array_equal(np.signbit(t), np.signbit(src))
    if fmt == "int8":
        np.testing.assert_array_equal(codes.astype(np.int64), np.clip(np.round(t), -128, 127).astype(np.int64))
    else:
        top = 448.0 if fmt == "e4m3fn" else 57344.0
        small = np.abs(t) < top
        ref = torch.from_numpy(t[small]).to(FMT[fmt]).view(torch.uint8).numpy()
        np.testing.assert_array_equal(codes[small], ref)
        sat = np.where(np.signbit(t[~small]), 0x80, 0) | (0x7E if fmt == "e4m3fn" else 0x7B)
        np.testing.assert_array_equal(codes[~small], sat.astype(np.uint8))


def _deinterleave(z):
    """The rope tail in output order (evens, then odds): the rotation's result
    with cos = 1, sin = 0."""
    return torch.cat([z[..., 0::2], z[..., 1::2]], dim=-1)


def _written_rows(d):
    from tests.parity import cache_rows
    rows = cache_rows(d)
    return rows[rows >= 0]


def _run_oracle(d):
    from tests.parity import run_oracle_kv
    return run_oracle_kv(d)


@pytest.mark.gpu
@pytest.mark.parametrize("rows", [16, 40000])
@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_gpu_codes_at_boundaries_exact(case, rows):
    import qk_rmsnorm_rope_amd as Q
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    path, fmt, dtype = case
    print(f"encoder pin {_ids(case)} rows={rows}", flush=True)
    d, vals = make_case(path, fmt, dtype, rows, "cuda")
    rep, r = check_kv(Q, d, f"encoders-{_ids(case)}-{rows}")
    name = "ckv_cache" if path == "v2" else "k_cache"
    got = host(d[name])
    ref = r[name]
    same = got.view(np.uint8) == ref.view(np.uint8)
    if not same.all():
        width = d[name].shape[-1]
        flat = np.flatnonzero(~same.reshape(-1))
        t = r["c_t" if path == "v2" else "k_t"]
        raise AssertionError(f"{int((~same).sum())} cache bytes differ from the oracle's codes; first at "
                             f"cache row {flat[0] // width}, channel {flat[0] % width}: gpu "
                             f"{got.reshape(-1)[flat[0]]} oracle {ref.reshape(-1)[flat[0]]}; "
                             f"t range [{t.min()}, {t.max()}]")
    print(rep)
