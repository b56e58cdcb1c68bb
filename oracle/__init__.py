"""fp64 CPU oracle for the fused QK / KV RMSNorm + RoPE (+ cache) operators.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it. The product library never imports,
links or calls anything here, and nothing here imports the product package.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, built with gcc by
:func:`build`); this module only marshals numpy arrays (storage bytes in,
storage bytes and exact fp64 values out) and broadcasts the quantisation
parameter shapes [1], [D], [1, D] to [N, D].

Parity pins: every function is checked in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16, F16, INT8, E4M3FN, E5M2 = 0, 1, 2, 3, 4, 5, 6
NORM, PA_BNSD, PA_BLK_BNSD = 0, 1, 2

# numpy storage views: 16-bit floats travel as uint16 bit patterns, fp8 as uint8
STORAGE = {F64: np.float64, F32: np.float32, BF16: np.uint16, F16: np.uint16,
           INT8: np.int8, E4M3FN: np.uint8, E5M2: np.uint8}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math:
    plain IEEE double arithmetic, no contraction on the x86-64 baseline ISA)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # QKNR_ORACLE_LIB points the wrapper at another build of oracle.c (the
        # mutation tests load copies with planted mistakes this way).
        path = os.environ.get("QKNR_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        p, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_decode.argtypes = [i32, p, p, i64]
        lib.oracle_decode.restype = None
        lib.oracle_encode.argtypes = [i32, p, p, i64]
        lib.oracle_encode.restype = None
        lib.oracle_qk_norm_rope_across_heads.argtypes = (
            [i64, i64, i64, i64, i32] + [p] * 6 + [f64, i32, i32] + [p] * 4 + [i32])
        lib.oracle_qk_norm_rope_across_heads.restype = i32
        lib.oracle_qk_norm_rope.argtypes = (
            [i64, i64, i64, i64, i32] + [p] * 6 + [f64, i32, i32, i32, p, p, f64, f64] + [p] * 4 + [i32])
        lib.oracle_qk_norm_rope.restype = i32
        lib.oracle_qk_sumsq.argtypes = [i64, i64, i64, i32, p, p]
        lib.oracle_qk_sumsq.restype = i32
        lib.oracle_linear.argtypes = [i64, i64, i64, i32, p, i32, p, p, i32, p, p, i32, p, p, i32]
        lib.oracle_linear.restype = i32
        lib.oracle_linear_mx.argtypes = [i64, i64, i64, p, p, p, i64, p, i64, p, i32, p, p, i32, p, p, i32]
        lib.oracle_linear_mx.restype = i32
        lib.oracle_kv_rmsnorm_rope_cache.argtypes = (
            [i64] * 7 + [i32] + [p] * 5 + [i64, p, i32, i64, i64, i32, i32, p, p]
            + [p] * 4 + [f64, i32] + [p] * 6 + [i32])
        lib.oracle_kv_rmsnorm_rope_cache.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected storage {np.dtype(dtype)}, got {a.dtype}")
    return a


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def decode(dtype: int, bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values of storage bits of the given type."""
    src = _c(bits, STORAGE[dtype])
    out = np.empty(src.shape, np.float64)
    _load().oracle_decode(dtype, _ptr(src), _ptr(out), src.size)
    return out


def encode(dtype: int, values) -> np.ndarray:
    """Round fp64 values once to the storage type (RNE; the FP8 formats saturating)."""
    src = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(src.shape, STORAGE[dtype])
    _load().oracle_encode(dtype, _ptr(src), _ptr(out), src.size)
    return out


def qk_norm_rope_across_heads(q, k, q_gamma, k_gamma, cos, sin, eps, n_q_heads,
                              n_k_heads, head_dim, dtype, apply_norm=True,
                              apply_rope=True, nthreads=None, values=True):
    """Across-heads RMSNorm + rotate-half RoPE of T tokens.

    q: [T, n_q*d], k: [T, n_k*d] or None, gammas [n*d], cos/sin [T, d], all in
    storage form of ``dtype`` (F32 float32 arrays, BF16/F16 uint16 bits).
    Returns (q_out, k_out, q_val, k_val): encoded outputs and exact fp64 values
    (None when ``values`` is false).
    """
    st = STORAGE[dtype]
    q = _c(q, st)
    T = q.shape[0]
    cq, ck = n_q_heads * head_dim, n_k_heads * head_dim
    assert q.shape == (T, cq)
    k = _c(k, st) if n_k_heads else None
    if k is not None:
        assert k.shape == (T, ck)
    q_gamma, k_gamma = _c(q_gamma, st), _c(k_gamma, st)
    cos, sin = _c(cos, st), _c(sin, st)
    q_out = np.empty((T, cq), st)
    k_out = np.empty((T, ck), st) if k is not None else None
    q_val = np.empty((T, cq), np.float64) if values else None
    k_val = np.empty((T, ck), np.float64) if (k is not None and values) else None
    rc = _load().oracle_qk_norm_rope_across_heads(
        T, n_q_heads, n_k_heads, head_dim, dtype, _ptr(q), _ptr(k), _ptr(q_gamma),
        _ptr(k_gamma), _ptr(cos), _ptr(sin), float(eps), int(bool(apply_norm)),
        int(bool(apply_rope)), _ptr(q_out), _ptr(k_out), _ptr(q_val), _ptr(k_val),
        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the dimensions")
    return q_out, k_out, q_val, k_val


def qk_norm_rope(q, k, q_gamma, k_gamma, cos, sin, eps, n_q_heads, n_k_heads, head_dim,
                 dtype, apply_norm=True, apply_rope=True, per_head=False, q_sumsq=None,
                 k_sumsq=None, q_channels=0, k_channels=0, nthreads=None, values=True):
    """QK RMSNorm + rotate-half RoPE in its three forms:

    * across heads (default): one RMS per token over the whole segment,
      gammas [n*d];
    * per head (``per_head``): one RMS per head over d channels, gammas [d]
      shared by every head;
    * the apply step of a split over ranks: ``q_sumsq``/``k_sumsq`` [T] are the
      summed squares of the whole segment (all ranks) and ``q_channels`` /
      ``k_channels`` its channel count; q/k hold this rank's heads only.

    Arguments otherwise as :func:`qk_norm_rope_across_heads`.
    """
    st = STORAGE[dtype]
    q = _c(q, st)
    T = q.shape[0]
    cq, ck = n_q_heads * head_dim, n_k_heads * head_dim
    assert q.shape == (T, cq)
    k = _c(k, st) if n_k_heads else None
    if k is not None:
        assert k.shape == (T, ck)
    gw = (head_dim, head_dim) if per_head else (cq, ck)
    q_gamma = _c(q_gamma, st)
    k_gamma = _c(k_gamma, st) if n_k_heads else None
    if apply_norm:
        assert q_gamma.size == gw[0] and (k_gamma is None or k_gamma.size == gw[1]), "gamma size"
    cos, sin = _c(cos, st), _c(sin, st)
    qs = _c(q_sumsq, np.float64)
    ks = _c(k_sumsq, np.float64) if n_k_heads else None
    for a in (qs, ks):
        assert a is None or a.shape == (T,)
    q_out = np.empty((T, cq), st)
    k_out = np.empty((T, ck), st) if k is not None else None
    q_val = np.empty((T, cq), np.float64) if values else None
    k_val = np.empty((T, ck), np.float64) if (k is not None and values) else None
    rc = _load().oracle_qk_norm_rope(
        T, n_q_heads, n_k_heads, head_dim, dtype, _ptr(q), _ptr(k), _ptr(q_gamma),
        _ptr(k_gamma), _ptr(cos), _ptr(sin), float(eps), int(bool(apply_norm)),
        int(bool(apply_rope)), int(bool(per_head)), _ptr(qs), _ptr(ks), float(q_channels),
        float(k_channels), _ptr(q_out), _ptr(k_out), _ptr(q_val), _ptr(k_val),
        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the dimensions")
    return q_out, k_out, q_val, k_val


def linear(a, w, a_dtype, w_dtype=None, bias=None, bias_dtype=None, a_scale=None, w_scale=None,
           out_dtype=None, nthreads=None):
    """The projection O = (A @ W^T) * a_scale[:, None] * w_scale[None, :] + bias.

    a: [S, H] storage of ``a_dtype``; w: [I, H] storage of ``w_dtype`` (a linear
    layer's [out, in] weight); bias [I] storage of ``bias_dtype``; scales fp64
    or None. Returns (encoded output in ``out_dtype`` or None, exact fp64 [S, I]).
    """
    w_dtype = a_dtype if w_dtype is None else w_dtype
    a = _c(a, STORAGE[a_dtype])
    w = _c(w, STORAGE[w_dtype])
    S, H = a.shape
    I = w.shape[0]
    assert w.shape == (I, H)
    bias_dtype = a_dtype if bias_dtype is None else bias_dtype
    b = _c(bias, STORAGE[bias_dtype]) if bias is not None else None
    asc = np.ascontiguousarray(a_scale, dtype=np.float64) if a_scale is not None else None
    wsc = np.ascontiguousarray(w_scale, dtype=np.float64) if w_scale is not None else None
    for name, sc, n in (("a_scale", asc, S), ("w_scale", wsc, I)):
        if sc is not None and sc.shape != (n,):
            raise ValueError(f"{name} must have {n} entries")
    out = np.empty((S, I), STORAGE[out_dtype]) if out_dtype is not None else None
    val = np.empty((S, I), np.float64)
    rc = _load().oracle_linear(S, H, I, a_dtype, _ptr(a), w_dtype, _ptr(w), _ptr(b), bias_dtype, _ptr(asc),
                               _ptr(wsc), out_dtype if out_dtype is not None else F64, _ptr(out), _ptr(val),
                               nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return out, val


def linear_mx(a, w, a_block_scale, w_block_scale, bias=None, bias_dtype=BF16, a_scale=None, w_scale=None,
              out_dtype=None, nthreads=None):
    """The projection with MXFP8 operands (OCP MX: E4M3 codes, one E8M0 scale
    per 32 values along H): O = (A*Xa) @ (W*Xw)^T * a_scale * w_scale + bias.

    a: [S, H] E4M3 codes (uint8); w: [I, H] E4M3 codes; a_block_scale [S, H/32],
    w_block_scale [I, H/32] E8M0 bytes (uint8); bias [I] storage of bias_dtype;
    ROW_MX scales fp64 or None. Returns (encoded output or None, exact fp64 [S, I]).
    """
    a = _c(a, np.uint8)
    w = _c(w, np.uint8)
    S, H = a.shape
    I = w.shape[0]
    assert w.shape == (I, H) and H % 32 == 0
    abs_ = _c(a_block_scale, np.uint8)
    wbs = _c(w_block_scale, np.uint8)
    assert abs_.shape == (S, H // 32) and wbs.shape == (I, H // 32)
    b = _c(bias, STORAGE[bias_dtype]) if bias is not None else None
    asc = np.ascontiguousarray(a_scale, dtype=np.float64) if a_scale is not None else None
    wsc = np.ascontiguousarray(w_scale, dtype=np.float64) if w_scale is not None else None
    out = np.empty((S, I), STORAGE[out_dtype]) if out_dtype is not None else None
    val = np.empty((S, I), np.float64)
    rc = _load().oracle_linear_mx(S, H, I, _ptr(a), _ptr(w), _ptr(abs_), H // 32, _ptr(wbs), H // 32, _ptr(b),
                                  bias_dtype, _ptr(asc), _ptr(wsc), out_dtype if out_dtype is not None else F64,
                                  _ptr(out), _ptr(val), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return out, val


def qk_sumsq(x, n_heads, head_dim, dtype):
    """Per-token sum of squares over one segment: x [T, n*d] -> fp64 [T]."""
    x = _c(x, STORAGE[dtype])
    T = x.shape[0]
    assert x.shape == (T, n_heads * head_dim)
    out = np.empty(T, np.float64)
    if _load().oracle_qk_sumsq(T, n_heads, head_dim, dtype, _ptr(x), _ptr(out)) != 0:
        raise ValueError("oracle rejected the dimensions")
    return out


def rotate_half_permutation(head_dim):
    """Lane j of a rotate-half head holds interleaved lane perm[j]: the even
    lanes 0, 2, ..., d-2 first, then the odd lanes 1, 3, ..., d-1, so that the
    interleaved pair (2j, 2j+1) becomes the rotate-half pair (j, j + d/2)."""
    return np.concatenate([np.arange(0, head_dim, 2), np.arange(1, head_dim, 2)])


def interleaved_to_rotate_half(a, head_dim, axis=-1, first=0, n_heads=None, inverse=False):
    """Permute `n_heads` blocks of `head_dim` lanes, starting at index `first`
    of `axis`, from the interleaved-pair layout to the rotate-half layout
    (``inverse``: back). Indices outside those blocks keep their values.
    Returns a new array."""
    a = np.asarray(a)
    axis = axis % a.ndim
    L = a.shape[axis]
    if n_heads is None:
        n_heads = (L - first) // head_dim
    if head_dim % 2 or first < 0 or first + n_heads * head_dim > L:
        raise ValueError("blocks outside the axis, or odd head_dim")
    dst = first + np.arange(n_heads * head_dim)
    src = first + (np.arange(n_heads)[:, None] * head_dim
                   + rotate_half_permutation(head_dim)[None, :]).ravel()
    idx = np.arange(L)
    if inverse:
        idx[src] = dst
    else:
        idx[dst] = src
    return np.take(a, idx, axis=axis)


def _expand_quant(p, heads, width):
    """Broadcast a quantisation parameter of shape [1], [D], [1, D] or [N, D]
    to [N, D] fp64 (the shapes the quant-parameter constraint table allows)."""
    if p is None:
        return None
    a = np.asarray(p, dtype=np.float64)
    if a.ndim == 2 and a.shape[0] not in (1, heads):
        raise ValueError("quant parameter rows must be 1 or N")
    return np.ascontiguousarray(np.broadcast_to(a.reshape((-1,) if a.ndim == 1 else a.shape),
                                                (heads, width)))


def kv_rmsnorm_rope_cache(kv, v, gamma, cos, sin, index, k_cache, ckv_cache, *,
                          rms_size, rope_size, eps, cache_mode, in_dtype, k_dtype,
                          ckv_dtype, block_size=0, k_scale=None, k_offset=None,
                          v_scale=None, v_offset=None, is_output_kv=False,
                          nthreads=None, copy_caches=True):
    """The KvRmsNormRopeCache operator on host arrays.

    kv [B, N, S, Dkv] and v [B, N, S, Dv] (or None for V1), gamma, cos/sin
    [B, N, S or 1, rope] in storage form of ``in_dtype``; index int64 (Norm
    [B, S], PA_BNSD [B*S], PA_BLK_BNSD [B*ceil(S/block_size)] block starts); the
    caches (storage arrays, Norm [B, N, Scache, D] or paged [blocks, bs, N, D]) are
    copied and the copies updated (``copy_caches=False`` updates the given
    C-contiguous arrays in place). Returns a dict with k_cache, ckv_cache,
    k_rope, c_kv (None unless is_output_kv), and the exact values k_x, c_x
    (fed to quantisation) and k_t, c_t (right before rounding).
    """
    st = STORAGE[in_dtype]
    kv = _c(kv, st)
    B, N, S, Dkv = kv.shape
    v = _c(v, st)
    Dv = v.shape[3] if v is not None else 0
    gamma, cos, sin = _c(gamma, st), _c(cos, st), _c(sin, st)
    rope_S = cos.shape[2]
    index = _c(index, np.int64)
    if cache_mode != NORM and block_size < 1:
        raise ValueError("paged caches need block_size >= 1")
    entries = B * (-(-S // block_size) if cache_mode == PA_BLK_BNSD else S)
    if index.size != entries:
        raise ValueError(f"index holds {index.size} entries, the cache mode needs {entries}")
    if copy_caches:
        k_cache = np.array(k_cache, copy=True, order="C")
        ckv_cache = np.array(ckv_cache, copy=True, order="C")
    elif not (k_cache.flags.c_contiguous and ckv_cache.flags.c_contiguous
              and k_cache.flags.writeable and ckv_cache.flags.writeable):
        raise ValueError("in-place caches must be writeable C-contiguous arrays")
    if k_cache.dtype != STORAGE[k_dtype] or ckv_cache.dtype != STORAGE[ckv_dtype]:
        raise TypeError("cache storage does not match its dtype code")
    dk = Dkv if v is not None else rope_size
    dc = Dv if v is not None else rms_size
    if cache_mode == NORM:
        cache_dim0 = k_cache.shape[2]
    else:
        cache_dim0 = k_cache.shape[0]
    ks, ko = _expand_quant(k_scale, N, dk), _expand_quant(k_offset, N, dk)
    vs, vo = _expand_quant(v_scale, N, dc), _expand_quant(v_offset, N, dc)
    k_rope = np.zeros((B, N, S, dk), st) if is_output_kv else None
    c_kv = np.zeros((B, N, S, dc), st) if is_output_kv else None
    k_x = np.empty((B, N, S, dk), np.float64)
    c_x = np.empty((B, N, S, dc), np.float64)
    k_t = np.empty((B, N, S, dk), np.float64)
    c_t = np.empty((B, N, S, dc), np.float64)
    rc = _load().oracle_kv_rmsnorm_rope_cache(
        B, N, S, Dkv, rms_size, rope_size, Dv, in_dtype, _ptr(kv), _ptr(v),
        _ptr(gamma), _ptr(cos), _ptr(sin), rope_S, _ptr(index), cache_mode,
        cache_dim0, block_size, k_dtype, ckv_dtype, _ptr(k_cache), _ptr(ckv_cache),
        _ptr(ks), _ptr(ko), _ptr(vs), _ptr(vo), float(eps), int(bool(is_output_kv)),
        _ptr(k_rope), _ptr(c_kv), _ptr(k_x), _ptr(c_x), _ptr(k_t), _ptr(c_t),
        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the dimensions")
    return dict(k_cache=k_cache, ckv_cache=ckv_cache, k_rope=k_rope, c_kv=c_kv,
                k_x=k_x, c_x=c_x, k_t=k_t, c_t=c_t)
