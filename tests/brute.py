"""Pure-Python brute force for tiny cases: a second, independent statement of
both operators, used only to cross-check the fp64 oracle.

It shares nothing with the oracle's C code: the storage encoders here search a
sorted list of every finite value the format can hold (nearest value, ties to
the even code) instead of scaling by powers of two, and the operators are
written as nested loops over Python floats straight from the formulas:

* across-heads RMSNorm + rotate-half RoPE: "Kernel reference: qkv_cte",
  Design sections 1 and 2;
* KvRmsNormRopeCache: formulas (1)-(5) and the cache/index constraint table.
"""
from __future__ import annotations

import bisect
import functools
import math
import struct


# ---------------------------------------------------------------- formats

def bf16_value(code: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (code & 0xFFFF) << 16))[0]


def f16_value(code: int) -> float:
    return struct.unpack("<e", struct.pack("<H", code & 0xFFFF))[0]


def e4m3fn_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1 + m / 8) * 2.0 ** (e - 7)


def e5m2_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 3
    if e == 0x1F:
        return s * math.inf if m == 0 else math.nan
    if e == 0:
        return s * m * 2.0 ** -16
    return s * (1 + m / 4) * 2.0 ** (e - 15)


@functools.lru_cache(maxsize=None)
def _codebook(fmt: str):
    """Sorted (value, code) pairs of every finite non-negative value."""
    if fmt == "bf16":
        codes = range(0, 0x7F80)
        val = bf16_value
    elif fmt == "f16":
        codes = range(0, 0x7C00)
        val = f16_value
    elif fmt == "e4m3fn":
        codes = range(0, 0x7F)
        val = e4m3fn_value
    elif fmt == "e5m2":
        codes = range(0, 0x7C)
        val = e5m2_value
    else:
        raise ValueError(fmt)
    pairs = sorted((val(c), c) for c in codes)
    return [p[0] for p in pairs], [p[1] for p in pairs]


def encode_nearest(fmt: str, x: float, saturate: bool = False) -> int:
    """Nearest representable value, ties to the even code; overflow past the
    largest finite value goes to inf (bf16/f16) or saturates (the FP8 formats)."""
    vals, codes = _codebook(fmt)
    sign = {"bf16": 0x8000, "f16": 0x8000, "e4m3fn": 0x80, "e5m2": 0x80}[fmt]
    neg = math.copysign(1.0, x) < 0
    a = abs(x)
    top = vals[-1]
    if a > top:
        if saturate:
            c = codes[-1]
        else:
            # the next binade's first value would be the overflow target
            ulp = top - vals[-2]
            if a >= top + ulp / 2:
                c = {"bf16": 0x7F80, "f16": 0x7C00}[fmt]
            else:
                c = codes[-1]
        return c | (sign if neg else 0)
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        c = codes[i]
    else:
        lo, hi = vals[i - 1], vals[i]
        dl, dh = a - lo, hi - a
        if dl < dh:
            c = codes[i - 1]
        elif dh < dl:
            c = codes[i]
        else:
            c = codes[i - 1] if codes[i - 1] % 2 == 0 else codes[i]
    return c | (sign if neg else 0)


def decode(fmt: str, code: int) -> float:
    return {"bf16": bf16_value, "f16": f16_value, "e4m3fn": e4m3fn_value, "e5m2": e5m2_value}[fmt](code)


def to_fp32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def round_half_even(t: float) -> int:
    f = math.floor(t)
    r = t - f
    if r > 0.5:
        return f + 1
    if r < 0.5:
        return f
    return f if f % 2 == 0 else f + 1


# ---------------------------------------------------------------- (a)

def across_heads(x, gamma, cos, sin, n_heads, d, eps, norm=True, rope=True):
    """One token's segment: x, gamma [n_heads*d]; cos, sin [d]. Floats."""
    C = n_heads * d
    if norm:
        ms = sum(v * v for v in x) / C
        inv = 1.0 / math.sqrt(ms + eps)
        y = [x[c] * inv * gamma[c] for c in range(C)]
    else:
        y = list(x)
    out = [0.0] * C
    h = d // 2
    for head in range(n_heads):
        b = head * d
        for i in range(d):
            if not rope:
                out[b + i] = y[b + i]
            elif i < h:
                out[b + i] = y[b + i] * cos[i] - y[b + i + h] * sin[i]
            else:
                out[b + i] = y[b + i] * cos[i] + y[b + i - h] * sin[i]
    return out


# ---------------------------------------------------------------- (b)

def rms_norm(x, gamma, eps):
    n = len(x)
    rms = math.sqrt(sum(v * v for v in x) / n + eps)
    return [x[i] / rms * gamma[i] for i in range(n)]


def interleave_rope(z, cos, sin):
    x1 = z[0::2]
    x2 = z[1::2]
    part1 = x1 + x2
    part2 = [-v for v in x2] + x1
    return [part1[j] * cos[j] + part2[j] * sin[j] for j in range(len(z))]


def quant_code(x, scale, offset, fmt):
    """Returns (code, t). fmt in {"int8", "e4m3fn", "e5m2", "bf16", "f16"}."""
    t = x
    if scale is not None:
        t = t * scale
    if offset is not None:
        t = t + offset
    if fmt == "int8":
        r = round_half_even(to_fp32(t))
        return max(-128, min(127, r)), t
    if fmt in ("e4m3fn", "e5m2"):
        return encode_nearest(fmt, to_fp32(t), saturate=True), t
    return encode_nearest(fmt, t), t


def kv_row(kv_row_vals, v_row_vals, gamma, cos, sin, rms_size, rope_size, eps):
    """Per (b, n, s) row: returns (rope_out, ckv_source)."""
    if v_row_vals is None:  # V1
        y = rms_norm(kv_row_vals[:rms_size], gamma, eps)
        rope_out = interleave_rope(kv_row_vals[rms_size:], cos, sin)
        return rope_out, y
    y = rms_norm(kv_row_vals, gamma, eps)  # V2: whole kv row
    rope = interleave_rope(y[:rope_size], cos, sin)
    return rope + y[rope_size:], list(v_row_vals)


def token_slot(mode, index, b, s, S, block_size):
    """The cache slot of token (b, s), or None when it writes no cache row.

    Norm: index[b][s]; PA_BNSD: index[b*S + s]; PA_BLK_BNSD: the tokens of
    batch b are cut into runs of block_size (the last run may be shorter) and
    run j fills consecutive slots from its start index[b*runs + j].
    """
    if mode == "norm":
        v = index[b][s]
    elif mode == "pa":
        v = index[b * S + s]
    else:
        runs = -(-S // block_size)
        j, k = divmod(s, block_size)
        start = index[b * runs + j]
        v = -1 if start < 0 else start + k
    return None if v < 0 else int(v)


def cache_row_address(mode, b, n, slot, N, Scache, block_size):
    """Row number of the cache row for token (b, ., s) and head n.

    Norm: [B, N, Scache, D] -> (b*N + n)*Scache + slot.
    PA_BNSD, PA_BLK_BNSD: [block_num, block_size, N, D] -> ((slot//bs)*bs + slot%bs)*N + n.
    """
    if mode == "norm":
        return (b * N + n) * Scache + slot
    blk, off = divmod(slot, block_size)
    return (blk * block_size + off) * N + n
