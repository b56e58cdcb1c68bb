"""Seeded synthetic inputs for the fused QK / KV RMSNorm + RoPE (+ cache) workloads.

This module only draws inputs: random activations, gammas, quantisation scales,
index permutations, cache pre-fill bytes, and the cos/sin position tables that
both operators take as plain input data. It holds none of the operators'
arithmetic (no normalisation, rotation, quantisation or scatter), and it is the
only code shared by the fp64 oracle and the HIP path.

Every tensor comes from a ``torch.Generator`` seeded from the workload's seed,
on the device the caller names: the multi-gigabyte Wan2.2-shaped inputs are
drawn directly in device memory; callers that need host copies (the oracle)
copy the same bytes back.

Shapes and value distributions follow the five workloads:

* ``tiny_across_heads`` -- B=1, S=64, Q and K 4 heads x 64 fp32 ~N(0,1),
  gammas [256] ~U(0.5,1.5), eps 1e-6, rotate-half tables for positions 0..63.
* ``wan22_self_attn`` -- S=75600 = 21x45x80 latent tokens (81 frames at
  720x1280 through the Wan latent-size formula of the context-parallelism page,
  section "Sequence Length Constraints"), Q and K 40 heads x 128 bf16 ~N(0,1),
  gammas [5120] bf16 ~U(0.5,1.5), eps 1e-6, cos/sin [S,128] from 3D (t,h,w)
  positions with the per-head split 44/42/42.
* ``mla_v1_prefill`` -- kv [8,1,4096,576] bf16, bf16 paged caches
  (block_size 128, 320 blocks), is_output_kv.
* ``mla_v1_decode_quant`` -- kv [512,1,1,576], int8 k cache (scale [64]
  ~U(0.01,0.05)), fp8-e4m3fn ckv cache (scale [512] ~U(0.5,2)), Norm caches of
  8192 rows.
* ``mla_v2_split`` -- kv [16,8,2048,192] + v [16,8,2048,128] bf16, int8 caches
  with per-head scale/offset, paged caches (block_size 128, 320 blocks).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

THETA = 10000.0

# Cache / mode names used in the generated dictionaries (plain strings, not an ABI).
NORM = "norm"
PA_BNSD = "pa_bnsd"
PA_BLK_BNSD = "pa_blk_bnsd"


def _gen(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev.type if dev.type != "cuda" else dev)
    g.manual_seed(int(seed))
    return g


def _uniform(shape, lo, hi, g, device, dtype=torch.float32):
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return (u * (hi - lo) + lo).to(dtype)


def _normal(shape, g, device, dtype):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


# ---------------------------------------------------------------------------
# Position tables (input data for both operators)
# ---------------------------------------------------------------------------

def rotate_half_table_1d(positions: torch.Tensor, d: int, theta: float = THETA):
    """cos/sin [len(positions), d] in the rotate-half layout: lanes i and i+d/2
    share the angle pos * theta**(-2i/d), i < d/2 (computed in fp64)."""
    pos = positions.to(torch.float64)
    j = torch.arange(d // 2, device=pos.device, dtype=torch.float64)
    inv = theta ** (-2.0 * j / d)
    ang = pos[:, None] * inv[None, :]
    ang = torch.cat([ang, ang], dim=-1)
    return torch.cos(ang), torch.sin(ang)


def wan_3d_table(frames: int, height: int, width: int, d: int = 128,
                 split=(44, 42, 42), theta: float = THETA, device="cpu"):
    """cos/sin [frames*height*width, d] for Wan-style 3D rotary positions.

    Token s sits at (t, h, w) = (s // (H*W), (s // W) % H, s % W). The head dim is
    split 44/42/42 between the t, h and w axes; axis a with width d_a contributes
    d_a/2 angle pairs pos_a * theta**(-2j/d_a). The 64 angles (t first, then h,
    then w) are laid out rotate-half: lanes p and p+64 share angle p. Only the
    table is built here; the operators take it as input.
    """
    assert sum(split) == d
    s = torch.arange(frames * height * width, device=device, dtype=torch.int64)
    coords = [s // (height * width), (s // width) % height, s % width]
    angs = []
    for c, da in zip(coords, split):
        j = torch.arange(da // 2, device=device, dtype=torch.float64)
        inv = theta ** (-2.0 * j / da)
        angs.append(c.to(torch.float64)[:, None] * inv[None, :])
    ang = torch.cat(angs, dim=-1)
    ang = torch.cat([ang, ang], dim=-1)
    return torch.cos(ang), torch.sin(ang)


# ---------------------------------------------------------------------------
# Across-heads QK workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class AcrossHeadsConfig:
    name: str
    batch: int
    seq: int
    n_q_heads: int
    n_k_heads: int
    head_dim: int
    dtype: torch.dtype
    eps: float
    seed: int
    table: str  # "1d" or "wan3d"
    with_v: bool = False  # allocate a V segment after K (it must stay untouched)
    wan_grid: tuple = (21, 45, 80)


TINY_ACROSS_HEADS = AcrossHeadsConfig(
    name="tiny_across_heads", batch=1, seq=64, n_q_heads=4, n_k_heads=4,
    head_dim=64, dtype=torch.float32, eps=1e-6, seed=1001, table="1d")

WAN22_SELF_ATTN = AcrossHeadsConfig(
    name="wan22_self_attn", batch=1, seq=75600, n_q_heads=40, n_k_heads=40,
    head_dim=128, dtype=torch.bfloat16, eps=1e-6, seed=1002, table="wan3d",
    wan_grid=(21, 45, 80))


def make_across_heads(cfg: AcrossHeadsConfig, device="cpu", **override):
    """Draw one batch of inputs for the across-heads QK norm + RoPE.

    Returns a dict with the BSD activation buffer ``qkv`` [B, S, I] where
    I = (n_q + n_k (+ n_k if with_v)) * d, Q at channel 0 and K at n_q*d,
    the two gammas, cos/sin [B, S, d] (materialised per batch), eps and dims.
    """
    cfg = dataclasses.replace(cfg, **override) if override else cfg
    g = _gen(cfg.seed, device)
    d = cfg.head_dim
    cq, ck = cfg.n_q_heads * d, cfg.n_k_heads * d
    width = cq + ck + (ck if cfg.with_v else 0)
    qkv = _normal((cfg.batch, cfg.seq, width), g, device, cfg.dtype)
    q_gamma = _uniform((cq,), 0.5, 1.5, g, device, cfg.dtype)
    k_gamma = _uniform((ck,), 0.5, 1.5, g, device, cfg.dtype) if ck else None
    if cfg.table == "wan3d":
        f, h, w = cfg.wan_grid
        cos, sin = wan_3d_table(f, h, w, d, device=device)
        n = cos.shape[0]
        if n < cfg.seq:
            raise ValueError("Wan grid smaller than the sequence")
        cos, sin = cos[: cfg.seq], sin[: cfg.seq]
    else:
        cos, sin = rotate_half_table_1d(torch.arange(cfg.seq, device=device), d)
    cos = cos.to(cfg.dtype)[None].expand(cfg.batch, -1, -1).contiguous()
    sin = sin.to(cfg.dtype)[None].expand(cfg.batch, -1, -1).contiguous()
    return dict(cfg=cfg, qkv=qkv, q_gamma=q_gamma, k_gamma=k_gamma, cos=cos,
                sin=sin, eps=cfg.eps, n_q_heads=cfg.n_q_heads,
                n_k_heads=cfg.n_k_heads, head_dim=d)


@dataclasses.dataclass(frozen=True)
class QkvProjectionConfig:
    """The projection that produces Q|K|V ahead of the across-heads norm:
    A [S, hidden] @ W^T with W [(n_q + 2 n_k) * d, hidden], plus bias."""
    name: str
    seq: int
    hidden: int
    n_q_heads: int
    n_k_heads: int
    head_dim: int
    dtype: torch.dtype
    eps: float
    seed: int
    operands: str = "bf16"   # "bf16"; "fp8": E4M3 codes with per-row / per-channel scales (ROW_MX);
    #                           "mxfp8": E4M3 codes with one E8M0 scale per 32 values of hidden (OCP MX)


# Wan2.2-A14B self-attention: hidden 5120, 40 heads of 128 for Q, K and V.
WAN22_QKV_PROJ = QkvProjectionConfig(
    name="wan22_qkv_projection", seq=75600, hidden=5120, n_q_heads=40, n_k_heads=40,
    head_dim=128, dtype=torch.bfloat16, eps=1e-6, seed=1006)
WAN22_QKV_PROJ_FP8 = dataclasses.replace(WAN22_QKV_PROJ, name="wan22_qkv_projection_fp8", seed=1007,
                                         operands="fp8")
WAN22_QKV_PROJ_MXFP8 = dataclasses.replace(WAN22_QKV_PROJ, name="wan22_qkv_projection_mxfp8", seed=1008,
                                           operands="mxfp8")


def quantize_rows_e4m3(x: torch.Tensor):
    """Row-wise FP8 E4M3 quantisation of the operands (what the producer of a
    ROW_MX operand hands over): scale = max|row| / 448, codes = RNE(x / scale).
    Returns (codes as float8_e4m3fn, fp32 scales)."""
    amax = x.float().abs().amax(dim=1).clamp_min(1e-12)
    scale = amax / 448.0
    codes = (x.float() / scale[:, None]).to(torch.float8_e4m3fn)
    return codes, scale.contiguous()


def quantize_mx_e4m3(x: torch.Tensor):
    """MXFP8 conversion of the operands along their last axis (what the
    producer of an MX operand hands over, following the OCP Microscaling
    format's conversion): per block of 32 values, the shared scale is the
    power of two X = 2^(floor(log2(max|block|)) - 8) (8 = the exponent of
    E4M3's largest normal, 448), stored as the E8M0 byte log2(X) + 127; the
    elements are RNE(x / X) in E4M3, clamped to +-448 first (x / X can reach
    just under 512). An all-zero block gets the scale 2^-127. Returns (codes
    as float8_e4m3fn, E8M0 scale bytes as uint8 [..., K/32])."""
    xb = x.float().unflatten(-1, (-1, 32))
    amax = xb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-38))) - 8.0, torch.full_like(amax, -127.0))
    e = e.clamp(-127.0, 127.0)
    codes = (xb / torch.exp2(e)[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).flatten(-2)
    return codes.contiguous(), (e + 127.0).to(torch.uint8).contiguous()


def make_qkv_projection(cfg: QkvProjectionConfig, device="cpu", **override):
    """Draw the projection's operands: activations A [S, hidden] ~ N(0, 1)
    (post-modulation hidden states), weight W [I, hidden] ~ N(0, 1/hidden) so
    that outputs are ~N(0, 1), bias [I] ~ N(0, 0.1^2); plus the norm's gammas
    ~U(0.5, 1.5) and the Wan 3D rotate-half tables for the sequence (1D tables
    when the sequence does not fill the 21x45x80 grid). Draw order: A, W,
    bias, q_gamma, k_gamma."""
    cfg = dataclasses.replace(cfg, **override) if override else cfg
    g = _gen(cfg.seed, device)
    d = cfg.head_dim
    I = (cfg.n_q_heads + 2 * cfg.n_k_heads) * d
    a = _normal((cfg.seq, cfg.hidden), g, device, cfg.dtype)
    w = (torch.randn((I, cfg.hidden), generator=g, device=device) / math.sqrt(cfg.hidden)).to(cfg.dtype)
    bias = (torch.randn((I,), generator=g, device=device) * 0.1).to(cfg.dtype)
    q_gamma = _uniform((cfg.n_q_heads * d,), 0.5, 1.5, g, device, cfg.dtype)
    k_gamma = _uniform((cfg.n_k_heads * d,), 0.5, 1.5, g, device, cfg.dtype)
    if cfg.seq == 21 * 45 * 80:
        cos, sin = wan_3d_table(21, 45, 80, d, device=device)
    else:
        cos, sin = rotate_half_table_1d(torch.arange(cfg.seq, device=device), d)
    d = dict(cfg=cfg, a=a, w=w, bias=bias, q_gamma=q_gamma, k_gamma=k_gamma,
             cos=cos.to(cfg.dtype)[None].contiguous(), sin=sin.to(cfg.dtype)[None].contiguous(),
             eps=cfg.eps, out_features=I)
    if cfg.operands == "fp8":
        # FP8 operands from the same draws, quantised per activation row and per output channel
        d["a8"], d["a_scale"] = quantize_rows_e4m3(a)
        d["w8"], d["w_scale"] = quantize_rows_e4m3(w)
    elif cfg.operands == "mxfp8":
        # MXFP8 operands from the same draws: one E8M0 scale per 32 values along hidden
        d["a8"], d["a_bs"] = quantize_mx_e4m3(a)
        d["w8"], d["w_bs"] = quantize_mx_e4m3(w)
    return d


def flops_qkv_projection(cfg: QkvProjectionConfig) -> int:
    """Multiply-adds of the projection counted as 2 flops each."""
    return 2 * cfg.seq * cfg.hidden * (cfg.n_q_heads + 2 * cfg.n_k_heads) * cfg.head_dim


# ---------------------------------------------------------------------------
# KV RMSNorm + RoPE + cache workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class KvCacheConfig:
    name: str
    batch: int
    heads: int
    seq: int
    kv_dim: int          # last dim of kv
    rms_size: int        # V1: Dv (first part of kv); V2: kv_dim
    rope_size: int       # rotated width
    v_dim: int           # V2 width of v_optional; 0 selects V1
    dtype: torch.dtype
    eps: float
    seed: int
    cache_mode: str      # NORM, PA_BNSD or PA_BLK_BNSD
    k_cache_dtype: torch.dtype
    ckv_cache_dtype: torch.dtype
    block_size: int = 0
    block_num: int = 0
    cache_rows: int = 0  # Norm: Scache
    k_scale: Optional[tuple] = None    # (lo, hi, shape-kind) with kind in {"1", "D", "1D", "ND"}
    k_offset: Optional[tuple] = None
    v_scale: Optional[tuple] = None
    v_offset: Optional[tuple] = None
    is_output_kv: bool = False
    index_kind: str = "perm"    # "perm": first B*S entries of a slot permutation; "rows": distinct rows
    rope_pos: str = "seq"       # "seq": position s; "index": position = index value (decode)
    invalid_every: int = 0      # >0: every k-th index entry is -1 (skipped token)


MLA_V1_PREFILL = KvCacheConfig(
    name="mla_v1_prefill", batch=8, heads=1, seq=4096, kv_dim=576, rms_size=512,
    rope_size=64, v_dim=0, dtype=torch.bfloat16, eps=1e-5, seed=1003,
    cache_mode=PA_BNSD, k_cache_dtype=torch.bfloat16,
    ckv_cache_dtype=torch.bfloat16, block_size=128, block_num=320,
    is_output_kv=True)

MLA_V1_DECODE_QUANT = KvCacheConfig(
    name="mla_v1_decode_quant", batch=512, heads=1, seq=1, kv_dim=576,
    rms_size=512, rope_size=64, v_dim=0, dtype=torch.bfloat16, eps=1e-5,
    seed=1004, cache_mode=NORM, k_cache_dtype=torch.int8,
    ckv_cache_dtype=torch.float8_e4m3fn, cache_rows=8192,
    k_scale=(0.01, 0.05, "D"), v_scale=(0.5, 2.0, "D"), is_output_kv=False,
    index_kind="rows", rope_pos="index")

MLA_V2_SPLIT = KvCacheConfig(
    name="mla_v2_split", batch=16, heads=8, seq=2048, kv_dim=192, rms_size=192,
    rope_size=64, v_dim=128, dtype=torch.bfloat16, eps=1e-5, seed=1005,
    cache_mode=PA_BNSD, k_cache_dtype=torch.int8, ckv_cache_dtype=torch.int8,
    block_size=128, block_num=320, k_scale=(8.0, 32.0, "ND"),
    k_offset=(-16.0, 16.0, "ND"), v_scale=(8.0, 32.0, "ND"),
    v_offset=(-16.0, 16.0, "ND"), is_output_kv=False)


def _quant_param(spec, heads, width, g, device):
    if spec is None:
        return None
    lo, hi, kind = spec
    shape = {"1": (1,), "D": (width,), "1D": (1, width), "ND": (heads, width)}[kind]
    return _uniform(shape, lo, hi, g, device, torch.float32)


def cache_shapes(cfg: KvCacheConfig):
    """(k_cache shape, ckv_cache shape, k width, ckv width) of a workload.

    Norm caches are [B, N, Scache, D]; paged caches are [block_num, block_size,
    N, D] (the shape the cache/index constraint table gives for PA/PA_BNSD).
    """
    if cfg.v_dim:
        dk, dc = cfg.kv_dim, cfg.v_dim
    else:
        dk, dc = cfg.kv_dim - cfg.rms_size, cfg.rms_size
    if cfg.cache_mode == NORM:
        lead = (cfg.batch, cfg.heads, cfg.cache_rows)
    else:
        lead = (cfg.block_num, cfg.block_size, cfg.heads)
    return lead + (dk,), lead + (dc,), dk, dc


def make_kv_cache(cfg: KvCacheConfig, device="cpu", prefill=True, **override):
    """Draw one batch of inputs for the KV RMSNorm + RoPE + cache operator.

    Draw order: activations (kv, then v), gamma, quant params (k scale, k
    offset, v scale, v offset), index, then the cache pre-fill bytes.
    """
    cfg = dataclasses.replace(cfg, **override) if override else cfg
    g = _gen(cfg.seed, device)
    B, N, S = cfg.batch, cfg.heads, cfg.seq
    kv = _normal((B, N, S, cfg.kv_dim), g, device, cfg.dtype)
    v = _normal((B, N, S, cfg.v_dim), g, device, cfg.dtype) if cfg.v_dim else None
    gamma = _uniform((cfg.rms_size,), 0.5, 1.5, g, device, cfg.dtype)
    k_shape, c_shape, dk, dc = cache_shapes(cfg)
    k_scale = _quant_param(cfg.k_scale, N, dk, g, device)
    k_offset = _quant_param(cfg.k_offset, N, dk, g, device)
    v_scale = _quant_param(cfg.v_scale, N, dc, g, device)
    v_offset = _quant_param(cfg.v_offset, N, dc, g, device)

    if cfg.cache_mode == NORM:
        # one row per (b, s) inside batch b's slab of Scache rows
        if cfg.index_kind == "rows":
            rows = torch.randperm(cfg.cache_rows, generator=_gen(cfg.seed + 7, "cpu"))
            rows = rows[: B * S] if B * S <= cfg.cache_rows else rows.repeat(B * S // cfg.cache_rows + 1)[: B * S]
            index = rows.reshape(B, S)
        else:
            index = torch.stack([torch.randperm(cfg.cache_rows, generator=_gen(cfg.seed + 7 + b, "cpu"))[:S]
                                 for b in range(B)])
    elif cfg.cache_mode == PA_BLK_BNSD:
        # one starting slot per run of block_size tokens of a batch: distinct
        # blocks, block-aligned starts ("blocks"), or starts at a random offset
        # inside even-numbered blocks so that a run spills into the unused odd
        # block after it ("blocks_unaligned")
        bs = cfg.block_size
        runs = B * -(-S // bs)
        gi = _gen(cfg.seed + 7, "cpu")
        if cfg.index_kind == "blocks_unaligned":
            blocks = torch.randperm(cfg.block_num // 2, generator=gi)[:runs] * 2
            index = blocks * bs + torch.randint(0, bs, (runs,), generator=gi)
        else:
            index = torch.randperm(cfg.block_num, generator=gi)[:runs] * bs
    else:
        slots = cfg.block_num * cfg.block_size
        index = torch.randperm(slots, generator=_gen(cfg.seed + 7, "cpu"))[: B * S].clone()
    if cfg.invalid_every:
        flat = index.view(-1)
        flat[:: cfg.invalid_every] = -1
    index = index.to(torch.int64).to(device)

    R = cfg.rope_size
    if cfg.rope_pos == "index":
        pos = index.reshape(B, 1, S).expand(B, N, S).clamp_min(0)
    else:
        pos = torch.arange(S, device=device).reshape(1, 1, S).expand(B, N, S)
    cos, sin = rotate_half_table_1d(pos.reshape(-1), R)
    cos = cos.to(cfg.dtype).reshape(B, N, S, R).contiguous()
    sin = sin.to(cfg.dtype).reshape(B, N, S, R).contiguous()

    def _cache(shape, dt):
        if not prefill:
            return torch.zeros(shape, dtype=dt, device=device)
        raw = torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.uint8)
        if dt.itemsize == 1:
            return raw.view(dt)
        # 16-bit caches: fill with random finite values (exponent field kept small)
        raw16 = torch.randint(0, 1 << 14, shape, generator=g, device=device, dtype=torch.int32).to(torch.int16)
        return raw16.view(dt)

    k_cache = _cache(k_shape, cfg.k_cache_dtype)
    ckv_cache = _cache(c_shape, cfg.ckv_cache_dtype)
    k_rope = torch.zeros((B, N, S, dk), dtype=cfg.dtype, device=device) if cfg.is_output_kv else None
    c_kv = torch.zeros((B, N, S, dc), dtype=cfg.dtype, device=device) if cfg.is_output_kv else None
    return dict(cfg=cfg, kv=kv, v=v, gamma=gamma, cos=cos, sin=sin, index=index,
                k_cache=k_cache, ckv_cache=ckv_cache, k_scale=k_scale,
                k_offset=k_offset, v_scale=v_scale, v_offset=v_offset,
                eps=cfg.eps, k_rope=k_rope, c_kv=c_kv, k_width=dk, c_width=dc)


ALL = {c.name: c for c in (TINY_ACROSS_HEADS, WAN22_SELF_ATTN, MLA_V1_PREFILL,
                           MLA_V1_DECODE_QUANT, MLA_V2_SPLIT)}


def algorithmic_bytes_qk_split(cfg: AcrossHeadsConfig, tp: int):
    """Bytes each pass of the split over `tp` ranks must move on one rank
    (n_q/tp and n_k/tp heads): (sum pass, apply pass).

    Sum pass: read the rank's Q and K once, write one fp32 sum per token and
    segment. Apply pass: read Q, K, cos, sin and the sums once, write Q and K
    once, read the rank's gamma slices once."""
    e = torch.tensor([], dtype=cfg.dtype).element_size()
    T = cfg.batch * cfg.seq
    cq, ck = cfg.n_q_heads // tp * cfg.head_dim, cfg.n_k_heads // tp * cfg.head_dim
    segs = 2 if ck else 1
    sums = e * T * (cq + ck) + 4 * segs * T
    apply = e * (T * (2 * (cq + ck) + 2 * cfg.head_dim) + cq + ck) + 4 * segs * T
    return sums, apply


def algorithmic_bytes_per_head(cfg: AcrossHeadsConfig) -> int:
    """As the across-heads pass, with one [head_dim] gamma per segment."""
    e = torch.tensor([], dtype=cfg.dtype).element_size()
    T = cfg.batch * cfg.seq
    cq, ck = cfg.n_q_heads * cfg.head_dim, cfg.n_k_heads * cfg.head_dim
    return e * (T * (2 * (cq + ck) + 2 * cfg.head_dim) + cfg.head_dim * (2 if ck else 1))


def algorithmic_bytes_across_heads(cfg: AcrossHeadsConfig) -> int:
    """Bytes the across-heads pass must move: Q and K read and written once,
    cos and sin read once per token, both gammas read once."""
    rd, wr = algorithmic_read_write_across_heads(cfg)
    return rd + wr


def algorithmic_read_write_across_heads(cfg: AcrossHeadsConfig):
    """The across-heads pass's algorithmic bytes split into (read, written)."""
    e = torch.tensor([], dtype=cfg.dtype).element_size()
    T = cfg.batch * cfg.seq
    cq, ck = cfg.n_q_heads * cfg.head_dim, cfg.n_k_heads * cfg.head_dim
    return e * (T * ((cq + ck) + 2 * cfg.head_dim) + cq + ck), e * T * (cq + ck)


def algorithmic_bytes_kv_cache(cfg: KvCacheConfig) -> int:
    """Bytes the KV operator must move: kv (and v), cos, sin and the index read
    once; one k row and one ckv row written per (b, n, s) token with a valid
    index; k_rope / c_kv written when requested; gamma and quant params read
    once."""
    rd, wr = algorithmic_read_write_kv_cache(cfg)
    return rd + wr


def algorithmic_read_write_kv_cache(cfg: KvCacheConfig):
    """The KV operator's algorithmic bytes split into (read, written)."""
    e = torch.tensor([], dtype=cfg.dtype).element_size()
    rows = cfg.batch * cfg.heads * cfg.seq
    tokens = cfg.batch * cfg.seq
    _, _, dk, dc = cache_shapes(cfg)
    ek = torch.tensor([], dtype=cfg.k_cache_dtype).element_size()
    ec = torch.tensor([], dtype=cfg.ckv_cache_dtype).element_size()
    entries = cfg.batch * -(-cfg.seq // cfg.block_size) if cfg.cache_mode == PA_BLK_BNSD else tokens
    rd = rows * e * (cfg.kv_dim + cfg.v_dim + 2 * cfg.rope_size) + entries * 8
    wr = rows * (dk * ek + dc * ec)
    if cfg.is_output_kv:
        wr += rows * e * (dk + dc)
    small = e * cfg.rms_size
    for spec, width in ((cfg.k_scale, dk), (cfg.k_offset, dk), (cfg.v_scale, dc), (cfg.v_offset, dc)):
        if spec is not None:
            n = {"1": 1, "D": width, "1D": width, "ND": cfg.heads * width}[spec[2]]
            small += 4 * n
    return rd + small, wr


def math_check():  # pragma: no cover - documentation helper
    """The Wan latent grid for 81 frames at 720x1280 (VAE stride 4 in time, 8 in
    space, patch 2x2): ((81-1)//4+1, (720//8)//2, (1280//8)//2) = (21, 45, 80)."""
    return ((81 - 1) // 4 + 1, (720 // 8) // 2, (1280 // 8) // 2), math.prod((21, 45, 80))
