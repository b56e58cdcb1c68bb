"""Host-side checks of the C ABI (no GPU, no compute calls): the library loads,
exports every function include/qknr.h declares, the ctypes mirrors match the C
struct layouts, and the host validation returns the documented status codes
for the constraint rules of the pages."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import qk_rmsnorm_rope_amd as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qknr.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char \*|int32_t )\s*(qknr_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) == set(Q.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", Q.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (qknr_\w+)$", out, re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(Q._lib, n)


def test_every_kernel_launch_stub_is_defined():
    """Each kernel the library launches has its host stub defined in the library
    (a kernel template whose host pass failed would leave it undefined, and the
    library would fail only when loaded on the GPU host)."""
    out = subprocess.run(["nm", Q.LIB_PATH], capture_output=True, text=True).stdout
    undefined = [ln for ln in out.splitlines() if "__device_stub__" in ln and " U " in ln]
    assert not undefined, undefined
    defined = [ln for ln in out.splitlines() if "__device_stub__" in ln]
    for kernel in ("qkv_proj_kernel", "qk_kernel", "kv_rmsnorm_rope_cache_kernel", "permute_kernel"):
        assert any(kernel in ln for ln in defined), kernel


def test_version_matches_header():
    m = re.search(r"#define QKNR_ABI_VERSION (\d+)", open(HEADER).read())
    assert Q.version() == int(m.group(1))


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (QKNR_\w+) (\d+)\b", text))
    assert consts["QKNR_OK"] == Q.OK and consts["QKNR_INVALID_ARGUMENT"] == Q.INVALID_ARGUMENT
    assert consts["QKNR_UNSUPPORTED"] == Q.UNSUPPORTED and consts["QKNR_DEVICE_ERROR"] == Q.DEVICE_ERROR
    assert consts["QKNR_BF16"] == Q.BF16 and consts["QKNR_F16"] == Q.F16 and consts["QKNR_F32"] == Q.F32
    assert consts["QKNR_INT8"] == Q.INT8 and consts["QKNR_FP8_E4M3FN"] == Q.FP8_E4M3FN
    assert consts["QKNR_FP8_E5M2"] == Q.FP8_E5M2
    assert consts["QKNR_CACHE_NORM"] == Q.CACHE_NORM and consts["QKNR_CACHE_PA_BNSD"] == Q.CACHE_PA_BNSD
    assert consts["QKNR_CACHE_PA_BLK_BNSD"] == Q.CACHE_PA_BLK_BNSD
    assert consts["QKNR_QSHAPE_HEAD_CHANNEL"] == Q.QSHAPE_HEAD_CHANNEL
    assert consts["QKNR_PROJ_SCALE_ROW"] == Q.PROJ_SCALE_ROW and consts["QKNR_PROJ_SCALE_MX32"] == Q.PROJ_SCALE_MX32


def test_struct_layouts_match_c(tmp_path):
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "qknr.h"', "int main(void) {"]
    structs = (("qknr_qk_args", Q.QkArgs), ("qknr_kv_args", Q.KvArgs), ("qknr_permute_args", Q.PermuteArgs),
               ("qknr_proj_args", Q.ProjArgs))
    for cname, py in structs:
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("cannot compile against hip_runtime_api.h here: " + r.stderr[-300:])
    got = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split("\n")
    for line in got:
        if not line:
            continue
        cname, field, val = line.split()
        py = dict(structs)[cname]
        expect = ctypes.sizeof(py) if field == "sizeof" else getattr(py, field).offset
        assert int(val) == expect, (cname, field)


# ---------------------------------------------------------------- (a) validation

def _qk(B=1, S=4, nq=2, nk=2, d=8, dtype=torch.bfloat16, **kw):
    qkv = torch.zeros(B, S, (nq + nk) * d, dtype=dtype)
    q = qkv[..., : nq * d].unflatten(-1, (nq, d))
    k = qkv[..., nq * d:].unflatten(-1, (nk, d)) if nk else None
    qg = torch.ones(nq * d, dtype=dtype)
    kg = torch.ones(nk * d, dtype=dtype) if nk else None
    cos = torch.ones(1, S, d, dtype=dtype)
    sin = torch.zeros(1, S, d, dtype=dtype)
    args = dict(eps=1e-6)
    args.update(kw)
    return Q.qk_args(q, k, qg, kg, cos, sin, **args)


def test_qk_valid_arguments_pass():
    assert Q.qk_validate(_qk()) == Q.OK
    assert Q.qk_validate(_qk(nk=0)) == Q.OK
    assert Q.qk_validate(_qk(dtype=torch.float32, d=64, nq=4, nk=4)) == Q.OK
    assert Q.qk_validate(_qk(nq=40, nk=40, d=128)) == Q.OK
    assert Q.qk_validate(_qk(S=0)) == Q.OK          # zero tokens: a no-op


@pytest.mark.parametrize("mutate, code", [
    (lambda a: setattr(a, "head_dim", 7), Q.INVALID_ARGUMENT),
    (lambda a: setattr(a, "n_q_heads", 0), Q.INVALID_ARGUMENT),
    (lambda a: setattr(a, "dtype", Q.INT8), Q.INVALID_ARGUMENT),
    (lambda a: setattr(a, "q_gamma", None), Q.INVALID_ARGUMENT),
    (lambda a: setattr(a, "cos", None), Q.INVALID_ARGUMENT),
    (lambda a: setattr(a, "k_in", None), Q.INVALID_ARGUMENT),
    (lambda a: setattr(a, "eps", -1.0), Q.INVALID_ARGUMENT),
    (lambda a: setattr(a, "in_head_stride", 4), Q.INVALID_ARGUMENT),
])
def test_qk_invalid_arguments(mutate, code):
    a = _qk()
    mutate(a)
    assert Q.qk_validate(a) == code
    assert Q.last_error() != ""


def test_qk_in_place_needs_equal_strides():
    a = _qk()
    a.q_out = a.q_in
    a.k_out = a.k_in
    assert Q.qk_validate(a) == Q.OK
    a.out_token_stride = a.in_token_stride * 2
    assert Q.qk_validate(a) == Q.INVALID_ARGUMENT


def test_qk_alignment_falls_back_or_is_unsupported():
    a = _qk(d=8)
    a.q_in = a.q_in + 4            # 4-byte offset: the 2-element path still applies
    a.q_out = a.q_out + 4
    assert Q.qk_validate(a) == Q.OK
    a.q_in = a.q_in + 2            # 2-byte offset: no 4-byte access possible
    assert Q.qk_validate(a) == Q.UNSUPPORTED


def _call(fn, a, *extra):
    return int(getattr(Q._lib, fn)(ctypes.byref(a), *extra, None))


def test_qk_new_entry_points_reject_invalid_arguments_on_the_host():
    """Each failing check returns before any device call."""
    fake = ctypes.c_void_p(0x100000)          # never dereferenced: validation fails first
    a = _qk()
    a.q_norm_channels = 4096                  # only the apply pass takes a total channel count
    assert _call("qknr_qk_norm_rope_across_heads", a) == Q.INVALID_ARGUMENT
    assert _call("qknr_qk_norm_rope_per_head", a) == Q.INVALID_ARGUMENT
    assert _call("qknr_qk_sumsq_across_heads", a, fake) == Q.INVALID_ARGUMENT
    b = _qk()
    assert _call("qknr_qk_sumsq_across_heads", b, None) == Q.INVALID_ARGUMENT      # sums buffer missing
    assert _call("qknr_qk_apply_across_heads", b, None) == Q.INVALID_ARGUMENT
    assert _call("qknr_qk_apply_across_heads", b, ctypes.c_void_p(0x100002)) == Q.INVALID_ARGUMENT  # misaligned
    c = _qk(apply_norm=False)
    assert _call("qknr_qk_apply_across_heads", c, fake) == Q.INVALID_ARGUMENT      # apply needs the norm
    d = _qk()
    d.q_norm_channels = 8                     # smaller than this call's own 2*8 channels
    assert _call("qknr_qk_apply_across_heads", d, fake) == Q.INVALID_ARGUMENT
    d.q_norm_channels = 1 << 24
    assert _call("qknr_qk_apply_across_heads", d, fake) == Q.INVALID_ARGUMENT
    e = _qk()
    e.q_gamma = None                          # per head still needs its gamma
    assert _call("qknr_qk_norm_rope_per_head", e) == Q.INVALID_ARGUMENT


def _perm(**kw):
    a = Q.PermuteArgs()
    a.elem_bytes, a.inverse, a.outer, a.axis_len, a.inner = 2, 0, 4, 24, 1
    a.first, a.n_heads, a.head_dim = 0, 3, 8
    a.src, a.dst = 0x100000, 0x200000
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw", [dict(elem_bytes=3), dict(head_dim=7), dict(n_heads=4), dict(first=1),
                                dict(axis_len=0), dict(inner=0), dict(outer=-1), dict(dst=0x100010),
                                dict(src=None)])
def test_permute_rejects_invalid_arguments(kw):
    assert int(Q._lib.qknr_interleaved_to_rotate_half(ctypes.byref(_perm(**kw)), None)) == Q.INVALID_ARGUMENT
    assert Q.last_error() != ""


def test_permute_empty_tensor_is_a_noop():
    assert int(Q._lib.qknr_interleaved_to_rotate_half(ctypes.byref(_perm(outer=0, src=None, dst=None)),
                                                       None)) == Q.OK


# a legal MXFP8 call: FP8 operands, K = 256 (8 blocks of 32), block scales 4-byte aligned
_MX = dict(dtype=Q.FP8_E4M3FN, scale_mode=Q.PROJ_SCALE_MX32, in_features=256, a_row_stride=256,
           w_row_stride=256, a_block_scale=0xA00000, a_block_scale_stride=8, w_block_scale=0xB00000,
           w_block_scale_stride=8)


def _proj(**kw):
    a = Q.ProjArgs()
    a.dtype, a.rows, a.in_features, a.out_features = Q.BF16, 300, 128, 384
    a.a, a.a_row_stride = 0x100000, 128
    a.w, a.w_row_stride = 0x200000, 128
    a.bias = None
    a.out, a.out_row_stride = 0x400000, 384
    a.q_cols, a.k_cols, a.sumsq = 128, 128, 0x800000
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw, code", [
    (dict(dtype=Q.F32), Q.UNSUPPORTED),
    (dict(dtype=Q.FP8_E4M3FN, in_features=64), Q.UNSUPPORTED),                     # FP8 K: 128-byte multiples
    (dict(a_scale=0x900002), Q.UNSUPPORTED),                                         # scale misaligned
    (dict(in_features=100, a_row_stride=104, w_row_stride=104), Q.UNSUPPORTED),    # K not a multiple of 64
    (dict(out_features=300, out_row_stride=304), Q.UNSUPPORTED),                   # N not a multiple of 128
    (dict(q_cols=64, k_cols=64), Q.INVALID_ARGUMENT),
    (dict(q_cols=128, k_cols=256), Q.INVALID_ARGUMENT),                              # k_cols must be 0 or q_cols
    (dict(q_cols=256, k_cols=256), Q.INVALID_ARGUMENT),                              # beyond out_features
    (dict(sumsq=None), Q.INVALID_ARGUMENT),
    (dict(sumsq=0x800002), Q.INVALID_ARGUMENT),
    (dict(a_row_stride=120), Q.INVALID_ARGUMENT),                                    # shorter than a row
    (dict(a_row_stride=(4 << 20) // 2 + 8), Q.UNSUPPORTED),                          # pitch above 4 MiB
    (dict(w_row_stride=(4 << 20) // 2 + 8), Q.UNSUPPORTED),
    (dict(out=0x100000 + 64), Q.INVALID_ARGUMENT),                                   # out overlaps a
    (dict(a=0x100008), Q.UNSUPPORTED),                                               # not 16-byte aligned
    (dict(rows=-1), Q.INVALID_ARGUMENT),
    (dict(scale_mode=7), Q.UNSUPPORTED),
    (dict(scale_mode=Q.PROJ_SCALE_MX32), Q.INVALID_ARGUMENT),                       # MX needs FP8 operands
    (dict(a_block_scale=0xA00000), Q.INVALID_ARGUMENT),                              # block scales without MX
] + [(dict(_MX, **kw), code) for kw, code in [
    (dict(a_block_scale=None), Q.INVALID_ARGUMENT),
    (dict(w_block_scale=0xB00002), Q.INVALID_ARGUMENT),                              # not 4-byte aligned
    (dict(a_block_scale_stride=4), Q.INVALID_ARGUMENT),                              # shorter than K/32 = 8
    (dict(w_block_scale_stride=10), Q.INVALID_ARGUMENT),                             # not a multiple of 4
    (dict(a_block_scale=0x400000 + 64), Q.INVALID_ARGUMENT),                         # overlaps out
]])
def test_projection_rejects_invalid_arguments(kw, code):
    assert int(Q._lib.qknr_qkv_projection(ctypes.byref(_proj(**kw)), None)) == code
    assert Q.last_error() != ""


def test_projection_mx_arguments_pass_validation():
    """A legal MXFP8 call gets past validation (then fails to launch on this
    GPU-less host, or would launch)."""
    rc = int(Q._lib.qknr_qkv_projection(ctypes.byref(_proj(**_MX)), None))
    assert rc in (Q.OK, Q.DEVICE_ERROR), Q.last_error()
    if rc == Q.DEVICE_ERROR:
        assert "launch failed" in Q.last_error()


def test_projection_zero_rows_is_a_noop():
    assert int(Q._lib.qknr_qkv_projection(ctypes.byref(_proj(rows=0, a=None, w=None, out=None)), None)) == Q.OK


def test_apply_partial_sums_only_in_the_apply_pass():
    a = _qk()
    a.sumsq_parts = 4
    assert Q.qk_validate(a) == Q.INVALID_ARGUMENT
    assert _call("qknr_qk_norm_rope_per_head", a) == Q.INVALID_ARGUMENT


def test_qk_too_many_heads_is_unsupported():
    assert Q.qk_validate(_qk(nq=300, nk=0, d=128)) == Q.UNSUPPORTED
    assert Q.qk_validate(_qk(nq=256, nk=0, d=128)) == Q.OK
    assert Q.qk_validate(_qk(nq=1, nk=0, d=4096)) == Q.UNSUPPORTED     # head wider than one wave's lanes


# ---------------------------------------------------------------- (b) validation

def _kv(v2=False, mode="PA_BNSD", kdt=torch.bfloat16, cdt=torch.bfloat16, B=2, N=1, S=8, bs=32, nb=4,
        ks=None, ko=None, vs=None, vo=None, out_kv=False, srope=None, dtype=torch.bfloat16):
    D = 192 if v2 else 576
    R = 64
    kv = torch.zeros(B, N, S, D, dtype=dtype)
    v = torch.zeros(B, N, S, 128, dtype=dtype) if v2 else None
    g = torch.ones(D if v2 else 512, dtype=dtype)
    cs = torch.ones(B, N, srope or S, R, dtype=dtype)
    dk, dc = (D, 128) if v2 else (R, 512)
    if mode == "Norm":
        kc = torch.zeros(B, N, 16, dk, dtype=kdt)
        cc = torch.zeros(B, N, 16, dc, dtype=cdt)
        idx = torch.zeros(B, S, dtype=torch.int64)
    else:
        kc = torch.zeros(nb, bs, N, dk, dtype=kdt)
        cc = torch.zeros(nb, bs, N, dc, dtype=cdt)
        idx = torch.zeros(B * (-(-S // bs) if mode == "PA_BLK_BNSD" else S), dtype=torch.int64)
    kr = torch.zeros(B, N, S, dk, dtype=dtype) if out_kv else None
    ck = torch.zeros(B, N, S, dc, dtype=dtype) if out_kv else None
    return Q.kv_args(kv, g, cs, cs, idx, kc, cc, k_rope_scale=ks, k_rope_offset=ko, c_kv_scale=vs,
                     c_kv_offset=vo, v=v, cache_mode=mode, is_output_kv=out_kv, k_rope=kr, c_kv=ck)


def f32(*shape):
    return torch.ones(*shape, dtype=torch.float32)


def test_kv_valid_arguments_pass():
    assert Q.kv_validate(_kv()) == Q.OK
    assert Q.kv_validate(_kv(out_kv=True)) == Q.OK
    assert Q.kv_validate(_kv(mode="Norm", kdt=torch.int8, cdt=torch.float8_e4m3fn, ks=f32(64), vs=f32(512))) == Q.OK
    assert Q.kv_validate(_kv(v2=True, N=8, kdt=torch.int8, cdt=torch.int8, ks=f32(8, 192), ko=f32(8, 192),
                             vs=f32(8, 128), vo=f32(8, 128), bs=128)) == Q.OK
    assert Q.kv_validate(_kv(mode="Norm", srope=1)) == Q.OK        # S-axis broadcast
    assert Q.kv_validate(_kv(kdt=torch.int8, ks=f32(1), bs=32)) == Q.OK   # scalar scale, V1
    assert Q.kv_validate(_kv(kdt=torch.float8_e5m2, cdt=torch.float8_e5m2, ks=f32(64), vs=f32(1, 512))) == Q.OK
    assert Q.kv_validate(_kv(mode="PA_BLK_BNSD", S=70, nb=6, out_kv=True)) == Q.OK
    assert Q.kv_validate(_kv(mode="PA_BLK_BNSD", v2=True, N=4, kdt=torch.int8, cdt=torch.float8_e5m2,
                             ks=f32(4, 192), vs=f32(4, 128), bs=128, S=300, nb=8)) == Q.OK


@pytest.mark.parametrize("kw, code", [
    (dict(N=2), Q.INVALID_ARGUMENT),                                             # V1 needs N = 1
    (dict(v2=True, N=3), Q.INVALID_ARGUMENT),                                    # V2 N in {1,2,4,8}
    (dict(kdt=torch.int8, ko=f32(64), bs=32), Q.INVALID_ARGUMENT),               # offset without scale
    (dict(kdt=torch.int8, bs=32), Q.INVALID_ARGUMENT),                           # quantised cache, no scale
    (dict(ks=f32(64)), Q.INVALID_ARGUMENT),                                      # bf16 cache with a scale
    (dict(kdt=torch.float16), Q.INVALID_ARGUMENT),                               # unquantised != kv dtype
    (dict(kdt=torch.int8, ks=f32(64), bs=16), Q.INVALID_ARGUMENT),               # block_size not 32-B aligned
    (dict(bs=32, nb=0), Q.INVALID_ARGUMENT),                                     # block_num too small
    (dict(S=0), Q.INVALID_ARGUMENT),                                             # empty tensor
    (dict(v2=True, N=2, kdt=torch.int8, ks=f32(192)), Q.INVALID_ARGUMENT),      # V2 needs [N, D]
    (dict(kdt=torch.int8, ks=f32(1, 64), srope=1, S=8), Q.INVALID_ARGUMENT),    # broadcast + quant paged
    (dict(dtype=torch.float32, kdt=torch.float32, cdt=torch.float32), Q.INVALID_ARGUMENT),  # kv must be 16-bit
    (dict(mode="PA_BLK_BNSD", S=70, nb=3), Q.INVALID_ARGUMENT),                 # block_num < floor(S/bs)*B
    (dict(mode="PA_BLK_BNSD", kdt=torch.float8_e5m2, ks=f32(64), bs=16), Q.INVALID_ARGUMENT),  # 32-B blocks
    (dict(mode="PA_BLK_BNSD", kdt=torch.int8, ks=f32(1, 64), srope=1), Q.INVALID_ARGUMENT),  # bcast + quant
    (dict(kdt=torch.float8_e5m2, ko=f32(64)), Q.INVALID_ARGUMENT),              # e5m2 offset without scale
])
def test_kv_invalid_arguments(kw, code):
    a = _kv(**kw)
    assert Q.kv_validate(a) == code
    assert Q.last_error() != ""


def test_kv_norm_cache_smaller_than_sequence():
    a = _kv(mode="Norm", S=32)
    assert Q.kv_validate(a) == Q.INVALID_ARGUMENT


def test_kv_output_kv_needs_buffers_when_effective():
    a = _kv(out_kv=True)
    a.k_rope = None
    assert Q.kv_validate(a) == Q.INVALID_ARGUMENT
    # Norm, V1, unquantised: is_output_kv has no effect, so no buffers are needed
    b = _kv(mode="Norm")
    b.is_output_kv = 1
    assert Q.kv_validate(b) == Q.OK


def test_kv_binding_checks_pa_blk_index_length():
    with pytest.raises(ValueError, match="ceil"):
        kv = torch.zeros(2, 1, 70, 576, dtype=torch.bfloat16)
        cs = torch.ones(2, 1, 70, 64, dtype=torch.bfloat16)
        Q.kv_args(kv, torch.ones(512, dtype=torch.bfloat16), cs, cs, torch.zeros(140, dtype=torch.int64),
                  torch.zeros(6, 32, 1, 64, dtype=torch.bfloat16), torch.zeros(6, 32, 1, 512, dtype=torch.bfloat16),
                  cache_mode="PA_BLK_BNSD")


def test_kv_unbuilt_modes_and_types_are_unsupported():
    a = _kv()
    a.cache_mode = 5                         # e.g. a FRACTAL_NZ layout
    assert Q.kv_validate(a) == Q.UNSUPPORTED
    b = _kv(kdt=torch.int8, ks=f32(64), bs=32)
    b.k_cache_dtype = 9                      # a cache encoding that is not built
    assert Q.kv_validate(b) == Q.UNSUPPORTED


def test_kv_strides_of_2_pow_32_elements_are_unsupported():
    """Strides are carried as 32-bit element counts (offsets are summed in 64 bits)."""
    a = _kv()
    a.kv_strides[0] = 1 << 32
    assert Q.kv_validate(a) == Q.UNSUPPORTED
    b = _kv()
    b.k_cache_strides[0] = (1 << 32) + 64
    assert Q.kv_validate(b) == Q.UNSUPPORTED
    c = _kv()
    c.kv_strides[0] = (1 << 32) - 576            # just below the limit: accepted
    assert Q.kv_validate(c) == Q.OK
