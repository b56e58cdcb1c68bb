"""Benchmark of the fused QK / KV RMSNorm + RoPE (+ cache) library on one MI355X.

One step is one pass of the across-heads QK norm + rotate-half RoPE over the
Wan2.2-A14B-shaped self-attention epilogue: S = 75600 tokens (21x45x80 latent
grid), Q and K 40 heads x 128 bf16 in a BSD buffer [1, 75600, 10240], written
out of place. Inputs are synthetic and already resident in HBM.

Printed: ONE JSON line with the headline throughput (algorithmic HBM GB/s over
the timed steps), tokens/s, the roofline of the kernel (bytes it must move /
its average launch time, measured with HIP events on the launch stream, vs
MI355X's 8 TB/s), the fp64 CPU oracle timed on a bounded sample of the same
workload and on every other workload (one thread and all cores), the
KvRmsNormRopeCache workloads (MLA V1 prefill, also with PA_BLK_BNSD indexing,
V1 decode quantised, also as a HIP-graph replay, V2 split) timed the same way,
hot (back to back) and cold (each launch alone after a 1 GiB pass that evicts
L2 and the MALL: frac_cold after writing 1 GiB, the stated protocol, and
frac_cold_read after reading it), and the other forms of the QK operator on the Wan2.2
shape: per-head norm, and the two passes of the across-heads norm split over
tp = 4 ranks at one rank's share (10 + 10 heads); and the QKV projection
(75600 x 5120 -> 15360 on the matrix cores, bf16 operands and FP8 ROW_MX
operands) with the norm's sums in its epilogue followed by the apply pass,
next to the unfused pipeline of a library GEMM (torch.addmm /
torch._scaled_mm, hipBLASLt) and the single-pass epilogue kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-kv] [--no-forms] [--no-proj]
       python bench.py --profile {across,per_head,split_sumsq,split_apply,proj,proj_fp8,proj_mxfp8,
                                  proj_lib,proj_fp8_lib,kv_v1_prefill,kv_v1_decode,kv_v2,copy}
       (a short fixed run of one kernel, for rocprofv3 counter collection)
       python bench.py --ceiling
       (plain stream kernels with the operators' read/write mixes at 32 MB - 3.1 GB,
       the bandwidth ceiling the operators are compared with)
       python bench.py --summarize DIR
       (turn the rocprofv3 CSVs under DIR into the text summaries and the
       traffic record under profiles/; CPU only)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 matrix-core peak
PEAK_FP8_TFLOPS = 5000.0           # MI355X dense fp8 matrix-core peak
METRIC = "achieved HBM GB/s (% of MI355X peak) + tokens/s for fused norm+RoPE(+cache)"
KERNEL_SOURCES = {
    "qk_across_heads": ["qk_rmsnorm_rope_amd/csrc/qk_across_heads.hip", "qk_rmsnorm_rope_amd/csrc/qk_kernel.h",
                        "qk_rmsnorm_rope_amd/csrc/device_common.h", "qk_rmsnorm_rope_amd/csrc/plan.cpp"],
    "qk_per_head": ["qk_rmsnorm_rope_amd/csrc/qk_per_head.hip", "qk_rmsnorm_rope_amd/csrc/qk_kernel.h",
                    "qk_rmsnorm_rope_amd/csrc/device_common.h", "qk_rmsnorm_rope_amd/csrc/plan.cpp"],
    "qk_split": ["qk_rmsnorm_rope_amd/csrc/qk_split.hip", "qk_rmsnorm_rope_amd/csrc/qk_kernel.h",
                 "qk_rmsnorm_rope_amd/csrc/device_common.h", "qk_rmsnorm_rope_amd/csrc/plan.cpp"],
    "qkv_proj": ["qk_rmsnorm_rope_amd/csrc/qkv_proj.hip", "qk_rmsnorm_rope_amd/csrc/device_common.h"],
    "kv_rmsnorm_rope_cache": ["qk_rmsnorm_rope_amd/csrc/kv_rmsnorm_rope_cache.hip",
                              "qk_rmsnorm_rope_amd/csrc/kv_rmsnorm_rope_cache_f16.hip",
                              "qk_rmsnorm_rope_amd/csrc/kv_kernel.h",
                              "qk_rmsnorm_rope_amd/csrc/device_common.h", "qk_rmsnorm_rope_amd/csrc/plan.cpp"],
}


def strip_comments(src):
    """C/C++ source without its comments and trailing blanks (string and
    character literals kept), so that an edit of comments alone does not mark
    the counters taken on the code as stale."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = [ln.rstrip() for ln in "".join(out).split("\n")]
    return "\n".join(ln for ln in lines if ln)


def source_hash(kernel):
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(workload)
    if not k or k.get("source_hash") != source_hash(kernel):
        return None
    return k.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-kv", action="store_true", help="skip the KvRmsNormRopeCache workloads")
    ap.add_argument("--no-forms", action="store_true", help="skip the per-head and split forms of (a)")
    ap.add_argument("--no-proj", action="store_true", help="skip the QKV projection")
    ap.add_argument("--cold-iters", type=int, default=50)
    ap.add_argument("--profile", default=None,
                    choices=["across", "per_head", "split_sumsq", "split_apply", "proj", "proj_fp8", "proj_mxfp8",
                             "proj_lib", "proj_fp8_lib", "kv_v1_prefill", "kv_v1_prefill_pa_blk", "kv_v1_decode",
                             "kv_v2", "copy"])
    ap.add_argument("--summarize", default=None, metavar="DIR")
    ap.add_argument("--ceiling", action="store_true",
                    help="sweep plain stream kernels with the operators' read/write mixes (bench_stream.hip)")
    return ap.parse_args()


def across_setup(torch, W, Q):
    cfg = W.WAN22_SELF_ATTN
    d = W.make_across_heads(cfg, device="cuda")
    qkv = d["qkv"]
    out = torch.empty_like(qkv)
    nq, nk, hd = cfg.n_q_heads, cfg.n_k_heads, cfg.head_dim
    q = qkv[..., : nq * hd].unflatten(-1, (nq, hd))
    k = qkv[..., nq * hd:].unflatten(-1, (nk, hd))
    qo = out[..., : nq * hd].unflatten(-1, (nq, hd))
    ko = out[..., nq * hd:].unflatten(-1, (nk, hd))

    step = Q.prepare_qk_norm_rope_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"],
                                               eps=cfg.eps, q_out=qo, k_out=ko)
    return cfg, d, step


def forms_setup(torch, W, Q, which, d=None):
    """Launchers of the other forms of (a) on the Wan2.2 shape: 'per_head'
    (all 40 + 40 heads, [128] gammas) and the split over tp = 4 ranks at one
    rank's share, 'split_sumsq' and 'split_apply' (10 + 10 heads)."""
    cfg = W.WAN22_SELF_ATTN
    if d is None:
        d = W.make_across_heads(cfg, device="cuda")
    nq, nk, hd = cfg.n_q_heads, cfg.n_k_heads, cfg.head_dim
    qkv = d["qkv"]
    q = qkv[..., : nq * hd].unflatten(-1, (nq, hd))
    k = qkv[..., nq * hd:].unflatten(-1, (nk, hd))
    if which == "per_head":
        out = torch.empty_like(qkv)
        qo = out[..., : nq * hd].unflatten(-1, (nq, hd))
        ko = out[..., nq * hd:].unflatten(-1, (nk, hd))
        gq, gk = d["q_gamma"][:hd].contiguous(), d["k_gamma"][:hd].contiguous()
        return Q.prepare_qk_norm_rope_per_head(q, k, gq, gk, d["cos"], d["sin"], eps=cfg.eps, q_out=qo, k_out=ko)
    tp = 4
    lq, lk = nq // tp, nk // tp
    qs = torch.empty(1, cfg.seq, lq + lk, hd, dtype=cfg.dtype, device="cuda")   # one rank's Q|K slice
    qs.copy_(torch.cat([q[:, :, :lq], k[:, :, :lk]], 2))
    sq, sk = qs[:, :, :lq], qs[:, :, lq:]
    sums = torch.empty(2, cfg.seq, dtype=torch.float32, device="cuda")
    sum_step = Q.prepare_qk_sumsq_across_heads(sq, sk, sums)
    if which == "split_sumsq":
        return sum_step
    sum_step()
    sums.mul_(tp)                                    # stands in for the other ranks' sums
    out = torch.empty_like(qs)
    gq, gk = d["q_gamma"][: lq * hd].contiguous(), d["k_gamma"][: lk * hd].contiguous()
    return Q.prepare_qk_apply_across_heads(sq, sk, gq, gk, d["cos"], d["sin"], sums, eps=cfg.eps,
                                           q_norm_channels=nq * hd, k_norm_channels=nk * hd,
                                           q_out=out[:, :, :lq], k_out=out[:, :, lq:])


def forms_measure(torch, W, Q, d, flush, cold_iters):
    cfg = W.WAN22_SELF_ATTN
    sums_b, apply_b = W.algorithmic_bytes_qk_split(cfg, 4)
    res = {}
    for name, nbytes, kernel in (("per_head", W.algorithmic_bytes_per_head(cfg), "qk_per_head"),
                                 ("split_sumsq", sums_b, "qk_split"), ("split_apply", apply_b, "qk_split")):
        step = forms_setup(torch, W, Q, name, d)
        for _ in range(5):
            step()
        hot = time_hot(torch, step, 50)
        res[name] = {"algorithmic_bytes": nbytes, "us_hot_mean": round(hot, 3),
                     "gbs_hot": round(nbytes / hot / 1e3, 1), "frac_hot": round(nbytes / hot / 1e3 / PEAK_HBM_GBS, 4)}
        res[name].update(cold_record(torch, step, cold_iters, flush, nbytes))
        res[name]["traffic"] = measured_traffic(kernel, "wan22_" + name)
        del step
        torch.cuda.empty_cache()
    res["per_head"]["workload"] = "Wan2.2 S=75600, 40+40 heads x 128 bf16, per-head RMS, [128] gammas, out of place"
    res["split_sumsq"]["workload"] = ("Wan2.2 S=75600 split over tp=4 ranks: one rank's 10+10 heads, "
                                      "per-token sums of squares -> fp32 [2, S]")
    res["split_apply"]["workload"] = ("the same rank's apply pass: sums of all ranks, 5120-channel RMS, "
                                      "gamma slices, RoPE, out of place")
    res["split_two_pass_us_hot"] = round(res["split_sumsq"]["us_hot_mean"] + res["split_apply"]["us_hot_mean"], 3)
    return res


def proj_setup(torch, W, Q):
    """The Wan2.2 QKV projection with the norm's sums (fused path), its apply
    pass, and the pieces of the unfused reference pipeline."""
    cfg = W.WAN22_QKV_PROJ
    d = W.make_qkv_projection(cfg, device="cuda")
    S, I, hd = cfg.seq, d["out_features"], cfg.head_dim
    nq, nk = cfg.n_q_heads, cfg.n_k_heads
    out = torch.empty(S, I, dtype=cfg.dtype, device="cuda")
    sums = torch.empty(2, S, nq * hd // 128, dtype=torch.float32, device="cuda")
    proj = Q.prepare_qkv_projection(d["a"], d["w"], d["bias"], out=out, q_cols=nq * hd, k_cols=nk * hd,
                                    sumsq=sums)
    q = out[:, : nq * hd].unflatten(-1, (nq, hd)).unsqueeze(0)
    k = out[:, nq * hd: (nq + nk) * hd].unflatten(-1, (nk, hd)).unsqueeze(0)
    qkv_n = torch.empty(1, S, (nq + nk) * hd, dtype=cfg.dtype, device="cuda")   # normalised Q|K
    qo = qkv_n[..., : nq * hd].unflatten(-1, (nq, hd))
    ko = qkv_n[..., nq * hd:].unflatten(-1, (nk, hd))
    apply = Q.prepare_qk_apply_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"], sums,
                                            eps=cfg.eps, q_norm_channels=0, q_out=qo, k_out=ko)
    fused_epilogue = Q.prepare_qk_norm_rope_across_heads(q, k, d["q_gamma"], d["k_gamma"], d["cos"], d["sin"],
                                                         eps=cfg.eps, q_out=qo, k_out=ko)
    out_lib = torch.empty_like(out)
    lib_gemm = lambda: torch.addmm(d["bias"], d["a"], d["w"].t(), out=out_lib)
    return cfg, d, proj, apply, fused_epilogue, lib_gemm


def proj_fp8_measure(torch, W, Q, apply, epilogue):
    """The same projection with FP8 E4M3 operands and ROW_MX scales, next to
    torch._scaled_mm with row-wise scales (hipBLASLt)."""
    cfg = W.WAN22_QKV_PROJ_FP8
    d = W.make_qkv_projection(cfg, device="cuda")
    S, I = cfg.seq, d["out_features"]
    flops = W.flops_qkv_projection(cfg)
    out = torch.empty(S, I, dtype=torch.bfloat16, device="cuda")
    sums = torch.empty(2, S, 40, dtype=torch.float32, device="cuda")
    proj = Q.prepare_qkv_projection(d["a8"], d["w8"], d["bias"], out=out, q_cols=5120, k_cols=5120, sumsq=sums,
                                    a_scale=d["a_scale"], w_scale=d["w_scale"])
    res = {"workload": "the same projection with FP8 E4M3 operands, per-row and per-channel fp32 scales (ROW_MX)"}
    for _ in range(3):
        proj()
    us = time_hot(torch, proj, 10)
    res["projection_with_sums_us"] = round(us, 1)
    res["projection_tflops"] = round(flops / us / 1e6, 1)
    res["projection_frac_fp8_peak"] = round(flops / us / 1e6 / PEAK_FP8_TFLOPS, 4)
    try:
        wt, sa, sb = d["w8"].t(), d["a_scale"][:, None].contiguous(), d["w_scale"][None, :].contiguous()
        lib = lambda: torch._scaled_mm(d["a8"], wt, scale_a=sa, scale_b=sb, bias=d["bias"], out_dtype=torch.bfloat16)
        for _ in range(3):
            lib()
        lus = time_hot(torch, lib, 10)
        res["library_gemm_torch_scaled_mm_us"] = round(lus, 1)
        res["library_gemm_tflops"] = round(flops / lus / 1e6, 1)
    except Exception as e:                      # the library path is a reference only
        res["library_gemm_error"] = str(e)[:200]
    return res


def proj_measure(torch, W, Q):
    cfg, d, proj, apply, epilogue, lib_gemm = proj_setup(torch, W, Q)
    flops = W.flops_qkv_projection(cfg)
    S, hd = cfg.seq, cfg.head_dim
    e = 2
    apply_bytes = S * (2 * (cfg.n_q_heads + cfg.n_k_heads) * hd * e + 2 * hd * e + 2 * 40 * 4) \
        + (cfg.n_q_heads + cfg.n_k_heads) * hd * e
    res = {"workload": "Wan2.2 self-attention QKV projection: A [75600, 5120] @ W^T, W [15360, 5120], "
                       "+ bias, bf16 in/out, fp32 accumulation; then the across-heads norm + RoPE of Q|K",
           "flops": flops}
    for name, fn, it in (("projection_with_sums", proj, 10), ("apply_pass", apply, 30),
                         ("library_gemm_torch_addmm", lib_gemm, 10), ("single_pass_epilogue", epilogue, 30)):
        for _ in range(3):
            fn()
        res[name + "_us"] = round(time_hot(torch, fn, it), 1)
    p_us, lib_us = res["projection_with_sums_us"], res["library_gemm_torch_addmm_us"]
    res["projection_tflops"] = round(flops / p_us / 1e6, 1)
    res["projection_frac_bf16_peak"] = round(flops / p_us / 1e6 / PEAK_BF16_TFLOPS, 4)
    res["library_gemm_tflops"] = round(flops / lib_us / 1e6, 1)
    res["apply_pass_gbs"] = round(apply_bytes / res["apply_pass_us"] / 1e3, 1)
    res["fused_pipeline_us"] = round(p_us + res["apply_pass_us"], 1)
    res["unfused_library_pipeline_us"] = round(lib_us + res["single_pass_epilogue_us"], 1)
    res["roofline"] = {"bound": "mfma", "achieved": res["projection_tflops"], "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": res["projection_frac_bf16_peak"],
                       "traffic": measured_traffic("qkv_proj", "wan22_qkv_projection")}
    del d, proj, lib_gemm
    torch.cuda.empty_cache()
    f8 = proj_fp8_measure(torch, W, Q, apply, epilogue)
    f8["fused_pipeline_us"] = round(f8["projection_with_sums_us"] + res["apply_pass_us"], 1)
    if "library_gemm_torch_scaled_mm_us" in f8:
        f8["unfused_library_pipeline_us"] = round(f8["library_gemm_torch_scaled_mm_us"] +
                                                  res["single_pass_epilogue_us"], 1)
    res["fp8_row_mx"] = f8
    torch.cuda.empty_cache()
    mx = proj_mx_measure(torch, W, Q)
    mx["fused_pipeline_us"] = round(mx["projection_with_sums_us"] + res["apply_pass_us"], 1)
    if "library_gemm_torch_scaled_mm_us" in mx:
        mx["unfused_library_pipeline_us"] = round(mx["library_gemm_torch_scaled_mm_us"] +
                                                  res["single_pass_epilogue_us"], 1)
    res["mxfp8"] = mx
    return res


def proj_mx_measure(torch, W, Q):
    """The same projection with MXFP8 operands (E4M3 codes, one E8M0 scale per
    32 values of hidden on both operands), next to torch._scaled_mm with the
    same block scales where the library supports them."""
    cfg = W.WAN22_QKV_PROJ_MXFP8
    d = W.make_qkv_projection(cfg, device="cuda")
    S, I = cfg.seq, d["out_features"]
    flops = W.flops_qkv_projection(cfg)
    out = torch.empty(S, I, dtype=torch.bfloat16, device="cuda")
    sums = torch.empty(2, S, 40, dtype=torch.float32, device="cuda")
    proj = Q.prepare_qkv_projection(d["a8"], d["w8"], d["bias"], out=out, q_cols=5120, k_cols=5120, sumsq=sums,
                                    a_block_scale=d["a_bs"], w_block_scale=d["w_bs"])
    res = {"workload": "the same projection with MXFP8 operands: E4M3 codes, one E8M0 scale per 32 values of "
                       "hidden on A and on W (OCP MX)"}
    for _ in range(3):
        proj()
    us = time_hot(torch, proj, 10)
    res["projection_with_sums_us"] = round(us, 1)
    res["projection_tflops"] = round(flops / us / 1e6, 1)
    res["projection_frac_fp8_peak"] = round(flops / us / 1e6 / PEAK_FP8_TFLOPS, 4)
    try:
        sa, sb = d["a_bs"].view(torch.float8_e8m0fnu), d["w_bs"].view(torch.float8_e8m0fnu)
        wt = d["w8"].t()
        lib = lambda: torch._scaled_mm(d["a8"], wt, scale_a=sa, scale_b=sb, bias=None, out_dtype=torch.bfloat16)
        for _ in range(3):
            lib()
        lus = time_hot(torch, lib, 10)
        res["library_gemm_torch_scaled_mm_us"] = round(lus, 1)
        res["library_gemm_tflops"] = round(flops / lus / 1e6, 1)
    except Exception as e:                      # the library path is a reference only
        res["library_gemm_error"] = str(e)[:200]
    return res


def kv_setup(torch, W, Q, cfg, **override):
    d = W.make_kv_cache(cfg, device="cuda", prefill=False, **override)
    cfg = d["cfg"]
    mode = {W.NORM: "Norm", W.PA_BNSD: "PA_BNSD", W.PA_BLK_BNSD: "PA_BLK_BNSD"}[cfg.cache_mode]

    def make(stream=None):
        return Q.prepare_kv_rmsnorm_rope_cache(
            d["kv"], d["gamma"], d["cos"], d["sin"], d["index"], d["k_cache"], d["ckv_cache"],
            k_rope_scale=d["k_scale"], k_rope_offset=d["k_offset"], c_kv_scale=d["v_scale"],
            c_kv_offset=d["v_offset"], v=d["v"], epsilon=cfg.eps, cache_mode=mode,
            is_output_kv=cfg.is_output_kv, k_rope=d["k_rope"], c_kv=d["c_kv"], stream=stream)
    step = make()
    step.make = make                   # a launcher on another stream (graph capture)
    return d, step


def time_hot(torch, step, iters):
    """Back-to-back launches bracketed by one event pair on the launch stream."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(iters):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3   # us per launch


def time_cold(torch, step, iters, flush, how="write"):
    """Median time of launches each timed alone after a pass over a 1 GiB
    scratch tensor that evicts L2 and the 256 MB MALL. how='write' fills the
    tensor (the stated cold protocol: the dirty lines it leaves are written
    back while the timed launch runs, as after any producer kernel);
    how='read' sums it, which leaves clean lines (nothing to write back)."""
    s = torch.cuda.current_stream()
    sink = torch.zeros((), dtype=flush.dtype, device=flush.device)
    times = []
    for i in range(iters):
        if how == "write":
            flush.fill_(float(i & 1))
        else:
            sink.copy_(flush.sum())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        step()
        e1.record(s)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    times.sort()
    return times[len(times) // 2]


def cold_record(torch, step, iters, flush, nbytes):
    """Cold medians under both flushes: us_cold_median / frac_cold after a
    1 GiB write (the stated protocol), us_cold_read_median / frac_cold_read
    after a 1 GiB read."""
    w = time_cold(torch, step, iters, flush, "write")
    r = time_cold(torch, step, iters, flush, "read")
    return {"us_cold_median": round(w, 3), "gbs_cold": round(nbytes / w / 1e3, 1),
            "frac_cold": round(nbytes / w / 1e3 / PEAK_HBM_GBS, 4),
            "us_cold_read_median": round(r, 3), "gbs_cold_read": round(nbytes / r / 1e3, 1),
            "frac_cold_read": round(nbytes / r / 1e3 / PEAK_HBM_GBS, 4)}


def cpu_baseline(torch, W, d, cfg):
    """The fp64 oracle on the first `n` tokens of the same workload."""
    import numpy as np
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    threads = max(1, min(threads, len(os.sched_getaffinity(0))))
    hd, nq, nk = cfg.head_dim, cfg.n_q_heads, cfg.n_k_heads
    qkv = d["qkv"]

    def sample(n):
        flat = qkv.reshape(-1, qkv.shape[-1])[:n]
        bits = flat.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        cs = d["cos"].reshape(-1, hd)[:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        sn = d["sin"].reshape(-1, hd)[:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        g = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        return (np.ascontiguousarray(bits[:, : nq * hd]), np.ascontiguousarray(bits[:, nq * hd:]),
                g(d["q_gamma"]), g(d["k_gamma"]), cs, sn)

    def run(n):
        args = sample(n)
        t0 = time.perf_counter()
        oracle.qk_norm_rope_across_heads(*args, cfg.eps, nq, nk, hd, oracle.BF16, nthreads=threads,
                                         values=False)
        return time.perf_counter() - t0

    def run1(n):
        args = sample(n)
        t0 = time.perf_counter()
        oracle.qk_norm_rope_across_heads(*args, cfg.eps, nq, nk, hd, oracle.BF16, nthreads=1, values=False)
        return time.perf_counter() - t0

    probe = 2048
    t_probe = run(probe)
    # about 20 s of oracle CPU time (threads x wall), at most the whole workload
    n = int(min(cfg.seq, max(probe, probe * 20.0 / max(t_probe * threads, 1e-6))))
    t = sorted(run(n) for _ in range(3))[1]
    n1 = 4096
    t1 = run1(n1)
    per_token = W.algorithmic_bytes_across_heads(cfg) / cfg.seq
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    res = {"value": round(n * per_token / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "tokens_per_s": round(n / t, 1), "seconds": round(t, 3), "cpu_model": model,
           "one_thread": {"value": round(n1 * per_token / t1 / 1e9, 4), "unit": "GB/s", "tokens": n1,
                          "seconds": round(t1, 3)},
           "sample": f"first {n} of {cfg.seq} tokens of the same workload (median of 3 runs), fp64 C oracle, "
                     f"OpenMP over tokens, {threads} threads, bf16 outputs encoded; one_thread: first {n1} "
                     f"tokens on 1 thread"}
    per = {"wan22_self_attn": {
        "tokens": cfg.seq, "sampled": n < cfg.seq,
        "all_cores": {"threads": threads, "tokens": n, "seconds": round(t, 4), "tokens_per_s": round(n / t, 1),
                      "gbs": res["value"]},
        "one_thread": {"threads": 1, "tokens": n1, "seconds": round(t1, 4), "tokens_per_s": round(n1 / t1, 1),
                       "gbs": round(n1 * per_token / t1 / 1e9, 4)}}}
    per.update(cpu_other_configs(torch, W, threads))
    res["per_config"] = per
    return res


def cpu_other_configs(torch, W, threads):
    """The oracle on the other four workloads, in full, on all cores (median
    of 3 runs) and on one thread (one run): the tiny across-heads case and the
    three MLA cache workloads (inputs drawn on the host with the same recipe,
    caches zero-filled host arrays updated in place)."""
    import numpy as np
    import oracle

    def host(t):
        t = t.contiguous()
        if t.dtype in (torch.bfloat16, torch.float16):
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2]

    def record(fn, tokens, nbytes, loops=1):
        out = {"tokens": tokens}
        for key, th, reps in (("all_cores", threads, 3), ("one_thread", 1, 1)):
            sec = timed(lambda: [fn(th) for _ in range(loops)], reps) / loops
            out[key] = {"threads": th, "seconds": round(sec, 6), "tokens_per_s": round(tokens / sec, 1),
                        "gbs": round(nbytes / sec / 1e9, 4)}
        return out

    per = {}
    c1 = W.TINY_ACROSS_HEADS
    d1 = W.make_across_heads(c1, device="cpu")
    hd, nq, nk = c1.head_dim, c1.n_q_heads, c1.n_k_heads
    flat = d1["qkv"].reshape(-1, d1["qkv"].shape[-1])
    args1 = (np.ascontiguousarray(host(flat[:, : nq * hd])), np.ascontiguousarray(host(flat[:, nq * hd:])),
             host(d1["q_gamma"]), host(d1["k_gamma"]), host(d1["cos"].reshape(-1, hd)),
             host(d1["sin"].reshape(-1, hd)))
    dt1 = {torch.float32: oracle.F32, torch.bfloat16: oracle.BF16}[c1.dtype]
    per[c1.name] = record(lambda th: oracle.qk_norm_rope_across_heads(*args1, c1.eps, nq, nk, hd, dt1, nthreads=th,
                                                                      values=False),
                          c1.batch * c1.seq, W.algorithmic_bytes_across_heads(c1), loops=200)
    codes = {torch.bfloat16: oracle.BF16, torch.float16: oracle.F16, torch.int8: oracle.INT8,
             torch.float8_e4m3fn: oracle.E4M3FN, torch.float8_e5m2: oracle.E5M2}
    modes = {W.NORM: oracle.NORM, W.PA_BNSD: oracle.PA_BNSD, W.PA_BLK_BNSD: oracle.PA_BLK_BNSD}
    for cfg in (W.MLA_V1_PREFILL, W.MLA_V1_DECODE_QUANT, W.MLA_V2_SPLIT):
        d = W.make_kv_cache(cfg, device="cpu", prefill=False)
        kc = np.zeros(tuple(d["k_cache"].shape), oracle.STORAGE[codes[cfg.k_cache_dtype]])
        cc = np.zeros(tuple(d["ckv_cache"].shape), oracle.STORAGE[codes[cfg.ckv_cache_dtype]])
        q = lambda t: None if t is None else t.numpy()
        ins = dict(kv=host(d["kv"]), v=None if d["v"] is None else host(d["v"]), gamma=host(d["gamma"]),
                   cos=host(d["cos"]), sin=host(d["sin"]), index=d["index"].numpy())

        def run(th, cfg=cfg, ins=ins, kc=kc, cc=cc, d=d):
            oracle.kv_rmsnorm_rope_cache(
                ins["kv"], ins["v"], ins["gamma"], ins["cos"], ins["sin"], ins["index"], kc, cc,
                rms_size=cfg.rms_size, rope_size=cfg.rope_size, eps=cfg.eps, cache_mode=modes[cfg.cache_mode],
                in_dtype=codes[cfg.dtype], k_dtype=codes[cfg.k_cache_dtype], ckv_dtype=codes[cfg.ckv_cache_dtype],
                block_size=cfg.block_size, k_scale=q(d["k_scale"]), k_offset=q(d["k_offset"]),
                v_scale=q(d["v_scale"]), v_offset=q(d["v_offset"]), is_output_kv=cfg.is_output_kv,
                nthreads=th, copy_caches=False)
        per[cfg.name] = record(run, cfg.batch * cfg.seq, W.algorithmic_bytes_kv_cache(cfg),
                               loops=20 if cfg.batch * cfg.heads * cfg.seq < 4096 else 1)
        del d, ins, kc, cc
    return per


def graph_replay_us(torch, step, calls=100, replays=20):
    """Per-call time of `calls` launches captured in one HIP graph, replayed
    back to back (launch overhead amortised)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    side = step.make(s)
    for _ in range(3):
        side()                         # warm up on a side stream, as capture requires
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step.make(torch.cuda.current_stream())
        for _ in range(calls):
            captured()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * calls)


def kv_measure(torch, W, Q, flush, cold_iters):
    out = {}
    torch.cuda.empty_cache()          # each workload's tensors come from fresh allocations
    for name, cfg, over in (("mla_v1_prefill", W.MLA_V1_PREFILL, {}),
                            ("mla_v1_prefill_pa_blk_bnsd", W.MLA_V1_PREFILL, {"cache_mode": W.PA_BLK_BNSD}),
                            ("mla_v1_decode_quant", W.MLA_V1_DECODE_QUANT, {}),
                            ("mla_v2_split", W.MLA_V2_SPLIT, {})):
        d, step = kv_setup(torch, W, Q, cfg, **over)
        cfg = d["cfg"]
        for _ in range(5):
            step()
        # back-to-back launches: one untimed run of 200 first (the first
        # milliseconds of a new workload run 2-4 % slower while the clocks
        # settle), then the median of three runs of 200
        time_hot(torch, step, 200)
        hot = sorted(time_hot(torch, step, 200) for _ in range(3))[1]
        nbytes = W.algorithmic_bytes_kv_cache(cfg)
        tokens = cfg.batch * cfg.seq
        rec = {"algorithmic_bytes": nbytes, "tokens": tokens, "rows": cfg.batch * cfg.heads * cfg.seq,
               "us_hot_mean": round(hot, 3), "gbs_hot": round(nbytes / hot / 1e3, 1),
               "frac_hot": round(nbytes / hot / 1e3 / PEAK_HBM_GBS, 4)}
        rec.update(cold_record(torch, step, cold_iters, flush, nbytes))
        rec["tokens_per_s_cold"] = round(tokens / rec["us_cold_median"] * 1e6, 1)
        rec["traffic"] = measured_traffic("kv_rmsnorm_rope_cache", name)
        if name == "mla_v1_decode_quant":
            rec["us_graph_replay_per_call"] = round(graph_replay_us(torch, step), 3)
        out[name] = rec
        del d, step
        torch.cuda.empty_cache()
    return out


def profile_run(torch, W, Q, which):
    """A short fixed run of one kernel for counter collection under rocprofv3."""
    if which == "copy":
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "copy", "bytes_read": n, "bytes_written": n, "launches": 5}))
        return
    if which == "across":
        cfg, d, step = across_setup(torch, W, Q)
    elif which in ("per_head", "split_sumsq", "split_apply"):
        step = forms_setup(torch, W, Q, which)
    elif which == "proj":
        step = proj_setup(torch, W, Q)[2]
    elif which == "proj_lib":                  # the library GEMM of the same projection (hipBLASLt)
        step = proj_setup(torch, W, Q)[5]
    elif which == "proj_fp8_lib":
        d = W.make_qkv_projection(W.WAN22_QKV_PROJ_FP8, device="cuda")
        wt, sa, sb = d["w8"].t(), d["a_scale"][:, None].contiguous(), d["w_scale"][None, :].contiguous()
        step = lambda: torch._scaled_mm(d["a8"], wt, scale_a=sa, scale_b=sb, bias=d["bias"],
                                        out_dtype=torch.bfloat16)
    elif which in ("proj_fp8", "proj_mxfp8"):
        mx = which == "proj_mxfp8"
        d = W.make_qkv_projection(W.WAN22_QKV_PROJ_MXFP8 if mx else W.WAN22_QKV_PROJ_FP8, device="cuda")
        out = torch.empty(d["cfg"].seq, d["out_features"], dtype=torch.bfloat16, device="cuda")
        sums = torch.empty(2, d["cfg"].seq, 40, dtype=torch.float32, device="cuda")
        sc = (dict(a_block_scale=d["a_bs"], w_block_scale=d["w_bs"]) if mx else
              dict(a_scale=d["a_scale"], w_scale=d["w_scale"]))
        step = Q.prepare_qkv_projection(d["a8"], d["w8"], d["bias"], out=out, q_cols=5120, k_cols=5120,
                                        sumsq=sums, **sc)
    elif which == "kv_v1_prefill_pa_blk":
        d, step = kv_setup(torch, W, Q, W.MLA_V1_PREFILL, cache_mode=W.PA_BLK_BNSD)
    else:
        cfg = {"kv_v1_prefill": W.MLA_V1_PREFILL, "kv_v1_decode": W.MLA_V1_DECODE_QUANT,
               "kv_v2": W.MLA_V2_SPLIT}[which]
        d, step = kv_setup(torch, W, Q, cfg)
    torch.cuda.synchronize()
    for _ in range(5):
        step()
    torch.cuda.synchronize()
    print(json.dumps({"profile": which, "launches": 5}))


# profile target -> (kernel source group, workload, a substring naming the kernel
# instantiation: the QK forms differ in the last template argument)
PROFILE_WORKLOADS = {
    "across": ("qk_across_heads", "wan22_self_attn", ", 0>(qknr::QkParams)"),
    "per_head": ("qk_per_head", "wan22_per_head", ", 1>(qknr::QkParams)"),
    "split_sumsq": ("qk_split", "wan22_split_sumsq", ", 2>(qknr::QkParams)"),
    "split_apply": ("qk_split", "wan22_split_apply", ", 3>(qknr::QkParams)"),
    "proj": ("qkv_proj", "wan22_qkv_projection", "qkv_proj_kernel<false, false, 384>"),
    "proj_fp8": ("qkv_proj", "wan22_qkv_projection_fp8", "qkv_proj_kernel<true, false, 384>"),
    "proj_mxfp8": ("qkv_proj", "wan22_qkv_projection_mxfp8", "qkv_proj_kernel<true, true, 256>"),
    "kv_v1_prefill": ("kv_rmsnorm_rope_cache", "mla_v1_prefill", "kv_rmsnorm_rope_cache_kernel"),
    "kv_v1_prefill_pa_blk": ("kv_rmsnorm_rope_cache", "mla_v1_prefill_pa_blk_bnsd", "kv_rmsnorm_rope_cache_kernel"),
    "kv_v1_decode": ("kv_rmsnorm_rope_cache", "mla_v1_decode_quant", "kv_rmsnorm_rope_cache_kernel"),
    "kv_v2": ("kv_rmsnorm_rope_cache", "mla_v2_split", "kv_rmsnorm_rope_cache_kernel"),
}


def summarize(prof_dir):
    """Write profiles/*.txt and profiles/pmc_traffic.json from rocprofv3 CSVs:
    <dir>/trace/*_kernel_trace.csv (kernel durations of a bench run) and
    <dir>/pmc_{fetch,write}_<workload>/*_counter_collection.csv."""
    import csv
    import glob
    import statistics
    import workloads as W

    def counters(kind, w):
        files = glob.glob(os.path.join(prof_dir, f"pmc_{kind}_{w}", "*counter_collection.csv"))
        vals = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    def pick(vals, needle):
        hits = [v for k, v in vals.items() if needle in k]
        return statistics.mean(hits[0]) if hits else None

    # calibration: the same counters on a plain 1 GiB copy (read 1 GiB, write 1 GiB)
    cf, cw = pick(counters("fetch", "copy"), "copy"), pick(counters("write", "copy"), "copy")
    kib = (1 << 30) / 1024
    f_scale, w_scale = kib / cf, kib / cw
    trace = glob.glob(os.path.join(prof_dir, "trace", "*kernel_trace.csv"))
    durs = {}
    for f in trace:
        for r in csv.DictReader(open(f)):
            if "qknr::" in r["Kernel_Name"]:
                key = (r["Kernel_Name"], r["Grid_Size_X"])
                durs.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    cfgs = {"wan22_self_attn": W.WAN22_SELF_ATTN, "mla_v1_prefill": W.MLA_V1_PREFILL,
            "mla_v1_prefill_pa_blk_bnsd": dataclasses.replace(W.MLA_V1_PREFILL, cache_mode=W.PA_BLK_BNSD),
            "mla_v1_decode_quant": W.MLA_V1_DECODE_QUANT, "mla_v2_split": W.MLA_V2_SPLIT}
    # trace lines are keyed by kernel and grid; workloads that share both share the line
    shared = {}
    for prof, (kernel, wname, needle) in PROFILE_WORKLOADS.items():
        kn = [k for k in counters("fetch", prof) if needle in k]
        if not kn:
            continue
        for fpath in glob.glob(os.path.join(prof_dir, f"pmc_fetch_{prof}", "*counter_collection.csv")):
            for g in {r["Grid_Size"] for r in csv.DictReader(open(fpath)) if r["Kernel_Name"] == kn[0]}:
                shared.setdefault((kn[0], g), []).append(wname)
    record = {"calibration": {"copy_bytes": 1 << 30, "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw,
                              "fetch_scale": f_scale, "write_scale": w_scale},
              "kernels": {}}
    lines_by_kernel = {}
    for prof, (kernel, wname, needle) in PROFILE_WORKLOADS.items():
        fv, wv = counters("fetch", prof), counters("write", prof)
        f, w = pick(fv, needle), pick(wv, needle)
        if f is None or w is None:
            continue
        if wname.startswith("wan22_qkv_projection"):
            c = W.WAN22_QKV_PROJ      # compulsory bytes: A, W (and scales), bias read once; out, sums written once
            eb = 1 if wname.endswith("fp8") else 2
            alg = eb * (c.seq * c.hidden + 15360 * c.hidden) + 2 * (15360 + c.seq * 15360) + 4 * 2 * 40 * c.seq
            if wname.endswith("mxfp8"):
                alg += (c.seq + 15360) * c.hidden // 32      # the E8M0 block scales
            elif eb == 1:
                alg += 4 * (c.seq + 15360)
        elif wname == "wan22_per_head":
            alg = W.algorithmic_bytes_per_head(W.WAN22_SELF_ATTN)
        elif wname.startswith("wan22_split"):
            alg = W.algorithmic_bytes_qk_split(W.WAN22_SELF_ATTN, 4)[0 if wname.endswith("sumsq") else 1]
        elif kernel == "qk_across_heads":
            alg = W.algorithmic_bytes_across_heads(cfgs[wname])
        else:
            alg = W.algorithmic_bytes_kv_cache(cfgs[wname])
        hbm = f * 1024 * f_scale + w * 1024 * w_scale
        record["kernels"][wname] = {"kernel": kernel, "source_hash": source_hash(kernel),
                                    "FETCH_SIZE_KiB": f, "WRITE_SIZE_KiB": w,
                                    "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes": alg,
                                    "traffic_over_algorithmic": round(hbm / alg, 4)}
        kname = [k for k in fv if needle in k][0]
        grids = set()
        for fpath in glob.glob(os.path.join(prof_dir, f"pmc_fetch_{prof}", "*counter_collection.csv")):
            grids |= {r["Grid_Size"] for r in csv.DictReader(open(fpath)) if r["Kernel_Name"] == kname}
        lines = lines_by_kernel.setdefault(kernel, [])
        lines.append(f"workload {wname}: kernel {kname}")
        for (k, g), v in sorted(durs.items()):
            if k == kname and g in grids:
                both = shared.get((k, g), [wname])
                note = f" (the dispatches of {' and '.join(both)})" if len(both) > 1 else ""
                lines.append(f"  trace grid {g}{note}: {len(v)} dispatches, median {statistics.median(v):.2f} us, "
                             f"mean {statistics.mean(v):.2f} us, min {min(v):.2f} us, max {max(v):.2f} us")
        lines.append(f"  FETCH_SIZE {f:.1f} KiB x {f_scale:.4f} + WRITE_SIZE {w:.1f} KiB x {w_scale:.4f} "
                     f"= {hbm / 1e6:.3f} MB per launch; algorithmic {alg / 1e6:.3f} MB "
                     f"(ratio {hbm / alg:.4f})")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json"), "w") as fjs:
        json.dump(record, fjs, indent=1)
    cmds = ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o bench -- "
            "python -u bench.py --steps 100 --warmup 10 --no-cpu\n"
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_fetch_<w> -o p -- "
            "python -u bench.py --profile <w>\n"
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_write_<w> -o p -- "
            "python -u bench.py --profile <w>\n"
            "  for <w> in across per_head split_sumsq split_apply proj proj_fp8 proj_mxfp8 kv_v1_prefill "
            "kv_v1_prefill_pa_blk kv_v1_decode kv_v2 copy;\n"
            "  then "
            "python bench.py --summarize <dir>\n")
    calib = (f"calibration (copy of 1 GiB, __amd_rocclr_copyBuffer): FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE "
             f"{cw:.1f} KiB -> scale fetch x{f_scale:.4f}, write x{w_scale:.4f}\n")
    names = {"qk_across_heads": "qk_across_heads_wan22_s75600.txt",
             "qk_per_head": "qk_per_head_wan22_s75600.txt",
             "qk_split": "qk_split_passes_wan22_tp4_shard.txt",
             "qkv_proj": "qkv_projection_wan22_s75600.txt",
             "kv_rmsnorm_rope_cache": "kv_rmsnorm_rope_cache_mla_workloads.txt"}
    for kernel, lines in lines_by_kernel.items():
        with open(os.path.join(ROOT, "profiles", names[kernel]), "w") as ftxt:
            ftxt.write(f"MI355X (gfx950), rocprofv3 summaries for {kernel}\n\ncommands:\n{cmds}\n{calib}\n")
            ftxt.write("\n".join(lines) + "\n")
    print(json.dumps(record, indent=1))


STREAM_LIB = os.path.join(ROOT, "libbench_stream.so")


def ceiling(torch, W, Q, cold_iters):
    """Same-process sweep of plain stream kernels (bench_stream.hip) that read
    and write the operators' byte mixes at 32 MB - 3.1 GB, hot (back to back)
    and cold after a 1 GiB write and after a 1 GiB read, next to the three
    bandwidth-bound operators at their own sizes; the persistent-grid form of
    the stream at the operators' sizes as well."""
    import ctypes
    lib = ctypes.CDLL(STREAM_LIB)
    lib.bench_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_void_p]
    lib.bench_stream.restype = ctypes.c_int
    mb = 1 << 20
    mixes = {"mla_v1_prefill": W.algorithmic_read_write_kv_cache(W.MLA_V1_PREFILL),
             "mla_v2_split": W.algorithmic_read_write_kv_cache(W.MLA_V2_SPLIT),
             "wan22_self_attn": W.algorithmic_read_write_across_heads(W.WAN22_SELF_ATTN),
             "write_only": (0, 1), "read_only": (1, 0)}
    own = {k: sum(v) for k, v in mixes.items() if k in ("mla_v1_prefill", "mla_v2_split", "wan22_self_attn")}
    sizes = sorted({32 * mb, 64 * mb, 256 * mb, 512 * mb, 1024 * mb, 3135 * mb} | set(own.values()))
    top = max(sizes)
    src = torch.empty(top, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(top, dtype=torch.uint8, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rows = []

    def measure(name, total, rfrac_pair, nt_store, grid):
        r, w = rfrac_pair
        rb = (total * r // (r + w)) // 16 * 16
        wb = (total - rb) // 16 * 16
        step = lambda: lib.bench_stream(src.data_ptr(), rb, dst.data_ptr(), wb, nt_store, grid, stream)
        if step() != 0:
            raise RuntimeError("stream launch failed")
        for _ in range(3):
            step()
        hot = sorted(time_hot(torch, step, 20) for _ in range(3))[1]
        rec = {"mix": name, "bytes": rb + wb, "read_bytes": rb, "write_bytes": wb, "nt_store": nt_store,
               "grid": grid or "one piece per thread", "us_hot": round(hot, 3),
               "frac_hot": round((rb + wb) / hot / 1e3 / PEAK_HBM_GBS, 4)}
        rec.update(cold_record(torch, step, cold_iters, flush, rb + wb))
        rows.append(rec)
        print(json.dumps(rec), flush=True)

    for name, pair in mixes.items():
        for total in sizes:
            for nt in (1, 0):
                measure(name, total, pair, nt, 0)
    for name in own:
        for grid in (1024, 2048, 4096, 8192):
            measure(name, own[name], mixes[name], 1, grid)
    del src, dst
    torch.cuda.empty_cache()
    ops = {}
    for name, cfg in (("mla_v1_prefill", W.MLA_V1_PREFILL), ("mla_v2_split", W.MLA_V2_SPLIT)):
        d, step = kv_setup(torch, W, Q, cfg)
        for _ in range(5):
            step()
        time_hot(torch, step, 200)
        hot = sorted(time_hot(torch, step, 200) for _ in range(3))[1]
        nbytes = W.algorithmic_bytes_kv_cache(cfg)
        ops[name] = {"bytes": nbytes, "us_hot": round(hot, 3), "frac_hot": round(nbytes / hot / 1e3 / PEAK_HBM_GBS, 4)}
        ops[name].update(cold_record(torch, step, cold_iters, flush, nbytes))
        del d, step
        torch.cuda.empty_cache()
    cfg, d, step = across_setup(torch, W, Q)
    for _ in range(5):
        step()
    nbytes = W.algorithmic_bytes_across_heads(cfg)
    hot = time_hot(torch, step, 20)
    ops["wan22_self_attn"] = {"bytes": nbytes, "us_hot": round(hot, 3),
                              "frac_hot": round(nbytes / hot / 1e3 / PEAK_HBM_GBS, 4)}
    ops["wan22_self_attn"].update(cold_record(torch, step, cold_iters, flush, nbytes))
    for name, rec in ops.items():
        print(json.dumps(dict(rec, operator=name)), flush=True)
    print(ceiling_table(rows, ops))


def ceiling_table(rows, ops):
    """The sweep as a text table: fraction of 8 TB/s hot / cold (write flush) /
    cold (read flush) per mix and size, best of the store kinds, and the
    operators at their sizes."""
    out = ["fraction of 8 TB/s: hot | cold after 1 GiB write | cold after 1 GiB read "
           "(plain stream, best of nt / ordinary stores, one piece per thread)"]
    mixes = []
    for r in rows:
        if r["mix"] not in mixes:
            mixes.append(r["mix"])
    for mix in mixes:
        out.append(f"{mix}:")
        sizes = sorted({r["bytes"] for r in rows if r["mix"] == mix and r["grid"] == "one piece per thread"})
        for b in sizes:
            rs = [r for r in rows if r["mix"] == mix and r["bytes"] == b and r["grid"] == "one piece per thread"]
            best = lambda k: max(r[k] for r in rs)
            out.append(f"  {b / 1e6:9.1f} MB  {best('frac_hot'):.3f} | {best('frac_cold'):.3f} | "
                       f"{best('frac_cold_read'):.3f}   ({min(r['us_cold_median'] for r in rs):.2f} us cold)")
        ps = [r for r in rows if r["mix"] == mix and r["grid"] != "one piece per thread"]
        for r in ps:
            out.append(f"  persistent grid {r['grid']:>5} blocks, {r['bytes'] / 1e6:.1f} MB: {r['frac_hot']:.3f} | "
                       f"{r['frac_cold']:.3f} | {r['frac_cold_read']:.3f}")
    out.append("operators (same process):")
    for name, r in ops.items():
        out.append(f"  {name:16s} {r['bytes'] / 1e6:9.1f} MB  {r['frac_hot']:.3f} | {r['frac_cold']:.3f} | "
                   f"{r['frac_cold_read']:.3f}   ({r['us_hot']:.2f} us hot, {r['us_cold_median']:.2f} us cold)")
    return "\n".join(out)


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is described, not built)"}))
        sys.exit(2)
    import torch
    import qk_rmsnorm_rope_amd as Q
    import workloads as W
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.profile:
        profile_run(torch, W, Q, args.profile)
        return
    if args.ceiling:
        ceiling(torch, W, Q, args.cold_iters)
        return

    cfg, d, step = across_setup(torch, W, Q)
    nbytes = W.algorithmic_bytes_across_heads(cfg)
    tokens = cfg.batch * cfg.seq
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_us = e0.elapsed_time(e1) / args.steps * 1e3
    achieved = nbytes / launch_us / 1e3          # GB/s per launch
    value = nbytes * args.steps / wall / 1e9

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")    # 1 GiB
    cold = cold_record(torch, step, args.cold_iters, flush, nbytes)
    copy_src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    copy_dst = torch.empty_like(copy_src)
    copy_us = time_hot(torch, lambda: copy_dst.copy_(copy_src), 20)
    del copy_src, copy_dst

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "io_dtype": "bf16", "data": "synthetic",
        "config": {"workload": "wan22_self_attn: across-heads QK RMSNorm + rotate-half RoPE, S=75600 "
                               "(21x45x80), Q and K 40 heads x 128, BSD [1,75600,10240] bf16, out of place",
                   "global_batch": 1, "seq_len": cfg.seq, "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(tokens * args.steps / wall, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("qk_across_heads", cfg.name),
                     "kernel": "qk_across_heads_kernel", "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(launch_us, 3), "cold_launch_us_median": cold["us_cold_median"],
                     "frac_cold": cold["frac_cold"], "cold_read_launch_us_median": cold["us_cold_read_median"],
                     "frac_cold_read": cold["frac_cold_read"]},
        "copy_reference": {"what": "1 GiB device-to-device copy (hipMemcpy), read + write bytes / time",
                           "gbs": round(2 * (1 << 30) / copy_us / 1e3, 1),
                           "frac": round(2 * (1 << 30) / copy_us / 1e3 / PEAK_HBM_GBS, 4)},
    }
    if not args.no_forms:
        result["qk_forms"] = forms_measure(torch, W, Q, d, flush, args.cold_iters)
    if not args.no_kv:
        result["kv_rmsnorm_rope_cache"] = kv_measure(torch, W, Q, flush, args.cold_iters)
    if not args.no_proj:
        result["qkv_projection"] = proj_measure(torch, W, Q)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(torch, W, d, cfg)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
