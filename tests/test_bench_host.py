"""Host-side checks of bench.py (no GPU): the one-GPU rule of its command line,
and that the committed HBM counter record still belongs to the committed kernel
sources (bench.py reports a traffic figure only while the source hash of the
kernel matches the one the counters were taken on; a kernel edited without
re-running the counters would silently lose its traffic figure)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (module import runs nothing: main() is behind __name__)

# profiled workload -> kernel source group, as bench.py's --summarize writes them
WORKLOAD_KERNEL = {
    "wan22_self_attn": "qk_across_heads", "wan22_per_head": "qk_per_head", "wan22_split_sumsq": "qk_split",
    "wan22_split_apply": "qk_split", "wan22_qkv_projection": "qkv_proj", "wan22_qkv_projection_fp8": "qkv_proj", "wan22_qkv_projection_mxfp8": "qkv_proj",
    "mla_v1_prefill": "kv_rmsnorm_rope_cache", "mla_v1_prefill_pa_blk_bnsd": "kv_rmsnorm_rope_cache",
    "mla_v1_decode_quant": "kv_rmsnorm_rope_cache",
    "mla_v2_split": "kv_rmsnorm_rope_cache",
}


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1]
    assert "one GPU" in json.loads(line)["error"]


def test_counter_record_matches_the_committed_kernel_sources():
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json")) as f:
        rec = json.load(f)
    assert set(rec["kernels"]) == set(WORKLOAD_KERNEL)
    for workload, kernel in WORKLOAD_KERNEL.items():
        entry = rec["kernels"][workload]
        assert entry["source_hash"] == bench.source_hash(kernel), (
            f"{workload}: the counters were taken on other {kernel} sources; re-run the counter passes")
        got = bench.measured_traffic(kernel, workload)
        assert isinstance(got, int) and got > 0


def test_traffic_is_within_a_few_percent_of_the_algorithmic_bytes():
    """The bandwidth kernels move what they must and little more (the decode
    launch's index and partial-line reads aside)."""
    import workloads as W
    alg = {"wan22_self_attn": W.algorithmic_bytes_across_heads(W.WAN22_SELF_ATTN),
           "mla_v1_prefill": W.algorithmic_bytes_kv_cache(W.MLA_V1_PREFILL),
           "mla_v2_split": W.algorithmic_bytes_kv_cache(W.MLA_V2_SPLIT)}
    for workload, nbytes in alg.items():
        kernel = WORKLOAD_KERNEL[workload]
        ratio = bench.measured_traffic(kernel, workload) / nbytes
        assert 0.99 < ratio < 1.02, (workload, ratio)


def test_source_hash_ignores_comments_but_not_code():
    src = 'int f(int a) {  // doubles a\n    /* the "result" */\n    return a * 2;   \n}\nconst char *s = "x // y";\n'
    assert bench.strip_comments(src) == bench.strip_comments(src.replace("doubles a", "twice a"))
    assert bench.strip_comments(src) != bench.strip_comments(src.replace("a * 2", "a * 3"))
    assert '"x // y"' in bench.strip_comments(src)
