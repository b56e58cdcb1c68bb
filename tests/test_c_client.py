"""The C ABI used from plain C, without Python: a C program includes
include/qknr.h, links libqknr.so and calls the host-only entry points
(version, argument validation, the thread's last error). Host memory stands
in for the device pointers: validation reads only the argument struct
(shapes, strides, types, flags and pointer alignment), never the data, and
nothing is launched. Checks: a legal V1 call into a paged bf16 cache
validates; a V1 call with N = 2, a quantised cache without its scale and an
odd rope size are INVALID_ARGUMENT with a message naming the problem; an
unbuilt cache mode is UNSUPPORTED; a NULL struct is rejected, not a crash.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "qk_rmsnorm_rope_amd")

C_SOURCE = r"""
#include <stdio.h>
#include <string.h>
#include "qknr.h"

/* host bytes standing in for device memory (validation never dereferences) */
static _Alignas(256) unsigned char mem[1 << 16];

static qknr_kv_args v1_paged(void) {
    const int64_t B = 2, N = 1, S = 130, D = 576, R = 64, bs = 128;
    qknr_kv_args a;
    memset(&a, 0, sizeof a);
    a.dtype = QKNR_BF16;
    a.heads = (int32_t)N; a.batch = B; a.seq = S;
    a.kv_dim = (int32_t)D; a.rms_size = (int32_t)(D - R); a.rope_size = (int32_t)R;
    a.kv = mem; a.gamma = mem; a.cos = mem; a.sin = mem; a.index = (const int64_t *)mem;
    a.kv_strides[0] = N * S * D; a.kv_strides[1] = S * D; a.kv_strides[2] = D;
    a.rope_strides[0] = N * S * R; a.rope_strides[1] = S * R; a.rope_strides[2] = R;
    a.cache_mode = QKNR_CACHE_PA_BNSD; a.block_size = (int32_t)bs; a.cache_rows = 4;
    a.k_cache = mem; a.ckv_cache = mem;
    a.k_cache_dtype = QKNR_BF16; a.ckv_cache_dtype = QKNR_BF16;
    a.k_cache_strides[0] = bs * N * R; a.k_cache_strides[1] = N * R; a.k_cache_strides[2] = R;
    a.ckv_cache_strides[0] = bs * N * (D - R); a.ckv_cache_strides[1] = N * (D - R);
    a.ckv_cache_strides[2] = D - R;
    a.eps = 1e-5f;
    return a;
}

static void report(const char *what, int32_t rc) {
    printf("%s %d %s\n", what, (int)rc, rc ? qknr_last_error() : "-");
}

int main(void) {
    printf("version %d\n", (int)qknr_version());
    qknr_kv_args a = v1_paged();
    report("valid", qknr_kv_validate(&a));
    a = v1_paged(); a.heads = 2;
    report("v1_two_heads", qknr_kv_validate(&a));
    a = v1_paged(); a.k_cache_dtype = QKNR_INT8;
    report("int8_without_scale", qknr_kv_validate(&a));
    a = v1_paged(); a.rope_size = 63; a.rms_size = 513;
    report("odd_rope", qknr_kv_validate(&a));
    a = v1_paged(); a.cache_mode = 7;
    report("unbuilt_mode", qknr_kv_validate(&a));
    report("null_args", qknr_kv_validate(NULL));
    return 0;
}
"""


def test_c_program_validates_through_the_abi(tmp_path):
    lib = os.path.join(LIB_DIR, "libqknr.so")
    if not os.path.exists(lib):
        pytest.skip("libqknr.so is not built")
    src = tmp_path / "client.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "client"
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src),
                        "-L", LIB_DIR, "-lqknr", f"-Wl,-rpath,{LIB_DIR}", "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("cannot build a C client here: " + r.stderr[-300:])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    res = {}
    for line in out.stdout.splitlines():
        name, code, msg = line.split(" ", 2) if line.count(" ") >= 2 else (line.split(" ") + [""])[:3]
        res[name] = (int(code), msg)
    import qk_rmsnorm_rope_amd as Q
    assert res["version"][0] == Q.version()
    assert res["valid"][0] == 0
    assert res["v1_two_heads"][0] == 1 and "N = 1" in res["v1_two_heads"][1]
    assert res["int8_without_scale"][0] == 1 and "k_scale" in res["int8_without_scale"][1]
    assert res["odd_rope"][0] == 1 and "rope_size" in res["odd_rope"][1]
    assert res["unbuilt_mode"][0] == 2
    assert res["null_args"][0] == 1
