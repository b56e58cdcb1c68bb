"""Runner of the sanitizer pass (started by tests/test_sanitizers.py in a
process with the ASan and UBSan runtimes preloaded).

argv[1]: a host-only build of the ABI layer (api.cpp + plan.cpp +
stub_launch.cpp) with -fsanitize=address,undefined. The binding's library
handle is swapped for it, every qknr_* function keeping the binding's
argument types, so that the host-side tests below validate and plan through
the instrumented code; QKNR_ORACLE_LIB (set by the caller) points the oracle
at its instrumented build. Then every seeded random KV and QK case goes
through the full entry point (validation, planning, the stub launcher's plan
checks), which must end in the stub's "no device" status.

Exit status: pytest's, or 1 if an entry point returned anything else.
"""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)


def swap_library(path):
    import qk_rmsnorm_rope_amd as Q
    san = ctypes.CDLL(path)
    for name, fn in list(Q._lib.__dict__.items()):
        if name.startswith("qknr_"):
            new = getattr(san, name)
            new.argtypes, new.restype = fn.argtypes, fn.restype
    Q._lib = san
    return Q


def full_calls(Q):
    """Each random case through its entry point: check, plan, stub launch."""
    import workloads as W
    from tests import test_gpu_kv_random as KR
    bad = 0
    for i in range(KR.N_CASES):
        base, over, lay = KR._draw(i)
        d = KR._relayout(W.make_kv_cache(base, device="cpu", **over), lay)
        rc = Q._lib.qknr_kv_rmsnorm_rope_cache(ctypes.byref(KR._args(Q, d)), None)
        if rc != Q.DEVICE_ERROR:
            print(f"kv random case {i}: status {rc} ({Q.last_error()})")
            bad += 1
    from tests import test_gpu_qk_random as QR
    for i in range(QR.N_CASES):
        rc = QR.host_call_status(Q, i)
        if rc != Q.DEVICE_ERROR:
            print(f"qk random case {i}: status {rc} ({Q.last_error()})")
            bad += 1
    return bad


def main():
    Q = swap_library(sys.argv[1])
    import pytest
    rc = pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      os.path.join(ROOT, "tests", "test_abi_host.py"),
                      os.path.join(ROOT, "tests", "test_gpu_kv_random.py"),
                      os.path.join(ROOT, "tests", "test_gpu_qk_random.py"),
                      os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                      os.path.join(ROOT, "tests", "test_gpu_encoders_exact.py"),
                      "--deselect", os.path.join(ROOT, "tests", "test_abi_host.py") +
                      "::test_library_exports_every_declared_function"])
    if rc != 0:
        sys.exit(int(rc))
    bad = full_calls(Q)
    print(f"full entry-point calls: {bad} unexpected statuses")
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main()
