"""The C ABI's validation layer and host planners under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; CPU only).  Builds the sanitizer
library when it is missing or older than the sources, then runs the CPU ABI
tests against it in a child process with the ASan runtime preloaded; any
sanitizer report aborts the child (UBSan does not recover)."""
import glob
import os
import subprocess
import sys

import pytest

import megatron_tensor_transformer_fwd_amd.build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale() -> bool:
    if not os.path.exists(B.SAN_LIB):
        return True
    built = os.path.getmtime(B.SAN_LIB)
    srcs = glob.glob(os.path.join(B.CSRC, "*")) + [os.path.join(ROOT, "include", "tp_shard.h")]
    return any(os.path.getmtime(p) > built for p in srcs)


def test_abi_validation_under_host_sanitizers():
    try:
        rt = B.asan_runtime()
        if _stale():
            B.build(verbose=False, sanitize=True)
    except RuntimeError as e:   # no ROCm toolchain here
        pytest.skip(str(e))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0", TPSHARD_LIB=B.SAN_LIB)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        "tests/test_abi_cpu.py", "tests/test_abi_exports.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
