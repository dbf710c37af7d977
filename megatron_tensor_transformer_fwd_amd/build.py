"""Build libtpshard.so in-tree with hipcc for gfx950.

Every HIP source is compiled for gfx950 only; the C ABI (tp_shard.cpp) is
compiled by hipcc too and everything is linked into one shared library next to
this file, with an rpath to the ROCm runtime.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtpshard.so")
ARCH = "gfx950"

SOURCES = ["shard_reduce.hip", "mlp.hip", "swiglu.hip", "attention.hip", "attention_bwd.hip", "attention_bwd_core.hip", "sp.hip", "vocab.hip", "tp_shard.cpp"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
        # keep the compiler from forming packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


# Per-source code-generation options.  The flash-attention backward kernels
# keep their MFMA accumulators in architectural VGPRs (the VALU softmax reads
# them directly); the default accumulation-register form made the compiler
# copy every score and fragment between the two register files.
SOURCE_FLAGS = {"attention_bwd_core.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


# Host-side sanitizer build (a CPU-only check of the C ABI's validation layer
# and the host planners): AddressSanitizer and UndefinedBehaviorSanitizer on
# the host half of every source; the device code is built as usual.  Each
# -fsanitize= is bound to the host pass.
SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()
SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libtpshard_san.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime to preload into an uninstrumented
    Python when loading SAN_LIB."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(cand):
            out = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                                 text=True).stdout.strip()
            if out and os.path.exists(out):
                return out
    raise RuntimeError("clang's AddressSanitizer runtime not found")


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc()] + common_flags() + SOURCE_FLAGS.get(src, []) + (SANITIZE_FLAGS if sanitize else [])
           + ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compile every source and link the library.  Always rebuilds.  With
    sanitize, the host-sanitizer build goes to SAN_LIB instead (the product
    library is untouched)."""
    out_dir, lib = (SAN_BUILD, SAN_LIB) if sanitize else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + [
        "-Wl,-rpath,/opt/rocm/lib", "-L/opt/rocm/lib", "-lamdhip64"]
    if sanitize:
        cmd += "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -shared-libasan".split()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build(sanitize=True)
        print(f"run the CPU ABI tests against it:\n  LD_PRELOAD={asan_runtime()} ASAN_OPTIONS=detect_leaks=0 "
              f"TPSHARD_LIB={SAN_LIB} python -m pytest tests/test_abi_cpu.py tests/test_abi_exports.py")
    else:
        build()
    sys.exit(0)
