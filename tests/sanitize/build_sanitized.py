"""Sanitizer builds for the CPU test suite (host code only; no GPU code is
built with a sanitizer).

  python tests/sanitize/build_sanitized.py OUT_DIR

writes OUT_DIR/libsaoracle_asan.so (the C oracle under gcc's address and
undefined-behaviour sanitizers) and OUT_DIR/libsparse_attn_asan.so (the C
ABI's host code, api.hip, with the host pass under clang's sanitizers, linked
with launch_stubs.cpp in place of the kernels).  tests/test_sanitizers.py
runs the oracle pins and the ABI tests against them."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "structured_sparse_causal_amd", "csrc")


def build_oracle(out_dir: str) -> str:
    out = os.path.join(out_dir, "libsaoracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                    "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", out, os.path.join(ROOT, "oracle", "sparse_attn_oracle.c"), "-lm"], check=True)
    return out


def build_abi(out_dir: str) -> str:
    out = os.path.join(out_dir, "libsparse_attn_asan.so")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wno-unused-command-line-argument"] + san +
                   [os.path.join(CSRC, "api.hip"), os.path.join(HERE, "launch_stubs.cpp"), "-o", out], check=True)
    return out


def runtimes():
    """Sanitizer runtimes to preload into the (uninstrumented) interpreter."""
    gcc_rt = [subprocess.run(["gcc", "-print-file-name=" + n], capture_output=True, text=True).stdout.strip()
              for n in ("libasan.so", "libubsan.so")]
    clang_rt = None
    for base in ("/opt/rocm/llvm/lib/clang", "/opt/rocm/lib/llvm/lib/clang"):
        if os.path.isdir(base):
            for ver in sorted(os.listdir(base), reverse=True):
                cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
                if os.path.exists(cand):
                    clang_rt = cand
                    break
        if clang_rt:
            break
    return gcc_rt, clang_rt


if __name__ == "__main__":
    d = sys.argv[1] if len(sys.argv) > 1 else "."
    os.makedirs(d, exist_ok=True)
    print(build_oracle(d))
    print(build_abi(d))
