"""Build librz.so (the HIP library behind include/rz.h) in-tree for gfx950.

    python -m invariant_logprob_is_amd.build [--sanitize]

compiles every csrc/*.hip with hipcc and links them into
invariant_logprob_is_amd/librz.so.  Always recompiles.

--sanitize builds librz_san.so instead: the same sources with the host code
instrumented by AddressSanitizer and UndefinedBehaviorSanitizer (the device
code is unchanged).  The CPU test tests/test_sanitized_abi.py runs the C-ABI
tests against it with the sanitizer runtime loaded.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librz.so")
SAN_LIB = os.path.join(PKG, "librz_san.so")
# host-only sanitizer flags: each -fsanitize= goes to the host compilation
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    # only the C ABI of include/rz.h is exported
    "-fvisibility=hidden",
    # keep the compiler from forming packed fp32 math on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # an atomic add by one lane stays one plain atomic: the wave-level
    # rewrite would read its result back at once and stall on it
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is noise
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime that hipcc's clang links against
    (it carries the UndefinedBehaviorSanitizer handlers too)."""
    return _run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"]).strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(BUILD_DIR, "san") if sanitize else BUILD_DIR
    lib = SAN_LIB if sanitize else LIB
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(bdir, s[:-4] + ".o") for s in srcs]

    def compile_one(i):
        return _run([hipcc, *CFLAGS, *extra, "-c", os.path.join(CSRC, srcs[i]), "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        outs = list(ex.map(compile_one, range(len(srcs))))
    tmp = lib + ".tmp"
    outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o",
                      tmp]))
    os.replace(tmp, lib)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv, sanitize="--sanitize" in sys.argv)
