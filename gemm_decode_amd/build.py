"""Builds libgemm_decode.so in-tree from csrc/ with hipcc for gfx950 only.

Every HIP source is compiled with packed-FP32 instruction selection turned
off and without fast-math, so float code maps to single IEEE operations in
the order written (the Q1_0 . q8_0 path is bit-exact by construction).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgemm_decode.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",  # MFMA results in VGPRs, not AGPRs read back one by one
    "-fno-fast-math", "-ffp-contract=off",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the CPU-only
# check of the entry points' validation (the device code is built as usual;
# each -fsanitize= applies to the host compilation only).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}{res.stderr}")
    return obj


def build(jobs: int = 8, sanitize: bool = False, out: str = LIB) -> str:
    """Compiles csrc/ into `out` (the in-tree library by default). With
    sanitize, the host code is built with ASan and UBSan into a separate
    build folder; load such a library only in a process that preloads the
    clang ASan runtime (see oracle/sanitize_check.py)."""
    build_dir = os.path.join(HERE, "_build_san" if sanitize else "_build")
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    extra = SANITIZE_HOST if sanitize else ()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    tmp = out + ".tmp"
    link_extra = (["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-shared-libsan"] if sanitize else [])
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
