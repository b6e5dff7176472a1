"""CPU-only sanitizer run (test infrastructure): the oracle under gcc's
AddressSanitizer + UndefinedBehaviorSanitizer with every CPU test that uses
it, and the HIP library's host code (argument validation of every entry
point) under clang's ASan + UBSan with the ABI tests. Each library runs in
its own process with its own sanitizer runtime preloaded; any report fails
the run.

    python oracle/sanitize_check.py

Builds oracle/liboracle_san.so and a sanitized copy of the library in a
temporary folder (the in-tree libgemm_decode.so is not touched).
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _instrumented(lib: str) -> bool:
    """True if the shared library calls into the ASan and UBSan runtimes."""
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    return "__asan_" in syms and "__ubsan_" in syms


def _run(cmd, env, cwd):
    print("+", " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=cwd).returncode


def main() -> int:
    sys.path.insert(0, ROOT)
    import oracle
    san = oracle.build(sanitize=True)
    if not _instrumented(san):
        print(f"{san} is not instrumented", file=sys.stderr)
        return 2
    base = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONDONTWRITEBYTECODE="1")
    # 1. the oracle: every CPU test that loads it
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    libubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(base, LD_PRELOAD=f"{libasan}:{libubsan}", GD_ORACLE_SANITIZED="1")
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")) +
                   [os.path.join(ROOT, "tests", "test_golden.py"), os.path.join(ROOT, "tests", "test_plane_layout.py")])
    rc = _run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests], env, ROOT)
    if rc != 0:
        return rc
    # 2. the library's host code, in a copy of the package with a sanitized build
    sys.path.insert(0, os.path.join(ROOT, "gemm_decode_amd"))
    import build as gdbuild
    clang_rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not clang_rt:
        print("clang ASan runtime not found", file=sys.stderr)
        return 2
    with tempfile.TemporaryDirectory() as tmp:
        for d in ("gemm_decode_amd", "include", "oracle", "tests", "workloads"):
            shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d),
                            ignore=shutil.ignore_patterns("_build*", "*.so", "__pycache__"))
        shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp)
        lib = gdbuild.build(sanitize=True, out=os.path.join(tmp, "gemm_decode_amd", "libgemm_decode.so"))
        if not _instrumented(lib):
            print(f"{lib} is not instrumented", file=sys.stderr)
            return 2
        env = dict(base, LD_PRELOAD=clang_rt[-1])
        rc = _run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                   os.path.join(tmp, "tests", "test_abi.py")], env, tmp)
    return rc


if __name__ == "__main__":
    sys.exit(main())
