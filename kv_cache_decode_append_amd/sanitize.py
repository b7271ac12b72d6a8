"""Host-code sanitizer run (CPU only, no GPU needed).

    python kv_cache_decode_append_amd/sanitize.py

Builds a copy of libkvc.so whose host code (the prefix-cache block manager,
the step scheduler, the C ABI's argument checks and every entry point's host
path) carries AddressSanitizer and UndefinedBehaviorSanitizer, then runs the
CPU tests that drive that host code against it: the prefix-cache manager
against its oracle over random operations, the scheduler's plans and batch
descriptors, the queue replay and the C ABI's rejection of bad arguments.
Device code is built as usual: each sanitizer flag is passed to the host
compilation only. The copy lives in a temporary directory; the in-tree
library is not touched. Exits with the test run's status; any sanitizer
report aborts the run.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
TESTS = ["tests/test_abi.py", "tests/test_prefix_cache.py", "tests/test_sched.py",
         "tests/test_replay.py"]


def asan_runtime() -> str:
    """clang's shared ASan runtime (it carries the UBSan handlers as well)."""
    clang = os.path.realpath(os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..",
                                          "lib", "llvm", "bin", "clang"))
    res = subprocess.run([clang, "-print-resource-dir"], capture_output=True, text=True)
    cands = glob.glob(os.path.join(res.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not cands:
        cands = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not cands:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found")
    return cands[0]


def build(dst_pkg: str) -> None:
    csrc = os.path.join(PKG, "csrc")
    objs = []
    for src in sorted(os.listdir(csrc)):
        if not src.endswith((".hip", ".cpp")):
            continue
        obj = os.path.join(dst_pkg, src + ".o")
        cmd = [HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", f"-I{os.path.join(ROOT, 'include')}",
               f"-I{csrc}", *HOST_SAN, "-c", os.path.join(csrc, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed for {src}:\n{res.stderr[-4000:]}")
        objs.append(obj)
    out = os.path.join(dst_pkg, "libkvc.so")
    res = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr[-4000:]}")
    for o in objs:
        os.remove(o)
    syms = subprocess.run(["nm", "-D", "--undefined-only", out], capture_output=True, text=True).stdout
    if "__asan_report" not in syms or "__ubsan_handle" not in syms:
        raise RuntimeError("the library carries no ASan / UBSan instrumentation")


def main() -> int:
    runtime = asan_runtime()
    with tempfile.TemporaryDirectory(prefix="kvc_sanitize_") as tmp:
        for name in ("kv_cache_decode_append_amd", "include", "oracle", "workloads", "tests"):
            shutil.copytree(os.path.join(ROOT, name), os.path.join(tmp, name),
                            ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.o"))
        shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp)
        print("building the sanitized library ...", flush=True)
        build(os.path.join(tmp, "kv_cache_decode_append_amd"))
        env = dict(os.environ)
        env["LD_PRELOAD"] = runtime
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
        env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
        cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *TESTS]
        print("running:", " ".join(cmd), f"(LD_PRELOAD={runtime})", flush=True)
        return subprocess.run(cmd, cwd=tmp, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
