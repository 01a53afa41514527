"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

sa_api.cpp (argument checks, workspace carving, launch planning) is rebuilt with the sanitizers on its host code
only (each -fsanitize= behind -Xarch_host: no GPU code is instrumented), linked with the kernels' ordinary objects
into a second libsa.so under _build/asan/, and tests/test_boundary.py runs against it in a child process that
preloads the sanitizer runtime (SA_LIB_PATH selects the library). Any out-of-bounds access, use after free, signed
overflow, misaligned or null dereference, or invalid shift in the validation and workspace-size paths ends the
child with the sanitizer's report."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from long_context_sparse_sa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "_build", "asan")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build_sanitized():
    kernel_objs = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES
                   if s != "sa_api.cpp"]
    missing = [o for o in kernel_objs if not os.path.exists(o)]
    if missing:
        pytest.skip(f"kernel objects not built yet ({missing[0]}): run python -m long_context_sparse_sa_amd.build")
    os.makedirs(OUT_DIR, exist_ok=True)
    obj = os.path.join(OUT_DIR, "sa_api.o")
    lib = os.path.join(OUT_DIR, "libsa.so")
    cc = [B.hipcc(), *B.FLAGS, "-O1", "-g", "-fno-omit-frame-pointer", *SAN, "-x", "hip",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(B.CSRC, "sa_api.cpp"), "-o", obj]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    ld = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *SAN, obj, *kernel_objs, "-o", lib]
    r = subprocess.run(ld, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


@pytest.mark.slow
def test_boundary_validation_under_asan_and_ubsan():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not found")
    rt = _runtime()
    if rt is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    lib = _build_sanitized()
    # the library is instrumented: its host code calls into the sanitizer runtime
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env["SA_LIB_PATH"] = lib
    # the sanitizer runtime must come first; anything already preloaded stays preloaded after it
    env["LD_PRELOAD"] = rt + (" " + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_boundary.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in report and "runtime error:" not in report, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
