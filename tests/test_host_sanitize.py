"""The library's host code (descriptor validation, sizing, argument checks)
built with the address and undefined-behaviour sanitizers and driven on the CPU
by tests/host_sanitize_driver.cpp.  The sanitizers apply to the host half of
each source only (-Xarch_host; the device code is built as usual and never
launched here), in a build folder of its own, so the library the other tests
load is untouched."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_pretraining_amd import build as lhbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(lhbuild.BUILD_DIR, "host_sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _host_flags():
    out = list(lhbuild.FLAGS)
    for f in SAN + ["-g"]:
        out += ["-Xarch_host", f]
    return out


@pytest.mark.skipif(not (os.path.exists(lhbuild.HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_host_code_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        cmd = [lhbuild.HIPCC, *_host_flags(), "-c", os.path.join(lhbuild.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-4000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=min(len(lhbuild.SOURCES), 4)) as ex:
        objs = list(ex.map(compile_one, lhbuild.SOURCES))
    exe = os.path.join(OUT, "host_sanitize_driver")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(lhbuild.HIPCC)), "lib")
    cmd = [CLANG, "-std=c++20", "-O1", "-g", *SAN, os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), *objs,
           f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "all checks passed" in r.stdout, out[-4000:]
    shutil.rmtree(OUT, ignore_errors=True)
