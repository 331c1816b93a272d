"""The host-side argument checks of libropekv, built with AddressSanitizer and
UndefinedBehaviorSanitizer on host code (device code unchanged) and driven by
tests/abi_errors_driver.c: every entry point's error paths and the workspace
sizing run with memory and undefined-behaviour errors fatal.  CPU only: the
driver launches nothing."""
import os
import shutil
import subprocess
import concurrent.futures as cf

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sliding_window_kv_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def test_argument_checks_under_sanitizers(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I",
             CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-w", *SAN]
    srcs = ["table.hip", "append.hip", "decode.hip", "decode_8bit.hip", "prefill.hip", "rerotate.hip", "api.cpp"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, *flags] + (["-x", "hip"] if src.endswith(".cpp") else []) + ["-c", os.path.join(CSRC, src),
                                                                                   "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(7, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv_o = str(tmp_path / "driver.o")
    r = subprocess.run([HIPCC, *SAN, "-g", "-I", os.path.join(ROOT, "include"), "-x", "c", "-c",
                        os.path.join(ROOT, "tests", "abi_errors_driver.c"), "-o", drv_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, drv_o, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "all argument checks ok" in r.stdout
