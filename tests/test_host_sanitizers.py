"""The C ABI's host code (planner, argument checks, workspace bookkeeping)
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
only, and run on the CPU by tests/sanitize/host_checks.cpp: the sanitizers
abort on any invalid memory access, integer overflow or other undefined
behaviour in the paths it drives.  Needs hipcc (the device code is compiled
as usual and never launched)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from chunked_kl_loss_seq_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# sanitizer flags for the host compilation only (the GPU code stays as built)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_host_code_under_asan_and_ubsan(tmp_path):
    try:
        cc = BLD.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    flags = [f for f in BLD.FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN
    srcs = [os.path.join(BLD.CSRC, s) for s in BLD.SOURCES] + [os.path.join(ROOT, "tests", "sanitize",
                                                                             "host_checks.cpp")]

    def comp(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        x = ["-x", "hip"] if src.endswith(".cpp") else []
        r = subprocess.run([cc, *flags, *x, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, srcs))
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([cc, f"--offload-arch={BLD.ARCH}", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", CKL_WORKSPACE_BYTES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert shutil.which(exe) or os.path.exists(exe)
