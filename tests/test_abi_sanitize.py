"""The C ABI's host paths under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_sanitize.cpp drives argument validation of every entry point, the
record / page / workspace size arithmetic and the decode split planner over
a grid of shapes, and the page pool against a plain model.  It is linked
with the library's sources rebuilt with the sanitizers on the host code only
(each -fsanitize= behind -Xarch_host; the device code is compiled as usual
and never launched), and must print "ok".  CPU only: nothing here touches a
GPU."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_bit_kitty_amd", "csrc")
LIB_SOURCES = ["kitty_abi.cpp", "decode.hip", "quantize.hip", "ceiling.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return path if os.path.exists(path) else None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_abi_host_paths_under_asan_ubsan(tmp_path):
    cc = _hipcc()
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *SAN,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = [([cc, *flags, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", str(tmp_path / (s + ".o"))])
            for s in LIB_SOURCES]
    jobs.append([cc, *flags, "-c", os.path.join(ROOT, "tests", "abi_sanitize.cpp"), "-o", str(tmp_path / "drv.o")])

    def run(cmd):
        return subprocess.run(cmd, capture_output=True, text=True)

    with ThreadPoolExecutor(len(jobs)) as ex:
        for r in ex.map(run, jobs):
            assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "abi_sanitize")
    objs = [str(tmp_path / (s + ".o")) for s in LIB_SOURCES] + [str(tmp_path / "drv.o")]
    r = run([cc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             *objs, "-o", exe])
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    # leak checking is off: the HIP runtime keeps allocations until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) > 100000  # the grid really ran
