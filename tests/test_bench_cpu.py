"""bench.py's host logic (CPU only): the kernel code hash that ties the
committed counter summaries to a kernel build, and the refusal of more
than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_hash_ignores_comments_only():
    src = {"a.hip": "int f(int x) {  // doubles\n  return 2 * x; /* done */\n}\n",
           "b.h": "#pragma once\n"}
    h0 = bench.source_hash(("a.hip", "b.h"), read=src.get)
    src2 = dict(src)
    src2["a.hip"] = "// header comment\n\nint f(int x) {\n  return 2 * x;   \n}\n/* a\nblock */\n"
    assert bench.source_hash(("a.hip", "b.h"), read=src2.get) == h0
    src3 = dict(src)
    src3["a.hip"] = src["a.hip"].replace("2 * x", "3 * x")
    assert bench.source_hash(("a.hip", "b.h"), read=src3.get) != h0


def test_code_hash_covers_compile_flags():
    src = {"a.hip": "int f(int x) { return 2 * x; }\n", "b.h": "#pragma once\n"}
    h0 = bench.source_hash(("a.hip", "b.h"), read=src.get, flags={"a.hip": ["-O3"]})
    assert bench.source_hash(("a.hip", "b.h"), read=src.get, flags={"a.hip": ["-O3"]}) == h0
    assert bench.source_hash(("a.hip", "b.h"), read=src.get, flags={"a.hip": ["-O3", "-mllvm", "-x"]}) != h0
    # the real hash takes the build's per-file flags of decode.hip
    from mixed_precision_bit_kitty_amd import build as kbuild
    other = dict(kbuild.SOURCES)
    other["decode.hip"] = other["decode.hip"] + ["-DSOMETHING_ELSE"]
    assert bench.source_hash(bench.DECODE_SOURCES, flags=other) != bench.source_hash(bench.DECODE_SOURCES)


def test_committed_traffic_needs_the_same_kernel_code():
    assert bench.committed_traffic("0" * 16, "llama3_8b", "step") is None
    assert bench.committed_traffic(bench.source_hash(bench.DECODE_SOURCES), "no_such_workload", "step") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_code_hash_covers_every_local_include():
    # a kernel's hash must change when any source it is compiled from changes:
    # the .hip file and every header it includes from csrc/, transitively
    import re
    csrc = os.path.join(os.path.dirname(bench.__file__), "mixed_precision_bit_kitty_amd", "csrc")

    def local_includes(name, seen):
        for inc in re.findall(r'#include\s+"([^"]+)"', open(os.path.join(csrc, name)).read()):
            base = os.path.basename(inc)
            if os.path.exists(os.path.join(csrc, base)) and base not in seen:
                seen.add(base)
                local_includes(base, seen)
        return seen

    for sources in (bench.DECODE_SOURCES, bench.QUANTIZE_SOURCES):
        need = local_includes(sources[0], {sources[0]})
        assert need <= set(sources), (sources, need - set(sources))
