"""The kernel-source hash that keys the committed traffic counters ignores
comments and whitespace and nothing else (host only)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_comments_and_whitespace_are_ignored():
    a = "int f(int x) {\n    return x + 1; // add one\n}\n"
    b = "/* f */ int f(int x)\n{\n  return x + 1;\n}\n"
    assert bench.strip_comments(a) == bench.strip_comments(b)


def test_code_and_literals_are_kept():
    assert bench.strip_comments("return x + 1;") != bench.strip_comments("return x + 2;")
    # comment markers inside literals are code
    s = 'asm("v_mov // not a comment"); char c = \'/\';'
    assert bench.strip_comments(s) == s
    assert bench.strip_comments('a = "x"; // y') == 'a = "x";'


def test_hash_is_stable_and_covers_the_kernels():
    h = bench.source_hash()
    assert len(h) == 16 and h == bench.source_hash()
    names = {os.path.basename(f) for f in bench.GEMM_SRCS}
    assert {"gemm.hip", "wide.hip", "strip.hip", "grouped.hip", "skinny.hip", "operands.h",
            "internal.h"} <= names


def test_kernel_hash_covers_its_own_source_only():
    """The hash keyed to one routed kernel covers its own file and the shared
    routing and operand code, not the other kernels' files."""
    srcs = {os.path.basename(f) for f in bench.kernel_srcs("weight-stream")}
    assert srcs == {"gemm.hip", "operands.h", "internal.h", "skinny.hip"}
    assert {os.path.basename(f) for f in bench.kernel_srcs("wide 64x160")} >= {"wide.hip"}
    assert "wide.hip" not in {os.path.basename(f) for f in bench.kernel_srcs("strip 32x128")}
    for name in ("tiled 64x160", "expert-slot", "grouped 32x128", "strip 32x128"):
        h = bench.source_hash(name)
        assert len(h) == 16 and h == bench.source_hash(name)
    assert bench.source_hash("wide 64x160") != bench.source_hash("strip 32x128")


def test_hash_covers_the_compile_flags(monkeypatch):
    """A change of the code-generation flags changes the hash (so counters
    taken with other flags are not reported as current); include paths,
    which differ between checkouts, are not part of them."""
    from bit_prefill_gemm_amd import build
    h = bench.source_hash()
    assert not any(f.startswith("/") for f in build.KERNEL_FLAGS)
    assert set(build.KERNEL_FLAGS) <= set(build.FLAGS)
    monkeypatch.setattr(build, "KERNEL_FLAGS", build.KERNEL_FLAGS + ["-O2"])
    assert bench.source_hash() != h
