"""bench.py's command line on the CPU: a request for more than one GPU is
refused with a message and a nonzero status (the library has one-GPU kernels
only), before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_bench_source_digest_ignores_comments(tmp_path):
    """The traffic measured on a kernel stays valid across comment edits: the
    digest covers the code only."""
    sys.path.insert(0, ROOT)
    import bench
    csrc = os.path.join(ROOT, "paged_kv_cache_amd", "csrc")
    d0 = bench.source_digest("device.h", "prefill.hip")
    assert len(d0) == 16 and d0 == bench.source_digest("device.h", "prefill.hip")
    assert d0 != bench.source_digest("device.h", "decode.hip")
    # the same function on edited copies: a comment change keeps it, a code change does not
    text = open(os.path.join(csrc, "scatter.hip")).read()
    orig_root = bench.ROOT
    try:
        fake = tmp_path / "paged_kv_cache_amd" / "csrc"
        fake.mkdir(parents=True)
        (fake / "k.hip").write_text(text)
        bench.ROOT = str(tmp_path)
        a = bench.source_digest("k.hip")
        (fake / "k.hip").write_text("// a new comment\n" + text.replace("{", "{ /* note */", 1))
        b = bench.source_digest("k.hip")
        (fake / "k.hip").write_text(text.replace("{", "{ int unused_x = 0; (void)unused_x;", 1))
        c = bench.source_digest("k.hip")
    finally:
        bench.ROOT = orig_root
    assert a == b and a != c
