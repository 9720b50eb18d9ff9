"""bench.py's host side (no GPU): the one-GPU contract, the latency
statistics, and that the committed profiles and HBM-counter summary belong to the
committed kernel sources (else the bench line's roofline.traffic is null)."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_latency_stats():
    st = bench.latency_stats([0.010, 0.020, 0.030, 0.040, 0.050])   # ms
    assert st == {"median": 30.0, "p20": 18.0, "p80": 42.0, "min": 10.0, "samples": 5}


def test_committed_counters_match_the_kernel_sources():
    traffic = bench.counters_traffic(bench.HEADLINE, bench.source_digest())
    assert traffic is not None, "profiles/ counter summary was taken from other kernel sources"
    assert 250e6 < traffic < 400e6
    # the summary holds the balanced schedule's kernel, so another path gets none
    assert bench.counters_traffic(bench.HEADLINE, bench.source_digest(), "pair") is None
    assert bench.counters_traffic(bench.HEADLINE, "0" * 16) is None


def test_every_committed_kernel_profile_names_the_current_sources():
    """Each rocprofv3 summary under profiles/ records the kernel-source
    digest it was taken from; all of them must be the current one."""
    import glob
    import re
    digest = bench.source_digest()
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*")))
    assert paths
    for path in paths:
        text = open(path).read()
        found = re.findall(r"\b[0-9a-f]{16}\b", text)
        assert digest in found, f"{os.path.basename(path)} was taken from other kernel sources"


def test_kernel_digest_reads_code_not_comments():
    """A comment-only edit leaves the kernel-source digest unchanged (the
    profiles stay valid); a code edit changes it."""
    src = 'int a = 1; // x\n/* y */ const char* s = "p//q /* r */";\n\n  float f; /* z\n w */ int b;\n'
    assert bench.code_only(src) == 'int a = 1;\n const char* s = "p//q /* r */";\n  float f;  int b;'
    assert bench.code_only(src.replace("// x", "// another note")) == bench.code_only(src)
    assert bench.code_only(src.replace("a = 1", "a = 2")) != bench.code_only(src)

