"""The committed rocprofv3 summaries describe the kernels in this tree.

Every summary under profiles/ records the hash of the kernel sources it was
taken with (bench.kernel_source_hash: code only, comments left out) and the
command that produced it.  A kernel change without new profiles fails here,
instead of leaving bench.py to report stale traffic as null without notice.
"""
import os
import re

import pytest

import bench
import synth

PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
GEMM_SHA = bench.kernel_source_hash()
ATTN_SHA = bench.kernel_source_hash(bench.ATTN_SOURCES)


def _summaries():
    return sorted(f for f in os.listdir(PROFILES) if f.endswith((".md", ".txt")))


def test_traffic_lines_cover_every_bench_line_with_current_sources():
    lines = [l for l in open(os.path.join(PROFILES, "hbm_traffic.txt")) if l.startswith("workload=")]
    seen = {}
    for line in lines:
        kv = dict(tok.split("=", 1) for tok in line.split() if "=" in tok and not tok.startswith('kernel="'))
        seen[kv["workload"]] = kv["kernel_sha"]
    wanted = [bench.HEADLINE] + list(bench.SECONDARY) + list(synth.ATTN_WORKLOADS)
    assert set(wanted) <= set(seen), set(wanted) - set(seen)
    for wl in wanted:
        want = ATTN_SHA if wl in synth.ATTN_WORKLOADS else GEMM_SHA
        assert seen[wl] == want, f"{wl}: traffic taken with kernel sources {seen[wl]}, tree has {want}"
        assert bench.load_traffic(wl) is not None


@pytest.mark.parametrize("name", _summaries())
def test_summary_names_current_sources_and_command(name):
    text = open(os.path.join(PROFILES, name)).read()
    shas = re.findall(r"kernel_sha[^:=\n]*[:=]\s*([0-9a-f]{16})", text)
    assert shas, f"{name} records no kernel_sha"
    assert set(shas) <= {GEMM_SHA, ATTN_SHA}, f"{name} was taken with other kernel sources: {set(shas)}"
    assert "rocprofv3" in text and "bench.py" in text, f"{name} does not give the command that made it"
    assert "_work" not in text, f"{name} names a working file"
