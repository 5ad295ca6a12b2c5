"""The committed rocprofv3 summaries that bench.py reads its HBM traffic from.

Each matrix-core kernel's profile ends with two machine-readable lines: the first 16 hex
digits of the SHA-256 of the kernel source the counters were taken on, and the calibrated
HBM bytes per launch.  bench.py reports `traffic` only while that hash matches the source;
these tests keep the committed profiles and kernels in step (re-collect the counters after
a kernel change) and check that each summary names the command that made it.
"""
import hashlib
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SRC = os.path.join(ROOT, "context_attention_lse_kv_amd", "csrc", "attn_bf16.hip")
PROFILES = ["bwd_kv_bf16_video_dit_shard.md", "fwd_bf16_video_dit_shard.md", "bwd_dqs_bf16_video_dit_shard.md"]


def _fields(name):
    vals = {}
    with open(os.path.join(ROOT, "profiles", name)) as f:
        text = f.read()
    for line in text.splitlines():
        if line.startswith(("kernel_source_sha256_16:", "traffic_bytes_per_launch:")):
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    return text, vals


@pytest.mark.parametrize("name", PROFILES)
def test_profile_matches_kernel_source(name):
    with open(KERNEL_SRC, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    text, vals = _fields(name)
    assert vals.get("kernel_source_sha256_16") == sha, (
        f"{name} was taken on another version of attn_bf16.hip: collect its counters again")
    assert int(vals["traffic_bytes_per_launch"]) > 0
    assert "rocprofv3 --kernel-trace --stats" in text and "rocprofv3 --pmc FETCH_SIZE" in text
    assert "rocprofv3 --pmc WRITE_SIZE" in text


def test_bench_reads_the_profiles():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for name in PROFILES:
        _, vals = _fields(name)
        assert bench.measured_traffic(name) == int(vals["traffic_bytes_per_launch"])
    assert bench.measured_traffic("no_such_profile.md") is None
