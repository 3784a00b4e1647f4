"""The committed profile summaries match the code they describe: every HBM
counter row of profiles/pmc_traffic.json carries the hash of its kernel source's
current code (bench.py reports a row only while that holds, so a kernel changed
without new counters would leave the bench line's traffic empty), the rows the
bench line reads exist for every workload it runs, and every summary gives a
command that runs committed files only."""
import glob
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def traffic():
    with open(bench.PMC_SUMMARY) as f:
        return json.load(f)


def test_counter_rows_match_current_sources():
    stale = [k for k, e in traffic()["kernels"].items()
             if bench.source_code_hash(os.path.join(bench.CSRC, e["source"]))
             != e["source_code_sha256"]]
    assert not stale, f"counter rows taken on older kernel code: {stale}"


def test_bench_lines_have_their_traffic_rows():
    rows = traffic()["kernels"]
    prefill = ["prefill_32k", "chunked_prefill", "prefill_32k_sel1", "prefill_32k_tokens"]
    staged = ["prefill_32k_fp8", "prefill_32k_fp8_sel1"]
    decode = ["decode_1m_b8", "decode_128k_b64", "decode_1m_b8_fp8", "decode_1m_b8_t4",
              "decode_ragged_b64", "decode_1m_b8_sel1"]
    for w in prefill:
        assert bench.attn_prefill_traffic(w, False) is not None, w
    for w in staged:
        assert bench.attn_prefill_traffic(w, True) is not None, w
    for w in decode:
        assert f"{w}:index_decode" in rows, w
        assert bench.measured_traffic(f"{w}:index_decode", "index_scores.hip") is not None, w
    assert bench.measured_traffic("prefill_32k:insert", "qk_insert.hip") is not None


def test_summaries_name_committed_commands():
    files = glob.glob(os.path.join(PROFILES, "*.md"))
    assert len(files) >= 14
    for f in files:
        text = open(f).read()
        assert "rocprofv3" in text and "bench.py" in text, f
        assert "_work" not in text, f
