"""GPU: a whole speculative verify step through the C ABI -- best-first tree build, masks and
plan, attention, combine, greedy accept, KV compaction -- chained on one stream with no host
sync between the stages, checked against the oracle chain (bench.py's step row does the
checking: every integer stage bit for bit, the attention on sampled rows within the bf16
tolerance; any mismatch raises).  Every case prints its name before it runs."""
import argparse
import os
import sys

import pytest

import workloads

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "kimi (1 x 64 nodes, 64 heads, 4096 cache)": "kimi",
    "ragged trees (3 requests, 64 nodes, 16 heads)":
        workloads.Spec("step_r", 80, 3, 64, 16, 512, 64, "bf16", None, ragged=(0, 1500), depth=8, topk=8),
    "decode shape (4 requests, one node, 64 heads)":
        workloads.Spec("step_d", 81, 4, 1, 64, 512, 64, "bf16", None, ragged=(1, 3000), tree="chain"),
    "wide trees (2 requests, 256 nodes, 2 heads, outliers)":
        workloads.Spec("step_w", 82, 2, 256, 2, 512, 64, "bf16", 700, depth=16, topk=16, outlier_p=0.01),
}


@pytest.mark.parametrize("name", list(CASES))
def test_verify_step_chain_matches_oracle(name):
    print(f"case step: {name}", flush=True)
    line = bench.run_step_row(argparse.Namespace(workload=CASES[name], seed=0, warmup=1, steps=2))
    assert line["attention_max_abs_err_sampled"] <= 2e-3
    assert set(line["stage_us"]) == {"tree_build", "prepare", "attend", "combine", "accept", "compact"}
    print(f"PASS step {name}: accepted {line['accepted_tokens']} tokens, {line['ms_per_step']} ms", flush=True)
