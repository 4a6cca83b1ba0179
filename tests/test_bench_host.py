"""bench.py's host-side logic, without a GPU: the one-GPU contract, the
algorithmic byte and FLOP counts the roofline divides by, the source-hash gate
on stored counter traffic, and the input fingerprint."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle.multi_query as MQ  # noqa: E402
from decode_attention_paged_attn_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]


def test_kv_bytes_counts_valid_tokens_only():
    # 4096 bytes per token at 8 KV heads, fp16 (K and V, 128 dims)
    assert bench.kv_bytes([10, 20, 0], 8) == 30 * 4096
    assert bench.kv_bytes([10, 20, 0], 8, elem=1) == 30 * 2048
    case = W.tiny()
    assert bench.kv_bytes(case.lens, case.Hkv) == (37 + 512) * 2 * 2 * 128 * 2


@pytest.mark.parametrize("causal", [True, False])
def test_multi_query_work_matches_the_visible_tokens(causal):
    lens, nq = [40, 5, 0, 100], [3, 7, 0, 100]
    case = W.build_mq_case(lens, nq, 8, 2, causal=causal, seed=1)
    nbytes, flops = bench.mq_work(case)
    vis = [[MQ.visible_tokens(n, q, i, causal) for i in range(q)] for n, q in zip(lens, nq)]
    want_bytes = sum(max(v) for v in vis if v) * 2 * 2 * 128 * 2
    want_flops = 4 * 128 * 8 * sum(sum(v) for v in vis)
    assert (nbytes, flops) == (want_bytes, want_flops)


def test_stored_traffic_needs_the_current_kernel_sources(monkeypatch):
    recs = json.load(open(bench.TRAFFIC_FILE))
    key, rec = next((k, r) for k, r in recs.items() if "/" in k)
    if rec["source_sha256_16"] == bench.source_hash("attention"):
        assert bench.measured_traffic(key) == rec["bytes_per_call"]
    monkeypatch.setattr(bench, "source_hash", lambda op="attention": "0" * 16)
    assert bench.measured_traffic(key) is None
    assert bench.measured_traffic("no such workload") is None


def test_input_fingerprint_follows_the_seed():
    a = bench.input_fingerprint(W.tiny(seed=0))
    assert a == bench.input_fingerprint(W.tiny(seed=0))
    b = bench.input_fingerprint(W.tiny(seed=1))
    assert a["q_sha256_16"] != b["q_sha256_16"] and a["k_pool_word_sum"] != b["k_pool_word_sum"]
    f8 = bench.input_fingerprint(W.tiny(seed=0, kv_dtype="fp8"))
    assert f8["q_sha256_16"] == a["q_sha256_16"] and f8["k_pool_word_sum"] != a["k_pool_word_sum"]
