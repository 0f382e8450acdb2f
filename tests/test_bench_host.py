"""CPU checks of bench.py's host logic: its closed-form pair count (used for
the FLOP count) equals the oracle's brute-force mask count, and a multi-GPU
request exits with a message."""
import os
import subprocess
import sys

import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("case", [
    ([300, 377, 890], [300, 377, 890], 4, 70, 9),
    ([300, 377, 890], [300, 377, 890], 4, 5, -3),
    ([100, 250, 0, 0], [80, 300, 0, 0], 0, 0, 0),
    ([0, 64, 64, 99], [0, 64, 64, 99], 4, 2147483647, 2147483647),
    ([300, 377, 890], [500, 577, 600], 2, 0, 0),
    ([300, 377, 890], [500, 577, 600], 3, 0, 0),
    ([900, 1000], [400, 1200], 3, 7, 7),
])
def test_pair_count_matches_oracle(case):
    cu_q, cu_kv, mode, pre, nxt = case
    assert bench.allowed_pairs(cu_q, cu_kv, mode, pre, nxt) == \
        oracle.count_pairs(cu_q, cu_kv, mode, pre, nxt)


@pytest.mark.parametrize("name", ["swa_bf16_b1_n16_s16384_d128_pre2048_next0",
                                  "varlen_bf16_n16_d128_8seq_256to4096"])
def test_pair_count_matches_oracle_on_workloads(name):
    w = workloads.WORKLOADS[name]
    p = workloads.make_problem(name)
    assert bench.allowed_pairs(p.cu_seqlens_q, p.cu_seqlens_kv, w.sparse_mode, w.pre_tokens,
                               w.next_tokens) == \
        oracle.count_pairs(p.cu_seqlens_q, p.cu_seqlens_kv, w.sparse_mode, w.pre_tokens,
                           w.next_tokens)


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
