"""Seeded random problems against the oracle over whole tensors (needs an
MI355X).

Each case draws its own sequence lengths (with empty sequences, ragged tails
and, for the modes that take them, key lengths different from query
lengths), mask mode and band, head counts (grouped key/value heads), head
dimension, input type and, for some, a dropout keep mask, and compares out,
the statistics, dq, dk and dv with the oracle element by element.  The cases
are small enough for the oracle to run each in well under a second.  Inputs
are drawn with standard deviation 0.5, and key lengths are at least half
the query lengths: with short key ranges, grouped heads and 1 / keep_prob
some dK / dV elements otherwise reach 5-10, where half a bf16 step of the
output alone is 1/64-1/32 and the absolute bf16 bound 2e-2 stops measuring
the kernels.
"""
import random

import pytest
import torch

import workloads
from parity_utils import compare_full, note, require_gpu, run_hip, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def draw_case(seed):
    r = random.Random(1000 + seed)
    mode = r.choice([0, 2, 3, 4])
    nseq = r.randint(1, 4)
    lengths_q = [r.choice([0, 1, r.randint(2, 64), r.randint(65, 700)]) for _ in range(nseq)]
    if sum(lengths_q) == 0:
        lengths_q[0] = r.randint(1, 300)
    if mode == 4:
        lengths_kv = list(lengths_q)  # the band is defined for equal lengths
    else:
        # at least half as many keys as queries: a few keys attended by
        # hundreds of rows give dK / dV elements near 10, beyond the range
        # where the absolute bf16 bound is meaningful (see above)
        lengths_kv = [r.choice([q, r.randint(max(1, q // 2), 700)]) if q else 0 for q in lengths_q]
    pre = r.randint(-64, 800)
    nxt = r.randint(-64, 800)
    if pre + nxt < 0:
        pre, nxt = -pre, -nxt
    nkv = r.choice([1, 2])
    g = r.choice([1, 1, 2, 3])
    kw = dict(lengths_q=lengths_q, lengths_kv=lengths_kv, num_heads=nkv * g, num_kv_heads=nkv,
              head_dim=r.choice([64, 128]), dtype=r.choice([torch.bfloat16, torch.float32]),
              sparse_mode=mode, pre_tokens=pre, next_tokens=nxt,
              std=0.5, seed=seed, extra_tokens=r.choice([0, 0, 3]))
    keep_prob = r.choice([1.0, 1.0, 0.9, 0.6])
    return kw, keep_prob


@pytest.mark.parametrize("seed", range(96))
def test_random_case_full_parity(dev, seed):
    kw, keep_prob = draw_case(seed)
    p = workloads.make_custom(name=f"random{seed}", **kw)
    mask = workloads.make_drop_mask(p, keep_prob) if keep_prob < 1.0 else None
    note(f"[parity] random{seed}: {kw['dtype']} D={kw['head_dim']} mode={kw['sparse_mode']} "
         f"pre={kw['pre_tokens']} next={kw['next_tokens']} heads={kw['num_heads']}/"
         f"{kw['num_kv_heads']} q={kw['lengths_q']} kv={kw['lengths_kv']} keep={keep_prob}")
    g = run_hip(p, dev, drop_mask=mask, keep_prob=keep_prob)
    o = run_oracle(p, chunk=None, drop_mask=mask, keep_prob=keep_prob)
    compare_full(p, g, o)
