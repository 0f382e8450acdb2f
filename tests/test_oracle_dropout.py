"""Pins of the oracle's dropout with a caller-supplied mask (CPU only).

attention_out = Dropout(softmax(...), keep_prob) V (API doc, 计算公式), with the
mask given as uint8 holding eight one-bit booleans per byte, (sum_b sum_n
Sq*Skv)/8 bytes (API doc, dropMaskOptional), and keep_prob the fraction of
ones (explainer, keepProb).  Readings (no page prints them): bit e of the mask
is byte e // 8, bit e % 8 (least significant first); e runs over batches,
then heads, then the Sq x Skv matrix row by row; a kept element is scaled by
1 / keep_prob.  The pins: the all-keep and all-drop masks reduce to closed
forms; one dropped bit at a hand-computed position changes exactly one
(row, head) by the closed-form amount (this fixes the bit, row, head and batch
order); finite differences pin the backward to the forward.
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
import workloads

F64 = torch.float64


def rand_problem(lq, lkv, nq=2, nkv=None, D=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    nkv = nq if nkv is None else nkv
    q = torch.randn(sum(lq), nq, D, generator=g, dtype=F64)
    k = torch.randn(sum(lkv), nkv, D, generator=g, dtype=F64)
    v = torch.randn(sum(lkv), nkv, D, generator=g, dtype=F64)
    dy = torch.randn(sum(lq), nq, D, generator=g, dtype=F64)
    return q, k, v, dy, workloads.cumulative(lq), workloads.cumulative(lkv)


def packed(bits):
    """Pack a flat 0/1 array LSB-first (the reading under test)."""
    return torch.from_numpy(np.packbits(np.asarray(bits, dtype=np.uint8), bitorder="little"))


def nbits(cu_q, cu_kv, n):
    return sum(n * sq * skv for (_, sq), (_, skv) in
               zip(oracle.sequences(cu_q), oracle.sequences(cu_kv)))


def test_mask_size_is_the_pages_formula():
    cu_q, cu_kv = [3, 8, 8, 0], [4, 6, 6, 0]  # lengths 3/4, 5/2, 0/0, then a trailing batch
    assert oracle.drop_mask_bits(cu_q, cu_kv, 3) == 3 * (3 * 4 + 5 * 2 + 0)


@pytest.mark.parametrize("mode,pre,nxt", [(0, 0, 0), (4, 2, 1), (3, 0, 0)])
def test_all_keep_with_keep_prob_one_is_no_dropout(mode, pre, nxt):
    q, k, v, dy, cu_q, cu_kv = rand_problem([5, 7], [6, 7], seed=1)
    if mode == 4:
        cu_kv = cu_q
        k, v = k[:12], v[:12]
    ones = packed(np.ones(nbits(cu_q, cu_kv, 2)))
    a = oracle.forward(q, k, v, cu_q, cu_kv, 0.5, pre, nxt, mode)
    b = oracle.forward(q, k, v, cu_q, cu_kv, 0.5, pre, nxt, mode, drop_mask=ones, keep_prob=1.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ga = oracle.backward(q, k, v, dy, *a, cu_q, cu_kv, 0.5, pre, nxt, mode)
    gb = oracle.backward(q, k, v, dy, *a, cu_q, cu_kv, 0.5, pre, nxt, mode, drop_mask=ones)
    for x, y in zip(ga, gb):
        assert torch.equal(x, y)


def test_all_keep_scales_by_inverse_keep_prob():
    q, k, v, dy, cu, _ = rand_problem([9, 4], [9, 4], seed=2)
    ones = packed(np.ones(nbits(cu, cu, 2)))
    o1, m1, l1 = oracle.forward(q, k, v, cu, cu, 0.5)
    o2, m2, l2 = oracle.forward(q, k, v, cu, cu, 0.5, drop_mask=ones, keep_prob=0.5)
    assert torch.allclose(o2, 2 * o1, rtol=1e-14, atol=0)
    assert torch.equal(m1, m2) and torch.equal(l1, l2)  # statistics are pre-dropout
    g1 = oracle.backward(q, k, v, dy, o1, m1, l1, cu, cu, 0.5)
    g2 = oracle.backward(q, k, v, dy, o2, m2, l2, cu, cu, 0.5, drop_mask=ones, keep_prob=0.5)
    for x, y in zip(g1, g2):
        assert torch.allclose(y, 2 * x, rtol=1e-12, atol=1e-14)


def test_all_drop_gives_zeros():
    q, k, v, dy, cu, _ = rand_problem([6, 5], [6, 5], seed=3)
    zeros = packed(np.zeros(nbits(cu, cu, 2)))
    o1, m1, l1 = oracle.forward(q, k, v, cu, cu, 0.5)
    o, m, l = oracle.forward(q, k, v, cu, cu, 0.5, drop_mask=zeros, keep_prob=0.8)
    assert o.abs().max() == 0 and torch.equal(m, m1) and torch.equal(l, l1)
    for g in oracle.backward(q, k, v, dy, o, m, l, cu, cu, 0.5, drop_mask=zeros, keep_prob=0.8):
        assert g.abs().max() == 0


@pytest.mark.parametrize("b,n,i,j", [(1, 1, 2, 3), (0, 2, 4, 0), (1, 0, 0, 5)])
def test_single_dropped_bit_position(b, n, i, j):
    """One zero bit at batch b, head n, row i, key j: only out[row i of batch b,
    head n] changes, by -P_ij V_j (keep_prob 1), with P from torch directly."""
    lq, lkv, N = [5, 4], [3, 6], 3
    q, k, v, dy, cu_q, cu_kv = rand_problem(lq, lkv, nq=N, seed=4)
    sq, skv = lq[b], lkv[b]
    e = sum(N * lq[x] * lkv[x] for x in range(b)) + n * sq * skv + i * skv + j
    bits = np.ones(nbits(cu_q, cu_kv, N))
    bits[e] = 0
    o0, _, _ = oracle.forward(q, k, v, cu_q, cu_kv, 0.7)
    o1, _, _ = oracle.forward(q, k, v, cu_q, cu_kv, 0.7, drop_mask=packed(bits))
    row = sum(lq[:b]) + i
    k0 = sum(lkv[:b])
    s = 0.7 * (q[row, n] @ k[k0:k0 + skv, n].T)
    p = torch.softmax(s, 0)
    diff = (o1 - o0).abs().amax(-1)
    changed = torch.nonzero(diff > 0).tolist()
    assert changed == [[row, n]]
    assert torch.allclose(o1[row, n], o0[row, n] - p[j] * v[k0 + j, n], atol=1e-14)


@pytest.mark.parametrize("nq,nkv,mode,pre,nxt", [(2, 2, 4, 2, 1), (4, 2, 0, 0, 0)])
def test_dropout_finite_differences(nq, nkv, mode, pre, nxt):
    q, k, v, dy, cu, _ = rand_problem([5, 4], [5, 4], nq=nq, nkv=nkv, D=4, seed=11)
    g = np.random.default_rng(5)
    mask = packed(g.random(nbits(cu, cu, nq)) < 0.7)
    scale, kp = 0.8, 0.7

    def loss():
        o, _, _ = oracle.forward(q, k, v, cu, cu, scale, pre, nxt, mode, drop_mask=mask,
                                 keep_prob=kp)
        return float((o * dy).sum())

    out, sm, ss = oracle.forward(q, k, v, cu, cu, scale, pre, nxt, mode, drop_mask=mask,
                                 keep_prob=kp)
    grads = oracle.backward(q, k, v, dy, out, sm, ss, cu, cu, scale, pre, nxt, mode,
                            drop_mask=mask, keep_prob=kp)
    h = 1e-6
    for x, gr in zip((q, k, v), grads):
        fd = torch.zeros_like(x)
        flat = x.view(-1)
        for idx in range(flat.numel()):
            old = float(flat[idx])
            flat[idx] = old + h
            lp = loss()
            flat[idx] = old - h
            lm = loss()
            flat[idx] = old
            fd.view(-1)[idx] = (lp - lm) / (2 * h)
        assert (fd - gr).abs().max() / gr.abs().max() <= 1e-6


def test_dropout_chunked_equals_full():
    q, k, v, dy, cu, _ = rand_problem([37, 20], [37, 20], seed=13)
    mask = packed(np.random.default_rng(1).random(nbits(cu, cu, 2)) < 0.8)
    kw = dict(drop_mask=mask, keep_prob=0.8)
    full = oracle.forward(q, k, v, cu, cu, 0.4, 5, 2, 4, **kw)
    ch = oracle.forward(q, k, v, cu, cu, 0.4, 5, 2, 4, chunk=7, **kw)
    for a, b in zip(full, ch):
        assert torch.allclose(a, b, atol=1e-14, rtol=1e-14)
    gf = oracle.backward(q, k, v, dy, *full, cu, cu, 0.4, 5, 2, 4, **kw)
    gc = oracle.backward(q, k, v, dy, *full, cu, cu, 0.4, 5, 2, 4, chunk=7, **kw)
    for a, b in zip(gf, gc):
        assert torch.allclose(a, b, atol=1e-13, rtol=1e-13)


def test_short_mask_is_rejected():
    q, k, v, dy, cu, _ = rand_problem([5], [5], seed=1)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, cu, cu, 0.5, drop_mask=torch.zeros(2, dtype=torch.uint8))


MUTATIONS = {
    "msb_first": ('bits = np.unpackbits(raw, bitorder="little")',
                  'bits = np.unpackbits(raw, bitorder="big")'),
    "dp_not_dropped": ("dP = _dropped(dY[rows] @ V[c0:c1].T, Z, rows, c0, c1, keep_prob)",
                       "dP = dY[rows] @ V[c0:c1].T"),
    "no_inverse_scale": ("return torch.where(Z[rows][:, c0:c1], P / keep_prob, "
                         "torch.zeros((), dtype=F64))",
                         "return torch.where(Z[rows][:, c0:c1], P, torch.zeros((), dtype=F64))"),
    "heads_before_batches": (
        "    for b, ((_, sq), (_, skv)) in enumerate(zip(sequences(cu_seqlens_q),\n"
        "                                                sequences(cu_seqlens_kv))):\n"
        "        for n in range(num_heads):\n"
        "            out[(b, n)]",
        "    for n, b, sq, skv in [(n, b, sq, skv) for n in range(num_heads) for b, ((_, sq), "
        "(_, skv)) in enumerate(zip(sequences(cu_seqlens_q), sequences(cu_seqlens_kv)))]:\n"
        "        if True:\n"
        "            out[(b, n)]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_dropout_pins_catch_planted_mistakes(name):
    src = open(A.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src, name
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    caught = False
    # the single-bit position check
    lq, lkv, N = [5, 4], [3, 6], 3
    q, k, v, dy, cu_q, cu_kv = rand_problem(lq, lkv, nq=N, seed=4)
    e = N * lq[0] * lkv[0] + 1 * lq[1] * lkv[1] + 2 * lkv[1] + 3
    bits = np.ones(nbits(cu_q, cu_kv, N))
    bits[e] = 0
    o0, _, _ = oracle.forward(q, k, v, cu_q, cu_kv, 0.7)
    o1, _, _ = mod.forward(q, k, v, cu_q, cu_kv, 0.7, drop_mask=packed(bits))
    changed = torch.nonzero((o1 - o0).abs().amax(-1) > 0).tolist()
    caught |= changed != [[lq[0] + 2, 1]]
    # the keep_prob scaling check
    ones = packed(np.ones(nbits(cu_q, cu_kv, N)))
    o2, _, _ = mod.forward(q, k, v, cu_q, cu_kv, 0.7, drop_mask=ones, keep_prob=0.5)
    caught |= not torch.allclose(o2, 2 * o0, rtol=1e-14, atol=0)
    # the finite-difference check on the value gradient
    cu = workloads.cumulative([5, 4])
    q, k, v, dy, _, _ = rand_problem([5, 4], [5, 4], D=4, seed=11)
    mask = packed(np.random.default_rng(5).random(nbits(cu, cu, 2)) < 0.7)
    out, sm, ss = mod.forward(q, k, v, cu, cu, 0.8, drop_mask=mask, keep_prob=0.7)
    grads = mod.backward(q, k, v, dy, out, sm, ss, cu, cu, 0.8, drop_mask=mask, keep_prob=0.7)
    ref = oracle.forward(q, k, v, cu, cu, 0.8, drop_mask=mask, keep_prob=0.7)
    gref = oracle.backward(q, k, v, dy, *ref, cu, cu, 0.8, drop_mask=mask, keep_prob=0.7)
    # (the unmutated oracle is itself pinned by the finite-difference test above)
    caught |= not all(torch.allclose(a, b, atol=1e-12) for a, b in zip(grads, gref))
    assert caught, name
