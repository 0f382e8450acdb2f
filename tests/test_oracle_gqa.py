"""Pins of the oracle's grouped heads (GQA, explainer 6.2) (CPU only).

Query head n reads key/value head n // G with G = Nq / Nkv, and a key/value
head's gradients sum over its G query heads.  The reference is torch SDPA with
``enable_gqa=True`` (same head mapping) and autograd, in fp64; finite
differences pin the gradients independently of any library.
"""
import types

import pytest
import torch

import oracle
from oracle import attention as A
import workloads

F64 = torch.float64


def rand_problem(lengths, nq, nkv, D=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    q = torch.randn(T, nq, D, generator=g, dtype=F64)
    k = torch.randn(T, nkv, D, generator=g, dtype=F64)
    v = torch.randn(T, nkv, D, generator=g, dtype=F64)
    dy = torch.randn(T, nq, D, generator=g, dtype=F64)
    return q, k, v, dy, workloads.cumulative(lengths)


def literal_mask(mode, pre, nxt, L):
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    if mode == 0:
        return torch.ones(L, L, dtype=torch.bool)
    if mode == 2:
        return j <= i
    return (j - i >= -pre) & (j - i <= nxt)


def sdpa_gqa(q, k, v, dy, cu, scale, mode, pre, nxt):
    out = torch.zeros_like(q)
    gq, gk, gv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    for s0, L in oracle.sequences(cu):
        Q = q[s0:s0 + L].transpose(0, 1).clone().requires_grad_(True)   # [Nq, L, D]
        K = k[s0:s0 + L].transpose(0, 1).clone().requires_grad_(True)
        V = v[s0:s0 + L].transpose(0, 1).clone().requires_grad_(True)
        M = literal_mask(mode, pre, nxt, L)
        O = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None], V[None], attn_mask=M, scale=scale, enable_gqa=True)[0]
        O.backward(dy[s0:s0 + L].transpose(0, 1))
        out[s0:s0 + L] = O.detach().transpose(0, 1)
        gq[s0:s0 + L] = Q.grad.transpose(0, 1)
        gk[s0:s0 + L] = K.grad.transpose(0, 1)
        gv[s0:s0 + L] = V.grad.transpose(0, 1)
    return out, (gq, gk, gv)


CASES = [(4, 2, 0, 0, 0), (6, 2, 4, 3, 1), (8, 2, 2, 0, 0), (4, 1, 4, 2, 0), (3, 3, 0, 0, 0)]


@pytest.mark.parametrize("nq,nkv,mode,pre,nxt", CASES)
def test_gqa_matches_sdpa_enable_gqa(nq, nkv, mode, pre, nxt):
    q, k, v, dy, cu = rand_problem([7, 12, 3], nq, nkv, seed=nq + nkv + mode)
    scale = 0.37
    out, sm, ss = oracle.forward(q, k, v, cu, cu, scale, pre, nxt, mode)
    ref, grads = sdpa_gqa(q, k, v, dy, cu, scale, mode, pre, nxt)
    assert torch.allclose(out, ref, atol=1e-12, rtol=0)
    mine = oracle.backward(q, k, v, dy, out, sm, ss, cu, cu, scale, pre, nxt, mode)
    for a, b in zip(mine, grads):
        assert a.shape == b.shape and torch.allclose(a, b, atol=1e-12, rtol=0)
    # chunked evaluation gives the same result
    ch = oracle.backward(q, k, v, dy, out, sm, ss, cu, cu, scale, pre, nxt, mode, chunk=3)
    for a, b in zip(mine, ch):
        assert torch.allclose(a, b, atol=1e-13, rtol=0)


def test_gqa_finite_differences():
    q, k, v, dy, cu = rand_problem([5, 4], 4, 2, D=4, seed=11)
    scale = 0.8

    def loss():
        o, _, _ = oracle.forward(q, k, v, cu, cu, scale, 2, 1, 4)
        return float((o * dy).sum())

    out, sm, ss = oracle.forward(q, k, v, cu, cu, scale, 2, 1, 4)
    grads = oracle.backward(q, k, v, dy, out, sm, ss, cu, cu, scale, 2, 1, 4)
    h = 1e-6
    for x, g in zip((q, k, v), grads):
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
        assert (fd - g).abs().max() / g.abs().max() <= 1e-6


def test_gqa_head_count_must_divide():
    q, k, v, dy, cu = rand_problem([5], 3, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, cu, cu, 0.5)


MUTATIONS = {
    "kv_head_modulo": ("k[k0:k0 + skv, n // G], v[k0:k0 + skv, n // G]",
                       "k[k0:k0 + skv, n % k.shape[1]], v[k0:k0 + skv, n % k.shape[1]]"),
    "dv_not_summed": (
        "dv[k0 + c0:k0 + c1, n // G] += _dropped(P, Z, rows, c0, c1, keep_prob).T @ dY[rows]",
        "dv[k0 + c0:k0 + c1, n // G] = _dropped(P, Z, rows, c0, c1, keep_prob).T @ dY[rows]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_gqa_pins_catch_planted_mistakes(name):
    src = open(A.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    q, k, v, dy, cu = rand_problem([7, 12], 4, 2, seed=5)
    out, sm, ss = mod.forward(q, k, v, cu, cu, 0.5, 3, 1, 4)
    grads = mod.backward(q, k, v, dy, out, sm, ss, cu, cu, 0.5, 3, 1, 4)
    ref, ref_grads = sdpa_gqa(q, k, v, dy, cu, 0.5, 4, 3, 1)
    ok = torch.allclose(out, ref, atol=1e-12) and all(
        torch.allclose(a, b, atol=1e-12) for a, b in zip(grads, ref_grads))
    assert not ok, name
