"""Pins of the oracle's causal sparse modes 2 and 3 (CPU only).

The pages list LEFT_UP_CAUSAL = 2 and RIGHT_DOWN_CAUSAL = 3 among the sparse
modes (op-plugin sliding-window blog, section 1.3 "SparseMode说明";
explainer 6.6) without printing their masks.  The reading: the causal diagonal
starts in the corner the name gives, so mode 2 keeps j <= i and mode 3 keeps
j - i <= Skv - Sq.  The masks are pinned to torch's own causal biases
(``causal_upper_left`` / ``causal_lower_right``), which state exactly these two
alignments, and the outputs and gradients to torch SDPA + autograd under those
biases, so no reference here goes through the oracle's mask code.
"""
import math
import types

import pytest
import torch
from torch.nn.attention.bias import causal_lower_right, causal_upper_left

import oracle
from oracle import attention as A
import workloads

F64 = torch.float64
SHAPES = [(1, 1), (4, 4), (3, 7), (7, 3), (9, 16), (16, 9), (1, 5), (5, 1)]


def torch_causal(mode, sq, skv):
    """torch's causal mask for the given alignment (True = attend)."""
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")  # lower-right with sq > skv warns about empty rows
        bias = causal_upper_left(sq, skv) if mode == 2 else causal_lower_right(sq, skv)
    return bias._materialize(torch.device("cpu")).to(torch.bool)


def rand_problem(lengths_q, lengths_kv, N=2, D=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(sum(lengths_q), N, D, generator=g, dtype=F64)
    k = torch.randn(sum(lengths_kv), N, D, generator=g, dtype=F64)
    v = torch.randn(sum(lengths_kv), N, D, generator=g, dtype=F64)
    dy = torch.randn(sum(lengths_q), N, D, generator=g, dtype=F64)
    return q, k, v, dy, workloads.cumulative(lengths_q), workloads.cumulative(lengths_kv)


@pytest.mark.parametrize("mode", [2, 3])
@pytest.mark.parametrize("sq,skv", SHAPES)
def test_causal_masks_equal_torch_biases(mode, sq, skv):
    got = oracle.allowed_mask(torch.arange(sq), torch.arange(skv), mode, 5, 7, sq, skv)
    assert torch.equal(got, torch_causal(mode, sq, skv))


@pytest.mark.parametrize("sq,skv", SHAPES + [(300, 1000), (1000, 300)])
def test_causal_pair_counts_closed_form(sq, skv):
    c2 = oracle.allowed_mask(torch.arange(sq), torch.arange(skv), 2, 0, 0, sq, skv).sum(1)
    c3 = oracle.allowed_mask(torch.arange(sq), torch.arange(skv), 3, 0, 0, sq, skv).sum(1)
    for i in range(sq):
        assert int(c2[i]) == min(i + 1, skv)
        assert int(c3[i]) == min(skv, max(0, i + skv - sq + 1))


def test_causal_modes_coincide_for_square_sequences():
    for L in (1, 6, 33):
        m2 = oracle.allowed_mask(torch.arange(L), torch.arange(L), 2, 0, 0, L, L)
        m3 = oracle.allowed_mask(torch.arange(L), torch.arange(L), 3, 0, 0, L, L)
        band = oracle.allowed_mask(torch.arange(L), torch.arange(L), 4, L, 0)
        assert torch.equal(m2, m3) and torch.equal(m2, band)


def sdpa_causal(q, k, v, dy, cu_q, cu_kv, scale, mode):
    """fp64 torch SDPA + autograd per (sequence, head) under torch's causal
    bias; rows with no key (lower-right, Sq > Skv) are left at zero."""
    out = torch.zeros(q.shape[0], q.shape[1], v.shape[2], dtype=F64)
    grads = [torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)]
    for (q0, sq), (k0, skv) in zip(oracle.sequences(cu_q), oracle.sequences(cu_kv)):
        M = torch_causal(mode, sq, skv)
        live = M.any(1)
        rows = torch.nonzero(live).flatten()
        if len(rows) == 0:
            continue
        for n in range(q.shape[1]):
            Q = q[q0:q0 + sq, n][rows].clone().requires_grad_(True)
            K = k[k0:k0 + skv, n].clone().requires_grad_(True)
            V = v[k0:k0 + skv, n].clone().requires_grad_(True)
            O = torch.nn.functional.scaled_dot_product_attention(
                Q[None], K[None], V[None], attn_mask=M[rows][None], scale=scale)[0]
            out[q0 + rows, n] = O.detach()
            O.backward(dy[q0:q0 + sq, n][rows])
            grads[0][q0 + rows, n] = Q.grad
            grads[1][k0:k0 + skv, n] = K.grad
            grads[2][k0:k0 + skv, n] = V.grad
    return out, grads


CASES = [
    (2, [5, 7], [5, 7]),
    (2, [6, 3, 9], [8, 3, 4]),
    (3, [5, 7], [5, 7]),
    (3, [4, 6, 2], [9, 6, 5]),
    (3, [9, 2], [4, 7]),        # Sq > Skv in the first sequence: its first rows are empty
]


@pytest.mark.parametrize("mode,lq,lkv", CASES)
def test_causal_forward_backward_match_sdpa(mode, lq, lkv):
    q, k, v, dy, cu_q, cu_kv = rand_problem(lq, lkv, N=3, seed=len(lq) + mode)
    scale = 0.41
    out, sm, ss = oracle.forward(q, k, v, cu_q, cu_kv, scale, 1, 1, mode)
    ref, (gq, gk, gv) = sdpa_causal(q, k, v, dy, cu_q, cu_kv, scale, mode)
    assert torch.allclose(out, ref, atol=1e-12, rtol=0)
    dq, dk, dv = oracle.backward(q, k, v, dy, out, sm, ss, cu_q, cu_kv, scale, 1, 1, mode)
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        assert torch.allclose(a, b, atol=1e-12, rtol=0)


def test_right_down_empty_rows():
    # Sq = 7 > Skv = 3: rows 0..3 see no key (j <= i - 4)
    q, k, v, dy, cu_q, cu_kv = rand_problem([7], [3], N=1, D=4, seed=2)
    out, sm, ss = oracle.forward(q, k, v, cu_q, cu_kv, 0.5, sparse_mode=3)
    for t in range(4):
        assert out[t].abs().max() == 0 and sm[t, 0] == -math.inf and ss[t, 0] == 0
    assert ss[4, 0] == 1 and torch.allclose(out[4, 0], v[0, 0], atol=1e-15)
    dq, dk, dv = oracle.backward(q, k, v, dy, out, sm, ss, cu_q, cu_kv, 0.5, sparse_mode=3)
    for t in range(4):
        assert dq[t].abs().max() == 0


@pytest.mark.parametrize("mode", [2, 3])
def test_causal_finite_differences(mode):
    q, k, v, dy, cu_q, cu_kv = rand_problem([5, 4], [3, 6], N=1, D=4, seed=11)
    scale = 0.8

    def loss():
        o, _, _ = oracle.forward(q, k, v, cu_q, cu_kv, scale, sparse_mode=mode)
        return float((o * dy).sum())

    out, sm, ss = oracle.forward(q, k, v, cu_q, cu_kv, scale, sparse_mode=mode)
    grads = oracle.backward(q, k, v, dy, out, sm, ss, cu_q, cu_kv, scale, sparse_mode=mode)
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


@pytest.mark.parametrize("mode", [2, 3])
def test_causal_chunked_and_sampled_equal_full(mode):
    q, k, v, dy, cu_q, cu_kv = rand_problem([37, 20], [30, 26], N=1, seed=13)
    full = oracle.forward(q, k, v, cu_q, cu_kv, 0.4, sparse_mode=mode)
    ch = oracle.forward(q, k, v, cu_q, cu_kv, 0.4, sparse_mode=mode, chunk=7)
    for a, b in zip(full, ch):
        assert torch.allclose(a, b, atol=1e-14, rtol=1e-14)
    gf = oracle.backward(q, k, v, dy, *full, cu_q, cu_kv, 0.4, sparse_mode=mode)
    gc = oracle.backward(q, k, v, dy, *full, cu_q, cu_kv, 0.4, sparse_mode=mode, chunk=7)
    for a, b in zip(gf, gc):
        assert torch.allclose(a, b, atol=1e-13, rtol=1e-13)
    # restrictions to a few rows / keys of the first sequence (Sq 37, Skv 30)
    Q, K, V, dY = q[:37, 0], k[:30, 0], v[:30, 0], dy[:37, 0]
    rows = [0, 3, 4, 5, 21, 36]
    o, m, l = oracle.forward_rows(Q, K, V, rows, 0.4, mode)
    assert torch.allclose(o, full[0][rows, 0], atol=1e-14)
    assert torch.allclose(oracle.backward_rows(Q, K, V, dY, rows, 0.4, mode), gf[0][rows, 0],
                          atol=1e-13)
    dk_s, dv_s = oracle.backward_keys(Q, K, V, dY, 10, 17, 0.4, mode)
    assert torch.allclose(dk_s, gf[1][10:17, 0], atol=1e-13)
    assert torch.allclose(dv_s, gf[2][10:17, 0], atol=1e-13)


MUTATIONS = {
    "left_up_strict": ("return d <= 0", "return d < 0"),
    "right_down_flipped": ("return d <= int(skv) - int(sq)", "return d <= int(sq) - int(skv)"),
    "right_down_window": ("lo, hi = 0, min(skv, r1 + skv - sq)", "lo, hi = 0, min(skv, r1)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_causal_pins_catch_planted_mistakes(name):
    src = open(A.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    caught = False
    for mode, lq, lkv in CASES:
        q, k, v, dy, cu_q, cu_kv = rand_problem(lq, lkv, N=1, seed=7)
        ref, _ = sdpa_causal(q, k, v, dy, cu_q, cu_kv, 0.5, mode)
        for chunk in (None, 3):
            out, _, _ = mod.forward(q, k, v, cu_q, cu_kv, 0.5, sparse_mode=mode, chunk=chunk)
            caught |= not torch.allclose(out, ref, atol=1e-12)
    assert caught, name
