"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each check is chosen so that a plausible mistake in the oracle (a dropped
scale, a wrong sign, a transposed operand, a mirrored band, a wrong softmax
statistic) fails at least one of them; ``test_pins_catch_planted_mistakes``
plants such mistakes in a copy of the oracle and asserts that they are caught.
"""
import json
import math
import os

import pytest
import torch

import oracle
from oracle import attention as A
import workloads

F64 = torch.float64


def rand_problem(lengths, N=2, D=8, seed=0, lengths_kv=None):
    g = torch.Generator().manual_seed(seed)
    lk = lengths if lengths_kv is None else lengths_kv
    q = torch.randn(sum(lengths), N, D, generator=g, dtype=F64)
    k = torch.randn(sum(lk), N, D, generator=g, dtype=F64)
    v = torch.randn(sum(lk), N, D, generator=g, dtype=F64)
    dy = torch.randn(sum(lengths), N, D, generator=g, dtype=F64)
    return q, k, v, dy, workloads.cumulative(lengths), workloads.cumulative(lk)


# ---------------------------------------------------------------- sequences

def test_sequences_trailing_zero_batches():
    # explainer section 6.4: real lengths [2, 3, 4, 5, 6], last two not participating
    assert oracle.sequences([2, 5, 9, 0, 0]) == [(0, 2), (2, 3), (5, 4)]
    assert oracle.sequences([0, 3, 3, 7]) == [(0, 0), (0, 3), (3, 0), (3, 4)]
    assert oracle.sequences([256]) == [(0, 256)]
    with pytest.raises(ValueError):
        oracle.sequences([5, 3])


# ---------------------------------------------------------------- band mask

@pytest.mark.parametrize("pre,nxt", [(2, 1), (0, 0), (3, -1), (-1, 2), (100, 100)])
def test_band_mask_equals_literal_rule(pre, nxt):
    sq = skv = 9
    got = oracle.allowed_mask(torch.arange(sq), torch.arange(skv), 4, pre, nxt)
    for i in range(sq):
        for j in range(skv):
            assert bool(got[i, j]) == (-pre <= j - i <= nxt)


def test_band_mask_hand_example():
    # pre_tokens = 2 keys to the left, next_tokens = 1 key to the right
    expect = torch.tensor([
        [1, 1, 0, 0, 0, 0],
        [1, 1, 1, 0, 0, 0],
        [1, 1, 1, 1, 0, 0],
        [0, 1, 1, 1, 1, 0],
        [0, 0, 1, 1, 1, 1],
        [0, 0, 0, 1, 1, 1]], dtype=torch.bool)
    got = oracle.allowed_mask(torch.arange(6), torch.arange(6), 4, 2, 1)
    assert torch.equal(got, expect)


def test_mode0_ignores_pre_next():
    assert oracle.allowed_mask(torch.arange(5), torch.arange(7), 0, 0, 0).all()


@pytest.mark.parametrize("L,pre,nxt", [(50, 7, 3), (50, 0, 0), (16384, 2048, 0), (30, 100, 2)])
def test_band_pair_counts_closed_form(L, pre, nxt):
    counts = oracle.allowed_mask(torch.arange(L), torch.arange(L), 4, pre, nxt).sum(1)
    for i in range(0, L, max(1, L // 64)):
        expect = max(0, min(L - 1, i + nxt) - max(0, i - pre) + 1)
        assert int(counts[i]) == expect
    if L > pre and L > nxt:
        total = L * (pre + nxt + 1) - pre * (pre + 1) // 2 - nxt * (nxt + 1) // 2
        assert int(counts.sum()) == total


def test_headline_pair_count():
    # 16K sliding window (pre 2048, next 0): 16384 * 2049 - 2048 * 2049 / 2 per head
    p = workloads.make_problem(workloads.HEADLINE)
    assert oracle.count_pairs(p.cu_seqlens_q, p.cu_seqlens_kv, 4, 2048, 0) == 31_472_640


# ---------------------------------------------------------------- library routine

def sdpa_reference(q, k, v, cu_q, cu_kv, scale, mode, pre, nxt, dy=None):
    """fp64 torch SDPA (+ autograd) per (sequence, head) with a boolean mask."""
    out = torch.zeros(q.shape[0], q.shape[1], v.shape[2], dtype=F64)
    grads = [torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)]
    for (q0, sq), (k0, skv) in zip(oracle.sequences(cu_q), oracle.sequences(cu_kv)):
        for n in range(q.shape[1]):
            Q = q[q0:q0 + sq, n].clone().requires_grad_(True)
            K = k[k0:k0 + skv, n].clone().requires_grad_(True)
            V = v[k0:k0 + skv, n].clone().requires_grad_(True)
            M = oracle.allowed_mask(torch.arange(sq), torch.arange(skv), mode, pre, nxt)
            O = torch.nn.functional.scaled_dot_product_attention(
                Q[None], K[None], V[None], attn_mask=M[None], scale=scale)[0]
            out[q0:q0 + sq, n] = O.detach()
            if dy is not None:
                O.backward(dy[q0:q0 + sq, n])
                grads[0][q0:q0 + sq, n] = Q.grad
                grads[1][k0:k0 + skv, n] = K.grad
                grads[2][k0:k0 + skv, n] = V.grad
    return out, grads


CASES = [
    ([5, 7], 0, 0, 0),
    ([13, 1, 9], 4, 3, 2),
    ([20, 6], 4, 4, 0),
    ([16, 11], 4, 0, 5),
]


@pytest.mark.parametrize("lengths,mode,pre,nxt", CASES)
def test_forward_backward_match_sdpa_autograd(lengths, mode, pre, nxt):
    q, k, v, dy, cu_q, cu_kv = rand_problem(lengths, N=3, D=8, seed=len(lengths) + pre)
    scale = 0.37
    out, sm, ss = oracle.forward(q, k, v, cu_q, cu_kv, scale, pre, nxt, mode)
    ref, (gq, gk, gv) = sdpa_reference(q, k, v, cu_q, cu_kv, scale, mode, pre, nxt, dy)
    assert torch.allclose(out, ref, atol=1e-12, rtol=0)
    dq, dk, dv = oracle.backward(q, k, v, dy, out, sm, ss, cu_q, cu_kv, scale, pre, nxt, mode)
    assert torch.allclose(dq, gq, atol=1e-12, rtol=0)
    assert torch.allclose(dk, gk, atol=1e-12, rtol=0)
    assert torch.allclose(dv, gv, atol=1e-12, rtol=0)


def test_dense_cross_sequence_mode0_with_unequal_lengths():
    # mode 0 allows Sq != Skv per batch
    q, k, v, dy, cu_q, cu_kv = rand_problem([4, 9], N=2, D=8, seed=3, lengths_kv=[7, 2])
    out, sm, ss = oracle.forward(q, k, v, cu_q, cu_kv, 0.5, sparse_mode=0)
    ref, (gq, gk, gv) = sdpa_reference(q, k, v, cu_q, cu_kv, 0.5, 0, 0, 0, dy)
    assert torch.allclose(out, ref, atol=1e-12, rtol=0)
    dq, dk, dv = oracle.backward(q, k, v, dy, out, sm, ss, cu_q, cu_kv, 0.5)
    assert torch.allclose(dk, gk, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("mode,pre,nxt", [(0, oracle.INT_MAX, oracle.INT_MAX), (4, 2, 1)])
def test_finite_differences(mode, pre, nxt):
    q, k, v, dy, cu, _ = rand_problem([5, 7], N=2, D=4, seed=11)
    scale = 0.8

    def loss(q_, k_, v_):
        o, _, _ = oracle.forward(q_, k_, v_, cu, cu, scale, pre, nxt, mode)
        return float((o * dy).sum())

    out, sm, ss = oracle.forward(q, k, v, cu, cu, scale, pre, nxt, mode)
    grads = oracle.backward(q, k, v, dy, out, sm, ss, cu, cu, scale, pre, nxt, mode)
    h = 1e-6
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        fd = torch.zeros_like(x)
        flat = x.view(-1)
        for idx in range(flat.numel()):
            old = float(flat[idx])
            flat[idx] = old + h
            lp = loss(q, k, v)
            flat[idx] = old - h
            lm = loss(q, k, v)
            flat[idx] = old
            fd.view(-1)[idx] = (lp - lm) / (2 * h)
        err = (fd - g).abs().max() / g.abs().max()
        assert err <= 1e-6, (which, float(err))


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("lengths,mode,pre,nxt", CASES)
def test_softmax_rows_sum_to_one(lengths, mode, pre, nxt):
    q, k, v, dy, cu_q, cu_kv = rand_problem(lengths, seed=5)
    _, sm, ss = oracle.forward(q, k, v, cu_q, cu_kv, 0.6, pre, nxt, mode)
    for (q0, sq), (k0, skv) in zip(oracle.sequences(cu_q), oracle.sequences(cu_kv)):
        for n in range(q.shape[1]):
            S = 0.6 * q[q0:q0 + sq, n] @ k[k0:k0 + skv, n].T
            M = oracle.allowed_mask(torch.arange(sq), torch.arange(skv), mode, pre, nxt)
            P = torch.exp(S - sm[q0:q0 + sq, n, None]) / ss[q0:q0 + sq, n, None]
            rows = (P * M).sum(1)
            assert (rows - 1).abs().max() <= 1e-12
            # softmax_max is the max over allowed scaled scores
            Sm = S.masked_fill(~M, -math.inf).max(1).values
            assert torch.allclose(Sm, sm[q0:q0 + sq, n], atol=1e-14, rtol=0)


@pytest.mark.parametrize("lengths,mode,pre,nxt", CASES)
def test_gradient_sum_invariants(lengths, mode, pre, nxt):
    # sum_j P_ij = 1  =>  sum_j dV_j = sum_i dY_i ;  sum_j dS_ij = 0  =>  sum_j dK_j = 0
    q, k, v, dy, cu_q, cu_kv = rand_problem(lengths, seed=9)
    out, sm, ss = oracle.forward(q, k, v, cu_q, cu_kv, 0.45, pre, nxt, mode)
    dq, dk, dv = oracle.backward(q, k, v, dy, out, sm, ss, cu_q, cu_kv, 0.45, pre, nxt, mode)
    for (q0, sq), (k0, skv) in zip(oracle.sequences(cu_q), oracle.sequences(cu_kv)):
        assert torch.allclose(dv[k0:k0 + skv].sum(0), dy[q0:q0 + sq].sum(0), atol=1e-12)
        assert dk[k0:k0 + skv].sum(0).abs().max() <= 1e-12


def test_varlen_equals_separate_calls_exactly():
    lengths = [6, 1, 11, 4]
    q, k, v, dy, cu, _ = rand_problem(lengths, N=2, D=8, seed=21)
    for mode, pre, nxt in [(0, 0, 0), (4, 3, 1)]:
        out, sm, ss = oracle.forward(q, k, v, cu, cu, 0.7, pre, nxt, mode)
        grads = oracle.backward(q, k, v, dy, out, sm, ss, cu, cu, 0.7, pre, nxt, mode)
        for s0, L in oracle.sequences(cu):
            sl = slice(s0, s0 + L)
            o1, m1, l1 = oracle.forward(q[sl], k[sl], v[sl], [L], [L], 0.7, pre, nxt, mode)
            assert torch.equal(o1, out[sl]) and torch.equal(m1, sm[sl]) and torch.equal(l1, ss[sl])
            g1 = oracle.backward(q[sl], k[sl], v[sl], dy[sl], o1, m1, l1, [L], [L], 0.7,
                                 pre, nxt, mode)
            for a, b in zip(g1, grads):
                assert torch.equal(a, b[sl])


def test_query_zero_gives_band_mean():
    q, k, v, dy, cu, _ = rand_problem([10], N=1, D=4, seed=2)
    q.zero_()
    out, sm, ss = oracle.forward(q, k, v, cu, cu, 1.0, 2, 1, 4)
    for i in range(10):
        lo, hi = max(0, i - 2), min(9, i + 1)
        assert torch.allclose(out[i, 0], v[lo:hi + 1, 0].mean(0), atol=1e-14)
        assert ss[i, 0] == hi - lo + 1 and sm[i, 0] == 0
    # backward with q = 0: dV_j = sum_{i attends j} dY_i / count_i
    dq, dk, dv = oracle.backward(q, k, v, dy, out, sm, ss, cu, cu, 1.0, 2, 1, 4)
    for j in range(10):
        exp = sum(dy[i, 0] / float(ss[i, 0]) for i in range(10) if -2 <= j - i <= 1)
        assert torch.allclose(dv[j, 0], exp, atol=1e-14)


def test_single_key_gives_value():
    q, k, v, dy, cu_q, cu_kv = rand_problem([5], N=2, D=4, seed=4, lengths_kv=[1])
    out, _, ss = oracle.forward(q, k, v, cu_q, cu_kv, 0.3)
    assert torch.allclose(out, v.expand(5, 2, 4), atol=1e-15)
    assert torch.all(ss == 1)


def test_key_shift_invariance():
    q, k, v, dy, cu, _ = rand_problem([9], N=1, D=4, seed=6)
    shift = torch.tensor([0.3, -1.2, 2.0, 0.5], dtype=F64)
    for mode, pre, nxt in [(0, 0, 0), (4, 2, 2)]:
        o1, m1, l1 = oracle.forward(q, k, v, cu, cu, 0.5, pre, nxt, mode)
        o2, m2, l2 = oracle.forward(q, k + shift, v, cu, cu, 0.5, pre, nxt, mode)
        assert torch.allclose(o1, o2, atol=1e-12)
        g1 = oracle.backward(q, k, v, dy, o1, m1, l1, cu, cu, 0.5, pre, nxt, mode)
        g2 = oracle.backward(q, k + shift, v, dy, o2, m2, l2, cu, cu, 0.5, pre, nxt, mode)
        assert torch.allclose(g1[0], g2[0], atol=1e-12)


# ---------------------------------------------------------------- worked examples

def test_varlen_forward_example_closed_form(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "varlen_fwd_constant_inputs.json")))
    p = fx["problem"]
    for case in fx["cases"]:
        x = torch.full((p["T"], p["N"], p["D"]), case["input_value"], dtype=F64)
        out, sm, ss = oracle.forward(x, x, x, p["cu_seqlens"], p["cu_seqlens"], p["scale"],
                                     p["pre_tokens"], p["next_tokens"], p["sparse_mode"])
        assert torch.allclose(out, torch.full_like(out, case["out"]), rtol=1e-14, atol=0)
        assert torch.allclose(sm, torch.full_like(sm, case["softmax_max"]), rtol=1e-14, atol=0)
        assert torch.allclose(ss, torch.full_like(ss, case["softmax_sum"]), rtol=1e-14, atol=0)


def test_unpadding_grad_example_closed_form(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "unpadding_grad_constant_inputs.json")))
    p = fx["problem"]
    shp = (p["T"], p["N"], p["D"])
    ones = torch.ones(shp, dtype=F64)
    st = torch.full((p["T"], p["N"], 8), 3.0, dtype=F64)
    dq, dk, dv = oracle.backward(ones, ones, ones, ones, ones, st, st, p["cu_seqlens"],
                                 p["cu_seqlens"], p["scale"], p["pre_tokens"],
                                 p["next_tokens"], p["sparse_mode"])
    assert dq.abs().max() == fx["dq"] and dk.abs().max() == fx["dk"]
    assert torch.allclose(dv, torch.full_like(dv, fx["dv"]), rtol=1e-12, atol=0)


# ---------------------------------------------------------------- edge cases

def test_empty_rows_and_nonparticipating_tokens():
    # pre 3, next -2: rows 0 and 1 of each sequence see no key
    q, k, v, dy, cu, _ = rand_problem([6, 3], N=1, D=4, seed=8)
    T = q.shape[0]
    extra = torch.randn(2, 1, 4, dtype=F64)
    q2, k2, v2, dy2 = (torch.cat([x, extra]) for x in (q, k, v, dy))
    cu2 = cu + [0, 0]  # two trailing non-participating batches; 2 tokens past the end
    out, sm, ss = oracle.forward(q2, k2, v2, cu2, cu2, 0.5, 3, -2, 4)
    for t in [0, 1, 6, 7, T, T + 1]:
        assert out[t].abs().max() == 0 and ss[t, 0] == 0 and sm[t, 0] == -math.inf
    assert ss[2, 0] == 1
    dq, dk, dv = oracle.backward(q2, k2, v2, dy2, out, sm, ss, cu2, cu2, 0.5, 3, -2, 4)
    for t in [0, 1, 6, 7, T, T + 1]:
        assert dq[t].abs().max() == 0
    # keys j >= L - 2 are never attended (j - i <= -2)
    for t in [4, 5, 8, T, T + 1]:
        assert dk[t].abs().max() == 0 and dv[t].abs().max() == 0


def test_zero_length_sequences():
    q, k, v, dy, _, _ = rand_problem([4], N=1, D=4, seed=1)
    cu = [0, 4, 4]
    out, sm, ss = oracle.forward(q, k, v, cu, cu, 0.5)
    o1, _, _ = oracle.forward(q, k, v, [4], [4], 0.5)
    assert torch.equal(out, o1)


# ---------------------------------------------------------------- evaluation order

@pytest.mark.parametrize("mode,pre,nxt", [(0, 0, 0), (4, 5, 2), (4, 0, 7)])
def test_chunked_equals_full(mode, pre, nxt):
    q, k, v, dy, cu, _ = rand_problem([37, 20], N=2, D=8, seed=13)
    full = oracle.forward(q, k, v, cu, cu, 0.4, pre, nxt, mode)
    ch = oracle.forward(q, k, v, cu, cu, 0.4, pre, nxt, mode, chunk=7)
    for a, b in zip(full, ch):
        assert torch.allclose(a, b, atol=1e-14, rtol=1e-14)
    gf = oracle.backward(q, k, v, dy, *full, cu, cu, 0.4, pre, nxt, mode)
    gc = oracle.backward(q, k, v, dy, *full, cu, cu, 0.4, pre, nxt, mode, chunk=7)
    for a, b in zip(gf, gc):
        assert torch.allclose(a, b, atol=1e-13, rtol=1e-13)


@pytest.mark.parametrize("mode,pre,nxt", [(0, 0, 0), (4, 5, 2)])
def test_sampled_restrictions_equal_full(mode, pre, nxt):
    q, k, v, dy, cu, _ = rand_problem([40], N=1, D=8, seed=17)
    out, sm, ss = oracle.forward(q, k, v, cu, cu, 0.4, pre, nxt, mode)
    dq, dk, dv = oracle.backward(q, k, v, dy, out, sm, ss, cu, cu, 0.4, pre, nxt, mode)
    Q, K, V, dY = q[:, 0], k[:, 0], v[:, 0], dy[:, 0]
    rows = [0, 3, 4, 5, 21, 39]
    o, m, l = oracle.forward_rows(Q, K, V, rows, 0.4, mode, pre, nxt)
    assert torch.allclose(o, out[rows, 0], atol=1e-14)
    assert torch.allclose(l, ss[rows, 0], atol=1e-13)
    assert torch.allclose(oracle.backward_rows(Q, K, V, dY, rows, 0.4, mode, pre, nxt),
                          dq[rows, 0], atol=1e-13)
    dk_s, dv_s = oracle.backward_keys(Q, K, V, dY, 10, 17, 0.4, mode, pre, nxt)
    assert torch.allclose(dk_s, dk[10:17, 0], atol=1e-13)
    assert torch.allclose(dv_s, dv[10:17, 0], atol=1e-13)


# ---------------------------------------------------------------- the pins bite

MUTATIONS = {
    "dk_without_scale": ("dk[k0 + c0:k0 + c1, n // G] += scale * (dS.T @ Q[rows])",
                         "dk[k0 + c0:k0 + c1, n // G] += (dS.T @ Q[rows])"),
    "dv_transposed_operand": (
        "dv[k0 + c0:k0 + c1, n // G] += _dropped(P, Z, rows, c0, c1, keep_prob).T @ dY[rows]",
        "dv[k0 + c0:k0 + c1, n // G] += (_dropped(P, Z, rows, c0, c1, keep_prob).T @ dY[rows])"
        ".flip(0)"),
    "ds_sign": ("dS = P * (dP - Dv[:, None])", "dS = P * (Dv[:, None] - dP)"),
    "band_mirrored": ("return (d >= -int(pre_tokens)) & (d <= int(next_tokens))",
                      "return (d >= -int(next_tokens)) & (d <= int(pre_tokens))"),
    "max_unscaled": ("S = scale * (Q[rows] @ K[c0:c1].T)", "S = (Q[rows] @ K[c0:c1].T)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistakes(name):
    """Plant a mistake in a private copy of the oracle; a pin must fail."""
    import types
    src = open(A.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    q, k, v, dy, cu, _ = rand_problem([6, 9], N=2, D=8, seed=31)
    mode, pre, nxt, scale = 4, 3, 1, 0.45
    out, sm, ss = mod.forward(q, k, v, cu, cu, scale, pre, nxt, mode)
    grads = mod.backward(q, k, v, dy, out, sm, ss, cu, cu, scale, pre, nxt, mode)
    ref, ref_grads = sdpa_reference(q, k, v, cu, cu, scale, 4, 3, 1, dy)
    # literal band rule, independent of the mutated mask
    band_ok = all(bool(mod.allowed_mask(torch.arange(6), torch.arange(6), 4, 3, 1)[i, j])
                  == (-3 <= j - i <= 1) for i in range(6) for j in range(6))
    fwd_ok = torch.allclose(out, ref, atol=1e-12)
    bwd_ok = all(torch.allclose(a, b, atol=1e-12) for a, b in zip(grads, ref_grads))
    assert not (band_ok and fwd_ok and bwd_ok), name


# ---------------------------------------------------------------- tile enumerator

# Tile tables derived by hand from the band rule -pre <= j - i <= next with 64 x 64
# tiles (P = partial, F = full, unlisted tiles skipped).  A tile is full only if
# all of its 64 x 64 elements lie inside the sequence and inside the band.
from oracle.tiles import FULL as F_, PARTIAL as P_  # noqa: E402
HAND_TILES = [
    # one 200-token sequence, pre 130, next 64: rows 192..199 form a ragged
    # query block and keys 192..199 a ragged key tile.  Per query block (rows
    # r..r+63) the offsets j - i of key tile t span [64 (t - b) - 63, 64 (t - b) + 63]
    # with b the block index: inside [-130, 64] for t - b in {-1, 0} (full if
    # complete), partly for t - b in {-2, 1}, never beyond.
    dict(lengths=[200], mode=4, pre=130, nxt=64, direction="fwd", expect={
        (0, 0): [(0, F_), (1, P_)],
        (0, 1): [(0, F_), (1, F_), (2, P_)],
        (0, 2): [(0, P_), (1, F_), (2, F_), (3, P_)],
        # ragged rows 192..199: tile 2 would be full if rows past the end counted
        (0, 3): [(0, P_), (1, P_), (2, P_), (3, P_)],
    }),
    # the same tiles seen from the key side (items = key blocks, tiles = query
    # blocks): the transpose of the table above
    dict(lengths=[200], mode=4, pre=130, nxt=64, direction="bwd", expect={
        (0, 0): [(0, F_), (1, F_), (2, P_), (3, P_)],
        (0, 1): [(0, P_), (1, F_), (2, F_), (3, P_)],
        (0, 2): [(1, P_), (2, F_), (3, P_)],
        (0, 3): [(2, P_), (3, P_)],
    }),
    # 130 tokens, pre 64, next 0 (the diagonal tile always misses j > i)
    dict(lengths=[130], mode=4, pre=64, nxt=0, direction="fwd", expect={
        (0, 0): [(0, P_)],
        (0, 1): [(0, P_), (1, P_)],
        (0, 2): [(1, P_), (2, P_)],
    }),
    # no mask, 130 queries over 70 keys (a second batch after a zero-length
    # one): only the complete 64 x 64 tiles are full
    dict(lengths=[0, 130], lengths_kv=[0, 70], mode=0, pre=0, nxt=0, direction="fwd", expect={
        (1, 0): [(0, F_), (1, P_)],
        (1, 1): [(0, F_), (1, P_)],
        (1, 2): [(0, P_), (1, P_)],
    }),
    # the same from the key side: key blocks 0..63 and 64..69 over query blocks
    dict(lengths=[0, 130], lengths_kv=[0, 70], mode=0, pre=0, nxt=0, direction="bwd", expect={
        (1, 0): [(0, F_), (1, F_), (2, P_)],
        (1, 1): [(0, P_), (1, P_), (2, P_)],
    }),
]


@pytest.mark.parametrize("case", range(len(HAND_TILES)))
def test_tile_enumerator_hand_tables(case):
    c = HAND_TILES[case]
    cu_q = workloads.cumulative(c["lengths"])
    cu_kv = workloads.cumulative(c.get("lengths_kv", c["lengths"]))
    got = oracle.enumerate_tiles(cu_q, cu_kv, c["mode"], c["pre"], c["nxt"], 64, 64,
                                 c["direction"])
    expect = dict(c["expect"])
    for key in got:          # items of zero-length sequences are absent from both
        expect.setdefault(key, [])
    assert got == expect


TILE_MUTATIONS = {
    "rows_past_the_end_count": ("m &= (rows < sq)[:, None] & (cols < skv)[None, :]",
                                "m &= (cols < skv)[None, :]"),
    "keys_past_the_end_count": ("m &= (rows < sq)[:, None] & (cols < skv)[None, :]",
                                "m &= (rows < sq)[:, None]"),
    "full_if_any": ("return FULL if mask_block.all() else PARTIAL",
                    "return FULL if mask_block.any() else PARTIAL"),
    "bwd_counts_from_query_length": ("-(-skv // block_item), -(-sq // block_tile)",
                                     "-(-sq // block_item), -(-skv // block_tile)"),
}


@pytest.mark.parametrize("name", sorted(TILE_MUTATIONS))
def test_tile_pins_catch_planted_mistakes(name):
    import types

    from oracle import tiles as T
    src = open(T.__file__).read()
    old, new = TILE_MUTATIONS[name]
    assert old in src
    src = src.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("tiles_mutant")
    exec(compile(src, "tiles_mutant", "exec"), mod.__dict__)
    caught = False
    for c in HAND_TILES:
        cu_q = workloads.cumulative(c["lengths"])
        cu_kv = workloads.cumulative(c.get("lengths_kv", c["lengths"]))
        got = mod.enumerate_tiles(cu_q, cu_kv, c["mode"], c["pre"], c["nxt"], 64, 64,
                                  c["direction"])
        got = {k: v for k, v in got.items() if v}
        caught |= got != c["expect"]
    assert caught, name
