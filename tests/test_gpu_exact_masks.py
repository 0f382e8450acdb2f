"""Bit-exact mask and skip patterns of the backward kernels (needs an MI355X).

The dK/dV kernels (one per key block) and the dQ kernels (one per query
block) each carry their own band and tail masks, so each is checked on inputs
that make every gradient an exact integer count of allowed (query, key)
pairs.  With the caller's statistics softmax_max = 0 and softmax_sum = 1,
all scores 0 (q = 0 or k = 0), out = 0 (so D = rowsum(dY o out) = 0),
v = 1 and dY_i = e_(i mod D):

    P_ij = 1 on allowed pairs, dP_ij = dY_i . V_j = 1, dS_ij = P_ij (dP_ij - 0) = 1,
    dV_j[c] = #{allowed i : i = c mod D},
    dQ_i[c] = scale #{allowed j : j = c mod D}   (k_j = e_(j mod D), q = 0),
    dK_j[c] = scale #{allowed i : i = c mod D}   (q_i = e_(i mod D), k = 0),

with dropout (keep bit Z, keep_prob 1/2) each allowed pair counting Z / keep_prob
instead of 1.  Small integers and their halves are exact in bf16 and fp32
whatever the summation order, so the results must equal the counts bit for
bit: a band edge or tail off by one row or key changes one count by one.
The counts come from the oracle's element mask (oracle.allowed_mask, pinned
to the literal rule by the CPU tests).
"""
import pytest
import torch
import torch.nn.functional as F

import oracle
import transformer_attention_tnd_amd as swa
import workloads
from parity_utils import note, require_gpu

pytestmark = pytest.mark.gpu
SCALE = 0.5


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def expected_counts(p, nq, nkv, D, keep=None, keep_prob=1.0):
    """Row counts by key class [Tq, Nq, D] and key counts by row class
    [Tkv, Nkv, D] (summed over each key/value head's query heads)."""
    G = nq // nkv
    rowc = torch.zeros(p.q.shape[0], nq, D)
    colc = torch.zeros(p.k.shape[0], nkv, D)
    for b, ((q0, sq), (k0, skv)) in enumerate(zip(oracle.sequences(p.cu_seqlens_q),
                                                  oracle.sequences(p.cu_seqlens_kv))):
        hot_k = F.one_hot(torch.arange(skv) % D, D).float()
        hot_q = F.one_hot(torch.arange(sq) % D, D).float()
        for r0 in range(0, sq, 2048):
            rows = torch.arange(r0, min(sq, r0 + 2048))
            M = oracle.allowed_mask(rows, torch.arange(skv), p.sparse_mode, p.pre_tokens,
                                    p.next_tokens, sq, skv).float()
            for n in range(nq):
                W = M if keep is None else M * keep[(b, n)][rows].float() / keep_prob
                rowc[q0 + rows, n] = W @ hot_k
                colc[k0:k0 + skv, n // G] += W.T @ hot_q[rows]
    return rowc, colc


def one_hot_rows(T, N, D, cu, dtype):
    x = torch.zeros(T, N, D, dtype=dtype)
    for s0, L in oracle.sequences(cu):
        x[s0 + torch.arange(L), :, torch.arange(L) % D] = 1
    return x


def backward_counts(p, dev, which, drop_mask=None, keep_prob=1.0):
    """Run the backward with the inputs of the module docstring: which = 'dq'
    (q = 0, k one-hot) or 'dk' (k = 0, q one-hot)."""
    T, N, D = p.q.shape
    Tk, Nk = p.k.shape[:2]
    dt = p.dtype
    if which == "dq":
        q = torch.zeros(T, N, D, dtype=dt)
        k = one_hot_rows(Tk, Nk, D, p.cu_seqlens_kv, dt)
    else:
        q = one_hot_rows(T, N, D, p.cu_seqlens_q, dt)
        k = torch.zeros(Tk, Nk, D, dtype=dt)
    v = torch.ones(Tk, Nk, D, dtype=dt)
    dy = one_hot_rows(T, N, D, p.cu_seqlens_q, dt)
    out = torch.zeros(T, N, D, dtype=dt)
    smax = torch.zeros(T, N, 8)
    ssum = torch.ones(T, N, 8)
    args = [x.to(dev) for x in (q, k, v, dy, out, smax, ssum)]
    mask = None if drop_mask is None else drop_mask.to(dev)
    dq, dk, dv = swa.backward(*args, p.cu_seqlens_q, p.cu_seqlens_kv, SCALE, p.pre_tokens,
                              p.next_tokens, p.sparse_mode, drop_mask=mask,
                              keep_prob=keep_prob)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def assert_equal_counts(name, got, expect):
    got = got.float()
    bad = got != expect
    if bad.any():
        idx = bad.nonzero()[0].tolist()
        raise AssertionError(f"{name}: {int(bad.sum())} elements differ from the counts, "
                             f"first at {idx}: {float(got[tuple(idx)])} != "
                             f"{float(expect[tuple(idx)])}")


CASES = {
    "band_ragged": dict(lengths_q=[300, 77, 513], sparse_mode=4, pre_tokens=70, next_tokens=9),
    "band_negative_pre": dict(lengths_q=[260, 129], sparse_mode=4, pre_tokens=-3,
                              next_tokens=9),
    "band_negative_next": dict(lengths_q=[150, 90], sparse_mode=4, pre_tokens=70,
                               next_tokens=-5),
    "band_wide_both_sides": dict(lengths_q=[700, 129], sparse_mode=4, pre_tokens=200,
                                 next_tokens=130),
    "left_up_causal_unequal": dict(lengths_q=[300, 513], lengths_kv=[700, 260],
                                   sparse_mode=2),
    "right_down_causal_unequal": dict(lengths_q=[513, 77, 300], lengths_kv=[260, 300, 301],
                                      sparse_mode=3),
    "dense_unequal_tails": dict(lengths_q=[77, 190], lengths_kv=[50, 260], sparse_mode=0),
    "gqa2_band": dict(lengths_q=[300, 77], num_heads=4, num_kv_heads=2, sparse_mode=4,
                      pre_tokens=100, next_tokens=3),
}
DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}
HEAD_DIMS = {"d128": 128, "d64": 64}


@pytest.mark.parametrize("hd", sorted(HEAD_DIMS))
@pytest.mark.parametrize("dt", sorted(DTYPES))
@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_mask_pattern_is_exact(dev, case, dt, hd):
    kw = dict(CASES[case])
    kw.setdefault("num_heads", 2)
    p = workloads.make_custom(head_dim=HEAD_DIMS[hd], dtype=DTYPES[dt], **kw)
    note(f"[exact backward] {case} {dt} {hd} cu_q={p.cu_seqlens_q} cu_kv={p.cu_seqlens_kv}")
    N, Nk, D = p.q.shape[1], p.k.shape[1], p.q.shape[2]
    rowc, colc = expected_counts(p, N, Nk, D)
    dq, dk, dv = backward_counts(p, dev, "dq")
    assert_equal_counts("dq", dq, SCALE * rowc)
    assert_equal_counts("dv", dv, colc)
    assert not dk.float().any()
    dq, dk, dv = backward_counts(p, dev, "dk")
    assert_equal_counts("dk", dk, SCALE * colc)
    assert_equal_counts("dv", dv, colc)
    assert not dq.float().any()


@pytest.mark.parametrize("dt", sorted(DTYPES))
@pytest.mark.parametrize("case", ["band_ragged", "right_down_causal_unequal", "gqa2_band"])
def test_backward_mask_pattern_with_dropout_is_exact(dev, case, dt):
    """The dropout instantiations apply the keep bits on top of the band."""
    kw = dict(CASES[case])
    kw.setdefault("num_heads", 2)
    p = workloads.make_custom(head_dim=128, dtype=DTYPES[dt], **kw)
    mask = workloads.make_drop_mask(p, 0.5)
    keep = oracle.unpack_drop_mask(mask, p.cu_seqlens_q, p.cu_seqlens_kv, p.q.shape[1])
    note(f"[exact backward dropout] {case} {dt}")
    rowc, colc = expected_counts(p, p.q.shape[1], p.k.shape[1], 128, keep, 0.5)
    dq, dk, dv = backward_counts(p, dev, "dq", mask, 0.5)
    assert_equal_counts("dq", dq, SCALE * rowc)
    assert_equal_counts("dv", dv, colc)
    dq, dk, dv = backward_counts(p, dev, "dk", mask, 0.5)
    assert_equal_counts("dk", dk, SCALE * colc)
    assert_equal_counts("dv", dv, colc)


def test_backward_mask_pattern_16k_window_is_exact(dev):
    """The band of the 16K sliding-window workload (pre 2048, next 0), one head."""
    p = workloads.make_custom([16384], num_heads=1, head_dim=128, sparse_mode=4,
                              pre_tokens=2048, next_tokens=0)
    note("[exact backward] 16K window")
    rowc, colc = expected_counts(p, 1, 1, 128)
    dq, dk, dv = backward_counts(p, dev, "dq")
    assert_equal_counts("dq", dq, SCALE * rowc)
    assert_equal_counts("dv", dv, colc)
    dq, dk, dv = backward_counts(p, dev, "dk")
    assert_equal_counts("dk", dk, SCALE * colc)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", sorted(DTYPES))
def test_forward_mask_pattern_with_dropout(dev, dt, D):
    """Forward with dropout, q = 0: softmax_sum is the undropped count of
    allowed keys exactly, softmax_max is 0, and with V_j = e_(j mod D) out is
    zero exactly where no kept allowed key falls in class c."""
    p = workloads.make_custom([300, 77, 513], num_heads=2, head_dim=D, dtype=DTYPES[dt],
                              sparse_mode=4, pre_tokens=70, next_tokens=9)
    mask = workloads.make_drop_mask(p, 0.5)
    keep = oracle.unpack_drop_mask(mask, p.cu_seqlens_q, p.cu_seqlens_kv, 2)
    p.q.zero_()
    p.v.copy_(one_hot_rows(p.v.shape[0], 2, D, p.cu_seqlens_kv, p.dtype))
    out, smax, ssum = swa.forward(*(x.to(dev) for x in (p.q, p.k, p.v)), p.cu_seqlens_q,
                                  p.cu_seqlens_kv, p.scale, p.pre_tokens, p.next_tokens,
                                  p.sparse_mode, drop_mask=mask.to(dev), keep_prob=0.5)
    torch.cuda.synchronize()
    out, smax, ssum = out.cpu().float(), smax.cpu(), ssum.cpu()
    rowc, _ = expected_counts(p, 2, 2, D, keep, 0.5)
    count, _ = expected_counts(p, 2, 2, D)
    n_allowed = count.sum(2)
    assert torch.equal(ssum[..., 0], n_allowed)
    assert not smax.any()
    expect = rowc / n_allowed.clamp_min(1)[..., None]
    assert torch.equal(out != 0, expect != 0), "mask pattern differs"
    assert ((out - expect).abs() <= expect.abs() * 2.0 ** -7 + 1e-6).all()
