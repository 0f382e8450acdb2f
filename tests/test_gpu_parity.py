"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Small problems (the two small workloads and hand-made varlen/band cases that
span several tiles and ragged tails) are compared element by element.  The
large workloads run in full on the GPU, in the launch configuration the
benchmark times, and are compared element by element too, streamed one
(sequence, key/value head) at a time through the oracle, after a fast
pre-check on sampled rows and keys and on invariants that hold at any size.
"""
import math

import pytest
import torch

import oracle
import transformer_attention_tnd_amd as swa
import workloads
from parity_utils import (StreamedErrors, assert_close, assert_stats, compare_full,
                          compare_streamed, note, require_gpu, run_hip, run_oracle)

pytestmark = pytest.mark.gpu
INT_MAX = 2147483647


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


# ------------------------------------------------------------ small, full parity

@pytest.mark.parametrize("name", ["dense_fp32_b1_n2_s128_d64", "dense_bf16_b1_n8_s512_d64"])
def test_small_workloads_full_parity(dev, name):
    p = workloads.make_problem(name)
    note(f"[parity] {name}")
    g = run_hip(p, dev)
    o = run_oracle(p)
    compare_full(p, g, o)


CUSTOM = {
    "bf16_d128_band_ragged": dict(lengths_q=[1, 130, 257, 700], num_heads=3, head_dim=128,
                                  sparse_mode=4, pre_tokens=64, next_tokens=0),
    "bf16_d128_dense_varlen": dict(lengths_q=[200, 513], num_heads=2, head_dim=128),
    "bf16_d64_band_both_sides": dict(lengths_q=[333, 129], num_heads=2, head_dim=64,
                                     sparse_mode=4, pre_tokens=100, next_tokens=37),
    "bf16_d128_dense_unequal_kv": dict(lengths_q=[77, 190], lengths_kv=[50, 260],
                                       num_heads=2, head_dim=128),
    "fp32_d128_band": dict(lengths_q=[300, 45], num_heads=2, head_dim=128, sparse_mode=4,
                           pre_tokens=90, next_tokens=20, dtype=torch.float32),
    "fp32_d64_dense_unequal_kv": dict(lengths_q=[77, 190], lengths_kv=[50, 260], num_heads=2,
                                      head_dim=64, dtype=torch.float32),
    "bf16_trailing_and_extra_tokens": dict(lengths_q=[100, 150], num_heads=2, head_dim=128,
                                           sparse_mode=4, pre_tokens=40, next_tokens=8,
                                           trailing=2, extra_tokens=5),
    "bf16_zero_length_sequences": dict(lengths_q=[0, 64, 0, 100], num_heads=2, head_dim=64),
    # a sequence with query rows but no keys: its rows attend nothing (out = 0, dq = 0)
    "bf16_d128_no_keys_for_a_sequence": dict(lengths_q=[140, 100], lengths_kv=[0, 120],
                                             num_heads=2, head_dim=128),
    "bf16_empty_rows_negative_next": dict(lengths_q=[150, 90], num_heads=2, head_dim=128,
                                          sparse_mode=4, pre_tokens=70, next_tokens=-5),
    "bf16_narrow_band_negative_pre": dict(lengths_q=[260], num_heads=1, head_dim=128,
                                          sparse_mode=4, pre_tokens=-3, next_tokens=9),
    "bf16_band_wider_than_sequence": dict(lengths_q=[190, 66], num_heads=2, head_dim=128,
                                          sparse_mode=4, pre_tokens=65536, next_tokens=65536),
    "bf16_single_token": dict(lengths_q=[1], num_heads=4, head_dim=128),
    # causal modes 2 (j <= i) and 3 (j - i <= Skv - Sq), with Sq != Skv per batch
    "bf16_d128_left_up_causal": dict(lengths_q=[300, 77, 513], lengths_kv=[700, 77, 260],
                                     num_heads=2, head_dim=128, sparse_mode=2),
    "bf16_d128_right_down_causal": dict(lengths_q=[300, 77, 513], lengths_kv=[700, 77, 260],
                                        num_heads=2, head_dim=128, sparse_mode=3),
    "bf16_d64_causal_square": dict(lengths_q=[390, 129], num_heads=3, head_dim=64,
                                   sparse_mode=2),
    "bf16_d64_right_down_short_kv": dict(lengths_q=[400, 5], lengths_kv=[130, 70], num_heads=2,
                                         head_dim=64, sparse_mode=3),
    "fp32_d128_right_down_causal": dict(lengths_q=[150, 260], lengths_kv=[333, 90],
                                        num_heads=2, head_dim=128, sparse_mode=3,
                                        dtype=torch.float32),
    "fp32_d64_left_up_causal": dict(lengths_q=[150, 260], lengths_kv=[333, 90], num_heads=2,
                                    head_dim=64, sparse_mode=2, dtype=torch.float32),
    # grouped key/value heads (query head n reads key/value head n // G); dk / dv
    # sum G heads, so the bf16 cases draw std 0.5 (as the 32-head varlen
    # workload does) to keep them near unit scale, where the absolute bf16
    # tolerance is above the output's own rounding
    "bf16_d128_gqa4_band": dict(lengths_q=[300, 77, 513], num_heads=8, num_kv_heads=2,
                                head_dim=128, sparse_mode=4, pre_tokens=100, next_tokens=0,
                                std=0.5),
    "bf16_d64_gqa3_dense_unequal_kv": dict(lengths_q=[77, 190], lengths_kv=[50, 260],
                                           num_heads=6, num_kv_heads=2, head_dim=64),
    "bf16_d128_mqa_causal": dict(lengths_q=[257, 130], lengths_kv=[400, 100], num_heads=4,
                                 num_kv_heads=1, head_dim=128, sparse_mode=3, std=0.5),
    "fp32_d128_gqa2_band": dict(lengths_q=[300, 45], num_heads=4, num_kv_heads=2,
                                head_dim=128, sparse_mode=4, pre_tokens=90, next_tokens=20,
                                dtype=torch.float32),
    "fp32_d64_gqa4_dense": dict(lengths_q=[150, 66], num_heads=4, num_kv_heads=1,
                                head_dim=64, dtype=torch.float32),
}


@pytest.mark.parametrize("case", sorted(CUSTOM))
def test_custom_cases_full_parity(dev, case):
    kw = dict(CUSTOM[case])
    p = workloads.make_custom(name=case, **kw)
    note(f"[parity] {case} cu_q={p.cu_seqlens_q} cu_kv={p.cu_seqlens_kv}")
    g = run_hip(p, dev)
    o = run_oracle(p, chunk=None)
    compare_full(p, g, o)
    # tokens past the last participating end: zeros / -inf / 0
    end = max(p.cu_seqlens_q)
    if end < p.q.shape[0]:
        assert g["out"][end:].abs().max() == 0 and g["dq"][end:].abs().max() == 0
        assert torch.isinf(g["smax"][end:]).all() and (g["ssum"][end:] == 0).all()
        endk = max(p.cu_seqlens_kv)
        assert g["dk"][endk:].abs().max() == 0 and g["dv"][endk:].abs().max() == 0


DROPOUT = {
    "bf16_d128_band_dropout": (dict(lengths_q=[1, 130, 257, 700], num_heads=3, head_dim=128,
                                    sparse_mode=4, pre_tokens=64, next_tokens=5), 0.8),
    "bf16_d64_dense_unequal_kv_dropout": (dict(lengths_q=[77, 190], lengths_kv=[50, 260],
                                               num_heads=2, head_dim=64), 0.6),
    "bf16_d128_gqa_causal_dropout": (dict(lengths_q=[257, 130], lengths_kv=[300, 100],
                                          num_heads=4, num_kv_heads=2, head_dim=128,
                                          sparse_mode=3, std=0.5), 0.9),
    "bf16_d64_gqa_band_dropout": (dict(lengths_q=[200, 333], num_heads=6, num_kv_heads=2,
                                       head_dim=64, sparse_mode=4, pre_tokens=100,
                                       next_tokens=20), 0.75),
    "fp32_d128_band_dropout": (dict(lengths_q=[300, 45], num_heads=2, head_dim=128,
                                    sparse_mode=4, pre_tokens=90, next_tokens=20,
                                    dtype=torch.float32), 0.7),
    "fp32_d64_dense_dropout": (dict(lengths_q=[150, 66], lengths_kv=[90, 130], num_heads=2,
                                    head_dim=64, dtype=torch.float32), 0.5),
}


@pytest.mark.parametrize("case", sorted(DROPOUT))
def test_dropout_cases_full_parity(dev, case):
    """Dropout with a seeded caller mask (packed keep bits) against the oracle."""
    kw, keep_prob = DROPOUT[case]
    p = workloads.make_custom(name=case, **kw)
    mask = workloads.make_drop_mask(p, keep_prob)
    note(f"[parity] {case} keep_prob={keep_prob} mask bytes={mask.numel()}")
    g = run_hip(p, dev, drop_mask=mask, keep_prob=keep_prob)
    o = run_oracle(p, chunk=None, drop_mask=mask, keep_prob=keep_prob)
    compare_full(p, g, o)


@pytest.mark.parametrize("D", [64, 128])
def test_dropout_keep_all_equals_no_dropout(dev, D):
    """An all-ones mask with keep_prob 1 reproduces the call without dropout:
    the forward bit for bit (the same tiles and order; each probability is
    multiplied by 1 and masked by all ones), the backward up to rounding
    (without dropout its dP chains start from -D, dS = P (dP - D) in one
    multiply, where with dropout D is subtracted after the chain)."""
    p = workloads.make_custom([300, 77, 700], num_heads=2, head_dim=D, sparse_mode=4,
                              pre_tokens=300, next_tokens=0)
    mask = workloads.make_drop_mask(p, 1.0)
    a = run_hip(p, dev)
    b = run_hip(p, dev, drop_mask=mask, keep_prob=1.0)
    for n in ("out", "smax", "ssum"):
        assert torch.equal(a[n], b[n]), n
    for n in ("dq", "dk", "dv"):
        assert (a[n].float() - b[n].float()).abs().max() <= 1e-2, n
    assert (a["smax"] - b["smax"]).abs().max() <= 1e-5
    assert ((a["ssum"] - b["ssum"]).abs() / b["ssum"].abs().clamp_min(1e-30)).max() <= 1e-4


# ------------------------------------------------------------ exact cases

def test_query_zero_counts_are_exact(dev):
    """q = 0 (fp32): every score is 0, so softmax_max = 0 and softmax_sum = the
    number of allowed keys exactly; with V_j = e_(j mod D), out[i, c] is the
    fraction of allowed keys j = c (mod D): the mask pattern shows bit-exactly."""
    lengths = [300, 77, 513]
    D = 64
    pre, nxt = 70, 9
    p = workloads.make_custom(lengths, num_heads=1, head_dim=D, dtype=torch.float32,
                              sparse_mode=4, pre_tokens=pre, next_tokens=nxt)
    p.q.zero_()
    T = p.k.shape[0]
    p.v.zero_()
    for s0, L in oracle.sequences(p.cu_seqlens_kv):
        for j in range(L):
            p.v[s0 + j, 0, j % D] = 1.0
    g = run_hip(p, dev, with_backward=False)
    assert torch.equal(g["smax"], torch.zeros_like(g["smax"]))
    for s0, L in oracle.sequences(p.cu_seqlens_q):
        M = oracle.allowed_mask(torch.arange(L), torch.arange(L), 4, pre, nxt)
        counts = M.sum(1)
        assert torch.equal(g["ssum"][s0:s0 + L, 0, 0], counts.float())
        per_c = torch.zeros(L, D)
        for c in range(D):
            per_c[:, c] = M[:, c::D].sum(1).float()
        expect = per_c / counts[:, None].float()
        out = g["out"][s0:s0 + L, 0]
        assert torch.equal(out != 0, expect != 0), "mask pattern differs"
        assert (out - expect).abs().max() <= 1e-6


ZERO_Q_BF16 = {
    "d128_band": dict(lengths_q=[300, 77, 513], head_dim=128, sparse_mode=4, pre=70, nxt=9),
    "d128_wide_band": dict(lengths_q=[700, 129], head_dim=128, sparse_mode=4, pre=200, nxt=130),
    "d64_left_up_causal": dict(lengths_q=[300, 513], lengths_kv=[700, 260], head_dim=64,
                               sparse_mode=2, pre=0, nxt=0),
    "d128_right_down_causal": dict(lengths_q=[513, 77], lengths_kv=[260, 300], head_dim=128,
                                   sparse_mode=3, pre=0, nxt=0),
}


@pytest.mark.parametrize("case", sorted(ZERO_Q_BF16))
def test_query_zero_counts_are_exact_bf16(dev, case):
    """The same count check on the bf16 forward (128-key tiles, each visited
    or mask-free by the classification of its two scheduler tiles): with q = 0
    every allowed probability is exactly 1, so softmax_sum equals the number of
    allowed keys and softmax_max is 0, bit for bit; out (the fraction of
    allowed keys j = c mod D) is zero exactly where no allowed key falls in
    class c, and otherwise within the bf16 rounding of the fraction."""
    kw = dict(ZERO_Q_BF16[case])
    D, mode, pre, nxt = kw.pop("head_dim"), kw.pop("sparse_mode"), kw.pop("pre"), kw.pop("nxt")
    p = workloads.make_custom(kw["lengths_q"], kw.get("lengths_kv"), num_heads=1, head_dim=D,
                              dtype=torch.bfloat16, sparse_mode=mode, pre_tokens=pre,
                              next_tokens=nxt)
    p.q.zero_()
    p.v.zero_()
    for s0, L in oracle.sequences(p.cu_seqlens_kv):
        for j in range(L):
            p.v[s0 + j, 0, j % D] = 1.0
    note(f"[zero-q bf16] {case} cu_q={p.cu_seqlens_q} cu_kv={p.cu_seqlens_kv}")
    g = run_hip(p, dev, with_backward=False)
    for (q0, Lq), (_, Lk) in zip(oracle.sequences(p.cu_seqlens_q), oracle.sequences(p.cu_seqlens_kv)):
        M = oracle.allowed_mask(torch.arange(Lq), torch.arange(Lk), mode, pre, nxt, Lq, Lk)
        counts = M.sum(1)
        assert torch.equal(g["ssum"][q0:q0 + Lq, 0, 0], counts.float()), "row counts differ"
        has = counts > 0
        assert torch.equal(g["smax"][q0:q0 + Lq, 0, 0][has], torch.zeros(int(has.sum())))
        per_c = torch.zeros(Lq, D)
        for c in range(D):
            per_c[:, c] = M[:, c::D].sum(1).float()
        expect = per_c / counts.clamp_min(1)[:, None].float()
        out = g["out"][q0:q0 + Lq, 0].float()
        assert torch.equal(out != 0, expect != 0), "mask pattern differs"
        assert ((out - expect).abs() <= expect.abs() * 2.0 ** -8 + 1e-7).all()


def test_forward_example_constant_inputs(dev):
    """VarLenScore API doc call example (T=256, N=1, D=128, scale 0.088388,
    pre/next 65536, mode 0) with q = k = v = 1: out = 1, softmax_max =
    128 * 0.088388, softmax_sum = 256."""
    x = torch.ones(256, 1, 128, dtype=torch.float32, device=dev)
    out, smax, ssum = swa.forward(x, x, x, [256], [256], 0.088388, 65536, 65536, 0)
    torch.cuda.synchronize()
    assert (out - 1).abs().max().item() <= 1e-6
    assert (smax - 128 * 0.088388).abs().max().item() <= 1e-5
    assert (ssum == 256).all()


def test_backward_example_uses_given_statistics(dev):
    """UnpaddingScoreGradV2 explainer call example: all-ones q/k/v/dy/out with
    softmax_max = softmax_sum = 3.0: dq = dk = 0 and dv = 256 exp(11.313664 - 3)/3."""
    x = torch.ones(256, 1, 128, dtype=torch.float32, device=dev)
    st = torch.full((256, 1, 8), 3.0, dtype=torch.float32, device=dev)
    dq, dk, dv = swa.backward(x, x, x, x, x, st, st, [256], [256], 0.088388, 65536, 65536, 0)
    torch.cuda.synchronize()
    assert dq.abs().max().item() == 0 and dk.abs().max().item() == 0
    expect = 256 * math.exp(128 * 0.088388 - 3) / 3
    assert ((dv - expect).abs() / expect).max().item() <= 1e-5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gqa_equals_replicated_heads(dev, dtype):
    """Grouped heads give the same out / dq as the ordinary multi-head call
    on K / V repeated per query head, and dk / dv equal to the group sums of
    that call's dk / dv (bf16: exact for out and dq, whose kernels read the
    same values; dk / dv differ only in summation order)."""
    G = 4
    p = workloads.make_custom([300, 77, 513], num_heads=8, num_kv_heads=2, head_dim=128,
                              dtype=dtype, sparse_mode=4, pre_tokens=100, next_tokens=3)
    g = run_hip(p, dev)
    rep = workloads.Problem(p.q, p.k.repeat_interleave(G, 1).contiguous(),
                            p.v.repeat_interleave(G, 1).contiguous(), p.dy, p.cu_seqlens_q,
                            p.cu_seqlens_kv, p.scale, p.pre_tokens, p.next_tokens,
                            p.sparse_mode)
    r = run_hip(rep, dev)
    assert torch.equal(g["out"], r["out"]) and torch.equal(g["smax"], r["smax"])
    if dtype == torch.bfloat16:
        assert torch.equal(g["dq"], r["dq"])
    for n in ("dk", "dv"):
        per_head = r[n].double().view(r[n].shape[0], 2, G, -1)
        summed = per_head.sum(2)
        err = (g[n].double() - summed).abs()
        if dtype == torch.bfloat16:
            # each side rounds to bf16 (unit roundoff 2^-8): G roundings of the
            # per-head values against one of the group sum, plus fp32 order
            bound = 2.0 ** -8 * (per_head.abs().sum(2) + summed.abs()) + 1e-5
            assert (err <= bound).all(), f"{n}: {float((err - bound).max()):.3e} over the bound"
        else:
            assert float(err.max()) <= 1e-4 * float(summed.abs().max())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_varlen_equals_separate_calls(dev, dtype):
    """Tiles align to each sequence's start, so a varlen call reproduces
    separate per-sequence calls bit for bit: out, statistics, dq, dk, dv (the
    two-pass backward has no atomics, for either input type)."""
    lengths = [130, 64, 257, 1]
    p = workloads.make_custom(lengths, num_heads=2, head_dim=128, sparse_mode=4,
                              pre_tokens=50, next_tokens=20, dtype=dtype)
    g = run_hip(p, dev)
    exact = ("out", "smax", "ssum", "dq", "dk", "dv")
    for s0, L in oracle.sequences(p.cu_seqlens_q):
        sl = slice(s0, s0 + L)
        sub = workloads.Problem(p.q[sl].clone(), p.k[sl].clone(), p.v[sl].clone(),
                                p.dy[sl].clone(), [L], [L], p.scale, p.pre_tokens,
                                p.next_tokens, p.sparse_mode)
        gs = run_hip(sub, dev)
        for n in exact:
            assert torch.equal(gs[n], g[n][sl]), n


def test_schedule_cache_on_and_off_agree(dev):
    """Schedules from the library's device cache and schedules uploaded into
    the workspace on every call give identical results (same tables, two
    places); problems that alternate keep hitting their own cache entries."""
    probs = [workloads.make_custom([700, 1500, 300], num_heads=4, head_dim=128, sparse_mode=4,
                                   pre_tokens=300, next_tokens=40),
             workloads.make_custom([333, 129], num_heads=2, head_dim=64, sparse_mode=2,
                                   lengths_kv=[400, 129])]
    try:
        swa.swa_schedule_cache_enable(False)
        off = [run_hip(p, dev) for p in probs]
        swa.swa_schedule_cache_enable(True)
        on = [run_hip(p, dev) for p in probs + probs]
    finally:
        swa.swa_schedule_cache_enable(True)
    for i, r in enumerate(on):
        for n in ("out", "smax", "ssum", "dq", "dk", "dv"):
            assert torch.equal(r[n], off[i % 2][n]), (i, n)


def test_concurrent_threads_and_streams(dev):
    """Host threads calling at once, each on a stream of its own (shared
    schedule cache entries, the pinned staging ring, per-thread error text),
    get the bits of the same calls made one at a time."""
    import threading
    probs = [workloads.make_custom([700, 1500, 300], num_heads=4, head_dim=128, sparse_mode=4,
                                   pre_tokens=300, next_tokens=40),
             workloads.make_custom([333, 129], num_heads=2, head_dim=64, sparse_mode=2,
                                   lengths_kv=[400, 129]),
             workloads.make_custom([520, 77], num_heads=2, head_dim=128, dtype=torch.float32)]
    ref = [run_hip(p, dev) for p in probs]
    n_threads, reps = 6, 3
    got = [[None] * reps for _ in range(n_threads)]
    errors = []
    bad = probs[0]

    def work(i):
        try:
            stream = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(stream):
                for r in range(reps):
                    if i % 2 == 0:  # a rejected call between the good ones: its own error text
                        q = bad.q.to(dev)
                        try:
                            swa.forward(q, q, q, bad.cu_seqlens_q, bad.cu_seqlens_kv, bad.scale,
                                        bad.pre_tokens, bad.next_tokens, 1)
                            errors.append((i, "sparse_mode 1 accepted"))
                        except ValueError as e:  # (invalid arguments raise ValueError)
                            if "sparse_mode" not in str(e):
                                errors.append((i, f"error text of another call: {e}"))
                    got[i][r] = run_hip(probs[i % len(probs)], dev)
        except BaseException as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i in range(n_threads):
        for r in range(reps):
            for n in ("out", "smax", "ssum", "dq", "dk", "dv"):
                assert torch.equal(got[i][r][n], ref[i % len(probs)][n]), (i, r, n)


def test_concurrent_calls_with_cache_eviction(dev):
    """More distinct problems than the schedule cache holds (64), called from
    four threads on their own streams: entries are evicted while other calls
    use theirs, and every result keeps the bits of the uncached call."""
    import threading
    probs = [workloads.make_custom([60 + 7 * i, 33], num_heads=2, head_dim=64, sparse_mode=4,
                                   pre_tokens=40, next_tokens=9) for i in range(72)]
    try:
        swa.swa_schedule_cache_enable(False)
        ref = [run_hip(p, dev) for p in probs]
    finally:
        swa.swa_schedule_cache_enable(True)
    n_threads = 4
    got = {}
    errors = []

    def work(i):
        try:
            stream = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(stream):
                for rep in range(2):
                    for j in range(i, len(probs), n_threads):
                        got[(j, rep)] = run_hip(probs[j], dev)
        except BaseException as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    assert len(got) == 2 * len(probs)
    for (j, rep), r in got.items():
        for n in ("out", "smax", "ssum", "dq", "dk", "dv"):
            assert torch.equal(r[n], ref[j][n]), (j, rep, n)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_is_deterministic(dev, dtype):
    """The backward uses no atomics: two calls give identical bits."""
    p = workloads.make_custom([700, 1500, 300], num_heads=4, head_dim=128, sparse_mode=4,
                              pre_tokens=300, next_tokens=40, dtype=dtype)
    g1 = run_hip(p, dev)
    g2 = run_hip(p, dev)
    for n in ("dq", "dk", "dv"):
        assert torch.equal(g1[n], g2[n]), n


# ------------------------------------------------------------ large workloads

def sampled_check(p, g, samples):
    """Compare GPU results with the oracle on (batch, head, first row/key) samples."""
    dt = p.dtype
    seqs = oracle.sequences(p.cu_seqlens_q)
    errs = {"out": [], "dq": [], "dk": [], "dv": []}
    smax_g, ssum_g, smax_o, ssum_o = [], [], [], []
    G = p.q.shape[1] // p.k.shape[1]  # query heads per key/value head
    for b, n, r0, width in samples:
        s0, L = seqs[b]
        r0 = min(r0, L - width)
        Q, dY = (x[s0:s0 + L, n] for x in (p.q, p.dy))
        K, V = (x[s0:s0 + L, n // G] for x in (p.k, p.v))
        rows = list(range(r0, r0 + width))
        O, m, l = oracle.forward_rows(Q, K, V, rows, p.scale, p.sparse_mode, p.pre_tokens,
                                      p.next_tokens)
        dq = oracle.backward_rows(Q, K, V, dY, rows, p.scale, p.sparse_mode, p.pre_tokens,
                                  p.next_tokens)
        # dk / dv of key/value head n // G sum over the query heads of its group
        dk, dv = 0, 0
        for nq in range((n // G) * G, (n // G + 1) * G):
            a_, b_ = oracle.backward_keys(p.q[s0:s0 + L, nq], K, V, p.dy[s0:s0 + L, nq], r0,
                                          r0 + width, p.scale, p.sparse_mode, p.pre_tokens,
                                          p.next_tokens)
            dk, dv = dk + a_, dv + b_
        t = slice(s0 + r0, s0 + r0 + width)
        errs["out"].append((g["out"][t, n], O))
        errs["dq"].append((g["dq"][t, n], dq))
        errs["dk"].append((g["dk"][t, n // G], dk))
        errs["dv"].append((g["dv"][t, n // G], dv))
        smax_g.append(g["smax"][t, n])
        ssum_g.append(g["ssum"][t, n])
        smax_o.append(m)
        ssum_o.append(l)
    for name, pairs in errs.items():
        assert_close(name, torch.cat([a.flatten() for a, _ in pairs]),
                     torch.cat([b.flatten() for _, b in pairs]), dt)
    assert_stats(torch.cat(smax_g), torch.cat(ssum_g), torch.cat(smax_o), torch.cat(ssum_o), dt)


def invariants_check(p, g):
    """sum_j dV_j = sum_i dY_i and sum_j dK_j = 0 per (sequence, head)."""
    for s0, L in oracle.sequences(p.cu_seqlens_q):
        dv_sum = g["dv"][s0:s0 + L].double().sum(0)
        nkv = dv_sum.shape[0]
        dy_sum = p.dy[s0:s0 + L].double().sum(0).view(nkv, -1, dv_sum.shape[1]).sum(1)
        dk_sum = g["dk"][s0:s0 + L].double().sum(0)
        scale_dv = float(g["dv"][s0:s0 + L].double().abs().sum(0).max())
        scale_dk = float(g["dk"][s0:s0 + L].double().abs().sum(0).max())
        e1 = float((dv_sum - dy_sum).abs().max()) / scale_dv
        e2 = float(dk_sum.abs().max()) / scale_dk
        note(f"  invariants seq@{s0}: |sum dV - sum dY|/sum|dV| = {e1:.2e}, "
             f"|sum dK|/sum|dK| = {e2:.2e}")
        assert e1 <= 1e-2 and e2 <= 1e-2


def test_maximum_sizes(dev):
    """The largest sizes the interface takes (explainer 6.3: T up to 1M tokens,
    N up to 256 heads): one 1,048,576-token sequence with a narrow band
    (every row and key against the oracle), and 256 heads (full parity).
    Exercises the 64-bit offsets of every kernel."""
    T = 1 << 20
    p = workloads.make_custom([T], num_heads=1, head_dim=128, sparse_mode=4, pre_tokens=192,
                              next_tokens=64, name="max_tokens")
    note(f"[parity] max_tokens T={T}")
    g = run_hip(p, dev)
    for key in ("out", "dq", "dk", "dv"):
        assert torch.isfinite(g[key].float()).all(), key
    acc = StreamedErrors(p.dtype)
    compare_streamed(p, g, range(p.k.shape[1]), acc)
    acc.check("max_tokens whole tensors")
    del g
    p = workloads.make_custom([300, 77], num_heads=256, head_dim=64, name="max_heads")
    note("[parity] max_heads N=256")
    compare_full(p, run_hip(p, dev), run_oracle(p, chunk=None))


# Each large workload runs once on the GPU, in the launch configuration the
# benchmark times (part 0: sampled rows and keys plus invariants, a fast
# pre-check), then every row and key of every head is compared with the
# oracle, a group of key/value heads per part; the last part checks the
# whole-tensor figures (max and mean |g - o| per output tensor over all
# elements, the worst statistic errors).
LARGE = {
    "varlen_bf16_n16_d128_8seq_256to4096":
        ([(0, 0, 0, 64), (3, 7, 1000, 64), (7, 15, 10**9, 48)], 2),
    "swa_bf16_b1_n16_s16384_d128_pre2048_next0":
        ([(0, 0, 0, 64), (0, 5, 2000, 96), (0, 11, 9000, 64), (0, 15, 10**9, 64)], 2),
    "varlen_swa_bf16_n32_d128_4seq_16kto32k_pre4096_next512":
        ([(0, 0, 0, 64), (1, 13, 4500, 64), (2, 31, 20000, 64), (3, 20, 10**9, 64)], 8),
    # causal: keys near the end (few rows attend them, so the oracle's
    # key-side check stays cheap); the row-side check covers each sample too
    "causal_bf16_b1_n16_s16384_d128":
        ([(0, 0, 16000, 64), (0, 9, 15000, 32), (0, 15, 10**9, 32)], 4),
    "gqa_swa_bf16_b1_n16kv4_s16384_d128_pre2048_next0":
        ([(0, 0, 0, 64), (0, 6, 5000, 64), (0, 15, 10**9, 64)], 2),
    "swa_fp32_b1_n16_s16384_d128_pre2048_next0":
        ([(0, 0, 0, 64), (0, 9, 7000, 64), (0, 15, 10**9, 64)], 2),
}
LARGE_CASES = [(n, part) for n, (_, parts) in LARGE.items() for part in range(parts + 1)]
_large = {}


def large_state(dev, name):
    """(problem, GPU results, per-part error accumulators) of one workload;
    only the most recent workload is kept."""
    if name not in _large:
        _large.clear()
        p = workloads.make_problem(name)
        note(f"[parity] {name} T={p.q.shape[0]} cu={p.cu_seqlens_q}")
        g = run_hip(p, dev)
        for key in ("out", "dq", "dk", "dv"):
            assert torch.isfinite(g[key].float()).all(), key
        _large[name] = (p, g, {})
    return _large[name]


@pytest.mark.parametrize("name,part", LARGE_CASES, ids=[f"{n}-{i}" for n, i in LARGE_CASES])
def test_large_workloads_parity(dev, name, part):
    samples, parts = LARGE[name]
    p, g, accs = large_state(dev, name)
    if part == 0:
        sampled_check(p, g, samples)
        invariants_check(p, g)
        return
    nkv = p.k.shape[1]
    heads = range((part - 1) * nkv // parts, part * nkv // parts)
    acc = StreamedErrors(p.dtype)
    compare_streamed(p, g, heads, acc)
    acc.check(f"key/value heads {heads.start}..{heads.stop - 1}:")
    accs[part] = acc
    if part == parts:
        assert sorted(accs) == list(range(1, parts + 1)), "a part of the workload was not run"
        whole = StreamedErrors(p.dtype)
        for a in accs.values():
            whole.merge(a)
        whole.check(f"{name} whole tensors:")
