"""swa_backward_noalloc, the backward for callers that cannot allocate device
memory, against swa_backward_ex on the same inputs (needs an MI355X).

Both run the same kernels, and the backward has no atomics, so the results
must agree bit for bit, for either input type.  Calls are
made back to back with different problems, a smaller one after a larger one
and the first again, because every call on a device shares the library's
fixed scratch (and skips re-uploading an unchanged schedule table).
"""
import pytest
import torch

import transformer_attention_tnd_amd as swa
import workloads
from parity_utils import note, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def prepare(p, dev, keep_prob=1.0):
    q, k, v, dy = (x.to(dev) for x in (p.q, p.k, p.v, p.dy))
    mask = None
    if keep_prob < 1.0:
        mask = workloads.make_drop_mask(p, keep_prob).to(dev)
    out, smax, ssum = swa.forward(q, k, v, p.cu_seqlens_q, p.cu_seqlens_kv, p.scale,
                                  p.pre_tokens, p.next_tokens, p.sparse_mode,
                                  drop_mask=mask, keep_prob=keep_prob)
    ref = swa.backward(q, k, v, dy, out, smax, ssum, p.cu_seqlens_q, p.cu_seqlens_kv, p.scale,
                       p.pre_tokens, p.next_tokens, p.sparse_mode, drop_mask=mask,
                       keep_prob=keep_prob)
    torch.cuda.synchronize()
    return (q, k, v, dy, out, smax, ssum, mask), [r.cpu() for r in ref]


def noalloc(p, args, keep_prob=1.0):
    q, k, v, dy, out, smax, ssum, mask = args
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for t in (dq, dk, dv):   # stale values must be overwritten
        t.fill_(7.0)
    swa.swa_backward_noalloc(q, k, v, dy, out, smax, ssum, p.cu_seqlens_q, p.cu_seqlens_kv,
                             p.scale, p.pre_tokens, p.next_tokens, p.sparse_mode, mask,
                             keep_prob, dq, dk, dv)
    torch.cuda.synchronize()
    return [dq.cpu(), dk.cpu(), dv.cpu()]


def assert_same(p, got, ref, label):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(g, r), f"{label} {name} differs from swa_backward_ex"


PROBLEMS = {
    "large_band": (dict(lengths_q=[4096, 3000, 77], num_heads=4, head_dim=128, sparse_mode=4,
                        pre_tokens=512, next_tokens=16), 1.0),
    "small_d64": (dict(lengths_q=[700, 129], num_heads=2, head_dim=64, sparse_mode=4,
                       pre_tokens=100, next_tokens=3, extra_tokens=9), 1.0),
    "gqa_dropout": (dict(lengths_q=[300, 513], lengths_kv=[500, 260], num_heads=4,
                         num_kv_heads=2, head_dim=128, sparse_mode=3, std=0.5), 0.8),
    "fp32_dense": (dict(lengths_q=[150, 66], num_heads=2, head_dim=64,
                        dtype=torch.float32), 1.0),
}


def test_noalloc_equals_workspace_backward(dev):
    prepared = {}
    # larger first, then smaller ones, then the first again (same schedule
    # table: the upload is skipped), twice
    for name in ["large_band", "small_d64", "gqa_dropout", "fp32_dense", "large_band",
                 "large_band", "small_d64"]:
        kw, keep = PROBLEMS[name]
        if name not in prepared:
            p = workloads.make_custom(name=name, **kw)
            prepared[name] = (p,) + prepare(p, dev, keep)
        p, args, ref = prepared[name]
        note(f"[noalloc] {name} cu_q={p.cu_seqlens_q}")
        assert_same(p, noalloc(p, args, keep), ref, name)


def test_noalloc_rejects_problems_beyond_its_scratch(dev):
    """A backward workspace above the fixed scratch (32 MiB) is refused before
    anything is enqueued, and the outputs are left untouched."""
    T, N, D = 1 << 20, 8, 64   # D and lse2 alone: 2 * 4 * 2^23 bytes = 64 MiB
    need = swa.swa_backward_workspace_size(1, T, T, N, D, swa.DTYPE_BF16)
    assert need > 32 << 20
    x = torch.zeros(T, N, D, dtype=torch.bfloat16, device=dev)
    st = torch.zeros(T, N, 8, dtype=torch.float32, device=dev)
    dq = torch.full_like(x, 3.0)
    with pytest.raises(ValueError, match="fixed 33554432 bytes"):
        swa.swa_backward_noalloc(x, x, x, x, x, st, st, [T], [T], 0.125, 64, 0, 4, None, 1.0,
                                 dq, dq, dq)
    torch.cuda.synchronize()
    assert bool((dq == 3.0).all())
