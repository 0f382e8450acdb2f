"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle,
compare with the tolerances of the method's precision contract.

Tolerances (per output tensor):
  fp32 inputs : max |g - o| / max |o| <= 1e-4 (out, dq, dk, dv); the
                statistics use the same relative bound.
  bf16 inputs : max |g - o| <= 2e-2 and mean |g - o| <= 5e-3 (out, dq, dk, dv,
                fp32 accumulation); softmax_max abs <= 1e-3 and softmax_sum
                rel <= 1e-3.
"""
from __future__ import annotations

import sys

import torch

import oracle
import transformer_attention_tnd_amd as swa

TOL_FP32_REL = 1e-4
# fp32 relative errors are taken against max(max |reference|, this floor): a
# tensor that vanishes in exact arithmetic (dq of a row that sees one key:
# dS = P (dP - D) with dP = D) is left with the rounding of its O(1) terms,
# ~1e-7, which is no relative error of the tensor's own size
TOL_FP32_FLOOR = 1e-2
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 5e-3
TOL_STAT_MAX_ABS = 1e-3
TOL_STAT_SUM_REL = 1e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    swa.load_library()
    return torch.device("cuda:0")


def run_hip(p, device, with_backward=True, drop_mask=None, keep_prob=1.0):
    """Forward (+ backward) of problem p through the C ABI; host copies.
    ``drop_mask`` (host uint8, packed keep bits) applies dropout."""
    q, k, v, dy = (x.to(device) for x in (p.q, p.k, p.v, p.dy))
    mask = None if drop_mask is None else drop_mask.to(device)
    out, smax, ssum = swa.forward(q, k, v, p.cu_seqlens_q, p.cu_seqlens_kv, p.scale,
                                  p.pre_tokens, p.next_tokens, p.sparse_mode,
                                  drop_mask=mask, keep_prob=keep_prob)
    res = {"out": out, "smax": smax, "ssum": ssum}
    if with_backward:
        dq, dk, dv = swa.backward(q, k, v, dy, out, smax, ssum, p.cu_seqlens_q,
                                  p.cu_seqlens_kv, p.scale, p.pre_tokens, p.next_tokens,
                                  p.sparse_mode, drop_mask=mask, keep_prob=keep_prob)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k_: v_.cpu() for k_, v_ in res.items()}


def run_oracle(p, chunk=256, drop_mask=None, keep_prob=1.0):
    kw = dict(drop_mask=drop_mask, keep_prob=keep_prob)
    out, sm, ss = oracle.forward(p.q, p.k, p.v, p.cu_seqlens_q, p.cu_seqlens_kv, p.scale,
                                 p.pre_tokens, p.next_tokens, p.sparse_mode, chunk=chunk, **kw)
    dq, dk, dv = oracle.backward(p.q, p.k, p.v, p.dy, out, sm, ss, p.cu_seqlens_q,
                                 p.cu_seqlens_kv, p.scale, p.pre_tokens, p.next_tokens,
                                 p.sparse_mode, chunk=chunk, **kw)
    return {"out": out, "smax": sm, "ssum": ss, "dq": dq, "dk": dk, "dv": dv}


def err_stats(g, o):
    g = g.double()
    o = o.double()
    d = (g - o).abs()
    return float(d.max()), float(d.mean()), float(o.abs().max())


def assert_close(name, g, o, dtype):
    mx, mean, ref = err_stats(g, o)
    if dtype == torch.float32:
        rel = mx / max(ref, TOL_FP32_FLOOR)
        note(f"  {name}: max_abs={mx:.3e} max_rel={rel:.3e} (|ref|max={ref:.3e})")
        assert rel <= TOL_FP32_REL, f"{name}: max relative error {rel:.3e} > {TOL_FP32_REL}"
    else:
        note(f"  {name}: max_abs={mx:.3e} mean_abs={mean:.3e} (|ref|max={ref:.3e})")
        assert mx <= TOL_BF16_MAX, f"{name}: max abs error {mx:.3e} > {TOL_BF16_MAX}"
        assert mean <= TOL_BF16_MEAN, f"{name}: mean abs error {mean:.3e} > {TOL_BF16_MEAN}"


def assert_stats(smax_g, ssum_g, smax_o, ssum_o, dtype, quiet=False):
    """Statistics [.., 8] from the GPU against oracle [..]; all 8 copies equal."""
    assert torch.equal(smax_g, smax_g[..., :1].expand_as(smax_g)), "softmax_max copies differ"
    assert torch.equal(ssum_g, ssum_g[..., :1].expand_as(ssum_g)), "softmax_sum copies differ"
    gm, gs = smax_g[..., 0].double(), ssum_g[..., 0].double()
    om, os_ = smax_o.double(), ssum_o.double()
    inf_g, inf_o = torch.isinf(gm), torch.isinf(om)
    assert torch.equal(inf_g, inf_o), "empty-row pattern of softmax_max differs"
    assert torch.equal(gs == 0, os_ == 0), "empty-row pattern of softmax_sum differs"
    fin = ~inf_o
    if fin.any():
        dm = float((gm[fin] - om[fin]).abs().max())
        ds = float(((gs[fin] - os_[fin]).abs() / os_[fin].abs()).max())
        if not quiet:
            note(f"  softmax_max: max_abs={dm:.3e}  softmax_sum: max_rel={ds:.3e}")
        if dtype == torch.float32:
            ref = float(om[fin].abs().max())
            assert dm <= TOL_FP32_REL * max(ref, 1.0)
            assert ds <= TOL_FP32_REL
        else:
            assert dm <= TOL_STAT_MAX_ABS
            assert ds <= TOL_STAT_SUM_REL


def compare_full(p, g, o):
    dt = p.dtype
    assert_close("out", g["out"], o["out"], dt)
    assert_stats(g["smax"], g["ssum"], o["smax"], o["ssum"], dt)
    for n in ("dq", "dk", "dv"):
        if n in g:
            assert_close(n, g[n], o[n], dt)


class StreamedErrors:
    """Running whole-tensor error figures, fed one (sequence, head group) at a
    time: max |g - o|, sum |g - o|, element count and max |o| per tensor, and
    the worst statistic errors.  Checks against the same tolerances as
    ``assert_close`` / ``assert_stats``."""

    def __init__(self, dtype):
        self.dtype = dtype
        self.t = {}
        self.stat_max_abs = 0.0
        self.stat_sum_rel = 0.0

    def add(self, name, g, o):
        d = (g.double() - o.double()).abs()
        mx, s, n, ref = self.t.get(name, (0.0, 0.0, 0, 0.0))
        self.t[name] = (max(mx, float(d.max()) if d.numel() else 0.0), s + float(d.sum()),
                        n + d.numel(), max(ref, float(o.abs().max()) if o.numel() else 0.0))

    def add_stats(self, smax_g, ssum_g, smax_o, ssum_o):
        assert_stats(smax_g, ssum_g, smax_o, ssum_o, self.dtype, quiet=True)
        gm, gs = smax_g[..., 0].double(), ssum_g[..., 0].double()
        fin = torch.isfinite(smax_o)
        if fin.any():
            self.stat_max_abs = max(self.stat_max_abs,
                                    float((gm[fin] - smax_o[fin]).abs().max()))
            self.stat_sum_rel = max(self.stat_sum_rel, float(
                ((gs[fin] - ssum_o[fin]).abs() / ssum_o[fin].abs()).max()))

    def merge(self, other):
        for name, (mx, s, n, ref) in other.t.items():
            a = self.t.get(name, (0.0, 0.0, 0, 0.0))
            self.t[name] = (max(a[0], mx), a[1] + s, a[2] + n, max(a[3], ref))
        self.stat_max_abs = max(self.stat_max_abs, other.stat_max_abs)
        self.stat_sum_rel = max(self.stat_sum_rel, other.stat_sum_rel)

    def check(self, label):
        for name, (mx, s, n, ref) in self.t.items():
            mean = s / max(n, 1)
            if self.dtype == torch.float32:
                rel = mx / max(ref, TOL_FP32_FLOOR)
                note(f"  {label} {name}: max_rel={rel:.3e} over {n} elements")
                assert rel <= TOL_FP32_REL, f"{name}: max relative error {rel:.3e}"
            else:
                note(f"  {label} {name}: max_abs={mx:.3e} mean_abs={mean:.3e} over {n} "
                     f"elements (|ref|max={ref:.3e})")
                assert mx <= TOL_BF16_MAX, f"{name}: max abs error {mx:.3e} > {TOL_BF16_MAX}"
                assert mean <= TOL_BF16_MEAN, f"{name}: mean abs error {mean:.3e}"
        note(f"  {label} softmax_max: max_abs={self.stat_max_abs:.3e}  softmax_sum: "
             f"max_rel={self.stat_sum_rel:.3e}")


def compare_streamed(p, g, kv_heads, acc, chunk=512):
    """Compare every row and key of the given key/value heads (with their
    query heads) of problem p against the oracle, one (sequence, key/value
    head) at a time on contiguous slices, so that no fp64 copy of the whole
    problem is held.  The oracle gives a varlen batch the results of separate
    per-sequence calls, so each slice is its own one-sequence problem."""
    G = p.q.shape[1] // p.k.shape[1]
    kw = dict(pre_tokens=p.pre_tokens, next_tokens=p.next_tokens,
              sparse_mode=p.sparse_mode, chunk=chunk)
    for (q0, lq), (k0, lk) in zip(oracle.sequences(p.cu_seqlens_q),
                                  oracle.sequences(p.cu_seqlens_kv)):
        tq, tk = slice(q0, q0 + lq), slice(k0, k0 + lk)
        for h in kv_heads:
            hq, hk = slice(h * G, (h + 1) * G), slice(h, h + 1)
            Q, dY = (x[tq, hq].contiguous() for x in (p.q, p.dy))
            K, V = (x[tk, hk].contiguous() for x in (p.k, p.v))
            out, sm, ss = oracle.forward(Q, K, V, [lq], [lk], p.scale, **kw)
            dq, dk, dv = oracle.backward(Q, K, V, dY, out, sm, ss, [lq], [lk], p.scale, **kw)
            acc.add("out", g["out"][tq, hq], out)
            acc.add("dq", g["dq"][tq, hq], dq)
            acc.add("dk", g["dk"][tk, hk], dk)
            acc.add("dv", g["dv"][tk, hk], dv)
            acc.add_stats(g["smax"][tq, hq], g["ssum"][tq, hq], sm, ss)
