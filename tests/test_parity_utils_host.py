"""CPU checks of the streamed whole-tensor comparison used by the GPU parity
tests: fed the oracle's own results (rounded to bf16) in place of GPU results,
it must report exactly the errors a direct whole-tensor comparison reports,
and a single planted error in one head must show up in its figures."""
import pytest
import torch

import workloads
from parity_utils import StreamedErrors, compare_streamed, run_oracle


def as_gpu_like(o):
    """Oracle results in the layout and precision the GPU path returns."""
    g = {n: o[n].to(torch.bfloat16) for n in ("out", "dq", "dk", "dv")}
    g["smax"] = o["smax"].float()[..., None].expand(-1, -1, 8).contiguous()
    g["ssum"] = o["ssum"].float()[..., None].expand(-1, -1, 8).contiguous()
    return g


@pytest.mark.parametrize("kw", [
    dict(lengths_q=[70, 33, 129], num_heads=3, head_dim=16, sparse_mode=4, pre_tokens=20,
         next_tokens=3),
    dict(lengths_q=[40, 90], lengths_kv=[65, 30], num_heads=4, num_kv_heads=2, head_dim=16,
         sparse_mode=3),
])
def test_streamed_equals_direct(kw):
    p = workloads.make_custom(**kw)
    o = run_oracle(p, chunk=None)
    g = as_gpu_like(o)
    acc = StreamedErrors(p.dtype)
    compare_streamed(p, g, range(p.k.shape[1]), acc, chunk=32)
    for n in ("out", "dq", "dk", "dv"):
        d = (g[n].double() - o[n]).abs()
        mx, s, cnt, ref = acc.t[n]
        assert cnt == d.numel() and abs(mx - float(d.max())) <= 1e-12
        assert abs(s - float(d.sum())) <= 1e-9 * max(1.0, float(d.sum()))
    acc.check("host")
    # one wrong element of dk in the last key/value head
    g["dk"][-1, -1, 0] += 0.5
    acc2 = StreamedErrors(p.dtype)
    compare_streamed(p, g, [p.k.shape[1] - 1], acc2, chunk=32)
    assert acc2.t["dk"][0] >= 0.49
    with pytest.raises(AssertionError):
        acc2.check("host")
