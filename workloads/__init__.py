"""Seeded synthetic inputs for the sliding-window attention path.

This module only draws random numbers and lays them out; it contains none of
the attention arithmetic.  Both the HIP path (through its Python binding) and
the fp64 oracle consume what it produces, so they see identical bits.

Recipe (shared by every workload):
  * ``g = torch.Generator('cpu').manual_seed(seed)`` (seed 42 by default, the
    seed used by the PyPTO-Gym FlashAttentionScoreGrad golden, section
    "验证 Golden").
  * Draw order: sequence lengths first (varlen workloads:
    ``torch.randint(lo, hi + 1, (nseq,), generator=g)``), then q, k, v, dy,
    each ``torch.randn(shape, generator=g, dtype=float32) * std`` and then
    ``.to(dtype)`` (round to nearest even).
  * BNSD workloads draw ``[B, N, S, D]`` and are permuted to TND
    ``[B*S, N, D]`` with one cumulative end per batch.
  * Sequence boundaries are inclusive cumulative end offsets, one per batch,
    no leading zero (the FlashAttentionVarLenScore API doc, parameter
    actualSeqQLenOptional; the aclnnFlashAttentionUnpaddingScoreGradV2
    explainer, section 6.4).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

INT_MAX = 2147483647


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    num_heads: int
    head_dim: int
    sparse_mode: int
    scale: float
    pre_tokens: int = INT_MAX
    next_tokens: int = INT_MAX
    std: float = 1.0
    # BNSD-shaped workloads: fixed batch / sequence length
    batch: int = 0
    seqlen: int = 0
    # varlen workloads: number of sequences and inclusive length bounds
    nseq: int = 0
    len_lo: int = 0
    len_hi: int = 0
    seed: int = 42
    num_kv_heads: int = 0   # 0: as many key/value heads as query heads
    note: str = field(default="", compare=False)


# Five workloads shaped like the pages' cases (the fourth is the headline
# sliding-window case: S = 16K, window of 2048 past tokens), then three that
# measure the other masks, grouped heads and fp32 inputs at the headline's shape.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("dense_fp32_b1_n2_s128_d64", torch.float32, 2, 64, 0, 1.0 / 8,
                 batch=1, seqlen=128),
        Workload("dense_bf16_b1_n8_s512_d64", torch.bfloat16, 8, 64, 0, 1.0 / 8,
                 batch=1, seqlen=512),
        Workload("varlen_bf16_n16_d128_8seq_256to4096", torch.bfloat16, 16, 128, 0,
                 1.0 / math.sqrt(128), nseq=8, len_lo=256, len_hi=4096),
        Workload("swa_bf16_b1_n16_s16384_d128_pre2048_next0", torch.bfloat16, 16, 128, 4,
                 1.0 / math.sqrt(128), pre_tokens=2048, next_tokens=0, batch=1, seqlen=16384),
        Workload("varlen_swa_bf16_n32_d128_4seq_16kto32k_pre4096_next512", torch.bfloat16,
                 32, 128, 4, 1.0 / math.sqrt(128), pre_tokens=4096, next_tokens=512, std=0.5,
                 nseq=4, len_lo=16384, len_hi=32768),
        # the 16K shape under the other masks and head layouts the library
        # takes: causal (sparse_mode 2) and 4:1 grouped key/value heads
        Workload("causal_bf16_b1_n16_s16384_d128", torch.bfloat16, 16, 128, 2,
                 1.0 / math.sqrt(128), batch=1, seqlen=16384),
        # (std 0.5: dK / dV sum four query heads, and at std 1 they reach ~10,
        # where one bf16 rounding step of the output alone (1/16) exceeds the
        # absolute tolerance; at 0.5 they stay near unit scale)
        Workload("gqa_swa_bf16_b1_n16kv4_s16384_d128_pre2048_next0", torch.bfloat16, 16, 128, 4,
                 1.0 / math.sqrt(128), pre_tokens=2048, next_tokens=0, std=0.5, batch=1,
                 seqlen=16384, num_kv_heads=4),
        # the 16K window workload with fp32 inputs (the fp32 kernels at full size)
        Workload("swa_fp32_b1_n16_s16384_d128_pre2048_next0", torch.float32, 16, 128, 4,
                 1.0 / math.sqrt(128), pre_tokens=2048, next_tokens=0, batch=1, seqlen=16384),
    ]
}

WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "swa_bf16_b1_n16_s16384_d128_pre2048_next0"


@dataclass
class Problem:
    """One synthetic problem in TND layout (host tensors)."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    dy: torch.Tensor
    cu_seqlens_q: list
    cu_seqlens_kv: list
    scale: float
    pre_tokens: int
    next_tokens: int
    sparse_mode: int
    name: str = ""

    @property
    def num_heads(self):
        return self.q.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def dtype(self):
        return self.q.dtype


def cumulative(lengths):
    out, acc = [], 0
    for L in lengths:
        acc += int(L)
        out.append(acc)
    return out


def _randn(g, shape, std, dtype):
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_problem(w: Workload | str, seed: int | None = None) -> Problem:
    """Draw the seeded inputs of a named workload (see the module docstring)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    heads = [w.num_heads, w.num_kv_heads or w.num_heads, w.num_kv_heads or w.num_heads,
             w.num_heads]  # q, k, v, dy
    if w.nseq:
        lengths = torch.randint(w.len_lo, w.len_hi + 1, (w.nseq,), generator=g).tolist()
        T = sum(lengths)
        tensors = [_randn(g, (T, n, w.head_dim), w.std, w.dtype) for n in heads]
    else:
        lengths = [w.seqlen] * w.batch
        tensors = [
            _randn(g, (w.batch, n, w.seqlen, w.head_dim), w.std, w.dtype).permute(
                0, 2, 1, 3).reshape(w.batch * w.seqlen, n, w.head_dim).contiguous()
            for n in heads
        ]
    cu = cumulative(lengths)
    q, k, v, dy = tensors
    return Problem(q, k, v, dy, cu, list(cu), w.scale, w.pre_tokens, w.next_tokens,
                   w.sparse_mode, name=w.name)


def make_custom(lengths_q, lengths_kv=None, num_heads=2, head_dim=64, dtype=torch.bfloat16,
                sparse_mode=0, pre_tokens=INT_MAX, next_tokens=INT_MAX, scale=None,
                std=1.0, seed=42, trailing=0, extra_tokens=0, name="custom",
                num_kv_heads=None) -> Problem:
    """Small seeded problem with explicit sequence lengths.

    ``trailing`` appends that many non-participating batches (zeros in the
    cumulative arrays); ``extra_tokens`` appends tokens after the last
    sequence that belong to no batch.  ``num_kv_heads`` (default: num_heads) gives k
    and v fewer heads than q (grouped heads).
    """
    lengths_kv = list(lengths_q) if lengths_kv is None else list(lengths_kv)
    g = torch.Generator("cpu").manual_seed(seed)
    tq = sum(lengths_q) + extra_tokens
    tkv = sum(lengths_kv) + extra_tokens
    q = _randn(g, (tq, num_heads, head_dim), std, dtype)
    nkv = num_heads if num_kv_heads is None else num_kv_heads
    k = _randn(g, (tkv, nkv, head_dim), std, dtype)
    v = _randn(g, (tkv, nkv, head_dim), std, dtype)
    dy = _randn(g, (tq, num_heads, head_dim), std, dtype)
    cu_q = cumulative(lengths_q) + [0] * trailing
    cu_kv = cumulative(lengths_kv) + [0] * trailing
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Problem(q, k, v, dy, cu_q, cu_kv, scale, pre_tokens, next_tokens, sparse_mode,
                   name=name)


def make_drop_mask(p: Problem, keep_prob: float, seed: int = 7) -> torch.Tensor:
    """Seeded dropout keep mask for problem p: one bit per (participating batch,
    query head, query row, key), each 1 with probability keep_prob, packed
    eight to a byte least significant bit first in (batch, head, row, key)
    order, and padded with zero bytes to whole 32-bit words (uint8 host tensor)."""
    import numpy as np
    g = torch.Generator("cpu").manual_seed(seed)
    lens_q, lens_kv, prev_q, prev_kv = [], [], 0, 0
    for cq, ck in zip(p.cu_seqlens_q, p.cu_seqlens_kv):
        if cq == 0 and prev_q > 0:
            break
        lens_q.append(cq - prev_q)
        lens_kv.append(ck - prev_kv)
        prev_q, prev_kv = cq, ck
    nbits = sum(p.num_heads * a * b for a, b in zip(lens_q, lens_kv))
    if keep_prob == 0.5:  # every bit a fair coin: draw whole random bytes
        packed = torch.randint(0, 256, ((nbits + 7) // 8,), generator=g,
                               dtype=torch.uint8).numpy()
        if nbits % 8:
            packed[-1] &= (1 << (nbits % 8)) - 1
    else:
        keep = (torch.rand(nbits, generator=g) < keep_prob).numpy().astype(np.uint8)
        packed = np.packbits(keep, bitorder="little")
    words = (packed.size + 3) // 4
    out = np.zeros(4 * max(words, 1), dtype=np.uint8)
    out[:packed.size] = packed
    return torch.from_numpy(out)

