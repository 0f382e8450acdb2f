"""Plain fp64 CPU definition of the attention forward and backward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything is computed
in float64 with torch CPU ops; S, P and dS are materialised explicitly.

What is computed, and where the pages define it:

* Forward, per sequence b and head n (FlashAttentionVarLenScore API doc,
  "计算公式"; aclnnFlashAttentionUnpaddingScoreGradV2 explainer, section 2.2),
  with no pse, no dropout (keep_prob = 1) and no explicit mask tensor:
      S = scale * Q K^T, masked entries set to -inf
      P = softmax(S) row-wise,   out = P V
* Saved statistics (PyPTO-Gym FlashAttentionScoreGrad article, "前向公式" and
  "反向公式"): softmax_max = row max of the scaled, masked scores;
  softmax_sum = sum_j exp(S_ij - softmax_max_i), so that
  P = exp(S - softmax_max) / softmax_sum.
* Backward (PyPTO-Gym FlashAttentionScoreGrad article, "反向公式";
  UnpaddingScoreGradV2 explainer, section 2.3):
      P  = exp(scale Q K^T - softmax_max) / softmax_sum   (caller's statistics)
      Dv = rowsum(dY * O)                                  (caller's O)
      dP = dY V^T,  dS = P * (dP - Dv)
      dV = P^T dY,  dQ = scale dS K,  dK = scale dS^T Q
* Masks (op-plugin sliding-window blog, section 1.3 "SparseMode说明"; API doc,
  preTokensOptional / nextTokensOptional; explainer 6.6), with
  sequence-local indices i (query) and j (key) of a sequence with Sq queries
  and Skv keys:
      sparse_mode 0 (no mask)          every key;
      sparse_mode 2 (LEFT_UP_CAUSAL)   j <= i        (causal, top-left corner);
      sparse_mode 3 (RIGHT_DOWN_CAUSAL) j - i <= Skv - Sq (causal, bottom-right);
      sparse_mode 4 (BAND)             -pre_tokens <= j - i <= next_tokens.
  The pages name modes 2 and 3 but print no formula; the reading here takes
  the corner in each name as the corner the diagonal starts from.  Modes 2
  and 3 ignore pre_tokens / next_tokens.
* Grouped heads (explainer 6.2): q has Nq heads and k / v have Nkv heads with
  Nq / Nkv = G a whole number; query head n reads key/value head n // G
  (floor division), and the gradients of a key/value head sum over the G
  query heads that read it.  G = 1 is the ordinary multi-head case.
* Dropout with a given mask (API doc, 计算公式 and dropMaskOptional /
  keepProbOptional; explainer 2.2, 6.3): attention_out = Dropout(P, keep_prob) V,
  where the mask keeps an element where its bit is 1 (keep_prob is the
  fraction of ones) and a kept element is scaled by 1 / keep_prob (the usual
  inverted dropout; the pages print no scaling).  The statistics are those
  of the undropped softmax.  The mask is uint8 holding 8 one-bit booleans per
  byte, (sum_b sum_n Sq*Skv)/8 bytes: bit e of the whole array is byte e // 8,
  bit e % 8 (least significant first), and e runs over batches, then heads,
  then the Sq x Skv matrix of that (batch, head) row by row.  The backward
  applies the same mask: dV = (P * Z / kp)^T dY, dP = (dY V^T) * Z / kp,
  dS = P * (dP - Dv) with Dv = rowsum(dY * O).  The byte order, bit order and
  the batch-before-head order are readings: the pages give only the size
  formula.
* Varlen TND packing (API doc, "算子功能" and inputLayout; explainer 4.2, 6.4):
  tokens of each batch are packed back to back; cumulative ends are inclusive,
  one per batch; trailing zeros mark batches that do not participate.

Readings where the pages are silent: empty rows (every key masked) give
out = 0, softmax_max = -inf, softmax_sum = 0 and dq = 0; keys no query attends
get dk = dv = 0; tokens after the last participating end get zeros; mode 0
ignores pre/next.

Row chunking (``chunk``) evaluates the same definition a block of rows at a
time over the columns the band can reach in that block; the dropped columns are
masked for every row of the block and contribute exactly zero.
"""
from __future__ import annotations

import math

import torch

INT_MAX = 2147483647
F64 = torch.float64


def sequences(cu_seqlens):
    """Return [(start, length)] for each participating batch.

    ``cu_seqlens`` holds inclusive cumulative ends, one per batch.  A zero that
    follows a positive entry starts the trailing run of non-participating
    batches (explainer section 6.4: ``[2, 5, 9, 0, 0]``).
    """
    out = []
    prev = 0
    for c in cu_seqlens:
        c = int(c)
        if c == 0 and prev > 0:
            break
        if c < prev:
            raise ValueError("cumulative sequence ends must be non-decreasing")
        out.append((prev, c - prev))
        prev = c
    return out


SPARSE_MODES = (0, 2, 3, 4)


def allowed_mask(rows, cols, sparse_mode, pre_tokens, next_tokens, sq=None, skv=None):
    """Boolean [len(rows), len(cols)]: True where query i may attend key j.

    ``sq`` / ``skv`` (the sequence's query and key lengths) are needed by
    sparse_mode 3 only, whose diagonal ends in the bottom-right corner.
    """
    i = torch.as_tensor(rows, dtype=torch.int64)[:, None]
    j = torch.as_tensor(cols, dtype=torch.int64)[None, :]
    d = j - i
    if sparse_mode == 0:
        return torch.ones(i.shape[0], j.shape[1], dtype=torch.bool)
    if sparse_mode == 2:
        return d <= 0
    if sparse_mode == 3:
        if sq is None or skv is None:
            raise ValueError("sparse_mode 3 needs the sequence lengths")
        return d <= int(skv) - int(sq)
    if sparse_mode == 4:
        return (d >= -int(pre_tokens)) & (d <= int(next_tokens))
    raise ValueError(f"The sparse_mode value should be 0, 2, 3 or 4, but got {sparse_mode}")


def _col_window(r0, r1, sq, skv, sparse_mode, pre, nxt, chunked):
    """Columns that rows [r0, r1) can reach; all columns unless chunked.

    Only used to skip columns that are masked for every row of the block.
    """
    if sparse_mode == 0 or not chunked:
        return 0, skv
    if sparse_mode == 2:
        lo, hi = 0, min(skv, r1)
    elif sparse_mode == 3:
        lo, hi = 0, min(skv, r1 + skv - sq)
    else:
        lo = max(0, r0 - int(pre))
        hi = min(skv, r1 - 1 + int(nxt) + 1)
    lo = min(lo, skv)
    return lo, max(lo, hi)


def _scores(Q, K, rows, c0, c1, scale, sparse_mode, pre, nxt):
    """Scaled, masked scores for rows x columns [c0, c1) (masked = -inf)."""
    S = scale * (Q[rows] @ K[c0:c1].T)
    M = allowed_mask(torch.as_tensor(rows), torch.arange(c0, c1), sparse_mode, pre, nxt,
                     Q.shape[0], K.shape[0])
    return S.masked_fill(~M, -math.inf), M


def _softmax_stats(S):
    """Row max, exp(S - max) and row sum; empty rows give -inf, 0, 0."""
    m = S.max(dim=1).values if S.shape[1] else torch.full((S.shape[0],), -math.inf, dtype=F64)
    finite = torch.isfinite(m)
    E = torch.where(finite[:, None], torch.exp(S - torch.where(finite, m, 0.0)[:, None]),
                    torch.zeros((), dtype=F64))
    E = torch.nan_to_num(E, nan=0.0)
    l = E.sum(dim=1)
    return m, E, l


def _dropped(P, Z, rows, c0, c1, keep_prob):
    """P * Z / keep_prob over rows x columns [c0, c1) (Z = None: no dropout)."""
    if Z is None:
        return P
    return torch.where(Z[rows][:, c0:c1], P / keep_prob, torch.zeros((), dtype=F64))


def _seq_head_forward(Q, K, V, scale, sparse_mode, pre, nxt, rows, chunked, Z=None,
                      keep_prob=1.0):
    r0, r1 = int(rows[0]), int(rows[-1]) + 1
    c0, c1 = _col_window(r0, r1, Q.shape[0], K.shape[0], sparse_mode, pre, nxt, chunked)
    S, _ = _scores(Q, K, rows, c0, c1, scale, sparse_mode, pre, nxt)
    m, E, l = _softmax_stats(S)
    P = torch.where(l[:, None] > 0, E / torch.where(l > 0, l, 1.0)[:, None],
                    torch.zeros((), dtype=F64))
    O = _dropped(P, Z, rows, c0, c1, keep_prob) @ V[c0:c1]
    return O, m, l


def _row_chunks(n, chunk):
    if n == 0:
        return []
    if not chunk:
        return [torch.arange(0, n)]
    return [torch.arange(r, min(n, r + chunk)) for r in range(0, n, chunk)]


def _as64(x):
    return x.detach().to("cpu").to(F64)


def drop_mask_bits(cu_seqlens_q, cu_seqlens_kv, num_heads):
    """Number of mask bits: sum over participating batches b and heads n of Sq*Skv."""
    return sum(num_heads * sq * skv for (_, sq), (_, skv) in
               zip(sequences(cu_seqlens_q), sequences(cu_seqlens_kv)))


def unpack_drop_mask(drop_mask, cu_seqlens_q, cu_seqlens_kv, num_heads):
    """{(b, n): bool [Sq, Skv]} from the packed mask (True = keep)."""
    import numpy as np
    raw = np.asarray(torch.as_tensor(drop_mask, dtype=torch.uint8).cpu().numpy(), dtype=np.uint8)
    nbits = drop_mask_bits(cu_seqlens_q, cu_seqlens_kv, num_heads)
    if raw.size * 8 < nbits:
        raise ValueError(f"drop mask has {raw.size} bytes, needs {(nbits + 7) // 8}")
    bits = np.unpackbits(raw, bitorder="little")
    out, e = {}, 0
    for b, ((_, sq), (_, skv)) in enumerate(zip(sequences(cu_seqlens_q),
                                                sequences(cu_seqlens_kv))):
        for n in range(num_heads):
            out[(b, n)] = torch.from_numpy(bits[e:e + sq * skv].reshape(sq, skv).astype(bool))
            e += sq * skv
    return out


def group_size(q, k):
    """Query heads per key/value head (explainer 6.2: Nq / Nkv a whole number)."""
    nq, nkv = q.shape[1], k.shape[1]
    if nkv < 1 or nq % nkv:
        raise ValueError(f"query heads ({nq}) must be a multiple of key/value heads ({nkv})")
    return nq // nkv


def forward(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, pre_tokens=INT_MAX,
            next_tokens=INT_MAX, sparse_mode=0, chunk=None, heads=None, drop_mask=None,
            keep_prob=1.0):
    """Attention forward over a TND batch.

    Returns (out [Tq, N, D], softmax_max [Tq, N], softmax_sum [Tq, N]) in fp64.
    ``chunk`` (rows per block) only changes evaluation order, not the result.
    ``drop_mask`` (packed uint8, see the module docstring) applies dropout with
    ``keep_prob``.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    Tq, N, D = q.shape
    G = group_size(q, k)
    Zs = None if drop_mask is None else unpack_drop_mask(drop_mask, cu_seqlens_q,
                                                         cu_seqlens_kv, N)
    out = torch.zeros(Tq, N, v.shape[2], dtype=F64)
    smax = torch.full((Tq, N), -math.inf, dtype=F64)
    ssum = torch.zeros((Tq, N), dtype=F64)
    sq_list, skv_list = sequences(cu_seqlens_q), sequences(cu_seqlens_kv)
    if len(sq_list) != len(skv_list):
        raise ValueError("query and key/value batches disagree")
    for b, ((q0, sq), (k0, skv)) in enumerate(zip(sq_list, skv_list)):
        for n in (range(N) if heads is None else heads):
            Q, K, V = q[q0:q0 + sq, n], k[k0:k0 + skv, n // G], v[k0:k0 + skv, n // G]
            Z = None if Zs is None else Zs[(b, n)]
            for rows in _row_chunks(sq, chunk):
                O, m, l = _seq_head_forward(Q, K, V, scale, sparse_mode, pre_tokens,
                                            next_tokens, rows, chunk is not None, Z, keep_prob)
                out[q0 + rows, n] = O
                smax[q0 + rows, n] = m
                ssum[q0 + rows, n] = l
    return out, smax, ssum


def _recompute_p(Q, K, rows, c0, c1, scale, sparse_mode, pre, nxt, m_rows, l_rows):
    """P = exp(S - softmax_max) / softmax_sum from the given statistics."""
    S, M = _scores(Q, K, rows, c0, c1, scale, sparse_mode, pre, nxt)
    ok = (l_rows > 0) & torch.isfinite(m_rows)
    mm = torch.where(ok, m_rows, 0.0)
    ll = torch.where(ok, l_rows, 1.0)
    P = torch.exp(S - mm[:, None]) / ll[:, None]
    P = torch.where(M & ok[:, None], P, torch.zeros((), dtype=F64))
    return P


def backward(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, scale,
             pre_tokens=INT_MAX, next_tokens=INT_MAX, sparse_mode=0, chunk=None, heads=None,
             drop_mask=None, keep_prob=1.0):
    """Attention backward; uses the caller's out and statistics verbatim.

    ``softmax_max``/``softmax_sum`` may be [T, N] or [T, N, 8] (column 0 is
    read, as the stored statistics keep the value in column 0).
    Returns (dq, dk, dv) in fp64.
    """
    q, k, v, dy, out = _as64(q), _as64(k), _as64(v), _as64(dy), _as64(out)
    sm, ss = _as64(softmax_max), _as64(softmax_sum)
    if sm.dim() == 3:
        sm, ss = sm[..., 0], ss[..., 0]
    Tq, N, D = q.shape
    G = group_size(q, k)
    Zs = None if drop_mask is None else unpack_drop_mask(drop_mask, cu_seqlens_q,
                                                         cu_seqlens_kv, N)
    dq = torch.zeros_like(q)
    dk = torch.zeros_like(k)
    dv = torch.zeros(v.shape, dtype=F64)
    for b, ((q0, sq), (k0, skv)) in enumerate(zip(sequences(cu_seqlens_q),
                                                  sequences(cu_seqlens_kv))):
        for n in (range(N) if heads is None else heads):
            Q, K, V = q[q0:q0 + sq, n], k[k0:k0 + skv, n // G], v[k0:k0 + skv, n // G]
            dY, O = dy[q0:q0 + sq, n], out[q0:q0 + sq, n]
            Z = None if Zs is None else Zs[(b, n)]
            for rows in _row_chunks(sq, chunk):
                c0, c1 = _col_window(int(rows[0]), int(rows[-1]) + 1, sq, skv, sparse_mode,
                                     pre_tokens, next_tokens, chunk is not None)
                P = _recompute_p(Q, K, rows, c0, c1, scale, sparse_mode, pre_tokens,
                                 next_tokens, sm[q0 + rows, n], ss[q0 + rows, n])
                Dv = (dY[rows] * O[rows]).sum(dim=1)
                dP = _dropped(dY[rows] @ V[c0:c1].T, Z, rows, c0, c1, keep_prob)
                dS = P * (dP - Dv[:, None])
                dv[k0 + c0:k0 + c1, n // G] += _dropped(P, Z, rows, c0, c1, keep_prob).T @ dY[rows]
                dq[q0 + rows, n] = scale * (dS @ K[c0:c1])
                dk[k0 + c0:k0 + c1, n // G] += scale * (dS.T @ Q[rows])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Restrictions of the same definition to a few rows or keys of one
# (sequence, head).  They let tests check sampled outputs of problems too large
# to evaluate in full.  Inputs are the sequence-local [S, D] slices.
# ---------------------------------------------------------------------------

def forward_rows(Q, K, V, rows, scale, sparse_mode=0, pre_tokens=INT_MAX,
                 next_tokens=INT_MAX, chunk=128):
    """out, softmax_max, softmax_sum of the given query rows (fp64).

    Rows are evaluated in groups of consecutive indices, ``chunk`` at a time.
    """
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    rows = torch.as_tensor(rows, dtype=torch.int64).reshape(-1)
    O = torch.zeros(len(rows), V.shape[1], dtype=F64)
    m = torch.full((len(rows),), -math.inf, dtype=F64)
    l = torch.zeros(len(rows), dtype=F64)
    start = 0
    while start < len(rows):
        end = start + 1
        while (end < len(rows) and end - start < chunk
               and int(rows[end]) == int(rows[end - 1]) + 1):
            end += 1
        o, mm, ll = _seq_head_forward(Q, K, V, scale, sparse_mode, pre_tokens, next_tokens,
                                      rows[start:end], True)
        O[start:end], m[start:end], l[start:end] = o, mm, ll
        start = end
    return O, m, l


def backward_rows(Q, K, V, dY, rows, scale, sparse_mode=0, pre_tokens=INT_MAX,
                  next_tokens=INT_MAX):
    """dq of the given query rows, end to end (statistics and O from forward_rows)."""
    Q, K, V, dY = _as64(Q), _as64(K), _as64(V), _as64(dY)
    rows = torch.as_tensor(rows, dtype=torch.int64)
    O, m, l = forward_rows(Q, K, V, rows, scale, sparse_mode, pre_tokens, next_tokens)
    dq = torch.zeros(len(rows), Q.shape[1], dtype=F64)
    for idx, r in enumerate(rows.tolist()):
        c0, c1 = _col_window(r, r + 1, Q.shape[0], K.shape[0], sparse_mode, pre_tokens,
                             next_tokens, True)
        rr = torch.tensor([r])
        P = _recompute_p(Q, K, rr, c0, c1, scale, sparse_mode, pre_tokens, next_tokens,
                         m[idx:idx + 1], l[idx:idx + 1])
        Dv = (dY[rr] * O[idx:idx + 1]).sum(dim=1)
        dS = P * (dY[rr] @ V[c0:c1].T - Dv[:, None])
        dq[idx] = scale * (dS @ K[c0:c1])[0]
    return dq


def backward_keys(Q, K, V, dY, key_lo, key_hi, scale, sparse_mode=0, pre_tokens=INT_MAX,
                  next_tokens=INT_MAX):
    """dk, dv of keys [key_lo, key_hi), end to end.

    Every query row that can attend one of these keys is evaluated in full
    (its statistics and O come from forward_rows over its whole band).
    """
    Q, K, V, dY = _as64(Q), _as64(K), _as64(V), _as64(dY)
    sq, skv = Q.shape[0], K.shape[0]
    if sparse_mode == 4:
        r0 = max(0, key_lo - int(next_tokens))
        r1 = min(sq, key_hi - 1 + int(pre_tokens) + 1)
    elif sparse_mode == 2:
        r0, r1 = min(sq, key_lo), sq
    elif sparse_mode == 3:
        r0, r1 = min(sq, max(0, key_lo - (skv - sq))), sq
    else:
        r0, r1 = 0, sq
    dk = torch.zeros(key_hi - key_lo, K.shape[1], dtype=F64)
    dv = torch.zeros(key_hi - key_lo, V.shape[1], dtype=F64)
    if r1 <= r0:
        return dk, dv
    rows = torch.arange(r0, r1)
    O, m, l = forward_rows(Q, K, V, rows, scale, sparse_mode, pre_tokens, next_tokens)
    P = _recompute_p(Q, K, rows, key_lo, key_hi, scale, sparse_mode, pre_tokens, next_tokens,
                     m, l)
    Dv = (dY[rows] * O).sum(dim=1)
    dS = P * (dY[rows] @ V[key_lo:key_hi].T - Dv[:, None])
    dv = P.T @ dY[rows]
    dk = scale * (dS.T @ Q[rows])
    return dk, dv
