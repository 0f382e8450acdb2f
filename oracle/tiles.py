"""Brute-force tile enumerator for the varlen band schedule.

TEST INFRASTRUCTURE ONLY (see the package docstring).

It classifies every (row block, column block) tile of every participating
sequence by evaluating the element mask itself (``attention.allowed_mask``),
with no closed-form shortcuts:

* skipped  - no element (i < Sq, j < Skv) of the tile is allowed;
* full     - every element of the complete BM x BN tile lies inside the
             sequence and is allowed;
* partial  - everything else (band edges and ragged tails).

Skipping tiles outside the band is how the FlashAttention kernels of the pages
turn the band of sparse_mode 4 into saved work (op-plugin sliding-window blog,
section 1.3; explainer section 8.1: the actual_seq values drive tiling).

``direction='fwd'`` iterates query blocks (items) over key tiles;
``direction='bwd'`` iterates key blocks (items) over query tiles.
"""
from __future__ import annotations

import numpy as np
import torch

from .attention import allowed_mask, sequences

PARTIAL, FULL = 1, 2


def _tile_kind(mask_block):
    if not mask_block.any():
        return 0
    return FULL if mask_block.all() else PARTIAL


def enumerate_tiles(cu_seqlens_q, cu_seqlens_kv, sparse_mode, pre_tokens, next_tokens,
                    block_item, block_tile, direction="fwd"):
    """Return {(seq, item_block): [(tile, kind), ...]} over visited tiles.

    Items with no visited tile map to an empty list.  ``block_item`` is the
    item block size (rows for 'fwd', keys for 'bwd'), ``block_tile`` the tile
    block size along the other axis.
    """
    out = {}
    for b, ((_, sq), (_, skv)) in enumerate(zip(sequences(cu_seqlens_q),
                                                sequences(cu_seqlens_kv))):
        if direction == "fwd":
            n_items, n_tiles, bm, bn = -(-sq // block_item), -(-skv // block_tile), \
                block_item, block_tile
        else:
            n_items, n_tiles, bm, bn = -(-skv // block_item), -(-sq // block_tile), \
                block_tile, block_item
        for it in range(n_items):
            # element mask of the whole item strip, padded to whole tiles
            if direction == "fwd":
                rows = torch.arange(it * bm, it * bm + bm)
                cols = torch.arange(0, n_tiles * bn)
            else:
                rows = torch.arange(0, n_tiles * bm)
                cols = torch.arange(it * bn, it * bn + bn)
            m = allowed_mask(rows, cols, sparse_mode, pre_tokens, next_tokens, sq, skv)
            m &= (rows < sq)[:, None] & (cols < skv)[None, :]
            m = m.numpy()
            if direction == "fwd":
                per_tile = m.reshape(bm, n_tiles, bn).transpose(1, 0, 2)
            else:
                per_tile = m.reshape(n_tiles, bm, bn)
            visited = []
            for t in range(n_tiles):
                kind = _tile_kind(per_tile[t])
                if kind:
                    visited.append((t, kind))
            out[(b, it)] = visited
    return out


def count_pairs(cu_seqlens_q, cu_seqlens_kv, sparse_mode, pre_tokens, next_tokens,
                row_chunk=1024):
    """Number of allowed (i, j) pairs per head, by summing the element mask."""
    total = 0
    for (_, sq), (_, skv) in zip(sequences(cu_seqlens_q), sequences(cu_seqlens_kv)):
        cols = torch.arange(skv)
        for r0 in range(0, sq, row_chunk):
            rows = torch.arange(r0, min(sq, r0 + row_chunk))
            total += int(allowed_mask(rows, cols, sparse_mode, pre_tokens,
                                      next_tokens, sq, skv).sum())
    return total


def summarize(tiles):
    """(visited, full, partial) tile counts of an enumerate_tiles result."""
    vis = sum(len(v) for v in tiles.values())
    full = sum(1 for v in tiles.values() for _, k in v if k == FULL)
    return vis, full, vis - full


__all__ = ["enumerate_tiles", "count_pairs", "summarize", "PARTIAL", "FULL", "np"]
