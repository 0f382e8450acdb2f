"""Host-side checks of the C ABI (CPU only: no kernel is launched).

* libswa.so loads and exports every function include/swa.h declares;
* validation returns the documented status for each bad argument, before
  anything touches the GPU;
* the tile schedule (swa_debug_tile_schedule) equals the brute-force
  enumeration of oracle/tiles.py tile by tile (the skip and mask pattern).
"""
import ctypes
import glob
import os
import re

import pytest

import oracle
import transformer_attention_tnd_amd as swa
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INT_MAX = 2147483647


def declared_functions():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(swa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = swa.load_library()
    names = declared_functions()
    assert {"swa_forward", "swa_backward", "swa_forward_workspace_size",
            "swa_backward_workspace_size", "swa_last_error",
            "swa_debug_tile_schedule"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    # and nothing is exported under those names that the binding does not wrap
    for n in names:
        assert hasattr(swa, n), n


def raw_forward(**kw):
    """Call swa_forward through ctypes with fake (never dereferenced) pointers."""
    lib = swa.load_library()
    a = dict(q=1, k=1, v=1, cu_q=[16], cu_kv=[16], t_q=16, t_kv=16, n=2, d=64, dtype=1,
             scale=0.125, pre=INT_MAX, nxt=INT_MAX, mode=0, out=1, smax=1, ssum=1, ws=1,
             ws_bytes=1 << 30)
    a.update(kw)
    cq = (ctypes.c_int64 * max(1, len(a["cu_q"])))(*a["cu_q"])
    ck = (ctypes.c_int64 * max(1, len(a["cu_kv"])))(*a["cu_kv"])
    nseq = a.get("nseq", len(a["cu_q"]))
    return lib.swa_forward(a["q"], a["k"], a["v"], cq, ck, nseq, a["t_q"], a["t_kv"], a["n"],
                           a["d"], a["dtype"], a["scale"], a["pre"], a["nxt"], a["mode"],
                           a["out"], a["smax"], a["ssum"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), swa.SWA_ERR_NULLPTR, "NULL"),
    (dict(ws=None), swa.SWA_ERR_NULLPTR, "NULL"),
    (dict(mode=1), swa.SWA_ERR_INVALID, "The sparse_mode value should be 0, 2, 3 or 4, but got 1"),
    (dict(mode=5), swa.SWA_ERR_INVALID, "should be 0, 2, 3 or 4"),
    (dict(mode=8), swa.SWA_ERR_INVALID, "should be 0, 2, 3 or 4"),
    (dict(nseq=0), swa.SWA_ERR_INVALID, "num_seqs"),
    (dict(t_q=0), swa.SWA_ERR_INVALID, "t_q"),
    (dict(t_q=(1 << 20) + 1, cu_q=[16]), swa.SWA_ERR_INVALID, "t_q"),
    (dict(n=257), swa.SWA_ERR_INVALID, "num_heads"),
    (dict(d=769), swa.SWA_ERR_INVALID, "head_dim"),
    (dict(d=96), swa.SWA_ERR_UNSUPPORTED, "head_dim"),
    (dict(dtype=2), swa.SWA_ERR_UNSUPPORTED, "fp16"),
    (dict(dtype=7), swa.SWA_ERR_INVALID, "dtype"),
    (dict(scale=float("nan")), swa.SWA_ERR_INVALID, "scale"),
    (dict(cu_q=[8, 4], cu_kv=[8, 4]), swa.SWA_ERR_INVALID, "non-decreasing"),
    (dict(cu_q=[8, 0, 4], cu_kv=[8, 0, 4]), swa.SWA_ERR_INVALID, "trailing"),
    (dict(cu_q=[8, 16], cu_kv=[8, 0]), swa.SWA_ERR_INVALID, "participate"),
    (dict(cu_q=[17], cu_kv=[17]), swa.SWA_ERR_INVALID, "exceeds t_q"),
    (dict(cu_q=[-1], cu_kv=[-1]), swa.SWA_ERR_INVALID, ">= 0"),
    (dict(mode=4, pre=3, nxt=-4), swa.SWA_ERR_INVALID, "pre_tokens + next_tokens"),
    (dict(mode=4, cu_q=[8, 16], cu_kv=[10, 16]), swa.SWA_ERR_UNSUPPORTED, "sparse_mode 4"),
    (dict(ws_bytes=16), swa.SWA_ERR_WORKSPACE, "workspace"),
])
def test_forward_validation_statuses(kw, status, needle):
    assert raw_forward(**kw) == status
    assert needle in swa.swa_last_error()


def raw_forward_ex(**kw):
    """Call swa_forward_ex through ctypes with fake (never dereferenced) pointers;
    only argument combinations that fail validation are used."""
    lib = swa.load_library()
    a = dict(q=1, k=1, v=1, cu_q=[16, 30], cu_kv=[16, 30], t_q=30, t_kv=30, n=4, nkv=2, d=64,
             dtype=1, scale=0.125, pre=INT_MAX, nxt=INT_MAX, mode=0, mask=256,
             mask_bytes=1 << 20, keep=0.9, out=1, smax=1, ssum=1, ws=1, ws_bytes=1 << 30)
    a.update(kw)
    cq = (ctypes.c_int64 * len(a["cu_q"]))(*a["cu_q"])
    ck = (ctypes.c_int64 * len(a["cu_kv"]))(*a["cu_kv"])
    return lib.swa_forward_ex(a["q"], a["k"], a["v"], cq, ck, len(a["cu_q"]), a["t_q"],
                              a["t_kv"], a["n"], a["nkv"], a["d"], a["dtype"], a["scale"],
                              a["pre"], a["nxt"], a["mode"], a["mask"], a["mask_bytes"],
                              a["keep"], a["out"], a["smax"], a["ssum"], a["ws"], a["ws_bytes"],
                              None)


# mask bits: 4 heads x (16*16 + 14*14) = 1808 bits -> 57 words = 228 bytes
@pytest.mark.parametrize("kw,needle", [
    (dict(keep=0.0), "keep_prob"),
    (dict(keep=1.5), "keep_prob"),
    (dict(keep=float("nan")), "keep_prob"),
    (dict(mask=258), "4-byte aligned"),
    (dict(mask_bytes=227), "drop_mask has 227 bytes, needs 228"),
    (dict(nkv=3), "multiple of num_kv_heads"),
    (dict(nkv=0), "multiple of num_kv_heads"),
    (dict(nkv=8), "multiple of num_kv_heads"),
])
def test_extended_call_validation(kw, needle):
    assert raw_forward_ex(**kw) == swa.SWA_ERR_INVALID
    assert needle in swa.swa_last_error()


def test_mode0_accepts_unequal_lengths_and_trailing_batches():
    # only the schedule is built (host); the dump proves validation passed
    rows, _, _ = swa.swa_debug_tile_schedule([5, 9, 0, 0], [7, 8, 0, 0], 9, 8, 64, 1,
                                             INT_MAX, INT_MAX, 0, 0)
    assert rows


@pytest.mark.parametrize("mode", [2, 3])
def test_causal_modes_accept_unequal_lengths_and_ignore_pre_next(mode):
    # the causal modes take Sq != Skv per batch, and pre/next play no part
    a = swa.swa_debug_tile_schedule([5, 900, 0], [70, 300, 0], 900, 300, 64, 1, 3, -50, mode, 0)
    b = swa.swa_debug_tile_schedule([5, 900, 0], [70, 300, 0], 900, 300, 64, 1, 0, 0, mode, 0)
    assert a[0] and a == b


def test_workspace_sizes_monotone_and_backward_holds_only_schedules_and_row_terms():
    f = swa.swa_forward_workspace_size(1, 16384, 16384, 16, 128, 1)
    b = swa.swa_backward_workspace_size(1, 16384, 16384, 16, 128, 1)
    # the schedules and the row terms D and lse2 (fp32 per row and head); no
    # gradient accumulator (the backward has no atomics for either type)
    assert f > 0 and 2 * 16384 * 16 * 4 <= b < 16384 * 16 * 128 * 4
    assert swa.swa_backward_workspace_size(1, 16384, 16384, 16, 128, 0) == b
    assert swa.swa_backward_workspace_size(4, 16384, 16384, 16, 128, 1) >= b
    with pytest.raises(ValueError):
        swa.swa_forward_workspace_size(1, 16, 16, 2, 80, 1)


def compare_schedule(cu_q, cu_kv, mode, pre, nxt, direction):
    t_q = max([c for c in cu_q] + [1])
    t_kv = max([c for c in cu_kv] + [1])
    rows, bi, bt = swa.swa_debug_tile_schedule(cu_q, cu_kv, t_q, t_kv, 128, 1, pre, nxt, mode,
                                               direction)
    got = {}
    order = []
    for seq, blk, tile, kind in rows:
        key = (seq, blk)
        if key not in got:
            got[key] = []
            order.append(key)
        if tile >= 0:
            got[key].append((tile, kind))
    # tiles of one item are listed contiguously and in increasing order
    assert len(order) == len(got)
    for v in got.values():
        assert [t for t, _ in v] == sorted(t for t, _ in v)
    # directions 0 (forward) and 2 (backward dQ) walk query blocks over
    # key tiles, direction 1 (backward dK/dV) key blocks over query tiles
    expect = oracle.enumerate_tiles(cu_q, cu_kv, mode, pre, nxt, bi, bt,
                                    "bwd" if direction == 1 else "fwd")
    # the oracle keys batches by participating index; map to batch index
    seqs = oracle.sequences(cu_q)
    exp = {(b, it): v for (b, it), v in expect.items()}
    assert got == exp
    return got


SCHEDULE_CASES = [
    ([128], [128], 0, INT_MAX, INT_MAX),
    ([1000], [1000], 4, 100, 30),
    ([1, 130, 257, 700, 701], [1, 130, 257, 700, 701], 4, 64, 0),
    ([300, 300, 800], [300, 300, 800], 4, 0, 200),
    ([0, 5, 5, 77], [0, 5, 5, 77], 0, 0, 0),
    ([200, 450, 0, 0], [130, 700, 0, 0], 0, 5, 5),
    ([513], [513], 4, 2048, 0),
    ([1024], [1024], 4, 5, -3),
    ([640], [640], 4, -64, 64),
    ([4096], [4096], 4, 127, 1),
    # causal modes 2 (top-left) and 3 (bottom-right), also with Sq != Skv
    ([1000], [1000], 2, 0, 0),
    ([1000], [1000], 3, 7, 7),
    ([300, 345, 1045, 0], [900, 945, 1205, 0], 2, 0, 0),
    ([300, 345, 1045, 0], [900, 945, 1205, 0], 3, 0, 0),
    ([129, 130, 643], [1, 129, 2000], 3, 0, 0),
    ([2000, 2064], [129, 640], 2, 0, 0),
    ([2000, 2064], [129, 640], 3, 0, 0),
]


@pytest.mark.parametrize("direction", [0, 1, 2])
@pytest.mark.parametrize("case", SCHEDULE_CASES)
def test_schedule_matches_bruteforce_enumeration(case, direction):
    compare_schedule(*case, direction)


@pytest.mark.parametrize("direction", [0, 1, 2])
def test_headline_schedule_skip_pattern(direction):
    p = workloads.make_problem(workloads.HEADLINE)
    got = compare_schedule(p.cu_seqlens_q, p.cu_seqlens_kv, 4, 2048, 0, direction)
    vis = sum(len(v) for v in got.values())
    full = sum(1 for v in got.values() for _, k in v if k == 2)
    # 128-row query blocks: 112 blocks see 2176 keys = 34 tiles of 64, block
    # qb < 16 sees 2 (qb + 1) tiles -> 112 * 34 + 272 = 4080 visited of the
    # 128 * 256 = 32768 tiles (12.45 %); 4 partial tiles per complete-band
    # block (two at each band edge) -> 480 partial.  The backward dK/dV
    # schedule (128-key blocks over 64-row tiles) is the mirror image, and the
    # dQ schedule uses the forward's 128-row blocks.
    assert (vis, full) == (4080, 3600)


def test_schedule_orders_longest_item_first():
    rows, _, _ = swa.swa_debug_tile_schedule([100, 4100], [100, 4100], 4100, 4100, 128, 1,
                                             INT_MAX, INT_MAX, 0, 0)
    counts = []
    last = None
    for seq, blk, tile, kind in rows:
        if (seq, blk) != last:
            counts.append(0)
            last = (seq, blk)
        counts[-1] += 1
    assert counts == sorted(counts, reverse=True)


I64_MAX, I64_MIN = 2**63 - 1, -2**63


@pytest.mark.parametrize("direction", [0, 1, 2])
@pytest.mark.parametrize("pre,nxt,same_as", [
    (I64_MAX, 0, (INT_MAX, 0)),
    (0, I64_MAX, (0, INT_MAX)),
    (I64_MAX, I64_MAX, (INT_MAX, INT_MAX)),
    (I64_MAX, -5, (INT_MAX, -5)),
    (-7, I64_MAX, (-7, INT_MAX)),
    # -pre = I64_MAX: every row is empty, as with -pre = INT_MAX
    (I64_MIN + 1, I64_MAX, (-INT_MAX, INT_MAX)),
])
def test_band_reach_beyond_int32_equals_widest_band(pre, nxt, same_as, direction):
    """pre_tokens / next_tokens are int64 in the interface: a reach of 2^63 - 1
    must schedule exactly what a reach of 2^31 - 1 does (both exceed any
    sequence), with no overflow in the schedule's index arithmetic."""
    cu = [300, 1000]
    got = swa.swa_debug_tile_schedule(cu, cu, 1000, 1000, 128, 1, pre, nxt, 4, direction)
    ref = swa.swa_debug_tile_schedule(cu, cu, 1000, 1000, 128, 1, *same_as, 4, direction)
    assert got == ref


@pytest.mark.parametrize("pre,nxt", [(I64_MAX, I64_MIN), (I64_MIN, I64_MAX), (I64_MIN, 0)])
def test_band_sum_below_zero_is_rejected_without_overflow(pre, nxt):
    # pre + next = -1 (or far below) in exact arithmetic: every row is empty
    assert raw_forward(mode=4, pre=pre, nxt=nxt) == swa.SWA_ERR_INVALID
    assert "pre_tokens + next_tokens" in swa.swa_last_error()
