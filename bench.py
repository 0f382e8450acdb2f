"""Benchmark of the sliding-window FlashAttention hot path on one MI355X.

One step = one forward + one backward pass (all kernels of the path) over the
16K sliding-window workload (B=1, N=16, S=16384, D=128, bf16, sparse_mode 4,
pre_tokens 2048, next_tokens 0) with seeded synthetic inputs resident in HBM.

Metric: effective TFLOP/s of forward + backward counting only unmasked
(query, key) pairs: 4*D flops per pair forward (Q K^T and P V), 10*D per pair
backward (the five products S, dP, dV, dK, dQ; recomputing S is part of the
method; the second recomputation of S and dP by the dQ kernel of the bf16
two-pass backward is not counted).  Also reported: the fraction of the bf16 dense MFMA peak, the
roofline position of the dominant kernel (timed with HIP events on the
launching stream), and the fp64 CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

# MI355X dense bf16 MFMA peak, published; roofline.frac and every pct_* field
# use this one figure (256 CU x 4096 flop/clk x 2.4 GHz = 2516.6 would put
# each percentage 0.66 % lower)
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
_CSRC = "transformer_attention_tnd_amd/csrc/"
_HDRS = tuple(_CSRC + f for f in ("swa_common.hpp", "swa_internal.hpp"))
# each kernel's source file and the headers it is built from (the traffic
# record of a kernel is valid only for the exact text of these files)
KERNEL_SOURCES = {
    "forward": (_CSRC + "swa_fwd.hip",) + _HDRS,
    "backward": (_CSRC + "swa_bwd_kv.hip", _CSRC + "swa_bwd_kv.hpp",
                 _CSRC + "swa_pipe.hpp") + _HDRS,
    "bwd_dq": (_CSRC + "swa_bwd_dq.hip", _CSRC + "swa_pipe.hpp") + _HDRS,
    "bwd_pre": (_CSRC + "swa_bwd.hip",) + _HDRS,
}
# fp32 inputs: the dK/dV and dQ kernels are those of swa_bwd.hip
KERNEL_SOURCES_FP32 = dict(KERNEL_SOURCES, backward=(_CSRC + "swa_bwd.hip",) + _HDRS,
                           bwd_dq=(_CSRC + "swa_bwd.hip",) + _HDRS)
BWD_KERNELS = ("bwd_pre", "backward", "bwd_dq")


def allowed_pairs(cu_q, cu_kv, mode, pre, nxt):
    """Unmasked (query, key) pairs per head, by a per-row closed form."""
    total = 0
    pq = pk = 0
    for cq, ck in zip(cu_q, cu_kv):
        cq, ck = int(cq), int(ck)
        if cq == 0 and pq > 0:
            break
        sq, skv = cq - pq, ck - pk
        pq, pk = cq, ck
        if mode == 0:
            total += sq * skv
        elif mode in (2, 3):  # causal from the top-left / bottom-right corner
            i = np.arange(sq, dtype=np.int64)
            hi = np.minimum(skv - 1, i if mode == 2 else i + skv - sq)
            total += int(np.clip(hi + 1, 0, None).sum())
        else:
            i = np.arange(sq, dtype=np.int64)
            hi = np.minimum(skv - 1, i + nxt)
            lo = np.maximum(0, i - pre)
            total += int(np.clip(hi - lo + 1, 0, None).sum())
    return total


def source_hash(files):
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(kernel, workload, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload, {}).get(kernel)
    if not rec or rec.get("source_sha256_16") != source_hash(sources[kernel]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(p, n_heads_total, pairs_per_head, budget_s=12.0):
    """The fp64 oracle, as it stands, on whole heads of the same workload
    until about budget_s of CPU work has run."""
    import torch

    import oracle
    D = p.head_dim
    t0 = time.perf_counter()
    done = 0
    G = p.q.shape[1] // p.k.shape[1]  # query heads per key/value head
    while done < n_heads_total:
        sl, skv = slice(done, done + 1), slice(done // G, done // G + 1)
        q, dy = (x[:, sl].contiguous() for x in (p.q, p.dy))
        k, v = (x[:, skv].contiguous() for x in (p.k, p.v))
        out, sm, ss = oracle.forward(q, k, v, p.cu_seqlens_q, p.cu_seqlens_kv, p.scale,
                                     p.pre_tokens, p.next_tokens, p.sparse_mode, chunk=256)
        oracle.backward(q, k, v, dy, out, sm, ss, p.cu_seqlens_q, p.cu_seqlens_kv, p.scale,
                        p.pre_tokens, p.next_tokens, p.sparse_mode, chunk=256)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    flops = 14 * D * pairs_per_head * done
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": torch.get_num_threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle forward+backward of heads 0..{done - 1} of {n_heads_total} "
                  f"(all rows, row chunks of 256), {el:.1f} s wall",
        "seconds": el,
        "os_cpu_count": os.cpu_count(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--keep-prob", type=float, default=1.0,
                    help="< 1: dropout with a seeded caller mask of this keep probability")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes "
                         "--steps times (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the attention path of this library runs on a "
              "single device (heads and sequences are independent; a multi-GPU run would "
              "shard them with no communication). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_attention_tnd_amd as swa
    import workloads

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "steps": args.steps}), flush=True)
        return

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    p = workloads.make_problem(name)
    dev = torch.device("cuda:0")
    swa.load_library()
    q, k, v, dy = (x.to(dev) for x in (p.q, p.k, p.v, p.dy))
    T, N, D = q.shape
    nseq = len(p.cu_seqlens_q)
    code = swa.DTYPE_BF16 if q.dtype == torch.bfloat16 else swa.DTYPE_FP32
    out = torch.empty_like(q)
    smax = torch.empty(T, N, 8, dtype=torch.float32, device=dev)
    ssum = torch.empty_like(smax)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_f = torch.empty(swa.swa_forward_workspace_size(nseq, T, k.shape[0], N, D, code),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(swa.swa_backward_workspace_size(nseq, T, k.shape[0], N, D, code),
                       dtype=torch.uint8, device=dev)
    args_common = (p.cu_seqlens_q, p.cu_seqlens_kv, p.scale, p.pre_tokens, p.next_tokens,
                   p.sparse_mode)
    drop = None
    if args.keep_prob < 1.0:
        drop = workloads.make_drop_mask(p, args.keep_prob).to(dev)

    def step():
        swa.swa_forward_ex(q, k, v, *args_common, drop, args.keep_prob, out, smax, ssum, ws_f)
        swa.swa_backward_ex(q, k, v, dy, out, smax, ssum, *args_common, drop, args.keep_prob, dq,
                            dk, dv, ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for kind in swa.KERNEL_KINDS:   # drop anything recorded before
        swa.swa_profile_read(kind)
    swa.swa_profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    swa.swa_profile_enable(False)
    total_ms = e0.elapsed_time(e1)
    kern = {}
    for kind in ("forward",) + BWD_KERNELS:
        ms, n = swa.swa_profile_read(kind)
        if n:
            kern[kind] = {"avg_ms": ms / n, "launches": n}

    pairs = allowed_pairs(p.cu_seqlens_q, p.cu_seqlens_kv, p.sparse_mode, p.pre_tokens,
                          p.next_tokens)
    f_fwd = 4.0 * D * pairs * N
    f_bwd = 10.0 * D * pairs * N
    ms_step = total_ms / args.steps
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    elem = q.element_size()
    # algorithmic work per launch of each kernel
    algo = {
        "forward": ("mfma", f_fwd / 1e12, "TFLOP/s"),
        # the dK/dV kernel does S, dP, dV, dK (8*D per pair), the dQ kernel
        # adds dQ (2*D; its recomputed S and dP are not counted)
        "backward": ("mfma", 0.8 * f_bwd / 1e12, "TFLOP/s"),
        "bwd_dq": ("mfma", 0.2 * f_bwd / 1e12, "TFLOP/s"),
        # fp32, per (token, head): read dY, O and two statistics; write D and lse2
        "bwd_pre": ("hbm", T * N * (2 * D * elem + 8 + 8) / 1e9, "GB/s"),
    }
    algo = {kk: vv for kk, vv in algo.items() if kk in kern}
    for kind, (bound, work, unit) in algo.items():
        kern[kind]["achieved"] = work / (kern[kind]["avg_ms"] * 1e-3)
        kern[kind]["unit"] = unit
        kern[kind]["bound"] = bound
    peak_mfma = PEAK_BF16_TFLOPS if q.dtype == torch.bfloat16 else PEAK_FP32_MATRIX_TFLOPS
    dominant = max(kern, key=lambda kk: kern[kk]["avg_ms"] * kern[kk]["launches"])
    bound, work, unit = algo[dominant]
    peak = peak_mfma if bound == "mfma" else PEAK_HBM_GBS
    achieved = kern[dominant]["achieved"]
    roofline = {"kernel": dominant, "bound": bound, "achieved": achieved, "peak": peak,
                "unit": unit, "frac": achieved / peak,
                "traffic": (traffic_record(dominant, name, KERNEL_SOURCES if q.dtype == torch.bfloat16
                                           else KERNEL_SOURCES_FP32)
                            if drop is None else None),
                "avg_launch_ms": kern[dominant]["avg_ms"]}

    cpu = None
    if not args.no_cpu_baseline and drop is None:  # (the oracle leg runs without dropout)
        cpu = cpu_baseline(p, N, pairs)

    t_f = kern["forward"]["avg_ms"]
    t_b = sum(kern[kk]["avg_ms"] for kk in BWD_KERNELS if kk in kern)
    line = {
        "metric": "effective TFLOP/s fwd+bwd (unmasked FLOPs) and % of bf16 MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if q.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded N(0,std) inputs shaped like the workload)",
        "config": {"workload": name, "tokens": T, "num_heads": N,
                   "num_kv_heads": k.shape[1], "head_dim": D,
                   "sparse_mode": p.sparse_mode, "pre_tokens": p.pre_tokens,
                   "next_tokens": p.next_tokens, "num_seqs": nseq, "keep_prob": args.keep_prob,
                   "cu_seqlens": p.cu_seqlens_q if nseq <= 16 else None},
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "fwd_tflops": f_fwd / (t_f * 1e-3) / 1e12,
        "bwd_tflops": f_bwd / (t_b * 1e-3) / 1e12,
        "fwd_pct_of_peak": 100.0 * f_fwd / (t_f * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "bwd_pct_of_peak": 100.0 * f_bwd / (t_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "unmasked_pairs_per_head": pairs,
        "kernels": kern,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
