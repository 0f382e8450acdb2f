"""Python binding of libswa, the gfx950 sliding-window FlashAttention library.

The functions named ``swa_*`` mirror the C entry points of ``include/swa.h``
one to one; they only marshal arguments (torch tensors -> device pointers,
Python ints -> host int64 arrays, the current torch stream -> hipStream_t).
Every step of the computation runs in the HIP kernels of ``libswa.so``;
there is no fallback: if the library is missing the calls raise.

``forward`` and ``backward`` are conveniences that allocate the outputs and
the workspace with torch and call ``swa_forward_ex`` / ``swa_backward_ex``
(grouped key/value heads when k has fewer heads than q; dropout when a mask
is given).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "INT_MAX", "SwaError", "load_library", "library_path",
    "swa_forward_workspace_size", "swa_backward_workspace_size",
    "swa_forward", "swa_backward", "swa_forward_ex", "swa_backward_ex", "swa_backward_noalloc",
    "swa_last_error", "swa_debug_tile_schedule",
    "swa_schedule_cache_enable", "swa_profile_enable", "swa_profile_read",
    "forward", "backward", "DTYPE_FP32", "DTYPE_BF16", "DTYPE_FP16",
]

INT_MAX = 2147483647
SWA_OK, SWA_ERR_NULLPTR, SWA_ERR_INVALID, SWA_ERR_UNSUPPORTED, SWA_ERR_WORKSPACE, SWA_ERR_HIP = range(6)
DTYPE_FP32, DTYPE_BF16, DTYPE_FP16 = 0, 1, 2
STATUS_NAMES = {0: "SWA_OK", 1: "SWA_ERR_NULLPTR", 2: "SWA_ERR_INVALID",
                3: "SWA_ERR_UNSUPPORTED", 4: "SWA_ERR_WORKSPACE", 5: "SWA_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_szp = ctypes.POINTER(ctypes.c_size_t)

_SIGNATURES = {
    "swa_forward_workspace_size": [_i64, _i64, _i64, _i64, _i64, _i32, _szp],
    "swa_backward_workspace_size": [_i64, _i64, _i64, _i64, _i64, _i32, _szp],
    "swa_forward": [_vp, _vp, _vp, _i64p, _i64p, _i64, _i64, _i64, _i64, _i64, _i32,
                    ctypes.c_double, _i64, _i64, _i64, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    "swa_backward": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64p, _i64, _i64, _i64, _i64,
                     _i64, _i32, ctypes.c_double, _i64, _i64, _i64, _vp, _vp, _vp, _vp,
                     ctypes.c_size_t, _vp],
    "swa_forward_ex": [_vp, _vp, _vp, _i64p, _i64p, _i64, _i64, _i64, _i64, _i64, _i64, _i32,
                       ctypes.c_double, _i64, _i64, _i64, _vp, ctypes.c_size_t, ctypes.c_double,
                       _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    "swa_backward_ex": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64p, _i64, _i64, _i64,
                        _i64, _i64, _i64, _i32, ctypes.c_double, _i64, _i64, _i64, _vp,
                        ctypes.c_size_t, ctypes.c_double, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                        _vp],
    "swa_backward_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64p, _i64p, _i64, _i64, _i64,
                             _i64, _i64, _i64, _i32, ctypes.c_double, _i64, _i64, _i64, _vp,
                             ctypes.c_size_t, ctypes.c_double, _vp, _vp, _vp, _vp],
    "swa_last_error": [],
    "swa_debug_tile_schedule": [_i64p, _i64p, _i64, _i64, _i64, _i64, _i32, _i64, _i64, _i64,
                                _i32, _i32p, _i64, _i64p, _i32p, _i32p],
    "swa_schedule_cache_enable": [_i32],
    "swa_profile_enable": [_i32],
    "swa_profile_read": [_i32, ctypes.POINTER(ctypes.c_double), _i64p],
}

KERNEL_KINDS = {"forward": 0, "bwd_pre": 1, "backward": 2, "fill": 4, "bwd_dq": 5}


class SwaError(RuntimeError):
    """A non-OK status from libswa; ``status`` holds the code."""

    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def library_path():
    return os.environ.get("SWA_LIBRARY", os.path.join(_HERE, "libswa.so"))


def load_library():
    """Load libswa.so (built in-tree by ``build.py``); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"libswa.so not found at {path}; run __graft_entry__.build() "
                          "or python transformer_attention_tnd_amd/build.py")
    lib = ctypes.CDLL(path)
    for name, argtypes in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name == "swa_last_error" else ctypes.c_int
    _lib = lib
    return lib


def swa_last_error():
    return load_library().swa_last_error().decode()


def _check(status):
    if status != SWA_OK:
        msg = swa_last_error()
        if status == SWA_ERR_HIP:
            raise SwaError(status, msg)
        err = SwaError(status, msg)
        raise ValueError(str(err)) from err


def _cu_array(cu):
    vals = [int(x) for x in (cu.tolist() if hasattr(cu, "tolist") else cu)]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals), len(vals)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return DTYPE_FP32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float16:
        return DTYPE_FP16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(t, stream):
    import torch
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def swa_forward_workspace_size(num_seqs, t_q, t_kv, num_heads, head_dim, dtype):
    out = ctypes.c_size_t(0)
    _check(load_library().swa_forward_workspace_size(num_seqs, t_q, t_kv, num_heads, head_dim,
                                                     dtype, ctypes.byref(out)))
    return out.value


def swa_backward_workspace_size(num_seqs, t_q, t_kv, num_heads, head_dim, dtype):
    out = ctypes.c_size_t(0)
    _check(load_library().swa_backward_workspace_size(num_seqs, t_q, t_kv, num_heads, head_dim,
                                                      dtype, ctypes.byref(out)))
    return out.value


def _shape_checks(q, k, v, extra_q=(), extra_kv=(), grouped=False):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be TND tensors [T, N, D]")
    heads_ok = (q.shape[1] % k.shape[1] == 0) if grouped else q.shape[1] == k.shape[1]
    if k.shape != v.shape or q.shape[2] != k.shape[2] or not heads_ok:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    for t in (q, k, v, *extra_q, *extra_kv):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dtype != q.dtype:
            raise ValueError("all element tensors must share one dtype")
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    for t in extra_q:
        if t.shape != q.shape:
            raise ValueError(f"expected shape {tuple(q.shape)}, got {tuple(t.shape)}")
    for t in extra_kv:
        if t.shape != k.shape:
            raise ValueError(f"expected shape {tuple(k.shape)}, got {tuple(t.shape)}")


def _stats_check(q, *stats):
    import torch
    for s in stats:
        if s.dtype != torch.float32 or tuple(s.shape) != (q.shape[0], q.shape[1], 8) or \
                not s.is_contiguous() or s.device != q.device:
            raise ValueError("softmax statistics must be contiguous float32 [T, N, 8] "
                             "on the device of q")


def swa_forward(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, pre_tokens, next_tokens,
                sparse_mode, out, softmax_max, softmax_sum, workspace, stream=None):
    """Marshal to the C entry point swa_forward (asynchronous on the stream)."""
    _shape_checks(q, k, v, extra_q=(out,))
    _stats_check(q, softmax_max, softmax_sum)
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_kv)
    if nq != nk:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
    _check(load_library().swa_forward(
        _ptr(q), _ptr(k), _ptr(v), cq, ck, nq, q.shape[0], k.shape[0], q.shape[1], q.shape[2],
        _dtype_code(q), float(scale), int(pre_tokens), int(next_tokens), int(sparse_mode),
        _ptr(out), _ptr(softmax_max), _ptr(softmax_sum), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q, stream)))


def swa_backward(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv,
                 scale, pre_tokens, next_tokens, sparse_mode, dq, dk, dv, workspace,
                 stream=None):
    """Marshal to the C entry point swa_backward (asynchronous on the stream)."""
    _shape_checks(q, k, v, extra_q=(dy, out, dq), extra_kv=(dk, dv))
    _stats_check(q, softmax_max, softmax_sum)
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_kv)
    if nq != nk:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
    _check(load_library().swa_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dy), _ptr(out), _ptr(softmax_max), _ptr(softmax_sum),
        cq, ck, nq, q.shape[0], k.shape[0], q.shape[1], q.shape[2], _dtype_code(q), float(scale),
        int(pre_tokens), int(next_tokens), int(sparse_mode), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q, stream)))


def _mask_args(drop_mask, keep_prob, device):
    import torch
    if drop_mask is None:
        return None, 0, 1.0
    if drop_mask.dtype != torch.uint8 or not drop_mask.is_contiguous() or \
            drop_mask.device != device:
        raise ValueError("drop_mask must be a contiguous uint8 tensor on the device of q")
    return _ptr(drop_mask), drop_mask.numel(), float(keep_prob)


def swa_forward_ex(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, pre_tokens, next_tokens,
                   sparse_mode, drop_mask, keep_prob, out, softmax_max, softmax_sum, workspace,
                   stream=None):
    """Marshal to swa_forward_ex: k and v may have fewer heads than q (a
    divisor); drop_mask (packed uint8 keep bits, or None) applies dropout."""
    _shape_checks(q, k, v, extra_q=(out,), grouped=True)
    _stats_check(q, softmax_max, softmax_sum)
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_kv)
    if nq != nk:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
    mp, mb, kp = _mask_args(drop_mask, keep_prob, q.device)
    _check(load_library().swa_forward_ex(
        _ptr(q), _ptr(k), _ptr(v), cq, ck, nq, q.shape[0], k.shape[0], q.shape[1], k.shape[1],
        q.shape[2], _dtype_code(q), float(scale), int(pre_tokens), int(next_tokens),
        int(sparse_mode), mp, mb, kp, _ptr(out), _ptr(softmax_max), _ptr(softmax_sum),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q, stream)))


def swa_backward_ex(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv,
                    scale, pre_tokens, next_tokens, sparse_mode, drop_mask, keep_prob, dq, dk,
                    dv, workspace, stream=None):
    """Marshal to swa_backward_ex: k, v, dk, dv may have fewer heads than q;
    drop_mask / keep_prob as in the forward call."""
    _shape_checks(q, k, v, extra_q=(dy, out, dq), extra_kv=(dk, dv), grouped=True)
    _stats_check(q, softmax_max, softmax_sum)
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_kv)
    if nq != nk:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
    mp, mb, kp = _mask_args(drop_mask, keep_prob, q.device)
    _check(load_library().swa_backward_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dy), _ptr(out), _ptr(softmax_max), _ptr(softmax_sum),
        cq, ck, nq, q.shape[0], k.shape[0], q.shape[1], k.shape[1], q.shape[2], _dtype_code(q),
        float(scale), int(pre_tokens), int(next_tokens), int(sparse_mode), mp, mb, kp, _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q, stream)))


def swa_backward_noalloc(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q,
                         cu_seqlens_kv, scale, pre_tokens, next_tokens, sparse_mode, drop_mask,
                         keep_prob, dq, dk, dv, stream=None):
    """Marshal to swa_backward_noalloc: swa_backward_ex without a workspace
    (the library's fixed per-device scratch is used; nothing is allocated)."""
    _shape_checks(q, k, v, extra_q=(dy, out, dq), extra_kv=(dk, dv), grouped=True)
    _stats_check(q, softmax_max, softmax_sum)
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_kv)
    if nq != nk:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
    mp, mb, kp = _mask_args(drop_mask, keep_prob, q.device)
    _check(load_library().swa_backward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dy), _ptr(out), _ptr(softmax_max), _ptr(softmax_sum),
        cq, ck, nq, q.shape[0], k.shape[0], q.shape[1], k.shape[1], q.shape[2], _dtype_code(q),
        float(scale), int(pre_tokens), int(next_tokens), int(sparse_mode), mp, mb, kp, _ptr(dq),
        _ptr(dk), _ptr(dv), _stream(q, stream)))


def swa_debug_tile_schedule(cu_seqlens_q, cu_seqlens_kv, t_q, t_kv, head_dim, dtype,
                            pre_tokens, next_tokens, sparse_mode, direction):
    """Host-only schedule dump: (rows [n, 4] as a list of tuples, block_item, block_tile)."""
    lib = load_library()
    cq, nq = _cu_array(cu_seqlens_q)
    ck, _ = _cu_array(cu_seqlens_kv)
    n = ctypes.c_int64(0)
    bi, bt = ctypes.c_int32(0), ctypes.c_int32(0)
    args = [cq, ck, nq, t_q, t_kv, head_dim, dtype, int(pre_tokens), int(next_tokens),
            int(sparse_mode), direction]
    _check(lib.swa_debug_tile_schedule(*args, None, 0, ctypes.byref(n), ctypes.byref(bi),
                                       ctypes.byref(bt)))
    buf = (ctypes.c_int32 * max(4, 4 * n.value))()
    _check(lib.swa_debug_tile_schedule(*args, buf, n.value, ctypes.byref(n), ctypes.byref(bi),
                                       ctypes.byref(bt)))
    rows = [tuple(buf[4 * i:4 * i + 4]) for i in range(n.value)]
    return rows, bi.value, bt.value


def swa_schedule_cache_enable(enable=True):
    """Turn the library's device cache of tile schedules on or off (off frees it)."""
    _check(load_library().swa_schedule_cache_enable(1 if enable else 0))


def swa_profile_enable(enable=True):
    _check(load_library().swa_profile_enable(1 if enable else 0))


def swa_profile_read(kernel):
    """(total_ms, launches) of completed launches of one kernel kind (name or id)."""
    kid = KERNEL_KINDS[kernel] if isinstance(kernel, str) else int(kernel)
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    _check(load_library().swa_profile_read(kid, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def _workspace(nbytes, device):
    import torch
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def forward(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, pre_tokens=INT_MAX,
            next_tokens=INT_MAX, sparse_mode=0, workspace=None, drop_mask=None, keep_prob=1.0):
    """Allocate (out, softmax_max, softmax_sum) and run swa_forward_ex (k / v may
    have fewer heads than q; drop_mask applies dropout)."""
    import torch
    out = torch.empty_like(q)
    smax = torch.empty(q.shape[0], q.shape[1], 8, dtype=torch.float32, device=q.device)
    ssum = torch.empty_like(smax)
    if workspace is None:
        nbytes = swa_forward_workspace_size(len(cu_seqlens_q), q.shape[0], k.shape[0],
                                            q.shape[1], q.shape[2], _dtype_code(q))
        workspace = _workspace(nbytes, q.device)
    swa_forward_ex(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, pre_tokens, next_tokens,
                   sparse_mode, drop_mask, keep_prob, out, smax, ssum, workspace)
    return out, smax, ssum


def backward(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, scale,
             pre_tokens=INT_MAX, next_tokens=INT_MAX, sparse_mode=0, workspace=None,
             drop_mask=None, keep_prob=1.0):
    """Allocate (dq, dk, dv) and run swa_backward_ex (k / v may have fewer heads
    than q; drop_mask / keep_prob as in the forward call)."""
    import torch
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nbytes = swa_backward_workspace_size(len(cu_seqlens_q), q.shape[0], k.shape[0],
                                             q.shape[1], q.shape[2], _dtype_code(q))
        workspace = _workspace(nbytes, q.device)
    swa_backward_ex(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv,
                    scale, pre_tokens, next_tokens, sparse_mode, drop_mask, keep_prob, dq, dk,
                    dv, workspace)
    return dq, dk, dv
