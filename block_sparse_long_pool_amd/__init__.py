"""MoBA (Mixture of Block Attention) on MI355X (gfx950): thin Python binding over
libmoba.so (prefill forward and backward, packed sequences, dense and decode paths).

Every step of the path runs in the library's HIP kernels; this module only checks
tensor arguments, allocates outputs and the workspace with torch, and passes raw
device pointers and torch's current HIP stream through ctypes.  If libmoba.so is
missing the import fails loudly: there is no CPU fallback.

    out, lse, idx = forward(q, k, v, block=4096, topk=12)

q [b, T, Hq, d], k and v [b, T, Hkv, d] bfloat16 on the GPU; out like q (bf16),
lse [b, Hq, T] float32 (natural log), idx [b, Hq, T, topk] int32 (ascending selected
blocks, -1 padded).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LIB_PATH", "MobaError", "check_args", "workspace_bytes", "forward",
    "pool_centroids", "gate_topk", "index_entries", "build_index", "strerror",
    "stage_workspace_bytes", "lib", "STAGES", "alloc_workspace", "dense_forward", "attention",
    "backward", "backward_workspace_bytes", "forward_varlen", "varlen_workspace_bytes",
    "key_short_conv", "backward_varlen", "backward_varlen_workspace_bytes", "decode",
    "decode_workspace_bytes", "forward_noalloc", "history_partials", "current_merge",
    "part_dim_order",
]

# names of the steps timed by profile=True, in the library's order
STAGES = ("pool", "gate", "index", "history", "current")

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoba.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python block_sparse_long_pool_amd/build.py` "
        "(hipcc --offload-arch=gfx950).  There is no fallback implementation.")

lib = ctypes.CDLL(LIB_PATH)

_i, _f, _vp, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "moba_check_args": (_i, [_i, _i, _i, _i, _i, _i, _i, _f]),
    "moba_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "moba_forward": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp,
                          _vp, _sz, _vp]),
    "moba_forward_noalloc": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                  _vp, _vp]),
    "moba_forward_profile": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp,
                                  _vp, _vp, _sz, _vp, ctypes.POINTER(_f)]),
    "moba_forward_timed": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp,
                                _vp, _sz, _vp, ctypes.POINTER(_vp)]),
    "moba_dense_forward": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp]),
    "moba_backward_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "moba_key_short_conv": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "moba_backward_varlen_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i,
                                                   ctypes.POINTER(_sz)]),
    "moba_backward_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                  _i, _i, _i, _f, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moba_varlen_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i,
                                          ctypes.POINTER(_sz)]),
    "moba_forward_varlen": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp,
                                 _vp, _vp, _vp, _sz, _vp]),
    "moba_backward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                           _vp, _vp, _vp, _vp, _sz, _vp]),
    "moba_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moba_decode": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _vp]),
    "moba_strerror": (ctypes.c_char_p, [_i]),
    "moba_stage_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "moba_pool_centroids": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "moba_gate_topk": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "moba_index_entries": (ctypes.c_int64, [_i, _i, _i, _i, _i, _i, _i]),
    "moba_build_index": (_i, [_vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _sz,
                              _vp]),
    "moba_history_partials": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp,
                                   _vp, ctypes.c_uint32, _vp, _vp, _vp, _sz, _vp]),
    "moba_current_merge": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp,
                                _vp, _vp, _vp, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

MOBA_OK, MOBA_ERR_INVALID_ARG, MOBA_ERR_UNSUPPORTED, MOBA_ERR_WORKSPACE, MOBA_ERR_HIP = (
    0, -1, -2, -3, -4)


class MobaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def strerror(status: int) -> str:
    return lib.moba_strerror(int(status)).decode()


def _raise(status: int, where: str):
    if status == MOBA_ERR_INVALID_ARG or status == MOBA_ERR_UNSUPPORTED:
        raise ValueError(f"{where}: {strerror(status)} (status {status})")
    if status != MOBA_OK:
        raise MobaError(status, where)


def check_args(batch, seqlen, hq, hkv, head_dim, block, topk, scale) -> int:
    """Host-only shape check; returns the status code."""
    return lib.moba_check_args(batch, seqlen, hq, hkv, head_dim, block, topk, float(scale))


def workspace_bytes(batch, seqlen, hq, hkv, head_dim, block, topk):
    """(bytes for all kv-heads in one pass, bytes for one kv-head per pass)."""
    mn = ctypes.c_size_t(0)
    full = lib.moba_workspace_bytes(batch, seqlen, hq, hkv, head_dim, block, topk,
                                    ctypes.byref(mn))
    return int(full), int(mn.value)


def stage_workspace_bytes(batch, seqlen, hq, hkv, head_dim, block, topk) -> int:
    return int(lib.moba_stage_workspace_bytes(batch, seqlen, hq, hkv, head_dim, block, topk))


def index_entries(batch, seqlen, hq, hkv, block, topk, kv_count) -> int:
    return int(lib.moba_index_entries(batch, seqlen, hq, hkv, block, topk, kv_count))


# ----------------------------------------------------------------------------- torch
def _torch():
    import torch
    return torch


def _stream_ptr():
    return _torch().cuda.current_stream().cuda_stream


def _need(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _one_device(*tensors):
    """Every tensor argument of a call lives on the first one's device."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t is not None and t.device != dev:
            raise ValueError(f"all tensors must be on {dev} (got one on {t.device})")


def _alloc_workspace(nbytes, device):
    torch = _torch()
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def alloc_workspace(q, k, block: int, topk: int, max_workspace_bytes: int | None = None):
    """A uint8 workspace tensor for these inputs: the all-heads-at-once size, reduced
    towards the one-kv-head size when it exceeds ``max_workspace_bytes`` (default: 60%
    of free device memory)."""
    torch = _torch()
    b, T, hq, d = q.shape
    hkv = k.shape[2]
    full, mn = workspace_bytes(b, T, hq, hkv, d, block, topk)
    if full == 0:
        _raise(MOBA_ERR_UNSUPPORTED, "moba_workspace_bytes")
    if max_workspace_bytes is None:
        free, _ = torch.cuda.mem_get_info(q.device)
        max_workspace_bytes = int(0.6 * free)
    size = full if full <= max_workspace_bytes else max(mn, max_workspace_bytes)
    return _alloc_workspace(size, q.device)


def forward(q, k, v, block: int, topk: int, scale: float | None = None, workspace=None,
            max_workspace_bytes: int | None = None, out=None, lse=None, idx=None,
            profile: bool = False, events=None):
    """MoBA prefill forward.  Returns (out bf16, lse fp32, idx int32), and with
    ``profile=True`` also a dict of per-step GPU milliseconds (HIP events on the
    current stream; the call then synchronises).  ``events``: len(STAGES) + 1
    torch.cuda.Event(enable_timing=True), each recorded once before (so that its HIP
    event exists); the library records them at the step boundaries on the current
    stream without synchronising.

    Outputs and the workspace are allocated with torch unless given."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    b, T, hq, d = q.shape
    if k.shape[0] != b or k.shape[1] != T or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    hkv = k.shape[2]
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _raise(check_args(b, T, hq, hkv, d, block, topk, scale), "moba_forward")
    if workspace is None:
        workspace = alloc_workspace(q, k, block, topk, max_workspace_bytes)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((b, hq, T), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((b, hq, T, topk), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(idx, "idx", torch.int32, 4)
    if out.shape != q.shape or lse.shape != (b, hq, T) or idx.shape != (b, hq, T, topk):
        raise ValueError("output shapes do not match the inputs")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), b, T, hq, hkv, d, block, topk,
            float(scale), out.data_ptr(), lse.data_ptr(), idx.data_ptr(),
            workspace.data_ptr(), workspace.numel(), _stream_ptr())
    _one_device(q, k, v, out, lse, idx, workspace)
    with torch.cuda.device(q.device):
        if profile:
            ms = (ctypes.c_float * len(STAGES))()
            st = lib.moba_forward_profile(*args, ms)
        elif events is not None:
            if len(events) != len(STAGES) + 1:
                raise ValueError(f"events: need {len(STAGES) + 1} events")
            handles = (_vp * len(events))(*[e.cuda_event for e in events])
            st = lib.moba_forward_timed(*args, handles)
        else:
            st = lib.moba_forward(*args)
    _raise(st, "moba_forward")
    if profile:
        return out, lse, idx, dict(zip(STAGES, (float(x) for x in ms)))
    return out, lse, idx


def forward_noalloc(q, k, v, block: int, topk: int, scale: float | None = None, out=None,
                    lse=None, idx=None):
    """``forward`` through moba_forward_noalloc: the library uses its own fixed 128 MiB
    device scratch (one per GPU) instead of a workspace, and allocates nothing.  Raises
    MobaError when one kv-head's workspace would exceed that scratch.  Outputs are
    allocated here with torch unless given."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    b, T, hq, d = q.shape
    if k.shape[0] != b or k.shape[1] != T or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _raise(check_args(b, T, hq, hkv, d, block, topk, scale), "moba_forward_noalloc")
    out = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((b, hq, T), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((b, hq, T, topk), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(idx, "idx", torch.int32, 4)
    if out.shape != q.shape or lse.shape != (b, hq, T) or idx.shape != (b, hq, T, topk):
        raise ValueError("output shapes do not match the inputs")
    _one_device(q, k, v, out, lse, idx)
    with torch.cuda.device(q.device):
        st = lib.moba_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, T, hq, hkv,
                                      d, block, topk, float(scale), out.data_ptr(),
                                      lse.data_ptr(), idx.data_ptr(), _stream_ptr())
    _raise(st, "moba_forward_noalloc")
    return out, lse, idx


def dense_forward(q, k, v, scale: float | None = None, out=None, lse=None):
    """Dense causal attention through the library (the full-attention layers of a
    hybrid model).  Returns (out bf16 [b,T,Hq,d], lse fp32 [b,Hq,T])."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    b, T, hq, d = q.shape
    if k.shape[0] != b or k.shape[1] != T or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((b, hq, T), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    if out.shape != q.shape or lse.shape != (b, hq, T):
        raise ValueError("output shapes do not match the inputs")
    _one_device(q, k, v, out, lse)
    with torch.cuda.device(q.device):
        st = lib.moba_dense_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, T, hq, hkv,
                                    d, float(scale), out.data_ptr(), lse.data_ptr(),
                                    _stream_ptr())
    _raise(st, "moba_dense_forward")
    return out, lse


def decode_workspace_bytes(batch, n_new, kv_len, hq, hkv, head_dim) -> int:
    """Workspace bytes of ``decode`` (0 when the shape is not supported)."""
    return int(lib.moba_decode_workspace_bytes(batch, n_new, kv_len, hq, hkv, head_dim))


def decode(q, k, v, scale: float | None = None, workspace=None, out=None, lse=None):
    """Full-attention decode after a prefill (the hand-off from a MoBA prefill to
    generation).  q [b, n_new, Hq, d] holds the new tokens, which are the last n_new
    positions of the cache k, v [b, kv_len, Hkv, d] (bf16); new token i attends keys
    0 .. kv_len - n_new + i.  Returns (out bf16 [b, n_new, Hq, d], lse fp32
    [b, Hq, n_new])."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    b, n, hq, d = q.shape
    Tk, hkv = k.shape[1], k.shape[2]
    if k.shape[0] != b or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        nbytes = decode_workspace_bytes(b, n, Tk, hq, hkv, d)
        if nbytes == 0:
            _raise(MOBA_ERR_UNSUPPORTED if hq % hkv == 0 and 1 <= n <= Tk
                   else MOBA_ERR_INVALID_ARG, "moba_decode_workspace_bytes")
        workspace = _alloc_workspace(nbytes, q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((b, hq, n), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    if out.shape != q.shape or lse.shape != (b, hq, n):
        raise ValueError("output shapes do not match the inputs")
    _one_device(q, k, v, out, lse, workspace)
    with torch.cuda.device(q.device):
        st = lib.moba_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, n, Tk, hq, hkv, d,
                             float(scale), out.data_ptr(), lse.data_ptr(),
                             workspace.data_ptr(), workspace.numel(), _stream_ptr())
    _raise(st, "moba_decode")
    return out, lse


def varlen_workspace_bytes(nseq, total, max_seqlen, hq, hkv, head_dim, block, topk):
    """(all-kv-heads size, one-kv-head size) of the packed-sequence workspace; (0, 0)
    when unsupported."""
    mn = _sz(0)
    full = lib.moba_varlen_workspace_bytes(nseq, total, max_seqlen, hq, hkv, head_dim, block,
                                           topk, ctypes.byref(mn))
    return int(full), int(mn.value)


def forward_varlen(q, k, v, cu_seqlens, block: int, topk: int, scale: float | None = None,
                   workspace=None, max_workspace_bytes: int | None = None, out=None,
                   lse=None, idx=None):
    """MoBA prefill over packed sequences of different lengths, each with its own block
    grid.  q [total, Hq, d], k and v [total, Hkv, d] bf16 on the GPU; cu_seqlens: the
    cumulative lengths [nseq + 1] (int, any device), checked here on the host.
    Returns (out [total, Hq, d] bf16, lse [Hq, total] fp32, idx [Hq, total, topk] int32,
    block ids counted within each sequence).  The call copies cu_seqlens to the device,
    so unlike ``forward`` it is not meant for graph capture."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    total, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape[0] != total or k.shape[2] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    cu_host = torch.as_tensor(cu_seqlens).to("cpu", torch.int64)
    if cu_host.dim() != 1 or cu_host.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with at least 2 entries")
    lens = cu_host[1:] - cu_host[:-1]
    if int(cu_host[0]) != 0 or int(cu_host[-1]) != total or bool((lens < 0).any()):
        raise ValueError("cu_seqlens must start at 0, not decrease and end at q.shape[0]")
    nseq = cu_host.numel() - 1
    max_seqlen = max(1, int(lens.max()))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        full, mn = varlen_workspace_bytes(nseq, total, max_seqlen, hq, hkv, d, block, topk)
        if full == 0:
            _raise(MOBA_ERR_UNSUPPORTED, "moba_varlen_workspace_bytes")
        if max_workspace_bytes is None:
            free, _ = torch.cuda.mem_get_info(q.device)
            max_workspace_bytes = int(0.6 * free)
        workspace = _alloc_workspace(full if full <= max_workspace_bytes
                                     else max(mn, max_workspace_bytes), q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    cu_dev = cu_host.to(device=q.device, dtype=torch.int32)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((hq, total), dtype=torch.float32, device=q.device) if lse is None else lse
    if idx is None:
        idx = torch.empty((hq, total, topk), dtype=torch.int32, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    _need(idx, "idx", torch.int32, 3)
    if out.shape != q.shape or lse.shape != (hq, total) or idx.shape != (hq, total, topk):
        raise ValueError("output shapes do not match the inputs")
    _one_device(q, k, v, out, lse, idx, workspace)
    with torch.cuda.device(q.device):
        st = lib.moba_forward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     cu_dev.data_ptr(), nseq, total, max_seqlen, hq, hkv, d,
                                     block, topk, float(scale), out.data_ptr(),
                                     lse.data_ptr(), idx.data_ptr(), workspace.data_ptr(),
                                     workspace.numel(), _stream_ptr())
    _raise(st, "moba_forward_varlen")
    return out, lse, idx


def key_short_conv(k, weight, block: int, cu_seqlens=None, out=None):
    """Short depthwise causal convolution of the keys within blocks.  k [b, T, Hkv, d]
    (or packed [total, Hkv, d] with cu_seqlens) bf16 on the GPU, weight [Hkv, d, width]
    float32 on the GPU (width <= 8).  Returns the convolved keys, bf16, like k."""
    torch = _torch()
    packed = cu_seqlens is not None
    _need(k, "k", torch.bfloat16, 3 if packed else 4)
    _need(weight, "weight", torch.float32, 3)
    hkv, d = k.shape[-2], k.shape[-1]
    if weight.shape[0] != hkv or weight.shape[1] != d:
        raise ValueError(f"weight must be [{hkv}, {d}, width] (got {tuple(weight.shape)})")
    if packed:
        cu_host = torch.as_tensor(cu_seqlens).to("cpu", torch.int64)
        lens = cu_host[1:] - cu_host[:-1]
        if (cu_host.dim() != 1 or cu_host.numel() < 2 or int(cu_host[0]) != 0
                or int(cu_host[-1]) != k.shape[0] or bool((lens < 0).any())):
            raise ValueError("cu_seqlens must start at 0, not decrease and end at k.shape[0]")
        batch, seqlen, total = cu_host.numel() - 1, max(1, int(lens.max())), k.shape[0]
        cu_dev = cu_host.to(device=k.device, dtype=torch.int32)
        cu_ptr = cu_dev.data_ptr()
    else:
        batch, seqlen, total = k.shape[0], k.shape[1], 0
        cu_ptr = None
    out = torch.empty_like(k) if out is None else out
    _need(out, "out", torch.bfloat16, k.dim())
    if out.shape != k.shape:
        raise ValueError("out must have the shape of k")
    with torch.cuda.device(k.device):
        st = lib.moba_key_short_conv(k.data_ptr(), weight.data_ptr(), cu_ptr, batch, seqlen,
                                     total, hkv, d, block, weight.shape[2], out.data_ptr(),
                                     _stream_ptr())
    _raise(st, "moba_key_short_conv")
    return out


def _cu_host(cu_seqlens, total):
    torch = _torch()
    cu_host = torch.as_tensor(cu_seqlens).to("cpu", torch.int64)
    if cu_host.dim() != 1 or cu_host.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with at least 2 entries")
    lens = cu_host[1:] - cu_host[:-1]
    if int(cu_host[0]) != 0 or int(cu_host[-1]) != total or bool((lens < 0).any()):
        raise ValueError("cu_seqlens must start at 0, not decrease and end at the token count")
    return cu_host, cu_host.numel() - 1, max(1, int(lens.max()))


def backward_varlen_workspace_bytes(nseq, total, max_seqlen, hq, hkv, head_dim, block, topk):
    """(all-kv-heads size, one-kv-head size) of the packed-sequence backward workspace."""
    mn = _sz(0)
    full = lib.moba_backward_varlen_workspace_bytes(nseq, total, max_seqlen, hq, hkv, head_dim,
                                                    block, topk, ctypes.byref(mn))
    return int(full), int(mn.value)


def backward_varlen(q, k, v, out, lse, idx, dout, cu_seqlens, block: int, topk: int,
                    scale: float | None = None, workspace=None,
                    max_workspace_bytes: int | None = None):
    """Gradients of ``forward_varlen`` with its selection ``idx`` held fixed.  Packed
    layouts as ``forward_varlen``; returns (dq, dk, dv) bf16 like q, k, v."""
    torch = _torch()
    for t, nme in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, nme, torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    _need(idx, "idx", torch.int32, 3)
    total, hq, d = q.shape
    hkv = k.shape[1]
    if (k.shape[0] != total or k.shape[2] != d or v.shape != k.shape or out.shape != q.shape
            or dout.shape != q.shape or lse.shape != (hq, total)
            or idx.shape != (hq, total, topk)):
        raise ValueError("shape mismatch between q, k, v, out, lse, idx, dout")
    cu_host, nseq, max_seqlen = _cu_host(cu_seqlens, total)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        full, mn = backward_varlen_workspace_bytes(nseq, total, max_seqlen, hq, hkv, d, block,
                                                   topk)
        if full == 0:
            _raise(MOBA_ERR_UNSUPPORTED, "moba_backward_varlen_workspace_bytes")
        if max_workspace_bytes is None:
            free, _ = torch.cuda.mem_get_info(q.device)
            max_workspace_bytes = int(0.6 * free)
        workspace = _alloc_workspace(full if full <= max_workspace_bytes
                                     else max(mn, max_workspace_bytes), q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    cu_dev = cu_host.to(device=q.device, dtype=torch.int32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _one_device(q, k, v, out, lse, idx, dout, workspace)
    with torch.cuda.device(q.device):
        st = lib.moba_backward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      lse.data_ptr(), idx.data_ptr(), dout.data_ptr(),
                                      cu_dev.data_ptr(), nseq, total, max_seqlen, hq, hkv, d,
                                      block, topk, float(scale), dq.data_ptr(), dk.data_ptr(),
                                      dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                      _stream_ptr())
    _raise(st, "moba_backward_varlen")
    return dq, dk, dv


def backward_workspace_bytes(batch, seqlen, hq, hkv, head_dim, block, topk):
    """(all-kv-heads size, one-kv-head size) of the backward workspace; (0, 0) when the
    backward does not support the shape."""
    mn = _sz(0)
    full = lib.moba_backward_workspace_bytes(batch, seqlen, hq, hkv, head_dim, block, topk,
                                             ctypes.byref(mn))
    return int(full), int(mn.value)


def backward(q, k, v, out, lse, idx, dout, block: int, topk: int, scale: float | None = None,
             workspace=None, max_workspace_bytes: int | None = None, dq=None, dk=None,
             dv=None):
    """Gradients of ``forward`` with its block selection ``idx`` held fixed.  q, k, v,
    out, lse, idx as given to / returned by ``forward``; dout like out.  Returns
    (dq like q, dk like k, dv like v), bf16."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(idx, "idx", torch.int32, 4)
    b, T, hq, d = q.shape
    hkv = k.shape[2]
    if (k.shape[0] != b or k.shape[1] != T or k.shape[3] != d or v.shape != k.shape
            or out.shape != q.shape or dout.shape != q.shape or lse.shape != (b, hq, T)
            or idx.shape != (b, hq, T, topk)):
        raise ValueError("shape mismatch between q, k, v, out, lse, idx, dout")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _raise(check_args(b, T, hq, hkv, d, block, topk, scale), "moba_backward")
    if workspace is None:
        full, mn = backward_workspace_bytes(b, T, hq, hkv, d, block, topk)
        if full == 0:
            _raise(MOBA_ERR_UNSUPPORTED, "moba_backward_workspace_bytes")
        if max_workspace_bytes is None:
            free, _ = torch.cuda.mem_get_info(q.device)
            max_workspace_bytes = int(0.6 * free)
        workspace = _alloc_workspace(full if full <= max_workspace_bytes
                                     else max(mn, max_workspace_bytes), q.device)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, 4)
    _need(dk, "dk", torch.bfloat16, 4)
    _need(dv, "dv", torch.bfloat16, 4)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("gradient shapes do not match the inputs")
    _one_device(q, k, v, out, lse, idx, dout, workspace)
    with torch.cuda.device(q.device):
        st = lib.moba_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), idx.data_ptr(), dout.data_ptr(), b, T, hq, hkv,
                               d, block, topk, float(scale), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                               _stream_ptr())
    _raise(st, "moba_backward")
    return dq, dk, dv


def attention(q, k, v, block: int, topk: int, scale: float | None = None, dense: bool = False,
              **kw):
    """One attention layer of a hybrid model: MoBA (returns out, lse, idx) or, with
    ``dense=True``, full causal attention (returns out, lse, None)."""
    if dense:
        out, lse = dense_forward(q, k, v, scale, kw.get("out"), kw.get("lse"))
        return out, lse, None
    return forward(q, k, v, block, topk, scale, **kw)


def pool_centroids(k, block: int):
    """Centroid mean-pool stage: float32 [b, Hkv, nb, d]."""
    torch = _torch()
    _need(k, "k", torch.bfloat16, 4)
    b, T, hkv, d = k.shape
    _raise(check_args(b, T, hkv, hkv, d, block, 1, 1.0), "moba_pool_centroids")
    ws = _alloc_workspace(stage_workspace_bytes(b, T, hkv, hkv, d, block, 1), k.device)
    # a partial last block is a block of its own: nb = ceil(T / block)
    cent = torch.empty((b, hkv, -(-T // block), d), dtype=torch.float32, device=k.device)
    with torch.cuda.device(k.device):
        st = lib.moba_pool_centroids(k.data_ptr(), b, T, hkv, d, block, cent.data_ptr(),
                                     ws.data_ptr(), ws.numel(), _stream_ptr())
    _raise(st, "moba_pool_centroids")
    return cent


def gate_topk(q, centroids, block: int, topk: int):
    """Gate + top-k stage from float32 centroids: int32 [b, Hq, T, topk]."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(centroids, "centroids", torch.float32, 4)
    b, T, hq, d = q.shape
    hkv = centroids.shape[1]
    if centroids.shape != (b, hkv, -(-T // block), d):
        raise ValueError(f"centroids must be [b, hkv, nb, d], got {tuple(centroids.shape)}")
    _raise(check_args(b, T, hq, hkv, d, block, topk, 1.0), "moba_gate_topk")
    ws = _alloc_workspace(stage_workspace_bytes(b, T, hq, hkv, d, block, topk), q.device)
    idx = torch.empty((b, hq, T, topk), dtype=torch.int32, device=q.device)
    with torch.cuda.device(q.device):
        st = lib.moba_gate_topk(q.data_ptr(), centroids.data_ptr(), b, T, hq, hkv, d, block,
                                topk, idx.data_ptr(), ws.data_ptr(), ws.numel(),
                                _stream_ptr())
    _raise(st, "moba_gate_topk")
    return idx


def build_index(idx, hkv: int, block: int, topk: int, kv_begin: int = 0,
                kv_count: int | None = None):
    """Inverted-index stage: (list_offsets int32 [b*kv_count*nb + 1], entries uint32
    as int32 [n])."""
    torch = _torch()
    _need(idx, "idx", torch.int32, 4)
    b, hq, T, k_ = idx.shape
    if k_ != topk:
        raise ValueError("idx last dim must equal topk")
    if kv_count is None:
        kv_count = hkv - kv_begin
    _raise(check_args(b, T, hq, hkv, 64, block, topk, 1.0), "moba_build_index")
    n = index_entries(b, T, hq, hkv, block, topk, kv_count)
    if n < 0:
        raise ValueError("bad kv range")
    nb = -(-T // block)
    ws = _alloc_workspace(stage_workspace_bytes(b, T, hq, hkv, 64, block, topk), idx.device)
    offs = torch.empty(b * kv_count * nb + 1, dtype=torch.int32, device=idx.device)
    ent = torch.empty(max(n, 1), dtype=torch.int32, device=idx.device)
    with torch.cuda.device(idx.device):
        st = lib.moba_build_index(idx.data_ptr(), b, T, hq, hkv, block, topk, kv_begin,
                                  kv_count, offs.data_ptr(), ent.data_ptr(), ws.data_ptr(),
                                  ws.numel(), _stream_ptr())
    _raise(st, "moba_build_index")
    return offs, ent[:n]


def part_dim_order(head_dim: int) -> list:
    """The head dimension held at each position of a ``history_partials`` part row:
    position p = dt*32 + j*16 + hf*8 + u*4 + r holds dimension dt*32 + (2j+u)*8 + hf*4 + r."""
    order = []
    for p in range(head_dim):
        dt, rem = divmod(p, 32)
        j, rem = divmod(rem, 16)
        hf, rem = divmod(rem, 8)
        u, r = divmod(rem, 4)
        order.append(dt * 32 + (2 * j + u) * 8 + hf * 4 + r)
    return order


def history_partials(q, k, v, list_offsets, entries, block: int, topk: int,
                     scale: float | None = None, kv_begin: int = 0,
                     kv_count: int | None = None, tile_order_seed: int = 0,
                     part_o=None, part_lse=None):
    """History-attention stage over an inverted index from ``build_index`` (same kv
    range): (part_o bf16 [b, kv_count*G, T, topk-1, d] with each row's d values in the
    order ``part_dim_order(d)``, part_lse float32 [topk-1, b, kv_count*G, T]).  Slots a row does not have are left as they were (zero
    when the buffers are allocated here).  ``tile_order_seed`` != 0 runs the tiles in a
    seeded permuted order (the parts must not change)."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    _need(list_offsets, "list_offsets", torch.int32, 1)
    _need(entries, "entries", torch.int32, 1)
    b, T, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (b, T, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [b, T, hkv, d] matching q")
    if kv_count is None:
        kv_count = hkv - kv_begin
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _raise(check_args(b, T, hq, hkv, d, block, topk, scale), "moba_history_partials")
    G = hq // hkv
    shape_o = (b, kv_count * G, T, max(topk - 1, 1), d)
    shape_l = (max(topk - 1, 1), b, kv_count * G, T)
    if part_o is None:
        part_o = torch.zeros(shape_o, dtype=torch.bfloat16, device=q.device)
    if part_lse is None:
        part_lse = torch.zeros(shape_l, dtype=torch.float32, device=q.device)
    if tuple(part_o.shape) != shape_o or tuple(part_lse.shape) != shape_l:
        raise ValueError("part_o / part_lse shapes do not match the kv range")
    _need(part_o, "part_o", torch.bfloat16, 5)
    _need(part_lse, "part_lse", torch.float32, 4)
    ws = _alloc_workspace(stage_workspace_bytes(b, T, hq, hkv, d, block, topk), q.device)
    _one_device(q, k, v, list_offsets, entries, part_o, part_lse, ws)
    with torch.cuda.device(q.device):
        st = lib.moba_history_partials(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, T, hq, hkv,
                                       d, block, topk, float(scale), kv_begin, kv_count,
                                       list_offsets.data_ptr(), entries.data_ptr(),
                                       int(tile_order_seed) & 0xffffffff, part_o.data_ptr(),
                                       part_lse.data_ptr(), ws.data_ptr(), ws.numel(),
                                       _stream_ptr())
    _raise(st, "moba_history_partials")
    return part_o, part_lse


def current_merge(q, k, v, part_o, part_lse, block: int, topk: int,
                  scale: float | None = None, kv_begin: int = 0, kv_count: int | None = None,
                  out=None, lse=None):
    """Current-block stage merged with the history parts of ``history_partials`` (same
    kv range): writes out [b, T, Hq, d] bf16 and lse [b, Hq, T] float32 at the heads of
    kv-heads [kv_begin, kv_begin + kv_count) and returns (out, lse)."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    b, T, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (b, T, hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [b, T, hkv, d] matching q")
    if kv_count is None:
        kv_count = hkv - kv_begin
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _raise(check_args(b, T, hq, hkv, d, block, topk, scale), "moba_current_merge")
    if topk > 1:
        _need(part_o, "part_o", torch.bfloat16, 5)
        _need(part_lse, "part_lse", torch.float32, 4)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((b, hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    if out.shape != q.shape or tuple(lse.shape) != (b, hq, T):
        raise ValueError("out / lse shapes do not match q")
    _one_device(q, k, v, out, lse, *([part_o, part_lse] if topk > 1 else []))
    with torch.cuda.device(q.device):
        st = lib.moba_current_merge(q.data_ptr(), k.data_ptr(), v.data_ptr(), b, T, hq, hkv, d,
                                    block, topk, float(scale), kv_begin, kv_count,
                                    part_o.data_ptr() if topk > 1 else None,
                                    part_lse.data_ptr() if topk > 1 else None,
                                    out.data_ptr(), lse.data_ptr(), _stream_ptr())
    _raise(st, "moba_current_merge")
    return out, lse
