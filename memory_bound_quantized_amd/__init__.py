"""memory_bound_quantized_amd -- Python binding of libmbq (include/mbq.h).

Argument marshalling only: every step runs in the library's HIP kernels on
the caller's current torch stream.  torch supplies device memory and streams.
If libmbq.so is missing, importing this package raises ImportError.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from ._lib import BF16, Q25, Q45, Q65, EXPORTS, MbqError, QWeightDesc, check, lib

EPI_STORE, EPI_ACCUMULATE, EPI_SILU_MUL = 0, 1, 2

__all__ = ["BF16", "Q45", "Q65", "Q25", "MbqError", "QWeight", "format_info", "plane_sizes",
           "pack", "unpack", "gemv_q", "gemv_q_gather", "gemv_fused", "EPI_STORE", "EPI_ACCUMULATE",
           "EPI_SILU_MUL", "xq_bytes", "xq_empty", "stage_x",
           "gemv_xq", "rmsnorm_xq", "silu_mul_xq", "rmsnorm", "layernorm", "silu_mul",
           "dequant_f32", "unpack_codes", "probe_read", "probe_copy", "version", "EXPORTS"]

_vp = ctypes.c_void_p


def version() -> int:
    return lib.mbq_version()


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _ptr(t) -> _vp:
    return _vp(0 if t is None else t.data_ptr())


def format_info(fmt: int):
    bpw = ctypes.c_double()
    bk = ctypes.c_int()
    check(lib.mbq_format_info(fmt, ctypes.byref(bpw), ctypes.byref(bk)))
    return bpw.value, bk.value


def plane_sizes(fmt: int, N: int, K: int):
    out = (ctypes.c_size_t * 4)()
    check(lib.mbq_plane_sizes(fmt, N, K, out))
    return [int(v) for v in out]


def pack(fmt: int, N: int, K: int, codes, scales=None, supers=None):
    """Host packer: one byte per weight (uint16 words for BF16) -> 4 planes."""
    sz = plane_sizes(fmt, N, K)
    planes = [np.zeros(s, np.uint8) if s else None for s in sz]
    codes = np.ascontiguousarray(codes, np.uint16 if fmt == BF16 else np.uint8)
    sc = None if scales is None else np.ascontiguousarray(scales)
    su = None if supers is None else np.ascontiguousarray(supers)
    arr = (_vp * 4)(*[None if p is None else p.ctypes.data for p in planes])
    check(lib.mbq_pack(fmt, N, K, codes.ctypes.data, None if sc is None else sc.ctypes.data,
                       None if su is None else su.ctypes.data, arr))
    return planes


def unpack(fmt: int, N: int, K: int, planes):
    """Exact inverse of pack: -> (codes, scales, super_scales) as numpy arrays."""
    sz = plane_sizes(fmt, N, K)
    keep = [None if p is None else np.ascontiguousarray(p, np.uint8) for p in planes]
    arr = (_vp * 4)(*[None if p is None else p.ctypes.data for p in keep])
    codes = np.zeros(N * K, np.uint16 if fmt == BF16 else np.uint8)
    scales = np.zeros(sz[2], np.uint8)
    supers = np.zeros(sz[3], np.uint8)
    check(lib.mbq_unpack(fmt, N, K, arr, codes.ctypes.data, scales.ctypes.data if sz[2] else None,
                         supers.ctypes.data if sz[3] else None))
    if fmt == Q65:
        return codes.reshape(N, K), scales.view(np.int8), supers.view(np.uint16)
    if fmt == BF16:
        return codes.reshape(N, K), None, None
    return codes.reshape(N, K), scales.view(np.uint16), None


class QWeight:
    """A weight matrix resident on the device: its planes as torch uint8 tensors."""

    def __init__(self, fmt: int, N: int, K: int, planes):
        import torch
        self.fmt, self.N, self.K = int(fmt), int(N), int(K)
        self.planes = list(planes) + [None] * (4 - len(planes))
        for p in self.planes:
            if p is not None:
                assert isinstance(p, torch.Tensor) and p.is_cuda and p.dtype == torch.uint8
        self.desc = QWeightDesc(self.fmt, 0, self.N, self.K,
                                *[None if p is None else p.data_ptr() for p in self.planes])

    @classmethod
    def from_host(cls, fmt: int, N: int, K: int, host_planes, device="cuda"):
        import torch
        dev = [None if p is None else torch.from_numpy(np.ascontiguousarray(p, np.uint8)).to(device)
               for p in host_planes]
        return cls(fmt, N, K, dev)

    def clone(self):
        return QWeight(self.fmt, self.N, self.K,
                       [None if p is None else p.clone() for p in self.planes])

    @property
    def nbytes(self) -> int:
        return sum(0 if p is None else p.numel() for p in self.planes)


def gemv_q(W: QWeight, x, out=None, accumulate: bool = False, stream=None):
    """y[M, N] (+)= x[M, K] @ W^T.  x: fp32 cuda tensor [K] or [M, K]."""
    import torch
    x2 = x if x.dim() == 2 else x.view(1, -1)
    M = x2.shape[0]
    if out is None:
        out = torch.empty((M, W.N) if x.dim() == 2 else (W.N,), dtype=torch.float32, device=x.device)
    y2 = out if out.dim() == 2 else out.view(1, -1)
    check(lib.mbq_gemv_q(ctypes.byref(W.desc), _ptr(x2), M, x2.stride(0) if M > 1 else W.K,
                         _ptr(y2), y2.stride(0) if M > 1 else W.N, int(bool(accumulate)),
                         _stream(stream)))
    return out


def gemv_q_gather(W_all: QWeight, rows_per_expert: int, idx, x, out=None, stream=None):
    """y[e, r] = W_all[idx[e] * R + r] . x; idx: int32 cuda tensor."""
    import torch
    n_sel = idx.numel()
    if out is None:
        out = torch.empty((n_sel, rows_per_expert), dtype=torch.float32, device=x.device)
    check(lib.mbq_gemv_q_gather(ctypes.byref(W_all.desc), rows_per_expert, _ptr(idx), n_sel,
                                _ptr(x), _ptr(out), _stream(stream)))
    return out


def gemv_fused(W: QWeight, x, gamma=None, eps: float = 0.0, epilogue: int = EPI_STORE,
               out=None, stream=None):
    """M = 1 product with an optional RMSNorm prologue (gamma) and a store,
    accumulate or silu(gate) * up epilogue (mbq_gemv_fused)."""
    import torch
    n_out = W.N // 2 if epilogue == EPI_SILU_MUL else W.N
    if out is None:
        out = torch.empty(n_out, dtype=torch.float32, device=x.device)
    check(lib.mbq_gemv_fused(ctypes.byref(W.desc), _ptr(x), _ptr(gamma), eps, epilogue,
                             _ptr(out), _stream(stream)))
    return out


def xq_bytes(fmt: int, M: int, K: int) -> int:
    out = ctypes.c_size_t()
    check(lib.mbq_xq_bytes(fmt, M, K, ctypes.byref(out)))
    return int(out.value)


def xq_empty(fmt: int, M: int, K: int, device="cuda"):
    """Device buffer for staged x (opaque; 4 bytes per value) of M rows of K."""
    import torch
    n = xq_bytes(fmt, M, K) // 4
    return torch.empty(n, dtype=torch.int32, device=device)


def stage_x(fmt: int, x, out=None, stream=None):
    """Staged form of fp32 x ([K] or [M, K]) for the products of format fmt."""
    x2 = x if x.dim() == 2 else x.view(1, -1)
    M, K = x2.shape
    if out is None:
        out = xq_empty(fmt, M, K, device=x.device)
    check(lib.mbq_stage_x(fmt, _ptr(x2), M, x2.stride(0) if M > 1 else K, K, _ptr(out),
                          _stream(stream)))
    return out


def gemv_xq(W: QWeight, xq, M: int = 1, out=None, accumulate: bool = False, stream=None):
    """gemv_q with x already staged for W's format (stage_x, rmsnorm_xq, ...)."""
    import torch
    if out is None:
        out = torch.empty((M, W.N) if M > 1 else (W.N,), dtype=torch.float32, device=xq.device)
    y2 = out if out.dim() == 2 else out.view(1, -1)
    check(lib.mbq_gemv_xq(ctypes.byref(W.desc), _ptr(xq), M, _ptr(y2),
                          y2.stride(0) if M > 1 else W.N, int(bool(accumulate)), _stream(stream)))
    return out


def gemv_xq_workspace_bytes(W: QWeight, M: int) -> int:
    out = ctypes.c_size_t()
    check(lib.mbq_gemv_xq_workspace_bytes(ctypes.byref(W.desc), M, ctypes.byref(out)))
    return int(out.value)


def gemv_xq_workspace(W: QWeight, M: int, device="cuda"):
    """A zero-filled workspace for gemv_xq_ws (calls leave it zero)."""
    import torch
    n = max(gemv_xq_workspace_bytes(W, M), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def gemv_xq_ws(W: QWeight, xq, M: int, workspace, out=None, accumulate: bool = False, stream=None):
    """gemv_xq with K split across workgroups through a zero-filled workspace."""
    import torch
    if out is None:
        out = torch.empty((M, W.N) if M > 1 else (W.N,), dtype=torch.float32, device=xq.device)
    y2 = out if out.dim() == 2 else out.view(1, -1)
    check(lib.mbq_gemv_xq_ws(ctypes.byref(W.desc), _ptr(xq), M, _ptr(y2),
                             y2.stride(0) if M > 1 else W.N, int(bool(accumulate)), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def rmsnorm_xq(x, gamma, eps: float, fmt: int, xq=None, out=None, write_y: bool = True,
               stream=None):
    """One row: y = rmsnorm(x) (unless write_y is False) and its staged form for fmt.
    Returns (y or None, xq)."""
    import torch
    n = x.numel()
    if xq is None:
        xq = xq_empty(fmt, 1, n, device=x.device)
    if write_y and out is None:
        out = torch.empty_like(x)
    y = out if write_y else None
    check(lib.mbq_rmsnorm_xq(_ptr(x), _ptr(gamma), eps, n, _ptr(y), fmt, _ptr(xq),
                             _stream(stream)))
    return y, xq


def silu_mul_xq(g, u, fmt: int, xq=None, stream=None):
    """Staged form for fmt of silu(g) * u."""
    n = g.numel()
    if xq is None:
        xq = xq_empty(fmt, 1, n, device=g.device)
    check(lib.mbq_silu_mul_xq(_ptr(g), _ptr(u), n, fmt, _ptr(xq), _stream(stream)))
    return xq


def rmsnorm(x, gamma, eps: float, out=None, stream=None):
    import torch
    n = x.shape[-1]
    rows = x.numel() // n if n else 0
    if out is None:
        out = torch.empty_like(x)
    check(lib.mbq_rmsnorm(_ptr(x), _ptr(gamma), eps, rows, n, _ptr(out), _stream(stream)))
    return out


def layernorm(x, gamma, beta, eps: float, out=None, stream=None):
    import torch
    n = x.shape[-1]
    rows = x.numel() // n if n else 0
    if out is None:
        out = torch.empty_like(x)
    check(lib.mbq_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), eps, rows, n, _ptr(out),
                            _stream(stream)))
    return out


def silu_mul(g, u, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty_like(g)
    check(lib.mbq_silu_mul(_ptr(g), _ptr(u), g.numel(), _ptr(out), _stream(stream)))
    return out


def dequant_f32(W: QWeight, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((W.N, W.K), dtype=torch.float32, device=W.planes[0].device)
    check(lib.mbq_dequant_f32(ctypes.byref(W.desc), _ptr(out), _stream(stream)))
    return out


def unpack_codes(W: QWeight, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((W.N, W.K), dtype=torch.uint8, device=W.planes[0].device)
    check(lib.mbq_unpack_codes(ctypes.byref(W.desc), _ptr(out), _stream(stream)))
    return out


def quantize(fmt: int, w, out: "QWeight | None" = None, stream=None) -> "QWeight":
    """fp32 cuda weights [N, K] (row stride a multiple of 4) -> a QWeight of
    format fmt made on the device (mbq_quantize).  out: a QWeight of the same
    format and shape whose planes are overwritten."""
    import torch
    N, K = w.shape
    if out is None:
        sz = plane_sizes(fmt, N, K)
        out = QWeight(fmt, N, K, [torch.empty(n, dtype=torch.uint8, device=w.device) if n else None
                                  for n in sz])
    arr = (_vp * 4)(*[None if p is None else p.data_ptr() for p in out.planes])
    check(lib.mbq_quantize(fmt, _ptr(w), N, K, w.stride(0), arr, _stream(stream)))
    return out


def attention_workspace_bytes(T: int, n_heads: int, n_kv_heads: int, head_dim: int = 128) -> int:
    out = ctypes.c_size_t()
    check(lib.mbq_attention_workspace_bytes(T, n_heads, n_kv_heads, head_dim, ctypes.byref(out)))
    return int(out.value)


def attention_decode(q, k_cache, v_cache, n_heads: int, n_kv_heads: int, T: int | None = None,
                     out=None, workspace=None, stream=None):
    """One token's attention over an fp16 KV cache (mbq_attention_decode).
    q: fp32 cuda [n_heads * 128]; k_cache, v_cache: fp16 (or int16) cuda
    [capacity, >= n_kv_heads * 128] with the same row stride; T positions."""
    import torch
    T = k_cache.shape[0] if T is None else int(T)
    if out is None:
        out = torch.empty(n_heads * 128, dtype=torch.float32, device=q.device)
    need = attention_workspace_bytes(T, n_heads, n_kv_heads)
    if workspace is None:
        workspace = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    assert k_cache.stride(0) == v_cache.stride(0)
    check(lib.mbq_attention_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), T, k_cache.stride(0),
                                   n_heads, n_kv_heads, 128, _ptr(out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def attention_decode_append(q, k_new, v_new, k_cache, v_cache, T: int, n_heads: int,
                            n_kv_heads: int, out=None, workspace=None, stream=None):
    """The new token's key and value stored at row T of the caches, then its
    attention over rows 0 .. T (mbq_attention_decode_append).  q: fp32 cuda
    [n_heads * 128]; k_new, v_new: fp32 cuda [n_kv_heads * 128]; k_cache,
    v_cache: fp16 (or int16) cuda [capacity > T, >= n_kv_heads * 128] with
    the same row stride, updated in place."""
    import torch
    T = int(T)
    if out is None:
        out = torch.empty(n_heads * 128, dtype=torch.float32, device=q.device)
    need = attention_workspace_bytes(T + 1, n_heads, n_kv_heads)
    if workspace is None:
        workspace = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    assert k_cache.stride(0) == v_cache.stride(0)
    if k_cache.shape[0] <= T or v_cache.shape[0] <= T:
        raise ValueError("the caches need room for row T")
    check(lib.mbq_attention_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                          _ptr(v_cache), T, k_cache.stride(0), n_heads, n_kv_heads,
                                          128, _ptr(out), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream)))
    return out


def probe_mixed(distinct, distinct_bytes: int, shared, shared_bytes: int, mode: int, blocks: int,
                sink, stream=None):
    """Per-compute-unit HBM and L2 streams (mbq_probe_mixed)."""
    check(lib.mbq_probe_mixed(_ptr(distinct), distinct_bytes, _ptr(shared), shared_bytes, mode, blocks,
                              _ptr(sink), _stream(stream)))


def probe_read(buf, sink, stream=None):
    check(lib.mbq_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                             _stream(stream)))


def probe_copy(dst, src, stream=None):
    check(lib.mbq_probe_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(),
                             _stream(stream)))


def probe_chase_init(buf, stream=None) -> int:
    """Write the pointer-chase chain into buf (a cuda tensor); returns the
    number of entries."""
    n = ctypes.c_uint32()
    check(lib.mbq_probe_chase_init(_ptr(buf), buf.numel() * buf.element_size(), ctypes.byref(n),
                                   _stream(stream)))
    return int(n.value)


def probe_chase(buf, entries: int, hops: int, sink, stream=None):
    """Follow `hops` hops of the chain of `entries` entries in buf, from the
    entry sink holds; the entry reached goes back to sink."""
    check(lib.mbq_probe_chase(_ptr(buf), int(entries), int(hops), _ptr(sink), _stream(stream)))


PEAK_MFMA_F16, PEAK_FMA_F32, PEAK_DOT4_I8, PEAK_MFMA_F16_32 = 0, 1, 2, 3


def probe_peak(kind: int, iters: int, sink, stream=None) -> int:
    """One issue-rate launch; returns the operations it executes."""
    ops = ctypes.c_int64()
    check(lib.mbq_probe_peak(int(kind), int(iters), _ptr(sink), ctypes.byref(ops), _stream(stream)))
    return int(ops.value)
