"""Decoder weight stream on the device: marshals a model for mbq_decode_step.

DecodeModel holds the device weights of a layer stack in the layout the
decode step reads (qkv rows concatenated, gate and up rows interleaved) and
the C descriptors that point at them; step() enqueues one token.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import QWeight, check, lib, _ptr, _stream
from ._lib import DecodeLayerDesc, DecodeModelDesc


def _row_planes(fmt: int, N: int, K: int, planes):
    """The planes as [N, bytes-per-row] arrays (None where unused)."""
    out = []
    for p in planes:
        if p is None:
            out.append(None)
        else:
            a = np.ascontiguousarray(p, np.uint8)
            out.append(a.reshape(N, a.size // N) if N else a.reshape(0, 0))
    return out


def concat_rows(mats):
    """Stack matrices of one format and K along N: (fmt, N, K, planes) tuples."""
    fmt, K = mats[0][0], mats[0][2]
    assert all(m[0] == fmt and m[2] == K for m in mats)
    rows = [_row_planes(*m) for m in mats]
    planes = [None if rows[0][p] is None else np.concatenate([r[p] for r in rows]).reshape(-1)
              for p in range(4)]
    return fmt, sum(m[1] for m in mats), K, planes


def interleave_rows(a, b):
    """Rows of a and b alternated: row 2i = a[i], row 2i+1 = b[i]."""
    fmt, N, K = a[0], a[1], a[2]
    assert b[0] == fmt and b[1] == N and b[2] == K
    ra, rb = _row_planes(*a), _row_planes(*b)
    planes = [None if ra[p] is None else np.stack([ra[p], rb[p]], axis=1).reshape(-1)
              for p in range(4)]
    return fmt, 2 * N, K, planes


class DecodeModel:
    """Device copy of a decoder stack for mbq_decode_step.

    layers: list of dicts with (fmt, N, K, planes) tuples under q, k, v, o,
    gate, up, down (workloads.config3's layout); g1, g2: fp32 [L * d];
    gf: fp32 [d]; vocab: (fmt, V, d, planes)."""

    def __init__(self, layers, vocab, g1, g2, gf, eps: float, device="cuda"):
        import torch
        L = len(layers)
        d = vocab[2]
        self.eps = float(eps)
        self.d, self.vocab = d, vocab[1]
        self.dq = layers[0]["q"][1] if L else 0
        self.dkv = layers[0]["k"][1] if L else 0
        self.f = layers[0]["gate"][1] if L else 0
        dev = torch.device(device)
        self._keep = []
        self.layer_w = []
        g1 = torch.from_numpy(np.ascontiguousarray(g1, np.float32)).to(dev)
        g2 = torch.from_numpy(np.ascontiguousarray(g2, np.float32)).to(dev)
        self.gf = torch.from_numpy(np.ascontiguousarray(gf, np.float32)).to(dev)
        self.g1, self.g2 = g1, g2
        descs = (DecodeLayerDesc * max(L, 1))()
        for l, lay in enumerate(layers):
            qkv = QWeight.from_host(*concat_rows([lay["q"], lay["k"], lay["v"]]), device=dev)
            o = QWeight.from_host(*lay["o"], device=dev)
            gu = QWeight.from_host(*interleave_rows(lay["gate"], lay["up"]), device=dev)
            dn = QWeight.from_host(*lay["down"], device=dev)
            self.layer_w.append((qkv, o, gu, dn))
            descs[l] = DecodeLayerDesc(qkv.desc, o.desc, gu.desc, dn.desc,
                                       g1[l * d:(l + 1) * d].data_ptr(), g2[l * d:(l + 1) * d].data_ptr())
        self.lm_head = QWeight.from_host(*vocab, device=dev)
        self._descs = descs
        self.desc = DecodeModelDesc(L, self.eps, d, self.dq, self.dkv, self.f, self.vocab,
                                    ctypes.cast(descs, ctypes.POINTER(DecodeLayerDesc)),
                                    self.gf.data_ptr(), self.lm_head.desc)
        nb = ctypes.c_size_t()
        check(lib.mbq_decode_workspace_bytes(ctypes.byref(self.desc), ctypes.byref(nb)))
        self.workspace = torch.empty(max(int(nb.value), 256), dtype=torch.uint8, device=dev)
        self.device = dev

    @property
    def weight_bytes(self) -> int:
        n = sum(w.nbytes for lay in self.layer_w for w in lay) + self.lm_head.nbytes
        return int(n)

    def step(self, h, logits, stream=None):
        """One token: h (fp32 [d], updated in place) -> logits (fp32 [vocab]);
        four launches per layer."""
        check(lib.mbq_decode_step(ctypes.byref(self.desc), _ptr(h), _ptr(logits),
                                  _ptr(self.workspace), self.workspace.numel(), _stream(stream)))
        return logits

    def kv_workspace(self, T: int):
        """A workspace for step_kv at T cached positions (mbq_decode_kv_workspace_bytes)."""
        import torch
        nb = ctypes.c_size_t()
        check(lib.mbq_decode_kv_workspace_bytes(ctypes.byref(self.desc), int(T), ctypes.byref(nb)))
        return torch.empty(max(int(nb.value), 256), dtype=torch.uint8, device=self.device)

    def step_kv(self, h, logits, k_caches, v_caches, T: int, workspace=None, stream=None):
        """One token with attention over the per-layer KV caches
        (mbq_decode_step_kv): row T of every cache takes the token's key and
        value, and attention covers rows 0 .. T.  k_caches, v_caches: lists of
        fp16 cuda tensors [capacity > T, >= dkv], one per layer, all with one
        row stride; updated in place."""
        L = len(self.layer_w)
        assert len(k_caches) == L and len(v_caches) == L
        ld = k_caches[0].stride(0) if L else self.dkv
        for c in list(k_caches) + list(v_caches):
            assert c.stride(0) == ld and c.shape[0] > T
        kp = (ctypes.c_void_p * max(L, 1))(*[c.data_ptr() for c in k_caches])
        vp = (ctypes.c_void_p * max(L, 1))(*[c.data_ptr() for c in v_caches])
        if workspace is None:
            workspace = self.kv_workspace(T)
        check(lib.mbq_decode_step_kv(ctypes.byref(self.desc), _ptr(h), _ptr(logits), kp, vp, int(T),
                                     ld, _ptr(workspace), workspace.numel(), _stream(stream)))
        return logits

    def step_noalloc(self, h, logits, stream=None):
        """One token without a workspace: mbq_decode_step_noalloc (the
        library's own per-GPU array holds the activations; allocates
        nothing)."""
        check(lib.mbq_decode_step_noalloc(ctypes.byref(self.desc), _ptr(h), _ptr(logits),
                                          _stream(stream)))
        return logits

    def prepare(self, stream=None):
        """Write the layer table the one-launch step reads into the workspace."""
        check(lib.mbq_decode_prepare(ctypes.byref(self.desc), _ptr(self.workspace),
                                     self.workspace.numel(), _stream(stream)))
        self._prepared = True

    def step_persistent(self, h, logits, stream=None):
        """One token in one launch (mbq_decode_step_persistent)."""
        if not getattr(self, "_prepared", False):
            self.prepare(stream)
        check(lib.mbq_decode_step_persistent(ctypes.byref(self.desc), _ptr(h), _ptr(logits),
                                             _ptr(self.workspace), self.workspace.numel(),
                                             _stream(stream)))
        return logits

    def status(self) -> int:
        """The one-launch step's status word (0: success), read after a sync."""
        return int(self.workspace[4:8].view(__import__("torch").int32).item())
