"""CPU oracle for the decode-step hot path -- TEST INFRASTRUCTURE ONLY.

Thin ctypes marshalling over ``oracle.c`` (plain C, double precision), plus
the exact closed forms in :mod:`oracle.closed_forms`.  Only the tests, the
smoke check and the bench's CPU-baseline leg may import this package; the
product library never does, and it shares no code with it.

Formats (see the header of ``oracle.c`` for the bit layouts):
``BF16 = 0``, ``Q45 = 1``, ``Q65 = 2``, ``Q25 = 3``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

BF16, Q45, Q65, Q25 = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-fPIC", "-shared",
                               "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_code.restype = ctypes.c_int
        L.oracle_code.argtypes = [ctypes.c_int, _vp, _i64, _i64, _i64, _i64]
        L.oracle_weight.restype = ctypes.c_double
        L.oracle_weight.argtypes = [ctypes.c_int, _vp, _i64, _i64, _i64, _i64]
        L.oracle_plane_bytes.restype = ctypes.c_int
        L.oracle_plane_bytes.argtypes = [ctypes.c_int, _i64, _i64, _vp]
        L.oracle_pack.restype = ctypes.c_int
        L.oracle_pack.argtypes = [ctypes.c_int, _i64, _i64, _vp, _vp, _vp, _vp]
        L.oracle_codes.restype = ctypes.c_int
        L.oracle_codes.argtypes = [ctypes.c_int, _vp, _i64, _i64, _vp]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [ctypes.c_int, _vp, _i64, _i64, _vp]
        L.oracle_gemv.restype = None
        L.oracle_gemv.argtypes = [ctypes.c_int, _vp, _i64, _i64, _vp, _i64, _i64,
                                  _vp, _i64, ctypes.c_int, _i64, _i64]
        L.oracle_gather.restype = None
        L.oracle_gather.argtypes = [ctypes.c_int, _vp, _i64, _i64, _i64, _vp, _i64,
                                    _vp, _vp, _i64, _i64]
        for name in ("oracle_rmsnorm", "oracle_rmsnorm_serial_f32"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [_vp, _vp, ctypes.c_float, _i64, _i64, _vp]
        for name in ("oracle_layernorm", "oracle_layernorm_serial_f32"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [_vp, _vp, _vp, ctypes.c_float, _i64, _i64, _vp]
        L.oracle_rmsnorm_tree_f32.restype = None
        L.oracle_rmsnorm_tree_f32.argtypes = [_vp, _vp, ctypes.c_float, _i64, _i64, _i64,
                                              _vp, _vp]
        L.oracle_silu_mul.restype = None
        L.oracle_silu_mul.argtypes = [_vp, _vp, _i64, _vp]
        L.oracle_f32_to_f16_sat.restype = ctypes.c_uint16
        L.oracle_f32_to_f16_sat.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_quantize.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _vp, _vp]
        L.oracle_attention_decode.restype = None
        L.oracle_attention_decode.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _vp,
                                              _vp, _vp, _i64, _vp, _vp]
        L.oracle_decode_token.restype = None
        L.oracle_decode_token.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                          _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                          _vp, _vp, _vp, _vp]
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a) -> int | None:
    return None if a is None else a.ctypes.data


class Planes:
    """The (up to) four host planes of one weight matrix, kept alive together."""

    def __init__(self, fmt: int, N: int, K: int, planes):
        self.fmt, self.N, self.K = int(fmt), int(N), int(K)
        self.planes = [None if p is None else np.ascontiguousarray(p) for p in planes]
        while len(self.planes) < 4:
            self.planes.append(None)
        self._arr = (_vp * 4)(*[_ptr(p) for p in self.planes])

    @property
    def cptr(self):
        return ctypes.cast(self._arr, _vp)


def plane_bytes(fmt: int, N: int, K: int):
    out = np.zeros(4, np.int64)
    rc = lib().oracle_plane_bytes(fmt, N, K, _ptr(out))
    if rc:
        raise ValueError("bad format or K for format %d: K=%d" % (fmt, K))
    return [int(v) for v in out]


def f16_to_f64(h: int) -> float:
    return lib().oracle_f16_to_f64(int(h) & 0xFFFF)


def bf16_to_f64(b: int) -> float:
    return lib().oracle_bf16_to_f64(int(b) & 0xFFFF)


def pack(fmt: int, N: int, K: int, codes, scales=None, supers=None) -> Planes:
    """One byte per weight (or uint16 words for BF16) -> planes."""
    sz = plane_bytes(fmt, N, K)
    planes = [np.zeros(s, np.uint8) if s else None for s in sz]
    codes = _c(codes, np.uint16 if fmt == BF16 else np.uint8)
    sc = None if scales is None else np.ascontiguousarray(scales)
    su = None if supers is None else np.ascontiguousarray(supers)
    arr = (_vp * 4)(*[_ptr(p) for p in planes])
    rc = lib().oracle_pack(fmt, N, K, _ptr(codes), _ptr(sc), _ptr(su), ctypes.cast(arr, _vp))
    if rc:
        raise ValueError("oracle_pack rejected the codes")
    return Planes(fmt, N, K, planes)


def codes(W: Planes) -> np.ndarray:
    out = np.zeros((W.N, W.K), np.uint8)
    lib().oracle_codes(W.fmt, W.cptr, W.N, W.K, _ptr(out))
    return out


def weight(W: Planes, n: int, k: int) -> float:
    return lib().oracle_weight(W.fmt, W.cptr, W.N, W.K, n, k)


def dequant(W: Planes) -> np.ndarray:
    out = np.zeros((W.N, W.K), np.float32)
    lib().oracle_dequant(W.fmt, W.cptr, W.N, W.K, _ptr(out))
    return out


def gemv(W: Planes, x: np.ndarray, y0: np.ndarray | None = None,
         rows: tuple[int, int] | None = None) -> np.ndarray:
    """y[M, N] = x[M, K] @ W^T (double accumulation, one rounding).

    If y0 is given the product is added to it (the accumulate form).  With
    ``rows=(r0, r1)`` only those output rows are computed (others are 0 or y0).
    """
    x = _c(np.atleast_2d(x), np.float32)
    M = x.shape[0]
    assert x.shape[1] == W.K
    y = np.zeros((M, W.N), np.float32) if y0 is None else _c(np.atleast_2d(y0), np.float32).copy()
    r0, r1 = (0, W.N) if rows is None else rows
    lib().oracle_gemv(W.fmt, W.cptr, W.N, W.K, _ptr(x), M, W.K, _ptr(y), W.N,
                      0 if y0 is None else 1, r0, r1)
    return y


def gemv_parallel(W: Planes, x: np.ndarray, threads: int | None = None,
                  y0: np.ndarray | None = None) -> np.ndarray:
    """Same result as gemv() (y0: the accumulate form); output rows split over
    threads (ctypes drops the GIL).  Every output row is computed by the same
    code in the same order as in gemv(), so the two agree bit for bit."""
    import concurrent.futures as cf
    x = _c(np.atleast_2d(x), np.float32)
    M = x.shape[0]
    y = np.zeros((M, W.N), np.float32) if y0 is None else _c(np.atleast_2d(y0), np.float32).copy()
    threads = threads or os.cpu_count() or 1
    bounds = np.linspace(0, W.N, threads + 1).astype(np.int64)
    L = lib()

    def run(i):
        L.oracle_gemv(W.fmt, W.cptr, W.N, W.K, _ptr(x), M, W.K, _ptr(y), W.N,
                      0 if y0 is None else 1, int(bounds[i]), int(bounds[i + 1]))

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, range(threads)))
    return y


def gather(W_all: Planes, rows_per_expert: int, idx: np.ndarray, x: np.ndarray,
           rows: tuple[int, int] | None = None) -> np.ndarray:
    idx = _c(idx, np.int32)
    x = _c(x, np.float32).reshape(-1)
    y = np.zeros((len(idx), rows_per_expert), np.float32)
    r0, r1 = (0, rows_per_expert) if rows is None else rows
    lib().oracle_gather(W_all.fmt, W_all.cptr, W_all.N, W_all.K, rows_per_expert,
                        _ptr(idx), len(idx), _ptr(x), _ptr(y), r0, r1)
    return y


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float32)
    g = _c(gamma, np.float32)
    y = np.empty_like(x)
    lib().oracle_rmsnorm(_ptr(x), _ptr(g), eps, x.shape[0], x.shape[1], _ptr(y))
    return y


def rmsnorm_serial_f32(x, gamma, eps: float) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float32)
    g = _c(gamma, np.float32)
    y = np.empty_like(x)
    lib().oracle_rmsnorm_serial_f32(_ptr(x), _ptr(g), eps, x.shape[0], x.shape[1], _ptr(y))
    return y


def rmsnorm_tree_f32(x, gamma, eps: float, threads: int = 256) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float32)
    g = _c(gamma, np.float32)
    y = np.empty_like(x)
    scratch = np.zeros(threads, np.float32)
    lib().oracle_rmsnorm_tree_f32(_ptr(x), _ptr(g), eps, x.shape[0], x.shape[1], threads,
                                  _ptr(scratch), _ptr(y))
    return y


def layernorm(x, gamma, beta, eps: float) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float32)
    g = _c(gamma, np.float32)
    b = _c(beta, np.float32)
    y = np.empty_like(x)
    lib().oracle_layernorm(_ptr(x), _ptr(g), _ptr(b), eps, x.shape[0], x.shape[1], _ptr(y))
    return y


def layernorm_serial_f32(x, gamma, beta, eps: float) -> np.ndarray:
    x = _c(np.atleast_2d(x), np.float32)
    g = _c(gamma, np.float32)
    b = _c(beta, np.float32)
    y = np.empty_like(x)
    lib().oracle_layernorm_serial_f32(_ptr(x), _ptr(g), _ptr(b), eps, x.shape[0], x.shape[1],
                                      _ptr(y))
    return y


def silu_mul(g, u) -> np.ndarray:
    g = _c(g, np.float32).reshape(-1)
    u = _c(u, np.float32).reshape(-1)
    out = np.empty_like(g)
    lib().oracle_silu_mul(_ptr(g), _ptr(u), g.size, _ptr(out))
    return out


def decode_token(layers, vocab: Planes, g1, g2, gf, eps: float, h0,
                 trace: bool = False):
    """The synthetic decode chain (attention omitted).

    layers: list of dicts with Planes under keys q, k, v, o, gate, up, down.
    Returns (h_final, logits[, h_trace]).
    """
    L = len(layers)
    order = ("q", "k", "v", "o", "gate", "up", "down")
    mats = [lay[key] for lay in layers for key in order] + [vocab]
    d = layers[0]["q"].K if L else vocab.K
    dq = layers[0]["q"].N if L else 0
    dkv = layers[0]["k"].N if L else 0
    f = layers[0]["gate"].N if L else 0
    V = vocab.N
    fmts = np.array([m.fmt for m in mats], np.int32)
    ptrs = (_vp * (4 * len(mats)))()
    for i, m in enumerate(mats):
        for p in range(4):
            ptrs[4 * i + p] = _ptr(m.planes[p])
    h = _c(h0, np.float32).copy()
    logits = np.zeros(V, np.float32)
    ws = np.zeros(dq + 2 * dkv + 3 * f + d, np.float32)
    htr = np.zeros((max(L, 1), d), np.float32)
    g1 = _c(g1, np.float32)
    g2 = _c(g2, np.float32)
    gf = _c(gf, np.float32)
    lib().oracle_decode_token(L, d, dq, dkv, f, V, _ptr(fmts), ctypes.cast(ptrs, _vp),
                              _ptr(g1), _ptr(g2), _ptr(gf), eps, _ptr(h), _ptr(logits),
                              _ptr(ws), _ptr(htr))
    if trace:
        return h, logits, htr[:L]
    return h, logits


def decode_token_parallel(layers, vocab: Planes, g1, g2, gf, eps: float, h0,
                          threads: int | None = None):
    """decode_token() with each matrix-vector product's output rows split over
    threads: the same steps in the same order (oracle_rmsnorm, oracle_gemv,
    oracle_silu_mul, fp32 between steps), so the result is decode_token()'s
    bit for bit.  For the full-size stack, where the single-threaded chain
    takes minutes.  Returns (h_final, logits)."""
    d = vocab.K
    h = _c(h0, np.float32).copy()
    g1 = _c(g1, np.float32)
    g2 = _c(g2, np.float32)
    for l, lay in enumerate(layers):
        a = rmsnorm(h, g1[l * d:(l + 1) * d], eps)[0]
        q = gemv_parallel(lay["q"], a, threads)[0]
        gemv_parallel(lay["k"], a, threads)          # computed, not consumed
        gemv_parallel(lay["v"], a, threads)
        h = gemv_parallel(lay["o"], q, threads, y0=h)[0]
        b = rmsnorm(h, g2[l * d:(l + 1) * d], eps)[0]
        g = gemv_parallel(lay["gate"], b, threads)[0]
        u = gemv_parallel(lay["up"], b, threads)[0]
        m = silu_mul(g, u)
        h = gemv_parallel(lay["down"], m, threads, y0=h)[0]
    z = rmsnorm(h, gf, eps)[0]
    logits = gemv_parallel(vocab, z, threads)[0]
    return h, logits


def decode_token_kv(layers, vocab: Planes, g1, g2, gf, eps: float, h0, kcaches, vcaches,
                    T: int, head_dim: int = 128, threads: int | None = None):
    """One decode token with attention over a KV cache in place of the
    stand-in ([roofline-holds] "Said before the run": each token also reads
    the keys and values of the positions before it).  Per layer l, with
    a = rmsnorm(h, g1[l]) and b = rmsnorm(h, g2[l]):
        q = Wq a;  k = Wk a;  v = Wv a
        K_l[T] = fp16(k);  V_l[T] = fp16(v)     (binary16, nearest even)
        o = attention(q, K_l[0 .. T], V_l[0 .. T])   (T + 1 positions)
        h += Wo o
        h += Wd (silu(Wg b) * (Wu b))
    then logits = Wvocab rmsnorm(h, gf).  The new position is stored before
    it is attended to, so it enters the scores as fp16, like every cached
    one.  kcaches[l], vcaches[l]: float16 arrays [capacity > T, >= dkv],
    head g of a row at g * head_dim; row T of each is overwritten.  Every
    step is the oracle's own (rmsnorm, gemv, silu_mul, attention_decode;
    fp32 between steps); the products' rows are split over threads as in
    gemv_parallel.  Returns (h_final, logits)."""
    d = vocab.K
    h = _c(h0, np.float32).copy()
    g1 = _c(g1, np.float32)
    g2 = _c(g2, np.float32)
    for l, lay in enumerate(layers):
        dq, dkv = lay["q"].N, lay["k"].N
        kc, vc = kcaches[l], vcaches[l]
        assert kc.dtype == np.float16 and vc.dtype == np.float16
        assert kc.shape[0] > T and kc.shape[1] >= dkv and vc.shape == kc.shape
        a = rmsnorm(h, g1[l * d:(l + 1) * d], eps)[0]
        q = gemv_parallel(lay["q"], a, threads)[0]
        k = gemv_parallel(lay["k"], a, threads)[0]
        v = gemv_parallel(lay["v"], a, threads)[0]
        kc[T, :dkv] = k.astype(np.float16)
        vc[T, :dkv] = v.astype(np.float16)
        o = attention_decode(q, kc[:T + 1], vc[:T + 1], dq // head_dim, dkv // head_dim, head_dim)
        h = gemv_parallel(lay["o"], o, threads, y0=h)[0]
        b = rmsnorm(h, g2[l * d:(l + 1) * d], eps)[0]
        g = gemv_parallel(lay["gate"], b, threads)[0]
        u = gemv_parallel(lay["up"], b, threads)[0]
        m = silu_mul(g, u)
        h = gemv_parallel(lay["down"], m, threads, y0=h)[0]
    z = rmsnorm(h, gf, eps)[0]
    logits = gemv_parallel(vocab, z, threads)[0]
    return h, logits


def f32_to_f16(x: float) -> int:
    """fp32 value -> binary16 bits (nearest even, saturating at 65504)."""
    return int(lib().oracle_f32_to_f16_sat(float(np.float32(x))))


def quantize(fmt: int, W: np.ndarray):
    """fp32 weights [N, K] -> (codes [N, K] uint8 (BF16: uint16 words),
    scales, supers) by the oracle's absmax rule (see oracle_quantize)."""
    W = _c(np.atleast_2d(W), np.float32)
    N, K = W.shape
    if fmt == BF16:
        codes = np.zeros((N, K), np.uint16)
        sc = su = None
    else:
        codes = np.zeros((N, K), np.uint8)
        sc = np.zeros(N * K // (16 if fmt == Q65 else 32), np.int8 if fmt == Q65 else np.uint16)
        su = np.zeros(N * K // 256, np.uint16) if fmt == Q65 else None
    rc = lib().oracle_quantize(fmt, N, K, _ptr(W), K, _ptr(codes), _ptr(sc), _ptr(su))
    if rc:
        raise ValueError("oracle_quantize: bad format or K")
    return codes, sc, su


def quantize_planes(fmt: int, W: np.ndarray) -> Planes:
    """quantize() packed into the format's planes."""
    codes, sc, su = quantize(fmt, W)
    N, K = np.atleast_2d(W).shape
    return pack(fmt, N, K, codes, sc, su)


def attention_decode(q, kc, vc, n_heads: int, n_kv: int, d: int, T: int | None = None):
    """One token's attention over a KV cache (see oracle_attention_decode).
    q: float [n_heads * d]; kc, vc: fp16 values or uint16 bits, [T, n_kv * d]
    (row stride = their second dimension).  Returns float [n_heads * d]."""
    q = _c(q, np.float32).reshape(-1)
    kc = np.ascontiguousarray(kc)
    vc = np.ascontiguousarray(vc)
    if kc.dtype == np.float16:
        kc = kc.view(np.uint16)
    if vc.dtype == np.float16:
        vc = vc.view(np.uint16)
    kc = kc.reshape(kc.shape[0], -1)
    vc = vc.reshape(vc.shape[0], -1)
    T = kc.shape[0] if T is None else int(T)
    out = np.zeros(n_heads * d, np.float32)
    scratch = np.zeros(max(T, 1), np.float64)
    lib().oracle_attention_decode(n_heads, n_kv, d, T, _ptr(q), _ptr(kc), _ptr(vc), kc.shape[1],
                                  _ptr(out), _ptr(scratch))
    return out
