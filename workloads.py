"""Seeded synthetic inputs for the five decode-step workloads.

This module only draws random numbers; it holds none of the method's
arithmetic (no decoding, no dot products, no norms).  Both the product path
(tests, bench) and the CPU oracle consume exactly the arrays it returns.

Weights are returned as their storage planes.  Every code field of every
format is uniform over its whole range, and the planes are bit-dense, so a
plane of independent uniform random bytes is exactly a plane of independent
uniform codes; scale planes are drawn separately as fp16 (or int8) values.

Plane order for every format: [codes, codes_hi, scales, super_scales]
(None where a format has no such plane):
  BF16 (0): [uint16 words N*K*2 B, None, None, None]
  Q45  (1): [N*K/2 B codes, None, fp16 N*K/32, None]
  Q65  (2): [N*K/2 B low bits, N*K/4 B high bits, int8 N*K/16, fp16 N*K/256]
  Q25  (3): [N*K/4 B codes, None, fp16 N*K/32, None]

Seeds: workload c (1..5) draws from numpy's default_rng fed by
SeedSequence(1000 + c).spawn(...), one child per tensor in a fixed order, so
each tensor is reproducible on its own.
"""
from __future__ import annotations

import numpy as np

BF16, Q45, Q65, Q25 = 0, 1, 2, 3
SCALE_LO, SCALE_HI = 0.001, 0.02


def _children(c: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(1000 + c).spawn(n)]


def _bytes(rng, n: int) -> np.ndarray:
    return np.frombuffer(rng.bytes(int(n)), dtype=np.uint8).copy()


def _fp16_uniform(rng, n: int, lo=SCALE_LO, hi=SCALE_HI) -> np.ndarray:
    """n fp16 values drawn U(lo, hi) in float64 and rounded to fp16 (RNE)."""
    return rng.uniform(lo, hi, size=int(n)).astype(np.float16).view(np.uint16)


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 words, nearest-even (input drawing only)."""
    b = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def weight_planes(rng, fmt: int, N: int, K: int, std: float = 0.02):
    """Random storage planes of an N x K weight in format fmt."""
    if fmt == BF16:
        w = rng.normal(0.0, std, size=N * K).astype(np.float32)
        return [bf16_from_f32(w).view(np.uint8), None, None, None]
    if fmt == Q45:
        assert K % 32 == 0
        return [_bytes(rng, N * K // 2), None,
                _fp16_uniform(rng, N * K // 32).view(np.uint8), None]
    if fmt == Q25:
        assert K % 32 == 0
        return [_bytes(rng, N * K // 4), None,
                _fp16_uniform(rng, N * K // 32).view(np.uint8), None]
    if fmt == Q65:
        assert K % 256 == 0
        return [_bytes(rng, N * K // 2), _bytes(rng, N * K // 4),
                _bytes(rng, N * K // 16), _fp16_uniform(rng, N * K // 256).view(np.uint8)]
    raise ValueError(fmt)


def normal(rng, n, loc=0.0, scale=1.0) -> np.ndarray:
    return rng.normal(loc, scale, size=n).astype(np.float32)


def uniform(rng, n, lo, hi) -> np.ndarray:
    return rng.uniform(lo, hi, size=n).astype(np.float32)


# ---------------------------------------------------------------------------
# The five workloads.  Sizes default to the full shapes; tests pass smaller
# ones that keep the same structure.
# ---------------------------------------------------------------------------

def config1(n: int = 4096, n_out: int = 512):
    """RMSNorm of one row x ~N(0,1), gamma ~U(0.5,1.5), eps 1e-6, then a bf16
    n_out x n GEMV with W ~N(0, 0.02) rounded to bf16."""
    r = _children(1, 3)
    return dict(x=normal(r[0], n), gamma=uniform(r[1], n, 0.5, 1.5), eps=1e-6,
                W=(BF16, n_out, n, weight_planes(r[2], BF16, n_out, n)))


def config2(n_up: int = 12288, k_up: int = 4096, n_down: int = 4096, k_down: int = 12288):
    """Q45 up table with x ~N(0,1)[k_up]; Q65 down table with its own x[k_down]."""
    r = _children(2, 4)
    return dict(up=(Q45, n_up, k_up, weight_planes(r[0], Q45, n_up, k_up)),
                x_up=normal(r[1], k_up),
                down=(Q65, n_down, k_down, weight_planes(r[2], Q65, n_down, k_down)),
                x_down=normal(r[3], k_down))


def config3(layers: int = 36, d: int = 4096, dq: int = 4096, dkv: int = 1024,
            f: int = 12288, vocab: int = 151936, only=None):
    """The synthetic 36-layer stack: per layer q, k, v, o, gate, up at Q45, down
    at Q65 in even layers and Q45 in odd ones; vocab at Q65; gammas
    ~U(0.5,1.5); h0 ~N(0,1); eps 1e-6.  only: generate just these layer
    indices (the same bytes as in the full stack; "layers" then lists them in
    that order and "layer_ids" names them)."""
    r = _children(3, 7 * layers + 5)
    lay = []
    ids = list(range(layers)) if only is None else list(only)
    for l in ids:
        shapes = dict(q=(Q45, dq, d), k=(Q45, dkv, d), v=(Q45, dkv, d), o=(Q45, d, dq),
                      gate=(Q45, f, d), up=(Q45, f, d),
                      down=(Q65 if l % 2 == 0 else Q45, d, f))
        entry = {}
        for j, name in enumerate(("q", "k", "v", "o", "gate", "up", "down")):
            fmt, N, K = shapes[name]
            entry[name] = (fmt, N, K, weight_planes(r[7 * l + j], fmt, N, K))
        lay.append(entry)
    i = 7 * layers
    V = (Q65, vocab, d, weight_planes(r[i], Q65, vocab, d))
    g1 = uniform(r[i + 1], layers * d, 0.5, 1.5)
    g2 = uniform(r[i + 2], layers * d, 0.5, 1.5)
    gf = uniform(r[i + 3], d, 0.5, 1.5)
    h0 = normal(r[i + 4], d)
    return dict(layers=lay, layer_ids=ids, vocab=V, g1=g1, g2=g2, gf=gf, h0=h0, eps=1e-6)


def config4(M: int, n: int = 12288, k: int = 4096):
    """The Q45 up table of workload 2 (same seed) against X ~N(0,1)[M, k]."""
    r = _children(2, 4)
    W = (Q45, n, k, weight_planes(r[0], Q45, n, k))
    rx = np.random.default_rng(np.random.SeedSequence(1004, spawn_key=(M,)))
    return dict(W=W, X=normal(rx, M * k).reshape(M, k))


def config5(experts: int = 64, rows: int = 1536, k: int = 4096, n_sel: int = 8,
            ln_rows: int = 4096, ln_n: int = 2048):
    """Q25 experts stacked along N, 8 distinct ids (first n_sel of a seeded
    permutation), x ~N(0,1); LayerNorm rows 3 + 2 N(0,1), gamma ~U(0.5,1.5),
    beta ~N(0,0.1), eps 1e-5."""
    r = _children(5, 7)
    W = (Q25, experts * rows, k, weight_planes(r[0], Q25, experts * rows, k))
    idx = r[1].permutation(experts)[:n_sel].astype(np.int32)
    x = normal(r[2], k)
    X = normal(r[3], ln_rows * ln_n, 3.0, 2.0).reshape(ln_rows, ln_n)
    return dict(W=W, rows_per_expert=rows, idx=idx, x=x, ln_x=X,
                ln_gamma=uniform(r[4], ln_n, 0.5, 1.5), ln_beta=normal(r[5], ln_n, 0.0, 0.1),
                ln_eps=1e-5)


def kv_caches(layers: int, rows: int, width: int, seed: int = 3000):
    """Per-layer fp16 key and value caches [rows, width] for the decode step
    with attention: entries N(0, 1) rounded to fp16, like the keys and values
    a 36-layer model of this width leaves for earlier positions (the pages
    give only their byte count, 2 bytes per value).  Returns (k_caches,
    v_caches), lists of float16 arrays; layer l's pair comes from children
    2 l and 2 l + 1 of SeedSequence(seed)."""
    rngs = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(2 * layers)]
    ks = [rngs[2 * l].standard_normal((rows, width), dtype=np.float32).astype(np.float16)
          for l in range(layers)]
    vs = [rngs[2 * l + 1].standard_normal((rows, width), dtype=np.float32).astype(np.float16)
          for l in range(layers)]
    return ks, vs
