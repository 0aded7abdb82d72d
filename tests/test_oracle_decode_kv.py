"""Pins of the oracle's decode token with attention over a KV cache
(oracle.decode_token_kv), against closed forms of the attention step rather
than against itself:

  * an empty cache (T = 0): softmax over the one new position gives weight
    1, so the attention output of query head h is the new value row of its
    group, rounded to fp16; the token then equals the plain chain with that
    row in place of the attention output, bit for bit;
  * cached keys all equal to the new key: uniform weights, so the output is
    the mean of the T + 1 value rows (the new one included);
  * the cache: row T of every layer holds fp16 of that layer's k and v
    products (numpy's binary16 conversion, nearest even), and no other row
    changes.
Small shapes (two query heads of 128 on one key/value head, or four on two)
keep every case to a fraction of a second.
"""
import numpy as np
import pytest

import oracle
import workloads

HD = 128


def model(L, d, dq, dkv, f, V, seed, fmt=oracle.Q45):
    rng = np.random.default_rng(seed)

    def P(N, K):
        return oracle.Planes(fmt, N, K, workloads.weight_planes(rng, fmt, N, K))

    layers = [{"q": P(dq, d), "k": P(dkv, d), "v": P(dkv, d), "o": P(d, dq),
               "gate": P(f, d), "up": P(f, d), "down": P(d, f)} for _ in range(L)]
    g1 = rng.uniform(0.5, 1.5, L * d).astype(np.float32)
    g2 = rng.uniform(0.5, 1.5, L * d).astype(np.float32)
    gf = rng.uniform(0.5, 1.5, d).astype(np.float32)
    h0 = rng.normal(size=d).astype(np.float32)
    return layers, P(V, d), g1, g2, gf, h0


def caches(L, cap, width, rng):
    return ([rng.normal(size=(cap, width)).astype(np.float16) for _ in range(L)],
            [rng.normal(size=(cap, width)).astype(np.float16) for _ in range(L)])


def chain_with(layers, vocab, g1, g2, gf, eps, h0, attn):
    """The token's chain written out with attn(l, q, k, v) as the attention
    output of layer l (oracle.gemv and friends, fp32 between steps)."""
    d = vocab.K
    h = h0.copy()
    for l, lay in enumerate(layers):
        a = oracle.rmsnorm(h, g1[l * d:(l + 1) * d], eps)[0]
        q = oracle.gemv(lay["q"], a)[0]
        k = oracle.gemv(lay["k"], a)[0]
        v = oracle.gemv(lay["v"], a)[0]
        h = oracle.gemv(lay["o"], attn(l, q, k, v), y0=h)[0]
        b = oracle.rmsnorm(h, g2[l * d:(l + 1) * d], eps)[0]
        m = oracle.silu_mul(oracle.gemv(lay["gate"], b)[0], oracle.gemv(lay["up"], b)[0])
        h = oracle.gemv(lay["down"], m, y0=h)[0]
    z = oracle.rmsnorm(h, gf, eps)[0]
    return h, oracle.gemv(vocab, z)[0]


def expand(rowvals, n_heads, n_kv):
    """Query head h takes key/value head h // (n_heads / n_kv)'s 128 values."""
    G = n_heads // n_kv
    return np.concatenate([rowvals[(h // G) * HD:(h // G + 1) * HD] for h in range(n_heads)])


@pytest.mark.parametrize("n_heads,n_kv", [(2, 1), (4, 2)])
def test_empty_cache_attends_to_the_new_value(n_heads, n_kv):
    L, d, f, V = 2, 256, 512, 64
    dq, dkv = n_heads * HD, n_kv * HD
    layers, vocab, g1, g2, gf, h0 = model(L, d, dq, dkv, f, V, 10 + n_heads)
    kcs, vcs = caches(L, 4, dkv, np.random.default_rng(1))
    k_before = [c.copy() for c in kcs]
    h, logits = oracle.decode_token_kv(layers, vocab, g1, g2, gf, 1e-6, h0, kcs, vcs, 0)
    seen = []

    def new_v(l, q, k, v):
        seen.append((k.astype(np.float16), v.astype(np.float16)))
        return expand(v.astype(np.float16).astype(np.float32), n_heads, n_kv)

    hr, lr = chain_with(layers, vocab, g1, g2, gf, 1e-6, h0, new_v)
    assert np.array_equal(h, hr)
    assert np.array_equal(logits, lr)
    for l in range(L):                                  # row 0 of every layer: its own k and v
        assert np.array_equal(kcs[l][0].view(np.uint16), seen[l][0].view(np.uint16))
        assert np.array_equal(vcs[l][0].view(np.uint16), seen[l][1].view(np.uint16))
        assert np.array_equal(kcs[l][1:].view(np.uint16), k_before[l][1:].view(np.uint16))


def test_equal_keys_average_every_value_row():
    """One layer; the cached keys are set to the fp16 key the token itself
    produces (learned from a first run at T = 0), so every score ties."""
    L, d, f, V, T = 1, 256, 512, 32, 9
    n_heads, n_kv = 4, 2
    dq, dkv = n_heads * HD, n_kv * HD
    layers, vocab, g1, g2, gf, h0 = model(L, d, dq, dkv, f, V, 20)
    rng = np.random.default_rng(2)
    k0, v0 = caches(L, 1, dkv, rng)
    oracle.decode_token_kv(layers, vocab, g1, g2, gf, 1e-6, h0, k0, v0, 0)
    knew = k0[0][0].copy()
    kcs = [np.tile(knew, (T + 3, 1))]
    vcs = [rng.normal(size=(T + 3, dkv)).astype(np.float16)]
    h, logits = oracle.decode_token_kv(layers, vocab, g1, g2, gf, 1e-6, h0, kcs, vcs, T)

    def mean_rows(l, q, k, v):
        rows = np.concatenate([vcs[0][:T].astype(np.float64),
                               v.astype(np.float16).astype(np.float64)[None, :]])
        return expand(rows.mean(axis=0).astype(np.float32), n_heads, n_kv)

    hr, lr = chain_with(layers, vocab, g1, g2, gf, 1e-6, h0, mean_rows)
    assert np.array_equal(h, hr)
    assert np.array_equal(logits, lr)


def test_cache_rows_written_and_kept():
    """Rows wider than the heads, T = 5: row T takes fp16 of k and v, every
    other row and the columns past the heads stay; the token agrees with the
    same chain whose attention is written out here in numpy (fp64)."""
    L, d, f, V, T, cap = 1, 256, 512, 16, 5, 8
    n_heads, n_kv = 2, 1
    dq, dkv = n_heads * HD, n_kv * HD
    width = dkv + 32
    layers, vocab, g1, g2, gf, h0 = model(L, d, dq, dkv, f, V, 30)
    kcs, vcs = caches(L, cap, width, np.random.default_rng(3))
    k_before = [c.copy() for c in kcs]
    v_before = [c.copy() for c in vcs]
    seen = []

    def numpy_attention(l, q, k, v):
        seen.append((k.astype(np.float16), v.astype(np.float16)))
        G = n_heads // n_kv
        kc = np.concatenate([k_before[l][:T, :dkv], k.astype(np.float16)[None, :]]).astype(np.float64)
        vc = np.concatenate([v_before[l][:T, :dkv], v.astype(np.float16)[None, :]]).astype(np.float64)
        out = np.zeros(dq, np.float32)
        for hq in range(n_heads):
            g = hq // G
            s = kc[:, g * HD:(g + 1) * HD] @ q[hq * HD:(hq + 1) * HD].astype(np.float64) / np.sqrt(HD)
            p = np.exp(s - s.max())
            out[hq * HD:(hq + 1) * HD] = (p @ vc[:, g * HD:(g + 1) * HD]) / p.sum()
        return out

    h, logits = oracle.decode_token_kv(layers, vocab, g1, g2, gf, 1e-6, h0, kcs, vcs, T)
    hr, lr = chain_with(layers, vocab, g1, g2, gf, 1e-6, h0, numpy_attention)
    assert np.max(np.abs(h - hr)) <= 1e-6 * np.max(np.abs(hr))
    assert np.max(np.abs(logits - lr)) <= 1e-6 * np.max(np.abs(lr))
    keep = np.ones(cap, bool)
    keep[T] = False
    assert np.array_equal(kcs[0][keep].view(np.uint16), k_before[0][keep].view(np.uint16))
    assert np.array_equal(vcs[0][keep].view(np.uint16), v_before[0][keep].view(np.uint16))
    assert np.array_equal(kcs[0][T, dkv:].view(np.uint16), k_before[0][T, dkv:].view(np.uint16))
    assert np.array_equal(vcs[0][T, dkv:].view(np.uint16), v_before[0][T, dkv:].view(np.uint16))
    assert np.array_equal(kcs[0][T, :dkv].view(np.uint16), seen[0][0].view(np.uint16))
    assert np.array_equal(vcs[0][T, :dkv].view(np.uint16), seen[0][1].view(np.uint16))
