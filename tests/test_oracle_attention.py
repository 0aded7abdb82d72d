"""Pins of the oracle's single-token attention over a KV cache, against
closed forms and invariances of softmax attention, not against itself:

  * one cached position: the output is that position's value row, exactly;
  * all keys equal: uniform weights, the output is the mean of the values;
  * two positions: the weights are 1 / (1 + e^a) and e^a / (1 + e^a) with
    a the score gap, written out with math.exp;
  * grouped heads: head h reads key/value head h // (H / Hkv) (a value head
    held constant shows up in exactly its group's outputs);
  * permuting the cached positions (key and value together) changes nothing;
  * scores of several hundred (exp would overflow without the max shift)
    give the value row of the winning position;
  * the 1/sqrt(d) scale: doubling q equals squaring each weight's odds.
"""
import math

import numpy as np

import oracle


def _cache(rng, T, width):
    return (rng.normal(size=(T, width)).astype(np.float16),
            rng.normal(size=(T, width)).astype(np.float16))


def test_single_position_returns_its_value_row():
    rng = np.random.default_rng(1)
    kc, vc = _cache(rng, 1, 256)
    q = rng.normal(size=4 * 64).astype(np.float32)
    out = oracle.attention_decode(q, kc, vc, 4, 4, 64)
    assert np.array_equal(out, vc[0].astype(np.float32))


def test_equal_keys_average_the_values():
    rng = np.random.default_rng(2)
    T, d = 37, 64
    kc = np.tile(rng.normal(size=(1, 2 * d)).astype(np.float16), (T, 1))
    vc = rng.normal(size=(T, 2 * d)).astype(np.float16)
    q = rng.normal(size=4 * d).astype(np.float32)
    out = oracle.attention_decode(q, kc, vc, 4, 2, d)
    mean = vc.astype(np.float64).mean(axis=0)            # exact sum of halves / T
    for h in range(4):
        g = h // 2
        assert np.array_equal(out[h * d:(h + 1) * d], mean[g * d:(g + 1) * d].astype(np.float32))


def test_two_positions_closed_form():
    d = 4
    q = np.array([1.0, 0.0, 0.0, 0.0], np.float32)
    kc = np.array([[0, 0, 0, 0], [2, 0, 0, 0]], np.float16)      # scores 0 and 2 / sqrt(4) = 1
    vc = np.array([[1, 2, 3, 4], [-4, 0.5, 8, 0]], np.float16)
    out = oracle.attention_decode(q, kc, vc, 1, 1, d)
    p1 = math.exp(1.0) / (1.0 + math.exp(1.0))
    ref = (1 - p1) * vc[0].astype(np.float64) + p1 * vc[1].astype(np.float64)
    assert np.max(np.abs(out - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_grouped_heads_read_their_group():
    rng = np.random.default_rng(3)
    T, d, H, Hkv = 20, 32, 8, 2
    kc, vc = _cache(rng, T, Hkv * d)
    vc[:, d:] = np.float16(7.0)                             # value head 1 constant
    q = rng.normal(size=H * d).astype(np.float32)
    out = oracle.attention_decode(q, kc, vc, H, Hkv, d).reshape(H, d)
    assert np.all(out[4:] == 7.0)                           # heads 4..7 read head 1
    assert not np.any(out[:4] == 7.0)


def test_position_permutation_invariance():
    rng = np.random.default_rng(4)
    T, d = 50, 128
    kc, vc = _cache(rng, T, 2 * d)
    q = rng.normal(size=8 * d).astype(np.float32)
    perm = rng.permutation(T)
    a = oracle.attention_decode(q, kc, vc, 8, 2, d)
    b = oracle.attention_decode(q, kc[perm], vc[perm], 8, 2, d)
    assert np.max(np.abs(a - b)) <= 1e-6 * np.max(np.abs(a))


def test_large_scores_pick_the_winning_position():
    d = 8
    q = np.full(d, 40.0, np.float32)
    kc = np.zeros((5, d), np.float16)
    kc[3] = 10.0                                             # score 40 * 10 * 8 / sqrt(8) ~ 1131
    kc[1] = 9.0                                              # ~113 below: weight e^-113
    vc = np.arange(5 * d, dtype=np.float16).reshape(5, d)
    out = oracle.attention_decode(q, kc, vc, 1, 1, d)
    assert np.all(np.isfinite(out))
    assert np.array_equal(out, vc[3].astype(np.float32))


def test_scale_doubling_q_squares_the_odds():
    d = 16
    q = np.zeros(d, np.float32)
    q[0] = 1.0
    kc = np.zeros((2, d), np.float16)
    kc[1, 0] = 3.0                                           # score gap a = 3 / 4
    vc = np.zeros((2, d), np.float16)
    vc[1, 0] = 1.0                                           # out[0] = weight of position 1
    w1 = float(oracle.attention_decode(q, kc, vc, 1, 1, d)[0])
    w2 = float(oracle.attention_decode(2 * q, kc, vc, 1, 1, d)[0])
    odds1, odds2 = w1 / (1 - w1), w2 / (1 - w2)
    assert abs(odds1 - math.exp(0.75)) <= 1e-6 * math.exp(0.75)
    assert abs(odds2 - odds1 ** 2) <= 1e-5 * odds2
