"""Pins of the oracle's quantizer (fp32 weights -> codes and scales) and of
its binary16 / bfloat16 encoders, against things other than the oracle:

  * the encoders against numpy's independent binary16 conversion, on normal,
    subnormal and tie values, and hand-written saturation cases;
  * hand-derived fixtures (tests/golden/quantize_fixtures.json, each with
    its derivation);
  * round trip: a block built as s (q - offset) with an exactly
    representable scale and one code at the extreme quantizes back to the
    same codes and scale, bit for bit (any wrong offset, level count, sign,
    index or rounding of the scale breaks it);
  * every unclamped weight within half a step of its dequantized value;
  * power-of-two scaling of the weights scales the scales, codes unchanged;
  * all-zero blocks.
The rule itself (this library's reading: symmetric absmax, decisions in
fp32) is written above oracle_quantize in oracle.c.
"""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_f16_encoder_matches_numpy():
    rng = np.random.default_rng(3)
    x = (rng.normal(size=50000) * 10.0 ** rng.integers(-9, 5, 50000)).astype(np.float32)
    x = x[np.abs(x) < 65504]
    mine = np.array([oracle.f32_to_f16(v) for v in x], np.uint16)
    assert np.array_equal(mine, x.astype(np.float16).view(np.uint16))
    # ties: midpoints between consecutive halves (exact in fp32), normal and subnormal
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt = (np.arange(0, 0x7BFF, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float32)
    mid = ((h.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    assert np.all(mid.astype(np.float64) == (h.astype(np.float64) + nxt.astype(np.float64)) / 2)
    mine = np.array([oracle.f32_to_f16(v) for v in mid], np.uint16)
    assert np.array_equal(mine, mid.astype(np.float16).view(np.uint16))
    assert np.all(mine % 2 == 0)        # ties go to the even fraction


def test_f16_encoder_saturates():
    assert oracle.f32_to_f16(65504.0) == 0x7BFF
    assert oracle.f32_to_f16(65519.0) == 0x7BFF
    assert oracle.f32_to_f16(65520.0) == 0x7BFF       # would round to inf
    assert oracle.f32_to_f16(3.0e38) == 0x7BFF
    assert oracle.f32_to_f16(-3.0e38) == 0xFBFF
    assert oracle.f32_to_f16(0.0) == 0 and oracle.f32_to_f16(-0.0) == 0x8000
    assert oracle.f32_to_f16(2.0 ** -24) == 1                  # smallest subnormal
    assert oracle.f32_to_f16(2.0 ** -25) == 0                  # tie to even: 0
    assert oracle.f32_to_f16(3 * 2.0 ** -25) == 2              # tie to even: 2


def test_bf16_encoder():
    L = oracle.lib()
    f = lambda v: int(L.oracle_f32_to_bf16(float(np.float32(v))))
    assert f(1.0) == 0x3F80 and f(-2.0) == 0xC000
    one_plus = np.array([0x3F808000], np.uint32).view(np.float32)[0]   # halfway above even 0x3F80: stays
    assert f(one_plus) == 0x3F80
    odd_half = np.array([0x3F818000], np.uint32).view(np.float32)[0]   # halfway above odd 0x3F81
    assert f(odd_half) == 0x3F82
    assert f(np.array([0x3F808001], np.uint32).view(np.float32)[0]) == 0x3F81


def test_hand_fixtures():
    cases = json.load(open(os.path.join(HERE, "golden", "quantize_fixtures.json")))["cases"]
    for c in cases:
        if c["fmt"] == 2:
            w = np.zeros((1, 256), np.float32)
            w[0, :16] = c["w_sub0"]
            codes, sc, su = oracle.quantize(2, w)
            assert list(su) == c["super_bits"], c["name"]
            assert list(sc[:2]) == c["sub_scales_first"] and np.all(sc[1:] == 0)
            assert list(codes[0, :16]) == c["codes_sub0"] and np.all(codes[0, 16:] == 32)
        else:
            w = np.array(c["w"], np.float32)[None, :]
            codes, sc, su = oracle.quantize(c["fmt"], w)
            assert list(sc) == c["scale_bits"], c["name"]
            assert list(codes[0]) == c["codes"], c["name"]


def _representable(fmt, N, K, rng):
    """Weights s (q - off) whose quantization is known: scales are binary16
    values and each block holds one code at the level that defines its
    scale (+-Qmax).  Returns (w, codes, scales, supers)."""
    if fmt in (1, 3):
        qmax, off, top = (7, 8, 15) if fmt == 1 else (1, 2, 3)
        nb = N * K // 32
        s = rng.uniform(0.001, 0.02, nb).astype(np.float16)
        codes = rng.integers(off - qmax, top + 1, size=(nb, 32)).astype(np.uint8)
        pos = rng.integers(0, 32, nb)
        codes[np.arange(nb), pos] = np.where(rng.random(nb) < 0.5, off - qmax, off + qmax)
        w = (s.astype(np.float64)[:, None] * (codes.astype(np.float64) - off)).astype(np.float32)
        return w.reshape(N, K), codes.reshape(N, K), s.view(np.uint16), None
    # Q65: per super-block d (binary16), sub-scales 1..127 with one 127;
    # each sub-block holds one code at 32 +- 31
    nsb = N * K // 256
    d = rng.uniform(1e-4, 2e-3, nsb).astype(np.float16)
    sc = rng.integers(1, 128, size=(nsb, 16)).astype(np.int8)
    sc[np.arange(nsb), rng.integers(0, 16, nsb)] = 127
    codes = rng.integers(1, 64, size=(nsb, 16, 16)).astype(np.uint8)
    ii = np.arange(nsb)[:, None]
    jj = np.arange(16)[None, :]
    codes[ii, jj, rng.integers(0, 16, (nsb, 16))] = np.where(rng.random((nsb, 16)) < 0.5, 1, 63)
    step = d.astype(np.float64)[:, None] * sc.astype(np.float64)
    w = (step[:, :, None] * (codes.astype(np.float64) - 32)).astype(np.float32)
    return w.reshape(N, K), codes.reshape(N, K), sc.reshape(-1), d.view(np.uint16)


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_round_trip_of_representable_blocks(fmt):
    rng = np.random.default_rng(40 + fmt)
    w, codes, sc, su = _representable(fmt, 8, 512, rng)
    c2, s2, u2 = oracle.quantize(fmt, w)
    assert np.array_equal(c2, codes)
    assert np.array_equal(np.asarray(s2).view(np.uint8), np.asarray(sc).view(np.uint8))
    if fmt == 2:
        assert np.array_equal(u2, su)


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_every_unclamped_weight_within_half_a_step(fmt):
    rng = np.random.default_rng(50 + fmt)
    w = rng.normal(0, 0.02, size=(16, 1024)).astype(np.float32)
    P = oracle.quantize_planes(fmt, w)
    codes, deq = oracle.codes(P), oracle.dequant(P).astype(np.float64)
    if fmt == 2:
        d = np.repeat(np.array([oracle.f16_to_f64(int(h)) for h in P.planes[3].view(np.uint16)]), 256)
        step = d * np.repeat(P.planes[2].view(np.int8).astype(np.float64), 16)
        top, lo = 63, 0
    else:
        step = np.repeat(np.array([oracle.f16_to_f64(int(h)) for h in P.planes[2].view(np.uint16)]), 32)
        top, lo = (15, 0) if fmt == 1 else (3, 0)
    step = step.reshape(w.shape)
    err = np.abs(w.astype(np.float64) - deq)
    unclamped = (codes > lo) & (codes < top)
    assert np.all(err[unclamped] <= step[unclamped] * (0.5 + 2.0 ** -20))
    # the symmetric rule clamps nothing for Q45 and Q25 (|w / s| <= Qmax up to
    # the rounding of s); where Q65 clamps, the error stays within one step
    assert np.all(err <= step * (1.0 + 2.0 ** -20))


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_power_of_two_scaling(fmt):
    """Exact while every scale stays a normal binary16: Q65's super-scale is
    about max|w| / 3937, subnormal for weights of N(0, 0.02) (there the
    rounding of d depends on the power of two), so Q65 uses N(0, 1)."""
    rng = np.random.default_rng(60 + fmt)
    w = rng.normal(0, 1.0 if fmt == 2 else 0.02, size=(4, 1024)).astype(np.float32)
    c1, s1, u1 = oracle.quantize(fmt, w)
    for j in (-3, 4):
        c2, s2, u2 = oracle.quantize(fmt, (w * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c1, c2)
        if fmt == 2:
            assert np.array_equal(s1, s2)
            assert np.all(u2.view(np.float16).astype(np.float64) == u1.view(np.float16).astype(np.float64) * 2.0 ** j)
        else:
            assert np.all(s2.view(np.float16).astype(np.float64) == s1.view(np.float16).astype(np.float64) * 2.0 ** j)


def test_zero_blocks():
    for fmt, off in ((1, 8), (2, 32), (3, 2)):
        codes, sc, su = oracle.quantize(fmt, np.zeros((2, 512), np.float32))
        assert np.all(codes == off) and np.all(np.asarray(sc) == 0)
        if fmt == 2:
            assert np.all(su == 0)
