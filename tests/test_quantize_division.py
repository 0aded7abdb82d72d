"""The quantizer kernel's shortcut for rint(w / s), checked on the CPU.

The kernel takes t = w * r with r = v_rcp_f32(s) (within 1 ulp of 1/s) and
uses rint(t) wherever t lies more than 2^-14 from the nearest k + 1/2 and
|t| < 64; otherwise it divides.  The claim is that this always equals rint
of the correctly rounded fp32 quotient (what the oracle computes).  Here the
same decision is emulated in numpy float32 with r taken as the correctly
rounded 1/s and as its neighbours one ulp below and above (the worst a
1-ulp reciprocal can be), over random quotients, quotients a few ulps from
a tie, exact ties, and the clamp region, for every scale range the formats
produce (binary16 scales, subnormal ones included, and Q65 steps d * sc).
"""
import numpy as np

MARGIN = np.float32(0.5 - 2.0 ** -14)


def exact(w, s):
    return np.rint(w / s)                       # float32 division is correctly rounded


def shortcut(w, s, r):
    t = w * r                                   # float32 product, rounded once
    f = np.rint(t)
    ok = (np.abs(t - f) < MARGIN) & (np.abs(t) < np.float32(64.0))
    return np.where(ok, f, exact(w, s)), ok


def reciprocals(s):
    r = (np.float32(1.0) / s).astype(np.float32)
    return [r, np.nextafter(r, np.float32(0.0)), np.nextafter(r, np.float32(np.inf))]


def check(w, s):
    w = w.astype(np.float32)
    s = s.astype(np.float32)
    ref = exact(w, s)
    taken = np.zeros(w.shape, bool)
    for r in reciprocals(s):
        got, ok = shortcut(w, s, r)
        assert np.array_equal(got, ref), (w[got != ref][:4], s[got != ref][:4])
        taken |= ok
    return taken


def half_scales(rng, n, lo=-24, hi=15):
    """Positive binary16 values spread over their exponent range."""
    e = rng.integers(lo, hi, n)
    m = rng.integers(1024, 2048, n) if hi > -14 else rng.integers(1, 1024, n)
    s = np.ldexp(m.astype(np.float64), e - 10)
    return np.clip(s, 2.0 ** -24, 65504.0).astype(np.float16).astype(np.float32)


def test_random_quotients_of_every_format():
    rng = np.random.default_rng(1)
    n = 400000
    for qmax in (7.0, 1.0, 31.0 * 1.5):          # Q45, Q25, Q65 (steps d * sc)
        s = half_scales(rng, n)
        w = (rng.uniform(-1.05, 1.05, n) * qmax * s).astype(np.float32)
        taken = check(w, s)
        assert taken.mean() > 0.999              # the shortcut is the common path


def test_quotients_next_to_a_tie():
    """k + 1/2 plus or minus a few ulps of the quotient: the shortcut must
    step aside (or agree) exactly where the rounded quotient changes side."""
    rng = np.random.default_rng(2)
    n = 200000
    s = half_scales(rng, n)
    k = rng.integers(-40, 40, n).astype(np.float64)
    ulps = rng.integers(-6, 7, n).astype(np.float64)
    q = (k + 0.5) * (1.0 + ulps * 2.0 ** -23)
    w = (q * s).astype(np.float32)
    check(w, s)


def test_exact_ties_take_the_division():
    rng = np.random.default_rng(3)
    n = 50000
    s = (2.0 ** rng.integers(-20, 10, n)).astype(np.float32)      # powers of two: w / s exact
    k = rng.integers(-30, 30, n).astype(np.float32)
    w = (s * (k + np.float32(0.5))).astype(np.float32)
    taken = check(w, s)
    assert not taken.any()                       # every exact tie is divided


def test_subnormal_scales_and_the_clamp_region():
    rng = np.random.default_rng(4)
    n = 100000
    s = half_scales(rng, n, lo=-24, hi=-14)      # binary16 subnormals as fp32
    w = (rng.uniform(-10.5, 10.5, n) * s).astype(np.float32)
    check(w, s)
    # quotients beyond 64 (only reachable through odd Q65 steps) divide
    s2 = half_scales(rng, n)
    w2 = (rng.uniform(60.0, 200.0, n) * s2 * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    check(w2, s2)


def test_q65_steps_d_times_sc():
    """Q65 divides by d * sc: a binary16 d times an int8 sub-scale, exact in
    fp32 (11 + 7 significant bits)."""
    rng = np.random.default_rng(5)
    n = 200000
    d = half_scales(rng, n)
    sc = rng.integers(1, 128, n).astype(np.float32)
    step = (d * sc).astype(np.float32)
    assert np.array_equal(step.astype(np.float64), d.astype(np.float64) * sc.astype(np.float64))
    w = (rng.uniform(-33.0, 33.0, n) * step).astype(np.float32)
    check(w, step)
