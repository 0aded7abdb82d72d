"""GPU special cases and wide-range activations on every product path.

Paths (all through the C ABI):
  m1         mbq_gemv_q, one token (the single-token kernel on fp32 x)
  m1_xq      mbq_stage_x + mbq_gemv_xq, one token (staged x)
  vec        mbq_gemv_q, 2 and 3 tokens (vector units, fp32 x)
  vec_xq     mbq_stage_x + mbq_gemv_xq, 3 tokens (vector units, staged x)
  mfma       mbq_gemv_q, Q45, 4 and 16 tokens (matrix cores, fp32 x)
  mfma_xq    mbq_stage_x + mbq_gemv_xq, Q45, 4, 16 and 64 tokens (matrix
             cores, staged tile form)

Exact cases (the special cases of the product that have a plain closed form):
  * every code at its format's offset: every weight is 0, so y == 0 exactly;
  * one non-zero code per row: y[n] = s[n] (q - offset) x[k] exactly, for x
    with few significant bits (so that no path rounds x or the product);
  * scaling x by a power of two scales y by the same power, bit for bit.

Wide-range activations: tokens with a few 32-value chunks 1e2..1e4 times the
rest, and tokens whose other chunks lie 2^20 or 2^30 below the token's
largest value (with single chunks down to 2^-60).  Half of the rows have
zero weights on the outlier chunks, so their outputs are made only of the small chunks: a path that rounds small
chunks relative to the token's largest value (not their own) shows there.
Bars: the element-wise forward-error bound and rel-L2 <= 1e-4 over all rows
(checks.check_gemv), plus rel-L2 <= 1e-4 per token over each half of the rows.
"""
import zlib

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from checks import GEMV_RTOL, check_gemv, rel_l2  # noqa: E402

OFFSET = {1: 8, 2: 32, 3: 2}
BITS = {1: 4, 2: 6, 3: 2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_quantized_amd  # noqa: F401


def mbq():
    import memory_bound_quantized_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


PATHS = [("m1", 1), ("m1_xq", 1), ("vec", 2), ("vec", 3), ("vec_xq", 3),
         ("mfma", 4), ("mfma", 16), ("mfma_xq", 4), ("mfma_xq", 16), ("mfma_xq", 64)]


def run_path(path, dw, X):
    """Y[M, N] = W X^T through one of the product paths."""
    m = mbq()
    M = X.shape[0]
    Xd = dev(X)
    if path == "m1":
        return m.gemv_q(dw, Xd[0]).cpu().numpy()[None, :]
    if path in ("vec", "mfma"):
        return m.gemv_q(dw, Xd).cpu().numpy().reshape(M, -1)
    xin = Xd[0] if M == 1 else Xd
    xq = m.stage_x(dw.fmt, xin)
    out = m.gemv_xq(dw, xq, M=M).cpu().numpy()
    return out.reshape(M, -1)


def cases(fmts):
    """(fmt, path, M) for every path that takes the format: the matrix-core
    paths take Q45 only."""
    return [pytest.param(f, p, M, id="fmt%d-%s-M%d" % (f, p, M))
            for f in fmts for p, M in PATHS if not p.startswith("mfma") or f == 1]


def planes_from(fmt, codes, scales, supers=None):
    return mbq().pack(fmt, codes.shape[0], codes.shape[1], codes, scales, supers)


# ---------------------------------------------------------------------------
# exact special cases
# ---------------------------------------------------------------------------

def offset_weight(fmt, N, K, rng):
    codes = np.full((N, K), OFFSET[fmt], np.uint8)
    if fmt == 2:
        sc = rng.integers(-128, 128, N * K // 16).astype(np.int8)
        d = workloads._fp16_uniform(rng, N * K // 256)
        return codes, sc, d
    return codes, workloads._fp16_uniform(rng, N * K // 32), None


@pytest.mark.parametrize("fmt,path,M", cases([1, 2, 3]))
def test_codes_at_offset_give_exact_zero(fmt, path, M):
    N, K = 300, 4096
    rng = np.random.default_rng(11 + fmt)
    codes, sc, d = offset_weight(fmt, N, K, rng)
    planes = planes_from(fmt, codes, sc, d)
    dw = mbq().QWeight.from_host(fmt, N, K, planes)
    X = rng.normal(size=(M, K)).astype(np.float32) * 3
    Y = run_path(path, dw, X)
    assert np.all(Y == 0.0), "max |y| = %g" % np.max(np.abs(Y))


def few_bit_x(rng, M, K):
    """Values m / 64 with |m| < 256: at most 8 significant bits."""
    return (rng.integers(-255, 256, size=(M, K)) / 64.0).astype(np.float32)


@pytest.mark.parametrize("fmt,path,M", cases([1, 2, 3]))
def test_one_hot_rows_are_exact(fmt, path, M):
    """One code off the offset per row: y[n] = w[n][k_n] x[k_n], a single
    product that every path must deliver without rounding."""
    N, K = 300, 4096
    rng = np.random.default_rng(21 + fmt + M)
    codes, sc, d = offset_weight(fmt, N, K, rng)
    kk = rng.integers(0, K, N)
    qv = rng.integers(0, 1 << BITS[fmt], N)
    qv[qv == OFFSET[fmt]] = OFFSET[fmt] + 1
    codes[np.arange(N), kk] = qv
    if fmt == 2:
        # Q65 weights d*sc*(q-32) carry up to 23 significant bits: x must be
        # a power of two for the single product to be exact
        X = (2.0 ** rng.integers(-6, 7, size=(M, K)) * rng.choice([-1, 1], size=(M, K))).astype(np.float32)
    else:
        X = few_bit_x(rng, M, K)
    planes = planes_from(fmt, codes, sc, d)
    ow = oracle.Planes(fmt, N, K, planes)
    dw = mbq().QWeight.from_host(fmt, N, K, planes)
    w = np.array([oracle.weight(ow, n, int(kk[n])) for n in range(N)])
    expect = (X[:, kk].astype(np.float64) * w[None, :]).astype(np.float32)
    assert np.array_equal(expect.astype(np.float64), X[:, kk].astype(np.float64) * w[None, :])
    Y = run_path(path, dw, X)
    bad = np.argwhere(Y != expect)
    assert bad.size == 0, "first mismatch (m, n) = %s: %r vs %r" % (
        tuple(bad[0]), Y[tuple(bad[0])], expect[tuple(bad[0])])


@pytest.mark.parametrize("fmt,path,M", cases([0, 1, 2, 3]))
def test_power_of_two_scaling_is_exact(fmt, path, M):
    N, K = 300, 4096
    rng = np.random.default_rng(31 + fmt + M)
    planes = workloads.weight_planes(rng, fmt, N, K)
    dw = mbq().QWeight.from_host(fmt, N, K, planes)
    X = rng.normal(size=(M, K)).astype(np.float32)
    Y = run_path(path, dw, X)
    for j in (-20, -3, 5, 24):
        Yj = run_path(path, dw, (X * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(Yj, (Y * np.float32(2.0 ** j)).astype(np.float32)), "2^%d" % j


# ---------------------------------------------------------------------------
# wide-range activations
# ---------------------------------------------------------------------------

CHUNK = 32


def outlier_case(kind, fmt, N, K, M, rng):
    """(planes, codes, X, big): X ~ N(0,1) with per-chunk factors; `big`
    are the chunks that hold the token's largest values.

    outliers:       three chunks 1e2, 1e3 and 1e4 times the rest;
    far_below:      the rest 2^-20 below the big chunks, three chunks
                    2^-30, 2^-40 and 2^-60 below;
    very_far_below: the rest 2^-30 below, two chunks 2^-45 below;
    mixed:          a 1e4 outlier, eight chunks 2^-20 below the rest."""
    X = rng.normal(size=(M, K)).astype(np.float64)
    nch = K // CHUNK
    perm = rng.permutation(nch)
    big, rest = perm[:3], perm[3:]
    base = {"outliers": 1.0, "far_below": 2.0 ** -20, "very_far_below": 2.0 ** -30,
            "mixed": 1.0}[kind]
    fac = np.full(nch, base)
    if kind == "outliers":
        fac[big] = (1e2, 1e3, 1e4)
    elif kind == "far_below":
        fac[big] = (1.0, 1.0, 4.0)
        fac[rest[:3]] = (2.0 ** -30, 2.0 ** -40, 2.0 ** -60)
    elif kind == "very_far_below":
        fac[big] = (1.0, 1.0, 4.0)
        fac[rest[:2]] = 2.0 ** -45
    else:
        fac[big] = (1e4, 1.0, 1.0)
        fac[rest[:8]] = 2.0 ** -20
    X = (X * np.repeat(fac, CHUNK)[None, :]).astype(np.float32)
    planes = workloads.weight_planes(rng, fmt, N, K)
    codes = oracle.codes(oracle.Planes(fmt, N, K, planes))
    return planes, codes, X, big


def zero_rows_on(fmt, planes, codes, N, K, rows, chunks):
    """Set the codes of `rows` to the offset on `chunks`: those weights are 0."""
    ow = oracle.Planes(fmt, N, K, planes)
    c = codes.copy()
    for ch in chunks:
        c[np.ix_(rows, np.arange(ch * CHUNK, (ch + 1) * CHUNK))] = OFFSET[fmt]
    sc = ow.planes[2].view(np.int8 if fmt == 2 else np.uint16).copy()
    su = ow.planes[3].view(np.uint16).copy() if fmt == 2 else None
    return mbq().pack(fmt, N, K, c, sc, su)


@pytest.mark.parametrize("kind", ["outliers", "far_below", "very_far_below", "mixed"])
@pytest.mark.parametrize("fmt,path,M", cases([1, 2, 3]))
def test_wide_range_tokens(kind, fmt, path, M):
    N, K = 300, 4096
    print("wide-range %s path=%s M=%d fmt=%d" % (kind, path, M, fmt), flush=True)
    rng = np.random.default_rng(zlib.crc32(("%s %s %d %d" % (kind, path, M, fmt)).encode()))
    planes, codes, X, big = outlier_case(kind, fmt, N, K, M, rng)
    even = np.arange(0, N, 2)
    planes = zero_rows_on(fmt, planes, codes, N, K, even, big)
    ow = oracle.Planes(fmt, N, K, planes)
    dw = mbq().QWeight.from_host(fmt, N, K, planes)
    Y = run_path(path, dw, X)
    ref = oracle.gemv_parallel(ow, X)
    check_gemv(Y, ow, X, ref)
    for m in range(M):
        for rows, name in ((even, "rows without the outlier chunks"), (np.arange(1, N, 2), "other rows")):
            e = rel_l2(Y[m, rows], ref[m, rows])
            assert e <= GEMV_RTOL, "token %d, %s: rel-L2 %.3e" % (m, name, e)
