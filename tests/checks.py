"""Numerical bars shared by the GPU parity tests (derived from the kernels'
arithmetic; see check_gemv)."""
import numpy as np

import oracle

GEMV_RTOL = 1e-4
NORM_ATOL = 1e-5


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (den if den > 0 else 1.0)


X_CHUNK = {0: None, 1: 32, 2: 32, 3: 32}   # values per x rounding block, by format


def check_gemv(y, ow, x, ref, y0=None, slack=None):
    """Two bars on a GEMV output.
    (1) every element lies within the forward-error bound of the kernel's
        arithmetic for any summation order: fp32 sums,
        (K + 4) 2^-24 sum_k |w_k x_k| (+ |y0|), plus, for the quantized formats,
        x rounded to 22 bits relative to the largest |x| of its block of 32
        values: 2^-22 sum_k |w_k| max_block(k) |x|;
    (2) the relative L2 error over the output vector is <= 1e-4 whenever the
        vector has at least 16 entries.  A single output can be arbitrarily
        ill-conditioned (its value near zero against large terms), so no fp32
        kernel can promise (2) for one entry; (1) is the bar there.
    slack: added to the per-element bound, for inputs known only within a
    tolerance (e.g. a norm computed on the device)."""
    x = np.atleast_2d(np.asarray(x, np.float64))
    y = np.atleast_2d(np.asarray(y, np.float64))
    ref = np.atleast_2d(np.asarray(ref, np.float64))
    absw = np.abs(oracle.dequant(ow).astype(np.float64))
    mag = np.abs(x) @ absw.T
    if y0 is not None:
        mag = mag + np.abs(np.atleast_2d(np.asarray(y0, np.float64)))
    bound = (ow.K + 4) * 2.0 ** -24 * mag + 1e-30
    ch = X_CHUNK[ow.fmt]
    if ch is not None and ow.K > 0:
        amax = np.abs(x).reshape(x.shape[0], -1, ch).max(axis=2)
        xmax = np.repeat(amax, ch, axis=1)
        bound = bound + 2.0 ** -22 * (xmax @ absw.T)
    if slack is not None:          # a known perturbation of x (per output)
        bound = bound + slack
    worst = np.max(np.abs(y - ref) / bound)
    assert worst <= 1.0, "element outside the fp32 forward-error bound (ratio %.3g)" % worst
    if y.size >= 16:
        e = rel_l2(y, ref)
        assert e <= GEMV_RTOL, "rel-L2 %.3e" % e
        return e
    return None
