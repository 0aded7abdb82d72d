"""GPU quantizer (mbq_quantize) against the oracle's quantizer, plane by
plane, bit for bit: every code and scale is an integer or a binary16 pattern
decided in fp32 on both sides, so any difference is a bug.

Inputs cover what decides the rule: ordinary weights of the pages' spread,
blocks whose largest |w| makes the scale saturate at 65504 or go subnormal,
all-zero blocks, values exactly halfway between two codes (ties go to the
even code), blocks spanning many decades, bfloat16 halfway cases, ragged row
counts, a row stride wider than K, and the full 12288 x 4096 table.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_quantized_amd  # noqa: F401  (fails loudly if libmbq.so is missing)


def mbq():
    import memory_bound_quantized_amd as m
    return m


BLOCK = {0: 8, 1: 32, 2: 256, 3: 32}
QMAX = {1: 7, 3: 1}


def weights(kind, fmt, N, K, rng):
    """fp32 [N, K] weights of one of the test kinds."""
    if kind == "normal":
        return rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    if kind == "unit":
        return rng.normal(0, 1.0, size=(N, K)).astype(np.float32)
    if kind == "decades":
        # each block's magnitudes drawn over 1e-8 .. 1e4, signs random
        mag = 10.0 ** rng.uniform(-8, 4, size=(N, K))
        return (mag * rng.choice([-1.0, 1.0], size=(N, K))).astype(np.float32)
    if kind == "saturate":
        # blocks whose scale exceeds binary16's range: s = 65504
        w = rng.normal(0, 1.0, size=(N, K)).astype(np.float32)
        w[:, : K // 2] *= np.float32(3e6)
        return w
    if kind == "tiny":
        # scales in binary16's subnormal range, and some that round to zero
        w = rng.normal(0, 1.0, size=(N, K)).astype(np.float32)
        w *= np.float32(1e-6)
        w[:, : K // 4] *= np.float32(1e-4)
        return w
    if kind == "zeros":
        w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
        blk = BLOCK[fmt]
        w.reshape(N, K // blk, blk)[:, ::3, :] = 0.0
        return w
    if kind == "ties":
        # fmt 1 / 3: s0 a power of two, one value at Qmax s0 (so s = s0
        # exactly) and the rest at s0 (k + 1/2): w / s lands on .5
        if fmt in QMAX:
            nb = N * K // 32
            s0 = 2.0 ** rng.integers(-12, -4, nb)
            q = QMAX[fmt]
            k = rng.integers(-q, q, size=(nb, 32)).astype(np.float64)
            w = s0[:, None] * (k + 0.5)
            w[np.arange(nb), rng.integers(0, 32, nb)] = s0 * q * np.where(rng.random(nb) < 0.5, -1, 1)
            return w.astype(np.float32).reshape(N, K)
        if fmt == 0:
            # bf16 halfway cases: low 16 bits exactly 0x8000, both parities
            bits = rng.integers(0x3C000000, 0x42000000, size=(N, K), dtype=np.uint32)
            bits = (bits & 0xFFFF0000) | 0x8000
            return bits.view(np.float32)
        return rng.normal(0, 1.0, size=(N, K)).astype(np.float32)
    raise ValueError(kind)


def device_planes(fmt, w_host, ldw=None):
    K = w_host.shape[1]
    if ldw is None or ldw == K:
        wd = torch.from_numpy(np.ascontiguousarray(w_host)).cuda()
    else:
        full = torch.zeros((w_host.shape[0], ldw), dtype=torch.float32)
        full[:, :K] = torch.from_numpy(w_host)
        wd = full.cuda()[:, :K]
    Q = mbq().quantize(fmt, wd)
    torch.cuda.synchronize()
    return [None if p is None else p.cpu().numpy() for p in Q.planes]


def assert_planes_equal(fmt, got, w):
    ref = oracle.quantize_planes(fmt, w).planes
    for i, (a, b) in enumerate(zip(got, ref)):
        assert (a is None) == (b is None), i
        if a is not None:
            b8 = np.asarray(b).view(np.uint8).reshape(-1)
            if not np.array_equal(a, b8):
                bad = np.flatnonzero(a != b8)
                raise AssertionError("plane %d: %d bytes differ, first at %d (%d vs %d)"
                                     % (i, bad.size, bad[0], a[bad[0]], b8[bad[0]]))


KINDS = ["normal", "unit", "decades", "saturate", "tiny", "zeros", "ties"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_quantize_matches_oracle_bit_for_bit(fmt, kind):
    print("quantize fmt=%d kind=%s" % (fmt, kind), flush=True)
    rng = np.random.default_rng(1000 * fmt + KINDS.index(kind))
    for N, K in ((1, 256), (37, 512), (5, 4096)):
        w = weights(kind, fmt, N, K, rng)
        assert_planes_equal(fmt, device_planes(fmt, w), w)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_quantize_row_stride_wider_than_k(fmt):
    print("quantize stride fmt=%d" % fmt, flush=True)
    rng = np.random.default_rng(77 + fmt)
    N, K = 9, 768
    w = weights("unit", fmt, N, K, rng)
    assert_planes_equal(fmt, device_planes(fmt, w, ldw=K + 36), w)


def test_quantize_empty_is_a_no_op():
    wd = torch.zeros((0, 256), dtype=torch.float32, device="cuda")
    Q = mbq().quantize(1, wd)
    assert Q.N == 0


@pytest.mark.parametrize("fmt,N,K", [(1, 12288, 4096), (2, 4096, 12288)])
def test_quantize_full_size_tables(fmt, N, K):
    print("quantize full fmt=%d %dx%d" % (fmt, N, K), flush=True)
    w = np.random.default_rng(5 + fmt).normal(0, 0.02, size=(N, K)).astype(np.float32)
    assert_planes_equal(fmt, device_planes(fmt, w), w)


def test_quantized_table_through_the_product():
    """The quantizer's output is a valid weight for the products: the M = 1
    product on it equals the oracle's product on the oracle's planes."""
    from checks import check_gemv
    rng = np.random.default_rng(3)
    N, K = 300, 4096
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    Q = mbq().quantize(1, torch.from_numpy(w).cuda())
    x = rng.normal(size=K).astype(np.float32)
    y = mbq().gemv_q(Q, torch.from_numpy(x).cuda()).cpu().numpy()
    ow = oracle.quantize_planes(1, w)
    ref = oracle.gemv(ow, x[None, :])[0]
    check_gemv(y[None, :], ow, x[None, :], ref[None, :])
