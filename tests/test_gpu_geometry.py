"""Every launch geometry of the products gives the default geometry's result.

Within one output row the sums run in the same order whatever the geometry
(a lane's chunks in order, one wave reduction per row, or per 4096-wide slice
for K = 12288, then the final add), so the M = 1 and small-batch kernels must
give bit-identical outputs for every rows-per-wave / row-group choice.  The
matrix-core kernel's token-tile count changes how K is split among its
waves, and so the order of the partial sums, so its variants are held to the
oracle's bar instead (and staged and fp32 x agree bit for bit in each).  Geometries are chosen
through the library's tuning variables (read because MBQ_TUNING is set in
conftest.py before the library loads).
"""
import os

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from checks import GEMV_RTOL, check_gemv, rel_l2  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.environ.get("MBQ_TUNING"), "geometry overrides need MBQ_TUNING"
    import memory_bound_quantized_amd  # noqa: F401


def mbq():
    import memory_bound_quantized_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def weights(fmt, N, K, seed):
    planes = workloads.weight_planes(np.random.default_rng(seed), fmt, N, K)
    return oracle.Planes(fmt, N, K, planes), mbq().QWeight.from_host(fmt, N, K, planes)


class env:
    """Set tuning variables for the calls inside the block."""
    def __init__(self, **kv):
        self.kv = {k: str(v) for k, v in kv.items()}

    def __enter__(self):
        os.environ.update(self.kv)

    def __exit__(self, *a):
        for k in self.kv:
            os.environ.pop(k, None)


def bits(t):
    return t.cpu().numpy().view(np.uint32)


M1_CASES = [(1, 1000, 4096), (2, 300, 12288), (1, 130, 12288), (3, 500, 4096), (0, 200, 4096),
            (1, 77, 4160), (0, 130, 4160)]


@pytest.mark.parametrize("fmt,N,K", M1_CASES)
def test_m1_every_geometry_bitwise(fmt, N, K):
    print("geometry m1 fmt=%d N=%d K=%d" % (fmt, N, K), flush=True)
    ow, dw = weights(fmt, N, K, 9900 + N)
    rng = np.random.default_rng(N + K)
    x = rng.normal(size=K).astype(np.float32)
    y0 = rng.normal(size=N).astype(np.float32)
    xd = dev(x)
    ref = mbq().gemv_q(dw, xd)
    check_gemv(ref.cpu().numpy(), ow, x, oracle.gemv(ow, x)[0])
    ref_acc = dev(y0)
    mbq().gemv_q(dw, xd, out=ref_acc, accumulate=True)
    for R in (1, 2, 4):
        for G in (1, 2, 3, 5):
            with env(MBQ_GEMV_ROWS=R, MBQ_GEMV_GROUPS=G):
                y = mbq().gemv_q(dw, xd)
                ya = dev(y0)
                mbq().gemv_q(dw, xd, out=ya, accumulate=True)
            assert np.array_equal(bits(y), bits(ref)), (R, G)
            assert np.array_equal(bits(ya), bits(ref_acc)), (R, G)


@pytest.mark.parametrize("fmt,N,K,silu", [(1, 6144, 4096, False), (2, 130, 12288, False),
                                          (1, 1024, 4096, True), (1, 256, 12288, True)])
def test_fused_every_geometry_bitwise(fmt, N, K, silu):
    print("geometry fused fmt=%d N=%d K=%d silu=%s" % (fmt, N, K, silu), flush=True)
    _, dw = weights(fmt, N, K, 9950 + N)
    rng = np.random.default_rng(N)
    x, g = dev(rng.normal(size=K).astype(np.float32)), dev(rng.uniform(0.5, 1.5, K).astype(np.float32))
    epi = mbq().EPI_SILU_MUL if silu else mbq().EPI_STORE
    ref = mbq().gemv_fused(dw, x, g, 1e-6, epi)
    for R in (1, 2, 4):
        for G in (1, 3, 4, 6, 8):
            with env(MBQ_GEMV_ROWS=R, MBQ_GEMV_GROUPS=G):
                y = mbq().gemv_fused(dw, x, g, 1e-6, epi)
            assert np.array_equal(bits(y), bits(ref)), (R, G)


def test_gather_every_geometry_bitwise():
    """Q25 expert gather (one chunk per lane, rows of a group may come from
    different experts): every geometry gives the default's bits."""
    print("geometry gather q25", flush=True)
    E, rpe, K = 8, 200, 4096
    ow, dw = weights(3, E * rpe, K, 9990)
    rng = np.random.default_rng(5)
    idx = rng.choice(E, 5, replace=False).astype(np.int32)
    x = rng.normal(size=K).astype(np.float32)
    xd, idd = dev(x), dev(idx)
    ref = mbq().gemv_q_gather(dw, rpe, idd, xd)
    assert rel_l2(ref.cpu().numpy(), oracle.gather(ow, rpe, idx, x)) <= GEMV_RTOL
    for R in (1, 2, 4):
        for G in (1, 2, 3, 6):
            with env(MBQ_GEMV_ROWS=R, MBQ_GEMV_GROUPS=G):
                y = mbq().gemv_q_gather(dw, rpe, idd, xd)
            assert np.array_equal(bits(y), bits(ref)), (R, G)


@pytest.mark.parametrize("fmt,M,N,K", [(1, 3, 1000, 4096), (1, 8, 1000, 4160), (2, 2, 300, 12288),
                                       (3, 5, 300, 4096), (0, 4, 200, 4096), (1, 6, 100, 4160)])
def test_smallm_every_geometry_bitwise(fmt, M, N, K):
    print("geometry smallm fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K), flush=True)
    _, dw = weights(fmt, N, K, 9970 + N + M)
    X = dev(np.random.default_rng(M * N).normal(size=(M, K)).astype(np.float32))
    ref = mbq().gemv_q(dw, X)
    for R in (1, 2, 3):
        for G in (1, 2, 4):
            with env(MBQ_SMALLM_ROWS=R, MBQ_SMALLM_GROUPS=G):
                y = mbq().gemv_q(dw, X)
            assert np.array_equal(bits(y), bits(ref)), (R, G)


MFMA_GEOM_CASES = [(16, 1000, 4096), (20, 1000, 4096), (40, 300, 2048), (64, 130, 1024),
                   (6, 77, 640), (33, 200, 2176), (17, 50, 128), (64, 300, 4096),
                   (50, 100, 12288), (4, 300, 4096)]


@pytest.mark.parametrize("M,N,K", MFMA_GEOM_CASES)
def test_mfma_every_geometry_matches_oracle(M, N, K):
    """Staged x on the matrix cores at every row-tile count (1-4 row tiles
    per workgroup) and token-tile count (1, 2 or 4 per workgroup); K = 640
    and 2176 leave some waves without a quad, K = 4096 and 12288 take the
    compile-time streams."""
    print("geometry mfma M=%d N=%d K=%d" % (M, N, K), flush=True)
    ow, dw = weights(1, N, K, 9990 + N)
    X = np.random.default_rng(M + N).normal(size=(M, K)).astype(np.float32)
    Xq = mbq().stage_x(1, dev(X))
    ref = oracle.gemv(ow, X)
    for rw in (1, 2, 3, 4):
        for tt in (1, 2, 4):
            with env(MBQ_MFMA_RW=rw, MBQ_MFMA_TT=tt):
                Y = mbq().gemv_xq(dw, Xq, M=M).cpu().numpy()
            check_gemv(Y, ow, X, ref)


@pytest.mark.parametrize("M,N,K", MFMA_GEOM_CASES)
def test_mfma_f32x_every_geometry_matches_oracle(M, N, K):
    """fp32 x through mbq_gemv_q on the matrix cores (x converted as each
    chunk enters LDS) at every row-tile and token-tile count; the staged and
    the fp32 forms give the same bits."""
    print("geometry mfma fp32 x M=%d N=%d K=%d" % (M, N, K), flush=True)
    ow, dw = weights(1, N, K, 9995 + N)
    X = np.random.default_rng(M + N + 1).normal(size=(M, K)).astype(np.float32)
    Xd = dev(X)
    ref = oracle.gemv(ow, X)
    Xq = mbq().stage_x(1, Xd)
    for rw in (1, 2, 3, 4):
        for tt in (1, 2, 4):
            with env(MBQ_MFMA_RW=rw, MBQ_MFMA_TT=tt):
                Y = mbq().gemv_q(dw, Xd).cpu().numpy()
                Ys = mbq().gemv_xq(dw, Xq, M=M).cpu().numpy()
            check_gemv(Y, ow, X, ref)
            assert np.array_equal(Y.view(np.uint32), Ys.view(np.uint32)), (rw, tt)
