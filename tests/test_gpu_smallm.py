"""GPU parity of the small-batch products through the C ABI: 2 <= M <= 8
tokens on the vector units, and Q45 batches of 6+ tokens with K % 1024 == 0
on the matrix cores (fp32 X through mbq_gemv_q, or tile-staged X).

Bars: on the vector units every token's row of Y is bit-identical to the
M = 1 product of that token (same staging, same sums in the same order), so
it inherits the M = 1 parity with the oracle; every case is also checked
against the oracle directly (fp32 forward-error bound, rel-L2 <= 1e-4), which
is the bar of the matrix-core cases.  Staged X (mbq_stage_x) gives the same
bits as fp32 X on the vector units.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from checks import check_gemv  # noqa: E402


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


CASES = [(1, 2, 1000, 4096), (1, 3, 37, 512), (1, 4, 300, 4096), (1, 8, 513, 4096), (1, 6, 300, 4096),
         (1, 3, 1000, 4096), (1, 5, 77, 12288),
         (1, 8, 64, 2080), (1, 2, 64, 12288), (2, 4, 300, 4096), (2, 8, 40, 512),
         (3, 5, 300, 4096), (3, 8, 100, 4160), (0, 6, 100, 1024), (0, 2, 64, 4096)]


@pytest.mark.parametrize("fmt,M,N,K", CASES)
def test_smallm_rows_equal_single_token_products(fmt, M, N, K):
    print("smallm fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K), flush=True)
    planes = workloads.weight_planes(np.random.default_rng(9000 + M + N), fmt, N, K)
    ow, dw = oracle.Planes(fmt, N, K, planes), mbq().QWeight.from_host(fmt, N, K, planes)
    ldx = K + 64
    X = np.random.default_rng(M * K).normal(size=(M, ldx)).astype(np.float32)
    Xd = dev(X)[:, :K]                     # row stride ldx
    Y = mbq().gemv_q(dw, Xd).cpu().numpy()
    cores = fmt == 1 and M >= 4 and K % 128 == 0           # matrix cores
    if not cores:
        for m in range(M):
            y1 = mbq().gemv_q(dw, dev(X[m, :K])).cpu().numpy()
            assert np.array_equal(Y[m].view(np.uint32), y1.view(np.uint32)), m
    ref = oracle.gemv(ow, X[:, :K])
    check_gemv(Y, ow, X[:, :K], ref)
    if fmt != 0:
        Xq = mbq().stage_x(fmt, dev(X[:, :K]))
        Ys = mbq().gemv_xq(dw, Xq, M=M).cpu().numpy()
        if fmt == 1 and M >= 4 and K % 128 == 0:
            # the tile form: Q45 batches of 4+ tokens on the matrix cores, per
            # 16 tokens 2 KB per 32-value block plus 64 exponent bytes per 128
            assert Xq.numel() * 4 == mbq().xq_bytes(1, M, K) == -(-M // 16) * ((K // 32) * 2048 + (K // 128) * 64)
            check_gemv(Ys, ow, X[:, :K], ref)
        else:
            assert np.array_equal(Ys.view(np.uint32), Y.view(np.uint32))


def test_smallm_accumulate_and_row_stride_of_y():
    fmt, M, N, K = 1, 3, 200, 4096
    planes = workloads.weight_planes(np.random.default_rng(9100), fmt, N, K)
    ow, dw = oracle.Planes(fmt, N, K, planes), mbq().QWeight.from_host(fmt, N, K, planes)
    rng = np.random.default_rng(2)
    X = rng.normal(size=(M, K)).astype(np.float32)
    ldy = N + 16
    Y0 = rng.normal(size=(M, ldy)).astype(np.float32)
    Yd = dev(Y0)
    mbq().gemv_q(dw, dev(X), out=Yd[:, :N], accumulate=True)
    Y = Yd.cpu().numpy()
    assert np.array_equal(Y[:, N:], Y0[:, N:])            # padding untouched
    check_gemv(Y[:, :N], ow, X, oracle.gemv(ow, X, y0=Y0[:, :N]), y0=Y0[:, :N])


def test_workload4_full_size_small_batches():
    """The 12288 x 4096 Q45 table against fp32 X[M, 4096] through mbq_gemv_q
    for M = 2 (vector units) and 4, 8, 16, 64 (matrix cores)."""
    for M in (2, 4, 8, 16, 64):
        print("workload4 fp32 M=%d" % M, flush=True)
        cfg = workloads.config4(M)
        fmt, N, K, planes = cfg["W"]
        ow, dw = oracle.Planes(fmt, N, K, planes), mbq().QWeight.from_host(fmt, N, K, planes)
        Y = mbq().gemv_q(dw, dev(cfg["X"])).cpu().numpy()
        ref = oracle.gemv_parallel(ow, cfg["X"])
        check_gemv(Y, ow, cfg["X"], ref)


# --------------------------------------------------------------------------
# Q45 on the matrix cores: tile-staged X and fp32 X converted in the product
# (both one power of two per 32-weight block and token)
# --------------------------------------------------------------------------

MFMA_CASES = [(6, 300, 4096), (16, 64, 4096), (17, 1000, 4096), (31, 130, 1024), (48, 64, 2048),
              (64, 12288, 4096), (80, 300, 4096), (16, 4096, 12288), (512, 1000, 4096),
              (200, 777, 1152)]


@pytest.mark.parametrize("M,N,K", MFMA_CASES)
def test_mfma_matches_oracle(M, N, K):
    print("mfma M=%d N=%d K=%d" % (M, N, K), flush=True)
    planes = workloads.weight_planes(np.random.default_rng(9500 + M + N), 1, N, K)
    ow, dw = oracle.Planes(1, N, K, planes), mbq().QWeight.from_host(1, N, K, planes)
    X = np.random.default_rng(M + K).normal(size=(M, K)).astype(np.float32)
    Xd = dev(X)
    Xt = mbq().stage_x(1, Xd)
    assert Xt.numel() * 4 == mbq().xq_bytes(1, M, K)
    Y = mbq().gemv_xq(dw, Xt, M=M).cpu().numpy()
    ref = oracle.gemv_parallel(ow, X) if N * K > 1 << 24 else oracle.gemv(ow, X)
    check_gemv(Y, ow, X, ref)
    # fp32 X: the same kernel converting x in registers; the same bits where
    # both forms take the same geometry (above 32 tokens on tables of more
    # than 4096 rows fp32 x takes two token tiles per workgroup where staged
    # x takes four, which changes the waves' split of K; the geometry tests
    # compare the two forms bit for bit at every forced geometry)
    Yv = mbq().gemv_q(dw, Xd).cpu().numpy()
    check_gemv(Yv, ow, X, ref)
    if M <= 32 or N <= 4096:
        assert np.array_equal(Yv.view(np.uint32), Y.view(np.uint32))


def test_mfma_token_scales_and_accumulate():
    """Tokens of very different magnitudes (each block of each token has its
    own power-of-two scale), an all-zero token, and the accumulate epilogue."""
    M, N, K = 20, 256, 4096
    planes = workloads.weight_planes(np.random.default_rng(9600), 1, N, K)
    ow, dw = oracle.Planes(1, N, K, planes), mbq().QWeight.from_host(1, N, K, planes)
    rng = np.random.default_rng(7)
    X = rng.normal(size=(M, K)).astype(np.float32)
    X[3] *= np.float32(1e25)
    X[4] *= np.float32(1e-25)
    X[5] = 0.0
    X[6, ::7] *= np.float32(2.0 ** 30)
    Y0 = rng.normal(size=(M, N)).astype(np.float32)
    ref = oracle.gemv(ow, X, y0=Y0)
    Yd = dev(Y0)
    mbq().gemv_xq(dw, mbq().stage_x(1, dev(X)), M=M, out=Yd, accumulate=True)
    check_gemv(Yd.cpu().numpy(), ow, X, ref, y0=Y0)
    # fp32 X on the matrix cores (a power of two per block and token), with
    # row strides on X and Y
    ldx, ldy = K + 32, N + 8
    Xs = np.zeros((M, ldx), np.float32)
    Xs[:, :K] = X
    Ys = np.full((M, ldy), 7.0, np.float32)
    Ys[:, :N] = Y0
    Ysd = dev(Ys)
    mbq().gemv_q(dw, dev(Xs)[:, :K], out=Ysd[:, :N], accumulate=True)
    Yf = Ysd.cpu().numpy()
    assert np.all(Yf[:, N:] == 7.0)                          # padding untouched
    check_gemv(Yf[:, :N], ow, X, ref, y0=Y0)
