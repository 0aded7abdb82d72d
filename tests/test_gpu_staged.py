"""GPU parity of the staged-x path: mbq_stage_x, mbq_gemv_xq, mbq_rmsnorm_xq
and mbq_silu_mul_xq, through the C ABI.

Bars:
  * a product on staged x is bit-identical to mbq_gemv_q on the same fp32 x
    (same staging, same sums in the same order) and within the fp32
    forward-error bound / rel-L2 1e-4 of the oracle;
  * a fused producer's staged output is bit-identical to staging its fp32
    output with mbq_stage_x, and its fp32 output is within 1e-5 (norms) of
    the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from checks import NORM_ATOL, check_gemv  # noqa: E402


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


def weights(fmt, N, K, seed):
    planes = workloads.weight_planes(np.random.default_rng(seed), fmt, N, K)
    return planes, oracle.Planes(fmt, N, K, planes), mbq().QWeight.from_host(fmt, N, K, planes)


def bits(t):
    return t.cpu().numpy().view(np.uint32)


XQ_CASES = [(1, 1, 32), (1, 37, 512), (1, 1000, 4096), (1, 64, 12288), (1, 12288, 4096),
            (2, 1, 256), (2, 37, 512), (2, 300, 4096), (2, 4096, 12288),
            (3, 1, 64), (3, 37, 512), (3, 1536, 4096),
            (0, 37, 520), (0, 512, 4096)]


@pytest.mark.parametrize("fmt,N,K", XQ_CASES)
def test_gemv_xq_matches_gemv_q_bitwise_and_oracle(fmt, N, K):
    print("gemv_xq fmt=%d N=%d K=%d" % (fmt, N, K), flush=True)
    _, ow, dw = weights(fmt, N, K, 7000 + fmt + N)
    x = np.random.default_rng(N + K).normal(size=K).astype(np.float32)
    xd = dev(x)
    y_q = mbq().gemv_q(dw, xd)
    xq = mbq().stage_x(fmt, xd)
    y_s = mbq().gemv_xq(dw, xq)
    assert np.array_equal(bits(y_s), bits(y_q))
    check_gemv(y_s.cpu().numpy(), ow, x, oracle.gemv(ow, x)[0])


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_gemv_xq_accumulate(fmt):
    N, K = 300, 512
    _, ow, dw = weights(fmt, N, K, 7100 + fmt)
    rng = np.random.default_rng(5)
    x = rng.normal(size=K).astype(np.float32)
    y0 = rng.normal(size=N).astype(np.float32)
    yd = dev(y0)
    mbq().gemv_xq(dw, mbq().stage_x(fmt, dev(x)), out=yd, accumulate=True)
    ref = oracle.gemv(ow, x, y0=y0)[0]
    check_gemv(yd.cpu().numpy(), ow, x, ref, y0=y0)


@pytest.mark.parametrize("kind", ["zeros", "one_hot", "tiny", "huge", "mixed_scales"])
def test_staging_edge_values(kind):
    """Chunks of zeros, a single non-zero, subnormals, values near 1e30 and
    chunks whose magnitudes differ by 2^40: staging keeps the bound."""
    fmt, N, K = 1, 64, 1024
    _, ow, dw = weights(fmt, N, K, 7200)
    rng = np.random.default_rng(11)
    x = rng.normal(size=K).astype(np.float32)
    if kind == "zeros":
        x[:256] = 0.0
    elif kind == "one_hot":
        x[:] = 0.0
        x[77] = 3.0
    elif kind == "tiny":
        x[:512] = (x[:512] * 1e-39).astype(np.float32)
    elif kind == "huge":
        x *= np.float32(1e30)
    else:
        x[::64] *= np.float32(2.0 ** 40)
    xd = dev(x)
    y = mbq().gemv_xq(dw, mbq().stage_x(fmt, xd))
    assert np.array_equal(bits(y), bits(mbq().gemv_q(dw, xd)))
    check_gemv(y.cpu().numpy(), ow, x, oracle.gemv(ow, x)[0])


def test_stage_x_rows_are_independent():
    fmt, M, K, ldx = 2, 3, 512, 640
    rng = np.random.default_rng(3)
    X = rng.normal(size=(M, ldx)).astype(np.float32)
    Xd = dev(X)
    xq = mbq().xq_empty(fmt, M, K)
    from memory_bound_quantized_amd import _lib
    import ctypes
    rc = _lib.lib.mbq_stage_x(fmt, ctypes.c_void_p(Xd.data_ptr()), M, ldx, K,
                              ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    for m in range(M):
        one = mbq().stage_x(fmt, dev(X[m, :K]))
        assert torch.equal(xq[m * K:(m + 1) * K].cpu(), one.cpu())


@pytest.mark.parametrize("fmt,n", [(1, 4096), (2, 4096), (3, 4096), (0, 4096), (1, 32), (3, 64),
                                   (1, 2048), (2, 8192), (1, 1056), (1, 1024), (3, 6144)])
def test_rmsnorm_xq(fmt, n):
    print("rmsnorm_xq fmt=%d n=%d" % (fmt, n), flush=True)
    rng = np.random.default_rng(n + fmt)
    x = rng.normal(size=n).astype(np.float32)
    g = rng.uniform(0.5, 1.5, n).astype(np.float32)
    xd, gd = dev(x), dev(g)
    y, xq = mbq().rmsnorm_xq(xd, gd, 1e-6, fmt)
    ref = oracle.rmsnorm(x, g, 1e-6)[0]
    assert np.max(np.abs(y.cpu().numpy() - ref)) <= NORM_ATOL
    assert torch.equal(y, mbq().rmsnorm(xd, gd, 1e-6))
    assert torch.equal(xq, mbq().stage_x(fmt, y))
    # without the fp32 output, and in place
    _, xq2 = mbq().rmsnorm_xq(xd, gd, 1e-6, fmt, write_y=False)
    assert torch.equal(xq2, xq)
    xc = xd.clone()
    mbq().rmsnorm_xq(xc, gd, 1e-6, fmt, out=xc)
    assert torch.equal(xc, y)


@pytest.mark.parametrize("fmt,n", [(2, 12288), (1, 12288), (3, 1024), (0, 1024), (1, 96)])
def test_silu_mul_xq(fmt, n):
    rng = np.random.default_rng(n)
    gv = (rng.normal(size=n) * 4).astype(np.float32)
    uv = rng.normal(size=n).astype(np.float32)
    gd, ud = dev(gv), dev(uv)
    m = mbq().silu_mul(gd, ud)
    xq = mbq().silu_mul_xq(gd, ud, fmt)
    assert torch.equal(xq, mbq().stage_x(fmt, m))


def test_decode_half_layer_through_staged_inputs():
    """rmsnorm_xq -> gemv_xq (gate) and (up) -> silu_mul_xq -> gemv_xq (down,
    accumulating into h): the chain at reduced width against the oracle's
    single steps."""
    d, f = 512, 1536
    rng = np.random.default_rng(99)
    h = rng.normal(size=d).astype(np.float32)
    gam = rng.uniform(0.5, 1.5, d).astype(np.float32)
    _, og, Wg = weights(1, f, d, 7301)
    _, ou, Wu = weights(1, f, d, 7302)
    _, od, Wd = weights(2, d, f, 7303)
    hd = dev(h)
    _, bq = mbq().rmsnorm_xq(hd, dev(gam), 1e-6, 1, write_y=False)
    gv = mbq().gemv_xq(Wg, bq)
    uv = mbq().gemv_xq(Wu, bq)
    mq = mbq().silu_mul_xq(gv, uv, 2)
    mbq().gemv_xq(Wd, mq, out=hd, accumulate=True)
    b = oracle.rmsnorm(h, gam, 1e-6)[0]
    g_ref = oracle.gemv(og, b)[0]
    u_ref = oracle.gemv(ou, b)[0]
    m_ref = oracle.silu_mul(g_ref, u_ref)
    h_ref = oracle.gemv(od, m_ref)[0].astype(np.float64) + h
    got = hd.cpu().numpy().astype(np.float64)
    e = np.linalg.norm(got - h_ref) / np.linalg.norm(h_ref)
    assert e <= 1e-4, e
