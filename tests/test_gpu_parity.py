"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars (written in each test):
  * integer codes and dequantized fp32 weights: bit-exact;
  * GEMV outputs: relative L2 error <= 1e-4 over the whole output;
  * norm outputs: max absolute error <= 1e-5.
Inputs are the seeded synthetic workloads (workloads.py) at sizes the oracle
finishes in seconds, plus the full-size shapes of the five workloads.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from checks import GEMV_RTOL, NORM_ATOL, check_gemv, rel_l2  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_quantized_amd  # noqa: F401  (fails loudly if libmbq.so is missing)


def mbq():
    import memory_bound_quantized_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def weights(fmt, N, K, seed):
    planes = workloads.weight_planes(np.random.default_rng(seed), fmt, N, K)
    return planes, oracle.Planes(fmt, N, K, planes), mbq().QWeight.from_host(fmt, N, K, planes)


# --------------------------------------------------------------------------
# in-register unpack: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,N,K", [(1, 37, 512), (1, 5, 4096), (2, 37, 512), (2, 3, 12288),
                                     (3, 37, 512), (3, 9, 4096), (0, 37, 520), (0, 3, 4096)])
def test_device_unpack_and_dequant_bit_exact(fmt, N, K):
    _, ow, dw = weights(fmt, N, K, 1000 + fmt)
    w = mbq().dequant_f32(dw).cpu().numpy()
    ref = oracle.dequant(ow)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))
    if fmt != 0:
        q = mbq().unpack_codes(dw).cpu().numpy()
        assert np.array_equal(q, oracle.codes(ow))


def test_device_dequant_of_hand_fixtures(golden_dir):
    import json, os
    cases = json.load(open(os.path.join(golden_dir, "format_fixtures.json")))["cases"]
    for c in cases:
        if c["fmt"] == 3 and c["K"] % 64:
            continue   # the Q25 kernels need K % 64 == 0
        if c["fmt"] == 0 and c["K"] % 8:
            continue
        planes = [None if p is None else np.array(p, np.uint8) for p in c["planes"]]
        dw = mbq().QWeight.from_host(c["fmt"], c["N"], c["K"], planes)
        w = mbq().dequant_f32(dw).cpu().numpy().astype(np.float64)
        assert np.array_equal(w, np.array(c["weights"])), c["name"]


# --------------------------------------------------------------------------
# M = 1 GEMV
# --------------------------------------------------------------------------

GEMV_CASES = [
    (1, 1, 32), (1, 64, 32), (1, 37, 512), (1, 300, 4096), (1, 1000, 2080), (1, 2500, 4096),
    (1, 9000, 256), (1, 70000, 256), (1, 64, 12288),
    (2, 1, 256), (2, 64, 256), (2, 37, 512), (2, 300, 4096), (2, 2500, 2304), (2, 9000, 256), (2, 40, 12288),
    (3, 1, 64), (3, 64, 64), (3, 37, 512), (3, 300, 4096), (3, 2500, 4160), (3, 9000, 256),
    (0, 1, 8), (0, 64, 8), (0, 37, 520), (0, 512, 4096), (0, 3000, 1024),
]


@pytest.mark.parametrize("fmt,N,K", GEMV_CASES)
def test_gemv_m1_matches_oracle(fmt, N, K):
    _, ow, dw = weights(fmt, N, K, 7 * N + K + fmt)
    x = np.random.default_rng(N + K).normal(size=K).astype(np.float32)
    y = mbq().gemv_q(dw, dev(x)).cpu().numpy()
    ref = oracle.gemv_parallel(ow, x)[0]
    check_gemv(y, ow, x, ref)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_gemv_m1_accumulate(fmt):
    N, K = 333, 1024
    _, ow, dw = weights(fmt, N, K, 77 + fmt)
    rng = np.random.default_rng(3)
    x = rng.normal(size=K).astype(np.float32)
    y0 = rng.normal(size=N).astype(np.float32) * 10
    yd = dev(y0)
    mbq().gemv_q(dw, dev(x), out=yd, accumulate=True)
    ref = oracle.gemv(ow, x, y0=y0)[0]
    check_gemv(yd.cpu().numpy(), ow, x, ref, y0=y0)


def test_gemv_k_zero_and_empty():
    m = mbq()
    dw = m.QWeight(1, 10, 0, [torch.zeros(16, dtype=torch.uint8, device="cuda"), None,
                             torch.zeros(16, dtype=torch.uint8, device="cuda"), None])
    y = torch.full((10,), 5.0, device="cuda")
    m.gemv_q(dw, torch.zeros(4, device="cuda"), out=y)
    assert torch.all(y == 0).item()
    y.fill_(5.0)
    m.gemv_q(dw, torch.zeros(4, device="cuda"), out=y, accumulate=True)
    assert torch.all(y == 5).item()


def test_gemv_special_case_codes_at_offset_give_zero():
    N, K = 100, 4096
    codes = np.full((N, K), 8, np.uint8)
    sc = np.full(N * K // 32, 0x3C00, np.uint16)
    planes = mbq().pack(1, N, K, codes, sc)
    dw = mbq().QWeight.from_host(1, N, K, planes)
    x = np.random.default_rng(0).normal(size=K).astype(np.float32)
    y = mbq().gemv_q(dw, dev(x)).cpu().numpy()
    # every weight is 0: the integer block sums are 0, so y is exactly 0
    assert np.all(y == 0.0), np.max(np.abs(y))


# --------------------------------------------------------------------------
# the full-size workloads
# --------------------------------------------------------------------------

def test_workload2_full_size():
    """Q45 12288 x 4096 and Q65 4096 x 12288, M = 1, every output checked."""
    cfg = workloads.config2()
    for key, xkey in (("up", "x_up"), ("down", "x_down")):
        fmt, N, K, planes = cfg[key]
        ow = oracle.Planes(fmt, N, K, planes)
        dw = mbq().QWeight.from_host(fmt, N, K, planes)
        y = mbq().gemv_q(dw, dev(cfg[xkey])).cpu().numpy()
        ref = oracle.gemv_parallel(ow, cfg[xkey])[0]
        e = check_gemv(y, ow, cfg[xkey], ref)
        print("workload2 %s rel_l2=%.3e" % (key, e))


def test_workload1_full_size():
    """RMSNorm of one 4096 row, then the bf16 512 x 4096 product."""
    cfg = workloads.config1()
    x, g = dev(cfg["x"]), dev(cfg["gamma"])
    h = mbq().rmsnorm(x, g, cfg["eps"])
    h_ref = oracle.rmsnorm(cfg["x"], cfg["gamma"], cfg["eps"])[0]
    assert np.max(np.abs(h.cpu().numpy() - h_ref)) <= NORM_ATOL
    fmt, N, K, planes = cfg["W"]
    dw = mbq().QWeight.from_host(fmt, N, K, planes)
    y = mbq().gemv_q(dw, h).cpu().numpy()
    ow = oracle.Planes(fmt, N, K, planes)
    ref = oracle.gemv(ow, h.cpu().numpy())[0]
    check_gemv(y, ow, h.cpu().numpy(), ref)
    # and against the chain computed entirely by the oracle
    assert rel_l2(y, oracle.gemv(ow, h_ref)[0]) <= GEMV_RTOL


def test_workload5_full_size():
    """8 selected Q25 experts of 1536 x 4096 in one launch; LayerNorm 4096 x 2048."""
    cfg = workloads.config5()
    fmt, N, K, planes = cfg["W"]
    ow = oracle.Planes(fmt, N, K, planes)
    dw = mbq().QWeight.from_host(fmt, N, K, planes)
    idx = cfg["idx"]
    y = mbq().gemv_q_gather(dw, cfg["rows_per_expert"], dev(idx), dev(cfg["x"])).cpu().numpy()
    R = cfg["rows_per_expert"]
    for i, e in enumerate(idx):
        sub = oracle.Planes(fmt, R, K, [None if p is None else p.reshape(N, -1)[e * R:(e + 1) * R].reshape(-1)
                                        for p in planes])
        check_gemv(y[i], sub, cfg["x"], oracle.gemv_parallel(sub, cfg["x"])[0])
    yl = mbq().layernorm(dev(cfg["ln_x"]), dev(cfg["ln_gamma"]), dev(cfg["ln_beta"]), cfg["ln_eps"])
    ref = oracle.layernorm(cfg["ln_x"], cfg["ln_gamma"], cfg["ln_beta"], cfg["ln_eps"])
    assert np.max(np.abs(yl.cpu().numpy() - ref)) <= NORM_ATOL


def test_gather_small_matches_oracle_gather():
    E, R, K = 6, 40, 512
    for fmt in (1, 2, 3, 0):
        _, ow, dw = weights(fmt, E * R, K, 90 + fmt)
        idx = np.array([5, 0, 3, 3], np.int32)
        x = np.random.default_rng(1).normal(size=K).astype(np.float32)
        y = mbq().gemv_q_gather(dw, R, dev(idx), dev(x)).cpu().numpy()
        assert rel_l2(y, oracle.gather(ow, R, idx, x)) <= GEMV_RTOL
        for i, e in enumerate(idx):
            sub = oracle.Planes(fmt, R, K, [None if p is None else p.reshape(E * R, -1)[e * R:(e + 1) * R].reshape(-1)
                                            for p in ow.planes])
            check_gemv(y[i], sub, x, oracle.gemv(sub, x)[0])


# --------------------------------------------------------------------------
# norms and glue
# --------------------------------------------------------------------------

@pytest.mark.parametrize("rows,n", [(1, 4096), (3, 4096), (2, 2048), (5, 1000), (2, 8192),
                                    (2, 10000), (1, 4), (1, 3), (64, 256), (1, 1024), (1, 1028),
                                    (2, 16384), (1, 32768), (1, 32772)])
def test_rmsnorm_matches_oracle(rows, n):
    """Every geometry of the single-pass kernel (256 threads up to 1024
    values, then 1024 threads with 1, 2, 4 or 8 float4s each up to 32768)
    and the any-n kernel beyond it or for n % 4 != 0."""
    rng = np.random.default_rng(rows * n)
    x = rng.normal(size=(rows, n)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, n).astype(np.float32)
    ref = oracle.rmsnorm(x, g, 1e-6)
    y = mbq().rmsnorm(dev(x), dev(g), 1e-6).cpu().numpy()
    assert np.max(np.abs(y - ref)) <= NORM_ATOL
    xd = dev(x)
    mbq().rmsnorm(xd, dev(g), 1e-6, out=xd)          # in place
    assert np.max(np.abs(xd.cpu().numpy() - ref)) <= NORM_ATOL


@pytest.mark.parametrize("rows,n", [(4, 2048), (1, 4096), (3, 1000), (2, 8192), (2, 9000),
                                    (1, 5), (128, 2048)])
def test_layernorm_matches_oracle(rows, n):
    rng = np.random.default_rng(rows + n)
    x = rng.normal(3, 2, size=(rows, n)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, n).astype(np.float32)
    b = rng.normal(0, 0.1, n).astype(np.float32)
    ref = oracle.layernorm(x, g, b, 1e-5)
    y = mbq().layernorm(dev(x), dev(g), dev(b), 1e-5).cpu().numpy()
    assert np.max(np.abs(y - ref)) <= NORM_ATOL
    xd = dev(x)
    mbq().layernorm(xd, dev(g), dev(b), 1e-5, out=xd)
    assert np.max(np.abs(xd.cpu().numpy() - ref)) <= NORM_ATOL


def test_norm_special_cases_on_device():
    m = mbq()
    g = np.random.default_rng(0).uniform(0.5, 1.5, 2048).astype(np.float32)
    b = np.random.default_rng(1).normal(0, 0.1, 2048).astype(np.float32)
    # constant row: LayerNorm gives beta exactly
    y = m.layernorm(dev(np.full((2, 2048), 7.25, np.float32)), dev(g), dev(b), 1e-5).cpu().numpy()
    assert np.array_equal(y, np.stack([b, b]))
    # small-integer rows: every partial sum is exact, so the cooperative
    # reduction equals the serial one bit for bit
    xi = np.random.default_rng(2).integers(-8, 9, size=(3, 2048)).astype(np.float32)
    ones = np.ones(2048, np.float32)
    y = m.rmsnorm(dev(xi), dev(ones), 0.0).cpu().numpy()
    assert np.array_equal(y, oracle.rmsnorm_serial_f32(xi, ones, 0.0))
    # power-of-two invariance
    x = np.random.default_rng(3).normal(size=(2, 4096)).astype(np.float32)
    g4 = np.ones(4096, np.float32)
    a = m.rmsnorm(dev(x), dev(g4), 1e-6).cpu().numpy()
    c = m.rmsnorm(dev(2 * x), dev(g4), 4e-6).cpu().numpy()
    assert np.array_equal(a, c)


def test_silu_mul_matches_oracle():
    rng = np.random.default_rng(5)
    g = rng.normal(0, 4, 12288).astype(np.float32)
    u = rng.normal(0, 4, 12288).astype(np.float32)
    y = mbq().silu_mul(dev(g), dev(u)).cpu().numpy()
    ref = oracle.silu_mul(g, u)
    assert np.max(np.abs(y - ref) / (np.abs(ref) + 1e-30)) <= 1e-5
