"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests touch the product library or a GPU.  Each pin is chosen
so that a plausible slip in the oracle (a wrong nibble order, a dropped
offset, a transposed index, an unbiased variance, a missing eps) fails one.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import closed_forms as cf

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden(name):
    with open(os.path.join(HERE, "golden", name)) as fh:
        return json.load(fh)


def _planes_from_fixture(case):
    return oracle.Planes(case["fmt"], case["N"], case["K"],
                         [None if p is None else np.array(p, np.uint8) for p in case["planes"]])


# ---------------------------------------------------------------------------
# scalar decoders
# ---------------------------------------------------------------------------

def test_f16_decoder_known_patterns():
    assert oracle.f16_to_f64(0x3C00) == 1.0
    assert oracle.f16_to_f64(0xC000) == -2.0
    assert oracle.f16_to_f64(0x7BFF) == 65504.0
    assert oracle.f16_to_f64(0x0400) == 2.0 ** -14          # smallest normal
    assert oracle.f16_to_f64(0x0001) == 2.0 ** -24          # smallest subnormal
    assert oracle.f16_to_f64(0x03FF) == 1023 * 2.0 ** -24   # largest subnormal
    assert oracle.f16_to_f64(0x3555) == 1365 * 2.0 ** -12   # 0.333251953125
    assert math.isinf(oracle.f16_to_f64(0x7C00)) and oracle.f16_to_f64(0xFC00) < 0
    assert math.isnan(oracle.f16_to_f64(0x7E00))
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0


def test_f16_decoder_matches_numpy_on_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_bf16_decoder():
    words = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x4049, 0x8000], np.uint16)
    ref = (words.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for w, r in zip(words, ref):
        assert oracle.bf16_to_f64(int(w)) == r
    assert oracle.bf16_to_f64(0x4049) == 3.140625


# ---------------------------------------------------------------------------
# storage sizes: bits per weight (pages: 4.5 / 6.5625; 144 and 210 B per 256)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,bpw", [(oracle.BF16, 16.0), (oracle.Q45, 4.5),
                                     (oracle.Q65, 6.5625), (oracle.Q25, 2.5)])
def test_bits_per_weight(fmt, bpw):
    for N, K in [(1, 256), (3, 512), (12288, 4096), (4096, 12288)]:
        total = sum(oracle.plane_bytes(fmt, N, K))
        assert total * 8 == bpw * N * K
        assert Fraction(total * 8, N * K) == cf.BITS_PER_WEIGHT[fmt]


def test_bytes_per_256_weights_match_pages():
    pages = _golden("page_numbers.json")
    assert sum(oracle.plane_bytes(oracle.Q45, 1, 256)) == pages["q4k_bytes_per_256"]["value"]
    assert sum(oracle.plane_bytes(oracle.Q65, 1, 256)) == pages["q6k_bytes_per_256"]["value"]
    assert float(cf.BITS_PER_WEIGHT[1]) == pages["q4_bits_per_weight"]["value"]
    assert float(cf.BITS_PER_WEIGHT[2]) == pages["q6_bits_per_weight"]["value"]


def test_plane_sizes_reject_ragged_blocks():
    for fmt, K in [(oracle.Q45, 48), (oracle.Q25, 16), (oracle.Q65, 128)]:
        with pytest.raises(ValueError):
            oracle.plane_bytes(fmt, 4, K)


# ---------------------------------------------------------------------------
# decoders against hand-derived fixtures
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _golden("format_fixtures.json")["cases"], ids=lambda c: c["name"])
def test_decode_fixture(case):
    W = _planes_from_fixture(case)
    if case["codes"] is not None:
        assert oracle.codes(W).tolist() == case["codes"]
    got = oracle.dequant(W).astype(np.float64)
    assert np.array_equal(got, np.array(case["weights"], np.float64))


@pytest.mark.parametrize("fmt,N,K", [(1, 5, 96), (2, 3, 512), (3, 4, 160)])
def test_pack_then_decode_round_trip(fmt, N, K):
    rng = np.random.default_rng(7)
    bits = {1: 4, 2: 6, 3: 2}[fmt]
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    if fmt == 2:
        sc = rng.integers(-128, 128, size=N * K // 16).astype(np.int8)
        su = np.float16(rng.uniform(0.001, 0.02, N * K // 256)).view(np.uint16)
    else:
        sc = np.float16(rng.uniform(0.001, 0.02, N * K // 32)).view(np.uint16)
        su = None
    W = oracle.pack(fmt, N, K, codes, sc, su)
    assert np.array_equal(oracle.codes(W), codes)


def test_pack_rejects_out_of_range_codes():
    codes = np.full((1, 32), 16, np.uint8)
    with pytest.raises(ValueError):
        oracle.pack(oracle.Q45, 1, 32, codes, np.zeros(1, np.uint16))


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_dequantized_weights_exact_in_binary32(fmt):
    """Every dequantized weight is a product that binary32 represents exactly,
    so the bit-exact dequant target is order-free."""
    import workloads
    rng = np.random.default_rng(11)
    W = oracle.Planes(fmt, 16, 512, workloads.weight_planes(rng, fmt, 16, 512))
    for n in range(16):
        for k in range(0, 512, 7):
            w = oracle.weight(W, n, k)
            assert float(np.float32(w)) == w


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------

def _rand_w(fmt, N, K, seed):
    import workloads
    return oracle.Planes(fmt, N, K, workloads.weight_planes(np.random.default_rng(seed), fmt, N, K))


@pytest.mark.parametrize("fmt,K", [(0, 64), (1, 64), (2, 256), (3, 64)])
def test_gemv_against_exact_rational_brute_force(fmt, K):
    """8 x K with exact rational sums (each weight taken from the pinned
    decoder); the oracle's single double rounding must land within one
    binary32 ulp of the exactly rounded result."""
    N = 8
    W = _rand_w(fmt, N, K, 100 + fmt)
    x = np.random.default_rng(5).normal(size=(2, K)).astype(np.float32)
    y = oracle.gemv(W, x)
    for m in range(2):
        for n in range(N):
            exact = sum(Fraction(oracle.weight(W, n, k)) * Fraction(float(x[m, k]))
                        for k in range(K))
            ref = np.float32(float(exact))
            assert abs(float(y[m, n]) - float(ref)) <= float(np.spacing(np.abs(ref))), (m, n)


def test_gemv_matches_library_matmul_of_decoded_weights():
    W = _rand_w(1, 37, 256, 3)
    x = np.random.default_rng(9).normal(size=(3, 256)).astype(np.float32)
    ref = (x.astype(np.float64) @ oracle.dequant(W).astype(np.float64).T).astype(np.float32)
    assert np.array_equal(oracle.gemv(W, x), ref) or \
        np.max(np.abs(oracle.gemv(W, x) - ref) / (np.abs(ref) + 1e-30)) < 1e-6


def test_gemv_special_cases():
    K, N = 96, 3
    x = np.random.default_rng(1).normal(size=K).astype(np.float32)
    one = np.full(N * K // 32, 0x3C00, np.uint16)
    # all codes at the offset -> exactly zero
    W0 = oracle.pack(1, N, K, np.full((N, K), 8, np.uint8), one)
    assert np.all(oracle.gemv(W0, x) == 0.0)
    # codes one above the offset with scale 1 -> the sum of x
    W1 = oracle.pack(1, N, K, np.full((N, K), 9, np.uint8), one)
    assert np.all(oracle.gemv(W1, x) == np.float32(math.fsum(float(v) for v in x)))
    # a single non-zero weight picks out one x, exactly
    c = np.full((N, K), 8, np.uint8)
    c[1, 77] = 15
    sc = one.copy()
    sc[1 * 3 + 77 // 32] = 0x4000          # 2.0 on the block holding k = 77
    Ws = oracle.pack(1, N, K, c, sc)
    y = oracle.gemv(Ws, x)[0]
    assert y[0] == 0 and y[2] == 0 and y[1] == np.float32(2.0 * 7 * float(x[77]))
    # Q25 with the same construction
    c2 = np.full((N, K), 2, np.uint8)
    c2[2, 5] = 0
    W2 = oracle.pack(3, N, K, c2, one)
    assert oracle.gemv(W2, x)[0].tolist() == [0.0, 0.0, float(np.float32(-2.0 * float(x[5])))]


def test_gemv_power_of_two_scaling_and_accumulate():
    W = _rand_w(2, 9, 512, 4)
    x = np.random.default_rng(2).normal(size=512).astype(np.float32)
    y = oracle.gemv(W, x)
    assert np.array_equal(oracle.gemv(W, x * np.float32(8)), y * np.float32(8))
    assert np.array_equal(oracle.gemv(W, x * np.float32(0.25)), y * np.float32(0.25))
    y0 = np.random.default_rng(3).normal(size=(1, 9)).astype(np.float32)
    ya = oracle.gemv(W, x, y0=y0)
    ref = (y0.astype(np.float64) + oracle.dequant(W).astype(np.float64) @ x.astype(np.float64))
    assert np.allclose(ya, ref.astype(np.float32), rtol=1e-6, atol=0)


def test_gemv_rows_of_a_batch_are_independent_and_row_ranges_compose():
    W = _rand_w(1, 20, 128, 8)
    X = np.random.default_rng(4).normal(size=(4, 128)).astype(np.float32)
    Y = oracle.gemv(W, X)
    for m in range(4):
        assert np.array_equal(Y[m], oracle.gemv(W, X[m])[0])
    part = oracle.gemv(W, X, rows=(5, 11))
    assert np.array_equal(part[:, 5:11], Y[:, 5:11])
    assert np.all(part[:, :5] == 0) and np.all(part[:, 11:] == 0)
    assert np.array_equal(oracle.gemv_parallel(W, X, threads=3), Y)


def test_gather_selects_expert_rows():
    E, R, K = 6, 4, 64
    codes = np.zeros((E * R, K), np.uint8)
    for e in range(E):
        codes[e * R:(e + 1) * R] = e % 4
    W = oracle.pack(3, E * R, K, codes, np.full(E * R * K // 32, 0x3C00, np.uint16))
    x = np.random.default_rng(6).normal(size=K).astype(np.float32)
    sx = math.fsum(float(v) for v in x)
    idx = np.array([5, 0, 3], np.int32)
    y = oracle.gather(W, R, idx, x)
    for i, e in enumerate(idx):
        assert np.all(y[i] == np.float32((e % 4 - 2) * sx))
    Wr = _rand_w(1, E * R, K, 12)
    yr = oracle.gather(Wr, R, idx, x)
    full = oracle.gemv(Wr, x)[0]
    for i, e in enumerate(idx):
        assert np.array_equal(yr[i], full[e * R:(e + 1) * R])


# ---------------------------------------------------------------------------
# norms
# ---------------------------------------------------------------------------

def test_rmsnorm_hand_values():
    y = oracle.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 1.0]), 0.0)[0]
    # mean square 12.5 -> 3/sqrt(12.5), 4/sqrt(12.5)
    assert y.tolist() == [np.float32(0.848528137423857), np.float32(1.131370849898476)]
    y = oracle.rmsnorm(np.array([2.0, -2.0, 2.0, -2.0]), np.array([1.0, 2.0, 3.0, 4.0]), 0.0)[0]
    assert y.tolist() == [1.0, -4.0 / 2, 3.0, -4.0]
    # eps inside the root: x = (1, 1), eps = 3 -> 1/sqrt(1 + 3) = 0.5
    assert oracle.rmsnorm(np.ones(2), np.ones(2), 3.0)[0].tolist() == [0.5, 0.5]


def test_rmsnorm_constant_row_and_power_of_two_invariance():
    g = np.random.default_rng(0).uniform(0.5, 1.5, 64).astype(np.float32)
    c, eps = np.float32(1.75), 1e-6
    y = oracle.rmsnorm(np.full(64, c), g, eps)[0]
    ref = (g.astype(np.float64) * c / math.sqrt(float(c) ** 2 + eps)).astype(np.float32)
    assert np.array_equal(y, ref)
    x = np.random.default_rng(1).normal(size=(3, 4096)).astype(np.float32)
    gg = np.random.default_rng(2).uniform(0.5, 1.5, 4096).astype(np.float32)
    assert np.array_equal(oracle.rmsnorm(2 * x, gg, 4e-6), oracle.rmsnorm(x, gg, 1e-6))


def test_serial_and_parallel_norms_agree():
    """The cooperative reduction must match the serial one to the last bit
    that matters ([one-serial-kernel] "One thread"): bit-identical on rows
    whose partial sums are all exact, within 1e-5 on random rows."""
    rng = np.random.default_rng(3)
    xi = rng.integers(-8, 9, size=(4, 2048)).astype(np.float32)
    g = np.ones(2048, np.float32)
    a = oracle.rmsnorm_serial_f32(xi, g, 0.0)
    b = oracle.rmsnorm_tree_f32(xi, g, 0.0, threads=256)
    c = oracle.rmsnorm(xi, g, 0.0)
    # sums of squares are exact integers in float; only the final scale rounds
    assert np.array_equal(a, b)
    assert np.max(np.abs(a - c)) <= 2 * np.max(np.spacing(np.abs(c)))
    xr = rng.normal(size=(4, 4096)).astype(np.float32)
    gr = rng.uniform(0.5, 1.5, 4096).astype(np.float32)
    ref = oracle.rmsnorm(xr, gr, 1e-6)
    assert np.max(np.abs(oracle.rmsnorm_serial_f32(xr, gr, 1e-6) - ref)) <= 1e-5
    assert np.max(np.abs(oracle.rmsnorm_tree_f32(xr, gr, 1e-6) - ref)) <= 1e-5
    xl = rng.normal(3, 2, size=(4, 2048)).astype(np.float32)
    be = rng.normal(0, 0.1, 2048).astype(np.float32)
    assert np.max(np.abs(oracle.layernorm_serial_f32(xl, g, be, 1e-5)
                         - oracle.layernorm(xl, g, be, 1e-5))) <= 1e-5


def test_layernorm_hand_values():
    y = oracle.layernorm(np.array([1.0, 2.0, 3.0, 4.0]), np.ones(4), np.zeros(4), 0.0)[0]
    # mean 2.5, biased variance 1.25
    s = 1.0 / math.sqrt(1.25)
    assert y.tolist() == [np.float32(-1.5 * s), np.float32(-0.5 * s),
                          np.float32(0.5 * s), np.float32(1.5 * s)]
    # biased (divide by n), not unbiased: (0, 2) -> variance 1 -> (-1, 1)
    assert oracle.layernorm(np.array([0.0, 2.0]), np.ones(2), np.zeros(2), 0.0)[0].tolist() == [-1.0, 1.0]
    # large common offset: 2^24 and 2^24 + 2 -> (-1, 1) * gamma + beta exactly
    y = oracle.layernorm(np.array([2.0 ** 24, 2.0 ** 24 + 2]), np.array([3.0, 5.0]),
                         np.array([0.5, -0.5]), 0.0)[0]
    assert y.tolist() == [-2.5, 4.5]


def test_layernorm_constant_row_is_beta_and_power_of_two_invariance():
    rng = np.random.default_rng(4)
    g = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    b = rng.normal(0, 0.1, 128).astype(np.float32)
    assert np.array_equal(oracle.layernorm(np.full(128, 7.25), g, b, 1e-5)[0], b)
    x = rng.normal(3, 2, size=(5, 2048)).astype(np.float32)
    g2 = rng.uniform(0.5, 1.5, 2048).astype(np.float32)
    b2 = rng.normal(0, 0.1, 2048).astype(np.float32)
    assert np.array_equal(oracle.layernorm(4 * x, g2, b2, 16e-5), oracle.layernorm(x, g2, b2, 1e-5))


def test_layernorm_matches_textbook_numpy():
    rng = np.random.default_rng(5)
    x = rng.normal(3, 2, size=(6, 2048)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 2048).astype(np.float32)
    b = rng.normal(0, 0.1, 2048).astype(np.float32)
    xd = x.astype(np.float64)
    ref = (xd - xd.mean(1, keepdims=True)) / np.sqrt(xd.var(1, keepdims=True) + 1e-5) * g + b
    assert np.max(np.abs(oracle.layernorm(x, g, b, 1e-5) - ref)) < 1e-6


def test_silu_mul():
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0], np.float32)
    u = np.array([5.0, 1.0, 2.0, 1.0, 1.0], np.float32)
    y = oracle.silu_mul(g, u)
    assert y[0] == 0.0
    assert y[1] == np.float32(1.0 / (1.0 + math.exp(-1.0)))
    # silu(t) - silu(-t) = t
    assert abs(float(oracle.silu_mul(np.array([1.0]), np.ones(1))[0])
               - float(oracle.silu_mul(np.array([-1.0]), np.ones(1))[0]) - 1.0) < 1e-7
    assert y[3] == np.float32(30.0 / (1.0 + math.exp(-30.0)))
    assert abs(float(y[4])) < 1e-11


# ---------------------------------------------------------------------------
# decode chain
# ---------------------------------------------------------------------------

def _tiny_model(L=2, d=256, dq=256, dkv=64, f=512, V=96, zero_residual=False):
    import workloads
    rng = np.random.default_rng(21)
    layers = []
    for l in range(L):
        lay = {}
        for name, (fmt, N, K) in dict(q=(1, dq, d), k=(1, dkv, d), v=(1, dkv, d), o=(1, d, dq),
                                      gate=(1, f, d), up=(1, f, d),
                                      down=(2 if l % 2 == 0 else 1, d, f)).items():
            if zero_residual and name in ("o", "down"):
                if fmt == 1:
                    codes = np.full((N, K), 8, np.uint8)
                    lay[name] = oracle.pack(1, N, K, codes, np.full(N * K // 32, 0x3C00, np.uint16))
                else:
                    codes = np.full((N, K), 32, np.uint8)
                    lay[name] = oracle.pack(2, N, K, codes, np.ones(N * K // 16, np.int8),
                                            np.full(N * K // 256, 0x3C00, np.uint16))
            else:
                lay[name] = oracle.Planes(fmt, N, K, workloads.weight_planes(rng, fmt, N, K))
        layers.append(lay)
    vocab = oracle.Planes(2, V, d, workloads.weight_planes(rng, 2, V, d))
    g1 = rng.uniform(0.5, 1.5, L * d).astype(np.float32)
    g2 = rng.uniform(0.5, 1.5, L * d).astype(np.float32)
    gf = rng.uniform(0.5, 1.5, d).astype(np.float32)
    h0 = rng.normal(size=d).astype(np.float32)
    return layers, vocab, g1, g2, gf, h0


def test_decode_chain_with_zero_residual_branches_keeps_h():
    layers, vocab, g1, g2, gf, h0 = _tiny_model(zero_residual=True)
    h, logits = oracle.decode_token(layers, vocab, g1, g2, gf, 1e-6, h0)
    assert np.array_equal(h, h0)
    assert np.array_equal(logits, oracle.gemv(vocab, oracle.rmsnorm(h0, gf, 1e-6))[0])


def test_decode_chain_is_the_composition_of_the_pinned_steps():
    layers, vocab, g1, g2, gf, h0 = _tiny_model()
    h, logits, trace = oracle.decode_token(layers, vocab, g1, g2, gf, 1e-6, h0, trace=True)
    d = h0.size
    hh = h0.copy()
    for l, lay in enumerate(layers):
        a = oracle.rmsnorm(hh, g1[l * d:(l + 1) * d], 1e-6)
        q = oracle.gemv(lay["q"], a)
        hh = oracle.gemv(lay["o"], q, y0=hh)[0]
        b = oracle.rmsnorm(hh, g2[l * d:(l + 1) * d], 1e-6)
        m = oracle.silu_mul(oracle.gemv(lay["gate"], b), oracle.gemv(lay["up"], b))
        hh = oracle.gemv(lay["down"], m, y0=hh)[0]
        assert np.array_equal(trace[l], hh)
    assert np.array_equal(h, hh)
    assert np.array_equal(logits, oracle.gemv(vocab, oracle.rmsnorm(hh, gf, 1e-6))[0])


def test_row_parallel_chain_equals_the_serial_chain_bit_for_bit():
    """decode_token_parallel (each product's rows split over threads, used for
    the full-size 36-layer token) is decode_token's result exactly."""
    layers, vocab, g1, g2, gf, h0 = _tiny_model(L=3)
    h, logits = oracle.decode_token(layers, vocab, g1, g2, gf, 1e-6, h0)
    for threads in (1, 3, 8):
        hp, lp = oracle.decode_token_parallel(layers, vocab, g1, g2, gf, 1e-6, h0, threads=threads)
        assert np.array_equal(hp, h) and np.array_equal(lp, logits)


def test_row_parallel_accumulate_equals_gemv():
    import workloads
    rng = np.random.default_rng(5)
    for fmt, N, K in ((1, 300, 512), (2, 77, 512), (3, 50, 256), (0, 33, 64)):
        W = oracle.Planes(fmt, N, K, workloads.weight_planes(rng, fmt, N, K))
        x = rng.normal(size=K).astype(np.float32)
        y0 = rng.normal(size=N).astype(np.float32)
        assert np.array_equal(oracle.gemv_parallel(W, x, 5, y0=y0), oracle.gemv(W, x, y0=y0))


def test_norms_per_token_match_page():
    """Two norms per layer plus one at the end: 73 for 36 layers
    ([one-serial-kernel] "One thread")."""
    pages = _golden("page_numbers.json")
    assert 2 * cf.LAYERS + 1 == pages["norms_per_token"]["value"]


# ---------------------------------------------------------------------------
# closed forms against the pages' printed numbers
# ---------------------------------------------------------------------------

def _r(v, digits):
    return round(v, digits)


def test_closed_forms_reproduce_page_numbers():
    P = {k: v for k, v in _golden("page_numbers.json").items() if not k.startswith("_")}
    V = lambda k: P[k]["value"]
    # sums per byte at 4.5 bits
    assert _r(cf.sums_per_byte(4.5), 1) == V("sums_per_byte_at_4p5_bits")
    # M* = (w/16)(R/BW): M4 numerator 1063 (BW in GB/s)
    assert int(cf.m_star(4.5, V("m4_sums_per_s"), 1e9)) == V("m4_mstar_numerator")
    assert _r(V("m3_sums_per_s") / V("m3_bw"), 0) == V("m3_sums_per_byte")
    assert _r(V("rtx5090_sums_per_s") / V("rtx5090_bw"), -1) == V("rtx5090_sums_per_byte")
    # tokens/s limits
    assert _r(cf.tokens_per_s_limit(V("m3_bw"), V("token_bytes")), 1) == V("m3_limit_tok_s")
    assert _r(cf.tokens_per_s_limit(V("m3_bw"), V("token_bytes") + V("kv_cache_bytes_512")), 1) \
        == V("m3_limit_512_tok_s")
    assert _r(cf.tokens_per_s_limit(V("m3_published_bw"), V("rtx_token_bytes_measured")), 1) \
        == V("m3_upper_bound_tok_s")
    # the ledger's vocab floor implies BW = 510504960 B / 300.06 us
    bw_ledger = cf.weight_bytes(2, cf.VOCAB * cf.D_MODEL) / Fraction("300.06e-6")
    assert cf.tokens_per_s_limit(float(bw_ledger), V("token_bytes")) < V("rtx_upper_bound_tok_s")
    assert _r(float(bw_ledger) / V("m3_bw"), 1) == V("bw_ratio")
    # floors
    assert _r(cf.floor_seconds(V("token_bytes"), V("m3_bw")) * 1e3, 0) == V("m3_floor_ms")
    assert _r(cf.floor_seconds(V("token_bytes"), V("rtx5090_bw")) * 1e3, 2) == V("rtx_floor_ms")
    vocab_bytes = cf.weight_bytes(2, cf.VOCAB * cf.D_MODEL)
    assert vocab_bytes == 510504960
    assert int(float(vocab_bytes) / 1e6) == V("vocab_bytes_mb")      # 510.5 MB, printed as 510
    assert _r(cf.floor_seconds(float(vocab_bytes), V("rtx5090_bw")) * 1e6, 0) == V("vocab_floor_us")
    # small tables at the ledger bandwidth
    kv = cf.weight_bytes(1, cf.D_KV * cf.D_MODEL)
    qo = cf.weight_bytes(1, cf.D_MODEL * cf.D_MODEL)
    assert _r(float(kv) / 1e6, 1) == V("kv_table_mb")
    lo, hi = V("small_table_floor_us")
    assert _r(cf.floor_seconds(float(kv), float(bw_ledger)) * 1e6, 1) == lo
    assert _r(cf.floor_seconds(float(qo), float(bw_ledger)) * 1e6, 1) in (hi, V("qo_table_floor_us"))
    # Little's law per microsecond of wait
    assert _r(cf.bytes_in_flight(float(bw_ledger), 1e-6) / 1e6, 1) * 1e6 == V("little_rtx_bytes_per_us")
    assert _r(cf.bytes_in_flight(V("m3_bw"), 1e-6) / 1e3, -1) * 1e3 == V("little_m3_bytes_per_us")
    # the copy method counts read and write: 45.0 GB copied = 90 GB/s of traffic
    assert _r(2 * V("m3_copy_gb_s") / 1e9, 0) == _r(V("m3_bw") / 1e9, 0)
    # tokens/s <-> ms per token on the M4 page
    assert _r(1e3 / V("decode_after_tok_s"), 1) == V("token_after_ms")
    assert _r(1e3 / V("decode_before_tok_s"), 1) == V("token_before_ms")


def test_token_census_close_to_page_figure():
    """The weight tables the stack reads come to 4.651 GB; the page's 4.68 GB
    counts the whole token (norm vectors and other small parts it lists in
    the model file), so the two agree to within 1 %."""
    B = cf.token_weight_bytes()
    assert B == 4651069440
    assert abs(B / _golden("page_numbers.json")["token_bytes"]["value"] - 1) < 0.01


def test_token_time_identity():
    # memory-bound: bytes win, F/R drops out
    t = cf.token_time(4.68e9, 89.9e9, 2 * 8e9, 3.152e12, 0.0)
    assert t == pytest.approx(4.68e9 / 89.9e9)
    t = cf.token_time(1.0, 1.0, 10.0, 1.0, 2.0)
    assert t == 12.0
