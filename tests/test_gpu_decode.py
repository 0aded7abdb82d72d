"""GPU parity of the fused products (mbq_gemv_fused) and of the decode step
(mbq_decode_step) against the CPU oracle, through the C ABI.

Bars: GEMV outputs within the fp32 forward-error bound and rel-L2 <= 1e-4
(checks.check_gemv) against the oracle applied step by step; the decode
step's final h and logits within rel-L2 1e-4 of oracle.decode_token (the
oracle's chain, fp32 between steps).  The norm prologue sums the row in a
different order from mbq_rmsnorm, so its result is compared with a tolerance:
max-abs 1e-5 on the normalised values is folded into the GEMV bound as an
input perturbation.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from checks import check_gemv, rel_l2  # noqa: E402


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


def mat(fmt, N, K, seed):
    return (fmt, N, K, workloads.weight_planes(np.random.default_rng(seed), fmt, N, K))


def check_after_norm(y, ow, a_ref, ref, y0=None):
    """GEMV bar on the normalised input a_ref, widened by what the norm bar
    allows: the device's normalised value may differ from a_ref by 1e-5 per
    element, which moves output n by at most 1e-5 * sum_k |w[n][k]|."""
    absw = np.abs(oracle.dequant(ow).astype(np.float64))
    check_gemv(y, ow, a_ref, ref, y0=y0, slack=1e-5 * absw.sum(axis=1))


@pytest.mark.parametrize("fmt,N,K", [(1, 1000, 4096), (1, 6144, 4096), (2, 300, 4096),
                                     (1, 256, 12288), (2, 64, 12288)])
def test_fused_rmsnorm_prologue(fmt, N, K):
    print("fused norm fmt=%d N=%d K=%d" % (fmt, N, K), flush=True)
    W = mat(fmt, N, K, 8000 + N + fmt)
    ow, dw = oracle.Planes(*W), mbq().QWeight.from_host(*W)
    rng = np.random.default_rng(K + N)
    x = rng.normal(size=K).astype(np.float32)
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    y = mbq().gemv_fused(dw, dev(x), dev(g), 1e-6).cpu().numpy()
    a = oracle.rmsnorm(x, g, 1e-6)[0]
    check_after_norm(y, ow, a, oracle.gemv(ow, a)[0])


@pytest.mark.parametrize("fmt,N,K", [(1, 1000, 4096), (1, 6144, 4096), (2, 300, 12288)])
def test_fused_rmsnorm_accumulate(fmt, N, K):
    """y += W rmsnorm(x): the norm's 1/rms scales each row's total before the
    add (ragged N, both K forms)."""
    print("fused norm accumulate fmt=%d N=%d K=%d" % (fmt, N, K), flush=True)
    W = mat(fmt, N, K, 8400 + N + fmt)
    ow, dw = oracle.Planes(*W), mbq().QWeight.from_host(*W)
    rng = np.random.default_rng(K + N + 7)
    x = rng.normal(size=K).astype(np.float32)
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    y0 = rng.normal(size=N).astype(np.float32)
    yd = dev(y0)
    mbq().gemv_fused(dw, dev(x), dev(g), 1e-6, mbq().EPI_ACCUMULATE, out=yd)
    a = oracle.rmsnorm(x, g, 1e-6)[0]
    check_after_norm(yd.cpu().numpy(), ow, a, oracle.gemv(ow, a, y0=y0)[0], y0=y0)


@pytest.mark.parametrize("fmt,f,K,norm", [(1, 512, 4096, True), (1, 512, 4096, False),
                                          (2, 300, 4096, True), (1, 128, 12288, False)])
def test_fused_silu_epilogue(fmt, f, K, norm):
    from memory_bound_quantized_amd.decode import interleave_rows
    print("fused silu fmt=%d f=%d K=%d norm=%s" % (fmt, f, K, norm), flush=True)
    G, U = mat(fmt, f, K, 8100 + f), mat(fmt, f, K, 8200 + f)
    dw = mbq().QWeight.from_host(*interleave_rows(G, U))
    rng = np.random.default_rng(f)
    x = rng.normal(size=K).astype(np.float32)
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    m = mbq().gemv_fused(dw, dev(x), dev(g) if norm else None, 1e-6,
                         mbq().EPI_SILU_MUL).cpu().numpy().astype(np.float64)
    a = oracle.rmsnorm(x, g, 1e-6)[0] if norm else x
    gr = oracle.gemv(oracle.Planes(*G), a)[0]
    ur = oracle.gemv(oracle.Planes(*U), a)[0]
    ref = oracle.silu_mul(gr, ur).astype(np.float64)
    # silu(g) * u moves a relative error of g, u by at most ~2x: rel-L2 bar on m
    assert rel_l2(m, ref) <= 1e-4


def test_fused_accumulate_without_norm():
    W = mat(1, 512, 4096, 8300)
    ow, dw = oracle.Planes(*W), mbq().QWeight.from_host(*W)
    rng = np.random.default_rng(1)
    x = rng.normal(size=4096).astype(np.float32)
    y0 = rng.normal(size=512).astype(np.float32)
    yd = dev(y0)
    mbq().gemv_fused(dw, dev(x), None, 0.0, mbq().EPI_ACCUMULATE, out=yd)
    check_gemv(yd.cpu().numpy(), ow, x, oracle.gemv(ow, x, y0=y0)[0], y0=y0)


def _oracle_chain(cfg):
    """oracle.decode_token on the stack (fp64 inside each step, fp32 between)."""
    lay = [{k: oracle.Planes(*v) for k, v in e.items()} for e in cfg["layers"]]
    return oracle.decode_token(lay, oracle.Planes(*cfg["vocab"]), cfg["g1"], cfg["g2"],
                               cfg["gf"], cfg["eps"], cfg["h0"])


@pytest.mark.parametrize("layers,vocab", [(2, 1000), (1, 4096)])
def test_decode_step_matches_oracle_chain(layers, vocab):
    from memory_bound_quantized_amd.decode import DecodeModel
    print("decode layers=%d vocab=%d" % (layers, vocab), flush=True)
    cfg = workloads.config3(layers=layers, vocab=vocab)
    model = DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])
    h = dev(cfg["h0"])
    logits = torch.empty(vocab, device="cuda")
    model.step(h, logits)
    h_ref, lg_ref = _oracle_chain(cfg)
    e_h = rel_l2(h.cpu().numpy(), h_ref)
    e_l = rel_l2(logits.cpu().numpy(), lg_ref)
    print("  rel-L2 h %.2e logits %.2e" % (e_h, e_l), flush=True)
    assert e_h <= 1e-4 and e_l <= 1e-4


def test_decode_step_graph_replays_match_eager():
    """The step captured in a HIP graph: every replay gives the eager result."""
    from memory_bound_quantized_amd.decode import DecodeModel
    cfg = workloads.config3(layers=2, vocab=512)
    model = DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])
    h0 = dev(cfg["h0"])
    h = h0.clone()
    lg = torch.empty(512, device="cuda")
    model.step(h, lg)
    torch.cuda.synchronize()
    h_e, lg_e = h.clone(), lg.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.copy_(h0)
        model.step(h, lg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        model.step(h, lg)
    for _ in range(3):
        h.copy_(h0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_e) and torch.equal(lg, lg_e)


# --------------------------------------------------------------------------
# the one-launch step (mbq_decode_step_persistent)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("layers,vocab", [(2, 1000), (3, 4096)])
def test_persistent_step_matches_oracle_chain(layers, vocab):
    from memory_bound_quantized_amd.decode import DecodeModel
    print("persistent layers=%d vocab=%d" % (layers, vocab), flush=True)
    cfg = workloads.config3(layers=layers, vocab=vocab)
    model = DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])
    h = dev(cfg["h0"])
    logits = torch.empty(vocab, device="cuda")
    model.step_persistent(h, logits)
    torch.cuda.synchronize()
    assert model.status() == 0
    h_ref, lg_ref = _oracle_chain(cfg)
    e_h = rel_l2(h.cpu().numpy(), h_ref)
    e_l = rel_l2(logits.cpu().numpy(), lg_ref)
    print("  rel-L2 h %.2e logits %.2e" % (e_h, e_l), flush=True)
    assert e_h <= 1e-4 and e_l <= 1e-4
    # the launch-per-step path on the same model agrees within the same bar
    h2 = dev(cfg["h0"])
    lg2 = torch.empty(vocab, device="cuda")
    model.step(h2, lg2)
    assert rel_l2(lg2.cpu().numpy(), logits.cpu().numpy()) <= 1e-4


@pytest.mark.parametrize("layers,vocab,head", [(1, 1001, "q65"), (0, 777, "q65"), (2, 2048, "q45")])
def test_persistent_step_edge_shapes(layers, vocab, head):
    """An odd vocabulary (rows split unevenly over the workgroups, the last
    ones short), no layers at all (the vocabulary product alone, h
    untouched), and a Q45 vocabulary head after Q65 and Q45 down products:
    each against the oracle chain and the launch chain."""
    from memory_bound_quantized_amd.decode import DecodeModel
    print("persistent edge layers=%d vocab=%d head=%s" % (layers, vocab, head), flush=True)
    cfg = workloads.config3(layers=layers, vocab=vocab)
    if head == "q45":
        rng = np.random.default_rng(4545)
        V = (workloads.Q45, vocab, 4096, workloads.weight_planes(rng, workloads.Q45, vocab, 4096))
        cfg["vocab"] = V
    model = DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])
    h = dev(cfg["h0"])
    logits = torch.empty(vocab, device="cuda")
    model.step_persistent(h, logits)
    torch.cuda.synchronize()
    assert model.status() == 0
    h_ref, lg_ref = _oracle_chain(cfg)
    e_h = rel_l2(h.cpu().numpy(), h_ref)
    e_l = rel_l2(logits.cpu().numpy(), lg_ref)
    print("  rel-L2 h %.2e logits %.2e" % (e_h, e_l), flush=True)
    assert e_h <= 1e-4 and e_l <= 1e-4
    if layers == 0:
        assert np.array_equal(h.cpu().numpy(), cfg["h0"])
    h2 = dev(cfg["h0"])
    lg2 = torch.empty(vocab, device="cuda")
    model.step(h2, lg2)
    torch.cuda.synchronize()
    assert rel_l2(lg2.cpu().numpy(), logits.cpu().numpy()) <= 1e-4


def test_persistent_step_repeated_tokens_and_table_guard():
    """Several tokens in a row reuse the prepared table; a workspace prepared
    for another model is refused on the device (status bit 1, h untouched)."""
    from memory_bound_quantized_amd.decode import DecodeModel
    cfg = workloads.config3(layers=1, vocab=512)
    a = DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])
    h = dev(cfg["h0"])
    lg = torch.empty(512, device="cuda")
    hp, lp = h.clone(), torch.empty(512, device="cuda")
    for _ in range(3):
        a.step_persistent(h, lg)
        a.step(hp, lp)
    torch.cuda.synchronize()
    assert a.status() == 0
    assert rel_l2(h.cpu().numpy(), hp.cpu().numpy()) <= 1e-4
    b = DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])
    b.workspace = a.workspace                      # a's table, b's pointers
    b._prepared = True
    h0 = h.clone()
    b.step_persistent(h, lg)
    torch.cuda.synchronize()
    assert b.status() & 2
    assert torch.equal(h, h0)


def test_workload3_full_size_layers():
    """Workload 3 at its full shapes.  Layers 0 (Q65 down), 1 (Q45 down) and
    35 of the 36-layer stack, each as a one-layer step from h0 (the layer's
    own weights and gammas, every matrix at full size), against the oracle's
    one-layer chain; layer 0 with the full 151936-row vocabulary product, the
    others with its first 512 rows.  (The whole 36-layer chain is one
    single-threaded oracle call of about a minute; the layers cover every
    shape of it.)"""
    from memory_bound_quantized_amd.decode import DecodeModel
    cfg = workloads.config3(only=(0, 1, 35))
    d = 4096
    fmtv, V, K, pv = cfg["vocab"]
    rows = lambda p, n: None if p is None else p.reshape(V, -1)[:n].reshape(-1)
    small_vocab = (fmtv, 512, K, [rows(p, 512) for p in pv])
    for lay, l in zip(cfg["layers"], cfg["layer_ids"]):
        vocab = cfg["vocab"] if l == 0 else small_vocab
        print("workload3 layer %d vocab %d" % (l, vocab[1]), flush=True)
        g1, g2 = cfg["g1"][l * d:(l + 1) * d], cfg["g2"][l * d:(l + 1) * d]
        model = DecodeModel([lay], vocab, g1, g2, cfg["gf"], cfg["eps"])
        h = dev(cfg["h0"])
        logits = torch.empty(vocab[1], device="cuda")
        model.step(h, logits)
        torch.cuda.synchronize()
        lay_o = {k: oracle.Planes(*v) for k, v in lay.items()}
        h_ref, lg_ref = oracle.decode_token([lay_o], oracle.Planes(*vocab), g1, g2, cfg["gf"],
                                            cfg["eps"], cfg["h0"])
        e_h = rel_l2(h.cpu().numpy(), h_ref)
        e_l = rel_l2(logits.cpu().numpy(), lg_ref)
        print("  rel-L2 h %.2e logits %.2e" % (e_h, e_l), flush=True)
        assert e_h <= 1e-4 and e_l <= 1e-4
        del model


def test_workload3_whole_token_both_forms():
    """Workload 3 whole: one token through all 36 full-size layers and the
    151936-row vocabulary product, as the launch chain (captured in a graph,
    as the benchmark runs it) and as the one-launch step, against the
    oracle's chain (decode_token_parallel: decode_token's result, each
    product's rows split over threads).  Error builds up over 36 layers; the
    bar is still rel-L2 <= 1e-4 on h and on the logits."""
    import os
    from memory_bound_quantized_amd.decode import DecodeModel
    print("workload3 whole token: generating 4.65 GB of weights", flush=True)
    cfg = workloads.config3()
    model = DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])
    h = dev(cfg["h0"])
    logits = torch.empty(model.vocab, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        model.step(h, logits)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    h.copy_(dev(cfg["h0"]))
    with torch.cuda.graph(g):
        model.step(h, logits)
    h.copy_(dev(cfg["h0"]))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    hp = dev(cfg["h0"])
    lp = torch.empty(model.vocab, device="cuda")
    model.step_persistent(hp, lp)
    torch.cuda.synchronize()
    assert model.status() == 0
    print("workload3 whole token: oracle chain on %d threads" % min(16, os.cpu_count() or 1), flush=True)
    lay = [{k: oracle.Planes(*v) for k, v in e.items()} for e in cfg["layers"]]
    h_ref, lg_ref = oracle.decode_token_parallel(lay, oracle.Planes(*cfg["vocab"]), cfg["g1"], cfg["g2"],
                                                 cfg["gf"], cfg["eps"], cfg["h0"],
                                                 threads=min(16, os.cpu_count() or 1))
    for name, hh, ll in (("graph of launches", h, logits), ("one launch", hp, lp)):
        e_h = rel_l2(hh.cpu().numpy(), h_ref)
        e_l = rel_l2(ll.cpu().numpy(), lg_ref)
        print("  %s: rel-L2 h %.2e logits %.2e" % (name, e_h, e_l), flush=True)
        assert e_h <= 1e-4 and e_l <= 1e-4, name
