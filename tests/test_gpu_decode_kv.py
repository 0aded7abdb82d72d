"""GPU parity of the decode step with attention over KV caches
(mbq_decode_step_kv) against the oracle's token (oracle.decode_token_kv),
through the C ABI.

Bars: final h and logits within rel-L2 1e-4 of the oracle (as for the step
without a cache); the caches bit for bit outside row T.  Row T holds fp16 of
each layer's k and v products, which the device computes in fp32 with a
different summation order from the oracle's, so a value within ~1e-6 of a
binary16 rounding boundary may round the other way: row T is held to one
binary16 ulp plus the products' fp32 error (1e-5 of the row's largest
value) of the oracle's row, and the last layer's row, whose fp32 k and v
are still in the workspace, to numpy's conversion of them bit for bit.

Cases: two full-width layers (32 query heads on 8 key/value heads of 128)
at T = 0 (the new position alone), 37 and 600 (ragged chunks); rows wider
than the heads; one layer at 8, 2 and 1 query heads per key/value head; three tokens in a row growing the same caches; the step
captured in a HIP graph; and the whole 36-layer model at 512 cached
positions, the configuration the benchmark times.
"""
import os

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from checks import rel_l2  # noqa: E402

DKV = 1024


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_quantized_amd  # noqa: F401


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def model_of(cfg):
    from memory_bound_quantized_amd.decode import DecodeModel
    return DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])


def host_caches(L, cap, width, seed):
    rng = np.random.default_rng(seed)
    return ([rng.normal(size=(cap, width)).astype(np.float16) for _ in range(L)],
            [rng.normal(size=(cap, width)).astype(np.float16) for _ in range(L)])


def to_dev(cs):
    return [torch.from_numpy(c.view(np.int16)).cuda() for c in cs]


def to_host(cs):
    return [c.cpu().numpy().view(np.float16) for c in cs]


def oracle_token(cfg, kcs, vcs, T, h0=None):
    lay = [{k: oracle.Planes(*v) for k, v in e.items()} for e in cfg["layers"]]
    return oracle.decode_token_kv(lay, oracle.Planes(*cfg["vocab"]), cfg["g1"], cfg["g2"], cfg["gf"],
                                  cfg["eps"], cfg["h0"] if h0 is None else h0, kcs, vcs, T,
                                  threads=min(16, os.cpu_count() or 1))


def close_after_rounding(a, b):
    """Elementwise bar on two binary16 rows rounded from fp32 values that
    differ by the products' fp32 error: one binary16 ulp (each side rounds
    by at most half of one) plus 1e-5 of the row's largest magnitude (the
    fp32 difference, ~1e-6 of the row scale at the measured rel-L2)."""
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    big = np.maximum(np.abs(a64), np.abs(b64))
    ulp = np.spacing(big.astype(np.float16)).astype(np.float64)
    return np.abs(a64 - b64) <= ulp + 1e-5 * np.abs(b64).max()


def check_caches(got_k, got_v, ref_k, ref_v, before_k, before_v, T):
    for l in range(len(got_k)):
        keep = np.ones(got_k[l].shape[0], bool)
        keep[T] = False
        for got, ref, before in ((got_k[l], ref_k[l], before_k[l]), (got_v[l], ref_v[l], before_v[l])):
            assert np.array_equal(got[keep].view(np.uint16), before[keep].view(np.uint16)), l
            assert np.array_equal(got[T, DKV:].view(np.uint16), before[T, DKV:].view(np.uint16)), l
            close = close_after_rounding(got[T, :DKV], ref[T, :DKV])
            assert close.all(), (l, np.flatnonzero(~close)[:4])


def last_layer_row_is_fp16_of_its_products(model, kd, vd, T):
    """The launch chain leaves the last layer's q|k|v in the workspace's first
    slot: row T must be numpy's binary16 conversion of its k and v."""
    ws = model._kv_ws.cpu().numpy()
    qkv = ws[:4 * (model.dq + 2 * DKV)].view(np.float32)
    k, v = qkv[model.dq:model.dq + DKV], qkv[model.dq + DKV:model.dq + 2 * DKV]
    kr = kd.cpu().numpy().view(np.float16)[T, :DKV]
    vr = vd.cpu().numpy().view(np.float16)[T, :DKV]
    assert np.array_equal(kr.view(np.uint16), k.astype(np.float16).view(np.uint16))
    assert np.array_equal(vr.view(np.uint16), v.astype(np.float16).view(np.uint16))


def run_step(model, cfg, kd, vd, T, h0=None):
    h = dev(cfg["h0"] if h0 is None else h0)
    logits = torch.empty(model.vocab, device="cuda")
    model._kv_ws = model.kv_workspace(T)
    model.step_kv(h, logits, kd, vd, T, workspace=model._kv_ws)
    torch.cuda.synchronize()
    return h.cpu().numpy(), logits.cpu().numpy()


@pytest.mark.parametrize("T,pad", [(0, 0), (37, 64), (600, 0)])
def test_step_kv_matches_oracle(T, pad):
    print("decode kv layers=2 T=%d pad=%d" % (T, pad), flush=True)
    cfg = workloads.config3(layers=2, vocab=1000)
    model = model_of(cfg)
    kh, vh = host_caches(2, T + 2, DKV + pad, 9000 + T)
    kb, vb = [c.copy() for c in kh], [c.copy() for c in vh]
    kd, vd = to_dev(kh), to_dev(vh)
    h, logits = run_step(model, cfg, kd, vd, T)
    h_ref, lg_ref = oracle_token(cfg, kh, vh, T)
    e_h, e_l = rel_l2(h, h_ref), rel_l2(logits, lg_ref)
    print("  rel-L2 h %.2e logits %.2e" % (e_h, e_l), flush=True)
    assert e_h <= 1e-4 and e_l <= 1e-4
    check_caches(to_host(kd), to_host(vd), kh, vh, kb, vb, T)
    last_layer_row_is_fp16_of_its_products(model, kd[-1], vd[-1], T)


@pytest.mark.parametrize("dq,dkv,T", [(4096, 512, 40), (2048, 1024, 300), (4096, 4096, 9)])
def test_step_kv_other_head_groups(dq, dkv, T):
    """Query heads per key/value head other than the model's 4: 8 (32 on 4),
    2 (16 on 8) and 1 (32 on 32), one layer each, caches as wide as dkv."""
    print("decode kv dq=%d dkv=%d T=%d" % (dq, dkv, T), flush=True)
    cfg = workloads.config3(layers=1, dq=dq, dkv=dkv, vocab=512)
    model = model_of(cfg)
    kh, vh = host_caches(1, T + 1, dkv, 9400 + dkv)
    kb, vb = [c.copy() for c in kh], [c.copy() for c in vh]
    kd, vd = to_dev(kh), to_dev(vh)
    h, logits = run_step(model, cfg, kd, vd, T)
    h_ref, lg_ref = oracle_token(cfg, kh, vh, T)
    e_h, e_l = rel_l2(h, h_ref), rel_l2(logits, lg_ref)
    print("  rel-L2 h %.2e logits %.2e" % (e_h, e_l), flush=True)
    assert e_h <= 1e-4 and e_l <= 1e-4
    got_k, got_v = to_host(kd), to_host(vd)
    for got, ref, before in ((got_k[0], kh[0], kb[0]), (got_v[0], vh[0], vb[0])):
        assert np.array_equal(got[:T].view(np.uint16), before[:T].view(np.uint16))
        assert close_after_rounding(got[T], ref[T]).all()


def test_three_tokens_grow_the_caches():
    """Tokens at T = 5, 6, 7 on the same caches (each token's input a new
    vector): the device's caches after each token feed the next, and the
    oracle runs the same sequence on its own copies."""
    print("decode kv three tokens", flush=True)
    cfg = workloads.config3(layers=2, vocab=512)
    model = model_of(cfg)
    kh, vh = host_caches(2, 9, DKV, 9100)
    kd, vd = to_dev(kh), to_dev(vh)
    rng = np.random.default_rng(9101)
    for T in (5, 6, 7):
        h0 = rng.normal(size=4096).astype(np.float32)
        h, logits = run_step(model, cfg, kd, vd, T, h0=h0)
        h_ref, lg_ref = oracle_token(cfg, kh, vh, T, h0=h0)
        e_h, e_l = rel_l2(h, h_ref), rel_l2(logits, lg_ref)
        print("  T=%d rel-L2 h %.2e logits %.2e" % (T, e_h, e_l), flush=True)
        assert e_h <= 1e-4 and e_l <= 1e-4
    got_k, got_v = to_host(kd), to_host(vd)
    for l in range(2):
        for got, ref in ((got_k[l], kh[l]), (got_v[l], vh[l])):
            assert np.array_equal(got[:5].view(np.uint16), ref[:5].view(np.uint16))
            for t in (5, 6, 7):
                assert close_after_rounding(got[t], ref[t]).all(), t
            assert np.array_equal(got[8].view(np.uint16), ref[8].view(np.uint16))


def test_step_kv_graph_replays_match_eager():
    """The step at fixed T captured in a HIP graph: each replay (h reset,
    row T and the workspace scribbled over between replays) gives the eager
    h, logits and caches bit for bit."""
    print("decode kv graph replays", flush=True)
    cfg = workloads.config3(layers=2, vocab=512)
    model = model_of(cfg)
    T = 100
    kh, vh = host_caches(2, T + 1, DKV, 9200)
    kd, vd = to_dev(kh), to_dev(vh)
    ws = model.kv_workspace(T)
    h0 = dev(cfg["h0"])
    h = h0.clone()
    lg = torch.empty(512, device="cuda")
    model.step_kv(h, lg, kd, vd, T, workspace=ws)
    torch.cuda.synchronize()
    h_e, lg_e = h.clone(), lg.clone()
    k_e, v_e = [c.clone() for c in kd], [c.clone() for c in vd]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.copy_(h0)
        model.step_kv(h, lg, kd, vd, T, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        model.step_kv(h, lg, kd, vd, T, workspace=ws)
    for i in range(3):
        h.copy_(h0)
        ws.fill_(0xFF)
        for c in kd + vd:
            c[T, :DKV].fill_(0)
        model.step(h0.clone(), torch.empty(512, device="cuda"))     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_e) and torch.equal(lg, lg_e), i
        assert all(torch.equal(a, b) for a, b in zip(kd + vd, k_e + v_e)), i


def test_workload3_whole_token_with_attention():
    """Workload 3 whole, with attention over 512 cached positions in every
    layer (the benchmark's configuration): one token through all 36
    full-size layers and the 151936-row vocabulary product, captured in a
    graph as the benchmark runs it, against the oracle's token."""
    print("workload3 kv T=512: generating 4.65 GB of weights", flush=True)
    cfg = workloads.config3()
    model = model_of(cfg)
    T = 512
    L = len(cfg["layers"])
    kh, vh = workloads.kv_caches(L, T + 1, DKV, seed=9300)
    kb, vb = [c.copy() for c in kh], [c.copy() for c in vh]
    kd, vd = to_dev(kh), to_dev(vh)
    ws = model.kv_workspace(T)
    h = dev(cfg["h0"])
    logits = torch.empty(model.vocab, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        model.step_kv(h, logits, kd, vd, T, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        model.step_kv(h, logits, kd, vd, T, workspace=ws)
    h.copy_(dev(cfg["h0"]))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    print("workload3 kv T=512: oracle token", flush=True)
    h_ref, lg_ref = oracle_token(cfg, kh, vh, T)
    e_h, e_l = rel_l2(h.cpu().numpy(), h_ref), rel_l2(logits.cpu().numpy(), lg_ref)
    print("  rel-L2 h %.2e logits %.2e" % (e_h, e_l), flush=True)
    assert e_h <= 1e-4 and e_l <= 1e-4
    check_caches(to_host(kd), to_host(vd), kh, vh, kb, vb, T)
