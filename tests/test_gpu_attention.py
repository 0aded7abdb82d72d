"""GPU decode attention (mbq_attention_decode) against the oracle's fp64
attention over the same fp16 cache.

Bar (derived from the arithmetic, fp32 throughout): a score s_t = q.k_t/sqrt(d)
is a 128-term fp32 dot product of exact products, off by at most
e_t = 130 * 2^-24 * sum_d |q_d k_td| / sqrt(d); a weight exp(s_t - max) then
carries a relative error of at most about 2 max_t e_t plus a few ulp of the
exponential, and so does the normalised output.  Per element:
|out - ref| <= (2 max_t e_t + 2^-18) * max_t |v_t| + 2^-20 |ref|, and the
relative L2 error over each head's output at most 1e-5 + 2 max_t e_t (the
score error scales with |q| |k|: scores of several hundred carry errors of
a few 1e-4).

Cases: the 36-layer model's shape (32 query heads on 8 key/value heads of
128) at 512 positions, one position, ragged counts across chunk edges, long
contexts split into many chunks, every group size the kernels take, a row
stride wider than the heads, scores of several hundred (the max shift),
equal keys (uniform weights), and one workspace full of NaN serving calls
of every length in turn (its contents need no initialisation).
"""
import os

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


D = 128


def run(q, kc, vc, H, Hkv, T=None):
    qd = torch.from_numpy(q).cuda()
    kd = torch.from_numpy(kc.view(np.int16)).cuda()
    vd = torch.from_numpy(vc.view(np.int16)).cuda()
    return mbq().attention_decode(qd, kd, vd, H, Hkv, T=T).cpu().numpy()


def check(out, q, kc, vc, H, Hkv, T):
    ref = oracle.attention_decode(q, kc[:T], vc[:T], H, Hkv, D).astype(np.float64)
    G = H // Hkv
    k = kc[:T].astype(np.float64).reshape(T, Hkv, D)
    v = vc[:T].astype(np.float64).reshape(T, Hkv, D)
    qq = q.astype(np.float64).reshape(H, D)
    for h in range(H):
        g = h // G
        e = 130 * 2.0 ** -24 * (np.abs(k[:, g, :]) @ np.abs(qq[h])).max() / np.sqrt(D)
        vmax = np.abs(v[:, g, :]).max()
        o, r = out[h * D:(h + 1) * D].astype(np.float64), ref[h * D:(h + 1) * D]
        bound = (2 * e + 2.0 ** -18) * vmax + 2.0 ** -20 * np.abs(r)
        worst = (np.abs(o - r) / bound).max()
        assert worst <= 1.0, "head %d: element outside the bound (ratio %.3g)" % (h, worst)
        nr = np.linalg.norm(r)
        if nr > 0:
            assert np.linalg.norm(o - r) <= (1e-5 + 2 * e) * nr, h


def cache(rng, T, width, scale=1.0):
    return ((rng.normal(size=(T, width)) * scale).astype(np.float16),
            rng.normal(size=(T, width)).astype(np.float16))


@pytest.mark.parametrize("T", [1, 5, 16, 17, 100, 512, 1000, 4097])
def test_model_shape_matches_oracle(T):
    print("attention H=32 Hkv=8 T=%d" % T, flush=True)
    rng = np.random.default_rng(T)
    H, Hkv = 32, 8
    kc, vc = cache(rng, T, Hkv * D)
    q = rng.normal(size=H * D).astype(np.float32)
    check(run(q, kc, vc, H, Hkv), q, kc, vc, H, Hkv, T)


@pytest.mark.parametrize("H,Hkv", [(8, 8), (16, 8), (32, 4), (64, 8)])
def test_every_group_size(H, Hkv):
    print("attention H=%d Hkv=%d" % (H, Hkv), flush=True)
    rng = np.random.default_rng(H * 100 + Hkv)
    T = 300
    kc, vc = cache(rng, T, Hkv * D)
    q = rng.normal(size=H * D).astype(np.float32)
    check(run(q, kc, vc, H, Hkv), q, kc, vc, H, Hkv, T)


def test_long_context_many_chunks():
    print("attention long T=40000", flush=True)
    rng = np.random.default_rng(7)
    H, Hkv, T = 32, 8, 40000
    kc, vc = cache(rng, T, Hkv * D)
    q = rng.normal(size=H * D).astype(np.float32)
    check(run(q, kc, vc, H, Hkv), q, kc, vc, H, Hkv, T)


def test_capacity_and_row_stride():
    """A cache with room for more positions than T, rows wider than the heads."""
    print("attention stride", flush=True)
    rng = np.random.default_rng(8)
    H, Hkv, T, cap, width = 32, 8, 333, 512, 8 * D + 64
    kc, vc = cache(rng, cap, width)
    q = rng.normal(size=H * D).astype(np.float32)
    out = run(q, kc, vc, H, Hkv, T=T)
    check(out, q, np.ascontiguousarray(kc[:, :Hkv * D]), np.ascontiguousarray(vc[:, :Hkv * D]), H, Hkv, T)


def test_large_scores_take_the_max_shift():
    """Scores in the hundreds: without the shift exp would overflow."""
    print("attention large scores", flush=True)
    rng = np.random.default_rng(9)
    H, Hkv, T = 32, 8, 200
    kc, vc = cache(rng, T, Hkv * D, scale=8.0)
    q = (rng.normal(size=H * D) * 8).astype(np.float32)
    out = run(q, kc, vc, H, Hkv)
    assert np.all(np.isfinite(out))
    check(out, q, kc, vc, H, Hkv, T)


def test_equal_keys_average_the_values():
    print("attention equal keys", flush=True)
    rng = np.random.default_rng(10)
    H, Hkv, T = 8, 2, 77
    kc = np.tile(rng.normal(size=(1, Hkv * D)).astype(np.float16), (T, 1))
    vc = rng.normal(size=(T, Hkv * D)).astype(np.float16)
    q = rng.normal(size=H * D).astype(np.float32)
    out = run(q, kc, vc, H, Hkv).reshape(H, D)
    mean = vc.astype(np.float64).mean(axis=0).reshape(Hkv, D)
    for h in range(H):
        assert np.max(np.abs(out[h] - mean[h // 4])) <= 2.0 ** -18 * np.abs(vc).max()


def test_workspace_needs_no_initialisation():
    """The workspace is scratch: one sized for the longest call, filled with
    NaN and then used by calls of other lengths in turn, gives the oracle's
    result every time."""
    print("attention NaN workspace", flush=True)
    rng = np.random.default_rng(11)
    H, Hkv, Tmax = 32, 8, 5000
    kc, vc = cache(rng, Tmax, Hkv * D)
    q = rng.normal(size=H * D).astype(np.float32)
    qd = torch.from_numpy(q).cuda()
    kd = torch.from_numpy(kc.view(np.int16)).cuda()
    vd = torch.from_numpy(vc.view(np.int16)).cuda()
    nb = mbq().attention_workspace_bytes(Tmax, H, Hkv)
    ws = torch.full(((nb + 15) // 16 * 4,), float("nan"), dtype=torch.float32, device="cuda")
    for T in (5000, 17, 600, 1, 4096, 5000):
        out = mbq().attention_decode(qd, kd, vd, H, Hkv, T=T, workspace=ws)
        check(out.cpu().numpy(), q, kc, vc, H, Hkv, T)


@pytest.mark.parametrize("P", [8, 32, 64])
@pytest.mark.parametrize("T", [777, 1000, 5000])
def test_every_chunking_of_the_positions(P, T):
    """About T / P positions per workgroup (a multiple of 16, at most 256),
    forced through MBQ_ATT_CHUNKS (read because MBQ_TUNING is set in
    conftest.py): ragged last chunks and up to 64 records per head for the
    combine step."""
    print("attention chunks P=%d T=%d" % (P, T), flush=True)
    assert os.environ.get("MBQ_TUNING"), "the override needs MBQ_TUNING"
    rng = np.random.default_rng(100 * P + T)
    H, Hkv = 32, 8
    kc, vc = cache(rng, T, Hkv * D, scale=3.0)
    q = rng.normal(size=H * D).astype(np.float32)
    os.environ["MBQ_ATT_CHUNKS"] = str(P)
    try:
        out = run(q, kc, vc, H, Hkv)
    finally:
        os.environ.pop("MBQ_ATT_CHUNKS", None)
    check(out, q, kc, vc, H, Hkv, T)


def test_attention_in_a_replayed_graph():
    """Both launches captured in a HIP graph and replayed with eager work and
    synchronizations in between; every replay equals the eager result bit for
    bit (the workspace is scratch, rewritten by every call)."""
    print("attention graph replays", flush=True)
    rng = np.random.default_rng(12)
    H, Hkv, T = 32, 8, 512
    kc, vc = cache(rng, T, Hkv * D)
    q = rng.normal(size=H * D).astype(np.float32)
    qd = torch.from_numpy(q).cuda()
    kd = torch.from_numpy(kc.view(np.int16)).cuda()
    vd = torch.from_numpy(vc.view(np.int16)).cuda()
    nb = mbq().attention_workspace_bytes(T, H, Hkv)
    ws = torch.zeros((nb + 15) // 16 * 4, dtype=torch.float32, device="cuda")
    eager = mbq().attention_decode(qd, kd, vd, H, Hkv, workspace=ws).clone()
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mbq().attention_decode(qd, kd, vd, H, Hkv, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mbq().attention_decode(qd, kd, vd, H, Hkv, out=out, workspace=ws)
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(float("nan"))
        mbq().attention_decode(qd, kd, vd, H, Hkv)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
    check(out.cpu().numpy(), q, kc, vc, H, Hkv, T)


# --------------------------------------------------------------------------
# the new position stored, then attended to (mbq_attention_decode_append)
# --------------------------------------------------------------------------

def append_case(T, H=32, Hkv=8, extra_rows=2, pad=64, seed=0):
    rng = np.random.default_rng(1000 + T + seed)
    width = Hkv * D + pad
    kc, vc = cache(rng, T + 1 + extra_rows, width)
    q = rng.normal(size=H * D).astype(np.float32)
    kn = rng.normal(size=Hkv * D).astype(np.float32)
    vn = rng.normal(size=Hkv * D).astype(np.float32)
    return q, kn, vn, kc, vc


def run_append(q, kn, vn, kc, vc, T, H, Hkv, workspace=None):
    kd = torch.from_numpy(kc.view(np.int16)).cuda()
    vd = torch.from_numpy(vc.view(np.int16)).cuda()
    out = mbq().attention_decode_append(dev(q), dev(kn), dev(vn), kd, vd, T, H, Hkv,
                                        workspace=workspace)
    return out.cpu().numpy(), kd.cpu().numpy().view(np.float16), vd.cpu().numpy().view(np.float16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("T", [0, 1, 15, 16, 511, 4095, 5000])
def test_append_stores_the_row_and_matches_oracle(T):
    """Row T takes fp16 of k_new and v_new (numpy's conversion, nearest
    even); every other row and the columns past the heads keep their bits;
    the output is the oracle's attention over rows 0 .. T of the updated
    caches."""
    print("attention append T=%d" % T, flush=True)
    H, Hkv = 32, 8
    q, kn, vn, kc, vc = append_case(T)
    out, k2, v2 = run_append(q, kn, vn, kc, vc, T, H, Hkv)
    keep = np.ones(kc.shape[0], bool)
    keep[T] = False
    assert np.array_equal(k2[keep].view(np.uint16), kc[keep].view(np.uint16))
    assert np.array_equal(v2[keep].view(np.uint16), vc[keep].view(np.uint16))
    assert np.array_equal(k2[T, Hkv * D:].view(np.uint16), kc[T, Hkv * D:].view(np.uint16))
    assert np.array_equal(k2[T, :Hkv * D].view(np.uint16), kn.astype(np.float16).view(np.uint16))
    assert np.array_equal(v2[T, :Hkv * D].view(np.uint16), vn.astype(np.float16).view(np.uint16))
    w = Hkv * D
    check(out, q, np.ascontiguousarray(k2[:, :w]), np.ascontiguousarray(v2[:, :w]), H, Hkv, T + 1)


@pytest.mark.parametrize("T,H,Hkv", [(0, 32, 8), (300, 8, 8), (777, 16, 8), (2000, 64, 8), (40, 32, 4)])
def test_append_equals_attention_over_the_stored_row(T, H, Hkv):
    """The fused call and mbq_attention_decode over the caches it leaves
    (T + 1 positions) read the same values in the same order: equal bits."""
    print("attention append vs plain H=%d Hkv=%d T=%d" % (H, Hkv, T), flush=True)
    q, kn, vn, kc, vc = append_case(T, H, Hkv, seed=1)
    out, k2, v2 = run_append(q, kn, vn, kc, vc, T, H, Hkv)
    kd = torch.from_numpy(k2.view(np.int16)).cuda()
    vd = torch.from_numpy(v2.view(np.int16)).cuda()
    plain = mbq().attention_decode(dev(q), kd, vd, H, Hkv, T=T + 1).cpu().numpy()
    assert np.array_equal(out.view(np.uint32), plain.view(np.uint32))


def test_append_rounds_like_binary16():
    """k_new and v_new values at binary16 ties (both parities), just off
    them, in the subnormal range, at the largest finite half and past it
    (to infinity, as an IEEE conversion does): the stored bits equal
    numpy's float16 conversion.  Only the stored row is compared (infinite
    keys make the scores meaningless)."""
    print("attention append rounding", flush=True)
    H, Hkv, T = 8, 8, 3
    rng = np.random.default_rng(77)
    n = Hkv * D
    one = np.float32(1.0)
    vals = np.concatenate([
        one + np.float32(2.0 ** -11) * np.arange(1, 200, 2, dtype=np.float32),    # ties
        one + np.float32(2.0 ** -11) * np.arange(1, 200, 2, dtype=np.float32) + np.float32(2.0 ** -23),
        np.float32(2.0 ** -24) * rng.uniform(0, 1024, 100).astype(np.float32),     # subnormal halves
        np.array([65504.0, 65519.0, 65520.0, 70000.0, 1e30, 6e-8, 3e-8, 2.9e-8], np.float32),
    ])
    vals = vals * np.where(rng.random(vals.size) < 0.5, -1, 1).astype(np.float32)
    kn = np.resize(vals, n).astype(np.float32)
    vn = np.resize(vals[::-1], n).astype(np.float32)
    q, _, _, kc, vc = append_case(T, H, Hkv, seed=2)
    _, k2, v2 = run_append(q, kn, vn, kc, vc, T, H, Hkv)
    with np.errstate(over="ignore"):                             # past 65520: infinity, as intended
        k16, v16 = kn.astype(np.float16), vn.astype(np.float16)
    assert np.isinf(k16).any()
    assert np.array_equal(k2[T, :n].view(np.uint16), k16.view(np.uint16))
    assert np.array_equal(v2[T, :n].view(np.uint16), v16.view(np.uint16))


def test_append_in_a_replayed_graph():
    """The fused call captured in a HIP graph, replayed with eager work and
    synchronizations in between; each replay stores the same row and gives
    the eager result bit for bit."""
    print("attention append graph replays", flush=True)
    H, Hkv, T = 32, 8, 512
    q, kn, vn, kc, vc = append_case(T, H, Hkv, seed=3)
    qd, knd, vnd = dev(q), dev(kn), dev(vn)
    kd = torch.from_numpy(kc.view(np.int16)).cuda()
    vd = torch.from_numpy(vc.view(np.int16)).cuda()
    ws = torch.zeros((mbq().attention_workspace_bytes(T + 1, H, Hkv) + 15) // 16 * 4,
                     dtype=torch.float32, device="cuda")
    eager = mbq().attention_decode_append(qd, knd, vnd, kd, vd, T, H, Hkv, workspace=ws).clone()
    k_eager = kd.clone()
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mbq().attention_decode_append(qd, knd, vnd, kd, vd, T, H, Hkv, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mbq().attention_decode_append(qd, knd, vnd, kd, vd, T, H, Hkv, out=out, workspace=ws)
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(float("nan"))
        kd[T, :Hkv * D].fill_(0)                                  # the row the call writes
        mbq().attention_decode(qd, kd, vd, H, Hkv, T=T)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        assert torch.equal(kd, k_eager), i
