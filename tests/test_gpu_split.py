"""The K-split matrix-core product (mbq_gemv_xq_ws) against the oracle.

Every split form is forced on (MBQ_MFMA_SPLIT=2, read because MBQ_TUNING is
set in conftest.py before the library loads); the default plan, which splits
only where it measured faster, is checked on its own.

The split changes only the order in which each output's partial sums are
added (S partial tiles over 1/S of K each, added in split order by the last
workgroup of a tile), so it is held to the oracle's bar, like the unsplit
kernel, and not to the unsplit kernel's bits.  Two calls on the same input
give the same bits (the order of the partial sums does not depend on which
workgroup finishes last), and every call leaves its workspace all zero,
which is what lets one workspace serve calls of any shape.

Cases cover each split the plan takes: 12288 rows (two parts of 6 row
tiles), 5000 rows (two of 4), 4096 and 1000 rows (four of 4); one, two and
four token tiles; ragged token counts and row counts; the two full-size
tables of the 36-layer model; K known only at run time (2048, 6144, 8192);
accumulate, a row stride wider than N; and shapes the plan does not split
(no workspace, the unsplit kernel).
"""
import os

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
    import memory_bound_quantized_amd  # noqa: F401  (fails loudly if libmbq.so is missing)


def mbq():
    import memory_bound_quantized_amd as m
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def weights(N, K, seed):
    planes = workloads.weight_planes(np.random.default_rng(seed), 1, N, K)
    return oracle.Planes(1, N, K, planes), mbq().QWeight.from_host(1, N, K, planes)


def bits(t):
    return t.cpu().numpy().view(np.uint32)


class split:
    """Set MBQ_MFMA_SPLIT for the calls inside the block (2: every split
    form; 1: none)."""
    def __init__(self, v):
        self.v = str(v)

    def __enter__(self):
        assert os.environ.get("MBQ_TUNING"), "the override needs MBQ_TUNING"
        os.environ["MBQ_MFMA_SPLIT"] = self.v

    def __exit__(self, *a):
        os.environ.pop("MBQ_MFMA_SPLIT", None)


SPLIT_CASES = [(16, 12288, 4096), (64, 12288, 4096), (16, 4096, 12288), (64, 4096, 12288),
               (6, 9000, 4096), (20, 12288, 12288), (17, 5000, 4096), (33, 5000, 4096),
               (40, 1000, 4096), (50, 4096, 12288), (7, 1000, 8192), (100, 4100, 4096),
               (16, 9000, 2048), (6, 5000, 6144), (16, 300, 4096)]


@pytest.mark.parametrize("M,N,K", SPLIT_CASES)
def test_split_matches_oracle(M, N, K):
    print("split M=%d N=%d K=%d" % (M, N, K), flush=True)
    ow, dw = weights(N, K, 7700 + N + K)
    X = np.random.default_rng(M + N).normal(size=(M, K)).astype(np.float32)
    Xq = mbq().stage_x(1, dev(X))
    with split(2):
        assert mbq().gemv_xq_workspace_bytes(dw, M) > 0
        ws = mbq().gemv_xq_workspace(dw, M)
        Y = mbq().gemv_xq_ws(dw, Xq, M, ws)
        Y2 = mbq().gemv_xq_ws(dw, Xq, M, ws)
    torch.cuda.synchronize()
    assert not bool(ws.any()), "the call left the workspace nonzero"
    assert np.array_equal(bits(Y), bits(Y2)), "two calls differ"
    check_gemv(Y.cpu().numpy(), ow, X, oracle.gemv(ow, X))


@pytest.mark.parametrize("M,N,K", [(16, 12288, 4096), (33, 4096, 12288), (6, 5000, 4096)])
def test_split_accumulate_and_row_stride(M, N, K):
    print("split accumulate M=%d N=%d K=%d" % (M, N, K), flush=True)
    ow, dw = weights(N, K, 7800 + N)
    rng = np.random.default_rng(N + 3)
    X = rng.normal(size=(M, K)).astype(np.float32)
    ldy = N + 40
    Y0 = rng.normal(size=(M, ldy)).astype(np.float32)
    Xq = mbq().stage_x(1, dev(X))
    out = dev(Y0)
    with split(2):
        ws = mbq().gemv_xq_workspace(dw, M)
        mbq().gemv_xq_ws(dw, Xq, M, ws, out=out[:, :N], accumulate=True)
    got = out.cpu().numpy()
    assert np.array_equal(got[:, N:], Y0[:, N:]), "wrote past N"
    ref = Y0[:, :N].astype(np.float64) + oracle.gemv(ow, X)
    check_gemv(got[:, :N], ow, X, ref, y0=Y0[:, :N])
    assert not bool(ws.any())


def test_one_workspace_serves_every_shape():
    """A workspace sized for the largest call, used by calls of other shapes
    in turn (their counters and partials land at other offsets): each result
    equals the one from a fresh workspace, bit for bit."""
    print("split shared workspace", flush=True)
    shapes = [(64, 12288, 4096), (16, 4096, 12288), (33, 5000, 4096), (16, 12288, 4096)]
    tabs = {}
    big = 0
    with split(2):
        for M, N, K in shapes:
            if (N, K) not in tabs:
                tabs[(N, K)] = weights(N, K, 7900 + N)[1]
            big = max(big, mbq().gemv_xq_workspace_bytes(tabs[(N, K)], M))
        shared = torch.zeros(big, dtype=torch.uint8, device="cuda")
        for i, (M, N, K) in enumerate(shapes):
            dw = tabs[(N, K)]
            Xq = mbq().stage_x(1, dev(np.random.default_rng(i).normal(size=(M, K)).astype(np.float32)))
            a = mbq().gemv_xq_ws(dw, Xq, M, shared)
            b = mbq().gemv_xq_ws(dw, Xq, M, mbq().gemv_xq_workspace(dw, M))
            assert np.array_equal(bits(a), bits(b)), (M, N, K)
    torch.cuda.synchronize()
    assert not bool(shared.any())


@pytest.mark.parametrize("M,N,K,force", [(3, 12288, 4096, 2), (1, 4096, 12288, 2), (16, 77, 1024, 2),
                                         (20, 9000, 2048, 2), (16, 20000, 4096, 2),
                                         (16, 12288, 4096, 0), (64, 12288, 4096, 0), (16, 4096, 4096, 0),
                                         (64, 4096, 12288, 1)])
def test_unsplit_shapes_take_the_unsplit_kernel(M, N, K, force):
    """Where the plan does not split (M below the matrix cores' range, too
    few quads for a whole step of every part, more than 3 row tiles per
    unit, a spilling variant, a shape where the split measured slower, or
    MBQ_MFMA_SPLIT=1), no workspace is needed and the call gives gemv_xq's
    bits."""
    print("split unsplit M=%d N=%d K=%d force=%d" % (M, N, K, force), flush=True)
    _, dw = weights(N, K, 8000 + N)
    X = dev(np.random.default_rng(M * N).normal(size=(M, K)).astype(np.float32))
    Xq = mbq().stage_x(1, X)
    with split(force):
        assert mbq().gemv_xq_workspace_bytes(dw, M) == 0
        ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
        a = mbq().gemv_xq_ws(dw, Xq, M, ws)
        b = mbq().gemv_xq(dw, Xq, M=M)
    assert np.array_equal(bits(a), bits(b))
    assert not bool(ws.any())


@pytest.mark.parametrize("M,N,K", [(16, 4096, 12288), (64, 4096, 4096), (64, 12288, 12288)])
def test_default_plan_splits_where_it_pays(M, N, K):
    """The default plan on shapes it splits: the 36-layer model's down
    table at any batch, the square table and the 12288-row, 12288-wide table
    above 32 tokens."""
    print("split default M=%d N=%d K=%d" % (M, N, K), flush=True)
    ow, dw = weights(N, K, 8200 + N)
    X = np.random.default_rng(M + K).normal(size=(M, K)).astype(np.float32)
    Xq = mbq().stage_x(1, dev(X))
    assert mbq().gemv_xq_workspace_bytes(dw, M) > 0
    ws = mbq().gemv_xq_workspace(dw, M)
    Y = mbq().gemv_xq_ws(dw, Xq, M, ws)
    torch.cuda.synchronize()
    assert not bool(ws.any())
    check_gemv(Y.cpu().numpy(), ow, X, oracle.gemv(ow, X))


def test_small_workspace_is_rejected():
    _, dw = weights(4096, 12288, 8100)
    M = 16
    Xq = mbq().stage_x(1, dev(np.ones((M, 12288), np.float32)))
    need = mbq().gemv_xq_workspace_bytes(dw, M)
    ws = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        mbq().gemv_xq_ws(dw, Xq, M, ws)


def test_split_in_a_replayed_graph():
    """The split product captured in a HIP graph (its counters and partials
    need no clearing node: every call leaves them zero), replayed several
    times with eager work and synchronizations in between; every replay
    equals the eager result bit for bit."""
    print("split graph replays", flush=True)
    M, N, K = 16, 4096, 12288
    _, dw = weights(N, K, 8300)
    rng = np.random.default_rng(8301)
    Xq = mbq().stage_x(1, dev(rng.normal(size=(M, K)).astype(np.float32)))
    ws = mbq().gemv_xq_workspace(dw, M)
    assert ws.numel() > 256
    eager = mbq().gemv_xq_ws(dw, Xq, M, ws)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mbq().gemv_xq_ws(dw, Xq, M, ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mbq().gemv_xq_ws(dw, Xq, M, ws, out=out)
    for i in range(4):
        out.fill_(float("nan"))
        mbq().gemv_xq(dw, Xq, M=M)                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(eager)), i
        assert not bool(ws.any()), i
