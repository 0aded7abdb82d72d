"""Host-side tests of libmbq: it loads, exports every declared symbol, its
packer/unpacker agree bit for bit with the oracle's, and every argument check
returns its documented status before any device work is enqueued.

No GPU is touched: pointer arguments here are fake device addresses that the
library only inspects (alignment, overlap), never dereferences.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads
from memory_bound_quantized_amd import _lib
import memory_bound_quantized_amd as mbq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = _lib.lib


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "mbq.h")) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mbq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared_symbols()
    assert len(declared) == 39
    assert sorted(_lib.EXPORTS) == declared
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert mbq.version() == 1


def test_format_info_and_plane_sizes_match_oracle():
    for fmt, bpw, bk in [(0, 16.0, 1), (1, 4.5, 32), (2, 6.5625, 256), (3, 2.5, 32)]:
        assert mbq.format_info(fmt) == (bpw, bk)
        for N, K in [(0, 256), (1, 256), (7, 512), (12288, 4096), (4096, 12288)]:
            assert mbq.plane_sizes(fmt, N, K) == oracle.plane_bytes(fmt, N, K)


def _random_codes(fmt, N, K, rng):
    if fmt == 0:
        return rng.integers(0, 65536, size=(N, K), dtype=np.uint16), None, None
    bits = {1: 4, 2: 6, 3: 2}[fmt]
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    if fmt == 2:
        sc = rng.integers(-128, 128, size=N * K // 16).astype(np.int8)
        su = np.float16(rng.uniform(0.001, 0.02, N * K // 256)).view(np.uint16)
        return codes, sc, su
    return codes, np.float16(rng.uniform(0.001, 0.02, N * K // 32)).view(np.uint16), None


@pytest.mark.parametrize("fmt,N,K", [(1, 1, 32), (1, 5, 96), (1, 3, 4096), (2, 1, 256),
                                     (2, 3, 512), (2, 2, 12288), (3, 1, 32), (3, 7, 160),
                                     (0, 3, 24)])
def test_host_pack_matches_oracle_pack_bit_for_bit(fmt, N, K):
    rng = np.random.default_rng(fmt * 1000 + N * 10 + K)
    codes, sc, su = _random_codes(fmt, N, K, rng)
    mine = mbq.pack(fmt, N, K, codes, sc, su)
    ref = oracle.pack(fmt, N, K, codes, sc, su)
    for a, b in zip(mine, ref.planes):
        assert (a is None) == (b is None)
        if a is not None:
            assert np.array_equal(a, b)
    c2, s2, u2 = mbq.unpack(fmt, N, K, mine)
    assert np.array_equal(c2, codes)
    if sc is not None:
        assert np.array_equal(s2.view(np.uint8), np.asarray(sc).view(np.uint8))
    if su is not None:
        assert np.array_equal(u2, su)


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_host_unpack_of_random_planes_matches_oracle_codes(fmt):
    rng = np.random.default_rng(40 + fmt)
    N, K = 6, 512
    planes = workloads.weight_planes(rng, fmt, N, K)
    codes, _, _ = mbq.unpack(fmt, N, K, planes)
    assert np.array_equal(codes, oracle.codes(oracle.Planes(fmt, N, K, planes)))


def test_pack_rejects_codes_wider_than_the_format():
    for fmt, bad in [(1, 16), (2, 64), (3, 4)]:
        N, K = 1, 256
        codes = np.zeros((N, K), np.uint8)
        codes[0, 100] = bad
        sc = np.zeros(N * K // (16 if fmt == 2 else 32), np.uint16 if fmt != 2 else np.int8)
        su = np.zeros(N * K // 256, np.uint16) if fmt == 2 else None
        with pytest.raises(mbq.MbqError) as ei:
            mbq.pack(fmt, N, K, codes, sc, su)
        assert ei.value.status == _lib.EINVAL


# --------------------------------------------------------------------------
# argument checks (fake, never-dereferenced device addresses)
# --------------------------------------------------------------------------

BASE = 0x7F0000000000


def _desc(fmt=1, N=64, K=256, off=0):
    return _lib.QWeightDesc(fmt, 0, N, K, BASE + off, BASE + 0x100000 if fmt == 2 else 0,
                            BASE + 0x200000, BASE + 0x300000 if fmt == 2 else 0)


def _gemv(d, x=BASE + 0x400000, M=1, ldx=None, y=BASE + 0x800000, ldy=None, acc=0):
    return L.mbq_gemv_q(ctypes.byref(d) if d is not None else None, x, M,
                        d.K if ldx is None and d is not None else (ldx or 0), y,
                        d.N if ldy is None and d is not None else (ldy or 0), acc, None)


def test_gemv_argument_checks():
    assert _gemv(None) == _lib.EINVAL
    assert _gemv(_desc(fmt=7)) == _lib.EINVAL
    assert _gemv(_desc(K=48)) == _lib.EINVAL                    # K not a block multiple
    assert _gemv(_desc(fmt=2, K=128)) == _lib.EINVAL
    d = _desc()
    d.reserved = 1
    assert _gemv(d) == _lib.EINVAL
    assert _gemv(_desc(), M=-1) == _lib.EINVAL
    assert _gemv(_desc(), ldx=100) == _lib.EINVAL               # ldx < K
    assert _gemv(_desc(), acc=2) == _lib.EINVAL
    assert _gemv(_desc(), M=0) == _lib.OK                       # empty: nothing enqueued
    assert _gemv(_desc(N=0)) == _lib.OK
    assert _gemv(_desc(), x=None) == _lib.EINVAL
    assert _gemv(_desc(), x=BASE + 0x400004) == _lib.EALIGN     # x not 16-B aligned
    assert _gemv(_desc(), y=BASE + 0x800002) == _lib.EALIGN
    assert _gemv(_desc(), y=BASE + 0x400000 + 512) == _lib.EINVAL  # y overlaps x
    assert _gemv(_desc(off=8)) == _lib.EALIGN                   # plane 0 misaligned
    d = _desc()
    d.scales = None
    assert _gemv(d) == _lib.EINVAL
    assert _gemv(_desc(fmt=3, K=96)) == _lib.EUNSUPPORTED       # Q25 kernels need K % 64
    assert _gemv(_desc(fmt=0, K=12)) == _lib.EUNSUPPORTED       # BF16 kernels need K % 8
    assert _gemv(_desc(K=65536)) == _lib.EUNSUPPORTED           # beyond the LDS-staged K
    assert _gemv(_desc(), M=9, ldx=256, ldy=63) == _lib.EINVAL      # ldy < N
    assert L.mbq_last_error()


def test_gather_argument_checks():
    d = _desc(N=6 * 32)
    g = lambda rpe=32, idx=BASE + 0x900000, n=3, x=BASE + 0x400000, y=BASE + 0x800000: \
        L.mbq_gemv_q_gather(ctypes.byref(d), rpe, idx, n, x, y, None)
    assert g(rpe=0) == _lib.EINVAL
    assert g(rpe=40) == _lib.EINVAL                             # N not a multiple
    assert g(n=0) == _lib.OK
    assert g(idx=None) == _lib.EINVAL
    assert g(idx=BASE + 0x900002) == _lib.EALIGN
    assert g(x=BASE + 0x400008) == _lib.EALIGN
    assert g(y=BASE + 0x400000) == _lib.EINVAL                  # overlap


def test_norm_argument_checks():
    x, gm, b, y = BASE, BASE + 0x100000, BASE + 0x200000, BASE + 0x300000
    rms = lambda x=x, g=gm, eps=1e-6, rows=4, n=4096, y=y: L.mbq_rmsnorm(x, g, eps, rows, n, y, None)
    assert rms(rows=-1) == _lib.EINVAL
    assert rms(eps=-1.0) == _lib.EINVAL
    assert rms(eps=float("nan")) == _lib.EINVAL
    assert rms(eps=float("inf")) == _lib.EINVAL
    assert rms(rows=0) == _lib.OK
    assert rms(n=0) == _lib.OK
    assert rms(g=None) == _lib.EINVAL
    assert rms(y=x + 2) == _lib.EALIGN
    assert rms(y=x + 4096) == _lib.EINVAL                      # partial overlap
    ln = lambda beta=b, y=y: L.mbq_layernorm(x, gm, beta, 1e-5, 4, 2048, y, None)
    assert ln(beta=None) == _lib.EINVAL
    assert ln(y=x + 16) == _lib.EINVAL
    assert L.mbq_silu_mul(x, gm, -1, y, None) == _lib.EINVAL
    assert L.mbq_silu_mul(x, gm, 0, y, None) == _lib.OK
    assert L.mbq_silu_mul(x, gm, 1024, x + 64, None) == _lib.EINVAL


def test_staged_x_argument_checks():
    sz = ctypes.c_size_t()
    assert L.mbq_xq_bytes(1, 3, 4096, ctypes.byref(sz)) == _lib.OK and sz.value == 3 * 4096 * 4
    assert L.mbq_xq_bytes(3, 1, 4096, ctypes.byref(sz)) == _lib.OK and sz.value == 4096 * 4
    assert L.mbq_xq_bytes(3, 1, 96, ctypes.byref(sz)) == _lib.EINVAL       # Q25 chunk is 64
    assert L.mbq_xq_bytes(1, 1, 48, ctypes.byref(sz)) == _lib.EINVAL
    assert L.mbq_xq_bytes(9, 1, 64, ctypes.byref(sz)) == _lib.EINVAL
    # Q45 with 4 or more tokens and K % 128 == 0: the matrix-core tile form
    # (2 KB per 16 tokens and 32 values, plus 64 exponent bytes per 16 tokens
    # and 128 values); the row form otherwise
    tile = lambda K: K // 32 * 2048 + K // 128 * 64
    assert L.mbq_xq_bytes(1, 17, 4096, ctypes.byref(sz)) == _lib.OK and sz.value == 2 * tile(4096)
    assert L.mbq_xq_bytes(1, 6, 4096, ctypes.byref(sz)) == _lib.OK and sz.value == tile(4096)
    assert L.mbq_xq_bytes(1, 6, 640, ctypes.byref(sz)) == _lib.OK and sz.value == tile(640)
    assert L.mbq_xq_bytes(1, 512, 4096, ctypes.byref(sz)) == _lib.OK and sz.value == 32 * tile(4096)
    assert L.mbq_xq_bytes(1, 4, 4096, ctypes.byref(sz)) == _lib.OK and sz.value == tile(4096)
    assert L.mbq_xq_bytes(1, 3, 4096, ctypes.byref(sz)) == _lib.OK and sz.value == 3 * 4096 * 4
    assert L.mbq_xq_bytes(1, 8, 2080, ctypes.byref(sz)) == _lib.OK and sz.value == 8 * 2080 * 4
    assert L.mbq_xq_bytes(2, 17, 4096, ctypes.byref(sz)) == _lib.OK and sz.value == 17 * 4096 * 4
    x, xq = BASE, BASE + 0x100000
    st = lambda fmt=1, x=x, M=1, ldx=4096, K=4096, xq=xq: L.mbq_stage_x(fmt, x, M, ldx, K, xq, None)
    assert st(K=4016) == _lib.EINVAL
    assert st(ldx=100) == _lib.EINVAL
    assert st(M=0) == _lib.OK
    assert st(x=None) == _lib.EINVAL
    assert st(x=x + 4) == _lib.EALIGN
    assert st(xq=xq + 8) == _lib.EALIGN
    assert st(xq=x + 4096) == _lib.EINVAL                                   # overlap
    assert st(K=65536, ldx=65536) == _lib.EUNSUPPORTED
    # K % 128 != 0: 16 tokens take the row form (4 bytes per value), not the tile form
    assert L.mbq_xq_bytes(1, 16, 2080, ctypes.byref(sz)) == _lib.OK and sz.value == 16 * 2080 * 4
    gx = lambda d, xq=xq, M=1, y=BASE + 0x800000, acc=0: \
        L.mbq_gemv_xq(ctypes.byref(d), xq, M, y, d.N, acc, None)
    assert gx(_desc(), xq=None) == _lib.EINVAL
    assert gx(_desc(), xq=xq + 4) == _lib.EALIGN
    assert gx(_desc(), y=xq + 64) == _lib.EINVAL                            # overlap
    assert gx(_desc(), acc=3) == _lib.EINVAL
    assert gx(_desc(), M=0) == _lib.OK
    assert gx(_desc(fmt=3, K=96)) == _lib.EUNSUPPORTED
    d = _desc(K=4096)
    d.scales = BASE + 0x200004
    assert gx(d, M=16) == _lib.EALIGN                                       # 8-byte aligned scales
    r = lambda n=4096, y=BASE + 0x200000, fmt=1, xq=xq, x=x, eps=1e-6: \
        L.mbq_rmsnorm_xq(x, BASE + 0x300000, eps, n, y, fmt, xq, None)
    assert r(n=-1) == _lib.EINVAL
    assert r(n=0) == _lib.OK
    assert r(eps=-1.0) == _lib.EINVAL
    assert r(n=4016) == _lib.EINVAL                                         # not a chunk multiple
    assert r(n=16384) == _lib.EUNSUPPORTED
    assert r(xq=None) == _lib.EINVAL
    assert r(y=BASE + 0x200004) == _lib.EALIGN
    assert r(xq=x + 1024) == _lib.EINVAL                                    # xq overlaps x
    assert r(y=x + 64) == _lib.EINVAL                                       # partial overlap
    sm = lambda n=12288, fmt=2, xq=xq, g=BASE + 0x400000: L.mbq_silu_mul_xq(g, BASE + 0x500000, n, fmt, xq, None)
    assert sm(n=0) == _lib.OK
    assert sm(n=100) == _lib.EINVAL
    assert sm(g=BASE + 0x400008) == _lib.EALIGN
    assert sm(xq=BASE + 0x500000) == _lib.EINVAL                            # xq overlaps u


def test_split_product_argument_checks():
    """mbq_gemv_xq_workspace_bytes is host arithmetic: a counter per output
    tile (rounded up to 256 bytes), then S partial tiles of M x N fp32; 0
    where the plan does not split.  mbq_gemv_xq_ws checks its workspace
    before any device call."""
    sz = ctypes.c_size_t()
    wb = lambda N, K, M: (L.mbq_gemv_xq_workspace_bytes(ctypes.byref(_desc(N=N, K=K)), M, ctypes.byref(sz)), sz.value)
    r256 = lambda b: (b + 255) // 256 * 256
    # 4096 x 12288: four parts of 4 row tiles (64 workgroups per part) at any batch
    assert wb(4096, 12288, 16) == (_lib.OK, r256(64 * 4) + 4 * 16 * 4096 * 4)
    assert wb(4096, 12288, 100) == (_lib.OK, r256(64 * 2 * 4) + 4 * 100 * 4096 * 4)
    # 4096 x 4096 and 6144 x 4096: split above 32 tokens only
    assert wb(4096, 4096, 16) == (_lib.OK, 0)
    assert wb(4096, 4096, 64) == (_lib.OK, r256(64 * 4) + 4 * 64 * 4096 * 4)
    assert wb(6144, 4096, 32) == (_lib.OK, 0)
    assert wb(6144, 4096, 33) == (_lib.OK, r256(96 * 4) + 2 * 33 * 6144 * 4)
    # 12288 rows: two parts of 6 row tiles, for K >= 12288 above 32 tokens
    assert wb(12288, 12288, 64) == (_lib.OK, r256(128 * 4) + 2 * 64 * 12288 * 4)
    assert wb(12288, 12288, 16) == (_lib.OK, 0)
    assert wb(12288, 4096, 64) == (_lib.OK, 0)
    assert wb(4096, 12288, 3) == (_lib.OK, 0)          # vector units
    assert wb(1000, 8192, 64) == (_lib.OK, r256(16 * 4) + 4 * 64 * 1000 * 4)
    assert wb(1000, 1024, 64) == (_lib.OK, 0)          # 8 quads: not a step of 4 parts of 4 waves
    assert wb(20000, 12288, 64) == (_lib.OK, 0)        # 5 row tiles per unit
    assert wb(4096, 12000, 16) == (_lib.OK, 0)         # K % 128 != 0: row form
    assert L.mbq_gemv_xq_workspace_bytes(None, 16, ctypes.byref(sz)) == _lib.EINVAL
    assert L.mbq_gemv_xq_workspace_bytes(ctypes.byref(_desc()), -1, ctypes.byref(sz)) == _lib.EINVAL
    d = _desc(N=4096, K=12288)
    need = 256 + 4 * 16 * 4096 * 4
    xq, y, ws = BASE + 0x4000000, BASE + 0x5000000, BASE + 0x6000000
    g = lambda xq=xq, y=y, ws=ws, wsb=need, acc=0, ldy=4096: \
        L.mbq_gemv_xq_ws(ctypes.byref(d), xq, 16, y, ldy, acc, ws, wsb, None)
    assert g(ws=None) == _lib.EINVAL
    assert g(wsb=need - 1) == _lib.EINVAL
    assert g(ws=ws + 16) == _lib.EALIGN
    assert g(ws=y + 256) == _lib.EINVAL                                      # overlaps y
    assert g(ws=xq) == _lib.EINVAL                                           # overlaps xq
    assert g(ws=BASE) == _lib.EINVAL                                         # overlaps the codes
    assert g(acc=2) == _lib.EINVAL
    assert g(ldy=100) == _lib.EINVAL
    assert g(xq=None) == _lib.EINVAL


def test_fused_gemv_argument_checks():
    x, gm, y = BASE + 0x400000, BASE + 0x500000, BASE + 0x800000
    fz = lambda d, x=x, g=gm, eps=1e-6, epi=0, y=y: L.mbq_gemv_fused(ctypes.byref(d), x, g, eps, epi, y, None)
    assert fz(_desc(K=4096), epi=3) == _lib.EINVAL
    assert fz(_desc(N=63, K=4096), epi=2) == _lib.EINVAL                    # silu needs even N
    assert fz(_desc(K=4096), eps=-1.0) == _lib.EINVAL
    assert fz(_desc(N=0, K=4096)) == _lib.OK
    assert fz(_desc(K=4096), x=None) == _lib.EINVAL
    assert fz(_desc(K=4096), g=gm + 4) == _lib.EALIGN
    assert fz(_desc(K=4096), y=x + 64) == _lib.EINVAL                       # y overlaps x
    assert fz(_desc(K=2048)) == _lib.EUNSUPPORTED                           # no fused kernel
    assert fz(_desc(fmt=3, K=4096)) == _lib.EUNSUPPORTED
    assert fz(_desc(fmt=0, K=4096), epi=2) == _lib.EUNSUPPORTED


def _model(L=1, d=4096, dq=4096, dkv=1024, f=12288, vocab=1000, fmt_down=2):
    lay = (_lib.DecodeLayerDesc * L)()
    off = 0

    def w(fmt, N, K):
        nonlocal off
        off += 0x10000000
        return _desc(fmt=fmt, N=N, K=K, off=off)
    for l in range(L):
        lay[l] = _lib.DecodeLayerDesc(w(1, dq + 2 * dkv, d), w(1, d, dq), w(1, 2 * f, d),
                                      w(fmt_down, d, f), BASE + 0x100, BASE + 0x200)
    m = _lib.DecodeModelDesc(L, 1e-6, d, dq, dkv, f, vocab, ctypes.cast(lay, ctypes.POINTER(_lib.DecodeLayerDesc)),
                             BASE + 0x300, w(2, vocab, d))
    m._keep = lay
    return m


def test_decode_argument_checks():
    m = _model()
    nb = ctypes.c_size_t()
    assert L.mbq_decode_workspace_bytes(ctypes.byref(m), ctypes.byref(nb)) == _lib.OK
    # status words, q|k|v and gated activations per layer, two h versions per
    # layer, then the one-launch step's table (header, vocabulary head, layers)
    table = 32 + 48 + 1 * 152
    assert nb.value == 2048 + (4096 + 2048) * 4 + 12288 * 4 + 2 * 4096 * 4 + (table + 255) // 256 * 256
    h, lg, ws = BASE + 0x7000000000, BASE + 0x7100000000, BASE + 0x7200000000
    st = lambda m, h=h, lg=lg, ws=ws, n=nb.value: L.mbq_decode_step(ctypes.byref(m), h, lg, ws, n, None)
    assert st(m, n=nb.value - 1) == _lib.EINVAL                             # workspace too small
    assert st(m, ws=ws + 16) == _lib.EINVAL                                 # 256-byte alignment
    assert st(m, h=h + 4) == _lib.EALIGN
    assert st(m, lg=ws + 64) == _lib.EINVAL                                 # logits overlap workspace
    bad = _model(dkv=512)
    bad.layers[0].qkv.N = 4096 + 2048                                       # not dq + 2 dkv
    assert st(bad) == _lib.EINVAL
    assert st(_model(d=2048, dq=2048)) == _lib.EUNSUPPORTED                 # no fused kernel for d=2048
    e = _model(vocab=0)
    e.eps = float("nan")
    assert st(e) == _lib.EINVAL
    # the one-launch step: same checks, plus its shape limits
    ps = lambda m, h=h, lg=lg, ws=ws, n=nb.value: L.mbq_decode_step_persistent(ctypes.byref(m), h, lg, ws, n, None)
    assert ps(m, n=nb.value - 1) == _lib.EINVAL
    assert ps(_model(dkv=512, f=8192)) in (_lib.EUNSUPPORTED,)               # f must be 12288
    q65o = _model()
    q65o.layers[0].o.fmt = 2
    q65o.layers[0].o.codes_hi = BASE + 0x900000
    q65o.layers[0].o.super_scales = BASE + 0xA00000
    assert ps(q65o) == _lib.EUNSUPPORTED                                    # o must be Q45
    assert L.mbq_decode_prepare(ctypes.byref(m), ws + 16, nb.value, None) == _lib.EINVAL
    assert L.mbq_last_error()


def test_decode_kv_argument_checks():
    m = _model(L=2)
    nb = ctypes.c_size_t()
    # q|k|v, the gated activations, the attention output, then one record per
    # query head and chunk for T + 1 = 512 positions (16 chunks of 32)
    assert L.mbq_decode_kv_workspace_bytes(ctypes.byref(m), 511, ctypes.byref(nb)) == _lib.OK
    assert nb.value == (4096 + 2048) * 4 + 12288 * 4 + 4096 * 4 + 32 * 16 * 132 * 4
    assert L.mbq_decode_kv_workspace_bytes(ctypes.byref(m), -1, ctypes.byref(nb)) == _lib.EINVAL
    assert L.mbq_decode_kv_workspace_bytes(ctypes.byref(_model(dq=4096, dkv=1000)), 5,
                                           ctypes.byref(nb)) == _lib.EUNSUPPORTED   # not whole heads
    assert L.mbq_decode_kv_workspace_bytes(ctypes.byref(_model(dkv=384)), 5,
                                           ctypes.byref(nb)) == _lib.EINVAL          # 32 on 3 heads
    assert L.mbq_decode_kv_workspace_bytes(ctypes.byref(_model(dq=3072)), 5,
                                           ctypes.byref(nb)) == _lib.EUNSUPPORTED   # 24 on 8: G = 3
    assert L.mbq_decode_kv_workspace_bytes(ctypes.byref(m), 511, ctypes.byref(nb)) == _lib.OK
    h, lg, ws = BASE + 0x7000000000, BASE + 0x7100000000, BASE + 0x7200000000
    kc = [BASE + 0x7300000000, BASE + 0x7400000000]
    vc = [BASE + 0x7500000000, BASE + 0x7600000000]

    def st(m=m, h=h, lg=lg, ws=ws, n=nb.value, k=kc, v=vc, T=511, ld=1024):
        ka = (ctypes.c_void_p * 2)(*k)
        va = (ctypes.c_void_p * 2)(*v)
        return L.mbq_decode_step_kv(ctypes.byref(m), h, lg, ka, va, T, ld, ws, n, None)

    assert st(n=nb.value - 1) == _lib.EINVAL                                # workspace too small
    assert st(ws=ws + 16) == _lib.EINVAL                                    # 256-byte alignment
    assert st(h=h + 4) == _lib.EALIGN
    assert st(T=-1) == _lib.EINVAL
    assert st(ld=1000) == _lib.EINVAL                                       # ld < dkv
    assert st(ld=1028) == _lib.EALIGN                                       # ld % 8
    assert st(k=[kc[0], 0]) == _lib.EINVAL                                  # a NULL cache
    assert st(v=[vc[0], vc[1] + 8]) == _lib.EALIGN
    assert st(v=[kc[0] + 1024, vc[1]]) == _lib.EINVAL                       # V inside K's rows
    assert st(k=[ws + 4096, kc[1]]) == _lib.EINVAL                          # K over the workspace
    assert st(k=[kc[0], h - 64]) == _lib.EINVAL                             # K's rows reach h
    assert L.mbq_decode_step_kv(ctypes.byref(m), h, lg, None, None, 511, 1024, ws, nb.value,
                                None) == _lib.EINVAL
    assert L.mbq_last_error()


def _attn_append(q=BASE, kn=BASE + 0x10000, vn=BASE + 0x20000, k=BASE + 0x1000000,
                 v=BASE + 0x2000000, T=511, ld=1024, H=32, Hkv=8, d=128, out=BASE + 0x3000000,
                 ws=BASE + 0x4000000, wsb=1 << 24):
    return L.mbq_attention_decode_append(q, kn, vn, k, v, T, ld, H, Hkv, d, out, ws, wsb, None)


def test_attention_append_argument_checks():
    assert _attn_append(T=-1) == _lib.EINVAL
    assert _attn_append(d=96) == _lib.EUNSUPPORTED
    assert _attn_append(H=24) == _lib.EUNSUPPORTED                          # G = 3
    assert _attn_append(ld=1000) == _lib.EINVAL
    assert _attn_append(ld=1028) == _lib.EALIGN
    assert _attn_append(kn=0) == _lib.EINVAL
    assert _attn_append(vn=BASE + 0x20004) == _lib.EALIGN
    # the workspace covers T + 1 positions: 512 at T = 511 (16 chunks of 32)
    assert _attn_append(wsb=32 * 16 * 132 * 4 - 4) == _lib.EINVAL
    assert _attn_append(kn=BASE + 0x1000000 + 511 * 2048) == _lib.EINVAL    # k_new on the row written
    assert _attn_append(vn=BASE + 0x3000000 + 64) == _lib.EINVAL            # v_new under out
    assert _attn_append(v=BASE + 0x1000000 + 1024) == _lib.EINVAL           # V inside K's rows
    assert _attn_append(ws=BASE + 0x2000000 + 4096) == _lib.EINVAL          # workspace over V
    assert _attn_append(out=BASE) == _lib.EINVAL                            # out over q
    assert L.mbq_last_error()


def test_row_concatenation_and_interleaving_match_the_oracle():
    from memory_bound_quantized_amd.decode import concat_rows, interleave_rows
    rng = np.random.default_rng(4)
    mk = lambda fmt, N, K: (fmt, N, K, workloads.weight_planes(rng, fmt, N, K))
    for fmt, K in ((1, 256), (2, 512), (3, 128), (0, 64)):
        a, b, c = mk(fmt, 5, K), mk(fmt, 3, K), mk(fmt, 5, K)
        wa, wb, wc = (oracle.dequant(oracle.Planes(*m)) for m in (a, b, c))
        cat = oracle.dequant(oracle.Planes(*concat_rows([a, b])))
        assert np.array_equal(cat, np.concatenate([wa, wb]))
        il = oracle.dequant(oracle.Planes(*interleave_rows(a, c)))
        assert np.array_equal(il[0::2], wa) and np.array_equal(il[1::2], wc)


def test_export_and_probe_argument_checks():
    d = _desc(fmt=0, K=64)
    assert L.mbq_unpack_codes(ctypes.byref(d), BASE + 0x900000, None) == _lib.EINVAL  # BF16
    assert L.mbq_dequant_f32(ctypes.byref(_desc()), BASE + 0x900004, None) == _lib.EALIGN
    assert L.mbq_dequant_f32(ctypes.byref(_desc(N=0)), None, None) == _lib.OK
    assert L.mbq_probe_read(BASE, 100, BASE + 0x100000, None) == _lib.EALIGN
    assert L.mbq_probe_copy(BASE, BASE + 64, 128, None) == _lib.EINVAL


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert L.mbq_status_str(s).startswith(b"MBQ_")
    assert L.mbq_status_str(5) == b"unknown status"


def test_one_hip_runtime_in_the_process():
    """libmbq binds to the HIP runtime torch already loaded (same SONAME);
    a second runtime in the process would not see the device torch uses."""
    import re
    with open("/proc/self/maps") as fh:
        libs = set(re.findall(r"\S*libamdhip64\S*", fh.read()))
    assert len(libs) == 1, libs


def _quantize(fmt=1, w=BASE, N=4, K=256, ldw=None, planes=None):
    if planes is None:
        ok = 0 <= fmt <= 3 and N >= 0 and K % (256 if fmt == 2 else 32) == 0
        sz = mbq.plane_sizes(fmt, N, K) if ok else [1, 1, 1, 1]
        planes = [BASE + 0x1000000 * (i + 1) if sz[i] else None for i in range(4)]
    arr = (ctypes.c_void_p * 4)(*planes)
    return L.mbq_quantize(fmt, w, N, K, K if ldw is None else ldw, arr, None)


def test_quantize_argument_checks():
    assert _quantize(fmt=9) == _lib.EINVAL
    assert _quantize(N=-1) == _lib.EINVAL
    assert _quantize(K=48) == _lib.EINVAL                       # not a block multiple
    assert _quantize(fmt=2, K=128) == _lib.EINVAL
    assert _quantize(N=0) == _lib.OK and _quantize(K=0) == _lib.OK   # empty: nothing enqueued
    assert _quantize(ldw=100) == _lib.EINVAL                    # ldw < K
    assert _quantize(w=0) == _lib.EINVAL
    assert _quantize(w=BASE + 4) == _lib.EALIGN
    assert _quantize(ldw=258) == _lib.EALIGN                    # ldw % 4
    assert _quantize(fmt=0, K=12) == _lib.EUNSUPPORTED          # BF16 needs K % 8
    assert _quantize(planes=[BASE + 0x1000000, None, None, None]) == _lib.EINVAL   # Q45 needs scales
    assert _quantize(planes=[BASE + 0x1000008, None, BASE + 0x3000000, None]) == _lib.EALIGN
    assert _quantize(planes=[BASE + 0x1000000, None, BASE + 0x3000002, None]) == _lib.EALIGN
    # a plane inside w's rows
    assert _quantize(planes=[BASE + 0x100, None, BASE + 0x3000000, None]) == _lib.EINVAL
    # planes overlapping each other
    assert _quantize(planes=[BASE + 0x1000000, None, BASE + 0x1000010, None]) == _lib.EINVAL
    assert _quantize(fmt=2, planes=[BASE + 0x1000000, None, BASE + 0x3000000, BASE + 0x4000000]) == _lib.EINVAL


def _attn(q=BASE, k=BASE + 0x1000000, v=BASE + 0x2000000, T=512, ld=1024, H=32, Hkv=8, d=128,
          out=BASE + 0x3000000, ws=BASE + 0x4000000, wsb=1 << 24):
    return L.mbq_attention_decode(q, k, v, T, ld, H, Hkv, d, out, ws, wsb, None)


def test_attention_argument_checks():
    sz = ctypes.c_size_t()
    # one 132-float record per query head and chunk: 512 positions in 16
    # chunks of 32
    assert L.mbq_attention_workspace_bytes(512, 32, 8, 128, ctypes.byref(sz)) == _lib.OK
    assert sz.value == 32 * 16 * 132 * 4
    # 4096 positions: 32 chunks of 128 per head
    assert L.mbq_attention_workspace_bytes(4096, 32, 8, 128, ctypes.byref(sz)) == _lib.OK
    assert sz.value == 32 * 32 * 132 * 4
    # 40000 positions: chunks of 256 (the most a workgroup holds), 157 of them
    assert L.mbq_attention_workspace_bytes(40000, 200, 200, 128, ctypes.byref(sz)) == _lib.OK
    assert sz.value == 200 * 157 * 132 * 4
    assert L.mbq_attention_workspace_bytes(0, 32, 8, 128, ctypes.byref(sz)) == _lib.EINVAL
    assert L.mbq_attention_workspace_bytes(512, 32, 8, 64, ctypes.byref(sz)) == _lib.EUNSUPPORTED
    assert L.mbq_attention_workspace_bytes(512, 24, 8, 128, ctypes.byref(sz)) == _lib.EUNSUPPORTED  # G = 3
    assert L.mbq_attention_workspace_bytes(512, 30, 8, 128, ctypes.byref(sz)) == _lib.EINVAL        # not a multiple
    assert _attn(T=0) == _lib.EINVAL
    assert _attn(d=96) == _lib.EUNSUPPORTED
    assert _attn(ld=1000) == _lib.EINVAL                       # ld < n_kv * d
    assert _attn(ld=1028) == _lib.EALIGN                       # ld % 8
    assert _attn(q=0) == _lib.EINVAL
    assert _attn(q=BASE + 4) == _lib.EALIGN
    assert _attn(wsb=16) == _lib.EINVAL                        # short workspace
    assert _attn(out=BASE + 0x1000000 + 64) == _lib.EINVAL     # out inside the key cache
    assert _attn(ws=BASE) == _lib.EINVAL                       # workspace over q
