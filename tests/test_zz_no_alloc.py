"""mbq_decode_step_noalloc: the decode step with no workspace argument.

It runs the same launches as mbq_decode_step, with q|k|v and the gated
activations in the library's own per-GPU array instead of the caller's
workspace, so its h and logits must equal mbq_decode_step's bit for bit.
Checked on two calls in a row through the C ABI, the second with a smaller
model (fewer layers, narrower k/v and feed-forward, smaller vocabulary), each
against the workspace step from the same h0 and against the oracle chain
(rel-L2 <= 1e-4); then the first model again, after the second has used
the array.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")

from checks import rel_l2  # noqa: E402


@pytest.fixture
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_quantized_amd  # noqa: F401


def _model(cfg):
    from memory_bound_quantized_amd.decode import DecodeModel
    return DecodeModel(cfg["layers"], cfg["vocab"], cfg["g1"], cfg["g2"], cfg["gf"], cfg["eps"])


def _check(cfg, model):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    h_ws, lg_ws = dev(cfg["h0"]), torch.empty(model.vocab, device="cuda")
    model.step(h_ws, lg_ws)
    h_na, lg_na = dev(cfg["h0"]), torch.full((model.vocab,), 7.0, device="cuda")
    model.step_noalloc(h_na, lg_na)
    torch.cuda.synchronize()
    assert torch.equal(h_na, h_ws) and torch.equal(lg_na, lg_ws)
    lay = [{k: oracle.Planes(*v) for k, v in e.items()} for e in cfg["layers"]]
    h_ref, lg_ref = oracle.decode_token_parallel(lay, oracle.Planes(*cfg["vocab"]), cfg["g1"],
                                                 cfg["g2"], cfg["gf"], cfg["eps"], cfg["h0"])
    e_h, e_l = rel_l2(h_na.cpu().numpy(), h_ref), rel_l2(lg_na.cpu().numpy(), lg_ref)
    print("  rel-L2 h %.2e logits %.2e" % (e_h, e_l), flush=True)
    assert e_h <= 1e-4 and e_l <= 1e-4


@pytest.mark.gpu
def test_noalloc_step_equals_workspace_step_on_two_calls(_gpu):
    big = workloads.config3(layers=2, vocab=1000)
    small = workloads.config3(layers=1, dkv=512, f=2048, vocab=300)
    print("no-alloc step: 2 layers, f 12288, vocab 1000", flush=True)
    mb = _model(big)
    _check(big, mb)
    print("no-alloc step: 1 layer, f 2048, vocab 300", flush=True)
    ms = _model(small)
    _check(small, ms)
    print("no-alloc step: the first model again", flush=True)
    _check(big, mb)


def test_noalloc_step_rejects_a_model_beyond_its_array():
    """Activations that do not fit the 1 MiB array: MBQ_EUNSUPPORTED from the
    host checks, before any device call (no GPU needed: the pointers are
    inspected, never dereferenced)."""
    from memory_bound_quantized_amd import _lib
    base = 0x7F0000000000
    desc = _lib.DecodeModelDesc(0, 1e-6, 4096, 0, 0, (1 << 18) + 64, 0, None, base, _lib.QWeightDesc())
    rc = _lib.lib.mbq_decode_step_noalloc(ctypes.byref(desc), base + 0x10000, None, None)
    assert rc == _lib.EUNSUPPORTED, rc
    assert b"limit" in _lib.lib.mbq_last_error()
