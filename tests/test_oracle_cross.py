"""The two oracle implementations (plain C loops, numpy with library matrix
products) agree on whole passes of every variant: they share nothing but the
pages' definitions, so an agreement to rounding means neither has a slip that
the other lacks."""
import numpy as np
import pytest

import synth
from oracle import native, reference_numpy

_KEYS = ("x0_0", "x0_1", "xL_0", "xL_1", "f0", "f1", "S", "logP", "u", "v")


def _agree(a, b, keys, rtol=1e-10, atol=1e-10):
    for k in keys:
        if k in a or k in b:
            np.testing.assert_allclose(a[k], b[k], rtol=rtol, atol=atol, err_msg=k)
    for k in ("matches0", "matches1"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    np.testing.assert_allclose(a["scores0"], b["scores0"], rtol=1e-9, atol=1e-14)


@pytest.mark.parametrize("bias_on", [False, True])
@pytest.mark.parametrize("cross,rope", [("standard", False), ("bidirectional", False), ("standard", True)])
def test_sinkhorn_pass(bias_on, cross, rope):
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = synth.make_weights(cfg, bias_on=bias_on, cross=cross, rope=rope)
    pair = synth.make_pair(cfg)
    _agree(native.superglue_match(pair, w, T=cfg.T), reference_numpy.superglue_match(pair, w, T=cfg.T), _KEYS)


def test_sinkhorn_pass_d256_unequal():
    cfg = synth.WORKLOADS["pair2048x1536_f32"]
    w = synth.make_weights(cfg, L=2)
    pair = synth.make_pair(cfg, M=70, N=45)
    _agree(native.superglue_match(pair, w, T=30), reference_numpy.superglue_match(pair, w, T=30), _KEYS)


def test_double_softmax_pass():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = synth.make_weights(cfg, bias_on=True)
    pair = synth.make_pair(cfg)
    _agree(native.double_softmax_match(pair, w), reference_numpy.double_softmax_match(pair, w),
           _KEYS + ("z0", "z1"))


def test_adaptive_pass():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = synth.make_weights(cfg, adaptive=True, bias_on=True, L=3)
    pair = synth.make_pair(cfg, M=40, N=33)
    kw = dict(depth_confidence=0.5, width_confidence=0.5, prune_min=8)
    a, b = native.adaptive_match(pair, w, **kw), reference_numpy.adaptive_match(pair, w, **kw)
    assert a["exit_layer"] == b["exit_layer"]
    np.testing.assert_array_equal(a["prune0"], b["prune0"])
    np.testing.assert_array_equal(a["prune1"], b["prune1"])
    _agree(a, b, ("f0", "f1", "logP"))
