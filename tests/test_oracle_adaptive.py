"""Pins of the oracle's adaptive depth and width ([LightGlue-review]
sections 2.6 and 2.7).  Most tests make every GNN update zero (W_2 = 0,
b_2 = 0), so the states stay the encoder's and each decision can be
recomputed by hand from them.  Chosen so that a plausible mistake fails:
the stop ratio taken over the remaining instead of the original points,
pruning that ignores the confidence guard or the point-count floor, a
wrong threshold schedule, matches not mapped back to the original indices,
the wrong layer's head at exit.
"""
import copy

import numpy as np
import pytest

import oracle
import synth
from golden_io import confidence_threshold_example


@pytest.fixture(autouse=True)
def _each_oracle(oracle_impl, monkeypatch):
    """Every pin runs against both oracle implementations (plain C, numpy)."""
    monkeypatch.setitem(globals(), "oracle", oracle_impl)



def _frozen(cfg, L=3, seed=None):
    """Adaptive weights whose GNN stages leave the states unchanged and whose
    encoder is zero: every layer's states are the descriptors."""
    w = synth.make_weights(cfg, L=L, adaptive=True, bias_on=True, seed=seed)
    w = copy.deepcopy(w)
    for st in w["stages"]:
        st["W2"][:] = 0
        st["b2"][:] = 0
    w["enc"] = [(0 * W, 0 * b) for W, b in w["enc"]]
    return w


def _sig(t):
    return 1.0 / (1.0 + np.exp(-t))


def test_threshold_schedule_matches_the_page():
    for layer, n_layers, want in confidence_threshold_example():
        assert round(oracle.confidence_threshold(layer, n_layers), 3) == want
    lam = [oracle.confidence_threshold(l, 9) for l in range(9)]
    assert lam[0] == pytest.approx(0.9) and all(a > b for a, b in zip(lam, lam[1:]))


def test_frozen_layers_keep_the_states():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = _frozen(cfg)
    pair = synth.make_pair(cfg)
    d = oracle.superglue_descriptors(pair, w)
    np.testing.assert_array_equal(d["xL_0"], pair["desc0"].astype(np.float64))


def test_no_adaptivity_is_the_full_double_softmax_pass():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = synth.make_weights(cfg, adaptive=True, bias_on=True)
    pair = synth.make_pair(cfg)
    a = oracle.adaptive_match(pair, w, early_exit=False, prune=False)
    r = oracle.double_softmax_match(pair, w)
    assert a["exit_layer"] == cfg.L - 1
    np.testing.assert_array_equal(a["matches0"], r["matches0"])
    np.testing.assert_allclose(a["logP"], r["logP"], rtol=0, atol=1e-12)


def test_forced_exit_uses_the_first_layers_head():
    """Confidence bias +40: every point is confident after layer 0, so the
    pass stops there and layer 0's own head gives the matches."""
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = copy.deepcopy(synth.make_weights(cfg, adaptive=True, bias_on=True))
    w["conf"] = [(0 * wc, 40.0) for wc, _ in w["conf"]]
    pair = synth.make_pair(cfg)
    a = oracle.adaptive_match(pair, w)
    assert a["exit_layer"] == 0
    d = oracle.superglue_descriptors(pair, w, L=1)     # states after stages 0 and 1
    Wf, bf, wz, bz = w["heads"][0]
    r = oracle.double_softmax_from_descriptors(oracle.final_projection(d["xL_0"], Wf, bf),
                                               oracle.final_projection(d["xL_1"], Wf, bf),
                                               d["xL_0"], d["xL_1"], wz, bz)
    np.testing.assert_array_equal(a["matches0"], r["matches0"])
    np.testing.assert_allclose(a["scores0"], r["scores0"], rtol=1e-12)


def test_never_confident_runs_every_layer():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = copy.deepcopy(synth.make_weights(cfg, adaptive=True, bias_on=True))
    w["conf"] = [(0 * wc, -40.0) for wc, _ in w["conf"]]
    pair = synth.make_pair(cfg)
    a = oracle.adaptive_match(pair, w, prune_min=0)
    r = oracle.double_softmax_match(pair, w)
    assert a["exit_layer"] == cfg.L - 1
    np.testing.assert_array_equal(a["matches0"], r["matches0"])   # unconfident points are never pruned


def test_stop_ratio_counts_pruned_points_as_confident():
    """Layer 0 prunes the points confident in channel 0 and unmatchable in
    channel 1; layer 1 judges confidence on channel 2.  The stop ratio of
    layer 1 divides the unconfident count by the original M + N: with the
    threshold placed just under that ratio the pass stops at layer 1 (a
    ratio over the remaining points would be smaller and run on)."""
    cfg = synth.WORKLOADS["pair10x12_f32"]
    L, D = 3, cfg.D
    w = _frozen(cfg, L=L)
    e = np.eye(D)
    w["conf"] = [(2000.0 * e[0], 0.0), (2000.0 * e[2], 0.0)]
    w["heads"] = [(h[0], h[1], 2000.0 * e[1], 0.0) for h in w["heads"]]
    pair = synth.make_pair(cfg, M=40, N=50)
    x = [pair["desc0"].astype(np.float64), pair["desc1"].astype(np.float64)]
    lam0, lam1 = oracle.confidence_threshold(0, L), oracle.confidence_threshold(1, L)
    c0 = [_sig(2000.0 * xi[:, 0]) for xi in x]
    u0 = sum(int((c < lam0).sum()) for c in c0)
    keep = [(_sig(2000.0 * xi[:, 1]) > 0.01) | (c <= lam0) for xi, c in zip(x, c0)]
    u1 = sum(int((_sig(2000.0 * xi[k, 2]) < lam1).sum()) for xi, k in zip(x, keep))
    pruned = sum(int((~k).sum()) for k in keep)
    ratio0, ratio1 = 1 - u0 / 90, 1 - u1 / 90
    alpha = ratio1 - 1e-9
    assert pruned > 0 and u1 > 0 and ratio0 <= alpha
    assert 1 - u1 / (90 - pruned) <= alpha           # the misreading would not stop
    a = oracle.adaptive_match(pair, w, depth_confidence=alpha, width_confidence=0.99, prune_min=0)
    assert a["exit_layer"] == 1
    assert list(a["kept0"]) == list(np.nonzero(keep[0])[0]) and list(a["kept1"]) == list(np.nonzero(keep[1])[0])


def test_pruning_bookkeeping_and_matches_mapped_back():
    """Matchability-only pruning (no early exit) on frozen states: layer 0
    keeps the points with sigmoid(z) > 1 - width_confidence, layer 1 keeps
    all; prune counts are 1 + steps survived; the exit head (the main head at
    the last layer) matches the kept subsets, mapped to original indices."""
    cfg = synth.WORKLOADS["pair10x12_f32"]
    L, D = 3, cfg.D
    w = _frozen(cfg, L=L)
    e = np.eye(D)
    w["heads"][0] = (w["heads"][0][0], w["heads"][0][1], 2000.0 * e[3], 0.0)
    w["heads"][1] = (w["heads"][1][0], w["heads"][1][1], 0.0 * e[3], 50.0)
    pair = synth.make_pair(cfg, M=30, N=26)
    a = oracle.adaptive_match(pair, w, early_exit=False, prune_min=0)
    x = [pair["desc0"].astype(np.float64), pair["desc1"].astype(np.float64)]
    keep = [np.nonzero(_sig(2000.0 * xi[:, 3]) > 0.01)[0] for xi in x]
    assert 0 < len(keep[0]) < 30 and 0 < len(keep[1]) < 26
    assert list(a["kept0"]) == list(keep[0]) and list(a["kept1"]) == list(keep[1])
    want0 = np.ones(30, np.int32)
    want0[keep[0]] = 3
    np.testing.assert_array_equal(a["prune0"], want0)
    assert a["exit_layer"] == L - 1
    f = [oracle.final_projection(xi[k], w["Wf"], w["bf"]) for xi, k in zip(x, keep)]
    r = oracle.double_softmax_from_descriptors(f[0], f[1], x[0][keep[0]], x[1][keep[1]], w["wz"], w["bz"])
    m0 = -np.ones(30, np.int32)
    for i, j in enumerate(r["matches0"]):
        if j >= 0:
            m0[keep[0][i]] = keep[1][j]
    np.testing.assert_array_equal(a["matches0"], m0)
    assert (a["matches0"][np.setdiff1d(np.arange(30), keep[0])] == -1).all()


def test_point_count_floor_and_empty_image():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    L, D = 3, cfg.D
    w = _frozen(cfg, L=L)
    w["heads"] = [(h[0], h[1], 0.0 * h[2], -50.0) for h in w["heads"]]   # nothing is matchable
    w["conf"] = [(0.0 * c[0], 40.0) for c in w["conf"]]                  # everything is confident
    pair = synth.make_pair(cfg, M=30, N=26)
    # depth_confidence 2: never stops; neither image has more than 30 points: no pruning
    a = oracle.adaptive_match(pair, w, depth_confidence=2.0, prune_min=30)
    assert a["exit_layer"] == L - 1 and (a["prune0"] == 1).all() and (a["prune1"] == 1).all()
    # A (30 points) exceeds the floor 27 and loses every point: the pass ends at layer 0
    b = oracle.adaptive_match(pair, w, depth_confidence=2.0, prune_min=27)
    assert b["exit_layer"] == 0 and (b["matches0"] == -1).all() and (b["matches1"] == -1).all()
