"""GPU parity of adaptive depth and width (sections 2.6 and 2.7 of the
LightGlue review) against the float64 oracle, one pair per call.

Decisions (exit layer, kept points) are compared exactly on constructions
whose confidences and matchabilities sit far from their thresholds; the
exit head's outputs are held to the double-softmax bars (log assignments
1e-3 for fp32 networks, matches equal except near ties).
"""
import copy
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_matches, dev, host, rel_rows

pytestmark = pytest.mark.gpu

sg = pytest.importorskip("learned_sparse_feature_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sg.lib()


def _run(pair, W, cfg, L=None, adaptive=None, **kw):
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")
    img = (*pair["image_size0"], *pair["image_size1"])
    out = sg.sg_match(*[dev(pair[k]) for k in keys], W, cfg.L if L is None else L, cfg.T, image_size=img,
                      want_logP=True, want_desc=True, adaptive=adaptive, **kw)
    torch.cuda.synchronize()
    return {k: host(v) if isinstance(v, torch.Tensor) else v for k, v in out.items()}


def _frozen(cfg, L=3, bias_on=True):
    """GNN updates zero and encoder zero: every layer's states are the descriptors."""
    w = copy.deepcopy(synth.make_weights(cfg, L=L, adaptive=True, bias_on=bias_on))
    for st in w["stages"]:
        st["W2"][:] = 0
        st["b2"][:] = 0
    w["enc"] = [(0 * W_, 0 * b) for W_, b in w["enc"]]
    return w


def _compare(g, r, M, N, logp_tol=1e-3):
    assert g["exit_layer"] == r["exit_layer"]
    np.testing.assert_array_equal(g["prune0"], r["prune0"])
    np.testing.assert_array_equal(g["prune1"], r["prune1"])
    if "kept0" not in r:
        assert (g["matches0"] == -1).all()
        return
    k0, k1 = r["kept0"], r["kept1"]
    lp = g["logP"][np.append(k0, M)][:, np.append(k1, N)]
    dl = np.abs(lp - r["logP"]).max()
    sub0 = np.where(g["matches0"][k0] >= 0, np.searchsorted(k1, np.maximum(g["matches0"][k0], 0)), -1)
    sub1 = np.where(g["matches1"][k1] >= 0, np.searchsorted(k0, np.maximum(g["matches1"][k1], 0)), -1)
    rs0 = np.where(r["matches0"][k0] >= 0, np.searchsorted(k1, np.maximum(r["matches0"][k0], 0)), -1)
    rs1 = np.where(r["matches1"][k1] >= 0, np.searchsorted(k0, np.maximum(r["matches1"][k1], 0)), -1)
    ex = check_matches(sub0, sub1, r["logP"], rs0, rs1)
    pruned0 = np.setdiff1d(np.arange(M), k0)
    assert (g["matches0"][pruned0] == -1).all() and (g["scores0"][pruned0] == 0).all()
    print(f"exit layer {g['exit_layer']}, kept {len(k0)}/{M} and {len(k1)}/{N}, |dlogP| {dl:.2e}, exempt {ex}")
    assert dl < logp_tol


def test_without_adaptive_flags_equals_the_double_softmax_pass():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = synth.make_weights(cfg, adaptive=True, bias_on=True)
    pair = synth.make_pair(cfg)
    a = _run(pair, sg.pack_weights(w, head="ds"), cfg)
    b = _run(pair, sg.pack_weights(dict(w, conf=None, heads=None), head="ds"), cfg)
    for k in ("matches0", "scores0", "logP", "f0"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("wl", ["pair10x12_f32", "pair512_f32"])
def test_never_confident_runs_every_layer_bitwise(wl):
    """Confidence bias -40 (no point ever confident, so none is pruned): the
    adaptive call runs every layer and equals the plain pass bitwise."""
    cfg = synth.WORKLOADS[wl]
    w = copy.deepcopy(synth.make_weights(cfg, adaptive=True, bias_on=True))
    w["conf"] = [(0 * wc, -40.0) for wc, _ in w["conf"]]
    pair = synth.make_pair(cfg)
    W = sg.pack_weights(w, head="ds")
    g = _run(pair, W, cfg, adaptive={"prune_min": 1})
    p = _run(pair, W, cfg)
    assert g["exit_layer"] == cfg.L - 1 and (g["prune0"] == 1).all()
    for k in ("matches0", "scores0", "matches1", "logP", "f0", "f1"):
        assert np.array_equal(g[k], p[k]), k


@pytest.mark.parametrize("wl,exit_at", [("pair10x12_f32", 0), ("pair512_f32", 0), ("pair512_f32", 3)])
def test_forced_exit(wl, exit_at):
    """Confidence bias -40 before layer `exit_at` and +40 from it on: the
    pass stops after that layer and its own head matches."""
    cfg = synth.WORKLOADS[wl]
    w = copy.deepcopy(synth.make_weights(cfg, adaptive=True, rope=(wl == "pair512_f32")))
    w["conf"] = [(0 * wc, 40.0 if l >= exit_at else -40.0) for l, (wc, _) in enumerate(w["conf"])]
    pair = synth.make_pair(cfg)
    r = oracle.adaptive_match(pair, w, prune=False)
    assert r["exit_layer"] == exit_at
    g = _run(pair, sg.pack_weights(w, head="ds"), cfg, adaptive={"prune": False})
    _compare(g, r, cfg.M, cfg.N)
    e = max(rel_rows(g["f0"], r["f0"]).max(), rel_rows(g["f1"], r["f1"]).max())
    assert e < 1e-4


def _crafted(cfg, L=3, ch_conf=(0, 2), ch_match=(1, 1), scale=2000.0):
    """Frozen states; layer l's confidence reads channel ch_conf[l] and its
    matchability channel ch_match[l], both scaled so that every decision is
    far from its threshold (descriptor channels are ~N(0, 1/D))."""
    w = _frozen(cfg, L=L)
    e = np.eye(cfg.D, dtype=np.float32)
    w["conf"] = [(scale * e[c], 0.0) for c in ch_conf[:L - 1]]
    w["heads"] = [(h[0], h[1], scale * e[c], 0.0) for h, c in zip(w["heads"], ch_match)]
    return w


def _margin_ok(pair, chans, scale=2000.0, margin=0.5):
    x = np.concatenate([pair["desc0"], pair["desc1"]]).astype(np.float64)
    return all((np.abs(scale * x[:, c]) > margin).all() for c in chans)


@pytest.mark.parametrize("M,N,prune_min", [(40, 50, 0), (300, 280, 100), (1500, 1300, 1024)])
def test_pruning_and_stop_on_crafted_states(M, N, prune_min):
    cfg = synth.WORKLOADS["pair10x12_f32"] if M < 1000 else synth.WORKLOADS["pair512_f32"]
    w = _crafted(cfg)
    pair = synth.make_pair(cfg, M=M, N=N, seed=M + N)
    r = oracle.adaptive_match(pair, w, depth_confidence=0.97, prune_min=prune_min)
    # (the library reads prune_min 0 as its default; 1 prunes the same images here)
    g = _run(pair, sg.pack_weights(w, head="ds"), cfg, L=3,
             adaptive={"depth_confidence": 0.97, "prune_min": max(prune_min, 1)})
    _compare(g, r, M, N)


def test_stop_ratio_counts_pruned_points_as_confident():
    """The oracle test's construction: layer 1 stops only because the ratio
    divides by the original point count."""
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = _crafted(cfg)
    pair = synth.make_pair(cfg, M=40, N=50)
    x = [pair["desc0"].astype(np.float64), pair["desc1"].astype(np.float64)]
    lam0, lam1 = oracle.confidence_threshold(0, 3), oracle.confidence_threshold(1, 3)
    sig = lambda t: 1 / (1 + np.exp(-t))
    keep = [(sig(2000 * xi[:, 1]) > 0.01) | (sig(2000 * xi[:, 0]) <= lam0) for xi in x]
    u1 = sum(int((sig(2000 * xi[k, 2]) < lam1).sum()) for xi, k in zip(x, keep))
    alpha = 1 - u1 / 90 - 1e-6
    r = oracle.adaptive_match(pair, w, depth_confidence=alpha, prune_min=0)
    assert r["exit_layer"] == 1
    g = _run(pair, sg.pack_weights(w, head="ds"), cfg, L=3, adaptive={"depth_confidence": alpha, "prune_min": 1})
    # prune_min 1 (0 selects the default) prunes the same images here: both have more than one point
    _compare(g, r, 40, 50)


def test_image_emptied_by_pruning():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = _frozen(cfg)
    w["heads"] = [(h[0], h[1], 0.0 * h[2], -50.0) for h in w["heads"]]   # nothing matchable
    w["conf"] = [(0.0 * c[0], 40.0) for c in w["conf"]]                  # everything confident
    pair = synth.make_pair(cfg, M=30, N=26)
    r = oracle.adaptive_match(pair, w, depth_confidence=2.0, prune_min=27)
    g = _run(pair, sg.pack_weights(w, head="ds"), cfg, L=3,
             adaptive={"depth_confidence": 2.0, "prune_min": 27})
    assert r["exit_layer"] == 0 and g["exit_layer"] == 0
    assert (g["matches0"] == -1).all() and (g["matches1"] == -1).all()
    np.testing.assert_array_equal(g["prune0"], r["prune0"])


def test_bf16_network_crafted_decisions():
    """bf16 weights: the decisions and the bookkeeping on crafted frozen
    states; the exit head against the oracle head on the same states."""
    cfg = synth.WORKLOADS["pair1024_bf16"]
    w = _crafted(cfg)
    pair = synth.make_pair(cfg, M=1300, N=1100, seed=5)
    r = oracle.adaptive_match(pair, w, depth_confidence=0.97)
    g = _run(pair, sg.pack_weights(w, head="ds"), cfg, L=3, adaptive={"depth_confidence": 0.97})
    assert g["exit_layer"] == r["exit_layer"]
    np.testing.assert_array_equal(g["prune0"], r["prune0"])
    np.testing.assert_array_equal(g["prune1"], r["prune1"])
    assert (g["matches0"][np.setdiff1d(np.arange(1300), r["kept0"])] == -1).all()
