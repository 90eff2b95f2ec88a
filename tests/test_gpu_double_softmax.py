"""Parity of the double-softmax matching head (section 2.4 of the LightGlue
review) on the GPU against the float64 oracle.

Tolerances, as for the Sinkhorn head: log assignments within 1e-3 absolute
(max(1e-3, 2e-6 max|logP|) where |logP| reaches hundreds and one fp32 ulp of
the scores is already ~1e-4); matches equal except near ties of the oracle's
log assignment; scores of equal matches within 2e-3 relative.  bf16 networks
are checked on the head from the GPU's own descriptors and states (the
network itself is held to the bf16 descriptor bar elsewhere).
"""
import dataclasses
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


def _head_inputs(M, N, D, seed, scale=3.0, zscale=2.0):
    """Matching descriptors with planted matches, N(0, 1) states and a
    matchability row giving logits of standard deviation about zscale."""
    fA, fB = synth.random_matching_descriptors(M, N, D, seed=seed, scale=scale)
    xA = synth.random_states(M, D, seed + 1)
    xB = synth.random_states(N, D, seed + 2)
    wz = np.ascontiguousarray(synth.random_states(1, D, seed + 3)[0] * (zscale / np.sqrt(D)), np.float32)
    return fA, fB, xA, xB, wz, 0.125


def _tol(ref_logP):
    return max(1e-3, 2e-6 * float(np.abs(ref_logP).max()))


def _bar_S(ref):
    """The real block is 2 S - lse_rows(S) - lse_cols(S) + ..., a difference of
    terms of size max|S|.  S is an fp32 inner product over D terms whose
    magnitudes sum to ~sqrt(D) |S|, so its rounding is ~sqrt(D) 2^-24 |S|
    (~1e-6 |S| at D = 256), and it enters the block four times: where nonzero
    biases grow S into the thousands the bar is 8e-6 max|S| (twice that)."""
    return max(_tol(ref["logP"]), 8e-6 * float(np.abs(ref["S"]).max()))


def _check(out, r, threshold=0.0):
    err = np.abs(host(out["logP"]) - r["logP"]).max()
    ex = check_matches(host(out["matches0"]), host(out["matches1"]), r["logP"], r["matches0"], r["matches1"],
                       threshold=threshold)
    ok = host(out["matches0"]) == r["matches0"]
    np.testing.assert_allclose(host(out["scores0"])[ok], r["scores0"][ok], rtol=2e-3, atol=1e-6)
    ok1 = host(out["matches1"]) == r["matches1"]
    np.testing.assert_allclose(host(out["scores1"])[ok1], r["scores1"][ok1], rtol=2e-3, atol=1e-6)
    return err, ex


@pytest.mark.parametrize("M,N,D", [(64, 64, 256), (3, 700, 256), (700, 3, 64), (257, 1025, 256), (1, 1, 64),
                                   (1, 300, 64), (300, 1, 64), (1024, 1024, 256), (2048, 1536, 256)])
def test_stage_parity(M, N, D):
    fA, fB, xA, xB, wz, bz = _head_inputs(M, N, D, seed=M * 7 + N)
    out = sg.sg_stage_match_ds(dev(fA), dev(fB), dev(xA), dev(xB), dev(wz), bz)
    torch.cuda.synchronize()
    r = oracle.double_softmax_from_descriptors(fA, fB, xA, xB, wz, bz)
    err, ex = _check(out, r)
    print(f"{M}x{N} D={D}: max |dlogP| {err:.2e} (|logP| up to {np.abs(r['logP']).max():.0f}), "
          f"matches {int((r['matches0'] >= 0).sum())}, near-tie exemptions {ex}")
    assert err < _tol(r["logP"])


@pytest.mark.parametrize("M,N", [(0, 5), (6, 0), (0, 0)])
def test_stage_empty(M, N):
    fA, fB, xA, xB, wz, bz = _head_inputs(max(M, 1), max(N, 1), 64, seed=3)
    out = sg.sg_stage_match_ds(dev(fA[:M]), dev(fB[:N]), dev(xA[:M]), dev(xB[:N]), dev(wz), bz)
    torch.cuda.synchronize()
    assert (host(out["matches0"]) == -1).all() and (host(out["scores0"]) == 0).all()
    assert (host(out["matches1"]) == -1).all() and (host(out["scores1"]) == 0).all()


@pytest.mark.parametrize("scale", [6.0, 9.0])
def test_stage_wide_score_range(scale):
    """Scores spanning hundreds of units: the row and column log-sum-exp must
    stay exact where most exponentials underflow."""
    fA, fB, xA, xB, wz, bz = _head_inputs(300, 280, 64, seed=5, scale=scale)
    out = sg.sg_stage_match_ds(dev(fA), dev(fB), dev(xA), dev(xB), dev(wz), bz)
    r = oracle.double_softmax_from_descriptors(fA, fB, xA, xB, wz, bz)
    err, _ = _check(out, r)
    print(f"scale {scale}: max |logP| {np.abs(r['logP']).max():.0f}, max |dlogP| {err:.2e}")
    assert np.abs(r["logP"]).max() > 100
    assert err < _tol(r["logP"])


def test_stage_extreme_matchability():
    """Logits of magnitude ~100: log sigmoid must neither overflow nor lose
    the linear tail (log sigmoid(-z) ~ -z)."""
    fA, fB, xA, xB, wz, bz = _head_inputs(200, 150, 64, seed=9, zscale=40.0)
    out = sg.sg_stage_match_ds(dev(fA), dev(fB), dev(xA), dev(xB), dev(wz), bz)
    r = oracle.double_softmax_from_descriptors(fA, fB, xA, xB, wz, bz)
    assert np.abs(r["z0"]).max() > 60
    err, _ = _check(out, r)
    assert np.isfinite(host(out["logP"])).all()
    assert err < _tol(r["logP"])


def test_stage_threshold():
    fA, fB, xA, xB, wz, bz = _head_inputs(300, 280, 256, seed=3, scale=2.0)
    r0 = oracle.double_softmax_from_descriptors(fA, fB, xA, xB, wz, bz)
    s = r0["scores0"][r0["matches0"] >= 0]
    thr = float(np.median(s))  # about half of the mutual matches pass
    out = sg.sg_stage_match_ds(dev(fA), dev(fB), dev(xA), dev(xB), dev(wz), bz, threshold=thr)
    r = oracle.double_softmax_from_descriptors(fA, fB, xA, xB, wz, bz, threshold=thr)
    _check(out, r, threshold=thr)
    n = int((host(out["matches0"]) >= 0).sum())
    assert 0 < n < int((r0["matches0"] >= 0).sum())


def test_stage_max_size():
    """4096 x 4096 points (the library's limit): sampled rows and the dustbin
    row of logP, and every match decision."""
    M = N = 4096
    fA, fB, xA, xB, wz, bz = _head_inputs(M, N, 64, seed=17)
    out = sg.sg_stage_match_ds(dev(fA), dev(fB), dev(xA), dev(xB), dev(wz), bz)
    r = oracle.double_softmax_from_descriptors(fA, fB, xA, xB, wz, bz)
    g = host(out["logP"])
    rows = np.concatenate([np.random.Generator(np.random.PCG64(0)).choice(M, 63, replace=False), [M]])
    assert np.abs(g[rows] - r["logP"][rows]).max() < _tol(r["logP"])
    assert np.abs(g[:, N] - r["logP"][:, N]).max() < 1e-3
    check_matches(host(out["matches0"]), host(out["matches1"]), r["logP"], r["matches0"], r["matches1"])


def test_stage_deterministic_and_graph_replay():
    """Repeated identical calls (the second is captured into a graph, later
    ones replay it) equal the first bitwise."""
    fA, fB, xA, xB, wz, bz = _head_inputs(600, 500, 256, seed=23)
    t = [dev(a) for a in (fA, fB, xA, xB, wz)]
    first = sg.sg_stage_match_ds(*t, bz)
    torch.cuda.synchronize()
    first = {k: v.clone() for k, v in first.items() if isinstance(v, torch.Tensor)}
    for _ in range(4):
        again = sg.sg_stage_match_ds(*t, bz)
        torch.cuda.synchronize()
        for k in first:
            assert torch.equal(again[k], first[k]), k


# ------------------------------------------------------------- whole pass

def _run(pair, W, cfg, **kw):
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")
    img = (*pair["image_size0"], *pair["image_size1"])
    out = sg.sg_match(*[dev(pair[k]) for k in keys], W, cfg.L, cfg.T, image_size=img, want_logP=True,
                      want_desc=True, **kw)
    torch.cuda.synchronize()
    return {k: host(v) if isinstance(v, torch.Tensor) else v for k, v in out.items()}


@functools.lru_cache(maxsize=None)
def _case(wl, bias_on):
    cfg = synth.WORKLOADS[wl]
    w = synth.make_weights(cfg, bias_on=bias_on)
    pair = synth.make_pair(cfg)
    return cfg, w, pair, oracle.double_softmax_match(pair, w)


@pytest.mark.parametrize("wl,bias_on", [
    ("pair10x12_f32", False),
    ("pair10x12_f32", True),
    ("pair512_f32", False),
    ("pair512_f32", True),
    ("pair2048x1536_f32", False),
])
def test_end_to_end_fp32(wl, bias_on):
    cfg, w, pair, ref = _case(wl, bias_on)
    g = _run(pair, sg.pack_weights(w, head="ds"), cfg)
    e = max(rel_rows(g["f0"], ref["f0"]).max(), rel_rows(g["f1"], ref["f1"]).max())
    dl = np.abs(g["logP"] - ref["logP"]).max()
    ex = check_matches(g["matches0"], g["matches1"], ref["logP"], ref["matches0"], ref["matches1"])
    print(f"{wl} bias={bias_on}: f rel err {e:.2e}, |dlogP| {dl:.2e} (|logP| up to "
          f"{np.abs(ref['logP']).max():.0f}), matches {int((ref['matches0'] >= 0).sum())}, exempt {ex}")
    assert e < 1e-4
    # with zero biases the bar is 1e-3; see _bar_S for the nonzero-bias scores
    tol = _bar_S(ref)
    print(f"max |S| {np.abs(ref['S']).max():.0f}, bar {tol:.2e}")
    assert dl < tol
    ok = g["matches0"] == ref["matches0"]
    np.testing.assert_allclose(g["scores0"][ok], ref["scores0"][ok], rtol=2e-3, atol=1e-6)


@pytest.mark.parametrize("wl,bias_on", [("pair1024_bf16", False), ("pair1024_bf16", True), ("pair512_f32", True)])
def test_head_on_gpu_states(wl, bias_on):
    """The head of sg_match against the oracle's head applied to the GPU's own
    last states and descriptors, which the stage entry points reproduce
    bitwise (checked on f): the bf16 network at 1024 x 1024, and the fp32
    network whose nonzero biases grow the scores to thousands."""
    cfg = synth.WORKLOADS[wl]
    w = synth.make_weights(cfg, bias_on=bias_on)
    pair = synth.make_pair(cfg)
    W = sg.pack_weights(w, head="ds")
    g = _run(pair, W, cfg)
    img = pair["image_size0"]
    xs = [sg.sg_stage_encode(dev(pair["kpts" + s]), dev(pair["conf" + s]), dev(pair["desc" + s]), W, img)
          for s in ("0", "1")]
    sg.sg_stage_gnn(xs[0], xs[1], W, 0, 2 * cfg.L)
    fs = [sg.sg_stage_project(x, W) for x in xs]
    torch.cuda.synchronize()
    assert np.array_equal(host(fs[0]), g["f0"]) and np.array_equal(host(fs[1]), g["f1"])
    r = oracle.double_softmax_from_descriptors(g["f0"], g["f1"], host(xs[0]), host(xs[1]), w["wz"], w["bz"])
    dl = np.abs(g["logP"] - r["logP"]).max()
    ex = check_matches(g["matches0"], g["matches1"], r["logP"], r["matches0"], r["matches1"])
    print(f"{wl} bias={bias_on}: |dlogP| {dl:.2e} (max |S| {np.abs(r['S']).max():.0f}), "
          f"matches {int((r['matches0'] >= 0).sum())}, exempt {ex}")
    assert dl < _bar_S(r)


def test_heads_share_the_network():
    """Both heads run the same encoder, GNN and projection: identical f."""
    cfg, w, pair, _ = _case("pair10x12_f32", True)
    a = _run(pair, sg.pack_weights(w), cfg)
    b = _run(pair, sg.pack_weights(w, head="ds"), cfg)
    assert np.array_equal(a["f0"], b["f0"]) and np.array_equal(a["f1"], b["f1"])


# ------------------------------------------------------------------ batch

_SMALL_BATCH = dataclasses.replace(synth.WORKLOADS["pair10x12_f32"], seed_id=5, batch=7, pad=40, planted="pair",
                                   n_range=(0, 40), frac_range=(0.2, 0.5))


def _run_batch(cfg, W, b):
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")
    img = (*b["image_size0"], *b["image_size1"])
    out = sg.sg_match_batch(b["M"], b["N"], *[dev(b[k]) for k in keys], W, cfg.L, cfg.T, image_size=img,
                            want_logP=True, want_desc=True)
    torch.cuda.synchronize()
    return {k: host(v) if isinstance(v, torch.Tensor) else v for k, v in out.items()}


@pytest.mark.parametrize("batch", [7, sg.SG_MAX_BATCH])
def test_batch_fp32_vs_oracle(batch):
    """A ragged fp32 batch (empty pairs included), of 7 pairs and of the
    largest size the boundary takes: every pair against the oracle end to
    end; padded entries -1 / 0."""
    cfg = _SMALL_BATCH
    w = synth.make_weights(synth.WORKLOADS["pair10x12_f32"], bias_on=True)
    b = synth.make_batch(cfg, seed=408, batch=batch)
    assert len(b["pairs"]) == batch and (b["M"] == 0).any() and (b["N"] == 0).any()
    g = _run_batch(cfg, sg.pack_weights(w, head="ds"), b)
    for i, p in enumerate(b["pairs"]):
        M, N = int(b["M"][i]), int(b["N"][i])
        ref = oracle.double_softmax_match(p, w)
        assert (g["matches0"][i, M:] == -1).all() and (g["scores0"][i, M:] == 0).all()
        assert (g["matches1"][i, N:] == -1).all()
        if M == 0 or N == 0:
            assert (g["matches0"][i] == -1).all() and (g["matches1"][i] == -1).all()
            continue
        check_matches(g["matches0"][i, :M], g["matches1"][i, :N], ref["logP"], ref["matches0"], ref["matches1"])
        dl = np.abs(g["logP"][i, :M + 1, :N + 1] - ref["logP"]).max()
        assert dl < 1e-3, (i, M, N, dl)


def test_batch_bf16_pairs_independent_and_close_to_single():
    """The 32-pair ragged bf16 batch: reversing the batch reverses the results
    bitwise, and sampled pairs agree with sg_match on the unpadded pair to the
    bf16 descriptor bar."""
    cfg = synth.WORKLOADS["ragged32_bf16"]
    w = synth.make_weights(cfg)
    b = synth.make_batch(cfg)
    W = sg.pack_weights(w, head="ds")
    g = _run_batch(cfg, W, b)
    order = np.arange(len(b["M"]))[::-1]
    rb = dict(b)
    for k in ("kpts0", "conf0", "desc0", "kpts1", "conf1", "desc1", "M", "N"):
        rb[k] = np.ascontiguousarray(b[k][order])
    r = _run_batch(cfg, W, rb)
    for k in ("matches0", "scores0", "matches1", "logP"):
        assert np.array_equal(r[k], g[k][order], equal_nan=True), k
    worst, agree = 0.0, []
    for i in range(0, len(b["M"]), 5):
        M, N = int(b["M"][i]), int(b["N"][i])
        s = _run(b["pairs"][i], W, cfg)
        worst = max(worst, rel_rows(g["f0"][i, :M], s["f0"]).max(), rel_rows(g["f1"][i, :N], s["f1"]).max())
        agree.append((g["matches0"][i, :M] == s["matches0"]).mean())
    print(f"ds batch vs single: f rel diff {worst:.2e}, match agreement {np.mean(agree):.3f}")
    assert worst < 2e-2 and np.mean(agree) > 0.9
