"""The scores, Sinkhorn and extraction stage entry points (sg_stage_scores,
sg_stage_sinkhorn, sg_stage_extract) against the oracle, through the C ABI
(GPU).

sg_stage_scores projects both images' last states and writes the bordered
score matrix: within 1e-4 of the oracle's final projection and score matrix
(relative to max |S| where that exceeds 1), the border exactly the dustbin
score; bf16 networks are compared on states rounded to bf16, the operands the
GPU's projection reads.

sg_stage_sinkhorn runs the pass's own sweep kernels on caller-given
couplings: duals u, v and the log assignment within 1e-3 absolute of the
oracle's (realcat notes, "Sinkhorn Algorithm"), column sums of exp(logP)
equal to the marginals b = [1_N, M].  sg_stage_extract runs the pass's
extraction kernels on a given log assignment: matches bit-exact (the argmax
decisions are comparisons of the same fp32 values), except where the
threshold decision lies within 1e-3 of log(threshold) (float against
double logarithm); scores within 1e-6 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_matches, dev, host

pytestmark = pytest.mark.gpu

sg = pytest.importorskip("learned_sparse_feature_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sg.lib()


def _couplings(M, N, seed, alpha=1.0, border="alpha"):
    """Scores of planted matching descriptors bordered by the dustbins: the
    constant alpha (as in the pass) or arbitrary per-entry dustbin values."""
    fA, fB = synth.random_matching_descriptors(M, N, 256, seed=seed)
    S = oracle.score_matrix(fA, fB)
    Z = np.full((M + 1, N + 1), alpha)
    Z[:M, :N] = S
    if border == "random":
        rng = np.random.Generator(np.random.PCG64(seed + 1))
        Z[M, :] = rng.uniform(-3, 3, N + 1)
        Z[:, N] = rng.uniform(-3, 3, M + 1)
    return np.ascontiguousarray(Z, np.float32)


def _oracle_sinkhorn(Z, T):
    M, N = Z.shape[0] - 1, Z.shape[1] - 1
    lmn = np.log(M + N)
    lmu = np.log(np.append(np.ones(M), N)) - lmn
    lnu = np.log(np.append(np.ones(N), M)) - lmn
    out, u, v = oracle.log_sinkhorn_iterations(Z.astype(np.float64), lmu, lnu, T, duals=True)
    return out + lmn, u, v


@pytest.mark.parametrize("M,N,T,border", [
    (3, 4, 0, "alpha"), (3, 4, 1, "alpha"), (5, 7, 20, "random"), (1, 1, 10, "alpha"), (1, 300, 50, "random"),
    (300, 1, 50, "alpha"), (64, 64, 100, "random"), (257, 1025, 100, "alpha"), (1024, 1024, 100, "alpha"),
    (1024, 1024, 100, "random"), (2048, 1536, 100, "alpha"), (4096, 333, 20, "random")])
def test_sinkhorn_stage_vs_oracle(M, N, T, border):
    Z = _couplings(M, N, seed=M * 31 + N, border=border)
    g = sg.sg_stage_sinkhorn(dev(Z), T)
    torch.cuda.synchronize()
    logP, u, v = _oracle_sinkhorn(Z, T)
    du = np.abs(host(g["u"]) - u).max()
    dv = np.abs(host(g["v"]) - v).max()
    dl = np.abs(host(g["logP"]) - logP).max()
    print(f"{M}x{N} T={T} {border}: |du| {du:.2e} |dv| {dv:.2e} |dlogP| {dl:.2e} (|logP| up to "
          f"{np.abs(logP).max():.0f})")
    assert max(du, dv, dl) < 1e-3
    if T >= 1:
        cs = np.exp(host(g["logP"]).astype(np.float64)).sum(axis=0)
        np.testing.assert_allclose(cs, np.append(np.ones(N), M), rtol=1e-4)
    else:
        assert (host(g["u"]) == 0).all() and (host(g["v"]) == 0).all()


def test_sinkhorn_stage_equals_the_pass():
    """With the constant dustbin the stage entry point runs the same sweeps as
    sg_stage_match (the pass's optimal-matching layer) on the same scores."""
    M, N, T = 700, 500, 100
    fA, fB = synth.random_matching_descriptors(M, N, 256, seed=5)
    m = sg.sg_stage_match(dev(fA), dev(fB), 1.0, T, sinkhorn="two")
    torch.cuda.synchronize()
    S = oracle.score_matrix(fA, fB)
    Z = np.full((M + 1, N + 1), 1.0)
    Z[:M, :N] = S
    g = sg.sg_stage_sinkhorn(dev(np.ascontiguousarray(Z, np.float32)), T)
    torch.cuda.synchronize()
    assert np.abs(host(g["logP"]) - host(m["logP"])).max() < 1e-3


def test_sinkhorn_stage_graph_replay():
    """Identical repeated calls replay a captured graph: every replay equals
    the eager result bitwise, with other work in between."""
    Z = dev(_couplings(200, 150, seed=9, border="random"))
    ref = sg.sg_stage_sinkhorn(Z, 30, graph=False)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}
    other = dev(_couplings(90, 40, seed=10))
    for _ in range(4):
        g = sg.sg_stage_sinkhorn(Z, 30)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(g[k], ref[k]), k
        sg.sg_stage_sinkhorn(other, 5, graph=False)
        torch.cuda.synchronize()


def _extract_case(M, N, seed, kind):
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "ties":
        # few distinct values: many equal maxima in rows and columns
        return np.ascontiguousarray(-0.5 * rng.integers(0, 4, (M + 1, N + 1)), np.float32)
    Z = _couplings(M, N, seed)
    logP, _, _ = _oracle_sinkhorn(Z, 100)
    return np.ascontiguousarray(logP, np.float32)


@pytest.mark.parametrize("M,N,kind,thr", [
    (6, 5, "ties", 0.0), (6, 5, "ties", 0.7), (40, 40, "ties", 0.3), (1, 1, "sinkhorn", 0.0),
    (1, 300, "sinkhorn", 0.0), (300, 1, "sinkhorn", 0.2), (257, 1025, "sinkhorn", 0.0),
    (1024, 1024, "sinkhorn", 0.0), (1024, 1024, "sinkhorn", 0.2), (2048, 1536, "sinkhorn", 0.5),
    (4096, 70, "ties", 0.5)])
def test_extract_stage_vs_oracle(M, N, kind, thr):
    P = _extract_case(M, N, seed=M + 7 * N, kind=kind)
    g = sg.sg_stage_extract(dev(P), threshold=thr)
    torch.cuda.synchronize()
    m0, s0, m1, s1 = oracle.extract_matches(P.astype(np.float64), thr)
    gm0, gm1 = host(g["matches0"]), host(g["matches1"])
    ex = check_matches(gm0, gm1, P.astype(np.float64), m0, m1, threshold=thr, gap=0.0)
    print(f"{M}x{N} {kind} thr={thr}: matches {int((m0 >= 0).sum())}, threshold exemptions {ex}")
    assert ex <= 2
    np.testing.assert_allclose(host(g["scores0"]), s0, rtol=1e-6, atol=1e-30)
    np.testing.assert_allclose(host(g["scores1"]), s1, rtol=1e-6, atol=1e-30)


@pytest.mark.parametrize("M,N", [(0, 5), (4, 0), (0, 0)])
def test_extract_stage_empty(M, N):
    P = torch.zeros((M + 1, N + 1), dtype=torch.float32, device="cuda")
    g = sg.sg_stage_extract(P)
    torch.cuda.synchronize()
    assert (host(g["matches0"]) == -1).all() and (host(g["scores0"]) == 0).all()
    assert (host(g["matches1"]) == -1).all() and (host(g["scores1"]) == 0).all()


def test_extract_after_sinkhorn_stage_is_the_pass():
    """sg_stage_sinkhorn then sg_stage_extract gives sg_stage_match's matches
    (away from near ties)."""
    M, N, T = 512, 640, 100
    fA, fB = synth.random_matching_descriptors(M, N, 256, seed=21)
    m = sg.sg_stage_match(dev(fA), dev(fB), 1.0, T)
    S = oracle.score_matrix(fA, fB)
    Z = np.full((M + 1, N + 1), 1.0)
    Z[:M, :N] = S
    g = sg.sg_stage_sinkhorn(dev(np.ascontiguousarray(Z, np.float32)), T)
    e = sg.sg_stage_extract(g["logP"])
    torch.cuda.synchronize()
    ref = oracle.match_from_descriptors(fA, fB, 1.0, T)
    check_matches(host(e["matches0"]), host(e["matches1"]), ref["logP"], host(m["matches0"]), host(m["matches1"]))


def _states(cfg, M, N, seed):
    return synth.random_states(M, cfg.D, seed=seed), synth.random_states(N, cfg.D, seed=seed + 1)


def _oracle_scores(cfg, w, xA, xB):
    rnd = synth.round_to_bf16 if cfg.dtype == "bf16" else (lambda a: a)
    M, N = xA.shape[0], xB.shape[0]
    Z = np.full((M + 1, N + 1), w["alpha"])
    fA = fB = None
    if M and N:
        fA = oracle.final_projection(rnd(xA), w["Wf"], w["bf"])
        fB = oracle.final_projection(rnd(xB), w["Wf"], w["bf"])
        Z[:M, :N] = oracle.score_matrix(fA, fB)
    return Z, fA, fB


@pytest.mark.parametrize("wl,M,N", [
    ("pair10x12_f32", 10, 12),
    ("pair512_f32", 300, 257),
    ("pair1024_bf16", 1024, 1024),
    ("pair2048x1536_f32", 2048, 1536),
    ("pair512_f32", 0, 7),
    ("pair512_f32", 5, 0),
    ("pair1024_bf16", 1, 33),
])
def test_scores_stage_vs_oracle(wl, M, N):
    cfg = synth.WORKLOADS[wl]
    w = synth.make_weights(cfg)
    W = sg.pack_weights(w)
    xA, xB = _states(cfg, M, N, seed=900 + 7 * M + N)
    Z = host(sg.sg_stage_scores(dev(xA), dev(xB), W))
    ref, _, _ = _oracle_scores(cfg, w, xA, xB)
    assert Z.shape == (M + 1, N + 1)
    assert (Z[M, :] == np.float32(w["alpha"])).all() and (Z[:, N] == np.float32(w["alpha"])).all()
    err = np.abs(Z - ref).max()
    big = np.abs(ref).max()
    print(f"{wl} {M}x{N}: max |dZ| {err:.2e}, max |Z| {big:.2f}")
    assert err < 1e-4 * max(1.0, big)


def test_stage_chain_scores_sinkhorn_extract():
    """From the last states through the stage entry points (scores, then
    Sinkhorn, then extraction) against the oracle's head on the oracle's
    projection of the same states."""
    cfg = synth.WORKLOADS["pair512_f32"]
    w = synth.make_weights(cfg)
    W = sg.pack_weights(w)
    M, N = 300, 257
    xA, xB = _states(cfg, M, N, seed=77)
    Z = sg.sg_stage_scores(dev(xA), dev(xB), W)
    r = sg.sg_stage_sinkhorn(Z, cfg.T)
    e = sg.sg_stage_extract(r["logP"])
    _, fA, fB = _oracle_scores(cfg, w, xA, xB)
    ref = oracle.match_from_descriptors(fA, fB, w["alpha"], cfg.T)
    err = np.abs(host(r["logP"]) - ref["logP"]).max()
    print(f"chain {M}x{N}: max |dlogP| {err:.2e}")
    assert err < 1e-3
    check_matches(host(e["matches0"]), host(e["matches1"]), ref["logP"], ref["matches0"], ref["matches1"])
