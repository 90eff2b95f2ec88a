"""Pins of the oracle's double-softmax matching head ([LightGlue-review]
section 2.4) against brute force, closed forms, symmetries and a library
routine, each chosen so that a plausible mistake fails: the same axis used
for both softmaxes, a dropped or sign-flipped sigmoid term, the dustbin row
and column exchanged, the matchability read from the wrong operand.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


@pytest.fixture(autouse=True)
def _each_oracle(oracle_impl, monkeypatch):
    """Every pin runs against both oracle implementations (plain C, numpy)."""
    monkeypatch.setitem(globals(), "oracle", oracle_impl)



def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_brute_force_probability_domain():
    """Every entry of exp(logP) from plain loops in the probability domain:
    a row-softmax probability times a column-softmax probability times two
    sigmoids; the dustbins as the complements 1 - sigmoid; the corner 1."""
    rng = _rng(11)
    M, N = 3, 5
    S = 2.0 * rng.standard_normal((M, N))
    z0 = 1.5 * rng.standard_normal(M)
    z1 = 1.5 * rng.standard_normal(N)
    P = np.exp(oracle.double_softmax_assignment(S, z0, z1))
    for i in range(M):
        for j in range(N):
            row = sum(math.exp(S[i, k]) for k in range(N))
            col = sum(math.exp(S[k, j]) for k in range(M))
            want = (math.exp(S[i, j]) / row) * (math.exp(S[i, j]) / col) * _sigmoid(z0[i]) * _sigmoid(z1[j])
            assert P[i, j] == pytest.approx(want, rel=1e-12)
        assert P[i, N] == pytest.approx(1.0 - _sigmoid(z0[i]), rel=1e-12)
    for j in range(N):
        assert P[M, j] == pytest.approx(1.0 - _sigmoid(z1[j]), rel=1e-12)
    assert P[M, N] == 1.0


def test_additive_scores_closed_form():
    """S_ij = a_i + b_j: the row softmax is b_j - log sum e^b, the column
    softmax a_i - log sum e^a (M != N, so a shared axis fails)."""
    rng = _rng(12)
    M, N = 4, 7
    a = 3.0 * rng.standard_normal(M)
    b = 3.0 * rng.standard_normal(N)
    z0 = rng.standard_normal(M)
    z1 = rng.standard_normal(N)
    S = a[:, None] + b[None, :]
    L = oracle.double_softmax_assignment(S, z0, z1)
    la = math.log(sum(math.exp(x) for x in a))
    lb = math.log(sum(math.exp(x) for x in b))
    ls0 = np.array([math.log(_sigmoid(x)) for x in z0])
    ls1 = np.array([math.log(_sigmoid(x)) for x in z1])
    want = (b[None, :] - lb) + (a[:, None] - la) + ls0[:, None] + ls1[None, :]
    np.testing.assert_allclose(L[:M, :N], want, rtol=0, atol=1e-12)


def test_constant_scores_closed_form():
    """S constant: both softmaxes are uniform, so the real block is
    -log N - log M + log sigmoid(z0_i) + log sigmoid(z1_j) for any constant."""
    M, N = 6, 3
    z0 = np.linspace(-3, 3, M)
    z1 = np.array([-1.0, 0.0, 2.0])
    for c in (-50.0, 0.0, 80.0):
        L = oracle.double_softmax_assignment(np.full((M, N), c), z0, z1)
        want = (-math.log(N) - math.log(M)
                + np.array([math.log(_sigmoid(x)) for x in z0])[:, None]
                + np.array([math.log(_sigmoid(x)) for x in z1])[None, :])
        np.testing.assert_allclose(L[:M, :N], want, rtol=0, atol=1e-12)


def test_single_column_normalises_over_rows():
    """N = 1: the row softmax is 1, so with sigmoid(z0) ~ 1 and z1 = 0 the
    column sums to sigmoid(0) = 1/2, and the dustbin row entry is log 1/2."""
    rng = _rng(13)
    M = 9
    S = 4.0 * rng.standard_normal((M, 1))
    L = oracle.double_softmax_assignment(S, np.full(M, 40.0), np.zeros(1))
    assert np.exp(L[:M, 0]).sum() == pytest.approx(0.5, abs=1e-15)
    assert L[M, 0] == pytest.approx(-math.log(2.0), abs=1e-15)
    # and symmetrically for one row
    L = oracle.double_softmax_assignment(S.T, np.zeros(1), np.full(M, 40.0))
    assert np.exp(L[0, :M]).sum() == pytest.approx(0.5, abs=1e-15)
    assert L[0, M] == pytest.approx(-math.log(2.0), abs=1e-15)


def test_transpose_symmetry():
    """Exchanging the images transposes the whole (M+1) x (N+1) matrix,
    dustbin row and column included."""
    rng = _rng(14)
    M, N = 5, 8
    S = 3.0 * rng.standard_normal((M, N))
    z0, z1 = rng.standard_normal(M), rng.standard_normal(N)
    L = oracle.double_softmax_assignment(S, z0, z1)
    LT = oracle.double_softmax_assignment(S.T, z1, z0)
    np.testing.assert_allclose(LT, L.T, rtol=0, atol=1e-12)


def test_permutation_equivariance():
    rng = _rng(15)
    M, N = 7, 6
    S = 3.0 * rng.standard_normal((M, N))
    z0, z1 = rng.standard_normal(M), rng.standard_normal(N)
    pi, pj = rng.permutation(M), rng.permutation(N)
    L = oracle.double_softmax_assignment(S, z0, z1)
    Lp = oracle.double_softmax_assignment(S[pi][:, pj], z0[pi], z1[pj])
    np.testing.assert_allclose(Lp[:M, :N], L[:M, :N][pi][:, pj], rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lp[:M, N], L[:M, N][pi], rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lp[M, :N], L[M, :N][pj], rtol=0, atol=1e-12)


def test_log_sigmoid_against_library_and_identities():
    z = np.concatenate([np.linspace(-60, 60, 241), [-1000.0, -1e5, 1000.0, 1e5, 0.0]])
    got = oracle.log_sigmoid(z)
    want = F.logsigmoid(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-300)
    assert oracle.log_sigmoid(0.0) == pytest.approx(-math.log(2.0), abs=1e-16)
    assert oracle.log_sigmoid(-1000.0) == pytest.approx(-1000.0, rel=1e-15)
    zz = np.linspace(-30, 30, 61)
    # log(sigmoid(z) / sigmoid(-z)) = z and sigmoid(z) + sigmoid(-z) = 1
    np.testing.assert_allclose(oracle.log_sigmoid(zz) - oracle.log_sigmoid(-zz), zz, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.exp(oracle.log_sigmoid(zz)) + np.exp(oracle.log_sigmoid(-zz)), 1.0,
                               rtol=0, atol=1e-15)


def test_matchability_one_hot_weights():
    """A one-hot weight row reads one coordinate of the state, plus the bias."""
    rng = _rng(16)
    x = rng.standard_normal((5, 12))
    w = np.zeros(12)
    w[7] = 1.0
    np.testing.assert_allclose(oracle.matchability(x, w, 0.25), x[:, 7] + 0.25, rtol=0, atol=0)


def test_diagonal_similarity_matches_and_scores():
    """A dominant diagonal gives mutual matches i <-> i whose score tends to
    sigmoid(z0_i) sigmoid(z1_i) (both softmax probabilities tend to 1)."""
    M = N = 6
    S = np.full((M, N), -1.0) + 60.0 * np.eye(M)
    z0 = np.linspace(-2, 2, M)
    z1 = np.linspace(1, -1, N)
    m0, s0, m1, s1 = oracle.extract_matches(oracle.double_softmax_assignment(S, z0, z1), 0.0)
    assert list(m0) == list(range(M)) and list(m1) == list(range(N))
    want = np.array([_sigmoid(a) * _sigmoid(b) for a, b in zip(z0, z1)])
    np.testing.assert_allclose(s0, want, rtol=1e-12)
    # a threshold above some scores drops exactly those matches, on both sides
    thr = float(np.median(want))
    m0, s0, m1, s1 = oracle.extract_matches(oracle.double_softmax_assignment(S, z0, z1), thr)
    keep = want > thr
    assert list(m0) == [i if k else -1 for i, k in enumerate(keep)]
    assert list(m1) == [j if k else -1 for j, k in enumerate(keep)]


def test_head_reads_states_for_matchability_and_descriptors_for_similarity():
    """double_softmax_from_descriptors: z from x (not f), S from f (not x)."""
    rng = _rng(17)
    M, N, D = 4, 5, 8
    fA, fB = rng.standard_normal((M, D)), rng.standard_normal((N, D))
    xA, xB = rng.standard_normal((M, D)), rng.standard_normal((N, D))
    w, b = rng.standard_normal(D), 0.3
    out = oracle.double_softmax_from_descriptors(fA, fB, xA, xB, w, b)
    np.testing.assert_allclose(out["z0"], [float(xA[i] @ w) + b for i in range(M)], rtol=1e-14)
    np.testing.assert_allclose(out["z1"], [float(xB[j] @ w) + b for j in range(N)], rtol=1e-14)
    np.testing.assert_allclose(out["S"], [[float(fA[i] @ fB[j]) / math.sqrt(D) for j in range(N)]
                                          for i in range(M)], rtol=1e-13)


def test_full_pass_empty_and_weights_present():
    cfg = synth.WORKLOADS["pair512_f32"]
    w = synth.make_weights(cfg, L=1)
    assert w["wz"].shape == (cfg.D,)
    pair = synth.make_pair(cfg, M=0, N=5)
    out = oracle.double_softmax_match(pair, w, L=1)
    assert out["matches0"].shape == (0,)
    assert list(out["matches1"]) == [-1] * 5
