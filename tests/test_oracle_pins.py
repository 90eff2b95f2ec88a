"""Pins of the float64 CPU oracle against what the pages and the mathematics fix.

Each test targets one step of the matching pass and is chosen so that a
plausible mistake in it (a dropped term, a wrong sign, index or axis, a
transposed operand, a sequential instead of simultaneous update) fails.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from golden_io import attention_example, normalize_example, sinkhorn_demo


@pytest.fixture(autouse=True)
def _each_oracle(oracle_impl, monkeypatch):
    """Every pin runs against both oracle implementations (plain C, numpy)."""
    monkeypatch.setitem(globals(), "oracle", oracle_impl)



def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_stage(rng, D, scale=0.3):
    st = {}
    for name, n_out, n_in in (("q", D, D), ("k", D, D), ("v", D, D), ("m", D, D),
                              ("1", 2 * D, 2 * D), ("2", D, 2 * D)):
        st["W" + name] = scale * rng.standard_normal((n_out, n_in))
        st["b" + name] = scale * rng.standard_normal(n_out)
    return st


# ----------------------------------------------------------------- attention

def test_attention_worked_example():
    """Scores [2,1,0] -> weights ~[0.665,0.245,0.090], message ~[0.665,0.245]."""
    ex = attention_example()
    s = ex["scores"]
    # one head of dimension 2: q = [sqrt(2), 0] and k_j = [s_j, 0] give q.k_j / sqrt(2) = s_j
    x = np.array([[np.sqrt(2.0), 0.0]])
    src = np.array([[s[0], 0.0], [s[1], 1.0], [s[2], 0.0]])
    st = {"Wq": np.eye(2), "bq": np.zeros(2),
          "Wk": np.array([[1.0, 0.0], [0.0, 0.0]]), "bk": np.zeros(2),
          # maps the sources to the page's values [1,0], [0,1], [0,0]
          "Wv": np.array([[0.5, -0.5], [0.0, 1.0]]), "bv": np.zeros(2),
          "Wm": np.eye(2), "bm": np.zeros(2)}
    v = src @ st["Wv"].T
    np.testing.assert_allclose(v, np.stack([ex["value0"], ex["value1"], ex["value2"]]), atol=1e-15)
    m = oracle.multi_head_attention(x, src, st, heads=1)[0]
    np.testing.assert_allclose(m, ex["message"], atol=5e-4)
    w = np.array([m[0], m[1], 1.0 - m[0] - m[1]])
    np.testing.assert_allclose(w, ex["weights"], atol=5e-4)


def test_attention_matches_torch_multihead_library():
    """Heads in contiguous channel blocks, 1/sqrt(d_head) scaling and the merge
    projection equal torch's multi-head attention routine (float64, CPU)."""
    rng = _rng(7)
    D, H, n, m = 32, 4, 7, 9
    st = _rand_stage(rng, D)
    x = rng.standard_normal((n, D))
    src = rng.standard_normal((m, D))
    ours = oracle.multi_head_attention(x, src, st, H)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    ref, _ = F.multi_head_attention_forward(
        t(x)[:, None, :], t(src)[:, None, :], t(src)[:, None, :], D, H,
        t(np.concatenate([st["Wq"], st["Wk"], st["Wv"]])),
        t(np.concatenate([st["bq"], st["bk"], st["bv"]])),
        None, None, False, 0.0, t(st["Wm"]), t(st["bm"]), training=False, need_weights=False)
    np.testing.assert_allclose(ours, ref[:, 0, :].numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ encoder

def test_normalize_keypoints_worked_example():
    w, h, px, expect = normalize_example()
    got = oracle.normalize_keypoints(px, w, h)
    np.testing.assert_allclose(got, expect, rtol=1e-4, atol=1e-8)


def test_encoder_matches_conv1d_stack():
    """Per-point linear layers = the pages' Conv1d(kernel 1) MLP, ReLU between."""
    rng = _rng(3)
    widths = [3, 16, 32, 64]
    layers = [(rng.standard_normal((widths[i + 1], widths[i])), rng.standard_normal(widths[i + 1]))
              for i in range(3)]
    kp = rng.uniform(-0.7, 0.7, (11, 2))
    c = rng.uniform(0, 1, 11)
    ours = oracle.keypoint_encoder(kp, c, layers)
    h = torch.from_numpy(np.concatenate([kp.T, c[None]], axis=0))[None]   # [1, 3, n]
    for i, (W, b) in enumerate(layers):
        h = F.conv1d(h, torch.from_numpy(W)[:, :, None], torch.from_numpy(b))
        if i < len(layers) - 1:
            h = torch.relu(h)
    np.testing.assert_allclose(ours, h[0].numpy().T, rtol=1e-12, atol=1e-12)


def test_encoder_no_relu_after_last_layer():
    layers = [(np.eye(3), np.zeros(3)), (-np.eye(3), np.zeros(3))]
    out = oracle.keypoint_encoder(np.array([[0.5, 0.25]]), np.array([0.75]), layers)
    np.testing.assert_allclose(out, [[-0.5, -0.25, -0.75]])


# ---------------------------------------------------------------------- GNN

def _mean_stage(D):
    """Weights whose update is delta_i = mean_j src_j for positive states:
    uniform attention (W_q = W_k = 0), v = src, merge = I, and an MLP that
    passes the message through (ReLU of a positive value)."""
    Z, I = np.zeros((D, D)), np.eye(D)
    return {"Wq": Z, "bq": np.zeros(D), "Wk": Z, "bk": np.zeros(D), "Wv": I, "bv": np.zeros(D),
            "Wm": I, "bm": np.zeros(D),
            "W1": np.block([[Z, I], [Z, Z]]), "b1": np.zeros(2 * D),
            "W2": np.block([I, Z]), "b2": np.zeros(D)}


def _zero_stage(D):
    st = _mean_stage(D)
    st["W2"] = np.zeros((D, 2 * D))
    return st


def test_gnn_first_stage_is_self():
    rng = _rng(11)
    D = 8
    xA, xB = rng.uniform(0.1, 1, (5, D)), rng.uniform(0.1, 1, (7, D))
    A, B = oracle.attentional_gnn(xA, xB, [_mean_stage(D), _zero_stage(D)], heads=2)
    np.testing.assert_allclose(A, xA + xA.mean(0), rtol=1e-13)
    np.testing.assert_allclose(B, xB + xB.mean(0), rtol=1e-13)


def test_gnn_second_stage_is_cross_and_simultaneous():
    rng = _rng(12)
    D = 8
    xA, xB = rng.uniform(0.1, 1, (5, D)), rng.uniform(0.1, 1, (7, D))
    A, B = oracle.attentional_gnn(xA, xB, [_zero_stage(D), _mean_stage(D)], heads=2)
    np.testing.assert_allclose(A, xA + xB.mean(0), rtol=1e-13)
    np.testing.assert_allclose(B, xB + xA.mean(0), rtol=1e-13)   # from A's pre-stage state


def test_gnn_stage_count_is_twice_L():
    rng = _rng(13)
    D = 8
    st = _zero_stage(D)
    st["b2"] = np.full(D, 0.25)
    xA, xB = rng.uniform(0.1, 1, (3, D)), rng.uniform(0.1, 1, (4, D))
    L = 3
    A, _ = oracle.attentional_gnn(xA, xB, [st] * (2 * L), heads=2)
    np.testing.assert_allclose(A, xA + 2 * L * 0.25, rtol=1e-13)


def _random_weights(wl="pair10x12_f32", bias_on=True):
    return synth.make_weights(synth.WORKLOADS[wl], bias_on=bias_on)


def test_gnn_permutation_equivariance():
    w = _random_weights()
    rng = _rng(14)
    xA, xB = rng.standard_normal((10, 64)), rng.standard_normal((12, 64))
    A, B = oracle.attentional_gnn(xA, xB, w["stages"], 4)
    p = rng.permutation(10)
    A2, B2 = oracle.attentional_gnn(xA[p], xB, w["stages"], 4)
    np.testing.assert_allclose(A2, A[p], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(B2, B, rtol=1e-11, atol=1e-11)


def test_gnn_swap_symmetry():
    w = _random_weights()
    rng = _rng(15)
    xA, xB = rng.standard_normal((10, 64)), rng.standard_normal((12, 64))
    A, B = oracle.attentional_gnn(xA, xB, w["stages"], 4)
    B2, A2 = oracle.attentional_gnn(xB, xA, w["stages"], 4)
    np.testing.assert_allclose(A2, A, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(B2, B, rtol=1e-11, atol=1e-11)


def test_full_pass_permutation_equivariance():
    """Permuting A's keypoints permutes matches0 and relabels matches1."""
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = _random_weights()
    pair = synth.make_pair(cfg)
    r = oracle.superglue_match(pair, w, T=cfg.T)
    p = _rng(16).permutation(cfg.M)
    pair2 = dict(pair)
    for k in ("kpts0", "conf0", "desc0"):
        pair2[k] = pair[k][p]
    r2 = oracle.superglue_match(pair2, w, T=cfg.T)
    np.testing.assert_array_equal(r2["matches0"], r["matches0"][p])
    inv = np.argsort(p)
    m1 = np.where(r["matches1"] >= 0, inv[np.maximum(r["matches1"], 0)], -1)
    np.testing.assert_array_equal(r2["matches1"], m1)
    np.testing.assert_allclose(r2["logP"][:-1], r["logP"][:-1][p], atol=1e-9)


# ---------------------------------------------------------- scores, OT

def test_score_matrix_brute_force():
    rng = _rng(17)
    fA, fB = rng.standard_normal((3, 16)), rng.standard_normal((5, 16))
    S = oracle.score_matrix(fA, fB)
    for i in range(3):
        for j in range(5):
            assert abs(S[i, j] - sum(fA[i, d] * fB[j, d] for d in range(16)) / 4.0) < 1e-12


def _marginals(M, N):
    a = np.concatenate([np.ones(M), [N]])
    b = np.concatenate([np.ones(N), [M]])
    return a, b


@pytest.mark.parametrize("T", [1, 3, 20])
def test_sinkhorn_rank_one_closed_form(T):
    """Z_ij = c + r_i + g_j: every iterate gives Z + u + v = log mu_i + log nu_j."""
    rng = _rng(18)
    M, N = 4, 6
    Z = 0.7 + rng.standard_normal(M + 1)[:, None] + rng.standard_normal(N + 1)[None, :]
    a, b = _marginals(M, N)
    log_mu, log_nu = np.log(a / (M + N)), np.log(b / (M + N))
    out = oracle.log_sinkhorn_iterations(Z, log_mu, log_nu, T)
    np.testing.assert_allclose(out, log_mu[:, None] + log_nu[None, :], atol=1e-12)


def test_optimal_transport_constant_scores_closed_form():
    """S = alpha everywhere: logP = log a_i + log b_j - log(M+N)."""
    M, N, alpha = 5, 3, 1.3
    logP = oracle.log_optimal_transport(np.full((M, N), alpha), alpha, 4)
    a, b = _marginals(M, N)
    np.testing.assert_allclose(logP, np.log(a)[:, None] + np.log(b)[None, :] - np.log(M + N), atol=1e-12)


def test_sinkhorn_row_shift_invariance():
    rng = _rng(19)
    M, N = 6, 5
    Z = 4 * rng.standard_normal((M + 1, N + 1))
    a, b = _marginals(M, N)
    lm, ln = np.log(a / (M + N)), np.log(b / (M + N))
    r = 10 * rng.standard_normal(M + 1)
    for T in (1, 7):
        # u absorbs the shift (u -> u - r), so Z + u + v is unchanged at every iterate
        np.testing.assert_allclose(oracle.log_sinkhorn_iterations(Z + r[:, None], lm, ln, T),
                                   oracle.log_sinkhorn_iterations(Z, lm, ln, T), atol=1e-11)


@pytest.mark.parametrize("T", [1, 5, 100])
def test_column_sums_exact_after_each_iteration(T):
    rng = _rng(20)
    M, N = 9, 6
    S = 20 * rng.standard_normal((M, N))
    P = np.exp(oracle.log_optimal_transport(S, 1.0, T))
    _, b = _marginals(M, N)
    np.testing.assert_allclose(P.sum(axis=0), b, rtol=1e-10)


@pytest.mark.parametrize("T", [1, 5, 20])
def test_log_domain_equals_exp_domain_sinkhorn_knopp(T):
    rng = _rng(21)
    M, N, alpha = 6, 8, 0.4
    S = 2 * rng.standard_normal((M, N))
    Zbar = np.full((M + 1, N + 1), alpha)
    Zbar[:M, :N] = S
    a, b = _marginals(M, N)
    Pk = oracle.sinkhorn_knopp_exp(Zbar, a, b, T)
    Pl = np.exp(oracle.log_optimal_transport(S, alpha, T))
    np.testing.assert_allclose(Pl, Pk, rtol=1e-10, atol=1e-14)


def test_marginals_converge():
    """Row sums reach a = [1_M, N] and column sums b = [1_N, M]."""
    rng = _rng(22)
    M, N = 7, 4
    S = rng.uniform(-2, 2, (M, N))
    P = np.exp(oracle.log_optimal_transport(S, 0.5, 3000))
    a, b = _marginals(M, N)
    np.testing.assert_allclose(P.sum(axis=1), a, atol=1e-6)
    np.testing.assert_allclose(P.sum(axis=0), b, atol=1e-9)


def _brute_force_assignment(Sbar_real, alpha):
    """All partial matchings of an MxN problem; objective sum S_ij + alpha (M+N-k)."""
    M, N = Sbar_real.shape
    best = []
    for k in range(0, min(M, N) + 1):
        for rows in itertools.combinations(range(M), k):
            for cols in itertools.permutations(range(N), k):
                val = sum(Sbar_real[i, j] for i, j in zip(rows, cols)) + alpha * (M + N - k)
                best.append((val, dict(zip(rows, cols))))
    best.sort(key=lambda t: -t[0])
    return best


def test_brute_force_enumeration_count():
    # sum_k C(3,k) P(4,k) = 1 + 12 + 36 + 24 = 73 partial matchings of a 3x4 problem
    assert len(_brute_force_assignment(np.zeros((3, 4)), 0.0)) == 73


def _check_assignment(S, alpha, beta=200.0, T=4000):
    ranked = _brute_force_assignment(S, alpha)
    (v0, opt), (v1, _) = ranked[0], ranked[1]
    if v0 - v1 < 0.1:
        return False
    logP = oracle.log_optimal_transport(beta * S, beta * alpha, T)
    m0, _, _, _ = oracle.extract_matches(logP, threshold=0.5)
    want = np.array([opt.get(i, -1) for i in range(S.shape[0])])
    np.testing.assert_array_equal(m0, want)
    # the transport objective approaches the LP optimum
    P = np.exp(logP)
    Sbar = np.full((S.shape[0] + 1, S.shape[1] + 1), alpha)
    Sbar[:-1, :-1] = S
    assert abs((P * Sbar).sum() - v0) < 0.05
    return True


def test_brute_force_optimal_assignment_demo_matrix():
    S, dust = sinkhorn_demo()
    assert _check_assignment(-S, -dust)     # cost -> similarity


def test_brute_force_optimal_assignment_random():
    rng = _rng(23)
    checked = 0
    for _ in range(150):
        S = rng.uniform(-1, 1, (3, 4))
        alpha = rng.uniform(-0.6, 0.6)
        checked += _check_assignment(S, alpha)
    assert checked > 50


# -------------------------------------------------------------- extraction

def _brute_extract(logP, thr):
    P = logP[:-1, :-1]
    M, N = P.shape
    m0, s0 = -np.ones(M, int), np.zeros(M)
    m1, s1 = -np.ones(N, int), np.zeros(N)
    for i in range(M):
        for j in range(N):
            row_first = all(P[i, jj] < P[i, j] for jj in range(j)) and all(P[i, jj] <= P[i, j] for jj in range(N))
            col_first = all(P[ii, j] < P[i, j] for ii in range(i)) and all(P[ii, j] <= P[i, j] for ii in range(M))
            if row_first and col_first:
                s0[i] = s1[j] = np.exp(P[i, j])
                if np.exp(P[i, j]) > thr:
                    m0[i], m1[j] = j, i
    return m0, s0, m1, s1


@pytest.mark.parametrize("seed", range(6))
def test_extraction_brute_force(seed):
    rng = _rng(100 + seed)
    M, N = rng.integers(1, 7), rng.integers(1, 7)
    logP = -rng.integers(0, 4, (M + 1, N + 1)).astype(float) * 0.5   # many ties
    thr = [0.0, 0.3, 0.7][seed % 3]
    got = oracle.extract_matches(logP, thr)
    want = _brute_extract(logP, thr)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w)


def test_empty_inputs():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = _random_weights()
    pair = synth.make_pair(cfg, M=0)
    r = oracle.superglue_match(pair, w, T=5)
    assert r["matches0"].shape == (0,)
    np.testing.assert_array_equal(r["matches1"], -np.ones(cfg.N))
    np.testing.assert_array_equal(r["scores1"], np.zeros(cfg.N))


def test_mlp_has_no_relu_after_last_layer():
    """A negative update survives: the second MLP layer is not rectified."""
    rng = _rng(24)
    D = 8
    st = _mean_stage(D)
    st["W2"] = -st["W2"]
    xA, xB = rng.uniform(0.1, 1, (5, D)), rng.uniform(0.1, 1, (7, D))
    A, B = oracle.attentional_gnn(xA, xB, [st, _zero_stage(D)], heads=2)
    np.testing.assert_allclose(A, xA - xA.mean(0), rtol=1e-13)


def test_final_projection_orientation():
    """f_i = W x_i + b with W stored [out][in], checked element by element."""
    rng = _rng(25)
    W, b, x = rng.standard_normal((5, 3)), rng.standard_normal(5), rng.standard_normal((4, 3))
    f = oracle.final_projection(x, W, b)
    for i in range(4):
        for o in range(5):
            assert abs(f[i, o] - (sum(W[o, k] * x[i, k] for k in range(3)) + b[o])) < 1e-12


def test_extraction_threshold_is_exact_for_tiny_probabilities():
    """A mutual match whose exp underflows in floating point still has a
    positive score in exact arithmetic, so it is valid at threshold 0."""
    logP = np.full((3, 3), -2000.0)
    logP[0, 0] = -800.0           # exp(-800) == 0.0 in float64
    logP[1, 1] = np.log(0.3)
    m0, s0, m1, _ = oracle.extract_matches(logP, 0.0)
    np.testing.assert_array_equal(m0, [0, 1])
    m0, _, _, _ = oracle.extract_matches(logP, 0.25)
    np.testing.assert_array_equal(m0, [-1, 1])
    m0, _, _, _ = oracle.extract_matches(logP, 0.35)
    np.testing.assert_array_equal(m0, [-1, -1])


def test_gnn_slice_starting_at_an_odd_stage_is_cross():
    rng = _rng(26)
    D = 8
    xA, xB = rng.uniform(0.1, 1, (5, D)), rng.uniform(0.1, 1, (7, D))
    A, B = oracle.attentional_gnn(xA, xB, [_mean_stage(D)], heads=2, first_stage=1)
    np.testing.assert_allclose(A, xA + xB.mean(0), rtol=1e-13)
    np.testing.assert_allclose(B, xB + xA.mean(0), rtol=1e-13)


def test_update_mlp_hidden_relu_and_bias_by_hand():
    """The update MLP's hidden layer, worked by hand: [realcat] "多层GNN"
    gives MLP([x || m]) with channels [2D, 2D, D] and a ReLU between the two
    layers.  One self stage with D = 2, one head, uniform attention (W_q =
    W_k = 0), v = x and merge = I, so m is the mean of the image's states.
    W1 maps [x || m] to (-m0, -m1, x0, x1) and b1 = (1.75, 0.5, -1.5, 0.25)
    shifts it, so that some hidden pre-activations are negative (the ReLU
    clips them) and every hidden unit depends on b1; W2 adds units (0, 2)
    and (1, 3).
      A = [[1, 3], [2, -1]]: m = (1.5, 1)
        row 0: h = (0.25, -0.5, -0.5, 3.25) -> ReLU (0.25, 0, 0, 3.25) -> (0.25, 3.25)
        row 1: h = (0.25, -0.5,  0.5, -0.75) -> ReLU (0.25, 0, 0.5, 0) -> (0.75, 0)
      B = [[0.5, 0.5]]: m = (0.5, 0.5)
        h = (1.25, 0, -1, 0.75) -> ReLU (1.25, 0, 0, 0.75) -> (1.25, 0.75)
    Dropping the ReLU or b1 changes every one of these rows."""
    Z2, I2 = np.zeros((2, 2)), np.eye(2)
    st = {"Wq": Z2, "bq": np.zeros(2), "Wk": Z2, "bk": np.zeros(2), "Wv": I2, "bv": np.zeros(2),
          "Wm": I2, "bm": np.zeros(2),
          "W1": np.block([[Z2, -I2], [I2, Z2]]), "b1": np.array([1.75, 0.5, -1.5, 0.25]),
          "W2": np.array([[1.0, 0.0, 1.0, 0.0], [0.0, 1.0, 0.0, 1.0]]), "b2": np.zeros(2)}
    xA = np.array([[1.0, 3.0], [2.0, -1.0]])
    xB = np.array([[0.5, 0.5]])
    A, B = oracle.attentional_gnn(xA, xB, [st], heads=1)
    np.testing.assert_allclose(A - xA, [[0.25, 3.25], [0.75, 0.0]], atol=1e-14)
    np.testing.assert_allclose(B - xB, [[1.25, 0.75]], atol=1e-14)
