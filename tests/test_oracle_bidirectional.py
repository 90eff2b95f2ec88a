"""Pins of the oracle's bidirectional cross-attention ([LightGlue-review]
section 2.3): one similarity per head, row softmax for image 0's messages and
column softmax for image 1's.  Chosen so that a plausible mistake fails: the
row softmax used for both directions, the similarity not transposed for the
second direction, the value of the wrong image, a missing 1/sqrt(d_h), the
merge projection skipped, or the stage routed to standard attention.
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


def _stage(rng, D, scale=0.3):
    st = {}
    for name, n_out, n_in in (("qk", D, D), ("v", D, D), ("m", D, D), ("1", 2 * D, 2 * D), ("2", D, 2 * D)):
        st["W" + name] = scale * rng.standard_normal((n_out, n_in))
        st["b" + name] = scale * rng.standard_normal(n_out)
    return st


def _torch_mha(x, src, st, heads, D):
    """torch's multi-head attention routine with the query and key projections
    tied to W_qk (float64, CPU)."""
    W = torch.from_numpy(np.concatenate([st["Wqk"], st["Wqk"], st["Wv"]]))
    b = torch.from_numpy(np.concatenate([st["bqk"], st["bqk"], st["bv"]]))
    q = torch.from_numpy(x)[:, None, :]
    kv = torch.from_numpy(src)[:, None, :]
    out, _ = F.multi_head_attention_forward(
        q, kv, kv, D, heads, W, b, None, None, False, 0.0,
        torch.from_numpy(st["Wm"]), torch.from_numpy(st["bm"]), training=False, need_weights=False)
    return out[:, 0, :].numpy()


def test_each_direction_is_tied_projection_attention_of_the_library():
    """m0 is attention of image 0 over image 1 and m1 of image 1 over image 0,
    each with W_q = W_k = W_qk: torch's routine gives both."""
    rng = _rng(21)
    D, H, M, N = 32, 4, 7, 11
    st = _stage(rng, D)
    x0, x1 = rng.standard_normal((M, D)), rng.standard_normal((N, D))
    m0, m1 = oracle.bidirectional_cross_attention(x0, x1, st, H)
    np.testing.assert_allclose(m0, _torch_mha(x0, x1, st, H, D), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(m1, _torch_mha(x1, x0, st, H, D), rtol=1e-11, atol=1e-12)


def test_one_head_brute_force():
    """One head, plain loops: the similarity matrix formed once; m0_i =
    sum_j softmax over j (row i) * v1_j; m1_j = sum_i softmax over i (column
    j) * v0_i; then the merge projection."""
    rng = _rng(22)
    D, M, N = 4, 3, 5
    st = _stage(rng, D, scale=0.7)
    x0, x1 = rng.standard_normal((M, D)), rng.standard_normal((N, D))
    proj = lambda W, b, x: [sum(W[o][c] * x[c] for c in range(D)) + b[o] for o in range(D)]
    qk0 = [proj(st["Wqk"], st["bqk"], x0[i]) for i in range(M)]
    qk1 = [proj(st["Wqk"], st["bqk"], x1[j]) for j in range(N)]
    v0 = [proj(st["Wv"], st["bv"], x0[i]) for i in range(M)]
    v1 = [proj(st["Wv"], st["bv"], x1[j]) for j in range(N)]
    sim = [[sum(qk0[i][c] * qk1[j][c] for c in range(D)) / math.sqrt(D) for j in range(N)] for i in range(M)]
    m0 = []
    for i in range(M):
        z = sum(math.exp(sim[i][j]) for j in range(N))
        m0.append([sum(math.exp(sim[i][j]) / z * v1[j][c] for j in range(N)) for c in range(D)])
    m1 = []
    for j in range(N):
        z = sum(math.exp(sim[i][j]) for i in range(M))
        m1.append([sum(math.exp(sim[i][j]) / z * v0[i][c] for i in range(M)) for c in range(D)])
    merge = lambda m: [proj(st["Wm"], st["bm"], r) for r in m]
    g0, g1 = oracle.bidirectional_cross_attention(x0, x1, st, 1)
    np.testing.assert_allclose(g0, merge(m0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g1, merge(m1), rtol=1e-12, atol=1e-12)


def test_swap_symmetry():
    rng = _rng(23)
    D, H = 16, 2
    st = _stage(rng, D)
    x0, x1 = rng.standard_normal((6, D)), rng.standard_normal((9, D))
    a0, a1 = oracle.bidirectional_cross_attention(x0, x1, st, H)
    b1, b0 = oracle.bidirectional_cross_attention(x1, x0, st, H)
    np.testing.assert_allclose(a0, b0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a1, b1, rtol=1e-12, atol=1e-13)


def test_constant_values_give_constant_messages():
    """W_v = 0: every attention weight row sums to one, so each message is
    W_m b_v + b_m whatever the similarity."""
    rng = _rng(24)
    D, H = 8, 2
    st = _stage(rng, D)
    st["Wv"] = np.zeros((D, D))
    x0, x1 = 5 * rng.standard_normal((4, D)), 5 * rng.standard_normal((7, D))
    m0, m1 = oracle.bidirectional_cross_attention(x0, x1, st, H)
    want = st["Wm"] @ st["bv"] + st["bm"]
    np.testing.assert_allclose(m0, np.tile(want, (4, 1)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(m1, np.tile(want, (7, 1)), rtol=1e-12, atol=1e-12)


def test_gnn_routes_bidirectional_cross_stages():
    """In the GNN, a cross stage with W_qk gives the same states as the
    standard stage with W_q = W_k = W_qk; the self stage is unchanged."""
    rng = _rng(25)
    D, H = 16, 4
    self_st = {**_stage(rng, D)}
    self_st = {"Wq": self_st["Wqk"], "bq": self_st["bqk"], "Wk": rng.standard_normal((D, D)) * 0.3,
               "bk": rng.standard_normal(D) * 0.3, **{k: v for k, v in self_st.items() if k not in ("Wqk", "bqk")}}
    cross_st = _stage(rng, D)
    tied = {"Wq": cross_st["Wqk"], "bq": cross_st["bqk"], "Wk": cross_st["Wqk"], "bk": cross_st["bqk"],
            **{k: v for k, v in cross_st.items() if k not in ("Wqk", "bqk")}}
    xA, xB = rng.standard_normal((5, D)), rng.standard_normal((8, D))
    got = oracle.attentional_gnn(xA, xB, [self_st, cross_st], H)
    want = oracle.attentional_gnn(xA, xB, [self_st, tied], H)
    np.testing.assert_allclose(got[0], want[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got[1], want[1], rtol=1e-11, atol=1e-12)


def test_generator_draws_shared_projection_for_cross_stages_only():
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = synth.make_weights(cfg, cross="bidirectional")
    assert w["cross"] == "bidirectional"
    for s, st in enumerate(w["stages"]):
        assert ("Wqk" in st) == (s % 2 == 1) and ("Wq" in st) == (s % 2 == 0)
    std = synth.make_weights(cfg)
    assert all("Wq" in st for st in std["stages"]) and std["cross"] == "standard"
