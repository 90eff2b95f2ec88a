"""Pins of the oracle's rotary position encoding in self-attention
([LightGlue-review] section 2.2).  Chosen so that a plausible mistake fails:
a sign flip in the rotation, pairs taken across heads or as (k, k + d/2),
the value rotated, the encoding applied in cross stages, angles from the
wrong image, or a dependence on absolute instead of relative position.
"""
import cmath
import math

import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(autouse=True)
def _each_oracle(oracle_impl, monkeypatch):
    """Every pin runs against both oracle implementations (plain C, numpy)."""
    monkeypatch.setitem(globals(), "oracle", oracle_impl)



def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _stage(rng, D, scale=0.4):
    st = {}
    for name, n_out, n_in in (("q", D, D), ("k", D, D), ("v", D, D), ("m", D, D), ("1", 2 * D, 2 * D),
                              ("2", D, 2 * D)):
        st["W" + name] = scale * rng.standard_normal((n_out, n_in))
        st["b" + name] = scale * rng.standard_normal(n_out)
    return st


def test_rotation_as_complex_multiplication():
    """Channel pair (2k, 2k+1) of each head read as a + ib and multiplied by
    exp(i theta_k): plain loops with complex numbers, two heads."""
    rng = _rng(31)
    n, H, dh = 3, 2, 6
    t = rng.standard_normal((n, H * dh))
    theta = rng.uniform(-3, 3, size=(n, dh // 2))
    got = oracle.rotate_pairs(t, theta, H)
    for i in range(n):
        for h in range(H):
            for k in range(dh // 2):
                z = complex(t[i, h * dh + 2 * k], t[i, h * dh + 2 * k + 1]) * cmath.exp(1j * theta[i, k])
                assert abs(got[i, h * dh + 2 * k] - z.real) < 1e-13
                assert abs(got[i, h * dh + 2 * k + 1] - z.imag) < 1e-13


def test_angles_are_basis_projections():
    pos = np.array([[0.25, -0.5], [1.0, 2.0]])
    basis = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, -3.0]])
    np.testing.assert_allclose(oracle.rope_angles(pos, basis), [[0.25, -0.5, 2.0], [1.0, 2.0, -4.0]], atol=0)


def test_logits_depend_on_relative_position_only():
    """<R(theta_i) q, R(theta_j) k> = <q, R(theta_j - theta_i) k> per pair:
    each logit equals the unrotated query against the key rotated by the
    angle of p_j - p_i."""
    rng = _rng(32)
    H, dh = 2, 8
    q, k = rng.standard_normal((1, H * dh)), rng.standard_normal((1, H * dh))
    basis = rng.standard_normal((dh // 2, 2))
    pi, pj = rng.standard_normal((1, 2)), rng.standard_normal((1, 2))
    rq = oracle.rotate_pairs(q, oracle.rope_angles(pi, basis), H)
    rk = oracle.rotate_pairs(k, oracle.rope_angles(pj, basis), H)
    rel = oracle.rotate_pairs(k, oracle.rope_angles(pj - pi, basis), H)
    for h in range(H):
        c = slice(h * dh, (h + 1) * dh)
        assert abs(float(rq[0, c] @ rk[0, c]) - float(q[0, c] @ rel[0, c])) < 1e-12


def test_self_attention_is_translation_invariant():
    """Shifting every point of the image by one vector leaves the messages
    unchanged (only relative positions enter), while a non-uniform change of
    positions changes them."""
    rng = _rng(33)
    D, H, n = 16, 2, 9
    st = _stage(rng, D)
    x = rng.standard_normal((n, D))
    basis = 3.0 * rng.standard_normal((D // H // 2, 2))
    pos = rng.uniform(-1, 1, size=(n, 2))
    th = oracle.rope_angles(pos, basis)
    m = oracle.multi_head_attention(x, x, st, H, rope=(th, th))
    th2 = oracle.rope_angles(pos + np.array([0.37, -1.2]), basis)
    np.testing.assert_allclose(oracle.multi_head_attention(x, x, st, H, rope=(th2, th2)), m, rtol=1e-10, atol=1e-12)
    th3 = oracle.rope_angles(pos * 1.5, basis)
    assert np.abs(oracle.multi_head_attention(x, x, st, H, rope=(th3, th3)) - m).max() > 1e-3


def test_zero_basis_is_plain_attention_and_rotation_keeps_norms():
    rng = _rng(34)
    D, H = 16, 4
    st = _stage(rng, D)
    x = rng.standard_normal((7, D))
    th = oracle.rope_angles(rng.standard_normal((7, 2)), np.zeros((D // H // 2, 2)))
    np.testing.assert_allclose(oracle.multi_head_attention(x, x, st, H, rope=(th, th)),
                               oracle.multi_head_attention(x, x, st, H), rtol=1e-13, atol=1e-13)
    t = rng.standard_normal((5, D))
    r = oracle.rotate_pairs(t, rng.uniform(-7, 7, size=(5, D // H // 2)), H)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(t, axis=1), rtol=1e-13)


def test_values_are_not_rotated():
    """W_q = W_k = 0: every logit is zero whatever the rotation, so each
    message is the merge of the mean value; a rotated v would change it."""
    rng = _rng(35)
    D, H, n = 8, 2, 6
    st = _stage(rng, D)
    st["Wq"][:] = 0
    st["Wk"][:] = 0
    st["bq"][:] = 0
    st["bk"][:] = 0
    x = rng.standard_normal((n, D))
    th = oracle.rope_angles(rng.standard_normal((n, 2)), 5.0 * rng.standard_normal((D // H // 2, 2)))
    v = x @ st["Wv"].T + st["bv"]
    want = v.mean(axis=0) @ st["Wm"].T + st["bm"]
    np.testing.assert_allclose(oracle.multi_head_attention(x, x, st, H, rope=(th, th)), np.tile(want, (n, 1)),
                               rtol=1e-12, atol=1e-12)


def test_gnn_rotates_self_stages_only():
    """A slice holding only a cross stage is unchanged by the encoding; a self
    stage uses each image's own angles (exchanging the images' angles
    changes the result)."""
    rng = _rng(36)
    D, H = 16, 2
    xA, xB = rng.standard_normal((5, D)), rng.standard_normal((7, D))
    thA = oracle.rope_angles(rng.standard_normal((5, 2)), 2.0 * rng.standard_normal((D // H // 2, 2)))
    thB = oracle.rope_angles(rng.standard_normal((7, 2)), 2.0 * rng.standard_normal((D // H // 2, 2)))
    cross = [_stage(rng, D)]
    a = oracle.attentional_gnn(xA, xB, cross, H, first_stage=1, rope=(thA, thB))
    b = oracle.attentional_gnn(xA, xB, cross, H, first_stage=1)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=0)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=0)
    st = _stage(rng, D)
    got = oracle.attentional_gnn(xA, xB, [st], H, rope=(thA, thB))
    wantA = xA + oracle.attentional_propagation(xA, xA, st, H, rope=(thA, thA))
    np.testing.assert_allclose(got[0], wantA, rtol=1e-13, atol=1e-13)
    assert np.abs(got[0] - oracle.attentional_gnn(xA, xB, [st], H)[0]).max() > 1e-4


def test_full_pass_uses_normalised_positions():
    """The whole pass with a rotary basis takes its angles from the
    normalised keypoints: translating the keypoints of one image in pixels
    (same image size) leaves the self-stage messages unchanged, so with the
    keypoint encoder switched off (zero weights) the descriptors do not move."""
    cfg = synth.WORKLOADS["pair10x12_f32"]
    w = synth.make_weights(cfg, rope=True, L=1)
    assert w["rope_basis"].shape == (cfg.D // cfg.H // 2, 2)
    w["enc"] = [(0 * W, 0 * b) for W, b in w["enc"]]
    pair = synth.make_pair(cfg)
    shifted = dict(pair, kpts0=pair["kpts0"] + np.array([13.0, -7.0], np.float32))
    a = oracle.superglue_descriptors(pair, w)
    b = oracle.superglue_descriptors(shifted, w)
    np.testing.assert_allclose(a["f0"], b["f0"], rtol=1e-9, atol=1e-10)
    c = oracle.superglue_descriptors(pair, dict(w, rope_basis=None))
    assert np.abs(a["f0"] - c["f0"]).max() > 1e-4
