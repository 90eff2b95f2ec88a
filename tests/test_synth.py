"""The seeded generator: deterministic, shapes and planted counts as configured."""
import numpy as np

import synth


def test_generator_is_deterministic():
    c = synth.WORKLOADS["pair10x12_f32"]
    a, b = synth.make_pair(c), synth.make_pair(c)
    for k in ("kpts0", "desc1", "conf0"):
        np.testing.assert_array_equal(a[k], b[k])
    wa, wb = synth.make_weights(c), synth.make_weights(c)
    np.testing.assert_array_equal(wa["stages"][1]["W1"], wb["stages"][1]["W1"])


def test_bf16_weights_are_representable():
    w = synth.make_weights(synth.WORKLOADS["pair1024_bf16"], L=1)
    W = w["stages"][0]["Wq"]
    assert np.all(W.view(np.uint32) & 0xFFFF == 0)


def test_round_to_bf16_ties_to_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], dtype=np.float32)
    np.testing.assert_array_equal(synth.round_to_bf16(x), np.array([1.0, 1.0 + 2.0 ** -6, 1.0], np.float32))


def test_planted_counts_and_ranges():
    p2 = synth.make_pair(synth.WORKLOADS["pair1024_bf16"])
    assert p2["n_planted"] == 410
    p3 = synth.make_pair(synth.WORKLOADS["pair2048x1536_f32"])
    assert p3["n_planted"] == 614
    for p in (p2, p3):
        for s in ("0", "1"):
            k = p["kpts" + s]
            assert k[:, 0].min() >= 0 and k[:, 0].max() < 640 and k[:, 1].min() >= 0 and k[:, 1].max() < 480
            np.testing.assert_allclose(np.linalg.norm(p["desc" + s], axis=1), 1.0, rtol=1e-5)


def test_batch_shapes():
    b = synth.make_batch(synth.WORKLOADS["ragged32_bf16"], batch=4)
    assert b["kpts0"].shape == (4, 2048, 2) and b["desc1"].shape == (4, 2048, 256)
    for i in range(4):
        assert 256 <= b["M"][i] <= 2048 and 256 <= b["N"][i] <= 2048
        assert np.all(b["desc0"][i, b["M"][i]:] == 0)


def test_weight_shapes_and_bias_rules():
    c = synth.WORKLOADS["pair10x12_f32"]
    w = synth.make_weights(c, bias_on=True)
    assert [W.shape for W, _ in w["enc"]] == [(16, 3), (32, 16), (64, 32)]
    assert np.all(w["enc"][-1][1] == 0) and np.any(w["enc"][0][1] != 0)
    st = w["stages"][0]
    assert st["W1"].shape == (128, 128) and st["W2"].shape == (64, 128)
    assert np.all(st["b2"] == 0) and np.any(st["b1"] != 0)
    assert len(w["stages"]) == 2 * c.L
