"""GPU parity of rotary position encoding in self-attention (section 2.2 of
the LightGlue review) against the float64 oracle: GNN stage slices with
positions, the whole pass with both heads and with bidirectional cross
stages, and the translation invariance the encoding is built for.

Tolerances as for the GNN without it: states within 1e-5 relative per row
(fp32) / 5e-3 (bf16) per few stages; end to end, descriptors 1e-4 (fp32) /
2e-2 (bf16), log assignments 1e-3 (fp32, zero biases), matches equal except
near ties.
"""
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


@functools.lru_cache(maxsize=None)
def _weights(wl, bias_on=False, cross="standard"):
    return synth.make_weights(synth.WORKLOADS[wl], bias_on=bias_on, cross=cross, rope=True)


@pytest.mark.parametrize("wl,M,N,stages,tol", [
    ("pair10x12_f32", 10, 12, (0, 4), 1e-5),  # d_h = 16: four rotary pairs per head
    ("pair512_f32", 512, 512, (0, 2), 1e-5),
    ("pair512_f32", 100, 77, (1, 4), 1e-5),  # starts at a cross stage
    ("pair2048x1536_f32", 2048, 1536, (0, 1), 1e-5),
    ("pair1024_bf16", 1024, 1024, (0, 2), 5e-3),
    ("pair1024_bf16", 33, 1, (0, 3), 5e-3),
    ("pair1024_bf16", 68, 2000, (6, 9), 5e-3),
])
def test_gnn_stage_parity(wl, M, N, stages, tol):
    cfg = synth.WORKLOADS[wl]
    w = _weights(wl, bias_on=True)
    W = sg.pack_weights(w)
    pair = synth.make_pair(cfg, M=M, N=N, seed=50 + cfg.seed_id)
    xA = synth.random_states(M, cfg.D, seed=60 + cfg.seed_id)
    xB = synth.random_states(N, cfg.D, seed=70 + cfg.seed_id)
    a, b = dev(xA), dev(xB)
    img = (*pair["image_size0"], *pair["image_size1"])
    sg.sg_stage_gnn(a, b, W, *stages, posA=dev(pair["kpts0"]), posB=dev(pair["kpts1"]), image_size=img)
    th = tuple(oracle.rope_angles(oracle.normalize_keypoints(pair["kpts" + s], *pair["image_size" + s]),
                                  w["rope_basis"]) for s in ("0", "1"))
    A, B = oracle.attentional_gnn(xA, xB, w["stages"][stages[0]:stages[1]], cfg.H, first_stage=stages[0], rope=th)
    ea, eb = rel_rows(host(a), A), rel_rows(host(b), B)
    print(f"{wl} {M}x{N} stages {stages}: max rel err A {ea.max():.2e} B {eb.max():.2e}")
    assert ea.max() < tol and eb.max() < tol


def test_positions_already_normalised():
    """Without an image size the positions are taken as normalised."""
    cfg = synth.WORKLOADS["pair512_f32"]
    w = _weights("pair512_f32")
    W = sg.pack_weights(w)
    pair = synth.make_pair(cfg, M=200, N=150, seed=9)
    pA = oracle.normalize_keypoints(pair["kpts0"], *pair["image_size0"]).astype(np.float32)
    pB = oracle.normalize_keypoints(pair["kpts1"], *pair["image_size1"]).astype(np.float32)
    xA, xB = synth.random_states(200, cfg.D, seed=1), synth.random_states(150, cfg.D, seed=2)
    a, b = dev(xA), dev(xB)
    sg.sg_stage_gnn(a, b, W, 0, 2, posA=dev(pA), posB=dev(pB))
    th = (oracle.rope_angles(pA, w["rope_basis"]), oracle.rope_angles(pB, w["rope_basis"]))
    A, B = oracle.attentional_gnn(xA, xB, w["stages"][:2], cfg.H, rope=th)
    assert rel_rows(host(a), A).max() < 1e-5 and rel_rows(host(b), B).max() < 1e-5


def _run(pair, W, cfg):
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")
    img = (*pair["image_size0"], *pair["image_size1"])
    out = sg.sg_match(*[dev(pair[k]) for k in keys], W, cfg.L, cfg.T, image_size=img, want_logP=True,
                      want_desc=True)
    torch.cuda.synchronize()
    return {k: host(v) if isinstance(v, torch.Tensor) else v for k, v in out.items()}


@pytest.mark.parametrize("wl,head,cross", [
    ("pair10x12_f32", "sinkhorn", "standard"),
    ("pair512_f32", "sinkhorn", "standard"),
    ("pair512_f32", "ds", "standard"),
    ("pair512_f32", "ds", "bidirectional"),
])
def test_end_to_end_fp32(wl, head, cross):
    cfg = synth.WORKLOADS[wl]
    w = _weights(wl, cross=cross)
    pair = synth.make_pair(cfg)
    ref = oracle.double_softmax_match(pair, w) if head == "ds" else oracle.superglue_match(pair, w, T=cfg.T)
    g = _run(pair, sg.pack_weights(w, head=head), cfg)
    e = max(rel_rows(g["f0"], ref["f0"]).max(), rel_rows(g["f1"], ref["f1"]).max())
    dl = np.abs(g["logP"] - ref["logP"]).max()
    ex = check_matches(g["matches0"], g["matches1"], ref["logP"], ref["matches0"], ref["matches1"])
    print(f"{wl} {head} {cross}: f rel err {e:.2e}, |dlogP| {dl:.2e}, exempt {ex}")
    assert e < 1e-4 and dl < 1e-3


def test_end_to_end_bf16_descriptors():
    cfg = synth.WORKLOADS["pair1024_bf16"]
    w = _weights("pair1024_bf16")
    pair = synth.make_pair(cfg)
    ref = oracle.superglue_descriptors(pair, w)
    g = _run(pair, sg.pack_weights(w), cfg)
    e = max(rel_rows(g["f0"], ref["f0"]).max(), rel_rows(g["f1"], ref["f1"]).max())
    print(f"pair1024_bf16 rope: f rel err {e:.2e}")
    assert e < 2e-2


def test_translation_invariance_on_the_gpu():
    """Encoder weights zero: shifting image A's keypoints by a pixel vector
    leaves the descriptors unchanged up to fp32 rounding of the angles; the
    rotary encoding does act (a zero basis changes them)."""
    cfg = synth.WORKLOADS["pair512_f32"]
    w = dict(_weights("pair512_f32", bias_on=True))
    w["enc"] = [(0 * W_, 0 * b) for W_, b in w["enc"]]
    pair = synth.make_pair(cfg)
    shifted = dict(pair, kpts0=pair["kpts0"] + np.array([21.0, -9.0], np.float32))
    W = sg.pack_weights(w)
    a, b = _run(pair, W, cfg), _run(shifted, W, cfg)
    d = rel_rows(a["f0"], b["f0"]).max()
    c = _run(pair, sg.pack_weights(dict(w, rope_basis=np.zeros_like(w["rope_basis"]))), cfg)
    print(f"shift: f0 rel change {d:.2e}; zero basis: {rel_rows(a['f0'], c['f0']).max():.2e}")
    assert d < 1e-4
    assert rel_rows(a["f0"], c["f0"]).max() > 1e-3


def test_batch_matches_single_pairs():
    cfg = synth.WORKLOADS["ragged32_bf16"]
    w = _weights("ragged32_bf16")
    W = sg.pack_weights(w)
    b = synth.make_batch(cfg, batch=12)
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")
    img = (*b["image_size0"], *b["image_size1"])
    out = sg.sg_match_batch(b["M"], b["N"], *[dev(b[k]) for k in keys], W, cfg.L, cfg.T, image_size=img,
                            want_desc=True)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items() if isinstance(v, torch.Tensor)}
    worst, agree = 0.0, []
    for i in range(0, 12, 4):
        M, N = int(b["M"][i]), int(b["N"][i])
        s = _run(b["pairs"][i], W, cfg)
        worst = max(worst, rel_rows(g["f0"][i, :M], s["f0"]).max(), rel_rows(g["f1"][i, :N], s["f1"]).max())
        agree.append((g["matches0"][i, :M] == s["matches0"]).mean())
    print(f"rope batch vs single: f rel diff {worst:.2e}, match agreement {np.mean(agree):.3f}")
    assert worst < 2e-2 and np.mean(agree) > 0.9
