"""GPU parity of bidirectional cross-attention (section 2.3 of the LightGlue
review): the GNN with shared query/key projections in its cross stages
against the float64 oracle, per stage and end to end with both heads.

Tolerances as for the standard GNN: states within 1e-5 relative per row
(fp32) and 5e-3 (bf16) per few stages; end to end, descriptors within 1e-4
(fp32) / 2e-2 (bf16), log assignments within 1e-3 (fp32, zero biases), match
indices equal except near ties.
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
def _weights(cid, bias_on=False):
    return synth.make_weights(synth.CONFIGS[cid], bias_on=bias_on, cross="bidirectional")


@pytest.mark.parametrize("cid,M,N,stages,tol", [
    (0, 10, 12, (0, 4), 1e-5),      # D = 64: the shared projection ends at column 64
    (1, 512, 512, (0, 2), 1e-5),
    (1, 100, 77, (1, 3), 1e-5),     # a slice that starts at a cross stage
    (3, 2048, 1536, (0, 2), 1e-5),
    (2, 1024, 1024, (0, 2), 5e-3),
    (2, 300, 45, (3, 5), 5e-3),
    (2, 33, 1, (0, 3), 5e-3),
    (2, 68, 2000, (5, 8), 5e-3),
])
def test_gnn_stage_parity(cid, M, N, stages, tol):
    cfg = synth.CONFIGS[cid]
    w = _weights(cid, bias_on=True)
    W = sg.pack_weights(w)
    xA = synth.random_states(M, cfg.D, seed=30 + cid)
    xB = synth.random_states(N, cfg.D, seed=40 + cid)
    a, b = dev(xA), dev(xB)
    sg.sg_stage_gnn(a, b, W, *stages)
    A, B = oracle.attentional_gnn(xA, xB, w["stages"][stages[0]:stages[1]], cfg.H, first_stage=stages[0])
    ea, eb = rel_rows(host(a), A), rel_rows(host(b), B)
    print(f"cfg{cid} {M}x{N} stages {stages}: max rel err A {ea.max():.2e} B {eb.max():.2e}")
    assert ea.max() < tol and eb.max() < tol


def _run(pair, W, cfg):
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")
    img = (*pair["image_size0"], *pair["image_size1"])
    out = sg.sg_match(*[dev(pair[k]) for k in keys], W, cfg.L, cfg.T, image_size=img, want_logP=True,
                      want_desc=True)
    torch.cuda.synchronize()
    return {k: host(v) if isinstance(v, torch.Tensor) else v for k, v in out.items()}


@pytest.mark.parametrize("head", ["sinkhorn", "ds"])
@pytest.mark.parametrize("cid", [0, 1])
def test_end_to_end_fp32(cid, head):
    cfg = synth.CONFIGS[cid]
    w = _weights(cid)
    pair = synth.make_pair(cfg)
    ref = oracle.double_softmax_match(pair, w) if head == "ds" else oracle.superglue_match(pair, w, T=cfg.T)
    g = _run(pair, sg.pack_weights(w, head=head), cfg)
    e = max(rel_rows(g["f0"], ref["f0"]).max(), rel_rows(g["f1"], ref["f1"]).max())
    dl = np.abs(g["logP"] - ref["logP"]).max()
    ex = check_matches(g["matches0"], g["matches1"], ref["logP"], ref["matches0"], ref["matches1"])
    print(f"cfg{cid} {head}: f rel err {e:.2e}, |dlogP| {dl:.2e}, matches {int((ref['matches0'] >= 0).sum())}, "
          f"exempt {ex}")
    assert e < 1e-4 and dl < 1e-3


def test_end_to_end_bf16_descriptors():
    cfg = synth.CONFIGS[2]
    w = _weights(2)
    pair = synth.make_pair(cfg)
    ref = oracle.superglue_descriptors(pair, w)
    g = _run(pair, sg.pack_weights(w), cfg)
    e = max(rel_rows(g["f0"], ref["f0"]).max(), rel_rows(g["f1"], ref["f1"]).max())
    print(f"cfg2 bidirectional: f rel err {e:.2e}")
    assert e < 2e-2


def test_variant_changes_only_cross_stages():
    """With W_qk = W_q = W_k of a standard network, the bidirectional blob
    gives the standard network's descriptors (same kernels, tied columns)."""
    cfg = synth.CONFIGS[0]
    std = synth.make_weights(cfg, bias_on=True)
    for s in range(1, len(std["stages"]), 2):
        std["stages"][s]["Wk"] = std["stages"][s]["Wq"].copy()
        std["stages"][s]["bk"] = std["stages"][s]["bq"].copy()
    bid = dict(std, cross="bidirectional", stages=[dict(st) for st in std["stages"]])
    for s in range(1, len(bid["stages"]), 2):
        st = bid["stages"][s]
        st["Wqk"], st["bqk"] = st.pop("Wq"), st.pop("bq")
        del st["Wk"], st["bk"]
    pair = synth.make_pair(cfg)
    a = _run(pair, sg.pack_weights(std), cfg)
    b = _run(pair, sg.pack_weights(bid), cfg)
    assert np.array_equal(a["f0"], b["f0"]) and np.array_equal(a["f1"], b["f1"])


def test_batch_matches_single_pairs():
    """The ragged bf16 batch with bidirectional cross stages: sampled pairs
    agree with sg_match on the unpadded pair to the bf16 descriptor bar."""
    cfg = synth.CONFIGS[4]
    w = _weights(4)
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
    print(f"bidirectional batch vs single: f rel diff {worst:.2e}, match agreement {np.mean(agree):.3f}")
    assert worst < 2e-2 and np.mean(agree) > 0.9
