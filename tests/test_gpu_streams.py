"""Concurrent calls on several streams (GPU).

A server handling independent requests may keep several calls in flight,
one per stream, each with its own workspace and outputs; the library then
captures and replays one graph per (stream buffers) key.  These tests put
single-pair calls of the 1024 x 1024 bf16 pair, and a batched call beside
them, on four streams at once, over the eager first call, the capturing
second and the replayed later ones, and require every output to be bitwise
equal to the same call made alone on the current stream.  The lone call's
parity against the oracle is covered by the end-to-end tests.
"""
import pytest
import torch

import synth
from parity import dev

pytestmark = pytest.mark.gpu

sg = pytest.importorskip("learned_sparse_feature_amd")

KEYS = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sg.lib()


def _outputs(M, device):
    return {"matches0": torch.empty(M, dtype=torch.int32, device=device),
            "scores0": torch.empty(M, dtype=torch.float32, device=device)}


@pytest.mark.parametrize("wl", ["pair1024_bf16", "pair512_f32"])
def test_single_pair_calls_on_four_streams(wl):
    cfg = synth.WORKLOADS[wl]
    W = sg.pack_weights(synth.make_weights(cfg))
    pair = synth.make_pair(cfg)
    t = [dev(pair[k]) for k in KEYS]
    img = (*pair["image_size0"], *pair["image_size1"])
    device = t[0].device
    ref = sg.sg_match(*t, W, cfg.L, cfg.T, image_size=img, graph=False)
    torch.cuda.synchronize()
    S = 4
    streams = [torch.cuda.Stream(device=device) for _ in range(S)]
    wss = [torch.empty(sg.workspace_size(W, cfg.M, cfg.N, 1), dtype=torch.uint8, device=device) for _ in range(S)]
    outs = [_outputs(cfg.M, device) for _ in range(S)]
    for rnd in range(4):  # eager, capture, replays
        for i in range(S):
            for v in outs[i].values():
                v.fill_(-7)  # on the current stream, ordered before the call by the synchronisation below
        torch.cuda.synchronize()
        for i in range(S):
            sg.sg_match(*t, W, cfg.L, cfg.T, image_size=img, workspace=wss[i], out=outs[i], stream=streams[i])
        torch.cuda.synchronize()
        for i in range(S):
            assert torch.equal(outs[i]["matches0"], ref["matches0"]), (wl, rnd, i)
            assert torch.equal(outs[i]["scores0"], ref["scores0"]), (wl, rnd, i)
    print(f"{wl}: {int((ref['matches0'] >= 0).sum())} matches, equal on {S} streams over 4 rounds")


def test_batch_beside_single_pairs():
    """A ragged batched call on one stream while single-pair calls run on
    three others: each equals its lone call."""
    cfg1 = synth.WORKLOADS["pair1024_bf16"]
    W = sg.pack_weights(synth.make_weights(cfg1))
    pair = synth.make_pair(cfg1)
    t = [dev(pair[k]) for k in KEYS]
    img = (*pair["image_size0"], *pair["image_size1"])
    device = t[0].device
    cfgb = synth.WORKLOADS["ragged32_bf16"]
    b = synth.make_batch(cfgb)
    tb = [torch.from_numpy(b[k]).to(device) for k in KEYS]
    imgb = (*b["image_size0"], *b["image_size1"])
    Ms, Ns = [int(x) for x in b["M"]], [int(x) for x in b["N"]]
    ref1 = sg.sg_match(*t, W, cfg1.L, cfg1.T, image_size=img, graph=False)
    refb = sg.sg_match_batch(Ms, Ns, *tb, W, cfgb.L, cfgb.T, image_size=imgb, want_matches1=False, graph=False)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=device) for _ in range(4)]
    wsb = torch.empty(sg.workspace_size(W, cfgb.pad, cfgb.pad, cfgb.batch), dtype=torch.uint8, device=device)
    outb = {"matches0": torch.empty((cfgb.batch, cfgb.pad), dtype=torch.int32, device=device),
            "scores0": torch.empty((cfgb.batch, cfgb.pad), dtype=torch.float32, device=device)}
    wss = [torch.empty(sg.workspace_size(W, cfg1.M, cfg1.N, 1), dtype=torch.uint8, device=device) for _ in range(3)]
    outs = [_outputs(cfg1.M, device) for _ in range(3)]
    for rnd in range(3):
        sg.sg_match_batch(Ms, Ns, *tb, W, cfgb.L, cfgb.T, image_size=imgb, workspace=wsb, want_matches1=False,
                          out=outb, stream=streams[0])
        for k in range(2):
            for i in range(3):
                sg.sg_match(*t, W, cfg1.L, cfg1.T, image_size=img, workspace=wss[i], out=outs[i],
                            stream=streams[1 + i])
        torch.cuda.synchronize()
        assert torch.equal(outb["matches0"], refb["matches0"]), rnd
        assert torch.equal(outb["scores0"], refb["scores0"]), rnd
        for i in range(3):
            assert torch.equal(outs[i]["matches0"], ref1["matches0"]), (rnd, i)
            assert torch.equal(outs[i]["scores0"], ref1["scores0"]), (rnd, i)
