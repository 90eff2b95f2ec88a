"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side validation rejects bad arguments before touching the GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from learned_sparse_feature_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(sg_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared()
    assert {"sg_match", "sg_match_batch", "sg_stage_match", "sg_last_error"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"


def _cfg(D=256, H=4, enc=(32, 64, 128, 256), L=9, dtype=_lib.SG_F32, blob=None, nbytes=0):
    w = _lib.SgWeights()
    w.D, w.H, w.n_enc, w.L_max, w.dtype = D, H, len(enc), L, dtype
    for i, e in enumerate(enc):
        w.enc[i] = e
    w.blob, w.blob_bytes = blob, nbytes
    return w


def test_weight_layout_parameter_count():
    """The layout holds 12,003,905 parameters at D=256, L=9 (encoder 109,376;
    18 stages of 657,152; final projection 65,792; the dustbin score)."""
    lib = _lib.load()
    w = _cfg()
    n = lib.sg_weights_count(C.byref(w))
    total = 0
    off, r, c = C.c_size_t(), C.c_int32(), C.c_int32()
    last_end = 0
    for i in range(n):
        assert lib.sg_weights_tensor(C.byref(w), i, C.byref(off), C.byref(r), C.byref(c)) == 0
        assert off.value % 256 == 0 and off.value >= last_end
        last_end = off.value + r.value * c.value * 4
        total += r.value * c.value
    assert total == 12_003_905
    assert lib.sg_weights_bytes(C.byref(w)) >= last_end
    wb = _cfg(dtype=_lib.SG_BF16)
    assert lib.sg_weights_bytes(C.byref(wb)) < lib.sg_weights_bytes(C.byref(w))


def test_config_validation():
    lib = _lib.load()
    assert lib.sg_weights_count(C.byref(_cfg(D=250))) == -1          # D % H
    assert lib.sg_weights_bytes(C.byref(_cfg(D=96, H=2))) == 0       # head dim 48 unsupported
    assert lib.sg_workspace_size(C.byref(_cfg()), 1024, 1024, 1) > 0
    assert lib.sg_workspace_size(C.byref(_cfg()), -1, 10, 1) == 0


def _match(lib, w, M=8, N=8, L=1, T=5, fake=0x1000, opts=None):
    p = C.c_void_p(fake)
    return lib.sg_match(p, p, p, M, p, p, p, N, C.byref(w), L, T, p, p, opts)


def test_match_rejects_bad_arguments_on_host():
    lib = _lib.load()
    fake = C.c_void_p(0x1000)
    good = _cfg(blob=fake, nbytes=1 << 30)
    assert _match(lib, _cfg(blob=None, nbytes=1 << 30)) == _lib.SG_ERR_INVALID_ARG
    assert _match(lib, _cfg(blob=fake, nbytes=1000)) == _lib.SG_ERR_WEIGHTS
    assert "weight blob" in lib.sg_last_error().decode()
    assert _match(lib, good, L=0) == _lib.SG_ERR_INVALID_ARG
    assert _match(lib, good, L=10) == _lib.SG_ERR_INVALID_ARG
    assert _match(lib, good, T=-1) == _lib.SG_ERR_INVALID_ARG
    assert _match(lib, good, M=-3) == _lib.SG_ERR_INVALID_ARG
    assert _match(lib, good, M=5000) == _lib.SG_ERR_UNSUPPORTED
    assert _match(lib, _cfg(D=96, H=2, blob=fake, nbytes=1 << 30)) == _lib.SG_ERR_UNSUPPORTED
    o = _lib.SgOpts()
    o.workspace, o.workspace_bytes = 0x2000, 16
    assert _match(lib, good, opts=C.byref(o)) == _lib.SG_ERR_WORKSPACE
    o = _lib.SgOpts()
    o.out_logP, o.logP_ld = 0x3000, 4
    assert _match(lib, good, opts=C.byref(o)) == _lib.SG_ERR_INVALID_ARG


def test_batch_rejects_bad_arguments_on_host():
    lib = _lib.load()
    fake = C.c_void_p(0x1000)
    good = _cfg(blob=fake, nbytes=1 << 30)
    Ms = (C.c_int32 * 2)(5, 9)
    Ns = (C.c_int32 * 2)(5, 5)
    args = [fake] * 6
    st = lib.sg_match_batch(2, 8, 8, Ms, Ns, *args, C.byref(good), 1, 5, fake, fake, None)
    assert st == _lib.SG_ERR_INVALID_ARG and "outside" in lib.sg_last_error().decode()
    st = lib.sg_match_batch(0, 8, 8, Ms, Ns, *args, C.byref(good), 1, 5, fake, fake, None)
    assert st == _lib.SG_ERR_INVALID_ARG
    st = lib.sg_match_batch(_lib.SG_MAX_BATCH + 1, 8, 8, Ms, Ns, *args, C.byref(good), 1, 5, fake, fake, None)
    assert st == _lib.SG_ERR_INVALID_ARG


def test_stage_entry_points_validate_on_host():
    lib = _lib.load()
    fake = C.c_void_p(0x1000)
    good = _cfg(blob=fake, nbytes=1 << 30)
    assert lib.sg_stage_gnn(fake, 4, fake, 4, C.byref(good), 3, 1, None) == _lib.SG_ERR_INVALID_ARG
    assert lib.sg_stage_gnn(fake, 4, fake, 4, C.byref(good), 0, 19, None) == _lib.SG_ERR_INVALID_ARG
    assert lib.sg_stage_match(fake, 4, fake, 4, 12, 1.0, 5, fake, fake, None) == _lib.SG_ERR_UNSUPPORTED
    assert lib.sg_stage_match(fake, 4, fake, 4, 64, 1.0, -1, fake, fake, None) == _lib.SG_ERR_INVALID_ARG
    assert lib.sg_stage_encode(fake, fake, fake, -1, 0.0, 0.0, C.byref(good), fake, None) == _lib.SG_ERR_INVALID_ARG
    assert lib.sg_stage_match_workspace_size(1024, 1024, 256) > 1024 * 1024 * 8


def test_double_softmax_head_layout_and_validation():
    """The double-softmax head appends the matchability Linear(D, 1) (D + 1
    parameters) after alpha; an unknown head is rejected; the stage entry
    point validates on the host; its workspace holds the full transpose."""
    lib = _lib.load()
    w = _cfg()
    wd = _cfg()
    wd.head = _lib.SG_HEAD_DOUBLE_SOFTMAX
    n, nd = lib.sg_weights_count(C.byref(w)), lib.sg_weights_count(C.byref(wd))
    assert nd == n + 2
    off, r, c = C.c_size_t(), C.c_int32(), C.c_int32()
    shapes = []
    for i in (n, n + 1):
        assert lib.sg_weights_tensor(C.byref(wd), i, C.byref(off), C.byref(r), C.byref(c)) == 0
        shapes.append((r.value, c.value))
    assert shapes == [(1, 256), (1, 1)]
    assert lib.sg_weights_bytes(C.byref(wd)) > lib.sg_weights_bytes(C.byref(w))
    bad = _cfg()
    bad.head = 7
    assert lib.sg_weights_count(C.byref(bad)) == -1
    fake = C.c_void_p(0x1000)
    bad.blob, bad.blob_bytes = fake, 1 << 30
    assert _match(lib, bad) == _lib.SG_ERR_INVALID_ARG and "head" in lib.sg_last_error().decode()
    f = fake
    assert lib.sg_stage_match_ds(f, f, 4, f, f, 4, 12, f, 0.0, f, f, None) == _lib.SG_ERR_UNSUPPORTED
    assert lib.sg_stage_match_ds(f, f, -1, f, f, 4, 64, f, 0.0, f, f, None) == _lib.SG_ERR_INVALID_ARG
    assert lib.sg_stage_match_ds(f, None, 4, f, f, 4, 64, f, 0.0, f, f, None) == _lib.SG_ERR_INVALID_ARG
    assert lib.sg_stage_match_ds(f, f, 4, f, f, 4, 64, None, 0.0, f, f, None) == _lib.SG_ERR_INVALID_ARG
    # Z and its full transpose at any size (the Sinkhorn workspace caps the transpose)
    big = lib.sg_stage_match_ds_workspace_size(4096, 4096, 256)
    assert 2 * 4096 * 4096 * 4 < big < 4 * 4096 * 4096 * 4
    assert lib.sg_workspace_size(C.byref(wd), 4096, 4096, 8) > 2 * 8 * 4096 * 4096 * 4


def test_bidirectional_cross_layout_and_validation():
    """Bidirectional cross stages store W_qk | W_v ([2D][D]) and their bias
    [2D]: D^2 + D fewer parameters per cross stage; an unknown variant is
    rejected."""
    lib = _lib.load()
    w, wb = _cfg(), _cfg()
    wb.cross = _lib.SG_CROSS_BIDIRECTIONAL
    assert lib.sg_weights_count(C.byref(wb)) == lib.sg_weights_count(C.byref(w))

    def params(cfg):
        off, r, c = C.c_size_t(), C.c_int32(), C.c_int32()
        total = 0
        for i in range(lib.sg_weights_count(C.byref(cfg))):
            assert lib.sg_weights_tensor(C.byref(cfg), i, C.byref(off), C.byref(r), C.byref(c)) == 0
            total += r.value * c.value
        return total
    assert params(w) - params(wb) == 9 * (256 * 256 + 256)
    bad = _cfg()
    bad.cross = 2
    assert lib.sg_weights_count(C.byref(bad)) == -1


def test_shared_similarity_validation_and_workspace():
    """SG_FLAG_SHARED_SIMILARITY: refused without bidirectional weights, with
    the adaptive flags and in batches (host validation, before any HIP
    call); a single pair's workspace holds every head's similarity, its
    transpose and both rows' log-sum-exp."""
    lib = _lib.load()
    fake = C.c_void_p(0x1000)
    plain = _cfg(blob=fake, nbytes=1 << 30)
    wb = _cfg(blob=fake, nbytes=1 << 30)
    wb.cross = _lib.SG_CROSS_BIDIRECTIONAL
    o = _lib.SgOpts()
    o.flags = _lib.SG_FLAG_SHARED_SIMILARITY
    assert _match(lib, plain, opts=C.byref(o)) == _lib.SG_ERR_INVALID_ARG
    assert "bidirectional" in lib.sg_last_error().decode()
    o.flags = _lib.SG_FLAG_SHARED_SIMILARITY | _lib.SG_FLAG_EARLY_EXIT
    assert _match(lib, wb, opts=C.byref(o)) == _lib.SG_ERR_UNSUPPORTED
    o.flags = _lib.SG_FLAG_SHARED_SIMILARITY
    Ms = (C.c_int32 * 1)(8)
    st = lib.sg_match_batch(1, 8, 8, Ms, Ms, *([fake] * 6), C.byref(wb), 1, 5, fake, fake, C.byref(o))
    assert st == _lib.SG_ERR_UNSUPPORTED
    M, N, H = 1000, 777, 4
    ld4 = lambda n: (n + 3) // 4 * 4
    extra = 4 * H * (M * ld4(N) + N * ld4(M) + M + N)
    d1 = lib.sg_workspace_size(C.byref(wb), M, N, 1) - lib.sg_workspace_size(C.byref(plain), M, N, 1)
    assert extra <= d1 < extra + 1024
    assert lib.sg_workspace_size(C.byref(wb), M, N, 2) == lib.sg_workspace_size(C.byref(plain), M, N, 2)


def test_rope_layout_and_validation():
    """Rotary weights append one fp32 [d_h/2][2] basis; the GNN stage entry
    point refuses them without positions (host validation, before any HIP
    call)."""
    lib = _lib.load()
    w, wr = _cfg(), _cfg()
    wr.rope = 1
    n = lib.sg_weights_count(C.byref(w))
    assert lib.sg_weights_count(C.byref(wr)) == n + 1
    off, r, c = C.c_size_t(), C.c_int32(), C.c_int32()
    assert lib.sg_weights_tensor(C.byref(wr), n, C.byref(off), C.byref(r), C.byref(c)) == 0
    assert (r.value, c.value) == (32, 2)
    bad = _cfg()
    bad.rope = 3
    assert lib.sg_weights_count(C.byref(bad)) == -1
    fake = C.c_void_p(0x1000)
    wr.blob, wr.blob_bytes = fake, 1 << 30
    assert lib.sg_stage_gnn(fake, 4, fake, 4, C.byref(wr), 0, 2, None) == _lib.SG_ERR_INVALID_ARG
    assert "positions" in lib.sg_last_error().decode()


def test_adaptive_layout_and_validation():
    """Adaptive weights append, per layer but the last, the confidence and
    the layer's head (6 tensors); they need the double-softmax head; the
    batch entry point refuses adaptive calls; bad adaptive options are
    rejected on the host."""
    lib = _lib.load()
    w = _cfg()
    w.head = _lib.SG_HEAD_DOUBLE_SOFTMAX
    wa = _cfg()
    wa.head, wa.adaptive = _lib.SG_HEAD_DOUBLE_SOFTMAX, 1
    assert lib.sg_weights_count(C.byref(wa)) == lib.sg_weights_count(C.byref(w)) + 6 * 8
    bad = _cfg()
    bad.adaptive = 1
    assert lib.sg_weights_count(C.byref(bad)) == -1
    fake = C.c_void_p(0x1000)
    wa.blob, wa.blob_bytes = fake, 1 << 30
    o = _lib.SgOpts()
    o.flags = _lib.SG_FLAG_EARLY_EXIT
    Ms = (C.c_int32 * 1)(8)
    st = lib.sg_match_batch(1, 8, 8, Ms, Ms, *([fake] * 6), C.byref(wa), 1, 5, fake, fake, C.byref(o))
    assert st == _lib.SG_ERR_UNSUPPORTED
    o.width_confidence = 1.5
    assert _match(lib, wa, opts=C.byref(o)) == _lib.SG_ERR_INVALID_ARG
    plain = _cfg(blob=fake, nbytes=1 << 30)
    o2 = _lib.SgOpts()
    o2.flags = _lib.SG_FLAG_PRUNE
    assert _match(lib, plain, opts=C.byref(o2)) == _lib.SG_ERR_INVALID_ARG


def test_sinkhorn_and_extract_stages_validate_on_host():
    """sg_stage_sinkhorn / sg_stage_extract refuse bad arguments before any
    HIP call, with nothing enqueued."""
    lib = _lib.load()
    f = C.c_void_p(0x1000)
    I = _lib.SG_ERR_INVALID_ARG
    # empty images: the optimal-matching layer runs on non-empty images only
    assert lib.sg_stage_sinkhorn(f, 5, 0, 4, 10, f, f, None, 0, None) == I
    assert "non-empty" in lib.sg_last_error().decode()
    assert lib.sg_stage_sinkhorn(f, 5, 3, 0, 10, f, f, None, 0, None) == I
    assert lib.sg_stage_sinkhorn(f, 5, 3, 4, -1, f, f, None, 0, None) == I          # T < 0
    assert lib.sg_stage_sinkhorn(f, 4, 3, 4, 10, f, f, None, 0, None) == I          # ldZ < N+1
    assert lib.sg_stage_sinkhorn(None, 5, 3, 4, 10, f, f, None, 0, None) == I
    assert lib.sg_stage_sinkhorn(f, 5, 3, 4, 10, None, f, None, 0, None) == I       # u NULL
    assert lib.sg_stage_sinkhorn(f, 5, 3, 4, 10, f, None, None, 0, None) == I       # v NULL
    assert lib.sg_stage_sinkhorn(f, 5, 3, 4, 10, f, f, f, 4, None) == I             # ldP < N+1
    assert lib.sg_stage_sinkhorn(f, 5000, 4097, 4, 10, f, f, None, 0, None) == _lib.SG_ERR_UNSUPPORTED
    assert lib.sg_stage_extract(f, 4, 3, 4, 0.0, f, f, None, None, None) == I        # ldP < N+1
    assert lib.sg_stage_extract(None, 5, 3, 4, 0.0, f, f, None, None, None) == I
    assert lib.sg_stage_extract(f, 5, 3, 4, 0.0, None, f, None, None, None) == I
    assert lib.sg_stage_extract(f, 5, 3, 4, 0.0, f, f, None, f, None) == I           # scores1 without matches1
    assert lib.sg_stage_extract(f, 5, -1, 4, 0.0, f, f, None, None, None) == I
    assert lib.sg_stage_extract(f, 5, 3, 4097, 0.0, f, f, None, None, None) == _lib.SG_ERR_UNSUPPORTED
    # the workspace holds Z, its transpose and the per-line vectors
    assert lib.sg_stage_sinkhorn_workspace_size(1024, 1024) >= 2 * 1024 * 1024 * 4
    assert lib.sg_stage_sinkhorn_workspace_size(-1, 3) == 0


def test_scores_stage_validates_on_host():
    """sg_stage_scores refuses bad arguments before any HIP call."""
    lib = _lib.load()
    w0 = _cfg()
    w = _cfg(blob=C.c_void_p(0x1000), nbytes=lib.sg_weights_bytes(C.byref(w0)))
    f = C.c_void_p(0x1000)
    I = _lib.SG_ERR_INVALID_ARG
    assert lib.sg_stage_scores(f, -1, f, 4, C.byref(w), f, 5, None) == I
    assert lib.sg_stage_scores(f, 3, f, 4, C.byref(w), None, 5, None) == I          # Z NULL
    assert lib.sg_stage_scores(f, 3, f, 4, C.byref(w), f, 4, None) == I             # ldZ < N+1
    assert lib.sg_stage_scores(None, 3, f, 4, C.byref(w), f, 5, None) == I          # states NULL
    assert lib.sg_stage_scores(f, 3, f, 4097, C.byref(w), f, 4098, None) == _lib.SG_ERR_UNSUPPORTED
    assert lib.sg_stage_scores(f, 3, f, 4, C.byref(w0), f, 5, None) == I            # no blob
    # f_A, f_B and the unbordered scores
    assert lib.sg_stage_scores_workspace_size(1024, 1024, 256) >= (2 * 1024 * 256 + 1024 * 1024) * 4
    assert lib.sg_stage_scores_workspace_size(-1, 3, 256) == 0
