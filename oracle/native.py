"""The plain C oracle (oracle/sg_oracle.c) behind the functions of the numpy oracle.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the CPU-baseline leg of the benchmark use it.

Every arithmetic step runs in the C library: float64 loops in index order,
no BLAS (see the header of sg_oracle.c for the pages each routine follows).
This module only converts arguments to float64 arrays, calls the routines in
the pages' order, and does the adaptive pass's bookkeeping (which points
remain, when to stop).  The functions, arguments and results are those of
oracle.reference_numpy, which serves as an independent cross-check.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sg_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CC = os.environ.get("CC", "gcc")
# sums stay in index order: no fused multiply-add contraction, no fast math
CFLAGS = ["-O2", "-std=gnu99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall"]


def build(verbose: bool = False) -> str:
    """Compile sg_oracle.c into liboracle.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [CC, *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_P = C.c_void_p
_I64 = C.c_int64
_D = C.c_double
_INT = C.c_int

_SIGS = {
    "orc_set_threads": (None, [_INT]),
    "orc_threads": (_INT, []),
    "orc_linear": (None, [_P, _I64, _INT, _P, _P, _INT, _P]),
    "orc_normalize_keypoints": (None, [_P, _I64, _D, _D, _P]),
    "orc_keypoint_encoder": (None, [_P, _P, _I64, _INT, _P, _P, _P, _P]),
    "orc_rotate_pairs": (None, [_P, _I64, _INT, _INT, _P, _P]),
    "orc_rope_angles": (None, [_P, _I64, _P, _INT, _P]),
    "orc_multi_head_attention": (None, [_P, _I64, _P, _I64, _INT, _INT, _P, _P, _P, _P]),
    "orc_bidirectional_cross_attention": (None, [_P, _I64, _P, _I64, _INT, _INT, _P, _P, _P]),
    "orc_update_mlp": (None, [_P, _P, _I64, _INT, _P, _P]),
    "orc_attentional_gnn": (None, [_P, _I64, _P, _I64, _INT, _INT, _P, _INT, _INT, _P, _P]),
    "orc_score_matrix": (None, [_P, _I64, _P, _I64, _INT, _P]),
    "orc_log_sinkhorn_iterations": (None, [_P, _I64, _I64, _P, _P, _INT, _P, _P, _P]),
    "orc_log_optimal_transport": (None, [_P, _I64, _I64, _D, _INT, _P, _P, _P]),
    "orc_sinkhorn_knopp_exp": (None, [_P, _I64, _I64, _P, _P, _INT, _P]),
    "orc_extract_matches": (None, [_P, _I64, _I64, _D, _P, _P, _P, _P]),
    "orc_log_sigmoid": (_D, [_D]),
    "orc_log_sigmoid_v": (None, [_P, _I64, _P]),
    "orc_matchability": (None, [_P, _I64, _INT, _P, _D, _P]),
    "orc_token_confidence": (None, [_P, _I64, _INT, _P, _D, _P]),
    "orc_confidence_threshold": (_D, [_INT, _INT]),
    "orc_double_softmax_assignment": (None, [_P, _I64, _I64, _P, _P, _P]),
}

_lib = None


def lib():
    """The compiled oracle; built once if absent.  A library older than its
    source is refused rather than silently used."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        elif os.path.getmtime(LIB) < os.path.getmtime(SRC):
            raise RuntimeError(f"{LIB} is older than {SRC}: rebuild it (oracle.native.build())")
        L = C.CDLL(LIB)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Threads for the row-parallel loops (0: the OpenMP default)."""
    lib().orc_set_threads(int(n))


def threads() -> int:
    return int(lib().orc_threads())


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


class _Stage(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("Wq", "bq", "Wk", "bk", "Wv", "bv", "Wm", "bm",
                                           "W1", "b1", "W2", "b2", "Wqk", "bqk")]


def _stages(stages):
    """A C array of orc_stage for the weight dictionaries, plus the float64
    arrays it points to (kept alive by the caller)."""
    arr = (_Stage * max(len(stages), 1))()
    keep = []
    for s, st in enumerate(stages):
        for name, _ in _Stage._fields_:
            if name in st:
                a = _f64(st[name])
                keep.append(a)
                setattr(arr[s], name, a.ctypes.data)
    return arr, keep


# ------------------------------------------------------------------ steps

def normalize_keypoints(kpts, width, height):
    kp = _f64(kpts).reshape(-1, 2)
    out = np.empty_like(kp)
    lib().orc_normalize_keypoints(_p(kp), len(kp), float(width), float(height), _p(out))
    return out


def keypoint_encoder(kpts_n, conf, layers):
    kp, cf = _f64(kpts_n).reshape(-1, 2), _f64(conf).reshape(-1)
    Ws = [_f64(W) for W, _ in layers]
    bs = [_f64(b) for _, b in layers]
    widths = (C.c_int * (len(layers) + 1))(3, *[W.shape[0] for W in Ws])
    Wp = (C.c_void_p * len(Ws))(*[W.ctypes.data for W in Ws])
    bp = (C.c_void_p * len(bs))(*[b.ctypes.data for b in bs])
    out = np.empty((len(kp), Ws[-1].shape[0]))
    lib().orc_keypoint_encoder(_p(kp), _p(cf), len(kp), len(layers), widths, Wp, bp, _p(out))
    return out


def rope_angles(pos, basis):
    p, b = _f64(pos).reshape(-1, 2), _f64(basis).reshape(-1, 2)
    out = np.empty((len(p), len(b)))
    lib().orc_rope_angles(_p(p), len(p), _p(b), len(b), _p(out))
    return out


def rotate_pairs(t, theta, heads):
    t = _f64(t)
    th = _f64(theta)
    out = np.empty_like(t)
    lib().orc_rotate_pairs(_p(t), t.shape[0], t.shape[1], int(heads), _p(th), _p(out))
    return out


def multi_head_attention(x, src, st, heads, rope=None):
    x, src = _f64(x), _f64(src)
    arr, keep = _stages([st])
    out = np.empty((x.shape[0], x.shape[1]))
    tx = ts = None
    if rope is not None:
        tx, ts = _f64(rope[0]), _f64(rope[1])
    lib().orc_multi_head_attention(_p(x), x.shape[0], _p(src), src.shape[0], x.shape[1], int(heads), arr,
                                   _p(tx), _p(ts), _p(out))
    return out


def bidirectional_cross_attention(x0, x1, st, heads):
    x0, x1 = _f64(x0), _f64(x1)
    arr, keep = _stages([st])
    m0 = np.empty((x0.shape[0], x0.shape[1]))
    m1 = np.empty((x1.shape[0], x1.shape[1]))
    lib().orc_bidirectional_cross_attention(_p(x0), x0.shape[0], _p(x1), x1.shape[0], x0.shape[1], int(heads), arr,
                                            _p(m0), _p(m1))
    return m0, m1


def _update_mlp(x, m, st):
    x, m = _f64(x), _f64(m)
    arr, keep = _stages([st])
    out = np.empty_like(x)
    lib().orc_update_mlp(_p(x), _p(m), x.shape[0], x.shape[1], arr, _p(out))
    return out


def attentional_propagation(x, src, st, heads, rope=None):
    return _update_mlp(x, multi_head_attention(x, src, st, heads, rope), st)


def attentional_gnn(xA, xB, stages, heads, first_stage=0, rope=None):
    A, B = _f64(xA).copy(), _f64(xB).copy()
    arr, keep = _stages(list(stages))
    tA = tB = None
    if rope is not None:
        tA, tB = _f64(rope[0]), _f64(rope[1])
    lib().orc_attentional_gnn(_p(A), A.shape[0], _p(B), B.shape[0], A.shape[1], int(heads), arr, len(stages),
                              int(first_stage), _p(tA), _p(tB))
    return A, B


def final_projection(x, Wf, bf):
    x, W, b = _f64(x), _f64(Wf), _f64(bf)
    out = np.empty((x.shape[0], W.shape[0]))
    lib().orc_linear(_p(x), x.shape[0], x.shape[1], _p(W), _p(b), W.shape[0], _p(out))
    return out


def score_matrix(fA, fB):
    fA, fB = _f64(fA), _f64(fB)
    S = np.empty((fA.shape[0], fB.shape[0]))
    lib().orc_score_matrix(_p(fA), fA.shape[0], _p(fB), fB.shape[0], fA.shape[1], _p(S))
    return S


def log_sinkhorn_iterations(Z, log_mu, log_nu, iters, duals=False):
    """Z + u + v after `iters` iterations; with duals=True also (u, v)."""
    Z, lm, ln = _f64(Z), _f64(log_mu), _f64(log_nu)
    out = np.empty_like(Z)
    u, v = np.empty(Z.shape[0]), np.empty(Z.shape[1])
    lib().orc_log_sinkhorn_iterations(_p(Z), Z.shape[0], Z.shape[1], _p(lm), _p(ln), int(iters), _p(u), _p(v),
                                      _p(out))
    return (out, u, v) if duals else out


def log_optimal_transport(S, alpha, iters, duals=False):
    """The (M+1) x (N+1) log assignment; with duals=True also (u, v)."""
    S = _f64(S)
    M, N = S.shape
    out = np.empty((M + 1, N + 1))
    u, v = np.empty(M + 1), np.empty(N + 1)
    lib().orc_log_optimal_transport(_p(S), M, N, float(alpha), int(iters), _p(out), _p(u), _p(v))
    return (out, u, v) if duals else out


def sinkhorn_knopp_exp(Zbar, a, b, iters):
    Z, a, b = _f64(Zbar), _f64(a), _f64(b)
    P = np.empty_like(Z)
    lib().orc_sinkhorn_knopp_exp(_p(Z), Z.shape[0], Z.shape[1], _p(a), _p(b), int(iters), _p(P))
    return P


def extract_matches(logP, threshold=0.0):
    P = _f64(logP)
    M, N = P.shape[0] - 1, P.shape[1] - 1
    m0, m1 = np.empty(M, np.int32), np.empty(N, np.int32)
    s0, s1 = np.empty(M), np.empty(N)
    lib().orc_extract_matches(_p(P), M, N, float(threshold), _p(m0), _p(s0), _p(m1), _p(s1))
    return m0, s0, m1, s1


def log_sigmoid(z):
    if np.ndim(z) == 0:
        return float(lib().orc_log_sigmoid(float(z)))
    z = _f64(z)
    out = np.empty_like(z)
    lib().orc_log_sigmoid_v(_p(z), z.size, _p(out))
    return out


def matchability(x, wz, bz):
    x, w = _f64(x), _f64(wz).reshape(-1)
    z = np.empty(x.shape[0])
    lib().orc_matchability(_p(x), x.shape[0], x.shape[1], _p(w), float(bz), _p(z))
    return z


def token_confidence(x, wc, bc):
    x, w = _f64(x), _f64(wc).reshape(-1)
    c = np.empty(x.shape[0])
    lib().orc_token_confidence(_p(x), x.shape[0], x.shape[1], _p(w), float(bc), _p(c))
    return c


def confidence_threshold(layer, n_layers):
    return float(lib().orc_confidence_threshold(int(layer), int(n_layers)))


def double_softmax_assignment(S, z0, z1):
    S = _f64(S)
    M, N = S.shape
    z0, z1 = _f64(z0).reshape(M), _f64(z1).reshape(N)
    out = np.empty((M + 1, N + 1))
    lib().orc_double_softmax_assignment(_p(S), M, N, _p(z0), _p(z1), _p(out))
    return out


# ------------------------------------------------------------ compositions

def superglue_descriptors(pair, weights, L=None):
    """Encoder + GNN + final projection for one unpadded pair ([realcat]
    "特征点Encode": x^(0) = d + MLP_enc(p); [forward-notes] forward: the
    keypoints are normalised by the image size first)."""
    L = weights["L"] if L is None else L
    H = weights["H"]
    out, xs, thetas = {}, [], []
    for side in ("0", "1"):
        w, h = pair["image_size" + side]
        kn = normalize_keypoints(pair["kpts" + side], w, h)
        x0 = _f64(pair["desc" + side]) + keypoint_encoder(kn, pair["conf" + side], weights["enc"])
        xs.append(x0)
        out["x0_" + side] = x0
        if weights.get("rope_basis") is not None:
            thetas.append(rope_angles(kn, weights["rope_basis"]))
    rope = tuple(thetas) if thetas else None
    xA, xB = attentional_gnn(xs[0], xs[1], weights["stages"][:2 * L], H, rope=rope)
    out["xL_0"], out["xL_1"] = xA, xB
    out["f0"] = final_projection(xA, weights["Wf"], weights["bf"])
    out["f1"] = final_projection(xB, weights["Wf"], weights["bf"])
    return out


def match_from_descriptors(fA, fB, alpha, T, threshold=0.0):
    """Scores, optimal transport and extraction from matching descriptors."""
    S = score_matrix(fA, fB)
    logP, u, v = log_optimal_transport(S, alpha, T, duals=True)
    m0, s0, m1, s1 = extract_matches(logP, threshold)
    return {"S": S, "logP": logP, "u": u, "v": v, "matches0": m0, "scores0": s0, "matches1": m1, "scores1": s1}


def _empty(M, N):
    return {"matches0": -np.ones(M, np.int32), "scores0": np.zeros(M),
            "matches1": -np.ones(N, np.int32), "scores1": np.zeros(N)}


def superglue_match(pair, weights, L=None, T=100, threshold=0.0):
    """The whole forward pass for one pair ([forward-notes] forward: with no
    keypoints in either image the matches are -1, the scores 0)."""
    M, N = len(pair["kpts0"]), len(pair["kpts1"])
    if M == 0 or N == 0:
        return _empty(M, N)
    out = superglue_descriptors(pair, weights, L)
    out.update(match_from_descriptors(out["f0"], out["f1"], weights["alpha"], T, threshold))
    return out


def double_softmax_from_descriptors(fA, fB, xA, xB, wz, bz, threshold=0.0):
    S = score_matrix(fA, fB)
    z0, z1 = matchability(xA, wz, bz), matchability(xB, wz, bz)
    logP = double_softmax_assignment(S, z0, z1)
    m0, s0, m1, s1 = extract_matches(logP, threshold)
    return {"S": S, "z0": z0, "z1": z1, "logP": logP,
            "matches0": m0, "scores0": s0, "matches1": m1, "scores1": s1}


def double_softmax_match(pair, weights, L=None, threshold=0.0):
    M, N = len(pair["kpts0"]), len(pair["kpts1"])
    if M == 0 or N == 0:
        return _empty(M, N)
    out = superglue_descriptors(pair, weights, L)
    out.update(double_softmax_from_descriptors(out["f0"], out["f1"], out["xL_0"], out["xL_1"],
                                               weights["wz"], weights["bz"], threshold))
    return out


def layer_head(weights, layer):
    """Layer `layer`'s own head (W_f, b_f, w_z, b_z); the network's last
    stored layer uses the main head ([LightGlue-review] section 2.5)."""
    heads = weights.get("heads") or []
    if layer < len(heads):
        return heads[layer]
    return weights["Wf"], weights["bf"], weights["wz"], weights["bz"]


def adaptive_match(pair, weights, L=None, depth_confidence=0.95, width_confidence=0.99,
                   prune_min=1024, early_exit=True, prune=True, threshold=0.0):
    """[LightGlue-review] sections 2.6 (adaptive depth) and 2.7 (adaptive
    width) with the double-softmax head of section 2.4, for one pair; the
    same contract as oracle.reference_numpy.adaptive_match.  Layer l runs
    stages 2l (self) and 2l + 1 (cross) on the remaining points; after every
    layer but the last the pass stops when the share of confident points
    (over the original M + N) exceeds depth_confidence, else images above
    prune_min points drop the points that are confidently unmatchable."""
    L = weights["L"] if L is None else L
    H = weights["H"]
    M, N = len(pair["kpts0"]), len(pair["kpts1"])
    out = {"matches0": -np.ones(M, np.int32), "scores0": np.zeros(M),
           "matches1": -np.ones(N, np.int32), "scores1": np.zeros(N),
           "prune0": np.ones(M, np.int32), "prune1": np.ones(N, np.int32), "exit_layer": -1}
    if M == 0 or N == 0:
        return out
    xs, pos = [], []
    for side in ("0", "1"):
        w, h = pair["image_size" + side]
        kn = normalize_keypoints(pair["kpts" + side], w, h)
        pos.append(kn)
        xs.append(_f64(pair["desc" + side]) + keypoint_encoder(kn, pair["conf" + side], weights["enc"]))
    ind = [np.arange(M), np.arange(N)]
    basis = weights.get("rope_basis")
    layer = 0
    for layer in range(L):
        rope = None
        if basis is not None:
            rope = (rope_angles(pos[0][ind[0]], basis), rope_angles(pos[1][ind[1]], basis))
        xs[0], xs[1] = attentional_gnn(xs[0], xs[1], weights["stages"][2 * layer:2 * layer + 2], H,
                                       first_stage=2 * layer, rope=rope)
        if layer == L - 1:
            break
        lam = confidence_threshold(layer, L)
        conf = None
        if early_exit:
            wc, bc = weights["conf"][layer]
            conf = [token_confidence(x, wc, bc) for x in xs]
            unconfident = sum(int((c < lam).sum()) for c in conf)
            if 1.0 - unconfident / (M + N) > depth_confidence:
                break
        if prune:
            _, _, wz, bz = layer_head(weights, layer)
            for k in (0, 1):
                if len(ind[k]) <= prune_min:
                    continue
                # sigma(z) of the layer's matchability (token_confidence is
                # exp(log sigma(<w, x> + b)))
                keep = token_confidence(xs[k], wz, bz) > 1.0 - width_confidence
                if conf is not None:
                    keep |= conf[k] <= lam
                xs[k], ind[k] = xs[k][keep], ind[k][keep]
                out["prune%d" % k][ind[k]] += 1
        if len(ind[0]) == 0 or len(ind[1]) == 0:
            break
    out["exit_layer"] = layer
    if len(ind[0]) == 0 or len(ind[1]) == 0:
        return out
    Wf, bf, wz, bz = layer_head(weights, layer)
    f0, f1 = final_projection(xs[0], Wf, bf), final_projection(xs[1], Wf, bf)
    r = double_softmax_from_descriptors(f0, f1, xs[0], xs[1], wz, bz, threshold)
    i0, i1 = ind
    out["matches0"][i0] = np.where(r["matches0"] >= 0, i1[np.maximum(r["matches0"], 0)], -1)
    out["scores0"][i0] = r["scores0"]
    out["matches1"][i1] = np.where(r["matches1"] >= 0, i0[np.maximum(r["matches1"], 0)], -1)
    out["scores1"][i1] = r["scores1"]
    out.update({"kept0": i0, "kept1": i1, "logP": r["logP"], "f0": f0, "f1": f1})
    return out
