"""Float64 numpy implementation of the oracle: the independent cross-check of
the plain C oracle (oracle/sg_oracle.c, front in oracle/native.py).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark import this package; the product path never
does, and this package imports nothing from the product.

Every function follows the pages it cites, in float64 with numpy.  Library
primitives (matrix products, exp, log) serve as steps; there is no blocking,
fusion or reordering beyond what the cited definitions state.  The C oracle
computes the same functions with plain loops and no library, so the two share
nothing but the definitions; the pins in tests/test_oracle_*.py run against
both.  Pages cited (by title):

* "SuperGlue 的注意力图神经网络怎样传递信息" (huluoboge.top blog)  -> [GNN-blog]
* "SuperGlue:Learning Feature Matching with Graph Neural Networks论文阅读"
  (realcat.vercel.app notes)                                        -> [realcat]
* "SuperGlue_model_forward_learning" (SuperGlue_Code_Learning notes) -> [forward-notes]
* "论文解读:LightGlue,让稀疏特征匹配随难度自适应地快" (vincentqin.tech) -> [LightGlue-review]

Readings taken where the pages are silent (each also pinned by a test):

* attention logits are scaled by 1/sqrt(d_head) per head;
* heads own contiguous channel blocks [h*d_head, (h+1)*d_head);
* the concatenated heads pass a Linear(D, D) merge projection with bias;
* batch normalisation between MLP layers is omitted (it folds into W, b);
* both images are updated from the pre-stage states of a stage;
* argmax ties go to the lowest index; the match threshold is strict '>';
* masked (padded) keys and points are simply absent: a padded pair is the
  unpadded pair;
* rotary encoding ([LightGlue-review] section 2.2): positions are the
  normalised keypoints above; channel pairs (2k, 2k+1) inside each head
  share angle k, the same for every head;
* double-softmax head ([LightGlue-review] section 2.4): the similarity is
  the same S = f_A f_B^T / sqrt(D) (the page divides each projected
  descriptor by D^(1/4)); the matchability logit reads the last GNN states
  x^(L), not the projected f; the log assignment is extracted with the same
  mutual argmax and threshold as the Sinkhorn head.

Parity status: every function below is pinned by `tests/test_oracle_*.py`
except the end-to-end composition with trained weights, which no page prints
(parity unpinned beyond the invariants and per-step pins).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "normalize_keypoints", "keypoint_encoder", "multi_head_attention",
    "attentional_propagation", "attentional_gnn", "final_projection",
    "score_matrix", "logsumexp", "log_sinkhorn_iterations",
    "log_optimal_transport", "extract_matches", "superglue_match",
    "superglue_descriptors", "sinkhorn_knopp_exp", "match_from_descriptors",
    "bidirectional_cross_attention", "rope_angles", "rotate_pairs",
    "log_sigmoid", "matchability", "double_softmax_assignment",
    "double_softmax_from_descriptors", "double_softmax_match",
    "confidence_threshold", "token_confidence", "layer_head", "adaptive_match",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def normalize_keypoints(kpts, width, height):
    """[forward-notes] normalize_keypoints: centre on (width/2, height/2) and
    divide both coordinates by 0.7 * max(width, height)."""
    kpts = _f64(kpts)
    size = np.array([width, height], dtype=np.float64)
    center = size / 2.0
    scaling = size.max() * 0.7
    return (kpts - center[None, :]) / scaling


def keypoint_encoder(kpts_n, conf, layers):
    """[realcat] section "特征点Encode" (KeypointEncoder / MLP): the input per
    point is (x, y, c); each layer is a per-point linear map W p + b
    (Conv1d with kernel 1), followed by ReLU except after the last layer."""
    h = np.concatenate([_f64(kpts_n), _f64(conf)[:, None]], axis=1)
    for i, (W, b) in enumerate(layers):
        h = h @ _f64(W).T + _f64(b)
        if i < len(layers) - 1:
            h = np.maximum(h, 0.0)
    return h


def _softmax_rows(e):
    """[GNN-blog] section "Attention 让节点自己选择消息来源": alpha_ij =
    exp(e_ij) / sum_r exp(e_ir) over the allowed sources of row i."""
    e = e - e.max(axis=1, keepdims=True)
    a = np.exp(e)
    return a / a.sum(axis=1, keepdims=True)


def rope_angles(pos, basis):
    """[LightGlue-review] section 2.2 (relative positions in self-attention):
    the per-head channels form d_h/2 two-dimensional subspaces; subspace k
    maps a point's position p onto its learned 2-D basis vector b_k, giving
    the angle theta_k = <b_k, p>.  Returns [n][d_h/2]."""
    return _f64(pos) @ _f64(basis).T


def rotate_pairs(t, theta, heads):
    """[LightGlue-review] section 2.2: rotate each 2-D subspace of every head
    by its angle: channels (2k, 2k+1) of head h (offset h*d_h) map
    (a, b) -> (a cos theta_k - b sin theta_k, a sin theta_k + b cos theta_k).
    Every head uses the same angles."""
    t = _f64(t).copy()
    D = t.shape[1]
    dh = D // heads
    c, s = np.cos(theta), np.sin(theta)
    for h in range(heads):
        a = t[:, h * dh:(h + 1) * dh:2].copy()
        b = t[:, h * dh + 1:(h + 1) * dh:2].copy()
        t[:, h * dh:(h + 1) * dh:2] = a * c - b * s
        t[:, h * dh + 1:(h + 1) * dh:2] = a * s + b * c
    return t


def multi_head_attention(x, src, st, heads, rope=None):
    """Message m for every query point of `x` from the source points `src`.

    [realcat] section "Attentional Aggregation": q_i = W1 x_i^Q + b1 from the
    query image, [k_j; v_j] = [W2; W3] x_j^S + [b2; b3] from the source image,
    m_i = sum_j alpha_ij v_j with alpha_ij = softmax_j(q_i^T k_j).
    [GNN-blog] section "Attention 让节点自己选择消息来源": logits divided by
    sqrt(d_k), d_k the per-head dimension.  Heads split D into contiguous
    blocks; the concatenated heads then pass the merge projection
    W_m m + b_m.  Stage weights `st` hold Wq,bq,Wk,bk,Wv,bv,Wm,bm.
    rope = (theta_x, theta_src): [LightGlue-review] section 2.2, q and k (not
    v) rotated by their points' angles after the projection.
    """
    x, src = _f64(x), _f64(src)
    D = x.shape[1]
    dh = D // heads
    q = x @ _f64(st["Wq"]).T + _f64(st["bq"])
    k = src @ _f64(st["Wk"]).T + _f64(st["bk"])
    v = src @ _f64(st["Wv"]).T + _f64(st["bv"])
    if rope is not None:
        q = rotate_pairs(q, rope[0], heads)
        k = rotate_pairs(k, rope[1], heads)
    msg = np.zeros((x.shape[0], D))
    for h in range(heads):
        c = slice(h * dh, (h + 1) * dh)
        e = (q[:, c] @ k[:, c].T) / np.sqrt(dh)
        msg[:, c] = _softmax_rows(e) @ v[:, c]
    return msg @ _f64(st["Wm"]).T + _f64(st["bm"])


def bidirectional_cross_attention(x0, x1, st, heads):
    """Messages (m0, m1) of both images from one shared similarity.

    [LightGlue-review] section 2.3 (bidirectional cross-attention): each image
    has a single projection qk = W_qk x + b_qk (no separate query) and a value
    projection v = W_v x + b_v; per head the similarity sim_ij =
    qk0_i^T qk1_j / sqrt(d_h) is formed once; its softmax over j (each row)
    aggregates image 1's values into m0, its softmax over i (each column)
    aggregates image 0's values into m1.  Heads as in multi_head_attention,
    then the merge projection W_m m + b_m.  Stage weights `st` hold
    Wqk,bqk,Wv,bv,Wm,bm.
    """
    x0, x1 = _f64(x0), _f64(x1)
    D = x0.shape[1]
    dh = D // heads
    qk0 = x0 @ _f64(st["Wqk"]).T + _f64(st["bqk"])
    qk1 = x1 @ _f64(st["Wqk"]).T + _f64(st["bqk"])
    v0 = x0 @ _f64(st["Wv"]).T + _f64(st["bv"])
    v1 = x1 @ _f64(st["Wv"]).T + _f64(st["bv"])
    m0 = np.zeros((x0.shape[0], D))
    m1 = np.zeros((x1.shape[0], D))
    for h in range(heads):
        c = slice(h * dh, (h + 1) * dh)
        sim = (qk0[:, c] @ qk1[:, c].T) / np.sqrt(dh)
        m0[:, c] = _softmax_rows(sim) @ v1[:, c]
        m1[:, c] = _softmax_rows(sim.T) @ v0[:, c]
    merge = lambda m: m @ _f64(st["Wm"]).T + _f64(st["bm"])
    return merge(m0), merge(m1)


def _update_mlp(x, m, st):
    """[realcat] section "多层GNN" (AttentionalPropagation): MLP([x || m]) with
    channels [2D, 2D, D], ReLU between the two layers."""
    h = np.concatenate([_f64(x), m], axis=1) @ _f64(st["W1"]).T + _f64(st["b1"])
    h = np.maximum(h, 0.0)
    return h @ _f64(st["W2"]).T + _f64(st["b2"])


def attentional_propagation(x, src, st, heads, rope=None):
    """[realcat] section "多层GNN" (AttentionalPropagation): the residual
    update MLP([x || m]) with channels [2D, 2D, D], ReLU between the two
    layers.  Returns the update (delta), not x + delta."""
    return _update_mlp(x, multi_head_attention(x, src, st, heads, rope), st)


def attentional_gnn(xA, xB, stages, heads, first_stage=0, rope=None):
    """[realcat] section "多层GNN" (AttentionalGNN) and [GNN-blog] section
    "多轮消息怎样回到同一幅图": stages alternate self (sources = own image)
    and cross (sources = the other image), self first; each stage has its own
    weights, shared by both images, and both deltas are computed from the
    states before the stage, then added.  `stages` may be a slice of the
    network starting at stage index `first_stage` (even = self).  A cross
    stage whose weights hold "Wqk" uses bidirectional_cross_attention
    ([LightGlue-review] section 2.3) for both messages, followed by the same
    update MLP.  rope = (theta_A, theta_B) (rope_angles of each image's
    points): self stages rotate q and k ([LightGlue-review] section 2.2: the
    encoding is the same for every layer and never enters cross stages)."""
    xA, xB = _f64(xA).copy(), _f64(xB).copy()
    for s, st in enumerate(stages, start=first_stage):
        if s % 2 == 1 and "Wqk" in st:   # bidirectional cross
            mA, mB = bidirectional_cross_attention(xA, xB, st, heads)
            dA, dB = _update_mlp(xA, mA, st), _update_mlp(xB, mB, st)
        else:
            ropeA = ropeB = None
            if s % 2 == 0:          # self
                srcA, srcB = xA, xB
                if rope is not None:
                    ropeA, ropeB = (rope[0], rope[0]), (rope[1], rope[1])
            else:                   # cross
                srcA, srcB = xB, xA
            dA = attentional_propagation(xA, srcA, st, heads, ropeA)
            dB = attentional_propagation(xB, srcB, st, heads, ropeB)
        xA, xB = xA + dA, xB + dB
    return xA, xB


def final_projection(x, Wf, bf):
    """[realcat] section "Attentional Aggregation" (last equation): matching
    descriptors f_i = W x_i^(L) + b."""
    return _f64(x) @ _f64(Wf).T + _f64(bf)


def score_matrix(fA, fB):
    """[realcat] section "匹配得分预测": S_ij = <f_i^A, f_j^B>; [forward-notes]
    forward: divided by sqrt(descriptor_dim)."""
    fA, fB = _f64(fA), _f64(fB)
    return (fA @ fB.T) / np.sqrt(fA.shape[1])


def logsumexp(X, axis):
    """log sum exp along `axis`, as max + log(sum(exp(X - max)))."""
    m = X.max(axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.exp(X - m).sum(axis=axis))


def _sinkhorn_duals(Z, log_mu, log_nu, iters):
    """[realcat] section "Sinkhorn Algorithm": alternating projections of the
    plan exp(Z + u + v) onto its row and column marginals, in the log
    domain.  A projection sets one side's duals so that the log-sum of
    Z + u + v along each of its lines equals the line's log marginal, the
    rows first, then the columns; the duals start at zero and exactly
    `iters` iterations run (no tolerance stop).  Returns (u, v)."""
    Z = _f64(Z)
    rows, cols = np.zeros(Z.shape[0]), np.zeros(Z.shape[1])
    for _ in range(iters):
        rows = _f64(log_mu) - logsumexp(Z + cols[None, :], axis=1)
        cols = _f64(log_nu) - logsumexp(Z + rows[:, None], axis=0)
    return rows, cols


def log_sinkhorn_iterations(Z, log_mu, log_nu, iters, duals=False):
    """Z + u + v after `iters` iterations of _sinkhorn_duals; with
    duals=True also (u, v)."""
    u, v = _sinkhorn_duals(Z, log_mu, log_nu, iters)
    out = _f64(Z) + u[:, None] + v[None, :]
    return (out, u, v) if duals else out


def log_optimal_transport(S, alpha, iters, duals=False):
    """[realcat] sections "遮挡以及可见性" and "Sinkhorn Algorithm": the
    scores get a dustbin row, column and corner of score alpha; the row
    marginals are a = (1, ..., 1, N) (M ones, the dustbin row can absorb all
    N points of B) and the column marginals b = (1, ..., 1, M), both divided
    by M + N; the log-domain iterations run on the bordered matrix; the
    result is multiplied back by M + N (log(M + N) added).  Returns the
    (M+1) x (N+1) log assignment, and with duals=True also (u, v)."""
    S = _f64(S)
    M, N = S.shape
    Z = np.pad(S, ((0, 1), (0, 1)), mode="constant", constant_values=float(alpha))
    a = np.append(np.ones(M), float(N))
    b = np.append(np.ones(N), float(M))
    total = np.log(float(M + N))
    u, v = _sinkhorn_duals(Z, np.log(a) - total, np.log(b) - total, iters)
    logP = Z + u[:, None] + v[None, :] + total
    return (logP, u, v) if duals else logP


def extract_matches(logP, threshold=0.0):
    """[forward-notes] forward, the matches whose score is above
    match_threshold, from the real block of the log assignment: every row
    picks its best column and every column its best row (the lowest index
    among equal maxima); a pair is kept when each is the other's pick and
    its probability exp(logP) exceeds the threshold.  Rows and columns
    without a kept pair get -1; a mutual pick's score is its probability
    (also when the threshold rejects it), other scores are 0.  Returns
    (matches0, scores0, matches1, scores1)."""
    real = _f64(logP)[:-1, :-1]
    M, N = real.shape
    pick_row = real.argmax(axis=1)          # best column of every row
    pick_col = real.argmax(axis=0)          # best row of every column
    rows = np.arange(M)
    mutual_row = pick_col[pick_row] == rows
    best = real[rows, pick_row]
    # exp(best) > threshold decided exactly: in log space for a positive
    # threshold, and always true otherwise (exp never reaches 0), so that the
    # underflow of exp for very negative log assignments cannot flip it
    above = best > np.log(threshold) if threshold > 0 else np.ones(M, dtype=bool)
    kept_row = mutual_row & above
    scores0 = np.where(mutual_row, np.exp(best), 0.0)
    matches0 = np.where(kept_row, pick_row, -1).astype(np.int32)
    mutual_col = pick_row[pick_col] == np.arange(N)
    scores1 = np.where(mutual_col, scores0[pick_col], 0.0)
    matches1 = np.where(mutual_col & kept_row[pick_col], pick_col, -1).astype(np.int32)
    return matches0, scores0, matches1, scores1


def superglue_descriptors(pair, weights, L=None):
    """Encoder + GNN + final projection for one unpadded pair; returns a dict
    with x0 (initial states), xL (last states) and f (matching descriptors)
    for both images.  [realcat] "特征点Encode": x^(0) = d + MLP_enc(p);
    [forward-notes] forward: normalise keypoints by the image size first."""
    L = weights["L"] if L is None else L
    H = weights["H"]
    out = {}
    xs, thetas = [], []
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


def superglue_match(pair, weights, L=None, T=100, threshold=0.0):
    """The whole forward pass for one pair.  [forward-notes] forward: with no
    keypoints in either image, matches are -1 and scores 0 and nothing else
    is computed."""
    M = len(pair["kpts0"])
    N = len(pair["kpts1"])
    if M == 0 or N == 0:
        return {"matches0": -np.ones(M, np.int32), "scores0": np.zeros(M),
                "matches1": -np.ones(N, np.int32), "scores1": np.zeros(N)}
    out = superglue_descriptors(pair, weights, L)
    out.update(match_from_descriptors(out["f0"], out["f1"], weights["alpha"], T, threshold))
    return out


def sinkhorn_knopp_exp(Zbar, a, b, iters):
    """Second, independent algorithm for the same iteration, in the
    probability domain: [realcat] section "Sinkhorn Algorithm" (the MATLAB
    demo's loop) with the kernel exp(+Zbar) of a similarity matrix: start from
    exp(Zbar) normalised to sum 1, then `iters` times scale the rows to sum to
    a and the columns to sum to b.  No early stop.  Test use only."""
    P = np.exp(_f64(Zbar))
    P = P / P.sum()
    a, b = _f64(a), _f64(b)
    for _ in range(iters):
        P = P * (a / P.sum(axis=1))[:, None]
        P = P * (b / P.sum(axis=0))[None, :]
    return P


# ------------------------------------------------- double-softmax head
# [LightGlue-review] section 2.4 (the matching head that replaces the
# optimal-transport layer with a closed form).


def log_sigmoid(z):
    """log(1 / (1 + exp(-z))), written as min(z, 0) - log(1 + exp(-|z|)) so
    that it is finite for any finite z."""
    z = _f64(z)
    return np.minimum(z, 0.0) - np.log1p(np.exp(-np.abs(z)))


def matchability(x, wz, bz):
    """[LightGlue-review] section 2.4: a unary matchability logit per point,
    a Linear(D, 1) of its state: z_i = <w, x_i> + b."""
    return _f64(x) @ _f64(wz).reshape(-1) + float(bz)


def double_softmax_assignment(S, z0, z1):
    """[LightGlue-review] section 2.4: the (M+1) x (N+1) log assignment.
    Real block: the log-softmax of S over j (each row) plus the log-softmax
    of S over i (each column) plus log sigmoid(z0_i) + log sigmoid(z1_j).
    Last column (i < M): log sigmoid(-z0_i); last row (j < N):
    log sigmoid(-z1_j); the corner stays 0."""
    S = _f64(S)
    M, N = S.shape
    z0, z1 = _f64(z0).reshape(M), _f64(z1).reshape(N)
    row_term = S - logsumexp(S, axis=1)[:, None]
    col_term = S - logsumexp(S, axis=0)[None, :]
    out = np.zeros((M + 1, N + 1))
    out[:M, :N] = row_term + col_term + log_sigmoid(z0)[:, None] + log_sigmoid(z1)[None, :]
    out[:M, N] = log_sigmoid(-z0)
    out[M, :N] = log_sigmoid(-z1)
    return out


def double_softmax_from_descriptors(fA, fB, xA, xB, wz, bz, threshold=0.0):
    """Similarity, matchability, log assignment and extraction of the
    double-softmax head from matching descriptors f and last states x."""
    S = score_matrix(fA, fB)
    z0, z1 = matchability(xA, wz, bz), matchability(xB, wz, bz)
    logP = double_softmax_assignment(S, z0, z1)
    m0, s0, m1, s1 = extract_matches(logP, threshold)
    return {"S": S, "z0": z0, "z1": z1, "logP": logP,
            "matches0": m0, "scores0": s0, "matches1": m1, "scores1": s1}


def double_softmax_match(pair, weights, L=None, threshold=0.0):
    """The whole forward pass with the double-softmax head for one pair: the
    encoder and GNN of superglue_descriptors, then the head above with
    weights["wz"] ([D]) and weights["bz"] (scalar)."""
    M = len(pair["kpts0"])
    N = len(pair["kpts1"])
    if M == 0 or N == 0:
        return {"matches0": -np.ones(M, np.int32), "scores0": np.zeros(M),
                "matches1": -np.ones(N, np.int32), "scores1": np.zeros(N)}
    out = superglue_descriptors(pair, weights, L)
    out.update(double_softmax_from_descriptors(out["f0"], out["f1"], out["xL_0"], out["xL_1"],
                                               weights["wz"], weights["bz"], threshold))
    return out


# ------------------------------------------------ adaptive depth and width
# [LightGlue-review] sections 2.6 (adaptive depth) and 2.7 (adaptive width).
# A "layer" is one self stage followed by one cross stage.


def confidence_threshold(layer, n_layers):
    """[LightGlue-review] section 2.6: the per-layer confidence threshold
    lambda_l = 0.8 + 0.1 exp(-4 l / L), clipped to [0, 1]."""
    return float(np.clip(0.8 + 0.1 * np.exp(-4.0 * layer / n_layers), 0.0, 1.0))


def token_confidence(x, wc, bc):
    """[LightGlue-review] section 2.5: a linear layer plus sigmoid on a point's
    current state: c_i = sigmoid(<w, x_i> + b)."""
    return np.exp(log_sigmoid(_f64(x) @ _f64(wc).reshape(-1) + float(bc)))


def layer_head(weights, layer):
    """The matching head of layer `layer`: its own (W_f, b_f, w_z, b_z) for
    every layer but the network's last stored one, which uses the main head
    ([LightGlue-review] section 2.5: every layer has a head)."""
    heads = weights.get("heads") or []
    if layer < len(heads):
        return heads[layer]
    return weights["Wf"], weights["bf"], weights["wz"], weights["bz"]


def adaptive_match(pair, weights, L=None, depth_confidence=0.95, width_confidence=0.99,
                   prune_min=1024, early_exit=True, prune=True, threshold=0.0):
    """[LightGlue-review] sections 2.6 and 2.7 with the double-softmax head
    of section 2.4, for one pair.

    Layer l runs stages 2l (self) and 2l+1 (cross) on the points that remain.
    After every layer but the last: if early_exit, each point's confidence
    c = token_confidence(x, weights["conf"][l]) and lambda_l; the pass stops
    when 1 - (number of remaining points with c < lambda_l) / (M + N) exceeds
    depth_confidence (M, N the original counts).  Otherwise, if prune, an
    image with more than prune_min remaining points keeps the points whose
    matchability sigmoid(z) (the layer's own head) exceeds 1 -
    width_confidence, or whose confidence is at most lambda_l (when
    early_exit computes it).  An image left without points ends the pass.
    The head of the last layer run gives the log assignment of the
    remaining points; matches map back to the original indices and pruned
    points get -1 / 0.  Also returns "exit_layer" and "prune0"/"prune1"
    (1 + the number of pruning steps each point survived)."""
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
                keep = np.exp(log_sigmoid(matchability(xs[k], wz, bz))) > 1.0 - width_confidence
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
