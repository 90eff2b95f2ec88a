"""Seeded synthetic inputs for the SuperGlue matching forward pass.

This module draws the random numbers that both the plain CPU oracle and the
HIP library consume: network weights, keypoint positions, detector
confidences, descriptors and planted correspondences.  It holds none of the
matching method's arithmetic (no encoder, attention, scores, Sinkhorn or
extraction); positions stay in pixels, so keypoint normalisation is left to
each implementation.

Workload shapes (WORKLOADS) are those the matching pass is measured on: a
tiny fp32 pair, the full 512/512 fp32 pair, the 1024/1024 bf16 pair, the
unequal 2048/1536 fp32 pair and the ragged 32-pair bf16 batch.
The pages measure on public benchmarks (MegaDepth-1500 with 2048 features,
Aachen with up to 4096, HPatches with 1024); the cost of the pass depends only
on the point counts and the network shape, so these synthetic pairs stand in
for them and no dataset item is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

IMAGE_W = 640.0
IMAGE_H = 480.0


@dataclass(frozen=True)
class Config:
    """Network and workload shape of one synthetic workload."""
    seed_id: int        # offset of the default weight and input seeds
    M: int
    N: int
    D: int
    H: int
    L: int
    enc: tuple          # hidden widths of the keypoint encoder (without 3 and D)
    T: int
    dtype: str          # "f32" or "bf16": operand type of the GNN contractions
    planted: Optional[str] = None    # None, "B" (fraction of N) or "A" (fraction of M)
    planted_frac: float = 0.0
    batch: int = 1      # > 1: ragged batch of independent pairs
    pad: int = 0        # padded point count of a ragged batch
    n_range: tuple = (0, 0)          # inclusive range of per-pair point counts
    frac_range: tuple = (0.0, 0.0)   # per-pair planted fraction range


# The synthetic workloads, by name: point counts, network (D, H, L, encoder
# widths), Sinkhorn iterations T and the GNN operand type.
WORKLOADS = {
    # 10 x 12 points, D 64, L 2, T 20, fp32: small enough for pure-Python checks
    "pair10x12_f32": Config(0, 10, 12, 64, 4, 2, (16, 32), 20, "f32"),
    # 512 x 512 points, D 256, H 4, L 9, T 100, fp32
    "pair512_f32": Config(1, 512, 512, 256, 4, 9, (32, 64, 128, 256), 100, "f32"),
    # 1024 x 1024 points, bf16 GNN operands, 40 % of B's points planted
    "pair1024_bf16": Config(2, 1024, 1024, 256, 4, 9, (32, 64, 128, 256), 100, "bf16", "B", 0.4),
    # 2048 x 1536 points, fp32, 30 % of A's points planted
    "pair2048x1536_f32": Config(3, 2048, 1536, 256, 4, 9, (32, 64, 128, 256), 100, "f32", "A", 0.3),
    # 32 independent pairs, M_b, N_b ~ U{256..2048} padded to 2048, bf16
    "ragged32_bf16": Config(4, 2048, 2048, 256, 4, 9, (32, 64, 128, 256), 100, "bf16", "pair", 0.0,
                            batch=32, pad=2048, n_range=(256, 2048), frac_range=(0.2, 0.5)),
}

WEIGHT_SEED_BASE = 1000
INPUT_SEED_BASE = 2000
BIAS_ON_SEED_BASE = 3000


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Used only so that the drawn weights of a bf16 network are exactly
    representable in bf16; both implementations then read identical values.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _xavier(rng: np.random.Generator, n_out: int, n_in: int) -> np.ndarray:
    bound = np.sqrt(6.0 / (n_in + n_out))
    return rng.uniform(-bound, bound, size=(n_out, n_in)).astype(np.float32)


def _bias(rng: np.random.Generator, n_out: int, n_in: int, bias_on: bool, zero: bool) -> np.ndarray:
    if not bias_on or zero:
        return np.zeros(n_out, dtype=np.float32)
    bound = 1.0 / np.sqrt(n_in)
    return rng.uniform(-bound, bound, size=n_out).astype(np.float32)


def make_weights(cfg: Config, seed: Optional[int] = None, bias_on: bool = False,
                 L: Optional[int] = None, alpha: float = 1.0, cross: str = "standard",
                 rope: bool = False, adaptive: bool = False) -> dict:
    """Draw the network weights of `cfg` (row-major [out][in] matrices).

    Every matrix is Xavier-uniform U(+-sqrt(6/(fan_in+fan_out))).  Biases are
    zero unless `bias_on`, in which case they are U(+-1/sqrt(fan_in)) except the
    last encoder bias and the last bias of every update MLP, which stay zero.
    For a bf16 network every value is rounded to bf16.  Draw order: encoder
    layers, then per stage q, k, v, merge, mlp1, mlp2 (each W then b), then the
    final projection, then the matchability weight and bias of the
    double-softmax head ("wz" [D], "bz").  The dustbin score is `alpha`.
    cross="bidirectional": every cross stage draws one shared query/key
    projection ("Wqk", "bqk") and "Wv", "bv" instead of q, k, v.
    rope=True: a rotary basis "rope_basis" [d_h/2][2] ~ N(0, 1) (kept fp32).
    adaptive=True: "conf" [(w_c, b_c)] and "heads" [(W_f, b_f, w_z, b_z)] for
    every layer but the last (adaptive depth and width).
    """
    if seed is None:
        seed = (BIAS_ON_SEED_BASE if bias_on else WEIGHT_SEED_BASE) + cfg.seed_id
    L = cfg.L if L is None else L
    if cross not in ("standard", "bidirectional"):
        raise ValueError(f"cross = {cross!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    D = cfg.D
    widths = [3] + list(cfg.enc) + [D]
    enc = []
    for i in range(len(widths) - 1):
        W = _xavier(rng, widths[i + 1], widths[i])
        b = _bias(rng, widths[i + 1], widths[i], bias_on, zero=(i == len(widths) - 2))
        enc.append((W, b))
    stages = []
    for s in range(2 * L):
        st = {}
        attn = ((("qk", D, D, False), ("v", D, D, False)) if cross == "bidirectional" and s % 2 == 1
                else (("q", D, D, False), ("k", D, D, False), ("v", D, D, False)))
        for name, n_out, n_in, zero in attn + (("m", D, D, False), ("1", 2 * D, 2 * D, False),
                                               ("2", D, 2 * D, True)):
            st["W" + name] = _xavier(rng, n_out, n_in)
            st["b" + name] = _bias(rng, n_out, n_in, bias_on, zero)
        stages.append(st)
    Wf = _xavier(rng, D, D)
    bf = _bias(rng, D, D, bias_on, zero=False)
    # matchability Linear(D, 1) of the double-softmax head, drawn last so
    # that every earlier tensor is the same with or without it
    wz = _xavier(rng, 1, D)[0]
    bz = _bias(rng, 1, D, bias_on, zero=False)[0]
    # rotary basis of self-attention ([d_h/2][2], N(0, 1)), drawn last
    basis = rng.standard_normal((D // cfg.H // 2, 2)).astype(np.float32) if rope else None
    # adaptive depth / width: per layer but the last, a confidence Linear(D, 1)
    # and a matching head (W_f, b_f, w_z, b_z), drawn last
    conf, heads = [], []
    if adaptive:
        for _ in range(L - 1):
            conf.append((_xavier(rng, 1, D)[0], float(_bias(rng, 1, D, bias_on, zero=False)[0])))
            heads.append((_xavier(rng, D, D), _bias(rng, D, D, bias_on, zero=False),
                          _xavier(rng, 1, D)[0], float(_bias(rng, 1, D, bias_on, zero=False)[0])))
    w = {"enc": enc, "stages": stages, "Wf": Wf, "bf": bf, "alpha": float(alpha),
         "wz": wz, "bz": float(bz), "D": D, "H": cfg.H, "L": L, "dtype": cfg.dtype, "cross": cross,
         "rope_basis": basis, "conf": conf if adaptive else None, "heads": heads if adaptive else None}
    if cfg.dtype == "bf16":
        w["enc"] = [(round_to_bf16(W), round_to_bf16(b)) for W, b in w["enc"]]
        w["stages"] = [{k: round_to_bf16(v) for k, v in st.items()} for st in w["stages"]]
        w["Wf"], w["bf"] = round_to_bf16(w["Wf"]), round_to_bf16(w["bf"])
        w["wz"] = round_to_bf16(w["wz"])
        w["bz"] = float(round_to_bf16(np.array([w["bz"]], np.float32))[0])
        r1 = lambda v: float(round_to_bf16(np.array([v], np.float32))[0])
        if adaptive:
            w["conf"] = [(round_to_bf16(a), r1(b)) for a, b in w["conf"]]
            w["heads"] = [(round_to_bf16(a), round_to_bf16(b), round_to_bf16(c), r1(d)) for a, b, c, d in w["heads"]]
    return w


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _random_points(rng, n, D):
    kp = np.stack([rng.uniform(0, IMAGE_W, n), rng.uniform(0, IMAGE_H, n)], axis=1)
    conf = rng.uniform(0.0, 1.0, n)
    desc = _unit_rows(rng.standard_normal((n, D)))
    return kp, conf, desc


def random_homography(rng: np.random.Generator) -> np.ndarray:
    """A 3x3 homography mapping the image corners to corners moved by up to 15 % of the size."""
    src = np.array([[0, 0], [IMAGE_W, 0], [IMAGE_W, IMAGE_H], [0, IMAGE_H]], dtype=np.float64)
    dst = src + np.stack([rng.uniform(-0.15 * IMAGE_W, 0.15 * IMAGE_W, 4),
                          rng.uniform(-0.15 * IMAGE_H, 0.15 * IMAGE_H, 4)], axis=1)
    A = np.zeros((8, 8))
    rhs = np.zeros(8)
    for i, ((x, y), (u, v)) in enumerate(zip(src, dst)):
        A[2 * i] = [x, y, 1, 0, 0, 0, -u * x, -u * y]
        A[2 * i + 1] = [0, 0, 0, x, y, 1, -v * x, -v * y]
        rhs[2 * i], rhs[2 * i + 1] = u, v
    h = np.linalg.solve(A, rhs)
    return np.append(h, 1.0).reshape(3, 3)


def _warp(Hm, pts):
    p = np.concatenate([pts, np.ones((len(pts), 1))], axis=1) @ Hm.T
    return p[:, :2] / p[:, 2:3]


def _pair(rng, M, N, D, planted_k_fn):
    """One pair; planted_k_fn(number of in-frame A points) -> points to plant."""
    kpA, confA, descA = _random_points(rng, M, D)
    kpB, confB, descB = _random_points(rng, N, D)
    gt = -np.ones(M, dtype=np.int64)
    k = 0
    if planted_k_fn is not None:
        Hm = random_homography(rng)
        w = _warp(Hm, kpA)
        inside = np.nonzero((w[:, 0] >= 0) & (w[:, 0] < IMAGE_W) & (w[:, 1] >= 0) & (w[:, 1] < IMAGE_H))[0]
        k = min(planted_k_fn(), len(inside), N)
        sel = rng.permutation(inside)[:k]
        pos = w[sel] + rng.standard_normal((k, 2))
        pos[:, 0] = np.clip(pos[:, 0], 0.0, np.nextafter(IMAGE_W, 0))
        pos[:, 1] = np.clip(pos[:, 1], 0.0, np.nextafter(IMAGE_H, 0))
        kpB[:k] = pos
        descB[:k] = _unit_rows(descA[sel] + 0.1 * rng.standard_normal((k, D)))
        perm = rng.permutation(N)       # B is shuffled after planting
        kpB, confB, descB = kpB[perm], confB[perm], descB[perm]
        inv = np.empty(N, dtype=np.int64)
        inv[perm] = np.arange(N)
        gt[sel] = inv[np.arange(k)]
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return {"kpts0": f32(kpA), "conf0": f32(confA), "desc0": f32(descA),
            "kpts1": f32(kpB), "conf1": f32(confB), "desc1": f32(descB),
            "image_size0": (IMAGE_W, IMAGE_H), "image_size1": (IMAGE_W, IMAGE_H),
            "gt_matches0": gt, "n_planted": int(k)}


def make_pair(cfg: Config, seed: Optional[int] = None, M: Optional[int] = None,
              N: Optional[int] = None) -> dict:
    """Draw one keypoint pair of `cfg` (pixel positions in a 640x480 image).

    Points: (u, v) ~ U[0,640) x U[0,480), confidence ~ U(0,1), descriptor
    ~ N(0, I_D) then L2-normalised.  Planted configurations map a random subset
    of A's points through a random homography (plus N(0,1) px noise) into B and
    copy their descriptors with N(0, 0.1^2) noise, renormalised; B is shuffled.
    """
    if seed is None:
        seed = INPUT_SEED_BASE + cfg.seed_id
    rng = np.random.Generator(np.random.PCG64(seed))
    M = cfg.M if M is None else M
    N = cfg.N if N is None else N
    if cfg.planted == "B":
        fn = lambda: int(round(cfg.planted_frac * N))
    elif cfg.planted == "A":
        fn = lambda: int(round(cfg.planted_frac * M))
    else:
        fn = None
    return _pair(rng, M, N, cfg.D, fn)


def make_batch(cfg: Config, seed: Optional[int] = None, batch: Optional[int] = None) -> dict:
    """Draw a ragged batch: per pair M_b, N_b ~ U{lo..hi}, planted fraction f ~ U[f_lo, f_hi]
    of min(M_b, N_b); arrays are zero-padded to `cfg.pad` points."""
    if seed is None:
        seed = INPUT_SEED_BASE + cfg.seed_id
    B = cfg.batch if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(seed))
    lo, hi = cfg.n_range
    Ms = rng.integers(lo, hi + 1, size=B)
    Ns = rng.integers(lo, hi + 1, size=B)
    fr = rng.uniform(cfg.frac_range[0], cfg.frac_range[1], size=B)
    P, D = cfg.pad, cfg.D
    out = {"M": Ms.astype(np.int32), "N": Ns.astype(np.int32), "pairs": [],
           "kpts0": np.zeros((B, P, 2), np.float32), "conf0": np.zeros((B, P), np.float32),
           "desc0": np.zeros((B, P, D), np.float32), "kpts1": np.zeros((B, P, 2), np.float32),
           "conf1": np.zeros((B, P), np.float32), "desc1": np.zeros((B, P, D), np.float32),
           "image_size0": (IMAGE_W, IMAGE_H), "image_size1": (IMAGE_W, IMAGE_H)}
    for b in range(B):
        m, n = int(Ms[b]), int(Ns[b])
        pr = _pair(rng, m, n, D, lambda: int(round(fr[b] * min(m, n))))
        out["pairs"].append(pr)
        for key, cnt in (("kpts0", m), ("conf0", m), ("desc0", m), ("kpts1", n), ("conf1", n), ("desc1", n)):
            out[key][b, :cnt] = pr[key]
    return out


def random_states(n: int, D: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Residual-stream states for single-stage tests: N(0, scale^2) entries, float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.ascontiguousarray(scale * rng.standard_normal((n, D)), dtype=np.float32)


def random_matching_descriptors(M: int, N: int, D: int, seed: int, scale: float = 3.0,
                                planted_frac: float = 0.4, noise: float = 0.3) -> tuple:
    """Matching descriptors for score/Sinkhorn/extraction tests (scale 3 gives |S| up to
    about 150 at D = 256, the range the full network produces).

    f_A ~ N(0, scale^2 I); a fraction of f_B's rows are noisy copies of f_A rows
    (so the score matrix has clear matches, as a trained network would give),
    the rest are independent.  Returns float32 (f_A, f_B).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    fA = scale * rng.standard_normal((M, D))
    fB = scale * rng.standard_normal((N, D))
    k = min(int(round(planted_frac * N)), M)
    sel = rng.permutation(M)[:k]
    fB[:k] = fA[sel] + noise * scale * rng.standard_normal((k, D))
    fB = fB[rng.permutation(N)]
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return f32(fA), f32(fB)
