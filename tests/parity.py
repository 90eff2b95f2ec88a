"""Helpers of the GPU parity tests: device upload and the comparison rules.

Tolerances (written in the tests that use them):
  * matching descriptors f: per keypoint ||f_gpu - f_oracle|| / ||f_oracle||
    <= 1e-4 for fp32 networks, <= 2e-2 for bf16 networks;
  * log assignments: |logP_gpu - logP_oracle| <= 1e-3 everywhere;
  * match indices: identical, except rows whose oracle top-2 gap (in the row,
    or in the column of the oracle's or the GPU's choice) is below 1e-4, and
    rows whose log assignment lies within 1e-3 of log(threshold).
"""
import numpy as np
import torch


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def host(t):
    return t.detach().cpu().numpy()


def rel_rows(got, want):
    """Per-row relative error ||got - want|| / ||want||."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return np.linalg.norm(got - want, axis=1) / np.maximum(np.linalg.norm(want, axis=1), 1e-30)


def top2_gap(X, axis):
    s = np.sort(X, axis=axis)
    if X.shape[axis] < 2:
        return np.full(X.shape[1 - axis], np.inf)
    if axis == 1:
        return s[:, -1] - s[:, -2]
    return s[-1, :] - s[-2, :]


def check_matches(m0_gpu, m1_gpu, logP_or, m0_or, m1_or, threshold=0.0, gap=1e-4, thr_tol=1e-3):
    """Matches equal except where the oracle's decision is a near tie.
    Returns the number of exempted rows (for reporting)."""
    P = np.asarray(logP_or)[:-1, :-1]
    M, N = P.shape
    rgap = top2_gap(P, 1)
    cgap = top2_gap(P, 0)
    amax_r = P.argmax(axis=1)
    near_thr = np.zeros(M, bool)
    if threshold > 0:
        near_thr = np.abs(P[np.arange(M), amax_r] - np.log(threshold)) < thr_tol
    exempt = 0
    bad = []
    for i in np.nonzero(np.asarray(m0_gpu) != np.asarray(m0_or))[0]:
        j_gpu = int(m0_gpu[i])
        ok = rgap[i] < gap or cgap[amax_r[i]] < gap or near_thr[i] or (j_gpu >= 0 and cgap[j_gpu] < gap)
        if ok:
            exempt += 1
        else:
            bad.append((int(i), int(m0_or[i]), j_gpu, float(rgap[i]), float(cgap[amax_r[i]])))
    amax_c = P.argmax(axis=0)
    for j in np.nonzero(np.asarray(m1_gpu) != np.asarray(m1_or))[0]:
        i_gpu = int(m1_gpu[j])
        ok = cgap[j] < gap or rgap[amax_c[j]] < gap or near_thr[amax_c[j]] or (i_gpu >= 0 and rgap[i_gpu] < gap)
        if ok:
            exempt += 1
        else:
            bad.append(("col", int(j), int(m1_or[j]), i_gpu, float(cgap[j])))
    assert not bad, f"{len(bad)} match decisions differ outside near ties, e.g. {bad[:5]}"
    return exempt
