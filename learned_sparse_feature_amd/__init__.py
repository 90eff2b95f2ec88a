"""Python binding of libsg, the MI355X (gfx950) SuperGlue matching forward pass.

Every entry point mirrors the C function of the same name in include/sg.h and
only marshals arguments: torch tensors supply device memory and the stream,
and every step of the pass runs in the library's HIP kernels.  There is no
CPU fallback: without the built library (or without a GPU) calls raise.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import (SG_BF16, SG_CROSS_BIDIRECTIONAL, SG_CROSS_STANDARD, SG_F32, SG_HEAD_DOUBLE_SOFTMAX,
                   SG_HEAD_SINKHORN, SG_K_ATTENTION, SG_K_GEMM,
                   SG_K_NONE, SG_K_SINKHORN, SG_MAX_BATCH, SG_N_STAGE_EVENTS, SgError, SgOpts, SgWeights)

__all__ = ["Weights", "weights_config", "pack_weights", "workspace_size", "sg_match",
           "sg_match_batch", "sg_stage_encode", "sg_stage_gnn", "sg_stage_project", "sg_stage_scores",
           "sg_stage_match", "sg_stage_match_ds", "sg_stage_sinkhorn", "sg_stage_sinkhorn_noalloc", "sg_stage_extract", "lib", "SgError", "SG_K_GEMM", "SG_K_ATTENTION", "SG_K_SINKHORN",
           "SG_N_STAGE_EVENTS"]


def lib():
    return _lib.load()


def _dtype_code(dtype: str) -> int:
    return {"f32": SG_F32, "bf16": SG_BF16}[dtype]


_HEADS = {"sinkhorn": SG_HEAD_SINKHORN, "ds": SG_HEAD_DOUBLE_SOFTMAX}
_CROSS = {"standard": SG_CROSS_STANDARD, "bidirectional": SG_CROSS_BIDIRECTIONAL}


def weights_config(D: int, H: int, enc: Sequence[int], L_max: int, dtype: str = "f32",
                   head: str = "sinkhorn", cross: str = "standard", rope: bool = False,
                   adaptive: bool = False) -> SgWeights:
    """head: "sinkhorn" (optimal transport) or "ds" (double softmax + matchability);
    cross: "standard" or "bidirectional" cross-attention; rope: rotary encoding
    in self-attention."""
    st = SgWeights()
    st.D, st.H, st.n_enc, st.L_max, st.dtype = D, H, len(enc), L_max, _dtype_code(dtype)
    st.head = _HEADS[head]
    st.cross = _CROSS[cross]
    st.rope = 1 if rope else 0
    st.adaptive = 1 if adaptive else 0
    for i, e in enumerate(enc):
        st.enc[i] = e
    return st


class Weights:
    """A device weight blob plus the sg_weights struct that describes it."""

    def __init__(self, struct: SgWeights, blob: torch.Tensor, L_max: int):
        self.struct = struct
        self.blob = blob
        self.L_max = L_max
        struct.blob = blob.data_ptr()
        struct.blob_bytes = blob.numel()

    @property
    def ref(self):
        return C.byref(self.struct)

    @property
    def D(self):
        return self.struct.D

    @property
    def head(self):
        return "ds" if self.struct.head == SG_HEAD_DOUBLE_SOFTMAX else "sinkhorn"


def _ordered_tensors(w: dict, head: str):
    out = []
    for W, b in w["enc"]:
        out += [W, b]
    for st in w["stages"]:
        if "Wqk" in st:   # bidirectional cross stage: qk | v
            out += [np.concatenate([st["Wqk"], st["Wv"]]), np.concatenate([st["bqk"], st["bv"]])]
        else:
            out += [np.concatenate([st["Wq"], st["Wk"], st["Wv"]]), np.concatenate([st["bq"], st["bk"], st["bv"]])]
        out += [st["Wm"], st["bm"], st["W1"], st["b1"], st["W2"], st["b2"]]
    out += [w["Wf"], w["bf"], np.array([w["alpha"]], dtype=np.float32)]
    if head == "ds":
        out += [np.asarray(w["wz"]).reshape(1, -1), np.array([w["bz"]], dtype=np.float32)]
    if w.get("rope_basis") is not None:
        out.append(np.asarray(w["rope_basis"]))
    if head == "ds" and w.get("conf"):
        for (wc, bc), (Wf, bf, wz, bz) in zip(w["conf"], w["heads"]):
            out += [np.asarray(wc).reshape(1, -1), np.array([bc], np.float32), Wf, bf,
                    np.asarray(wz).reshape(1, -1), np.array([bz], np.float32)]
    return out


def pack_weights(w: dict, device="cuda", head: str = "sinkhorn") -> Weights:
    """Lay the weight dictionary (row-major [out][in] matrices) out as the
    library's blob, in the blob dtype, and upload it.  head="ds" selects the
    double-softmax head and appends the matchability weights wz, bz."""
    enc = [W.shape[0] for W, _ in w["enc"][:-1]]
    L_max = len(w["stages"]) // 2
    rope = w.get("rope_basis") is not None
    adaptive = head == "ds" and bool(w.get("conf"))
    st = weights_config(w["D"], w["H"], enc, L_max, w["dtype"], head, w.get("cross", "standard"), rope, adaptive)
    L = lib()
    nbytes = L.sg_weights_bytes(C.byref(st))
    count = L.sg_weights_count(C.byref(st))
    if nbytes == 0 or count <= 0:
        raise SgError(-1, "sg_weights_bytes")
    tensors = _ordered_tensors(w, head)
    # alpha and the rotary basis are always float32
    n_adapt = 6 * (L_max - 1) if adaptive else 0
    alpha_index = count - n_adapt - (3 if head == "ds" else 1) - (1 if rope else 0)
    f32_index = {alpha_index, alpha_index + (3 if head == "ds" else 1)} if rope else {alpha_index}
    if len(tensors) != count:
        raise ValueError(f"weight dictionary has {len(tensors)} tensors, the layout {count}")
    host = torch.zeros(nbytes, dtype=torch.uint8)
    tdt = torch.bfloat16 if w["dtype"] == "bf16" else torch.float32
    off, rows, cols = C.c_size_t(), C.c_int32(), C.c_int32()
    for i, arr in enumerate(tensors):
        _lib.check(L.sg_weights_tensor(C.byref(st), i, C.byref(off), C.byref(rows), C.byref(cols)),
                   "sg_weights_tensor")
        arr = np.ascontiguousarray(arr, dtype=np.float32).reshape(-1)
        if arr.size != rows.value * cols.value:
            raise ValueError(f"tensor {i}: {arr.size} values, layout {rows.value}x{cols.value}")
        t = torch.from_numpy(arr).to(torch.float32 if i in f32_index else tdt)
        raw = t.view(torch.uint8)
        host[off.value: off.value + raw.numel()] = raw
    return Weights(st, host.to(device), L_max)


def workspace_size(weights: Weights, Mmax: int, Nmax: int, batch: int = 1) -> int:
    return int(lib().sg_workspace_size(weights.ref, Mmax, Nmax, batch))


_ws_cache = {}


def _workspace(device, nbytes):
    key = torch.device(device).index or 0
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        _ws_cache[key] = t
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _check_tensor(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _events_array(events):
    if not events:
        return None, 0
    arr = (C.c_void_p * len(events))(*[e.cuda_event for e in events])
    return arr, len(events)


def make_events(n: int):
    """Timing events usable by the library (created on the current stream)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()  # materialise the underlying hipEvent
    return evs


_SINKHORN_FLAGS = {"auto": 0, "two": _lib.SG_FLAG_SINKHORN_TWO_SWEEP, "one": _lib.SG_FLAG_SINKHORN_ONE_SWEEP}


def _transposed_extra(sinkhorn, B, M, N):
    """Workspace bytes beyond workspace_size() for a forced two-sweep schedule
    (the transposed scores, [N][ld4(M)] fp32 per pair)."""
    return B * N * ((M + 3) // 4 * 4) * 4 if sinkhorn == "two" else 0


def _opts(device, *, threshold=0.0, image_size=None, workspace=None, ws_bytes=0, m1=None, s1=None,
          fA=None, fB=None, logP=None, logP_ld=0, stage_events=None, timed_kernel=SG_K_NONE,
          kernel_events=None, stream=None, graph=True, sinkhorn="auto", adaptive=None,
          shared_similarity=False):
    o = SgOpts()
    o.flags = (0 if graph else _lib.SG_FLAG_NO_GRAPH) | _SINKHORN_FLAGS[sinkhorn]
    if shared_similarity:
        o.flags |= _lib.SG_FLAG_SHARED_SIMILARITY
    if adaptive is not None:
        o.flags |= (_lib.SG_FLAG_EARLY_EXIT if adaptive.get("early_exit", True) else 0)
        o.flags |= (_lib.SG_FLAG_PRUNE if adaptive.get("prune", True) else 0)
        o.depth_confidence = float(adaptive.get("depth_confidence", 0.0))
        o.width_confidence = float(adaptive.get("width_confidence", 0.0))
        o.prune_min_points = int(adaptive.get("prune_min", 0))
    s = stream if stream is not None else torch.cuda.current_stream(device)
    o.stream = s.cuda_stream
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel()
    o.match_threshold = float(threshold)
    if image_size is not None:
        for i, v in enumerate(image_size):
            o.image_size[i] = float(v)
    o.out_matches1 = None if m1 is None else m1.data_ptr()
    o.out_scores1 = None if s1 is None else s1.data_ptr()
    o.out_desc_A = None if fA is None else fA.data_ptr()
    o.out_desc_B = None if fB is None else fB.data_ptr()
    o.out_logP = None if logP is None else logP.data_ptr()
    o.logP_ld = logP_ld
    keep = []
    arr, n = _events_array(stage_events)
    if arr is not None:
        o.stage_events, o.n_stage_events = C.cast(arr, C.c_void_p), n
        keep.append(arr)
    arr, n = _events_array(kernel_events)
    if arr is not None:
        o.timed_kernel = timed_kernel
        o.kernel_events, o.n_kernel_events = C.cast(arr, C.c_void_p), n
        keep.append(arr)
    count = C.c_int32(0)
    o.n_kernel_launches = C.pointer(count)
    keep.append(count)
    return o, keep, count


def sg_match(kptsA, descA, confA, kptsB, descB, confB, weights: Weights, L: int, T: int, *,
             threshold: float = 0.0, image_size=None, want_matches1=True, want_logP=False,
             want_desc=False, workspace=None, stage_events=None, timed_kernel=SG_K_NONE,
             kernel_events=None, stream=None, graph=True, out: Optional[dict] = None,
             sinkhorn: str = "auto", adaptive: Optional[dict] = None,
             shared_similarity: bool = False) -> dict:
    """One pair.  kpts [n][2] (pixels if image_size=(wA, hA, wB, hB) is given),
    desc [n][D], conf [n]: float32 CUDA tensors.  Returns device tensors;
    `out` may supply them (same keys) so that repeated calls reuse buffers.
    sinkhorn: "auto", or "two" / "one" to force a Sinkhorn schedule.
    adaptive (adaptive weights only): {"early_exit": bool, "prune": bool,
    "depth_confidence": a, "width_confidence": b, "prune_min": n} (0 = the
    library's default); adds "exit_layer", "prune0", "prune1" to the result.
    shared_similarity (bidirectional weights): each cross stage forms every
    head's similarity once and both directions read it."""
    dev = descA.device
    M, N, D = kptsA.shape[0], kptsB.shape[0], weights.D
    for t, nm, shp in ((kptsA, "kptsA", (M, 2)), (descA, "descA", (M, D)), (confA, "confA", (M,)),
                       (kptsB, "kptsB", (N, 2)), (descB, "descB", (N, D)), (confB, "confB", (N,))):
        _check_tensor(t, nm, torch.float32, shp)
    if out is None:
        out = {"matches0": torch.empty(M, dtype=torch.int32, device=dev),
               "scores0": torch.empty(M, dtype=torch.float32, device=dev)}
        if want_matches1:
            out["matches1"] = torch.empty(N, dtype=torch.int32, device=dev)
            out["scores1"] = torch.empty(N, dtype=torch.float32, device=dev)
        if want_logP:
            out["logP"] = torch.empty((M + 1, N + 1), dtype=torch.float32, device=dev)
        if want_desc:
            out["f0"] = torch.empty((M, D), dtype=torch.float32, device=dev)
            out["f1"] = torch.empty((N, D), dtype=torch.float32, device=dev)
    else:
        out = dict(out)
        for k, dt_, shp in (("matches0", torch.int32, (M,)), ("scores0", torch.float32, (M,)),
                            ("matches1", torch.int32, (N,)), ("scores1", torch.float32, (N,)),
                            ("logP", torch.float32, (M + 1, N + 1)), ("f0", torch.float32, (M, D)),
                            ("f1", torch.float32, (N, D))):
            if k in out:
                _check_tensor(out[k], k, dt_, shp)
    if workspace is None:
        workspace = _workspace(dev, workspace_size(weights, M, N, 1) + _transposed_extra(sinkhorn, 1, M, N))
    o, keep, count = _opts(dev, threshold=threshold, image_size=image_size, workspace=workspace,
                           m1=out.get("matches1"), s1=out.get("scores1"), fA=out.get("f0"),
                           fB=out.get("f1"), logP=out.get("logP"), logP_ld=N + 1,
                           stage_events=stage_events, timed_kernel=timed_kernel,
                           kernel_events=kernel_events, stream=stream, graph=graph, sinkhorn=sinkhorn,
                           adaptive=adaptive, shared_similarity=shared_similarity)
    exit_layer = C.c_int32(-1)
    if adaptive is not None:
        out["prune0"] = torch.empty(M, dtype=torch.int32, device=dev)
        out["prune1"] = torch.empty(N, dtype=torch.int32, device=dev)
        o.out_prune0, o.out_prune1 = out["prune0"].data_ptr(), out["prune1"].data_ptr()
        o.out_exit_layer = C.pointer(exit_layer)
    st = lib().sg_match(_ptr(kptsA), _ptr(descA), _ptr(confA), M, _ptr(kptsB), _ptr(descB), _ptr(confB), N,
                        weights.ref, L, T, _ptr(out["matches0"]), _ptr(out["scores0"]), C.byref(o))
    _lib.check(st, "sg_match")
    out["n_kernel_launches"] = count.value
    if adaptive is not None:
        out["exit_layer"] = exit_layer.value
    return out


def sg_match_batch(M, N, kptsA, descA, confA, kptsB, descB, confB, weights: Weights, L: int, T: int, *,
                   threshold: float = 0.0, image_size=None, want_matches1=True, want_logP=False,
                   want_desc=False, workspace=None, stage_events=None, timed_kernel=SG_K_NONE,
                   kernel_events=None, stream=None, graph=True, sinkhorn: str = "auto",
                   out: Optional[dict] = None) -> dict:
    """B padded pairs: kptsA [B][Mpad][2], descA [B][Mpad][D], confA [B][Mpad] (and B
    likewise); M, N: sequences of the true counts.  `out` may supply the output
    tensors (same keys and shapes) so that repeated calls reuse buffers."""
    dev = descA.device
    B, Mpad, Npad, D = kptsA.shape[0], kptsA.shape[1], kptsB.shape[1], weights.D
    for t, nm, shp in ((kptsA, "kptsA", (B, Mpad, 2)), (descA, "descA", (B, Mpad, D)), (confA, "confA", (B, Mpad)),
                       (kptsB, "kptsB", (B, Npad, 2)), (descB, "descB", (B, Npad, D)), (confB, "confB", (B, Npad))):
        _check_tensor(t, nm, torch.float32, shp)
    Ma = (C.c_int32 * B)(*[int(x) for x in M])
    Na = (C.c_int32 * B)(*[int(x) for x in N])
    if out is None:
        out = {"matches0": torch.empty((B, Mpad), dtype=torch.int32, device=dev),
               "scores0": torch.empty((B, Mpad), dtype=torch.float32, device=dev)}
        if want_matches1:
            out["matches1"] = torch.empty((B, Npad), dtype=torch.int32, device=dev)
            out["scores1"] = torch.empty((B, Npad), dtype=torch.float32, device=dev)
        if want_logP:
            out["logP"] = torch.full((B, Mpad + 1, Npad + 1), float("nan"), dtype=torch.float32, device=dev)
        if want_desc:
            out["f0"] = torch.zeros((B, Mpad, D), dtype=torch.float32, device=dev)
            out["f1"] = torch.zeros((B, Npad, D), dtype=torch.float32, device=dev)
    else:
        out = dict(out)
        for k, dt_, shp in (("matches0", torch.int32, (B, Mpad)), ("scores0", torch.float32, (B, Mpad)),
                            ("matches1", torch.int32, (B, Npad)), ("scores1", torch.float32, (B, Npad)),
                            ("logP", torch.float32, (B, Mpad + 1, Npad + 1)), ("f0", torch.float32, (B, Mpad, D)),
                            ("f1", torch.float32, (B, Npad, D))):
            if k in out:
                _check_tensor(out[k], k, dt_, shp)
    if workspace is None:
        workspace = _workspace(dev, workspace_size(weights, Mpad, Npad, B) + _transposed_extra(sinkhorn, B, Mpad, Npad))
    o, keep, count = _opts(dev, threshold=threshold, image_size=image_size, workspace=workspace,
                           m1=out.get("matches1"), s1=out.get("scores1"), fA=out.get("f0"),
                           fB=out.get("f1"), logP=out.get("logP"), logP_ld=Npad + 1,
                           stage_events=stage_events, timed_kernel=timed_kernel,
                           kernel_events=kernel_events, stream=stream, graph=graph, sinkhorn=sinkhorn)
    st = lib().sg_match_batch(B, Mpad, Npad, Ma, Na, _ptr(kptsA), _ptr(descA), _ptr(confA), _ptr(kptsB),
                              _ptr(descB), _ptr(confB), weights.ref, L, T, _ptr(out["matches0"]),
                              _ptr(out["scores0"]), C.byref(o))
    _lib.check(st, "sg_match_batch")
    out["n_kernel_launches"] = count.value
    return out


def sg_stage_encode(kpts, conf, desc, weights: Weights, image_size=(0.0, 0.0), workspace=None) -> torch.Tensor:
    n, D = desc.shape[0], weights.D
    _check_tensor(kpts, "kpts", torch.float32, (n, 2))
    _check_tensor(conf, "conf", torch.float32, (n,))
    _check_tensor(desc, "desc", torch.float32, (n, D))
    x = torch.empty((n, D), dtype=torch.float32, device=desc.device)
    if workspace is None:
        workspace = _workspace(desc.device, workspace_size(weights, n, 0, 1))
    o, keep, _ = _opts(desc.device, workspace=workspace)
    _lib.check(lib().sg_stage_encode(_ptr(kpts), _ptr(conf), _ptr(desc), n, float(image_size[0]),
                                     float(image_size[1]), weights.ref, _ptr(x), C.byref(o)),
               "sg_stage_encode")
    return x


def sg_stage_gnn(xA, xB, weights: Weights, s0: int, s1: int, workspace=None, timed_kernel=SG_K_NONE,
                 kernel_events=None, posA=None, posB=None, image_size=None, shared_similarity=False):
    """Runs stages [s0, s1) in place on float32 states xA [M][D], xB [N][D].
    posA [M][2], posB [N][2]: point positions (rotary self-attention), normalised,
    or pixels with image_size=(wA, hA, wB, hB).  shared_similarity: as for
    sg_match (bidirectional weights)."""
    M, N, D = xA.shape[0], xB.shape[0], weights.D
    _check_tensor(xA, "xA", torch.float32, (M, D))
    _check_tensor(xB, "xB", torch.float32, (N, D))
    if posA is not None:
        _check_tensor(posA, "posA", torch.float32, (M, 2))
        _check_tensor(posB, "posB", torch.float32, (N, 2))
    if workspace is None:
        workspace = _workspace(xA.device, workspace_size(weights, M, N, 1))
    o, keep, count = _opts(xA.device, workspace=workspace, timed_kernel=timed_kernel,
                           kernel_events=kernel_events, image_size=image_size,
                           shared_similarity=shared_similarity)
    _lib.check(lib().sg_stage_gnn_pos(_ptr(xA), _ptr(posA), M, _ptr(xB), _ptr(posB), N, weights.ref, s0, s1,
                                      C.byref(o)), "sg_stage_gnn_pos")
    return count.value


def sg_stage_project(x, weights: Weights) -> torch.Tensor:
    n, D = x.shape[0], weights.D
    _check_tensor(x, "x", torch.float32, (n, D))
    f = torch.empty((n, D), dtype=torch.float32, device=x.device)
    o, keep, _ = _opts(x.device)
    _lib.check(lib().sg_stage_project(_ptr(x), n, weights.ref, _ptr(f), C.byref(o)), "sg_stage_project")
    return f


def sg_stage_scores(xA, xB, weights: Weights, *, workspace=None) -> torch.Tensor:
    """The final projection of both images' states xA [M][D], xB [N][D] (fp32)
    and their bordered score matrix: Z [(M+1)][N+1] (natural log), the real
    block f_A f_B^T / sqrt(D) and the dustbin row and column holding the
    network's dustbin score."""
    M, N, D = xA.shape[0], xB.shape[0], weights.D
    _check_tensor(xA, "xA", torch.float32, (M, D))
    _check_tensor(xB, "xB", torch.float32, (N, D))
    dev = xA.device
    Z = torch.empty((M + 1, N + 1), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib().sg_stage_scores_workspace_size(M, N, D)))
    o, keep, _ = _opts(dev, workspace=workspace)
    _lib.check(lib().sg_stage_scores(_ptr(xA), M, _ptr(xB), N, weights.ref, _ptr(Z), N + 1, C.byref(o)),
               "sg_stage_scores")
    return Z


def sg_stage_match(fA, fB, alpha: float, T: int, *, threshold: float = 0.0, want_logP=True,
                   workspace=None, stage_events=None, timed_kernel=SG_K_NONE, kernel_events=None,
                   sinkhorn: str = "auto") -> dict:
    """Scores, dustbin, T Sinkhorn iterations and extraction from matching descriptors."""
    M, N, D = fA.shape[0], fB.shape[0], fA.shape[1]
    _check_tensor(fA, "fA", torch.float32, (M, D))
    _check_tensor(fB, "fB", torch.float32, (N, D))
    dev = fA.device
    out = {"matches0": torch.empty(M, dtype=torch.int32, device=dev),
           "scores0": torch.empty(M, dtype=torch.float32, device=dev),
           "matches1": torch.empty(N, dtype=torch.int32, device=dev),
           "scores1": torch.empty(N, dtype=torch.float32, device=dev)}
    if want_logP:
        out["logP"] = torch.empty((M + 1, N + 1), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib().sg_stage_match_workspace_size(M, N, D))
                               + _transposed_extra(sinkhorn, 1, M, N))
    o, keep, count = _opts(dev, threshold=threshold, workspace=workspace, m1=out["matches1"], s1=out["scores1"],
                           logP=out.get("logP"), logP_ld=N + 1, stage_events=stage_events,
                           timed_kernel=timed_kernel, kernel_events=kernel_events, sinkhorn=sinkhorn)
    _lib.check(lib().sg_stage_match(_ptr(fA), M, _ptr(fB), N, D, float(alpha), T, _ptr(out["matches0"]),
                                    _ptr(out["scores0"]), C.byref(o)), "sg_stage_match")
    out["n_kernel_launches"] = count.value
    return out


def sg_stage_match_ds(fA, fB, xA, xB, wz, bz: float, *, threshold: float = 0.0, want_logP=True,
                      workspace=None, stage_events=None, timed_kernel=SG_K_NONE, kernel_events=None) -> dict:
    """Double-softmax head from matching descriptors f and last states x (float32
    CUDA tensors [n][D]) with matchability weights wz (float32 CUDA [D]) and bz."""
    M, N, D = fA.shape[0], fB.shape[0], fA.shape[1]
    _check_tensor(fA, "fA", torch.float32, (M, D))
    _check_tensor(fB, "fB", torch.float32, (N, D))
    _check_tensor(xA, "xA", torch.float32, (M, D))
    _check_tensor(xB, "xB", torch.float32, (N, D))
    _check_tensor(wz, "wz", torch.float32, (D,))
    dev = fA.device
    out = {"matches0": torch.empty(M, dtype=torch.int32, device=dev),
           "scores0": torch.empty(M, dtype=torch.float32, device=dev),
           "matches1": torch.empty(N, dtype=torch.int32, device=dev),
           "scores1": torch.empty(N, dtype=torch.float32, device=dev)}
    if want_logP:
        out["logP"] = torch.empty((M + 1, N + 1), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib().sg_stage_match_ds_workspace_size(M, N, D)))
    o, keep, count = _opts(dev, threshold=threshold, workspace=workspace, m1=out["matches1"], s1=out["scores1"],
                           logP=out.get("logP"), logP_ld=N + 1, stage_events=stage_events,
                           timed_kernel=timed_kernel, kernel_events=kernel_events)
    _lib.check(lib().sg_stage_match_ds(_ptr(fA), _ptr(xA), M, _ptr(fB), _ptr(xB), N, D, _ptr(wz), float(bz),
                                       _ptr(out["matches0"]), _ptr(out["scores0"]), C.byref(o)),
               "sg_stage_match_ds")
    out["n_kernel_launches"] = count.value
    return out


def sg_stage_sinkhorn(Z, T: int, *, want_logP=True, workspace=None, stream=None, graph=True) -> dict:
    """T log-domain Sinkhorn iterations on the couplings Z [(M+1)][N+1] (float32
    CUDA tensor, natural log, last row and column the dustbins).  Returns the
    duals u [M+1], v [N+1] and (want_logP) logP = Z + u + v + log(M+N)."""
    if Z.dim() != 2:
        raise ValueError("Z must be [(M+1)][(N+1)]")
    M, N = Z.shape[0] - 1, Z.shape[1] - 1
    _check_tensor(Z, "Z", torch.float32)
    dev = Z.device
    out = {"u": torch.empty(M + 1, dtype=torch.float32, device=dev),
           "v": torch.empty(N + 1, dtype=torch.float32, device=dev)}
    if want_logP:
        out["logP"] = torch.empty((M + 1, N + 1), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib().sg_stage_sinkhorn_workspace_size(max(M, 0), max(N, 0))))
    o, keep, _ = _opts(dev, workspace=workspace, stream=stream, graph=graph)
    _lib.check(lib().sg_stage_sinkhorn(_ptr(Z), N + 1, M, N, int(T), _ptr(out["u"]), _ptr(out["v"]),
                                       _ptr(out.get("logP")), N + 1, C.byref(o)), "sg_stage_sinkhorn")
    return out


def sg_stage_extract(logP, *, threshold: float = 0.0, want_matches1=True, workspace=None, stream=None,
                     graph=True) -> dict:
    """Mutual-argmax extraction from the log assignment logP [(M+1)][N+1]
    (float32 CUDA tensor, natural log)."""
    if logP.dim() != 2:
        raise ValueError("logP must be [(M+1)][(N+1)]")
    M, N = logP.shape[0] - 1, logP.shape[1] - 1
    _check_tensor(logP, "logP", torch.float32)
    dev = logP.device
    out = {"matches0": torch.empty(M, dtype=torch.int32, device=dev),
           "scores0": torch.empty(M, dtype=torch.float32, device=dev)}
    if want_matches1:
        out["matches1"] = torch.empty(N, dtype=torch.int32, device=dev)
        out["scores1"] = torch.empty(N, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(dev, int(lib().sg_stage_sinkhorn_workspace_size(max(M, 0), max(N, 0))))
    o, keep, _ = _opts(dev, workspace=workspace, stream=stream, graph=graph)
    _lib.check(lib().sg_stage_extract(_ptr(logP), N + 1, M, N, float(threshold), _ptr(out["matches0"]),
                                      _ptr(out["scores0"]), _ptr(out.get("matches1")), _ptr(out.get("scores1")),
                                      C.byref(o)), "sg_stage_extract")
    return out


def sg_stage_sinkhorn_noalloc(Z, T: int, *, u=None, v=None, logP=None, stream=None) -> dict:
    """sg_stage_sinkhorn with the library's fixed scratch array instead of a
    workspace: the call allocates nothing (the outputs u [M+1], v [N+1] and
    optionally logP [(M+1)][N+1] may be passed in; omitted ones are
    allocated here, outside the call)."""
    if Z.dim() != 2:
        raise ValueError("Z must be [(M+1)][(N+1)]")
    M, N = Z.shape[0] - 1, Z.shape[1] - 1
    _check_tensor(Z, "Z", torch.float32)
    dev = Z.device
    u = torch.empty(M + 1, dtype=torch.float32, device=dev) if u is None else u
    v = torch.empty(N + 1, dtype=torch.float32, device=dev) if v is None else v
    _check_tensor(u, "u", torch.float32, (M + 1,))
    _check_tensor(v, "v", torch.float32, (N + 1,))
    if logP is not None:
        _check_tensor(logP, "logP", torch.float32, (M + 1, N + 1))
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _lib.check(lib().sg_stage_sinkhorn_noalloc(_ptr(Z), N + 1, M, N, int(T), _ptr(u), _ptr(v), _ptr(logP), N + 1,
                                               C.c_void_p(s.cuda_stream)), "sg_stage_sinkhorn_noalloc")
    out = {"u": u, "v": v}
    if logP is not None:
        out["logP"] = logP
    return out
