"""The allocation-free Sinkhorn stage (sg_stage_sinkhorn_noalloc, for callers
that cannot allocate) against sg_stage_sinkhorn, through the C ABI (GPU):
two calls in a row, the second with a smaller input, each equal to the
allocating entry point's output (the same kernels on the same inputs: u, v
and logP are expected bitwise, and held to the 1e-3 log-assignment bar)."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
from parity import dev, host

pytestmark = pytest.mark.gpu

sg = pytest.importorskip("learned_sparse_feature_amd")


def _couplings(M, N, seed):
    fA, fB = synth.random_matching_descriptors(M, N, 256, seed=seed)
    S = fA.astype(np.float64) @ fB.astype(np.float64).T / 16.0
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    Z = np.empty((M + 1, N + 1))
    Z[:M, :N] = S
    Z[M, :] = rng.uniform(-2, 2, N + 1)
    Z[:, N] = rng.uniform(-2, 2, M + 1)
    return np.ascontiguousarray(Z, np.float32)


def _noalloc(Zd, T):
    M, N = Zd.shape[0] - 1, Zd.shape[1] - 1
    u = torch.full((M + 1,), np.nan, dtype=torch.float32, device="cuda")
    v = torch.full((N + 1,), np.nan, dtype=torch.float32, device="cuda")
    logP = torch.full((M + 1, N + 1), np.nan, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    st = sg.lib().sg_stage_sinkhorn_noalloc(C.c_void_p(Zd.data_ptr()), N + 1, M, N, T, C.c_void_p(u.data_ptr()),
                                            C.c_void_p(v.data_ptr()), C.c_void_p(logP.data_ptr()), N + 1,
                                            C.c_void_p(stream))
    assert st == 0, sg.lib().sg_last_error()
    torch.cuda.synchronize()
    return {"u": host(u), "v": host(v), "logP": host(logP)}


def test_noalloc_equals_sg_stage_sinkhorn_on_two_calls():
    assert torch.cuda.is_available()
    for (M, N, T, seed) in ((1500, 1100, 100, 3), (300, 77, 40, 4)):
        Zd = dev(_couplings(M, N, seed))
        a = _noalloc(Zd, T)
        ref = sg.sg_stage_sinkhorn(Zd, T, graph=False)
        torch.cuda.synchronize()
        for k in ("u", "v", "logP"):
            d = float(np.abs(a[k] - host(ref[k])).max())
            print(f"{M}x{N} T={T}: {k} max diff {d:.2e}, bitwise {np.array_equal(a[k], host(ref[k]))}")
            assert np.isfinite(a[k]).all() and d <= 1e-3, (M, N, k, d)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """A workspace beyond the fixed array is refused on the host, before any
    HIP call, with nothing enqueued."""
    f = C.c_void_p(0x1000)
    st = sg.lib().sg_stage_sinkhorn_noalloc(f, 4097, 4096, 4096, 10, f, f, None, 0, None)
    assert st == -2 and b"scratch" in sg.lib().sg_last_error()
