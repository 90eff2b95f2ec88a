"""Benchmark of the SuperGlue matching forward pass on one MI355X.

One step = one whole forward pass (encoder, 2L attention stages, final
projection, scores + dustbin, T Sinkhorn iterations, mutual-argmax
extraction) over one synthetic 1024 x 1024 pair (D = 256, H = 4, L = 9,
T = 100, bf16 GNN operands with fp32 accumulation, fp32 Sinkhorn), inputs
resident in HBM before the timed region.  Prints one JSON line on stdout;
progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--head ds]

--head ds replaces the Sinkhorn head by the double-softmax + matchability
head (section 2.4 of the LightGlue review) on the same network and pair;
--cross bidirectional gives the cross stages one shared query/key projection
(section 2.3 of the review); --rope rotates q and k of the self stages by the
keypoints' positions (section 2.2).  --adaptive adds the adaptive depth /
width measurements (sections 2.6 and 2.7) beside the headline number.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "image pairs/sec (L=9 GNN + T=100 Sinkhorn) at M=N=1024; MFMA util %"
METRIC_DS = "image pairs/sec (L=9 GNN + double-softmax head) at M=N=1024"
PEAK = {"hbm_GBps": 8000.0, "bf16_TFLOPs": 2500.0, "f32_TFLOPs": 157.3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_launches(cfg, M, N, cross="standard"):
    """(label, operand dtype, algorithmic flops) of every GEMM-class launch of
    one pass, in launch order (real rows only): per stage the QKV projection,
    the first MLP layer over [x || a] (the merge projection folded in) and the
    second with the residual, then the final projection and the scores.  The
    merge fold itself (W1[:, D:] Wm for every stage, weights only) runs in
    the encoder's launch and is not a GEMM-class launch; the merge projection
    it removes from every stage (2 (M+N) D^2) is counted nowhere.
    Bidirectional cross stages project qk | v (2D outputs) instead of q | k | v."""
    R, D, S = M + N, cfg.D, 2 * cfg.L
    out = []
    for s in range(S):
        out.append(("qkv", cfg.dtype, 2.0 * R * D * (2 if (s % 2 == 1 and cross == "bidirectional") else 3) * D))
        out.append(("mlp1", cfg.dtype, 2.0 * R * 2 * D * 2 * D))
        out.append(("mlp2_residual", cfg.dtype, 2.0 * R * 2 * D * D))
    out.append(("final_projection", cfg.dtype, 2.0 * R * D * D))
    out.append(("scores", "f32", 2.0 * M * N * D))
    return out


def gemm_bytes(cfg, M, N, label, pairs=1):
    """Algorithmic HBM bytes of one GEMM-class launch over `pairs` pairs:
    activations read once and outputs written once per pair, the weights read
    once per launch (bf16 networks keep q, k, v, the MLP hidden layer and a
    copy of the residual stream in bf16; the residual stream itself and the
    final descriptors are fp32)."""
    R, D = M + N, cfg.D
    os_ = 2 if cfg.dtype == "bf16" else 4
    if label == "qkv":
        return pairs * (R * D * os_ + 3 * R * D * os_) + 3 * D * D * os_
    if label == "mlp1":
        return pairs * (2 * R * D * os_ + 2 * R * D * os_) + 4 * D * D * os_
    if label == "mlp2_residual":
        return pairs * (2 * R * D * os_ + 2 * R * D * 4 + (R * D * 2 if os_ == 2 else 0)) + 2 * D * D * os_
    if label == "final_projection":
        return pairs * (R * D * 4 + R * D * 4) + D * D * os_
    if label == "scores":
        return pairs * (R * D * 4 + M * N * 4)
    raise ValueError(label)


def own_roofline(flops, nbytes, us):
    """The launch against its own roofline: the larger of its flops at the
    bf16 dense peak and its bytes at the HBM peak."""
    t_mfma = flops / (PEAK["bf16_TFLOPs"] * 1e12) * 1e6
    t_hbm = nbytes / (PEAK["hbm_GBps"] * 1e9) * 1e6
    floor = max(t_mfma, t_hbm)
    return {"bound": "mfma" if t_mfma >= t_hbm else "hbm", "roofline_us": round(floor, 2),
            "frac_of_roofline": round(floor / us, 4)}


def gemm_flops(cfg, M, N, cross="standard"):
    """(operand dtype, flops) of every GEMM-class launch (see gemm_launches)."""
    return [(d, f) for _, d, f in gemm_launches(cfg, M, N, cross)]


def attention_flops(cfg, M, N):
    """Per launch (stage): self 4D(M^2+N^2), cross 8DMN (QK^T and PV)."""
    D = cfg.D
    return [4.0 * D * (M * M + N * N) if s % 2 == 0 else 8.0 * D * M * N for s in range(2 * cfg.L)]


def sinkhorn_bytes(M, N, T):
    """Algorithmic bytes per Sinkhorn launch.  The method's work per
    iteration is one fused fp32 read of the (M+1)x(N+1) couplings,
    4 (M+1)(N+1) bytes; the two-sweep schedule spends two launches on an
    iteration (rows of Z, then rows of its transpose), so each launch is
    credited with half of it.  Reading Z and Z^T in full is the schedule's
    own extra traffic (traffic_ratio ~2), not algorithmic work."""
    return [2.0 * (M + 1) * (N + 1)] * (2 * T)


def ds_bytes(M, N, D):
    """One launch of the double-softmax statistics: Z and its transpose read
    once, every point's fp32 state read once, u, v and the dustbin entries
    written."""
    return [8.0 * M * N + 4.0 * D * (M + N) + 8.0 * (M + N)]


def profiled_traffic(kernel, profile="superglue_pair1024_bf16_hbm_traffic.txt"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when it is missing or the kernel's source has
    changed since the counters were taken (the summary records its hash)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    for line in open(path):
        if not line.startswith("traffic_bytes_per_launch"):
            continue
        kv = dict(x.split("=", 1) for x in line.split()[1:])
        if kernel not in kv.get("kernel", ""):
            continue
        src = os.path.join(ROOT, kv["source"])
        if not os.path.exists(src):
            return None
        if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != kv["sha256_16"]:
            return None
        return float(kv["bytes"])
    return None


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pass_flops(cfg, M, N, cross="standard"):
    """Algorithmic flops of one pass as the method states it (encoder, GNN
    with its merge projections, final projection, scores): the work of the
    plain oracle, which forms every merge projection instead of folding it."""
    widths = [3] + list(cfg.enc) + [cfg.D]
    enc = 2.0 * (M + N) * sum(a * b for a, b in zip(widths[:-1], widths[1:]))
    gemm = sum(f for _, _, f in gemm_launches(cfg, M, N, cross))
    merge = 2.0 * (M + N) * cfg.D * cfg.D * 2 * cfg.L
    return enc + gemm + merge + sum(attention_flops(cfg, M, N))


def cpu_baseline(cfg, w, pair, head="sinkhorn"):
    """The plain C oracle, single-threaded, on a bounded sample of the pass:
    the encoder of both images, one GNN layer (stage 0, self, and stage 1,
    cross), the final projection and the whole head (scores, T Sinkhorn
    iterations, extraction).  The L layers of the pass have identical shapes
    and work, so the per-pair time is encoder + L x layer + head."""
    import numpy as np

    import oracle
    oracle.set_threads(1)
    t = {}
    t0 = time.perf_counter()
    xs = []
    for side in ("0", "1"):
        wd, ht = pair["image_size" + side]
        kn = oracle.normalize_keypoints(pair["kpts" + side], wd, ht)
        xs.append(np.asarray(pair["desc" + side], np.float64) + oracle.keypoint_encoder(kn, pair["conf" + side], w["enc"]))
    t["encoder"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    xa, xb = oracle.attentional_gnn(xs[0], xs[1], w["stages"][:2], w["H"])
    t["layer"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    f0 = oracle.final_projection(xa, w["Wf"], w["bf"])
    f1 = oracle.final_projection(xb, w["Wf"], w["bf"])
    if head == "ds":
        oracle.double_softmax_from_descriptors(f0, f1, xa, xb, w["wz"], w["bz"])
    else:
        oracle.match_from_descriptors(f0, f1, w["alpha"], cfg.T)
    t["head"] = time.perf_counter() - t0
    oracle.set_threads(0)
    per_pair = t["encoder"] + cfg.L * t["layer"] + t["head"]
    flops = pass_flops(cfg, cfg.M, cfg.N)
    sampled = sum(t.values())
    return {"value": round(1.0 / per_pair, 5), "unit": "pairs/s", "cores": 1, "kind": "oracle",
            "threads": 1, "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
            "s_per_pair": round(per_pair, 2), "gflops_per_s": round(flops / per_pair / 1e9, 3),
            "pass_gflop": round(flops / 1e9, 2),
            "sample": (f"plain C float64 oracle (oracle/sg_oracle.c), one thread, on the 1024x1024 pair: encoder "
                       f"{t['encoder']:.2f} s, one self + cross layer {t['layer']:.2f} s (x L={cfg.L}), final "
                       f"projection + {'double-softmax head' if head == 'ds' else f'scores + T={cfg.T} Sinkhorn'} + "
                       f"extraction {t['head']:.2f} s; {sampled:.1f} s sampled")}


def profiled_mfma_busy(profile="superglue_pair1024_bf16_mfma_busy.txt"):
    """Counter-based MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES) per kernel of
    the one-pair pass from the committed rocprofv3 summary, or None when it is
    missing or a kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    out = {}
    for line in open(path):
        if not line.startswith("mfma_busy_frac"):
            continue
        kv = dict(x.split("=", 1) for x in line.split()[1:])
        src = os.path.join(ROOT, kv["source"])
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != kv["sha256_16"]:
            return None
        out[kv["class"]] = float(kv["busy"])
    return out or None


def adaptive_bench(args, cfg, dev, sg, synth, np, torch):
    """Adaptive depth and width of one pair with the double-softmax head:
    the same pass with the confidence forced low (no exit: the per-layer
    statistics and synchronisations are pure overhead), forced high from a
    given layer (exit after it), and point pruning on a 2048 x 2048 pair whose
    matchability drops about a quarter of the points after layer 0.  Adaptive
    calls run eagerly, so the plain pass is timed eagerly too."""
    import copy
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / reps

    reps = max(5, min(30, args.steps // 3))
    base = synth.make_weights(cfg, adaptive=True, cross=args.cross, rope=args.rope)
    pair = synth.make_pair(cfg)
    t = [torch.from_numpy(pair[k]).to(dev) for k in keys]
    img = (*pair["image_size0"], *pair["image_size1"])
    res = {"pair": "1024x1024, L=9"}

    def with_conf(w, first_confident):
        w = copy.deepcopy(w)
        w["conf"] = [(0 * wc, 40.0 if l >= first_confident else -40.0) for l, (wc, _) in enumerate(w["conf"])]
        return sg.pack_weights(w, device=dev, head="ds")

    Wn = with_conf(base, cfg.L)  # never confident
    res["plain_graph_ms"] = round(timed(lambda: sg.sg_match(*t, Wn, cfg.L, cfg.T, image_size=img), reps), 4)
    res["plain_eager_ms"] = round(timed(lambda: sg.sg_match(*t, Wn, cfg.L, cfg.T, image_size=img, graph=False), reps), 4)
    res["adaptive_no_exit_ms"] = round(timed(lambda: sg.sg_match(*t, Wn, cfg.L, cfg.T, image_size=img,
                                                                  adaptive={"prune": False}), reps), 4)
    for k in (1, 4):
        Wk = with_conf(base, k)
        o = sg.sg_match(*t, Wk, cfg.L, cfg.T, image_size=img, adaptive={"prune": False})
        assert o["exit_layer"] == k, o["exit_layer"]
        res[f"exit_after_layer_{k}_ms"] = round(timed(lambda: sg.sg_match(*t, Wk, cfg.L, cfg.T, image_size=img,
                                                                           adaptive={"prune": False}), reps), 4)
    # pruning: states frozen through layer 0's decision are not needed; the
    # matchability of layer 0 reads one descriptor channel scaled so that a
    # quarter of the points are confidently unmatchable
    big = synth.make_pair(cfg, M=2048, N=2048, seed=77)
    tb = [torch.from_numpy(big[k]).to(dev) for k in keys]
    wp = copy.deepcopy(base)
    e = np.eye(cfg.D, dtype=np.float32)
    wp["conf"] = [(2000.0 * e[0], 0.0)] + [(0 * wc, -40.0) for wc, _ in wp["conf"][1:]]
    wp["heads"] = [(h[0], h[1], 2000.0 * e[1] if l == 0 else 0 * h[2], 0.0 if l == 0 else 40.0)
                   for l, h in enumerate(wp["heads"])]
    Wp = sg.pack_weights(wp, device=dev, head="ds")
    ws = torch.empty(sg.workspace_size(Wp, 2048, 2048, 1), dtype=torch.uint8, device=dev)
    o = sg.sg_match(*tb, Wp, cfg.L, cfg.T, image_size=img, adaptive={}, workspace=ws)
    kept = (int((o["prune0"] > 1).sum().item()), int((o["prune1"] > 1).sum().item()))
    res["prune_pair"] = "2048x2048, L=9, layer 0 drops confident unmatchable points"
    res["prune_kept_points"] = kept
    res["prune_plain_eager_ms"] = round(timed(lambda: sg.sg_match(*tb, Wp, cfg.L, cfg.T, image_size=img,
                                                                   graph=False, workspace=ws), reps), 4)
    res["prune_adaptive_ms"] = round(timed(lambda: sg.sg_match(*tb, Wp, cfg.L, cfg.T, image_size=img,
                                                                adaptive={}, workspace=ws), reps), 4)
    log(f"adaptive: {res}")
    return res


def batch_kernels(args, cfg, sg, np, torch, bstep, B, M, N, ds):
    """Per kernel class of one batched call: launches, time, and the fraction
    of the MFMA or HBM peak.  Launches here run 25-200 us, so the ~2.5 us of
    the events bracketing each launch is left in."""
    classes = {"gemm": sg.SG_K_GEMM, "attention": sg.SG_K_ATTENTION, "sinkhorn": sg.SG_K_SINKHORN}
    res = {}
    evs = sg.make_events(1024)
    for name, kind in classes.items():
        tot, nl = None, None
        reps = 3
        for _ in range(reps):
            o = bstep(timed_kernel=kind, kernel_events=evs)
            torch.cuda.synchronize()
            nl = o["n_kernel_launches"]
            assert 0 < nl < 512, (name, nl)
            d = np.array([evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(nl)])
            tot = d if tot is None else tot + d
        dur_us = tot / reps * 1e3
        r = {"launches": nl, "total_us": round(float(dur_us.sum()), 1), "avg_us": round(float(dur_us.mean()), 2)}
        if name == "gemm":
            labs = gemm_launches(cfg, M, N, args.cross)
            assert nl == len(labs), ("batched GEMM launches", nl, len(labs))
            mult = (lambda lab: B)
            bf = [(f * mult(lab), d) for (lab, dt_, f), d in zip(labs, dur_us) if dt_ == "bf16"]
            ach = float(sum(f for f, _ in bf) / sum(d for _, d in bf) / 1e6)
            r.update(achieved_TFLOPs_bf16=round(ach, 1), frac_mfma=round(ach / PEAK["bf16_TFLOPs"], 4))
            per = {}
            for (lab, _, f), d in zip(labs, dur_us):
                per.setdefault(lab, []).append((f * mult(lab), d))
            r["per_launch_kind"] = {}
            for k, v in per.items():
                if k == "scores":
                    continue
                avg = float(np.mean([d for _, d in v]))
                fl = float(np.mean([f for f, _ in v]))
                nb = gemm_bytes(cfg, M, N, k, B)
                r["per_launch_kind"][k] = {
                    "launches": len(v), "avg_us": round(avg, 2),
                    "frac_mfma": round(float(sum(f for f, _ in v) / sum(d for _, d in v) / 1e6 / PEAK["bf16_TFLOPs"]), 4),
                    "algorithmic_bytes": nb, **own_roofline(fl, nb, avg)}
        elif name == "attention":
            fl = attention_flops(cfg, M, N)
            assert nl == len(fl), ("batched attention launches", nl, len(fl))
            ach = float(sum(fl) * B / dur_us.sum() / 1e6)
            r.update(achieved_TFLOPs=round(ach, 1), frac_mfma=round(ach / PEAK["bf16_TFLOPs"], 4))
            # q, k, v read and the messages written once per stage
            nb = 4 * (M + N) * cfg.D * (2 if cfg.dtype == "bf16" else 4) * B
            r.update(algorithmic_bytes_per_launch=nb,
                     **own_roofline(float(np.mean(fl)) * B, nb, float(dur_us.mean())))
        elif ds:
            r["kernel"] = "k_ds_stats"
            byt = ds_bytes(M, N, cfg.D)[0] * B
            r.update(achieved_GBps=round(float(byt / dur_us.sum() / 1e3), 1),
                     frac_hbm=round(float(byt / dur_us.sum() / 1e3) / PEAK["hbm_GBps"], 4))
        else:
            # one read of every pair's couplings per iteration, over the time
            # of the iteration's launches (row pass + column reduction)
            byt = 4.0 * (M + 1) * (N + 1) * B * cfg.T
            r.update(bytes_per_iteration=4.0 * (M + 1) * (N + 1) * B,
                     achieved_GBps=round(float(byt / dur_us.sum() / 1e3), 1),
                     frac_hbm=round(float(byt / dur_us.sum() / 1e3) / PEAK["hbm_GBps"], 4))
            if nl == cfg.T + 1:
                # one-pass schedule, fused iterations: each launch reduces the
                # previous block partials into v (every workgroup of a pair),
                # updates u and writes its own partials from one read of Z;
                # one column reduction follows the last iteration
                it, fin = dur_us[:cfg.T], dur_us[cfg.T]
                per_it = 4.0 * (M + 1) * (N + 1) * B
                r["iteration"] = {"kernel": "k_sink_iter", "launches": cfg.T, "avg_us": round(float(it.mean()), 2),
                                  "algorithmic_bytes": per_it,
                                  "achieved_GBps": round(float(per_it / it.mean() / 1e3), 1),
                                  "frac_hbm": round(float(per_it / it.mean() / 1e3 / PEAK["hbm_GBps"]), 4)}
                r["final_column_reduction_us"] = round(float(fin), 2)
        res[name] = r
    return res


def latency_percentiles(step, sg, torch, n):
    """p10 / p50 / p90 of single-pass latency: each pass bracketed by its own
    pair of events on the library's stream, one pass at a time."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    ts = []
    for a, b in evs:
        a.record()
        step()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    q = lambda f: round(ts[min(n - 1, int(f * n))], 4)
    return {"passes": n, "p10_ms": q(0.1), "p50_ms": q(0.5), "p90_ms": q(0.9)}


def graph_iteration_us(sg, torch, step, steps, T, reps=3):
    """Microseconds per Sinkhorn iteration inside the replayed graph of the
    pass: (time of a pass with T iterations - time of the same pass with
    none) / T, each the median over `reps` runs of `steps` back-to-back
    replays bracketed by HIP events on the current stream (the library's)."""
    if T <= 0:
        return None

    def per_pass(t_iter):
        for _ in range(3):  # eager, capture, replay
            step(T=t_iter)
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                step(T=t_iter)
            e.record()
            e.synchronize()
            out.append(a.elapsed_time(e) * 1e3 / steps)
        return sorted(out)[reps // 2]
    return (per_pass(T) - per_pass(0)) / T


def concurrent_calls(args, sg, torch, W, t, img, cfg, M, N, dev, calls=400):
    """Single-pair calls (the headline's pair, one per call) spread round-robin
    over S streams of default priority, each stream with its own workspace
    and outputs (so each replays its own captured graph) and the inputs
    shared: pairs/s over `calls` calls, and the mean time from a call's
    enqueue to its end on its stream.  Context for serving independent
    requests; the headline value stays one call in flight."""
    res = {}
    for S in sorted({2, args.streams} if args.streams > 2 else {2}):
        streams = [torch.cuda.Stream(device=dev) for _ in range(S)]
        wss = [torch.empty(sg.workspace_size(W, M, N, 1), dtype=torch.uint8, device=dev) for _ in range(S)]
        outs = [{"matches0": torch.empty(M, dtype=torch.int32, device=dev),
                 "scores0": torch.empty(M, dtype=torch.float32, device=dev)} for _ in range(S)]

        def call(i):
            sg.sg_match(*t, W, cfg.L, cfg.T, image_size=img, workspace=wss[i], out=outs[i], stream=streams[i],
                        sinkhorn=args.sinkhorn)
        for _ in range(3):  # eager, capture, replay
            for i in range(S):
                call(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(calls):
            call(k % S)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        # per-call time with S calls in flight: each stream's calls run back to
        # back, so a call takes the stream's wall time over its calls
        res[f"streams_{S}"] = {"calls": calls, "pairs_per_s": round(calls / dt, 1),
                               "ms_per_call_per_stream": round(1e3 * dt / (calls / S), 3)}
        same = all(bool(torch.equal(outs[0]["matches0"], o["matches0"])) for o in outs[1:])
        res[f"streams_{S}"]["outputs_equal_across_streams"] = same
    return res


def workload_names(synth, spec):
    """Workload names from a comma-separated list of names or of positions in
    synth.WORKLOADS."""
    table = list(synth.WORKLOADS)
    out = []
    for c in (c.strip() for c in spec.split(",")):
        if not c:
            continue
        name = table[int(c)] if c.isdigit() else c
        if name not in synth.WORKLOADS:
            raise SystemExit(f"unknown workload {c!r}; one of {table}")
        out.append(name)
    return out


def per_config(sg, synth, np, torch, dev, names_run, reps=10):
    """The pass of each named workload (single pairs one per call, the ragged
    32-pair batch per call): median wall time per call over graph replays and
    the stage times of an eager pass with stage events (context beside the
    headline)."""
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")
    names = ["encoder", "gnn", "projection_scores", "sinkhorn", "extraction"]
    res = {}
    for wl in names_run:
        cfg = synth.WORKLOADS[wl]
        w = synth.make_weights(cfg)
        W = sg.pack_weights(w, device=dev)
        if cfg.batch > 1:
            b = synth.make_batch(cfg)
            t = [torch.from_numpy(b[k]).to(dev) for k in keys]
            img = (*b["image_size0"], *b["image_size1"])
            Ms, Ns = [int(x) for x in b["M"]], [int(x) for x in b["N"]]
            coupling_bytes = sum(4.0 * (m + 1) * (n + 1) for m, n in zip(Ms, Ns))
            ws = torch.empty(sg.workspace_size(W, cfg.pad, cfg.pad, cfg.batch), dtype=torch.uint8, device=dev)
            bbufs = {"matches0": torch.empty((cfg.batch, cfg.pad), dtype=torch.int32, device=dev),
                     "scores0": torch.empty((cfg.batch, cfg.pad), dtype=torch.float32, device=dev)}

            def call(**kw):
                return sg.sg_match_batch(Ms, Ns, *t, W, cfg.L, cfg.T, image_size=img, workspace=ws,
                                         want_matches1=False, out=bbufs, **kw)
            pairs = cfg.batch
        else:
            pair = synth.make_pair(cfg)
            coupling_bytes = 4.0 * (cfg.M + 1) * (cfg.N + 1)
            t = [torch.from_numpy(pair[k]).to(dev) for k in keys]
            img = (*pair["image_size0"], *pair["image_size1"])
            ws = torch.empty(sg.workspace_size(W, cfg.M, cfg.N, 1), dtype=torch.uint8, device=dev)
            bufs = {"matches0": torch.empty(cfg.M, dtype=torch.int32, device=dev),
                    "scores0": torch.empty(cfg.M, dtype=torch.float32, device=dev)}

            def call(**kw):
                return sg.sg_match(*t, W, cfg.L, cfg.T, image_size=img, workspace=ws, out=bufs, **kw)
            pairs = 1
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            e.record()
            e.synchronize()
            ts.append(a.elapsed_time(e))
        ev = sg.make_events(sg.SG_N_STAGE_EVENTS)
        acc = np.zeros(sg.SG_N_STAGE_EVENTS - 1)
        for _ in range(3):
            call(stage_events=ev)
            torch.cuda.synchronize()
            acc += [ev[i].elapsed_time(ev[i + 1]) for i in range(sg.SG_N_STAGE_EVENTS - 1)]
        med = float(np.median(ts))
        res[wl] = {"M": int(cfg.M) if pairs == 1 else "U{256..2048}", "N": int(cfg.N) if pairs == 1 else "U{256..2048}",
                   "pairs_per_call": pairs, "dtype": cfg.dtype, "T": cfg.T, "L": cfg.L,
                   "ms_per_call_p50": round(med, 4), "pairs_per_s": round(pairs / med * 1e3, 2),
                   "stages_ms": {n: round(float(v / 3), 4) for n, v in zip(names, acc)}}
        # the Sinkhorn stage against one fused read of the couplings per
        # iteration (the stage's T iterations and its final reduction)
        sk_us = float(acc[names.index("sinkhorn")] / 3) * 1e3
        if cfg.T > 0 and sk_us > 0:
            res[wl]["sinkhorn"] = {"us_per_iteration": round(sk_us / cfg.T, 3),
                                   "bytes_per_iteration": coupling_bytes,
                                   "frac_hbm": round(coupling_bytes * cfg.T / (sk_us * 1e-6) / 1e9 / PEAK["hbm_GBps"], 4)}
        log(f"{wl}: {res[wl]}")
    return res


def launch_floor(torch, n=200, reps=10):
    """Per-launch time of graph-replayed chains of n dependent launches: a
    one-element add (the dispatch floor) and a row sum over a 1025 x 1024
    fp32 matrix (the size of a Sinkhorn sweep's read).  torch's own kernels
    serve as the reference; only the dependency and the replay matter."""
    out = {}
    dev = torch.device("cuda:0")
    x = torch.zeros(1, device=dev)
    Z = torch.randn(1025, 1024, device=dev)
    r = torch.empty(1025, device=dev)
    for name, fn in (("empty_us", lambda: x.add_(1.0)), ("row_sum_4MB_us", lambda: torch.sum(Z, dim=1, out=r))):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        best = 1e9
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            best = min(best, a.elapsed_time(b))
        out[name] = round(1e3 * best / n, 3)
    return out


def summarize_trace(path, pattern):
    """Dispatch durations and the gaps between consecutive dispatches of the
    kernels whose name contains `pattern`, from a rocprofv3 kernel trace
    (run_kernel_trace.csv): gap = next dispatch's start - this one's end,
    for consecutive dispatches that both match and lie within 20 us (the
    back-to-back launches of one replayed pass)."""
    import csv
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    dur = [(e - s) / 1e3 for s, e, n in rows if pattern in n]
    gaps = [(rows[i + 1][0] - rows[i][1]) / 1e3 for i in range(len(rows) - 1)
            if pattern in rows[i][2] and pattern in rows[i + 1][2] and rows[i + 1][0] - rows[i][1] < 20000]
    import statistics as st
    return {"kernel": pattern, "dispatches": len(dur), "exec_mean_us": round(st.mean(dur), 3),
            "exec_median_us": round(st.median(dur), 3), "gap_pairs": len(gaps),
            "gap_mean_us": round(st.mean(gaps), 3) if gaps else None,
            "gap_median_us": round(st.median(gaps), 3) if gaps else None,
            "period_median_us": round(st.median(dur) + st.median(gaps), 3) if gaps else None}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--batch", type=int, default=32,
                    help="also time sg_match_batch on this many 1024x1024 pairs per call (0: skip)")
    ap.add_argument("--sinkhorn", choices=["auto", "two", "one"], default="auto",
                    help="Sinkhorn schedule (default: chosen by problem size)")
    ap.add_argument("--head", choices=["sinkhorn", "ds"], default="sinkhorn",
                    help="matching head: Sinkhorn (default) or double softmax + matchability")
    ap.add_argument("--cross", choices=["standard", "bidirectional"], default="standard",
                    help="cross-attention of the odd stages")
    ap.add_argument("--rope", action="store_true", help="rotary position encoding in self-attention")
    ap.add_argument("--shared-similarity", action="store_true",
                    help="(--cross bidirectional) each cross stage forms its similarity once for both directions; "
                         "the single-pair line only (no batch, no per-kernel timing)")
    ap.add_argument("--adaptive", action="store_true",
                    help="also time adaptive depth / width (forced exits and pruning) with the double-softmax head")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration context timings")
    ap.add_argument("--configs", default="pair10x12_f32,pair512_f32,pair2048x1536_f32,ragged32_bf16",
                    help="comma-separated workloads of the per-configuration timings: names from synth.WORKLOADS, "
                         "or their positions in it (0-4)")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="before the steps, copy this many MiB with a plain device copy (counter scaling)")
    ap.add_argument("--streams", type=int, default=4,
                    help="also time single-pair calls spread over 2..this many streams (context; 1: skip)")
    ap.add_argument("--no-launch-floor", action="store_true",
                    help="skip the dependent-launch floor of a replayed graph (launch_floor_us)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("CSV", "KERNEL"),
                    help="print execution and gap statistics of KERNEL from a rocprofv3 kernel trace and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(json.dumps(summarize_trace(*args.summarize_trace)))
        return
    if args.gpus != 1:
        log(f"bench.py runs on one GPU only: the matching pass is measured on a single MI355X "
            f"(pairs are independent: several GPUs would each match their own share of the pairs). --gpus {args.gpus} refused.")
        sys.exit(2)
    if args.shared_similarity:
        if args.cross != "bidirectional":
            log("--shared-similarity needs --cross bidirectional")
            sys.exit(2)
        args.batch, args.no_kernel_timing = 0, True

    import numpy as np
    import torch

    import learned_sparse_feature_amd as sg
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = synth.WORKLOADS["pair1024_bf16"]
    w = synth.make_weights(cfg, cross=args.cross, rope=args.rope)
    pair = synth.make_pair(cfg)
    W = sg.pack_weights(w, device=dev, head=args.head)
    ds = args.head == "ds"
    # launches and algorithmic bytes of the head's normalisation kernels
    norm_work = ds_bytes(cfg.M, cfg.N, cfg.D) if ds else sinkhorn_bytes(cfg.M, cfg.N, cfg.T)
    keys = ("kpts0", "desc0", "conf0", "kpts1", "desc1", "conf1")
    t = [torch.from_numpy(pair[k]).to(dev) for k in keys]
    img = (*pair["image_size0"], *pair["image_size1"])
    M, N = cfg.M, cfg.N
    ws = torch.empty(sg.workspace_size(W, M, N, 1) + 4 * M * N, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibrate_copy} MiB read + written")

    # outputs are preallocated so that every step is the same call (replayed as a HIP graph)
    bufs = {"matches0": torch.empty(M, dtype=torch.int32, device=dev),
            "scores0": torch.empty(M, dtype=torch.float32, device=dev)}

    def step(T=None, **kw):
        return sg.sg_match(*t, W, cfg.L, cfg.T if T is None else T, image_size=img, workspace=ws, out=bufs,
                           sinkhorn=args.sinkhorn,
                           shared_similarity=args.shared_similarity, **kw)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = 1e3 * dt / args.steps
    value = args.steps / dt
    log(f"{ms:.3f} ms/step, {value:.1f} pairs/s; matches {(out['matches0'] >= 0).sum().item()}")
    latency = latency_percentiles(step, sg, torch, max(10, min(100, args.steps)))
    log(f"latency: {latency}")
    concurrent = None
    if args.streams > 1:
        concurrent = concurrent_calls(args, sg, torch, W, t, img, cfg, M, N, dev)
        log(f"concurrent single-pair calls: {concurrent}")

    # per-stage times (a separate pass: stage events perturb the stream slightly)
    stages = {}
    ev = sg.make_events(sg.SG_N_STAGE_EVENTS)
    nrep = max(3, min(20, args.steps))
    acc = np.zeros(sg.SG_N_STAGE_EVENTS - 1)
    for _ in range(nrep):
        step(stage_events=ev)
        torch.cuda.synchronize()
        acc += [ev[i].elapsed_time(ev[i + 1]) for i in range(sg.SG_N_STAGE_EVENTS - 1)]
    names = ["encoder", "gnn", "projection_scores", "ds_stats" if ds else "sinkhorn", "extraction"]
    stages = {n: round(float(v / nrep), 4) for n, v in zip(names, acc)}
    log(f"stages (ms): {stages}")

    kernels = {}
    roofline = None
    mfma_util = None
    if not args.no_kernel_timing:
        specs = {
            "sinkhorn": (sg.SG_K_SINKHORN, norm_work),
            "attention": (sg.SG_K_ATTENTION, attention_flops(cfg, M, N)),
            "gemm": (sg.SG_K_GEMM, [f for _, f in gemm_flops(cfg, M, N, args.cross)]),
        }
        durs = {}
        for name, (kind, work) in specs.items():
            nl = len(work)
            evs = sg.make_events(2 * nl)
            reps = max(2, min(10, args.steps))
            tot = np.zeros(nl)
            for _ in range(reps):
                o = step(timed_kernel=kind, kernel_events=evs)
                torch.cuda.synchronize()
                assert o["n_kernel_launches"] == nl, (name, o["n_kernel_launches"], nl)
                tot += [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(nl)]
            dur = tot / reps  # ms per launch
            durs[name] = dur
            kernels[name] = {"launches": nl, "avg_us": round(float(dur.mean() * 1e3), 3),
                             "total_us": round(float(dur.sum() * 1e3), 2)}
            if name == "sinkhorn":
                kernels[name]["achieved_GBps"] = round(float(sum(work) / dur.sum() / 1e6), 1)
            elif name == "attention":
                kernels[name]["achieved_TFLOPs"] = round(float(sum(work) / dur.sum() / 1e9), 2)
            else:
                bf = [(f, d) for (dt_, f), d in zip(gemm_flops(cfg, M, N, args.cross), dur) if dt_ == "bf16"]
                kernels[name]["achieved_TFLOPs_bf16"] = round(float(sum(f for f, _ in bf) / sum(d for _, d in bf) / 1e9), 2)
            log(f"{name}: {kernels[name]}")
        # Sinkhorn sweeps run back to back: their average launch time is the
        # Sinkhorn stage time (stage events, no event between the launches)
        # over the 2T launches.  Bracketing each launch with its own pair of
        # events adds the event and dispatch latency (~2.5 us) to every launch.
        nn = len(norm_work)
        per = stages["sinkhorn"] * 1e3 / nn if not ds else None
        kernels["sinkhorn"]["bracketed_avg_us"] = kernels["sinkhorn"]["avg_us"]
        if ds:
            kernels["ds_stats"] = kernels.pop("sinkhorn")
            kernels["ds_stats"]["kernel"] = "k_ds_stats (row / column lse over Z and Z^T + matchability)"
            tr = profiled_traffic("k_ds_stats", "superglue_pair1024_bf16_ds_head_hbm_traffic.txt")
            kernels["ds_stats"]["traffic"] = None if tr is None else round(tr)
        # The bracketing latency is removed from the other classes' bracketed
        # launch times.  It is measured on the GNN stage, whose 2L attention
        # and 6L GEMM launches run back to back between two stage events: the
        # sum of their bracketed times exceeds the stage time by the bracketing
        # cost of 8L launches.
        nk = "ds_stats" if ds else "sinkhorn"
        n_gnn = 8 * cfg.L  # 2L attention launches and 6L GEMMs
        bracketed_gnn_ms = float(durs["attention"].sum() + durs["gemm"][:6 * cfg.L].sum())
        over = max(0.0, (bracketed_gnn_ms - stages["gnn"]) * 1e3 / n_gnn)
        # the double-softmax head has a single statistics launch, whose stage
        # time holds the events' own latency: its bracketed time less the
        # bracketing latency is used instead
        if ds:
            per = max(kernels[nk]["bracketed_avg_us"] - over, 1e-3)
        kernels[nk]["avg_us"] = round(per, 3)
        kernels[nk]["total_us"] = round(per * nn, 2)
        kernels[nk]["achieved_GBps"] = round(norm_work[0] / (per * 1e-6) / 1e9, 1)
        kernels[nk]["frac_hbm"] = round(norm_work[0] / (per * 1e-6) / 1e9 / PEAK["hbm_GBps"], 4)
        for k in ("attention", "gemm"):
            kk = kernels[k]
            kk["bracketed_avg_us"] = kk["avg_us"]
            kk["avg_us"] = round(max(kk["avg_us"] - over, 1e-3), 3)
            kk["total_us"] = round(kk["avg_us"] * kk["launches"], 2)
            scale = kk["bracketed_avg_us"] / kk["avg_us"]
            for f in ("achieved_TFLOPs", "achieved_TFLOPs_bf16"):
                if f in kk:
                    kk[f] = round(kk[f] * scale, 2)
        kernels["bracket_latency_us"] = round(over, 3)
        # MFMA utilisation of the headline pair's contraction kernels (the
        # metric's "MFMA util %"): algorithmic flops over the launch times
        # above, against the bf16 dense peak
        mfma_util = {"attention": round(100 * kernels["attention"]["achieved_TFLOPs"] / PEAK["bf16_TFLOPs"], 2),
                     "gemm_bf16": round(100 * kernels["gemm"]["achieved_TFLOPs_bf16"] / PEAK["bf16_TFLOPs"], 2),
                     "basis": "flop-based: algorithmic flops / (launch time x 2.5 PFLOP/s), launch times from "
                              "HIP events on the library's stream less the bracketing latency"}
        busy = profiled_mfma_busy()
        if busy is not None:
            mfma_util["counter_busy"] = {k: round(100 * v, 2) for k, v in busy.items()}
        dom = max((nk, "attention", "gemm"), key=lambda k: kernels[k]["total_us"])
        if dom == "ds_stats":
            per_launch = norm_work[0]
            ach = per_launch / (kernels[dom]["avg_us"] * 1e-6) / 1e9
            roofline = {"kernel": kernels[dom]["kernel"], "bound": "hbm", "achieved": round(ach, 1),
                        "peak": PEAK["hbm_GBps"], "unit": "GB/s", "frac": round(ach / PEAK["hbm_GBps"], 4),
                        "traffic": kernels[dom]["traffic"], "algorithmic_bytes_per_launch": per_launch,
                        "traffic_ratio": (None if kernels[dom]["traffic"] is None
                                          else round(kernels[dom]["traffic"] / per_launch, 3)),
                        "avg_launch_us": kernels[dom]["avg_us"]}
        elif dom == "sinkhorn":
            per_launch = norm_work[0]
            ach = per_launch / (kernels[dom]["avg_us"] * 1e-6) / 1e9
            tr = profiled_traffic("k_lse") if args.sinkhorn != "one" else None
            roofline = {"kernel": "k_lse_one (Sinkhorn sweep over Z or Z^T, one pair)", "bound": "hbm", "achieved": round(ach, 1),
                        "peak": PEAK["hbm_GBps"], "unit": "GB/s", "frac": round(ach / PEAK["hbm_GBps"], 4),
                        "traffic": None if tr is None else round(tr), "algorithmic_bytes_per_launch": per_launch,
                        "traffic_ratio": None if tr is None else round(tr / per_launch, 3),
                        "algorithmic_bytes_per_iteration": 2 * per_launch,
                        "iteration_us": round(2 * kernels[dom]["avg_us"], 3),
                        "avg_launch_us": kernels[dom]["avg_us"]}
            # the same iterations inside the replayed graph the headline runs:
            # the pass with T iterations against the same pass with none (its
            # extraction then takes the column argmax of Z itself), both timed
            # with HIP events around back-to-back replays on the library's stream
            it_graph = graph_iteration_us(sg, torch, step, args.steps, cfg.T)
            if it_graph is not None:
                ach_g = 2 * per_launch / (it_graph * 1e-6) / 1e9
                roofline["graph_replayed"] = {"iteration_us": round(it_graph, 3), "achieved": round(ach_g, 1),
                                              "frac": round(ach_g / PEAK["hbm_GBps"], 4)}
        elif dom == "attention":
            fl = attention_flops(cfg, M, N)
            ach = (sum(fl) / len(fl)) / (kernels[dom]["avg_us"] * 1e-6) / 1e12
            roofline = {"kernel": "k_attention", "bound": "mfma", "achieved": round(ach, 2),
                        "peak": PEAK["bf16_TFLOPs"], "unit": "TFLOP/s", "frac": round(ach / PEAK["bf16_TFLOPs"], 4),
                        "traffic": None, "algorithmic_flops_per_launch": sum(fl) / len(fl)}
        else:
            ach = kernels[dom]["achieved_TFLOPs_bf16"]
            roofline = {"kernel": "k_gemm (bf16 GNN projections)", "bound": "mfma", "achieved": ach,
                        "peak": PEAK["bf16_TFLOPs"], "unit": "TFLOP/s", "frac": round(ach / PEAK["bf16_TFLOPs"], 4),
                        "traffic": None}

    batch = None
    if args.batch:
        Bn = args.batch
        pairs = [synth.make_pair(cfg, seed=synth.INPUT_SEED_BASE + 100 + i) for i in range(Bn)]
        bt = {k: torch.from_numpy(np.stack([p[k] for p in pairs])).to(dev) for k in keys}
        Ms, Ns = [M] * Bn, [N] * Bn
        wsb = torch.empty(sg.workspace_size(W, M, N, Bn) + 4 * Bn * M * N, dtype=torch.uint8, device=dev)
        bbufs = {"matches0": torch.empty((Bn, M), dtype=torch.int32, device=dev),
                 "scores0": torch.empty((Bn, M), dtype=torch.float32, device=dev)}

        def bstep(T=None, **kw):
            return sg.sg_match_batch(Ms, Ns, *[bt[k] for k in keys], W, cfg.L, cfg.T if T is None else T,
                                     image_size=img, workspace=wsb, want_matches1=False, sinkhorn=args.sinkhorn,
                                     out=bbufs, **kw)
        for _ in range(max(2, args.warmup)):
            bstep()
        torch.cuda.synchronize()
        nb = max(3, args.steps // 10)
        t0 = time.perf_counter()
        for _ in range(nb):
            bstep()
        torch.cuda.synchronize()
        dtb = time.perf_counter() - t0
        batch = {"pairs_per_call": Bn, "calls": nb, "ms_per_call": round(1e3 * dtb / nb, 3),
                 "pairs_per_s": round(nb * Bn / dtb, 2)}
        if not args.no_kernel_timing:
            batch["kernels"] = batch_kernels(args, cfg, sg, np, torch, bstep, Bn, M, N, ds)
        if not ds and cfg.T > 0:
            # the Sinkhorn stage as the single pair's is measured: one event
            # pair around the stage's launches (T fused iterations and the
            # final column reduction) in an eager pass (stage events run the
            # call without its graph), against one read of every pair's
            # couplings per iteration; no per-launch events in between
            ev = sg.make_events(sg.SG_N_STAGE_EVENTS)
            sk = []
            for _ in range(3):
                bstep(stage_events=ev)
                torch.cuda.synchronize()
                sk.append(ev[3].elapsed_time(ev[4]) * 1e3)
            per_it = 4.0 * (M + 1) * (N + 1) * Bn
            us_it = float(np.median(sk)) / cfg.T
            batch["sinkhorn_stage"] = {"stage_us": round(float(np.median(sk)), 1), "us_per_iteration": round(us_it, 2),
                                       "bytes_per_iteration": per_it,
                                       "achieved_GBps": round(per_it / us_it / 1e3, 1),
                                       "frac_hbm": round(per_it / us_it / 1e3 / PEAK["hbm_GBps"], 4)}
        log(f"batch: {batch}")

    adaptive = adaptive_bench(args, cfg, dev, sg, synth, np, torch) if args.adaptive else None
    floor = None if args.no_launch_floor else launch_floor(torch)
    if floor:
        log(f"launch floor: {floor}")
        if roofline is not None and "k_lse" in roofline.get("kernel", ""):
            # the sweep against a plain graph-replayed read of the same matrix
            roofline["launch_floor_us"] = floor
            roofline["avg_launch_over_row_sum_floor"] = round(roofline["avg_launch_us"] / floor["row_sum_4MB_us"], 3)
    configs = None
    if not args.no_configs and args.head == "sinkhorn" and args.cross == "standard" and not args.rope:
        configs = per_config(sg, synth, np, torch, dev, workload_names(synth, args.configs))

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(cfg, w, pair, head=args.head)
        log(f"cpu: {cpu}")

    rec = {
        "metric": METRIC_DS if ds else METRIC, "value": round(value, 3), "unit": "pairs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded planted-homography pair, random Xavier weights)",
        "config": {"workload": ("one 1024x1024 keypoint pair per step: D=256, H=4, L=9 (18 stages), "
                                + ("bidirectional cross-attention, " if args.cross == "bidirectional" else "")
                                + ("rotary self-attention, " if args.rope else "")
                                + ("double-softmax + matchability head, " if ds else "T=100, ")
                                + "bf16 GNN operands / fp32 accumulation, fp32 scores + "
                                + ("head" if ds else "Sinkhorn")),
                   "pairs_per_step": 1, "M": M, "N": N, "D": cfg.D, "L": cfg.L, "T": None if ds else cfg.T,
                   "head": args.head, "cross_attention": args.cross, "rope": args.rope,
                   "shared_similarity": args.shared_similarity},
        "roofline": roofline, "mfma_util_pct": mfma_util, "cpu_baseline": cpu, "latency": latency,
        "stages_ms": stages, "kernels": kernels,
        "batch_throughput": batch, "concurrent_streams": concurrent, "launch_floor_us": floor,
        "per_config": configs,
        "adaptive": adaptive,
        "baseline_context": {"pages_ms_per_pair": {"GTX1080_1024kp": 87.0, "unstated_hw_2048kp": 70.0},
                             "pages_pairs_per_s": {"GTX1080_1024kp": 11.5, "unstated_hw_aachen_4096kp": 6.5}},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
