// Host side of libsg: argument validation, weight-blob layout, workspace
// layout and the launch sequence of the matching forward pass.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "sg_internal.h"

namespace {

using namespace sg;

thread_local std::string g_err;

sg_status fail(sg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

sg_status hip_fail(hipError_t e, const char* where) {
  return fail(SG_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int round32(int n) { return (n + 31) & ~31; }

// ------------------------------------------------------------ weight layout

struct Tensor {
  size_t off;
  int rows, cols;
};

struct WLayout {
  std::vector<Tensor> t;
  size_t bytes = 0;
  int enc_first = 0;    // index of encoder layer 0 W
  int stage_first = 0;  // index of stage 0 W_qkv
  int final_first = 0;  // index of W_f
  int alpha = 0;        // index of alpha
  int wz = -1;          // index of the matchability weight (double-softmax head)
  int rope = -1;        // index of the rotary basis
  int adapt = -1;       // index of layer 0's confidence weight (6 tensors per layer)
};

constexpr int kPerLayerAdaptive = 6;  // w_c, b_c, W_f, b_f, w_z, b_z

constexpr int kPerStage = 8;  // W_qkv, b_qkv, W_m, b_m, W_1, b_1, W_2, b_2

sg_status check_config(const sg_weights* w) {
  if (!w) return fail(SG_ERR_INVALID_ARG, "weights is NULL");
  if (w->D <= 0 || w->H <= 0) return fail(SG_ERR_INVALID_ARG, "D and H must be positive");
  if (w->D % w->H) return fail(SG_ERR_INVALID_ARG, "D (%d) is not a multiple of H (%d)", w->D, w->H);
  if (w->n_enc < 1 || w->n_enc > SG_MAX_ENC)
    return fail(SG_ERR_INVALID_ARG, "n_enc must be in [1, %d]", SG_MAX_ENC);
  for (int i = 0; i < w->n_enc; ++i)
    if (w->enc[i] <= 0) return fail(SG_ERR_INVALID_ARG, "encoder width %d is not positive", i);
  if (w->L_max < 1) return fail(SG_ERR_INVALID_ARG, "L_max must be >= 1");
  if (w->dtype != SG_F32 && w->dtype != SG_BF16) return fail(SG_ERR_INVALID_ARG, "unknown dtype %d", w->dtype);
  if (w->head != SG_HEAD_SINKHORN && w->head != SG_HEAD_DOUBLE_SOFTMAX)
    return fail(SG_ERR_INVALID_ARG, "unknown head %d", w->head);
  if (w->cross != SG_CROSS_STANDARD && w->cross != SG_CROSS_BIDIRECTIONAL)
    return fail(SG_ERR_INVALID_ARG, "unknown cross-attention variant %d", w->cross);
  if (w->rope != 0 && w->rope != 1) return fail(SG_ERR_INVALID_ARG, "rope must be 0 or 1 (got %d)", w->rope);
  if (w->adaptive != 0 && w->adaptive != 1)
    return fail(SG_ERR_INVALID_ARG, "adaptive must be 0 or 1 (got %d)", w->adaptive);
  if (w->adaptive && w->head != SG_HEAD_DOUBLE_SOFTMAX)
    return fail(SG_ERR_INVALID_ARG, "adaptive depth / width needs the double-softmax head");
  const int dh = w->D / w->H;
  if (dh != 16 && dh != 64) return fail(SG_ERR_UNSUPPORTED, "head dimension %d (supported: 16, 64)", dh);
  if (w->D % 32 || w->D > 1024) return fail(SG_ERR_UNSUPPORTED, "D = %d (supported: multiples of 32 up to 1024)", w->D);
  // the fused encoder keeps hidden layers in LDS and runs them on 32x32 MFMAs
  for (int i = 0; i < w->n_enc; ++i) {
    if (w->enc[i] > kMaxEncWidth || w->enc[i] % 16 || (i > 0 && w->enc[i] % 32))
      return fail(SG_ERR_UNSUPPORTED, "encoder width %d (hidden widths: multiples of 32 up to %d; the first may be 16)",
                  w->enc[i], kMaxEncWidth);
  }
  return SG_OK;
}

WLayout layout_of(const sg_weights* w) {
  WLayout L;
  const size_t es = w->dtype == SG_BF16 ? 2 : 4;
  size_t off = 0;
  auto add = [&](int rows, int cols, size_t elt) {
    L.t.push_back({off, rows, cols});
    off = align256(off + (size_t)rows * cols * elt);
  };
  const int D = w->D;
  L.enc_first = 0;
  int prev = 3;
  for (int i = 0; i <= w->n_enc; ++i) {
    const int out = i < w->n_enc ? w->enc[i] : D;
    add(out, prev, es);
    add(1, out, es);
    prev = out;
  }
  L.stage_first = (int)L.t.size();
  for (int s = 0; s < 2 * w->L_max; ++s) {
    const int nqkv = (s & 1) && w->cross == SG_CROSS_BIDIRECTIONAL ? 2 : 3;  // projections of the stage
    add(nqkv * D, D, es); add(1, nqkv * D, es);
    add(D, D, es); add(1, D, es);
    add(2 * D, 2 * D, es); add(1, 2 * D, es);
    add(D, 2 * D, es); add(1, D, es);
  }
  L.final_first = (int)L.t.size();
  add(D, D, es);
  add(1, D, es);
  L.alpha = (int)L.t.size();
  add(1, 1, 4);
  if (w->head == SG_HEAD_DOUBLE_SOFTMAX) {
    L.wz = (int)L.t.size();
    add(1, D, es);
    add(1, 1, es);
  }
  if (w->rope) {
    L.rope = (int)L.t.size();
    add(D / w->H / 2, 2, 4);  // always fp32
  }
  if (w->adaptive) {
    L.adapt = (int)L.t.size();
    for (int l = 0; l + 1 < w->L_max; ++l) {
      add(1, D, es); add(1, 1, es);   // token confidence
      add(D, D, es); add(1, D, es);   // layer l's final projection
      add(1, D, es); add(1, 1, es);   // layer l's matchability
    }
  }
  L.bytes = off;
  return L;
}

sg_status check_weights(const sg_weights* w, WLayout* out) {
  sg_status s = check_config(w);
  if (s != SG_OK) return s;
  if (!w->blob) return fail(SG_ERR_INVALID_ARG, "weights->blob is NULL");
  WLayout L = layout_of(w);
  if (w->blob_bytes < L.bytes)
    return fail(SG_ERR_WEIGHTS, "weight blob has %zu bytes, the configuration needs %zu", w->blob_bytes, L.bytes);
  *out = L;
  return SG_OK;
}

// ---------------------------------------------------------- workspace layout

struct WsLayout {
  size_t X, XB, QK, VT, KS, VS, MB, HB, WF, WFB, F, Z, ZT, P, PD, P2, PD2, PV, PI, U, V, UD, VD, IDX1, ROPE, ADAPT, SS,
      SS_bytes, total;
  int ldvt, ldqk;
};

WsLayout ws_layout_raw(long D, size_t os, long R, long zf, long ztf, long pf, long pd, long uf, long vf,
                       long nb, long ropef = 0, bool adaptive = false, long nstage = 0, long ssf = 0) {
  WsLayout L;
  // row strides are kept off powers of two (+64 / +16 bytes) so that the
  // strided accesses of the attention kernel spread over the L2 channels
  // fp32 networks keep q | k row-major and v transposed (VT); bf16 networks
  // keep q row-major and k, v in the tile-swizzled KS, VS (see AttnArgs)
  const bool bf = os == 2;
  L.ldvt = (int)((R + 63) & ~63L) + 32;
  L.ldqk = (int)((bf ? 1 : 2) * D + 8);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  L.X = take((size_t)R * D * 4);
  L.XB = take(bf ? (size_t)R * D * 2 : 0);  // bf16 copy of X: the operand of the QKV and MLP GEMMs
  L.QK = take((size_t)R * L.ldqk * os);
  L.VT = take(bf ? 0 : (size_t)D * L.ldvt * os);
  L.KS = take(bf ? (size_t)R * D * os : 0);
  L.VS = take(bf ? (size_t)R * D * os : 0);
  L.MB = take((size_t)R * D * os);
  L.HB = take((size_t)R * 2 * D * os);
  // per stage: the update MLP's first layer with the merge projection folded in
  L.WF = take((size_t)nstage * 4 * D * D * os);
  L.WFB = take((size_t)nstage * 2 * D * os);
  L.F = take((size_t)R * D * 4);
  L.Z = take((size_t)zf * 4);
  L.ZT = take((size_t)ztf * 4);
  L.P = take((size_t)pf * 4);
  L.PD = take((size_t)pd * 4);
  // the fused one-pass iteration reads one partial buffer and writes the other
  L.P2 = take((size_t)pf * 4);
  L.PD2 = take((size_t)pd * 4);
  L.PV = take((size_t)pf * 4);
  L.PI = take((size_t)pf * 4);
  L.U = take((size_t)uf * 4);
  L.V = take((size_t)vf * 4);
  L.UD = take((size_t)uf * 4);  // dustbin entries of the double-softmax head
  L.VD = take((size_t)vf * 4);
  L.IDX1 = take((size_t)nb * 4);
  L.ROPE = take((size_t)ropef * 8);  // (cos, sin) per row and rotary pair
  // adaptive calls: 10 per-row int / float arrays, the stop flag and the
  // exit head's (M+1) x (N+1) log assignment (at most zf + R + 1 floats)
  L.ADAPT = take(adaptive ? (size_t)(10 * R + 128 + zf + R + 1) * 4 : 0);
  // the shared similarity of a bidirectional cross stage of one pair (every
  // head's S and S^T, then their rows' log-sum-exp; SG_FLAG_SHARED_SIMILARITY)
  L.SS_bytes = (size_t)ssf * 4;
  L.SS = take(L.SS_bytes);
  L.total = o;
  return L;
}

// Floats of the shared similarity of one M x N pair with H heads (S [H][M][ld4(N)],
// S^T [H][N][ld4(M)], the rows' log-sum-exp [H][M] and [H][N]), zero unless
// the network has bidirectional cross stages.
long shared_sim_floats(const sg_weights* w, long M, long N) {
  if (w->cross != SG_CROSS_BIDIRECTIONAL) return 0;
  return (long)w->H * (M * ld4((int)N) + N * ld4((int)M) + M + N);
}

WsLayout ws_layout(const sg_weights* w, long R, long zf, long ztf, long pf, long pd, long uf, long vf, long nb,
                   long ssf = 0) {
  return ws_layout_raw(w->D, w->dtype == SG_BF16 ? 2 : 4, R, zf, ztf, pf, pd, uf, vf, nb,
                       w->rope ? R * (w->D / w->H / 2) : 0, w->adaptive != 0, 2L * w->L_max, ssf);
}

// ----------------------------------------------------------- library workspace

struct OwnedWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
OwnedWs g_ws[64];

sg_status get_workspace(const sg_opts* o, size_t need, void** ptr) {
  if (o && o->workspace) {
    if (o->workspace_bytes < need)
      return fail(SG_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", o->workspace_bytes, need);
    *ptr = o->workspace;
    return SG_OK;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(SG_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_ws_mu);
  OwnedWs& w = g_ws[dev];
  if (w.bytes < need) {
    if (w.ptr) {
      // the buffer may still be in use by enqueued work on any stream
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    e = hipMalloc(&w.ptr, need);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    w.bytes = need;
  }
  *ptr = w.ptr;
  return SG_OK;
}

// -------------------------------------------------------------- timing hooks

struct Timer {
  const sg_opts* o;
  hipStream_t st;
  int launches = 0;
  void stage(int k) {
    if (o && o->stage_events && k < o->n_stage_events) (void)hipEventRecord((hipEvent_t)o->stage_events[k], st);
  }
  bool bracket(int kind) const {
    return o && o->kernel_events && o->timed_kernel == kind && 2 * (launches + 1) <= o->n_kernel_events;
  }
  template <class F>
  hipError_t run(int kind, F&& f) {
    if (bracket(kind)) {
      (void)hipEventRecord((hipEvent_t)o->kernel_events[2 * launches], st);
      hipError_t e = f();
      (void)hipEventRecord((hipEvent_t)o->kernel_events[2 * launches + 1], st);
      ++launches;
      return e;
    }
    return f();
  }
  void finish() {
    if (o && o->n_kernel_launches) *o->n_kernel_launches = launches;
  }
};

// ------------------------------------------------------------- the pipeline

struct Problem {
  int B = 1, Mpad = 0, Npad = 0;
  int flags = 0;  // SG_FLAG_*
  int head = SG_HEAD_SINKHORN;
  std::vector<int> M, N;
  const float *kp[2] = {nullptr, nullptr}, *cf[2] = {nullptr, nullptr}, *de[2] = {nullptr, nullptr};
  float img[4] = {0, 0, 0, 0};
};

struct Plan {
  SegTable seg;
  PairTable pt;
  int R = 0;
  long zf = 0, ztf = 0, pf = 0, pd = 0, uf = 0, vf = 0, nb = 0;
  bool two_sweep = false;  // Sinkhorn schedule (see SG_FLAG_SINKHORN_*)
  bool fused = false;      // one-pass schedule with the fused iteration (k_sink_iter)
  int ru = 0, rv = 0;  // flattened u rows (sum of M+1) and v rows (sum of N+1)
  std::vector<int> rowB;
};

void make_plan(const Problem& p, Plan& pl) {
  memset(&pl.seg, 0, sizeof(pl.seg));
  memset(&pl.pt, 0, sizeof(pl.pt));
  pl.rowB.assign(p.B, 0);
  pl.uf = pl.vf = 0;
  int R = 0;
  long zf = 0, ztf = 0, pf = 0;
  pl.pt.n_pairs = p.B;
  // Sinkhorn schedule: forced by a flag, else by the score matrices' size:
  // two sweeps up to SG_TWO_SWEEP_MAX_BYTES, one pass with a column
  // reduction beyond
  long zbytes = 0;
  for (int b = 0; b < p.B; ++b) zbytes += 4L * p.M[b] * ld4(p.N[b]);
  // (the double-softmax head reads Z and ZT once each, whatever their size)
  pl.two_sweep = p.head == SG_HEAD_DOUBLE_SOFTMAX || (p.flags & SG_FLAG_SINKHORN_TWO_SWEEP) ||
                 (!(p.flags & SG_FLAG_SINKHORN_ONE_SWEEP) && zbytes <= (long)SG_TWO_SWEEP_MAX_BYTES);
  // one-pass schedule: the fused iteration's row blocks where every row fits
  // its registers, else the row pass + column reduction pair's
  pl.fused = !pl.two_sweep && sink_iter_rows_per_block(p.N.data(), p.B) > 0;
  pl.pt.rb = pl.fused ? sink_iter_rows_per_block(p.N.data(), p.B) : sink_rows_per_block(p.M.data(), p.N.data(), p.B);
  pl.seg.n_seg = 2 * p.B;
  for (int b = 0; b < p.B; ++b) {
    const int M = p.M[b], N = p.N[b];
    const int sa = 2 * b, sb = 2 * b + 1;
    pl.seg.row0[sa] = R; pl.seg.n[sa] = M; pl.seg.in_off[sa] = b * p.Mpad; pl.seg.side[sa] = 0; pl.seg.partner[sa] = sb;
    R += round32(M);
    pl.seg.row0[sb] = R; pl.seg.n[sb] = N; pl.seg.in_off[sb] = b * p.Npad; pl.seg.side[sb] = 1; pl.seg.partner[sb] = sa;
    pl.rowB[b] = R;
    R += round32(N);
    pl.pt.M[b] = M; pl.pt.N[b] = N; pl.pt.rowA[b] = pl.seg.row0[sa];
    pl.pt.z_off[b] = (int)zf;
    pl.pt.zt_off[b] = (int)ztf;
    pl.pt.p_off[b] = (int)pf;
    zf += (long)M * ld4(N);
    ztf += (long)N * ld4(M);
    const int G = pl.fused ? sink_iter_blocks(M, pl.pt.rb) : (M + 1 + pl.pt.rb - 1) / pl.pt.rb;
    pf += (long)G * ld4(N);
    pl.pt.gpre[b + 1] = pl.pt.gpre[b] + G;
    pl.pt.upre[b + 1] = pl.pt.upre[b] + M + 1;
    pl.pt.vpre[b + 1] = pl.pt.vpre[b] + N + 1;
    pl.pt.uoff[b] = (int)pl.uf;
    pl.pt.voff[b] = (int)pl.vf;
    pl.uf += ld4(M + 1);
    pl.vf += ld4(N + 1);
  }
  // the fused iteration dispatches the blocks of the widest rows first, so
  // that the last blocks to start are the cheapest
  {
    int ord[SG_MAX_BATCH];
    for (int b = 0; b < p.B; ++b) ord[b] = b;
    std::stable_sort(ord, ord + p.B, [&](int a, int c) { return p.N[a] > p.N[c]; });
    for (int k = 0; k < p.B; ++k) {
      pl.pt.ord[k] = (unsigned char)ord[k];
      pl.pt.opre[k + 1] = pl.pt.opre[k] + pl.pt.gpre[ord[k] + 1] - pl.pt.gpre[ord[k]];
    }
  }
  pl.R = R;
  pl.zf = zf; pl.pf = pf; pl.pd = pl.pt.gpre[p.B];
  pl.ztf = pl.two_sweep ? ztf : 0;
  if (p.head == SG_HEAD_DOUBLE_SOFTMAX) pl.pf = pl.pd = 0;  // no column partials
  pl.ru = pl.pt.upre[p.B]; pl.rv = pl.pt.vpre[p.B];
  pl.nb = pl.rv - p.B;
}

template <class T>
const T* at(const sg_weights* w, const WLayout& L, int idx) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(w->blob) + L.t[idx].off);
}
const void* atv(const sg_weights* w, const WLayout& L, int idx) {
  return reinterpret_cast<const char*>(w->blob) + L.t[idx].off;
}

struct Outputs {
  int32_t* m0 = nullptr; float* s0 = nullptr;
  int32_t* m1 = nullptr; float* s1 = nullptr;
  float* descA = nullptr; float* descB = nullptr;
  float* logP = nullptr; int64_t logP_ld = 0; int64_t logP_stride = 0;
};

GemmBatch single(int rows, int n_out, int ldc, int c_off = 0) {
  GemmBatch b;
  memset(&b, 0, sizeof(b));
  b.n = 1;
  b.p[0] = GemmProblem{0, 0, rows, n_out, c_off, 0, ldc, 0};
  return b;
}

#define HIPCHK(expr, where)                      \
  do {                                            \
    hipError_t e_ = (expr);                       \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// Encoder: layer 0 (with normalisation) then GEMM layers; the last adds into X.
FoldArgs make_fold(const sg_weights* w, const WLayout& L, int c0, int n, char* ws, const WsLayout& wl);

// The encoder; with fold_n > 0 the merge fold of stages [0, fold_n) runs in
// the same launch (at most kMaxFold stages).
sg_status run_encoder(const Problem& p, const Plan& pl, const sg_weights* w, const WLayout& L,
                      char* ws, const WsLayout& wl, Timer& tm, hipStream_t st, int fold_n = 0) {
  (void)tm;
  EncArgs e;
  memset(&e, 0, sizeof(e));
  for (int i = 0; i < 2; ++i) { e.kpts[i] = p.kp[i]; e.conf[i] = p.cf[i]; e.desc[i] = p.de[i]; }
  memcpy(e.img, p.img, sizeof(e.img));
  e.D = w->D;
  e.ldx = w->D;
  e.n_layers = w->n_enc + 1;
  e.width[0] = 3;
  for (int i = 0; i < w->n_enc; ++i) e.width[i + 1] = w->enc[i];
  e.width[w->n_enc + 1] = w->D;
  for (int i = 0; i <= w->n_enc; ++i) {
    e.W[i] = atv(w, L, L.enc_first + 2 * i);
    e.b[i] = atv(w, L, L.enc_first + 2 * i + 1);
  }
  e.X = reinterpret_cast<float*>(ws + wl.X);
  e.XB = w->dtype == SG_BF16 ? ws + wl.XB : nullptr;
  if (fold_n > 0) {
    const FoldArgs f = make_fold(w, L, 0, fold_n, ws, wl);
    HIPCHK(launch_encoder(w->dtype, w->dtype, e, pl.seg, st, &f), "encoder and merge fold");
  } else {
    HIPCHK(launch_encoder(w->dtype, w->dtype, e, pl.seg, st), "encoder");
  }
  return SG_OK;
}

// Rotary table of the self stages from the positions of the problem.
sg_status run_rope_table(const Problem& p, const Plan& pl, const sg_weights* w, const WLayout& L, char* ws,
                         const WsLayout& wl, hipStream_t st, const int* ind = nullptr) {
  EncArgs e;
  memset(&e, 0, sizeof(e));
  for (int i = 0; i < 2; ++i) e.kpts[i] = p.kp[i];
  memcpy(e.img, p.img, sizeof(e.img));
  HIPCHK(launch_rope_table(e, pl.seg, at<float>(w, L, L.rope), w->D / w->H, pl.R, ind,
                           reinterpret_cast<float2*>(ws + wl.ROPE), st), "rotary table");
  return SG_OK;
}

// Folds the merge projection of stages [s0, s1) into their update MLPs'
// first layers (workspace WF / WFB, indexed by stage).  Every call redoes
// it, so that weights changed in place between calls take effect.
// The fold arguments of stages [c0, c0 + n), n <= kMaxFold.
FoldArgs make_fold(const sg_weights* w, const WLayout& L, int c0, int n, char* ws, const WsLayout& wl) {
  const int D = w->D;
  const size_t os = w->dtype == SG_BF16 ? 2 : 4;
  FoldArgs f;
  memset(&f, 0, sizeof(f));
  f.D = D;
  f.n = n;
  for (int i = 0; i < f.n; ++i) {
    const int base = L.stage_first + kPerStage * (c0 + i);
    f.wm[i] = atv(w, L, base + 2);
    f.bm[i] = atv(w, L, base + 3);
    f.w1[i] = atv(w, L, base + 4);
    f.b1[i] = atv(w, L, base + 5);
  }
  f.wf = ws + wl.WF + (size_t)c0 * 4 * D * D * os;
  f.bf = ws + wl.WFB + (size_t)c0 * 2 * D * os;
  return f;
}

sg_status run_fold(const sg_weights* w, const WLayout& L, int s0, int s1, char* ws, const WsLayout& wl, Timer& tm,
                   hipStream_t st) {
  for (int c0 = s0; c0 < s1; c0 += kMaxFold) {
    const FoldArgs f = make_fold(w, L, c0, std::min(kMaxFold, s1 - c0), ws, wl);
    HIPCHK(tm.run(SG_K_GEMM, [&] { return launch_fold_merge(w->dtype, f, st); }), "merge fold");
  }
  return SG_OK;
}

// Stages [s0, s1) in place on X (compact rows of every image of the plan);
// the merge projections of these stages must have been folded (run_fold).
// xb_valid: the bf16 copy XB of the states is current (the encoder writes
// it); otherwise bf16 networks refresh it first.
sg_status run_gnn(const Plan& pl, const sg_weights* w, const WLayout& L, int s0, int s1, char* ws,
                  const WsLayout& wl, int flags, Timer& tm, hipStream_t st, const int* stop = nullptr,
                  bool xb_valid = false) {
  const int D = w->D, op = w->dtype, R = pl.R;
  float* X = reinterpret_cast<float*>(ws + wl.X);
  // bf16 networks read the states as bf16 (the QKV and MLP GEMMs would round
  // them on load anyway); the residual GEMM keeps the copy current
  void* XB = op == SG_BF16 ? ws + wl.XB : nullptr;
  if (XB && !xb_valid && s0 < s1) HIPCHK(launch_to_bf16(X, XB, R * D, st), "bf16 states");
  void* QK = ws + wl.QK;
  void* VT = ws + wl.VT;
  void* MB = ws + wl.MB;
  void* HB = ws + wl.HB;
  const size_t os = op == SG_BF16 ? 2 : 4;
  const float log2e = 1.4426950408889634f;
  for (int s = s0; s < s1; ++s) {
    const int base = L.stage_first + kPerStage * s;
    // q | k | v = x W_qkv^T + b_qkv  (v written transposed or swizzled); a
    // bidirectional cross stage projects qk | v and writes qk as both q and k
    {
      const bool tied = (s & 1) && w->cross == SG_CROSS_BIDIRECTIONAL;
      const int nout = (tied ? 2 : 3) * D;
      GemmArgs g;
      memset(&g, 0, sizeof(g));
      g.A0 = XB ? XB : X; g.lda0 = D; g.K0 = D; g.K = D;
      g.W = atv(w, L, base); g.ldw = D; g.bias = atv(w, L, base + 1);
      g.C = QK; g.C2 = op == SG_BF16 ? ws + wl.VS : VT; g.C3 = ws + wl.KS;
      g.split = nout - D; g.tied = tied; g.stop = stop;
      if (w->rope && !(s & 1)) {  // self stage: rotate q and k
        g.rope = reinterpret_cast<const float2*>(ws + wl.ROPE);
        g.rope_dh = D / w->H;
      }
      GemmBatch b = single(R, nout, wl.ldqk);
      b.p[0].ldct = wl.ldvt;
      HIPCHK(tm.run(SG_K_GEMM, [&] { return launch_gemm(op, XB == nullptr, op, 0, EPI_QKV, g, b, R, nout, st); }),
             "qkv GEMM");
    }
    // multi-head attention: self on even stages, cross on odd stages
    {
      AttnArgs a;
      memset(&a, 0, sizeof(a));
      a.qk = QK; a.vt = VT; a.ks = ws + wl.KS; a.vs = ws + wl.VS;
      a.out = MB; a.D = D; a.ldvt = wl.ldvt; a.ldqk = wl.ldqk; a.cross = s & 1; a.stop = stop;
      a.heads = w->H;
      const int dh = D / w->H;
      a.scale2 = log2e / sqrtf((float)dh);
      // (an image with no points: the plain kernel, which gives the other
      // image's queries zero messages)
      const bool shared = (flags & SG_FLAG_SHARED_SIMILARITY) && (s & 1) && w->cross == SG_CROSS_BIDIRECTIONAL &&
                          pl.seg.n_seg == 2 && wl.SS_bytes > 0 && pl.seg.n[0] > 0 && pl.seg.n[1] > 0;
      if (shared) {
        // the similarity of each head formed once, S = qk_A qk_B^T (scaled to
        // base 2) and its transpose from the same accumulators, then the
        // rows' log-sum-exp of both, then both images' messages from them
        const int M = pl.seg.n[0], N = pl.seg.n[1], H = w->H;
        float* SS = reinterpret_cast<float*>(ws + wl.SS);
        const long sA = (long)M * ld4(N), sB = (long)N * ld4(M);
        float* LSE = SS + H * (sA + sB);
        for (int h = 0; h < H; ++h) {
          GemmArgs g;
          memset(&g, 0, sizeof(g));
          g.A0 = static_cast<char*>(QK) + (size_t)h * dh * os; g.lda0 = wl.ldqk; g.K0 = dh; g.K = dh;
          g.W = g.A0; g.ldw = wl.ldqk;
          g.C = SS; g.C2 = SS + H * sA; g.scale = a.scale2; g.stop = stop;
          GemmBatch b;
          memset(&b, 0, sizeof(b));
          b.n = 1;
          b.p[0] = GemmProblem{pl.seg.row0[0], pl.seg.row0[1], M, N, (int)(h * sA), (int)(h * sB), ld4(N), ld4(M)};
          HIPCHK(tm.run(SG_K_ATTENTION, [&] { return launch_gemm(op, 0, op, 1, EPI_SCORE, g, b, M, N, st); }),
                 "shared similarity");
        }
        HIPCHK(tm.run(SG_K_ATTENTION, [&] { return launch_rows_lse(SS, ld4(N), H * M, N, LSE, st); }),
               "similarity rows");
        HIPCHK(tm.run(SG_K_ATTENTION, [&] { return launch_rows_lse(SS + H * sA, ld4(M), H * N, M, LSE + H * M, st); }),
               "similarity columns");
        a.sm = SS; a.lse = LSE; a.scale2 = 1.f;
        a.s_off[0] = 0; a.s_hs[0] = sA; a.s_ld[0] = ld4(N);
        a.s_off[1] = H * sA; a.s_hs[1] = sB; a.s_ld[1] = ld4(M);
        a.l_off[0] = 0; a.l_hs[0] = M;
        a.l_off[1] = H * M; a.l_hs[1] = N;
        HIPCHK(tm.run(SG_K_ATTENTION, [&] { return launch_attention_shared(op, dh, a, pl.seg, H, st); }),
               "attention (shared similarity)");
      } else {
        HIPCHK(tm.run(SG_K_ATTENTION, [&] { return launch_attention(op, dh, a, pl.seg, w->H, st); }), "attention");
      }
    }
    // h = ReLU(W_1 [x || m] + b_1) with m = W_m a + b_m folded in (run_fold):
    // h = ReLU(W_f [x || a] + b_f), a = the attention output
    {
      GemmArgs g;
      memset(&g, 0, sizeof(g));
      g.A0 = XB ? XB : X; g.lda0 = D; g.K0 = D; g.A1 = MB; g.lda1 = D; g.K = 2 * D;
      g.W = ws + wl.WF + (size_t)s * 4 * D * D * os; g.ldw = 2 * D; g.bias = ws + wl.WFB + (size_t)s * 2 * D * os;
      g.C = HB; g.stop = stop;
      GemmBatch b = single(R, 2 * D, 2 * D);
      HIPCHK(tm.run(SG_K_GEMM, [&] { return launch_gemm(op, XB == nullptr, op, op == SG_F32, EPI_RELU, g, b, R, 2 * D, st); }),
             "mlp1 GEMM");
    }
    // x += W_2 h + b_2
    {
      GemmArgs g;
      memset(&g, 0, sizeof(g));
      g.A0 = HB; g.lda0 = 2 * D; g.K0 = 2 * D; g.K = 2 * D;
      g.W = atv(w, L, base + 6); g.ldw = 2 * D; g.bias = atv(w, L, base + 7);
      g.C = X; g.C2 = XB; g.stop = stop;
      GemmBatch b = single(R, D, D);
      HIPCHK(tm.run(SG_K_GEMM, [&] { return launch_gemm(op, op == SG_F32, op, 1, EPI_RESID, g, b, R, D, st); }), "mlp2 GEMM");
    }
  }
  return SG_OK;
}

// Final projection of every row of X into F (fp32).
sg_status run_project(const Plan& pl, const sg_weights* w, const WLayout& L, const float* X, float* F,
                      Timer& tm, hipStream_t st, int wf_index = -1) {
  const int D = w->D, op = w->dtype;
  if (wf_index < 0) wf_index = L.final_first;
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A0 = X; g.lda0 = D; g.K0 = D; g.K = D;
  g.W = atv(w, L, wf_index); g.ldw = D; g.bias = atv(w, L, wf_index + 1);
  g.C = F;
  GemmBatch b = single(pl.R, D, D);
  HIPCHK(tm.run(SG_K_GEMM, [&] { return launch_gemm(op, 1, op, 1, EPI_BIAS, g, b, pl.R, D, st); }), "final projection");
  return SG_OK;
}

// Inputs of the double-softmax head: the last states X [R][D] (fp32, rows
// of the plan) and the matchability weights (w_dtype) with the bias at
// bz_dev, or the host value bz when bz_dev is null.
struct DsHead {
  const float* X = nullptr;
  int w_dtype = SG_F32;
  const void* wz = nullptr;
  const void* bz_dev = nullptr;
  float bz = 0.f;
};

// Scores, the head (Sinkhorn or double softmax) and extraction from F (rows
// of the plan).  ds == nullptr: Sinkhorn.
sg_status run_matching(const Problem& p, const Plan& pl, int D, float alpha, const float* alpha_dev,
                       int T, float thr, const DsHead* ds,
                       const float* F, char* ws, const WsLayout& wl, const Outputs& out, Timer& tm,
                       hipStream_t st) {
  const float log2e = 1.4426950408889634f;
  float* Z = reinterpret_cast<float*>(ws + wl.Z);
  float* ZT = reinterpret_cast<float*>(ws + wl.ZT);
  float* P = reinterpret_cast<float*>(ws + wl.P);
  float* Pd = reinterpret_cast<float*>(ws + wl.PD);
  float* P2 = reinterpret_cast<float*>(ws + wl.P2);
  float* Pd2 = reinterpret_cast<float*>(ws + wl.PD2);
  float* PV = reinterpret_cast<float*>(ws + wl.PV);
  int* PI = reinterpret_cast<int*>(ws + wl.PI);
  float* U = reinterpret_cast<float*>(ws + wl.U);
  float* V = reinterpret_cast<float*>(ws + wl.V);
  int* idx1 = reinterpret_cast<int*>(ws + wl.IDX1);
  const float alpha2 = alpha * log2e;
  // S * log2(e) / sqrt(D) into Z (and its transpose into ZT for two sweeps)
  {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.A0 = F; g.lda0 = D; g.K0 = D; g.K = D;
    g.W = F; g.ldw = D;
    g.C = Z; g.C2 = pl.two_sweep ? ZT : nullptr;
    g.scale = log2e / sqrtf((float)D);
    GemmBatch b;
    memset(&b, 0, sizeof(b));
    b.n = p.B;
    int mr = 0, mn = 0;
    for (int i = 0; i < p.B; ++i) {
      b.p[i] = GemmProblem{pl.pt.rowA[i], pl.rowB[i], p.M[i], p.N[i], pl.pt.z_off[i], pl.pt.zt_off[i],
                           ld4(p.N[i]), ld4(p.M[i])};
      mr = std::max(mr, p.M[i]);
      mn = std::max(mn, p.N[i]);
    }
    HIPCHK(tm.run(SG_K_GEMM, [&] { return launch_gemm(SG_F32, 1, SG_F32, 1, EPI_SCORE, g, b, mr, mn, st); }), "score GEMM");
  }
  tm.stage(SG_EV_SCORES);
  if (ds) {
    // one sweep over the rows of Z and of ZT: row / column log-sum-exp and
    // matchability; then the same extraction with the real block 2 Z + u + v
    float* UD = reinterpret_cast<float*>(ws + wl.UD);
    float* VD = reinterpret_cast<float*>(ws + wl.VD);
    HIPCHK(tm.run(SG_K_SINKHORN, [&] {
             return launch_ds_stats(Z, ZT, pl.pt, ds->X, D, ds->w_dtype, ds->wz, ds->bz_dev, ds->bz, U, V, UD, VD, st);
           }), "double-softmax statistics");
    tm.stage(SG_EV_SINKHORN);
    HIPCHK(launch_col_argmax(ZT, pl.pt, U, idx1, p.Npad, out.m1, out.s1, EXT_DS, st), "column argmax");
    HIPCHK(launch_sink_extract(Z, pl.pt, U, V, idx1, p.Mpad, p.Npad, thr, out.m0, out.s0, out.m1, out.s1, EXT_DS, st),
           "extract");
    if (out.logP)
      HIPCHK(launch_ds_write_logp(Z, pl.pt, U, V, UD, VD, out.logP, out.logP_ld, out.logP_stride, pl.ru, st),
             "logP");
    return SG_OK;
  }
  if (pl.two_sweep) {
    // T iterations: u = log mu - lse_j(Z + v) over the rows of Z, then
    // v = log nu - lse_i(Z + u) over the rows of ZT.  For one pair the last
    // column sweep, which reads Z + u with the final u, also takes the
    // column argmax of the extraction.
    const bool fused_arg = pl.pt.n_pairs == 1 && T > 0;
    for (int it = 0; it < T; ++it) {
      const bool arg = fused_arg && it == T - 1;
      HIPCHK(tm.run(SG_K_SINKHORN, [&] { return launch_lse(Z, pl.pt, 0, it == 0 ? nullptr : V, U, alpha2, alpha_dev, pl.ru, st); }),
             "sinkhorn rows");
      HIPCHK(tm.run(SG_K_SINKHORN, [&] {
               return launch_lse(ZT, pl.pt, 1, U, V, alpha2, alpha_dev, pl.rv, st, arg ? idx1 : nullptr,
                                 arg ? out.m1 : nullptr, arg ? out.s1 : nullptr);
             }), "sinkhorn cols");
    }
    if (T == 0) {
      HIPCHK(launch_fill_f32(U, 0.f, (int)pl.uf, st), "zero u");
      HIPCHK(launch_fill_f32(V, 0.f, (int)pl.vf, st), "zero v");
    }
    tm.stage(SG_EV_SINKHORN);
    if (!fused_arg)
      HIPCHK(launch_col_argmax(ZT, pl.pt, U, idx1, p.Npad, out.m1, out.s1, EXT_SINKHORN, st), "column argmax");
  } else if (pl.fused) {
    // T fused iterations: each reduces the previous iteration's block
    // partials into v, then updates u and writes its own partials (the two
    // partial buffers alternate); the last one also leaves the per-block
    // column argmax of Z + u.  One column reduction turns the last partials
    // into v and the column argmax.
    float* Pb[2] = {P, P2};
    float* Pdb[2] = {Pd, Pd2};
    for (int it = 0; it < T; ++it) {
      const bool last = it == T - 1;
      HIPCHK(tm.run(SG_K_SINKHORN, [&] {
               return launch_sink_iter(Z, pl.pt, it == 0 ? nullptr : Pb[(it + 1) & 1],
                                       it == 0 ? nullptr : Pdb[(it + 1) & 1], U, Pb[it & 1], Pdb[it & 1],
                                       last ? PV : nullptr, last ? PI : nullptr, alpha2, alpha_dev, 1, st);
             }), "sinkhorn iteration");
    }
    if (T > 0) {
      HIPCHK(tm.run(SG_K_SINKHORN, [&] {
               return launch_sink_cols(pl.pt, Pb[(T - 1) & 1], Pdb[(T - 1) & 1], V, PV, PI, idx1, 1, p.Npad, out.m1,
                                       out.s1, st);
             }), "sinkhorn cols");
    } else {
      HIPCHK(launch_fill_f32(U, 0.f, (int)pl.uf, st), "zero u");
      HIPCHK(launch_fill_f32(V, 0.f, (int)pl.vf, st), "zero v");
      HIPCHK(launch_sink_iter(Z, pl.pt, nullptr, nullptr, U, P, Pd, PV, PI, alpha2, alpha_dev, 0, st), "column argmax");
      HIPCHK(launch_sink_cols(pl.pt, P, Pd, V, PV, PI, idx1, 0, p.Npad, out.m1, out.s1, st), "column argmax");
    }
    tm.stage(SG_EV_SINKHORN);
  } else {
    // T iterations: u = log mu - lse_j(Z + v) with the column partials of
    // Z + u in the same pass; then v = log nu - lse over the partials.  The
    // last pass also leaves the per-block column argmax of Z + u.
    for (int it = 0; it < T; ++it) {
      const bool last = it == T - 1;
      HIPCHK(tm.run(SG_K_SINKHORN, [&] {
               return launch_sink_rows(Z, pl.pt, it == 0 ? nullptr : V, U, P, Pd, last ? PV : nullptr,
                                       last ? PI : nullptr, alpha2, alpha_dev, 1, st);
             }), "sinkhorn rows");
      HIPCHK(tm.run(SG_K_SINKHORN, [&] {
               return launch_sink_cols(pl.pt, P, Pd, V, last ? PV : nullptr, last ? PI : nullptr, idx1, 1, p.Npad,
                                       out.m1, out.s1, st);
             }), "sinkhorn cols");
    }
    if (T == 0) {
      HIPCHK(launch_fill_f32(U, 0.f, (int)pl.uf, st), "zero u");
      HIPCHK(launch_fill_f32(V, 0.f, (int)pl.vf, st), "zero v");
      HIPCHK(launch_sink_rows(Z, pl.pt, nullptr, U, P, Pd, PV, PI, alpha2, alpha_dev, 0, st), "column argmax");
      HIPCHK(launch_sink_cols(pl.pt, P, Pd, V, PV, PI, idx1, 0, p.Npad, out.m1, out.s1, st), "column argmax");
    }
    tm.stage(SG_EV_SINKHORN);
  }
  HIPCHK(launch_sink_extract(Z, pl.pt, U, V, idx1, p.Mpad, p.Npad, thr, out.m0, out.s0, out.m1, out.s1, EXT_SINKHORN, st),
         "extract");
  if (out.logP)
    HIPCHK(launch_write_logp(Z, pl.pt, U, V, alpha2, alpha_dev, out.logP, out.logP_ld, out.logP_stride, pl.ru, st),
           "logP");
  return SG_OK;
}

// ------------------------------------------- Sinkhorn / extraction stages
//
// The stage entry points on caller-given matrices run the pass's own sweep
// and extraction kernels on one pair, through the same internal layout:
// the real block in Z and ZT (base-2 scaled for Sinkhorn, as given for
// extraction), the dustbin column and row (Sinkhorn: any values, not only
// the constant alpha of the pass), the base-2 duals and the column argmax.

struct StageWs {
  size_t Z, ZT, BCOL, BROW, U, V, IDX1, total;
};

StageWs stage_ws(long M, long N) {
  StageWs L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  L.Z = take((size_t)M * ld4((int)N) * 4);
  L.ZT = take((size_t)N * ld4((int)M) * 4);
  L.BCOL = take((size_t)ld4((int)M + 1) * 4);
  L.BROW = take((size_t)ld4((int)N + 1) * 4);
  L.U = take((size_t)ld4((int)M + 1) * 4);
  L.V = take((size_t)ld4((int)N + 1) * 4);
  L.IDX1 = take((size_t)ld4((int)N) * 4);
  L.total = o;
  return L;
}

template <class T>
T* ws_at(char* ws, size_t off) {
  return reinterpret_cast<T*>(ws + off);
}

// T iterations on C [(M+1)][ldc] (M, N >= 1): u_i = log mu_i - lse_j, then
// v_j = log nu_j - lse_i, with mu = [1_M, N] / (M+N), nu = [1_N, M] / (M+N)
// (the pass's marginals); then the natural-log duals and logP.
sg_status enqueue_stage_sinkhorn(const float* C, int64_t ldc, int M, int N, int T, float* u, float* v, float* logP,
                                 int64_t ldp, char* ws, const StageWs& L, hipStream_t st) {
  float* Z = ws_at<float>(ws, L.Z);
  float* ZT = ws_at<float>(ws, L.ZT);
  float* bcol = ws_at<float>(ws, L.BCOL);
  float* brow = ws_at<float>(ws, L.BROW);
  float* U = ws_at<float>(ws, L.U);
  float* V = ws_at<float>(ws, L.V);
  HIPCHK(launch_stage_couplings(C, ldc, M, N, 1.4426950408889634f, Z, ZT, bcol, brow, st), "stage couplings");
  // the same single-precision logarithms as the pass's sweeps
  const float lmn = std::log2((float)(M + N));
  for (int it = 0; it < T; ++it) {
    HIPCHK(launch_lse_explicit(Z, it == 0 ? nullptr : V, U, M, N, 0.f - lmn, std::log2((float)N) - lmn, bcol, brow,
                               st),
           "sinkhorn rows");
    HIPCHK(launch_lse_explicit(ZT, U, V, N, M, 0.f - lmn, std::log2((float)M) - lmn, brow, bcol, st),
           "sinkhorn cols");
  }
  if (T == 0) {
    HIPCHK(launch_fill_f32(U, 0.f, M + 1, st), "zero u");
    HIPCHK(launch_fill_f32(V, 0.f, N + 1, st), "zero v");
  }
  HIPCHK(launch_stage_duals(C, ldc, M, N, U, V, u, v, logP, ldp, st), "duals");
  return SG_OK;
}

// Mutual-argmax extraction of the real block of a natural-log assignment
// P [(M+1)][ldp] (M, N >= 1), through the pass's extraction kernels.
sg_status enqueue_stage_extract(const float* P, int64_t ldp, int M, int N, float thr, int32_t* m0, float* s0,
                                int32_t* m1, float* s1, char* ws, const StageWs& L, hipStream_t st) {
  Problem p;
  p.B = 1; p.Mpad = M; p.Npad = N; p.M = {M}; p.N = {N};
  Plan pl;
  make_plan(p, pl);
  float* Z = ws_at<float>(ws, L.Z);
  float* ZT = ws_at<float>(ws, L.ZT);
  int* idx1 = ws_at<int>(ws, L.IDX1);
  HIPCHK(launch_stage_couplings(P, ldp, M, N, 1.f, Z, ZT, nullptr, nullptr, st), "stage assignment");
  HIPCHK(launch_col_argmax(ZT, pl.pt, nullptr, idx1, N, m1, s1, EXT_RAW, st), "column argmax");
  HIPCHK(launch_sink_extract(Z, pl.pt, nullptr, nullptr, idx1, M, N, thr, m0, s0, m1, s1, EXT_RAW, st), "extract");
  return SG_OK;
}

sg_status check_stage_sinkhorn(const float* Z, int64_t ldZ, int32_t M, int32_t N, int32_t T, const float* u,
                               const float* v, const float* logP, int64_t ldP) {
  if (M < 1 || N < 1)
    return fail(SG_ERR_INVALID_ARG, "M = %d, N = %d: the optimal-matching layer runs on non-empty images", M, N);
  if (M > 4096 || N > 4096) return fail(SG_ERR_UNSUPPORTED, "more than 4096 points per image");
  if (T < 0) return fail(SG_ERR_INVALID_ARG, "T < 0");
  if (!Z || !u || !v) return fail(SG_ERR_INVALID_ARG, "Z, u or v is NULL");
  if (ldZ < (int64_t)N + 1) return fail(SG_ERR_INVALID_ARG, "ldZ < N+1");
  if (logP && ldP < (int64_t)N + 1) return fail(SG_ERR_INVALID_ARG, "ldP < N+1");
  return SG_OK;
}

// ------------------------------------------ allocation-free Sinkhorn stage
//
// sg_stage_sinkhorn_noalloc keeps its workspace in one fixed device array
// per GPU (held from the library's load until the process ends) instead of
// a caller or library allocation.  In host code `scratch` only names the
// symbol: its device address is looked up once per device with that device
// current, and only that address reaches kernels.  Every call on a GPU
// shares the array and overwrites what the previous call left in it.
constexpr size_t kScratchBytes = size_t(40) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
char* g_scratch_addr[64] = {};

sg_status scratch_address(char** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(SG_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    HIPCHK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SG_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_addr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_addr[dev];
  return SG_OK;
}

sg_status check_opts(const sg_opts* o) {
  if (!o) return SG_OK;
  if (o->workspace && o->workspace_bytes == 0) return fail(SG_ERR_WORKSPACE, "workspace given with 0 bytes");
  if (o->kernel_events && o->n_kernel_events < 0) return fail(SG_ERR_INVALID_ARG, "n_kernel_events < 0");
  if ((o->flags & SG_FLAG_SINKHORN_TWO_SWEEP) && (o->flags & SG_FLAG_SINKHORN_ONE_SWEEP))
    return fail(SG_ERR_INVALID_ARG, "both Sinkhorn schedules forced");
  if (o->depth_confidence < 0.f || o->width_confidence < 0.f || o->width_confidence > 1.f || o->prune_min_points < 0)
    return fail(SG_ERR_INVALID_ARG, "adaptive options out of range");
  return SG_OK;
}

hipStream_t stream_of(const sg_opts* o) { return o ? (hipStream_t)o->stream : (hipStream_t)0; }

// ------------------------------------------------------------ graph replay
//
// The launch sequence of a call depends only on its shapes and pointers, so
// it is captured once into a HIP graph (on a private capture stream) and
// replayed on the caller's stream afterwards, which removes most of the
// per-kernel launch cost of the ~300 small kernels of one pass.  Calls that
// ask for timing events, set SG_FLAG_NO_GRAPH, or arrive on a stream that
// the caller is capturing run eagerly.

struct GraphCache {
  std::mutex mu;
  std::vector<std::pair<std::string, hipGraphExec_t>> entries;
  std::vector<std::string> seen;  // keys called once so far
  hipStream_t cap[64] = {};
};
GraphCache g_graphs;
constexpr size_t kMaxGraphs = 64;

template <class F>
sg_status run_maybe_graph(const std::string& key_in, const sg_opts* o, hipStream_t st, F&& enqueue) {
  bool use = !(o && (o->stage_events || o->kernel_events || (o->flags & SG_FLAG_NO_GRAPH)));
  if (use) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (st && hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone) use = false;
  }
  if (!use) return enqueue(st);
  int dev = 0;
  HIPCHK(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= 64) return enqueue(st);
  std::string key = key_in;
  key.append(reinterpret_cast<const char*>(&dev), sizeof(dev));
  std::lock_guard<std::mutex> lk(g_graphs.mu);
  for (auto& e : g_graphs.entries)
    if (e.first == key) {
      HIPCHK(hipGraphLaunch(e.second, st), "hipGraphLaunch");
      return SG_OK;
    }
  // capture only calls that repeat: the first call with a key runs eagerly
  bool seen = false;
  for (auto& k : g_graphs.seen) seen = seen || k == key;
  if (!seen) {
    if (g_graphs.seen.size() >= 4 * kMaxGraphs) g_graphs.seen.clear();
    g_graphs.seen.push_back(key);
    return enqueue(st);
  }
  if (!g_graphs.cap[dev]) HIPCHK(hipStreamCreateWithFlags(&g_graphs.cap[dev], hipStreamNonBlocking), "capture stream");
  hipStream_t cap = g_graphs.cap[dev];
  HIPCHK(hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
  sg_status s = enqueue(cap);
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(cap, &graph);
  if (s != SG_OK || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return s != SG_OK ? s : hip_fail(e, "hipStreamEndCapture");
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
  if (g_graphs.entries.size() >= kMaxGraphs) {
    // replays already enqueued keep their executable alive until they finish
    HIPCHK(hipDeviceSynchronize(), "hipDeviceSynchronize");
    for (auto& x : g_graphs.entries) (void)hipGraphExecDestroy(x.second);
    g_graphs.entries.clear();
  }
  g_graphs.entries.emplace_back(key, exec);
  HIPCHK(hipGraphLaunch(exec, st), "hipGraphLaunch");
  return SG_OK;
}

template <class T>
void put(std::string& k, const T& v) {
  k.append(reinterpret_cast<const char*>(&v), sizeof(T));
}

std::string call_key(int kind, const Problem& p, const sg_weights* w, int Lst, int T, const Outputs& out,
                     const sg_opts* o, const void* ws) {
  std::string k;
  put(k, kind); put(k, p.B); put(k, p.Mpad); put(k, p.Npad);
  for (int b = 0; b < p.B; ++b) { put(k, p.M[b]); put(k, p.N[b]); }
  for (int i = 0; i < 2; ++i) { put(k, p.kp[i]); put(k, p.cf[i]); put(k, p.de[i]); }
  put(k, p.img);
  if (w) {
    put(k, w->D); put(k, w->H); put(k, w->n_enc);
    for (int i = 0; i < w->n_enc; ++i) put(k, w->enc[i]);
    put(k, w->L_max); put(k, w->dtype); put(k, w->head); put(k, w->cross); put(k, w->rope); put(k, w->adaptive);
    put(k, w->blob); put(k, w->blob_bytes);
  }
  put(k, Lst); put(k, T); put(k, out);
  put(k, o ? o->match_threshold : 0.f);
  put(k, o ? o->flags : 0);
  put(k, ws);
  return k;
}

sg_status enqueue_full(const Problem& p, const Plan& pl, const WsLayout& wl, char* ws, const sg_weights* w,
                       const WLayout& L, int Lst, int T, const Outputs& out, const sg_opts* o, hipStream_t st);

sg_status run_full(const Problem& p, const sg_weights* w, const WLayout& L, int Lst, int T,
                   const Outputs& out, const sg_opts* o) {
  Plan pl;
  make_plan(p, pl);
  const long ssf = (o && (o->flags & SG_FLAG_SHARED_SIMILARITY) && p.B == 1) ? shared_sim_floats(w, p.M[0], p.N[0]) : 0;
  WsLayout wl = ws_layout(w, pl.R, pl.zf, pl.ztf, pl.pf, pl.pd, pl.uf, pl.vf, pl.nb, ssf);
  void* wsp = nullptr;
  sg_status s = get_workspace(o, wl.total, &wsp);
  if (s != SG_OK) return s;
  return run_maybe_graph(call_key(0, p, w, Lst, T, out, o, wsp), o, stream_of(o), [&](hipStream_t st) {
    return enqueue_full(p, pl, wl, reinterpret_cast<char*>(wsp), w, L, Lst, T, out, o, st);
  });
}

sg_status enqueue_full(const Problem& p, const Plan& pl, const WsLayout& wl, char* ws, const sg_weights* w,
                       const WLayout& L, int Lst, int T, const Outputs& out, const sg_opts* o, hipStream_t st) {
  sg_status s;
  Timer tm{o, st};
  // alpha stays in device memory: the Sinkhorn and logP kernels read it there
  const float* alpha_dev = at<float>(w, L, L.alpha);
  tm.stage(SG_EV_START);
  // the merge fold of the pass's stages runs beside the encoder, in its launch
  const int nf = std::min(2 * Lst, kMaxFold);
  if ((s = run_encoder(p, pl, w, L, ws, wl, tm, st, nf)) != SG_OK) return s;
  if (w->rope && (s = run_rope_table(p, pl, w, L, ws, wl, st)) != SG_OK) return s;
  tm.stage(SG_EV_ENCODED);
  if ((s = run_fold(w, L, nf, 2 * Lst, ws, wl, tm, st)) != SG_OK) return s;
  if ((s = run_gnn(pl, w, L, 0, 2 * Lst, ws, wl, o ? o->flags : 0, tm, st, nullptr, true)) != SG_OK) return s;
  tm.stage(SG_EV_GNN);
  float* F = reinterpret_cast<float*>(ws + wl.F);
  if ((s = run_project(pl, w, L, reinterpret_cast<float*>(ws + wl.X), F, tm, st)) != SG_OK) return s;
  for (int b = 0; b < p.B; ++b) {
    if (out.descA && p.M[b])
      HIPCHK(hipMemcpyAsync(out.descA + (size_t)b * p.Mpad * w->D, F + (size_t)pl.seg.row0[2 * b] * w->D,
                            (size_t)p.M[b] * w->D * 4, hipMemcpyDeviceToDevice, st), "copy f_A");
    if (out.descB && p.N[b])
      HIPCHK(hipMemcpyAsync(out.descB + (size_t)b * p.Npad * w->D, F + (size_t)pl.seg.row0[2 * b + 1] * w->D,
                            (size_t)p.N[b] * w->D * 4, hipMemcpyDeviceToDevice, st), "copy f_B");
  }
  const float thr = o ? o->match_threshold : 0.f;
  DsHead ds;
  if (w->head == SG_HEAD_DOUBLE_SOFTMAX) {
    ds.X = reinterpret_cast<const float*>(ws + wl.X);
    ds.w_dtype = w->dtype;
    ds.wz = atv(w, L, L.wz);
    ds.bz_dev = atv(w, L, L.wz + 1);
  }
  if ((s = run_matching(p, pl, w->D, 0.f, alpha_dev, T, thr, w->head == SG_HEAD_DOUBLE_SOFTMAX ? &ds : nullptr, F,
                        ws, wl, out, tm, st)) != SG_OK)
    return s;
  tm.stage(SG_EV_END);
  tm.finish();
  return SG_OK;
}

// ------------------------------------------------- adaptive depth and width
//
// One pair, eager, with the host waiting for every layer's statistics: the
// stop decision and the kept counts are posted into host-visible memory, and
// the host re-plans the row space when points are dropped (as the page's own
// loop does with its Python control flow).

std::mutex g_pin_mu;
int* g_pin[64] = {};      // host-visible, coherent post box per device
int* g_pin_dev[64] = {};  // its device address
int g_adaptive_calls = 0;
// Post slots: layer l posts into slot l % kPostSlots, so that the layer
// enqueued ahead of the host's wait cannot overwrite the post being waited
// for (the host may be descheduled for longer than a layer takes).
constexpr int kPostSlots = 64, kPostSlotInts = 16;

sg_status post_box(int** host, int** dev_ptr) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(SG_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_pin_mu);
  if (!g_pin[dev]) {
    HIPCHK(hipHostMalloc((void**)&g_pin[dev], kPostSlots * kPostSlotInts * sizeof(int),
                         hipHostMallocMapped | hipHostMallocCoherent),
           "hipHostMalloc");
    HIPCHK(hipHostGetDevicePointer((void**)&g_pin_dev[dev], g_pin[dev], 0), "hipHostGetDevicePointer");
    for (int k = 0; k < kPostSlots; ++k) g_pin[dev][k * kPostSlotInts] = -1;
  }
  *host = g_pin[dev];
  *dev_ptr = g_pin_dev[dev];
  return SG_OK;
}

// Spins until the statistics kernel of the layer posts `seq` (bounded: an
// error after ten seconds).
sg_status wait_post(volatile int* box, int seq, hipStream_t st) {
  const auto t0 = std::chrono::steady_clock::now();
  long n = 0;
  while (box[0] != seq) {
    if ((++n & 0xFFFF) == 0) {
      const hipError_t e = hipStreamQuery(st);
      if (e != hipSuccess && e != hipErrorNotReady) return hip_fail(e, "adaptive statistics");
      if (e == hipSuccess && box[0] != seq) return fail(SG_ERR_HIP, "adaptive statistics did not post");
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10))
        return fail(SG_ERR_HIP, "adaptive statistics: no post after 10 s");
    }
  }
  return SG_OK;
}

sg_status run_adaptive(const Problem& p0, const sg_weights* w, const WLayout& L, int Lst, const Outputs& out,
                       const sg_opts* o) {
  hipStream_t st = stream_of(o);
  if (st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
      return fail(SG_ERR_INVALID_ARG, "adaptive calls wait on the host for every layer and cannot be captured");
  }
  const bool depth = o->flags & SG_FLAG_EARLY_EXIT, width = o->flags & SG_FLAG_PRUNE;
  const float alpha = o->depth_confidence > 0.f ? o->depth_confidence : 0.95f;
  const float beta = o->width_confidence > 0.f ? o->width_confidence : 0.99f;
  const int pmin = o->prune_min_points > 0 ? o->prune_min_points : 1024;
  Plan pl;
  make_plan(p0, pl);
  WsLayout wl = ws_layout(w, pl.R, pl.zf, pl.ztf, pl.pf, pl.pd, pl.uf, pl.vf, pl.nb);
  void* wsp = nullptr;
  sg_status s = get_workspace(o, wl.total, &wsp);
  if (s != SG_OK) return s;
  int *box = nullptr, *box_dev = nullptr;
  if ((s = post_box(&box, &box_dev)) != SG_OK) return s;
  char* ws = reinterpret_cast<char*>(wsp);
  const int M = p0.M[0], N = p0.N[0], D = w->D, R0 = pl.R;
  float* X = reinterpret_cast<float*>(ws + wl.X);
  int* IND = reinterpret_cast<int*>(ws + wl.ADAPT);
  int* IND2 = IND + R0;
  int* KEEP = IND + 2 * R0;
  int* NEWIDX = IND + 3 * R0;
  int* CNT = IND + 4 * R0;  // the stop flag at [0]
  int* STOP = CNT;
  int* PART = CNT + 64;      // per-workgroup counts: 4 per 4 points, at most R0 + 4
  int* PR = PART + R0 + 64;
  int32_t* TM0 = PR + R0;
  float* TS0 = reinterpret_cast<float*>(TM0 + R0);
  int32_t* TM1 = reinterpret_cast<int32_t*>(TS0 + R0);
  float* TS1 = reinterpret_cast<float*>(TM1 + R0);
  float* LT = TS1 + R0;
  Timer tm{o, st};
  tm.stage(SG_EV_START);
  HIPCHK(launch_fill_empty(out.m0, out.s0, M, st), "empty output");
  if (out.m1) HIPCHK(launch_fill_empty(out.m1, out.s1, N, st), "empty output");
  HIPCHK(launch_fill_i32(PR, 1, M + N, st), "prune counts");
  HIPCHK(launch_fill_i32(CNT, 0, 64, st), "counters and stop flag");
  if ((s = run_encoder(p0, pl, w, L, ws, wl, tm, st)) != SG_OK) return s;
  HIPCHK(launch_iota_rows(pl.seg, R0, IND, st), "row index");
  if (w->rope && (s = run_rope_table(p0, pl, w, L, ws, wl, st, IND)) != SG_OK) return s;
  tm.stage(SG_EV_ENCODED);
  if ((s = run_fold(w, L, 0, 2 * Lst, ws, wl, tm, st)) != SG_OK) return s;
  const int call = ++g_adaptive_calls & 0xFFFFF;
  const int stat_flags = (depth ? 1 : 0) | (width ? 2 : 0);
  Problem pc = p0;
  Plan cur = pl;
  // Layer l's stages, then (all layers but the last) its statistics, which
  // post their counters and set the device stop flag; every kernel of a
  // later layer checks that flag, so the host may enqueue layer l + 1 before
  // layer l's decision arrives whenever no pruning can reshape the rows.
  bool xb_ok = true;  // the bf16 copy of the states matches X (compaction moves X only)
  auto enqueue_layer = [&](int l) -> sg_status {
    sg_status r = run_gnn(cur, w, L, 2 * l, 2 * l + 2, ws, wl, o->flags, tm, st, STOP, xb_ok);
    xb_ok = true;
    if (r != SG_OK || l == Lst - 1 || !stat_flags) return r;
    const int base = L.adapt + kPerLayerAdaptive * l;
    const float lam = std::min(1.f, std::max(0.f, 0.8f + 0.1f * std::exp(-4.f * l / Lst)));
    HIPCHK(launch_adaptive_stats(X, cur.seg, D, w->dtype, atv(w, L, base), atv(w, L, base + 1),
                                 atv(w, L, base + 4), atv(w, L, base + 5), lam, 1.f - beta, stat_flags, alpha, M + N,
                                 (call << 8) | l, KEEP, PART, STOP, box_dev + kPostSlotInts * (l % kPostSlots), st),
           "confidence");
    return SG_OK;
  };
  int exit_layer = Lst - 1;
  bool empty = false;
  if ((s = enqueue_layer(0)) != SG_OK) return s;
  for (int l = 0; l + 1 < Lst; ++l) {
    // layer l (and its statistics) are enqueued
    if (!stat_flags) {
      if ((s = enqueue_layer(l + 1)) != SG_OK) return s;
      continue;
    }
    const int curM = pc.M[0], curN = pc.N[0];
    const bool may_prune = width && (curM > pmin || curN > pmin);
    if (!may_prune && (s = enqueue_layer(l + 1)) != SG_OK) return s;  // speculative
    volatile int* slot = box + kPostSlotInts * (l % kPostSlots);
    if ((s = wait_post(slot, (call << 8) | l, st)) != SG_OK) return s;
    const int stopped = slot[1], kA = slot[3], kB = slot[5];
    if (stopped) {
      exit_layer = l;
      break;
    }
    if (may_prune) {
      const bool pA = curM > pmin && kA < curM, pB = curN > pmin && kB < curN;
      if (pA || pB) {
        const int mask = (pA ? 1 : 0) | (pB ? 2 : 0);
        Problem pn = pc;
        pn.M = {pA ? kA : curM};
        pn.N = {pB ? kB : curN};
        pn.Mpad = pn.M[0];
        pn.Npad = pn.N[0];
        Plan nx;
        make_plan(pn, nx);
        float* XT = reinterpret_cast<float*>(ws + wl.HB);  // free between layers, at least R D floats
        HIPCHK(launch_prune_scan(cur.seg, KEEP, mask, NEWIDX, st), "prune scan");
        HIPCHK(launch_compact_rows(X, IND, NEWIDX, cur.seg, nx.seg, cur.R, nx.R, D, mask, M, XT, IND2, PR, st),
               "compact rows");
        if (nx.R > 0) {
          HIPCHK(hipMemcpyAsync(X, XT, (size_t)nx.R * D * 4, hipMemcpyDeviceToDevice, st), "copy states");
          HIPCHK(hipMemcpyAsync(IND, IND2, (size_t)nx.R * 4, hipMemcpyDeviceToDevice, st), "copy index");
        }
        pc = pn;
        cur = nx;
        xb_ok = false;
        if (w->rope && (s = run_rope_table(pc, cur, w, L, ws, wl, st, IND)) != SG_OK) return s;
      }
      if (pc.M[0] == 0 || pc.N[0] == 0) {
        exit_layer = l;
        empty = true;
        break;
      }
      if ((s = enqueue_layer(l + 1)) != SG_OK) return s;
    }
  }
  tm.stage(SG_EV_GNN);
  if (!empty) {
    const bool own = exit_layer < w->L_max - 1;  // the layer's own head, else the main one
    const int hb = L.adapt + kPerLayerAdaptive * exit_layer;
    float* F = reinterpret_cast<float*>(ws + wl.F);
    if ((s = run_project(cur, w, L, X, F, tm, st, own ? hb + 2 : L.final_first)) != SG_OK) return s;
    DsHead ds;
    ds.X = X;
    ds.w_dtype = w->dtype;
    ds.wz = atv(w, L, own ? hb + 4 : L.wz);
    ds.bz_dev = atv(w, L, own ? hb + 5 : L.wz + 1);
    Outputs to;
    to.m0 = TM0; to.s0 = TS0; to.m1 = TM1; to.s1 = TS1;
    to.logP = out.logP ? LT : nullptr;
    to.logP_ld = pc.N[0] + 1;
    if ((s = run_matching(pc, cur, D, 0.f, nullptr, 0, o->match_threshold, &ds, F, ws, wl, to, tm, st)) != SG_OK)
      return s;
    HIPCHK(launch_scatter_outputs(cur.seg, IND, TM0, TS0, TM1, TS1, out.m0, out.s0, out.m1, out.s1, F, D, out.descA,
                                  out.descB, to.logP, M, N, out.logP, out.logP_ld, cur.R, st), "scatter outputs");
  }
  if (o->out_prune0 && M) HIPCHK(hipMemcpyAsync(o->out_prune0, PR, (size_t)M * 4, hipMemcpyDeviceToDevice, st), "prune0");
  if (o->out_prune1 && N) HIPCHK(hipMemcpyAsync(o->out_prune1, PR + M, (size_t)N * 4, hipMemcpyDeviceToDevice, st), "prune1");
  if (o->out_exit_layer) *o->out_exit_layer = exit_layer;
  tm.stage(SG_EV_END);
  tm.finish();
  return SG_OK;
}

}  // namespace

extern "C" {

const char* sg_last_error(void) { return g_err.c_str(); }
const char* sg_version(void) { return "sg-mi355x 0.1 (gfx950)"; }

int32_t sg_weights_count(const sg_weights* w) {
  if (check_config(w) != SG_OK) return -1;
  return (int32_t)layout_of(w).t.size();
}

sg_status sg_weights_tensor(const sg_weights* w, int32_t index, size_t* offset, int32_t* rows, int32_t* cols) {
  sg_status s = check_config(w);
  if (s != SG_OK) return s;
  WLayout L = layout_of(w);
  if (index < 0 || index >= (int32_t)L.t.size()) return fail(SG_ERR_INVALID_ARG, "tensor index %d out of range", index);
  if (offset) *offset = L.t[index].off;
  if (rows) *rows = L.t[index].rows;
  if (cols) *cols = L.t[index].cols;
  return SG_OK;
}

size_t sg_weights_bytes(const sg_weights* w) {
  if (check_config(w) != SG_OK) return 0;
  return layout_of(w).bytes;
}

size_t sg_workspace_size(const sg_weights* w, int32_t Mmax, int32_t Nmax, int32_t batch) {
  if (check_config(w) != SG_OK || Mmax < 0 || Nmax < 0 || batch < 1) return 0;
  const long B = batch;
  const long R = B * (round32(Mmax) + round32(Nmax));
  // the transposed scores exist only for the two-sweep schedule, which the
  // default rule picks for at most SG_TWO_SWEEP_MAX_BYTES of Z (ZT exceeds Z
  // by at most its row padding), and for the double-softmax head
  const long ztf = w->head == SG_HEAD_DOUBLE_SOFTMAX
                       ? B * Nmax * ld4(Mmax)
                       : std::min(B * Nmax * ld4(Mmax), (long)(SG_TWO_SWEEP_MAX_BYTES / 4) + 3 * B * Nmax);
  // column partials: at most ceil((Mmax+1)/4) row blocks per pair
  const long G = (Mmax + 4) / 4;
  const bool ds = w->head == SG_HEAD_DOUBLE_SOFTMAX;  // no column partials
  // (one pair of a bidirectional network: room for SG_FLAG_SHARED_SIMILARITY)
  WsLayout wl = ws_layout(w, R, B * Mmax * ld4(Nmax), ztf, ds ? 0 : B * G * ld4(Nmax), ds ? 0 : B * G,
                          B * ld4(Mmax + 1), B * ld4(Nmax + 1), B * Nmax, B == 1 ? shared_sim_floats(w, Mmax, Nmax) : 0);
  return wl.total;
}

size_t sg_stage_match_workspace_size(int32_t M, int32_t N, int32_t D) {
  if (M < 0 || N < 0 || D <= 0) return 0;
  const long R = round32(M) + round32(N);
  const long ztf = std::min((long)N * ld4(M), (long)(SG_TWO_SWEEP_MAX_BYTES / 4) + 3L * N);
  const long G = (M + 4) / 4;
  return ws_layout_raw(D, 4, R, (long)M * ld4(N), ztf, G * ld4(N), G, ld4(M + 1), ld4(N + 1), N).total;
}

sg_status sg_match(const float* kptsA, const float* descA, const float* confA, int32_t M,
                   const float* kptsB, const float* descB, const float* confB, int32_t N,
                   const sg_weights* weights, int32_t L, int32_t T, int32_t* out_matches,
                   float* out_scores, const sg_opts* opts) {
  g_err.clear();
  WLayout WL;
  sg_status s = check_weights(weights, &WL);
  if (s != SG_OK) return s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (M < 0 || N < 0) return fail(SG_ERR_INVALID_ARG, "negative point count");
  if (M > 4096 || N > 4096) return fail(SG_ERR_UNSUPPORTED, "more than 4096 points per image");
  if (L < 1 || L > weights->L_max) return fail(SG_ERR_INVALID_ARG, "L = %d outside [1, %d]", L, weights->L_max);
  if (T < 0) return fail(SG_ERR_INVALID_ARG, "T < 0");
  if ((M > 0 && !out_matches) || (M > 0 && !out_scores)) return fail(SG_ERR_INVALID_ARG, "out_matches/out_scores is NULL");
  if (M > 0 && N > 0 && (!kptsA || !descA || !confA || !kptsB || !descB || !confB))
    return fail(SG_ERR_INVALID_ARG, "input pointer is NULL");
  if (opts && opts->out_logP && opts->logP_ld < N + 1) return fail(SG_ERR_INVALID_ARG, "logP_ld < N+1");
  hipStream_t st = stream_of(opts);
  if (M == 0 || N == 0) {
    HIPCHK(launch_fill_empty(out_matches, out_scores, M, st), "empty output");
    if (opts && opts->out_matches1) HIPCHK(launch_fill_empty(opts->out_matches1, opts->out_scores1, N, st), "empty output");
    return SG_OK;
  }
  Problem p;
  p.flags = opts ? opts->flags : 0;
  p.head = weights->head;
  p.B = 1; p.Mpad = M; p.Npad = N;
  p.M = {M}; p.N = {N};
  p.kp[0] = kptsA; p.cf[0] = confA; p.de[0] = descA;
  p.kp[1] = kptsB; p.cf[1] = confB; p.de[1] = descB;
  if (opts) memcpy(p.img, opts->image_size, sizeof(p.img));
  Outputs out;
  out.m0 = out_matches; out.s0 = out_scores;
  if (opts) {
    out.m1 = opts->out_matches1; out.s1 = opts->out_scores1;
    out.descA = opts->out_desc_A; out.descB = opts->out_desc_B;
    out.logP = opts->out_logP; out.logP_ld = opts->logP_ld; out.logP_stride = 0;
  }
  if (opts && (opts->flags & SG_FLAG_SHARED_SIMILARITY)) {
    if (weights->cross != SG_CROSS_BIDIRECTIONAL)
      return fail(SG_ERR_INVALID_ARG, "a shared similarity needs bidirectional cross-attention weights");
    if (opts->flags & (SG_FLAG_EARLY_EXIT | SG_FLAG_PRUNE))
      return fail(SG_ERR_UNSUPPORTED, "a shared similarity is not combined with adaptive depth / width");
  }
  if (opts && (opts->flags & (SG_FLAG_EARLY_EXIT | SG_FLAG_PRUNE))) {
    if (!weights->adaptive) return fail(SG_ERR_INVALID_ARG, "adaptive flags need adaptive weights");
    return run_adaptive(p, weights, WL, L, out, opts);
  }
  return run_full(p, weights, WL, L, T, out, opts);
}

sg_status sg_match_batch(int32_t B, int32_t Mpad, int32_t Npad, const int32_t* M, const int32_t* N,
                         const float* kptsA, const float* descA, const float* confA,
                         const float* kptsB, const float* descB, const float* confB,
                         const sg_weights* weights, int32_t L, int32_t T, int32_t* out_matches,
                         float* out_scores, const sg_opts* opts) {
  g_err.clear();
  WLayout WL;
  sg_status s = check_weights(weights, &WL);
  if (s != SG_OK) return s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (B < 1 || B > SG_MAX_BATCH) return fail(SG_ERR_INVALID_ARG, "B = %d outside [1, %d]", B, SG_MAX_BATCH);
  if (opts && (opts->flags & (SG_FLAG_EARLY_EXIT | SG_FLAG_PRUNE)))
    return fail(SG_ERR_UNSUPPORTED, "adaptive depth / width runs one pair per call (sg_match)");
  if (opts && (opts->flags & SG_FLAG_SHARED_SIMILARITY))
    return fail(SG_ERR_UNSUPPORTED, "the shared similarity runs one pair per call (sg_match)");
  if (!M || !N) return fail(SG_ERR_INVALID_ARG, "M/N host arrays are NULL");
  if (Mpad < 0 || Npad < 0 || Mpad > 4096 || Npad > 4096) return fail(SG_ERR_UNSUPPORTED, "Mpad/Npad outside [0, 4096]");
  for (int b = 0; b < B; ++b)
    if (M[b] < 0 || M[b] > Mpad || N[b] < 0 || N[b] > Npad)
      return fail(SG_ERR_INVALID_ARG, "pair %d: counts (%d, %d) outside [0, pad]", b, M[b], N[b]);
  if (L < 1 || L > weights->L_max) return fail(SG_ERR_INVALID_ARG, "L = %d outside [1, %d]", L, weights->L_max);
  if (T < 0) return fail(SG_ERR_INVALID_ARG, "T < 0");
  if (!out_matches || !out_scores) return fail(SG_ERR_INVALID_ARG, "out_matches/out_scores is NULL");
  if (!kptsA || !descA || !confA || !kptsB || !descB || !confB) return fail(SG_ERR_INVALID_ARG, "input pointer is NULL");
  if (opts && opts->out_logP && opts->logP_ld < Npad + 1) return fail(SG_ERR_INVALID_ARG, "logP_ld < Npad+1");
  Problem p;
  p.flags = opts ? opts->flags : 0;
  p.head = weights->head;
  p.B = B; p.Mpad = Mpad; p.Npad = Npad;
  p.M.assign(M, M + B); p.N.assign(N, N + B);
  p.kp[0] = kptsA; p.cf[0] = confA; p.de[0] = descA;
  p.kp[1] = kptsB; p.cf[1] = confB; p.de[1] = descB;
  if (opts) memcpy(p.img, opts->image_size, sizeof(p.img));
  Outputs out;
  out.m0 = out_matches; out.s0 = out_scores;
  if (opts) {
    out.m1 = opts->out_matches1; out.s1 = opts->out_scores1;
    out.descA = opts->out_desc_A; out.descB = opts->out_desc_B;
    out.logP = opts->out_logP; out.logP_ld = opts->logP_ld; out.logP_stride = (int64_t)(Mpad + 1) * opts->logP_ld;
  }
  return run_full(p, weights, WL, L, T, out, opts);
}

sg_status sg_stage_encode(const float* kpts, const float* conf, const float* desc, int32_t n, float image_w,
                          float image_h, const sg_weights* weights, float* x_out, const sg_opts* opts) {
  g_err.clear();
  WLayout WL;
  sg_status s = check_weights(weights, &WL);
  if (s != SG_OK) return s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (n < 0 || n > 4096) return fail(SG_ERR_INVALID_ARG, "n = %d outside [0, 4096]", n);
  if (n == 0) return SG_OK;
  if (!kpts || !conf || !desc || !x_out) return fail(SG_ERR_INVALID_ARG, "NULL pointer");
  Problem p;
  p.flags = opts ? opts->flags : 0;
  p.B = 1; p.Mpad = n; p.Npad = 0; p.M = {n}; p.N = {0};
  p.kp[0] = kpts; p.cf[0] = conf; p.de[0] = desc;
  p.kp[1] = kpts; p.cf[1] = conf; p.de[1] = desc;
  p.img[0] = image_w; p.img[1] = image_h;
  Plan pl;
  make_plan(p, pl);
  WsLayout wl = ws_layout(weights, pl.R, 0, 0, 0, 0, 0, 0, 0);
  void* wsp;
  if ((s = get_workspace(opts, wl.total, &wsp)) != SG_OK) return s;
  hipStream_t st = stream_of(opts);
  Timer tm{opts, st};
  if ((s = run_encoder(p, pl, weights, WL, reinterpret_cast<char*>(wsp), wl, tm, st)) != SG_OK) return s;
  HIPCHK(hipMemcpyAsync(x_out, reinterpret_cast<char*>(wsp) + wl.X, (size_t)n * weights->D * 4,
                        hipMemcpyDeviceToDevice, st), "copy x");
  tm.finish();
  return SG_OK;
}

sg_status sg_stage_gnn_pos(float* xA, const float* posA, int32_t M, float* xB, const float* posB, int32_t N,
                           const sg_weights* weights, int32_t s0, int32_t s1, const sg_opts* opts) {
  g_err.clear();
  WLayout WL;
  sg_status s = check_weights(weights, &WL);
  if (s != SG_OK) return s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (M < 0 || N < 0 || M > 4096 || N > 4096) return fail(SG_ERR_INVALID_ARG, "counts outside [0, 4096]");
  if (s0 < 0 || s1 < s0 || s1 > 2 * weights->L_max) return fail(SG_ERR_INVALID_ARG, "stage range [%d, %d) invalid", s0, s1);
  if ((M && !xA) || (N && !xB)) return fail(SG_ERR_INVALID_ARG, "NULL state pointer");
  if (weights->rope && ((M && !posA) || (N && !posB)))
    return fail(SG_ERR_INVALID_ARG, "rotary self-attention needs the point positions");
  const bool shared = opts && (opts->flags & SG_FLAG_SHARED_SIMILARITY);
  if (shared && weights->cross != SG_CROSS_BIDIRECTIONAL)
    return fail(SG_ERR_INVALID_ARG, "a shared similarity needs bidirectional cross-attention weights");
  Problem p;
  p.flags = opts ? opts->flags : 0;
  p.B = 1; p.Mpad = M; p.Npad = N; p.M = {M}; p.N = {N};
  p.kp[0] = posA; p.kp[1] = posB;
  if (opts) memcpy(p.img, opts->image_size, sizeof(p.img));
  Plan pl;
  make_plan(p, pl);
  WsLayout wl = ws_layout(weights, pl.R, 0, 0, 0, 0, 0, 0, 0, shared ? shared_sim_floats(weights, M, N) : 0);
  void* wsp;
  if ((s = get_workspace(opts, wl.total, &wsp)) != SG_OK) return s;
  char* ws = reinterpret_cast<char*>(wsp);
  hipStream_t st = stream_of(opts);
  const size_t rb = (size_t)weights->D * 4;
  float* X = reinterpret_cast<float*>(ws + wl.X);
  if (M) HIPCHK(hipMemcpyAsync(X, xA, M * rb, hipMemcpyDeviceToDevice, st), "copy xA");
  if (N) HIPCHK(hipMemcpyAsync(X + (size_t)pl.seg.row0[1] * weights->D, xB, N * rb, hipMemcpyDeviceToDevice, st), "copy xB");
  // the 32-row padding of each image is zero, as the encoder leaves it
  HIPCHK(launch_fill_f32(X + (size_t)M * weights->D, 0.f, (pl.seg.row0[1] - M) * weights->D, st), "zero padding A");
  HIPCHK(launch_fill_f32(X + (size_t)(pl.seg.row0[1] + N) * weights->D, 0.f, (pl.R - pl.seg.row0[1] - N) * weights->D, st),
         "zero padding B");
  if (weights->rope && (s = run_rope_table(p, pl, weights, WL, ws, wl, st)) != SG_OK) return s;
  Timer tm{opts, st};
  if ((s = run_fold(weights, WL, s0, s1, ws, wl, tm, st)) != SG_OK) return s;
  if ((s = run_gnn(pl, weights, WL, s0, s1, ws, wl, opts ? opts->flags : 0, tm, st)) != SG_OK) return s;
  if (M) HIPCHK(hipMemcpyAsync(xA, X, M * rb, hipMemcpyDeviceToDevice, st), "copy xA back");
  if (N) HIPCHK(hipMemcpyAsync(xB, X + (size_t)pl.seg.row0[1] * weights->D, N * rb, hipMemcpyDeviceToDevice, st), "copy xB back");
  tm.finish();
  return SG_OK;
}

sg_status sg_stage_gnn(float* xA, int32_t M, float* xB, int32_t N, const sg_weights* weights, int32_t s0,
                       int32_t s1, const sg_opts* opts) {
  return sg_stage_gnn_pos(xA, nullptr, M, xB, nullptr, N, weights, s0, s1, opts);
}

sg_status sg_stage_project(const float* x, int32_t n, const sg_weights* weights, float* f_out, const sg_opts* opts) {
  g_err.clear();
  WLayout WL;
  sg_status s = check_weights(weights, &WL);
  if (s != SG_OK) return s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (n < 0) return fail(SG_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return SG_OK;
  if (!x || !f_out) return fail(SG_ERR_INVALID_ARG, "NULL pointer");
  Plan pl;
  pl.R = n;
  hipStream_t st = stream_of(opts);
  Timer tm{opts, st};
  if ((s = run_project(pl, weights, WL, x, f_out, tm, st)) != SG_OK) return s;
  tm.finish();
  return SG_OK;
}

// Workspace of sg_stage_scores: f_A [M][D], f_B [N][D], S [M][ld4(N)].
static size_t scores_ws(int32_t M, int32_t N, int32_t D, size_t* oB, size_t* oS) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t a = up((size_t)M * D * 4), b = up((size_t)N * D * 4), c = up((size_t)M * ld4(N) * 4);
  if (oB) *oB = a;
  if (oS) *oS = a + b;
  return std::max<size_t>(a + b + c, 256);
}

size_t sg_stage_scores_workspace_size(int32_t M, int32_t N, int32_t D) {
  if (M < 0 || N < 0 || D <= 0) return 0;
  return scores_ws(M, N, D, nullptr, nullptr);
}

sg_status sg_stage_scores(const float* xA, int32_t M, const float* xB, int32_t N, const sg_weights* weights,
                          float* Z, int64_t ldZ, const sg_opts* opts) {
  g_err.clear();
  WLayout WL;
  sg_status s = check_weights(weights, &WL);
  if (s != SG_OK) return s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (M < 0 || N < 0) return fail(SG_ERR_INVALID_ARG, "negative point count");
  if (M > 4096 || N > 4096) return fail(SG_ERR_UNSUPPORTED, "more than 4096 points per image");
  if (!Z) return fail(SG_ERR_INVALID_ARG, "Z is NULL");
  if (ldZ < (int64_t)N + 1) return fail(SG_ERR_INVALID_ARG, "ldZ < N+1");
  if ((M > 0 && !xA) || (N > 0 && !xB)) return fail(SG_ERR_INVALID_ARG, "NULL states");
  const int D = weights->D;
  size_t oB, oS;
  void* wsp;
  if ((s = get_workspace(opts, scores_ws(M, N, D, &oB, &oS), &wsp)) != SG_OK) return s;
  char* ws = reinterpret_cast<char*>(wsp);
  float* FA = reinterpret_cast<float*>(ws);
  float* FB = reinterpret_cast<float*>(ws + oB);
  float* S = reinterpret_cast<float*>(ws + oS);
  hipStream_t st = stream_of(opts);
  Timer tm{opts, st};
  const float* alpha_dev = at<float>(weights, WL, WL.alpha);
  if (M > 0 && N > 0) {
    Plan pa, pb;
    pa.R = M;
    pb.R = N;
    if ((s = run_project(pa, weights, WL, xA, FA, tm, st)) != SG_OK) return s;
    if ((s = run_project(pb, weights, WL, xB, FB, tm, st)) != SG_OK) return s;
    // S = f_A f_B^T / sqrt(D), natural log (the pass keeps it times log2 e)
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.A0 = FA; g.lda0 = D; g.K0 = D; g.K = D;
    g.W = FB; g.ldw = D;
    g.C = S; g.C2 = nullptr;
    g.scale = 1.f / sqrtf((float)D);
    GemmBatch b;
    memset(&b, 0, sizeof(b));
    b.n = 1;
    b.p[0] = GemmProblem{0, 0, M, N, 0, 0, ld4(N), 0};
    HIPCHK(tm.run(SG_K_GEMM, [&] { return launch_gemm(SG_F32, 1, SG_F32, 1, EPI_SCORE, g, b, M, N, st); }),
           "score GEMM");
  }
  HIPCHK(launch_stage_border(S, ld4(N), M, N, alpha_dev, Z, ldZ, st), "bordered scores");
  tm.finish();
  return SG_OK;
}

sg_status sg_stage_match(const float* fA, int32_t M, const float* fB, int32_t N, int32_t D, float alpha, int32_t T,
                         int32_t* out_matches, float* out_scores, const sg_opts* opts) {
  g_err.clear();
  sg_status s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (M < 0 || N < 0) return fail(SG_ERR_INVALID_ARG, "negative point count");
  if (M > 4096 || N > 4096) return fail(SG_ERR_UNSUPPORTED, "more than 4096 points per image");
  if (D <= 0 || D % 8) return fail(SG_ERR_UNSUPPORTED, "D = %d (must be a positive multiple of 8)", D);
  if (T < 0) return fail(SG_ERR_INVALID_ARG, "T < 0");
  if (M > 0 && (!out_matches || !out_scores)) return fail(SG_ERR_INVALID_ARG, "NULL output");
  if (M > 0 && N > 0 && (!fA || !fB)) return fail(SG_ERR_INVALID_ARG, "NULL descriptors");
  if (opts && opts->out_logP && opts->logP_ld < N + 1) return fail(SG_ERR_INVALID_ARG, "logP_ld < N+1");
  hipStream_t st = stream_of(opts);
  if (M == 0 || N == 0) {
    HIPCHK(launch_fill_empty(out_matches, out_scores, M, st), "empty output");
    if (opts && opts->out_matches1) HIPCHK(launch_fill_empty(opts->out_matches1, opts->out_scores1, N, st), "empty output");
    return SG_OK;
  }
  Problem p;
  p.flags = opts ? opts->flags : 0;
  p.B = 1; p.Mpad = M; p.Npad = N; p.M = {M}; p.N = {N};
  Plan pl;
  make_plan(p, pl);
  // f_A and f_B are staged into the compact F rows of the workspace
  WsLayout wl = ws_layout_raw(D, 4, pl.R, pl.zf, pl.ztf, pl.pf, pl.pd, pl.uf, pl.vf, pl.nb);
  void* wsp;
  if ((s = get_workspace(opts, wl.total, &wsp)) != SG_OK) return s;
  char* ws = reinterpret_cast<char*>(wsp);
  float* F = reinterpret_cast<float*>(ws + wl.F);
  Outputs out;
  out.m0 = out_matches; out.s0 = out_scores;
  if (opts) {
    out.m1 = opts->out_matches1; out.s1 = opts->out_scores1;
    out.logP = opts->out_logP; out.logP_ld = opts->logP_ld;
  }
  p.kp[0] = fA; p.kp[1] = fB;  // part of the replay key
  std::string key = call_key(1, p, nullptr, D, T, out, opts, wsp);
  key.append(reinterpret_cast<const char*>(&alpha), sizeof(alpha));
  return run_maybe_graph(key, opts, st, [&](hipStream_t cs) -> sg_status {
    HIPCHK(hipMemcpyAsync(F, fA, (size_t)M * D * 4, hipMemcpyDeviceToDevice, cs), "copy fA");
    HIPCHK(hipMemcpyAsync(F + (size_t)pl.seg.row0[1] * D, fB, (size_t)N * D * 4, hipMemcpyDeviceToDevice, cs),
           "copy fB");
    Timer tm{opts, cs};
    tm.stage(SG_EV_GNN);
    sg_status r = run_matching(p, pl, D, alpha, nullptr, T, opts ? opts->match_threshold : 0.f, nullptr, F, ws, wl,
                               out, tm, cs);
    if (r != SG_OK) return r;
    tm.stage(SG_EV_END);
    tm.finish();
    return SG_OK;
  });
}

size_t sg_stage_match_ds_workspace_size(int32_t M, int32_t N, int32_t D) {
  if (M < 0 || N < 0 || D <= 0) return 0;
  const long R = round32(M) + round32(N);
  return ws_layout_raw(D, 4, R, (long)M * ld4(N), (long)N * ld4(M), 0, 0, ld4(M + 1), ld4(N + 1), N).total;
}

sg_status sg_stage_match_ds(const float* fA, const float* xA, int32_t M, const float* fB, const float* xB,
                            int32_t N, int32_t D, const float* w_z, float b_z, int32_t* out_matches,
                            float* out_scores, const sg_opts* opts) {
  g_err.clear();
  sg_status s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (M < 0 || N < 0) return fail(SG_ERR_INVALID_ARG, "negative point count");
  if (M > 4096 || N > 4096) return fail(SG_ERR_UNSUPPORTED, "more than 4096 points per image");
  if (D <= 0 || D % 8) return fail(SG_ERR_UNSUPPORTED, "D = %d (must be a positive multiple of 8)", D);
  if (M > 0 && (!out_matches || !out_scores)) return fail(SG_ERR_INVALID_ARG, "NULL output");
  if (M > 0 && N > 0 && (!fA || !fB || !xA || !xB || !w_z)) return fail(SG_ERR_INVALID_ARG, "NULL input");
  if (opts && opts->out_logP && opts->logP_ld < N + 1) return fail(SG_ERR_INVALID_ARG, "logP_ld < N+1");
  hipStream_t st = stream_of(opts);
  if (M == 0 || N == 0) {
    HIPCHK(launch_fill_empty(out_matches, out_scores, M, st), "empty output");
    if (opts && opts->out_matches1) HIPCHK(launch_fill_empty(opts->out_matches1, opts->out_scores1, N, st), "empty output");
    return SG_OK;
  }
  Problem p;
  p.flags = opts ? opts->flags : 0;
  p.head = SG_HEAD_DOUBLE_SOFTMAX;
  p.B = 1; p.Mpad = M; p.Npad = N; p.M = {M}; p.N = {N};
  Plan pl;
  make_plan(p, pl);
  // f and x are staged into the compact F and X rows of the workspace
  WsLayout wl = ws_layout_raw(D, 4, pl.R, pl.zf, pl.ztf, pl.pf, pl.pd, pl.uf, pl.vf, pl.nb);
  void* wsp;
  if ((s = get_workspace(opts, wl.total, &wsp)) != SG_OK) return s;
  char* ws = reinterpret_cast<char*>(wsp);
  float* F = reinterpret_cast<float*>(ws + wl.F);
  float* X = reinterpret_cast<float*>(ws + wl.X);
  Outputs out;
  out.m0 = out_matches; out.s0 = out_scores;
  if (opts) {
    out.m1 = opts->out_matches1; out.s1 = opts->out_scores1;
    out.logP = opts->out_logP; out.logP_ld = opts->logP_ld;
  }
  p.kp[0] = fA; p.kp[1] = fB; p.cf[0] = xA; p.cf[1] = xB; p.de[0] = w_z;  // part of the replay key
  std::string key = call_key(2, p, nullptr, D, 0, out, opts, wsp);
  key.append(reinterpret_cast<const char*>(&b_z), sizeof(b_z));
  DsHead ds;
  ds.X = X; ds.w_dtype = SG_F32; ds.wz = w_z; ds.bz = b_z;
  return run_maybe_graph(key, opts, st, [&](hipStream_t cs) -> sg_status {
    const size_t rb = (size_t)D * 4;
    const size_t rowB = (size_t)pl.seg.row0[1] * D;
    HIPCHK(hipMemcpyAsync(F, fA, M * rb, hipMemcpyDeviceToDevice, cs), "copy fA");
    HIPCHK(hipMemcpyAsync(F + rowB, fB, N * rb, hipMemcpyDeviceToDevice, cs), "copy fB");
    HIPCHK(hipMemcpyAsync(X, xA, M * rb, hipMemcpyDeviceToDevice, cs), "copy xA");
    HIPCHK(hipMemcpyAsync(X + rowB, xB, N * rb, hipMemcpyDeviceToDevice, cs), "copy xB");
    Timer tm{opts, cs};
    tm.stage(SG_EV_GNN);
    sg_status r = run_matching(p, pl, D, 0.f, nullptr, 0, opts ? opts->match_threshold : 0.f, &ds, F, ws, wl, out,
                               tm, cs);
    if (r != SG_OK) return r;
    tm.stage(SG_EV_END);
    tm.finish();
    return SG_OK;
  });
}

size_t sg_stage_sinkhorn_workspace_size(int32_t M, int32_t N) {
  if (M < 0 || N < 0) return 0;
  return stage_ws(M, N).total;
}

sg_status sg_stage_sinkhorn(const float* Z, int64_t ldZ, int32_t M, int32_t N, int32_t T, float* u, float* v,
                            float* logP, int64_t ldP, const sg_opts* opts) {
  g_err.clear();
  sg_status s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if ((s = check_stage_sinkhorn(Z, ldZ, M, N, T, u, v, logP, ldP)) != SG_OK) return s;
  const StageWs L = stage_ws(M, N);
  void* wsp;
  if ((s = get_workspace(opts, L.total, &wsp)) != SG_OK) return s;
  std::string key;
  put(key, 3); put(key, Z); put(key, ldZ); put(key, M); put(key, N); put(key, T); put(key, u); put(key, v);
  put(key, logP); put(key, ldP); put(key, wsp);
  return run_maybe_graph(key, opts, stream_of(opts), [&](hipStream_t cs) -> sg_status {
    return enqueue_stage_sinkhorn(Z, ldZ, M, N, T, u, v, logP, ldP, reinterpret_cast<char*>(wsp), L, cs);
  });
}

sg_status sg_stage_extract(const float* logP, int64_t ldP, int32_t M, int32_t N, float threshold,
                           int32_t* out_matches0, float* out_scores0, int32_t* out_matches1, float* out_scores1,
                           const sg_opts* opts) {
  g_err.clear();
  sg_status s;
  if ((s = check_opts(opts)) != SG_OK) return s;
  if (M < 0 || N < 0) return fail(SG_ERR_INVALID_ARG, "negative point count");
  if (M > 4096 || N > 4096) return fail(SG_ERR_UNSUPPORTED, "more than 4096 points per image");
  if (M > 0 && (!out_matches0 || !out_scores0)) return fail(SG_ERR_INVALID_ARG, "out_matches0/out_scores0 is NULL");
  if (out_scores1 && !out_matches1) return fail(SG_ERR_INVALID_ARG, "out_scores1 without out_matches1");
  if (M > 0 && N > 0 && !logP) return fail(SG_ERR_INVALID_ARG, "logP is NULL");
  if (M > 0 && N > 0 && ldP < (int64_t)N + 1) return fail(SG_ERR_INVALID_ARG, "ldP < N+1");
  hipStream_t st = stream_of(opts);
  if (M == 0 || N == 0) {
    HIPCHK(launch_fill_empty(out_matches0, out_scores0, M, st), "empty output");
    if (out_matches1) HIPCHK(launch_fill_empty(out_matches1, out_scores1, N, st), "empty output");
    return SG_OK;
  }
  const StageWs L = stage_ws(M, N);
  void* wsp;
  if ((s = get_workspace(opts, L.total, &wsp)) != SG_OK) return s;
  std::string key;
  put(key, 4); put(key, logP); put(key, ldP); put(key, M); put(key, N); put(key, threshold); put(key, out_matches0);
  put(key, out_scores0); put(key, out_matches1); put(key, out_scores1); put(key, wsp);
  return run_maybe_graph(key, opts, st, [&](hipStream_t cs) -> sg_status {
    return enqueue_stage_extract(logP, ldP, M, N, threshold, out_matches0, out_scores0, out_matches1, out_scores1,
                                 reinterpret_cast<char*>(wsp), L, cs);
  });
}

sg_status sg_stage_sinkhorn_noalloc(const float* Z, int64_t ldZ, int32_t M, int32_t N, int32_t T, float* u,
                                    float* v, float* logP, int64_t ldP, sg_stream_t stream) {
  g_err.clear();
  sg_status s;
  if ((s = check_stage_sinkhorn(Z, ldZ, M, N, T, u, v, logP, ldP)) != SG_OK) return s;
  const StageWs L = stage_ws(M, N);
  if (L.total > kScratchBytes)
    return fail(SG_ERR_UNSUPPORTED, "%d x %d points need %zu bytes of scratch, the fixed array holds %zu", M, N,
                L.total, kScratchBytes);
  char* ws = nullptr;
  if ((s = scratch_address(&ws)) != SG_OK) return s;
  return enqueue_stage_sinkhorn(Z, ldZ, M, N, T, u, v, logP, ldP, ws, L, (hipStream_t)stream);
}

}  // extern "C"
