// Adaptive depth and width of one pair (gfx950), after sections 2.6 and 2.7
// of the vincentqin.tech review of LightGlue ("论文解读:LightGlue,让稀疏
// 特征匹配随难度自适应地快").
//
// Between layers the pair's points live in the compact row space of the
// current plan (image A's remaining points, then B's, each padded to 32
// rows); `ind` maps every row to the point's original index (-1 on padding).
//  * k_adaptive_stats: one wave per remaining point: token confidence and
//    matchability dot products, the keep decision, per-workgroup counts;
//    k_adaptive_decide sums them, takes the stop decision on the device and
//    posts the counts to host-visible memory.
//  * k_prune_scan: one workgroup per image: the rank of each kept row.
//  * k_compact_rows: copies kept rows (state and index) into the next plan's
//    layout, zeroes its padding rows and counts the pruning steps survived.
//  * k_scatter_*: the exit head's outputs, computed on the remaining points,
//    written to the original indices.
#include <algorithm>

#include "sg_device.h"

namespace sg {

namespace {
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float sigmoid(float t) { return 1.f / (1.f + expf(-t)); }

// segment (image) of compact row r: the last one starting at or before it
__device__ __forceinline__ int seg_of_row(const SegTable& seg, int r) {
  int s = 0;
  while (s + 1 < seg.n_seg && seg.row0[s + 1] <= r) ++s;
  return s;
}
}  // namespace

__global__ void k_iota_rows(SegTable seg, int R, int* __restrict__ ind) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const int s = seg_of_row(seg, r);
  const int p = r - seg.row0[s];
  ind[r] = p < seg.n[s] ? p : -1;
}

__global__ void k_fill_i32(int* __restrict__ p, int v, int n) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < n) p[t] = v;
}

// One remaining point (image s, position t): confidence and matchability
// dot products (one wave) and the keep decision; returns (unconfident, kept)
// in lane 0.
template <typename WT>
__device__ __forceinline__ int2 point_stats(const float* __restrict__ X, const SegTable& seg, int D,
                                            const WT* __restrict__ wc, const WT* __restrict__ bc,
                                            const WT* __restrict__ wz, const WT* __restrict__ bz, float lam,
                                            float min_match, int flags, int* __restrict__ keep, int s, int t,
                                            int lane) {
  const int r = seg.row0[s] + t;
  const float* x = X + (size_t)r * D;
  float ac = 0.f, az = 0.f;
  for (int d = 4 * lane; d < D; d += 256) {
    const float4 v = *reinterpret_cast<const float4*>(x + d);
    if (flags & 1) {
      ac = fmaf(v.x, to_f(wc[d]), ac);
      ac = fmaf(v.y, to_f(wc[d + 1]), ac);
      ac = fmaf(v.z, to_f(wc[d + 2]), ac);
      ac = fmaf(v.w, to_f(wc[d + 3]), ac);
    }
    if (flags & 2) {
      az = fmaf(v.x, to_f(wz[d]), az);
      az = fmaf(v.y, to_f(wz[d + 1]), az);
      az = fmaf(v.z, to_f(wz[d + 2]), az);
      az = fmaf(v.w, to_f(wz[d + 3]), az);
    }
  }
  ac = wave_sum(ac);
  az = wave_sum(az);
  bool unconfident = false, kept = true;
  float c = 0.f;
  if (flags & 1) {
    c = sigmoid(ac + to_f(bc[0]));
    unconfident = c < lam;
  }
  if (flags & 2) {
    kept = sigmoid(az + to_f(bz[0])) > min_match;
    if (flags & 1) kept = kept || c <= lam;
  }
  if (lane == 0) keep[r] = kept ? 1 : 0;
  return make_int2(unconfident ? 1 : 0, kept ? 1 : 0);
}

// One wave per remaining point.  Each workgroup writes its counts to
// part[4 blockIdx.x + ...] = {unconfident A, kept A, unconfident B, kept B}
// with plain stores (no atomics, no fences: k_adaptive_decide reads them
// after the kernel boundary).  flags: 1 = confidence (early exit), 2 =
// pruning.  Nothing runs once *stop is set.
template <typename WT>
__global__ __launch_bounds__(256) void k_adaptive_stats(const float* __restrict__ X, SegTable seg, int D,
                                                        const WT* __restrict__ wc, const WT* __restrict__ bc,
                                                        const WT* __restrict__ wz, const WT* __restrict__ bz,
                                                        float lam, float min_match, int flags,
                                                        const int* __restrict__ stop, int* __restrict__ keep,
                                                        int* __restrict__ part) {
  if (*stop) return;  // the pass stopped at an earlier layer
  __shared__ int sm[4][4];
  const int lane = threadIdx.x & 63, wave = wave_id();
  int t = blockIdx.x * 4 + wave;
  int s = 0;
  while (s < seg.n_seg && t >= seg.n[s]) t -= seg.n[s++];
  int2 v = make_int2(0, 0);
  if (s < seg.n_seg) v = point_stats(X, seg, D, wc, bc, wz, bz, lam, min_match, flags, keep, s, t, lane);
  if (lane == 0) {
    sm[wave][0] = s == 0 ? v.x : 0;
    sm[wave][1] = s == 0 ? v.y : 0;
    sm[wave][2] = s == 1 ? v.x : 0;
    sm[wave][3] = s == 1 ? v.y : 0;
  }
  __syncthreads();
  if (threadIdx.x < 4)
    part[4 * blockIdx.x + threadIdx.x] = sm[0][threadIdx.x] + sm[1][threadIdx.x] + sm[2][threadIdx.x] + sm[3][threadIdx.x];
}

// One workgroup: sums the nb partial counts, decides the stop (flags bit 1:
// 1 - unconfident / total > alpha) into *stop, and posts {stop, unconfident
// A, kept A, unconfident B, kept B} to post[1..5], then seq to post[0]
// (host-visible memory, seq last).  Nothing runs once *stop is set.
__global__ __launch_bounds__(256) void k_adaptive_decide(const int* __restrict__ part, int nb, int flags, float alpha,
                                                         int total, int seq, int* __restrict__ stop,
                                                         int* __restrict__ post) {
  if (*stop) return;
  __shared__ int sm[4][256];
  int acc[4] = {0, 0, 0, 0};
  for (int b = threadIdx.x; b < nb; b += 256)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += part[4 * b + k];
#pragma unroll
  for (int k = 0; k < 4; ++k) sm[k][threadIdx.x] = acc[k];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w)
#pragma unroll
      for (int k = 0; k < 4; ++k) sm[k][threadIdx.x] += sm[k][threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const int uA = sm[0][0], kA = sm[1][0], uB = sm[2][0], kB = sm[3][0];
  const int st = (flags & 1) && 1.0 - (double)(uA + uB) / (double)total > (double)alpha;
  if (st) *stop = 1;
  post[1] = st; post[2] = uA; post[3] = kA; post[4] = uB; post[5] = kB;
  __threadfence_system();
  post[0] = seq;
}

// newidx[r] for the rows of image blockIdx.x: the rank of the row among the
// kept rows when the image is pruned (prune_mask bit), its own position
// otherwise; -1 for dropped rows.
__global__ __launch_bounds__(256) void k_prune_scan(SegTable seg, const int* __restrict__ keep, int prune_mask,
                                                    int* __restrict__ newidx) {
  constexpr int PER = 16;  // rows per thread: 256 * 16 = 4096, the per-image limit
  __shared__ int part[256];
  const int s = blockIdx.x;
  const int n = seg.n[s], r0 = seg.row0[s];
  const bool pruned = (prune_mask >> s) & 1;
  const int tid = threadIdx.x;
  int k[PER], local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int p = tid * PER + q;
    k[q] = p < n ? (pruned ? keep[r0 + p] : 1) : 0;
    local += k[q];
  }
  part[tid] = local;
  __syncthreads();
  // inclusive scan of the 256 partial counts (Hillis-Steele in LDS)
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int rank = part[tid] - local;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int p = tid * PER + q;
    if (p < n) newidx[r0 + p] = k[q] ? rank : -1;
    rank += k[q];
  }
}

// Job j < R_old: old row j moves to row row0_new + newidx (if kept); job
// R_old + q: row q of the new layout is zeroed if it is padding.  One
// workgroup per job.  pr (original index space, A then B) counts the
// pruning steps survived by the points of pruned images.
__global__ __launch_bounds__(256) void k_compact_rows(const float* __restrict__ Xo, const int* __restrict__ ind_o,
                                                      const int* __restrict__ newidx, SegTable so, SegTable sn,
                                                      int R_old, int R_new, int D, int prune_mask, int M,
                                                      float* __restrict__ Xn, int* __restrict__ ind_n,
                                                      int* __restrict__ pr) {
  const int j = blockIdx.x, tid = threadIdx.x;
  if (j < R_old) {
    const int s = seg_of_row(so, j);
    if (j - so.row0[s] >= so.n[s]) return;  // padding of the old layout
    const int ni = newidx[j];
    if (ni < 0) return;
    const int q = sn.row0[s] + ni;
    for (int d = 4 * tid; d < D; d += 1024)
      *reinterpret_cast<float4*>(Xn + (size_t)q * D + d) = *reinterpret_cast<const float4*>(Xo + (size_t)j * D + d);
    if (tid == 0) {
      ind_n[q] = ind_o[j];
      if ((prune_mask >> s) & 1) pr[(s ? M : 0) + ind_o[j]] += 1;
    }
  } else {
    const int q = j - R_old;
    if (q >= R_new) return;
    const int s = seg_of_row(sn, q);
    if (q - sn.row0[s] < sn.n[s]) return;  // a real row, written by its job
    for (int d = 4 * tid; d < D; d += 1024)
      *reinterpret_cast<float4*>(Xn + (size_t)q * D + d) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid == 0) ind_n[q] = -1;
  }
}

// Matches and scores of the remaining points (compact order, tm0 [nA],
// tm1 [nB] index the other image's remaining points) at the original
// indices.
__global__ void k_scatter_matches(SegTable seg, const int* __restrict__ ind, const int32_t* __restrict__ tm0,
                                  const float* __restrict__ ts0, const int32_t* __restrict__ tm1,
                                  const float* __restrict__ ts1, int32_t* __restrict__ m0, float* __restrict__ s0,
                                  int32_t* __restrict__ m1, float* __restrict__ s1) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int nA = seg.n[0], nB = seg.n[1];
  if (t < nA) {
    const int o = ind[seg.row0[0] + t], m = tm0[t];
    m0[o] = m >= 0 ? ind[seg.row0[1] + m] : -1;
    s0[o] = ts0[t];
  } else if (t < nA + nB && m1) {
    const int u = t - nA;
    const int o = ind[seg.row0[1] + u], m = tm1[u];
    m1[o] = m >= 0 ? ind[seg.row0[0] + m] : -1;
    if (s1) s1[o] = ts1[u];
  }
}

// Rows of F (the exit head's descriptors) to the caller's [M][D] / [N][D].
__global__ void k_scatter_desc(SegTable seg, const int* __restrict__ ind, const float* __restrict__ F, int D,
                               float* __restrict__ fA, float* __restrict__ fB) {
  const int r = blockIdx.x;
  const int s = seg_of_row(seg, r);
  if (r - seg.row0[s] >= seg.n[s]) return;
  float* out = s == 0 ? fA : fB;
  if (!out) return;
  const int o = ind[r];
  for (int d = threadIdx.x; d < D; d += 256) out[(size_t)o * D + d] = F[(size_t)r * D + d];
}

// The (nA+1) x (nB+1) log assignment lt (leading dimension nB+1) into the
// caller's (M+1) x (N+1) matrix: row i -> ind_A[i] (the dustbin row nA -> M),
// column j -> ind_B[j] (nB -> N).
__global__ void k_scatter_logp(SegTable seg, const int* __restrict__ ind, const float* __restrict__ lt, int M,
                               int N, float* __restrict__ logP, int64_t ld) {
  const int nA = seg.n[0], nB = seg.n[1];
  const int i = blockIdx.y;
  if (i > nA) return;
  const int oi = i < nA ? ind[seg.row0[0] + i] : M;
  for (int j = blockIdx.x * 256 + threadIdx.x; j <= nB; j += gridDim.x * 256) {
    const int oj = j < nB ? ind[seg.row0[1] + j] : N;
    logP[(int64_t)oi * ld + oj] = lt[(size_t)i * (nB + 1) + j];
  }
}

// ------------------------------------------------------------- launchers

hipError_t launch_iota_rows(const SegTable& seg, int R, int* ind, hipStream_t st) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_iota_rows, dim3((R + 255) / 256), dim3(256), 0, st, seg, R, ind);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int* p, int v, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

hipError_t launch_adaptive_stats(const float* X, const SegTable& seg, int D, int w_dtype, const void* wc,
                                 const void* bc, const void* wz, const void* bz, float lam, float min_match,
                                 int flags, float alpha, int total, int seq, int* keep, int* part, int* stop,
                                 int* post, hipStream_t st) {
  int n = 0;
  for (int s = 0; s < seg.n_seg; ++s) n += seg.n[s];
  if (D % 4 || !(flags & 3)) return hipErrorInvalidValue;
  const int nb = (n + 3) / 4;
  if (nb > 0) {
    if (w_dtype == SG_BF16)
      hipLaunchKernelGGL(k_adaptive_stats<bf16>, dim3(nb), dim3(256), 0, st, X, seg, D, static_cast<const bf16*>(wc),
                         static_cast<const bf16*>(bc), static_cast<const bf16*>(wz), static_cast<const bf16*>(bz),
                         lam, min_match, flags, stop, keep, part);
    else
      hipLaunchKernelGGL(k_adaptive_stats<float>, dim3(nb), dim3(256), 0, st, X, seg, D,
                         static_cast<const float*>(wc), static_cast<const float*>(bc), static_cast<const float*>(wz),
                         static_cast<const float*>(bz), lam, min_match, flags, stop, keep, part);
  }
  hipLaunchKernelGGL(k_adaptive_decide, dim3(1), dim3(256), 0, st, part, nb, flags, alpha, total, seq, stop, post);
  return hipGetLastError();
}

hipError_t launch_prune_scan(const SegTable& seg, const int* keep, int prune_mask, int* newidx, hipStream_t st) {
  for (int s = 0; s < seg.n_seg; ++s)
    if (seg.n[s] > 4096) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prune_scan, dim3(seg.n_seg), dim3(256), 0, st, seg, keep, prune_mask, newidx);
  return hipGetLastError();
}

hipError_t launch_compact_rows(const float* Xo, const int* ind_o, const int* newidx, const SegTable& so,
                               const SegTable& sn, int R_old, int R_new, int D, int prune_mask, int M, float* Xn,
                               int* ind_n, int* pr, hipStream_t st) {
  if (R_old + R_new <= 0) return hipSuccess;
  if (D % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_compact_rows, dim3(R_old + R_new), dim3(256), 0, st, Xo, ind_o, newidx, so, sn, R_old, R_new,
                     D, prune_mask, M, Xn, ind_n, pr);
  return hipGetLastError();
}

hipError_t launch_scatter_outputs(const SegTable& seg, const int* ind, const int32_t* tm0, const float* ts0,
                                  const int32_t* tm1, const float* ts1, int32_t* m0, float* s0, int32_t* m1,
                                  float* s1, const float* F, int D, float* fA, float* fB, const float* lt, int M,
                                  int N, float* logP, int64_t ld, int R, hipStream_t st) {
  const int nA = seg.n[0], nB = seg.n[1];
  if (nA + nB > 0)
    hipLaunchKernelGGL(k_scatter_matches, dim3((nA + nB + 255) / 256), dim3(256), 0, st, seg, ind, tm0, ts0, tm1,
                       ts1, m0, s0, m1, s1);
  if ((fA || fB) && R > 0)
    hipLaunchKernelGGL(k_scatter_desc, dim3(R), dim3(256), 0, st, seg, ind, F, D, fA, fB);
  if (logP && lt)
    hipLaunchKernelGGL(k_scatter_logp, dim3((nB + 1 + 255) / 256, nA + 1), dim3(256), 0, st, seg, ind, lt, M, N,
                       logP, ld);
  return hipGetLastError();
}

}  // namespace sg
