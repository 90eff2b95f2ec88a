// Double-softmax matching head (gfx950): the closed-form alternative to
// optimal transport described in section 2.4 of the vincentqin.tech review
// of LightGlue ("论文解读:LightGlue,让稀疏特征匹配随难度自适应地快").
//
// The log assignment of a pair is the log-softmax of S over each row plus the
// log-softmax of S over each column plus the log-sigmoid of the two points'
// matchability logits z = <w_z, x> + b_z (x: last GNN states); the dustbin
// column holds log-sigmoid(-z0_i), the dustbin row log-sigmoid(-z1_j), the
// corner 0.  With Z = S log2(e) (the score GEMM's output) and base-2 logs,
// the real block is
//     logP2_ij = 2 Z_ij + u_i + v_j,
//     u_i = ls2(z0_i) - lse2_j Z_ij,   v_j = ls2(z1_j) - lse2_i Z_ij,
// (ls2 = log2 of the sigmoid), so the mutual-argmax extraction is the
// Sinkhorn head's with Z doubled.  k_ds_stats computes u, v and the dustbin
// entries in one launch: one wave per real row of Z (side A) or of its
// transpose ZT (side B), reading the row and the point's state once.
#include <algorithm>

#include "sg_device.h"

namespace sg {

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }

template <int NV4, typename WT>
__global__ __launch_bounds__(256) void k_ds_stats(const float* __restrict__ Z,
                                                  const float* __restrict__ ZT, PairTable pt,
                                                  const float* __restrict__ X, int D,
                                                  const WT* __restrict__ wz,
                                                  const WT* __restrict__ bz_dev, float bz,
                                                  float* __restrict__ u, float* __restrict__ v,
                                                  float* __restrict__ ud, float* __restrict__ vd) {
  const int which = blockIdx.y;  // 0: rows of Z (points of A), 1: rows of ZT (points of B)
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + wave_id();
  const int* pre = which ? pt.vpre : pt.upre;
  const int b = find_pair(pre, pt.n_pairs, g);
  if (b >= pt.n_pairs) return;
  const int i = g - pre[b];
  const int M = pt.M[b], N = pt.N[b];
  const int nr = which ? N : M, nc = which ? M : N;
  if (i >= nr) return;  // the flattening's dustbin slot: no row
  const float* row = which ? ZT + pt.zt_off[b] + (size_t)i * ld4(M) : Z + pt.z_off[b] + (size_t)i * ld4(N);
  // issue the score row and the state row before reducing either
  float4 zr[NV4];
#pragma unroll
  for (int k = 0; k < NV4; ++k) {
    const int j = 4 * (lane + 64 * k);
    zr[k] = j < nc ? *reinterpret_cast<const float4*>(row + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float* xs = X + (size_t)(pt.rowA[b] + (which ? ((M + 31) & ~31) : 0) + i) * D;
  float acc = 0.f;
  for (int d = 4 * lane; d < D; d += 256) {
    const float4 xv = *reinterpret_cast<const float4*>(xs + d);
    acc = fmaf(xv.x, to_f(wz[d]), acc);
    acc = fmaf(xv.y, to_f(wz[d + 1]), acc);
    acc = fmaf(xv.z, to_f(wz[d + 2]), acc);
    acc = fmaf(xv.w, to_f(wz[d + 3]), acc);
  }
  float x[NV4][4];
#pragma unroll
  for (int k = 0; k < NV4; ++k) {
    const int j = 4 * (lane + 64 * k);
    x[k][0] = j < nc ? zr[k].x : -INFINITY;
    x[k][1] = j + 1 < nc ? zr[k].y : -INFINITY;
    x[k][2] = j + 2 < nc ? zr[k].z : -INFINITY;
    x[k][3] = j + 3 < nc ? zr[k].w : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < NV4; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) mx = fmaxf(mx, x[k][c]);
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NV4; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) sum += exp2_fast(x[k][c] - mx);
  sum = wave_sum(sum);
  acc = wave_sum(acc);
  if (lane == 0) {
    const float z = acc + (bz_dev ? to_f(bz_dev[0]) : bz);
    // log sigmoid(+-z) = min(+-z, 0) - log(1 + e^-|z|), finite for every finite z
    const float t = log1pf(expf(-fabsf(z)));
    const float ls = fminf(z, 0.f) - t, lsn = fminf(-z, 0.f) - t;
    const int o = (which ? pt.voff[b] : pt.uoff[b]) + i;
    // (an empty other side leaves no real block; its u / v are never read)
    (which ? v : u)[o] = nc > 0 ? ls * kLog2e - (mx + log2_fast(sum)) : 0.f;
    (which ? vd : ud)[o] = lsn * kLog2e;
  }
}

// Optional output: the (M+1) x (N+1) log assignment of every pair (natural
// log): ln2 (2 Z + u_i + v_j) on the real block, the dustbin entries, 0 in
// the corner.
__global__ __launch_bounds__(256) void k_ds_write_logp(const float* __restrict__ Zbase, PairTable pt,
                                                       const float* __restrict__ u,
                                                       const float* __restrict__ v,
                                                       const float* __restrict__ ud,
                                                       const float* __restrict__ vd,
                                                       float* __restrict__ logP, int64_t ld,
                                                       int64_t pair_stride) {
  const int g = blockIdx.y;
  const int b = find_pair(pt.upre, pt.n_pairs, g);
  if (b >= pt.n_pairs) return;
  const int i = g - pt.upre[b];
  const int M = pt.M[b], N = pt.N[b];
  const float* row = Zbase + pt.z_off[b] + (size_t)i * ld4(N);
  float* out = logP + b * pair_stride + (int64_t)i * ld;
  for (int j = blockIdx.x * 256 + threadIdx.x; j <= N; j += gridDim.x * 256) {
    float r;
    if (i < M && j < N) r = kLn2 * (2.f * row[j] + u[pt.uoff[b] + i] + v[pt.voff[b] + j]);
    else if (i < M) r = kLn2 * ud[pt.uoff[b] + i];
    else if (j < N) r = kLn2 * vd[pt.voff[b] + j];
    else r = 0.f;
    out[j] = r;
  }
}

// ------------------------------------------------------------- launchers

hipError_t launch_ds_stats(const float* Z, const float* ZT, const PairTable& pt, const float* X, int D,
                           int w_dtype, const void* wz, const void* bz_dev, float bz, float* u, float* v,
                           float* ud, float* vd, hipStream_t st) {
  int nc = 0;
  for (int b = 0; b < pt.n_pairs; ++b) nc = std::max(nc, std::max(pt.M[b], pt.N[b]));
  const int rows = std::max(pt.upre[pt.n_pairs], pt.vpre[pt.n_pairs]);
  if (rows <= 0 || nc <= 0) return hipSuccess;
  if (D <= 0 || D % 4) return hipErrorInvalidValue;
  int nv4 = 1;
  while (256 * nv4 < nc) nv4 *= 2;
  dim3 grid((rows + 3) / 4, 2);
#define SG_DS(NV)                                                                                           \
  if (nv4 == NV) {                                                                                          \
    if (w_dtype == SG_BF16)                                                                                 \
      hipLaunchKernelGGL((k_ds_stats<NV, bf16>), grid, dim3(256), 0, st, Z, ZT, pt, X, D,                   \
                         static_cast<const bf16*>(wz), static_cast<const bf16*>(bz_dev), bz, u, v, ud, vd); \
    else                                                                                                    \
      hipLaunchKernelGGL((k_ds_stats<NV, float>), grid, dim3(256), 0, st, Z, ZT, pt, X, D,                  \
                         static_cast<const float*>(wz), static_cast<const float*>(bz_dev), bz, u, v, ud,    \
                         vd);                                                                               \
    return hipGetLastError();                                                                               \
  }
  SG_DS(1) SG_DS(2) SG_DS(4) SG_DS(8) SG_DS(16)
#undef SG_DS
  return hipErrorInvalidValue;
}

hipError_t launch_ds_write_logp(const float* Z, const PairTable& pt, const float* u, const float* v,
                                const float* ud, const float* vd, float* logP, int64_t ld, int64_t pair_stride,
                                int total_rows, hipStream_t st) {
  if (total_rows <= 0) return hipSuccess;
  int nc = 0;
  for (int b = 0; b < pt.n_pairs; ++b) nc = std::max(nc, pt.N[b] + 1);
  hipLaunchKernelGGL(k_ds_write_logp, dim3((nc + 255) / 256, total_rows), dim3(256), 0, st, Z, pt, u, v, ud,
                     vd, logP, ld, pair_stride);
  return hipGetLastError();
}

}  // namespace sg
