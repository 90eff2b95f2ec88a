// Log-domain Sinkhorn normalisation and mutual-argmax extraction (gfx950).
//
// The couplings are never materialised with their dustbins: Z holds
// S*log2(e) for the real block and ZT its transpose; the dustbin row, column
// and corner are the constant alpha*log2(e).  All exponentials and logarithms
// are base 2.
#include <algorithm>

#include "sg_device.h"

namespace sg {

// --------------------------------------------------------------- Sinkhorn
//
// One wave per row of Z (which = 0: rows i of the (M+1)x(N+1) couplings,
// producing u) or of ZT (which = 1: columns j, producing v):
//   out_i = log2 marginal_i - log2 sum_j 2^(Z2_ij + w_j),
// with the dustbin row/column equal to alpha2 and the base-2 marginals
// -log2(M+N) (real rows) and log2(count of the other side) - log2(M+N)
// (dustbin).  w_in == nullptr stands for w = 0 (the first iteration).

template <int NV4>
__global__ __launch_bounds__(256) void k_lse(const float* __restrict__ Zbase, PairTable pt,
                                             int which, const float* __restrict__ w_in,
                                             float* __restrict__ w_out, float alpha2,
                                             const float* __restrict__ alpha_dev) {
  if (alpha_dev) alpha2 = alpha_dev[0] * kLog2e;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int* pre = which ? pt.vpre : pt.upre;
  const int b = find_pair(pre, pt.n_pairs, g);
  if (b >= pt.n_pairs) return;
  const int i = g - pre[b];
  const int M = pt.M[b], N = pt.N[b];
  const int nr = which ? N : M, nc = which ? M : N;
  const float* wv = w_in ? w_in + (which ? pt.uoff[b] : pt.voff[b]) : nullptr;
  const int last4 = ld4(nc) - 4;  // last float4 of a row (rows are padded to ld4(nc))
  // every lane owns NV4 float4 groups of the row: columns 4*(lane + 64 t) .. +3
  float x[4 * NV4];
  if (nc == 0) {  // an empty other side: only the dustbin column remains
#pragma unroll
    for (int k = 0; k < 4 * NV4; ++k) x[k] = -INFINITY;
  } else if (i < nr) {
    const float* row = Zbase + (which ? pt.zt_off[b] + (size_t)i * ld4(M) : pt.z_off[b] + (size_t)i * ld4(N));
#pragma unroll
    for (int t = 0; t < NV4; ++t) {
      const int j = 4 * (lane + 64 * t);
      const int jc = min(j, last4);  // clamped: loads are unconditional and in bounds
      float4 z = *reinterpret_cast<const float4*>(row + jc);
      float4 w = wv ? *reinterpret_cast<const float4*>(wv + jc) : make_float4(0.f, 0.f, 0.f, 0.f);
      x[4 * t + 0] = j + 0 < nc ? z.x + w.x : -INFINITY;
      x[4 * t + 1] = j + 1 < nc ? z.y + w.y : -INFINITY;
      x[4 * t + 2] = j + 2 < nc ? z.z + w.z : -INFINITY;
      x[4 * t + 3] = j + 3 < nc ? z.w + w.w : -INFINITY;
    }
  } else {  // the dustbin row: alpha everywhere
#pragma unroll
    for (int t = 0; t < NV4; ++t) {
      const int j = 4 * (lane + 64 * t);
      const int jc = min(j, last4);
      float4 w = wv ? *reinterpret_cast<const float4*>(wv + jc) : make_float4(0.f, 0.f, 0.f, 0.f);
      x[4 * t + 0] = j + 0 < nc ? alpha2 + w.x : -INFINITY;
      x[4 * t + 1] = j + 1 < nc ? alpha2 + w.y : -INFINITY;
      x[4 * t + 2] = j + 2 < nc ? alpha2 + w.z : -INFINITY;
      x[4 * t + 3] = j + 3 < nc ? alpha2 + w.w : -INFINITY;
    }
  }
  // the dustbin column (j = nc) is alpha for every row
  const float xd = alpha2 + (wv ? wv[nc] : 0.f);
  float mx = xd;
#pragma unroll
  for (int k = 0; k < 4 * NV4; ++k) mx = fmaxf(mx, x[k]);
  mx = wave_max(mx);
  float sum = lane == 0 ? exp2_fast(xd - mx) : 0.f;
#pragma unroll
  for (int k = 0; k < 4 * NV4; ++k) sum += exp2_fast(x[k] - mx);
  sum = wave_sum(sum);
  if (lane == 0) {
    const float lm = (i < nr ? 0.f : log2f((float)nc)) - log2f((float)(M + N));
    w_out[(which ? pt.voff[b] : pt.uoff[b]) + i] = lm - (mx + log2_fast(sum));
  }
}

// ------------------------------------------------------------- extraction
//
// Row argmax over the real block of the final log assignment (row i:
// argmax_j Z2_ij + v_j, since u_i is constant along the row) and column
// argmax (column j: argmax_i Z2_ij + u_i, read from ZT).  Lowest index wins
// ties.  Waves [0, rowsA) take rows of A, the rest columns.

template <int MAXV>
__global__ __launch_bounds__(256) void k_argmax(const float* __restrict__ Zb,
                                                const float* __restrict__ ZTb, PairTable pt,
                                                const float* __restrict__ u,
                                                const float* __restrict__ v, int* __restrict__ idx0,
                                                float* __restrict__ val0, int* __restrict__ idx1,
                                                int rowsA, int rowsB) {
  const int lane = threadIdx.x & 63;
  int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= rowsA + rowsB) return;
  const int which = g >= rowsA ? 1 : 0;
  if (which) g -= rowsA;
  // flattened real rows: prefix of M is upre[b] - b, prefix of N is vpre[b] - b
  int b = 0;
  const int* pre = which ? pt.vpre : pt.upre;
  while (b < pt.n_pairs && g >= pre[b + 1] - (b + 1)) ++b;
  if (b >= pt.n_pairs) return;
  const int i = g - (pre[b] - b);
  const int M = pt.M[b], N = pt.N[b];
  const int nc = which ? M : N;
  const float* row = which ? ZTb + pt.zt_off[b] + (size_t)i * ld4(M) : Zb + pt.z_off[b] + (size_t)i * ld4(N);
  const float* wv = which ? u + pt.uoff[b] : v + pt.voff[b];
  float best = -INFINITY;
  int bj = 0x7fffffff;
#pragma unroll
  for (int t = 0; t < MAXV; ++t) {
    const int j = lane + 64 * t;
    if (j < nc) {
      const float x = row[j] + wv[j];
      if (x > best) { best = x; bj = j; }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ob = __shfl_xor(best, o);
    const int oj = __shfl_xor(bj, o);
    if (ob > best || (ob == best && oj < bj)) { best = ob; bj = oj; }
  }
  if (lane == 0) {
    if (which) {
      idx1[g] = bj;
    } else {
      idx0[g] = bj;
      val0[g] = best;
    }
  }
}

// Mutual check, score and threshold for both sides of every pair; padded
// entries (and pairs with an empty image) get -1 / 0.
__global__ __launch_bounds__(256) void k_finalize(PairTable pt, const int* __restrict__ idx0,
                                                  const float* __restrict__ val0,
                                                  const int* __restrict__ idx1,
                                                  const float* __restrict__ u, int Mpad, int Npad,
                                                  float thr, int32_t* __restrict__ m0,
                                                  float* __restrict__ s0, int32_t* __restrict__ m1,
                                                  float* __restrict__ s1) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int M = pt.M[b], N = pt.N[b];
  const bool empty = M == 0 || N == 0;
  const int mpre = pt.upre[b] - b, npre = pt.vpre[b] - b;
  const float lmn = empty ? 0.f : log2f((float)(M + N));
  // exp(logP) > thr decided in the log domain (exact for any finite logP:
  // exp never reaches 0, so a non-positive threshold accepts every mutual match)
  const float lthr = thr > 0.f ? log2f(thr) : -INFINITY;
  if (t < Mpad) {
    const size_t o = (size_t)b * Mpad + t;
    int mo = -1;
    float so = 0.f;
    if (t < M && !empty) {
      const int j = idx0[mpre + t];
      if (idx1[npre + j] == t) {
        const float lp2 = val0[mpre + t] + u[pt.uoff[b] + t] + lmn;
        so = exp2f(lp2);
        if (lp2 > lthr) mo = j;
      }
    }
    m0[o] = mo;
    s0[o] = so;
  }
  if (m1 && t < Npad) {
    const size_t o = (size_t)b * Npad + t;
    int mo = -1;
    float so = 0.f;
    if (t < N && !empty) {
      const int i = idx1[npre + t];
      if (idx0[mpre + i] == t) {
        const float lp2 = val0[mpre + i] + u[pt.uoff[b] + i] + lmn;
        so = exp2f(lp2);
        if (lp2 > lthr) mo = i;
      }
    }
    m1[o] = mo;
    if (s1) s1[o] = so;
  }
}

// Optional output: the (M+1) x (N+1) log assignment of every pair,
// logP = ln2 * (Z2 + u + v + log2(M+N)).
__global__ __launch_bounds__(256) void k_write_logp(const float* __restrict__ Zbase, PairTable pt,
                                                    const float* __restrict__ u,
                                                    const float* __restrict__ v, float alpha2,
                                                    const float* __restrict__ alpha_dev,
                                                    float* __restrict__ logP, int64_t ld,
                                                    int64_t pair_stride) {
  if (alpha_dev) alpha2 = alpha_dev[0] * kLog2e;
  const int g = blockIdx.y;
  const int b = find_pair(pt.upre, pt.n_pairs, g);
  if (b >= pt.n_pairs) return;
  const int i = g - pt.upre[b];
  const int M = pt.M[b], N = pt.N[b];
  const float lmn = log2f((float)(M + N));
  const float ui = u[pt.uoff[b] + i];
  const float* row = Zbase + pt.z_off[b] + (size_t)i * ld4(N);
  for (int j = blockIdx.x * 256 + threadIdx.x; j <= N; j += gridDim.x * 256) {
    const float z = (i < M && j < N) ? row[j] : alpha2;
    logP[b * pair_stride + (int64_t)i * ld + j] = kLn2 * (z + ui + v[pt.voff[b] + j] + lmn);
  }
}

__global__ void k_fill_f32(float* p, float v, int n) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < n) p[t] = v;
}

__global__ void k_fill_empty(int32_t* m, float* s, int n) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < n) {
    m[t] = -1;
    if (s) s[t] = 0.f;
  }
}

static int max_cols(const PairTable& pt, int which) {
  int m = 0;
  for (int b = 0; b < pt.n_pairs; ++b) m = std::max(m, (which ? pt.M[b] : pt.N[b]) + 1);
  return m;
}

hipError_t launch_lse(const float* Z, const PairTable& pt, int which, const float* w_in,
                      float* w_out, float alpha2, const float* alpha_dev, int total_rows,
                      hipStream_t st) {
  if (total_rows <= 0) return hipSuccess;
  const int nc = max_cols(pt, which) - 1;  // real columns of the longest row
  dim3 grid((total_rows + 3) / 4);
#define SG_LSE(NV) hipLaunchKernelGGL(k_lse<NV>, grid, dim3(256), 0, st, Z, pt, which, w_in, w_out, alpha2, alpha_dev)
  if (nc <= 256) SG_LSE(1);
  else if (nc <= 512) SG_LSE(2);
  else if (nc <= 1024) SG_LSE(4);
  else if (nc <= 2048) SG_LSE(8);
  else if (nc <= 4096) SG_LSE(16);
  else return hipErrorInvalidValue;
#undef SG_LSE
  return hipGetLastError();
}

hipError_t launch_argmax(const float* Z, const float* ZT, const PairTable& pt, const float* u,
                         const float* v, int* idx0, float* val0, int* idx1, int rowsA, int rowsB,
                         hipStream_t st) {
  if (rowsA + rowsB <= 0) return hipSuccess;
  const int nc = std::max(max_cols(pt, 0), max_cols(pt, 1));
  dim3 grid((rowsA + rowsB + 3) / 4);
  if (nc <= 256) hipLaunchKernelGGL(k_argmax<4>, grid, dim3(256), 0, st, Z, ZT, pt, u, v, idx0, val0, idx1, rowsA, rowsB);
  else if (nc <= 576) hipLaunchKernelGGL(k_argmax<9>, grid, dim3(256), 0, st, Z, ZT, pt, u, v, idx0, val0, idx1, rowsA, rowsB);
  else if (nc <= 1088) hipLaunchKernelGGL(k_argmax<17>, grid, dim3(256), 0, st, Z, ZT, pt, u, v, idx0, val0, idx1, rowsA, rowsB);
  else if (nc <= 2112) hipLaunchKernelGGL(k_argmax<33>, grid, dim3(256), 0, st, Z, ZT, pt, u, v, idx0, val0, idx1, rowsA, rowsB);
  else if (nc <= 4160) hipLaunchKernelGGL(k_argmax<65>, grid, dim3(256), 0, st, Z, ZT, pt, u, v, idx0, val0, idx1, rowsA, rowsB);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_finalize(const PairTable& pt, const int* idx0, const float* val0, const int* idx1,
                           const float* u, int Mpad, int Npad, float thr, int32_t* m0, float* s0,
                           int32_t* m1, float* s1, hipStream_t st) {
  const int n = std::max(Mpad, m1 ? Npad : 0);
  if (n <= 0 || pt.n_pairs <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_finalize, dim3((n + 255) / 256, pt.n_pairs), dim3(256), 0, st, pt, idx0,
                     val0, idx1, u, Mpad, Npad, thr, m0, s0, m1, s1);
  return hipGetLastError();
}

hipError_t launch_write_logp(const float* Z, const PairTable& pt, const float* u, const float* v,
                             float alpha2, const float* alpha_dev, float* logP, int64_t ld,
                             int64_t pair_stride, int total_rows, hipStream_t st) {
  if (total_rows <= 0) return hipSuccess;
  const int nc = max_cols(pt, 0);
  hipLaunchKernelGGL(k_write_logp, dim3((nc + 255) / 256, total_rows), dim3(256), 0, st, Z, pt, u,
                     v, alpha2, alpha_dev, logP, ld, pair_stride);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float v, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3((n + 255) / 256), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

hipError_t launch_fill_empty(int32_t* m, float* s, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_empty, dim3((n + 255) / 256), dim3(256), 0, st, m, s, n);
  return hipGetLastError();
}

}  // namespace sg
