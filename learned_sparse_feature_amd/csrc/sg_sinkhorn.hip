// Log-domain Sinkhorn normalisation and mutual-argmax extraction (gfx950).
//
// The couplings are never materialised with their dustbins: Z holds
// S*log2(e) for the real block of every pair ([M][ld4(N)]); the dustbin row,
// column and corner are the constant alpha*log2(e).  All exponentials and
// logarithms are base 2, so u and v below are the dual variables times
// log2(e).
//
// One iteration reads Z once (the two updates of the page's loop are split
// so that no transposed copy is needed):
//  * k_sink_rows: a workgroup takes RB = 4*RPW consecutive rows of one pair
//    (the dustbin row included), each of its four waves RPW whole rows.
//    Per row, with t = Z + v: m_i = max_j t_ij, e_ij = 2^(t_ij - m_i),
//    s_i = sum_j e_ij and the row update u_i = log2 mu_i - m_i - log2 s_i.
//    The block's column partial lse2_{i in block}(Z_ij + u_i) reuses e:
//    2^(Z_ij + u_i) = e_ij 2^(m_i + u_i) 2^(-v_j) and m_i + u_i =
//    log2(mu_i / s_i), so relative to W = -log2(M+N) the row weights are
//    c_i / s_i (c_i = 1, N on the dustbin row) and the partial is
//    log2(sum_i e_ij c_i / s_i) + W - v_j: one FMA per entry.  A term lost
//    to underflow of e is below 2^-126, so a sum of at least 2^-100 is exact
//    to fp32 rounding; a smaller one is recomputed as the plain log-sum-exp
//    over the block's rows.
//  * k_sink_cols: v_j = log2 nu_j - lse2_g P[g][j].
// After the last iteration the per-block column maxima of Z + u (argmax
// over the real rows) are reduced the same way, and k_sink_extract takes the
// row argmax, the mutual check, the scores and the threshold.
#include <algorithm>
#include <cmath>

#include "sg_device.h"

namespace sg {

constexpr float kSumFloor = 0x1p-100f;

__device__ __forceinline__ float f4c(const float4& q, int c) {
  return c == 0 ? q.x : c == 1 ? q.y : c == 2 ? q.z : q.w;
}

// P: [G][ld4(N)] partials of the real columns, Pd: [G] partials of the
// dustbin column (flattened over pairs by gpre).  ARG: also the per-block
// column argmax of Z + u over the real rows into PV / PI.  update_u = 0
// (no Sinkhorn iteration) takes u = 0 and writes only PV / PI.

template <int RPW, int NV4, bool ARG>
__global__ __launch_bounds__(256) void k_sink_rows(const float* __restrict__ Zb, PairTable pt,
                                                   const float* __restrict__ v_in,
                                                   float* __restrict__ u_out, float* __restrict__ P,
                                                   float* __restrict__ Pd, float* __restrict__ PV,
                                                   int* __restrict__ PI, float alpha2,
                                                   const float* __restrict__ alpha_dev, int update_u) {
  constexpr int RB = 4 * RPW;
  constexpr int NG = 64 * NV4;  // float4 column groups of a row held by one wave
  __shared__ float4 sm[4][NG];
  __shared__ float sm_u[RB], sm_d[4];
  if (alpha_dev) alpha2 = alpha_dev[0] * kLog2e;
  const int b = find_pair(pt.gpre, pt.n_pairs, blockIdx.x);
  if (b >= pt.n_pairs) return;
  const int gb = blockIdx.x - pt.gpre[b];
  const int M = pt.M[b], N = pt.N[b];
  const int i0 = gb * RB;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int ldz = ld4(N);
  const float* zp = Zb + pt.z_off[b];
  const float lmn = log2f((float)(M + N));
  const float* vv = v_in ? v_in + pt.voff[b] : nullptr;

  float vc[NV4][4];
#pragma unroll
  for (int k = 0; k < NV4; ++k) {
    const int j = 4 * (lane + 64 * k);
    const float4 q = (vv && j < N) ? *reinterpret_cast<const float4*>(vv + j) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int c = 0; c < 4; ++c) vc[k][c] = f4c(q, c);
  }
  const float vN = vv ? vv[N] : 0.f;

  // ---- row update of the wave's rows; e keeps 2^(t - m)
  float e[RPW][NV4][4], wgt[RPW];
  float dT = 0.f;  // lane 0: this wave's dustbin-column partial
  // all of the wave's row loads are issued before any row is reduced (at a
  // real row and column, clamped in bounds; replaced below where the entry
  // is the dustbin row, a masked column or a row past it)
  if (M > 0 && N > 0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int ic = min(i0 + w * RPW + r, M - 1);
#pragma unroll
      for (int k = 0; k < NV4; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(zp + (size_t)ic * ldz + min(4 * (lane + 64 * k), ldz - 4));
#pragma unroll
        for (int c = 0; c < 4; ++c) e[r][k][c] = f4c(q, c);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int i = i0 + w * RPW + r;
    if (i > M) {  // past the dustbin row: no contribution
      wgt[r] = 0.f;
#pragma unroll
      for (int k = 0; k < NV4; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c) e[r][k][c] = 0.f;
      if (lane == 0) sm_u[w * RPW + r] = -INFINITY;
      continue;
    }
#pragma unroll
    for (int k = 0; k < NV4; ++k) {
      const int j = 4 * (lane + 64 * k);
#pragma unroll
      for (int c = 0; c < 4; ++c) e[r][k][c] = j + c < N ? (i < M ? e[r][k][c] : alpha2) + vc[k][c] : -INFINITY;
    }
    float mx = lane == 0 ? alpha2 + vN : -INFINITY;
#pragma unroll
    for (int k = 0; k < NV4; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, e[r][k][c]);
    mx = wave_max(mx);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NV4; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        e[r][k][c] = exp2_fast(e[r][k][c] - mx);
        s += e[r][k][c];
      }
    const float ed = lane == 0 ? exp2_fast(alpha2 + vN - mx) : 0.f;
    s = wave_sum(s + ed);
    const float cr = i < M ? 1.f : (float)N;
    const float ur = log2f(cr) - lmn - mx - log2_fast(s);
    wgt[r] = cr / s;
    dT += ed * wgt[r];
    if (lane == 0) {
      sm_u[w * RPW + r] = update_u ? ur : 0.f;
      if (update_u) u_out[pt.uoff[b] + i] = ur;
    }
  }

  const size_t pbase = (size_t)pt.p_off[b] + (size_t)gb * ldz;
  if (update_u) {
#pragma unroll
    for (int k = 0; k < NV4; ++k) {
      float t[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t[c] = e[0][k][c] * wgt[0];
#pragma unroll
        for (int r = 1; r < RPW; ++r) t[c] = fmaf(e[r][k][c], wgt[r], t[c]);
      }
      sm[w][lane + 64 * k] = make_float4(t[0], t[1], t[2], t[3]);
    }
    if (lane == 0) sm_d[w] = dT;
  }
  __syncthreads();

  // exact partial of column jj over the block's rows (jj == N: the dustbin)
  auto exact = [&](int jj) -> float {
    float y[RB];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int i = i0 + r;
      const float z = (i < M && jj < N) ? zp[(size_t)i * ldz + jj] : alpha2;
      y[r] = i <= M ? z + sm_u[r] : -INFINITY;
      mx = fmaxf(mx, y[r]);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RB; ++r) s += exp2_fast(y[r] - mx);
    return mx + log2_fast(s);
  };

  if (update_u) {
    for (int q = threadIdx.x; q < NG; q += 256) {
      const int j = 4 * q;
      if (j >= N) break;
      const float4 a0 = sm[0][q], a1 = sm[1][q], a2 = sm[2][q], a3 = sm[3][q];
      const float4 vq = vv ? *reinterpret_cast<const float4*>(vv + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float T = (f4c(a0, c) + f4c(a1, c)) + (f4c(a2, c) + f4c(a3, c));
        if (j + c >= N) o[c] = -INFINITY;
        else if (T >= kSumFloor) o[c] = log2_fast(T) - lmn - f4c(vq, c);
        else o[c] = exact(j + c);
      }
      *reinterpret_cast<float4*>(P + pbase + j) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (threadIdx.x == 0) {
      const float T = (sm_d[0] + sm_d[1]) + (sm_d[2] + sm_d[3]);
      Pd[pt.gpre[b] + gb] = T >= kSumFloor ? log2_fast(T) - lmn - vN : exact(N);
    }
  }

  if constexpr (ARG) {
    // column argmax of Z + u over the wave's real rows (lowest row on ties),
    // then over the four waves (rows ascending with the wave index)
    __shared__ int4 smi[4][NG];
    __syncthreads();  // the partial sums in sm have been read
#pragma unroll
    for (int k = 0; k < NV4; ++k) {
      const int j = 4 * (lane + 64 * k);
      float bv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      int bi[4] = {-1, -1, -1, -1};
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int i = i0 + w * RPW + r;
        if (i < M && j < N) {
          const float4 q = *reinterpret_cast<const float4*>(zp + (size_t)i * ldz + j);
          const float ua = sm_u[w * RPW + r];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float y = f4c(q, c) + ua;
            if (y > bv[c]) {
              bv[c] = y;
              bi[c] = i;
            }
          }
        }
      }
      sm[w][lane + 64 * k] = make_float4(bv[0], bv[1], bv[2], bv[3]);
      smi[w][lane + 64 * k] = make_int4(bi[0], bi[1], bi[2], bi[3]);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < NG; q += 256) {
      const int j = 4 * q;
      if (j >= N) break;
      float bv[4];
      int bi[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bv[c] = f4c(sm[0][q], c);
        bi[c] = c == 0 ? smi[0][q].x : c == 1 ? smi[0][q].y : c == 2 ? smi[0][q].z : smi[0][q].w;
      }
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        const float4 a = sm[ww][q];
        const int4 ai = smi[ww][q];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float y = f4c(a, c);
          if (y > bv[c]) {
            bv[c] = y;
            bi[c] = c == 0 ? ai.x : c == 1 ? ai.y : c == 2 ? ai.z : ai.w;
          }
        }
      }
      *reinterpret_cast<float4*>(PV + pbase + j) = make_float4(bv[0], bv[1], bv[2], bv[3]);
      *reinterpret_cast<int4*>(PI + pbase + j) = make_int4(bi[0], bi[1], bi[2], bi[3]);
    }
  }
}

// One fused iteration of the one-pass schedule (batches of pairs).  A
// workgroup of W waves takes RB = W RPW consecutive rows of one pair, each
// wave RPW of them, RS rows at a time with the next RS rows' loads in
// flight; a pair has G = max(1, ceil(M / RB)) blocks, the last one holding
// the dustbin row (as an extra row when M is a multiple of RB).
//  * Phase 1: the column duals of the previous iteration, v_j = log2 nu_j -
//    lse2_g Pin[g][j] over the pair's G block partials (Pdin: the dustbin
//    column), into LDS.  Every workgroup of the pair repeats this small
//    reduction (G (N+1) partials against its RB (N+1) couplings), so that no
//    separate column launch sits between two iterations.  Pin == nullptr: v = 0
//    (the first iteration, or no iteration at all).
//  * Phase 2: the row update u_i and the block's column partials into Pout /
//    Pdout, as k_sink_rows (one FMA per entry on the row exponentials, the
//    exact per-block log-sum-exp where the sum falls below 2^-100; the
//    dustbin column's partial always in closed form), and with ARG the
//    per-block column argmax of Z + u into PV / PI.
// The partials are double-buffered by the caller: iteration t reads the
// buffer iteration t - 1 wrote and writes the other one.
// One workgroup's share of the iteration for pair b, with rows of up to
// 256 NV4 columns held in registers (NV4 float4 per lane).  The LDS arrays
// come from the kernel, sized for its widest rows (NGS float4 column groups):
// sm [W][NGS], vl [NGS + 1] (vl[NGS].x: the dustbin column's dual), sm_u
// [RB + 1] (+1: the dustbin row may follow the block's last row), smi
// [W][NGS] (ARG only).
// The fields of the pair that a workgroup of the fused iteration works on.
struct IterPair {
  int gb;     // the workgroup's row block within the pair
  int M, N;   // the pair's point counts
  int G;      // its row blocks
  int gpre;   // its first row block over the batch (dustbin-column partials)
  int z_off;  // float offsets of its couplings, its column partials and its u
  int p_off;
  int uoff;
};

template <int W, int RPW, int NV4, int RS, bool ARG, int NGS>
__device__ __forceinline__ void sink_iter_block(const float* __restrict__ Zb, const IterPair& ip,
                                                const float* __restrict__ Pin, const float* __restrict__ Pdin,
                                                float* __restrict__ u_out, float* __restrict__ Pout,
                                                float* __restrict__ Pdout, float* __restrict__ PV,
                                                int* __restrict__ PI, float alpha2, int update_u,
                                                float4 (*sm)[NGS], float4* vl, float* sm_u, int4 (*smi)[NGS]) {
  static_assert(RPW % RS == 0, "rows per wave must be a multiple of the rows per step");
  static_assert(64 * NV4 <= NGS, "the LDS arrays hold the widest rows");
  constexpr int NT = 64 * W;    // threads
  constexpr int RB = W * RPW;
  constexpr int NG = 64 * NV4;  // float4 column groups of a row held by one wave
  constexpr int NSTEP = RPW / RS;
  const int G = ip.G, gb = ip.gb;
  const int M = ip.M, N = ip.N;
  const int i0 = gb * RB;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int ldz = ld4(N);
  const float* zp = Zb + ip.z_off;
  const float lmn = log2f((float)(M + N));

  // loads of step p of the wave's rows (at a real row and column, clamped in
  // bounds; rows at or past the dustbin row do not use them)
  auto load_step = [&](int p, float4 (&dst)[RS][NV4]) {
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const int ic = max(min(i0 + w * RPW + p * RS + r, M - 1), 0);
#pragma unroll
      for (int k = 0; k < NV4; ++k)
        dst[r][k] = (M > 0 && N > 0)
                        ? *reinterpret_cast<const float4*>(zp + (size_t)ic * ldz + min(4 * (lane + 64 * k), ldz - 4))
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  // the first rows' loads go out before phase 1, which does not need them
  float4 zbuf[2][RS][NV4];
  load_step(0, zbuf[0]);

  // ---- phase 1: the column duals of the previous iteration
  if (Pin) {
    const float* pp = Pin + ip.p_off;
    constexpr int U = 8;
    for (int q = threadIdx.x; 4 * q < N; q += NT) {
      const int j = 4 * q;
      float mx[4], sum[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        mx[c] = -INFINITY;
        sum[c] = 0.f;
      }
      for (int g0 = 0; g0 < G; g0 += U) {
        float4 x[U];
#pragma unroll
        for (int r = 0; r < U; ++r) x[r] = *reinterpret_cast<const float4*>(pp + (size_t)min(g0 + r, G - 1) * ldz + j);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float m2 = mx[c];
#pragma unroll
          for (int r = 0; r < U; ++r)
            if (g0 + r < G) m2 = fmaxf(m2, f4c(x[r], c));
          float t = mx[c] == -INFINITY ? 0.f : sum[c] * exp2_fast(mx[c] - m2);
#pragma unroll
          for (int r = 0; r < U; ++r)
            if (g0 + r < G) t += exp2_fast(f4c(x[r], c) - m2);
          sum[c] = t;
          mx[c] = m2;
        }
      }
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = j + c < N ? -lmn - (mx[c] + log2_fast(sum[c])) : -INFINITY;
      vl[q] = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (w == 0) {  // the dustbin column: v_N = log2 M - log2(M+N) - lse2_g Pdin[g]
      const float* pd = Pdin + ip.gpre;
      float m = -INFINITY, sum = 0.f;
      for (int g = lane; g < G; g += 64) {
        const float x = pd[g];
        const float m2 = fmaxf(m, x);
        sum = (m == -INFINITY ? 0.f : sum * exp2_fast(m - m2)) + exp2_fast(x - m2);
        m = m2;
      }
      const float wm = wave_max(m);
      sum = wave_sum(m == -INFINITY ? 0.f : sum * exp2_fast(m - wm));
      if (lane == 0) vl[NGS].x = log2f((float)M) - lmn - (wm + log2_fast(sum));
    }
    for (int q = (N + 3) / 4 + threadIdx.x; q < NG; q += NT) vl[q] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  } else {
    for (int q = threadIdx.x; q < NG; q += NT) {
      const int j = 4 * q;
      vl[q] = make_float4(j < N ? 0.f : -INFINITY, j + 1 < N ? 0.f : -INFINITY, j + 2 < N ? 0.f : -INFINITY,
                          j + 3 < N ? 0.f : -INFINITY);
    }
    if (threadIdx.x == 0) vl[NGS] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();

  // ---- phase 2: row update of the wave's rows and the block's column partials
  // The duals of masked columns are -inf in vl, so that t = Z + v needs no
  // select (the loads are clamped in bounds and finite); the dustbin column
  // (the same entry alpha + v_N for every lane) joins each row's sum once,
  // after the wave reduction; the dustbin row is done after the real rows.
  // The duals stay in registers, except for the widest rows (VCL), which
  // read them from LDS for every row: their 32 registers buy a wave per SIMD.
  constexpr bool VCL = NV4 >= 8;
  float vc[VCL ? 1 : NV4][4];
  if constexpr (!VCL) {
#pragma unroll
    for (int k = 0; k < NV4; ++k) {
      const float4 q = vl[lane + 64 * k];
#pragma unroll
      for (int c = 0; c < 4; ++c) vc[k][c] = f4c(q, c);
    }
  }
  const float vN = vl[NGS].x;
  const float xd = alpha2 + vN;  // the dustbin-column entry of every row
  float acc[NV4][4];
#pragma unroll
  for (int k = 0; k < NV4; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[k][c] = 0.f;
  // one row: t = x + v (x the row's entries, or alpha for the dustbin row),
  // its update u, and its weighted exponentials into acc
  auto row = [&](const float4 (&zq)[NV4], bool dust, int ri) {
    float t[NV4][4];
    float mx = xd;
#pragma unroll
    for (int k = 0; k < NV4; ++k) {
      float4 vq;
      if constexpr (VCL) vq = vl[lane + 64 * k];
      else vq = make_float4(vc[k][0], vc[k][1], vc[k][2], vc[k][3]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t[k][c] = (dust ? alpha2 : f4c(zq[k], c)) + f4c(vq, c);
        mx = fmaxf(mx, t[k][c]);
      }
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < NV4; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        t[k][c] = exp2_fast(t[k][c] - mx);
        sum += t[k][c];
      }
    const float ed = exp2_fast(xd - mx);
    sum = wave_sum(sum) + ed;
    const float cr = dust ? (float)N : 1.f;
    const float ur = (dust ? log2f((float)N) - lmn : -lmn) - mx - log2_fast(sum);
    const float wgt = cr * __builtin_amdgcn_rcpf(sum);
#pragma unroll
    for (int k = 0; k < NV4; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[k][c] = fmaf(t[k][c], wgt, acc[k][c]);
    if (lane == 0) {
      sm_u[w * RPW + ri] = update_u ? ur : 0.f;
      if (update_u) u_out[ip.uoff + i0 + w * RPW + ri] = ur;
    }
  };
  const int nreal = min(max(M - (i0 + w * RPW), 0), RPW);  // the wave's real rows (a prefix of its rows)
#pragma unroll
  for (int p = 0; p < NSTEP; ++p) {
    if (p + 1 < NSTEP) load_step(p + 1, zbuf[(p + 1) & 1]);
#pragma unroll
    for (int r = 0; r < RS; ++r)
      if (p * RS + r < nreal) row(zbuf[p & 1][r], false, p * RS + r);
  }
  {
    // the dustbin row's place among the wave's rows; a pair whose real rows
    // fill whole blocks gets it as an extra row of its last block (last wave)
    const int rd = M - (i0 + w * RPW);
    if (rd >= 0 && (rd < RPW || (w == W - 1 && rd == RPW))) row(zbuf[0][0], true, rd);
    if (lane == 0)
      for (int r = max(rd + 1, 0); r < RPW; ++r) sm_u[w * RPW + r] = -INFINITY;  // past the dustbin row
    if (w == W - 1 && lane == 0 && rd != RPW) sm_u[RB] = -INFINITY;
  }

  const size_t pbase = (size_t)ip.p_off + (size_t)gb * ldz;
  if (update_u) {
#pragma unroll
    for (int k = 0; k < NV4; ++k) sm[w][lane + 64 * k] = make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
  }
  __syncthreads();

  // exact partial of the real column jj over the block's rows (and the
  // dustbin row when the block takes it as an extra row)
  auto exact = [&](int jj) -> float {
    float mx = -INFINITY;
    for (int r = 0; r <= RB; ++r) {
      const int i = i0 + r;
      if (i > M) break;
      const float z = i < M ? zp[(size_t)i * ldz + jj] : alpha2;
      mx = fmaxf(mx, z + sm_u[r]);
    }
    float sum = 0.f;
    for (int r = 0; r <= RB; ++r) {
      const int i = i0 + r;
      if (i > M) break;
      const float z = i < M ? zp[(size_t)i * ldz + jj] : alpha2;
      sum += exp2_fast(z + sm_u[r] - mx);
    }
    return mx + log2_fast(sum);
  };

  if (update_u) {
    for (int q = threadIdx.x; q < NG; q += NT) {
      const int j = 4 * q;
      if (j >= N) break;
      float T[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const float4 a = sm[ww][q];
#pragma unroll
        for (int c = 0; c < 4; ++c) T[c] += f4c(a, c);
      }
      const float4 vq = vl[q];
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (j + c >= N) o[c] = -INFINITY;
        else if (T[c] >= kSumFloor) o[c] = log2_fast(T[c]) - lmn - f4c(vq, c);
        else o[c] = exact(j + c);
      }
      *reinterpret_cast<float4*>(Pout + pbase + j) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (w == 0) {
      // the dustbin column holds alpha in every row, so its partial is
      // exactly alpha + lse2 of the block's u (no exponential of a row's
      // entries can lose it, however far alpha lies below the rows' maxima)
      float mx = -INFINITY;
      for (int r = lane; r <= RB; r += 64)
        if (i0 + r <= M) mx = fmaxf(mx, sm_u[r]);
      mx = wave_max(mx);
      float sum = 0.f;
      for (int r = lane; r <= RB; r += 64)
        if (i0 + r <= M) sum += exp2_fast(sm_u[r] - mx);
      sum = wave_sum(sum);
      if (lane == 0) Pdout[ip.gpre + gb] = alpha2 + mx + log2_fast(sum);
    }
  }

  if constexpr (ARG) {
    // column argmax of Z + u over the block's real rows (lowest row on ties):
    // each wave over its rows, then over the waves (rows ascending with the
    // wave index)
    __syncthreads();  // the partial sums in sm have been read
#pragma unroll
    for (int k = 0; k < NV4; ++k) {
      const int j = 4 * (lane + 64 * k);
      float bv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      int bi[4] = {-1, -1, -1, -1};
      for (int r = 0; r < RPW; ++r) {
        const int i = i0 + w * RPW + r;
        if (i < M && j < N) {
          const float4 q = *reinterpret_cast<const float4*>(zp + (size_t)i * ldz + j);
          const float ua = sm_u[w * RPW + r];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float y = f4c(q, c) + ua;
            if (y > bv[c]) {
              bv[c] = y;
              bi[c] = i;
            }
          }
        }
      }
      sm[w][lane + 64 * k] = make_float4(bv[0], bv[1], bv[2], bv[3]);
      smi[w][lane + 64 * k] = make_int4(bi[0], bi[1], bi[2], bi[3]);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < NG; q += NT) {
      const int j = 4 * q;
      if (j >= N) break;
      float bv[4];
      int bi[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bv[c] = f4c(sm[0][q], c);
        bi[c] = c == 0 ? smi[0][q].x : c == 1 ? smi[0][q].y : c == 2 ? smi[0][q].z : smi[0][q].w;
      }
#pragma unroll
      for (int ww = 1; ww < W; ++ww) {
        const float4 a = sm[ww][q];
        const int4 ai = smi[ww][q];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float y = f4c(a, c);
          if (y > bv[c]) {
            bv[c] = y;
            bi[c] = c == 0 ? ai.x : c == 1 ? ai.y : c == 2 ? ai.z : ai.w;
          }
        }
      }
      *reinterpret_cast<float4*>(PV + pbase + j) = make_float4(bv[0], bv[1], bv[2], bv[3]);
      *reinterpret_cast<int4*>(PI + pbase + j) = make_int4(bi[0], bi[1], bi[2], bi[3]);
    }
  }
}

// The kernel: each workgroup runs the register layout of its own pair's row
// width (a wave-uniform choice), so that the narrow pairs of a ragged batch
// do not pay for the widest one; rows of more than 1024 columns take one row
// per step (their two-step buffer would not fit the registers).  The LDS
// arrays are shared by the layouts, sized for NVMAX.
template <int W, int RPW, int NVMAX, int RS, bool ARG>
__global__ __launch_bounds__(64 * W) void k_sink_iter(const float* __restrict__ Zb, PairTable pt,
                                                      const float* __restrict__ Pin, const float* __restrict__ Pdin,
                                                      float* __restrict__ u_out, float* __restrict__ Pout,
                                                      float* __restrict__ Pdout, float* __restrict__ PV,
                                                      int* __restrict__ PI, float alpha2,
                                                      const float* __restrict__ alpha_dev, int update_u) {
  constexpr int NGS = 64 * NVMAX;
  __shared__ float4 sm[W][NGS];
  __shared__ float4 vl[NGS + 1];
  __shared__ float sm_u[W * RPW + 1];
  __shared__ int4 smi[ARG ? W : 1][ARG ? NGS : 1];
  // The workgroup's pair and row block from one round of table reads: lane
  // l reads entry l of every per-pair array (vector loads, all in flight
  // together), the pair in dispatch order is the count of pairs whose blocks
  // end at or before this one (a ballot over the prefix sums), and its fields
  // are read out of the lanes.  (A search over the prefix sums and lookups
  // through the dispatch order would be a chain of dependent scalar loads,
  // all on the path to the first row load.)
  static_assert(SG_MAX_BATCH <= 64, "one lane per pair");
  const int lane = threadIdx.x & 63, g = blockIdx.x;
  const int np = pt.n_pairs;
  const int e_end = pt.opre[lane + 1], e_beg = pt.opre[lane], e_ord = pt.ord[lane];
  const int e_M = pt.M[lane], e_N = pt.N[lane], e_z = pt.z_off[lane], e_p = pt.p_off[lane], e_u = pt.uoff[lane];
  const int e_g0 = pt.gpre[lane], e_g1 = pt.gpre[lane + 1];
  if (alpha_dev) alpha2 = alpha_dev[0] * kLog2e;
  const int k = __popcll(__ballot(lane < np && g >= e_end));
  if (k >= np) return;
  const int b = __builtin_amdgcn_readlane(e_ord, k);
  IterPair ip;
  ip.gb = g - __builtin_amdgcn_readlane(e_beg, k);
  ip.M = __builtin_amdgcn_readlane(e_M, b);
  ip.N = __builtin_amdgcn_readlane(e_N, b);
  ip.gpre = __builtin_amdgcn_readlane(e_g0, b);
  ip.G = __builtin_amdgcn_readlane(e_g1, b) - ip.gpre;
  ip.z_off = __builtin_amdgcn_readlane(e_z, b);
  ip.p_off = __builtin_amdgcn_readlane(e_p, b);
  ip.uoff = __builtin_amdgcn_readlane(e_u, b);
  const int N = ip.N;
  int4 (*const smip)[NGS] = reinterpret_cast<int4 (*)[NGS]>(&smi[0][0]);  // (used only with ARG)
#define SG_BLOCK(NV, R)                                                                                      \
  sink_iter_block<W, RPW, NV, R, ARG, NGS>(Zb, ip, Pin, Pdin, u_out, Pout, Pdout, PV, PI, alpha2, update_u, sm, vl, \
                                           sm_u, smip)
  if constexpr (NVMAX >= 8) {
    if (N > 1024) {
      SG_BLOCK(8, 1);
      return;
    }
  }
  if constexpr (NVMAX >= 4) {
    if (N > 512) {
      SG_BLOCK(4, RS);
      return;
    }
  }
  if constexpr (NVMAX >= 2) {
    if (N > 256) {
      SG_BLOCK(2, RS);
      return;
    }
  }
  SG_BLOCK(1, RS);
#undef SG_BLOCK
}

// Column reduction of the block partials of every pair: v_j = log2 nu_j -
// lse2_g P[g][j] (write_v), and after the last iteration the column argmax
// over the real rows (idx1) plus the default (-1 / 0) side-B outputs.
// A workgroup takes 64 real columns of one pair (16 lanes x float4, so that
// each partial row is read in whole 256-byte runs); its 16 row lanes
// (threadIdx / 16) take the partial rows g = gl (mod 16).  Loads are
// unconditional at clamped addresses and masked afterwards, so that all of a
// thread's loads are in flight together.  The workgroup that holds column N
// also reduces the dustbin column's partials Pd.
template <bool ARG>
__global__ __launch_bounds__(256) void k_sink_cols(PairTable pt, const float* __restrict__ P,
                                                   const float* __restrict__ Pd,
                                                   float* __restrict__ v_out,
                                                   const float* __restrict__ PV,
                                                   const int* __restrict__ PI, int* __restrict__ idx1,
                                                   int write_v, int Npad, int32_t* __restrict__ m1,
                                                   float* __restrict__ s1) {
  constexpr int GL = 16, U = ARG ? 8 : 16;
  __shared__ float sm_m[GL][64], sm_s[GL][64], sm_b[GL][64];
  __shared__ int sm_i[GL][64];
  const int b = blockIdx.y;
  const int M = pt.M[b], N = pt.N[b];
  if (blockIdx.x * 64 > N) return;
  const int G = pt.gpre[b + 1] - pt.gpre[b];
  const int tid = threadIdx.x;
  const int cl = tid % 16, gl = tid / 16;
  const int js = blockIdx.x * 64 + 4 * cl;  // first of this lane's four columns
  const int ldp = ld4(N);
  const bool real = js < N;
  const int jsc = real ? js : max(ldp - 4, 0);  // an in-bounds address for the masked lanes
  const float* pp = P + pt.p_off[b] + jsc;
  const float lmn = log2f((float)(M + N));
  float mx[4], s[4], best[4];
  int bi[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    mx[c] = -INFINITY;
    s[c] = 0.f;
    best[c] = -INFINITY;
    bi[c] = 0x7fffffff;
  }
  if (N > 0 && (write_v || ARG)) {
    for (int g0 = gl; g0 < G; g0 += GL * U) {
      float4 xs[U];
      int4 bx[ARG ? U : 1];
      float4 bv[ARG ? U : 1];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const size_t o = (size_t)min(g0 + GL * q, G - 1) * ldp;
        xs[q] = *reinterpret_cast<const float4*>(pp + o);
        if constexpr (ARG) {
          bv[q] = *reinterpret_cast<const float4*>(PV + pt.p_off[b] + jsc + o);
          bx[q] = *reinterpret_cast<const int4*>(PI + pt.p_off[b] + jsc + o);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float m2 = mx[c];
#pragma unroll
        for (int q = 0; q < U; ++q)
          if (g0 + GL * q < G) m2 = fmaxf(m2, f4c(xs[q], c));
        float t = mx[c] == -INFINITY ? 0.f : s[c] * exp2_fast(mx[c] - m2);
#pragma unroll
        for (int q = 0; q < U; ++q)
          if (g0 + GL * q < G) t += exp2_fast(f4c(xs[q], c) - m2);
        s[c] = t;
        mx[c] = m2;
        if constexpr (ARG) {
#pragma unroll
          for (int q = 0; q < U; ++q)
            if (g0 + GL * q < G) {
              const int4 ix = bx[q];
              argmax_merge(best[c], bi[c], f4c(bv[q], c), c == 0 ? ix.x : c == 1 ? ix.y : c == 2 ? ix.z : ix.w);
            }
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    sm_m[gl][4 * cl + c] = mx[c];
    sm_s[gl][4 * cl + c] = s[c];
    sm_b[gl][4 * cl + c] = best[c];
    sm_i[gl][4 * cl + c] = bi[c];
  }
  __syncthreads();
  const int t = tid;
  const int j = blockIdx.x * 64 + t;
  if (t < 64 && j < N) {
    float mm = -INFINITY;
#pragma unroll
    for (int q = 0; q < GL; ++q) mm = fmaxf(mm, sm_m[q][t]);
    float ss = 0.f, bb = -INFINITY;
    int ii = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < GL; ++q) {
      if (sm_m[q][t] != -INFINITY) ss += sm_s[q][t] * exp2_fast(sm_m[q][t] - mm);
      argmax_merge(bb, ii, sm_b[q][t], sm_i[q][t]);
    }
    if (write_v) v_out[pt.voff[b] + j] = -lmn - (mm + log2_fast(ss));
    if (ARG) {
      idx1[pt.vpre[b] - b + j] = ii;
      if (m1) {
        m1[(size_t)b * Npad + j] = -1;
        if (s1) s1[(size_t)b * Npad + j] = 0.f;
      }
    }
  }
  // the dustbin column: v_N = log2 M - log2(M+N) - lse2_g Pd[g]
  if (write_v && blockIdx.x == N / 64) {
    __syncthreads();
    const float* pd = Pd + pt.gpre[b];
    float m = -INFINITY, sum = 0.f;
    for (int g = tid; g < G; g += 256) {
      const float x = pd[g];
      const float m2 = fmaxf(m, x);
      sum = (m == -INFINITY ? 0.f : sum * exp2_fast(m - m2)) + exp2_fast(x - m2);
      m = m2;
    }
    const float wm = wave_max(m);
    sum = wave_sum(m == -INFINITY ? 0.f : sum * exp2_fast(m - wm));
    if ((tid & 63) == 0) {
      sm_m[0][tid >> 6] = wm;
      sm_s[0][tid >> 6] = sum;
    }
    __syncthreads();
    if (tid == 0) {
      float mm = -INFINITY;
      for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sm_m[0][w]);
      float ss = 0.f;
      for (int w = 0; w < 4; ++w)
        if (sm_m[0][w] != -INFINITY) ss += sm_s[0][w] * exp2_fast(sm_m[0][w] - mm);
      v_out[pt.voff[b] + N] = log2f((float)M) - lmn - (mm + log2_fast(ss));
    }
  }
}

// ---------------------------------------------------- two-sweep variant
//
// For problems whose Z and its transpose ZT stay resident in the L2 caches
// the two updates run as separate sweeps, one wave per row of Z (which = 0:
// rows i of the couplings, producing u) or of ZT (which = 1: columns j,
// producing v), so that only the duals cross between kernels:
//   out_i = log2 marginal_i - log2 sum_j 2^(Z2_ij + w_j),
// with the dustbin row/column equal to alpha2 and the base-2 marginals
// -log2(M+N) (real rows) and log2(count of the other side) - log2(M+N)
// (dustbin).  w_in == nullptr stands for w = 0 (the first iteration).
// The row statistics of one sweep for one row i of Z (WHICH = 0) or ZT
// (WHICH = 1): lane-owned float4 groups zq / wq of the row and of the
// other side's duals (columns 4*(lane + 64 k) .. +3, loaded clamped in
// bounds: entries past nc and the dustbin row i == nr are replaced here).
// XB (explicit dustbins, the stage entry points on caller-given couplings):
// zq of the dustbin row holds that row's own entries and `dust` is the
// row's dustbin-column entry (the corner for i == nr); otherwise both are
// the constant alpha2.
template <int NV4, bool XB = false>
__device__ __forceinline__ float lse_row(const float4 (&zq)[NV4], const float4 (&wq)[NV4], float wd, float alpha2,
                                         int i, int nr, int nc, int lane, float dust = 0.f) {
  float x[NV4][4];
#pragma unroll
  for (int k = 0; k < NV4; ++k) {
    const int j = 4 * (lane + 64 * k);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      x[k][c] = j + c < nc ? ((XB || i < nr) ? f4c(zq[k], c) : alpha2) + f4c(wq[k], c) : -INFINITY;
  }
  // the dustbin column (j = nc): alpha for every row, or the row's own entry
  const float xd = (XB ? dust : alpha2) + wd;
  float mx = xd;
#pragma unroll
  for (int k = 0; k < NV4; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) mx = fmaxf(mx, x[k][c]);
  mx = wave_max(mx);
  float sum = lane == 0 ? exp2_fast(xd - mx) : 0.f;
#pragma unroll
  for (int k = 0; k < NV4; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) sum += exp2_fast(x[k][c] - mx);
  sum = wave_sum(sum);
  return mx + log2_fast(sum);
}

// Loads of lse_row's operands, unconditional at a real row and column
// clamped in bounds (the dustbin row reads the last real row), so that all
// of them are in flight together.  row: the row's first entry; wv: the
// duals (nullptr: zero).
template <int NV4>
__device__ __forceinline__ void lse_loads(const float* row, const float* wv, int nr, int nc, int lane,
                                          float4 (&zq)[NV4], float4 (&wq)[NV4]) {
  const int ldz = ld4(nc);
#pragma unroll
  for (int k = 0; k < NV4; ++k) zq[k] = wq[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (nc <= 0) return;  // (wave-uniform conditions)
#pragma unroll
  for (int k = 0; k < NV4; ++k) {
    const int jc = min(4 * (lane + 64 * k), ldz - 4);
    if (nr > 0) zq[k] = *reinterpret_cast<const float4*>(row + jc);
    if (wv) wq[k] = *reinterpret_cast<const float4*>(wv + jc);
  }
}

// WHICH: the sweep (0: rows of Z, 1: rows of ZT), fixed at compile time so
// that the table entries sit at fixed offsets once the pair is known.
template <int NV4, int WHICH>
__global__ __launch_bounds__(256) void k_lse(const float* __restrict__ Zbase, PairTable pt,
                                             const float* __restrict__ w_in, float* __restrict__ w_out,
                                             float alpha2, const float* __restrict__ alpha_dev) {
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + wave_id();
  const int* pre = WHICH ? pt.vpre : pt.upre;
  const int b = find_pair(pre, pt.n_pairs, g);
  if (b >= pt.n_pairs) return;
  const int i = g - pre[b];
  const int M = pt.M[b], N = pt.N[b];
  const int nr = WHICH ? N : M, nc = WHICH ? M : N;
  const float* wv = w_in ? w_in + (WHICH ? pt.uoff[b] : pt.voff[b]) : nullptr;
  float4 zq[NV4], wq[NV4];
  lse_loads<NV4>(Zbase + (WHICH ? pt.zt_off[b] : pt.z_off[b]) + (size_t)max(min(i, nr - 1), 0) * ld4(nc), wv, nr, nc,
                 lane, zq, wq);
  const float wd = wv ? wv[nc] : 0.f;
  if (alpha_dev) alpha2 = alpha_dev[0] * kLog2e;  // needed only once the row loads are in flight
  const float l = lse_row<NV4>(zq, wq, wd, alpha2, i, nr, nc, lane);
  if (lane == 0) {
    const float lm = (i < nr ? 0.f : log2f((float)nc)) - log2f((float)(M + N));
    w_out[(WHICH ? pt.voff[b] : pt.uoff[b]) + i] = lm - l;
  }
}

// The same sweep for a single pair, with its sizes and offsets as plain
// arguments: every scalar the row loads need arrives in one round of
// argument loads (no pair search, no table lookups ahead of them).
// Z: the pair's Z or ZT; wv / w_out: the duals read / written (offsets
// applied); nr: rows (the dustbin row is nr); nc: columns; lmn = log2(M+N).
// XB: explicit dustbins (stage entry points): bown [nr + 1] holds each row's
// dustbin-column entry (the corner last) and bcross [ld4(nc + 1)] the
// dustbin row's entries; alpha2 / alpha_dev are unused.
// ARG (the last column sweep over ZT, whose duals wv are the final u): each
// real row j of ZT also leaves the column argmax argmax_i Z2_ij + u_i over
// the real rows (lowest index on ties) in idx1[j], and the default -1 / 0 in
// m1[j] / s1[j] (when given), which k_col_argmax would otherwise compute in
// a launch of its own: the sweep already holds every one of those sums.
template <int NV4, bool XB, bool ARG = false>
__global__ __launch_bounds__(256) void k_lse_one(const float* __restrict__ Z, const float* __restrict__ wv,
                                                 float* __restrict__ w_out, int nr, int nc, float alpha2,
                                                 const float* __restrict__ alpha_dev, float lm_real,
                                                 float lm_dust, const float* __restrict__ bown,
                                                 const float* __restrict__ bcross, int* __restrict__ idx1 = nullptr,
                                                 int32_t* __restrict__ m1 = nullptr, float* __restrict__ s1 = nullptr) {
  static_assert(!(ARG && XB), "the fused column argmax belongs to the pass's own sweep");
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave_id();
  if (i > nr) return;
  float4 zq[NV4], wq[NV4];
  const float* row = (XB && i >= nr) ? bcross : Z + (size_t)max(min(i, nr - 1), 0) * ld4(nc);
  lse_loads<NV4>(row, wv, XB ? 1 : nr, nc, lane, zq, wq);
  if constexpr (ARG) {
    if (i < nr) {  // (wave-uniform)
      float best = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int k = 0; k < NV4; ++k) {
        const int r = 4 * (lane + 64 * k);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float y = f4c(zq[k], c) + f4c(wq[k], c);
          if (r + c < nc && y > best) {
            best = y;
            bi = r + c;
          }
        }
      }
      wave_argmax(best, bi);
      if (lane == 0) {
        idx1[i] = bi;
        if (m1) {
          m1[i] = -1;
          if (s1) s1[i] = 0.f;
        }
      }
    }
  }
  const float wd = wv ? wv[nc] : 0.f;
  const float dust = XB ? bown[i] : 0.f;
  if (!XB && alpha_dev) alpha2 = alpha_dev[0] * kLog2e;
  const float l = lse_row<NV4, XB>(zq, wq, wd, alpha2, i, nr, nc, lane, dust);
  if (lane == 0) w_out[i] = (i < nr ? lm_real : lm_dust) - l;
}

// Column argmax over the real rows (argmax_i Z2_ij + u_i, lowest index on
// ties) from the rows of ZT, one wave per column; also the default (-1 / 0)
// side-B outputs that the extraction overwrites for mutual matches.
template <int NV4, int MODE>
__global__ __launch_bounds__(256) void k_col_argmax(const float* __restrict__ ZTb, PairTable pt,
                                                    const float* __restrict__ u,
                                                    int* __restrict__ idx1, int Npad,
                                                    int32_t* __restrict__ m1, float* __restrict__ s1) {
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + wave_id();
  // flattened real columns: the prefix of N over the pairs is vpre[b] - b
  int b = 0;
  while (b < pt.n_pairs && g >= pt.vpre[b + 1] - (b + 1)) ++b;
  if (b >= pt.n_pairs) return;
  const int j = g - (pt.vpre[b] - b);
  const int M = pt.M[b];
  const float* row = ZTb + pt.zt_off[b] + (size_t)j * ld4(M);
  const float* uu = MODE == EXT_RAW ? nullptr : u + pt.uoff[b];
  float best = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NV4; ++k) {
    const int i = 4 * (lane + 64 * k);
    if (i < M) {
      const float4 z = *reinterpret_cast<const float4*>(row + i);
      const float4 q = MODE == EXT_RAW ? make_float4(0.f, 0.f, 0.f, 0.f) : *reinterpret_cast<const float4*>(uu + i);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float y = (MODE == EXT_DS ? 2.f * f4c(z, c) : f4c(z, c)) + f4c(q, c);
        if (i + c < M && y > best) {
          best = y;
          bi = i + c;
        }
      }
    }
  }
  wave_argmax(best, bi);
  if (lane == 0) {
    idx1[g] = bi;
    if (m1) {
      m1[(size_t)b * Npad + j] = -1;
      if (s1) s1[(size_t)b * Npad + j] = 0.f;
    }
  }
}

// Row argmax of the final log assignment (argmax_j Z_ij + v_j; lowest index
// on ties), mutual check against idx1, score exp(logP), threshold; side-B
// outputs of mutual pairs; -1 / 0 for padded entries and empty pairs.  MODE:
// see EXT_* above (the double-softmax head has no marginal normalisation to
// undo; a raw assignment is read as given).
template <int NV4, int MODE>
__global__ __launch_bounds__(256) void k_sink_extract(const float* __restrict__ Zb, PairTable pt,
                                                      const float* __restrict__ u,
                                                      const float* __restrict__ v,
                                                      const int* __restrict__ idx1, int Mpad,
                                                      int Npad, float thr, int32_t* __restrict__ m0,
                                                      float* __restrict__ s0,
                                                      int32_t* __restrict__ m1,
                                                      float* __restrict__ s1) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave_id();
  const int M = pt.M[b], N = pt.N[b];
  const bool empty = M == 0 || N == 0;
  if (m1 && t >= N && t < Npad && lane == 0) {  // padded side-B entries
    m1[(size_t)b * Npad + t] = -1;
    if (s1) s1[(size_t)b * Npad + t] = 0.f;
  }
  if (empty && m1 && t < N && lane == 0) {
    m1[(size_t)b * Npad + t] = -1;
    if (s1) s1[(size_t)b * Npad + t] = 0.f;
  }
  if (t >= Mpad) return;
  if (t >= M || empty) {
    if (lane == 0) {
      m0[(size_t)b * Mpad + t] = -1;
      s0[(size_t)b * Mpad + t] = 0.f;
    }
    return;
  }
  const int ldz = ld4(N);
  const float* row = Zb + pt.z_off[b] + (size_t)t * ldz;
  const float* vv = MODE == EXT_RAW ? nullptr : v + pt.voff[b];
  float best = -INFINITY;
  int bj = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NV4; ++k) {
    const int j = 4 * (lane + 64 * k);
    if (j < N) {
      const float4 z = *reinterpret_cast<const float4*>(row + j);
      const float4 q = MODE == EXT_RAW ? make_float4(0.f, 0.f, 0.f, 0.f) : *reinterpret_cast<const float4*>(vv + j);
      const float zm = MODE == EXT_DS ? 2.f : 1.f;
      const float x[4] = {zm * z.x + q.x, zm * z.y + q.y, zm * z.z + q.z, zm * z.w + q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < N && x[e] > best) { best = x[e]; bj = j + e; }
    }
  }
  wave_argmax(best, bj);
  if (lane != 0) return;
  // (bj stays out of range only when no entry of the row compares, e.g. NaN scores)
  const bool mutual = bj < N && idx1[pt.vpre[b] - b + bj] == t;
  float score = 0.f;
  int mo = -1;
  if (mutual) {
    // exp(logP) > thr decided in the log domain (exact for any finite logP:
    // exp never reaches 0, so a non-positive threshold accepts every mutual match)
    if (MODE == EXT_RAW) {
      score = expf(best);
      if (thr <= 0.f || best > logf(thr)) mo = bj;
    } else {
      const float lp2 = best + u[pt.uoff[b] + t] + (MODE == EXT_DS ? 0.f : log2f((float)(M + N)));
      score = exp2f(lp2);
      if (thr <= 0.f || lp2 > log2f(thr)) mo = bj;
    }
    if (m1) {
      m1[(size_t)b * Npad + bj] = mo >= 0 ? t : -1;
      if (s1) s1[(size_t)b * Npad + bj] = score;
    }
  }
  m0[(size_t)b * Mpad + t] = mo;
  s0[(size_t)b * Mpad + t] = score;
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

// ------------------------------------------------- stage entry points
//
// Caller-given (M+1) x (N+1) matrices C (natural log, leading dimension ldc)
// enter the sweeps and the extraction through the same internal layout as
// the pass: the real block scaled by `scale` into Z [M][ld4(N)] and its
// transpose ZT [N][ld4(M)] (32 x 32 tiles through LDS, so that both sides
// are written in whole rows); with bcol / brow non-null, the dustbin column
// C[i][N] (i <= M, the corner last) and row C[M][j] (j <= N, the corner
// last), scaled, for the explicit-dustbin sweeps.
__global__ __launch_bounds__(256) void k_stage_couplings(const float* __restrict__ C, int64_t ldc, int M, int N,
                                                         float scale, float* __restrict__ Z, float* __restrict__ ZT,
                                                         float* __restrict__ bcol, float* __restrict__ brow) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + ty + 8 * r, j = j0 + tx;
    float x = 0.f;
    if (i < M && j < N) {
      x = C[(int64_t)i * ldc + j] * scale;
      Z[(size_t)i * ld4(N) + j] = x;
    }
    tile[ty + 8 * r][tx] = x;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = j0 + ty + 8 * r, i = i0 + tx;
    if (i < M && j < N) ZT[(size_t)j * ld4(M) + i] = tile[tx][ty + 8 * r];
  }
  if (bcol && blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = threadIdx.x; i <= M; i += 256) bcol[i] = C[(int64_t)i * ldc + N] * scale;
    for (int j = threadIdx.x; j <= N; j += 256) brow[j] = C[(int64_t)M * ldc + j] * scale;
  }
}

// Outputs of the Sinkhorn stage entry point: the natural-log duals u = ln2 u2,
// v = ln2 v2, and (logP non-null) logP = C + u + v + log(M+N) over the
// (M+1) x (N+1) block, from the caller's own C.
__global__ __launch_bounds__(256) void k_stage_duals(const float* __restrict__ C, int64_t ldc, int M, int N,
                                                     const float* __restrict__ u2, const float* __restrict__ v2,
                                                     float* __restrict__ u, float* __restrict__ v,
                                                     float* __restrict__ logP, int64_t ldp, float lmn) {
  const int i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j > N) return;
  const float ui = kLn2 * u2[i], vj = kLn2 * v2[j];
  if (j == 0) u[i] = ui;
  if (i == 0) v[j] = vj;
  if (logP) logP[(int64_t)i * ldp + j] = C[(int64_t)i * ldc + j] + ((ui + vj) + lmn);
}

// The bordered couplings of the scores stage entry point: the real block S
// [M][lds] (natural log) copied into C and the dustbin row and column set to
// the dustbin score, read on the device.  One thread per entry of a row.
__global__ __launch_bounds__(256) void k_stage_border(const float* __restrict__ S, int lds, int M, int N,
                                                      const float* __restrict__ alpha_dev, float* __restrict__ C,
                                                      int64_t ldc) {
  const int i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j > N) return;
  C[(int64_t)i * ldc + j] = (i < M && j < N) ? S[(size_t)i * lds + j] : alpha_dev[0];
}

hipError_t launch_stage_border(const float* S, int lds, int M, int N, const float* alpha_dev, float* C, int64_t ldc,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_stage_border, dim3((N + 1 + 255) / 256, M + 1), dim3(256), 0, st, S, lds, M, N, alpha_dev, C,
                     ldc);
  return hipGetLastError();
}

hipError_t launch_stage_couplings(const float* C, int64_t ldc, int M, int N, float scale, float* Z, float* ZT,
                                  float* bcol, float* brow, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stage_couplings, dim3((N + 31) / 32, (M + 31) / 32), dim3(256), 0, st, C, ldc, M, N, scale,
                     Z, ZT, bcol, brow);
  return hipGetLastError();
}

hipError_t launch_stage_duals(const float* C, int64_t ldc, int M, int N, const float* u2, const float* v2, float* u,
                              float* v, float* logP, int64_t ldp, hipStream_t st) {
  const float lmn = logf((float)(M + N));
  hipLaunchKernelGGL(k_stage_duals, dim3((N + 1 + 255) / 256, M + 1), dim3(256), 0, st, C, ldc, M, N, u2, v2, u, v,
                     logP, ldp, lmn);
  return hipGetLastError();
}

static int sink_nv4(int max_n);

// One explicit-dustbin sweep (k_lse_one<.., true>) over the nr + 1 rows of Z
// (or ZT): w_out = lm - lse2 over the row of Z2 + w_in.
hipError_t launch_lse_explicit(const float* Z, const float* w_in, float* w_out, int nr, int nc, float lm_real,
                               float lm_dust, const float* bown, const float* bcross, hipStream_t st) {
  const int nv4 = sink_nv4(nc);
  dim3 grid((nr + 1 + 3) / 4);
#define SG_LSEX(NV)                                                                                       \
  if (nv4 == NV) {                                                                                        \
    hipLaunchKernelGGL((k_lse_one<NV, true>), grid, dim3(256), 0, st, Z, w_in, w_out, nr, nc, 0.f, nullptr, \
                       lm_real, lm_dust, bown, bcross, nullptr, nullptr, nullptr);                        \
    return hipGetLastError();                                                                             \
  }
  SG_LSEX(1) SG_LSEX(2) SG_LSEX(4) SG_LSEX(8) SG_LSEX(16)
#undef SG_LSEX
  return hipErrorInvalidValue;
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

// ------------------------------------------------------------- launchers

static int max_n(const PairTable& pt) {
  int m = 0;
  for (int b = 0; b < pt.n_pairs; ++b) m = std::max(m, pt.N[b]);
  return m;
}
// float4 groups per lane that cover the longest row of the batch (power of two)
static int sink_nv4(int max_n) {
  int nv4 = 1;
  while (256 * nv4 < max_n) nv4 *= 2;
  return nv4;
}

int sink_rows_per_block(const int* M, const int* N, int n_pairs) {
  (void)M;
  int mn = 0;
  for (int b = 0; b < n_pairs; ++b) mn = std::max(mn, N[b]);
  // two rows per wave (eight per workgroup) up to 2048 columns, where the
  // row values still fit the registers; one beyond
  return sink_nv4(mn) <= 8 ? 8 : 4;
}

hipError_t launch_sink_rows(const float* Z, const PairTable& pt, const float* v_in, float* u_out,
                            float* P, float* Pd, float* PV, int* PI, float alpha2, const float* alpha_dev,
                            int update_u, hipStream_t st) {
  const int blocks = pt.gpre[pt.n_pairs];
  if (blocks <= 0) return hipSuccess;
  const int nv4 = sink_nv4(max_n(pt));
  const int rpw = pt.rb / 4;
  if (rpw * nv4 > 16 || rpw * 4 != pt.rb) return hipErrorInvalidValue;
  const bool arg = PV != nullptr;
#define SG_ROWS(R, NV)                                                                                   \
  if (rpw == R && nv4 == NV) {                                                                            \
    if (arg)                                                                                             \
      hipLaunchKernelGGL((k_sink_rows<R, NV, true>), dim3(blocks), dim3(256), 0, st, Z, pt, v_in, u_out, P, \
                         Pd, PV, PI, alpha2, alpha_dev, update_u);                                        \
    else                                                                                                 \
      hipLaunchKernelGGL((k_sink_rows<R, NV, false>), dim3(blocks), dim3(256), 0, st, Z, pt, v_in, u_out, \
                         P, Pd, PV, PI, alpha2, alpha_dev, update_u);                                     \
    return hipGetLastError();                                                                             \
  }
  SG_ROWS(2, 1) SG_ROWS(2, 2) SG_ROWS(2, 4) SG_ROWS(2, 8)
  SG_ROWS(1, 1) SG_ROWS(1, 2) SG_ROWS(1, 4) SG_ROWS(1, 8) SG_ROWS(1, 16)
#undef SG_ROWS
  return hipErrorInvalidValue;
}

// Rows per workgroup of the fused one-pass iteration (four waves of 16 rows,
// two rows at a time), and the widest rows it takes.  Measured on 32 pairs of
// 1024 x 1024 (graph-replayed, 100 iterations): 27.3-28.2 us per iteration
// against 28.7 us with eight waves of 8 rows, 29.4 us with 32-row blocks and
// 35.0 us for the row pass + column reduction pair.  On 32 ragged pairs (M, N
// from 256 to 2048, 174 MB of couplings): 39.0 us against 54.8 us for the pair
// of launches; the same kernel took 52.3 us with one register layout for
// every pair (the widest), 47.3 us with per-pair layouts, and the duals of the
// widest rows in registers (169 registers: two waves per SIMD), widest-first
// order included.
constexpr int kIterRows = 64;
constexpr int kIterWaves = 4;
constexpr int kIterMaxCols = 2048;

int sink_iter_blocks(int M, int rb) { return std::max(1, (M + rb - 1) / rb); }

int sink_iter_rows_per_block(const int* N, int n_pairs) {
  for (int b = 0; b < n_pairs; ++b)
    if (N[b] > kIterMaxCols) return 0;
  return kIterRows;
}

hipError_t launch_sink_iter(const float* Z, const PairTable& pt, const float* Pin, const float* Pdin, float* u_out,
                            float* Pout, float* Pdout, float* PV, int* PI, float alpha2, const float* alpha_dev,
                            int update_u, hipStream_t st) {
  const int blocks = pt.gpre[pt.n_pairs];
  if (blocks <= 0) return hipSuccess;
  if (pt.rb != kIterRows) return hipErrorInvalidValue;
  const int nv4 = sink_nv4(max_n(pt));
  const bool arg = PV != nullptr;
#define SG_ITER(NV, RS)                                                                                    \
  if (nv4 == NV) {                                                                                         \
    if (arg)                                                                                               \
      hipLaunchKernelGGL((k_sink_iter<kIterWaves, kIterRows / kIterWaves, NV, RS, true>), dim3(blocks),     \
                         dim3(64 * kIterWaves), 0, st, Z, pt, Pin, Pdin, u_out, Pout, Pdout, PV, PI, alpha2, \
                         alpha_dev, update_u);                                                             \
    else                                                                                                   \
      hipLaunchKernelGGL((k_sink_iter<kIterWaves, kIterRows / kIterWaves, NV, RS, false>), dim3(blocks),    \
                         dim3(64 * kIterWaves), 0, st, Z, pt, Pin, Pdin, u_out, Pout, Pdout, PV, PI, alpha2, \
                         alpha_dev, update_u);                                                             \
    return hipGetLastError();                                                                              \
  }
  SG_ITER(1, 2) SG_ITER(2, 2) SG_ITER(4, 2) SG_ITER(8, 2)
#undef SG_ITER
  return hipErrorInvalidValue;
}

hipError_t launch_sink_cols(const PairTable& pt, const float* P, const float* Pd, float* v_out, const float* PV,
                            const int* PI, int* idx1, int write_v, int Npad, int32_t* m1, float* s1,
                            hipStream_t st) {
  if (pt.n_pairs <= 0) return hipSuccess;
  dim3 grid((max_n(pt) + 1 + 63) / 64, pt.n_pairs);
  if (PV)
    hipLaunchKernelGGL(k_sink_cols<true>, grid, dim3(256), 0, st, pt, P, Pd, v_out, PV, PI, idx1, write_v, Npad, m1, s1);
  else
    hipLaunchKernelGGL(k_sink_cols<false>, grid, dim3(256), 0, st, pt, P, Pd, v_out, PV, PI, idx1, write_v, Npad, m1, s1);
  return hipGetLastError();
}

hipError_t launch_lse(const float* Z, const PairTable& pt, int which, const float* w_in, float* w_out,
                      float alpha2, const float* alpha_dev, int total_rows, hipStream_t st, int* idx1, int32_t* m1,
                      float* s1) {
  if (total_rows <= 0) return hipSuccess;
  if (idx1 && (pt.n_pairs != 1 || which != 1 || !w_in)) return hipErrorInvalidValue;
  int nc = 0;
  for (int b = 0; b < pt.n_pairs; ++b) nc = std::max(nc, which ? pt.M[b] : pt.N[b]);
  const int nv4 = sink_nv4(nc);
  dim3 grid((total_rows + 3) / 4);
  if (pt.n_pairs == 1) {
    const int M = pt.M[0], N = pt.N[0], nr = which ? N : M;
    const float* zp = Z + (which ? pt.zt_off[0] : pt.z_off[0]);
    const float* wv = w_in ? w_in + (which ? pt.uoff[0] : pt.voff[0]) : nullptr;
    float* wo = w_out + (which ? pt.voff[0] : pt.uoff[0]);
    // the same single-precision logarithms as the pair-table kernel
    const float lmn = std::log2((float)(M + N));
    const float lr = 0.f - lmn, ld = std::log2((float)nc) - lmn;
#define SG_LSE(NV)                                                                                             \
    if (nv4 == NV) {                                                                                           \
      if (idx1)                                                                                                \
        hipLaunchKernelGGL((k_lse_one<NV, false, true>), grid, dim3(256), 0, st, zp, wv, wo, nr, nc, alpha2,    \
                           alpha_dev, lr, ld, nullptr, nullptr, idx1, m1, s1);                                 \
      else                                                                                                     \
        hipLaunchKernelGGL((k_lse_one<NV, false>), grid, dim3(256), 0, st, zp, wv, wo, nr, nc, alpha2, alpha_dev, \
                           lr, ld, nullptr, nullptr, nullptr, nullptr, nullptr);                               \
      return hipGetLastError();                                                                                \
    }
    SG_LSE(1) SG_LSE(2) SG_LSE(4) SG_LSE(8) SG_LSE(16)
#undef SG_LSE
    return hipErrorInvalidValue;
  }
#define SG_LSE(NV)                                                                                            \
  if (nv4 == NV) {                                                                                            \
    if (which) hipLaunchKernelGGL((k_lse<NV, 1>), grid, dim3(256), 0, st, Z, pt, w_in, w_out, alpha2, alpha_dev); \
    else hipLaunchKernelGGL((k_lse<NV, 0>), grid, dim3(256), 0, st, Z, pt, w_in, w_out, alpha2, alpha_dev);       \
    return hipGetLastError();                                                                                 \
  }
  SG_LSE(1) SG_LSE(2) SG_LSE(4) SG_LSE(8) SG_LSE(16)
#undef SG_LSE
  return hipErrorInvalidValue;
}

hipError_t launch_col_argmax(const float* ZT, const PairTable& pt, const float* u, int* idx1, int Npad,
                             int32_t* m1, float* s1, int mode, hipStream_t st) {
  int cols = 0, mr = 0;
  for (int b = 0; b < pt.n_pairs; ++b) {
    cols += pt.N[b];
    mr = std::max(mr, pt.M[b]);
  }
  if (cols <= 0) return hipSuccess;
  const int nv4 = sink_nv4(mr);
  dim3 grid((cols + 3) / 4);
#define SG_CA(NV)                                                                                             \
  if (nv4 == NV) {                                                                                            \
    if (mode == EXT_DS)                                                                                       \
      hipLaunchKernelGGL((k_col_argmax<NV, EXT_DS>), grid, dim3(256), 0, st, ZT, pt, u, idx1, Npad, m1, s1);  \
    else if (mode == EXT_RAW)                                                                                 \
      hipLaunchKernelGGL((k_col_argmax<NV, EXT_RAW>), grid, dim3(256), 0, st, ZT, pt, u, idx1, Npad, m1, s1); \
    else                                                                                                      \
      hipLaunchKernelGGL((k_col_argmax<NV, EXT_SINKHORN>), grid, dim3(256), 0, st, ZT, pt, u, idx1, Npad, m1, \
                         s1);                                                                                 \
    return hipGetLastError();                                                                                 \
  }
  SG_CA(1) SG_CA(2) SG_CA(4) SG_CA(8) SG_CA(16)
#undef SG_CA
  return hipErrorInvalidValue;
}

hipError_t launch_sink_extract(const float* Z, const PairTable& pt, const float* u, const float* v,
                               const int* idx1, int Mpad, int Npad, float thr, int32_t* m0, float* s0,
                               int32_t* m1, float* s1, int mode, hipStream_t st) {
  const int n = std::max(Mpad, m1 ? Npad : 0);
  if (n <= 0 || pt.n_pairs <= 0) return hipSuccess;
  const int nc = max_n(pt);
  const int nv4 = (nc + 255) / 256;
  dim3 grid((n + 3) / 4, pt.n_pairs);
#define SG_EXT(NV)                                                                                              \
  if (mode == EXT_DS)                                                                                           \
    hipLaunchKernelGGL((k_sink_extract<NV, EXT_DS>), grid, dim3(256), 0, st, Z, pt, u, v, idx1, Mpad, Npad, thr, \
                       m0, s0, m1, s1);                                                                         \
  else if (mode == EXT_RAW)                                                                                     \
    hipLaunchKernelGGL((k_sink_extract<NV, EXT_RAW>), grid, dim3(256), 0, st, Z, pt, u, v, idx1, Mpad, Npad,    \
                       thr, m0, s0, m1, s1);                                                                    \
  else                                                                                                          \
    hipLaunchKernelGGL((k_sink_extract<NV, EXT_SINKHORN>), grid, dim3(256), 0, st, Z, pt, u, v, idx1, Mpad,     \
                       Npad, thr, m0, s0, m1, s1)
  if (nv4 <= 1) SG_EXT(1);
  else if (nv4 <= 2) SG_EXT(2);
  else if (nv4 <= 4) SG_EXT(4);
  else if (nv4 <= 8) SG_EXT(8);
  else if (nv4 <= 16) SG_EXT(16);
  else return hipErrorInvalidValue;
#undef SG_EXT
  return hipGetLastError();
}

hipError_t launch_write_logp(const float* Z, const PairTable& pt, const float* u, const float* v,
                             float alpha2, const float* alpha_dev, float* logP, int64_t ld,
                             int64_t pair_stride, int total_rows, hipStream_t st) {
  if (total_rows <= 0) return hipSuccess;
  const int nc = max_n(pt) + 1;
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
