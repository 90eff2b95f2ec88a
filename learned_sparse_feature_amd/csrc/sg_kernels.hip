// HIP kernels (gfx950 / CDNA4) of the SuperGlue matching forward pass.
//
// Layout conventions (all device memory, row-major):
//  * compact rows: every image of the call occupies a block of rows padded to
//    a multiple of 32 (so tiles never straddle images and row starts are
//    aligned); padding rows hold unspecified values and are never read as
//    data;
//  * states X [R][D] fp32; q|k [R][2D] and the message [R][D] in the operand
//    type; v is stored transposed, VT [D][ldvt], so that the P.V product
//    reads contiguous keys;
//  * scores are stored pre-multiplied by log2(e): all exponentials and
//    logarithms of softmax and Sinkhorn are base 2 (v_exp_f32 / v_log_f32).
//
// MFMA lane layouts used (checked on the device): for
// v_mfma_f32_32x32x16_bf16 lane l holds A[l%32][8*(l/32) + t] and
// B[8*(l/32) + t][l%32] (t = 0..7); for v_mfma_f32_32x32x2f32 lane l holds
// A[l%32][l/32] and B[l/32][l%32]; both return C[8*(i/4) + 4*(l/32) + i%4][l%32]
// in accumulator i.  Because a contraction index may be relabelled freely as
// long as A and B agree, the kernels map MFMA k-slots to whatever
// contiguous memory suits each lane.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "sg_internal.h"

namespace sg {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return (float)v; }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- encoder

// First encoder layer for every point of every image: normalise (x, y) by
// the image size ((k - size/2) / (0.7 max(w, h))), h0 = ReLU(W0 [x, y, c] + b0);
// also initialise the states X with the descriptors (the encoder output is
// added to them by the last encoder layer).
template <typename WT>
__global__ __launch_bounds__(256) void k_encode_l0(const float* __restrict__ kA,
                                                   const float* __restrict__ cA,
                                                   const float* __restrict__ dA,
                                                   const float* __restrict__ kB,
                                                   const float* __restrict__ cB,
                                                   const float* __restrict__ dB, float4 imgA,
                                                   float4 imgB, SegTable seg, int D,
                                                   const WT* __restrict__ W0,
                                                   const WT* __restrict__ b0, int w0,
                                                   float* __restrict__ H0,
                                                   float* __restrict__ X) {
  int t = blockIdx.x, s = 0;
  for (; s < seg.n_seg; ++s) {
    int nt = (seg.n[s] + 31) >> 5;
    if (t < nt) break;
    t -= nt;
  }
  if (s >= seg.n_seg) return;
  const int p0 = t * 32, n = seg.n[s];
  const int np = min(32, n - p0);
  const bool isA = seg.side[s] == 0;
  const float* kp = (isA ? kA : kB) + 2 * (size_t)(seg.in_off[s] + p0);
  const float* cf = (isA ? cA : cB) + (size_t)(seg.in_off[s] + p0);
  const float* de = (isA ? dA : dB) + (size_t)D * (seg.in_off[s] + p0);
  const float4 img = isA ? imgA : imgB;
  const size_t row0 = (size_t)seg.row0[s] + p0;
  // descriptors -> X (float4 copies)
  const int d4 = D / 4;
  for (int e = threadIdx.x; e < np * d4; e += blockDim.x) {
    int r = e / d4, c = e % d4;
    reinterpret_cast<float4*>(X + (row0 + r) * D)[c] =
        reinterpret_cast<const float4*>(de + (size_t)r * D)[c];
  }
  for (int e = threadIdx.x; e < np * w0; e += blockDim.x) {
    int r = e / w0, o = e % w0;
    float x = kp[2 * r], y = kp[2 * r + 1];
    if (img.x > 0.f) {
      float sc = 0.7f * fmaxf(img.x, img.y);
      x = (x - 0.5f * img.x) / sc;
      y = (y - 0.5f * img.y) / sc;
    }
    float c = cf[r];
    float h = to_f32(W0[3 * o]) * x + to_f32(W0[3 * o + 1]) * y + to_f32(W0[3 * o + 2]) * c +
              to_f32(b0[o]);
    H0[(row0 + r) * w0 + o] = fmaxf(h, 0.f);
  }
}

// ---------------------------------------------------------------- GEMM
//
// C = A W^T (+ epilogue) with A [rows][K] (optionally two sources split at
// column K0: the [x || m] concatenation of the update MLP) and W [n][K] the
// row-major Linear weight.  64x64 output tile per 256-thread workgroup, four
// waves of 32x32, each a chain of 32x32 MFMAs over K; A and W tiles are
// converted to the operand type while staged through LDS.

template <typename SrcT, typename OpT, int G>
__device__ __forceinline__ void load_group(const SrcT* p, OpT* dst) {
  if constexpr (std::is_same<SrcT, float>::value) {
#pragma unroll
    for (int i = 0; i < G; i += 4) {
      float4 v = *reinterpret_cast<const float4*>(p + i);
      dst[i] = (OpT)v.x; dst[i + 1] = (OpT)v.y; dst[i + 2] = (OpT)v.z; dst[i + 3] = (OpT)v.w;
    }
  } else {
    // bf16 source: 8 (G == 8) or 4 (G == 4) elements
    if constexpr (G == 8) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = (OpT)(float)v[i];
    } else {
      bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = (OpT)(float)v[i];
    }
  }
}

template <typename OpT, typename A0T, typename WT, typename OutT, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g, GemmBatch bt) {
  constexpr bool BF = std::is_same<OpT, bf16>::value;
  constexpr int BM = 64, BN = 64;
  constexpr int BK = BF ? 32 : 16;
  constexpr int G = BF ? 8 : 4;  // elements per thread per staged tile
  constexpr int PITCH = BK + (BF ? 8 : 4);
  __shared__ __attribute__((aligned(16))) OpT As[BM * PITCH];
  __shared__ __attribute__((aligned(16))) OpT Ws[BN * PITCH];

  const GemmProblem P = bt.p[blockIdx.z];
  const int r0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  if (r0 >= P.rows || n0 >= P.n_out) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = tid / (BK / G), lk = (tid % (BK / G)) * G;

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  for (int k0 = 0; k0 < g.K; k0 += BK) {
    OpT av[G], wv[G];
    const int k = k0 + lk;
    const int r = r0 + lr;
    if (r < P.rows && k < g.K) {
      if (k < g.K0)
        load_group<A0T, OpT, G>(reinterpret_cast<const A0T*>(g.A0) +
                                    (size_t)(P.a_row0 + r) * g.lda0 + k, av);
      else
        load_group<OpT, OpT, G>(reinterpret_cast<const OpT*>(g.A1) +
                                    (size_t)(P.a_row0 + r) * g.lda1 + (k - g.K0), av);
    } else {
#pragma unroll
      for (int i = 0; i < G; ++i) av[i] = (OpT)0.f;
    }
    const int n = n0 + lr;
    if (n < P.n_out && k < g.K) {
      load_group<WT, OpT, G>(reinterpret_cast<const WT*>(g.W) + (size_t)(P.w_row0 + n) * g.ldw + k,
                             wv);
    } else {
#pragma unroll
      for (int i = 0; i < G; ++i) wv[i] = (OpT)0.f;
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      As[lr * PITCH + lk + i] = av[i];
      Ws[lr * PITCH + lk + i] = wv[i];
    }
    __syncthreads();
    const OpT* ap = As + (wm * 32 + (lane & 31)) * PITCH;
    const OpT* wp = Ws + (wn * 32 + (lane & 31)) * PITCH;
    if constexpr (BF) {
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(ap + s * 16 + (lane >> 5) * 8);
        bf16x8 b = *reinterpret_cast<const bf16x8*>(wp + s * 16 + (lane >> 5) * 8);
        acc = mfma(a, b, acc);
      }
    } else {
#pragma unroll
      for (int s = 0; s < BK / 2; ++s) {
        // k-slot (l/32) of step s is column 8*(l/32) + s of the staged tile
        acc = mfma(ap[(lane >> 5) * 8 + s], wp[(lane >> 5) * 8 + s], acc);
      }
    }
    __syncthreads();
  }

  const int n = n0 + wn * 32 + (lane & 31);
  if (n >= P.n_out) return;
  float bias = 0.f;
  if (EPI != EPI_SCORE && g.bias) bias = to_f32(reinterpret_cast<const WT*>(g.bias)[n]);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (r >= P.rows) continue;
    float v = acc[i] + bias;
    if constexpr (EPI == EPI_BIAS || EPI == EPI_RELU) {
      if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
      reinterpret_cast<OutT*>(g.C)[P.c_off + (size_t)r * P.ldc + n] = (OutT)v;
    } else if constexpr (EPI == EPI_RESID) {
      float* c = reinterpret_cast<float*>(g.C) + P.c_off + (size_t)r * P.ldc + n;
      *c = *c + v;
    } else if constexpr (EPI == EPI_QKV) {
      if (n < g.split)
        reinterpret_cast<OutT*>(g.C)[P.c_off + (size_t)r * P.ldc + n] = (OutT)v;
      else
        reinterpret_cast<OutT*>(g.C2)[P.ct_off + (size_t)(n - g.split) * P.ldct + r] = (OutT)v;
    } else {  // EPI_SCORE
      v = acc[i] * g.scale;
      reinterpret_cast<float*>(g.C)[P.c_off + (size_t)r * P.ldc + n] = v;
      reinterpret_cast<float*>(g.C2)[P.ct_off + (size_t)n * P.ldct + r] = v;
    }
  }
}

// ------------------------------------------------------------- attention
//
// One workgroup = 32 queries of one image and one head; its four waves split
// the keys of the source image (tiles of 32, interleaved) and each keeps an
// online softmax (running max, running sum, unnormalised output) in
// registers.  S^T = K Q^T is formed so that every lane owns one query
// column: the row statistics then need only the lane and its partner lane
// l^32.  P never leaves registers: its accumulator layout is reused directly
// as the B operand of O^T = V^T P^T.  The four partial softmaxes are merged
// through LDS at the end.

template <typename OpT, int DH>
__global__ __launch_bounds__(256) void k_attention(AttnArgs a, SegTable seg) {
  constexpr bool BF = std::is_same<OpT, bf16>::value;
  constexpr int NCB = (DH + 31) / 32;
  __shared__ float sm_m[4][32], sm_l[4][32];
  __shared__ float sm_o[4][NCB * 32][33];

  int t = blockIdx.x, s = 0;
  for (; s < seg.n_seg; ++s) {
    int nt = (seg.n[s] + 31) >> 5;
    if (t < nt) break;
    t -= nt;
  }
  if (s >= seg.n_seg) return;
  const int q0 = t * 32, nq = seg.n[s], qrow0 = seg.row0[s];
  const int src = a.cross ? seg.partner[s] : s;
  const int nk = seg.n[src], krow0 = seg.row0[src];
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hi = lane >> 5, lq = lane & 31;
  const int D = a.D, ld2 = 2 * a.D;
  const OpT* __restrict__ qk = reinterpret_cast<const OpT*>(a.qk);
  const OpT* __restrict__ vt = reinterpret_cast<const OpT*>(a.vt);

  const int qi = q0 + lq;
  const bool qvalid = qi < nq;
  // Q^T operand, kept in registers for the whole key loop
  constexpr int QS = BF ? DH / 16 : DH / 2;
  typedef typename std::conditional<BF, bf16x8, float>::type QT;
  QT Qr[QS];
  {
    const OpT* qp = qk + (size_t)(qrow0 + (qvalid ? qi : 0)) * ld2 + h * DH;
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < QS; ++i) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + i * 16 + hi * 8);
        if (!qvalid) v = (bf16x8)(bf16)0.f;
        Qr[i] = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < QS; i += 4) {
        float4 v = *reinterpret_cast<const float4*>(qp + hi * (DH / 2) + i);
        Qr[i] = qvalid ? v.x : 0.f; Qr[i + 1] = qvalid ? v.y : 0.f;
        Qr[i + 2] = qvalid ? v.z : 0.f; Qr[i + 3] = qvalid ? v.w : 0.f;
      }
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 O[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[c][i] = 0.f;

  const int ntk = (nk + 31) >> 5;
  for (int kt = w; kt < ntk; kt += 4) {
    const int k0 = kt * 32;
    const bool tail = k0 + 32 > nk;
    const int ki = k0 + lq;
    const bool kvalid = ki < nk;
    const OpT* kp = qk + (size_t)(krow0 + (kvalid ? ki : 0)) * ld2 + D + h * DH;
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < QS; ++i) {
        bf16x8 kv = *reinterpret_cast<const bf16x8*>(kp + i * 16 + hi * 8);
        if (!kvalid) kv = (bf16x8)(bf16)0.f;
        S = mfma(kv, Qr[i], S);
      }
    } else {
#pragma unroll
      for (int i = 0; i < QS; i += 4) {
        float4 v = *reinterpret_cast<const float4*>(kp + hi * (DH / 2) + i);
        if (!kvalid) v = make_float4(0.f, 0.f, 0.f, 0.f);
        S = mfma(v.x, Qr[i], S);
        S = mfma(v.y, Qr[i + 1], S);
        S = mfma(v.z, Qr[i + 2], S);
        S = mfma(v.w, Qr[i + 3], S);
      }
    }
    float e[16], tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = k0 + 8 * (i >> 2) + 4 * hi + (i & 3);
      e[i] = kk < nk ? S[i] * a.scale2 : -INFINITY;
      tmax = fmaxf(tmax, e[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float corr = exp2_fast(m_run - m_new);
    float p[16], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = exp2_fast(e[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[c][i] *= corr;

    if constexpr (BF) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (bf16)p[8 * j + i];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int c = cb * 32 + lq;
          bf16x8 va = (bf16x8)(bf16)0.f;
          if (c < DH) {
            const OpT* vp = vt + (size_t)(h * DH + c) * a.ldvt + krow0 + k0 + 16 * j + 4 * hi;
            if (!tail) {
              bf16x4 x0 = *reinterpret_cast<const bf16x4*>(vp);
              bf16x4 x1 = *reinterpret_cast<const bf16x4*>(vp + 8);
              va = (bf16x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            } else {
              const int kb = k0 + 16 * j + 4 * hi;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                va[i] = kb + i < nk ? vp[i] : (bf16)0.f;
                va[4 + i] = kb + 8 + i < nk ? vp[8 + i] : (bf16)0.f;
              }
            }
          }
          O[cb] = mfma(va, pb, O[cb]);
        }
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int c = cb * 32 + lq;
        const OpT* vp = vt + (size_t)(h * DH + (c < DH ? c : 0)) * a.ldvt + krow0 + k0 + 4 * hi;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (c < DH) {
            if (!tail) {
              v = *reinterpret_cast<const float4*>(vp + 8 * g4);
            } else {
              const int kb = k0 + 8 * g4 + 4 * hi;
              v.x = kb < nk ? vp[8 * g4] : 0.f;
              v.y = kb + 1 < nk ? vp[8 * g4 + 1] : 0.f;
              v.z = kb + 2 < nk ? vp[8 * g4 + 2] : 0.f;
              v.w = kb + 3 < nk ? vp[8 * g4 + 3] : 0.f;
            }
          }
          O[cb] = mfma(v.x, p[4 * g4], O[cb]);
          O[cb] = mfma(v.y, p[4 * g4 + 1], O[cb]);
          O[cb] = mfma(v.z, p[4 * g4 + 2], O[cb]);
          O[cb] = mfma(v.w, p[4 * g4 + 3], O[cb]);
        }
      }
    }
  }

  l_run += __shfl_xor(l_run, 32);
  if (hi == 0) {
    sm_m[w][lq] = m_run;
    sm_l[w][lq] = l_run;
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = cb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
      if (c < DH) sm_o[w][c][lq] = O[cb][i];
    }
  __syncthreads();
  OpT* out = reinterpret_cast<OpT*>(a.out);
  for (int idx = threadIdx.x; idx < 32 * DH; idx += 256) {
    const int q = idx / DH, c = idx % DH;
    if (q0 + q >= nq) continue;
    float mm = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) mm = fmaxf(mm, sm_m[ww][q]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float sc = sm_m[ww][q] == -INFINITY ? 0.f : exp2_fast(sm_m[ww][q] - mm);
      L += sm_l[ww][q] * sc;
      o += sm_o[ww][c][q] * sc;
    }
    out[(size_t)(qrow0 + q0 + q) * D + h * DH + c] = (OpT)(L > 0.f ? o / L : 0.f);
  }
}

// --------------------------------------------------------------- Sinkhorn
//
// One wave per row of Z (which = 0: rows i of the (M+1)x(N+1) couplings,
// producing u) or of ZT (which = 1: columns j, producing v):
//   out_i = log2 marginal_i - log2 sum_j 2^(Z2_ij + w_j),
// with the dustbin row/column equal to alpha2 and the base-2 marginals
// -log2(M+N) (real rows) and log2(count of the other side) - log2(M+N)
// (dustbin).  w_in == nullptr stands for w = 0 (the first iteration).

__device__ __forceinline__ int find_pair(const int* pre, int n_pairs, int g) {
  int b = 0;
  while (b < n_pairs && g >= pre[b + 1]) ++b;
  return b;
}

template <int MAXV>
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
  const float* row = Zbase + (which ? pt.zt_off[b] + (size_t)i * ld4(M) : pt.z_off[b] + (size_t)i * ld4(N));
  const float* wv = w_in ? w_in + (which ? pt.upre[b] : pt.vpre[b]) : nullptr;
  const bool real = i < nr;
  float vals[MAXV];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < MAXV; ++t) {
    const int j = lane + 64 * t;
    float x = -INFINITY;
    if (j <= nc) {
      x = (real && j < nc) ? row[j] : alpha2;
      if (wv) x += wv[j];
    }
    vals[t] = x;
    mx = fmaxf(mx, x);
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < MAXV; ++t) sum += exp2_fast(vals[t] - mx);
  sum = wave_sum(sum);
  if (lane == 0) {
    const float lm = (real ? 0.f : log2f((float)nc)) - log2f((float)(M + N));
    w_out[pre[b] + i] = lm - (mx + log2_fast(sum));
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
  const float* wv = which ? u + pt.upre[b] : v + pt.vpre[b];
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
        const float lp2 = val0[mpre + t] + u[pt.upre[b] + t] + lmn;
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
        const float lp2 = val0[mpre + i] + u[pt.upre[b] + i] + lmn;
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
  const float ui = u[pt.upre[b] + i];
  const float* row = Zbase + pt.z_off[b] + (size_t)i * ld4(N);
  for (int j = blockIdx.x * 256 + threadIdx.x; j <= N; j += gridDim.x * 256) {
    const float z = (i < M && j < N) ? row[j] : alpha2;
    logP[b * pair_stride + (int64_t)i * ld + j] = kLn2 * (z + ui + v[pt.vpre[b] + j] + lmn);
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

// ------------------------------------------------------------- launchers

hipError_t launch_encode_l0(const float* kptsA, const float* confA, const float* descA,
                            const float* kptsB, const float* confB, const float* descB,
                            const float img[4], const SegTable& seg, int R, int D,
                            const void* W0, const void* b0, int w0, int dtype, float* H0,
                            float* X, hipStream_t st) {
  int tiles = 0;
  for (int s = 0; s < seg.n_seg; ++s) tiles += (seg.n[s] + 31) / 32;
  (void)R;
  if (tiles == 0) return hipSuccess;
  const float4 ia = make_float4(img[0], img[1], 0.f, 0.f), ib = make_float4(img[2], img[3], 0.f, 0.f);
  if (dtype == SG_BF16)
    hipLaunchKernelGGL(k_encode_l0<bf16>, dim3(tiles), dim3(256), 0, st, kptsA, confA, descA, kptsB,
                       confB, descB, ia, ib, seg, D, (const bf16*)W0, (const bf16*)b0, w0, H0, X);
  else
    hipLaunchKernelGGL(k_encode_l0<float>, dim3(tiles), dim3(256), 0, st, kptsA, confA, descA,
                       kptsB, confB, descB, ia, ib, seg, D, (const float*)W0, (const float*)b0, w0,
                       H0, X);
  return hipGetLastError();
}

template <typename OpT, typename A0T, typename WT, typename OutT, int EPI>
static void gemm_go(const GemmArgs& g, const GemmBatch& b, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((k_gemm<OpT, A0T, WT, OutT, EPI>), grid, dim3(256), 0, st, g, b);
}

hipError_t launch_gemm(int op, int a0f, int wd, int outf, int epi, const GemmArgs& g,
                       const GemmBatch& b, int max_rows, int max_n, hipStream_t st) {
  if (max_rows <= 0 || max_n <= 0 || b.n <= 0) return hipSuccess;
  dim3 grid((max_n + 63) / 64, (max_rows + 63) / 64, b.n);
  // The combinations the pipeline uses.
  if (op == SG_F32) {
    // fp32 operands: A0 fp32, weights in the blob type, fp32 out
    if (wd == SG_F32) {
      switch (epi) {
        case EPI_BIAS: gemm_go<float, float, float, float, EPI_BIAS>(g, b, grid, st); break;
        case EPI_RELU: gemm_go<float, float, float, float, EPI_RELU>(g, b, grid, st); break;
        case EPI_RESID: gemm_go<float, float, float, float, EPI_RESID>(g, b, grid, st); break;
        case EPI_QKV: gemm_go<float, float, float, float, EPI_QKV>(g, b, grid, st); break;
        case EPI_SCORE: gemm_go<float, float, float, float, EPI_SCORE>(g, b, grid, st); break;
        default: return hipErrorInvalidValue;
      }
    } else {  // fp32 encoder on a bf16 blob
      switch (epi) {
        case EPI_RELU: gemm_go<float, float, bf16, float, EPI_RELU>(g, b, grid, st); break;
        case EPI_RESID: gemm_go<float, float, bf16, float, EPI_RESID>(g, b, grid, st); break;
        default: return hipErrorInvalidValue;
      }
    }
  } else {
    if (wd != SG_BF16) return hipErrorInvalidValue;
    if (a0f) {
      switch (epi) {
        case EPI_QKV: gemm_go<bf16, float, bf16, bf16, EPI_QKV>(g, b, grid, st); break;
        case EPI_RELU: gemm_go<bf16, float, bf16, bf16, EPI_RELU>(g, b, grid, st); break;
        case EPI_BIAS:
          if (outf) gemm_go<bf16, float, bf16, float, EPI_BIAS>(g, b, grid, st);
          else gemm_go<bf16, float, bf16, bf16, EPI_BIAS>(g, b, grid, st);
          break;
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (epi) {
        case EPI_BIAS: gemm_go<bf16, bf16, bf16, bf16, EPI_BIAS>(g, b, grid, st); break;
        case EPI_RESID: gemm_go<bf16, bf16, bf16, float, EPI_RESID>(g, b, grid, st); break;
        default: return hipErrorInvalidValue;
      }
    }
  }
  return hipGetLastError();
}

hipError_t launch_attention(int op, int dh, const AttnArgs& a, const SegTable& seg, int heads,
                            hipStream_t st) {
  int tiles = 0;
  for (int s = 0; s < seg.n_seg; ++s) tiles += (seg.n[s] + 31) / 32;
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, heads);
  if (op == SG_BF16) {
    if (dh == 64) hipLaunchKernelGGL((k_attention<bf16, 64>), grid, dim3(256), 0, st, a, seg);
    else if (dh == 16) hipLaunchKernelGGL((k_attention<bf16, 16>), grid, dim3(256), 0, st, a, seg);
    else return hipErrorInvalidValue;
  } else {
    if (dh == 64) hipLaunchKernelGGL((k_attention<float, 64>), grid, dim3(256), 0, st, a, seg);
    else if (dh == 16) hipLaunchKernelGGL((k_attention<float, 16>), grid, dim3(256), 0, st, a, seg);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
  const int nc = max_cols(pt, which);
  dim3 grid((total_rows + 3) / 4);
  if (nc <= 256) hipLaunchKernelGGL(k_lse<4>, grid, dim3(256), 0, st, Z, pt, which, w_in, w_out, alpha2, alpha_dev);
  else if (nc <= 576) hipLaunchKernelGGL(k_lse<9>, grid, dim3(256), 0, st, Z, pt, which, w_in, w_out, alpha2, alpha_dev);
  else if (nc <= 1088) hipLaunchKernelGGL(k_lse<17>, grid, dim3(256), 0, st, Z, pt, which, w_in, w_out, alpha2, alpha_dev);
  else if (nc <= 2112) hipLaunchKernelGGL(k_lse<33>, grid, dim3(256), 0, st, Z, pt, which, w_in, w_out, alpha2, alpha_dev);
  else if (nc <= 4160) hipLaunchKernelGGL(k_lse<65>, grid, dim3(256), 0, st, Z, pt, which, w_in, w_out, alpha2, alpha_dev);
  else return hipErrorInvalidValue;
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
