// Multi-head attention of one GNN stage (self or cross) on MFMA (gfx950).
//
// One workgroup = 32 queries of one image and one head.  Its NW waves split
// the 32-key tiles of the source image round robin; each wave keeps an
// online softmax (running max, running sum, unnormalised output) in
// registers and prefetches its next K/V tile while it works on the current
// one.  S^T = K Q^T is formed so that every lane owns one query column: the
// softmax statistics of a query then need only the lane and its partner
// lane l^32.  P never leaves registers: its accumulator layout is reused as
// the B operand of O^T = V^T P^T, with V read from the transposed copy VT.
// The NW partial softmaxes are merged through LDS at the end.
#include "sg_device.h"

namespace sg {

template <typename OpT, int DH, int NW>
__global__ __launch_bounds__(64 * NW) void k_attention(AttnArgs a, SegTable seg) {
  constexpr bool BF = std::is_same<OpT, bf16>::value;
  constexpr int NCB = (DH + 31) / 32;  // 32-channel blocks of the output
  constexpr int QS = BF ? DH / 16 : DH / 8;  // Q / K registers: bf16x8 or float4 per lane
  __shared__ float sm_m[NW][32], sm_l[NW][32];
  __shared__ float sm_o[NW][DH][33];

  // Workgroup id = tile * H + head: consecutive ids go to different XCDs, so
  // with 4 heads an XCD serves one head and keeps that head's K/V in its L2.
  const int H = a.heads;
  int t = blockIdx.x / H;
  const int s = find_segment(seg, &t);
  if (s >= seg.n_seg) return;
  const int q0 = t * 32, nq = seg.n[s], qrow0 = seg.row0[s];
  const int src = a.cross ? seg.partner[s] : s;
  const int nk = seg.n[src], krow0 = seg.row0[src];
  const int h = blockIdx.x % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hi = lane >> 5, lq = lane & 31;
  const int D = a.D, ld2 = a.ldqk;
  const OpT* __restrict__ qk = reinterpret_cast<const OpT*>(a.qk);
  const OpT* __restrict__ vt = reinterpret_cast<const OpT*>(a.vt);

  typedef typename std::conditional<BF, bf16x8, float4>::type KT;
  typedef typename std::conditional<BF, bf16x4, float4>::type VT;
  constexpr int NV = BF ? 4 * NCB : 4 * NCB;  // V registers per lane per tile

  // Q^T operand, kept in registers for the whole key loop.  bf16: lane half
  // hi holds dims 16 i + 8 hi .. +7; fp32: dims hi*DH/2 + 4 i .. +3.
  const int qi = q0 + lq;
  const bool qvalid = qi < nq;
  KT Qr[QS];
  {
    const OpT* qp = qk + (size_t)(qrow0 + (qvalid ? qi : 0)) * ld2 + h * DH;
#pragma unroll
    for (int i = 0; i < QS; ++i) {
      KT v = BF ? *reinterpret_cast<const KT*>(qp + i * 16 + hi * 8)
                : *reinterpret_cast<const KT*>(qp + hi * (DH / 2) + 4 * i);
      if (!qvalid) v = (KT)(OpT)0.f;
      Qr[i] = v;
    }
  }

  // K / V registers of one key tile (32 keys from k0).  V for channel block
  // cb: bf16: keys k0 + 16 j + 4 hi .. +3 and +8 .. +11 (index 2 (2 cb + j) + 0/1);
  // fp32: keys k0 + 8 g + 4 hi .. +3 (index 4 cb + g).
  auto load_tile = [&](int kt, KT* kr, VT* vr) {
    const int k0 = kt * 32;
    const bool tail = k0 + 32 > nk;
    const int ki = k0 + lq;
    const bool kvalid = ki < nk;
    const OpT* kp = qk + (size_t)(krow0 + (kvalid ? ki : 0)) * ld2 + D + h * DH;
#pragma unroll
    for (int i = 0; i < QS; ++i) {
      KT v = BF ? *reinterpret_cast<const KT*>(kp + i * 16 + hi * 8)
                : *reinterpret_cast<const KT*>(kp + hi * (DH / 2) + 4 * i);
      if (!kvalid) v = (KT)(OpT)0.f;
      kr[i] = v;
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = cb * 32 + lq;
      const bool cvalid = c < DH;
      const OpT* vp = vt + (size_t)(h * DH + (cvalid ? c : 0)) * a.ldvt + krow0 + k0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // bf16: e = 2 j + half -> keys 16 j + 8 half + 4 hi; fp32: e = g -> keys 8 g + 4 hi
        const int koff = BF ? 16 * (e >> 1) + 8 * (e & 1) + 4 * hi : 8 * e + 4 * hi;
        VT v = (VT)(OpT)0.f;
        if (cvalid) {
          if (!tail) {
            v = *reinterpret_cast<const VT*>(vp + koff);
          } else {
#pragma unroll
            for (int x = 0; x < 4; ++x) v[x] = k0 + koff + x < nk ? vp[koff + x] : (OpT)0.f;
          }
        }
        vr[4 * cb + e] = v;
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 O[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) O[c] = zero16();

  const int ntk = (nk + 31) >> 5;
  // PT tiles of this wave are in flight at once (register slots 0..PT-1):
  // slot j holds tile w + NW (base + j); after it is processed the slot is
  // refilled with the tile PT rounds ahead.
  constexpr int PT = BF ? 4 : 2;
  KT kr[PT][QS];
  VT vr[PT][NV];
#pragma unroll
  for (int j = 0; j < PT; ++j)
    if (w + NW * j < ntk) load_tile(w + NW * j, kr[j], vr[j]);
  for (int base = 0; w + NW * base < ntk; base += PT) {
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int kt = w + NW * (base + j);
    if (kt >= ntk) break;
    const KT* kc = kr[j];
    const VT* vc = vr[j];
    const int k0 = kt * 32;
    f32x16 S = zero16();
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < QS; ++i) S = mfma(kc[i], Qr[i], S);
    } else {
#pragma unroll
      for (int i = 0; i < QS; ++i) {
        S = mfma(kc[i].x, Qr[i].x, S);
        S = mfma(kc[i].y, Qr[i].y, S);
        S = mfma(kc[i].z, Qr[i].z, S);
        S = mfma(kc[i].w, Qr[i].w, S);
      }
    }
    float e[16], tmax = -INFINITY;
    if (k0 + 32 <= nk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        e[i] = S[i] * a.scale2;
        tmax = fmaxf(tmax, e[i]);
      }
    } else {  // the last, partial tile: keys past the image are masked
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = k0 + 8 * (i >> 2) + 4 * hi + (i & 3);
        e[i] = kk < nk ? S[i] * a.scale2 : -INFINITY;
        tmax = fmaxf(tmax, e[i]);
      }
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
          const bf16x4 x0 = vc[4 * cb + 2 * j], x1 = vc[4 * cb + 2 * j + 1];
          const bf16x8 va = (bf16x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          O[cb] = mfma(va, pb, O[cb]);
        }
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 v = vc[4 * cb + g4];
          O[cb] = mfma(v.x, p[4 * g4], O[cb]);
          O[cb] = mfma(v.y, p[4 * g4 + 1], O[cb]);
          O[cb] = mfma(v.z, p[4 * g4 + 2], O[cb]);
          O[cb] = mfma(v.w, p[4 * g4 + 3], O[cb]);
        }
    }
    const int kt_next = kt + NW * PT;
    if (kt_next < ntk) load_tile(kt_next, kr[j], vr[j]);
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
  for (int idx = threadIdx.x; idx < 32 * DH; idx += 64 * NW) {
    const int q = idx / DH, c = idx % DH;
    if (q0 + q >= nq) continue;
    float mm = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, sm_m[ww][q]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float sc = sm_m[ww][q] == -INFINITY ? 0.f : exp2_fast(sm_m[ww][q] - mm);
      L += sm_l[ww][q] * sc;
      o += sm_o[ww][c][q] * sc;
    }
    out[(size_t)(qrow0 + q0 + q) * D + h * DH + c] = (OpT)(L > 0.f ? o / L : 0.f);
  }
}

hipError_t launch_attention(int op, int dh, const AttnArgs& a, const SegTable& seg, int heads,
                            hipStream_t st) {
  int tiles = 0;
  for (int s = 0; s < seg.n_seg; ++s) tiles += (seg.n[s] + 31) / 32;
  if (tiles == 0) return hipSuccess;
  constexpr int NW = 8;
  dim3 grid(tiles * heads);
  if (op == SG_BF16) {
    if (dh == 64) hipLaunchKernelGGL((k_attention<bf16, 64, NW>), grid, dim3(64 * NW), 0, st, a, seg);
    else if (dh == 16) hipLaunchKernelGGL((k_attention<bf16, 16, NW>), grid, dim3(64 * NW), 0, st, a, seg);
    else return hipErrorInvalidValue;
  } else {
    if (dh == 64) hipLaunchKernelGGL((k_attention<float, 64, NW>), grid, dim3(64 * NW), 0, st, a, seg);
    else if (dh == 16) hipLaunchKernelGGL((k_attention<float, 16, NW>), grid, dim3(64 * NW), 0, st, a, seg);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sg
