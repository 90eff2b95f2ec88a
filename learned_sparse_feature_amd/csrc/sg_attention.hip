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

// Throughput variant (bf16, many workgroups): 128 queries of one image and
// one head per workgroup, one wave per 32 queries, every wave running over
// all keys.  64-key tiles of K and of V^T are staged through LDS with
// coalesced 16-byte loads (double buffered: the next tile is in flight while
// the current one is consumed) and shared by the four waves.
template <int DH>
__global__ __launch_bounds__(256) void k_attention_wide(AttnArgs a, SegTable seg) {
  constexpr int BQ = 128, BKEY = 64;
  constexpr int KP = DH + 8;    // K tile row pitch (keys x dims)
  constexpr int VP = BKEY + 8;  // V^T tile row pitch (dims x keys)
  constexpr int KCH = BKEY * DH / 8 / 256;  // 16-byte chunks per thread per K (and V) tile
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BKEY * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][DH * VP];

  const int H = a.heads;
  int t = blockIdx.x / H;
  const int h = blockIdx.x % H;
  int s = 0;
  for (; s < seg.n_seg; ++s) {
    const int nt = (seg.n[s] + BQ - 1) / BQ;
    if (t < nt) break;
    t -= nt;
  }
  if (s >= seg.n_seg) return;
  const int q0 = t * BQ, nq = seg.n[s], qrow0 = seg.row0[s];
  const int src = a.cross ? seg.partner[s] : s;
  const int nk = seg.n[src], krow0 = seg.row0[src];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5, lq = lane & 31;
  const int D = a.D, ldq = a.ldqk;
  const bf16* __restrict__ qk = reinterpret_cast<const bf16*>(a.qk);
  const bf16* __restrict__ vt = reinterpret_cast<const bf16*>(a.vt);

  const int qi = q0 + 32 * w + lq;
  const bool qvalid = qi < nq;
  bf16x8 Qr[DH / 16];
  {
    const bf16* qp = qk + (size_t)(qrow0 + (qvalid ? qi : 0)) * ldq + h * DH;
#pragma unroll
    for (int i = 0; i < DH / 16; ++i) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + i * 16 + hi * 8);
      if (!qvalid) v = (bf16x8)(bf16)0.f;
      Qr[i] = v;
    }
  }

  // cooperative tile loads: K chunk c -> key c / (DH/8), dims (c % (DH/8)) * 8;
  // V^T chunk c -> dim c / 8, keys (c % 8) * 8
  bf16x8 kreg[KCH], vreg[KCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int key = c / (DH / 8), part = c % (DH / 8);
      bf16x8 v = (bf16x8)(bf16)0.f;
      if (k0 + key < nk) v = *reinterpret_cast<const bf16x8*>(qk + (size_t)(krow0 + k0 + key) * ldq + D + h * DH + part * 8);
      kreg[i] = v;
      const int dim = c / 8, kp = (c % 8) * 8;
      const bf16* vp = vt + (size_t)(h * DH + dim) * a.ldvt + krow0 + k0 + kp;
      if (k0 + kp + 8 <= nk) {
        v = *reinterpret_cast<const bf16x8*>(vp);
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = k0 + kp + x < nk ? vp[x] : (bf16)0.f;
      }
      vreg[i] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<bf16x8*>(&Ks[buf][(c / (DH / 8)) * KP + (c % (DH / 8)) * 8]) = kreg[i];
      *reinterpret_cast<bf16x8*>(&Vs[buf][(c / 8) * VP + (c % 8) * 8]) = vreg[i];
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 O[DH / 32];
#pragma unroll
  for (int c = 0; c < DH / 32; ++c) O[c] = zero16();

  const int ntk = (nk + BKEY - 1) / BKEY;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < ntk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ntk) gload((kt + 1) * BKEY);
#pragma unroll
    for (int kb = 0; kb < BKEY / 32; ++kb) {
      const int k0 = kt * BKEY + kb * 32;
      if (k0 >= nk) break;
      f32x16 S = zero16();
#pragma unroll
      for (int i = 0; i < DH / 16; ++i) {
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(&Ks[cur][(kb * 32 + lq) * KP + i * 16 + hi * 8]);
        S = mfma(kv, Qr[i], S);
      }
      float e[16], tmax = -INFINITY;
      if (k0 + 32 <= nk) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          e[i] = S[i] * a.scale2;
          tmax = fmaxf(tmax, e[i]);
        }
      } else {
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
      float psum = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2_fast(e[i] - m_new);
        psum += p;
        pb[i >> 3][i & 7] = (bf16)p;
      }
      l_run = l_run * corr + psum;
      m_run = m_new;
      if (__ballot(corr != 1.f)) {
#pragma unroll
        for (int c = 0; c < DH / 32; ++c)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[c][i] *= corr;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int cb = 0; cb < DH / 32; ++cb) {
          const bf16* vp = &Vs[cur][(cb * 32 + lq) * VP + kb * 32 + 16 * j + 4 * hi];
          const bf16x4 x0 = *reinterpret_cast<const bf16x4*>(vp);
          const bf16x4 x1 = *reinterpret_cast<const bf16x4*>(vp + 8);
          const bf16x8 va = (bf16x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          O[cb] = mfma(va, pb[j], O[cb]);
        }
    }
    if (kt + 1 < ntk) sstore(cur ^ 1);
    __syncthreads();
  }

  l_run += __shfl_xor(l_run, 32);
  if (qvalid) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16* out = reinterpret_cast<bf16*>(a.out) + (size_t)(qrow0 + qi) * D + h * DH;
#pragma unroll
    for (int cb = 0; cb < DH / 32; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o;
#pragma unroll
        for (int x = 0; x < 4; ++x) o[x] = (bf16)(O[cb][4 * g + x] * inv);
        *reinterpret_cast<bf16x4*>(out + cb * 32 + 8 * g + 4 * hi) = o;
      }
  }
}

hipError_t launch_attention(int op, int dh, const AttnArgs& a, const SegTable& seg, int heads,
                            hipStream_t st) {
  int tiles = 0, wide_tiles = 0;
  for (int s = 0; s < seg.n_seg; ++s) {
    tiles += (seg.n[s] + 31) / 32;
    wide_tiles += (seg.n[s] + 127) / 128;
  }
  if (tiles == 0) return hipSuccess;
  // with enough work for the whole chip, 128-query workgroups sharing LDS
  // tiles; otherwise 32-query workgroups that split the keys over 8 waves
  if (op == SG_BF16 && dh == 64 && wide_tiles * heads >= 1024) {
    hipLaunchKernelGGL((k_attention_wide<64>), dim3(wide_tiles * heads), dim3(256), 0, st, a, seg);
    return hipGetLastError();
  }
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
