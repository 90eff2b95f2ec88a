// Multi-head attention of one GNN stage (self or cross) on MFMA (gfx950).
//
// One workgroup = 32 queries of one image and one head.  Its NW waves split
// the key tiles of the source image round robin; each wave keeps an online
// softmax (running max, running sum, unnormalised output) in registers.
// With NW = 8 (two waves per SIMD, at most 256 registers each) a wave holds
// one K/V tile at a time and the other wave of its SIMD covers the load
// latency; with fewer waves each prefetches its next tile while it works on
// the current one.  S^T = K Q^T is formed so that every lane owns one query column: the
// softmax statistics of a query then need only the lane and its partner
// lane l^32.  P never leaves registers: its accumulator layout is reused as
// the B operand of O^T = V^T P^T, with V read from the transposed copy VT.
// The NW partial softmaxes are merged through LDS at the end.
#include "sg_device.h"

namespace sg {

// PAIR1: the two segments of a single pair (each the other's partner),
// whose entries then sit at fixed argument offsets.  SH (with PAIR1, the
// bidirectional cross stage with one similarity): the scores are not formed
// here but read from the similarity a.sm, already scaled to base 2, and every
// query's normaliser is its row's log-sum-exp a.lse, so the probabilities are
// exp2(s - lse) with no running maximum; the wave merge then sums outputs
// whose weights already total one.
template <typename OpT, int DH, int NW, bool PAIR1, bool SH = false>
__global__ __launch_bounds__(64 * NW) void k_attention(AttnArgs a, SegTable seg) {
  static_assert(!SH || PAIR1, "the shared similarity is laid out for one pair");
  if constexpr (PAIR1)
    args_in_sgprs(a.qk, a.vt, a.ks, a.vs, a.D, a.ldqk, a.ldvt, a.cross, a.heads, a.scale2, a.stop, seg.n[0],
                  seg.n[1], seg.row0[0], seg.row0[1]);
  if (a.stop && *a.stop) return;  // a later layer of a pass that has already stopped
  constexpr bool BF = std::is_same<OpT, bf16>::value;
  constexpr int NCB = (DH + 31) / 32;        // 32-channel blocks of the output
  constexpr int QS = BF ? DH / 16 : DH / 8;  // Q / K registers per 32 keys: bf16x8 or float4 per lane
  constexpr int KB = BF ? 2 : 1;             // 32-key blocks per key tile (64 keys in bf16)
  __shared__ float sm_m[NW][32], sm_l[NW][32];
  __shared__ float sm_o[NW][DH][33];

  // Workgroup id = tile * H + head: consecutive ids go to different XCDs, so
  // with 4 heads an XCD serves one head and keeps that head's K/V in its L2.
  const int H = a.heads;
  int t = blockIdx.x / H;
  int nq, qrow0, nk, krow0;
  int sgi = 0;  // (SH) the query image: 0 = A, 1 = B
  if constexpr (PAIR1) {
    const int n0 = seg.n[0], n1 = seg.n[1], nt0 = (n0 + 31) >> 5;
    if (t >= nt0 + ((n1 + 31) >> 5)) return;
    const bool s1 = t >= nt0;
    if (s1) t -= nt0;
    if constexpr (SH) sgi = s1 ? 1 : 0;
    const bool k1 = a.cross ? !s1 : s1;
    nq = s1 ? n1 : n0;
    qrow0 = s1 ? seg.row0[1] : seg.row0[0];
    nk = k1 ? n1 : n0;
    krow0 = k1 ? seg.row0[1] : seg.row0[0];
  } else {
    const int s = find_segment(seg, &t);
    if (s >= seg.n_seg) return;
    nq = seg.n[s];
    qrow0 = seg.row0[s];
    const int src = a.cross ? seg.partner[s] : s;
    nk = seg.n[src];
    krow0 = seg.row0[src];
  }
  const int q0 = t * 32;
  const int h = blockIdx.x % H;
  const int lane = threadIdx.x & 63, w = wave_id(), hi = lane >> 5, lq = lane & 31;
  const int D = a.D, ld2 = a.ldqk;
  const OpT* __restrict__ qk = reinterpret_cast<const OpT*>(a.qk);
  const OpT* __restrict__ vt = reinterpret_cast<const OpT*>(a.vt);

  typedef typename std::conditional<BF, bf16x8, float4>::type KT;
  typedef typename std::conditional<BF, bf16x8, float4>::type VT;
  constexpr int NV = BF ? 2 * NCB : 4 * NCB;  // V registers per lane per 32 keys

  // Every image occupies a whole number of 32-row tiles of the row space, so
  // Q, K and V^T loads of any 32-key block of the image stay in bounds
  // without masks; scores and values of keys past the image are masked, and
  // queries past the image are not stored.
  // Q^T operand, kept in registers for the whole key loop.  bf16: lane half
  // hi holds dims 16 i + 8 hi .. +7; fp32: dims hi*DH/2 + 4 i .. +3.
  KT Qr[QS];
  if constexpr (!SH) {
    const OpT* qp = qk + (size_t)(qrow0 + q0 + lq) * ld2 + h * DH;
#pragma unroll
    for (int i = 0; i < QS; ++i)
      Qr[i] = BF ? *reinterpret_cast<const KT*>(qp + i * 16 + hi * 8)
                 : *reinterpret_cast<const KT*>(qp + hi * (DH / 2) + 4 * i);
  }
  // (SH) this lane's similarity row (its query; rows past the image read the
  // last one and are not stored) and its log-sum-exp
  const float* srow = nullptr;
  float lse_q = 0.f;
  if constexpr (SH) {
    const int qc = min(q0 + lq, nq - 1);
    srow = a.sm + a.s_off[sgi] + (size_t)h * a.s_hs[sgi] + (size_t)qc * a.s_ld[sgi];
    lse_q = a.lse[a.l_off[sgi] + h * a.l_hs[sgi] + qc];
  }

  // K / V registers of one 32-key block from key k0.  bf16: the swizzled
  // blocks of ks / vs give each lane its MFMA operand as one 16-byte load:
  // K chunk i (dims 16 i.. of the head), V chunk 2 cb + j (output rows =
  // the 32 features of block f = (h DH + 32 cb) / 32, keys 16 j..).  fp32:
  // K row-major (dims hi*DH/2 + 4 i), V^T rows, keys 8 g + 4 hi .. +3 (index
  // 4 cb + g); channels past DH (DH < 32) read channel DH - 1 and are zeroed.
  auto load_block = [&](int k0, KT* kr, VT* vr) {
    if constexpr (BF) {
      const size_t tile = (size_t)((krow0 + k0) >> 5);
      if constexpr (!SH) {
        const bf16* kp = reinterpret_cast<const bf16*>(a.ks) + (tile * (D / 16) + h * (DH / 16)) * 512 + lane * 8;
#pragma unroll
        for (int i = 0; i < QS; ++i) kr[i] = *reinterpret_cast<const bf16x8*>(kp + i * 512);
      }
      const bf16* vp = reinterpret_cast<const bf16*>(a.vs) + (tile * (D / 32) + (h * DH) / 32) * 1024 + lane * 8;
#pragma unroll
      for (int e = 0; e < NV; ++e) vr[e] = *reinterpret_cast<const bf16x8*>(vp + e * 512);
    } else {
      if constexpr (!SH) {
        const OpT* kp = qk + (size_t)(krow0 + k0 + lq) * ld2 + D + h * DH;
#pragma unroll
        for (int i = 0; i < QS; ++i) kr[i] = *reinterpret_cast<const KT*>(kp + hi * (DH / 2) + 4 * i);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int c = cb * 32 + lq;
        const OpT* vp = vt + (size_t)(h * DH + min(c, DH - 1)) * a.ldvt + krow0 + k0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          VT v = *reinterpret_cast<const VT*>(vp + 8 * e + 4 * hi);
          if (DH < 32 && c >= DH) v = (VT)(OpT)0.f;
          vr[4 * cb + e] = v;
        }
      }
    }
  };
  // a key tile = KB blocks; a block past the image (possible in the last
  // tile) re-reads the image's last block and is fully masked below
  const int nkb = (nk + 31) >> 5;
  auto load_tile = [&](int kt, KT (*kr)[QS], VT (*vr)[NV]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) load_block(32 * min(kt * KB + kb, nkb - 1), kr[kb], vr[kb]);
  };

  float m_run = SH ? lse_q : -INFINITY, l_run = 0.f;
  f32x16 O[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) O[c] = zero16();

  // one key tile: S^T = K Q^T per block, online softmax (base 2) over the
  // tile's 64 keys, O^T += V^T P^T
  auto process = [&](KT (*kc)[QS], VT (*vc)[NV], int kt) {
    f32x16 S[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) S[kb] = zero16();
    if constexpr (SH) {
      // element i of block kb: key 32 kb + 8 (i / 4) + 4 hi + i % 4 of the
      // tile, four consecutive keys per 16-byte load (clamped into the row;
      // keys past the image are masked below)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int key = kt * 32 * KB + 32 * kb + 8 * g4 + 4 * hi;
          const float4 v = *reinterpret_cast<const float4*>(srow + min(key, ((nk - 1) & ~3)));
          S[kb][4 * g4] = v.x;
          S[kb][4 * g4 + 1] = v.y;
          S[kb][4 * g4 + 2] = v.z;
          S[kb][4 * g4 + 3] = v.w;
        }
    } else if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < QS; ++i)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) S[kb] = mfma(kc[kb][i], Qr[i], S[kb]);
    } else {
#pragma unroll
      for (int i = 0; i < QS; ++i)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          S[kb] = mfma(kc[kb][i].x, Qr[i].x, S[kb]);
          S[kb] = mfma(kc[kb][i].y, Qr[i].y, S[kb]);
          S[kb] = mfma(kc[kb][i].z, Qr[i].z, S[kb]);
          S[kb] = mfma(kc[kb][i].w, Qr[i].w, S[kb]);
        }
    }
    const int k0 = kt * 32 * KB;
    // keys past the image (partial last tile): scores -inf, values 0 (padding
    // rows of V may hold anything a caller staged there)
    VT vm[KB][NV];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < NV; ++e) vm[kb][e] = vc[kb][e];
    if (k0 + 32 * KB > nk) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (k0 + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3) >= nk) S[kb][i] = -INFINITY;
        if constexpr (BF) {
          // element t of chunk 2 cb + j: key 16 j + 8 (t / 4) + 4 hi + t % 4
#pragma unroll
          for (int e = 0; e < NV; ++e)
#pragma unroll
            for (int x = 0; x < 8; ++x)
              if (k0 + 32 * kb + 16 * (e & 1) + 8 * (x >> 2) + 4 * hi + (x & 3) >= nk) vm[kb][e][x] = (OpT)0.f;
        } else {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int x = 0; x < 4; ++x)
                if (k0 + 32 * kb + 8 * e + 4 * hi + x >= nk) vm[kb][4 * cb + e][x] = (OpT)0.f;
        }
      }
    }
    float tmax = S[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, S[kb][i]);
    tmax = half_swap_max(tmax);
    const float m_new = SH ? m_run : fmaxf(m_run, tmax * a.scale2);
    // rescale the running output only when some query's maximum moved
    if (!SH && __ballot(m_new != m_run)) {
      const float corr = exp2_fast(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[c][i] *= corr;
      m_run = m_new;
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = exp2_fast(fmaf(S[kb][i], a.scale2, -m_run));
        l_run += p[i];
      }
      if constexpr (BF) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x8 pb;
#pragma unroll
          for (int i = 0; i < 8; ++i) pb[i] = (bf16)p[8 * j + i];
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) O[cb] = mfma(vm[kb][2 * cb + j], pb, O[cb]);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4 v = vm[kb][4 * cb + g4];
            O[cb] = mfma(v.x, p[4 * g4], O[cb]);
            O[cb] = mfma(v.y, p[4 * g4 + 1], O[cb]);
            O[cb] = mfma(v.z, p[4 * g4 + 2], O[cb]);
            O[cb] = mfma(v.w, p[4 * g4 + 3], O[cb]);
          }
      }
    }
  };

  // Wave w takes key tiles w, w + NW, ...  PT of them are in flight: slot j
  // of round r holds the wave's tile PT r + j.  Rounds whose refills are all
  // needed run unconditionally (so every path keeps the same loads in
  // flight); the last one or two rounds drain the ring.
  const int ntk = (nk + 32 * KB - 1) / (32 * KB);
  const int mine = ntk > w ? (ntk - w + NW - 1) / NW : 0;
  constexpr int PT = NW >= 8 ? 1 : 2;
  if (mine > 0) {
    KT kr[PT][KB][QS];
    VT vr[PT][KB][NV];
#pragma unroll
    for (int j = 0; j < PT; ++j) load_tile(w + NW * min(j, mine - 1), kr[j], vr[j]);
    int r0 = 0;
    for (; r0 + 2 * PT <= mine; r0 += PT) {
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        process(kr[j], vr[j], w + NW * (r0 + j));
        load_tile(w + NW * (r0 + j + PT), kr[j], vr[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      if (r0 + j < mine) process(kr[j], vr[j], w + NW * (r0 + j));
      if (r0 + j + PT < mine) load_tile(w + NW * (r0 + j + PT), kr[j], vr[j]);
    }
#pragma unroll
    for (int j = 0; j < PT; ++j)
      if (r0 + PT + j < mine) process(kr[j], vr[j], w + NW * (r0 + PT + j));
  }

  l_run = half_swap_sum(l_run);
  if (hi == 0) {
    sm_m[w][lq] = m_run;
    sm_l[w][lq] = l_run;
  }
  // output row rho of channel block cb is channel 32 cb + rho of the head
  // (bf16 with DH < 32: the V block's 32 features start at a multiple of 32,
  // so head h's channels are rows (h DH) % 32 ..)
  const int row_off = (BF && DH < 32) ? (h * DH) % 32 : 0;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = cb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3) - row_off;
      if (c >= 0 && c < DH) sm_o[w][c][lq] = O[cb][i];
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
// all keys.  64-key tiles of K and V are staged through LDS as their
// swizzled 1 KB blocks (contiguous 16-byte loads; double buffered: the next
// tile is in flight while the current one is consumed) and shared by the
// four waves, which read their MFMA operands as one 16-byte LDS load each.
template <int DH>
__global__ __launch_bounds__(256, 4) void k_attention_wide(AttnArgs a, SegTable seg) {
  if (a.stop && *a.stop) return;  // a later layer of a pass that has already stopped
  constexpr int BQ = 128, BKEY = 64;
  constexpr int KBLK = DH / 16, VBLK = DH / 16;  // 512-element blocks per 32 keys (K: dim chunks; V: 2 j x DH/32)
  constexpr int TILE = (BKEY / 32) * (KBLK + VBLK) * 512;  // elements of one staged tile
  constexpr int KCH = TILE / 8 / 256;                      // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) bf16 Ts[2][TILE];

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
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), hi = lane >> 5, lq = lane & 31;
  const int D = a.D, ldq = a.ldqk;
  const bf16* __restrict__ qk = reinterpret_cast<const bf16*>(a.qk);
  const bf16* __restrict__ ks = reinterpret_cast<const bf16*>(a.ks);
  const bf16* __restrict__ vs = reinterpret_cast<const bf16*>(a.vs);

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

  // Staged tile layout: for each 32-key block kb, the head's KBLK K blocks,
  // then its VBLK V blocks (2 cb + j), 512 elements each.  Chunk c of the
  // tile is element 8 c; a 32-key block past the image's last one re-reads
  // that block (its keys are masked).
  const int nkb = (nk + 31) >> 5;
  // Tiles go from global memory straight into LDS (global_load_lds: lane
  // l of a wave writes 16 bytes at the wave's LDS base + 16 l), so no
  // registers hold the tile in flight; chunk c = tid + 256 i lands at
  // element 8 c of the buffer.
  auto chunk_src = [&](int k0, int i) -> const bf16* {
    const int c = tid + 256 * i;
    const int kb = c / ((KBLK + VBLK) * 64), r = c % ((KBLK + VBLK) * 64);
    const size_t tile = (size_t)((krow0 + 32 * min(k0 / 32 + kb, nkb - 1)) >> 5);
    return r < KBLK * 64 ? ks + (tile * (D / 16) + h * (DH / 16)) * 512 + 8 * r
                         : vs + (tile * (D / 32) + (h * DH) / 32) * 1024 + 8 * (r - KBLK * 64);
  };
  // a tile wholly inside the image starts 64 D elements (two 32-key blocks of
  // K and of V) after the previous one: its chunk addresses are those of the
  // first tile plus that step; only the partial tile needs the clamped form
  const bf16* src0[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) src0[i] = chunk_src(0, i);
  auto gload = [&](int k0, int buf) {
    if (k0 + BKEY <= nk) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) lds_dma16(src0[i] + (size_t)k0 * D, &Ts[buf][8 * (64 * w + 256 * i)]);
    } else {
#pragma unroll
      for (int i = 0; i < KCH; ++i) lds_dma16(chunk_src(k0, i), &Ts[buf][8 * (64 * w + 256 * i)]);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 O[DH / 32];
#pragma unroll
  for (int c = 0; c < DH / 32; ++c) O[c] = zero16();

  const int ntk = (nk + BKEY - 1) / BKEY;
  gload(0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // the tile is in LDS
  __syncthreads();
  // Both 32-key blocks of a tile are taken together: two independent QK^T
  // chains, one maximum, one rescale of O and 32 exponentials per lane.  The
  // tiles that lie wholly inside the image run without any masking code; the
  // last, partial tile (TAIL) masks keys past the image.
  static_assert(BKEY == 64, "two 32-key blocks per tile");
  auto step = [&](int kt, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    const int cur = kt & 1;
    if (kt + 1 < ntk) gload((kt + 1) * BKEY, cur ^ 1);  // (buffer cur ^ 1 was released by the last barrier)
    const int k0 = kt * BKEY;
    const bf16* tb0 = &Ts[cur][lane * 8];
    const bf16* tb1 = tb0 + (KBLK + VBLK) * 512;
    f32x16 S0 = zero16(), S1 = zero16();
#pragma unroll
    for (int i = 0; i < DH / 16; ++i) {
      S0 = mfma(*reinterpret_cast<const bf16x8*>(tb0 + i * 512), Qr[i], S0);
      S1 = mfma(*reinterpret_cast<const bf16x8*>(tb1 + i * 512), Qr[i], S1);
    }
    if constexpr (TAIL) {  // keys past the image (a block past it re-read the last block)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = k0 + 8 * (i >> 2) + 4 * hi + (i & 3);
        if (kk >= nk) S0[i] = -INFINITY;
        if (kk + 32 >= nk) S1[i] = -INFINITY;
      }
    }
    // the maximum is taken over the raw scores (the scale is positive) with
    // the three-operand maximum, which takes the accumulators as they are
    // (the scores are never NaN), and the scale folded into the exponent's FMA
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = __builtin_elementwise_maximum(tmax, __builtin_elementwise_maximum(S0[i], S1[i]));
    tmax = half_swap_max(tmax);
    const float m_new = fmaxf(m_run, tmax * a.scale2);
    const float corr = exp2_fast(m_run - m_new);
    float psum = 0.f;
    // P in bf16, packed two keys per 32-bit word by the converter itself
    bf16x8 pb[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 u;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = 8 * j + 2 * x;
          const float p0 = exp2_fast(fmaf(b ? S1[i] : S0[i], a.scale2, -m_new));
          const float p1 = exp2_fast(fmaf(b ? S1[i + 1] : S0[i + 1], a.scale2, -m_new));
          psum += p0;
          psum += p1;
          const bf16x2 pp = {(bf16)p0, (bf16)p1};
          u[x] = __builtin_bit_cast(uint32_t, pp);
        }
        pb[b][j] = __builtin_bit_cast(bf16x8, u);
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
    for (int b = 0; b < 2; ++b) {
      const int kb0 = k0 + 32 * b;
      if (TAIL && kb0 >= nk) break;
      const bf16* tb = b ? tb1 : tb0;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int cb = 0; cb < DH / 32; ++cb) {
          bf16x8 va = *reinterpret_cast<const bf16x8*>(tb + (KBLK + 2 * cb + j) * 512);
          if constexpr (TAIL) {
            // values of keys past the image are zeroed (their P is 0, but
            // padding rows may hold anything a caller staged there)
            if (kb0 + 32 > nk) {
#pragma unroll
              for (int x = 0; x < 8; ++x)
                if (kb0 + 16 * j + 8 * (x >> 2) + 4 * hi + (x & 3) >= nk) va[x] = (bf16)0.f;
            }
          }
          O[cb] = mfma(va, pb[b][j], O[cb]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next tile is in LDS
    __syncthreads();
  };
  const int ntf = nk / BKEY;  // tiles wholly inside the image
  for (int kt = 0; kt < ntf; ++kt) step(kt, std::false_type{});
  if (ntf < ntk) step(ntf, std::true_type{});

  l_run = half_swap_sum(l_run);
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

// Base-2 log-sum-exp of every row of a row-major [rows][ld] fp32 matrix over
// its first `cols` entries, one wave per row (the normalisers of the shared
// similarity's two directions: rows of S for image A, rows of S^T for B).
__global__ __launch_bounds__(256) void k_rows_lse(const float* __restrict__ S, int ld, int rows, int cols,
                                                  float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave_id();
  if (r >= rows) return;
  const float* row = S + (size_t)r * ld;
  float mx = -INFINITY;
  for (int j = lane; j < cols; j += 64) mx = fmaxf(mx, row[j]);
  mx = wave_max(mx);
  float sum = 0.f;
  for (int j = lane; j < cols; j += 64) sum += exp2_fast(row[j] - mx);
  sum = wave_sum(sum);
  if (lane == 0) out[r] = mx + log2_fast(sum);
}

hipError_t launch_rows_lse(const float* S, int ld, int rows, int cols, float* out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (cols <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rows_lse, dim3((rows + 3) / 4), dim3(256), 0, st, S, ld, rows, cols, out);
  return hipGetLastError();
}

// The messages of a bidirectional cross stage of one pair from its shared
// similarity (a.sm, a.lse; see AttnArgs): both images' queries in one launch.
hipError_t launch_attention_shared(int op, int dh, const AttnArgs& a, const SegTable& seg, int heads,
                                   hipStream_t st) {
  if (seg.n_seg != 2 || !a.cross || !a.sm || !a.lse) return hipErrorInvalidValue;
  const int tiles = (seg.n[0] + 31) / 32 + (seg.n[1] + 31) / 32;
  if (tiles == 0 || seg.n[0] == 0 || seg.n[1] == 0) return hipSuccess;
  constexpr int NW = 8;
  dim3 grid(tiles * heads);
#define SG_ATT(T, DHV) hipLaunchKernelGGL((k_attention<T, DHV, NW, true, true>), grid, dim3(64 * NW), 0, st, a, seg)
  if (op == SG_BF16) {
    if (dh == 64) SG_ATT(bf16, 64);
    else if (dh == 16) SG_ATT(bf16, 16);
    else return hipErrorInvalidValue;
  } else {
    if (dh == 64) SG_ATT(float, 64);
    else if (dh == 16) SG_ATT(float, 16);
    else return hipErrorInvalidValue;
  }
#undef SG_ATT
  return hipGetLastError();
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
  // eight waves (two per SIMD) split the key tiles
  constexpr int NW = 8;
  dim3 grid(tiles * heads);
  const bool one = seg.n_seg == 2;  // a single pair
#define SG_ATT(T, DHV)                                                                            \
  if (one) hipLaunchKernelGGL((k_attention<T, DHV, NW, true>), grid, dim3(64 * NW), 0, st, a, seg); \
  else hipLaunchKernelGGL((k_attention<T, DHV, NW, false>), grid, dim3(64 * NW), 0, st, a, seg)
  if (op == SG_BF16) {
    if (dh == 64) SG_ATT(bf16, 64);
    else if (dh == 16) SG_ATT(bf16, 16);
    else return hipErrorInvalidValue;
  } else {
    if (dh == 64) SG_ATT(float, 64);
    else if (dh == 16) SG_ATT(float, 16);
    else return hipErrorInvalidValue;
  }
#undef SG_ATT
  return hipGetLastError();
}

}  // namespace sg
