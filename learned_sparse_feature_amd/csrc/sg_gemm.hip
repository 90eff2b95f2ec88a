// Per-point linear layers of the matching network as MFMA GEMMs (gfx950).
//
// C = A W^T (+ epilogue) with A [rows][K] (optionally two sources split at
// column K0: the [x || m] concatenation of the update MLP) and W [n][K] the
// row-major weight of a kernel-1 Conv1d / Linear layer.  A 256-thread
// workgroup computes a BM x BN output tile as 2 x 2 waves; each wave owns
// (BM/2) x (BN/2) as 32x32 MFMA blocks.  A and W tiles are converted to the
// operand type (bf16 or fp32) on their way into LDS (double buffered).
//
// Two shapes are instantiated:
//  * 64 x 64 tiles with up to 8 K steps in flight (PF = 8) for small
//    problems: a single pair has too few tiles to fill the chip, and the
//    kernel is bound by the latency of its loads, so the whole K range is
//    requested before the first MFMA;
//  * 128 x 128 tiles with one K step in flight (PF = 2) for large problems
//    (batches): each 64x64 wave tile reuses every LDS fragment twice, and
//    several resident workgroups per CU hide the load latency.
// Tile order is XCD-aware: the dispatcher sends workgroup i to XCD i % 8, so
// workgroup i takes tile (i % 8) * ceil(T / 8) + i / 8 of the row-major tile
// sequence (column tiles innermost).  Each XCD then walks a contiguous run of
// tiles, the column tiles of one row tile run together on one XCD, and each
// A row tile is fetched into that XCD's L2 once instead of once per column
// tile.
#include <algorithm>

#include "sg_device.h"
#include "sg_fold.h"

namespace sg {

namespace {

template <typename OpT, int CH>
struct Chunk {
  typedef OpT type __attribute__((ext_vector_type(CH)));
};

// Load CH consecutive elements of SrcT and convert them to OpT.
template <typename SrcT, typename OpT, int CH>
__device__ __forceinline__ typename Chunk<OpT, CH>::type load_chunk(const SrcT* p) {
  typename Chunk<OpT, CH>::type v;
  if constexpr (std::is_same<SrcT, float>::value) {
#pragma unroll
    for (int i = 0; i < CH; i += 4) {
      const float4 f = *reinterpret_cast<const float4*>(p + i);
      v[i] = (OpT)f.x; v[i + 1] = (OpT)f.y; v[i + 2] = (OpT)f.z; v[i + 3] = (OpT)f.w;
    }
  } else if constexpr (CH == 8) {
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (OpT)(float)b[i];
  } else {
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (OpT)(float)b[i];
  }
  return v;
}

// Stores one 32 x 32 accumulator block (value(e) for accumulator e of this
// lane: row 8 (e / 4) + 4 (lane / 32) + e % 4, column lane % 32) as bf16
// into row-major dst (row stride ld) at rows r0.., columns c0.. through the
// wave-private LDS tile tt [32][40]: two 16-byte stores along rows per lane
// instead of sixteen 2-byte ones.  Rows at or past `rows` are not stored.
// Wave-level only: LDS operations of a wave complete in order.
template <class F>
__device__ __forceinline__ void store_block_bf16(bf16* tt, int lane, F value, bf16* dst, size_t ld, int r0, int c0,
                                                 int rows) {
  const int nl = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int e = 0; e < 16; ++e) tt[(8 * (e >> 2) + 4 * hi + (e & 3)) * 40 + nl] = (bf16)value(e);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int c = lane + 64 * x, row = c >> 2, part = c & 3;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(tt + row * 40 + 8 * part);
    if (r0 + row < rows) *reinterpret_cast<bf16x8*>(dst + (size_t)(r0 + row) * ld + c0 + 8 * part) = v;
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace

// Dynamic LDS of the DMA variant (below).
extern __shared__ __attribute__((aligned(16))) unsigned char g_gemm_dyn_lds[];

// ONE: a single problem, whose descriptor then sits at fixed argument
// offsets (no indexed lookup ahead of the first load).
// DMA (bf16 operands, 64 x 64 tiles, K and K0 multiples of 64): every K step
// of the tile is requested at once straight into LDS (global_load_lds, one
// 16-byte slot per lane), nk x 16 KB of dynamic LDS, then one barrier and
// the whole MFMA chain.  Slot s of a step's operand holds row s / 8 and
// 16-byte chunk (s % 8) ^ (row % 8) of the step's 64 columns (an XOR swizzle
// instead of row padding, which a per-lane DMA slot cannot skip).  The
// MFMA order along K is that of the staged variant, so results are equal.
// RING (bf16 operands, 128 x 128 tiles, K and K0 multiples of 32): the K
// loop runs in 32-wide steps through a ring of RS 16 KB LDS slots filled
// with global_load_lds RS - 1 steps ahead of the MFMAs; slot s of an operand
// holds row s / 4 and 16-byte chunk (s % 4) ^ ((row / 4) % 4), which keeps
// the operand reads of 16 consecutive rows on distinct banks.  Same MFMA
// order along K.
template <typename OpT, typename A0T, typename WT, typename OutT, int EPI, int BM, int BN, int PF, bool ONE,
          bool DMA = false, bool RING = false>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs g, GemmBatch bt) {
  constexpr bool BF = std::is_same<OpT, bf16>::value;
  constexpr int CH = BF ? 8 : 4;   // elements per 16-byte chunk
  constexpr int KC = 8;            // chunks per tile row and K step
  constexpr int BK = KC * CH;      // 64 bf16 or 32 fp32 per K step
  constexpr int PITCH = BK + CH;   // rows padded by 16 bytes
  constexpr int AC = BM * KC / 256, WC = BN * KC / 256;  // chunks per thread per K step
  constexpr int MB = BM / 64, NB = BN / 64;            // 32x32 blocks per wave
  typedef typename Chunk<OpT, CH>::type VecT;
  static_assert(!DMA || (std::is_same<OpT, bf16>::value && std::is_same<A0T, bf16>::value &&
                          std::is_same<WT, bf16>::value && BM == 64 && BN == 64),
                "the DMA variant takes bf16 operands and 64 x 64 tiles");
  static_assert(!RING || (std::is_same<OpT, bf16>::value && std::is_same<A0T, bf16>::value &&
                           std::is_same<WT, bf16>::value && BM == 128 && BN == 128 && !DMA),
                "the ring variant takes bf16 operands and 128 x 128 tiles");
  constexpr bool STAGED = !DMA && !RING;
  // ring slots: three of 16 KB (48 KB of LDS, three workgroups per CU)
  constexpr int RS = 3, RSLOT = 2 * 128 * 32;  // elements per slot: A rows, then W rows
  __shared__ __attribute__((aligned(16))) OpT As[STAGED ? 2 : 1][STAGED ? BM * PITCH : 8];
  __shared__ __attribute__((aligned(16))) OpT Ws[STAGED ? 2 : 1][STAGED ? BN * PITCH : 8];
  __shared__ __attribute__((aligned(16))) bf16 Ring[RING ? RS * RSLOT : 8];
  // LDS scratch of the epilogues (32 x 40 elements per wave at most)
  OpT* const scratch = DMA ? reinterpret_cast<OpT*>(g_gemm_dyn_lds) : RING ? reinterpret_cast<OpT*>(Ring) : &As[0][0];

  if constexpr (ONE)
    args_in_sgprs(g.A0, g.A1, g.W, g.lda0, g.lda1, g.ldw, g.K0, g.K, g.gx, g.gy, g.stop, bt.p[0].a_row0,
                  bt.p[0].w_row0, bt.p[0].rows, bt.p[0].n_out);
  if (g.stop && *g.stop) return;  // a later layer of a pass that has already stopped
  const int T = g.gx * g.gy * (ONE ? 1 : bt.n);
  const int t = (int)(blockIdx.x % 8) * ((T + 7) / 8) + (int)(blockIdx.x / 8);
  if (t >= T) return;
  const int ty = t % g.gy, tx = (t / g.gy) % g.gx, tz = ONE ? 0 : t / (g.gy * g.gx);
  const GemmProblem P = bt.p[tz];
  const int r0 = tx * BM, n0 = ty * BN;
  if (r0 >= P.rows || n0 >= P.n_out) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;

  // chunk c = tid + 256 h of a tile covers row c / KC, columns (c % KC) * CH;
  // register slot q holds K step kb + q of the current round
  VecT ra[PF][AC], rw[PF][WC];
  auto gload = [&](int k0, int q) {
#pragma unroll
    for (int h = 0; h < AC; ++h) {
      const int c = tid + 256 * h, row = c / KC, k = k0 + (c % KC) * CH;
      const int r = r0 + row;
      if (r < P.rows && k < g.K) {
        if (k < g.K0)
          ra[q][h] = load_chunk<A0T, OpT, CH>(reinterpret_cast<const A0T*>(g.A0) + (size_t)(P.a_row0 + r) * g.lda0 + k);
        else
          ra[q][h] = load_chunk<OpT, OpT, CH>(reinterpret_cast<const OpT*>(g.A1) + (size_t)(P.a_row0 + r) * g.lda1 + (k - g.K0));
      } else {
        ra[q][h] = (VecT)(OpT)0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < WC; ++h) {
      const int c = tid + 256 * h, row = c / KC, k = k0 + (c % KC) * CH;
      const int n = n0 + row;
      if (n < P.n_out && k < g.K)
        rw[q][h] = load_chunk<WT, OpT, CH>(reinterpret_cast<const WT*>(g.W) + (size_t)(P.w_row0 + n) * g.ldw + k);
      else
        rw[q][h] = (VecT)(OpT)0.f;
    }
  };
  auto sstore = [&](int buf, int q) {
#pragma unroll
    for (int h = 0; h < AC; ++h) {
      const int c = tid + 256 * h;
      *reinterpret_cast<VecT*>(&As[buf][(c / KC) * PITCH + (c % KC) * CH]) = ra[q][h];
    }
#pragma unroll
    for (int h = 0; h < WC; ++h) {
      const int c = tid + 256 * h;
      *reinterpret_cast<VecT*>(&Ws[buf][(c / KC) * PITCH + (c % KC) * CH]) = rw[q][h];
    }
  };
  f32x16 acc[MB][NB];
  auto compute = [&](int cur) {
    const OpT* ap = &As[cur][(wm * (BM / 2) + (lane & 31)) * PITCH];
    const OpT* wp = &Ws[cur][(wn * (BN / 2) + (lane & 31)) * PITCH];
    if constexpr (BF) {
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        bf16x8 a[MB], b[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) a[i] = *reinterpret_cast<const bf16x8*>(ap + i * 32 * PITCH + s * 16 + (lane >> 5) * 8);
#pragma unroll
        for (int j = 0; j < NB; ++j) b[j] = *reinterpret_cast<const bf16x8*>(wp + j * 32 * PITCH + s * 16 + (lane >> 5) * 8);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma(a[i], b[j], acc[i][j]);
      }
    } else {
      // k-slot l/32 of the MFMAs covers tile columns 16*(l/32) .. +15
#pragma unroll
      for (int s4 = 0; s4 < BK / 8; ++s4) {
        float4 a[MB], b[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) a[i] = *reinterpret_cast<const float4*>(ap + i * 32 * PITCH + (lane >> 5) * (BK / 2) + 4 * s4);
#pragma unroll
        for (int j = 0; j < NB; ++j) b[j] = *reinterpret_cast<const float4*>(wp + j * 32 * PITCH + (lane >> 5) * (BK / 2) + 4 * s4);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            acc[i][j] = mfma(a[i].x, b[j].x, acc[i][j]);
            acc[i][j] = mfma(a[i].y, b[j].y, acc[i][j]);
            acc[i][j] = mfma(a[i].z, b[j].z, acc[i][j]);
            acc[i][j] = mfma(a[i].w, b[j].w, acc[i][j]);
          }
      }
    }
  };

#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = zero16();
  // The residual tile is requested all at once, not one element after
  // another behind the epilogue's stores (which the compiler may not move
  // the loads past): before the main loop for the small tiles, where its
  // latency then overlaps the K loop, and after it for the large ones, whose
  // main loop has no registers to spare.
  // It is read in the row-major form the epilogue writes: chunk x of a
  // 32 x 32 block is row (lane + 64 x) / 8, columns 4 ((lane + 64 x) % 8) ..
  // +3, one 16-byte load.
  constexpr int RM = EPI == EPI_RESID ? MB : 1, RN = EPI == EPI_RESID ? NB : 1;
  float4 cres[RM][RN][4];
  auto load_resid = [&]() {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int c = lane + 64 * x;
          const int r = r0 + wm * (BM / 2) + i * 32 + (c >> 3), n = n0 + wn * (BN / 2) + j * 32 + 4 * (c & 7);
          cres[i][j][x] = (r < P.rows && n < P.n_out)
                              ? *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(g.C) + P.c_off +
                                                                 (size_t)r * P.ldc + n)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        }
  };
  if constexpr (EPI == EPI_RESID && PF > 2) load_resid();
  const int nk = (g.K + BK - 1) / BK;
  if constexpr (DMA) {
    bf16* const LA = reinterpret_cast<bf16*>(g_gemm_dyn_lds);  // [nk][64 x 64]
    bf16* const LW = LA + (size_t)nk * 4096;                    // [nk][64 x 64]
    const bf16* const A0 = reinterpret_cast<const bf16*>(g.A0);
    const bf16* const A1 = reinterpret_cast<const bf16*>(g.A1);
    const bf16* const Wp = reinterpret_cast<const bf16*>(g.W);
    for (int q = 0; q < nk; ++q) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // instruction h of wave w fills slots 64 (2 w + h) .. +63 of both operands
        const int sb = 64 * (2 * wave + h), sl = sb + lane, row = sl >> 3, kc = (sl & 7) ^ (row & 7);
        const int k = q * 64 + 8 * kc;
        const int ra = P.a_row0 + min(r0 + row, P.rows - 1);   // rows past the end: any valid row (never stored)
        const int rw = P.w_row0 + min(n0 + row, P.n_out - 1);
        const bf16* srcA = k < g.K0 ? A0 + (size_t)ra * g.lda0 + k : A1 + (size_t)ra * g.lda1 + (k - g.K0);
        lds_dma16(srcA, LA + (size_t)q * 4096 + 8 * sb);
        lds_dma16(Wp + (size_t)rw * g.ldw + k, LW + (size_t)q * 4096 + 8 * sb);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // every step is in LDS
    __syncthreads();
    const int ar = wm * 32 + (lane & 31), wr = wn * 32 + (lane & 31);
    for (int q = 0; q < nk; ++q) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kc = 2 * st + (lane >> 5);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(LA + (size_t)q * 4096 + ar * 64 + 8 * (kc ^ (ar & 7)));
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(LW + (size_t)q * 4096 + wr * 64 + 8 * (kc ^ (wr & 7)));
        acc[0][0] = mfma(a, b, acc[0][0]);
      }
    }
  } else if constexpr (RING) {
    const bf16* const A0 = reinterpret_cast<const bf16*>(g.A0);
    const bf16* const A1 = reinterpret_cast<const bf16*>(g.A1);
    const bf16* const Wp = reinterpret_cast<const bf16*>(g.W);
    const int ns = g.K / 32;
    // step q into slot q % RS: instruction h of wave w fills slots
    // 256 h + 64 w .. +63 of both operands
    auto issue = [&](int q) {
      bf16* const base = Ring + (q % RS) * RSLOT;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sb = 256 * h + 64 * wave, sl = sb + lane, row = sl >> 2, kc = (sl & 3) ^ ((row >> 2) & 3);
        const int k = 32 * q + 8 * kc;
        const int ra = P.a_row0 + min(r0 + row, P.rows - 1);  // rows past the end: any valid row (never stored)
        const int rw = P.w_row0 + min(n0 + row, P.n_out - 1);
        const bf16* srcA = k < g.K0 ? A0 + (size_t)ra * g.lda0 + k : A1 + (size_t)ra * g.lda1 + (k - g.K0);
        lds_dma16(srcA, base + 8 * sb);
        lds_dma16(Wp + (size_t)rw * g.ldw + k, base + 128 * 32 + 8 * sb);
      }
    };
    for (int q = 0; q < RS - 1 && q < ns; ++q) issue(q);
    for (int q = 0; q < ns; ++q) {
      // step q has landed once at most the later steps' 4 instructions each are pending
      const int later = min(ns - 1, q + RS - 2) - q;
      if (later >= 2) wait_vm<8>();
      else if (later == 1) wait_vm<4>();
      else wait_vm<0>();
      // ... in every lane; and every wave is done with step q - 1's slot
      // (__syncthreads() would also wait for the steps still in flight)
      bare_barrier();
      if (q + RS - 1 < ns) issue(q + RS - 1);
      const bf16* const base = Ring + (q % RS) * RSLOT;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int kc = 2 * st + (lane >> 5);
        bf16x8 a[MB], b[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int ar = wm * (BM / 2) + i * 32 + (lane & 31);
          a[i] = *reinterpret_cast<const bf16x8*>(base + ar * 32 + 8 * (kc ^ ((ar >> 2) & 3)));
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int wr = wn * (BN / 2) + j * 32 + (lane & 31);
          b[j] = *reinterpret_cast<const bf16x8*>(base + 128 * 32 + wr * 32 + 8 * (kc ^ ((wr >> 2) & 3)));
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma(a[i], b[j], acc[i][j]);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < PF; ++q)
      if (q < nk) gload(q * BK, q);
    for (int kb = 0; kb < nk; kb += PF) {
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        const int kt = kb + q;
        if (kt >= nk) break;
        const int cur = kt & 1;
        sstore(cur, q);
        __syncthreads();
        if (kt + PF < nk) gload((kt + PF) * BK, q);
        compute(cur);
      }
    }
  }

  if constexpr (EPI == EPI_RESID && PF <= 2) load_resid();
  if constexpr (EPI == EPI_QKV) {
    // The bias is added to the accumulators here, once.  Self stages with a
    // rotary table then rotate every channel pair (2c, 2c+1) of q and k
    // (columns [0, 2D)) by the row's angle c mod d_h / 2: the pair's other
    // column sits in the neighbouring lane (same row), one DPP swap away.
    const int Dq = g.tied ? g.split : g.split / 2;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int rr0 = r0 + wm * (BM / 2) + i * 32, nn0 = n0 + wn * (BN / 2) + j * 32;
        if (rr0 >= P.rows || nn0 >= P.n_out) continue;
        const int n = nn0 + (lane & 31);
        const float bias = g.bias ? (float)reinterpret_cast<const WT*>(g.bias)[n] : 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] += bias;
        if (g.rope && nn0 < 2 * Dq) {
          const int hp = g.rope_dh / 2, kc = (n % g.rope_dh) >> 1;
          const float sg = (n & 1) ? 1.f : -1.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = rr0 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const float2 cs = g.rope[(size_t)r * hp + kc];
            const float other = dpp_f<kDppXor1>(acc[i][j][e]);
            acc[i][j][e] = fmaf(sg * other, cs.y, acc[i][j][e] * cs.x);
          }
        }
      }
  }

  if constexpr (EPI == EPI_QKV && BF) {
    // bf16 q | k | v, per 32x32 block: q row-major into C; k through a
    // wave-private LDS transposition into the tile-swizzled C3; v straight
    // from the accumulators into the tile-swizzled C2 (its layout is the
    // accumulator layout).  Column ranges: q [0, D), k [D, 2D), v [2D, 3D)
    // with D = split / 2; tied (one shared query/key projection): qk [0, D)
    // written as both q and k, v [D, 2D) with D = split.  The QKV GEMM covers
    // the whole row space, so the problem's rows are the compact rows (32-row
    // tiles stay aligned).
    const int Dm = g.tied ? g.split : g.split / 2;
    constexpr int TP = 32 + 8;
    bf16* tt = reinterpret_cast<bf16*>(scratch) + wave * 32 * TP;
    bf16* const cq = reinterpret_cast<bf16*>(g.C);
    bf16* const cv = reinterpret_cast<bf16*>(g.C2);
    bf16* const ck = reinterpret_cast<bf16*>(g.C3);
    const int nl = lane & 31;
    __syncthreads();  // every wave is done with the A tiles: As is scratch now
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int rr0 = r0 + wm * (BM / 2) + i * 32, nn0 = n0 + wn * (BN / 2) + j * 32;
        if (rr0 >= P.rows || nn0 >= P.n_out) continue;
        const float bias = 0.f;  // added to the accumulators above
        const int tile = rr0 >> 5;
        if (nn0 < Dm)
          store_block_bf16(tt, lane, [&](int e) { return acc[i][j][e] + bias; }, cq + P.c_off, P.ldc, rr0, nn0,
                           P.rows);
        if (nn0 < g.split && (g.tied || nn0 >= Dm)) {
          const int kc = g.tied ? nn0 : nn0 - Dm;  // column of k
          // the block row-major in LDS (row = key, 32 columns = dims) ...
#pragma unroll
          for (int e = 0; e < 16; ++e)
            tt[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * TP + nl] = (bf16)(acc[i][j][e] + bias);
          __builtin_amdgcn_wave_barrier();
          // ... so that chunk c (16-dim half `which` of the block's 32
          // columns, lane slot L: key L % 32, dims 16 which + 8 (L / 32) ..
          // +7) is one 16-byte LDS read
#pragma unroll
          for (int c = lane; c < 128; c += 64) {
            const int L = c & 63, which = c >> 6;
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(tt + (L & 31) * TP + 16 * which + 8 * (L >> 5));
            const size_t blk = (size_t)tile * (Dm / 16) + kc / 16 + which;
            *reinterpret_cast<bf16x8*>(ck + blk * 512 + L * 8) = v;
          }
          __builtin_amdgcn_wave_barrier();
        } else if (nn0 >= g.split) {
          bf16* base = cv + ((size_t)tile * (Dm / 32) + (nn0 - g.split) / 32) * 1024 + lane * 8;
          bf16x8 lo, hi8;
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            lo[x] = (bf16)(acc[i][j][x] + bias);
            hi8[x] = (bf16)(acc[i][j][8 + x] + bias);
          }
          *reinterpret_cast<bf16x8*>(base) = lo;
          *reinterpret_cast<bf16x8*>(base + 512) = hi8;
        }
      }
    return;
  }
  if constexpr (EPI == EPI_QKV) {
    if (n0 >= g.split) {
      // V columns: written transposed (VT [n - split][r]).  Each 32x32 block
      // is turned around in LDS so that the stores run along rows of VT.
      constexpr int TP = 32 + 16 / (int)sizeof(OutT);
      OutT* tt = reinterpret_cast<OutT*>(scratch) + wave * 32 * TP;
      constexpr int CO = 16 / (int)sizeof(OutT);  // elements per 16-byte store
      typedef typename Chunk<OutT, CO>::type OVec;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int nl = lane & 31;
          const float bias = 0.f;  // added to the accumulators above
          __syncthreads();
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int rl = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            tt[nl * TP + rl] = (OutT)(acc[i][j][e] + bias);
          }
          __syncthreads();
          for (int c = lane; c < 32 * (32 / CO); c += 64) {
            const int nlc = c / (32 / CO), part = c % (32 / CO);
            const int n = n0 + wn * (BN / 2) + j * 32 + nlc;
            const int r = r0 + wm * (BM / 2) + i * 32 + part * CO;
            if (n < P.n_out && r < P.rows) {
              OVec v;
#pragma unroll
              for (int x = 0; x < CO; ++x) v[x] = tt[nlc * TP + part * CO + x];
              *reinterpret_cast<OVec*>(reinterpret_cast<OutT*>(g.C2) + P.ct_off + (size_t)(n - g.split) * P.ldct + r) = v;
            }
          }
        }
      return;
    }
  }

  if constexpr (EPI == EPI_RESID) {
    // x = x + (acc + bias) and its bf16 copy: each 32 x 32 block of acc + bias
    // goes through a wave-private fp32 LDS tile (32 rows, pitch 36), so that
    // the residual read and both writes run along rows, 16 (8) bytes per lane
    constexpr int TP = 36;
    float* tt = reinterpret_cast<float*>(scratch) + wave * 32 * TP;
    __syncthreads();  // every wave is done with the operand tiles: their LDS is scratch now
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int rr0 = r0 + wm * (BM / 2) + i * 32, nn0 = n0 + wn * (BN / 2) + j * 32;
        if (rr0 >= P.rows || nn0 >= P.n_out) continue;
        const float bias = g.bias ? (float)reinterpret_cast<const WT*>(g.bias)[nn0 + (lane & 31)] : 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) tt[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * TP + (lane & 31)] = acc[i][j][e] + bias;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int c = lane + 64 * x, row = c >> 3, part = c & 7;
          const int r = rr0 + row, n = nn0 + 4 * part;
          if (r < P.rows && n < P.n_out) {
            const float4 v = *reinterpret_cast<const float4*>(tt + row * TP + 4 * part);
            const float4 res = cres[i][j][x];
            const float4 xo = make_float4(res.x + v.x, res.y + v.y, res.z + v.z, res.w + v.w);
            const size_t off = P.c_off + (size_t)r * P.ldc + n;
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(g.C) + off) = xo;
            if (g.C2) {
              bf16x4 xb;
              xb[0] = (bf16)xo.x; xb[1] = (bf16)xo.y; xb[2] = (bf16)xo.z; xb[3] = (bf16)xo.w;
              *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(g.C2) + off) = xb;
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    return;
  }

  if constexpr ((EPI == EPI_BIAS || EPI == EPI_RELU) && std::is_same<OutT, bf16>::value) {
    // bf16 outputs: each 32 x 32 block through a wave-private LDS tile
    // (the n_out of these GEMMs are multiples of 32)
    bf16* tt = reinterpret_cast<bf16*>(scratch) + wave * 32 * 40;
    __syncthreads();  // every wave is done with the A tiles: As is scratch now
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int rr0 = r0 + wm * (BM / 2) + i * 32, nn0 = n0 + wn * (BN / 2) + j * 32;
        if (rr0 >= P.rows || nn0 >= P.n_out) continue;
        const float bias = g.bias ? (float)reinterpret_cast<const WT*>(g.bias)[nn0 + (lane & 31)] : 0.f;
        store_block_bf16(tt, lane, [&](int e) {
          const float v = acc[i][j][e] + bias;
          return EPI == EPI_RELU ? fmaxf(v, 0.f) : v;
        }, reinterpret_cast<bf16*>(g.C) + P.c_off, P.ldc, rr0, nn0, P.rows);
      }
    return;
  }
  if constexpr (EPI == EPI_SCORE ||
                ((EPI == EPI_BIAS || EPI == EPI_RELU || EPI == EPI_QKV) && std::is_same<OutT, float>::value)) {
    // fp32 outputs: each 32 x 32 block through a wave-private LDS tile
    // (pitch 36), stored as 16-byte row runs; the scores' transposed copy
    // as 16-byte runs along the rows of the transpose.  (QKV: the q | k
    // columns of an fp32 network, bias already in the accumulators; a tied
    // projection writes them as k too, at + split.)
    constexpr int TP = 36;
    float* tt = reinterpret_cast<float*>(scratch) + wave * 32 * TP;
    __syncthreads();  // every wave is done with the operand tiles: their LDS is scratch now
    const int nl = lane & 31;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int rr0 = r0 + wm * (BM / 2) + i * 32, nn0 = n0 + wn * (BN / 2) + j * 32;
        if (rr0 >= P.rows || nn0 >= P.n_out) continue;
        float bias = 0.f;
        if (EPI != EPI_SCORE && EPI != EPI_QKV && g.bias && nn0 + nl < P.n_out)
          bias = (float)reinterpret_cast<const WT*>(g.bias)[nn0 + nl];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float v = EPI == EPI_SCORE ? acc[i][j][e] * g.scale : acc[i][j][e] + bias;
          if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
          tt[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * TP + nl] = v;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int c = lane + 64 * x, row = c >> 3, part = c & 7;
          const int r = rr0 + row, n = nn0 + 4 * part;
          if (r < P.rows && n < P.n_out) {
            const float4 v = *reinterpret_cast<const float4*>(tt + row * TP + 4 * part);
            float* dst = reinterpret_cast<float*>(g.C) + P.c_off + (size_t)r * P.ldc + n;
            if (n + 3 < P.n_out) {
              *reinterpret_cast<float4*>(dst) = v;
              if (EPI == EPI_QKV && g.tied) *reinterpret_cast<float4*>(dst + g.split) = v;
            } else {
              dst[0] = v.x;
              if (n + 1 < P.n_out) dst[1] = v.y;
              if (n + 2 < P.n_out) dst[2] = v.z;
              if (EPI == EPI_QKV && g.tied) {
                dst[g.split] = v.x;
                if (n + 1 < P.n_out) dst[g.split + 1] = v.y;
                if (n + 2 < P.n_out) dst[g.split + 2] = v.z;
              }
            }
          }
        }
        if (EPI == EPI_SCORE && g.C2) {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int c = lane + 64 * x, col = c >> 3, part = c & 7;
            const int n = nn0 + col, r = rr0 + 4 * part;
            if (n < P.n_out && r < P.rows) {
              const float4 v = make_float4(tt[(4 * part) * TP + col], tt[(4 * part + 1) * TP + col],
                                           tt[(4 * part + 2) * TP + col], tt[(4 * part + 3) * TP + col]);
              float* dst = reinterpret_cast<float*>(g.C2) + P.ct_off + (size_t)n * P.ldct + r;
              if (r + 3 < P.rows) {
                *reinterpret_cast<float4*>(dst) = v;
              } else {
                dst[0] = v.x;
                if (r + 1 < P.rows) dst[1] = v.y;
                if (r + 2 < P.rows) dst[2] = v.z;
              }
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
    if (n >= P.n_out) continue;
    float bias = 0.f;
    if (EPI != EPI_SCORE && EPI != EPI_QKV && g.bias) bias = (float)reinterpret_cast<const WT*>(g.bias)[n];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = r0 + wm * (BM / 2) + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (r >= P.rows) continue;
        float v = acc[i][j][e] + bias;
        if constexpr (EPI == EPI_BIAS || EPI == EPI_RELU || EPI == EPI_QKV) {
          if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
          reinterpret_cast<OutT*>(g.C)[P.c_off + (size_t)r * P.ldc + n] = (OutT)v;
          // tied query/key projection: the same column is k as well (k at +split)
          if (EPI == EPI_QKV && g.tied) reinterpret_cast<OutT*>(g.C)[P.c_off + (size_t)r * P.ldc + n + g.split] = (OutT)v;
        } else {  // EPI_SCORE
          v = acc[i][j][e] * g.scale;
          reinterpret_cast<float*>(g.C)[P.c_off + (size_t)r * P.ldc + n] = v;
          if (g.C2) reinterpret_cast<float*>(g.C2)[P.ct_off + (size_t)n * P.ldct + r] = v;
        }
      }
  }
}

__global__ void k_to_bf16(const float* __restrict__ x, bf16* __restrict__ y, int n4) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(x)[t];
  bf16x4 o;
  o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
  reinterpret_cast<bf16x4*>(y)[t] = o;
}

hipError_t launch_to_bf16(const float* x, void* y, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_to_bf16, dim3((n / 4 + 255) / 256), dim3(256), 0, st, x, static_cast<bf16*>(y), n / 4);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(64) void k_fold_merge(FoldArgs f) {
  fold_block<T>(f, blockIdx.x, blockIdx.y, blockIdx.z);
}

hipError_t launch_fold_merge(int w_dtype, const FoldArgs& f, hipStream_t st) {
  if (f.n <= 0) return hipSuccess;
  if (f.n > kMaxFold || f.D % 32) return hipErrorInvalidValue;
  dim3 grid(2 * f.D / 32, f.D / 32 + 1, f.n);
  if (w_dtype == SG_BF16) hipLaunchKernelGGL(k_fold_merge<bf16>, grid, dim3(64), 0, st, f);
  else hipLaunchKernelGGL(k_fold_merge<float>, grid, dim3(64), 0, st, f);
  return hipGetLastError();
}

constexpr int kGemmDmaMaxK = 512;  // 128 KB of LDS: one workgroup per CU

template <typename OpT, typename A0T, typename WT, typename OutT, int EPI>
static void gemm_go(const GemmArgs& g, const GemmBatch& b, int max_rows, int max_n, hipStream_t st) {
  // large problems (several tiles per CU even at 128 x 128): the LDS-efficient shape
  const long big_tiles = (long)((max_rows + 127) / 128) * ((max_n + 127) / 128) * b.n;
  GemmArgs a = g;
  // (a QKV split must fall on a tile edge: 128-wide tiles need it at a multiple of 128)
  constexpr bool DMAOK = std::is_same<OpT, bf16>::value && std::is_same<A0T, bf16>::value &&
                         std::is_same<WT, bf16>::value;
  if (big_tiles >= 1024 && !(EPI == EPI_QKV && g.split % 128)) {
    a.gx = (max_rows + 127) / 128;
    a.gy = (max_n + 127) / 128;
    const int T = a.gx * a.gy * b.n;
    if (DMAOK && b.n == 1 && g.K % 32 == 0 && g.K0 % 32 == 0)
      hipLaunchKernelGGL((k_gemm<OpT, A0T, WT, OutT, EPI, 128, 128, 2, true, false, DMAOK>), dim3(8 * ((T + 7) / 8)),
                         dim3(256), 0, st, a, b);
    else
      hipLaunchKernelGGL((k_gemm<OpT, A0T, WT, OutT, EPI, 128, 128, 2, false>), dim3(8 * ((T + 7) / 8)), dim3(256), 0, st,
                         a, b);
  } else {
    a.gx = (max_rows + 63) / 64;
    a.gy = (max_n + 63) / 64;
    const int T = a.gx * a.gy * b.n;
    if (DMAOK && b.n == 1 && g.K % 64 == 0 && g.K0 % 64 == 0 && g.K <= kGemmDmaMaxK) {
      // every K step in LDS: nk x 16 KB (two workgroups per CU up to K = 256)
      // (at least the 18 KB the fp32 epilogues stage through it)
      const unsigned lds = std::max((unsigned)(g.K / 64) * 16384u, 18432u);
      static bool attr = false;  // (per instantiation)
      if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<OpT, A0T, WT, OutT, EPI, 64, 64, 8, true, DMAOK>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kGemmDmaMaxK / 64 * 16384);
        attr = true;
      }
      hipLaunchKernelGGL((k_gemm<OpT, A0T, WT, OutT, EPI, 64, 64, 8, true, DMAOK>), dim3(8 * ((T + 7) / 8)), dim3(256),
                         lds, st, a, b);
    } else if (b.n == 1)
      hipLaunchKernelGGL((k_gemm<OpT, A0T, WT, OutT, EPI, 64, 64, 8, true>), dim3(8 * ((T + 7) / 8)), dim3(256), 0, st, a, b);
    else
      hipLaunchKernelGGL((k_gemm<OpT, A0T, WT, OutT, EPI, 64, 64, 8, false>), dim3(8 * ((T + 7) / 8)), dim3(256), 0, st, a, b);
  }
}

hipError_t launch_gemm(int op, int a0f, int wd, int outf, int epi, const GemmArgs& g,
                       const GemmBatch& b, int max_rows, int max_n, hipStream_t st) {
  if (max_rows <= 0 || max_n <= 0 || b.n <= 0) return hipSuccess;
  if (g.K % 8 || g.K0 % 8) return hipErrorInvalidValue;
  if (epi == EPI_QKV && g.split % 64) return hipErrorInvalidValue;  // V columns start on a tile edge
  // bf16 outputs are stored in 16-byte row runs of whole 32-column blocks
  if (op == SG_BF16 && !outf && epi != EPI_RESID && epi != EPI_SCORE) {
    for (int i = 0; i < b.n; ++i)
      if (b.p[i].n_out % 32 || b.p[i].ldc % 8 || b.p[i].c_off % 8) return hipErrorInvalidValue;
  }
  // the residual epilogue reads and writes 4-column row runs
  if (epi == EPI_RESID) {
    for (int i = 0; i < b.n; ++i)
      if (b.p[i].n_out % 4 || b.p[i].ldc % 4 || b.p[i].c_off % 4) return hipErrorInvalidValue;
  }
  // fp32 outputs (and the scores' transposed copy) are stored in 16-byte runs
  if (epi == EPI_SCORE || (outf && (epi == EPI_BIAS || epi == EPI_RELU || epi == EPI_QKV))) {
    for (int i = 0; i < b.n; ++i) {
      if (b.p[i].ldc % 4 || b.p[i].c_off % 4) return hipErrorInvalidValue;
      if (epi == EPI_SCORE && g.C2 && (b.p[i].ldct % 4 || b.p[i].ct_off % 4)) return hipErrorInvalidValue;
    }
  }
#define SG_GO(O, A, W, OUT, E) gemm_go<O, A, W, OUT, E>(g, b, max_rows, max_n, st)
  // The operand-type / epilogue combinations the pipeline uses.
  if (op == SG_F32) {
    if (wd != SG_F32) return hipErrorInvalidValue;
    switch (epi) {
      case EPI_BIAS: SG_GO(float, float, float, float, EPI_BIAS); break;
      case EPI_RELU: SG_GO(float, float, float, float, EPI_RELU); break;
      case EPI_RESID: SG_GO(float, float, float, float, EPI_RESID); break;
      case EPI_QKV: SG_GO(float, float, float, float, EPI_QKV); break;
      case EPI_SCORE: SG_GO(float, float, float, float, EPI_SCORE); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    if (wd != SG_BF16) return hipErrorInvalidValue;
    if (a0f) {
      switch (epi) {
        case EPI_QKV: SG_GO(bf16, float, bf16, bf16, EPI_QKV); break;
        case EPI_RELU: SG_GO(bf16, float, bf16, bf16, EPI_RELU); break;
        case EPI_BIAS:
          if (outf) SG_GO(bf16, float, bf16, float, EPI_BIAS);
          else SG_GO(bf16, float, bf16, bf16, EPI_BIAS);
          break;
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (epi) {
        case EPI_BIAS: SG_GO(bf16, bf16, bf16, bf16, EPI_BIAS); break;
        case EPI_RESID: SG_GO(bf16, bf16, bf16, float, EPI_RESID); break;
        case EPI_QKV: SG_GO(bf16, bf16, bf16, bf16, EPI_QKV); break;
        case EPI_RELU: SG_GO(bf16, bf16, bf16, bf16, EPI_RELU); break;
        case EPI_SCORE: SG_GO(bf16, bf16, bf16, float, EPI_SCORE); break;  // (a shared similarity)
        default: return hipErrorInvalidValue;
      }
    }
  }
#undef SG_GO
  return hipGetLastError();
}

}  // namespace sg
