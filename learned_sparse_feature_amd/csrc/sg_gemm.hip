// Per-point linear layers of the matching network as MFMA GEMMs (gfx950).
//
// C = A W^T (+ epilogue) with A [rows][K] (optionally two sources split at
// column K0: the [x || m] concatenation of the update MLP) and W [n][K] the
// row-major weight of a kernel-1 Conv1d / Linear layer.  One 256-thread
// workgroup computes a 64x64 output tile as four waves of 32x32.  The K loop
// is double buffered: the next K tile is fetched from global memory into
// registers while the MFMAs consume the current one from LDS, and it is
// converted to the operand type (bf16 or fp32) on its way into LDS.
#include "sg_device.h"

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

}  // namespace

template <typename OpT, typename A0T, typename WT, typename OutT, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g, GemmBatch bt) {
  constexpr bool BF = std::is_same<OpT, bf16>::value;
  constexpr int BM = 64, BN = 64;
  constexpr int CH = BF ? 8 : 4;   // elements per 16-byte chunk
  constexpr int BK = 8 * CH;       // 64 bf16 or 32 fp32 per K step
  constexpr int PITCH = BK + CH;   // rows padded by 16 bytes
  typedef typename Chunk<OpT, CH>::type VecT;
  __shared__ __attribute__((aligned(16))) OpT As[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) OpT Ws[2][BN * PITCH];

  const GemmProblem P = bt.p[blockIdx.z];
  // blockIdx.x walks the row tiles: consecutive workgroups are dispatched to
  // different XCDs, so each XCD's L2 holds only its share of the A rows
  // (while every XCD reads the - smaller - weight tile columns)
  const int r0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  if (r0 >= P.rows || n0 >= P.n_out) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Each thread stages two 16-byte chunks of A and of W per K step:
  // chunk c = tid + 256 h covers row c / 8, columns (c % 8) * CH ...
  // Register slot q holds K step kb + q of the current round.
  constexpr int PF = 8;
  VecT ra[PF][2], rw[PF][2];
  auto gload = [&](int k0, int q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + 256 * h, row = c >> 3, k = k0 + (c & 7) * CH;
      const int r = r0 + row, n = n0 + row;
      if (r < P.rows && k < g.K) {
        if (k < g.K0)
          ra[q][h] = load_chunk<A0T, OpT, CH>(reinterpret_cast<const A0T*>(g.A0) + (size_t)(P.a_row0 + r) * g.lda0 + k);
        else
          ra[q][h] = load_chunk<OpT, OpT, CH>(reinterpret_cast<const OpT*>(g.A1) + (size_t)(P.a_row0 + r) * g.lda1 + (k - g.K0));
      } else {
        ra[q][h] = (VecT)(OpT)0.f;
      }
      if (n < P.n_out && k < g.K)
        rw[q][h] = load_chunk<WT, OpT, CH>(reinterpret_cast<const WT*>(g.W) + (size_t)(P.w_row0 + n) * g.ldw + k);
      else
        rw[q][h] = (VecT)(OpT)0.f;
    }
  };
  auto sstore = [&](int buf, int q) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + 256 * h, row = c >> 3, col = (c & 7) * CH;
      *reinterpret_cast<VecT*>(&As[buf][row * PITCH + col]) = ra[q][h];
      *reinterpret_cast<VecT*>(&Ws[buf][row * PITCH + col]) = rw[q][h];
    }
  };
  f32x16 acc;
  auto compute = [&](int cur) {
    const OpT* ap = &As[cur][(wm * 32 + (lane & 31)) * PITCH];
    const OpT* wp = &Ws[cur][(wn * 32 + (lane & 31)) * PITCH];
    if constexpr (BF) {
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap + s * 16 + (lane >> 5) * 8);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(wp + s * 16 + (lane >> 5) * 8);
        acc = mfma(a, b, acc);
      }
    } else {
      // k-slot l/32 of the 16 MFMAs covers tile columns 16*(l/32) .. +15
#pragma unroll
      for (int s4 = 0; s4 < BK / 8; ++s4) {
        const float4 a = *reinterpret_cast<const float4*>(ap + (lane >> 5) * (BK / 2) + 4 * s4);
        const float4 b = *reinterpret_cast<const float4*>(wp + (lane >> 5) * (BK / 2) + 4 * s4);
        acc = mfma(a.x, b.x, acc);
        acc = mfma(a.y, b.y, acc);
        acc = mfma(a.z, b.z, acc);
        acc = mfma(a.w, b.w, acc);
      }
    }
  };

  acc = zero16();
  const int nk = (g.K + BK - 1) / BK;
  // Up to PF K steps are in flight at once: at these sizes a GEMM is bound by
  // the latency of its global loads, not by the MFMAs, so the whole K range
  // (K <= PF * BK) is requested before the first MFMA.
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

  const int n = n0 + wn * 32 + (lane & 31);
  if (n >= P.n_out) return;
  float bias = 0.f;
  if (EPI != EPI_SCORE && g.bias) bias = (float)reinterpret_cast<const WT*>(g.bias)[n];
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

template <typename OpT, typename A0T, typename WT, typename OutT, int EPI>
static void gemm_go(const GemmArgs& g, const GemmBatch& b, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((k_gemm<OpT, A0T, WT, OutT, EPI>), grid, dim3(256), 0, st, g, b);
}

hipError_t launch_gemm(int op, int a0f, int wd, int outf, int epi, const GemmArgs& g,
                       const GemmBatch& b, int max_rows, int max_n, hipStream_t st) {
  if (max_rows <= 0 || max_n <= 0 || b.n <= 0) return hipSuccess;
  if (g.K % 8 || g.K0 % 8) return hipErrorInvalidValue;
  dim3 grid((max_rows + 63) / 64, (max_n + 63) / 64, b.n);
  // The operand-type / epilogue combinations the pipeline uses.
  if (op == SG_F32) {
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

}  // namespace sg
