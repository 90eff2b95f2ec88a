// Keypoint encoder MLP_enc([x, y, c]) added to the descriptors (gfx950).
//
// One fused kernel: a 512-thread workgroup takes 32 points of one image,
// normalises their positions, runs the whole MLP with the hidden
// activations kept in LDS (layer 0 on the VALU, K = 3; the other layers on
// MFMA in the operand type of the network), and writes x0 = d + MLP_enc(p)
// as fp32 states.  The eight waves (two per SIMD) split each layer's outputs
// into 32-column blocks, so that a 256-wide layer is one block per wave and
// all of its weight loads are in flight together; weights stream from L2.
#include "sg_device.h"
#include "sg_fold.h"

namespace sg {

constexpr int kEncThreads = 512, kEncWaves = kEncThreads / 64;

template <typename OpT>
constexpr int enc_ldh() { return kMaxEncWidth + (std::is_same<OpT, bf16>::value ? 8 : 4); }

// Tile t (32 points) of the encoder; hbuf: the workgroup's two hidden-layer
// buffers [2][32 * enc_ldh].
template <typename OpT, typename WT>
__device__ __forceinline__ void encoder_tile(const EncArgs& e, const SegTable& seg, int t,
                                             OpT (*hbuf)[32 * enc_ldh<OpT>()]) {
  constexpr bool BF = std::is_same<OpT, bf16>::value;
  constexpr int LDH = enc_ldh<OpT>();
  const int s = find_segment(seg, &t);
  if (s >= seg.n_seg) return;
  const int p0 = t * 32, np = min(32, seg.n[s] - p0);
  const bool isA = seg.side[s] == 0;
  const float* kp = e.kpts[isA ? 0 : 1] + 2 * (size_t)(seg.in_off[s] + p0);
  const float* cf = e.conf[isA ? 0 : 1] + (size_t)(seg.in_off[s] + p0);
  const float* de = e.desc[isA ? 0 : 1] + (size_t)e.D * (seg.in_off[s] + p0);
  const float iw = e.img[isA ? 0 : 2], ih = e.img[isA ? 1 : 3];
  const size_t row0 = (size_t)seg.row0[s] + p0;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();

  // layer 0 (3 -> w1) with ReLU; rows past the image are zero
  {
    const WT* W0 = reinterpret_cast<const WT*>(e.W[0]);
    const WT* b0 = reinterpret_cast<const WT*>(e.b[0]);
    const int w1 = e.width[1];
    for (int idx = tid; idx < 32 * w1; idx += kEncThreads) {
      const int r = idx / w1, o = idx % w1;
      float h = 0.f;
      if (r < np) {
        float x = kp[2 * r], y = kp[2 * r + 1];
        if (iw > 0.f) {
          const float sc = 0.7f * fmaxf(iw, ih);
          x = (x - 0.5f * iw) / sc;
          y = (y - 0.5f * ih) / sc;
        }
        h = (float)W0[3 * o] * x + (float)W0[3 * o + 1] * y + (float)W0[3 * o + 2] * cf[r] + (float)b0[o];
        h = fmaxf(h, 0.f);
      }
      hbuf[0][r * LDH + o] = (OpT)h;
    }
  }
  __syncthreads();

  int cur = 0;
  for (int l = 1; l < e.n_layers; ++l) {
    const int K = e.width[l], n_out = e.width[l + 1];
    const bool last = l == e.n_layers - 1;
    const WT* W = reinterpret_cast<const WT*>(e.W[l]);
    const WT* bias = reinterpret_cast<const WT*>(e.b[l]);
    const OpT* hin = hbuf[cur];
    OpT* hout = hbuf[cur ^ 1];
    for (int nb = wave; nb * 32 < n_out; nb += kEncWaves) {
      const int n = nb * 32 + (lane & 31);
      const WT* wrow = W + (size_t)n * K;
      f32x16 acc = zero16();
      // the last layer adds the descriptors: requested with the weights, all
      // at once (behind the state stores the compiler could not move them)
      float dv[16];
      if (last) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          dv[i] = r < np ? de[(size_t)r * e.D + n] : 0.f;
        }
      }
      // the whole weight row slice of this lane is requested before the MFMAs
      // (the loop is bound by load latency, not by the contraction)
      constexpr int KMAX = kMaxEncWidth;
      if constexpr (BF) {
        bf16x8 wb[KMAX / 16];
#pragma unroll
        for (int q = 0; q < KMAX / 16; ++q)
          if (q * 16 < K) wb[q] = *reinterpret_cast<const bf16x8*>(wrow + q * 16 + (lane >> 5) * 8);
#pragma unroll
        for (int q = 0; q < KMAX / 16; ++q)
          if (q * 16 < K) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(hin + (lane & 31) * LDH + q * 16 + (lane >> 5) * 8);
            acc = mfma(a, wb[q], acc);
          }
      } else {
        // k-slot l/32 covers the half [ (l/32) K/2, (l/32 + 1) K/2 ) of the contraction
        const int kh = (lane >> 5) * (K / 2);
        float4 wb[KMAX / 8];
#pragma unroll
        for (int q = 0; q < KMAX / 8; ++q)
          if (q * 4 < K / 2) wb[q] = *reinterpret_cast<const float4*>(wrow + kh + 4 * q);
#pragma unroll
        for (int q = 0; q < KMAX / 8; ++q)
          if (q * 4 < K / 2) {
            const float4 a = *reinterpret_cast<const float4*>(hin + (lane & 31) * LDH + kh + 4 * q);
            acc = mfma(a.x, wb[q].x, acc);
            acc = mfma(a.y, wb[q].y, acc);
            acc = mfma(a.z, wb[q].z, acc);
            acc = mfma(a.w, wb[q].w, acc);
          }
      }
      const float bv = (float)bias[n];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const float v = acc[i] + bv;
        if (!last) {
          hout[r * LDH + n] = (OpT)fmaxf(v, 0.f);
        } else {
          // rows past the image (the tile's padding) are zero, so that every
          // later product over the padded row space stays finite
          const float xv = r < np ? dv[i] + v : 0.f;
          e.X[(row0 + r) * e.ldx + n] = xv;
          if (e.XB) static_cast<bf16*>(e.XB)[(row0 + r) * e.ldx + n] = (bf16)xv;
        }
      }
    }
    __syncthreads();
    cur ^= 1;
  }
}

template <typename OpT, typename WT>
__global__ __launch_bounds__(kEncThreads) void k_encoder(EncArgs e, SegTable seg) {
  __shared__ __attribute__((aligned(16))) OpT hbuf[2][32 * enc_ldh<OpT>()];
  encoder_tile<OpT, WT>(e, seg, blockIdx.x, hbuf);
}

// The pass's prologue in one launch: workgroups [0, tiles) run the encoder,
// the others the merge fold of every stage (one fold block per wave), two
// independent latency-bound kernels that would otherwise run one after the
// other.
template <typename OpT, typename WT>
__global__ __launch_bounds__(kEncThreads) void k_encoder_fold(EncArgs e, SegTable seg, FoldArgs f, int tiles) {
  __shared__ __attribute__((aligned(16))) OpT hbuf[2][32 * enc_ldh<OpT>()];
  if ((int)blockIdx.x < tiles) {
    encoder_tile<OpT, WT>(e, seg, blockIdx.x, hbuf);
    return;
  }
  const int b = ((int)blockIdx.x - tiles) * kEncWaves + wave_id();
  if (b < fold_blocks(f)) fold_block_linear<WT>(f, b);
}

// Rotary table of self-attention (section 2.2 of the LightGlue review):
// for every compact row, (cos, sin) of theta_k = <b_k, p> for k < d_h / 2,
// with p the point's position normalised as for the encoder; padding rows
// get angle 0.  Computed once per call and read by every self stage's QKV
// epilogue.
__global__ __launch_bounds__(256) void k_rope_table(EncArgs e, SegTable seg, const float* __restrict__ basis,
                                                    int hp, int R, const int* __restrict__ ind,
                                                    float2* __restrict__ table) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * hp) return;
  const int r = idx / hp, k = idx % hp;
  // the image of row r: the last segment starting at or before it
  int s = 0;
  while (s + 1 < seg.n_seg && seg.row0[s + 1] <= r) ++s;
  // the point's index in the caller's arrays: its row within the image, or
  // the map `ind` once points have been dropped
  const int p = ind ? ind[r] : (r - seg.row0[s] < seg.n[s] ? r - seg.row0[s] : -1);
  float th = 0.f;
  if (p >= 0) {
    const bool isA = seg.side[s] == 0;
    const float* kp = e.kpts[isA ? 0 : 1] + 2 * (size_t)(seg.in_off[s] + p);
    const float iw = e.img[isA ? 0 : 2], ih = e.img[isA ? 1 : 3];
    float x = kp[0], y = kp[1];
    if (iw > 0.f) {
      const float sc = 0.7f * fmaxf(iw, ih);
      x = (x - 0.5f * iw) / sc;
      y = (y - 0.5f * ih) / sc;
    }
    th = fmaf(basis[2 * k], x, basis[2 * k + 1] * y);
  }
  float sn, cs;
  sincosf(th, &sn, &cs);
  table[idx] = make_float2(cs, sn);
}

hipError_t launch_rope_table(const EncArgs& e, const SegTable& seg, const float* basis, int dh, int R,
                             const int* ind, float2* table, hipStream_t st) {
  const int hp = dh / 2;
  if (R <= 0 || hp <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((R * hp + 255) / 256), dim3(256), 0, st, e, seg, basis, hp, R, ind, table);
  return hipGetLastError();
}

hipError_t launch_encoder(int op, int wd, const EncArgs& e, const SegTable& seg, hipStream_t st,
                          const FoldArgs* fold) {
  int tiles = 0;
  for (int s = 0; s < seg.n_seg; ++s) tiles += (seg.n[s] + 31) / 32;
  for (int l = 1; l < e.n_layers; ++l)
    if (e.width[l] > kMaxEncWidth) return hipErrorInvalidValue;
  for (int l = 1; l < e.n_layers; ++l)
    if (e.width[l] % 16 || e.width[l + 1] % 32) return hipErrorInvalidValue;
  if (op != wd || (op != SG_BF16 && op != SG_F32)) return hipErrorInvalidValue;
  const bool bf = op == SG_BF16;
  if (fold && fold->n > 0) {
    if (fold->n > kMaxFold || fold->D % 32) return hipErrorInvalidValue;
    const dim3 grid(tiles + (fold_blocks(*fold) + kEncWaves - 1) / kEncWaves);
    if (bf) hipLaunchKernelGGL((k_encoder_fold<bf16, bf16>), grid, dim3(kEncThreads), 0, st, e, seg, *fold, tiles);
    else hipLaunchKernelGGL((k_encoder_fold<float, float>), grid, dim3(kEncThreads), 0, st, e, seg, *fold, tiles);
    return hipGetLastError();
  }
  if (tiles == 0) return hipSuccess;
  if (bf) hipLaunchKernelGGL((k_encoder<bf16, bf16>), dim3(tiles), dim3(kEncThreads), 0, st, e, seg);
  else hipLaunchKernelGGL((k_encoder<float, float>), dim3(tiles), dim3(kEncThreads), 0, st, e, seg);
  return hipGetLastError();
}

}  // namespace sg
