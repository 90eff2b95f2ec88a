// The merge fold's device code, shared by its own kernel (k_fold_merge) and
// the pass's prologue launch, which runs it beside the keypoint encoder.
#pragma once
#include "sg_device.h"

namespace sg {

// Merge fold (FoldArgs): block (x, y, z), one wave, = 32 rows n0 = 32 x of
// stage z.  y < D / 32: the 32 x 32 tile (n0, D + 32 y) of Wf, W1[:, D:] Wm on
// MFMA (operand A: rows of W1's message half, contraction along them; B:
// Wm read down its columns, 32 lanes covering 64 contiguous bytes of a row
// per load); y = D / 32: the copied x half of the 32 rows and their bias.
template <typename T>
__device__ __forceinline__ void fold_block(const FoldArgs& f, int bx, int by, int bz) {
  const int s = bz, D = f.D, D2 = 2 * D;
  const T* __restrict__ W1 = static_cast<const T*>(f.w1[s]);
  const T* __restrict__ Wm = static_cast<const T*>(f.wm[s]);
  T* __restrict__ Wf = static_cast<T*>(f.wf) + (size_t)s * D2 * D2;
  const int lane = threadIdx.x & 63, lr = lane & 31, hi = lane >> 5;
  const int n0 = bx * 32;
  if (by < D / 32) {
    const int k0 = by * 32;
    const T* arow = W1 + (size_t)(n0 + lr) * D2 + D;
    f32x16 acc = zero16();
    // K in chunks of four MFMA steps whose loads are all issued before the
    // first of them (the steps past D of the last chunk are skipped)
    if constexpr (std::is_same<T, bf16>::value) {
      for (int j0 = 0; j0 < D; j0 += 64) {
        bf16x8 a[4], b[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int jj = j0 + 16 * q + 8 * hi;
          if (j0 + 16 * q < D) {
            a[q] = *reinterpret_cast<const bf16x8*>(arow + jj);
#pragma unroll
            for (int t = 0; t < 8; ++t) b[q][t] = Wm[(size_t)(jj + t) * D + k0 + lr];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (j0 + 16 * q < D) acc = mfma(a[q], b[q], acc);
      }
    } else {
      for (int j0 = 0; j0 < D; j0 += 32) {  // D is a multiple of 32
        float a[16], b[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          a[q] = arow[j0 + 2 * q + hi];
          b[q] = Wm[(size_t)(j0 + 2 * q + hi) * D + k0 + lr];
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) acc = mfma(a[q], b[q], acc);
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e)
      Wf[(size_t)(n0 + 8 * (e >> 2) + 4 * hi + (e & 3)) * D2 + D + k0 + lr] = (T)acc[e];
    return;
  }
  // x half of the 32 rows, 16 bytes per lane and step
  constexpr int CH = 16 / sizeof(T);
  typedef T Vec __attribute__((ext_vector_type(CH)));
  for (int idx = lane; idx < 32 * (D / CH); idx += 64) {
    const int r = n0 + idx / (D / CH), c = (idx % (D / CH)) * CH;
    *reinterpret_cast<Vec*>(Wf + (size_t)r * D2 + c) = *reinterpret_cast<const Vec*>(W1 + (size_t)r * D2 + c);
  }
  // bf = b1 + W1[:, D:] bm: lane half hi takes half of the contraction
  const T* __restrict__ bm = static_cast<const T*>(f.bm[s]);
  const T* __restrict__ b1 = static_cast<const T*>(f.b1[s]);
  const T* arow = W1 + (size_t)(n0 + lr) * D2 + D;
  float acc = 0.f;
  for (int j = hi * (D / 2); j < (hi + 1) * (D / 2); j += CH) {
    const Vec a = *reinterpret_cast<const Vec*>(arow + j), b = *reinterpret_cast<const Vec*>(bm + j);
#pragma unroll
    for (int t = 0; t < CH; ++t) acc = fmaf((float)a[t], (float)b[t], acc);
  }
  acc = half_swap_sum(acc);
  if (hi == 0) static_cast<T*>(f.bf)[(size_t)s * D2 + n0 + lr] = (T)((float)b1[n0 + lr] + acc);
}

// the fold's blocks (x, y, z): 2D / 32 row groups, D / 32 + 1 column groups
// (the last: the copied x half and the bias), f.n stages
__host__ __device__ inline int fold_blocks(const FoldArgs& f) { return (2 * f.D / 32) * (f.D / 32 + 1) * f.n; }

// block number b in x-fastest order
template <typename T>
__device__ __forceinline__ void fold_block_linear(const FoldArgs& f, int b) {
  const int gx = 2 * f.D / 32, gy = f.D / 32 + 1;
  fold_block<T>(f, b % gx, (b / gx) % gy, b / (gx * gy));
}

}  // namespace sg
