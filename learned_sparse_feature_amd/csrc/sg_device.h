// Device-side helpers shared by the HIP kernels of libsg (gfx950 / CDNA4).
//
// MFMA lane layouts used (checked on the device): for
// v_mfma_f32_32x32x16_bf16 lane l holds A[l%32][8*(l/32) + t] and
// B[8*(l/32) + t][l%32] (t = 0..7); for v_mfma_f32_32x32x2f32 lane l holds
// A[l%32][l/32] and B[l/32][l%32]; both return C[8*(i/4) + 4*(l/32) + i%4][l%32]
// in accumulator i.  A contraction index may be relabelled freely as long as
// A and B agree, so the kernels map MFMA k-slots to whatever contiguous
// memory suits each lane.
#pragma once

#include <math.h>

#include <type_traits>

#include "sg_internal.h"

namespace sg {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

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

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Segment (image) of a flattened 32-row tile index; returns the tile's first
// row within the image in *t, or n_seg when the index is past the last tile.
__device__ __forceinline__ int find_segment(const SegTable& seg, int* t) {
  int s = 0;
  for (; s < seg.n_seg; ++s) {
    const int nt = (seg.n[s] + 31) >> 5;
    if (*t < nt) break;
    *t -= nt;
  }
  return s;
}

// Pair of a flattened row index given prefix sums `pre` of per-pair rows.
__device__ __forceinline__ int find_pair(const int* pre, int n_pairs, int g) {
  int b = 0;
  while (b < n_pairs && g >= pre[b + 1]) ++b;
  return b;
}

}  // namespace sg
