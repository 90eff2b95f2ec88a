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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Index of this thread's wave in the workgroup, as a scalar: deriving loop
// bounds and addresses from it keeps wave-uniform control flow on the scalar
// unit instead of exec-mask branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Cross-lane moves inside each row of 16 lanes (DPP): quad_perm [1,0,3,2]
// and [2,3,0,1] swap neighbours and pairs, row_half_mirror (0x141) and
// row_mirror (0x140) reverse 8- and 16-lane groups.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Wave-wide reduction, result in every lane: four DPP steps leave each row
// of 16 lanes holding its row's result, then the four rows are combined from
// scalar reads of lanes 0, 16, 32, 48.  Call with the whole wave active.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_f<kDppXor1>(v));
  v = op(v, dpp_f<kDppXor2>(v));
  v = op(v, dpp_f<kDppHalfMirror>(v));
  v = op(v, dpp_f<kDppMirror>(v));
  return op(op(lane_f(v, 0), lane_f(v, 16)), op(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

// The value of lane l ^ 32 combined with the lane's own, in every lane:
// v_permlane32_swap exchanges the two 32-lane halves in one VALU
// instruction (a cross-lane shuffle would go through the LDS crossbar).
// Applied to (v, v) it returns (lower half of v in both halves, upper half
// in both), so op of the two is op(v[l % 32], v[l % 32 + 32]).
__device__ __forceinline__ float half_swap_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// global_load_lds of 16 bytes per lane: lane l of the wave writes the 16
// bytes at src (its own address) to LDS at the wave-uniform lds_base + 16 l;
// counted by vmcnt.  The source is cast to the global address space
// explicitly: left to an implicit conversion, the host pass of some kernel
// template instantiations drops their launch stubs without a diagnostic.
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds_base) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

// s_waitcnt with vmcnt = N and the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(), whose
// release also waits for every global_load_lds still in flight: for loops
// that keep later LDS loads in flight across the barrier and wait for the
// ones they need with wait_vm first.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// (value, index) argmax over the wave: the larger value wins, the lower
// index among equal values.  Result in every lane.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp_f<CTRL>(v);
  const int oi = dpp_i<CTRL>(i);
  argmax_merge(v, i, ov, oi);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<kDppXor1>(v, i);
  argmax_step<kDppXor2>(v, i);
  argmax_step<kDppHalfMirror>(v, i);
  argmax_step<kDppMirror>(v, i);
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) argmax_merge(bv, bi, lane_f(v, r), __builtin_amdgcn_readlane(i, r));
  v = bv;
  i = bi;
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

// Pins kernel arguments in scalar registers at this point, so that their
// loads are issued together, in one round, ahead of a kernel's first early
// exit.  (Left alone, the compiler sinks each load past the exits that
// precede its first use; every round then waits on a miss, since the
// argument block of every launch is new to the scalar cache.)
template <class T>
__device__ __forceinline__ void arg_in_sgprs(const T& v) {
  asm volatile("" ::"s"(v));
}
template <class... T>
__device__ __forceinline__ void args_in_sgprs(const T&... v) {
  (arg_in_sgprs(v), ...);
}

// Pair of a flattened row index g (the same in every lane of the wave) given
// prefix sums `pre` of per-pair rows (n_pairs + 1 entries, n_pairs <= 64):
// the count of pairs whose rows end at or before g, from one load per lane
// and a ballot.  (A search over the sums would chain up to n_pairs dependent
// scalar loads before the kernel's first data load.)  Call with the whole
// wave active; returns n_pairs when g is past the last pair.
static_assert(SG_MAX_BATCH <= 64, "find_pair takes one lane per pair");
__device__ __forceinline__ int find_pair(const int* pre, int n_pairs, int g) {
  const int lane = threadIdx.x & 63;
  const int e = lane < n_pairs ? pre[lane + 1] : 0;
  return __popcll(__ballot(lane < n_pairs && g >= e));
}

}  // namespace sg
