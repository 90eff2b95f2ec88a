// Internal declarations shared by the HIP kernels and the host side of libsg.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sg.h"

namespace sg {

constexpr int kMaxSeg = 2 * SG_MAX_BATCH;  // one segment per image

// Images of the call in the compact row space (rows of every image stacked,
// A then B for each pair).  Passed by value as a kernel argument.
struct SegTable {
  int n_seg;
  int row0[kMaxSeg];     // first compact row of the image
  int n[kMaxSeg];        // points of the image
  int in_off[kMaxSeg];   // first point of the image in the caller's (padded) inputs
  int side[kMaxSeg];     // 0: image A inputs, 1: image B inputs
  int partner[kMaxSeg];  // segment of the other image of the pair
};

// Pairs of the call, for the score matrix, Sinkhorn and extraction.
// Z holds S*log2(e) of the real block only ([M][ldz], ldz = N rounded up to
// 4); ZT its transpose ([N][ldzt], ldzt = M rounded up to 4).  The dustbin
// row, column and corner are the constant alpha and are never stored.
// u (M+1 entries per pair) and v (N+1) are base-2 dual variables, stored
// flattened over the pairs at upre[b] and vpre[b].
struct PairTable {
  int n_pairs;
  int rb;                                          // Sinkhorn rows per workgroup (4 or 8)
  int M[SG_MAX_BATCH], N[SG_MAX_BATCH];
  int rowA[SG_MAX_BATCH];                          // compact row of f_A (f_B follows at +M)
  int z_off[SG_MAX_BATCH];                         // float offset of Z ([M][ld4(N)])
  int zt_off[SG_MAX_BATCH];                        // float offset of ZT ([N][ld4(M)]), two-sweep only
  int p_off[SG_MAX_BATCH];                         // float offset of the column partials ([G][ld4(N)])
  int upre[SG_MAX_BATCH + 1];                      // prefix sums of (M+1): flattened u rows
  int vpre[SG_MAX_BATCH + 1];                      // prefix sums of (N+1): flattened v rows
  int gpre[SG_MAX_BATCH + 1];                      // prefix sums of G = ceil((M+1)/rb): row blocks
  int uoff[SG_MAX_BATCH], voff[SG_MAX_BATCH];      // storage offsets of u, v (multiples of 4)
  // dispatch order of the fused Sinkhorn iteration's row blocks: the pairs
  // ord[0], ord[1], ... (widest rows first), pair ord[k] taking blocks
  // [opre[k], opre[k + 1])
  int opre[SG_MAX_BATCH + 1];
  unsigned char ord[SG_MAX_BATCH];
};

__host__ __device__ inline int ld4(int n) { return (n + 3) & ~3; }

// One GEMM problem: rows of A starting at a_row0 times rows of W starting at
// w_row0 (the score matrix uses f_B as "W").
struct GemmProblem {
  int a_row0, w_row0, rows, n_out, c_off, ct_off, ldc, ldct;
};
struct GemmBatch {
  int n;
  GemmProblem p[SG_MAX_BATCH];
};

enum Epilogue {
  EPI_BIAS = 0,   // C = A W^T + b
  EPI_RELU = 1,   // C = max(A W^T + b, 0)
  EPI_RESID = 2,  // C (fp32) = C + A W^T + b   (in place residual add)
  EPI_QKV = 3,    // columns < split: QK = A W^T + b (tied: q and k); others: VT / VS
  EPI_SCORE = 4   // C = scale * A W^T and CT = its transpose (fp32)
};

struct GemmArgs {
  const void* A0; int lda0; int K0;  // columns [0, K0) of A
  const void* A1; int lda1;          // columns [K0, K) of A (operand type)
  const void* W; int ldw;            // weights [n_out][K]
  const void* bias;                  // [n_out] or null
  int K;
  void* C; void* C2;                 // outputs (C2: VT / VS, ZT, or the bf16 shadow of C for EPI_RESID)
  void* C3;                          // EPI_QKV, bf16: KS
  float scale;
  int split;                         // EPI_QKV: first column that goes to VT (VS)
  int tied;                          // EPI_QKV: columns [0, split) are both q and k
  const float2* rope;                // EPI_QKV: per-row (cos, sin) of the rotary angles, [rows][rope_dh/2], or null
  int rope_dh;                       // head dimension of the rotary table
  const int* stop;                   // or null: the launch does nothing when *stop != 0 (adaptive depth)
  int gx, gy;                        // row and column tiles (set by the launcher)
};

// Fused keypoint encoder: linear layers [3 -> width[1] -> ... -> D].
constexpr int kMaxEncWidth = 256;  // widest hidden layer (held in LDS)
struct EncArgs {
  const float* kpts[2];  // image A / B inputs (caller layout, padded in batch mode)
  const float* conf[2];
  const float* desc[2];
  float img[4];          // wA, hA, wB, hB; 0 = positions already normalised
  int D, ldx, n_layers;  // n_layers linear layers (n_enc + 1)
  int width[SG_MAX_ENC + 2];
  const void* W[SG_MAX_ENC + 1];
  const void* b[SG_MAX_ENC + 1];
  float* X;              // states [R][ldx]
  void* XB;              // or null: their bf16 copy [R][ldx] (bf16 networks)
};

// Attention operands.  fp32 networks: qk [R][ldqk] holds q (columns
// h*dh..) and k (columns D + h*dh..), vt [D][ldvt] holds v transposed.
// bf16 networks: qk holds q only; k and v are tile-swizzled so that every
// MFMA operand fragment is 16 contiguous bytes per lane (one 1 KB load per
// wave):
//   ks: [R/32][D/16][64][8]: block (tile, c) holds rows 32 tile.. and
//       columns 16 c..; lane L, element t is k[32 tile + L%32][16 c + 8 (L/32) + t];
//   vs: [R/32][D/32][2][64][8]: block (tile, f, j), lane L, element t is
//       v[32 tile + 16 j + 8 (t/4) + 4 (L/32) + t%4][32 f + L%32], which is
//       the accumulator layout of a 32x32 MFMA block (elements 8j..8j+7).
struct AttnArgs {
  const void* qk;
  const void* vt;    // fp32
  const void* ks;    // bf16
  const void* vs;    // bf16
  void* out;         // [R][D] message (heads concatenated)
  int D, ldvt, ldqk, cross, heads;
  float scale2;      // log2(e) / sqrt(dh)
  const int* stop;   // or null: the launch does nothing when *stop != 0 (adaptive depth)
  // shared similarity (bidirectional cross stage of one pair): the queries of
  // segment g (0: image A, 1: image B) read their base-2 scaled similarity
  // rows from sm + s_off[g] + h s_hs[g] (row pitch s_ld[g]) and the rows'
  // base-2 log-sum-exp from lse + l_off[g] + h l_hs[g]
  const float* sm;
  const float* lse;
  long s_off[2], s_hs[2];
  int s_ld[2], l_off[2], l_hs[2];
};

struct FoldArgs;

// Host-side launchers.  The encoder; with `fold` (stages of the merge fold,
// see FoldArgs) the fold runs in the same launch, beside the encoder tiles.
hipError_t launch_encoder(int op_dtype, int w_dtype, const EncArgs& e, const SegTable& seg,
                          hipStream_t st, const FoldArgs* fold = nullptr);
// (cos, sin) of the rotary angles of every compact row ([R][dh/2]) from the
// positions in e.kpts / e.img (normalised as for the encoder); ind (or
// null): the caller's point index of every row, -1 on padding.
hipError_t launch_rope_table(const EncArgs& e, const SegTable& seg, const float* basis, int dh, int R,
                             const int* ind, float2* table, hipStream_t st);
hipError_t launch_gemm(int op_dtype, int a0_is_f32, int w_dtype, int out_is_f32, int epi,
                       const GemmArgs& g, const GemmBatch& b, int max_rows, int max_n,
                       hipStream_t st);
// y (bf16) = x (fp32) rounded to nearest even, n a multiple of 4.
hipError_t launch_to_bf16(const float* x, void* y, int n, hipStream_t st);

// Merge projection folded into the update MLP's first layer, per stage:
// W1 [2D][2D] (input [x || m]), m = Wm a + bm  =>  W1 [x || m] + b1 =
// Wf [x || a] + bf with Wf = [W1[:, :D] | W1[:, D:] Wm], bf = b1 + W1[:, D:] bm.
// Up to kMaxFold stages per launch; wf / bf: [n][2D][2D] / [n][2D] in the
// weights' type.
constexpr int kMaxFold = 32;
struct FoldArgs {
  const void* w1[kMaxFold];
  const void* b1[kMaxFold];
  const void* wm[kMaxFold];
  const void* bm[kMaxFold];
  void* wf;
  void* bf;
  int D, n;
};
hipError_t launch_fold_merge(int w_dtype, const FoldArgs& f, hipStream_t st);
hipError_t launch_attention(int op_dtype, int dh, const AttnArgs& a, const SegTable& seg,
                            int heads, hipStream_t st);
// Base-2 log-sum-exp of each of `rows` rows ([rows][ld], first `cols` entries).
hipError_t launch_rows_lse(const float* S, int ld, int rows, int cols, float* out, hipStream_t st);
// A bidirectional cross stage of one pair from its shared similarity
// (AttnArgs::sm / lse, scale2 = 1): the messages of both images.
hipError_t launch_attention_shared(int op_dtype, int dh, const AttnArgs& a, const SegTable& seg, int heads,
                                   hipStream_t st);
// alpha_dev (device pointer to the dustbin score) overrides alpha2 when non-null.
// Sinkhorn rows per workgroup (4 or 8) for a batch of pairs.
int sink_rows_per_block(const int* M, const int* N, int n_pairs);
hipError_t launch_sink_rows(const float* Z, const PairTable& pt, const float* v_in, float* u_out,
                            float* P, float* Pd, float* PV, int* PI, float alpha2, const float* alpha_dev,
                            int update_u, hipStream_t st);
// Fused one-pass iteration (k_sink_iter): rows per workgroup for a batch
// (0: some row is too wide, use launch_sink_rows + launch_sink_cols), and
// the launch.  Pin / Pdin: the previous iteration's partials (nullptr: v =
// 0); Pout / Pdout: this iteration's (a different buffer).
int sink_iter_rows_per_block(const int* N, int n_pairs);
// Row blocks of a pair in the fused iteration (the last one takes the dustbin row).
int sink_iter_blocks(int M, int rb);
hipError_t launch_sink_iter(const float* Z, const PairTable& pt, const float* Pin, const float* Pdin, float* u_out,
                            float* Pout, float* Pdout, float* PV, int* PI, float alpha2, const float* alpha_dev,
                            int update_u, hipStream_t st);
hipError_t launch_sink_cols(const PairTable& pt, const float* P, const float* Pd, float* v_out, const float* PV,
                            const int* PI, int* idx1, int write_v, int Npad, int32_t* m1, float* s1,
                            hipStream_t st);
// idx1 (one pair, which = 1, w_in the final u only): the sweep also leaves
// the column argmax and the default side-B outputs (k_col_argmax's work)
hipError_t launch_lse(const float* Z, const PairTable& pt, int which, const float* w_in, float* w_out,
                      float alpha2, const float* alpha_dev, int total_rows, hipStream_t st, int* idx1 = nullptr,
                      int32_t* m1 = nullptr, float* s1 = nullptr);
// What the extraction kernels read as the real block of the log assignment
// (their `mode`): EXT_SINKHORN: Z2 + u + v + log2(M+N) (base 2); EXT_DS: the
// double-softmax head, 2 Z2 + u + v (base 2, see sg_double_softmax.hip);
// EXT_RAW: Z itself, a natural-log assignment given by the caller (u, v unused).
enum { EXT_SINKHORN = 0, EXT_DS = 1, EXT_RAW = 2 };
hipError_t launch_col_argmax(const float* ZT, const PairTable& pt, const float* u, int* idx1, int Npad,
                             int32_t* m1, float* s1, int mode, hipStream_t st);
hipError_t launch_sink_extract(const float* Z, const PairTable& pt, const float* u, const float* v,
                               const int* idx1, int Mpad, int Npad, float thr, int32_t* m0, float* s0,
                               int32_t* m1, float* s1, int mode, hipStream_t st);
// Stage entry points on caller-given (M+1) x (N+1) matrices C (leading
// dimension ldc): the real block times `scale` into Z [M][ld4(N)] and ZT
// [N][ld4(M)]; with bcol / brow non-null, the dustbin column (M+1 entries,
// the corner last) and row (N+1 entries) times `scale`.
hipError_t launch_stage_couplings(const float* C, int64_t ldc, int M, int N, float scale, float* Z, float* ZT,
                                  float* bcol, float* brow, hipStream_t st);
// C [(M+1)][ldc] = S [M][lds] bordered by the dustbin score *alpha_dev.
hipError_t launch_stage_border(const float* S, int lds, int M, int N, const float* alpha_dev, float* C, int64_t ldc,
                               hipStream_t st);
// u = ln2 u2, v = ln2 v2 and (logP non-null) logP = C + u + v + log(M+N).
hipError_t launch_stage_duals(const float* C, int64_t ldc, int M, int N, const float* u2, const float* v2, float* u,
                              float* v, float* logP, int64_t ldp, hipStream_t st);
// One Sinkhorn sweep with explicit dustbins over the nr + 1 rows of Z (or
// ZT): bown [nr + 1] the rows' dustbin-column entries (corner last), bcross
// [ld4(nc + 1)] the dustbin row's entries.
hipError_t launch_lse_explicit(const float* Z, const float* w_in, float* w_out, int nr, int nc, float lm_real,
                               float lm_dust, const float* bown, const float* bcross, hipStream_t st);
hipError_t launch_write_logp(const float* Z, const PairTable& pt, const float* u, const float* v,
                             float alpha2, const float* alpha_dev, float* logP, int64_t ld,
                             int64_t pair_stride, int total_rows, hipStream_t st);
// Double-softmax head: u, v (base-2 row / column terms) and ud, vd (dustbin
// entries) from Z, ZT and the states X [R][D] with the matchability weights
// wz [D], bias at bz_dev (device, w_dtype) or bz (bz_dev == nullptr).
hipError_t launch_ds_stats(const float* Z, const float* ZT, const PairTable& pt, const float* X, int D,
                           int w_dtype, const void* wz, const void* bz_dev, float bz, float* u, float* v,
                           float* ud, float* vd, hipStream_t st);
hipError_t launch_ds_write_logp(const float* Z, const PairTable& pt, const float* u, const float* v,
                                const float* ud, const float* vd, float* logP, int64_t ld, int64_t pair_stride,
                                int total_rows, hipStream_t st);
hipError_t launch_fill_f32(float* p, float v, int n, hipStream_t st);

// Adaptive depth and width of one pair (sg_adaptive.hip).
hipError_t launch_iota_rows(const SegTable& seg, int R, int* ind, hipStream_t st);
hipError_t launch_fill_i32(int* p, int v, int n, hipStream_t st);
// Per-point statistics (keep flags, per-workgroup counts in part[4 nb]),
// then one workgroup that decides the stop (1 - unconfident / total > alpha
// with flags bit 1) into *stop and posts seq, stop and the counts to the
// host-visible post[0..5] (seq last).  Nothing runs once *stop is set.
hipError_t launch_adaptive_stats(const float* X, const SegTable& seg, int D, int w_dtype, const void* wc,
                                 const void* bc, const void* wz, const void* bz, float lam, float min_match,
                                 int flags, float alpha, int total, int seq, int* keep, int* part, int* stop,
                                 int* post, hipStream_t st);
hipError_t launch_prune_scan(const SegTable& seg, const int* keep, int prune_mask, int* newidx, hipStream_t st);
hipError_t launch_compact_rows(const float* Xo, const int* ind_o, const int* newidx, const SegTable& so,
                               const SegTable& sn, int R_old, int R_new, int D, int prune_mask, int M, float* Xn,
                               int* ind_n, int* pr, hipStream_t st);
hipError_t launch_scatter_outputs(const SegTable& seg, const int* ind, const int32_t* tm0, const float* ts0,
                                  const int32_t* tm1, const float* ts1, int32_t* m0, float* s0, int32_t* m1,
                                  float* s1, const float* F, int D, float* fA, float* fB, const float* lt, int M,
                                  int N, float* logP, int64_t ld, int R, hipStream_t st);
hipError_t launch_fill_empty(int32_t* m, float* s, int n, hipStream_t st);

}  // namespace sg
