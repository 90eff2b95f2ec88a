/*
 * sg_oracle.c - plain float64 CPU oracle of the SuperGlue matching forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the HIP library is checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark load it (through
 * oracle/native.py); the product path never does, and nothing here is shared
 * with the product: no header, kernel, helper or table.
 *
 * Every routine is a plain loop over the definition it cites, in double
 * precision, with each sum taken in index order; there is no BLAS, no
 * blocking and no reordering of a sum.  The only concession to speed is that
 * OpenMP may hand independent output rows (points, matrix rows or columns)
 * to different threads; every output is still computed by one thread with
 * the same sequential loop, so the results do not depend on the thread count.
 *
 * Pages cited (by title):
 *   [GNN-blog]   "SuperGlue 的注意力图神经网络怎样传递信息" (huluoboge.top blog)
 *   [realcat]    "SuperGlue:Learning Feature Matching with Graph Neural Networks论文阅读"
 *                (realcat.vercel.app notes)
 *   [forward]    "SuperGlue_model_forward_learning" (SuperGlue_Code_Learning notes)
 *   [LightGlue]  "论文解读:LightGlue,让稀疏特征匹配随难度自适应地快" (vincentqin.tech)
 *
 * Layouts: row-major; a weight matrix W is [out][in] (a kernel-1 Conv1d or
 * Linear weight), points are rows ([n][D]).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef int64_t i64;

/* ------------------------------------------------------------ threads */

static int g_threads = 0; /* 0: the OpenMP default */

void orc_set_threads(int n) { g_threads = n; }

int orc_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

#define PAR_FOR _Pragma("omp parallel for schedule(static) num_threads(orc_threads())")

/* ------------------------------------------------------------ helpers */

/* sum_{k < n} a[k] b[k], in index order */
static double dot(const double* a, const double* b, i64 n) {
  double s = 0.0;
  for (i64 k = 0; k < n; ++k) s += a[k] * b[k];
  return s;
}

/* log sum_k exp(x[k * stride]) over n terms, written as the pages' code
   computes it: the maximum m first, then m + log sum exp(x - m); -inf when
   every term is -inf (or n == 0). */
static double log_sum_exp(const double* x, i64 n, i64 stride) {
  double m = -INFINITY;
  for (i64 k = 0; k < n; ++k)
    if (x[k * stride] > m) m = x[k * stride];
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (i64 k = 0; k < n; ++k) s += exp(x[k * stride] - m);
  return m + log(s);
}

static void* must_alloc(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) abort();
  return p;
}

/* -------------------------------------------------- linear layers */

/* y[i][o] = sum_k W[o][k] x[i][k] + b[o]: a per-point linear map (Conv1d with
   kernel 1), [realcat] "特征点Encode" and "Attentional Aggregation".  b may
   be NULL (no bias). */
void orc_linear(const double* x, i64 n, int in, const double* W, const double* b, int out, double* y) {
  PAR_FOR
  for (i64 i = 0; i < n; ++i)
    for (int o = 0; o < out; ++o) y[i * out + o] = dot(W + (i64)o * in, x + i * in, in) + (b ? b[o] : 0.0);
}

/* [forward] normalize_keypoints: centre on (w/2, h/2), divide both
   coordinates by 0.7 * max(w, h). */
void orc_normalize_keypoints(const double* kp, i64 n, double w, double h, double* out) {
  const double scale = (w > h ? w : h) * 0.7;
  for (i64 i = 0; i < n; ++i) {
    out[2 * i] = (kp[2 * i] - w / 2.0) / scale;
    out[2 * i + 1] = (kp[2 * i + 1] - h / 2.0) / scale;
  }
}

/* [realcat] "特征点Encode" (KeypointEncoder / MLP): the input of point i is
   (x_i, y_i, c_i); layer l maps it by W_l p + b_l, with a ReLU after every
   layer but the last.  widths[0] = 3, widths[n_layers] = the output width. */
void orc_keypoint_encoder(const double* kpn, const double* conf, i64 n, int n_layers, const int* widths,
                          const double* const* W, const double* const* b, double* out) {
  int wmax = 3;
  for (int l = 0; l <= n_layers; ++l)
    if (widths[l] > wmax) wmax = widths[l];
  const int dout = widths[n_layers];
#pragma omp parallel num_threads(orc_threads())
  {
    double* h = (double*)must_alloc(sizeof(double) * wmax);
    double* g = (double*)must_alloc(sizeof(double) * wmax);
#pragma omp for schedule(static)
    for (i64 i = 0; i < n; ++i) {
      h[0] = kpn[2 * i];
      h[1] = kpn[2 * i + 1];
      h[2] = conf[i];
      for (int l = 0; l < n_layers; ++l) {
        const int in = widths[l], o_n = widths[l + 1];
        for (int o = 0; o < o_n; ++o) {
          double t = dot(W[l] + (i64)o * in, h, in) + b[l][o];
          if (l < n_layers - 1 && t < 0.0) t = 0.0;
          g[o] = t;
        }
        memcpy(h, g, sizeof(double) * o_n);
      }
      memcpy(out + i * dout, h, sizeof(double) * dout);
    }
    free(h);
    free(g);
  }
}

/* ------------------------------------------------------- attention */

/* One stage's weights.  Standard stages hold W_q, W_k, W_v; a bidirectional
   cross stage ([LightGlue] section 2.3) holds W_qk (and W_v) instead and has
   W_q == NULL. */
typedef struct {
  const double *Wq, *bq, *Wk, *bk, *Wv, *bv, *Wm, *bm, *W1, *b1, *W2, *b2, *Wqk, *bqk;
} orc_stage;

/* [LightGlue] section 2.2: channels (2k, 2k+1) of every head of t [n][D]
   rotated by the angle theta[i][k] (k < D/H/2; the same angles in every head):
   (a, b) -> (a cos - b sin, a sin + b cos). */
void orc_rotate_pairs(const double* t, i64 n, int D, int H, const double* theta, double* out) {
  const int dh = D / H, nk = dh / 2;
  for (i64 i = 0; i < n; ++i)
    for (int h = 0; h < H; ++h)
      for (int k = 0; k < nk; ++k) {
        const double a = t[i * D + h * dh + 2 * k], c = t[i * D + h * dh + 2 * k + 1];
        const double th = theta[i * nk + k];
        out[i * D + h * dh + 2 * k] = a * cos(th) - c * sin(th);
        out[i * D + h * dh + 2 * k + 1] = a * sin(th) + c * cos(th);
      }
}

/* [LightGlue] section 2.2: theta[i][k] = <basis_k, p_i> for the 2-D basis
   vectors basis[k] (k < nk) and positions p [n][2]. */
void orc_rope_angles(const double* pos, i64 n, const double* basis, int nk, double* theta) {
  for (i64 i = 0; i < n; ++i)
    for (int k = 0; k < nk; ++k) theta[i * nk + k] = pos[2 * i] * basis[2 * k] + pos[2 * i + 1] * basis[2 * k + 1];
}

/* Per head h (channels [h dh, (h+1) dh)): for query i,
   alpha_ij = softmax_j(q_i . k_j / sqrt(dh)) over the m sources and
   msg_i = sum_j alpha_ij v_j ([GNN-blog] "Attention 让节点自己选择消息来源";
   [realcat] "Attentional Aggregation").  The softmax subtracts the row
   maximum before exp, as the worked example's normalisation allows. */
static void attention_heads(const double* q, i64 n, const double* k, const double* v, i64 m, int D, int H,
                            double* msg) {
  const int dh = D / H;
  const double scale = sqrt((double)dh);
#pragma omp parallel num_threads(orc_threads())
  {
    double* e = (double*)must_alloc(sizeof(double) * (m > 0 ? m : 1));
#pragma omp for schedule(static)
    for (i64 i = 0; i < n; ++i)
      for (int h = 0; h < H; ++h) {
        const int c0 = h * dh;
        double mx = -INFINITY;
        for (i64 j = 0; j < m; ++j) {
          e[j] = dot(q + i * D + c0, k + j * D + c0, dh) / scale;
          if (e[j] > mx) mx = e[j];
        }
        double s = 0.0;
        for (i64 j = 0; j < m; ++j) {
          e[j] = exp(e[j] - mx);
          s += e[j];
        }
        for (int d = 0; d < dh; ++d) {
          double acc = 0.0;
          for (i64 j = 0; j < m; ++j) acc += (e[j] / s) * v[j * D + c0 + d];
          msg[i * D + c0 + d] = m > 0 ? acc : 0.0;
        }
      }
    free(e);
  }
}

/* Message of every query point of x [n][D] from the sources src [m][D]
   ([realcat] "Attentional Aggregation"): q = W_q x + b_q from the query
   image, k = W_k src + b_k and v = W_v src + b_v from the source image, the
   heads of attention_heads, then the merge projection W_m msg + b_m of the
   concatenated heads.  theta_x / theta_src (or NULL): rotary angles of the
   query and source points ([LightGlue] section 2.2: q and k rotated, v not). */
void orc_multi_head_attention(const double* x, i64 n, const double* src, i64 m, int D, int H, const orc_stage* st,
                              const double* theta_x, const double* theta_src, double* out) {
  double* q = (double*)must_alloc(sizeof(double) * n * D);
  double* k = (double*)must_alloc(sizeof(double) * m * D);
  double* v = (double*)must_alloc(sizeof(double) * m * D);
  double* msg = (double*)must_alloc(sizeof(double) * n * D);
  orc_linear(x, n, D, st->Wq, st->bq, D, q);
  orc_linear(src, m, D, st->Wk, st->bk, D, k);
  orc_linear(src, m, D, st->Wv, st->bv, D, v);
  if (theta_x) {
    double* r = (double*)must_alloc(sizeof(double) * (n > m ? n : m) * D);
    orc_rotate_pairs(q, n, D, H, theta_x, r);
    memcpy(q, r, sizeof(double) * n * D);
    orc_rotate_pairs(k, m, D, H, theta_src, r);
    memcpy(k, r, sizeof(double) * m * D);
    free(r);
  }
  attention_heads(q, n, k, v, m, D, H, msg);
  orc_linear(msg, n, D, st->Wm, st->bm, D, out);
  free(q);
  free(k);
  free(v);
  free(msg);
}

/* [LightGlue] section 2.3 (bidirectional cross-attention): per image one
   projection qk = W_qk x + b_qk and v = W_v x + b_v.  Per head the
   similarity sim_ij = qk0_i . qk1_j / sqrt(dh) is formed once; its softmax
   over j (row i) aggregates image 1's values into m0_i, its softmax over i
   (column j) aggregates image 0's values into m1_j.  Both then pass the
   merge projection. */
void orc_bidirectional_cross_attention(const double* x0, i64 n0, const double* x1, i64 n1, int D, int H,
                                       const orc_stage* st, double* m0, double* m1) {
  const int dh = D / H;
  const double scale = sqrt((double)dh);
  double* qk0 = (double*)must_alloc(sizeof(double) * n0 * D);
  double* qk1 = (double*)must_alloc(sizeof(double) * n1 * D);
  double* v0 = (double*)must_alloc(sizeof(double) * n0 * D);
  double* v1 = (double*)must_alloc(sizeof(double) * n1 * D);
  double* a0 = (double*)must_alloc(sizeof(double) * n0 * D);
  double* a1 = (double*)must_alloc(sizeof(double) * n1 * D);
  double* sim = (double*)must_alloc(sizeof(double) * (n0 * n1 > 0 ? n0 * n1 : 1));
  orc_linear(x0, n0, D, st->Wqk, st->bqk, D, qk0);
  orc_linear(x1, n1, D, st->Wqk, st->bqk, D, qk1);
  orc_linear(x0, n0, D, st->Wv, st->bv, D, v0);
  orc_linear(x1, n1, D, st->Wv, st->bv, D, v1);
  for (int h = 0; h < H; ++h) {
    const int c0 = h * dh;
    PAR_FOR
    for (i64 i = 0; i < n0; ++i)
      for (i64 j = 0; j < n1; ++j) sim[i * n1 + j] = dot(qk0 + i * D + c0, qk1 + j * D + c0, dh) / scale;
    /* softmax over j of row i -> m0_i */
    PAR_FOR
    for (i64 i = 0; i < n0; ++i) {
      const double l = log_sum_exp(sim + i * n1, n1, 1);
      for (int d = 0; d < dh; ++d) {
        double acc = 0.0;
        for (i64 j = 0; j < n1; ++j) acc += exp(sim[i * n1 + j] - l) * v1[j * D + c0 + d];
        a0[i * D + c0 + d] = acc;
      }
    }
    /* softmax over i of column j -> m1_j */
    PAR_FOR
    for (i64 j = 0; j < n1; ++j) {
      const double l = log_sum_exp(sim + j, n0, n1);
      for (int d = 0; d < dh; ++d) {
        double acc = 0.0;
        for (i64 i = 0; i < n0; ++i) acc += exp(sim[i * n1 + j] - l) * v0[i * D + c0 + d];
        a1[j * D + c0 + d] = acc;
      }
    }
  }
  orc_linear(a0, n0, D, st->Wm, st->bm, D, m0);
  orc_linear(a1, n1, D, st->Wm, st->bm, D, m1);
  free(qk0);
  free(qk1);
  free(v0);
  free(v1);
  free(a0);
  free(a1);
  free(sim);
}

/* [realcat] "多层GNN" (AttentionalPropagation): the update
   delta_i = W2 ReLU(W1 [x_i || m_i] + b1) + b2 with channels [2D, 2D, D]. */
void orc_update_mlp(const double* x, const double* m, i64 n, int D, const orc_stage* st, double* delta) {
#pragma omp parallel num_threads(orc_threads())
  {
    double* cat = (double*)must_alloc(sizeof(double) * 2 * D);
    double* hid = (double*)must_alloc(sizeof(double) * 2 * D);
#pragma omp for schedule(static)
    for (i64 i = 0; i < n; ++i) {
      memcpy(cat, x + i * D, sizeof(double) * D);
      memcpy(cat + D, m + i * D, sizeof(double) * D);
      for (int o = 0; o < 2 * D; ++o) {
        const double t = dot(st->W1 + (i64)o * 2 * D, cat, 2 * D) + st->b1[o];
        hid[o] = t > 0.0 ? t : 0.0;
      }
      for (int o = 0; o < D; ++o) delta[i * D + o] = dot(st->W2 + (i64)o * 2 * D, hid, 2 * D) + st->b2[o];
    }
    free(cat);
    free(hid);
  }
}

/* [realcat] "多层GNN" (AttentionalGNN), [GNN-blog] "多轮消息怎样回到同一幅图":
   stages alternate self (sources: the image itself) and cross (sources: the
   other image), self first; stage index s = first_stage + position, even s
   = self.  Both images' updates are computed from the states before the
   stage and then added (x <- x + delta).  A cross stage whose W_q is NULL
   is bidirectional ([LightGlue] section 2.3).  thetaA / thetaB (or NULL):
   rotary angles of each image's points, applied in self stages only
   ([LightGlue] section 2.2).  xA [M][D] and xB [N][D] are updated in place. */
void orc_attentional_gnn(double* xA, i64 M, double* xB, i64 N, int D, int H, const orc_stage* stages, int n_stages,
                         int first_stage, const double* thetaA, const double* thetaB) {
  double* mA = (double*)must_alloc(sizeof(double) * M * D);
  double* mB = (double*)must_alloc(sizeof(double) * N * D);
  double* dA = (double*)must_alloc(sizeof(double) * M * D);
  double* dB = (double*)must_alloc(sizeof(double) * N * D);
  for (int t = 0; t < n_stages; ++t) {
    const orc_stage* st = stages + t;
    const int s = first_stage + t;
    if (s % 2 == 1 && st->Wq == NULL) {
      orc_bidirectional_cross_attention(xA, M, xB, N, D, H, st, mA, mB);
    } else if (s % 2 == 0) {
      orc_multi_head_attention(xA, M, xA, M, D, H, st, thetaA, thetaA, mA);
      orc_multi_head_attention(xB, N, xB, N, D, H, st, thetaB, thetaB, mB);
    } else {
      orc_multi_head_attention(xA, M, xB, N, D, H, st, NULL, NULL, mA);
      orc_multi_head_attention(xB, N, xA, M, D, H, st, NULL, NULL, mB);
    }
    orc_update_mlp(xA, mA, M, D, st, dA);
    orc_update_mlp(xB, mB, N, D, st, dB);
    for (i64 i = 0; i < M * D; ++i) xA[i] += dA[i];
    for (i64 i = 0; i < N * D; ++i) xB[i] += dB[i];
  }
  free(mA);
  free(mB);
  free(dA);
  free(dB);
}

/* ------------------------------------------------ scores and transport */

/* [realcat] "匹配得分预测": S_ij = <fA_i, fB_j>; [forward] forward: divided
   by sqrt(descriptor_dim). */
void orc_score_matrix(const double* fA, i64 M, const double* fB, i64 N, int D, double* S) {
  const double scale = sqrt((double)D);
  PAR_FOR
  for (i64 i = 0; i < M; ++i)
    for (i64 j = 0; j < N; ++j) S[i * N + j] = dot(fA + i * D, fB + j * D, D) / scale;
}

/* [realcat] "Sinkhorn Algorithm", the log-domain iteration on the R x C
   matrix Z with log marginals log_mu [R], log_nu [C]: the duals start at
   zero; every iteration first sets each row's dual so that the row's
   log-sum of Z + u + v equals its log marginal,
       u_i = log_mu_i - log sum_j exp(Z_ij + v_j),
   then each column's,
       v_j = log_nu_j - log sum_i exp(Z_ij + u_i).
   Exactly `iters` iterations, no tolerance stop.  Outputs the duals and
   out = Z + u + v (NULL outputs are skipped). */
void orc_log_sinkhorn_iterations(const double* Z, i64 R, i64 C, const double* log_mu, const double* log_nu,
                                 int iters, double* u_out, double* v_out, double* out) {
  double* u = (double*)must_alloc(sizeof(double) * R);
  double* v = (double*)must_alloc(sizeof(double) * C);
  for (i64 i = 0; i < R; ++i) u[i] = 0.0;
  for (i64 j = 0; j < C; ++j) v[j] = 0.0;
  for (int it = 0; it < iters; ++it) {
#pragma omp parallel num_threads(orc_threads())
    {
      double* t = (double*)must_alloc(sizeof(double) * (R > C ? R : C));
#pragma omp for schedule(static)
      for (i64 i = 0; i < R; ++i) {
        for (i64 j = 0; j < C; ++j) t[j] = Z[i * C + j] + v[j];
        u[i] = log_mu[i] - log_sum_exp(t, C, 1);
      }
#pragma omp for schedule(static)
      for (i64 j = 0; j < C; ++j) {
        for (i64 i = 0; i < R; ++i) t[i] = Z[i * C + j] + u[i];
        v[j] = log_nu[j] - log_sum_exp(t, R, 1);
      }
      free(t);
    }
  }
  if (out)
    for (i64 i = 0; i < R; ++i)
      for (i64 j = 0; j < C; ++j) out[i * C + j] = Z[i * C + j] + u[i] + v[j];
  if (u_out) memcpy(u_out, u, sizeof(double) * R);
  if (v_out) memcpy(v_out, v, sizeof(double) * C);
  free(u);
  free(v);
}

/* [realcat] sections "遮挡以及可见性" and "Sinkhorn Algorithm": the M x N
   scores S bordered by a dustbin column, row and corner of score alpha; the
   marginals a = [1 (M times), N] and b = [1 (N times), M], each divided by
   M + N (log a_i - log(M+N)); `iters` log-domain iterations; then the
   division by M + N undone: logP = Z + u + v + log(M+N).  logP is
   (M+1) x (N+1); u, v (or NULL) receive the duals. */
void orc_log_optimal_transport(const double* S, i64 M, i64 N, double alpha, int iters, double* logP, double* u,
                               double* v) {
  const i64 R = M + 1, C = N + 1;
  double* Z = (double*)must_alloc(sizeof(double) * R * C);
  double* lmu = (double*)must_alloc(sizeof(double) * R);
  double* lnu = (double*)must_alloc(sizeof(double) * C);
  for (i64 i = 0; i < R; ++i)
    for (i64 j = 0; j < C; ++j) Z[i * C + j] = (i < M && j < N) ? S[i * N + j] : alpha;
  const double lmn = log((double)(M + N));
  for (i64 i = 0; i < R; ++i) lmu[i] = log(i < M ? 1.0 : (double)N) - lmn;
  for (i64 j = 0; j < C; ++j) lnu[j] = log(j < N ? 1.0 : (double)M) - lmn;
  orc_log_sinkhorn_iterations(Z, R, C, lmu, lnu, iters, u, v, logP);
  for (i64 k = 0; k < R * C; ++k) logP[k] += lmn;
  free(Z);
  free(lmu);
  free(lnu);
}

/* [realcat] "Sinkhorn Algorithm" (the MATLAB demo's loop), a second and
   independent algorithm for the same iteration in the probability domain,
   used only to cross-check the log-domain one: P = exp(Zbar) normalised to
   sum 1, then `iters` times scale every row to sum a_i and every column to
   sum b_j.  No early stop. */
void orc_sinkhorn_knopp_exp(const double* Zbar, i64 R, i64 C, const double* a, const double* b, int iters,
                            double* P) {
  double tot = 0.0;
  for (i64 k = 0; k < R * C; ++k) {
    P[k] = exp(Zbar[k]);
    tot += P[k];
  }
  for (i64 k = 0; k < R * C; ++k) P[k] /= tot;
  for (int it = 0; it < iters; ++it) {
    for (i64 i = 0; i < R; ++i) {
      double s = 0.0;
      for (i64 j = 0; j < C; ++j) s += P[i * C + j];
      for (i64 j = 0; j < C; ++j) P[i * C + j] *= a[i] / s;
    }
    for (i64 j = 0; j < C; ++j) {
      double s = 0.0;
      for (i64 i = 0; i < R; ++i) s += P[i * C + j];
      for (i64 i = 0; i < R; ++i) P[i * C + j] *= b[j] / s;
    }
  }
}

/* [forward] forward, the matches whose score is above match_threshold, on
   the real block of the (M+1) x (N+1) log assignment logP:
     - each row i picks its best column (the first maximum over j < N), each
       column j its best row (the first maximum over i < M);
     - i and j are mutual when each is the other's pick;
     - a mutual row scores exp(logP_ij), a non-mutual one 0;
     - the match is kept when mutual and the score exceeds the threshold,
       decided in log space (logP_ij > log thr for thr > 0; exp never reaches
       0, so a non-positive threshold keeps every mutual pick);
     - a column takes its mutual row's score, and keeps the match when that
       row kept it.  Unmatched entries are -1. */
void orc_extract_matches(const double* logP, i64 M, i64 N, double thr, int32_t* m0, double* s0, int32_t* m1,
                         double* s1) {
  const i64 C = N + 1;
  i64* best_col = (i64*)must_alloc(sizeof(i64) * (M > 0 ? M : 1));
  i64* best_row = (i64*)must_alloc(sizeof(i64) * (N > 0 ? N : 1));
  char* keep = (char*)must_alloc(M > 0 ? M : 1);
  for (i64 i = 0; i < M; ++i) {
    i64 bj = 0;
    for (i64 j = 1; j < N; ++j)
      if (logP[i * C + j] > logP[i * C + bj]) bj = j;
    best_col[i] = bj;
  }
  for (i64 j = 0; j < N; ++j) {
    i64 bi = 0;
    for (i64 i = 1; i < M; ++i)
      if (logP[i * C + j] > logP[bi * C + j]) bi = i;
    best_row[j] = bi;
  }
  for (i64 i = 0; i < M; ++i) {
    const i64 j = best_col[i];
    const int mutual = N > 0 && best_row[j] == i;
    const double lp = N > 0 ? logP[i * C + j] : -INFINITY;
    s0[i] = mutual ? exp(lp) : 0.0;
    keep[i] = (char)(mutual && (thr <= 0.0 || lp > log(thr)));
    m0[i] = keep[i] ? (int32_t)j : -1;
  }
  for (i64 j = 0; j < N; ++j) {
    const i64 i = best_row[j];
    const int mutual = M > 0 && best_col[i] == j;
    s1[j] = mutual ? s0[i] : 0.0;
    m1[j] = (mutual && keep[i]) ? (int32_t)i : -1;
  }
  free(best_col);
  free(best_row);
  free(keep);
}

/* ------------------------------------------------ double-softmax head */

/* log sigma(z) = log(1 / (1 + exp(-z))), written as min(z, 0) -
   log(1 + exp(-|z|)) so that it is finite for every finite z. */
double orc_log_sigmoid(double z) { return (z < 0.0 ? z : 0.0) - log1p(exp(-fabs(z))); }

void orc_log_sigmoid_v(const double* z, i64 n, double* out) {
  for (i64 i = 0; i < n; ++i) out[i] = orc_log_sigmoid(z[i]);
}

/* [LightGlue] section 2.4: the matchability logit z_i = <w, x_i> + b. */
void orc_matchability(const double* x, i64 n, int D, const double* w, double b, double* z) {
  for (i64 i = 0; i < n; ++i) z[i] = dot(w, x + i * D, D) + b;
}

/* [LightGlue] section 2.5: the token confidence c_i = sigma(<w, x_i> + b). */
void orc_token_confidence(const double* x, i64 n, int D, const double* w, double b, double* c) {
  for (i64 i = 0; i < n; ++i) c[i] = exp(orc_log_sigmoid(dot(w, x + i * D, D) + b));
}

/* [LightGlue] section 2.6: lambda_l = 0.8 + 0.1 exp(-4 l / L), clipped to [0, 1]. */
double orc_confidence_threshold(int layer, int n_layers) {
  const double t = 0.8 + 0.1 * exp(-4.0 * layer / n_layers);
  return t < 0.0 ? 0.0 : (t > 1.0 ? 1.0 : t);
}

/* [LightGlue] section 2.4: the (M+1) x (N+1) log assignment.  Real block:
   the log-softmax of S over j (row i) plus the log-softmax of S over i
   (column j) plus log sigma(z0_i) + log sigma(z1_j).  Last column (i < M):
   log sigma(-z0_i); last row (j < N): log sigma(-z1_j); corner 0. */
void orc_double_softmax_assignment(const double* S, i64 M, i64 N, const double* z0, const double* z1, double* out) {
  const i64 C = N + 1;
  double* lr = (double*)must_alloc(sizeof(double) * (M > 0 ? M : 1));
  double* lc = (double*)must_alloc(sizeof(double) * (N > 0 ? N : 1));
  PAR_FOR
  for (i64 i = 0; i < M; ++i) lr[i] = log_sum_exp(S + i * N, N, 1);
  PAR_FOR
  for (i64 j = 0; j < N; ++j) lc[j] = log_sum_exp(S + j, M, N);
  for (i64 i = 0; i < M; ++i) {
    for (i64 j = 0; j < N; ++j)
      out[i * C + j] = (S[i * N + j] - lr[i]) + (S[i * N + j] - lc[j]) + orc_log_sigmoid(z0[i]) +
                       orc_log_sigmoid(z1[j]);
    out[i * C + N] = orc_log_sigmoid(-z0[i]);
  }
  for (i64 j = 0; j < N; ++j) out[M * C + j] = orc_log_sigmoid(-z1[j]);
  out[M * C + N] = 0.0;
  free(lr);
  free(lc);
}
