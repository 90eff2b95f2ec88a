/*
 * sg.h - C ABI of the MI355X (gfx950) SuperGlue matching forward pass.
 *
 * The method: a keypoint encoder MLP over (x, y, c) added to each descriptor,
 * 2L attentional message-passing stages alternating self and cross attention
 * with residual MLP updates, a final linear projection, an inner-product
 * score matrix augmented with a dustbin row and column, log-domain Sinkhorn
 * normalisation, and mutual-argmax match extraction.  Sources (by page title):
 *   "SuperGlue 的注意力图神经网络怎样传递信息" (huluoboge.top blog),
 *   "SuperGlue:Learning Feature Matching with Graph Neural Networks论文阅读"
 *   (realcat.vercel.app notes), "SuperGlue_model_forward_learning"
 *   (SuperGlue_Code_Learning notes).  The optional double-softmax head
 *   (sg_weights.head) follows section 2.4 of "论文解读:LightGlue,让稀疏特征
 *   匹配随难度自适应地快" (vincentqin.tech review of LightGlue).
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers unless marked "host".  All buffers belong
 *    to the caller; the library never frees them.
 *  - Point-major layouts: kpts [n][2] (x, y), conf [n], desc [n][D],
 *    matrices row-major [out][in] (a kernel-1 Conv1d / Linear weight).
 *  - Every call is asynchronous on opts->stream (NULL = default stream):
 *    it validates its arguments on the host, enqueues kernels and returns.
 *    Outputs are valid once the caller synchronises that stream.  No call
 *    copies between host and device or synchronises.
 *  - All validation happens before the first HIP call: on any error nothing
 *    is enqueued and outputs are untouched; sg_last_error() describes it.
 *  - Graph replay: the second call with given shapes, pointers and options
 *    captures its launch sequence into a HIP graph (on a private stream) and
 *    every later identical call replays it on opts->stream (the first one
 *    enqueues its kernels directly).  Calls with
 *    timing events or SG_FLAG_NO_GRAPH, or on a stream being captured by the
 *    caller, enqueue their kernels directly.  Up to 64 graphs are cached.
 *  - Scratch memory: the caller may pass a workspace of at least
 *    sg_workspace_size() bytes; with none, the library keeps one grow-only
 *    buffer per device (allocated on first use, held until process exit).
 *    Calls that share a workspace (or the library's) must not overlap in
 *    time on different streams.
 */
#ifndef SG_H
#define SG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* sg_stream_t; /* identical to hipStream_t */
typedef struct ihipEvent_t* sg_event_t;   /* identical to hipEvent_t  */

typedef enum {
  SG_OK = 0,
  SG_ERR_INVALID_ARG = -1, /* NULL pointer, negative size, bad L/T/D/H ... */
  SG_ERR_UNSUPPORTED = -2, /* shape with no kernel specialisation          */
  SG_ERR_WEIGHTS = -3,     /* weight blob too small / inconsistent config  */
  SG_ERR_WORKSPACE = -4,   /* caller workspace smaller than required       */
  SG_ERR_HIP = -5          /* HIP runtime error (message in sg_last_error) */
} sg_status;

typedef enum { SG_F32 = 0, SG_BF16 = 1 } sg_dtype;

/* Matching head (sg_weights.head).
 * SG_HEAD_SINKHORN: the score matrix with a dustbin row and column of score
 *   alpha, T log-domain Sinkhorn iterations (SuperGlue).
 * SG_HEAD_DOUBLE_SOFTMAX: no iteration (T is ignored): the log assignment is
 *   log_softmax_j(S_ij) + log_softmax_i(S_ij) + log sigmoid(z_A,i) +
 *   log sigmoid(z_B,j) on the real block, log sigmoid(-z_A,i) in the dustbin
 *   column, log sigmoid(-z_B,j) in the dustbin row, 0 in the corner, where
 *   z = <w_z, x> + b_z is the matchability logit of a point's last GNN state
 *   x (section 2.4 of the LightGlue review).  S is the same S = f_A f_B^T /
 *   sqrt(D) as for the Sinkhorn head; extraction is the same mutual argmax
 *   with threshold. */
typedef enum { SG_HEAD_SINKHORN = 0, SG_HEAD_DOUBLE_SOFTMAX = 1 } sg_head;

/* Cross-attention of the odd stages (sg_weights.cross).
 * SG_CROSS_STANDARD: q from the query image, k and v from the other image,
 *   three projections per stage (SuperGlue).
 * SG_CROSS_BIDIRECTIONAL: one shared query/key projection qk = W_qk x + b_qk
 *   and v = W_v x + b_v per image; per head the similarity
 *   qk_A,i . qk_B,j / sqrt(d_h) is shared by both directions: its softmax
 *   over j gives A's messages, its softmax over i gives B's (section 2.3 of
 *   the LightGlue review).  Each direction is evaluated as attention with
 *   the query and key projections tied, which computes the same messages. */
typedef enum { SG_CROSS_STANDARD = 0, SG_CROSS_BIDIRECTIONAL = 1 } sg_cross;

/* Rotary position encoding of the self stages (sg_weights.rope = 1), after
 * section 2.2 of the LightGlue review: inside each head, channel pairs
 * (2k, 2k+1) of q and k (never v, never in cross stages) are rotated by the
 * angle theta_k = <b_k, p>, where p is the point's position normalised as
 * for the encoder and b_k (k < d_h / 2) is a learned 2-D basis stored in
 * the blob.  Every head and every self stage uses the same angles; the
 * (cos, sin) table is computed once per call. */

/* Adaptive depth and width (sg_weights.adaptive = 1, double-softmax head
 * only), after sections 2.6 and 2.7 of the LightGlue review.  A layer is one
 * self stage and one cross stage.  After every layer l but the last, each
 * remaining point gets a confidence c = sigmoid(<w_c,l, x> + b_c,l) and the
 * threshold is lambda_l = 0.8 + 0.1 exp(-4 l / L).  With SG_FLAG_EARLY_EXIT
 * the pass stops when 1 - (remaining points with c < lambda_l) / (M + N)
 * exceeds opts->depth_confidence.  Otherwise, with SG_FLAG_PRUNE, an image
 * with more than opts->prune_min_points remaining points drops the points
 * whose matchability sigmoid(<w_z,l, x> + b_z,l) (layer l's head) is at most
 * 1 - opts->width_confidence, unless (with SG_FLAG_EARLY_EXIT) their
 * confidence is at most lambda_l; an image left without points ends the
 * pass.  The head of the last layer run (W_f,l, w_z,l; the main head for
 * layer L_max - 1) matches the remaining points; pruned points get -1 / 0.
 * Adaptive calls exist for sg_match only.  They read a few counters back
 * after every layer (the device posts them into host-visible memory and the
 * call waits for each post on the host), always run eagerly (never captured
 * into a graph) and are refused on a stream that the caller is capturing. */
#define SG_MAX_ENC 8     /* hidden layers of the keypoint encoder          */
#define SG_MAX_BATCH 64  /* pairs per sg_match_batch call                  */

/*
 * Network description plus a device weight blob.
 *
 * D: descriptor dimension; H: attention heads (D % H == 0; supported head
 * dimensions 16 and 64).  enc[0..n_enc-1]: hidden widths of the keypoint
 * encoder MLP [3, enc..., D] ("特征点Encode" section of the realcat notes;
 * the pages' batch normalisation is folded away).  L_max: self+cross pairs
 * stored (2*L_max stages).  dtype: type of every matrix and bias in the blob
 * and of the GNN's contraction operands (accumulation is always fp32; the
 * residual stream, the encoder, scores and Sinkhorn are always fp32).
 *
 * Blob layout: tensors in the order below, each starting at a 256-byte
 * aligned offset (sg_weights_tensor() enumerates offsets and shapes):
 *   encoder layer i = 0..n_enc: W [w_{i+1}][w_i], b [w_{i+1}]
 *   stage s = 0..2*L_max-1 (even s = self, odd s = cross):
 *     W_qkv [3D][D] (rows: q, then k, then v), b_qkv [3D]
 *       (SG_CROSS_BIDIRECTIONAL cross stages: W_qkv [2D][D], rows qk then v,
 *       b_qkv [2D]),
 *     W_m [D][D], b_m [D]          (merge of the concatenated heads),
 *     W_1 [2D][2D], b_1 [2D]       (columns 0..D-1 multiply x, D..2D-1 m),
 *     W_2 [D][2D], b_2 [D]
 *   W_f [D][D], b_f [D]            (final projection)
 *   alpha: one float32             (dustbin score, always fp32)
 *   SG_HEAD_DOUBLE_SOFTMAX only:
 *   w_z [1][D], b_z [1]            (matchability Linear(D, 1))
 *   rope = 1 only:
 *   B_rot [D/H/2][2]               (rotary basis, always fp32)
 *   adaptive = 1 only, for each layer l = 0..L_max-2:
 *     w_c [1][D], b_c [1]          (token confidence Linear(D, 1))
 *     W_f [D][D], b_f [D], w_z [1][D], b_z [1]   (layer l's matching head)
 * Head h owns channels [h*D/H, (h+1)*D/H) of q, k, v and of the merge input.
 */
typedef struct {
  int32_t D, H;
  int32_t n_enc;
  int32_t enc[SG_MAX_ENC];
  int32_t L_max;
  int32_t dtype;       /* sg_dtype */
  int32_t head;        /* sg_head */
  int32_t cross;       /* sg_cross */
  int32_t rope;        /* 1: rotary encoding in self-attention */
  int32_t adaptive;    /* 1: per-layer confidence and heads (adaptive depth / width) */
  const void* blob;    /* device pointer, caller-owned */
  size_t blob_bytes;
} sg_weights;

/* Optional per-stage / per-kernel timing (hipEvents created by the caller). */
enum {
  SG_EV_START = 0,     /* before the encoder                       */
  SG_EV_ENCODED = 1,   /* after the encoder                        */
  SG_EV_GNN = 2,       /* after the 2L stages                      */
  SG_EV_SCORES = 3,    /* after final projection + score matrix    */
  SG_EV_SINKHORN = 4,  /* after the T iterations (double-softmax head:
                          after its row / column statistics)         */
  SG_EV_END = 5,       /* after extraction (and optional outputs)  */
  SG_N_STAGE_EVENTS = 6
};
enum { /* kernel classes that can be bracketed by kernel_events */
  SG_K_NONE = 0, SG_K_GEMM = 1, SG_K_ATTENTION = 2,
  SG_K_SINKHORN = 3 /* the head's normalisation: Sinkhorn sweeps, or the
                       double-softmax statistics kernel */
};

typedef struct {
  sg_stream_t stream;          /* NULL = default stream */
  void* workspace;             /* NULL = library-owned per-device buffer */
  size_t workspace_bytes;
  float match_threshold;       /* valid match iff mutual and exp(logP) > threshold */
  float image_size[4];         /* wA, hA, wB, hB (pixels); all 0: kpts already normalised */
  int32_t* out_matches1;       /* optional [N] (batch: [B][Npad]) */
  float* out_scores1;          /* optional [N] */
  float* out_desc_A;           /* optional matching descriptors f, [M][D] fp32 */
  float* out_desc_B;           /* optional [N][D] fp32 */
  float* out_logP;             /* optional (M+1) x (N+1) log assignment, fp32 */
  int64_t logP_ld;             /* leading dimension of out_logP (>= N+1)    */
  sg_event_t* stage_events;    /* optional: SG_N_STAGE_EVENTS events, recorded at the boundaries */
  int32_t n_stage_events;
  int32_t timed_kernel;        /* SG_K_* class to bracket with kernel_events */
  sg_event_t* kernel_events;   /* optional: 2 per launch (before, after), in launch order */
  int32_t n_kernel_events;     /* capacity; launches beyond it are not bracketed */
  int32_t* n_kernel_launches;  /* host: receives the number of bracketed launches */
  int32_t flags;               /* SG_FLAG_* */
  /* adaptive calls (SG_FLAG_EARLY_EXIT / SG_FLAG_PRUNE with adaptive weights):
     0 selects the default in brackets */
  float depth_confidence;      /* stop when the confident share exceeds it [0.95] */
  float width_confidence;      /* prune points with matchability <= 1 - it [0.99] */
  int32_t prune_min_points;    /* prune only images with more points [1024] */
  int32_t* out_exit_layer;     /* host, optional: the layer whose head matched */
  int32_t* out_prune0;         /* optional [M]: 1 + pruning steps each point of A survived */
  int32_t* out_prune1;         /* optional [N] */
} sg_opts;

/* sg_opts.flags: run eagerly instead of replaying the captured HIP graph. */
#define SG_FLAG_NO_GRAPH 1
/* sg_opts.flags: Sinkhorn schedule.  By default a call whose score matrices
 * total at most SG_TWO_SWEEP_MAX_BYTES runs two sweeps per iteration (rows
 * of Z, then rows of its transpose, which the score GEMM also writes) and a
 * larger one reads Z once per iteration (row update plus per-block column
 * partials, then a column reduction).  Both compute the same iteration of
 * the page's algorithm; these flags force one schedule (setting both is
 * SG_ERR_INVALID_ARG).  A forced two-sweep schedule above the threshold
 * needs a workspace beyond sg_workspace_size().  The double-softmax head
 * always reads Z and its transpose once and ignores these flags. */
#define SG_FLAG_SINKHORN_TWO_SWEEP 2
#define SG_FLAG_SINKHORN_ONE_SWEEP 4
#define SG_TWO_SWEEP_MAX_BYTES (48u << 20)
/* sg_opts.flags: adaptive depth and width (see sg_weights.adaptive).  In an
 * adaptive call out_logP, out_desc_A and out_desc_B hold the exit layer's
 * values for the remaining points, in the original order; the rows and
 * columns of pruned points are left untouched. */
#define SG_FLAG_EARLY_EXIT 8
#define SG_FLAG_PRUNE 16
/* sg_opts.flags, sg_match and sg_stage_gnn with SG_CROSS_BIDIRECTIONAL
 * weights: every cross stage forms its similarity once per head,
 * sim = qk_A qk_B^T / sqrt(d_h), and takes both directions from it, as
 * section 2.3 of the LightGlue review describes: the similarity and its
 * transpose are written once (fp32), the rows' and columns' log-sum-exp
 * taken from them, and each image's messages read them.  The default forms
 * it once per direction inside the attention kernel (the same values up to
 * rounding).  One pair per call: with sg_match_batch, or combined with the
 * adaptive flags, SG_ERR_UNSUPPORTED; other weights: SG_ERR_INVALID_ARG.
 * Workspace: sg_workspace_size(w, M, N, 1) includes it
 * (H (M N + N M + M + N) floats, rows padded to 4). */
#define SG_FLAG_SHARED_SIMILARITY 32

/* Number of tensors in the blob (the alpha scalar counts as one). */
int32_t sg_weights_count(const sg_weights* w);
/* Offset (bytes), rows and cols of tensor `index` (biases: rows = 1; alpha: 1 x 1). */
sg_status sg_weights_tensor(const sg_weights* w, int32_t index, size_t* offset,
                            int32_t* rows, int32_t* cols);
/* Total blob bytes for this configuration. */
size_t sg_weights_bytes(const sg_weights* w);

/* Workspace bytes for pairs of at most Mmax x Nmax points, `batch` pairs. */
size_t sg_workspace_size(const sg_weights* w, int32_t Mmax, int32_t Nmax, int32_t batch);

/*
 * The whole forward pass for one pair (A: M points, B: N points), using the
 * first L self+cross pairs of the blob and T Sinkhorn iterations.
 * Outputs: out_matches [M] int32 (index into B, or -1), out_scores [M]
 * (exp of the log assignment of a mutual match, else 0).  Optional outputs
 * in opts.  M == 0 or N == 0: matches -1, scores 0, nothing else computed
 * (the forward walk-through of the SuperGlue_Code_Learning notes).
 * kpts: pixels when opts->image_size is set, else already normalised as
 * (kpt - size/2) / (0.7 max(w, h)).  desc: float32 [n][D].
 */
sg_status sg_match(const float* kptsA, const float* descA, const float* confA, int32_t M,
                   const float* kptsB, const float* descB, const float* confB, int32_t N,
                   const sg_weights* weights, int32_t L, int32_t T,
                   int32_t* out_matches, float* out_scores, const sg_opts* opts);

/*
 * B independent pairs in one call: sg_match on every pair (the pass above;
 * the forward walk-through of the SuperGlue_Code_Learning notes), with the
 * pairs' point counts given separately.  Inputs are padded: kptsA [B][Mpad][2],
 * descA [B][Mpad][D], confA [B][Mpad] (B likewise with Npad); M, N are HOST
 * arrays of the true counts (0 <= M[b] <= Mpad).  Padded points are absent
 * from every softmax, from Sinkhorn (whose marginals use the true counts) and
 * from the outputs: each pair's result equals sg_match on the unpadded pair.
 * Outputs: out_matches [B][Mpad], out_scores [B][Mpad]; padded entries are
 * -1 / 0.  opts->out_matches1/out_scores1 are [B][Npad]; out_logP is
 * [B][Mpad+1][logP_ld] with logP_ld >= Npad+1 (entries beyond a pair's
 * (M+1) x (N+1) block are left untouched); out_desc_* are [B][Mpad|Npad][D].
 */
sg_status sg_match_batch(int32_t B, int32_t Mpad, int32_t Npad, const int32_t* M, const int32_t* N,
                         const float* kptsA, const float* descA, const float* confA,
                         const float* kptsB, const float* descB, const float* confB,
                         const sg_weights* weights, int32_t L, int32_t T,
                         int32_t* out_matches, float* out_scores, const sg_opts* opts);

/* ---- stage entry points (same conventions; for per-stage parity and timing) ---- */

/* Encoder (realcat notes, section "特征点Encode": KeypointEncoder adds an
   MLP of (x, y, c) to each descriptor; the keypoints are normalised as in
   the SuperGlue_Code_Learning notes' normalize_keypoints):
   x0 [n][D] fp32 = desc + MLP_enc(normalised kpts, conf), ReLU between the
   layers, none after the last.  image_w/image_h > 0: kpts in pixels; both
   0: already normalised.  kpts [n][2], conf [n], desc [n][D] fp32 inputs;
   x_out [n][D] caller-owned.  n == 0 enqueues nothing. */
sg_status sg_stage_encode(const float* kpts, const float* conf, const float* desc, int32_t n,
                          float image_w, float image_h, const sg_weights* weights,
                          float* x_out, const sg_opts* opts);

/* Stages s0 .. s1-1 of the attentional GNN (realcat notes, sections
   "Attentional Aggregation" and "多层GNN"; the huluoboge.top blog's
   message-passing sections): even stages self, odd stages cross; per stage
   multi-head attention with logits scaled by 1/sqrt(D/H), the merge
   projection, and x += W2 ReLU(W1 [x || m] + b1) + b2 for both images from
   their pre-stage states.  In place on the caller's fp32 states xA [M][D],
   xB [N][D]; 0 <= s0 <= s1 <= 2 L_max (SG_ERR_INVALID_ARG otherwise). */
sg_status sg_stage_gnn(float* xA, int32_t M, float* xB, int32_t N, const sg_weights* weights,
                       int32_t s0, int32_t s1, const sg_opts* opts);

/* As sg_stage_gnn, with the point positions posA [M][2], posB [N][2] that
   rotary self-attention needs (normalised, or pixels when
   opts->image_size is set); they may be NULL for weights without rope.
   sg_stage_gnn is this call with NULL positions. */
sg_status sg_stage_gnn_pos(float* xA, const float* posA, int32_t M, float* xB, const float* posB, int32_t N,
                           const sg_weights* weights, int32_t s0, int32_t s1, const sg_opts* opts);

/* Final projection of the SuperGlue_Code_Learning notes' forward (the
   matching descriptors, realcat notes section "Attentional Aggregation",
   last equation): f [n][D] fp32 = W_f x + b_f from the fp32 states
   x [n][D]; f_out caller-owned. */
sg_status sg_stage_project(const float* x, int32_t n, const sg_weights* weights, float* f_out,
                           const sg_opts* opts);

/*
 * The scores of the optimal-matching layer from the last GNN states xA
 * [M][D], xB [N][D] (fp32, device): the final projection f = W_f x + b_f of
 * both images (realcat notes section "Attentional Aggregation", last
 * equation), the scores S = f_A f_B^T / sqrt(D) (section "匹配得分预测"; the
 * forward notes' scaling) and the dustbin row and column of the network's
 * dustbin score alpha (section "遮挡以及可见性"), written as the bordered
 * (M+1) x (N+1) matrix Z [(M+1)][ldZ] fp32, natural log, caller-owned: the
 * input sg_stage_sinkhorn takes.  M or N may be 0 (only the border is
 * written).  Errors: negative counts, NULL Z or states, ldZ < N+1 ->
 * SG_ERR_INVALID_ARG; M or N above 4096 -> SG_ERR_UNSUPPORTED.  Workspace:
 * sg_stage_scores_workspace_size.
 */
sg_status sg_stage_scores(const float* xA, int32_t M, const float* xB, int32_t N, const sg_weights* weights,
                          float* Z, int64_t ldZ, const sg_opts* opts);

/* Workspace bytes of sg_stage_scores for M x N points of dimension D. */
size_t sg_stage_scores_workspace_size(int32_t M, int32_t N, int32_t D);

/* The optimal-matching layer from matching descriptors fA [M][D], fB [N][D]
   (fp32): scores S = fA fB^T / sqrt(D) (realcat notes section "匹配得分预测";
   the forward notes' scaling), the dustbin row and column of score alpha
   (section "遮挡以及可见性"), T log-domain Sinkhorn iterations (section
   "Sinkhorn Algorithm") and the mutual-argmax extraction of the forward
   notes.  Outputs and options as sg_match; D a positive multiple of 8. */
sg_status sg_stage_match(const float* fA, int32_t M, const float* fB, int32_t N, int32_t D,
                         float alpha, int32_t T, int32_t* out_matches, float* out_scores,
                         const sg_opts* opts);

/* Workspace bytes of sg_stage_match for M x N points of dimension D. */
size_t sg_stage_match_workspace_size(int32_t M, int32_t N, int32_t D);

/* The double-softmax head (SG_HEAD_DOUBLE_SOFTMAX above) from matching
   descriptors fA [M][D], fB [N][D] and last GNN states xA [M][D], xB [N][D]
   (all fp32): S = fA fB^T / sqrt(D), matchability z = x w_z + b_z with w_z a
   DEVICE fp32 [D] vector and b_z a host value, the log assignment and the
   mutual-argmax extraction (section 2.4 of the LightGlue review).  Outputs
   and options as sg_stage_match (out_logP: the (M+1) x (N+1) log
   assignment); D must be a positive multiple of 8. */
sg_status sg_stage_match_ds(const float* fA, const float* xA, int32_t M, const float* fB,
                            const float* xB, int32_t N, int32_t D, const float* w_z, float b_z,
                            int32_t* out_matches, float* out_scores, const sg_opts* opts);

/* Workspace bytes of sg_stage_match_ds for M x N points of dimension D. */
size_t sg_stage_match_ds_workspace_size(int32_t M, int32_t N, int32_t D);

/*
 * The log-domain Sinkhorn iterations of the optimal-matching layer on
 * caller-given couplings (realcat notes, section "Sinkhorn Algorithm":
 * log_optimal_transport / log_sinkhorn_iterations).
 *   Z [(M+1)][ldZ] fp32, natural log: row M and column N are the dustbin
 *     row and column (any values; the pass itself uses the constant alpha).
 *   Marginals: a = [1 (M times), N] and b = [1 (N times), M], each divided
 *     by M + N.  From u = v = 0, T iterations of
 *       u_i = log(a_i / (M+N)) - log sum_j exp(Z_ij + v_j),   i <= M,
 *       v_j = log(b_j / (M+N)) - log sum_i exp(Z_ij + u_i),   j <= N.
 *   Outputs (device, caller-owned): u [M+1], v [N+1] (natural log; T == 0
 *     gives zeros) and, when logP is non-NULL, the log assignment
 *     logP [(M+1)][ldP] = Z + u + v + log(M+N).
 * Runs the pass's own sweep kernels (two per iteration, over Z and its
 * transpose) in fp32 with base-2 exponentials.  Errors: M < 1 or N < 1 (the
 * pages run the layer only on non-empty images), T < 0, NULL Z / u / v,
 * ldZ < N+1 or (with logP) ldP < N+1 -> SG_ERR_INVALID_ARG; M or N above
 * 4096 -> SG_ERR_UNSUPPORTED.  Workspace: sg_stage_sinkhorn_workspace_size.
 */
sg_status sg_stage_sinkhorn(const float* Z, int64_t ldZ, int32_t M, int32_t N, int32_t T, float* u, float* v,
                            float* logP, int64_t ldP, const sg_opts* opts);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments and errors as sg_stage_sinkhorn, enqueued directly
 * on `stream` (never captured into a graph by the library), with its
 * workspace in a fixed 40 MiB device array per GPU instead of an allocation;
 * the call allocates nothing.  Shapes whose workspace
 * (sg_stage_sinkhorn_workspace_size) exceeds 40 MiB -> SG_ERR_UNSUPPORTED
 * (every M, N <= 2048 fits).  All calls on one GPU share the array, which
 * keeps the last call's contents: calls that overlap in time on one GPU
 * (different streams, or host threads) race and must be serialised by the
 * caller.
 */
sg_status sg_stage_sinkhorn_noalloc(const float* Z, int64_t ldZ, int32_t M, int32_t N, int32_t T, float* u,
                                    float* v, float* logP, int64_t ldP, sg_stream_t stream);

/* Workspace bytes of sg_stage_sinkhorn and sg_stage_extract for M x N points. */
size_t sg_stage_sinkhorn_workspace_size(int32_t M, int32_t N);

/*
 * Match extraction from a given log assignment logP [(M+1)][ldP] fp32
 * (natural log), after the SuperGlue_Code_Learning notes' forward ("Get the
 * matches with score above match_threshold"): on the real block, each row's
 * best column and each column's best row (the lowest index among equal
 * maxima); a pair is a match when each is the other's pick and exp(logP) >
 * threshold (decided in log space; threshold <= 0 keeps every mutual pick).
 * Outputs (device, caller-owned): out_matches0 [M] (index into B or -1),
 * out_scores0 [M] (exp(logP) of a mutual pick, else 0); optional
 * out_matches1 / out_scores1 [N] likewise.  M == 0 or N == 0: -1 / 0.
 * Errors: negative counts, NULL required pointers, ldP < N+1 ->
 * SG_ERR_INVALID_ARG; M or N above 4096 -> SG_ERR_UNSUPPORTED.  Workspace:
 * sg_stage_sinkhorn_workspace_size(M, N).
 */
sg_status sg_stage_extract(const float* logP, int64_t ldP, int32_t M, int32_t N, float threshold,
                           int32_t* out_matches0, float* out_scores0, int32_t* out_matches1, float* out_scores1,
                           const sg_opts* opts);

/* Message of the last failing call on this thread ("" if none). */
const char* sg_last_error(void);

/* Library version string. */
const char* sg_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SG_H */
