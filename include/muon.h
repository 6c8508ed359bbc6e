/*
 * muon.h - C ABI of the MI355X (gfx950) per-matrix Muon update library (libmuon_amd.so).
 *
 * What one call computes, per matrix (see the citations at each entry point):
 *   M' = mu*M + G;  U = G + mu*M' (Nesterov) or U = M'
 *   X0 = U / (||U||_F + eps), on the short side (tall matrices are handled as U^T)
 *   quintic Newton-Schulz with coefficients (a, b, c): plain rounds, or the Gram-space
 *   form with segments (default 2+2+1)
 *   W' = W*(1 - lr*wd) - lr*O, with O the NS result in W's orientation
 *
 * Sources: "MuonX" article (Baidu Baige, damodev.csdn.net), sections 2 and 3.2 (Gram NS);
 * "DMuon: Efficient Distributed Muon Training with Near-Adam Overhead" (gist.science
 * summary), technical summary sections 2.2 (Gram NS, symmetric SYRK Gram product,
 * batching of similar shapes) and 2.4 (shape-adaptive kernel choice, cached).
 *
 * Conventions for every entry point:
 *   - every function returns an int status (MUON_OK or a negative MUON_ERR_*) and never
 *     throws, aborts or exits;
 *   - every argument is validated on the host before anything is enqueued: on any error
 *     nothing has been launched and W, M are untouched;
 *   - device pointers are plain device addresses on the context's device; host pointers
 *     are read during the call only;
 *   - the library allocates no device memory: scratch space is the caller's workspace.
 */
#ifndef MUON_AMD_H
#define MUON_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MUON_OK 0
#define MUON_ERR_ARG -1          /* null pointer, bad size, bad hyper-parameter, bad dtype */
#define MUON_ERR_WORKSPACE -2    /* workspace null, too small or misaligned (needs 256 B) */
#define MUON_ERR_DEVICE -3       /* device index invalid or not a gfx950 GPU */
#define MUON_ERR_HIP -4          /* a HIP runtime call or kernel launch failed */
#define MUON_ERR_UNSUPPORTED -5  /* valid request the library does not implement */

/* ---- storage dtypes ---- */
#define MUON_F32 0
#define MUON_BF16 1

/* ---- Newton-Schulz form ---- */
#define MUON_NS_AUTO 0   /* per shape: the dispatcher picks plain or Gram (with the given
                            segments) by cost: the shape's measured stage times once its tiles
                            are measured, else the MuonX article's dense FLOP count */
#define MUON_NS_PLAIN 1  /* sum(segments) plain rounds (segments ignored otherwise) */
#define MUON_NS_GRAM 2   /* Gram-space NS with the given segments */
#define MUON_NS_AUTO_SCHEDULE 3  /* per shape: plain NS or Gram NS with k segments, chosen below */

#define MUON_MAX_SEGMENTS 8

/* ---- muon_init flags ---- */
#define MUON_FLAG_MODEL_ONLY 1u  /* no timed tile tuning: static tile choice only */
#define MUON_FLAG_PROFILE 2u     /* bracket every launch with hipEvents (muon_profile_read) */
#define MUON_FLAG_STAGED_ONLY 4u /* never use the single-workgroup kernel for small matrices */
#define MUON_FLAG_ONE_STREAM 8u  /* run every shape group on the caller's stream, in order */

typedef struct muon_ctx muon_ctx; /* opaque; owned by the library */

/* One 2-D weight. All three arrays are rows x cols, row-major, leading dimension cols,
 * on the context's device, in the dtypes named by muon_hparams. W and M are updated in
 * place; G is read only. Arrays of different matrices must not overlap. rows and cols
 * are each in [1, 2^20] (else MUON_ERR_ARG). A shape whose padded iterate exceeds 4 GiB
 * (past the direct-load tiles' 32-bit offsets) runs on the register-staged tiles. */
typedef struct muon_matrix {
  void *W;
  const void *G;
  void *M;
  int64_t rows;
  int64_t cols;
} muon_matrix;

/* Hyper-parameters of one call (shared by every matrix of the call).
 *   lr, weight_decay:   W' = W*(1 - lr*weight_decay) - lr*O   (lr > 0 not required)
 *   momentum (mu):      0 <= mu < 1
 *   eps:                >= 0, added to the Frobenius norm
 *   nesterov:           0 or 1
 *   a, b, c:            quintic NS coefficients (finite)
 *   n_segments, segments[]: 1..MUON_MAX_SEGMENTS segments, each >= 1; their sum is the
 *                       number of NS rounds (at most 64). With ns_dtype MUON_BF16 a Gram
 *                       segment longer than 3 rounds returns MUON_ERR_UNSUPPORTED: the
 *                       fp16 Gram-space recurrence loses the small singular directions
 *                       of low-rank inputs from the fourth round on.
 *   mode:               MUON_NS_AUTO | MUON_NS_PLAIN | MUON_NS_GRAM | MUON_NS_AUTO_SCHEDULE
 *                       AUTO_SCHEDULE (MuonX article, section 3.2: the best segment split
 *                       depends on shape and precision): every Gram segmentation of the
 *                       R = sum(segments) rounds, like plain NS, reaches the same result in
 *                       exact arithmetic, so per shape the cheapest is run: plain NS or Gram
 *                       NS with k balanced segments (longer ones first, each at most 3
 *                       rounds on the bf16 path). A Gram segment count k costs k SYRK and k
 *                       apply products plus 4R - 3k m'xm' products, plain NS R of each; the
 *                       costs are the measured times of the shape's stages once a step has
 *                       measured its tiles, else the FLOP counts the kernels perform. The
 *                       choice may change once the tiles are measured; the workspace size
 *                       covers the Gram form for every shape, so it does not change.
 *   w_dtype:            MUON_F32 or MUON_BF16
 *   g_dtype, m_dtype:   MUON_F32 or MUON_BF16
 *   ns_dtype:           MUON_BF16: bf16 iterate with fp32-accumulate MFMA, the m'xm'
 *                       recurrence in fp16 (prescaled); MUON_F32: fp32 throughout        */
typedef struct muon_hparams {
  float lr;
  float momentum;
  float weight_decay;
  float eps;
  int32_t nesterov;
  float a, b, c;
  int32_t n_segments;
  int32_t segments[MUON_MAX_SEGMENTS];
  int32_t mode;
  int32_t w_dtype;
  int32_t g_dtype;
  int32_t m_dtype;
  int32_t ns_dtype;
} muon_hparams;

/* Per-matrix plan as chosen by the dispatcher (muon_plan_info). */
typedef struct muon_plan_entry {
  int32_t mode;          /* MUON_NS_PLAIN or MUON_NS_GRAM actually used */
  int32_t n_segments;    /* the schedule used: Gram segments, or the rounds of plain NS as
                            one entry */
  int32_t segments[MUON_MAX_SEGMENTS];
  int32_t transposed;    /* 1 if rows > cols (processed as the transpose) */
  int64_t m, n;          /* canonical short side m' and long side n' */
  int32_t group;         /* same-shape group index (one batched launch per stage) */
  int32_t tile_sym;      /* tile configuration of the m' x m' products (muon_debug_gemm ids):
                            the measured choice once a step has run, else the static one */
  int32_t tile_apply;    /* tile configuration of the apply products, likewise */
  int32_t single_wg;     /* 1: the whole update of each matrix runs in one workgroup of
                            one launch; chosen on the bf16 path when every matrix of the list
                            has m' <= 128 and m' n' <= 65536 after padding to multiples of
                            64 (without MUON_FLAG_STAGED_ONLY); tile_sym and tile_apply are
                            then -1 */
  double dense_flops;    /* matmul FLOPs as the MuonX article counts them (2m'^2n', 2m'^3) */
  double kernel_flops;   /* FLOPs the kernels actually perform (symmetric outputs halved on
                            the staged path; dense in the single-workgroup kernel) */
} muon_plan_entry;

/* Aggregated launch timings of one stage kind, shape and tile (muon_profile_read). */
typedef struct muon_profile_entry {
  char stage[32];        /* "table", "momentum_norm" (first pass over G and M: the partial
                            sums of U^2), "norm_finalize", "momentum" (second pass: M' and
                            the normalised iterate in both layouts), "syrk" (Gram product of
                            the iterate), "square", "apply", "apply_update", "single_wg" */
  int64_t m, n;          /* canonical shape of the group the launches served */
  int32_t count;         /* matrices per launch */
  int32_t launches;      /* launches aggregated */
  int32_t tile;          /* tile configuration of GEMM stages (muon_debug_gemm ids), else -1 */
  int32_t reserved;
  double total_ms;       /* sum of event-measured launch durations */
  double flops;          /* algorithmic FLOPs of those launches (one triangle for
                            symmetric outputs) */
  double bytes;          /* algorithmic HBM bytes (elementwise stages, W in the update) */
} muon_profile_entry;

/* Defaults: lr 0.02, momentum 0.95 Nesterov, wd 0, eps 1e-7, (a, b, c) =
 * (3.4445, -4.7750, 2.0315), segments 2+2+1, mode AUTO, W fp32, G and M bf16, NS bf16. */
void muon_hparams_default(muon_hparams *hp);

/* Context, workspace and status calls (muon_init, muon_workspace_size, muon_destroy,
 * muon_status_str): the pages describe the integration only as naming the participating
 * matrices and replacing the optimizer (MuonX article, section 3.3; DMuon announcement,
 * "three lines of code"); these calls are this library's own interface around it.
 *
 * Create a context on HIP device `device`. The device must be gfx950, else
 * MUON_ERR_DEVICE. device == -1 creates a host-only context (no HIP call is made; it
 * plans for a 256-CU MI355X): muon_workspace_size and muon_plan_info work, muon_step and
 * muon_debug_gemm validate their arguments and then return MUON_ERR_DEVICE.
 * `flags` is 0 or a combination of MUON_FLAG_MODEL_ONLY, MUON_FLAG_PROFILE,
 * MUON_FLAG_STAGED_ONLY and MUON_FLAG_ONE_STREAM. *out receives the context; it is owned by the
 * caller until muon_destroy. No device memory is allocated (the device's copy of the
 * muon_step_static scratch array comes with the library's code, which this call looks up). */
int muon_init(muon_ctx **out, int device, uint32_t flags);

/* Bytes of device workspace muon_step needs for this list and these hyper-parameters
 * (deterministic for a given list of shapes and hparams). Same validation as muon_step
 * except that array pointers may be null. */
int muon_workspace_size(muon_ctx *ctx, const muon_matrix *mats, int count,
                        const muon_hparams *hp, size_t *bytes);

/* One Muon update of `count` matrices (count == 0 is a no-op), enqueued on `stream`
 * (a hipStream_t; null = the default stream). Asynchronous: returns after enqueueing,
 * with no host synchronisation; W, G, M and the workspace must stay valid until the
 * stream work completes. `workspace` is device memory of at least muon_workspace_size
 * bytes, 256-byte aligned, owned by the caller and not used by anything else until the
 * step completes. Each matrix's result equals a separate call for it (grouping only
 * batches launches). Launch failures return MUON_ERR_HIP; device faults surface at the
 * caller's next synchronisation. A context must not be used by two threads at once.
 * Shape-adaptive tiles (DMuon summary, section 2.4: per-shape kernel configurations,
 * measured once and cached): unless the context has MUON_FLAG_MODEL_ONLY, the first
 * step that meets a new (stage, shape, batch) times the candidate tile configurations on
 * its own workspace buffers, synchronising the stream once for it, and caches the
 * fastest for the process; later steps make no host synchronisation.
 * Concurrency: once every shape group of the list has its tiles measured, groups
 * (matrices of one canonical shape) too small to fill the GPU (under 1e11 FLOPs of update)
 * run on up to three streams beside `stream`, which runs the larger groups in order; the
 * extra streams are created by the context on its device at default priority, forked from
 * `stream` and joined back into it with events, so the work still completes in `stream`'s
 * order for the caller (also under stream capture). With MUON_FLAG_PROFILE or
 * MUON_FLAG_ONE_STREAM all launches stay on `stream`. */
int muon_step(muon_ctx *ctx, const muon_matrix *mats, int count, const muon_hparams *hp,
              void *workspace, size_t workspace_bytes, void *stream);

/* Init-time profiling (DMuon summary, section 2.3: at initialisation the time of every
 * distinct matrix shape is measured for several batch sizes and kernel schemes; section
 * 2.4: the chosen kernel configurations are cached and reused): runs the list's update
 * twice on synthetic data held in the workspace, measuring the tile configuration of every
 * stage not measured yet (as muon_step's first call would, but before any training step),
 * then times one more such run on `stream` and stores its duration in *ms (may be null).
 * Synthetic run: the momentum stages are replaced by a seeded iterate of unit Frobenius norm
 * (no G or M traffic) and the last product writes the workspace instead of W (no W
 * traffic), so *ms is the Newton-Schulz part of the step. W, G and M are neither read nor
 * written: their pointers may be null; rows and cols are used. The workspace is as for
 * muon_step (muon_workspace_size bytes). Synchronises the stream; afterwards muon_step on
 * the same shapes makes no host synchronisation and runs independent shape groups
 * concurrently from its first call. Errors as muon_step. */
int muon_prepare(muon_ctx *ctx, const muon_matrix *mats, int count, const muon_hparams *hp,
                 void *workspace, size_t workspace_bytes, void *stream, double *ms);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same update as muon_step, with the
 * scratch space in a library-owned device array of MUON_STATIC_SCRATCH_BYTES instead of a
 * workspace argument. Each GPU the library initialises a context on holds its own copy of
 * the array (reserved when the library's code is loaded on the device, looked up by
 * muon_init) until the process ends. A list whose muon_workspace_size exceeds the array
 * returns MUON_ERR_WORKSPACE before anything is launched. The call allocates nothing and
 * creates no HIP object: it measures no tiles (it uses the choices muon_step measured or
 * loaded for the same shapes, else the static ones), records no profiler events and runs
 * every group on `stream`; the scratch holds nothing that must start at zero. Every call on
 * one GPU shares that GPU's array: calls whose work overlaps on one GPU (on different
 * streams, or from different contexts or threads without ordering) race and corrupt each
 * other's results; calls ordered on one stream do not. Results equal muon_step's bitwise
 * when the tile choices are the same. */
#define MUON_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
int muon_step_static(muon_ctx *ctx, const muon_matrix *mats, int count, const muon_hparams *hp,
                     void *stream);

/* Measured tile choices, shared by every context of the process, to and from a text file,
 * so that another process starts with the same choices instead of measuring again
 * (DMuon summary, section 2.4: per-shape configurations measured once and cached). One
 * choice per line: "stage path padded_m padded_n batch tile ms" (stage: 1 m' x m'
 * product, 2 apply, 4 Gram product of the iterate (0 is the bf16 Gram product that only
 * muon_debug_gemm runs); path: 0 bf16, 1 fp32; tile: as in muon_debug_gemm; ms: the
 * measured time of one launch with that tile, which MUON_NS_AUTO and
 * MUON_NS_AUTO_SCHEDULE use as the stage's cost, negative or absent when unknown).
 * muon_tune_save writes the choices made on the context's device (overwriting the file).
 * muon_tune_load validates the whole file first and then adds its choices for the
 * context's device, replacing choices already held for the same key; *n_loaded (may be
 * null) receives their number. A missing or unreadable file, a malformed line or a tile
 * unavailable for its stage returns MUON_ERR_ARG and changes nothing. Host-only contexts
 * save and load too. */
int muon_tune_save(muon_ctx *ctx, const char *path);
int muon_tune_load(muon_ctx *ctx, const char *path, int *n_loaded);

/* Plan of matrix `index` of the list (host-only; nothing is launched). */
int muon_plan_info(muon_ctx *ctx, const muon_matrix *mats, int count,
                   const muon_hparams *hp, int index, muon_plan_entry *out);

/* Test-only entry point: one GEMM stage of the pipeline on caller buffers, enqueued on
 * `stream`. All products are A B^T with A (M x K) and B (N x K) row-major:
 *   kind 0: C = alpha * A A^T, symmetric (upper tiles computed, mirrored); A is bf16 with
 *           C fp16 (ns_dtype MUON_BF16) or both fp32 (MUON_F32); B is ignored.
 *   kind 1: C = alpha * A B^T + beta * E + gamma * I with symmetric output; A, B, E, C
 *           fp16 (MUON_BF16) or fp32; E (M x N) may be null.
 *   kind 2: v = alpha * A B^T + beta * E^T with E stored N x M (may be null);
 *           C (M x N) = oscale * v and, if C2 is not null, C2 (N x M) = oscale * v^T;
 *           operands and outputs fp16 (MUON_BF16) or fp32.
 * tile selects the workgroup tile configuration (operands staged through registers:
 * 0 = 64x64, 1 = 128x128, 2 = 256x128 (kind 2 only), 3 = 256x256; with direct global->LDS
 * loads: 4 = 64x64, 5 = 128x128, 6 = 256x128 (kind 2 only), 7 = 256x256, 8 = 256x256 with
 * 4 waves, 9 = 64x64 and 10 = 128x128 with two k-groups, 11 = 256x256 with 64-byte K
 * slices, 12 = 128x128 with two k-groups and 64-byte K slices, 13 = 256x192 (kind 2 only),
 * 14 = 256x256 with 4 waves and 64-byte K slices; 2, 3, 6, 7, 8, 11, 13 and 14 not fp32);
 * an unavailable combination returns MUON_ERR_UNSUPPORTED.
 * Leading dimensions equal the column counts; M, N, K must be multiples of 64. */
int muon_debug_gemm(muon_ctx *ctx, int kind, int ns_dtype, int tile, int64_t M, int64_t N,
                    int64_t K, const void *A, const void *B, const void *E, void *C, void *C2,
                    float alpha, float beta, float gamma, float oscale, void *stream);

/* Test-only entry point: one element-wise stage of the pipeline, or the weight update, on a
 * single matrix (W, G, M as in muon_step; hp as in muon_step), enqueued on `stream`:
 *   MUON_STAGE_NORM:    out (device, 1 fp32) = 1 / (||U||_F + eps), U = G + mu (mu M + G)
 *                       (or mu M + G without Nesterov); G and M are only read.
 *   MUON_STAGE_ITERATE: M <- mu M + G, and the normalised iterate times *scale (a power of
 *                       two chosen by the library, 1 on the fp32 path) in the canonical
 *                       orientation: out = scale X0 (Mp x Np row-major) and out2 = its
 *                       transpose (Np x Mp), Mp, Np the canonical sizes rounded up to 64,
 *                       zero outside m' x n'; fp16 for ns_dtype MUON_BF16, else fp32.
 *   MUON_STAGE_UPDATE:  W <- W (1 - lr wd) - lr O with O = Q X, Q = in (Mp x Mp) and out2
 *                       holding scale X^T (Np x Mp) as MUON_STAGE_ITERATE writes it, both in
 *                       the iterate's type; O's canonical m' x n' block goes to W through the
 *                       orientation map (transposed for rows > cols); out must be non-null
 *                       (unused). G and M may be null.
 * The stages run the kernel forms muon_step runs for this matrix alone (G and M over
 * 128 MB take the large-group forms). *scale (host, may be null) receives the iterate's
 * scale. The workspace needs 512 bytes plus 4 per 4096 elements of the matrix (rounded up
 * to 256), 256-byte aligned. Validation
 * as muon_step (MUON_ERR_ARG also for a null operand the stage uses). */
#define MUON_STAGE_NORM 0
#define MUON_STAGE_ITERATE 1
#define MUON_STAGE_UPDATE 2
int muon_debug_stage(muon_ctx *ctx, int stage, const muon_matrix *mat, const muon_hparams *hp,
                     const void *in, void *out, void *out2, float *scale, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Profiler read-out for a context created with MUON_FLAG_PROFILE: waits for the last
 * recorded launch, aggregates all launches recorded since the previous read by (stage,
 * shape, batch, tile) in first-seen order into out[0..capacity), stores the number of entries
 * in *n_out and clears the record. Returns MUON_ERR_ARG when the context was created
 * without the flag or when more than `capacity` entries exist (then *n_out tells how
 * many are needed and the record is cleared). */
int muon_profile_read(muon_ctx *ctx, muon_profile_entry *out, int capacity, int *n_out);

/* Release a context (null is accepted). Work already enqueued is not affected. */
int muon_destroy(muon_ctx *ctx);

/* ---- AdamW for the parameters Muon does not update ----
 * MuonX article, section 2: the hidden 2-D weight matrices go to Muon, embeddings, biases
 * and similar parameters stay with AdamW, which adjusts each element from running
 * averages of the gradient and of its square. Per element, at step t (1-based):
 *   W <- W (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
 *   W <- W - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
 * computed in fp32 (decoupled weight decay, bias-corrected moments). */
typedef struct muon_adamw_tensor {
  void *W;          /* numel elements in w_dtype, updated in place */
  const void *G;    /* numel elements in g_dtype, read only */
  float *m;         /* first moment, fp32, numel elements, updated in place */
  float *v;         /* second moment, fp32, numel elements, updated in place */
  int64_t numel;    /* >= 0; 0 skips the tensor (its pointers may then be null) */
} muon_adamw_tensor;

typedef struct muon_adamw_hparams {
  float lr;            /* finite */
  float beta1, beta2;  /* each in [0, 1) */
  float eps;           /* finite, >= 0 */
  float weight_decay;  /* finite */
  int32_t step;        /* t >= 1, for the bias corrections */
  int32_t w_dtype;     /* MUON_F32 or MUON_BF16 */
  int32_t g_dtype;     /* MUON_F32 or MUON_BF16 */
} muon_adamw_hparams;

/* Defaults: lr 1e-3, betas (0.9, 0.999), eps 1e-8, weight_decay 0.01, step 1, W fp32,
 * G bf16. */
void muon_adamw_hparams_default(muon_adamw_hparams *hp);

/* One AdamW step over `count` tensors (count == 0 is a no-op), enqueued on `stream`
 * (asynchronous, no workspace, no host synchronisation). Arrays must not overlap. Every
 * argument is validated before the first launch (MUON_ERR_ARG: null context or arrays,
 * negative numel, null pointers of a non-empty tensor, hyper-parameters out of range);
 * a host-only context returns MUON_ERR_DEVICE after validation. Launch failures return
 * MUON_ERR_HIP. */
int muon_adamw_step(muon_ctx *ctx, const muon_adamw_tensor *tensors, int count,
                    const muon_adamw_hparams *hp, void *stream);

/* ---- Owner assignment: which rank updates which matrix ----
 * DMuon summary (gist.science), section 2.3 (compute-aware load balancing): the update
 * cost varies strongly with the matrix shape, so each matrix is given one owner rank to
 * minimise the predicted makespan (the largest per-rank load), from the measured time of
 * several batch sizes per distinct shape, by an exact optimisation with a greedy fallback
 * for large search spaces; DMuon announcement (agentren.cn), improvement 3. Host-only: no
 * context and no device are needed.
 *
 * Cost model: a rank owning k matrices of one shape updates them in c(k) ms, read off the
 * shape's measured points (batch[i], ms[i]): c(0) = 0, linear from the origin to the first
 * point and between points, past the last point extended with the last segment's slope
 * (the single point's mean rate when n_points == 1). A rank's load is the sum of c over
 * its shapes. */
#define MUON_MAX_COST_POINTS 16
#define MUON_MAX_PLAN_RANKS 4096
#define MUON_PLAN_GREEDY 1u            /* skip the exact search */
#define MUON_PLAN_DEFAULT_NODES 2000000 /* search nodes when max_nodes == 0 */
typedef struct muon_shape_cost {
  int32_t n_points;                     /* 1..MUON_MAX_COST_POINTS */
  int32_t batch[MUON_MAX_COST_POINTS];  /* strictly increasing batch sizes, each >= 1 */
  double ms[MUON_MAX_COST_POINTS];      /* measured time of one update of batch[i] matrices,
                                           finite, >= 0 */
} muon_shape_cost;

/* Owners for `count` matrices, matrix i being of shape shape_of[i] (0..n_shapes-1), over
 * `ranks` ranks (1..MUON_MAX_PLAN_RANKS). The greedy plan (shapes by decreasing per-matrix
 * cost, each matrix to the rank whose load grows least, then single-matrix moves off the
 * most loaded rank while the makespan drops) starts a branch-and-bound search over the
 * per-shape counts of every rank (skipped with MUON_PLAN_GREEDY) that stops after
 * max_nodes nodes (0: MUON_PLAN_DEFAULT_NODES). Outputs: owner[i] in 0..ranks-1 (the
 * matrices of one shape dealt in list order, each to the rank with the largest share of
 * its count still open); rank_ms[r] (may be null) the predicted load of rank r;
 * *makespan_ms (may be null) the largest of them; *optimal (may be null) 1 when the search
 * completed, so the makespan is the least any assignment reaches under the cost model,
 * else 0. Arrays are host memory. MUON_ERR_ARG on a bad argument (nothing written). */
int muon_owner_plan(const int32_t *shape_of, int count, const muon_shape_cost *shapes, int n_shapes,
                    int ranks, uint32_t flags, int64_t max_nodes, int32_t *owner, double *rank_ms,
                    double *makespan_ms, int32_t *optimal);

/* Static, human-readable text for a status code. */
const char *muon_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MUON_AMD_H */
