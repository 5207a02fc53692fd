/*
 * kdkl.h — C-ABI of libkdkl.so: the fused chunked KL-divergence loss for
 * offline top-K distillation, on one AMD Instinct MI355X (gfx950).
 *
 * Operation. For student hidden states H [N, d] and the output-projection
 * weight W [V, d] (the lm-head), and a cached teacher top-K per position
 * (ids [N, K], logits [N, K]), the loss is
 *
 *     s_i   = (W H_i) / T                        student logits at temperature T
 *     q_i   = softmax(s_i) over all V entries    full-vocabulary student distribution
 *     p_i   = softmax(logits_i / T) over K       teacher top-K, renormalised; zero elsewhere
 *     KL_i  = sum_k p_ik (log p_ik - log q_i[ids_ik])
 *     loss  = (1/N) sum_i KL_i
 *
 * The pages name three mathematically equivalent ways to compute this loss
 * and describe the fused chunked one: per slice of positions, project the
 * hidden states to logits, fold the slice into the running loss and drop it,
 * so the vocabulary x sequence logit grid is never built; the backward pass
 * recomputes each slice's projection [P1 "Making knowledge distillation cheap
 * enough to run at scale", section "Two system changes", fused chunked KL
 * bullet; P4 "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits
 * and a Fused Chunked KL Loss", section 2 "fused chunked KL loss"]. The teacher
 * side is the offline cache of the 100 most likely tokens per position [P1,
 * same section, offline distillation paragraph].
 *
 * Readings where the pages say nothing: forward KL(teacher || student);
 * temperature divides both teacher and student logits, and no T^2 factor is
 * applied; the reduction is the mean over the N positions.
 *
 * Gradient (with upstream scalar g = dL_total/dloss; N counts the kept
 * positions, see "Ignored positions" below):
 *     dZ_i = g / (N T) * (q_i - scatter(ids_i, p_i))     [V]
 *     dH   = dZ W        dW = dZ^T H
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, 16-byte aligned.
 *     H and W share the storage dtype (KDKL_F32 or KDKL_BF16); d must be a
 *     multiple of 8 (bf16) or 4 (fp32).
 *   - The caller owns every buffer, including the workspace sized by
 *     kdkl_workspace_size(). The library allocates no device memory, keeps no
 *     pointer after returning, and enqueues all work on `stream` (a
 *     hipStream_t; NULL = the default stream) without synchronising the host.
 *     Buffers must stay alive until the stream has passed the call.
 *   - Arguments are checked before any HIP call; a failed check returns a
 *     status and touches nothing. A failed launch returns KDKL_ERR_HIP.
 *   - Preconditions not checked: ids of a row distinct and in [0, V). A
 *     repeated id is gathered once per entry (KL_i above, entry by entry) and
 *     the gradient adds its masses. An id outside [0, V) never faults: it
 *     keeps its share of the teacher's softmax over K (so of sum p log p),
 *     but the student has no entry for it: its gathered logit reads as 0,
 *     outside the student's normalisation (its term is p_k (log p_k +
 *     logsumexp_v s_iv)), and it adds nothing to the gradient.
 *   - Ignored positions: a position whose FIRST teacher id is -1 has no
 *     teacher target (padding, packing boundaries). It adds nothing: its
 *     per-row KL is 0, its gradient row (dZ, hence dH) is 0, and the mean
 *     and the gradient scale count only the kept positions. With no kept
 *     position the loss is NaN and every gradient is 0. The rest of an
 *     ignored row's ids and logits are never used. This is a reading: the
 *     pages only mention that sequence packing was studied [P1 "Making
 *     knowledge distillation cheap enough to run at scale", section "The
 *     resulting student model"].
 *   - Results are bitwise reproducible run to run (fixed reduction orders, no
 *     floating-point atomics).
 */
#ifndef KDKL_H
#define KDKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDKL_ABI_VERSION 2
/* Bytes of device workspace kdkl_logits_backward needs (any N, V, K). */
#define KDKL_LOGITS_BWD_WORKSPACE 256
/* Bytes of device workspace kdkl_check_ids needs (any N, V, K). */
#define KDKL_CHECK_IDS_WORKSPACE 16384

typedef enum {
  KDKL_OK = 0,
  KDKL_ERR_NULL = 1,      /* a required pointer is NULL */
  KDKL_ERR_SHAPE = 2,     /* a size is out of range (d, K, chunk, V, N) */
  KDKL_ERR_VALUE = 3,     /* T not finite or T <= 0 */
  KDKL_ERR_DTYPE = 4,     /* dtype is neither KDKL_F32 nor KDKL_BF16 */
  KDKL_ERR_WORKSPACE = 5, /* workspace smaller than kdkl_workspace_size() */
  KDKL_ERR_OVERFLOW = 6,  /* a size product overflows */
  KDKL_ERR_HIP = 7,       /* a HIP launch or runtime call failed */
  KDKL_ERR_ALIGN = 8,     /* a pointer is not 16-byte aligned */
  KDKL_ERR_OPTION = 9     /* a kdkl_options field is out of range or not
                             available for these sizes and dtype */
} kdkl_status;

typedef enum { KDKL_F32 = 0, KDKL_BF16 = 1 } kdkl_dtype;

/* Loss computed by kdkl_forward / kdkl_backward (kdkl_options.loss). */
typedef enum {
  KDKL_LOSS_KL = 0,  /* forward KL(teacher top-K || student), the pages' loss */
  KDKL_LOSS_JSD = 1, /* generalised Jensen-Shannon divergence, weight beta */
  KDKL_LOSS_SKL = 2, /* skew KL(P || alpha P + (1 - alpha) q), alpha = beta */
  KDKL_LOSS_SRKL = 3, /* skew reverse KL(q || alpha q + (1 - alpha) P), alpha = beta */
  KDKL_LOSS_TRKL = 4  /* reverse KL over the teacher's top-K support */
} kdkl_loss;

/* The alternative losses (readings: the pages report ablations on the
 * choice of loss function without naming the losses [P1 "Making knowledge
 * distillation cheap enough to run at scale", section "The resulting student
 * model"]). With P_i the teacher's renormalised top-K probabilities placed
 * on the vocabulary (repeated ids add their mass, ids outside [0, V) have no
 * entry) and q_i the student's softmax(s_i) over all V entries:
 *   KDKL_LOSS_JSD   M_i = beta P_i + (1 - beta) q_i, 0 < beta < 1:
 *                   L_i = beta KL(P_i || M_i) + (1 - beta) KL(q_i || M_i),
 *                   g_iv = (1 - beta) log(q_iv / M_iv);
 *                   beta = 1/2 is the Jensen-Shannon divergence.
 *   KDKL_LOSS_SKL   M_i = alpha P_i + (1 - alpha) q_i, 0 <= alpha < 1:
 *                   L_i = KL(P_i || M_i), g_iv = -(1 - alpha) P_iv / M_iv;
 *                   alpha = 0 is the forward KL (where every id is in range).
 *   KDKL_LOSS_SRKL  M_i = alpha q_i + (1 - alpha) P_i, 0 < alpha <= 1:
 *                   L_i = KL(q_i || M_i),
 *                   g_iv = log(q_iv / M_iv) + 1 - alpha q_iv / M_iv;
 *                   finite although P_i is zero off the top-K.
 * with alpha passed in kdkl_options.beta, and for each of them
 *     loss  = (1/N) sum_i L_i          (row_kl holds L_i)
 *     dZ_iv = g / (N T) q_iv (g_iv - sum_u q_iu g_iu).
 * They run on the same fused products (the vocabulary x sequence grid is
 * never built): the forward's projection epilogue keeps the student's logit
 * at each teacher entry, and the backward forms the support terms in its dZ
 * epilogue from the recomputed logits. Their saved per-position state is
 * two floats, so row_lse is [2, N] for these losses: each position's
 * logsumexp, then sum_v q_iv g_iv. Ignored positions as for the KL. Only the
 * fused calls (kdkl_forward, kdkl_forward_noalloc, kdkl_backward) take
 * them.
 *   KDKL_LOSS_TRKL  the reverse KL over the teacher's top-K support (no
 *                   parameter): with S_i = {v : P_iv > 0} (at most K ids)
 *                   and the student's distribution restricted to S_i and
 *                   renormalised there, qt_iv = exp(s_iv) / sum_{u in S_i}
 *                   exp(s_iu),
 *                   L_i = KL(qt_i || P_i) = sum_{v in S_i} qt_iv log(qt_iv / P_iv)
 *                   (0 for an empty support), loss = (1/N) sum_i L_i, and
 *                   dZ_iv = g / (N T) qt_iv (log(qt_iv / P_iv) - L_i) on S_i,
 *                   0 elsewhere. It needs the student's logits at S_i only:
 *                   the forward forms them as dot products of W's rows with
 *                   H (no projection over the vocabulary); the backward
 *                   forms dZ at S_i the same way, dH from the same rows of
 *                   W, and dW from the entries sorted by id (each row of dW
 *                   summed in position order).
 *                   row_lse is [2, N]: the logsumexp of s_i over S_i (-inf
 *                   for an empty support), then L_i. */

/* Per-call options of the fused calls. NULL, or a zero-filled struct, means
 * the defaults: the loss above and the library's own blocking, which it
 * chooses from the sizes alone (the library reads no environment variable
 * and keeps no setting between calls). The same options must be passed to
 * kdkl_workspace_size, kdkl_forward and kdkl_backward of one problem: the
 * workspace size depends on them. Blocking options never change results
 * beyond floating-point rounding order.
 *   loss             kdkl_loss value.
 *   chunks_per_group 0: the library's choice; n >= 1: take n slices of
 *                    `chunk` positions per launch (both calls); n > 1 needs
 *                    the bf16 main loop (bf16 storage, d a multiple of 64).
 *   vocab_slices     0: the library's choice; n >= 1 (at most 1024): the
 *                    backward covers a group's vocabulary in slices of
 *                    ceil(V/n) rows rounded up to whole tiles (so at most n
 *                    slices; kdkl_plan_info reports the count); its dZ buffer
 *                    holds group rows x one slice, and dW's fp32
 *                    read-modify-write happens once per group and slice.
 *   The library's choice (fields 0) on the bf16 main loop: the largest group
 *   of 16, 8, 4 or 2 chunks (no more than there are) that has a vocabulary
 *   slicing whose dZ buffer stays within 4 GiB and whose slices give the dW
 *   product whole rounds of workgroups (at least one per compute unit, 95%
 *   full), with its fewest slices; else one chunk at a time. It depends on
 *   the sizes only, and on N only while there are fewer than 16 chunks; the
 *   fp32 / generic path takes one chunk and the whole vocabulary. A set
 *   field is kept and the other chosen around it. Smaller groups and more
 *   slices trade speed for memory (e.g. chunks_per_group 4, vocab_slices 4
 *   on the 256K gpt-oss-like workload: 2.2 GiB less, about 2% slower).
 *   dh_w_in_place    0: the library's choice; 1: the dH product reads W in
 *                    place (no V x d transposed copy in the workspace; needs
 *                    the bf16 main loop); 2: it reads a W^T copy written once
 *                    per backward call.
 *   beta             parameter of the loss, where it has one (ignored
 *                    otherwise): the JSD's weight, 0 < beta < 1; the skew
 *                    losses' alpha, 0 <= alpha < 1 (KDKL_LOSS_SKL) or
 *                    0 < alpha <= 1 (KDKL_LOSS_SRKL).
 *   reserved         must be zero. */
typedef struct {
  int32_t loss;
  int32_t chunks_per_group;
  int32_t vocab_slices;
  int32_t dh_w_in_place;
  float beta;
  int32_t reserved[3];
} kdkl_options;

/* The blocking the fused calls use for given sizes and options
 * (kdkl_plan_info). */
typedef struct {
  int32_t chunks_per_group; /* slices of `chunk` positions per launch */
  int32_t vocab_slices;     /* vocabulary slices per group in the backward */
  int32_t dh_splits;        /* split-K count of the dH product per launch */
  int32_t dh_w_in_place;    /* 1: dH reads W in place; 0: a W^T copy */
  int32_t vocab_tile;       /* vocabulary rows per workgroup of the projections */
  int32_t hidden_tile;      /* hidden-size columns per workgroup of dH and dW */
  int32_t bf16_main_loop;   /* 1: the bf16 main loop; 0: the generic one */
  int32_t reserved;
  uint64_t fwd_bytes;       /* = kdkl_workspace_size's *fwd_bytes */
  uint64_t bwd_bytes;       /* = kdkl_workspace_size's *bwd_bytes */
} kdkl_plan;

/* Version of this ABI (KDKL_ABI_VERSION). */
int kdkl_abi_version(void);

/* Human-readable name of a status; static storage, never NULL. */
const char* kdkl_status_string(int status);

/* Bytes of device workspace needed by kdkl_forward (*fwd_bytes) and by
 * kdkl_backward (*bwd_bytes) for these sizes and options (NULL: defaults).
 * Either output may be NULL. Host-only; the same validation as the compute
 * calls. On the bf16 path the backward workspace may hold a transposed copy
 * of W (V * d elements) for the dH product: by default the library keeps it
 * only where the time it saves over reading W in place is worth it (at least
 * about 0.3 ms per call by the library's model: at the gpt-oss-like head,
 * d = 2880 and V = 201088 with chunks of 2048, from N = 16385 on), so the
 * backward workspace steps up by that copy at one N; dh_w_in_place selects
 * either layout explicitly. The default group of chunks (and with it the
 * dZ buffer and the forward's per-group products) also grows with N until
 * N spans 16 chunks, then stays fixed (see kdkl_options). */
kdkl_status kdkl_workspace_size(int64_t N, int64_t d, int64_t V, int32_t K,
                                int64_t chunk, int dtype, const kdkl_options* opts,
                                size_t* fwd_bytes, size_t* bwd_bytes);

/* The blocking the calls will use for these sizes and options (host-only,
 * the same validation as kdkl_workspace_size), written to *out (not NULL).
 * The blocking never changes the results beyond rounding order; it is
 * reported so that callers and tests can tell which launch shapes a size
 * exercises. The slices themselves are the chunks over positions that the
 * loss is computed in [P1 "Making knowledge distillation cheap enough to
 * run at scale", section "Two system changes", fused chunked KL bullet]. */
kdkl_status kdkl_plan_info(int64_t N, int64_t d, int64_t V, int32_t K,
                           int64_t chunk, int dtype, const kdkl_options* opts,
                           kdkl_plan* out);

/* Forward pass of the fused chunked KL loss.
 *   H [N, d] dtype, W [V, d] dtype, topk_ids [N, K] int32, topk_logits
 *   [N, K] fp32; T > 0; chunk = positions per slice (>= 1; the last slice may
 *   be short); 1 <= K <= min(V, 1024); opts as for kdkl_workspace_size.
 * Outputs (device): loss [1] fp32 (mean KL over kept positions; NaN when
 *   none, e.g. N == 0),
 *   row_lse [N] fp32 = logsumexp_v(s_iv) (keep it for kdkl_backward; [2, N]
 *     for the alternative losses, see above),
 *   row_kl [N] fp32 per-position KL, or NULL if not wanted.
 * Workspace: >= *fwd_bytes from kdkl_workspace_size. */
kdkl_status kdkl_forward(const void* H, const void* W,
                         const int32_t* topk_ids, const float* topk_logits,
                         int64_t N, int64_t d, int64_t V, int32_t K,
                         float T, int64_t chunk, int dtype, const kdkl_options* opts,
                         float* loss, float* row_lse, float* row_kl,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- allocation-free forward ------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving or evaluation loops, harnesses that forbid
 * allocation. kdkl_forward_noalloc computes what kdkl_forward computes (the
 * same arguments and outputs, bit for bit equal results) without a workspace
 * argument: its scratch is a static device array of
 * KDKL_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds from
 * the library's load until the process ends. Its address is looked up on
 * the first call on each device (no allocation). row_kl is required (not
 * NULL). Where the library chooses the blocking (opts NULL or
 * chunks_per_group 0), it takes fewer chunks per launch until the forward's
 * scratch fits the array; sizes whose scratch does not fit even one chunk at
 * a time (or at the chunks per group the options fix) return
 * KDKL_ERR_WORKSPACE before any HIP call. Every call on one GPU uses that
 * GPU's one array, which keeps the last call's contents (the forward clears
 * nothing it needs: every region is written before it is read): calls that
 * overlap on one GPU, from several streams or threads, race and must be
 * serialised by the caller. The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine. */
#define KDKL_NOALLOC_SCRATCH_BYTES (64u << 20)
kdkl_status kdkl_forward_noalloc(const void* H, const void* W,
                                 const int32_t* topk_ids, const float* topk_logits,
                                 int64_t N, int64_t d, int64_t V, int32_t K,
                                 float T, int64_t chunk, int dtype, const kdkl_options* opts,
                                 float* loss, float* row_lse, float* row_kl, void* stream);

/* Backward pass: recomputes each slice's logits and writes
 *   dH [N, d] in the storage dtype, dW [V, d] fp32.
 * row_lse is the forward's output for the same inputs and options. grad_loss is a device
 * pointer to the upstream scalar g (NULL means g = 1). accumulate_dW != 0
 * adds into dW instead of overwriting it (gradient accumulation across
 * micro-batches). Workspace: >= *bwd_bytes from kdkl_workspace_size. */
kdkl_status kdkl_backward(const void* H, const void* W,
                          const int32_t* topk_ids, const float* topk_logits,
                          int64_t N, int64_t d, int64_t V, int32_t K,
                          float T, int64_t chunk, int dtype, const kdkl_options* opts,
                          const float* row_lse, const float* grad_loss,
                          void* dH, float* dW, int accumulate_dW,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- forward-chunked KL: the student's logit grid is given ----------------
 * The pages' middle variant: the teacher stays sparse (its cached top-K per
 * position), the loss is computed slice by slice over positions, and the
 * student's own logits Z [N, V] are computed in full by the output layer and
 * kept for the backward pass [P1 "Making knowledge distillation cheap enough
 * to run at scale", section "Two system changes", forward-chunked KL bullet].
 * Same loss, readings and id conventions as kdkl_forward with z_i = Z_i; the
 * caller's output layer turns dZ into its own gradients. Both calls stream Z
 * once (bound by HBM bandwidth); rows are processed independently, so no
 * chunk size and no workspace are needed.
 *
 * kdkl_logits_forward:
 *   Z [N, V] dtype (row-major, 16-byte aligned base; any V >= 1),
 *   topk_ids [N, K] int32, topk_logits [N, K] fp32, 1 <= K <= min(V, 1024),
 *   T > 0. Outputs (device): loss [1] fp32 (mean KL over kept positions,
 *   NaN when none),
 *   row_lse [N] = logsumexp_v(Z_iv / T) (keep it for the backward),
 *   row_kl [N] per-position KL (required: the loss is reduced from it). */
kdkl_status kdkl_logits_forward(const void* Z, const int32_t* topk_ids,
                                const float* topk_logits, int64_t N, int64_t V,
                                int32_t K, float T, int dtype, float* loss,
                                float* row_lse, float* row_kl, void* stream);
/* kdkl_logits_backward: writes dZ [N, V] in Z's dtype,
 *   dZ_i = g / (N_kept T) * (softmax(Z_i / T) - scatter(ids_i, p_i))
 * (zero rows for ignored positions), with g read from the device scalar
 * grad_loss (NULL means 1) and row_lse the forward's output for the same
 * inputs. dZ may be Z itself (the gradient then overwrites the logits in
 * place); otherwise the two must not overlap. dZ and the workspace (at least
 * KDKL_LOGITS_BWD_WORKSPACE bytes, caller-owned) must be 16-byte aligned. */
kdkl_status kdkl_logits_backward(const void* Z, const int32_t* topk_ids,
                                 const float* topk_logits, int64_t N, int64_t V,
                                 int32_t K, float T, int dtype,
                                 const float* row_lse, const float* grad_loss,
                                 void* dZ, void* workspace, size_t workspace_bytes,
                                 void* stream);
/* ---- dense KL: the pages' correctness baseline ------------------------------
 * The textbook computation the pages use as their correctness baseline: the
 * full teacher probability grid is rebuilt from the cached top-K (zero
 * elsewhere) and compared with the student's full log-probability grid; both
 * vocabulary x position grids are kept for the backward pass [P1 "Making
 * knowledge distillation cheap enough to run at scale", section "Two system
 * changes", dense KL bullet]. Same loss, gradient and conventions as
 * kdkl_forward / kdkl_backward; what differs is memory: the caller owns a
 * `saved` buffer holding both grids in fp32 (about 8 N V bytes), plus one
 * logit grid of workspace in each call. Useful to reproduce the pages'
 * memory comparison, not for training.
 *
 * kdkl_dense_sizes: bytes of the forward workspace, of the saved grids
 *   (written by the forward, read by the backward) and of the backward
 *   workspace. Host-only. */
kdkl_status kdkl_dense_sizes(int64_t N, int64_t d, int64_t V, int32_t K, int dtype,
                             size_t* fwd_bytes, size_t* saved_bytes, size_t* bwd_bytes);
/* kdkl_dense_forward: arguments and outputs as kdkl_forward (no chunk);
 * fills `saved` (>= *saved_bytes, 16-byte aligned) for the backward. */
kdkl_status kdkl_dense_forward(const void* H, const void* W,
                               const int32_t* topk_ids, const float* topk_logits,
                               int64_t N, int64_t d, int64_t V, int32_t K, float T,
                               int dtype, float* loss, float* row_lse, float* row_kl,
                               void* saved, size_t saved_bytes,
                               void* workspace, size_t workspace_bytes, void* stream);
/* kdkl_dense_backward: as kdkl_backward, from the grids the forward saved. */
kdkl_status kdkl_dense_backward(const void* H, const void* W,
                                const int32_t* topk_ids, const float* topk_logits,
                                int64_t N, int64_t d, int64_t V, int32_t K, float T,
                                int dtype, const void* saved, size_t saved_bytes,
                                const float* grad_loss, void* dH, float* dW,
                                int accumulate_dW, void* workspace,
                                size_t workspace_bytes, void* stream);
/* ---- optional validation of the teacher ids --------------------------------
 * kdkl_check_ids: counts, over the kept positions (first id not -1), the ids
 * outside [0, V) and the positions holding some id more than once, and writes
 * them to counts[0] and counts[1] (int64, DEVICE memory). The loss does not
 * need this: it drops out-of-range ids and adds the mass of repeated ones
 * (see the preconditions above); the check tells a caller whether its cache
 * breaks the pages' setting of K distinct in-vocabulary ids per position.
 * The workspace (>= KDKL_CHECK_IDS_WORKSPACE bytes, caller-owned) and counts
 * must be 8-byte aligned. K in [1, 1024]; N = 0 writes zero counts. Enqueued
 * on `stream`, deterministic; the host reads the counts after synchronising. */
kdkl_status kdkl_check_ids(const int32_t* topk_ids, int64_t N, int32_t K, int64_t V,
                           int64_t* counts, void* workspace, size_t workspace_bytes,
                           void* stream);
/* ---- measurement aid: per-kernel timing with HIP events ------------------
 * Between kdkl_profile_begin() and kdkl_profile_end(), every kernel launched
 * by the compute calls is bracketed by two HIP events recorded on
 * the launch stream. kdkl_profile_end() waits for those events and returns,
 * per kernel name, the launch count, the summed event time and the summed
 * algorithmic work (flop and HBM bytes by the formulas the library states for
 * each kernel). The timing table is the library's only process-wide mutable
 * state besides kdkl_forward_noalloc's scratch (and its per-device address,
 * set once): one table for the process, guarded by a lock (a compute call
 * on another thread while profiling is switched on or off is timed or not,
 * never torn). It creates HIP events but allocates no device buffers. */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
  double flops;  /* algorithmic floating-point operations, summed */
  double bytes;  /* algorithmic HBM bytes, summed */
} kdkl_kernel_stat;

kdkl_status kdkl_profile_begin(void);
/* Fills up to `capacity` entries of `out`, stores the number of kernel names
 * seen in *count, and stops profiling. */
kdkl_status kdkl_profile_end(kdkl_kernel_stat* out, int capacity, int* count);

#ifdef __cplusplus
}
#endif

#endif /* KDKL_H */
