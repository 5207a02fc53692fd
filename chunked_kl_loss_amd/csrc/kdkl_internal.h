// Internal interface between the C-ABI layer (kdkl_api.hip) and the device
// kernels (kdkl_kernels.hip). Host-side declarations only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kdkl {

// Tile of the vocabulary handled by one workgroup of the projection GEMMs
// (the forward and dZ products): 256 rows, or 384 on the bf16 main loop (see
// gemm_vocab_tile). The teacher preparation builds its per-tile index with
// the same width.
constexpr int kVocabTile = 256;
// Token-axis tile of the projection GEMMs; chunk buffers are padded to it.
constexpr int kTokenTile = 256;

enum KernelId {
  K_TEACHER = 0,
  K_FWD_GEMM,
  K_MERGE,
  K_LOSS,
  K_TRANSPOSE_W,
  K_TRANSPOSE_H,
  K_DZ_GEMM,
  K_DH_GEMM,
  K_DH_REDUCE,
  K_DW_GEMM,
  K_LOGITS_FWD,
  K_LOGITS_BWD,
  K_GRAD_SCALE,
  K_DENSE_GEMM,
  K_DENSE_STUDENT,
  K_DENSE_TEACHER,
  K_DENSE_KL,
  K_DENSE_GRAD,
  K_JSD_MERGE,
  K_JSD_PREP,
  K_TOPK_RKL,
  K_TOPK_DW,
  K_COUNT
};

const char* kernel_name(int id);

// One slice ("chunk") of positions [r0, r0 + rows).
struct TeacherArgs {
  const int32_t* ids;     // [N, K] (whole problem)
  const float* logits;    // [N, K]
  int64_t r0;
  int rows;
  int K;
  float inv_T;
  int vt;                 // rows per vocabulary tile
  int n_vt;               // vocabulary tiles (ceil(V / vt))
  int64_t Cp;             // padded chunk capacity (row pitch of tstart)
  int2* ent;              // [Cp, K]   (id, bits of its teacher probability), ids ascending
  float* erow;            // [Cp]      sum_k p log p
  float* keep;            // [Cp]      1 for a kept position, 0 for an ignored one (first id -1)
  uint16_t* tstart;       // [n_vt + 1, Cp] first sorted index >= tile start
};

struct GemmArgs {
  const void* A;  int64_t lda;   // [M, K] rows of A, K contiguous
  const void* B;  int64_t ldb;   // [N, K] rows of B, K contiguous
  int M, N;                      // valid rows of A / of B
  int64_t k_end;                 // K extent (multiple of 16 bytes of elements)
  int64_t k_split;               // K per split (multiple of the k-step)
  int tiles_m, tiles_n, splits;
  // projection epilogues (A = W rows = vocabulary, B = H rows = tokens)
  float inv_T;
  int V;                         // valid A rows (vocabulary rows of this launch; rows >= V are padding)
  int v0;                        // vocabulary row of A's first row (a slice of W in the backward)
  int tm0;                       // its vocabulary tile: v0 / vocabulary tile
  int K;                         // teacher top-K
  int64_t Cp;                    // token capacity: row pitch of tstart, dz_vc and the dH partials
  int n_vt;
  const int2* ent;               // [Cp, K] teacher entries (id, bits of p), ids ascending per row
  const uint16_t* tstart;
  float4* part;                  // forward: [Cp, n_vt] (max, sumexp, gamma, -)
  float* sk;                     // forward, alternative losses: s = z / T at each sorted teacher entry [Cp, K] (else NULL)
  const float* row_lse;          // backward: lse of this chunk's rows
  const float* scale;            // backward: device scalar g / (N_kept * T)
  const float* keep;             // backward: keep flags of this chunk's rows [Cp]
  const float* rowcoef;          // backward, alternative losses: per-row coefficient of q in dZ [Cp] (else scale[0])
  float beta;                    // EPI_DZJ: the loss's parameter (JSD beta, skew alpha); the entries hold P per id
  int alt;                       // EPI_DZJ: which alternative loss (kdkl_loss value)
  int raw;                       // EPI_DZ only: store the logits z themselves (dense path)
  void* dz_cv;                   // [Cp, Vp]
  void* dz_vc;                   // [Vp, Cp]
  int64_t Vp;                    // row pitch of dz_cv (vocabulary columns held)
  // dH split-K partials [splits, Cp, d] and dW [V, d]
  float* out;
  int64_t ldo;
  int accumulate;
  // Operand layouts of the bf16 main loop: LAYOUT_KC = rows along the
  // output axis with K contiguous; LAYOUT_MC = rows along K with the output
  // axis contiguous (fragments through the LDS transpose read). For MC, the
  // operand has *_krows valid rows and *_mcols valid columns; reads past
  // them are clamped (their products are zero or masked).
  int a_layout, b_layout;
  int bn;                        // N-tile width: 256 (or 0), or 320 for dH / dW (see gemm_d_tile)
  int bm;                        // M-tile height: 256 (or 0), or 384 for the forward / dZ products (see gemm_vocab_tile)
  int64_t a_krows, a_mcols, b_krows, b_mcols;
};

enum { LAYOUT_KC = 0, LAYOUT_MC = 1 };

// True when the bf16 main loop (direct-to-LDS loads, no zero fill) serves
// the projections: bf16 storage, d a multiple of the 64-element k-step, and
// every operand's leading dimension (d, padded V, padded chunk) small enough
// for 32-bit load offsets within a tile.
bool gemm_fast_path(int dtype, int64_t d, int64_t Vp, int64_t Cp);
// N-tile width of the products whose N axis is the hidden size d (dH, dW):
// 320 on the fast path when it pads d less than 256 does, else 256.
int gemm_d_tile(bool fast, int64_t d);
// Vocabulary tile (M-tile height) of the forward and dZ products for V rows
// and `token_tiles` 256-wide token tiles per launch: 384 on the bf16 main loop
// when that takes fewer workgroup rounds' time (a 384 x 256 tile reads fewer
// operand bytes through LDS per flop than 256 x 256), else 256.
int gemm_vocab_tile(bool fast, int64_t V, int64_t token_tiles);

struct MergeArgs {
  const float4* part;   // [Cp, n_vt]
  int n_vt;
  int rows;
  const float* erow;
  const float* keep;    // [Cp] keep flags
  float* row_lse;       // chunk-offset
  float* row_kl;        // chunk-offset
};

// The alternative losses, numbered as kdkl_loss (the C-ABI checks the match).
enum AltLoss { ALT_JSD = 1, ALT_SKL = 2, ALT_SRKL = 3 };

// The alternative losses (generalised Jensen-Shannon divergence, skew KL,
// skew reverse KL): one wavefront per position of a group of rows.
struct JsdArgs {
  int64_t V;
  int rows, K;
  int loss;                 // kdkl_loss value (one of the alternative losses)
  float beta;               // the loss's parameter (JSD beta, skew alpha)
  float log_beta, log_omb;  // log(beta), log(1 - beta) (-inf at 0)
  int2* ent;             // [Cp, K] sorted teacher entries (id, bits of p); jsd_prep writes .y
  const float* sk;       // forward: [Cp, K] s = z / T at each sorted entry (from the epilogue)
  const float* keep;     // [Cp]
  const float4* part;    // forward: split-vocabulary partials [Cp, n_vt]
  int n_vt;
  float* row_lse;        // forward outputs (group-offset): logsumexp, JSD, gbar
  float* row_kl;
  float* row_gbar;
  const float* row_gbar_in;  // backward: the forward's gbar (group-offset)
  const float* scale;    // backward: device scalar g / (N_kept T)
  float* rowcoef;        // backward: [Cp] coefficient of q in dZ
};
hipError_t launch_jsd_merge(const JsdArgs& a, hipStream_t s);
hipError_t launch_jsd_prep(const JsdArgs& a, hipStream_t s);

// The reverse KL over the teacher's top-K support. Per position, the support
// is the first sorted entry of each teacher id in [0, V) with teacher mass
// (the masses of repeated ids added); the student's logits there are dot
// products of W's rows with the position's H (no vocabulary-wide work).
// Forward: their logsumexp and the loss per position. Backward: the loss's
// gradient g / (N_kept T) dTRKL/ds at each support entry (0 at every other
// sorted entry), from the forward's logsumexp and loss, and dH = dZ W over
// those entries (each position's row by its own wavefront, in entry order).
struct TopkArgs {
  const void* H;      // [rows, d] storage dtype, the group's first position
  const void* W;      // [V, d]
  int64_t V, d;
  int rows, K;
  float inv_T;
  const int2* ent;    // [Cp, K] sorted teacher entries (id, bits of p)
  const float* keep;  // [Cp]
  float* row_lse;     // forward out, backward in (group-offset): logsumexp of s over the support
  float* row_loss;    // forward out, backward in (group-offset): the loss per position
  float* row_kl;      // forward out (group-offset): the loss, 0 at ignored positions
  const float* scale; // backward: device scalar g / (N_kept T)
  float* dz;          // backward out: [Cp, K] per sorted entry
  void* dH;           // backward out: [rows, d] storage dtype (group-offset), sum_k dz_k W[id_k]
};
hipError_t launch_topk_rkl(int dtype, const TopkArgs& a, bool backward, hipStream_t s);
// whether the backward reads each support row of W once (rows of at most 6
// 16-byte vectors per lane: d <= 3072 in bf16, 1536 in fp32) or twice
inline bool topk_rkl_one_pass(int dtype, int64_t d) { return d / (dtype == 1 ? 8 : 4) <= 64 * 6; }
// dW (+)= the reverse KL's dZ^T H for one group of `rows` positions, from the
// entry gradients dz [rows, K] at the sorted entries `ent`, without a dense
// product: the nonzero entries sorted by id in position order, then each id's
// entries summed in order by one workgroup per run of 1024 (a bucket of
// several runs through fp32 partial rows added in run order); unless
// accumulating, each row of dW is written rather than added to (zeros for
// the ids without entries). Workspace: cnt (trkl_count_bytes), scans
// (trkl_scan_bytes), list [rows K] int2, part (trkl_part_bytes).
inline int64_t trkl_count_bytes(int64_t rows, int64_t V) {
  const int64_t nb = (rows + 255) / 256;  // positions per counting block: 256
  return (nb * V * 4 + 15) / 16 * 16;
}
inline int64_t trkl_scan_bytes(int64_t V, int64_t entries) {
  // five int64 arrays of V + 1 and four of the 256-id tiles' sums, then the
  // id of each run of 1024 entries (at most V + entries / 1024) and of each
  // bucket of several runs (at most entries / 1024), int32
  const int64_t tables = (V + 2 * (entries / 1024) + 2) * 4;
  return (5 * (V + 1) + 4 * ((V + 255) / 256)) * 8 + (tables + 15) / 16 * 16;
}
inline int64_t trkl_part_bytes(int64_t entries, int64_t d) {
  // buckets of more than one run of 1024 entries hold at most 2 entries / 1024 runs
  return (2 * (entries / 1024) + 1) * d * 4;
}
hipError_t launch_trkl_dw(int dtype, const int2* ent, const float* dz, int rows, int K, int64_t V,
                          const void* H, int64_t d, float* dW, bool accumulate, int* cnt, int64_t* scans,
                          int2* list, float* part, hipStream_t s);

hipError_t launch_teacher(const TeacherArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
// Ignored positions: the first teacher id of the row is kIgnoreId.
constexpr int32_t kIgnoreId = -1;
// loss = sum_i KL_i / (number of kept positions), fixed order; NaN if none.
hipError_t launch_loss(const float* row_kl, const int32_t* ids, int K, int64_t N, float* loss,
                       hipStream_t s);
// out[0] = g / (N_kept T) with g = grad[0] (1 if grad is NULL); 0 if none kept.
hipError_t launch_grad_scale(const int32_t* ids, int K, int64_t N, const float* grad, float T,
                             float* out, hipStream_t s);
// The same two reductions in two deterministic stages (many workgroups, then
// one), with kReduceBytes of workspace `part` (16-byte aligned).
constexpr int kReduceBlocks = 512;
constexpr size_t kReduceBytes = (size_t)kReduceBlocks * 16;
hipError_t launch_loss_ws(const float* row_kl, const int32_t* ids, int K, int64_t N, void* part, float* loss,
                          hipStream_t s);
hipError_t launch_grad_scale_ws(const int32_t* ids, int K, int64_t N, const float* grad, float T, void* part,
                                float* out, hipStream_t s);
// out[c, r] = in[r, c] for r < R, 0 for R <= r < Rp; c < C.
hipError_t launch_transpose(int elem_bytes, const void* in, int64_t R, int64_t C,
                            int64_t ldi, void* out, int64_t Rp, int64_t ldo,
                            hipStream_t s);
hipError_t launch_zero(float* p, int64_t n, hipStream_t s);
// Teacher-id validation (kdkl_check_ids): at most kCheckIdsMaxBlocks blocks
// write two int64 partial counts each into `partial`, then one block sums
// them in a fixed order into out[0..1].
constexpr int kCheckIdsMaxBlocks = 1024;
int check_ids_blocks(int64_t N);
hipError_t launch_check_ids(const int32_t* ids, int64_t N, int K, int64_t V, void* partial, int64_t* out,
                            hipStream_t s);
// out[r, c] = acc_in[r, c] (if not NULL) + sum over s of part[s, r, c], in
// split order, for r < rows; out in dtype (fp32 or bf16), acc_in fp32 and
// out may alias it. The partials have row pitch d and split pitch Cp * d.
hipError_t launch_dh_reduce(int dtype, const float* part, int splits, int rows,
                            int64_t d, int64_t Cp, const float* acc_in, void* out, hipStream_t s);

// EPI_DZJ: the dZ epilogue of the alternative losses (support corrections
// formed at the teacher entries), a kernel of its own so that the KL's is
// untouched.
enum Epilogue { EPI_FWD = 0, EPI_DZ = 1, EPI_DH = 2, EPI_DW = 3, EPI_DZJ = 4 };
// dtype: 0 = fp32, 1 = bf16
hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s);
int gemm_k_step(int dtype);  // elements per k-step of the GEMM main loop

// Forward-chunked KL over a given logit grid (one wavefront per row).
struct LogitsArgs {
  const void* Z;        // [N, V] storage dtype, row-major, 16-byte aligned base
  void* dZ;             // [N, V] backward output (may be Z itself)
  const int32_t* ids;   // [N, K]
  const float* logits;  // [N, K]
  int64_t N, V;
  int K;                // 1..1024
  float inv_T;
  float* row_lse;       // [N] forward output, backward input
  float* row_kl;        // [N] forward output
  const float* scale;   // backward: device scalar g / (N_kept T)
};
hipError_t launch_logits_fwd(int dtype, const LogitsArgs& a, hipStream_t s);

// Dense KL (the pages' baseline): full student log-probability and teacher
// probability grids, row pitch ldv (the padded vocabulary), one wavefront
// per row.
struct DenseArgs {
  const void* Z;        // [rows_pad, ldv] storage dtype: the projected logits
  float* logq;          // [N, ldv] fp32 student log-probabilities
  float* P;             // [N, ldv] fp32 teacher probabilities, zero off the top-K
  void* dZ;             // [rows_pad, ldv] storage dtype (backward; zero past N rows and V columns)
  const int32_t* ids;   // [N, K]
  const float* logits;  // [N, K]
  int64_t N, V, ldv, rows_pad;
  int K;
  float inv_T;
  float* row_lse;       // [N]
  float* row_kl;        // [N]
  const float* scale;   // backward: device scalar g / (N_kept T)
};
hipError_t launch_dense_student(int dtype, const DenseArgs& a, hipStream_t s);
hipError_t launch_dense_teacher(const DenseArgs& a, hipStream_t s);
hipError_t launch_dense_kl(const DenseArgs& a, hipStream_t s);
hipError_t launch_dense_grad(int dtype, const DenseArgs& a, hipStream_t s);
hipError_t launch_logits_bwd(int dtype, const LogitsArgs& a, hipStream_t s);

}  // namespace kdkl
