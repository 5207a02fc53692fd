// C-ABI entry points of libkdkl.so: argument checks, workspace plan, and the
// per-chunk launch sequence of the fused chunked KL loss (forward: project,
// fold into the running loss, drop; backward: recompute each chunk's
// projection) [P1 "Making knowledge distillation cheap enough to run at
// scale", section "Two system changes", fused chunked KL bullet].
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/kdkl.h"
#include "kdkl_internal.h"

namespace kdkl {

const char* kernel_name(int id) {
  static const char* names[K_COUNT] = {
      "teacher_prep", "fwd_gemm_lse", "split_merge", "loss_reduce", "transpose_w",
      "transpose_h",  "dz_gemm",      "dh_gemm",     "dh_reduce",   "dw_gemm",
      "logits_fwd",   "logits_bwd",   "grad_scale",  "dense_gemm",  "dense_student",
      "dense_teacher", "dense_kl",    "dense_grad",  "jsd_merge",     "jsd_prep",
      "topk_rkl",      "topk_dw"};
  return (id >= 0 && id < K_COUNT) ? names[id] : "?";
}

// ------------------------------ profiling ---------------------------------
namespace {
struct Rec {
  int kid;
  hipEvent_t a, b;
  double flops, bytes;
};
// The library's only process-wide mutable state: the timing table. `on` is
// read without the lock on every launch (atomically) and re-read under the
// lock before anything is recorded.
struct Prof {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
} g_prof;

hipEvent_t prof_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` bracketed by events when profiling is on.
template <class F>
hipError_t timed(int kid, double flops, double bytes, hipStream_t s, F&& launch) {
  if (!g_prof.on.load(std::memory_order_acquire)) return launch();
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.on.load(std::memory_order_relaxed)) return launch();
  hipEvent_t a = prof_event(), b = prof_event();
  auto give_back = [&] {  // events not recorded go back to the pool
    if (a) g_prof.pool.push_back(a);
    if (b) g_prof.pool.push_back(b);
  };
  if (!a || !b) {
    give_back();
    return hipErrorOutOfMemory;
  }
  hipError_t e = hipEventRecord(a, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e != hipSuccess) {
    give_back();
    return e;
  }
  g_prof.recs.push_back({kid, a, b, flops, bytes});
  return hipSuccess;
}
}  // namespace

// ------------------------------ planning ----------------------------------
static inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Compute units of the MI355X; the dH split count is sized for them.
constexpr int64_t kComputeUnits = 256;

struct Plan {
  int64_t N, d, V, K, chunk;
  int dtype;
  int64_t es;      // element bytes of H, W, dZ, dH
  int64_t Cp;      // chunk capacity (multiple of the token tile)
  int64_t Vp;      // padded vocabulary (multiple of the vocabulary tile)
  int vt;          // vocabulary tile: rows per workgroup of the forward and dZ products
  int64_t n_vt;    // vocabulary tiles
  int dh_splits;
  int64_t dh_ksplit;
  // The backward visits `bg` consecutive chunks at a time ("group", token
  // capacity Cg) in n_parts slices of the vocabulary, vpart rows each: the dZ
  // buffer [Cg, vpart] holds as many elements as one chunk's [Cp, Vp], and dW
  // takes one read-modify-write per group and slice instead of one per chunk.
  int bg;
  int64_t Cg;
  int64_t vpart;
  int n_parts;
  bool fast;       // bf16 main loop: reads W, H and dZ in place (no transposes)
  bool wt;         // the dH product reads W^T written once per backward call (else W in place)
  int dtile;       // N-tile width of the dH and dW products (hidden-size axis)
  int loss;        // kdkl_loss
  float beta;      // the loss's parameter (JSD beta, skew alpha)
  bool epi_alt;    // an alternative loss formed in the projections' epilogues (JSD, skew KL, skew reverse KL)
  bool trkl;       // the reverse KL over the top-K support (no vocabulary-wide forward)
  // offsets into the forward workspace
  size_t f_ent, f_erow, f_keep, f_tstart, f_part, f_sk, f_red, f_rowkl, f_bytes;
  // offsets into the backward workspace
  size_t b_ent, b_erow, b_keep, b_scale, b_red, b_tstart, b_rowcoef, b_dzent, b_cnt, b_scans, b_list, b_part,
      b_wt, b_ht, b_dzcv, b_dzvc, b_dhpart, b_dhacc, b_bytes;
};

// The dH product on the bf16 main loop reads either a W^T copy written once
// per backward call or W in place through the LDS transpose read (V * d * 2
// fewer bytes of workspace, no transpose, but each dH launch measured about
// 2% slower on 256-wide hidden-size tiles and 4% on 320-wide ones). The plan
// keeps the copy only when the modelled extra time of one call's dH launches
// read in place (at about 1.2 PFLOP/s) exceeds the transpose (W read and
// written at about 5 TB/s) by at least 0.3 ms: Llama-like heads at 8K
// positions and gpt-oss-like heads up to 16K read W in place, gpt-oss-like
// heads beyond keep the copy (a 1.2 GB step of the workspace at that N, paid
// only where the copy saves time).
static bool dh_reads_w_in_place(const Plan& P, int64_t N) {
  const int64_t group = P.bg * P.chunk;
  const double launches = (double)((N + group - 1) / group) * (double)P.n_parts;
  const double dh_ms = 2.0 * (double)P.Cg * (double)P.vpart * (double)P.d / 1.2e12;
  const double penalty = P.dtile == 256 ? 0.02 : 0.04;
  const double transpose_ms = 4.0 * (double)P.V * (double)P.d / 5.0e9;
  return launches * dh_ms * penalty < transpose_ms + 0.3;
}
// The dH split count keeps the device within this share of as busy as the
// best split count does.
constexpr double kDhBusy = 0.96;
// Largest accepted kdkl_options.vocab_slices and chunks_per_group.
constexpr int kMaxVocabSlices = 1024;
constexpr int kMaxChunksPerGroup = 64;
// Largest group of the library's own blocking (chunks per backward launch),
// and the least share (percent) of dW's last round of workgroups its slices
// must fill.
constexpr int kMaxOwnGroup = 16;
constexpr int64_t kDwRoundFill = 95;
// Largest dZ buffer (group rows x slice rows x element bytes) of the
// library's own blocking: about 1.5% of the device's memory, independent of
// the number of positions.
constexpr int64_t kDzBudget = (int64_t)4 << 30;

// Rows of each vocabulary slice (the last one may be shorter) when a group's
// vocabulary is cut in `slices`: slices start on a tile boundary of both the
// dZ product (vt rows) and the dW product (256 rows).
static int64_t slice_rows(const Plan& P, int64_t slices) {
  if (slices <= 1) return P.Vp;
  const int64_t align = P.vt % 256 == 0 ? P.vt : P.vt * 2;
  return round_up((P.V + slices - 1) / slices, align);
}

// Whether a slice of `vpart` rows gives the dW product at least one full
// round of workgroups (one per compute unit) and fills its rounds to 95% or
// more (a partial last round costs more than the read-modify-writes a
// larger group saves).
static bool dw_fills(const Plan& P, int64_t vpart) {
  const int64_t tiles = (vpart + 255) / 256 * ((P.d + P.dtile - 1) / P.dtile);
  const int64_t rounds = (tiles + kComputeUnits - 1) / kComputeUnits;
  return tiles >= kComputeUnits && tiles * 100 >= rounds * kComputeUnits * kDwRoundFill;
}

// The fewest vocabulary slices for a group of `rows` (padded) positions
// whose dZ buffer fits kDzBudget and, with `fill`, whose slices fill dW's
// rounds; 0 if there is none.
static int64_t fewest_slices(const Plan& P, int64_t rows, bool fill) {
  for (int64_t s = 1; s <= kMaxVocabSlices; ++s) {
    const int64_t vp = slice_rows(P, s);
    if (s > 1 && vp == slice_rows(P, s - 1)) continue;  // the same slicing as s - 1
    if (vp * rows * P.es > kDzBudget) continue;
    if (!fill || dw_fills(P, vp)) return s;
  }
  return 0;
}

// The library's own blocking on the bf16 main loop (kdkl_options fields 0):
// the largest group of 16, 8, 4 or 2 chunks (no more than there are) that has
// such a slicing, with its fewest slices; else one chunk per group. Larger
// groups lengthen dW's contraction (one fp32 read-modify-write of dW per
// group and slice) and let dH fill the device with fewer split-K partials;
// fewer slices mean fewer dZ and dH launches and running sums. A set option
// is kept and the other field chosen around it. The generic main loop (fp32,
// or d not a multiple of 64) keeps one chunk and the whole vocabulary.
static void choose_blocking(const Plan& P, int64_t N, int bg_set, int64_t slices_set, int* bg_out,
                            int64_t* slices_out) {
  const int64_t chunks = (N + P.chunk - 1) / P.chunk;
  auto group_rows = [&](int bg) { return round_up((int64_t)bg * P.chunk, kTokenTile); };
  // the fewest slices within the budget for a group, filling dW's rounds if
  // any slicing does; the most slices if even they exceed the budget
  auto own_slices = [&](int bg) {
    int64_t s = fewest_slices(P, group_rows(bg), true);
    if (s == 0) s = fewest_slices(P, group_rows(bg), false);
    return s > 0 ? s : (int64_t)kMaxVocabSlices;
  };
  *bg_out = bg_set > 0 ? bg_set : 1;
  *slices_out = slices_set > 0 ? slices_set : 1;
  if (!P.fast) return;  // the generic path: one chunk at a time over the whole vocabulary
  if (bg_set > 0) {     // a set group size: the library's slices around it
    if (slices_set == 0) *slices_out = own_slices(bg_set);
    return;
  }
  for (int bg = kMaxOwnGroup; bg > 1; bg >>= 1) {
    if (bg > chunks || !gemm_fast_path(P.dtype, P.d, P.Vp, group_rows(bg))) continue;
    if (slices_set > 0) {  // a set slicing: the largest group whose dZ buffer it keeps within the budget
      if (slice_rows(P, slices_set) * group_rows(bg) * P.es <= kDzBudget) {
        *bg_out = bg;
        return;
      }
      continue;
    }
    const int64_t s = fewest_slices(P, group_rows(bg), true);
    if (s > 0) {
      *bg_out = bg;
      *slices_out = s;
      return;
    }
  }
  if (slices_set == 0) *slices_out = own_slices(1);
}

static bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_mul_overflow(a, b, out) && *out >= 0;
}

// Adds a 256-byte aligned region of `bytes` at *cursor; false on overflow.
static bool region(size_t* cursor, int64_t bytes, size_t* off) {
  const size_t c = (size_t)round_up((int64_t)*cursor, 256);
  if (bytes < 0 || c > SIZE_MAX - (size_t)bytes) return false;
  *off = c;
  *cursor = c + (size_t)bytes;
  return true;
}

static_assert((int)ALT_JSD == (int)KDKL_LOSS_JSD && (int)ALT_SKL == (int)KDKL_LOSS_SKL && (int)ALT_SRKL == (int)KDKL_LOSS_SRKL,
              "the kernels number the alternative losses as the C-ABI does");


static kdkl_status check_options(const kdkl_options* o) {
  if (o == nullptr) return KDKL_OK;
  const float a = o->beta;
  switch (o->loss) {
    case KDKL_LOSS_KL: break;
    case KDKL_LOSS_JSD: if (!(a > 0.f && a < 1.f)) return KDKL_ERR_OPTION; break;
    case KDKL_LOSS_SKL: if (!(a >= 0.f && a < 1.f)) return KDKL_ERR_OPTION; break;
    case KDKL_LOSS_SRKL: if (!(a > 0.f && a <= 1.f)) return KDKL_ERR_OPTION; break;
    case KDKL_LOSS_TRKL: break;
    default: return KDKL_ERR_OPTION;
  }
  if (o->chunks_per_group < 0 || o->chunks_per_group > kMaxChunksPerGroup) return KDKL_ERR_OPTION;
  if (o->vocab_slices < 0 || o->vocab_slices > kMaxVocabSlices) return KDKL_ERR_OPTION;
  if (o->dh_w_in_place < 0 || o->dh_w_in_place > 2) return KDKL_ERR_OPTION;
  for (int i = 0; i < 3; ++i)
    if (o->reserved[i] != 0) return KDKL_ERR_OPTION;
  return KDKL_OK;
}

static kdkl_status make_plan(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int dtype,
                             const kdkl_options* opts, Plan* P) {
  if (dtype != KDKL_F32 && dtype != KDKL_BF16) return KDKL_ERR_DTYPE;
  const int64_t dmul = dtype == KDKL_BF16 ? 8 : 4;
  if (N < 0 || d <= 0 || V <= 0 || K <= 0 || chunk <= 0) return KDKL_ERR_SHAPE;
  if (d % dmul != 0 || K > 1024 || K > V) return KDKL_ERR_SHAPE;
  if (N > INT32_MAX || V > INT32_MAX - 4096 || d > (1 << 24)) return KDKL_ERR_OVERFLOW;
  P->N = N; P->d = d; P->V = V; P->K = K; P->dtype = dtype;
  P->es = dtype == KDKL_BF16 ? 2 : 4;
  P->chunk = chunk < N ? chunk : (N > 0 ? N : 1);
  P->Cp = round_up(P->chunk, kTokenTile);
  P->vt = kVocabTile;
  P->Vp = round_up(V, P->vt);
  P->fast = gemm_fast_path(dtype, d, P->Vp, P->Cp);
  const int vt = gemm_vocab_tile(P->fast, V, P->Cp / kTokenTile);
  if (vt != P->vt && gemm_fast_path(dtype, d, round_up(V, vt), P->Cp)) {
    P->vt = vt;
    P->Vp = round_up(V, vt);
  }
  P->dtile = gemm_d_tile(P->fast, d);
  P->n_vt = P->Vp / P->vt;
  if (P->Cp > INT32_MAX / 4) return KDKL_ERR_OVERFLOW;
  kdkl_status ost = check_options(opts);
  if (ost != KDKL_OK) return ost;
  const kdkl_options o = opts ? *opts : kdkl_options{};
  P->loss = o.loss;
  P->epi_alt = o.loss == KDKL_LOSS_JSD || o.loss == KDKL_LOSS_SKL || o.loss == KDKL_LOSS_SRKL;
  P->trkl = o.loss == KDKL_LOSS_TRKL;
  P->beta = P->epi_alt ? o.beta : 0.f;
  int bg = 1;
  int64_t slices = 1;
  if (P->fast) {
    // the vocabulary tile was chosen for one chunk's token tiles, but the
    // projections launch a whole group: choose it for the group the
    // library's own blocking takes (not the options', so that blocking
    // options never change it, nor the results' rounding)
    choose_blocking(*P, N, 0, 0, &bg, &slices);
    const int64_t rows = round_up((int64_t)bg * P->chunk, kTokenTile);
    const int vtg = gemm_vocab_tile(true, V, rows / kTokenTile);
    if (bg > 1 && vtg != P->vt && gemm_fast_path(dtype, d, round_up(V, vtg), rows)) {
      P->vt = vtg;
      P->Vp = round_up(V, vtg);
      P->n_vt = P->Vp / P->vt;
    }
  }
  if (o.chunks_per_group > 1) {
    // more than one chunk per launch needs the bf16 main loop, whose 32-bit
    // load offsets must still cover the group's operands
    if (!P->fast || !gemm_fast_path(dtype, d, P->Vp, round_up((int64_t)o.chunks_per_group * P->chunk, kTokenTile)))
      return KDKL_ERR_OPTION;
  }
  choose_blocking(*P, N, o.chunks_per_group, o.vocab_slices, &bg, &slices);
  P->bg = bg;
  P->Cg = round_up(P->bg * P->chunk, kTokenTile);
  if (P->Cg > INT32_MAX / 4) return KDKL_ERR_OVERFLOW;
  P->vpart = slice_rows(*P, slices);
  P->n_parts = (int)((V + P->vpart - 1) / P->vpart);
  if (o.dh_w_in_place == 1 && !P->fast) return KDKL_ERR_OPTION;
  // (the top-K reverse KL forms dH from W's rows at the support: no W^T)
  P->wt = !P->trkl &&
          (!P->fast || (o.dh_w_in_place == 2) || (o.dh_w_in_place == 0 && !dh_reads_w_in_place(*P, N)));
  // dH split-K: the fewest splits S whose launch keeps the 256 compute units
  // within 4% as busy as the best S does, when every workgroup does 1/S of a
  // tile's work and the units take them in rounds (fewer splits, fewer fp32
  // partials), with each split at least 8 k-steps.
  const int64_t tiles = ((P->Cg + 255) / 256) * ((d + P->dtile - 1) / P->dtile);
  const int64_t kstep = dtype == KDKL_BF16 ? 64 : 32;
  int64_t smax = P->vpart / (8 * kstep);
  if (smax > 16) smax = 16;
  if (smax < 1) smax = 1;
  auto busy = [&](int64_t c) {  // share of the rounds' workgroup slots in use
    const int64_t r = (tiles * c + kComputeUnits - 1) / kComputeUnits;
    return (double)(tiles * c) / (double)(r * kComputeUnits);
  };
  double best = 0.0;
  for (int64_t c = 1; c <= smax; ++c) best = busy(c) > best ? busy(c) : best;
  int64_t S = 1;
  while (S < smax && busy(S) < kDhBusy * best) ++S;
  P->dh_splits = (int)S;
  P->dh_ksplit = round_up((P->vpart + S - 1) / S, kstep);

  int64_t t0, t1, t2;
  size_t cur = 0;
  bool ok = true;
  // the forward takes the backward's groups too (bigger launches fill the
  // device's rounds better; results per row do not depend on it)
  ok &= mul_ok(P->Cg, K, &t0) && mul_ok(t0, 8, &t0);
  ok &= region(&cur, t0, &P->f_ent);
  ok &= region(&cur, P->Cg * 4, &P->f_erow) && region(&cur, P->Cg * 4, &P->f_keep);
  ok &= mul_ok(P->n_vt + 1, P->Cg, &t1) && mul_ok(t1, 2, &t1);
  ok &= region(&cur, t1, &P->f_tstart);
  ok &= mul_ok(P->Cg, P->n_vt, &t2) && mul_ok(t2, 16, &t2);
  ok &= region(&cur, t2, &P->f_part);
  // the alternative losses' student logits at the sorted teacher entries [Cg, K]
  int64_t sk = 0;
  if (P->epi_alt) ok &= mul_ok(P->Cg, K, &sk) && mul_ok(sk, 4, &sk);
  P->f_sk = 0;
  if (sk) ok &= region(&cur, sk, &P->f_sk);
  ok &= region(&cur, (int64_t)kReduceBytes, &P->f_red);  // the loss's partial sums
  ok &= region(&cur, (N > 0 ? N : 1) * 4, &P->f_rowkl);
  P->f_bytes = cur;

  cur = 0;
  int64_t g0, g1;
  ok &= mul_ok(P->Cg, K, &g0) && mul_ok(g0, 8, &g0);
  ok &= mul_ok(P->n_vt + 1, P->Cg, &g1) && mul_ok(g1, 2, &g1);
  ok &= region(&cur, g0, &P->b_ent);
  ok &= region(&cur, P->Cg * 4, &P->b_erow) && region(&cur, P->Cg * 4, &P->b_keep);
  ok &= region(&cur, 16, &P->b_scale);
  ok &= region(&cur, (int64_t)kReduceBytes, &P->b_red);  // the kept count's partial sums
  ok &= region(&cur, g1, &P->b_tstart);
  P->b_rowcoef = 0;
  if (P->epi_alt) ok &= region(&cur, P->Cg * 4, &P->b_rowcoef);
  P->b_dzent = P->b_cnt = P->b_scans = P->b_list = P->b_part = 0;
  if (P->trkl) {
    // the entry gradients [Cg, K] fp32 and the sparse dW's counting sort:
    // per-block counts, the scans over the ids (int64), the sorted entries,
    // and the partial rows of the ids with more than one run of entries
    ok &= region(&cur, g0 / 2, &P->b_dzent);
    ok &= region(&cur, trkl_count_bytes(P->Cg, V), &P->b_cnt);
    ok &= region(&cur, trkl_scan_bytes(V, P->Cg * K), &P->b_scans);
    ok &= region(&cur, g0, &P->b_list);
    ok &= region(&cur, trkl_part_bytes(P->Cg * K, d), &P->b_part);
    P->b_wt = P->b_ht = P->b_dzcv = P->b_dzvc = P->b_dhpart = P->b_dhacc = 0;
    P->b_bytes = cur;
    return ok ? KDKL_OK : KDKL_ERR_OVERFLOW;  // (no dZ buffer, W^T or dH partials)
  }
  int64_t wt, ht, dz, dhp;
  ok &= mul_ok(d, P->Vp, &wt) && mul_ok(wt, P->es, &wt);
  ok &= mul_ok(d, P->Cg, &ht) && mul_ok(ht, P->es, &ht);
  ok &= mul_ok(P->Cg, P->vpart, &dz) && mul_ok(dz, P->es, &dz);
  P->b_wt = 0;
  if (P->wt) ok &= region(&cur, wt, &P->b_wt);
  if (P->fast) {
    // dW reads the token-major dZ in place through the LDS transpose read and
    // H_g^T (one small transpose per group); dH reads W in place the same
    // way unless the plan keeps W^T.
    P->b_dzvc = 0;
    ok &= region(&cur, ht, &P->b_ht);
    ok &= region(&cur, dz, &P->b_dzcv);
  } else {
    ok &= region(&cur, ht, &P->b_ht);
    ok &= region(&cur, dz, &P->b_dzcv) && region(&cur, dz, &P->b_dzvc);
  }
  ok &= mul_ok(S * P->Cg, d, &dhp) && mul_ok(dhp, 4, &dhp);
  P->b_dhpart = 0;
  if (!P->trkl) ok &= region(&cur, dhp, &P->b_dhpart);  // (the top-K reverse KL forms dH itself)
  P->b_dhacc = 0;
  if (P->n_parts > 1 && !P->trkl) {
    int64_t acc;
    ok &= mul_ok(P->Cg, d, &acc) && mul_ok(acc, 4, &acc);
    ok &= region(&cur, acc, &P->b_dhacc);
  }
  P->b_bytes = cur;
  return ok ? KDKL_OK : KDKL_ERR_OVERFLOW;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static kdkl_status check_common(const void* H, const void* W, const int32_t* ids, const float* lg,
                                int64_t N, float T) {
  if (!W) return KDKL_ERR_NULL;
  if (N > 0 && (!H || !ids || !lg)) return KDKL_ERR_NULL;
  if (!(T > 0.f) || !isfinite(T)) return KDKL_ERR_VALUE;
  if (!aligned16(H) || !aligned16(W)) return KDKL_ERR_ALIGN;
  return KDKL_OK;
}

static TeacherArgs teacher_args(const Plan& P, const int32_t* ids, const float* lg, float T, int64_t r0,
                                int rows, int64_t pitch, char* ws, size_t o_ent, size_t o_erow,
                                size_t o_keep, size_t o_tstart) {
  TeacherArgs t;
  t.ids = ids; t.logits = lg; t.r0 = r0; t.rows = rows; t.K = (int)P.K;
  t.inv_T = 1.0f / T; t.vt = P.vt; t.n_vt = (int)P.n_vt; t.Cp = pitch;
  t.ent = (int2*)(ws + o_ent);
  t.erow = (float*)(ws + o_erow); t.keep = (float*)(ws + o_keep); t.tstart = (uint16_t*)(ws + o_tstart);
  return t;
}

static GemmArgs projection_args(const Plan& P, const void* H, const void* W, float T, int64_t r0,
                                int rows, char* ws, size_t o_ent, size_t o_tstart) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = W; g.lda = P.d;
  g.B = (const char*)H + r0 * P.d * P.es; g.ldb = P.d;
  g.M = (int)P.V; g.N = rows;
  g.k_end = P.d; g.k_split = P.d;
  g.tiles_m = (int)P.n_vt; g.tiles_n = (int)((rows + kTokenTile - 1) / kTokenTile); g.splits = 1;
  g.bm = P.vt;
  g.inv_T = 1.0f / T; g.V = (int)P.V; g.K = (int)P.K; g.Cp = P.Cp; g.n_vt = (int)P.n_vt;
  g.ent = (const int2*)(ws + o_ent);
  g.tstart = (const uint16_t*)(ws + o_tstart);
  g.Vp = P.Vp;
  g.a_layout = g.b_layout = LAYOUT_KC;
  return g;
}

static JsdArgs jsd_args(const Plan& P, int rows, char* ws, size_t o_ent, size_t o_keep) {
  JsdArgs j;
  memset(&j, 0, sizeof(j));
  j.V = P.V; j.rows = rows; j.K = (int)P.K; j.loss = P.loss; j.beta = P.beta;
  j.log_beta = (float)log((double)P.beta);
  j.log_omb = (float)log1p(-(double)P.beta);
  j.ent = (int2*)(ws + o_ent); j.keep = (const float*)(ws + o_keep);
  return j;
}

static TopkArgs topk_args(const Plan& P, const void* H, const void* W, float T, int64_t r0, int rows, char* ws,
                          size_t o_ent, size_t o_keep) {
  TopkArgs t;
  memset(&t, 0, sizeof(t));
  t.H = (const char*)H + r0 * P.d * P.es; t.W = W;
  t.V = P.V; t.d = P.d; t.rows = rows; t.K = (int)P.K; t.inv_T = 1.0f / T;
  t.ent = (const int2*)(ws + o_ent); t.keep = (const float*)(ws + o_keep);
  return t;
}

}  // namespace kdkl

using namespace kdkl;

extern "C" {

int kdkl_abi_version(void) { return KDKL_ABI_VERSION; }

const char* kdkl_status_string(int s) {
  switch (s) {
    case KDKL_OK: return "KDKL_OK";
    case KDKL_ERR_NULL: return "KDKL_ERR_NULL: a required pointer is NULL";
    case KDKL_ERR_SHAPE: return "KDKL_ERR_SHAPE: a size is out of range";
    case KDKL_ERR_VALUE: return "KDKL_ERR_VALUE: temperature must be finite and > 0";
    case KDKL_ERR_DTYPE: return "KDKL_ERR_DTYPE: unsupported dtype";
    case KDKL_ERR_WORKSPACE: return "KDKL_ERR_WORKSPACE: workspace too small";
    case KDKL_ERR_OVERFLOW: return "KDKL_ERR_OVERFLOW: size overflow";
    case KDKL_ERR_HIP: return "KDKL_ERR_HIP: HIP launch or runtime failure";
    case KDKL_ERR_ALIGN: return "KDKL_ERR_ALIGN: pointer not 16-byte aligned";
    case KDKL_ERR_OPTION: return "KDKL_ERR_OPTION: an option is out of range or not available for these sizes";
    default: return "KDKL_ERR_UNKNOWN";
  }
}

kdkl_status kdkl_workspace_size(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int dtype,
                                const kdkl_options* opts, size_t* fwd_bytes, size_t* bwd_bytes) {
  Plan P;
  kdkl_status st = make_plan(N, d, V, K, chunk, dtype, opts, &P);
  if (st != KDKL_OK) return st;
  if (fwd_bytes) *fwd_bytes = P.f_bytes;
  if (bwd_bytes) *bwd_bytes = P.b_bytes;
  return KDKL_OK;
}

kdkl_status kdkl_plan_info(int64_t N, int64_t d, int64_t V, int32_t K, int64_t chunk, int dtype,
                           const kdkl_options* opts, kdkl_plan* out) {
  if (!out) return KDKL_ERR_NULL;
  Plan P;
  kdkl_status st = make_plan(N, d, V, K, chunk, dtype, opts, &P);
  if (st != KDKL_OK) return st;
  memset(out, 0, sizeof(*out));
  out->chunks_per_group = P.bg;
  out->vocab_slices = P.n_parts;
  out->dh_splits = P.dh_splits;
  out->dh_w_in_place = P.wt ? 0 : 1;
  out->vocab_tile = P.vt;
  out->hidden_tile = P.dtile;
  out->bf16_main_loop = P.fast ? 1 : 0;
  out->fwd_bytes = P.f_bytes;
  out->bwd_bytes = P.b_bytes;
  return KDKL_OK;
}

// The forward's launch sequence on a checked workspace `ws`: per group of
// rows, the teacher products, the projection with its online logsumexp and
// teacher-gather epilogue, and the split merge; then the loss.
static hipError_t forward_launches(const Plan& P, const void* H, const void* W, const int32_t* ids,
                                  const float* lg, float T, float* loss, float* row_lse, float* kl, char* ws,
                                  hipStream_t s) {
  const int64_t N = P.N, V = P.V, d = P.d;
  hipError_t e = hipSuccess;
  const int64_t group = P.bg * P.chunk;  // rows per launch: the backward's group
  for (int64_t r0 = 0; r0 < N && e == hipSuccess; r0 += group) {
    const int rows = (int)((N - r0) < group ? (N - r0) : group);
    TeacherArgs ta =
        teacher_args(P, ids, lg, T, r0, rows, P.Cg, ws, P.f_ent, P.f_erow, P.f_keep, P.f_tstart);
    e = timed(K_TEACHER, 0.0, (double)rows * P.K * 8.0 * 2.0, s, [&] { return launch_teacher(ta, s); });
    if (e != hipSuccess) break;
    if (P.trkl) {
      // the student's logits at the support only: no projection
      TopkArgs t = topk_args(P, H, W, T, r0, rows, ws, P.f_ent, P.f_keep);
      t.row_lse = row_lse + r0; t.row_loss = row_lse + N + r0; t.row_kl = kl + r0;
      e = timed(K_TOPK_RKL, 2.0 * rows * (double)P.K * d, (double)rows * P.K * (d * P.es + 8.0), s,
                [&] { return launch_topk_rkl(P.dtype, t, false, s); });
      continue;
    }
    GemmArgs g = projection_args(P, H, W, T, r0, rows, ws, P.f_ent, P.f_tstart);
    g.Cp = P.Cg;
    g.part = (float4*)(ws + P.f_part);
    // the alternative losses need s at each teacher entry: the epilogue
    // keeps it as it meets the entry
    g.sk = P.epi_alt ? (float*)(ws + P.f_sk) : nullptr;
    const double fl = 2.0 * rows * (double)V * d;
    const double by = ((double)V + rows) * d * P.es + (double)rows * P.n_vt * 16.0;
    e = timed(K_FWD_GEMM, fl, by, s, [&] { return launch_gemm(P.dtype, EPI_FWD, g, s); });
    if (e != hipSuccess) break;
    if (P.epi_alt) {
      // lse, the loss and gbar per row from the partials and the kept student
      // logits; gbar is saved after the N logsumexps for the backward
      JsdArgs j = jsd_args(P, rows, ws, P.f_ent, P.f_keep);
      j.sk = (const float*)(ws + P.f_sk);
      j.part = (const float4*)(ws + P.f_part); j.n_vt = (int)P.n_vt;
      j.row_lse = row_lse + r0; j.row_kl = kl + r0; j.row_gbar = row_lse + N + r0;
      e = timed(K_JSD_MERGE, 0.0, (double)rows * (P.n_vt * 16.0 + P.K * 12.0), s,
                [&] { return launch_jsd_merge(j, s); });
      continue;
    }
    MergeArgs m;
    m.part = (const float4*)(ws + P.f_part); m.n_vt = (int)P.n_vt; m.rows = rows;
    m.erow = (const float*)(ws + P.f_erow); m.keep = (const float*)(ws + P.f_keep);
    m.row_lse = row_lse + r0; m.row_kl = kl + r0;
    e = timed(K_MERGE, 0.0, (double)rows * P.n_vt * 16.0, s, [&] { return launch_merge(m, s); });
  }
  if (e == hipSuccess)
    e = timed(K_LOSS, 0.0, (double)N * 8.0, s,
              [&] { return launch_loss_ws(kl, ids, (int)P.K, N, ws + P.f_red, loss, s); });
  return e;
}

kdkl_status kdkl_forward(const void* H, const void* W, const int32_t* ids, const float* lg, int64_t N,
                         int64_t d, int64_t V, int32_t K, float T, int64_t chunk, int dtype,
                         const kdkl_options* opts, float* loss, float* row_lse, float* row_kl, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Plan P;
  kdkl_status st = make_plan(N, d, V, K, chunk, dtype, opts, &P);
  if (st != KDKL_OK) return st;
  if ((st = check_common(H, W, ids, lg, N, T)) != KDKL_OK) return st;
  if (!loss || (N > 0 && !row_lse) || !workspace) return KDKL_ERR_NULL;
  if (workspace_bytes < P.f_bytes) return KDKL_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KDKL_ERR_ALIGN;
  char* ws = (char*)workspace;
  float* kl = row_kl ? row_kl : (float*)(ws + P.f_rowkl);
  const hipError_t e = forward_launches(P, H, W, ids, lg, T, loss, row_lse, kl, ws, (hipStream_t)stream);
  return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
}

// ---------------------- allocation-free forward ------------------------------
// For callers that cannot allocate device memory, the forward's workspace can
// be a file-scope device array. Its name in host code is a host-side
// stand-in, not a device address: the address is looked up once per device
// (with that device current) by hipGetSymbolAddress, and only that pointer
// is ever passed to kernels. The forward needs no part of its workspace
// cleared (every region is written before it is read), so the array keeps
// whatever the last call left in it.
static_assert(KDKL_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch holds whole 256-byte regions");
static __device__ __align__(256) char scratch[KDKL_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];  // per device, set once

// Device address of `scratch` on the device of `stream` (NULL: the current
// device).
static hipError_t scratch_address(hipStream_t stream, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (stream != nullptr && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

kdkl_status kdkl_forward_noalloc(const void* H, const void* W, const int32_t* ids, const float* lg, int64_t N,
                                 int64_t d, int64_t V, int32_t K, float T, int64_t chunk, int dtype,
                                 const kdkl_options* opts, float* loss, float* row_lse, float* row_kl,
                                 void* stream) {
  Plan P;
  kdkl_status st = make_plan(N, d, V, K, chunk, dtype, opts, &P);
  if (st != KDKL_OK) return st;
  if ((st = check_common(H, W, ids, lg, N, T)) != KDKL_OK) return st;
  if (!loss || (N > 0 && (!row_lse || !row_kl))) return KDKL_ERR_NULL;
  // row_kl is the caller's, so the forward needs its workspace up to the
  // per-row KL scratch (the last region); where the library chooses the
  // group size, take fewer chunks per group until that fits the array
  kdkl_options o = opts ? *opts : kdkl_options{};
  if (o.chunks_per_group == 0) {
    for (int bg = P.bg; bg > 1 && P.f_rowkl > (size_t)KDKL_NOALLOC_SCRATCH_BYTES;) {
      bg /= 2;
      o.chunks_per_group = bg;
      if ((st = make_plan(N, d, V, K, chunk, dtype, &o, &P)) != KDKL_OK) return st;
    }
  }
  if (P.f_rowkl > (size_t)KDKL_NOALLOC_SCRATCH_BYTES) return KDKL_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  hipError_t e = scratch_address(s, &ws);
  if (e == hipSuccess) e = forward_launches(P, H, W, ids, lg, T, loss, row_lse, row_kl, (char*)ws, s);
  return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
}

// dW_slice (+)= dZ^T H_g for vocabulary slice `part` of one group of rows.
static hipError_t dw_product(const Plan& P, int dtype, char* ws, int rows, int part, float* dW, bool accumulate,
                             hipStream_t s) {
  const int64_t d = P.d;
  const int64_t v0 = part * P.vpart;
  const int64_t vlen = P.V - v0 < P.vpart ? P.V - v0 : P.vpart;
  const int64_t rows_pad = round_up(rows, kTokenTile);
  const double fl = 2.0 * rows * (double)vlen * d;
  GemmArgs w;
  memset(&w, 0, sizeof(w));
  if (P.fast) {
    w.A = ws + P.b_dzcv; w.lda = P.vpart; w.a_layout = LAYOUT_MC; w.a_krows = P.Cg; w.a_mcols = P.vpart;
  } else {
    w.A = ws + P.b_dzvc; w.lda = P.Cg; w.a_layout = LAYOUT_KC;
  }
  w.B = ws + P.b_ht; w.ldb = P.Cg; w.b_layout = LAYOUT_KC;
  w.M = (int)vlen; w.N = (int)d; w.k_end = rows_pad; w.k_split = rows_pad;
  w.tiles_m = (int)((vlen + 255) / 256); w.tiles_n = (int)((d + P.dtile - 1) / P.dtile); w.splits = 1;
  w.bn = P.dtile;
  w.out = dW + v0 * d; w.ldo = d; w.accumulate = accumulate ? 1 : 0;
  return timed(K_DW_GEMM, fl, ((double)vlen * rows + (double)rows * d) * P.es + 8.0 * vlen * d, s,
            [&] { return launch_gemm(dtype, EPI_DW, w, s); });
}

// dH and dW (+)= of one group of rows [r0, r0 + rows) and vocabulary slice
// `part` from its dZ in the backward workspace (token-major [Cg, vpart]; the
// generic path, which has a single slice, also vocabulary-major), W (read in
// place through the LDS transpose read on the bf16 main loop, else as the
// W^T the call wrote) and the group's H^T: dH_g (+)= dZ W_slice split over
// the slice's vocabulary and summed in a fixed order (slices in order, each
// slice's splits in order), dW_slice (+)= dZ^T H_g.
static hipError_t part_products(const Plan& P, int dtype, const void* W, char* ws, int64_t r0, int rows, int part,
                                void* dH, float* dW, bool accumulate, hipStream_t s) {
  const int64_t d = P.d;
  const int64_t v0 = part * P.vpart;
  const int64_t vlen = P.V - v0 < P.vpart ? P.V - v0 : P.vpart;  // valid vocabulary rows
  const int64_t kv = P.Vp - v0 < P.vpart ? P.Vp - v0 : P.vpart;  // padded: zero past vlen
  const double fl = 2.0 * rows * (double)vlen * d;
  GemmArgs h;
  memset(&h, 0, sizeof(h));
  h.A = ws + P.b_dzcv; h.lda = P.vpart; h.a_layout = LAYOUT_KC;
  if (!P.wt) {
    // W rows v0.. as k rows (the hidden size contiguous); rows past the
    // slice's vocabulary are clamped to its last row (dZ is zero there)
    h.B = (const char*)W + v0 * P.d * P.es; h.ldb = P.d; h.b_layout = LAYOUT_MC;
    h.b_krows = vlen; h.b_mcols = P.d;
  } else {
    h.B = ws + P.b_wt + v0 * P.es; h.ldb = P.Vp; h.b_layout = LAYOUT_KC;
  }
  h.M = rows; h.N = (int)d; h.k_end = kv; h.k_split = P.dh_ksplit;
  h.tiles_m = (int)((rows + 255) / 256); h.tiles_n = (int)((d + P.dtile - 1) / P.dtile); h.bn = P.dtile;
  h.splits = (int)((kv + P.dh_ksplit - 1) / P.dh_ksplit);
  h.out = (float*)(ws + P.b_dhpart); h.ldo = d; h.Cp = P.Cg;
  const int splits = h.splits;
  // the first slice starts the fp32 sum, the last one writes dH in its dtype
  // (a read-modify-write of the split partials by each later slice instead
  // of this pass measured slower: the epilogue's scattered 4-byte reads cost
  // more per dH launch than the pass)
  const bool first = part == 0, last = part == P.n_parts - 1;
  const float* acc_in = first ? nullptr : (const float*)(ws + P.b_dhacc);
  void* out = last ? (void*)((char*)dH + r0 * d * P.es) : (void*)(ws + P.b_dhacc);
  const int out_dtype = last ? dtype : (int)KDKL_F32;
  const double sum_bytes = (first ? 0.0 : 4.0 * rows * d) + (double)rows * d * (last ? P.es : 4);
  hipError_t e = timed(K_DH_GEMM, fl, ((double)vlen * rows + (double)vlen * d) * P.es + 4.0 * splits * rows * d,
                       s, [&] { return launch_gemm(dtype, EPI_DH, h, s); });
  if (e == hipSuccess)
    e = timed(K_DH_REDUCE, 0.0, 4.0 * splits * rows * d + sum_bytes, s, [&] {
      return launch_dh_reduce(out_dtype, (const float*)(ws + P.b_dhpart), splits, rows, d, P.Cg, acc_in, out, s);
    });
  if (e != hipSuccess) return e;
  return dw_product(P, dtype, ws, rows, part, dW, accumulate, s);
}

kdkl_status kdkl_backward(const void* H, const void* W, const int32_t* ids, const float* lg, int64_t N,
                          int64_t d, int64_t V, int32_t K, float T, int64_t chunk, int dtype,
                          const kdkl_options* opts, const float* row_lse, const float* grad_loss, void* dH,
                          float* dW, int accumulate_dW, void* workspace, size_t workspace_bytes,
                          void* stream) {
  Plan P;
  kdkl_status st = make_plan(N, d, V, K, chunk, dtype, opts, &P);
  if (st != KDKL_OK) return st;
  if ((st = check_common(H, W, ids, lg, N, T)) != KDKL_OK) return st;
  if (!dW || !workspace || (N > 0 && (!row_lse || !dH))) return KDKL_ERR_NULL;
  if (workspace_bytes < P.b_bytes) return KDKL_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(dW) || !aligned16(dH)) return KDKL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t e = hipSuccess;
  if (N == 0) {
    if (!accumulate_dW) e = launch_zero(dW, V * d, s);
    return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
  }
  // W^T [d, Vp], zero-padded, once per call when the dH product reads both
  // operands K-contiguous (the generic path, or a build that keeps W^T)
  if (P.wt)
    e = timed(K_TRANSPOSE_W, 0.0, 2.0 * (double)V * d * P.es, s, [&] {
        return launch_transpose((int)P.es, W, V, d, d, ws + P.b_wt, P.Vp, P.Vp, s);
      });
  // g / (N_kept T): the mean runs over the positions that are not ignored
  if (e == hipSuccess)
    e = timed(K_GRAD_SCALE, 0.0, (double)N * 4.0, s, [&] {
      return launch_grad_scale_ws(ids, K, N, grad_loss, T, ws + P.b_red, (float*)(ws + P.b_scale), s);
    });
  const int64_t group = P.bg * P.chunk;
  for (int64_t r0 = 0; r0 < N && e == hipSuccess; r0 += group) {
    const int rows = (int)((N - r0) < group ? (N - r0) : group);
    const int64_t rows_pad = round_up(rows, kTokenTile);
    TeacherArgs ta = teacher_args(P, ids, lg, T, r0, rows, P.Cg, ws, P.b_ent, P.b_erow, P.b_keep,
                                  P.b_tstart);
    e = timed(K_TEACHER, 0.0, (double)rows * P.K * 8.0 * 2.0, s, [&] { return launch_teacher(ta, s); });
    if (e != hipSuccess) break;
    // H_g^T [d, Cg], zero-padded past the group's rows: the dW product
    // contracts over the group's tokens.
    const char* Hg = (const char*)H + r0 * d * P.es;
    if (!P.trkl)
      e = timed(K_TRANSPOSE_H, 0.0, 2.0 * (double)rows * d * P.es, s, [&] {
        return launch_transpose((int)P.es, Hg, rows, d, d, ws + P.b_ht, rows_pad, P.Cg, s);
      });
    if (e == hipSuccess && P.trkl) {
      // the loss's gradient at each support entry, from the forward's
      // logsumexp and loss, and dH over those entries; then dW over them
      TopkArgs t = topk_args(P, H, W, T, r0, rows, ws, P.b_ent, P.b_keep);
      t.row_lse = const_cast<float*>(row_lse) + r0; t.row_loss = const_cast<float*>(row_lse) + N + r0;
      t.scale = (const float*)(ws + P.b_scale); t.dz = (float*)(ws + P.b_dzent);
      t.dH = (char*)dH + r0 * d * P.es;
      // each support row of W read once or twice, H read and dH written
      const double w_reads = topk_rkl_one_pass(dtype, d) ? 1.0 : 2.0;
      e = timed(K_TOPK_RKL, 4.0 * rows * (double)P.K * d,
                (double)rows * (P.K * (w_reads * d * P.es + 12.0) + 2.0 * d * P.es), s,
                [&] { return launch_topk_rkl(dtype, t, true, s); });
      if (e == hipSuccess)
        // dW written (4 V d bytes) or read and written (8 V d)
        e = timed(K_TOPK_DW, 2.0 * rows * (double)P.K * d,
                  (double)rows * P.K * (d * P.es + 16.0) + ((r0 > 0 || accumulate_dW) ? 8.0 : 4.0) * V * d, s,
                  [&] {
                    return launch_trkl_dw(dtype, (const int2*)(ws + P.b_ent), (const float*)(ws + P.b_dzent), rows,
                                          (int)P.K, V, Hg, d, dW, r0 > 0 || accumulate_dW, (int*)(ws + P.b_cnt),
                                          (int64_t*)(ws + P.b_scans), (int2*)(ws + P.b_list),
                                          (float*)(ws + P.b_part), s);
                  });
      continue;
    }
    if (e == hipSuccess && P.epi_alt) {
      // from the forward's gbar, each row's coefficient of q in dZ; the
      // teacher mass of each distinct id over its first entry
      JsdArgs j = jsd_args(P, rows, ws, P.b_ent, P.b_keep);
      j.row_gbar_in = row_lse + N + r0; j.scale = (const float*)(ws + P.b_scale);
      j.rowcoef = (float*)(ws + P.b_rowcoef);
      e = timed(K_JSD_PREP, 0.0, (double)rows * (P.K * 16.0 + 8.0), s, [&] { return launch_jsd_prep(j, s); });
    }
    for (int part = 0; part < P.n_parts && e == hipSuccess; ++part) {
      // recompute the group's logits over the slice's vocabulary rows and
      // form dZ (token-major; the generic path also writes the
      // vocabulary-major copy)
      const int64_t v0 = part * P.vpart;
      const int64_t vlen = V - v0 < P.vpart ? V - v0 : P.vpart;
      GemmArgs g = projection_args(P, H, W, T, r0, rows, ws, P.b_ent, P.b_tstart);
      g.A = (const char*)W + v0 * d * P.es;
      g.M = (int)vlen; g.V = (int)vlen; g.v0 = (int)v0; g.tm0 = (int)(v0 / P.vt);
      g.tiles_m = (int)((vlen + P.vt - 1) / P.vt);
      g.Cp = P.Cg; g.Vp = P.vpart;
      g.row_lse = row_lse + r0; g.scale = (const float*)(ws + P.b_scale); g.keep = (const float*)(ws + P.b_keep);
      const bool alt = P.epi_alt;
      g.rowcoef = alt ? (const float*)(ws + P.b_rowcoef) : nullptr;
      g.beta = alt ? P.beta : 0.f;
      g.alt = alt ? P.loss : 0;
      g.dz_cv = ws + P.b_dzcv; g.dz_vc = P.fast ? nullptr : ws + P.b_dzvc;
      const double fl = 2.0 * rows * (double)vlen * d;
      e = timed(K_DZ_GEMM, fl,
                ((double)vlen + rows) * d * P.es + (P.fast ? 1.0 : 2.0) * rows * (double)vlen * P.es, s,
                [&] { return launch_gemm(dtype, alt ? EPI_DZJ : EPI_DZ, g, s); });
      if (e != hipSuccess) break;
      e = part_products(P, dtype, W, ws, r0, rows, part, dH, dW, r0 > 0 || accumulate_dW, s);
    }
  }
  return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
}

// ---------------------- forward-chunked KL (logit grid) --------------------

static kdkl_status check_logits(const void* Z, const int32_t* ids, const float* lg, int64_t N, int64_t V,
                                int32_t K, float T, int dtype) {
  if (dtype != KDKL_F32 && dtype != KDKL_BF16) return KDKL_ERR_DTYPE;
  if (N < 0 || V <= 0 || K <= 0 || K > 1024 || K > V) return KDKL_ERR_SHAPE;
  if (V > ((int64_t)1 << 40) || N > ((int64_t)1 << 40)) return KDKL_ERR_OVERFLOW;
  if (N > 0 && V > ((int64_t)1 << 60) / N) return KDKL_ERR_OVERFLOW;  // N V elements, without forming N V
  if (N > 0 && (!Z || !ids || !lg)) return KDKL_ERR_NULL;
  if (!(T > 0.f) || !isfinite(T)) return KDKL_ERR_VALUE;
  if (!aligned16(Z)) return KDKL_ERR_ALIGN;
  return KDKL_OK;
}

kdkl_status kdkl_logits_forward(const void* Z, const int32_t* ids, const float* lg, int64_t N, int64_t V,
                                int32_t K, float T, int dtype, float* loss, float* row_lse, float* row_kl,
                                void* stream) {
  kdkl_status st = check_logits(Z, ids, lg, N, V, K, T, dtype);
  if (st != KDKL_OK) return st;
  if (!loss || (N > 0 && (!row_lse || !row_kl))) return KDKL_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  LogitsArgs a;
  memset(&a, 0, sizeof(a));
  a.Z = Z; a.ids = ids; a.logits = lg; a.N = N; a.V = V; a.K = K; a.inv_T = 1.0f / T;
  a.row_lse = row_lse; a.row_kl = row_kl;
  const double es = dtype == KDKL_BF16 ? 2.0 : 4.0;
  hipError_t e = timed(K_LOGITS_FWD, 0.0, (double)N * (V * es + K * 8.0 + 8.0), s,
                       [&] { return launch_logits_fwd(dtype, a, s); });
  if (e == hipSuccess)
    e = timed(K_LOSS, 0.0, (double)N * 8.0, s, [&] { return launch_loss(row_kl, ids, K, N, loss, s); });
  return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
}

kdkl_status kdkl_logits_backward(const void* Z, const int32_t* ids, const float* lg, int64_t N, int64_t V,
                                 int32_t K, float T, int dtype, const float* row_lse, const float* grad_loss,
                                 void* dZ, void* workspace, size_t workspace_bytes, void* stream) {
  kdkl_status st = check_logits(Z, ids, lg, N, V, K, T, dtype);
  if (st != KDKL_OK) return st;
  if (N > 0 && (!row_lse || !dZ || !workspace)) return KDKL_ERR_NULL;
  if (!aligned16(dZ) || !aligned16(workspace)) return KDKL_ERR_ALIGN;
  if (N == 0) return KDKL_OK;
  if (workspace_bytes < KDKL_LOGITS_BWD_WORKSPACE) return KDKL_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  LogitsArgs a;
  memset(&a, 0, sizeof(a));
  a.Z = Z; a.dZ = dZ; a.ids = ids; a.logits = lg; a.N = N; a.V = V; a.K = K; a.inv_T = 1.0f / T;
  a.row_lse = const_cast<float*>(row_lse); a.scale = (const float*)workspace;
  const double es = dtype == KDKL_BF16 ? 2.0 : 4.0;
  hipError_t e = timed(K_GRAD_SCALE, 0.0, (double)N * 4.0, s,
                       [&] { return launch_grad_scale(ids, K, N, grad_loss, T, (float*)workspace, s); });
  if (e == hipSuccess) e = timed(K_LOGITS_BWD, 0.0, (double)N * (2.0 * V * es + K * 8.0 + 4.0), s,
                       [&] { return launch_logits_bwd(dtype, a, s); });
  return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
}

// --------------------------- teacher-id check ------------------------------

kdkl_status kdkl_check_ids(const int32_t* ids, int64_t N, int32_t K, int64_t V, int64_t* counts,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 0 || K < 1 || K > 1024 || V <= 0) return KDKL_ERR_SHAPE;
  if (N > ((int64_t)1 << 40) || V > ((int64_t)1 << 40)) return KDKL_ERR_OVERFLOW;
  if (!counts || !workspace || (N > 0 && !ids)) return KDKL_ERR_NULL;
  if (((uintptr_t)counts & 7u) || ((uintptr_t)workspace & 7u)) return KDKL_ERR_ALIGN;
  if (workspace_bytes < (size_t)KDKL_CHECK_IDS_WORKSPACE) return KDKL_ERR_WORKSPACE;
  static_assert(KDKL_CHECK_IDS_WORKSPACE >= kCheckIdsMaxBlocks * 2 * 8, "workspace holds every partial");
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = launch_check_ids(N > 0 ? ids : nullptr, N, K, V, workspace, counts, s);
  return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
}

// ------------------------------ dense KL ------------------------------------
// The pages' correctness baseline: the full student log-probability grid and
// the full teacher probability grid are built, compared grid-wide and kept
// for the backward pass. The GEMMs are those of the fused path run over one
// chunk of all N rows (the projection in raw-store mode).

struct DensePlan {
  Plan P;                      // chunk = N
  size_t f_z, f_rowkl, f_bytes;  // forward workspace: the logits [Cp, Vp]
  size_t s_logq, s_p, s_bytes;   // saved grids: logq and P, [N, Vp] fp32 each
};

static kdkl_status make_dense_plan(int64_t N, int64_t d, int64_t V, int32_t K, int dtype, DensePlan* D) {
  // the dense baseline keeps its whole dZ grid: one chunk of every position,
  // one vocabulary slice
  kdkl_options o{};
  o.chunks_per_group = 1;
  o.vocab_slices = 1;
  kdkl_status st = make_plan(N, d, V, K, N > 0 ? N : 1, dtype, &o, &D->P);
  if (st != KDKL_OK) return st;
  const Plan& P = D->P;
  int64_t z, g;
  size_t cur = 0;
  bool ok = mul_ok(P.Cp, P.Vp, &z) && mul_ok(z, P.es, &z);
  ok &= region(&cur, z, &D->f_z) && region(&cur, (N > 0 ? N : 1) * 4, &D->f_rowkl);
  D->f_bytes = cur;
  cur = 0;
  ok &= mul_ok(N > 0 ? N : 1, P.Vp, &g) && mul_ok(g, 4, &g);
  ok &= region(&cur, g, &D->s_logq) && region(&cur, g, &D->s_p);
  D->s_bytes = cur;
  return ok ? KDKL_OK : KDKL_ERR_OVERFLOW;
}

static DenseArgs dense_args(const DensePlan& D, const int32_t* ids, const float* lg, float T, char* saved) {
  DenseArgs a;
  memset(&a, 0, sizeof(a));
  a.logq = (float*)(saved + D.s_logq); a.P = (float*)(saved + D.s_p);
  a.ids = ids; a.logits = lg; a.N = D.P.N; a.V = D.P.V; a.ldv = D.P.Vp; a.rows_pad = D.P.Cp;
  a.K = (int)D.P.K; a.inv_T = 1.0f / T;
  return a;
}

kdkl_status kdkl_dense_sizes(int64_t N, int64_t d, int64_t V, int32_t K, int dtype, size_t* fwd_bytes,
                             size_t* saved_bytes, size_t* bwd_bytes) {
  DensePlan D;
  kdkl_status st = make_dense_plan(N, d, V, K, dtype, &D);
  if (st != KDKL_OK) return st;
  if (fwd_bytes) *fwd_bytes = D.f_bytes;
  if (saved_bytes) *saved_bytes = D.s_bytes;
  if (bwd_bytes) *bwd_bytes = D.P.b_bytes;
  return KDKL_OK;
}

kdkl_status kdkl_dense_forward(const void* H, const void* W, const int32_t* ids, const float* lg, int64_t N,
                               int64_t d, int64_t V, int32_t K, float T, int dtype, float* loss, float* row_lse,
                               float* row_kl, void* saved, size_t saved_bytes, void* workspace,
                               size_t workspace_bytes, void* stream) {
  DensePlan D;
  kdkl_status st = make_dense_plan(N, d, V, K, dtype, &D);
  if (st != KDKL_OK) return st;
  if ((st = check_common(H, W, ids, lg, N, T)) != KDKL_OK) return st;
  if (!loss || !saved || !workspace || (N > 0 && !row_lse)) return KDKL_ERR_NULL;
  if (workspace_bytes < D.f_bytes || saved_bytes < D.s_bytes) return KDKL_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(saved)) return KDKL_ERR_ALIGN;
  const Plan& P = D.P;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* kl = row_kl ? row_kl : (float*)(ws + D.f_rowkl);
  hipError_t e = hipSuccess;
  if (N > 0) {
    // the logit grid Z = H W^T [Cp, Vp] (zero past V)
    GemmArgs g = projection_args(P, H, W, T, 0, (int)N, ws, 0, 0);
    g.ent = nullptr; g.tstart = nullptr;
    g.raw = 1; g.dz_cv = ws + D.f_z; g.dz_vc = nullptr;
    e = timed(K_DENSE_GEMM, 2.0 * N * (double)V * d, ((double)V + N) * d * P.es + (double)N * V * P.es, s,
              [&] { return launch_gemm(dtype, EPI_DZ, g, s); });
    DenseArgs a = dense_args(D, ids, lg, T, (char*)saved);
    a.Z = ws + D.f_z; a.row_lse = row_lse; a.row_kl = kl;
    const double grid4 = (double)N * V * 4.0;
    if (e == hipSuccess)
      e = timed(K_DENSE_STUDENT, 0.0, 2.0 * N * (double)V * P.es + grid4, s,
                [&] { return launch_dense_student(dtype, a, s); });
    if (e == hipSuccess)
      e = timed(K_DENSE_TEACHER, 0.0, grid4 + (double)N * K * 8.0, s, [&] { return launch_dense_teacher(a, s); });
    if (e == hipSuccess)
      e = timed(K_DENSE_KL, 0.0, 2.0 * grid4, s, [&] { return launch_dense_kl(a, s); });
  }
  if (e == hipSuccess)
    e = timed(K_LOSS, 0.0, (double)N * 8.0, s, [&] { return launch_loss(kl, ids, K, N, loss, s); });
  return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
}

kdkl_status kdkl_dense_backward(const void* H, const void* W, const int32_t* ids, const float* lg, int64_t N,
                                int64_t d, int64_t V, int32_t K, float T, int dtype, const void* saved,
                                size_t saved_bytes, const float* grad_loss, void* dH, float* dW,
                                int accumulate_dW, void* workspace, size_t workspace_bytes, void* stream) {
  DensePlan D;
  kdkl_status st = make_dense_plan(N, d, V, K, dtype, &D);
  if (st != KDKL_OK) return st;
  if ((st = check_common(H, W, ids, lg, N, T)) != KDKL_OK) return st;
  if (!dW || !workspace || !saved || (N > 0 && !dH)) return KDKL_ERR_NULL;
  const Plan& P = D.P;
  if (workspace_bytes < P.b_bytes || saved_bytes < D.s_bytes) return KDKL_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(saved) || !aligned16(dW) || !aligned16(dH)) return KDKL_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t e = hipSuccess;
  if (N == 0) {
    if (!accumulate_dW) e = launch_zero(dW, V * d, s);
    return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
  }
  if (P.wt)
    e = timed(K_TRANSPOSE_W, 0.0, 2.0 * (double)V * d * P.es, s, [&] {
        return launch_transpose((int)P.es, W, V, d, d, ws + P.b_wt, P.Vp, P.Vp, s);
      });
  if (e == hipSuccess)
    e = timed(K_GRAD_SCALE, 0.0, (double)N * 4.0, s,
              [&] { return launch_grad_scale(ids, K, N, grad_loss, T, (float*)(ws + P.b_scale), s); });
  if (e == hipSuccess)
    e = timed(K_TRANSPOSE_H, 0.0, 2.0 * (double)N * d * P.es, s, [&] {
      return launch_transpose((int)P.es, H, N, d, d, ws + P.b_ht, P.Cp, P.Cp, s);
    });

  // dZ = g/(N_kept T) (exp(logq) - P), token-major [Cp, Vp], from the saved grids
  DenseArgs a = dense_args(D, ids, lg, T, (char*)const_cast<void*>(saved));
  a.dZ = ws + P.b_dzcv; a.scale = (const float*)(ws + P.b_scale);
  if (e == hipSuccess)
    e = timed(K_DENSE_GRAD, 0.0, 2.0 * N * (double)V * 4.0 + (double)P.Cp * P.Vp * P.es, s,
              [&] { return launch_dense_grad(dtype, a, s); });
  if (e == hipSuccess && !P.fast)  // the generic dW product reads dZ vocabulary-major
    e = launch_transpose((int)P.es, ws + P.b_dzcv, P.Cp, P.Vp, P.Vp, ws + P.b_dzvc, P.Cp, P.Cp, s);
  if (e == hipSuccess) e = part_products(P, dtype, W, ws, 0, (int)N, 0, dH, dW, accumulate_dW != 0, s);
  return e == hipSuccess ? KDKL_OK : KDKL_ERR_HIP;
}

kdkl_status kdkl_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (auto& r : g_prof.recs) {
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  g_prof.on = true;
  return KDKL_OK;
}

kdkl_status kdkl_profile_end(kdkl_kernel_stat* out, int capacity, int* count) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = false;
  kdkl_kernel_stat acc[K_COUNT];
  memset(acc, 0, sizeof(acc));
  kdkl_status st = KDKL_OK;
  for (auto& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      st = KDKL_ERR_HIP;
    kdkl_kernel_stat& k = acc[r.kid];
    k.launches += 1;
    k.total_ms += ms;
    k.flops += r.flops;
    k.bytes += r.bytes;
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  int n = 0;
  for (int i = 0; i < K_COUNT; ++i) {
    if (acc[i].launches == 0) continue;
    if (out && n < capacity) {
      out[n] = acc[i];
      strncpy(out[n].name, kernel_name(i), sizeof(out[n].name) - 1);
      out[n].name[sizeof(out[n].name) - 1] = 0;
    }
    ++n;
  }
  if (count) *count = n;
  return st;
}

}  // extern "C"
