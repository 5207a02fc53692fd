// Device kernels of the alternative losses on the fused chunked path's
// products: the generalised Jensen-Shannon divergence, the skew KL and the
// skew reverse KL between the teacher's top-K distribution and the student's
// full-vocabulary distribution.
//
// The pages report ablations on the choice of loss for the distilled
// student without naming the losses [P1 "Making knowledge distillation cheap
// enough to run at scale", section "The resulting student model"]; these are
// the readings taken. Per position, with P the teacher's top-K probabilities
// placed on the vocabulary (repeated ids add their mass, ids outside [0, V)
// have no entry), q = softmax(s), s = z / T, and a parameter a:
//   JSD   = a KL(P || M) + (1 - a) KL(q || M),  M = a P + (1 - a) q
//   SKL   = KL(P || M),                         M = a P + (1 - a) q
//   SRKL  = KL(q || M),                         M = a q + (1 - a) P
// Each gradient has the form dZ_v = coef q_v (g_v - gbar), gbar = sum_v q_v
// g_v, with g_v the derivative of the loss in q_v:
//   JSD   g = (1 - a) log(q / M)             off the support: -(1 - a) log(1 - a)
//   SKL   g = -(1 - a) P / M                 off the support: 0
//   SRKL  g = log(q / M) + 1 - a q / M       off the support: -log(a)
// Off the teacher's support each loss adds a constant per unit of student
// mass there (-(1 - a) log(1 - a), 0 and -log(a) respectively), so only the
// support (at most K entries per position) needs the student's logits
// individually. The projection epilogue forms dZ as a per-position
// coefficient of q_v, coef (g_off - gbar) >= 0 (g_v <= g_off on the support
// for all three), minus coef q_v (g_off - g_v) at each support entry, the
// same shape as the KL's softmax-minus-teacher; gbar comes from the forward
// (saved per position beside the logsumexp), so the backward needs no pass
// over the support before its projections.
//
// Two kernels, one wavefront per position:
//   jsd_merge  forward: lse from the split-vocabulary partials, then, from
//              s at each teacher entry (kept by the projection epilogue as it
//              meets the entry), the loss and gbar
//   jsd_prep   backward: each position's coefficient of q in dZ, and the
//              teacher mass of each distinct id written over its first
//              entry's probability (0 over repeats) for the dZ epilogue
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kdkl_internal.h"

namespace kdkl {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRowsPerBlock = 4;          // one wavefront per position

__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float log_hw(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

__device__ __forceinline__ float wsum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

struct Sums {
  float t;   // the support's part of the loss
  float gq;  // the support's part of gbar: sum_S q g
  float qs;  // sum_S q
};

// log(exp(u) + exp(w)), either of them possibly -inf (not both)
__device__ __forceinline__ float log_add(float u, float w) {
  const float hi = fmaxf(u, w), lo = fminf(u, w);
  return hi + log1pf(exp_hw(lo - hi));
}

// The support terms of one position (each lane its share of the sorted
// entries; not yet summed over the wavefront).
__device__ __forceinline__ Sums support_terms(const JsdArgs& a, int row, float lse) {
  const int lane = threadIdx.x & 63;
  const int2* ent = a.ent + (int64_t)row * a.K;
  const float* sk = a.sk + (int64_t)row * a.K;
  const float al = a.beta, oma = 1.f - al;
  Sums r{0.f, 0.f, 0.f};
  for (int j = lane; j < a.K; j += 64) {
    const int2 e = ent[j];
    if (e.x < 0 || e.x >= a.V || (j > 0 && ent[j - 1].x == e.x)) continue;
    float P = __int_as_float(e.y);
    for (int j2 = j + 1; j2 < a.K && ent[j2].x == e.x; ++j2) P += __int_as_float(ent[j2].y);
    if (!(P > 0.f)) continue;  // no teacher mass: the entry is off the support
    const float lq = sk[j] - lse;  // log q
    const float q = exp_hw(lq);
    const float lp = log_hw(P);
    if (a.loss == ALT_SRKL) {
      // log M = log(a q + (1 - a) P)
      const float rq = lq - log_add(a.log_beta + lq, a.log_omb + lp);  // log(q / M)
      r.t += q * rq;
      r.gq += q * (rq + 1.f - al * exp_hw(rq));
    } else {
      // log M = log(a P + (1 - a) q)
      const float lm = log_add(a.log_beta + lp, a.log_omb + lq);
      if (a.loss == ALT_SKL) {
        r.t += P * (lp - lm);
        r.gq += -oma * exp_hw(lq + lp - lm);  // q P / M as one bounded exponential
      } else {
        r.t += al * P * (lp - lm) + oma * q * (lq - lm);
        r.gq += oma * q * (lq - lm);
      }
    }
    r.qs += q;
  }
  return r;
}

// The loss's value and g per unit of student mass off the teacher's support.
__device__ __forceinline__ float off_support(const JsdArgs& a) {
  if (a.loss == ALT_SKL) return 0.f;
  if (a.loss == ALT_SRKL) return -a.log_beta;
  return -(1.f - a.beta) * a.log_omb;
}

// Online logsumexp of one position's split-vocabulary partials (max, sum of
// exp, -, -), natural log; the same merge as the KL forward's.
__device__ __forceinline__ float lse_of_partials(const float4* p, int n_vt) {
  const int lane = threadIdx.x & 63;
  float m = kNegInf, s = 0.f;
  for (int t = lane; t < n_vt; t += 64) {
    const float4 v = p[t];
    if (v.x > kNegInf) {
      const float nm = fmaxf(m, v.x);
      s = s * exp_hw(m - nm) + v.y * exp_hw(v.x - nm);
      m = nm;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const float os = __shfl_xor(s, o, 64);
    const float nm = fmaxf(m, om);
    if (nm > kNegInf) {
      s = (m > kNegInf ? s * exp_hw(m - nm) : 0.f) + (om > kNegInf ? os * exp_hw(om - nm) : 0.f);
      m = nm;
    }
  }
  return m + log_hw(s);
}

__global__ __launch_bounds__(64 * kRowsPerBlock) void jsd_merge_kernel(JsdArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const bool keep = a.keep[row] != 0.f;
  const float lse = lse_of_partials(a.part + (int64_t)row * a.n_vt, a.n_vt);
  // an ignored position's entries were never met by the epilogue
  Sums r = keep ? support_terms(a, row, lse) : Sums{0.f, 0.f, 0.f};
  r.t = wsum(r.t);
  r.gq = wsum(r.gq);
  r.qs = wsum(r.qs);
  if (lane == 0) {
    // the off-support entries: the same constant in the loss and in g
    const float off = off_support(a) * (1.f - r.qs);
    a.row_lse[row] = lse;
    a.row_kl[row] = keep ? r.t + off : 0.f;
    a.row_gbar[row] = keep ? r.gq + off : 0.f;  // sum_v q_v g_v
  }
}

__global__ __launch_bounds__(64 * kRowsPerBlock) void jsd_prep_kernel(JsdArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const bool keep = a.keep[row] != 0.f;
  int2* ent = a.ent + (int64_t)row * a.K;
  // each lane reads its entries' runs before any lane writes: the masses
  // are summed into registers first
  constexpr int kMaxPerLane = 1024 / 64;
  float mass[kMaxPerLane];
#pragma unroll
  for (int t = 0; t < kMaxPerLane; ++t) {
    mass[t] = 0.f;
    const int j = lane + 64 * t;
    if (!keep || j >= a.K) continue;
    const int id = ent[j].x;
    if (id < 0 || id >= a.V || (j > 0 && ent[j - 1].x == id)) continue;
    float P = __int_as_float(ent[j].y);
    for (int j2 = j + 1; j2 < a.K && ent[j2].x == id; ++j2) P += __int_as_float(ent[j2].y);
    mass[t] = P;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int t = 0; t < kMaxPerLane; ++t) {
    const int j = lane + 64 * t;
    if (j < a.K) ent[j].y = __float_as_int(mass[t]);
  }
  if (lane == 0) a.rowcoef[row] = keep ? a.scale[0] * (off_support(a) - a.row_gbar_in[row]) : 0.f;
}

dim3 rows_grid(int rows) { return dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)); }

// ---------------------------------------------------------------------------
// Reverse KL over the teacher's top-K support (one wavefront per position):
// the student's distribution restricted to the support S (the distinct
// in-range teacher ids with mass) and renormalised there, qt = softmax(s_S),
// and TRKL = sum_S qt (log qt - log P). It needs the student's logits at S
// only: each is a dot product of a row of W with the position's H, read as
// 16-byte vectors across the wavefront. Its gradient in s is
// qt (log(qt / P) - TRKL) on S and 0 elsewhere.
// ---------------------------------------------------------------------------
template <typename TE>
struct Vec16;
template <>
struct Vec16<uint16_t> {  // bf16 bits
  static constexpr int kN = 8;
  __device__ static void unpack(const uint4& u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __builtin_bit_cast(float, w[j] << 16);
      x[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
    }
  }
  __device__ static void store(uint16_t* p, float v) { *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
  __device__ static void store_vec(uint16_t* p, const float (&x)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2 * j])) |
             ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2 * j + 1])) << 16);
    *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec16<float> {
  static constexpr int kN = 4;
  __device__ static void unpack(const uint4& u, float (&x)[4]) {
    x[0] = __builtin_bit_cast(float, u.x);
    x[1] = __builtin_bit_cast(float, u.y);
    x[2] = __builtin_bit_cast(float, u.z);
    x[3] = __builtin_bit_cast(float, u.w);
  }
  __device__ static void store(float* p, float v) { *p = v; }
  __device__ static void store_vec(float* p, const float (&x)[4]) { *(float4*)p = make_float4(x[0], x[1], x[2], x[3]); }
};

__device__ __forceinline__ float wmax(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// The support of a kept position and its masses, each lane its entries: an
// id's first entry (the entries are sorted by id) gets the summed mass of its
// repeats, every other entry 0, and so does every entry of an id outside
// [0, V) and of an ignored position.
__device__ __forceinline__ void support_masses(const int2* ent, int K, int64_t V, bool keep, int lane, float* sP) {
  for (int k = lane; k < K; k += 64) {
    const int2 e = ent[k];
    float P = 0.f;
    if (keep && e.x >= 0 && e.x < V && (k == 0 || ent[k - 1].x != e.x)) {
      P = __int_as_float(e.y);
      for (int k2 = k + 1; k2 < K && ent[k2].x == e.x; ++k2) P += __int_as_float(ent[k2].y);
    }
    sP[k] = P;
  }
  __builtin_amdgcn_wave_barrier();
}

// a row's gradient at one support entry from its logit, the forward's
// logsumexp over the support and the forward's loss
__device__ __forceinline__ float trkl_grad(float s, float P, float lse, float L, float coef) {
  const float lq = s - lse;
  return coef * exp_hw(lq) * (lq - log_hw(P) - L);
}

// The forward's outputs of a position from its support logits sS and masses
// sP (each lane its entries): the logsumexp over the support (-inf for an
// empty one) and the loss.
__device__ __forceinline__ void trkl_forward_out(const TopkArgs& a, int row, int lane, int K, bool keep,
                                                 const float* sS, const float* sP) {
  float m = kNegInf;
  for (int k = lane; k < K; k += 64)
    if (sP[k] > 0.f) m = fmaxf(m, sS[k]);
  m = wmax(m);
  float se = 0.f;
  for (int k = lane; k < K; k += 64)
    if (sP[k] > 0.f) se += exp_hw(sS[k] - m);
  se = wsum(se);
  const float lse = m > kNegInf ? m + log_hw(se) : kNegInf;
  float L = 0.f;
  for (int k = lane; k < K; k += 64) {
    const float P = sP[k];
    if (P > 0.f) {
      const float lq = sS[k] - lse;
      L += exp_hw(lq) * (lq - log_hw(P));
    }
  }
  L = wsum(L);
  if (lane == 0) {
    a.row_lse[row] = lse;
    a.row_loss[row] = L;
    a.row_kl[row] = keep ? L : 0.f;
  }
}

template <typename TE, int KMAX>  // K <= KMAX
__global__ __launch_bounds__(64 * kRowsPerBlock) void topk_rkl_kernel(TopkArgs a, int backward) {
  __shared__ float s_s[kRowsPerBlock][KMAX];  // s at each sorted entry of the support
  __shared__ float s_P[kRowsPerBlock][KMAX];  // its teacher mass (0 off the support)
  constexpr int VEC = Vec16<TE>::kN;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * kRowsPerBlock + w;
  if (row >= a.rows) return;
  const int K = a.K;
  const int2* ent = a.ent + (int64_t)row * K;
  const bool keep = a.keep[row] != 0.f;
  const int64_t nvec = a.d / VEC;
  const uint4* hp = (const uint4*)((const TE*)a.H + (int64_t)row * a.d);
  support_masses(ent, K, a.V, keep, lane, s_P[w]);
  // the student's logits there, kDots entries at a time across the
  // wavefront (their rows of W read together; an entry off the support
  // reads row 0 and is not kept)
  constexpr int kDots = 4;
  for (int k0 = 0; k0 < K; k0 += kDots) {
    const uint4* wp[kDots];
    bool on[kDots];
#pragma unroll
    for (int q = 0; q < kDots; ++q) {
      const int k = k0 + q;
      const int kc = k < K ? k : K - 1;
      on[q] = k < K && s_P[w][kc] > 0.f;
      wp[q] = (const uint4*)((const TE*)a.W + (on[q] ? (int64_t)ent[kc].x : 0) * a.d);
    }
    float acc[kDots] = {};
    for (int64_t j = lane; j < nvec; j += 64) {
      float y[VEC];
      Vec16<TE>::unpack(hp[j], y);
#pragma unroll
      for (int q = 0; q < kDots; ++q) {
        float x[VEC];
        Vec16<TE>::unpack(wp[q][j], x);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[q] = __builtin_fmaf(x[i], y[i], acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kDots; ++q) {
      const float sv = wsum(acc[q]) * a.inv_T;
      if (lane == 0 && k0 + q < K) s_s[w][k0 + q] = on[q] ? sv : 0.f;
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (!backward) {
    trkl_forward_out(a, row, lane, K, keep, s_s[w], s_P[w]);
    return;
  }
  // the gradient at each sorted entry, from the forward's logsumexp and loss
  // (kept in s_s in place of s)
  const float lse = a.row_lse[row], L = a.row_loss[row];
  const float coef = keep ? a.scale[0] : 0.f;
  for (int k = lane; k < K; k += 64) {
    const float P = s_P[w][k];
    const float gk = P > 0.f ? trkl_grad(s_s[w][k], P, lse, L, coef) : 0.f;
    a.dz[(int64_t)row * K + k] = gk;
    s_s[w][k] = gk;
  }
  __builtin_amdgcn_wave_barrier();
  // dH row = sum over the support of dz_k W[id_k], in entry order: kRep
  // vectors per lane at a time, the rows of kDots entries read together
  constexpr int kRep = 2;
  TE* dh = (TE*)a.dH + (int64_t)row * a.d;
  for (int64_t j0 = 0; j0 < nvec; j0 += 64 * kRep) {
    float acc[kRep][VEC] = {};
    for (int k0 = 0; k0 < K; k0 += kDots) {
      const uint4* wp[kDots];
      float gq[kDots];
#pragma unroll
      for (int q = 0; q < kDots; ++q) {
        const int k = k0 + q;
        const int kc = k < K ? k : K - 1;
        gq[q] = k < K ? s_s[w][kc] : 0.f;
        wp[q] = (const uint4*)((const TE*)a.W + (gq[q] != 0.f ? (int64_t)ent[kc].x : 0) * a.d);
      }
#pragma unroll
      for (int r = 0; r < kRep; ++r) {
        const int64_t j = j0 + lane + 64 * r;
        if (j < nvec) {
#pragma unroll
          for (int q = 0; q < kDots; ++q) {
            float x[VEC];
            Vec16<TE>::unpack(wp[q][j], x);
            // (an entry without gradient read row 0, which must add nothing)
#pragma unroll
            for (int i = 0; i < VEC; ++i) acc[r][i] = gq[q] != 0.f ? __builtin_fmaf(gq[q], x[i], acc[r][i]) : acc[r][i];
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRep; ++r) {
      const int64_t j = j0 + lane + 64 * r;
      if (j < nvec) Vec16<TE>::store_vec(dh + j * VEC, acc[r]);
    }
  }
}

// Both calls with each support row of W read once, into registers, for rows
// of at most 64 JMAX 16-byte vectors: the forward takes each row's dot
// product; the backward, with the forward's logsumexp and loss at hand, needs
// only an entry's own logit for its gradient, so it adds the row's share of
// the dH row while the row is still in registers (half the bytes of the
// two-pass form above, whose second pass reads the rows again). Rows go
// kDots at a time, two groups in flight. The products and the order of every
// sum are those of the two-pass kernel (the dot products lane by lane in
// vector order, dH in entry order), so both give the same bits.
template <typename TE, int KMAX, int JMAX, bool BWD>
__global__ __launch_bounds__(64 * kRowsPerBlock) void topk_rkl_rows_kernel(TopkArgs a) {
  __shared__ float s_g[kRowsPerBlock][KMAX];  // forward: s at each sorted entry; backward: the gradient there
  __shared__ float s_P[kRowsPerBlock][KMAX];  // its teacher mass (0 off the support)
  constexpr int VEC = Vec16<TE>::kN;
  constexpr int kDots = 2;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * kRowsPerBlock + w;
  if (row >= a.rows) return;
  const int K = a.K;
  const int2* ent = a.ent + (int64_t)row * K;
  const bool keep = a.keep[row] != 0.f;
  const int nvec = (int)(a.d / VEC);  // <= 64 JMAX
  // each lane's vectors of a row, clamped to the row's last so that every
  // load is a whole 16-byte load (the vectors past the row are not used)
  int jv[JMAX];
#pragma unroll
  for (int r = 0; r < JMAX; ++r) jv[r] = min(lane + 64 * r, nvec - 1);
  const uint4* hp = (const uint4*)((const TE*)a.H + (int64_t)row * a.d);
  uint4 hv[JMAX];
#pragma unroll
  for (int r = 0; r < JMAX; ++r) hv[r] = hp[jv[r]];
  support_masses(ent, K, a.V, keep, lane, s_P[w]);
  const float lse = BWD ? a.row_lse[row] : 0.f, L = BWD ? a.row_loss[row] : 0.f;
  const float coef = BWD && keep ? a.scale[0] : 0.f;
  float acc[JMAX][VEC] = {};
  // a group's rows (an entry off the support, or past K, reads row 0 and is
  // not kept)
  auto load_group = [&](uint4 (&xv)[kDots][JMAX], float (&P)[kDots], int k0) {
#pragma unroll
    for (int q = 0; q < kDots; ++q) {
      const int k = k0 + q;
      const int kc = k < K ? k : K - 1;
      P[q] = k < K ? s_P[w][kc] : 0.f;
      const int id = __builtin_amdgcn_readfirstlane(P[q] > 0.f ? ent[kc].x : 0);
      const uint4* wp = (const uint4*)((const TE*)a.W + (int64_t)id * a.d);
#pragma unroll
      for (int r = 0; r < JMAX; ++r) xv[q][r] = wp[jv[r]];
    }
  };
  // its dot products, gradients and shares of the dH row
  auto use_group = [&](const uint4 (&xv)[kDots][JMAX], const float (&P)[kDots], int k0) {
#pragma unroll
    for (int q = 0; q < kDots; ++q) {
      float dot = 0.f;
#pragma unroll
      for (int r = 0; r < JMAX; ++r) {
        if (lane + 64 * r < nvec) {
          float x[VEC], y[VEC];
          Vec16<TE>::unpack(xv[q][r], x);
          Vec16<TE>::unpack(hv[r], y);
#pragma unroll
          for (int i = 0; i < VEC; ++i) dot = __builtin_fmaf(x[i], y[i], dot);
        }
      }
      const float sv = wsum(dot) * a.inv_T;
      if (!BWD) {
        if (lane == 0 && k0 + q < K) s_g[w][k0 + q] = P[q] > 0.f ? sv : 0.f;
        continue;
      }
      const float gk = P[q] > 0.f ? trkl_grad(sv, P[q], lse, L, coef) : 0.f;
      if (lane == 0 && k0 + q < K) s_g[w][k0 + q] = gk;
      if (gk != 0.f) {  // (wave-uniform)
#pragma unroll
        for (int r = 0; r < JMAX; ++r) {
          float x[VEC];
          Vec16<TE>::unpack(xv[q][r], x);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[r][i] = __builtin_fmaf(gk, x[i], acc[r][i]);
        }
      }
    }
  };
  // two groups in flight: the next group's loads go out before the current
  // group's arithmetic
  uint4 xa[kDots][JMAX], xb[kDots][JMAX];
  float Pa[kDots], Pb[kDots];
  load_group(xa, Pa, 0);
  for (int k0 = 0; k0 < K; k0 += 2 * kDots) {
    load_group(xb, Pb, k0 + kDots);
    use_group(xa, Pa, k0);
    load_group(xa, Pa, k0 + 2 * kDots);
    use_group(xb, Pb, k0 + kDots);
  }
  __builtin_amdgcn_wave_barrier();
  if (!BWD) {
    trkl_forward_out(a, row, lane, K, keep, s_g[w], s_P[w]);
    return;
  }
  for (int k = lane; k < K; k += 64) a.dz[(int64_t)row * K + k] = s_g[w][k];
  TE* dh = (TE*)a.dH + (int64_t)row * a.d;
#pragma unroll
  for (int r = 0; r < JMAX; ++r)
    if (lane + 64 * r < nvec) Vec16<TE>::store_vec(dh + (int64_t)(lane + 64 * r) * VEC, acc[r]);
}

__global__ __launch_bounds__(256) void zero16_kernel(uint4* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------
// dW of the reverse KL over the top-K support without a dense product:
// dW_v = sum over the positions r whose support holds v of dz_rv H_r, summed
// in position order. The support entries (nonzero entry gradients) are
// bucketed by id with a counting sort that keeps position order: per block
// of kBucketRows positions, counts per id (integer atomics: the counts do not
// depend on their order); an exclusive scan over the blocks per id and over
// the ids; then each block's workgroup walks its positions in order and
// places their entries (one entry per id per position, so the atomic that
// hands out slots runs in position order); one workgroup per id then sums
// its bucket.
// ---------------------------------------------------------------------------
constexpr int kBucketRows = 256;
static_assert(kBucketRows == 256, "trkl_count_bytes counts blocks of 256 positions");

__global__ __launch_bounds__(256) void trkl_count_kernel(const int2* ent, const float* dz, int64_t n, int K,
                                                         int64_t V, int* cnt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n || dz[i] == 0.f) return;
  const int v = ent[i].x;
  if (v < 0 || v >= V) return;  // (a nonzero gradient is only ever at an id in range)
  const int64_t b = (i / K) / kBucketRows;
  atomicAdd(&cnt[b * V + v], 1);
}

// per id: the counts of the blocks turned into exclusive offsets within the
// id's bucket, and the bucket's size
__global__ __launch_bounds__(256) void trkl_scan_blocks_kernel(int* cnt, int nb, int64_t V, int64_t* total) {
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  int acc = 0;
  for (int b = 0; b < nb; ++b) {
    const int c = cnt[(int64_t)b * V + v];
    cnt[(int64_t)b * V + v] = acc;
    acc += c;
  }
  total[v] = acc;
}

// A bucket of more than kChunk entries is summed by several workgroups, one
// per run of kChunk entries, into fp32 partial rows that a second pass adds
// to dW in run order (the Zipf-like head of the teacher ids puts one id at
// nearly every position).
constexpr int64_t kChunk = 1024;
__device__ __forceinline__ int64_t trkl_runs(int64_t n) { return (n + kChunk - 1) / kChunk; }

__device__ __forceinline__ int64_t shfl_up64(int64_t v, int d) {
  const int lo = __shfl_up((int)(uint32_t)v, d, 64), hi = __shfl_up((int)(v >> 32), d, 64);
  return ((int64_t)hi << 32) | (uint32_t)lo;
}
// the four quantities an id's bucket adds to the scans below
__device__ __forceinline__ void trkl_terms(int64_t n, int64_t (&x)[4]) {
  const int64_t r = trkl_runs(n);
  x[0] = n;
  x[1] = r;
  x[2] = r > 1 ? r : 0;
  x[3] = r > 1 ? 1 : 0;
}

// Exclusive scans over the ids, each with its total at index V:
//   base:   bucket sizes (the bucket's first slot in the sorted list)
//   rstart: runs of kChunk entries (the workgroup of a bucket's first run)
//   pstart: the same over the buckets of more than one run (partial rows)
//   mstart: the buckets of more than one run
// in three passes over tiles of 256 ids (one per thread): the tiles' sums,
// their exclusive scan (one workgroup), and each tile's scan from its offset.
constexpr int kScanTile = 256;
constexpr int kScanWaves = kScanTile / 64;

// inclusive prefix sums of x across the workgroup's threads (wavefront
// scans, then the scan of the wavefront totals); tot gets the total
__device__ __forceinline__ void block_scan4(int64_t (&x)[4], int64_t (&tot)[4], int64_t (*s_w)[kScanWaves]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t y = shfl_up64(x[c], d);
      if (lane >= d) x[c] += y;
    }
    if (lane == 63) s_w[c][w] = x[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int64_t off = 0;
    tot[c] = 0;
    for (int u = 0; u < kScanWaves; ++u) {
      off += u < w ? s_w[c][u] : 0;
      tot[c] += s_w[c][u];
    }
    x[c] += off;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kScanTile) void trkl_scan_tiles_kernel(const int64_t* total, int64_t V, int64_t* tsum) {
  __shared__ int64_t s_w[4][kScanWaves];
  const int64_t i = (int64_t)blockIdx.x * kScanTile + threadIdx.x;
  int64_t x[4] = {0, 0, 0, 0}, tot[4];
  if (i < V) trkl_terms(total[i], x);
  block_scan4(x, tot, s_w);
  if (threadIdx.x < 4) tsum[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = tot[threadIdx.x];
}

// exclusive scan of the tiles' sums (nt of each quantity), in place, in
// chunks of 1024 with a running offset
__global__ __launch_bounds__(kScanTile) void trkl_scan_sums_kernel(int64_t* tsum, int64_t nt) {
  __shared__ int64_t s_w[4][kScanWaves];
  int64_t run[4] = {0, 0, 0, 0};
  for (int64_t t0 = 0; t0 < nt; t0 += kScanTile) {
    const int64_t t = t0 + threadIdx.x;
    int64_t x[4], own[4], tot[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) own[c] = x[c] = t < nt ? tsum[c * nt + t] : 0;
    block_scan4(x, tot, s_w);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (t < nt) tsum[c * nt + t] = run[c] + x[c] - own[c];
      run[c] += tot[c];
    }
  }
}

// Also the tables that map a run to its id and a bucket of several runs to
// its id (for the workgroups that sum them).
__global__ __launch_bounds__(kScanTile) void trkl_scan_out_kernel(const int64_t* total, int64_t V, const int64_t* tsum,
                                                                 int64_t* base, int64_t* rstart, int64_t* pstart,
                                                                 int64_t* mstart, int* run_id, int* multi_id) {
  __shared__ int64_t s_w[4][kScanWaves];
  int64_t* out[4] = {base, rstart, pstart, mstart};
  const int64_t nt = gridDim.x;
  const int64_t i = (int64_t)blockIdx.x * kScanTile + threadIdx.x;
  int64_t x[4] = {0, 0, 0, 0}, own[4], tot[4];
  if (i < V) trkl_terms(total[i], x);
#pragma unroll
  for (int c = 0; c < 4; ++c) own[c] = x[c];
  block_scan4(x, tot, s_w);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t off = tsum[c * nt + blockIdx.x];
    if (i < V) out[c][i] = off + x[c] - own[c];
    if (blockIdx.x == nt - 1 && threadIdx.x == 0) out[c][V] = off + tot[c];
    x[c] = off + x[c] - own[c];  // this id's exclusive offset
  }
  if (i < V) {
    for (int64_t r = 0; r < own[1]; ++r) run_id[x[1] + r] = (int)i;
    if (own[3]) multi_id[x[3]] = (int)i;
  }
}

__global__ __launch_bounds__(256) void trkl_place_kernel(const int2* ent, const float* dz, int rows, int K,
                                                         int64_t V, int* cnt, const int64_t* base, int2* list) {
  const int b = blockIdx.x;
  const int r0 = b * kBucketRows;
  const int r1 = r0 + kBucketRows < rows ? r0 + kBucketRows : rows;
  for (int r = r0; r < r1; ++r) {
    for (int k = threadIdx.x; k < K; k += 256) {
      const int64_t i = (int64_t)r * K + k;
      const float g = dz[i];
      const int v = ent[i].x;
      if (g != 0.f && v >= 0 && v < V) {
        const int o = atomicAdd(&cnt[(int64_t)b * V + v], 1);
        list[base[v] + o] = make_int2(r, __float_as_int(g));
      }
    }
    __syncthreads();  // the next position's slots after this one's
  }
}

// One workgroup per run of a bucket (launched for the most runs there can
// be; the ones past the total exit): the run's sum of dz H_r over its
// entries in order, added to dW's row for a bucket of one run (written over
// it when dW is overwritten), else written as the run's partial row.
template <typename TE>
__global__ __launch_bounds__(256) void trkl_dw_runs_kernel(const int2* list, const int64_t* base,
                                                           const int64_t* rstart, const int64_t* pstart,
                                                           const int* run_id, int64_t V, const void* H, int64_t d,
                                                           float* dW, float* part, int overwrite) {
  constexpr int VEC = Vec16<TE>::kN;
  constexpr int kRep = 2;
  const int64_t w = blockIdx.x;
  if (w >= rstart[V]) return;
  const int64_t v = run_id[w];
  const int64_t c = w - rstart[v];
  const int64_t runs = rstart[v + 1] - rstart[v];
  const int64_t lo = base[v] + c * kChunk;
  const int64_t hi = lo + kChunk < base[v + 1] ? lo + kChunk : base[v + 1];
  const int64_t nvec = d / VEC;
  const uint4* h = (const uint4*)H;
  float* out = runs == 1 ? dW + v * d : part + (pstart[v] + c) * d;
  for (int64_t j0 = 0; j0 < nvec; j0 += 256 * kRep) {
    float acc[kRep][VEC] = {};
    for (int64_t e = lo; e < hi; ++e) {
      const int2 en = list[e];
      const float g = __int_as_float(en.y);
#pragma unroll
      for (int q = 0; q < kRep; ++q) {
        const int64_t j = j0 + threadIdx.x + 256 * q;
        if (j < nvec) {
          float x[VEC];
          Vec16<TE>::unpack(h[(int64_t)en.x * nvec + j], x);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[q][i] = __builtin_fmaf(g, x[i], acc[q][i]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kRep; ++q) {
      const int64_t j = j0 + threadIdx.x + 256 * q;
      if (j < nvec) {
        float4* o4 = (float4*)(out + j * VEC);
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
          float4 y = make_float4(acc[q][4 * i], acc[q][4 * i + 1], acc[q][4 * i + 2], acc[q][4 * i + 3]);
          if (runs == 1 && !overwrite) {  // dW += the bucket's sum
            const float4 old = o4[i];
            y.x += old.x; y.y += old.y; y.z += old.z; y.w += old.w;
          }
          o4[i] = y;
        }
      }
    }
  }
}

// One workgroup per bucket of more than one run: dW's row += its runs'
// partial rows, in run order (from zero when dW is overwritten).
__global__ __launch_bounds__(256) void trkl_dw_combine_kernel(const int64_t* rstart, const int64_t* pstart,
                                                              const int64_t* mstart, const int* multi_id, int64_t V,
                                                              int64_t d, const float* part, float* dW,
                                                              int overwrite) {
  const int64_t m = blockIdx.x;
  if (m >= mstart[V]) return;
  const int64_t v = multi_id[m];
  const int64_t runs = rstart[v + 1] - rstart[v];
  const float* p = part + pstart[v] * d;
  float* out = dW + v * d;
  for (int64_t j = threadIdx.x; j < d / 4; j += 256) {
    float4 y = overwrite ? make_float4(0.f, 0.f, 0.f, 0.f) : ((const float4*)out)[j];
    for (int64_t c = 0; c < runs; ++c) {
      const float4 x = ((const float4*)(p + c * d))[j];
      y.x += x.x; y.y += x.y; y.z += x.z; y.w += x.w;
    }
    ((float4*)out)[j] = y;
  }
}

// dW's rows of the ids without entries, when dW is written rather than added
// to (the other rows are written whole by the runs or their combination)
__global__ __launch_bounds__(256) void trkl_zero_rows_kernel(const int64_t* total, int64_t V, int64_t d, float* dW) {
  const int64_t v = blockIdx.x;
  if (v >= V || total[v] != 0) return;
  float4* out = (float4*)(dW + v * d);
  for (int64_t j = threadIdx.x; j < d / 4; j += 256) out[j] = make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t zero_bytes(void* p, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p, n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_jsd_merge(const JsdArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.K < 1 || a.K > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(jsd_merge_kernel, rows_grid(a.rows), dim3(64 * kRowsPerBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_jsd_prep(const JsdArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.K < 1 || a.K > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(jsd_prep_kernel, rows_grid(a.rows), dim3(64 * kRowsPerBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk_rkl(int dtype, const TopkArgs& a, bool backward, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.K < 1 || a.K > 1024) return hipErrorInvalidValue;
  if (a.d % (dtype == 1 ? 8 : 4) != 0) return hipErrorInvalidValue;  // rows of whole 16-byte vectors
  const dim3 grid = rows_grid(a.rows), block(64 * kRowsPerBlock);
  const int b = backward ? 1 : 0;
  if (topk_rkl_one_pass(dtype, a.d)) {
    if (dtype == 1) {
      if (a.K <= 128) {
        if (backward) hipLaunchKernelGGL((topk_rkl_rows_kernel<uint16_t, 128, 6, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((topk_rkl_rows_kernel<uint16_t, 128, 6, false>), grid, block, 0, s, a);
      } else {
        if (backward) hipLaunchKernelGGL((topk_rkl_rows_kernel<uint16_t, 1024, 6, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((topk_rkl_rows_kernel<uint16_t, 1024, 6, false>), grid, block, 0, s, a);
      }
    } else {
      if (a.K <= 128) {
        if (backward) hipLaunchKernelGGL((topk_rkl_rows_kernel<float, 128, 6, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((topk_rkl_rows_kernel<float, 128, 6, false>), grid, block, 0, s, a);
      } else {
        if (backward) hipLaunchKernelGGL((topk_rkl_rows_kernel<float, 1024, 6, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((topk_rkl_rows_kernel<float, 1024, 6, false>), grid, block, 0, s, a);
      }
    }
    return hipGetLastError();
  }
  if (dtype == 1) {
    if (a.K <= 128) hipLaunchKernelGGL((topk_rkl_kernel<uint16_t, 128>), grid, block, 0, s, a, b);
    else hipLaunchKernelGGL((topk_rkl_kernel<uint16_t, 1024>), grid, block, 0, s, a, b);
  } else {
    if (a.K <= 128) hipLaunchKernelGGL((topk_rkl_kernel<float, 128>), grid, block, 0, s, a, b);
    else hipLaunchKernelGGL((topk_rkl_kernel<float, 1024>), grid, block, 0, s, a, b);
  }
  return hipGetLastError();
}

hipError_t launch_trkl_dw(int dtype, const int2* ent, const float* dz, int rows, int K, int64_t V,
                          const void* H, int64_t d, float* dW, bool accumulate, int* cnt, int64_t* scans,
                          int2* list, float* part, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K < 1 || K > 1024 || d % (dtype == 1 ? 8 : 4) != 0 || V >= INT32_MAX) return hipErrorInvalidValue;
  const int nb = (rows + kBucketRows - 1) / kBucketRows;
  const int64_t n = (int64_t)rows * K;
  int64_t* total = scans;
  int64_t* base = scans + (V + 1);
  int64_t* rstart = scans + 2 * (V + 1);
  int64_t* pstart = scans + 3 * (V + 1);
  int64_t* mstart = scans + 4 * (V + 1);
  // after the tiles' sums: the id of each run, then of each bucket of several runs
  int* run_id = (int*)(scans + 5 * (V + 1) + 4 * ((V + kScanTile - 1) / kScanTile));
  int* multi_id = run_id + V + n / kChunk + 1;
  hipError_t e = zero_bytes(cnt, trkl_count_bytes(rows, V), s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(trkl_count_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ent, dz, n, K, V, cnt);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(trkl_scan_blocks_kernel, dim3((unsigned)((V + 255) / 256)), dim3(256), 0, s, cnt, nb, V,
                       total);
    e = hipGetLastError();
  }
  if (e == hipSuccess && !accumulate) {  // (d a multiple of 4: whole float4 rows)
    hipLaunchKernelGGL(trkl_zero_rows_kernel, dim3((unsigned)V), dim3(256), 0, s, total, V, d, dW);
    e = hipGetLastError();
  }
  const int64_t nt = (V + kScanTile - 1) / kScanTile;
  int64_t* tsum = scans + 5 * (V + 1);  // [4, nt]
  if (e == hipSuccess) {
    hipLaunchKernelGGL(trkl_scan_tiles_kernel, dim3((unsigned)nt), dim3(kScanTile), 0, s, total, V, tsum);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(trkl_scan_sums_kernel, dim3(1), dim3(kScanTile), 0, s, tsum, nt);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(trkl_scan_out_kernel, dim3((unsigned)nt), dim3(kScanTile), 0, s, total, V, tsum, base, rstart,
                       pstart, mstart, run_id, multi_id);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    hipLaunchKernelGGL(trkl_place_kernel, dim3((unsigned)nb), dim3(256), 0, s, ent, dz, rows, K, V, cnt, base, list);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  // at most one run per id plus one per kChunk entries; at most n / kChunk
  // ids have more than one run
  const dim3 run_grid((unsigned)(V + n / kChunk + 1)), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(trkl_dw_runs_kernel<uint16_t>, run_grid, block, 0, s, list, base, rstart, pstart, run_id, V,
                       H, d, dW, part, accumulate ? 0 : 1);
  else
    hipLaunchKernelGGL(trkl_dw_runs_kernel<float>, run_grid, block, 0, s, list, base, rstart, pstart, run_id, V, H,
                       d, dW, part, accumulate ? 0 : 1);
  e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(trkl_dw_combine_kernel, dim3((unsigned)(n / kChunk + 1)), block, 0, s, rstart, pstart,
                       mstart, multi_id, V, d, part, dW, accumulate ? 0 : 1);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kdkl
