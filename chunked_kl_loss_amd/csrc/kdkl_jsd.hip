// Device kernels of the alternative loss: the generalised Jensen-Shannon
// divergence between the teacher's top-K distribution and the student's
// full-vocabulary distribution, on the fused chunked path's products.
//
// The pages report ablations on the choice of loss for the distilled
// student without naming the losses [P1 "Making knowledge distillation cheap
// enough to run at scale", section "The resulting student model"]; this is
// the reading taken. Per position, with P the teacher's top-K probabilities
// placed on the vocabulary (repeated ids add their mass, ids outside [0, V)
// have no entry), q = softmax(s), s = z / T, and M = beta P + (1 - beta) q:
//   JSD = beta KL(P || M) + (1 - beta) KL(q || M).
// Off the teacher's support M = (1 - beta) q, so those V - |S| entries add
// -(1 - beta) log(1 - beta) (1 - sum_S q) in closed form; only the support
// (at most K entries per position) needs the student's logits individually.
// The gradient is dZ_v = coef q_v (g_v - gbar) with g_v = (1 - beta)
// log(q_v / M_v) (= -(1 - beta) log(1 - beta) off the support) and gbar =
// sum_v q_v g_v. The projection epilogue forms it as a per-position
// coefficient of q_v, coef (g_off - gbar), minus at each support entry
// coef (1 - beta) q log(1 + beta P / ((1 - beta) q)), the same shape as the
// KL's softmax-minus-teacher; gbar comes from the forward (saved per
// position beside the logsumexp), so the backward needs no pass over the
// support before its projections.
//
// Two kernels, one wavefront per position:
//   jsd_merge  forward: lse from the split-vocabulary partials, then, from
//              s at each teacher entry (kept by the projection epilogue as it
//              meets the entry), JSD and gbar
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
  float tp;  // beta sum_S P log(P / M)
  float tq;  // (1 - beta) sum_S q log(q / M)
  float qs;  // sum_S q
};

// The support terms of one position (each lane its share of the sorted
// entries; not yet summed over the wavefront).
__device__ __forceinline__ Sums support_terms(const JsdArgs& a, int row, float lse) {
  const int lane = threadIdx.x & 63;
  const int2* ent = a.ent + (int64_t)row * a.K;
  const float* sk = a.sk + (int64_t)row * a.K;
  const float beta = a.beta, omb = 1.f - beta;
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
    // log M = log(beta P + (1 - beta) q), in the log domain
    const float u = a.log_beta + lp, w = a.log_omb + lq;
    const float hi = fmaxf(u, w), lo = fminf(u, w);
    const float lm = hi + log1pf(exp_hw(lo - hi));
    r.tp += beta * P * (lp - lm);
    r.tq += omb * q * (lq - lm);
    r.qs += q;
  }
  return r;
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
  r.tp = wsum(r.tp);
  r.tq = wsum(r.tq);
  r.qs = wsum(r.qs);
  if (lane == 0) {
    const float omb = 1.f - a.beta;
    // the off-support entries: (1 - beta) q log(1 / (1 - beta)) each
    const float off = -omb * a.log_omb * (1.f - r.qs);
    a.row_lse[row] = lse;
    a.row_kl[row] = keep ? r.tp + r.tq + off : 0.f;
    a.row_gbar[row] = keep ? r.tq + off : 0.f;  // sum_v q_v g_v
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
  if (lane == 0) {
    const float goff = -(1.f - a.beta) * a.log_omb;  // g off the support
    a.rowcoef[row] = keep ? a.scale[0] * (goff - a.row_gbar_in[row]) : 0.f;
  }
}

dim3 rows_grid(int rows) { return dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)); }

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

}  // namespace kdkl
