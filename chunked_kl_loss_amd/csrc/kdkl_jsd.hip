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
// sum_v q_v g_v; the projection epilogue forms it as a per-position dense
// coefficient times q_v minus a per-entry correction at the support, the
// same shape as the KL's softmax-minus-teacher.
//
// Three kernels, one wavefront per position:
//   gather_logits  s at each sorted teacher entry: a dot product of the
//                  entry's W row with the position's H row, over 1/T
//   jsd_merge      forward: lse from the split-vocabulary partials, then JSD
//   jsd_prep       backward: gbar from the saved lse, the dense coefficient,
//                  and the support corrections written over the entries'
//                  probabilities for the dZ epilogue
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
constexpr int kMaxPerLane = 1024 / 64;    // sorted entries per lane (K <= 1024)

__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float log_hw(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

__device__ __forceinline__ float wsum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Dot product of two 16-byte vectors of the storage type, fp32 accumulation.
template <typename TE>
struct Dot16;

template <>
struct Dot16<uint16_t> {  // eight bf16
  __device__ static float lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
  __device__ static float hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
  __device__ static float dot(uint4 a, uint4 b, float acc) {
    acc = fmaf(lo(a.x), lo(b.x), acc); acc = fmaf(hi(a.x), hi(b.x), acc);
    acc = fmaf(lo(a.y), lo(b.y), acc); acc = fmaf(hi(a.y), hi(b.y), acc);
    acc = fmaf(lo(a.z), lo(b.z), acc); acc = fmaf(hi(a.z), hi(b.z), acc);
    acc = fmaf(lo(a.w), lo(b.w), acc); acc = fmaf(hi(a.w), hi(b.w), acc);
    return acc;
  }
};

template <>
struct Dot16<float> {  // four fp32
  __device__ static float f(uint32_t u) { return __builtin_bit_cast(float, u); }
  __device__ static float dot(uint4 a, uint4 b, float acc) {
    acc = fmaf(f(a.x), f(b.x), acc); acc = fmaf(f(a.y), f(b.y), acc);
    acc = fmaf(f(a.z), f(b.z), acc); acc = fmaf(f(a.w), f(b.w), acc);
    return acc;
  }
};

// s at every sorted teacher entry of position `row` of the group (0 for an
// id outside [0, V) and for an ignored position). Repeated ids are adjacent
// after the sort; each distinct id is computed once.
template <typename TE>
__global__ __launch_bounds__(64 * kRowsPerBlock) void gather_logits_kernel(JsdArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  constexpr int EPC = 16 / (int)sizeof(TE);  // elements per 16-byte vector
  const int64_t nvec = a.d / EPC;            // d is a multiple of EPC
  const uint4* hrow = (const uint4*)((const TE*)a.H + (a.r0 + row) * a.d);
  const int2* ent = a.ent + (int64_t)row * a.K;
  float* sk = a.sk + (int64_t)row * a.K;
  const bool keep = a.keep[row] != 0.f;
  int prev = -1;
  float prev_s = 0.f;
  for (int h = 0; h < a.K; ++h) {
    const int id = ent[h].x;  // the same entry for every lane
    float s = 0.f;
    if (keep && id >= 0 && id < a.V) {
      if (id == prev) {
        s = prev_s;
      } else {
        const uint4* wrow = (const uint4*)((const TE*)a.W + (int64_t)id * a.d);
        float acc = 0.f;
        for (int64_t c = lane; c < nvec; c += 64) acc = Dot16<TE>::dot(hrow[c], wrow[c], acc);
        s = wsum(acc) * a.inv_T;
        prev = id;
        prev_s = s;
      }
    }
    if (lane == 0) sk[h] = s;
  }
}

struct Sums {
  float tp;  // beta sum_S P log(P / M)
  float tq;  // (1 - beta) sum_S q log(q / M)
  float qs;  // sum_S q
};

// The support terms of one position (each lane its share of the sorted
// entries; not yet summed over the wavefront). With `corr`, also each
// entry's correction of the dZ epilogue, -(1 - beta) q log((1 - beta) q / M)
// on the first entry of each distinct id (0 elsewhere).
__device__ __forceinline__ Sums support_terms(const JsdArgs& a, int row, float lse, float (&corr)[kMaxPerLane]) {
  const int lane = threadIdx.x & 63;
  const int2* ent = a.ent + (int64_t)row * a.K;
  const float* sk = a.sk + (int64_t)row * a.K;
  const float beta = a.beta, omb = 1.f - beta;
  Sums r{0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < kMaxPerLane; ++t) {
    corr[t] = 0.f;
    const int j = lane + 64 * t;
    if (j >= a.K) continue;
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
    corr[t] = -omb * q * (a.log_omb + lq - lm);
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
  const float lse = lse_of_partials(a.part + (int64_t)row * a.n_vt, a.n_vt);
  float corr[kMaxPerLane];
  Sums r = support_terms(a, row, lse, corr);
  r.tp = wsum(r.tp);
  r.tq = wsum(r.tq);
  r.qs = wsum(r.qs);
  if (lane == 0) {
    const float omb = 1.f - a.beta;
    // the off-support entries: (1 - beta) q log(1 / (1 - beta)) each
    const float jsd = r.tp + r.tq - omb * a.log_omb * (1.f - r.qs);
    a.row_lse[row] = lse;
    a.row_kl[row] = a.keep[row] != 0.f ? jsd : 0.f;
  }
}

__global__ __launch_bounds__(64 * kRowsPerBlock) void jsd_prep_kernel(JsdArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const bool keep = a.keep[row] != 0.f;
  const float lse = a.row_lse_in[row];
  float corr[kMaxPerLane];
  Sums r = support_terms(a, row, lse, corr);
  r.tq = wsum(r.tq);
  r.qs = wsum(r.qs);
  // every lane has read all the entries it needs: now overwrite the
  // probabilities with the corrections (0 for an ignored position)
  __builtin_amdgcn_wave_barrier();
  int2* ent = a.ent + (int64_t)row * a.K;
#pragma unroll
  for (int t = 0; t < kMaxPerLane; ++t) {
    const int j = lane + 64 * t;
    if (j < a.K) ent[j].y = __float_as_int(keep ? corr[t] : 0.f);
  }
  if (lane == 0) {
    const float omb = 1.f - a.beta;
    const float goff = -omb * a.log_omb;                   // g off the support
    const float gbar = r.tq + goff * (1.f - r.qs);         // sum_v q_v g_v
    a.rowcoef[row] = keep ? a.scale[0] * (goff - gbar) : 0.f;
  }
}

dim3 rows_grid(int rows) { return dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)); }

}  // namespace

hipError_t launch_gather_logits(int dtype, const JsdArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.K < 1 || a.K > 1024 || a.d % (dtype == 1 ? 8 : 4) != 0) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(gather_logits_kernel<uint16_t>, rows_grid(a.rows), dim3(64 * kRowsPerBlock), 0, s, a);
  else
    hipLaunchKernelGGL(gather_logits_kernel<float>, rows_grid(a.rows), dim3(64 * kRowsPerBlock), 0, s, a);
  return hipGetLastError();
}

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
