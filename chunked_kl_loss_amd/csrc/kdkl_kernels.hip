// Device kernels of the fused chunked KL loss for gfx950 (CDNA4).
//
// The loss follows the fused chunked KL of P1 "Making knowledge distillation
// cheap enough to run at scale" (section "Two system changes", fused chunked
// KL bullet): per slice of positions the hidden states are projected to
// logits, folded into the running loss and dropped; the backward pass
// recomputes each slice's projection. All projection work runs on one MFMA
// GEMM main loop (both operands contiguous along the contraction axis) with
// per-use epilogues:
//   EPI_FWD  Z^T tile = W_tile . H_tile^T; per token: max, sum exp, and the
//            teacher-weighted logit sum over the tile's vocabulary rows.
//   EPI_DZ   same product; dZ = coef * (softmax - teacher) written to the
//            token-major chunk buffer (and a vocab-major copy on the generic
//            path).
//   EPI_DH   dH partial = dZ . W over a split of the vocabulary (split-K).
//   EPI_DW   dW (+)= dZ^T . H over the chunk's tokens.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kdkl_internal.h"

namespace kdkl {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

static constexpr float kNegInf = -__builtin_huge_valf();
static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

// exp(x) and log(x) through the hardware base-2 instructions.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// ---------------------------------------------------------------------------
// Teacher preparation (one wavefront per position of the chunk):
//   p_k = softmax_k(l_k / T), e = sum_k p_k log p_k,
//   (id, p) pairs sorted by id, and for each vocabulary tile t the number of
//   sorted ids below t * vt (so a tile's teacher entries are the
//   contiguous range [tstart[t], tstart[t+1])).
// A workgroup takes kTeacherRows consecutive positions; their tile starts
// are staged in LDS and written as one 16-byte vector per tile (the table is
// position-minor, [n_vt + 1, Cp], for the projection epilogues' reads).
// ---------------------------------------------------------------------------
constexpr int kTeacherRows = 8;
constexpr int kTeacherTiles = 512;  // tile starts staged per pass
__global__ __launch_bounds__(64 * kTeacherRows) void teacher_prep_kernel(TeacherArgs a) {
  __shared__ __attribute__((aligned(16))) int32_t s_ids[kTeacherRows][1024];
  __shared__ int32_t s_sorted[kTeacherRows][1024];
  __shared__ __attribute__((aligned(16))) uint16_t s_ts[kTeacherTiles][kTeacherRows];
  const int w = threadIdx.x >> 6;
  const int row = blockIdx.x * kTeacherRows + w;
  const int lane = threadIdx.x & 63;
  const int K = a.K;
  const bool valid = row < a.rows;  // uniform per wavefront; every thread reaches each barrier
  const int64_t g = (a.r0 + (valid ? row : 0)) * (int64_t)K;
  const bool keep = valid && a.ids[g] != kIgnoreId;  // an ignored row's teacher is never used
  constexpr int MAXE = 1024 / 64;
  float av[MAXE];
  int32_t iv[MAXE];
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < MAXE; ++j) {
    const int k = lane + 64 * j;
    if (valid && k < K) {
      av[j] = a.logits[g + k] * a.inv_T;
      iv[j] = a.ids[g + k];
      s_ids[w][k] = iv[j];
      mx = fmaxf(mx, av[j]);
    } else {
      av[j] = kNegInf;
      iv[j] = 0;
    }
  }
  // pad the ids to a multiple of four with the largest int, which no rank
  // comparison below counts (ids are compared as (o < id) or (o == id and
  // o's position < id's position, which a pad's position never is)
  const int K4 = (K + 3) & ~3;
  if (valid && K + lane < K4) s_ids[w][K + lane] = INT32_MAX;
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < MAXE; ++j)
    if (lane + 64 * j < K) se += fast_exp(av[j] - mx);
  for (int o = 32; o > 0; o >>= 1) se += shfl_xor(se, o);
  const float lse = mx + fast_log(se);
  __syncthreads();
  if (valid) {
    float ent = 0.f;
#pragma unroll
    for (int j = 0; j < MAXE; ++j) {
      const int k = lane + 64 * j;
      if (k < K) {
        const float lp = av[j] - lse;
        const float p = keep ? fast_exp(lp) : 0.f;
        ent += p * lp;
        // rank of (id, k) in ascending id order, ties by position; the ids
        // are read four at a time
        int rank = 0;
        const int id = iv[j];
        for (int q = 0; q < K4; q += 4) {
          const int4 o = *(const int4*)&s_ids[w][q];
          rank += (o.x < id) | ((o.x == id) & (q < k));
          rank += (o.y < id) | ((o.y == id) & (q + 1 < k));
          rank += (o.z < id) | ((o.z == id) & (q + 2 < k));
          rank += (o.w < id) | ((o.w == id) & (q + 3 < k));
        }
        a.ent[(int64_t)row * K + rank] = make_int2(id, __float_as_int(p));
        s_sorted[w][rank] = id;
      }
    }
    for (int o = 32; o > 0; o >>= 1) ent += shfl_xor(ent, o);
    if (lane == 0) {
      a.erow[row] = keep ? ent : 0.f;
      a.keep[row] = keep ? 1.f : 0.f;
    }
  }
  // tile starts, kTeacherTiles at a time: each wavefront fills its column of
  // the staging table, then the workgroup writes one 16-byte row per tile
  // (positions past the chunk get 0; the epilogues never read them)
  for (int t0 = 0; t0 <= a.n_vt; t0 += kTeacherTiles) {
    __syncthreads();
    for (int tt = lane; tt < kTeacherTiles && t0 + tt <= a.n_vt; tt += 64) {
      int lo = 0;
      if (valid) {
        const int64_t bound = (int64_t)(t0 + tt) * a.vt;
        int hi = K;  // first index with sorted id >= bound
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((int64_t)s_sorted[w][mid] < bound) lo = mid + 1; else hi = mid;
        }
      }
      s_ts[tt][w] = (uint16_t)lo;
    }
    __syncthreads();
    for (int tt = threadIdx.x; tt < kTeacherTiles && t0 + tt <= a.n_vt; tt += 64 * kTeacherRows)
      *(uint4*)(a.tstart + (int64_t)(t0 + tt) * a.Cp + (int64_t)blockIdx.x * kTeacherRows) = *(const uint4*)s_ts[tt];
  }
}

hipError_t launch_teacher(const TeacherArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  // the 16-byte rows of the tile-start table need a position pitch that
  // covers whole workgroups of rows
  if (a.Cp % kTeacherRows != 0 || a.Cp < (int64_t)(a.rows + kTeacherRows - 1) / kTeacherRows * kTeacherRows)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(teacher_prep_kernel, dim3((a.rows + kTeacherRows - 1) / kTeacherRows),
                     dim3(64 * kTeacherRows), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-vocabulary merge (one wavefront per position): combine the per-tile
// (max, sum exp, gamma) partials into lse = M + log sum_t S_t e^{m_t - M} and
// KL = e - gamma + lse, in a fixed order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.rows) return;
  const float4* p = a.part + (int64_t)row * a.n_vt;
  float m = kNegInf, s = 0.f, gsum = 0.f;
  for (int t = lane; t < a.n_vt; t += 64) {
    const float4 v = p[t];
    gsum += v.z;
    if (v.x > kNegInf) {
      const float nm = fmaxf(m, v.x);
      s = s * fast_exp(m - nm) + v.y * fast_exp(v.x - nm);
      m = nm;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float om = shfl_xor(m, o);
    const float os = shfl_xor(s, o);
    gsum += shfl_xor(gsum, o);
    const float nm = fmaxf(m, om);
    if (nm > kNegInf) {
      s = (m > kNegInf ? s * fast_exp(m - nm) : 0.f) + (om > kNegInf ? os * fast_exp(om - nm) : 0.f);
      m = nm;
    }
  }
  if (lane == 0) {
    const float lse = m + fast_log(s);
    a.row_lse[row] = lse;
    a.row_kl[row] = a.keep[row] != 0.f ? a.erow[row] - gsum + lse : 0.f;
  }
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((a.rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Loss: sum_i KL_i / N_kept, fp64 accumulation in a fixed order (ignored
// positions have KL 0 and are not counted); and the backward's scale
// g / (N_kept T). One workgroup; the count reads each row's first id.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void block_sum2(double& a, long long& c) {
  __shared__ double ra[1024];
  __shared__ long long rc[1024];
  ra[threadIdx.x] = a;
  rc[threadIdx.x] = c;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      ra[threadIdx.x] += ra[threadIdx.x + w];
      rc[threadIdx.x] += rc[threadIdx.x + w];
    }
    __syncthreads();
  }
  a = ra[0];
  c = rc[0];
}

__global__ __launch_bounds__(1024) void loss_kernel(const float* row_kl, const int32_t* ids, int K, int64_t N,
                                                    float* loss) {
  double acc = 0.0;
  long long kept = 0;
  // independent strided reads: unrolled so that many are in flight at once
#pragma unroll 8
  for (int64_t i = threadIdx.x; i < N; i += 1024) {
    acc += (double)row_kl[i];
    kept += ids[i * K] != kIgnoreId;
  }
  block_sum2(acc, kept);
  if (threadIdx.x == 0) loss[0] = (float)(acc / (double)kept);  // NaN when nothing is kept
}

hipError_t launch_loss(const float* row_kl, const int32_t* ids, int K, int64_t N, float* loss,
                       hipStream_t s) {
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(1024), 0, s, row_kl, ids, K, N, loss);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void grad_scale_kernel(const int32_t* ids, int K, int64_t N, const float* grad,
                                                          float T, float* out) {
  double unused = 0.0;
  long long kept = 0;
#pragma unroll 8
  for (int64_t i = threadIdx.x; i < N; i += 1024) kept += ids[i * K] != kIgnoreId;
  block_sum2(unused, kept);
  if (threadIdx.x == 0) {
    const double g = grad ? (double)grad[0] : 1.0;
    out[0] = kept ? (float)(g / ((double)kept * (double)T)) : 0.f;
  }
}

hipError_t launch_grad_scale(const int32_t* ids, int K, int64_t N, const float* grad, float T, float* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(grad_scale_kernel, dim3(1), dim3(1024), 0, s, ids, K, N, grad, T, out);
  return hipGetLastError();
}

// The same two reductions in two stages for long inputs: up to
// kReduceBlocks workgroups each sum one contiguous range of rows (KL in fp64
// and the kept count) in a fixed order, then one workgroup sums their
// partials in block order. Deterministic; every row is read by many compute
// units at once instead of one.
template <int NT>
__device__ __forceinline__ void block_sum_pair(double& a, double& c, double* ra, double* rc) {
  ra[threadIdx.x] = a;
  rc[threadIdx.x] = c;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      ra[threadIdx.x] += ra[threadIdx.x + w];
      rc[threadIdx.x] += rc[threadIdx.x + w];
    }
    __syncthreads();
  }
  a = ra[0];
  c = rc[0];
}

__global__ __launch_bounds__(256) void rows_partial_kernel(const float* row_kl, const int32_t* ids, int K, int64_t N,
                                                          int64_t per, double2* part) {
  __shared__ double ra[256], rc[256];
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < N ? b0 + per : N;
  double acc = 0.0, kept = 0.0;
#pragma unroll 4
  for (int64_t i = b0 + threadIdx.x; i < b1; i += 256) {
    if (row_kl) acc += (double)row_kl[i];
    kept += ids[i * K] != kIgnoreId ? 1.0 : 0.0;
  }
  block_sum_pair<256>(acc, kept, ra, rc);
  if (threadIdx.x == 0) part[blockIdx.x] = make_double2(acc, kept);
}

// mode 0: loss = sum / kept (NaN when nothing is kept); mode 1: the
// backward's scale g / (kept T), 0 when nothing is kept.
__global__ __launch_bounds__(kReduceBlocks) void rows_finish_kernel(const double2* part, int nb, int mode,
                                                                   const float* grad, float T, float* out) {
  __shared__ double ra[kReduceBlocks], rc[kReduceBlocks];
  double acc = 0.0, kept = 0.0;
  if ((int)threadIdx.x < nb) {
    const double2 v = part[threadIdx.x];
    acc = v.x;
    kept = v.y;
  }
  block_sum_pair<kReduceBlocks>(acc, kept, ra, rc);
  if (threadIdx.x != 0) return;
  if (mode == 0) {
    out[0] = (float)(acc / kept);
  } else {
    const double g = grad ? (double)grad[0] : 1.0;
    out[0] = kept > 0.0 ? (float)(g / (kept * (double)T)) : 0.f;
  }
}

static hipError_t launch_rows_two_stage(const float* row_kl, const int32_t* ids, int K, int64_t N, void* part,
                                        int mode, const float* grad, float T, float* out, hipStream_t s) {
  const int64_t per = N > 0 ? (N + kReduceBlocks - 1) / kReduceBlocks : 1;
  const int nb = N > 0 ? (int)((N + per - 1) / per) : 0;
  if (nb > 0)
    hipLaunchKernelGGL(rows_partial_kernel, dim3(nb), dim3(256), 0, s, row_kl, ids, K, N, per, (double2*)part);
  hipLaunchKernelGGL(rows_finish_kernel, dim3(1), dim3(kReduceBlocks), 0, s, (const double2*)part, nb, mode, grad,
                     T, out);
  return hipGetLastError();
}

hipError_t launch_loss_ws(const float* row_kl, const int32_t* ids, int K, int64_t N, void* part, float* loss,
                          hipStream_t s) {
  return launch_rows_two_stage(row_kl, ids, K, N, part, 0, nullptr, 1.f, loss, s);
}

hipError_t launch_grad_scale_ws(const int32_t* ids, int K, int64_t N, const float* grad, float T, void* part,
                                float* out, hipStream_t s) {
  return launch_rows_two_stage(nullptr, ids, K, N, part, 1, grad, T, out, s);
}

// ---------------------------------------------------------------------------
// Transpose with zero padding: out[c, r] = in[r, c] (r < R), 0 (R <= r < Rp).
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E* __restrict__ in, int64_t R, int64_t C,
                                                        int64_t ldi, E* __restrict__ out, int64_t Rp,
                                                        int64_t ldo) {
  __shared__ E tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? in[r * ldi + c] : (E)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) out[c * ldo + r] = tile[tx][i];
  }
}

// 16-bit transpose with 16-byte accesses on both sides: a 64 x 64 tile is
// read as rows of 8-element vectors, and each output vector gathers 8 rows
// of one column from LDS. Needs C, ldi, ldo and Rp multiples of 8 and
// 16-byte aligned rows.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ in, int64_t R, int64_t C,
                                                          int64_t ldi, uint16_t* __restrict__ out, int64_t Rp,
                                                          int64_t ldo) {
  constexpr int P = 72;  // row pitch in elements (144 bytes: 16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * P];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = q * 256 + t, row = idx >> 3, ch = idx & 7;
    const int64_t r = r0 + row, c = c0 + ch * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < R && c < C) v = *(const uint4*)(in + r * ldi + c);
    *(uint4*)(tile + row * P + ch * 8) = v;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = q * 256 + t, oc = idx >> 3, orr = idx & 7;
    const int64_t c = c0 + oc, r = r0 + orr * 8;
    if (c >= C || r >= Rp) continue;
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = tile[(orr * 8 + j) * P + oc];
    uint4 o;
    o.x = e[0] | ((uint32_t)e[1] << 16);
    o.y = e[2] | ((uint32_t)e[3] << 16);
    o.z = e[4] | ((uint32_t)e[5] << 16);
    o.w = e[6] | ((uint32_t)e[7] << 16);
    *(uint4*)(out + c * ldo + r) = o;
  }
}

hipError_t launch_transpose(int elem_bytes, const void* in, int64_t R, int64_t C, int64_t ldi,
                            void* out, int64_t Rp, int64_t ldo, hipStream_t s) {
  if (Rp <= 0 || C <= 0) return hipSuccess;
  dim3 grid((unsigned)((Rp + 63) / 64), (unsigned)((C + 63) / 64));
  const bool vec = elem_bytes == 2 && C % 8 == 0 && ldi % 8 == 0 && ldo % 8 == 0 && Rp % 8 == 0 &&
                   ((uintptr_t)in & 15u) == 0 && ((uintptr_t)out & 15u) == 0;
  if (vec) {
    hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, s, (const uint16_t*)in, R, C, ldi,
                       (uint16_t*)out, Rp, ldo);
    return hipGetLastError();
  }
  if (elem_bytes == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)in, R, C,
                       ldi, (uint16_t*)out, Rp, ldo);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, (const float*)in, R, C, ldi,
                       (float*)out, Rp, ldo);
  return hipGetLastError();
}

// Fill n floats with zero (used instead of a memset so that captured graphs
// hold only kernel nodes).
__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dH = sum over splits of the fp32 partials, in split order, added to the
// sum of the earlier vocabulary slices when the backward runs in slices.
// ---------------------------------------------------------------------------
template <int BF16>
__global__ __launch_bounds__(256) void dh_reduce_kernel(const float* __restrict__ part, int splits,
                                                        int64_t n_elems, int64_t stride,
                                                        const float* acc_in, void* dH) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= n_elems) return;
  float4 acc = acc_in ? *(const float4*)(acc_in + i4) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < splits; ++s) {
    const float4 v = *(const float4*)(part + (int64_t)s * stride + i4);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (BF16) {
    ushort4 o;
    o.x = f32_to_bf16_bits(acc.x); o.y = f32_to_bf16_bits(acc.y);
    o.z = f32_to_bf16_bits(acc.z); o.w = f32_to_bf16_bits(acc.w);
    *(ushort4*)((uint16_t*)dH + i4) = o;
  } else {
    *(float4*)((float*)dH + i4) = acc;
  }
}

hipError_t launch_dh_reduce(int dtype, const float* part, int splits, int rows, int64_t d, int64_t Cp,
                            const float* acc_in, void* dH, hipStream_t s) {
  const int64_t n = (int64_t)rows * d;  // d is a multiple of 4
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n / 4 + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL(dh_reduce_kernel<1>, dim3(blocks), dim3(256), 0, s, part, splits, n, Cp * d, acc_in, dH);
  else
    hipLaunchKernelGGL(dh_reduce_kernel<0>, dim3(blocks), dim3(256), 0, s, part, splits, n, Cp * d, acc_in, dH);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Projection GEMMs.
//
// C[m, n] = sum_k A[m, k] B[n, k]; A and B row-major with k contiguous.
// Workgroup tile 256 x 256 split over a grid of wavefronts; each wavefront
// owns a sub-tile of 32 x 32 MFMA blocks. LDS rows hold 128 bytes of k
// (64 bf16 or 32 fp32) as eight 16-byte chunks stored at position
// chunk ^ ((row >> 1) & 7), or 64 bytes as four chunks at chunk ^ ((row >> 2)
// & 3). gfx950 serves a 128-bit LDS read 16 lanes (256 bytes, all 64 banks)
// at a time, and both layouts give the 16 rows read by one lane group 16
// distinct 16-byte bank slots.
//
// MFMA operand layout (32 x 32 output block): lane l feeds row (l & 31) of A
// and column (l & 31) of B with 8 consecutive k elements taken at offset
// 8 * (l >> 5) of the current 16-element k-group; accumulator register r of
// lane l holds output row 8 * (r >> 2) + 4 * (l >> 5) + (r & 3), column
// (l & 31).
// ---------------------------------------------------------------------------
constexpr int BM = 256, BN = 256;      // workgroup tile of the generic main loop
constexpr int kDwPitch = BN + 8;       // fp32 row pitch of the dW staging tile
constexpr int kEpiSmem = 128 * kDwPitch * 4;

// Wavefront grid of a TM x TN workgroup tile. TM x TN is 256 x 256 except
// for the products whose N axis is the hidden size, which may use 320-wide
// tiles (a hidden size of 2880 is 9 x 320 but 11.25 x 256), and the forward
// and dZ products on the bf16 main loop, which use 384 x 256.
template <int WAVES_M, int WAVES_N, int TN = 256, int TM = 256>
struct Grid {
  static constexpr int kWavesM = WAVES_M, kWavesN = WAVES_N;
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = TM, BN = TN;
  static constexpr int WM = TM / WAVES_M, WN = TN / WAVES_N;
  static constexpr int MB = WM / 32, NB = WN / 32;
  // Above 160 accumulator registers per lane (two wavefronts per SIMD share
  // 512), the B fragments of the next k-group are read into the registers
  // of the current one as each is consumed instead of a second buffer.
  static constexpr bool kSingleB = MB * NB * 16 > 160;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wavefront tiles are whole 32 x 32 blocks");
  static __device__ __forceinline__ int wm() { return (int)(threadIdx.x >> 6) / WAVES_N; }
  static __device__ __forceinline__ int wn() { return (int)(threadIdx.x >> 6) % WAVES_N; }
};
using Grid4 = Grid<2, 2>;   // 4 wavefronts of 128 x 128
using Grid8 = Grid<2, 4>;   // 8 wavefronts of 128 x 64 (two per SIMD)
using Grid16 = Grid<4, 4>;  // 16 wavefronts of 64 x 64 (four per SIMD)

__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

// Output row of accumulator register r of block mb in this lane, tile-relative.
template <class G>
__device__ __forceinline__ int acc_row(int wm, int mb, int r, int lane) {
  return wm * G::WM + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

struct Tile {
  int tm, tn, ks;
};

// XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
// each XCD gets a contiguous run of tiles (neighbours share an A tile and
// stay in that XCD's L2). An N axis of 16 tiles or more is taken in bands of
// kNBand tiles: an XCD's 32 concurrent workgroups then cover a few A tiles
// by one band of B tiles, instead of one A tile by all the B tiles, whose
// bytes would be fetched again in every round. Returns false for the
// padding workgroups.
constexpr int kNBand = 8;
__device__ __forceinline__ bool tile_of(const GemmArgs& p, Tile& t) {
  const int total = p.tiles_m * p.tiles_n * p.splits;
  const int per = (total + 7) >> 3;
  const int L = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (L >= total) return false;
  const int mn = p.tiles_m * p.tiles_n;
  t.ks = L / mn;
  const int l = L - t.ks * mn;
  const int nb = p.tiles_n >= 2 * kNBand ? kNBand : p.tiles_n;  // band width
  const int band = l / (nb * p.tiles_m);  // every band before the last is full
  const int w = min(nb, p.tiles_n - band * nb);
  const int r = l - band * nb * p.tiles_m;
  t.tm = r / w;
  t.tn = band * nb + r % w;
  return true;
}

// Accumulator slot (mb * 16 + r) of launch-relative vocabulary row `id` in
// this lane, or -1.
template <class G>
__device__ __forceinline__ int hit_slot(int id, int V, int m0, int wm, int lane) {
  const int r = id - m0 - wm * G::WM;
  if (id >= V || r < 0 || r >= G::WM) return -1;
  const int rin = r & 31;
  if (((rin >> 2) & 1) != (lane >> 5)) return -1;
  return (r >> 5) * 16 + ((rin >> 3) << 2) + (rin & 3);
}

#ifndef KDKL_EPI_NT
#define KDKL_EPI_NT 1
#endif
// Epilogue streams written (dZ chunk, dW) or read once per launch (old dW):
// far larger than the caches, so they go out with the nontemporal hint.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_nt_t;
__device__ __forceinline__ void store16_stream(void* p, uint4 v) {
  if (KDKL_EPI_NT)
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, (u32x4_t*)p);
  else
    *(uint4*)p = v;
}
__device__ __forceinline__ void store16_stream(float* p, float4 v) {
  if (KDKL_EPI_NT)
    __builtin_nontemporal_store(f32x4_nt_t{v.x, v.y, v.z, v.w}, (f32x4_nt_t*)p);
  else
    *(float4*)p = v;
}
__device__ __forceinline__ float4 load16_stream(const float* p) {
  if (KDKL_EPI_NT) {
    const f32x4_nt_t v = __builtin_nontemporal_load((const f32x4_nt_t*)p);
    return make_float4(v.x, v.y, v.z, v.w);
  }
  return *(const float4*)p;
}

template <class G, int ES, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& p, f32x16_t (&acc)[G::MB][G::NB], const Tile& t,
                                              char* smem) {
  constexpr int MB = G::MB, NB = G::NB, NT = G::kThreads;
  constexpr int BM = G::BM, BN = G::BN;
  constexpr int kDzPitch = BM + 8;  // bf16 row pitch of the dZ staging tile
  constexpr bool DZ = EPI == EPI_DZ || EPI == EPI_DZJ;  // the two dZ epilogues
  static_assert(BM == 256 || EPI == EPI_FWD || DZ, "vocabulary-row tiles of dH / dW are 256 high");
  static_assert(BN == 256 || EPI == EPI_DH || EPI == EPI_DW, "token-axis tiles are 256 wide");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wm = G::wm(), wn = G::wn();
  const int m0 = t.tm * BM, n0 = t.tn * BN;
  // Rows past V exist only in the last vocabulary tile; the others skip the mask.
  const bool full_rows = m0 + BM <= p.V;
  auto row_ok = [&](int mb, int r) { return m0 + acc_row<G>(wm, mb, r, lane) < p.V; };
  // exp(s - m) with s = z / T as exp2(z * c2 - m2): one fused multiply-add per element
  const float c2 = p.inv_T * kLog2e;
  // Per-column inputs of the forward and dZ epilogues: the column's teacher
  // entries in this tile ([lo, hi) into its sorted list) and, for dZ, the
  // scale qs and base-2 lse of its softmax (qs = 0 and lse2 = +inf for a
  // column past the chunk or of an ignored position, so q = 0). One thread
  // per column loads them into an LDS table past the epilogue's other LDS
  // use: all columns' loads are in flight together, and the column blocks
  // below keep no per-column registers (which would spill next to the
  // accumulators).
  constexpr int kRedBytes = G::kWavesM * BN * 3 * 4;
  constexpr int kStageBytes = (DZ && ES == 2) ? 128 * kDzPitch * 2 : 0;
  constexpr int kInfoOff = ((kRedBytes > kStageBytes ? kRedBytes : kStageBytes) + 255) / 256 * 256;
  static_assert(kInfoOff + BN * 16 <= 128 * 1024, "the column table fits every projection kernel's LDS");
  const int4* info = (const int4*)(smem + kInfoOff);
  if constexpr (EPI == EPI_FWD || DZ) {
    if (!p.raw) {
      for (int c = tid; c < BN; c += NT) {
        const int col = n0 + c;
        int4 v = make_int4(0, 0, 0, __float_as_int(__builtin_huge_valf()));
        if (col < p.N) {
          v.x = p.tstart[(int64_t)(p.tm0 + t.tm) * p.Cp + col];
          v.y = p.tstart[(int64_t)(p.tm0 + t.tm + 1) * p.Cp + col];
          if constexpr (DZ) {
            if (p.keep[col] != 0.f) {
              v.z = __float_as_int(p.rowcoef ? p.rowcoef[col] : p.scale[0]);
              v.w = __float_as_int(p.row_lse[col] * kLog2e);
            }
          }
        }
        ((int4*)(smem + kInfoOff))[c] = v;
      }
      __syncthreads();
    }
  }
  if constexpr (EPI == EPI_FWD) {
    // s = z / T over the tile's vocabulary rows (A rows), per token column:
    // max, sum of exp(s - max), and sum of p * s over the teacher ids here.
    // The max is taken over z (T > 0 preserves order) and scaled once.
    float* red = (float*)smem;  // [WAVES_M][BN][3]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int ct = wn * G::WN + nb * 32 + (lane & 31);
      const int col = n0 + ct;
      float zmax = kNegInf;
      if (full_rows) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) zmax = fmaxf(zmax, acc[mb][nb][r]);
      } else {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) zmax = fmaxf(zmax, row_ok(mb, r) ? acc[mb][nb][r] : kNegInf);
      }
      zmax = fmaxf(zmax, shfl_xor(zmax, 32));
      float se = 0.f;
      if (zmax > kNegInf) {
        const float off = zmax * c2;
        if (full_rows) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) se += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mb][nb][r], c2, -off));
        } else {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mb][nb][r], c2, -off));
              se += row_ok(mb, r) ? e : 0.f;
            }
        }
      }
      se += shfl_xor(se, 32);
      const float mx = zmax * p.inv_T;
      float gz = 0.f;  // sum of p * z; times 1/T below
      const int4 ci = p.raw ? make_int4(0, 0, 0, 0) : info[ct];
      for (int h = ci.x; h < ci.y; ++h) {
        const int2 e = p.ent[(int64_t)col * p.K + h];
        const int slot = hit_slot<G>(e.x - p.v0, p.V, m0, wm, lane);
        if (slot < 0) continue;
        float v = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) v = (mb * 16 + rr == slot) ? acc[mb][nb][rr] : v;
        gz += __int_as_float(e.y) * v;
        // the JSD keeps s at each teacher entry (met by exactly this lane of
        // this tile)
        if (p.sk) p.sk[(int64_t)col * p.K + h] = v * p.inv_T;
      }
      gz += shfl_xor(gz, 32);
      const float gam = gz * p.inv_T;
      if (lane < 32) {
        float* e = red + (wm * BN + ct) * 3;
        e[0] = mx;
        e[1] = se;
        e[2] = gam;
      }
    }
    __syncthreads();
    for (int c = tid; c < BN; c += NT) {
      const int col = n0 + c;
      if (col >= p.N) continue;
      float m = kNegInf, g = 0.f;
#pragma unroll
      for (int w = 0; w < G::kWavesM; ++w) {
        m = fmaxf(m, red[(w * BN + c) * 3]);
        g += red[(w * BN + c) * 3 + 2];
      }
      float s = 0.f;
      if (m > kNegInf) {
#pragma unroll
        for (int w = 0; w < G::kWavesM; ++w) {
          const float* e = red + (w * BN + c) * 3;
          if (e[0] > kNegInf) s += e[1] * fast_exp(e[0] - m);
        }
      }
      p.part[(int64_t)col * p.n_vt + t.tm] = make_float4(m, s, g, 0.f);
    }
  } else if constexpr (DZ) {
    // dZ = coef * (softmax(s) - teacher) for the tile (for the JSD, the
    // column's own coefficient times softmax(s) minus the support
    // corrections held where the KL holds the teacher probabilities), written to the chunk
    // buffers token-major (dz_cv [Cp, Vp]) and vocabulary-major (dz_vc [Vp, Cp]).
    // coef = g / (N_kept T); an ignored position's column is zero (its
    // teacher mass is zero as well). In raw mode (the dense path) the tile of
    // logits z itself is stored (coef 1, zero outside the valid rows).
    const float coef = p.raw ? 1.f : p.scale[0];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = n0 + wn * G::WN + nb * 32 + (lane & 31);
      const bool cval = col < p.N;
      if (p.raw) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + acc_row<G>(wm, mb, r, lane);
            acc[mb][nb][r] = (row < p.V && cval) ? acc[mb][nb][r] : 0.f;
          }
        continue;
      }
      // coef * q = qs * exp2(z * c2 - lse2)
      const int4 ci = info[wn * G::WN + nb * 32 + (lane & 31)];
      const float qs = __int_as_float(ci.z), lse2 = __int_as_float(ci.w);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[mb][nb][r] = qs * __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mb][nb][r], c2, -lse2));
      if (!full_rows) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][nb][r] = row_ok(mb, r) ? acc[mb][nb][r] : 0.f;
      }
      for (int h = ci.x; h < ci.y; ++h) {
        const int2 e = p.ent[(int64_t)col * p.K + h];
        const int slot = hit_slot<G>(e.x - p.v0, p.V, m0, wm, lane);
        if (slot < 0) continue;
        float pk = coef * __int_as_float(e.y);
        if constexpr (EPI == EPI_DZJ) {
          // The entry holds the teacher mass P of its id (0 on a repeat);
          // with q = acc / qs here (acc = qs q, qs >= 0), the correction is
          // coef q (g_off - g) at the entry, a = the loss's parameter:
          //   JSD   coef (1 - a) q log(1 + a P / ((1 - a) q))
          //   SKL   coef (1 - a) P q / M,  M = a P + (1 - a) q   (coef P at a = 0)
          //   SRKL  coef q (-log(1 - u) - u),  u = (1 - a) P / M,  M = a q + (1 - a) P
          //         (as coef q (y - 1 - log y), y = 1 - u = a q / M, where u
          //         is not small; 0 once a q underflows, where q is)
          float v = 0.f;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) v = (mb * 16 + rr == slot) ? acc[mb][nb][rr] : v;
          const float P = __int_as_float(e.y), a = p.beta, oma = 1.f - a;
          const float q = qs > 0.f ? v / qs : 0.f;
          if (!(P > 0.f)) {
            pk = 0.f;
          } else if (p.alt == ALT_SKL) {
            // at a = 0 the KL's teacher term, whatever q (which may underflow)
            pk = a == 0.f ? coef * P : coef * oma * P * (q / (a * P + oma * q));
          } else if (!(q > 0.f)) {
            pk = 0.f;
          } else if (p.alt == ALT_SRKL) {
            const float M = a * q + oma * P;
            const float u = oma * P / M, y = a * q / M;
            const float t = u < 0.5f ? -log1pf(-u) - u : (y > 0.f ? y - 1.f - logf(y) : 0.f);
            pk = coef * q * t;
          } else {
            pk = coef * oma * q * log1pf(a * P / (oma * q));
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            acc[mb][nb][rr] = (mb * 16 + rr == slot) ? acc[mb][nb][rr] - pk : acc[mb][nb][rr];
      }
    }
    if constexpr (ES == 2) {
      // Stage 128 token columns at a time as bf16 [128 n][BM v] in LDS, then
      // write both layouts with 16-byte stores.
      uint16_t* T = (uint16_t*)smem;
      uint16_t* cv = (uint16_t*)p.dz_cv;
      uint16_t* vc = (uint16_t*)p.dz_vc;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        __syncthreads();
        if ((wn * G::WN) / 128 == half) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4) {
                const int nl = wn * G::WN + nb * 32 + (lane & 31) - half * 128;
                const int vl = acc_row<G>(wm, mb, r4 * 4, lane);
                ushort4 o;
                o.x = f32_to_bf16_bits(acc[mb][nb][r4 * 4 + 0]);
                o.y = f32_to_bf16_bits(acc[mb][nb][r4 * 4 + 1]);
                o.z = f32_to_bf16_bits(acc[mb][nb][r4 * 4 + 2]);
                o.w = f32_to_bf16_bits(acc[mb][nb][r4 * 4 + 3]);
                *(ushort4*)(T + nl * kDzPitch + vl) = o;
              }
        }
        __syncthreads();
        const int nb0 = n0 + half * 128;
        // token-major rows: BM * 2 bytes of vocabulary each
        constexpr int CV = BM / 8;  // 16-byte chunks per row
#pragma unroll 4
        for (int j = tid; j < 128 * CV; j += NT) {
          const int i = j / CV, c = j % CV;
          store16_stream(cv + (int64_t)(nb0 + i) * p.Vp + m0 + c * 8, *(const uint4*)(T + i * kDzPitch + c * 8));
        }
        // vocabulary-major rows: 256 bytes of tokens each (only for the
        // generic path, whose dW product needs K-contiguous operands)
        if (vc == nullptr) continue;
#pragma unroll 4
        for (int j = tid; j < BM * 16; j += NT) {
          const int v = j % BM, c = j / BM;
          uint16_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) e[q] = T[(c * 8 + q) * kDzPitch + v];
          uint4 o;
          o.x = e[0] | ((uint32_t)e[1] << 16);
          o.y = e[2] | ((uint32_t)e[3] << 16);
          o.z = e[4] | ((uint32_t)e[5] << 16);
          o.w = e[6] | ((uint32_t)e[7] << 16);
          *(uint4*)(vc + (int64_t)(m0 + v) * p.Cp + nb0 + c * 8) = o;
        }
      }
    } else {
      float* cv = (float*)p.dz_cv;
      float* vc = (float*)p.dz_vc;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = n0 + wn * G::WN + nb * 32 + (lane & 31);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int row = m0 + acc_row<G>(wm, mb, r4 * 4, lane);
            const float v0 = acc[mb][nb][r4 * 4 + 0], v1 = acc[mb][nb][r4 * 4 + 1];
            const float v2 = acc[mb][nb][r4 * 4 + 2], v3 = acc[mb][nb][r4 * 4 + 3];
            *(float4*)(cv + (int64_t)col * p.Vp + row) = make_float4(v0, v1, v2, v3);
            if (vc == nullptr) continue;
            vc[(int64_t)(row + 0) * p.Cp + col] = v0;
            vc[(int64_t)(row + 1) * p.Cp + col] = v1;
            vc[(int64_t)(row + 2) * p.Cp + col] = v2;
            vc[(int64_t)(row + 3) * p.Cp + col] = v3;
          }
      }
    }
  } else if constexpr (EPI == EPI_DH) {
    // fp32 partial of split ks: out[ks, row, col]
    float* out = p.out + (int64_t)t.ks * p.Cp * p.ldo;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = n0 + wn * G::WN + nb * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + acc_row<G>(wm, mb, r, lane);
          if (row < p.M) out[(int64_t)row * p.ldo + col] = acc[mb][nb][r];
        }
    }
  } else {
    // EPI_DW: dW[row, col] (+)= tile, staged through LDS PR rows at a time
    // so the read-modify-write of dW uses 16-byte accesses on whole rows.
    // The old values of each part are loaded into registers before that
    // part's accumulators go through LDS, so the load latency overlaps the
    // staging (and, after the first part, the previous part's stores).
    constexpr int PR = BN == 256 ? 128 : 64;  // rows per staged part (fits the LDS)
    constexpr int PITCH = BN + 8;
    constexpr int C4 = BN / 4;                // float4 per row
    constexpr int ITER = PR * C4 / NT;
    static_assert(PR % G::WM == 0 && (PR * C4) % NT == 0, "dW staging takes whole wavefront tiles");
    static_assert(PR * PITCH * 4 <= kEpiSmem, "dW staging fits the shared buffer");
    float* F = (float*)smem;
    float4 o[ITER];
    // Rows and columns past the edge read a clamped (valid) address; their
    // sums are never stored.
    auto load_old = [&](int part) {
#pragma unroll
      for (int u = 0; u < ITER; ++u) o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p.accumulate) {
#pragma unroll
        for (int u = 0; u < ITER; ++u) {
          const int j = u * NT + tid;
          const int row = min(m0 + part * PR + j / C4, p.M - 1), col = min(n0 + (j % C4) * 4, p.N - 4);
          o[u] = load16_stream(p.out + (int64_t)row * p.ldo + col);
        }
      }
    };
    load_old(0);
#pragma unroll
    for (int part = 0; part < BM / PR; ++part) {
      __syncthreads();
      if ((wm * G::WM) / PR == part) {
        const int rb = wm * G::WM - part * PR;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              F[(rb + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * PITCH + wn * G::WN + nb * 32 +
                (lane & 31)] = acc[mb][nb][r];
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < ITER; ++u) {
        const int j = u * NT + tid;
        const int r = j / C4, c4 = j % C4;
        const int row = m0 + part * PR + r, col = n0 + c4 * 4;
        if (row < p.M && col < p.N) {
          const float4 v = *(const float4*)(F + r * PITCH + c4 * 4);
          store16_stream(p.out + (int64_t)row * p.ldo + col,
                         make_float4(o[u].x + v.x, o[u].y + v.y, o[u].z + v.z, o[u].w + v.w));
        }
      }
      if (part + 1 < BM / PR) load_old(part + 1);
    }
  }
}

template <class G>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[G::MB][G::NB]) {
#pragma unroll
  for (int i = 0; i < G::MB; ++i)
#pragma unroll
    for (int j = 0; j < G::NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// ------------------------- generic main loop --------------------------------
// Register-staged loads with zero fill past M / N rows and past the K extent.
// Serves fp32 and any K that is not a multiple of the 64-element k-step.
template <typename TE>
struct Mfma;

template <>
struct Mfma<uint16_t> {  // bf16 storage
  struct Frag {
    bf16x8_t v;
  };
  static __device__ __forceinline__ Frag load(const char* s, int row, int kk, int lane) {
    const int c = kk * 2 + (lane >> 5);
    Frag f;
    f.v = *(const bf16x8_t*)(s + row * 128 + ((c ^ swz8(row)) << 4));
    return f;
  }
  static __device__ __forceinline__ void mma(const Frag& a, const Frag& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  struct Frag {
    f32x4_t lo, hi;
  };
  static __device__ __forceinline__ Frag load(const char* s, int row, int kk, int lane) {
    const int c = kk * 4 + (lane >> 5) * 2;
    Frag f;
    f.lo = *(const f32x4_t*)(s + row * 128 + ((c ^ swz8(row)) << 4));
    f.hi = *(const f32x4_t*)(s + row * 128 + (((c + 1) ^ swz8(row)) << 4));
    return f;
  }
  static __device__ __forceinline__ void mma(const Frag& a, const Frag& b, f32x16_t& c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[e], b.hi[e], c, 0, 0, 0);
  }
};

template <int ROWS>
__device__ __forceinline__ void g2r(uint4 (&r)[ROWS * 8 / 256], const char* __restrict__ base, int64_t ld_bytes,
                                    int row0, int nrows, int64_t k0_bytes, int64_t kend_bytes, int tid) {
#pragma unroll
  for (int i = 0; i < ROWS * 8 / 256; ++i) {
    const int idx = i * 256 + tid;
    const int row = idx >> 3, c = idx & 7;
    const int gr = row0 + row;
    const int64_t kb = k0_bytes + c * 16;
    if (gr < nrows && kb < kend_bytes)
      r[i] = *(const uint4*)(base + (int64_t)gr * ld_bytes + kb);
    else
      r[i] = make_uint4(0, 0, 0, 0);
  }
}

template <int ROWS>
__device__ __forceinline__ void r2s(const uint4 (&r)[ROWS * 8 / 256], char* s, int tid) {
#pragma unroll
  for (int i = 0; i < ROWS * 8 / 256; ++i) {
    const int idx = i * 256 + tid;
    const int row = idx >> 3, c = idx & 7;
    *(uint4*)(s + row * 128 + ((c ^ swz8(row)) << 4)) = r[i];
  }
}

template <typename TE, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_generic_kernel(const GemmArgs p) {
  using G = Grid4;
  using M_ = Mfma<TE>;
  constexpr int ES = sizeof(TE);
  constexpr int BK = 128 / ES;
  constexpr int kStage = (BM + BN) * 128;
  constexpr int SMEM = 2 * kStage > kEpiSmem ? 2 * kStage : kEpiSmem;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  Tile t;
  if (!tile_of(p, t)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wm = G::wm(), wn = G::wn();
  const int m0 = t.tm * BM, n0 = t.tn * BN;
  const int64_t kb = (int64_t)t.ks * p.k_split;
  const int64_t ke = kb + p.k_split < p.k_end ? kb + p.k_split : p.k_end;
  const int nk = ke > kb ? (int)((ke - kb + BK - 1) / BK) : 0;

  f32x16_t acc[G::MB][G::NB];
  zero_acc<G>(acc);

  const char* Ab = (const char*)p.A;
  const char* Bb = (const char*)p.B;
  const int64_t lda_b = p.lda * ES, ldb_b = p.ldb * ES;
  const int64_t kend_b = ke * ES;
  uint4 ra[BM * 8 / 256], rb[BN * 8 / 256];

  if (nk > 0) {
    g2r<BM>(ra, Ab, lda_b, m0, p.M, kb * ES, kend_b, tid);
    g2r<BN>(rb, Bb, ldb_b, n0, p.N, kb * ES, kend_b, tid);
    r2s<BM>(ra, smem, tid);
    r2s<BN>(rb, smem + BM * 128, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) {
        const int64_t k0b = (kb + (int64_t)(kt + 1) * BK) * ES;
        g2r<BM>(ra, Ab, lda_b, m0, p.M, k0b, kend_b, tid);
        g2r<BN>(rb, Bb, ldb_b, n0, p.N, k0b, kend_b, tid);
      }
      const char* sA = smem + (kt & 1) * kStage;
      const char* sB = sA + BM * 128;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        typename M_::Frag fa[G::MB], fb[G::NB];
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb) fa[mb] = M_::load(sA, wm * G::WM + mb * 32 + (lane & 31), kk, lane);
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) fb[nb] = M_::load(sB, wn * G::WN + nb * 32 + (lane & 31), kk, lane);
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < G::NB; ++nb) M_::mma(fa[mb], fb[nb], acc[mb][nb]);
      }
      if (more) {
        char* s = smem + ((kt + 1) & 1) * kStage;
        r2s<BM>(ra, s, tid);
        r2s<BN>(rb, s + BM * 128, tid);
      }
      __syncthreads();
    }
  }
  gemm_epilogue<G, ES, EPI>(p, acc, t, smem);
}

// ----------------------------- bf16 main loop -------------------------------
// For K extents that are whole 64-element steps. Global->LDS loads go
// straight into LDS (global_load_lds_dwordx4: each lane's 16 bytes land at
// lane * 16 of the wave's 1 KiB destination), so the bank-spreading layout
// is produced by choosing which global chunk each lane fetches. Rows past
// M / N are clamped to the last valid row (their outputs are masked in the
// epilogue). BK-element k-steps, NSTAGE stages in flight: the loads for
// k-step kt + NSTAGE - 1 are issued while k-step kt is multiplied and only
// the oldest stage is waited for; the LDS fragments of the next 16-element
// k-group are read while the MFMAs of the current one run.
typedef __attribute__((address_space(3))) void lds_void;

// Word 3 of a raw buffer resource on CDNA (32-bit data format, no swizzle).
constexpr int kBufferRsrcWord3 = 0x00020000;

// 16 bytes per lane from base + off (off < 2^31) straight into LDS at the
// wavefront's 1 KiB destination `lds` (lane i lands at lds + 16 i).
__device__ __forceinline__ void load16_lds(const void* base, uint32_t off, void* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufferRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}

// Workgroup barrier for the main loops, which wait for their own loads with
// explicit vmcnt counts: a bare s_barrier (no implicit wait for every
// outstanding load, unlike __syncthreads, which would drain the prefetched
// stages), fenced so that neither the compiler's IR passes (memory clobber)
// nor its scheduler (MFMAs included, which touch only registers) move
// anything across it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// ds_read_b64_tr_b16 as assembly. For the builtin form the compiler's
// wait-count pass knows no address, so it waits for every outstanding
// direct-to-LDS stage load (vmcnt(0)) before each such read, twice per
// k-step, although a stage being read is never the one in flight. Issued
// here as plain assembly, the reads' results are waited for explicitly by
// lds_ready before the MFMAs that use them.
__device__ __forceinline__ s16x4_t ds_read_tr16(const char* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  s16x4_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a) : "memory");
  return v;
}

// Waits for every outstanding LDS access, then ties the fragments to the
// wait so that their uses stay after it.
template <int N>
__device__ __forceinline__ void lds_ready(bf16x8_t (&f)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(f[i]));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Main-loop configuration of the bf16 path (wave grid, k-step, stages).
#ifndef KDKL_GEMM_WAVES
#define KDKL_GEMM_WAVES 8
#endif
#ifndef KDKL_GEMM_BK
#define KDKL_GEMM_BK 64
#endif
#ifndef KDKL_GEMM_STAGES
#define KDKL_GEMM_STAGES 2
#endif
#ifndef KDKL_DMA_SPREAD
#define KDKL_DMA_SPREAD 3
#endif
#ifndef KDKL_DMA_SPREAD_EB
#define KDKL_DMA_SPREAD_EB 2
#endif
#ifndef KDKL_DW_GRID42
#define KDKL_DW_GRID42 1
#endif
#ifndef KDKL_EARLY_BARRIER
#define KDKL_EARLY_BARRIER 1
#endif
#ifndef KDKL_FRAG_FENCE
#define KDKL_FRAG_FENCE 1
#endif
// Keeps the fragment reads of the next k-group where the source puts them,
// ahead of the MFMAs of the current one: left to itself the scheduler sinks
// them below most of those MFMAs (giving both fragment buffers the same
// registers), and the next k-group then waits for reads issued one to three
// MFMAs earlier. Applied where the fragments are double-buffered (dH, dW);
// the forward and dZ tiles, whose B fragments are single-buffered, spill
// under it.
template <bool ON>
__device__ __forceinline__ void frag_fence() {
  if constexpr (ON && KDKL_FRAG_FENCE) __builtin_amdgcn_sched_barrier(0);
}

template <class G, int EPI, int BK, int NSTAGE, int LA, int LB>
__global__ __launch_bounds__(G::kThreads, 1) void gemm_bf16_kernel(const GemmArgs p) {
  constexpr int MB = G::MB, NB = G::NB;
  constexpr int RB = BK * 2;                 // bytes of one k-contiguous LDS row
  constexpr int CPR = RB / 16;               // 16-byte chunks per such row
  constexpr int TILE = G::BM * RB;           // bytes of the A tile per stage
  constexpr int TILE_B = G::BN * RB;         // bytes of the B tile per stage
  constexpr int STG = TILE + TILE_B;
  constexpr int SMEM = NSTAGE * STG > kEpiSmem ? NSTAGE * STG : kEpiSmem;
  constexpr int LPO = TILE / (1024 * G::kWaves);     // direct loads per wave for A per stage
  constexpr int LPO_B = TILE_B / (1024 * G::kWaves);  // and for B
  constexpr int LPS = LPO + LPO_B;
  constexpr int KG = BK / 16;                // 16-element k-groups per step
  static_assert(LPO * 1024 * G::kWaves == TILE && LPO_B * 1024 * G::kWaves == TILE_B, "whole loads per wave");
  static_assert((LA == LAYOUT_KC || G::BM == 256 || G::BM == 320) &&
                    (LB == LAYOUT_KC || G::BN == 256 || G::BN == 320),
                "k-major LDS rows hold 256 or 320 elements");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  Tile t;
  if (!tile_of(p, t)) return;
  // The wavefront index is uniform across a wavefront; reading it through
  // readfirstlane lets every LDS destination (M0) be computed in scalar
  // registers instead of a vector-to-scalar move per load.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / G::kWavesN, wn = wid % G::kWavesN;
  const int m0 = t.tm * G::BM, n0 = t.tn * G::BN;
  const int64_t kb = (int64_t)t.ks * p.k_split;
  const int64_t ke = kb + p.k_split < p.k_end ? kb + p.k_split : p.k_end;
  const int nk = ke > kb ? (int)((ke - kb) / BK) : 0;

  auto swz = [](int row) { return CPR == 8 ? swz8(row) : swz4(row); };

  // Direct loads go through buffer instructions (buffer_load ... lds): the
  // compiler's wait-count pass treats the global_load form as a FLAT access
  // to both memory and LDS and then waits for every outstanding LDS read
  // (lgkmcnt(0)) at each use, which serializes fragment reads with MFMAs.
  // The buffer resource holds a wavefront-uniform base per k-step; each lane
  // adds a 32-bit byte offset (the host keeps a tile's span below 2 GiB).
  // KC: lane offset = 16-byte chunk of an output-axis row, fixed over the
  // k-steps (the base advances RB bytes per step). MC: 16-byte unit of a k
  // row; the k row is clamped to the last one per step. An MC stage holds
  // BK rows of W_ (256 or 320) elements; global unit u of row k sits at LDS
  // unit mc_unit(k, u) of that row: rows of 512 bytes are XORed by 4 units
  // per k mod 4, rows of 640 bytes (128 bytes mod the 256-byte bank span)
  // rotated by 4 units when bit 1 of k is set, so that the four rows a
  // transposed read touches fall in four distinct 64-byte bank quarters.
  struct Src {
    uint32_t off;  // KC: byte offset from the tile base; MC: column byte offset
    int krow;      // MC: k row within the stage
  };
  auto make_src = [&](int layout, int64_t ld, int rows, int row0, int64_t mcols, int i, int W_) {
    Src s;
    const int slot = (i * G::kWaves + wid) * 64 + lane;
    if (layout == LAYOUT_KC) {
      const int row = slot / CPR, c = (slot % CPR) ^ swz(row);
      const int g = min(row0 + row, rows - 1);
      s.off = (uint32_t)(((int64_t)(g - row0) * ld) * 2 + c * 16);
      s.krow = 0;
    } else {
      const int U = W_ / 8;  // 16-byte units per k row
      const int kr = slot / U, su = slot % U;
      const int u = W_ == 256 ? su ^ (4 * (kr & 3)) : (su + U - 4 * ((kr >> 1) & 1)) % U;
      const int64_t col = min((int64_t)row0 + u * 8, mcols - 8);
      s.off = (uint32_t)(col * 2);
      s.krow = kr;
    }
    return s;
  };
  Src sa[LPO], sb[LPO_B];
#pragma unroll
  for (int i = 0; i < LPO; ++i) sa[i] = make_src(LA, p.lda, p.M, m0, p.a_mcols, i, G::BM);
#pragma unroll
  for (int i = 0; i < LPO_B; ++i) sb[i] = make_src(LB, p.ldb, p.N, n0, p.b_mcols, i, G::BN);
  // Uniform base of one operand's stage kt.
  auto stage_base = [&](int layout, const void* X, int64_t ld, int row0, int kt) -> const char* {
    const int64_t k0 = kb + (int64_t)kt * BK;
    if (layout == LAYOUT_KC) return (const char*)X + ((int64_t)row0 * ld + k0) * 2;
    return (const char*)X + k0 * ld * 2;
  };
  auto lane_off = [&](int layout, const Src& s, int64_t ld, int64_t krows, int kt) -> uint32_t {
    if (layout == LAYOUT_KC) return s.off;
    const int64_t k0 = kb + (int64_t)kt * BK;
    const int64_t kr = min((int64_t)s.krow, krows - 1 - k0);
    return (uint32_t)(kr * ld * 2) + s.off;
  };
  auto issue = [&](int kt) {
    char* base = smem + (kt % NSTAGE) * STG;
    const char* ba = stage_base(LA, p.A, p.lda, m0, kt);
    const char* bb = stage_base(LB, p.B, p.ldb, n0, kt);
#pragma unroll
    for (int i = 0; i < LPO; ++i)
      load16_lds(ba, lane_off(LA, sa[i], p.lda, p.a_krows, kt), base + (i * G::kWaves + wid) * 1024);
#pragma unroll
    for (int i = 0; i < LPO_B; ++i)
      load16_lds(bb, lane_off(LB, sb[i], p.ldb, p.b_krows, kt), base + TILE + (i * G::kWaves + wid) * 1024);
  };
  // Part `part` of NPART of a stage's loads (A loads first, then B): the
  // loads of the next stage are spread over the k-groups of the current step
  // so that their LDS writes do not arrive as one burst against the fragment
  // reads (three parts, in the first three of four k-groups; two with EB,
  // whose last load then still has two k-groups to land before the barrier:
  // measured 1% faster per step than two parts everywhere).
  // With two stages the k-step barrier can sit before the last k-group's
  // MFMAs instead of after them (EB): by then every fragment of the stage is
  // in registers, so the next stage's first fragments are read while those
  // MFMAs run rather than after the barrier, when all wavefronts would read
  // at once with the matrix cores idle. The next stage's loads then go out
  // over the k-groups before the last one. Measured per product, this pays
  // only for dW (about 5% per launch); dH and the 256 x 256 tiles ran 3-6%
  // slower with it, and the forward and dZ tiles (single-buffered B
  // fragments) no longer fit their registers.
  constexpr bool EB = KDKL_EARLY_BARRIER && EPI == EPI_DW && NSTAGE == 2 && KG >= 2 && !G::kSingleB;
  constexpr int KGI = EB ? KG - 1 : KG;  // k-groups that issue loads
  constexpr int SPREAD = EB ? KDKL_DMA_SPREAD_EB : KDKL_DMA_SPREAD;
  constexpr int NPART = SPREAD < KGI ? SPREAD : KGI;
  auto issue_part = [&](int kt, int part) {
    char* base = smem + (kt % NSTAGE) * STG;
    const char* ba = stage_base(LA, p.A, p.lda, m0, kt);
    const char* bb = stage_base(LB, p.B, p.ldb, n0, kt);
#pragma unroll
    for (int q = 0; q < LPS; ++q) {
      if (q * NPART / LPS != part) continue;
      if (q < LPO)
        load16_lds(ba, lane_off(LA, sa[q], p.lda, p.a_krows, kt), base + (q * G::kWaves + wid) * 1024);
      else
        load16_lds(bb, lane_off(LB, sb[q - LPO], p.ldb, p.b_krows, kt),
                   base + TILE + ((q - LPO) * G::kWaves + wid) * 1024);
    }
  };

  f32x16_t acc[MB][NB];
  zero_acc<G>(acc);
  constexpr bool SB = G::kSingleB;
  bf16x8_t fa[2][MB], fb[SB ? 1 : 2][NB];
  // One MFMA operand fragment (8 consecutive k of output row/column `r0 +
  // (lane & 31)`) from an operand tile in either layout.
  auto frag = [&](int layout, const char* s, int r0, int kk, int W_) -> bf16x8_t {
    if (layout == LAYOUT_KC) {
      const int row = r0 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      return *(const bf16x8_t*)(s + row * RB + ((c ^ swz(row)) << 4));
    } else {
      // 8-byte item q of k row k sits at item mc_unit(k, q / 2) * 2 + q % 2
      const int q = ((r0 + 16 * ((lane >> 4) & 1)) >> 2) + (lane & 3);
      bf16x8_t v;
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const int k = kk * 16 + 8 * (lane >> 5) + 4 * j2 + ((lane & 15) >> 2);
        const int pq = W_ == 256 ? q ^ (8 * (k & 3)) : (q + 8 * ((k >> 1) & 1)) % (W_ / 4);
        const s16x4_t h = ds_read_tr16(s + k * (W_ * 2) + pq * 8);
        const bf16x4_t hb = __builtin_bit_cast(bf16x4_t, h);
        v[4 * j2 + 0] = hb[0];
        v[4 * j2 + 1] = hb[1];
        v[4 * j2 + 2] = hb[2];
        v[4 * j2 + 3] = hb[3];
      }
      return v;
    }
  };
  auto load_frags = [&](int kt, int kk, int buf, bool with_b) {
    const char* sA = smem + (kt % NSTAGE) * STG;
    const char* sB = sA + TILE;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) fa[buf][mb] = frag(LA, sA, wm * G::WM + mb * 32, kk, G::BM);
    if (with_b)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) fb[SB ? 0 : buf][nb] = frag(LB, sB, wn * G::WN + nb * 32, kk, G::BN);
  };

  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
      if (s < nk) issue(s);
    if (nk >= NSTAGE - 1)
      wait_vmcnt<LPS * (NSTAGE - 2)>();
    else
      wait_vmcnt<0>();
    phase_barrier();
    load_frags(0, 0, 0, true);
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + NSTAGE - 1 < nk;
      const bool next = kt + 1 < nk;
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        // fragments of this k-group read through the transpose (assembly,
        // issued one k-group earlier) are waited for before anything else;
        // the fence keeps the previous k-group's MFMAs ahead of that wait
        if constexpr (LA == LAYOUT_MC || LB == LAYOUT_MC) __builtin_amdgcn_sched_barrier(0);
        if constexpr (LA == LAYOUT_MC) lds_ready(fa[kk & 1]);
        if constexpr (LB == LAYOUT_MC) lds_ready(fb[SB ? 0 : (kk & 1)]);
        if (more) {
#pragma unroll
          for (int part = 0; part < NPART; ++part)
            if (part * KGI / NPART == kk) issue_part(kt + NSTAGE - 1, part);
        }
        if (EB && kk == KG - 1) {
          // this wavefront's fragment reads and stage loads are complete;
          // after the barrier so are everyone's (the stage may be reused and
          // the next one has landed)
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          wait_vmcnt<0>();
          phase_barrier();
        }
        if (kk + 1 < KG)
          load_frags(kt, kk + 1, (kk + 1) & 1, !SB);
        else if (EB && next)
          load_frags(kt + 1, 0, 0, !SB);
        frag_fence<!SB>();
        if constexpr (SB) {
          // each B fragment is replaced by the next k-group's once its MFMAs
          // are issued (with EB, after the last k-group: the next stage's first)
          const char* sB = smem + (kt % NSTAGE) * STG + TILE;
          const char* sBn = smem + ((kt + 1) % NSTAGE) * STG + TILE;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][mb], fb[0][nb], acc[mb][nb], 0, 0, 0);
            frag_fence<false>();
            if (kk + 1 < KG)
              fb[0][nb] = frag(LB, sB, wn * G::WN + nb * 32, kk + 1, G::BN);
            else if (EB && next)
              fb[0][nb] = frag(LB, sBn, wn * G::WN + nb * 32, 0, G::BN);
            frag_fence<false>();
          }
        } else {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[mb][nb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][mb], fb[kk & 1][nb], acc[mb][nb], 0, 0, 0);
        }
      }
      if constexpr (!EB) {
        // stage kt + 1 must have landed; later stages may still be in flight
        if (more)
          wait_vmcnt<LPS * (NSTAGE - 2)>();
        else
          wait_vmcnt<0>();
        phase_barrier();
        if (next) load_frags(kt + 1, 0, 0, true);
      }
    }
  }
  gemm_epilogue<G, 2, EPI>(p, acc, t, smem);
}

using FastGrid = typename std::conditional<
    KDKL_GEMM_WAVES == 16, Grid16, typename std::conditional<KDKL_GEMM_WAVES == 8, Grid8, Grid4>::type>::type;

// Byte span of one stage's direct loads from its buffer-resource base: the
// lane offsets are 32-bit and the resource's range is 2^31 - 1 bytes.
static bool span_fits(int layout, int64_t ld, int64_t mcols) {
  const int64_t span = layout == LAYOUT_KC ? (384 * ld + KDKL_GEMM_BK) * 2 : (KDKL_GEMM_BK * ld + mcols) * 2;
  return span < ((int64_t)1 << 31);
}

bool gemm_fast_path(int dtype, int64_t d, int64_t Vp, int64_t Cp) {
  const int64_t ld = d > Vp ? (d > Cp ? d : Cp) : (Vp > Cp ? Vp : Cp);
  return dtype == 1 && d % KDKL_GEMM_BK == 0 && span_fits(LAYOUT_KC, ld, 0) && span_fits(LAYOUT_MC, Vp, Vp);
}

// dW multiplies a k-major dZ tile (two transposed LDS reads per fragment)
// by a K-contiguous H^T tile: a 4 x 2 wave grid (64 x 128 per wave) gives
// each wave fewer dZ fragments than the 2 x 4 grid of the other products.
using DwGrid = typename std::conditional<KDKL_GEMM_WAVES == 8 && KDKL_DW_GRID42, Grid<4, 2>, FastGrid>::type;

#ifndef KDKL_D320
#define KDKL_D320 1
#endif
#ifndef KDKL_V384
#define KDKL_V384 1
#endif
int gemm_vocab_tile(bool fast, int64_t V, int64_t token_tiles) {
  if (!fast || !KDKL_V384) return 256;
  // Workgroups run in rounds of one per compute unit; a 384-row tile does
  // 1.5x the work of a 256-row one at about 5% better throughput. Keep 384
  // only when it takes less time over whole rounds (small or ragged
  // launches lose more to the partial last round than they gain).
  auto rounds = [&](int64_t vt) { return ((V + vt - 1) / vt * token_tiles + 255) / 256; };
  return rounds(384) * 384 * 19 < rounds(256) * 256 * 20 ? 384 : 256;
}

int gemm_d_tile(bool fast, int64_t d) {
  if (!fast || !KDKL_D320) return 256;
  const int64_t pad256 = (d + 255) / 256 * 256, pad320 = (d + 319) / 320 * 320;
  return pad320 < pad256 ? 320 : 256;
}

template <int EPI, int LA, int LB>
static hipError_t launch_fast(const GemmArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (EPI == EPI_FWD || EPI == EPI_DZ || EPI == EPI_DZJ) {
    if (a.bm == 384) {
      // 384 x 256 tiles on a 4 x 2 grid: wavefront tiles of 96 x 128
      using GV = Grid<4, 2, 256, 384>;
      hipLaunchKernelGGL((gemm_bf16_kernel<GV, EPI, KDKL_GEMM_BK, KDKL_GEMM_STAGES, LA, LB>), grid,
                         dim3(GV::kThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.bm != 0 && a.bm != 256) return hipErrorInvalidValue;
  if constexpr (EPI == EPI_DH || EPI == EPI_DW) {
    if (a.bn == 320) {
      // 256 x 320 tiles on a 4 x 2 grid: wavefront tiles of 64 x 160
      using GW = Grid<4, 2, 320>;
      hipLaunchKernelGGL((gemm_bf16_kernel<GW, EPI, KDKL_GEMM_BK, KDKL_GEMM_STAGES, LA, LB>), grid,
                         dim3(GW::kThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.bn != 0 && a.bn != 256) return hipErrorInvalidValue;
  using GG = typename std::conditional<EPI == EPI_DW, DwGrid, FastGrid>::type;
  hipLaunchKernelGGL((gemm_bf16_kernel<GG, EPI, KDKL_GEMM_BK, KDKL_GEMM_STAGES, LA, LB>), grid,
                     dim3(GG::kThreads), 0, s, a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t launch_gemm_e(int dtype, const GemmArgs& a, hipStream_t s) {
  const int total = a.tiles_m * a.tiles_n * a.splits;
  if (total <= 0) return hipSuccess;
  const int per = (total + 7) / 8;
  const dim3 grid(per * 8);
  const bool fast = dtype == 1 && a.k_end % KDKL_GEMM_BK == 0 && a.k_split % KDKL_GEMM_BK == 0 &&
                    span_fits(a.a_layout, a.lda, a.a_mcols) && span_fits(a.b_layout, a.ldb, a.b_mcols);
  if (fast) {
    // the operand layouts each projection uses
    if (a.a_layout == LAYOUT_KC && a.b_layout == LAYOUT_KC) {
      return launch_fast<EPI, LAYOUT_KC, LAYOUT_KC>(a, grid, s);
    }
    if constexpr (EPI == EPI_DW)
      if (a.a_layout == LAYOUT_MC && a.b_layout == LAYOUT_KC) return launch_fast<EPI, LAYOUT_MC, LAYOUT_KC>(a, grid, s);
    if constexpr (EPI == EPI_DH)
      if (a.a_layout == LAYOUT_KC && a.b_layout == LAYOUT_MC) return launch_fast<EPI, LAYOUT_KC, LAYOUT_MC>(a, grid, s);
    return hipErrorInvalidValue;
  }
  if (a.a_layout != LAYOUT_KC || a.b_layout != LAYOUT_KC) return hipErrorInvalidValue;
  if ((a.bn != 0 && a.bn != 256) || (a.bm != 0 && a.bm != 256)) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL((gemm_generic_kernel<uint16_t, EPI>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_generic_kernel<float, EPI>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_FWD: return launch_gemm_e<EPI_FWD>(dtype, a, s);
    case EPI_DZ: return launch_gemm_e<EPI_DZ>(dtype, a, s);
    case EPI_DZJ: return launch_gemm_e<EPI_DZJ>(dtype, a, s);
    case EPI_DH: return launch_gemm_e<EPI_DH>(dtype, a, s);
    default: return launch_gemm_e<EPI_DW>(dtype, a, s);
  }
}

int gemm_k_step(int dtype) { return dtype == 1 ? KDKL_GEMM_BK : 32; }

}  // namespace kdkl
