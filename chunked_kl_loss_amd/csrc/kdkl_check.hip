// Optional validation of the teacher top-K ids (kdkl_check_ids). The loss
// itself does not need it: an id outside [0, V) is dropped and repeated ids
// add their mass. A caller that wants to know whether its cache holds such
// entries counts them here. Deterministic: per-block partial counts, then a
// fixed-order sum by one block (no atomics).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kdkl_internal.h"

namespace kdkl {

namespace {

constexpr int kCheckThreads = 256;  // four wavefronts, one row each at a time

__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// partial[2 b] = ids outside [0, V) in kept rows handled by block b,
// partial[2 b + 1] = kept rows of block b holding some id twice.
__global__ __launch_bounds__(kCheckThreads) void check_ids_kernel(const int32_t* __restrict__ ids, int64_t N,
                                                                  int K, int64_t V,
                                                                  long long* __restrict__ partial) {
  __shared__ long long red[kCheckThreads / 64][2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  long long bad = 0, dup_rows = 0;
  for (int64_t row = (int64_t)blockIdx.x * (kCheckThreads / 64) + w; row < N;
       row += (int64_t)gridDim.x * (kCheckThreads / 64)) {
    const int32_t* r = ids + row * K;
    if (r[0] == kIgnoreId) continue;  // ignored position: its ids are never used
    long long b = 0;
    int dup = 0;
    for (int k = lane; k < K; k += 64) {
      const int32_t id = r[k];
      b += (id < 0 || (int64_t)id >= V) ? 1 : 0;
      for (int j = k + 1; j < K; ++j) dup |= r[j] == id;
    }
    b = wave_sum_ll(b);
    dup = (int)wave_sum_ll(dup);
    if (lane == 0) {
      bad += b;
      dup_rows += dup > 0 ? 1 : 0;
    }
  }
  if (lane == 0) {
    red[w][0] = bad;
    red[w][1] = dup_rows;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long a = 0, c = 0;
    for (int i = 0; i < kCheckThreads / 64; ++i) {
      a += red[i][0];
      c += red[i][1];
    }
    partial[2 * blockIdx.x] = a;
    partial[2 * blockIdx.x + 1] = c;
  }
}

__global__ __launch_bounds__(64) void check_ids_sum_kernel(const long long* __restrict__ partial, int blocks,
                                                           int64_t* __restrict__ out) {
  if (threadIdx.x != 0) return;
  long long a = 0, c = 0;
  for (int b = 0; b < blocks; ++b) {
    a += partial[2 * b];
    c += partial[2 * b + 1];
  }
  out[0] = a;
  out[1] = c;
}

}  // namespace

int check_ids_blocks(int64_t N) {
  const int64_t b = (N + kCheckThreads / 64 - 1) / (kCheckThreads / 64);
  return (int)(b < kCheckIdsMaxBlocks ? (b > 0 ? b : 1) : kCheckIdsMaxBlocks);
}

hipError_t launch_check_ids(const int32_t* ids, int64_t N, int K, int64_t V, void* partial, int64_t* out,
                            hipStream_t s) {
  const int blocks = check_ids_blocks(N);
  hipLaunchKernelGGL(check_ids_kernel, dim3(blocks), dim3(kCheckThreads), 0, s, ids, N, K, V,
                     (long long*)partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(check_ids_sum_kernel, dim3(1), dim3(64), 0, s, (const long long*)partial, blocks, out);
  return hipGetLastError();
}

}  // namespace kdkl
