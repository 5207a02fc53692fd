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
//            chunk buffers in two layouts (token-major and vocab-major).
//   EPI_DH   dH partial = dZ . W over a split of the vocabulary (split-K).
//   EPI_DW   dW (+)= dZ^T . H over the chunk's tokens.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kdkl_internal.h"

namespace kdkl {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

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
//   sorted ids below t * kVocabTile (so a tile's teacher entries are the
//   contiguous range [tstart[t], tstart[t+1])).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void teacher_prep_kernel(TeacherArgs a) {
  __shared__ int32_t s_ids[1024];
  __shared__ int32_t s_sorted[1024];
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const int K = a.K;
  const int64_t g = (a.r0 + row) * (int64_t)K;
  constexpr int MAXE = 1024 / 64;
  float av[MAXE];
  int32_t iv[MAXE];
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < MAXE; ++j) {
    const int k = lane + 64 * j;
    if (k < K) {
      av[j] = a.logits[g + k] * a.inv_T;
      iv[j] = a.ids[g + k];
      s_ids[k] = iv[j];
      mx = fmaxf(mx, av[j]);
    } else {
      av[j] = kNegInf;
      iv[j] = 0;
    }
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < MAXE; ++j)
    if (lane + 64 * j < K) se += fast_exp(av[j] - mx);
  for (int o = 32; o > 0; o >>= 1) se += shfl_xor(se, o);
  const float lse = mx + fast_log(se);
  __syncthreads();
  float ent = 0.f;
#pragma unroll
  for (int j = 0; j < MAXE; ++j) {
    const int k = lane + 64 * j;
    if (k < K) {
      const float lp = av[j] - lse;
      const float p = fast_exp(lp);
      ent += p * lp;
      // rank of (id, k) in ascending id order, ties by position
      int rank = 0;
      const int id = iv[j];
      for (int q = 0; q < K; ++q) {
        const int o = s_ids[q];
        rank += (o < id) | ((o == id) & (q < k));
      }
      a.sids[(int64_t)row * K + rank] = id;
      a.sp[(int64_t)row * K + rank] = p;
      s_sorted[rank] = id;
    }
  }
  for (int o = 32; o > 0; o >>= 1) ent += shfl_xor(ent, o);
  if (lane == 0) a.erow[row] = ent;
  __syncthreads();
  for (int t = lane; t <= a.n_vt; t += 64) {
    const int64_t bound = (int64_t)t * kVocabTile;
    int lo = 0, hi = K;  // first index with sorted id >= bound
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)s_sorted[mid] < bound) lo = mid + 1; else hi = mid;
    }
    a.tstart[(int64_t)t * a.Cp + row] = (uint16_t)lo;
  }
}

hipError_t launch_teacher(const TeacherArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(teacher_prep_kernel, dim3(a.rows), dim3(64), 0, s, a);
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
    a.row_kl[row] = a.erow[row] - gsum + lse;
  }
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((a.rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Loss: (1/N) sum_i KL_i, fp64 accumulation in a fixed order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void loss_kernel(const float* row_kl, int64_t N, float* loss) {
  __shared__ double red[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) acc += (double)row_kl[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(red[0] / (double)N);
}

hipError_t launch_loss(const float* row_kl, int64_t N, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(1024), 0, s, row_kl, N, loss);
  return hipGetLastError();
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

hipError_t launch_transpose(int elem_bytes, const void* in, int64_t R, int64_t C, int64_t ldi,
                            void* out, int64_t Rp, int64_t ldo, hipStream_t s) {
  if (Rp <= 0 || C <= 0) return hipSuccess;
  dim3 grid((unsigned)((Rp + 63) / 64), (unsigned)((C + 63) / 64));
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
// dH = sum over splits of the fp32 partials, in split order.
// ---------------------------------------------------------------------------
template <int BF16>
__global__ __launch_bounds__(256) void dh_reduce_kernel(const float* __restrict__ part, int splits,
                                                        int64_t n_elems, int64_t stride,
                                                        void* __restrict__ dH) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= n_elems) return;
  float4 acc = *(const float4*)(part + i4);
  for (int s = 1; s < splits; ++s) {
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
                            void* dH, hipStream_t s) {
  const int64_t n = (int64_t)rows * d;  // d is a multiple of 4
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n / 4 + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL(dh_reduce_kernel<1>, dim3(blocks), dim3(256), 0, s, part, splits, n, Cp * d, dH);
  else
    hipLaunchKernelGGL(dh_reduce_kernel<0>, dim3(blocks), dim3(256), 0, s, part, splits, n, Cp * d, dH);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MFMA GEMM main loop.
//
// C[m, n] = sum_k A[m, k] B[n, k]; A and B row-major with k contiguous.
// Workgroup tile BM x BN, 4 wavefronts in a 2 x 2 grid, each owning a
// (BM/2) x (BN/2) sub-tile made of 32 x 32 MFMA blocks. Each LDS row holds
// 128 bytes of k (64 bf16 or 32 fp32) as eight 16-byte chunks stored at
// chunk ^ (row & 7), so the 32 lanes that read one column of chunks from 32
// consecutive rows hit distinct banks. Two LDS stages; global loads for the
// next k-step are issued before the MFMAs of the current one.
//
// MFMA operand layout used (32 x 32 output block): lane l feeds row (l & 31)
// of A and column (l & 31) of B with 8 consecutive k elements taken at
// offset 8 * (l >> 5) of the current 16-element k-group; accumulator
// register r of lane l holds output row 8 * (r >> 2) + 4 * (l >> 5) + (r & 3),
// column (l & 31).
// ---------------------------------------------------------------------------
template <typename TE>
struct Mfma;

template <>
struct Mfma<uint16_t> {  // bf16 storage
  struct Frag { bf16x8_t v; };
  static __device__ __forceinline__ Frag load(const char* p) {
    Frag f;
    f.v = *(const bf16x8_t*)p;
    return f;
  }
  static __device__ __forceinline__ void mma(const Frag& a, const Frag& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
  }
  static constexpr int kChunksPerGroup = 1;  // 16-byte chunks per lane per k-group
};

template <>
struct Mfma<float> {
  struct Frag { f32x4_t lo, hi; };
  static __device__ __forceinline__ Frag load(const char* p0, const char* p1) {
    Frag f;
    f.lo = *(const f32x4_t*)p0;
    f.hi = *(const f32x4_t*)p1;
    return f;
  }
  static __device__ __forceinline__ void mma(const Frag& a, const Frag& b, f32x16_t& c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[e], b.hi[e], c, 0, 0, 0);
  }
  static constexpr int kChunksPerGroup = 2;
};

template <typename TE, int ROWS>
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
    *(uint4*)(s + row * 128 + ((c ^ (row & 7)) << 4)) = r[i];
  }
}

__device__ __forceinline__ int acc_row(int wm, int WMr, int mb, int r, int lane) {
  return wm * WMr + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <typename TE, int BM, int BN, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_kernel(const GemmArgs p) {
  using M_ = Mfma<TE>;
  constexpr int ES = sizeof(TE);
  constexpr int BK = 128 / ES;  // elements per k-step
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
  // give each XCD a contiguous run of tiles (neighbours share an A tile).
  const int total = p.tiles_m * p.tiles_n * p.splits;
  const int per = (total + 7) >> 3;
  const int L = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (L >= total) return;
  const int tn = L % p.tiles_n;
  const int tm = (L / p.tiles_n) % p.tiles_m;
  const int ks = L / (p.tiles_n * p.tiles_m);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t kb = (int64_t)ks * p.k_split;
  const int64_t ke = kb + p.k_split < p.k_end ? kb + p.k_split : p.k_end;
  const int nk = ke > kb ? (int)((ke - kb + BK - 1) / BK) : 0;

  // Teacher ranges of this lane's token columns, fetched before the main loop.
  int hit_lo[NB], hit_hi[NB];
  if constexpr (EPI == EPI_FWD || EPI == EPI_DZ) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = n0 + wn * WN + nb * 32 + (lane & 31);
      if (col < p.N) {
        hit_lo[nb] = p.tstart[(int64_t)tm * p.Cp + col];
        hit_hi[nb] = p.tstart[(int64_t)(tm + 1) * p.Cp + col];
      } else {
        hit_lo[nb] = hit_hi[nb] = 0;
      }
    }
  }

  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const char* Ab = (const char*)p.A;
  const char* Bb = (const char*)p.B;
  const int64_t lda_b = p.lda * ES, ldb_b = p.ldb * ES;
  const int64_t kend_b = ke * ES;
  uint4 ra[BM * 8 / 256], rb[BN * 8 / 256];

  if (nk > 0) {
    g2r<TE, BM>(ra, Ab, lda_b, m0, p.M, kb * ES, kend_b, tid);
    g2r<TE, BN>(rb, Bb, ldb_b, n0, p.N, kb * ES, kend_b, tid);
    r2s<BM>(ra, smem, tid);
    r2s<BN>(rb, smem + BM * 128, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) {
        const int64_t k0b = (kb + (int64_t)(kt + 1) * BK) * ES;
        g2r<TE, BM>(ra, Ab, lda_b, m0, p.M, k0b, kend_b, tid);
        g2r<TE, BN>(rb, Bb, ldb_b, n0, p.N, k0b, kend_b, tid);
      }
      const char* sA = smem + (kt & 1) * STAGE;
      const char* sB = sA + BM * 128;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        typename M_::Frag fa[MB], fb[NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = wm * WM + mb * 32 + (lane & 31);
          if constexpr (M_::kChunksPerGroup == 1) {
            const int c = kk * 2 + (lane >> 5);
            fa[mb] = M_::load(sA + row * 128 + ((c ^ (row & 7)) << 4));
          } else {
            const int c = kk * 4 + (lane >> 5) * 2;
            fa[mb] = M_::load(sA + row * 128 + ((c ^ (row & 7)) << 4),
                              sA + row * 128 + (((c + 1) ^ (row & 7)) << 4));
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int row = wn * WN + nb * 32 + (lane & 31);
          if constexpr (M_::kChunksPerGroup == 1) {
            const int c = kk * 2 + (lane >> 5);
            fb[nb] = M_::load(sB + row * 128 + ((c ^ (row & 7)) << 4));
          } else {
            const int c = kk * 4 + (lane >> 5) * 2;
            fb[nb] = M_::load(sB + row * 128 + ((c ^ (row & 7)) << 4),
                              sB + row * 128 + (((c + 1) ^ (row & 7)) << 4));
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) M_::mma(fa[mb], fb[nb], acc[mb][nb]);
      }
      if (more) {
        char* s = smem + ((kt + 1) & 1) * STAGE;
        r2s<BM>(ra, s, tid);
        r2s<BN>(rb, s + BM * 128, tid);
      }
      __syncthreads();
    }
  }

  // ------------------------------- epilogues -------------------------------
  if constexpr (EPI == EPI_FWD) {
    // s = z / T for the tile's vocabulary rows (A rows) and token columns.
    float* red = (float*)smem;  // [2][BN][3]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int ct = wn * WN + nb * 32 + (lane & 31);
      const int col = n0 + ct;
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + acc_row(wm, WM, mb, r, lane);
          const float s = row < p.V ? acc[mb][nb][r] * p.inv_T : kNegInf;
          acc[mb][nb][r] = s;
          mx = fmaxf(mx, s);
        }
      mx = fmaxf(mx, shfl_xor(mx, 32));
      float se = 0.f;
      if (mx > kNegInf) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) se += fast_exp(acc[mb][nb][r] - mx);
      }
      se += shfl_xor(se, 32);
      // teacher-weighted logits of the ids that fall in this lane's rows
      float gam = 0.f;
      for (int h = hit_lo[nb]; h < hit_hi[nb]; ++h) {
        const int id = p.sids[(int64_t)col * p.K + h];
        const int r = id - m0 - wm * WM;
        if (id >= p.V || r < 0 || r >= WM) continue;
        const int rin = r & 31;
        if (((rin >> 2) & 1) != (lane >> 5)) continue;
        const int slot = (r >> 5) * 16 + ((rin >> 3) << 2) + (rin & 3);
        float v = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) v = (mb * 16 + rr == slot) ? acc[mb][nb][rr] : v;
        gam += p.sp[(int64_t)col * p.K + h] * v;
      }
      gam += shfl_xor(gam, 32);
      if (lane < 32) {
        float* e = red + (wm * BN + ct) * 3;
        e[0] = mx; e[1] = se; e[2] = gam;
      }
    }
    __syncthreads();
    for (int c = tid; c < BN; c += 256) {
      const int col = n0 + c;
      if (col >= p.N) continue;
      const float* e0 = red + c * 3;
      const float* e1 = red + (BN + c) * 3;
      const float m = fmaxf(e0[0], e1[0]);
      float s = 0.f;
      if (m > kNegInf) {
        if (e0[0] > kNegInf) s += e0[1] * fast_exp(e0[0] - m);
        if (e1[0] > kNegInf) s += e1[1] * fast_exp(e1[0] - m);
      }
      p.part[(int64_t)col * p.n_vt + tm] = make_float4(m, s, e0[2] + e1[2], 0.f);
    }
  } else if constexpr (EPI == EPI_DZ) {
    const float g = p.grad ? p.grad[0] : 1.0f;
    const float coef = g * p.coef_base;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int ct = wn * WN + nb * 32 + (lane & 31);
      const int col = n0 + ct;
      const bool cval = col < p.N;
      const float lse = cval ? p.row_lse[col] : 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + acc_row(wm, WM, mb, r, lane);
          const float q = fast_exp(acc[mb][nb][r] * p.inv_T - lse);
          acc[mb][nb][r] = (row < p.V && cval) ? q : 0.f;
        }
      for (int h = hit_lo[nb]; h < hit_hi[nb]; ++h) {
        const int id = p.sids[(int64_t)col * p.K + h];
        const int r = id - m0 - wm * WM;
        if (id >= p.V || r < 0 || r >= WM) continue;
        const int rin = r & 31;
        if (((rin >> 2) & 1) != (lane >> 5)) continue;
        const int slot = (r >> 5) * 16 + ((rin >> 3) << 2) + (rin & 3);
        const float pk = p.sp[(int64_t)col * p.K + h];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            acc[mb][nb][rr] = (mb * 16 + rr == slot) ? acc[mb][nb][rr] - pk : acc[mb][nb][rr];
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int row = m0 + acc_row(wm, WM, mb, r4 * 4, lane);  // 4 consecutive rows
          const float v0 = acc[mb][nb][r4 * 4 + 0] * coef, v1 = acc[mb][nb][r4 * 4 + 1] * coef;
          const float v2 = acc[mb][nb][r4 * 4 + 2] * coef, v3 = acc[mb][nb][r4 * 4 + 3] * coef;
          if constexpr (ES == 2) {
            uint16_t* cv = (uint16_t*)p.dz_cv;
            uint16_t* vc = (uint16_t*)p.dz_vc;
            ushort4 o;
            o.x = f32_to_bf16_bits(v0); o.y = f32_to_bf16_bits(v1);
            o.z = f32_to_bf16_bits(v2); o.w = f32_to_bf16_bits(v3);
            *(ushort4*)(cv + (int64_t)col * p.Vp + row) = o;
            vc[(int64_t)(row + 0) * p.Cp + col] = o.x;
            vc[(int64_t)(row + 1) * p.Cp + col] = o.y;
            vc[(int64_t)(row + 2) * p.Cp + col] = o.z;
            vc[(int64_t)(row + 3) * p.Cp + col] = o.w;
          } else {
            float* cv = (float*)p.dz_cv;
            float* vc = (float*)p.dz_vc;
            *(float4*)(cv + (int64_t)col * p.Vp + row) = make_float4(v0, v1, v2, v3);
            vc[(int64_t)(row + 0) * p.Cp + col] = v0;
            vc[(int64_t)(row + 1) * p.Cp + col] = v1;
            vc[(int64_t)(row + 2) * p.Cp + col] = v2;
            vc[(int64_t)(row + 3) * p.Cp + col] = v3;
          }
        }
    }
  } else {
    // EPI_DH: out = partials of split ks, [Cp, ldo]; EPI_DW: out = dW [V, ldo]
    float* out = p.out + (EPI == EPI_DH ? (int64_t)ks * p.Cp * p.ldo : 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = n0 + wn * WN + nb * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + acc_row(wm, WM, mb, r, lane);
          if (row < p.M) {
            float* o = out + (int64_t)row * p.ldo + col;
            if (EPI == EPI_DW && p.accumulate)
              *o += acc[mb][nb][r];
            else
              *o = acc[mb][nb][r];
          }
        }
    }
  }
}

template <typename TE, int EPI>
static hipError_t launch_gemm_t(const GemmArgs& a, hipStream_t s) {
  const int total = a.tiles_m * a.tiles_n * a.splits;
  if (total <= 0) return hipSuccess;
  const int per = (total + 7) / 8;
  hipLaunchKernelGGL((gemm_kernel<TE, 256, 256, EPI>), dim3(per * 8), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& a, hipStream_t s) {
  if (dtype == 1) {
    switch (epi) {
      case EPI_FWD: return launch_gemm_t<uint16_t, EPI_FWD>(a, s);
      case EPI_DZ: return launch_gemm_t<uint16_t, EPI_DZ>(a, s);
      case EPI_DH: return launch_gemm_t<uint16_t, EPI_DH>(a, s);
      default: return launch_gemm_t<uint16_t, EPI_DW>(a, s);
    }
  }
  switch (epi) {
    case EPI_FWD: return launch_gemm_t<float, EPI_FWD>(a, s);
    case EPI_DZ: return launch_gemm_t<float, EPI_DZ>(a, s);
    case EPI_DH: return launch_gemm_t<float, EPI_DH>(a, s);
    default: return launch_gemm_t<float, EPI_DW>(a, s);
  }
}

int gemm_k_step(int dtype) { return dtype == 1 ? 64 : 32; }

}  // namespace kdkl
