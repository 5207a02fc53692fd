// Device kernels of the forward-chunked KL loss: the student's logit grid
// Z [N, V] is given (the output layer computed it in full and keeps it for
// the backward pass) and the teacher stays sparse, its cached top-K per
// position [P1 "Making knowledge distillation cheap enough to run at scale",
// section "Two system changes", forward-chunked KL bullet].
//
// Both passes stream Z once and are bound by HBM bandwidth. Rows are
// independent, so the pages' slicing over positions is the grid itself and
// no chunk buffer exists: in the forward one wavefront owns one row
// (position); the backward gives a long row of whole 16-byte vectors to
// 256-thread workgroups in contiguous pieces (consecutive workgroups stream
// consecutive memory) and any other row to one wavefront.
//   forward : lse_i = log sum_v exp(z_iv / T) (online, base 2), and
//             KL_i = e_i - gamma_i + lse_i with e_i = sum_k p_ik log p_ik and
//             gamma_i = sum_k p_ik z_i[id_ik] / T.
//   backward: dZ_iv = g/(N T) (exp(z_iv / T - lse_i) - sum_k p_ik [v = id_ik]).
// An id outside [0, V) adds nothing to gamma or to the gradient (its teacher
// mass is dropped) and is never dereferenced. A position whose first teacher
// id is -1 is ignored: KL 0 and a zero gradient row; the mean and the
// gradient scale count only kept positions.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kdkl_internal.h"

namespace kdkl {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRowsPerBlock = 4;  // one wavefront per row

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += wave_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, wave_xor(v, o));
  return v;
}

// Element access for the two storage types. A 16-byte vector holds
// kVec elements.
template <typename TE>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 bits
  static constexpr int kVec = 8;
  __device__ static float load(const uint16_t* p) { return __builtin_bit_cast(float, (uint32_t)*p << 16); }
  __device__ static void store(uint16_t* p, float v) {
    *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  }
  __device__ static void unpack(const uint4& u, float (&x)[kVec]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __builtin_bit_cast(float, w[j] << 16);
      x[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
    }
  }
  __device__ static uint4 pack(const float (&y)[kVec]) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y[2 * j]));
      const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y[2 * j + 1]));
      w[j] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
  __device__ static void unpack(const uint4& u, float (&x)[kVec]) {
    x[0] = __builtin_bit_cast(float, u.x);
    x[1] = __builtin_bit_cast(float, u.y);
    x[2] = __builtin_bit_cast(float, u.z);
    x[3] = __builtin_bit_cast(float, u.w);
  }
  __device__ static uint4 pack(const float (&y)[kVec]) {
    return make_uint4(__builtin_bit_cast(uint32_t, y[0]), __builtin_bit_cast(uint32_t, y[1]),
                      __builtin_bit_cast(uint32_t, y[2]), __builtin_bit_cast(uint32_t, y[3]));
  }
};

// A row of V elements starting at element offset `start` of a 16-byte
// aligned buffer: `head` scalar elements up to the first 16-byte boundary,
// `nvec` whole vectors, then `tail` scalar elements.
struct RowSplit {
  int head, tail;
  int64_t nvec;
};

template <int VEC>
__device__ __forceinline__ RowSplit split_row(int64_t start, int64_t V) {
  RowSplit r;
  const int64_t mis = start % VEC;
  int64_t head = mis ? VEC - mis : 0;
  if (head > V) head = V;
  r.head = (int)head;
  r.nvec = (V - head) / VEC;
  r.tail = (int)(V - head - r.nvec * VEC);
  return r;
}

// Teacher top-K of one row, spread over the wavefront (entry k on lane
// k % 64, slot k / 64; KPL slots per lane hold K <= 64 KPL entries):
// p_k = softmax_k(l_k / T), e = sum_k p_k log p_k, and the student logit z at
// each in-range id (read before anything is written, so dZ may share storage
// with Z).
template <typename TE, int KPL>
struct TeacherRow {
  float p[KPL];
  float z[KPL];
  int id[KPL];
  bool ok[KPL];
  float e;  // wavefront total

  float av[KPL];  // l / T between request() and finish()

  // Requests the row's entries and, with gather, the student logits at their
  // ids (z stays 0 otherwise). Every lane issues its loads unconditionally
  // (clamped to valid addresses) and nothing waits for them here but the
  // gathers' own wait for the ids, so the requests stay in flight while the
  // caller goes on; finish() uses them.
  __device__ void request(const LogitsArgs& a, int64_t row, int lane, bool gather = true) {
    const int K = a.K;
    const int64_t g = row * (int64_t)K;
    const TE* zr = (const TE*)a.Z + row * a.V;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int k = lane + 64 * j;
      const int kk = k < K ? k : K - 1;
      av[j] = a.logits[g + kk];
      id[j] = a.ids[g + kk];
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (lane + 64 * j >= K) id[j] = -1;
      ok[j] = id[j] >= 0 && (int64_t)id[j] < a.V;
      z[j] = gather ? Elem<TE>::load(zr + (ok[j] ? id[j] : 0)) : 0.f;
    }
  }
  // p = softmax over K of l / T and e = sum_k p_k log p_k (wavefront total);
  // z at an id outside [0, V) reads as 0.
  __device__ void finish(const LogitsArgs& a, int lane) {
    const int K = a.K;
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      av[j] = lane + 64 * j < K ? av[j] * a.inv_T : kNegInf;
      mx = fmaxf(mx, av[j]);
      z[j] = ok[j] ? z[j] : 0.f;
    }
    mx = wave_max(mx);
    float se = 0.f;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (lane + 64 * j < K) se += exp2_hw((av[j] - mx) * kLog2e);
    const float lt = mx + log2_hw(wave_sum(se)) * kLn2;  // natural-log normaliser
    float ent = 0.f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      p[j] = 0.f;
      if (lane + 64 * j < K) {
        const float lp = av[j] - lt;
        p[j] = exp2_hw(lp * kLog2e);
        ent += p[j] * lp;
      }
    }
    e = wave_sum(ent);
  }
  __device__ void load(const LogitsArgs& a, int64_t row, int lane, bool gather = true) {
    request(a, row, lane, gather);
    finish(a, lane);
  }
};

// Sum of a vector of terms as a balanced tree (shorter dependency chains
// than a running sum; N a power of two).
template <int N>
__device__ __forceinline__ float tree_sum(const float (&e)[N]) {
  float t[N];
#pragma unroll
  for (int j = 0; j < N; ++j) t[j] = e[j];
#pragma unroll
  for (int w = N / 2; w > 0; w /= 2)
#pragma unroll
    for (int j = 0; j < w; ++j) t[j] = t[2 * j] + t[2 * j + 1];
  return t[0];
}

// Online (max, sum 2^(c (z - max))) over raw logits z with c = log2(e) / T:
// the max is taken over z itself (c > 0 keeps the order), so each term is
// one fused multiply-add and one exp2. The logsumexp of s = z / T is
// (m c + log2 sum) ln 2.
struct OnlineLse {
  float c, m = kNegInf, s = 0.f;
  __device__ explicit OnlineLse(float c_) : c(c_) {}
  __device__ void add(float z) {
    if (z == kNegInf) return;
    if (z > m) {
      s = s * exp2_hw((m - z) * c) + 1.f;
      m = z;
    } else {
      s += exp2_hw(__builtin_fmaf(z, c, -m * c));
    }
  }
  template <int N>
  __device__ void add_vec(const float (&z)[N]) {
    float mv = z[0];
#pragma unroll
    for (int j = 1; j < N; ++j) mv = fmaxf(mv, z[j]);
    if (mv == kNegInf) return;
    if (mv > m) {
      s *= exp2_hw((m - mv) * c);
      m = mv;
    }
    const float mc = -m * c;
    float e[N];
#pragma unroll
    for (int j = 0; j < N; ++j) e[j] = exp2_hw(__builtin_fmaf(z[j], c, mc));
    s += tree_sum(e);
  }
  // A group of U vectors of storage type TE with the running max allowed to
  // lag: the terms are formed against the current max and may exceed 1 (up
  // to 2^kLag) before it is raised, so the rescale runs only when some lane
  // of the wavefront meets a value that far above it (in practice at the
  // row's first group), and that group's terms are then formed again.
  static constexpr float kLag = 64.f;
  template <typename TE, int U>
  __device__ float group_terms(const uint4 (&u)[U], float& mv) const {
    constexpr int N = Elem<TE>::kVec;
    const float mc = m == kNegInf ? 0.f : -m * c;
    float sg = 0.f;
#pragma unroll
    for (int q = 0; q < U; ++q) {
      float z[N], e[N];
      Elem<TE>::unpack(u[q], z);
#pragma unroll
      for (int j = 0; j < N; ++j) {
        mv = fmaxf(mv, z[j]);
        e[j] = exp2_hw(__builtin_fmaf(z[j], c, mc));
      }
      sg += tree_sum(e);
    }
    return sg;
  }
  template <typename TE, int U>
  __device__ void add_group(const uint4 (&u)[U]) {
    float mv = kNegInf;
    float sg = group_terms<TE>(u, mv);
    // (mv - m) c is NaN, so false, for a group of -inf under m = -inf
    if (__builtin_amdgcn_ballot_w64((mv - m) * c > kLag) != 0) {
      const float nm = fmaxf(m, mv);
      if (nm > m) {
        s *= exp2_hw((m - nm) * c);
        m = nm;
        float unused = kNegInf;
        sg = group_terms<TE>(u, unused);
      }
    }
    s += sg;
  }
  __device__ void wave_merge() {
    for (int o = 32; o > 0; o >>= 1) {
      const float om = wave_xor(m, o), os = wave_xor(s, o);
      const float nm = fmaxf(m, om);
      if (nm > kNegInf) {
        s = (m > kNegInf ? s * exp2_hw((m - nm) * c) : 0.f) + (om > kNegInf ? os * exp2_hw((om - nm) * c) : 0.f);
        m = nm;
      }
    }
  }
  // natural-log logsumexp of z / T (after wave_merge)
  __device__ float lse() const { return (m * c + log2_hw(s)) * kLn2; }
};

constexpr int kUnroll = 4;  // 16-byte loads in flight per lane

// Streaming access to the logit grid: each byte is read once (and dZ written
// once), so both go out with the nontemporal hint. Besides keeping the caches
// for the reused data, it leaves no dirty dZ lines in the caches to be
// written back while the next pass streams Z.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, (u32x4_t*)p);
}
// kUnroll vectors STRIDE apart from p (one wavefront-wide group)
template <int STRIDE = 64>
__device__ __forceinline__ void load_group(uint4 (&u)[kUnroll], const uint4* p) {
#pragma unroll
  for (int q = 0; q < kUnroll; ++q) u[q] = load_stream(p + STRIDE * q);
}

template <typename TE, int KPL>
__global__ __launch_bounds__(64 * kRowsPerBlock) void logits_fwd_kernel(LogitsArgs a) {
  const int lane = threadIdx.x & 63;
  // the row is uniform over the wavefront: its addresses live in scalar registers
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= a.N) return;
  constexpr int VEC = Elem<TE>::kVec;
  const int64_t start = row * a.V;
  const TE* zr = (const TE*)a.Z + start;
  const RowSplit rs = split_row<VEC>(start, a.V);
  const uint4* vp = (const uint4*)(zr + rs.head);
  // Whole groups of kUnroll vectors per lane (the same count for every lane
  // of the wavefront), streamed with two register buffers: the next group
  // is in flight while the current one is reduced. The row's first group is
  // requested before the teacher entries, so their round trips overlap.
  const int64_t G = rs.nvec / (64 * kUnroll);
  const uint4* gp = vp + lane;
  uint4 A[kUnroll], B[kUnroll];
  if (G > 0) load_group(A, gp);
  TeacherRow<TE, KPL> t;
  t.request(a, row, lane);
  const bool keep = a.ids[row * a.K] != kIgnoreId;

  OnlineLse acc(kLog2e * a.inv_T);
  if (lane < rs.head) acc.add(Elem<TE>::load(zr + lane));
  auto reduce = [&](const uint4(&u)[kUnroll]) { acc.add_group<TE>(u); };
  // (the loads in the loop are unconditional, so each wait covers only the
  // group about to be used)
  int64_t g = 0;
  for (; g + 2 < G; g += 2) {
    load_group(B, gp + (g + 1) * 64 * kUnroll);
    reduce(A);
    load_group(A, gp + (g + 2) * 64 * kUnroll);
    reduce(B);
  }
  if (g + 1 < G) {
    load_group(B, gp + (g + 1) * 64 * kUnroll);
    reduce(A);
    reduce(B);
  } else if (g < G) {
    reduce(A);
  }
  int64_t i = G * 64 * kUnroll + lane;
  for (; i < rs.nvec; i += 64) {
    float x[VEC];
    Elem<TE>::unpack(load_stream(vp + i), x);
    acc.add_vec(x);
  }
  if (lane < rs.tail) acc.add(Elem<TE>::load(zr + rs.head + rs.nvec * VEC + lane));
  acc.wave_merge();
  t.finish(a, lane);
  float gam = 0.f;
#pragma unroll
  for (int j = 0; j < KPL; ++j) gam += t.p[j] * t.z[j];
  gam = wave_sum(gam) * a.inv_T;
  if (lane == 0) {
    const float lse = acc.lse();
    a.row_lse[row] = lse;
    a.row_kl[row] = keep ? t.e - gam + lse : 0.f;
  }
}

template <typename TE, int KPL>
__global__ __launch_bounds__(64 * kRowsPerBlock) void logits_bwd_kernel(LogitsArgs a) {
  __shared__ int32_t s_id[kRowsPerBlock][64 * KPL];
  __shared__ float s_p[kRowsPerBlock][64 * KPL];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + w;
  if (row >= a.N) return;
  constexpr int VEC = Elem<TE>::kVec;
  TeacherRow<TE, KPL> t;
  t.load(a, row, lane);
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int k = lane + 64 * j;
    if (k < a.K) {
      s_id[w][k] = t.id[j];
      s_p[w][k] = t.p[j];
    }
  }
  __builtin_amdgcn_wave_barrier();
  // The gathered logits must have been read before any store of this row
  // (dZ may be Z).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const bool keep = a.ids[row * a.K] != kIgnoreId;
  const float coef = keep ? a.scale[0] : 0.f;  // an ignored row's gradient is zero
  const float c = kLog2e * a.inv_T;
  const float lse2 = a.row_lse[row] * kLog2e;
  const int64_t start = row * a.V;
  const TE* zr = (const TE*)a.Z + start;
  TE* dr = (TE*)a.dZ + start;
  const RowSplit rs = split_row<VEC>(start, a.V);
  if (lane < rs.head) Elem<TE>::store(dr + lane, coef * exp2_hw(Elem<TE>::load(zr + lane) * c - lse2));
  const uint4* vp = (const uint4*)(zr + rs.head);
  uint4* op = (uint4*)(dr + rs.head);
  int64_t i = lane;
  for (; i + 64 * (kUnroll - 1) < rs.nvec; i += 64 * kUnroll) {
    uint4 u[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) u[q] = load_stream(vp + i + 64 * q);
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      float x[VEC];
      Elem<TE>::unpack(u[q], x);
#pragma unroll
      for (int j = 0; j < VEC; ++j) x[j] = coef * exp2_hw(x[j] * c - lse2);
      store_stream(op + i + 64 * q, Elem<TE>::pack(x));
    }
  }
  for (; i < rs.nvec; i += 64) {
    float x[VEC];
    Elem<TE>::unpack(load_stream(vp + i), x);
#pragma unroll
    for (int j = 0; j < VEC; ++j) x[j] = coef * exp2_hw(x[j] * c - lse2);
    store_stream(op + i, Elem<TE>::pack(x));
  }
  if (lane < rs.tail) {
    const int64_t v = rs.head + rs.nvec * VEC + lane;
    Elem<TE>::store(dr + v, coef * exp2_hw(Elem<TE>::load(zr + v) * c - lse2));
  }
  // Teacher entries: overwrite with the full value once the dense stores of
  // this wavefront have been performed (same addresses, written later).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    if (keep && lane + 64 * j < a.K && t.ok[j]) {
      float mass = 0.f;  // duplicates of an id add their mass
      for (int q = 0; q < a.K; ++q) mass += s_id[w][q] == t.id[j] ? s_p[w][q] : 0.f;
      Elem<TE>::store(dr + t.id[j], coef * (exp2_hw(t.z[j] * c - lse2) - mass));
    }
  }
}

// The backward on rows that are whole 16-byte vectors (V a multiple of the
// vector width), each row cut into `pieces` contiguous pieces of `len`
// vectors with one 256-thread workgroup per piece. Consecutive workgroups
// then stream consecutive memory (one wavefront per row interleaves four
// rows per workgroup), which the memory system serves faster for a read and
// write stream. The workgroup gathers the student logits at the row's teacher
// ids inside its piece before anything is written (so dZ may be Z), streams
// the dense part coef * q, and then rewrites those entries with the teacher
// mass subtracted (one rounding, as the row kernel does).
constexpr int kPieceThreads = 256;
constexpr int64_t kPieceVec = 16384;    // target 16-byte vectors per piece
constexpr int64_t kPieceMinVec = 2048;  // shorter rows take one wavefront each

template <typename TE, int KPS>  // teacher entries per thread: K <= 256 KPS
__global__ __launch_bounds__(kPieceThreads) void logits_bwd_piece_kernel(LogitsArgs a, int pieces, int64_t len) {
  constexpr int NT = kPieceThreads;
  __shared__ int32_t s_id[NT * KPS];
  __shared__ float s_p[NT * KPS];
  __shared__ float s_z[NT * KPS];
  constexpr int VEC = Elem<TE>::kVec;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t row = blockIdx.x / (unsigned)pieces;
  const int64_t pc = blockIdx.x - row * pieces;
  const int64_t nvec = a.V / VEC;
  const int64_t v0 = pc * len;
  const int64_t v1 = v0 + len < nvec ? v0 + len : nvec;
  const int64_t c0 = v0 * VEC, c1 = v1 * VEC;  // the piece's columns
  const TE* zr = (const TE*)a.Z + row * a.V;
  TE* dr = (TE*)a.dZ + row * a.V;
  const uint4* vp = (const uint4*)zr;
  uint4* op = (uint4*)dr;
  // Whole groups of kUnroll vectors per thread (the same count for the whole
  // workgroup), streamed with two register buffers A and B, one group ahead.
  // The first two groups are requested around the teacher entries, so the
  // piece's first round trips overlap.
  const int64_t G = (v1 - v0) / (NT * kUnroll);
  const uint4* gp = vp + v0 + tid;
  uint4* go = op + v0 + tid;
  uint4 A[kUnroll], B[kUnroll];
  if (G > 0) load_group<NT>(A, gp);
  // The teacher entries (loads clamped to valid addresses, unconditional).
  const int K = a.K;
  const int32_t* idr = a.ids + row * K;
  const float* lgr = a.logits + row * K;
  int id[KPS];
  float l[KPS], z[KPS];
#pragma unroll
  for (int j = 0; j < KPS; ++j) {
    const int k = tid + NT * j;
    const int kk = k < K ? k : K - 1;
    id[j] = idr[kk];
    l[j] = lgr[kk] * a.inv_T;
  }
  const float scale = a.scale[0];
  const float lse2 = a.row_lse[row] * kLog2e;
  // the student logits at the ids inside this piece, read before any store
  // of the piece (dZ may be Z)
#pragma unroll
  for (int j = 0; j < KPS; ++j) {
    if (tid + NT * j >= K) id[j] = -1;
    const bool in = id[j] >= c0 && id[j] < c1;
    z[j] = Elem<TE>::load(zr + (in ? id[j] : c0));
  }
  if (G > 1) load_group<NT>(B, gp + NT * kUnroll);
  const bool keep = __builtin_amdgcn_readfirstlane(idr[0]) != kIgnoreId;
  const float coef = keep ? scale : 0.f;  // an ignored row's gradient is zero
  if (keep) {
    // p = softmax over K of l / T over the whole workgroup
    __shared__ float s_red[NT / 64];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < KPS; ++j) mx = fmaxf(mx, tid + NT * j < K ? l[j] : kNegInf);
    mx = wave_max(mx);
    if (lane == 0) s_red[tid >> 6] = mx;
    __syncthreads();
    mx = s_red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) mx = fmaxf(mx, s_red[w]);
    float se = 0.f;
#pragma unroll
    for (int j = 0; j < KPS; ++j)
      if (tid + NT * j < K) se += exp2_hw((l[j] - mx) * kLog2e);
    se = wave_sum(se);
    __syncthreads();  // every wavefront has read the maxima
    if (lane == 0) s_red[tid >> 6] = se;
    __syncthreads();
    se = s_red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) se += s_red[w];
    const float lt = mx + log2_hw(se) * kLn2;
#pragma unroll
    for (int j = 0; j < KPS; ++j) {
      s_id[tid + NT * j] = id[j];
      s_p[tid + NT * j] = tid + NT * j < K ? exp2_hw((l[j] - lt) * kLog2e) : 0.f;
      s_z[tid + NT * j] = z[j];
    }
  }
  // Every gather of the workgroup has completed before any store: each
  // thread waits for its own, then the barrier.
  __syncthreads();
  const float c = kLog2e * a.inv_T;
  auto dense = [&](const uint4& v) {
    float x[VEC];
    Elem<TE>::unpack(v, x);
#pragma unroll
    for (int j = 0; j < VEC; ++j) x[j] = coef * exp2_hw(__builtin_fmaf(x[j], c, -lse2));
    return Elem<TE>::pack(x);
  };
  auto write = [&](const uint4(&u)[kUnroll], int64_t g) {
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) store_stream(go + g * NT * kUnroll + NT * q, dense(u[q]));
  };
  // A holds group g and B group g + 1 (in flight) at the top of each step;
  // the loads in the loop are unconditional, so each wait covers only the
  // group about to be written
  int64_t g = 0;
  for (; g + 3 < G; g += 2) {
    write(A, g);
    load_group<NT>(A, gp + (g + 2) * NT * kUnroll);
    write(B, g + 1);
    load_group<NT>(B, gp + (g + 3) * NT * kUnroll);
  }
  if (g + 2 < G) {
    write(A, g);
    load_group<NT>(A, gp + (g + 2) * NT * kUnroll);
    write(B, g + 1);
    write(A, g + 2);
  } else if (g + 1 < G) {
    write(A, g);
    write(B, g + 1);
  } else if (g < G) {
    write(A, g);
  }
  for (int64_t i = v0 + G * NT * kUnroll + tid; i < v1; i += NT) store_stream(op + i, dense(load_stream(vp + i)));
  if (!keep) return;
  // Teacher entries of the piece: overwritten with the full value once every
  // wavefront's dense stores have been performed (same addresses, written
  // later). Repeated ids add their mass; the first entry of an id writes.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KPS; ++j) {
    const int k = tid + NT * j;
    const int idk = k < K ? s_id[k] : -1;
    if (idk < c0 || idk >= c1) continue;
    float mass = 0.f;
    bool first = true;
    for (int q = 0; q < K; ++q) {
      if (s_id[q] == idk) {
        mass += s_p[q];
        first = first && q >= k;
      }
    }
    if (first) Elem<TE>::store(dr + idk, coef * (exp2_hw(__builtin_fmaf(s_z[k], c, -lse2)) - mass));
  }
}

// ------------------------------ dense KL ------------------------------------
// The pages' dense baseline builds the full teacher probability grid from the
// cached top-K and compares it with the student's full log-probability grid
// [P1, section "Two system changes", dense KL bullet]; both grids are kept for
// the backward pass. Rows are 16-byte aligned (pitch ldv, a multiple of 8
// elements), so every pass streams whole vectors plus a scalar tail.

template <typename TE>
__global__ __launch_bounds__(64 * kRowsPerBlock) void dense_student_kernel(DenseArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.N) return;
  constexpr int VEC = Elem<TE>::kVec;
  const TE* zr = (const TE*)a.Z + row * a.ldv;
  float* lq = a.logq + row * a.ldv;
  const int64_t nvec = a.V / VEC;
  const int tail = (int)(a.V - nvec * VEC);
  const float c = kLog2e * a.inv_T;
  const uint4* vp = (const uint4*)zr;
  OnlineLse acc(c);
  for (int64_t i = lane; i < nvec; i += 64) {
    float x[VEC];
    Elem<TE>::unpack(load_stream(vp + i), x);
    acc.add_vec(x);
  }
  if (lane < tail) acc.add(Elem<TE>::load(zr + nvec * VEC + lane));
  acc.wave_merge();
  const float lse = acc.lse();
  for (int64_t i = lane; i < nvec; i += 64) {
    float x[VEC];
    Elem<TE>::unpack(load_stream(vp + i), x);
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q)
      store_stream((uint4*)(lq + i * VEC) + q,
                   make_uint4(__builtin_bit_cast(uint32_t, x[4 * q] * a.inv_T - lse),
                              __builtin_bit_cast(uint32_t, x[4 * q + 1] * a.inv_T - lse),
                              __builtin_bit_cast(uint32_t, x[4 * q + 2] * a.inv_T - lse),
                              __builtin_bit_cast(uint32_t, x[4 * q + 3] * a.inv_T - lse)));
  }
  if (lane < tail) lq[nvec * VEC + lane] = Elem<TE>::load(zr + nvec * VEC + lane) * a.inv_T - lse;
  if (lane == 0) a.row_lse[row] = lse;
}

template <int KPL>
__global__ __launch_bounds__(64 * kRowsPerBlock) void dense_teacher_kernel(DenseArgs a) {
  __shared__ int32_t s_id[kRowsPerBlock][64 * KPL];
  __shared__ float s_p[kRowsPerBlock][64 * KPL];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + w;
  if (row >= a.N) return;
  LogitsArgs la;
  la.Z = nullptr; la.ids = a.ids; la.logits = a.logits; la.V = a.V; la.K = a.K; la.inv_T = a.inv_T;
  TeacherRow<float, KPL> t;
  t.load(la, row, lane, false);
  const bool keep = a.ids[row * a.K] != kIgnoreId;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int k = lane + 64 * j;
    if (k < a.K) {
      s_id[w][k] = t.id[j];
      s_p[w][k] = t.p[j];
    }
  }
  __builtin_amdgcn_wave_barrier();
  float* pr = a.P + row * a.ldv;
  const int64_t nvec = a.V / 4;
  for (int64_t i = lane; i < nvec; i += 64) store_stream((uint4*)pr + i, make_uint4(0u, 0u, 0u, 0u));
  if (lane < (int)(a.V - nvec * 4)) pr[nvec * 4 + lane] = 0.f;
  // teacher entries after the zeros of this wavefront have been performed
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    if (keep && lane + 64 * j < a.K && t.ok[j]) {
      float mass = 0.f;  // duplicates of an id add their mass
      for (int q = 0; q < a.K; ++q) mass += s_id[w][q] == t.id[j] ? s_p[w][q] : 0.f;
      pr[t.id[j]] = mass;
    }
  }
}

__global__ __launch_bounds__(64 * kRowsPerBlock) void dense_kl_kernel(DenseArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.N) return;
  const float* pr = a.P + row * a.ldv;
  const float* lq = a.logq + row * a.ldv;
  const int64_t nvec = a.V / 4;
  auto term = [](float p, float l) { return p > 0.f ? p * (log2_hw(p) * kLn2 - l) : 0.f; };
  float kl = 0.f;
  for (int64_t i = lane; i < nvec; i += 64) {
    const uint4 pu = load_stream((const uint4*)pr + i), lu = load_stream((const uint4*)lq + i);
    kl += term(__builtin_bit_cast(float, pu.x), __builtin_bit_cast(float, lu.x)) +
          term(__builtin_bit_cast(float, pu.y), __builtin_bit_cast(float, lu.y)) +
          term(__builtin_bit_cast(float, pu.z), __builtin_bit_cast(float, lu.z)) +
          term(__builtin_bit_cast(float, pu.w), __builtin_bit_cast(float, lu.w));
  }
  if (lane < (int)(a.V - nvec * 4)) kl += term(pr[nvec * 4 + lane], lq[nvec * 4 + lane]);
  kl = wave_sum(kl);
  if (lane == 0) a.row_kl[row] = kl;  // an ignored row's P is zero, so its KL is 0
}

template <typename TE>
__global__ __launch_bounds__(64 * kRowsPerBlock) void dense_grad_kernel(DenseArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows_pad) return;
  constexpr int VEC = Elem<TE>::kVec;
  uint4* out = (uint4*)((TE*)a.dZ + row * a.ldv);
  const int64_t nvec = a.ldv / VEC;  // whole row including the zero padding
  if (row >= a.N) {
    for (int64_t i = lane; i < nvec; i += 64) store_stream(out + i, make_uint4(0u, 0u, 0u, 0u));
    return;
  }
  const bool keep = a.ids[row * a.K] != kIgnoreId;
  const float coef = keep ? a.scale[0] : 0.f;
  const uint4* pr = (const uint4*)(a.P + row * a.ldv);
  const uint4* lq = (const uint4*)(a.logq + row * a.ldv);
  for (int64_t i = lane; i < nvec; i += 64) {
    float y[VEC];
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const uint4 pu = load_stream(pr + i * (VEC / 4) + q), lu = load_stream(lq + i * (VEC / 4) + q);
      const float pv[4] = {__builtin_bit_cast(float, pu.x), __builtin_bit_cast(float, pu.y),
                           __builtin_bit_cast(float, pu.z), __builtin_bit_cast(float, pu.w)};
      const float lv[4] = {__builtin_bit_cast(float, lu.x), __builtin_bit_cast(float, lu.y),
                           __builtin_bit_cast(float, lu.z), __builtin_bit_cast(float, lu.w)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t v = i * VEC + 4 * q + j;
        y[4 * q + j] = v < a.V ? coef * (exp2_hw(lv[j] * kLog2e) - pv[j]) : 0.f;
      }
    }
    store_stream(out + i, Elem<TE>::pack(y));
  }
}

}  // namespace

// Slots per lane for the teacher entries: the smallest of 2, 4, 16 with
// K <= 64 * slots.
template <template <typename, int> class Launch, typename TE>
static hipError_t launch_k(const LogitsArgs& a, hipStream_t s) {
  if (a.K <= 128) return Launch<TE, 2>::go(a, s);
  if (a.K <= 256) return Launch<TE, 4>::go(a, s);
  return Launch<TE, 16>::go(a, s);
}

template <typename TE, int KPL>
struct FwdLaunch {
  static hipError_t go(const LogitsArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + kRowsPerBlock - 1) / kRowsPerBlock));
    hipLaunchKernelGGL((logits_fwd_kernel<TE, KPL>), grid, dim3(64 * kRowsPerBlock), 0, s, a);
    return hipGetLastError();
  }
};

template <typename TE, int KPL>
struct BwdLaunch {
  static hipError_t go(const LogitsArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((a.N + kRowsPerBlock - 1) / kRowsPerBlock));
    hipLaunchKernelGGL((logits_bwd_kernel<TE, KPL>), grid, dim3(64 * kRowsPerBlock), 0, s, a);
    return hipGetLastError();
  }
};

hipError_t launch_logits_fwd(int dtype, const LogitsArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if (a.K < 1 || a.K > 1024) return hipErrorInvalidValue;
  return dtype == 1 ? launch_k<FwdLaunch, uint16_t>(a, s) : launch_k<FwdLaunch, float>(a, s);
}

template <typename TE>
static hipError_t launch_bwd(const LogitsArgs& a, hipStream_t s) {
  constexpr int64_t VEC = Elem<TE>::kVec;
  const int64_t nvec = a.V / VEC;
  if (a.V % VEC == 0 && nvec >= kPieceMinVec) {
    const int64_t pieces = (nvec + kPieceVec - 1) / kPieceVec;
    const int64_t len = (nvec + pieces - 1) / pieces;
    if (a.N * pieces <= INT32_MAX) {
      const dim3 grid((unsigned)(a.N * pieces)), block(kPieceThreads);
      if (a.K <= kPieceThreads)
        hipLaunchKernelGGL((logits_bwd_piece_kernel<TE, 1>), grid, block, 0, s, a, (int)pieces, len);
      else if (a.K <= 2 * kPieceThreads)
        hipLaunchKernelGGL((logits_bwd_piece_kernel<TE, 2>), grid, block, 0, s, a, (int)pieces, len);
      else
        hipLaunchKernelGGL((logits_bwd_piece_kernel<TE, 4>), grid, block, 0, s, a, (int)pieces, len);
      return hipGetLastError();
    }
  }
  return launch_k<BwdLaunch, TE>(a, s);
}

hipError_t launch_logits_bwd(int dtype, const LogitsArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if (a.K < 1 || a.K > 1024) return hipErrorInvalidValue;
  return dtype == 1 ? launch_bwd<uint16_t>(a, s) : launch_bwd<float>(a, s);
}

static dim3 dense_grid(int64_t rows) { return dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)); }

hipError_t launch_dense_student(int dtype, const DenseArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if (a.ldv % 8 != 0) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(dense_student_kernel<uint16_t>, dense_grid(a.N), dim3(64 * kRowsPerBlock), 0, s, a);
  else
    hipLaunchKernelGGL(dense_student_kernel<float>, dense_grid(a.N), dim3(64 * kRowsPerBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_teacher(const DenseArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if (a.K < 1 || a.K > 1024 || a.ldv % 8 != 0) return hipErrorInvalidValue;
  const dim3 g = dense_grid(a.N), b(64 * kRowsPerBlock);
  if (a.K <= 128)
    hipLaunchKernelGGL(dense_teacher_kernel<2>, g, b, 0, s, a);
  else if (a.K <= 256)
    hipLaunchKernelGGL(dense_teacher_kernel<4>, g, b, 0, s, a);
  else
    hipLaunchKernelGGL(dense_teacher_kernel<16>, g, b, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_kl(const DenseArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  if (a.ldv % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dense_kl_kernel, dense_grid(a.N), dim3(64 * kRowsPerBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_grad(int dtype, const DenseArgs& a, hipStream_t s) {
  if (a.rows_pad <= 0) return hipSuccess;
  if (a.ldv % 8 != 0 || a.rows_pad < a.N) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(dense_grad_kernel<uint16_t>, dense_grid(a.rows_pad), dim3(64 * kRowsPerBlock), 0, s, a);
  else
    hipLaunchKernelGGL(dense_grad_kernel<float>, dense_grid(a.rows_pad), dim3(64 * kRowsPerBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace kdkl
