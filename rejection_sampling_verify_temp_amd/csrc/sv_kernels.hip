// HIP kernels of the speculative-sampling verify step for gfx950 (CDNA4).
//
// One step is four launches on the caller's stream:
//   1. row_stats   streams every needed logits row once, split into
//                  vocabulary chunks: per chunk the max and the sum of
//                  exp2(l * c + ref) (sampling rows) or the max and its lowest
//                  index (greedy rows).  HBM-bound; this is the hot loop.
//   2. decide      one wavefront per request, one lane per drafted position:
//                  combines the chunk partials, draws the Philox uniforms,
//                  forms p(x)/q(x) in fp64, ballots the accept bits and takes
//                  the first rejection with a count-trailing-zeros.
//   3. resid_sums  for requests rejected on a probabilistic draft: per chunk
//                  the sum of max(0, p - q) over the rejected row pair.
//   4. locate      one workgroup per sampling request: prefix over the chunk
//                  sums, then an LDS scan of the one chunk holding u * S.
//
// Method (page title, section): "深入推测解码：从概念到实现" 保证原始分布
// (accept with min(1, p/q), resample from max(0, p - q)); "RTP-LLM
// Speculative Engine 深度解析" 拒绝采样算法 (uniform vs p/q per position,
// stop at the first rejection); "投机采样" 投机解码算法 steps 3-5 (accepted
// count, adjusted law, extra token from the last target row).
#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_internal.h"

namespace sv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; tiny results flush to 0
}

// Sampling iff T is a positive, normal, finite float (NaN compares false).
__device__ __forceinline__ bool is_sampling(float T) {
  return T >= FLT_MIN && T <= FLT_MAX;
}

// c = log2(e) / T, rounded once to float; every exponent in the step is
// l * c + ref with this c.
__device__ __forceinline__ float temp_scale(float T) {
  return (float)(1.4426950408889634074 / (double)T);
}

// Exponent reference of a block whose maximum is m.
__device__ __forceinline__ float ref_of(float m, float c) { return -(m * c); }

__device__ __forceinline__ int clamp_drafts(int n, int K) {
  return n < 0 ? 0 : (n > K ? K : n);
}

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 64x64->128 multiplies; the key is bumped by the two Weyl constants after
// every round.
__device__ void philox4x64_10(uint64_t ctr[4], uint64_t k0, uint64_t k1) {
  const uint64_t kMul0 = 0xD2E7470EE14C6C93ull, kMul1 = 0xCA5A826395121157ull;
  const uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull, kWeyl1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kMul0, ctr[0]), lo0 = kMul0 * ctr[0];
    const uint64_t hi1 = __umul64hi(kMul1, ctr[2]), lo1 = kMul1 * ctr[2];
    const uint64_t n0 = hi1 ^ ctr[1] ^ k0, n2 = hi0 ^ ctr[3] ^ k1;
    ctr[0] = n0;
    ctr[1] = lo1;
    ctr[2] = n2;
    ctr[3] = lo0;
    k0 += kWeyl0;
    k1 += kWeyl1;
  }
}

// Uniforms of request b at position j: word 0 accepts, word 1 draws.
__device__ void uniforms(uint64_t seed, uint64_t offset, int b, int j,
                         double* u_acc, double* u_rec) {
  uint64_t ctr[4] = {offset, (uint64_t)b, (uint64_t)j, 0};
  philox4x64_10(ctr, seed, 0);
  *u_acc = (double)(ctr[0] >> 40) * 0x1p-24;
  *u_rec = (double)(ctr[1] >> 40) * 0x1p-24;
}

// ---------------------------------------------------------------------------
// Element formats
// ---------------------------------------------------------------------------
template <int DT>
struct Elt;

template <>
struct Elt<SV_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ static float at(const void* row, int i) {
    return static_cast<const float*>(row)[i];
  }
  __device__ static void unpack(const u32x4 d, float* x) {
    x[0] = __uint_as_float(d.x);
    x[1] = __uint_as_float(d.y);
    x[2] = __uint_as_float(d.z);
    x[3] = __uint_as_float(d.w);
  }
  __device__ static u32x4 neg_inf() {
    return u32x4{0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
  }
};

template <>
struct Elt<SV_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kVec = 8;
  __device__ static float at(const void* row, int i) {
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(row)[i] << 16);
  }
  // bf16 is the top half of a float: low half-word <<16, high half masked.
  __device__ static void unpack(const u32x4 d, float* x) {
    x[0] = __uint_as_float(d.x << 16);
    x[1] = __uint_as_float(d.x & 0xffff0000u);
    x[2] = __uint_as_float(d.y << 16);
    x[3] = __uint_as_float(d.y & 0xffff0000u);
    x[4] = __uint_as_float(d.z << 16);
    x[5] = __uint_as_float(d.z & 0xffff0000u);
    x[6] = __uint_as_float(d.w << 16);
    x[7] = __uint_as_float(d.w & 0xffff0000u);
  }
  __device__ static u32x4 neg_inf() {
    return u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
  }
};

__device__ __forceinline__ const void* row_ptr(const void* base, int dt,
                                               size_t row, int V) {
  const size_t bytes = dt == SV_BF16 ? 2 : 4;
  return static_cast<const char*>(base) + row * (size_t)V * bytes;
}

__device__ __forceinline__ float load_elem(const void* base, int dt,
                                           size_t row, int V, int i) {
  const void* r = row_ptr(base, dt, row, V);
  return dt == SV_BF16 ? Elt<SV_BF16>::at(r, i) : Elt<SV_F32>::at(r, i);
}

// Chunk [c0, c1) of a row = scalar head [c0, v0) up to the first 16-byte
// boundary, 16-byte vectors [v0, t0), scalar tail [t0, c1).
struct Geo {
  int c0, c1, v0, nvec, t0;
};

template <int DT>
__device__ __forceinline__ Geo chunk_geo(const void* row, int c0, int c1) {
  Geo g;
  g.c0 = c0;
  g.c1 = c1;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row) + (uintptr_t)c0 * Elt<DT>::kBytes;
  int head = (int)(((16u - (unsigned)(a & 15u)) & 15u) / Elt<DT>::kBytes);
  head = head < (c1 - c0) ? head : (c1 - c0);
  g.v0 = c0 + head;
  g.nvec = (c1 - g.v0) / Elt<DT>::kVec;
  g.t0 = g.v0 + g.nvec * Elt<DT>::kVec;
  return g;
}

// ---------------------------------------------------------------------------
// Per-thread accumulators
// ---------------------------------------------------------------------------
// Online softmax statistics: S = sum exp2(l * c + R) over the thread's
// elements, R = ref_of(M, c), M the running max.  The reference is moved
// only when the max grows, and the exponent reference stays an exact float
// so the chunk combine can rescale without bias.
struct SmAcc {
  float M, R, S;
};

template <int N>
__device__ __forceinline__ float pairwise_sum(float (&e)[N]) {
#pragma unroll
  for (int stride = 1; stride < N; stride *= 2) {
#pragma unroll
    for (int i = 0; i + stride < N; i += 2 * stride) e[i] += e[i + stride];
  }
  return e[0];
}

template <int N>
__device__ __forceinline__ void sm_tile(SmAcc& a, const float (&x)[N], float c) {
  float t = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) t = fmaxf(t, x[i]);
  if (t > a.M) {
    const float rn = ref_of(t, c);
    a.S = (a.M == kNegInf) ? 0.f : a.S * fast_exp2(rn - a.R);
    a.R = rn;
    a.M = t;
  }
  float e[N];
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = fast_exp2(fmaf(x[i], c, a.R));
  a.S += pairwise_sum(e);
}

// Running max and the lowest index attaining it (elements are visited in
// increasing index order per thread).
struct AmAcc {
  float M;
  int I;
};

template <int N>
__device__ __forceinline__ void am_tile(AmAcc& a, const float (&x)[N],
                                        const int (&idx)[N]) {
  float t = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) t = fmaxf(t, x[i]);
  if (t > a.M || (t == a.M && a.I == INT32_MAX)) {
    int best = INT32_MAX;
#pragma unroll
    for (int i = N - 1; i >= 0; --i)
      if (x[i] == t) best = idx[i];
    a.M = t;
    a.I = best;
  }
}

// ---------------------------------------------------------------------------
// Wavefront / workgroup reductions (fixed butterfly order: every lane ends
// with the same bits, results are reproducible run to run)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void wave_argmax(float& m, int& i) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float om = __shfl_xor(m, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (om > m || (om == m && oi < i)) {
      m = om;
      i = oi;
    }
  }
}

template <int NT>
__device__ float block_max(float v, float* lds) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) lds[w] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k) r = fmaxf(r, lds[k]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ double block_sum(double v, double* lds) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) lds[w] = v;
  __syncthreads();
  double r = lds[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k) r += lds[k];
  __syncthreads();
  return r;
}

template <int NT>
__device__ void block_argmax(float& m, int& i, float* ldsm, int* ldsi) {
  wave_argmax(m, i);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    ldsm[w] = m;
    ldsi[w] = i;
  }
  __syncthreads();
  m = ldsm[0];
  i = ldsi[0];
#pragma unroll
  for (int k = 1; k < NT / 64; ++k)
    if (ldsm[k] > m || (ldsm[k] == m && ldsi[k] < i)) {
      m = ldsm[k];
      i = ldsi[k];
    }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Chunk streaming
// ---------------------------------------------------------------------------
constexpr int kUnroll = 4;  // 16-byte loads in flight per thread per step

template <int DT>
__device__ __forceinline__ SmAcc chunk_softmax_stats(const void* row, int c0, int c1, float c) {
  using E = Elt<DT>;
  constexpr int kN = kUnroll * E::kVec;
  SmAcc a{kNegInf, 0.f, 0.f};
  const Geo g = chunk_geo<DT>(row, c0, c1);
  const int tid = threadIdx.x;
  if (g.c0 + tid < g.v0) {  // head (< one vector)
    const float x[1] = {E::at(row, g.c0 + tid)};
    sm_tile(a, x, c);
  }
  const u32x4* vp = reinterpret_cast<const u32x4*>(
      static_cast<const char*>(row) + (size_t)g.v0 * E::kBytes);
  for (int v = tid; v < g.nvec; v += kStatsThreads * kUnroll) {
    u32x4 d[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int vi = v + u * kStatsThreads;
      d[u] = vi < g.nvec ? __builtin_nontemporal_load(vp + vi) : E::neg_inf();
    }
    float x[kN];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) E::unpack(d[u], x + u * E::kVec);
    sm_tile(a, x, c);
  }
  if (g.t0 + tid < g.c1) {  // tail (< one vector)
    const float x[1] = {E::at(row, g.t0 + tid)};
    sm_tile(a, x, c);
  }
  return a;
}

template <int DT>
__device__ __forceinline__ AmAcc chunk_argmax(const void* row, int c0, int c1) {
  using E = Elt<DT>;
  constexpr int kN = kUnroll * E::kVec;
  AmAcc a{kNegInf, INT32_MAX};
  const Geo g = chunk_geo<DT>(row, c0, c1);
  const int tid = threadIdx.x;
  if (g.c0 + tid < g.v0) {
    const float x[1] = {E::at(row, g.c0 + tid)};
    const int ix[1] = {g.c0 + tid};
    am_tile(a, x, ix);
  }
  const u32x4* vp = reinterpret_cast<const u32x4*>(
      static_cast<const char*>(row) + (size_t)g.v0 * E::kBytes);
  for (int v = tid; v < g.nvec; v += kStatsThreads * kUnroll) {
    u32x4 d[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int vi = v + u * kStatsThreads;
      d[u] = vi < g.nvec ? __builtin_nontemporal_load(vp + vi) : E::neg_inf();
    }
    float x[kN];
    int ix[kN];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      E::unpack(d[u], x + u * E::kVec);
      const int vi = v + u * kStatsThreads;
#pragma unroll
      for (int e = 0; e < E::kVec; ++e)
        ix[u * E::kVec + e] = vi < g.nvec ? g.v0 + vi * E::kVec + e : INT32_MAX;
    }
    am_tile(a, x, ix);
  }
  if (g.t0 + tid < g.c1) {
    const float x[1] = {E::at(row, g.t0 + tid)};
    const int ix[1] = {g.t0 + tid};
    am_tile(a, x, ix);
  }
  return a;
}

// Reduce a workgroup's softmax accumulators to (chunk max, chunk sum relative
// to ref_of(chunk max)).  The rescale of each thread's sum is exact in fp64
// up to the final rounding of exp2.
__device__ __forceinline__ void reduce_softmax(const SmAcc& a, float c, float* ldsf, double* ldsd,
                               float* m_out, double* z_out) {
  const float m = block_max<kStatsThreads>(a.M, ldsf);
  double contrib = 0.0;
  if (a.S != 0.f && m != kNegInf)
    contrib = (double)a.S * exp2((double)ref_of(m, c) - (double)a.R);
  const double z = block_sum<kStatsThreads>(contrib, ldsd);
  *m_out = m;
  *z_out = z;
}

// Which rows a request needs.  Slots 0..K are target rows j = slot, slots
// K+1..2K are draft rows j = slot - K - 1.
struct ReqInfo {
  int n;
  float T;
  bool sampling;
  bool onehot;
};

__device__ __forceinline__ ReqInfo req_info(const RunParams& p, int b) {
  ReqInfo r;
  r.n = clamp_drafts(p.nd[b], p.K);
  r.T = p.temps[b];
  r.sampling = is_sampling(r.T);
  r.onehot = !p.has_draft || (p.mode != nullptr && p.mode[b] != 0);
  return r;
}

// ---------------------------------------------------------------------------
// Kernel 1: row statistics
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void row_stats_body(const void* row, int c0, int c1, const ReqInfo& ri,
                               Partial* out) {
  __shared__ float ldsf[kStatsThreads / 64];
  __shared__ double ldsd[kStatsThreads / 64];
  __shared__ int ldsi[kStatsThreads / 64];
  Partial r;
  if (ri.sampling) {
    const float c = temp_scale(ri.T);
    const SmAcc a = chunk_softmax_stats<DT>(row, c0, c1, c);
    reduce_softmax(a, c, ldsf, ldsd, &r.m, &r.z);
    r.idx = -1;
  } else {
    AmAcc a = chunk_argmax<DT>(row, c0, c1);
    block_argmax<kStatsThreads>(a.M, a.I, ldsf, ldsi);
    r.m = a.M;
    r.idx = a.I == INT32_MAX ? c0 : a.I;
    r.z = 0.0;
  }
  if (threadIdx.x == 0) *out = r;
}

template <int TDT, int DDT>
__global__ __launch_bounds__(kStatsThreads) void k_row_stats(const RunParams p) {
  const int nslot = 2 * p.K + 1;
  const int bid = blockIdx.x;
  const int row = bid / p.nchunk, chunk = bid - row * p.nchunk;
  const int b = row / nslot, s = row - b * nslot;
  const ReqInfo ri = req_info(p, b);
  const int c0 = chunk * p.chunk;
  const int c1 = min(p.V, c0 + p.chunk);
  Partial* out = p.part + (size_t)row * p.nchunk + chunk;
  if (s <= p.K) {
    if (s > ri.n) return;
    const void* r = row_ptr(p.target, TDT, (size_t)b * (p.K + 1) + s, p.V);
    row_stats_body<TDT>(r, c0, c1, ri, out);
  } else {
    const int j = s - p.K - 1;
    if (j >= ri.n || !ri.sampling || ri.onehot || p.draft_is_probs) return;
    const void* r = row_ptr(p.draft, DDT, (size_t)b * p.K + j, p.V);
    row_stats_body<DDT>(r, c0, c1, ri, out);
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: decisions
// ---------------------------------------------------------------------------
// Combine the chunk partials of a sampling row: reference of the row max and
// the row total relative to it.
__device__ void combine_softmax(const Partial* part, int nchunk, float c,
                                float* ref_out, double* z_out) {
  float m = kNegInf;
  for (int k = 0; k < nchunk; ++k) m = fmaxf(m, part[k].m);
  const float ref = ref_of(m, c);
  double z = 0.0;
  for (int k = 0; k < nchunk; ++k)
    if (part[k].z != 0.0)
      z += part[k].z * exp2((double)ref - (double)ref_of(part[k].m, c));
  *ref_out = ref;
  *z_out = z;
}

// Greedy row: max and lowest index attaining it (chunks are in index order).
__device__ void combine_argmax(const Partial* part, int nchunk, float* m_out,
                               int* i_out) {
  float m = part[0].m;
  int i = part[0].idx;
  for (int k = 1; k < nchunk; ++k)
    if (part[k].m > m) {
      m = part[k].m;
      i = part[k].idx;
    }
  *m_out = m;
  *i_out = i;
}

__device__ __forceinline__ double prob_of(float l, float c, float ref, double z) {
  return exp2((double)l * (double)c + (double)ref) / z;
}

template <int TDT, int DDT>
__global__ __launch_bounds__(kDecideThreads) void k_decide(const RunParams p) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int K = p.K, V = p.V, nslot = 2 * K + 1;
  const int nraw = p.nd[b];
  const ReqInfo ri = req_info(p, b);
  const int n = ri.n;
  if (lane == 0 && nraw != n) atomicOr(p.flags, SV_DEVERR_BAD_NUM_DRAFTS);
  const float c = ri.sampling ? temp_scale(ri.T) : 0.f;
  const Partial* part_b = p.part + (size_t)b * nslot * p.nchunk;

  // Decision of position j = lane.
  const int j = lane;
  bool accept = false;
  float dbg_p = __builtin_nanf(""), dbg_q = __builtin_nanf("");
  if (j < n) {
    const int x = p.ids[(size_t)b * K + j];
    const bool valid = x >= 0 && x < V;
    if (!valid) atomicOr(p.flags, SV_DEVERR_BAD_DRAFT_ID);
    const Partial* pt = part_b + (size_t)j * p.nchunk;
    const size_t trow = (size_t)b * (K + 1) + j;
    if (!ri.sampling) {
      float m;
      int im;
      combine_argmax(pt, p.nchunk, &m, &im);
      accept = valid && load_elem(p.target, TDT, trow, V, x) == m;
    } else {
      float ref_p;
      double z_p;
      combine_softmax(pt, p.nchunk, c, &ref_p, &z_p);
      const double px = valid ? prob_of(load_elem(p.target, TDT, trow, V, x), c, ref_p, z_p) : 0.0;
      double qx = 1.0;
      if (!ri.onehot) {
        const size_t drow = (size_t)b * K + j;
        if (p.draft_is_probs) {
          qx = valid ? (double)load_elem(p.draft, DDT, drow, V, x) : 0.0;
        } else {
          float ref_q;
          double z_q;
          combine_softmax(part_b + (size_t)(K + 1 + j) * p.nchunk, p.nchunk, c, &ref_q, &z_q);
          qx = valid ? prob_of(load_elem(p.draft, DDT, drow, V, x), c, ref_q, z_q) : 0.0;
        }
      }
      double ratio;
      if (!valid) ratio = 0.0;
      else if (qx > 0.0) ratio = px / qx;
      else ratio = px > 0.0 ? __builtin_inf() : 0.0;
      double u_acc, u_rec;
      uniforms(p.seed, p.offset, b, j, &u_acc, &u_rec);
      accept = u_acc < ratio;
      dbg_p = valid ? (float)px : dbg_p;
      dbg_q = valid ? (float)qx : dbg_q;
    }
  }
  // First rejection: lanes >= n vote false, so ~mask has a bit at n or below.
  const uint64_t mask = __ballot(accept);
  const int first_rej = (int)__builtin_ctzll(~mask);
  const int n_acc = first_rej < n ? first_rej : n;

  // Outputs other than the emitted token.
  if (lane <= K && lane != n_acc) {
    const int32_t tok = lane < n_acc ? p.ids[(size_t)b * K + lane] : -1;
    p.out_tokens[(size_t)b * (K + 1) + lane] = tok;
  }
  if (lane == 0) p.out_nacc[b] = n_acc;
  if (p.out_dbg != nullptr && lane < K) {
    p.out_dbg[((size_t)b * K + lane) * 2 + 0] = dbg_p;
    p.out_dbg[((size_t)b * K + lane) * 2 + 1] = dbg_q;
  }

  // The emitted position: greedy writes its argmax now, sampling requests
  // leave a draw descriptor for the locate kernel.
  if (lane == n_acc) {
    const int je = n_acc;
    const Partial* pt = part_b + (size_t)je * p.nchunk;
    DrawDesc d{};
    d.j = je;
    d.x = -1;
    if (!ri.sampling) {
      float m;
      int im;
      combine_argmax(pt, p.nchunk, &m, &im);
      p.out_tokens[(size_t)b * (K + 1) + je] = im;
      d.kind = kDrawNone;
    } else {
      d.c = c;
      combine_softmax(pt, p.nchunk, c, &d.ref_p, &d.z_p);
      double u_acc, u_rec;
      uniforms(p.seed, p.offset, b, je, &u_acc, &u_rec);
      d.u = u_rec;
      d.kind = kDrawSingle;
      if (je < n) {  // rejected at je
        const int x = p.ids[(size_t)b * K + je];
        d.x = (x >= 0 && x < V) ? x : -1;
        if (!ri.onehot) {
          d.kind = kDrawPair;
          double kap;
          if (p.draft_is_probs) {
            d.ref_q = 0.f;
            kap = d.z_p;  // p - q = (p~ - Z_p q) / Z_p
          } else {
            double z_q;
            combine_softmax(part_b + (size_t)(K + 1 + je) * p.nchunk, p.nchunk, c, &d.ref_q, &z_q);
            kap = d.z_p / z_q;  // p - q = (p~ - (Z_p / Z_q) q~) / Z_p
          }
          d.kap_hi = (float)kap;
          d.kap_lo = (float)(kap - (double)d.kap_hi);
        }
      }
    }
    p.desc[b] = d;
  }
}

// ---------------------------------------------------------------------------
// Residual elements (unnormalized, relative to the draw descriptor)
// ---------------------------------------------------------------------------
// Pair: r~ = max(0, p~ - kappa q~) with p~ = exp2(l_p c + ref_p) and q~ =
// exp2(l_q c + ref_q) (or q itself for probability drafts); the split kappa
// keeps the difference accurate to the rounding of p~ and q~.
__device__ __forceinline__ float pair_resid(float lp, float lq, const DrawDesc& d,
                                            bool probs) {
  const float pt = fast_exp2(fmaf(lp, d.c, d.ref_p));
  const float qt = probs ? lq : fast_exp2(fmaf(lq, d.c, d.ref_q));
  float r = fmaf(-qt, d.kap_hi, pt);
  r = fmaf(-qt, d.kap_lo, r);
  return r > 0.f ? r : 0.f;
}

__device__ __forceinline__ float single_resid(float lp, const DrawDesc& d) {
  return fast_exp2(fmaf(lp, d.c, d.ref_p));
}

// ---------------------------------------------------------------------------
// Kernel 3: per-chunk sums of max(0, p - q) for rejected probabilistic drafts
// ---------------------------------------------------------------------------
template <int TDT, int DDT>
__global__ __launch_bounds__(kStatsThreads) void k_resid_sums(const RunParams p) {
  __shared__ double ldsd[kStatsThreads / 64];
  const int bid = blockIdx.x;
  const int b = bid / p.nchunk, chunk = bid - b * p.nchunk;
  const DrawDesc d = p.desc[b];
  if (d.kind != kDrawPair) return;
  const int K = p.K, V = p.V;
  const void* prow = row_ptr(p.target, TDT, (size_t)b * (K + 1) + d.j, V);
  const void* qrow = row_ptr(p.draft, DDT, (size_t)b * K + d.j, V);
  const bool probs = p.draft_is_probs != 0;
  const int c0 = chunk * p.chunk, c1 = min(V, c0 + p.chunk);
  const int tid = threadIdx.x;
  float acc = 0.f;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(prow) + (uintptr_t)c0 * Elt<TDT>::kBytes;
  const uintptr_t qa = reinterpret_cast<uintptr_t>(qrow) + (uintptr_t)c0 * Elt<DDT>::kBytes;
  const bool aligned = ((pa | qa) & 15u) == 0;
  int done = c0;
  if (aligned) {
    // groups of 8 elements: one or two 16-byte loads per row
    const int ngrp = (c1 - c0) / 8;
    for (int g = tid; g < ngrp; g += kStatsThreads) {
      const int i0 = c0 + g * 8;
      float lp[8], lq[8];
      if (TDT == SV_BF16) {
        Elt<SV_BF16>::unpack(__builtin_nontemporal_load(
                                 reinterpret_cast<const u32x4*>(static_cast<const char*>(prow) + (size_t)i0 * 2)),
                             lp);
      } else {
        const u32x4* v = reinterpret_cast<const u32x4*>(static_cast<const char*>(prow) + (size_t)i0 * 4);
        Elt<SV_F32>::unpack(__builtin_nontemporal_load(v), lp);
        Elt<SV_F32>::unpack(__builtin_nontemporal_load(v + 1), lp + 4);
      }
      if (DDT == SV_BF16) {
        Elt<SV_BF16>::unpack(__builtin_nontemporal_load(
                                 reinterpret_cast<const u32x4*>(static_cast<const char*>(qrow) + (size_t)i0 * 2)),
                             lq);
      } else {
        const u32x4* v = reinterpret_cast<const u32x4*>(static_cast<const char*>(qrow) + (size_t)i0 * 4);
        Elt<SV_F32>::unpack(__builtin_nontemporal_load(v), lq);
        Elt<SV_F32>::unpack(__builtin_nontemporal_load(v + 1), lq + 4);
      }
      float e[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = (i0 + k == d.x) ? 0.f : pair_resid(lp[k], lq[k], d, probs);
      acc += pairwise_sum(e);
    }
    done = c0 + ngrp * 8;
  }
  for (int i = done + tid; i < c1; i += kStatsThreads) {
    const float r = (i == d.x) ? 0.f
                               : pair_resid(Elt<TDT>::at(prow, i), Elt<DDT>::at(qrow, i), d, probs);
    acc += r;
  }
  const double s = block_sum<kStatsThreads>((double)acc, ldsd);
  if (tid == 0) p.rsum[(size_t)b * p.nchunk + chunk] = s;
}

// ---------------------------------------------------------------------------
// Kernel 4: inverse-CDF draw of the emitted token
// ---------------------------------------------------------------------------
// Sum of chunk k of the draw law, from the first-pass partials (single) or
// the residual sums (pair).
__device__ double chunk_mass(const RunParams& p, const DrawDesc& d, int b, int k,
                             int kind, double excl_mass, int excl_chunk) {
  if (kind == kDrawPair) return p.rsum[(size_t)b * p.nchunk + k];
  const Partial& q = p.part[((size_t)b * (2 * p.K + 1) + d.j) * p.nchunk + k];
  double s = 0.0;
  if (q.z != 0.0) s = q.z * exp2((double)d.ref_p - (double)ref_of(q.m, d.c));
  if (k == excl_chunk) s -= excl_mass;
  return s > 0.0 ? s : 0.0;
}

template <int TDT, int DDT>
__global__ __launch_bounds__(kLocateThreads) void k_locate(const RunParams p) {
  extern __shared__ float lds_r[];  // chunk residuals, then scan scratch
  __shared__ double sh_q[kLocateThreads + 1];
  __shared__ double sh_wave[kLocateThreads / 64];
  __shared__ int sh_cstar, sh_y, sh_last;
  __shared__ double sh_theta;
  __shared__ int sh_kind, sh_excl;

  const int b = blockIdx.x;
  const DrawDesc d = p.desc[b];
  if (d.kind == kDrawNone) return;
  const int K = p.K, V = p.V, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const size_t trow = (size_t)b * (K + 1) + d.j;
  const void* prow = row_ptr(p.target, TDT, trow, V);
  const void* qrow = d.kind == kDrawPair ? row_ptr(p.draft, DDT, (size_t)b * K + d.j, V) : nullptr;
  const bool probs = p.draft_is_probs != 0;

  // --- chunk selection (wavefront 0) ---
  if (w == 0) {
    int kind = d.kind;
    double excl_mass = 0.0;
    int excl_chunk = -1;
    if (kind == kDrawSingle && d.x >= 0) {
      excl_chunk = d.x / p.chunk;
      excl_mass = exp2((double)load_elem(p.target, TDT, trow, V, d.x) * (double)d.c + (double)d.ref_p);
    }
    for (int attempt = 0; attempt < 2; ++attempt) {
      const int per = (p.nchunk + 63) / 64;
      const int k0 = lane * per, k1 = min(p.nchunk, k0 + per);
      double tot = 0.0;
      for (int k = k0; k < k1; ++k) tot += chunk_mass(p, d, b, k, kind, excl_mass, excl_chunk);
      // inclusive scan of lane totals (Hillis-Steele, fixed order)
      double incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const double S = __shfl(incl, 63, 64);
      if (!(S > 0.0) && attempt == 0) {  // no residual mass: draw from p
        if (lane == 0) atomicOr(p.flags, SV_DEVERR_ZERO_RESIDUAL);
        kind = kDrawSingle;
        excl_chunk = -1;
        excl_mass = 0.0;
        continue;
      }
      const double theta = d.u * S;
      const double before = incl - tot;  // exclusive prefix of this lane
      int found = -1;
      double th = 0.0;
      if (before <= theta && tot > 0.0) {
        double acc = before;
        for (int k = k0; k < k1; ++k) {
          const double s = chunk_mass(p, d, b, k, kind, excl_mass, excl_chunk);
          if (s > 0.0 && acc + s > theta) {
            found = k;
            th = theta - acc;
            break;
          }
          acc += s;
        }
      }
      const uint64_t hit = __ballot(found >= 0);
      int src = hit ? (int)__builtin_ctzll(hit) : -1;
      int cstar;
      double thp;
      if (src >= 0) {
        cstar = __shfl(found, src, 64);
        thp = __shfl(th, src, 64);
      } else {
        // rounding left theta at or past the total: last chunk with mass
        int lastk = -1;
        for (int k = k1 - 1; k >= k0; --k)
          if (chunk_mass(p, d, b, k, kind, excl_mass, excl_chunk) > 0.0) {
            lastk = k;
            break;
          }
        const uint64_t has = __ballot(lastk >= 0);
        const int srcl = has ? 63 - (int)__builtin_clzll(has) : 0;
        cstar = __shfl(lastk, srcl, 64);
        thp = __builtin_inf();
        if (lane == 0) atomicOr(p.flags, SV_DEVERR_DRAW_ROUNDING);
      }
      if (lane == 0) {
        sh_cstar = cstar < 0 ? 0 : cstar;
        sh_theta = thp;
        sh_kind = kind;
        sh_excl = attempt == 0 ? d.x : -1;  // the fallback draws from p whole
      }
      break;
    }
    if (lane == 0) {
      sh_y = INT32_MAX;
      sh_last = -1;
    }
  }
  __syncthreads();

  // --- scan of the selected chunk ---
  const int kind = sh_kind;
  const int c0 = sh_cstar * p.chunk, c1 = min(V, c0 + p.chunk);
  const int len = c1 - c0;
  const int xr = sh_excl;
  for (int i = tid; i < len; i += kLocateThreads) {
    const int gi = c0 + i;
    float r;
    if (gi == xr) r = 0.f;
    else if (kind == kDrawPair) r = pair_resid(Elt<TDT>::at(prow, gi), Elt<DDT>::at(qrow, gi), d, probs);
    else r = single_resid(Elt<TDT>::at(prow, gi), d);
    lds_r[i] = r;
  }
  __syncthreads();
  const int per = (len + kLocateThreads - 1) / kLocateThreads;
  const int s0 = min(len, tid * per), s1 = min(len, s0 + per);
  double s = 0.0;
  int lastpos = -1;
  for (int i = s0; i < s1; ++i) {
    s += (double)lds_r[i];
    if (lds_r[i] > 0.f) lastpos = i;
  }
  // exclusive scan across the workgroup: wave scans + sequential wave offsets
  double incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sh_wave[w] = incl;
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    for (int k = 0; k < kLocateThreads / 64; ++k) {
      const double t = sh_wave[k];
      sh_wave[k] = acc;
      acc += t;
    }
    sh_q[kLocateThreads] = acc;
  }
  __syncthreads();
  const double q = sh_wave[w] + (incl - s);
  sh_q[tid] = q;
  if (lastpos >= 0) atomicMax(&sh_last, lastpos);
  __syncthreads();
  const double qn = sh_q[tid + 1];
  const double theta = sh_theta;
  if (s1 > s0 && q <= theta && theta < qn) {
    int y = -1, lp = -1;
    double L = 0.0;
    for (int i = s0; i < s1; ++i) {
      const float r = lds_r[i];
      L += (double)r;
      if (r > 0.f) lp = i;
      if (r > 0.f && q + L > theta) {
        y = i;
        break;
      }
    }
    if (y < 0) y = lp;  // rounding tie inside the segment
    if (y >= 0) atomicMin(&sh_y, y);
  }
  __syncthreads();
  if (tid == 0) {
    int y = sh_y;
    if (y == INT32_MAX) {  // theta past the recomputed chunk total
      y = sh_last >= 0 ? sh_last : 0;
      if (theta != __builtin_inf()) atomicOr(p.flags, SV_DEVERR_DRAW_ROUNDING);
    }
    p.out_tokens[(size_t)b * (K + 1) + d.j] = c0 + y;
  }
}

template <int TDT, int DDT>
hipError_t launch_all(const RunParams& p, hipStream_t s, hipEvent_t* ev) {
  const int nslot = 2 * p.K + 1;
  auto rec = [&](int k) -> hipError_t {
    return ev ? hipEventRecord(ev[k], s) : hipSuccess;
  };
  hipError_t e;
  if ((e = rec(0)) != hipSuccess) return e;
  const uint64_t g1 = (uint64_t)p.B * nslot * p.nchunk;
  hipLaunchKernelGGL((k_row_stats<TDT, DDT>), dim3((unsigned)g1), dim3(kStatsThreads), 0, s, p);
  if ((e = rec(1)) != hipSuccess) return e;
  if ((e = rec(2)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_decide<TDT, DDT>), dim3(p.B), dim3(kDecideThreads), 0, s, p);
  if ((e = rec(3)) != hipSuccess) return e;
  if ((e = rec(4)) != hipSuccess) return e;
  if (p.has_draft) {
    const uint64_t g3 = (uint64_t)p.B * p.nchunk;
    hipLaunchKernelGGL((k_resid_sums<TDT, DDT>), dim3((unsigned)g3), dim3(kStatsThreads), 0, s, p);
  }
  if ((e = rec(5)) != hipSuccess) return e;
  if ((e = rec(6)) != hipSuccess) return e;
  const size_t lds = (size_t)p.chunk * sizeof(float);
  hipLaunchKernelGGL((k_locate<TDT, DDT>), dim3(p.B), dim3(kLocateThreads), lds, s, p);
  if ((e = rec(7)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const RunParams& p, int tdt, int ddt, hipStream_t s,
                       hipEvent_t* ev) {
  if (tdt == SV_F32 && ddt == SV_F32) return launch_all<SV_F32, SV_F32>(p, s, ev);
  if (tdt == SV_F32 && ddt == SV_BF16) return launch_all<SV_F32, SV_BF16>(p, s, ev);
  if (tdt == SV_BF16 && ddt == SV_F32) return launch_all<SV_BF16, SV_F32>(p, s, ev);
  return launch_all<SV_BF16, SV_BF16>(p, s, ev);
}

const char* kernel_name(int i) {
  static const char* names[kNumKernels] = {"row_stats", "decide", "resid_sums", "locate"};
  return (i >= 0 && i < kNumKernels) ? names[i] : nullptr;
}

}  // namespace sv
