// Device helpers shared by the HIP sources of the library: the temperature
// scale and exponent references, Philox4x64-10 and the uniform layouts, the
// element formats (bf16 as the top half of a float), chunk geometry,
// buffer-resource loads, per-thread accumulators and the wavefront /
// workgroup reductions.  Each
// source that includes it gets its own internal copies.
#pragma once

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

// 2^(r - rw) for finite floats r <= rw, the factor that moves a sum of
// exponentials from reference rw to reference r: the difference is exact in
// double; its integer part goes to the exponent and v_exp_f32 takes the
// fraction, so the factor is as accurate as the element exponentials that
// the sum holds, at a fraction of a double exp2's cost.
__device__ __forceinline__ double exp2_diff(float r, float rw) {
  const double d = (double)r - (double)rw;
  const double n = floor(d);
  return ldexp((double)fast_exp2((float)(d - n)), (int)n);
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

// The draft sampler's uniform for row j of request b: word 0 of the block at
// counter (offset, b, j, 1); the verify step's counters have word 3 = 0.
[[maybe_unused]] __device__ double draft_uniform(uint64_t seed, uint64_t offset, int b, int j) {
  uint64_t ctr[4] = {offset, (uint64_t)b, (uint64_t)j, 1};
  philox4x64_10(ctr, seed, 0);
  return (double)(ctr[0] >> 40) * 0x1p-24;
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

// A run of 16-byte vectors as a buffer resource: base address and size in
// bytes.  The hardware checks each load's offset register against the size
// and returns 0 past it without touching memory, so a round of loads needs
// no branches, and one offset register per load replaces a 64-bit address.
// (The scalar offset operand is not checked: offsets go in the register.)
// The base is the same for the whole workgroup; readfirstlane states it.
struct VecBuf {
  __amdgpu_buffer_rsrc_t r;
};

__device__ __forceinline__ VecBuf make_vec_buf(const void* base16, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base16);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  // word 3: 32-bit data format, as the gfx9 family takes for raw loads
  return VecBuf{__builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000)};
}

// The vector at byte offset off, or 0 past the end; NT marks it nontemporal
// (read once: streamed past the caches).
template <bool NT>
__device__ __forceinline__ u32x4 buf_load(const VecBuf& b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0u, NT ? 2 : 0);
}

// ---------------------------------------------------------------------------
// Per-thread accumulators
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ float pairwise_sum(float (&e)[N]) {
#pragma unroll
  for (int stride = 1; stride < N; stride *= 2) {
#pragma unroll
    for (int i = 0; i + stride < N; i += 2 * stride) e[i] += e[i + stride];
  }
  return e[0];
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
// Wavefront max and sum by DPP lane moves, which stay in the register file
// (a few cycles each) where a shuffle goes through the LDS crossbar: row_shr
// 1, 2, 4 and 8 leave each 16-lane row's total in its lane 15; row_bcast:15
// adds row 0's into row 1 and row 2's into row 3; row_bcast:31 adds lane
// 31's into rows 2 and 3; lane 63 then holds the total, read back for every
// lane.  A lane whose source is out of range keeps a neutral value.  The
// whole wavefront must be active.
template <int CTRL, int ROWS, int BANKS = 0xf>
__device__ __forceinline__ int dpp_move(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, BANKS, false);
}

// A double moved by DPP, 0 where the lane is masked or its source is out of
// range.
template <int CTRL, int ROWS, int BANKS = 0xf>
__device__ __forceinline__ double dpp_move_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)dpp_move<CTRL, ROWS, BANKS>(0, (int)(uint32_t)b);
  const uint32_t hi = (uint32_t)dpp_move<CTRL, ROWS, BANKS>(0, (int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v) {
  const int b = __float_as_int(v);
  return fmaxf(v, __int_as_float(dpp_move<CTRL, ROWS>(b, b)));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_sum_step(double v) {
  return v + dpp_move_f64<CTRL, ROWS>(v);
}

constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr3 = 0x113, kDppShr4 = 0x114,
              kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max_step<kDppShr1, 0xf>(v);
  v = dpp_max_step<kDppShr2, 0xf>(v);
  v = dpp_max_step<kDppShr4, 0xf>(v);
  v = dpp_max_step<kDppShr8, 0xf>(v);
  v = dpp_max_step<kDppBcast15, 0xa>(v);
  v = dpp_max_step<kDppBcast31, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_sum_step_f32(float v) {
  const int b = __float_as_int(v);
  return v + __int_as_float(dpp_move<CTRL, ROWS>(0, b));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v = dpp_sum_step_f32<kDppShr1, 0xf>(v);
  v = dpp_sum_step_f32<kDppShr2, 0xf>(v);
  v = dpp_sum_step_f32<kDppShr4, 0xf>(v);
  v = dpp_sum_step_f32<kDppShr8, 0xf>(v);
  v = dpp_sum_step_f32<kDppBcast15, 0xa>(v);
  v = dpp_sum_step_f32<kDppBcast31, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ double wave_sum(double v) {
  v = dpp_sum_step<kDppShr1, 0xf>(v);
  v = dpp_sum_step<kDppShr2, 0xf>(v);
  v = dpp_sum_step<kDppShr4, 0xf>(v);
  v = dpp_sum_step<kDppShr8, 0xf>(v);
  v = dpp_sum_step<kDppBcast15, 0xa>(v);
  v = dpp_sum_step<kDppBcast31, 0xc>(v);
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ void dpp_argmax_step(float& m, int& i) {
  const float om = __int_as_float(dpp_move<CTRL, ROWS>(__float_as_int(m), __float_as_int(m)));
  const int oi = dpp_move<CTRL, ROWS>(i, i);
  if (om > m || (om == m && oi < i)) {
    m = om;
    i = oi;
  }
}

// The max and the lowest index attaining it, for every lane (DPP as above).
__device__ __forceinline__ void wave_argmax(float& m, int& i) {
  dpp_argmax_step<kDppShr1, 0xf>(m, i);
  dpp_argmax_step<kDppShr2, 0xf>(m, i);
  dpp_argmax_step<kDppShr4, 0xf>(m, i);
  dpp_argmax_step<kDppShr8, 0xf>(m, i);
  dpp_argmax_step<kDppBcast15, 0xa>(m, i);
  dpp_argmax_step<kDppBcast31, 0xc>(m, i);
  m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_isum_step(int v) {
  return v + dpp_move<CTRL, ROWS>(0, v);
}

__device__ __forceinline__ int wave_sum_int(int v) {
  v = dpp_isum_step<kDppShr1, 0xf>(v);
  v = dpp_isum_step<kDppShr2, 0xf>(v);
  v = dpp_isum_step<kDppShr4, 0xf>(v);
  v = dpp_isum_step<kDppShr8, 0xf>(v);
  v = dpp_isum_step<kDppBcast15, 0xa>(v);
  v = dpp_isum_step<kDppBcast31, 0xc>(v);
  return __builtin_amdgcn_readlane(v, 63);
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
__device__ int block_sum_int(int v, int* lds) {
  v = wave_sum_int(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) lds[w] = v;
  __syncthreads();
  int r = lds[0];
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


// Value of lane src, for a src the same in every lane (a register read
// instead of a shuffle through the LDS crossbar).
__device__ __forceinline__ int lane_i32(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ float lane_f32(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ double lane_f64(double v, int src) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The previous lane's value (0 in lane 0): DPP wave_shr:1.
constexpr int kDppWaveShr1 = 0x138;
__device__ __forceinline__ double lane_before(double v) {
  return dpp_move_f64<kDppWaveShr1, 0xf>(v);
}

// Inclusive prefix sum over the wavefront by DPP: the lane's own value plus
// the three before it in its row, then row_shr 4 into banks 1-3 and row_shr 8
// into banks 2-3 complete each row's scan; row_bcast:15 and row_bcast:31
// carry the row totals forward.  The whole wavefront must be active.
__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
  (void)lane;
  const double x = v;
  v += dpp_move_f64<kDppShr1, 0xf>(x);
  v += dpp_move_f64<kDppShr2, 0xf>(x);
  v += dpp_move_f64<kDppShr3, 0xf>(x);
  v += dpp_move_f64<kDppShr4, 0xf, 0xe>(v);
  v += dpp_move_f64<kDppShr8, 0xf, 0xc>(v);
  v += dpp_move_f64<kDppBcast15, 0xa>(v);
  v += dpp_move_f64<kDppBcast31, 0xc>(v);
  return v;
}

}  // namespace
}  // namespace sv
