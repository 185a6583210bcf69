// n-gram prompt-lookup proposer on gfx950, and its C entry point.
//
// Source: "深入推测解码：从概念到实现" (Exploring Speculative Decoding), section
// n-gram.  The last n tokens of a request's context are looked up earlier in
// the context, and the k tokens that followed that earlier occurrence become
// the drafts; n is the longest match in [min_n, max_n].  The page's host code
// runs a KMP search per request on the CPU.  Here one workgroup per request
// tests every end position in parallel: thread t compares the tokens ending
// at positions N-2-t, N-2-t-256, ... backwards against the suffix and stops at
// the first mismatch, so on ordinary text most positions cost one compare.
// The context is staged through LDS in tiles of 4096 tokens (plus the 31
// tokens before a tile that a comparison can reach), so the comparisons read
// LDS and each tile costs one round trip to memory.  The best (length, end)
// pair is a 64-bit max over the workgroup: the longest match, and among
// equals the most recent one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {
namespace {

constexpr int kNgramThreads = 256;
constexpr int kMaxNgram = SPEC_NGRAM_MAX_N;

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

constexpr int kTile = 4096;               // context tokens per LDS tile
constexpr int kHalo = kMaxNgram - 1;      // earlier tokens a comparison can reach

__global__ __launch_bounds__(kNgramThreads) void k_ngram(const int32_t* __restrict__ ctx,
                                                         int stride,
                                                         const int32_t* __restrict__ lens,
                                                         int min_n, int max_n, int k,
                                                         int max_model_len, int32_t* out,
                                                         int32_t* out_num) {
  // tile [e0 - kHalo, e0 + kTile) of the context; lds[kHalo + i] = t[e0 + i]
  __shared__ int32_t lds[kHalo + kTile];
  __shared__ uint64_t s_best[kNgramThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int32_t* t = ctx + (size_t)b * stride;
  int N = lens[b];
  N = N < 0 ? 0 : (N > stride ? stride : N);
  const int nmax = min(max_n, N - 1);  // longest usable match

  // the suffix, last token first (uniform: scalar loads)
  int32_t suf[kMaxNgram];
#pragma unroll
  for (int i = 0; i < kMaxNgram; ++i) suf[i] = i < nmax ? t[N - 1 - i] : 0;

  // key = (match length << 32) | (end + 1); 0 = no match of length >= min_n.
  // End positions e run over [0, N - 2], one LDS tile at a time.
  uint64_t best = 0;
  for (int e0 = 0; e0 <= N - 2; e0 += kTile) {
    const int lo = max(0, e0 - kHalo), hi = min(N - 1, e0 + kTile);  // tokens [lo, hi)
    if (e0 > 0) __syncthreads();  // the previous tile is no longer read
    const bool vec = ((reinterpret_cast<uintptr_t>(t + e0) & 15u) == 0);
    if (vec) {  // 16-byte loads for the tile body, single loads for the rest
      const int nv = (hi - e0) / 4;
      const int4* v = reinterpret_cast<const int4*>(t + e0);
      for (int i = tid; i < nv; i += kNgramThreads) {
        const int4 x = v[i];
        int32_t* d = lds + kHalo + 4 * i;
        d[0] = x.x;
        d[1] = x.y;
        d[2] = x.z;
        d[3] = x.w;
      }
      for (int i = e0 + 4 * nv + tid; i < hi; i += kNgramThreads) lds[kHalo + i - e0] = t[i];
    } else {
      for (int i = e0 + tid; i < hi; i += kNgramThreads) lds[kHalo + i - e0] = t[i];
    }
    for (int i = lo + tid; i < e0; i += kNgramThreads) lds[kHalo + i - e0] = t[i];
    __syncthreads();
    const int e1 = min(N - 2, e0 + kTile - 1);
    for (int e = e1 - tid; e >= e0; e -= kNgramThreads) {
      int len = 0;
      bool alive = true;
#pragma unroll
      for (int i = 0; i < kMaxNgram; ++i) {
        if (alive) {
          alive = i < nmax && i <= e && lds[kHalo + e - e0 - i] == suf[i];
          len += alive;
        }
      }
      if (len >= min_n) {
        const uint64_t key = ((uint64_t)len << 32) | (uint32_t)(e + 1);
        best = key > best ? key : best;
      }
    }
  }
  best = wave_max_u64(best);
  if ((tid & 63) == 0) s_best[tid >> 6] = best;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kNgramThreads / 64; ++w) best = s_best[w] > best ? s_best[w] : best;

  int count = 0, start = 0;
  if (best != 0) {
    start = (int)(uint32_t)best;  // first token after the occurrence
    count = min(k, min(N - start, max_model_len - N));
    if (count < 0) count = 0;
  }
  for (int i = tid; i < k; i += kNgramThreads)
    out[(size_t)b * k + i] = i < count ? t[start + i] : -1;
  if (tid == 0) out_num[b] = count;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace
}  // namespace sv

extern "C" int spec_ngram_propose(int32_t B, const int32_t* context, int32_t stride,
                                  const int32_t* context_lens, int32_t min_n, int32_t max_n,
                                  int32_t k, int32_t max_model_len, int32_t* out_drafts,
                                  int32_t* out_num_drafts, void* stream) {
  if (B < 0 || k < 0 || max_model_len < 0 || min_n < 1 || max_n < min_n ||
      max_n > SPEC_NGRAM_MAX_N)
    return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (stride < 1 || context == nullptr || context_lens == nullptr ||
      out_num_drafts == nullptr || (k > 0 && out_drafts == nullptr))
    return SV_ERR_INVALID_ARG;
  if (!sv::aligned4(context) || !sv::aligned4(context_lens) || !sv::aligned4(out_num_drafts) ||
      (out_drafts != nullptr && !sv::aligned4(out_drafts)))
    return SV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(sv::k_ngram, dim3((unsigned)B), dim3(sv::kNgramThreads), 0,
                     static_cast<hipStream_t>(stream), context, stride, context_lens, min_n,
                     max_n, k, max_model_len, out_drafts, out_num_drafts);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
