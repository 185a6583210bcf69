// HIP kernels of the speculative-sampling verify step for gfx950 (CDNA4).
//
// One step is four launches on the caller's stream:
//   1. stats   streams every needed logits row once, split into vocabulary
//              chunks: per chunk the max and the sum of exp2(l * c + ref)
//              (sampling rows) or the max and its lowest index (greedy rows).
//              HBM-bound; this is the hot loop.  A dynamic LDS request caps
//              its resident workgroups per CU (more only lengthen the queues).
//   2. decide  one wavefront per request: lane s folds the chunk partials
//              of row slot s; then lane j draws the Philox uniforms of
//              position j, forms p(x)/q(x) in fp64, a ballot of the accept
//              bits gives the first rejection by count-trailing-zeros, and
//              the outputs and a draw descriptor are written.
//   3. resid   requests rejected on a probabilistic draft: the sum of
//              max(0, p - q) over each part of each chunk of that row pair
//              (2 parts per chunk for bf16 rows, 4 with an fp32 row).
//   4. locate  one workgroup per sampling request: a prefix over the chunk
//              sums finds the chunk holding u * S (and, for a pair, the
//              part); each of its 1024, 512 or 256 threads takes
//              16384 / threads consecutive residuals of that range in
//              registers, and a workgroup scan of the segment sums finds
//              the token.
//
// Method (page title, section): "深入推测解码：从概念到实现" 保证原始分布
// (accept with min(1, p/q), resample from max(0, p - q)); "RTP-LLM
// Speculative Engine 深度解析" 拒绝采样算法 (uniform vs p/q per position,
// stop at the first rejection); "投机采样" 投机解码算法 steps 3-5 (accepted
// count, adjusted law, extra token from the last target row).
#include <float.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_device.h"
#include "sv_internal.h"

namespace sv {
namespace {

// ---------------------------------------------------------------------------
// Chunk streaming
// ---------------------------------------------------------------------------
// Build-time tuning knobs (-D on the compiler line).  The defaults are the
// fastest measured on MI355X for the bf16 verify step: 8 loads in flight per
// thread (12 was 6% slower) and nontemporal loads (temporal ones 14% slower).
#ifndef SV_LOADS_IN_FLIGHT
#define SV_LOADS_IN_FLIGHT 8
#endif
#ifndef SV_STREAM_NT
#define SV_STREAM_NT 1
#endif
constexpr int kUnroll = SV_LOADS_IN_FLIGHT;  // 16-byte loads in flight per thread

// Streaming 16-byte load; rows are read once per step.
__device__ __forceinline__ u32x4 stream_load(const u32x4* p) {
#if SV_STREAM_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

// Raw bits of element i of a row, and their value.
template <int DT>
__device__ __forceinline__ uint32_t raw_elem(const void* row, int i) {
  if constexpr (DT == SV_BF16)
    return static_cast<const uint16_t*>(row)[i];
  else
    return static_cast<const uint32_t*>(row)[i];
}

template <int DT>
__device__ __forceinline__ float raw_to_float(uint32_t w) {
  return __uint_as_float(DT == SV_BF16 ? w << 16 : w);
}

// The raw bits of element k of a 16-byte vector replaced by -inf, which
// takes the element out of a chunk's max and sums.
template <int DT>
__device__ __forceinline__ u32x4 mask_elem(u32x4 d, int k) {
  uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == SV_BF16) {
      const uint32_t lo = (w[i] & 0xffff0000u) | 0xff80u, hi = (w[i] & 0xffffu) | 0xff800000u;
      w[i] = k == 2 * i ? lo : (k == 2 * i + 1 ? hi : w[i]);
    } else {
      w[i] = k == i ? 0xff800000u : w[i];
    }
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Softmax statistics of one chunk, by the whole workgroup.  A pass holds
// kUnroll 16-byte vectors per thread in registers (all loads in flight
// together); the workgroup takes the max of the pass first, moves the shared
// exponent reference R = ref_of(M, c) if the max grew, and only then sums
// exp2(l * c + R).  With one reference for the workgroup the thread sums add
// without rescaling, and no element needs a running-max test.  The loads go
// through a buffer resource over the chunk's vectors: a round issues all of
// them with no branch, and past the chunk the hardware returns 0 without
// touching memory; those vectors are not folded (the test is uniform in all
// but one wave of a pass).
// COUNT: also count the chunk's elements above lx (into *above).
// EXCL: element xi of the chunk is left out of the sums (the draft of a
// one-hot row: a correction draws from the chunk without it); the max and
// so the reference still include it.
template <int DT, bool COUNT, bool EXCL = false>
__device__ __forceinline__ void chunk_softmax_block(const void* row, int c0, int c1, float c,
                                                    float* ldsf, double* ldsd, float* m_out,
                                                    double* z_out, float lx = 0.f,
                                                    int* ldsi = nullptr, int* above = nullptr,
                                                    int xi = -1) {
  using E = Elt<DT>;
  const Geo g = chunk_geo<DT>(row, c0, c1);
  const int tid = threadIdx.x;
  const u32x4* vp = reinterpret_cast<const u32x4*>(
      static_cast<const char*>(row) + (size_t)g.v0 * E::kBytes);
  const VecBuf vb = make_vec_buf(vp, (uint32_t)g.nvec * 16u);
  float M = kNegInf, R = 0.f, S = 0.f;
  int cnt = 0;  // COUNT: elements above lx seen by this wavefront (uniform)
  for (int base = 0; base == 0 || base < g.nvec; base += kThreads * kUnroll) {
    const int v = base + tid;
    // head and tail (each under one vector) ride along with the first pass.
    // Their loads go first and every lane makes them, at an index clamped
    // into the chunk: loads complete in issue order for the wait counter, so
    // waiting for them then does not wait for the vectors (each vector is
    // folded as it arrives), and no branch makes the compiler wait at its end.
    uint32_t h = 0, tl = 0;  // raw element bits
    if (base == 0) {  // uniform
      h = raw_elem<DT>(row, min(g.c0 + tid, g.c1 - 1));
      tl = raw_elem<DT>(row, min(g.t0 + tid, g.c1 - 1));
    }
    u32x4 d[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      d[u] = buf_load<SV_STREAM_NT != 0>(vb, (uint32_t)(v + u * kThreads) * 16u);
    // the head and tail bits are first used past this point, after every
    // load of the pass is issued (the clobber keeps the loads above it)
    asm volatile("" : "+v"(h), "+v"(tl) : : "memory");
    float ht[2];
    ht[0] = base == 0 && g.c0 + tid < g.v0 ? raw_to_float<DT>(h) : kNegInf;
    ht[1] = base == 0 && g.t0 + tid < g.c1 ? raw_to_float<DT>(tl) : kNegInf;
    float t = fmaxf(ht[0], ht[1]);
    // a compare per element, counted across the wavefront by a scalar
    // popcount of its lane mask instead of a per-lane add
    if (COUNT) cnt += __popcll(__ballot(ht[0] > lx)) + __popcll(__ballot(ht[1] > lx));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (v + u * kThreads < g.nvec) {
        float x[E::kVec];
        E::unpack(d[u], x);
#pragma unroll
        for (int k = 0; k < E::kVec; ++k) {
          t = fmaxf(t, x[k]);
          if (COUNT) cnt += __popcll(__ballot(x[k] > lx));
        }
      }
    }
    const float pm = block_max<kThreads>(t, ldsf);
    if (pm > M) {  // uniform across the workgroup
      const float rn = ref_of(pm, c);
      S = (M == kNegInf) ? 0.f : S * fast_exp2(rn - R);
      R = rn;
      M = pm;
    }
    // EXCL: xi stays in the max (the chunk's reference may include it) but
    // leaves the sums: its bits become -inf in the sum phase's copy of the
    // one vector or scalar that holds it
    if (EXCL && base == 0 && xi < g.v0 && g.c0 + tid == xi) ht[0] = kNegInf;
    if (EXCL && base == 0 && xi >= g.t0 && g.t0 + tid == xi) ht[1] = kNegInf;
    float s = fast_exp2(fmaf(ht[0], c, R)) + fast_exp2(fmaf(ht[1], c, R));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (v + u * kThreads < g.nvec) {
        // unpack again rather than keep 64 floats live: the empty asm hides
        // the first unpack from common-subexpression elimination
        u32x4 w = d[u];
        asm volatile("" : "+v"(w));
        if (EXCL && xi >= g.v0 && xi < g.t0 && v + u * kThreads == (xi - g.v0) / E::kVec)
          w = mask_elem<DT>(w, (xi - g.v0) % E::kVec);
        float e[E::kVec];
        E::unpack(w, e);
#pragma unroll
        for (int k = 0; k < E::kVec; ++k) e[k] = fast_exp2(fmaf(e[k], c, R));
        s += pairwise_sum(e);
      }
    }
    S += s;
  }
  *z_out = block_sum<kThreads>((double)S, ldsd);
  *m_out = M;
  if (COUNT) *above = block_sum_int<kThreads>((tid & 63) == 0 ? cnt : 0, ldsi);
}

template <int DT>
__device__ __forceinline__ AmAcc chunk_argmax(const void* row, int c0, int c1) {
  using E = Elt<DT>;
  constexpr int kSub = 16 / E::kVec;
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
  for (int v = tid; v < g.nvec; v += kThreads * kUnroll) {
    u32x4 d[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      d[u] = E::neg_inf();
      if (v + u * kThreads < g.nvec) d[u] = stream_load(vp + v + u * kThreads);
    }
#pragma unroll
    for (int u0 = 0; u0 < kUnroll; u0 += kSub) {
      float x[kSub * E::kVec];
#pragma unroll
      for (int u = 0; u < kSub; ++u) E::unpack(d[u0 + u], x + u * E::kVec);
      float t = x[0];
#pragma unroll
      for (int k = 1; k < kSub * E::kVec; ++k) t = fmaxf(t, x[k]);
      if (t > a.M || (t == a.M && a.I == INT32_MAX)) {  // rare: locate it
        int best = INT32_MAX;
#pragma unroll
        for (int k = kSub * E::kVec - 1; k >= 0; --k) {
          const int vi = v + (u0 + k / E::kVec) * kThreads;
          if (x[k] == t && vi < g.nvec) best = g.v0 + vi * E::kVec + k % E::kVec;
        }
        if (best != INT32_MAX) {
          a.M = t;
          a.I = best;
        }
      }
    }
  }
  if (g.t0 + tid < g.c1) {
    const float x[1] = {E::at(row, g.t0 + tid)};
    const int ix[1] = {g.t0 + tid};
    am_tile(a, x, ix);
  }
  return a;
}

// ---------------------------------------------------------------------------
// Requests
// ---------------------------------------------------------------------------
// Row slots of request b: 0..K are target rows j = slot, K+1..2K draft rows
// j = slot - K - 1.  In the draft sampler a request is one draft row, with
// K = 0 and the row in slot 0.
struct ReqInfo {
  int n;             // drafts, clamped into [0, K]
  float T;
  bool sampling;     // else greedy
  bool onehot;       // no draft distribution
  bool draft_stats;  // draft rows are logits whose softmax is needed
  bool active;       // sampler: the row is below the request's draft count
  bool bad_n;        // the request's draft count was outside [0, K]
  int rb, rj;        // sampler: request and position of the row
};

__device__ __forceinline__ ReqInfo req_info(const RunParams& p, int b) {
  ReqInfo r;
  const bool sampler = p.sample_k > 0;
  r.rb = sampler ? b / p.sample_k : b;
  r.rj = b - r.rb * (sampler ? p.sample_k : 1);
  // the per-request loads go out together as scalar loads, so a workgroup
  // knows after one round trip whether its row slot is needed.  A missing
  // count array reads the temperature's address instead (that value is
  // unused); the mode byte comes from its aligned word, which lies in the
  // byte's own page.
  const float* tp = p.temps + r.rb;
  const int32_t* np = p.nd != nullptr ? p.nd + r.rb : reinterpret_cast<const int32_t*>(tp);
  const int nv = *np;
  r.T = *tp;
  uint32_t mv = 0;
  if (p.mode != nullptr) {
    const uint8_t* m = p.mode + r.rb;
    const uint32_t sh = reinterpret_cast<uintptr_t>(m) & 3u;
    mv = (*reinterpret_cast<const uint32_t*>(m - sh) >> (8 * sh)) & 0xffu;
  }
  asm volatile("" ::"s"(nv), "s"(r.T), "s"(mv));  // no load waits for another
  if (sampler) {
    const int nb = p.nd != nullptr ? nv : p.sample_k;
    r.bad_n = nb < 0 || nb > p.sample_k;
    r.active = r.rj < clamp_drafts(nb, p.sample_k);
    r.n = 0;
    r.onehot = true;
  } else {
    r.n = clamp_drafts(nv, p.K);
    r.bad_n = nv != r.n;
    r.active = true;
    r.onehot = !p.has_draft || (p.mode != nullptr && mv != 0);
  }
  r.sampling = is_sampling(r.T);
  r.draft_stats = r.sampling && !r.onehot && !p.draft_is_probs;
  return r;
}

__device__ __forceinline__ bool slot_needed(const ReqInfo& r, int s, int K) {
  return r.active && (s <= K ? s <= r.n : (s - K - 1 < r.n && r.draft_stats));
}

// Whether target row j's statistics leave out its draft x (= xid): a one-hot
// sampling request's drafted rows.  A correction at j then draws from the
// row's partials as they are, and the decision adds x's share back to the
// row total in fp64.  The same test is made on both sides of the hand-off.
__device__ __forceinline__ bool excl_draft(const RunParams& p, const ReqInfo& r, int j, int xid) {
  return p.sample_k == 0 && !p.typical && r.sampling && r.onehot && j < r.n && xid >= 0 &&
         xid < p.V;
}

// ---------------------------------------------------------------------------
// Decisions of one request (one wavefront)
// ---------------------------------------------------------------------------
// Lane s first owns row slot s and folds that row's chunk partials; lane j
// then decides drafted position j with the combined target row j and draft
// row j.  The draw descriptor goes to *d_out (shared memory); with `outputs`
// the accepted tokens, counts, debug probabilities, greedy tokens and the
// descriptor in global memory are written too.
template <int TDT, int DDT>
__device__ void decide_request(const RunParams& p, int b, const ReqInfo& ri, bool outputs,
                               DrawDesc* d_out) {
  const int K = p.K, V = p.V, nslot = 2 * K + 1, n = ri.n;
  const int lane = threadIdx.x & 63;
  const float c = ri.sampling ? temp_scale(ri.T) : 0.f;

  // independent loads first, so they share one round trip: the first
  // kBatch chunk partials of row slot `lane` (clamped into the request's
  // slots and chunks; unused ones are ignored) and this lane's draft id
  constexpr int kBatch = 16;
  const Partial* pr = p.part + ((size_t)b * nslot + min(lane, nslot - 1)) * p.nchunk;
  Partial q[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) q[u] = pr[min(u, p.nchunk - 1)];
  int x = -1;
  if (lane < n) x = p.ids[(size_t)b * K + lane];

  // lanes 0..n draw their Philox blocks once, while the loads are in flight:
  // word 0 decides position j, word 1 is the draw uniform if the walk stops
  // there
  double u_acc = 0.0, u_rec = 0.0;
  if (ri.sampling && p.sample_k == 0 && lane <= n)
    uniforms(p.seed, p.offset, p.b_base + b, lane, &u_acc, &u_rec);

  // values of the drafted tokens
  float lt = __builtin_nanf(""), ld = __builtin_nanf("");
  if (lane < n && x >= 0 && x < V) {
    lt = load_elem(p.target, TDT, (size_t)b * (K + 1) + lane, V, x);
    if (ri.sampling && !ri.onehot) ld = load_elem(p.draft, DDT, (size_t)b * K + lane, V, x);
  }

  // combine: lane s owns row slot s (target rows 0..K, draft rows K+1..2K)
  // and folds its chunk partials sequentially, so no cross-lane traffic
  float r_ref = 0.f;  // sampling: exponent reference; greedy: row max
  double r_z = 0.0;   // sampling: row total relative to the reference
  int r_idx = 0;      // greedy: lowest index of the max
  int rank = 0;       // typical acceptance: elements above the draft's logit
  if (lane < nslot && slot_needed(ri, lane, K)) {
    float m = kNegInf;
    int im = INT32_MAX;
    const bool counts = p.typical && p.top_k > 0 && ri.sampling && lane < n;
    for (int k0 = 0; k0 < p.nchunk; k0 += kBatch) {
      if (k0 > 0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) q[u] = pr[min(k0 + u, p.nchunk - 1)];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (k0 + u < p.nchunk && q[u].m > m) {  // chunks ascend: first max wins
          m = q[u].m;
          im = q[u].idx;
        }
        if (counts && k0 + u < p.nchunk) rank += q[u].idx;
      }
    }
    // a one-hot row's chunk sums leave out its draft (its max keeps it): the
    // row total takes x back, exactly (lt is x's logit)
    const bool excl = excl_draft(p, ri, lane, x);
    if (ri.sampling) {
      r_ref = ref_of(m, c);
      for (int k0 = 0; k0 < p.nchunk; k0 += kBatch) {
        if (k0 > 0 || p.nchunk > kBatch) {
#pragma unroll
          for (int u = 0; u < kBatch; ++u) q[u] = pr[min(k0 + u, p.nchunk - 1)];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (k0 + u < p.nchunk && q[u].z != 0.0)
            r_z += q[u].z * exp2_diff(r_ref, ref_of(q[u].m, c));
      }
      if (excl) r_z += exp2((double)lt * (double)c + (double)r_ref);
    } else {
      r_ref = m;
      r_idx = im == INT32_MAX ? 0 : im;
    }
  }
  // lane j gathers its target row (own) and its draft row (lane K + 1 + j)
  const float t_ref = r_ref;
  const double t_z = r_z;
  const int t_idx = r_idx;
  const int dl = min(K + 1 + lane, 63);
  const float d_ref = __shfl(r_ref, dl, 64);
  const double d_z = __shfl(r_z, dl, 64);

  // decision of position j = lane
  bool accept = false;
  float dbg_p = __builtin_nanf(""), dbg_q = __builtin_nanf("");
  if (lane < n) {
    const bool valid = x >= 0 && x < V;
    if (!valid && outputs) atomicOr(p.flags, SV_DEVERR_BAD_DRAFT_ID);
    if (!ri.sampling) {
      accept = valid && lt == t_ref;
    } else if (valid) {
      const double px = exp2((double)lt * (double)c + (double)t_ref) / t_z;
      double qx = 1.0;
      if (!ri.onehot) {
        if (p.draft_is_probs)
          qx = (double)ld;
        else
          qx = exp2((double)ld * (double)c + (double)d_ref) / d_z;
      }
      double ratio;
      if (qx > 0.0) ratio = px / qx;
      else ratio = px > 0.0 ? __builtin_inf() : 0.0;
      if (p.typical)  // threshold or top-k: no uniform
        accept = px > (double)p.eps || rank < p.top_k;
      else
        accept = u_acc < ratio;
      dbg_p = (float)px;
      dbg_q = (float)qx;
    }
  }
  // first rejection: lanes >= n vote false, so ~mask has a bit at n or below
  const uint64_t mask = __ballot(accept);
  const int first_rej = (int)__builtin_ctzll(~mask);
  const int n_acc = first_rej < n ? first_rej : n;

  if (outputs && lane <= K && lane != n_acc)
    p.out_tokens[(size_t)b * (K + 1) + lane] = lane < n_acc ? x : -1;
  if (outputs && lane == 0) {
    if (p.out_nacc != nullptr) p.out_nacc[b] = n_acc;
    if (ri.bad_n && ri.rj == 0) atomicOr(p.flags, SV_DEVERR_BAD_NUM_DRAFTS);
  }
  if (outputs && p.out_dbg != nullptr && lane < K) {
    p.out_dbg[((size_t)b * K + lane) * 2 + 0] = dbg_p;
    p.out_dbg[((size_t)b * K + lane) * 2 + 1] = dbg_q;
  }

  // the emitted position: greedy writes its argmax, sampling requests leave a
  // draw descriptor for the residual and draw kernels
  DrawDesc d{};
  if (lane == n_acc) {
    const int je = n_acc;
    d.j = je;
    d.x = -1;
    d.cstar = -1;
    if (!ri.active) {  // sampler row past the request's draft count
      if (outputs) p.out_tokens[b] = -1;
      if (outputs && p.out_q != nullptr) p.out_q[b] = __builtin_nanf("");
      d.kind = kDrawNone;
    } else if (!ri.sampling) {
      if (outputs) p.out_tokens[(size_t)b * (K + 1) + je] = t_idx;
      if (outputs && p.out_q != nullptr) p.out_q[b] = 1.f;  // a point mass
      d.kind = kDrawNone;
    } else {
      d.c = c;
      d.ref_p = t_ref;
      d.z_p = t_z;
      if (p.sample_k > 0)
        d.u = draft_uniform(p.seed, p.offset, p.b_base + ri.rb, ri.rj);
      else
        d.u = u_rec;  // this lane is je = n_acc <= n
      d.kind = kDrawSingle;
      if (je < n && !p.typical) {  // rejected at je (typical: draw from p itself)
        d.x = (x >= 0 && x < V) ? x : -1;
        if (!ri.onehot) {
          d.kind = kDrawPair;
          double kap;
          if (p.draft_is_probs) {
            d.ref_q = 0.f;
            kap = d.z_p;  // p - q = (p~ - Z_p q) / Z_p
          } else {
            d.ref_q = d_ref;
            kap = d.z_p / d_z;  // p - q = (p~ - (Z_p / Z_q) q~) / Z_p
          }
          d.kap_hi = (float)kap;
          d.kap_lo = (float)(kap - (double)d.kap_hi);
        }
      }
    }
  }

  // a single-row draw (from p, less an excluded one-hot draft) is placed in
  // its chunk here, one lane per chunk: chunk masses are the row's partials
  // rescaled to ref_p, the values the fold above summed
  if (lane_i32(d.kind, n_acc) == kDrawSingle) {
    const int je = n_acc;
    const float dc = lane_f32(d.c, je), dref = lane_f32(d.ref_p, je);
    const double du = lane_f64(d.u, je);
    int excl = lane_i32(d.x, je);
    const float lx = lane_f32(lt, je);
    // chunk masses: the row's partials at ref_p (a one-hot row's already
    // leave out its draft x, so a correction needs no subtraction)
    double mass = 0.0;
    if (lane < p.nchunk) {
      const Partial q = p.part[((size_t)b * nslot + je) * p.nchunk + lane];
      if (q.z != 0.0) mass = q.z * exp2_diff(dref, ref_of(q.m, dc));
    }
    double mx = mass > 0.0 ? mass : 0.0;
    double incl = wave_incl_scan(mx, lane);
    double S = lane_f64(incl, 63);
    if (!(S > 0.0) && excl >= 0) {  // no mass without x: draw from p itself
      if (outputs && lane == 0) atomicOr(p.flags, SV_DEVERR_ZERO_RESIDUAL);
      if (excl / p.chunk == lane) mx += exp2((double)lx * (double)dc + (double)dref);
      excl = -1;
      incl = wave_incl_scan(mx, lane);
      S = lane_f64(incl, 63);
    }
    const double theta = du * S;
    double before = lane_before(incl);
    if (lane == 0) before = 0.0;
    const uint64_t hits = __ballot(mx > 0.0 && before <= theta && theta < incl);
    int cstar;
    double th;
    if (hits) {
      cstar = (int)__builtin_ctzll(hits);
      th = theta - lane_f64(before, cstar);
    } else {  // rounding left theta at or past the total: last chunk with mass
      const uint64_t has = __ballot(mx > 0.0);
      cstar = has ? 63 - (int)__builtin_clzll(has) : 0;
      th = __builtin_inf();
      if (outputs && lane == 0) atomicOr(p.flags, SV_DEVERR_DRAW_ROUNDING);
    }
    if (lane == je) {
      d.cstar = cstar;
      d.th = th;
      d.x = excl;
    }
  }
  if (lane == n_acc) {
    *d_out = d;
    if (outputs) p.desc[b] = d;
  }
}

// ---------------------------------------------------------------------------
// Kernel 1: row statistics
// ---------------------------------------------------------------------------
// Statistics of chunk `chunk` of row slot s of request b (all threads).
template <int TDT, int DDT>
__device__ __forceinline__ void stats_item(const RunParams& p, int b, int s, int chunk,
                                           const ReqInfo& ri, float* ldsf, double* ldsd,
                                           int* ldsi) {
  const int c0 = chunk * p.chunk;
  const int c1 = min(p.V, c0 + p.chunk);
  const bool is_target = s <= p.K;
  const void* r = is_target ? row_ptr(p.target, TDT, (size_t)b * (p.K + 1) + s, p.V)
                            : row_ptr(p.draft, DDT, (size_t)b * p.K + (s - p.K - 1), p.V);
  Partial out;
  if (ri.sampling) {
    const float c = temp_scale(ri.T);
    if (p.typical && p.top_k > 0 && s < ri.n) {
      // typical acceptance with a top-k clause: also count the elements
      // above the draft's logit (an invalid id counts nothing)
      const int x = p.ids[(size_t)b * p.K + s];
      const float lx = (x >= 0 && x < p.V) ? load_elem(p.target, TDT, (size_t)b * (p.K + 1) + s, p.V, x)
                                          : __builtin_inff();
      int above = 0;
      chunk_softmax_block<TDT, true>(r, c0, c1, c, ldsf, ldsd, &out.m, &out.z, lx, ldsi, &above);
      out.idx = above;
    } else if (is_target && excl_draft(p, ri, s, 0) &&
               excl_draft(p, ri, s, p.ids[(size_t)b * p.K + s]) &&
               p.ids[(size_t)b * p.K + s] >= c0 && p.ids[(size_t)b * p.K + s] < c1) {
      // a one-hot row's draft (loaded only here) leaves its chunk's sums
      chunk_softmax_block<TDT, false, true>(r, c0, c1, c, ldsf, ldsd, &out.m, &out.z, 0.f,
                                            nullptr, nullptr, p.ids[(size_t)b * p.K + s]);
      out.idx = -1;
    } else if (is_target) {
      chunk_softmax_block<TDT, false>(r, c0, c1, c, ldsf, ldsd, &out.m, &out.z);
      out.idx = -1;
    } else {
      chunk_softmax_block<DDT, false>(r, c0, c1, c, ldsf, ldsd, &out.m, &out.z);
      out.idx = -1;
    }
  } else {  // greedy rows are target rows
    AmAcc a = chunk_argmax<TDT>(r, c0, c1);
    block_argmax<kThreads>(a.M, a.I, ldsf, ldsi);
    out.m = a.M;
    out.idx = a.I == INT32_MAX ? c0 : a.I;
    out.z = 0.0;
  }
  if (threadIdx.x == 0)
    p.part[((size_t)b * (2 * p.K + 1) + s) * p.nchunk + chunk] = out;
}

// Row slots in the stats grid per request: target rows 0..K, and draft rows
// only when some request may need a draft softmax.  Typical acceptance, runs
// without draft rows and probability drafts never do; the host knows that
// without reading device data, and the grid then has no draft slots to skip
// (an empty workgroup still costs its launch: 4 us at B=512 K=3).
__host__ __device__ __forceinline__ int stats_slots(const RunParams& p) {
  return (p.typical || !p.has_draft || p.draft_is_probs) ? p.K + 1 : 2 * p.K + 1;
}

// Tuning knob: a minimum-waves-per-SIMD hint for the stats kernel (1 = none;
// 8, which caps it at 64 registers, measured no faster).
#ifndef SV_STATS_WAVES_PER_EU
#define SV_STATS_WAVES_PER_EU 1
#endif
// Tuning knobs: stats workgroups resident per compute unit.  The kernel
// streams rows at the memory system's limit, and once that is saturated more
// resident workgroups only lengthen the memory queues.  Best measured on
// MI355X: 6 for bf16 target rows and 4 for fp32 ones (half the arithmetic per
// byte); 0 (no cap) when typical acceptance also counts elements, which adds
// arithmetic per byte.  The limit without a cap is 8 (the kernel's registers).
#ifndef SV_STATS_WG_CAP_BF16
#define SV_STATS_WG_CAP_BF16 6
#endif
#ifndef SV_STATS_WG_CAP_F32
#define SV_STATS_WG_CAP_F32 4
#endif
// One workgroup per (request, row slot, chunk); unneeded slots exit at once.
template <int TDT, int DDT>
__global__ __launch_bounds__(kThreads, SV_STATS_WAVES_PER_EU) void k_stats(const RunParams p) {
  __shared__ float ldsf[kThreads / 64];
  __shared__ double ldsd[kThreads / 64];
  __shared__ int ldsi[kThreads / 64];
  const int nslot = stats_slots(p);
  const int bid = blockIdx.x;
  // kernels of the step that set flags run after this one on the stream
  if (p.clear_flags && bid == 0 && threadIdx.x == 0) *p.flags = 0u;
  const int row = bid / p.nchunk, chunk = bid - row * p.nchunk;
  const int b = row / nslot, s = row - b * nslot;
  const ReqInfo ri = req_info(p, b);
  if (!slot_needed(ri, s, p.K)) return;
  stats_item<TDT, DDT>(p, b, s, chunk, ri, ldsf, ldsd, ldsi);
}

// ---------------------------------------------------------------------------
// Residual elements (unnormalized, relative to the draw descriptor)
// ---------------------------------------------------------------------------
// Pair: r~ = max(0, p~ - kappa q~) with p~ = exp2(l_p c + ref_p) and q~ =
// exp2(l_q c + ref_q) (or q itself for probability drafts); kappa split in
// two floats keeps the difference accurate to the rounding of p~ and q~.
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

// Eight consecutive elements from a 16-byte aligned address, as raw words
// (one 16-byte load for bf16, two for f32) and unpacked later.
template <int DT>
struct Raw8 {
  u32x4 w[DT == SV_BF16 ? 1 : 2];
};


template <int DT>
__device__ __forceinline__ void unpack8(const Raw8<DT>& r, float* x) {
  if (DT == SV_BF16) {
    Elt<SV_BF16>::unpack(r.w[0], x);
  } else {
    Elt<SV_F32>::unpack(r.w[0], x);
    Elt<SV_F32>::unpack(r.w[DT == SV_BF16 ? 0 : 1], x + 4);
  }
}

// Groups of 8 elements per thread per round: enough for one round over a
// default chunk (15360 bf16 or 8192 fp32 elements) within 128 VGPRs.
// Parts per chunk of a residual pair (the residual pass runs one workgroup
// per part).
template <int TDT, int DDT>
constexpr int resid_split() {
  return (TDT == SV_F32 || DDT == SV_F32) ? SV_RESID_SPLIT_F32 : SV_RESID_SPLIT_BF16;
}
static_assert(SV_RESID_SPLIT_BF16 >= 1 && SV_RESID_SPLIT_F32 >= 1, "a chunk has one part or more");

template <int TDT, int DDT>
constexpr int resid_groups() {
  constexpr int g = ((TDT == SV_F32 || DDT == SV_F32) ? 4 : 8) / resid_split<TDT, DDT>();
  return g > 0 ? g : 1;
}

// Sum over [c0, c1) of max(0, p~ - kappa q~), token x excluded.  All loads of
// a round (resid_groups() groups of eight elements of both rows per thread)
// are issued before any is used; validity is tested per group, and the
// excluded token's residual is subtracted once from its own loads.
template <int TDT, int DDT>
__device__ __forceinline__ double pair_chunk_sum(const void* prow, const void* qrow, int c0,
                                                 int c1, const DrawDesc& d, bool probs,
                                                 double* ldsd) {
  constexpr int kResidGroups = resid_groups<TDT, DDT>();
  const int tid = threadIdx.x;
  double acc = 0.0;
  // the excluded token's elements, loaded with the rest
  const bool has_x = tid == 0 && d.x >= c0 && d.x < c1;
  float xp = 0.f, xq = 0.f;
  if (has_x) {
    xp = Elt<TDT>::at(prow, d.x);
    xq = Elt<DDT>::at(qrow, d.x);
  }
  const uintptr_t pa = reinterpret_cast<uintptr_t>(prow) + (uintptr_t)c0 * Elt<TDT>::kBytes;
  const uintptr_t qa = reinterpret_cast<uintptr_t>(qrow) + (uintptr_t)c0 * Elt<DDT>::kBytes;
  int done = c0;
  if (((pa | qa) & 15u) == 0) {
    const int ngrp = (c1 - c0) / 8;
    // buffer loads: every load of a round is issued unconditionally (past the
    // groups the hardware returns 0) with one offset register each
    constexpr int kPB = 8 * Elt<TDT>::kBytes, kQB = 8 * Elt<DDT>::kBytes;  // bytes per group
    const VecBuf pb = make_vec_buf(reinterpret_cast<const void*>(pa), (uint32_t)ngrp * kPB);
    const VecBuf qb = make_vec_buf(reinterpret_cast<const void*>(qa), (uint32_t)ngrp * kQB);
    for (int g = tid; g < ngrp; g += kThreads * kResidGroups) {
      Raw8<TDT> rp[kResidGroups];
      Raw8<DDT> rq[kResidGroups];
#pragma unroll
      for (int u = 0; u < kResidGroups; ++u) {
        const int gi = g + u * kThreads;
#pragma unroll
        for (int h = 0; h < kPB / 16; ++h) rp[u].w[h] = buf_load<true>(pb, (uint32_t)gi * kPB + 16 * h);
#pragma unroll
        for (int h = 0; h < kQB / 16; ++h) rq[u].w[h] = buf_load<true>(qb, (uint32_t)gi * kQB + 16 * h);
      }
      float s[kResidGroups];
#pragma unroll
      for (int u = 0; u < kResidGroups; ++u) {
        float lp[8], lq[8], e[8];
        unpack8<TDT>(rp[u], lp);
        unpack8<DDT>(rq[u], lq);
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = pair_resid(lp[k], lq[k], d, probs);
        const float sg = pairwise_sum(e);
        s[u] = g + u * kThreads < ngrp ? sg : 0.f;
      }
      acc += (double)pairwise_sum(s);
    }
    done = c0 + ngrp * 8;
  }
  float tail = 0.f;
  for (int i = done + tid; i < c1; i += kThreads)
    tail += pair_resid(Elt<TDT>::at(prow, i), Elt<DDT>::at(qrow, i), d, probs);
  acc += (double)tail;
  if (has_x) acc -= (double)pair_resid(xp, xq, d, probs);
  return block_sum<kThreads>(acc, ldsd);
}

// ---------------------------------------------------------------------------
// Inverse-CDF draw of the emitted token (one workgroup)
// ---------------------------------------------------------------------------
// The draw of one request runs NT threads, each owning 16384 / NT
// consecutive elements of the chosen chunk.  Few draws take 1024 threads
// (short per-thread work), more take 512, many take 256 (more draws
// resident per CU).
template <int NT>
constexpr int seg_len() { return 16384 / NT; }
static_assert(seg_len<1024>() * 1024 >= kMaxChunkElems, "a chunk must fit the segments");

// Raw bits of SEG consecutive elements of a row, kept in registers instead
// of floats (half the registers for bf16); element k is unpacked on use.
template <int DT, int SEG>
struct SegWords {
  static constexpr int kWords = SEG * Elt<DT>::kBytes / 4;
  uint32_t w[kWords];
  __device__ __forceinline__ float at(int k) const {
    if constexpr (DT == SV_BF16)
      return __uint_as_float((k & 1) ? (w[k >> 1] & 0xffff0000u) : (w[k >> 1] << 16));
    else
      return __uint_as_float(w[k]);
  }
};

// Elements [i0, i0 + n) of a row, n <= SEG (16-byte loads when the segment
// is whole and aligned).  Words past n hold `pad` (a bit pattern whose
// residual is 0), so no element needs a validity test later.
template <int DT, int SEG>
__device__ __forceinline__ void load_words(const void* row, int i0, int n, uint32_t pad,
                                           SegWords<DT, SEG>& s) {
  using E = Elt<DT>;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row) + (uintptr_t)i0 * E::kBytes;
  if (n == SEG && (a & 15u) == 0) {
    const u32x4* v = reinterpret_cast<const u32x4*>(a);
#pragma unroll
    for (int k = 0; k < SegWords<DT, SEG>::kWords / 4; ++k) {
      const u32x4 d = v[k];
      s.w[4 * k] = d.x;
      s.w[4 * k + 1] = d.y;
      s.w[4 * k + 2] = d.z;
      s.w[4 * k + 3] = d.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < SEG; ++k) {
      if constexpr (DT == SV_BF16) {
        const uint32_t h = k < n ? static_cast<const uint16_t*>(row)[i0 + k] : (pad & 0xffffu);
        s.w[k >> 1] = (k & 1) ? (s.w[k >> 1] | (h << 16)) : h;
      } else {
        s.w[k] = k < n ? static_cast<const uint32_t*>(row)[i0 + k] : pad;
      }
    }
  }
}

template <bool IS_PAIR, int TDT, int DDT, int SEG>
__device__ __forceinline__ float seg_resid(const SegWords<TDT, SEG>& P,
                                           const SegWords<DDT, SEG>& Q, const DrawDesc& d,
                                           bool probs, int k) {
  return IS_PAIR ? pair_resid(P.at(k), Q.at(k), d, probs) : single_resid(P.at(k), d);
}

// Residual sum of a whole segment with element ex (the excluded token, or
// -1) set to 0 before it is summed (fp32 within groups of 8, fp64 across
// them): the sum is exact to the rounding of the elements that remain, even
// when the excluded one held nearly all of the chunk.
template <bool IS_PAIR, int TDT, int DDT, int SEG>
__device__ __forceinline__ double seg_sum(const SegWords<TDT, SEG>& P,
                                          const SegWords<DDT, SEG>& Q, const DrawDesc& d,
                                          bool probs, int ex) {
  double seg = 0.0;
#pragma unroll
  for (int g = 0; g < SEG; g += 8) {
    float r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      r[k] = seg_resid<IS_PAIR>(P, Q, d, probs, g + k);
      r[k] = g + k == ex ? 0.f : r[k];
    }
    seg += (double)pairwise_sum(r);
  }
  return seg;
}

// Walk of a segment (q = mass before it, ex = excluded offset or -1): the
// offset of the first element whose running sum passes theta, else of the
// last element with positive residual (-1 if none).  Two levels keep the
// serial fp64 chain short: the group sums of seg_sum (recomputed bit for
// bit, the excluded element zeroed alike) find the group, then that group's
// 8 elements are walked.  *logit receives the target logit of the chosen
// element.
template <bool IS_PAIR, int TDT, int DDT, int SEG>
__device__ __forceinline__ int seg_walk(const SegWords<TDT, SEG>& P,
                                        const SegWords<DDT, SEG>& Q, const DrawDesc& d,
                                        bool probs, int ex, double q, double theta,
                                        float* logit) {
  constexpr int NG = SEG / 8;
  // (1) the group holding theta, else the last group with mass
  double L = q;
  int gstar = -1, glast = -1;
  double Lstar = 0.0, Llast = 0.0;  // mass before gstar / glast
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      r[k] = seg_resid<IS_PAIR>(P, Q, d, probs, 8 * g + k);
      r[k] = 8 * g + k == ex ? 0.f : r[k];
    }
    const double sg = (double)pairwise_sum(r);
    const bool has = sg > 0.0;
    const bool hit = gstar < 0 && has && L + sg > theta;
    Lstar = hit ? L : Lstar;
    gstar = hit ? g : gstar;
    Llast = has ? L : Llast;
    glast = has ? g : glast;
    L += sg;
    asm volatile("" : "+v"(gstar), "+v"(glast), "+v"(L), "+v"(Lstar), "+v"(Llast));
  }
  const int gw = gstar >= 0 ? gstar : glast;
  if (gw < 0) return -1;
  L = gstar >= 0 ? Lstar : Llast;
  // (2) walk that group: its words are picked out with selects (a dynamic
  // register index would go to scratch)
  SegWords<TDT, 8> P8;
  SegWords<DDT, 8> Q8;
#pragma unroll
  for (int i = 0; i < SegWords<TDT, 8>::kWords; ++i) {
    uint32_t v = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) v = g == gw ? P.w[g * SegWords<TDT, 8>::kWords + i] : v;
    P8.w[i] = v;
  }
  if (IS_PAIR) {
#pragma unroll
    for (int i = 0; i < SegWords<DDT, 8>::kWords; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int g = 0; g < NG; ++g) v = g == gw ? Q.w[g * SegWords<DDT, 8>::kWords + i] : v;
      Q8.w[i] = v;
    }
  }
  const int exg = ex - 8 * gw;
  int y = -1, lp = -1;
  float ly = 0.f, llp = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float r = seg_resid<IS_PAIR>(P8, Q8, d, probs, k);
    r = k != exg ? r : 0.f;
    L += (double)r;
    const bool pos = r > 0.f;
    const bool hit = y < 0 && pos && L > theta;
    y = hit ? k : y;
    ly = hit ? P8.at(k) : ly;
    lp = pos ? k : lp;
    llp = pos ? P8.at(k) : llp;
  }
  *logit = y < 0 ? llp : ly;
  const int yk = y < 0 ? lp : y;
  return yk < 0 ? -1 : 8 * gw + yk;
}

// PAIR = false: a batch with no draft rows (no residual pairs).
// A pair draw's residual part sums (wavefront 0, lane = chunk): their
// addresses need only the request, so the draw kernel loads them with the
// descriptor.
template <int TDT, int DDT>
struct ResidParts {
  double v[resid_split<TDT, DDT>()];
};

template <int TDT, int DDT, bool PAIR, int NT>
__device__ __forceinline__ void locate(const RunParams& p, int b, const DrawDesc& d,
                                       const ResidParts<TDT, DDT>& pre) {
  constexpr int SEG = seg_len<NT>();
  constexpr int kSplit = resid_split<TDT, DDT>();
  __shared__ int s_r0, s_rlen, s_kind, s_excl, s_y, s_lastseg;
  __shared__ double s_theta;
  __shared__ double s_woff[NT / 64];
  const int K = p.K, V = p.V, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const size_t trow = (size_t)b * (K + 1) + d.j;
  const void* prow = row_ptr(p.target, TDT, trow, V);
  const void* qrow = d.kind == kDrawPair ? row_ptr(p.draft, DDT, (size_t)b * K + d.j, V) : nullptr;
  const bool probs = p.draft_is_probs != 0;

  // (a) the range holding u * S: a chunk, or for a pair draw the part of a
  // chunk that one residual workgroup summed.  Single-row draws were placed
  // in their chunk by the decision kernel; pair draws scan the residual sums
  // here (wavefront 0, lane = chunk).
  if (d.cstar >= 0) {
    if (tid == 0) {
      s_r0 = d.cstar * p.chunk;
      s_rlen = min(V, s_r0 + p.chunk) - s_r0;
      s_theta = d.th;
      s_kind = d.kind;
      s_excl = d.x;
      s_y = INT32_MAX;
      s_lastseg = -1;
    }
  } else if (w == 0) {
    int kind = d.kind, excl = d.x;
    for (int attempt = 0; attempt < 2; ++attempt) {
      double mass = 0.0;
      double part[kSplit];  // a pair's part sums of chunk `lane`
#pragma unroll
      for (int h = 0; h < kSplit; ++h) part[h] = 0.0;
      if (lane < p.nchunk) {
        if (kind == kDrawPair) {
#pragma unroll
          for (int h = 0; h < kSplit; ++h) part[h] = pre.v[h];
          mass = part[0];
#pragma unroll
          for (int h = 1; h < kSplit; ++h) mass += part[h];
        } else {  // a pair draw's retry from p (single draws arrive placed)
          const Partial q = p.part[((size_t)b * (2 * K + 1) + d.j) * p.nchunk + lane];
          if (q.z != 0.0) mass = q.z * exp2_diff(d.ref_p, ref_of(q.m, d.c));
        }
        if (!(mass > 0.0)) mass = 0.0;
      }
      const double incl = wave_incl_scan(mass, lane);
      const double S = lane_f64(incl, 63);
      if (!(S > 0.0) && attempt == 0) {  // no residual mass: draw from p
        if (lane == 0) atomicOr(p.flags, SV_DEVERR_ZERO_RESIDUAL);
        kind = kDrawSingle;
        excl = -1;
        continue;
      }
      const double theta = d.u * S;
      double before = lane_before(incl);
      if (lane == 0) before = 0.0;
      const bool hit = mass > 0.0 && before <= theta && theta < incl;
      const uint64_t hits = __ballot(hit);
      int cstar;
      double th;
      if (hits) {
        const int src = (int)__builtin_ctzll(hits);
        cstar = src;
        th = theta - lane_f64(before, src);
      } else {  // rounding left theta at or past the total: last chunk with mass
        const uint64_t has = __ballot(mass > 0.0);
        cstar = has ? 63 - (int)__builtin_clzll(has) : 0;
        th = __builtin_inf();
        if (lane == 0) atomicOr(p.flags, SV_DEVERR_DRAW_ROUNDING);
      }
      int r0 = cstar * p.chunk, rlen = min(V, r0 + p.chunk) - r0;
      if (kind == kDrawPair && kSplit > 1) {
        // the part: running sums in the order that gave the chunk's mass, so
        // the last one equals it; the parts' bounds are the residual pass's
        const int plen = ((rlen + kSplit - 1) / kSplit + 63) & ~63;
        int hs = -1, hlast = 0;
        double c = 0.0, c_before = 0.0;
#pragma unroll
        for (int h = 0; h < kSplit; ++h) {
          const double v = lane_f64(part[h], cstar);
          const double cn = h == 0 ? v : c + v;
          if (v > 0.0) hlast = h;
          if (hs < 0 && th < cn) {
            hs = h;
            c_before = c;
          }
          c = cn;
        }
        if (hs < 0) {  // theta at or past the chunk's last running sum
          hs = hlast;
          if (th != __builtin_inf() && lane == 0) atomicOr(p.flags, SV_DEVERR_DRAW_ROUNDING);
          th = __builtin_inf();
        } else {
          th -= c_before;
        }
        r0 += min(rlen, hs * plen);
        rlen = min(plen, max(0, rlen - hs * plen));
      }
      if (lane == 0) {
        s_r0 = r0;
        s_rlen = rlen;
        s_theta = th;
        s_kind = kind;
        s_excl = excl;
        s_y = INT32_MAX;
        s_lastseg = -1;
      }
      break;
    }
  }
  __syncthreads();

  // (b) thread t owns range elements [t SEG, t SEG + SEG): their raw words
  // stay in registers, the residual sum is taken in fp64
  const int kind = s_kind, excl = s_excl;
  const int c0 = s_r0, len = s_rlen;
  const int i0 = tid * SEG;
  const int nseg = max(0, min(SEG, len - i0));
  const bool pair = PAIR && kind == kDrawPair;
  SegWords<TDT, SEG> P;
  SegWords<DDT, SEG> Q;
  // padding with residual 0: a -inf logit, or probability 0
  const uint32_t pad_p = Elt<TDT>::kBytes == 2 ? 0xff80ff80u : 0xff800000u;
  const uint32_t pad_q = probs ? 0u : (Elt<DDT>::kBytes == 2 ? 0xff80ff80u : 0xff800000u);
  load_words<TDT>(prow, c0 + min(i0, len), nseg, pad_p, P);
  if (pair) load_words<DDT>(qrow, c0 + min(i0, len), nseg, pad_q, Q);
  int ex = excl >= 0 ? excl - c0 - i0 : -1;  // excluded token in the segment
  if (ex >= nseg) ex = -1;
  double seg = pair ? seg_sum<true>(P, Q, d, probs, ex) : seg_sum<false>(P, Q, d, probs, ex);
  if (!(seg > 0.0)) seg = 0.0;

  // (c) exclusive scan of the segment sums
  const double incl = wave_incl_scan(seg, lane);
  if (lane == 63) s_woff[w] = incl;
  double q = lane_before(incl);
  if (lane == 0) q = 0.0;
  // the last segment with mass: one atomic per wavefront, not per thread
  const uint64_t has = __ballot(seg > 0.0);
  if (lane == 0 && has != 0) atomicMax(&s_lastseg, w * 64 + 63 - (int)__builtin_clzll(has));
  __syncthreads();
  for (int k = 0; k < w; ++k) q += s_woff[k];

  // (d) the segment holding theta walks its registers; if rounding left
  // theta past every segment, the last segment with mass takes its last
  // positive element
  const double theta = s_theta;
  const bool mine = seg > 0.0 && q <= theta && theta < q + seg;
  const bool past = s_lastseg == tid && !(theta < q + seg);
  int ymine = INT32_MAX;
  float lmine = 0.f;  // target logit at ymine
  if (mine || past) {
    // recompute the residuals rather than keep SEG floats live across the
    // barrier: the empty asm hides the first computation from CSE
#pragma unroll
    for (int k = 0; k < SegWords<TDT, SEG>::kWords; ++k) asm volatile("" : "+v"(P.w[k]));
    if (pair) {
#pragma unroll
      for (int k = 0; k < SegWords<DDT, SEG>::kWords; ++k) asm volatile("" : "+v"(Q.w[k]));
    }
    const double th = mine ? theta : __builtin_inf();
    const int yo = pair ? seg_walk<true>(P, Q, d, probs, ex, q, th, &lmine)
                        : seg_walk<false>(P, Q, d, probs, ex, q, th, &lmine);
    if (yo >= 0) ymine = i0 + yo;
    if (mine) atomicMin(&s_y, ymine);
  }
  __syncthreads();
  int y = s_y;
  bool writer = y != INT32_MAX && y == ymine;  // segments are disjoint: one thread
  if (y == INT32_MAX) {  // theta past the chunk's recomputed total
    writer = s_lastseg >= 0 ? s_lastseg == tid : tid == 0;
    const bool have = s_lastseg >= 0 && ymine != INT32_MAX;
    // no element with mass at all (only reachable when every element left
    // underflows at the row's reference): a token of the range that is not
    // the excluded draft
    const int y0 = (c0 == excl && len > 1) ? 1 : 0;
    y = have ? ymine : y0;
    if (!have) lmine = Elt<TDT>::at(prow, c0 + y0);
    if (writer && theta != __builtin_inf()) atomicOr(p.flags, SV_DEVERR_DRAW_ROUNDING);
  }
  if (writer) {
    p.out_tokens[(size_t)b * (K + 1) + d.j] = c0 + y;
    if (p.out_q != nullptr)  // sampler: q(x) of the drawn token
      p.out_q[b] = (float)(exp2((double)lmine * (double)d.c + (double)d.ref_p) / d.z_p);
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: decisions (one wavefront per request)
// ---------------------------------------------------------------------------
template <int TDT, int DDT>
__global__ __launch_bounds__(64) void k_decide(const RunParams p) {
  __shared__ DrawDesc s_d;
  const int b = blockIdx.x;
  decide_request<TDT, DDT>(p, b, req_info(p, b), true, &s_d);
}

// ---------------------------------------------------------------------------
// Kernel 3: residual chunk sums of requests rejected on a probabilistic draft
// ---------------------------------------------------------------------------
template <int TDT, int DDT>
__global__ __launch_bounds__(kThreads) void k_resid(
    const RunParams p) {
  __shared__ double ldsd[kThreads / 64];
  constexpr int kSplit = resid_split<TDT, DDT>();
  const int bid = blockIdx.x;
  const int rb = bid / (p.nchunk * kSplit), part = bid - rb * (p.nchunk * kSplit);
  const int chunk = part / kSplit, h = part - chunk * kSplit;
  const int b = p.B - 1 - rb;  // last request first (measured the same as first first)
  const DrawDesc d = p.desc[b];
  if (d.kind != kDrawPair) return;
  const int K = p.K, V = p.V;
  const void* prow = row_ptr(p.target, TDT, (size_t)b * (K + 1) + d.j, V);
  const void* qrow = row_ptr(p.draft, DDT, (size_t)b * K + d.j, V);
  // part h of the chunk: a multiple of 64 elements, so every part starts on
  // a 16-byte boundary when the chunk does
  const int ch0 = chunk * p.chunk, ch1 = min(V, ch0 + p.chunk);
  const int plen = ((ch1 - ch0 + kSplit - 1) / kSplit + 63) & ~63;
  const int c0 = min(ch1, ch0 + h * plen), c1 = min(ch1, c0 + plen);
  const double s = pair_chunk_sum<TDT, DDT>(prow, qrow, c0, c1, d, p.draft_is_probs != 0, ldsd);
  if (threadIdx.x == 0) p.rsum[((size_t)b * p.nchunk + chunk) * kSplit + h] = s;
}

// ---------------------------------------------------------------------------
// Kernel 4: the draw of every sampling request
// ---------------------------------------------------------------------------
template <int TDT, int DDT, bool PAIR, int NT>
__global__ __launch_bounds__(NT) void k_locate(const RunParams p) {
  constexpr int kSplit = resid_split<TDT, DDT>();
  const int b = blockIdx.x, tid = threadIdx.x;
  const DrawDesc d = p.desc[b];
  ResidParts<TDT, DDT> pre;
#pragma unroll
  for (int h = 0; h < kSplit; ++h) pre.v[h] = 0.0;
  if (PAIR && tid < 64 && tid < p.nchunk) {  // read by pair draws only
    const double* rs = p.rsum + ((size_t)b * p.nchunk + tid) * kSplit;
#pragma unroll
    for (int h = 0; h < kSplit; ++h) pre.v[h] = rs[h];
  }
  if (d.kind == kDrawNone) return;  // uniform
  locate<TDT, DDT, PAIR, NT>(p, b, d, pre);
}

// Draft sampler: the draw of one row without a decision kernel.  Wavefront 0
// folds the row's chunk partials (lane = chunk) into the row max and total
// and places u * S in its chunk; the workgroup then walks that chunk.
template <int DT, int NT>
__global__ __launch_bounds__(NT) void k_sample(const RunParams p) {
  __shared__ DrawDesc s_d;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  // the row's partials are loaded with the request's count and temperature
  // (a row past the count wastes one small load)
  Partial q{kNegInf, INT32_MAX, 0.0};
  if (tid < 64 && lane < p.nchunk) q = p.part[(size_t)b * p.nchunk + lane];
  const ReqInfo ri = req_info(p, b);
  if (tid == 0 && ri.bad_n && ri.rj == 0) atomicOr(p.flags, SV_DEVERR_BAD_NUM_DRAFTS);
  if (!ri.active) {  // row past the request's draft count
    if (tid == 0) {
      p.out_tokens[b] = -1;
      if (p.out_q != nullptr) p.out_q[b] = __builtin_nanf("");
    }
    return;
  }
  if (tid < 64) {
    if (!ri.sampling) {  // greedy: the lowest index of the row max
      float m = q.m;
      int i = lane < p.nchunk ? q.idx : INT32_MAX;
      wave_argmax(m, i);
      if (lane == 0) {
        p.out_tokens[b] = i == INT32_MAX ? 0 : i;
        if (p.out_q != nullptr) p.out_q[b] = 1.f;
      }
    } else {
      const float c = temp_scale(ri.T);
      const float ref = ref_of(wave_max(q.m), c);
      double mass = 0.0;
      if (lane < p.nchunk && q.z != 0.0) mass = q.z * exp2_diff(ref, ref_of(q.m, c));
      const double incl = wave_incl_scan(mass, lane);
      const double S = lane_f64(incl, 63);
      const double u = draft_uniform(p.seed, p.offset, p.b_base + ri.rb, ri.rj);
      const double theta = u * S;
      double before = lane_before(incl);
      if (lane == 0) before = 0.0;
      const uint64_t hits = __ballot(mass > 0.0 && before <= theta && theta < incl);
      int cstar;
      double th;
      if (hits) {
        cstar = (int)__builtin_ctzll(hits);
        th = theta - lane_f64(before, cstar);
      } else {  // rounding left theta at or past the total: last chunk with mass
        const uint64_t has = __ballot(mass > 0.0);
        cstar = has ? 63 - (int)__builtin_clzll(has) : 0;
        th = __builtin_inf();
        if (lane == 0) atomicOr(p.flags, SV_DEVERR_DRAW_ROUNDING);
      }
      if (lane == 0) {
        DrawDesc d{};
        d.kind = kDrawSingle;
        d.j = 0;
        d.x = -1;
        d.cstar = cstar;
        d.c = c;
        d.ref_p = ref;
        d.z_p = S;
        d.u = u;
        d.th = th;
        s_d = d;
      }
    }
  }
  if (!ri.sampling) return;  // uniform across the workgroup
  __syncthreads();
  locate<DT, DT, false, NT>(p, b, s_d, ResidParts<DT, DT>{});
}

// Tuning knob: batches of at most this many draws use 1024-thread draws.
// Verify draws at 512 requests: 11.5 us against 12.5 for 512 threads; the
// sampler's whole-chunk draws at 768 rows: even.
#ifndef SV_LOC_WIDE_MAX_DRAWS
#define SV_LOC_WIDE_MAX_DRAWS 768
#endif
constexpr int kLocWideMaxDraws = SV_LOC_WIDE_MAX_DRAWS;
// Tuning knob: batches of at most this many draws (and more than the above)
// use 512-thread draws; larger ones 256.  At 962 sampler rows 256 threads
// take 17.1 us, 512 about the same and 1024 20.7 us.
#ifndef SV_LOC_MID_MAX_DRAWS
#define SV_LOC_MID_MAX_DRAWS 896
#endif
constexpr int kLocMidMaxDraws = SV_LOC_MID_MAX_DRAWS;

template <int TDT, int DDT, bool PAIR>
void launch_locate(const RunParams& p, hipStream_t s) {
  if (p.B <= kLocWideMaxDraws)
    hipLaunchKernelGGL((k_locate<TDT, DDT, PAIR, 1024>), dim3(p.B), dim3(1024), 0, s, p);
  else if (p.B <= kLocMidMaxDraws)
    hipLaunchKernelGGL((k_locate<TDT, DDT, PAIR, 512>), dim3(p.B), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((k_locate<TDT, DDT, PAIR, 256>), dim3(p.B), dim3(256), 0, s, p);
}

}  // namespace

bool kernel_launched(int k, const RunParams& p) {
  if (k == kKernelDecide) return p.sample_k == 0;
  if (k == kKernelResid) return p.has_draft != 0;
  return true;
}

namespace {

// Dynamic LDS of a stats launch: a request that lets at most the cap's
// number of workgroups share a compute unit's LDS (1 KB is left for the
// kernel's static LDS and the allocation granularity).  0 means no cap.
size_t stats_lds_bytes(const RunParams& p, int tdt, int lds_per_cu) {
  const int cap = (p.typical && p.top_k > 0) ? 0
                  : tdt == SV_F32            ? SV_STATS_WG_CAP_F32
                                             : SV_STATS_WG_CAP_BF16;
  if (cap <= 0 || lds_per_cu <= 0) return 0;
  const int bytes = lds_per_cu / cap - 1024;
  return bytes > lds_per_cu / (cap + 1) ? (size_t)bytes : 0;
}

template <int TDT, int DDT>
void launch_one(int k, const RunParams& p, int lds_per_cu, hipStream_t s) {
  switch (k) {
    case kKernelStats: {
      const uint64_t g = (uint64_t)p.B * stats_slots(p) * p.nchunk;
      hipLaunchKernelGGL((k_stats<TDT, DDT>), dim3((unsigned)g), dim3(kThreads),
                         stats_lds_bytes(p, TDT, lds_per_cu), s, p);
      break;
    }
    case kKernelDecide:
      hipLaunchKernelGGL((k_decide<TDT, DDT>), dim3(p.B), dim3(64), 0, s, p);
      break;
    case kKernelResid:
      hipLaunchKernelGGL((k_resid<TDT, DDT>),
                         dim3((unsigned)((uint64_t)p.B * p.nchunk * resid_split<TDT, DDT>())),
                         dim3(kThreads),
                         0, s, p);
      break;
    default:
      if (p.sample_k > 0) {
        if (p.B <= kLocWideMaxDraws)
          hipLaunchKernelGGL((k_sample<TDT, 1024>), dim3(p.B), dim3(1024), 0, s, p);
        else if (p.B <= kLocMidMaxDraws)
          hipLaunchKernelGGL((k_sample<TDT, 512>), dim3(p.B), dim3(512), 0, s, p);
        else
          hipLaunchKernelGGL((k_sample<TDT, 256>), dim3(p.B), dim3(256), 0, s, p);
      } else if (p.has_draft) {
        launch_locate<TDT, DDT, true>(p, s);
      } else {
        launch_locate<TDT, DDT, false>(p, s);
      }
      break;
  }
}

}  // namespace

hipError_t launch_kernel(int k, const RunParams& p, int tdt, int ddt, int lds_per_cu,
                         hipStream_t s) {
  if (!kernel_launched(k, p)) return hipSuccess;
  if (tdt == SV_F32 && ddt == SV_F32) launch_one<SV_F32, SV_F32>(k, p, lds_per_cu, s);
  else if (tdt == SV_F32 && ddt == SV_BF16) launch_one<SV_F32, SV_BF16>(k, p, lds_per_cu, s);
  else if (tdt == SV_BF16 && ddt == SV_F32) launch_one<SV_BF16, SV_F32>(k, p, lds_per_cu, s);
  else launch_one<SV_BF16, SV_BF16>(k, p, lds_per_cu, s);
  return hipGetLastError();
}

const char* kernel_name(int i) {
  static const char* names[kNumKernels] = {"stats", "decide", "resid", "locate"};
  return (i >= 0 && i < kNumKernels) ? names[i] : nullptr;
}

}  // namespace sv
