// Token-tree verification on gfx950, and its C entry point.
//
// Source: "投机采样" (razer666.cn), section 验证阶段的策略 / 验证方案: draft
// sequences that share prefixes are merged into a token tree and the target
// scores every node at once.  The multi-branch rule is the page's chain rule
// applied child by child (multi-step speculative sampling; the header of
// include/spec_verify.h states it).
//
// One 1024-thread workgroup per request walks its tree and streams only the
// rows of the nodes it visits:
//   - at node v, one pass over target row v (and draft row v) gives the row
//     max and normalizer (or the lowest argmax for greedy requests);
//   - the children of v are tested in index order; after k rejections the
//     law is max(0, p - c_k q) / Z_k, and each further sibling test needs
//     Z_k, one more pass over the row pair;
//   - where the walk stops, the emitted token is drawn by inverse CDF: one
//     pass sums the law per slot of 64 vectors, a workgroup scan over the
//     slot sums finds the slot holding u * S, and one wavefront re-reads that
//     slot to find the element.
// Row passes issue 160-224 KiB of 16-byte loads per workgroup before using any
// (one round trip per round), through buffer resources, so the loads of a
// round cost no address registers and no branches, and no round waits at a
// workgroup barrier.  The walk is sequential per request; requests run in
// parallel, one per compute unit at the usual batch sizes.  A walk left
// running alone is bound by its compute unit's arithmetic (~6 VALU slots per
// element) more than by memory, so the inner loops keep per-element work to
// the minimum: uniform tests for the row's end, fp32 sums per round.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / 64;
constexpr int kMaxNodes = SPEC_TREE_MAX_NODES;

struct RowStats {
  float m;     // row max
  float ref;   // exponent reference ref_of(m, c)
  double z;    // sum of exp2(l c + ref)
  int arg;     // lowest index of the max (greedy)
};

// A row is a scalar head [0, v0) up to the first 16-byte boundary, nvec
// vectors from v0 and a scalar tail [t0, V) (chunk_geo over the whole row).
// A pass takes the vectors in rounds: every thread issues all its loads of a
// round (vectors b0 + u * 1024 + tid) before it uses any, so one round trip
// to memory covers kRowVecs * 16 KiB of a single row (160 KiB), or kPairVecs
// * 16 KiB of each row of a pair (224 KiB).  The 10 or 14 vectors take 40 or
// 56 of the 128 registers a thread of a 1024-thread workgroup has; the
// walk's own state takes most of the rest.
constexpr int kRowVecs = 10;
constexpr int kPairVecs = 7;
constexpr int kRound = kTreeThreads;  // vectors per unroll step of a round

// Draw slots: slot 0 is the head, slot 1 + k the 64 vectors [64 k, 64 k + 64)
// (one wavefront's share of one unroll step), the last slot the tail.
__device__ __forceinline__ int num_slots(const Geo& g) { return (g.nvec + 63) / 64 + 2; }

__device__ __forceinline__ const u32x4* vec_base(const void* row, const Geo& g, int bytes) {
  return reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + (size_t)g.v0 * bytes);
}

// The vectors of a row as a buffer resource (loads past the row return 0).
__device__ __forceinline__ VecBuf vec_buf(const void* row, const Geo& g, int bytes) {
  return make_vec_buf(vec_base(row, g, bytes), (uint32_t)g.nvec * 16u);
}

// Vector b0 + tid + u * kRound of the row, or 0 past its end.
__device__ __forceinline__ u32x4 vec_load(const VecBuf& vb, int b0, int u, int tid) {
  return buf_load<false>(vb, (uint32_t)(b0 + u * kRound + tid) * 16u);
}

// The thread index, hidden from loop-invariant code motion: each pass
// recomputes what it derives from it (per-vector masks, slot indices) rather
// than the compiler hoisting all of them out of the walk, where they would
// hold registers through every pass.
__device__ __forceinline__ int pass_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Statistics of one row (whole workgroup).  Sampling rows take each round in
// two phases per wavefront: the wavefront's max of the round first, which
// fixes one exponent reference for its 64 lanes, then the sums of
// exp2(l c + ref) with no per-element max test.  A later round that raises a
// wavefront's max rescales its sums once.  No round needs a workgroup
// barrier, so the wavefronts drift apart and one's loads overlap another's
// arithmetic; the wavefronts' sums meet once, at the row's reference.
// Greedy rows keep the max and its lowest index.
template <int DT>
__device__ __forceinline__ RowStats row_stats(const void* row, int V, bool sampling, float c,
                                              float* ldsf, double* ldsd, int* ldsi) {
  using E = Elt<DT>;
  constexpr int U = kRowVecs;
  const int tid = pass_tid();
  const Geo g = chunk_geo<DT>(row, 0, V);
  const VecBuf vb = vec_buf(row, g, E::kBytes);
  // each thread's scalar elements: one of the head, one of the tail
  const bool has_h = tid < g.v0, has_t = g.t0 + tid < V;
  const float hx = has_h ? E::at(row, tid) : kNegInf;
  const float tx = has_t ? E::at(row, g.t0 + tid) : kNegInf;
  RowStats st;
  if (!sampling) {
    AmAcc a{kNegInf, INT32_MAX};
    if (has_h) {
      const float x[1] = {hx};
      const int ix[1] = {tid};
      am_tile(a, x, ix);
    }
    for (int b0 = 0; b0 < g.nvec; b0 += U * kRound) {
      u32x4 d[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b0 + u * kRound + tid < g.nvec) d[u] = vec_load(vb, b0, u, tid);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int vi = b0 + u * kRound + tid;
        if (vi < g.nvec) {
          float x[E::kVec];
          int ix[E::kVec];
          E::unpack(d[u], x);
#pragma unroll
          for (int k = 0; k < E::kVec; ++k) ix[k] = g.v0 + vi * E::kVec + k;
          am_tile(a, x, ix);
        }
      }
    }
    if (has_t) {
      const float x[1] = {tx};
      const int ix[1] = {g.t0 + tid};
      am_tile(a, x, ix);
    }
    block_argmax<kTreeThreads>(a.M, a.I, ldsf, ldsi);
    st.m = a.M;
    st.arg = a.I == INT32_MAX ? 0 : a.I;
    st.ref = 0.f;
    st.z = 0.0;
    return st;
  }
  float Mw = kNegInf, Rw = 0.f;  // the wavefront's max and reference so far
  double S = 0.0;                // this thread's sum, relative to Rw
  for (int b0 = 0; b0 == 0 || b0 < g.nvec; b0 += U * kRound) {
    u32x4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = vec_load(vb, b0, u, tid);
    // vectors past the row are skipped by a test that is uniform in all but
    // one wavefront of the row (the loads there returned 0)
    float t = b0 == 0 ? fmaxf(hx, tx) : kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b0 + u * kRound + tid < g.nvec) {
        float x[E::kVec];
        E::unpack(d[u], x);
#pragma unroll
        for (int k = 0; k < E::kVec; ++k) t = fmaxf(t, x[k]);
      }
    }
    const float wm = wave_max(t);
    if (wm > Mw) {  // uniform across the wavefront
      const float rn = ref_of(wm, c);
      if (Mw != kNegInf) S *= (double)fast_exp2(rn - Rw);
      Rw = rn;
      Mw = wm;
    }
    // the round's sum in fp32, added to the fp64 total once
    float sr = b0 == 0 ? fast_exp2(fmaf(hx, c, Rw)) + fast_exp2(fmaf(tx, c, Rw)) : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b0 + u * kRound + tid < g.nvec) {
        // unpack again rather than keep the floats live: the empty asm hides
        // the first unpack from common-subexpression elimination
        u32x4 wv = d[u];
        asm volatile("" : "+v"(wv));
        float e[E::kVec];
        E::unpack(wv, e);
#pragma unroll
        for (int k = 0; k < E::kVec; ++k) e[k] = fast_exp2(fmaf(e[k], c, Rw));
        sr += pairwise_sum(e);
        asm volatile("" : "+v"(sr));  // fold in order: no sums wait in registers
      }
    }
    S += (double)sr;
  }
  const float M = block_max<kTreeThreads>(Mw, ldsf);
  const float R = ref_of(M, c);
  const double f = Mw == kNegInf ? 0.0 : (Mw == M ? 1.0 : exp2_diff(R, Rw));
  st.m = M;
  st.ref = R;
  st.z = block_sum<kTreeThreads>(S * f, ldsd);
  st.arg = 0;
  return st;
}

// The law the stop node draws from, per element (unnormalized, relative to
// the target row's reference): p~ = exp2(l_p c + ref_p); for a pair,
// max(0, p~ - kappa q~) with q~ = exp2(l_q c + ref_q) (or q itself for
// probability drafts) and kappa split in two floats.
struct Law {
  bool pair;
  float c, ref_p, ref_q, kap_hi, kap_lo;
  bool probs;
};

__device__ __forceinline__ float law_of(const Law& L, float lp, float lq) {
  const float pt = fast_exp2(fmaf(lp, L.c, L.ref_p));
  if (!L.pair) return pt;
  const float qt = L.probs ? lq : fast_exp2(fmaf(lq, L.c, L.ref_q));
  float r = fmaf(-qt, L.kap_hi, pt);
  r = fmaf(-qt, L.kap_lo, r);
  return r > 0.f ? r : 0.f;
}

template <int TDT, int DDT>
__device__ __forceinline__ float law_at(const Law& L, const void* prow, const void* qrow, int i) {
  return law_of(L, Elt<TDT>::at(prow, i), L.pair ? Elt<DDT>::at(qrow, i) : 0.f);
}

// The law at the kVec elements of target vector vi.  The draft row's
// elements come by one vector load when both rows have the same element
// type and alignment (qvec), else element by element.
template <int TDT, int DDT>
__device__ __forceinline__ void law_vec(const Law& L, const void* prow, const void* qrow,
                                        const Geo& g, int vi, bool qvec, float* r) {
  using EP = Elt<TDT>;
  float lp[EP::kVec], lq[EP::kVec];
  EP::unpack(vec_base(prow, g, EP::kBytes)[vi], lp);
  if (L.pair) {
    if constexpr (TDT == DDT) {
      if (qvec) {
        EP::unpack(vec_base(qrow, g, EP::kBytes)[vi], lq);
      } else {
#pragma unroll
        for (int k = 0; k < EP::kVec; ++k) lq[k] = Elt<DDT>::at(qrow, g.v0 + vi * EP::kVec + k);
      }
    } else {
#pragma unroll
      for (int k = 0; k < EP::kVec; ++k) lq[k] = Elt<DDT>::at(qrow, g.v0 + vi * EP::kVec + k);
    }
  }
#pragma unroll
  for (int k = 0; k < EP::kVec; ++k) r[k] = law_of(L, lp[k], L.pair ? lq[k] : 0.f);
}

__device__ __forceinline__ bool same_alignment(const void* a, const void* b) {
  return ((reinterpret_cast<uintptr_t>(a) ^ reinterpret_cast<uintptr_t>(b)) & 15u) == 0;
}

// One pass over the law of a row (and, for a pair, of its draft row): calls
// f(b, s) once per unroll step of every round, convergently, with s the
// thread's fp32 sum of the law over its vector b + tid (0 past the vectors).
// When the draft row has the target's element type and 16-byte alignment,
// both rows' vectors of a round are loaded together, kPairVecs each (or
// kRowVecs of a single row); otherwise the draft elements are loaded one by
// one, a vector of the target at a time.
template <int TDT, int DDT, typename F>
__device__ __forceinline__ void law_pass(const Law& L, const void* prow, const void* qrow,
                                         const Geo& g, F&& f) {
  using EP = Elt<TDT>;
  constexpr int KV = EP::kVec;
  const int tid = pass_tid();
  const VecBuf pb = vec_buf(prow, g, EP::kBytes);
  if (!L.pair) {
    for (int b0 = 0; b0 < g.nvec; b0 += kRowVecs * kRound) {
      u32x4 d[kRowVecs];
#pragma unroll
      for (int u = 0; u < kRowVecs; ++u) d[u] = vec_load(pb, b0, u, tid);
#pragma unroll
      for (int u = 0; u < kRowVecs; ++u) {
        float sv = 0.f;  // vectors past the row: a test uniform in all but one wavefront
        if (b0 + u * kRound + tid < g.nvec) {
          float r[KV];
          EP::unpack(d[u], r);
#pragma unroll
          for (int k = 0; k < KV; ++k) r[k] = law_of(L, r[k], 0.f);
          sv = pairwise_sum(r);
        }
        f(b0 + u * kRound, sv);
      }
    }
    return;
  }
  if constexpr (TDT == DDT) {
    if (same_alignment(prow, qrow)) {
      const VecBuf qb = vec_buf(qrow, g, EP::kBytes);
      for (int b0 = 0; b0 < g.nvec; b0 += kPairVecs * kRound) {
        u32x4 dp[kPairVecs], dq[kPairVecs];
#pragma unroll
        for (int u = 0; u < kPairVecs; ++u) {
          dp[u] = vec_load(pb, b0, u, tid);
          dq[u] = vec_load(qb, b0, u, tid);
        }
#pragma unroll
        for (int u = 0; u < kPairVecs; ++u) {
          float sv = 0.f;
          if (b0 + u * kRound + tid < g.nvec) {
            float lp[KV], lq[KV], r[KV];
            EP::unpack(dp[u], lp);
            EP::unpack(dq[u], lq);
#pragma unroll
            for (int k = 0; k < KV; ++k) r[k] = law_of(L, lp[k], lq[k]);
            sv = pairwise_sum(r);
          }
          f(b0 + u * kRound, sv);
        }
      }
      return;
    }
  }
  for (int b0 = 0; b0 < g.nvec; b0 += kRound) {
    float sv = 0.f;
    if (b0 + tid < g.nvec) {
      float r[KV];
      law_vec<TDT, DDT>(L, prow, qrow, g, b0 + tid, false, r);
      sv = pairwise_sum(r);
    }
    f(b0, sv);
  }
}

// Sum of the law over the row (whole workgroup, fp64 across vectors).
template <int TDT, int DDT>
__device__ __forceinline__ double law_sum(const Law& L, const void* prow, const void* qrow, int V, double* ldsd) {
  const int tid = pass_tid();
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  double acc = 0.0;
  if (tid < g.v0) acc += (double)law_at<TDT, DDT>(L, prow, qrow, tid);
  // eight vector sums in fp32, then one fp64 add (every thread makes the
  // same number of calls, so the flush is uniform)
  float part = 0.f;
  int nv = 0;
  law_pass<TDT, DDT>(L, prow, qrow, g, [&](int, float sv) {
    part += sv;
    asm volatile("" : "+v"(part));  // fold in order: no sums wait in registers
    if (++nv == 8) {
      acc += (double)part;
      part = 0.f;
      nv = 0;
    }
  });
  acc += (double)part;
  if (g.t0 + tid < V) acc += (double)law_at<TDT, DDT>(L, prow, qrow, g.t0 + tid);
  return block_sum<kTreeThreads>(acc, ldsd);
}

// The law's sums per draw slot, by one pass over the row (or row pair).
template <int TDT, int DDT>
__device__ __forceinline__ void slot_pass(const Law& L, const void* prow, const void* qrow, int V,
                          double* s_slot) {
  const int tid = pass_tid(), lane = tid & 63, w = tid >> 6;
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  const int npieces = (g.nvec + 63) / 64, nslot = npieces + 2;
  law_pass<TDT, DDT>(L, prow, qrow, g, [&](int b, float sv) {
    const int piece = b / 64 + w;
    const double ws = (double)wave_sum_f32(sv);  // 64 vector sums: fp32 is ample
    if (lane == 0 && piece < npieces) s_slot[1 + piece] = ws;
  });
  if (w == 0) {
    const double h = wave_sum(lane < g.v0 ? (double)law_at<TDT, DDT>(L, prow, qrow, lane) : 0.0);
    const double t =
        wave_sum(g.t0 + lane < V ? (double)law_at<TDT, DDT>(L, prow, qrow, g.t0 + lane) : 0.0);
    if (lane == 0) {
      s_slot[0] = h;
      s_slot[nslot - 1] = t;
    }
  }
}

__device__ __forceinline__ bool excluded(const int* ex, int nex, int i) {
  for (int k = 0; k < nex; ++k)
    if (ex[k] == i) return true;
  return false;
}

// The draw slot holding element i of the row.
__device__ __forceinline__ int slot_of(const Geo& g, int nslot, int kv, int i) {
  return i < g.v0 ? 0 : (i >= g.t0 ? nslot - 1 : 1 + (i - g.v0) / kv / 64);
}

// Inverse-CDF draw from the law with uniform u (whole workgroup), given its
// sums per draw slot in s_slot (written by slot_pass); the
// tokens in ex[0..nex) are removed.  A workgroup scan over the slot sums
// finds the slot holding u * S, and wavefront 0 re-reads only that slot (one
// vector per lane) to find the element.  Returns the token; *rounding is set
// if u * S fell past the recomputed total, *empty if the law is 0.  A slot
// that holds removed tokens is summed again with them zeroed (not reduced
// by their values: a removed sibling can hold nearly all of the slot, and
// the difference of two rounded sums would leave a residue far above the
// mass that remains).
template <int TDT, int DDT>
__device__ __forceinline__ int draw_from_slots(const Law& L, const void* prow, const void* qrow, int V,
                               const int* ex, int nex, double u, double* s_slot, double* s_woff,
                               int* s_sel, double* s_th, bool* rounding, bool* empty) {
  using EP = Elt<TDT>;
  constexpr int KV = EP::kVec;
  const int tid = pass_tid(), lane = tid & 63, w = tid >> 6;
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  const bool qvec = L.pair && same_alignment(prow, qrow);
  const int nslot = num_slots(g);
  __syncthreads();
  if (w == 0) {  // slots holding removed tokens, summed again without them
    for (int k = 0; k < nex; ++k) {  // uniform over the wavefront
      const int sl = slot_of(g, nslot, KV, ex[k]);
      bool seen = false;
      for (int k2 = 0; k2 < k; ++k2) seen = seen || slot_of(g, nslot, KV, ex[k2]) == sl;
      if (seen) continue;
      float r[KV];
      int base;
#pragma unroll
      for (int j = 0; j < KV; ++j) r[j] = 0.f;
      if (sl == 0 || sl == nslot - 1) {
        base = sl == 0 ? lane : g.t0 + lane;
        if (sl == 0 ? lane < g.v0 : base < V) r[0] = law_at<TDT, DDT>(L, prow, qrow, base);
      } else {
        const int vi = (sl - 1) * 64 + lane;
        base = g.v0 + vi * KV;
        if (vi < g.nvec) law_vec<TDT, DDT>(L, prow, qrow, g, vi, qvec, r);
      }
      for (int e = 0; e < nex; ++e) {  // a select per element, no early exit
        const int t = ex[e];
#pragma unroll
        for (int j = 0; j < KV; ++j) r[j] = t == base + j ? 0.f : r[j];
      }
      // the same sums slot_pass makes: a scalar per lane for the head and
      // tail slots, fp32 vector sums otherwise
      const double sum = (sl == 0 || sl == nslot - 1) ? wave_sum((double)r[0])
                                                       : (double)wave_sum_f32(pairwise_sum(r));
      if (lane == 0) s_slot[sl] = sum;
    }
    if (lane == 0) *s_sel = -1;
  }
  __syncthreads();

  // (2) scan of the slot sums: thread t takes slots [t sp, t sp + sp)
  const int sp = (nslot + kTreeThreads - 1) / kTreeThreads;
  const int k0 = min(nslot, tid * sp), k1 = min(nslot, k0 + sp);
  double loc = 0.0;
  int lastpos = -1;
  for (int k = k0; k < k1; ++k) {
    loc += s_slot[k];
    if (s_slot[k] > 0.0) lastpos = k;
  }
  const double incl = wave_incl_scan(loc, lane);
  if (lane == 63) s_woff[w] = incl;
  double q = lane_before(incl);
  if (lane == 0) q = 0.0;
  __syncthreads();
  double total = 0.0;
  for (int k = 0; k < kTreeWaves; ++k) {
    if (k < w) q += s_woff[k];
    total += s_woff[k];
  }
  *empty = !(total > 0.0);
  if (*empty) {
    __syncthreads();
    return -1;
  }
  const double theta = u * total;
  if (loc > 0.0 && q <= theta && theta < q + loc) {
    double acc = q;
    for (int k = k0; k < k1; ++k) {
      if (s_slot[k] > 0.0 && theta < acc + s_slot[k]) {
        *s_sel = k;
        *s_th = theta - acc;
        break;
      }
      acc += s_slot[k];
    }
  }
  __syncthreads();
  *rounding = false;
  if (*s_sel < 0) {  // theta at or past the total: the last slot with mass
    *rounding = true;
    __syncthreads();
    if (lastpos >= 0) atomicMax(s_sel, lastpos);
    if (tid == 0) *s_th = __builtin_inf();
    __syncthreads();
  }
  const int sel = *s_sel;
  const double th = *s_th;

  // (3) wavefront 0 finds the element inside slot sel
  if (w == 0) {
    float r[KV];
    int base;  // index of r[0]
    int cnt;   // valid elements in r
    if (sel == 0 || sel == nslot - 1) {
      base = sel == 0 ? lane : g.t0 + lane;
      cnt = (sel == 0 ? lane < g.v0 : g.t0 + lane < V) ? 1 : 0;
      r[0] = cnt ? law_at<TDT, DDT>(L, prow, qrow, base) : 0.f;
#pragma unroll
      for (int k = 1; k < KV; ++k) r[k] = 0.f;
    } else {
      const int vi = (sel - 1) * 64 + lane;
      base = g.v0 + vi * KV;
      cnt = vi < g.nvec ? KV : 0;
      if (cnt) {
        law_vec<TDT, DDT>(L, prow, qrow, g, vi, qvec, r);
      } else {
#pragma unroll
        for (int k = 0; k < KV; ++k) r[k] = 0.f;
      }
    }
    // removed tokens: a uniform loop over the list with a select per
    // element (no per-lane search with an early exit)
    for (int e = 0; e < nex; ++e) {
      const int t = ex[e];
#pragma unroll
      for (int k = 0; k < KV; ++k) r[k] = t == base + k ? 0.f : r[k];
    }
#pragma unroll
    for (int k = 0; k < KV; ++k) r[k] = k < cnt ? r[k] : 0.f;
    double ls = 0.0;
#pragma unroll
    for (int k = 0; k < KV; ++k) ls += (double)r[k];
    const double li = wave_incl_scan(ls, lane);
    double before = lane_before(li);
    if (lane == 0) before = 0.0;
    const uint64_t hit = __ballot(ls > 0.0 && before <= th && th < li);
    const uint64_t has = __ballot(ls > 0.0);
    const int src = hit ? (int)__builtin_ctzll(hit) : (has ? 63 - (int)__builtin_clzll(has) : 0);
    if (lane == src) {
      double a = before;
      int y = -1, lp = -1;
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        a += (double)r[k];
        if (r[k] > 0.f) {
          if (y < 0 && a > th) y = base + k;
          lp = base + k;
        }
      }
      if (!hit) *rounding = true;
      *s_sel = y >= 0 ? y : (lp >= 0 ? lp : base);
      if (!hit || y < 0) *s_th = -1.0;  // marks a rounding fallback
    }
  }
  __syncthreads();
  const int token = *s_sel;
  if (*s_th == -1.0) *rounding = true;
  __syncthreads();
  return token;
}

// The walk's per-child scalar math (fp64 exponentials, Philox).  Every lane
// computes the same value.
struct Odds {
  double px;     // p(x)
  double ratio;  // acceptance ratio of x under the current law
};

// mode 0: one-hot drafts (ratio p(x) / Zk, 0 for a removed token); 1: draft
// logits; 2: draft probabilities.
__device__ __forceinline__ Odds child_odds(float lp, float lq, float c, float pref, double pz,
                                        float qref, double qz, double ck, double Zk, int mode,
                                        bool removed) {
  Odds o;
  o.px = exp2((double)lp * (double)c + (double)pref) / pz;
  if (mode == 0) {
    o.ratio = removed ? 0.0 : o.px / Zk;
  } else {
    const double qx = mode == 2 ? (double)lq : exp2((double)lq * (double)c + (double)qref) / qz;
    double num = o.px - ck * qx;
    num = num > 0.0 ? num / Zk : 0.0;
    o.ratio = qx > 0.0 ? num / qx : (num > 0.0 ? __builtin_inf() : 0.0);
  }
  return o;
}

struct Uniforms {
  double acc, rec;
};

__device__ __forceinline__ Uniforms tree_uniforms(uint64_t seed, uint64_t offset, int b, int i) {
  Uniforms u;
  uniforms(seed, offset, b, i, &u.acc, &u.rec);
  return u;
}

template <int TDT, int DDT, bool HAS_DRAFT>
__global__ __launch_bounds__(kTreeThreads) void k_tree(const TreeParams p) {
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_ex[kMaxNodes];
  __shared__ float ldsf[kTreeWaves];
  __shared__ double ldsd[kTreeWaves];
  __shared__ int ldsi[kTreeWaves];
  __shared__ double s_woff[kTreeWaves];
  __shared__ double s_slot[kMaxVocab / 256 + 2];  // draw slots: 64 vectors each
  __shared__ int s_sel;
  __shared__ double s_th;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int N = p.N, V = p.V;
  int n = p.nn[b];
  const bool bad_n = n < 1 || n > N;
  n = n < 1 ? 1 : (n > N ? N : n);
  for (int i = tid; i < n; i += kTreeThreads) {
    s_par[i] = p.parents[(size_t)b * N + i];
    s_tok[i] = p.tokens[(size_t)b * N + i];
  }
  __syncthreads();
  uint32_t fl = bad_n ? SV_DEVERR_BAD_NUM_DRAFTS : 0u;
  if (tid == 0)
    for (int i = 1; i < n; ++i)
      if (s_par[i] < 0 || s_par[i] >= i) fl |= SV_DEVERR_BAD_TREE;

  const float T = p.temps[b];
  const bool sampling = is_sampling(T);
  const float c = sampling ? temp_scale(T) : 0.f;
  const bool probs = p.draft_is_probs != 0;
  int v = 0, nacc = 0, y = 0;
  int32_t* out = p.out_tokens + (size_t)b * N;

  for (;;) {
    const void* prow = row_ptr(p.target, TDT, (size_t)b * N + v, V);
    const void* qrow = HAS_DRAFT ? row_ptr(p.draft, DDT, (size_t)b * N + v, V) : nullptr;
    const RowStats ps = row_stats<TDT>(prow, V, sampling, c, ldsf, ldsd, ldsi);
    RowStats qs{0.f, 0.f, 1.0, 0};
    if (HAS_DRAFT && sampling && !probs) qs = row_stats<DDT>(qrow, V, true, c, ldsf, ldsd, ldsi);

    // the children of v, in index order
    double ck = 0.0, Zk = 1.0;  // law after k rejections (probabilistic)
    int nex = 0, nrej = 0, next = -1;
    for (int ch = v + 1; ch < n; ++ch) {
      if (s_par[ch] != v) continue;
      const int x = s_tok[ch];
      const bool valid = x >= 0 && x < V;
      if (!valid) fl |= SV_DEVERR_BAD_DRAFT_ID;
      bool accept;
      if (!sampling) {
        accept = valid && Elt<TDT>::at(prow, x) == ps.m;
      } else {
        double ratio = 0.0, px = 0.0;
        if (valid) {
          const float lq = HAS_DRAFT ? Elt<DDT>::at(qrow, x) : 0.f;
          const Odds o = child_odds(Elt<TDT>::at(prow, x), lq, c, ps.ref, ps.z, qs.ref, qs.z, ck,
                                    Zk, !HAS_DRAFT ? 0 : (probs ? 2 : 1),
                                    !HAS_DRAFT && excluded(s_ex, nex, x));
          px = o.px;
          ratio = o.ratio;
        }
        const Uniforms un = tree_uniforms(p.seed, p.offset, p.b_base + b, ch - 1);
        accept = un.acc < ratio;
        // one-hot: a rejected token leaves the law, which is renormalized
        if (!accept && !HAS_DRAFT && valid && !excluded(s_ex, nex, x)) Zk -= px;
      }
      if (accept) {
        next = ch;
        break;
      }
      ++nrej;
      if (sampling && !HAS_DRAFT) {
        if (valid && !excluded(s_ex, nex, x)) {
          __syncthreads();
          if (tid == 0) s_ex[nex] = x;
          __syncthreads();
          ++nex;
        }
      } else if (sampling) {  // the law left by this rejection: needs Z_{k+1}
        ck += Zk;
        bool more = false;
        for (int c2 = ch + 1; c2 < n && !more; ++c2) more = s_par[c2] == v;
        if (more) {
          Law L{true, c, ps.ref, qs.ref, 0.f, 0.f, probs};
          const double kap = ck * ps.z / (probs ? 1.0 : qs.z);
          L.kap_hi = (float)kap;
          L.kap_lo = (float)(kap - (double)L.kap_hi);
          Zk = law_sum<TDT, DDT>(L, prow, qrow, V, ldsd) / ps.z;
        }
      }
    }
    if (next >= 0) {
      if (tid == 0) out[nacc] = s_tok[next];
      ++nacc;
      v = next;
      continue;
    }
    // every child rejected, or a leaf: the emitted token is drawn at v
    if (!sampling) {
      y = ps.arg;
    } else {
      const double u_rec = tree_uniforms(p.seed, p.offset, p.b_base + b, v).rec;
      Law L{false, c, ps.ref, qs.ref, 0.f, 0.f, probs};
      if (HAS_DRAFT && nrej > 0) {
        L.pair = true;
        const double kap = ck * ps.z / (probs ? 1.0 : qs.z);
        L.kap_hi = (float)kap;
        L.kap_lo = (float)(kap - (double)L.kap_hi);
      }
      slot_pass<TDT, DDT>(L, prow, qrow, V, s_slot);
      bool rounding = false, empty = false;
      y = draw_from_slots<TDT, DDT>(L, prow, qrow, V, s_ex, nex, u_rec, s_slot, s_woff, &s_sel,
                                    &s_th, &rounding, &empty);
      if (empty) {  // no mass left: draw from p itself
        fl |= SV_DEVERR_ZERO_RESIDUAL;
        L.pair = false;
        slot_pass<TDT, DDT>(L, prow, qrow, V, s_slot);
        y = draw_from_slots<TDT, DDT>(L, prow, qrow, V, s_ex, 0, u_rec, s_slot, s_woff, &s_sel,
                                      &s_th, &rounding, &empty);
      }
      if (rounding) fl |= SV_DEVERR_DRAW_ROUNDING;
    }
    break;
  }
  for (int i = nacc + 1 + tid; i < N; i += kTreeThreads) out[i] = -1;
  if (tid == 0) {
    out[nacc] = y;
    p.out_nacc[b] = nacc;
    p.out_last[b] = v;
    if (fl) atomicOr(p.flags, fl);
  }
}

}  // namespace

hipError_t launch_tree(const TreeParams& p, int tdt, int ddt, hipStream_t s) {
  const dim3 g((unsigned)p.B), t(kTreeThreads);
  const bool d = p.draft != nullptr;
#define SV_TREE_LAUNCH(T, D)                                                   \
  if (d)                                                                       \
    hipLaunchKernelGGL((k_tree<T, D, true>), g, t, 0, s, p);                   \
  else                                                                         \
    hipLaunchKernelGGL((k_tree<T, D, false>), g, t, 0, s, p);
  if (tdt == SV_F32 && ddt == SV_F32) {
    SV_TREE_LAUNCH(SV_F32, SV_F32)
  } else if (tdt == SV_F32) {
    SV_TREE_LAUNCH(SV_F32, SV_BF16)
  } else if (ddt == SV_F32) {
    SV_TREE_LAUNCH(SV_BF16, SV_F32)
  } else {
    SV_TREE_LAUNCH(SV_BF16, SV_BF16)
  }
#undef SV_TREE_LAUNCH
  return hipGetLastError();
}

}  // namespace sv
