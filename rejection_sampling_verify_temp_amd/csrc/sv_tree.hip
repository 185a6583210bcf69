// Token-tree verification on gfx950, and its C entry point.
//
// Source: "投机采样" (razer666.cn), section 验证阶段的策略 / 验证方案: draft
// sequences that share prefixes are merged into a token tree and the target
// scores every node at once.  The multi-branch rule is the page's chain rule
// applied child by child (multi-step speculative sampling; the header of
// include/spec_verify.h states it).
//
// A team of G workgroups walks one request's tree and streams only the rows
// of the nodes it visits.  Each workgroup of the team takes a fixed share of
// every row (G contiguous runs of 64-vector pieces), so a row pass runs on G
// compute units at once, all on one XCD:
//   - at node v, one pass over target row v (and draft row v) gives each
//     share's max and normalizer (or its lowest argmax for greedy requests);
//     the team exchanges the shares and every workgroup folds them in the same
//     fixed order (one share per lane), so all hold the same row statistics;
//   - the children of v are tested in index order by every workgroup alike
//     (the same loads, the same Philox block, the same fp64 arithmetic); after
//     k rejections the law is max(0, p - c_k q) / Z_k, and each further
//     sibling test needs Z_k: one more pass over the row pair and one more
//     exchange;
//   - where the walk stops, the emitted token is drawn by inverse CDF: each
//     workgroup sums the law per slot of 64 vectors of its share (at a node
//     without children, whose law is p, its statistics pass already did), the
//     team exchanges the share totals, and the workgroup whose share holds
//     u * S scans its slots and re-reads one slot to find the element.
// An exchange writes each value beside the exchange's tag in one agent-scope
// atomic store, and spins until every member's words carry the tag.  A team
// is launched only when all teams fit the device at once, so on an idle
// device every member runs; the wait is still bounded, and a member that
// times out finishes the walk alone over whole rows, with the same results.
// At large batches (more requests than teams the device holds) each team
// walks several requests in turn, taking the next free request from a
// launch-wide counter whenever a walk ends.  One 1024-thread workgroup per
// request, with no exchanges, remains where the device's team capacity is
// unknown, or on request.
//
// Row passes issue all of a round's 16-byte loads (10 vectors of a row, or 5
// of each row of a pair, per thread) before using any (one round trip per
// round), through buffer resources, so the loads of a round cost no address
// registers and no branches, and no round waits at a workgroup barrier.  A walk that a single compute unit runs alone is bound by
// that unit's arithmetic (~6 VALU slots per element) more than by memory;
// spreading each row over a team's units is what shortens the longest walks,
// which set the kernel's time once most requests are done.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_tree.h"


namespace sv {
namespace {

constexpr int kSoloThreads = 1024;  // the workgroup of a walk without a team
constexpr int kTeamThreads = 256;   // a team member's workgroup
constexpr int kMaxNodes = SPEC_TREE_MAX_NODES;

struct RowStats {
  float m;     // row max
  float ref;   // exponent reference ref_of(m, c)
  double z;    // sum of exp2(l c + ref)
  int arg;     // lowest index of the max (greedy)
};

// A row is a scalar head [0, v0) up to the first 16-byte boundary, nvec
// vectors from v0 and a scalar tail [t0, V) (chunk_geo over the whole row).
// Workgroup gi of a team of G takes the vectors [vb, vb + nv): the row's
// pieces of 64 vectors split into G contiguous runs, the head going to the
// first workgroup and the tail to the last (gi < 0: the whole row).
struct Rng {
  int vb, nv;
  bool head, tail;
};

template <int G>
__device__ __forceinline__ Rng row_range(const Geo& g, int gi) {
  if (G == 1 || gi < 0) return Rng{0, g.nvec, true, true};  // the whole row
  const int per = ((g.nvec + G - 1) / G + 63) / 64 * 64;
  const int vb = min(g.nvec, gi * per);
  Rng r;
  r.vb = vb;
  r.nv = min(g.nvec, vb + per) - vb;
  r.head = gi == 0;
  r.tail = gi == G - 1;
  return r;
}

// A pass takes the share's vectors in rounds: every thread issues all its
// loads of a round (vectors b0 + u * NT + tid of the share) before it uses
// any, so one round trip to memory covers kRowVecs * 16 bytes per thread of
// a single row, or kPairVecs * 16 of each row of a pair (the residual
// passes).  The 10 vectors take 40 of the 128 registers a thread has at four
// wavefronts per SIMD; the walk's own state takes most of the rest.  Pairs
// of 5 rather than 7 leave the team kernels fewer spills and measured ~1%
// faster.
constexpr int kRowVecs = 10;
constexpr int kPairVecs = 5;

// Draw slots of a share: slot 0 is the row's head (empty but in the first
// workgroup), slot 1 + k the share's 64 vectors [64 k, 64 k + 64) (one
// wavefront's share of one unroll step), the last slot the row's tail.
__device__ __forceinline__ int num_slots(const Rng& r) { return (r.nv + 63) / 64 + 2; }

__device__ __forceinline__ const u32x4* vec_base(const void* row, const Geo& g, int bytes) {
  return reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + (size_t)g.v0 * bytes);
}

// The share's vectors as a buffer resource (loads past the share return 0).
__device__ __forceinline__ VecBuf vec_buf(const void* row, const Geo& g, const Rng& r, int bytes) {
  return make_vec_buf(vec_base(row, g, bytes) + r.vb, (uint32_t)r.nv * 16u);
}

// Vector b0 + tid + u * NT of the share, or 0 past its end.
template <int NT>
__device__ __forceinline__ u32x4 vec_load(const VecBuf& vb, int b0, int u, int tid) {
  return buf_load<false>(vb, (uint32_t)(b0 + u * NT + tid) * 16u);
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

// ---------------------------------------------------------------------------
// The team: its workgroups exchange up to eight 32-bit values each per step
// ---------------------------------------------------------------------------
constexpr int kXWords = 8;  // words per member and exchange

struct Team {
  uint64_t* xdat;  // [teams][2][G][kXWords]: (exchange tag << 32) | value bits,
                   // double-buffered by the exchange's parity; all 0 between launches
  uint32_t* xdone; // [teams]: members that finished this launch; 0 between launches
  int t, gi;       // team index, this workgroup's index in the team
  uint32_t k;      // exchanges made so far in this launch
  bool solo;       // a wait timed out: this workgroup walks alone from there
  uint64_t spin;   // the wait's bound in ticks of the 100 MHz real-time clock
};

// A double as two floats whose sum is within 2^-48 of it, and back.
__device__ __forceinline__ void split_f64(double v, float& hi, float& lo) {
  hi = (float)v;
  lo = (float)(v - (double)hi);
}
__device__ __forceinline__ double join_f64(float hi, float lo) { return (double)hi + (double)lo; }

// Every workgroup of the team calls this with its values mine[0..nw) (the
// same in all of its threads); on return s_all[kXWords g + j] holds member
// g's value j, in every workgroup.  Wavefront 0 stores and polls; the others
// run `idle` meanwhile (work the caller needs only after the exchange).  Each value travels in a 64-bit word
// beside the exchange's tag k + 1, written by one agent-scope atomic store,
// so a reader that sees the tag in a word has that word's value: one round
// trip per poll, and nothing for the writer to wait for.  Double buffering is
// enough: a member can write exchange k + 2 only after every member has
// written k + 1, which each does after reading exchange k.  The tags restart
// at 1 in every launch, since team_done() returns the words to 0.
//
// The wait is bounded.  A member whose partners do not all show the tag
// within the bound (a partner not yet running on a device shared with other
// work) turns solo: s_all is not filled, and from then on the workgroup
// computes every member's share itself, in member order, and folds the same
// words the exchange would have carried.  Alone or in the team, every member
// therefore computes the same outputs, bit for bit, and the request's results
// do not depend on which members finish it.
struct NoIdle {
  __device__ void operator()() const {}
};

template <int G, typename Idle = NoIdle>
__device__ __forceinline__ void exchange(Team& tm, const float (&mine)[kXWords], int nw,
                                         float* s_all, int* s_solo, const Idle& idle = Idle{}) {
  const int tid = threadIdx.x;
  __syncthreads();  // s_all's previous contents are read
  if (tid >= 64) {
    idle();  // the other wavefronts' work while wavefront 0 waits
  } else {
    bool solo = false;
    uint64_t* slot = tm.xdat + ((size_t)tm.t * 2 + (tm.k & 1u)) * G * kXWords;
    const uint32_t tag = tm.k + 1u;
    const int j = tid & (kXWords - 1), g = tid / kXWords;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < kXWords; ++i) v = j == i ? mine[i] : v;
    if (tid < kXWords && j < nw)
      __hip_atomic_store(slot + tm.gi * kXWords + j,
                         ((uint64_t)tag << 32) | __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    const bool reader = g < G && j < nw;
    uint64_t w = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
      if (reader) w = __hip_atomic_load(slot + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__all(!reader || (uint32_t)(w >> 32) == tag)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > tm.spin) {
        solo = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!solo && tid < kXWords * G) s_all[tid] = __builtin_bit_cast(float, (uint32_t)w);
    if (tid == 0) *s_solo = solo ? 1 : 0;
  }
  __syncthreads();
  tm.solo = *s_solo != 0;
  ++tm.k;
}

// The end of a team's launch: the last member to arrive returns the team's
// words and its counter to 0.  Every member arrives only after its last
// exchange's reads, so no member still reads what is cleared.
template <int G>
__device__ __forceinline__ void team_done(Team& tm, uint32_t* next_req, int teams) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t before =
        __hip_atomic_fetch_add(tm.xdone + tm.t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == G - 1) {
      uint64_t* w = tm.xdat + (size_t)tm.t * 2 * G * kXWords;
      for (int i = 0; i < 2 * G * kXWords; ++i)
        __hip_atomic_store(w + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the words are clear before the count
      __hip_atomic_store(tm.xdone + tm.t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // teams that walked several requests: the last team returns the
      // request counter to 0 (every member has taken its last request)
      if (next_req != nullptr &&
          __hip_atomic_fetch_add(next_req + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (uint32_t)teams - 1) {
        __hip_atomic_store(next_req, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __hip_atomic_store(next_req + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// The team's next request once a walk is done (teams that walk several
// requests): member 0 takes the next free one from the launch's counter and
// sends it in an exchange, so the team walks it together.  A workgroup
// alone (a wait timed out) takes its own.  Every request is taken once, and
// the workgroup that took it walks it, in the team or alone.
template <int G>
__device__ __forceinline__ int next_request(Team& tm, uint32_t* next_req, int teams, float* s_x,
                                            int* s_solo, int* s_next) {
  const bool take = tm.solo || tm.gi == 0;
  __syncthreads();
  if (take && threadIdx.x == 0)
    *s_next = teams + (int)__hip_atomic_fetch_add(next_req, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int nb = take ? *s_next : 0;
  if (tm.solo) return nb;
  float mine[kXWords] = {};
  mine[0] = __builtin_bit_cast(float, nb);
  exchange<G>(tm, mine, 1, s_x, s_solo);
  if (!tm.solo) return __builtin_bit_cast(int, s_x[0]);  // member 0's
  if (tm.gi == 0) return nb;  // alone now, with the request it took
  __syncthreads();
  if (threadIdx.x == 0)
    *s_next = teams + (int)__hip_atomic_fetch_add(next_req, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_next;
}

// ---------------------------------------------------------------------------
// Row statistics
// ---------------------------------------------------------------------------

// One wavefront's part of a sampling row's statistics over this
// workgroup's share: the wavefront's max Mw (the same in its 64 lanes; its
// reference is ref_of(Mw, c)) and this thread's sum of exp2(l c +
// ref_of(Mw, c)).  Each round goes in two phases per wavefront: the
// wavefront's max of the round first, which fixes one exponent reference for
// its 64 lanes, then the sums of exp2(l c + ref) with no per-element max
// test.  A later round that raises a wavefront's max rescales its sums once.
// No round needs a workgroup barrier, so the wavefronts drift apart and one's
// loads overlap another's arithmetic.
//
// SLOTS (at a node whose draw is from p alone): the same pass also leaves the
// draw's slot sums of the share in s_slot, each relative to the reference
// its wavefront held when it summed the slot, which goes to s_sref
// (rescale_slots moves them to the row's reference).  The slot of 64 vectors
// is one wavefront's share of one unroll step, as in slot_pass.
struct WavePart {
  float Mw;
  double S;
};

template <int DT, int NT, int G, bool SLOTS>
__device__ __forceinline__ WavePart wave_pass(const void* row, int V, float c, int gi,
                                              double* s_slot, float* s_sref) {
  using E = Elt<DT>;
  constexpr int U = kRowVecs;
  const int tid = pass_tid();
  const Geo g = chunk_geo<DT>(row, 0, V);
  const Rng rg = row_range<G>(g, gi);
  const VecBuf vb = vec_buf(row, g, rg, E::kBytes);
  // the head's scalar elements in the first workgroup, the tail's in the last
  const bool has_h = rg.head && tid < g.v0, has_t = rg.tail && g.t0 + tid < V;
  const float hx = has_h ? E::at(row, tid) : kNegInf;
  const float tx = has_t ? E::at(row, g.t0 + tid) : kNegInf;
  float Mw = kNegInf, Rw = 0.f;  // the wavefront's max and reference so far
  double S = 0.0;                // this thread's sum, relative to Rw
  for (int b0 = 0; b0 == 0 || b0 < rg.nv; b0 += U * NT) {
    u32x4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = vec_load<NT>(vb, b0, u, tid);
    // vectors past the share are skipped by a test that is uniform in all
    // but one wavefront (the loads there returned 0)
    float t = b0 == 0 ? fmaxf(hx, tx) : kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (b0 + u * NT + tid < rg.nv) {
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
    float sr = 0.f;
    if (b0 == 0) {
      const float eh = fast_exp2(fmaf(hx, c, Rw)), et = fast_exp2(fmaf(tx, c, Rw));
      sr = eh + et;
      if constexpr (SLOTS) {
        if ((tid >> 6) == 0) {  // the head and tail lie in wavefront 0
          const float hs = wave_sum_f32(eh), ts = wave_sum_f32(et);
          if (tid == 0) {
            const int last = num_slots(rg) - 1;
            s_slot[0] = (double)hs;
            s_slot[last] = (double)ts;
            s_sref[0] = Rw;
            s_sref[last] = Rw;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sv = 0.f;
      if (b0 + u * NT + tid < rg.nv) {
        // unpack again rather than keep the floats live: the empty asm hides
        // the first unpack from common-subexpression elimination
        u32x4 wv = d[u];
        asm volatile("" : "+v"(wv));
        float e[E::kVec];
        E::unpack(wv, e);
#pragma unroll
        for (int k = 0; k < E::kVec; ++k) e[k] = fast_exp2(fmaf(e[k], c, Rw));
        sv = pairwise_sum(e);
        sr += sv;
        asm volatile("" : "+v"(sr));  // fold in order: no sums wait in registers
      }
      if constexpr (SLOTS) {  // convergent: every lane, past the share or not
        const float ws = wave_sum_f32(sv);
        const int piece = (b0 + u * NT) / 64 + (tid >> 6);
        if ((tid & 63) == 0 && piece < (rg.nv + 63) / 64) {
          s_slot[1 + piece] = (double)ws;
          s_sref[1 + piece] = Rw;
        }
      }
    }
    S += (double)sr;
  }
  return WavePart{Mw, S};
}

// A sum of parts, each with its own max m_k (its sum z_k relative to
// ref_of(m_k, c)), moved to the reference R of the overall max M: lane k
// holds part k (mine) and scales it, and the wavefront adds the lanes in
// one fixed DPP order.  Every wavefront, every member of a team and a member
// alone therefore get the same bits, and the parts' scale factors take one
// latency instead of one each in turn.
__device__ __forceinline__ double lane_fold(bool mine, float mk, double zk, float M, float R,
                                            float c) {
  const double t =
      (!mine || mk == kNegInf) ? 0.0 : (mk == M ? zk : zk * exp2_diff(R, ref_of(mk, c)));
  return wave_sum(t);
}

// Two such sums at once: lanes 0..31 hold the first sum's parts and lanes
// 32..63 the second's, and the DPP steps of wave_sum stop where each half of
// the wavefront has its own total (lanes 31 and 63).
__device__ __forceinline__ void lane_fold2(bool mine, float mk, double zk, float M, float R,
                                           float c, double& z0, double& z1) {
  double t = (!mine || mk == kNegInf) ? 0.0 : (mk == M ? zk : zk * exp2_diff(R, ref_of(mk, c)));
  t = dpp_sum_step<kDppShr1, 0xf>(t);
  t = dpp_sum_step<kDppShr2, 0xf>(t);
  t = dpp_sum_step<kDppShr4, 0xf>(t);
  t = dpp_sum_step<kDppShr8, 0xf>(t);
  t = dpp_sum_step<kDppBcast15, 0xa>(t);
  const uint64_t b = (uint64_t)__double_as_longlong(t);
  const uint32_t lo0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 31);
  const uint32_t hi0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 31);
  const uint32_t lo1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  z0 = __longlong_as_double((long long)(((uint64_t)hi0 << 32) | lo0));
  z1 = __longlong_as_double((long long)(((uint64_t)hi1 << 32) | lo1));
}

// Statistics of this workgroup's share of one row.  Sampling rows: the
// wavefront parts of wave_pass meet once, at the share's reference.  Greedy
// rows keep the max and its lowest index (INT32_MAX: none).
template <int DT, int NT, int G, bool SLOTS = false>
__device__ __forceinline__ RowStats row_stats(const void* row, int V, bool sampling, float c,
                                              int gi, float* ldsf, double* ldsd, int* ldsi,
                                              double* s_slot = nullptr, float* s_sref = nullptr) {
  using E = Elt<DT>;
  constexpr int U = kRowVecs;
  const int tid = pass_tid();
  const Geo g = chunk_geo<DT>(row, 0, V);
  const Rng rg = row_range<G>(g, gi);
  const VecBuf vb = vec_buf(row, g, rg, E::kBytes);
  // the head's scalar elements in the first workgroup, the tail's in the last
  const bool has_h = rg.head && tid < g.v0, has_t = rg.tail && g.t0 + tid < V;
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
    for (int b0 = 0; b0 < rg.nv; b0 += U * NT) {
      u32x4 d[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b0 + u * NT + tid < rg.nv) d[u] = vec_load<NT>(vb, b0, u, tid);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int vi = b0 + u * NT + tid;
        if (vi < rg.nv) {
          float x[E::kVec];
          int ix[E::kVec];
          E::unpack(d[u], x);
#pragma unroll
          for (int k = 0; k < E::kVec; ++k) ix[k] = g.v0 + (rg.vb + vi) * E::kVec + k;
          am_tile(a, x, ix);
        }
      }
    }
    if (has_t) {
      const float x[1] = {tx};
      const int ix[1] = {g.t0 + tid};
      am_tile(a, x, ix);
    }
    block_argmax<NT>(a.M, a.I, ldsf, ldsi);
    st.m = a.M;
    st.arg = a.I;
    st.ref = 0.f;
    st.z = 0.0;
    return st;
  }
  const WavePart wp = wave_pass<DT, NT, G, SLOTS>(row, V, c, gi, s_slot, s_sref);
  const float M = block_max<NT>(wp.Mw, ldsf);
  const float R = ref_of(M, c);
  const double f =
      wp.Mw == kNegInf ? 0.0 : (wp.Mw == M ? 1.0 : exp2_diff(R, ref_of(wp.Mw, c)));
  st.m = M;
  st.ref = R;
  st.z = block_sum<NT>(wp.S * f, ldsd);
  st.arg = 0;
  return st;
}

// Target and draft statistics of this workgroup's shares of a row pair
// (sampling): both passes first, then one LDS exchange of the wavefront
// parts for the two folds, so the draft row's loads follow the target's
// arithmetic with no block reduction in between.
template <int TDT, int DDT, int NT, int G>
__device__ __forceinline__ void pair_stats(const void* prow, const void* qrow, int V, float c,
                                           int gi, float* s_wm, double* s_ws, RowStats& ps,
                                           RowStats& qs) {
  constexpr int W = NT / 64;
  const WavePart a = wave_pass<TDT, NT, G, false>(prow, V, c, gi, nullptr, nullptr);
  const WavePart d = wave_pass<DDT, NT, G, false>(qrow, V, c, gi, nullptr, nullptr);
  const double sa = wave_sum(a.S), sd = wave_sum(d.S);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    s_wm[w] = a.Mw;
    s_wm[W + w] = d.Mw;
    s_ws[w] = sa;
    s_ws[W + w] = sd;
  }
  __syncthreads();
  // both rows' folds in one pass: the target's parts in the wavefront's lower
  // half, the draft's in the upper
  static_assert(W <= 32, "one half-wavefront per row");
  float Mp = kNegInf, Mq = kNegInf;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    Mp = fmaxf(Mp, s_wm[k]);
    Mq = fmaxf(Mq, s_wm[W + k]);
  }
  const float Rp = ref_of(Mp, c), Rq = ref_of(Mq, c);
  const bool upper = lane >= 32;
  const int k = lane & 31, at = (upper ? W : 0) + (k < W ? k : 0);
  double zp, zq;
  lane_fold2(k < W, s_wm[at], s_ws[at], upper ? Mq : Mp, upper ? Rq : Rp, c, zp, zq);
  ps = RowStats{Mp, Rp, zp, 0};
  qs = RowStats{Mq, Rq, zq, 0};
  __syncthreads();  // s_wm and s_ws are free again
}

// A share's statistics as the words a member sends: target max, its sum
// split in two floats (or its argmax, greedy), draft max and sum.
__device__ __forceinline__ void stat_words(const RowStats& a, const RowStats& bq, bool sampling,
                                           float (&w)[kXWords]) {
  w[0] = a.m;
  if (sampling) {
    split_f64(a.z, w[1], w[2]);
  } else {
    w[1] = __builtin_bit_cast(float, a.arg);
    w[2] = 0.f;
  }
  w[3] = bq.m;
  split_f64(bq.z, w[4], w[5]);
}

// The row's statistics from the team's shares: member g's words at
// x[kXWords g + o ...] are its max and then its sum (sampling: relative to its
// own reference, split in two floats) or lowest argmax (greedy).  The shares
// are folded in one fixed order (lane_fold), so every member gets the same
// bits.
template <int G>
__device__ __forceinline__ RowStats fold_stats(const float* x, int o, bool sampling, float c) {
  RowStats st;
  float M = kNegInf;
#pragma unroll
  for (int g = 0; g < G; ++g) M = fmaxf(M, x[kXWords * g + o]);
  st.m = M;
  if (!sampling) {
    int arg = INT32_MAX;
#pragma unroll
    for (int g = 0; g < G; ++g)  // the shares are in index order: the first one at M
      if (arg == INT32_MAX && x[kXWords * g + o] == M)
        arg = __builtin_bit_cast(int, x[kXWords * g + o + 1]);
    st.arg = arg == INT32_MAX ? 0 : arg;
    st.ref = 0.f;
    st.z = 0.0;
    return st;
  }
  const float R = ref_of(M, c);
  const int lane = threadIdx.x & 63, g = lane < G ? lane : 0;
  st.ref = R;
  st.z = lane_fold(lane < G, x[kXWords * g + o],
                   join_f64(x[kXWords * g + o + 1], x[kXWords * g + o + 2]), M, R, c);
  st.arg = 0;
  return st;
}

// The target's and the draft's statistics from the team's shares of a row
// pair (sampling; member g's words at x[kXWords g ...]: target max and sum,
// draft max and sum), both folded in one pass as in pair_stats.
template <int G>
__device__ __forceinline__ void fold_pair(const float* x, float c, RowStats& ps, RowStats& qs) {
  static_assert(G <= 32, "one half-wavefront per row");
  float Mp = kNegInf, Mq = kNegInf;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Mp = fmaxf(Mp, x[kXWords * g]);
    Mq = fmaxf(Mq, x[kXWords * g + 3]);
  }
  const float Rp = ref_of(Mp, c), Rq = ref_of(Mq, c);
  const int lane = threadIdx.x & 63, k = lane & 31;
  const bool upper = lane >= 32;
  const int at = kXWords * (k < G ? k : 0) + (upper ? 3 : 0);
  double zp, zq;
  lane_fold2(k < G, x[at], join_f64(x[at + 1], x[at + 2]), upper ? Mq : Mp, upper ? Rq : Rp, c,
             zp, zq);
  ps = RowStats{Mp, Rp, zp, 0};
  qs = RowStats{Mq, Rq, zq, 0};
}

// The sum of a value that every member sent split at x[kXWords g], one
// member per lane, added in one fixed order.
template <int G>
__device__ __forceinline__ double fold_sum(const float* x) {
  const int lane = threadIdx.x & 63, g = lane < G ? lane : 0;
  return wave_sum(lane < G ? join_f64(x[kXWords * g], x[kXWords * g + 1]) : 0.0);
}

// A workgroup's own share as the whole row's statistics (a team of one).
__device__ __forceinline__ RowStats solo_stats(RowStats st, bool sampling) {
  if (!sampling && st.arg == INT32_MAX) st.arg = 0;
  return st;
}

// ---------------------------------------------------------------------------
// The law the stop node draws from, and passes over it
// ---------------------------------------------------------------------------

// Per element (unnormalized, relative to the target row's reference):
// p~ = exp2(l_p c + ref_p); for a pair, max(0, p~ - kappa q~) with
// q~ = exp2(l_q c + ref_q) (or q itself for probability drafts) and kappa
// split in two floats.
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

// The law at the kVec elements of target vector vi (an index over the whole
// row).  The draft row's elements come by one vector load when both rows have
// the same element type and alignment (qvec), else element by element.
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

// One pass over the law on this workgroup's share of a row (and, for a pair,
// of its draft row): calls f(b, s) once per unroll step of every round,
// convergently, with s the thread's fp32 sum of the law over the share's
// vector b + tid (0 past the share).  When the draft row has the target's
// element type and 16-byte alignment, both rows' vectors of a round are
// loaded together, kPairVecs each (or kRowVecs of a single row); otherwise
// the draft elements are loaded one by one, a vector of the target at a time.
template <int TDT, int DDT, int NT, typename F>
__device__ __forceinline__ void law_pass(const Law& L, const void* prow, const void* qrow,
                                         const Geo& g, const Rng& rg, F&& f) {
  using EP = Elt<TDT>;
  constexpr int KV = EP::kVec;
  const int tid = pass_tid();
  const VecBuf pb = vec_buf(prow, g, rg, EP::kBytes);
  if (!L.pair) {
    for (int b0 = 0; b0 < rg.nv; b0 += kRowVecs * NT) {
      u32x4 d[kRowVecs];
#pragma unroll
      for (int u = 0; u < kRowVecs; ++u) d[u] = vec_load<NT>(pb, b0, u, tid);
#pragma unroll
      for (int u = 0; u < kRowVecs; ++u) {
        float sv = 0.f;  // vectors past the share: a test uniform in all but one wavefront
        if (b0 + u * NT + tid < rg.nv) {
          float r[KV];
          EP::unpack(d[u], r);
#pragma unroll
          for (int k = 0; k < KV; ++k) r[k] = law_of(L, r[k], 0.f);
          sv = pairwise_sum(r);
        }
        f(b0 + u * NT, sv);
      }
    }
    return;
  }
  if constexpr (TDT == DDT) {
    if (same_alignment(prow, qrow)) {
      const VecBuf qb = vec_buf(qrow, g, rg, EP::kBytes);
      for (int b0 = 0; b0 < rg.nv; b0 += kPairVecs * NT) {
        u32x4 dp[kPairVecs], dq[kPairVecs];
#pragma unroll
        for (int u = 0; u < kPairVecs; ++u) {
          dp[u] = vec_load<NT>(pb, b0, u, tid);
          dq[u] = vec_load<NT>(qb, b0, u, tid);
        }
#pragma unroll
        for (int u = 0; u < kPairVecs; ++u) {
          float sv = 0.f;
          if (b0 + u * NT + tid < rg.nv) {
            float lp[KV], lq[KV], r[KV];
            EP::unpack(dp[u], lp);
            EP::unpack(dq[u], lq);
#pragma unroll
            for (int k = 0; k < KV; ++k) r[k] = law_of(L, lp[k], lq[k]);
            sv = pairwise_sum(r);
          }
          f(b0 + u * NT, sv);
        }
      }
      return;
    }
  }
  for (int b0 = 0; b0 < rg.nv; b0 += NT) {
    float sv = 0.f;
    if (b0 + tid < rg.nv) {
      float r[KV];
      law_vec<TDT, DDT>(L, prow, qrow, g, rg.vb + b0 + tid, false, r);
      sv = pairwise_sum(r);
    }
    f(b0, sv);
  }
}

// Sum of the law over this workgroup's share (fp64 across vectors).
template <int TDT, int DDT, int NT, int G>
__device__ __forceinline__ double law_sum(const Law& L, const void* prow, const void* qrow, int V,
                                          int gi, double* ldsd) {
  const int tid = pass_tid();
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  const Rng rg = row_range<G>(g, gi);
  double acc = 0.0;
  if (rg.head && tid < g.v0) acc += (double)law_at<TDT, DDT>(L, prow, qrow, tid);
  // eight vector sums in fp32, then one fp64 add (every thread makes the
  // same number of calls, so the flush is uniform)
  float part = 0.f;
  int nv = 0;
  law_pass<TDT, DDT, NT>(L, prow, qrow, g, rg, [&](int, float sv) {
    part += sv;
    asm volatile("" : "+v"(part));  // fold in order: no sums wait in registers
    if (++nv == 8) {
      acc += (double)part;
      part = 0.f;
      nv = 0;
    }
  });
  acc += (double)part;
  if (rg.tail && g.t0 + tid < V) acc += (double)law_at<TDT, DDT>(L, prow, qrow, g.t0 + tid);
  return block_sum<NT>(acc, ldsd);
}

// The law's sums per draw slot of this workgroup's share, by one pass.
template <int TDT, int DDT, int NT, int G>
__device__ __forceinline__ void slot_pass(const Law& L, const void* prow, const void* qrow, int V,
                                          int gi, double* s_slot) {
  const int tid = pass_tid(), lane = tid & 63, w = tid >> 6;
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  const Rng rg = row_range<G>(g, gi);
  const int npieces = (rg.nv + 63) / 64, nslot = npieces + 2;
  law_pass<TDT, DDT, NT>(L, prow, qrow, g, rg, [&](int b, float sv) {
    const int piece = b / 64 + w;
    const double ws = (double)wave_sum_f32(sv);  // 64 vector sums: fp32 is ample
    if (lane == 0 && piece < npieces) s_slot[1 + piece] = ws;
  });
  if (w == 0) {
    const double h =
        wave_sum(rg.head && lane < g.v0 ? (double)law_at<TDT, DDT>(L, prow, qrow, lane) : 0.0);
    const double t = wave_sum(rg.tail && g.t0 + lane < V
                                  ? (double)law_at<TDT, DDT>(L, prow, qrow, g.t0 + lane)
                                  : 0.0);
    if (lane == 0) {
      s_slot[0] = h;
      s_slot[nslot - 1] = t;
    }
  }
}

// Slot sums that a SLOTS statistics pass left relative to its wavefronts'
// references, moved to the law's reference ref (a factor 2^(ref - sref) <= 1;
// an empty slot stays 0 whatever its reference).
template <int NT>
__device__ __forceinline__ void rescale_slots(int nslot, float ref, double* s_slot,
                                              const float* s_sref) {
  __syncthreads();  // the pass's slot writes are visible
  for (int k = pass_tid(); k < nslot; k += NT)
    if (s_slot[k] > 0.0) s_slot[k] *= s_sref[k] == ref ? 1.0 : exp2_diff(ref, s_sref[k]);
}

// The law's slot sums of share sh in s_slot.  fused: the law is p alone and
// the node's statistics pass kept its slot sums, so they are made again by
// that pass (the bits the member of share sh got), not by a slot pass.
template <int TDT, int DDT, int NT, int G>
__device__ __forceinline__ void share_slots(const Law& L, const void* prow, const void* qrow, int V,
                                            int sh, bool fused, double* s_slot, float* s_sref,
                                            float* ldsf, double* ldsd, int* ldsi) {
  if (fused) {
    (void)row_stats<TDT, NT, G, true>(prow, V, true, L.c, sh, ldsf, ldsd, ldsi, s_slot, s_sref);
    const Geo g = chunk_geo<TDT>(prow, 0, V);
    rescale_slots<NT>(num_slots(row_range<G>(g, sh)), L.ref_p, s_slot, s_sref);
  } else {
    slot_pass<TDT, DDT, NT, G>(L, prow, qrow, V, sh, s_slot);
  }
}

__device__ __forceinline__ bool excluded(const int* ex, int nex, int i) {
  for (int k = 0; k < nex; ++k)
    if (ex[k] == i) return true;
  return false;
}

// The draw slot of this workgroup's share that holds element i of the row,
// or -1 if another member's share holds it.
__device__ __forceinline__ int slot_of(const Geo& g, const Rng& rg, int nslot, int kv, int i) {
  if (i < g.v0) return rg.head ? 0 : -1;
  if (i >= g.t0) return rg.tail ? nslot - 1 : -1;
  const int vi = (i - g.v0) / kv;
  if (vi < rg.vb || vi >= rg.vb + rg.nv) return -1;
  return 1 + (vi - rg.vb) / 64;
}

struct DrawOut {
  int token;      // the drawn token (in the member that found it; -1 elsewhere)
  bool rounding;  // u * S fell past a recomputed total: nearest token with mass taken
  bool empty;     // the law is 0
};

// A thread's part of the scan over a share's slot sums: slots [k0, k1),
// their sum, the sum of the slots before them, the last one with mass, and
// the share's total.
struct SlotScan {
  double q, loc, total;
  int k0, k1, lastpos;
};

// The slot sums of share sh after slot_pass: slots that hold removed tokens
// (ex[0..nex)) are summed again with them zeroed (not reduced by their
// values: a removed sibling can hold nearly all of the slot, and the
// difference of two rounded sums would leave a residue far above the mass
// that remains), then scanned.
template <int TDT, int DDT, int NT, int G>
__device__ __forceinline__ SlotScan slot_scan(const Law& L, const void* prow, const void* qrow,
                                              int V, int sh, const int* ex, int nex, double* s_slot,
                                              double* s_woff) {
  using EP = Elt<TDT>;
  constexpr int KV = EP::kVec;
  constexpr int W = NT / 64;
  const int tid = pass_tid(), lane = tid & 63, w = tid >> 6;
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  const Rng rg = row_range<G>(g, sh);
  const bool qvec = L.pair && same_alignment(prow, qrow);
  const int nslot = num_slots(rg);
  __syncthreads();
  if (w == 0) {
    for (int k = 0; k < nex; ++k) {  // uniform over the wavefront
      const int sl = slot_of(g, rg, nslot, KV, ex[k]);
      if (sl < 0) continue;
      bool seen = false;
      for (int k2 = 0; k2 < k; ++k2) seen = seen || slot_of(g, rg, nslot, KV, ex[k2]) == sl;
      if (seen) continue;
      float r[KV];
      int base;
#pragma unroll
      for (int j = 0; j < KV; ++j) r[j] = 0.f;
      if (sl == 0 || sl == nslot - 1) {
        base = sl == 0 ? lane : g.t0 + lane;
        if (sl == 0 ? lane < g.v0 : base < V) r[0] = law_at<TDT, DDT>(L, prow, qrow, base);
      } else {
        const int vi = rg.vb + (sl - 1) * 64 + lane;
        base = g.v0 + vi * KV;
        if (vi < rg.vb + rg.nv) law_vec<TDT, DDT>(L, prow, qrow, g, vi, qvec, r);
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
  }
  __syncthreads();
  // thread t takes slots [t sp, t sp + sp)
  SlotScan sc;
  const int sp = (nslot + NT - 1) / NT;
  sc.k0 = min(nslot, tid * sp);
  sc.k1 = min(nslot, sc.k0 + sp);
  sc.loc = 0.0;
  sc.lastpos = -1;
  for (int k = sc.k0; k < sc.k1; ++k) {
    sc.loc += s_slot[k];
    if (s_slot[k] > 0.0) sc.lastpos = k;
  }
  const double incl = wave_incl_scan(sc.loc, lane);
  if (lane == 63) s_woff[w] = incl;
  sc.q = lane_before(incl);
  if (lane == 0) sc.q = 0.0;
  __syncthreads();
  sc.total = 0.0;
  for (int k = 0; k < W; ++k) {
    if (k < w) sc.q += s_woff[k];
    sc.total += s_woff[k];
  }
  __syncthreads();  // s_woff is free again
  return sc;
}

// The element of share sh that holds theta, from its scan sc (the share's
// slot sums still in s_slot): the slot whose running sum, after `before` (the
// shares ahead of this one), passes theta, then wavefront 0 re-reads only
// that slot (one vector per lane) to find the element.  past: theta is at
// or past the law's total, which takes the share's last slot with mass.
template <int TDT, int DDT, int NT, int G>
__device__ __forceinline__ int slot_find(const Law& L, const void* prow, const void* qrow, int V,
                                         int sh, const int* ex, int nex, const SlotScan& sc,
                                         double before, double theta, bool past,
                                         const double* s_slot, int* s_sel, double* s_th,
                                         bool* rounding) {
  using EP = Elt<TDT>;
  constexpr int KV = EP::kVec;
  const int tid = pass_tid(), lane = tid & 63, w = tid >> 6;
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  const Rng rg = row_range<G>(g, sh);
  const bool qvec = L.pair && same_alignment(prow, qrow);
  const int nslot = num_slots(rg);
  if (tid == 0) *s_sel = -1;
  __syncthreads();
  if (!past && sc.loc > 0.0 && before + sc.q <= theta && theta < before + sc.q + sc.loc) {
    double acc = before + sc.q;
    for (int k = sc.k0; k < sc.k1; ++k) {
      if (s_slot[k] > 0.0 && theta < acc + s_slot[k]) {
        *s_sel = k;
        *s_th = theta - acc;
        break;
      }
      acc += s_slot[k];
    }
  }
  __syncthreads();
  *rounding = past;
  if (*s_sel < 0) {  // theta at or past the share's total: its last slot with mass
    *rounding = true;
    __syncthreads();
    if (sc.lastpos >= 0) atomicMax(s_sel, sc.lastpos);
    if (tid == 0) *s_th = __builtin_inf();
    __syncthreads();
  }
  // no slot with mass (sums that no longer agree with the share's total):
  // the head slot, whose loads stay within the row whatever it holds
  const int sel = *s_sel < 0 ? 0 : *s_sel;
  const double th = *s_th;
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
      const int vi = rg.vb + (sel - 1) * 64 + lane;
      base = g.v0 + vi * KV;
      cnt = vi < rg.vb + rg.nv ? KV : 0;
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
    double lb = lane_before(li);
    if (lane == 0) lb = 0.0;
    const uint64_t hit = __ballot(ls > 0.0 && lb <= th && th < li);
    const uint64_t has = __ballot(ls > 0.0);
    const int src = hit ? (int)__builtin_ctzll(hit) : (has ? 63 - (int)__builtin_clzll(has) : 0);
    if (lane == src) {
      double a = lb;
      int y = -1, lp = -1;
#pragma unroll
      for (int k = 0; k < KV; ++k) {
        a += (double)r[k];
        if (r[k] > 0.f) {
          if (y < 0 && a > th) y = base + k;
          lp = base + k;
        }
      }
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

// Inverse-CDF draw from the law with uniform u at the stop node (whole
// team).  Each member sums the law per slot of its share and the team
// exchanges the share totals; the member whose share holds u * S finds the
// element.  A workgroup alone after a timed-out exchange goes through every
// share in member order, with the totals rounded as the exchange rounds
// them, so it draws the token the team would.  A team of one takes its one
// share's total as it is.  fused: the law is p alone and s_slot holds this
// workgroup's share's slot sums from the node's statistics pass (relative to
// that pass's references), so no slot pass is needed.
template <int TDT, int DDT, int NT, int G>
__device__ __forceinline__ DrawOut team_draw(const Law& L, const void* prow, const void* qrow, int V,
                                             Team& tm, const int* ex, int nex, double u, bool fused,
                                             double* s_slot, float* s_sref, double* s_woff,
                                             int* s_sel, double* s_th, float* s_x, int* s_solo,
                                             float* ldsf, double* ldsd, int* ldsi) {
  DrawOut out{-1, false, false};
  const int tid = threadIdx.x;
  SlotScan sc;
  int sc_share;  // the share whose slot sums are in s_slot
  double total, before = 0.0;
  int owner = 0;
  bool past = false;
  const Geo geo = chunk_geo<TDT>(prow, 0, V);
  if constexpr (G == 1) {
    if (fused)
      rescale_slots<NT>(num_slots(row_range<G>(geo, -1)), L.ref_p, s_slot, s_sref);
    else
      slot_pass<TDT, DDT, NT, G>(L, prow, qrow, V, -1, s_slot);
    sc = slot_scan<TDT, DDT, NT, G>(L, prow, qrow, V, -1, ex, nex, s_slot, s_woff);
    sc_share = -1;
    total = sc.total;
  } else {
    bool have = false;  // s_x holds every share's total
    if (!tm.solo) {  // never alone so far: s_slot holds this member's share if fused
      if (fused)
        rescale_slots<NT>(num_slots(row_range<G>(geo, tm.gi)), L.ref_p, s_slot, s_sref);
      else
        slot_pass<TDT, DDT, NT, G>(L, prow, qrow, V, tm.gi, s_slot);
      sc = slot_scan<TDT, DDT, NT, G>(L, prow, qrow, V, tm.gi, ex, nex, s_slot, s_woff);
      sc_share = tm.gi;
      float mine[kXWords] = {};
      split_f64(sc.total, mine[0], mine[1]);
      exchange<G>(tm, mine, 2, s_x, s_solo);
      have = !tm.solo;
    }
    if (!have) {  // alone: every share in member order
      for (int m = 0; m < G; ++m) {
        share_slots<TDT, DDT, NT, G>(L, prow, qrow, V, m, fused, s_slot, s_sref, ldsf, ldsd, ldsi);
        sc = slot_scan<TDT, DDT, NT, G>(L, prow, qrow, V, m, ex, nex, s_slot, s_woff);
        sc_share = m;
        if (tid == 0) split_f64(sc.total, s_x[kXWords * m], s_x[kXWords * m + 1]);
      }
      __syncthreads();
    }
    total = 0.0;
    double acc = 0.0;
    int lastm = 0;
    owner = -1;
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const double tmm = join_f64(s_x[kXWords * m], s_x[kXWords * m + 1]);
      total += tmm;
    }
    const double theta = u * total;
#pragma unroll
    for (int m = 0; m < G; ++m) {
      const double tmm = join_f64(s_x[kXWords * m], s_x[kXWords * m + 1]);
      if (tmm > 0.0) {
        lastm = m;
        if (owner < 0 && acc <= theta && theta < acc + tmm) {
          owner = m;
          before = acc;
        }
      }
      acc += tmm;
    }
    if (owner < 0) {  // theta at or past the total: the last share with mass
      owner = lastm;
      past = true;
      before = 0.0;
#pragma unroll
      for (int m = 0; m < G; ++m)
        if (m < owner) before += join_f64(s_x[kXWords * m], s_x[kXWords * m + 1]);
    }
  }
  out.empty = !(total > 0.0);
  if (out.empty) return out;
  out.rounding = past;
  const int mine_share = G == 1 ? -1 : (tm.solo ? owner : tm.gi);
  if (G > 1 && owner != mine_share) return out;  // another member draws
  if (G > 1 && sc_share != owner) {  // alone: the owner's slot sums again
    share_slots<TDT, DDT, NT, G>(L, prow, qrow, V, owner, fused, s_slot, s_sref, ldsf, ldsd, ldsi);
    sc = slot_scan<TDT, DDT, NT, G>(L, prow, qrow, V, owner, ex, nex, s_slot, s_woff);
  }
  bool rounding = false;
  out.token = slot_find<TDT, DDT, NT, G>(L, prow, qrow, V, G == 1 ? -1 : owner, ex, nex, sc, before,
                                         u * total, past, s_slot, s_sel, s_th, &rounding);
  out.rounding = rounding;
  return out;
}

// The walk's per-child scalar math (fp64 exponentials, Philox).  Every lane
// computes the same value.
struct Odds {
  double px;     // p(x)
  double ratio;  // acceptance ratio of x under the current law
};

// 2^x for x <= 0 (an exponent against a row's reference): the integer part
// to the exponent, v_exp_f32 for the fraction, so as accurate as the
// exponentials the row sums hold (a few 1e-8 relative); 0 far below.
__device__ __forceinline__ double exp2_nonpos(double x) {
  if (!(x > -1070.0)) return 0.0;
  const double n = floor(x);
  return ldexp((double)fast_exp2((float)(x - n)), (int)n);
}

// mode 0: one-hot drafts (ratio p(x) / Zk, 0 for a removed token); 1: draft
// logits; 2: draft probabilities.
__device__ __forceinline__ Odds child_odds(float lp, float lq, float c, float pref, double pz,
                                        float qref, double qz, double ck, double Zk, int mode,
                                        bool removed) {
  Odds o;
  o.px = exp2_nonpos((double)lp * (double)c + (double)pref) / pz;
  if (mode == 0) {
    o.ratio = removed ? 0.0 : o.px / Zk;
  } else {
    const double qx =
        mode == 2 ? (double)lq : exp2_nonpos((double)lq * (double)c + (double)qref) / qz;
    double num = o.px - ck * qx;
    num = num > 0.0 ? num / Zk : 0.0;
    o.ratio = qx > 0.0 ? num / qx : (num > 0.0 ? __builtin_inf() : 0.0);
  }
  return o;
}

// The children of v among nodes [base, base + 64) below n, as a mask (bit
// l: node base + l), by one LDS read per lane and a ballot; the same in
// every wavefront.  A node is v's child iff it comes after v and names v as
// its parent, so a node whose parent is not an earlier node is nobody's.
__device__ __forceinline__ uint64_t kids_in(const int* s_par, int v, int base, int n) {
  const int j = base + (int)(threadIdx.x & 63);
  return __ballot(j > v && j < n && s_par[j] == v);
}

// The first child of v at or after node `from` (below n), or -1.
__device__ __forceinline__ int first_kid(const int* s_par, int v, int from, int n) {
  for (int base = from; base < n; base += 64) {
    const uint64_t k = kids_in(s_par, v, base, n);
    if (k != 0) return base + (int)__builtin_ctzll(k);
  }
  return -1;
}

struct Uniforms {
  double acc, rec;
};

__device__ __forceinline__ Uniforms tree_uniforms(uint64_t seed, uint64_t offset, int b, int i) {
  Uniforms u;
  uniforms(seed, offset, b, i, &u.acc, &u.rec);
  return u;
}

// NT threads per workgroup, G workgroups per team.  Team t walks request t,
// then (where teams are fewer than requests) the next free request from the
// launch's counter after each walk; member 0 writes the accepted path, the
// count, the last node and the padding, the member that draws writes the
// emitted token.
template <int TDT, int DDT, bool HAS_DRAFT, int NT, int G>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void k_tree(
    const TreeParams p) {
  constexpr int W = NT / 64;
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_ex[kMaxNodes];
  __shared__ float ldsf[W];
  __shared__ double ldsd[W];
  __shared__ int ldsi[W];
  __shared__ double s_woff[W];
  __shared__ float s_wm[2 * W];  // wavefront parts of a row pair's statistics
  __shared__ double s_ws[2 * W];
  __shared__ double s_slot[kMaxVocab / (256 * G) + 4];  // draw slots of a share: 64 vectors each
  __shared__ float s_sref[kMaxVocab / (256 * G) + 4];   // their references, from a statistics pass
  __shared__ int s_sel;
  __shared__ double s_th;
  __shared__ float s_x[kXWords * G];
  __shared__ int s_solo;
  __shared__ int s_path[kMaxNodes];  // the accepted path's tokens
  __shared__ int s_next;
  // the request's uniforms at each node index (24-bit values, exact in a
  // float): acceptance of child j + 1 from s_ua[j], the draw at node j from
  // s_ur[j]
  __shared__ float s_ua[kMaxNodes], s_ur[kMaxNodes];
  const int tid = threadIdx.x;
  const int N = p.N, V = p.V;
  Team tm;
  tm.xdat = p.xdat;
  tm.xdone = p.xdone;
  // a team's members on one XCD: workgroup i runs on XCD i % 8 under the
  // round-robin dispatch, and the grid is a whole number of 8 G workgroups
  // (team t's members are workgroups 8 (G (t / 8) + gi) + t % 8).  On one
  // XCD, members start together: the XCDs start a launch's workgroups up to
  // ~3 us apart, which a team spread over them waits out at its first
  // exchange.  The exchanges stay agent-scope, so placement only moves time.
  if constexpr (G == 1) {
    tm.gi = 0;
    tm.t = (int)blockIdx.x;
  } else {
    const int x = (int)(blockIdx.x % 8), j = (int)(blockIdx.x / 8);
    tm.gi = j % G;
    tm.t = (j / G) * 8 + x;
  }
  tm.k = 0;
  tm.solo = false;
  tm.spin = p.spin_ticks;
  const int teams = G == 1 ? (int)gridDim.x : (int)(gridDim.x / G);

  // the first request by team index; where teams walk several requests,
  // each further one is the next free request, taken at the end of a walk
  for (int b = tm.t; b < p.B;) {
    int n = p.nn[b];
    const float T = p.temps[b];  // in the same round trip as the count
    const bool bad_n = n < 1 || n > N;
    n = n < 1 ? 1 : (n > N ? N : n);
    __syncthreads();  // the previous request's tree is no longer read
    for (int i = tid; i < n; i += NT) {
      s_par[i] = p.parents[(size_t)b * N + i];
      s_tok[i] = p.tokens[(size_t)b * N + i];
    }
    __syncthreads();
    uint32_t fl = bad_n ? SV_DEVERR_BAD_NUM_DRAFTS : 0u;
    if (tm.gi == 0 && tid < 64) {  // every parent an earlier node: one ballot per 64 nodes
      bool bad = false;
      for (int i = tid; i < n; i += 64) bad |= i > 0 && (s_par[i] < 0 || s_par[i] >= i);
      if (__ballot(bad) != 0) fl |= SV_DEVERR_BAD_TREE;
    }

    const bool sampling = is_sampling(T);
    // one Philox block per node index, the request's indices in parallel
    // (the walk's tests and draw read them after the first pass's barriers)
    if (sampling)
      for (int j = tid; j < n; j += NT) {
        const Uniforms un = tree_uniforms(p.seed, p.offset, p.b_base + b, j);
        s_ua[j] = (float)un.acc;
        s_ur[j] = (float)un.rec;
      }
    const float c = sampling ? temp_scale(T) : 0.f;
    const bool probs = p.draft_is_probs != 0;
    int v = 0, nacc = 0, y = 0;
    bool drew = false;  // this member drew the emitted token
    int32_t* out = p.out_tokens + (size_t)b * N;

    for (;;) {
      const void* prow = row_ptr(p.target, TDT, (size_t)b * N + v, V);
      const void* qrow = HAS_DRAFT ? row_ptr(p.draft, DDT, (size_t)b * N + v, V) : nullptr;
      // q's statistics serve only the child tests: a node without children
      // draws from p alone
      const int kid0 = first_kid(s_par, v, v + 1, n);
      const bool has_kids = kid0 >= 0;
      const bool need_q = HAS_DRAFT && sampling && !probs && has_kids;
      // a sampling node without children draws from p alone: its statistics
      // pass keeps the draw's slot sums too, which saves the draw a pass
      const bool fuse = sampling && !has_kids;
      // the row statistics: the team's shares folded in member order; a
      // workgroup alone after a timed-out exchange computes every share itself
      // and folds the same words, so it gets the same bits
      RowStats ps, qs{0.f, 0.f, 1.0, 0};
      if constexpr (G == 1) {  // pair_stats measured slower at 1024 threads
        ps = solo_stats(fuse ? row_stats<TDT, NT, G, true>(prow, V, true, c, -1, ldsf, ldsd, ldsi,
                                                          s_slot, s_sref)
                             : row_stats<TDT, NT, G>(prow, V, sampling, c, -1, ldsf, ldsd, ldsi),
                        sampling);
        if (need_q) qs = row_stats<DDT, NT, G>(qrow, V, true, c, -1, ldsf, ldsd, ldsi);
      } else {
        bool have = false;
        for (int m = tm.solo ? 0 : tm.gi; !have; ++m) {  // own share; alone: 0 .. G-1
          RowStats a, bq{0.f, 0.f, 1.0, 0};
          if (need_q)
            pair_stats<TDT, DDT, NT, G>(prow, qrow, V, c, m, s_wm, s_ws, a, bq);
          else
            a = fuse ? row_stats<TDT, NT, G, true>(prow, V, true, c, m, ldsf, ldsd, ldsi, s_slot,
                                                   s_sref)
                     : row_stats<TDT, NT, G>(prow, V, sampling, c, m, ldsf, ldsd, ldsi);
          float mine[kXWords] = {};
          stat_words(a, bq, sampling, mine);
          if (!tm.solo) {
            exchange<G>(tm, mine, need_q ? 6 : (sampling ? 3 : 2), s_x, &s_solo);
            if (tm.solo) m = -1;  // timed out: start over, alone
            have = !tm.solo;
          } else {
            if (threadIdx.x == 0)
              for (int j = 0; j < 6; ++j) s_x[kXWords * m + j] = mine[j];
            __syncthreads();
            have = m == G - 1;
          }
        }
        if (need_q)
          fold_pair<G>(s_x, c, ps, qs);
        else
          ps = fold_stats<G>(s_x, 0, sampling, c);
      }

      // the children of v, in index order
      double ck = 0.0, Zk = 1.0;  // law after k rejections (probabilistic)
      int nex = 0, nrej = 0, next = -1;
      for (int ch = kid0; ch >= 0;) {
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
            const Odds o = child_odds(Elt<TDT>::at(prow, x), lq, c, ps.ref, ps.z, qs.ref,
                                      qs.z, ck, Zk, !HAS_DRAFT ? 0 : (probs ? 2 : 1),
                                      !HAS_DRAFT && excluded(s_ex, nex, x));
            px = o.px;
            ratio = o.ratio;
          }
          accept = (double)s_ua[ch - 1] < ratio;
          // one-hot: a rejected token leaves the law, which is renormalized
          if (!accept && !HAS_DRAFT && valid && !excluded(s_ex, nex, x)) Zk -= px;
        }
        if (accept) {
          next = ch;
          break;
        }
        ++nrej;
        const int after = first_kid(s_par, v, ch + 1, n);  // the next sibling
        if (sampling && !HAS_DRAFT) {
          if (valid && !excluded(s_ex, nex, x)) {
            __syncthreads();
            if (tid == 0) s_ex[nex] = x;
            __syncthreads();
            ++nex;
          }
        } else if (sampling) {  // the law left by this rejection: needs Z_{k+1}
          ck += Zk;
          if (after >= 0) {
            Law L{true, c, ps.ref, qs.ref, 0.f, 0.f, probs};
            const double kap = ck * ps.z / (probs ? 1.0 : qs.z);
            L.kap_hi = (float)kap;
            L.kap_lo = (float)(kap - (double)L.kap_hi);
            double zs;
            if constexpr (G == 1) {
              zs = law_sum<TDT, DDT, NT, G>(L, prow, qrow, V, -1, ldsd);
            } else {  // as for the row statistics
              bool have = false;
              for (int m = tm.solo ? 0 : tm.gi; !have; ++m) {
                const double zm = law_sum<TDT, DDT, NT, G>(L, prow, qrow, V, m, ldsd);
                float mine[kXWords] = {};
                split_f64(zm, mine[0], mine[1]);
                if (!tm.solo) {
                  exchange<G>(tm, mine, 2, s_x, &s_solo);
                  if (tm.solo) m = -1;
                  have = !tm.solo;
                } else {
                  if (threadIdx.x == 0) {
                    s_x[kXWords * m] = mine[0];
                    s_x[kXWords * m + 1] = mine[1];
                  }
                  __syncthreads();
                  have = m == G - 1;
                }
              }
              zs = fold_sum<G>(s_x);
            }
            Zk = zs / ps.z;
          }
        }
        ch = after;
      }
      if (next >= 0) {
        if (tid == 0) s_path[nacc] = s_tok[next];
        ++nacc;
        v = next;
        continue;
      }
      // every child rejected, or a leaf: the emitted token is drawn at v
      if (!sampling) {
        y = ps.arg;
        drew = tm.gi == 0 || tm.solo;
      } else {
        const double u_rec = (double)s_ur[v];
        Law L{false, c, ps.ref, qs.ref, 0.f, 0.f, probs};
        if (HAS_DRAFT && nrej > 0) {
          L.pair = true;
          const double kap = ck * ps.z / (probs ? 1.0 : qs.z);
          L.kap_hi = (float)kap;
          L.kap_lo = (float)(kap - (double)L.kap_hi);
        }
        DrawOut d = team_draw<TDT, DDT, NT, G>(L, prow, qrow, V, tm, s_ex, nex, u_rec, fuse, s_slot,
                                               s_sref, s_woff, &s_sel, &s_th, s_x, &s_solo, ldsf,
                                               ldsd, ldsi);
        if (d.empty) {  // no mass left: draw from p itself
          fl |= SV_DEVERR_ZERO_RESIDUAL;
          L.pair = false;
          d = team_draw<TDT, DDT, NT, G>(L, prow, qrow, V, tm, s_ex, 0, u_rec, false, s_slot, s_sref,
                                         s_woff, &s_sel, &s_th, s_x, &s_solo, ldsf, ldsd, ldsi);
        }
        y = d.token;
        drew = d.token >= 0;
        if (d.empty) {  // p itself has no mass (a row of -inf)
          y = -1;
          drew = tm.gi == 0 || tm.solo;
        }
        if (d.rounding) fl |= SV_DEVERR_DRAW_ROUNDING;
      }
      break;
    }
    if (tm.solo) fl |= SV_DEVERR_TREE_SYNC;
    // member 0 writes the path, the count and the last node, and any member
    // that finished the walk alone writes them too (the same values)
    const bool writer = tm.gi == 0 || tm.solo;
    __syncthreads();  // s_path is complete
    if (writer)
      for (int i = tid; i < N; i += NT)
        if (i != nacc) out[i] = i < nacc ? s_path[i] : -1;
    if (tid == 0) {
      if (drew) out[nacc] = y;
      if (writer) {
        p.out_nacc[b] = nacc;
        p.out_last[b] = v;
      }
      if (fl) atomicOr(p.flags, fl);
    }
    if constexpr (G == 1) {
      break;  // one request per workgroup
    } else {
      if (teams >= p.B) break;  // one request per team
      b = next_request<G>(tm, p.next_req, teams, s_x, &s_solo, &s_next);
    }
  }
  if constexpr (G > 1) team_done<G>(tm, teams < p.B ? p.next_req : nullptr, teams);
}

template <int TDT, int DDT, bool HD, int G>
const void* team_kernel() {
  return reinterpret_cast<const void*>(&k_tree<TDT, DDT, HD, kTeamThreads, G>);
}

template <int TDT, int DDT, bool HD, int G>
hipError_t launch_team(const TreeParams& p, int teams, hipStream_t s) {
  hipLaunchKernelGGL((k_tree<TDT, DDT, HD, kTeamThreads, G>), dim3((unsigned)(teams * G)),
                     dim3(kTeamThreads), 0, s, p);
  return hipGetLastError();
}

template <int TDT, int DDT, bool HD>
hipError_t launch_one(const TreeParams& p, int g, int teams, hipStream_t s) {
  if (g == 8) return launch_team<TDT, DDT, HD, 8>(p, teams, s);
  if (g == 4) return launch_team<TDT, DDT, HD, 4>(p, teams, s);
  hipLaunchKernelGGL((k_tree<TDT, DDT, HD, kSoloThreads, 1>), dim3((unsigned)p.B),
                     dim3(kSoloThreads), 0, s, p);
  return hipGetLastError();
}

template <int G>
const void* team_kernel_for(int tdt, int ddt, bool has_draft) {
  const bool t32 = tdt == SV_F32, d32 = ddt == SV_F32;
  if (has_draft)
    return t32 ? (d32 ? team_kernel<SV_F32, SV_F32, true, G>() : team_kernel<SV_F32, SV_BF16, true, G>())
               : (d32 ? team_kernel<SV_BF16, SV_F32, true, G>()
                      : team_kernel<SV_BF16, SV_BF16, true, G>());
  return t32 ? (d32 ? team_kernel<SV_F32, SV_F32, false, G>() : team_kernel<SV_F32, SV_BF16, false, G>())
             : (d32 ? team_kernel<SV_BF16, SV_F32, false, G>()
                    : team_kernel<SV_BF16, SV_BF16, false, G>());
}

}  // namespace

int tree_team_words() { return 2 * kXWords; }

int tree_team_capacity(int device, int tdt, int ddt, bool has_draft, int g) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (g != 4 && g != 8) return 0;
  const void* f = g == 8 ? team_kernel_for<8>(tdt, ddt, has_draft)
                         : team_kernel_for<4>(tdt, ddt, has_draft);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kTeamThreads, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return per_cu * cus / g;
}

int tree_team_pick(int B, const int cap[2]) {
  // measured on MI355X (random trees of 16 nodes, V = 152064 bf16): eight
  // members per request while the teams of eight that fit the device walk
  // at most two requests each (B <= 256 on 256 compute units: B = 160 103
  // against 116 us with teams of four, B = 192 113 against 118, B = 224 125
  // against 131, B = 256 144 against 146), four beyond (B = 288: 143 against
  // 152; B = 512: 208 against 234), where teams of four that walk several
  // requests each also beat one 1024-thread workgroup per request (B = 320:
  // 165 against 235 us; B = 512: 226 against 297; B = 768: 302 against 402)
  const int fit8 = cap[1] / 8 * 8;
  if (fit8 >= 8 && tree_team_slots(B) <= 2 * fit8) return 8;
  if (cap[0] >= 8) return 4;
  return 1;
}

int tree_team_count(int B, int g, const int cap[2]) {
  if (g <= 1) return B;
  const int fit = cap[g == 8 ? 1 : 0] / 8 * 8;
  const int slots = tree_team_slots(B);
  return slots < fit ? slots : fit;
}

hipError_t launch_tree(const TreeParams& p, int tdt, int ddt, int g, int teams, hipStream_t s) {
  const bool d = p.draft != nullptr;
#define SV_TREE_LAUNCH(T, D) \
  return d ? launch_one<T, D, true>(p, g, teams, s) : launch_one<T, D, false>(p, g, teams, s);
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
}

}  // namespace sv
