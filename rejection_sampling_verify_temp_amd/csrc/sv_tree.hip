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
//   - where the walk stops, the emitted token is drawn by inverse CDF: each
//     wavefront sums its 64-vector slot of every strided pass, a workgroup
//     scan over the slot sums finds the slot holding u * S, and one
//     wavefront re-reads that slot to find the element.
// All row passes use 16-byte loads, four per thread in flight.
// The walk is sequential per request; requests run in parallel.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / 64;
constexpr int kMaxNodes = SPEC_TREE_MAX_NODES;

// Online softmax of the elements a thread visits (in increasing order).
__device__ __forceinline__ void sm_add(float x, float c, float& m, float& R, float& S) {
  if (x > m) {
    const float rn = ref_of(x, c);
    S = (m == kNegInf) ? 0.f : S * fast_exp2(rn - R);
    R = rn;
    m = x;
  }
  S += fast_exp2(fmaf(x, c, R));
}

struct RowStats {
  float m;     // row max
  float ref;   // exponent reference ref_of(m, c)
  double z;    // sum of exp2(l c + ref)
  int arg;     // lowest index of the max (greedy)
};

// A row is a scalar head [0, v0) up to the first 16-byte boundary, nvec
// vectors from v0 and a scalar tail [t0, V) (chunk_geo over the whole row).
// Vectors are strided over the workgroup, 4 per thread in flight.
constexpr int kTreeUnroll = 4;

__device__ __forceinline__ const u32x4* vec_base(const void* row, const Geo& g, int bytes) {
  return reinterpret_cast<const u32x4*>(static_cast<const char*>(row) + (size_t)g.v0 * bytes);
}

// Statistics of one row (whole workgroup).  Each thread visits its elements
// in increasing index order (head, its vectors, tail), so the first max it
// meets is its lowest.
template <int DT>
__device__ RowStats row_stats(const void* row, int V, bool sampling, float c, float* ldsf,
                              double* ldsd, int* ldsi) {
  using E = Elt<DT>;
  const int tid = threadIdx.x;
  const Geo g = chunk_geo<DT>(row, 0, V);
  const u32x4* vp = vec_base(row, g, E::kBytes);
  float m = kNegInf, R = 0.f, S = 0.f;
  int arg = INT32_MAX;
  auto visit = [&](float x, int i) {
    if (sampling) {
      sm_add(x, c, m, R, S);
    } else if (x > m) {
      m = x;
      arg = i;
    }
  };
  if (tid < g.v0) visit(E::at(row, tid), tid);
  for (int v = tid; v < g.nvec; v += kTreeUnroll * kTreeThreads) {
    u32x4 d[kTreeUnroll];
#pragma unroll
    for (int u = 0; u < kTreeUnroll; ++u)
      if (v + u * kTreeThreads < g.nvec) d[u] = vp[v + u * kTreeThreads];
#pragma unroll
    for (int u = 0; u < kTreeUnroll; ++u) {
      const int vi = v + u * kTreeThreads;
      if (vi < g.nvec) {
        float x[E::kVec];
        E::unpack(d[u], x);
#pragma unroll
        for (int k = 0; k < E::kVec; ++k) visit(x[k], g.v0 + vi * E::kVec + k);
      }
    }
  }
  if (g.t0 + tid < V) visit(E::at(row, g.t0 + tid), g.t0 + tid);
  RowStats st;
  if (sampling) {
    st.m = block_max<kTreeThreads>(m, ldsf);
    st.ref = ref_of(st.m, c);
    double contrib = 0.0;
    if (S != 0.f && st.m != kNegInf) contrib = (double)S * exp2((double)st.ref - (double)R);
    st.z = block_sum<kTreeThreads>(contrib, ldsd);
    st.arg = 0;
  } else {
    block_argmax<kTreeThreads>(m, arg, ldsf, ldsi);
    st.m = m;
    st.arg = arg == INT32_MAX ? 0 : arg;
    st.ref = 0.f;
    st.z = 0.0;
  }
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

// Sum of the law over the row (whole workgroup, fp64 across threads).
template <int TDT, int DDT>
__device__ double law_sum(const Law& L, const void* prow, const void* qrow, int V, double* ldsd) {
  using EP = Elt<TDT>;
  const int tid = threadIdx.x;
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  const bool qvec = L.pair && same_alignment(prow, qrow);
  double acc = 0.0;
  if (tid < g.v0) acc += (double)law_at<TDT, DDT>(L, prow, qrow, tid);
  for (int v = tid; v < g.nvec; v += kTreeUnroll * kTreeThreads) {
    float s[kTreeUnroll];
#pragma unroll
    for (int u = 0; u < kTreeUnroll; ++u) {
      s[u] = 0.f;
      if (v + u * kTreeThreads < g.nvec) {
        float r[EP::kVec];
        law_vec<TDT, DDT>(L, prow, qrow, g, v + u * kTreeThreads, qvec, r);
        s[u] = pairwise_sum(r);
      }
    }
    acc += (double)pairwise_sum(s);
  }
  if (g.t0 + tid < V) acc += (double)law_at<TDT, DDT>(L, prow, qrow, g.t0 + tid);
  return block_sum<kTreeThreads>(acc, ldsd);
}

__device__ __forceinline__ bool excluded(const int* ex, int nex, int i) {
  for (int k = 0; k < nex; ++k)
    if (ex[k] == i) return true;
  return false;
}

// Inverse-CDF draw from the law with uniform u (whole workgroup); the tokens
// in ex[0..nex) are removed.  The row is cut into slots: 0 = the head, then
// one slot per 64 vectors (one wavefront's share of one strided iteration,
// summed by that wavefront), then the tail.  A workgroup scan over the slot
// sums finds the slot holding u * S, and wavefront 0 re-reads only that slot
// (one vector per lane) to find the element.  Returns the token; *rounding
// is set if u * S fell past the recomputed total, *empty if the law is 0.
template <int TDT, int DDT>
__device__ int law_draw(const Law& L, const void* prow, const void* qrow, int V, const int* ex,
                        int nex, double u, double* s_slot, double* s_woff, int* s_sel,
                        double* s_th, bool* rounding, bool* empty) {
  using EP = Elt<TDT>;
  constexpr int KV = EP::kVec;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const Geo g = chunk_geo<TDT>(prow, 0, V);
  const bool qvec = L.pair && same_alignment(prow, qrow);
  const int npieces = (g.nvec + 63) / 64, nslot = npieces + 2;

  // (1) slot sums
  for (int j = 0; j * kTreeThreads < g.nvec; ++j) {
    const int vi = j * kTreeThreads + tid;
    float sv = 0.f;
    if (vi < g.nvec) {
      float r[KV];
      law_vec<TDT, DDT>(L, prow, qrow, g, vi, qvec, r);
      sv = pairwise_sum(r);
    }
    const double ws = wave_sum((double)sv);
    if (lane == 0 && j * kTreeWaves + w < npieces) s_slot[1 + j * kTreeWaves + w] = ws;
  }
  if (w == 0) {
    const double h = wave_sum(lane < g.v0 ? (double)law_at<TDT, DDT>(L, prow, qrow, lane) : 0.0);
    const double t =
        wave_sum(g.t0 + lane < V ? (double)law_at<TDT, DDT>(L, prow, qrow, g.t0 + lane) : 0.0);
    if (lane == 0) {
      s_slot[0] = h;
      s_slot[nslot - 1] = t;
    }
  }
  __syncthreads();
  if (tid == 0) {  // removed tokens leave their slots
    for (int k = 0; k < nex; ++k) {
      const int e = ex[k];
      const int sl = e < g.v0 ? 0 : (e >= g.t0 ? nslot - 1 : 1 + (e - g.v0) / KV / 64);
      s_slot[sl] -= (double)law_at<TDT, DDT>(L, prow, qrow, e);
    }
    for (int k = 0; k < nex; ++k) {  // rounding can leave a tiny negative
      const int e = ex[k];
      const int sl = e < g.v0 ? 0 : (e >= g.t0 ? nslot - 1 : 1 + (e - g.v0) / KV / 64);
      if (!(s_slot[sl] > 0.0)) s_slot[sl] = 0.0;
    }
    *s_sel = -1;
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
  double q = __shfl_up(incl, 1, 64);
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
#pragma unroll
    for (int k = 0; k < KV; ++k)
      if (k >= cnt || (nex > 0 && excluded(ex, nex, base + k))) r[k] = 0.f;
    double ls = 0.0;
#pragma unroll
    for (int k = 0; k < KV; ++k) ls += (double)r[k];
    const double li = wave_incl_scan(ls, lane);
    double before = __shfl_up(li, 1, 64);
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
          px = exp2((double)Elt<TDT>::at(prow, x) * (double)c + (double)ps.ref) / ps.z;
          if (!HAS_DRAFT) {
            ratio = excluded(s_ex, nex, x) ? 0.0 : px / Zk;
          } else {
            const double lq = (double)Elt<DDT>::at(qrow, x);
            const double qx = probs ? lq : exp2(lq * (double)c + (double)qs.ref) / qs.z;
            double num = px - ck * qx;
            num = num > 0.0 ? num / Zk : 0.0;
            ratio = qx > 0.0 ? num / qx : (num > 0.0 ? __builtin_inf() : 0.0);
          }
        }
        double u_acc, u_rec;
        uniforms(p.seed, p.offset, b, ch - 1, &u_acc, &u_rec);
        accept = u_acc < ratio;
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
      double u_acc, u_rec;
      uniforms(p.seed, p.offset, b, v, &u_acc, &u_rec);
      Law L{false, c, ps.ref, qs.ref, 0.f, 0.f, probs};
      if (HAS_DRAFT && nrej > 0) {
        L.pair = true;
        const double kap = ck * ps.z / (probs ? 1.0 : qs.z);
        L.kap_hi = (float)kap;
        L.kap_lo = (float)(kap - (double)L.kap_hi);
      }
      bool rounding = false, empty = false;
      y = law_draw<TDT, DDT>(L, prow, qrow, V, s_ex, nex, u_rec, s_slot, s_woff, &s_sel, &s_th,
                             &rounding, &empty);
      if (empty) {  // no residual mass: draw from p itself
        fl |= SV_DEVERR_ZERO_RESIDUAL;
        L.pair = false;
        y = law_draw<TDT, DDT>(L, prow, qrow, V, s_ex, 0, u_rec, s_slot, s_woff, &s_sel, &s_th,
                               &rounding, &empty);
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

bool aligned(const void* ptr, int a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

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
