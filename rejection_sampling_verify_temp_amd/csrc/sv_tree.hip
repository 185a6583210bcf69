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
//   - where the walk stops, the emitted token is drawn by inverse CDF:
//     every thread sums a contiguous segment, a workgroup scan finds the
//     segment holding u * S, and its thread walks it.
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

// Statistics of one row (whole workgroup; strided, 8 loads in flight).
template <int DT>
__device__ RowStats row_stats(const void* row, int V, bool sampling, float c, float* ldsf,
                              double* ldsd, int* ldsi) {
  const int tid = threadIdx.x;
  float m = kNegInf, R = 0.f, S = 0.f;
  int arg = INT32_MAX;
  for (int i0 = tid; i0 < V; i0 += 8 * kTreeThreads) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kTreeThreads;
      x[u] = i < V ? Elt<DT>::at(row, i) : kNegInf;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kTreeThreads;
      if (i >= V) continue;
      if (sampling) {
        sm_add(x[u], c, m, R, S);
      } else if (x[u] > m) {  // indices ascend per thread: first max wins
        m = x[u];
        arg = i;
      }
    }
  }
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

template <int TDT, int DDT>
__device__ __forceinline__ float law_at(const Law& L, const void* prow, const void* qrow, int i) {
  const float pt = fast_exp2(fmaf(Elt<TDT>::at(prow, i), L.c, L.ref_p));
  if (!L.pair) return pt;
  const float lq = Elt<DDT>::at(qrow, i);
  const float qt = L.probs ? lq : fast_exp2(fmaf(lq, L.c, L.ref_q));
  float r = fmaf(-qt, L.kap_hi, pt);
  r = fmaf(-qt, L.kap_lo, r);
  return r > 0.f ? r : 0.f;
}

// Sum of the law over the row (whole workgroup, fp64 across threads).
template <int TDT, int DDT>
__device__ double law_sum(const Law& L, const void* prow, const void* qrow, int V, double* ldsd) {
  double acc = 0.0;
  for (int i0 = threadIdx.x; i0 < V; i0 += 8 * kTreeThreads) {
    float r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kTreeThreads;
      r[u] = i < V ? law_at<TDT, DDT>(L, prow, qrow, i) : 0.f;
    }
    acc += (double)pairwise_sum(r);
  }
  return block_sum<kTreeThreads>(acc, ldsd);
}

__device__ __forceinline__ bool excluded(const int* ex, int nex, int i) {
  for (int k = 0; k < nex; ++k)
    if (ex[k] == i) return true;
  return false;
}

// Inverse-CDF draw from the law with uniform u (whole workgroup).  The
// tokens in ex[0..nex) are removed.  Returns the token; *rounding is set if
// u * S fell past the recomputed total.
template <int TDT, int DDT>
__device__ int law_draw(const Law& L, const void* prow, const void* qrow, int V, const int* ex,
                        int nex, double u, double* s_woff, int* s_y, int* s_lastseg,
                        bool* rounding, bool* empty) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int seglen = (V + kTreeThreads - 1) / kTreeThreads;
  const int i0 = min(V, tid * seglen), i1 = min(V, i0 + seglen);
  double seg = 0.0;
  for (int i = i0; i < i1; ++i) seg += (double)law_at<TDT, DDT>(L, prow, qrow, i);
  for (int k = 0; k < nex; ++k)  // removed tokens: their owner takes them out
    if (ex[k] >= i0 && ex[k] < i1 && !excluded(ex, k, ex[k]))
      seg -= (double)law_at<TDT, DDT>(L, prow, qrow, ex[k]);
  if (!(seg > 0.0)) seg = 0.0;
  // exclusive scan of the segment sums
  const double incl = wave_incl_scan(seg, lane);
  if (lane == 63) s_woff[w] = incl;
  double q = __shfl_up(incl, 1, 64);
  if (lane == 0) q = 0.0;
  if (tid == 0) {
    *s_y = INT32_MAX;
    *s_lastseg = -1;
  }
  __syncthreads();
  if (seg > 0.0) atomicMax(s_lastseg, tid);
  double total = 0.0;
  for (int k = 0; k < kTreeWaves; ++k) {
    if (k < w) q += s_woff[k];
    total += s_woff[k];
  }
  __syncthreads();
  *empty = !(total > 0.0);
  if (*empty) return -1;
  const double theta = u * total;
  const bool mine = seg > 0.0 && q <= theta && theta < q + seg;
  const bool past = *s_lastseg == tid && !(theta < q + seg);
  int ymine = INT32_MAX;
  if (mine || past) {
    double acc = q;
    int y = -1, lp = -1;
    for (int i = i0; i < i1; ++i) {
      float r = law_at<TDT, DDT>(L, prow, qrow, i);
      if (nex > 0 && excluded(ex, nex, i)) r = 0.f;
      acc += (double)r;
      if (r > 0.f) {
        if (y < 0 && mine && acc > theta) y = i;
        lp = i;
      }
    }
    ymine = y >= 0 ? y : lp;
    if (ymine < 0) ymine = INT32_MAX;
    if (mine) atomicMin(s_y, ymine);
  }
  __syncthreads();
  int y = *s_y;
  *rounding = false;
  if (y == INT32_MAX) {  // theta past the recomputed total: last positive element
    *rounding = true;
    __syncthreads();
    if (past && ymine != INT32_MAX) *s_y = ymine;
    __syncthreads();
    y = *s_y;
    if (y == INT32_MAX) y = 0;
  }
  return y;
}

template <int TDT, int DDT, bool HAS_DRAFT>
__global__ __launch_bounds__(kTreeThreads) void k_tree(const TreeParams p) {
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_ex[kMaxNodes];
  __shared__ float ldsf[kTreeWaves];
  __shared__ double ldsd[kTreeWaves];
  __shared__ int ldsi[kTreeWaves];
  __shared__ double s_woff[kTreeWaves];
  __shared__ int s_y, s_lastseg;
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
      y = law_draw<TDT, DDT>(L, prow, qrow, V, s_ex, nex, u_rec, s_woff, &s_y, &s_lastseg,
                             &rounding, &empty);
      if (empty) {  // no residual mass: draw from p itself
        fl |= SV_DEVERR_ZERO_RESIDUAL;
        L.pair = false;
        y = law_draw<TDT, DDT>(L, prow, qrow, V, s_ex, 0, u_rec, s_woff, &s_y, &s_lastseg,
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
