// Internal types shared by the host API and the kernels of the verify step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

constexpr int kThreads = 256;        // every workgroup: four wavefronts
constexpr int kMaxChunkElems = 15360; // the draw stages one chunk of floats in LDS
constexpr int kMinChunkElems = 256;
constexpr int kMaxChunks = 64;     // one lane per chunk when a request is combined
// Tuning knobs: workgroups that share one chunk of a residual pair, each
// summing a contiguous part of it, for bf16 rows and for pairs with an fp32
// row.  The residual sums hold kResidSplitMax values per chunk.
#ifndef SV_RESID_SPLIT_BF16
#define SV_RESID_SPLIT_BF16 2
#endif
#ifndef SV_RESID_SPLIT_F32
#define SV_RESID_SPLIT_F32 4
#endif
constexpr int kResidSplitMax =
    SV_RESID_SPLIT_BF16 > SV_RESID_SPLIT_F32 ? SV_RESID_SPLIT_BF16 : SV_RESID_SPLIT_F32;
constexpr int kMaxVocab = kMaxChunks * kMaxChunkElems;
constexpr int kMaxDrafts = 31;       // the 2K+1 row slots fit one wavefront

// Per (row, vocabulary chunk) statistics.  Sampling rows: m = chunk max,
// z = sum over the chunk of exp2(l_i * c + ref(m, c)), idx = the count of
// elements above the draft's logit under typical acceptance (else unused).
// Greedy rows: m = chunk max, idx = lowest index attaining it.
struct __align__(16) Partial {
  float m;
  int32_t idx;
  double z;
};

enum DrawKind : int32_t {
  kDrawNone = 0,    // greedy request: token already written
  kDrawSingle = 1,  // draw from the target row (x removed if x >= 0)
  kDrawPair = 2     // draw from max(0, p - q) of a row pair
};

// Per-request draw descriptor written by the decision kernel.
struct __align__(16) DrawDesc {
  int32_t kind;
  int32_t j;       // position whose token is drawn
  int32_t x;       // token removed from the law, or -1
  int32_t cstar;   // chunk holding the draw, or -1 if the draw kernel picks it
  float c;         // log2(e) / T
  float ref_p;     // exponent reference of the target row
  float ref_q;     // exponent reference of the draft row (logit drafts)
  float kap_hi;    // kappa = Z_p / Z_q (or Z_p for probability drafts),
  float kap_lo;    //   split into two floats
  float pad1;
  double z_p;      // target row total relative to ref_p
  double u;        // draw uniform
  double th;       // with cstar >= 0: u * S less the mass of chunks before cstar
                   // (relative to ref_p); +inf if rounding left u * S past the end
};

struct RunParams {
  const void* target;
  const void* draft;
  const uint8_t* mode;
  const int32_t* ids;
  const int32_t* nd;
  const float* temps;
  int32_t* out_tokens;
  int32_t* out_nacc;
  float* out_dbg;
  Partial* part;
  DrawDesc* desc;
  double* rsum;
  uint32_t* flags;
  uint64_t seed;
  uint64_t offset;
  int32_t B, K, V;
  int32_t chunk;    // elements per chunk
  int32_t nchunk;   // ceil(V / chunk)
  int32_t draft_is_probs;
  int32_t has_draft;
  int32_t b_base;      // batch index of request 0 (Philox counters use b_base + b)
  // Draft sampler: 0 for the verify step.  Otherwise each "request" is one
  // draft row (b / sample_k, b % sample_k) of a [B][sample_k][V] logits
  // buffer (passed as `target`, K = 0), drawn from softmax(l / T_b).
  int32_t sample_k;
  float* out_q;        // sampler: q(x) of each drawn token, or nullptr
  // Typical acceptance (no draft rows): accept x_j iff p_j(x_j) > eps or
  // #{i : l_i > l_x} < top_k; the statistics pass then also counts, per
  // chunk, the elements above l_x (into Partial::idx).
  int32_t typical;
  float eps;
  int32_t top_k;
  // Nonzero: the statistics kernel zeroes *flags before any kernel of the
  // step can set a bit (a step that owns no sticky flag word).
  int32_t clear_flags;
};

constexpr int kNumKernels = 4;
enum KernelId { kKernelStats = 0, kKernelDecide = 1, kKernelResid = 2, kKernelLocate = 3 };

// Enqueue kernel k of a step (for the requests p describes) on `stream`.
// lds_per_cu (bytes of LDS per compute unit, 0 if unknown) sets the stats
// kernel's occupancy cap.
hipError_t launch_kernel(int k, const RunParams& p, int target_dtype, int draft_dtype,
                         int lds_per_cu, hipStream_t stream);

const char* kernel_name(int i);

// Whether launch_kernel(k, p, ...) launches anything for these parameters
// (the draft sampler has no decisions; runs without draft rows no residual).
bool kernel_launched(int k, const RunParams& p);

}  // namespace sv
