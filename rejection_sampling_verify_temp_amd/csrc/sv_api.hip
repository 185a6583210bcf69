// Host side of the verify-step C ABI: argument checks, the workspace, and
// the launches (see spec_verify.h for the contract).
#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>

#include "sv_internal.h"
#include "sv_tree.h"

namespace {

constexpr int kTimingSlots = 64;
constexpr int kEventsPerRun = 2 * sv::kNumKernels;

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(dev) == hipSuccess) ok = true;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elt_bytes(int dt) { return dt == SV_BF16 ? 2 : 4; }

// Chunk length: about 32 KiB of the wider input per workgroup, at least
// V / 64 (a request's chunks are combined one per lane), balanced so the
// chunks of a row are of near-equal length, a multiple of 64 elements.
int pick_chunk(const sv_config& c) {
  int want = c.chunk_elems;
  if (want == 0) {
    const int wide = elt_bytes(c.target_dtype) > elt_bytes(c.draft_dtype)
                         ? elt_bytes(c.target_dtype) : elt_bytes(c.draft_dtype);
    want = 32768 / wide;
  }
  const int V = c.vocab;
  int n = (V + want - 1) / want;
  if (n > sv::kMaxChunks) n = sv::kMaxChunks;
  int ch = (V + n - 1) / n;
  ch = ((ch + 63) / 64) * 64;
  if (ch < sv::kMinChunkElems) ch = sv::kMinChunkElems;
  if (ch > sv::kMaxChunkElems) ch = sv::kMaxChunkElems;
  return ch;
}

// The checks spec_verify_create makes on a configuration (status code).
int check_config(const sv_config& c) {
  if (c.max_batch < 1 || c.max_drafts < 0 || c.max_drafts > sv::kMaxDrafts ||
      c.vocab < 1 || c.vocab > sv::kMaxVocab || c.device < 0)
    return SV_ERR_INVALID_ARG;
  if ((c.target_dtype != SV_F32 && c.target_dtype != SV_BF16) ||
      (c.draft_dtype != SV_F32 && c.draft_dtype != SV_BF16) ||
      (c.draft_is_probs != 0 && c.draft_is_probs != 1))
    return SV_ERR_UNSUPPORTED;
  if (c.chunk_elems != 0 &&
      (c.chunk_elems % 64 != 0 || c.chunk_elems < sv::kMinChunkElems ||
       c.chunk_elems > sv::kMaxChunkElems))
    return SV_ERR_INVALID_ARG;
  return SV_OK;
}

// The argument checks of a verify step (status code; SV_OK for B == 0 too).
int check_run_args(const sv_config& c, int32_t B, int32_t K, const void* target_logits,
                   const void* draft_probs, const int32_t* draft_ids,
                   const int32_t* num_drafts_per_req, const float* temperatures,
                   const int32_t* out_tokens, const int32_t* out_num_accepted,
                   const float* out_debug_probs) {
  if (B < 0 || K < 0) return SV_ERR_INVALID_ARG;
  if (B > c.max_batch || K > c.max_drafts) return SV_ERR_CAPACITY;
  if (B == 0) return SV_OK;
  if (target_logits == nullptr || num_drafts_per_req == nullptr ||
      temperatures == nullptr || out_tokens == nullptr || out_num_accepted == nullptr ||
      (K > 0 && draft_ids == nullptr))
    return SV_ERR_INVALID_ARG;
  if (!aligned(target_logits, elt_bytes(c.target_dtype)) ||
      (draft_probs != nullptr && !aligned(draft_probs, elt_bytes(c.draft_dtype))) ||
      (draft_ids != nullptr && !aligned(draft_ids, 4)) || !aligned(num_drafts_per_req, 4) ||
      !aligned(temperatures, 4) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
      (out_debug_probs != nullptr && !aligned(out_debug_probs, 4)))
    return SV_ERR_INVALID_ARG;
  return SV_OK;
}

// Parameters of a verify step (the workspace pointers are left to the caller).
sv::RunParams verify_params(const sv_config& c, int chunk, int nchunk, int32_t B, int32_t K,
                            const void* target_logits, const void* draft_probs,
                            const uint8_t* draft_mode, const int32_t* draft_ids,
                            const int32_t* num_drafts_per_req, const float* temperatures,
                            uint64_t philox_seed, uint64_t philox_offset,
                            int32_t* out_tokens, int32_t* out_num_accepted,
                            float* out_debug_probs) {
  sv::RunParams p{};
  p.target = target_logits;
  p.draft = draft_probs;
  p.mode = draft_mode;
  p.ids = draft_ids;
  p.nd = num_drafts_per_req;
  p.temps = temperatures;
  p.out_tokens = out_tokens;
  p.out_nacc = out_num_accepted;
  p.out_dbg = out_debug_probs;
  p.seed = philox_seed;
  p.offset = philox_offset;
  p.B = B;
  p.K = K;
  p.V = c.vocab;
  p.chunk = chunk;
  p.nchunk = nchunk;
  p.draft_is_probs = c.draft_is_probs;
  p.has_draft = draft_probs != nullptr;
  return p;
}

}  // namespace

struct spec_verify_s {
  sv_config cfg;
  int chunk = 0;
  int nchunk = 0;
  sv::Partial* part = nullptr;
  sv::DrawDesc* desc = nullptr;
  double* rsum = nullptr;
  uint32_t* flags = nullptr;
  hipStream_t last_stream = nullptr;
  bool has_run = false;
  int32_t b_base = 0;  // global index of request 0 (spec_verify_set_request_base)
  int lds_per_cu = 0;  // bytes of LDS per compute unit (0: unknown, stats launches uncapped)
  // token trees: teams of 4 and 8 resident at once (without and with draft
  // rows; 0: no team walks) and their exchange words and counters (all 0
  // between launches)
  int tree_cap[2][2] = {{0, 0}, {0, 0}};
  uint64_t* tree_xdat = nullptr;
  uint32_t* tree_xdone = nullptr;
  uint32_t* tree_next = nullptr;  // [2] request counter of teams that walk several
  uint64_t tree_wait_ticks = 2000000;
  int tree_force = 0;  // members per request set by the caller (0: the pick)  // 20 ms of the 100 MHz real-time clock
  // timing: per run, one start/stop pair per kernel
  bool timing = false;
  hipEvent_t ev[kTimingSlots][kEventsPerRun] = {};
  uint32_t ev_launched[kTimingSlots] = {};  // per event set: the kernels it timed
  int ev_pending = 0;  // event sets recorded and not yet read
  int ev_next = 0;     // next ring slot
  double tot_ms[sv::kNumKernels] = {};
  int runs = 0;
};

namespace {

void free_all(spec_verify_s* h) {
  if (h->part) (void)hipFree(h->part);
  if (h->desc) (void)hipFree(h->desc);
  if (h->rsum) (void)hipFree(h->rsum);
  if (h->flags) (void)hipFree(h->flags);
  if (h->tree_xdat) (void)hipFree(h->tree_xdat);
  if (h->tree_xdone) (void)hipFree(h->tree_xdone);
  if (h->tree_next) (void)hipFree(h->tree_next);
  for (int s = 0; s < kTimingSlots; ++s)
    for (int k = 0; k < kEventsPerRun; ++k)
      if (h->ev[s][k]) (void)hipEventDestroy(h->ev[s][k]);
}

// Fold the oldest pending event set into the totals.
hipError_t drain_one(spec_verify_s* h) {
  const int slot = (h->ev_next - h->ev_pending + kTimingSlots) % kTimingSlots;
  for (int k = 0; k < sv::kNumKernels; ++k) {
    if (!(h->ev_launched[slot] & (1u << k))) continue;  // not launched in that run
    hipEvent_t* e = &h->ev[slot][2 * k];
    hipError_t err = hipEventSynchronize(e[1]);
    if (err != hipSuccess) return err;
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, e[0], e[1]);
    if (err != hipSuccess) return err;
    h->tot_ms[k] += ms;
  }
  h->runs++;
  h->ev_pending--;
  return hipSuccess;
}

// Enqueue the step's kernels on `stream`, with per-kernel events when
// timing is on.
int enqueue(spec_verify_s* h, const sv::RunParams& p, int tdt, int ddt, void* stream) {
  DeviceGuard g(h->cfg.device);
  if (!g.ok) return SV_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = nullptr;
  if (h->timing) {
    if (h->ev_pending == kTimingSlots && drain_one(h) != hipSuccess) return SV_ERR_HIP;
    ev = h->ev[h->ev_next];
  }
  bool ok = true;
  uint32_t launched = 0;
  for (int k = 0; ok && k < sv::kNumKernels; ++k) {
    if (!sv::kernel_launched(k, p)) continue;
    launched |= 1u << k;
    hipEvent_t* e = ev ? &ev[2 * k] : nullptr;
    ok = (!e || hipEventRecord(e[0], s) == hipSuccess) &&
         sv::launch_kernel(k, p, tdt, ddt, h->lds_per_cu, s) == hipSuccess &&
         (!e || hipEventRecord(e[1], s) == hipSuccess);
  }
  if (!ok) return SV_ERR_HIP;
  if (h->timing) {
    h->ev_launched[h->ev_next] = launched;
    h->ev_next = (h->ev_next + 1) % kTimingSlots;
    h->ev_pending++;
  }
  h->last_stream = s;
  h->has_run = true;
  return SV_OK;
}

}  // namespace

extern "C" {

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported dtype or option";
    case SV_ERR_CAPACITY: return "batch or draft count above the handle's maxima";
    case SV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* spec_verify_kernel_name(int32_t i) { return sv::kernel_name(i); }

int spec_verify_create(const sv_config* cfg, spec_verify_t* out) {
  if (out == nullptr) return SV_ERR_INVALID_ARG;
  *out = nullptr;
  if (cfg == nullptr) return SV_ERR_INVALID_ARG;
  const sv_config c = *cfg;
  const int rc = check_config(c);
  if (rc != SV_OK) return rc;

  DeviceGuard g(c.device);
  if (!g.ok) return SV_ERR_HIP;
  const int chunk = pick_chunk(c);
  const int nchunk = (c.vocab + chunk - 1) / chunk;
  if (nchunk > sv::kMaxChunks) return SV_ERR_UNSUPPORTED;

  spec_verify_s* h = new (std::nothrow) spec_verify_s();
  if (h == nullptr) return SV_ERR_HIP;
  h->cfg = c;
  h->chunk = chunk;
  h->nchunk = nchunk;
  if (hipDeviceGetAttribute(&h->lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                            c.device) != hipSuccess) {
    h->lds_per_cu = 0;
    (void)hipGetLastError();  // not reported by a later launch
  }
  const size_t rows = (size_t)c.max_batch * (2 * (size_t)c.max_drafts + 1);
  bool ok = hipMalloc(&h->part, rows * nchunk * sizeof(sv::Partial)) == hipSuccess &&
            hipMalloc(&h->desc, (size_t)c.max_batch * (c.max_drafts > 1 ? c.max_drafts : 1) *
                                    sizeof(sv::DrawDesc)) == hipSuccess &&
            hipMalloc(&h->rsum, (size_t)c.max_batch * nchunk * sv::kResidSplitMax * sizeof(double)) == hipSuccess &&
            hipMalloc(&h->flags, sizeof(uint32_t)) == hipSuccess &&
            hipMemset(h->flags, 0, sizeof(uint32_t)) == hipSuccess;
  if (ok) {
    size_t members = 0, teams = 0;  // the most over both team sizes
    for (int d = 0; d < 2; ++d)
      for (int k = 0; k < 2; ++k) {
        const int g = k == 0 ? 4 : 8;
        const int cap = sv::tree_team_capacity(c.device, c.target_dtype, c.draft_dtype, d != 0, g);
        h->tree_cap[d][k] = cap;
        if ((size_t)cap * g > members) members = (size_t)cap * g;
        if ((size_t)cap > teams) teams = (size_t)cap;
      }
    if (teams > 0) {
      const size_t bytes = members * sv::tree_team_words() * sizeof(uint64_t);
      ok = hipMalloc(&h->tree_xdat, bytes) == hipSuccess &&
           hipMalloc(&h->tree_xdone, teams * sizeof(uint32_t)) == hipSuccess &&
           hipMalloc(&h->tree_next, 2 * sizeof(uint32_t)) == hipSuccess &&
           hipMemset(h->tree_xdat, 0, bytes) == hipSuccess &&
           hipMemset(h->tree_xdone, 0, teams * sizeof(uint32_t)) == hipSuccess &&
           hipMemset(h->tree_next, 0, 2 * sizeof(uint32_t)) == hipSuccess;
    }
  }
  // the zeroed words are in place before any stream can launch on them (a
  // stream created non-blocking does not wait for the null stream's work)
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    free_all(h);
    delete h;
    return SV_ERR_HIP;
  }
  *out = h;
  return SV_OK;
}

int spec_verify_run(spec_verify_t h, int32_t B, int32_t K, const void* target_logits,
                    const void* draft_probs, const uint8_t* draft_mode,
                    const int32_t* draft_ids, const int32_t* num_drafts_per_req,
                    const float* temperatures, uint64_t philox_seed,
                    uint64_t philox_offset, int32_t* out_tokens,
                    int32_t* out_num_accepted, float* out_debug_probs, void* stream) {
  if (h == nullptr) return SV_ERR_INVALID_ARG;
  const sv_config& c = h->cfg;
  const int rc = check_run_args(c, B, K, target_logits, draft_probs, draft_ids,
                                num_drafts_per_req, temperatures, out_tokens,
                                out_num_accepted, out_debug_probs);
  if (rc != SV_OK || B == 0) return rc;
  sv::RunParams full = verify_params(c, h->chunk, h->nchunk, B, K, target_logits, draft_probs,
                                     draft_mode, draft_ids, num_drafts_per_req, temperatures,
                                     philox_seed, philox_offset, out_tokens, out_num_accepted,
                                     out_debug_probs);
  full.part = h->part;
  full.desc = h->desc;
  full.rsum = h->rsum;
  full.flags = h->flags;
  full.b_base = h->b_base;

  return enqueue(h, full, c.target_dtype, c.draft_dtype, stream);
}

int spec_verify_run_typical(spec_verify_t h, int32_t B, int32_t K, const void* target_logits,
                            const int32_t* draft_ids, const int32_t* num_drafts_per_req,
                            const float* temperatures, float threshold, int32_t top_k,
                            uint64_t philox_seed, uint64_t philox_offset, int32_t* out_tokens,
                            int32_t* out_num_accepted, float* out_debug_probs, void* stream) {
  if (h == nullptr || B < 0 || K < 0 || !(threshold >= 0.f && threshold <= FLT_MAX) ||
      top_k < 0)
    return SV_ERR_INVALID_ARG;
  if (B > h->cfg.max_batch || K > h->cfg.max_drafts) return SV_ERR_CAPACITY;
  if (B == 0) return SV_OK;
  const sv_config& c = h->cfg;
  if (target_logits == nullptr || num_drafts_per_req == nullptr || temperatures == nullptr ||
      out_tokens == nullptr || out_num_accepted == nullptr || (K > 0 && draft_ids == nullptr))
    return SV_ERR_INVALID_ARG;
  if (!aligned(target_logits, elt_bytes(c.target_dtype)) ||
      (draft_ids != nullptr && !aligned(draft_ids, 4)) || !aligned(num_drafts_per_req, 4) ||
      !aligned(temperatures, 4) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
      (out_debug_probs != nullptr && !aligned(out_debug_probs, 4)))
    return SV_ERR_INVALID_ARG;

  sv::RunParams full{};
  full.target = target_logits;
  full.ids = draft_ids;
  full.nd = num_drafts_per_req;
  full.temps = temperatures;
  full.out_tokens = out_tokens;
  full.out_nacc = out_num_accepted;
  full.out_dbg = out_debug_probs;
  full.part = h->part;
  full.desc = h->desc;
  full.rsum = h->rsum;
  full.flags = h->flags;
  full.seed = philox_seed;
  full.offset = philox_offset;
  full.B = B;
  full.K = K;
  full.V = c.vocab;
  full.chunk = h->chunk;
  full.nchunk = h->nchunk;
  full.typical = 1;
  full.eps = threshold;
  full.top_k = top_k;
  full.b_base = h->b_base;
  return enqueue(h, full, c.target_dtype, c.draft_dtype, stream);
}

int spec_verify_run_tree(spec_verify_t h, int32_t B, int32_t N, const void* target_logits,
                         const void* draft_logits, const int32_t* tokens,
                         const int32_t* parents, const int32_t* num_nodes,
                         const float* temperatures, uint64_t philox_seed,
                         uint64_t philox_offset, int32_t* out_tokens,
                         int32_t* out_num_accepted, int32_t* out_last_node, void* stream) {
  if (h == nullptr || B < 0 || N < 1 || N > SPEC_TREE_MAX_NODES) return SV_ERR_INVALID_ARG;
  if (B > h->cfg.max_batch) return SV_ERR_CAPACITY;
  if (B == 0) return SV_OK;
  const sv_config& c = h->cfg;
  if (target_logits == nullptr || tokens == nullptr || parents == nullptr ||
      num_nodes == nullptr || temperatures == nullptr || out_tokens == nullptr ||
      out_num_accepted == nullptr || out_last_node == nullptr)
    return SV_ERR_INVALID_ARG;
  if (!aligned(target_logits, elt_bytes(c.target_dtype)) ||
      (draft_logits != nullptr && !aligned(draft_logits, elt_bytes(c.draft_dtype))) ||
      !aligned(tokens, 4) || !aligned(parents, 4) || !aligned(num_nodes, 4) ||
      !aligned(temperatures, 4) || !aligned(out_tokens, 4) || !aligned(out_num_accepted, 4) ||
      !aligned(out_last_node, 4))
    return SV_ERR_INVALID_ARG;
  sv::TreeParams tp{};
  tp.target = target_logits;
  tp.draft = draft_logits;
  tp.tokens = tokens;
  tp.parents = parents;
  tp.nn = num_nodes;
  tp.temps = temperatures;
  tp.out_tokens = out_tokens;
  tp.out_nacc = out_num_accepted;
  tp.out_last = out_last_node;
  tp.flags = h->flags;
  tp.seed = philox_seed;
  tp.offset = philox_offset;
  tp.B = B;
  tp.N = N;
  tp.V = c.vocab;
  tp.draft_is_probs = c.draft_is_probs;
  tp.b_base = h->b_base;
  tp.xdat = h->tree_xdat;
  tp.xdone = h->tree_xdone;
  tp.next_req = h->tree_next;
  tp.spin_ticks = h->tree_wait_ticks;
  DeviceGuard g(c.device);
  if (!g.ok) return SV_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int* cap = h->tree_cap[draft_logits != nullptr];
  const int team = h->tree_force ? h->tree_force : sv::tree_team_pick(B, cap);
  const int teams = sv::tree_team_count(B, team, cap);
  if (sv::launch_tree(tp, c.target_dtype, c.draft_dtype, team, teams, s) != hipSuccess)
    return SV_ERR_HIP;
  h->last_stream = s;
  h->has_run = true;
  return SV_OK;
}

int spec_verify_set_request_base(spec_verify_t h, int32_t base) {
  if (h == nullptr || base < 0) return SV_ERR_INVALID_ARG;
  h->b_base = base;
  return SV_OK;
}

int spec_draft_sample(spec_verify_t h, int32_t B, int32_t K, const void* draft_logits,
                      const int32_t* num_drafts_per_req, const float* temperatures,
                      uint64_t philox_seed, uint64_t philox_offset, int32_t* out_ids,
                      float* out_q, void* stream) {
  if (h == nullptr || B < 0 || K < 0) return SV_ERR_INVALID_ARG;
  if (B > h->cfg.max_batch || K > h->cfg.max_drafts) return SV_ERR_CAPACITY;
  const sv_config& c = h->cfg;
  if (c.draft_is_probs) return SV_ERR_UNSUPPORTED;  // needs draft logits
  if (B == 0 || K == 0) return SV_OK;
  if (draft_logits == nullptr || temperatures == nullptr || out_ids == nullptr)
    return SV_ERR_INVALID_ARG;
  if (!aligned(draft_logits, elt_bytes(c.draft_dtype)) ||
      (num_drafts_per_req != nullptr && !aligned(num_drafts_per_req, 4)) ||
      !aligned(temperatures, 4) || !aligned(out_ids, 4) ||
      (out_q != nullptr && !aligned(out_q, 4)))
    return SV_ERR_INVALID_ARG;

  sv::RunParams full{};
  full.target = draft_logits;  // row (b, j) is "request" b * K + j, slot 0
  full.nd = num_drafts_per_req;
  full.temps = temperatures;
  full.out_tokens = out_ids;
  full.out_q = out_q;
  full.part = h->part;
  full.desc = h->desc;
  full.rsum = h->rsum;
  full.flags = h->flags;
  full.seed = philox_seed;
  full.offset = philox_offset;
  full.B = B * K;
  full.K = 0;
  full.V = c.vocab;
  full.chunk = h->chunk;
  full.nchunk = h->nchunk;
  full.sample_k = K;
  full.b_base = h->b_base;
  return enqueue(h, full, c.draft_dtype, c.draft_dtype, stream);
}

int spec_verify_get_device_errors(spec_verify_t h, uint32_t* host_flags, int32_t clear) {
  if (h == nullptr || host_flags == nullptr) return SV_ERR_INVALID_ARG;
  DeviceGuard g(h->cfg.device);
  if (!g.ok) return SV_ERR_HIP;
  if (h->has_run && hipStreamSynchronize(h->last_stream) != hipSuccess) return SV_ERR_HIP;
  if (hipMemcpy(host_flags, h->flags, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return SV_ERR_HIP;
  if (clear && hipMemset(h->flags, 0, sizeof(uint32_t)) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int spec_verify_timing_enable(spec_verify_t h, int32_t enable) {
  if (h == nullptr) return SV_ERR_INVALID_ARG;
  DeviceGuard g(h->cfg.device);
  if (!g.ok) return SV_ERR_HIP;
  if (enable && h->ev[0][0] == nullptr) {
    for (int s = 0; s < kTimingSlots; ++s)
      for (int k = 0; k < kEventsPerRun; ++k)
        if (hipEventCreate(&h->ev[s][k]) != hipSuccess) return SV_ERR_HIP;
  }
  while (h->ev_pending > 0)
    if (drain_one(h) != hipSuccess) return SV_ERR_HIP;
  for (int k = 0; k < sv::kNumKernels; ++k) h->tot_ms[k] = 0.0;
  h->runs = 0;
  h->timing = enable != 0;
  return SV_OK;
}

int spec_verify_timing_read(spec_verify_t h, float* total_ms, int32_t n, int32_t* runs) {
  if (h == nullptr || (n > 0 && total_ms == nullptr)) return SV_ERR_INVALID_ARG;
  DeviceGuard g(h->cfg.device);
  if (!g.ok) return SV_ERR_HIP;
  while (h->ev_pending > 0)
    if (drain_one(h) != hipSuccess) return SV_ERR_HIP;
  for (int k = 0; k < n && k < sv::kNumKernels; ++k) total_ms[k] = (float)h->tot_ms[k];
  if (runs) *runs = h->runs;
  return SV_OK;
}

int32_t spec_verify_chunk_elems(spec_verify_t h) { return h ? h->chunk : 0; }

int spec_verify_set_tree_wait_us(spec_verify_t h, int32_t microseconds) {
  if (h == nullptr || microseconds < 0) return SV_ERR_INVALID_ARG;
  h->tree_wait_ticks = (uint64_t)microseconds * 100u;
  return SV_OK;
}

int spec_verify_set_tree_team_size(spec_verify_t h, int32_t members) {
  if (h == nullptr || (members != 0 && members != 1 && members != 4 && members != 8))
    return SV_ERR_INVALID_ARG;
  if (members == 4 || members == 8) {  // a group of eight teams must fit, with or without drafts
    const int k = members == 8 ? 1 : 0;
    if (h->tree_cap[0][k] < 8 || h->tree_cap[1][k] < 8) return SV_ERR_UNSUPPORTED;
  }
  h->tree_force = members;
  return SV_OK;
}

int32_t spec_verify_tree_team_size(spec_verify_t h, int32_t B, int32_t has_draft) {
  if (h == nullptr || B < 1) return 0;
  return h->tree_force ? h->tree_force : sv::tree_team_pick(B, h->tree_cap[has_draft != 0]);
}

int spec_verify_destroy(spec_verify_t h) {
  if (h == nullptr) return SV_OK;
  int rc = SV_OK;
  {
    DeviceGuard g(h->cfg.device);
    if (!g.ok || hipDeviceSynchronize() != hipSuccess) rc = SV_ERR_HIP;
    free_all(h);
  }
  delete h;
  return rc;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// spec_verify_run_noalloc: the verify step with its workspace in a fixed
// device array instead of a handle's allocation.
// ---------------------------------------------------------------------------
namespace {

// Bytes of the array: the chunk partials, draw descriptors, residual sums and
// a flag word of one step.  Each GPU that runs the entry point holds its own
// copy until the process ends.
constexpr size_t kScratchBytes = SPEC_VERIFY_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Per device: the array's device address (from hipGetSymbolAddress; the
// name `scratch` in host code is only a host-side stand-in) and the bytes of
// LDS per compute unit.  Filled once, on the device's first call.
struct ScratchDev {
  void* ptr = nullptr;
  int lds_per_cu = 0;
};
ScratchDev g_scratch[kScratchDevices];
std::mutex g_scratch_mu;

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Layout of one step in the array: flag word, partials, descriptors,
// residual sums (each region 256-byte aligned).
struct ScratchLayout {
  size_t part, desc, rsum, total;
};

ScratchLayout scratch_layout(int32_t B, int32_t K, int nchunk) {
  ScratchLayout l;
  l.part = 256;
  l.desc = l.part + align256((size_t)B * (2 * (size_t)K + 1) * nchunk * sizeof(sv::Partial));
  l.rsum = l.desc + align256((size_t)B * sizeof(sv::DrawDesc));
  l.total = l.rsum + align256((size_t)B * nchunk * sv::kResidSplitMax * sizeof(double));
  return l;
}

// The array's address on `device` (the current device), looked up on its
// first use.  nullptr if the lookup fails.
const ScratchDev* scratch_on(int device) {
  if (device < 0 || device >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchDev& d = g_scratch[device];
  if (d.ptr == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              device) != hipSuccess) {
      lds = 0;
      (void)hipGetLastError();
    }
    d.lds_per_cu = lds;
    d.ptr = ptr;
  }
  return &d;
}

}  // namespace

extern "C" {

int spec_verify_run_noalloc(const sv_config* cfg, int32_t B, int32_t K,
                            const void* target_logits, const void* draft_probs,
                            const uint8_t* draft_mode, const int32_t* draft_ids,
                            const int32_t* num_drafts_per_req, const float* temperatures,
                            uint64_t philox_seed, uint64_t philox_offset, int32_t* out_tokens,
                            int32_t* out_num_accepted, float* out_debug_probs,
                            uint32_t* out_device_flags, void* stream) {
  if (cfg == nullptr) return SV_ERR_INVALID_ARG;
  const sv_config c = *cfg;
  int rc = check_config(c);
  if (rc != SV_OK) return rc;
  rc = check_run_args(c, B, K, target_logits, draft_probs, draft_ids, num_drafts_per_req,
                      temperatures, out_tokens, out_num_accepted, out_debug_probs);
  if (rc != SV_OK || B == 0) return rc;
  if (out_device_flags != nullptr && !aligned(out_device_flags, 4)) return SV_ERR_INVALID_ARG;
  const int chunk = pick_chunk(c);
  const int nchunk = (c.vocab + chunk - 1) / chunk;
  if (nchunk > sv::kMaxChunks) return SV_ERR_UNSUPPORTED;
  const ScratchLayout lay = scratch_layout(B, K, nchunk);
  if (lay.total > kScratchBytes) return SV_ERR_CAPACITY;

  DeviceGuard g(c.device);
  if (!g.ok) return SV_ERR_HIP;
  const ScratchDev* sd = scratch_on(c.device);
  if (sd == nullptr) return SV_ERR_HIP;
  unsigned char* base = static_cast<unsigned char*>(sd->ptr);
  sv::RunParams p = verify_params(c, chunk, nchunk, B, K, target_logits, draft_probs,
                                  draft_mode, draft_ids, num_drafts_per_req, temperatures,
                                  philox_seed, philox_offset, out_tokens, out_num_accepted,
                                  out_debug_probs);
  p.part = reinterpret_cast<sv::Partial*>(base + lay.part);
  p.desc = reinterpret_cast<sv::DrawDesc*>(base + lay.desc);
  p.rsum = reinterpret_cast<double*>(base + lay.rsum);
  p.flags = out_device_flags != nullptr ? out_device_flags : reinterpret_cast<uint32_t*>(base);
  p.clear_flags = 1;  // the step's first kernel zeroes the flag word
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int k = 0; k < sv::kNumKernels; ++k)
    if (sv::launch_kernel(k, p, c.target_dtype, c.draft_dtype, sd->lds_per_cu, s) != hipSuccess)
      return SV_ERR_HIP;
  return SV_OK;
}

}  // extern "C"
