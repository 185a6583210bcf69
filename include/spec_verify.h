/*
 * spec_verify.h -- C ABI of the speculative-sampling verify step (chains,
 * typical acceptance, token trees), and of the draft-token sampler and the
 * n-gram proposer that feed it, on MI355X (gfx950).
 *
 * The operation (sources by page title and section):
 *   - "深入推测解码：从概念到实现" (Exploring Speculative Decoding), section
 *     保证原始分布: a draft token x sampled from the draft law q is accepted
 *     with probability min(1, p(x)/q(x)); on rejection a correction token is
 *     sampled from max(0, p - q).
 *   - "RTP-LLM Speculative Engine 深度解析", section 拒绝采样算法: per drafted
 *     position a Uniform(0,1) draw is compared with p/q, the first rejection
 *     resamples from normalize(max(0, p - q)) and stops the walk; full
 *     probability rows per position are the inputs.
 *   - "投机采样" (razer666.cn), section 投机解码算法, steps 3-5: the accepted
 *     count n, the adjusted law norm(max(0, p_{n+1} - q_{n+1})), and one
 *     extra token from the last target row when every draft passes, so the
 *     output length is n + 1 in [1, K + 1]; section 验证阶段的策略 / 精确匹配:
 *     greedy exact match against the max-probability token.
 *
 * Conventions
 *   - p = softmax(target_logits / T_b); q = softmax(draft_logits / T_b), or
 *     the draft rows as given when the handle was created with
 *     draft_is_probs = 1.
 *   - T_b that is not a positive, normal, finite float selects greedy for
 *     request b: a draft is accepted iff its target logit equals the row
 *     maximum, and the emitted token is the lowest index of the maximum.
 *   - One-hot (n-gram) drafts have no q: x is accepted with probability p(x)
 *     and the correction is drawn from p with x removed.
 *   - Uniforms come from Philox4x64-10 (Salmon et al., SC'11) with key
 *     (philox_seed, 0) and counter (philox_offset, b, j, 0); output word 0
 *     is the acceptance uniform of position j, word 1 the draw uniform;
 *     u = (w >> 40) * 2^-24.  A decision accepts iff u < p(x)/q(x); a draw
 *     takes the smallest i whose running sum exceeds u * S.
 *
 * Ownership and execution
 *   - The caller owns every input and output buffer (device memory).  The
 *     library owns only the workspace it allocates in spec_verify_create.
 *   - spec_verify_run only enqueues kernels on `stream` (a hipStream_t;
 *     NULL = the null stream).  It neither allocates nor synchronizes.  One
 *     handle must not be used by two streams at once: its workspace is
 *     reused by every run.
 *   - Errors are returned as sv_status codes before anything is enqueued;
 *     nothing is thrown across the ABI.  Bad device-side data (draft ids
 *     outside [0, V), draft counts outside [0, K]) never faults: it is
 *     clamped or rejected and recorded in a sticky bitmask that
 *     spec_verify_get_device_errors returns.
 *   - The same inputs and (seed, offset) give bit-identical outputs.
 *   - The rows a step reads are expected to hold finite logits (-inf counts
 *     as probability 0) or, with draft_is_probs, probabilities.  NaN or +inf
 *     there gives unspecified tokens, but never a fault or an access outside
 *     the buffers.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_verify_s *spec_verify_t;

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = -1, /* null / misaligned pointer, bad size */
  SV_ERR_UNSUPPORTED = -2, /* dtype or option not supported */
  SV_ERR_CAPACITY = -3,    /* B or K above the handle's maxima */
  SV_ERR_HIP = -4          /* a HIP runtime call failed */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Sticky device-side conditions (spec_verify_get_device_errors). */
#define SV_DEVERR_BAD_DRAFT_ID 1u   /* id outside [0, V): never accepted */
#define SV_DEVERR_BAD_NUM_DRAFTS 2u /* count clamped into [0, K] */
#define SV_DEVERR_ZERO_RESIDUAL 4u  /* residual mass 0: drawn from p */
#define SV_DEVERR_DRAW_ROUNDING 8u  /* draw landed past a chunk's recomputed
                                       total (a rounding tie); nearest token
                                       with mass taken */
#define SV_DEVERR_BAD_TREE 16u      /* a tree node whose parent is not an
                                       earlier node: never visited */
#define SV_DEVERR_TREE_SYNC 32u     /* a team walk's exchange did not complete
                                       within its time bound (a member not yet
                                       running): the walk was finished by
                                       single workgroups, outputs valid */

typedef struct {
  int32_t max_batch;      /* largest B of any run, >= 1 */
  int32_t max_drafts;     /* largest K of any run, 0..31 */
  int32_t vocab;          /* V, 1 .. 983040 (64 chunks of at most 15360) */
  int32_t target_dtype;   /* sv_dtype of target_logits */
  int32_t draft_dtype;    /* sv_dtype of draft_probs */
  int32_t draft_is_probs; /* 0: draft rows are logits (softmax at T_b);
                             1: draft rows are normalized probabilities */
  int32_t device;         /* HIP device ordinal */
  int32_t chunk_elems;    /* vocabulary elements per work chunk; 0 picks a
                             default; else a multiple of 64 in [256, 15360]
                             (raised to ceil(V / 64) if smaller) */
} sv_config;

/* Creates a handle on cfg->device and allocates its workspace (zeroing its
 * counters, then waiting for the device, so any stream may use the handle
 * once this returns).  A setup call: it allocates and synchronizes.
 * Returns SV_ERR_INVALID_ARG for a null argument or a field out of range,
 * SV_ERR_UNSUPPORTED for an unknown dtype, SV_ERR_HIP if allocation fails.
 * On failure *out is set to NULL. */
int spec_verify_create(const sv_config *cfg, spec_verify_t *out);

/* Enqueues one verify step for B requests with up to K drafts each.
 *
 *   target_logits      device [B][K+1][V], cfg.target_dtype, row-major,
 *                      aligned to its element size.  Rows j > n_b are never
 *                      read.
 *   draft_probs        device [B][K][V], cfg.draft_dtype: draft logits, or
 *                      probabilities if cfg.draft_is_probs.  Rows j >= n_b,
 *                      rows of one-hot requests and rows of greedy requests
 *                      are never read.  NULL: every request is one-hot.
 *   draft_mode         device [B] uint8: 0 probabilistic, nonzero one-hot.
 *                      NULL: every request is probabilistic (if draft_probs
 *                      is given).  The kernels read each byte through the
 *                      aligned 4-byte word that holds it, so the bytes of
 *                      those words next to the array must be readable memory
 *                      (as in any device allocation; their values are not
 *                      used).
 *   draft_ids          device [B][K] int32: the drafted tokens x_j.
 *   num_drafts_per_req device [B] int32: n_b, expected in [0, K].
 *   temperatures       device [B] float: T_b (see Conventions).
 *   philox_seed, philox_offset: the uniform stream; advance the offset by
 *                      one per step.
 *   out_tokens         device [B][K+1] int32: x_0..x_{n_acc-1}, then the
 *                      emitted token, then -1.
 *   out_num_accepted   device [B] int32: n_acc in [0, n_b].
 *   out_debug_probs    device [B][K][2] float (p_j(x_j), q_j(x_j)) for every
 *                      j < n_b of a sampling request (q = 1 for one-hot),
 *                      NaN elsewhere; or NULL.
 *   stream             hipStream_t to enqueue on.
 *
 * Returns SV_ERR_INVALID_ARG (null or misaligned pointer, B < 0, K < 0),
 * SV_ERR_CAPACITY (B > max_batch or K > max_drafts) or SV_ERR_HIP (launch
 * failure).  B == 0 enqueues nothing and returns SV_OK. */
int spec_verify_run(spec_verify_t h, int32_t B, int32_t K,
                    const void *target_logits, const void *draft_probs,
                    const uint8_t *draft_mode, const int32_t *draft_ids,
                    const int32_t *num_drafts_per_req,
                    const float *temperatures, uint64_t philox_seed,
                    uint64_t philox_offset, int32_t *out_tokens,
                    int32_t *out_num_accepted, float *out_debug_probs,
                    void *stream);

/* Bytes of the fixed device array spec_verify_run_noalloc works in (one per
 * GPU). */
#define SPEC_VERIFY_NOALLOC_SCRATCH_BYTES (8u << 20)

/* spec_verify_run for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * There is no handle and nothing is allocated.  The step's workspace lives
 * in one fixed array of SPEC_VERIFY_NOALLOC_SCRATCH_BYTES of device memory
 * per GPU, the library's own, held until the process ends: chunk partials,
 * draw descriptors, residual sums and a flag word.  The kernels and the
 * outputs are those of spec_verify_run with the same configuration (request
 * base 0).
 *
 *   cfg              as for spec_verify_create (checked the same way); B <=
 *                    cfg->max_batch and K <= cfg->max_drafts.
 *   other arguments  as for spec_verify_run.
 *   out_device_flags device uint32 receiving the step's SV_DEVERR_* bits
 *                    (zeroed by the step itself, so not sticky across
 *                    calls), or NULL to leave them in the array.
 *
 * Limit: with nchunk = ceil(V / chunk) (the chunk spec_verify_chunk_elems
 * reports for a handle of the same cfg), the step needs 256 +
 * a(B (2K+1) nchunk 16) + a(B 64) + a(B nchunk 32) bytes, a() rounding up to
 * 256; above the array's size the call returns SV_ERR_CAPACITY and enqueues
 * nothing.  V = 152064 (10 chunks) with B = 256, K = 7 needs 0.7 MB.
 *
 * Every call on one GPU shares that GPU's array, and a call leaves it
 * holding its own step.  Calls ordered on one stream are safe; calls that
 * overlap on one GPU (two streams, two host threads) race and give wrong
 * outputs.  The first call on a device looks up the array's address
 * (hipGetSymbolAddress); later calls only enqueue.  Returns the status codes
 * of spec_verify_run, SV_ERR_CAPACITY as above, SV_ERR_HIP if the array's
 * address cannot be found. */
int spec_verify_run_noalloc(const sv_config *cfg, int32_t B, int32_t K,
                            const void *target_logits, const void *draft_probs,
                            const uint8_t *draft_mode, const int32_t *draft_ids,
                            const int32_t *num_drafts_per_req,
                            const float *temperatures, uint64_t philox_seed,
                            uint64_t philox_offset, int32_t *out_tokens,
                            int32_t *out_num_accepted, float *out_debug_probs,
                            uint32_t *out_device_flags, void *stream);

/* Enqueues a verify step with typical acceptance instead of rejection
 * sampling.  Source: "投机采样" (razer666.cn), section 验收标准, Typical
 * Acceptance: a draft token is accepted when its probability exceeds a hard
 * threshold, the threshold may be relaxed through a top-k constraint, and
 * the longest accepted run is kept.  The rule is lossy: outputs no longer
 * follow p exactly.
 *
 * Readings: x_j is accepted iff p_j(x_j) > threshold or x_j ranks among the
 * top_k tokens of target row j, i.e. #{i : l_i > l_x} < top_k (top_k = 0:
 * the threshold alone); the walk stops at the first rejection; the token at
 * that position, or the bonus token after n_b acceptances, is drawn from
 * p itself with the draw uniform of spec_verify_run (word 1 of the block at
 * counter (philox_offset, b, j, 0)); greedy requests keep exact matching.
 * There are no draft rows: only ids.
 *
 * Arguments as spec_verify_run without draft_probs and draft_mode;
 * threshold >= 0 and finite, top_k >= 0.  out_debug_probs holds
 * (p_j(x_j), 1).  Returns SV_ERR_INVALID_ARG (bad threshold or top_k, null
 * or misaligned pointer, B < 0, K < 0), SV_ERR_CAPACITY or SV_ERR_HIP. */
int spec_verify_run_typical(spec_verify_t h, int32_t B, int32_t K,
                            const void *target_logits,
                            const int32_t *draft_ids,
                            const int32_t *num_drafts_per_req,
                            const float *temperatures, float threshold,
                            int32_t top_k, uint64_t philox_seed,
                            uint64_t philox_offset, int32_t *out_tokens,
                            int32_t *out_num_accepted, float *out_debug_probs,
                            void *stream);

/* Enqueues the draft-token sampler: the step that produces the drafts the
 * verify step checks.  Sources: "深入推测解码：从概念到实现" (Exploring
 * Speculative Decoding), section 引言, the propose pseudo-code (each draft
 * step samples one token from the draft model's logits); "投机采样"
 * (razer666.cn), section 投机解码算法, 第一步 - 采样 (guess x_i is sampled
 * from the draft model's distribution q_i).
 *
 * For every request b and draft position j < n_b, x_j is drawn from
 * q_j = softmax(draft_logits[b][j] / T_b) by the same inverse CDF as the
 * verify step's draws, with the uniform u = word 0 of the Philox block at
 * counter (philox_offset, b, j, 1), key (philox_seed, 0).  Counter word 3 is
 * 1 here and 0 in spec_verify_run, so the two never share a uniform.  A
 * greedy T_b (see Conventions) takes the lowest index of the row maximum.
 * Rows are independent: a caller drafting autoregressively calls this once
 * per position with K = 1 (and that position's index folded into
 * philox_offset or the row layout).
 *
 *   draft_logits       device [B][K][V], cfg.draft_dtype, row-major, aligned
 *                      to its element size.  Rows j >= n_b are never read.
 *   num_drafts_per_req device [B] int32: n_b, expected in [0, K]; counts
 *                      outside are clamped and flagged.  NULL: n_b = K.
 *   temperatures       device [B] float: T_b.
 *   out_ids            device [B][K] int32: x_j, or -1 for j >= n_b.
 *   out_q              device [B][K] float: q_j(x_j) (1 for greedy rows,
 *                      NaN for j >= n_b), or NULL.
 *
 * Shares the handle's workspace with spec_verify_run (same stream rules).
 * Returns SV_ERR_UNSUPPORTED if the handle was created with
 * draft_is_probs = 1 (the sampler needs logits), SV_ERR_INVALID_ARG (null
 * or misaligned pointer, B < 0, K < 0), SV_ERR_CAPACITY (B > max_batch or
 * K > max_drafts) or SV_ERR_HIP.  B == 0 or K == 0 enqueues nothing. */
int spec_draft_sample(spec_verify_t h, int32_t B, int32_t K,
                      const void *draft_logits,
                      const int32_t *num_drafts_per_req,
                      const float *temperatures, uint64_t philox_seed,
                      uint64_t philox_offset, int32_t *out_ids, float *out_q,
                      void *stream);

/* Most nodes (root included) of one request's tree in spec_verify_run_tree. */
#define SPEC_TREE_MAX_NODES 256

/* Enqueues token-tree verification.  Source: "投机采样" (razer666.cn),
 * section 验证阶段的策略 / 验证方案: draft sequences with shared prefixes
 * form a token tree (a trie) that the target scores in one pass (tree
 * attention, each node seeing only its ancestors); SpecInfer and Spectr are
 * named for the multi-branch rule, which the page does not give.
 *
 * Reading: the chain rule of spec_verify_run applied child by child, which
 * keeps the target law (multi-step speculative sampling).  At node v (the
 * walk starts at the root, node 0) the children (nodes whose parent is v, in
 * index order) are tested in turn; after k rejections at v the law is
 *   probabilistic tree: p'_k = max(0, p - c_k q) / Z_k, c_0 = 0, Z_0 = 1,
 *     c_{k+1} = c_k + Z_k, Z_k = sum_i max(0, p_i - c_k q_i); child x is
 *     accepted iff u < p'_k(x) / q(x);
 *   one-hot tree (draft_logits NULL): p'_k = p without the rejected
 *     siblings' tokens, renormalized; accepted iff u < p'_k(x);
 *   greedy T_b: the first child whose token attains the row maximum.
 * An accepted child becomes v; when every child of v is rejected, or v is a
 * leaf, one token is drawn at v from p'_k (p at a leaf, the lowest argmax
 * for greedy requests).  p at node i = softmax(target_logits[b][i] / T_b);
 * q = softmax(draft_logits[b][i] / T_b) (or draft rows as given with
 * draft_is_probs), the law node i's children were drawn from.  Uniforms: the
 * Philox block at counter (philox_offset, b, i, 0) gives in word 0 the
 * acceptance uniform of node i + 1 and in word 1 the draw uniform at node i,
 * so a chain-shaped tree (parent of i = i - 1) reproduces spec_verify_run.
 *
 *   target_logits  device [B][N][V], cfg.target_dtype: the target's logits
 *                  after each node (node 0: after the last committed token).
 *   draft_logits   device [B][N][V], cfg.draft_dtype, or NULL (one-hot).
 *   tokens         device [B][N] int32: the draft token of each node
 *                  (node 0 unused); ids outside [0, V) are never accepted.
 *   parents        device [B][N] int32: the parent of node i >= 1, an
 *                  earlier node; other nodes are never visited (flagged).
 *   num_nodes      device [B] int32: nodes in use, clamped into [1, N].
 *   temperatures   device [B] float.
 *   out_tokens     device [B][N] int32: the accepted path's tokens, the
 *                  emitted token, then -1.
 *   out_num_accepted device [B] int32; out_last_node device [B] int32: the
 *                  deepest accepted node (0 = root).
 *
 * A team of workgroups walks each request's tree and reads only the rows of
 * the nodes it visits: eight (or four) workgroups on different compute units
 * of one XCD each take a share of every row and exchange their partial
 * statistics through device memory.  Eight while the teams of eight that fit
 * the device at once walk at most two requests each; beyond that, teams of
 * four that walk several requests each.  A team that walks several takes the
 * next free request whenever its walk ends
 * (spec_verify_tree_team_size, spec_verify_set_tree_team_size).  Calls on one
 * handle share its exchange buffers and request counter and must not
 * overlap.  Returns SV_ERR_INVALID_ARG (null or misaligned pointer,
 * B < 0, N outside [1, SPEC_TREE_MAX_NODES]), SV_ERR_CAPACITY (B >
 * max_batch) or SV_ERR_HIP. */
int spec_verify_run_tree(spec_verify_t h, int32_t B, int32_t N,
                         const void *target_logits, const void *draft_logits,
                         const int32_t *tokens, const int32_t *parents,
                         const int32_t *num_nodes, const float *temperatures,
                         uint64_t philox_seed, uint64_t philox_offset,
                         int32_t *out_tokens, int32_t *out_num_accepted,
                         int32_t *out_last_node, void *stream);

/* Longest n-gram spec_ngram_propose matches. */
#define SPEC_NGRAM_MAX_N 32

/* Enqueues the n-gram prompt-lookup proposer.  Source: "深入推测解码：从概念
 * 到实现" (Exploring Speculative Decoding), section n-gram: the last n tokens
 * of a request's context are found earlier in the context, and the k tokens
 * that followed that occurrence are proposed; n is the longest match in
 * [min_n, max_n] (prompt_lookup_min / max), and proposals stop at
 * max_model_len.
 *
 * Readings where the page is silent: the earlier occurrence must end before
 * the last token (it may overlap the suffix); among occurrences of the
 * longest matching n-gram the most recent is used; the count is
 * min(k, tokens after the occurrence, max_model_len - N); no match of length
 * >= min_n gives no drafts.  The output feeds spec_verify_run as one-hot
 * drafts (draft_mode 1, draft_ids = out_drafts, num_drafts = out_num).
 *
 *   context        device [B][stride] int32 token ids, row-major.
 *   context_lens   device [B] int32: N_b, the tokens of row b in use;
 *                  clamped into [0, stride].
 *   min_n, max_n   1 <= min_n <= max_n <= SPEC_NGRAM_MAX_N.
 *   k              drafts per request, >= 0.
 *   max_model_len  >= 0; a request with N_b >= max_model_len gets none.
 *   out_drafts     device [B][k] int32: the proposed tokens, then -1 (may
 *                  be NULL when k == 0).
 *   out_num_drafts device [B] int32: the count.
 *
 * Needs no handle; runs on the device of `stream` (a hipStream_t).  Only
 * enqueues.  Returns SV_ERR_INVALID_ARG for a bad size or a null or
 * misaligned pointer, SV_ERR_HIP on a launch failure.  B == 0 enqueues
 * nothing. */
int spec_ngram_propose(int32_t B, const int32_t *context, int32_t stride,
                       const int32_t *context_lens, int32_t min_n,
                       int32_t max_n, int32_t k, int32_t max_model_len,
                       int32_t *out_drafts, int32_t *out_num_drafts,
                       void *stream);

/* Global index of the handle's request 0, for a batch split into shards
 * (across GPUs, or across calls).  Every later run on the handle draws its
 * Philox counters for request b at request index base + b, in place of b:
 * in spec_verify_run, spec_verify_run_typical, spec_verify_run_tree, and
 * in spec_draft_sample, where b is the request (row / K).  A shard
 * [base, base + B_s) of a batch, run with that base and the batch's seed and
 * offset, therefore gives exactly the rows the whole batch gives in one
 * call.  Default 0.  Host-only; takes effect for runs enqueued after it.
 * Returns SV_ERR_INVALID_ARG for a null handle or base < 0. */
int spec_verify_set_request_base(spec_verify_t h, int32_t base);

/* Waits for the handle's last run, copies the sticky SV_DEVERR_* bitmask to
 * *host_flags and, if clear != 0, resets it.  Synchronizing call. */
int spec_verify_get_device_errors(spec_verify_t h, uint32_t *host_flags,
                                  int32_t clear);

/* Per-kernel timing with HIP events recorded on the run's stream.
 * enable != 0 starts recording (and resets the totals); each later run adds
 * the duration of each of its kernels.  spec_verify_timing_read waits for
 * the last run and writes up to n totals in milliseconds (kernel order as
 * spec_verify_kernel_name) and the number of timed runs.  A kernel a run
 * does not launch (the decision kernel of the draft sampler, the residual
 * kernel of runs without draft rows) adds nothing to its total. */
int spec_verify_timing_enable(spec_verify_t h, int32_t enable);
int spec_verify_timing_read(spec_verify_t h, float *total_ms, int32_t n,
                            int32_t *runs);
/* Name of kernel i of a run (NULL past the last one). */
const char *spec_verify_kernel_name(int32_t i);

/* Chunk length (vocabulary elements per work item) the handle uses. */
int32_t spec_verify_chunk_elems(spec_verify_t h);

/* Workgroups that walk each request's tree in spec_verify_run_tree for a
 * batch of B (has_draft != 0: with draft rows): 8 or 4 for a team walk, 1
 * for one 1024-thread workgroup per request; 0 for a null handle or B < 1.
 * Unless set by spec_verify_set_tree_team_size, the handle picks it by B
 * against the teams its device holds at once (measured crossovers, stated
 * where the pick is made): 8 while the teams of eight that fit walk at most
 * two requests each, else 4, whose teams then walk several requests each; 1
 * only if the device's team capacity is unknown.  Host-only. */
int32_t spec_verify_tree_team_size(spec_verify_t h, int32_t B, int32_t has_draft);

/* Sets the workgroups per request of later spec_verify_run_tree calls on the
 * handle: 0 restores the handle's pick, 1 is one 1024-thread workgroup per
 * request, 4 or 8 a team of that size (whose teams walk several requests
 * each when they outnumber the teams that fit).  Team sizes fold a row's
 * sums in different orders, so outputs can differ only where a draw or an
 * acceptance test falls within rounding of a boundary.  Host-only; for runs
 * enqueued after it.  Returns SV_ERR_INVALID_ARG for a
 * null handle or another value, SV_ERR_UNSUPPORTED if fewer than eight
 * teams of that size fit the device. */
int spec_verify_set_tree_team_size(spec_verify_t h, int32_t members);

/* Bound, in microseconds, on how long a team member of spec_verify_run_tree
 * waits for its partners at an exchange (default 20000).  A member that
 * reaches it sets SV_DEVERR_TREE_SYNC and finishes the walk alone, computing
 * every member's share itself in member order, so the outputs are the same
 * bit for bit; only the time differs.  0 makes members stop waiting at once
 * (the outputs still match).  Host-only; for runs enqueued after it.
 * Returns SV_ERR_INVALID_ARG for a null handle or a negative bound. */
int spec_verify_set_tree_wait_us(spec_verify_t h, int32_t microseconds);

/* Frees the workspace and the handle (waits for the device first).
 * NULL is accepted. */
int spec_verify_destroy(spec_verify_t h);

/* Static text for a status code. */
const char *spec_verify_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
