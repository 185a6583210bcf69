// Types and entry points of token-tree verification (sv_tree.hip), shared
// with the host API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// Token-tree verification of a batch (a team of workgroups per request).
struct TreeParams {
  const void* target;  // [B][N][V]
  const void* draft;   // [B][N][V] or nullptr (one-hot tree)
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* nn;
  const float* temps;
  int32_t* out_tokens;
  int32_t* out_nacc;
  int32_t* out_last;
  uint32_t* flags;
  uint64_t seed, offset;
  int B, N, V;
  int draft_is_probs;
  int b_base;  // global index of request 0 (Philox counters use b_base + b)
  // Team walks (several workgroups per request): the exchange words and the
  // per-team counters, all 0 between launches (zeroed once; every launch
  // returns them to 0).
  uint64_t* xdat;   // [teams][2][team size][8]
  uint32_t* xdone;  // [teams]
  uint64_t spin_ticks;  // bound of an exchange's wait (100 MHz ticks)
  uint32_t* next_req;   // [2]: requests handed out past the first round, and
                        // teams done (teams that walk several requests); 0
                        // between launches
};

// 64-bit exchange words per team member.
int tree_team_words();

// Teams of g members (4 or 8) that can be resident at once on `device` for
// these dtypes, or 0 if that cannot be known.
int tree_team_capacity(int device, int target_dtype, int draft_dtype, bool has_draft, int g);

// Teams a launch for a batch of B runs: B rounded up to whole groups of
// eight (one team per XCD in each group; the extra teams have no request).
inline int tree_team_slots(int B) { return (B + 7) / 8 * 8; }

// Members per request for a batch of B, given the capacities of teams of 4
// and 8 (cap[0], cap[1]): eight while the teams of eight that fit the device
// walk at most two requests each, else four (each team then walks several
// requests in turn); 1, one 1024-thread workgroup per request, only where no
// team capacity is known.
int tree_team_pick(int B, const int cap[2]);

// Teams a launch with g members per request runs for a batch of B: one per
// request in whole groups of eight, at most as many whole groups as fit
// (team t then walks request t first and takes the next free request from
// a launch-wide counter at the end of each walk); B for g = 1.
int tree_team_count(int B, int g, const int cap[2]);

// Enqueues the walk with g members per request and `teams` teams (from
// tree_team_pick and tree_team_count).
hipError_t launch_tree(const TreeParams& p, int target_dtype, int draft_dtype, int g, int teams,
                       hipStream_t stream);

}  // namespace sv
