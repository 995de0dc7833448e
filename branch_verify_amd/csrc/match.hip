// State-equality walk over the draft tree (one wave).
//
// SpecFold, introduction: drafted states and their logits are cached, and a
// later main-branch state equal to a cached draft reuses that draft's logits
// instead of another target pass.  SPOT ("How does SPOT draft and verify?"):
// the target accepts the longest prefix consistent with its own trajectory;
// with shared noise that is state equality (Proposition 2).
//
// One wave of 64 lanes, one lane per branch (B1 <= 64): the lanes check each
// draft against its parent, hash every drafted state and every next state
// (64-bit FNV-1a over the tokens), then walk from the main branch.  Each hop
// ballots the drafts whose hash equals the current next state and confirms
// the lowest candidate by full comparison across the lanes.
#include "common.h"
#include "internal.h"

namespace sfv {
namespace {

__device__ __forceinline__ uint64_t fnv1a(const int32_t* s, int N) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (int n = 0; n < N; ++n) {
    const unsigned u = (unsigned)s[n];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      h ^= (u >> (8 * b)) & 0xFFu;
      h *= 0x100000001b3ull;
    }
  }
  return h;
}

__global__ __launch_bounds__(64) void match_kernel(const int32_t* state, const int32_t* next_state,
                                                   const int32_t* commit_pos, TreeArgs tree, int N,
                                                   int k_max, int S_max, int32_t* chain,
                                                   int32_t* n_accepted, int32_t* status) {
  const int lane = threadIdx.x;
  const int B1 = tree.B1;
  bool bad = false;
  if (S_max >= 0 && lane >= 1 && lane < B1) {
    const int p = tree.parent[lane];
    int fresh = 0;
    for (int n = 0; n < N; ++n) {
      const int sp = state[p * N + n], sc = state[lane * N + n];
      if (sp != -1) {
        bad = bad || (sc != sp);
      } else if (sc != -1) {
        ++fresh;
      }
    }
    bad = bad || (fresh > S_max);
  }
  if (__any(bad)) {
    if (lane < B1) chain[lane] = -1;
    if (lane == 0) {
      *n_accepted = 0;
      *status = -4;  // SFV_E_STATE
    }
    return;
  }
  const uint64_t hs = lane < B1 ? fnv1a(state + lane * N, N) : 0ull;
  const uint64_t hn = lane < B1 ? fnv1a(next_state + lane * N, N) : 0ull;
  int cur = 0, h = 0;
  while (h < B1 - 1) {
    if (commit_pos[cur * k_max] == -1) break;
    const uint64_t target = __shfl(hn, cur, kWave);
    unsigned long long cand = __ballot(lane >= 1 && lane < B1 && hs == target);
    int found = -1;
    while (cand) {
      const int j = __ffsll((long long)cand) - 1;
      cand &= cand - 1;
      bool diff = false;
      for (int n = lane; n < N; n += kWave) diff = diff || (state[j * N + n] != next_state[cur * N + n]);
      if (!__any(diff)) {
        found = j;
        break;
      }
    }
    if (found < 0) break;
    if (lane == 0) chain[h] = found;
    ++h;
    cur = found;
  }
  if (lane >= h && lane < B1) chain[lane] = -1;
  if (lane == 0) {
    *n_accepted = h;
    *status = 0;
  }
}

}  // namespace

hipError_t launch_match(const int32_t* state, const int32_t* next_state, const int32_t* commit_pos,
                        const TreeArgs& tree, int N, int k_max, int S_max, int32_t* chain,
                        int32_t* n_accepted, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(match_kernel, dim3(1), dim3(64), 0, stream, state, next_state, commit_pos, tree,
                     N, k_max, S_max, chain, n_accepted, status);
  return hipGetLastError();
}

}  // namespace sfv
