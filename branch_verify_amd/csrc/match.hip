// State-equality walk over the draft tree.
//
// SpecFold, introduction: drafted states and their logits are cached, and a
// later main-branch state equal to a cached draft reuses that draft's logits
// instead of another target pass.  SPOT ("How does SPOT draft and verify?"):
// the target accepts the longest prefix consistent with its own trajectory;
// with shared noise that is state equality (Proposition 2).
//
// One workgroup of four waves.  Both state arrays and the first commit
// position of every branch are first copied into LDS by all threads (the
// state arrays into launch-sized dynamic LDS), so every
// later step (and each hop of the walk, whose reads depend on the previous
// hop) reads LDS rather than waiting on global memory.  Phase 1 spreads the
// (row, position) elements of the 2*B1 rows (every drafted state and every
// next state) over all threads: each row's 64-bit hash is the sum over
// positions of mix(n, token), order-free, so LDS atomic adds build it; every
// draft position is checked against its parent's.
// Phase 2 is the walk, in wave 0: each hop ballots the drafts one tree level
// below the current branch whose hash equals its next state and confirms the
// lowest candidate by a full comparison, so a hash collision can never
// produce a false match.  Only the next level counts: a draft at depth d
// commits with the noise of step step0 + d, so one at another depth holding
// the right state would continue the run with another step's noise and leave
// the draft-free trajectory (SPOT, "Is the output exact when the target
// samples?", Proposition 2).
#include "common.h"
#include "internal.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;

// SplitMix64 finalizer (Steele, Lea, Flood: "Fast splittable pseudorandom
// number generators", 2014) of the (position, token) pair.
__device__ __forceinline__ uint64_t mix(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

__global__ __launch_bounds__(kThreads) void match_kernel(const int32_t* state, const int32_t* next_state,
                                                         const int32_t* commit_pos, TreeArgs tree, int N,
                                                         int k_max, int S_max, int32_t* chain,
                                                         int32_t* n_accepted, int32_t* status) {
  __shared__ unsigned long long hs[kMaxBranches];  // hash of state[i]
  __shared__ unsigned long long hn[kMaxBranches];  // hash of next_state[i]
  __shared__ int fresh[kMaxBranches];              // positions a draft unmasks over its parent
  __shared__ int bad_s;
  __shared__ int lc[kMaxBranches];  // commit_pos[i][0]
  // state then next_state, [B1][N] each, sized at launch (2 * B1 * N ints)
  extern __shared__ int lstage[];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int B1 = tree.B1;
  const int total = B1 * N;
  int* ls = lstage;
  int* ln = lstage + total;
  for (int e = t; e < total; e += kThreads) {
    ls[e] = state[e];
    ln[e] = next_state[e];
  }
  if (t < B1) {
    lc[t] = commit_pos[t * k_max];
    hs[t] = 0ull;
    hn[t] = 0ull;
    fresh[t] = 0;
  }
  if (t == 0) bad_s = 0;
  __syncthreads();

  // Every (row, position) of the 2*B1 rows at once: the hashes are sums, so
  // their order does not matter and LDS atomic adds build them; each draft
  // position is also checked against its parent's.
  const int elems = 2 * B1 * N;
  for (int e = t; e < elems; e += kThreads) {
    const int row = e / N, n = e % N;
    const bool is_next = row >= B1;
    const int i = is_next ? row - B1 : row;
    const int v = (is_next ? ln : ls)[i * N + n];
    atomicAdd(&(is_next ? hn : hs)[i], (unsigned long long)mix(((uint64_t)(uint32_t)n << 32) | (uint32_t)v));
    if (!is_next && S_max >= 0 && i >= 1) {
      // a draft keeps every unmasked token of its parent and unmasks at most S_max more
      const int sp = ls[tree.parent[i] * N + n];
      if (sp != -1) {
        if (v != sp) bad_s = 1;
      } else if (v != -1) {
        atomicAdd(&fresh[i], 1);
      }
    }
  }
  __syncthreads();
  if (S_max >= 0 && t >= 1 && t < B1 && fresh[t] > S_max) bad_s = 1;
  __syncthreads();

  if (wave != 0) return;
  if (bad_s) {
    for (int j = lane; j < B1; j += kWave) chain[j] = -1;
    if (lane == 0) {
      *n_accepted = 0;
      *status = -4;  // SFV_E_STATE
    }
    return;
  }
  const uint64_t my_hs = lane < B1 ? hs[lane] : 0ull;
  const int my_depth = lane < B1 ? (int)tree.depth[lane] : -1;
  int cur = 0, h = 0, cur_depth = 0;
  while (h < B1 - 1) {
    if (lc[cur] == -1) break;
    const uint64_t target = hn[cur];
    unsigned long long cand =
        __ballot(lane >= 1 && lane < B1 && my_depth == cur_depth + 1 && my_hs == target);
    int found = -1;
    while (cand) {
      const int j = __ffsll((long long)cand) - 1;
      cand &= cand - 1;
      bool diff = false;
      for (int n = lane; n < N; n += kWave)
        diff = diff || (ls[j * N + n] != ln[cur * N + n]);
      if (!__any(diff)) {
        found = j;
        break;
      }
    }
    if (found < 0) break;
    if (lane == 0) chain[h] = found;
    ++h;
    cur = found;
    ++cur_depth;
  }
  for (int j = h + lane; j < B1; j += kWave) chain[j] = -1;
  if (lane == 0) {
    *n_accepted = h;
    *status = 0;
  }
}

}  // namespace

hipError_t launch_match(const int32_t* state, const int32_t* next_state, const int32_t* commit_pos,
                        const TreeArgs& tree, int N, int k_max, int S_max, int32_t* chain,
                        int32_t* n_accepted, int32_t* status, hipStream_t stream) {
  // Only the staged arrays are sized at launch: a small tree leaves room on a
  // CU beside long-running workgroups of other streams.  Above 64 KB (up to
  // 128 KB at 64 branches x 256 positions) the kernel's limit is raised first.
  const size_t lds = 2 * (size_t)tree.B1 * N * sizeof(int);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&match_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(match_kernel, dim3(1), dim3(kThreads), lds, stream, state, next_state, commit_pos,
                     tree, N, k_max, S_max, chain, n_accepted, status);
  return hipGetLastError();
}

}  // namespace sfv
