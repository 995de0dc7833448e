// State-equality walk over the draft tree.
//
// SpecFold, introduction: drafted states and their logits are cached, and a
// later main-branch state equal to a cached draft reuses that draft's logits
// instead of another target pass.  SPOT ("How does SPOT draft and verify?"):
// the target accepts the longest prefix consistent with its own trajectory;
// with shared noise that is state equality (Proposition 2).
//
// One workgroup of four waves.  Phase 1 spreads the 2*B1 rows (every drafted
// state and every next state) over the waves: each wave checks a draft
// against its parent and folds a row into a 64-bit hash, sum over positions
// of mix(n, token) (order-free, so the lanes reduce it with shuffles).
// Phase 2 is the walk, in wave 0: each hop ballots the drafts whose hash
// equals the current next state and confirms the lowest candidate by a full,
// coalesced comparison, so a hash collision can never produce a false match.
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

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)v, o, kWave);
    const unsigned hi = __shfl_xor((unsigned)(v >> 32), o, kWave);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void match_kernel(const int32_t* state, const int32_t* next_state,
                                                         const int32_t* commit_pos, TreeArgs tree, int N,
                                                         int k_max, int S_max, int32_t* chain,
                                                         int32_t* n_accepted, int32_t* status) {
  __shared__ uint64_t hs[kMaxBranches];  // hash of state[i]
  __shared__ uint64_t hn[kMaxBranches];  // hash of next_state[i]
  __shared__ int bad_s;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int B1 = tree.B1;
  if (t == 0) bad_s = 0;
  __syncthreads();

  for (int row = wave; row < 2 * B1; row += kThreads / kWave) {
    const bool is_next = row >= B1;
    const int i = is_next ? row - B1 : row;
    const int32_t* src = (is_next ? next_state : state) + (size_t)i * N;
    uint64_t h = 0;
    for (int n = lane; n < N; n += kWave) h += mix(((uint64_t)(uint32_t)n << 32) | (uint32_t)src[n]);
    h = wave_sum_u64(h);
    if (lane == 0) (is_next ? hn : hs)[i] = h;
    if (!is_next && S_max >= 0 && i >= 1) {
      // a draft keeps every unmasked token of its parent and unmasks at most S_max more
      const int32_t* par = state + (size_t)tree.parent[i] * N;
      bool bad = false;
      int fresh = 0;
      for (int n = lane; n < N; n += kWave) {
        const int sp = par[n], sc = src[n];
        if (sp != -1) bad = bad || (sc != sp);
        else fresh += (sc != -1);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) fresh += __shfl_xor(fresh, o, kWave);
      if (__any(bad) || fresh > S_max) {
        if (lane == 0) bad_s = 1;
      }
    }
  }
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
  int cur = 0, h = 0;
  while (h < B1 - 1) {
    if (commit_pos[cur * k_max] == -1) break;
    const uint64_t target = hn[cur];
    unsigned long long cand = __ballot(lane >= 1 && lane < B1 && my_hs == target);
    int found = -1;
    while (cand) {
      const int j = __ffsll((long long)cand) - 1;
      cand &= cand - 1;
      bool diff = false;
      for (int n = lane; n < N; n += kWave)
        diff = diff || (state[(size_t)j * N + n] != next_state[(size_t)cur * N + n]);
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
  hipLaunchKernelGGL(match_kernel, dim3(1), dim3(kThreads), 0, stream, state, next_state, commit_pos,
                     tree, N, k_max, S_max, chain, n_accepted, status);
  return hipGetLastError();
}

}  // namespace sfv
