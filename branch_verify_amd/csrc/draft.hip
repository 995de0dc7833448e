// Drafting from stale conditionals: top-K per masked row, and a best-first
// draft tree (SSD-style confidence chain or BlockSpec-style confidence tree).
//
// SPOT ("On the SPOT: ...", "Important context"; "How does SPOT draft and
// verify?"; "How does SPOT differ from Spiffy, SSD and BlockSpec?"): the
// drafter reads the target's latest top-32 probabilities at each masked
// position and grows block states by predicting the next committed position,
// high-probability branches first, up to D drafted states; it applies the
// target's own Gumbel noise (coupled-noise match).
//
// stale_topk_kernel: one workgroup per masked row of the chosen branch.  The
// K-th largest of the 256 per-thread maxima bounds the row's K-th largest
// value from below, so one more pass collects every element at or above it
// (typically a few dozen) into LDS and ranks them by (value desc, id asc).
// Rows with more than kCap such elements (many ties) fall back to K exact
// passes.
//
// draft_tree_kernel: one workgroup builds the whole tree.  Nodes keep their
// committed positions as a bitmap; candidates (probability, parent, position)
// live in LDS and the best one is found by a block reduction each step.
// Every floating-point decision is taken in the order the definition gives
// (fp64 sums in increasing position, fp32 keys without contraction).
#include "common.h"
#include "internal.h"
#include "noise.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;
constexpr int kCap = 2048;  // collected candidates per row before the fallback

__device__ __forceinline__ bool key_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

struct TopkArgs {
  const float* logits;
  const int32_t* rows;
  const float* conf;
  int M, V, N, branch, K;
  int32_t* top_ids;
  float* top_logit;
  float* conf_pos;
};

// Block-wide best (value desc, id asc); every thread gets the result.
__device__ void block_best(float& v, int& i, float* sv, int* si) {
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(i, o, kWave);
    if (key_better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
  __syncthreads();
  if (lane == 0) {
    sv[wave] = v;
    si[wave] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int w = 1; w < kThreads / kWave; ++w)
    if (key_better(sv[w], si[w], v, i)) {
      v = sv[w];
      i = si[w];
    }
}

__global__ __launch_bounds__(kThreads) void stale_topk_kernel(TopkArgs a) {
  __shared__ float s_max[kThreads];
  __shared__ float s_cv[kCap];
  __shared__ int s_ci[kCap];
  __shared__ int s_cnt;
  __shared__ float s_tau;
  __shared__ float s_rv[kThreads / kWave];
  __shared__ int s_ri[kThreads / kWave];
  const int t = threadIdx.x;
  const int r = blockIdx.x;
  const int f = a.rows[r];
  if (f < 0 || f / a.N != a.branch) return;  // uniform: not a row of the chosen branch
  const int n = f % a.N;
  const float* row = a.logits + (size_t)r * a.V;
  const int K = a.K;

  float lmax = -INFINITY;
  for (int v = t; v < a.V; v += kThreads) lmax = fmaxf(lmax, row[v]);
  s_max[t] = lmax;
  if (t == 0) s_cnt = 0;
  __syncthreads();
  {  // tau = K-th largest per-thread maximum (ties by thread index)
    int rank = 0;
    for (int u = 0; u < kThreads; ++u) rank += (s_max[u] > lmax || (s_max[u] == lmax && u < t));
    if (rank == K - 1) s_tau = lmax;
  }
  __syncthreads();
  const float tau = s_tau;
  for (int v = t; v < a.V; v += kThreads) {
    const float x = row[v];
    if (x >= tau) {
      const int c = atomicAdd(&s_cnt, 1);
      if (c < kCap) {
        s_cv[c] = x;
        s_ci[c] = v;
      }
    }
  }
  __syncthreads();
  const int cnt = s_cnt;
  int32_t* oid = a.top_ids + (size_t)n * K;
  float* oval = a.top_logit + (size_t)n * K;
  if (cnt <= kCap) {
    for (int c = t; c < cnt; c += kThreads) {
      const float x = s_cv[c];
      const int id = s_ci[c];
      int rank = 0;
      for (int e = 0; e < cnt; ++e) rank += key_better(s_cv[e], s_ci[e], x, id);
      if (rank < K) {
        oid[rank] = id;
        oval[rank] = x;
      }
    }
  } else {
    // many ties at the bound: K exact passes, each the best element below the previous one
    float pv = INFINITY;
    int pi = -1;
    for (int k = 0; k < K; ++k) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int v = t; v < a.V; v += kThreads) {
        const float x = row[v];
        if (key_better(pv, pi, x, v) && key_better(x, v, bv, bi)) {
          bv = x;
          bi = v;
        }
      }
      block_best(bv, bi, s_rv, s_ri);
      if (t == 0) {
        oid[k] = bi;
        oval[k] = bv;
      }
      pv = bv;
      pi = bi;
    }
  }
  if (t == 0) a.conf_pos[n] = a.conf[r];
}

// ---------------------------------------------------------------------------
// draft tree
// ---------------------------------------------------------------------------
constexpr int kMaxNodes = kMaxBranches;  // root + up to 63 drafts
constexpr int kMaxWidth = 16;
constexpr int kMaxCand = kMaxNodes * kMaxWidth;
constexpr int kWords = kMaxBlock / 32;

struct TreeDraftArgs {
  const int32_t* root;
  const int32_t* top_ids;
  const float* top_logit;
  const float* conf;
  int N, K, D, W;
  bool noisy;
  float inv_t;
  uint64_t seed, step0;
  int64_t pos0;
  int32_t* parent;
  int32_t* states;
  int32_t* n_drafts;
};

__device__ __forceinline__ bool cand_better(double p, int u, int n, double bp, int bu, int bn) {
  return p > bp || (p == bp && (u < bu || (u == bu && n < bn)));
}

__global__ __launch_bounds__(kThreads) void draft_tree_kernel(TreeDraftArgs a) {
  __shared__ int s_root[kMaxBlock];
  __shared__ float s_conf[kMaxBlock];
  __shared__ int s_ord[kMaxBlock];
  __shared__ int nd_parent[kMaxNodes], nd_pos[kMaxNodes], nd_tok[kMaxNodes], nd_depth[kMaxNodes];
  __shared__ double nd_P[kMaxNodes];
  __shared__ unsigned nd_bits[kMaxNodes][kWords];
  __shared__ double c_P[kMaxCand];
  __shared__ int c_u[kMaxCand], c_n[kMaxCand];
  __shared__ unsigned char c_alive[kMaxCand];
  __shared__ int s_nmask, s_ncand, s_nodes, s_pick;
  __shared__ double s_total;
  __shared__ double r_P[kThreads / kWave];
  __shared__ int r_u[kThreads / kWave], r_n[kThreads / kWave], r_c[kThreads / kWave];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int N = a.N, K = a.K;
  const int W = a.W < 1 ? 1 : a.W;

  for (int n = t; n < N; n += kThreads) {
    s_root[n] = a.root[n];
    s_conf[n] = a.conf[n];
  }
  if (t < kWords) nd_bits[0][t] = 0u;
  if (t == 0) {
    nd_parent[0] = -1;
    nd_pos[0] = -1;
    nd_tok[0] = -1;
    nd_depth[0] = 0;
    nd_P[0] = 1.0;
    s_ncand = 0;
    s_nodes = 1;
  }
  __syncthreads();
  // confidence order of the root's masked positions: c descending, then position
  for (int n = t; n < N; n += kThreads) {
    if (s_root[n] != -1) continue;
    const float c = s_conf[n];
    int rank = 0;
    for (int m = 0; m < N; ++m)
      if (s_root[m] == -1) rank += (s_conf[m] > c || (s_conf[m] == c && m < n));
    s_ord[rank] = n;
  }
  if (t == 0) {
    int m = 0;
    for (int n = 0; n < N; ++n) m += s_root[n] == -1;
    s_nmask = m;
  }
  __syncthreads();

  int u = 0;  // node to offer children of (uniform)
  for (;;) {
    // offer u's W most confident masked positions
    if (t == 0) {
      double total = 0.0;  // increasing position, fp64
      for (int n = 0; n < N; ++n)
        if (s_root[n] == -1 && !((nd_bits[u][n >> 5] >> (n & 31)) & 1u)) total = total + (double)s_conf[n];
      s_total = total;
    }
    __syncthreads();
    if (wave == 0) {
      int taken = 0;
      for (int b0 = 0; b0 < s_nmask && taken < W; b0 += kWave) {
        const int k = b0 + lane;
        const int n = k < s_nmask ? s_ord[k] : 0;
        const bool free_n = k < s_nmask && !((nd_bits[u][n >> 5] >> (n & 31)) & 1u);
        const unsigned long long bal = __ballot(free_n);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        if (free_n && taken + before < W) {
          const int c = s_ncand + taken + before;
          c_P[c] = (nd_P[u] * (double)s_conf[n]) / s_total;
          c_u[c] = u;
          c_n[c] = n;
          c_alive[c] = 1;
        }
        taken += __popcll(bal);
      }
      if (lane == 0) s_ncand += min(taken, W);
    }
    __syncthreads();
    if (s_nodes >= a.D + 1) break;

    // best live candidate
    double bp = -1.0;
    int bu = 0x7FFFFFFF, bn = 0x7FFFFFFF, bc = -1;
    for (int c = t; c < s_ncand; c += kThreads) {
      if (c_alive[c] && (bc < 0 || cand_better(c_P[c], c_u[c], c_n[c], bp, bu, bn))) {
        bp = c_P[c];
        bu = c_u[c];
        bn = c_n[c];
        bc = c;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double op = __shfl_xor(bp, o, kWave);
      const int ou = __shfl_xor(bu, o, kWave), on = __shfl_xor(bn, o, kWave), oc = __shfl_xor(bc, o, kWave);
      if (oc >= 0 && (bc < 0 || cand_better(op, ou, on, bp, bu, bn))) {
        bp = op;
        bu = ou;
        bn = on;
        bc = oc;
      }
    }
    if (lane == 0) {
      r_P[wave] = bp;
      r_u[wave] = bu;
      r_n[wave] = bn;
      r_c[wave] = bc;
    }
    __syncthreads();
    if (t == 0) {
      int best = -1;
      for (int w = 0; w < kThreads / kWave; ++w) {
        if (r_c[w] < 0) continue;
        if (best < 0 || cand_better(r_P[w], r_u[w], r_n[w], r_P[best], r_u[best], r_n[best])) best = w;
      }
      s_pick = best < 0 ? -1 : r_c[best];
    }
    __syncthreads();
    const int pick = s_pick;
    if (pick < 0) break;
    const int pu = c_u[pick], pn = c_n[pick];
    const int b = s_nodes;
    // drafted token: stale argmax, or the Gumbel-max over the K candidates
    int tok;
    if (!a.noisy) {
      tok = a.top_ids[(size_t)pn * K];
    } else {
      float kv = -INFINITY;
      int ki = 0x7FFFFFFF;
      if (wave == 0 && lane < K) {
        const int id = a.top_ids[(size_t)pn * K + lane];
        const float l = a.top_logit[(size_t)pn * K + lane];
        const uint64_t step = a.step0 + (uint64_t)nd_depth[pu];
        const uint64_t pos = (uint64_t)(a.pos0 + pn);
        kv = (l * a.inv_t) + gumbel_exact(noise_word(a.seed, step, pos, (uint64_t)id));
        ki = id;
      }
      if (wave == 0) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ov = __shfl_xor(kv, o, kWave);
          const int oi = __shfl_xor(ki, o, kWave);
          if (key_better(ov, oi, kv, ki)) {
            kv = ov;
            ki = oi;
          }
        }
      }
      tok = ki;
    }
    if (t == 0) {
      c_alive[pick] = 0;
      nd_parent[b] = pu;
      nd_pos[b] = pn;
      nd_tok[b] = tok;
      nd_depth[b] = nd_depth[pu] + 1;
      nd_P[b] = c_P[pick];
      s_nodes = b + 1;
    }
    if (t < kWords) nd_bits[b][t] = nd_bits[pu][t] | ((pn >> 5) == t ? (1u << (pn & 31)) : 0u);
    __syncthreads();
    u = b;
  }

  // outputs: parents, states (the root with each path's commits), padding
  const int nodes = s_nodes;
  for (int b = t; b <= a.D; b += kThreads) a.parent[b] = b == 0 ? -1 : (b < nodes ? nd_parent[b] : 0);
  for (int e = t; e < (a.D + 1) * N; e += kThreads) {
    const int b = e / N, n = e % N;
    int v = s_root[n];
    if (b < nodes && v == -1 && ((nd_bits[b][n >> 5] >> (n & 31)) & 1u)) {
      int c = b;
      while (nd_pos[c] != n) c = nd_parent[c];
      v = nd_tok[c];
    }
    a.states[e] = v;
  }
  if (t == 0) a.n_drafts[0] = nodes - 1;
}

}  // namespace

hipError_t launch_stale_topk(const float* logits, const int32_t* rows, const float* conf, int M, int V, int N,
                             int branch, int K, int32_t* top_ids, float* top_logit, float* conf_pos,
                             hipStream_t stream) {
  if (M == 0) return hipSuccess;
  TopkArgs a{logits, rows, conf, M, V, N, branch, K, top_ids, top_logit, conf_pos};
  hipLaunchKernelGGL(stale_topk_kernel, dim3(M), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_draft_tree(const int32_t* root, const int32_t* top_ids, const float* top_logit,
                             const float* conf, int N, int K, int D, int W, float temperature, uint64_t seed,
                             uint64_t step0, int64_t pos0, int32_t* parent, int32_t* states, int32_t* n_drafts,
                             hipStream_t stream) {
  TreeDraftArgs a;
  a.root = root;
  a.top_ids = top_ids;
  a.top_logit = top_logit;
  a.conf = conf;
  a.N = N;
  a.K = K;
  a.D = D;
  a.W = W;
  a.noisy = temperature != 0.f;
  a.inv_t = a.noisy ? 1.0f / temperature : 0.f;
  a.seed = seed;
  a.step0 = step0;
  a.pos0 = pos0;
  a.parent = parent;
  a.states = states;
  a.n_drafts = n_drafts;
  hipLaunchKernelGGL(draft_tree_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sfv
