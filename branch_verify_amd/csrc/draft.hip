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
// Stale top-K: each masked row of the chosen branch is cut into up to 16
// chunks, one workgroup each.  In a chunk, the K-th largest of the 256
// per-thread maxima bounds the chunk's K-th largest value from below, so one
// more pass collects every element at or above it (typically a few dozen)
// into LDS, where they are ranked by (value desc, id asc); chunks with more
// than kCap such elements (many ties) fall back to K exact passes.  A second
// kernel ranks the chunks' candidates of each row.
//
// draft_tree_kernel: one wave builds the whole tree.  Nodes keep their
// committed positions as a bitmap; candidates (probability, parent, position)
// live in LDS and the best one is found by a wave reduction each step.
// Every floating-point decision is taken in the order the definition gives
// (the fp64 normalising sum as a fixed pairwise tree over 256 leaves, which
// one wave computes with shuffles; fp32 keys without contraction).
#include "common.h"
#include "internal.h"
#include "noise.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;
constexpr int kCap = 2048;  // collected candidates per row before the fallback

// Comparisons use bitwise & and | (no short circuit) so that they compile to
// lane-mask arithmetic instead of branches.
__device__ __forceinline__ bool key_better(float v, int i, float bv, int bi) {
  return (v > bv) | ((v == bv) & (i < bi));
}

struct TopkArgs {
  const float* logits;
  const int32_t* rows;
  const float* conf;
  int M, V, N, branch, K;
  int S, C;         // chunks per row, ids per chunk
  float* ws_val;    // [M][S][K] chunk candidates
  int* ws_id;
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

constexpr int kUnroll = 4;

// Top-K of one chunk [c0, c1) of one row (chunk size >= K): the K-th largest
// per-thread maximum bounds the chunk's K-th largest value from below, one
// more pass collects every element at or above it, and the collected ones are
// ranked.  Pads with (-inf, INT_MAX) when the chunk is shorter than K.
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(TopkArgs a) {
  __shared__ float s_max[kThreads];
  __shared__ float s_cv[kCap];
  __shared__ int s_ci[kCap];
  __shared__ int s_cnt;
  __shared__ float s_tau;
  __shared__ float s_rv[kThreads / kWave];
  __shared__ int s_ri[kThreads / kWave];
  const int t = threadIdx.x;
  const int r = blockIdx.x / a.S, sc = blockIdx.x % a.S;
  const int f = a.rows[r];
  if (f < 0 || f / a.N != a.branch) return;  // uniform: not a row of the chosen branch
  const float* row = a.logits + (size_t)r * a.V;
  const int c0 = sc * a.C, c1 = min(a.V, c0 + a.C);
  const int K = a.K;
  float* ov = a.ws_val + ((size_t)r * a.S + sc) * K;
  int* oi = a.ws_id + ((size_t)r * a.S + sc) * K;
  if (c0 >= c1) {
    for (int k = t; k < K; k += kThreads) {
      ov[k] = -INFINITY;
      oi[k] = 0x7FFFFFFF;
    }
    return;
  }

  // per-thread maximum over the thread's own elements only: each is then a
  // distinct element of the chunk, which makes the K-th largest a lower bound
  float lmax = -INFINITY;
  for (int v0 = c0 + t; v0 < c1; v0 += kThreads * kUnroll) {
    float x[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) x[j] = row[min(v0 + j * kThreads, c1 - 1)];  // loads unconditional
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) lmax = fmaxf(lmax, v0 + j * kThreads < c1 ? x[j] : -INFINITY);
  }
  s_max[t] = lmax;
  if (t == 0) s_cnt = 0;
  __syncthreads();
  const int kk = min(K, c1 - c0);
  {  // tau = kk-th largest per-thread maximum (ties by thread index)
    int rank = 0;
#pragma unroll 8
    for (int u = 0; u < kThreads; u += 4) {
      const float4 m4 = *(const float4*)&s_max[u];
      rank += (m4.x > lmax || (m4.x == lmax && u + 0 < t));
      rank += (m4.y > lmax || (m4.y == lmax && u + 1 < t));
      rank += (m4.z > lmax || (m4.z == lmax && u + 2 < t));
      rank += (m4.w > lmax || (m4.w == lmax && u + 3 < t));
    }
    if (rank == kk - 1) s_tau = lmax;
  }
  __syncthreads();
  const float tau = s_tau;
  for (int v0 = c0 + t; v0 < c1; v0 += kThreads * kUnroll) {
    float x[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) x[j] = row[min(v0 + j * kThreads, c1 - 1)];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int v = v0 + j * kThreads;
      if (v < c1 && x[j] >= tau) {
        const int c = atomicAdd(&s_cnt, 1);
        if (c < kCap) {
          s_cv[c] = x[j];
          s_ci[c] = v;
        }
      }
    }
  }
  __syncthreads();
  const int cnt = s_cnt;
  for (int k = kk + t; k < K; k += kThreads) {
    ov[k] = -INFINITY;
    oi[k] = 0x7FFFFFFF;
  }
  if (cnt <= kCap) {
    for (int c = t; c < cnt; c += kThreads) {
      const float x = s_cv[c];
      const int id = s_ci[c];
      int rank = 0;
      for (int e = 0; e < cnt; ++e) rank += key_better(s_cv[e], s_ci[e], x, id);
      if (rank < kk) {
        ov[rank] = x;
        oi[rank] = id;
      }
    }
  } else {
    // many ties at the bound: kk exact passes, each the best element below the previous one
    float pv = INFINITY;
    int pi = -1;
    for (int k = 0; k < kk; ++k) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
      for (int v = c0 + t; v < c1; v += kThreads) {
        const float x = row[v];
        if (key_better(pv, pi, x, v) && key_better(x, v, bv, bi)) {
          bv = x;
          bi = v;
        }
      }
      block_best(bv, bi, s_rv, s_ri);
      if (t == 0) {
        ov[k] = bv;
        oi[k] = bi;
      }
      pv = bv;
      pi = bi;
    }
  }
}

// Top-K of a row from its chunks' sorted candidate lists, into the
// position-indexed outputs: one wave, lane s holds the head of chunk s's list,
// and each of K rounds takes the best head.
__global__ __launch_bounds__(kWave) void topk_merge_kernel(TopkArgs a) {
  const int lane = threadIdx.x;
  const int r = blockIdx.x;
  const int f = a.rows[r];
  if (f < 0 || f / a.N != a.branch) return;
  const int n = f % a.N;
  const int K = a.K;
  const float* lv = a.ws_val + ((size_t)r * a.S + lane) * K;
  const int* li = a.ws_id + ((size_t)r * a.S + lane) * K;
  const bool has = lane < a.S;
  int p = 0;
  for (int k = 0; k < K; ++k) {
    float v = -INFINITY;
    int id = 0x7FFFFFFF;
    if (has && p < K) {
      v = lv[p];
      id = li[p];
    }
    float bv = v;
    int bi = id;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (key_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (has && id == bi && id != 0x7FFFFFFF) ++p;  // ids are distinct: exactly one lane advances
    if (lane == 0) {
      a.top_ids[(size_t)n * K + k] = bi;
      a.top_logit[(size_t)n * K + k] = bv;
    }
  }
  if (lane == 0) a.conf_pos[n] = a.conf[r];
}

// ---------------------------------------------------------------------------
// draft tree
// ---------------------------------------------------------------------------
constexpr int kMaxNodes = kMaxBranches;  // root + up to 63 drafts
constexpr int kMaxWidth = 16;
constexpr int kMaxCand = kMaxNodes * kMaxWidth;
constexpr int kWords = kMaxBlock / 32;
static_assert(kMaxBlock == 4 * kWave, "the pairwise sum gives each lane 4 of the 256 leaves");

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
  return (p > bp) | ((p == bp) & ((u < bu) | ((u == bu) & (n < bn))));
}

static_assert(kMaxTopkChunks <= kWave, "one merge lane per chunk");
constexpr int kCandPerLane = kMaxCand / kWave;

// Four waves rank the positions by confidence; then wave 0 alone builds the
// tree (no barrier per node).  Each node keeps the (position, token) commits
// of its path in LDS, so the state rows are written once, at the end.
constexpr int kTreeThreads = 4 * kWave;

// Orders this wave's LDS accesses around the point (the tree loop runs in a
// single wave, so no workgroup barrier is involved).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}
static_assert(kMaxBlock == kTreeThreads, "one thread per position for the ranking");

__global__ __launch_bounds__(kTreeThreads) void draft_tree_kernel(TreeDraftArgs a) {
  __shared__ int s_root[kMaxBlock];
  __shared__ float s_key[kMaxBlock];  // confidence of masked positions, -1 elsewhere
  __shared__ int s_top1[kMaxBlock];
  __shared__ int s_ord[kMaxBlock];
  __shared__ unsigned char nd_ppos[kMaxNodes][kMaxNodes];
  __shared__ int nd_ptok[kMaxNodes][kMaxNodes];
  __shared__ int nd_depth[kMaxNodes];
  __shared__ double nd_P[kMaxNodes];
  __shared__ unsigned nd_bits[kMaxNodes][kWords];
  __shared__ double c_P[kMaxCand];
  __shared__ int c_un[kMaxCand];  // parent << 16 | position; -1 once taken
  const int tid = threadIdx.x, lane = tid % kWave;
  const int N = a.N, K = a.K, D = a.D;
  const int W = a.W < 1 ? 1 : a.W;

  {
    const int n = tid;
    const int v = n < N ? a.root[n] : 0;
    const bool m = n < N && v == -1;
    s_root[n] = v;
    s_key[n] = m ? a.conf[n] : -1.f;  // confidences are >= 0
    s_top1[n] = m ? a.top_ids[(size_t)n * K] : 0;
  }
  if (tid < kWords) nd_bits[0][tid] = 0u;
  if (tid == 0) {
    nd_depth[0] = 0;
    nd_P[0] = 1.0;
    a.parent[0] = -1;
  }
  for (int c = tid; c < kMaxCand; c += kTreeThreads) c_un[c] = -1;
  __syncthreads();
  // confidence order of the root's masked positions (c descending, then
  // position): thread n ranks position n
  {
    const int n = tid;
    const float kc = s_key[n];
    int rank = 0;
#pragma unroll 4
    for (int q = 0; q < kMaxBlock; q += 4) {
      const float4 k4 = *(const float4*)&s_key[q];
      const float kq[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) rank += (kq[j] >= 0.f) & ((kq[j] > kc) | ((kq[j] == kc) & (q + j < n)));
    }
    if (kc >= 0.f) s_ord[rank] = n;
  }
  __syncthreads();
  if (tid >= kWave) return;  // the tree is one wave's work
  int nmask = 0;
  for (int q = lane; q < kMaxBlock; q += kWave) nmask += __popcll(__ballot(s_key[q] >= 0.f));

  int ncand = 0, nodes = 1, u = 0;
  for (;;) {
    // offer u's W most confident masked positions; the normaliser is the
    // pairwise tree over 256 leaves (zero where not masked), lane l holding
    // leaves 4l .. 4l+3
    double x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = 4 * lane + e;
      const float kn = s_key[n];
      x[e] = (kn >= 0.f && !((nd_bits[u][n >> 5] >> (n & 31)) & 1u)) ? (double)kn : 0.0;
    }
    double total = (x[0] + x[1]) + (x[2] + x[3]);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) total = total + __shfl_xor(total, o, kWave);
    const double Pu = nd_P[u];
    int taken = 0;
    for (int b0 = 0; b0 < nmask && taken < W; b0 += kWave) {
      const int k = b0 + lane;
      const int n = k < nmask ? s_ord[k] : 0;
      const bool free_n = k < nmask && !((nd_bits[u][n >> 5] >> (n & 31)) & 1u);
      const unsigned long long bal = __ballot(free_n);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (free_n && taken + before < W) {
        const int c = ncand + taken + before;
        c_P[c] = (Pu * (double)s_key[n]) / total;
        c_un[c] = (u << 16) | n;
      }
      taken += __popcll(bal);
    }
    ncand += min(taken, W);
    wave_sync();
    if (nodes >= D + 1) break;

    // best live candidate: probability, then parent index, then position
    double bp = -1.0;
    int bun = 0x7FFFFFFF, bc = -1;
#pragma unroll
    for (int j = 0; j < kCandPerLane; ++j) {
      const int c = j * kWave + lane;
      const int un = c_un[c];  // -1: never offered, or taken
      const double p = c_P[c];
      const bool take = (un >= 0) & ((bc < 0) | cand_better(p, un >> 16, un & 0xFFFF, bp, bun >> 16, bun & 0xFFFF));
      bp = take ? p : bp;
      bun = take ? un : bun;
      bc = take ? c : bc;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double op = __shfl_xor(bp, o, kWave);
      const int oun = __shfl_xor(bun, o, kWave), oc = __shfl_xor(bc, o, kWave);
      const bool take = (oc >= 0) & ((bc < 0) | cand_better(op, oun >> 16, oun & 0xFFFF, bp, bun >> 16, bun & 0xFFFF));
      bp = take ? op : bp;
      bun = take ? oun : bun;
      bc = take ? oc : bc;
    }
    if (bc < 0) break;  // uniform after the reduction
    const int pu = bun >> 16, pn = bun & 0xFFFF;
    const int b = nodes;
    // drafted token: stale argmax, or the Gumbel-max over the K candidates
    int tok;
    if (!a.noisy) {
      tok = s_top1[pn];
    } else {
      float kv = -INFINITY;
      int ki = 0x7FFFFFFF;
      if (lane < K) {
        const int id = a.top_ids[(size_t)pn * K + lane];
        const float l = a.top_logit[(size_t)pn * K + lane];
        const uint64_t step = a.step0 + (uint64_t)nd_depth[pu];
        const uint64_t pos = (uint64_t)(a.pos0 + pn);
        kv = (l * a.inv_t) + gumbel_exact(noise_word(a.seed, step, pos, (uint64_t)id));
        ki = id;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(kv, o, kWave);
        const int oi = __shfl_xor(ki, o, kWave);
        if (key_better(ov, oi, kv, ki)) {
          kv = ov;
          ki = oi;
        }
      }
      tok = ki;
    }
    // the child's path: its parent's commits and (pn, tok)
    const int dpu = nd_depth[pu];
    if (lane < dpu) {
      nd_ppos[b][lane] = nd_ppos[pu][lane];
      nd_ptok[b][lane] = nd_ptok[pu][lane];
    }
    if (lane == 0) {
      nd_ppos[b][dpu] = (unsigned char)pn;
      nd_ptok[b][dpu] = tok;
      c_un[bc] = -1;
      nd_depth[b] = nd_depth[pu] + 1;
      nd_P[b] = bp;
      a.parent[b] = pu;
    }
    if (lane < kWords) nd_bits[b][lane] = nd_bits[pu][lane] | ((pn >> 5) == lane ? (1u << (pn & 31)) : 0u);
    nodes = b + 1;
    u = b;
    wave_sync();
  }

  // rows: the root with each node's path commits; then copies of the root
  for (int b = 0; b <= D; ++b) {
    const int db = b < nodes ? nd_depth[b] : 0;
    for (int n = lane; n < N; n += kWave) {
      int v = s_root[n];
      if (b < nodes && v == -1 && ((nd_bits[b][n >> 5] >> (n & 31)) & 1u)) {
        for (int k = 0; k < db; ++k)
          if (nd_ppos[b][k] == n) v = nd_ptok[b][k];
      }
      a.states[(size_t)b * N + n] = v;
    }
  }
  for (int b = nodes + lane; b <= D; b += kWave) a.parent[b] = 0;
  if (lane == 0) a.n_drafts[0] = nodes - 1;
}

}  // namespace

TopkPlan topk_plan(int M, int V, int K) {
  TopkPlan pl;
  int S = (V + kTopkChunkTarget - 1) / kTopkChunkTarget;
  S = S < 1 ? 1 : (S > kMaxTopkChunks ? kMaxTopkChunks : S);
  int C = (V + S - 1) / S;
  if (C < K) C = K;
  S = (V + C - 1) / C;
  pl.S = S;
  pl.C = C;
  pl.ws_bytes = (size_t)M * S * K * (sizeof(float) + sizeof(int));
  return pl;
}

hipError_t launch_stale_topk(const float* logits, const int32_t* rows, const float* conf, int M, int V, int N,
                             int branch, int K, int32_t* top_ids, float* top_logit, float* conf_pos, void* ws,
                             const TopkPlan& plan, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  TopkArgs a;
  a.logits = logits;
  a.rows = rows;
  a.conf = conf;
  a.M = M;
  a.V = V;
  a.N = N;
  a.branch = branch;
  a.K = K;
  a.S = plan.S;
  a.C = plan.C;
  a.ws_val = (float*)ws;
  a.ws_id = (int*)((char*)ws + (size_t)M * plan.S * K * sizeof(float));
  a.top_ids = top_ids;
  a.top_logit = top_logit;
  a.conf_pos = conf_pos;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(M * plan.S), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(M), dim3(kWave), 0, stream, a);
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
  hipLaunchKernelGGL(draft_tree_kernel, dim3(1), dim3(kTreeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sfv
