// Commit of every branch: token per masked row (greedy or Gumbel-max with
// counter-based noise shared by branches of equal depth), max-softmax
// confidence, and the per-branch unmask-argmax.  Also the masked-row scan.
//
// SPOT ("On the SPOT: ... Commit-Order Prediction"): exact decoding commits
// one masked position per target pass ("Important context", commit order);
// the drafter and the target share per-position Gumbel noise, so given the
// noise the target's transition is deterministic (coupled-noise match,
// Proposition 2).  SpecFold, introduction: an unmasking rule picks the
// high-confidence masked positions.
//
// Exactness: tokens and committed positions must equal the CPU definition
// bit for bit.  The vocabulary sweep runs a fast fp32 path with a proven
// error bound and re-decides exactly whatever falls inside the bound:
//  * Gumbel keys: each id's noise word falls in one of kGumbelBuckets runs
//    of words, with fp32 bounds lo <= g <= hi on its exact value (a table,
//    certified over all 2^32 words by sfv_selfcheck_bounds).  Rounding is
//    monotone, so fl32(x + lo) <= key <= fl32(x + hi).  The wave keeps the
//    best lower bound so far, and any id whose upper bound reaches it is
//    re-evaluated with fp64 logarithms, exactly as defined.  The exact argmax
//    is always among those.
//  * S = sum exp(l - max l): fp32 exp2 terms summed in fp64, with a running
//    bound E on |S - S_exact|.  A branch whose best and runner-up intervals
//    [S - E, S + E] overlap is re-decided from S summed with fp64 exp.
// This translation unit is compiled with -ffp-contract=off.
#include <mutex>

#include "common.h"
#include "gumbel_bounds.h"
#include "internal.h"
#include "noise.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;
constexpr int kPerIter = 8 * kThreads;  // vocab ids per workgroup iteration
constexpr int kItemRows = kItemRowsHost;
// The widest Gumbel bucket with 1% to spare: the distance from an id's upper key
// bound down to a certain lower bound of its key, beside the rounding term.
constexpr float kLowSlack = kGumbelMaxWidth * 1.01f;  // rows sharing one noise sweep
constexpr float kLog2e = kLog2eF;
// error model of one fast term (internal.h): |t / exp(x - m) - 1| <= kC1 * a + kC2
constexpr float kC1 = kExpC1;
constexpr float kC2 = kExpC2;

struct Item {
  int nrows;
  int pos;    // block position n
  int level;  // depth of the rows' branches
  int rows[kItemRows];
  int pad;
};

struct Partial {
  float lmax;  // max logit in the range
  int lidx;    // lowest id attaining it
  float kmax;  // max exact Gumbel key (T > 0)
  int kidx;    // lowest id attaining it
  double S;    // sum exp(l - lmax) over the range
  float E;     // bound on |S - S_exact|
  int pad;
};

struct WsLayout {
  int32_t* count;   // [1] work items
  Item* items;      // [items_max]
  Partial* part;    // [M][splits]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline WsLayout ws_layout(void* base, int B1, int N, int M, int items_max) {
  char* b = (char*)base;
  WsLayout w;
  size_t off = 0;
  w.count = (int32_t*)(b + off);
  off = align256(off + 16);
  w.items = (Item*)(b + off);
  off = align256(off + sizeof(Item) * (size_t)items_max);
  w.part = (Partial*)(b + off);
  return w;
}

size_t ws_bytes(int B1, int N, int M, int items_max, int splits) {
  size_t off = align256(16);
  off = align256(off + sizeof(Item) * (size_t)items_max);
  return off + sizeof(Partial) * (size_t)M * splits;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The bucket of a noise word in kGumbelBounds: w itself in the lower half
// (u < 1/2), ~w in the upper half, classed by the sign, exponent and top 4
// mantissa bits of its fp32 value (the generator's bucket_of_word).
__device__ __forceinline__ int gumbel_bucket(unsigned w) {
  const unsigned up = w >> 31;
  const unsigned t = w ^ (0u - up);
  const unsigned bits = __float_as_uint((float)t);
  return (int)(max(bits, 0x3F780000u) >> 19) - 2031 + (int)(up * 498u);
}

// Lexicographic "better" for (value, index): larger value, then lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// The exact key fl32(fl32(l_v / T) + g) of id v of a row, g from its noise word.
template <bool UNIT_T>
__device__ __forceinline__ float exact_key_t(const float* row, int v, unsigned w, float inv_t) {
  const float x = row[v];
  return (UNIT_T ? x : x * inv_t) + gumbel_exact(w);
}

// ---------------------------------------------------------------------------
// masked-row scan (one workgroup)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void masked_rows_kernel(const int32_t* state, int total,
                                                           int32_t* rows, int32_t* count) {
  __shared__ int wsum[16];
  __shared__ int base_s;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  if (t == 0) base_s = 0;
  __syncthreads();
  for (int f0 = 0; f0 < total; f0 += 1024) {
    const int f = f0 + t;
    const int flag = (f < total && state[f] == -1) ? 1 : 0;
    const unsigned long long bal = __ballot(flag);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int off = base_s;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (flag) rows[off + before] = f;
    __syncthreads();
    if (t == 0) {
      int s = 0;
      for (int w = 0; w < 16; ++w) s += wsum[w];
      base_s += s;
    }
    __syncthreads();
  }
  if (t == 0) *count = base_s;
}

// ---------------------------------------------------------------------------
// plan: row map and (for T > 0) work items grouping rows of equal (depth, n)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void commit_plan_kernel(const int32_t* rows, int M, int N,
                                                               TreeArgs tree, bool noisy, WsLayout ws) {
  __shared__ int wsum[kThreads / kWave];
  // flat position -> row, -1 if not masked: B1 * N ints, sized at launch so
  // that the kernel fits beside long-running workgroups of other streams
  extern __shared__ int rowmap[];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  if (!noisy) {
    if (t == 0) *ws.count = M;
    return;
  }
  const int total = tree.B1 * N;
  for (int f = t; f < total; f += kThreads) rowmap[f] = -1;
  __syncthreads();
  for (int r = t; r < M; r += kThreads) {
    const int f = rows[r];
    if (f >= 0 && f < total) rowmap[f] = r;  // ids outside the block are ignored
  }
  __syncthreads();
  // pairs p = level * N + n, contiguous ranges per thread
  const int pairs = tree.levels * N;
  const int per = (pairs + kThreads - 1) / kThreads;
  const int pb = t * per, pe = min(pairs, pb + per);
  int mine = 0;
  for (int p = pb; p < pe; ++p) {
    const int lv = p / N, n = p % N;
    int cnt = 0;
    for (int a = tree.level_start[lv]; a < tree.level_start[lv + 1]; ++a)
      cnt += rowmap[tree.by_level[a] * N + n] >= 0;
    mine += (cnt + kItemRows - 1) / kItemRows;
  }
  // exclusive prefix sum of the item counts over the threads, in thread order
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int up = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += up;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int off = incl - mine;
  for (int w = 0; w < wave; ++w) off += wsum[w];
  for (int p = pb; p < pe; ++p) {
    const int lv = p / N, n = p % N;
    Item it;
    it.nrows = 0;
    it.pos = n;
    it.level = lv;
    it.pad = 0;
    for (int a = tree.level_start[lv]; a < tree.level_start[lv + 1]; ++a) {
      const int r = rowmap[tree.by_level[a] * N + n];
      if (r < 0) continue;
#pragma unroll
      for (int k = 0; k < kItemRows; ++k)  // constant slot indices keep the item in registers
        if (k == it.nrows) it.rows[k] = r;
      if (++it.nrows == kItemRows) {
        ws.items[off++] = it;
        it.nrows = 0;
      }
    }
    if (it.nrows > 0) {
#pragma unroll
      for (int k = 0; k < kItemRows; ++k)
        if (k >= it.nrows) it.rows[k] = -1;
      ws.items[off++] = it;
    }
  }
  if (t == kThreads - 1) *ws.count = off;
}

// ---------------------------------------------------------------------------
// vocabulary sweep of one work item over one vocab range
// ---------------------------------------------------------------------------
// Adds 8 consecutive ids v .. v + 7 of one row to its running max, first
// argmax (IDX only: the sampled commit takes its token from the keys, and
// the maximum's value does not depend on it) and confidence sum: one max
// update per 8 ids, the 8 fast terms summed in fp32 (at most 7 roundings of a
// sum of positive terms: below 2^-21 of it) and the group sum added in fp64,
// with the bound E.
template <bool IDX>
__device__ __forceinline__ void group8(const float (&x)[8], int v, float& lmax, int& lidx, double& S, float& E) {
  float m8 = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) m8 = fmaxf(m8, x[e]);
  if (m8 > lmax) {
    if constexpr (IDX) {
      int e8 = 7;
#pragma unroll
      for (int e = 6; e >= 0; --e) e8 = x[e] == m8 ? e : e8;
      lidx = v + e8;
    }
    if (lmax != -INFINITY) {
      const float af = m8 - lmax;
      const float f = fast_exp2(-af * kLog2e);
      S *= (double)f;
      E = E * f + (float)S * (kC1 * af + kC2);
    }
    lmax = m8;
  }
  // sum of terms and sum of term * argument, started from the first term
  // (0 + t is t for every t >= 0, so the sums are those of a zero start)
  const float am0 = lmax - x[0];
  const float t0 = fast_exp2(-am0 * kLog2e);
  float gs = t0, ga = t0 * am0;
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    const float am = lmax - x[e];
    const float tt = fast_exp2(-am * kLog2e);
    gs += tt;
    ga += tt * am;
  }
  S += (double)gs;
  E += kC1 * ga + (kC2 + 4.76837158e-7f) * gs;
}

// The sampled sweep's form of group8: S and E are kept against a reference ref
// that moves only when a group's max passes it by more than kLazyMargin, so
// they are rescaled at a lane's first group and rarely after (each term is at
// most e^kLazyMargin, and the error model holds with |a|); the running max is
// kept beside it for the confidence.  No index: the sampled commit takes its
// token from the keys.
__device__ __forceinline__ void group8_lazy(const float (&x)[8], float& lmax, float& ref, double& S, float& E) {
  float m8 = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) m8 = fmaxf(m8, x[e]);
  lmax = fmaxf(lmax, m8);
  if (m8 - ref > kLazyMargin) {  // (a difference, exact when the two are close: no rounding of ref + margin)
    if (ref != -INFINITY) {
      const float af = m8 - ref;
      const float f = fast_exp2(-af * kLog2e);
      S *= (double)f;
      E = E * f + (float)S * (kC1 * af + kC2);
    }
    ref = m8;
  }
  const float am0 = ref - x[0];
  const float t0 = fast_exp2(-am0 * kLog2e);
  float gs = t0, ga = t0 * fabsf(am0);
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    const float am = ref - x[e];
    const float tt = fast_exp2(-am * kLog2e);
    gs += tt;
    ga += tt * fabsf(am);
  }
  S += (double)gs;
  E += kC1 * ga + (kC2 + 4.76837158e-7f) * gs;
}

struct RowsArgs {
  const float* logits;
  const int32_t* rows;
  int M, N, V;
  int splits, chunk;
  float inv_t;
  uint64_t seed, step0, pos0;
};

// UNIT_T: T = 1, where l * (1/T) = l exactly and the multiply is left out.
// Four waves per SIMD (at most 128 registers): the sampled sweep is bound by
// VALU issue and loses more from a lower occupancy than it saves elsewhere.
template <bool NOISY, int R, bool UNIT_T = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void commit_rows_kernel(RowsArgs a,
                                                                                                   WsLayout ws) {
  __shared__ float red_f[kThreads / kWave][R][2];
  __shared__ int red_i[kThreads / kWave][R][2];
  __shared__ double red_d[kThreads / kWave][R];
  __shared__ float red_e[kThreads / kWave][R];
  __shared__ float wg_lmax[R];
  __shared__ float2 gtab[NOISY ? kGumbelBuckets : 1];  // Gumbel bounds (lo, hi) per bucket

  const int item = blockIdx.x / a.splits;
  const int split = blockIdx.x % a.splits;
  if (NOISY && item >= *ws.count) return;  // at T = 0 there is one item per row, M in all
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  if (NOISY) {
    for (int i = t; i < kGumbelBuckets; i += kThreads) gtab[i] = make_float2(kGumbelBounds[2 * i], kGumbelBounds[2 * i + 1]);
    __syncthreads();
  }

  int nrows, row[R];
  uint64_t step = 0, pos = 0;
  if (NOISY) {
    const Item it = ws.items[item];
    nrows = it.nrows;
    __builtin_assume(nrows >= 1);  // the plan writes no empty item
#pragma unroll
    for (int k = 0; k < R; ++k) row[k] = k < nrows ? it.rows[k] : -1;
    step = a.step0 + (uint64_t)it.level;
    pos = a.pos0 + (uint64_t)it.pos;
  } else {
    nrows = 1;
    row[0] = item;
  }

  const int vb = split * a.chunk;
  const int ve = min(a.V, vb + a.chunk);

  float lmax[R], E[R], wbest[R], kmax[R];
  int lidx[R], kidx[R];
  double S[R];
  // T > 0: the lane's best key candidate so far as an interval blo <= key <=
  // bhi (equal once its exact key is known), its id and noise word
  float blo[R], bhi[R];
  unsigned bwd[R];
  float sref[R];  // T > 0: the reference S and E are kept against (group8_lazy)
#pragma unroll
  for (int k = 0; k < R; ++k) {
    lmax[k] = -INFINITY;
    lidx[k] = 0x7FFFFFFF;
    S[k] = 0.0;
    E[k] = 0.f;
    wbest[k] = -INFINITY;
    kmax[k] = -INFINITY;
    kidx[k] = 0x7FFFFFFF;
    blo[k] = -INFINITY;
    bhi[k] = -INFINITY;
    bwd[k] = 0;
    sref[k] = -INFINITY;
  }

  // Logit loads are unconditional: a lane past the range end reads the last
  // 8 ids of the range and then drops them, so the compiler never has to
  // drain outstanding loads at a branch.
  const float* rbase[R];  // rows past the item's last read that one again (an L1 hit, never used)
  int last_row = row[0];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    last_row = k < nrows ? row[k] : last_row;
    rbase[k] = a.logits + (size_t)last_row * a.V;
  }
  const int vlast = ve - 8;  // ve - vb >= 8: both are multiples of 8

  if constexpr (!NOISY) {
    // Greedy sweep.  Two iterations' logits are in flight in two register
    // sets used in turn (no register copies, which would make the compiler
    // wait for the newest loads).
    auto load8 = [&](float4& x0, float4& x1, int v) {
      const int vc = min(v, vlast);
      x0 = *(const float4*)(rbase[0] + vc);
      x1 = *(const float4*)(rbase[0] + vc + 4);
    };
    auto take8 = [&](const float4& x0, const float4& x1, int v) {
      if (v >= ve) return;  // ve and v are multiples of 8
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      group8<true>(x, v, lmax[0], lidx[0], S[0], E[0]);
    };
    float4 a0, a1, b0, b1;
    load8(a0, a1, vb + 8 * t);
    load8(b0, b1, vb + kPerIter + 8 * t);
    for (int v0 = vb; v0 < ve; v0 += 2 * kPerIter) {
      const int v = v0 + 8 * t;
      take8(a0, a1, v);
      load8(a0, a1, v + 2 * kPerIter);
      take8(b0, b1, v + kPerIter);
      load8(b0, b1, v + 3 * kPerIter);
    }
  } else {
    // The trip count is uniform across the workgroup (cross-lane reductions
    // run inside the loop); a lane past the range end keeps every value at
    // -inf.
    // Each row's logits are loaded two rows ahead of their use (the first two
    // before the noise, whose arithmetic covers their latency); all loads are
    // unconditional.
    constexpr int kRowsAhead = 2;
    for (int v0 = vb; v0 < ve; v0 += kPerIter) {
      const int v = v0 + 8 * t;
      const bool active = v < ve;  // ve and v are multiples of 8
      const int vc = min(v, vlast);
      float4 xa[R][2];
#pragma unroll
      for (int k = 0; k < kRowsAhead && k < R; ++k) {
        xa[k][0] = *(const float4*)(rbase[k] + vc);
        xa[k][1] = *(const float4*)(rbase[k] + vc + 4);
      }
      unsigned wd[8];
      float2 gb[8];  // bounds on the Gumbel noise of the 8 ids
      noise_block(a.seed, step, pos, (uint64_t)(v >> 3), wd);
#pragma unroll
      for (int e = 0; e < 8; ++e) gb[e] = gtab[gumbel_bucket(wd[e])];
      // (predicated blocks, not breaks, so that every loop unrolls and the
      // small arrays stay in registers)
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if (k + kRowsAhead < R) {
          xa[k + kRowsAhead][0] = *(const float4*)(rbase[k + kRowsAhead] + vc);
          xa[k + kRowsAhead][1] = *(const float4*)(rbase[k + kRowsAhead] + vc + 4);
        }
        if (k < nrows) {
          const float4 x0 = xa[k][0];
          const float4 x1 = xa[k][1];
          // (an inactive lane's values are never used: the sums below and
          // the exact keys are guarded, and its key bounds are -inf)
          const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          // running max / first argmax and the confidence sum (this lane's
          // ids), one max update per 8 ids as in the greedy sweep
          if (active) group8_lazy(x, lmax[k], sref[k], S[k], E[k]);
          // key bounds fl32(x/T + lo) <= key <= fl32(x/T + hi); wbest is a
          // lower bound of the wave's largest key so far, so every id whose key
          // can reach that key has its upper bound at or above it
          float kh[8], hm = -INFINITY;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xs = UNIT_T ? x[e] : x[e] * a.inv_t;
            kh[e] = xs + gb[e].y;
            hm = fmaxf(hm, kh[e]);
          }
          if (!active) hm = -INFINITY;
          // A lower bound of the key of the id whose upper bound is hm: its lower
          // bound lies at most the widest bucket below, plus the two fp32
          // roundings (each below 2^-24 of the sum), both covered with margin.
          const float lm = hm - fmaf(fabsf(hm), 0x1p-21f, kLowSlack);
          // (the wave max only when some lane's bound beats the best so far:
          // otherwise it would leave wbest as it is)
          if (__any(lm > wbest[k])) wbest[k] = fmaxf(wbest[k], wave_max_dpp(lm));
          // (the per-id tests only when some lane has a candidate)
          // A candidate replaces the lane's best when its interval lies above
          // the best's; where the two overlap, their exact keys decide (larger
          // key, then lower id); one whose upper end does not pass the best's
          // lower end cannot win (a tie at that end goes to the best, whose id
          // is lower: a lane meets its ids in increasing order).
          if (__any(hm >= wbest[k])) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (active && kh[e] >= wbest[k] && kh[e] > blo[k]) {
                const float xs = UNIT_T ? x[e] : x[e] * a.inv_t;
                const float lo = xs + gb[e].x;
                if (lo > bhi[k]) {
                  blo[k] = lo;
                  bhi[k] = kh[e];
                  kidx[k] = v + e;
                  bwd[k] = wd[e];
                } else {
                  const float ke = xs + gumbel_exact(wd[e]);
                  const float kb = blo[k] == bhi[k] ? blo[k] : exact_key_t<UNIT_T>(rbase[k], kidx[k], bwd[k], a.inv_t);
                  if (better(ke, v + e, kb, kidx[k])) {
                    kidx[k] = v + e;
                    bwd[k] = wd[e];
                    blo[k] = bhi[k] = ke;
                  } else {
                    blo[k] = bhi[k] = kb;
                  }
                }
              }
            }
          }
        }
      }
    }
  }

  // The thread index after the sweep is rebuilt from the wave's index (a
  // uniform value) and the lane id, so that no register holds it through the
  // loop.
  const int we = wave_u;
  int le;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(le));
  const int te = we * kWave + le;

  if constexpr (NOISY) {
    // Every id whose key can reach the wave's largest key has its upper end
    // at or above wbest, and the lane's best is the only such id of the lane
    // that can win: its exact key enters the reduction.
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (k >= nrows) break;
      if (bhi[k] != -INFINITY && bhi[k] >= wbest[k])
        kmax[k] = blo[k] == bhi[k] ? blo[k] : exact_key_t<UNIT_T>(rbase[k], kidx[k], bwd[k], a.inv_t);
      else
        kidx[k] = 0x7FFFFFFF;
    }
  }

  // ---- reduce over the workgroup, row by row ----
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k >= nrows) break;
    float bm = lmax[k];
    int bi = lidx[k];
    float km = kmax[k];
    int ki = kidx[k];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float om = __shfl_xor(bm, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(om, oi, bm, bi)) {
        bm = om;
        bi = oi;
      }
      if (NOISY) {
        const float okm = __shfl_xor(km, o, kWave);
        const int oki = __shfl_xor(ki, o, kWave);
        if (better(okm, oki, km, ki)) {
          km = okm;
          ki = oki;
        }
      }
    }
    if (le == 0) {
      red_f[we][k][0] = bm;
      red_i[we][k][0] = bi;
      red_f[we][k][1] = km;
      red_i[we][k][1] = ki;
    }
  }
  __syncthreads();
  if (te < R && te < nrows) {
    float bm = red_f[0][te][0];
    int bi = red_i[0][te][0];
    for (int w = 1; w < kThreads / kWave; ++w)
      if (better(red_f[w][te][0], red_i[w][te][0], bm, bi)) {
        bm = red_f[w][te][0];
        bi = red_i[w][te][0];
      }
    wg_lmax[te] = bm;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k >= nrows) break;
    const float M = wg_lmax[k];
    double s = 0.0;
    float e = 0.f;
    // (S and E are kept against lmax in the greedy sweep, against sref in the
    // sampled one)
    const float sr = NOISY ? sref[k] : lmax[k];
    if (sr != -INFINITY) {
      const double f = exp((double)sr - (double)M);  // fp64: exact to ~1 ulp
      s = S[k] * f;
      e = (float)((double)E[k] * f) + (float)s * 1e-12f;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      s += __shfl_xor(s, o, kWave);
      e += __shfl_xor(e, o, kWave);
    }
    if (le == 0) {
      red_d[we][k] = s;
      red_e[we][k] = e;
    }
  }
  __syncthreads();
  if (te < R && te < nrows) {
    double s = 0.0;
    float e = 0.f;
    float km = red_f[0][te][1];
    int ki = red_i[0][te][1];
    for (int w = 0; w < kThreads / kWave; ++w) {
      s += red_d[w][te];
      e += red_e[w][te];
      if (w && better(red_f[w][te][1], red_i[w][te][1], km, ki)) {
        km = red_f[w][te][1];
        ki = red_i[w][te][1];
      }
    }
    float bm = red_f[0][te][0];
    int bi = red_i[0][te][0];
    for (int w = 1; w < kThreads / kWave; ++w)
      if (better(red_f[w][te][0], red_i[w][te][0], bm, bi)) {
        bm = red_f[w][te][0];
        bi = red_i[w][te][0];
      }
    Partial pr;
    pr.lmax = bm;
    pr.lidx = bi;
    pr.kmax = km;
    pr.kidx = ki;
    pr.S = s;
    pr.E = e * 1.0001f + (float)(s * 1e-13);
    pr.pad = 0;
    ws.part[(size_t)row[te] * a.splits + split] = pr;
  }
}

// ---------------------------------------------------------------------------
// finalize: merge ranges, token/conf per row, unmask-argmax per branch
// ---------------------------------------------------------------------------
struct FinArgs {
  const float* logits;
  const int32_t* rows;
  const int32_t* state;
  int32_t* next_state;
  int32_t* commit_pos;
  int32_t* token;
  float* conf;
  int M, N, V, splits;
  int k_max;
  float tau;
  bool noisy;
};

// One workgroup per branch.
__global__ __launch_bounds__(kThreads) void commit_finalize_kernel(FinArgs a, WsLayout ws) {
  __shared__ int lmap[kMaxBlock];  // position -> masked row, -1 if none
  __shared__ double sS[kMaxBlock];
  __shared__ float sE[kMaxBlock];
  __shared__ float sM[kMaxBlock];
  __shared__ int sTok[kMaxBlock];
  __shared__ int sCand[kMaxBlock];
  __shared__ double red[kThreads / kWave];
  __shared__ int best_n_s, ncand_s;
  __shared__ double sX[kMaxBlock];  // S used for the ranking (exact where an interval is ambiguous)
  __shared__ int sNeed[kMaxBlock];
  __shared__ int sSel[kMaxBlock];
  __shared__ double sU;
  static_assert(kMaxBlock <= kThreads, "one thread per position below");

  const int i = blockIdx.x;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int N = a.N;
  const int f0 = i * N;
  for (int n = t; n < N; n += kThreads) lmap[n] = -1;
  __syncthreads();
  for (int r = t; r < a.M; r += kThreads) {  // the rows of this branch's positions
    const int f = a.rows[r];
    if (f >= f0 && f < f0 + N) lmap[f - f0] = r;
  }
  __syncthreads();

  // merge the vocab ranges of each masked position: token, S and its error bound
  for (int n = t; n < N; n += kThreads) {
    sS[n] = -1.0;  // not masked
    const int r = lmap[n];
    if (a.state[f0 + n] != -1 || r < 0) continue;
    const Partial* pp = ws.part + (size_t)r * a.splits;
    float M = -INFINITY, km = -INFINITY;
    int mi = 0x7FFFFFFF, ki = 0x7FFFFFFF;
    for (int s = 0; s < a.splits; ++s) {
      if (better(pp[s].lmax, pp[s].lidx, M, mi)) {
        M = pp[s].lmax;
        mi = pp[s].lidx;
      }
      if (better(pp[s].kmax, pp[s].kidx, km, ki)) {
        km = pp[s].kmax;
        ki = pp[s].kidx;
      }
    }
    double S = 0.0, E = 0.0;
    for (int s = 0; s < a.splits; ++s) {
      if (pp[s].lmax == -INFINITY) continue;
      const double f2 = exp((double)pp[s].lmax - (double)M);
      S += pp[s].S * f2;
      E += (double)pp[s].E * f2;
    }
    E = E * 1.0001 + S * 1e-13;
    const int tok = a.noisy ? ki : mi;
    a.token[r] = tok;
    a.conf[r] = (float)(1.0 / S);
    sS[n] = S;
    sE[n] = (float)E;
    sM[n] = M;
    sTok[n] = tok;
  }
  __syncthreads();

  // Smallest S (highest confidence), ties to the lowest position, then every
  // position whose interval [S - E, S + E] reaches the best one's upper end.
  if (wave == 0) {
    double bs = 0.0;
    int bn = -1;
    for (int n = lane; n < N; n += kWave) {
      if (sS[n] >= 0.0 && (bn < 0 || sS[n] < bs)) {
        bs = sS[n];
        bn = n;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double os = __shfl_xor(bs, o, kWave);
      const int on = __shfl_xor(bn, o, kWave);
      if (on >= 0 && (bn < 0 || os < bs || (os == bs && on < bn))) {
        bs = os;
        bn = on;
      }
    }
    int cnt = 0;
    if (bn >= 0) {
      const double hi = bs + (double)sE[bn];
      for (int base = 0; base < N; base += kWave) {
        const int n = base + lane;
        const bool c = n < N && sS[n] >= 0.0 && sS[n] - (double)sE[n] <= hi;
        const unsigned long long bal = __ballot(c);
        if (c) sCand[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = n;
        cnt += __popcll(bal);
      }
    }
    if (lane == 0) {
      best_n_s = bn;
      ncand_s = cnt;
    }
  }
  __syncthreads();

  // Exact S of position n: fp64 exp summed in a fixed order by the workgroup.
  auto exact_S = [&](int n) -> double {
    const float* src = a.logits + (size_t)lmap[n] * a.V;
    const double M = (double)sM[n];
    double s = 0.0;
    for (int v = t; v < a.V; v += kThreads) s += exp((double)src[v] - M);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, kWave);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    double tot = 0.0;
    for (int w = 0; w < kThreads / kWave; ++w) tot += red[w];
    __syncthreads();
    return tot;
  };

  if (a.k_max == 1) {
    int best = best_n_s;
    if (ncand_s > 1) {  // re-decide exactly among the overlapping intervals
      double bestS = 0.0;
      best = -1;
      for (int c = 0; c < ncand_s; ++c) {
        const int n = sCand[c];
        const double tot = exact_S(n);
        if (best < 0 || tot < bestS) {
          best = n;
          bestS = tot;
        }
      }
    }
    for (int n = t; n < N; n += kThreads) {
      const int f = f0 + n;
      a.next_state[f] = (n == best) ? sTok[n] : a.state[f];
    }
    if (t == 0) a.commit_pos[i] = best;
    return;
  }

  // Threshold commit of up to k_max positions (SpecFold, evaluation setup,
  // "Models and baselines": the decoders unmask the positions whose
  // confidence clears a threshold, 0.9 there): in
  // (S ascending, position ascending) order, the first position, then the
  // following ones while fewer than k_max are taken and fl32(1/S) >= tau.
  // Candidates are the positions whose interval [S - E, S + E] starts at or
  // below U, the k_max-th smallest upper end: no other can be among the first
  // k_max.  A candidate gets its exact S when its interval overlaps another
  // candidate's or when its two ends fall on different sides of tau.
  const bool mk = t < N && sS[t] >= 0.0;
  const double lo = mk ? sS[t] - (double)sE[t] : 0.0;
  const double hi = mk ? sS[t] + (double)sE[t] : 0.0;
  const int nm = __syncthreads_count(mk);
  const int kk = min(a.k_max, nm);
  if (mk) {
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      if (m == t || sS[m] < 0.0) continue;
      const double hm = sS[m] + (double)sE[m];
      rank += (hm < hi || (hm == hi && m < t));
    }
    if (rank == kk - 1) sU = hi;
  }
  __syncthreads();
  const double U = nm > 0 ? sU : 0.0;
  const bool inC = mk && lo <= U;
  if (t < kMaxBlock) {
    bool need = false;
    if (inC) {
      for (int m = 0; m < N; ++m) {
        if (m == t || sS[m] < 0.0) continue;
        const double lm = sS[m] - (double)sE[m], hm = sS[m] + (double)sE[m];
        if (lm <= U && lo <= hm && lm <= hi) need = true;
      }
      const bool c_lo = (float)(1.0 / hi) >= a.tau;  // confidence at the interval's ends
      const bool c_hi = (float)(1.0 / lo) >= a.tau;
      if (c_lo != c_hi) need = true;
    }
    sNeed[t] = need;
    sSel[t] = 0;
    sX[t] = mk ? sS[t] : -1.0;
  }
  __syncthreads();
  for (int n = 0; n < N; ++n) {  // uniform: every thread reads the same flags
    if (!sNeed[n]) continue;
    const double e = exact_S(n);
    if (t == 0) sX[n] = e;
  }
  __syncthreads();
  if (t == 0) {
    int taken = 0;
    while (taken < kk) {
      int bn = -1;
      double bs = 0.0;
      for (int n = 0; n < N; ++n) {
        if (sS[n] < 0.0 || sSel[n] || sS[n] - (double)sE[n] > U) continue;
        if (bn < 0 || sX[n] < bs) {
          bn = n;
          bs = sX[n];
        }
      }
      if (bn < 0) break;
      if (taken > 0 && !((float)(1.0 / bs) >= a.tau)) break;
      sSel[bn] = 1;
      a.commit_pos[i * a.k_max + taken] = bn;
      ++taken;
    }
    for (int j = taken; j < a.k_max; ++j) a.commit_pos[i * a.k_max + j] = -1;
  }
  __syncthreads();
  for (int n = t; n < N; n += kThreads) {
    const int f = f0 + n;
    a.next_state[f] = sSel[n] ? sTok[n] : a.state[f];
  }
}

// ---------------------------------------------------------------------------
// greedy commit from the fused LM head's tile partials
// ---------------------------------------------------------------------------
// Workgroup (row group g, chunk c): rows 4 g .. 4 g + 3 and the partials of
// chunk c (one per vocab tile).  Thread t takes row 4 g + t % 4 and every
// 64th partial from t / 4 (the four rows of a tile are 64 contiguous bytes;
// a thread's loads are issued before the merging starts) into a running
// (max, first argmax, S, E) with the sweep's error model: a partial's S is
// rescaled by a fast factor when the running max moves or lies above the
// partial's.  The 64 threads of a row then merge by shuffles with fast
// factors of the same model and across the four waves in fp64, and the row's
// partial for chunk c is written in the layout the finalize kernel reads.
struct Run {
  float m;
  int i;
  double S;
  float E;
};

// Adds the partial (m2, i2, S2, E2) to r (fast factors, bounded).
__device__ __forceinline__ void run_add(Run& r, float m2, int i2, double S2, float E2) {
  if (m2 == -INFINITY) return;
  if (m2 > r.m) {
    if (r.m != -INFINITY) {
      const float a = m2 - r.m;
      const float f = fast_exp2(-a * kLog2e);
      r.S *= (double)f;
      r.E = r.E * f + (float)r.S * (kC1 * a + kC2);
    }
    r.m = m2;
    r.i = i2;
  } else if (m2 == r.m && i2 < r.i) {
    r.i = i2;
  }
  const float a = r.m - m2;
  const float f = fast_exp2(-a * kLog2e);
  const double sf = S2 * (double)f;
  r.S += sf;
  r.E += E2 * f + (float)sf * (kC1 * a + kC2);
}

constexpr int kMergeRows = 4;                       // rows per workgroup
constexpr int kMergeLanes = kThreads / kMergeRows;  // partial lanes per row
constexpr int kMergeUnroll = 10;                    // loads in flight per thread

__global__ __launch_bounds__(kThreads) void greedy_merge_kernel(const GreedyPart* gp, int nparts, int M,
                                                                WsLayout ws) {
  __shared__ float wm[kThreads / kWave][kMergeRows];
  __shared__ int wi[kThreads / kWave][kMergeRows];
  __shared__ double wsum[kThreads / kWave][kMergeRows];
  __shared__ float we[kThreads / kWave][kMergeRows];
  const int g = blockIdx.x / kGreedyChunks;
  const int c = blockIdx.x % kGreedyChunks;
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int rr = t % kMergeRows, j = t / kMergeRows;
  const int m = g * kMergeRows + rr;
  const int mm = min(m, M - 1);  // pad rows read row M - 1 (in bounds) and are never written
  const int per = (nparts + kGreedyChunks - 1) / kGreedyChunks;
  const int s0 = c * per, s1 = min(nparts, s0 + per);
  Run r{-INFINITY, 0x7FFFFFFF, 0.0, 0.f};
  for (int sb = s0; sb < s1; sb += kMergeLanes * kMergeUnroll) {
    GreedyPart e[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int st = min(sb + u * kMergeLanes + j, nparts - 1);
      e[u] = gp[(size_t)st * M + mm];
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u)
      if (sb + u * kMergeLanes + j < s1) {
        // (a partial's S is an fp32 sum; 2^-23 of it covers one more rounding)
        run_add(r, e[u].m, e[u].idx, (double)e[u].S, e[u].E + e[u].S * 1.1920929e-7f);
      }
  }
#pragma unroll
  for (int o = kMergeRows; o < kWave; o <<= 1) {  // lanes of the same row
    const float m2 = __shfl_xor(r.m, o, kWave);
    const int i2 = __shfl_xor(r.i, o, kWave);
    const double S2 = __shfl_xor(r.S, o, kWave);
    const float E2 = __shfl_xor(r.E, o, kWave);
    run_add(r, m2, i2, S2, E2);
  }
  if (lane < kMergeRows) {
    wm[wave][rr] = r.m;
    wi[wave][rr] = r.i;
    wsum[wave][rr] = r.S;
    we[wave][rr] = r.E;
  }
  __syncthreads();
  if (t < kMergeRows && m < M) {
    float bm = wm[0][t];
    int bi = wi[0][t];
    for (int w = 1; w < kThreads / kWave; ++w)
      if (better(wm[w][t], wi[w][t], bm, bi)) {
        bm = wm[w][t];
        bi = wi[w][t];
      }
    double tot = 0.0, err = 0.0;
    for (int w = 0; w < kThreads / kWave; ++w) {
      if (wm[w][t] == -INFINITY) continue;
      const double f = exp((double)wm[w][t] - (double)bm);  // fp64: exact to ~1 ulp
      tot += wsum[w][t] * f;
      err += (double)we[w][t] * f;
    }
    Partial pr;
    pr.lmax = bm;
    pr.lidx = bi;
    pr.kmax = -INFINITY;
    pr.kidx = 0x7FFFFFFF;
    pr.S = tot;
    pr.E = (float)(err * 1.0001 + tot * 1e-13);
    pr.pad = 0;
    ws.part[(size_t)m * kGreedyChunks + c] = pr;
  }
}

// ---------------------------------------------------------------------------
// self-check of the fast-path bounds
// ---------------------------------------------------------------------------
__device__ __forceinline__ void atomic_max_pos_double(double* addr, double v) {
  atomicMax((unsigned long long*)addr, (unsigned long long)__double_as_longlong(v));
}

// out[0] = max over all 2^32 words of how far the exact noise value (the
// exact path's gumbel_exact) lies outside its bucket's bounds: 0 certifies
// the table.
__global__ __launch_bounds__(256) void selfcheck_gumbel_kernel(double* out) {
  const uint64_t total = 1ull << 32;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  double worst = 0.0;
  for (uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total; w += stride) {
    const int b = gumbel_bucket((unsigned)w);
    const double g = (double)gumbel_exact((unsigned)w);
    const double lo = (double)kGumbelBounds[2 * b], hi = (double)kGumbelBounds[2 * b + 1];
    worst = fmax(worst, fmax(lo - g, g - hi));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) worst = fmax(worst, __shfl_xor(worst, o, kWave));
  if (threadIdx.x % kWave == 0) atomic_max_pos_double(out, worst);
}

// gumbel_exact of the words first .. first + count - 1 (the defined noise
// value the commit's exact path uses), one per thread, grid-stride.
__global__ __launch_bounds__(256) void gumbel_words_kernel(uint32_t first, uint32_t count, float* out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    out[i] = gumbel_exact(first + (uint32_t)i);
}

__global__ __launch_bounds__(256) void selfcheck_exp2_kernel(double* out) {
  // every fp32 x in [-126, 0] (bit patterns 0x80000000 .. 0xC2FC0000) and in
  // [0, kExp2ArgMax] (0x00000000 .. the bits of kExp2ArgMax)
  const uint64_t nneg = 0xC2FC0000ull - 0x80000000ull + 1;
  const uint64_t total = nneg + __float_as_uint(kExp2ArgMax) + 1;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  double worst = 0.0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const unsigned b = i < nneg ? (unsigned)(0x80000000ull + i) : (unsigned)(i - nneg);
    const float x = __uint_as_float(b);
    const double ref = exp2((double)x);
    const double err = fabs((double)fast_exp2(x) - ref) / ref;
    worst = fmax(worst, err);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) worst = fmax(worst, __shfl_xor(worst, o, kWave));
  if (threadIdx.x % kWave == 0) atomic_max_pos_double(out + 1, worst);
}

__global__ void zero2_kernel(double* out) {
  if (threadIdx.x < 2) out[threadIdx.x] = 0.0;
}

}  // namespace

CommitPlan commit_plan(int B1, int N, int M, int V, int items_max, bool noisy) {
  CommitPlan pl;
  pl.items_max = items_max;
  const int max_splits = (V + kPerIter - 1) / kPerIter;
  const int base = items_max > 0 ? items_max : 1;
  int splits = ((noisy ? 2048 : 1024) + base - 1) / base;
  if (splits > max_splits) splits = max_splits;
  if (splits > 64) splits = 64;
  if (splits < 1) splits = 1;
  int chunk = (V + splits - 1) / splits;
  chunk = (chunk + kPerIter - 1) / kPerIter * kPerIter;
  splits = (V + chunk - 1) / chunk;
  pl.splits = splits;
  pl.chunk = chunk;
  pl.ws_bytes = ws_bytes(B1, N, M, items_max, splits);
  return pl;
}

// Workspace of sfv_commit_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  In host code `scratch` only names the
// symbol; its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept.
namespace {
static __device__ __align__(256) unsigned char scratch[kCommitScratchBytes];
constexpr int kMaxDevices = 64;
}  // namespace

hipError_t commit_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_masked_rows(const int32_t* state, int B1, int N, int32_t* rows, int32_t* count,
                              hipStream_t stream) {
  hipLaunchKernelGGL(masked_rows_kernel, dim3(1), dim3(1024), 0, stream, state, B1 * N, rows, count);
  return hipGetLastError();
}

hipError_t launch_commit(const float* logits, const int32_t* rows, int M, const int32_t* state,
                         const TreeArgs& tree, int N, int V, float temperature, uint64_t seed,
                         uint64_t step0, int64_t pos0, int k_max, float tau, int32_t* next_state,
                         int32_t* commit_pos,
                         int32_t* token, float* conf, void* ws_base, const CommitPlan& plan,
                         hipStream_t stream) {
  const bool noisy = temperature > 0.f;
  WsLayout ws = ws_layout(ws_base, tree.B1, N, M, plan.items_max);
  hipError_t e = hipSuccess;
  if (noisy) {  // work items group the rows of equal (depth, position); at T = 0 an item is a row
    const size_t lds = (size_t)tree.B1 * N * sizeof(int);  // at most 64 KB (64 branches x 256)
    hipLaunchKernelGGL(commit_plan_kernel, dim3(1), dim3(kThreads), lds, stream, rows, M, N, tree, noisy, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (M > 0) {
    RowsArgs ra;
    ra.logits = logits;
    ra.rows = rows;
    ra.M = M;
    ra.N = N;
    ra.V = V;
    ra.splits = plan.splits;
    ra.chunk = plan.chunk;
    ra.inv_t = noisy ? 1.0f / temperature : 0.f;
    ra.seed = seed;
    ra.step0 = step0;
    ra.pos0 = (uint64_t)pos0;
    const unsigned blocks = (unsigned)plan.items_max * plan.splits;
    if (noisy && ra.inv_t == 1.0f) {
      hipLaunchKernelGGL((commit_rows_kernel<true, kItemRows, true>), dim3(blocks), dim3(kThreads), 0, stream, ra, ws);
    } else if (noisy) {
      hipLaunchKernelGGL((commit_rows_kernel<true, kItemRows>), dim3(blocks), dim3(kThreads), 0, stream, ra, ws);
    } else {
      hipLaunchKernelGGL((commit_rows_kernel<false, 1>), dim3(blocks), dim3(kThreads), 0, stream, ra, ws);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  FinArgs fa;
  fa.logits = logits;
  fa.rows = rows;
  fa.M = M;
  fa.state = state;
  fa.next_state = next_state;
  fa.commit_pos = commit_pos;
  fa.token = token;
  fa.conf = conf;
  fa.N = N;
  fa.V = V;
  fa.splits = plan.splits;
  fa.k_max = k_max;
  fa.tau = tau;
  fa.noisy = noisy;
  hipLaunchKernelGGL(commit_finalize_kernel, dim3(tree.B1), dim3(kThreads), 0, stream, fa, ws);
  return hipGetLastError();
}

size_t commit_greedy_ws_bytes(int B1, int N, int M) { return ws_bytes(B1, N, M, 0, kGreedyChunks); }

hipError_t launch_commit_greedy(const GreedyPart* gpart, int nparts, const float* logits,
                                const int32_t* rows, int M, const int32_t* state, const TreeArgs& tree,
                                int N, int V, int k_max, float tau, int32_t* next_state, int32_t* commit_pos,
                                int32_t* token, float* conf, void* ws_base, hipStream_t stream) {
  WsLayout ws = ws_layout(ws_base, tree.B1, N, M, 0);
  if (M > 0) {
    const unsigned blocks = (unsigned)((M + kMergeRows - 1) / kMergeRows) * kGreedyChunks;
    hipLaunchKernelGGL(greedy_merge_kernel, dim3(blocks), dim3(kThreads), 0, stream, gpart, nparts, M, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  FinArgs fa;
  fa.logits = logits;
  fa.rows = rows;
  fa.M = M;
  fa.state = state;
  fa.next_state = next_state;
  fa.commit_pos = commit_pos;
  fa.token = token;
  fa.conf = conf;
  fa.N = N;
  fa.V = V;
  fa.splits = kGreedyChunks;
  fa.k_max = k_max;
  fa.tau = tau;
  fa.noisy = false;
  hipLaunchKernelGGL(commit_finalize_kernel, dim3(tree.B1), dim3(kThreads), 0, stream, fa, ws);
  return hipGetLastError();
}

hipError_t launch_gumbel_words(uint32_t first, uint32_t count, float* out, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  const uint64_t blocks = ((uint64_t)count + 255) / 256;
  hipLaunchKernelGGL(gumbel_words_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream,
                     first, count, out);
  return hipGetLastError();
}

hipError_t launch_selfcheck(double* out, hipStream_t stream) {
  hipLaunchKernelGGL(zero2_kernel, dim3(1), dim3(64), 0, stream, out);
  hipLaunchKernelGGL(selfcheck_gumbel_kernel, dim3(4096), dim3(256), 0, stream, out);
  hipLaunchKernelGGL(selfcheck_exp2_kernel, dim3(4096), dim3(256), 0, stream, out);
  return hipGetLastError();
}

}  // namespace sfv
