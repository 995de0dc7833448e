// LM head over the masked rows: logits[r][v] = <hidden[rows[r]], w[v]>,
// bf16 in, fp32 accumulate and out, on v_mfma_f32_32x32x16_bf16.
//
// SpecFold, Appendix B, keeps the LM head as a plain dense library product;
// here it is the dominant step of a one-layer verify pass: the weight is
// ~1.2 GB of bf16 and must be streamed from HBM once per pass.  Both kernels
// compute the product transposed (vocab x rows), so that each lane ends with
// 4 consecutive vocab ids of one row, and both gather the masked rows through
// `rows`.
//
// lm_head_tiled (M <= 32): 128 vocab x 128 rows x 64 k tiles, four waves of
// 64 x 64, double-buffered LDS with the next k-tile prefetched into registers.
//
// lm_head_big8 (M > 32): 256-id vocab tiles of 256 or 192 rows, eight waves,
// the next two k-tiles in flight; the row tiles of one vocab tile get
// consecutive logical ids on one XCD, so the weight tile they share is read
// from HBM once and then hit in L2.  From a few hundred rows on it is bound by
// the MFMAs; below that by streaming the weight, which it does faster than a
// kernel built for it (a weight-streaming kernel with every row in one
// workgroup and W loaded straight into MFMA operand registers served 33..160
// rows until this kernel overtook it at every row count).
//
// Every global load is unconditional: pad vocab ids and pad rows read a
// clamped, in-bounds address and the outputs they pollute are never stored.
// (A conditional load makes the compiler drain all outstanding loads, the
// prefetched stages included, before each use.)
#include "common.h"
#include "internal.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;
constexpr int BV = 128;  // vocab per tile
constexpr int BM = 128;  // rows per tile
constexpr int BK = 64;   // k per stage
constexpr int LDK = BK + 8;
constexpr int kTiledRows = 32;    // largest row count served by lm_head_tiled

struct Params {
  const unsigned short* hidden;
  const int32_t* rows;
  const unsigned short* w;
  float* logits;
  int M, D, V, R;
  int vt, mt;          // tile counts
  GreedyPart* gpart;   // large-tile kernel only: tile partials [vocab tiles][M], or null
  int big_a, big_b;    // large-tile kernel: row tiles of 256 rows, then of 192
};

__global__ __launch_bounds__(kThreads) void lm_head_tiled(Params p) {
  __shared__ unsigned short ws[2][BV][LDK];
  __shared__ unsigned short hs[2][BM][LDK];

  const int lid = xcd_logical_block(blockIdx.x, gridDim.x);
  const int mt = lid % p.mt;
  const int vt = lid / p.mt;
  const int v0 = vt * BV;
  const int m0 = mt * BM;

  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wave = t / kWave;
  const int half = lane / 32;
  const int col = lane % 32;
  const int wv = wave / 2;  // wave's vocab half of the tile
  const int wm = wave % 2;  // wave's row half of the tile

  // Each thread stages 4 chunks of 16 bytes of W and of hidden per k-tile:
  // chunk c = t + 256*i -> tile row c / 8, k part c % 8.
  // Loads are unconditional (clamped in-bounds addresses for pad vocab ids
  // and pad rows, whose outputs are never stored), so that the compiler keeps
  // the prefetch of the next k-tile in flight across the MFMAs.
  const unsigned short* wsrc[4];
  const unsigned short* hsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + kThreads * i;
    const int r = c / 8, part = c % 8;
    const int v = min(v0 + r, p.V - 1);
    wsrc[i] = p.w + (size_t)v * p.D + part * 8;
    const int m = min(m0 + r, p.M - 1);
    const int hr = min(max(p.rows[m], 0), p.R - 1);  // never leave hidden
    hsrc[i] = p.hidden + (size_t)hr * p.D + part * 8;
  }

  u32x4 wreg[4], hreg[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wreg[i] = ld16(wsrc[i] + k0);
      hreg[i] = ld16(hsrc[i] + k0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t + kThreads * i;
      const int r = c / 8, part = c % 8;
      st16(&ws[buf][r][part * 8], wreg[i]);
      st16(&hs[buf][r][part * 8], hreg[i]);
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = floatx16{};

  const int ksteps = p.D / BK;
  const int klast = (ksteps - 1) * BK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    fetch(min((ks + 1) * BK, klast));  // past the end: re-reads the last tile (L2 hit)
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      u32x4 af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = ld16(&ws[buf][wv * 64 + a * 32 + col][kk * 16 + half * 8]);
#pragma unroll
      for (int b = 0; b < 2; ++b) bfr[b] = ld16(&hs[buf][wm * 64 + b * 32 + col][kk * 16 + half * 8]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[a]), as_bf16x8(bfr[b]),
                                                               acc[a][b], 0, 0, 0);
    }
    stash(buf ^ 1);
    __syncthreads();
  }

  // lane holds vocab v0 + wv*64 + a*32 + 8*(r/4) + 4*half + r%4 of row m0 + wm*64 + b*32 + col
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = m0 + wm * 64 + b * 32 + col;
    if (m >= p.M) continue;
    float* out = p.logits + (size_t)m * p.V;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int v = v0 + wv * 64 + a * 32 + 8 * q4 + 4 * half;
        const float4 val = make_float4(acc[a][b][4 * q4], acc[a][b][4 * q4 + 1],
                                       acc[a][b][4 * q4 + 2], acc[a][b][4 * q4 + 3]);
        if (v + 3 < p.V && (p.V % 4) == 0) {
          *(float4*)(out + v) = val;
        } else {
          if (v + 0 < p.V) out[v + 0] = val.x;
          if (v + 1 < p.V) out[v + 1] = val.y;
          if (v + 2 < p.V) out[v + 2] = val.z;
          if (v + 3 < p.V) out[v + 3] = val.w;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// greedy tile partials
// ---------------------------------------------------------------------------
// Greedy partial of one row over a 32-id strip held by a lane pair: this
// lane's 16 values are ids v0 + 8 q + j (q, j < 4; the partner lane, 32
// away, holds v0 + 4 + 8 q + j).  Ids at or past V are left out.  Both lanes
// return the strip's partial:
//  * max and the lowest id attaining it (the lane's ids ascend, and the pair
//    breaks a tie of maxima toward the lower id);
//  * S = sum of fast terms exp2((x - max) log2e) in fp32 and E, a bound on
//    |S - sum exp(x - max)|: each term within kExpC1 a + kExpC2 of its value
//    (a = max - x), at most 15 roundings of a positive fp32 sum (below
//    2^-20 of it) per lane, and the pair's rescale by fast factors of the same
//    model plus 2 roundings (2^-22).
__device__ __forceinline__ GreedyPart strip_partial(const floatx16& x, int v0, int V) {
  float mx = -INFINITY;
  int ix = 0x7FFFFFFF;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = v0 + 8 * q + j;
      const float xv = v < V ? x[4 * q + j] : -INFINITY;
      if (xv > mx) {
        mx = xv;
        ix = v;
      }
    }
  float S = 0.f, A = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = v0 + 8 * q + j;
        const float am = mx - x[4 * q + j];
        const float tt = v < V ? __builtin_amdgcn_exp2f(-am * kLog2eF) : 0.f;
        S += tt;
        A += tt * am;
      }
  }
  float E = kExpC1 * A + (kExpC2 + 9.5367431640625e-07f) * S;
  const float mo = __shfl_xor(mx, 32, kWave);
  const int io = __shfl_xor(ix, 32, kWave);
  const float So = __shfl_xor(S, 32, kWave);
  const float Eo = __shfl_xor(E, 32, kWave);
  GreedyPart g;
  g.m = fmaxf(mx, mo);
  g.idx = (mo > mx || (mo == mx && io < ix)) ? io : ix;
  if (g.m == -INFINITY) {
    g.S = 0.f;
    g.E = 0.f;
    return g;
  }
  float s2 = 0.f, e2 = 0.f;
  if (mx != -INFINITY) {
    const float a = g.m - mx;
    const float f = __builtin_amdgcn_exp2f(-a * kLog2eF);
    s2 += S * f;
    e2 += E * f + S * f * (kExpC1 * a + kExpC2);
  }
  if (mo != -INFINITY) {
    const float a = g.m - mo;
    const float f = __builtin_amdgcn_exp2f(-a * kLog2eF);
    s2 += So * f;
    e2 += Eo * f + So * f * (kExpC1 * a + kExpC2);
  }
  g.S = s2;
  g.E = e2 + s2 * 2.384185791015625e-07f;
  return g;
}

// r += e for two greedy partials of one row over disjoint id ranges, e's ids
// above r's: the max, the lowest id attaining it, and the rescaled sum with
// its bound (fast factors of the same model, 3 roundings: 2^-22).
__device__ __forceinline__ void part_add(GreedyPart& r, const GreedyPart& e) {
  if (e.m == -INFINITY) return;
  if (r.m == -INFINITY) {
    r = e;
    return;
  }
  const float mx = fmaxf(r.m, e.m);
  const int idx = e.m > r.m ? e.idx : r.idx;  // a tie keeps r's (lower) id
  const float a1 = mx - r.m, a2 = mx - e.m;
  const float f1 = __builtin_amdgcn_exp2f(-a1 * kLog2eF);
  const float f2 = __builtin_amdgcn_exp2f(-a2 * kLog2eF);
  const float s = r.S * f1 + e.S * f2;
  r.E = r.E * f1 + e.E * f2 + r.S * f1 * (kExpC1 * a1 + kExpC2) + e.S * f2 * (kExpC1 * a2 + kExpC2) +
        s * 2.384185791015625e-07f;
  r.S = s;
  r.m = mx;
  r.idx = idx;
}

// ---------------------------------------------------------------------------
// large-tile kernel for many rows (the MFMA-bound regime)
// ---------------------------------------------------------------------------
// Tile 256 vocab x 256 rows x 64 k, eight waves as 2 (vocab) x 4 (rows) of
// 128 x 64, two waves per SIMD so that one wave's LDS traffic and barrier
// waits overlap the other's MFMAs; double-buffered LDS (one workgroup per CU)
// with the next two k-tiles in flight in two register sets (with one, the
// loads' latency under load outlasts a k-tile's MFMAs).  A wave reads 3/4 KB
// of LDS per MFMA (1 KB for the 64 x 64 wave tiles of lm_head_tiled).
// The waves form WV (vocab) x 8/WV (rows) groups of NA x NB 32-blocks each:
// <2, 4, 2> is 256 vocab x 256 rows (128 x 64 per wave); <4, 2, 3> is 256 x 192
// (64 x 96 per wave).  A launch mixes the two so that the rows are padded
// least (M = 384: two 192-row tiles; M = 402: one of each, 448 rows, where
// 256-row tiles alone compute 512).
constexpr int kBigV = 256, kBigRows = 256;  // LDS rows of the large-tile kernel

// The k-loop has an explicit instruction schedule: every MFMA sits in a
// fenced slot (sched_barrier) that also carries a fixed share of the other
// work.  The compiler, left to itself, read each A fragment into the same
// registers right before its MFMAs and waited on it there.  Here:
//  * A fragment q (k16 step q / NA, block q % NA) is read kSchedLA MFMA
//    groups (of NB MFMAs) before its group, into a ring of kSchedLA + 1;
//  * the next k16 step's B fragments are read kSchedGB groups before the
//    step's last group;
//  * the global loads of k-tile ks + 2 are spread over the first k16 step
//    (their register set was stored to LDS in the previous k-tile), and the
//    LDS stores of k-tile ks + 1 over the slots from step kSchedSK to the
//    k-tile's barrier (their buffer was last read before the previous one);
//  * the one barrier per k-tile comes kSchedTB groups before its end, so that
//    the next k-tile's first fragments are read while its last MFMAs run.
// The sums run in the same order as without the schedule: the logits are the
// same bit for bit.
constexpr int kSchedLA = 3;
constexpr int kSchedGB = 1;
constexpr int kSchedSK = 1;
constexpr int kSchedTB = 2;

template <int WV, int NA, int NB>
__device__ __forceinline__ void big_tile(const Params& p, int v0, int m0, unsigned short (*ws)[kBigV][LDK],
                                         unsigned short (*hs)[kBigRows][LDK]) {
  constexpr int NT = 512;
  constexpr int WM = 8 / WV;
  constexpr int TVB = WV * NA * 32, BR = WM * NB * 32;
  constexpr int CA = TVB * 8 / NT;
  constexpr int CB = BR * 8 / NT;
  constexpr int NLD = CA + CB;      // global loads (and LDS stores) per thread per k-tile
  constexpr int KK = BK / 16;       // k16 steps per k-tile
  constexpr int SL = NA * NB;       // MFMA slots per k16 step
  static_assert(TVB * 8 % NT == 0 && BR * 8 % NT == 0, "tile rows must spread evenly over the threads");
  static_assert(TVB <= kBigV && BR <= kBigRows, "tile larger than its LDS");
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wave = t / kWave;
  const int half = lane / 32;
  const int col = lane % 32;
  const int wv = wave / WM;
  const int wm = wave % WM;

  const unsigned short* wsrc[CA];
  const unsigned short* hsrc[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = t + NT * i;
    const int v = min(v0 + c / 8, p.V - 1);
    wsrc[i] = p.w + (size_t)v * p.D + (c % 8) * 8;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = t + NT * i;
    const int m = min(m0 + c / 8, p.M - 1);
    const int hr = min(max(p.rows[m], 0), p.R - 1);
    hsrc[i] = p.hidden + (size_t)hr * p.D + (c % 8) * 8;
  }
  u32x4 wreg[2][CA], hreg[2][CB];
  auto load1 = [&](int k0, int set, int i) {  // global load i of a k-tile
    if (i < CA)
      wreg[set][i] = ld16(wsrc[i] + k0);
    else
      hreg[set][i - CA] = ld16(hsrc[i - CA] + k0);
  };
  auto store1 = [&](int buf, int set, int i) {  // LDS store i of a k-tile
    if (i < CA) {
      const int c = t + NT * i;
      st16(&ws[buf][c / 8][(c % 8) * 8], wreg[set][i]);
    } else {
      const int c = t + NT * (i - CA);
      st16(&hs[buf][c / 8][(c % 8) * 8], hreg[set][i - CA]);
    }
  };
  floatx16 acc[NA][NB];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = floatx16{};

  const int ksteps = p.D / BK;
  const int klast = (ksteps - 1) * BK;
#pragma unroll
  for (int i = 0; i < NLD; ++i) load1(0, 0, i);
#pragma unroll
  for (int i = 0; i < NLD; ++i) load1(min(BK, klast), 1, i);
#pragma unroll
  for (int i = 0; i < NLD; ++i) store1(0, 0, i);
  __syncthreads();
  // A fragment q (k16 step q / NA, block q % NA) is read LA MFMA groups before
  // its group, into ring entry q % (LA + 1); the B fragments of step kk + 1
  // during step kk.  The ring runs on across k-tiles: the k-tile's one barrier
  // comes TB groups before its end, once its own fragments are all read and
  // the next k-tile's LDS stores are done, and the next k-tile's first
  // fragments are read during those last TB groups.
  constexpr int LA = kSchedLA;
  constexpr int NG = KK * NA;            // MFMA groups (of NB) per k-tile
  constexpr int TB = kSchedTB;           // groups after the barrier
  constexpr int GBAR = NG - 1 - TB;      // the barrier follows this group
  constexpr int GB = NA > kSchedGB ? NA - 1 - kSchedGB : 0;  // B read at this block of a step
  static_assert(NG % (LA + 1) == 0 && KK % 2 == 0, "the fragment ring must wrap at k-tile ends");
  static_assert(LA >= TB && LA + 1 <= NG, "own fragments read before the barrier");
  static_assert((KK - 1) * NA + GB > GBAR && (KK - 2) * NA + GB <= GBAR, "B fragments on their side of the barrier");
  constexpr int SW = (GBAR - kSchedSK * NA + 1) * NB;  // store slots, step kSchedSK .. the barrier
  static_assert(SW >= NLD, "a slot for every LDS store");
  u32x4 fa[LA + 1], fb[2][NB];
  auto rdA = [&](int buf, int kk, int a) { return ld16(&ws[buf][wv * NA * 32 + a * 32 + col][kk * 16 + half * 8]); };
  auto rdB = [&](int buf, int kk, int b) { return ld16(&hs[buf][wm * NB * 32 + b * 32 + col][kk * 16 + half * 8]); };
#pragma unroll
  for (int b = 0; b < NB; ++b) fb[0][b] = rdB(0, 0, b);
#pragma unroll
  for (int q = 0; q < LA; ++q) fa[q] = rdA(0, q / NA, q % NA);
  __builtin_amdgcn_sched_barrier(0);
  for (int ks0 = 0; ks0 < ksteps; ks0 += 4) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int ks = ks0 + jj;
      if (ks >= ksteps) break;
      const int buf = jj & 1;
      const int knext2 = min((ks + 2) * BK, klast);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int bs = kk & 1;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          const int g = kk * NA + a;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const int slot = a * NB + b;  // within this k16 step
            if (b == 0) {
              // this k-tile's fragment g + LA, or the next k-tile's first ones
              if (g + LA < NG) fa[(g + LA) % (LA + 1)] = rdA(buf, (g + LA) / NA, (g + LA) % NA);
#pragma unroll
              for (int q = 0; q < LA; ++q)
                if (g == (GBAR + 1 > NG - LA + q ? GBAR + 1 : NG - LA + q)) fa[q] = rdA(buf ^ 1, q / NA, q % NA);
            }
            if (a == GB) fb[bs ^ 1][b] = kk + 1 < KK ? rdB(buf, kk + 1, b) : rdB(buf ^ 1, 0, b);
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[g % (LA + 1)]), as_bf16x8(fb[bs][b]),
                                                                acc[a][b], 0, 0, 0);
            // k-tile ks + 2's global loads over the first step, k-tile ks + 1's
            // LDS stores over the slots from step kSchedSK to the barrier
            if (kk == 0) {
#pragma unroll
              for (int i = 0; i < NLD; ++i)
                if (i * SL / NLD == slot) load1(knext2, buf, i);
            }
            if (g >= kSchedSK * NA && g <= GBAR) {
              const int s = (g - kSchedSK * NA) * NB + b;
#pragma unroll
              for (int i = 0; i < NLD; ++i)
                if (i * SW / NLD == s) store1(buf ^ 1, buf ^ 1, i);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (g == GBAR && b == NB - 1) {
              __syncthreads();
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
    }
  }
  __syncthreads();  // the last k-tile's reads of the (unused) next buffer are done
  if (p.gpart) {
    // Greedy partial of every row over this 256-id vocab tile: a wave merges
    // its NA strips in id order, then the WV vocab groups are merged in id
    // order through LDS (past the k-loop's last barrier nothing reads the
    // weight tiles).
    GreedyPart* gx = reinterpret_cast<GreedyPart*>(&ws[0][0][0]);  // [WV][BR]
    static_assert(WV * BR * sizeof(GreedyPart) <= sizeof(unsigned short) * kBigV * LDK, "LDS for partials");
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int vw = v0 + wv * NA * 32 + 4 * half;
      GreedyPart r = strip_partial(acc[0][b], vw, p.V);
#pragma unroll
      for (int a = 1; a < NA; ++a) part_add(r, strip_partial(acc[a][b], vw + a * 32, p.V));
      if (half == 0) gx[wv * BR + wm * NB * 32 + b * 32 + col] = r;
    }
    __syncthreads();
    if (t < BR && m0 + t < p.M) {
      GreedyPart r = gx[t];
      for (int w = 1; w < WV; ++w) part_add(r, gx[w * BR + t]);
      p.gpart[(size_t)(v0 / kBigV) * p.M + m0 + t] = r;
    }
  }

  // Lane (col, half) holds vocab v0 + wv*NA*32 + a*32 + 8*(r/4) + 4*half + r%4
  // of row m0 + wm*NB*32 + b*32 + col: stored straight from the registers, a
  // store instruction would write 32 rows x 32 bytes.  Instead each wave
  // stages a 32-row block of its tile in its own slice of the k-loop's LDS
  // (rows of NA * 32 floats plus 4 of padding) and reads it back so that
  // consecutive lanes hold consecutive ids of one row: every store
  // instruction then writes whole 128-byte lines.
  {
    if (p.gpart) __syncthreads();  // the partials' LDS has been read
    constexpr int TW = NA * 32;       // ids per wave row
    constexpr int SROW = TW + 4;      // staged row stride (floats)
    constexpr int C4 = TW / 4;        // float4 per row
    static_assert(4 * 32 * SROW * 4 <= (int)sizeof(unsigned short) * 2 * kBigV * LDK, "LDS for staging");
    // (the thread index passes through an empty asm statement here, so that
    // nothing derived from it is computed before the k-loop, where every
    // register is taken)
    int tt = t;
    asm volatile("" : "+v"(tt));
    const int lane = tt % kWave, wave = tt / kWave, half = lane / 32, col = lane % 32;
    // waves 0-3 stage in the weight buffers, 4-7 in the hidden ones
    float* st = reinterpret_cast<float*>(wave < 4 ? &ws[0][0][0] : &hs[0][0][0]) + (wave % 4) * 32 * SROW;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(floatx4*)&st[col * SROW + a * 32 + 8 * q4 + 4 * half] =
              floatx4{acc[a][b][4 * q4], acc[a][b][4 * q4 + 1], acc[a][b][4 * q4 + 2], acc[a][b][4 * q4 + 3]};
#pragma unroll
      for (int i = 0; i < 32 * C4 / kWave; ++i) {
        const int c = lane + kWave * i;
        const int row = c / C4, f = (c % C4) * 4;
        const floatx4 val = *(const floatx4*)&st[row * SROW + f];
        const int m = m0 + wm * NB * 32 + b * 32 + row;
        const int v = v0 + wv * NA * 32 + f;
        if (m >= p.M) continue;
        float* out = p.logits + (size_t)m * p.V;
        if (v + 3 < p.V && (p.V % 4) == 0) {
          *(floatx4*)(out + v) = val;
        } else {
          if (v + 0 < p.V) out[v + 0] = val[0];
          if (v + 1 < p.V) out[v + 1] = val[1];
          if (v + 2 < p.V) out[v + 2] = val[2];
          if (v + 3 < p.V) out[v + 3] = val[3];
        }
      }
    }
  }
}

// One launch covers the rows with big_a tiles of 256 rows and then big_b of
// 192; the row tiles of one vocab tile get consecutive logical ids on one XCD.
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void lm_head_big8(Params p) {
  __shared__ __attribute__((aligned(16))) unsigned short ws[2][kBigV][LDK];
  __shared__ __attribute__((aligned(16))) unsigned short hs[2][kBigRows][LDK];
  const int mtiles = p.big_a + p.big_b;
  const int lid = xcd_logical_block(blockIdx.x, gridDim.x);
  const int mt = lid % mtiles;
  const int v0 = (lid / mtiles) * kBigV;
  if (mt < p.big_a) {
    big_tile<2, 4, 2>(p, v0, mt * 256, ws, hs);
  } else {
    big_tile<4, 2, 3>(p, v0, p.big_a * 256 + (mt - p.big_a) * 192, ws, hs);
  }
}

hipError_t launch_big8(const Params& p0, hipStream_t stream) {
  // a tiles of 256 rows and b of 192 covering M with the fewest padded rows
  // (ties: more 256-row tiles, whose waves read less LDS per MFMA)
  Params p = p0;
  int best_a = (p.M + 255) / 256, best_b = 0, best_pad = best_a * 256 - p.M;
  for (int a = best_a - 1; a >= 0; --a) {
    const int b = (p.M - 256 * a + 191) / 192;
    const int pad = 256 * a + 192 * b - p.M;
    if (pad < best_pad) {
      best_a = a;
      best_b = b;
      best_pad = pad;
    }
  }
  p.big_a = best_a;
  p.big_b = best_b;
  const int vt = (p.V + kBigV - 1) / kBigV;
  hipLaunchKernelGGL(lm_head_big8, dim3(vt * (best_a + best_b)), dim3(512), 0, stream, p);
  return hipGetLastError();
}

// One workgroup checks every row id: *status = -1 (SFV_E_INVAL) when some
// id is outside [0, R), else 0.
__global__ __launch_bounds__(256) void rows_status_kernel(const int32_t* rows, int M, int R, int32_t* status) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int mine = 0;
  for (int m = threadIdx.x; m < M; m += 256) {
    const int r = rows[m];
    mine |= (r < 0 || r >= R);
  }
  if (__any(mine) && threadIdx.x % kWave == 0) bad = 1;  // (racing writes of the same value)
  __syncthreads();
  if (threadIdx.x == 0) *status = bad ? -1 : 0;
}

hipError_t launch_tiled(const Params& p, hipStream_t stream) {
  hipLaunchKernelGGL(lm_head_tiled, dim3(p.vt * p.mt), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rows_status(const int32_t* rows, int M, int R, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(rows_status_kernel, dim3(1), dim3(256), 0, stream, rows, M, R, status);
  return hipGetLastError();
}

hipError_t launch_lm_head(const void* hidden, const int32_t* rows, int M, int R, const void* w,
                          int D, int V, float* logits, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  Params p;
  p.hidden = (const unsigned short*)hidden;
  p.rows = rows;
  p.w = (const unsigned short*)w;
  p.logits = logits;
  p.M = M;
  p.D = D;
  p.V = V;
  p.R = R;
  p.vt = (V + BV - 1) / BV;
  p.mt = (M + BM - 1) / BM;
  p.gpart = nullptr;
  p.big_a = p.big_b = 0;
  // Up to 32 rows: the tiled kernel.  More: the large-tile kernel (from 33
  // rows on it beats the tiled kernel, whose row tile re-reads the hidden
  // rows with one k-tile in flight).
  if (M <= kTiledRows) return launch_tiled(p, stream);
  return launch_big8(p, stream);
}

// From 33 rows on, the LM head (the large-tile kernel) writes one greedy
// partial per row and 256-id vocab tile beside the logits.
int lm_head_greedy_parts(int M, int V, int D) {
  if (M <= kTiledRows || D % 64 != 0 || V < 1) return 0;
  return (V + kBigV - 1) / kBigV;
}

hipError_t launch_lm_head_greedy(const void* hidden, const int32_t* rows, int M, int R, const void* w,
                                 int D, int V, float* logits, GreedyPart* gpart, hipStream_t stream) {
  if (lm_head_greedy_parts(M, V, D) == 0 || gpart == nullptr) return hipErrorInvalidValue;
  Params p;
  p.hidden = (const unsigned short*)hidden;
  p.rows = rows;
  p.w = (const unsigned short*)w;
  p.logits = logits;
  p.M = M;
  p.D = D;
  p.V = V;
  p.R = R;
  p.vt = (V + BV - 1) / BV;
  p.mt = (M + BM - 1) / BM;
  p.gpart = gpart;
  p.big_a = p.big_b = 0;
  return launch_big8(p, stream);
}

}  // namespace sfv
