// Shared-prefix attention of every branch (bf16 in, fp32 accumulate, MFMA).
//
// SpecFold ("Folding Multi-Branch Redundancy ..."), introduction and App. A.1:
// every block position of a branch attends, bidirectionally, to the shared
// context keys and to all of its own block keys, and the streaming-softmax
// state (m, Z, O) over [context | block] gives the output.  The pages' kernel
// (a FlashAttention-style Triton kernel over a zero-copy view of the prefix,
// Sec. 3.3 and App. B) is prior art; this is the gfx950 design:
//
//  * All B1*N*G query rows of one kv head form one matrix (branch-major), so
//    a workgroup of 128 rows streams each context K/V tile once from HBM for
//    up to 128 rows of several branches; the context is read once per row
//    tile, not once per branch.
//  * Scores are computed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16,
//    so each lane owns one query row (lane % 32): the online max/sum and the
//    rescale of O are lane-local, and the P tile feeds O^T = V^T P^T straight
//    from the score registers (V is staged transposed in LDS).
//  * The block phase concatenates the block keys of the branches present in
//    the tile; a key is visible to a row only if both belong to one branch.
//  * Long contexts are split into key ranges (split-KV) whose (m, l, O)
//    states are merged by log-sum-exp in a second kernel.
//  * With `causal`, a row sees the block keys of its branch only up to its
//    own position (an autoregressive target verifying drafted trays, each
//    tray a branch continuing the shared context).
//  * Folded verification (SpecFold App. A.1 and B) runs the same kernel in
//    two more modes.  kCtx: only the compacted recomputed slots, against the
//    context keys alone, leaving their (m, l, O) states in the workspace
//    (workgroups past the live row count exit at once).  kBlock: every slot,
//    with its resolved query (the source branch's at that position), against
//    its own branch's block keys read through the slots' resolved sources;
//    the epilogue merges in the context state of the slot's source row.  A
//    folded slot's query equals its source's, and the context is shared, so
//    the source's context state is exactly the folded row's: folded rows
//    skip the context and nothing is subtracted.
#include "common.h"
#include "internal.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kRows = 128;     // query rows per workgroup, 32 per wave
constexpr int kKeys = 64;      // keys per LDS tile
constexpr int kPad = 8;        // bf16 elements of row padding of the key tiles in LDS
constexpr int kSlots = 512;    // workgroups resident at once: two per CU, 256 CUs
// Row padding of the transposed value tiles: a row is 34 dwords, so the
// 8-byte reads of 32 consecutive rows (one per lane) fall on 32 distinct bank
// pairs; with 36 dwords they met in pairs (two-way bank conflicts).
constexpr int kVPad = 4;
// The pipelined context pass keeps the softmax reference max until a row's
// scores exceed it by more than this (log2 units): P <= 2^8, well inside the
// range of bf16 and fp32, and the D / 2 rescale multiplies per lane (D / 32
// accumulator blocks of 16) run only on such a jump, not on every tile where
// some row's max moved.
constexpr float kLazyLog2 = 8.f;

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Hardware exp2 (v_exp_f32).  Results below 2^-126 may flush to zero; such
// terms are below 2^-126 of the row's largest term.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

struct Params {
  const unsigned short* q;
  const unsigned short* k_blk;
  const unsigned short* v_blk;
  const unsigned short* k_ctx;
  const unsigned short* v_ctx;
  unsigned short* o;
  float* lse;
  float* ws;  // split partials: O [splits][Hkv][rows][d], m, l [splits][Hkv][rows]
  const int32_t* qrows;  // folded path: recomputed slots i*N+n, in order
  const int32_t* src;    // folded path: resolved source branch of every slot [B1][N]
  const int32_t* count;  // folded path: number of recomputed slots (device)
  const int32_t* rec_pos;  // folded path: index of each recomputed slot in qrows [B1][N]
  int B1, N, L, Hq, Hkv, G;
  int rows_total, row_tiles, splits, chunk;
  int tile0, tiles;       // this launch's row tiles: tile0 .. tile0 + tiles - 1
  int ws_row0, ws_rows;   // split states cover rows ws_row0 .. ws_row0 + ws_rows - 1
  float scale_log2;  // softmax scale * log2(e), applied inside the exp2
  bool causal;       // block keys visible only up to the row's own position
};

template <int D>
struct Smem {
  unsigned short k[2][kKeys][D + kPad];   // key tiles, row-major (double buffered)
  unsigned short vt[2][D][kKeys + kVPad];  // value tiles, transposed
};

// Which keys tile j of this workgroup covers: the context tiles of its split,
// then (last split only) the block keys of the branches in its row tile.
struct TileRange {
  bool ctx;
  int key0, count;
};

__device__ __forceinline__ TileRange tile_range(const Params& p, int j, int split, int ctx_tiles,
                                                int blk_keys) {
  TileRange tr;
  if (j < ctx_tiles) {
    tr.ctx = true;
    tr.key0 = split * p.chunk + j * kKeys;
    tr.count = min(kKeys, min(p.L, (split + 1) * p.chunk) - tr.key0);
  } else {
    tr.ctx = false;
    tr.key0 = (j - ctx_tiles) * kKeys;
    tr.count = min(kKeys, blk_keys - tr.key0);
  }
  return tr;
}

enum Mode { kDense = 0, kCtx = 1, kBlock = 2 };

__device__ __forceinline__ int rec_count(const Params& p) { return min(max(*p.count, 0), p.B1 * p.N); }

// Query rows live in this launch: every row, or G per recomputed slot.
template <int MODE>
__device__ __forceinline__ int live_rows(const Params& p) {
  if (MODE != kCtx) return p.rows_total;
  return rec_count(p) * p.G;
}

// Slot (i*N + n) of query row r (r < live rows).
template <int MODE>
__device__ __forceinline__ int slot_of(const Params& p, int r) {
  if (MODE != kCtx) return r / p.G;
  return min(max(p.qrows[r / p.G], 0), p.B1 * p.N - 1);
}

// Resolved source slot of `slot`: the slot whose q/k/v it holds.
__device__ __forceinline__ int source_slot(const Params& p, int slot) {
  const int sb = min(max(p.src[slot], 0), p.B1 - 1);
  return sb * p.N + slot % p.N;
}

// Row of k_blk / v_blk holding block key `key` (0-based over the branches
// i_lo, i_lo+1, ...): the branch's own row, or on the folded path the row of
// the slot's resolved source branch.
template <bool FOLD>
__device__ __forceinline__ size_t block_key_row(const Params& p, int i_lo, int key) {
  const int slot = i_lo * p.N + key;
  if (!FOLD) return (size_t)slot;
  return (size_t)source_slot(p, slot);
}

// Registers holding one K/V tile between its global loads and its LDS stores.
// K: chunk c = t + 256*i (i < D/32) is key c / (D/8), dims (c % (D/8)) * 8.
// V: thread t < 2*D takes keys 4*(t%16) .. +4 and dims 8*(t/16) .. +8, so that
// its transposed stores (4 keys of one dim, 8 bytes) from 16 consecutive
// lanes fill one 128-byte LDS row segment.
template <int D>
struct TileRegs {
  u32x4 k[D / 32];
  u32x4 v[4];
};

// Loads are unconditional: rows past `count` re-read the tile's last key
// (their scores are masked to -inf and their probabilities are 0).
template <int D, bool FOLD>
__device__ __forceinline__ void tile_load(TileRegs<D>& tr, const Params& p, const TileRange& r, int g,
                                          int i_lo) {
  const int t = threadIdx.x;
  constexpr int parts = D / 8;
  const int last = r.count - 1;
  if (FOLD && !r.ctx) {  // block keys through the slots' resolved sources
    const size_t stride = (size_t)p.Hkv * D;
    const unsigned short* kb = p.k_blk + (size_t)g * D;
    const unsigned short* vb = p.v_blk + (size_t)g * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int c = t + kThreads * i;
      const size_t row = block_key_row<true>(p, i_lo, r.key0 + min(c / parts, last));
      tr.k[i] = ld16(kb + row * stride + (c % parts) * 8);
    }
    if (t < 2 * D) {
      const int kg = t % 16, dg = t / 16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t row = block_key_row<true>(p, i_lo, r.key0 + min(kg * 4 + q, last));
        tr.v[q] = ld16(vb + row * stride + dg * 8);
      }
    }
    return;
  }
  // The context rows are D elements apart (a compile-time stride, so the
  // per-tile addresses are a uniform base plus shifts); block rows Hkv * D.
  if (r.ctx) {
    const size_t tile0 = ((size_t)g * p.L + r.key0) * D;  // uniform
    const unsigned short* kbase = p.k_ctx + tile0;
    const unsigned short* vbase = p.v_ctx + tile0;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int c = t + kThreads * i;
      const int key = min(c / parts, last);
      tr.k[i] = ld16(kbase + key * D + (c % parts) * 8);
    }
    if (t < 2 * D) {
      const int kg = t % 16, dg = t / 16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int key = min(kg * 4 + q, last);
        tr.v[q] = ld16(vbase + key * D + dg * 8);
      }
    }
    return;
  }
  const int stride = p.Hkv * D;
  const size_t tile0 = (((size_t)i_lo * p.N + r.key0) * p.Hkv + g) * D;
  const unsigned short* kbase = p.k_blk + tile0;
  const unsigned short* vbase = p.v_blk + tile0;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int c = t + kThreads * i;
    const int key = min(c / parts, last);
    tr.k[i] = ld16(kbase + (size_t)key * stride + (c % parts) * 8);
  }
  if (t < 2 * D) {
    const int kg = t % 16, dg = t / 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int key = min(kg * 4 + q, last);
      tr.v[q] = ld16(vbase + (size_t)key * stride + dg * 8);
    }
  }
}

template <int D>
__device__ __forceinline__ void tile_store(Smem<D>& sm, int buf, const TileRegs<D>& tr) {
  const int t = threadIdx.x;
  constexpr int parts = D / 8;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int c = t + kThreads * i;
    st16(&sm.k[buf][c / parts][(c % parts) * 8], tr.k[i]);
  }
  if (t < 2 * D) {
    const int kg = t % 16, dg = t / 16;
    // 4 keys x 8 dims -> for each dim e, the 4 keys as two bf16 pairs
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e / 2;
      const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of two words
      uint2 out;
      out.x = __builtin_amdgcn_perm(tr.v[1][w], tr.v[0][w], sel);
      out.y = __builtin_amdgcn_perm(tr.v[3][w], tr.v[2][w], sel);
      *(uint2*)(&sm.vt[buf][dg * 8 + e][kg * 4]) = out;
    }
  }
}

// Software-pipelined pass over the full context tiles 0 .. nf - 1 (nf >= 2)
// of a workgroup's key range.  Step j computes the scores of tile j + 1 on
// the matrix cores while the softmax of tile j runs on the vector ALUs, then
// tile j's P V^T.  K is staged two tiles ahead and V one, in the same two
// LDS buffers as the generic loop: step j reads K buffer (j + 1) & 1 and V
// buffer j & 1, and stores K of tile j + 2 into K buffer j & 1 and V of tile
// j + 1 into V buffer (j + 1) & 1, each last read in step j - 1 (one barrier
// per step).  The scores, products and sums are the generic loop's, in its
// order; only the softmax reference max moves lazily (kLazyLog2).
//
// A full context tile is kKeys * D contiguous elements: thread t's K chunks
// sit at byte t * 16 + 4096 * i of it and its V rows at a fixed offset, so
// the loads are a uniform tile base plus fixed 32-bit lane offsets.
template <int D>
__device__ __forceinline__ void ctx_load_k(TileRegs<D>& tr, const unsigned short* tile, unsigned klane) {
  const char* b = reinterpret_cast<const char*>(tile);
#pragma unroll
  for (int i = 0; i < D / 32; ++i) tr.k[i] = ld16(b + (size_t)(klane + 4096u * i));
}

template <int D>
__device__ __forceinline__ void ctx_load_v(TileRegs<D>& tr, const unsigned short* tile, unsigned vlane) {
  if (2 * D >= kThreads || threadIdx.x < 2 * D) {
    const char* b = reinterpret_cast<const char*>(tile);
#pragma unroll
    for (int q = 0; q < 4; ++q) tr.v[q] = ld16(b + (size_t)(vlane + 2u * D * q));
  }
}

template <int D>
__device__ __forceinline__ void store_k(Smem<D>& sm, int buf, const TileRegs<D>& tr) {
  const int t = threadIdx.x;
  constexpr int parts = D / 8;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int c = t + kThreads * i;
    st16(&sm.k[buf][c / parts][(c % parts) * 8], tr.k[i]);
  }
}

template <int D>
__device__ __forceinline__ void store_v(Smem<D>& sm, int buf, const TileRegs<D>& tr) {
  const int t = threadIdx.x;
  if (2 * D >= kThreads || t < 2 * D) {
    const int kg = t % 16, dg = t / 16;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e / 2;
      const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint2 out;
      out.x = __builtin_amdgcn_perm(tr.v[1][w], tr.v[0][w], sel);
      out.y = __builtin_amdgcn_perm(tr.v[3][w], tr.v[2][w], sel);
      *(uint2*)(&sm.vt[buf][dg * 8 + e][kg * 4]) = out;
    }
  }
}

// S^T of one key tile: 2 blocks of 32 keys x 32 rows, each summed over the
// head dim in order s = 0, 1, ...  With AHEAD > 0 the key fragment of MFMA i
// is read before MFMA i - AHEAD is issued; the fences order only LDS reads
// and MFMAs, so vector ALU work (the softmax of the previous tile) is still
// scheduled in between.
template <int D, int AHEAD = 0>
__device__ __forceinline__ void tile_scores(floatx16 (&st)[2], const Smem<D>& sm, int buf,
                                            const u32x4 (&qf)[D / 16], int col, int half) {
  constexpr int n = 2 * (D / 16);  // MFMAs: (s, kb) for s < D / 16, kb < 2
  auto kread = [&](int i) { return ld16(&sm.k[buf][(i % 2) * 32 + col][(i / 2) * 16 + half * 8]); };
  st[0] = floatx16{};
  st[1] = floatx16{};
  if (AHEAD == 0) {
#pragma unroll
    for (int i = 0; i < n; ++i)
      st[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kread(i)), as_bf16x8(qf[i / 2]), st[i % 2], 0,
                                                          0, 0);
    return;
  }
  constexpr int kAluMayCross = 0x0002 | 0x0004 | 0x0400;  // VALU, SALU, transcendental
  u32x4 kf[n];
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) kf[i] = kread(i);
  __builtin_amdgcn_sched_barrier(kAluMayCross);
#pragma unroll
  for (int i = 0; i < n; ++i) {
    if (i + AHEAD < n) kf[i + AHEAD] = kread(i + AHEAD);
    st[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[i]), as_bf16x8(qf[i / 2]), st[i % 2], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(kAluMayCross);
  }
}

// O^T += V^T P^T over one key tile (A = V^T rows, B = P^T), in the order
// (kb, t2, b).  With AHEAD > 0 the value fragment of MFMA i is read before
// MFMA i - AHEAD is issued (scheduling fences keep that order, so several
// LDS reads are in flight while the matrix cores run).
template <int D, int AHEAD = 0>
__device__ __forceinline__ void tile_pv(floatx16 (&acc)[D / 32], const Smem<D>& sm, int buf,
                                        const unsigned (&pk)[2][2][4], int col, int half) {
  constexpr int DB = D / 32;
  constexpr int n = 4 * DB;  // MFMAs of the tile
  auto vread = [&](int i) {
    const int kb = i / (2 * DB), t2 = (i / DB) % 2, b = i % DB;
    const int kbase = kb * 32 + 16 * t2 + 4 * half;
    const uint2 lo = *(const uint2*)(&sm.vt[buf][b * 32 + col][kbase]);
    const uint2 hi = *(const uint2*)(&sm.vt[buf][b * 32 + col][kbase + 8]);
    u32x4 vf;
    vf[0] = lo.x;
    vf[1] = lo.y;
    vf[2] = hi.x;
    vf[3] = hi.y;
    return vf;
  };
  auto mfma = [&](int i, const u32x4& vf) {
    const int kb = i / (2 * DB), t2 = (i / DB) % 2, b = i % DB;
    u32x4 pb;
    pb[0] = pk[kb][t2][0];
    pb[1] = pk[kb][t2][1];
    pb[2] = pk[kb][t2][2];
    pb[3] = pk[kb][t2][3];
    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pb), acc[b], 0, 0, 0);
  };
  if (AHEAD == 0) {
#pragma unroll
    for (int i = 0; i < n; ++i) mfma(i, vread(i));
    return;
  }
  u32x4 vf[n];
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) vf[i] = vread(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < n; ++i) {
    if (i + AHEAD < n) vf[i + AHEAD] = vread(i + AHEAD);
    mfma(i, vf[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One pipelined step (tile j, parity PAR = j & 1); NEXT: tile j + 1 exists.
template <int D, bool NEXT, int PAR>
__device__ __forceinline__ void ctx_step(Smem<D>& sm, const unsigned short* kbase, const unsigned short* vbase,
                                         unsigned klane, unsigned vlane, int j, int nf, float scale_log2,
                                         const u32x4 (&qf)[D / 16], floatx16 (&cur)[2], floatx16 (&nxt)[2],
                                         floatx16 (&acc)[D / 32], float& m_run, float& l_run, int col,
                                         int half) {
  constexpr size_t tile_elems = (size_t)kKeys * D;
  TileRegs<D> tr;
  const bool k2 = j + 2 < nf;
  if (k2) ctx_load_k<D>(tr, kbase + (size_t)(j + 2) * tile_elems, klane);
  if (NEXT) ctx_load_v<D>(tr, vbase + (size_t)(j + 1) * tile_elems, vlane);

  // Softmax of tile j (no key is masked in a full context tile), in pieces:
  // the running max over 8 scores at a time, then the max of the two
  // half-waves, then the exponentials a pair of scores at a time.  The order
  // of every sum and max is that of the generic loop.
  float tmax = -INFINITY;
  float m_new = 0.f, alpha = 1.f, mc = 0.f;
  bool moved = false;
  float psum = 0.f;
  unsigned pk[2][2][4];
  auto max_piece = [&](int q) {
#pragma unroll
    for (int i = 8 * q; i < 8 * q + 8; ++i) tmax = fmaxf(tmax, cur[i / 16][i % 16]);
  };
  auto finish_max = [&]() {
    // the other half-wave's max (lane ^ 32) by a lane swap, not through LDS:
    // the swap returns the low half's value in [0] and the high half's in [1]
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
    tmax = fmaxf(tmax, __uint_as_float(half ? sw[0] : sw[1]));
    // Lazy rescaling: the exponentials stay relative to the reference max
    // m_run until some row's tile max exceeds it by more than kLazyLog2 (in
    // log2 units), so P <= 2^kLazyLog2 and O and l hold their rescale; the
    // reference then moves to the new max.
    const bool far = (tmax - m_run) * scale_log2 > kLazyLog2 || m_run == -INFINITY;
    m_new = __any(far) ? fmaxf(m_run, tmax) : m_run;
    moved = m_new > m_run;
    alpha = moved ? exp2_fast((m_run - m_new) * scale_log2) : 1.f;
    mc = m_new == -INFINITY ? 0.f : m_new * scale_log2;
  };
  auto exp_pair = [&](int pidx) {  // scores 2 * pidx, 2 * pidx + 1 of block kb
    const int kb = pidx / 8, r = (pidx % 8) * 2;
    floatx2 pp;
    pp[0] = exp2_fast(fmaf(cur[kb][r], scale_log2, -mc));
    pp[1] = exp2_fast(fmaf(cur[kb][r + 1], scale_log2, -mc));
    psum += pp[0] + pp[1];
    pk[kb][r / 8][(r % 8) / 2] = __builtin_bit_cast(unsigned, __builtin_convertvector(pp, bf16x2));
  };
  if (NEXT) {
    // The scores of tile j + 1 (n MFMAs, key fragments read two ahead), with
    // the softmax of tile j dealt over them: the max in the first two MFMA
    // slots, the 16 exponential pairs over the others.  Fences keep each
    // slot's work in its slot.
    constexpr int n = 2 * (D / 16);
    constexpr int AH = 2;
    const int nb = PAR ^ 1;
    auto kread = [&](int i) { return ld16(&sm.k[nb][(i % 2) * 32 + col][(i / 2) * 16 + half * 8]); };
    nxt[0] = floatx16{};
    nxt[1] = floatx16{};
    u32x4 kf[n];
#pragma unroll
    for (int i = 0; i < AH; ++i) kf[i] = kread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < n; ++i) {
      if (i + AH < n) kf[i + AH] = kread(i + AH);
      nxt[i % 2] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[i]), as_bf16x8(qf[i / 2]), nxt[i % 2], 0, 0, 0);
      if (i == 0) {
        max_piece(0);
        max_piece(1);
      } else if (i == 1) {
        max_piece(2);
        max_piece(3);
        finish_max();
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (2 + q * (n - 2) / 16 == i) exp_pair(q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) max_piece(q);
    finish_max();
#pragma unroll
    for (int q = 0; q < 16; ++q) exp_pair(q);
  }
  // Pin P here, beside the scores of tile j + 1, rather than letting the
  // compiler sink its exponentials past the rescale branch (an empty asm
  // statement that only names the registers; it emits no instruction).
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
      asm volatile("" : "+v"(pk[kb][t2][0]), "+v"(pk[kb][t2][1]), "+v"(pk[kb][t2][2]), "+v"(pk[kb][t2][3]));
  asm volatile("" : "+v"(psum));
  // O and l are rescaled only when some lane's running max moved.
  if (__any(moved)) {
    l_run *= alpha;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
  }
  m_run = m_new;
  l_run += psum;
  tile_pv<D, 3>(acc, sm, PAR, pk, col, half);
  if (k2) store_k<D>(sm, PAR, tr);
  if (NEXT) store_v<D>(sm, PAR ^ 1, tr);
  __syncthreads();
}

template <int D>
__device__ __forceinline__ void ctx_pipelined(Smem<D>& sm, const Params& p, int g, int key0, int nf,
                                              const u32x4 (&qf)[D / 16], floatx16 (&acc)[D / 32],
                                              float& m_run, float& l_run, int col, int half) {
  const int t = threadIdx.x;
  const size_t base = ((size_t)g * p.L + key0) * D;
  const unsigned short* kbase = p.k_ctx + base;
  const unsigned short* vbase = p.v_ctx + base;
  const unsigned klane = 16u * t;
  const unsigned vlane = 2u * ((4u * (t % 16)) * D + 8u * (t / 16));
  constexpr size_t tile_elems = (size_t)kKeys * D;
  {
    TileRegs<D> tr;
    ctx_load_k<D>(tr, kbase, klane);
    ctx_load_v<D>(tr, vbase, vlane);
    store_k<D>(sm, 0, tr);
    store_v<D>(sm, 0, tr);
    ctx_load_k<D>(tr, kbase + tile_elems, klane);
    store_k<D>(sm, 1, tr);
  }
  __syncthreads();
  floatx16 sa[2], sb[2];
  tile_scores<D>(sa, sm, 0, qf, col, half);
  int j = 0;
  for (; j + 2 < nf; j += 2) {
    ctx_step<D, true, 0>(sm, kbase, vbase, klane, vlane, j, nf, p.scale_log2, qf, sa, sb, acc, m_run, l_run, col, half);
    ctx_step<D, true, 1>(sm, kbase, vbase, klane, vlane, j + 1, nf, p.scale_log2, qf, sb, sa, acc, m_run, l_run, col,
                         half);
  }
  if (j + 1 < nf) {
    ctx_step<D, true, 0>(sm, kbase, vbase, klane, vlane, j, nf, p.scale_log2, qf, sa, sb, acc, m_run, l_run, col, half);
    ctx_step<D, false, 1>(sm, kbase, vbase, klane, vlane, j + 1, nf, p.scale_log2, qf, sb, sa, acc, m_run, l_run, col,
                          half);
  } else {
    ctx_step<D, false, 0>(sm, kbase, vbase, klane, vlane, j, nf, p.scale_log2, qf, sa, sb, acc, m_run, l_run, col,
                          half);
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_kernel(Params p) {
  __shared__ Smem<D> sm;
  constexpr int DS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DB = D / 32;  // 32-wide output blocks of the head dim

  const int total = gridDim.x;
  const int lid = xcd_logical_block(blockIdx.x, total);
  const int tile = p.tile0 + lid % p.tiles;
  const int gs = lid / p.tiles;
  const int nsplit = MODE == kBlock ? 1 : p.splits;  // the block pass has no context splits
  const int split = gs % nsplit;
  const int g = gs / nsplit;

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int half = lane / 32;
  const int col = lane % 32;

  const int row0 = tile * kRows;
  const int rows_live = live_rows<MODE>(p);
  if (MODE == kCtx && row0 >= rows_live) return;  // whole workgroup: no barrier reached yet
  const int rho = row0 + wave * 32 + col;  // this lane's query row
  const bool row_ok = rho < rows_live;
  const int rq = min(rho, rows_live - 1);
  const int bn_q = slot_of<MODE>(p, rq);
  const int my_branch = row_ok ? bn_q / p.N : -1;

  // Q fragment of this lane's row: dims s*16 + half*8 .. +8 for each step s
  u32x4 qf[DS];
  {
    const int j = rq % p.G;
    const int qslot = MODE == kBlock ? source_slot(p, bn_q) : bn_q;
    const size_t qoff = ((size_t)qslot * p.Hq + (size_t)g * p.G + j) * D;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = ld16(p.q + qoff + s * 16 + half * 8);
  }

  floatx16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = floatx16{};
  float m_run = -INFINITY;  // running max of the raw scores q.k
  float l_run = 0.f;        // running denominator (scaled to m_run), this half's keys only

  const int last_row = min(row0 + kRows, rows_live) - 1;
  const int i_lo = slot_of<MODE>(p, row0) / p.N;
  const int i_hi = slot_of<MODE>(p, last_row) / p.N;
  const int ctx_lo = split * p.chunk;
  const int ctx_keys = MODE == kBlock ? 0 : max(0, min(p.L, ctx_lo + p.chunk) - ctx_lo);
  const int ctx_tiles = (ctx_keys + kKeys - 1) / kKeys;
  const int blk_keys = MODE == kCtx ? 0
                       : (MODE == kBlock || split == p.splits - 1) ? (i_hi - i_lo + 1) * p.N : 0;
  const int ntiles = ctx_tiles + (blk_keys + kKeys - 1) / kKeys;

  // full context tiles: the pipelined pass; then the rest (a partial context
  // tile, the block keys) in the generic loop
  int j0 = 0;
  if (MODE != kBlock && ctx_keys / kKeys >= 2) {
    j0 = ctx_keys / kKeys;
    ctx_pipelined<D>(sm, p, g, ctx_lo, j0, qf, acc, m_run, l_run, col, half);
  }
  TileRegs<D> tr;
  if (ntiles > j0) {
    tile_load<D, MODE == kBlock>(tr, p, tile_range(p, j0, split, ctx_tiles, blk_keys), g, i_lo);
    tile_store<D>(sm, 0, tr);
  }
  __syncthreads();
  for (int j = j0; j < ntiles; ++j) {
    const int buf = (j - j0) & 1;
    const TileRange cur = tile_range(p, j, split, ctx_tiles, blk_keys);
    const bool more = j + 1 < ntiles;
    if (more) tile_load<D, MODE == kBlock>(tr, p, tile_range(p, j + 1, split, ctx_tiles, blk_keys), g, i_lo);

    // S^T tile: 2 blocks of 32 keys x 32 rows
    floatx16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = floatx16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const u32x4 kf = ld16(&sm.k[buf][kb * 32 + col][s * 16 + half * 8]);
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[s]), st[kb], 0, 0, 0);
      }
    }
    // Mask (partial context tiles and block tiles only) and tile max of the
    // raw scores; register r holds key kb*32 + 8*(r/4) + 4*half + r%4.
    float tmax = -INFINITY;
    if (cur.ctx && cur.count == kKeys) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[kb][r]);
    } else {
      // visible keys: kk < count and, in the block phase, kk in this row's branch
      int lo = 0, hi = cur.count;
      if (!cur.ctx) {
        lo = max(lo, (my_branch - i_lo) * p.N - cur.key0);
        const int last = p.causal ? bn_q % p.N : p.N - 1;  // the row's last visible block position
        hi = min(hi, (my_branch - i_lo) * p.N + last + 1 - cur.key0);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          const float sv = (kk >= lo && kk < hi) ? st[kb][r] : -INFINITY;
          st[kb][r] = sv;
          tmax = fmaxf(tmax, sv);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    // O and l are rescaled only when some lane's running max moved (elsewhere
    // the factor is exactly 1).
    if (__any(m_new > m_run)) {
      const float alpha = m_new > m_run ? exp2_fast((m_run - m_new) * p.scale_log2) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
    }
    m_run = m_new;
    const float mc = m_new == -INFINITY ? 0.f : m_new * p.scale_log2;
    float psum = 0.f;
    unsigned pk[2][2][4];  // [kb][t2][pair] packed bf16 P
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        floatx2 pp;
        pp[0] = exp2_fast(fmaf(st[kb][r], p.scale_log2, -mc));
        pp[1] = exp2_fast(fmaf(st[kb][r + 1], p.scale_log2, -mc));
        psum += pp[0] + pp[1];
        pk[kb][r / 8][(r % 8) / 2] = __builtin_bit_cast(unsigned, __builtin_convertvector(pp, bf16x2));
      }
    }
    l_run += psum;
    // O^T += V^T P^T : A = V^T rows (dims), B = P^T (keys x rows)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        u32x4 pb;
        pb[0] = pk[kb][t2][0];
        pb[1] = pk[kb][t2][1];
        pb[2] = pk[kb][t2][2];
        pb[3] = pk[kb][t2][3];
        const int kbase = kb * 32 + 16 * t2 + 4 * half;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const uint2 lo = *(const uint2*)(&sm.vt[buf][b * 32 + col][kbase]);
          const uint2 hi = *(const uint2*)(&sm.vt[buf][b * 32 + col][kbase + 8]);
          u32x4 vf;
          vf[0] = lo.x;
          vf[1] = lo.y;
          vf[2] = hi.x;
          vf[3] = hi.y;
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pb), acc[b], 0, 0, 0);
        }
      }
    }
    if (more) tile_store<D>(sm, buf ^ 1, tr);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (!row_ok) return;
  if (MODE == kBlock) {
    // merge the context state of the source row (kCtx partials), then write
    const size_t orow = ((size_t)bn_q * p.Hq + (size_t)g * p.G + rho % p.G);
    const float mb = m_run * p.scale_log2;
    float M = mb;
    size_t crow = 0;
    const size_t nstate = (size_t)p.splits * p.Hkv * p.rows_total;
    const float* mp = p.ws + nstate * D;
    if (p.L > 0) {
      const int ss = source_slot(p, bn_q);
      const int cidx = min(max(p.rec_pos[ss], 0), max(rec_count(p) - 1, 0));
      crow = (size_t)cidx * p.G + rho % p.G;
      for (int sp = 0; sp < p.splits; ++sp) M = fmaxf(M, mp[((size_t)sp * p.Hkv + g) * p.rows_total + crow]);
    }
    const float fb = exp2_fast(mb - M);
    float Z = l_tot * fb;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[b][r] *= fb;
    if (p.L > 0) {
      for (int sp = 0; sp < p.splits; ++sp) {
        const size_t prow = ((size_t)sp * p.Hkv + g) * p.rows_total + crow;
        const float w = mp[nstate + prow] * exp2_fast(mp[prow] - M);
        Z += w;
        const float* op = p.ws + prow * D;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 v = *(const float4*)(op + b * 32 + 8 * q4 + 4 * half);
            acc[b][4 * q4 + 0] = fmaf(w, v.x, acc[b][4 * q4 + 0]);
            acc[b][4 * q4 + 1] = fmaf(w, v.y, acc[b][4 * q4 + 1]);
            acc[b][4 * q4 + 2] = fmaf(w, v.z, acc[b][4 * q4 + 2]);
            acc[b][4 * q4 + 3] = fmaf(w, v.w, acc[b][4 * q4 + 3]);
          }
        }
      }
    }
    const float inv = 1.f / Z;
    unsigned short* out = p.o + orow * D;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dcol = b * 32 + 8 * q4 + 4 * half;
        uint2 w;
        w.x = pack_bf16x2(acc[b][4 * q4 + 0] * inv, acc[b][4 * q4 + 1] * inv);
        w.y = pack_bf16x2(acc[b][4 * q4 + 2] * inv, acc[b][4 * q4 + 3] * inv);
        *(uint2*)(out + dcol) = w;
      }
    }
    if (half == 0) p.lse[orow] = (M + log2f(Z)) * 0.69314718055994531f;
    return;
  }
  const float inv_l = 1.f / l_tot;
  if (MODE == kDense && p.splits == 1) {
    const size_t orow = ((size_t)bn_q * p.Hq + (size_t)g * p.G + rho % p.G);
    unsigned short* out = p.o + orow * D;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dcol = b * 32 + 8 * q4 + 4 * half;
        uint2 w;
        w.x = pack_bf16x2(acc[b][4 * q4 + 0] * inv_l, acc[b][4 * q4 + 1] * inv_l);
        w.y = pack_bf16x2(acc[b][4 * q4 + 2] * inv_l, acc[b][4 * q4 + 3] * inv_l);
        *(uint2*)(out + dcol) = w;
      }
    }
    if (half == 0) p.lse[orow] = m_run * p.scale_log2 * 0.69314718055994531f + logf(l_tot);
  } else {
    const size_t prow = ((size_t)split * p.Hkv + g) * p.ws_rows + (rho - p.ws_row0);
    float* op = p.ws + prow * D;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dcol = b * 32 + 8 * q4 + 4 * half;
        *(float4*)(op + dcol) = make_float4(acc[b][4 * q4 + 0] * inv_l, acc[b][4 * q4 + 1] * inv_l,
                                            acc[b][4 * q4 + 2] * inv_l, acc[b][4 * q4 + 3] * inv_l);
      }
    }
    if (half == 0) {
      const size_t nstate = (size_t)p.splits * p.Hkv * p.ws_rows;
      float* mp = p.ws + nstate * D;
      mp[prow] = m_run * p.scale_log2;  // log2 domain (m_run is finite: every split sees a key)
      mp[nstate + prow] = l_tot;
    }
  }
}

// Log-sum-exp merge of the split states of rows ws_row0 .. ws_row0 + ws_rows
// - 1 (those below rows_total): one thread per (kv head, row, 4 dims).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(Params p) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  constexpr int Q4 = D / 4;
  const size_t n_items = (size_t)p.Hkv * p.ws_rows * Q4;
  if (tid >= n_items) return;
  const int q4 = tid % Q4;
  const size_t gr = tid / Q4;  // g * ws_rows + (rho - ws_row0)
  const int g = gr / p.ws_rows;
  const int rho = p.ws_row0 + (int)(gr % p.ws_rows);
  if (rho >= p.rows_total) return;
  const size_t nstate = (size_t)p.splits * p.Hkv * p.ws_rows;
  const float* mp = p.ws + nstate * D;
  const float* lp = mp + nstate;
  float m = -INFINITY;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, mp[(size_t)s * p.Hkv * p.ws_rows + gr]);
  float z = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < p.splits; ++s) {
    const size_t prow = (size_t)s * p.Hkv * p.ws_rows + gr;
    const float w = lp[prow] * exp2f(mp[prow] - m);
    const float4 v = *(const float4*)(p.ws + prow * D + q4 * 4);
    z += w;
    o.x += w * v.x;
    o.y += w * v.y;
    o.z += w * v.z;
    o.w += w * v.w;
  }
  const float inv = 1.f / z;
  const int bn = rho / p.G, j = rho % p.G;
  const size_t orow = ((size_t)bn * p.Hq + (size_t)g * p.G + j);
  uint2 w2;
  w2.x = pack_bf16x2(o.x * inv, o.y * inv);
  w2.y = pack_bf16x2(o.z * inv, o.w * inv);
  *(uint2*)(p.o + orow * D + q4 * 4) = w2;
  if (q4 == 0) p.lse[orow] = m * 0.69314718055994531f + logf(z);
}

// One dense launch over the row tiles [p.tile0, p.tile0 + p.tiles) with
// p.splits context splits, then (split) the merge of their states.
template <int D>
hipError_t launch_dense_range(const Params& p, hipStream_t stream) {
  const int blocks = p.tiles * p.Hkv * p.splits;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_kernel<D, kDense>), dim3(blocks), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const size_t items = (size_t)p.Hkv * p.ws_rows * (D / 4);
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Dense attention: every row tile with the plan's splits; or, with a tail,
// the row tiles before it unsplit and the tail's split over the context.
template <int D>
hipError_t launch_d(const Params& p0, const AttnPlan& plan, hipStream_t stream) {
  Params p = p0;
  p.tile0 = 0;
  p.tiles = plan.row_tiles - plan.tail_tiles;
  p.ws_row0 = 0;
  p.ws_rows = plan.rows_total;
  hipError_t e = launch_dense_range<D>(p, stream);
  if (e != hipSuccess || plan.tail_tiles == 0) return e;
  p.tile0 = plan.row_tiles - plan.tail_tiles;
  p.tiles = plan.tail_tiles;
  p.splits = plan.tail_splits;
  p.chunk = plan.tail_chunk;
  p.ws_row0 = p.tile0 * kRows;
  p.ws_rows = plan.tail_tiles * kRows;
  return launch_dense_range<D>(p, stream);
}

// Folded: context states of the recomputed rows, then every row's block keys
// merged with its source row's context state.
template <int D>
hipError_t launch_folded_d(const Params& p, hipStream_t stream) {
  if (p.L > 0) {
    hipLaunchKernelGGL((attn_kernel<D, kCtx>), dim3(p.row_tiles * p.Hkv * p.splits), dim3(kThreads), 0, stream,
                       p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_kernel<D, kBlock>), dim3(p.row_tiles * p.Hkv), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int B1, int N, int L, int Hq, int Hkv, int d) {
  AttnPlan pl;
  const int G = Hq / Hkv;
  pl.rows_total = B1 * N * G;
  pl.row_tiles = (pl.rows_total + kRows - 1) / kRows;
  const int base = pl.row_tiles * Hkv;
  int splits = 1;
  if (L > 0) {
    const int want = (512 + base - 1) / base;       // aim for >= 512 workgroups
    // at least 512 context keys per split: a shorter split's fixed costs (Q
    // loads, the fp32 partial state, the merge) outweigh the parallelism
    const int most = L / 512 > 0 ? L / 512 : 1;
    splits = want < most ? want : most;
    if (splits < 1) splits = 1;
    if (splits > 16) splits = 16;
  }
  int chunk = L > 0 ? (L + splits - 1) / splits : 0;
  chunk = (chunk + kKeys - 1) / kKeys * kKeys;
  if (L > 0) splits = (L + chunk - 1) / chunk;
  pl.splits = splits;
  pl.chunk = chunk;
  pl.ws_bytes = splits > 1 ? (size_t)splits * Hkv * pl.rows_total * (d + 2) * sizeof(float) : 0;
  pl.ws_bytes_folded = L > 0 ? (size_t)splits * Hkv * pl.rows_total * (d + 2) * sizeof(float) : 0;
  // Tail split.  Unsplit, the workgroups run in rounds of kSlots (two per CU
  // on 256 CUs); when they overshoot whole rounds by at most a quarter round,
  // that last round would run a few long workgroups on a few CUs.  The row
  // tiles of that remainder (the last ones of every kv head) are then split
  // over the context into up to kSlots short workgroups instead (at most 8
  // splits: at 4096 keys, 8 splits of 512 keys ran the attention 2-4% faster
  // than 16 of 256, with half the states to merge), whose states are merged,
  // and the others run unsplit in whole rounds.
  pl.tail_tiles = 0;
  pl.tail_splits = 1;
  pl.tail_chunk = chunk;
  const int wgs = pl.row_tiles * Hkv;
  const int rem = wgs % kSlots;
  if (splits == 1 && L >= 2 * kKeys && wgs > kSlots && rem > 0 && rem <= kSlots / 4) {
    const int tt = (rem + Hkv - 1) / Hkv;
    int ts = kSlots / (tt * Hkv);
    const int most = L / (2 * kKeys);  // at least two context tiles per split
    if (ts > most) ts = most;
    if (ts > 8) ts = 8;
    if (ts >= 2) {
      int tc = (L + ts - 1) / ts;
      tc = (tc + kKeys - 1) / kKeys * kKeys;
      pl.tail_tiles = tt;
      pl.tail_splits = (L + tc - 1) / tc;
      pl.tail_chunk = tc;
      pl.ws_bytes = (size_t)pl.tail_splits * Hkv * (tt * kRows) * (d + 2) * sizeof(float);
    }
  }
  return pl;
}

hipError_t launch_attention(const void* q, const void* k_blk, const void* v_blk,
                            const void* k_ctx, const void* v_ctx, int B1, int N, int L,
                            int Hq, int Hkv, int d, float scale, void* o, float* lse,
                            void* ws, const AttnPlan& plan, hipStream_t stream,
                            const int32_t* rec_rows, const int32_t* src, const int32_t* rec_count,
                            const int32_t* rec_pos, bool causal) {
  Params p;
  p.causal = causal;
  p.qrows = rec_rows;
  p.src = src;
  p.count = rec_count;
  p.rec_pos = rec_pos;
  p.q = (const unsigned short*)q;
  p.k_blk = (const unsigned short*)k_blk;
  p.v_blk = (const unsigned short*)v_blk;
  p.k_ctx = (const unsigned short*)k_ctx;
  p.v_ctx = (const unsigned short*)v_ctx;
  p.o = (unsigned short*)o;
  p.lse = lse;
  p.ws = (float*)ws;
  p.B1 = B1;
  p.N = N;
  p.L = L;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.rows_total = plan.rows_total;
  p.row_tiles = plan.row_tiles;
  p.splits = plan.splits;
  p.chunk = plan.chunk;
  p.tile0 = 0;
  p.tiles = plan.row_tiles;
  p.ws_row0 = 0;
  p.ws_rows = plan.rows_total;
  p.scale_log2 = scale * 1.4426950408889634f;
  const bool fold = rec_rows != nullptr;
  switch (d) {
    case 32: return fold ? launch_folded_d<32>(p, stream) : launch_d<32>(p, plan, stream);
    case 64: return fold ? launch_folded_d<64>(p, stream) : launch_d<64>(p, plan, stream);
    case 128: return fold ? launch_folded_d<128>(p, stream) : launch_d<128>(p, plan, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sfv
