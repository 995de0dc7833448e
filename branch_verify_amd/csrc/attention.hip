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
#include "common.h"
#include "internal.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kRows = 128;     // query rows per workgroup, 32 per wave
constexpr int kKeys = 64;      // keys per LDS tile
constexpr int kPad = 8;        // bf16 elements of row padding in LDS

struct Params {
  const unsigned short* q;
  const unsigned short* k_blk;
  const unsigned short* v_blk;
  const unsigned short* k_ctx;
  const unsigned short* v_ctx;
  unsigned short* o;
  float* lse;
  float* ws;  // split partials: O [splits][Hkv][rows][d], m, l [splits][Hkv][rows]
  int B1, N, L, Hq, Hkv, G;
  int rows_total, row_tiles, splits, chunk;
  float scale_log2;  // softmax scale * log2(e): scores kept in the log2 domain
};

template <int D>
struct Smem {
  unsigned short k[kKeys][D + kPad];   // key tile, row-major
  unsigned short vt[D][kKeys + kPad];  // value tile, transposed
};

// Stage keys [key0, key0 + count) of one phase into LDS.  In the context phase
// key k lives at k_ctx[(g*L + k)*D]; in the block phase flat block key k
// (branch i_lo + k / N) lives at k_blk[((i_lo*N + k)*Hkv + g)*D].
template <int D>
__device__ __forceinline__ void load_tile(Smem<D>& sm, const Params& p, bool ctx, int g, int i_lo,
                                          int key0, int count) {
  const int t = threadIdx.x;
  constexpr int parts = D / 8;  // 16-byte chunks per key row
  const unsigned short* kbase;
  const unsigned short* vbase;
  size_t stride;
  if (ctx) {
    kbase = p.k_ctx + ((size_t)g * p.L + key0) * D;
    vbase = p.v_ctx + ((size_t)g * p.L + key0) * D;
    stride = D;
  } else {
    kbase = p.k_blk + (((size_t)i_lo * p.N + key0) * p.Hkv + g) * D;
    vbase = p.v_blk + (((size_t)i_lo * p.N + key0) * p.Hkv + g) * D;
    stride = (size_t)p.Hkv * D;
  }
  // keys: 64 rows x parts chunks
#pragma unroll
  for (int c = t; c < kKeys * parts; c += kThreads) {
    const int key = c / parts, part = c % parts;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (key < count) val = *(const uint4*)(kbase + key * stride + part * 8);
    *(uint4*)(&sm.k[key][part * 8]) = val;
  }
  // values: items of 4 keys x 8 dims, written transposed as 4-key runs
#pragma unroll
  for (int it = t; it < (kKeys / 4) * parts; it += kThreads) {
    const int dg = it % parts, kg = it / parts;
    uint4 rows4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kg * 4 + r;
      rows4[r] = make_uint4(0, 0, 0, 0);
      if (key < count) rows4[r] = *(const uint4*)(vbase + key * stride + dg * 8);
    }
    const unsigned short* e0 = (const unsigned short*)&rows4[0];
    const unsigned short* e1 = (const unsigned short*)&rows4[1];
    const unsigned short* e2 = (const unsigned short*)&rows4[2];
    const unsigned short* e3 = (const unsigned short*)&rows4[3];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 w;
      w.x = (unsigned)e0[e] | ((unsigned)e1[e] << 16);
      w.y = (unsigned)e2[e] | ((unsigned)e3[e] << 16);
      *(uint2*)(&sm.vt[dg * 8 + e][kg * 4]) = w;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(Params p) {
  __shared__ Smem<D> sm;
  constexpr int DS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DB = D / 32;  // 32-wide output blocks of the head dim

  const int total = gridDim.x;
  const int lid = xcd_logical_block(blockIdx.x, total);
  const int tile = lid % p.row_tiles;
  const int gs = lid / p.row_tiles;
  const int split = gs % p.splits;
  const int g = gs / p.splits;

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int half = lane / 32;
  const int col = lane % 32;

  const int row0 = tile * kRows;
  const int rho = row0 + wave * 32 + col;  // this lane's query row
  const bool row_ok = rho < p.rows_total;
  const int NG = p.N * p.G;
  const int my_branch = row_ok ? rho / NG : -1;

  // Q fragment of this lane's row: dims s*16 + half*8 .. +8 for each step s
  uint4 qf[DS];
  {
    size_t qoff = 0;
    if (row_ok) {
      const int bn = rho / p.G, j = rho % p.G;
      qoff = ((size_t)bn * p.Hq + (size_t)g * p.G + j) * D;
    }
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qf[s] = row_ok ? *(const uint4*)(p.q + qoff + s * 16 + half * 8) : make_uint4(0, 0, 0, 0);
    }
  }

  floatx16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = floatx16{};
  float m_run = -INFINITY;  // running max (log2 domain)
  float l_run = 0.f;        // running denominator, this half's keys only

  const int last_row = min(row0 + kRows, p.rows_total) - 1;
  const int i_lo = row0 / NG;
  const int i_hi = last_row / NG;

  // phase 0: context keys of this split; phase 1: block keys (last split only)
  for (int phase = 0; phase < 2; ++phase) {
    int key_begin, key_end;
    if (phase == 0) {
      key_begin = split * p.chunk;
      key_end = min(p.L, key_begin + p.chunk);
    } else {
      if (split != p.splits - 1) break;
      key_begin = 0;
      key_end = (i_hi - i_lo + 1) * p.N;
    }
    for (int k0 = key_begin; k0 < key_end; k0 += kKeys) {
      const int count = min(kKeys, key_end - k0);
      __syncthreads();
      load_tile<D>(sm, p, phase == 0, g, i_lo, k0, count);
      __syncthreads();

      // S^T tile: 2 blocks of 32 keys x 32 rows
      floatx16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = floatx16{};
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          const uint4 kf = *(const uint4*)(&sm.k[kb * 32 + col][s * 16 + half * 8]);
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[s]), st[kb], 0, 0, 0);
        }
      }
      // scale, mask, tile max (register r holds key kb*32 + 8*(r/4) + 4*half + r%4)
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kb * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          bool vis = kk < count;
          if (phase == 1) vis = vis && (i_lo + (k0 + kk) / p.N == my_branch);
          const float sv = vis ? st[kb][r] * p.scale_log2 : -INFINITY;
          st[kb][r] = sv;
          tmax = fmaxf(tmax, sv);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      const float m_new = fmaxf(m_run, tmax);
      float alpha, m_use;
      if (m_new == -INFINITY) {  // nothing visible yet for this row
        alpha = 1.f;
        m_use = 0.f;
      } else {
        alpha = exp2f(m_run - m_new);
        m_use = m_new;
      }
      m_run = m_new;
      float psum = 0.f;
      unsigned pk[2][2][4];  // [kb][t2][pair] packed bf16 P
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = exp2f(st[kb][r] - m_use);
          const float p1 = exp2f(st[kb][r + 1] - m_use);
          psum += p0 + p1;
          pk[kb][r / 8][(r % 8) / 2] = pack_bf16x2(p0, p1);
        }
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
      }
      // O^T += V^T P^T : A = V^T rows (dims), B = P^T (keys x rows)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          uint4 pb;
          pb.x = pk[kb][t2][0];
          pb.y = pk[kb][t2][1];
          pb.z = pk[kb][t2][2];
          pb.w = pk[kb][t2][3];
          const int kbase = kb * 32 + 16 * t2 + 4 * half;
#pragma unroll
          for (int b = 0; b < DB; ++b) {
            const uint2 lo = *(const uint2*)(&sm.vt[b * 32 + col][kbase]);
            const uint2 hi = *(const uint2*)(&sm.vt[b * 32 + col][kbase + 8]);
            const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pb), acc[b], 0, 0, 0);
          }
        }
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (!row_ok) return;
  const float inv_l = 1.f / l_tot;
  if (p.splits == 1) {
    const int bn = rho / p.G, j = rho % p.G;
    const size_t orow = ((size_t)bn * p.Hq + (size_t)g * p.G + j);
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
    if (half == 0) p.lse[orow] = m_run * 0.69314718055994531f + logf(l_tot);
  } else {
    const size_t prow = ((size_t)split * p.Hkv + g) * p.rows_total + rho;
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
      const size_t nstate = (size_t)p.splits * p.Hkv * p.rows_total;
      float* mp = p.ws + nstate * D;
      mp[prow] = m_run;
      mp[nstate + prow] = l_tot;
    }
  }
}

// Log-sum-exp merge of the split states: one thread per (kv head, row, 4 dims).
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(Params p) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  constexpr int Q4 = D / 4;
  const size_t n_items = (size_t)p.Hkv * p.rows_total * Q4;
  if (tid >= n_items) return;
  const int q4 = tid % Q4;
  const size_t gr = tid / Q4;  // g * rows_total + rho
  const int g = gr / p.rows_total;
  const int rho = gr % p.rows_total;
  const size_t nstate = (size_t)p.splits * p.Hkv * p.rows_total;
  const float* mp = p.ws + nstate * D;
  const float* lp = mp + nstate;
  float m = -INFINITY;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, mp[(size_t)s * p.Hkv * p.rows_total + gr]);
  float z = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < p.splits; ++s) {
    const size_t prow = (size_t)s * p.Hkv * p.rows_total + gr;
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

template <int D>
hipError_t launch_d(const Params& p, hipStream_t stream) {
  const int blocks = p.row_tiles * p.Hkv * p.splits;
  hipLaunchKernelGGL(attn_kernel<D>, dim3(blocks), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const size_t items = (size_t)p.Hkv * p.rows_total * (D / 4);
  hipLaunchKernelGGL(attn_merge_kernel<D>, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, p);
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
    const int most = L / 128 > 0 ? L / 128 : 1;     // at least 128 context keys per split
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
  return pl;
}

hipError_t launch_attention(const void* q, const void* k_blk, const void* v_blk,
                            const void* k_ctx, const void* v_ctx, int B1, int N, int L,
                            int Hq, int Hkv, int d, float scale, void* o, float* lse,
                            void* ws, const AttnPlan& plan, hipStream_t stream) {
  Params p;
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
  p.scale_log2 = scale * 1.4426950408889634f;
  switch (d) {
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sfv
