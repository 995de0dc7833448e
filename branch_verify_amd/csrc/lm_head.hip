// LM head over the masked rows: logits[r][v] = <hidden[rows[r]], w[v]>,
// bf16 in, fp32 accumulate and out, on v_mfma_f32_32x32x16_bf16.
//
// SpecFold, Appendix B, keeps the LM head as a plain dense library product;
// here it is the dominant step of a one-layer verify pass (the weight is
// ~1.2 GB of bf16 and is streamed once per pass).  Design for gfx950:
//  * The product is computed transposed (vocab x rows) so that each lane ends
//    with 4 consecutive vocab ids of one row and stores them as one 16-byte
//    write of the row-major logits.
//  * Workgroup tile 128 vocab x 128 rows x 64 k, four waves of 64 x 64,
//    double-buffered LDS with the next k-tile prefetched into registers.
//  * The row tiles of one vocab tile get consecutive logical ids on one XCD,
//    so the weight tile they share is read from HBM once and then hit in L2.
//  * Masked rows are gathered on the fly from hidden through `rows`.
#include "common.h"
#include "internal.h"

namespace sfv {
namespace {

constexpr int kThreads = 256;
constexpr int BV = 128;  // vocab per tile
constexpr int BM = 128;  // rows per tile
constexpr int BK = 64;   // k per stage
constexpr int LDK = BK + 8;

struct Params {
  const unsigned short* hidden;
  const int32_t* rows;
  const unsigned short* w;
  float* logits;
  int M, D, V, R;
  int vt, mt;  // tile counts
};

__global__ __launch_bounds__(kThreads) void lm_head_kernel(Params p) {
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
  const unsigned short* wsrc[4];
  const unsigned short* hsrc[4];
  bool wok[4], hok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + kThreads * i;
    const int r = c / 8, part = c % 8;
    const int v = v0 + r;
    wok[i] = v < p.V;
    wsrc[i] = p.w + (size_t)(wok[i] ? v : 0) * p.D + part * 8;
    const int m = m0 + r;
    hok[i] = m < p.M;
    const int hr = hok[i] ? min(max(p.rows[m], 0), p.R - 1) : 0;  // never leave hidden
    hsrc[i] = p.hidden + (size_t)hr * p.D + part * 8;
  }

  uint4 wreg[4], hreg[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wreg[i] = wok[i] ? *(const uint4*)(wsrc[i] + k0) : make_uint4(0, 0, 0, 0);
      hreg[i] = hok[i] ? *(const uint4*)(hsrc[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = t + kThreads * i;
      const int r = c / 8, part = c % 8;
      *(uint4*)(&ws[buf][r][part * 8]) = wreg[i];
      *(uint4*)(&hs[buf][r][part * 8]) = hreg[i];
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = floatx16{};

  const int ksteps = p.D / BK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < ksteps) fetch((ks + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      uint4 af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = *(const uint4*)(&ws[buf][wv * 64 + a * 32 + col][kk * 16 + half * 8]);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bfr[b] = *(const uint4*)(&hs[buf][wm * 64 + b * 32 + col][kk * 16 + half * 8]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af[a]), as_bf16x8(bfr[b]),
                                                               acc[a][b], 0, 0, 0);
    }
    if (ks + 1 < ksteps) stash(buf ^ 1);
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

}  // namespace

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
  hipLaunchKernelGGL(lm_head_kernel, dim3(p.vt * p.mt), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sfv
