// SpecFold folded verification: the parent-child gate, source resolution
// and the compacted recomputed list.
//
// SpecFold ("Folding Multi-Branch Redundancy for Faster Speculative Decoding
// in Diffusion Language Models"), Sec. 3.2 and App. B:
//  * Gate (Eq. 4-5): slot n of draft i folds when the relative residual of
//    its layer-input hidden state against the parent's at n is at most delta;
//    the main branch recomputes every slot.  Decided as num <= delta^2 * den
//    with both squared norms accumulated in fp64 (one wave per slot).
//  * Sources (App. B): a folded slot takes its Q/K/V from the nearest
//    ancestor in which the position is recomputed.  The pages chase the
//    chains hop by hop; here one pass over the branches in index order (a
//    parent's index is below its child's) gives every slot its source.
//  * Compaction (App. B): the recomputed slots in (branch, position) order,
//    with per-branch offsets and each recomputed slot's list index, by a
//    block-wide prefix sum (the pages use atomic counters; a scan keeps the
//    order fixed).
// The folded attention itself is the attention kernel's kCtx/kBlock modes.
#include "common.h"
#include "internal.h"

namespace sfv {
namespace {

constexpr int kGateWaves = 4;

__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// One wave per slot (i, n): recompute[i*N+n] = 1 unless i >= 1 and
// ||H_i[n] - H_p[n]||^2 <= delta^2 * ||H_p[n]||^2 (fp64 sums of exact terms).
__global__ __launch_bounds__(kGateWaves* kWave) void fold_gate_kernel(const unsigned short* H, TreeArgs tree,
                                                                      int N, int D, float delta,
                                                                      int32_t* recompute) {
  const int lane = threadIdx.x % kWave;
  const int slot = blockIdx.x * kGateWaves + threadIdx.x / kWave;
  if (slot >= tree.B1 * N) return;
  const int i = slot / N, n = slot % N;
  if (i == 0 || delta < 0.f) {
    if (lane == 0) recompute[slot] = 1;
    return;
  }
  const int p = tree.parent[i];
  const unsigned short* hc = H + (size_t)slot * D;
  const unsigned short* hp = H + ((size_t)p * N + n) * D;
  double num = 0.0, den = 0.0;
  for (int k = lane * 8; k < D; k += kWave * 8) {  // D % 8 == 0
    const u32x4 a = ld16(hc + k);
    const u32x4 b = ld16(hp + k);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const double x = bf16_to_f32((unsigned short)(a[w] >> (16 * hlf)));
        const double y = bf16_to_f32((unsigned short)(b[w] >> (16 * hlf)));
        const double dxy = x - y;
        num = fma(dxy, dxy, num);
        den = fma(y, y, den);
      }
    }
  }
  num = wave_sum_f64(num);
  den = wave_sum_f64(den);
  const double d2 = (double)delta * (double)delta;
  if (lane == 0) recompute[slot] = num <= d2 * den ? 0 : 1;
}

// One workgroup: sources, the compacted recomputed list, each slot's index
// in it, and branch offsets.  The flags are staged in LDS once.
constexpr int kResolveThreads = 256;

__global__ __launch_bounds__(kResolveThreads) void fold_resolve_kernel(const int32_t* recompute, TreeArgs tree,
                                                                       int N, int32_t* src, int32_t* rec_rows,
                                                                       int32_t* rec_count, int32_t* rec_pos,
                                                                       int32_t* branch_off) {
  __shared__ unsigned char flag[kMaxBranches * kMaxBlock];
  __shared__ unsigned char col[kMaxBranches][kResolveThreads];  // sources of thread t's position
  __shared__ int wave_tot[kResolveThreads / kWave];
  __shared__ int bcount[kMaxBranches];
  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int B1 = tree.B1;
  const int total = B1 * N;
  for (int f = t; f < total; f += kResolveThreads) flag[f] = recompute[f] != 0;
  __syncthreads();

  // sources: branches in index order, so a parent's entry is final before
  // its children read it (one LDS column per thread)
  for (int n = t; n < N; n += kResolveThreads) {
    for (int i = 0; i < B1; ++i) {
      const int f = i * N + n;
      const int s = (i == 0 || flag[f]) ? i : col[tree.parent[i]][t];
      col[i][t] = (unsigned char)s;
      src[f] = s;
    }
  }
  for (int i = t; i < B1; i += kResolveThreads) {
    int c = 0;
    for (int n = 0; n < N; ++n) c += flag[i * N + n];
    bcount[i] = c;
  }
  // compaction: thread t owns the contiguous slots [t*per, (t+1)*per)
  const int per = (total + kResolveThreads - 1) / kResolveThreads;
  const int lo = min(t * per, total), hi = min(lo + per, total);
  int mine = 0;
  for (int f = lo; f < hi; ++f) mine += flag[f];
  int incl = mine;  // inclusive prefix within the wave
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = incl - mine;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  for (int f = lo; f < hi; ++f) {
    if (flag[f]) {
      rec_rows[base] = f;
      rec_pos[f] = base++;
    } else {
      rec_pos[f] = -1;
    }
  }
  if (t == 0) {
    int acc = 0;
    for (int i = 0; i < B1; ++i) {
      branch_off[i] = acc;
      acc += bcount[i];
    }
    branch_off[B1] = acc;
    rec_count[0] = acc;
  }
}

}  // namespace

hipError_t launch_fold_gate(const void* H, const TreeArgs& tree, int N, int D, float delta,
                            int32_t* recompute, int32_t* src, int32_t* rec_rows, int32_t* rec_count,
                            int32_t* rec_pos, int32_t* branch_off, hipStream_t stream) {
  const int slots = tree.B1 * N;
  hipLaunchKernelGGL(fold_gate_kernel, dim3((slots + kGateWaves - 1) / kGateWaves), dim3(kGateWaves * kWave), 0,
                     stream, (const unsigned short*)H, tree, N, D, delta, recompute);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fold_resolve_kernel, dim3(1), dim3(kResolveThreads), 0, stream, recompute, tree, N, src,
                     rec_rows, rec_count, rec_pos, branch_off);
  return hipGetLastError();
}

}  // namespace sfv
