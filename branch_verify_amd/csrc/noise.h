// Counter-based noise shared by the commit and the drafter: the Gumbel noise
// of (seed, step, position, vocab id).
//
// SPOT, coupled-noise match: the target and the drafter use the same
// per-position Gumbel noise, so given the noise every transition is
// deterministic.  Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11) keyed by (seed, 0) on the counter
// (id >> 3, position, step, stream); id's word is half (id & 1) of output
// (id & 7) >> 1; g = -ln(-ln u) with u = (word + 1/2) 2^-32.  Stream 0 is
// the commit's and drafter's noise; streams 1 and 2 are the rejection
// sampler's acceptance uniforms and residual/bonus draws.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfv {

// 128-bit product of a 64-bit word and a 64-bit constant from four 32 x 32 ->
// 64 multiply-adds (v_mad_u64_u32), each partial sum carrying the previous
// one's high half, so no sum can overflow 64 bits: the same (hi, lo) as the
// plain 64 x 64 product, in fewer and cheaper instructions than the
// compiler's separate low and high products.
template <uint64_t B>
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t& hi, uint64_t& lo) {
  constexpr uint32_t b0 = (uint32_t)B, b1 = (uint32_t)(B >> 32);
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint64_t p00 = (uint64_t)a0 * b0;
  const uint64_t t = (uint64_t)a1 * b0 + (p00 >> 32);
  const uint64_t u = (uint64_t)a0 * b1 + (uint32_t)t;
  lo = (u << 32) | (uint32_t)p00;
  hi = (uint64_t)a1 * b1 + (t >> 32) + (u >> 32);
}

__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t lo0, hi0, lo1, hi1;
    mulhilo64<M0>(c[0], hi0, lo0);
    mulhilo64<M1>(c[2], hi1, lo1);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// The 8 noise words of ids 8*blk .. 8*blk+7: word j = half (j & 1) of output (j >> 1).
__device__ __forceinline__ void noise_block(uint64_t seed, uint64_t step, uint64_t pos, uint64_t blk,
                                            unsigned w[8], uint64_t stream = 0) {
  uint64_t c[4] = {blk, pos, step, stream};
  philox4x64_10(c, seed, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[2 * j] = (unsigned)(c[j] & 0xFFFFFFFFull);
    w[2 * j + 1] = (unsigned)(c[j] >> 32);
  }
}

// The defined value: fl32(-ln(-ln u)) with both logarithms in fp64.
__device__ __forceinline__ float gumbel_exact(unsigned w) {
  const double u = ((double)w + 0.5) * 2.3283064365386962890625e-10;
  return (float)(-log(-log(u)));
}

__device__ __forceinline__ double gumbel_exact_f64(unsigned w) {
  const double u = ((double)w + 0.5) * 2.3283064365386962890625e-10;
  return -log(-log(u));
}

// The noise word of one vocab id.
__device__ __forceinline__ unsigned noise_word(uint64_t seed, uint64_t step, uint64_t pos, uint64_t id,
                                               uint64_t stream = 0) {
  uint64_t c[4] = {id >> 3, pos, step, stream};
  philox4x64_10(c, seed, 0);
  const int j = (int)((id & 7) >> 1);
  const uint64_t w = j == 0 ? c[0] : j == 1 ? c[1] : j == 2 ? c[2] : c[3];
  return (id & 1) ? (unsigned)(w >> 32) : (unsigned)(w & 0xFFFFFFFFull);
}

}  // namespace sfv
