// Device helpers shared by the libsfv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
// 16 bytes as a first-class vector (uint4 is a struct: copying it from global
// memory goes through memcpy and can keep register arrays out of registers).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin

// Workgroup ids are dealt to the XCDs round-robin (id % 8).  This returns a
// logical id such that consecutive logical ids run on the same XCD, so tiles
// that share data (and so L2 lines) can be given consecutive logical ids.
__device__ __forceinline__ int xcd_logical_block(int b, int total) {
  const int xcd = b % kXcds;
  const int slot = b / kXcds;
  const int per = total / kXcds;
  const int extra = total % kXcds;
  return xcd * per + (xcd < extra ? xcd : extra) + slot;
}

__device__ __forceinline__ float bf16_bits_to_float(unsigned short h) {
  return __uint_as_float(((unsigned)h) << 16);
}

// fp32 -> bf16 round to nearest even (inputs are finite).
__device__ __forceinline__ unsigned short float_to_bf16_bits(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return (unsigned)float_to_bf16_bits(lo) | ((unsigned)float_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }


__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Maximum over the 64 lanes of a wave, returned as a wave-uniform value:
// rotations by 1, 2, 4 and 8 within each 16-lane row give every lane its
// row's maximum, two row broadcasts carry rows 0-2 into row 3, and lane 63 is
// read out.  All VALU (DPP) and one readlane, no LDS round trip; every lane
// must be active.  The maximum does not depend on the order of combination, so
// the result equals any other reduction's.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_keep(float x) {
  // lanes outside the row mask (and lanes whose source is out of range) keep x
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), kCtrl, kRowMask, 0xF, false));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_keep<0x121, 0xF>(v));  // row_ror:1
  v = fmaxf(v, dpp_keep<0x122, 0xF>(v));  // row_ror:2
  v = fmaxf(v, dpp_keep<0x124, 0xF>(v));  // row_ror:4
  v = fmaxf(v, dpp_keep<0x128, 0xF>(v));  // row_ror:8
  v = fmaxf(v, dpp_keep<0x142, 0xA>(v));  // row_bcast:15 into rows 1 and 3
  v = fmaxf(v, dpp_keep<0x143, 0xC>(v));  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace sfv
