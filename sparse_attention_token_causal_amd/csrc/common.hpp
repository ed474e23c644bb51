// Device-side building blocks shared by the indexer kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

enum Fmt : int { F32 = 0, BF16 = 1, FP8 = 2 };

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;

// Order-preserving map float -> uint32 (larger float -> larger key).  -0 is
// canonicalised to +0 first so that the two compare equal, as the tie rule
// requires.  Every finite value maps above kKeyExcluded, which marks an
// entry that is not eligible (masked).
constexpr uint32_t kKeyExcluded = 0u;

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key (for keys of finite values).
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float neg_inf() { return __uint_as_float(0xFF800000u); }

// bfloat16 bits of an exactly representable float (truncation is exact when
// the low 16 bits are zero, as for every widened FP8 E4M3 value).
__device__ __forceinline__ uint32_t bf16_hi(float f) { return __float_as_uint(f) >> 16; }

// Round-to-nearest-even float -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four OCP E4M3 codes (one dword) -> four bfloat16 values packed in two
// dwords (low code first).  gfx950's packed conversion (scale 1.0) is exact:
// E4M3 has 3 mantissa bits and a narrower exponent range than bfloat16.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t codes, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true));
}

__device__ __forceinline__ float fp8_to_f32(uint32_t code) {
  auto a = __builtin_amdgcn_cvt_pk_f32_fp8(code & 0xFFu, false);
  return a[0];
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, kWave); }

// Wave-wide inclusive prefix sum of an int on DPP lane moves (VALU, no LDS
// round trips): shifts by 1, 2, 4 and 8 inside each row of 16 lanes (a lane
// without a source adds 0), then row 0's total into row 1 and row 2's into
// row 3 (row_bcast:15), then the total of rows 0-1 into rows 2-3
// (row_bcast:31).  Every lane must be active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Wave-wide maximum of an unsigned int on DPP lane moves (the same row
// shifts and broadcasts as the prefix sum, with max for +), returned
// wave-uniform.  Every lane must be active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Wave-wide sum (every lane active), returned wave-uniform.
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), kWave - 1);
}

}  // namespace idx
