// Device helpers shared by the SR-SWA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uocr {

constexpr int kBlock = 32;     // tokens per KV block
constexpr int kDim = 128;      // head_dim == index_dim
constexpr int kWave = 64;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// 16-byte load of data that is read once and not reused by this launch
// (streamed KV-cache tiles): a non-temporal load, which does not keep the
// line in the caches at normal priority.  Measured on the 128K decode step:
// the indexer keys stream at 6.2 TB/s this way against 5.5-5.8 TB/s with
// ordinary loads.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// c + a.lo*b.lo + a.hi*b.hi on two packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Dot product of 8 bf16 pairs held as two uint4.
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b) {
  float s = dot2_bf16(a.x, b.x, 0.0f);
  s = dot2_bf16(a.y, b.y, s);
  s = dot2_bf16(a.z, b.z, s);
  return dot2_bf16(a.w, b.w, s);
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
// quad_perm [1,0,3,2] and [2,3,0,1] reduce each quad, row_half_mirror pairs
// the two quads of each half row, row_mirror pairs the two halves.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}

__device__ __forceinline__ float shfl_xor_f32(float v, int m) { return __shfl_xor(v, m, kWave); }

// Maximum over the 16 lanes of a DPP row (the exchanges of row16_sum).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  return fmaxf(v, dpp_f32<0x140>(v));
}
__device__ __forceinline__ int row16_max_i32(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
  return max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
}

// Combine a value with the one of lane l ^ 16 (or l ^ 32), in every lane,
// with the gfx950 lane swaps (one VALU op each, no LDS permute).  With both
// operands x, element 0 + element 1 of v_permlane16_swap is x[l] + x[l ^ 16]
// in every lane (likewise v_permlane32_swap for l ^ 32), the same two values
// a __shfl_xor exchange adds.
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) { float a, b; swap16(x, a, b); return a + b; }
__device__ __forceinline__ float sum_xor32(float x) { float a, b; swap32(x, a, b); return a + b; }
__device__ __forceinline__ float max_xor16(float x) { float a, b; swap16(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float max_xor32(float x) { float a, b; swap32(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ uint32_t sum_xor16_u32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return r[0] + r[1];
}
__device__ __forceinline__ uint32_t sum_xor32_u32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] + r[1];
}

// Sum, maximum over all 64 lanes of a wave, in every lane: the DPP row
// reduction, then the lane swaps across rows (no LDS permutes).
__device__ __forceinline__ float wave_sum_f32(float v) { return sum_xor32(sum_xor16(row16_sum(v))); }
__device__ __forceinline__ float wave_max_f32(float v) { return max_xor32(max_xor16(row16_max(v))); }
__device__ __forceinline__ int wave_max_i32(int v) {
  v = row16_max_i32(v);
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = max((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return max((int)r[0], (int)r[1]);
}

// Block-max reduction of key scores: NaN-propagating maximum (a block with a
// NaN key scores NaN, like a maximum over the set taken in the plain
// definition; ranked last).  On gfx950 it is v_maximum(3)_f32, with no
// operand canonicalisation.
__device__ __forceinline__ float max_keep_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Order-preserving map float32 -> uint32: a > b (as numbers) <=> key(a) >
// key(b); -0.0 maps like +0.0; NaN maps to 0, below every number.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum over the 64 lanes of a wave: inside each 16-lane
// DPP row by shifts of 1, 2, 4 and 8 lanes (a lane shifted in from outside
// the row adds 0), then the totals of the rows before (lanes 15, 31, 47).
// Every lane of the wave takes part.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int lane = lane_id();
  return x + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

__device__ __forceinline__ int clamp_ctx(int32_t L, int32_t max_blocks) {
  const int hi = max_blocks * kBlock;
  return L < 0 ? 0 : (L > hi ? hi : L);
}

}  // namespace uocr
