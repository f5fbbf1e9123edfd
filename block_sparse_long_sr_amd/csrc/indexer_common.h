// One wave's score of one indexer-K block (SR-SWA step 2,
// news.rkmt.cn/news/25027 Sec. 5): the maximum over the block's 32 keys of
// the key's dot product with the one-head 128-dim indexer query.  Shared by
// the decode scoring kernel and the fused decode-step kernel.
//
// Load k (k = 0..7) brings, in lane order, 1 KB = 4 key rows of the 8 KB
// tile, so lane l holds dims 8*(l%16)..+8 of key 4k + l/16 and every load
// instruction reads a fully contiguous 1 KB.  qv is the lane's 8-dim slice
// of the query (dims 8*(l%16)..+8).  Partial dots (v_dot2_f32_bf16, fp32
// accumulation of exact bf16 products) are summed over the 16 lanes of a DPP
// row; the block max is taken in-lane over k and across the four rows with
// two lane swaps.  A NaN key makes the block NaN.
#pragma once

#include "device_common.h"

namespace uocr {

// The wave's share of one 8 KB tile: lane l gets dims 8*(l%16)..+8 of keys
// 4k + l/16, k = 0..7 (non-temporal loads: every tile is read once).
__device__ __forceinline__ void load_index_tile(const uint16_t* tile, uint4 (&kv)[8]) {
  const uint4* base = reinterpret_cast<const uint4*>(tile);
  const int lane = lane_id();
#pragma unroll
  for (int k = 0; k < 8; ++k) kv[k] = load_stream16(base + k * kWave + lane);
}

// Block max of a tile already in registers (every lane gets it).
__device__ __forceinline__ float block_max_of_tile(const uint4 (&kv)[8], const uint4& qv) {
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max_keep_nan(m, row16_sum(dot8_bf16(kv[k], qv)));
  float a, b;
  swap16(m, a, b);
  m = max_keep_nan(a, b);
  swap32(m, a, b);
  return max_keep_nan(a, b);
}

__device__ __forceinline__ float score_block_wave(const uint16_t* tile, const uint4& qv) {
  uint4 kv[8];
  load_index_tile(tile, kv);
  return block_max_of_tile(kv, qv);
}

}  // namespace uocr
