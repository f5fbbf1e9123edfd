// Online-softmax attention update of one wave for one 32-token block of one
// head (SR-SWA step 4, news.rkmt.cn/news/25027 Sec. 5), shared by the sparse
// gather attention and the dense full-context comparator.
//
// A wave reads the block's 8 KB K tile and 8 KB V tile with contiguous 1 KB
// loads: lane l holds dims 8*(l%16)..+8 of keys 4k + l/16 (k = 0..7), which
// are exactly the keys whose probabilities it needs for its V slice, so the
// scores never leave the lane's DPP row.  Logits are scaled by
// sm_scale*log2(e) and exponentiated with exp2; tokens past p are masked and
// their V is never read into the sum.  State: m (running max, log2 units,
// wave-uniform), l (running sum over the lane's key group), o[8] (the lane's
// slice of the unnormalised output).
#pragma once

#include "device_common.h"

namespace uocr {

// The wave's share of a block's K and V tiles: lane l holds dims
// 8*(l%16)..+8 of keys 4k + l/16, k = 0..7 (eight 1 KB loads per tile).
__device__ __forceinline__ void load_block_tiles(const uint16_t* k_tile, const uint16_t* v_tile, uint4 (&kv)[8],
                                                 uint4 (&vv)[8]) {
  const int lane = lane_id();
  const uint4* kt = reinterpret_cast<const uint4*>(k_tile);
  const uint4* vt = reinterpret_cast<const uint4*>(v_tile);
#pragma unroll
  for (int k = 0; k < 8; ++k) kv[k] = kt[k * kWave + lane];
#pragma unroll
  for (int k = 0; k < 8; ++k) vv[k] = vt[k * kWave + lane];
}

// Online-softmax update of (m, l, o) with block j of a query at position p,
// from tiles already in registers.
__device__ __forceinline__ void attend_loaded_block(const uint4 (&kv)[8], const uint4 (&vv)[8], int j, int p,
                                                    const uint4& qv, float scale_log2, float& m, float& l,
                                                    float (&o)[8]) {
  const int g = lane_id() >> 4;  // key row group within a 4-key slab
  const bool full = j * kBlock + (kBlock - 1) <= p;
  float s[8];
  float bm = -INFINITY;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float z = row16_sum(dot8_bf16(kv[k], qv)) * scale_log2;
    if (!full && j * kBlock + 4 * k + g > p) z = -INFINITY;
    s[k] = z;
    bm = fmaxf(bm, z);
  }
  bm = max_xor16(bm);
  bm = max_xor32(bm);
  const float m_new = fmaxf(m, bm);
  const float alpha = exp2f(m - m_new);
  l *= alpha;
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] *= alpha;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool valid = full || (j * kBlock + 4 * k + g <= p);
    const float pk = valid ? exp2f(s[k] - m_new) : 0.0f;
    l += pk;
    if (valid) {
      o[0] += pk * bf16_lo(vv[k].x);
      o[1] += pk * bf16_hi(vv[k].x);
      o[2] += pk * bf16_lo(vv[k].y);
      o[3] += pk * bf16_hi(vv[k].y);
      o[4] += pk * bf16_lo(vv[k].z);
      o[5] += pk * bf16_hi(vv[k].z);
      o[6] += pk * bf16_lo(vv[k].w);
      o[7] += pk * bf16_hi(vv[k].w);
    }
  }
  m = m_new;
}

__device__ __forceinline__ void attend_block(const uint16_t* k_tile, const uint16_t* v_tile, int j, int p,
                                             const uint4& qv, float scale_log2, float& m, float& l, float (&o)[8]) {
  uint4 kv[8], vv[8];
  load_block_tiles(k_tile, v_tile, kv, vv);
  attend_loaded_block(kv, vv, j, p, qv, scale_log2, m, l, o);
}

// Sum of a wave's four key groups (lanes l, l^16, l^32, l^48) of l and o.
__device__ __forceinline__ void reduce_key_groups(float& l, float (&o)[8]) {
  l = sum_xor16(l);
  l = sum_xor32(l);
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    o[d] = sum_xor16(o[d]);
    o[d] = sum_xor32(o[d]);
  }
}

}  // namespace uocr
