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
// kStream: the tiles are read once by this launch (decode), so the loads
// are non-temporal; prefill rows share tiles and keep ordinary loads.
template <bool kStream>
__device__ __forceinline__ void load_block_tiles(const uint16_t* k_tile, const uint16_t* v_tile, uint4 (&kv)[8],
                                                 uint4 (&vv)[8]) {
  const int lane = lane_id();
  const uint4* kt = reinterpret_cast<const uint4*>(k_tile);
  const uint4* vt = reinterpret_cast<const uint4*>(v_tile);
#pragma unroll
  for (int k = 0; k < 8; ++k) kv[k] = kStream ? load_stream16(kt + k * kWave + lane) : kt[k * kWave + lane];
#pragma unroll
  for (int k = 0; k < 8; ++k) vv[k] = kStream ? load_stream16(vt + k * kWave + lane) : vt[k * kWave + lane];
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

template <bool kStream>
__device__ __forceinline__ void attend_block(const uint16_t* k_tile, const uint16_t* v_tile, int j, int p,
                                             const uint4& qv, float scale_log2, float& m, float& l, float (&o)[8]) {
  uint4 kv[8], vv[8];
  load_block_tiles<kStream>(k_tile, v_tile, kv, vv);
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

// LDS of wave_attn_finish: one online-softmax state per wave.
template <int NT>
struct AttendSmem {
  float m[NT / kWave];
  float l[NT / kWave];
  float o[NT / kWave][kDim];
};

// One wave's online-softmax state of a query head: m (running max, log2
// units, wave-uniform), l (running sum over the lane's key group), o (the
// lane's 8-dim slice of the unnormalised output) and the lane's query slice.
struct WaveAttn {
  float m;
  float l;
  float o[8];
  uint4 qv;
};

__device__ __forceinline__ void wave_attn_init(WaveAttn& st, const uint16_t* q_head) {
  st.qv = *reinterpret_cast<const uint4*>(q_head + (lane_id() & 15) * 8);
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int d = 0; d < 8; ++d) st.o[d] = 0.0f;
}

// Block j of the sequence (table: its block-table row) into the wave's
// state; blocks starting after p and out-of-range pool indices are skipped.
template <bool kStream>
__device__ __forceinline__ void wave_attn_block(const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* table,
                                                int64_t num_blocks, int heads, int h, int j, int p, float scale_log2,
                                                WaveAttn& st) {
  if (j * kBlock > p) return;
  const int pb = __builtin_amdgcn_readfirstlane(table[j]);
  if (pb < 0 || (int64_t)pb >= num_blocks) return;
  const int64_t tile = ((int64_t)pb * heads + h) * (kBlock * kDim);
  attend_block<kStream>(k_pool + tile, v_pool + tile, j, p, st.qv, scale_log2, st.m, st.l, st.o);
}

// Entries e = wave, wave + NW, ... of sel[0 .. topk) into the wave's state;
// -1 entries and ids outside [0, j_end) are skipped (j_end = max_blocks for
// all of them; a smaller j_end leaves out blocks already attended).
template <int NT, bool kStream>
__device__ __forceinline__ void wave_attn_sel(const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* table,
                                              int64_t num_blocks, int heads, int h, int j_end, int p,
                                              const int32_t* sel, int topk, float scale_log2, WaveAttn& st) {
  constexpr int NW = NT / kWave;
  for (int e = wave_id(); e < topk; e += NW) {
    const int j = __builtin_amdgcn_readfirstlane(sel[e]);
    if (j < 0 || j >= j_end) continue;
    wave_attn_block<kStream>(k_pool, v_pool, table, num_blocks, heads, h, j, p, scale_log2, st);
  }
}

// As wave_attn_sel, with the tiles of the wave's entries e and e + NW
// loaded together before either is attended (two blocks' K and V in flight:
// 128 VGPRs of tiles, for kernels with 256 VGPRs per wave); the blocks are
// attended in the same order, so the result is the same.
template <int NT, bool kStream>
__device__ __forceinline__ void wave_attn_sel_pairs(const uint16_t* k_pool, const uint16_t* v_pool,
                                                    const int32_t* table, int64_t num_blocks, int heads, int h,
                                                    int j_end, int p, const int32_t* sel, int topk, float scale_log2,
                                                    WaveAttn& st) {
  constexpr int NW = NT / kWave;
  for (int e = wave_id(); e < topk; e += 2 * NW) {
    const int e2 = e + NW;
    const int ja = __builtin_amdgcn_readfirstlane(sel[e]);
    const int jb = e2 < topk ? __builtin_amdgcn_readfirstlane(sel[e2]) : -1;
    bool oka = ja >= 0 && ja < j_end && ja * kBlock <= p;
    bool okb = jb >= 0 && jb < j_end && jb * kBlock <= p;
    const int pba = oka ? __builtin_amdgcn_readfirstlane(table[ja]) : -1;
    const int pbb = okb ? __builtin_amdgcn_readfirstlane(table[jb]) : -1;
    oka = oka && pba >= 0 && (int64_t)pba < num_blocks;
    okb = okb && pbb >= 0 && (int64_t)pbb < num_blocks;
    uint4 ka[8], va[8], kb[8], vb[8];
    if (oka) {
      const int64_t tile = ((int64_t)pba * heads + h) * (kBlock * kDim);
      load_block_tiles<kStream>(k_pool + tile, v_pool + tile, ka, va);
    }
    if (okb) {
      const int64_t tile = ((int64_t)pbb * heads + h) * (kBlock * kDim);
      load_block_tiles<kStream>(k_pool + tile, v_pool + tile, kb, vb);
    }
    if (oka) attend_loaded_block(ka, va, ja, p, st.qv, scale_log2, st.m, st.l, st.o);
    if (okb) attend_loaded_block(kb, vb, jb, p, st.qv, scale_log2, st.m, st.l, st.o);
  }
}

// The workgroup's NT/64 wave states merged through LDS into the head's
// normalised output (128 floats) and its lse (natural log; lse_out may be
// null); every thread calls it.
template <int NT>
__device__ __forceinline__ void wave_attn_finish(WaveAttn& st, float* out_head, float* lse_out, AttendSmem<NT>& sm) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wave = wave_id();
  const int c8 = (lane & 15) * 8;
  reduce_key_groups(st.l, st.o);
  if (lane == 0) {
    sm.m[wave] = st.m;
    sm.l[wave] = st.l;
  }
  if (lane < 16) {
#pragma unroll
    for (int d = 0; d < 8; ++d) sm.o[wave][c8 + d] = st.o[d];
  }
  __syncthreads();
  if (threadIdx.x < kDim) {
    const int d = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w]);
    float res = 0.0f, lse_v = -INFINITY;
    if (M != -INFINITY) {
      float Lsum = 0.0f, acc = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(sm.m[w] - M);
        Lsum += sm.l[w] * f;
        acc += sm.o[w][d] * f;
      }
      res = acc / Lsum;
      lse_v = (M + log2f(Lsum)) * kLn2;
    }
    out_head[d] = res;
    if (lse_out != nullptr && d == 0) *lse_out = lse_v;
  }
}

// Attention of one query head at position p over the kept blocks
// sel[0 .. topk) (global or LDS memory; -1 and out-of-range entries, blocks
// starting after p and blocks whose pool index is out of range are
// skipped).  The blocks are split over the NT/64 waves of the workgroup
// (split-K), whose states are merged through LDS; every thread calls it.
// kStream as for load_block_tiles.
//   k_pool, v_pool : [num_blocks][heads][32][128] bf16;  table : the
//   sequence's block-table row;  q_head : the head's 128 query dims;
//   out_head : 128 floats;  lse_out : one float or null (natural log).
template <int NT, bool kStream>
__device__ __forceinline__ void attend_query_wg(const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* table,
                                                int64_t num_blocks, int heads, int h, int max_blocks, int p,
                                                const uint16_t* q_head, const int32_t* sel, int topk,
                                                float scale_log2, float* out_head, float* lse_out,
                                                AttendSmem<NT>& sm) {
  WaveAttn st;
  wave_attn_init(st, q_head);
  wave_attn_sel<NT, kStream>(k_pool, v_pool, table, num_blocks, heads, h, max_blocks, p, sel, topk, scale_log2, st);
  wave_attn_finish<NT>(st, out_head, lse_out, sm);
}

}  // namespace uocr
