// Register-resident top-k block selection shared by the decode selection
// kernel and the fused selection + attention kernel (SR-SWA step 3,
// news.rkmt.cn/news/25027 Sec. 5): keep a query's local blocks and the
// (topk - local) highest-scoring remote candidates, ranked by score
// descending with the lower block id first on ties.
#pragma once

#include "device_common.h"

namespace uocr {

template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  constexpr int kWaves = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  v = (uint32_t)wave_incl_sum((int)v);
  if (lane == kWave - 1) scratch[wave] = v;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    uint32_t s = scratch[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// Trivial selections of a query with nb blocks: every block when there are
// no more candidates than remote slots, only the local window when there are
// no remote slots.  Writes out[0 .. topk) and returns true in those cases.
__device__ __forceinline__ bool select_trivial(int nb, int ncand, int R, int topk, int32_t* out, int nt) {
  const int tid = threadIdx.x;
  if (ncand <= R) {
    // Every block 0..nb-1 is kept (remote candidates then the local window).
    for (int i = tid; i < topk; i += nt) out[i] = i < nb ? i : -1;
    return true;
  }
  if (R == 0) {
    for (int i = tid; i < topk; i += nt) out[i] = ncand + i;
    return true;
  }
  return false;
}

// ---------------------------------------------------------------------------
// Fast variant: NT threads, up to KPT candidate keys per thread in registers.
//
//  1. keys are loaded once, branch-free (one memory round trip);
//  2. radix pass on the top byte: nearly every key of a score distribution
//     shares one or two top bytes, so each wave counts one digit at a time
//     (a uniform loop over the distinct digits it holds) and adds one wave
//     sum per digit instead of 64 serialised same-address LDS adds;
//  3. radix pass on the second byte among keys with the chosen top byte
//     (spread digits: plain LDS adds);
//  4. keys above the 16-bit prefix are kept; keys sharing it ("maybe", few)
//     are ranked exactly by (key desc, id asc) with one counting pass; the
//     kept ids are put in ascending order by counting.
// When too many keys share the 16-bit prefix (heavy exact ties), or R is
// large, it finishes with the two remaining radix passes and an ordered
// compaction instead.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
  v = sum_xor16_u32(v);
  v = sum_xor32_u32(v);
  return v;
}

// Wave 0 finds the digit holding the `remaining`-th largest key from the
// 256-bin histogram (bins scanned from the top digit down).
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t remaining, uint32_t* s_digit,
                                           uint32_t* s_remaining) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    // lane holds digits 255-4*lane .. 252-4*lane (descending)
    uint32_t c[4];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = hist[255 - 4 * lane - i];
      sum += c[i];
    }
    const uint32_t incl = (uint32_t)wave_incl_sum((int)sum);
    uint32_t cum = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t nc = cum + c[i];
      if (nc >= remaining && cum < remaining) {
        *s_digit = 255u - 4u * lane - i;
        *s_remaining = remaining - cum;
      }
      cum = nc;
    }
  }
}


// Working storage of select_sorted_reg (LDS).
template <int NT>
struct SelectSmem {
  static constexpr int kCap = 512;
  uint32_t hist[256];
  uint32_t scan_scratch[NT / kWave];
  uint32_t s_digit, s_remaining, s_nin, s_nmaybe;
  int32_t s_sel[kCap];
  uint64_t s_maybe[kCap];
};

// Non-trivial case (ncand > R >= 1): writes the R remote ids ascending, then
// the local window, into out[0 .. R + local_blocks).  `out` may point to
// global or LDS memory.  Every thread of the NT-thread workgroup calls it.
// With page tags (`tags` not null; news.rkmt.cn/news/25027 Sec. 5, the
// page-aware candidate constraint) a candidate's tier -- 1 when its tag
// equals `qpage` -- takes the top bit of its ranking key and the score's
// order key the 31 bits below, so the query's page's blocks rank first.
// kCoherent: the scores were written by other workgroups of the same launch
// (device-scope stores) and are read with device-scope loads, which need no
// cache invalidation before them.
template <int NT, int KPT, bool kCoherent = false>
__device__ __forceinline__ void select_sorted_reg(const float* sc, int ncand, int R, int local_blocks, int32_t* out,
                                                  SelectSmem<NT>& sm, const int32_t* tags = nullptr,
                                                  int32_t qpage = 0) {
  constexpr int kCap = SelectSmem<NT>::kCap;
  uint32_t* hist = sm.hist;
  uint32_t* scan_scratch = sm.scan_scratch;
  uint32_t& s_digit = sm.s_digit;
  uint32_t& s_remaining = sm.s_remaining;
  uint32_t& s_nin = sm.s_nin;
  uint32_t& s_nmaybe = sm.s_nmaybe;
  int32_t* s_sel = sm.s_sel;
  uint64_t* s_maybe = sm.s_maybe;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  uint32_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = tid + i * NT;
    const float* src = sc + (j < ncand ? j : ncand - 1);
    key[i] = kCoherent ? __hip_atomic_load(reinterpret_cast<const uint32_t*>(src), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)
                       : __float_as_uint(*src);
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = (tid + i * NT < ncand) ? order_key(__uint_as_float(key[i])) : 0u;
  if (tags != nullptr) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = tid + i * NT;
      const bool tier = tags[j < ncand ? j : ncand - 1] == qpage;
      key[i] = tier ? (0x80000000u | (key[i] >> 1)) : (key[i] >> 1);
    }
  }

  // ---- pass A: top byte, one wave sum per distinct digit -------------------
  if (tid < 256) hist[tid] = 0;
  if (tid == 0) {
    s_nin = 0;
    s_nmaybe = 0;
  }
  __syncthreads();
  {
    static_assert(KPT <= 64, "pending holds one bit per key of the thread");
    uint64_t pending = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) pending |= (tid + i * NT < ncand) ? (1ull << i) : 0ull;
    while (__ballot(pending != 0) != 0) {
      const uint64_t act = __ballot(pending != 0);
      const int leader = __builtin_ctzll(act);
      uint32_t first = 0;
#pragma unroll
      for (int i = KPT - 1; i >= 0; --i)
        if (pending & (1ull << i)) first = key[i] >> 24;
      const uint32_t d = __builtin_amdgcn_readlane(first, leader);
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool hit = (pending & (1ull << i)) && (key[i] >> 24) == d;
        cnt += hit ? 1u : 0u;
        pending &= hit ? ~(1ull << i) : ~0ull;
      }
      cnt = wave_sum_u32(cnt);
      if (lane == 0) atomicAdd(&hist[d], cnt);
    }
  }
  __syncthreads();
  find_digit<NT>(hist, (uint32_t)R, &s_digit, &s_remaining);
  __syncthreads();
  const uint32_t dA = s_digit;
  const uint32_t remA = s_remaining;
  __syncthreads();

  // ---- pass B: second byte among keys with top byte dA ---------------------
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (tid + i * NT < ncand && (key[i] >> 24) == dA) atomicAdd(&hist[(key[i] >> 16) & 255u], 1u);
  }
  __syncthreads();
  find_digit<NT>(hist, remA, &s_digit, &s_remaining);
  __syncthreads();
  const uint32_t P16 = (dA << 8) | s_digit;  // top 16 bits of the cutoff key
  const uint32_t rem16 = s_remaining;           // slots left for keys with prefix P16

  // ---- gather: keys above the prefix are in; keys on it are ranked ---------
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = tid + i * NT;
    if (j < ncand) {
      const uint32_t hi = key[i] >> 16;
      if (hi > P16) {
        const uint32_t pos = atomicAdd(&s_nin, 1u);  // exactly R - rem16 of them
        if (pos < (uint32_t)kCap) s_sel[pos] = j;
      } else if (hi == P16) {
        const uint32_t pos = atomicAdd(&s_nmaybe, 1u);
        if (pos < (uint32_t)kCap) s_maybe[pos] = ((uint64_t)key[i] << 32) | (0xFFFFFFFFu - (uint32_t)j);
      }
    }
  }
  __syncthreads();
  const uint32_t nin = s_nin;
  const uint32_t nmaybe = s_nmaybe;
  if (R <= kCap && nmaybe <= (uint32_t)kCap) {
    for (uint32_t e = tid; e < nmaybe; e += NT) {
      const uint64_t my = s_maybe[e];
      uint32_t r = 0;
      for (uint32_t k = 0; k < nmaybe; ++k) r += s_maybe[k] > my ? 1u : 0u;
      if (r < rem16) s_sel[nin + r] = (int32_t)(0xFFFFFFFFu - (uint32_t)my);
    }
    __syncthreads();
    for (int r = tid; r < R; r += NT) {
      const int32_t my = s_sel[r];
      int pos = 0;
      for (int k = 0; k < R; ++k) pos += s_sel[k] < my ? 1 : 0;
      out[pos] = my;
    }
  } else {
    // ---- fallback: radix passes on bytes 1 and 0, ordered compaction -------
    uint32_t prefix = P16 << 16, prefix_mask = 0xFFFF0000u, remaining = rem16;
#pragma unroll
    for (int pass = 2; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (tid + i * NT < ncand && (key[i] & prefix_mask) == prefix)
          atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
      }
      __syncthreads();
      find_digit<NT>(hist, remaining, &s_digit, &s_remaining);
      __syncthreads();
      prefix |= s_digit << shift;
      prefix_mask |= 255u << shift;
      remaining = s_remaining;
      __syncthreads();
    }
    const uint32_t T = prefix;
    const uint32_t need_eq = remaining;
    uint32_t eq_seen = 0, taken = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = tid + i * NT;
      const bool in = j < ncand;
      const uint32_t eq = (in && key[i] == T) ? 1u : 0u;
      uint32_t eq_total;
      const uint32_t eq_incl = block_incl_scan<NT>(eq, scan_scratch, &eq_total);
      const uint32_t eq_before = eq_seen + eq_incl - eq;
      const uint32_t take = (in && (key[i] > T || (eq && eq_before < need_eq))) ? 1u : 0u;
      uint32_t take_total;
      const uint32_t take_incl = block_incl_scan<NT>(take, scan_scratch, &take_total);
      const uint32_t pos = taken + take_incl - 1;
      if (take && pos < (uint32_t)R) out[pos] = j;
      eq_seen += eq_total;
      taken += take_total;
    }
  }
  // Local window after the remote ids (all larger than every candidate).
  for (int i = tid; i < local_blocks; i += NT) out[R + i] = ncand + i;
}

}  // namespace uocr
