// Chunked-prefill indexer scoring on bf16 MFMA with fused block max and
// per-split partial selection (SR-SWA steps 2-3 for T query rows,
// news.rkmt.cn/news/25027 Sec. 5; leheavengame.com OCR 2 release article,
// Sec. 3, on the [tokens, context/32] temporary that this kernel avoids).
//
// The indexer product [T x 128] . [128 x keys] is a real dense contraction.
// Work is tiled as 256 query rows x one context split per workgroup (4 waves,
// 64 rows each).  Per 32-key block the workgroup stages the 8 KB indexer tile
// in LDS (rows padded to 272 B, double-buffered); each wave multiplies it with
// its two resident 32-row query tiles using v_mfma_f32_32x32x16_bf16 with the
// keys on the M axis and the queries on N.  A lane then holds 16 of the 32
// key scores of one query column, so the block max is 16 in-lane maxima and
// one exchange with lane l^32.  Blocks beyond a row's causal candidate limit
// (j <= (q_start+t)/32 - local) are skipped per row.  Each lane keeps a
// sorted list of its row's best (topk - local) blocks of the split; only
// those lists are written, never the [T, context/32] score matrix.
//
// The 128-dim contraction is split into 8 MFMA steps of 16; lane half h of an
// operand covers dims 64h + 8s .. +8 in step s for both A and B, a consistent
// permutation of the summation order that lets every lane read 128
// contiguous bytes.
#include "device_common.h"
#include "kernels.h"

namespace uocr {

namespace {
constexpr int kPfThreads = 256;
constexpr int kPfRows = 256;       // query rows per workgroup
constexpr int kLdsRow = 272;       // bytes per staged key row (256 + 16 pad)
constexpr int kLdsTile = kBlock * kLdsRow;
}  // namespace

template <int R>
__global__ __launch_bounds__(kPfThreads) void indexer_prefill_kernel(IndexerPrefillArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kLdsTile];

  const PrefillPlan P = a.plan;
  // XCD-aware order: workgroup i runs on XCD i % 8; the row tiles of a split
  // are consecutive on one XCD so the split's keys come from one L2.
  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  const int slot = wg >> 3;
  const int group = slot / P.n_tiles;
  const int tile = slot - group * P.n_tiles;
  const int split = group * 8 + xcd;
  if (split >= P.nsplit) return;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int h = lane >> 5;
  const int n = lane & 31;

  const int t0 = tile * kPfRows;
  const int t_own = t0 + wave * 64 + h * 32 + n;  // row whose list this lane keeps
  const bool row_ok = t_own < a.T;
  const int lim_own = row_ok ? (a.q_start + t_own) / kBlock - a.local_blocks : -1;
  const int t_last = min(t0 + kPfRows - 1, a.T - 1);
  const int lim_wg = (a.q_start + t_last) / kBlock - a.local_blocks;
  const int jb = split * P.bps;
  const int je = min(min(jb + P.bps, lim_wg + 1), a.max_blocks);

  uint32_t lk[R];
  int32_t li[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    lk[r] = 0u;
    li[r] = -1;
  }

  if (jb < je) {
    // Resident query fragments: tile c, step s -> dims 64h + 8s .. +8 of row
    // t0 + 64*wave + 32c + n (rows past T read row T-1 and are never kept).
    uint4 qf[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int t = min(t0 + wave * 64 + c * 32 + n, a.T - 1);
      const uint4* src = reinterpret_cast<const uint4*>(a.q_idx + (int64_t)t * kDim + 64 * h);
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[c][s] = src[s];
    }

    // Staging: thread tid moves uint4 numbers tid and 256 + tid of the 8 KB
    // tile into the padded LDS rows.
    const int st0 = (tid >> 4) * kLdsRow + (tid & 15) * 16;
    const int st1 = ((256 + tid) >> 4) * kLdsRow + (tid & 15) * 16;
    uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0;
    bool ok_cur;
    {
      const int pb = __builtin_amdgcn_readfirstlane(a.block_table[jb]);
      ok_cur = pb >= 0 && (int64_t)pb < a.num_blocks;
      if (ok_cur) {
        const uint4* src = reinterpret_cast<const uint4*>(a.kidx_pool + (int64_t)pb * (kBlock * kDim));
        x0 = src[tid];
        x1 = src[256 + tid];
      }
      *reinterpret_cast<uint4*>(lds + st0) = x0;
      *reinterpret_cast<uint4*>(lds + st1) = x1;
    }
    __syncthreads();

    for (int j = jb; j < je; ++j) {
      const int buf = (j - jb) & 1;
      bool ok_next = false;
      if (j + 1 < je) {
        const int pb = __builtin_amdgcn_readfirstlane(a.block_table[j + 1]);
        ok_next = pb >= 0 && (int64_t)pb < a.num_blocks;
        if (ok_next) {
          const uint4* src = reinterpret_cast<const uint4*>(a.kidx_pool + (int64_t)pb * (kBlock * kDim));
          x0 = src[tid];
          x1 = src[256 + tid];
        } else {
          x0 = make_uint4(0, 0, 0, 0);
          x1 = x0;
        }
      }

      // A fragments: key n, dims 64h + 8s .. +8.
      const unsigned char* at = lds + buf * kLdsTile + n * kLdsRow + h * 128;
      f32x16_t acc0 = {0}, acc1 = {0};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 av = *reinterpret_cast<const uint4*>(at + s * 16);
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8_t, qf[0][s]), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8_t, qf[1][s]), acc1, 0, 0, 0);
      }
      float pm0 = acc0[0], pm1 = acc1[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        pm0 = fmaxf(pm0, acc0[r]);
        pm1 = fmaxf(pm1, acc1[r]);
      }
      // Lane l (h=0) owns tile 0's column n, lane l+32 owns tile 1's; each
      // hands the other the partial max it needs.
      const float send = h ? pm0 : pm1;
      const float recv = shfl_xor_f32(send, 32);
      float bsc = fmaxf(h ? pm1 : pm0, recv);
      if (!ok_cur) bsc = __builtin_nanf("");
      const uint32_t key = order_key(bsc);
      const bool valid = j <= lim_own;  // false for rows past T (lim_own = -1)
      if (valid && (key > lk[R - 1] || li[R - 1] < 0)) {
        // Sorted insertion (descending key, equal keys keep the earlier id):
        // slot r takes the new entry if it beats slot r but not slot r-1, and
        // slot r-1's entry if it beats both.
#pragma unroll
        for (int r = R - 1; r >= 0; --r) {
          const bool b_r = key > lk[r] || li[r] < 0;
          if (r > 0) {
            const bool b_prev = key > lk[r - 1] || li[r - 1] < 0;
            if (b_r) {
              lk[r] = b_prev ? lk[r - 1] : key;
              li[r] = b_prev ? li[r - 1] : j;
            }
          } else if (b_r) {
            lk[0] = key;
            li[0] = j;
          }
        }
      }

      if (j + 1 < je) {
        unsigned char* nb = lds + (buf ^ 1) * kLdsTile;
        *reinterpret_cast<uint4*>(nb + st0) = x0;
        *reinterpret_cast<uint4*>(nb + st1) = x1;
      }
      ok_cur = ok_next;
      __syncthreads();
    }
  }

  if (row_ok) {
    const size_t off = ((size_t)t_own * P.nsplit + split) * R;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      a.cand_keys[off + r] = lk[r];
      a.cand_idx[off + r] = li[r];
    }
  }
}

PrefillPlan prefill_plan(int32_t T, int32_t max_blocks, int32_t topk, int32_t local_blocks) {
  PrefillPlan p{};
  p.R = topk - local_blocks;
  p.n_tiles = (T + kPfRows - 1) / kPfRows;
  if (T <= 0 || p.R <= 0) {
    p.bps = max_blocks;
    p.nsplit = 1;
    p.ws_bytes = 0;
    return p;
  }
  // ~512 workgroups, at least 16 blocks per split, at most 64 splits.
  int64_t bps = ((int64_t)max_blocks * p.n_tiles + 511) / 512;
  if (bps < 16) bps = 16;
  const int64_t min_bps = ((int64_t)max_blocks + 63) / 64;
  if (bps < min_bps) bps = min_bps;
  p.bps = (int32_t)bps;
  p.nsplit = (int32_t)(((int64_t)max_blocks + bps - 1) / bps);
  const size_t n = (size_t)T * (size_t)p.nsplit * (size_t)p.R;
  p.ws_bytes = prefill_idx_offset(p, T) + n * sizeof(int32_t);
  return p;
}

hipError_t launch_indexer_prefill(const IndexerPrefillArgs& a, hipStream_t stream) {
  const PrefillPlan& P = a.plan;
  if (a.T == 0 || P.R <= 0) return hipSuccess;
  const int nsplit_pad = (P.nsplit + 7) / 8 * 8;
  dim3 grid(P.n_tiles * nsplit_pad);
  switch (P.R) {
#define UOCR_CASE(RR) \
  case RR: hipLaunchKernelGGL(indexer_prefill_kernel<RR>, grid, dim3(kPfThreads), 0, stream, a); break;
    UOCR_CASE(1) UOCR_CASE(2) UOCR_CASE(3) UOCR_CASE(4) UOCR_CASE(5) UOCR_CASE(6) UOCR_CASE(7) UOCR_CASE(8)
    UOCR_CASE(9) UOCR_CASE(10) UOCR_CASE(11) UOCR_CASE(12) UOCR_CASE(13) UOCR_CASE(14) UOCR_CASE(15)
    UOCR_CASE(16)
#undef UOCR_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of the per-split lists (SR-SWA step 3 for prefill rows): one wave per
// row, lane s holds split s's sorted list; R rounds of a wave-wide arg-max on
// the composite (key, -id) pick the remote blocks in rank order, which are
// then written ascending, followed by the row's local window.
// ---------------------------------------------------------------------------

template <int R>
__global__ __launch_bounds__(256) void topk_prefill_kernel(TopkPrefillArgs a) {
  const PrefillPlan P = a.plan;
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= a.T) return;
  const int p = a.q_start + t;
  const int nb = p / kBlock + 1;
  const int ncand = nb - a.local_blocks > 0 ? nb - a.local_blocks : 0;
  int32_t* out = a.block_idx + (int64_t)t * a.topk;
  if (a.n_sel != nullptr && lane == 0) a.n_sel[t] = nb < a.topk ? nb : a.topk;
  if (ncand <= R) {
    for (int i = lane; i < a.topk; i += kWave) out[i] = i < nb ? i : -1;
    return;
  }

  if constexpr (R > 0) {
  uint32_t lk[R];
  int32_t li[R];
  const size_t off = ((size_t)t * P.nsplit + lane) * R;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool have = lane < P.nsplit;
    lk[r] = have ? a.cand_keys[off + r] : 0u;
    li[r] = have ? a.cand_idx[off + r] : -1;
  }

  int32_t mine = -1;  // lane w keeps the w-th winner
#pragma unroll
  for (int w = 0; w < R; ++w) {
    // Composite rank key: (score key, 0xFFFFFFFF - id); empty slot = (0, 0).
    uint32_t hi = li[0] >= 0 ? lk[0] : 0u;
    uint32_t lo = li[0] >= 0 ? 0xFFFFFFFFu - (uint32_t)li[0] : 0u;
    const uint32_t my_hi = hi, my_lo = lo;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const uint32_t ohi = __shfl_xor(hi, m, kWave);
      const uint32_t olo = __shfl_xor(lo, m, kWave);
      const bool take = ohi > hi || (ohi == hi && olo > lo);
      hi = take ? ohi : hi;
      lo = take ? olo : lo;
    }
    if (hi == 0u && lo == 0u) break;
    const int32_t id = (int32_t)(0xFFFFFFFFu - lo);
    if (lane == w) mine = id;
    if (my_hi == hi && my_lo == lo) {
#pragma unroll
      for (int r = 0; r + 1 < R; ++r) {
        lk[r] = lk[r + 1];
        li[r] = li[r + 1];
      }
      lk[R - 1] = 0u;
      li[R - 1] = -1;
    }
  }

  // Ascending order of the R winners: rank by counting smaller ids.
  int rank = 0;
  for (int v = 0; v < R; ++v) {
    const int32_t other = __shfl(mine, v, kWave);
    rank += (other < mine) ? 1 : 0;
  }
  if (lane < R && mine >= 0) out[rank] = mine;
  }
  for (int i = lane; i < a.local_blocks; i += kWave) out[R + i] = ncand + i;
}

hipError_t launch_topk_prefill(const TopkPrefillArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  dim3 grid((a.T + 3) / 4);
  switch (a.plan.R) {
#define UOCR_CASE(RR) \
  case RR: hipLaunchKernelGGL(topk_prefill_kernel<RR>, grid, dim3(256), 0, stream, a); break;
    UOCR_CASE(0) UOCR_CASE(1) UOCR_CASE(2) UOCR_CASE(3) UOCR_CASE(4) UOCR_CASE(5) UOCR_CASE(6) UOCR_CASE(7)
    UOCR_CASE(8) UOCR_CASE(9) UOCR_CASE(10) UOCR_CASE(11) UOCR_CASE(12) UOCR_CASE(13) UOCR_CASE(14)
    UOCR_CASE(15) UOCR_CASE(16)
#undef UOCR_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace uocr
