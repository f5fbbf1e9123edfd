// Chunked-prefill indexer scoring on bf16 MFMA with fused block max and
// per-split partial selection (SR-SWA steps 2-3 for T query rows,
// news.rkmt.cn/news/25027 Sec. 5; leheavengame.com OCR 2 release article,
// Sec. 3, on the [tokens, context/32] temporary that this kernel avoids).
//
// The indexer product [T x 128] . [128 x keys] is a real dense contraction.
// Work is tiled as 256 query rows x one context split per workgroup (4 waves,
// 64 rows each).  Per 32-key block the workgroup stages the 8 KB indexer tile
// in LDS (rows padded to 272 B, two buffers, fetched three blocks ahead);
// each wave multiplies it with
// its two resident 32-row query tiles using v_mfma_f32_32x32x16_bf16 with the
// keys on the M axis and the queries on N.  A lane then holds 16 of the 32
// key scores of one query column, so the block max is 16 in-lane maxima and
// one permlane32 swap.  The loop is software-pipelined: block j+1's products
// are issued before block j's epilogue (two accumulator sets), so matrix and
// vector work of one wave overlap.  Blocks beyond a row's causal candidate limit
// (j <= (q_start+t)/32 - local) are skipped per row.  Each lane keeps a
// sorted list of its row's best (topk - local) blocks of the split; only
// those lists are written, never the [T, context/32] score matrix.
//
// A list entry packs the block score's 32-bit order key with its low idbits
// replaced by the (complemented) in-split block index.  Ranking therefore
// uses scores truncated to 2^-(23 - idbits) relative (2^-17 at 128K
// context), equal truncated scores going to the lower block id.  Entries are
// unique, so a sorted insertion is one min and one max per slot.
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

// Candidate key of a block score: the order-preserving key, at least 1, so
// that an empty list slot (key 0) ranks below every block, NaN included.
__device__ __forceinline__ uint32_t cand_key(float f) {
  const uint32_t k = order_key(f);
  return k > 1u ? k : 1u;
}

// A fragments of one staged key tile: key n, dims 64h + 8s .. +8 (s = 0..7).
__device__ __forceinline__ void read_a(const unsigned char* tile, int n, int h, uint4 (&a)[8]) {
  const unsigned char* at = tile + n * kLdsRow + h * 128;
#pragma unroll
  for (int s = 0; s < 8; ++s) a[s] = *reinterpret_cast<const uint4*>(at + s * 16);
}

__device__ __forceinline__ void mfma_block(const uint4 (&a)[8], const uint4 (&qf)[2][8], f32x16_t& acc0,
                                           f32x16_t& acc1) {
  acc0 = f32x16_t{0};
  acc1 = f32x16_t{0};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a[s]);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8_t, qf[0][s]), acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, __builtin_bit_cast(bf16x8_t, qf[1][s]), acc1, 0, 0, 0);
  }
}

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

  // Sorted list of this lane's row: packed keys descending, empty slots 0.
  uint32_t lk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) lk[r] = 0u;

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

    // Staging: thread tid moves uint4 numbers tid and 256 + tid of an 8 KB
    // key tile into the padded rows of one of two LDS buffers.  Tiles are
    // fetched into a four-slot register ring three blocks before they are
    // staged, so about three blocks of matrix work hide each fetch.
    const int st0 = (tid >> 4) * kLdsRow + (tid & 15) * 16;
    const int st1 = ((256 + tid) >> 4) * kLdsRow + (tid & 15) * 16;
    // Branch-free fetch (an invalid pool index reads pool block 0 and is
    // flagged), so the number of loads in flight is the same on every path
    // and the wait before staging only covers the block being staged.
#define UOCR_FETCH(jj, Y0, Y1, OK)                                                                        \
  do {                                                                                                    \
    const int pb_ = __builtin_amdgcn_readfirstlane(a.block_table[(jj)]);                                  \
    OK = pb_ >= 0 && (int64_t)pb_ < a.num_blocks;                                                         \
    const uint4* src_ = reinterpret_cast<const uint4*>(a.kidx_pool + (int64_t)(OK ? pb_ : 0) * (kBlock * kDim)); \
    Y0 = src_[tid];                                                                                       \
    Y1 = src_[256 + tid];                                                                                 \
  } while (0)
#define UOCR_STAGE(BUF, Y0, Y1)                                                        \
  do {                                                                                 \
    unsigned char* dst_ = lds + (BUF) * kLdsTile;                                      \
    *reinterpret_cast<uint4*>(dst_ + st0) = Y0;                                        \
    *reinterpret_cast<uint4*>(dst_ + st1) = Y1;                                        \
  } while (0)

    // Bit (k mod 64) of `okbits` says whether block jb + k has a valid pool
    // index; it is written when the block is fetched and read at its epilogue.
    uint64_t okbits = 0;
    uint4 r0a, r0b, r1a, r1b, r2a, r2b, r3a, r3b;
    {
      uint4 t0, t1;
      bool ok;
      UOCR_FETCH(jb, t0, t1, ok);
      okbits |= ok ? 1ull : 0ull;
      UOCR_STAGE(0, t0, t1);
      UOCR_FETCH(min(jb + 1, je - 1), t0, t1, ok);
      okbits |= ok ? 2ull : 0ull;
      UOCR_STAGE(1, t0, t1);
      // Fetches past the split re-read its last block; they are never used.
      UOCR_FETCH(min(jb + 2, je - 1), r2a, r2b, ok);
      okbits |= ok ? 4ull : 0ull;
      UOCR_FETCH(min(jb + 3, je - 1), r3a, r3b, ok);
      okbits |= ok ? 8ull : 0ull;
      UOCR_FETCH(min(jb + 4, je - 1), r0a, r0b, ok);
      okbits |= ok ? 16ull : 0ull;
    }
    __syncthreads();

    uint4 av[8];
    f32x16_t accA0, accA1, accB0, accB1;
    read_a(lds, n, h, av);
    mfma_block(av, qf, accA0, accA1);

    int j = jb;
    // One block: fetch block j+5 into ring slot (j+5)%4, issue block j+1's
    // products, run block j's epilogue, stage block j+2 from ring slot
    // (j+2)%4 into LDS buffer j%2.  Block j+1's products come first (on the
    // last block they recompute a staged tile and are never read), in one
    // branch-free region with block j's epilogue so that the scheduler can
    // interleave the matrix instructions with the vector ones.
#define UOCR_STEP(LDA, LDB, STA, STB, BUF_MFMA, BUF_STAGE, CUR0, CUR1, NXT0, NXT1)                       \
  do {                                                                                                    \
    const int k_ = j - jb;                                                                                \
    {                                                                                                     \
      bool okf_;                                                                                          \
      UOCR_FETCH(min(j + 5, je - 1), LDA, LDB, okf_);                                                    \
      const uint64_t bit_ = 1ull << ((k_ + 5) & 63); /* reused 64 blocks later only */                    \
      okbits = okf_ ? (okbits | bit_) : (okbits & ~bit_);                                                 \
    }                                                                                                     \
    read_a(lds + (BUF_MFMA) * kLdsTile, n, h, av);                                                        \
    mfma_block(av, qf, NXT0, NXT1);                                                                       \
    epilogue(CUR0, CUR1, ((okbits >> (k_ & 63)) & 1ull) != 0);                                            \
    _Pragma("unroll") for (int i_ = 0; i_ < 16; ++i_) {                                                   \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* one MFMA */                                   \
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0); /* then up to five VALU */                       \
    }                                                                                                     \
    if (j + 2 < je) UOCR_STAGE(BUF_STAGE, STA, STB);                                                     \
    __syncthreads();                                                                                      \
    ++j;                                                                                                  \
  } while (0)

    // Block max, candidate key and sorted insertion of block j for this lane's row.
    auto epilogue = [&](const f32x16_t& cur0, const f32x16_t& cur1, bool ok) __attribute__((always_inline)) {
      float pm0 = cur0[0], pm1 = cur1[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        pm0 = fmaxf(pm0, cur0[r]);
        pm1 = fmaxf(pm1, cur1[r]);
      }
      // Lanes 0-31 end with tile 0's block max of column n, lanes 32-63 with
      // tile 1's: permlane32_swap pairs each half with the other half.
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm0), __float_as_uint(pm1), false, false);
      float bsc = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      if (!ok) bsc = __builtin_nanf("");
      // Packed candidate: order bits of the score above `idbits`, the
      // in-split index below (complemented, so the lower block id ranks first
      // among equal truncated scores).  Packed keys of one split are distinct,
      // so inserting into the sorted list is new[r] = med3(L[r], L[r-1], k).
      const uint32_t key = cand_key(bsc);
      const uint32_t idmask = (1u << P.idbits) - 1u;
      const uint32_t kbase = key > idmask ? key : idmask + 1u;  // NaN (key 1) stays above empty
      uint32_t kp = (kbase & ~idmask) | (idmask - (uint32_t)(j - jb));
      kp = j <= lim_own ? kp : 0u;  // rows past T have lim_own = -1
#pragma unroll
      for (int r = R - 1; r > 0; --r) lk[r] = max(lk[r], min(lk[r - 1], kp));
      lk[0] = max(lk[0], kp);
    };

    // Ring slot of block jb + m is m % 4; LDS buffer is m % 2.
    while (true) {
      UOCR_STEP(r1a, r1b, r2a, r2b, 1, 0, accA0, accA1, accB0, accB1);  // m = 0 mod 4
      if (j >= je) break;
      UOCR_STEP(r2a, r2b, r3a, r3b, 0, 1, accB0, accB1, accA0, accA1);  // m = 1
      if (j >= je) break;
      UOCR_STEP(r3a, r3b, r0a, r0b, 1, 0, accA0, accA1, accB0, accB1);  // m = 2
      if (j >= je) break;
      UOCR_STEP(r0a, r0b, r1a, r1b, 0, 1, accB0, accB1, accA0, accA1);  // m = 3
      if (j >= je) break;
    }
#undef UOCR_STEP
#undef UOCR_STAGE
#undef UOCR_FETCH
  }

  if (row_ok) {
    const size_t off = ((size_t)t_own * P.nsplit + split) * R;
#pragma unroll
    for (int r = 0; r < R; ++r) a.cand_keys[off + r] = lk[r];
  }
}

PrefillPlan prefill_plan(int32_t T, int32_t max_blocks, int32_t topk, int32_t local_blocks) {
  PrefillPlan p{};
  p.R = topk - local_blocks;
  p.n_tiles = (T + kPfRows - 1) / kPfRows;
  if (T <= 0 || p.R <= 0) {
    p.bps = max_blocks;
    p.nsplit = 1;
    p.idbits = 1;
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
  p.idbits = 1;
  while ((1 << p.idbits) < p.bps) ++p.idbits;
  p.ws_bytes = (size_t)T * (size_t)p.nsplit * (size_t)p.R * sizeof(uint32_t);
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
  // Lane s holds split s's list, decoded into (truncated score, id) pairs.
  const uint32_t idmask = (1u << P.idbits) - 1u;
  uint32_t lk[R];
  int32_t li[R];
  const size_t off = ((size_t)t * P.nsplit + lane) * R;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t kp = lane < P.nsplit ? a.cand_keys[off + r] : 0u;
    lk[r] = kp >> P.idbits;  // >= 1 for every real candidate
    li[r] = kp != 0u ? lane * P.bps + (int32_t)(idmask - (kp & idmask)) : -1;
  }

  int32_t mine = -1;  // lane w keeps the w-th winner
#pragma unroll
  for (int w = 0; w < R; ++w) {
    // Composite rank key: (truncated score, 0xFFFFFFFF - id); empty = (0, 0).
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
