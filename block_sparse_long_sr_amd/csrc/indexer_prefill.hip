// Chunked-prefill indexer scoring on bf16 MFMA with fused block max and
// per-split partial selection (SR-SWA steps 2-3 for T query rows,
// news.rkmt.cn/news/25027 Sec. 5; leheavengame.com OCR 2 release article,
// Sec. 3, on the [tokens, context/32] temporary that this kernel avoids).
//
// The indexer product [T x 128] . [128 x keys] is a real dense contraction.
// Work is tiled as 512 query rows x one context split per workgroup of 8
// waves, two per SIMD; each wave holds two 32-row query tiles in registers.
// Each 32-key block's 8 KB indexer tile is copied from memory straight into
// one of eight LDS buffers (global_load_lds, six blocks ahead, 1 KB per
// wave); each wave multiplies it with its query tiles using
// v_mfma_f32_32x32x16_bf16 with the keys on the M axis and the queries on N.
// A lane then holds 16 of the 32 key scores of one query column per tile,
// and the block max is 16 in-lane maxima and one permlane32 swap, after which
// lane half h owns the row of tile h.
//
// The two waves of a SIMD take turns: between consecutive barriers one of
// them issues the products of two blocks (four independent accumulator
// chains) while the other runs the block max and list insertion of the two
// blocks it multiplied before (and reads the A fragments of its next two
// blocks from LDS), so the matrix unit stays busy while the vector unit does
// the epilogue.  Both waves run the same straight-line step, the
// second one barrier behind the first; with a single code path the compiler
// tracks which tile buffer each LDS read depends on and leaves the copies of
// the other buffers in flight.  Blocks beyond a row's causal candidate limit
// (j <= (q_start+t)/32 - local) are skipped per row.  Each lane keeps a
// sorted list of its row's best (topk - local) blocks of the split; only
// those lists are written, never the [T, context/32] score matrix.
//
// A list entry packs the block score's 32-bit order key with its low idbits
// replaced by the (complemented) in-split block index.  Ranking therefore
// uses scores truncated to 2^-(23 - idbits) relative (2^-17 at 128K
// context, one bit less with the page tier in the top bit), equal truncated
// scores going to the lower block id.  Entries are
// unique, so a sorted insertion is one median of three per slot.
//
// The 128-dim contraction is split into 8 MFMA steps of 16; lane half h of an
// operand covers dims 64h + 8s .. +8 in step s for both A and B, a consistent
// permutation of the summation order.  In LDS, key row r keeps its 16-byte
// chunk c at slot c ^ (r mod 16) of a 256-byte row, so that both the copy
// (16 lanes per row) and the A fragment reads (one chunk of 32 rows) are free
// of bank conflicts.
#include "device_common.h"
#include "kernels.h"

namespace uocr {

namespace {
constexpr int kPfThreads = 512;
constexpr int kPfWaves = kPfThreads / kWave;      // 8
constexpr int kPfRows = kPfWaves * 64;            // 512 query rows per workgroup
constexpr int kTileBytes = kBlock * kDim * 2;     // 8 KB indexer tile
constexpr int kMaxBps = 1 << kMaxIdBits;          // blocks per split (pool indices in LDS)
constexpr int kAhead = 6;                         // copies run this many blocks ahead (eight buffers)
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
}  // namespace

// s_waitcnt with only the vector-memory counter limited to n (expcnt and
// lgkmcnt at their maxima, no wait).
#define UOCR_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// s_waitcnt lgkmcnt(0) only.
#define UOCR_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))

__device__ __forceinline__ float max16(const f32x16_t& v) {
  float m = max_keep_nan(max_keep_nan(v[0], v[1]), v[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = max_keep_nan(max_keep_nan(m, v[r]), v[r + 1]);
  return max_keep_nan(m, v[15]);
}

// Insert kp into the descending list lk (unique entries): the new slot r is
// the median of (old slot r-1, kp, old slot r), one v_med3_u32.
template <int R>
__device__ __forceinline__ void insert_sorted(uint32_t (&lk)[R], uint32_t kp) {
#pragma unroll
  for (int r = R - 1; r > 0; --r) lk[r] = max(min(lk[r - 1], kp), min(max(lk[r - 1], kp), lk[r]));
  lk[0] = max(lk[0], kp);
}

// Which of the two waves of its SIMD this wave is (0 or 1, from the order in
// which the waves of the workgroup register).  Only the overlap depends on
// it: either role computes the same results.
__device__ __forceinline__ int simd_turn(uint32_t* counters) {
  // HW_ID bits 5:4 hold the SIMD of the wave.
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
  const uint32_t simd = (hw >> 4) & 3u;
  uint32_t rank = 0;
  if (lane_id() == 0) rank = atomicAdd(&counters[simd], 1u);
  return (int)(__builtin_amdgcn_readfirstlane(rank) & 1u);
}

// The block loop of one workgroup.  The eight tile buffers and the
// pool-index table are separate LDS objects, so the compiler knows that
// reading one buffer does not depend on copies still landing in another and
// leaves those waits to the explicit counts below.  GATE selects the
// page-aware ranking at compile time, keeping its test out of the loop.
template <int R, bool GATE>
__device__ __forceinline__ void prefill_blocks(const IndexerPrefillArgs& a, int jb, int je, int tw, int lim,
                                               int turn, int32_t qpage, lds_u8* __restrict__ B0,
                                               lds_u8* __restrict__ B1, lds_u8* __restrict__ B2,
                                               lds_u8* __restrict__ B3, lds_u8* __restrict__ B4,
                                               lds_u8* __restrict__ B5, lds_u8* __restrict__ B6,
                                               lds_u8* __restrict__ B7, lds_i32* __restrict__ tbl,
                                               lds_i32* __restrict__ tags, const unsigned char* __restrict__ pool,
                                               uint32_t (&lk)[R]) {
  const PrefillPlan& P = a.plan;
  lim = min(lim, je - 1);  // steps past the split's end keep nothing
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int h = lane >> 5;
  const int n = lane & 31;

  for (int i = tid; i < je - jb; i += kPfThreads) {
    tbl[i] = a.block_table[jb + i];
    if (GATE) tags[i] = a.block_page[jb + i];
  }

  // Resident query fragments: tile c, step s -> dims 64h + 8s .. +8 of row
  // tw + 32c + n (rows past T read row T-1 and are never kept).
  bf16x8_t qf[2][8];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int t = min(tw + c * 32 + n, a.T - 1);
    const uint4* src = reinterpret_cast<const uint4*>(a.q_idx + (int64_t)t * kDim + 64 * h);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[c][s] = __builtin_bit_cast(bf16x8_t, src[s]);
  }
  __syncthreads();

  // Copy share of this wave: 1 KB piece `wave` of a tile, i.e. rows
  // 4*wave + lane/16; lane reads the chunk stored at its slot.
  const int crow = 4 * wave + (lane >> 4);
  const uint32_t goff = (uint32_t)(crow * 256 + (((lane & 15) ^ (crow & 15)) * 16));
  const int ldsoff = wave * 1024;
  // A fragment of step s: row n, chunk 8h + s.
  uint32_t raddr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) raddr[s] = (uint32_t)(n * 256 + (((8 * h + s) ^ (n & 15)) * 16));

  // Copy of block jj, whose pool index is PB, into buffer BUF (an invalid
  // pool index copies pool block 0 and is flagged in okbits at bit
  // (jj - jb) mod 64).
  const uint32_t nb32 = a.num_blocks < 0x7FFFFFFF ? (uint32_t)a.num_blocks : 0x7FFFFFFFu;
  uint64_t okbits = 0;
#define UOCR_COPY(jj, BUF, PB)                                                                            \
  do {                                                                                                    \
    const int k_ = (jj) - jb;                                                                             \
    const uint32_t pb_ = (PB);                                                                            \
    const bool ok_ = pb_ < nb32; /* negative indices wrap to large values */                              \
    const unsigned char* src_ = pool + (size_t)(ok_ ? pb_ : 0u) * kTileBytes;                             \
    __builtin_amdgcn_global_load_lds(src_ + goff, (BUF) + ldsoff, 16, 0, 0);                              \
    const uint64_t bit_ = 1ull << (k_ & 63);                                                              \
    okbits = (okbits & ~bit_) | (bit_ & (0ull - (uint64_t)ok_));                                          \
  } while (0)
#define UOCR_POOL_INDEX(jj) ((uint32_t)__builtin_amdgcn_readfirstlane(tbl[(jj) - jb]))
#define UOCR_BARRIER()                     \
  do {                                     \
    __builtin_amdgcn_sched_barrier(0);     \
    asm volatile("" ::: "memory");         \
    __builtin_amdgcn_s_barrier();          \
    asm volatile("" ::: "memory");         \
    __builtin_amdgcn_sched_barrier(0);     \
  } while (0)
#define UOCR_READ_A(AV, BUF)                                                  \
  do {                                                                        \
    _Pragma("unroll") for (int s_ = 0; s_ < 8; ++s_) AV[s_] = *(lds_bf16x8*)((BUF) + raddr[s_]); \
  } while (0)

  bf16x8_t av0[8], av1[8];  // A fragments of the two blocks this wave multiplies next
  f32x16_t c0, c1, c2, c3;  // products of the two blocks it multiplied last

#define UOCR_MFMA2()                                                                                      \
  do {                                                                                                    \
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av0[0], qf[0][0], f32x16_t{0}, 0, 0, 0);               \
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av0[0], qf[1][0], f32x16_t{0}, 0, 0, 0);               \
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av1[0], qf[0][0], f32x16_t{0}, 0, 0, 0);               \
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av1[0], qf[1][0], f32x16_t{0}, 0, 0, 0);               \
    _Pragma("unroll") for (int s_ = 1; s_ < 8; ++s_) {                                                    \
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av0[s_], qf[0][s_], c0, 0, 0, 0);                     \
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av0[s_], qf[1][s_], c1, 0, 0, 0);                     \
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av1[s_], qf[0][s_], c2, 0, 0, 0);                     \
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av1[s_], qf[1][s_], c3, 0, 0, 0);                     \
    }                                                                                                     \
    /* the products belong to this half step: keep them before its barrier */                            \
    asm volatile("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));                                          \
  } while (0)

  // Block max, candidate key and sorted insertion of block JJ for this
  // lane's row from its products (CA, CB) with query tiles 0 and 1.
#define UOCR_EPI(JJ, CA, CB)                                                                              \
  do {                                                                                                    \
    const int jj_ = (JJ);                                                                                 \
    const bool ok_ = ((okbits >> ((jj_ - jb) & 63)) & 1ull) != 0;                                        \
    const auto sw_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(max16(CA)), __float_as_uint(max16(CB)), \
                                                      false, false);                                     \
    float b_ = max_keep_nan(__uint_as_float(sw_[0]), __uint_as_float(sw_[1]));                           \
    b_ = ok_ ? b_ : __builtin_nanf("");                                                                   \
    const uint32_t idmask_ = (1u << P.idbits) - 1u;                                                      \
    uint32_t o_ = order_key(b_);                                                                          \
    if (GATE) { /* page tier in the top bit, the score's order key below it */                           \
      const bool tier_ = tags[jj_ - jb] == qpage;                                                         \
      o_ = tier_ ? (0x80000000u | (o_ >> 1)) : (o_ >> 1);                                                 \
    }                                                                                                     \
    /* empty slots are 0; the order bits are raised to at least idmask + 1 so */                         \
    /* that every candidate, NaN (order key 0) included, stays above empty */                             \
    uint32_t p_ = (max(o_, idmask_ + 1u) & ~idmask_) | (idmask_ - (uint32_t)(jj_ - jb));                 \
    p_ = jj_ <= lim ? p_ : 0u; /* rows past T have lim = -1 */                                            \
    insert_sorted<R>(lk, p_);                                                                             \
    /* the insertion belongs to this half step as well */                                                 \
    _Pragma("unroll") for (int r_ = 0; r_ < R; ++r_) asm volatile("" : "+v"(lk[r_]));                     \
  } while (0)

  // One step for blocks j and j+1, the same for both turns: start the copies
  // of blocks j+6 and j+7 into the buffers that held blocks j-2 and j-1
  // (their pool indices were read from LDS in the previous step), issue the
  // products of blocks j and j+1, barrier; read the A fragments of blocks
  // j+2 and j+3, read the pool indices of blocks j+8 and j+9, run the
  // epilogues of blocks j and j+1, wait for this wave's copies up to block
  // j+5, barrier.  Turn 1 runs one barrier behind turn 0, so each wave's
  // products overlap the other wave's epilogues.  With barriers counted from
  // the prologue's (0) and j = jb + 2k, turn 0 multiplies between barriers 2k
  // and 2k+1 and reads blocks j+2, j+3 after 2k+1; turn 1 multiplies between
  // 2k+1 and 2k+2 and reads after 2k+2.  Every wave has its share of blocks
  // up to j+3 in LDS by barrier 2k+1 (turn 0 waited at 2k, turn 1 at 2k+1),
  // and all reads of blocks j-2 and j-1 complete before barrier 2k-1, before
  // their buffers are refilled after barrier 2k.  Buffer of block jb + i is
  // i % 8.
#define UOCR_STEP(BN0, BN1, BF0, BF1)                                                                     \
  do {                                                                                                    \
    UOCR_COPY(min(j + kAhead, je - 1), BF0, pb0);                                                         \
    UOCR_COPY(min(j + kAhead + 1, je - 1), BF1, pb1);                                                     \
    UOCR_MFMA2();                                                                                         \
    UOCR_WAIT_VM(kAhead - 2);                                                                             \
    UOCR_BARRIER();                                                                                       \
    UOCR_READ_A(av0, BN0);                                                                                \
    UOCR_READ_A(av1, BN1);                                                                                \
    const int32_t t0_ = tbl[min(j + kAhead + 2, je - 1) - jb];                                            \
    const int32_t t1_ = tbl[min(j + kAhead + 3, je - 1) - jb];                                            \
    UOCR_EPI(j, c0, c1);                                                                                  \
    UOCR_EPI(j + 1, c2, c3);                                                                              \
    UOCR_WAIT_VM(kAhead - 4);                                                                             \
    UOCR_WAIT_LGKM0();                                                                                    \
    pb0 = (uint32_t)__builtin_amdgcn_readfirstlane(t0_);                                                  \
    pb1 = (uint32_t)__builtin_amdgcn_readfirstlane(t1_);                                                  \
    UOCR_BARRIER();                                                                                       \
    j += 2;                                                                                               \
  } while (0)

  // Prologue: copies of blocks jb .. jb+5 (copies past the split re-read its
  // last block and are never used); blocks jb .. jb+3 land before the first
  // barrier, after which both turns read the A fragments of blocks jb, jb+1.
  uint32_t pb0 = UOCR_POOL_INDEX(min(jb + kAhead, je - 1));
  uint32_t pb1 = UOCR_POOL_INDEX(min(jb + kAhead + 1, je - 1));
  UOCR_COPY(jb, B0, UOCR_POOL_INDEX(jb));
  UOCR_COPY(min(jb + 1, je - 1), B1, UOCR_POOL_INDEX(min(jb + 1, je - 1)));
  UOCR_COPY(min(jb + 2, je - 1), B2, UOCR_POOL_INDEX(min(jb + 2, je - 1)));
  UOCR_COPY(min(jb + 3, je - 1), B3, UOCR_POOL_INDEX(min(jb + 3, je - 1)));
  UOCR_COPY(min(jb + 4, je - 1), B4, UOCR_POOL_INDEX(min(jb + 4, je - 1)));
  UOCR_COPY(min(jb + 5, je - 1), B5, UOCR_POOL_INDEX(min(jb + 5, je - 1)));
  UOCR_WAIT_VM(kAhead - 4);
  UOCR_BARRIER();
  UOCR_READ_A(av0, B0);
  UOCR_READ_A(av1, B1);
  UOCR_WAIT_LGKM0();
  if (turn != 0) UOCR_BARRIER();

  int j = jb;
  // Whole groups of eight blocks; steps past the split's last block compute
  // on re-read tiles whose keys the row limit (capped at je - 1) discards.
  do {
    UOCR_STEP(B2, B3, B6, B7);
    UOCR_STEP(B4, B5, B0, B1);
    UOCR_STEP(B6, B7, B2, B3);
    UOCR_STEP(B0, B1, B4, B5);
  } while (j < je);
  // Both turns pass the same number of barriers.
  if (turn == 0) UOCR_BARRIER();
  // No copy may still be landing in LDS when the workgroup ends.
  UOCR_WAIT_VM(0);
#undef UOCR_STEP
#undef UOCR_EPI
#undef UOCR_MFMA2
#undef UOCR_READ_A
#undef UOCR_BARRIER
#undef UOCR_POOL_INDEX
#undef UOCR_COPY
}

template <int R, bool GATE>
__global__ __launch_bounds__(kPfThreads, 1) void indexer_prefill_kernel(IndexerPrefillArgs a) {
  // Eight tile buffers as separate objects: the compiler then knows that an
  // LDS read of one buffer never depends on a copy landing in another.
  __shared__ __attribute__((aligned(16))) unsigned char tb0[kTileBytes], tb1[kTileBytes], tb2[kTileBytes],
      tb3[kTileBytes], tb4[kTileBytes], tb5[kTileBytes], tb6[kTileBytes], tb7[kTileBytes];
  __shared__ int32_t s_tbl[kMaxBps];  // pool indices of the split's blocks
  __shared__ int32_t s_tag[kMaxBps];  // page tags of the split's blocks (page-aware ranking)
  __shared__ uint32_t s_turns[4];

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

  if (threadIdx.x < 4) s_turns[threadIdx.x] = 0u;
  __syncthreads();
  const int turn = simd_turn(s_turns);

  const int lane = lane_id();
  const int h = lane >> 5;
  const int n = lane & 31;
  const int t0 = tile * kPfRows;
  const int tw = t0 + wave_id() * 64;  // first row of this wave
  const int row = tw + h * 32 + n;     // row whose list this lane keeps (tile h)
  const int lim = row < a.T ? (a.q_start + row) / kBlock - a.local_blocks : -1;
  const int t_last = min(t0 + kPfRows - 1, a.T - 1);
  const int lim_wg = (a.q_start + t_last) / kBlock - a.local_blocks;
  const int jb = split * P.bps;
  const int je = min(min(jb + P.bps, lim_wg + 1), a.max_blocks);

  // Sorted list of this lane's row: packed keys descending, empty slots 0.
  uint32_t lk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) lk[r] = 0u;
  if (jb < je) {
    const int32_t qpage = (GATE && row < a.T) ? a.row_page[row] : 0;
    prefill_blocks<R, GATE>(a, jb, je, tw, lim, turn, qpage, (lds_u8*)tb0, (lds_u8*)tb1, (lds_u8*)tb2, (lds_u8*)tb3,
                      (lds_u8*)tb4, (lds_u8*)tb5, (lds_u8*)tb6, (lds_u8*)tb7, (lds_i32*)s_tbl, (lds_i32*)s_tag, reinterpret_cast<const unsigned char*>(a.kidx_pool), lk);
  }
  // Lists are stored split-major, [nsplit][T][R]: the 64 consecutive rows of
  // a wave write one contiguous run.
  if (row < a.T) {
    uint32_t* dst = a.cand_keys + ((size_t)split * a.T + row) * R;
#pragma unroll
    for (int r = 0; r < R; ++r) dst[r] = lk[r];
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
  // About one workgroup per compute unit (more for long chunks), 16 to
  // kMaxBps blocks per split, at most 64 splits (max_blocks <= 64 * kMaxBps).
  // Up to 64 * 256 blocks a split holds at most 256 blocks, so in-split ids
  // take at most 8 bits (ranking to 2^-15 relative, 2^-14 with page tiers);
  // only longer contexts need 9 (2^-14, plain ranking only).
  int64_t bps = ((int64_t)max_blocks * p.n_tiles + 255) / 256;
  if (bps < 16) bps = 16;
  if (bps > kMaxBps) bps = kMaxBps;
  if (max_blocks <= kMaxBlocksPrefillTiered && bps > kMaxBps / 2) bps = kMaxBps / 2;
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
#define UOCR_CASE(RR)                                                                                   \
  case RR:                                                                                              \
    if (a.block_page != nullptr)                                                                        \
      hipLaunchKernelGGL((indexer_prefill_kernel<RR, true>), grid, dim3(kPfThreads), 0, stream, a);     \
    else                                                                                                \
      hipLaunchKernelGGL((indexer_prefill_kernel<RR, false>), grid, dim3(kPfThreads), 0, stream, a);    \
    break;
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
// then written ascending, followed by the row's local window.  The arg-max
// runs on DPP row operations and the gfx950 lane swaps (a quad, the two
// halves of a row, the two halves of each 16-lane row, lanes l ^ 16 and
// l ^ 32), not LDS permutes, so a round is a short chain of VALU ops.
// ---------------------------------------------------------------------------

// A 64-bit key of the lane's DPP partner (both halves moved with the same
// control; every lane has a source for the patterns used below).
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, kCtrl, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), kCtrl, 0xF, 0xF, true);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t larger_u64(uint64_t a, uint64_t b) { return b > a ? b : a; }

// Larger of the lane's key and the one of lane l ^ 16 (l ^ 32 with W = 32):
// v_permlane*_swap of (x, x) leaves both values in every lane.
template <int W>
__device__ __forceinline__ uint64_t swap_larger(uint64_t k) {
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  const auto l2 = W == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                          : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h2 = W == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                          : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return larger_u64(((uint64_t)h2[0] << 32) | l2[0], ((uint64_t)h2[1] << 32) | l2[1]);
}

// Every lane gets the wave's largest key: a quad (two quad permutations),
// the halves of a row, the two halves of each 16-lane row, then lanes l ^ 16
// and l ^ 32; each step is two lane moves, one 64-bit compare and two
// selects.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  k = larger_u64(k, dpp_u64<0xB1>(k));   // quad_perm [1,0,3,2]
  k = larger_u64(k, dpp_u64<0x4E>(k));   // quad_perm [2,3,0,1]
  k = larger_u64(k, dpp_u64<0x141>(k));  // row_half_mirror
  k = larger_u64(k, dpp_u64<0x140>(k));  // row_mirror
  k = swap_larger<16>(k);
  return swap_larger<32>(k);
}

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
  uint32_t kp[R];
  const size_t off = ((size_t)lane * a.T + t) * R;  // [nsplit][T][R]
  if (lane < P.nsplit) {
    if constexpr (R % 4 == 0) {  // 16-byte aligned lists: R / 4 vector loads
      const uint4* src = reinterpret_cast<const uint4*>(a.cand_keys + off);
#pragma unroll
      for (int r4 = 0; r4 < R / 4; ++r4) {
        const uint4 v = src[r4];
        kp[4 * r4] = v.x;
        kp[4 * r4 + 1] = v.y;
        kp[4 * r4 + 2] = v.z;
        kp[4 * r4 + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) kp[r] = a.cand_keys[off + r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) kp[r] = 0u;
  }
  // Composite rank keys (truncated score, 0xFFFFFFFF - block id), unique and
  // descending in each lane; empty slots 0.
  uint64_t ck[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t id = (uint32_t)(lane * P.bps) + (idmask - (kp[r] & idmask));
    ck[r] = kp[r] != 0u ? ((uint64_t)(kp[r] >> P.idbits) << 32) | (0xFFFFFFFFu - id) : 0ull;
  }

  int32_t mine = -1;  // lane w keeps the w-th winner
#pragma unroll
  for (int w = 0; w < R; ++w) {
    const uint64_t best = wave_max_u64(ck[0]);
    if (best == 0ull) break;
    if (lane == w) mine = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
    if (ck[0] == best) {  // the one lane that held it moves to its next entry
#pragma unroll
      for (int r = 0; r + 1 < R; ++r) ck[r] = ck[r + 1];
      ck[R - 1] = 0ull;
    }
  }

  // Ascending order of the R winners: rank by counting smaller ids.
  int rank = 0;
#pragma unroll
  for (int v = 0; v < R; ++v) {
    const int32_t other = __builtin_amdgcn_readlane(mine, v);
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
