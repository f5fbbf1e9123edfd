// Block-major sparse attention for a chunked-prefill chunk (SR-SWA step 4,
// news.rkmt.cn/news/25027 Sec. 5; the chunked prefill of the leheavengame.com
// OCR 2 release article, Sec. 3): the same exact softmax over each row's kept
// tokens as the row-major gather kernel, organised so that every K/V tile is
// read once per chunk instead of once per row that keeps it.
//
// Rows of one chunk keep mostly different remote blocks, so a row-major
// gather moves ~12 remote tiles per (row, head) through L2 with little reuse.
// Here the (row, slot) pairs are bucketed by block (a counting sort in LDS,
// split over a few workgroups by block range), cut into chunks of at most
// 32 rows; one wave per (chunk, head) reads the head's K and V tiles once,
// scores all rows of the chunk with one chain of v_mfma_f32_32x32x16_bf16
// (keys on M, rows on N, fp32 accumulation of exact bf16 products), takes
// the block's softmax per row (max, exp2, sum: each lane owns 16 distinct
// scores of one row) and forms P.V in fp32 (each lane two output dims over
// all 32 keys), writing the
// row's partial state (m, l, o[128]) for the slot.  The local window is
// taken apart: a row's slots holding the window blocks of its own position
// (shared by every row of a 32-row block) are attended per row block and
// leave one partial per row instead of one per slot.  A merge pass combines
// the partials of each (row, head) in log-sum-exp form.
//
// Slot rule, shared by the bucket and merge passes: slot s of row t holds
// block j = block_idx[t][s]; it contributes iff 0 <= j < max_blocks and
// 32 j <= p (p = q_start + t).  A block whose pool index is out of range
// contributes nothing (partial m = -inf, l = 0).
#include <mutex>

#include "attn_common.h"
#include "device_common.h"
#include "kernels.h"

namespace uocr {

namespace {
constexpr int kRowsPerChunk = 32;               // the MFMA's N
constexpr int kBucketThreads = 1024;
constexpr int kBlockWaves = 4;                  // one (chunk, head) per wave
constexpr int kPStride = 36;                    // P row stride in LDS (floats), padded against bank conflicts
constexpr int kMergeWaves = 4;
constexpr int kPairUnroll = 32;                 // pairs per thread kept in registers by the bucket pass
constexpr int kPairTail = 4;                    // pairs per thread and round beyond those
constexpr int kPartStride = kDim;               // o[128]: 512 B (four whole cache lines) per (row, head, slot)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsView {
  int32_t* pairs;  // [T*topk] flat pair indices t*topk + s, bucketed by block
  int4* desc;      // [max_chunks] chunk descriptors: block j (-1: no chunk), first pair, rows, pool block
  float* part;     // [T][H][topk][kPartStride] unnormalised outputs o
  float2* ml;      // [T][H][topk] (m, l): the 16 slots of a (row, head) share one cache line
};

__device__ __forceinline__ WsView ws_view(const PrefillAttnArgs& a) {
  unsigned char* w = static_cast<unsigned char*>(a.ws);
  return {reinterpret_cast<int32_t*>(w + a.plan.pairs_off), reinterpret_cast<int4*>(w + a.plan.chunk_off),
          reinterpret_cast<float*>(w + a.plan.part_off), reinterpret_cast<float2*>(w + a.plan.ml_off)};
}

__device__ __forceinline__ bool slot_counts(int j, int p, int max_blocks) {
  return j >= 0 && j < max_blocks && j * kBlock <= p;
}

// Window slots: block j lies in the lw-block window ending at the block of
// position p.  They are attended per row block by the local pass, not per
// slot (a counting slot is either a window slot or a bucketed one).
__device__ __forceinline__ bool in_window(int j, int p, int lw) {
  const int bp = p >> 5;
  return lw > 0 && j > bp - lw && j <= bp;
}

// Sum of a lane's 8 output dims over the wave's four key groups
// (lanes l, l ^ 16, l ^ 32, l ^ 48), split over them: lanes l and l ^ 32
// keep dims 0-3 or 4-7 of the slice, then lanes l and l ^ 16 two of those,
// so lane l returns dims 8 (l % 16) + 4 (kg / 2) + 2 (kg % 2) and + 1
// (kg = l / 16).  Each v_permlane*_swap of two registers leaves one
// register's pair of values in the keeping lane (its own and its partner's).
__device__ __forceinline__ void reduce_scatter_dims(const float (&acc)[8], float& d0, float& d1) {
  float k1[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[d]), __float_as_uint(acc[4 + d]), false, false);
    k1[d] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  }
  const auto y0 = __builtin_amdgcn_permlane16_swap(__float_as_uint(k1[0]), __float_as_uint(k1[2]), false, false);
  const auto y1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(k1[1]), __float_as_uint(k1[3]), false, false);
  d0 = __uint_as_float(y0[0]) + __uint_as_float(y0[1]);
  d1 = __uint_as_float(y1[0]) + __uint_as_float(y1[1]);
}

// Row blocks of a chunk: runs of rows whose positions share one 32-token
// block.
__device__ __forceinline__ int row_blocks(const AttnArgs& A) {
  return A.nq > 0 ? ((A.q_start + A.nq - 1) >> 5) - (A.q_start >> 5) + 1 : 0;
}

// i / d for 0 <= i < 2^31 and 1 <= d: the high product with floor((2^32-1)/d)
// is floor(i/d) or one less; one correction step fixes it.
__device__ __forceinline__ int div_by(int i, int d, uint32_t magic) {
  int q = (int)__umulhi((uint32_t)i, magic);
  if ((q + 1) * d <= i) ++q;
  return q;
}
}  // namespace

// Bucket the chunk's (row, slot) pairs by block.  Each of G workgroups
// counts every pair into LDS (the atomics return each pair's rank in its
// bucket) and scans the bucket sizes and their chunk counts (each thread
// owns a contiguous range of blocks), so every workgroup knows where each
// bucket starts without hearing from the others; workgroup g then writes
// the chunk descriptors and the pairs of the blocks that wave g's threads
// own, and nothing else.  The order of pairs inside a bucket is not fixed,
// and does not need to be: each pair's partial has its own slot.
//
// Each thread keeps kPairUnroll pairs of the first round in registers
// (their blocks, -1 where the slot is not bucketed), so a chunk of up to
// kBucketThreads * kPairUnroll pairs (2048 rows x 16 slots) reads block_idx
// once per workgroup; larger chunks load the rest in narrower rounds, once
// for the counts and again for the scatter.  With 16-byte loads of four
// slots of one row (first_round), the row's bucketing bound is computed once
// per four slots: on one compute unit the per-slot division and tests, not
// the loads, were the first round's cost.

// Flat index of the pair a thread keeps in entry x of its first round: runs
// of four pairs for 16-byte loads (VEC), else consecutive lanes take
// consecutive pairs.
template <bool VEC>
__device__ __forceinline__ int first_round_pair(int tid, int x) {
  return VEC ? 4 * (tid + (x >> 2) * kBucketThreads) + (x & 3) : tid + x * kBucketThreads;
}

// Block of pair i if its slot is bucketed (counts and is no window slot),
// else -1.
__device__ __forceinline__ int bucketed_block(const AttnArgs& A, int j, int i, uint32_t magic, int lw) {
  const int p = A.q_start + div_by(i, A.topk, magic);
  return j >= 0 && slot_counts(j, p, A.max_blocks) && !in_window(j, p, lw) ? j : -1;
}

// The first round's loads are branch-free (indices clamped into the array,
// results past it replaced by -1) so that all of them are in flight at once.
// VEC (chosen by the host): block_idx is 16-byte aligned and topk is a
// multiple of 4, so each 16-byte load holds four slots of one row, whose
// bucketing test is then 0 <= j <= min(max_blocks - 1, bp - lw) with bp the
// block of the row's position (a slot counts iff j <= bp and is a window
// slot iff bp - lw < j <= bp).
template <bool VEC>
__device__ __forceinline__ void first_round(const AttnArgs& A, int tid, int npairs, uint32_t magic, int lw,
                                            int (&jv)[kPairUnroll]) {
  if constexpr (VEC) {
#pragma unroll
    for (int u = 0; u < kPairUnroll / 4; ++u) {
      const int i0 = first_round_pair<VEC>(tid, 4 * u);
      const int4 v = *reinterpret_cast<const int4*>(A.block_idx + min(i0, npairs - 4));
      const int bp = (A.q_start + div_by(i0, A.topk, magic)) >> 5;
      const int top = i0 < npairs ? max(-1, min(A.max_blocks - 1, bp - max(lw, 0))) : -1;
      const uint32_t n = (uint32_t)(top + 1);  // bucketed iff (unsigned)j < n
      jv[4 * u] = (uint32_t)v.x < n ? v.x : -1;
      jv[4 * u + 1] = (uint32_t)v.y < n ? v.y : -1;
      jv[4 * u + 2] = (uint32_t)v.z < n ? v.z : -1;
      jv[4 * u + 3] = (uint32_t)v.w < n ? v.w : -1;
    }
  } else {
#pragma unroll
    for (int x = 0; x < kPairUnroll; ++x) {
      const int i = first_round_pair<VEC>(tid, x);
      const int v = A.block_idx[min(i, npairs - 1)];
      jv[x] = i < npairs ? v : -1;
    }
#pragma unroll
    for (int x = 0; x < kPairUnroll; ++x)
      jv[x] = bucketed_block(A, jv[x], first_round_pair<VEC>(tid, x), magic, lw);
  }
}

// A later round (chunks of more than kBucketThreads * kPairUnroll pairs):
// pairs i0 + kBucketThreads u.
__device__ __forceinline__ void tail_round(const AttnArgs& A, int i0, int npairs, uint32_t magic, int lw,
                                           int (&jv)[kPairTail]) {
#pragma unroll
  for (int u = 0; u < kPairTail; ++u) {
    const int i = i0 + u * kBucketThreads;
    jv[u] = i < npairs ? A.block_idx[i] : -1;
  }
#pragma unroll
  for (int u = 0; u < kPairTail; ++u) jv[u] = bucketed_block(A, jv[u], i0 + u * kBucketThreads, magic, lw);
}

// CNT bounds max_blocks.  With STAGE > 0 (npairs <= STAGE, so every pair is
// in the first round) the workgroup's pairs go to bucket start + rank in an
// LDS copy of its part of the pairs array, written out with coalesced
// stores (4-byte stores scattered over the array would touch a separate
// cache line per lane); otherwise they are scattered through LDS cursors.
template <int CNT, int STAGE, bool VEC>
__global__ __launch_bounds__(kBucketThreads) void attn_prefill_bucket_kernel(PrefillAttnArgs a) {
  static_assert(STAGE <= kBucketThreads * kPairUnroll, "staged pairs must all be in the first round");
  __shared__ int32_t s_cnt[CNT];
  __shared__ int32_t s_wsum[2][kBucketThreads / kWave];  // per-wave sums of the two scans
  __shared__ int32_t s_stage[STAGE > 0 ? STAGE : 1];
  __shared__ int32_t s_range[2];  // the pairs of this workgroup's blocks: [s_range[0], s_range[1])
  const AttnArgs& A = a.attn;
  const WsView w = ws_view(a);
  const int M = A.max_blocks;
  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int lw = a.plan.local_win;
  constexpr int kRound = kBucketThreads * kPairUnroll;

  const int npairs = A.nq * A.topk;
  const uint32_t magic = 0xFFFFFFFFu / (uint32_t)A.topk;
  constexpr int kSeg = (CNT + kBucketThreads - 1) / kBucketThreads;
  const int seg = (M + kBucketThreads - 1) / kBucketThreads;  // <= kSeg
  const int j0 = min(tid * seg, M), j1 = min(j0 + seg, M);
  const bool own = tid / kWave == g;  // this thread's blocks are this workgroup's
  const int jlo = min(g * kWave * seg, M), jhi = min((g + 1) * kWave * seg, M);
  // pool indices of this thread's own blocks (for the descriptors; sequence
  // 0), read now so that the load overlaps the pair loads and the counting
  // (for up to 4 blocks per thread; more would crowd out the pairs)
  constexpr int kPre = kSeg <= 4 ? kSeg : 1;
  int pbs[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) pbs[k] = kSeg <= 4 ? A.block_table[min(j0 + k, M - 1)] : -1;
  int jf[kPairUnroll];  // the first round's blocks, kept for the scatter
  constexpr bool kVec = VEC && STAGE > 0;  // wide loads where the registers allow
  first_round<kVec>(A, tid, npairs, magic, lw, jf);
  for (int j = tid; j < M; j += kBucketThreads) s_cnt[j] = 0;
  __syncthreads();
  int rk[kPairUnroll];  // STAGE > 0: each pair's rank in its bucket
#pragma unroll
  for (int u = 0; u < kPairUnroll; ++u) {
    if constexpr (STAGE > 0) {
      rk[u] = jf[u] >= 0 ? atomicAdd(&s_cnt[jf[u]], 1) : 0;
    } else {
      if (jf[u] >= 0) atomicAdd(&s_cnt[jf[u]], 1);
    }
  }
  if constexpr (STAGE == 0) {
    for (int i0 = tid + kRound; i0 < npairs; i0 += kBucketThreads * kPairTail) {
      int jv[kPairTail];
      tail_round(A, i0, npairs, magic, lw, jv);
#pragma unroll
      for (int u = 0; u < kPairTail; ++u)
        if (jv[u] >= 0) atomicAdd(&s_cnt[jv[u]], 1);
    }
  }
  __syncthreads();

  int sp = 0, sc = 0;
  for (int j = j0; j < j1; ++j) {
    const int c = s_cnt[j];
    sp += c;
    sc += (c + kRowsPerChunk - 1) / kRowsPerChunk;
  }
  // exclusive scans of both sums: within each wave, then over the 16 wave
  // sums (held by lanes 0-15 of every wave after one barrier)
  constexpr int kWaves = kBucketThreads / kWave;
  const int lane = tid & (kWave - 1), wv = wave_id();
  const int ip = wave_incl_sum(sp), ic = wave_incl_sum(sc);
  if (lane == kWave - 1) {
    s_wsum[0][wv] = ip;
    s_wsum[1][wv] = ic;
  }
  __syncthreads();
  const int wp = wave_incl_sum(lane < kWaves ? s_wsum[0][lane] : 0);
  const int wc = wave_incl_sum(lane < kWaves ? s_wsum[1][lane] : 0);
  const int before_p = wv > 0 ? __builtin_amdgcn_readlane(wp, wv - 1) : 0;
  const int before_c = wv > 0 ? __builtin_amdgcn_readlane(wc, wv - 1) : 0;
  const int tot_c = __builtin_amdgcn_readlane(wc, kWaves - 1);
  int po = before_p + ip - sp, co = before_c + ic - sc;
  if (own && lane == 0) s_range[0] = po;
  if (own && lane == kWave - 1) s_range[1] = po + sp;
  // the descriptors of the thread's own blocks; s_cnt becomes each bucket's
  // cursor
  auto block_descs = [&](int k, int pb_pre) {
    const int j = j0 + k;
    const int c = s_cnt[j];
    const int nch = (c + kRowsPerChunk - 1) / kRowsPerChunk;
    if (own && nch > 0) {
      const int pb = kSeg <= 4 ? pb_pre : A.block_table[j];
      for (int q = 0; q < nch; ++q)
        w.desc[co + q] = make_int4(j, po + q * kRowsPerChunk, min(kRowsPerChunk, c - q * kRowsPerChunk), pb);
    }
    s_cnt[j] = po;
    po += c;
    co += nch;
  };
  if constexpr (kSeg <= 4) {
#pragma unroll
    for (int k = 0; k < kSeg; ++k)
      if (j0 + k < j1) block_descs(k, pbs[k]);
  } else {
#pragma unroll 1
    for (int k = 0; j0 + k < j1; ++k) block_descs(k, -1);
  }
  // descriptors past the last chunk: none (spread over the workgroups)
  for (int x = tot_c + g * kBucketThreads + tid; x < a.plan.max_chunks; x += (int)gridDim.x * kBucketThreads)
    w.desc[x] = make_int4(-1, 0, 0, -1);
  __syncthreads();
  if constexpr (STAGE > 0) {
    // s_cnt holds each bucket's first position; start + rank - lo stays
    // below hi - lo <= npairs <= STAGE.
    const int lo = s_range[0], hi = s_range[1];
#pragma unroll
    for (int u = 0; u < kPairUnroll; ++u)
      if (jf[u] >= jlo && jf[u] < jhi) s_stage[s_cnt[jf[u]] + rk[u] - lo] = first_round_pair<kVec>(tid, u);
    __syncthreads();
    for (int k = tid; k < hi - lo; k += kBucketThreads) w.pairs[lo + k] = s_stage[k];
  } else {
#pragma unroll
    for (int u = 0; u < kPairUnroll; ++u)
      if (jf[u] >= jlo && jf[u] < jhi) w.pairs[atomicAdd(&s_cnt[jf[u]], 1)] = first_round_pair<kVec>(tid, u);
    for (int i0 = tid + kRound; i0 < npairs; i0 += kBucketThreads * kPairTail) {
      int jv[kPairTail];
      tail_round(A, i0, npairs, magic, lw, jv);
#pragma unroll
      for (int u = 0; u < kPairTail; ++u)
        if (jv[u] >= jlo && jv[u] < jhi) w.pairs[atomicAdd(&s_cnt[jv[u]], 1)] = i0 + u * kBucketThreads;
    }
  }
}

// One wave per (chunk, head).  Lane l works on chunk row n = l % 32 and
// half hh = l / 32 for the scores.
//  * A fragment of step s (dims 16 s + 8 hh .. +8, the summation-order
//    permutation shared by A and B): K row n, read from a wave-private LDS
//    copy of the tile; B fragment: q of chunk row n (rows past the chunk
//    repeat row 0; their results are never used).  The K tile reaches LDS
//    through eight 1 KB-contiguous non-temporal loads (like V below), its
//    16-byte chunk c of row r stored at c ^ (r % 16) so that neither the
//    copy nor the fragment reads of 32 rows at one column conflict in banks.
//  * C register r of lane l holds the score of key 8 (r / 4) + 4 hh + r % 4
//    for chunk row n.
//  * P goes through a wave-private LDS tile [32 rows][kPStride].
//  * V is read with eight 1 KB-contiguous non-temporal loads (each reads
//    whole cache lines once, so V does not displace other lines from the
//    caches): lane l holds dims 8 (l % 16) .. +8 of keys 4 i + kg, i = 0..7,
//    kg = l / 16, widened to fp32 once.  V of keys past every row's position
//    is replaced by 0 (such slots may hold anything, NaN included, and a
//    masked key's probability 0 must not meet it).
//  * For each chunk row, a lane sums its 8 keys into its 8 dims; the four
//    key groups are then added with two lane swaps that also split the dims
//    (reduce-scatter: l ^ 32 keeps dims 0-3 or 4-7 of the slice, l ^ 16 two
//    of those), so lane l ends with dims 8 (l % 16) + 4 (kg / 2) + 2 (kg % 2)
//    and + 1, and the row's 128 outputs are one 512-byte store.
__global__ __launch_bounds__(kBlockWaves * kWave) void attn_prefill_block_kernel(PrefillAttnArgs a) {
  // per wave: the K tile (16-byte chunk c of row r at c ^ (r % 16)), then,
  // once the fragments are in registers, the P tile in the same bytes
  __shared__ __attribute__((aligned(16))) uint4 s_k[kBlockWaves][kBlock * 16];
  static_assert(kRowsPerChunk * kPStride * 4 <= kBlock * 16 * 16, "P fits in the K tile's bytes");
  const AttnArgs& A = a.attn;
  const WsView w = ws_view(a);
  const int wave = wave_id();
  const int64_t unit = (int64_t)blockIdx.x * kBlockWaves + wave;
  const int g = (int)(unit / A.heads);
  const int h = (int)(unit - (int64_t)g * A.heads);
  if (g >= a.plan.max_chunks) return;
  // one descriptor read, then the tiles and this lane's pair load together
  const int4 d = w.desc[g];
  const int j = __builtin_amdgcn_readfirstlane(d.x);
  if (j < 0) return;
  const int start = __builtin_amdgcn_readfirstlane(d.y);
  const int n_rows = __builtin_amdgcn_readfirstlane(d.z);
  const int pb = __builtin_amdgcn_readfirstlane(d.w);
  const bool ok = pb >= 0 && (int64_t)pb < A.num_blocks;
  const int lane = lane_id();
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int pair_v = w.pairs[start + (n < n_rows ? n : 0)];  // this lane's chunk row
  const int t_n = pair_v / A.topk;
  const int p_n = A.q_start + t_n;

  float m_row = -INFINITY, l_row = 0.0f;
  const int kg = lane >> 4;  // key group of the lane's V rows
  float vf[8][8];            // V[4 i + kg][8 (lane % 16) + d], fp32
  float* P = reinterpret_cast<float*>(s_k[wave]);
  if (ok) {
    const int64_t tile = ((int64_t)pb * A.heads + h) * (kBlock * kDim);
    const uint16_t* kt = A.k_pool + tile;
    const uint16_t* vt = A.v_pool + tile;
    const uint16_t* qr = A.q + ((int64_t)t_n * A.heads + h) * kDim;
    // K and V depend only on the descriptor: issued first, while this
    // lane's pair (and with it the row of q) is still in flight
    bf16x8_t av[8], bq[8];
    uint4 kw[8];  // row 4 i + lane / 16, chunk lane % 16
#pragma unroll
    for (int i = 0; i < 8; ++i) kw[i] = load_stream16(reinterpret_cast<const uint4*>(kt) + i * kWave + lane);
    uint4 vw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vw[i] = load_stream16(reinterpret_cast<const uint4*>(vt) + i * kWave + lane);
#pragma unroll
    for (int st = 0; st < 8; ++st) bq[st] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * st + 8 * hh);
    uint4* K = s_k[wave];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      K[r * 16 + ((lane & 15) ^ (r & 15))] = kw[i];
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
      av[st] = __builtin_bit_cast(bf16x8_t, K[n * 16 + ((2 * st + hh) ^ (n & 15))]);
    f32x16_t c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[0], bq[0], f32x16_t{0}, 0, 0, 0);
#pragma unroll
    for (int st = 1; st < 8; ++st) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[st], bq[st], c, 0, 0, 0);

    // Softmax of the block for chunk row n (tokens past p_n masked).
    const int key0 = j * kBlock + 4 * hh;
    float z[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + (r & 3);
      z[r] = key <= p_n ? c[r] * A.scale_log2 : -INFINITY;
      mx = fmaxf(mx, z[r]);
    }
    m_row = max_xor32(mx);  // at least key 32j <= p_n is visible
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      z[r] = exp2f(z[r] - m_row);
      sum += z[r];
    }
    l_row = sum_xor32(sum);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(P + n * kPStride + 8 * q4 + 4 * hh) =
          make_float4(z[4 * q4], z[4 * q4 + 1], z[4 * q4 + 2], z[4 * q4 + 3]);
    // Largest position among the chunk's rows: keys past it are masked for all.
    const int pmax = wave_max_i32(n < n_rows ? p_n : -1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool seen = j * kBlock + 4 * i + kg <= pmax;
      const uint32_t w4[4] = {vw[i].x, vw[i].y, vw[i].z, vw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[i][2 * e] = seen ? bf16_lo(w4[e]) : 0.0f;
        vf[i][2 * e + 1] = seen ? bf16_hi(w4[e]) : 0.0f;
      }
    }
  }
  // (m, l) of chunk row n, written by its lane in the lower half.
  if (hh == 0 && n < n_rows) {
    const int s_n = pair_v - t_n * A.topk;
    w.ml[((int64_t)t_n * A.heads + h) * A.topk + s_n] = make_float2(m_row, l_row);
  }
  for (int r = 0; r < n_rows; ++r) {
    const int i = __builtin_amdgcn_readlane(pair_v, r);
    const int t = i / A.topk;
    const int s_ = i - t * A.topk;
    float o0 = 0.0f, o1 = 0.0f;
    if (ok) {
      float acc[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pr = P[r * kPStride + 4 * i + kg];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] += pr * vf[i][d];
      }
      reduce_scatter_dims(acc, o0, o1);
    }
    float* dst = w.part + (((int64_t)t * A.heads + h) * A.topk + s_) * kPartStride;
    *reinterpret_cast<float2*>(dst + 8 * (lane & 15) + 4 * (kg >> 1) + 2 * (kg & 1)) = make_float2(o0, o1);
  }
}

// The window slots of a row block in one pass.  Rows whose positions lie
// in block bp share the window blocks bp - lw + 1 .. bp (lw = the local
// window), which nearly every row keeps: one wave per (row block, head)
// reads each window block's K and V tiles once and carries each row's
// online-softmax state (m, l, o) over all of its window slots (a block a row
// keeps c times counts c times; rows that do not keep it mask all of its
// keys).  The state is written as one partial at the row's first window
// slot; the bucket pass leaves window slots out and the merge reads only
// that one, so the window adds no per-slot partials.
//  * Scores: the block pass's MFMA layout (keys on M, rows on N); lane
//    (n, hh) holds row n's scores of keys 8 (r / 4) + 4 hh + r % 4.
//  * P.V on the matrix cores as well: O (rows x 128 dims, four 32-dim
//    tiles) += P (rows x keys) V (keys x dims).  The A fragment of k-step st
//    is the lane's own probabilities r = 8 st .. 8 st + 7 (k index 8 hh + e
//    <-> key 4 hh + 16 st + 8 (e / 4) + e % 4, a summation-order permutation
//    that B follows), split exactly into three bf16 terms (truncations of p
//    and of the remainders: 8 + 8 + 8 mantissa bits), so the three products
//    with the bf16 V are exact and summed in fp32.  B fragments are read
//    from a transposed copy of the V tile in LDS (dims x keys; two 8-byte
//    reads give a lane its 8 keys of one dim).  C register r of lane l holds
//    row 8 (r / 4) + 4 hh + r % 4, dim l % 32 of the tile; the rescaling by
//    each row's alpha reads the alphas from LDS.
//  * V keys past every row's position are written to the copy as 0 (such
//    slots may hold anything, NaN included).  K and V use ordinary loads: a
//    window tile is shared by lw row blocks.
constexpr int kVtStride = 36;  // keys per dim row of the transposed V copy (bf16), padded
constexpr int kLocalIds = 16;  // block ids per row held in registers (topk <= 16, a multiple of 4)

__device__ __forceinline__ bf16x8_t bf16x8_bits(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(a, b, c, d));
}

__global__ __launch_bounds__(kBlockWaves * kWave) void attn_prefill_local_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[kBlockWaves][kDim * kVtStride];
  __shared__ __attribute__((aligned(16))) float s_alpha[kBlockWaves][kRowsPerChunk];
  __shared__ int32_t s_first[kBlockWaves][kRowsPerChunk];
  const AttnArgs& A = a.attn;
  const WsView w = ws_view(a);
  const int wave = wave_id();
  const int lw = a.plan.local_win;
  // XCD-aware order: workgroup g runs on XCD g % 8.  Each XCD takes a
  // contiguous range of row blocks for every head, head-major, so the waves
  // of a workgroup and its neighbours on the XCD are consecutive row blocks
  // of one head, which share lw - 1 of their lw window tiles through that
  // XCD's L2 instead of each XCD fetching them from memory again.
  const int nrb = row_blocks(A);
  const int per_xcd = (nrb + 7) >> 3;
  const int64_t u = (int64_t)(blockIdx.x >> 3) * kBlockWaves + wave;  // unit within the XCD
  const int h = (int)(u / per_xcd);
  const int rb = (int)(blockIdx.x & 7) * per_xcd + (int)(u - (int64_t)h * per_xcd);
  if (h >= A.heads || rb >= nrb) return;
  const int bp = (A.q_start >> 5) + rb;
  const int t0 = max(0, bp * kBlock - A.q_start);
  const int nrows = min(A.nq, (bp + 1) * kBlock - A.q_start) - t0;  // 1 .. 32
  const int lane = lane_id();
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int kg = lane >> 4;
  const bool row_ok = n < nrows;
  const int t_n = t0 + (row_ok ? n : 0);
  const int p_n = A.q_start + t_n;
  const int32_t* ids = A.block_idx + (int64_t)t_n * A.topk;
  // up to 16 block ids of the row in registers (one 16-byte load per 4), so
  // the window bookkeeping below reads memory once
  const bool reg_ids = A.topk <= kLocalIds && (A.topk & 3) == 0 && (reinterpret_cast<uintptr_t>(A.block_idx) & 15) == 0;
  int idr[kLocalIds];
#pragma unroll
  for (int k4 = 0; k4 < kLocalIds / 4; ++k4) {
    int4 v = make_int4(-1, -1, -1, -1);
    if (reg_ids && 4 * k4 < A.topk) v = *reinterpret_cast<const int4*>(ids + 4 * k4);
    idr[4 * k4] = v.x;
    idr[4 * k4 + 1] = v.y;
    idr[4 * k4 + 2] = v.z;
    idr[4 * k4 + 3] = v.w;
  }
  // the row's first window slot: where its partial goes (-1: none)
  int sf = -1;
  if (reg_ids) {
#pragma unroll
    for (int s_ = kLocalIds - 1; s_ >= 0; --s_)
      if (slot_counts(idr[s_], p_n, A.max_blocks) && in_window(idr[s_], p_n, lw)) sf = s_;
  } else {
    for (int s_ = A.topk - 1; s_ >= 0; --s_) {
      const int j = ids[s_];
      if (slot_counts(j, p_n, A.max_blocks) && in_window(j, p_n, lw)) sf = s_;
    }
  }
  if (!row_ok) sf = -1;
  if (__ballot(sf >= 0) == 0) return;
  if (hh == 0) s_first[wave][n] = sf;
  const uint16_t* qr = A.q + ((int64_t)t_n * A.heads + h) * kDim;
  bf16x8_t bq[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) bq[st] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * st + 8 * hh);
  const int pmax = A.q_start + t0 + nrows - 1;  // keys past it are masked for every row
  uint16_t* vt_l = s_vt[wave];

  float m_row = -INFINITY, l_row = 0.0f;
  f32x16_t acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16_t{0};
  // Window blocks one at a time.  A block no row keeps, outside the table
  // or with an out-of-range pool index is skipped: it changes nothing.
  for (int jj = 0; jj < lw; ++jj) {
    {
      const int j = bp - lw + 1 + jj;
      if (j < 0 || j >= A.max_blocks) continue;
      int c = 0;  // how many of row n's slots keep block j
      if (row_ok) {
        if (reg_ids) {
#pragma unroll
          for (int s_ = 0; s_ < kLocalIds; ++s_) c += idr[s_] == j ? 1 : 0;
        } else {
          for (int s_ = 0; s_ < A.topk; ++s_) c += ids[s_] == j ? 1 : 0;
        }
      }
      if (__ballot(c > 0) == 0) continue;
      const int pb = __builtin_amdgcn_readfirstlane(A.block_table[j]);  // sequence 0
      if (pb < 0 || (int64_t)pb >= A.num_blocks) continue;
      const int64_t tile = ((int64_t)pb * A.heads + h) * (kBlock * kDim);
      const uint16_t* kt = A.k_pool + tile;
      const uint16_t* vt = A.v_pool + tile;
      bf16x8_t av[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) av[st] = *reinterpret_cast<const bf16x8_t*>(kt + n * kDim + 16 * st + 8 * hh);
      uint4 vw[8];  // V[4 i + kg][8 (lane % 16) .. +8]
#pragma unroll
      for (int i = 0; i < 8; ++i) vw[i] = reinterpret_cast<const uint4*>(vt)[i * kWave + lane];
      f32x16_t cc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[0], bq[0], f32x16_t{0}, 0, 0, 0);
#pragma unroll
      for (int st = 1; st < 8; ++st) cc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[st], bq[st], cc, 0, 0, 0);

      const int key0 = j * kBlock + 4 * hh;
      float z[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + (r & 3);
        z[r] = (c > 0 && key <= p_n) ? cc[r] * A.scale_log2 : -INFINITY;
        mx = fmaxf(mx, z[r]);
      }
      const float m_new = fmaxf(m_row, max_xor32(mx));
      // 1 when the max does not move (also for rows that saw no key yet)
      const float alpha = m_new == m_row ? 1.0f : exp2f(m_row - m_new);
      const float cf = (float)c;
      float sum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        z[r] = z[r] == -INFINITY ? 0.0f : cf * exp2f(z[r] - m_new);
        sum += z[r];
      }
      l_row = l_row * alpha + sum_xor32(sum);
      m_row = m_new;
      if (hh == 0) s_alpha[wave][n] = alpha;
      // transposed V copy: vt_l[dim * kVtStride + key]
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = 4 * i + kg;
        const bool seen = j * kBlock + key <= pmax;
        const uint32_t w4[4] = {vw[i].x, vw[i].y, vw[i].z, vw[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dim = 8 * (lane & 15) + 2 * e;
          vt_l[dim * kVtStride + key] = seen ? (uint16_t)(w4[e] & 0xFFFFu) : (uint16_t)0;
          vt_l[(dim + 1) * kVtStride + key] = seen ? (uint16_t)(w4[e] >> 16) : (uint16_t)0;
        }
      }
      // rescale O by each row's alpha (rows 8 q + 4 hh + 0..3 of the C layout)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 al = *reinterpret_cast<const float4*>(&s_alpha[wave][8 * q + 4 * hh]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          acc[dt][4 * q] *= al.x;
          acc[dt][4 * q + 1] *= al.y;
          acc[dt][4 * q + 2] *= al.z;
          acc[dt][4 * q + 3] *= al.w;
        }
      }
      // exact three-term bf16 split of P, A fragments of k-steps 0 and 1
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        uint32_t t1[8], t2[8], t3[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = z[8 * st + e];
          const uint32_t b1 = __float_as_uint(pv) & 0xFFFF0000u;
          const float r1 = pv - __uint_as_float(b1);
          const uint32_t b2 = __float_as_uint(r1) & 0xFFFF0000u;
          const float r2 = r1 - __uint_as_float(b2);
          t1[e] = b1 >> 16;
          t2[e] = b2 >> 16;
          t3[e] = __float_as_uint(r2) >> 16;
        }
        const bf16x8_t a1 = bf16x8_bits(t1[0] | t1[1] << 16, t1[2] | t1[3] << 16, t1[4] | t1[5] << 16, t1[6] | t1[7] << 16);
        const bf16x8_t a2 = bf16x8_bits(t2[0] | t2[1] << 16, t2[2] | t2[3] << 16, t2[4] | t2[5] << 16, t2[6] | t2[7] << 16);
        const bf16x8_t a3 = bf16x8_bits(t3[0] | t3[1] << 16, t3[2] | t3[3] << 16, t3[4] | t3[5] << 16, t3[6] | t3[7] << 16);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint16_t* src = vt_l + (32 * dt + n) * kVtStride + 4 * hh + 16 * st;
          const uint2 lo = *reinterpret_cast<const uint2*>(src);
          const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
          const bf16x8_t bv = bf16x8_bits(lo.x, lo.y, hi.x, hi.y);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bv, acc[dt], 0, 0, 0);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, bv, acc[dt], 0, 0, 0);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, bv, acc[dt], 0, 0, 0);
        }
      }
    }
  }
  // partial of each row with a window slot: row 8 q + 4 hh + u, dim 32 dt + n
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 8 * q + 4 * hh + u;
      if (r < nrows) {
        const int sr = s_first[wave][r];
        if (sr >= 0) {
          float* dst = w.part + (((int64_t)(t0 + r) * A.heads + h) * A.topk + sr) * kPartStride + n;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) dst[32 * dt] = acc[dt][4 * q + u];
        }
      }
    }
  }
  if (hh == 0 && sf >= 0) w.ml[((int64_t)t_n * A.heads + h) * A.topk + sf] = make_float2(m_row, l_row);
}

// One wave per (row, head): log-sum-exp merge of the row's partials.  Lane s
// (< 64) takes slot s's (m, l) and weight; then every slot's two output
// values per lane are loaded together (weight 0 for slots that keep nothing;
// non-temporal loads, each reading whole lines of a record read once) and
// lane d produces dims d and d + 64.  No kept token gives out = 0,
// lse = -inf.
__global__ __launch_bounds__(kMergeWaves * kWave) void attn_prefill_merge_kernel(PrefillAttnArgs a) {
  const AttnArgs& A = a.attn;
  const WsView w = ws_view(a);
  const int item = blockIdx.x * kMergeWaves + wave_id();
  if (item >= A.nq * A.heads) return;
  const int t = item / A.heads;
  const int p = A.q_start + t;
  const int lane = lane_id();
  const int32_t* sel = A.block_idx + (int64_t)t * A.topk;
  const float* base = w.part + (int64_t)item * A.topk * kPartStride;
  const float2* mls = w.ml + (int64_t)item * A.topk;

  // the row's first window slot holds the partial of all its window slots
  const int lw = a.plan.local_win;
  int sfirst = -1;
  for (int s0 = 0; lw > 0 && s0 < A.topk; s0 += kWave) {
    const int s = s0 + lane;
    const int j = s < A.topk ? sel[s] : -1;
    const uint64_t win = __ballot(s < A.topk && slot_counts(j, p, A.max_blocks) && in_window(j, p, lw));
    if (win != 0) {
      sfirst = s0 + __builtin_ctzll(win);
      break;
    }
  }
  float res0 = 0.0f, res1 = 0.0f, L = 0.0f, M = -INFINITY;
  for (int s0 = 0; s0 < A.topk; s0 += kWave) {  // one round for topk <= 64
    const int s = s0 + lane;
    const int js = s < A.topk ? sel[s] : -1;
    const bool valid = s < A.topk && slot_counts(js, p, A.max_blocks) && (!in_window(js, p, lw) || s == sfirst);
    float2 ml = make_float2(-INFINITY, 0.0f);
    if (valid) ml = mls[s];
    const float Mr = wave_max_f32(ml.x);
    if (Mr == -INFINITY) continue;
    // rescale what earlier rounds accumulated
    const float Mn = fmaxf(M, Mr);
    const float sc = exp2f(M - Mn);
    res0 *= sc;
    res1 *= sc;
    L *= sc;
    M = Mn;
    const float f = valid ? exp2f(ml.x - M) : 0.0f;
    L += wave_sum_f32(ml.y * f);
    const int ns = min(kWave, A.topk - s0);
    for (int u0 = 0; u0 < ns; u0 += 16) {
      float o0[16], o1[16], fu[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        fu[u] = u0 + u < ns ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(f), u0 + u)) : 0.0f;
        const float* ps = base + (int64_t)(s0 + u0 + u) * kPartStride;
        o0[u] = fu[u] != 0.0f ? __builtin_nontemporal_load(ps + lane) : 0.0f;
        o1[u] = fu[u] != 0.0f ? __builtin_nontemporal_load(ps + lane + kWave) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        res0 += o0[u] * fu[u];
        res1 += o1[u] * fu[u];
      }
    }
  }
  float lse_v = -INFINITY;
  if (M != -INFINITY) {
    res0 /= L;
    res1 /= L;
    lse_v = (M + log2f(L)) * kLn2;
  } else {
    res0 = res1 = 0.0f;
  }
  float* out = A.out + (int64_t)item * kDim;
  out[lane] = res0;
  out[lane + kWave] = res1;
  if (A.lse != nullptr && lane == 0) A.lse[item] = lse_v;
}

PrefillAttnPlan prefill_attn_plan(int32_t T, int32_t heads, int32_t topk, int32_t max_blocks) {
  PrefillAttnPlan p{};
  if (T <= 0 || heads <= 0 || topk <= 0 || max_blocks <= 0 || max_blocks > kMaxBlocksAttnBucket) return p;
  const int64_t npairs = (int64_t)T * topk;
  if (npairs >= ((int64_t)1 << 31) / 2) return p;  // flat pair indices stay in int32
  p.max_chunks = (int32_t)(max_blocks + (npairs + kRowsPerChunk - 1) / kRowsPerChunk);
  size_t at = 0;
  p.pairs_off = at;
  at = align256(at + (size_t)npairs * 4);
  p.chunk_off = at;
  at = align256(at + (size_t)p.max_chunks * 16);
  p.part_off = at;
  at = align256(at + (size_t)npairs * heads * kPartStride * 4);
  p.ml_off = at;
  at = align256(at + (size_t)npairs * heads * 8);
  p.ws_bytes = at;
  return p;
}

namespace {
int row_blocks_host(const AttnArgs& A) {
  return A.nq > 0 ? ((A.q_start + A.nq - 1) >> 5) - (A.q_start >> 5) + 1 : 0;
}

// The window pass does not depend on the bucketing, and the bucketing runs
// in a few workgroups, so the window pass runs beside it on a second stream
// (default priority, non-blocking), forked from and joined back to the
// caller's stream with two events: one stream and two events per device,
// created on first use and held until the process ends.  A mutex per device
// keeps each call's fork, launch and join together.  If they cannot be
// created, the window pass runs on the caller's stream.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipError_t status = hipSuccess;
  std::mutex mu;
};
constexpr int kMaxDevices = 64;
std::once_flag g_side_once[kMaxDevices];
SideStream g_side[kMaxDevices];

SideStream* side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_side_once[dev], [dev] {
    SideStream& s = g_side[dev];
    s.status = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking);
    if (s.status == hipSuccess) s.status = hipEventCreateWithFlags(&s.fork, hipEventDisableTiming);
    if (s.status == hipSuccess) s.status = hipEventCreateWithFlags(&s.join, hipEventDisableTiming);
  });
  return g_side[dev].status == hipSuccess ? &g_side[dev] : nullptr;
}
}  // namespace

hipError_t launch_attn_prefill_blocks(const PrefillAttnArgs& a, hipStream_t stream) {
  const AttnArgs& A = a.attn;
  if (A.nq == 0) return hipSuccess;
  // window pass: 8 XCDs x the workgroups of one XCD's row-block range for
  // every head (see attn_prefill_local_kernel)
  const int64_t lunits = a.plan.local_win > 0 ? (int64_t)row_blocks_host(A) * A.heads : 0;
  const int64_t lunits_xcd = (int64_t)((row_blocks_host(A) + 7) / 8) * A.heads;
  const dim3 lgrid((unsigned)(8 * ((lunits_xcd + kBlockWaves - 1) / kBlockWaves)));
  SideStream* side = lunits > 0 ? side_stream() : nullptr;
  std::unique_lock<std::mutex> lock;
  if (side != nullptr) {
    lock = std::unique_lock<std::mutex>(side->mu);
    hipError_t e = hipEventRecord(side->fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_prefill_local_kernel, lgrid, dim3(kBlockWaves * kWave), 0, side->stream, a);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipEventRecord(side->join, side->stream);
    if (e != hipSuccess) return e;
  } else if (lunits > 0) {
    hipLaunchKernelGGL(attn_prefill_local_kernel, lgrid, dim3(kBlockWaves * kWave), 0, stream, a);
  }
  // One bucketing workgroup per wave's worth of blocks in the scan (at most
  // 16).  Staged bucketing: counts for up to 4096 blocks (16 KB) and up to
  // 32768 pairs (128 KB) in LDS, beside the 8 KB scan.
  const int seg = (A.max_blocks + kBucketThreads - 1) / kBucketThreads;
  const dim3 bgrid((unsigned)((A.max_blocks + kWave * seg - 1) / (kWave * seg)));
  const int64_t npairs = (int64_t)A.nq * A.topk;
  const bool vec = (reinterpret_cast<uintptr_t>(A.block_idx) & 15) == 0 && A.topk % 4 == 0;
  if (A.max_blocks <= 4096 && npairs <= 32768 && vec)
    hipLaunchKernelGGL((attn_prefill_bucket_kernel<4096, 32768, true>), bgrid, dim3(kBucketThreads), 0, stream, a);
  else if (A.max_blocks <= 4096 && npairs <= 32768)
    hipLaunchKernelGGL((attn_prefill_bucket_kernel<4096, 32768, false>), bgrid, dim3(kBucketThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_prefill_bucket_kernel<kMaxBlocksAttnBucket, 0, false>), bgrid, dim3(kBucketThreads), 0,
                       stream, a);
  const int64_t units = (int64_t)a.plan.max_chunks * A.heads;
  hipLaunchKernelGGL(attn_prefill_block_kernel, dim3((unsigned)((units + kBlockWaves - 1) / kBlockWaves)),
                     dim3(kBlockWaves * kWave), 0, stream, a);
  if (side != nullptr) {  // the merge reads the window partials
    const hipError_t e = hipStreamWaitEvent(stream, side->join, 0);
    if (e != hipSuccess) return e;
  }
  const int64_t items = (int64_t)A.nq * A.heads;
  hipLaunchKernelGGL(attn_prefill_merge_kernel, dim3((unsigned)((items + kMergeWaves - 1) / kMergeWaves)),
                     dim3(kMergeWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uocr
