// Block-major sparse attention for a chunked-prefill chunk (SR-SWA step 4,
// news.rkmt.cn/news/25027 Sec. 5; the chunked prefill of the leheavengame.com
// OCR 2 release article, Sec. 3): the same exact softmax over each row's kept
// tokens as the row-major gather kernel, organised so that every K/V tile is
// read once per chunk instead of once per row that keeps it.
//
// Rows of one chunk keep mostly different remote blocks, so a row-major
// gather moves ~12 remote tiles per (row, head) through L2 with little reuse.
// Here the (row, slot) pairs are bucketed by block (one workgroup, counting
// sort in LDS), cut into chunks of at most 32 rows; one wave per (chunk,
// head) reads the head's K and V tiles once, scores all rows of the chunk
// with one chain of v_mfma_f32_32x32x16_bf16 (keys on M, rows on N, fp32
// accumulation of exact bf16 products), takes the block's softmax per row
// (max, exp2, sum: each lane owns 16 distinct scores of one row) and forms
// P.V in fp32 (each lane two output dims over all 32 keys), writing the
// row's partial state (m, l, o[128]) for the slot.  A merge pass combines
// the partials of each (row, head) in log-sum-exp form.
//
// Slot rule, shared by the bucket and merge passes: slot s of row t holds
// block j = block_idx[t][s]; it contributes iff 0 <= j < max_blocks and
// 32 j <= p (p = q_start + t).  A block whose pool index is out of range
// contributes nothing (partial m = -inf, l = 0).
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
constexpr int kPartStride = kDim + 4;           // o[128], m, l, pad: 528 B per (row, head, slot)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsView {
  int32_t* off;    // [M+1] first pair of each block's bucket
  int32_t* choff;  // [M+1] first chunk of each block; choff[M] = number of chunks
  int32_t* pairs;  // [T*topk] flat pair indices t*topk + s, bucketed by block
  int32_t* chunk;  // [max_chunks] block of each chunk
  float* part;     // [T][H][topk][kPartStride]
};

__device__ __forceinline__ WsView ws_view(const PrefillAttnArgs& a) {
  unsigned char* w = static_cast<unsigned char*>(a.ws);
  return {reinterpret_cast<int32_t*>(w + a.plan.off_off), reinterpret_cast<int32_t*>(w + a.plan.choff_off),
          reinterpret_cast<int32_t*>(w + a.plan.pairs_off), reinterpret_cast<int32_t*>(w + a.plan.chunk_off),
          reinterpret_cast<float*>(w + a.plan.part_off)};
}

__device__ __forceinline__ bool slot_counts(int j, int p, int max_blocks) {
  return j >= 0 && j < max_blocks && j * kBlock <= p;
}

// i / d for 0 <= i < 2^31 and 1 <= d: the high product with floor((2^32-1)/d)
// is floor(i/d) or one less; one correction step fixes it.
__device__ __forceinline__ int div_by(int i, int d, uint32_t magic) {
  int q = (int)__umulhi((uint32_t)i, magic);
  if ((q + 1) * d <= i) ++q;
  return q;
}
}  // namespace

// Bucket the chunk's (row, slot) pairs by block: counts in LDS, one exclusive
// scan for the bucket offsets and one for the chunk offsets (each thread owns
// a contiguous range of blocks), then a scatter through LDS cursors.  The
// order of pairs inside a bucket is not fixed, and does not need to be: each
// pair's partial has its own slot.
//
// Each thread loads its first kPairUnroll pairs in one round and keeps their
// blocks (-1 where the slot does not count) in registers for the scatter, so
// a chunk of up to kBucketThreads * kPairUnroll pairs (2048 rows x 16 slots)
// reads block_idx once, with one memory round trip; larger chunks load the
// rest in narrower rounds, once for the counts and again for the scatter.
template <int N>
__device__ __forceinline__ void bucket_round(const AttnArgs& A, int i0, int npairs, int topk, uint32_t magic, int M,
                                             int (&jv)[N]) {
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int i = i0 + u * kBucketThreads;
    jv[u] = i < npairs ? A.block_idx[i] : -1;
  }
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int i = i0 + u * kBucketThreads;
    if (jv[u] >= 0 && !slot_counts(jv[u], A.q_start + div_by(i, topk, magic), M)) jv[u] = -1;
  }
}

// CNT bounds max_blocks.  With STAGE > 0 (npairs <= STAGE, so every pair is
// in the first round) the counting atomics return each pair's rank in its
// bucket, the pairs go to bucket start + rank in an LDS copy of the pairs
// array without a second round of atomics, and that copy is written out with
// coalesced stores: one workgroup scattering 4-byte stores over the whole
// pairs array touches a separate cache line per lane.
template <int CNT, int STAGE>
__global__ __launch_bounds__(kBucketThreads) void attn_prefill_bucket_kernel(PrefillAttnArgs a) {
  static_assert(STAGE <= kBucketThreads * kPairUnroll, "staged pairs must all be in the first round");
  __shared__ int32_t s_cnt[CNT];
  __shared__ int32_t s_scan[2][kBucketThreads];
  __shared__ int32_t s_stage[STAGE > 0 ? STAGE : 1];
  const AttnArgs& A = a.attn;
  const WsView w = ws_view(a);
  const int M = A.max_blocks, topk = A.topk;
  const int tid = threadIdx.x;
  constexpr int kRound = kBucketThreads * kPairUnroll;

  // Consecutive lanes take consecutive pairs (slots of a few rows), which keeps
  // same-block LDS atomics within a wave to a few lanes.
  const int npairs = A.nq * topk;
  const uint32_t magic = 0xFFFFFFFFu / (uint32_t)topk;
  int jf[kPairUnroll];  // the first round's blocks, kept for the scatter
  bucket_round(A, tid, npairs, topk, magic, M, jf);
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
      bucket_round(A, i0, npairs, topk, magic, M, jv);
#pragma unroll
      for (int u = 0; u < kPairTail; ++u)
        if (jv[u] >= 0) atomicAdd(&s_cnt[jv[u]], 1);
    }
  }
  __syncthreads();

  const int seg = (M + kBucketThreads - 1) / kBucketThreads;
  const int j0 = min(tid * seg, M), j1 = min(j0 + seg, M);
  int sp = 0, sc = 0;
  for (int j = j0; j < j1; ++j) {
    const int c = s_cnt[j];
    sp += c;
    sc += (c + kRowsPerChunk - 1) / kRowsPerChunk;
  }
  s_scan[0][tid] = sp;
  s_scan[1][tid] = sc;
  __syncthreads();
  for (int d = 1; d < kBucketThreads; d <<= 1) {  // inclusive scan of both sums
    const int x0 = tid >= d ? s_scan[0][tid - d] : 0;
    const int x1 = tid >= d ? s_scan[1][tid - d] : 0;
    __syncthreads();
    s_scan[0][tid] += x0;
    s_scan[1][tid] += x1;
    __syncthreads();
  }
  int po = s_scan[0][tid] - sp, co = s_scan[1][tid] - sc;
  for (int j = j0; j < j1; ++j) {
    const int c = s_cnt[j];
    const int nch = (c + kRowsPerChunk - 1) / kRowsPerChunk;
    w.off[j] = po;
    w.choff[j] = co;
    for (int q = 0; q < nch; ++q) w.chunk[co + q] = j;
    s_cnt[j] = po;  // becomes the bucket's cursor
    po += c;
    co += nch;
  }
  if (tid == kBucketThreads - 1) {
    w.off[M] = s_scan[0][kBucketThreads - 1];
    w.choff[M] = s_scan[1][kBucketThreads - 1];
  }
  __syncthreads();
  if constexpr (STAGE > 0) {
    // s_cnt now holds each bucket's first position; start + rank stays below
    // the number of counted pairs (<= npairs <= STAGE).
#pragma unroll
    for (int u = 0; u < kPairUnroll; ++u)
      if (jf[u] >= 0) s_stage[s_cnt[jf[u]] + rk[u]] = tid + u * kBucketThreads;
    __syncthreads();
    const int total = s_scan[0][kBucketThreads - 1];
    for (int k = tid; k < total; k += kBucketThreads) w.pairs[k] = s_stage[k];
  } else {
#pragma unroll
    for (int u = 0; u < kPairUnroll; ++u)
      if (jf[u] >= 0) w.pairs[atomicAdd(&s_cnt[jf[u]], 1)] = tid + u * kBucketThreads;
    for (int i0 = tid + kRound; i0 < npairs; i0 += kBucketThreads * kPairTail) {
      int jv[kPairTail];
      bucket_round(A, i0, npairs, topk, magic, M, jv);
#pragma unroll
      for (int u = 0; u < kPairTail; ++u)
        if (jv[u] >= 0) w.pairs[atomicAdd(&s_cnt[jv[u]], 1)] = i0 + u * kBucketThreads;
    }
  }
}

// One wave per (chunk, head).  Lane l works on chunk row n = l % 32 and
// half hh = l / 32 for the scores, and on output dims 2l, 2l+1 for P.V.
//  * A fragment of step s (dims 64 hh + 8 s .. +8, the summation-order
//    permutation shared by A and B): K row n; B fragment: q of chunk row n
//    (rows past the chunk repeat row 0; their results are never used).
//  * C register r of lane l holds the score of key 8 (r / 4) + 4 hh + r % 4
//    for chunk row n.
//  * P goes through a wave-private LDS tile [32 rows][kPStride]; each output
//    row then reads its 32 probabilities (broadcast reads) against the lane's
//    two V columns, kept in fp32.  V of keys past every row's position is
//    replaced by 0 (such slots may hold anything, NaN included, and a masked
//    key's probability 0 must not meet it).
__global__ __launch_bounds__(kBlockWaves * kWave) void attn_prefill_block_kernel(PrefillAttnArgs a) {
  __shared__ __attribute__((aligned(16))) float s_p[kBlockWaves][kRowsPerChunk * kPStride];
  const AttnArgs& A = a.attn;
  const WsView w = ws_view(a);
  const int wave = wave_id();
  const int64_t unit = (int64_t)blockIdx.x * kBlockWaves + wave;
  const int g = (int)(unit / A.heads);
  const int h = (int)(unit - (int64_t)g * A.heads);
  if (g >= w.choff[A.max_blocks]) return;
  const int j = w.chunk[g];
  const int start = w.off[j] + (g - w.choff[j]) * kRowsPerChunk;
  const int n_rows = min(kRowsPerChunk, w.off[j + 1] - start);
  const int pb = A.block_table[j];  // sequence 0
  const bool ok = pb >= 0 && (int64_t)pb < A.num_blocks;
  const int lane = lane_id();
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int pair_v = w.pairs[start + (n < n_rows ? n : 0)];  // this lane's chunk row
  const int t_n = pair_v / A.topk;
  const int p_n = A.q_start + t_n;

  float m_row = -INFINITY, l_row = 0.0f;
  float vlo[kBlock], vhi[kBlock];  // V[k][2 lane], V[k][2 lane + 1]
  float* P = s_p[wave];
  if (ok) {
    const int64_t tile = ((int64_t)pb * A.heads + h) * (kBlock * kDim);
    const uint16_t* kt = A.k_pool + tile;
    const uint16_t* vt = A.v_pool + tile;
    const uint16_t* qr = A.q + ((int64_t)t_n * A.heads + h) * kDim;
    bf16x8_t av[8], bq[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      av[st] = *reinterpret_cast<const bf16x8_t*>(kt + n * kDim + 64 * hh + 8 * st);
      bq[st] = *reinterpret_cast<const bf16x8_t*>(qr + 64 * hh + 8 * st);
    }
    uint32_t vw[kBlock];
#pragma unroll
    for (int k = 0; k < kBlock; ++k) vw[k] = reinterpret_cast<const uint32_t*>(vt + k * kDim)[lane];
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
    int pmax = n < n_rows ? p_n : -1;
#pragma unroll
    for (int m_ = 1; m_ < kWave; m_ <<= 1) pmax = max(pmax, __shfl_xor(pmax, m_, kWave));
#pragma unroll
    for (int k = 0; k < kBlock; ++k) {
      const bool seen = j * kBlock + k <= pmax;
      vlo[k] = seen ? bf16_lo(vw[k]) : 0.0f;
      vhi[k] = seen ? bf16_hi(vw[k]) : 0.0f;
    }
  }
  // (m, l) of chunk row n, written by its lane in the lower half.
  if (hh == 0 && n < n_rows) {
    const int s_n = pair_v - t_n * A.topk;
    float* dst = w.part + (((int64_t)t_n * A.heads + h) * A.topk + s_n) * kPartStride;
    *reinterpret_cast<float2*>(dst + kDim) = make_float2(m_row, l_row);
  }
  for (int r = 0; r < n_rows; ++r) {
    const int i = __builtin_amdgcn_readlane(pair_v, r);
    const int t = i / A.topk;
    const int s_ = i - t * A.topk;
    float o0 = 0.0f, o1 = 0.0f;
    if (ok) {
#pragma unroll
      for (int k4 = 0; k4 < kBlock / 4; ++k4) {
        const float4 pr = *reinterpret_cast<const float4*>(P + r * kPStride + 4 * k4);
        o0 += pr.x * vlo[4 * k4] + pr.y * vlo[4 * k4 + 1] + pr.z * vlo[4 * k4 + 2] + pr.w * vlo[4 * k4 + 3];
        o1 += pr.x * vhi[4 * k4] + pr.y * vhi[4 * k4 + 1] + pr.z * vhi[4 * k4 + 2] + pr.w * vhi[4 * k4 + 3];
      }
    }
    float* dst = w.part + (((int64_t)t * A.heads + h) * A.topk + s_) * kPartStride;
    *reinterpret_cast<float2*>(dst + 2 * lane) = make_float2(o0, o1);
  }
}

// One wave per (row, head): log-sum-exp merge of the row's partials.  Lane s
// (< 64) takes slot s's (m, l) and weight; then every slot's two output
// values per lane are loaded together (weight 0 for slots that keep nothing)
// and lane d produces dims d and d + 64.  No kept token gives out = 0,
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

  float res0 = 0.0f, res1 = 0.0f, L = 0.0f, M = -INFINITY;
  for (int s0 = 0; s0 < A.topk; s0 += kWave) {  // one round for topk <= 64
    const int s = s0 + lane;
    const bool valid = s < A.topk && slot_counts(sel[s], p, A.max_blocks);
    float2 ml = make_float2(-INFINITY, 0.0f);
    if (valid) ml = *reinterpret_cast<const float2*>(base + (int64_t)s * kPartStride + kDim);
    float Mr = ml.x;
#pragma unroll
    for (int m_ = 1; m_ < kWave; m_ <<= 1) Mr = fmaxf(Mr, __shfl_xor(Mr, m_, kWave));
    if (Mr == -INFINITY) continue;
    // rescale what earlier rounds accumulated
    const float Mn = fmaxf(M, Mr);
    const float sc = exp2f(M - Mn);
    res0 *= sc;
    res1 *= sc;
    L *= sc;
    M = Mn;
    const float f = valid ? exp2f(ml.x - M) : 0.0f;
    float lf = ml.y * f;
#pragma unroll
    for (int m_ = 1; m_ < kWave; m_ <<= 1) lf += __shfl_xor(lf, m_, kWave);
    L += lf;
    const int ns = min(kWave, A.topk - s0);
    for (int u0 = 0; u0 < ns; u0 += 16) {
      float o0[16], o1[16], fu[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        fu[u] = u0 + u < ns ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(f), u0 + u)) : 0.0f;
        const float* ps = base + (int64_t)(s0 + u0 + u) * kPartStride;
        o0[u] = fu[u] != 0.0f ? ps[lane] : 0.0f;
        o1[u] = fu[u] != 0.0f ? ps[lane + kWave] : 0.0f;
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
  p.off_off = at;
  at = align256(at + (size_t)(max_blocks + 1) * 4);
  p.choff_off = at;
  at = align256(at + (size_t)(max_blocks + 1) * 4);
  p.pairs_off = at;
  at = align256(at + (size_t)npairs * 4);
  p.chunk_off = at;
  at = align256(at + (size_t)p.max_chunks * 4);
  p.part_off = at;
  at = align256(at + (size_t)npairs * heads * kPartStride * 4);
  p.ws_bytes = at;
  return p;
}

hipError_t launch_attn_prefill_blocks(const PrefillAttnArgs& a, hipStream_t stream) {
  const AttnArgs& A = a.attn;
  if (A.nq == 0) return hipSuccess;
  // Staged bucketing: counts for up to 4096 blocks (16 KB) and up to 32768
  // pairs (128 KB) in LDS, beside the 8 KB scan.
  if (A.max_blocks <= 4096 && (int64_t)A.nq * A.topk <= 32768)
    hipLaunchKernelGGL((attn_prefill_bucket_kernel<4096, 32768>), dim3(1), dim3(kBucketThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_prefill_bucket_kernel<kMaxBlocksAttnBucket, 0>), dim3(1), dim3(kBucketThreads), 0,
                       stream, a);
  const int64_t units = (int64_t)a.plan.max_chunks * A.heads;
  hipLaunchKernelGGL(attn_prefill_block_kernel, dim3((unsigned)((units + kBlockWaves - 1) / kBlockWaves)),
                     dim3(kBlockWaves * kWave), 0, stream, a);
  const int64_t items = (int64_t)A.nq * A.heads;
  hipLaunchKernelGGL(attn_prefill_merge_kernel, dim3((unsigned)((items + kMergeWaves - 1) / kMergeWaves)),
                     dim3(kMergeWaves * kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uocr
