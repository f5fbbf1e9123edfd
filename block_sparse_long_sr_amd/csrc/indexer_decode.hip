// Decode indexer scoring with fused block max (SR-SWA step 2,
// news.rkmt.cn/news/25027 Sec. 5): for each sequence, every key of every
// remote-candidate block is scored against the one-head 128-dim indexer
// query, and each block keeps the maximum of its 32 key scores.
//
// The indexer-K cache is streamed once at HBM rate: one wave scores 8 KB
// blocks (block_max_of_tile in indexer_common.h), two at a time.
#include "device_common.h"
#include "indexer_common.h"
#include "kernels.h"

namespace uocr {

// Work units are (sequence, chunk of `chunk` blocks), numbered sequence-major
// and taken in a grid-stride loop.  Batches of up to kIdxThreads sequences
// number only the live units (those holding remote candidates): thread b
// counts sequence b's units, a workgroup scan puts each sequence's first
// unit in LDS, and a unit's sequence is found with ballots over those first
// units, so every workgroup's units are live ones, spread evenly; the
// non-candidate entries (local window, future, padding: -inf) of sequence b
// are written by workgroup b mod gridDim.  Larger batches take every
// (sequence, chunk) unit, where an empty unit costs its workgroup one round
// trip and the -inf stores.  Each wave keeps two 8 KB tiles in flight
// (blocks j and j + 4 of the unit).
constexpr int kIdxThreads = 256;
constexpr int kIdxWaves = kIdxThreads / kWave;
constexpr int kIdxGrid = 2048;  // resident workgroups: 8 per CU

// Blocks [j0, jend) of sequence b (all remote candidates).
__device__ __forceinline__ void score_unit(const IndexerDecodeArgs& a, int b, int j0, int jend) {
  const int lane = lane_id();
  const int wave = wave_id();
  const int M = a.max_blocks;
  float* out = a.block_scores + (int64_t)b * M;
  const uint4 qv = *reinterpret_cast<const uint4*>(a.q_idx + (int64_t)b * kDim + (lane & 15) * 8);
  const int32_t* table = a.block_table + (int64_t)b * M;
  for (int j = j0 + wave; j < jend; j += 2 * kIdxWaves) {
    const int j2 = j + kIdxWaves;
    const int pb = __builtin_amdgcn_readfirstlane(table[j]);
    const int pb2 = j2 < jend ? __builtin_amdgcn_readfirstlane(table[j2]) : -1;
    const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks;
    const bool ok2 = pb2 >= 0 && (int64_t)pb2 < a.num_blocks;
    uint4 kv[8], kv2[8];
    load_index_tile(a.kidx_pool + (int64_t)(ok ? pb : 0) * (kBlock * kDim), kv);
    load_index_tile(a.kidx_pool + (int64_t)(ok2 ? pb2 : 0) * (kBlock * kDim), kv2);
    const float s1 = ok ? block_max_of_tile(kv, qv) : __builtin_nanf("");
    const float s2 = ok2 ? block_max_of_tile(kv2, qv) : __builtin_nanf("");
    if (lane == 0) {
      out[j] = s1;
      if (j2 < jend) out[j2] = s2;
    }
  }
}

__device__ __forceinline__ int remote_candidates(const IndexerDecodeArgs& a, int b) {
  const int L = clamp_ctx(a.ctx_lens[b], a.max_blocks);
  const int nb = (L + kBlock - 1) / kBlock;
  return nb - a.local_blocks > 0 ? nb - a.local_blocks : 0;
}

template <bool LIVE>
__global__ __launch_bounds__(kIdxThreads) void indexer_decode_kernel(IndexerDecodeArgs a) {
  const int M = a.max_blocks;
  const int C = (M + a.chunk - 1) / a.chunk;
  if constexpr (LIVE) {
    __shared__ int32_t s_first[kIdxThreads];  // first live unit of each sequence
    __shared__ int32_t s_ncand[kIdxThreads];
    __shared__ int32_t s_wsum[kIdxWaves];
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = wave_id();
    const int nc = tid < a.batch ? remote_candidates(a, tid) : 0;
    const int nu = (nc + a.chunk - 1) / a.chunk;
    const int incl = wave_incl_sum(nu);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kIdxWaves; ++w) {
      before += w < wave ? s_wsum[w] : 0;
      total += s_wsum[w];
    }
    if (tid < a.batch) {
      s_first[tid] = before + incl - nu;
      s_ncand[tid] = nc;
    }
    __syncthreads();
    for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
      float* out = a.block_scores + (int64_t)b * M;
      for (int j = s_ncand[b] + tid; j < M; j += kIdxThreads) out[j] = -INFINITY;
    }
    for (int u = blockIdx.x; u < total; u += gridDim.x) {
      // the unit's sequence: the last one whose first unit is at or below u
      int cnt = 0;
      for (int b0 = 0; b0 < a.batch; b0 += kWave) {
        const int b = b0 + lane;
        cnt += __popcll(__ballot(b < a.batch && s_first[b] <= u));
      }
      const int b = cnt - 1;
      const int j0 = (u - s_first[b]) * a.chunk;
      score_unit(a, b, j0, min(j0 + a.chunk, s_ncand[b]));
    }
  } else {
    const int64_t units = (int64_t)a.batch * C;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
      const int b = (int)(u / C);
      const int j0 = (int)(u - (int64_t)b * C) * a.chunk;
      const int ncand = remote_candidates(a, b);
      const int jend_all = min(j0 + a.chunk, M);
      float* out = a.block_scores + (int64_t)b * M;
      // Non-candidate entries of this unit (local, future, padding): -inf.
      for (int j = max(j0, ncand) + (int)threadIdx.x; j < jend_all; j += kIdxThreads) out[j] = -INFINITY;
      const int jend = min(jend_all, ncand);
      if (j0 < jend) score_unit(a, b, j0, jend);
    }
  }
}

int32_t indexer_decode_chunk(int32_t batch, int32_t max_blocks) {
  // One round of two tiles per wave: 8 blocks per unit.
  (void)batch;
  return max_blocks < 2 * kIdxWaves ? max_blocks : 2 * kIdxWaves;
}

hipError_t launch_indexer_decode(const IndexerDecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int64_t units = (int64_t)a.batch * ((a.max_blocks + a.chunk - 1) / a.chunk);
  const int64_t grid = units < kIdxGrid ? units : kIdxGrid;
  if (a.batch <= kIdxThreads)
    hipLaunchKernelGGL(indexer_decode_kernel<true>, dim3((unsigned)grid), dim3(kIdxThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(indexer_decode_kernel<false>, dim3((unsigned)grid), dim3(kIdxThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uocr
