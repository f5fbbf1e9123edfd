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
// and taken in a grid-stride loop, so a ragged batch's empty units (past a
// short sequence's candidates) cost a workgroup one -inf store each instead
// of a whole launch slot, and the live units spread over every workgroup.
// Each wave keeps two 8 KB tiles in flight (blocks j and j + 4 of the unit).
constexpr int kIdxThreads = 256;
constexpr int kIdxWaves = kIdxThreads / kWave;
constexpr int kIdxGrid = 2048;  // resident workgroups: 8 per CU

__global__ __launch_bounds__(kIdxThreads) void indexer_decode_kernel(IndexerDecodeArgs a) {
  const int lane = lane_id();
  const int wave = wave_id();
  const int M = a.max_blocks;
  const int C = (M + a.chunk - 1) / a.chunk;
  const int64_t units = (int64_t)a.batch * C;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int b = (int)(u / C);
    const int j0 = (int)(u - (int64_t)b * C) * a.chunk;
    const int L = clamp_ctx(a.ctx_lens[b], M);
    const int nb = (L + kBlock - 1) / kBlock;
    const int ncand = nb - a.local_blocks > 0 ? nb - a.local_blocks : 0;
    const int jend_all = min(j0 + a.chunk, M);
    float* out = a.block_scores + (int64_t)b * M;

    // Non-candidate entries of this unit (local, future, padding): -inf.
    for (int j = max(j0, ncand) + (int)threadIdx.x; j < jend_all; j += kIdxThreads) out[j] = -INFINITY;

    const int jend = min(jend_all, ncand);
    if (j0 >= jend) continue;
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
  hipLaunchKernelGGL(indexer_decode_kernel, dim3((unsigned)grid), dim3(kIdxThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uocr
