// Decode indexer scoring with fused block max (SR-SWA step 2,
// news.rkmt.cn/news/25027 Sec. 5): for each sequence, every key of every
// remote-candidate block is scored against the one-head 128-dim indexer
// query, and each block keeps the maximum of its 32 key scores.
//
// The indexer-K cache is streamed once at HBM rate: one wave scores one 8 KB
// block at a time (score_block_wave in indexer_common.h), the workgroups of
// a sequence split its blocks into chunks.
#include "device_common.h"
#include "indexer_common.h"
#include "kernels.h"

namespace uocr {

__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerDecodeArgs a) {
  const int b = blockIdx.y;
  const int j0 = blockIdx.x * a.chunk;
  if (j0 >= a.max_blocks) return;
  const int L = clamp_ctx(a.ctx_lens[b], a.max_blocks);
  const int nb = (L + kBlock - 1) / kBlock;
  const int ncand = nb - a.local_blocks > 0 ? nb - a.local_blocks : 0;
  const int jend_all = min(j0 + a.chunk, a.max_blocks);
  float* out = a.block_scores + (int64_t)b * a.max_blocks;

  // Non-candidate entries of this chunk (local, future, padding): -inf.
  for (int j = max(j0, ncand) + (int)threadIdx.x; j < jend_all; j += blockDim.x) out[j] = -INFINITY;

  const int jend = min(jend_all, ncand);
  if (j0 >= jend) return;

  const int lane = lane_id();
  const int wave = wave_id();
  const int nwaves = blockDim.x / kWave;
  const uint4 qv = *reinterpret_cast<const uint4*>(a.q_idx + (int64_t)b * kDim + (lane & 15) * 8);
  const int32_t* table = a.block_table + (int64_t)b * a.max_blocks;

  for (int j = j0 + wave; j < jend; j += nwaves) {
    const int pb = __builtin_amdgcn_readfirstlane(table[j]);
    const float score = (pb < 0 || (int64_t)pb >= a.num_blocks)
                            ? __builtin_nanf("")
                            : score_block_wave(a.kidx_pool + (int64_t)pb * (kBlock * kDim), qv);
    if (lane == 0) out[j] = score;
  }
}

int32_t indexer_decode_chunk(int32_t batch, int32_t max_blocks) {
  // Aim at ~2048 workgroups (8 per CU) so that enough 8 KB loads are in flight.
  int64_t total = (int64_t)batch * max_blocks;
  int64_t c = (total + 2047) / 2048;
  if (c < 8) c = 8;
  c = (c + 3) & ~int64_t(3);
  if (c > max_blocks) c = max_blocks;
  return (int32_t)c;
}

hipError_t launch_indexer_decode(const IndexerDecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  dim3 grid((a.max_blocks + a.chunk - 1) / a.chunk, a.batch);
  hipLaunchKernelGGL(indexer_decode_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uocr
