// Decode block selection (SR-SWA step 3, news.rkmt.cn/news/25027 Sec. 5):
// keep the query's local blocks and the (topk - local) highest-scoring remote
// candidates, ranked by score descending with the lower block id first on
// ties.
//
// One 256-thread workgroup per sequence.  Scores become order-preserving
// uint32 keys (NaN lowest, -0.0 == +0.0).  A 4-pass radix select (8-bit
// digits, LDS histogram, block-wide scan) finds the exact key T of the last
// remote slot and how many keys equal to T are taken; a compaction pass in
// block-id order then emits every key > T and the first such keys == T, so
// the output is ascending and the lowest-id tie rule holds by construction.
#include "device_common.h"
#include "kernels.h"

namespace uocr {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Inclusive prefix sum over the 256 threads of the workgroup.  `scratch`
// holds kWaves entries.  Returns the inclusive sum; *total gets the block sum.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
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

}  // namespace

__global__ __launch_bounds__(kThreads) void topk_decode_kernel(TopkDecodeArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_scratch[kWaves];
  __shared__ uint32_t s_digit, s_remaining;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = clamp_ctx(a.ctx_lens[b], a.max_blocks);
  const int nb = (L + kBlock - 1) / kBlock;
  const int ncand = nb - a.local_blocks > 0 ? nb - a.local_blocks : 0;
  const int R = a.topk - a.local_blocks;
  int32_t* out = a.block_idx + (int64_t)b * a.topk;
  if (a.n_sel != nullptr && tid == 0) a.n_sel[b] = nb < a.topk ? nb : a.topk;

  if (ncand <= R) {
    // Every block 0..nb-1 is kept (remote candidates then the local window).
    for (int i = tid; i < a.topk; i += kThreads) out[i] = i < nb ? i : -1;
    return;
  }

  if (R == 0) {
    // Only the local window is kept.
    for (int i = tid; i < a.topk; i += kThreads) out[i] = ncand + i;
    return;
  }

  const float* sc = a.block_scores + (int64_t)b * a.max_blocks;

  // ---- radix select of the R-th largest key --------------------------------
  uint32_t prefix = 0, prefix_mask = 0, remaining = (uint32_t)R;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < ncand; j += kThreads) {
      const uint32_t key = order_key(sc[j]);
      if ((key & prefix_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // Thread t looks at digit 255 - t: an inclusive scan from the top digit
    // down finds the digit whose bin holds the remaining-th largest key.
    const uint32_t c = hist[255 - tid];
    uint32_t total;
    const uint32_t cum = block_incl_scan(c, scan_scratch, &total);
    if (cum >= remaining && cum - c < remaining) {
      s_digit = 255u - (uint32_t)tid;
      s_remaining = remaining - (cum - c);
    }
    __syncthreads();
    prefix |= s_digit << shift;
    prefix_mask |= 255u << shift;
    remaining = s_remaining;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = remaining;  // keys == T to take, lowest ids first

  // ---- compaction in block-id order ----------------------------------------
  uint32_t eq_seen = 0, taken = 0;
  for (int base = 0; base < ncand; base += kThreads) {
    const int j = base + tid;
    uint32_t key = 0;
    bool in = j < ncand;
    if (in) key = order_key(sc[j]);
    const uint32_t eq = (in && key == T) ? 1u : 0u;
    uint32_t eq_total;
    const uint32_t eq_incl = block_incl_scan(eq, scan_scratch, &eq_total);
    const uint32_t eq_before = eq_seen + eq_incl - eq;
    const uint32_t take = (in && (key > T || (eq && eq_before < need_eq))) ? 1u : 0u;
    uint32_t take_total;
    const uint32_t take_incl = block_incl_scan(take, scan_scratch, &take_total);
    const uint32_t pos = taken + take_incl - 1;
    if (take && pos < (uint32_t)R) out[pos] = j;
    eq_seen += eq_total;
    taken += take_total;
  }
  // Local window after the remote ids (all larger than every candidate).
  for (int i = tid; i < a.local_blocks; i += kThreads) out[R + i] = ncand + i;
}

hipError_t launch_topk_decode(const TopkDecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_decode_kernel, dim3(a.batch), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uocr
