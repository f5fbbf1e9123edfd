// Decode block selection (SR-SWA step 3, news.rkmt.cn/news/25027 Sec. 5):
// keep the query's local blocks and the (topk - local) highest-scoring remote
// candidates, ranked by score descending with the lower block id first on
// ties.
//
// One workgroup per sequence.  Scores become order-preserving uint32 keys
// (NaN lowest, -0.0 == +0.0).  A 4-pass radix select (8-bit digits, LDS
// histogram, block-wide scan) finds the exact key T of the last remote slot
// and how many keys equal to T are taken (the lowest ids among them).
//
// A register-resident fast variant serves contexts whose candidates fit
// (described below); very long contexts use the generic variant, which
// re-reads the scores from memory on every pass.
#include "device_common.h"
#include "kernels.h"
#include "select_common.h"

namespace uocr {

namespace {

// Shared prelude: query geometry, n_sel, trivial selections.  Returns true
// when the row is complete.
__device__ __forceinline__ bool topk_prelude(const TopkDecodeArgs& a, int b, int nt, int& ncand, int& R,
                                             int32_t*& out) {
  const int L = clamp_ctx(a.ctx_lens[b], a.max_blocks);
  const int nb = (L + kBlock - 1) / kBlock;
  ncand = nb - a.local_blocks > 0 ? nb - a.local_blocks : 0;
  R = a.topk - a.local_blocks;
  out = a.block_idx + (int64_t)b * a.topk;
  if (a.n_sel != nullptr && threadIdx.x == 0) a.n_sel[b] = nb < a.topk ? nb : a.topk;
  return select_trivial(nb, ncand, R, a.topk, out, nt);
}

}  // namespace

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_decode_reg_kernel(TopkDecodeArgs a) {
  __shared__ SelectSmem<NT> sm;
  const int b = blockIdx.x;
  int ncand, R;
  int32_t* out;
  if (topk_prelude(a, b, NT, ncand, R, out)) return;
  select_sorted_reg<NT, KPT>(a.block_scores + (int64_t)b * a.max_blocks, ncand, R, a.local_blocks, out, sm);
}

// ---------------------------------------------------------------------------
// Generic variant: any number of candidates, scores re-read on every pass.
// ---------------------------------------------------------------------------
constexpr int kGenThreads = 256;

__global__ __launch_bounds__(kGenThreads) void topk_decode_global_kernel(TopkDecodeArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_scratch[kGenThreads / kWave];
  __shared__ uint32_t s_digit, s_remaining;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int ncand, R;
  int32_t* out;
  if (topk_prelude(a, b, kGenThreads, ncand, R, out)) return;
  const float* sc = a.block_scores + (int64_t)b * a.max_blocks;

  uint32_t prefix = 0, prefix_mask = 0, remaining = (uint32_t)R;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < ncand; j += kGenThreads) {
      const uint32_t key = order_key(sc[j]);
      if ((key & prefix_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t c = hist[255 - tid];
    uint32_t total;
    const uint32_t cum = block_incl_scan<kGenThreads>(c, scan_scratch, &total);
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
  const uint32_t need_eq = remaining;

  uint32_t eq_seen = 0, taken = 0;
  for (int base = 0; base < ncand; base += kGenThreads) {
    const int j = base + tid;
    uint32_t key = 0;
    const bool in = j < ncand;
    if (in) key = order_key(sc[j]);
    const uint32_t eq = (in && key == T) ? 1u : 0u;
    uint32_t eq_total;
    const uint32_t eq_incl = block_incl_scan<kGenThreads>(eq, scan_scratch, &eq_total);
    const uint32_t eq_before = eq_seen + eq_incl - eq;
    const uint32_t take = (in && (key > T || (eq && eq_before < need_eq))) ? 1u : 0u;
    uint32_t take_total;
    const uint32_t take_incl = block_incl_scan<kGenThreads>(take, scan_scratch, &take_total);
    const uint32_t pos = taken + take_incl - 1;
    if (take && pos < (uint32_t)R) out[pos] = j;
    eq_seen += eq_total;
    taken += take_total;
  }
  for (int i = tid; i < a.local_blocks; i += kGenThreads) out[R + i] = ncand + i;
}

hipError_t launch_topk_decode(const TopkDecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int64_t max_cand = (int64_t)a.max_blocks - a.local_blocks;
  if (max_cand <= 256 * 16) {
    hipLaunchKernelGGL((topk_decode_reg_kernel<256, 16>), dim3(a.batch), dim3(256), 0, stream, a);
  } else if (max_cand <= 1024 * 16) {
    hipLaunchKernelGGL((topk_decode_reg_kernel<1024, 16>), dim3(a.batch), dim3(1024), 0, stream, a);
  } else {
    hipLaunchKernelGGL(topk_decode_global_kernel, dim3(a.batch), dim3(kGenThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace uocr
