// Sparse gather attention over the kept blocks (SR-SWA step 4,
// news.rkmt.cn/news/25027 Sec. 5): per head, exact softmax over the tokens of
// the kept blocks that the query may see (token <= p), times V.  Decode and
// chunked prefill share the kernel; a prefill row is a query of sequence 0
// at p = q_start + row.
//
// One workgroup per (query, head): the kept blocks are split over its waves
// (split-K; with 1024 threads and 16 kept blocks every block's K and V loads
// are in flight at once), each wave keeps an online-softmax state (running
// max, sum, 128-dim accumulator; attend_block in attn_common.h) and the
// waves' states are merged through LDS at the end.  Arithmetic is fp32 with
// exp2 on log2e-scaled logits; the output is fp32.
#include "attn_common.h"
#include "device_common.h"
#include "kernels.h"
#include "select_common.h"

namespace uocr {

// Workgroup size: 1024 threads (16 waves, one kept block each: every K and V
// load of a head is in flight at once) when the (query, head) workgroups fit
// in one round on the chip; 512 threads (8 waves, two blocks each; three
// workgroups per CU for the fused kernel, two for the plain one) for larger
// launches, whose 1024-thread workgroups
// would run in several rounds of one per CU.  Measured on 16 queries: 15.2
// against 17.3 us; on 64 ragged queries: 31.4 against 41.5 us.
namespace {
int attn_threads(int64_t workgroups) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0) cus = c;
  }
  return workgroups > cus ? 512 : 1024;
}
}  // namespace

// Attention of query qi, head h over the kept blocks in sel[0 .. topk)
// (global or LDS memory); every thread of the NT-thread workgroup calls it.
// `row` (global or LDS), when given, is the query's block-table row.
template <int NT>
__device__ __forceinline__ void attend_query(const AttnArgs& a, int qi, int h, const int32_t* sel,
                                             const int32_t* row = nullptr) {
  __shared__ AttendSmem<NT> sm;
  int seq, p;
  if (a.prefill) {
    seq = 0;
    p = a.q_start + qi;
  } else {
    seq = qi;
    p = clamp_ctx(a.ctx_lens[qi], a.max_blocks) - 1;
  }
  const int64_t head_row = (int64_t)qi * a.heads + h;
  const int32_t* table = row != nullptr ? row : a.block_table + (int64_t)seq * a.max_blocks;
  float* lse = a.lse != nullptr ? a.lse + head_row : nullptr;
  if (a.prefill)  // rows of a chunk share tiles: cached loads
    attend_query_wg<NT, false>(a.k_pool, a.v_pool, table, a.num_blocks, a.heads, h, a.max_blocks, p,
                               a.q + head_row * kDim, sel, a.topk, a.scale_log2, a.out + head_row * kDim, lse, sm);
  else  // decode: every kept tile is read once
    attend_query_wg<NT, true>(a.k_pool, a.v_pool, table, a.num_blocks, a.heads, h, a.max_blocks, p,
                              a.q + head_row * kDim, sel, a.topk, a.scale_log2, a.out + head_row * kDim, lse, sm);
}

template <int NT>
__global__ __launch_bounds__(NT) void attn_kernel(AttnArgs a) {
  attend_query<NT>(a, blockIdx.x, blockIdx.y, a.block_idx + (int64_t)blockIdx.x * a.topk);
}

// Decode steps 3 and 4 in one launch (with page tags, the page-aware
// ranking of step 3): workgroup (b, h) selects the kept blocks of sequence b
// itself (the 10 head workgroups of a sequence repeat
// the same deterministic selection), keeps them in LDS and attends; the head-0
// workgroup also writes the selection out.  This saves the separate
// selection launch and its drain/fill gap between the scoring and attention
// launches of a layer.
// The sequence's block-table row is copied to LDS (rows up to
// kFusedTableCache entries) while the scores are read and ranked, so the
// kept ids are followed by one memory round trip, the K and V tiles.
constexpr int kFusedTableCache = 4096;

// The 512-thread variant is held to 80 VGPRs (six waves per SIMD, three
// workgroups per CU), so a batch's (query, head) workgroups up to three per
// CU are resident at once (64 ragged queries, 640 workgroups: 34.5 -> 33.4
// us; at 100 VGPRs two per CU left a second round).  The plain attention
// kernel measured slower under the same bound (28.6 -> 31.2 us) and keeps
// its registers.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 512 ? 6 : 4))) void select_attn_kernel(
    SelAttnArgs sa) {
  __shared__ SelectSmem<NT> sm;
  __shared__ int32_t s_blocks[kMaxFusedTopk];
  __shared__ int32_t s_table[kFusedTableCache];
  const AttnArgs& a = sa.attn;
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int L = clamp_ctx(a.ctx_lens[b], a.max_blocks);
  const int nb = (L + kBlock - 1) / kBlock;
  const int ncand = nb - sa.local_blocks > 0 ? nb - sa.local_blocks : 0;
  const int R = a.topk - sa.local_blocks;
  const bool cached = a.max_blocks <= kFusedTableCache;
  if (cached) {
    const int32_t* row = a.block_table + (int64_t)b * a.max_blocks;
    for (int i = threadIdx.x; i < nb; i += NT) s_table[i] = row[i];
  }
  if (!select_trivial(nb, ncand, R, a.topk, s_blocks, NT))
    select_sorted_reg<NT, KPT>(sa.block_scores + (int64_t)b * a.max_blocks, ncand, R, sa.local_blocks, s_blocks, sm,
                               sa.block_page != nullptr ? sa.block_page + (int64_t)b * a.max_blocks : nullptr,
                               sa.block_page != nullptr ? sa.query_page[b] : 0);
  __syncthreads();
  if (h == 0) {
    for (int i = threadIdx.x; i < a.topk; i += NT) sa.block_idx_out[(int64_t)b * a.topk + i] = s_blocks[i];
    if (sa.n_sel != nullptr && threadIdx.x == 0) sa.n_sel[b] = nb < a.topk ? nb : a.topk;
  }
  attend_query<NT>(a, b, h, s_blocks, cached ? s_table : nullptr);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  const dim3 grid(a.nq, a.heads);
  if (attn_threads((int64_t)a.nq * a.heads) == 512)
    hipLaunchKernelGGL(attn_kernel<512>, grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_kernel<1024>, grid, dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select_attn(const SelAttnArgs& a, hipStream_t stream) {
  if (a.attn.nq == 0) return hipSuccess;
  const int64_t max_cand = (int64_t)a.attn.max_blocks - a.local_blocks;
  const dim3 grid(a.attn.nq, a.attn.heads);
  // 512 threads hold up to 16 candidate keys each (8192 candidates); longer
  // contexts keep 1024 threads
  if (attn_threads((int64_t)a.attn.nq * a.attn.heads) == 512 && max_cand <= 512 * 16) {
    if (max_cand <= 512 * 4)
      hipLaunchKernelGGL((select_attn_kernel<512, 4>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((select_attn_kernel<512, 16>), grid, dim3(512), 0, stream, a);
  } else if (max_cand <= 1024 * 4) {
    hipLaunchKernelGGL((select_attn_kernel<1024, 4>), grid, dim3(1024), 0, stream, a);
  } else if (max_cand <= 1024 * 16) {
    hipLaunchKernelGGL((select_attn_kernel<1024, 16>), grid, dim3(1024), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace uocr
