// Sparse gather attention over the kept blocks (SR-SWA step 4,
// news.rkmt.cn/news/25027 Sec. 5): per head, exact softmax over the tokens of
// the kept blocks that the query may see (token <= p), times V.  Decode and
// chunked prefill share the kernel; a prefill row is a query of sequence 0
// at p = q_start + row.
//
// One 1024-thread workgroup per (query, head): the kept blocks are split over
// its 16 waves (split-K; at 16 kept blocks every block's K and V loads are in
// flight at once), each wave keeps an online-softmax state (running
// max, sum, 128-dim accumulator; attend_block in attn_common.h) and the
// waves' states are merged through LDS at the end.  Arithmetic is fp32 with
// exp2 on log2e-scaled logits; the output is fp32.
#include "attn_common.h"
#include "device_common.h"
#include "kernels.h"
#include "select_common.h"

namespace uocr {

namespace {
constexpr int kAttnThreads = 1024;
}  // namespace

// Attention of query qi, head h over the kept blocks in sel[0 .. topk)
// (global or LDS memory); every thread of the 1024-thread workgroup calls it.
__device__ __forceinline__ void attend_query(const AttnArgs& a, int qi, int h, const int32_t* sel) {
  __shared__ AttendSmem<kAttnThreads> sm;
  int seq, p;
  if (a.prefill) {
    seq = 0;
    p = a.q_start + qi;
  } else {
    seq = qi;
    p = clamp_ctx(a.ctx_lens[qi], a.max_blocks) - 1;
  }
  const int64_t head_row = (int64_t)qi * a.heads + h;
  const int32_t* table = a.block_table + (int64_t)seq * a.max_blocks;
  float* lse = a.lse != nullptr ? a.lse + head_row : nullptr;
  if (a.prefill)  // rows of a chunk share tiles: cached loads
    attend_query_wg<kAttnThreads, false>(a.k_pool, a.v_pool, table, a.num_blocks, a.heads, h, a.max_blocks, p,
                                         a.q + head_row * kDim, sel, a.topk, a.scale_log2, a.out + head_row * kDim,
                                         lse, sm);
  else  // decode: every kept tile is read once
    attend_query_wg<kAttnThreads, true>(a.k_pool, a.v_pool, table, a.num_blocks, a.heads, h, a.max_blocks, p,
                                        a.q + head_row * kDim, sel, a.topk, a.scale_log2, a.out + head_row * kDim,
                                        lse, sm);
}

__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnArgs a) {
  attend_query(a, blockIdx.x, blockIdx.y, a.block_idx + (int64_t)blockIdx.x * a.topk);
}

// Decode steps 3 and 4 in one launch (with page tags, the page-aware
// ranking of step 3): workgroup (b, h) selects the kept blocks of sequence b
// itself (the 10 head workgroups of a sequence repeat
// the same deterministic selection), keeps them in LDS and attends; the head-0
// workgroup also writes the selection out.  This saves the separate
// selection launch and its drain/fill gap between the scoring and attention
// launches of a layer.
template <int KPT>
__global__ __launch_bounds__(kAttnThreads) void select_attn_kernel(SelAttnArgs sa) {
  __shared__ SelectSmem<kAttnThreads> sm;
  __shared__ int32_t s_blocks[kMaxFusedTopk];
  const AttnArgs& a = sa.attn;
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int L = clamp_ctx(a.ctx_lens[b], a.max_blocks);
  const int nb = (L + kBlock - 1) / kBlock;
  const int ncand = nb - sa.local_blocks > 0 ? nb - sa.local_blocks : 0;
  const int R = a.topk - sa.local_blocks;
  if (!select_trivial(nb, ncand, R, a.topk, s_blocks, kAttnThreads))
    select_sorted_reg<kAttnThreads, KPT>(sa.block_scores + (int64_t)b * a.max_blocks, ncand, R, sa.local_blocks,
                                         s_blocks, sm,
                                         sa.block_page != nullptr ? sa.block_page + (int64_t)b * a.max_blocks : nullptr,
                                         sa.block_page != nullptr ? sa.query_page[b] : 0);
  __syncthreads();
  if (h == 0) {
    for (int i = threadIdx.x; i < a.topk; i += kAttnThreads) sa.block_idx_out[(int64_t)b * a.topk + i] = s_blocks[i];
    if (sa.n_sel != nullptr && threadIdx.x == 0) sa.n_sel[b] = nb < a.topk ? nb : a.topk;
  }
  attend_query(a, b, h, s_blocks);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.nq == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_kernel, dim3(a.nq, a.heads), dim3(kAttnThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select_attn(const SelAttnArgs& a, hipStream_t stream) {
  if (a.attn.nq == 0) return hipSuccess;
  const int64_t max_cand = (int64_t)a.attn.max_blocks - a.local_blocks;
  const dim3 grid(a.attn.nq, a.attn.heads);
  if (max_cand <= kAttnThreads * 4) {
    hipLaunchKernelGGL(select_attn_kernel<4>, grid, dim3(kAttnThreads), 0, stream, a);
  } else if (max_cand <= kAttnThreads * 16) {
    hipLaunchKernelGGL(select_attn_kernel<16>, grid, dim3(kAttnThreads), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace uocr
