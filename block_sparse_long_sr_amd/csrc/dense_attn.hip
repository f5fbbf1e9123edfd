// Dense full-context decode attention: the comparator for the pages'
// per-step speed claim against full attention (leheavengame.com OCR 2
// release article, Sec. 1: per-step decoding 7.0x faster than full
// attention).  Each query attends to every cached token 0..p of its
// sequence (p = ctx_len - 1), per head, with the same block-major caches,
// arithmetic and output conventions as the sparse path (SR-SWA step 4 over
// all blocks instead of the kept ones).
//
// Split-K flash decoding: workgroup (split, head, sequence) streams one
// range of blocks with 4 waves, one block per wave at a time (attend_block);
// the waves' online-softmax states are merged in LDS and written as the
// split's partial (max, sum, 128-dim unnormalised output) to the workspace.
// A second kernel merges a query-head's partials into out and lse.  The
// K/V caches are read exactly once, so the kernel is bound by HBM.
#include "attn_common.h"
#include "device_common.h"
#include "kernels.h"

namespace uocr {

namespace {
constexpr int kDenseThreads = 256;
constexpr int kDenseWaves = kDenseThreads / kWave;
}  // namespace

DensePlan dense_plan(int32_t batch, int32_t heads, int32_t max_blocks) {
  DensePlan p{};
  // Splits of at least 64 blocks, about 2048 workgroups over the launch.
  const int64_t pairs = (int64_t)batch * heads;
  int64_t nsplit = pairs > 0 ? (2048 + pairs - 1) / pairs : 1;
  const int64_t max_split = (max_blocks + 63) / 64;
  if (nsplit > max_split) nsplit = max_split;
  if (nsplit < 1) nsplit = 1;
  p.nsplit = (int32_t)nsplit;
  p.bps = (int32_t)((max_blocks + nsplit - 1) / nsplit);
  p.ws_bytes = (size_t)pairs * (size_t)p.nsplit * (kDim + 2) * sizeof(float);
  return p;
}

__global__ __launch_bounds__(kDenseThreads) void dense_attn_partial_kernel(DenseArgs a) {
  __shared__ float s_m[kDenseWaves];
  __shared__ float s_l[kDenseWaves];
  __shared__ float s_o[kDenseWaves][kDim];
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = lane_id();
  const int wave = wave_id();
  const int c8 = (lane & 15) * 8;

  const int L = clamp_ctx(a.ctx_lens[b], a.max_blocks);
  const int p = L - 1;
  const int nb = (L + kBlock - 1) / kBlock;
  const int j0 = split * a.plan.bps;
  const int j1 = min(j0 + a.plan.bps, nb);
  const int64_t head_row = (int64_t)b * a.heads + h;
  const uint4 qv = *reinterpret_cast<const uint4*>(a.q + head_row * kDim + c8);
  const int32_t* table = a.block_table + (int64_t)b * a.max_blocks;

  float m = -INFINITY, l = 0.0f, o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = 0.0f;
  for (int j = j0 + wave; j < j1; j += kDenseWaves) {
    const int pb = __builtin_amdgcn_readfirstlane(table[j]);
    if (pb < 0 || (int64_t)pb >= a.num_blocks) continue;
    const int64_t tile = ((int64_t)pb * a.heads + h) * (kBlock * kDim);
    attend_block<true>(a.k_pool + tile, a.v_pool + tile, j, p, qv, a.scale_log2, m, l, o);
  }
  reduce_key_groups(l, o);
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
  if (lane < 16) {
#pragma unroll
    for (int d = 0; d < 8; ++d) s_o[wave][c8 + d] = o[d];
  }
  __syncthreads();

  // Partial of this split: max M over the waves, sum and output rescaled to M.
  float* part = a.ws + (head_row * a.plan.nsplit + split) * (kDim + 2);
  if (threadIdx.x < kDim) {
    const int d = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDenseWaves; ++w) M = fmaxf(M, s_m[w]);
    float Ls = 0.0f, acc = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDenseWaves; ++w) {
        const float f = exp2f(s_m[w] - M);
        Ls += s_l[w] * f;
        acc += s_o[w][d] * f;
      }
    }
    part[2 + d] = acc;
    if (d == 0) {
      part[0] = M;
      part[1] = Ls;
    }
  }
}

__global__ __launch_bounds__(kDim) void dense_attn_merge_kernel(DenseArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int64_t head_row = (int64_t)b * a.heads + h;
  const float* part = a.ws + head_row * a.plan.nsplit * (kDim + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.plan.nsplit; ++s) M = fmaxf(M, part[s * (kDim + 2)]);
  float res = 0.0f, lse_v = -INFINITY;
  if (M != -INFINITY) {
    float Ls = 0.0f, acc = 0.0f;
    for (int s = 0; s < a.plan.nsplit; ++s) {
      const float* ps = part + s * (kDim + 2);
      const float f = exp2f(ps[0] - M);
      Ls += ps[1] * f;
      acc += ps[2 + d] * f;
    }
    res = acc / Ls;
    lse_v = (M + log2f(Ls)) * kLn2;
  }
  a.out[head_row * kDim + d] = res;
  if (a.lse != nullptr && d == 0) a.lse[head_row] = lse_v;
}

hipError_t launch_dense_attn(const DenseArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(dense_attn_partial_kernel, dim3(a.plan.nsplit, a.heads, a.batch), dim3(kDenseThreads), 0,
                     stream, a);
  hipLaunchKernelGGL(dense_attn_merge_kernel, dim3(a.heads, a.batch), dim3(kDim), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uocr
