// page2d rotary position encoding and the KV-cache write (the step that
// produces the pre-rotated caches of the attention path; news.rkmt.cn/news/25027
// Sec. 4 and Sec. 6).
//
// The 64 rotation pairs (i, i + 64) of a 128-dim row (rotate-half layout:
// angles cat(tok, page) doubled) take angle tok_pos * 10000^(-2i/126) for
// the 63 token pairs (the token axis samples its own 126-dim spectrum) and
// (page_pos mod 2) * 256^0 for the page pair.  One wave rotates one row: lane
// i owns pair i.  Angles, sincos and the rotation run in fp64, and the result
// is rounded once to bf16 (nearest, ties to even), so it is the correctly
// rounded rotation of the bf16 input.  The cache write scatters each new
// token's rotated K rows (every head), V rows (copied) and rotated indexer K
// row into the block-major pools through the block table.
#include "device_common.h"
#include "kernels.h"

// The rotation is x1*c - x2*s and x2*c + x1*s with separately rounded
// products (no fused multiply-add), the rounding the oracle states.
#pragma clang fp contract(off)

namespace uocr {

namespace {
constexpr int kRopeThreads = 256;
constexpr int kRowsPerWg = kRopeThreads / kWave;
constexpr int kTokPairs = 63;
constexpr double kTokTheta = 10000.0;
constexpr double kPageTheta = 256.0;
}  // namespace

// Nearest-even bf16 bits of a finite double (sign of zero kept).
__device__ __forceinline__ uint16_t bf16_nearest(double y) {
  int e;
  (void)frexp(y, &e);                        // y = m * 2^e, 0.5 <= |m| < 1
  const double scale = ldexp(1.0, e - 8);    // 8 significant bits
  const double r = y == 0.0 ? y : rint(y / scale) * scale;
  return (uint16_t)(__float_as_uint((float)r) >> 16);
}

// Frequency of rotation pair i: token pairs 10000^(-2i/126), the page pair
// 256^0 (computed once per wave).
__device__ __forceinline__ double pair_freq(int i) {
  return i < kTokPairs ? pow(kTokTheta, -2.0 * i / (2.0 * kTokPairs)) : pow(kPageTheta, 0.0);
}

// Rotate pair (i, i + 64) of row `src` into `dst` (both 128 bf16).
__device__ __forceinline__ void rotate_row(const uint16_t* src, uint16_t* dst, int i, double freq, int32_t tok_pos,
                                           int32_t page_pos) {
  const double x1 = (double)__uint_as_float((uint32_t)src[i] << 16);
  const double x2 = (double)__uint_as_float((uint32_t)src[i + 64] << 16);
  const double coord = i < kTokPairs ? (double)tok_pos : (double)(((page_pos % 2) + 2) % 2);
  double s, c;
  sincos(coord * freq, &s, &c);
  dst[i] = bf16_nearest(x1 * c - x2 * s);
  dst[i + 64] = bf16_nearest(x2 * c + x1 * s);
}

__global__ __launch_bounds__(kRopeThreads) void rope_cache_write_kernel(RopeWriteArgs a) {
  const int rows_per_tok = a.heads + 1;  // K heads, then the indexer row
  const int64_t rows = (int64_t)a.n * rows_per_tok;
  const int lane = lane_id();
  const double freq = pair_freq(lane);
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerWg + wave_id(); row < rows;
       row += (int64_t)gridDim.x * kRowsPerWg) {
    const int t = (int)(row / rows_per_tok);
    const int r = (int)(row - (int64_t)t * rows_per_tok);
    const int seq = a.seq[t];
    const int pos = a.pos[t];
    if (seq < 0 || seq >= a.batch || pos < 0 || pos >= a.max_blocks * kBlock) continue;
    const int pb = a.block_table[(int64_t)seq * a.max_blocks + pos / kBlock];
    if (pb < 0 || (int64_t)pb >= a.num_blocks) continue;
    const int slot = pos % kBlock;
    const int32_t tp = a.tok_pos[t], pp = a.page_pos[t];
    if (r < a.heads) {
      const int64_t dst = (((int64_t)pb * a.heads + r) * kBlock + slot) * kDim;
      const int64_t src = ((int64_t)t * a.heads + r) * kDim;
      rotate_row(a.k_new + src, a.k_pool + dst, lane, freq, tp, pp);
      reinterpret_cast<uint32_t*>(a.v_pool + dst)[lane] = reinterpret_cast<const uint32_t*>(a.v_new + src)[lane];
    } else {
      const int64_t dst = ((int64_t)pb * kBlock + slot) * kDim;
      rotate_row(a.kidx_new + (int64_t)t * kDim, a.kidx_pool + dst, lane, freq, tp, pp);
    }
  }
}

__global__ __launch_bounds__(kRopeThreads) void rope_queries_kernel(RopeQueryArgs a) {
  const int rows_per_tok = a.heads + 1;  // q heads, then the indexer query
  const int64_t rows = (int64_t)a.n * rows_per_tok;
  const int lane = lane_id();
  const double freq = pair_freq(lane);
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerWg + wave_id(); row < rows;
       row += (int64_t)gridDim.x * kRowsPerWg) {
    const int t = (int)(row / rows_per_tok);
    const int r = (int)(row - (int64_t)t * rows_per_tok);
    uint16_t* x = r < a.heads ? (a.q != nullptr ? a.q + ((int64_t)t * a.heads + r) * kDim : nullptr)
                              : (a.q_idx != nullptr ? a.q_idx + (int64_t)t * kDim : nullptr);
    if (x == nullptr) continue;
    // in place: both values of the pair are read before either is written
    rotate_row(x, x, lane, freq, a.tok_pos[t], a.page_pos[t]);
  }
}

namespace {
// Up to 1024 workgroups (4 per CU); each wave then loops over its rows.
unsigned rope_grid(int64_t rows) {
  const int64_t wgs = (rows + kRowsPerWg - 1) / kRowsPerWg;
  return (unsigned)(wgs < 1024 ? wgs : 1024);
}
}  // namespace

hipError_t launch_rope_cache_write(const RopeWriteArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_cache_write_kernel, dim3(rope_grid((int64_t)a.n * (a.heads + 1))), dim3(kRopeThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_rope_queries(const RopeQueryArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_queries_kernel, dim3(rope_grid((int64_t)a.n * (a.heads + 1))), dim3(kRopeThreads), 0,
                     stream, a);
  return hipGetLastError();
}

// page2d coordinates (news.rkmt.cn/news/25027 Sec. 4: the page coordinate
// counts page markers, the token coordinate runs inside the page; decoding
// advances a {page, tok} state per token, a marker moving to the next page
// and sending tok back to the page's start).  One workgroup per sequence
// scans its tokens in tiles of kCoordThreads: an inclusive scan of the marker
// count and a max-scan of the last marker's position, carried across tiles;
// the state after the last token is written back.
namespace {
constexpr int kCoordThreads = 256;
}

__global__ __launch_bounds__(kCoordThreads) void page_coords_kernel(PageCoordArgs a) {
  __shared__ int32_t s_cnt[kCoordThreads];
  __shared__ int32_t s_last[kCoordThreads];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* tok_in = a.tokens + (int64_t)b * a.n;
  int32_t page = a.state[2 * b];
  int32_t tok = a.state[2 * b + 1];
  for (int64_t base = 0; base < a.n; base += kCoordThreads) {
    const int64_t i = base + tid;
    const bool valid = i < a.n;
    const bool mk = valid && tok_in[i] == a.marker;
    s_cnt[tid] = mk ? 1 : 0;
    s_last[tid] = mk ? tid : -1;
    __syncthreads();
    for (int d = 1; d < kCoordThreads; d <<= 1) {
      const int c = tid >= d ? s_cnt[tid - d] : 0;
      const int l = tid >= d ? s_last[tid - d] : -1;
      __syncthreads();
      s_cnt[tid] += c;
      s_last[tid] = max(s_last[tid], l);
      __syncthreads();
    }
    const int32_t my_page = page + s_cnt[tid];
    const int32_t my_tok = s_last[tid] >= 0 ? tid - s_last[tid] : tok + 1 + tid;
    if (valid) {
      a.tok_pos[(int64_t)b * a.n + i] = my_tok;
      a.page_pos[(int64_t)b * a.n + i] = my_page;
    }
    // carry: the state after the tile's last token
    const int last = (int)min<int64_t>(kCoordThreads, a.n - base) - 1;
    const int32_t c_last = s_cnt[last], l_last = s_last[last];
    page += c_last;
    tok = l_last >= 0 ? last - l_last : tok + 1 + last;
    __syncthreads();
  }
  if (tid == 0) {
    a.state[2 * b] = page;
    a.state[2 * b + 1] = tok;
  }
}

hipError_t launch_page_coords(const PageCoordArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(page_coords_kernel, dim3(a.batch), dim3(kCoordThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uocr
