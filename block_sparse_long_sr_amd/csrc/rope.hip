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

}  // namespace uocr
