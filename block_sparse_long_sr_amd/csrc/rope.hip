// page2d rotary position encoding and the KV-cache write (the step that
// produces the pre-rotated caches of the attention path; news.rkmt.cn/news/25027
// Sec. 4 and Sec. 6).
//
// The 64 rotation pairs (i, i + 64) of a 128-dim row (rotate-half layout:
// angles cat(tok, page) doubled) take angle tok_pos * 10000^(-2i/126) for
// the 63 token pairs (the token axis samples its own 126-dim spectrum) and
// (page_pos mod 2) * 256^0 for the page pair.  One wave rotates all rows of
// one token: lane i owns pair i and takes its sine and cosine once.  Angles,
// sincos and the rotation run in fp64, and the result is rounded once to bf16
// (nearest, ties to even), so it is the correctly rounded rotation of the
// bf16 input.  The cache write scatters each new token's rotated K rows
// (every head), V rows (copied) and rotated indexer K row into the
// block-major pools through the block table.
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

// Nearest-even bf16 bits of a finite double (sign of zero kept): rounded to
// 8 significant bits by scaling with powers of two (exact), then converted.
__device__ __forceinline__ uint16_t bf16_nearest(double y) {
  int e;
  (void)frexp(y, &e);  // y = m * 2^e, 0.5 <= |m| < 1
  const double r = y == 0.0 ? y : ldexp(rint(ldexp(y, 8 - e)), e - 8);
  return (uint16_t)(__float_as_uint((float)r) >> 16);
}

// Frequency of rotation pair i: token pairs 10000^(-2i/126), the page pair
// 256^0 (computed once per wave).
__device__ __forceinline__ double pair_freq(int i) {
  return i < kTokPairs ? pow(kTokTheta, -2.0 * i / (2.0 * kTokPairs)) : pow(kPageTheta, 0.0);
}

// The token's angle of rotation pair i, as (sin, cos).
__device__ __forceinline__ void pair_sincos(int i, double freq, int32_t tok_pos, int32_t page_pos, double& s,
                                            double& c) {
  const double coord = i < kTokPairs ? (double)tok_pos : (double)(((page_pos % 2) + 2) % 2);
  sincos(coord * freq, &s, &c);
}

// Rotated bf16 pair (x1*c - x2*s, x2*c + x1*s) of the bf16 pair (x1, x2).
__device__ __forceinline__ void rotate_pair(uint16_t x1, uint16_t x2, double s, double c, uint16_t& y1, uint16_t& y2) {
  const double d1 = (double)__uint_as_float((uint32_t)x1 << 16);
  const double d2 = (double)__uint_as_float((uint32_t)x2 << 16);
  y1 = bf16_nearest(d1 * c - d2 * s);
  y2 = bf16_nearest(d2 * c + d1 * s);
}

// Rows of one token a wave handles per round (10 heads and the indexer row
// fit in one): all their loads are issued before any store.
constexpr int kRowGroup = 12;

// One wave per token: lane i takes the sine and cosine of pair i once and
// rotates that pair in all of the token's rows (every K head, then the
// indexer row), and copies the token's V rows.
__global__ __launch_bounds__(kRopeThreads) void rope_cache_write_kernel(RopeWriteArgs a) {
  const int lane = lane_id();
  const double freq = pair_freq(lane);
  const int rows = a.heads + 1;
  for (int64_t t = (int64_t)blockIdx.x * kRowsPerWg + wave_id(); t < a.n; t += (int64_t)gridDim.x * kRowsPerWg) {
    const int seq = a.seq[t];
    const int pos = a.pos[t];
    if (seq < 0 || seq >= a.batch || pos < 0 || pos >= a.max_blocks * kBlock) continue;
    const int pb = a.block_table[(int64_t)seq * a.max_blocks + pos / kBlock];
    if (pb < 0 || (int64_t)pb >= a.num_blocks) continue;
    const int slot = pos % kBlock;
    double s, c;
    pair_sincos(lane, freq, a.tok_pos[t], a.page_pos[t], s, c);
    for (int r0 = 0; r0 < rows; r0 += kRowGroup) {
      uint16_t x1[kRowGroup], x2[kRowGroup];
      uint32_t v[kRowGroup];
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j) {
        const int r = r0 + j;
        if (r < a.heads) {
          const uint16_t* src = a.k_new + (t * a.heads + r) * kDim;
          x1[j] = src[lane];
          x2[j] = src[lane + 64];
          v[j] = reinterpret_cast<const uint32_t*>(a.v_new + (t * a.heads + r) * kDim)[lane];
        } else if (r == a.heads) {
          x1[j] = a.kidx_new[t * kDim + lane];
          x2[j] = a.kidx_new[t * kDim + lane + 64];
        }
      }
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j) {
        const int r = r0 + j;
        if (r > a.heads) break;
        uint16_t* dst = r < a.heads ? a.k_pool + (((int64_t)pb * a.heads + r) * kBlock + slot) * kDim
                                    : a.kidx_pool + ((int64_t)pb * kBlock + slot) * kDim;
        rotate_pair(x1[j], x2[j], s, c, dst[lane], dst[lane + 64]);
        if (r < a.heads)
          reinterpret_cast<uint32_t*>(a.v_pool + (((int64_t)pb * a.heads + r) * kBlock + slot) * kDim)[lane] = v[j];
      }
    }
  }
}

// One wave per token, like the cache write: q heads, then the indexer query,
// rotated in place.
__global__ __launch_bounds__(kRopeThreads) void rope_queries_kernel(RopeQueryArgs a) {
  const int lane = lane_id();
  const double freq = pair_freq(lane);
  const int rows = a.heads + 1;
  for (int64_t t = (int64_t)blockIdx.x * kRowsPerWg + wave_id(); t < a.n; t += (int64_t)gridDim.x * kRowsPerWg) {
    double s, c;
    pair_sincos(lane, freq, a.tok_pos[t], a.page_pos[t], s, c);
    for (int r0 = 0; r0 < rows; r0 += kRowGroup) {
      uint16_t* x[kRowGroup];
      uint16_t x1[kRowGroup], x2[kRowGroup];
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j) {
        const int r = r0 + j;
        x[j] = r < a.heads ? (a.q != nullptr ? a.q + (t * a.heads + r) * kDim : nullptr)
                           : (r == a.heads && a.q_idx != nullptr ? a.q_idx + t * kDim : nullptr);
        if (x[j] != nullptr) {
          x1[j] = x[j][lane];
          x2[j] = x[j][lane + 64];
        }
      }
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j)
        if (x[j] != nullptr) rotate_pair(x1[j], x2[j], s, c, x[j][lane], x[j][lane + 64]);
    }
  }
}

namespace {
// One wave per token, up to 1024 workgroups (4 per CU); waves then loop.
unsigned rope_grid(int64_t tokens) {
  const int64_t wgs = (tokens + kRowsPerWg - 1) / kRowsPerWg;
  return (unsigned)(wgs < 1024 ? wgs : 1024);
}
}  // namespace

hipError_t launch_rope_cache_write(const RopeWriteArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_cache_write_kernel, dim3(rope_grid(a.n)), dim3(kRopeThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rope_queries(const RopeQueryArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_queries_kernel, dim3(rope_grid(a.n)), dim3(kRopeThreads), 0, stream, a);
  return hipGetLastError();
}

// page2d coordinates (news.rkmt.cn/news/25027 Sec. 4: the page coordinate
// counts page markers, the token coordinate runs inside the page; decoding
// advances a {page, tok} state per token, a marker moving to the next page
// and sending tok back to the page's start).  One workgroup per sequence
// scans its tokens in tiles of kCoordTile, each thread taking kCoordPer
// consecutive tokens: the marker count is summed and the last marker's
// position max-scanned, first inside the thread, then across the wave by lane
// shuffles, then across the waves through LDS; both are carried across
// tiles, and the state after the last token is written back.
namespace {
constexpr int kCoordThreads = 256;
constexpr int kCoordPer = 4;
constexpr int kCoordTile = kCoordThreads * kCoordPer;
constexpr int kCoordWaves = kCoordThreads / kWave;
}  // namespace

__global__ __launch_bounds__(kCoordThreads) void page_coords_kernel(PageCoordArgs a) {
  __shared__ int32_t s_cnt[2][kCoordWaves];  // per wave: markers, last marker (tile index or -1)
  __shared__ int32_t s_last[2][kCoordWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / kWave;
  const int32_t* tok_in = a.tokens + (int64_t)b * a.n;
  int32_t page = a.state[2 * b];
  int32_t tok = a.state[2 * b + 1];
  int buf = 0;
  for (int64_t base = 0; base < a.n; base += kCoordTile, buf ^= 1) {
    const int k0 = tid * kCoordPer;  // first token of this thread, tile-relative
    bool mk[kCoordPer];
#pragma unroll
    for (int j = 0; j < kCoordPer; ++j) mk[j] = base + k0 + j < a.n && tok_in[base + k0 + j] == a.marker;
    int cnt[kCoordPer], last[kCoordPer];  // inclusive inside the thread
    int c = 0, l = -1;
#pragma unroll
    for (int j = 0; j < kCoordPer; ++j) {
      c += mk[j] ? 1 : 0;
      l = mk[j] ? k0 + j : l;
      cnt[j] = c;
      last[j] = l;
    }
    // inclusive scan of the thread totals over the wave
    int wc = c, wl = l;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int oc = __shfl_up(wc, d);
      const int ol = __shfl_up(wl, d);
      if (lane >= d) {
        wc += oc;
        wl = max(wl, ol);
      }
    }
    const int ec = wc - c;  // markers in the wave's earlier threads
    int el = __shfl_up(wl, 1);
    if (lane == 0) el = -1;
    if (lane == kWave - 1) {
      s_cnt[buf][w] = wc;
      s_last[buf][w] = wl;
    }
    __syncthreads();  // the other buffer is rewritten only after the next tile's barrier
    int pc = 0, pl = -1, tc = 0, tl = -1;  // earlier waves; the whole tile
#pragma unroll
    for (int v = 0; v < kCoordWaves; ++v) {
      if (v < w) {
        pc += s_cnt[buf][v];
        pl = max(pl, s_last[buf][v]);
      }
      tc += s_cnt[buf][v];
      tl = max(tl, s_last[buf][v]);
    }
#pragma unroll
    for (int j = 0; j < kCoordPer; ++j) {
      const int64_t i = base + k0 + j;
      if (i < a.n) {
        const int k = k0 + j;
        const int lk = max(max(pl, el), last[j]);
        a.tok_pos[(int64_t)b * a.n + i] = lk >= 0 ? k - lk : tok + 1 + k;
        a.page_pos[(int64_t)b * a.n + i] = page + pc + ec + cnt[j];
      }
    }
    // carry: the state after the tile's last token
    const int len = (int)min<int64_t>(kCoordTile, a.n - base);
    page += tc;
    tok = tl >= 0 ? len - 1 - tl : tok + len;
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
