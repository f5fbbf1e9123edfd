// Device fill of the seeded synthetic workloads: the same bits as
// synth/rng.py and synth/workloads.py (SplitMix64 counter streams, an
// Irwin-Hall(8) integer sum scaled once in float32 and rounded to bf16
// nearest-even, or small integers -2..2), written straight into the
// block-major pools.  Compiled with -ffp-contract=off so that the float32
// operations of the direction edit round exactly as on the host.
// Nothing here computes any step of the attention method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint32_t kNormalScaleBits = 0x371CC471u;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t word(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * kGamma); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t value(uint64_t key, uint64_t i, int mode) {
  if (mode == 0) {
    const uint64_t w0 = word(key, 2 * i), w1 = word(key, 2 * i + 1);
    int64_t s = 0;
#pragma unroll
    for (int sh = 0; sh < 64; sh += 16) s += (int64_t)((w0 >> sh) & 0xFFFFu) + (int64_t)((w1 >> sh) & 0xFFFFu);
    const float x = (float)(int32_t)(2 * s - 524280);
    return f32_to_bf16(x * __uint_as_float(kNormalScaleBits));
  }
  const uint64_t w = word(key, i);
  const int v = (int)((w >> 48) % 5u) - 2;
  return f32_to_bf16((float)v);
}

// Eight consecutive elements starting at logical index i0, packed as uint4.
__device__ __forceinline__ uint4 value8(uint64_t key, uint64_t i0, int mode) {
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = value(key, i0 + e, mode);
  return make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16), v[4] | ((uint32_t)v[5] << 16),
                    v[6] | ((uint32_t)v[7] << 16));
}

// Main K or V of one (layer, seq): element (t, h, d) has logical index
// (t*H + h)*D + d and lives at pool[((pb*H + h)*32 + t%32)*D + d].
__global__ void fill_kv_kernel(uint16_t* pool, const int32_t* table_row, int32_t ntok, int32_t H, int32_t D,
                               uint64_t key, int32_t mode) {
  const int64_t vec = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = (int64_t)H * D / 8;
  if (vec >= (int64_t)ntok * per_tok) return;
  const int64_t t = vec / per_tok;
  const int64_t r = vec - t * per_tok;
  const int h = (int)(r * 8 / D);
  const int d = (int)(r * 8 - (int64_t)h * D);
  const int pb = table_row[t / 32];
  const uint64_t i0 = (uint64_t)((t * H + h) * D + d);
  uint4* dst = reinterpret_cast<uint4*>(pool + (((int64_t)pb * H + h) * 32 + (t % 32)) * D + d);
  *dst = value8(key, i0, mode);
}

// Indexer K of one (layer, seq): element (t, d) has index t*Di + d and lives
// at pool[(pb*32 + t%32)*Di + d].
__global__ void fill_kidx_kernel(uint16_t* pool, const int32_t* table_row, int32_t ntok, int32_t Di, uint64_t key,
                                 int32_t mode) {
  const int64_t vec = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = Di / 8;
  if (vec >= (int64_t)ntok * per_tok) return;
  const int64_t t = vec / per_tok;
  const int d = (int)(vec - t * per_tok) * 8;
  const int pb = table_row[t / 32];
  uint4* dst = reinterpret_cast<uint4*>(pool + ((int64_t)pb * 32 + (t % 32)) * Di + d);
  *dst = value8(key, (uint64_t)(t * Di + d), mode);
}

__global__ void fill_dense_kernel(uint16_t* out, int64_t n8, uint64_t key, int32_t mode) {
  const int64_t vec = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (vec >= n8) return;
  reinterpret_cast<uint4*>(out)[vec] = value8(key, (uint64_t)vec * 8, mode);
}

// k <- bf16(f32(k) + f32(coef * f32(q))) on the listed indexer-key rows.
__global__ void add_direction_kernel(uint16_t* pool, const int32_t* table_row, const int64_t* tokens, int32_t ntok,
                                     const uint16_t* q, float coef, int32_t Di) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)ntok * Di) return;
  const int64_t t = tokens[i / Di];
  const int d = (int)(i % Di);
  const int pb = table_row[t / 32];
  uint16_t* k = pool + ((int64_t)pb * 32 + (t % 32)) * Di + d;
  const float kf = __uint_as_float((uint32_t)*k << 16);
  const float qf = __uint_as_float((uint32_t)q[d] << 16);
  const float step = coef * qf;
  *k = f32_to_bf16(kf + step);
}

inline dim3 grid_for(int64_t n, int threads) { return dim3((unsigned)((n + threads - 1) / threads)); }

}  // namespace

extern "C" {

int synth_fill_kv(uint16_t* pool, const int32_t* table_row, int32_t ntok, int32_t H, int32_t D, uint64_t key,
                  int32_t mode, void* stream) {
  if (ntok <= 0) return 0;
  const int64_t n = (int64_t)ntok * H * D / 8;
  hipLaunchKernelGGL(fill_kv_kernel, grid_for(n, 256), dim3(256), 0, (hipStream_t)stream, pool, table_row, ntok, H, D,
                     key, mode);
  return (int)hipGetLastError();
}

int synth_fill_kidx(uint16_t* pool, const int32_t* table_row, int32_t ntok, int32_t Di, uint64_t key, int32_t mode,
                    void* stream) {
  if (ntok <= 0) return 0;
  const int64_t n = (int64_t)ntok * Di / 8;
  hipLaunchKernelGGL(fill_kidx_kernel, grid_for(n, 256), dim3(256), 0, (hipStream_t)stream, pool, table_row, ntok,
                     Di, key, mode);
  return (int)hipGetLastError();
}

int synth_fill_dense(uint16_t* out, int64_t n, uint64_t key, int32_t mode, void* stream) {
  if (n <= 0) return 0;
  if (n % 8) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_dense_kernel, grid_for(n / 8, 256), dim3(256), 0, (hipStream_t)stream, out, n / 8, key,
                     mode);
  return (int)hipGetLastError();
}

int synth_add_direction(uint16_t* pool, const int32_t* table_row, const int64_t* tokens, int32_t ntok,
                        const uint16_t* q, float coef, int32_t Di, void* stream) {
  if (ntok <= 0) return 0;
  const int64_t n = (int64_t)ntok * Di;
  hipLaunchKernelGGL(add_direction_kernel, grid_for(n, 256), dim3(256), 0, (hipStream_t)stream, pool, table_row,
                     tokens, ntok, q, coef, Di);
  return (int)hipGetLastError();
}

}  // extern "C"
