// The whole sparse decode step of a batch in one launch: for every layer and
// sequence, indexer scoring with the block max, top-k block selection and
// the sparse gather attention (SR-SWA steps 2-4, news.rkmt.cn/news/25027
// Sec. 5).
//
// Work items, handed out in ticket order by one atomic counter (a workgroup
// takes its next ticket while it works on the current item):
//   * scoring item (layer l, sequence b, chunk c): `chunk` blocks of the
//     sequence's candidates, two 8 KB blocks per wave in flight.  The
//     workgroup that completes the last chunk of (l, b) then runs the
//     selection of (l, b) once and publishes the kept block ids;
//   * attention item (l, b, head h): the attention of head h over the
//     published selection.
// "Slot" s = l * batch + b.  The ticket order is: the scoring items of slot
// s, then the attention items of slot s - lag, for s = 0, 1, ...; the last
// `lag` slots' attention items close the list.  With lag < batch, each item
// depends only on items with lower tickets:
//   * an attention item waits until the selection of its slot is published;
//   * a scoring item of layer l > 0 waits until every head of (l - 1, b) is
//     attended (the layer order of one sequence).
// A workgroup holding a ticket is running, so the lowest unfinished ticket
// always makes progress: the waits end.  Each wait is also bounded (about a
// second of polling); on expiry it sets the error word of the counters and
// goes on, so the launch always finishes.
//
// Publication: data that another workgroup reads inside the launch (block
// scores, selections) is written with device-scope atomic stores, which the
// L2 of the writing XCD writes through; every wave waits for its stores to
// complete, the workgroup meets at a barrier, then one thread increments the
// completion counter.  A reader polls the counter, then takes a device-scope
// acquire fence (an L1/L2 invalidation of its XCD) before reading, so it
// cannot hit a stale line.  No L2 write-back is needed on the writer's side.
// A clear kernel zeroes the counters before each launch.
#include <atomic>

#include "attn_common.h"
#include "device_common.h"
#include "indexer_common.h"
#include "kernels.h"
#include "select_common.h"

namespace uocr {

namespace {
// 512 threads: the selection holds 8 candidate keys per thread (contexts up
// to 4096 candidate blocks) and the kernel fits 128 VGPRs, so two
// workgroups share a CU and one's item boundary is covered by the other.
constexpr int kStepThreads = 512;
constexpr int kStepWaves = kStepThreads / kWave;
constexpr int kMaxStepChunk = 32;  // blocks per scoring item, at most
constexpr uint32_t kSpinLimit = 1u << 20;  // polls of one wait: a device-scope load (~1 us) + s_sleep 2 each, about a second

struct Item {
  int attention;  // 0: scoring item, 1: attention item
  int slot;
  int idx;        // chunk or head
};

__device__ __forceinline__ Item item_of(uint32_t t, int S, int C, int H, int D) {
  const uint32_t head = (uint32_t)D * C;
  if (t < head) return {0, (int)(t / C), (int)(t % C)};
  t -= head;
  const uint32_t unit = (uint32_t)(C + H);
  const uint32_t mid = (uint32_t)(S - D) * unit;
  if (t < mid) {
    const int s = D + (int)(t / unit);
    const int r = (int)(t % unit);
    return r < C ? Item{0, s, r} : Item{1, s - D, r - C};
  }
  t -= mid;
  return {1, S - D + (int)(t / H), (int)(t % H)};
}

// Thread 0 only: poll *ctr (relaxed, device scope) until it reaches need,
// then one acquire fence at device scope (a single cache invalidation, not
// one per poll).
__device__ __forceinline__ void wait_count(uint32_t* ctr, uint32_t need, uint32_t* err) {
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Device-scope (write-through) store of a value other workgroups read.
template <typename T>
__device__ __forceinline__ void publish(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread, before the barrier that precedes a counter increment: wait
// until the wave's own stores have completed (a barrier alone does not).
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }

// Thread 0, after drain_stores and a barrier: count one completion; returns
// the count before it.
__device__ __forceinline__ uint32_t count_done(uint32_t* ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace

__global__ __launch_bounds__(kStepThreads) void decode_step_clear_kernel(uint32_t* counters, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) counters[i] = 0u;
}

template <int KPT>
__global__ __launch_bounds__(kStepThreads) __attribute__((amdgpu_waves_per_eu(4))) void decode_step_kernel(
    DecodeStepArgs a) {
  __shared__ SelectSmem<kStepThreads> sel_sm;
  __shared__ AttendSmem<kStepThreads> att_sm;
  __shared__ int32_t s_blocks[kMaxFusedTopk];
  __shared__ uint32_t s_ticket;
  __shared__ int s_last;
  __shared__ float s_chunk[kMaxStepChunk];  // an item's block scores

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int B = a.batch, M = a.max_blocks, H = a.heads;
  const int S = a.n_layers * B;
  const int chunk = a.chunk;  // a multiple of 2 * kStepWaves
  const int C = (M + chunk - 1) / chunk;
  const int D = a.lag;  // < B, so every wait is on a lower ticket
  const uint32_t total = (uint32_t)S * (uint32_t)(C + H);
  uint32_t* ticket = a.counters;
  uint32_t* err = a.counters + 1;
  uint32_t* score_done = a.counters + 2;
  uint32_t* sel_done = score_done + S;
  uint32_t* attn_done = sel_done + S;

  if (tid == 0) s_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  uint32_t t = s_ticket;
  while (t < total) {
    __syncthreads();  // every thread has read s_ticket
    if (tid == 0) s_ticket = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const Item it = item_of(t, S, C, H, D);
    const int l = it.slot / B;
    const int b = it.slot - l * B;
    const int L = clamp_ctx(a.ctx_lens[b], M);
    const int nb = (L + kBlock - 1) / kBlock;
    const int ncand = nb - a.local_blocks > 0 ? nb - a.local_blocks : 0;
    float* scores = a.block_scores + (int64_t)it.slot * M;
    int32_t* sel_out = a.block_idx + (int64_t)it.slot * a.topk;
    const int32_t* table = a.block_table + (int64_t)b * M;

    if (!it.attention) {
      if (l > 0) {
        if (tid == 0) wait_count(attn_done + (it.slot - B), (uint32_t)H, err);
        __syncthreads();
      }
      const int j0 = it.idx * chunk;
      const int jend_all = min(j0 + chunk, M);
      const int jend = min(jend_all, ncand);
      if (j0 < jend) {
        const uint4 qv = *reinterpret_cast<const uint4*>(a.q_idx + (int64_t)it.slot * kDim + (lane & 15) * 8);
        const uint16_t* kidx = a.kidx_pool + (int64_t)l * a.kidx_layer_stride;
        // blocks j and j + kStepWaves of the wave are loaded together
        for (int j = j0 + wave; j < jend; j += 2 * kStepWaves) {
          const int j2 = j + kStepWaves;
          const int pb = __builtin_amdgcn_readfirstlane(table[j]);
          const int pb2 = j2 < jend ? __builtin_amdgcn_readfirstlane(table[j2]) : -1;
          const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks;
          const bool ok2 = pb2 >= 0 && (int64_t)pb2 < a.num_blocks;
          uint4 kv[8], kv2[8];
          load_index_tile(kidx + (int64_t)(ok ? pb : 0) * (kBlock * kDim), kv);
          load_index_tile(kidx + (int64_t)(ok2 ? pb2 : 0) * (kBlock * kDim), kv2);
          const float s1 = ok ? block_max_of_tile(kv, qv) : __builtin_nanf("");
          const float s2 = ok2 ? block_max_of_tile(kv2, qv) : __builtin_nanf("");
          if (lane == 0) {
            s_chunk[j - j0] = s1;
            if (j2 < jend) s_chunk[j2 - j0] = s2;
          }
        }
      }
      __syncthreads();
      // one coalesced store of the item's scores (non-candidates: -inf)
      for (int j = j0 + tid; j < jend_all; j += kStepThreads)
        publish(scores + j, j < jend ? s_chunk[j - j0] : -INFINITY);
      drain_stores();
      __syncthreads();
      if (tid == 0) {
        const bool last = count_done(score_done + it.slot) == (uint32_t)(C - 1);
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every chunk's scores are visible
        s_last = last;
      }
      __syncthreads();
      if (s_last) {
        // the slot's scoring is complete: select once for its heads
        const int R = a.topk - a.local_blocks;
        if (!select_trivial(nb, ncand, R, a.topk, s_blocks, kStepThreads))
          select_sorted_reg<kStepThreads, KPT>(scores, ncand, R, a.local_blocks, s_blocks, sel_sm,
                                               a.block_page != nullptr ? a.block_page + (int64_t)b * M : nullptr,
                                               a.block_page != nullptr ? a.query_page[b] : 0);
        __syncthreads();
        for (int i = tid; i < a.topk; i += kStepThreads) publish(sel_out + i, s_blocks[i]);
        if (a.n_sel != nullptr && tid == 0) a.n_sel[it.slot] = nb < a.topk ? nb : a.topk;
        drain_stores();
        __syncthreads();
        if (tid == 0) count_done(sel_done + it.slot);
      }
    } else {
      if (tid == 0) wait_count(sel_done + it.slot, 1u, err);
      __syncthreads();
      for (int i = tid; i < a.topk; i += kStepThreads) s_blocks[i] = sel_out[i];
      __syncthreads();
      const int h = it.idx;
      const int64_t head_row = (int64_t)it.slot * H + h;
      const int64_t kv_off = (int64_t)l * a.kv_layer_stride;
      attend_query_wg<kStepThreads, true>(a.k_pool + kv_off, a.v_pool + kv_off, table, a.num_blocks, H, h, M,
                                          L - 1, a.q + head_row * kDim, s_blocks, a.topk, a.scale_log2,
                                          a.out + head_row * kDim, a.lse != nullptr ? a.lse + head_row : nullptr,
                                          att_sm);
      drain_stores();
      __syncthreads();
      if (tid == 0) count_done(attn_done + it.slot);
    }
    __syncthreads();  // the next ticket is in s_ticket; LDS of this item is free
    t = s_ticket;
  }
}

DecodeStepPlan decode_step_plan(int32_t n_layers, int32_t batch, int32_t heads, int32_t max_blocks) {
  DecodeStepPlan p{};
  const int64_t S = (int64_t)n_layers * batch;
  // Slots between a slot's scoring items and its attention items: long
  // enough for the slot's scoring and selection to finish, short enough for
  // its attention to finish before the sequence's next layer comes up, which
  // is batch slots later.  Half the batch (below batch, as the ticket order
  // requires); measured best at 16 sequences x 128K.
  p.lag = batch / 2;
  // Blocks per scoring item: 32 (256 KB of indexer keys) at long contexts,
  // 16 below 2048 blocks, so that a sequence's scoring spreads over many
  // workgroups and finishes soon after its first item starts.
  p.chunk = max_blocks >= 2048 ? kMaxStepChunk : 16;
  p.counter_words = 2 + 3 * S;
  p.ws_bytes = (size_t)((p.counter_words * 4 + 255) / 256 * 256);
  p.items = S * (((int64_t)max_blocks + p.chunk - 1) / p.chunk + heads);
  return p;
}

namespace {
template <int KPT>
hipError_t launch_step(const DecodeStepArgs& a, int64_t items, hipStream_t stream) {
  // One resident wave of workgroups (they loop over the tickets); a grid
  // larger than what fits is also correct, the extra groups find no ticket.
  // The count is computed once per device (threads that race here store
  // the same value).
  static std::atomic<int> resident[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int fit = resident[dev].load(std::memory_order_relaxed);
  if (fit == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_step_kernel<KPT>, kStepThreads, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    fit = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    resident[dev].store(fit, std::memory_order_relaxed);
  }
  const int64_t grid = items < fit ? items : fit;
  hipLaunchKernelGGL(decode_step_kernel<KPT>, dim3((unsigned)grid), dim3(kStepThreads), 0, stream, a);
  return hipGetLastError();
}
}  // namespace

bool decode_step_one_launch(int32_t n_layers, int32_t batch, int32_t max_blocks) {
  // The one launch overlaps one sequence's selection and attention with the
  // scoring of others, but a sequence's layers stay in order: each layer of
  // a sequence must be scored, selected and attended within the time the
  // other sequences' scoring of that layer takes, about batch * max_blocks *
  // 8 KB at HBM rate.  Measured at 16 sequences x 12 layers: per-layer
  // launches win up to 64K tokens (2048 blocks), the two are even at 96K
  // (3072 blocks) and the one launch wins at 128K; with one layer there is
  // no layer order to overlap.
  return n_layers >= 2 && (int64_t)batch * max_blocks >= 57344;
}

hipError_t launch_decode_step(const DecodeStepArgs& a, const DecodeStepPlan& plan, bool one_launch,
                              hipStream_t stream) {
  if (a.batch == 0 || a.n_layers == 0) return hipSuccess;
  const int B = a.batch, M = a.max_blocks, H = a.heads;
  if (!one_launch) {
    // per-layer launches of the scoring kernel and the fused selection +
    // attention kernel, on the caller's stream
    for (int l = 0; l < a.n_layers; ++l) {
      IndexerDecodeArgs ia{};
      ia.kidx_pool = a.kidx_pool + (int64_t)l * a.kidx_layer_stride;
      ia.block_table = a.block_table;
      ia.ctx_lens = a.ctx_lens;
      ia.q_idx = a.q_idx + (int64_t)l * B * kDim;
      ia.block_scores = a.block_scores + (int64_t)l * B * M;
      ia.num_blocks = a.num_blocks;
      ia.batch = B;
      ia.max_blocks = M;
      ia.local_blocks = a.local_blocks;
      ia.chunk = indexer_decode_chunk(B, M);
      hipError_t e = launch_indexer_decode(ia, stream);
      if (e != hipSuccess) return e;
      SelAttnArgs sa{};
      AttnArgs& at = sa.attn;
      at.k_pool = a.k_pool + (int64_t)l * a.kv_layer_stride;
      at.v_pool = a.v_pool + (int64_t)l * a.kv_layer_stride;
      at.block_table = a.block_table;
      at.ctx_lens = a.ctx_lens;
      at.q = a.q + (int64_t)l * B * H * kDim;
      at.block_idx = nullptr;
      at.out = a.out + (int64_t)l * B * H * kDim;
      at.lse = a.lse != nullptr ? a.lse + (int64_t)l * B * H : nullptr;
      at.num_blocks = a.num_blocks;
      at.nq = B;
      at.heads = H;
      at.max_blocks = M;
      at.topk = a.topk;
      at.scale_log2 = a.scale_log2;
      at.prefill = 0;
      at.q_start = 0;
      sa.block_scores = ia.block_scores;
      sa.block_idx_out = a.block_idx + (int64_t)l * B * a.topk;
      sa.n_sel = a.n_sel != nullptr ? a.n_sel + (int64_t)l * B : nullptr;
      sa.local_blocks = a.local_blocks;
      sa.block_page = a.block_page;
      sa.query_page = a.query_page;
      e = launch_select_attn(sa, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  hipLaunchKernelGGL(decode_step_clear_kernel, dim3(1), dim3(kStepThreads), 0, stream, a.counters,
                     (int)plan.counter_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t max_cand = (int64_t)a.max_blocks - a.local_blocks;
  if (max_cand <= kStepThreads * 8) return launch_step<8>(a, plan.items, stream);
  if (max_cand <= kStepThreads * 32) return launch_step<32>(a, plan.items, stream);
  return hipErrorInvalidValue;
}

}  // namespace uocr
