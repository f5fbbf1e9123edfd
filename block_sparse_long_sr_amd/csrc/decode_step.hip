// The whole sparse decode step of a batch in one launch: for every layer and
// sequence, indexer scoring with the block max, top-k block selection and
// the sparse gather attention (SR-SWA steps 2-4, news.rkmt.cn/news/25027
// Sec. 5).
//
// Work items, handed out in ticket order by one atomic counter (a workgroup
// takes its next ticket as it publishes the current item's results, so the
// request's round trip overlaps the stores' and items start in about the
// order of their tickets):
//   * scoring item (layer l, sequence b, chunk c): `chunk` blocks of the
//     sequence's candidates, two 8 KB blocks per wave in flight.  The
//     workgroup that completes the last chunk of (l, b) then runs the
//     selection of (l, b) once and publishes the kept block ids;
//   * attention item (l, b, head h): the attention of head h over the
//     published selection; its local-window blocks, kept whatever the
//     ranking, are attended while the selection is awaited.
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
// cannot hit a stale line; the layer-order wait of a scoring item reads
// nothing the launch produced and takes no fence.  Below 2048 blocks an
// attention item instead polls the published ids themselves with
// device-scope loads (the id output is filled with a pending marker before
// the launch), which needs neither the counter nor the fence.  No L2
// write-back is needed on the writer's side.  A clear kernel zeroes the
// counters (and writes the markers) before each launch.
#include <mutex>

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
constexpr int kTableCache = 4096;  // block-table rows up to this many entries are read into LDS
constexpr int32_t kSelPending = INT32_MIN;  // an id slot not yet published (never a valid output)

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
// then, with ACQ, one acquire fence at device scope (a single cache
// invalidation, not one per poll) before the waiter reads what the counted
// items published.  A wait that only orders work (the next layer's scoring
// reads no data produced inside the launch) takes no fence: each fence
// invalidates the caches of the waiter's XCD for every workgroup on it
// (16 x 12 x 32K: 430 against 412-420 us with the fence on those waits).
template <bool ACQ>
__device__ __forceinline__ void wait_count(uint32_t* ctr, uint32_t need, uint32_t* err, int32_t* status_out) {
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) {
      if (ACQ) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (status_out != nullptr) __hip_atomic_store(status_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Wave 0 only: poll the topk published ids of a slot (device-scope loads)
// until none is kSelPending, and copy them to LDS.  Bounded like wait_count.
__device__ __forceinline__ void wait_ids(const int32_t* sel, int topk, int32_t* s_out, uint32_t* err,
                                         int32_t* status_out) {
  const int lane = lane_id();
  for (int i0 = 0; i0 < topk; i0 += kWave) {
    const int i = i0 + lane;
    int32_t v = 0;
    bool done = false;
    for (uint32_t it = 0; it < kSpinLimit; ++it) {
      v = i < topk ? __hip_atomic_load(sel + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      if (__ballot(v == kSelPending) == 0) {
        done = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!done && lane == 0) {
      __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (status_out != nullptr) __hip_atomic_store(status_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (i < topk) s_out[i] = v;
  }
}

// Device-scope (write-through) store of a value other workgroups read.
template <typename T>
__device__ __forceinline__ void publish(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread, before the barrier that precedes a counter increment: wait
// until the wave's own stores have completed (a barrier alone does not).
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }

// Thread 0: the next work item's ticket.  A workgroup asks for it while
// publishing its current item (after the result stores, before their
// drain), not when the item starts: a ticket taken one item ahead would
// start up to a whole item (5-25 us) after it was handed out, spreading one
// sequence's scoring items over that much time and lengthening its layer
// chain (16 x 12 x 32K: 427 against 452 us).
__device__ __forceinline__ uint32_t take_ticket(uint32_t* ticket) {
  return __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0, after drain_stores and a barrier: count one completion; returns
// the count before it.
__device__ __forceinline__ uint32_t count_done(uint32_t* ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace

// Zeroes the counters and, for a launch whose attention items poll the
// published ids, fills the id output with kSelPending.
__global__ __launch_bounds__(kStepThreads) void decode_step_clear_kernel(uint32_t* counters, int n,
                                                                         int32_t* status_out, int32_t* sel,
                                                                         int64_t nsel) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) counters[i] = 0u;
  for (int64_t i = threadIdx.x; i < nsel; i += blockDim.x) sel[i] = kSelPending;
  if (status_out != nullptr && threadIdx.x == 0) *status_out = 0;
}

// WIDE: the launch keeps one workgroup per compute unit (contexts below 2048
// blocks), so a wave may use 256 VGPRs, and an attention item's wave loads
// the tiles of both its remote blocks before attending either.
template <int KPT, bool WIDE>
__global__ __launch_bounds__(kStepThreads) __attribute__((amdgpu_waves_per_eu(WIDE ? 2 : 4))) void decode_step_kernel(
    DecodeStepArgs a) {
  __shared__ SelectSmem<kStepThreads> sel_sm;
  __shared__ AttendSmem<kStepThreads> att_sm;
  __shared__ int32_t s_blocks[kMaxFusedTopk];
  __shared__ int32_t s_table[kTableCache];
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

  if (tid == 0) s_ticket = take_ticket(ticket);
  __syncthreads();
  uint32_t t = s_ticket;
  while (t < total) {
    uint32_t next_t = 0;  // thread 0: the ticket of the next item
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
      const int j0 = it.idx * chunk;
      const int jend_all = min(j0 + chunk, M);
      const int jend = min(jend_all, ncand);
      // Chunks past the sequence's candidates (ragged batches) hold only -inf
      // scores, which nothing in the launch reads: such an item skips the
      // layer-order wait, the publication and the count, and the slot's
      // selection waits for its cb candidate chunks only.
      const int cb = ncand > 0 ? (ncand + chunk - 1) / chunk : 1;
      if (it.idx >= cb) {
        for (int j = j0 + tid; j < jend_all; j += kStepThreads) scores[j] = -INFINITY;
        if (tid == 0) next_t = take_ticket(ticket);
      } else {
        // the pool indices of the wave's first two blocks are read before the
        // wait for the previous layer (the table does not depend on it)
        const int jA = j0 + wave, jB = jA + kStepWaves;
        const int pbA = jA < jend ? __builtin_amdgcn_readfirstlane(table[jA]) : -1;
        const int pbB = jB < jend ? __builtin_amdgcn_readfirstlane(table[jB]) : -1;
        if (l > 0) {
          if (tid == 0) wait_count<false>(attn_done + (it.slot - B), (uint32_t)H, err, a.status_out);
          __syncthreads();
        }
        if (j0 < jend) {
          const uint4 qv = *reinterpret_cast<const uint4*>(a.q_idx + (int64_t)it.slot * kDim + (lane & 15) * 8);
          const uint16_t* kidx = a.kidx_pool + (int64_t)l * a.kidx_layer_stride;
          // blocks j and j + kStepWaves of the wave are loaded together
          for (int j = jA; j < jend; j += 2 * kStepWaves) {
            const int j2 = j + kStepWaves;
            const int pb = j == jA ? pbA : __builtin_amdgcn_readfirstlane(table[j]);
            const int pb2 = j == jA ? pbB : (j2 < jend ? __builtin_amdgcn_readfirstlane(table[j2]) : -1);
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
        if (tid == 0) next_t = take_ticket(ticket);
        drain_stores();
        __syncthreads();
        if (tid == 0) {
          // the last chunk's workgroup selects.  With one workgroup per CU it
          // reads the other chunks' scores with device-scope loads and takes
          // no cache invalidation of its XCD (16 x 12 x 32K: 381-382 ->
          // 369-377 us); with two, the fence and ordinary loads measured
          // 0.5% faster (128K: 1073-1079 against 1080-1087 us)
          const bool last = count_done(score_done + it.slot) == (uint32_t)(cb - 1);
          if (last && !WIDE) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every chunk's scores are visible
          s_last = last;
        }
        __syncthreads();
        if (s_last) {
          // the slot's scoring is complete: select once for its heads
          const int R = a.topk - a.local_blocks;
          if (!select_trivial(nb, ncand, R, a.topk, s_blocks, kStepThreads))
            select_sorted_reg<kStepThreads, KPT, WIDE>(scores, ncand, R, a.local_blocks, s_blocks, sel_sm,
                                                 a.block_page != nullptr ? a.block_page + (int64_t)b * M : nullptr,
                                                 a.block_page != nullptr ? a.query_page[b] : 0);
          __syncthreads();
          for (int i = tid; i < a.topk; i += kStepThreads) publish(sel_out + i, s_blocks[i]);
          if (a.n_sel != nullptr && tid == 0) a.n_sel[it.slot] = nb < a.topk ? nb : a.topk;
          if (!a.poll_sel) {
            // the attention items wait for this count (with id polling they
            // read the ids themselves, and nothing waits for the stores here)
            drain_stores();
            __syncthreads();
            if (tid == 0) count_done(sel_done + it.slot);
          }
        }
      }
    } else {
      const int h = it.idx;
      const int64_t head_row = (int64_t)it.slot * H + h;
      const int64_t kv_off = (int64_t)l * a.kv_layer_stride;
      const uint16_t* kp = a.k_pool + kv_off;
      const uint16_t* vp = a.v_pool + kv_off;
      // The local window (blocks ncand .. nb - 1) is kept whatever the
      // ranking: the last waves attend it while the selection is awaited, so
      // only the remote blocks' tiles follow the kept ids (16 x 12 x 32K:
      // 400 -> 387-392 us; 128K within its spread, 1084 -> 1080-1083 us).
      WaveAttn st;
      wave_attn_init(st, a.q + head_row * kDim);
      for (int i = kStepWaves - 1 - wave; i < nb - ncand; i += kStepWaves)
        wave_attn_block<true>(kp, vp, table, a.num_blocks, H, h, ncand + i, L - 1, a.scale_log2, st);
      // the sequence's table row goes to LDS meanwhile, so the kept ids are
      // followed by one memory round trip (the tiles)
      const bool cached = M <= kTableCache;
      if (cached)
        for (int i = tid; i < M; i += kStepThreads) s_table[i] = table[i];
      if (a.poll_sel) {
        // the ids themselves are polled: one round trip fewer than the
        // counter, a fence and a read of the ids
        if (wave == 0) wait_ids(sel_out, a.topk, s_blocks, err, a.status_out);
      } else {
        if (tid == 0) wait_count<true>(sel_done + it.slot, 1u, err, a.status_out);
        __syncthreads();
        for (int i = tid; i < a.topk; i += kStepThreads) s_blocks[i] = sel_out[i];
      }
      __syncthreads();
      // the remote blocks: every kept id below ncand
      if (WIDE)
        wave_attn_sel_pairs<kStepThreads, true>(kp, vp, cached ? s_table : table, a.num_blocks, H, h, ncand, L - 1,
                                                s_blocks, a.topk, a.scale_log2, st);
      else
        wave_attn_sel<kStepThreads, true>(kp, vp, cached ? s_table : table, a.num_blocks, H, h, ncand, L - 1,
                                          s_blocks, a.topk, a.scale_log2, st);
      wave_attn_finish<kStepThreads>(st, a.out + head_row * kDim, a.lse != nullptr ? a.lse + head_row : nullptr,
                                     att_sm);
      if (tid == 0) next_t = take_ticket(ticket);
      drain_stores();
      __syncthreads();
      if (tid == 0) count_done(attn_done + it.slot);
    }
    if (tid == 0) s_ticket = next_t;
    __syncthreads();  // the next ticket is in s_ticket; LDS of this item is free
    t = s_ticket;
  }
}

DecodeStepPlan decode_step_plan(int32_t n_layers, int32_t batch, int32_t heads, int32_t max_blocks) {
  DecodeStepPlan p{};
  const int64_t S = (int64_t)n_layers * batch;
  // Blocks per scoring item: 32 (256 KB of indexer keys) at long contexts
  // and for batches of at least 16384 blocks, where an item's fixed cost
  // (its layer-order poll, the store drain and the completion count, one
  // memory round trip each) is worth spreading over more bytes; 16 for
  // smaller batches, so that a sequence's scoring spreads over many
  // workgroups and finishes soon after its first item starts (us per step,
  // 12 layers, one workgroup per CU, chunk 16 / 32 at the lag below:
  // 16 x 32K 410-414 / 399; 16 x 48K 548 / 494; 32 x 32K 766 / 700;
  // 16 x 16K 344 / 368; 8 x 32K 296 / 329; 16 x 8K 313 / 336).
  const int64_t batch_blocks = (int64_t)batch * max_blocks;
  p.chunk = (max_blocks >= 2048 || batch_blocks >= 16384) ? kMaxStepChunk : 16;
  // Workgroups per CU: two at long contexts; one below 2048 blocks, where a
  // sequence's layer chain (scoring, selection, attention) rather than
  // bandwidth sets the pace and half the bytes in flight shorten the memory
  // latency every step of the chain sees (16 x 12 x 32K: 447-464 us against
  // 598 us with two; at 128K two are better, 1103 against 1138 us).
  p.groups_per_cu = max_blocks >= 2048 ? 2 : 1;
  // Slots between a slot's scoring items and its attention items: long
  // enough for the slot's scoring and selection to finish, short enough for
  // its attention to finish before the sequence's next layer comes up, which
  // is batch slots later (below batch, as the ticket order requires).  Half
  // the batch with two workgroups per CU (16 x 128K: lag 8 1082, 6 1080 us);
  // three eighths with one, whose attention items attend their local window
  // while the selection is awaited and so may arrive earlier (us per step at
  // lag 3B/8 / B/2: 16 x 32K 378 / 395; 16 x 16K 335 / 349; 16 x 48K 487 /
  // 488; 32 x 32K 714 / 714).
  p.lag = p.groups_per_cu == 1 ? (3 * batch) / 8 : batch / 2;
  // Attention items poll the published ids directly (the id output is
  // filled with kSelPending before the launch) where the layer chain sets
  // the pace: one memory round trip less per layer (16 x 12 x 32K: 398-406
  // against 408-414 us); at long contexts, where bandwidth does, it measured
  // 0-20 us slower than the counter, which stays there.
  p.poll_sel = p.groups_per_cu == 1 ? 1 : 0;
  p.counter_words = 2 + 3 * S;
  p.ws_bytes = (size_t)((p.counter_words * 4 + 255) / 256 * 256);
  p.items = S * (((int64_t)max_blocks + p.chunk - 1) / p.chunk + heads);
  return p;
}

namespace {
// At most two workgroups of the step kernel share a compute unit: its launch
// bounds allow 128 VGPRs per lane at 4 waves per SIMD, i.e. two 8-wave
// workgroups, and its LDS (well under half of the 160 KB of a CU) does not
// lower that.
static_assert(sizeof(SelectSmem<kStepThreads>) + sizeof(AttendSmem<kStepThreads>) + 4 * kMaxFusedTopk +
                      4 * kTableCache + 4 * kMaxStepChunk + 64 <=
                  160 * 1024 / 2,
              "two step workgroups must fit in one CU's LDS");

template <int KPT, bool WIDE>
hipError_t launch_step(const DecodeStepArgs& a, const DecodeStepPlan& plan, hipStream_t stream) {
  // One resident wave of workgroups (they loop over the tickets).  A grid
  // larger than what fits is also correct: a workgroup takes a ticket only
  // once it runs, so late ones find none left.
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t fit = (int64_t)plan.groups_per_cu * (cus > 0 ? cus : 1);
  const int64_t grid = plan.items < fit ? plan.items : fit;
  hipLaunchKernelGGL((decode_step_kernel<KPT, WIDE>), dim3((unsigned)grid), dim3(kStepThreads), 0, stream, a);
  return hipGetLastError();
}
}  // namespace

// The counters of uocr_sparse_decode_step_static, for callers that cannot
// allocate a workspace: a fixed device array, one copy per GPU, held until
// the process ends.  In host code `scratch` only names the symbol; its
// device address on the current GPU comes from hipGetSymbolAddress, looked up
// once per device and kept below.
static __device__ __align__(256) uint32_t scratch[kStaticStepWords];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
uint32_t* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];
}  // namespace

hipError_t decode_step_static_counters(uint32_t** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  });
  if (g_scratch_status[dev] != hipSuccess) return g_scratch_status[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

bool decode_step_one_launch(int32_t n_layers, int32_t batch, int32_t max_blocks) {
  // The one launch overlaps one sequence's selection and attention with the
  // scoring of others, but a sequence's layers stay in order: each layer of
  // a sequence must be scored, selected and attended within the time the
  // other sequences' scoring of that layer takes, about batch * max_blocks *
  // 8 KB at HBM rate, and the first and last layers run with little to
  // overlap.  Measured (us per step, one launch / per-layer launches, 12
  // layers unless stated): below 2048 blocks (one workgroup per CU) 16 x 4K
  // 261/231, 16 x 8K 296/269, 16 x 16K 327/331, 16 x 24K 355/398, 4 x 32K
  // 256/250, 8 x 32K 286/327, 32 x 8K 392/433, 64 x 4K 515/582, 32 x 16K
  // 459/552, 16 x 32K with 2, 4 and 8 layers 83/76, 142/151, 257/299; from
  // 2048 blocks (two per CU) 8 x 64K 486/455, 4 x 128K 435/442, 16 x 64K
  // 668/703, 8 x 128K 617/701.  Hence: at least 4 layers, and a batch of
  // at least 8192 blocks and 8 sequences below 2048 blocks, of at least
  // 32768 blocks from there.
  const int64_t blocks = (int64_t)batch * max_blocks;
  if (n_layers < 4) return false;
  return max_blocks < 2048 ? (batch >= 8 && blocks >= 8192) : blocks >= 32768;
}

hipError_t launch_decode_step(const DecodeStepArgs& a, const DecodeStepPlan& plan, bool one_launch,
                              hipStream_t stream) {
  if (a.batch == 0 || a.n_layers == 0) return hipSuccess;
  const int B = a.batch, M = a.max_blocks, H = a.heads;
  if (!one_launch) {
    // per-layer launches of the scoring kernel and the fused selection +
    // attention kernel, on the caller's stream (no waits: a status word
    // only needs its 0)
    if (a.status_out != nullptr) {
      hipLaunchKernelGGL(decode_step_clear_kernel, dim3(1), dim3(kStepThreads), 0, stream, a.counters, 0,
                         a.status_out, a.block_idx, (int64_t)0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
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
                     (int)plan.counter_words, a.status_out, a.block_idx,
                     a.poll_sel ? (int64_t)a.n_layers * a.batch * a.topk : (int64_t)0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t max_cand = (int64_t)a.max_blocks - a.local_blocks;
  if (max_cand <= kStepThreads * 2 && plan.groups_per_cu == 1) return launch_step<2, true>(a, plan, stream);
  if (max_cand <= kStepThreads * 8) {
    if (plan.groups_per_cu == 1) return launch_step<8, true>(a, plan, stream);
    return launch_step<8, false>(a, plan, stream);
  }
  if (max_cand <= kStepThreads * 32) return launch_step<32, false>(a, plan, stream);
  return hipErrorInvalidValue;
}

}  // namespace uocr
