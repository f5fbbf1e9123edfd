// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the caller and
// returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace uocr {

struct IndexerDecodeArgs {
  const uint16_t* kidx_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const uint16_t* q_idx;
  float* block_scores;
  int64_t num_blocks;
  int32_t batch;
  int32_t max_blocks;
  int32_t local_blocks;
  int32_t chunk;  // blocks per workgroup
};
hipError_t launch_indexer_decode(const IndexerDecodeArgs& a, hipStream_t stream);
int32_t indexer_decode_chunk(int32_t batch, int32_t max_blocks);

struct TopkDecodeArgs {
  const float* block_scores;
  const int32_t* ctx_lens;
  int32_t* block_idx;
  int32_t* n_sel;
  int32_t batch;
  int32_t max_blocks;
  int32_t topk;
  int32_t local_blocks;
};
hipError_t launch_topk_decode(const TopkDecodeArgs& a, hipStream_t stream);

struct AttnArgs {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;  // decode only
  const uint16_t* q;        // [nq][H][D]
  const int32_t* block_idx; // [nq][topk]
  float* out;               // [nq][H][D]
  float* lse;               // [nq][H] or null
  int64_t num_blocks;
  int32_t nq;
  int32_t heads;
  int32_t max_blocks;
  int32_t topk;
  float scale_log2;         // sm_scale * log2(e)
  int32_t prefill;          // 0: query i is sequence i at ctx_lens[i]-1; 1: row i of sequence 0 at q_start+i
  int32_t q_start;
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

// Block-major prefill attention: the chunk's (row, slot) pairs bucketed by
// block, one pass over each block's K/V tiles writing per-slot partials, a
// log-sum-exp merge per (row, head).
constexpr int32_t kMaxBlocksAttnBucket = 16384;  // bucket counts live in LDS
struct PrefillAttnPlan {
  int32_t max_chunks;  // upper bound of the number of row chunks
  int32_t local_win;   // window blocks attended per row block (the local window; 0: none), set by the caller
  size_t pairs_off, chunk_off, part_off, ml_off;  // byte offsets in the workspace
  size_t ws_bytes;     // 0: sizes not supported by this path
};
PrefillAttnPlan prefill_attn_plan(int32_t T, int32_t heads, int32_t topk, int32_t max_blocks);
struct PrefillAttnArgs {
  AttnArgs attn;  // prefill rows: nq = T
  void* ws;
  PrefillAttnPlan plan;
};
hipError_t launch_attn_prefill_blocks(const PrefillAttnArgs& a, hipStream_t stream);

// Fused decode selection + attention (steps 3 and 4).
constexpr int32_t kMaxFusedTopk = 256;
constexpr int32_t kMaxFusedCandidates = 1024 * 16;
struct SelAttnArgs {
  AttnArgs attn;               // prefill = 0; block_idx unused
  const float* block_scores;   // [B][max_blocks]
  int32_t* block_idx_out;      // [B][topk], written
  int32_t* n_sel;              // [B] or null
  int32_t local_blocks;
  const int32_t* block_page;   // [B][max_blocks] page tags or null (plain ranking)
  const int32_t* query_page;   // [B] query pages (with block_page)
};
hipError_t launch_select_attn(const SelAttnArgs& a, hipStream_t stream);

// The whole decode step of a batch over n_layers layers in one launch
// (scoring, selection and attention as ticket-ordered work items).  Pools,
// queries and outputs are layer-major: layer l of k_pool/v_pool starts at
// l * kv_layer_stride elements, of kidx_pool at l * kidx_layer_stride;
// q_idx [L][B][Di], q [L][B][H][D], block_scores [L][B][M], block_idx
// [L][B][topk], out [L][B][H][D], lse [L][B][H], n_sel [L][B].
struct DecodeStepArgs {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const uint16_t* kidx_pool;
  int64_t kv_layer_stride;
  int64_t kidx_layer_stride;
  const int32_t* block_table;  // [B][M], shared by the layers
  const int32_t* ctx_lens;     // [B]
  const int32_t* block_page;   // [B][M] page tags or null
  const int32_t* query_page;   // [B]
  const uint16_t* q_idx;
  const uint16_t* q;
  float* block_scores;
  int32_t* block_idx;
  float* out;
  float* lse;                  // or null
  int32_t* n_sel;              // or null
  uint32_t* counters;          // workspace: ticket, error word, per-slot completion counts
  int32_t* status_out;         // or null: 0 at the start, 1 if a dependency wait gave up
  int64_t num_blocks;
  int32_t n_layers;
  int32_t batch;
  int32_t max_blocks;
  int32_t heads;
  int32_t topk;
  int32_t local_blocks;
  int32_t lag;
  int32_t chunk;               // blocks per scoring item, a multiple of 16
  int32_t poll_sel;            // 1: attention items poll block_idx itself (cleared to INT32_MIN first)
  float scale_log2;
};
struct DecodeStepPlan {
  int32_t lag;            // slots between a slot's scoring and its attention items
  int32_t chunk;          // blocks per scoring item
  int64_t counter_words;  // 2 + 3 * n_layers * batch
  int64_t items;          // work items of the launch
  int32_t groups_per_cu;  // resident workgroups per compute unit
  int32_t poll_sel;       // attention items poll the published ids (see DecodeStepArgs)
  size_t ws_bytes;
};
DecodeStepPlan decode_step_plan(int32_t n_layers, int32_t batch, int32_t heads, int32_t max_blocks);
// Whether the automatic schedule runs the step as one launch (otherwise as
// per-layer launches of the scoring and fused selection + attention kernels).
bool decode_step_one_launch(int32_t n_layers, int32_t batch, int32_t max_blocks);
hipError_t launch_decode_step(const DecodeStepArgs& a, const DecodeStepPlan& plan, bool one_launch,
                              hipStream_t stream);
// Counters of the no-workspace variant: a static device array of
// kStaticStepWords words (ticket, error word, three per layer-sequence slot);
// *ptr gets its address on the current device (looked up once per device).
constexpr int64_t kStaticStepWords = 65536;  // 256 KiB per GPU
hipError_t decode_step_static_counters(uint32_t** ptr);

// Dense full-context decode attention (comparator): split-K partials in a
// workspace, then a merge.
struct DensePlan {
  int32_t nsplit;   // block-range splits per (sequence, head)
  int32_t bps;      // blocks per split
  size_t ws_bytes;  // batch * heads * nsplit * (128 + 2) floats
};
DensePlan dense_plan(int32_t batch, int32_t heads, int32_t max_blocks);
struct DenseArgs {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const uint16_t* q;   // [B][H][D]
  float* out;          // [B][H][D]
  float* lse;          // [B][H] or null
  float* ws;           // partials
  int64_t num_blocks;
  int32_t batch;
  int32_t heads;
  int32_t max_blocks;
  float scale_log2;
  DensePlan plan;
};
hipError_t launch_dense_attn(const DenseArgs& a, hipStream_t stream);

// page2d rotary encoding: cache write of n new tokens and queries in place.
struct RopeWriteArgs {
  uint16_t* k_pool;            // [P][H][32][D], written
  uint16_t* v_pool;            // [P][H][32][D], written
  uint16_t* kidx_pool;         // [P][32][Di], written
  const int32_t* block_table;  // [batch][max_blocks]
  const int32_t* seq;          // [n]
  const int32_t* pos;          // [n]
  const int32_t* tok_pos;      // [n]
  const int32_t* page_pos;     // [n]
  const uint16_t* k_new;       // [n][H][D]
  const uint16_t* v_new;       // [n][H][D]
  const uint16_t* kidx_new;    // [n][Di]
  int64_t num_blocks;
  int32_t batch;
  int32_t max_blocks;
  int32_t heads;
  int32_t n;
};
hipError_t launch_rope_cache_write(const RopeWriteArgs& a, hipStream_t stream);
struct RopeQueryArgs {
  uint16_t* q;                 // [n][H][D] or null, rotated in place
  uint16_t* q_idx;             // [n][Di] or null, rotated in place
  const int32_t* tok_pos;      // [n]
  const int32_t* page_pos;     // [n]
  int32_t heads;
  int32_t n;
};
hipError_t launch_rope_queries(const RopeQueryArgs& a, hipStream_t stream);

// page2d coordinates of token streams: a page marker opens page + 1 at token
// coordinate 0, any other token advances the in-page count.
struct PageCoordArgs {
  const int32_t* tokens;  // [batch][n]
  int32_t* state;         // [batch][2]: page, tok of the token before; updated
  int32_t* tok_pos;       // [batch][n]
  int32_t* page_pos;      // [batch][n]
  int32_t batch;
  int32_t n;
  int32_t marker;
};
hipError_t launch_page_coords(const PageCoordArgs& a, hipStream_t stream);

// Chunked-prefill scoring: partition of the context into splits.
struct PrefillPlan {
  int32_t n_tiles;   // ceil(T / 256) row tiles
  int32_t bps;       // blocks per split
  int32_t nsplit;    // splits (<= 64)
  int32_t R;         // remote slots = topk - local
  int32_t idbits;    // low key bits that carry the in-split block index
  size_t ws_bytes;   // candidate workspace size
};
PrefillPlan prefill_plan(int32_t T, int32_t max_blocks, int32_t topk, int32_t local_blocks);

struct IndexerPrefillArgs {
  const uint16_t* kidx_pool;
  const int32_t* block_table;  // row of sequence 0
  const uint16_t* q_idx;       // [T][128]
  uint32_t* cand_keys;         // [nsplit][T][R] packed keys, 0 = empty
  int64_t num_blocks;
  int32_t T;
  int32_t q_start;
  int32_t max_blocks;
  int32_t local_blocks;
  PrefillPlan plan;
  const int32_t* block_page;   // row of sequence 0: page tags, or null (plain ranking)
  const int32_t* row_page;     // [T] page of each row (with block_page)
};
hipError_t launch_indexer_prefill(const IndexerPrefillArgs& a, hipStream_t stream);

struct TopkPrefillArgs {
  const uint32_t* cand_keys;
  int32_t* block_idx;  // [T][topk]
  int32_t* n_sel;
  int32_t T;
  int32_t q_start;
  int32_t topk;
  int32_t local_blocks;
  PrefillPlan plan;
};
hipError_t launch_topk_prefill(const TopkPrefillArgs& a, hipStream_t stream);

// Largest in-split index width: packed prefill keys keep 32 - idbits order
// bits, i.e. scores are ranked to 2^-(23 - idbits) relative.
constexpr int32_t kMaxIdBits = 9;
// Longest context (in blocks) of a page-tiered prefill scoring: up to here
// splits hold at most 256 blocks (idbits <= 8), so with the tier bit a score
// still ranks to 2^-14 relative, inside the 1e-4 band of selection parity.
constexpr int32_t kMaxBlocksPrefillTiered = 64 * 256;

}  // namespace uocr
