// C ABI of the SR-SWA hot path: host-side argument checks, then kernel
// launches.  No HIP call is made before every check of a call has passed, so
// the checks run (and are tested) on machines without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/uocr_sparse.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return UOCR_OK;
}

}  // namespace

namespace uocr {
// Status and error text for the host-only parts of the library (pool.cpp):
// UOCR_OK clears the text.
int set_error(int status, const char* fmt, ...) {
  if (status == UOCR_OK) {
    g_last_error[0] = '\0';
    return UOCR_OK;
  }
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}
}  // namespace uocr

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int32_t kMaxTopk = 4096;
constexpr int32_t kMaxBatch = 65535;
constexpr int32_t kMaxBlocks = 1 << 20;
constexpr int32_t kMaxHeads = 64;
constexpr int32_t kMaxRemotePrefill = 16;
constexpr int32_t kMaxBlocksPrefill = 32768;  // 64 splits of <= 512 blocks (in-split index <= 9 bits)

int check_cfg(const uocr_sparse_cfg* c) {
  if (c == nullptr) return fail(UOCR_EINVAL, "cfg is NULL");
  if (c->block_size != 32) return fail(UOCR_EINVAL, "block_size must be 32 (got %d)", c->block_size);
  if (c->head_dim != 128) return fail(UOCR_EINVAL, "head_dim must be 128 (got %d)", c->head_dim);
  if (c->index_dim != 128) return fail(UOCR_EINVAL, "index_dim must be 128 (got %d)", c->index_dim);
  if (c->local_blocks < 1) return fail(UOCR_EINVAL, "local_blocks must be >= 1 (got %d)", c->local_blocks);
  if (c->topk_blocks < c->local_blocks || c->topk_blocks > kMaxTopk)
    return fail(UOCR_EINVAL, "topk_blocks must be in [local_blocks, %d] (got %d, local %d)", kMaxTopk,
                c->topk_blocks, c->local_blocks);
  if (c->num_heads < 1 || c->num_heads > kMaxHeads)
    return fail(UOCR_EINVAL, "num_heads must be in [1, %d] (got %d)", kMaxHeads, c->num_heads);
  if (!std::isfinite(c->sm_scale) || !(c->sm_scale > 0.0f))
    return fail(UOCR_EINVAL, "sm_scale must be finite and > 0");
  return UOCR_OK;
}

int check_dims(int32_t batch, int32_t max_blocks) {
  if (batch < 0 || batch > kMaxBatch) return fail(UOCR_ESHAPE, "batch must be in [0, %d] (got %d)", kMaxBatch, batch);
  if (max_blocks < 1 || max_blocks > kMaxBlocks)
    return fail(UOCR_ESHAPE, "max_blocks must be in [1, %d] (got %d)", kMaxBlocks, max_blocks);
  return UOCR_OK;
}

#define REQ_PTR16(p, name)                                                             \
  do {                                                                                 \
    if ((p) == nullptr) return fail(UOCR_EINVAL, "%s is NULL", name);                  \
    if (!aligned16(p)) return fail(UOCR_EINVAL, "%s is not 16-byte aligned", name);    \
  } while (0)
#define REQ_PTR4(p, name)                                                              \
  do {                                                                                 \
    if ((p) == nullptr) return fail(UOCR_EINVAL, "%s is NULL", name);                  \
    if (!aligned4(p)) return fail(UOCR_EINVAL, "%s is not 4-byte aligned", name);      \
  } while (0)
#define OPT_PTR4(p, name)                                                              \
  do {                                                                                 \
    if ((p) != nullptr && !aligned4(p)) return fail(UOCR_EINVAL, "%s is not 4-byte aligned", name); \
  } while (0)
#define OPT_PTR16(p, name)                                                             \
  do {                                                                                 \
    if ((p) != nullptr && !aligned16(p)) return fail(UOCR_EINVAL, "%s is not 16-byte aligned", name); \
  } while (0)
#define TRY(expr)                  \
  do {                             \
    int _rc = (expr);              \
    if (_rc != UOCR_OK) return _rc; \
  } while (0)

int check_kv(const uocr_kv* kv, bool need_kidx, bool need_kv) {
  if (kv == nullptr) return fail(UOCR_EINVAL, "kv is NULL");
  TRY(check_dims(kv->batch, kv->max_blocks));
  if (kv->batch == 0) return UOCR_OK;
  if (kv->num_blocks < 1) return fail(UOCR_ESHAPE, "kv->num_blocks must be >= 1");
  if (need_kidx) REQ_PTR16(kv->kidx_pool, "kv->kidx_pool");
  if (need_kv) {
    REQ_PTR16(kv->k_pool, "kv->k_pool");
    REQ_PTR16(kv->v_pool, "kv->v_pool");
  }
  REQ_PTR4(kv->block_table, "kv->block_table");
  return UOCR_OK;
}

// Optional page tags (uocr_kv.block_page / query_page): both or neither.
int check_page_gate(const uocr_kv* kv) {
  if (kv->block_page == nullptr) return UOCR_OK;
  REQ_PTR4(kv->block_page, "kv->block_page");
  REQ_PTR4(kv->query_page, "kv->query_page (required with kv->block_page)");
  return UOCR_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(UOCR_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_prefill_range(const uocr_kv* kv, int32_t q_start, int32_t T) {
  if (kv->batch != 1) return fail(UOCR_ESHAPE, "prefill needs kv->batch == 1 (got %d)", kv->batch);
  if (q_start < 0) return fail(UOCR_ESHAPE, "q_start must be >= 0 (got %d)", q_start);
  if (T < 0) return fail(UOCR_ESHAPE, "T must be >= 0 (got %d)", T);
  if ((int64_t)q_start + T > (int64_t)kv->max_blocks * 32)
    return fail(UOCR_ESHAPE, "q_start + T (%lld) exceeds 32 * max_blocks (%lld)", (long long)q_start + T,
                (long long)kv->max_blocks * 32);
  return UOCR_OK;
}

int check_prefill_selection(const uocr_sparse_cfg* cfg, int32_t max_blocks) {
  if (cfg->topk_blocks - cfg->local_blocks > kMaxRemotePrefill)
    return fail(UOCR_EUNSUPPORTED, "prefill supports topk_blocks - local_blocks <= %d (got %d)", kMaxRemotePrefill,
                cfg->topk_blocks - cfg->local_blocks);
  if (max_blocks > kMaxBlocksPrefill)
    return fail(UOCR_EUNSUPPORTED, "prefill supports max_blocks <= %d (got %d)", kMaxBlocksPrefill, max_blocks);
  return UOCR_OK;
}

}  // namespace

extern "C" {

int uocr_indexer_score_decode(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q_idx,
                              float* block_scores, void* stream) {
  TRY(check_cfg(cfg));
  TRY(check_kv(kv, true, false));
  if (kv->batch == 0) return ok();
  REQ_PTR4(kv->ctx_lens, "kv->ctx_lens");
  REQ_PTR16(q_idx, "q_idx");
  REQ_PTR4(block_scores, "block_scores");
  uocr::IndexerDecodeArgs a{};
  a.kidx_pool = kv->kidx_pool;
  a.block_table = kv->block_table;
  a.ctx_lens = kv->ctx_lens;
  a.q_idx = q_idx;
  a.block_scores = block_scores;
  a.num_blocks = kv->num_blocks;
  a.batch = kv->batch;
  a.max_blocks = kv->max_blocks;
  a.local_blocks = cfg->local_blocks;
  a.chunk = uocr::indexer_decode_chunk(kv->batch, kv->max_blocks);
  return hip_status(uocr::launch_indexer_decode(a, static_cast<hipStream_t>(stream)), "indexer_score_decode");
}

int uocr_block_topk_decode(const uocr_sparse_cfg* cfg, const float* block_scores, const int32_t* ctx_lens,
                           int32_t batch, int32_t max_blocks, int32_t* block_idx, int32_t* n_sel, void* stream) {
  TRY(check_cfg(cfg));
  TRY(check_dims(batch, max_blocks));
  if (batch == 0) return ok();
  REQ_PTR4(block_scores, "block_scores");
  REQ_PTR4(ctx_lens, "ctx_lens");
  REQ_PTR4(block_idx, "block_idx");
  OPT_PTR4(n_sel, "n_sel");
  uocr::TopkDecodeArgs a{};
  a.block_scores = block_scores;
  a.ctx_lens = ctx_lens;
  a.block_idx = block_idx;
  a.n_sel = n_sel;
  a.batch = batch;
  a.max_blocks = max_blocks;
  a.topk = cfg->topk_blocks;
  a.local_blocks = cfg->local_blocks;
  return hip_status(uocr::launch_topk_decode(a, static_cast<hipStream_t>(stream)), "block_topk_decode");
}

static int attn_common(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q, const int32_t* block_idx,
                       float* out, float* lse, int32_t nq, int prefill, int32_t q_start, void* ws, size_t ws_bytes,
                       void* stream) {
  REQ_PTR16(q, "q");
  REQ_PTR4(block_idx, "block_idx");
  REQ_PTR4(out, "out");
  OPT_PTR4(lse, "lse");
  uocr::AttnArgs a{};
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.block_table = kv->block_table;
  a.ctx_lens = kv->ctx_lens;
  a.q = q;
  a.block_idx = block_idx;
  a.out = out;
  a.lse = lse;
  a.num_blocks = kv->num_blocks;
  a.nq = nq;
  a.heads = cfg->num_heads;
  a.max_blocks = kv->max_blocks;
  a.topk = cfg->topk_blocks;
  a.scale_log2 = cfg->sm_scale * 1.44269504088896340736f;
  a.prefill = prefill;
  a.q_start = q_start;
  if (prefill && ws != nullptr) {
    const uocr::PrefillAttnPlan P = uocr::prefill_attn_plan(nq, cfg->num_heads, cfg->topk_blocks, kv->max_blocks);
    if (P.ws_bytes > 0) {
      if (ws_bytes < P.ws_bytes)
        return fail(UOCR_EWORKSPACE, "ws holds %zu bytes, block-major prefill attention needs %zu", ws_bytes,
                    P.ws_bytes);
      if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(UOCR_EINVAL, "ws must be 256-byte aligned");
      uocr::PrefillAttnArgs pa{};
      pa.attn = a;
      pa.ws = ws;
      pa.plan = P;
      pa.plan.local_win = cfg->local_blocks > 0 ? cfg->local_blocks : 0;
      return hip_status(uocr::launch_attn_prefill_blocks(pa, static_cast<hipStream_t>(stream)), "sparse_attn_prefill");
    }
  }
  return hip_status(uocr::launch_attn(a, static_cast<hipStream_t>(stream)),
                    prefill ? "sparse_attn_prefill" : "sparse_attn_decode");
}

int uocr_sparse_attn_decode(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q,
                            const int32_t* block_idx, float* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
  (void)ws;
  (void)ws_bytes;  // this implementation needs no workspace (size query returns 0)
  TRY(check_cfg(cfg));
  TRY(check_kv(kv, false, true));
  if (kv->batch == 0) return ok();
  REQ_PTR4(kv->ctx_lens, "kv->ctx_lens");
  return attn_common(cfg, kv, q, block_idx, out, lse, kv->batch, 0, 0, nullptr, 0, stream);
}

int uocr_topk_attn_decode(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q,
                          const float* block_scores, int32_t* block_idx, int32_t* n_sel, float* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;  // no workspace needed (size query returns 0)
  TRY(check_cfg(cfg));
  TRY(check_kv(kv, false, true));
  if (cfg->topk_blocks > uocr::kMaxFusedTopk)
    return fail(UOCR_EUNSUPPORTED, "fused selection + attention supports topk_blocks <= %d (got %d)",
                uocr::kMaxFusedTopk, cfg->topk_blocks);
  if ((int64_t)kv->max_blocks - cfg->local_blocks > uocr::kMaxFusedCandidates)
    return fail(UOCR_EUNSUPPORTED, "fused selection + attention supports max_blocks - local_blocks <= %d",
                uocr::kMaxFusedCandidates);
  if (kv->batch == 0) return ok();
  REQ_PTR4(kv->ctx_lens, "kv->ctx_lens");
  REQ_PTR16(q, "q");
  REQ_PTR4(block_scores, "block_scores");
  REQ_PTR4(block_idx, "block_idx");
  OPT_PTR4(n_sel, "n_sel");
  REQ_PTR4(out, "out");
  OPT_PTR4(lse, "lse");
  TRY(check_page_gate(kv));
  uocr::SelAttnArgs sa{};
  uocr::AttnArgs& a = sa.attn;
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.block_table = kv->block_table;
  a.ctx_lens = kv->ctx_lens;
  a.q = q;
  a.block_idx = nullptr;
  a.out = out;
  a.lse = lse;
  a.num_blocks = kv->num_blocks;
  a.nq = kv->batch;
  a.heads = cfg->num_heads;
  a.max_blocks = kv->max_blocks;
  a.topk = cfg->topk_blocks;
  a.scale_log2 = cfg->sm_scale * 1.44269504088896340736f;
  a.prefill = 0;
  a.q_start = 0;
  sa.block_scores = block_scores;
  sa.block_idx_out = block_idx;
  sa.n_sel = n_sel;
  sa.local_blocks = cfg->local_blocks;
  sa.block_page = kv->block_page;
  sa.query_page = kv->block_page != nullptr ? kv->query_page : nullptr;
  return hip_status(uocr::launch_select_attn(sa, static_cast<hipStream_t>(stream)), "topk_attn_decode");
}

}  // extern "C"

namespace {

// Shared by the two decode-step entry points.  counters: the caller's
// workspace (ws, ws_bytes) or, with use_static, the library's static scratch
// array, whose address is looked up only after every argument check passed.
int decode_step_common(const uocr_sparse_cfg* cfg, const uocr_kv* kv, int32_t n_layers, int32_t schedule,
                       const uint16_t* q_idx, const uint16_t* q, float* block_scores, int32_t* block_idx,
                       int32_t* n_sel, float* out, float* lse, void* ws, size_t ws_bytes, bool use_static,
                       int32_t* status, void* stream, const char* name) {
  TRY(check_cfg(cfg));
  TRY(check_kv(kv, true, true));
  if (n_layers < 0) return fail(UOCR_ESHAPE, "n_layers must be >= 0 (got %d)", n_layers);
  if (schedule != UOCR_STEP_AUTO && schedule != UOCR_STEP_ONE_LAUNCH && schedule != UOCR_STEP_PER_LAYER)
    return fail(UOCR_EINVAL, "schedule must be UOCR_STEP_AUTO, UOCR_STEP_ONE_LAUNCH or UOCR_STEP_PER_LAYER (got %d)",
                schedule);
  if (cfg->topk_blocks > uocr::kMaxFusedTopk)
    return fail(UOCR_EUNSUPPORTED, "the one-launch decode step supports topk_blocks <= %d (got %d)",
                uocr::kMaxFusedTopk, cfg->topk_blocks);
  if ((int64_t)kv->max_blocks - cfg->local_blocks > uocr::kMaxFusedCandidates)
    return fail(UOCR_EUNSUPPORTED, "the one-launch decode step supports max_blocks - local_blocks <= %d",
                uocr::kMaxFusedCandidates);
  if (n_layers == 0 || kv->batch == 0) return ok();
  const uocr::DecodeStepPlan plan = uocr::decode_step_plan(n_layers, kv->batch, cfg->num_heads, kv->max_blocks);
  if (plan.items >= ((int64_t)1 << 31))
    return fail(UOCR_EUNSUPPORTED, "%lld work items (n_layers * batch * (ceil(max_blocks/chunk) + heads)) exceed 2^31",
                (long long)plan.items);
  REQ_PTR4(kv->ctx_lens, "kv->ctx_lens");
  REQ_PTR16(q_idx, "q_idx");
  REQ_PTR16(q, "q");
  REQ_PTR4(block_scores, "block_scores");
  REQ_PTR4(block_idx, "block_idx");
  OPT_PTR4(n_sel, "n_sel");
  REQ_PTR4(out, "out");
  OPT_PTR4(lse, "lse");
  OPT_PTR4(status, "status");
  TRY(check_page_gate(kv));
  const bool one_launch = schedule == UOCR_STEP_ONE_LAUNCH ||
                          (schedule == UOCR_STEP_AUTO &&
                           uocr::decode_step_one_launch(n_layers, kv->batch, kv->max_blocks));
  uint32_t* counters = nullptr;
  if (use_static) {
    if (one_launch && plan.counter_words > uocr::kStaticStepWords)
      return fail(UOCR_EUNSUPPORTED,
                  "the one launch without a workspace supports n_layers * batch <= %lld (got %lld); pass a "
                  "workspace to uocr_sparse_decode_step",
                  (long long)((uocr::kStaticStepWords - 2) / 3), (long long)n_layers * kv->batch);
    if (one_launch) {
      const hipError_t e = uocr::decode_step_static_counters(&counters);
      if (e != hipSuccess) return fail(UOCR_EHIP, "%s: scratch address: %s", name, hipGetErrorString(e));
    }
  } else {
    if (ws == nullptr) return fail(UOCR_EWORKSPACE, "ws is NULL (%zu bytes needed)", plan.ws_bytes);
    if (ws_bytes < plan.ws_bytes)
      return fail(UOCR_EWORKSPACE, "ws holds %zu bytes, %zu needed", ws_bytes, plan.ws_bytes);
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(UOCR_EINVAL, "ws is not 256-byte aligned");
    counters = static_cast<uint32_t*>(ws);
  }
  uocr::DecodeStepArgs a{};
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.kidx_pool = kv->kidx_pool;
  a.kv_layer_stride = kv->num_blocks * cfg->num_heads * 32 * cfg->head_dim;
  a.kidx_layer_stride = kv->num_blocks * 32 * cfg->index_dim;
  a.block_table = kv->block_table;
  a.ctx_lens = kv->ctx_lens;
  a.block_page = kv->block_page;
  a.query_page = kv->block_page != nullptr ? kv->query_page : nullptr;
  a.q_idx = q_idx;
  a.q = q;
  a.block_scores = block_scores;
  a.block_idx = block_idx;
  a.out = out;
  a.lse = lse;
  a.n_sel = n_sel;
  a.counters = counters;
  a.status_out = status;
  a.num_blocks = kv->num_blocks;
  a.n_layers = n_layers;
  a.batch = kv->batch;
  a.max_blocks = kv->max_blocks;
  a.heads = cfg->num_heads;
  a.topk = cfg->topk_blocks;
  a.local_blocks = cfg->local_blocks;
  a.lag = plan.lag;
  a.chunk = plan.chunk;
  a.poll_sel = plan.poll_sel;
  a.scale_log2 = cfg->sm_scale * 1.44269504088896340736f;
  return hip_status(uocr::launch_decode_step(a, plan, one_launch, static_cast<hipStream_t>(stream)), name);
}

}  // namespace

extern "C" {

int uocr_sparse_decode_step(const uocr_sparse_cfg* cfg, const uocr_kv* kv, int32_t n_layers, int32_t schedule,
                            const uint16_t* q_idx,
                            const uint16_t* q, float* block_scores, int32_t* block_idx, int32_t* n_sel, float* out,
                            float* lse, void* ws, size_t ws_bytes, void* stream) {
  return decode_step_common(cfg, kv, n_layers, schedule, q_idx, q, block_scores, block_idx, n_sel, out, lse, ws,
                            ws_bytes, false, nullptr, stream, "sparse_decode_step");
}

int uocr_sparse_decode_step_static(const uocr_sparse_cfg* cfg, const uocr_kv* kv, int32_t n_layers,
                                   int32_t schedule, const uint16_t* q_idx, const uint16_t* q, float* block_scores,
                                   int32_t* block_idx, int32_t* n_sel, float* out, float* lse, int32_t* status,
                                   void* stream) {
  return decode_step_common(cfg, kv, n_layers, schedule, q_idx, q, block_scores, block_idx, n_sel, out, lse,
                            nullptr, 0, true, status, stream, "sparse_decode_step_static");
}

int uocr_dense_attn_decode(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q, float* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream) {
  TRY(check_cfg(cfg));
  TRY(check_kv(kv, false, true));
  if (kv->batch == 0) return ok();
  REQ_PTR4(kv->ctx_lens, "kv->ctx_lens");
  REQ_PTR16(q, "q");
  REQ_PTR4(out, "out");
  OPT_PTR4(lse, "lse");
  const uocr::DensePlan plan = uocr::dense_plan(kv->batch, cfg->num_heads, kv->max_blocks);
  if (ws == nullptr) return fail(UOCR_EWORKSPACE, "ws is NULL (%zu bytes needed)", plan.ws_bytes);
  if (!aligned16(ws)) return fail(UOCR_EINVAL, "ws is not 16-byte aligned");
  if (ws_bytes < plan.ws_bytes) return fail(UOCR_EWORKSPACE, "ws has %zu bytes, %zu needed", ws_bytes, plan.ws_bytes);
  uocr::DenseArgs a{};
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.block_table = kv->block_table;
  a.ctx_lens = kv->ctx_lens;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.ws = static_cast<float*>(ws);
  a.num_blocks = kv->num_blocks;
  a.batch = kv->batch;
  a.heads = cfg->num_heads;
  a.max_blocks = kv->max_blocks;
  a.scale_log2 = cfg->sm_scale * 1.44269504088896340736f;
  a.plan = plan;
  return hip_status(uocr::launch_dense_attn(a, static_cast<hipStream_t>(stream)), "dense_attn_decode");
}

int uocr_indexer_score_prefill(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q_idx,
                               int32_t q_start, int32_t T, void* cand_ws, size_t cand_ws_bytes, void* stream) {
  TRY(check_cfg(cfg));
  TRY(check_kv(kv, true, false));
  TRY(check_prefill_range(kv, q_start, T));
  TRY(check_prefill_selection(cfg, kv->max_blocks));
  const uocr::PrefillPlan plan = uocr::prefill_plan(T, kv->max_blocks, cfg->topk_blocks, cfg->local_blocks);
  if (T == 0 || plan.R == 0) return ok();
  REQ_PTR16(q_idx, "q_idx");
  if (cand_ws == nullptr) return fail(UOCR_EWORKSPACE, "cand_ws is NULL (%zu bytes needed)", plan.ws_bytes);
  if (!aligned16(cand_ws)) return fail(UOCR_EINVAL, "cand_ws is not 16-byte aligned");
  if (cand_ws_bytes < plan.ws_bytes)
    return fail(UOCR_EWORKSPACE, "cand_ws has %zu bytes, %zu needed", cand_ws_bytes, plan.ws_bytes);
  TRY(check_page_gate(kv));
  if (kv->block_page != nullptr && kv->max_blocks > uocr::kMaxBlocksPrefillTiered)
    return fail(UOCR_EUNSUPPORTED, "page-tiered prefill scoring supports max_blocks <= %d (got %d)",
                uocr::kMaxBlocksPrefillTiered, kv->max_blocks);
  uocr::IndexerPrefillArgs a{};
  a.kidx_pool = kv->kidx_pool;
  a.block_table = kv->block_table;
  a.q_idx = q_idx;
  a.cand_keys = static_cast<uint32_t*>(cand_ws);
  a.num_blocks = kv->num_blocks;
  a.T = T;
  a.q_start = q_start;
  a.max_blocks = kv->max_blocks;
  a.local_blocks = cfg->local_blocks;
  a.plan = plan;
  a.block_page = kv->block_page;
  a.row_page = kv->block_page != nullptr ? kv->query_page : nullptr;
  return hip_status(uocr::launch_indexer_prefill(a, static_cast<hipStream_t>(stream)), "indexer_score_prefill");
}

int uocr_block_topk_prefill(const uocr_sparse_cfg* cfg, const void* cand_ws, size_t cand_ws_bytes, int32_t q_start,
                            int32_t T, int32_t max_blocks, int32_t* block_idx, int32_t* n_sel, void* stream) {
  TRY(check_cfg(cfg));
  TRY(check_dims(1, max_blocks));
  if (q_start < 0) return fail(UOCR_ESHAPE, "q_start must be >= 0 (got %d)", q_start);
  if (T < 0) return fail(UOCR_ESHAPE, "T must be >= 0 (got %d)", T);
  if ((int64_t)q_start + T > (int64_t)max_blocks * 32)
    return fail(UOCR_ESHAPE, "q_start + T exceeds 32 * max_blocks");
  TRY(check_prefill_selection(cfg, max_blocks));
  if (T == 0) return ok();
  REQ_PTR4(block_idx, "block_idx");
  OPT_PTR4(n_sel, "n_sel");
  const uocr::PrefillPlan plan = uocr::prefill_plan(T, max_blocks, cfg->topk_blocks, cfg->local_blocks);
  if (plan.ws_bytes > 0) {
    if (cand_ws == nullptr) return fail(UOCR_EWORKSPACE, "cand_ws is NULL (%zu bytes needed)", plan.ws_bytes);
    if (!aligned16(cand_ws)) return fail(UOCR_EINVAL, "cand_ws is not 16-byte aligned");
    if (cand_ws_bytes < plan.ws_bytes)
      return fail(UOCR_EWORKSPACE, "cand_ws has %zu bytes, %zu needed", cand_ws_bytes, plan.ws_bytes);
  }
  uocr::TopkPrefillArgs a{};
  a.cand_keys = static_cast<const uint32_t*>(cand_ws);
  a.block_idx = block_idx;
  a.n_sel = n_sel;
  a.T = T;
  a.q_start = q_start;
  a.topk = cfg->topk_blocks;
  a.local_blocks = cfg->local_blocks;
  a.plan = plan;
  return hip_status(uocr::launch_topk_prefill(a, static_cast<hipStream_t>(stream)), "block_topk_prefill");
}

int uocr_sparse_attn_prefill(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q, int32_t q_start,
                             int32_t T, const int32_t* block_idx, float* out, float* lse, void* ws, size_t ws_bytes,
                             void* stream) {
  TRY(check_cfg(cfg));
  TRY(check_kv(kv, false, true));
  TRY(check_prefill_range(kv, q_start, T));
  if (T == 0) return ok();
  return attn_common(cfg, kv, q, block_idx, out, lse, T, 1, q_start, ws, ws_bytes, stream);
}

int uocr_rope_cache_write(const uocr_sparse_cfg* cfg, const uocr_kv* kv, int32_t n, const int32_t* seq,
                          const int32_t* pos, const int32_t* tok_pos, const int32_t* page_pos,
                          const uint16_t* k_new, const uint16_t* v_new, const uint16_t* kidx_new, void* stream) {
  TRY(check_cfg(cfg));
  TRY(check_kv(kv, true, true));
  if (n < 0) return fail(UOCR_ESHAPE, "n must be >= 0 (got %d)", n);
  if (n == 0 || kv->batch == 0) return ok();
  REQ_PTR4(seq, "seq");
  REQ_PTR4(pos, "pos");
  REQ_PTR4(tok_pos, "tok_pos");
  REQ_PTR4(page_pos, "page_pos");
  REQ_PTR16(k_new, "k_new");
  REQ_PTR16(v_new, "v_new");
  REQ_PTR16(kidx_new, "kidx_new");
  uocr::RopeWriteArgs a{};
  a.k_pool = const_cast<uint16_t*>(kv->k_pool);
  a.v_pool = const_cast<uint16_t*>(kv->v_pool);
  a.kidx_pool = const_cast<uint16_t*>(kv->kidx_pool);
  a.block_table = kv->block_table;
  a.seq = seq;
  a.pos = pos;
  a.tok_pos = tok_pos;
  a.page_pos = page_pos;
  a.k_new = k_new;
  a.v_new = v_new;
  a.kidx_new = kidx_new;
  a.num_blocks = kv->num_blocks;
  a.batch = kv->batch;
  a.max_blocks = kv->max_blocks;
  a.heads = cfg->num_heads;
  a.n = n;
  return hip_status(uocr::launch_rope_cache_write(a, static_cast<hipStream_t>(stream)), "rope_cache_write");
}

int uocr_rope_queries(const uocr_sparse_cfg* cfg, int32_t n, const int32_t* tok_pos, const int32_t* page_pos,
                      uint16_t* q, uint16_t* q_idx, void* stream) {
  TRY(check_cfg(cfg));
  if (n < 0) return fail(UOCR_ESHAPE, "n must be >= 0 (got %d)", n);
  if (n == 0 || (q == nullptr && q_idx == nullptr)) return ok();
  REQ_PTR4(tok_pos, "tok_pos");
  REQ_PTR4(page_pos, "page_pos");
  OPT_PTR16(q, "q");
  OPT_PTR16(q_idx, "q_idx");
  uocr::RopeQueryArgs a{};
  a.q = q;
  a.q_idx = q_idx;
  a.tok_pos = tok_pos;
  a.page_pos = page_pos;
  a.heads = cfg->num_heads;
  a.n = n;
  return hip_status(uocr::launch_rope_queries(a, static_cast<hipStream_t>(stream)), "rope_queries");
}

int uocr_page_coords(int32_t batch, int32_t n, const int32_t* tokens, int32_t marker, int32_t* state,
                     int32_t* tok_pos, int32_t* page_pos, void* stream) {
  if (batch < 0 || n < 0) return fail(UOCR_ESHAPE, "batch and n must be >= 0 (got %d, %d)", batch, n);
  if (batch == 0 || n == 0) return ok();
  if ((int64_t)batch * n > INT64_C(1) << 40) return fail(UOCR_ESHAPE, "batch * n too large");
  REQ_PTR4(tokens, "tokens");
  REQ_PTR4(state, "state");
  REQ_PTR4(tok_pos, "tok_pos");
  REQ_PTR4(page_pos, "page_pos");
  uocr::PageCoordArgs a{};
  a.tokens = tokens;
  a.state = state;
  a.tok_pos = tok_pos;
  a.page_pos = page_pos;
  a.batch = batch;
  a.n = n;
  a.marker = marker;
  return hip_status(uocr::launch_page_coords(a, static_cast<hipStream_t>(stream)), "page_coords");
}

size_t uocr_workspace_size(const uocr_sparse_cfg* cfg, int32_t op, int32_t rows, int32_t max_blocks) {
  if (check_cfg(cfg) != UOCR_OK || rows < 0 || max_blocks < 1 || max_blocks > kMaxBlocks) return 0;
  switch (op) {
    case UOCR_OP_DENSE_ATTN_DECODE:
      return uocr::dense_plan(rows, cfg->num_heads, max_blocks).ws_bytes;
    case UOCR_OP_DECODE_STEP:
      return uocr::decode_step_plan(1, rows, cfg->num_heads, max_blocks).ws_bytes;
    case UOCR_OP_ATTN_PREFILL:
      return uocr::prefill_attn_plan(rows, cfg->num_heads, cfg->topk_blocks, max_blocks).ws_bytes;
    case UOCR_OP_INDEXER_PREFILL:
    case UOCR_OP_TOPK_PREFILL:
      if (cfg->topk_blocks - cfg->local_blocks > kMaxRemotePrefill || max_blocks > kMaxBlocksPrefill) return 0;
      return uocr::prefill_plan(rows, max_blocks, cfg->topk_blocks, cfg->local_blocks).ws_bytes;
    default:
      return 0;
  }
}

const char* uocr_status_string(int32_t status) {
  switch (status) {
    case UOCR_OK: return "UOCR_OK";
    case UOCR_EINVAL: return "UOCR_EINVAL: invalid argument";
    case UOCR_ESHAPE: return "UOCR_ESHAPE: size or offset out of range";
    case UOCR_EWORKSPACE: return "UOCR_EWORKSPACE: workspace missing or too small";
    case UOCR_EHIP: return "UOCR_EHIP: HIP launch error";
    case UOCR_EUNSUPPORTED: return "UOCR_EUNSUPPORTED: configuration not supported";
    case UOCR_ECAPACITY: return "UOCR_ECAPACITY: block pool exhausted";
    default: return "unknown status";
  }
}

const char* uocr_last_error(void) { return g_last_error; }

int32_t uocr_abi_version(void) { return UOCR_ABI_VERSION; }

}  // extern "C"
