/*
 * uocr_sparse.h -- C ABI of the SR-SWA block-sparse attention hot path
 * (gfx950 / MI355X).
 *
 * The method (news.rkmt.cn/news/25027, Unlimited-OCR-2 architecture
 * walk-through, Sec. 5 "SR-SWA", steps 1-4; www.lqnn.cn/news/271890,
 * KV-cache section):
 *   1. cached keys are grouped in blocks of 32 tokens;
 *   2. a one-head 128-dim indexer scores every cached key against the query
 *      and a block scores the maximum of its keys;
 *   3. each query keeps its 4 most recent ("local") blocks and the 12
 *      highest-scoring earlier ("remote") blocks, 16 x 32 = 512 tokens;
 *   4. exact causal softmax attention runs over the kept tokens only, 10
 *      heads x 128 dims, K/V heads equal to query heads, K stored rotated.
 * Decode runs steps 2-4 for one query per sequence; chunked prefill runs
 * them for T consecutive rows of one sequence (leheavengame.com OCR 2
 * release article, Sec. 3: the prefill scoring temporary of shape
 * [tokens, context/32] is never materialised here).
 *
 * Conventions for every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns.  Every pointer
 *    argument, unless stated otherwise, is a DEVICE pointer, 16-byte aligned,
 *    owned by the caller.  The library never allocates, frees or
 *    synchronises; scratch memory comes from caller-provided workspaces whose
 *    size uocr_workspace_size() returns.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous and ordered on that stream.
 *  - Return value: UOCR_OK or an error code.  All argument checks run on the
 *    host before any HIP call; a call that fails them launches nothing and
 *    writes nothing.  uocr_last_error() gives a thread-local message.
 *  - Values read on the device (ctx_lens, block tables, block ids) are not
 *    visible to the host checks; kernels clamp a context length to
 *    [0, 32*max_blocks] and skip any block id or pool index out of range, so
 *    corrupt tables cannot make a kernel access memory out of bounds.
 *  - Query at position p sees keys 0..p; its own K/V (and, in prefill, the
 *    whole chunk's) must already be in the cache.
 */
#ifndef UOCR_SPARSE_H
#define UOCR_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UOCR_ABI_VERSION 4

/* Status codes. */
enum {
  UOCR_OK = 0,
  UOCR_EINVAL = 1,      /* null pointer, misaligned pointer, bad config field  */
  UOCR_ESHAPE = 2,      /* sizes or offsets out of the supported range          */
  UOCR_EWORKSPACE = 3,  /* workspace missing or smaller than required           */
  UOCR_EHIP = 4,        /* a HIP launch reported an error                       */
  UOCR_EUNSUPPORTED = 5, /* valid but not supported by this build (see fields)  */
  UOCR_ECAPACITY = 6     /* the block pool has too few free blocks              */
};

/* Operation ids for uocr_workspace_size(). */
enum {
  UOCR_OP_INDEXER_DECODE = 0,
  UOCR_OP_TOPK_DECODE = 1,
  UOCR_OP_ATTN_DECODE = 2,
  UOCR_OP_INDEXER_PREFILL = 3,
  UOCR_OP_TOPK_PREFILL = 4,
  UOCR_OP_ATTN_PREFILL = 5,
  UOCR_OP_DENSE_ATTN_DECODE = 6,
  UOCR_OP_DECODE_STEP = 7      /* rows = n_layers * batch */
};

/*
 * Sparse-attention configuration; the field names follow the released
 * model's sparse_attention_config (news.rkmt.cn/news/25027 Sec. 5 step 3).
 */
typedef struct uocr_sparse_cfg {
  int32_t block_size;   /* sparse_block_size: tokens per block; must be 32              */
  int32_t topk_blocks;  /* sparse_topk_blocks: kept blocks per query, local included
                           (16); local_blocks <= topk_blocks <= 4096                    */
  int32_t local_blocks; /* sparse_local_block: most recent blocks always kept (4);
                           >= 1                                                         */
  int32_t num_heads;    /* attention heads H (10), K/V heads equal; 1..64               */
  int32_t head_dim;     /* D; must be 128                                               */
  int32_t index_dim;    /* indexer dim Di; must be 128                                  */
  float sm_scale;       /* softmax scale applied to q.k (1/sqrt(128)); finite, > 0      */
} uocr_sparse_cfg;

/*
 * One layer's KV cache, block-major.  Pool block b holds 32 consecutive
 * tokens of one sequence:
 *   k_pool, v_pool : [num_blocks][H][32][D] bf16, K already rotated
 *   kidx_pool      : [num_blocks][32][Di]  bf16 (indexer keys)
 *   block_table    : [batch][max_blocks] int32, pool block of each logical
 *                    block of each sequence (entries past a sequence's end are
 *                    ignored)
 *   ctx_lens       : [batch] int32, tokens in the cache per sequence
 * A block x head of K or V is one contiguous 8 KB row group, an indexer block
 * one contiguous 8 KB tile, so every gather is fully coalesced.
 *
 * Page-aware candidates (optional; news.rkmt.cn/news/25027 Sec. 5, the
 * page-aware candidate constraint: the query's own page's image blocks, the
 * local window and a global fallback; leheavengame.com OCR 2 release article
 * Sec. 2 route A, Page Gate).  When block_page is not NULL the remote
 * candidates of a query are ranked by tier first -- tier 1 for blocks tagged
 * with the query's page, tier 0 for all others -- then by score descending
 * and lower block id; the local window is unchanged.  So the query's page's
 * image blocks are kept first and the remaining slots fall back to the best
 * other blocks.
 *   block_page : [batch][max_blocks] int32, the page whose image tokens the
 *                logical block holds, or -1 for blocks holding none
 *   query_page : decode: [batch] int32, the page of each sequence's query;
 *                prefill: [T] int32, the page of each chunk row.  Required
 *                (UOCR_EINVAL otherwise) when block_page is set.
 * Both NULL: plain ranking.  With tiers, a score keeps one bit less of
 * precision in the ranking key (decode: 2^-22 relative; prefill: see
 * uocr_indexer_score_prefill).  Honoured by uocr_topk_attn_decode and
 * uocr_indexer_score_prefill (whose lists uocr_block_topk_prefill merges);
 * uocr_block_topk_decode, which takes no kv, always ranks plainly, and the
 * scoring and attention entries do not use them.
 */
typedef struct uocr_kv {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const uint16_t* kidx_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  int64_t num_blocks;  /* pool blocks P (>= 1)                               */
  int32_t batch;       /* sequences B (>= 0)                                 */
  int32_t max_blocks;  /* block-table row length (>= 1, <= 1,048,576)        */
  const int32_t* block_page; /* optional page tags, see above (NULL: off)   */
  const int32_t* query_page; /* optional query pages, see above              */
} uocr_kv;

/* ---------------------------------------------------------------- decode */

/*
 * Steps 2 (scoring + block max) for one decode query per sequence
 * (news.rkmt.cn/news/25027 Sec. 5 step 2).
 *   q_idx        : [batch][Di] bf16 indexer query of each sequence
 *   block_scores : [batch][max_blocks] float32, written.  For sequence b with
 *                  p = ctx_len-1 and nb = p/32+1 blocks, entry j < nb-local
 *                  (a remote candidate) is max over the block's 32 keys of
 *                  q_idx . kidx (float32 accumulation of exact bf16 products;
 *                  NaN if any of the 32 scores is NaN, which ranks last);
 *                  every other entry is -inf.
 * Uses the k_pool/v_pool fields of kv only for validation (may be NULL).
 */
int uocr_indexer_score_decode(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q_idx,
                              float* block_scores, void* stream);

/*
 * Step 3 for one decode query per sequence (news.rkmt.cn/news/25027 Sec. 5
 * step 3): keeps blocks nb-local..nb-1 and the (topk-local) highest-scoring
 * candidates 0..nb-local-1, ranked by score descending with the lower block id
 * first on ties (-0.0 equals +0.0, NaN ranks last); all candidates when there
 * are no more of them than remote slots.
 *   block_scores : [batch][max_blocks] float32 (as written above)
 *   ctx_lens     : [batch] int32
 *   block_idx    : [batch][topk_blocks] int32, written: kept block ids
 *                  ascending, then -1 padding
 *   n_sel        : [batch] int32 or NULL, written: min(topk, nb)
 */
int uocr_block_topk_decode(const uocr_sparse_cfg* cfg, const float* block_scores, const int32_t* ctx_lens,
                           int32_t batch, int32_t max_blocks, int32_t* block_idx, int32_t* n_sel,
                           void* stream);

/*
 * Step 4 for one decode query per sequence (news.rkmt.cn/news/25027 Sec. 5
 * step 4): per head h, softmax over the kept tokens (blocks in block_idx,
 * tokens <= p) of sm_scale * q_h . k_h, times V.
 *   q         : [batch][H][D] bf16
 *   block_idx : [batch][topk_blocks] int32, distinct block ids in any order;
 *               entries < 0 or >= max_blocks are skipped
 *   out       : [batch][H][D] float32, written (0 when no token is kept)
 *   lse       : [batch][H] float32 or NULL, natural-log log-sum-exp of the
 *               scaled logits (-inf when no token is kept)
 *   ws        : workspace of uocr_workspace_size(cfg, UOCR_OP_ATTN_DECODE,
 *               batch, max_blocks) bytes (NULL allowed when that is 0)
 */
int uocr_sparse_attn_decode(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q,
                            const int32_t* block_idx, float* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * Decode steps 3 and 4 in one launch (news.rkmt.cn/news/25027 Sec. 5 steps
 * 3-4): the selection of uocr_block_topk_decode followed by the attention of
 * uocr_sparse_attn_decode over it, with identical results (each head's
 * workgroup repeats the sequence's selection, so no selection launch sits
 * between a layer's scoring and attention).
 *   q            : [batch][H][D] bf16
 *   block_scores : [batch][max_blocks] float32, as uocr_indexer_score_decode
 *                  writes them
 *   block_idx    : [batch][topk_blocks] int32, written (the selection)
 *   n_sel        : [batch] int32 or NULL
 *   out, lse     : as uocr_sparse_attn_decode
 *   ws           : workspace of uocr_workspace_size(cfg, UOCR_OP_ATTN_DECODE,
 *                  ...) bytes (NULL allowed when that is 0)
 * Requires topk_blocks <= 256 and max_blocks - local_blocks <= 16384;
 * UOCR_EUNSUPPORTED otherwise (use the two separate calls).
 */
int uocr_topk_attn_decode(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q,
                          const float* block_scores, int32_t* block_idx, int32_t* n_sel, float* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * The decode step of a batch over n_layers layers: for every layer l and
 * sequence b, steps 2, 3 and 4 of uocr_indexer_score_decode,
 * uocr_block_topk_decode and uocr_sparse_attn_decode (news.rkmt.cn/news/25027
 * Sec. 5 steps 2-4), with the same scores and selections bit for bit and the
 * same attention up to float32 summation order; layer l + 1 of a sequence is
 * computed after its layer l.  schedule:
 *   UOCR_STEP_ONE_LAUNCH: ONE launch of the whole step.  Work items (scoring
 *     chunks of 16 or 32 blocks, a sequence's selection, per-head attention)
 *     are taken in a fixed ticket order by a grid that stays resident; a
 *     sequence's selection and attention start as soon as its own scoring is
 *     done, overlapping the scoring of other sequences, with no launch gaps.
 *     It needs every layer's q and q_idx in memory before it starts: it
 *     keeps the layer order of each sequence, but it cannot wait for a
 *     layer's queries to be produced from the previous layer's output.  A
 *     model that computes layer l + 1's queries from layer l's attention
 *     calls the step once per layer (n_layers = 1), which runs the per-layer
 *     launches below.
 *   UOCR_STEP_PER_LAYER: per layer, the scoring launch and the fused
 *     selection + attention launch of uocr_topk_attn_decode.
 *   UOCR_STEP_AUTO: the one launch when n_layers >= 4 and either
 *     max_blocks < 2048, batch >= 8 and batch * max_blocks >= 8192, or
 *     batch * max_blocks >= 32768 (the one launch needs enough other
 *     sequences' scoring to hide each sequence's layer-to-layer latency, and
 *     enough layers to amortise its start and end), otherwise per layer.
 * kv describes layer 0 and holds every layer, layer-major:
 *   kv->k_pool, kv->v_pool : [n_layers][num_blocks][H][32][D] bf16
 *   kv->kidx_pool          : [n_layers][num_blocks][32][Di] bf16
 *   block_table, ctx_lens and the page tags are shared by the layers.
 *   q_idx        : [n_layers][batch][Di] bf16
 *   q            : [n_layers][batch][H][D] bf16
 *   block_scores : [n_layers][batch][max_blocks] float32, written
 *   block_idx    : [n_layers][batch][topk_blocks] int32, written (a one
 *                  launch below 2048 blocks first fills it with INT32_MIN,
 *                  which its attention items poll for, and then overwrites
 *                  every entry; other workgroups read it during the call)
 *   n_sel        : [n_layers][batch] int32 or NULL
 *   out          : [n_layers][batch][H][D] float32, written
 *   lse          : [n_layers][batch][H] float32 or NULL
 *   ws           : workspace of uocr_workspace_size(cfg, UOCR_OP_DECODE_STEP,
 *                  n_layers * batch, max_blocks) bytes, 256-byte aligned,
 *                  required whatever the schedule (completion counters of
 *                  the one launch; a clear kernel zeroes them at the start
 *                  of the call, so stale contents do not matter).  After a
 *                  one-launch call the second 32-bit word is nonzero if a
 *                  dependency wait gave up after about a second (never
 *                  expected; the results are then undefined).  Calls that
 *                  share a workspace must be stream-ordered.
 * Requires topk_blocks <= 256, max_blocks - local_blocks <= 16384 and
 * n_layers * batch * (ceil(max_blocks / chunk) + H) < 2^31 work items
 * (chunk = 32 blocks per scoring item from max_blocks 2048 up and when
 * batch * max_blocks >= 16384, 16 otherwise);
 * UOCR_EUNSUPPORTED otherwise.  UOCR_EWORKSPACE when ws is NULL or too
 * small, UOCR_EINVAL when it is not 256-byte aligned or schedule is not one
 * of the three values.
 */
enum { UOCR_STEP_AUTO = 0, UOCR_STEP_ONE_LAUNCH = 1, UOCR_STEP_PER_LAYER = 2 };
int uocr_sparse_decode_step(const uocr_sparse_cfg* cfg, const uocr_kv* kv, int32_t n_layers, int32_t schedule,
                            const uint16_t* q_idx,
                            const uint16_t* q, float* block_scores, int32_t* block_idx, int32_t* n_sel, float* out,
                            float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * uocr_sparse_decode_step without a workspace, for callers that cannot
 * allocate one: code under HIP graph capture, tight serving loops, harnesses
 * that forbid device allocation.  It computes exactly what
 * uocr_sparse_decode_step computes (same kernels, same results bit for bit)
 * and calls no allocating routine; the one launch keeps its completion
 * counters in a static device array of the library, 256 KiB per GPU, which
 * each GPU the library runs on holds until the process ends.
 *   status : [1] int32 or NULL, written: 0, or 1 if a dependency wait of the
 *            one launch gave up (the results are then undefined; never
 *            expected).  It takes the place of the workspace's error word.
 * Limit: when the one launch is taken (UOCR_STEP_ONE_LAUNCH, or
 * UOCR_STEP_AUTO choosing it), n_layers * batch <= 21844;
 * UOCR_EUNSUPPORTED beyond (pass a workspace to uocr_sparse_decode_step).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, two threads) race and give undefined results; calls ordered
 * on one stream are safe, each clears the counters it uses first.  Other
 * requirements and errors as uocr_sparse_decode_step, less the workspace's.
 */
int uocr_sparse_decode_step_static(const uocr_sparse_cfg* cfg, const uocr_kv* kv, int32_t n_layers,
                                   int32_t schedule, const uint16_t* q_idx, const uint16_t* q, float* block_scores,
                                   int32_t* block_idx, int32_t* n_sel, float* out, float* lse, int32_t* status,
                                   void* stream);

/*
 * Dense full-context decode attention, the comparator for the pages'
 * per-step speed claim against full attention (leheavengame.com OCR 2
 * release article, Sec. 1): per head h, softmax over ALL tokens 0..p of the
 * sequence (p = ctx_len-1) of sm_scale * q_h . k_h, times V -- step 4
 * without steps 2-3.  Same caches and conventions as uocr_sparse_attn_decode.
 *   q      : [batch][H][D] bf16
 *   out    : [batch][H][D] float32, written (0 for an empty context)
 *   lse    : [batch][H] float32 or NULL (-inf for an empty context)
 *   ws     : workspace of uocr_workspace_size(cfg, UOCR_OP_DENSE_ATTN_DECODE,
 *            batch, max_blocks) bytes (split-K partials), 16-byte aligned;
 *            UOCR_EWORKSPACE if missing or smaller
 */
int uocr_dense_attn_decode(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q, float* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- chunked prefill */

/*
 * Step 2 for rows t = 0..T-1 of a prefill chunk of sequence 0 of kv
 * (kv->batch must be 1), row t at position p = q_start + t
 * (leheavengame.com OCR 2 release article, Sec. 3, chunked prefill;
 * news.rkmt.cn/news/25027 Sec. 5 step 2).  The dense [T x keys] indexer
 * product runs on bf16 MFMA; scores are max-reduced per block in registers
 * and only each row's best (topk-local) candidates per context split are
 * written to cand_ws (an opaque workspace consumed by
 * uocr_block_topk_prefill), never the [T, context/32] score matrix.
 *   q_idx   : [T][Di] bf16
 *   cand_ws : workspace of uocr_workspace_size(cfg, UOCR_OP_INDEXER_PREFILL,
 *             T, max_blocks) bytes
 * Ranking precision: a list entry keeps a block score's order bits above an
 * in-split block index of idbits = ceil(log2(blocks per split)) bits, so rows
 * are ranked on scores truncated to 2^-(23-idbits) relative, equal truncated
 * scores going to the lower block id.  Up to 16384 blocks a split holds at
 * most 256 blocks (idbits <= 8: 2^-17 at 128K context, 2^-15 at worst);
 * longer contexts take 9 bits (2^-14).  Page tiers take one more bit.
 * Requires 0 <= q_start, T >= 0, q_start + T <= 32 * max_blocks <= 32 * 32768,
 * topk_blocks - local_blocks <= 16, and with page tags max_blocks <= 16384
 * (UOCR_EUNSUPPORTED beyond; the tier bit then keeps scores ranked to 2^-14
 * relative).  With page tags, kv->query_page holds one page per row ([T]).
 */
int uocr_indexer_score_prefill(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q_idx,
                               int32_t q_start, int32_t T, void* cand_ws, size_t cand_ws_bytes, void* stream);

/*
 * Step 3 for the rows scored by uocr_indexer_score_prefill with the same
 * cfg, q_start, T and max_blocks: merges each row's per-split candidates
 * under the decode ranking rule and adds the row's local blocks.
 *   block_idx : [T][topk_blocks] int32, written (ascending, -1 padded)
 *   n_sel     : [T] int32 or NULL
 */
int uocr_block_topk_prefill(const uocr_sparse_cfg* cfg, const void* cand_ws, size_t cand_ws_bytes,
                            int32_t q_start, int32_t T, int32_t max_blocks, int32_t* block_idx,
                            int32_t* n_sel, void* stream);

/*
 * Step 4 for prefill rows: as uocr_sparse_attn_decode with one query per row
 * at p = q_start + t, all rows in sequence 0 of kv (kv->batch must be 1).
 *   q   : [T][H][D] bf16;  block_idx : [T][topk_blocks] int32
 *   out : [T][H][D] float32;  lse : [T][H] float32 or NULL
 *   ws  : NULL, or a 256-byte aligned workspace of uocr_workspace_size(cfg,
 *         UOCR_OP_ATTN_PREFILL, T, max_blocks) bytes.  With it, the chunk's
 *         (row, slot) pairs are bucketed by block and each block's K/V tiles
 *         are read once per chunk, each row's per-block partial softmax states
 *         being merged afterwards (block-major); with ws NULL every row
 *         gathers its own tiles (row-major).  Both give the same result up to
 *         float32 summation order.  The size query returns 0 when this path
 *         does not apply (max_blocks > 16384), and the row-major path then runs
 *         whatever ws is.  UOCR_EWORKSPACE: ws non-NULL and too small;
 *         UOCR_EINVAL: ws not 256-byte aligned.
 *         The block-major path attends each 32-row block's local-window blocks
 *         in a pass of its own, which it runs on a second stream of the
 *         library's (one per device, default priority, created with two events
 *         on the first such call and kept until the process ends): forked from
 *         `stream` with an event and joined back before the merge, so the call
 *         stays ordered on `stream` and can be captured in a HIP graph.  If the
 *         stream or events cannot be created, that pass runs on `stream`.
 */
int uocr_sparse_attn_prefill(const uocr_sparse_cfg* cfg, const uocr_kv* kv, const uint16_t* q, int32_t q_start,
                             int32_t T, const int32_t* block_idx, float* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------ page2d rotary + cache */

/*
 * page2d rotary position encoding (news.rkmt.cn/news/25027 Sec. 4 and
 * Sec. 6), the step that produces the pre-rotated K the attention path reads.
 * A 128-dim row's 64 rotation pairs (i, i+64) -- rotate-half layout, the
 * angles cat(tok, page) doubled -- turn by tok_pos * 10000^(-2i/126) for the
 * 63 token pairs (the token axis samples its own 126-dim spectrum) and by
 * (page_pos mod 2) * 256^0 for the page pair.  tok_pos is the token's offset
 * inside its page and page_pos its page number; the main attention's q/k and
 * the indexer's q/k share them.  The rotation is computed in float64 and
 * rounded once to bf16 (nearest, ties to even).  The coordinates are inputs
 * here; uocr_page_coords derives them from the token stream.
 *
 * uocr_rope_cache_write stores n new tokens into the caches of kv: token t
 * of sequence seq[t] at position pos[t] gets its K rows (every head) and its
 * indexer-K row rotated and its V rows copied into pool block
 * block_table[seq[t]][pos[t]/32], row pos[t]%32.  This entry WRITES the pools
 * that kv points to.  Tokens whose seq, pos or pool block is out of range are
 * skipped on the device.
 *   seq, pos, tok_pos, page_pos : [n] int32
 *   k_new, v_new : [n][H][D] bf16;  kidx_new : [n][Di] bf16
 */
int uocr_rope_cache_write(const uocr_sparse_cfg* cfg, const uocr_kv* kv, int32_t n, const int32_t* seq,
                          const int32_t* pos, const int32_t* tok_pos, const int32_t* page_pos,
                          const uint16_t* k_new, const uint16_t* v_new, const uint16_t* kidx_new, void* stream);

/*
 * Rotates n query tokens in place with the same encoding:
 *   q     : [n][H][D] bf16 or NULL;  q_idx : [n][Di] bf16 or NULL
 *   tok_pos, page_pos : [n] int32
 */
int uocr_rope_queries(const uocr_sparse_cfg* cfg, int32_t n, const int32_t* tok_pos, const int32_t* page_pos,
                      uint16_t* q, uint16_t* q_idx, void* stream);

/*
 * page2d coordinates of token streams (news.rkmt.cn/news/25027 Sec. 4: the
 * page coordinate counts page markers and the token coordinate runs inside
 * the page; in decoding a {page, tok} state advances per token, a marker
 * moving to the next page and sending tok back to the page's start).  For
 * each of `batch` streams of n tokens, from its state (page, tok of the token
 * before the stream): a token equal to `marker` gets (tok 0, page + 1), any
 * other token (tok + 1, page).  A prefill chunk is one stream (batch 1, n =
 * chunk length); a decode step is batch sequences of one token each; calls
 * carrying the state compose exactly like one call over the concatenation.
 *   tokens            : [batch][n] int32
 *   state             : [batch][2] int32 (page, tok), read and updated in place
 *                       (start of a document: page 0, tok -1)
 *   tok_pos, page_pos : [batch][n] int32, written
 */
int uocr_page_coords(int32_t batch, int32_t n, const int32_t* tokens, int32_t marker, int32_t* state,
                     int32_t* tok_pos, int32_t* page_pos, void* stream);

/* ------------------------------------- block pool and page-window schedule */

/*
 * Host-side block pool of the paged caches: it hands out the physical block
 * ids that block_table rows hold (a block = 32 token slots of the K, V and
 * indexer-K pools).  K is stored already rotated with page-local
 * coordinates, so kept blocks can be renumbered: releasing part of a
 * sequence and compacting its table moves no cache data.  Not thread-safe;
 * no GPU calls.
 *
 * uocr_pool_create: num_blocks physical blocks (ids 0..num_blocks-1), up to
 *   max_seqs sequences, all empty; NULL on bad sizes (uocr_last_error says
 *   why).  Free ids are handed out lowest first.
 * uocr_pool_append: grow sequence seq by n_tokens, taking blocks as the
 *   length crosses 32-token boundaries; UOCR_ECAPACITY (nothing changed) when
 *   too few blocks are free.
 * uocr_pool_keep: keep only the blocks that cover the token ranges
 *   [ranges[2r], ranges[2r+1]) (ascending, inside the sequence), in order,
 *   and release the others; the kept blocks become logical blocks 0, 1, ...
 *   and the length becomes 32 per kept block, except that a kept last block
 *   keeps its fill.  The tokens of kept blocks are all kept (ranges are
 *   rounded out to whole blocks).  Bad ranges give UOCR_ESHAPE and change
 *   nothing.
 * uocr_pool_table: the sequence's block-table row (-1 padded to max_blocks
 *   entries) and its length in tokens, for upload as block_table / ctx_lens.
 * uocr_pool_used / uocr_pool_peak: blocks in use now / at most since creation
 *   (-1 for a NULL pool).
 */
typedef struct uocr_pool uocr_pool;
uocr_pool* uocr_pool_create(int32_t num_blocks, int32_t max_seqs);
void uocr_pool_destroy(uocr_pool* pool);
int uocr_pool_append(uocr_pool* pool, int32_t seq, int64_t n_tokens);
int uocr_pool_keep(uocr_pool* pool, int32_t seq, const int64_t* ranges, int32_t n_ranges);
int uocr_pool_table(const uocr_pool* pool, int32_t seq, int32_t* table, int32_t max_blocks, int64_t* length);
int64_t uocr_pool_used(const uocr_pool* pool);
int64_t uocr_pool_peak(const uocr_pool* pool);

/*
 * Page-window schedule of continuous decoding (leheavengame.com OCR 2
 * release article, Sec. 2: parse the document in page windows, adjacent
 * windows sharing one page; on entering the next window keep that page's
 * visual KV and the text at the end of the previous window, release the
 * rest; Sec. 3: the serving deployment's base window of 10 pages).
 * Runs a document of n_pages pages (page k: image_tokens[k] visual tokens,
 * text_tokens[k] parsed-text tokens) through empty sequence seq of pool:
 * window w covers pages w(W-1) .. w(W-1)+W-1 (W = window_pages >= 2); it
 * appends the visual tokens of its pages (all but the shared first page
 * when w > 0), then their text; before the next window, uocr_pool_keep
 * keeps the visual tokens of the window's last page and its last
 * text_tail_tokens text tokens.  window_peaks[w] (if not NULL; max_windows
 * entries) gets the most blocks in use during window w; *n_windows (if not
 * NULL) the number of windows, 0 for no page and 1 + (n_pages - 2) / (W - 1)
 * otherwise, written once the arguments have passed their checks.  Errors: UOCR_EINVAL
 * for NULL arguments, UOCR_ESHAPE for a bad config, a non-empty sequence,
 * negative page sizes or too small a window_peaks (all checked before any
 * change), UOCR_ECAPACITY when the pool runs out part-way (the sequence then
 * holds what the schedule had reached).
 */
typedef struct uocr_page_window {
  int32_t window_pages;
  int32_t text_tail_tokens;
} uocr_page_window;
int uocr_page_window_run(const uocr_page_window* cfg, const int32_t* image_tokens, const int32_t* text_tokens,
                         int32_t n_pages, uocr_pool* pool, int32_t seq, int64_t* window_peaks, int32_t max_windows,
                         int32_t* n_windows);

/* ------------------------------------------------------------- utilities */

/*
 * Bytes of workspace operation `op` needs for `rows` queries (decode: batch;
 * prefill: T) and a block-table row length `max_blocks`; 0 when the
 * operation needs none or the arguments are invalid.
 */
size_t uocr_workspace_size(const uocr_sparse_cfg* cfg, int32_t op, int32_t rows, int32_t max_blocks);

/* Static text of a status code. */
const char* uocr_status_string(int32_t status);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* uocr_last_error(void);

/* UOCR_ABI_VERSION of the built library. */
int32_t uocr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UOCR_SPARSE_H */
