// Block pool of the paged KV cache and the page-window schedule of
// continuous decoding (leheavengame.com OCR 2 release article, Sec. 2: the
// document is parsed in page windows, adjacent windows share one page, on
// entering the next window that page's visual KV and the text at the end of
// the previous window are kept and everything else is released; Sec. 3 on the
// page-window size of the serving deployment).
//
// Host-side bookkeeping only: the pool hands out physical block ids of the
// K/V/indexer-K pools that the kernels index through block tables.  K is
// stored already rotated with page-local coordinates, so kept blocks can be
// renumbered freely: releasing and compacting a sequence is a rewrite of its
// block-table row, never a copy of cache data.
#include <algorithm>
#include <cstdint>
#include <functional>
#include <new>
#include <vector>

#include "../../include/uocr_sparse.h"

namespace uocr {
int set_error(int status, const char* fmt, ...);  // api.cpp: thread-local error text
}  // namespace uocr

struct uocr_pool {
  std::vector<int32_t> free_ids;                 // min-heap: the smallest free id is handed out first
  std::vector<std::vector<int32_t>> seq_blocks;  // physical ids of each sequence, logical order
  std::vector<int64_t> seq_len;                  // tokens of each sequence
  int32_t num_blocks = 0;
  int64_t used = 0;
  int64_t peak = 0;
};

namespace {
constexpr int64_t kBlockTokens = 32;

int64_t blocks_for(int64_t tokens) { return (tokens + kBlockTokens - 1) / kBlockTokens; }

void release_ids(uocr_pool* p, const std::vector<int32_t>& ids) {
  for (int32_t id : ids) {
    p->free_ids.push_back(id);
    std::push_heap(p->free_ids.begin(), p->free_ids.end(), std::greater<int32_t>());
  }
  p->used -= (int64_t)ids.size();
}

int32_t take_id(uocr_pool* p) {
  std::pop_heap(p->free_ids.begin(), p->free_ids.end(), std::greater<int32_t>());
  const int32_t id = p->free_ids.back();
  p->free_ids.pop_back();
  return id;
}

// Host allocations can fail; no C++ exception crosses the C ABI.
template <typename F>
int guarded(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return uocr::set_error(UOCR_EINVAL, "out of host memory");
  } catch (...) {
    return uocr::set_error(UOCR_EINVAL, "unexpected host error");
  }
}

int check_seq(const uocr_pool* p, int32_t seq) {
  if (p == nullptr) return uocr::set_error(UOCR_EINVAL, "pool is NULL");
  if (seq < 0 || seq >= (int32_t)p->seq_blocks.size())
    return uocr::set_error(UOCR_ESHAPE, "seq %d outside [0, %d)", seq, (int)p->seq_blocks.size());
  return UOCR_OK;
}
}  // namespace

extern "C" {

uocr_pool* uocr_pool_create(int32_t num_blocks, int32_t max_seqs) {
  if (num_blocks < 0 || max_seqs < 0) {
    uocr::set_error(UOCR_ESHAPE, "num_blocks and max_seqs must be >= 0 (got %d, %d)", num_blocks, max_seqs);
    return nullptr;
  }
  uocr_pool* p = nullptr;
  const int st = guarded([&] {
    p = new uocr_pool;
    p->num_blocks = num_blocks;
    p->free_ids.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) p->free_ids[i] = i;  // ascending order is already a min-heap
    p->seq_blocks.resize(max_seqs);
    p->seq_len.assign(max_seqs, 0);
    return uocr::set_error(UOCR_OK, "");
  });
  if (st != UOCR_OK) {
    delete p;
    return nullptr;
  }
  return p;
}

void uocr_pool_destroy(uocr_pool* pool) { delete pool; }

int uocr_pool_append(uocr_pool* pool, int32_t seq, int64_t n_tokens) {
  return guarded([&] {
    if (int st = check_seq(pool, seq)) return st;
    if (n_tokens < 0) return uocr::set_error(UOCR_ESHAPE, "n_tokens must be >= 0 (got %lld)", (long long)n_tokens);
    const int64_t need = blocks_for(pool->seq_len[seq] + n_tokens) - (int64_t)pool->seq_blocks[seq].size();
    if (need > (int64_t)pool->free_ids.size())
      return uocr::set_error(UOCR_ECAPACITY, "pool exhausted: %lld more blocks needed, %zu free", (long long)need,
                             pool->free_ids.size());
    if (need > 0) pool->seq_blocks[seq].reserve(pool->seq_blocks[seq].size() + need);  // may throw: nothing changed yet
    for (int64_t i = 0; i < need; ++i) pool->seq_blocks[seq].push_back(take_id(pool));
    pool->seq_len[seq] += n_tokens;
    pool->used += need;
    pool->peak = std::max(pool->peak, pool->used);
    return uocr::set_error(UOCR_OK, "");
  });
}

int uocr_pool_keep(uocr_pool* pool, int32_t seq, const int64_t* ranges, int32_t n_ranges) {
  return guarded([&] {
    if (int st = check_seq(pool, seq)) return st;
    if (n_ranges < 0 || (n_ranges > 0 && ranges == nullptr))
      return uocr::set_error(UOCR_EINVAL, "ranges must hold n_ranges >= 0 pairs");
    const int64_t len = pool->seq_len[seq];
    std::vector<char> keep(pool->seq_blocks[seq].size(), 0);
    int64_t prev_hi = 0;
    for (int32_t r = 0; r < n_ranges; ++r) {
      const int64_t lo = ranges[2 * r], hi = ranges[2 * r + 1];
      if (lo < prev_hi || hi < lo || hi > len)
        return uocr::set_error(UOCR_ESHAPE, "range %d [%lld, %lld) not ascending inside [0, %lld)", r, (long long)lo,
                               (long long)hi, (long long)len);
      prev_hi = hi;
      if (hi == lo) continue;  // an empty range keeps nothing
      for (int64_t b = lo / kBlockTokens; b < blocks_for(hi); ++b) keep[b] = 1;
    }
    std::vector<int32_t> kept, dropped;
    int64_t last_fill = 0;
    const int64_t nblk = (int64_t)pool->seq_blocks[seq].size();
    for (int64_t b = 0; b < nblk; ++b) {
      if (keep[b]) {
        kept.push_back(pool->seq_blocks[seq][b]);
        last_fill = (b == nblk - 1) ? len - b * kBlockTokens : kBlockTokens;
      } else {
        dropped.push_back(pool->seq_blocks[seq][b]);
      }
    }
    pool->free_ids.reserve(pool->free_ids.size() + dropped.size());  // may throw: nothing changed yet
    pool->seq_blocks[seq].swap(kept);
    pool->seq_len[seq] = pool->seq_blocks[seq].empty()
                             ? 0
                             : (int64_t)(pool->seq_blocks[seq].size() - 1) * kBlockTokens + last_fill;
    release_ids(pool, dropped);
    return uocr::set_error(UOCR_OK, "");
  });
}

int uocr_pool_table(const uocr_pool* pool, int32_t seq, int32_t* table, int32_t max_blocks, int64_t* length) {
  if (int st = check_seq(pool, seq)) return st;
  const auto& ids = pool->seq_blocks[seq];
  if (max_blocks < (int32_t)ids.size())
    return uocr::set_error(UOCR_ESHAPE, "table row of %d entries, sequence holds %zu blocks", max_blocks, ids.size());
  if (max_blocks > 0 && table == nullptr) return uocr::set_error(UOCR_EINVAL, "table is NULL");
  for (int32_t i = 0; i < max_blocks; ++i) table[i] = i < (int32_t)ids.size() ? ids[i] : -1;
  if (length != nullptr) *length = pool->seq_len[seq];
  return uocr::set_error(UOCR_OK, "");
}

int64_t uocr_pool_used(const uocr_pool* pool) { return pool == nullptr ? -1 : pool->used; }

int64_t uocr_pool_peak(const uocr_pool* pool) { return pool == nullptr ? -1 : pool->peak; }

int uocr_page_window_run(const uocr_page_window* cfg, const int32_t* image_tokens, const int32_t* text_tokens,
                         int32_t n_pages, uocr_pool* pool, int32_t seq, int64_t* window_peaks, int32_t max_windows,
                         int32_t* n_windows_out) {
  if (cfg == nullptr || image_tokens == nullptr || text_tokens == nullptr)
    return uocr::set_error(UOCR_EINVAL, "cfg, image_tokens and text_tokens must not be NULL");
  if (int st = check_seq(pool, seq)) return st;
  if (cfg->window_pages < 2 || cfg->text_tail_tokens < 0 || n_pages < 0)
    return uocr::set_error(UOCR_ESHAPE, "window_pages >= 2, text_tail_tokens >= 0, n_pages >= 0 required");
  if (pool->seq_len[seq] != 0) return uocr::set_error(UOCR_ESHAPE, "sequence %d is not empty", seq);
  for (int32_t k = 0; k < n_pages; ++k)
    if (image_tokens[k] < 0 || text_tokens[k] < 0) return uocr::set_error(UOCR_ESHAPE, "negative page size");
  const int32_t W = cfg->window_pages;
  const int32_t n_windows = n_pages <= 1 ? n_pages : 1 + (n_pages - 2) / (W - 1);
  if (window_peaks != nullptr && max_windows < n_windows)
    return uocr::set_error(UOCR_ESHAPE, "window_peaks holds %d entries, the document has %d windows", max_windows,
                           n_windows);
  if (n_windows_out != nullptr) *n_windows_out = n_windows;
  // Window w covers pages [w(W-1), w(W-1) + W); its first page (w > 0) is the
  // page shared with window w-1: image reused, text already produced.
  for (int32_t w = 0; w < n_windows; ++w) {
    const int32_t first = w * (W - 1);
    const int32_t last = std::min(first + W, n_pages);  // exclusive
    const int32_t new_first = w == 0 ? first : first + 1;
    const int64_t peak_before = pool->used;
    int64_t window_peak = peak_before;
    // image tokens of the window's new pages, then their text
    int64_t shared_image_lo = 0, shared_image_hi = 0;
    for (int32_t k = new_first; k < last; ++k) {
      if (k == last - 1) shared_image_lo = pool->seq_len[seq];
      if (int st = uocr_pool_append(pool, seq, image_tokens[k])) return st;
      if (k == last - 1) shared_image_hi = pool->seq_len[seq];
      window_peak = std::max(window_peak, pool->used);
    }
    for (int32_t k = new_first; k < last; ++k) {
      if (int st = uocr_pool_append(pool, seq, text_tokens[k])) return st;
      window_peak = std::max(window_peak, pool->used);
    }
    if (window_peaks != nullptr) window_peaks[w] = window_peak;
    if (w + 1 < n_windows) {
      // keep the shared page's image and the last text_tail_tokens of text
      int64_t text_end = pool->seq_len[seq];
      int64_t text_start = shared_image_hi;  // the window's text follows its images
      int64_t tail_lo = std::max(text_start, text_end - (int64_t)cfg->text_tail_tokens);
      int64_t ranges[4] = {shared_image_lo, shared_image_hi, tail_lo, text_end};
      if (int st = uocr_pool_keep(pool, seq, ranges, 2)) return st;
    }
  }
  return uocr::set_error(UOCR_OK, "");
}

}  // extern "C"
