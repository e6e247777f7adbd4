// Host-side pool of 128-token cache pages and per-sequence page-table rows (the block manager a paged
// serving engine runs beside the kernels: block_size 128 in blog.hypho.cn, "KV-cache 量化终于能跑生产了？
// KVarN 用方差归一化打破 vLLM 的吞吐量魔咒", section "工程实践：一行配置启用").
//
// A page holds the records of one 128-token tile for every kv head of a sequence; the caller's cache
// pool is num_pages * page_stride bytes.  A sequence needs a page only for a tile that is full: the
// newest len % 128 tokens live in the fp16 tail, and kvarn_append_token writes a tile's page when its
// 128th token arrives.  So reserving for a length L means pages for tiles 0 .. L/128 - 1; a caller that
// replays several decode steps without returning to the host reserves for the length after the last of
// them.  Pure host code: no HIP calls.
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "libkvarn.h"

struct kvarn_page_pool {
  std::mutex mu;
  std::vector<int32_t> free_ids;  // stack; the next page handed out is at the back
  std::vector<uint8_t> in_use;    // per page id
};

namespace {

constexpr int32_t kTile = 128;
constexpr int32_t kNoPage = -1;

int32_t full_tiles(int32_t len) { return len / kTile; }

}  // namespace

extern "C" kvarn_status kvarn_page_pool_create(int32_t num_pages, kvarn_page_pool** out) {
  if (out == nullptr || num_pages < 0) return KVARN_E_INVALID_ARG;
  *out = nullptr;
  kvarn_page_pool* p = new (std::nothrow) kvarn_page_pool;
  if (p == nullptr) return KVARN_E_INVALID_ARG;
  try {
    p->free_ids.resize(static_cast<size_t>(num_pages));
    p->in_use.assign(static_cast<size_t>(num_pages), 0);
  } catch (...) {
    delete p;
    return KVARN_E_INVALID_ARG;
  }
  // ascending ids come out first
  for (int32_t i = 0; i < num_pages; ++i) p->free_ids[static_cast<size_t>(i)] = num_pages - 1 - i;
  *out = p;
  return KVARN_OK;
}

extern "C" void kvarn_page_pool_destroy(kvarn_page_pool* pool) { delete pool; }

extern "C" int32_t kvarn_page_pool_num_free(kvarn_page_pool* pool) {
  if (pool == nullptr) return -1;
  std::lock_guard<std::mutex> lock(pool->mu);
  return static_cast<int32_t>(pool->free_ids.size());
}

extern "C" kvarn_status kvarn_page_pool_reserve(kvarn_page_pool* pool, int32_t num_seqs, const int32_t* new_lens,
                                                int32_t* page_table, int32_t max_pages_per_seq,
                                                int32_t* num_owned) {
  if (pool == nullptr || num_seqs < 0 || max_pages_per_seq < 0) return KVARN_E_INVALID_ARG;
  if (num_seqs == 0) return KVARN_OK;
  if (new_lens == nullptr || page_table == nullptr || num_owned == nullptr) return KVARN_E_INVALID_ARG;
  // validate the whole batch and count, before taking anything
  int64_t need = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (new_lens[s] < 0 || num_owned[s] < 0 || num_owned[s] > max_pages_per_seq) return KVARN_E_INVALID_ARG;
    const int32_t want = full_tiles(new_lens[s]);
    if (want > max_pages_per_seq) return KVARN_E_INVALID_ARG;
    if (want > num_owned[s]) need += want - num_owned[s];
  }
  std::lock_guard<std::mutex> lock(pool->mu);
  if (need > static_cast<int64_t>(pool->free_ids.size())) return KVARN_E_OUT_OF_PAGES;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t* row = page_table + static_cast<int64_t>(s) * max_pages_per_seq;
    for (int32_t p = num_owned[s]; p < full_tiles(new_lens[s]); ++p) {
      const int32_t id = pool->free_ids.back();
      pool->free_ids.pop_back();
      pool->in_use[static_cast<size_t>(id)] = 1;
      row[p] = id;
    }
    if (full_tiles(new_lens[s]) > num_owned[s]) num_owned[s] = full_tiles(new_lens[s]);
  }
  return KVARN_OK;
}

extern "C" kvarn_status kvarn_page_pool_release(kvarn_page_pool* pool, int32_t* page_table_row,
                                                int32_t max_pages_per_seq, int32_t* num_owned) {
  if (pool == nullptr || num_owned == nullptr || max_pages_per_seq < 0) return KVARN_E_INVALID_ARG;
  const int32_t n = *num_owned;
  if (n < 0 || n > max_pages_per_seq || (n > 0 && page_table_row == nullptr)) return KVARN_E_INVALID_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  const int32_t num_pages = static_cast<int32_t>(pool->in_use.size());
  // every id must be a page this pool handed out and not yet returned, and appear once
  std::vector<uint8_t> seen;
  for (int32_t p = 0; p < n; ++p) {
    const int32_t id = page_table_row[p];
    if (id < 0 || id >= num_pages || !pool->in_use[static_cast<size_t>(id)]) return KVARN_E_INVALID_ARG;
    if (seen.empty()) seen.assign(static_cast<size_t>(num_pages), 0);
    if (seen[static_cast<size_t>(id)]) return KVARN_E_INVALID_ARG;
    seen[static_cast<size_t>(id)] = 1;
  }
  // most recently reserved pages go back on top
  for (int32_t p = n - 1; p >= 0; --p) {
    const int32_t id = page_table_row[p];
    pool->in_use[static_cast<size_t>(id)] = 0;
    pool->free_ids.push_back(id);
    page_table_row[p] = kNoPage;
  }
  *num_owned = 0;
  return KVARN_OK;
}
