// Host-side manager of the adapter page pool (see include/lora_pool.h):
// free pages as ordered ranges, resident adapters in least-recently-used
// order, and the upload of packed adapter pages into the pool.
//
// [MLSP] "Unified Paging Architecture" and "Tiered Storage Hierarchy";
// [MLSA] "S-LoRA unified paging", "The cold-load path and routing" and "An
// adapter-cache LRU simulator".
#include "lora_pool.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <list>
#include <map>
#include <new>
#include <unordered_map>
#include <vector>

struct lora_page_cache {
  int32_t num_pages = 0;
  int32_t free_count = 0;
  std::map<int32_t, int32_t> free_ranges;  // first page -> length, disjoint, never adjacent
  struct Entry {
    std::vector<int32_t> pages;
    std::list<int64_t>::iterator pos;  // in lru (front = most recently used)
    bool pinned = false;
  };
  std::list<int64_t> lru;
  std::unordered_map<int64_t, Entry> resident;

  // lowest n free page ids, removed from the free ranges
  void take(int32_t n, int32_t* out) {
    int32_t got = 0;
    while (got < n) {
      auto it = free_ranges.begin();
      const int32_t start = it->first, len = it->second;
      const int32_t k = std::min(len, n - got);
      for (int32_t i = 0; i < k; ++i) out[got++] = start + i;
      free_ranges.erase(it);
      if (k < len) free_ranges.emplace(start + k, len - k);
    }
    free_count -= n;
  }

  // return pages to the free ranges, merging neighbours
  void give(const std::vector<int32_t>& pages) {
    std::vector<int32_t> p(pages);
    std::sort(p.begin(), p.end());
    for (size_t i = 0; i < p.size();) {
      size_t j = i + 1;
      while (j < p.size() && p[j] == p[j - 1] + 1) ++j;
      int32_t start = p[i], len = static_cast<int32_t>(j - i);
      auto next = free_ranges.lower_bound(start);
      if (next != free_ranges.end() && next->first == start + len) {
        len += next->second;
        next = free_ranges.erase(next);
      }
      if (next != free_ranges.begin()) {
        auto prev = std::prev(next);
        if (prev->first + prev->second == start) {
          prev->second += len;
          i = j;
          continue;
        }
      }
      free_ranges.emplace(start, len);
      i = j;
    }
    free_count += static_cast<int32_t>(pages.size());
  }
};

extern "C" {

lora_status_t lora_cache_create(int32_t num_pages, lora_page_cache_t** out) {
  if (num_pages < 1 || !out) return LORA_ERR_INVALID_ARG;
  lora_page_cache_t* c = new (std::nothrow) lora_page_cache_t();
  if (!c) return LORA_ERR_POOL_FULL;
  c->num_pages = num_pages;
  c->free_count = num_pages;
  c->free_ranges.emplace(0, num_pages);
  *out = c;
  return LORA_OK;
}

void lora_cache_destroy(lora_page_cache_t* cache) { delete cache; }

int32_t lora_cache_free_pages(const lora_page_cache_t* cache) { return cache ? cache->free_count : 0; }

int32_t lora_cache_num_resident(const lora_page_cache_t* cache) {
  return cache ? static_cast<int32_t>(cache->resident.size()) : 0;
}

lora_status_t lora_cache_admit(lora_page_cache_t* c, int64_t key, int32_t n_pages, int32_t* pages_out, int32_t* hit,
                               int64_t* evicted_out, int32_t max_evicted, int32_t* n_evicted) {
  if (!c || n_pages < 1 || !pages_out || !hit || !n_evicted || max_evicted < 0 ||
      (max_evicted > 0 && !evicted_out))
    return LORA_ERR_INVALID_ARG;
  auto found = c->resident.find(key);
  if (found != c->resident.end()) {
    auto& e = found->second;
    if (static_cast<int32_t>(e.pages.size()) != n_pages) return LORA_ERR_INVALID_ARG;
    c->lru.splice(c->lru.begin(), c->lru, e.pos);  // most recently used
    std::copy(e.pages.begin(), e.pages.end(), pages_out);
    *hit = 1;
    *n_evicted = 0;
    return LORA_OK;
  }
  if (n_pages > c->num_pages) return LORA_ERR_POOL_FULL;
  // choose the victims first (least recently used, unpinned), change nothing
  // unless the admission can succeed
  std::vector<int64_t> victims;
  int32_t avail = c->free_count;
  for (auto it = c->lru.rbegin(); it != c->lru.rend() && avail < n_pages; ++it) {
    const auto& e = c->resident.at(*it);
    if (e.pinned) continue;
    victims.push_back(*it);
    avail += static_cast<int32_t>(e.pages.size());
  }
  if (avail < n_pages || static_cast<int32_t>(victims.size()) > max_evicted) return LORA_ERR_POOL_FULL;
  for (size_t i = 0; i < victims.size(); ++i) {
    auto it = c->resident.find(victims[i]);
    c->give(it->second.pages);
    c->lru.erase(it->second.pos);
    c->resident.erase(it);
    evicted_out[i] = victims[i];
  }
  lora_page_cache::Entry e;
  e.pages.resize(n_pages);
  c->take(n_pages, e.pages.data());
  std::copy(e.pages.begin(), e.pages.end(), pages_out);
  c->lru.push_front(key);
  e.pos = c->lru.begin();
  c->resident.emplace(key, std::move(e));
  *hit = 0;
  *n_evicted = static_cast<int32_t>(victims.size());
  return LORA_OK;
}

lora_status_t lora_cache_lookup(const lora_page_cache_t* c, int64_t key, int32_t* pages_out, int32_t max_pages,
                                int32_t* n_pages) {
  if (!c || !n_pages || max_pages < 0 || (max_pages > 0 && !pages_out)) return LORA_ERR_INVALID_ARG;
  auto it = c->resident.find(key);
  const int32_t n = it == c->resident.end() ? 0 : static_cast<int32_t>(it->second.pages.size());
  if (max_pages > 0 && max_pages < n) return LORA_ERR_INVALID_ARG;
  *n_pages = n;
  if (max_pages > 0 && n > 0) std::copy(it->second.pages.begin(), it->second.pages.end(), pages_out);
  return LORA_OK;
}

lora_status_t lora_cache_set_pinned(lora_page_cache_t* c, int64_t key, int32_t pinned) {
  if (!c) return LORA_ERR_INVALID_ARG;
  auto it = c->resident.find(key);
  if (it == c->resident.end()) return LORA_ERR_INVALID_ARG;
  it->second.pinned = pinned != 0;
  return LORA_OK;
}

lora_status_t lora_cache_release(lora_page_cache_t* c, int64_t key) {
  if (!c) return LORA_ERR_INVALID_ARG;
  auto it = c->resident.find(key);
  if (it == c->resident.end()) return LORA_ERR_INVALID_ARG;
  c->give(it->second.pages);
  c->lru.erase(it->second.pos);
  c->resident.erase(it);
  return LORA_OK;
}

lora_status_t lora_upload_pages(const lora_pool_t* pool, const void* host_src, const int32_t* pages_host,
                                int32_t n_pages, void* stream) {
  if (!pool || !pool->base || n_pages < 0 || (n_pages > 0 && (!host_src || !pages_host))) return LORA_ERR_INVALID_ARG;
  if (pool->dtype != LORA_DTYPE_BF16 && pool->dtype != LORA_DTYPE_F32) return LORA_ERR_UNSUPPORTED;
  if (pool->page_width < 1 || pool->num_pages < 1) return LORA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n_pages; ++i)
    if (pages_host[i] < 0 || pages_host[i] >= pool->num_pages) return LORA_ERR_PAGE_RANGE;
  const size_t elem = pool->dtype == LORA_DTYPE_BF16 ? 2 : 4;
  const size_t page_bytes = static_cast<size_t>(LORA_PAGE_ROWS) * pool->page_width * elem;
  const char* src = static_cast<const char*>(host_src);
  char* base = static_cast<char*>(pool->base);
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t i = 0; i < n_pages;) {
    int32_t j = i + 1;
    while (j < n_pages && pages_host[j] == pages_host[j - 1] + 1) ++j;  // one transfer per run
    if (hipMemcpyAsync(base + static_cast<size_t>(pages_host[i]) * page_bytes, src + static_cast<size_t>(i) * page_bytes,
                       static_cast<size_t>(j - i) * page_bytes, hipMemcpyHostToDevice, st) != hipSuccess)
      return LORA_ERR_HIP;
    i = j;
  }
  return LORA_OK;
}

}  // extern "C"
