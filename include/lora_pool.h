/*
 * lora_pool.h -- the adapter page pool's host-side manager: which pages of
 * the unified pool hold which adapter, which adapters to evict when a new one
 * is admitted, and the upload of an adapter's packed pages into the pool.
 *
 * Sources:
 *   [MLSP] "Multi-LoRA Serving in Production: Architecture, Dynamic Adapter
 *          Swapping, and GPU Memory Management", sections "Unified Paging
 *          Architecture" (adapter weights live in fixed-size pages of one
 *          pool and are addressed through physical page ids), "Tiered
 *          Storage Hierarchy" (hot adapters in GPU memory, the rest in pinned
 *          host memory, moved in on demand) and "Production Engineering
 *          Guidelines", item 1 (a miss starts a non-blocking copy from pinned
 *          host memory into the pool while scheduling goes on).
 *   [MLSA] "Multi-LoRA Serving Architecture: Serving Hundreds of Fine-Tuned
 *          Adapters on One GPU with vLLM and S-LoRA (2026)", sections
 *          "S-LoRA unified paging", "The cold-load path and routing" and "An
 *          adapter-cache LRU simulator" (a fixed number of resident adapters,
 *          least recently used one evicted on a miss).
 *
 * The page format is the one of lora.h: page p is 16 x page_width elements
 * at pool->base + p*16*page_width.  An adapter occupies whole pages; the
 * caller decides how many (for the tables of lora.h: the sum over its
 * projections of ceil(r/16) * (ceil(d_in/PW) + ceil(d_out/PW))) and builds the
 * page tables from the page ids returned here.
 *
 * The cache is host state owned by the caller through an opaque handle; it is
 * not thread-safe (one thread, or the caller's lock).  It allocates host
 * memory only (std containers); no call below allocates device memory.
 */
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lora.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lora_page_cache lora_page_cache_t;

/* A cache over pool pages [0, num_pages), all free.  *out receives the
 * handle.  Errors: INVALID_ARG (num_pages < 1 or out NULL), POOL_FULL (host
 * memory for the handle could not be allocated). */
lora_status_t lora_cache_create(int32_t num_pages, lora_page_cache_t** out);

/* Frees the handle (NULL is allowed). */
void lora_cache_destroy(lora_page_cache_t* cache);

/* Pages currently free, and adapters currently resident. */
int32_t lora_cache_free_pages(const lora_page_cache_t* cache);
int32_t lora_cache_num_resident(const lora_page_cache_t* cache);

/* Admit adapter `key` with n_pages pages ([MLSA] "The cold-load path"):
 *  - resident: *hit = 1, it becomes the most recently used, and its pages
 *    are written to pages_out (host, n_pages entries; n_pages must equal the
 *    count it was admitted with);
 *  - not resident: *hit = 0; least recently used unpinned adapters are
 *    evicted until n_pages pages are free, the lowest free page ids are
 *    assigned (in ascending order) and written to pages_out, and the evicted
 *    keys are written to evicted_out (host, oldest first, *n_evicted of
 *    them).  The caller uploads the adapter's pages (lora_upload_pages) and
 *    rewrites the tables of the evicted adapters.
 * Errors, with nothing changed: INVALID_ARG (bad pointers, n_pages < 1, a
 * resident key with another page count), POOL_FULL (not enough pages even
 * after evicting every unpinned adapter, or more evictions than
 * max_evicted). */
lora_status_t lora_cache_admit(lora_page_cache_t* cache, int64_t key, int32_t n_pages, int32_t* pages_out,
                               int32_t* hit, int64_t* evicted_out, int32_t max_evicted, int32_t* n_evicted);

/* Residency query that leaves the recency order alone: *n_pages receives the
 * adapter's page count (0 if it is not resident) and, when max_pages is at
 * least that count, its pages are written to pages_out (host).  max_pages 0
 * with pages_out NULL asks for the count only.  Errors: INVALID_ARG (cache
 * or n_pages NULL, max_pages < 0, pages_out NULL with max_pages > 0, or
 * 0 < max_pages < the page count). */
lora_status_t lora_cache_lookup(const lora_page_cache_t* cache, int64_t key, int32_t* pages_out, int32_t max_pages,
                                int32_t* n_pages);

/* Pin (pinned != 0) or unpin a resident adapter: a pinned adapter is never
 * evicted.  Uses: keeping the most requested adapters resident ([MLSA] "The
 * cold-load path and routing" and "Practical Recommendations"), and keeping
 * the adapters of a batch that is still in flight from being overwritten.
 * Errors: INVALID_ARG (not resident). */
lora_status_t lora_cache_set_pinned(lora_page_cache_t* cache, int64_t key, int32_t pinned);

/* Remove a resident adapter and free its pages.  Errors: INVALID_ARG (not
 * resident). */
lora_status_t lora_cache_release(lora_page_cache_t* cache, int64_t key);

/* Copy n_pages pages from host memory into the pool: page i of host_src
 * (pages of 16*page_width elements, page-major, element type of the pool)
 * goes to pool page pages_host[i] (host array).  Runs of consecutive page
 * ids are copied with one transfer each, asynchronously on `stream` (a
 * hipStream_t; NULL = default stream).  For the copy to overlap kernels on
 * other streams host_src must be pinned (allocated with hipHostMalloc, e.g.
 * a torch tensor made with pin_memory=True).  The caller keeps host_src
 * alive until the stream has passed the copy.  Errors (before anything is
 * enqueued): INVALID_ARG, UNSUPPORTED (pool), PAGE_RANGE (a page id outside
 * the pool), HIP. */
lora_status_t lora_upload_pages(const lora_pool_t* pool, const void* host_src, const int32_t* pages_host,
                                int32_t n_pages, void* stream);

#ifdef __cplusplus
}
#endif
