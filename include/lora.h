/*
 * lora.h -- C ABI of liblora.so, the MI355X (gfx950) multi-LoRA adapter
 * branch over a paged pool of heterogeneous-rank adapters.
 *
 * Sources (the three web pages this library follows):
 *   [MLSP] "Multi-LoRA Serving in Production: Architecture, Dynamic Adapter
 *          Swapping, and GPU Memory Management" (llms.blog)
 *   [MLSA] "Multi-LoRA Serving Architecture: Serving Hundreds of Fine-Tuned
 *          Adapters on One GPU with vLLM and S-LoRA (2026)"
 *   [LAST] "LoRA Adapters at Serve Time with vLLM Multi-LoRA"
 *
 * What the library computes, for every token t of a mixed batch whose
 * adapter is a = ids[t] (the adapted-layer equation of [MLSP] "The
 * Mathematical Anatomy of Heterogeneous Batches"):
 *
 *     Y[t] = Y_base[t] + (alpha_a / r_a) * (X[t] A_a) B_a
 *
 * A_a is d_in x r_a and B_a is r_a x d_out.  The base product X W0 is not
 * computed here: the caller passes it as Y_base.  A_a B_a is never formed
 * ([LAST] "Architecture of Multi-LoRA in vLLM"), each adapter is read at its
 * own rank with no padding to the largest rank in the batch ([MLSP] "Multi-
 * Size Batched Gather Kernels (MBGMV and MBGMM)"), and the weights are read
 * straight from a pool of fixed-size pages through page tables ([MLSP]
 * "Unified Paging Architecture"; [MLSA] "S-LoRA unified paging").
 *
 * General rules
 *  - Pointers are device pointers unless a comment says "host".  The caller
 *    owns every buffer; the library allocates no memory and keeps no state
 *    between calls except cached device properties (reentrant).
 *  - Every call enqueues asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream) and never synchronises the device.
 *  - Host-side argument checks run before anything is enqueued; on error the
 *    call returns a negative status and enqueues nothing.  Data-dependent
 *    conditions found on the device never abort: tokens with bad ids or
 *    ranks are counted (lora_segments_t.counts) and keep Y_base; a page id
 *    outside the pool reads as zero weights and sets LORA_FLAG_PAGE_RANGE
 *    in the counters' flag word.
 *  - No exception crosses this interface.
 *
 * Element types: LORA_DTYPE_BF16 -> X, Y_base, Y and the pool hold bf16;
 * LORA_DTYPE_F32 -> all fp32 (validation mode).  Rank-r intermediates,
 * alpha and every accumulation are fp32; Y is Y_base + s*acc computed in
 * fp32 and rounded once (round to nearest even) to the element type.
 */
#ifndef LORA_H
#define LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lora_status_t;
#define LORA_OK 0
#define LORA_ERR_INVALID_ARG (-1) /* null pointer, negative size, bad stride */
#define LORA_ERR_RANK (-2)        /* a rank outside [1, LORA_MAX_RANK] (validator) */
#define LORA_ERR_PAGE_RANGE (-3)  /* page id outside the pool (validator) */
#define LORA_ERR_WORKSPACE (-4)   /* workspace or segment buffer too small */
#define LORA_ERR_HIP (-5)         /* a HIP runtime call or kernel launch failed */
#define LORA_ERR_UNSUPPORTED (-6) /* unknown dtype, page geometry, batch past the size limits */
#define LORA_ERR_ALIGNMENT (-7)   /* pointer or leading dimension not 16-byte aligned */
#define LORA_ERR_POOL_FULL (-8)   /* too few evictable pages in the pool (lora_pool.h) */

#define LORA_DTYPE_F32 0
#define LORA_DTYPE_BF16 1

#define LORA_PAGE_ROWS 16    /* ranks per page ("16-row pages") */
#define LORA_MAX_RANK 128
#define LORA_KSLICE 512      /* input columns per shrink partial sum */
#define LORA_MAX_ADAPTERS (1 << 20)
/* Size limits of one call (32-bit indices inside the kernels): T tokens with
 * T * LORA_MAX_RANK < 2^31, and per launch group of up to 16 projections at
 * most LORA_MAX_LAUNCH_ITEMS work items, bounded on the host by
 *   sum over the group of ceil(d_in/512) * (21 T + 2)          (shrink)
 *   sum over the group of ceil(d_out/cols) * (6 T + 2)         (expand)
 * with cols = 512 (bf16) or 256 (fp32).  Past either limit a call returns
 * LORA_ERR_UNSUPPORTED before any device work; split the batch or pass fewer
 * projections per call. */
#define LORA_MAX_TOKENS ((1 << 24) - 1)
#define LORA_MAX_LAUNCH_ITEMS (1 << 30)

/* Adapter set: one rank and one alpha per adapter, shared by every layer and
 * projection (each sequence's adapter has its own rank r_i, [MLSP]
 * "Mathematical Anatomy").  rank[] and alpha[] are device arrays of
 * num_adapters entries. */
typedef struct {
  const int32_t* rank;
  const float* alpha;
  int32_t num_adapters;
} lora_adapters_t;

/* The physical page pool ([MLSP] "Unified Paging Architecture": fixed-size
 * pages; adapter weights sliced along their rank dimension).  Page p is the
 * 16 x page_width block of elements starting at base + p*16*page_width.
 * base must be 16-byte aligned; page_width a power of two in [64, 65536]. */
typedef struct {
  void* base;
  int32_t num_pages;
  int32_t page_width;
  int32_t dtype; /* LORA_DTYPE_* */
} lora_pool_t;

/* One adapted projection (one layer's q_proj, say) of the batch.
 *
 * X      : [T][ldx]  row-major activations, ldx >= d_in
 * Y_base : [T][ldyb] base output X W0, ldyb >= d_out
 * Y      : [T][ldy]  output; may alias Y_base (then ldy must equal ldyb)
 * d_in, d_out : multiples of 8; ldx, ldyb, ldy multiples of 8 elements;
 *               X, Y_base, Y 16-byte aligned.
 *
 * Page tables (CSR over adapters, int32 device arrays), in the orientation of
 * [MLSA] "Context and Background" (A is r x d_in, B is d_out x r), sliced into
 * 16-rank groups g and page_width-wide blocks c of the feature dimension:
 *   A: page a_pages[a_indptr[a] + g*ceil(d_in/PW) + c] holds ranks 16g..16g+15
 *      (rows) x inputs c*PW..c*PW+PW-1 (columns): element (rank k, input i)
 *      at in-page offset (k-16g)*PW + (i-c*PW).
 *   B: page b_pages[b_indptr[a] + g*ceil(d_out/PW) + c] holds outputs
 *      c*PW..c*PW+PW-1 x ranks 16g..16g+15 as two halves of 8 ranks each:
 *      element (output j, rank k) at in-page offset
 *      h*8*PW + (j-c*PW)*8 + (k-16g-8h), h = (k-16g)/8.  The 8 ranks of an
 *      output column in one half are contiguous (16 bytes in bf16), and a
 *      rank group with at most 8 ranks uses only the first half.
 * Adapter a owns ceil(r_a/16)*ceil(d/PW) slots of each table.  Page rows or
 * columns beyond r_a or d are never read. */
typedef struct {
  const void* X;
  int64_t ldx;
  const void* Y_base;
  int64_t ldyb;
  void* Y;
  int64_t ldy;
  int32_t d_in;
  int32_t d_out;
  const int32_t* a_indptr;
  const int32_t* a_pages;
  const int32_t* b_indptr;
  const int32_t* b_pages;
} lora_proj_t;

/* Segments: the batch's tokens grouped by adapter ([MLSP] "Segmented Gather
 * Matrix-Vector Multiplication (SGMV)": requests grouped by target adapter),
 * plus the work plan the kernels walk.  All arrays are device memory carved
 * from one caller buffer by lora_segments_init (host fields T and
 * num_adapters record the capacity).  S_max = min(T, num_adapters).
 *   perm[T]               grouped valid tokens (ascending token index inside a
 *                         group, groups in ascending adapter id), then the
 *                         tokens that use no adapter, ascending
 *   seg_indptr[S_max+1]   token range of segment s in perm
 *   seg_adapter[S_max]    adapter of segment s
 *   v_indptr[S_max+1]     offset of segment s in the ragged rank-r
 *                         intermediate v: v[v_indptr[s] + i*r + k]
 *   plan                  the work plan the kernels walk (internal layout,
 *                         sized for the capacity (T, num_adapters))
 *   counts[16]            {S, n_invalid, T_valid, V_total, internal
 *                         work-plan totals, device error flags (index 8),
 *                         the built token count (9), a check word (10)}
 * A token is valid when 0 <= ids[t] < num_adapters and its adapter's rank is
 * in [1, 128].  ids[t] == -1 marks a base-model token ([MLSA] "What vLLM
 * actually gives you": base-model requests share the server); other invalid
 * tokens are counted in n_invalid.  Neither kind gets an adapter term. */
typedef struct {
  int32_t T;
  int32_t num_adapters;
  int32_t* perm;
  int32_t* seg_indptr;
  int32_t* seg_adapter;
  int32_t* v_indptr;
  int32_t* plan;
  int32_t* counts;
} lora_segments_t;

#define LORA_COUNT_S 0
#define LORA_COUNT_INVALID 1
#define LORA_COUNT_T_VALID 2
#define LORA_COUNT_V_TOTAL 3
#define LORA_COUNT_FLAGS 8
#define LORA_COUNT_T 9       /* the token count the segments were built for */
#define LORA_FLAG_PAGE_RANGE 1 /* a page id outside the pool was skipped (read as 0) */
/* The segment buffer was not walked: never built, built for another token
 * count than the call's T (lora_apply) or for more than its capacity, or its
 * counters exceed the capacity it was laid out for.  The launch wrote
 * nothing. */
#define LORA_FLAG_SEGMENTS 2
/* The single-launch kernel of lora_apply gave up waiting for its shrink
 * phase (its grid could not run all at once: another kernel held compute
 * units for longer than the wait's bound, lora_set_wait_limit).  Y of that
 * call is invalid; the segment buffer stays usable for later calls. */
#define LORA_FLAG_SYNC 4

/* Bytes of the device buffer that holds segments for T tokens and
 * num_adapters adapters. */
size_t lora_segments_size(int32_t T, int32_t num_adapters);  /* 0 outside the limits */

/* Fill *out with pointers carved from `buf` (device, `bytes` long, 16-byte
 * aligned).  Enqueues nothing.  Errors: INVALID_ARG, ALIGNMENT, WORKSPACE,
 * UNSUPPORTED (T > LORA_MAX_TOKENS). */
lora_status_t lora_segments_init(void* buf, size_t bytes, int32_t T, int32_t num_adapters,
                                 lora_segments_t* out);

/* Workspace bytes for lora_build_segments and lora_apply with n_projs
 * projections whose largest input width is max_d_in (0 outside the limits). */
size_t lora_workspace_size(int32_t T, int32_t num_adapters, int32_t n_projs, int32_t max_d_in);

/* Number of shrink partial slices for an input width: ceil(d_in / 512). */
int32_t lora_v_slices(int32_t d_in);

/* Group the batch's tokens by adapter and build the work plan (a
 * deterministic stable counting sort; [MLSP] "Segmented Gather Matrix-Vector
 * Multiplication (SGMV)": requests grouped by their adapter).  ids: device
 * [T].  segs: laid out by lora_segments_init with a capacity of at least
 * (T, adapters->num_adapters); a buffer laid out for a larger batch serves
 * any smaller one (the built T is recorded in counts[LORA_COUNT_T]).  The
 * result depends only on ids and ranks; build once per batch and reuse for
 * every layer and projection.  ws: device, >= lora_workspace_size(T, N, 0, 0)
 * bytes.  Errors: INVALID_ARG, WORKSPACE (capacity or workspace too small),
 * UNSUPPORTED, HIP. */
lora_status_t lora_build_segments(const int32_t* ids, int32_t T, const lora_adapters_t* adapters,
                                  const lora_segments_t* segs, void* ws, size_t ws_bytes,
                                  void* stream);

/* Shrink ([MLSP] SGMV: v_i = x_i A_i, the rank-r intermediate) for n_projs
 * projections of one batch (projs: host array), one kernel launch per group
 * of up to 16 projections -- the first launch of lora_apply.  v: host array
 * of n_projs device pointers; v[i] is fp32 [lora_v_slices(d_in_i)][v_stride]
 * and its slice q holds the partial sum over inputs q*512 ..
 * min((q+1)*512, d_in)-1 in the ragged layout of v_indptr; v = the sum of
 * the slices in ascending q.  v_stride >= T*128.
 * Errors: INVALID_ARG, ALIGNMENT, UNSUPPORTED, HIP. */
lora_status_t lora_shrink(const lora_proj_t* projs, int32_t n_projs, const lora_adapters_t* adapters,
                          const lora_segments_t* segs, const lora_pool_t* pool, float* const* v,
                          int64_t v_stride, void* stream);

/* Expand ([MLSP] SGMV: y_i = v_i B_i scaled by alpha_i/r_i and added to the
 * base output) for n_projs projections -- the second launch of lora_apply.
 * v as written by lora_shrink.  v_slices: 0 -> lora_v_slices(d_in_i) slices
 * for projection i (what lora_shrink wrote); k >= 1 -> k slices for every
 * projection (k = 1: v given whole).  Rows of tokens without an adapter
 * receive Y_base.  With at least three MBGMM expand items per work-group of
 * the grid (prefill batches) the launch hands out its items through queues
 * in the segment buffer, which its last work-groups put back to zero: calls
 * that share one segment buffer must not run concurrently.  Errors as
 * lora_shrink. */
lora_status_t lora_expand(const lora_proj_t* projs, int32_t n_projs, const lora_adapters_t* adapters,
                          const lora_segments_t* segs, const lora_pool_t* pool, const float* const* v,
                          int32_t v_slices, int64_t v_stride, void* stream);

/* The whole adapter branch for n_projs projections of one batch: for every
 * token, Y = Y_base + (alpha/r) (X A) B, the adapted-layer equation of
 * [MLSP] "The Mathematical Anatomy of Heterogeneous Batches", computed as
 * the gather / shrink / expand sequence of [MLSP] "Segmented Gather
 * Matrix-Vector Multiplication (SGMV)" over segments of tokens that share an
 * adapter, with weights read through the page tables ([MLSP] "Unified Paging
 * Architecture").  Per group of up to 16 projections either one kernel
 * launch (the fused operations of [MLSP] "Custom CUDA Kernels: SGMV and
 * MBGMV": its waves write the shrink partial sums, wait once for the whole
 * grid's, and run the expand) or the two launches of lora_shrink and
 * lora_expand -- see lora_set_launch_mode; the arithmetic, and Y, are the
 * same bit for bit.  The single launch keeps its wait's bookkeeping in the
 * segment buffer, and so does the expand launch of a large batch (per-XCD
 * item queues, from three MBGMM expand items per work-group of its grid),
 * so calls that share one segment buffer must not run concurrently (issue
 * them on one stream).
 *   ids != NULL, segs != NULL : build segments into *segs, then apply
 *   ids != NULL, segs == NULL : build segments inside the workspace
 *   ids == NULL, segs != NULL : reuse prebuilt segments (built by
 *                               lora_build_segments or an earlier call)
 * T = 0 (the empty batch) needs neither ids nor segs: its segments are
 * always built (into the workspace when segs is NULL), all counts zero, and
 * nothing else is written.  Descriptor pointers must still
 * be valid (non-null, aligned).
 * projs: host array of n_projs descriptors.  T: the batch's tokens, at most
 * the capacity segs->T.  Prebuilt segments must have been built for exactly
 * T tokens; if they were not (or were never built) the kernels compute
 * nothing and set LORA_FLAG_SEGMENTS in segs->counts[LORA_COUNT_FLAGS].
 * ws: device workspace of lora_workspace_size(T, N, n_projs, max d_in) bytes.
 * Errors: INVALID_ARG, ALIGNMENT, UNSUPPORTED, WORKSPACE, HIP. */
lora_status_t lora_apply(const int32_t* ids, const lora_segments_t* segs, int32_t T,
                         const lora_proj_t* projs, int32_t n_projs,
                         const lora_adapters_t* adapters, const lora_pool_t* pool, void* ws,
                         size_t ws_bytes, void* stream);

/* lora_apply without a workspace argument, for callers that cannot allocate
 * device memory when they call (code under HIP graph capture, serving loops
 * that must not allocate, harnesses that forbid it).  The workspace is a
 * fixed array of LORA_NOALLOC_SCRATCH_BYTES owned by the library: one copy
 * per GPU, allocated when the library's code is loaded on that GPU and held
 * until the process ends.  Arguments, segment handling and results are those
 * of lora_apply; nothing is allocated by the call.
 * Every call on one GPU uses that GPU's array, and the array keeps the last
 * call's contents (nothing in it has to start at zero): calls that may
 * overlap on one GPU (different streams, or different host threads without
 * ordering) race on it and must not be issued.
 * Errors: those of lora_apply, and WORKSPACE when lora_workspace_size(T, N,
 * n_projs, max d_in) exceeds LORA_NOALLOC_SCRATCH_BYTES (a decode batch fits:
 * 1024 tokens over 1000 adapters with three 4096-wide or one 11008-wide
 * projection per call need 12.7 MiB and 11.7 MiB). */
#define LORA_NOALLOC_SCRATCH_BYTES (64u << 20)
lora_status_t lora_apply_noalloc(const int32_t* ids, const lora_segments_t* segs, int32_t T,
                                 const lora_proj_t* projs, int32_t n_projs,
                                 const lora_adapters_t* adapters, const lora_pool_t* pool,
                                 void* stream);

/* How lora_apply launches a group (process-wide).  LORA_LAUNCH_SINGLE: one
 * launch (shrink phase, wait, expand phase), which needs its grid resident
 * at once -- a kernel on another stream holding compute units for longer
 * than the wait's bound makes the call give up (LORA_FLAG_SYNC).
 * LORA_LAUNCH_TWO: a shrink launch then an expand launch, no such
 * requirement (what a caller running other kernels concurrently should
 * use).  LORA_LAUNCH_AUTO (default): one launch for batches of at most 2048
 * tokens, two above; both give bit-identical Y.  Errors: INVALID_ARG. */
#define LORA_LAUNCH_AUTO 0
#define LORA_LAUNCH_SINGLE 1
#define LORA_LAUNCH_TWO 2
lora_status_t lora_set_launch_mode(int32_t mode);

/* Bound on the internal wait of lora_apply's single-launch kernel: its
 * expand phase waits until every work-group of the grid has written its
 * shrink partial sums, which needs the whole grid resident at once (the grid
 * is sized from the kernel's occupancy).  Process-wide; for diagnostics and
 * tests.  ns > 0 sets the bound, 0 restores the default (50 ms), ns < 0
 * makes every such wait give up after |ns| ns (exercises the give-up path:
 * LORA_FLAG_SYNC, no hang). */
void lora_set_wait_limit(int64_t ns);

/* Host-side check of page tables (all arguments host copies): every adapter
 * owns exactly ceil(r/16)*ceil(d/PW) slots and every page id lies in
 * [0, num_pages) ([MLSA] "Trade-offs, Gotchas": validate shape and rank
 * before admission).  Returns OK, RANK, PAGE_RANGE or INVALID_ARG. */
lora_status_t lora_validate_tables(int32_t num_adapters, const int32_t* rank_host, int32_t d_in,
                                   int32_t d_out, int32_t page_width, int32_t num_pages,
                                   const int32_t* a_indptr_host, const int32_t* a_pages_host,
                                   const int32_t* b_indptr_host, const int32_t* b_pages_host);

/* Static string for a status code. */
const char* lora_status_string(lora_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* LORA_H */
