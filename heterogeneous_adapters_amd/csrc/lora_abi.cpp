// C ABI of liblora.so: argument checks, buffer carving, work-group sizing and
// kernel launches.  Every check that depends only on host-visible arguments
// runs before the first HIP call, so invalid calls return an error code
// without touching the device.
//
// Sources:
//   [MLSP] "Multi-LoRA Serving in Production: Architecture, Dynamic Adapter
//          Swapping, and GPU Memory Management"
//   [MLSA] "Multi-LoRA Serving Architecture: Serving Hundreds of Fine-Tuned
//          Adapters on One GPU with vLLM and S-LoRA (2026)"
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "lora.h"
#include "lora_kernels.h"
#include "lora_plan.h"

using namespace lora;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int smax_of(int32_t T, int32_t N) { return std::max(0, std::min(T, N)); }

struct SegSizes {
  size_t perm, seg_indptr, seg_adapter, v_indptr, plan, counts, total;
};

SegSizes seg_sizes(int32_t T, int32_t N) {
  const size_t sm = (size_t)smax_of(T, N);
  SegSizes z;
  z.perm = align_up(sizeof(int32_t) * std::max<int32_t>(T, 1));
  z.seg_indptr = align_up(sizeof(int32_t) * (sm + 1));
  z.seg_adapter = align_up(sizeof(int32_t) * std::max<size_t>(sm, 1));
  z.v_indptr = z.seg_indptr;
  z.plan = align_up(sizeof(int32_t) * (size_t)plan_layout(T, N).total);
  z.counts = align_up(sizeof(int32_t) * kNumCounts);
  z.total = z.perm + z.seg_indptr + z.seg_adapter + z.v_indptr + z.plan + z.counts;
  return z;
}

// Pointers of the plan area of a segment buffer laid out for (T, N).
struct PlanPtrs {
  int32_t *seg_desc, *shr_m, *shr_v, *exp_m, *exp_v, *sync;
};
PlanPtrs plan_ptrs(const lora_segments_t* s) {
  const PlanLayout L = plan_layout(s->T, s->num_adapters);
  return PlanPtrs{s->plan + L.seg_desc, s->plan + L.shrink_mfma, s->plan + L.shrink_valu, s->plan + L.expand_mfma,
                  s->plan + L.expand_valu, s->plan + L.sync};
}

size_t hist_bytes(int32_t T, int32_t N) {
  const size_t nchunk = (size_t)std::max(1, ceil_div_i(std::max(T, 0), kSegChunk));
  return align_up(nchunk * (size_t)(N + 2) * sizeof(int32_t));
}

size_t v_bytes_per_proj(int32_t T, int32_t d_in) {
  return align_up((size_t)lora_v_slices(d_in) * (size_t)std::max(T, 1) * LORA_MAX_RANK * sizeof(float));
}

lora_status_t check_adapters(const lora_adapters_t* ad) {
  if (!ad || !ad->rank || !ad->alpha) return LORA_ERR_INVALID_ARG;
  if (ad->num_adapters < 1 || ad->num_adapters > LORA_MAX_ADAPTERS) return LORA_ERR_INVALID_ARG;
  return LORA_OK;
}

lora_status_t check_segs(const lora_segments_t* s) {
  if (!s || !s->perm || !s->seg_indptr || !s->seg_adapter || !s->v_indptr || !s->plan || !s->counts)
    return LORA_ERR_INVALID_ARG;
  if (s->T < 0 || s->num_adapters < 1) return LORA_ERR_INVALID_ARG;
  return LORA_OK;
}

lora_status_t check_pool(const lora_pool_t* pool) {
  if (!pool || !pool->base || pool->num_pages < 1) return LORA_ERR_INVALID_ARG;
  if (pool->dtype != LORA_DTYPE_BF16 && pool->dtype != LORA_DTYPE_F32) return LORA_ERR_UNSUPPORTED;
  const int pw = pool->page_width;
  if (pw < 64 || pw > 65536 || (pw & (pw - 1)) != 0) return LORA_ERR_UNSUPPORTED;
  if (!aligned16(pool->base)) return LORA_ERR_ALIGNMENT;
  return LORA_OK;
}

lora_status_t check_proj(const lora_proj_t* p) {
  if (!p || !p->X || !p->Y_base || !p->Y) return LORA_ERR_INVALID_ARG;
  if (!p->a_indptr || !p->a_pages || !p->b_indptr || !p->b_pages) return LORA_ERR_INVALID_ARG;
  if (p->d_in <= 0 || p->d_out <= 0 || (p->d_in % 8) != 0 || (p->d_out % 8) != 0) return LORA_ERR_INVALID_ARG;
  if (p->ldx < p->d_in || p->ldyb < p->d_out || p->ldy < p->d_out) return LORA_ERR_INVALID_ARG;
  if (p->Y == p->Y_base && p->ldy != p->ldyb) return LORA_ERR_INVALID_ARG;
  if ((p->ldx % 8) != 0 || (p->ldyb % 8) != 0 || (p->ldy % 8) != 0) return LORA_ERR_ALIGNMENT;
  if (!aligned16(p->X) || !aligned16(p->Y_base) || !aligned16(p->Y)) return LORA_ERR_ALIGNMENT;
  return LORA_OK;
}

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Per-device launch geometry, cached on first use (the only state kept).
struct DeviceInfo {
  std::atomic<int> ready{0};
  int cus = 0;
  int occ_shrink[2] = {0, 0};
  int occ_expand[2] = {0, 0};
  int occ_apply[2] = {0, 0};
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];

lora_status_t device_info(const DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LORA_ERR_HIP;
  DeviceInfo& d = g_dev[dev];
  if (!d.ready.load(std::memory_order_acquire)) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return LORA_ERR_HIP;
    int s0 = 0, e0 = 0, a0 = 0, s1 = 0, e1 = 0, a1 = 0;
    if (occupancy(LORA_DTYPE_F32, &s0, &e0, &a0) != hipSuccess) return LORA_ERR_HIP;
    if (occupancy(LORA_DTYPE_BF16, &s1, &e1, &a1) != hipSuccess) return LORA_ERR_HIP;
    d.cus = std::max(cus, 1);
    d.occ_shrink[0] = std::max(s0, 1);
    d.occ_expand[0] = std::max(e0, 1);
    d.occ_apply[0] = std::max(a0, 1);
    d.occ_shrink[1] = std::max(s1, 1);
    d.occ_expand[1] = std::max(e1, 1);
    d.occ_apply[1] = std::max(a1, 1);
    d.ready.store(1, std::memory_order_release);
  }
  *out = &d;
  return LORA_OK;
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Bound of the apply kernel's phase wait (lora_set_wait_limit): ns > 0 a
// bound, 0 the default, < 0 a forced give-up after |ns|.
constexpr int64_t kDefaultWaitNs = 50'000'000;
std::atomic<int64_t> g_wait_ns{0};

// Launch mode of lora_apply (lora_set_launch_mode).  Automatic: one launch
// per group for batches of at most kSingleLaunchMaxTokens tokens, two above.
// Measured on MI355X: one launch is 4 % faster on a 256-token batch and at
// parity on 512 and 1024-token decode batches, but 3-5 % slower on a mixed
// 2495-token batch and a 38,781-token prefill, whose shrink phase runs
// faster at the shrink kernel's own occupancy.
constexpr int32_t kSingleLaunchMaxTokens = 2048;
std::atomic<int32_t> g_launch_mode{LORA_LAUNCH_AUTO};
bool single_launch(int32_t T) {
  const int32_t m = g_launch_mode.load(std::memory_order_relaxed);
  return m == LORA_LAUNCH_SINGLE || (m == LORA_LAUNCH_AUTO && T <= kSingleLaunchMaxTokens);
}

void wait_params(KArgs& K) {
  const int64_t ns = g_wait_ns.load(std::memory_order_relaxed);
  const int64_t bound = ns == 0 ? kDefaultWaitNs : (ns > 0 ? ns : -ns);
  K.wait_ticks = std::max<int64_t>(bound / 10, 1);  // s_memrealtime counts at 100 MHz
  K.wait_bias = ns < 0 ? 1 : 0;
}

KProj make_kproj(const lora_proj_t& p, float* v, int nv, int dtype) {
  KProj k;
  memset(&k, 0, sizeof k);
  const bool bf16 = dtype == LORA_DTYPE_BF16;
  k.X = p.X;
  k.Yb = p.Y_base;
  k.Y = p.Y;
  k.v = v;
  k.a_indptr = p.a_indptr;
  k.a_pages = p.a_pages;
  k.b_indptr = p.b_indptr;
  k.b_pages = p.b_pages;
  k.ldx = p.ldx;
  k.ldyb = p.ldyb;
  k.ldy = p.ldy;
  k.d_in = p.d_in;
  k.d_out = p.d_out;
  k.nq = lora_v_slices(p.d_in);
  k.njs = ceil_div_i(p.d_out, expand_cols(bf16));
  k.nv = nv;
  return k;
}

// T: the call's token count (lora_apply: the segments must have been built
// for exactly T tokens), or -1 for the split entry points (any built T up to
// the buffer's capacity).
void fill_common(KArgs& K, const lora_segments_t* s, const lora_pool_t* pool, int64_t v_stride, int32_t T) {
  const PlanPtrs pp = plan_ptrs(s);
  const PlanLayout L = plan_layout(s->T, s->num_adapters);
  K.perm = s->perm;
  K.seg_desc = reinterpret_cast<const int4*>(pp.seg_desc);
  K.shr_item_m = pp.shr_m;
  K.shr_item_v = pp.shr_v;
  K.exp_item_m = pp.exp_m;
  K.exp_item_v = pp.exp_v;
  K.counts = s->counts;
  K.pool = pool->base;
  K.v_stride = v_stride;
  K.num_pages = pool->num_pages;
  K.pw_log2 = log2_exact(pool->page_width);
  K.T = T >= 0 ? T : s->T;
  K.t_exact = T >= 0;
  K.s_cap = (int32_t)L.s_cap;
  K.cap_sm = (int32_t)L.cap_shrink_mfma;
  K.cap_sv = (int32_t)L.cap_shrink_valu;
  K.cap_em = (int32_t)L.cap_expand_mfma;
  K.cap_ev = (int32_t)L.cap_expand_valu;
  K.sync = pp.sync;
  wait_params(K);
}

// Projections of one launch that read the same activations (q/k/v, gate/up
// of a transformer block): the shrink then walks their items side by side so
// the shared X rows are re-read from L2 rather than HBM.
void mark_shared_x(KArgs& K) {
  K.xshare = K.np > 1;
  for (int i = 1; i < K.np; ++i)
    if (K.p[i].X != K.p[0].X || K.p[i].ldx != K.p[0].ldx || K.p[i].d_in != K.p[0].d_in) K.xshare = 0;
}

// The size limits of every launch group of a call, checked before the call
// enqueues anything (bounds as in run()).
lora_status_t check_limits(const lora_proj_t* projs, int32_t n_projs, int32_t T, int dtype) {
  if (T > LORA_MAX_TOKENS) return LORA_ERR_UNSUPPORTED;
  const int cols = expand_cols(dtype == LORA_DTYPE_BF16);
  for (int base = 0; base < n_projs; base += kProjsPerLaunch) {
    int64_t bs = 0, be = 0;
    for (int i = base; i < std::min(n_projs, base + kProjsPerLaunch); ++i) {
      bs += (int64_t)lora_v_slices(projs[i].d_in) * (21LL * T + 2);
      be += (int64_t)ceil_div_i(projs[i].d_out, cols) * (6LL * T + 2);
    }
    if (bs > LORA_MAX_LAUNCH_ITEMS || be > LORA_MAX_LAUNCH_ITEMS) return LORA_ERR_UNSUPPORTED;
  }
  return LORA_OK;
}

lora_status_t run(const KArgs& K, int dtype, bool do_shrink, bool do_expand, hipStream_t stream) {
  if (K.T > LORA_MAX_TOKENS) return LORA_ERR_UNSUPPORTED;
  // upper bounds of the launch's item totals (MBGMM + MBGMV per slice or
  // column block); the kernels index items with 32-bit ints
  int64_t bs = 0, be = 0;
  for (int p = 0; p < K.np; ++p) {
    bs += (int64_t)K.p[p].nq * (21LL * K.T + 2);
    be += (int64_t)K.p[p].njs * (6LL * K.T + 2);
  }
  if ((do_shrink && bs > LORA_MAX_LAUNCH_ITEMS) || (do_expand && be > LORA_MAX_LAUNCH_ITEMS))
    return LORA_ERR_UNSUPPORTED;
  const DeviceInfo* d = nullptr;
  if (lora_status_t st = device_info(&d)) return st;
  const int di = dtype == LORA_DTYPE_BF16 ? 1 : 0;
  if (do_shrink && do_expand && single_launch(K.T))  // one launch; its grid is resident at once
    return launch_apply(K, dtype, launch_grid(d->cus * d->occ_apply[di], ceil_div64(std::max(bs, be), kWaves)),
                        stream) == hipSuccess
               ? LORA_OK
               : LORA_ERR_HIP;
  // items are per wave: kWaves items per work-group
  if (do_shrink && launch_shrink(K, dtype, launch_grid(d->cus * d->occ_shrink[di], ceil_div64(bs, kWaves)), stream) !=
                       hipSuccess)
    return LORA_ERR_HIP;
  if (do_expand && launch_expand(K, dtype, launch_grid(d->cus * d->occ_expand[di], ceil_div64(be, kWaves)), stream) !=
                       hipSuccess)
    return LORA_ERR_HIP;
  return LORA_OK;
}

lora_status_t build_into(const int32_t* ids, int32_t T, const lora_adapters_t* ad, const lora_segments_t* segs,
                         int32_t* hist, hipStream_t stream) {
  const PlanPtrs pp = plan_ptrs(segs);
  SegOut o{segs->perm, segs->seg_indptr, segs->seg_adapter, segs->v_indptr, pp.seg_desc, pp.shr_m,
           pp.shr_v,   pp.exp_m,         pp.exp_v,          segs->counts,   pp.sync};
  return launch_build_segments(ids, T, ad->num_adapters, ad->rank, ad->alpha, hist, o, stream) == hipSuccess
             ? LORA_OK
             : LORA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* lora_status_string(lora_status_t s) {
  switch (s) {
    case LORA_OK: return "ok";
    case LORA_ERR_INVALID_ARG: return "invalid argument";
    case LORA_ERR_RANK: return "rank outside [1, 128]";
    case LORA_ERR_PAGE_RANGE: return "page id outside the pool";
    case LORA_ERR_WORKSPACE: return "workspace or segment buffer too small";
    case LORA_ERR_HIP: return "HIP runtime error";
    case LORA_ERR_UNSUPPORTED: return "unsupported dtype, page geometry or projection count";
    case LORA_ERR_ALIGNMENT: return "pointer or leading dimension not 16-byte aligned";
    case LORA_ERR_POOL_FULL: return "too few evictable pages in the pool";
    default: return "unknown status";
  }
}

void lora_set_wait_limit(int64_t ns) { g_wait_ns.store(ns, std::memory_order_relaxed); }

lora_status_t lora_set_launch_mode(int32_t mode) {
  if (mode != LORA_LAUNCH_AUTO && mode != LORA_LAUNCH_SINGLE && mode != LORA_LAUNCH_TWO) return LORA_ERR_INVALID_ARG;
  g_launch_mode.store(mode, std::memory_order_relaxed);
  return LORA_OK;
}

int32_t lora_v_slices(int32_t d_in) { return d_in <= 0 ? 0 : ceil_div_i(d_in, LORA_KSLICE); }

size_t lora_segments_size(int32_t T, int32_t num_adapters) {
  if (T < 0 || T > LORA_MAX_TOKENS || num_adapters < 1 || num_adapters > LORA_MAX_ADAPTERS) return 0;
  return seg_sizes(T, num_adapters).total;
}

lora_status_t lora_segments_init(void* buf, size_t bytes, int32_t T, int32_t num_adapters, lora_segments_t* out) {
  if (!buf || !out || T < 0 || num_adapters < 1 || num_adapters > LORA_MAX_ADAPTERS) return LORA_ERR_INVALID_ARG;
  if (T > LORA_MAX_TOKENS) return LORA_ERR_UNSUPPORTED;
  if (!aligned16(buf)) return LORA_ERR_ALIGNMENT;
  const SegSizes z = seg_sizes(T, num_adapters);
  if (bytes < z.total) return LORA_ERR_WORKSPACE;
  char* p = static_cast<char*>(buf);
  out->T = T;
  out->num_adapters = num_adapters;
  out->perm = reinterpret_cast<int32_t*>(p); p += z.perm;
  out->seg_indptr = reinterpret_cast<int32_t*>(p); p += z.seg_indptr;
  out->seg_adapter = reinterpret_cast<int32_t*>(p); p += z.seg_adapter;
  out->v_indptr = reinterpret_cast<int32_t*>(p); p += z.v_indptr;
  out->plan = reinterpret_cast<int32_t*>(p); p += z.plan;
  out->counts = reinterpret_cast<int32_t*>(p);
  return LORA_OK;
}

size_t lora_workspace_size(int32_t T, int32_t num_adapters, int32_t n_projs, int32_t max_d_in) {
  if (T < 0 || T > LORA_MAX_TOKENS || num_adapters < 1 || num_adapters > LORA_MAX_ADAPTERS || n_projs < 0 ||
      max_d_in < 0)
    return 0;
  return seg_sizes(T, num_adapters).total + hist_bytes(T, num_adapters) +
         (size_t)std::min(n_projs, kProjsPerLaunch) * v_bytes_per_proj(T, max_d_in);
}

lora_status_t lora_build_segments(const int32_t* ids, int32_t T, const lora_adapters_t* adapters,
                                  const lora_segments_t* segs, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || (T > 0 && !ids)) return LORA_ERR_INVALID_ARG;
  if (T > LORA_MAX_TOKENS) return LORA_ERR_UNSUPPORTED;
  if (lora_status_t st = check_adapters(adapters)) return st;
  if (lora_status_t st = check_segs(segs)) return st;
  if (T > segs->T || adapters->num_adapters > segs->num_adapters) return LORA_ERR_WORKSPACE;
  if (!ws) return LORA_ERR_INVALID_ARG;
  if (ws_bytes < hist_bytes(T, adapters->num_adapters)) return LORA_ERR_WORKSPACE;
  // the plan keeps the layout of the buffer's capacity (segs->T,
  // segs->num_adapters) whatever T is; the built T is recorded in counts[]
  return build_into(ids, T, adapters, segs, static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream));
}

// Shared body of lora_shrink / lora_expand: groups of up to kProjsPerLaunch
// projections per launch, the launch geometry of lora_apply.
static lora_status_t run_split(const lora_proj_t* projs, int32_t n_projs, const lora_adapters_t* adapters,
                               const lora_segments_t* segs, const lora_pool_t* pool, float* const* v,
                               int32_t v_slices, int64_t v_stride, bool shrink, void* stream) {
  if (n_projs < 0 || (n_projs > 0 && (!projs || !v))) return LORA_ERR_INVALID_ARG;
  if (lora_status_t st = check_adapters(adapters)) return st;
  if (lora_status_t st = check_segs(segs)) return st;
  if (lora_status_t st = check_pool(pool)) return st;
  if (v_slices < 0 || v_stride < (int64_t)segs->T * LORA_MAX_RANK) return LORA_ERR_INVALID_ARG;
  for (int i = 0; i < n_projs; ++i) {
    if (lora_status_t st = check_proj(&projs[i])) return st;
    if (!v[i]) return LORA_ERR_INVALID_ARG;
  }
  if (lora_status_t st = check_limits(projs, n_projs, segs->T, pool->dtype)) return st;
  for (int base = 0; base < n_projs; base += kProjsPerLaunch) {
    KArgs K;
    memset(&K, 0, sizeof K);
    fill_common(K, segs, pool, v_stride, -1);
    K.np = std::min(kProjsPerLaunch, n_projs - base);
    for (int i = 0; i < K.np; ++i) {
      const lora_proj_t& p = projs[base + i];
      const int nv = (shrink || v_slices == 0) ? lora_v_slices(p.d_in) : v_slices;
      K.p[i] = make_kproj(p, v[base + i], nv, pool->dtype);
    }
    mark_shared_x(K);
    if (lora_status_t e = run(K, pool->dtype, shrink, !shrink, static_cast<hipStream_t>(stream))) return e;
  }
  return LORA_OK;
}

lora_status_t lora_shrink(const lora_proj_t* projs, int32_t n_projs, const lora_adapters_t* adapters,
                          const lora_segments_t* segs, const lora_pool_t* pool, float* const* v, int64_t v_stride,
                          void* stream) {
  return run_split(projs, n_projs, adapters, segs, pool, v, 0, v_stride, true, stream);
}

lora_status_t lora_expand(const lora_proj_t* projs, int32_t n_projs, const lora_adapters_t* adapters,
                          const lora_segments_t* segs, const lora_pool_t* pool, const float* const* v,
                          int32_t v_slices, int64_t v_stride, void* stream) {
  return run_split(projs, n_projs, adapters, segs, pool, const_cast<float* const*>(v), v_slices, v_stride, false,
                   stream);
}

lora_status_t lora_apply(const int32_t* ids, const lora_segments_t* segs, int32_t T, const lora_proj_t* projs,
                         int32_t n_projs, const lora_adapters_t* adapters, const lora_pool_t* pool, void* ws,
                         size_t ws_bytes, void* stream) {
  if (T < 0 || n_projs < 0 || (n_projs > 0 && !projs)) return LORA_ERR_INVALID_ARG;
  if (T > 0 && !ids && !segs) return LORA_ERR_INVALID_ARG;
  if (T > LORA_MAX_TOKENS) return LORA_ERR_UNSUPPORTED;
  if (lora_status_t st = check_adapters(adapters)) return st;
  if (lora_status_t st = check_pool(pool)) return st;
  if (segs) {
    if (lora_status_t st = check_segs(segs)) return st;
    if (T > segs->T || adapters->num_adapters > segs->num_adapters) return LORA_ERR_INVALID_ARG;
  }
  int32_t max_d_in = 0;
  for (int i = 0; i < n_projs; ++i) {
    if (lora_status_t st = check_proj(&projs[i])) return st;
    max_d_in = std::max(max_d_in, projs[i].d_in);
  }
  if (lora_status_t st = check_limits(projs, n_projs, T, pool->dtype)) return st;
  if (!ws) return LORA_ERR_INVALID_ARG;
  if (ws_bytes < lora_workspace_size(T, adapters->num_adapters, n_projs, max_d_in)) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGNMENT;

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  lora_segments_t local;
  const lora_segments_t* S = segs;
  const size_t seg_total = seg_sizes(T, adapters->num_adapters).total;
  if (!segs) {
    lora_segments_init(w, seg_total, T, adapters->num_adapters, &local);
    S = &local;
  }
  char* hist = w + seg_total;
  char* vbase = hist + hist_bytes(T, adapters->num_adapters);
  // An empty batch is built whatever ids is (it needs none): a null ids
  // then cannot leave the kernels reading counts of a buffer never built.
  if (ids || T == 0) {
    if (lora_status_t e = build_into(ids, T, adapters, S, reinterpret_cast<int32_t*>(hist), st)) return e;
  }
  if (n_projs == 0) return LORA_OK;
  const size_t vpp = v_bytes_per_proj(T, max_d_in);
  const int64_t v_stride = (int64_t)std::max(T, 1) * LORA_MAX_RANK;
  for (int base = 0; base < n_projs; base += kProjsPerLaunch) {
    KArgs K;
    memset(&K, 0, sizeof K);
    fill_common(K, S, pool, v_stride, T);
    K.np = std::min(kProjsPerLaunch, n_projs - base);
    for (int i = 0; i < K.np; ++i) {
      float* v = reinterpret_cast<float*>(vbase + (size_t)i * vpp);
      K.p[i] = make_kproj(projs[base + i], v, lora_v_slices(projs[base + i].d_in), pool->dtype);
    }
    mark_shared_x(K);
    if (lora_status_t e = run(K, pool->dtype, true, true, st)) return e;
  }
  return LORA_OK;
}

lora_status_t lora_validate_tables(int32_t num_adapters, const int32_t* rank_host, int32_t d_in, int32_t d_out,
                                   int32_t page_width, int32_t num_pages, const int32_t* a_indptr_host,
                                   const int32_t* a_pages_host, const int32_t* b_indptr_host,
                                   const int32_t* b_pages_host) {
  if (num_adapters < 1 || !rank_host || !a_indptr_host || !a_pages_host || !b_indptr_host || !b_pages_host)
    return LORA_ERR_INVALID_ARG;
  if (d_in <= 0 || d_out <= 0 || page_width <= 0 || num_pages < 1) return LORA_ERR_INVALID_ARG;
  const int nci = ceil_div_i(d_in, page_width), nco = ceil_div_i(d_out, page_width);
  for (int a = 0; a < num_adapters; ++a) {
    const int r = rank_host[a];
    if (r < 1 || r > LORA_MAX_RANK) return LORA_ERR_RANK;
    const int G = rank_groups(r);
    if (a_indptr_host[a] < 0 || b_indptr_host[a] < 0) return LORA_ERR_INVALID_ARG;
    if (a_indptr_host[a + 1] - a_indptr_host[a] != G * nci) return LORA_ERR_INVALID_ARG;
    if (b_indptr_host[a + 1] - b_indptr_host[a] != G * nco) return LORA_ERR_INVALID_ARG;
    for (int i = a_indptr_host[a]; i < a_indptr_host[a + 1]; ++i)
      if (a_pages_host[i] < 0 || a_pages_host[i] >= num_pages) return LORA_ERR_PAGE_RANGE;
    for (int i = b_indptr_host[a]; i < b_indptr_host[a + 1]; ++i)
      if (b_pages_host[i] < 0 || b_pages_host[i] >= num_pages) return LORA_ERR_PAGE_RANGE;
  }
  return LORA_OK;
}

}  // extern "C"
