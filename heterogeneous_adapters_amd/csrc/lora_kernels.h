// Kernel argument blocks and launchers of liblora (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_plan.h"

namespace lora {

constexpr int kSegScanThreads = 1024;
// One projection as the kernels see it.
struct KProj {
  const void* X;
  const void* Yb;
  void* Y;
  float* v;                 // shrink output / expand input: [slices][v_stride] fp32
  const int32_t* a_indptr;
  const int32_t* a_pages;
  const int32_t* b_indptr;
  const int32_t* b_pages;
  int64_t ldx, ldyb, ldy;
  int32_t d_in, d_out;
  int32_t nq;     // shrink slices written: ceil(d_in / 512)
  int32_t njs;    // MBGMV expand column blocks: ceil(d_out / expand_cols)
  int32_t nv;     // v slices the expand sums
};

struct KArgs {
  KProj p[kProjsPerLaunch];
  const int32_t* perm;
  const int4* seg_desc;  // per segment: {a, r, t0, n}, {v_offset, shrink item0, expand item0, alpha bits}
  const int32_t* shr_item_m;
  const int32_t* shr_item_v;
  const int32_t* exp_item_m;
  const int32_t* exp_item_v;
  int32_t* counts;
  const void* pool;
  int64_t v_stride;
  int32_t num_pages;
  int32_t pw_log2;
  int32_t T;        // tokens of the call (t_exact) or the segment buffer's token capacity
  int32_t t_exact;  // the segments must have been built for exactly T tokens (else for at most T)
  // capacities of the segment buffer's plan (segments, items per table);
  // counts beyond them mean the buffer was not built as laid out
  int32_t s_cap, cap_sm, cap_sv, cap_em, cap_ev;
  int32_t np;
  int32_t xshare;  // every projection of the launch reads the same X (same pointer, ldx, d_in)
  // the apply kernel's phase barrier: the segment buffer's sync area, the
  // bound of the wait in 100 MHz ticks, and an offset added to the wait's
  // target (> 0 only to force the give-up path in tests)
  int32_t* sync;
  int64_t wait_ticks;
  int32_t wait_bias;
};

struct SegOut {
  int32_t* perm;
  int32_t* seg_indptr;
  int32_t* seg_adapter;
  int32_t* v_indptr;
  int32_t* seg_desc;
  int32_t* shr_item_m;
  int32_t* shr_item_v;
  int32_t* exp_item_m;
  int32_t* exp_item_v;
  int32_t* counts;
  int32_t* sync;
};

hipError_t launch_build_segments(const int32_t* ids, int T, int N, const int32_t* rank, const float* alpha,
                                 int32_t* hist, const SegOut& out, hipStream_t stream);
hipError_t launch_shrink(const KArgs& K, int dtype, int grid, hipStream_t stream);
hipError_t launch_expand(const KArgs& K, int dtype, int grid, hipStream_t stream);
hipError_t launch_apply(const KArgs& K, int dtype, int grid, hipStream_t stream);
hipError_t occupancy(int dtype, int* shrink_blocks, int* expand_blocks, int* apply_blocks);

}  // namespace lora
