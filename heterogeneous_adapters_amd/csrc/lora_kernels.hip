// gfx950 (CDNA4) kernels of the multi-LoRA adapter branch.
//
// Sources:
//   [MLSP] "Multi-LoRA Serving in Production: Architecture, Dynamic Adapter
//          Swapping, and GPU Memory Management" (llms.blog)
//   [MLSA] "Multi-LoRA Serving Architecture: Serving Hundreds of Fine-Tuned
//          Adapters on One GPU with vLLM and S-LoRA (2026)"
//   [LAST] "LoRA Adapters at Serve Time with vLLM Multi-LoRA"
//
// Kernels
//   seg_hist_kernel, seg_scan_kernel, seg_scatter_kernel
//       group tokens by adapter ([MLSP] SGMV grouping): a stable counting
//       sort, deterministic (integer atomics only count), plus the work plan.
//   shrink_kernel
//       v = X A for every segment ([MLSP] SGMV shrink), read straight from
//       the paged pool ([MLSP] "Unified Paging Architecture").  Short
//       segments take the MBGMV path (vector ALU dot products, wavefront
//       reductions across d_in); long ones the MBGMM path (16x16 MFMA
//       tiles).  Each work item covers one 512-column slice of d_in and
//       writes a partial v; the expand sums the slices in ascending order,
//       so every result is bitwise deterministic.
//   expand_kernel
//       Y = Y_base + (alpha/r) v B ([MLSP] SGMV expand), same two paths; v
//       of an item's tokens is staged in LDS.
//
// Both compute kernels are persistent grids that walk a device-side item
// list (no host read-back of the segment count).  Items are dealt to the 8
// XCDs in contiguous ranges so the items that share an adapter slice run on
// the XCD whose L2 already holds it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora.h"
#include "lora_kernels.h"
#include "lora_plan.h"

namespace lora {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ element types
struct Bf16 {
  typedef uint16_t T;
  static constexpr int kEpv = 8;  // elements per 16-byte vector
  static constexpr int kShrinkBlocks = 4;  // occupancy targets (work-groups per CU)
  static constexpr int kExpandBlocks = 3;
};
struct F32 {
  typedef float T;
  static constexpr int kEpv = 4;
  static constexpr int kShrinkBlocks = 3;
  static constexpr int kExpandBlocks = 2;
};

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f_to_bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f_to_bf(lo) | ((uint32_t)f_to_bf(hi) << 16);
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Y is written once and read by nothing in the launch or the next one, so its
// stores carry the non-temporal hint: they do not fill L2 and the MALL with
// dirty lines that the next launch's weights and metadata would have to
// displace (measured: the shrink after an expand 3.5 % faster, prefill 2 %).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void stg16_nt(void* p, uint4 u) {
  __builtin_nontemporal_store(u32x4{u.x, u.y, u.z, u.w}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void stg4_nt(void* p, uint32_t u) {
  __builtin_nontemporal_store(u, reinterpret_cast<uint32_t*>(p));
}

// Loads of metadata that no kernel of the call writes (segments, page
// tables), through the constant address space so that wave-uniform
// addresses become scalar loads.
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ int cld(const int32_t* p) { return *(const __attribute__((address_space(4))) int32_t*)(p); }
__device__ __forceinline__ int4 cld4(const int4* p) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i v = *(const __attribute__((address_space(4))) v4i*)(p);
  return make_int4(v.x, v.y, v.z, v.w);
}
#else
__device__ int cld(const int32_t* p);
__device__ int4 cld4(const int4* p);
#endif
__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// The rank-r partial sums v: plain loads and stores between two launches;
// in the single-launch apply kernel (CO) agent-scope atomic accesses, since
// a partial written by a wave on one XCD is read by waves on others while
// the kernel runs.  On gfx950 these are ordinary loads and stores with the
// sc1 bit (coherent at agent scope, write-through) -- no cache maintenance.
template <bool CO>
__device__ __forceinline__ float vld(const float* p) {
  if constexpr (CO) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
template <bool CO>
__device__ __forceinline__ void vst(float* p, float x) {
  if constexpr (CO) __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = x;
}

// 8-wide bf16 dot product accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot16(uint4 w, uint4 x, float acc, Bf16) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, x.w), acc, false);
  return acc;
}
// 4-wide fp32 dot product.
__device__ __forceinline__ float dot16(uint4 w, uint4 x, float acc, F32) {
  acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
  acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
  acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
  acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
  return acc;
}

// C[16x16] += A[16xK] B[Kx16] from one 16-byte vector per lane and operand.
// bf16: one v_mfma_f32_16x16x32_bf16 (K = 32).  fp32: four
// v_mfma_f32_16x16x4_f32 (K = 4 each), element e of every lane's vector in
// MFMA e.  Both operands are loaded with the same lane -> K mapping, so the
// order in which K is visited does not matter.
__device__ __forceinline__ void mma(f4& c, uint4 a, uint4 b, Bf16) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f4& c, uint4 a, uint4 b, F32) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
}

// Pack kEpv fp32 values (index < n valid, rest zero) into one MFMA operand.
__device__ __forceinline__ uint4 pack_operand(const float* v, int n, Bf16) {
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = i < n ? v[i] : 0.0f;
  return make_uint4(pack_bf2(e[0], e[1]), pack_bf2(e[2], e[3]), pack_bf2(e[4], e[5]), pack_bf2(e[6], e[7]));
}
__device__ __forceinline__ uint4 pack_operand(const float* v, int n, F32) {
  float e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = i < n ? v[i] : 0.0f;
  return make_uint4(__float_as_uint(e[0]), __float_as_uint(e[1]), __float_as_uint(e[2]), __float_as_uint(e[3]));
}

__device__ __forceinline__ float to_f(uint16_t h) { return bf_to_f(h); }
__device__ __forceinline__ float to_f(float f) { return f; }
__device__ __forceinline__ void from_f(uint16_t* p, float f) { *p = f_to_bf(f); }
__device__ __forceinline__ void from_f(float* p, float f) { *p = f; }

// ------------------------------------------------------------ pool access
template <class E>
__device__ __forceinline__ const typename E::T* page_ptr(const KArgs& K, int page) {
  if ((unsigned)page >= (unsigned)K.num_pages) {
    atomicOr(&K.counts[kCountFlags], LORA_FLAG_PAGE_RANGE);
    return nullptr;
  }
  return reinterpret_cast<const typename E::T*>(K.pool) + ((int64_t)page << (K.pw_log2 + 4));
}

// Page base with the range check folded in: an id outside the pool sets the
// device flag, the load is redirected to page 0 and `ok` zeroes its value.
template <class E>
__device__ __forceinline__ const typename E::T* page_base(const KArgs& K, int page, bool& ok) {
  ok = (unsigned)page < (unsigned)K.num_pages;
  if (!ok) atomicOr(&K.counts[kCountFlags], LORA_FLAG_PAGE_RANGE);
  return reinterpret_cast<const typename E::T*>(K.pool) + ((int64_t)(ok ? page : 0) << (K.pw_log2 + 4));
}

// Keep the first kn (1..kEpv) elements of a vector, zero the rest.
__device__ __forceinline__ uint4 keep_first(uint4 w, int kn, Bf16) {
  auto m = [kn](int d) { return kn > 2 * d + 1 ? 0xffffffffu : (kn > 2 * d ? 0x0000ffffu : 0u); };
  return make_uint4(w.x & m(0), w.y & m(1), w.z & m(2), w.w & m(3));
}
__device__ __forceinline__ uint4 keep_first(uint4 w, int kn, F32) {
  return make_uint4(kn > 0 ? w.x : 0u, kn > 1 ? w.y : 0u, kn > 2 ? w.z : 0u, kn > 3 ? w.w : 0u);
}

// In-page element offset of the B vector holding ranks kin..kin+kEpv-1
// (kin = rank - 16g, a multiple of kEpv) of page column jp: half kin/8 at
// kin/8 * 8*pw, then 8 ranks per column.  `upper` (the group has more than 8
// ranks) false reads the lower half instead (see the note above).
__device__ __forceinline__ int b_off(int jp, int kin, int pw, bool upper) {
  return (upper ? (kin >> 3) * 8 * pw : 0) + jp * 8 + (kin & 7);
}

// B vectors (kEpv consecutive ranks of one output column; a B page holds
// its 16 rank slots as two halves of 8, so the 8 ranks of a column in one
// half are one 16- or 32-byte run) are loaded unconditionally from valid
// addresses -- the upper half of a rank group with at most 8 ranks from the
// same column's lower half (bytes the lower half's own load fetches, so such
// a group moves only its used half), a rank group past the adapter's from
// its last group, a page outside the pool from page 0 -- and zeroed where
// they are used.  A skipped load
// would write zeros into registers that an older load may still target, and
// the compiler then waits for that older load.

// Largest s with ptr[s] <= u (ptr strictly increasing, ptr[0] = 0).
__device__ __forceinline__ int find_segment(const int32_t* ptr, int S, int u) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ptr[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Wave64 reduce-scatter of 32 per-lane values: afterwards lanes 2i and 2i+1
// hold the sum over all 64 lanes of value i.  Each step halves the values a
// lane keeps while summing over one more lane bit: bit 5 with
// v_permlane32_swap (lane l <-> l^32 between two registers), bit 4 with
// v_permlane16_swap (l <-> l^16), bit 3 with a DPP row rotation by 8, bit 2
// with a swizzle, bits 1 and 0 with DPP quad permutations.  Exchanges are
// commutative adds, so a value's sum is the same whichever lane holds it.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppQuadXor2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xb1;  // quad_perm [1,0,3,2]

__device__ __forceinline__ float wave_reduce_scatter32(float (&v)[32], int lane) {
  float a[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // lanes with bit 5 clear keep value i, set keep i+16
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 16]), false, false);
    a[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  float b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // bit 4 clear keeps a[i], set keeps a[i+8]
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(a[i + 8]), false, false);
    b[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const bool u3 = (lane & 8) != 0, u2 = (lane & 4) != 0, u1 = (lane & 2) != 0;
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {   // bit 3
    const float send = u3 ? b[i] : b[i + 4];
    c[i] = (u3 ? b[i + 4] : b[i]) + dpp_f<kDppRowRor8>(send);
  }
  float d[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {   // bit 2
    const float send = u2 ? c[i] : c[i + 2];
    d[i] = (u2 ? c[i + 2] : c[i]) +
           __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(send), (4 << 10) | 0x1f));
  }
  const float send = u1 ? d[0] : d[1];  // bit 1
  const float e = (u1 ? d[1] : d[0]) + dpp_f<kDppQuadXor2>(send);
  return e + dpp_f<kDppQuadXor1>(e);    // bit 0
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }


// The kernels take one by-value KArgs argument, which sits at offset 0 of the
// kernel-argument segment.  They read it through the segment pointer, so a
// descriptor picked by a run-time projection index is a scalar load from
// that segment, never a private copy of the whole struct.
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ const KArgs& kernel_args() {
  return *reinterpret_cast<const KArgs*>(__builtin_amdgcn_kernarg_segment_ptr());
}
#else
__device__ const KArgs& kernel_args();
#endif

// The segment buffer's counters, read (scalar loads) before any plan entry.
// A buffer that was never built (check word), built for another token count
// than the call's, or whose totals exceed the capacity the plan was laid out
// for, is not walked: the launch computes nothing and raises
// LORA_FLAG_SEGMENTS, so such a buffer never leads to an access outside it.
struct PlanCounts {
  int S, T, t_valid, shr_m, shr_v, exp_m, exp_v;
  bool ok;
};
__device__ __forceinline__ PlanCounts read_counts(const KArgs& K) {
  PlanCounts c;
  c.S = cld(K.counts + kCountS);
  c.T = cld(K.counts + kCountT);
  c.t_valid = cld(K.counts + kCountTValid);
  c.shr_m = cld(K.counts + kCountShrinkMfma);
  c.shr_v = cld(K.counts + kCountShrinkValu);
  c.exp_m = cld(K.counts + kCountExpandMfma);
  c.exp_v = cld(K.counts + kCountExpandValu);
  const int chk = cld(K.counts + kCountCheck);
  c.ok = chk == segments_check_word(c.T) && c.T >= 0 && (K.t_exact ? c.T == K.T : c.T <= K.T) &&
         c.S >= 0 && c.S <= min(c.T, K.s_cap) && c.t_valid >= 0 && c.t_valid <= c.T && c.shr_m >= 0 &&
         c.shr_m <= K.cap_sm && c.shr_v >= 0 && c.shr_v <= K.cap_sv && c.exp_m >= 0 && c.exp_m <= K.cap_em &&
         c.exp_v >= 0 && c.exp_v <= K.cap_ev;
  if (!c.ok && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&K.counts[kCountFlags], LORA_FLAG_SEGMENTS);
  return c;
}

// The expand side of the apply kernel's phase barrier.  Every wave waits,
// once, before it first reads v: the counter of XCDs whose work-groups have
// all written their shrink partial sums must reach its target.  The wait is
// bounded (s_memrealtime, a 100 MHz clock); past the bound the wave gives
// up, raises LORA_FLAG_SYNC and goes on (the call's Y is then invalid).  In
// the two-launch kernels `done` is null and nothing is waited for.
struct PhaseWait {
  const int* done;
  int target;
  long long ticks;
  bool passed;
  __device__ bool ready() const { return passed; }
  __device__ void wait(const KArgs& K) {
    if (passed) return;
    passed = true;
    if (!done) return;
    const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
    for (;;) {
      const int v = uniform(__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (v >= target) return;
      if ((long long)__builtin_amdgcn_s_memrealtime() - t0 > ticks) {
        if ((threadIdx.x & 63) == 0) atomicOr(&K.counts[kCountFlags], LORA_FLAG_SYNC);
        return;
      }
      __builtin_amdgcn_s_sleep(4);
    }
  }
};

// The MBGMV item sequence of one wave: first() gives its first item (-1:
// none), issue() / resolve() the next one (-1: none left).
struct StaticWalk {
  TwoClassWalk tw;
  int pend;
  __device__ StaticWalk(int total, int Wm, int R, int wave) : tw(total, Wm, R, wave, gridDim.x, blockIdx.x) {}
  __device__ int first() { return tw.i < tw.end ? tw.i : -1; }
  __device__ void issue() { pend = tw.next(); tw.i = pend; }
  __device__ int resolve() { return pend < tw.end ? pend : -1; }
};

// ================================================================ shrink
// MBGMV item (one wave): (segment, rank group g, <= 2 tokens, 512-column
// slice q).  Each lane streams one 16-byte vector (8 bf16 / 4 fp32 columns)
// of each of the group's 16 page rows -- a wave reads 1 KiB contiguous per
// row -- together with the same columns of the tokens' activation rows (the
// gathered activations of [MLSP] SGMV), forms partial dot products, and the
// 64 lanes are reduced across the wave.  All loads are issued before the
// first product, so an item costs one memory round trip after its page
// lookup.
// Metadata of one MBGMV shrink item, loaded one item ahead (scalar loads
// issued while the previous item's loads are in flight): the segment
// descriptor, the adapter's A-table slot, the page id of the slice (when the
// slice lies in one page) and the activation rows of its tokens.
struct ShrinkItem {
  int p, q;           // projection, 512-column slice
  int4 d0, d1;        // segment descriptor
  int g, tb, nt;      // rank group, first token (in the segment), tokens
  int slot0, pid;     // A-table slot of the group's first page; page id of the slice
  int xr[kValuTokens];  // activation rows of the tokens (past nt: the last one)
};

template <bool WIDE>
__device__ __forceinline__ ShrinkItem fetch_shrink_item(const KArgs& K, int i, int Uv) {
  ShrinkItem it;
  int u;
  if (K.xshare) {
    it.p = i % K.np;
    const int rest = i / K.np;
    it.q = rest / Uv;
    u = rest - it.q * Uv;
  } else {
    int rem = i, p = 0;
    while (rem >= K.p[p].nq * Uv) { rem -= K.p[p].nq * Uv; ++p; }
    it.p = p;
    it.q = rem / Uv;
    u = rem - it.q * Uv;
  }
  const KProj& P = K.p[it.p];
  const int4* dv = reinterpret_cast<const int4*>(K.shr_item_v) + 2 * u;  // the segment's descriptor
  it.d0 = cld4(dv);
  it.d1 = cld4(dv + 1);
  const int local = u - it.d1.y;
  const int n = it.d0.w;
  const int nch = ceil_div_i(n, kValuTokens);
  it.g = local / nch;
  it.tb = (local - it.g * nch) * kValuTokens;
  it.nt = min(kValuTokens, n - it.tb);
  it.slot0 = cld(P.a_indptr + it.d0.x) + it.g * ((P.d_in + (1 << K.pw_log2) - 1) >> K.pw_log2);
  it.pid = WIDE ? cld(P.a_pages + it.slot0 + ((it.q * kKSlice) >> K.pw_log2)) : 0;
#pragma unroll
  for (int tt = 0; tt < kValuTokens; ++tt) it.xr[tt] = cld(K.perm + it.d0.z + it.tb + min(tt, it.nt - 1));
  return it;
}

// The loads of one MBGMV shrink item, held in registers until its products.
template <class E>
struct ShrinkLoads {
  static constexpr int NVEC = kKSlice / (64 * E::kEpv);  // vectors per lane and row (bf16 1, fp32 2)
  uint4 x[kValuTokens][NVEC];
  uint4 w[16][NVEC];
  bool ok[NVEC];  // lane inside d_in and page inside the pool
};

// Issue every load of an item.  Every load is unconditional and in bounds:
// rows past the rank re-read the group's last row, tokens past the item its
// last token, lanes past d_in the slice's last vector.  Their products are
// never stored (rows, tokens) or are zeroed before the reduction (lanes), so
// no load is ever skipped -- a skipped load's zero fill would make the
// compiler wait for older loads into the same registers.
template <class E, bool WIDE>
__device__ __forceinline__ void shrink_valu_issue(const KArgs& K, const KProj& P, const ShrinkItem& item, int lane,
                                                  ShrinkLoads<E>& L) {
  typedef typename E::T T;
  constexpr int EPV = E::kEpv;
  constexpr int NVEC = ShrinkLoads<E>::NVEC;
  constexpr int NV = kValuTokens;
  const int q = item.q;
  const int r = item.d0.y;
  const int g = item.g;
  const int col0 = q * kKSlice;
  const int ncols = min(kKSlice, P.d_in - col0);  // a multiple of 8
  const int pw = 1 << K.pw_log2;
  const int rows = min(16, r - g * 16);
  const T* X = reinterpret_cast<const T*>(P.X);
  int cl[NVEC];
  bool lane_ok[NVEC];
#pragma unroll
  for (int v = 0; v < NVEC; ++v) {
    const int c = v * 64 * EPV + lane * EPV;
    lane_ok[v] = c < ncols;
    cl[v] = lane_ok[v] ? c : ncols - EPV;
  }
  const T* pg[NVEC];
  bool pok[NVEC];
  if constexpr (WIDE) {  // the slice lies in one page: a wave-uniform lookup
    bool ok;
    const T* p = page_base<E>(K, item.pid, ok);
#pragma unroll
    for (int v = 0; v < NVEC; ++v) {
      pg[v] = p;
      pok[v] = ok;
    }
  } else {
#pragma unroll
    for (int v = 0; v < NVEC; ++v) pg[v] = page_base<E>(K, P.a_pages[item.slot0 + ((col0 + cl[v]) >> K.pw_log2)], pok[v]);
  }
#pragma unroll
  for (int v = 0; v < NVEC; ++v) L.ok[v] = lane_ok[v] && pok[v];
  // X first, then the rows in product order: vector memory returns in issue
  // order, so the products of row rr wait only for X and rows 0..rr
#pragma unroll
  for (int tt = 0; tt < NV; ++tt) {
    const int64_t row = (int64_t)item.xr[tt] * P.ldx + col0;
#pragma unroll
    for (int v = 0; v < NVEC; ++v) L.x[tt][v] = ldg16(X + row + cl[v]);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int rr = 0; rr < 16; ++rr)
#pragma unroll
    for (int v = 0; v < NVEC; ++v) L.w[rr][v] = ldg16(pg[v] + min(rr, rows - 1) * pw + ((col0 + cl[v]) & (pw - 1)));
}

// The products, the wave reduction and the stores of an item's partial sums.
template <class E, bool CO>
__device__ __forceinline__ void shrink_valu_finish(const KArgs& K, const KProj& P, const ShrinkItem& item, int lane,
                                                   const ShrinkLoads<E>& L) {
  constexpr int NVEC = ShrinkLoads<E>::NVEC;
  constexpr int NV = kValuTokens;
  const int r = item.d0.y;
  const int rows = min(16, r - item.g * 16);
  static_assert(16 * NV == 32, "one 32-value wave reduction per item");
  float acc[32];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr)
#pragma unroll
    for (int tt = 0; tt < NV; ++tt) {
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < NVEC; ++v) {
        const float d = dot16(L.w[rr][v], L.x[tt][v], 0.0f, E());
        s += L.ok[v] ? d : 0.0f;
      }
      acc[rr * NV + tt] = s;
    }
  const float sum = wave_reduce_scatter32(acc, lane);
  const int vi = lane >> 1;
  const int rr = vi / NV, tt = vi % NV;
  if ((lane & 1) == 0 && rr < rows && tt < item.nt)
    vst<CO>(P.v + (int64_t)item.q * K.v_stride + item.d1.x + (int64_t)(item.tb + tt) * r + item.g * 16 + rr, sum);
}

// MBGMV item (one wave): (segment, rank group g, <= 2 tokens, 512-column
// slice q).  Each lane streams one 16-byte vector (8 bf16 / 4 fp32 columns)
// of each of the group's 16 page rows -- a wave reads 1 KiB contiguous per
// row -- together with the same columns of the tokens' activation rows (the
// gathered activations of [MLSP] SGMV), forms partial dot products, and the
// 64 lanes are reduced across the wave.  All loads are issued before the
// first product, so an item costs one memory round trip; the next item's
// metadata is fetched while they are in flight.
template <class E, bool WIDE, bool CO, class Prefetch>
__device__ __forceinline__ void shrink_valu(const KArgs& K, const KProj& P, const ShrinkItem& item, int lane,
                                            Prefetch&& prefetch) {
  ShrinkLoads<E> L;
  shrink_valu_issue<E, WIDE>(K, P, item, lane, L);
  __builtin_amdgcn_sched_barrier(0);
  prefetch();
  __builtin_amdgcn_sched_barrier(0);
  shrink_valu_finish<E, CO>(K, P, item, lane, L);
}

// MBGMM item (one wave): (segment, 16*NTT-token tile, GG rank groups from
// g0, slice q): C[rank][token] += A^T[rank][col] * X^T[col][token] over the
// slice's 512 columns, as GG x NTT 16x16 MFMA tiles -- each A operand shared
// by the NTT token tiles (A, re-read from L2 for every tile of a segment, is
// read once per 16*NTT tokens) and each X operand by the GG rank groups (the
// tile's activations are read once per GG groups) -- with the operands of
// SIF K steps requested before the first of their MFMAs.  The items of one
// token tile (its group sets) are consecutive, so they re-read the tile's
// activations from the L2 that holds them.
template <class E, bool WIDE, int NTT, int GG, bool CO>
__device__ __forceinline__ void shrink_mfma(const KArgs& K, const KProj& P, int q, int4 d0, int4 d1, int local,
                                            int lane) {
  typedef typename E::T T;
  constexpr int EPV = E::kEpv;
  constexpr int STEP = 4 * EPV;
  constexpr int NSTEP = kKSlice / STEP;
  constexpr int TILE = 16 * NTT;                          // tokens per item
  // K steps in flight: 8 (A + NTT X) operand pairs with one group, two with
  // groups sharing X (GG A + NTT X operands each).  A K step reads 64 bytes
  // of every operand row, so two steps request each 128-byte line whole in
  // one burst: requested one step apart, the line's second half was often
  // fetched again, evicted by the other waves' loads in between (the prefill
  // shrink read 1.31x its bytes with one step, 1.06x with two)
  constexpr int SIF = GG == 1 ? 8 / NTT : 2;
  static_assert(NSTEP % SIF == 0, "steps in flight divide the slice");
  const int a = d0.x, r = d0.y, t0 = d0.z, n = d0.w;
  const int G = rank_groups(r);
  const int GQ = ceil_div_i(G, GG);  // group sets per token tile
  const int tt = local / GQ;
  const int g0 = (local - tt * GQ) * GG;
  const int tb = tt * TILE;
  const int nt = min(TILE, n - tb);
  const int li = lane & 15, qq = lane >> 4;
  const int col0 = q * kKSlice;
  const int ncols = min(kKSlice, P.d_in - col0);  // a multiple of 8
  const int pw = 1 << K.pw_log2;
  const int nci = (P.d_in + pw - 1) >> K.pw_log2;
  const int abase = cld(P.a_indptr + a);
  // group gi of the item is g0 + gi, or (past the adapter's last group) the
  // last group again: its loads stay in bounds and its products are skipped
  int slot[GG];
  bool ok1[GG];
  const T* pg1[GG];
#pragma unroll
  for (int gi = 0; gi < GG; ++gi) {
    slot[gi] = abase + min(g0 + gi, G - 1) * nci;
    ok1[gi] = true;
    pg1[gi] = WIDE ? page_base<E>(K, cld(P.a_pages + slot[gi] + (col0 >> K.pw_log2)), ok1[gi]) : nullptr;
  }
  // Operands are loaded row-contiguously -- lane l reads chunk l & 3 of row
  // l >> 2, so a quarter-wave covers 4 rows x 64 contiguous bytes -- and
  // moved to the MFMA layout (lane L holds chunk L >> 4 of row L & 15) with a
  // cross-lane permute.  Loaded in the MFMA layout directly, every
  // quarter-wave would touch 16 rows (16 cache lines per 256 bytes).
  // Loads are unconditional and in bounds (see shrink_valu_issue): rank rows
  // past r re-read the group's last row (their outputs are never stored),
  // tokens past the tile its first token (never stored); K positions past
  // d_in are zeroed at the product.
  const int lr = lane >> 2, lk = lane & 3;
  const int src = ((lane & 15) * 4 + (lane >> 4)) * 4;  // byte address of the source lane
  int lrow[GG];
#pragma unroll
  for (int gi = 0; gi < GG; ++gi) lrow[gi] = min(lr, r - min(g0 + gi, G - 1) * 16 - 1);
  const T* X = reinterpret_cast<const T*>(P.X);
  int64_t xrow[NTT];
#pragma unroll
  for (int s = 0; s < NTT; ++s) xrow[s] = (int64_t)K.perm[t0 + tb + (s * 16 + lr < nt ? s * 16 + lr : 0)] * P.ldx;
  auto permute = [src](uint4 v) {
    return make_uint4(__builtin_amdgcn_ds_bpermute(src, (int)v.x), __builtin_amdgcn_ds_bpermute(src, (int)v.y),
                      __builtin_amdgcn_ds_bpermute(src, (int)v.z), __builtin_amdgcn_ds_bpermute(src, (int)v.w));
  };
  f4 acc[GG][NTT];
#pragma unroll
  for (int gi = 0; gi < GG; ++gi)
#pragma unroll
    for (int s = 0; s < NTT; ++s) acc[gi][s] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int st0 = 0; st0 < NSTEP; st0 += SIF) {
    uint4 av[SIF][GG], xv[SIF][NTT];
    bool okv[SIF][GG];
#pragma unroll
    for (int j = 0; j < SIF; ++j) {
      const int cl = (st0 + j) * STEP + lk * EPV;       // this lane's load chunk
      const int col = col0 + min(cl, ncols - EPV);
      const bool inside = (st0 + j) * STEP + qq * EPV < ncols;  // the chunk it holds after the permute
#pragma unroll
      for (int gi = 0; gi < GG; ++gi) {
        okv[j][gi] = inside;
        if constexpr (!WIDE) {
          // the page of the chunk this lane will hold decides its mask; the
          // page of the chunk it loads, the address
          bool okh, okl;
          page_base<E>(K, P.a_pages[slot[gi] + ((col0 + min((st0 + j) * STEP + qq * EPV, ncols - EPV)) >> K.pw_log2)],
                       okh);
          okv[j][gi] = okv[j][gi] && okh;
          const T* pl = page_base<E>(K, P.a_pages[slot[gi] + (col >> K.pw_log2)], okl);
          av[j][gi] = ldg16(pl + lrow[gi] * pw + (col & (pw - 1)));
        } else {
          av[j][gi] = ldg16(pg1[gi] + lrow[gi] * pw + (col & (pw - 1)));
        }
      }
#pragma unroll
      for (int s = 0; s < NTT; ++s) xv[j][s] = ldg16(X + xrow[s] + col);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < SIF; ++j) {
      // permute with every lane active (a permute reads 0 from an inactive
      // lane), then zero the K positions past d_in with a mask
      uint4 xp[NTT];
#pragma unroll
      for (int s = 0; s < NTT; ++s) xp[s] = permute(xv[j][s]);
#pragma unroll
      for (int gi = 0; gi < GG; ++gi) {
        if (GG > 1 && g0 + gi >= G) continue;  // uniform
        const uint4 ap = permute(av[j][gi]);
        const uint32_t m = (okv[j][gi] && ok1[gi]) ? 0xffffffffu : 0u;
        const uint4 am = make_uint4(ap.x & m, ap.y & m, ap.z & m, ap.w & m);
#pragma unroll
        for (int s = 0; s < NTT; ++s) mma(acc[gi][s], am, xp[s], E());
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < GG; ++gi) {
    if (GG > 1 && g0 + gi >= G) continue;
    const int k0 = (g0 + gi) * 16 + qq * 4;
#pragma unroll
    for (int s = 0; s < NTT; ++s) {
      if (s * 16 + li < nt) {
        float* dst = P.v + (int64_t)q * K.v_stride + d1.x + (int64_t)(tb + s * 16 + li) * r + k0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + i < r) vst<CO>(dst + i, acc[gi][s][i]);
      }
    }
  }
}

// WIDE: pages hold at least one whole 512-column slice, so every page
// lookup of an item is wave-uniform; chosen by the host from the page width.
// The shrink items of one wave: its MBGMM items (the static XCD-aware walk),
// then its MBGMV items in the order `walk` gives them.
template <class E, bool WIDE, bool CO, class Walk>
__device__ __forceinline__ void shrink_items(const KArgs& K, Walk walk, int total, int Um, int Uv, int wave,
                                             int lane) {
  const int grid = gridDim.x, block = blockIdx.x;
  // The wave's first MBGMV item's metadata is requested before the MBGMM pass.
  ShrinkItem cur;
  const int i0 = walk.first();
  if (i0 >= 0) cur = fetch_shrink_item<WIDE>(K, i0, Uv);
  // Item order: projection-major, or -- when every projection of the launch
  // reads the same X -- projection-minor, so the siblings' items for one
  // (slice, item) run side by side and their X rows come from L2.
  for (WaveWalk it(total, wave, kWaves, grid, block); it.i < it.end; it.i += it.stride) {
    int p, q, u;
    if (K.xshare) {
      p = it.i % K.np;
      const int rest = it.i / K.np;
      q = rest / Um;
      u = rest - q * Um;
    } else {
      int rem = it.i;
      p = 0;
      while (rem >= K.p[p].nq * Um) { rem -= K.p[p].nq * Um; ++p; }
      q = rem / Um;
      u = rem - q * Um;
    }
    const int s = cld(K.shr_item_m + u);
    const int4 d0 = cld4(K.seg_desc + 2 * s), d1 = cld4(K.seg_desc + 2 * s + 1);
    const int gg = shrink_item_groups(d0.w, d0.y);  // uniform
    if (gg == 2)
      shrink_mfma<E, WIDE, kMfmaShrinkTokensLong / 16, 2, CO>(K, K.p[p], q, d0, d1, u - d1.y, lane);
    else
      shrink_mfma<E, WIDE, kMfmaShrinkTokensShort / 16, 1, CO>(K, K.p[p], q, d0, d1, u - d1.y, lane);
  }
  if (i0 < 0) return;
  for (;;) {
    walk.issue();
    int ni = -1;
    ShrinkItem nxt;
    shrink_valu<E, WIDE, CO>(K, K.p[cur.p], cur, lane, [&]() {
      ni = walk.resolve();
      if (ni >= 0) nxt = fetch_shrink_item<WIDE>(K, ni, Uv);
    });
    if (ni < 0) break;
    cur = nxt;
  }
}

template <class E, bool WIDE, bool CO>
__device__ __forceinline__ void shrink_phase(const KArgs& K, const PlanCounts& pc) {
  if (pc.S <= 0) return;
  const int Um = pc.shr_m, Uv = pc.shr_v;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // MBGMM items first, then MBGMV items; each path walks its own item list,
  // so the two register footprints never share a loop body.  The wave's
  // first MBGMV item's metadata is requested before the MBGMM pass.
  int total_v = 0;
  for (int p = 0; p < K.np; ++p) total_v += K.p[p].nq * Uv;
  int total = 0;
  for (int p = 0; p < K.np; ++p) total += K.p[p].nq * Um;
  const int grid = gridDim.x, block = blockIdx.x;
  int Wm, R;
  shrink_walk_split(total, total_v, wave, grid, block, Wm, R);
  shrink_items<E, WIDE, CO>(K, StaticWalk(total_v, Wm, R, wave), total, Um, Uv, wave, lane);
}

template <class E, bool WIDE>
__global__ __launch_bounds__(kThreads, E::kShrinkBlocks) void shrink_kernel(KArgs) {
  const KArgs& K = kernel_args();
  const PlanCounts pc = read_counts(K);
  if (!pc.ok) return;
  shrink_phase<E, WIDE, false>(K, pc);
}

// ================================================================ expand
// v of tokens [tb, tb+nt) of a segment into LDS rows of G*16 floats, ranks
// >= r zero-filled, by NT threads (one wave, or a whole block).  The chunk's
// v is nt*r contiguous floats in every partial slice.  Each thread sums M of
// them over the slices, SF slices' loads in flight at a time (M*SF = 16);
// every element is summed in ascending slice order whatever M and SF are.
// In steps, so that a caller may issue the first round of loads before
// other loads and add it later.
template <int M, int SF>
struct RowStage {
  float acc[M];
  float x[SF][M];
};

template <int NT, int M, int SF, bool CO>
__device__ __forceinline__ void row_load(const KArgs& K, const KProj& P, const float* src, int q, int e0, int ne,
                                         int tid, RowStage<M, SF>& st) {
#pragma unroll
  for (int j = 0; j < SF; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int e = e0 + tid + NT * m;
      st.x[j][m] = (q + j < P.nv && e < ne) ? vld<CO>(src + (int64_t)(q + j) * K.v_stride + e) : 0.0f;
    }
}

template <int M, int SF>
__device__ __forceinline__ void row_add(RowStage<M, SF>& st) {
#pragma unroll
  for (int j = 0; j < SF; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) st.acc[m] += st.x[j][m];
}

template <int NT, int M, int SF>
__device__ __forceinline__ void row_store(const RowStage<M, SF>& st, int e0, int ne, int r, int rs, float* vs,
                                          int tid) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = e0 + tid + NT * m;
    if (e < ne) {
      const int t = e / r;
      vs[t * rs + (e - t * r)] = st.acc[m];
    }
  }
}

template <int NT, int M, int SF, bool CO>
__device__ __forceinline__ void stage_v_pass(const KArgs& K, const KProj& P, const float* src, int e0, int ne,
                                             int r, int rs, float* vs, int tid) {
  RowStage<M, SF> st;
#pragma unroll
  for (int m = 0; m < M; ++m) st.acc[m] = 0.0f;
  for (int q = 0; q < P.nv; q += SF) {
    row_load<NT, M, SF, CO>(K, P, src, q, e0, ne, tid, st);
    row_add<M, SF>(st);
  }
  row_store<NT, M, SF>(st, e0, ne, r, rs, vs, tid);
}

// zero the rank padding (ranks r .. G*16) of nt staged rows
template <int NT>
__device__ __forceinline__ void stage_v_pad(int r, int nt, float* vs, int tid) {
  const int rs = rank_groups(r) * 16;
  for (int idx = tid; idx < nt * (rs - r); idx += NT) {
    const int t = idx / (rs - r);
    vs[t * rs + r + (idx - t * (rs - r))] = 0.0f;
  }
}

template <int NT, bool CO>
__device__ __forceinline__ void stage_v_rows(const KArgs& K, const KProj& P, int voff, int r, int tb, int nt,
                                             float* vs, int tid) {
  const int rs = rank_groups(r) * 16;
  const int ne = nt * r;
  const float* src = P.v + voff + (int64_t)tb * r;
  if (ne <= 2 * NT) stage_v_pass<NT, 2, 8, CO>(K, P, src, 0, ne, r, rs, vs, tid);
  else
    for (int e0 = 0; e0 < ne; e0 += NT * 8) stage_v_pass<NT, 8, 2, CO>(K, P, src, e0, ne, r, rs, vs, tid);
  stage_v_pad<NT>(r, nt, vs, tid);
}

// one wave stages its own rows
template <bool CO>
__device__ __forceinline__ void stage_v(const KArgs& K, const KProj& P, int voff, int r, int tb, int nt,
                                        float* vs, int lane) {
  stage_v_rows<64, CO>(K, P, voff, r, tb, nt, vs, lane);
  wave_sync();
}

// v of the tokens of a chunk as packed bf16 pairs in the wave's LDS rows,
// for products with packed bf16 B on the dot2 instructions: every fp32 value
// (the ascending-slice sum) is rounded to bf16 once, as the MBGMM path rounds
// its MFMA operand (relative 2^-9; the products and their sums stay fp32).
// Layout per token and rank group g (8 dwords): pairs (ranks 2j, 2j+1),
// j = 0..7.  Ranks >= r are zero.
// The staging of M (token, rank pair) entries per lane, in steps: set up
// the entries, load one round of SF slices, add it, store the pairs.  A
// caller may issue the first round before other loads and add it later.
template <int M>
struct SplitStage {
  static constexpr int SF = M >= 8 ? 1 : 8 / M;  // slices per round
  float acc[M][2];
  float x[SF][M][2];
  int e[M], kk[M];  // the pair's LDS slot is its index p0 + lane + 64 m
};

template <int M>
__device__ __forceinline__ void split_setup(SplitStage<M>& st, int p0, int np, int r, int G, int lane) {
  const int hp = G * 8;  // rank pairs per token
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int p = p0 + lane + 64 * m;
    const int t = p / hp, kp = p - t * hp;  // pair kp = ranks 2kp, 2kp+1
    st.kk[m] = p < np ? 2 * kp : LORA_MAX_RANK;  // past the end: nothing loaded or stored
    st.e[m] = t * r + 2 * kp;
    st.acc[m][0] = st.acc[m][1] = 0.0f;
  }
}

template <int M, bool CO>
__device__ __forceinline__ void split_load(const KArgs& K, const KProj& P, const float* src, int q, int r,
                                           SplitStage<M>& st) {
#pragma unroll
  for (int j = 0; j < SplitStage<M>::SF; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float* a = src + (int64_t)(q + j) * K.v_stride + st.e[m];
      const bool ok = q + j < P.nv;
      st.x[j][m][0] = ok && st.kk[m] < r ? vld<CO>(a) : 0.0f;
      st.x[j][m][1] = ok && st.kk[m] + 1 < r ? vld<CO>(a + 1) : 0.0f;
    }
}

template <int M>
__device__ __forceinline__ void split_add(SplitStage<M>& st) {
#pragma unroll
  for (int j = 0; j < SplitStage<M>::SF; ++j)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      st.acc[m][0] += st.x[j][m][0];
      st.acc[m][1] += st.x[j][m][1];
    }
}

// Pair p (token t, pair kp) goes to LDS dword t * (G * 8) + kp, which is p.
template <int M>
__device__ __forceinline__ void split_store(const SplitStage<M>& st, int p0, int lane, uint32_t* vs) {
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (st.kk[m] < LORA_MAX_RANK) vs[p0 + lane + 64 * m] = pack_bf2(st.acc[m][0], st.acc[m][1]);
}

template <int M, bool CO>
__device__ __forceinline__ void stage_v_split_pass(const KArgs& K, const KProj& P, const float* src, int p0,
                                                   int np, int r, int G, uint32_t* vs, int lane) {
  SplitStage<M> st;
  split_setup<M>(st, p0, np, r, G, lane);
  for (int q = 0; q < P.nv; q += SplitStage<M>::SF) {
    split_load<M, CO>(K, P, src, q, r, st);
    split_add<M>(st);
  }
  split_store<M>(st, p0, lane, vs);
}

template <bool CO>
__device__ __forceinline__ void stage_v_split(const KArgs& K, const KProj& P, int voff, int r, int n, uint32_t* vs,
                                              int lane) {
  const int G = rank_groups(r);
  const int np = n * G * 8;
  const float* src = P.v + voff;
  const int mm = ceil_div_i(np, 64);
  if (mm <= 1) stage_v_split_pass<1, CO>(K, P, src, 0, np, r, G, vs, lane);
  else if (mm <= 2) stage_v_split_pass<2, CO>(K, P, src, 0, np, r, G, vs, lane);
  else
    for (int p0 = 0; p0 < np; p0 += 64 * 4) stage_v_split_pass<4, CO>(K, P, src, p0, np, r, G, vs, lane);
  wave_sync();
}

// dot products of one 16-byte B vector (8 ranks of one column, packed bf16
// pairs) with the bf16 v of the same 8 ranks of one token.
__device__ __forceinline__ float dot8(uint4 w, uint4 v, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), __builtin_bit_cast(bf16x2, v.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), __builtin_bit_cast(bf16x2, v.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), __builtin_bit_cast(bf16x2, v.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), __builtin_bit_cast(bf16x2, v.w), acc, false);
  return acc;
}

// B element k (rank within the group) of lane-local column c, from the 4
// vectors (64 bytes) a lane holds per rank group.
__device__ __forceinline__ float b_elem(const uint4 (&b)[4], int c, int k, Bf16) {
  const uint32_t u = (&b[0].x)[(c * 16 + k) >> 1];
  return (k & 1) ? bf_hi(u) : bf_lo(u);
}
__device__ __forceinline__ float b_elem(const uint4 (&b)[4], int c, int k, F32) {
  return __uint_as_float((&b[0].x)[c * 16 + k]);
}

// Metadata of one MBGMV expand item, loaded one item ahead (scalar loads
// issued while the previous item's weight loads are in flight): the
// segment descriptor, the adapter's B-table offset and the page ids of its
// first kValuGroupBatch rank groups (when the item's columns lie in one page).
constexpr int kValuGroupBatch = 4;
struct ValuItem {
  int p, jb, local;  // projection, column block, item index inside the segment
  int copy;          // != 0: a copy of rows without an adapter (chunk = local)
  int4 d0, d1;       // segment descriptor
  int pg[kValuGroupBatch];
};

// Items per column block of a projection: Uv, plus the copy items when Y is
// not Y_base; dUv divides by Uv (every column block of a batch without
// tokens to copy).
template <class E>
__device__ __forceinline__ ValuItem fetch_valu_item(const KArgs& K, int i, int Uv, int ncopy, const FastDiv& dUv) {
  ValuItem it;
  int rem = i, p = 0;
  int Up = Uv + (K.p[0].Y != K.p[0].Yb ? ncopy : 0);
  while (rem >= K.p[p].njs * Up) {
    rem -= K.p[p].njs * Up;
    ++p;
    Up = Uv + (K.p[p].Y != K.p[p].Yb ? ncopy : 0);
  }
  const KProj& P = K.p[p];
  it.p = p;
  it.jb = Up == Uv ? dUv.div(rem) : rem / Up;
  const int u = rem - it.jb * Up;
  it.copy = u >= Uv;
  if (it.copy) {
    it.local = u - Uv;
    return it;
  }
  const int4* dv = reinterpret_cast<const int4*>(K.exp_item_v) + 2 * u;  // the segment's descriptor
  it.d0 = cld4(dv);
  it.d1 = cld4(dv + 1);
  it.local = u - it.d1.z;
  constexpr int CB = kValuSubBlocks * 64 * (4 / (int)sizeof(typename E::T));
  const int pw = 1 << K.pw_log2;
  if (pw >= CB) {
    const int ncolB = (P.d_out + pw - 1) >> K.pw_log2;
    const int base = cld(P.b_indptr + it.d0.x) + ((it.jb * CB) >> K.pw_log2);
    const int G = rank_groups(it.d0.y);
    const int32_t* pt = P.b_pages + base;
    it.pg[0] = cld(pt);
#pragma unroll
    for (int g = 1; g < kValuGroupBatch; ++g) {
      it.pg[g] = 0;
      if (g < G) it.pg[g] = cld(pt + g * ncolB);  // uniform
    }
  }
  return it;
}

// Y_base / Y access of the CPL adjacent columns a lane owns: one dword (two
// bf16 or one fp32), kept packed until used.
template <class T>
__device__ __forceinline__ uint32_t load_dword(const T* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ float unpack_col(uint32_t u, int c, Bf16) { return c == 0 ? bf_lo(u) : bf_hi(u); }
__device__ __forceinline__ float unpack_col(uint32_t u, int, F32) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t pack_cols(const float (&y)[2]) { return pack_bf2(y[0], y[1]); }
__device__ __forceinline__ uint32_t pack_cols(const float (&y)[1]) { return __float_as_uint(y[0]); }

// MBGMV expand item (one wave): (segment, part of a column block, chunk of
// <= kValuExpandTokens of the segment's tokens).  A column block is kValuSubBlocks = 4 sub-blocks
// of 64 lanes x CPL adjacent columns (2 in bf16, 1 in fp32); the 8 ranks of
// a column in each half of the B page are adjacent, so a lane reads 32
// contiguous bytes from each half per sub-block and rank group (the lower
// half only, for a group of at most 8 ranks).  A segment with 1, 2 or more rank groups
// covers the block in 1, 2 or 4 parts of nsub = 4, 2 or 1 sub-blocks, so
// every item holds four (sub-block, rank group) pairs -- 16 KiB of B per wave
// in bf16 -- all requested at once with the Y_base rows of every token of
// the chunk.  Pair i is (sub-block i % nsub, group g0 + i / nsub).  v of the
// chunk's tokens is staged once; the tokens are then produced one at a time
// from the B registers.
template <class E, bool ONE_PAGE, bool CO, class Prefetch>
__device__ __forceinline__ void expand_valu_body(const KArgs& K, const KProj& P, const ValuItem& item, float* vs,
                                                 int lane, PhaseWait& sw, bool fresh, Prefetch&& prefetch) {
  typedef typename E::T T;
  constexpr int EPV = E::kEpv;
  constexpr int CPL = 4 / (int)sizeof(T);
  constexpr int SUBW = 64 * CPL;  // columns per sub-block
  constexpr int NP = kValuSubBlocks;  // (sub-block, group) pairs per item
  const int4 d0 = item.d0, d1 = item.d1;
  const int a = d0.x, r = d0.y;
  // item = (part, chunk): chunks of one part are consecutive items, so they
  // run side by side on one XCD and re-read the part's B from its L2
  const int nch = valu_expand_chunks(d0.w);
  // part = local / nch with nch <= 8 and local < 32 (an MBGMV segment has
  // under 16 tokens): (local + 1/2) / nch lies at least 1/16 from an
  // integer, far beyond the reciprocal's error, so the floor is exact
  const int part = (int)(((float)item.local + 0.5f) * __builtin_amdgcn_rcpf((float)nch));
  const int chunk = item.local - part * nch;
  const int tb = chunk * kValuExpandTokens;
  const int t0 = d0.z + tb, n = min(kValuExpandTokens, d0.w - tb);
  const float scale = __int_as_float(d1.w) / (float)r;
  const int G = rank_groups(r);
  const int rs = G * 16;
  // sub-blocks per part: 4, 2 or 1 for 1, 2 or more rank groups (as a shift:
  // the pair index is split with shifts and masks, not run-time divisions)
  const int nsh = G == 1 ? 2 : (G == 2 ? 1 : 0);
  const int nsub = 1 << nsh;
  const int ngb = NP >> nsh;  // rank groups per batch of loads
  const int pw = 1 << K.pw_log2;
  const int ncolB = (P.d_out + pw - 1) >> K.pw_log2;
  const int jblk = item.jb * (kValuSubBlocks * SUBW);
  // first column this lane owns in each of the item's sub-blocks; a lane past
  // d_out works on the last column (never stored)
  int jc[NP];
  bool live[NP];
#pragma unroll
  for (int sb = 0; sb < NP; ++sb) {
    const int j = jblk + (part * nsub + sb) * SUBW + lane * CPL;
    live[sb] = sb < nsub && j < P.d_out;  // d_out is a multiple of 8: a lane's columns are all in or all out
    jc[sb] = j < P.d_out ? j : P.d_out - CPL;
  }
  // page ids of the batch's rank groups (one-page case), as four scalars: an
  // array indexed by the run-time group of a pair would live in scratch
  int pid0 = item.pg[0], pid1 = item.pg[1], pid2 = item.pg[2], pid3 = item.pg[3];
  uint4 b[NP][4];
  bool okp[NP];  // page of the pair inside the pool
  // The two page-lookup cases are separate instantiations: a page id read
  // per lane (block spanning pages) must be waited for before its data load,
  // and a shared path puts that wait in front of every pair's loads.
  auto load_batch = [&](int g0) {
    if constexpr (ONE_PAGE) {  // page ids are wave-uniform scalars: all 16 loads go out back to back
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int gi = i >> nsh;
        const int jcol = nsub == 4 ? jc[i] : (nsub == 2 ? jc[i & 1] : jc[0]);
        // a group past the adapter's has page id 0 here (never used)
        const T* pg = page_base<E>(K, gi == 0 ? pid0 : gi == 1 ? pid1 : gi == 2 ? pid2 : pid3, okp[i]);
        const bool up = r - 16 * (g0 + gi) > 8;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          b[i][q] = ldg16(pg + b_off((jcol & (pw - 1)) + q / (16 / EPV), (q % (16 / EPV)) * EPV, pw, up));
      }
    } else {  // per-lane page ids, all requested before the first data load
      int pl[NP];
      const int base = cld(P.b_indptr + a);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int g = min(g0 + (i >> nsh), G - 1);
        const int jcol = nsub == 4 ? jc[i] : (nsub == 2 ? jc[i & 1] : jc[0]);
        pl[i] = P.b_pages[base + g * ncolB + (jcol >> K.pw_log2)];
      }
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int jcol = nsub == 4 ? jc[i] : (nsub == 2 ? jc[i & 1] : jc[0]);
        const T* pg = page_base<E>(K, pl[i], okp[i]);
        const bool up = r - 16 * (g0 + (i >> nsh)) > 8;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          b[i][q] = ldg16(pg + b_off((jcol & (pw - 1)) + q / (16 / EPV), (q % (16 / EPV)) * EPV, pw, up));
      }
    }
  };
  const T* Yb = reinterpret_cast<const T*>(P.Yb);
  T* Y = reinterpret_cast<T*>(P.Y);
  // Y_base of every token of the chunk (one dword per sub-block), requested
  // with the weights: a token's row loaded after the previous token's
  // products would cost each token one more memory round trip.  Loads are
  // unconditional (tokens past the chunk re-read its last row, sub-blocks
  // past the part re-read a valid column); such values are never stored.
  uint32_t ybt[kValuExpandTokens][NP];
  auto load_yb_all = [&]() {
#pragma unroll
    for (int t = 0; t < kValuExpandTokens; ++t) {
      const int64_t row = cld(K.perm + t0 + min(t, n - 1));
#pragma unroll
      for (int sb = 0; sb < NP; ++sb) ybt[t][sb] = load_dword(Yb + row * P.ldyb + jc[sb]);
    }
  };
  // Vector memory returns in issue order, so data loaded after the weights
  // is waited for behind them.  When the chunk's v needs at most one
  // (token, rank pair) per lane, the first round of its loads goes out before
  // the weights, and summing it overlaps their round trip.
  [[maybe_unused]] SplitStage<1> st1;
  [[maybe_unused]] const float* vsrc = P.v + d1.x + tb * r;
  [[maybe_unused]] const bool early = EPV == 8 && n * G * 8 <= 64;
  // apply kernel: v is final only once the phase barrier has been passed
  // (fresh); an early round issued before that is issued again after the wait
  if constexpr (EPV == 8) {
    if (early) {
      split_setup<1>(st1, 0, n * G * 8, r, G, lane);
      split_load<1, CO>(K, P, vsrc, 0, r, st1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  load_batch(0);
  load_yb_all();
  // the next item's metadata, while this item's loads are in flight
  __builtin_amdgcn_sched_barrier(0);
  prefetch();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (CO) sw.wait(K);
  if constexpr (EPV == 8) {
    if (early) {
      // Each path sums its own loads: summed after the paths join, the sum's
      // wait would cover the longer path, and the early round (issued before
      // the weights) would wait for every weight load too.  The empty asm
      // statements keep the sums apart (the compiler does not merge them).
      if (fresh) {
        split_add<1>(st1);
        asm volatile("" : "+v"(st1.acc[0][0]), "+v"(st1.acc[0][1]));
      } else {
        split_load<1, CO>(K, P, vsrc, 0, r, st1);
        split_add<1>(st1);
        asm volatile("" : "+v"(st1.acc[0][0]), "+v"(st1.acc[0][1]));
      }
      for (int q = SplitStage<1>::SF; q < P.nv; q += SplitStage<1>::SF) {
        split_load<1, CO>(K, P, vsrc, q, r, st1);
        split_add<1>(st1);
      }
      split_store<1>(st1, 0, lane, reinterpret_cast<uint32_t*>(vs));
      wave_sync();
    } else {
      stage_v_split<CO>(K, P, d1.x + tb * r, r, n, reinterpret_cast<uint32_t*>(vs), lane);
    }
  } else {
    stage_v<CO>(K, P, d1.x, r, tb, n, vs, lane);
  }
  // Masks of a loaded batch, applied once in place (the token loop reuses the
  // registers): a page outside the pool reads as zeros, and in the last
  // group of a rank below a multiple of 16 the ranks >= r are zeroed.  With
  // wave-uniform page ids the page test is a branch, not a select per word.
  auto mask_batch = [&](int g0) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int g = g0 + (i >> nsh);
      if (g >= G) continue;
      uint4 (&w)[4] = b[i];
      if constexpr (ONE_PAGE) {
        if (!okp[i]) {
#pragma unroll
          for (int q = 0; q < 4; ++q) w[q] = zero4();
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = okp[i] ? w[q] : zero4();
      }
      if (r - g * 16 < 16) {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int v = 0; v < 16 / EPV; ++v) {
            // bf16: a vector wholly past r is an upper half, whose products
            // are skipped (see the token loop), so only a partly used vector
            // is masked; fp32 multiplies every vector
            const int kn = r - g * 16 - v * EPV;
            if (kn < EPV && (kn > 0 || EPV != 8))
              w[c * (16 / EPV) + v] = keep_first(w[c * (16 / EPV) + v], kn, E());
          }
      }
    }
  };
  mask_batch(0);
  for (int t = 0; t < n; ++t) {
    uint32_t (&yb)[NP] = ybt[0];  // token t's row; the rows move up one slot per token
    float acc[NP][CPL];  // per pair
#pragma unroll
    for (int i = 0; i < NP; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[i][c] = 0.0f;
    for (int g0 = 0; g0 < G; g0 += ngb) {
      // more than one batch of rank groups (only with nsub == 1): the batches
      // are loaded in turn, for every token
      if (g0 > 0 || (t > 0 && G > ngb)) {
        if constexpr (ONE_PAGE) {
          const int base = cld(P.b_indptr + a) + (jblk >> K.pw_log2);
          pid0 = cld(P.b_pages + base + g0 * ncolB);
          pid1 = g0 + 1 < G ? cld(P.b_pages + base + (g0 + 1) * ncolB) : 0;
          pid2 = g0 + 2 < G ? cld(P.b_pages + base + (g0 + 2) * ncolB) : 0;
          pid3 = g0 + 3 < G ? cld(P.b_pages + base + (g0 + 3) * ncolB) : 0;
        }
        load_batch(g0);
        mask_batch(g0);
      }
      uint4 vv[4];  // v of the current group: bf16 ranks {0-7, 8-15}; fp32 ranks 0-15
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int g = g0 + (i >> nsh);
        if (g >= G) continue;
        if ((i & (nsub - 1)) == 0) {  // first pair of a group: its v, once
          if constexpr (EPV == 8) {
            const uint4* vt = reinterpret_cast<const uint4*>(reinterpret_cast<const uint32_t*>(vs) + t * (G * 8) + g * 8);
            vv[0] = vt[0];
            vv[1] = vt[1];
          } else {
            const uint4* vt = reinterpret_cast<const uint4*>(vs + t * rs + g * 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) vv[q] = vt[q];
          }
        }
        const uint4 (&w)[4] = b[i];
        if constexpr (EPV == 8) {  // bf16: packed B against packed bf16 v (see stage_v_split)
          // a group of at most 8 ranks has only zeros in its upper half:
          // its products would add exact zeros, and are skipped
          if (r - g * 16 > 8) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[i][c] = dot8(w[c * 2 + 1], vv[1], dot8(w[c * 2], vv[0], acc[i][c]));
          } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[i][c] = dot8(w[c * 2], vv[0], acc[i][c]);
          }
        } else {
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[i][c] = fmaf(__uint_as_float((&vv[k4].x)[e]), b_elem(w, c, k4 * 4 + e, E()), acc[i][c]);
        }
      }
    }
    // pairs of one sub-block summed in ascending group order
    if (nsub == 2) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        acc[0][c] += acc[2][c];
        acc[1][c] += acc[3][c];
      }
    } else if (nsub == 1) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[0][c] = ((acc[0][c] + acc[1][c]) + acc[2][c]) + acc[3][c];
    }
    const int64_t row = cld(K.perm + t0 + t);
#pragma unroll
    for (int sb = 0; sb < NP; ++sb) {
      if (live[sb]) {
        float y[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) y[c] = unpack_col(yb[sb], c, E()) + scale * acc[sb][c];
        stg4_nt(Y + row * P.ldy + jc[sb], pack_cols(y));
      }
    }
#pragma unroll
    for (int tt = 0; tt + 1 < kValuExpandTokens; ++tt)
#pragma unroll
      for (int sb = 0; sb < NP; ++sb) ybt[tt][sb] = ybt[tt + 1][sb];
  }
}

// Y_base / Y access of 4 consecutive output columns (the 4 C values a lane
// holds for one token).
__device__ __forceinline__ void load4(const uint16_t* p, float (&y)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  y[0] = bf_lo(u.x); y[1] = bf_hi(u.x); y[2] = bf_lo(u.y); y[3] = bf_hi(u.y);
}
__device__ __forceinline__ void load4(const float* p, float (&y)[4]) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w;
}
__device__ __forceinline__ void store4(uint16_t* p, const float (&y)[4]) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]));
}
__device__ __forceinline__ void store4(float* p, const float (&y)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(y[0], y[1], y[2], y[3]);
}

// LDS floats per wave row set of the expand: a staged 16-token v tile
// (16 x LORA_MAX_RANK) or 16 output rows of up to 128 columns plus padding.
constexpr int kExpandRowFloats = kMfmaExpandTokens * (LORA_MAX_RANK + 4);

// MBGMM expand item, one wave's share: (segment, 16-token tile, wc output
// columns).  v of the tile is staged once (by the block); the columns are
// walked in parts of CT 16-column tiles, the B operands and Y_base values of
// part p+1 requested while part p is multiplied.
// C[col][token] += B^T[col][rank] * v^T[rank][token]: B pages hold the 16
// ranks of an output column contiguously, so each lane's operand is one
// 16-byte load, and a lane's four C values are four adjacent columns of one
// token (one 8- or 16-byte Y access).
template <class E, int NKS, bool WIDE, bool CO, class Next>
__device__ __forceinline__ void expand_mfma_body(const KArgs& K, const KProj& P, int j0, int jend, int wc, int a,
                                                 int r, int t0, int nt, float scale, float* vs, float* cw, int voff,
                                                 int tb, int lane, Next&& next) {
  typedef typename E::T T;
  constexpr int EPV = E::kEpv;
  constexpr int KSTEP = 4 * EPV;
  // 16-column tiles per part: the operands of two parts (current and next)
  // stay within 64 VGPRs (bf16: 128 columns for r <= 32, 64 for r <= 64).
  constexpr int CT = NKS >= 8 ? 1 : 8 / NKS;
  constexpr int PART = 16 * CT;
  const int li = lane & 15, qq = lane >> 4;
  const int rs = rank_groups(r) * 16;
  const int pw = 1 << K.pw_log2;
  const int ncolB = (P.d_out + pw - 1) >> K.pw_log2;
  // [j0, j0+wc) is wc-aligned, so it lies in one page of each group when
  // pw >= wc; always (wc <= pw is chosen by the caller)
  const bool one_page = WIDE || pw >= wc;
  const int bbase = cld(P.b_indptr + a);
  const T* Yb = reinterpret_cast<const T*>(P.Yb);
  T* Y = reinterpret_cast<T*>(P.Y);
  // Y_base / Y go through LDS in token rows: the MFMA result (a lane holds 4
  // columns of one token) is written to the wave's LDS rows and read back so
  // that each lane reads and writes one 16-byte chunk of a token row, a
  // quarter-wave covering whole 128-byte row segments (the MFMA layout itself
  // would touch 16 rows per quarter-wave with 8-byte accesses).
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = PART / EPC;           // chunks per token row of a part
  constexpr int TPR = 64 / CPR;             // token rows per round of the wave
  constexpr int ROUNDS = 16 / TPR;
  constexpr int LDC = PART + 4;             // LDS row stride (floats)
  static_assert(16 * LDC <= kExpandRowFloats, "output rows fit the wave's LDS rows");
  const int ch = lane % CPR;
  int64_t yrow[ROUNDS];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int tk = rd * TPR + lane / CPR;
    yrow[rd] = K.perm[t0 + min(tk, nt - 1)];  // tokens past the tile: the last one (never stored)
  }
  const int G = rank_groups(r);
  // page of each of this lane's K steps; a step past the last rank group
  // reads the last group and is zeroed by the rank mask
  // A wave with no columns in the item (jend <= 0: past d_out in the item's
  // last column block) looks up page column 0: its own column may lie past
  // the adapter's last page column, i.e. past its row of the page table.
  const int jpage = (jend > 0 ? j0 : 0) >> K.pw_log2;
  const T* pgk[NKS];
  bool okk[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int g = min((ks * KSTEP + qq * EPV) >> 4, G - 1);
    pgk[ks] = page_base<E>(K, one_page ? cld(P.b_pages + bbase + g * ncolB + jpage) : 0, okk[ks]);
  }
  auto load_part = [&](int part, uint4 (&bv)[CT][NKS], uint4 (&ybv)[ROUNDS], bool (&okc)[CT][NKS]) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      // columns past the block are clamped to its last column (never stored)
      const int j = j0 + min(part * PART + ct * 16 + li, jend - 1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int k0 = ks * KSTEP + qq * EPV;
        const int g = min(k0 >> 4, G - 1);
        // unconditional (see load_b's note); a K step wholly past the rank
        // reads the last group and is skipped at the product
        bool ok = okk[ks];
        const T* pg = one_page ? pgk[ks] : page_base<E>(K, P.b_pages[bbase + g * ncolB + (j >> K.pw_log2)], ok);
        bv[ct][ks] = ldg16(pg + b_off(j & (pw - 1), k0 & 15, pw, r - 16 * g > 8));
        okc[ct][ks] = ok;
      }
    }
    const int col = min(part * PART + ch * EPC, jend - EPC);  // jend is a multiple of 8
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) ybv[rd] = ldg16(Yb + yrow[rd] * P.ldyb + j0 + col);
  };
  uint4 bcur[CT][NKS], bnext[CT][NKS];
  uint4 ycur[ROUNDS], ynext[ROUNDS];
  bool okcur[CT][NKS], oknext[CT][NKS];
  const bool active = jend > 0;  // the wave has columns in this item
  const int np = active ? ceil_div_i(jend, PART) : 0;
  // The tile's v is staged while the first part's B and Y_base are in
  // flight.  Vector memory returns in issue order, so when the tile needs
  // one round of staging loads (at most two entries per thread), that round
  // goes out first and is summed without waiting for the part's loads.
  const int ne = nt * r;
  const float* vsrc = P.v + voff + (int64_t)tb * r;
  const bool early = ne <= 2 * kThreads;
  RowStage<2, 8> st0;
  if (early) {
    st0.acc[0] = st0.acc[1] = 0.0f;
    row_load<kThreads, 2, 8, CO>(K, P, vsrc, 0, 0, ne, threadIdx.x, st0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (active) load_part(0, bcur, ycur, okcur);
  __builtin_amdgcn_sched_barrier(0);
  if (early) {
    row_add<2, 8>(st0);
    for (int q = 8; q < P.nv; q += 8) {
      row_load<kThreads, 2, 8, CO>(K, P, vsrc, q, 0, ne, threadIdx.x, st0);
      row_add<2, 8>(st0);
    }
    row_store<kThreads, 2, 8>(st0, 0, ne, r, rs, vs, threadIdx.x);
    stage_v_pad<kThreads>(r, nt, vs, threadIdx.x);
  } else {
    stage_v_rows<kThreads, CO>(K, P, voff, r, tb, nt, vs, threadIdx.x);
  }
  __syncthreads();
  next();  // the block's next item, requested while this one runs
  uint4 vv[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int k0 = ks * KSTEP + qq * EPV;
    vv[ks] = (li < nt && k0 < r) ? pack_operand(vs + li * rs + k0, EPV, E()) : zero4();
  }
  for (int part = 0; part < np; ++part) {
    if (part + 1 < np) load_part(part + 1, bnext, ynext, oknext);
    f4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      acc[ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks * KSTEP >= r) continue;  // uniform
        // ranks past r in this lane's vector, and pages outside the pool, are
        // masked here, at the use
        uint4 w = (ks + 1) * KSTEP > r ? keep_first(bcur[ct][ks], r - (ks * KSTEP + qq * EPV), E()) : bcur[ct][ks];
        if (!okcur[ct][ks]) w = zero4();
        mma(acc[ct], w, vv[ks], E());
      }
    }
    // C[col][token] -> LDS token rows -> 16-byte chunks of Y rows
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) *reinterpret_cast<f4*>(cw + li * LDC + ct * 16 + qq * 4) = acc[ct];
    wave_sync();
    // Every lane stores, so the loop has no conditional store: a store
    // skipped on some paths makes the compiler wait for every store at the
    // part's end (vmcnt(0)) before the next part's operands count as
    // arrived.  A lane past the tile's tokens takes the last token's row and
    // a lane past the wave's columns the last chunk (as its Y_base load
    // did): its value and address are those of a lane inside, so the
    // duplicate writes are identical.
    const int colp = min(part * PART + ch * EPC, jend - EPC);  // jend is a multiple of 8
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      const int tk = min(rd * TPR + lane / CPR, nt - 1);
      {
        const float* c = cw + tk * LDC + (colp - part * PART);
        uint4 out;
        if constexpr (EPC == 8) {
          const f4 c0 = *reinterpret_cast<const f4*>(c), c1 = *reinterpret_cast<const f4*>(c + 4);
          const uint4 yb = ycur[rd];
          out.x = pack_bf2(bf_lo(yb.x) + scale * c0[0], bf_hi(yb.x) + scale * c0[1]);
          out.y = pack_bf2(bf_lo(yb.y) + scale * c0[2], bf_hi(yb.y) + scale * c0[3]);
          out.z = pack_bf2(bf_lo(yb.z) + scale * c1[0], bf_hi(yb.z) + scale * c1[1]);
          out.w = pack_bf2(bf_lo(yb.w) + scale * c1[2], bf_hi(yb.w) + scale * c1[3]);
        } else {
          const f4 c0 = *reinterpret_cast<const f4*>(c);
          const uint4 yb = ycur[rd];
          out = make_uint4(__float_as_uint(__uint_as_float(yb.x) + scale * c0[0]),
                           __float_as_uint(__uint_as_float(yb.y) + scale * c0[1]),
                           __float_as_uint(__uint_as_float(yb.z) + scale * c0[2]),
                           __float_as_uint(__uint_as_float(yb.w) + scale * c0[3]));
        }
        stg16_nt(Y + yrow[rd] * P.ldy + j0 + colp, out);
      }
    }
    wave_sync();  // the rows are rewritten by the next part
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        bcur[ct][ks] = bnext[ct][ks];
        okcur[ct][ks] = oknext[ct][ks];
      }
    }
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) ycur[rd] = ynext[rd];
  }
}

// MBGMM expand item (one block): (segment, 16-token tile, 4*wc columns).  The
// block stages v of the tile once into shared LDS rows; wave w then produces
// columns [w*wc, (w+1)*wc) of the item.  next() runs once v is staged,
// publish() just before the block's last barrier of the item.
template <class E, bool WIDE, bool CO, class Next, class Publish>
__device__ __forceinline__ void expand_mfma(const KArgs& K, const KProj& P, int jb, int wc, int4 d0, int4 d1,
                                            int local, float* vs, float* cw, int wave, int lane, Next&& next,
                                            Publish&& publish) {
  constexpr int KSTEP = 4 * E::kEpv;
  constexpr int MAXKS = LORA_MAX_RANK / KSTEP;
  const int a = d0.x, r = d0.y;
  const int tb = local * kMfmaExpandTokens;
  const int t0 = d0.z + tb;
  const int nt = min(kMfmaExpandTokens, d0.w - tb);
  const float scale = __int_as_float(d1.w) / (float)r;
  const int j0 = (jb * kWaves + wave) * wc;
  const int jend = min(wc, P.d_out - j0);  // <= 0: no columns for this wave (it still stages v)
  // K steps past the rank are skipped inside the body, so two variants cover
  // every rank; the choice is the same for the whole block (one segment)
  const int nks = ceil_div_i(r, KSTEP);
  if (WIDE && nks <= MAXKS / 4)  // bf16: one K step (r <= 32), so twice the columns per part
    expand_mfma_body<E, MAXKS / 4, WIDE, CO>(K, P, j0, jend, wc, a, r, t0, nt, scale, vs, cw, d1.x, tb, lane, next);
  else if (nks <= MAXKS / 2)
    expand_mfma_body<E, MAXKS / 2, WIDE, CO>(K, P, j0, jend, wc, a, r, t0, nt, scale, vs, cw, d1.x, tb, lane, next);
  else expand_mfma_body<E, MAXKS, WIDE, CO>(K, P, j0, jend, wc, a, r, t0, nt, scale, vs, cw, d1.x, tb, lane, next);
  publish();
  __syncthreads();  // the rows are restaged by the block's next item
}

// Item index i of the MBGMM expand list -> (projection p, column block jb,
// item u of the segment tables); nb(p) is the column blocks of projection p.
__device__ __forceinline__ void expand_mfma_item(const KArgs& K, int i, int wc, int Um, int& p, int& jb, int& u) {
  int rem = i;
  p = 0;
  int nb = ceil_div_i(K.p[0].d_out, kWaves * wc);
  while (rem >= nb * Um) {
    rem -= nb * Um;
    ++p;
    nb = ceil_div_i(K.p[p].d_out, kWaves * wc);
  }
  jb = rem / Um;
  u = rem - jb * Um;
}

// Rows of tokens without an adapter: Y = Y_base (only when Y is not Y_base),
// kCopyTokens rows x one column block per item.
template <class E>
__device__ __forceinline__ void expand_copy(const KArgs& K, const KProj& P, int jb, int chunk, int t_valid, int nT,
                                            int lane) {
  typedef typename E::T T;
  constexpr int CPL = 4 / (int)sizeof(T);
  constexpr int SUBW = 64 * CPL;
  const int t_beg = t_valid + chunk * kCopyTokens;
  const int t_end = min(nT, t_beg + kCopyTokens);
  const T* Yb = reinterpret_cast<const T*>(P.Yb);
  T* Y = reinterpret_cast<T*>(P.Y);
  for (int i = t_beg; i < t_end; ++i) {
    const int64_t row = cld(K.perm + i);
#pragma unroll
    for (int sb = 0; sb < kValuSubBlocks; ++sb) {
      const int j = (jb * kValuSubBlocks + sb) * SUBW + lane * CPL;
      if (j < P.d_out) stg4_nt(Y + row * P.ldy + j, load_dword(Yb + row * P.ldyb + j));
    }
  }
}

// WIDE: pages hold at least one whole MBGMV column block (expand_cols), so
// every page lookup of an item is wave-uniform; chosen by the host from the
// page width (the other instantiation looks pages up per lane).
// The MBGMV expand items and copies of rows without an adapter of one wave,
// in the order `walk` gives them.
template <class E, bool WIDE, bool CO, class Walk>
__device__ __forceinline__ void expand_valu_items(const KArgs& K, Walk walk, const PlanCounts& pc, int Uv, int ncopy,
                                                  float* vs, int lane, PhaseWait& sw) {
  const int i0 = walk.first();
  if (i0 < 0) return;
  const FastDiv dUv(Uv > 0 ? Uv : 1);  // (Uv = 0: only copy items, divided by Up)
  ValuItem cur = fetch_valu_item<E>(K, i0, Uv, ncopy, dUv);
  for (;;) {
    walk.issue();
    int ni = -1;
    ValuItem nxt;
    if (cur.copy) {
      expand_copy<E>(K, K.p[cur.p], cur.jb, cur.local, pc.t_valid, pc.T, lane);
      ni = walk.resolve();
      if (ni >= 0) nxt = fetch_valu_item<E>(K, ni, Uv, ncopy, dUv);
    } else {
      const bool fresh = !CO || sw.ready();
      expand_valu_body<E, WIDE, CO>(K, K.p[cur.p], cur, vs, lane, sw, fresh, [&]() {
        ni = walk.resolve();
        if (ni >= 0) nxt = fetch_valu_item<E>(K, ni, Uv, ncopy, dUv);
      });
      wave_sync();
    }
    if (ni < 0) break;
    cur = nxt;
  }
}

// vs_all: per-wave LDS rows (MBGMV staging, MBGMM output tiles) and, in row
// kWaves, the block's staged v tile of an MBGMM item.
template <class E, bool WIDE, bool CO>
__device__ __forceinline__ void expand_phase(const KArgs& K, const PlanCounts& pc,
                                             float (*vs_all)[kExpandRowFloats], PhaseWait& sw) {
  const int t_valid = pc.t_valid;
  const int Um = pc.S > 0 ? pc.exp_m : 0;
  const int Uv = pc.S > 0 ? pc.exp_v : 0;
  const int ncopy = ceil_div_i(pc.T - t_valid, kCopyTokens);
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float* vs = vs_all[wave];
  // MBGMM items first (whole-block items), then MBGMV items and the copies of
  // rows without an adapter (one wave each); each path walks its own item
  // list.  (Covering the grid twice over with MBGMM items, with narrower
  // items, left each block two or three items in a row, each one memory
  // round trip.)
  const int grid = gridDim.x, block = blockIdx.x;
  int total_v = 0;
  for (int p = 0; p < K.np; ++p) total_v += K.p[p].njs * (Uv + (K.p[p].Y != K.p[p].Yb ? ncopy : 0));
  int total = 0, wc = 0;
  if (Um > 0) wc = expand_mfma_cols(K.np, [&](int p) { return K.p[p].d_out; }, K.pw_log2, Um, grid, total);
  // The expand kernel with at least kQueueItems MBGMM items per work-group
  // of the grid (prefill batches) takes them from per-XCD queues; otherwise
  // (and always in the apply kernel, whose phase barrier holds the grid) the
  // items of an XCD's part go round robin.
  constexpr int kQueueItems = 3;
  if (CO || !(Um > 0 && 8LL * total >= total_v && total >= kQueueItems * grid)) {
    // each XCD takes a contiguous part of the list (for a decode batch,
    // whole column blocks: every XCD reads its own columns of B)
    const ExpandSplit es = expand_walk_split(total, total_v, grid, block);
    if (Um > 0) {
      // apply kernel: the block's MBGMM items read v from their start (the
      // tile's staging overlaps its first B loads), so their waves wait for
      // the phase barrier before the first one
      if constexpr (CO) {
        if (es.first < es.end_m) sw.wait(K);
      }
      for (int i = es.first; i < es.end_m; i += es.step) {
        int p, jb, u;
        expand_mfma_item(K, i, wc, Um, p, jb, u);
        const int s = cld(K.exp_item_m + u);
        const int4 d0 = cld4(K.seg_desc + 2 * s), d1 = cld4(K.seg_desc + 2 * s + 1);
        expand_mfma<E, WIDE, CO>(K, K.p[p], jb, wc, d0, d1, u - d1.z, vs_all[kWaves], vs_all[wave], wave, lane,
                                 [] {}, [] {});
      }
    }
    expand_valu_items<E, WIDE, CO>(K, StaticWalk(total_v, es.Gm * kWaves, es.R, wave), pc, Uv, ncopy, vs, lane, sw);
  } else {
    // Queues: the items go to the XCDs in blocks of consecutive items dealt
    // round robin (an eighth of the list per XCD would tie an XCD's load to
    // the ranks of the segments there).  Work-group beta of an XCD starts
    // with its item beta; later items come from the XCD's queue, one at a
    // time per work-group, so that blocks that drew slow items (high rank)
    // take fewer of them.  Thread 0 takes the next ticket while the current
    // item runs and hands it to the block through LDS.  Every work-group of
    // the grid takes part (Gm = the XCD's work-groups).
    const QueueSplit qs = expand_queue_split(total, total_v, grid, block);
    if (qs.beta < qs.Gm) {
      __shared__ int ticket;
      const int sh = xcd_shift(grid);
      int* tq = K.sync + queue_line(qs.x);
      int* dq = K.sync + queue_line(8 + qs.x);
      // The XCD's last Gm items (about one per block: the last round) are
      // handed out in halves of their columns, so that the blocks finish
      // within about half an item of each other: tickets [0, split) are
      // items, tickets from split are half items.
      const int split = qs.m - min(qs.Gm, qs.m);
      const int tickets = 2 * qs.m - split;
      int t = qs.beta;
      int tk = 0;
      while (t < tickets) {
        int p, jb, u;
        const int h = t < split ? -1 : (t - split) & 1;
        const int li = t < split ? t : split + ((t - split) >> 1);
        expand_mfma_item(K, xcd_block_item(li, qs.x, sh), wc, Um, p, jb, u);
        const int s = cld(K.exp_item_m + u);
        const int4 d0 = cld4(K.seg_desc + 2 * s), d1 = cld4(K.seg_desc + 2 * s + 1);
        // half h of column block jb at width wc is column block 2 jb + h at wc / 2
        expand_mfma<E, WIDE, CO>(
            K, K.p[p], h < 0 ? jb : 2 * jb + h, h < 0 ? wc : wc >> 1, d0, d1, u - d1.z, vs_all[kWaves], vs_all[wave],
            wave, lane,
            [&] {
              if (threadIdx.x == 0)
                tk = qs.Gm + __hip_atomic_fetch_add(tq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            },
            [&] {
              if (threadIdx.x == 0) ticket = tk;
            });
        t = uniform(ticket);  // written before the item's last barrier
      }
      // every work-group of the XCD's set arrives once, after its last
      // ticket (or none, past the XCD's items); the last one finds no block
      // still taking tickets
      if (threadIdx.x == 0 &&
          __hip_atomic_fetch_add(dq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == qs.Gm - 1) {
        __hip_atomic_store(tq, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dq, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    expand_valu_items<E, WIDE, CO>(K, StaticWalk(total_v, qs.Gm * kWaves, qs.R, wave), pc, Uv, ncopy, vs, lane, sw);
  }
}

template <class E, bool WIDE>
__global__ __launch_bounds__(kThreads, E::kExpandBlocks) void expand_kernel(KArgs) {
  const KArgs& K = kernel_args();
  __shared__ __attribute__((aligned(16))) float vs_all[kWaves + 1][kExpandRowFloats];
  const PlanCounts pc = read_counts(K);
  if (!pc.ok) return;
  PhaseWait sw{nullptr, 0, 0, true};
  expand_phase<E, WIDE, false>(K, pc, vs_all, sw);
}

// ================================================================ apply
// The whole branch for a launch group in one launch ([MLSP] "Custom CUDA
// Kernels: SGMV and MBGMV": fused operations rather than a launch per step).
// Every wave runs its shrink items (partial sums of v written with
// agent-coherent stores), arrives at the phase barrier, then runs its expand
// items; before its first read of v it waits until every work-group of the
// grid has arrived.  The waves of a work-group arrive through an LDS counter,
// the last one through a per-XCD counter, the last work-group of an XCD
// through the count of finished XCDs (the waited-on counter), and the very
// last arrival flips the epoch.  Items, their order and their arithmetic are
// those of shrink_kernel followed by expand_kernel, so Y is bit-identical.
// The grid is sized from this kernel's occupancy so that it is resident at
// once; a wave that still finds the barrier closed after the bound gives up
// (LORA_FLAG_SYNC).
template <class E, bool WS, bool WE>
__global__ __launch_bounds__(kThreads, E::kExpandBlocks) void apply_kernel(KArgs) {
  const KArgs& K = kernel_args();
  __shared__ __attribute__((aligned(16))) float vs_all[kWaves + 1][kExpandRowFloats];
  __shared__ int arrived;
  const PlanCounts pc = read_counts(K);
  if (!pc.ok) return;
  // with no adapter rows (only copies of Y_base) there is nothing to wait for
  const bool sync = pc.S > 0;
  const int epoch = sync ? uniform(__hip_atomic_load(K.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) : 0;
  int* bank = K.sync + sync_bank(epoch & 1);
  if (sync) {  // the other bank, for the next launch: two words of each of its lines
    int* other = K.sync + sync_bank((epoch & 1) ^ 1);
    for (int l = blockIdx.x * kThreads + threadIdx.x; l < 2 * kSyncBankLines; l += gridDim.x * kThreads)
      __hip_atomic_store(other + (l >> 1) * kSyncLine + (l & 1), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == 0) arrived = 0;
  __syncthreads();
  shrink_phase<E, WS, true>(K, pc);
  // Arrival.  The partial sums were written through to the coherence point
  // (agent-scope stores); waiting for every outstanding access of the wave
  // makes them complete before the wave is counted.
  __builtin_amdgcn_s_waitcnt(0);
  const int nx = xcd_count(gridDim.x);
  if (sync && (threadIdx.x & 63) == 0 && atomicAdd(&arrived, 1) == kWaves - 1) {
    if (__hip_atomic_fetch_add(bank + (blockIdx.x % nx) * kSyncLine, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            (int)gridDim.x / nx - 1 &&
        __hip_atomic_fetch_add(bank + 8 * kSyncLine, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nx - 1)
      __hip_atomic_store(K.sync, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  PhaseWait sw{bank + 8 * kSyncLine, nx + K.wait_bias, K.wait_ticks, !sync};
  expand_phase<E, WE, true>(K, pc, vs_all, sw);
}

// ================================================================ segments
__device__ __forceinline__ bool token_valid(int id, int N, const int32_t* rank) {
  if (id < 0 || id >= N) return false;
  const int r = rank[id];
  return r >= 1 && r <= LORA_MAX_RANK;
}

// Per-chunk histogram: hist[c][a] = tokens of chunk c on adapter a;
// hist[c][N] = base-model tokens (id -1); hist[c][N+1] = other invalid.
// Lanes with equal keys are merged before the atomic add.
__global__ __launch_bounds__(kThreads) void seg_hist_kernel(const int32_t* ids, int T, int N,
                                                            const int32_t* rank, int32_t* hist) {
  int32_t* row = hist + (int64_t)blockIdx.x * (N + 2);
  for (int i = threadIdx.x; i < N + 2; i += kThreads) row[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  for (int base = blockIdx.x * kSegChunk; base < min(T, (blockIdx.x + 1) * kSegChunk); base += kThreads) {
    const int t = base + threadIdx.x;
    const bool in = t < T && t < (blockIdx.x + 1) * kSegChunk;
    int key = -1;
    if (in) {
      const int id = ids[t];
      key = token_valid(id, N, rank) ? id : (id == -1 ? N : N + 1);
    }
    uint64_t active = __ballot(in);
    while (active) {
      const int leader = __builtin_ctzll(active);
      const int lk = __shfl(key, leader);
      const uint64_t same = __ballot(in && key == lk) & active;
      if (lane == leader) atomicAdd(&row[lk], (int)__popcll(same));
      active &= ~same;
    }
  }
}

// Block-wide exclusive scan of one int per thread (kSegScanThreads threads);
// *total receives the block sum.  wsum has kSegScanThreads/64 + 1 entries.
__device__ int block_exclusive_scan(int x, int* wsum, int* total) {
  constexpr int NW = kSegScanThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int v = wsum[w];
      wsum[w] = run;
      run += v;
    }
    wsum[NW] = run;
  }
  __syncthreads();
  const int res = incl - x + wsum[wave];
  *total = wsum[NW];
  __syncthreads();  // wsum is reused by the next call
  return res;
}

// One work-group: column prefix of the chunk histograms, segment arrays,
// ragged v offsets, work plan, counters.
__global__ __launch_bounds__(kSegScanThreads) void seg_scan_kernel(int T, int N, int nchunk,
                                                                   const int32_t* rank, const float* alpha,
                                                                   int32_t* hist, SegOut out) {
  __shared__ int wsum[kSegScanThreads / 64 + 1];
  __shared__ int carry[8];
  if (threadIdx.x < 8) carry[threadIdx.x] = 0;
  __syncthreads();
  const int W = N + 2;
  for (int base = 0; base < N; base += kSegScanThreads) {
    const int a = base + threadIdx.x;
    int cnt = 0;
    if (a < N) {
      // prefix within this adapter's tokens over the chunks; each batch's
      // loads are issued before its stores, so a long batch (many chunks)
      // costs one memory round trip per 16 chunks, not one per chunk
      for (int c0 = 0; c0 < nchunk; c0 += 16) {
        int h[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) h[j] = c0 + j < nchunk ? hist[(int64_t)(c0 + j) * W + a] : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (c0 + j < nchunk) hist[(int64_t)(c0 + j) * W + a] = cnt;
          cnt += h[j];
        }
      }
    }
    const int r = (a < N && cnt > 0) ? rank[a] : 0;
    const bool has = cnt > 0;
    // {tokens, segments, v entries, MBGMM shrink, MBGMV shrink, MBGMM expand, MBGMV expand}
    const int vals[7] = {cnt, has ? 1 : 0, cnt * r, has ? shrink_items_mfma(cnt, r) : 0,
                         has ? shrink_items_valu(cnt, r) : 0, has ? expand_items_mfma(cnt) : 0,
                         has ? expand_items_valu(cnt, r) : 0};
    int pre[7], tots[7];
#pragma unroll
    for (int f = 0; f < 7; ++f) {
      pre[f] = block_exclusive_scan(vals[f], wsum, &tots[f]) + carry[f];
    }
    if (a < N && has) {
      const int si = pre[1];
      const bool mf = is_mfma_segment(cnt);
      out.seg_adapter[si] = a;
      out.seg_indptr[si] = pre[0];
      out.v_indptr[si] = pre[2];
      const int4 d0 = make_int4(a, r, pre[0], cnt);
      const int4 d1 = make_int4(pre[2], mf ? pre[3] : pre[4], mf ? pre[5] : pre[6], __float_as_int(alpha[a]));
      int4* desc = reinterpret_cast<int4*>(out.seg_desc) + 2 * si;
      desc[0] = d0;
      desc[1] = d1;
      if (mf) {
        for (int i = 0; i < vals[3]; ++i) out.shr_item_m[pre[3] + i] = si;
        for (int i = 0; i < vals[5]; ++i) out.exp_item_m[pre[5] + i] = si;
      } else {  // MBGMV tables: the descriptor per item
        static_assert(kValuItemInts == 8, "two int4 per MBGMV item");
        int4* sv = reinterpret_cast<int4*>(out.shr_item_v) + 2 * pre[4];
        for (int i = 0; i < vals[4]; ++i) {
          sv[2 * i] = d0;
          sv[2 * i + 1] = d1;
        }
        int4* ev = reinterpret_cast<int4*>(out.exp_item_v) + 2 * pre[6];
        for (int i = 0; i < vals[6]; ++i) {
          ev[2 * i] = d0;
          ev[2 * i + 1] = d1;
        }
      }
      for (int c0 = 0; c0 < nchunk; c0 += 16) {
        int h[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) h[j] = c0 + j < nchunk ? hist[(int64_t)(c0 + j) * W + a] : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (c0 + j < nchunk) hist[(int64_t)(c0 + j) * W + a] = h[j] + pre[0];
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int f = 0; f < 7; ++f) carry[f] += tots[f];
    }
    __syncthreads();
  }
  // excluded tokens: chunk-ordered offsets after the grouped ones
  if (threadIdx.x == 0) {
    const int S = carry[1], t_valid = carry[0];
    out.seg_indptr[S] = t_valid;
    out.v_indptr[S] = carry[2];
    int run = t_valid, n_invalid = 0;
    for (int c0 = 0; c0 < nchunk; c0 += 16) {
      int base_only[16], bad[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        base_only[j] = c0 + j < nchunk ? hist[(int64_t)(c0 + j) * W + N] : 0;
        bad[j] = c0 + j < nchunk ? hist[(int64_t)(c0 + j) * W + N + 1] : 0;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (c0 + j < nchunk) hist[(int64_t)(c0 + j) * W + N] = run;
        run += base_only[j] + bad[j];
        n_invalid += bad[j];
      }
    }
    out.counts[kCountS] = S;
    out.counts[kCountInvalid] = n_invalid;
    out.counts[kCountTValid] = t_valid;
    out.counts[kCountVTotal] = carry[2];
    out.counts[kCountShrinkMfma] = carry[3];
    out.counts[kCountShrinkValu] = carry[4];
    out.counts[kCountExpandMfma] = carry[5];
    out.counts[kCountExpandValu] = carry[6];
    for (int i = kCountFlags; i < kNumCounts; ++i) out.counts[i] = 0;
    out.counts[kCountT] = T;
    out.counts[kCountCheck] = segments_check_word(T);
  }
  // the apply kernel's phase-barrier counters start from zero for this batch
  for (int i = threadIdx.x; i < kSyncInts; i += kSegScanThreads) out.sync[i] = 0;
}

// Stable scatter: each block sorts its chunk's (adapter, position) keys in
// LDS (bitonic) and writes perm[]; ties keep token order, so the whole
// grouping equals a stable sort by adapter id.
__global__ __launch_bounds__(kSegChunk) void seg_scatter_kernel(const int32_t* ids, int T, int N,
                                                                const int32_t* rank,
                                                                const int32_t* hist, int32_t* perm) {
  __shared__ uint32_t keys[kSegChunk];
  const int c = blockIdx.x;
  const int i = threadIdx.x;
  const int t = c * kSegChunk + i;
  // class of tokens without an adapter; kept below 0x3FFFFF so that no real
  // key (class << 10 | position) can equal the 0xFFFFFFFF padding key
  constexpr uint32_t kExcluded = 0x3FFFFEu;
  uint32_t key = 0xFFFFFFFFu;
  if (t < T) {
    const int id = ids[t];
    key = ((token_valid(id, N, rank) ? (uint32_t)(id + 1) : kExcluded) << 10) | (uint32_t)i;
  }
  keys[i] = key;
  __syncthreads();
  for (int k = 2; k <= kSegChunk; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int ixj = i ^ j;
      if (ixj > i) {
        const uint32_t x = keys[i], y = keys[ixj];
        const bool up = (i & k) == 0;
        if ((x > y) == up) {
          keys[i] = y;
          keys[ixj] = x;
        }
      }
      __syncthreads();
    }
  }
  const uint32_t kk = keys[i];
  if (kk == 0xFFFFFFFFu) return;
  const uint32_t hi = kk >> 10;
  // first position of this key class in the sorted chunk
  int lo = 0, hi_i = i;
  const uint32_t first = hi << 10;
  while (lo < hi_i) {
    const int mid = (lo + hi_i) >> 1;
    if (keys[mid] < first) lo = mid + 1; else hi_i = mid;
  }
  const int within = i - lo;
  const int W = N + 2;
  const int dst = (hi == kExcluded) ? hist[(int64_t)c * W + N] + within
                                    : hist[(int64_t)c * W + (int)(hi - 1)] + within;
  perm[dst] = c * kSegChunk + (int)(kk & 1023u);
}

// ================================================================ launchers
static hipError_t launch_err() { return hipGetLastError(); }

hipError_t launch_build_segments(const int32_t* ids, int T, int N, const int32_t* rank, const float* alpha,
                                 int32_t* hist, const SegOut& out, hipStream_t stream) {
  const int nchunk = ceil_div_i(T, kSegChunk);
  if (nchunk > 0) {
    seg_hist_kernel<<<nchunk, kThreads, 0, stream>>>(ids, T, N, rank, hist);
    if (hipError_t e = launch_err()) return e;
  }
  seg_scan_kernel<<<1, kSegScanThreads, 0, stream>>>(T, N, nchunk, rank, alpha, hist, out);
  if (hipError_t e = launch_err()) return e;
  if (nchunk > 0) {
    seg_scatter_kernel<<<nchunk, kSegChunk, 0, stream>>>(ids, T, N, rank, hist, out.perm);
    if (hipError_t e = launch_err()) return e;
  }
  return hipSuccess;
}

hipError_t launch_shrink(const KArgs& K, int dtype, int grid, hipStream_t stream) {
  const bool wide = (1 << K.pw_log2) >= kKSlice;
  if (dtype == LORA_DTYPE_BF16) {
    if (wide) shrink_kernel<Bf16, true><<<grid, kThreads, 0, stream>>>(K);
    else shrink_kernel<Bf16, false><<<grid, kThreads, 0, stream>>>(K);
  } else {
    if (wide) shrink_kernel<F32, true><<<grid, kThreads, 0, stream>>>(K);
    else shrink_kernel<F32, false><<<grid, kThreads, 0, stream>>>(K);
  }
  return launch_err();
}

hipError_t launch_expand(const KArgs& K, int dtype, int grid, hipStream_t stream) {
  const bool bf16 = dtype == LORA_DTYPE_BF16;
  const bool wide = (1 << K.pw_log2) >= expand_cols(bf16);
  if (bf16) {
    if (wide) expand_kernel<Bf16, true><<<grid, kThreads, 0, stream>>>(K);
    else expand_kernel<Bf16, false><<<grid, kThreads, 0, stream>>>(K);
  } else {
    if (wide) expand_kernel<F32, true><<<grid, kThreads, 0, stream>>>(K);
    else expand_kernel<F32, false><<<grid, kThreads, 0, stream>>>(K);
  }
  return launch_err();
}

hipError_t launch_apply(const KArgs& K, int dtype, int grid, hipStream_t stream) {
  const bool bf16 = dtype == LORA_DTYPE_BF16;
  const bool ws = (1 << K.pw_log2) >= kKSlice, we = (1 << K.pw_log2) >= expand_cols(bf16);
  if (bf16) {  // both page-width thresholds are 512 columns
    if (ws) apply_kernel<Bf16, true, true><<<grid, kThreads, 0, stream>>>(K);
    else apply_kernel<Bf16, false, false><<<grid, kThreads, 0, stream>>>(K);
  } else {
    if (ws) apply_kernel<F32, true, true><<<grid, kThreads, 0, stream>>>(K);
    else if (we) apply_kernel<F32, false, true><<<grid, kThreads, 0, stream>>>(K);
    else apply_kernel<F32, false, false><<<grid, kThreads, 0, stream>>>(K);
  }
  return launch_err();
}

// Work-groups per CU of each kernel.  The apply kernel's grid must be
// resident at once, so its count is the minimum over its instantiations.
hipError_t occupancy(int dtype, int* shrink_blocks, int* expand_blocks, int* apply_blocks) {
  hipError_t e;
  int a0 = 0, a1 = 0, a2 = 0;
  if (dtype == LORA_DTYPE_BF16) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(shrink_blocks, shrink_kernel<Bf16, true>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(expand_blocks, expand_kernel<Bf16, true>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a0, apply_kernel<Bf16, true, true>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a1, apply_kernel<Bf16, false, false>, kThreads, 0);
    a2 = a1;
  } else {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(shrink_blocks, shrink_kernel<F32, true>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(expand_blocks, expand_kernel<F32, true>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a0, apply_kernel<F32, true, true>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a1, apply_kernel<F32, false, true>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a2, apply_kernel<F32, false, false>, kThreads, 0);
  }
  *apply_blocks = min(a0, min(a1, a2));
  return e;
}

}  // namespace lora
