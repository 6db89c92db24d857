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
//       segments take the MBGMV path (vector ALU, token rows staged in LDS,
//       wavefront reductions); long ones the MBGMM path (16x16 MFMA tiles).
//       Each work item covers one 1024-column slice of d_in and writes a
//       partial v; the expand sums the slices in ascending order, so every
//       result is bitwise deterministic.
//   expand_kernel
//       Y = Y_base + (alpha/r) v B ([MLSP] SGMV expand), same two paths.
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
};
struct F32 {
  typedef float T;
  static constexpr int kEpv = 4;
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
__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

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

// Load n (< kEpv) leading elements of a vector, zero the rest; never touches
// the elements beyond n (page padding is not read).
template <class E>
__device__ __forceinline__ uint4 load_partial(const typename E::T* p, int n) {
  typename E::T e[E::kEpv];
#pragma unroll
  for (int i = 0; i < E::kEpv; ++i) e[i] = i < n ? p[i] : (typename E::T)0;
  return __builtin_bit_cast(uint4, e);
}

__device__ __forceinline__ float to_f(uint16_t h) { return bf_to_f(h); }
__device__ __forceinline__ float to_f(float f) { return f; }
__device__ __forceinline__ void from_f(uint16_t* p, float f) { *p = f_to_bf(f); }
__device__ __forceinline__ void from_f(float* p, float f) { *p = f; }

// ------------------------------------------------------------ pool access
template <class E>
__device__ __forceinline__ const typename E::T* page_ptr(const KArgs& K, int page) {
  if ((unsigned)page >= (unsigned)K.num_pages) {
    atomicOr(&K.counts[LORA_COUNT_FLAGS], LORA_FLAG_PAGE_RANGE);
    return nullptr;
  }
  return reinterpret_cast<const typename E::T*>(K.pool) + ((int64_t)page << (K.pw_log2 + 4));
}

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
// hold the sum over all 64 lanes of value i (32 cross-lane exchanges
// instead of 32 full butterflies).
__device__ __forceinline__ float wave_reduce_scatter32(float (&v)[32], int lane) {
#pragma unroll
  for (int step = 0; step < 5; ++step) {
    const int half = 16 >> step;
    const int mask = 32 >> step;
    const bool upper = (lane & mask) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? v[i] : v[i + half];
      const float keep = upper ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, mask);
    }
  }
  return v[0] + __shfl_xor(v[0], 1);
}

// XCD-aware item walk: item range [0, total) is cut into 8 contiguous parts,
// part x served by the work-groups with blockIdx.x % 8 == x.
struct ItemWalk {
  int i, end, stride;
  __device__ ItemWalk(int total) {
    const int nx = (gridDim.x % 8 == 0) ? 8 : 1;
    const int x = blockIdx.x % nx;
    const int per = gridDim.x / nx;
    const int lo = (int)(((int64_t)total * x) / nx);
    end = (int)(((int64_t)total * (x + 1)) / nx);
    i = lo + (int)(blockIdx.x / nx);
    stride = per;
  }
};

// ================================================================ shrink
// MBGMV item: (segment s, rank group g, token chunk of <= 8 tokens, slice q).
// The chunk's token rows (the gathered activations of [MLSP] SGMV) are staged
// in LDS; wave w takes page rows 4w..4w+3 of the 16-rank group, each lane
// streams 16-byte vectors of those rows (a wave reads 1 KiB contiguous per
// row and instruction) and the 64 lanes' partial dot products are reduced
// across the wave.
template <class E>
__device__ void shrink_valu(const KArgs& K, const KProj& P, int q, int s, int local, char* smem) {
  typedef typename E::T T;
  constexpr int EPV = E::kEpv;
  constexpr int NCH = kKSlice / (64 * EPV);
  constexpr int NV = kValuTokens;
  const int a = K.seg_adapter[s];
  const int r = K.rank[a];
  const int t0 = K.seg_indptr[s];
  const int n = K.seg_indptr[s + 1] - t0;
  const int nch = ceil_div_i(n, NV);
  const int g = local / nch;
  const int tb = (local - g * nch) * NV;
  const int nt = min(NV, n - tb);
  const int col0 = q * kKSlice;
  const int ncols = min(kKSlice, P.d_in - col0);
  const int pw = 1 << K.pw_log2;

  T* xs = reinterpret_cast<T*>(smem);  // [NV][kKSlice]
  constexpr int VPR = kKSlice / EPV;
  for (int idx = threadIdx.x; idx < nt * VPR; idx += kThreads) {
    const int tt = idx / VPR;
    const int c = (idx - tt * VPR) * EPV;
    uint4 val = zero4();
    if (c < ncols) val = ldg16(reinterpret_cast<const T*>(P.X) + (int64_t)K.perm[t0 + tb + tt] * P.ldx + col0 + c);
    *reinterpret_cast<uint4*>(xs + tt * kKSlice + c) = val;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = min(16, r - g * 16);
  const int row0 = wave * 4;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.0f;
  if (row0 < rows) {
    const int ncolA = (P.d_in + pw - 1) >> K.pw_log2;
    const int slot0 = P.a_indptr[a] + g * ncolA;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = i * 64 * EPV + lane * EPV;
      if (c < ncols) {
        const int col = col0 + c;
        const T* pg = page_ptr<E>(K, P.a_pages[slot0 + (col >> K.pw_log2)]);
        uint4 w[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          w[rr] = (pg != nullptr && row0 + rr < rows) ? ldg16(pg + (row0 + rr) * pw + (col & (pw - 1))) : zero4();
        uint4 x[NV];
#pragma unroll
        for (int tt = 0; tt < NV; ++tt) x[tt] = *reinterpret_cast<const uint4*>(xs + tt * kKSlice + c);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int tt = 0; tt < NV; ++tt) acc[rr * NV + tt] = dot16(w[rr], x[tt], acc[rr * NV + tt], E());
      }
    }
  }
  const float sum = wave_reduce_scatter32(acc, lane);
  const int vi = lane >> 1;
  const int rr = vi / NV, tt = vi - rr * NV;
  if (row0 < rows && (lane & 1) == 0 && row0 + rr < rows && tt < nt)
    P.v[(int64_t)q * K.v_stride + K.v_indptr[s] + (int64_t)(tb + tt) * r + g * 16 + row0 + rr] = sum;
}

// MBGMM item: (segment s, token chunk, slice q), every rank group at once so
// each activation byte is read once.  C[rank][token] += A^T[rank][col] *
// X^T[col][token]; wave w covers columns 256w..256w+255 of the slice and the
// four partial tiles are summed through LDS in wave order.
template <class E, int GM, int NTT>
__device__ void shrink_mfma_body(const KArgs& K, const KProj& P, int q, int s, int a, int r, int t0,
                                 int tb, int nt, char* smem) {
  typedef typename E::T T;
  constexpr int EPV = E::kEpv;
  constexpr int STEP = 4 * EPV;
  constexpr int WCOLS = kKSlice / 4;
  constexpr int NSTEP = WCOLS / STEP;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, qq = lane >> 4;
  const int G = rank_groups(r);
  const int col0 = q * kKSlice;
  const int ncols = min(kKSlice, P.d_in - col0);
  const int pw = 1 << K.pw_log2;
  const int ncolA = (P.d_in + pw - 1) >> K.pw_log2;
  const T* X = reinterpret_cast<const T*>(P.X);

  int slot[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) slot[g] = P.a_indptr[a] + g * ncolA;
  int xrow[NTT];  // row offsets of the tile's tokens, -1 past the segment
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int tok = tt * 16 + li;
    xrow[tt] = tok < nt ? K.perm[t0 + tb + tok] : -1;
  }
  f4 acc[GM][NTT];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[g][tt] = f4{0.f, 0.f, 0.f, 0.f};

  if (wave * WCOLS < ncols) {
#pragma unroll 2
    for (int st = 0; st < NSTEP; ++st) {
      const int c = wave * WCOLS + st * STEP + qq * EPV;
      const bool ok = c < ncols;
      const int col = col0 + c;
      uint4 av[GM], xv[NTT];
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        av[g] = zero4();
        if (g < G && ok && g * 16 + li < r) {
          const T* pg = page_ptr<E>(K, P.a_pages[slot[g] + (col >> K.pw_log2)]);
          if (pg != nullptr) av[g] = ldg16(pg + li * pw + (col & (pw - 1)));
        }
      }
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) xv[tt] = (ok && xrow[tt] >= 0) ? ldg16(X + (int64_t)xrow[tt] * P.ldx + col) : zero4();
#pragma unroll
      for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) mma(acc[g][tt], av[g], xv[tt], E());
    }
  }

  float* red = reinterpret_cast<float*>(smem);  // [3][GM*NTT][64][4], GM*NTT <= 8
  if (wave > 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
        *reinterpret_cast<f4*>(red + (((wave - 1) * GM * NTT + g * NTT + tt) * 64 + lane) * 4) = acc[g][tt];
  }
  __syncthreads();
  if (wave == 0) {
    float* vout = P.v + (int64_t)q * K.v_stride + K.v_indptr[s];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        f4 c = acc[g][tt];
#pragma unroll
        for (int w = 0; w < 3; ++w) c += *reinterpret_cast<const f4*>(red + ((w * GM * NTT + g * NTT + tt) * 64 + lane) * 4);
        const int tok = tt * 16 + li;
        const int k0 = g * 16 + qq * 4;
        if (g < G && tok < nt) {
          float* dst = vout + (int64_t)(tb + tok) * r + k0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + i < r) dst[i] = c[i];
        }
      }
    }
  }
}

template <class E>
__device__ void shrink_mfma(const KArgs& K, const KProj& P, int q, int s, int local, char* smem) {
  const int a = K.seg_adapter[s];
  const int r = K.rank[a];
  const int t0 = K.seg_indptr[s];
  const int n = K.seg_indptr[s + 1] - t0;
  const int G = rank_groups(r);
  const int tch = 16 * mfma_token_tiles(G);
  const int tb = local * tch;
  const int nt = min(tch, n - tb);
  if (G <= 1) shrink_mfma_body<E, 1, 8>(K, P, q, s, a, r, t0, tb, nt, smem);
  else if (G == 2) shrink_mfma_body<E, 2, 4>(K, P, q, s, a, r, t0, tb, nt, smem);
  else if (G <= 4) shrink_mfma_body<E, 4, 2>(K, P, q, s, a, r, t0, tb, nt, smem);
  else shrink_mfma_body<E, 8, 1>(K, P, q, s, a, r, t0, tb, nt, smem);
}

template <class E>
__global__ __launch_bounds__(kThreads) void shrink_kernel(KArgs K) {
  __shared__ __attribute__((aligned(16))) char smem[kShrinkSmem];
  const int S = K.counts[LORA_COUNT_S];
  const int U = K.counts[4];
  if (S <= 0) return;
  int total = 0;
  for (int p = 0; p < K.np; ++p) total += K.p[p].nq * U;
  for (ItemWalk it(total); it.i < it.end; it.i += it.stride) {
    int rem = it.i, p = 0;
    while (rem >= K.p[p].nq * U) { rem -= K.p[p].nq * U; ++p; }
    const KProj& P = K.p[p];
    const int q = rem / U;
    const int u = rem - q * U;
    const int s = find_segment(K.shr_ptr, S, u);
    const int local = u - K.shr_ptr[s];
    const int n = K.seg_indptr[s + 1] - K.seg_indptr[s];
    if (is_mfma_segment(n)) shrink_mfma<E>(K, P, q, s, local, smem);
    else shrink_valu<E>(K, P, q, s, local, smem);
    __syncthreads();
  }
}

// ================================================================ expand
// MBGMV expand item: (segment s of < 16 tokens, 256-column slice).  v of the
// segment (slices summed in ascending order) sits in LDS; every thread owns
// one output column j, reads the 16 ranks of B for j in each rank group as
// 16-byte vectors, and produces Y for all the segment's tokens.
template <class E>
__device__ void expand_valu(const KArgs& K, const KProj& P, int js, int s, char* smem) {
  typedef typename E::T T;
  constexpr int EPV = E::kEpv;
  const int a = K.seg_adapter[s];
  const int r = K.rank[a];
  const int t0 = K.seg_indptr[s];
  const int n = K.seg_indptr[s + 1] - t0;
  const float scale = K.alpha[a] / (float)r;
  float* vs = reinterpret_cast<float*>(smem);  // [n][r]
  const float* vsrc = P.v + K.v_indptr[s];
  for (int idx = threadIdx.x; idx < n * r; idx += kThreads) {
    float sum = 0.0f;
    for (int q = 0; q < P.nv; ++q) sum += vsrc[(int64_t)q * K.v_stride + idx];
    vs[idx] = sum;
  }
  __syncthreads();
  const int j = js * kExpandCols + threadIdx.x;
  if (j >= P.d_out) return;
  const int pw = 1 << K.pw_log2;
  const int ncolB = (P.d_out + pw - 1) >> K.pw_log2;
  const int slot0 = P.b_indptr[a] + (j >> K.pw_log2);
  const int G = rank_groups(r);
  float acc[kMfmaMinTokens];
#pragma unroll
  for (int tt = 0; tt < kMfmaMinTokens; ++tt) acc[tt] = 0.0f;
  for (int g = 0; g < G; ++g) {
    const T* pg = page_ptr<E>(K, P.b_pages[slot0 + g * ncolB]);
    const int kmax = min(16, r - g * 16);
    float b[16];
    if (pg != nullptr) {
      const T* row = pg + (j & (pw - 1)) * 16;
#pragma unroll
      for (int v = 0; v < 16 / EPV; ++v) {
        const int kv = v * EPV;
        uint4 raw = (kv + EPV <= kmax) ? ldg16(row + kv) : (kv < kmax ? load_partial<E>(row + kv, kmax - kv) : zero4());
        const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int i = 0; i < EPV; ++i) b[kv + i] = to_f(e[i]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) b[k] = 0.0f;
    }
#pragma unroll
    for (int tt = 0; tt < kMfmaMinTokens; ++tt) {
      if (tt < n) {
        const float* vt = vs + tt * r + g * 16;
        float sacc = acc[tt];
        if (kmax == 16) {
#pragma unroll
          for (int k = 0; k < 16; ++k) sacc = fmaf(vt[k], b[k], sacc);
        } else {
          for (int k = 0; k < kmax; ++k) sacc = fmaf(vt[k], b[k], sacc);
        }
        acc[tt] = sacc;
      }
    }
  }
  const T* Yb = reinterpret_cast<const T*>(P.Yb);
  T* Y = reinterpret_cast<T*>(P.Y);
#pragma unroll
  for (int tt = 0; tt < kMfmaMinTokens; ++tt) {
    if (tt < n) {
      const int64_t row = K.perm[t0 + tt];
      from_f(Y + row * P.ldy + j, to_f(Yb[row * P.ldyb + j]) + scale * acc[tt]);
    }
  }
}

// MBGMM expand item: (segment s, chunk of <= 64 tokens, 256-column slice).
// C[col][token] += B^T[col][rank] * v^T[rank][token]; B pages hold the 16
// ranks of an output column contiguously, so each lane's operand is one
// 16-byte load.  Wave w covers columns 64w..64w+63 (four 16-column tiles).
template <class E>
__device__ void expand_mfma(const KArgs& K, const KProj& P, int js, int s, int local, char* smem) {
  typedef typename E::T T;
  constexpr int EPV = E::kEpv;
  constexpr int KSTEP = 4 * EPV;
  const int a = K.seg_adapter[s];
  const int r = K.rank[a];
  const int t0 = K.seg_indptr[s];
  const int n = K.seg_indptr[s + 1] - t0;
  const float scale = K.alpha[a] / (float)r;
  const int tb = local * kExpandTokens;
  const int nt = min(kExpandTokens, n - tb);
  float* vs = reinterpret_cast<float*>(smem);  // [nt][r]
  const float* vsrc = P.v + K.v_indptr[s] + (int64_t)tb * r;
  for (int idx = threadIdx.x; idx < nt * r; idx += kThreads) {
    float sum = 0.0f;
    for (int q = 0; q < P.nv; ++q) sum += vsrc[(int64_t)q * K.v_stride + idx];
    vs[idx] = sum;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, qq = lane >> 4;
  const int pw = 1 << K.pw_log2;
  const int ncolB = (P.d_out + pw - 1) >> K.pw_log2;
  const int jw = js * kExpandCols + wave * 64;
  f4 acc[4][4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[ct][tt] = f4{0.f, 0.f, 0.f, 0.f};
  if (jw < P.d_out) {
    const int nks = ceil_div_i(r, KSTEP);
    for (int ks = 0; ks < nks; ++ks) {
      const int k0 = ks * KSTEP + qq * EPV;
      const int kn = min(EPV, r - k0);  // valid ranks in this lane's vector (may be <= 0)
      const int g = k0 >> 4;
      uint4 bv[4], vv[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int j = jw + ct * 16 + li;
        bv[ct] = zero4();
        if (j < P.d_out && kn > 0) {
          const T* pg = page_ptr<E>(K, P.b_pages[P.b_indptr[a] + g * ncolB + (j >> K.pw_log2)]);
          if (pg != nullptr) {
            const T* src = pg + (j & (pw - 1)) * 16 + (k0 & 15);
            bv[ct] = kn >= EPV ? ldg16(src) : load_partial<E>(src, kn);
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int tok = tt * 16 + li;
        vv[tt] = (tok < nt && kn > 0) ? pack_operand(vs + tok * r + k0, kn, E()) : zero4();
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) mma(acc[ct][tt], bv[ct], vv[tt], E());
    }
  }
  const T* Yb = reinterpret_cast<const T*>(P.Yb);
  T* Y = reinterpret_cast<T*>(P.Y);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int tok = tt * 16 + li;
    if (tok >= nt) continue;
    const int64_t row = K.perm[t0 + tb + tok];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int col = jw + ct * 16 + qq * 4;
      if (col >= P.d_out) continue;
      const T* yb = Yb + row * P.ldyb + col;
      T* y = Y + row * P.ldy + col;
#pragma unroll
      for (int i = 0; i < 4; ++i) from_f(y + i, to_f(yb[i]) + scale * acc[ct][tt][i]);
    }
  }
}

// Rows of tokens without an adapter: Y = Y_base (only when Y is not Y_base).
template <class E>
__device__ void expand_copy(const KArgs& K, const KProj& P, int js, int chunk, int t_valid) {
  typedef typename E::T T;
  const int j = js * kExpandCols + threadIdx.x;
  if (j >= P.d_out) return;
  const int t_beg = t_valid + chunk * kExpandTokens;
  const int t_end = min(K.T, t_beg + kExpandTokens);
  const T* Yb = reinterpret_cast<const T*>(P.Yb);
  T* Y = reinterpret_cast<T*>(P.Y);
  for (int i = t_beg; i < t_end; ++i) {
    const int64_t row = K.perm[i];
    Y[row * P.ldy + j] = Yb[row * P.ldyb + j];
  }
}

template <class E>
__global__ __launch_bounds__(kThreads) void expand_kernel(KArgs K) {
  __shared__ __attribute__((aligned(16))) char smem[kExpandSmem];
  const int S = K.counts[LORA_COUNT_S];
  const int t_valid = K.counts[LORA_COUNT_T_VALID];
  const int Ue = S > 0 ? K.counts[5] : 0;
  const int ncopy = ceil_div_i(K.T - t_valid, kExpandTokens);
  int total = 0;
  for (int p = 0; p < K.np; ++p) total += K.p[p].njs * (Ue + (K.p[p].Y != K.p[p].Yb ? ncopy : 0));
  for (ItemWalk it(total); it.i < it.end; it.i += it.stride) {
    int rem = it.i, p = 0;
    int Up = Ue + (K.p[0].Y != K.p[0].Yb ? ncopy : 0);
    while (rem >= K.p[p].njs * Up) {
      rem -= K.p[p].njs * Up;
      ++p;
      Up = Ue + (K.p[p].Y != K.p[p].Yb ? ncopy : 0);
    }
    const KProj& P = K.p[p];
    const int js = rem / Up;
    const int u = rem - js * Up;
    if (u >= Ue) {
      expand_copy<E>(K, P, js, u - Ue, t_valid);
    } else {
      const int s = find_segment(K.exp_ptr, S, u);
      const int local = u - K.exp_ptr[s];
      const int n = K.seg_indptr[s + 1] - K.seg_indptr[s];
      if (is_mfma_segment(n)) expand_mfma<E>(K, P, js, s, local, smem);
      else expand_valu<E>(K, P, js, s, smem);
    }
    __syncthreads();
  }
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
                                                                   const int32_t* rank, int32_t* hist,
                                                                   SegOut out) {
  __shared__ int wsum[kSegScanThreads / 64 + 1];
  __shared__ int carry[6];
  if (threadIdx.x < 6) carry[threadIdx.x] = 0;
  __syncthreads();
  const int W = N + 2;
  for (int base = 0; base < N; base += kSegScanThreads) {
    const int a = base + threadIdx.x;
    int cnt = 0;
    if (a < N) {
      for (int c = 0; c < nchunk; ++c) {
        const int h = hist[(int64_t)c * W + a];
        hist[(int64_t)c * W + a] = cnt;  // prefix within this adapter's tokens
        cnt += h;
      }
    }
    const int r = (a < N && cnt > 0) ? rank[a] : 0;
    const int vals[5] = {cnt, cnt > 0 ? 1 : 0, cnt * r, cnt > 0 ? shrink_items(cnt, r) : 0,
                         cnt > 0 ? expand_items(cnt) : 0};
    int pre[5], tots[5];
#pragma unroll
    for (int f = 0; f < 5; ++f) {
      pre[f] = block_exclusive_scan(vals[f], wsum, &tots[f]) + carry[f];
    }
    if (a < N && cnt > 0) {
      const int si = pre[1];
      out.seg_adapter[si] = a;
      out.seg_indptr[si] = pre[0];
      out.v_indptr[si] = pre[2];
      out.shr_ptr[si] = pre[3];
      out.exp_ptr[si] = pre[4];
      for (int c = 0; c < nchunk; ++c) hist[(int64_t)c * W + a] += pre[0];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int f = 0; f < 5; ++f) carry[f] += tots[f];
    }
    __syncthreads();
  }
  // excluded tokens: chunk-ordered offsets after the grouped ones
  if (threadIdx.x == 0) {
    const int S = carry[1], t_valid = carry[0];
    out.seg_indptr[S] = t_valid;
    out.v_indptr[S] = carry[2];
    out.shr_ptr[S] = carry[3];
    out.exp_ptr[S] = carry[4];
    int run = t_valid, n_invalid = 0;
    for (int c = 0; c < nchunk; ++c) {
      const int base_only = hist[(int64_t)c * W + N];
      const int bad = hist[(int64_t)c * W + N + 1];
      hist[(int64_t)c * W + N] = run;
      run += base_only + bad;
      n_invalid += bad;
    }
    out.counts[LORA_COUNT_S] = S;
    out.counts[LORA_COUNT_INVALID] = n_invalid;
    out.counts[LORA_COUNT_T_VALID] = t_valid;
    out.counts[LORA_COUNT_V_TOTAL] = carry[2];
    out.counts[4] = carry[3];
    out.counts[5] = carry[4];
    out.counts[LORA_COUNT_FLAGS] = 0;
    out.counts[7] = 0;
  }
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
  constexpr uint32_t kExcluded = 0x3FFFFFu;
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

hipError_t launch_build_segments(const int32_t* ids, int T, int N, const int32_t* rank, int32_t* hist,
                                 const SegOut& out, hipStream_t stream) {
  const int nchunk = ceil_div_i(T, kSegChunk);
  if (nchunk > 0) {
    seg_hist_kernel<<<nchunk, kThreads, 0, stream>>>(ids, T, N, rank, hist);
    if (hipError_t e = launch_err()) return e;
  }
  seg_scan_kernel<<<1, kSegScanThreads, 0, stream>>>(T, N, nchunk, rank, hist, out);
  if (hipError_t e = launch_err()) return e;
  if (nchunk > 0) {
    seg_scatter_kernel<<<nchunk, kSegChunk, 0, stream>>>(ids, T, N, rank, hist, out.perm);
    if (hipError_t e = launch_err()) return e;
  }
  return hipSuccess;
}

hipError_t launch_shrink(const KArgs& K, int dtype, int grid, hipStream_t stream) {
  if (dtype == LORA_DTYPE_BF16) shrink_kernel<Bf16><<<grid, kThreads, 0, stream>>>(K);
  else shrink_kernel<F32><<<grid, kThreads, 0, stream>>>(K);
  return launch_err();
}

hipError_t launch_expand(const KArgs& K, int dtype, int grid, hipStream_t stream) {
  if (dtype == LORA_DTYPE_BF16) expand_kernel<Bf16><<<grid, kThreads, 0, stream>>>(K);
  else expand_kernel<F32><<<grid, kThreads, 0, stream>>>(K);
  return launch_err();
}

hipError_t occupancy(int dtype, int* shrink_blocks, int* expand_blocks) {
  hipError_t e;
  if (dtype == LORA_DTYPE_BF16) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(shrink_blocks, shrink_kernel<Bf16>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(expand_blocks, expand_kernel<Bf16>, kThreads, 0);
  } else {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(shrink_blocks, shrink_kernel<F32>, kThreads, 0);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(expand_blocks, expand_kernel<F32>, kThreads, 0);
  }
  return e;
}

}  // namespace lora
