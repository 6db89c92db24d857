// Internal work-decomposition constants of liblora (host and device).
//
// The batch is cut into segments (tokens of one adapter, [MLSP] "Segmented
// Gather Matrix-Vector Multiplication (SGMV)").  Each segment is processed by
// one of two paths, chosen by its token count n:
//   * n <  kMfmaMinTokens : the MBGMV path -- vector ALU dot products with the
//     token rows staged in LDS and wavefront reductions across d_in
//     ([MLSP] "Multi-Size Batched Gather Kernels": decode, few tokens);
//   * n >= kMfmaMinTokens : the MBGMM path -- 16x16 MFMA tiles over token
//     tiles of the segment (a real dense contraction: every weight element
//     is reused by >= 16 tokens).
// [MLSP] = "Multi-LoRA Serving in Production: Architecture, Dynamic Adapter
// Swapping, and GPU Memory Management".
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define LORA_HD __host__ __device__
#else
#define LORA_HD
#endif

namespace lora {

constexpr int kThreads = 256;             // work-group size (4 wave64)
constexpr int kKSlice = 1024;             // input columns per shrink item
constexpr int kValuTokens = 8;            // tokens per MBGMV shrink item
constexpr int kMfmaMinTokens = 16;        // segment length that switches to MFMA
constexpr int kExpandTokens = 64;         // tokens per MBGMM expand item
constexpr int kExpandCols = 256;          // output columns per expand item
constexpr int kProjsPerLaunch = 16;       // projection descriptors per launch
constexpr int kSegChunk = 1024;           // tokens per segment-builder block

LORA_HD inline int ceil_div_i(int a, int b) { return (a + b - 1) / b; }
LORA_HD inline int rank_groups(int r) { return (r + 15) >> 4; }

// MBGMM shrink: accumulators are rank_groups x token_tiles 16x16 tiles; the
// product is kept at 8 tiles (32 accumulator registers per lane).
LORA_HD inline int mfma_token_tiles(int groups) {
  return groups <= 1 ? 8 : groups == 2 ? 4 : groups <= 4 ? 2 : 1;
}

LORA_HD inline bool is_mfma_segment(int n) { return n >= kMfmaMinTokens; }

// Shrink work items of one segment (per 1024-column slice).
LORA_HD inline int shrink_items(int n, int r) {
  const int G = rank_groups(r);
  if (is_mfma_segment(n)) return ceil_div_i(n, 16 * mfma_token_tiles(G));
  return G * ceil_div_i(n, kValuTokens);
}

// Expand work items of one segment (per 256-column slice).
LORA_HD inline int expand_items(int n) {
  return is_mfma_segment(n) ? ceil_div_i(n, kExpandTokens) : 1;
}

}  // namespace lora
