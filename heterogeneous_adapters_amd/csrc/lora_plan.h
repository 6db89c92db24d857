// Internal work-decomposition constants of liblora (host and device).
//
// The batch is cut into segments (tokens of one adapter, [MLSP] "Segmented
// Gather Matrix-Vector Multiplication (SGMV)").  Each segment is processed by
// one of two paths, chosen by its token count n:
//   * n <  kMfmaMinTokens : the MBGMV path -- vector ALU dot products with
//     wavefront reductions across d_in ([MLSP] "Multi-Size Batched Gather
//     Kernels": decode, a few tokens per adapter);
//   * n >= kMfmaMinTokens : the MBGMM path -- 16x16 MFMA tiles over token
//     tiles of the segment (a real dense contraction: every weight element
//     is reused by >= 16 tokens).
// Work is cut into wave-sized items that every wave of a persistent grid
// walks independently, so a compute unit keeps many independent
// page-table-to-data load chains in flight.
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
constexpr int kWaves = kThreads / 64;
constexpr int kKSlice = 512;              // input columns per shrink item (one partial slice)
constexpr int kValuTokens = 2;            // tokens per MBGMV shrink item
constexpr int kValuExpandTokens = 8;      // tokens per MBGMV expand item
constexpr int kMfmaExpandTokens = 16;     // tokens per MBGMM expand item (one tile)
constexpr int kProjsPerLaunch = 16;       // projection descriptors per launch
constexpr int kSegChunk = 1024;           // tokens per segment-builder block
#ifndef LORA_MFMA_MIN_TOKENS
#define LORA_MFMA_MIN_TOKENS 16
#endif
constexpr int kMfmaMinTokens = LORA_MFMA_MIN_TOKENS;  // segment length that switches to MFMA

// Output columns per expand item: 4 per lane in bf16, 2 per lane in fp32.
LORA_HD inline int expand_cols(bool bf16) { return bf16 ? 256 : 128; }

LORA_HD inline int ceil_div_i(int a, int b) { return (a + b - 1) / b; }
LORA_HD inline int rank_groups(int r) { return (r + 15) >> 4; }

// MBGMM shrink: accumulators are rank_groups x token_tiles 16x16 tiles; the
// product is kept at 4 tiles (8 for rank > 64), so the operands of several K
// steps fit in registers at once.
LORA_HD inline int mfma_token_tiles(int groups) {
  return groups <= 1 ? 4 : groups == 2 ? 2 : 1;
}

LORA_HD inline bool is_mfma_segment(int n) { return n >= kMfmaMinTokens; }

// Shrink work items of one segment (per 512-column slice).
LORA_HD inline int shrink_items(int n, int r) {
  const int G = rank_groups(r);
  if (is_mfma_segment(n)) return ceil_div_i(n, 16 * mfma_token_tiles(G));
  return G * ceil_div_i(n, kValuTokens);
}

// Expand work items of one segment (per expand column block).
LORA_HD inline int expand_items(int n) {
  return ceil_div_i(n, is_mfma_segment(n) ? kMfmaExpandTokens : kValuExpandTokens);
}

// Capacity of the per-batch item tables (entries), from T alone:
// shrink items <= sum G*(n/2 + 1) <= 4T + 8S <= 12T, expand items <= T/8 + S <= 2T.
LORA_HD inline long long shrink_item_capacity(int T) { return 12LL * (T > 0 ? T : 0) + 1; }
LORA_HD inline long long expand_item_capacity(int T) { return 2LL * (T > 0 ? T : 0) + 1; }

}  // namespace lora
