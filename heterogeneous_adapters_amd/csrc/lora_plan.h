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
// Tokens per MBGMV expand item (a chunk of the segment).  Every token's
// Y_base row is requested with the item's weights, so the chunk's rows live
// in registers for the whole item: 2 fits beside 16 KiB of B, 4 spills.
constexpr int kValuExpandTokens = 2;
constexpr int kCopyTokens = 8;            // rows per copy item (tokens without an adapter)
constexpr int kMfmaExpandTokens = 16;     // tokens per MBGMM expand item (one tile)
// Tokens per MBGMM shrink item (16-token MFMA tiles sharing each A operand):
// 64 for segments of at least kMfmaLongSegment tokens (prefill sequences: A
// is re-read from L2 once per 64 tokens), 32 for shorter ones (a decode
// batch's hot adapters and prefill chunks of a mixed batch: items of half
// the load rounds, twice as many).
constexpr int kMfmaShrinkTokensShort = 32, kMfmaShrinkTokensLong = 64, kMfmaLongSegment = 512;
constexpr int kProjsPerLaunch = 16;       // projection descriptors per launch
constexpr int kSegChunk = 1024;           // tokens per segment-builder block
constexpr int kMfmaMinTokens = 16;       // segment length that switches to MFMA (one full tile)

// Output columns of an MBGMV expand column block: 4 sub-blocks of 64 lanes x
// (2 bf16 | 1 fp32) columns, i.e. 64 bytes of B per lane, sub-block and rank
// group.
constexpr int kValuSubBlocks = 4;
LORA_HD inline int expand_cols(bool bf16) { return kValuSubBlocks * 64 * (bf16 ? 2 : 1); }

LORA_HD inline int ceil_div_i(int a, int b) { return (a + b - 1) / b; }
LORA_HD inline int rank_groups(int r) { return (r + 15) >> 4; }

LORA_HD inline bool is_mfma_segment(int n) { return n >= kMfmaMinTokens; }
LORA_HD inline int shrink_tile_tokens(int n) { return n >= kMfmaLongSegment ? kMfmaShrinkTokensLong : kMfmaShrinkTokensShort; }

// Work items of one segment, per 512-column shrink slice or per expand
// column block.  MBGMV shrink: (rank group, <= kValuTokens tokens); MBGMM
// shrink: (16-token tile, rank group); MBGMV expand: (part, chunk of <= 2
// tokens), the column block split in 1, 2 or 4 parts for 1, 2 or more rank
// groups (every part holds at most 4 (sub-block, rank group) pairs of B);
// MBGMM expand: one 16-token tile.
LORA_HD inline int shrink_items_valu(int n, int r) {
  return is_mfma_segment(n) ? 0 : rank_groups(r) * ceil_div_i(n, kValuTokens);
}
LORA_HD inline int shrink_items_mfma(int n, int r) {
  return is_mfma_segment(n) ? rank_groups(r) * ceil_div_i(n, shrink_tile_tokens(n)) : 0;
}
LORA_HD inline int valu_expand_parts(int r) { return rank_groups(r) == 1 ? 1 : rank_groups(r) == 2 ? 2 : 4; }
LORA_HD inline int valu_expand_chunks(int n) { return ceil_div_i(n, kValuExpandTokens); }
LORA_HD inline int expand_items_valu(int n, int r) {
  return is_mfma_segment(n) ? 0 : valu_expand_parts(r) * valu_expand_chunks(n);
}
LORA_HD inline int expand_items_mfma(int n) { return is_mfma_segment(n) ? ceil_div_i(n, kMfmaExpandTokens) : 0; }

// counters (int32) written by the segment builder
constexpr int kCountS = 0, kCountInvalid = 1, kCountTValid = 2, kCountVTotal = 3;
constexpr int kCountShrinkMfma = 4, kCountShrinkValu = 5, kCountExpandMfma = 6, kCountExpandValu = 7;
constexpr int kCountFlags = 8;
// the token count the segments were built for, and a check word derived
// from it: a compute kernel that finds the pair inconsistent (a buffer never
// built, or garbage) or built for another batch size computes nothing
constexpr int kCountT = 9, kCountCheck = 10;
constexpr int kNumCounts = 16;
LORA_HD inline int segments_check_word(int T) { return (int)(0x4C6F5261u ^ (unsigned)T); }

// The internal plan area: per-segment descriptors (2 x int4: {adapter,
// rank, first token, tokens}, {v offset, first shrink item, first expand
// item, alpha bits}) and the item tables of the two paths.  The MBGMM
// tables map an item to its segment; the MBGMV tables hold the segment's
// descriptor itself (kValuItemInts int32 per item), so the walk of the many
// short decode items reaches the descriptor in one load, not two.
// Offsets in int32 units, each a multiple of 64.
constexpr int kValuItemInts = 8;
struct PlanLayout {
  long long seg_desc, shrink_mfma, shrink_valu, expand_mfma, expand_valu, total;
  // capacities: segments, and items of each table
  long long s_cap, cap_shrink_mfma, cap_shrink_valu, cap_expand_mfma, cap_expand_valu;
};
LORA_HD inline long long align64(long long x) { return (x + 63) / 64 * 64; }
LORA_HD inline PlanLayout plan_layout(int T, int N) {
  const long long t = T > 0 ? T : 0;
  const long long smax = (T < N ? t : (N > 0 ? N : 0));
  PlanLayout L;
  L.s_cap = smax;
  // MBGMM shrink items <= 8*(T/16 + S) <= 9T; MBGMV <= 8*(T/2 + S) <= 12T
  L.cap_shrink_mfma = 9 * t + 1;
  L.cap_shrink_valu = 12 * t + 1;
  // MBGMM expand items <= T/16 + S <= 2T; MBGMV <= 4*(T/K + S) <= (4/K + 4)T
  // for chunks of K = kValuExpandTokens tokens
  L.cap_expand_mfma = 2 * t + 1;
  L.cap_expand_valu = (4 / kValuExpandTokens + 4) * t + 1;
  L.seg_desc = 0;
  L.shrink_mfma = align64(8 * (smax > 0 ? smax : 1));
  L.shrink_valu = L.shrink_mfma + align64(L.cap_shrink_mfma);
  L.expand_mfma = L.shrink_valu + align64(kValuItemInts * L.cap_shrink_valu);
  L.expand_valu = L.expand_mfma + align64(L.cap_expand_mfma);
  L.total = L.expand_valu + align64(kValuItemInts * L.cap_expand_valu);
  return L;
}

}  // namespace lora
