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
// MBGMM shrink items: 16-token MFMA tiles x 16-rank groups, each A operand
// shared by the item's token tiles and each activation operand by its rank
// groups.  Segments shorter than kMfmaLongSegment (a decode batch's hot
// adapters, prefill chunks of a mixed batch): 32 tokens x 1 group.  Longer
// ones (prefill sequences): 64 tokens x 2 groups, so that two of every three
// operand loads in flight are activations (ranks above 32 take two items
// per tile, which run side by side and meet the tile's activations in L2).
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

// Exact quotient n / d for 0 <= n < 2^31 and 1 <= d < 2^31: one multiply-
// high, an add and a shift, with the divisor's multiplier m = floor(2^32 *
// (2^s - d) / d) + 1, s = ceil(log2 d), built once (the round-up method of
// division by invariant integers; n < 2^31 keeps mulhi(n, m) + n in 32 bits).
// A run-time division is a long instruction sequence; this one is per item.
struct FastDiv {
  unsigned m;
  int s;
  LORA_HD FastDiv() : m(1u), s(0) {}
  LORA_HD explicit FastDiv(int d) : m(1u), s(0) {
    while ((1u << s) < (unsigned)d) ++s;
    m = (unsigned)(((((unsigned long long)1) << 32) * ((((unsigned long long)1) << s) - (unsigned)d)) / (unsigned)d + 1u);
  }
  LORA_HD int div(int n) const {
    const unsigned hi = (unsigned)(((unsigned long long)(unsigned)n * m) >> 32);
    return (int)((hi + (unsigned)n) >> s);
  }
};
LORA_HD inline int rank_groups(int r) { return (r + 15) >> 4; }

LORA_HD inline bool is_mfma_segment(int n) { return n >= kMfmaMinTokens; }

// Work items of one segment, per 512-column shrink slice or per expand
// column block.  MBGMV shrink: (rank group, <= kValuTokens tokens); MBGMM
// shrink: (16-token tile, rank group); MBGMV expand: (part, chunk of <= 2
// tokens), the column block split in 1, 2 or 4 parts for 1, 2 or more rank
// groups (every part holds at most 4 (sub-block, rank group) pairs of B);
// MBGMM expand: one 16-token tile.
LORA_HD inline int shrink_items_valu(int n, int r) {
  return is_mfma_segment(n) ? 0 : rank_groups(r) * ceil_div_i(n, kValuTokens);
}
LORA_HD inline int shrink_item_groups(int n, int r) {
  return n < kMfmaLongSegment ? 1 : 2;
}
LORA_HD inline int shrink_tile_tokens(int n, int r) {
  return shrink_item_groups(n, r) == 2 ? kMfmaShrinkTokensLong : kMfmaShrinkTokensShort;
}
LORA_HD inline int shrink_items_mfma(int n, int r) {
  return is_mfma_segment(n) ? ceil_div_i(rank_groups(r), shrink_item_groups(n, r)) * ceil_div_i(n, shrink_tile_tokens(n, r))
                            : 0;
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
// The phase barrier of the single-launch apply kernel, in the plan (int32
// units, one 128-byte line per counter, so that atomics on different
// counters do not share a line):
//   line 0               epoch E: the launch in progress uses bank E & 1
//   bank b, lines 0..7   work-groups of XCD x that have written their shrink
//                        partial sums
//   bank b, line 8       XCDs all of whose work-groups have
// A launch zeroes the other bank at its start and flips E when its last
// work-group arrives, so every launch finds its bank zeroed without any
// reset between launches; the segment builder zeroes the whole area.
// After the banks, the expand kernel's MBGMM item queues:
//   queue line x         items of XCD x handed out from its queue so far
//   queue line 8 + x     work-groups of XCD x done with their MBGMM items
// The last work-group of an XCD to finish puts both back to zero, so every
// launch finds them zeroed.
constexpr int kSyncLine = 32;
constexpr int kSyncBankLines = 9;
constexpr int kQueueLines = 16;
constexpr int kSyncInts = kSyncLine * (1 + 2 * kSyncBankLines + kQueueLines);
LORA_HD inline int sync_bank(int b) { return kSyncLine * (1 + kSyncBankLines * b); }
LORA_HD inline int queue_line(int l) { return kSyncLine * (1 + 2 * kSyncBankLines + l); }

struct PlanLayout {
  long long seg_desc, shrink_mfma, shrink_valu, expand_mfma, expand_valu, sync, total;
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
  L.sync = L.expand_valu + align64(kValuItemInts * L.cap_expand_valu);
  L.total = L.sync + kSyncInts;
  return L;
}

// ------------------------------------------------------------ work walks
// The compute kernels are persistent grids (grid work-groups of kWaves
// waves) whose waves walk the item lists below.  The walks depend only on
// the grid size, the work-group index and the item totals, and are written
// for host and device alike, so that a host test can enumerate every wave's
// items and check that each item is taken exactly once.
//
// XCD-aware wave walk: the item range [0, total) is cut into 8 contiguous
// parts, part x served by the waves of the work-groups with index % 8 == x
// (work-groups are dealt to the 8 XCDs round robin), so items that share an
// adapter slice are read through the same L2.  Every wave walks its own
// items: no work-group barrier couples the waves.
LORA_HD inline int xcd_count(int grid) { return (grid % 8 == 0) ? 8 : 1; }
// log2 of xcd_count: the walks split ranges with shifts, not divisions (a
// 64-bit division is a long scalar sequence in every wave's prologue)
LORA_HD inline int xcd_shift(int grid) { return (grid % 8 == 0) ? 3 : 0; }
// start of XCD part x of [0, total): floor(total * x / 2^sh)
LORA_HD inline int xcd_part(int total, int x, int sh) { return (int)(((long long)total * x) >> sh); }

// Grid of a persistent launch: enough work-groups for the items (bound), at
// most `resident` (compute units x work-groups per unit), rounded to a
// multiple of 8 when that stays within `resident` (so every XCD gets the same
// share), else down to one.  Never above `resident`: the single-launch
// kernel's phase barrier needs every work-group of its grid resident at once.
LORA_HD inline int launch_grid(int resident, long long bound) {
  if (resident < 1) resident = 1;
  long long g = bound < 1 ? 1 : bound;
  if (g > resident) g = resident;
  const long long up = (g + 7) / 8 * 8;
  if (up <= resident) return (int)up;
  const long long down = g / 8 * 8;
  return (int)(down >= 8 ? down : g);
}

struct WaveWalk {
  int i, end, stride, lo;
  // `walkers` items are taken per work-group at a time (kWaves: one per wave;
  // 1: whole-block items), `w` is this walker's index in the work-group.
  LORA_HD WaveWalk(int total, int w, int walkers, int grid, int block) {
    const int sh = xcd_shift(grid);
    const int x = block & ((1 << sh) - 1);
    lo = xcd_part(total, x, sh);
    end = xcd_part(total, x + 1, sh);
    i = lo + (block >> sh) * walkers + w;
    stride = (grid >> sh) * walkers;
  }
};

// The MBGMV walk when the first Wm waves of each XCD run the MBGMM items:
// the other waves take R rounds of the XCD's MBGMV items among themselves (R:
// the MBGMV items that take as long as one wave's MBGMM items), then every
// wave takes items in turn.
struct TwoClassWalk {
  int i, end, nV, W, ib, ka;  // ka: first-phase items left after the current one (-1: second phase)
  int lo;                     // start of this XCD's part of the range
  LORA_HD TwoClassWalk(int total, int Wm, int R, int wv, int grid, int block) {
    const int sh = xcd_shift(grid);
    const int x = block & ((1 << sh) - 1), G = grid >> sh;
    const int w = (block >> sh) * kWaves + wv;  // walker index inside the XCD
    lo = xcd_part(total, x, sh);
    end = xcd_part(total, x + 1, sh);
    W = G * kWaves;
    Wm = Wm < W ? Wm : W;
    nV = W - Wm;
    ib = lo + R * nV + w;
    if (w >= Wm && R > 0) {
      i = lo + (w - Wm);
      ka = R - 1;
    } else {
      i = ib;
      ka = -1;
    }
  }
  LORA_HD int next() {
    if (ka > 0) {
      --ka;
      return i + nV;
    }
    if (ka == 0) {
      ka = -1;
      return ib;
    }
    return i + W;
  }
};

// MBGMV rounds one MBGMM shrink item is worth (measured: 2 and 4 were slower)
constexpr int kShrinkMfmaRounds = 3;

// Shrink: the MBGMM items go to the first waves of each XCD's walk.  When
// they are a small share of the items (under one in eight: a decode batch's
// hot adapters, whose segments are short enough for 32-token items), those
// waves skip the first rounds of MBGMV items: a 32-token MBGMM item is four
// rounds of loads against one for an MBGMV item.  Returns (Wm, R) of the
// MBGMV walk.
LORA_HD inline void shrink_walk_split(int total_m, int total_v, int wave, int grid, int block, int& Wm, int& R) {
  Wm = 0;
  R = 0;
  if (total_m > 0 && 8 * (long long)total_m < total_v) {
    WaveWalk im(total_m, wave, kWaves, grid, block);
    const int m = im.end - im.lo;
    Wm = m < im.stride ? m : im.stride;
    R = kShrinkMfmaRounds * ceil_div_i(m, im.stride);
  }
}

// Expand: the MBGMM items are whole-block items.  When they are a small share
// of the launch's items (a decode batch with a few hot adapters: under one in
// eight), they go to the first third of each XCD's work-groups (one per CU),
// so the other waves start streaming MBGMV weights at once and the MBGMM
// items' round trips overlap them; otherwise (prefill, mixed batches) to
// every work-group.  This work-group takes MBGMM items first, lo_m + beta,
// lo_m + beta + Gm, ... below end_m (when beta < Gm); Gm and R parameterise
// the MBGMV walk (the other work-groups take R first rounds alone).
struct ExpandSplit {
  int Gm, R, first, lo_m, end_m, step;
};
LORA_HD inline ExpandSplit expand_walk_split(int total_m, int total_v, int grid, int block) {
  ExpandSplit e{0, 0, 0, 0, 0, 1};
  if (total_m <= 0) return e;
  const int sh = xcd_shift(grid);
  const int x = block & ((1 << sh) - 1), beta = block >> sh, G = grid >> sh;
  const int lo_m = xcd_part(total_m, x, sh);
  e.lo_m = lo_m;
  e.end_m = xcd_part(total_m, x + 1, sh);
  const int m = e.end_m - lo_m;
  const int third = G / 3 > 1 ? G / 3 : 1;
  e.Gm = m <= 0 ? 0 : 8 * (long long)total_m >= total_v ? G : (third < m ? third : m);
  e.R = e.Gm > 0 ? ceil_div_i(6 * m, 10 * e.Gm) : 0;  // an MBGMM item took ~0.6 MBGMV item times
  e.first = beta < e.Gm ? lo_m + beta : e.end_m;
  e.step = e.Gm > 0 ? e.Gm : 1;
  return e;
}

// The expand kernel's MBGMM items go to the XCDs in blocks of
// kExpandItemBlock consecutive items (token tiles of one segment and column
// block, which re-read the same B from that XCD's L2), block k to XCD
// k mod 2^sh.  Handing each XCD a contiguous eighth of the list instead
// ties its load to the ranks of the segments there: segments of rank 64
// take twice the time of rank <= 32 ones per item.
constexpr int kExpandItemBlock = 16;
// items of XCD x
LORA_HD inline int xcd_block_items(int total, int x, int sh) {
  const int nx = 1 << sh;
  const int nblocks = ceil_div_i(total, kExpandItemBlock);
  if (nblocks <= x) return 0;
  int n = ((nblocks - 1 - x) / nx + 1) * kExpandItemBlock;
  const int rem = total % kExpandItemBlock;
  if (rem > 0 && (nblocks - 1) % nx == x) n -= kExpandItemBlock - rem;  // the last block is short
  return n;
}
// the l-th item of XCD x (l < xcd_block_items(total, x, sh))
LORA_HD inline int xcd_block_item(int l, int x, int sh) {
  return (((l / kExpandItemBlock) << sh) + x) * kExpandItemBlock + l % kExpandItemBlock;
}
// The expand kernel's split: MBGMM items of XCD x by xcd_block_items (the
// work-groups Gm of the XCD take them from its queue), the rest as in
// expand_walk_split.
struct QueueSplit {
  int Gm, R, m, x, beta;
};
LORA_HD inline QueueSplit expand_queue_split(int total_m, int total_v, int grid, int block) {
  const int sh = xcd_shift(grid);
  QueueSplit e{0, 0, 0, block & ((1 << sh) - 1), block >> sh};
  if (total_m <= 0) return e;
  const int G = grid >> sh;
  e.m = xcd_block_items(total_m, e.x, sh);
  const int third = G / 3 > 1 ? G / 3 : 1;
  e.Gm = e.m <= 0 ? 0 : 8 * (long long)total_m >= total_v ? G : (third < e.m ? third : e.m);
  e.R = e.Gm > 0 ? ceil_div_i(6 * e.m, 10 * e.Gm) : 0;
  return e;
}

// Columns per wave of an MBGMM expand item (128..512, at most the page
// width), halved until the items cover the grid once, so a few hot segments
// still spread over every compute unit; wide items stage a token tile's v
// once for more columns.  d_out(p) gives projection p's output width.
template <class DOut>
LORA_HD inline int expand_mfma_cols(int np, DOut d_out, int pw_log2, int Um, int grid, int& total) {
  int wc = (1 << pw_log2) < 512 ? (1 << pw_log2) : 512;
  for (;; wc >>= 1) {
    total = 0;
    for (int p = 0; p < np; ++p) total += ceil_div_i(d_out(p), kWaves * wc) * Um;
    if (wc <= 128 || total >= grid) break;
  }
  return wc;
}

}  // namespace lora
