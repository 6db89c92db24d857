/*
 * CPU oracle for the multi-LoRA adapter branch -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or helper with
 * the HIP library: it reads the adapter pool through its own page-table
 * arithmetic and rounds to bf16 with its own routine.
 *
 * Sources (the three web pages this project follows):
 *   [MLSP] "Multi-LoRA Serving in Production: Architecture, Dynamic Adapter
 *          Swapping, and GPU Memory Management" (llms.blog)
 *   [MLSA] "Multi-LoRA Serving Architecture: Serving Hundreds of Fine-Tuned
 *          Adapters on One GPU with vLLM and S-LoRA (2026)"
 *   [LAST] "LoRA Adapters at Serve Time with vLLM Multi-LoRA"
 *
 * What it computes (plain definition, evaluated token by token):
 *   Y[t] = Y_base[t] + (alpha_a / r_a) * (X[t] A_a) B_a,   a = ids[t]
 * with A_a of shape d_in x r_a and B_a of shape r_a x d_out, the adapted
 * layer equation of [MLSP] "The Mathematical Anatomy of Heterogeneous
 * Batches".  The shrink (v = x A) and the expand (v B, scaled by alpha/r,
 * added to the base output) are the two steps of [MLSP] "Segmented Gather
 * Matrix-Vector Multiplication (SGMV)"; A and B are never multiplied together
 * ([LAST] "Architecture of Multi-LoRA in vLLM").  Each adapter is read at its
 * own rank, with no padding to the largest rank ([MLSP] "Multi-Size Batched
 * Gather Kernels (MBGMV and MBGMM)"), through page tables of physical page
 * indices ([MLSP] "Unified Paging Architecture").
 *
 * Precision: every sum is a sequential fp32 sum in ascending index order
 * (built with -ffp-contract=off, no fast-math); bf16 inputs widen exactly to
 * fp32; the output is Y_base + s*acc in fp32 with one final round-to-nearest-
 * even to the output dtype.  s = (float)alpha / (float)r, one fp32 division.
 *
 * Page format (see the generator): page = 16 x PW elements.  A element
 * (input i, rank k) lives in A-table slot (k/16)*ceil(d_in/PW) + i/PW at
 * offset (k%16)*PW + i%PW.  B element (rank k, output j) lives in B-table slot
 * (k/16)*ceil(d_out/PW) + j/PW at offset ((k%16)/8)*8*PW + (j%PW)*8 + k%8
 * (two halves of 8 ranks, each holding PW columns of 8 contiguous ranks).
 *
 * Token classes: ids[t] == -1 is a base-model token ([MLSA] "What vLLM
 * actually gives you": base-model requests share the server); any other id
 * outside [0, N), or an adapter whose rank is outside [1, 128], makes the
 * token invalid.  Both keep Y[t] = Y_base[t]; invalid ones are counted.
 */
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DT_F32 0
#define ORACLE_DT_BF16 1
#define ORACLE_MAX_RANK 128

static float bf16_bits_to_float(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round-to-nearest-even fp32 -> bf16; NaN stays NaN (quiet). */
static uint16_t float_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t keep = u >> 16;
  uint32_t rest = u & 0xffffu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

uint16_t oracle_round_bf16(float f) { return float_to_bf16_bits(f); }

static float load_elem(const void* base, int dtype, int64_t idx) {
  if (dtype == ORACLE_DT_BF16) return bf16_bits_to_float(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int token_valid(int32_t id, int32_t N, const int32_t* rank) {
  return id >= 0 && id < N && rank[id] >= 1 && rank[id] <= ORACLE_MAX_RANK;
}

/* ---------------------------------------------------------------- segments
 * Group tokens by adapter ([MLSP] SGMV: requests are grouped by the adapter
 * they target).  Reading taken where the pages are silent: a stable order
 * (ascending token index inside a group), groups in ascending adapter id,
 * empty groups never emitted; tokens that use no adapter follow the grouped
 * ones in ascending token index.  Outputs:
 *   perm[T]: grouped valid tokens, then excluded tokens
 *   seg_indptr[S+1], seg_adapter[S], v_indptr[S+1] (v offsets: tokens*rank)
 *   counts[4] = {S, n_invalid, T_valid, V_total}
 * Written out as the definition: for each adapter, scan every token. */
int oracle_segments(const int32_t* ids, int32_t T, const int32_t* rank, int32_t N,
                    int32_t* perm, int32_t* seg_indptr, int32_t* seg_adapter,
                    int32_t* v_indptr, int32_t* counts) {
  if (T < 0 || N < 0) return -1;
  int32_t pos = 0, S = 0, n_invalid = 0;
  int64_t v = 0;
  seg_indptr[0] = 0;
  v_indptr[0] = 0;
  for (int32_t a = 0; a < N; ++a) {
    int32_t cnt = 0;
    for (int32_t t = 0; t < T; ++t)
      if (ids[t] == a && token_valid(ids[t], N, rank)) { perm[pos++] = t; ++cnt; }
    if (cnt > 0) {
      seg_adapter[S] = a;
      seg_indptr[S + 1] = pos;
      v += (int64_t)cnt * rank[a];
      v_indptr[S + 1] = (int32_t)v;
      ++S;
    }
  }
  int32_t t_valid = pos;
  for (int32_t t = 0; t < T; ++t) {
    if (!token_valid(ids[t], N, rank)) {
      perm[pos++] = t;
      if (ids[t] != -1) ++n_invalid;
    }
  }
  counts[0] = S;
  counts[1] = n_invalid;
  counts[2] = t_valid;
  counts[3] = (int32_t)v;
  return 0;
}

/* ------------------------------------------------------- page-table reads */
typedef struct {
  const void* pool;
  int dtype;
  int32_t num_pages;
  int32_t pw;
  const int32_t* a_indptr;
  const int32_t* a_pages;
  const int32_t* b_indptr;
  const int32_t* b_pages;
  int32_t d_in, d_out;
} oracle_tables;

/* A[i][k] of adapter a (d_in x r orientation).  Returns 0 and sets *out, or
 * -1 when the table points outside the pool. */
static int a_elem(const oracle_tables* tb, int32_t a, int32_t i, int32_t k, float* out) {
  int64_t ncol = ceil_div(tb->d_in, tb->pw);
  int64_t slot = (int64_t)tb->a_indptr[a] + (k / 16) * ncol + i / tb->pw;
  int32_t page = tb->a_pages[slot];
  if (page < 0 || page >= tb->num_pages) return -1;
  int64_t off = (int64_t)page * 16 * tb->pw + (int64_t)(k % 16) * tb->pw + (i % tb->pw);
  *out = load_elem(tb->pool, tb->dtype, off);
  return 0;
}

/* B[k][j] of adapter a (r x d_out orientation). */
static int b_elem(const oracle_tables* tb, int32_t a, int32_t k, int32_t j, float* out) {
  int64_t ncol = ceil_div(tb->d_out, tb->pw);
  int64_t slot = (int64_t)tb->b_indptr[a] + (k / 16) * ncol + j / tb->pw;
  int32_t page = tb->b_pages[slot];
  if (page < 0 || page >= tb->num_pages) return -1;
  int64_t off = (int64_t)page * 16 * tb->pw + (int64_t)((k % 16) / 8) * 8 * tb->pw + (int64_t)(j % tb->pw) * 8 +
                (k % 8);
  *out = load_elem(tb->pool, tb->dtype, off);
  return 0;
}

static oracle_tables make_tables(const void* pool, int dtype, int32_t num_pages, int32_t pw,
                                 const int32_t* a_indptr, const int32_t* a_pages,
                                 const int32_t* b_indptr, const int32_t* b_pages,
                                 int32_t d_in, int32_t d_out) {
  oracle_tables tb;
  tb.pool = pool; tb.dtype = dtype; tb.num_pages = num_pages; tb.pw = pw;
  tb.a_indptr = a_indptr; tb.a_pages = a_pages; tb.b_indptr = b_indptr; tb.b_pages = b_pages;
  tb.d_in = d_in; tb.d_out = d_out;
  return tb;
}

/* Dense copies of one adapter's A (d_in x r, row-major) and B (r x d_out),
 * read element by element through the page tables. */
int oracle_gather_adapter(const void* pool, int dtype, int32_t num_pages, int32_t pw,
                          const int32_t* a_indptr, const int32_t* a_pages,
                          const int32_t* b_indptr, const int32_t* b_pages,
                          int32_t d_in, int32_t d_out, int32_t a, int32_t r,
                          float* A_out, float* B_out) {
  oracle_tables tb = make_tables(pool, dtype, num_pages, pw, a_indptr, a_pages, b_indptr,
                                 b_pages, d_in, d_out);
  for (int32_t i = 0; i < d_in; ++i)
    for (int32_t k = 0; k < r; ++k)
      if (a_elem(&tb, a, i, k, &A_out[(int64_t)i * r + k])) return -3;
  for (int32_t k = 0; k < r; ++k)
    for (int32_t j = 0; j < d_out; ++j)
      if (b_elem(&tb, a, k, j, &B_out[(int64_t)k * d_out + j])) return -3;
  return 0;
}

/* ------------------------------------------------------- shrink, one token
 * v[k] = sum_i X[t][i] * A_a[i][k], k < r_a  ([MLSP] SGMV shrink). */
static int token_shrink(const oracle_tables* tb, const void* X, int dtype, int64_t ldx,
                        int32_t t, int32_t a, int32_t r, float* v) {
  for (int32_t k = 0; k < r; ++k) {
    float acc = 0.0f;
    for (int32_t i = 0; i < tb->d_in; ++i) {
      float w;
      if (a_elem(tb, a, i, k, &w)) return -3;
      acc += load_elem(X, dtype, (int64_t)t * ldx + i) * w;
    }
    v[k] = acc;
  }
  return 0;
}

/* -------------------------------------------------------------- apply
 * Y[t][j] = round(Y_base[t][j] + s * sum_k v[k] * B_a[k][j]),  s = alpha/r
 * ([MLSP] SGMV expand: scaled by alpha_i/r_i and added to the base output).
 * Tokens without a valid adapter copy Y_base.  OpenMP over tokens only: each
 * token's arithmetic is the same sequential loop whatever the thread count.
 * Returns 0, or -3 if a page index lies outside the pool. */
int oracle_apply(int32_t T, int32_t d_in, int32_t d_out, int dtype,
                 const void* X, int64_t ldx, const void* Y_base, int64_t ldyb,
                 void* Y, int64_t ldy, const int32_t* ids, int32_t N,
                 const int32_t* rank, const float* alpha,
                 const int32_t* a_indptr, const int32_t* a_pages,
                 const int32_t* b_indptr, const int32_t* b_pages,
                 const void* pool, int32_t num_pages, int32_t pw, int32_t nthreads) {
  if (T < 0 || d_in <= 0 || d_out <= 0 || pw <= 0) return -1;
  oracle_tables tb = make_tables(pool, dtype, num_pages, pw, a_indptr, a_pages, b_indptr,
                                 b_pages, d_in, d_out);
  int status = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int32_t t = 0; t < T; ++t) {
    float v[ORACLE_MAX_RANK];
    int32_t a = ids[t];
    int ok = token_valid(a, N, rank);
    int32_t r = ok ? rank[a] : 0;
    float s = ok ? alpha[a] / (float)r : 0.0f;
    if (ok && token_shrink(&tb, X, dtype, ldx, t, a, r, v)) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = -3;
      continue;
    }
    for (int32_t j = 0; j < d_out; ++j) {
      float yb = load_elem(Y_base, dtype, (int64_t)t * ldyb + j);
      float y = yb;
      if (ok) {
        float acc = 0.0f;
        for (int32_t k = 0; k < r; ++k) {
          float w = 0.0f;
          if (b_elem(&tb, a, k, j, &w)) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = -3;
          }
          acc += v[k] * w;
        }
        y = yb + s * acc;
      }
      if (dtype == ORACLE_DT_BF16)
        ((uint16_t*)Y)[(int64_t)t * ldy + j] = float_to_bf16_bits(y);
      else
        ((float*)Y)[(int64_t)t * ldy + j] = y;
    }
  }
  return status;
}

/* v of every token in the grouped order of the segments: v_out[v_indptr[s] +
 * i*r + k] for the i-th token of segment s ([MLSP] SGMV shrink output). */
int oracle_shrink(int32_t d_in, int dtype, const void* X, int64_t ldx,
                  const int32_t* perm, const int32_t* seg_indptr, const int32_t* seg_adapter,
                  const int32_t* v_indptr, int32_t S, const int32_t* rank,
                  const int32_t* a_indptr, const int32_t* a_pages,
                  const void* pool, int32_t num_pages, int32_t pw, float* v_out, int32_t nthreads) {
  oracle_tables tb = make_tables(pool, dtype, num_pages, pw, a_indptr, a_pages, NULL, NULL,
                                 d_in, 1);
  int status = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int32_t s = 0; s < S; ++s) {
    int32_t a = seg_adapter[s], r = rank[a];
    for (int32_t i = seg_indptr[s]; i < seg_indptr[s + 1]; ++i) {
      float* v = v_out + v_indptr[s] + (int64_t)(i - seg_indptr[s]) * r;
      if (token_shrink(&tb, X, dtype, ldx, perm[i], a, r, v)) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
        status = -3;
      }
    }
  }
  return status;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
