/*
 * sgb_oracle.c -- CPU reference ("oracle") for the pooled embedding-bag
 * backward with deduplication by sort + run-length encoding.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or constant with the GPU library: every rule below is
 * restated here from the pages, in plain single-threaded loops with double
 * precision accumulation, rounded once to fp32 where an fp32 result is asked
 * for.
 *
 * Sources (pages by title; sections named by the kernel or function they
 * fall in):
 *  [P1] "fbgemm_gpu/codegen/embedding_backward_split_template.cu" (FBGEMM):
 *       host entry `..._exact_cuda`, kernels `grad_mean_kernel`,
 *       `find_long_segments`, `..._kernel_cta_per_row_1`,
 *       `..._kernel_warp_per_row_1`.
 *  [P2] "tt_embeddings_cuda.cu" (FBTT-Embedding): `compute_rowidx_kernel`,
 *       `cache_backward_dense_kernel`, `cache_backward_sgd_kernel`,
 *       `cache_backward_rowwise_adagrad_approx_kernel`,
 *       `update_tt_cores_adagrad_kernel`.
 *  [P3] "Function _embedding_bwd_kernel" (tinygrad nn/__init__.py).
 *
 * Readings taken where the pages are silent are listed next to the code that
 * takes them (marked "Reading").
 *
 * Every function here is pinned by the CPU test suite against something other
 * than itself: hand-worked cases, a dense one-hot matrix product, the mass
 * invariant, closed forms of the optimizer steps and brute-force run
 * structure; the bf16 weight rows by the generator's published known-answer
 * vectors, torch's fp32 -> bf16 conversion, exhaustive rounding counts and
 * binomial bounds; the fp16 rows by numpy's and torch's IEEE fp32 -> fp16
 * conversion, exhaustive rounding counts and closed forms.  No function is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status codes of the oracle (its own; the test suite maps them by name). */
enum {
  ORC_OK = 0,
  ORC_INVALID_ARGUMENT = 1,
  ORC_UNSUPPORTED = 2,
  ORC_INDEX_OUT_OF_RANGE = 4,
  ORC_BAD_OFFSETS = 5
};

enum { ORC_POOL_SUM = 0, ORC_POOL_MEAN = 1, ORC_POOL_NONE = 2 };
enum { ORC_DENSE = 0, ORC_SGD = 1, ORC_ROWWISE_ADAGRAD = 2 };

/* One backward problem, all arrays on the host. */
typedef struct {
  int32_t T;                      /* number of tables, > 0                  */
  int32_t B;                      /* bags per table (bag mode), > 0         */
  int64_t N;                      /* number of lookups                      */
  const int64_t* hash_size_cumsum;/* [T+1], [0]=0, strictly increasing      */
  const int32_t* D_offsets;       /* [T+1], column start of table t in a bag
                                     row of grad_output                     */
  const int64_t* offsets;         /* [B*T+1], table-major (t*B+b); may be
                                     NULL only for nobag with T == 1        */
  const int64_t* indices;         /* [N], row index within the table        */
  const float* per_sample_weights;/* [N] or NULL                            */
  int32_t pooling;                /* ORC_POOL_*                             */
  const void* grad_output;        /* bag: [B][D_offsets[T]]; nobag: [N][D]  */
  int32_t grad_is_bf16;           /* 0: fp32, 1: bf16 bit patterns (uint16) */
} orc_problem;

/* ------------------------------------------------------------------------ */
/* Small helpers                                                              */
/* ------------------------------------------------------------------------ */

/* bf16 -> fp32 is exact: the 16 bits are the top half of an fp32. */
static double orc_bf16_to_double(uint16_t h) {
  uint32_t bits = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Element (row, col) of grad_output with `width` columns per row, widened. */
static double orc_grad(const orc_problem* p, int64_t row, int64_t width,
                       int64_t col) {
  if (p->grad_is_bf16) {
    const uint16_t* g = (const uint16_t*)p->grad_output;
    return orc_bf16_to_double(g[row * width + col]);
  }
  const float* g = (const float*)p->grad_output;
  return (double)g[row * width + col];
}

static int orc_table_D(const orc_problem* p, int32_t t) {
  return p->D_offsets[t + 1] - p->D_offsets[t];
}

/* Bag (t, b) spans lookups [offsets[t*B+b], offsets[t*B+b+1]) -- table-major
 * bag order [P1 `grad_mean_kernel` reads offsets[t * B + b]; P2
 * `compute_rowidx_kernel` writes rowidx = bag % B, tableidx = bag / B].
 * Nobag with no offsets array and a single table: every lookup is its own
 * segment of table 0. */
static void orc_bag_range(const orc_problem* p, int32_t t, int32_t b,
                          int64_t* s, int64_t* e) {
  if (p->offsets == NULL) {
    *s = 0;
    *e = p->N;
    return;
  }
  *s = p->offsets[(int64_t)t * p->B + b];
  *e = p->offsets[(int64_t)t * p->B + b + 1];
}

static int32_t orc_num_bags(const orc_problem* p) {
  return p->offsets == NULL ? 1 : p->B;
}

/* ------------------------------------------------------------------------ */
/* Validation                                                                 */
/* ------------------------------------------------------------------------ */

/* Checks the host entry makes or implies [P1 host entry `..._exact_cuda`:
 * T > 0, B > 0, offsets has B*T+1 entries; P2 host wrappers: D % 4 == 0],
 * plus the readings:
 *  - Reading: offsets start at 0, never decrease and end at N (a bag is a
 *    contiguous range of the indices array).
 *  - Reading: an index outside [0, E_t) is an error.  The FBGEMM page does
 *    not check; the tinygrad page clips.  We neither clip nor ignore.
 *  - Reading: 4 <= D_t <= 8192 and D_t % 4 == 0 (the pages read rows in
 *    groups of 4; 8192 is this library's stated maximum).
 *  - Nobag exists only unweighted [P1: the nobag variant is generated only
 *    when not weighted].  Nobag tables share one D [P1 nobag kernels take a
 *    single D].
 *  - hash_size_cumsum starts at 0 and strictly increases (no empty and no
 *    shared tables).
 */
static int orc_validate_lookups(const orc_problem* p);

int orc_validate(const orc_problem* p) {
  if (p->N > 0 && p->grad_output == NULL) return ORC_INVALID_ARGUMENT;
  return orc_validate_lookups(p);
}

/* The rules above except the gradient buffer (the forward reads weights). */
static int orc_validate_lookups(const orc_problem* p) {
  if (p->T <= 0 || p->N < 0 || p->hash_size_cumsum == NULL ||
      p->D_offsets == NULL)
    return ORC_INVALID_ARGUMENT;
  if (p->pooling < ORC_POOL_SUM || p->pooling > ORC_POOL_NONE)
    return ORC_INVALID_ARGUMENT;
  const int nobag = p->pooling == ORC_POOL_NONE;
  if (nobag && p->per_sample_weights != NULL) return ORC_UNSUPPORTED;
  if (p->offsets == NULL && !(nobag && p->T == 1)) return ORC_INVALID_ARGUMENT;
  if (p->offsets != NULL && p->B <= 0) return ORC_INVALID_ARGUMENT;
  if (p->hash_size_cumsum[0] != 0) return ORC_INVALID_ARGUMENT;
  if (p->D_offsets[0] != 0) return ORC_INVALID_ARGUMENT;
  for (int32_t t = 0; t < p->T; ++t) {
    if (p->hash_size_cumsum[t + 1] <= p->hash_size_cumsum[t])
      return ORC_INVALID_ARGUMENT;
    int D = orc_table_D(p, t);
    if (D < 4 || D > 8192 || D % 4 != 0) return ORC_INVALID_ARGUMENT;
    if (nobag && D != orc_table_D(p, 0)) return ORC_INVALID_ARGUMENT;
  }
  if (p->N > 0 && p->indices == NULL) return ORC_INVALID_ARGUMENT;
  if (p->offsets != NULL) {
    int64_t nb = (int64_t)p->B * p->T;
    if (p->offsets[0] != 0 || p->offsets[nb] != p->N) return ORC_BAD_OFFSETS;
    for (int64_t k = 0; k < nb; ++k)
      if (p->offsets[k + 1] < p->offsets[k]) return ORC_BAD_OFFSETS;
  }
  for (int32_t t = 0; t < p->T; ++t) {
    int64_t E = p->hash_size_cumsum[t + 1] - p->hash_size_cumsum[t];
    for (int32_t b = 0; b < orc_num_bags(p); ++b) {
      int64_t s, e;
      orc_bag_range(p, t, b, &s, &e);
      for (int64_t i = s; i < e; ++i)
        if (p->indices[i] < 0 || p->indices[i] >= E)
          return ORC_INDEX_OUT_OF_RANGE;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Per-lookup linear id, info and coefficient, in original order             */
/* ------------------------------------------------------------------------ */

/* For lookup i of bag (t, b):
 *   key  = hash_size_cumsum[t] + indices[i]
 *          (Reading: the inverse of the kernels' `idx = linear_index -
 *          hash_size_cumsum[t_0]` [P1 `..._kernel_warp_per_row_1`]);
 *   info = t*B + b in bag mode, i*T + t in nobag mode [P1 kernels decode
 *          `b_t` into (t, b) with a divisor B, and nobag `l_t` into
 *          l = l_t / T, t = l_t % T];
 *   coef = (per-sample weight or 1) * (1/L under MEAN pooling, L > 0)
 *          [P1 `grad_mean_kernel` scales the bag's output gradient by 1/L
 *          and leaves empty bags alone; the weighted kernels multiply by the
 *          sorted per-sample weight].  Reading: the two compose.
 * Requires a valid problem (orc_validate == ORC_OK). */
int orc_linearize(const orc_problem* p, int64_t* keys, int64_t* infos,
                  double* coefs) {
  int st = orc_validate(p);
  if (st != ORC_OK) return st;
  const int nobag = p->pooling == ORC_POOL_NONE;
  for (int32_t t = 0; t < p->T; ++t) {
    for (int32_t b = 0; b < orc_num_bags(p); ++b) {
      int64_t s, e;
      orc_bag_range(p, t, b, &s, &e);
      int64_t L = e - s;
      double scale = (p->pooling == ORC_POOL_MEAN && L > 0) ? 1.0 / (double)L
                                                            : 1.0;
      for (int64_t i = s; i < e; ++i) {
        keys[i] = p->hash_size_cumsum[t] + p->indices[i];
        infos[i] = nobag ? i * (int64_t)p->T + t : (int64_t)t * p->B + b;
        double w = p->per_sample_weights ? (double)p->per_sample_weights[i]
                                         : 1.0;
        coefs[i] = w * scale;
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Run structure: stable sort, run-length encoding, long runs                 */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t key;
  int64_t pos;
} orc_keypos;

static int orc_cmp_keypos(const void* a, const void* b) {
  const orc_keypos* x = (const orc_keypos*)a;
  const orc_keypos* y = (const orc_keypos*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
  return 0;
}

/* Sorts the lookups by linear id, keeping the original order among equal
 * ids (Reading: the page re-sorts the per-sample weights by the same keys in
 * a second pass and expects them to line up with the sorted infos, which
 * only holds for a stable sort [P1 host entry, weighted branch]).  Then:
 *   unique_ids[r]       the r-th distinct id, ascending;
 *   cumulative[r]       position of its first lookup, cumulative[U] = N;
 *   run_lengths[r]      cumulative[r+1] - cumulative[r];
 *   long_run_ids        { r : run_lengths[r] >= thr }, ascending
 *                       [P1 `find_long_segments` uses >=; the page emits the
 *                       set in atomic-counter order, we list it ascending].
 * Sorted keys/infos/positions are written in sorted order.  `thr` >= 1. */
int orc_runs(int64_t N, const int64_t* keys, const int64_t* infos, int64_t thr,
             int64_t* sorted_keys, int64_t* sorted_infos, int64_t* sorted_pos,
             int64_t* unique_ids, int64_t* run_lengths, int64_t* cumulative,
             int64_t* num_runs, int64_t* long_run_ids, int64_t* num_long) {
  if (N < 0 || thr < 1) return ORC_INVALID_ARGUMENT;
  orc_keypos* kp = (orc_keypos*)malloc(sizeof(orc_keypos) * (size_t)(N > 0 ? N : 1));
  if (kp == NULL) return ORC_INVALID_ARGUMENT;
  for (int64_t i = 0; i < N; ++i) {
    kp[i].key = keys[i];
    kp[i].pos = i;
  }
  qsort(kp, (size_t)N, sizeof(orc_keypos), orc_cmp_keypos);
  int64_t U = 0;
  for (int64_t i = 0; i < N; ++i) {
    sorted_keys[i] = kp[i].key;
    sorted_infos[i] = infos[kp[i].pos];
    sorted_pos[i] = kp[i].pos;
    if (i == 0 || kp[i].key != kp[i - 1].key) {
      unique_ids[U] = kp[i].key;
      cumulative[U] = i;
      ++U;
    }
  }
  cumulative[U] = N;
  int64_t nl = 0;
  for (int64_t r = 0; r < U; ++r) {
    run_lengths[r] = cumulative[r + 1] - cumulative[r];
    if (run_lengths[r] >= thr) long_run_ids[nl++] = r;
  }
  *num_runs = U;
  *num_long = nl;
  free(kp);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Aggregated row gradients                                                   */
/* ------------------------------------------------------------------------ */

static int64_t orc_find(const int64_t* sorted, int64_t n, int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (sorted[mid] < x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return (lo < n && sorted[lo] == x) ? lo : -1;
}

/* G[k][d] = sum over lookups i with linear id rows[k] of
 *           coef_i * grad_output[b_i][D_offsets[t] + d]     (bag mode)
 *           grad_output[i][d]                                (nobag)
 * for d < D_t, accumulated in double; columns d >= D_t are left 0.
 * This is the plain definition the pages' kernels compute: the dense
 * gradient kernel adds every occurrence's output-gradient row into the
 * table row [P2 `cache_backward_dense_kernel`; P3 `_embedding_bwd_kernel`,
 * which also widens a 16-bit gradient to fp32 first], with the bag's mean
 * scale [P1 `grad_mean_kernel`] and per-sample weight [P1 weighted kernels]
 * folded in.  `rows` must be sorted ascending and distinct; `hits[k]` gets
 * the number of lookups of rows[k]. */
int orc_row_grads(const orc_problem* p, int64_t nreq, const int64_t* rows,
                  int32_t ldg, double* G, int64_t* hits) {
  int st = orc_validate(p);
  if (st != ORC_OK) return st;
  for (int64_t k = 1; k < nreq; ++k)
    if (rows[k] <= rows[k - 1]) return ORC_INVALID_ARGUMENT;
  memset(G, 0, sizeof(double) * (size_t)nreq * (size_t)ldg);
  memset(hits, 0, sizeof(int64_t) * (size_t)nreq);
  const int nobag = p->pooling == ORC_POOL_NONE;
  const int64_t width = p->D_offsets[p->T];
  for (int32_t t = 0; t < p->T; ++t) {
    const int D = orc_table_D(p, t);
    if (D > ldg) return ORC_INVALID_ARGUMENT;
    for (int32_t b = 0; b < orc_num_bags(p); ++b) {
      int64_t s, e;
      orc_bag_range(p, t, b, &s, &e);
      int64_t L = e - s;
      double scale = (p->pooling == ORC_POOL_MEAN && L > 0) ? 1.0 / (double)L
                                                            : 1.0;
      for (int64_t i = s; i < e; ++i) {
        int64_t k = orc_find(rows, nreq, p->hash_size_cumsum[t] + p->indices[i]);
        if (k < 0) continue;
        hits[k] += 1;
        double* g = G + k * (int64_t)ldg;
        if (nobag) {
          for (int d = 0; d < D; ++d) g[d] += orc_grad(p, i, D, d);
        } else {
          double c = scale * (p->per_sample_weights
                                  ? (double)p->per_sample_weights[i]
                                  : 1.0);
          for (int d = 0; d < D; ++d)
            g[d] += c * orc_grad(p, b, width, p->D_offsets[t] + d);
        }
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Row updates                                                                */
/* ------------------------------------------------------------------------ */

/* Applies the output step to `nrows` rows, once per distinct row, on the
 * aggregated gradient G (row k has D[k] columns, leading dimension ldg):
 *  ORC_DENSE, accumulate=0: out = G, the fresh dense gradient whose other
 *        rows are zero [P1 host entry: grad_dev_weights = zeros_like(...),
 *        kernels store grad_sum into the row].
 *  ORC_DENSE, accumulate=1: out = out0 + G [P3 adds into grad_weight].
 *  ORC_SGD: w = w0 - lr * G [P2 `cache_backward_sgd_kernel`,
 *        `update_tt_cores_sgd_kernel`].
 *  ORC_ROWWISE_ADAGRAD: m = m0 + (1/D) * sum_d G[d]^2;
 *        w = w0 - lr * G / (sqrt(m) + eps)
 *        [P2 `cache_backward_rowwise_adagrad_approx_kernel`: the state grows
 *        by the mean square of the row gradient and the multiplier uses the
 *        grown state, with eps outside the square root, as also in
 *        `update_tt_cores_adagrad_kernel`].  Reading: applied once per
 *        distinct row on the summed gradient (the "exact" method), not once
 *        per occurrence as the approximate page kernel does.
 * Everything is computed in double and rounded once to fp32.
 * rows: in/out [nrows][ldg] (w0/out0 in, result out); mom: in/out [nrows]. */
int orc_update_rows(int32_t mode, int32_t accumulate, int64_t nrows,
                    const int32_t* D, int32_t ldg, const double* G, float lr,
                    float eps, float* rows, float* mom) {
  for (int64_t k = 0; k < nrows; ++k) {
    const double* g = G + k * (int64_t)ldg;
    float* w = rows + k * (int64_t)ldg;
    const int Dk = D[k];
    if (Dk <= 0 || Dk > ldg) return ORC_INVALID_ARGUMENT;
    if (mode == ORC_DENSE) {
      for (int d = 0; d < Dk; ++d)
        w[d] = accumulate ? (float)((double)w[d] + g[d]) : (float)g[d];
    } else if (mode == ORC_SGD) {
      for (int d = 0; d < Dk; ++d)
        w[d] = (float)((double)w[d] - (double)lr * g[d]);
    } else if (mode == ORC_ROWWISE_ADAGRAD) {
      double sumsq = 0.0;
      for (int d = 0; d < Dk; ++d) sumsq += g[d] * g[d];
      double m = (double)mom[k] + sumsq / (double)Dk;
      double mult = (double)lr / (sqrt(m) + (double)eps);
      for (int d = 0; d < Dk; ++d)
        w[d] = (float)((double)w[d] - g[d] * mult);
      mom[k] = (float)m;
    } else {
      return ORC_INVALID_ARGUMENT;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Pooled forward                                                             */
/* ------------------------------------------------------------------------ */

/* The pooled lookup that the backward above differentiates:
 *   out[b][D_offsets[t] + d] = sum over lookups i of bag (t, b) of
 *                              coef_i * W_t[indices[i]][d]        (bag mode)
 *   out[i][d]                = W_t[indices[i]][d]                 (nobag)
 * for d < D_t, with coef_i = per_sample_weights[i] (or 1) times 1/L for a
 * mean bag of L lookups; an empty bag gives a zero row.  The FBTT cache
 * forward sums the weight rows of a segment's lookups into the segment's
 * output row [P2 `cache_forward_kernel`]; the mean scale and the per-sample
 * weight are the factors the backward applies [P1 `grad_mean_kernel`,
 * weighted kernels], so forward and backward are adjoint.
 * W is one flat fp32 array, table t from woff[t] = sum_{t'<t} E_t' * D_t',
 * row-major.  out is [B][D_offsets[T]] (bag) or [N][D] (nobag).  Sums in
 * double, rounded once to fp32. */
int orc_forward(const orc_problem* p, const float* W, float* out) {
  int st = orc_validate_lookups(p);
  if (st != ORC_OK) return st;
  if (W == NULL || out == NULL) return ORC_INVALID_ARGUMENT;
  const int nobag = p->pooling == ORC_POOL_NONE;
  const int64_t width = nobag ? (int64_t)orc_table_D(p, 0) : (int64_t)p->D_offsets[p->T];
  const int64_t rows = nobag ? p->N : (int64_t)orc_num_bags(p);
  memset(out, 0, sizeof(float) * (size_t)(rows * width));
  double* acc = (double*)malloc(sizeof(double) * 8192);
  if (acc == NULL) return ORC_INVALID_ARGUMENT;
  int64_t woff = 0;
  for (int32_t t = 0; t < p->T; ++t) {
    const int D = orc_table_D(p, t);
    const int64_t E = p->hash_size_cumsum[t + 1] - p->hash_size_cumsum[t];
    for (int32_t b = 0; b < orc_num_bags(p); ++b) {
      int64_t s, e;
      orc_bag_range(p, t, b, &s, &e);
      const int64_t L = e - s;
      const double scale = (p->pooling == ORC_POOL_MEAN && L > 0) ? 1.0 / (double)L : 1.0;
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      for (int64_t i = s; i < e; ++i) {
        const float* wr = W + woff + p->indices[i] * (int64_t)D;
        if (nobag) {
          for (int d = 0; d < D; ++d) out[i * width + d] = wr[d];
          continue;
        }
        const double c = scale * (p->per_sample_weights ? (double)p->per_sample_weights[i] : 1.0);
        for (int d = 0; d < D; ++d) acc[d] += c * (double)wr[d];
      }
      if (!nobag)
        for (int d = 0; d < D; ++d) out[(int64_t)b * width + p->D_offsets[t] + d] = (float)acc[d];
    }
    woff += E * (int64_t)D;
  }
  free(acc);
  return ORC_OK;
}


/* ------------------------------------------------------------------------ */
/* bf16 weight rows: round to nearest even, or stochastic rounding          */
/* ------------------------------------------------------------------------ */

/* The FBGEMM page stores an updated row into 16-bit weights with stochastic
 * rounding when asked for it, drawing from a Philox generator seeded per
 * call [P1, the split-kernel weight store: `stochastic_rounding_init`, the
 * row's `set_stoc_state`]; the bodies of the rounding and of the state are
 * not printed.  Readings:
 *  - the generator is Philox4x32-10 as published (Salmon, Moraes, Dror and
 *    Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): 10 rounds,
 *    multipliers 0xD2511F53 / 0xCD9E8D57, key increments 0x9E3779B9 /
 *    0xBB67AE85, the key bumped before every round after the first;
 *  - the element (linear row id r, column d) takes word d % 4 of the block
 *    with counter (d / 4, r mod 2^32, r / 2^32, offset) and key
 *    (seed mod 2^32, seed / 2^32): one block per 4 columns of a row, so the
 *    bits depend on the row and column and not on any launch shape;
 *  - the fp32 result of the update (computed as for fp32 rows, rounded once
 *    to fp32) is rounded to bf16 stochastically by adding the word's high 16
 *    bits to the fp32 bit pattern and keeping the high half: the magnitude
 *    rounds up with probability (dropped bits) / 2^16, so the rounding is
 *    unbiased; without stochastic rounding it is round-to-nearest-even;
 *  - infinities keep their high half, NaNs stay (quiet) NaNs. */

static uint32_t orc_mulhi32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * (uint64_t)b) >> 32);
}

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = orc_mulhi32(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = orc_mulhi32(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static uint32_t orc_f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}

/* non-finite: keep the high half; a NaN keeps its quiet bit set */
static int orc_bf16_special(uint32_t u, uint16_t* h) {
  if ((u & 0x7F800000u) != 0x7F800000u) return 0;
  *h = (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x0040u : 0u));
  return 1;
}

uint16_t orc_bf16_rne(float x) {
  const uint32_t u = orc_f32_bits(x);
  uint16_t h;
  if (orc_bf16_special(u, &h)) return h;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

uint16_t orc_bf16_sr(float x, uint32_t rnd) {
  const uint32_t u = orc_f32_bits(x);
  uint16_t h;
  if (orc_bf16_special(u, &h)) return h;
  return (uint16_t)((u + (rnd >> 16)) >> 16);
}

/* Rounds n fp32 values; rnd == NULL: nearest even, else stochastic with rnd[i]. */
void orc_bf16_round_array(const float* x, const uint32_t* rnd, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = rnd ? orc_bf16_sr(x[i], rnd[i]) : orc_bf16_rne(x[i]);
}

/* The Philox word of element (row, col), as read above. */
static uint32_t orc_sr_word(uint64_t seed, uint32_t offset, int64_t row, int col) {
  const uint32_t ctr[4] = {(uint32_t)(col >> 2), (uint32_t)(uint64_t)row,
                           (uint32_t)((uint64_t)row >> 32), offset};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return out[col & 3];
}

/* SGD or row-wise Adagrad on bf16 rows: each row is widened exactly to fp32,
 * updated as orc_update_rows does (fp64, rounded once to fp32), and rounded
 * to bf16.  rows: [nrows][ldg] bf16 bit patterns, updated in place; row_ids:
 * the rows' linear ids (the stochastic-rounding counter). */
int orc_update_rows_bf16(int32_t mode, int64_t nrows, const int32_t* D, int32_t ldg,
                         const double* G, float lr, float eps, uint16_t* rows, float* mom,
                         const int64_t* row_ids, int32_t stochastic, uint64_t seed,
                         uint32_t offset) {
  if (mode != ORC_SGD && mode != ORC_ROWWISE_ADAGRAD) return ORC_INVALID_ARGUMENT;
  float* tmp = (float*)malloc(sizeof(float) * (size_t)(ldg > 0 ? ldg : 1));
  if (tmp == NULL) return ORC_INVALID_ARGUMENT;
  int st = ORC_OK;
  for (int64_t k = 0; k < nrows && st == ORC_OK; ++k) {
    uint16_t* h = rows + k * (int64_t)ldg;
    const int Dk = D[k];
    if (Dk <= 0 || Dk > ldg) {
      st = ORC_INVALID_ARGUMENT;
      break;
    }
    for (int d = 0; d < Dk; ++d) {
      const uint32_t u = ((uint32_t)h[d]) << 16;
      memcpy(&tmp[d], &u, 4);
    }
    st = orc_update_rows(mode, 0, 1, &D[k], ldg, G + k * (int64_t)ldg, lr, eps, tmp,
                         mom ? &mom[k] : NULL);
    for (int d = 0; d < Dk && st == ORC_OK; ++d)
      h[d] = stochastic ? orc_bf16_sr(tmp[d], orc_sr_word(seed, offset, row_ids[k], d))
                        : orc_bf16_rne(tmp[d]);
  }
  free(tmp);
  return st;
}

/* ------------------------------------------------------------------------ */
/* fp16 weight rows: round to nearest even, or stochastic rounding          */
/* ------------------------------------------------------------------------ */

/* The page's 16-bit weight rows may also be IEEE binary16 (fp16).  Readings
 * (the rounding bodies are not printed; the generator and the element's
 * random word are those read above for bf16 rows):
 *  - the grid: binary16 values, spacing u = 2^(e - 10) in binade
 *    [2^e, 2^(e+1)) for e >= -14 and u = 2^-24 below 2^-14 (gradual
 *    underflow), continued without an upper bound; a magnitude above the
 *    largest finite value 65504 becomes infinity;
 *  - nearest even: IEEE 754 rounding to that grid (so 65520, the midpoint
 *    above 65504, and anything larger become infinity);
 *  - stochastic: with lo the grid point at or below |x| and f = (|x| - lo)
 *    / u, the magnitude rounds up to lo + u iff the element's full 32-bit
 *    word w satisfies w < f * 2^32 (probability f, so the rounding is
 *    unbiased where no overflow occurs);
 *  - infinities keep their sign; a NaN becomes the quiet NaN 0x7E00 with its
 *    sign. */

/* Grid point at or below a >= 0 (as a count q of spacings u) and the
 * fraction of a spacing above it; all exact in double for an fp32 a. */
static double orc_f16_grid(double a, double* u, double* frac) {
  if (a < ldexp(1.0, -14)) {
    *u = ldexp(1.0, -24);
  } else {
    int k;
    (void)frexp(a, &k);  /* a = m * 2^k, m in [0.5, 1): binade e = k - 1 */
    *u = ldexp(1.0, k - 1 - 10);
  }
  const double q = floor(a / *u);
  *frac = a / *u - q;
  return q;
}

/* binary16 bits of sign and magnitude v (a grid point, or beyond 65504) */
static uint16_t orc_f16_encode(int neg, double v) {
  const uint16_t s = neg ? 0x8000u : 0u;
  if (v > 65504.0) return (uint16_t)(s | 0x7C00u);
  if (v < ldexp(1.0, -14)) return (uint16_t)(s | (uint16_t)(v * ldexp(1.0, 24)));
  int k;
  (void)frexp(v, &k);
  const int e = k - 1;
  const uint16_t mant = (uint16_t)((v / ldexp(1.0, e) - 1.0) * 1024.0);
  return (uint16_t)(s | (uint16_t)((e + 15) << 10) | mant);
}

/* non-finite inputs; returns 1 when x was one */
static int orc_f16_special(float x, uint16_t* h) {
  if (isnan(x)) {
    *h = (uint16_t)((signbit(x) ? 0x8000u : 0u) | 0x7E00u);
    return 1;
  }
  if (isinf(x)) {
    *h = (uint16_t)((x < 0 ? 0x8000u : 0u) | 0x7C00u);
    return 1;
  }
  return 0;
}

uint16_t orc_f16_rne(float x) {
  uint16_t h;
  if (orc_f16_special(x, &h)) return h;
  double u, f;
  const double a = fabs((double)x);
  double q = orc_f16_grid(a, &u, &f);
  if (f > 0.5 || (f == 0.5 && fmod(q, 2.0) == 1.0)) q += 1.0;
  return orc_f16_encode(signbit(x) != 0, q * u);
}

uint16_t orc_f16_sr(float x, uint32_t rnd) {
  uint16_t h;
  if (orc_f16_special(x, &h)) return h;
  double u, f;
  const double a = fabs((double)x);
  double q = orc_f16_grid(a, &u, &f);
  if ((double)rnd < f * 4294967296.0) q += 1.0;
  return orc_f16_encode(signbit(x) != 0, q * u);
}

/* binary16 -> fp32, exact */
static float orc_f16_to_f32(uint16_t h) {
  const int neg = (h >> 15) & 1, ex = (h >> 10) & 31, man = h & 1023;
  double v;
  if (ex == 31) v = man ? NAN : INFINITY;
  else if (ex == 0) v = ldexp((double)man, -24);
  else v = ldexp(1.0 + man / 1024.0, ex - 15);
  return (float)(neg ? -v : v);
}

/* Rounds n fp32 values; rnd == NULL: nearest even, else stochastic with rnd[i]. */
void orc_f16_round_array(const float* x, const uint32_t* rnd, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = rnd ? orc_f16_sr(x[i], rnd[i]) : orc_f16_rne(x[i]);
}

void orc_f16_widen_array(const uint16_t* h, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(h[i]);
}

/* SGD or row-wise Adagrad on fp16 rows: widened exactly to fp32, updated as
 * orc_update_rows does (fp64, rounded once to fp32), rounded to fp16.  rows:
 * [nrows][ldg] binary16 bit patterns, updated in place; row_ids: the rows'
 * linear ids (the stochastic-rounding counter). */
int orc_update_rows_f16(int32_t mode, int64_t nrows, const int32_t* D, int32_t ldg,
                        const double* G, float lr, float eps, uint16_t* rows, float* mom,
                        const int64_t* row_ids, int32_t stochastic, uint64_t seed,
                        uint32_t offset) {
  if (mode != ORC_SGD && mode != ORC_ROWWISE_ADAGRAD) return ORC_INVALID_ARGUMENT;
  float* tmp = (float*)malloc(sizeof(float) * (size_t)(ldg > 0 ? ldg : 1));
  if (tmp == NULL) return ORC_INVALID_ARGUMENT;
  int st = ORC_OK;
  for (int64_t k = 0; k < nrows && st == ORC_OK; ++k) {
    uint16_t* h = rows + k * (int64_t)ldg;
    const int Dk = D[k];
    if (Dk <= 0 || Dk > ldg) {
      st = ORC_INVALID_ARGUMENT;
      break;
    }
    for (int d = 0; d < Dk; ++d) tmp[d] = orc_f16_to_f32(h[d]);
    st = orc_update_rows(mode, 0, 1, &D[k], ldg, G + k * (int64_t)ldg, lr, eps, tmp,
                         mom ? &mom[k] : NULL);
    for (int d = 0; d < Dk && st == ORC_OK; ++d)
      h[d] = stochastic ? orc_f16_sr(tmp[d], orc_sr_word(seed, offset, row_ids[k], d))
                        : orc_f16_rne(tmp[d]);
  }
  free(tmp);
  return st;
}

/* ------------------------------------------------------------------------ */
/* INT8 row-wise quantized weight rows                                       */
/* ------------------------------------------------------------------------ */

/* The FBGEMM page keeps 8-bit rows with per-row quantization parameters
 * stored in the row (row width D + kINT8QparamsBytes), loads the row with
 * its parameters, and after the update computes new parameters from the
 * updated row (`thrust_find_qparams`) before storing it [P1, split-kernel
 * weight store]; the bodies are not printed.  Readings:
 *  - a row is D uint8 codes followed by two fp32 values, scale then bias
 *    (D + 8 bytes; D % 4 == 0, so the pair is 4-byte aligned);
 *  - a code c stands for fmaf(c, scale, bias) (fp32, fused);
 *  - the update is the fp32-row update (fp64, rounded once to fp32);
 *  - new parameters: bias = min of the updated row, scale = (max - min) / 255
 *    in fp32;
 *  - code = rint((w - bias) / scale) (fp32 subtraction and division, round
 *    half to even), clamped to [0, 255]; a constant row (scale 0) gets
 *    code 0. */

static float orc_i8_value(uint8_t c, float scale, float bias) {
  return fmaf((float)c, scale, bias);
}

static void orc_i8_quantize_row(const float* w, int D, uint8_t* row) {
  float mn = w[0], mx = w[0];
  for (int d = 1; d < D; ++d) {
    if (w[d] < mn) mn = w[d];
    if (w[d] > mx) mx = w[d];
  }
  const float scale = (mx - mn) / 255.0f;
  const float bias = mn;
  for (int d = 0; d < D; ++d) {
    float q = scale > 0.0f ? rintf((w[d] - bias) / scale) : 0.0f;
    if (q < 0.0f) q = 0.0f;
    if (q > 255.0f) q = 255.0f;
    row[d] = (uint8_t)q;
  }
  memcpy(row + D, &scale, 4);
  memcpy(row + D + 4, &bias, 4);
}

/* Quantizes n rows of D fp32 values into rows of D + 8 bytes. */
void orc_i8_quantize(const float* w, int64_t n, int32_t D, uint8_t* rows) {
  for (int64_t k = 0; k < n; ++k)
    orc_i8_quantize_row(w + k * (int64_t)D, D, rows + k * (int64_t)(D + 8));
}

/* Dequantizes n rows of D + 8 bytes into D fp32 values each. */
void orc_i8_dequantize(const uint8_t* rows, int64_t n, int32_t D, float* w) {
  for (int64_t k = 0; k < n; ++k) {
    const uint8_t* r = rows + k * (int64_t)(D + 8);
    float scale, bias;
    memcpy(&scale, r + D, 4);
    memcpy(&bias, r + D + 4, 4);
    for (int d = 0; d < D; ++d) w[k * (int64_t)D + d] = orc_i8_value(r[d], scale, bias);
  }
}

/* SGD or row-wise Adagrad on INT8 rows: rows[k] holds row k's D[k] codes and
 * its parameters at byte offset k * ldr (ldr >= D[k] + 8); the row is
 * dequantized, updated as orc_update_rows does, and quantized again. */
int orc_update_rows_int8(int32_t mode, int64_t nrows, const int32_t* D, int32_t ldg,
                         const double* G, float lr, float eps, uint8_t* rows, int32_t ldr,
                         float* mom) {
  if (mode != ORC_SGD && mode != ORC_ROWWISE_ADAGRAD) return ORC_INVALID_ARGUMENT;
  float* tmp = (float*)malloc(sizeof(float) * (size_t)(ldg > 0 ? ldg : 1));
  if (tmp == NULL) return ORC_INVALID_ARGUMENT;
  int st = ORC_OK;
  for (int64_t k = 0; k < nrows && st == ORC_OK; ++k) {
    const int Dk = D[k];
    if (Dk <= 0 || Dk > ldg || Dk + 8 > ldr) {
      st = ORC_INVALID_ARGUMENT;
      break;
    }
    uint8_t* r = rows + k * (int64_t)ldr;
    orc_i8_dequantize(r, 1, Dk, tmp);
    st = orc_update_rows(mode, 0, 1, &D[k], ldg, G + k * (int64_t)ldg, lr, eps, tmp,
                         mom ? &mom[k] : NULL);
    if (st == ORC_OK) orc_i8_quantize_row(tmp, Dk, r);
  }
  free(tmp);
  return st;
}
