/*
 * sgb_atomic.h -- C ABI of the atomic scatter-add backward (libsgb_atomic.so).
 *
 * A comparison baseline, kept out of libsgb.so: the design the deduplicated
 * path replaces.  Every lookup adds its bag's gradient row, scaled, straight
 * into the looked-up table row with fp32 atomic adds, with no sort and no
 * run-length encoding; lookups of a hot row contend on the same addresses and
 * the summation order (so the rounding) varies from run to run.
 *
 * Defining passages (pages by title, sections by kernel or function):
 *  - "tt_embeddings_cuda.cu" (FBTT-Embedding): `cache_backward_dense_kernel`
 *    (grad[row] += grad_output[bag], one atomic add per element) and
 *    `cache_backward_sgd_kernel` (w[row] += -lr * grad_output[bag]).
 *  - "Function _embedding_bwd_kernel" (tinygrad): the nobag form, an fp32
 *    atomic scatter-add of each token's (possibly 16-bit) gradient row into
 *    grad_weight, agent-scope relaxed atomics on AMD GPUs.
 * Pooling follows the same definitions as sgb.h: a lookup's coefficient is
 * its per-sample weight (1 without weights) times 1/L for a mean bag of L
 * lookups.  Row-wise Adagrad has no atomic form (its per-row state must be
 * grown once per distinct row before the row is written) and is not offered.
 *
 * Conventions: plain C, device pointers on the current HIP device, owned by
 * the caller; work is enqueued on `stream` (a hipStream_t as void*, NULL =
 * null stream) and the call returns at once.  Argument errors are detected on
 * the host before anything is enqueued (nothing is written).  The kernel does
 * not validate array contents: a lookup whose index lies outside its table is
 * skipped, and offsets are clamped to [0, num_indices], so no access leaves
 * the buffers; results for such inputs are unspecified.
 */
#ifndef SGB_ATOMIC_H
#define SGB_ATOMIC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SGB_ATOMIC_OK 0
#define SGB_ATOMIC_ERR_INVALID_ARGUMENT 1
#define SGB_ATOMIC_ERR_UNSUPPORTED 2
#define SGB_ATOMIC_ERR_HIP 3

/*
 * out[woff[t] + idx * D_t + d] += scale * coef_i * grad_output[row_i][col_t + d]
 * for every lookup i (of table t, index idx) and column d < D_t, by fp32
 * atomic adds.  Bag mode: row_i = b for a lookup of bag (t, b), col_t =
 * D_offsets[t]; nobag: row_i = i, col_t = 0.
 *
 *  T                  number of tables (> 0); nobag requires T == 1.
 *  hash_size_cumsum   device int64 [T+1]: table t holds rows
 *                     [hash_size_cumsum[t], hash_size_cumsum[t+1]) of the
 *                     linear id space (E_t = difference).
 *  D_offsets          device int32 [T+1]: column offsets; D_t % 4 == 0.
 *  table_offsets      device int64 [T+1]: element offset of table t in `out`
 *                     (sum of E_t' * D_t' over t' < t).
 *  max_D              host: the largest D_t (sets the launch shape), 4..8192.
 *  total_elems        host: elements of `out` (table_offsets[T]); used by
 *                     zero_first.
 *  pooling            0 sum, 1 mean, 2 none (nobag).
 *  grad_output        device, fp32 (grad_dtype 0) or bf16 (grad_dtype 1),
 *                     [B][D_offsets[T]] (bag) or [num_indices][D] (nobag),
 *                     16-byte aligned rows.
 *  indices            device int64 [num_indices], index within the table.
 *  offsets            device int64 [B*T+1], table-major (bag (t, b) covers
 *                     lookups [offsets[t*B+b], offsets[t*B+b+1]));
 *                     must be NULL for nobag.
 *  B                  bags per table (> 0) for bag mode; ignored for nobag.
 *  per_sample_weights device fp32 [num_indices] or NULL (NULL for nobag).
 *  out                device fp32 [total_elems]: dense gradient, or weights
 *                     for SGD (then scale = -lr); 16-byte aligned.
 *  scale              multiplies every added term.
 *  zero_first         nonzero: `out` is set to zero first (a fresh dense
 *                     gradient); 0: added into its current contents.
 */
int sgb_atomic_backward(int32_t T, const int64_t* hash_size_cumsum, const int32_t* D_offsets,
                        const int64_t* table_offsets, int32_t max_D, int64_t total_elems,
                        int32_t pooling, const void* grad_output, int32_t grad_dtype,
                        const int64_t* indices, int64_t num_indices, const int64_t* offsets,
                        int32_t B, const float* per_sample_weights, float* out, float scale,
                        int32_t zero_first, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SGB_ATOMIC_H */
