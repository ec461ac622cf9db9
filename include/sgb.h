/*
 * sgb.h -- C ABI of the MI355X (gfx950) pooled embedding-bag backward.
 *
 * The library computes the backward pass of pooled embedding bags: the
 * per-bag output gradient grad_output[B][sum_t D_t] (sum, mean or
 * per-sample-weighted pooling), or the per-token gradient [N][D] of the
 * unpooled ("nobag") case, is scattered onto the table rows named by
 * (indices, offsets).  The work is deduplicated: linear row ids are sorted,
 * run-length encoded, and each run (one distinct row) is reduced once, then
 * written once as a dense fp32 gradient row or as an in-place SGD or
 * row-wise Adagrad update.
 *
 * Defining passages (pages by title, sections by kernel or function):
 *  - "fbgemm_gpu/codegen/embedding_backward_split_template.cu" (FBGEMM):
 *    host entry `split_embedding{_nobag}_backward_codegen_{opt}_{w}_exact_cuda`
 *    (argument list, checks T > 0 and B > 0, empty-input early return,
 *    table-major offsets of length B*T+1, `hash_size_cumsum`, `D_offsets`,
 *    `max_segment_length_per_warp`), `find_long_segments`, `grad_mean_kernel`,
 *    the cta-per-row and warp-per-row kernels (per-run reduction and the
 *    dense-gradient store).
 *  - "tt_embeddings_cuda.cu" (FBTT-Embedding): the three output modes
 *    (SGD, Adagrad, dense) and the formulas of the dense, SGD and row-wise
 *    Adagrad cache-backward kernels; D % 4 == 0 checks.
 *  - "Function _embedding_bwd_kernel" (tinygrad): the nobag backward, fp32
 *    accumulation of a 16-bit gradient into a dense grad_weight.
 *
 * Conventions for every entry point:
 *  - All functions are plain C; no C++ or torch types cross the boundary.
 *  - "device pointer" means memory on the GPU the plan was created on;
 *    "host pointer" means ordinary CPU memory.  The caller owns every buffer
 *    it passes (including the workspace) and keeps it alive until the work
 *    enqueued on `stream` has finished.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Work is enqueued asynchronously; functions return as soon as it is
 *    enqueued.  Only sgb_device_status() synchronises.
 *  - Argument errors are detected on the host before anything is enqueued;
 *    nothing is written in that case.  Errors in the *contents* of device
 *    arrays (an index outside its table, offsets that decrease or do not
 *    start at 0 / end at N) are detected by the kernels, recorded in a
 *    sticky status word in the workspace and reported by sgb_device_status();
 *    the kernels never read or write outside the buffers, but the outputs are
 *    then unspecified.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *  - A plan is immutable after creation and may be used from several host
 *    threads; concurrent calls need distinct workspaces.
 */
#ifndef SGB_H
#define SGB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sgb_plan_s* sgb_plan;

typedef enum {
  SGB_OK = 0,
  SGB_ERR_INVALID_ARGUMENT = 1,   /* bad argument, detected on the host        */
  SGB_ERR_UNSUPPORTED = 2,        /* valid request this library does not do    */
  SGB_ERR_WORKSPACE_TOO_SMALL = 3,
  SGB_ERR_INDEX_OUT_OF_RANGE = 4, /* device-detected: index outside [0, E_t)   */
  SGB_ERR_BAD_OFFSETS = 5,        /* device-detected: offsets malformed        */
  SGB_ERR_HIP = 6,                /* a HIP runtime call failed                 */
  SGB_ERR_INTERNAL = 7            /* device-detected: a bounded wait expired,
                                     or sgb_apply() on a workspace prepared for
                                     other lookups (its N or B differ)        */
} sgb_status;

/* Pooling of the forward pass, FBGEMM page host entry `pooling_mode` and the
 * nobag variant.  SGB_POOL_NONE is the nobag (per-token) case. */
typedef enum { SGB_POOL_SUM = 0, SGB_POOL_MEAN = 1, SGB_POOL_NONE = 2 } sgb_pooling;

/* Element type of grad_output (F32, BF16) and of weight rows (F32, BF16,
 * F16: IEEE binary16, INT8: row-wise quantized rows; the last two weights
 * only). */
typedef enum { SGB_F32 = 0, SGB_BF16 = 1, SGB_INT8 = 2, SGB_F16 = 3 } sgb_dtype;

/* Output mode, FBTT page OPTIM_{SGD, ADAGRAD, DENSE} (Adagrad is row-wise). */
typedef enum { SGB_DENSE_GRAD = 0, SGB_SGD = 1, SGB_ROWWISE_ADAGRAD = 2 } sgb_mode;

/*
 * sgb_plan_create -- immutable table metadata for a set of T tables.
 *  out                  receives the plan (host pointer to a handle).
 *  T                    number of tables, 1 <= T <= 65536.
 *  hash_size_cumsum     host, int64[T+1]: [0] = 0, strictly increasing;
 *                       table t owns linear ids [hsc[t], hsc[t+1]), so
 *                       E_t = hsc[t+1] - hsc[t] rows (FBGEMM host entry).
 *                       hsc[T] <= 2^40 (SGB_ERR_UNSUPPORTED above).
 *  D_offsets            host, int32[T+1]: [0] = 0, D_t = D_offsets[t+1] -
 *                       D_offsets[t] with D_t % 4 == 0 and 4 <= D_t <= 8192;
 *                       D_offsets[t] is table t's first column in a bag row
 *                       of grad_output.  Nobag plans need one common D_t.
 *  pooling              an sgb_pooling value.
 *  max_segment_length_per_warp
 *                       >= 1.  Runs with at least this many lookups are
 *                       "long" (FBGEMM `find_long_segments`, test `>=`) and
 *                       are split across many wavefronts.
 * The host arrays are copied; the plan allocates a few small device arrays on
 * the device current at creation.  Returns SGB_ERR_INVALID_ARGUMENT on any
 * violated rule, SGB_ERR_HIP if a device allocation fails.
 */
sgb_status sgb_plan_create(sgb_plan* out, int32_t T, const int64_t* hash_size_cumsum,
                           const int32_t* D_offsets, int32_t pooling,
                           int32_t max_segment_length_per_warp);

/* Frees the plan and its device arrays.  NULL is ignored. */
void sgb_plan_destroy(sgb_plan plan);

/*
 * sgb_workspace_bytes -- size of the device workspace needed by one
 * sgb_backward() call with `num_indices` lookups and `B` bags per table
 * (B is ignored for a nobag call without offsets; pass 0).  Also the size
 * needed by sgb_device_status()/sgb_runs_view_get() on that workspace.
 * Grows with num_indices and with 1 / max_segment_length_per_warp.
 * Limits: 0 <= num_indices < 2^30, B * T < 2^31.
 */
sgb_status sgb_workspace_bytes(sgb_plan plan, int64_t num_indices, int32_t B, size_t* bytes);

/* One batch of inputs; every pointer is a device pointer, read only. */
typedef struct {
  const void* grad_output;          /* bag: [B][D_offsets[T]] row-major;
                                       nobag: [num_indices][D] row-major    */
  int32_t grad_dtype;               /* an sgb_dtype value                   */
  const int64_t* indices;           /* [num_indices], row within its table  */
  int64_t num_indices;              /* N                                    */
  const int64_t* offsets;           /* [B*T+1] table-major (bag t*B+b spans
                                       [offsets[t*B+b], offsets[t*B+b+1]));
                                       may be NULL only for nobag with T == 1 */
  int32_t B;                        /* bags per table (0 if offsets NULL)   */
  const float* per_sample_weights;  /* [num_indices] or NULL; must be NULL
                                       for nobag (FBGEMM: nobag is generated
                                       only unweighted)                     */
} sgb_batch;

/* Where and how the result is written; device pointers, caller-owned. */
typedef struct {
  int32_t mode;      /* an sgb_mode value                                        */
  void* weights;     /* SGD / Adagrad: flat rows of weights_dtype elements, table
                        t row i at element woff[t] + i * D_t with
                        woff[t] = sum_{t'<t} E_t' * D_t'; INT8: table t row i
                        at byte woff8[t] + i * (D_t + 8) with woff8[t] =
                        sum_{t'<t} E_t' * (D_t' + 8), the row's D_t uint8
                        codes followed by its fp32 scale and fp32 bias       */
  float* momentum;   /* Adagrad: fp32[sum_t E_t], one value per row, indexed by
                        linear id hsc[t] + i                                      */
  float* grad;       /* DENSE: fp32, same layout as weights                       */
  int32_t accumulate;/* DENSE: 0 = the whole buffer is overwritten (zeros except
                        touched rows, which get their gradient); 1 = touched rows
                        get grad[row] += G_row, all others untouched             */
  float lr;          /* SGD / Adagrad learning rate                               */
  float eps;         /* Adagrad epsilon (added outside the square root)          */
  /* 16-bit weights (FBGEMM page, split-kernel weight store: a 16-bit row is
     stored with stochastic rounding from a Philox state seeded per call).
     A zero-initialised tail keeps fp32 weights.                               */
  int32_t weights_dtype;       /* SGB_F32, SGB_BF16, SGB_F16 or SGB_INT8 (the
                                  last three SGD / Adagrad only: with DENSE
                                  they are SGB_ERR_UNSUPPORTED).  INT8 rows
                                  (FBGEMM page: 8-bit rows carry their
                                  quantization parameters, recomputed from
                                  the updated row): code c stands for
                                  fmaf(c, scale, bias); after the fp32-row
                                  update, bias = row min, scale = (max - min)
                                  / 255, code = rint((w - bias) / scale)
                                  clamped to [0, 255] (0 if scale is 0), fp32
                                  arithmetic with correctly rounded division */
  int32_t stochastic_rounding; /* 16-bit rows: 1 = stochastic, 0 = nearest
                                  even.  The updated value is formed in fp32
                                  as for fp32 rows; element (linear id r,
                                  column d) draws word w = word d % 4 of
                                  Philox4x32-10(counter = (d / 4, r mod 2^32,
                                  r / 2^32, sr_offset mod 2^32), key = (sr_seed
                                  mod 2^32, sr_seed / 2^32)).  bf16: adds the
                                  high 16 bits of w to the fp32 bit pattern
                                  and keeps the high half.  fp16: with f the
                                  fraction of the binary16 spacing (2^-24
                                  below 2^-14) by which the magnitude exceeds
                                  the grid point below it, rounds the
                                  magnitude up iff w < f * 2^32; beyond 65504
                                  the result is infinity.  Nearest even is
                                  IEEE rounding to either format.              */
  uint64_t sr_seed;            /* Philox key                                   */
  uint64_t sr_offset;          /* its low 32 bits: counter word 3 (e.g. the
                                  step), so steps draw different bits         */
} sgb_update;

/*
 * sgb_backward -- enqueue one backward pass on `stream`.
 *  For every distinct linear row r touched by the batch, with
 *    G_r[d] = sum over lookups i of row r of coef_i * grad_output[b_i][D_offsets[t] + d]
 *    (nobag: grad_output[i][d]); coef_i = per_sample_weight_i (or 1) times
 *    1/L_b under MEAN pooling (FBGEMM `grad_mean_kernel`):
 *   DENSE       grad[r] = G_r (accumulate=0, other rows zeroed) or
 *               grad[r] += G_r (accumulate=1)          (FBGEMM dense store;
 *                                                       tinygrad grad_weight add)
 *   SGD         w_r -= lr * G_r                          (FBTT SGD kernel)
 *   ROWWISE_ADAGRAD  m_r += mean_d G_r[d]^2; w_r -= lr * G_r / (sqrt(m_r) + eps)
 *                                         (FBTT row-wise Adagrad kernel, once
 *                                          per distinct row on the summed G)
 *  Each touched row is read and written once; untouched rows and state are
 *  not written (a fresh dense gradient is zeroed whole first, then its
 *  touched rows are written).  A row's sum is accumulated in fp64 in a fixed
 *  order and rounded once to fp32; each term is a product coef * grad
 *  element, except in the short-run reducer, which first adds the fp32
 *  products of two consecutive lookups in fp32 (so a row's result is not the
 *  fp64 sum rounded once, but stays within 1e-4 + 1e-5 |G| of the exact sum
 *  on the tested workloads).  num_indices == 0 is a no-op (a fresh dense
 *  grad is still zero-filled).  Allocates nothing.
 *  Part of the work runs on two side streams the plan owns (the zero fill of
 *  a fresh dense gradient, and the short-run reduction); they start after
 *  everything enqueued on `stream` before the call, and `stream` waits for
 *  them before any work enqueued after the call, so the call behaves as if
 *  it ran on `stream` alone.  Calls with one plan share its side streams.
 *  Batches of at most 16384 lookups run on `stream` alone.
 */
sgb_status sgb_backward(sgb_plan plan, const sgb_batch* batch, const sgb_update* update,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * sgb_prepare / sgb_apply -- sgb_backward() in two parts, so that the part
 * that reads only the lookups can run ahead (FBGEMM host entry: the sort and
 * run-length steps depend on indices and offsets alone, the reduction on
 * grad_output and the rows).
 *  sgb_prepare enqueues on `stream` the linearisation, radix sort, run-length
 *  encoding and long-run list of `batch` into `workspace` (it reads
 *  indices, offsets, per_sample_weights and num_indices/B; grad_output may
 *  be NULL).  sgb_apply enqueues the rest -- the zero fill of a fresh dense
 *  gradient, the reductions and the row updates -- reading the run
 *  structure from `workspace`.
 *  Contract: an sgb_apply() call must see, in stream order, a completed
 *  sgb_prepare() of the same plan with the same lookups (indices, offsets,
 *  per_sample_weights, num_indices, B) into the same workspace, and no later
 *  sgb_prepare() or sgb_backward() into that workspace may start before the
 *  sgb_apply() has finished; the host cannot check this (the run structure
 *  lives on the device).  Results, errors and determinism are those of
 *  sgb_backward(): sgb_prepare() followed by sgb_apply() on one stream is the
 *  same computation.  With two workspaces a caller can prepare batch i+1 on
 *  one stream while batch i is applied on another; applies that update the
 *  same rows must still be ordered.  sgb_apply() uses the plan's side streams
 *  as sgb_backward() does (one apply of a plan at a time).  Arguments and
 *  host-detected errors as for sgb_backward(); sgb_prepare() checks no
 *  update, sgb_apply() repeats the batch checks.
 */
sgb_status sgb_prepare(sgb_plan plan, const sgb_batch* batch, void* workspace,
                       size_t workspace_bytes, void* stream);
sgb_status sgb_apply(sgb_plan plan, const sgb_batch* batch, const sgb_update* update,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * sgb_backward_noalloc -- sgb_backward() for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is a fixed scratch array
 * the library holds on every GPU it runs on (one copy per GPU, kept until the
 * process ends), so the caller passes only inputs and outputs.
 *  Limit: batches whose sgb_workspace_bytes() exceeds 64 MiB (about a
 *  million lookups of rows up to 256 wide) return SGB_ERR_WORKSPACE_TOO_SMALL
 *  before anything is enqueued.
 *  Same kernels, results and errors as sgb_backward(); it calls no hipMalloc,
 *  hipFree or other allocating routine.  Every call on one GPU uses that
 *  GPU's single scratch copy, which keeps the last call's contents: calls that
 *  overlap on one GPU (other streams, other host threads, other plans) race
 *  and must be serialised by the caller.  sgb_device_status() and
 *  sgb_runs_view_get() read this scratch when given a NULL workspace.
 *  SGB_ERR_HIP if the scratch's address could not be found at plan creation.
 */
sgb_status sgb_backward_noalloc(sgb_plan plan, const sgb_batch* batch, const sgb_update* update,
                                void* stream);

/* Timed regions of sgb_backward() (see sgb_backward_timed): one per kernel,
 * in launch order, plus SGB_STAGE_SORT spanning every radix pass. */
typedef enum {
  SGB_STAGE_LINEARIZE = 0,     /* bags -> packed (linear id, info) words, and the
                                  first radix pass's digit histogram             */
  SGB_STAGE_SORT_PASS = 1,     /* the first radix pass alone                     */
  SGB_STAGE_SORT = 2,          /* all radix passes                               */
  SGB_STAGE_RLE = 3,           /* run heads, first run index of every tile,
                                  unique ids, run starts                          */
  SGB_STAGE_RUNS = 4,          /* run lengths, long-run list, chunk prefix        */
  SGB_STAGE_FILL = 5,          /* zeros of the whole gradient (fresh dense only)  */
  SGB_STAGE_REDUCE_LONG = 6,   /* long runs: chunked reduction + fused row write  */
  SGB_STAGE_REDUCE_SHORT = 7,  /* short runs: reduction + fused row write         */
  SGB_NUM_STAGES = 8
} sgb_stage;

/*
 * sgb_backward_timed -- sgb_backward() that also records HIP events on
 * `stream` around each timed region: events[2k] just before region k's first
 * kernel and events[2k+1] just after its last (hipEvent_t passed as void*).  NULL
 * entries, and stages that do not run in this call, are skipped.  `events`
 * has 2 * SGB_NUM_STAGES entries or is NULL.  For measurement only: the
 * kernels and results are those of sgb_backward(), but with events given all
 * of them run one after another on `stream` (no side streams), so that each
 * timed region holds its kernel alone.
 */
sgb_status sgb_backward_timed(sgb_plan plan, const sgb_batch* batch, const sgb_update* update,
                              void* workspace, size_t workspace_bytes, void* stream,
                              void* const* events);

/*
 * sgb_device_status -- synchronises `stream`, then stores in *out the first
 * error the kernels recorded in `workspace` during the last sgb_backward()
 * that used it (SGB_OK if none).  The return value reports failures of this
 * call itself (SGB_ERR_HIP).  workspace NULL: the scratch of
 * sgb_backward_noalloc() on the plan's GPU.
 */
sgb_status sgb_device_status(sgb_plan plan, const void* workspace, void* stream, int32_t* out);

/*
 * Introspection of the run structure the last sgb_backward() left in
 * `workspace` (device pointers into it; valid until the workspace is reused).
 * Same kernels, no second code path.  Sorted entries are packed 64-bit words
 * (linear_id << info_bits) | info, info = t*B + b (bag) or i*T + t (nobag),
 * in stable sorted order (FBGEMM `transpose_embedding_input` outputs, with the
 * id and info carried in one word).  Counts live on the device.
 * sgb_runs_view_get needs the num_indices and B of that last call (they fix
 * the workspace layout); the call recorded them in the workspace, and a
 * mismatch returns SGB_ERR_INVALID_ARGUMENT.  It reads them back with a
 * synchronous copy (it waits for the device).  workspace NULL: the scratch of
 * sgb_backward_noalloc() on the plan's GPU.
 */
typedef struct {
  const uint64_t* sorted_packed;    /* [N]                                     */
  int32_t info_bits;
  const int64_t* unique_ids;        /* [num_runs]   sorted distinct linear ids */
  const int32_t* run_lengths;       /* [num_runs]                              */
  const int32_t* cumulative;        /* [num_runs+1] start of each run, [U] = N */
  const int32_t* num_runs;          /* [1]                                     */
  const int32_t* long_run_ids;      /* [num_long]   ascending                  */
  const int64_t* num_long_run_ids;  /* [1]                                     */
} sgb_runs_view;

sgb_status sgb_runs_view_get(sgb_plan plan, const void* workspace, int64_t num_indices,
                             int32_t B, sgb_runs_view* out);

/* Lookups of a forward call; every pointer is a device pointer, read only.
 * The fields mean what they mean in sgb_batch. */
typedef struct {
  const int64_t* indices;           /* [num_indices], row within its table  */
  int64_t num_indices;              /* N                                    */
  const int64_t* offsets;           /* [B*T+1] table-major, or NULL only for
                                       nobag with T == 1                    */
  int32_t B;                        /* bags per table (0 if offsets NULL)   */
  const float* per_sample_weights;  /* [num_indices] or NULL (bag only)     */
} sgb_lookups;

/*
 * sgb_forward -- enqueue the pooled forward on `stream`: the operation that
 * sgb_backward() differentiates.  With coef_i = per_sample_weight_i (or 1)
 * times 1/L under MEAN pooling (FBGEMM `grad_mean_kernel`), for bag (t, b)
 * and d < D_t:
 *     output[b][D_offsets[t] + d] = sum over lookups i of the bag of
 *                                   coef_i * W_t[indices[i]][d]
 * (an empty bag gives zeros), and for nobag output[i][d] = W_t[indices[i]][d]
 * (FBTT `cache_forward_kernel` sums the weight rows of a segment's lookups
 * into its output row).
 *  weights  device fp32, the layout of sgb_update.weights (table t row i at
 *           woff[t] + i * D_t), 16-byte aligned; read only.
 *  output   device fp32, caller-owned, 16-byte aligned: [B][D_offsets[T]]
 *           (bag) or [num_indices][D] (nobag); every element is written.
 *  Sums are accumulated in fp64 and rounded once.  Allocates nothing.
 *  workspace: device, 256-byte aligned, at least 128 bytes (any size that
 *  sgb_workspace_bytes() returns); only its status header is used, so
 *  sgb_device_status() reports this call's device-detected errors
 *  (SGB_ERR_INDEX_OUT_OF_RANGE, SGB_ERR_BAD_OFFSETS; output unspecified
 *  then).  Host-detected errors (SGB_ERR_INVALID_ARGUMENT for NULL or
 *  misaligned buffers and inconsistent sizes, SGB_ERR_UNSUPPORTED for
 *  weighted nobag) return before anything is enqueued.
 */
sgb_status sgb_forward(sgb_plan plan, const sgb_lookups* lookups, const float* weights,
                       float* output, void* workspace, size_t workspace_bytes, void* stream);

/* Static string naming a status code. */
const char* sgb_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* SGB_H */
