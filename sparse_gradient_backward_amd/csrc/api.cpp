// api.cpp -- the C ABI declared in include/sgb.h: plan creation, host-side
// validation, workspace layout and the launch sequence of one backward pass.
//
// Host checks follow the FBGEMM page "embedding_backward_split_template.cu",
// host entry `split_embedding{_nobag}_backward_codegen_..._exact_cuda`
// (T > 0, B > 0, offsets of length B*T+1, early return when there are no
// indices, the embedding-dimension bound), and the FBTT page
// "tt_embeddings_cuda.cu" (D % 4 == 0).  Nothing here touches the data:
// every step of the computation runs in the kernels of kernels.hip.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/sgb.h"
#include "internal.h"

using namespace sgb;

struct sgb_plan_s {
  int device = 0;
  int32_t T = 0;
  int32_t pooling = 0;
  int32_t thr = 1;
  int32_t Dmax = 0;
  int32_t Dmin = 0;
  // bound on (chunk, column block) items per lookup of a long run:
  // max over tables of col_blocks(D) / chunk_min(D), as a fraction
  int64_t items_num = 0, items_den = 1;
  int64_t total_rows = 0;   // sum of E_t
  int64_t total_elems = 0;  // sum of E_t * D_t
  int key_bits = 0;
  std::vector<int64_t> hsc, woff, woff8;
  std::vector<int32_t> doff;
  int64_t* d_hsc = nullptr;
  int32_t* d_doff = nullptr;
  int64_t* d_woff = nullptr;
  int64_t* d_woff8 = nullptr;  // byte offsets of INT8 weight tables
  FillBlock* d_fill = nullptr;
  int32_t n_fill = 0;
  int num_cus = 1;
  int red_grid[2] = {1, 1};  // persistent grid of the long-run reducer (f32, bf16)
  int wide_grid[4] = {1, 1, 1, 1};  // resident workgroups of the wide-row reducer (see launch_reduce_short)
  // side streams (default priority): [0] clears a fresh dense gradient while
  // the ids are sorted, [1] reduces the short runs while the long-run list is
  // built and the long runs are reduced; the events fork and join them.  The
  // mutex keeps one call's fork/join sequence from interleaving with another's.
  hipStream_t aux[2] = {nullptr, nullptr};
  // fork, fill done, sorted (or rle done), short done (the join), rle done
  hipEvent_t ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  std::mutex mu;
  // this device's copy of the fixed scratch of sgb_backward_noalloc (NULL if
  // its lookup failed)
  void* scratch = nullptr;
};

namespace {

int bitlen(uint64_t v) {  // number of bits needed to hold v (0 for 0)
  int b = 0;
  while (v) {
    ++b;
    v >>= 1;
  }
  return b;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// A fresh 24-bit tag per call (never 0): device-detected errors carry the tag
// of the call that found them, so the status word needs no clearing.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  for (;;) {
    const uint32_t e = (counter.fetch_add(1, std::memory_order_relaxed) + 1u) & 0xFFFFFFu;
    if (e) return e;
  }
}

struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = (prev == dev) || (hipSetDevice(dev) == hipSuccess);
  }
  ~DeviceGuard() {
    if (ok && prev >= 0) (void)hipSetDevice(prev);
  }
};

// Workspace layout of one call; every piece 256-byte aligned.
struct Layout {
  int info_bits = 0;
  int npasses = 0;
  int pass_bits[kMaxPasses] = {};
  int pass_key_shift[kMaxPasses] = {};
  int pass_shape[kMaxPasses] = {};
  int64_t pass_tiles[kMaxPasses] = {};
  int64_t scan_tiles = 0;
  int64_t max_long = 0;   // bound on the number of long runs
  int64_t max_items = 0;  // bound on the (chunk, column block) items over all long runs
  size_t hdr = 0, hist0 = 0, zero_begin = 0, hist[kMaxPasses] = {}, sort_lb[kMaxPasses] = {},
         rle_lb = 0, post_lb = 0, zero_end = 0;
  size_t kvA = 0, kvB = 0, coefA = 0, coefB = 0, uniq = 0, cum = 0, headrun = 0, lens = 0, longs = 0,
         chunkb = 0, longrec = 0, runtk = 0, sctk = 0, tile_runs = 0, part = 0, total = 0;
};

sgb_status make_layout(const sgb_plan_s* p, int64_t N, int32_t B, bool has_offsets, Layout* L) {
  if (N < 0 || N >= (1ll << 30)) return SGB_ERR_INVALID_ARGUMENT;
  const bool nobag = p->pooling == SGB_POOL_NONE;
  uint64_t info_max = 0;
  if (nobag) {
    info_max = N > 0 ? (uint64_t)(N - 1) * (uint64_t)p->T + (uint64_t)(p->T - 1) : 0;
  } else {
    if (B <= 0) return SGB_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * p->T >= (1ll << 31)) return SGB_ERR_INVALID_ARGUMENT;
    info_max = (uint64_t)B * (uint64_t)p->T - 1;
  }
  if (has_offsets && (int64_t)B * p->T >= (1ll << 31)) return SGB_ERR_INVALID_ARGUMENT;
  if (info_max >= (1ull << 32)) return SGB_ERR_UNSUPPORTED;
  L->info_bits = bitlen(info_max);
  if (L->info_bits + p->key_bits > 64) return SGB_ERR_UNSUPPORTED;
  L->npasses = (p->key_bits + kMaxDigitBits - 1) / kMaxDigitBits;
  if (L->npasses > kMaxPasses) return SGB_ERR_UNSUPPORTED;  // linear ids >= 2^40
  int at = 0;
  for (int i = 0; i < L->npasses; ++i) {
    // the wider digits first: every later pass's digits fit the tables of
    // the pass before it
    L->pass_bits[i] = p->key_bits / L->npasses + (i < p->key_bits % L->npasses ? 1 : 0);
    L->pass_key_shift[i] = at;
    at += L->pass_bits[i];
    L->pass_shape[i] = sort_shape_for(N, L->pass_bits[i], p->num_cus);
    const int64_t tile = sort_tile_items(L->pass_shape[i]);
    L->pass_tiles[i] = (N + tile - 1) / tile;
  }
  L->scan_tiles = (N + kScanTile - 1) / kScanTile;
  L->max_long = N / p->thr + 1;
  // a long run of len lookups in a table of width D has ceil(len / chunk_len)
  // <= len / chunk_min(D, base) + 1 chunks of col_blocks(D) items each, for
  // any chunk base >= kChunkBaseMin
  L->max_items = (N * p->items_num + p->items_den - 1) / p->items_den +
                 (L->max_long + 1) * col_blocks(p->Dmax);

  size_t o = 0;
  auto take = [&](size_t bytes) {
    o = align_up(o, 256);
    const size_t at_ = o;
    o += bytes;
    return at_;
  };
  L->hdr = take(sizeof(Header));
  // the first pass's digit histogram (cleared by k_linearize's first workgroup)
  L->hist0 = take(sizeof(uint32_t) * kHistSlices * kRadixMax);
  // cleared by k_linearize for the kernels after it: the later passes'
  // histograms, the look-back words of each radix pass, of the run-length
  // encoding and of the run post-processing, the long-run combine tickets
  L->zero_begin = align_up(o, 256);
  L->hist[0] = L->hist0;
  for (int i = 1; i < L->npasses; ++i) L->hist[i] = take(sizeof(uint32_t) * kHistSlices << L->pass_bits[i]);
  const size_t scan_words =
      (size_t)(L->scan_tiles + (L->scan_tiles + kLbScalarGroupTiles - 1) / kLbScalarGroupTiles);
  L->rle_lb = take(sizeof(uint32_t) * scan_words);
  L->post_lb = take(sizeof(uint64_t) * scan_words);
  L->runtk = take(sizeof(uint32_t) * (size_t)L->max_items);
  L->sctk = take(sizeof(uint32_t) * (size_t)L->max_items);
  // the radix passes' look-back words, packed by this batch's tile shapes
  // (only they are cleared), in room for the most tiles any shape gives, so
  // that a workspace sized for N fits every smaller batch
  const size_t lb0 = align_up(o, 256);
  size_t used = 0, room = 0;
  auto lb_words = [](int64_t tiles) {  // tile words and group words
    return (size_t)(tiles + (tiles + kSortLbGroup - 1) / kSortLbGroup);
  };
  for (int i = 0; i < L->npasses; ++i) {
    L->sort_lb[i] = lb0 + used;
    used += align_up(sizeof(uint32_t) * lb_words(L->pass_tiles[i]) << L->pass_bits[i], 256);
    room += align_up(sizeof(uint32_t) * lb_words((N + kSortTileMin - 1) / kSortTileMin)
                         << L->pass_bits[i], 256);
  }
  L->zero_end = lb0 + used;
  o = lb0 + room;
  L->kvA = take(sizeof(uint64_t) * (size_t)N);
  L->kvB = take(sizeof(uint64_t) * (size_t)N);
  L->coefA = take(sizeof(float) * (size_t)N);
  L->coefB = take(sizeof(float) * (size_t)N);
  L->uniq = take(sizeof(int64_t) * (size_t)N);
  L->cum = take(sizeof(int32_t) * (size_t)(N + 1));
  L->headrun = take(sizeof(int32_t) * (size_t)N);
  L->tile_runs = take(sizeof(uint32_t) * (size_t)L->scan_tiles);
  L->lens = take(sizeof(int32_t) * (size_t)N);
  L->longs = take(sizeof(int32_t) * (size_t)L->max_long);
  L->longrec = take(sizeof(LongRun) * (size_t)L->max_long);
  L->chunkb = take(sizeof(uint32_t) * (size_t)(L->max_long + 1));
  L->part = take(sizeof(double) * (size_t)L->max_items * (size_t)kColBlock);
  L->total = align_up(o, 256);
  return SGB_OK;
}

// Workgroups of the zero fill: one per SGB_FILL_CUS_PER_WG compute units.
// The fill overlaps latency-bound kernels on other streams; a small grid
// still saturates HBM with stores and leaves them the CU slots.
int fill_grid(const sgb_plan_s* p) {
  const int g = std::max(1, p->num_cus / std::max(1, (int)SGB_FILL_CUS_PER_WG));
  return std::max(1, std::min(p->n_fill, g));
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// which part of the path an enqueue call runs (see enqueue)
enum Part { kPartAll, kPartFront, kPartReduce };
sgb_status enqueue(sgb_plan p, const sgb_batch* b, const sgb_update* u, void* ws,
                   size_t ws_bytes, void* stream_, void* const* events, Part part);

}  // namespace

extern "C" {

const char* sgb_status_string(int32_t s) {
  switch (s) {
    case SGB_OK: return "SGB_OK";
    case SGB_ERR_INVALID_ARGUMENT: return "SGB_ERR_INVALID_ARGUMENT";
    case SGB_ERR_UNSUPPORTED: return "SGB_ERR_UNSUPPORTED";
    case SGB_ERR_WORKSPACE_TOO_SMALL: return "SGB_ERR_WORKSPACE_TOO_SMALL";
    case SGB_ERR_INDEX_OUT_OF_RANGE: return "SGB_ERR_INDEX_OUT_OF_RANGE";
    case SGB_ERR_BAD_OFFSETS: return "SGB_ERR_BAD_OFFSETS";
    case SGB_ERR_HIP: return "SGB_ERR_HIP";
    case SGB_ERR_INTERNAL: return "SGB_ERR_INTERNAL";
    default: return "SGB_UNKNOWN_STATUS";
  }
}

sgb_status sgb_plan_create(sgb_plan* out, int32_t T, const int64_t* hsc, const int32_t* doff,
                           int32_t pooling, int32_t thr) {
  if (!out) return SGB_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (T < 1 || T > 65536 || !hsc || !doff || thr < 1) return SGB_ERR_INVALID_ARGUMENT;
  if (pooling != SGB_POOL_SUM && pooling != SGB_POOL_MEAN && pooling != SGB_POOL_NONE)
    return SGB_ERR_INVALID_ARGUMENT;
  if (hsc[0] != 0 || doff[0] != 0) return SGB_ERR_INVALID_ARGUMENT;
  for (int32_t t = 0; t < T; ++t) {
    if (hsc[t + 1] <= hsc[t]) return SGB_ERR_INVALID_ARGUMENT;
    const int32_t D = doff[t + 1] - doff[t];
    if (D < 4 || D > kMaxD || D % 4 != 0) return SGB_ERR_INVALID_ARGUMENT;
    if (pooling == SGB_POOL_NONE && D != doff[1] - doff[0]) return SGB_ERR_INVALID_ARGUMENT;
  }
  if (hsc[T] > (1ll << 40)) return SGB_ERR_UNSUPPORTED;  // linear ids must fit 4 radix passes

  sgb_plan_s* p = new (std::nothrow) sgb_plan_s();
  if (!p) return SGB_ERR_HIP;
  if (hipGetDevice(&p->device) != hipSuccess) {
    delete p;
    return SGB_ERR_HIP;
  }
  p->T = T;
  p->pooling = pooling;
  p->thr = thr;
  p->hsc.assign(hsc, hsc + T + 1);
  p->doff.assign(doff, doff + T + 1);
  p->woff.assign(T + 1, 0);
  p->woff8.assign(T + 1, 0);
  std::vector<FillBlock> fill;
  for (int32_t t = 0; t < T; ++t) {
    const int64_t E = hsc[t + 1] - hsc[t];
    const int32_t D = doff[t + 1] - doff[t];
    p->Dmax = std::max(p->Dmax, D);
    p->Dmin = t == 0 ? D : std::min(p->Dmin, D);
    const int64_t num = col_blocks(D), den = chunk_min(D, kChunkBaseMin);
    if (num * p->items_den > p->items_num * den) {
      p->items_num = num;
      p->items_den = den;
    }
    p->woff[t + 1] = p->woff[t] + E * D;
    p->woff8[t + 1] = p->woff8[t] + E * (D + 8);
    const int64_t rows_per = std::max<int64_t>(1, 16384 / D);
    for (int64_t r0 = 0; r0 < E; r0 += rows_per)
      fill.push_back(FillBlock{t, (int32_t)std::min<int64_t>(rows_per, E - r0), r0});
  }
  p->total_rows = hsc[T];
  p->total_elems = p->woff[T];
  p->key_bits = bitlen((uint64_t)(p->total_rows - 1));
  p->n_fill = (int32_t)fill.size();

  int cus = 0;  // a scalar attribute: no versioned property struct crosses the runtime
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device) ==
          hipSuccess &&
      cus > 0)
    p->num_cus = cus;
  p->red_grid[0] = p->num_cus * reduce_long_blocks_per_cu(false);
  p->red_grid[1] = p->num_cus * reduce_long_blocks_per_cu(true);
  reduce_wide_blocks_per_cu(p->wide_grid);
  for (int i = 0; i < 4; ++i) p->wide_grid[i] *= p->num_cus;

  bool ok = hipStreamCreateWithFlags(&p->aux[0], hipStreamNonBlocking) == hipSuccess &&
            hipStreamCreateWithFlags(&p->aux[1], hipStreamNonBlocking) == hipSuccess;
  for (int i = 0; i < 5 && ok; ++i)
    // the fork events order work between the plan's streams on this device
    // only and need no system-scope release at their records; the join event
    // (ev[3]) keeps it, so that a host waiting on the caller's stream sees the
    // side stream's writes
    ok = hipEventCreateWithFlags(&p->ev[i], hipEventDisableTiming |
                                                (i != 3 ? hipEventDisableSystemFence : 0)) ==
         hipSuccess;
  ok = ok && hipMalloc(&p->d_hsc, sizeof(int64_t) * (T + 1)) == hipSuccess &&
            hipMalloc(&p->d_doff, sizeof(int32_t) * (T + 1)) == hipSuccess &&
            hipMalloc(&p->d_woff, sizeof(int64_t) * (T + 1)) == hipSuccess &&
            hipMalloc(&p->d_woff8, sizeof(int64_t) * (T + 1)) == hipSuccess &&
            hipMalloc(&p->d_fill, sizeof(FillBlock) * fill.size()) == hipSuccess;
  ok = ok && hipMemcpy(p->d_hsc, p->hsc.data(), sizeof(int64_t) * (T + 1),
                       hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemcpy(p->d_doff, p->doff.data(), sizeof(int32_t) * (T + 1),
                       hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemcpy(p->d_woff, p->woff.data(), sizeof(int64_t) * (T + 1),
                       hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemcpy(p->d_woff8, p->woff8.data(), sizeof(int64_t) * (T + 1),
                       hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemcpy(p->d_fill, fill.data(), sizeof(FillBlock) * fill.size(),
                       hipMemcpyHostToDevice) == hipSuccess;
  if (!ok) {
    sgb_plan_destroy(p);
    return SGB_ERR_HIP;
  }
  if (scratch_address(&p->scratch) != hipSuccess) p->scratch = nullptr;
  *out = p;
  return SGB_OK;
}

void sgb_plan_destroy(sgb_plan p) {
  if (!p) return;
  DeviceGuard g(p->device);
  if (p->d_hsc) (void)hipFree(p->d_hsc);
  if (p->d_doff) (void)hipFree(p->d_doff);
  if (p->d_woff) (void)hipFree(p->d_woff);
  if (p->d_woff8) (void)hipFree(p->d_woff8);
  if (p->d_fill) (void)hipFree(p->d_fill);
  for (hipEvent_t e : p->ev)
    if (e) (void)hipEventDestroy(e);
  for (hipStream_t s : p->aux)
    if (s) (void)hipStreamDestroy(s);
  delete p;
}

sgb_status sgb_workspace_bytes(sgb_plan p, int64_t N, int32_t B, size_t* bytes) {
  if (!p || !bytes) return SGB_ERR_INVALID_ARGUMENT;
  Layout L;
  const bool nobag_no_off = p->pooling == SGB_POOL_NONE && B == 0;
  if (nobag_no_off && p->T != 1) return SGB_ERR_INVALID_ARGUMENT;
  sgb_status st = make_layout(p, N, B, !nobag_no_off, &L);
  if (st != SGB_OK) return st;
  *bytes = L.total;
  return SGB_OK;
}

sgb_status sgb_backward(sgb_plan p, const sgb_batch* b, const sgb_update* u, void* ws,
                        size_t ws_bytes, void* stream_) {
  return enqueue(p, b, u, ws, ws_bytes, stream_, nullptr, kPartAll);
}

sgb_status sgb_prepare(sgb_plan p, const sgb_batch* b, void* ws, size_t ws_bytes, void* stream_) {
  return enqueue(p, b, nullptr, ws, ws_bytes, stream_, nullptr, kPartFront);
}

sgb_status sgb_apply(sgb_plan p, const sgb_batch* b, const sgb_update* u, void* ws,
                     size_t ws_bytes, void* stream_) {
  return enqueue(p, b, u, ws, ws_bytes, stream_, nullptr, kPartReduce);
}

sgb_status sgb_backward_noalloc(sgb_plan p, const sgb_batch* b, const sgb_update* u,
                                void* stream_) {
  if (!p || !b || !u) return SGB_ERR_INVALID_ARGUMENT;
  if (!p->scratch) return SGB_ERR_HIP;
  // the batch must fit the fixed scratch (the workspace sgb_backward would need)
  Layout L;
  const bool with_offsets = b->offsets != nullptr;
  if (b->num_indices > 0) {
    const sgb_status st = make_layout(p, b->num_indices, with_offsets ? b->B : 0, with_offsets, &L);
    if (st != SGB_OK) return st;
    if (L.total > kScratchBytes) return SGB_ERR_WORKSPACE_TOO_SMALL;
  }
  return enqueue(p, b, u, p->scratch, kScratchBytes, stream_, nullptr, kPartAll);
}

sgb_status sgb_backward_timed(sgb_plan p, const sgb_batch* b, const sgb_update* u, void* ws,
                              size_t ws_bytes, void* stream_, void* const* events) {
  return enqueue(p, b, u, ws, ws_bytes, stream_, events, kPartAll);
}

}  // extern "C"

namespace {

// The whole path (kPartAll), or the part of it that reads only the lookups
// (kPartFront: linearise, sort, run-length encoding, run post-processing),
// or the rest (kPartReduce: zero fill, reducers, row updates), which needs
// the run structure a kPartFront call with the same lookups left in `ws`.
sgb_status enqueue(sgb_plan p, const sgb_batch* b, const sgb_update* u, void* ws,
                   size_t ws_bytes, void* stream_, void* const* events, Part part) {
  const bool do_front = part != kPartReduce, do_reduce = part != kPartFront;
  if (!p || !b || (do_reduce && !u)) return SGB_ERR_INVALID_ARGUMENT;
  // the front never reads the update; a neutral one keeps the shared checks simple
  const sgb_update front_only{};
  if (!do_reduce) u = &front_only;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const int64_t N = b->num_indices;
  const bool nobag = p->pooling == SGB_POOL_NONE;
  if (N < 0 || N >= (1ll << 30)) return SGB_ERR_INVALID_ARGUMENT;
  if (b->grad_dtype != SGB_F32 && b->grad_dtype != SGB_BF16) return SGB_ERR_INVALID_ARGUMENT;
  if (nobag && b->per_sample_weights) return SGB_ERR_UNSUPPORTED;
  if (!b->offsets && !(nobag && p->T == 1)) return SGB_ERR_INVALID_ARGUMENT;
  if (b->offsets && b->B <= 0) return SGB_ERR_INVALID_ARGUMENT;
  if (do_reduce) {
    if (u->mode != SGB_DENSE_GRAD && u->mode != SGB_SGD && u->mode != SGB_ROWWISE_ADAGRAD)
      return SGB_ERR_INVALID_ARGUMENT;
    if (u->mode == SGB_DENSE_GRAD && !u->grad) return SGB_ERR_INVALID_ARGUMENT;
    if (u->mode == SGB_SGD && !u->weights) return SGB_ERR_INVALID_ARGUMENT;
    if (u->mode == SGB_ROWWISE_ADAGRAD && (!u->weights || !u->momentum))
      return SGB_ERR_INVALID_ARGUMENT;
    if (u->weights_dtype != SGB_F32 && u->weights_dtype != SGB_BF16 &&
        u->weights_dtype != SGB_INT8 && u->weights_dtype != SGB_F16)
      return SGB_ERR_INVALID_ARGUMENT;
    if (u->mode == SGB_DENSE_GRAD && u->weights_dtype != SGB_F32) return SGB_ERR_UNSUPPORTED;
  }
  const bool w_f16 = u->mode != SGB_DENSE_GRAD && u->weights_dtype == SGB_F16;
  const bool w_bf16 = u->mode != SGB_DENSE_GRAD && (u->weights_dtype == SGB_BF16 || w_f16);
  const bool w_int8 = u->mode != SGB_DENSE_GRAD && u->weights_dtype == SGB_INT8;
  void* outv = u->mode == SGB_DENSE_GRAD ? static_cast<void*>(u->grad) : u->weights;
  if (do_reduce && !aligned(outv, 16)) return SGB_ERR_INVALID_ARGUMENT;
  float* out = (w_bf16 || w_int8) ? nullptr : static_cast<float*>(outv);
  const bool fresh = do_reduce && u->mode == SGB_DENSE_GRAD && !u->accumulate;
  DeviceGuard guard(p->device);
  if (!guard.ok) return SGB_ERR_HIP;
  auto mark_on = [&](hipStream_t s, int stage, int end) {
    void* ev = events ? events[2 * stage + end] : nullptr;
    if (ev) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev), s);
  };
  auto mark = [&](int stage, int end) { mark_on(stream, stage, end); };

  if (N == 0) {  // FBGEMM host entry: no indices -> nothing to do (dense grad stays zero)
    // clear the status word so sgb_device_status() reports this call
    if (do_front && ws && aligned(ws, 256) && ws_bytes >= sizeof(Header) &&
        launch_init(ws, sizeof(Header), stream) != hipSuccess)
      return SGB_ERR_HIP;
    if (fresh && p->n_fill > 0) {
      FillParams f{out, p->d_fill, p->n_fill, p->d_doff, p->d_woff};
      if (launch_fill(f, fill_grid(p), stream) != hipSuccess) return SGB_ERR_HIP;
    }
    return SGB_OK;
  }
  if (!b->indices || (do_reduce && !b->grad_output)) return SGB_ERR_INVALID_ARGUMENT;
  if (do_reduce && !aligned(b->grad_output, b->grad_dtype == SGB_F32 ? 16 : 8))
    return SGB_ERR_INVALID_ARGUMENT;
  if (!ws || !aligned(ws, 256)) return SGB_ERR_INVALID_ARGUMENT;
  Layout L;
  sgb_status st = make_layout(p, N, b->offsets ? b->B : 0, b->offsets != nullptr, &L);
  if (st != SGB_OK) return st;
  if (ws_bytes < L.total) return SGB_ERR_WORKSPACE_TOO_SMALL;

  Header* hdr = at<Header>(ws, L.hdr);
  uint32_t* status = &hdr->status;
  const uint32_t epoch = next_epoch();
  const bool has_coef = (p->pooling == SGB_POOL_MEAN) || (b->per_sample_weights != nullptr);
  // (no separate clearing step: linearisation resets the header's counters)

  // the plan's side streams and fork/join events: one call's sequence at a time
  std::lock_guard<std::mutex> lock(p->mu);
  // the timed variant runs every kernel in order on `stream`, so that each
  // kernel's events bracket that kernel alone; so do small batches
  const bool overlap = events == nullptr && N > kSerialMaxN;
  hipStream_t fill_s = overlap ? p->aux[0] : stream, short_s = overlap ? p->aux[1] : stream;
  if (fresh) {
    // fork: the fresh gradient is cleared on a side stream, overlapping the
    // steps up to run-length encoding
    if (hipEventRecord(p->ev[0], stream) != hipSuccess ||
        hipStreamWaitEvent(fill_s, p->ev[0], 0) != hipSuccess)
      return SGB_ERR_HIP;
    FillParams f{out, p->d_fill, p->n_fill, p->d_doff, p->d_woff};
    mark_on(fill_s, SGB_STAGE_FILL, 0);
    if (launch_fill(f, fill_grid(p), fill_s) != hipSuccess) return SGB_ERR_HIP;
    mark_on(fill_s, SGB_STAGE_FILL, 1);
    if (hipEventRecord(p->ev[1], fill_s) != hipSuccess) return SGB_ERR_HIP;
  }

  // linearise (+ clear look-back words and combine tickets)
  LinParams lp{};
  lp.indices = b->indices;
  lp.offsets = b->offsets;
  lp.psw = b->per_sample_weights;
  lp.hsc = p->d_hsc;
  lp.N = N;
  lp.B = b->offsets ? b->B : 0;
  lp.T = p->T;
  lp.pooling = p->pooling;
  lp.info_bits = L.info_bits;
  lp.kv_out = at<uint64_t>(ws, L.kvA);
  lp.coef_out = has_coef ? at<float>(ws, L.coefA) : nullptr;
  lp.status = status;
  lp.epoch = epoch;
  lp.header = hdr;
  lp.zero_begin = at<uint4>(ws, L.zero_begin);
  lp.zero_vec4 = (int64_t)((L.zero_end - L.zero_begin) / 16);
  lp.hist = L.npasses > 0 ? at<uint32_t>(ws, L.hist0) : nullptr;
  lp.hist_bits = L.npasses > 0 ? L.pass_bits[0] : 0;
  lp.hist_ready = &hdr->hist_ready;
  const int64_t lin_tiles = b->offsets ? ((int64_t)b->B * p->T + kLinBags - 1) / kLinBags
                                       : (N + kLinLookups - 1) / kLinLookups;
  const int lin_grid =
      (int)std::max<int64_t>(1, std::min<int64_t>(lin_tiles, (int64_t)SGB_LIN_WG_PER_CU * p->num_cus));
  mark(SGB_STAGE_LINEARIZE, 0);
  if (do_front && launch_linearize(lp, lin_grid, stream) != hipSuccess) return SGB_ERR_HIP;
  mark(SGB_STAGE_LINEARIZE, 1);

  // LSD radix passes, ping-pong between A and B
  uint64_t* kv_in = at<uint64_t>(ws, L.kvA);
  uint64_t* kv_out = at<uint64_t>(ws, L.kvB);
  float* cf_in = has_coef ? at<float>(ws, L.coefA) : nullptr;
  float* cf_out = has_coef ? at<float>(ws, L.coefB) : nullptr;
  if (L.npasses > 0) mark(SGB_STAGE_SORT, 0);
  for (int ps = 0; ps < L.npasses; ++ps) {
    SortParams sp{};
    sp.kv_in = kv_in;
    sp.coef_in = cf_in;
    sp.kv_out = kv_out;
    sp.coef_out = cf_out;
    sp.N = N;
    sp.tiles = (int32_t)L.pass_tiles[ps];
    sp.shape = L.pass_shape[ps];
    sp.shift = L.info_bits + L.pass_key_shift[ps];
    sp.bits = L.pass_bits[ps];
    sp.hist = at<uint32_t>(ws, L.hist[ps]);
    const bool last = ps + 1 == L.npasses;
    sp.hist_next = last ? nullptr : at<uint32_t>(ws, L.hist[ps + 1]);
    sp.shift_next = last ? 0 : L.info_bits + L.pass_key_shift[ps + 1];
    sp.bits_next = last ? 0 : L.pass_bits[ps + 1];
    sp.lookback = at<uint32_t>(ws, L.sort_lb[ps]);
    sp.tile_ctr = &hdr->sort_tile_ctr[ps];
    sp.status = status;
    sp.epoch = epoch;
    if (ps == 0) mark(SGB_STAGE_SORT_PASS, 0);
    if (do_front && launch_sort_pass(sp, stream) != hipSuccess) return SGB_ERR_HIP;
    if (ps == 0) mark(SGB_STAGE_SORT_PASS, 1);
    std::swap(kv_in, kv_out);
    std::swap(cf_in, cf_out);
  }
  if (L.npasses > 0) mark(SGB_STAGE_SORT, 1);
  const uint64_t* kv_sorted = kv_in;
  const float* cf_sorted = cf_in;
  // early fork: with the ids sorted, the reducer of short runs of rows up to
  // 512 columns finds the run lengths itself (scan_runs) and starts on the
  // side stream here, overlapping run-length encoding and the long-run list
  const bool early = overlap && N <= kEarlyForkMaxN && do_front && do_reduce &&
                     p->thr <= kScanRunsMaxThr && p->Dmin <= 512;
  if (early && (hipEventRecord(p->ev[2], stream) != hipSuccess ||
                hipStreamWaitEvent(short_s, p->ev[2], 0) != hipSuccess))
    return SGB_ERR_HIP;

  RleParams rp{};
  rp.kv = kv_sorted;
  rp.N = N;
  rp.info_bits = L.info_bits;
  rp.unique_ids = at<int64_t>(ws, L.uniq);
  rp.cum = at<int32_t>(ws, L.cum);
  rp.head_run = at<int32_t>(ws, L.headrun);
  rp.num_runs = &hdr->num_runs;
  rp.tiles = L.scan_tiles;
  rp.lookback = at<uint32_t>(ws, L.rle_lb);
  rp.tile_ctr = &hdr->rle_tile_ctr;
  rp.tile_runs = at<uint32_t>(ws, L.tile_runs);
  rp.one_pass = L.scan_tiles <= kOnePassTiles ? 1 : 0;
  rp.fuse_scan = L.scan_tiles <= kFuseScanTiles ? 1 : 0;
  rp.status = status;
  rp.epoch = epoch;
  mark(SGB_STAGE_RLE, 0);
  if (do_front && launch_rle(rp, stream) != hipSuccess) return SGB_ERR_HIP;
  mark(SGB_STAGE_RLE, 1);
  if (early && p->Dmax > 512 && hipEventRecord(p->ev[4], stream) != hipSuccess)
    return SGB_ERR_HIP;

  PostParams pp{};
  pp.cum = rp.cum;
  pp.num_runs = rp.num_runs;
  pp.unique_ids = rp.unique_ids;
  pp.kv = kv_sorted;
  pp.doff = p->d_doff;
  pp.info_bits = L.info_bits;
  pp.B = b->offsets ? b->B : 0;
  pp.T = p->T;
  pp.nobag = nobag ? 1 : 0;
  pp.chunk_base = chunk_base_for(N);
  pp.hsc = p->d_hsc;
  pp.woff = p->d_woff;
  pp.thr = p->thr;
  pp.run_lengths = at<int32_t>(ws, L.lens);
  pp.long_ids = at<int32_t>(ws, L.longs);
  pp.chunk_begin = at<uint32_t>(ws, L.chunkb);
  pp.long_recs = at<LongRun>(ws, L.longrec);
  pp.num_long = &hdr->num_long;
  pp.total_items = &hdr->total_items;
  pp.tiles = L.scan_tiles;
  pp.lookback = at<uint64_t>(ws, L.post_lb);
  pp.tile_ctr = &hdr->post_tile_ctr;
  pp.status = status;
  pp.epoch = epoch;

  RedParams q{};
  q.grad = b->grad_output;
  q.kv = kv_sorted;
  q.coef = has_coef ? cf_sorted : nullptr;
  q.hsc = p->d_hsc;
  q.doff = p->d_doff;
  q.woff = p->d_woff;
  q.unique_ids = rp.unique_ids;
  q.cum = rp.cum;
  q.head_run = rp.head_run;
  q.long_ids = pp.long_ids;
  q.chunk_begin = pp.chunk_begin;
  q.long_recs = pp.long_recs;
  q.num_runs = rp.num_runs;
  q.total_items = pp.total_items;
  q.num_long = &hdr->num_long;
  q.header = hdr;
  q.sc_ticket = at<uint32_t>(ws, L.sctk);
  q.run_ticket = at<uint32_t>(ws, L.runtk);
  q.partials = at<double>(ws, L.part);
  q.out = out;
  q.out_h = w_bf16 ? static_cast<uint16_t*>(outv) : nullptr;
  q.out_q = w_int8 ? static_cast<uint8_t*>(outv) : nullptr;
  q.woff8 = p->d_woff8;
  q.w_kind = w_int8 ? 2 : (w_f16 ? 3 : (w_bf16 ? 1 : 0));
  q.sr = (w_bf16 && u->stochastic_rounding) ? 1 : 0;
  q.sr_key0 = (uint32_t)u->sr_seed;
  q.sr_key1 = (uint32_t)(u->sr_seed >> 32);
  q.sr_ctr3 = (uint32_t)u->sr_offset;
  q.mom = u->mode == SGB_ROWWISE_ADAGRAD ? u->momentum : nullptr;
  q.status = status;
  q.N = N;
  q.row_stride = nobag ? (int64_t)p->doff[1] : (int64_t)p->doff[p->T];
  q.info_bits = L.info_bits;
  q.B = b->offsets ? b->B : 0;
  q.T = p->T;
  q.nobag = nobag ? 1 : 0;
  q.thr = p->thr;
  q.chunk_base = pp.chunk_base;
  q.mode = u->mode;
  q.accumulate = u->accumulate ? 1 : 0;
  q.lr = u->lr;
  q.eps = u->eps;
  q.scan_runs = early ? 1 : 0;
  const bool bf16 = b->grad_dtype == SGB_BF16;
  // short runs need only the sorted words and run starts: side stream from
  // here on (after the zero fill), while the long-run list is built and the
  // long runs are reduced here; the two write disjoint rows
  if (do_reduce) {
    if (early) {
      // the side stream already waits for the sort; the wider rows' reducer
      // reads the run starts, so it waits for run-length encoding too
      if (fresh && hipStreamWaitEvent(short_s, p->ev[1], 0) != hipSuccess) return SGB_ERR_HIP;
      if (launch_reduce_short(q, bf16, p->Dmin, p->Dmax, p->wide_grid, kShortRows, short_s) !=
          hipSuccess)
        return SGB_ERR_HIP;
      if (p->Dmax > 512 &&
          (hipStreamWaitEvent(short_s, p->ev[4], 0) != hipSuccess ||
           launch_reduce_short(q, bf16, p->Dmin, p->Dmax, p->wide_grid, kWideRows, short_s) !=
               hipSuccess))
        return SGB_ERR_HIP;
    } else {
      if (hipEventRecord(p->ev[2], stream) != hipSuccess ||
          hipStreamWaitEvent(short_s, p->ev[2], 0) != hipSuccess ||
          (fresh && hipStreamWaitEvent(short_s, p->ev[1], 0) != hipSuccess))
        return SGB_ERR_HIP;
      mark_on(short_s, SGB_STAGE_REDUCE_SHORT, 0);
      if (launch_reduce_short(q, bf16, p->Dmin, p->Dmax, p->wide_grid, kShortRows | kWideRows,
                              short_s) != hipSuccess)
        return SGB_ERR_HIP;
      mark_on(short_s, SGB_STAGE_REDUCE_SHORT, 1);
    }
    if (hipEventRecord(p->ev[3], short_s) != hipSuccess) return SGB_ERR_HIP;
  }
  if (do_front) {
    mark(SGB_STAGE_RUNS, 0);
    if (launch_post(pp, (int)L.scan_tiles, stream) != hipSuccess) return SGB_ERR_HIP;
    mark(SGB_STAGE_RUNS, 1);
  }
  if (!do_reduce) return SGB_OK;
  if (fresh && hipStreamWaitEvent(stream, p->ev[1], 0) != hipSuccess) return SGB_ERR_HIP;
  mark(SGB_STAGE_REDUCE_LONG, 0);
  if (launch_reduce_long(q, bf16, p->red_grid[bf16 ? 1 : 0], stream) != hipSuccess)
    return SGB_ERR_HIP;
  mark(SGB_STAGE_REDUCE_LONG, 1);
  // join: the call's work is complete when `stream` reaches this point
  if (hipStreamWaitEvent(stream, p->ev[3], 0) != hipSuccess) return SGB_ERR_HIP;
  return SGB_OK;
}

}  // namespace

extern "C" {

sgb_status sgb_forward(sgb_plan p, const sgb_lookups* lk, const float* weights, float* output,
                       void* ws, size_t ws_bytes, void* stream_) {
  if (!p || !lk || !output) return SGB_ERR_INVALID_ARGUMENT;
  const int64_t N = lk->num_indices;
  const bool nobag = p->pooling == SGB_POOL_NONE;
  if (N < 0 || N >= (1ll << 30)) return SGB_ERR_INVALID_ARGUMENT;
  if (nobag && lk->per_sample_weights) return SGB_ERR_UNSUPPORTED;
  if (!lk->offsets && !(nobag && p->T == 1)) return SGB_ERR_INVALID_ARGUMENT;
  if (lk->offsets && (lk->B <= 0 || (int64_t)lk->B * p->T >= (1ll << 31)))
    return SGB_ERR_INVALID_ARGUMENT;
  if (N > 0 && (!lk->indices || !weights)) return SGB_ERR_INVALID_ARGUMENT;
  if (!aligned(output, 16) || (weights && !aligned(weights, 16))) return SGB_ERR_INVALID_ARGUMENT;
  if (!ws || !aligned(ws, 256) || ws_bytes < sizeof(Header)) return SGB_ERR_INVALID_ARGUMENT;
  DeviceGuard guard(p->device);
  if (!guard.ok) return SGB_ERR_HIP;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  Header* hdr = at<Header>(ws, 0);
  FwdParams f{};
  f.indices = lk->indices;
  f.offsets = lk->offsets;
  f.psw = lk->per_sample_weights;
  f.weights = weights;
  f.out = output;
  f.hsc = p->d_hsc;
  f.doff = p->d_doff;
  f.woff = p->d_woff;
  f.N = N;
  f.B = lk->offsets ? lk->B : 0;
  f.T = p->T;
  f.pooling = p->pooling;
  f.lpl = lanes_per_row(p->Dmin);
  f.Dmax = p->Dmax;
  f.segs_per_table = lk->offsets ? (int64_t)lk->B : N;
  f.waves_per_table = (f.segs_per_table + (64 / f.lpl) - 1) / (64 / f.lpl);
  f.out_stride = nobag ? (int64_t)p->doff[1] : (int64_t)p->doff[p->T];
  f.status = &hdr->status;
  f.epoch = next_epoch();
  f.header = hdr;
  if (f.waves_per_table == 0) {  // no segments: nothing to write; report this call clean
    return launch_init(ws, sizeof(Header), stream) == hipSuccess ? SGB_OK : SGB_ERR_HIP;
  }
  return launch_forward(f, stream) == hipSuccess ? SGB_OK : SGB_ERR_HIP;
}

sgb_status sgb_device_status(sgb_plan p, const void* ws, void* stream_, int32_t* out) {
  if (p && !ws) ws = p->scratch;  // the no-allocation entry point's scratch
  if (!p || !ws || !out) return SGB_ERR_INVALID_ARGUMENT;
  DeviceGuard guard(p->device);
  if (!guard.ok) return SGB_ERR_HIP;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  uint32_t v[2] = {0, 0};  // status word, epoch of the last call
  static_assert(offsetof(Header, status) == 0 && offsetof(Header, epoch) == 4, "header layout");
  if (hipMemcpyAsync(v, ws, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return SGB_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SGB_ERR_HIP;
  *out = (v[0] >> 8) == v[1] ? (int32_t)(v[0] & 0xFFu) : (int32_t)SGB_OK;
  return SGB_OK;
}

sgb_status sgb_runs_view_get(sgb_plan p, const void* ws, int64_t N, int32_t B,
                             sgb_runs_view* out) {
  if (p && !ws) ws = p->scratch;  // the no-allocation entry point's scratch
  if (!p || !ws || !out) return SGB_ERR_INVALID_ARGUMENT;
  Layout L;
  const bool nobag_no_off = p->pooling == SGB_POOL_NONE && B == 0;
  sgb_status st = make_layout(p, N, B, !nobag_no_off, &L);
  if (st != SGB_OK) return st;
  // the layout must be the one the last call on this workspace used: it
  // recorded its N and B in the header
  {
    DeviceGuard guard(p->device);
    if (!guard.ok) return SGB_ERR_HIP;
    Header h;
    if (hipMemcpy(&h, ws, sizeof(Header), hipMemcpyDeviceToHost) != hipSuccess) return SGB_ERR_HIP;
    if (h.num_indices != N || (N > 0 && h.B != (nobag_no_off ? 0 : B)))
      return SGB_ERR_INVALID_ARGUMENT;
  }
  void* w = const_cast<void*>(ws);
  Header* hdr = at<Header>(w, L.hdr);
  out->sorted_packed = at<uint64_t>(w, (L.npasses % 2 == 0) ? L.kvA : L.kvB);
  out->info_bits = L.info_bits;
  out->unique_ids = at<int64_t>(w, L.uniq);
  out->run_lengths = at<int32_t>(w, L.lens);
  out->cumulative = at<int32_t>(w, L.cum);
  out->num_runs = &hdr->num_runs;
  out->long_run_ids = at<int32_t>(w, L.longs);
  out->num_long_run_ids = &hdr->num_long;
  return SGB_OK;
}

}  // extern "C"
