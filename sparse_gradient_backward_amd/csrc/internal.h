// internal.h -- definitions shared by the library's host code (api.cpp) and
// its gfx950 kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>


namespace sgb {

// ---------------------------------------------------------------- limits
constexpr int kMaxDigitBits = 10;     // LSD digits of <= 10 bits
constexpr int kMaxPasses = 4;         // linear ids below 2^40
constexpr int kRadixMax = 1 << kMaxDigitBits;
constexpr int kColBlock = 256;        // columns one wave covers per pass (64 lanes x 4)
constexpr int kMaxD = 8192;

// Tuning knobs (compile-time; the defaults are the measured best).
#ifndef SGB_SHORT_UNR
#define SGB_SHORT_UNR 2
#endif
#ifndef SGB_LONG_UNR
#define SGB_LONG_UNR 8
#endif
#ifndef SGB_MAX_CHUNKS
#define SGB_MAX_CHUNKS 1024
#endif
#ifndef SGB_CHUNK_DIV
#define SGB_CHUNK_DIV 8192
#endif
#ifndef SGB_CHUNK_FLOOR
#define SGB_CHUNK_FLOOR 128
#endif
#ifndef SGB_SHORT_SUB8
#define SGB_SHORT_SUB8 1
#endif
#ifndef SGB_SHORT_SUB16
#define SGB_SHORT_SUB16 2
#endif
#ifndef SGB_WIDE_CPL
#define SGB_WIDE_CPL 8
#endif
#ifndef SGB_WIDE_UNR
#define SGB_WIDE_UNR 4
#endif
#ifndef SGB_WIDE_UNR16
#define SGB_WIDE_UNR16 4
#endif
#ifndef SGB_WIDE_WAVES
#define SGB_WIDE_WAVES 8
#endif
#ifndef SGB_WIDE_GRID_MULT
#define SGB_WIDE_GRID_MULT 16
#endif
#ifndef SGB_SHORT8_WAVES
#define SGB_SHORT8_WAVES 6
#endif
#ifndef SGB_FILL_CUS_PER_WG
#define SGB_FILL_CUS_PER_WG 1
#endif
#ifndef SGB_FILL_THREADS
#define SGB_FILL_THREADS 256
#endif
#ifndef SGB_LIN_WG_PER_CU
#define SGB_LIN_WG_PER_CU 6
#endif
#ifndef SGB_LOOKBACK
#define SGB_LOOKBACK 4
#endif
#ifndef SGB_SERIAL_MAX_N
#define SGB_SERIAL_MAX_N 16384
#endif
#ifndef SGB_EARLY_FORK_MAX_N
#define SGB_EARLY_FORK_MAX_N (1 << 22)
#endif
#ifndef SGB_ONE_PASS_TILES
#define SGB_ONE_PASS_TILES 128
#endif
#ifndef SGB_FUSE_SCAN_TILES
#define SGB_FUSE_SCAN_TILES 4096
#endif
constexpr int kSortLbGroup = 16;  // tiles per look-back group of a radix pass

// Radix pass tiling.  A pass is one kernel (k_sort_pass) whose workgroups
// each sort one tile of TPB threads x ITEMS items; the shape depends on the
// batch and on the pass's digit width (its LDS holds the tile and one digit
// table per wave, so 10-bit digits take the smaller tiles):
//   huge     512 x 12 ( 6144 items), digits up to 9 bits, N > kSortHugeN
//   large   1024 x I  (I = 8..12), digits up to 9 bits, N > kSortLargeN: the
//           fewest items per thread that keep the tiles within the CUs, so
//           that every tile is resident at once and the pass is one round
//           (more than 12 would exceed the LDS)
//   medium   512 x 8  ( 4096 items), N > kSortMediumN
//   small    256 x 8  ( 2048 items)
// (A batch of a few thousand lookups sorts in a handful of tiles, each one
// latency chain: medium tiles, with twice the waves ranking, take the chain
// in half the rounds.)
// (A large tile fills one CU.  Beyond 12 x 1024 items per CU the pass takes
// several rounds, and two half-size tiles per CU overlap one's loads with
// the other's ranking.)
#ifndef SGB_SORT_HUGE_N
#define SGB_SORT_HUGE_N (1 << 22)
#endif
#ifndef SGB_SORT_LARGE_N
#define SGB_SORT_LARGE_N (1 << 20)
#endif
#ifndef SGB_SORT_MEDIUM_N
#define SGB_SORT_MEDIUM_N (1 << 12)
#endif
// shape codes: kSortLarge8 + (I - 8) is the large shape with I items
enum SortShape {
  kSortSmall = 0,
  kSortMedium = 1,
  kSortHuge = 2,
  kSortLarge8 = 3,
  kSortLarge12 = kSortLarge8 + 4
};
__host__ __device__ inline int sort_shape_for(int64_t N, int bits, int cus) {
  if (N > (int64_t)SGB_SORT_HUGE_N && bits <= 9) return kSortHuge;
  if (N > (int64_t)SGB_SORT_LARGE_N && bits <= 9) {
    int items = 8;
    while (items < 12 && (N + 1024 * items - 1) / (1024 * items) > (int64_t)cus) ++items;
    return kSortLarge8 + (items - 8);
  }
  if (N > (int64_t)SGB_SORT_MEDIUM_N) return kSortMedium;
  return kSortSmall;
}
__host__ __device__ inline int sort_tile_items(int shape) {
  if (shape >= kSortLarge8 && shape <= kSortLarge12) return 1024 * (8 + shape - kSortLarge8);
  return shape == kSortHuge ? 512 * 12 : (shape == kSortMedium ? 512 * 8 : 256 * 8);
}
// fewest items of any tile shape: bounds the tiles of a batch
constexpr int kSortTileMin = 256 * 8;
// copies of each pass's global digit histogram: workgroups add their counts
// into copy (workgroup id mod kHistSlices), spreading same-address atomics;
// readers sum the copies
constexpr int kHistSlices = 8;

// zero fill: threads of each (looping) workgroup
constexpr int kFillThreads = SGB_FILL_THREADS;

// groups of tiles of the scalar look-backs (run-length encoding, run
// post-processing): their look-back words are [tiles] then [groups]
constexpr int kLbScalarGroupTiles = 32;

// run-length encoding: up to kOnePassTiles tiles k_rle_write alone (each
// tile's first run index by look-back over the tiles' head counts); up to
// kFuseScanTiles k_rle_count, then k_rle_write summing the counts before its
// tile; beyond that k_rle_count, k_rle_scan and k_rle_write
constexpr int kOnePassTiles = SGB_ONE_PASS_TILES;
constexpr int kFuseScanTiles = SGB_FUSE_SCAN_TILES;
// Batches of at most kSerialMaxN lookups run every kernel on the caller's
// stream: their kernels are a few microseconds each, and the fork to the
// plan's side streams and the join cost more than the overlap returns.
constexpr int64_t kSerialMaxN = SGB_SERIAL_MAX_N;
// Batches of kSerialMaxN to kEarlyForkMaxN lookups start the reducer of short
// runs (rows up to 512 columns) as soon as the ids are sorted: it finds the
// length of each window's last run by scanning the sorted words after the
// window, and runs beside run-length encoding and the long-run list instead
// of after them.  That needs a long-run threshold that bounds the scan to a
// few reads (kScanRunsMaxThr words).  Larger batches fork after run-length
// encoding: their short-run reducer fills the chip for hundreds of
// microseconds, and sharing it with the scans delays the long-run reducer by
// more than the early start returns.
constexpr int64_t kEarlyForkMaxN = SGB_EARLY_FORK_MAX_N;
constexpr int kScanRunsMaxThr = 4096;

// run-length encoding / run post-processing tiling
constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanTile = kScanThreads * kScanItems;

// linearisation: bags per tile, lookups per inner step
constexpr int kLinThreads = 256;
constexpr int kLinBags = 64;
constexpr int kLinLookups = 4 * kLinThreads;
constexpr int kLinPer = 8;            // lookups per thread whose loads are issued together
constexpr int kLinHistCopies = 4;     // copies of the first-pass digit histogram in LDS
static_assert(kLinBags < kLinThreads, "one thread per bag offset of a tile");
static_assert((kLinBags & (kLinBags - 1)) == 0, "the bag search halves a power of two");

// short runs: sorted positions of one window of the short-run reducer, and
// log2 of the waves sharing a window (each serves the runs starting in its
// part), for rows up to 512 columns and for wider rows
constexpr int kShortSpan = 64;
constexpr int kShortSub8 = SGB_SHORT_SUB8;
constexpr int kShortSub16 = SGB_SHORT_SUB16;
static_assert(kShortSub8 >= 0 && kShortSub8 <= 6 && kShortSub16 >= 0 && kShortSub16 <= 6,
              "a window of 64 positions splits into at most 64 parts");

// short runs of rows wider than 512 columns: columns per lane (4, 8 or 16) of
// a dense / SGD item and lookups gathered per round; row-wise Adagrad items
// always take 16 columns per lane (a whole row of up to 1024)
constexpr int kWideCpl = SGB_WIDE_CPL;
constexpr int kWideUnr = SGB_WIDE_UNR;
constexpr int kWideUnr16 = SGB_WIDE_UNR16;
// workgroups of the wide-row reducer: this many times those resident at once
constexpr int kWideGridMult = SGB_WIDE_GRID_MULT;
static_assert(kWideCpl == 4 || kWideCpl == 8 || kWideCpl == 16, "pieces of 4 columns, 256 apart");

// long runs: chunk sizing and two-level combine
constexpr int kMaxChunks = SGB_MAX_CHUNKS;  // a run is cut into at most this many chunks
constexpr int kSuperChunk = 32;       // chunks combined per first-level ticket

// Lanes that cover a row of D columns at 4 columns per lane: the power of two
// covering D / 4, between 4 and 64 (wider rows take several 256-column blocks).
__host__ __device__ inline int lanes_per_row(int D) {
  const int need = (D + 3) >> 2;
  int l = 4;
  while (l < need && l < 64) l <<= 1;
  return l;
}

// 256-column blocks a row of D columns spans.
__host__ __device__ inline int col_blocks(int D) { return (D + kColBlock - 1) / kColBlock; }

// Chunk base of one call: lookups per chunk of a long run in a one-block row.
// Larger batches have more long-run work, so their chunks are larger (fewer
// items, less fixed cost each); small batches need more, shorter items to
// fill the GPU.  A power of two in [kChunkBaseMin, kChunkBaseMax].
constexpr int kChunkBaseMin = 128;
constexpr int kChunkBaseMax = 512;
__host__ __device__ inline int chunk_base_for(int64_t N) {
  int b = kChunkBaseMin;
  while (b < kChunkBaseMax && (int64_t)b * 2 * SGB_CHUNK_DIV <= N) b *= 2;
  return b;
}

// Fewest lookups in one chunk of a long run.  A work item is one chunk times
// one 256-column block; a row of several blocks already spreads a chunk over
// several waves, so its chunks are proportionally shorter (down to a floor).
__host__ __device__ inline int chunk_min(int D, int base) {
  const int c = base / col_blocks(D);
  return c > SGB_CHUNK_FLOOR ? c : SGB_CHUNK_FLOOR;
}

// Lookups per chunk of a long run of `len` lookups in a table of width D.
__host__ __device__ inline int chunk_len(int len, int D, int base) {
  const int c = (len + kMaxChunks - 1) / kMaxChunks;
  const int m = chunk_min(D, base);
  return c > m ? c : m;
}

// bounded waits (look-back): iterations of ~1 us before giving up
constexpr uint32_t kSpinLimit = 1u << 21;

// status codes written by kernels (values match sgb_status)
constexpr uint32_t kStIndex = 4;
constexpr uint32_t kStOffsets = 5;
constexpr uint32_t kStInternal = 7;

enum { kPoolSum = 0, kPoolMean = 1, kPoolNone = 2 };
enum { kModeDense = 0, kModeSgd = 1, kModeAdagrad = 2 };

// Workspace header (offset 0).
// Nothing in it needs clearing between calls: errors are tagged with the
// call's epoch (a call reads as error-free unless its own epoch is in the
// status word), and linearisation resets the tile counter.
struct Header {
  uint32_t status;                    // epoch << 8 | first device-detected error of that call
  uint32_t epoch;                     // epoch of the last call (set while linearising)
  uint32_t post_tile_ctr;             // dynamic tile ids of the run post-processing
  uint32_t rle_tile_ctr;              // dynamic tile ids of the run-length encoding
  int32_t num_runs;                   // U
  uint32_t total_items;               // chunks over all long runs
  int64_t num_long;                   // number of long runs
  int64_t num_indices;                // N of the last call (its run structure's layout)
  int32_t B;                          // B of the last call (0: nobag without offsets)
  uint32_t hist_ready;                // epoch once the first pass's histogram is zeroed
  uint32_t sort_tile_ctr[4];          // dynamic tile ids of each radix pass
  uint32_t pad[16];
};
static_assert(sizeof(Header) <= 128, "header too large");
static_assert(offsetof(Header, num_indices) % 8 == 0, "aligned counts");

// A long run as the long-run reducer needs it (written by k_post).
struct LongRun {
  int32_t start;   // first sorted position
  int32_t len;     // lookups
  int32_t t;       // table
  int32_t ncb;     // 256-column blocks of its row
  uint32_t cbeg;   // first work item / partial slot
  int32_t nch;     // chunks
  int64_t id;      // linear row id
  int32_t D;       // row width
  int32_t gcol;    // first grad_output column of its table (0 without bags)
  int64_t out;     // element offset of its row in the weights / dense grad
  int64_t mom;     // its Adagrad state index (its row among all tables)
};

// A block of rows of one table that the dense zero-fill covers.
struct FillBlock {
  int32_t t;
  int32_t nrows;
  int64_t row0;
};

// ---------------------------------------------------------------- kernel parameters

struct LinParams {
  const int64_t* indices;
  const int64_t* offsets;   // NULL: nobag, single table, no bags
  const float* psw;
  const int64_t* hsc;       // [T+1]
  int64_t N;
  int32_t B;
  int32_t T;
  int32_t pooling;
  int32_t info_bits;
  uint64_t* kv_out;
  float* coef_out;          // NULL when every coefficient is 1
  uint32_t* status;
  uint32_t epoch;
  Header* header;           // epoch and counters reset by the first workgroup
  uint4* zero_begin;        // region zeroed for the later kernels
  int64_t zero_vec4;
  // digit histogram of the first radix pass ([kHistSlices][1 << hist_bits]),
  // NULL when the ids need no sorting: zeroed by workgroup 0, which then
  // publishes the call's epoch in hist_ready; every workgroup adds its counts
  // once it sees that epoch
  uint32_t* hist;
  int32_t hist_bits;        // the first pass's digit: the low hist_bits bits of the id
  uint32_t* hist_ready;
};

struct SortParams {
  const uint64_t* kv_in;
  const float* coef_in;     // NULL when there are no coefficients
  uint64_t* kv_out;
  float* coef_out;
  int64_t N;
  int32_t tiles;            // tiles of sort_tile_items(shape) lookups
  int32_t shape;            // sort_shape_for(N, bits, CUs)
  int32_t shift;
  int32_t bits;
  const uint32_t* hist;     // [kHistSlices][1 << bits]: this pass's digit totals
  uint32_t* hist_next;      // [kHistSlices][1 << bits_next] (zeroed), or NULL on the last pass
  int32_t shift_next;
  int32_t bits_next;
  uint32_t* lookback;       // (zeroed) [tiles][1 << bits]: each tile's digit counts, then
                            // its inclusive prefix over the tiles; then
                            // [ceil(tiles / 16)][1 << bits]: per group of 16 tiles, its
                            // total, then the inclusive prefix at its end
  uint32_t* tile_ctr;       // (zeroed) tile ids in start order
  uint32_t* status;
  uint32_t epoch;
};

struct RleParams {
  const uint64_t* kv;       // sorted
  int64_t N;
  int64_t tiles;            // tiles of kScanTile positions
  int32_t info_bits;
  int64_t* unique_ids;
  int32_t* cum;
  int32_t* head_run;        // [N]: run index at each run's first position
  int32_t* num_runs;
  uint32_t* lookback;       // zeroed per call: [tiles] then [groups of 32 tiles] look-back words
  uint32_t* tile_ctr;       // dynamic tile ids (zeroed per call)
  uint32_t* tile_runs;      // [tiles]: runs starting in each tile, then the first run index
  int32_t one_pass;         // tiles <= kOnePassTiles: k_rle_write alone, by look-back
  int32_t fuse_scan;        // tiles <= kFuseScanTiles: k_rle_write sums the counts itself
  uint32_t* status;
  uint32_t epoch;
};

struct PostParams {
  const int32_t* cum;
  const int32_t* num_runs;
  const int64_t* unique_ids;
  const uint64_t* kv;       // sorted packed words (table of a run from its info)
  const int32_t* doff;
  int32_t info_bits;
  int32_t B;
  int32_t T;
  int32_t nobag;
  int32_t thr;
  int32_t chunk_base;       // chunk_base_for(N)
  const int64_t* hsc;       // [T+1]
  const int64_t* woff;      // [T+1]
  int32_t* run_lengths;
  int32_t* long_ids;
  uint32_t* chunk_begin;    // [num_long + 1]: first (chunk, column block) item of each long run
  LongRun* long_recs;       // [num_long]
  int64_t* num_long;
  uint32_t* total_items;
  int64_t tiles;            // tiles of kScanTile runs the grid covers at most
  uint64_t* lookback;       // zeroed per call: [tiles] then [groups of 32 tiles]
  uint32_t* tile_ctr;
  uint32_t* status;
  uint32_t epoch;
};

struct FillParams {
  float* out;
  const FillBlock* blocks;
  int32_t nblocks;
  const int32_t* doff;
  const int64_t* woff;
};

struct RedParams {
  const void* grad;
  const uint64_t* kv;       // sorted packed (id << info_bits | info)
  const float* coef;        // sorted coefficients or NULL
  const int64_t* hsc;
  const int32_t* doff;
  const int64_t* woff;
  const int64_t* unique_ids;
  const int32_t* cum;
  const int32_t* head_run;
  const int32_t* long_ids;
  const uint32_t* chunk_begin;
  const LongRun* long_recs;
  const int32_t* num_runs;
  const uint32_t* total_items;
  const int64_t* num_long;
  const Header* header;     // the workspace's header: N and B of the run structure
  uint32_t* sc_ticket;
  uint32_t* run_ticket;
  double* partials;         // fp64 partial sums of long-run work items
  float* out;               // fp32 weights (SGD/Adagrad) or dense grad
  uint16_t* out_h;          // bf16 or fp16 weights (SGD/Adagrad), w_kind 1 or 3
  uint8_t* out_q;           // INT8 weight rows (D codes, fp32 scale, fp32 bias), w_kind 2
  const int64_t* woff8;     // [T+1] byte offset of table t's INT8 rows
  float* mom;               // Adagrad state
  uint32_t* status;
  int64_t N;
  int64_t row_stride;       // elements per grad_output row
  int32_t info_bits;
  int32_t B;
  int32_t T;
  int32_t nobag;
  int32_t thr;
  int32_t chunk_base;       // chunk_base_for(N)
  int32_t sub_log;          // short-run reducer: log2 of the waves per window
  int32_t scan_runs;        // short-run reducer: find the length of a window's last run
                            // from the sorted words after it, not from the run starts
  int32_t wide_ncb;         // wide-row reducer: column blocks per run
  int32_t mode;
  int32_t accumulate;
  float lr;
  float eps;
  int32_t w_kind;           // weights: 0 fp32 (out), 1 bf16 (out_h), 2 INT8 rows (out_q),
                            // 3 fp16 (out_h)
  int32_t sr;               // 16-bit rows: stochastic rounding, else nearest even
  uint32_t sr_key0, sr_key1, sr_ctr3;  // Philox key (seed) and counter word 3 (offset)
};

struct FwdParams {
  const int64_t* indices;
  const int64_t* offsets;   // NULL: nobag, one table, every lookup its own segment
  const float* psw;
  const float* weights;
  float* out;
  const int64_t* hsc;       // [T+1]
  const int32_t* doff;      // [T+1]
  const int64_t* woff;      // [T+1]
  int64_t N;
  int32_t B;
  int32_t T;
  int32_t pooling;
  int32_t lpl;              // lanes per segment: lanes_per_row(narrowest D)
  int32_t Dmax;             // widest D
  int64_t segs_per_table;   // B, or N without offsets
  int64_t waves_per_table;  // ceil(segs_per_table / (64 / lpl))
  int64_t out_stride;       // elements per output row
  uint32_t* status;
  uint32_t epoch;
  Header* header;
};

// ---------------------------------------------------------------- launchers (kernels.hip)

// Fixed device scratch of sgb_backward_noalloc: bytes of the per-GPU array,
// and its address on the current device (looked up once per device).
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_address(void** out);

hipError_t launch_init(void* header_and_hist, size_t bytes, hipStream_t s);
hipError_t launch_linearize(const LinParams& p, int grid, hipStream_t s);
hipError_t launch_sort_pass(const SortParams& p, hipStream_t s);
hipError_t launch_rle(const RleParams& p, hipStream_t s);
hipError_t launch_post(const PostParams& p, int grid, hipStream_t s);
hipError_t launch_fill(const FillParams& p, int grid, hipStream_t s);
hipError_t launch_reduce_long(const RedParams& p, bool bf16, int grid, hipStream_t s);
// wide_grid: blocks of the wide-row reducer, {fp32 Adagrad, fp32 other, bf16 Adagrad, bf16 other};
// parts: kShortRows (rows up to 512 columns) and/or kWideRows (wider rows)
constexpr int kShortRows = 1, kWideRows = 2;
hipError_t launch_reduce_short(const RedParams& p, bool bf16, int dmin, int dmax,
                               const int* wide_grid, int parts, hipStream_t s);
void reduce_wide_blocks_per_cu(int out[4]);
int reduce_long_blocks_per_cu(bool bf16);
hipError_t launch_forward(const FwdParams& p, hipStream_t s);

}  // namespace sgb
