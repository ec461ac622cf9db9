// kernels.hip -- gfx950 kernels of the pooled embedding-bag backward.
//
// Pipeline (no host synchronisation; the caller's stream unless noted):
//   k_init         zero the workspace header (empty batches only)
//   k_linearize    bags -> per-lookup packed word (linear id << info_bits | info)
//                  and coefficient; range and offset checks; zeroes the
//                  region the later kernels count in; counts the first radix
//                  pass's digits
//   k_sort_pass    one stable LSD radix pass (<= 10-bit digits) in a single
//                  sweep: each tile ranks its items by ballots, finds the
//                  items of each digit in earlier tiles by a decoupled
//                  look-back, and scatters through LDS; it counts the next
//                  pass's digits on the way
//   k_rle_count / k_rle_scan / k_rle_write
//                  run heads of the sorted ids -> unique ids, run starts, count
//                  (few tiles: k_rle_write alone, each tile's first run index
//                  by a two-level look-back over the tiles' head counts; more:
//                  the counts first, summed in k_rle_write; many: all three)
//   k_post         run lengths, ascending long-run list and records
//   k_fill         zeros of a fresh dense gradient (side stream, from the start)
//   k_reduce_short8 short runs of rows up to 512 columns (side stream, after
//                  run-length encoding; for mid-sized batches right after the
//                  sort, the length of a window's last run then read from the
//                  sorted ids after the window): the runs starting in a part
//                  of a 64-position window, one per lane group
//   k_reduce_wide  short runs of wider rows (same stream): (run, column
//                  block) items dealt round-robin to waves, several times
//                  more workgroups than fit at once
//   k_reduce_long  (chunk, column block) items of long runs, fp64 partials
//                  combined in a fixed order by the last-arriving workgroup
//   Every reducer finishes each row with the fused dense / SGD / row-wise
//   Adagrad step, on fp32, bf16 or fp16 (nearest-even or stochastic
//   rounding) or INT8 row-wise quantized weight rows (one instance per weight
//   kind), reading the table metadata through scalar loads and the weight
//   rows non-temporally.
//
// Method: "fbgemm_gpu/codegen/embedding_backward_split_template.cu" (FBGEMM),
// host entry `..._exact_cuda` (linearise, sort, run-length encode, long
// segments, per-run reduction, dense store or optimizer row update) and
// "tt_embeddings_cuda.cu" (FBTT-Embedding) for the SGD / row-wise Adagrad
// formulas.  The kernels here are designed for wave64 CDNA4; see the notes at
// each kernel for where they depart from the pages' CUDA design.
#include <mutex>

#include "internal.h"
#include "sgb.h"

namespace sgb {
namespace {

constexpr uint32_t kFlagA32 = 1u << 30;   // look-back word: aggregate only
constexpr uint32_t kFlagP32 = 2u << 30;   // look-back word: inclusive prefix
constexpr uint32_t kVal32 = (1u << 30) - 1;
constexpr uint64_t kFlagA64 = 1ull << 62;
constexpr uint64_t kFlagP64 = 2ull << 62;
constexpr uint64_t kVal64 = (1ull << 62) - 1;
constexpr uint64_t kField = (1ull << 31) - 1;  // two 31-bit fields in a 64-bit word

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t bits_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Records `code` as this call's error unless the call already has one: the
// status word holds epoch << 8 | code, and a word from an earlier epoch counts
// as no error.
__device__ __forceinline__ void set_status(uint32_t* st, uint32_t epoch, uint32_t code) {
  const uint32_t mine = (epoch << 8) | code;
  uint32_t old = __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while ((old >> 8) != epoch) {
    const uint32_t seen = atomicCAS(st, old, mine);
    if (seen == old) break;
    old = seen;
  }
}

// Records `code` if any lane of the wave has `bad`, with one atomic per wave
// (an error path must not turn into millions of same-address atomics).
// Wave-uniform call.
__device__ __forceinline__ void set_status_wave(uint32_t* st, uint32_t epoch, uint32_t code,
                                                bool bad) {
  const uint64_t m = __ballot(bad);
  if (m && lane_id() == __builtin_ctzll(m)) set_status(st, epoch, code);
}

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T x) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Exclusive scan over the W waves of a block (one value per thread).  `tmp`
// holds W values of LDS.  Contains two barriers.
template <typename T, int W = 4>
__device__ __forceinline__ T block_excl_scan(T x, T* tmp, T& total) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const T inc = wave_incl_scan(x);
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const T v = tmp[i];
    if (i < w) before += v;
    all += v;
  }
  __syncthreads();
  total = all;
  return before + inc - x;
}

// Decoupled look-back over scalar per-tile values for one whole wave
// (Merrill & Garland, "Single-pass Parallel Prefix Scan with Decoupled
// Look-back", 2016): publish this tile's aggregate, sum the earlier tiles'
// words back to the nearest inclusive prefix, publish ours.  Tile ids come
// from an atomic counter, so every tile waited on belongs to a workgroup that
// started earlier and is resident; the wait is still bounded and records
// kStInternal if it ever expires.  The word's top two bits flag an aggregate
// (A) or an inclusive prefix (P).
template <typename W>
struct LB;
template <>
struct LB<uint32_t> {
  static constexpr uint32_t A = kFlagA32, P = kFlagP32, V = kVal32;
  static constexpr int S = 30;
};
template <>
struct LB<uint64_t> {
  static constexpr uint64_t A = kFlagA64, P = kFlagP64, V = kVal64;
  static constexpr int S = 62;
};

// Two levels, for any number of tiles: the earlier tiles of this
// tile's group of kLbScalarGroup (one load per lane), then whole groups --
// each group's last tile publishes the group's total as soon as it has it,
// then the inclusive prefix at the group's end -- 64 groups per load round.
// Tiles that start together need a few rounds, not one per 64 tiles before
// them.  lbg has a word per group.  Wave-uniform call.
constexpr int kLbScalarGroup = kLbScalarGroupTiles;

template <typename W>
__device__ W wave_lookback2(W* lbt, W* lbg, uint32_t tile, W agg, uint32_t* status,
                            uint32_t epoch) {
  const int lane = lane_id();
  if (lane == 0)
    __hip_atomic_store(&lbt[tile], (tile == 0 ? LB<W>::P : LB<W>::A) | agg, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t grp = tile / kLbScalarGroup;
  const int nin = (int)(tile - grp * kLbScalarGroup);
  const bool glast = tile % kLbScalarGroup == kLbScalarGroup - 1;
  W excl = 0;
  bool done = tile == 0;
  uint32_t spins = 0;
  if (!done && nin > 0) {
    for (;;) {
      const bool in = lane < nin;
      const W v = in ? __hip_atomic_load(&lbt[tile - 1 - lane], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : (W)0;
      const uint32_t flag = (uint32_t)(v >> LB<W>::S);
      const uint64_t pref = __ballot(in && flag == 2);
      const uint64_t notready = __ballot(in && flag == 0);
      const int first = pref ? __builtin_ctzll(pref) : nin - 1;
      const uint64_t upto = (2ull << first) - 1ull;
      if (notready & upto) {
        if (++spins > kSpinLimit) {
          if (lane == 0) set_status(status, epoch, kStInternal);
          done = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        continue;
      }
      excl = wave_sum<W>(lane <= first ? (v & LB<W>::V) : (W)0);
      done = pref != 0;
      break;
    }
  }
  if (!done && glast && lane == 0)
    __hip_atomic_store(&lbg[grp], LB<W>::A | (excl + agg), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  int64_t top = (int64_t)grp - 1;
  while (!done) {
    const int64_t idx = top - lane;
    const W v = idx >= 0 ? __hip_atomic_load(&lbg[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : LB<W>::P;  // before group 0: prefix 0
    const uint32_t flag = (uint32_t)(v >> LB<W>::S);
    const uint64_t pref = __ballot(flag == 2);
    const uint64_t notready = __ballot(flag == 0);
    const int first = pref ? __builtin_ctzll(pref) : 64;
    const uint64_t upto = first >= 64 ? ~0ull : ((2ull << first) - 1ull);
    if (notready & upto) {
      if (++spins > kSpinLimit) {
        if (lane == 0) set_status(status, epoch, kStInternal);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    excl += wave_sum<W>(lane <= first ? (v & LB<W>::V) : (W)0);
    if (first < 64) break;
    top -= 64;
  }
  if (lane == 0) {
    const W incl = LB<W>::P | (excl + agg);
    __hip_atomic_store(&lbt[tile], incl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (glast) __hip_atomic_store(&lbg[grp], incl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return excl;
}

// ------------------------------------------------------------------ k_init

__global__ void k_init(uint4* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ------------------------------------------------------------------ k_linearize
//
// Bag (t, b) covers lookups [offsets[t*B+b], offsets[t*B+b+1]) in table-major
// order (FBGEMM `grad_mean_kernel`; FBTT `compute_rowidx_kernel` expands the
// same layout per lookup).  Each workgroup takes kLinBags consecutive bags,
// stages their offsets in LDS and maps every lookup of the range to its bag
// by binary search in LDS, so reads of `indices` and writes of the packed
// words are fully coalesced whatever the bag lengths.  The linear id is
// hash_size_cumsum[t] + index; the info is the bag number t*B + b (nobag:
// i*T + t); the coefficient folds the per-sample weight and the 1/L of MEAN
// pooling into one fp32 (the page instead writes a scaled copy of the whole
// grad_output in `grad_mean_kernel` and sorts the weights a second time).
// Malformed offsets are clamped and made non-decreasing per tile so that no
// access leaves the arrays; the error is recorded.

__global__ __launch_bounds__(kLinThreads) void k_linearize(LinParams p) {
  __shared__ int64_t s_off[kLinBags + 1];
  __shared__ int64_t s_h0[kLinBags];
  __shared__ int64_t s_E[kLinBags];
  __shared__ int32_t s_t[kLinBags];
  __shared__ float s_scale[kLinBags];
  // this workgroup's first-pass digit counts, in kLinHistCopies copies: lane
  // l adds into copy l % kLinHistCopies, so that the lanes of a hot digit
  // (skewed ids) do not all add to one address
  __shared__ uint32_t s_dig[kLinHistCopies][kRadixMax];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int radix0 = p.hist ? (1 << p.hist_bits) : 0;
  const uint32_t dmask0 = (uint32_t)radix0 - 1u;
  if (blockIdx.x == 0) {
    if (tid == 0) {
      p.header->epoch = p.epoch;
      p.header->num_indices = p.N;
      p.header->B = p.B;
      p.header->post_tile_ctr = 0u;
      p.header->rle_tile_ctr = 0u;
#pragma unroll
      for (int i = 0; i < kMaxPasses; ++i) p.header->sort_tile_ctr[i] = 0u;
    }
    // the first pass's histogram starts from zero: cleared here, before the
    // epoch is published in hist_ready (the other workgroups add their counts
    // only after they have seen it)
    for (int i = tid; i < kHistSlices * radix0; i += kLinThreads)
      __hip_atomic_store(&p.hist[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (tid == 0 && radix0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(p.hist_ready, p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  for (int i = tid; i < kLinHistCopies * radix0; i += kLinThreads)
    s_dig[i / radix0][i % radix0] = 0u;
  __syncthreads();

  for (int64_t q = blockIdx.x * (int64_t)kLinThreads + tid; q < p.zero_vec4;
       q += (int64_t)gridDim.x * kLinThreads)
    p.zero_begin[q] = make_uint4(0u, 0u, 0u, 0u);

  if (p.offsets == nullptr) {
    // nobag with a single table and no offsets: lookup i is token i of table 0
    const int64_t E = p.hsc[1];
    const int64_t tiles = (p.N + kLinLookups - 1) / kLinLookups;
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
      for (int k = 0; k < kLinLookups / kLinThreads; ++k) {
        const int64_t i = tile * kLinLookups + k * kLinThreads + tid;
        const bool valid = i < p.N;
        uint64_t key = 0;
        bool bad = false;
        if (valid) {
          int64_t idx = p.indices[i];
          if (idx < 0 || idx >= E) {
            bad = true;
            idx = idx < 0 ? 0 : E - 1;
          }
          key = (uint64_t)idx;
          p.kv_out[i] = (key << p.info_bits) | (uint64_t)i;
        }
        set_status_wave(p.status, p.epoch, kStIndex, bad);
        if (radix0 && valid) atomicAdd(&s_dig[tid % kLinHistCopies][(uint32_t)key & dmask0], 1u);
      }
    }
  } else {
    const int64_t nbags = (int64_t)p.B * p.T;
    const int64_t tiles = (nbags + kLinBags - 1) / kLinBags;
    // offsets of a tile's bags and the row range of each bag's table (the
    // table of bag t*B+b is known without offsets), loaded together; the next
    // tile's are loaded while this tile's lookups are in flight
    int64_t nov = 0, nh0 = 0, nh1 = 0;
    auto load_tile_meta = [&](int64_t tl) {
      const int64_t b = tl * kLinBags;
      const int n = (int)min((int64_t)kLinBags, nbags - b);
      if (tid <= n) nov = p.offsets[b + tid];
      if (tid < n) {
        int t = (int)((b + tid) / p.B);
        t = t < p.T ? t : p.T - 1;
        nh0 = p.hsc[t];
        nh1 = p.hsc[t + 1];
      }
    };
    if ((int64_t)blockIdx.x < tiles) load_tile_meta(blockIdx.x);
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
      const int64_t b0 = tile * kLinBags;
      const int nb = (int)min((int64_t)kLinBags, nbags - b0);
      if (tid == 0) s_bad = 0;
      const int64_t ov = nov, h0 = nh0, h1 = nh1;
      if (tid < nb) {
        const int t = (int)((b0 + tid) / p.B);
        s_t[tid] = t < p.T ? t : p.T - 1;
      }
      if (tile + gridDim.x < tiles) load_tile_meta(tile + gridDim.x);
      __syncthreads();
      if (tid <= nb) {
        const bool bad = ov < 0 || ov > p.N || (b0 + tid == 0 && ov != 0) ||
                         (b0 + tid == nbags && ov != p.N);
        if (bad) s_bad = 1;
        s_off[tid] = ov < 0 ? 0 : (ov > p.N ? p.N : ov);
      }
      if (tid < nb) {
        s_h0[tid] = h0;
        s_E[tid] = h1 - h0;
      }
      __syncthreads();
      if (tid >= 1 && tid <= nb && s_off[tid] < s_off[tid - 1]) s_bad = 1;
      __syncthreads();
      if (s_bad) {
        if (tid == 0) {
          set_status(p.status, p.epoch, kStOffsets);
          for (int j = 1; j <= nb; ++j)
            if (s_off[j] < s_off[j - 1]) s_off[j] = s_off[j - 1];
        }
        __syncthreads();
      }
      if (tid < nb) {
        const int64_t L = s_off[tid + 1] - s_off[tid];
        s_scale[tid] = (p.pooling == kPoolMean && L > 0) ? 1.0f / (float)L : 1.0f;
      }
      __syncthreads();
      const int64_t i0 = s_off[0], i1 = s_off[nb];
      for (int64_t c = i0; c < i1; c += kLinThreads * kLinPer) {
        // every load of the chunk first, then the work
        int64_t idx[kLinPer];
        float w[kLinPer];
#pragma unroll
        for (int k = 0; k < kLinPer; ++k) {
          const int64_t i = c + k * kLinThreads + tid;
          idx[k] = i < i1 ? p.indices[i] : 0;
          w[k] = (i < i1 && p.psw) ? p.psw[i] : 1.0f;
        }
#pragma unroll
        for (int k = 0; k < kLinPer; ++k) {
          const int64_t i = c + k * kLinThreads + tid;
          const bool valid = i < i1;
          uint64_t key = 0;
          bool bad = false;
          if (valid) {
            // the bag of lookup i: the last lo < nb with s_off[lo] <= i (empty
            // bags are passed over).  A fixed number of steps, so that the
            // searches of the kLinPer lookups overlap their LDS reads.
            int lo = 0;
#pragma unroll
            for (int step = kLinBags / 2; step >= 1; step >>= 1)
              if (lo + step < nb && s_off[lo + step] <= i) lo += step;
            const int t = s_t[lo];
            const int64_t E = s_E[lo];
            int64_t x = idx[k];
            if (x < 0 || x >= E) {
              bad = true;
              x = x < 0 ? 0 : E - 1;
            }
            key = (uint64_t)(s_h0[lo] + x);
            const uint64_t info = p.pooling == kPoolNone ? (uint64_t)i * (uint64_t)p.T + (uint64_t)t
                                                         : (uint64_t)(b0 + lo);
            p.kv_out[i] = (key << p.info_bits) | info;
            if (p.coef_out) p.coef_out[i] = s_scale[lo] * w[k];
          }
          set_status_wave(p.status, p.epoch, kStIndex, bad);
          if (radix0 && valid)
            atomicAdd(&s_dig[tid % kLinHistCopies][(uint32_t)key & dmask0], 1u);
        }
      }
      __syncthreads();
    }
  }
  if (!radix0) return;
  // add this workgroup's counts into one copy of the first pass's histogram,
  // once workgroup 0 has cleared it (it does so first, waiting for nothing)
  __syncthreads();
  if (tid == 0) {
    uint32_t spins = 0;
    while (__hip_atomic_load(p.hist_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != p.epoch) {
      if (++spins > kSpinLimit) {
        set_status(p.status, p.epoch, kStInternal);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    // pairs with the clearing workgroup's release fence: its zero stores are
    // visible to the adds below (ordered after this by the barrier)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  uint32_t* h = p.hist + (size_t)(blockIdx.x % kHistSlices) * radix0;
  for (int d = tid; d < radix0; d += kLinThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < kLinHistCopies; ++i) c += s_dig[i][d];
    if (c) __hip_atomic_fetch_add(&h[d], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------------ radix sort
//
// One stable LSD pass over `bits` (<= 10) digit bits at `shift` of the packed
// word is ONE kernel (a single sweep over the keys; the decoupled look-back of
// Merrill & Garland, "Single-pass Parallel Prefix Scan with Decoupled
// Look-back", 2016, kept per digit as in Adinets & Merrill, "Onesweep", 2022):
//   - each workgroup takes the next tile id from a counter, so ids follow the
//     order in which workgroups start and every earlier tile is running or
//     done;
//   - it ranks its items by digit, stably: the lanes of one item round find
//     their same-digit peers with one ballot per digit bit (a lane's peers
//     agree with it on every bit); rank = the wave's running count of the
//     digit + peers in lower lanes.  Items are loaded wave-striped, so
//     (wave, item, lane) order is input order.  The cost does not depend on
//     the data (LDS atomics would serialise on the hot digits of skewed ids);
//   - it publishes its per-digit counts, then, per digit, sums the counts of
//     earlier tiles back to the nearest tile that has published its
//     inclusive prefix (64 digits per wave, kLookback tiles per load round),
//     and publishes its own inclusive prefix;
//   - an item goes to base[digit] + items of its digit in earlier tiles +
//     its rank in the tile, base being the exclusive scan of the pass's
//     global digit histogram.  The histogram is counted before the pass: the
//     first pass's by k_linearize, each later pass's by the pass before it
//     (digit totals do not depend on the order of the keys).
// The tile is reordered by digit in LDS so that each digit's writes are
// contiguous; keys, then coefficients, pass through the same LDS buffer.

__device__ __forceinline__ uint32_t digit_of(uint64_t kv, int shift, uint32_t dmask) {
  return (uint32_t)(kv >> shift) & dmask;
}

// Look-back rounds: tiles whose published words one lane loads at once.
constexpr int kLookback = SGB_LOOKBACK;
// Tiles per look-back group (the first level of the look-back).
constexpr int kLbGroup = kSortLbGroup;

template <int TPB, int ITEMS, int RMAX>
__global__ __launch_bounds__(TPB) void k_sort_pass(SortParams p) {
  constexpr int W = TPB / 64;
  constexpr int TILE = TPB * ITEMS;
  constexpr int DPT = (RMAX + TPB - 1) / TPB;  // consecutive digits owned by a thread
  constexpr int CPW = (RMAX / 64 + W - 1) / W;  // 64-digit columns a wave looks back for
  // copies of the next pass's digit counts: lane l adds into copy l % NC, so
  // that the lanes of a hot digit (skewed ids) do not all hit one address
  constexpr int NC = RMAX <= 512 ? 8 : 4;
  static_assert(TILE < 65536, "16-bit wave offsets");
  __shared__ uint64_t s_kv[TILE];               // keys, then coefficients, in tile order by digit
  __shared__ uint16_t s_wcnt[W][RMAX];          // each wave's digit counts, then its offsets
  __shared__ uint32_t s_cnt[RMAX];              // the tile's count of each digit
  __shared__ uint32_t s_local[RMAX];            // the tile's exclusive offset of each digit
  __shared__ int32_t s_gbase[RMAX];             // destination of the digit's slot 0 minus s_local
  __shared__ uint32_t s_next[NC][RMAX];         // the tile's counts of the next pass's digits
  __shared__ uint32_t s_tmp[W];
  __shared__ uint32_t s_tile;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int radix = 1 << p.bits;
  const uint32_t dmask = (uint32_t)radix - 1u;
  const int radix_n = p.hist_next ? (1 << p.bits_next) : 0;
  const uint32_t nmask = (uint32_t)radix_n - 1u;
  const bool has_coef = p.coef_in != nullptr;
  if (tid == 0) s_tile = atomicAdd(p.tile_ctr, 1u);
  for (int i = tid; i < W * RMAX; i += TPB) (&s_wcnt[0][0])[i] = 0u;
  for (int i = tid; i < NC * RMAX; i += TPB) (&s_next[0][0])[i] = 0u;
  __syncthreads();
  const uint32_t tile = s_tile;
  if (tile >= (uint32_t)p.tiles) {  // a stale tile counter: never proceed out of range
    if (tid == 0) set_status(p.status, p.epoch, kStInternal);
    return;
  }
  const int64_t base = (int64_t)tile * TILE;
  const int tile_n = (int)min((int64_t)TILE, p.N - base);

  uint64_t kv[ITEMS];
  float cf[ITEMS];
  uint32_t rank[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int e = w * 64 * ITEMS + k * 64 + lane;
    const bool valid = e < tile_n;
    kv[k] = valid ? p.kv_in[base + e] : 0ull;
    cf[k] = (valid && has_coef) ? p.coef_in[base + e] : 0.0f;
  }
  // digit totals of the pass (sum of the histogram copies), owned digits
  uint32_t tot[DPT];
#pragma unroll
  for (int h = 0; h < DPT; ++h) {
    const int d = tid * DPT + h;
    uint32_t t = 0;
    if (d < radix) {
#pragma unroll
      for (int sl = 0; sl < kHistSlices; ++sl) t += p.hist[sl * radix + d];
    }
    tot[h] = t;
  }
  // rank within the wave.  First every item's same-digit peers (bit-major,
  // so that the ballots of the ITEMS items are independent work for the
  // scheduler), then the short chain through the wave's LDS counts; the
  // next pass's digits are counted on the way.
  uint32_t dg[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) dg[k] = digit_of(kv[k], p.shift, dmask);
  uint32_t mlo[ITEMS], mhi[ITEMS];  // lanes that differ from this one on some digit bit
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) mlo[k] = mhi[k] = 0u;
#pragma unroll
  for (int b = 0; b < kMaxDigitBits; ++b) {
    if (b < p.bits) {  // uniform
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) {
        // bit b of the digit as 0 or all ones (one sign-extending bit-field
        // extract), its ballot, and the lanes that disagree on it
        const int32_t t = (int32_t)(dg[k] << (31 - b));  // bit b in the sign
        const uint64_t m = __ballot(t < 0);
        const uint32_t sx = (uint32_t)(t >> 31);         // 0 or all ones
        mlo[k] |= (uint32_t)m ^ sx;
        mhi[k] |= (uint32_t)(m >> 32) ^ sx;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int e = w * 64 * ITEMS + k * 64 + lane;
    const bool valid = e < tile_n;
    const uint64_t live = __ballot(valid);
    const uint64_t peers = valid ? (~(((uint64_t)mhi[k] << 32) | mlo[k]) & live) : 0ull;
    const uint32_t d = dg[k];
    const uint32_t below = bits_below(peers);
    const uint32_t before = valid ? (uint32_t)s_wcnt[w][d] : 0u;
    rank[k] = before + below;
    if (valid && below == 0) s_wcnt[w][d] = (uint16_t)(before + (uint32_t)__popcll(peers));
    if (radix_n && valid) atomicAdd(&s_next[lane % NC][digit_of(kv[k], p.shift_next, nmask)], 1u);
  }
  __syncthreads();

  // per digit: exclusive offsets of the waves and the tile's count, published
  // at once for the look-back of later tiles (tile 0's count is already its
  // inclusive prefix)
  uint32_t cnt[DPT];
#pragma unroll
  for (int h = 0; h < DPT; ++h) {
    const int d = tid * DPT + h;
    uint32_t acc = 0;
    if (d < radix) {
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const uint32_t c = s_wcnt[ww][d];
        s_wcnt[ww][d] = (uint16_t)acc;
        acc += c;
      }
      s_cnt[d] = acc;
      __hip_atomic_store(&p.lookback[(size_t)tile * radix + d], (tile == 0 ? kFlagP32 : kFlagA32) | acc,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    cnt[h] = acc;
  }
  {
    uint32_t tot_all, dsum = 0, csum = 0;
#pragma unroll
    for (int h = 0; h < DPT; ++h) {
      dsum += tot[h];
      csum += cnt[h];
    }
    uint32_t g = block_excl_scan<uint32_t, W>(dsum, s_tmp, tot_all);
    uint32_t ex = block_excl_scan<uint32_t, W>(csum, s_tmp, tot_all);
#pragma unroll
    for (int h = 0; h < DPT; ++h) {
      const int d = tid * DPT + h;
      if (d < radix) {
        s_local[d] = ex;
        s_gbase[d] = (int32_t)g;
        // each wave's offset becomes its tile offset: one table read per
        // item below (the sum stays below TILE < 2^16)
#pragma unroll
        for (int ww = 0; ww < W; ++ww) s_wcnt[ww][d] = (uint16_t)(s_wcnt[ww][d] + ex);
      }
      g += tot[h];
      ex += cnt[h];
    }
  }
  __syncthreads();
  // tile position of every item: keys through LDS to their digit groups
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int e = w * 64 * ITEMS + k * 64 + lane;
    if (e < tile_n) {
      rank[k] += (uint32_t)s_wcnt[w][dg[k]];
      s_kv[rank[k]] = kv[k];
    }
  }
  // look-back in two levels: wave w serves the digit columns w, w + W, ...
  // (lane = digit).  First the earlier tiles of this tile's group of
  // kLbGroup; unless one of them already holds an inclusive prefix, the
  // group's last tile then publishes the group's total at once, and the walk
  // continues over the words of earlier groups (a group total, or the
  // inclusive prefix at the group's end).  Tiles that start together thus
  // need a few load rounds, not one per kLookback tiles before them.
  const uint32_t grp = tile / kLbGroup, gfirst = grp * kLbGroup;
  const bool glast = tile % kLbGroup == kLbGroup - 1;
  const int nin = (int)(tile - gfirst);  // earlier tiles of the group
  uint32_t* lbt = p.lookback;                              // [tiles][radix]
  uint32_t* lbg = p.lookback + (size_t)p.tiles * radix;    // [groups][radix]
#pragma unroll 1
  for (int ci = 0; ci < CPW; ++ci) {
    const int col = w + ci * W;
    if (col * 64 >= radix) break;  // uniform
    const int d = col * 64 + lane;
    const bool live = d < radix;  // fewer than 64 digits: the other lanes idle
    uint32_t excl = 0, spins = 0;
    bool done = tile == 0 || !live;
    bool in_done = done || nin == 0;
    while (__ballot(!in_done)) {
      uint32_t v[kLbGroup - 1];
#pragma unroll
      for (int j = 0; j < kLbGroup - 1; ++j)
        v[j] = (!in_done && j < nin)
                   ? __hip_atomic_load(&lbt[(size_t)(tile - 1 - j) * radix + d], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : 0u;
      bool wait = false;
      if (!in_done) {
        uint32_t sum = 0;
        bool found = false, ready = true;
#pragma unroll
        for (int j = 0; j < kLbGroup - 1; ++j) {
          if (j < nin && !found) {
            const uint32_t f = v[j] >> 30;
            ready = ready && f != 0u;
            sum += v[j] & kVal32;
            found = f == 2u;
          }
        }
        if (ready) {
          excl = sum;
          in_done = true;
          done = found;
        } else if (++spins > kSpinLimit) {
          set_status(p.status, p.epoch, kStInternal);
          in_done = done = true;
        } else {
          wait = true;
        }
      }
      if (__ballot(wait)) __builtin_amdgcn_s_sleep(1);
    }
    if (glast && live && !done)
      __hip_atomic_store(&lbg[(size_t)grp * radix + d], kFlagA32 | (excl + s_cnt[d]),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int64_t top = (int64_t)grp - 1;
    while (__ballot(!done)) {
      uint32_t v[kLookback];
#pragma unroll
      for (int j = 0; j < kLookback; ++j) {
        const int64_t gi = top - j;
        v[j] = (!done && gi >= 0) ? __hip_atomic_load(&lbg[(size_t)gi * radix + d],
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                  : kFlagP32;  // before group 0: prefix 0
      }
      bool wait = false;
      if (!done) {
        uint32_t sum = 0;
        bool found = false, ready = true;
#pragma unroll
        for (int j = 0; j < kLookback; ++j) {
          if (!found) {
            const uint32_t f = v[j] >> 30;
            ready = ready && f != 0u;
            sum += v[j] & kVal32;
            found = f == 2u;
          }
        }
        if (ready) {
          excl += sum;
          done = found;
          top -= kLookback;
        } else if (++spins > kSpinLimit) {
          set_status(p.status, p.epoch, kStInternal);
          done = true;
        } else {
          wait = true;
        }
      }
      if (__ballot(wait)) __builtin_amdgcn_s_sleep(1);
    }
    if (live) {
      const uint32_t incl = kFlagP32 | (excl + s_cnt[d]);
      __hip_atomic_store(&lbt[(size_t)tile * radix + d], incl, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (glast)
        __hip_atomic_store(&lbg[(size_t)grp * radix + d], incl, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      s_gbase[d] += (int32_t)excl - (int32_t)s_local[d];
    }
  }
  __syncthreads();
  // every slot's key and destination first (all LDS reads in flight), then
  // the stores; slot q of the tile goes to s_gbase[its digit] + q
  uint64_t v[ITEMS];
  int32_t pos[ITEMS];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int q = k * TPB + tid;
    v[k] = s_kv[q < tile_n ? q : 0];
  }
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) pos[k] = s_gbase[digit_of(v[k], p.shift, dmask)] + k * TPB + tid;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int q = k * TPB + tid;
    const bool okp = pos[k] >= 0 && (int64_t)pos[k] < p.N;
    if (q < tile_n) {
      if (okp)
        p.kv_out[pos[k]] = v[k];
      else
        bad = true;
    }
  }
  set_status_wave(p.status, p.epoch, kStInternal, bad);
  if (has_coef) {
    // coefficients the same way, through the same buffer once every key has
    // been read from it
    __syncthreads();
    float* s_cf = reinterpret_cast<float*>(s_kv);
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int e = w * 64 * ITEMS + k * 64 + lane;
      if (e < tile_n) s_cf[rank[k]] = cf[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int q = k * TPB + tid;
      if (q < tile_n && pos[k] >= 0 && (int64_t)pos[k] < p.N) p.coef_out[pos[k]] = s_cf[q];
    }
  }
  // the next pass's digit counts of this tile, into one copy of its histogram
  if (radix_n) {
    uint32_t* hn = p.hist_next + (size_t)(tile % kHistSlices) * radix_n;
    for (int d = tid; d < radix_n; d += TPB) {
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < NC; ++i) c += s_next[i][d];
      if (c) __hip_atomic_fetch_add(&hn[d], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ run-length encoding
//
// Run-length encoding of the sorted ids: position i starts a run when its id
// differs from position i-1.  Each tile counts its heads and needs the number
// of heads before it (its first run index); every head then writes its unique
// id and its start (the exclusive scan of run lengths, FBGEMM
// `sorted_linear_indices_cumulative_run_lengths`) and its run index at its
// position, and the last tile writes the run count U and the closing start N.
// The first run index comes one of three ways, by tile count:
//   <= kOnePassTiles   k_rle_write alone: tiles taken in order from an atomic
//                      counter, two-level decoupled look-back over the tiles'
//                      head counts (one read of the ids)
//   <= kFuseScanTiles  k_rle_count stores every tile's count, k_rle_write
//                      sums the counts before its tile
//   more               k_rle_count, k_rle_scan (one workgroup scans the
//                      counts), k_rle_write
// Beyond about a hundred tiles the one-pass look-back waits cost more than a
// second read of the ids (measured: 2561 tiles 56 us in one pass, 43 us with
// the counts first; 800 tiles 19 us and 15 us).  Items are read coalesced (item k of thread t is
// position k*256 + t); a position's predecessor is the previous lane, or for
// lane 0 the last lane of the wave before it in that order (through LDS).

// Ids of this thread's kScanItems positions and which of them start a run.
// Returns the head bits; ids land in key[].
__device__ __forceinline__ uint32_t rle_heads(const RleParams& p, int64_t base, int n,
                                              uint64_t* key, uint64_t (*s_edge)[kScanThreads / 64]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int q = k * kScanThreads + tid;
    key[k] = (q < n ? p.kv[base + q] : 0ull) >> p.info_bits;
  }
  const uint64_t before_tile =
      (tid == 0 && base > 0) ? (p.kv[base - 1] >> p.info_bits) : ~0ull;
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) s_edge[k][w] = key[k];
  }
  __syncthreads();
  uint32_t heads = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int q = k * kScanThreads + tid;
    uint64_t prev = __shfl_up(key[k], 1, 64);
    if (lane == 0) {
      if (w > 0)
        prev = s_edge[k][w - 1];
      else if (k > 0)
        prev = s_edge[k - 1][kScanThreads / 64 - 1];
      else
        prev = before_tile;
    }
    if (q < n && (base + q == 0 || key[k] != prev)) heads |= 1u << k;
  }
  return heads;
}

__global__ __launch_bounds__(kScanThreads) void k_rle_count(RleParams p) {
  __shared__ uint64_t s_edge[kScanItems][kScanThreads / 64];
  __shared__ uint32_t s_w[kScanThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanTile;
  const int n = (int)min((int64_t)kScanTile, p.N - base);
  uint64_t key[kScanItems];
  const uint32_t heads = rle_heads(p, base, n, key, s_edge);
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) c += (uint32_t)__popcll(__ballot((heads >> k) & 1u));
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int ww = 0; ww < kScanThreads / 64; ++ww) t += s_w[ww];
    p.tile_runs[blockIdx.x] = t;
  }
}

// one workgroup: tile counts -> first run index of every tile, U and the
// closing start N
__global__ __launch_bounds__(kScanThreads) void k_rle_scan(RleParams p) {
  __shared__ uint32_t s_tmp[kScanThreads / 64];
  const int tid = threadIdx.x;
  uint32_t carry = 0;
  for (int64_t c0 = 0; c0 < p.tiles; c0 += (int64_t)kScanThreads * kScanItems) {
    uint32_t v[kScanItems];
    uint32_t sum = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const int64_t j = c0 + (int64_t)tid * kScanItems + k;
      v[k] = j < p.tiles ? p.tile_runs[j] : 0u;
      sum += v[k];
    }
    uint32_t total;
    uint32_t run = carry + block_excl_scan<uint32_t>(sum, s_tmp, total);
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const int64_t j = c0 + (int64_t)tid * kScanItems + k;
      if (j < p.tiles) p.tile_runs[j] = run;
      run += v[k];
    }
    carry += total;
  }
  if (tid == 0) {
    p.cum[carry] = (int32_t)p.N;
    *p.num_runs = (int32_t)carry;
  }
}

__global__ __launch_bounds__(kScanThreads) void k_rle_write(RleParams p) {
  __shared__ uint64_t s_edge[kScanItems][kScanThreads / 64];
  __shared__ uint32_t s_off[kScanItems * (kScanThreads / 64)];
  __shared__ uint32_t s_tile, s_first;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t tile = blockIdx.x;
  if (p.one_pass) {
    if (tid == 0)
      s_tile = __hip_atomic_fetch_add(p.tile_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    tile = s_tile;
  }
  const int64_t base = (int64_t)tile * kScanTile;
  const int n = (int)min((int64_t)kScanTile, p.N - base);
  uint64_t key[kScanItems];
  const uint32_t heads = rle_heads(p, base, n, key, s_edge);
  if (!p.one_pass) {
    if (p.fuse_scan) {
      // each thread sums every 256th tile count, then a block sum
      __shared__ uint32_t s_sum[2][kScanThreads / 64];
      uint32_t before = 0, all = 0;
#pragma unroll 4
      for (int64_t j = tid; j < p.tiles; j += kScanThreads) {
        const uint32_t c = p.tile_runs[j];
        all += c;
        before += j < (int64_t)tile ? c : 0u;
      }
      before = wave_sum(before);
      all = wave_sum(all);
      if (lane == 0) {
        s_sum[0][w] = before;
        s_sum[1][w] = all;
      }
      __syncthreads();
      if (tid == 0) {
        before = 0;
        all = 0;
#pragma unroll
        for (int i = 0; i < kScanThreads / 64; ++i) {
          before += s_sum[0][i];
          all += s_sum[1][i];
        }
        s_first = before;
        if ((int64_t)tile == p.tiles - 1) {
          p.cum[all] = (int32_t)p.N;
          *p.num_runs = (int32_t)all;
        }
      }
    } else if (tid == 0) {
      s_first = p.tile_runs[tile];
    }
  }
  // heads of every (item round, wave) in tile order, then their exclusive
  // scan; in one pass also the tile's first run index by look-back
  uint64_t bal[kScanItems];
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    bal[k] = __ballot((heads >> k) & 1u);
    if (lane == 0) s_off[k * (kScanThreads / 64) + w] = (uint32_t)__popcll(bal[k]);
  }
  __syncthreads();
  if (w == 0) {
    static_assert(kScanItems * (kScanThreads / 64) == 64, "one lane per (item round, wave)");
    const uint32_t c = s_off[lane];
    uint32_t incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    s_off[lane] = incl - c;
    if (p.one_pass) {
      const uint32_t total = __shfl(incl, 63, 64);
      const uint32_t f = wave_lookback2<uint32_t>(p.lookback, p.lookback + p.tiles, tile, total,
                                                  p.status, p.epoch);
      if (lane == 0) {
        s_first = f;
        if ((int64_t)tile == p.tiles - 1) {
          p.cum[f + total] = (int32_t)p.N;
          *p.num_runs = (int32_t)(f + total);
        }
      }
    }
  }
  __syncthreads();
  const uint32_t first = s_first;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    if (!((heads >> k) & 1u)) continue;
    const int q = k * kScanThreads + tid;
    const uint32_t run = first + s_off[k * (kScanThreads / 64) + w] + bits_below(bal[k]);
    p.unique_ids[run] = (int64_t)key[k];
    p.cum[run] = (int32_t)(base + q);
    p.head_run[base + q] = (int32_t)run;
  }
}

// ------------------------------------------------------------------ k_post
//
// Run lengths, and the long runs -- length >= thr, FBGEMM `find_long_segments`
// -- compacted in ascending run order (the page appends them through an
// atomic counter in arbitrary order).  Each long run is cut into chunks of
// chunk_len() lookups (set by the row width) times the 256-column blocks of
// its row; a combined scan gives every long run its first work item.  (The
// combine tickets of the work items are cleared with the workspace's zeroed
// region.)

// Table metadata staged in LDS for up to kMetaT tables (read from global
// memory beyond that).  The loads are issued with the tile's first loads, so
// staging adds no memory round trip.
constexpr int kMetaT = 512;
constexpr int kMetaPer = (kMetaT + 1 + kScanThreads - 1) / kScanThreads;

struct MetaLds {
  int32_t doff[kMetaT + 1];
  int64_t hsc[kMetaT + 1];
  int64_t woff[kMetaT + 1];
};

// Table of linear id `id`: the last t with hsc[t] <= id (binary search over
// hsc[0..T), in LDS or global memory).
template <typename H>
__device__ __forceinline__ int table_of_id(const H* hsc, int T, int64_t id) {
  int lo = 0, hi = T;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (hsc[mid] <= id)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Work items of a long run of `len` lookups in a row of width D: nch
// chunks x ncb column blocks.
__device__ __forceinline__ uint32_t long_items(int len, int D, int base) {
  const int cl = chunk_len(len, D, base);
  return (uint32_t)(((len + cl - 1) / cl) * col_blocks(D));
}

__global__ __launch_bounds__(kScanThreads) void k_post(PostParams p) {
  __shared__ int32_t s_cum[kScanTile + 1];
  __shared__ uint32_t s_items[kScanTile];  // work items of each run (0: short)
  __shared__ int16_t s_lq[kScanTile];   // tile positions of the tile's long runs
  __shared__ uint32_t s_lc[kScanTile];  // their first work items
  __shared__ uint64_t s_tmp[4];
  __shared__ uint32_t s_tile;
  __shared__ uint64_t s_excl;
  __shared__ MetaLds s_meta;
  const int tid = threadIdx.x;
  const int U = *p.num_runs;
  // the grid is sized for N runs; workgroups past the last run leave before
  // taking a tile id, so the ids handed out are exactly the tiles of U runs
  if ((int64_t)blockIdx.x * kScanTile >= U) return;
  // table metadata loads first, so that they are in flight with the tile id
  const bool staged = p.T <= kMetaT;
  int32_t md[kMetaPer];
  int64_t mh[kMetaPer], mo[kMetaPer];
  if (staged) {
#pragma unroll
    for (int i = 0; i < kMetaPer; ++i) {
      const int j = min(i * kScanThreads + tid, p.T);
      md[i] = p.doff[j];
      mh[i] = p.hsc[j];
      mo[i] = p.woff[j];
    }
  }
  if (tid == 0) s_tile = __hip_atomic_fetch_add(p.tile_ctr, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t tile = s_tile;
  const int64_t base = (int64_t)tile * kScanTile;
  const int n = (int)min((int64_t)kScanTile, (int64_t)U - base);
  // run starts base .. base+n (n+1 values) and the run ids (used by long
  // runs only; loaded with the starts, from indices clamped into the tile,
  // so that no load waits for another)
  int32_t v[kScanItems];
  int64_t idv[kScanItems];
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int q = k * kScanThreads + tid;
    v[k] = p.cum[base + (q < n ? q : 0)];
    idv[k] = p.unique_ids[base + (q < n ? q : 0)];
  }
  const int32_t last = p.cum[base + n];
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int q = k * kScanThreads + tid;
    if (q < n) s_cum[q] = v[k];
  }
  if (tid == 0) s_cum[n] = last;
  if (staged) {
#pragma unroll
    for (int i = 0; i < kMetaPer; ++i) {
      const int j = i * kScanThreads + tid;
      if (j <= p.T) {
        s_meta.doff[j] = md[i];
        s_meta.hsc[j] = mh[i];
        s_meta.woff[j] = mo[i];
      }
    }
  }
  __syncthreads();
  auto doff_at = [&](int t) { return staged ? s_meta.doff[t] : p.doff[t]; };
  // work items of every run (0 for a short one), runs spread over the
  // threads: the long runs are usually a few adjacent ones
  uint32_t tmask = 0;  // runs of this thread (position k * kScanThreads + tid) that are long
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int q = k * kScanThreads + tid;
    if (q < n) {
      const bool lg = s_cum[q + 1] - s_cum[q] >= p.thr;
      int32_t D = 0;
      if (lg) {
        tmask |= 1u << k;
        const int t = staged ? table_of_id(s_meta.hsc, p.T, idv[k]) : table_of_id(p.hsc, p.T, idv[k]);
        D = doff_at(t + 1) - doff_at(t);
      }
      s_items[q] = (uint32_t)D;  // (the width for now)
    }
  }
#pragma unroll 1
  for (uint32_t m = tmask; m; m &= m - 1u) {
    const int q = __builtin_ctz(m) * kScanThreads + tid;
    s_items[q] = long_items(s_cum[q + 1] - s_cum[q], (int)s_items[q], p.chunk_base);
  }
  __syncthreads();
  // this thread's kScanItems consecutive runs: which are long, and their items
  uint32_t longmask = 0;
  uint64_t sum = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int q = tid * kScanItems + k;
    if (q < n && s_cum[q + 1] - s_cum[q] >= p.thr) {
      longmask |= 1u << k;
      sum += (1ull << 31) | s_items[q];
    }
  }
  uint64_t total;
  const uint64_t before = block_excl_scan<uint64_t>(sum, s_tmp, total);
  if (tid < 64) {
    const uint64_t ex = wave_lookback2<uint64_t>(p.lookback, p.lookback + p.tiles, tile, total,
                                                 p.status, p.epoch);
    if (tid == 0) s_excl = ex;
  }
  // run lengths, coalesced
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int q = k * kScanThreads + tid;
    if (q < n) p.run_lengths[base + q] = s_cum[q + 1] - s_cum[q];
  }
  __syncthreads();
  // the tile's long runs in order: tile-local slot -> position and first work
  // item (this thread's runs), then their records written by all threads in
  // parallel
  {
    uint64_t at = s_excl + before;
    uint32_t li = (uint32_t)(before >> 31);
#pragma unroll 1
    for (uint32_t m = longmask; m; m &= m - 1u) {
      const int q = tid * kScanItems + __builtin_ctz(m);
      s_lq[li] = (int16_t)q;
      s_lc[li] = (uint32_t)(at & kField);
      at += (1ull << 31) | s_items[q];
      ++li;
    }
  }
  __syncthreads();
  const uint32_t g0 = (uint32_t)(s_excl >> 31);
  const uint32_t nl_tile = (uint32_t)(total >> 31);
#pragma unroll 1
  for (uint32_t i = tid; i < nl_tile; i += kScanThreads) {
    const int q = s_lq[i];
    const int start = s_cum[q];
    const int len = s_cum[q + 1] - start;
    const int64_t id = p.unique_ids[base + q];
    const int t = staged ? table_of_id(s_meta.hsc, p.T, id) : table_of_id(p.hsc, p.T, id);
    const int d0 = doff_at(t), D = doff_at(t + 1) - d0;
    const int64_t h0 = staged ? s_meta.hsc[t] : p.hsc[t];
    const int64_t E = (staged ? s_meta.hsc[t + 1] : p.hsc[t + 1]) - h0;
    const int64_t wo = staged ? s_meta.woff[t] : p.woff[t];
    const int cl = chunk_len(len, D, p.chunk_base);
    int64_t row = id - h0;
    row = row < 0 ? 0 : (row < E ? row : E - 1);
    LongRun rec;
    rec.start = start;
    rec.len = len;
    rec.t = t;
    rec.ncb = col_blocks(D);
    rec.cbeg = s_lc[i];
    rec.nch = (len + cl - 1) / cl;
    rec.id = id;
    rec.D = D;
    rec.gcol = p.nobag ? 0 : d0;
    rec.out = wo + row * (int64_t)D;
    rec.mom = h0 + row;
    p.long_ids[g0 + i] = (int32_t)(base + q);
    p.chunk_begin[g0 + i] = s_lc[i];
    p.long_recs[g0 + i] = rec;
  }
  if (tid == 0 && base + n == U) {
    const uint64_t all = s_excl + total;
    const uint32_t nl = (uint32_t)(all >> 31);
    *p.num_long = nl;
    *p.total_items = (uint32_t)(all & kField);
    p.chunk_begin[nl] = (uint32_t)(all & kField);
  }
}

// ------------------------------------------------------------------ k_fill
//
// A fresh dense gradient starts from zeros (FBGEMM host entry starts from
// zeros_like(dev_weights)).  The whole buffer is cleared on a side stream
// while the ids are linearised and sorted; the reducers write the touched
// rows after it.

__global__ __launch_bounds__(kFillThreads) void k_fill(FillParams p) {
  // few workgroups, each looping over fill blocks: the fill saturates HBM
  // without holding the CU slots that the concurrent latency-bound kernels need
  for (int b = blockIdx.x; b < p.nblocks; b += gridDim.x) {
    const FillBlock fb = p.blocks[b];
    const int D = p.doff[fb.t + 1] - p.doff[fb.t];
    float4* out = reinterpret_cast<float4*>(p.out + p.woff[fb.t] + fb.row0 * (int64_t)D);
    const uint32_t total = (uint32_t)fb.nrows * (uint32_t)(D >> 2);
    for (uint32_t q = threadIdx.x; q < total; q += blockDim.x) out[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ------------------------------------------------------------------ reducers
//
// G_r[d] = sum over the lookups j of run r of coef_j * grad_output[row_j][col_t + d]
// (FBGEMM warp-per-row / cta-per-row kernels), then the row is written once.
// Lanes form groups of LPL lanes with 4 columns per lane (LPL = 4..64, the
// power of two covering D/4, capped at one wave); a row wider than 256
// columns is covered in column blocks of 256.
//
// k_reduce_short8: one wave per 64 consecutive sorted positions.  The wave
//   reads the packed words of its window once, finds the run heads in it
//   (id differs from the previous position), takes each run's length from the
//   run starts, and serves the short runs (length < thr) that start in the
//   window, one run per lane group, so a wave carries 64/LPL rows at a time.
//   Metadata of the window is broadcast lane to lane with the whole wave
//   active; the row's old value is fetched before the gather so the two
//   overlap.  Balanced by lookups, and the grid is fixed on the host.
// k_reduce_long: persistent waves take the long runs' (chunk, column block)
//   items round-robin.  For D < 256 the wave's lane groups take
//   contiguous shares of the chunk, merge adjacent lookups of one bag, and
//   are folded by a fixed xor tree.  A run of several chunks writes one fp64
//   partial per item; the last wave of each group of kSuperChunk chunks
//   (arrival ticket) adds them in chunk order, and the last group adds the
//   group sums in order and finishes the row: a deterministic reduction
//   across many workgroups without float atomics (the page keeps a long run
//   inside one block).

// Four grad_output elements as stored (4 x bf16 or 4 x fp32) and their fp32
// values.  Gathers load the raw bits under their condition and widen them
// only after every load of a round has been issued: widening inside the
// conditional block would make each load wait for its data before the next
// one starts.
template <bool BF16>
struct Raw4;
template <>
struct Raw4<true> {
  uint2 u;
};
template <>
struct Raw4<false> {
  float4 f;
};

template <bool BF16>
__device__ __forceinline__ Raw4<BF16> load_raw4(const void* base, int64_t elem) {
  if constexpr (BF16)
    return {*reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + elem)};
  else
    return {*reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem)};
}

template <bool BF16>
__device__ __forceinline__ Raw4<BF16> zero_raw4() {
  if constexpr (BF16)
    return {make_uint2(0u, 0u)};
  else
    return {make_float4(0.f, 0.f, 0.f, 0.f)};
}

// bf16 -> fp32 is exact: the 16 bits become the high half of the fp32 word.
template <bool BF16>
__device__ __forceinline__ float4 widen4(const Raw4<BF16>& r) {
  if constexpr (BF16)
    return make_float4(__uint_as_float(r.u.x << 16), __uint_as_float(r.u.x & 0xffff0000u),
                       __uint_as_float(r.u.y << 16), __uint_as_float(r.u.y & 0xffff0000u));
  else
    return r.f;
}

// Four fp64 accumulators.  Every product coef * value of fp32 (or widened
// bf16) operands is exact in fp64, and the sums of a row stay in fp64 until
// the row is written, where they are rounded once to fp32 -- so the result
// does not depend on the order in which lookups are summed beyond fp64
// rounding, however long or cancelling the run.
struct d4 {
  double x, y, z, w;
};

__device__ __forceinline__ d4 d4_zero() { return d4{0.0, 0.0, 0.0, 0.0}; }

__device__ __forceinline__ void d4_fma(d4& a, float c, const float4& v) {
  const double cd = (double)c;
  a.x = fma(cd, (double)v.x, a.x);
  a.y = fma(cd, (double)v.y, a.y);
  a.z = fma(cd, (double)v.z, a.z);
  a.w = fma(cd, (double)v.w, a.w);
}

__device__ __forceinline__ void d4_add(d4& a, const d4& b) {
  a.x += b.x;
  a.y += b.y;
  a.z += b.z;
  a.w += b.w;
}

__device__ __forceinline__ d4 d4_xor(const d4& a, int off) {
  return d4{__shfl_xor(a.x, off, 64), __shfl_xor(a.y, off, 64), __shfl_xor(a.z, off, 64),
            __shfl_xor(a.w, off, 64)};
}

__device__ __forceinline__ double d4_sumsq(const d4& a) {
  return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
}

__device__ __forceinline__ uint64_t info_mask(const RedParams& p) {
  return p.info_bits >= 64 ? ~0ull : ((1ull << p.info_bits) - 1ull);
}

__device__ __forceinline__ int table_of(const RedParams& p, uint32_t info) {
  const int t = p.nobag ? (int)(info % (uint32_t)p.T) : (int)(info / (uint32_t)p.B);
  return t < p.T ? t : p.T - 1;
}

// The run structure a reducer reads must be the one the linearisation of
// this call's lookups wrote (sgb_apply after sgb_prepare into the same
// workspace): the header records that call's N and B.  On a mismatch the
// reducer records an internal error and does nothing, instead of walking
// another batch's runs.  (The header is one value for the whole grid, so
// every wave takes the same branch.)
__device__ __forceinline__ bool runs_match(const RedParams& p) {
  const Header* h = p.header;
  const bool ok = h->num_indices == p.N && h->B == p.B;
  if (!ok && blockIdx.x == 0 && threadIdx.x == 0) set_status(p.status, h->epoch, kStInternal);
  return ok;
}

// Row of grad_output that a lookup of table t reads.
__device__ __forceinline__ int grad_row_of(const RedParams& p, uint32_t info, int t) {
  if (p.nobag) {
    const int64_t l = info / (uint32_t)p.T;
    return (int)(l < p.N ? l : p.N - 1);
  }
  const int64_t b = (int64_t)info - (int64_t)t * p.B;
  return (int)(b < 0 ? 0 : (b < p.B ? b : p.B - 1));
}

__device__ __forceinline__ float4 ld4(const float* q) { return *reinterpret_cast<const float4*>(q); }
__device__ __forceinline__ void st4(float* q, float4 v) { *reinterpret_cast<float4*>(q) = v; }

// A reducer reads each touched weight row once and writes it once: those
// accesses are non-temporal (streamed through the caches), which leaves the
// caches to the grad_output rows that many lookups gather (32 tables of 1M
// rows, 10.5M lookups, row-wise Adagrad: short-run reducer 490 -> 474 us).
typedef float f4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 ld4_nt(const float* q) {
  const f4v x = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(q));
  return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st4_nt(float* q, float4 v) {
  const f4v x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f4v*>(q));
}
__device__ __forceinline__ uint2 ld2_nt(const void* q) {
  const u2v x = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(q));
  return make_uint2(x.x, x.y);
}
__device__ __forceinline__ void st2_nt(void* q, uint2 v) {
  const u2v x = {v.x, v.y};
  __builtin_nontemporal_store(x, reinterpret_cast<u2v*>(q));
}

// Weight kinds of the reducer instances: fp32 rows (or a dense gradient),
// bf16 rows, INT8 rows (codes then the row's fp32 scale and bias), fp16 rows.
// Each kind has instances of its own, so that no instance carries another
// kind's rounding code (or its registers).
constexpr int kWF32 = 0, kWBF16 = 1, kWINT8 = 2, kWF16 = 3;
// the 16-bit kinds share their row layout and loads
constexpr bool is16(int wk) { return wk == kWBF16 || wk == kWF16; }

struct RowDst {
  void* out;    // the row's first element (fp32 / bf16) or first byte (INT8)
  float* mom;   // its Adagrad state
  int64_t lin;  // its linear id (the stochastic-rounding counter)
  int32_t D;    // its width (INT8: the parameters follow the D codes)
};

// A table's metadata for a wave-uniform table index, through scalar loads:
// the plan's arrays are read-only while a kernel runs, so they are read as
// constant memory (the scalar data cache) instead of through the vector
// memory path, where each lookup would wait behind the wave's gathers.
template <typename T>
__device__ __forceinline__ T ld_const(const T* a, int64_t i) {
  typedef const __attribute__((address_space(4))) T* cptr;
  return ((cptr)a)[i];
}

struct TabMeta {
  int32_t D;     // row width
  int32_t dcol;  // first column of the table in a grad_output row
  int64_t h0;    // first linear id
  int64_t E;     // rows
  int64_t wo;    // first element (INT8: byte) of the table's rows
};

template <int WK>
__device__ __forceinline__ TabMeta tab_meta(const RedParams& p, int t) {
  const int32_t d0 = ld_const(p.doff, t), d1 = ld_const(p.doff, t + 1);
  const int64_t h0 = ld_const(p.hsc, t), h1 = ld_const(p.hsc, t + 1);
  const int64_t wo = ld_const(WK == kWINT8 ? p.woff8 : p.woff, t);
  return TabMeta{d1 - d0, d0, h0, h1 - h0, wo};
}

template <int WK>
__device__ __forceinline__ RowDst row_dest(const RedParams& p, const TabMeta& tm, int64_t lin) {
  int64_t row = lin - tm.h0;
  row = row < 0 ? 0 : (row < tm.E ? row : tm.E - 1);
  RowDst d;
  if constexpr (WK == kWINT8)
    d.out = p.out_q + tm.wo + row * (int64_t)(tm.D + 8);
  else if constexpr (is16(WK))
    d.out = p.out_h + tm.wo + row * (int64_t)tm.D;
  else
    d.out = p.out + tm.wo + row * (int64_t)tm.D;
  d.mom = p.mom ? p.mom + tm.h0 + row : nullptr;
  d.lin = tm.h0 + row;
  d.D = tm.D;
  return d;
}

// ---- bf16 weight rows
//
// SGD and row-wise Adagrad may keep their rows in bf16.  A row is widened
// exactly to fp32, updated as an fp32 row is (fp64, rounded once to fp32),
// and rounded to bf16: to nearest even, or stochastically as the FBGEMM
// page's 16-bit weight store does with a Philox state seeded per call (the
// bodies are not printed; the generator here is the published
// Philox4x32-10 of Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3", SC'11).  Element (linear id r, column d) takes word
// d % 4 of the block with counter (d / 4, r mod 2^32, r / 2^32, offset) and
// key (seed mod 2^32, seed / 2^32), so the bits depend on the row and the
// column, never on which wave writes them.  Stochastic rounding adds the
// word's high 16 bits to the fp32 pattern and keeps the high half (the
// magnitude rounds up with probability dropped bits / 2^16); infinities keep
// their high half and NaNs stay quiet NaNs.

struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = U4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

__device__ __forceinline__ uint32_t bf16_nonfinite(uint32_t u) {
  return (u >> 16) | ((u & 0x007FFFFFu) ? 0x0040u : 0u);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u) return bf16_nonfinite(u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t bf16_sr(float x, uint32_t rnd) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u) return bf16_nonfinite(u);
  return (u + (rnd >> 16)) >> 16;
}

// ---- fp16 weight rows
//
// The 16-bit rows may also be IEEE binary16 (weight kind kWF16, with the
// layout and loads of bf16 rows).  Widening is exact.  Rounding works on the
// fp32 bit pattern: the significand m (implicit bit included) is cut at the
// binary16 grid of its binade (spacing 2^(max(E, -14) - 10) for fp32 exponent
// E, so values below 2^-14 land on the subnormal grid of 2^-24); the sh
// dropped bits decide the rounding, and a carry out of the kept bits moves to
// the next binade, to infinity past 65504.  Nearest even rounds up past half
// a spacing and on ties to an odd count; stochastic rounding rounds the
// magnitude up iff the element's 32-bit word w satisfies w < f * 2^32, f the
// dropped fraction (w an integer, so against the ceiling of f * 2^32).
// Infinities keep their sign; a NaN becomes the quiet NaN 0x7E00 with its
// sign.

__device__ __forceinline__ float f16_widen(uint32_t h) {
  // a normal binary16 value: its exponent rebased by 112 and its significand
  // moved up 13 bits (equal to the general path below for every input)
  if (((h >> 10) & 31u) - 1u < 30u)
    return __uint_as_float(((h & 0x8000u) << 16) | (((h & 0x7FFFu) + (112u << 10)) << 13));
  const uint32_t s = (h & 0x8000u) << 16, ex = (h >> 10) & 31u, man = h & 1023u;
  if (ex == 31u) return __uint_as_float(s | 0x7F800000u | (man << 13));
  if (ex != 0u) return __uint_as_float(s | ((ex + 112u) << 23) | (man << 13));
  // subnormal or zero: man * 2^-24, exact in fp32
  const float v = (float)man * 5.9604644775390625e-08f;
  return s ? -v : v;
}

__device__ __forceinline__ uint32_t f16_round(float x, uint32_t rnd, bool sr) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a - 0x38800000u < 0x0F000000u) {
    // 2^-14 <= |x| < 2^16, a normal binary16 binade: the dropped bits are the
    // low 13 of the fp32 pattern and the kept ones its exponent (rebased by
    // 112) and top 10 significand bits, so a carry from the rounding moves
    // into the exponent, and to infinity past 65504, by itself.  (Equal to
    // the general path below for every fp32 input.)
    const uint32_t rem = a & 0x1FFFu;
    const bool up = sr ? rnd < (rem << 19)
                       : (rem > 0x1000u || (rem == 0x1000u && ((a >> 13) & 1u)));
    return s | (((a >> 13) - 0x1C000u) + (up ? 1u : 0u));
  }
  if (a >= 0x7F800000u) return s | (a > 0x7F800000u ? 0x7E00u : 0x7C00u);
  if (a >= 0x47800000u) return s | 0x7C00u;  // |x| >= 65536
  const int e = (int)(a >> 23);
  const uint32_t m = (a & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  const int E = e ? e - 127 : -126;
  const int Eg = E > -14 ? E : -14;
  const int sh = 13 + (Eg - E);  // dropped bits, >= 13
  const uint32_t q = sh >= 24 ? 0u : m >> sh;
  const uint32_t rem = sh >= 24 ? m : (m & ((1u << sh) - 1u));
  bool up;
  if (!sr) {
    const uint32_t half = 1u << (sh - 1 < 31 ? sh - 1 : 31);
    up = sh <= 24 && (rem > half || (rem == half && (q & 1u)));
  } else {
    uint64_t thr;
    if (sh <= 32) {
      thr = (uint64_t)rem << (32 - sh);
    } else {
      const int k = sh - 32;
      thr = k >= 32 ? (uint64_t)(rem != 0u) : (((uint64_t)rem + (1ull << k) - 1ull) >> k);
    }
    up = (uint64_t)rnd < thr;
  }
  return s | ((((uint32_t)(Eg + 14)) << 10) + q + (up ? 1u : 0u));
}

// The row's old values at columns [col + off, col + off + 4): fp32, or bf16 /
// fp16 widened exactly.  The address is formed as (row + col) + off: the
// short-run reducer keeps row + col across its pieces, and forming
// row + (col + off) instead costs it a register (and a spill).
template <int WK>
__device__ __forceinline__ float4 ldw4(const RedParams& p, const RowDst& d, int col, int off = 0) {
  if constexpr (WK == kWF32) {
    return ld4_nt(static_cast<const float*>(d.out) + col + off);
  } else if constexpr (is16(WK)) {
    const uint2 u = ld2_nt(static_cast<const uint16_t*>(d.out) + col + off);
    if constexpr (WK == kWF16)
      return make_float4(f16_widen(u.x & 0xffffu), f16_widen(u.x >> 16), f16_widen(u.y & 0xffffu),
                         f16_widen(u.y >> 16));
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  } else {
    // code c stands for fmaf(c, scale, bias)
    const uint8_t* r = static_cast<const uint8_t*>(d.out);
    const uint32_t c = *reinterpret_cast<const uint32_t*>(r + col + off);
    const float scale = *reinterpret_cast<const float*>(r + d.D);
    const float bias = *reinterpret_cast<const float*>(r + d.D + 4);
    return make_float4(fmaf((float)(c & 0xffu), scale, bias),
                       fmaf((float)((c >> 8) & 0xffu), scale, bias),
                       fmaf((float)((c >> 16) & 0xffu), scale, bias),
                       fmaf((float)(c >> 24), scale, bias));
  }
}

// Stores the row's new values at columns [col, col+4) (col % 4 == 0).
template <int WK>
__device__ __forceinline__ void stw4(const RedParams& p, const RowDst& d, int col, float4 v,
                                     int off = 0) {
  if constexpr (WK == kWINT8) {
    return;  // never reached: INT8 rows are requantized whole (store_codes4)
  } else if constexpr (WK == kWF32) {
    st4_nt(static_cast<float*>(d.out) + col + off, v);
    return;
  } else {
  col += off;
  uint32_t h0, h1, h2, h3;
  if (p.sr) {
    const U4 r = philox4x32_10(
        U4{(uint32_t)col >> 2, (uint32_t)d.lin, (uint32_t)((uint64_t)d.lin >> 32), p.sr_ctr3},
        p.sr_key0, p.sr_key1);
    if constexpr (WK == kWF16) {
      h0 = f16_round(v.x, r.x, true);
      h1 = f16_round(v.y, r.y, true);
      h2 = f16_round(v.z, r.z, true);
      h3 = f16_round(v.w, r.w, true);
    } else {
      h0 = bf16_sr(v.x, r.x);
      h1 = bf16_sr(v.y, r.y);
      h2 = bf16_sr(v.z, r.z);
      h3 = bf16_sr(v.w, r.w);
    }
  } else if constexpr (WK == kWF16) {
    h0 = f16_round(v.x, 0u, false);
    h1 = f16_round(v.y, 0u, false);
    h2 = f16_round(v.z, 0u, false);
    h3 = f16_round(v.w, 0u, false);
  } else {
    h0 = bf16_rne(v.x);
    h1 = bf16_rne(v.y);
    h2 = bf16_rne(v.z);
    h3 = bf16_rne(v.w);
  }
  st2_nt(static_cast<uint16_t*>(d.out) + col, make_uint2(h0 | (h1 << 16), h2 | (h3 << 16)));
  }
}

// ---- INT8 weight rows
//
// The FBGEMM page keeps 8-bit rows with their quantization parameters in the
// row, loads a row with its parameters and, after the update, finds new
// parameters from the updated row before storing it (bodies not printed).
// Here a row is its D codes followed by fp32 scale and bias; code c stands
// for fmaf(c, scale, bias).  After the update (fp64, rounded once to fp32,
// as for fp32 rows) the new bias is the row's minimum, the new scale
// (max - min) / 255, and each code rint((w - bias) / scale) clamped to
// [0, 255] (0 for a constant row), all in fp32 with correctly rounded
// division.  A row is served whole by one lane group, so the minimum and
// maximum are a group reduction.

__device__ __forceinline__ float group_min(float x, int lpl) {
  for (int off = lpl / 2; off > 0; off >>= 1) x = fminf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ float group_max(float x, int lpl) {
  for (int off = lpl / 2; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ void minmax4(const float4& v, float& mn, float& mx) {
  mn = fminf(fminf(mn, v.x), fminf(fminf(v.y, v.z), v.w));
  mx = fmaxf(fmaxf(mx, v.x), fmaxf(fmaxf(v.y, v.z), v.w));
}

__device__ __forceinline__ uint32_t code_of(float w, float scale, float bias) {
  if (!(scale > 0.f)) return 0u;
  const float q = __builtin_rintf(__fdiv_rn(w - bias, scale));
  return (uint32_t)fminf(fmaxf(q, 0.f), 255.f);
}

// Codes of 4 values, packed little-endian (column col + k in byte k).
__device__ __forceinline__ uint32_t codes4(const float4& v, float scale, float bias) {
  return code_of(v.x, scale, bias) | (code_of(v.y, scale, bias) << 8) |
         (code_of(v.z, scale, bias) << 16) | (code_of(v.w, scale, bias) << 24);
}

// New parameters of a row from its lanes' partial minimum and maximum.
__device__ __forceinline__ float2 qparams_of(float mn, float mx, int lpl) {
  mn = group_min(mn, lpl);
  mx = group_max(mx, lpl);
  return make_float2(__fdiv_rn(mx - mn, 255.0f), mn);
}

__device__ __forceinline__ void store_codes4(const RowDst& d, int col, const float4& v, float2 qp) {
  *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(d.out) + col) = codes4(v, qp.x, qp.y);
}

__device__ __forceinline__ void store_qparams(const RowDst& d, float2 qp) {
  uint8_t* r = static_cast<uint8_t*>(d.out);
  *reinterpret_cast<float*>(r + d.D) = qp.x;
  *reinterpret_cast<float*>(r + d.D + 4) = qp.y;
}

// Lane groups of a long-run item: lpl lanes per group (the power of two
// covering D/4, 4..64), 64/lpl groups per wave.  lpl is a wave-uniform
// runtime value, so one code path -- and one register budget -- serves every
// row width.
struct Groups {
  int lpl;         // lanes per group
  int g;           // this lane's group
  int lig;         // this lane's index in its group
  int gb;          // first lane of its group
  uint64_t gmask;  // the lanes of its group
};

__device__ __forceinline__ Groups groups_of(int lpl) {
  const int lane = lane_id();
  Groups q;
  q.lpl = lpl;
  q.lig = lane & (lpl - 1);
  q.gb = lane - q.lig;
  q.g = lane >> __builtin_ctz((unsigned)lpl);
  q.gmask = lpl == 64 ? ~0ull : (((1ull << lpl) - 1ull) << q.gb);
  return q;
}

// One gathered grad_output row of a long run: the element offset of the row
// and the sum of the coefficients of the run's consecutive lookups that read
// it.
struct MergedRow {
  int64_t base;
  double coef;
};

// Sum over lookups j in [first, last) of coef_j * grad row_j at elements
// [colofs, colofs+4), where each lane group passes its own range (uniform
// within the group; the ranges of a wave differ by at most lpl).  Within a
// run the lookups are ordered by bag, so lookups of one bag -- one
// grad_output row -- are adjacent: each slice of lpl lookups is merged into
// (row, summed coefficient) entries first (segmented sum across the lanes,
// fp64), the entries are compacted into the wave's LDS list `q`, and only
// they are gathered, UNR rows per lane at a time: the row offsets are read
// from the list first, then every load of the round is issued before any
// value is used.  The next slice's metadata is loaded while the current one
// is gathered.  Called with the whole wave active.
template <int UNR, bool BF16>
__device__ __forceinline__ d4 gather_merged(const RedParams& p, const Groups& G, int first, int last,
                                            int slices, int t, int64_t colofs, bool col_ok,
                                            MergedRow* q) {
  const int lane = lane_id();
  const int lpl = G.lpl, lig = G.lig, gb = G.gb;
  const uint64_t imask = info_mask(p);
  const bool has_coef = p.coef != nullptr;
  auto clampj = [&](int j) { return j < last ? j : (last > first ? last - 1 : first); };
  d4 acc = d4_zero();
  // metadata of this lane's lookup in slice 0 (loads from a valid index even
  // when there is nothing to read, so no branch holds them up)
  int j = first + lig;
  uint64_t w = p.kv[clampj(j)];
  float c = has_coef ? p.coef[clampj(j)] : 1.0f;
  for (int s = 0; s < slices; ++s) {
    const bool ok = j < last;
    const int jn = j + lpl;
    const uint64_t wn = p.kv[clampj(jn)];
    const float cn = has_coef ? p.coef[clampj(jn)] : 1.0f;
    const int row = ok ? grad_row_of(p, (uint32_t)(w & imask), t) : -1 - lane;
    // segments of equal rows (adjacent lanes of the group) summed into their
    // first lane
    double cs = ok ? (double)c : 0.0;
    const int prow = __shfl_up(row, 1, 64);
    const bool head = ok && (lig == 0 || prow != row);
    for (int off = 1; off < lpl; off <<= 1) {
      const double o = __shfl_down(cs, off, 64);
      const int orow = __shfl_down(row, off, 64);
      if (lig + off < lpl && orow == row) cs += o;
    }
    const uint64_t hm = __ballot(head) & G.gmask;
    const int cnt = __popcll(hm);
    if (head) {
      const int at = __popcll(hm & ((1ull << lane) - 1ull));
      q[gb + at] = MergedRow{(int64_t)row * p.row_stride, cs};
    }
    // (a wave's LDS accesses are performed in order: the list is complete
    // for the reads below)
    for (int jj = 0; jj < cnt; jj += UNR) {
      int64_t eb[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) eb[u] = q[gb + min(jj + u, lpl - 1)].base;
      Raw4<BF16> r[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        r[u] = (jj + u < cnt && col_ok) ? load_raw4<BF16>(p.grad, eb[u] + colofs) : zero_raw4<BF16>();
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const double cf = (jj + u < cnt && col_ok) ? q[gb + min(jj + u, lpl - 1)].coef : 0.0;
        const float4 v = widen4<BF16>(r[u]);
        acc.x = fma(cf, (double)v.x, acc.x);
        acc.y = fma(cf, (double)v.y, acc.y);
        acc.z = fma(cf, (double)v.z, acc.z);
        acc.w = fma(cf, (double)v.w, acc.w);
      }
    }
    j = jn;
    w = wn;
    c = cn;
  }
  return acc;
}

// Adds the lane groups of a wave (fixed xor tree; all groups get the sum).
__device__ __forceinline__ d4 fold_groups(d4 a, int lpl) {
  for (int off = 32; off >= lpl; off >>= 1) d4_add(a, d4_xor(a, off));
  return a;
}

// Sum over the lanes of a group (fixed xor tree).
__device__ __forceinline__ double group_sum(double x, int lpl) {
  for (int off = lpl / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}


// One fp32 result from an fp64 value, rounded once.
__device__ __forceinline__ float4 round4(double x, double y, double z, double w) {
  return make_float4((float)x, (float)y, (float)z, (float)w);
}

// Finishes column blocks [cb_lo, cb_hi) of one row whose gradient for block
// cb is getG(cb) (this lane's 4 columns).  getG is called by the whole wave.
// Row-wise Adagrad: the state grows by the mean square of the row gradient,
// then the step uses the grown state with eps outside the root (FBTT
// `cache_backward_rowwise_adagrad_approx_kernel`), here once per distinct row
// on the summed gradient; a row wider than 256 columns recomputes blocks
// after its mean square is known.  SGD: w -= lr * G (FBTT
// `cache_backward_sgd_kernel`).  Dense: store, or add for an accumulating
// grad_weight (tinygrad `_embedding_bwd_kernel`).  The old row value is read
// before getG so that the read overlaps the gather.
template <int WK, class F>
__device__ __forceinline__ void finish_row(const RedParams& p, const Groups& G, const RowDst& dst,
                                           int D, bool write, int cb_lo, int cb_hi, F&& getG) {
  const int lig = G.lig;
  if constexpr (WK == kWINT8) {
    // the whole row: the step (Adagrad: the mean square over every block
    // first), the new values' range, then the codes
    const int ncb = col_blocks(D);
    const bool adagrad = p.mode == kModeAdagrad;
    const float m0 = (write && adagrad) ? *dst.mom : 0.f;
    double mult = (double)p.lr, m = 0.0;
    if (adagrad) {
      double ss = 0.0;
#pragma unroll 1
      for (int cb = 0; cb < ncb; ++cb) {
        const d4 g = getG(cb);
        if (cb * kColBlock + 4 * lig < D) ss += d4_sumsq(g);
      }
      ss = group_sum(ss, G.lpl);
      m = (double)m0 + ss / (double)D;
      mult = (double)p.lr / (sqrt(m) + (double)p.eps);
    }
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll 1
    for (int cb = 0; cb < ncb; ++cb) {
      const int col = cb * kColBlock + 4 * lig;
      const d4 g = getG(cb);
      if (col < D) {
        const float4 o = write ? ldw4<WK>(p, dst, col) : make_float4(0.f, 0.f, 0.f, 0.f);
        minmax4(round4((double)o.x - g.x * mult, (double)o.y - g.y * mult,
                       (double)o.z - g.z * mult, (double)o.w - g.w * mult), mn, mx);
      }
    }
    const float2 qp = qparams_of(mn, mx, G.lpl);
#pragma unroll 1
    for (int cb = 0; cb < ncb; ++cb) {
      const int col = cb * kColBlock + 4 * lig;
      const d4 g = getG(cb);
      if (write && col < D) {
        const float4 o = ldw4<WK>(p, dst, col);
        store_codes4(dst, col, round4((double)o.x - g.x * mult, (double)o.y - g.y * mult,
                                      (double)o.z - g.z * mult, (double)o.w - g.w * mult), qp);
      }
    }
    if (write && lig == 0) {
      store_qparams(dst, qp);
      if (adagrad) *dst.mom = (float)m;
    }
    return;
  } else {
  if (p.mode == kModeAdagrad) {
    const bool w0ok = write && 4 * lig < D;
    const float4 w0 = w0ok ? ldw4<WK>(p, dst, 4 * lig) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float m0 = write ? *dst.mom : 0.f;
    const int ncb = col_blocks(D);
    const d4 g0 = getG(0);
    double ss = 0.0;
    if (4 * lig < D) ss = d4_sumsq(g0);
#pragma unroll 1
    for (int cb = 1; cb < ncb; ++cb) {
      const d4 g = getG(cb);
      if (cb * kColBlock + 4 * lig < D) ss += d4_sumsq(g);
    }
    ss = group_sum(ss, G.lpl);
    const double m = (double)m0 + ss / (double)D;
    const double mult = (double)p.lr / (sqrt(m) + (double)p.eps);
    if (w0ok)
      stw4<WK>(p, dst, 4 * lig, round4((double)w0.x - g0.x * mult, (double)w0.y - g0.y * mult,
                                    (double)w0.z - g0.z * mult, (double)w0.w - g0.w * mult));
#pragma unroll 1
    for (int cb = 1; cb < ncb; ++cb) {
      const d4 g = getG(cb);
      const int col = cb * kColBlock + 4 * lig;
      if (write && col < D) {
        const float4 wv = ldw4<WK>(p, dst, col);
        stw4<WK>(p, dst, col, round4((double)wv.x - g.x * mult, (double)wv.y - g.y * mult,
                                  (double)wv.z - g.z * mult, (double)wv.w - g.w * mult));
      }
    }
    if (write && lig == 0) *dst.mom = (float)m;
    return;
  }
  const bool needs_old = p.mode == kModeSgd || p.accumulate;
  const double lr = (double)p.lr;
#pragma unroll 1
  for (int cb = cb_lo; cb < cb_hi; ++cb) {
    const int col = cb * kColBlock + 4 * lig;
    const bool ok = write && col < D;
    const float4 old = (ok && needs_old) ? ldw4<WK>(p, dst, col) : make_float4(0.f, 0.f, 0.f, 0.f);
    const d4 g = getG(cb);
    if (!ok) continue;
    float4 wv;
    if (p.mode == kModeSgd)
      wv = round4((double)old.x - lr * g.x, (double)old.y - lr * g.y, (double)old.z - lr * g.z,
                  (double)old.w - lr * g.w);
    else if (p.accumulate)
      wv = round4((double)old.x + g.x, (double)old.y + g.y, (double)old.z + g.z,
                  (double)old.w + g.w);
    else
      wv = round4(g.x, g.y, g.z, g.w);
    stw4<WK>(p, dst, col, wv);
  }
  }
}

// Update of one 256-column block cb of a row whose gradient g (this lane's 4
// columns, fp64) is complete, from the old values `old` (and Adagrad state
// m0) read before g was gathered.  Row-wise Adagrad here covers a row of one
// block; wider rows take finish_row.
template <int WK>
__device__ __forceinline__ void update_block(const RedParams& p, const Groups& G, const RowDst& dst,
                                             int D, bool write, int cb, const float4& old, float m0,
                                             const d4& g) {
  const int lig = G.lig;
  const int col = cb * kColBlock + 4 * lig;
  const bool ok = write && col < D;
  if constexpr (WK == kWINT8) {
    // a row of one block: the step, the range over the group, the codes
    const bool adagrad = p.mode == kModeAdagrad;
    double mult = (double)p.lr, m = 0.0;
    if (adagrad) {
      const double ss = group_sum(col < D ? d4_sumsq(g) : 0.0, G.lpl);
      m = (double)m0 + ss / (double)D;
      mult = (double)p.lr / (sqrt(m) + (double)p.eps);
    }
    const float4 nw = round4((double)old.x - g.x * mult, (double)old.y - g.y * mult,
                             (double)old.z - g.z * mult, (double)old.w - g.w * mult);
    float mn = INFINITY, mx = -INFINITY;
    if (col < D) minmax4(nw, mn, mx);
    const float2 qp = qparams_of(mn, mx, G.lpl);
    if (ok) store_codes4(dst, col, nw, qp);
    if (write && lig == 0) {
      store_qparams(dst, qp);
      if (adagrad) *dst.mom = (float)m;
    }
    return;
  }
  if (p.mode == kModeAdagrad) {
    const double ss = group_sum(col < D ? d4_sumsq(g) : 0.0, G.lpl);
    const double m = (double)m0 + ss / (double)D;
    const double mult = (double)p.lr / (sqrt(m) + (double)p.eps);
    if (ok)
      stw4<WK>(p, dst, col, round4((double)old.x - g.x * mult, (double)old.y - g.y * mult,
                                (double)old.z - g.z * mult, (double)old.w - g.w * mult));
    if (write && lig == 0) *dst.mom = (float)m;
    return;
  }
  if (!ok) return;
  float4 wv;
  if (p.mode == kModeSgd) {
    const double lr = (double)p.lr;
    wv = round4((double)old.x - lr * g.x, (double)old.y - lr * g.y, (double)old.z - lr * g.z,
                (double)old.w - lr * g.w);
  } else if (p.accumulate) {
    wv = round4((double)old.x + g.x, (double)old.y + g.y, (double)old.z + g.z, (double)old.w + g.w);
  } else {
    wv = round4(g.x, g.y, g.z, g.w);
  }
  stw4<WK>(p, dst, col, wv);
}
// Partials travel between waves on different XCDs.  They are written and read
// with device-scope (agent) atomic accesses, which the hardware keeps coherent
// across the XCDs' L2 caches by themselves; an agent-scope release/acquire
// fence pair would instead write back and invalidate a whole L2 per ticket,
// which measured as most of the long-run kernel's time.
__device__ __forceinline__ void store_partial(double* q, const d4& v) {
  uint64_t* u = reinterpret_cast<uint64_t*>(q);
  __hip_atomic_store(u, (uint64_t)__double_as_longlong(v.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(u + 1, (uint64_t)__double_as_longlong(v.y), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(u + 2, (uint64_t)__double_as_longlong(v.z), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(u + 3, (uint64_t)__double_as_longlong(v.w), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ d4 load_partial(const double* q) {
  uint64_t* u = reinterpret_cast<uint64_t*>(const_cast<double*>(q));
  d4 r;
  r.x = __longlong_as_double((long long)__hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  r.y = __longlong_as_double(
      (long long)__hip_atomic_load(u + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  r.z = __longlong_as_double(
      (long long)__hip_atomic_load(u + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  r.w = __longlong_as_double(
      (long long)__hip_atomic_load(u + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return r;
}

// Last-arrival ticket: waits until this wave's partial stores have completed
// (s_waitcnt vmcnt(0): on this architecture the vector-memory counter also
// covers stores, and agent-scope atomic stores complete at the level where
// every XCD sees them), counts the arrival with a device-scope atomic, and
// reports whether this wave completes the group.  The caller reads the
// members' partials only after this returns true, i.e. after the atomic's
// result came back, with device-scope loads.  The signal fences keep the
// compiler from moving the partial stores below the wait or the partial
// loads above the ticket (they emit no instruction).
__device__ __forceinline__ bool ticket_last(uint32_t* ctr, uint32_t members) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t old = 0;
  if (lane_id() == 0)
    old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, 64);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return old + 1 == members;
}

// Partial slot of chunk c, column block cb, of a long run whose items start
// at slot `cbeg`: kColBlock fp64 values each, chunk-major.
__device__ __forceinline__ double* slot_of(const RedParams& p, uint32_t cbeg, int c, int ncb,
                                           int cb) {
  return p.partials + ((int64_t)cbeg + (int64_t)c * ncb + cb) * kColBlock;
}


// Sum of the partials of chunks first, first+stride, ... (count of them) for
// column block cb, groups interleaved, each group adding its partials in
// order and the groups folded by a fixed tree.  Four partials per lane are in
// flight at a time.
__device__ __forceinline__ d4 sum_slots(const RedParams& p, const Groups& G, uint32_t cbeg, int ncb,
                                        int first, int count, int stride, int cb, int D) {
  const int ng = 64 / G.lpl;
  const int col = 4 * G.lig;
  d4 acc = d4_zero();
  if (cb * kColBlock + col < D) {
    int i = G.g;
    for (; i + 3 * ng < count; i += 4 * ng) {
      const d4 a0 = load_partial(slot_of(p, cbeg, first + i * stride, ncb, cb) + col);
      const d4 a1 = load_partial(slot_of(p, cbeg, first + (i + ng) * stride, ncb, cb) + col);
      const d4 a2 = load_partial(slot_of(p, cbeg, first + (i + 2 * ng) * stride, ncb, cb) + col);
      const d4 a3 = load_partial(slot_of(p, cbeg, first + (i + 3 * ng) * stride, ncb, cb) + col);
      d4_add(acc, a0);
      d4_add(acc, a1);
      d4_add(acc, a2);
      d4_add(acc, a3);
    }
    for (; i < count; i += ng) d4_add(acc, load_partial(slot_of(p, cbeg, first + i * stride, ncb, cb) + col));
  }
  return fold_groups(acc, G.lpl);
}

// The output row of a long run.
template <int WK>
__device__ __forceinline__ RowDst long_row(const RedParams& p, const LongRun& rec) {
  RowDst d;
  if constexpr (WK == kWINT8)
    d.out = p.out_q + p.woff8[rec.t] + (rec.mom - p.hsc[rec.t]) * (int64_t)(rec.D + 8);
  else if constexpr (is16(WK))
    d.out = p.out_h + rec.out;
  else
    d.out = p.out + rec.out;
  d.mom = p.mom ? p.mom + rec.mom : nullptr;
  d.lin = rec.mom;
  d.D = rec.D;
  return d;
}

template <bool BF16, int WK>
__device__ __forceinline__ void long_item(const RedParams& p, const LongRun& rec, int c, int cb) {
  const int t = rec.t, start = rec.start, len = rec.len, D = rec.D;
  const Groups G = groups_of(lanes_per_row(D));
  const int ng = 64 / G.lpl, g = G.g, lig = G.lig;
  const int ncb = rec.ncb;
  const int chl = chunk_len(len, D, p.chunk_base);
  const int nch = rec.nch;
  const int lo = start + c * chl;
  const int hi = min(lo + chl, start + len);
  // Adagrad needs the whole row in one wave: item cb 0 covers every block
  const bool adagrad = p.mode == kModeAdagrad;
  const bool whole = adagrad || WK == kWINT8;  // INT8 rows are requantized whole
  const int cb_lo = whole ? 0 : cb;
  const int cb_hi = whole ? ncb : cb + 1;
  const int64_t gcol = rec.gcol;
  const RowDst dst = long_row<WK>(p, rec);
  // each lane group takes a contiguous share of the chunk, so that the
  // adjacent lookups of one bag stay together for merging
  const int per = (hi - lo + ng - 1) / ng;
  const int glo = min(lo + g * per, hi), ghi = min(glo + per, hi);
  const int slices = (per + G.lpl - 1) / G.lpl;
  __shared__ MergedRow s_rows[4][64];
  MergedRow* q = s_rows[threadIdx.x >> 6];
  // The only chunk of a row that needs nothing beyond this item (Adagrad: a
  // row of one block) updates the row itself; otherwise each block's sum is
  // this item's partial.  One gather site keeps the register budget that of
  // a single gather loop.
  const bool direct = nch == 1 && (!whole || ncb == 1);
  const bool needs_old = p.mode != kModeDense || p.accumulate;
  const uint32_t cbeg = rec.cbeg;
#pragma unroll 1
  for (int cbx = cb_lo; cbx < cb_hi; ++cbx) {
    const int col = cbx * kColBlock + 4 * lig;
    const bool col_ok = col < D;
    // the old row (and state) is read before the gather so the two overlap
    const bool rd = direct && g == 0 && col_ok && needs_old;
    const float4 old = rd ? ldw4<WK>(p, dst, col) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float mom0 = (direct && adagrad && g == 0) ? *dst.mom : 0.f;
    const d4 a = fold_groups(
        gather_merged<SGB_LONG_UNR, BF16>(p, G, glo, ghi, slices, t, gcol + col, col_ok, q), G.lpl);
    if (direct)
      update_block<WK>(p, G, dst, D, g == 0, cbx, old, mom0, a);
    else if (g == 0 && col_ok)
      store_partial(slot_of(p, cbeg, c, ncb, cbx) + 4 * lig, a);
  }
  if (direct) return;
  const int m0 = (c / kSuperChunk) * kSuperChunk;
  const int members = min(kSuperChunk, nch - m0);
  if (!ticket_last(p.sc_ticket + cbeg + (int64_t)m0 * ncb + cb_lo, (uint32_t)members)) return;
  const int nsc = (nch + kSuperChunk - 1) / kSuperChunk;
  if (nsc == 1) {
    finish_row<WK>(p, G, dst, D, g == 0, cb_lo, cb_hi, [&](int cbx) {
      return sum_slots(p, G, cbeg, ncb, 0, nch, 1, cbx, D);
    });
    return;
  }
#pragma unroll 1
  for (int cbx = cb_lo; cbx < cb_hi; ++cbx) {
    const d4 a = sum_slots(p, G, cbeg, ncb, m0, members, 1, cbx, D);
    if (g == 0 && cbx * kColBlock + 4 * lig < D)
      store_partial(slot_of(p, cbeg, m0, ncb, cbx) + 4 * lig, a);
  }
  if (!ticket_last(p.run_ticket + cbeg + cb_lo, (uint32_t)nsc)) return;
  finish_row<WK>(p, G, dst, D, g == 0, cb_lo, cb_hi, [&](int cbx) {
    return sum_slots(p, G, cbeg, ncb, 0, nsc, kSuperChunk, cbx, D);
  });
}

// Index k of the long run holding work item w: chunk_begin[k] <= w <
// chunk_begin[k+1].  A 64-way search: every lane probes one point of the
// interval, so each round shrinks it 64-fold (2 rounds for 4096 runs).
__device__ __forceinline__ int find_long_run(const uint32_t* cbeg, int nlong, uint32_t w) {
  const int lane = lane_id();
  int lo = 0, hi = nlong;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int probe = lo + lane * step;
    const bool le = probe < hi && cbeg[probe] <= w;
    const uint64_t m = __ballot(le);
    const int last = 63 - __builtin_clzll(m);  // lane 0 always qualifies
    lo = lo + last * step;
    hi = min(lo + step, hi);
  }
  return __builtin_amdgcn_readfirstlane(lo);
}

// A wave-uniform copy of a long-run record (its fields steer the wave's
// control flow).
__device__ __forceinline__ int32_t uni32(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ LongRun uniform_rec(const LongRun& r) {
  LongRun u;
  u.start = uni32(r.start);
  u.len = uni32(r.len);
  u.t = uni32(r.t);
  u.ncb = uni32(r.ncb);
  u.cbeg = (uint32_t)uni32((int32_t)r.cbeg);
  u.nch = uni32(r.nch);
  u.id = uni64(r.id);
  u.D = uni32(r.D);
  u.gcol = uni32(r.gcol);
  u.out = uni64(r.out);
  u.mom = uni64(r.mom);
  return u;
}

template <bool BF16, int WK>
__global__ __launch_bounds__(256) void k_reduce_long(RedParams p) {
  if (!runs_match(p)) return;
  const uint32_t n_items = *p.total_items;
  const int nlong = (int)*p.num_long;
  // items are dealt round-robin: consecutive chunks of a hot run go to
  // different waves, tables of different row widths mix on every wave, and no
  // shared counter is contended
  const uint32_t nw = gridDim.x * (blockDim.x / 64);
  for (uint32_t w = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); w < n_items; w += nw) {
    const int k = find_long_run(p.chunk_begin, nlong, w);
    const LongRun rec = uniform_rec(p.long_recs[k]);
    const int local = (int)(w - rec.cbeg);
    const int c = local / rec.ncb, cb = local % rec.ncb;
    if ((p.mode == kModeAdagrad || WK == kWINT8) && cb != 0) continue;
    long_item<BF16, WK>(p, rec, c, cb);
  }
}

// Short runs, CPL columns per lane (8; rows wider than 512 go to
// k_reduce_wide): lane groups of lpl lanes, lpl = the power of two covering D / CPL, at most one
// wave.  The group width is a runtime value so that one code path (and one
// register budget) serves every row width.
template <int CPL>
__device__ __forceinline__ int short_lpl(int D) {
  const int need = (D + CPL - 1) / CPL;
  int l = 1;
  while (l < need && l < 64) l <<= 1;
  return l;
}

// One batch of short runs of table t, CPL columns per lane in pieces of 4
// striped across a lane group of lpl lanes (piece i at column
// col + 4 * lpl * i), in the CPL*64-column block cb.  With k runs in the
// batch (the set bits of `sel`, window lanes holding run heads) and 64 / lpl
// groups, each run gets the largest power-of-two number of groups that fits:
// its groups take interleaved slices of lpl lookups and are folded by a fixed
// xor tree, and the first of them writes the row.  Called with the whole wave
// active.  The row's old value and Adagrad state are loaded together with the
// first gather round.
template <int CPL, bool BF16, int WK>
__device__ __forceinline__ void short_batch(const RedParams& p, uint64_t sel, int lpl, int64_t base,
                                            int len, uint64_t key, int rowi, float cf, int t,
                                            const TabMeta& tm, int cb) {
  const int D = tm.D;
  constexpr int NP = CPL / 4;
  const int lg = __builtin_ctz(lpl);
  const int lane = lane_id(), g = lane >> lg, lig = lane & (lpl - 1), gb = g << lg;
  const int ng = 64 >> lg;
  const int k = __popcll(sel);
  int glg = 0;  // log2 of the groups per run
  while ((k << (glg + 1)) <= ng) ++glg;
  const int rg = g >> glg, q = g & ((1 << glg) - 1);
  uint64_t m = sel;
  for (int i = 0; i < rg; ++i) m &= m - 1;
  const bool active = m != 0;
  const bool lead = active && q == 0;
  const int src = active ? __builtin_ctzll(m) : 0;
  // every shuffle here runs with the whole wave active: a masked-off source
  // lane would read as 0
  const int nn = __shfl(len, src, 64);
  const uint64_t id = __shfl(key, src, 64);
  const int wl = src + (q << lg) + lig;  // window lane of this lane's first lookup
  const int prow = __shfl(rowi, wl < 64 ? wl : 63, 64);
  const float pcf = __shfl(cf, wl < 64 ? wl : 63, 64);
  const int n = active ? nn : 0;
  const int s = (int)base + src;
  const int col = cb * 64 * CPL + 4 * lig;
  int vmask = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i)
    if (active && col + 4 * lpl * i < D) vmask |= 1 << i;
  const int wmask = lead ? vmask : 0;
  RowDst dst{nullptr, nullptr, 0, 0};
  if (lead) dst = row_dest<WK>(p, tm, (int64_t)id);
  const bool needs_old = p.mode != kModeDense || p.accumulate;
  const int64_t gcol = (p.nobag ? 0 : tm.dcol) + col;
  const uint64_t imask = info_mask(p);
  const bool has_coef = p.coef != nullptr;
  d4 acc[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) acc[i] = d4_zero();
  // one round: the group's lookups jj .. jj + UNR - 1 of its current slice
  // (lane gb + j holds lookup j's grad_output row and coefficient)
  auto gather = [&](Raw4<BF16> (&r)[SGB_SHORT_UNR][NP], float (&c)[SGB_SHORT_UNR], int ri, float ci,
                    int jj, int cnt) {
    // every shuffle first (unconditional), then the loads: no wait for a
    // coefficient sits between two of the round's gathers
    int ro[SGB_SHORT_UNR];
#pragma unroll
    for (int u = 0; u < SGB_SHORT_UNR; ++u) {
      const int srcl = gb + min(jj + u, lpl - 1);
      ro[u] = __shfl(ri, srcl, 64);
      c[u] = __shfl(ci, srcl, 64);
    }
#pragma unroll
    for (int u = 0; u < SGB_SHORT_UNR; ++u) {
      const bool ok = jj + u < cnt;
      c[u] = ok ? c[u] : 0.f;
      const int64_t e = (int64_t)ro[u] * p.row_stride + gcol;
#pragma unroll
      for (int i = 0; i < NP; ++i)
        r[u][i] = (ok && ((vmask >> i) & 1)) ? load_raw4<BF16>(p.grad, e + 4 * lpl * i)
                                             : zero_raw4<BF16>();
    }
  };
  // the round's few products are summed in fp32, the run's sum in fp64
  auto accumulate = [&](const Raw4<BF16> (&r)[SGB_SHORT_UNR][NP], const float (&c)[SGB_SHORT_UNR]) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < SGB_SHORT_UNR; ++u) {
        const float4 v = widen4<BF16>(r[u][i]);
        t.x = fmaf(c[u], v.x, t.x);
        t.y = fmaf(c[u], v.y, t.y);
        t.z = fmaf(c[u], v.z, t.z);
        t.w = fmaf(c[u], v.w, t.w);
      }
      d4_add(acc[i], d4{(double)t.x, (double)t.y, (double)t.z, (double)t.w});
    }
  };
  // The group takes slices of lpl lookups of its run, every (1 << glg)-th
  // one.  The first round of its first slice (whose metadata comes from the
  // window when it lies inside it) is loaded together with the old row and
  // its Adagrad state, with nothing waited for in between: a run of at most
  // SGB_SHORT_UNR lookups costs one memory round trip.
  const int j0f = s + (q << lg);
  int ri = 0;
  float ci = 0.f;
  if (wl < 64) {
    ri = prow;
    ci = pcf;
  } else if (j0f + lig < s + n) {
    ri = grad_row_of(p, (uint32_t)(p.kv[j0f + lig] & imask), t);
    ci = has_coef ? p.coef[j0f + lig] : 1.0f;
  }
  const int cnt0 = min(lpl, s + n - j0f);  // <= 0 for a group with nothing to gather
  Raw4<BF16> r[SGB_SHORT_UNR][NP];
  float c[SGB_SHORT_UNR];
  gather(r, c, ri, ci, 0, cnt0);
  float4 old[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i)
    old[i] = (needs_old && ((wmask >> i) & 1)) ? ldw4<WK>(p, dst, col, 4 * lpl * i)
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
  // every lane loads (the others the first state word), so that the load sits
  // outside a branch and nothing waits for it before the sums need it
  const float m0 = p.mode == kModeAdagrad ? *(lead ? dst.mom : p.mom) : 0.f;
  accumulate(r, c);
  for (int jj = SGB_SHORT_UNR; jj < cnt0; jj += SGB_SHORT_UNR) {
    gather(r, c, ri, ci, jj, cnt0);
    accumulate(r, c);
  }
  for (int j0 = j0f + (lpl << glg); j0 < s + n; j0 += lpl << glg) {
    const int jm = j0 + lig;
    ri = 0;
    ci = 0.f;
    if (jm < s + n) {
      ri = grad_row_of(p, (uint32_t)(p.kv[jm] & imask), t);
      ci = has_coef ? p.coef[jm] : 1.0f;
    }
    const int cnt = min(lpl, s + n - j0);
    for (int jj = 0; jj < cnt; jj += SGB_SHORT_UNR) {
      gather(r, c, ri, ci, jj, cnt);
      accumulate(r, c);
    }
  }
  // fold the groups of each run (uniform trip count: the whole wave takes part)
  for (int off = lpl; off < (lpl << glg); off <<= 1) {
#pragma unroll
    for (int i = 0; i < NP; ++i) d4_add(acc[i], d4_xor(acc[i], off));
  }
  if constexpr (WK == kWINT8) {
    // the whole row sits in this lane group: step, range, codes
    double mult = (double)p.lr, mm = 0.0;
    if (p.mode == kModeAdagrad) {
      double ss = 0.0;
#pragma unroll
      for (int i = 0; i < NP; ++i)
        if ((vmask >> i) & 1) ss += d4_sumsq(acc[i]);
      for (int off = lpl >> 1; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
      mm = (double)m0 + ss / (double)D;
      mult = (double)p.lr / (sqrt(mm) + (double)p.eps);
    }
    float4 nw[NP];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      nw[i] = round4((double)old[i].x - acc[i].x * mult, (double)old[i].y - acc[i].y * mult,
                     (double)old[i].z - acc[i].z * mult, (double)old[i].w - acc[i].w * mult);
      if ((vmask >> i) & 1) minmax4(nw[i], mn, mx);
    }
    const float2 qp = qparams_of(mn, mx, lpl);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if ((wmask >> i) & 1) store_codes4(dst, col + 4 * lpl * i, nw[i], qp);
    if (lead && lig == 0) {
      store_qparams(dst, qp);
      if (p.mode == kModeAdagrad) *dst.mom = (float)mm;
    }
    return;
  }
  if (p.mode == kModeAdagrad) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if ((vmask >> i) & 1) ss += d4_sumsq(acc[i]);
    for (int off = lpl >> 1; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const double mm = (double)m0 + ss / (double)D;
    const double mult = (double)p.lr / (sqrt(mm) + (double)p.eps);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if ((wmask >> i) & 1)
        stw4<WK>(p, dst, col,
            round4((double)old[i].x - acc[i].x * mult, (double)old[i].y - acc[i].y * mult,
                   (double)old[i].z - acc[i].z * mult, (double)old[i].w - acc[i].w * mult),
            4 * lpl * i);
    if (lead && lig == 0) *dst.mom = (float)mm;
    return;
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (!((wmask >> i) & 1)) continue;
    const d4& a = acc[i];
    const double lr = (double)p.lr;
    float4 w;
    if (p.mode == kModeSgd)
      w = round4((double)old[i].x - lr * a.x, (double)old[i].y - lr * a.y,
                 (double)old[i].z - lr * a.z, (double)old[i].w - lr * a.w);
    else if (p.accumulate)
      w = round4((double)old[i].x + a.x, (double)old[i].y + a.y, (double)old[i].z + a.z,
                 (double)old[i].w + a.w);
    else
      w = round4(a.x, a.y, a.z, a.w);
    stw4<WK>(p, dst, col, w, 4 * lpl * i);
  }
}

// Windows of 64 sorted positions, each shared by 2^sub_log waves.  Run heads
// are where the id changes; a run's length is the distance to the next head
// in the window, and only a run that reaches the window's end needs more: its
// run index at the head and the run starts, or, with p.scan_runs, the sorted
// words after the window, read 64 at a time (the first 64 with the window's
// own) until a different id shows where the run ends or thr positions past
// its head are passed.  The scan makes the reducer independent of run-length
// encoding, so that it can start as soon as the ids are sorted.  A wave
// serves the short runs (length < thr) that start in its 64 >> sub_log
// positions, in batches of at most 64/lpl runs of one table.  Rows wider than
// 512 columns are skipped here (k_reduce_wide serves them).
template <int CPL, bool BF16, int WK>
__device__ __forceinline__ void reduce_short(const RedParams& p) {
  const int lane = lane_id();
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int cb = blockIdx.y;
  const int64_t base = (unit >> p.sub_log) * kShortSpan;
  const int part = (int)(unit & ((1 << p.sub_log) - 1));
  if (base >= p.N) return;
  const uint64_t imask = info_mask(p);
  const int64_t pos = base + lane;
  const bool in = pos < p.N;
  const uint64_t kv = in ? p.kv[pos] : 0ull;
  const bool in_next = p.scan_runs && pos + 64 < p.N;
  const uint64_t key_next = in_next ? (p.kv[pos + 64] >> p.info_bits) : 0ull;
  const uint64_t key = kv >> p.info_bits;
  uint64_t prev = __shfl_up(key, 1, 64);
  if (lane == 0) prev = base > 0 ? (p.kv[base - 1] >> p.info_bits) : ~0ull;
  const bool head = in && (pos == 0 || key != prev);
  const uint64_t heads = __ballot(head);
  if (heads == 0) return;
  const uint32_t info = (uint32_t)(kv & imask);
  const int t = in ? table_of(p, info) : 0;
  const int rowi = in ? grad_row_of(p, info, t) : 0;
  const float cf = (in && p.coef) ? p.coef[pos] : 1.0f;
  // length to the next head in the window; the run of the last head may go on
  const uint64_t after = lane < 63 ? (heads & (~0ull << (lane + 1))) : 0ull;
  int last_len = 0;  // with p.scan_runs: the length of the last head's run, or >= thr
  if (p.scan_runs) {
    const int hl = 63 - __builtin_clzll(heads);
    const int64_t hpos = base + hl;
    const int vl = (int)min((int64_t)63, p.N - 1 - base);   // the window's last position
    const uint64_t klast = __shfl(key, vl, 64);               // the last run's id
    int64_t end = -1;
    if (base + 64 >= p.N) {
      end = p.N;
    } else {
      const uint64_t m = __ballot(in_next && key_next != klast);
      if (m) end = base + 64 + __builtin_ctzll(m);
      else if (base + 128 >= p.N) end = p.N;
    }
    // (rare) the run goes on past the next window: further words, until its
    // end or until it is known to be long
    for (int64_t b2 = base + 128; end < 0 && b2 < hpos + p.thr; b2 += 64) {
      const int64_t q = b2 + lane;
      const bool v = q < p.N;
      const uint64_t k2 = v ? (p.kv[q] >> p.info_bits) : 0ull;
      const uint64_t m = __ballot(v && k2 != klast);
      if (m) end = b2 + __builtin_ctzll(m);
      else if (b2 + 64 >= p.N) end = p.N;
    }
    last_len = end < 0 ? p.thr : (int)min(end - hpos, (int64_t)p.thr);
  }
  int len = 0;
  if (head) {
    if (after) {
      len = __builtin_ctzll(after) - lane;
    } else if (p.scan_runs) {
      len = last_len;
    } else {
      const int r = p.head_run[pos];
      len = p.cum[r + 1] - (int)pos;
    }
  }
  const bool todo = head && len < p.thr && (lane >> (6 - p.sub_log)) == part;
  uint64_t pending = __ballot(todo);
  while (pending) {
    const int lead = __builtin_ctzll(pending);
    const int t0 = __builtin_amdgcn_readfirstlane(__shfl(t, lead, 64));
    const uint64_t same = __ballot(todo && t == t0) & pending;
    const TabMeta tm = tab_meta<WK>(p, t0);
    const int D = tm.D;
    const int lpl = short_lpl<CPL>(D);
    uint64_t sel = 0, rest = same;
    for (int i = 0; i < 64 / lpl && rest; ++i) {
      const uint64_t low = rest & (~rest + 1ull);
      sel |= low;
      rest ^= low;
    }
    pending &= ~sel;
    if (D > 512 || cb * 64 * CPL >= D) continue;  // wider rows: k_reduce_wide
    short_batch<CPL, BF16, WK>(p, sel, lpl, base, len, key, rowi, cf, t0, tm, cb);
  }
}

// 8 columns per lane with fp64 sums fits about 80 VGPRs: 6 waves per SIMD overlap
// the runs' dependent memory steps.  The 16-bit and INT8 row instances are
// held to the same budget: the bf16 and fp16 ones spill a few registers,
// which costs less than a wave less per SIMD.
template <bool BF16, int WK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SGB_SHORT8_WAVES,
                                                                     SGB_SHORT8_WAVES)))
void k_reduce_short8(RedParams p) {
  if (!runs_match(p)) return;
  reduce_short<8, BF16, WK>(p);
}


// ------------------------------------------------------------ k_reduce_wide
//
// Short runs of rows wider than 512 columns.  The row update of such a run
// (read and write of the old row, 8 bytes per column) outweighs the gather of
// its few lookups, and a wave that served every run of a 64-position window
// in turn paid two memory round trips per run.  Here the work is dealt by
// run: items (run, column block of 64*CPL columns) go round-robin to the
// waves, the whole wave serves one item (each lane CPL columns, pieces of 4
// columns 256 apart), and before a wave gathers its current item it has
// issued the loads of the next item's first sorted words and of the run
// starts of the item after that, so an item costs about one round trip.
// Items differ in cost (runs of 1 to thr - 1 lookups), so the grid holds
// several times the workgroups that fit at once: a wave takes few items, and
// the hardware starts new waves where short items finished, instead of
// leaving a fixed set of waves to wait for the one that drew a long run.
// Lookups are gathered UNR at a time from wave-uniform row offsets (readlane),
// accumulated with fp64 FMAs.  Runs of length >= thr belong to the long-run
// reducer, rows of 512 columns or fewer to k_reduce_short8.

// Start and end of the run of an item (end = next run's start; zero length
// past the last item).
struct WideRun {
  int s, e;
};

__device__ __forceinline__ WideRun wide_run(const RedParams& p, int64_t item, int64_t items,
                                            int ncb) {
  WideRun m{0, 0};
  if (item < items) {
    const int r = (int)(item / ncb);
    m.s = p.cum[r];  // the same word in every lane: made wave-uniform where used
    m.e = p.cum[r + 1];
  }
  return m;
}

// This lane's sorted word and coefficient of lookup s + j0 + lane of a run.
struct WideLane {
  uint64_t kv;
  float cf;
};

__device__ __forceinline__ WideLane wide_lane(const RedParams& p, const WideRun& m, int j0) {
  const int j = uni32(m.s) + j0 + lane_id();
  WideLane d{0ull, 1.0f};
  if (j < uni32(m.e)) {
    d.kv = p.kv[j];
    if (p.coef) d.cf = p.coef[j];
  }
  return d;
}

__device__ __forceinline__ int rl32(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float rlf(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ uint64_t rl64(uint64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int32_t)(x >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// A short run of a row-wise Adagrad or INT8 row wider than one item holds
// (1024 columns): the whole wave serves the run, and finish_row takes the
// row's 256-column blocks from a gather of the run's lookups, repeated on
// each of its passes (mean square, then the update; INT8 rows also their
// range), so nothing beyond 4 columns per lane is held at a time.
template <bool BF16, int WK>
__device__ __forceinline__ void wide_run_multi(const RedParams& p, const WideRun& m,
                                            const WideLane& d0, int t, const TabMeta& tm,
                                            int64_t lin) {
  constexpr int UNR = 4;
  const int D = tm.D;
  const Groups G = groups_of(64);
  const RowDst dst = row_dest<WK>(p, tm, lin);
  const uint64_t imask = info_mask(p);
  const int len = m.e - m.s;
  const int64_t gbase = p.nobag ? 0 : tm.dcol;
  auto getG = [&](int cb) -> d4 {
    const int col = cb * kColBlock + 4 * lane_id();
    const bool ok = col < D;
    const int64_t gcol = gbase + col;
    d4 acc = d4_zero();
    for (int j0 = 0; j0 < len; j0 += 64) {
      const WideLane dl = j0 == 0 ? d0 : wide_lane(p, m, j0);
      const int rowi = grad_row_of(p, (uint32_t)(dl.kv & imask), t);
      const int cnt = min(64, len - j0);
      for (int u0 = 0; u0 < cnt; u0 += UNR) {
        Raw4<BF16> r[UNR];
        float c[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const bool in = u0 + u < cnt;
          const int src = in ? u0 + u : cnt - 1;
          c[u] = in ? rlf(dl.cf, src) : 0.f;
          r[u] = (in && ok) ? load_raw4<BF16>(p.grad, (int64_t)rl32(rowi, src) * p.row_stride + gcol)
                            : zero_raw4<BF16>();
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) d4_fma(acc, c[u], widen4<BF16>(r[u]));
      }
    }
    return acc;
  };
  finish_row<WK>(p, G, dst, D, true, 0, col_blocks(D), getG);
}

template <int CPL, int UNR, bool BF16, int WK>
__device__ __forceinline__ void wide_item(const RedParams& p, const WideRun& m,
                                          const WideLane& d0, int cb) {
  constexpr int NP = CPL / 4;
  const int len = uni32(m.e) - uni32(m.s);
  if (len <= 0 || len >= p.thr) return;
  const uint64_t imask = info_mask(p);
  const uint64_t kv0 = rl64(d0.kv, 0);
  const int t = uni32(table_of(p, (uint32_t)(kv0 & imask)));
  const TabMeta tm = tab_meta<WK>(p, t);
  const int D = tm.D;
  // whole rows wider than one item are served by k_reduce_wide_multi
  if ((p.mode == kModeAdagrad || WK == kWINT8) && D > 64 * CPL) return;
  if (D <= 512 || cb * 64 * CPL >= D) return;
  const int col = cb * 64 * CPL + 4 * lane_id();
  int vmask = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i)
    if (col + 256 * i < D) vmask |= 1 << i;
  const RowDst dst = row_dest<WK>(p, tm, (int64_t)(kv0 >> p.info_bits));
  const bool needs_old = p.mode != kModeDense || p.accumulate;
  float4 old[NP];
  d4 acc[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    old[i] = (needs_old && ((vmask >> i) & 1)) ? ldw4<WK>(p, dst, col, 256 * i)
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
    acc[i] = d4_zero();
  }
  // (outside a branch: the state is waited for only where the sums need it;
  // without Adagrad state the first sorted word stands in)
  const float mv0 = *(p.mode == kModeAdagrad ? dst.mom : reinterpret_cast<const float*>(p.kv));
  const float m0 = p.mode == kModeAdagrad ? mv0 : 0.f;
  const int64_t gcol = (p.nobag ? 0 : tm.dcol) + col;
  for (int j0 = 0; j0 < len; j0 += 64) {
    const WideLane dl = j0 == 0 ? d0 : wide_lane(p, m, j0);
    const int rowi = grad_row_of(p, (uint32_t)(dl.kv & imask), t);
    const int cnt = min(64, len - j0);
    for (int u0 = 0; u0 < cnt; u0 += UNR) {
      Raw4<BF16> r[UNR][NP];
      float c[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const bool ok = u0 + u < cnt;
        const int src = ok ? u0 + u : cnt - 1;
        const int64_t e = (int64_t)rl32(rowi, src) * p.row_stride + gcol;
        c[u] = ok ? rlf(dl.cf, src) : 0.f;
#pragma unroll
        for (int i = 0; i < NP; ++i)
          r[u][i] = (ok && ((vmask >> i) & 1)) ? load_raw4<BF16>(p.grad, e + 256 * i)
                                               : zero_raw4<BF16>();
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int i = 0; i < NP; ++i) d4_fma(acc[i], c[u], widen4<BF16>(r[u][i]));
    }
  }
  if constexpr (WK == kWINT8) {
    // one item holds the whole row (up to 1024 columns)
    double mult = (double)p.lr, mm = 0.0;
    if (p.mode == kModeAdagrad) {
      double ss = 0.0;
#pragma unroll
      for (int i = 0; i < NP; ++i)
        if ((vmask >> i) & 1) ss += d4_sumsq(acc[i]);
      ss = group_sum(ss, 64);
      mm = (double)m0 + ss / (double)D;
      mult = (double)p.lr / (sqrt(mm) + (double)p.eps);
    }
    float4 nw[NP];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      nw[i] = round4((double)old[i].x - acc[i].x * mult, (double)old[i].y - acc[i].y * mult,
                     (double)old[i].z - acc[i].z * mult, (double)old[i].w - acc[i].w * mult);
      if ((vmask >> i) & 1) minmax4(nw[i], mn, mx);
    }
    const float2 qp = qparams_of(mn, mx, 64);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if ((vmask >> i) & 1) store_codes4(dst, col + 256 * i, nw[i], qp);
    if (lane_id() == 0) {
      store_qparams(dst, qp);
      if (p.mode == kModeAdagrad) *dst.mom = (float)mm;
    }
    return;
  }
  if (p.mode == kModeAdagrad) {
    // one item holds the whole row (up to 1024 columns)
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if ((vmask >> i) & 1) ss += d4_sumsq(acc[i]);
    ss = group_sum(ss, 64);
    const double mm = (double)m0 + ss / (double)D;
    const double mult = (double)p.lr / (sqrt(mm) + (double)p.eps);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if ((vmask >> i) & 1)
        stw4<WK>(p, dst, col,
            round4((double)old[i].x - acc[i].x * mult, (double)old[i].y - acc[i].y * mult,
                   (double)old[i].z - acc[i].z * mult, (double)old[i].w - acc[i].w * mult),
            256 * i);
    if (lane_id() == 0) *dst.mom = (float)mm;
    return;
  }
  const double lr = (double)p.lr;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (!((vmask >> i) & 1)) continue;
    const d4& a = acc[i];
    float4 w;
    if (p.mode == kModeSgd)
      w = round4((double)old[i].x - lr * a.x, (double)old[i].y - lr * a.y,
                 (double)old[i].z - lr * a.z, (double)old[i].w - lr * a.w);
    else if (p.accumulate)
      w = round4((double)old[i].x + a.x, (double)old[i].y + a.y, (double)old[i].z + a.z,
                 (double)old[i].w + a.w);
    else
      w = round4(a.x, a.y, a.z, a.w);
    stw4<WK>(p, dst, col, w, 256 * i);
  }
}

template <int CPL, int UNR, bool BF16, int WK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, SGB_WIDE_WAVES)))
void k_reduce_wide(RedParams p) {
  if (!runs_match(p)) return;
  const int64_t nw = (int64_t)gridDim.x * 4;
  int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ncb = p.wide_ncb;
  const int64_t items = (int64_t)(*p.num_runs) * ncb;
  if (item >= items) return;
  WideRun m0 = wide_run(p, item, items, ncb);
  WideLane d0 = wide_lane(p, m0, 0);
  WideRun m1 = wide_run(p, item + nw, items, ncb);
  for (; item < items; item += nw) {
    const WideRun m2 = wide_run(p, item + 2 * nw, items, ncb);
    const WideLane d1 = wide_lane(p, m1, 0);
    wide_item<CPL, UNR, BF16, WK>(p, m0, d0, (int)(item % ncb));
    m0 = m1;
    d0 = d1;
    m1 = m2;
  }
}


// Short runs of row-wise Adagrad / INT8 rows wider than 1024 columns: one
// wave per run (grid-stride over the runs), launched only when a table is
// that wide.
template <bool BF16, int WK>
__global__ __launch_bounds__(256) void k_reduce_wide_multi(RedParams p) {
  if (!runs_match(p)) return;
  const int64_t runs = *p.num_runs;
  const int64_t nw = (int64_t)gridDim.x * 4;
  const uint64_t imask = info_mask(p);
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < runs; r += nw) {
    WideRun m;
    m.s = uni32(p.cum[r]);
    m.e = uni32(p.cum[r + 1]);
    const int len = m.e - m.s;
    if (len <= 0 || len >= p.thr) continue;
    const WideLane d0 = wide_lane(p, m, 0);
    const uint64_t kv0 = rl64(d0.kv, 0);
    const int t = uni32(table_of(p, (uint32_t)(kv0 & imask)));
    const TabMeta tm = tab_meta<WK>(p, t);
    if (tm.D <= 1024) continue;
    wide_run_multi<BF16, WK>(p, m, d0, t, tm, (int64_t)(kv0 >> p.info_bits));
  }
}

// ------------------------------------------------------------------ k_forward
//
// Pooled forward, the operation the backward differentiates: the output row
// of bag (t, b) is the sum over its lookups of coef * weight row (FBTT
// `cache_forward_kernel` sums the weight rows of a segment's lookups into
// the segment's output row); coef is the backward's, the per-sample weight
// times 1/L for a mean bag.  Nobag: a lookup's output row is its weight row.
// A lane group of lpl lanes (4 columns per lane; one width for all tables,
// that of the narrowest) takes one bag and a wave 64/lpl bags of one table;
// wider rows take several column blocks.  A slice of lpl lookups has its
// indices and coefficients loaded one per lane, then broadcast by shuffles
// while UNR weight rows per lane are in flight.  Sums in fp64, rounded once.
// UNR lookups x NB column blocks of weight rows are in flight per lane: the
// launcher takes NB = 1 when every row fits one block, more for wider rows
// (and for nobag, whose segments are single lookups, UNR = 1).
template <int UNR, int NB, bool NOBAG>
__global__ __launch_bounds__(256) void k_forward(FwdParams p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) p.header->epoch = p.epoch;
  const int lane = lane_id();
  const int lpl = p.lpl, lg = __builtin_ctz((unsigned)lpl), G = 64 >> lg;
  const int g = lane >> lg, lig = lane & (lpl - 1), gb = g << lg;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tw = wave / p.waves_per_table;
  if (tw >= p.T) return;  // (wave-uniform)
  const int t = (int)tw;
  const int64_t seg = (wave - tw * p.waves_per_table) * G + g;
  const bool live = seg < p.segs_per_table;
  const int D = p.doff[t + 1] - p.doff[t];
  const int64_t E = p.hsc[t + 1] - p.hsc[t];
  const float* W = p.weights + p.woff[t];
  // the segment's lookups [s, e): a bag, or one lookup without offsets
  int64_t s = 0, e = 0;
  bool bad_off = false;
  if (live) {
    if (p.offsets) {
      const int64_t bag = (int64_t)t * p.B + seg;
      s = p.offsets[bag];
      e = p.offsets[bag + 1];
      bad_off = s < 0 || e < s || e > p.N || (bag == 0 && s != 0) ||
                (bag == (int64_t)p.T * p.B - 1 && e != p.N);
      if (bad_off) {
        s = min(max(s, (int64_t)0), p.N);
        e = s;
      }
    } else {
      s = seg;
      e = seg + 1;
    }
  }
  set_status_wave(p.status, p.epoch, kStOffsets, bad_off);
  const float scale = (p.pooling == kPoolMean && e > s) ? 1.0f / (float)(e - s) : 1.0f;
  // slices of the wave's longest bag (a uniform trip count: shuffles below
  // need the whole wave)
  int64_t maxlen = e - s;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) maxlen = max(maxlen, __shfl_xor(maxlen, off, 64));
  const int64_t nslices = (maxlen + lpl - 1) / lpl;
  const int span = 4 * lpl;  // columns of one block
  bool bad_idx = false;
#pragma unroll 1
  for (int c0 = 0; c0 < D; c0 += span * NB) {
    bool cok[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) cok[k] = live && c0 + k * span + 4 * lig < D;
    d4 acc[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) acc[k] = d4_zero();
#pragma unroll 1
    for (int64_t sl = 0; sl < nslices; ++sl) {
      const int64_t j0 = s + sl * lpl;
      const int64_t j = j0 + lig;
      // this lane's lookup of the slice (loaded only when the group has one
      // left; the index is inside [s, e) then)
      int64_t x = 0;
      float cf = 0.f;
      if (live && j < e) {
        x = p.indices[j];
        cf = (p.psw ? p.psw[j] : 1.0f) * scale;
        if (x < 0 || x >= E) {
          bad_idx = true;
          x = x < 0 ? 0 : E - 1;
        }
      }
      const int64_t cnt = live ? min((int64_t)lpl, e - j0) : 0;
#pragma unroll 1
      for (int jj = 0; jj < lpl; jj += UNR) {
        if (!__ballot(jj < cnt)) break;
        float4 v[UNR][NB];
        float co[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int src = gb + min(jj + u, lpl - 1);
          const int64_t ro = __shfl(x, src, 64);
          co[u] = __shfl(cf, src, 64);
#pragma unroll
          for (int k = 0; k < NB; ++k) {
            const bool ok = cok[k] && jj + u < cnt;
            v[u][k] = ok ? ld4(W + ro * D + c0 + k * span + 4 * lig) : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
        if constexpr (NOBAG) {
#pragma unroll
          for (int u = 0; u < UNR; ++u)
#pragma unroll
            for (int k = 0; k < NB; ++k)
              if (cok[k] && jj + u < cnt)
                st4(p.out + (j0 + jj + u) * p.out_stride + c0 + k * span + 4 * lig, v[u][k]);
        } else {
#pragma unroll
          for (int u = 0; u < UNR; ++u)
#pragma unroll
            for (int k = 0; k < NB; ++k) d4_fma(acc[k], co[u], v[u][k]);
        }
      }
    }
    if constexpr (!NOBAG) {
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (cok[k])
          st4(p.out + seg * p.out_stride + p.doff[t] + c0 + k * span + 4 * lig,
              round4(acc[k].x, acc[k].y, acc[k].z, acc[k].w));
    }
  }
  set_status_wave(p.status, p.epoch, kStIndex, bad_idx);
}

}  // namespace

// ------------------------------------------------------------------ no-allocation scratch
//
// The workspace of sgb_backward_noalloc, for callers that cannot allocate
// device memory: a file-scope device array, one copy on every GPU the library
// runs on, held until the process ends.  In host code its name is only a
// stand-in for the symbol; the device address of the current GPU's copy is
// looked up once per device and kept.

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------ launchers

hipError_t launch_init(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t want = (n + 255) / 256;
  const int grid = (int)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(k_init, dim3(grid > 0 ? grid : 1), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(p), n);
  return hipGetLastError();
}

hipError_t launch_linearize(const LinParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_linearize, dim3(grid), dim3(kLinThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_sort_pass(const SortParams& p, hipStream_t s) {
  if (p.bits < 1 || p.bits > kMaxDigitBits || (p.hist_next && p.bits_next > p.bits) ||
      p.tiles < 1)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)p.tiles);
  const int64_t tile = sort_tile_items(p.shape);
  if ((int64_t)p.tiles != (p.N + tile - 1) / tile) return hipErrorInvalidValue;
  switch (p.shape) {
    case kSortHuge:
      if (p.bits > 9) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_sort_pass<512, 12, 512>), grid, dim3(512), 0, s, p);
      break;
    case kSortLarge8:
    case kSortLarge8 + 1:
    case kSortLarge8 + 2:
    case kSortLarge8 + 3:
    case kSortLarge12:
      if (p.bits > 9) return hipErrorInvalidValue;
      switch (p.shape - kSortLarge8) {
        case 0: hipLaunchKernelGGL((k_sort_pass<1024, 8, 512>), grid, dim3(1024), 0, s, p); break;
        case 1: hipLaunchKernelGGL((k_sort_pass<1024, 9, 512>), grid, dim3(1024), 0, s, p); break;
        case 2: hipLaunchKernelGGL((k_sort_pass<1024, 10, 512>), grid, dim3(1024), 0, s, p); break;
        case 3: hipLaunchKernelGGL((k_sort_pass<1024, 11, 512>), grid, dim3(1024), 0, s, p); break;
        default: hipLaunchKernelGGL((k_sort_pass<1024, 12, 512>), grid, dim3(1024), 0, s, p);
      }
      break;
    case kSortMedium:
      if (p.bits <= 9)
        hipLaunchKernelGGL((k_sort_pass<512, 8, 512>), grid, dim3(512), 0, s, p);
      else
        hipLaunchKernelGGL((k_sort_pass<512, 8, 1024>), grid, dim3(512), 0, s, p);
      break;
    default:
      if (p.bits <= 9)
        hipLaunchKernelGGL((k_sort_pass<256, 8, 512>), grid, dim3(256), 0, s, p);
      else
        hipLaunchKernelGGL((k_sort_pass<256, 8, 1024>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_rle(const RleParams& p, hipStream_t s) {
  const unsigned tiles = (unsigned)p.tiles;
  if (!p.one_pass) hipLaunchKernelGGL(k_rle_count, dim3(tiles), dim3(kScanThreads), 0, s, p);
  if (!p.one_pass && !p.fuse_scan)
    hipLaunchKernelGGL(k_rle_scan, dim3(1), dim3(kScanThreads), 0, s, p);
  hipLaunchKernelGGL(k_rle_write, dim3(tiles), dim3(kScanThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_post(const PostParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_post, dim3(grid), dim3(kScanThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fill(const FillParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_fill, dim3(grid), dim3(kFillThreads), 0, s, p);
  return hipGetLastError();
}

// Each reducer has an instance per (grad_output dtype, weight kind): the
// fp32-weight instances carry no bf16 or INT8 code (nor its registers).
template <template <bool, int> class L, class... A>
void by_kind(bool bf16, int wk, A&&... a) {
  if (bf16) {
    if (wk == kWINT8) L<true, kWINT8>::go(a...);
    else if (wk == kWBF16) L<true, kWBF16>::go(a...);
    else if (wk == kWF16) L<true, kWF16>::go(a...);
    else L<true, kWF32>::go(a...);
  } else {
    if (wk == kWINT8) L<false, kWINT8>::go(a...);
    else if (wk == kWBF16) L<false, kWBF16>::go(a...);
    else if (wk == kWF16) L<false, kWF16>::go(a...);
    else L<false, kWF32>::go(a...);
  }
}

template <bool BF16, int WK>
struct LongLaunch {
  static void go(const RedParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((k_reduce_long<BF16, WK>), dim3(grid), dim3(256), 0, s, p);
  }
};

hipError_t launch_reduce_long(const RedParams& p, bool bf16, int grid, hipStream_t s) {
  by_kind<LongLaunch>(bf16, p.w_kind, p, grid, s);
  return hipGetLastError();
}

// Row-wise Adagrad and INT8 rows need a whole row in one item: 16 columns
// per lane (rows up to 1024); dense and SGD rows take SGB_WIDE_CPL columns
// per lane.
// The grid is kWideGridMult times the resident workgroups, capped at one
// wave per item of the largest run count the batch allows (N runs).
template <bool BF16, int WK>
struct WideLaunch {
  static unsigned blocks(const RedParams& q, int resident) {
    const int64_t cap = (q.N * q.wide_ncb + 3) / 4;
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>((int64_t)resident * kWideGridMult, cap));
  }
  static void go(RedParams q, int dmax, const int* grid, hipStream_t s) {
    if (q.mode == kModeAdagrad || WK == kWINT8) {
      q.wide_ncb = 1;  // one item per run: a whole row of up to 1024 columns
      hipLaunchKernelGGL((k_reduce_wide<16, kWideUnr16, BF16, WK>), dim3(blocks(q, grid[0])),
                         dim3(256), 0, s, q);
      if (dmax > 1024) {
        // wider rows: one wave per run, as many workgroups as the runs allow
        // up to the wide reducer's grid
        hipLaunchKernelGGL((k_reduce_wide_multi<BF16, WK>), dim3(blocks(q, grid[0])), dim3(256), 0,
                           s, q);
      }
    } else {
      q.wide_ncb = (dmax + 64 * kWideCpl - 1) / (64 * kWideCpl);
      hipLaunchKernelGGL((k_reduce_wide<kWideCpl, kWideUnr, BF16, WK>), dim3(blocks(q, grid[1])),
                         dim3(256), 0, s, q);
    }
  }
};

void launch_reduce_wide(const RedParams& p, bool bf16, int dmax, const int* grid, hipStream_t s) {
  by_kind<WideLaunch>(bf16, p.w_kind, p, dmax, bf16 ? grid + 2 : grid, s);
}

// Resident blocks per CU of the wide-row reducer instances (fp32 weights; the
// grid of the other weight kinds is the same), in the order
// {fp32 whole-row, fp32 other, bf16 whole-row, bf16 other} of grad_output dtypes.
void reduce_wide_blocks_per_cu(int out[4]) {
  const void* k[4] = {
      reinterpret_cast<const void*>(k_reduce_wide<16, kWideUnr16, false, kWF32>),
      reinterpret_cast<const void*>(k_reduce_wide<kWideCpl, kWideUnr, false, kWF32>),
      reinterpret_cast<const void*>(k_reduce_wide<16, kWideUnr16, true, kWF32>),
      reinterpret_cast<const void*>(k_reduce_wide<kWideCpl, kWideUnr, true, kWF32>)};
  for (int i = 0; i < 4; ++i) {
    int n = 0;
    out[i] = (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k[i], 256, 0) == hipSuccess && n > 0)
                 ? n
                 : 2;
  }
}

template <bool BF16, int WK>
struct Short8Launch {
  static void go(const RedParams& q, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((k_reduce_short8<BF16, WK>), grid, dim3(256), 0, s, q);
  }
};

hipError_t launch_reduce_short(const RedParams& p, bool bf16, int dmin, int dmax,
                               const int* wide_grid, int parts, hipStream_t s) {
  const int64_t windows = (p.N + kShortSpan - 1) / kShortSpan;
  // waves per window, reduced when the grid would pass 2^32 threads
  auto sub_for = [&](int want) {
    int sub = want;
    while (sub > 0 && (windows << sub) > (1ll << 25)) --sub;
    return sub;
  };
  if ((parts & kShortRows) && dmin <= 512) {
    // rows up to 512 columns: 8 columns per lane, one wave per row at most
    RedParams q = p;
    q.sub_log = sub_for(kShortSub8);
    const dim3 grid((unsigned)(((windows << q.sub_log) + 3) / 4), 1);
    by_kind<Short8Launch>(bf16, p.w_kind, q, grid, s);
  }
  if ((parts & kWideRows) && dmax > 512) launch_reduce_wide(p, bf16, dmax, wide_grid, s);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdParams& p, hipStream_t s) {
  const int64_t waves = p.waves_per_table * p.T;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  const int span = 4 * p.lpl;
  if (p.pooling == kPoolNone)
    hipLaunchKernelGGL((k_forward<1, 8, true>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else if (p.Dmax <= span)
    hipLaunchKernelGGL((k_forward<4, 1, false>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_forward<2, 4, false>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

int reduce_long_blocks_per_cu(bool bf16) {
  int n = 0;
  hipError_t e = bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_reduce_long<true, kWF32>, 256, 0)
                      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_reduce_long<false, kWF32>, 256, 0);
  return (e == hipSuccess && n > 0) ? n : 2;
}

}  // namespace sgb
