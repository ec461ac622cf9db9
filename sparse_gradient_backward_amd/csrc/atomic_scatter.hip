// atomic_scatter.hip -- the atomic scatter-add backward (libsgb_atomic.so), a
// comparison baseline for the deduplicated path of libsgb.so.
//
// What it computes is fixed by the FBTT-Embedding page's
// `cache_backward_dense_kernel` / `cache_backward_sgd_kernel` (each lookup
// adds its bag's gradient row into the looked-up row, one atomic add per
// element) and tinygrad's `_embedding_bwd_kernel` (the nobag form: fp32
// agent-scope relaxed atomic adds of each token's gradient row).  It shares
// no code with libsgb.so.
//
// One wave per (bag, 256-column block): each lane holds 4 columns of the
// bag's gradient row (loaded once), the wave loads the indices and
// coefficients of up to 64 of the bag's lookups at a time (one per lane) and
// then, lookup by lookup (wave-uniform via readlane), issues 4 fp32 atomic
// adds per lane into the looked-up row.  Atomics return nothing, so a wave
// issues a whole bag's adds without waiting on any of them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgb_atomic.h"

namespace {

struct AtomicParams {
  const int64_t* hsc;
  const int32_t* doff;
  const int64_t* woff;
  const void* grad;
  const int64_t* indices;
  const int64_t* offsets;  // NULL: nobag (one table, every lookup its own row)
  const float* psw;
  float* out;
  int64_t N;
  int64_t nbags;  // B*T, or N for nobag
  int32_t T;
  int32_t B;
  int32_t ncb;  // 256-column blocks of the widest row
  int32_t mean;
  int32_t bf16;
  float scale;
};

__global__ __launch_bounds__(256) void k_atomic_zero(float4* p, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

__device__ __forceinline__ float4 load_grad4(const AtomicParams& p, int64_t elem) {
  if (p.bf16) {
    // bf16 -> fp32 is exact: the 16 bits become the high half of the word
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p.grad) + elem);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.grad) + elem);
}

__device__ __forceinline__ void atomic_add4(float* q, float c, const float4& g) {
  __hip_atomic_fetch_add(q + 0, c * g.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_add(q + 1, c * g.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_add(q + 2, c * g.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_add(q + 3, c * g.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void k_atomic_scatter(AtomicParams p) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.nbags * p.ncb) return;
  const int lane = (int)(threadIdx.x & 63);
  const int64_t bag = item / p.ncb;
  const int cb = (int)(item % p.ncb);
  int t = 0;
  int64_t s = bag, e = bag + 1, grow = bag, gcol0 = 0;
  if (p.offsets) {
    t = (int)(bag / p.B);
    grow = bag - (int64_t)t * p.B;
    s = clamp64(p.offsets[bag], 0, p.N);
    e = clamp64(p.offsets[bag + 1], s, p.N);
    gcol0 = p.doff[t];
  }
  const int D = p.doff[t + 1] - p.doff[t];
  if (e <= s || cb * 256 >= D) return;
  const int col = cb * 256 + 4 * lane;
  const bool on = col < D;
  const int64_t row_stride = p.offsets ? p.doff[p.T] : D;
  const float4 g = on ? load_grad4(p, grow * row_stride + gcol0 + col) : make_float4(0.f, 0.f, 0.f, 0.f);
  const float inv = p.mean ? 1.0f / (float)(e - s) : 1.0f;
  const int64_t E = p.hsc[t + 1] - p.hsc[t];
  float* base = p.out + p.woff[t] + col;
  for (int64_t j0 = s; j0 < e; j0 += 64) {
    const int64_t j = j0 + lane;
    int64_t my_idx = -1;
    float my_c = 0.f;
    if (j < e) {
      my_idx = p.indices[j];
      my_c = p.scale * (p.psw ? p.psw[j] : 1.0f) * inv;
    }
    const int cnt = (int)(e - j0 < 64 ? e - j0 : 64);
    for (int u = 0; u < cnt; ++u) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)my_idx, u);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int32_t)(my_idx >> 32), u);
      const int64_t idx = (int64_t)(((uint64_t)hi << 32) | lo);
      const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_c), u));
      if (idx < 0 || idx >= E) continue;  // outside the table: skipped
      if (on) atomic_add4(base + idx * D, c, g);
    }
  }
}

}  // namespace

extern "C" int sgb_atomic_backward(int32_t T, const int64_t* hash_size_cumsum,
                                   const int32_t* D_offsets, const int64_t* table_offsets,
                                   int32_t max_D, int64_t total_elems, int32_t pooling,
                                   const void* grad_output, int32_t grad_dtype,
                                   const int64_t* indices, int64_t num_indices,
                                   const int64_t* offsets, int32_t B,
                                   const float* per_sample_weights, float* out, float scale,
                                   int32_t zero_first, void* stream) {
  if (T <= 0 || !hash_size_cumsum || !D_offsets || !table_offsets || !out)
    return SGB_ATOMIC_ERR_INVALID_ARGUMENT;
  if (max_D < 4 || max_D > 8192 || max_D % 4 != 0 || total_elems < 0 || total_elems % 4 != 0)
    return SGB_ATOMIC_ERR_INVALID_ARGUMENT;
  if (pooling < 0 || pooling > 2 || (grad_dtype != 0 && grad_dtype != 1))
    return SGB_ATOMIC_ERR_INVALID_ARGUMENT;
  const bool nobag = pooling == 2;
  if (nobag && (T != 1 || offsets || per_sample_weights)) return SGB_ATOMIC_ERR_UNSUPPORTED;
  if (!nobag && (B <= 0 || !offsets || (int64_t)B * T >= (1ll << 31)))
    return SGB_ATOMIC_ERR_INVALID_ARGUMENT;
  if (num_indices < 0 || num_indices >= (1ll << 31)) return SGB_ATOMIC_ERR_INVALID_ARGUMENT;
  if (num_indices > 0 && (!indices || !grad_output)) return SGB_ATOMIC_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)out % 16 != 0 || (uintptr_t)grad_output % 16 != 0)
    return SGB_ATOMIC_ERR_INVALID_ARGUMENT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (zero_first && total_elems > 0) {
    const int64_t n4 = total_elems / 4;
    const int64_t blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(k_atomic_zero, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                       s, reinterpret_cast<float4*>(out), n4);
  }
  AtomicParams p{};
  p.hsc = hash_size_cumsum;
  p.doff = D_offsets;
  p.woff = table_offsets;
  p.grad = grad_output;
  p.indices = indices;
  p.offsets = nobag ? nullptr : offsets;
  p.psw = per_sample_weights;
  p.out = out;
  p.N = num_indices;
  p.nbags = nobag ? num_indices : (int64_t)B * T;
  p.T = T;
  p.B = nobag ? 1 : B;
  p.ncb = (max_D + 255) / 256;
  p.mean = pooling == 1;
  p.bf16 = grad_dtype == 1;
  p.scale = scale;
  const int64_t items = p.nbags * p.ncb;
  if (items > 0 && num_indices > 0) {
    const int64_t blocks = (items + 3) / 4;
    if (blocks >= (1ll << 31)) return SGB_ATOMIC_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(k_atomic_scatter, dim3((unsigned)blocks), dim3(256), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? SGB_ATOMIC_OK : SGB_ATOMIC_ERR_HIP;
}
