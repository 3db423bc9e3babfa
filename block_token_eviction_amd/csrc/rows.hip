// Gather-compaction of kept rows and in-place scatter of new K/V rows, gfx950.
//
// Gather (FOCUS paper Section 4.2, H_reduced = H at the kept set; App. E.2.3,
// destinations from a prefix sum):   dst[cu[b] + t] = src[b, idx[b, t]]
// Scatter (ES-dLLM notes page, key design 2, in-place partial cache update;
// FOCUS paper App. E.2.4, sparse cache fill at processing indices):
//   cache[row_base[b] + pos(b, t)] = new[cu[b] + t],  pos = idx or pos_map[b, idx]
//
// Both are pure byte copies of 16-byte-aligned rows. The per-sequence counts
// live on the device, so the grid covers the upper bound batch * k_max rows
// and a workgroup whose slot t >= count[b] exits at once. Each thread moves up
// to kUnroll 16-byte chunks per pass with all loads issued before the stores.
#include "bte_device.h"

namespace bte {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ void copy_row(const char* __restrict__ s, char* __restrict__ d,
                                         size_t chunks) {
  for (size_t base = 0; base < chunks; base += (size_t)kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t c = base + (size_t)u * kThreads + threadIdx.x;
      if (c < chunks) v[u] = ld16_stream(s + 16 * c);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t c = base + (size_t)u * kThreads + threadIdx.x;
      if (c < chunks) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(d + 16 * c));
    }
  }
}

__global__ __launch_bounds__(kThreads) void gather_rows_kernel(
    const char* __restrict__ src, const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
    const int32_t* __restrict__ cu, char* __restrict__ dst, int n, int k_max, size_t row_bytes) {
  const int b = blockIdx.x / k_max;
  const int t = blockIdx.x - b * k_max;
  if (t >= count[b]) return;
  const int j = idx[(size_t)b * k_max + t];
  copy_row(src + ((size_t)b * n + j) * row_bytes, dst + ((size_t)cu[b] + t) * row_bytes,
           row_bytes / 16);
}

__global__ __launch_bounds__(kThreads) void scatter_rows_kernel(
    const char* __restrict__ new_k, const char* __restrict__ new_v, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ count, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ pos_map, int n, const int64_t* __restrict__ row_base,
    char* __restrict__ cache_k, char* __restrict__ cache_v, int k_max, size_t row_bytes) {
  const int b = blockIdx.x / k_max;
  const int t = blockIdx.x - b * k_max;
  if (t >= count[b]) return;
  const int j = idx[(size_t)b * k_max + t];
  const int64_t pos = pos_map ? pos_map[(size_t)b * n + j] : j;
  const size_t dst_row = (size_t)(row_base[b] + pos);
  const size_t src_row = (size_t)cu[b] + t;
  const char* s = blockIdx.y == 0 ? new_k : new_v;
  char* d = blockIdx.y == 0 ? cache_k : cache_v;
  copy_row(s + src_row * row_bytes, d + dst_row * row_bytes, row_bytes / 16);
}

}  // namespace
}  // namespace bte

extern "C" int bte_gather_rows(const void* src, const int32_t* idx, const int32_t* count,
                               const int32_t* cu, void* dst, int batch, int n, int k_max,
                               size_t row_bytes, hipStream_t stream) {
  using namespace bte;
  if (!src || !idx || !count || !cu || !dst) return BTE_ERR_NULL;
  if (batch <= 0 || n <= 0 || k_max < 0 || row_bytes == 0) return BTE_ERR_DIM;
  if (row_bytes % 16 != 0 || !aligned16(src) || !aligned16(dst)) return BTE_ERR_ALIGN;
  if (k_max == 0) return BTE_OK;
  const size_t grid = (size_t)batch * (size_t)k_max;
  if (grid > 0x7fffffffu) return BTE_ERR_DIM;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     (const char*)src, idx, count, cu, (char*)dst, n, k_max, row_bytes);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

extern "C" int bte_kv_scatter(const void* new_k, const void* new_v, const int32_t* idx,
                              const int32_t* count, const int32_t* cu, const int32_t* pos_map,
                              int n, const int64_t* row_base, void* cache_k, void* cache_v,
                              int batch, int k_max, size_t row_bytes, hipStream_t stream) {
  using namespace bte;
  if (!new_k || !idx || !count || !cu || !row_base || !cache_k) return BTE_ERR_NULL;
  if ((new_v == nullptr) != (cache_v == nullptr)) return BTE_ERR_NULL;
  if (batch <= 0 || k_max < 0 || row_bytes == 0 || (pos_map && n <= 0)) return BTE_ERR_DIM;
  if (row_bytes % 16 != 0 || !aligned16(new_k) || !aligned16(cache_k)) return BTE_ERR_ALIGN;
  if (new_v && (!aligned16(new_v) || !aligned16(cache_v))) return BTE_ERR_ALIGN;
  if (k_max == 0) return BTE_OK;
  const size_t grid = (size_t)batch * (size_t)k_max;
  if (grid > 0x7fffffffu) return BTE_ERR_DIM;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)grid, new_v ? 2 : 1), dim3(kThreads), 0,
                     stream, (const char*)new_k, (const char*)new_v, idx, count, cu, pos_map, n,
                     row_base, (char*)cache_k, (char*)cache_v, k_max, row_bytes);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}
