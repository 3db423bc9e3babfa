// Gather-compaction of kept rows and in-place scatter of new K/V rows, gfx950.
//
// Gather (FOCUS paper Section 4.2, H_reduced = H at the kept set; App. E.2.3,
// destinations from a prefix sum):   dst[cu[b] + t] = src[b, idx[b, t]]
// Scatter (ES-dLLM notes page, key design 2, in-place partial cache update;
// FOCUS paper App. E.2.4, sparse cache fill at processing indices):
//   cache[row_base[b] + pos(b, t)] = new[cu[b] + t],  pos = idx or pos_map[b, idx]
//
// Both are pure byte copies of 16-byte-aligned rows, with non-temporal hints
// (every byte is touched once) and kUnroll chunks in flight per thread, all
// loads issued before the stores. The per-sequence counts live on the device,
// so grids are sized from k_max and surplus workgroups exit at once. The
// gather (hidden rows, 8 KB at the workloads) takes one workgroup per row;
// the scatter (K/V rows of a few KB) treats a sequence's kept K and V rows as
// one flat space of chunks split evenly over n_split workgroups (about
// kScatterTarget in all: four per sequence at a batch of 1,024, one from a
// batch of 4,096). All three keep a sequence's workgroups on one XCD, in order
// (xcd_seq_part): measured 10-45 % faster than sequence-major or slot-major
// grids, whose real rows pile up on a few XCDs or lose write locality.
#include "bte_device.h"

namespace bte {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kPass = kThreads * kUnroll;   // chunks one workgroup moves per pass
constexpr int kMaxTensors = 8;             // tensors of one multi-row gather
constexpr int kScatterUnroll = 8;          // chunks in flight per thread in the scatter
constexpr int kScatterTarget = 4096;       // workgroups a scatter launch aims at

// Row and chunk of flat chunk index c, with chunks per row cpr and its float
// reciprocal (exact after the +-1 correction for c < 2^24).
__device__ __forceinline__ void split_chunk(uint32_t c, uint32_t cpr, float inv_cpr, uint32_t& row,
                                            uint32_t& chunk) {
  uint32_t t = (uint32_t)((float)c * inv_cpr);
  if (t * cpr > c) --t;
  if ((t + 1) * cpr <= c) ++t;
  row = t;
  chunk = c - t * cpr;
}

// This workgroup's share [lo, hi) of sequence b's `total` chunks: part s of
// n_split near-equal parts.
__device__ __forceinline__ bool share(uint32_t total, uint32_t n_split, uint32_t s, uint32_t& lo,
                                      uint32_t& hi) {
  lo = (uint32_t)((uint64_t)total * s / n_split);
  hi = (uint32_t)((uint64_t)total * (s + 1) / n_split);
  return lo < hi;
}

// Gather: one workgroup per (sequence, slot t < k_max) in the XCD-grouped
// mapping (sequence b's slots in order on XCD b % 8, so one XCD writes a
// sequence's compacted rows one after another and the XCDs share the rows
// evenly whatever k_max is); a slot past count[b] exits. Large rows (hidden
// states) give every thread whole chunks of one row.
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(
    const char* __restrict__ src, const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
    const int32_t* __restrict__ cu, char* __restrict__ dst, int batch, int n, int k_max,
    size_t row_bytes) {
  int b, t;
  if (!xcd_seq_part(batch, k_max, b, t) || t >= count[b]) return;
  const char* s = src + ((size_t)b * n + idx[(size_t)b * k_max + t]) * row_bytes;
  char* d = dst + ((size_t)cu[b] + t) * row_bytes;
  const size_t chunks = row_bytes / 16;
  for (size_t base = 0; base < chunks; base += kPass) {
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

// Several row tensors compacted with one index set in one launch (FOCUS paper
// App. E.2.3: hidden states, residual, RoPE positions and cache indices).
// One workgroup per (sequence, slot), mapped as in the gather above; each
// tensor's row is copied in 16-byte chunks when its size and pointers allow,
// else in 4-byte words.
struct MultiRows {
  const char* src[kMaxTensors];
  char* dst[kMaxTensors];
  uint32_t row_bytes[kMaxTensors];
  uint32_t wide[kMaxTensors];
  int n_tensors;
};

// Source row of kept slot t: b * n + idx, or src_cu[b] + idx when the source
// rows are themselves compacted by sequence.
__global__ __launch_bounds__(kThreads) void gather_multi_kernel(
    MultiRows m, const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ src_cu, int batch, int n,
    int k_max) {
  int b, t;
  if (!xcd_seq_part(batch, k_max, b, t) || t >= count[b]) return;
  const size_t src_row = (src_cu ? (size_t)src_cu[b] : (size_t)b * n) + idx[(size_t)b * k_max + t];
  const size_t dst_row = (size_t)cu[b] + t;
  for (int k = 0; k < m.n_tensors; ++k) {
    const size_t rb = m.row_bytes[k];
    const char* s = m.src[k] + src_row * rb;
    char* d = m.dst[k] + dst_row * rb;
    if (m.wide[k]) {
      for (size_t c = threadIdx.x; c < rb / 16; c += kThreads)
        __builtin_nontemporal_store(ld16_stream(s + 16 * c), reinterpret_cast<u32x4*>(d + 16 * c));
    } else {
      for (size_t c = threadIdx.x; c < rb / 4; c += kThreads)
        reinterpret_cast<uint32_t*>(d)[c] = reinterpret_cast<const uint32_t*>(s)[c];
    }
  }
}

// Scatter destination: contiguous (row_base[b] + pos) or, with a page table,
// logical position pos_base[b] + pos at row block_table[b][p >> lg] * page +
// p % page of the page pool.
struct ScatterMap {
  const int64_t* row_base;
  const int32_t* pos_base;
  const int32_t* block_table;
  int max_pages;
  int lg_page;
};

// Scatter: sequence b's kept rows of new_k and then of new_v form one flat
// space of (1 or 2) * count[b] * chunks-per-row chunks, split evenly over the
// sequence's n_split workgroups, so one workgroup moves K and V rows alike and
// each thread keeps kScatterUnroll chunks in flight.
template <bool kPaged>
__global__ __launch_bounds__(kThreads) void scatter_rows_kernel(
    const char* __restrict__ new_k, const char* __restrict__ new_v, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ count, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ pos_map, int n, ScatterMap map, char* __restrict__ cache_k,
    char* __restrict__ cache_v, int batch, int k_max, size_t row_bytes, int n_split,
    float inv_cpr) {
  int b, part;
  if (!xcd_seq_part(batch, n_split, b, part)) return;
  const uint32_t cpr = (uint32_t)(row_bytes / 16);
  const uint32_t rows = (uint32_t)count[b];
  const uint32_t tensors = new_v ? 2u : 1u;
  uint32_t lo, hi;
  if (!share(tensors * rows * cpr, (uint32_t)n_split, (uint32_t)part, lo, hi)) return;
  const int32_t* ib = idx + (size_t)b * k_max;
  const int32_t* pm = pos_map ? pos_map + (size_t)b * n : nullptr;
  const int64_t rb = kPaged ? (int64_t)map.pos_base[b] : map.row_base[b];
  const int32_t* bt = kPaged ? map.block_table + (size_t)b * map.max_pages : nullptr;
  const size_t first = (size_t)cu[b];
  for (uint32_t base = lo; base < hi; base += kThreads * kScatterUnroll) {
    u32x4 v[kScatterUnroll];
    char* d[kScatterUnroll];
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u) {
      const uint32_t c = base + u * kThreads + threadIdx.x;
      d[u] = nullptr;
      if (c < hi) {
        uint32_t q, ch;
        split_chunk(c, cpr, inv_cpr, q, ch);
        const bool is_v = q >= rows;
        const uint32_t t = is_v ? q - rows : q;
        const int j = ib[t];
        const int64_t p = rb + (pm ? pm[j] : j);
        size_t row = (size_t)p;
        if constexpr (kPaged) {
          const int lg = map.lg_page;
          row = ((size_t)bt[p >> lg] << lg) + (size_t)(p & ((1 << lg) - 1));
        }
        v[u] = ld16_stream((is_v ? new_v : new_k) + (first + t) * row_bytes + 16 * (size_t)ch);
        d[u] = (is_v ? cache_v : cache_k) + row * row_bytes + 16 * (size_t)ch;
      }
    }
#pragma unroll
    for (int u = 0; u < kScatterUnroll; ++u)
      if (d[u])
        __builtin_nontemporal_store(v[u], (__attribute__((address_space(1))) u32x4*)d[u]);
  }
}

// Workgroups per sequence: about kScatterTarget workgroups in all (one per
// sequence at large batches), but no more than one chunk per thread at k_max
// rows of every tensor. Each sequence's real rows are split evenly over its
// workgroups on the device.
struct Split {
  int n_split;
  bool ok;
};

Split plan(int batch, int k_max, size_t row_bytes, int tensors) {
  const uint64_t cpr = row_bytes / 16;
  const uint64_t chunks = (uint64_t)tensors * k_max * cpr;   // largest flat space of a sequence
  if (chunks >= (1u << 24)) return {0, false};
  const uint64_t want = (kScatterTarget + batch - 1) / batch;
  const uint64_t most = (chunks + kThreads - 1) / kThreads;
  uint64_t n_split = want < most ? want : most;
  if (n_split < 1) n_split = 1;
  if ((uint64_t)(batch + kXcds - 1) / kXcds * kXcds * n_split > 0x7fffffffu) return {0, false};
  return {(int)n_split, true};
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
  const size_t grid = (size_t)(batch + kXcds - 1) / kXcds * kXcds * (size_t)k_max;
  if (grid > 0x7fffffffu) return BTE_ERR_DIM;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     (const char*)src, idx, count, cu, (char*)dst, batch, n, k_max, row_bytes);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

static int scatter_args_ok(const void* new_k, const void* new_v, const int32_t* idx,
                           const int32_t* count, const int32_t* cu, const int32_t* pos_map, int n,
                           const void* cache_k, const void* cache_v, int batch, int k_max,
                           size_t row_bytes) {
  using namespace bte;
  if (!new_k || !idx || !count || !cu || !cache_k) return BTE_ERR_NULL;
  if ((new_v == nullptr) != (cache_v == nullptr)) return BTE_ERR_NULL;
  if (batch <= 0 || k_max < 0 || row_bytes == 0 || (pos_map && n <= 0)) return BTE_ERR_DIM;
  if (row_bytes % 16 != 0 || !aligned16(new_k) || !aligned16(cache_k)) return BTE_ERR_ALIGN;
  if (new_v && (!aligned16(new_v) || !aligned16(cache_v))) return BTE_ERR_ALIGN;
  return BTE_OK;
}

template <bool kPaged>
static int scatter_launch(const void* new_k, const void* new_v, const int32_t* idx,
                          const int32_t* count, const int32_t* cu, const int32_t* pos_map, int n,
                          bte::ScatterMap map, void* cache_k, void* cache_v, int batch, int k_max,
                          size_t row_bytes, hipStream_t stream) {
  using namespace bte;
  const Split sp = plan(batch, k_max, row_bytes, new_v ? 2 : 1);
  if (!sp.ok) return BTE_ERR_DIM;
  const unsigned grid = (unsigned)((batch + kXcds - 1) / kXcds * kXcds * sp.n_split);
  hipLaunchKernelGGL(scatter_rows_kernel<kPaged>, dim3(grid), dim3(kThreads), 0,
                     stream, (const char*)new_k, (const char*)new_v, idx, count, cu, pos_map, n,
                     map, (char*)cache_k, (char*)cache_v, batch, k_max, row_bytes, sp.n_split,
                     1.0f / (float)(row_bytes / 16));
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

extern "C" int bte_kv_scatter(const void* new_k, const void* new_v, const int32_t* idx,
                              const int32_t* count, const int32_t* cu, const int32_t* pos_map,
                              int n, const int64_t* row_base, void* cache_k, void* cache_v,
                              int batch, int k_max, size_t row_bytes, hipStream_t stream) {
  using namespace bte;
  if (!row_base) return BTE_ERR_NULL;
  const int st = scatter_args_ok(new_k, new_v, idx, count, cu, pos_map, n, cache_k, cache_v, batch,
                                 k_max, row_bytes);
  if (st != BTE_OK || k_max == 0) return st;
  return scatter_launch<false>(new_k, new_v, idx, count, cu, pos_map, n,
                               ScatterMap{row_base, nullptr, nullptr, 0, 0}, cache_k, cache_v,
                               batch, k_max, row_bytes, stream);
}

extern "C" int bte_kv_scatter_paged(const void* new_k, const void* new_v, const int32_t* idx,
                                    const int32_t* count, const int32_t* cu,
                                    const int32_t* pos_map, int n, const int32_t* pos_base,
                                    const int32_t* block_table, int max_pages, int page_size,
                                    void* cache_k, void* cache_v, int batch, int k_max,
                                    size_t row_bytes, hipStream_t stream) {
  using namespace bte;
  if (!pos_base || !block_table) return BTE_ERR_NULL;
  const int st = scatter_args_ok(new_k, new_v, idx, count, cu, pos_map, n, cache_k, cache_v, batch,
                                 k_max, row_bytes);
  if (st != BTE_OK) return st;
  if (max_pages <= 0) return BTE_ERR_DIM;
  if (page_size < 1 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return BTE_ERR_UNSUPPORTED;
  if (k_max == 0) return BTE_OK;
  int lg = 0;
  while ((1 << lg) < page_size) ++lg;
  return scatter_launch<true>(new_k, new_v, idx, count, cu, pos_map, n,
                              ScatterMap{nullptr, pos_base, block_table, max_pages, lg}, cache_k,
                              cache_v, batch, k_max, row_bytes, stream);
}

static int gather_multi(const bte_rows_tensor* tensors, int n_tensors, const int32_t* src_cu,
                        const int32_t* idx, const int32_t* count, const int32_t* cu, int batch,
                        int n, int k_max, hipStream_t stream) {
  using namespace bte;
  if (!tensors || !idx || !count || !cu) return BTE_ERR_NULL;
  if (n_tensors < 1 || n_tensors > kMaxTensors || batch <= 0 || n <= 0 || k_max < 0)
    return BTE_ERR_DIM;
  MultiRows m{};
  m.n_tensors = n_tensors;
  for (int k = 0; k < n_tensors; ++k) {
    const bte_rows_tensor& t = tensors[k];
    if (!t.src || !t.dst) return BTE_ERR_NULL;
    if (t.row_bytes == 0 || t.row_bytes > 0xffffffffu) return BTE_ERR_DIM;
    if (t.row_bytes % 4 != 0 || ((uintptr_t)t.src & 3u) || ((uintptr_t)t.dst & 3u))
      return BTE_ERR_ALIGN;
    m.src[k] = (const char*)t.src;
    m.dst[k] = (char*)t.dst;
    m.row_bytes[k] = (uint32_t)t.row_bytes;
    m.wide[k] = (t.row_bytes % 16 == 0 && aligned16(t.src) && aligned16(t.dst)) ? 1u : 0u;
  }
  if (k_max == 0) return BTE_OK;
  const size_t grid = (size_t)(batch + kXcds - 1) / kXcds * kXcds * (size_t)k_max;
  if (grid > 0x7fffffffu) return BTE_ERR_DIM;
  hipLaunchKernelGGL(gather_multi_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, m, idx,
                     count, cu, src_cu, batch, n, k_max);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

extern "C" int bte_gather_rows_multi(const bte_rows_tensor* tensors, int n_tensors,
                                     const int32_t* idx, const int32_t* count, const int32_t* cu,
                                     int batch, int n, int k_max, hipStream_t stream) {
  return gather_multi(tensors, n_tensors, nullptr, idx, count, cu, batch, n, k_max, stream);
}

extern "C" int bte_gather_rows_multi_ragged(const bte_rows_tensor* tensors, int n_tensors,
                                            const int32_t* src_cu, const int32_t* idx,
                                            const int32_t* count, const int32_t* cu, int batch,
                                            int k_max, hipStream_t stream) {
  if (!src_cu) return BTE_ERR_NULL;
  return gather_multi(tensors, n_tensors, src_cu, idx, count, cu, batch, 1, k_max, stream);
}
