// ES-dLLM early-skip importance score, gfx950.
//
// ES-dLLM notes page, key design 1: for survivor s of sequence b at absolute
// position p = surv_pos[b, s],
//   score = alpha * conf[b, p] + (1 - alpha) * |x - y|_1 / (sqrt(d) * |y|_2)
// with x this iteration's hidden row and y the cached previous one.
//
// One wave per survivor row: each lane streams its 16-byte chunks of x and y
// (all loads of a pass issued before any use), accumulates |x - y| and y^2 in
// fp32, and the wave reduces with a fixed xor butterfly, so the result is
// bitwise reproducible. sqrt and the division are IEEE correctly rounded, so
// scaling both rows by a power of two leaves the score bitwise unchanged and
// an unchanged row scores alpha * conf exactly.
#include <math.h>

#include "bte_device.h"

namespace bte {
namespace {

constexpr int kRowsPerWG = 4;
constexpr int kUnroll = 8;

template <bool BF16>
__device__ __forceinline__ void accumulate(u32x4 xv, u32x4 yv, float& l1, float& sq) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (BF16) {
      const float x0 = bf16_bits_to_f32(xv[e] & 0xffffu), x1 = bf16_bits_to_f32(xv[e] >> 16);
      const float y0 = bf16_bits_to_f32(yv[e] & 0xffffu), y1 = bf16_bits_to_f32(yv[e] >> 16);
      l1 += fabsf(x0 - y0) + fabsf(x1 - y1);
      sq = fmaf(y0, y0, sq);
      sq = fmaf(y1, y1, sq);
    } else {
      const float x = __uint_as_float(xv[e]), y = __uint_as_float(yv[e]);
      l1 += fabsf(x - y);
      sq = fmaf(y, y, sq);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(64 * kRowsPerWG) void esdllm_kernel(
    const char* __restrict__ h_new, const char* __restrict__ h_prev,
    const int32_t* __restrict__ surv_pos, const float* __restrict__ conf, float alpha,
    float* __restrict__ out, int batch, int n_surv, int seq_len, size_t row_bytes,
    float sqrt_hidden) {
  const int lane = threadIdx.x & (kWave - 1);
  const size_t row = (size_t)blockIdx.x * kRowsPerWG + (threadIdx.x >> 6);
  if (row >= (size_t)batch * n_surv) return;
  const size_t b = row / n_surv;
  const int p = surv_pos[row];
  const char* x = h_new + row * row_bytes;
  const char* y = h_prev + (b * seq_len + p) * row_bytes;
  const size_t chunks = row_bytes / 16;

  float l1 = 0.f, sq = 0.f;
  for (size_t base = 0; base < chunks; base += (size_t)kWave * kUnroll) {
    u32x4 xv[kUnroll], yv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t c = base + (size_t)u * kWave + lane;
      if (c < chunks) {
        xv[u] = ld16_stream(x + 16 * c);
        yv[u] = ld16_stream(y + 16 * c);
      } else {
        xv[u] = yv[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) accumulate<BF16>(xv[u], yv[u], l1, sq);
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    l1 += __shfl_xor(l1, d, kWave);
    sq += __shfl_xor(sq, d, kWave);
  }
  if (lane == 0) {
    const float v = l1 == 0.f ? 0.f : l1 / (sqrt_hidden * sqrtf(sq));
    out[row] = alpha * conf[b * seq_len + p] + (1.0f - alpha) * v;
  }
}

// Score and in-place hidden-cache update of one survivor row per wave
// (ES-dLLM notes page, key design 2: at a skip layer every survivor scores its
// new state against the cached one, then its new state replaces the cached
// one; skipped positions keep theirs). Survivor s < count[b] of sequence b is
// row r = cu[b] + s of h_new and surv_pos (r = b * cap + s without count/cu).
// Each lane loads its chunks of x and y, then stores its x chunks over the y
// chunks it has read: a lane only overwrites bytes it has already loaded, and
// distinct survivors of a sequence own distinct cache rows, so no lane reads a
// byte another lane writes. Slots s >= count[b] score -inf (ineligible for the
// top-K) and touch no row.
template <bool BF16>
__global__ __launch_bounds__(64 * kRowsPerWG) void esdllm_update_kernel(
    const char* __restrict__ h_new, char* __restrict__ h_cache,
    const int32_t* __restrict__ surv_pos, const int32_t* __restrict__ count,
    const int32_t* __restrict__ cu, const float* __restrict__ conf, float alpha,
    float* __restrict__ out, int batch, int cap, int seq_len, size_t row_bytes,
    float sqrt_hidden) {
  const int lane = threadIdx.x & (kWave - 1);
  const size_t item = (size_t)blockIdx.x * kRowsPerWG + (threadIdx.x >> 6);
  if (item >= (size_t)batch * cap) return;
  const size_t b = item / cap;
  const int s = (int)(item - b * cap);
  const int n = count ? count[b] : cap;
  if (s >= n) {
    if (lane == 0) out[item] = -INFINITY;
    return;
  }
  const size_t r = cu ? (size_t)cu[b] + s : item;
  const int p = surv_pos[r];
  const char* x = h_new + r * row_bytes;
  char* y = h_cache + (b * seq_len + p) * row_bytes;
  const size_t chunks = row_bytes / 16;

  float l1 = 0.f, sq = 0.f;
  for (size_t base = 0; base < chunks; base += (size_t)kWave * kUnroll) {
    u32x4 xv[kUnroll], yv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t c = base + (size_t)u * kWave + lane;
      if (c < chunks) {
        xv[u] = ld16_stream(x + 16 * c);
        yv[u] = ld16_stream(y + 16 * c);
      } else {
        xv[u] = yv[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) accumulate<BF16>(xv[u], yv[u], l1, sq);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t c = base + (size_t)u * kWave + lane;
      if (c < chunks) st16_stream(y + 16 * c, xv[u]);
    }
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    l1 += __shfl_xor(l1, d, kWave);
    sq += __shfl_xor(sq, d, kWave);
  }
  if (lane == 0) {
    const float v = l1 == 0.f ? 0.f : l1 / (sqrt_hidden * sqrtf(sq));
    out[item] = alpha * conf[b * seq_len + p] + (1.0f - alpha) * v;
  }
}

// Iteration bookkeeping of ES-dLLM's skipping (ES-dLLM notes page, key design
// 2): one workgroup per sequence. Thread 0 decides whether this iteration runs
// without skipping (the initial full pass, iteration 0, and every period-th
// iteration after it), writes the skip layers' keep counts and advances the
// counter; all threads reset the first skip layer's survivors to the block.
struct EsKeep {
  int32_t k[BTE_ES_MAX_SKIP_LAYERS];
};

__global__ __launch_bounds__(256) void esdllm_schedule_kernel(
    int32_t* __restrict__ iter, const int32_t* __restrict__ block_start, int block_len, int period,
    EsKeep keep, int n_layers, int32_t* __restrict__ surv_pos, int32_t* __restrict__ count,
    int32_t* __restrict__ cu, int32_t* __restrict__ keep_out, uint8_t* __restrict__ refresh_out,
    int batch) {
  const int b = blockIdx.x;
  const int base = block_start[b];
  for (int j = threadIdx.x; j < block_len; j += blockDim.x)
    surv_pos[(size_t)b * block_len + j] = base + j;
  if (threadIdx.x == 0) {
    const int it = iter[b];
    const bool refresh = it == 0 || (period > 0 && it % period == 0);
    count[b] = block_len;
    cu[b] = b * block_len;
    if (b == batch - 1) cu[batch] = batch * block_len;
    for (int l = 0; l < n_layers; ++l) keep_out[(size_t)l * batch + b] = refresh ? block_len : keep.k[l];
    refresh_out[b] = refresh ? 1 : 0;
    iter[b] = it + 1;
  }
}

}  // namespace
}  // namespace bte

extern "C" int bte_esdllm_score(const void* h_new, const void* h_prev, const int32_t* surv_pos,
                                const float* conf, float alpha, float* score_out, int batch,
                                int n_surv, int seq_len, int hidden, bte_dtype dtype,
                                hipStream_t stream) {
  using namespace bte;
  if (!h_new || !h_prev || !surv_pos || !conf || !score_out) return BTE_ERR_NULL;
  if (batch <= 0 || n_surv <= 0 || seq_len <= 0 || hidden <= 0) return BTE_ERR_DIM;
  if (dtype != BTE_F32 && dtype != BTE_BF16) return BTE_ERR_UNSUPPORTED;
  const size_t es = dtype == BTE_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)hidden * es;
  if (row_bytes % 16 != 0) return BTE_ERR_UNSUPPORTED;
  if (!aligned16(h_new) || !aligned16(h_prev)) return BTE_ERR_ALIGN;
  const size_t rows = (size_t)batch * n_surv;
  const size_t grid = (rows + kRowsPerWG - 1) / kRowsPerWG;
  if (grid > 0x7fffffffu) return BTE_ERR_DIM;
  const float sh = (float)sqrt((double)hidden);
  if (dtype == BTE_BF16) {
    hipLaunchKernelGGL(esdllm_kernel<true>, dim3((unsigned)grid), dim3(64 * kRowsPerWG), 0, stream,
                       (const char*)h_new, (const char*)h_prev, surv_pos, conf, alpha, score_out,
                       batch, n_surv, seq_len, row_bytes, sh);
  } else {
    hipLaunchKernelGGL(esdllm_kernel<false>, dim3((unsigned)grid), dim3(64 * kRowsPerWG), 0, stream,
                       (const char*)h_new, (const char*)h_prev, surv_pos, conf, alpha, score_out,
                       batch, n_surv, seq_len, row_bytes, sh);
  }
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

extern "C" int bte_esdllm_score_update(const void* h_new, void* h_cache, const int32_t* surv_pos,
                                       const int32_t* count, const int32_t* cu, const float* conf,
                                       float alpha, float* score_out, int batch, int cap,
                                       int seq_len, int hidden, bte_dtype dtype,
                                       hipStream_t stream) {
  using namespace bte;
  if (!h_new || !h_cache || !surv_pos || !conf || !score_out) return BTE_ERR_NULL;
  if ((count == nullptr) != (cu == nullptr)) return BTE_ERR_NULL;
  if (batch <= 0 || cap <= 0 || seq_len <= 0 || hidden <= 0) return BTE_ERR_DIM;
  if (dtype != BTE_F32 && dtype != BTE_BF16) return BTE_ERR_UNSUPPORTED;
  const size_t es = dtype == BTE_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)hidden * es;
  if (row_bytes % 16 != 0) return BTE_ERR_UNSUPPORTED;
  if (!aligned16(h_new) || !aligned16(h_cache)) return BTE_ERR_ALIGN;
  const size_t items = (size_t)batch * cap;
  const size_t grid = (items + kRowsPerWG - 1) / kRowsPerWG;
  if (grid > 0x7fffffffu) return BTE_ERR_DIM;
  const float sh = (float)sqrt((double)hidden);
  if (dtype == BTE_BF16) {
    hipLaunchKernelGGL(esdllm_update_kernel<true>, dim3((unsigned)grid), dim3(64 * kRowsPerWG), 0,
                       stream, (const char*)h_new, (char*)h_cache, surv_pos, count, cu, conf, alpha,
                       score_out, batch, cap, seq_len, row_bytes, sh);
  } else {
    hipLaunchKernelGGL(esdllm_update_kernel<false>, dim3((unsigned)grid), dim3(64 * kRowsPerWG), 0,
                       stream, (const char*)h_new, (char*)h_cache, surv_pos, count, cu, conf, alpha,
                       score_out, batch, cap, seq_len, row_bytes, sh);
  }
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

extern "C" int bte_esdllm_schedule(int32_t* iter, const int32_t* block_start, int block_len,
                                   int period, const int32_t* keep, int n_layers,
                                   int32_t* surv_pos_out, int32_t* count_out, int32_t* cu_out,
                                   int32_t* keep_out, uint8_t* refresh_out, int batch,
                                   hipStream_t stream) {
  using namespace bte;
  if (!iter || !block_start || !surv_pos_out || !count_out || !cu_out || !refresh_out)
    return BTE_ERR_NULL;
  if (n_layers > 0 && (!keep || !keep_out)) return BTE_ERR_NULL;
  if (batch <= 0 || block_len <= 0 || period < 0 || n_layers < 0 ||
      n_layers > BTE_ES_MAX_SKIP_LAYERS)
    return BTE_ERR_DIM;
  if ((int64_t)batch * block_len > 0x7fffffff) return BTE_ERR_DIM;
  EsKeep k{};
  for (int l = 0; l < n_layers; ++l) {
    const int prev = l ? keep[l - 1] : block_len;
    if (keep[l] < 0 || keep[l] > prev) return BTE_ERR_DIM;
    k.k[l] = keep[l];
  }
  hipLaunchKernelGGL(esdllm_schedule_kernel, dim3((unsigned)batch), dim3(256), 0, stream, iter,
                     block_start, block_len, period, k, n_layers, surv_pos_out, count_out, cu_out,
                     keep_out, refresh_out, batch);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}
