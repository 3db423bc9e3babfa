// Per-sequence top-K selection and kept-row prefix sum, gfx950.
//
// FOCUS paper Section 4.2 (indices of the top-K masked tokens by delta),
// ES-dLLM notes page key design 1 (keep the top-(1-r)|S| survivors), FOCUS
// paper App. E.2.3 (compaction destinations from a prefix sum).
//
// Order: score descending, then index ascending, with -0.0 == +0.0; NaN and
// -inf are not eligible. Each score becomes a 32-bit key that is monotone in
// that order (sign-flip map, -0 folded into +0, ineligible -> 0), and each
// position's exact rank is counted against every other key of its row held
// in LDS: rank = #{greater keys} + #{equal keys at lower index}. A position
// is kept iff rank < K_eff, which gives the unique result even under ties.
// Kept positions are written in ascending index order using a wave ballot
// prefix (mbcnt) plus the counts of earlier waves of the row.
//
// A second single-workgroup kernel turns the per-row counts into the
// exclusive prefix sum cu[]; both run on the caller's stream, with no host
// synchronisation.
#include "bte_device.h"

namespace bte {
namespace {

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  const bool eligible = !(s != s) && s != -INFINITY;
  if ((u << 1) == 0u) u = 0u;                      // -0.0 -> +0.0
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return eligible ? key : 0u;
}

// NT threads per row (NT = 64 packs 256/64 rows per workgroup).
template <int NT>
__global__ __launch_bounds__(NT < 256 ? 256 : NT) void topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kbud,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ count_out, int batch, int n, int k_max) {
  constexpr int WG = NT < 256 ? 256 : NT;
  constexpr int RPW = WG / NT;                 // rows per workgroup
  constexpr int WPR = NT / kWave;              // waves per row
  __shared__ uint32_t keys[RPW][NT];
  __shared__ int wcnt[RPW][WPR];
  __shared__ int wsel[RPW][WPR];

  const int slot = threadIdx.x / NT;
  const int j = threadIdx.x % NT;
  const int wv = j / kWave;
  const int b = blockIdx.x * RPW + slot;
  const bool row_ok = b < batch;

  const uint32_t key = (row_ok && j < n) ? order_key(scores[(size_t)b * n + j]) : 0u;
  keys[slot][j] = key;
  const uint64_t em = __ballot(key != 0u);
  if ((threadIdx.x & (kWave - 1)) == 0) wcnt[slot][wv] = __popcll(em);
  __syncthreads();

  int n_elig = 0;
#pragma unroll
  for (int v = 0; v < WPR; ++v) n_elig += wcnt[slot][v];
  int keff = row_ok ? kbud[b] : 0;
  keff = keff < 0 ? 0 : keff;
  keff = keff < n_elig ? keff : n_elig;
  keff = keff < k_max ? keff : k_max;

  int rank = 0;
  for (int i = 0; i < n; ++i) {
    const uint32_t o = keys[slot][i];
    rank += (o > key) | ((o == key) & (i < j));
  }
  const bool sel = key != 0u && rank < keff;
  const uint64_t sm = __ballot(sel);
  if ((threadIdx.x & (kWave - 1)) == 0) wsel[slot][wv] = __popcll(sm);
  __syncthreads();
  if (!row_ok) return;

  int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
  for (int v = 0; v < wv; ++v) pos += wsel[slot][v];
  int32_t* row = idx_out + (size_t)b * k_max;
  if (sel) row[pos] = j;
  for (int t = keff + j; t < k_max; t += NT) row[t] = -1;
  if (j == 0) count_out[b] = keff;
}

// cu[0] = 0, cu[b + 1] = cu[b] + count[b]; one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void exclusive_scan_kernel(const int32_t* __restrict__ count,
                                                              int32_t* __restrict__ cu, int batch) {
  __shared__ int wtot[16];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  int carry = 0;
  if (threadIdx.x == 0) cu[0] = 0;
  for (int base = 0; base < batch; base += 1024) {
    const int i = base + threadIdx.x;
    int v = i < batch ? count[i] : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(v, d, kWave);
      if (lane >= d) v += o;
    }
    if (lane == kWave - 1) wtot[w] = v;
    __syncthreads();
    int before = carry;
    for (int u = 0; u < w; ++u) before += wtot[u];
    if (i < batch) cu[i + 1] = before + v;
    int total = 0;
    for (int u = 0; u < 16; ++u) total += wtot[u];
    carry += total;
    __syncthreads();
  }
}

}  // namespace
}  // namespace bte

extern "C" int bte_topk_select(const float* scores, const int32_t* k, int32_t* idx_out,
                               int32_t* count_out, int32_t* cu_out, int batch, int n, int k_max,
                               hipStream_t stream) {
  using namespace bte;
  if (!scores || !k || !count_out || !cu_out || (k_max > 0 && !idx_out)) return BTE_ERR_NULL;
  if (batch <= 0 || n < 1 || n > 1024 || k_max < 0) return BTE_ERR_DIM;
  int32_t* idx = k_max > 0 ? idx_out : nullptr;
  if (n <= 64) {
    hipLaunchKernelGGL(topk_kernel<64>, dim3((batch + 3) / 4), dim3(256), 0, stream, scores, k, idx,
                       count_out, batch, n, k_max);
  } else if (n <= 256) {
    hipLaunchKernelGGL(topk_kernel<256>, dim3(batch), dim3(256), 0, stream, scores, k, idx,
                       count_out, batch, n, k_max);
  } else {
    hipLaunchKernelGGL(topk_kernel<1024>, dim3(batch), dim3(1024), 0, stream, scores, k, idx,
                       count_out, batch, n, k_max);
  }
  if (hipGetLastError() != hipSuccess) return BTE_ERR_LAUNCH;
  hipLaunchKernelGGL(exclusive_scan_kernel, dim3(1), dim3(1024), 0, stream, count_out, cu_out, batch);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}
