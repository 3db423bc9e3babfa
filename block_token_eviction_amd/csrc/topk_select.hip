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
#include <math.h>

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

// Rank of `key`, held by position j, in row[0 .. n): the keys above it plus the
// equal keys at lower positions. Eight keys per iteration come from two
// 16-byte LDS reads that are in flight together (one read per key waited for
// each in turn: 9 us for rows of 256). row is 16-byte aligned and holds 0,
// below every eligible key, from n up to n rounded to 8.
__device__ __forceinline__ int rank_in_row(const uint32_t* row, int n, uint32_t key, int j) {
  int rank = 0;
  for (int i0 = 0; i0 < n; i0 += 8) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(row + i0);
    const u32x4 c = *reinterpret_cast<const u32x4*>(row + i0 + 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      rank += (a[u] > key) | ((a[u] == key) & (i0 + u < j));
      rank += (c[u] > key) | ((c[u] == key) & (i0 + 4 + u < j));
    }
  }
  return rank;
}

// NT threads per row (NT = 64 packs 256/64 rows per workgroup).
template <int NT>
__global__ __launch_bounds__(NT < 256 ? 256 : NT) void topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ kbud,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ count_out, int batch, int n, int k_max) {
  constexpr int WG = NT < 256 ? 256 : NT;
  constexpr int RPW = WG / NT;                 // rows per workgroup
  constexpr int WPR = NT / kWave;              // waves per row
  __shared__ __attribute__((aligned(16))) uint32_t keys[RPW][NT];   // 0 past n
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

  const int rank = rank_in_row(keys[slot], n, key, j);
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


// ---------------------------------------------------------------------------
// FOCUS dynamic budget (FOCUS notes page, key design 2; FOCUS paper Section
// 4.1 and App. E.3.2):  K = min(B, max(ceil(alpha * N_bar), N_sigma)).
// One wave per sequence; lanes load the block positions 64 at a time. The
// integer-deciding arithmetic is float64 with no contraction and the sums run
// over the positions in ascending order (each value taken from its lane in a
// wave-uniform loop), so the result is the same on every run and matches a
// plain float64 evaluation of the same steps. N_sigma counts masked positions
// (finite delta) with delta >= sigma (mode 0: tested exactly as delta >= 0 and
// delta^2 >= variance) or delta > mu + sigma (mode 1, App. E.2.2:
// d = delta - mu > 0 and d^2 > variance); mu and the variance are the
// population ones over the masked positions.
constexpr int kSeqPerBlock = 4;                 // sequences (waves) per workgroup

__device__ __forceinline__ float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__global__ __launch_bounds__(64 * kSeqPerBlock) void focus_budget_kernel(
    const float* __restrict__ delta, const int32_t* __restrict__ token_sum,
    const int32_t* __restrict__ total_steps, double alpha, int mode, int32_t* __restrict__ k_out,
    int batch, int B) {
#pragma clang fp contract(off)
  const int b = blockIdx.x * kSeqPerBlock + (int)(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (b >= batch) return;                                        // wave-uniform
  const float* row = delta + (size_t)b * B;
  int n = 0;
  double total = 0.0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const float x = c0 + lane < B ? row[c0 + lane] : -INFINITY;
    n += __popcll(__ballot(isfinite(x)));
    const int cnt = min(kWave, B - c0);
    for (int l = 0; l < cnt; ++l) {
      const float v = lane_value(x, l);
      if (isfinite(v)) total += (double)v;
    }
  }
  int nsig = 0;
  if (n > 0) {
    const double mu = total / (double)n;
    double ss = 0.0;
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const float x = c0 + lane < B ? row[c0 + lane] : -INFINITY;
      const int cnt = min(kWave, B - c0);
      for (int l = 0; l < cnt; ++l) {
        const float v = lane_value(x, l);
        if (isfinite(v)) {
          const double d = (double)v - mu;
          ss += d * d;
        }
      }
    }
    const double var = ss / (double)n;
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const float x = c0 + lane < B ? row[c0 + lane] : -INFINITY;
      bool hit = false;
      if (isfinite(x)) {
        if (mode == 0) {
          const double xd = (double)x;
          hit = xd >= 0.0 && xd * xd >= var;
        } else {
          const double d = (double)x - mu;
          hit = d > 0.0 && d * d > var;
        }
      }
      nsig += __popcll(__ballot(hit));
    }
  }
  if (lane == 0) {
    const int steps = total_steps[b];
    const double nbar = steps > 0 ? (double)token_sum[b] / (double)steps : 1.0;
    const double kh = ceil(alpha * nbar);
    const int khist = kh >= (double)B ? B : (kh <= 0.0 ? 0 : (int)kh);
    const int k = khist > nsig ? khist : nsig;
    k_out[b] = k < B ? k : B;
  }
}

// Per-sequence decoding history (FOCUS paper App. E.3.1): positions decoded
// now but not before are added to token_sum; total_steps advances by one.
// One wave per sequence.
__global__ __launch_bounds__(64 * kSeqPerBlock) void history_update_kernel(
    const uint8_t* __restrict__ prev, const uint8_t* __restrict__ now,
    int32_t* __restrict__ token_sum, int32_t* __restrict__ total_steps, int batch, int B) {
  const int b = blockIdx.x * kSeqPerBlock + (int)(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (b >= batch) return;
  const size_t base = (size_t)b * B;
  int n = 0;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int j = c0 + lane;
    n += __popcll(__ballot(j < B && now[base + j] != 0 && prev[base + j] == 0));
  }
  if (lane == 0) {
    token_sum[b] += n;
    total_steps[b] += 1;
  }
}

// FOCUS token eviction with its structural constraints in one pass (FOCUS
// paper Section 4.2 and App. E.2.2). One wave per sequence, lane j = block
// position (B <= 64):
//   candidates: the top-K eligible positions (not decoded, finite delta), in
//     the top-K order above (exact rank, ties to the lower index);
//   AR context: the predecessor i-1 of every candidate i;
//   placeholder integrity: every masked position j with
//     rightmost_processed < j < max(candidates);
//   |S| >= 1: an empty set takes the first position of the order over all
//     positions (-inf above NaN).
// Writes S ascending (-1 padded to B), |S|, and rightmost_processed =
// max(previous, max(S)) (App. E.3.1).
__global__ __launch_bounds__(256) void focus_select_kernel(
    const float* __restrict__ delta, const int32_t* __restrict__ kbud,
    const uint8_t* __restrict__ decoded, int32_t* __restrict__ rightmost,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ count_out, int batch, int B) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[4][kWave];   // 0 past B
  const int slot = threadIdx.x / kWave;
  const int j = threadIdx.x % kWave;
  const int b = blockIdx.x * 4 + slot;
  const bool row_ok = b < batch;
  const bool pos_ok = row_ok && j < B;
  const float x = pos_ok ? delta[(size_t)b * B + j] : __builtin_nanf("");
  const bool dec = pos_ok ? decoded[(size_t)b * B + j] != 0 : true;
  const uint32_t key = (pos_ok && !dec) ? order_key(x) : 0u;
  keys[slot][j] = key;
  __syncthreads();
  if (!row_ok) return;

  const int n_elig = __popcll(__ballot(key != 0u));
  int keff = kbud[b];
  keff = keff < 0 ? 0 : (keff < n_elig ? keff : n_elig);
  const int rank = rank_in_row(keys[slot], B, key, j);
  const bool cand = key != 0u && rank < keff;
  const uint64_t cm = __ballot(cand);
  const int maxc = cm ? 63 - __clzll(cm) : -1;
  const int rp = rightmost[b];
  const bool pred = j + 1 < B && ((cm >> (j + 1)) & 1ull);
  const bool hold = pos_ok && !dec && j > rp && j < maxc;
  bool in_s = pos_ok && (cand || pred || hold);
  uint64_t sm = __ballot(in_s);
  if (sm == 0) {
    // First position of the order over all positions: largest order key with
    // -inf included and NaN lowest, ties to the lower index.
    uint32_t k2 = 0u;
    if (pos_ok && !(x != x)) {
      uint32_t u = __float_as_uint(x);
      if ((u << 1) == 0u) u = 0u;
      k2 = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    uint64_t best = pos_ok ? (((uint64_t)k2 << 32) | (uint32_t)(kWave - 1 - j)) : 0ull;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const uint64_t o = __shfl_xor(best, d, kWave);
      best = o > best ? o : best;
    }
    in_s = pos_ok && j == kWave - 1 - (int)(uint32_t)best;
    sm = __ballot(in_s);
  }
  const int cnt = __popcll(sm);
  const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
  int32_t* row = idx_out + (size_t)b * B;
  if (in_s) row[pos] = j;
  for (int t = cnt + j; t < B; t += kWave) row[t] = -1;
  if (j == 0) {
    count_out[b] = cnt;
    const int top = 63 - __clzll(sm);
    rightmost[b] = rp > top ? rp : top;
  }
}


// Neighbour-aware delayed commit of block KV states (FOCUS paper Section 4.3,
// App. E.3.1, App. E.3.3). One wave per sequence, lanes over the positions:
// position i commits in this step if it is not cached yet and both it and its
// right neighbour are decoded (the block's last position: once the whole
// block is decoded). `cached` is updated in place; block_done = every
// position cached.
__global__ __launch_bounds__(64 * kSeqPerBlock) void commit_mask_kernel(
    const uint8_t* __restrict__ decoded, uint8_t* __restrict__ cached,
    uint8_t* __restrict__ commit, int32_t* __restrict__ block_done, int batch, int B) {
  const int b = blockIdx.x * kSeqPerBlock + (int)(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (b >= batch) return;
  const size_t base = (size_t)b * B;
  const uint8_t* d = decoded + base;
  bool whole = true;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int j = c0 + lane;
    whole = whole && __ballot(j < B && d[j] == 0) == 0;
  }
  bool done = true;
  for (int c0 = 0; c0 < B; c0 += kWave) {
    const int j = c0 + lane;
    bool open = false;                                  // not cached after this step
    if (j < B) {
      const bool right = j + 1 < B ? d[j + 1] != 0 : whole;
      const bool was = cached[base + j] != 0;
      const bool now = !was && d[j] != 0 && right;
      commit[base + j] = now ? 1 : 0;
      if (now) cached[base + j] = 1;
      open = !(was || now);
    }
    done = done && __ballot(open) == 0;
  }
  if (lane == 0 && block_done) block_done[b] = done ? 1 : 0;
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

extern "C" int bte_focus_budget(const float* delta, const int32_t* token_sum,
                                const int32_t* total_steps, float alpha, int threshold_mode,
                                int32_t* k_out, int batch, int block, hipStream_t stream) {
  using namespace bte;
  if (!delta || !token_sum || !total_steps || !k_out) return BTE_ERR_NULL;
  if (batch <= 0 || block < 1 || block > 1024) return BTE_ERR_DIM;
  if (!(alpha >= 0.f) || !isfinite(alpha) || (threshold_mode != 0 && threshold_mode != 1))
    return BTE_ERR_DIM;
  hipLaunchKernelGGL(focus_budget_kernel, dim3((batch + kSeqPerBlock - 1) / kSeqPerBlock),
                     dim3(64 * kSeqPerBlock), 0, stream, delta,
                     token_sum, total_steps, (double)alpha, threshold_mode, k_out, batch, block);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

extern "C" int bte_focus_history_update(const uint8_t* decoded_prev, const uint8_t* decoded_now,
                                        int32_t* token_sum, int32_t* total_steps, int batch,
                                        int block, hipStream_t stream) {
  using namespace bte;
  if (!decoded_prev || !decoded_now || !token_sum || !total_steps) return BTE_ERR_NULL;
  if (batch <= 0 || block < 1 || block > 1024) return BTE_ERR_DIM;
  hipLaunchKernelGGL(history_update_kernel, dim3((batch + kSeqPerBlock - 1) / kSeqPerBlock),
                     dim3(64 * kSeqPerBlock), 0, stream,
                     decoded_prev, decoded_now, token_sum, total_steps, batch, block);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

extern "C" int bte_focus_select(const float* delta, const int32_t* k, const uint8_t* decoded,
                                int32_t* rightmost_processed, int32_t* idx_out, int32_t* count_out,
                                int32_t* cu_out, int batch, int block, hipStream_t stream) {
  using namespace bte;
  if (!delta || !k || !decoded || !rightmost_processed || !idx_out || !count_out || !cu_out)
    return BTE_ERR_NULL;
  if (batch <= 0 || block < 1) return BTE_ERR_DIM;
  if (block > kWave) return BTE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(focus_select_kernel, dim3((batch + 3) / 4), dim3(256), 0, stream, delta, k,
                     decoded, rightmost_processed, idx_out, count_out, batch, block);
  if (hipGetLastError() != hipSuccess) return BTE_ERR_LAUNCH;
  hipLaunchKernelGGL(exclusive_scan_kernel, dim3(1), dim3(1024), 0, stream, count_out, cu_out, batch);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

extern "C" int bte_focus_commit_mask(const uint8_t* decoded, uint8_t* cached, uint8_t* commit_out,
                                     int32_t* block_done_out, int batch, int block,
                                     hipStream_t stream) {
  using namespace bte;
  if (!decoded || !cached || !commit_out) return BTE_ERR_NULL;
  if (batch <= 0 || block < 1 || block > 1024) return BTE_ERR_DIM;
  hipLaunchKernelGGL(commit_mask_kernel, dim3((batch + kSeqPerBlock - 1) / kSeqPerBlock),
                     dim3(64 * kSeqPerBlock), 0, stream, decoded,
                     cached, commit_out, block_done_out, batch, block);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}
