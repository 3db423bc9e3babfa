// FOCUS importance delta on gfx950.
//
// Computes, per sequence b and block key j (FOCUS: DLLMs Know How to Tame
// Their Compute Bound, Section 3.1 Eq. 2 and Section 3.2 Eq. 3; App. E.2.1):
//   I_l[j]  = sum_{h, i} softmax_j( maxpool_j( q_l[i,h] . k_l[j,g(h)] / sqrt(D) ) )
//   dI[j]   = I_1[j] - I_0[j], -inf where decoded.
//
// Work layout: one workgroup per sequence, one wave per KV-head group g
// (looping when there are more groups than waves). A wave streams the tiles
// of its group, 32 rows each (K of layer 0, K of layer 1, then the Q tiles of
// the G query heads, layers interleaved), from HBM straight into a two-stage
// LDS ring with coalesced non-temporal copies (whole rows, no registers), so
// the next tile is in flight while one is used. Key tiles are copied from LDS
// into registers once per group; query tiles are read from LDS as MFMA
// operands. 16-byte chunks of a tile row are XOR-swizzled by the row so that
// the operand reads spread over the LDS banks.
//
// Score tile: S^T = K . Q^T on the matrix cores, keys as MFMA rows and query
// rows as MFMA columns. Key row m of the MFMA is fed from block key
// pi(m) = 16*((m/4)%2) + m%4 + 4*(m/8), which makes lane l own query row l%32
// and the 16 contiguous keys 16*(l/32) .. +15 in registers 0..15. Pooling,
// row max, exp and row sum are then in-lane; the only cross-lane traffic per
// tile is the R boundary keys and two scalars with lane l^32. Column sums are
// accumulated per lane over all tiles and reduced across lanes and waves once,
// in a fixed order (no atomics), so results are bitwise reproducible and two
// identical layers give dI = +0.0 exactly. Blocks of 33 to 64 positions take
// a second kernel (two key and two query-row tiles; described below).
#include <math.h>

#include "bte_device.h"

namespace bte {
namespace {

// One tile: 32 rows of D elements. Copied 16 bytes per lane, kRpi rows per
// wave-wide copy; a lane's MFMA operand is half a row (kHalf chunks).
template <int D, bool BF16>
struct Tile {
  static constexpr int kRowBytes = D * (BF16 ? 2 : 4);
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kHalf = kChunks / 2;
  static constexpr int kRpi = 64 / kChunks;
  static constexpr int kCopies = 32 / kRpi;           // wave-wide copies per tile
  static constexpr int kBytes = 32 * kRowBytes;
};

// LDS position of 16-byte chunk c of tile row `row`.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

// Cache policy of the HBM->LDS copies: non-temporal (every byte is read once).
constexpr int kStreamPolicy = 2;

// Compute units of an MI355X (256 over 8 XCDs).
constexpr int kCUs = 256;

// Sequences per workgroup (1, 2 or 4) for the static-tile kernels below, which
// run one workgroup per CU: the choice with the least modelled time, i.e.
// rounds of kCUs workgroups x sequences each workgroup streams x the measured
// cost per sequence (1, 0.92 and 0.89 for 1, 2 and 4 per workgroup: 118.9,
// 109.6 and 105.3 us at batch 1,024). A grid just past a multiple of kCUs
// leaves a last round of few workgroups, each as long as a whole round:
// batch 1,027 at 4 per workgroup (257 workgroups) measured 340 us against
// 246 us at one per workgroup, for the 64-key kernel.
inline int seqs_per_workgroup(int batch) {
  constexpr int kSeqs[3] = {1, 2, 4};
  constexpr int kCost[3] = {100, 92, 89};
  int best = 1;
  long best_cost = -1;
  for (int i = 0; i < 3; ++i) {
    const long wgs = (batch + kSeqs[i] - 1) / kSeqs[i];
    const long cost = (wgs + kCUs - 1) / kCUs * kSeqs[i] * kCost[i];
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = kSeqs[i];
    }
  }
  return best;
}

// This lane's MFMA operand: half h of one tile row, as kHalf 16-byte chunks.
template <int D, bool BF16>
struct HalfRow {
  u32x4 v[Tile<D, BF16>::kHalf];
};

// Plain LDS loads: the compiler then also waits for the other stage's copy in
// flight before them, so about one tile per wave is in flight. Reading through
// inline asm instead (which keeps both stages in flight) measured slower,
// 123 us against 115 us at batch 1,024: these tiles are 32 scattered 256-byte
// rows each, and fewer outstanding requests stream them better.
template <int D, bool BF16>
__device__ __forceinline__ void read_half(HalfRow<D, BF16>& r, const char* tile, int row, int h) {
  using Tl = Tile<D, BF16>;
#pragma unroll
  for (int c = 0; c < Tl::kHalf; ++c)
    r.v[c] = ld16(tile + row * Tl::kRowBytes + (swz(row, h * Tl::kHalf + c) << 4));
}

// S^T tile (32 keys x 32 query rows): contraction over the lane-halves' D/2
// elements each; both operands use the same element order, so the sum is
// over all D.
template <int D, bool BF16>
__device__ __forceinline__ f32x16 score_tile(const HalfRow<D, BF16>& k, const HalfRow<D, BF16>& q) {
  f32x16 acc = {};
  if constexpr (BF16) {
#pragma unroll
    for (int c = 0; c < Tile<D, BF16>::kHalf; ++c) acc = mfma_bf16(k.v[c], q.v[c], acc);
  } else {
#pragma unroll
    for (int c = 0; c < Tile<D, BF16>::kHalf; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = mfma_f32(__uint_as_float(k.v[c][e]), __uint_as_float(q.v[c][e]), acc);
  }
  return acc;
}

// Max over windows of 2R+1 entries of ext (NK + 2R entries): out[r] covers
// ext[r .. r + 2R]. Doubling: after the pass of width w, a[x] = max(ext[x..x+2w-1]).
template <int R, int NK>
__device__ __forceinline__ void sliding_max(float (&ext)[NK + 2 * R], float (&out)[NK]) {
  constexpr int W = 2 * R + 1;
  constexpr int N = NK + 2 * R;
  if constexpr (R == 0) {
#pragma unroll
    for (int r = 0; r < NK; ++r) out[r] = ext[r];
  } else {
    float a[N];
#pragma unroll
    for (int x = 0; x < N; ++x) a[x] = ext[x];
    int w = 1;
#pragma unroll
    for (int pass = 0; pass < 5; ++pass) {
      if (2 * w <= W) {
#pragma unroll
        for (int x = 0; x + w < N; ++x) a[x] = fmaxf(a[x], a[x + w]);
        w *= 2;
      }
    }
#pragma unroll
    for (int r = 0; r < NK; ++r) out[r] = fmaxf(a[r], a[r + W - w]);
  }
}

// Pool along keys (radius R, compile time; R < 0 selects the runtime radius
// rt_r), softmax over the row, and add the row's weights into acc.
// s[r] is the score of this lane's query row with key 16*h + r (masked keys
// are -inf). row_ok = 0 for padding query rows; keys >= B are padding.
// kPair: the tile holds two blocks of 16 (see focus_delta_kernel); this lane's
// half of the row belongs to its query's block iff own_half, else it is
// removed again after the pooling (the scores were already -inf there, but a
// window next to the halves' edge pools the other block's scores into it).
template <int R, bool kPair = false>
__device__ __forceinline__ void pool_softmax_accumulate(const f32x16& s, int h, int rt_r, int B,
                                                        float c, bool row_ok, float (&acc)[16],
                                                        bool own_half = true) {
  float m = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
  m = fmaxf(m, swap_halves(m));

  float p[16];
  if constexpr (R >= 0) {
    float ext[16 + 2 * R];
    if constexpr (R > 0) {
#pragma unroll
      for (int t = 0; t < R; ++t) {
        // lower half sends its top R keys, upper half its bottom R keys
        const float recv = swap_halves(h ? s[t] : s[16 - R + t]);
        ext[t] = h ? recv : -INFINITY;                 // keys 16h - R + t
        ext[R + 16 + t] = h ? -INFINITY : recv;        // keys 16h + 16 + t
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ext[R + r] = s[r];
    sliding_max<R, 16>(ext, p);
  } else {
    // Any radius: bring the whole 32-key row into the lane.
    float full[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float o = swap_halves(s[r]);
      full[r] = h ? o : s[r];
      full[16 + r] = h ? s[r] : o;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 16 * h + r;
      float v = -INFINITY;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int d = j - key;
        v = (d <= rt_r && -d <= rt_r) ? fmaxf(v, full[j]) : v;
      }
      p[r] = v;
    }
  }

  // Keys past the block end are padding: a window next to the edge pools a
  // real score into them, so they are removed again after the pooling.
  if (B < 32) {
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = (16 * h + r < B) ? p[r] : -INFINITY;
  }
  if constexpr (kPair) {
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = own_half ? p[r] : -INFINITY;
  }

  const float mc = m * c;
  float e[16];
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    e[r] = fast_exp2(fmaf(p[r], c, -mc));
    sum += e[r];
  }
  sum += swap_halves(sum);
  const float inv = row_ok ? 1.0f / sum : 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = fmaf(e[r], inv, acc[r]);
}

// Copies tile t of KV group g of sequence b into LDS at dst: t = 0, 1 -> K of
// layer 0, 1; t = 2 + 2e + l -> Q of query head e of the group, layer l. Lane
// (lrow, lslot) copies chunk swz(row, lslot) of row kRpi*i + lrow to LDS chunk
// lslot of that row, for each of the kCopies wave-wide copies i. Rows past the
// block repeat its last row (their scores are masked).
template <int D, bool BF16>
__device__ __forceinline__ void issue_tile(const char* __restrict__ q0, const char* __restrict__ k0,
                                           const char* __restrict__ q1, const char* __restrict__ k1,
                                           int b, int B, int hq, int hkv, int g, int t, char* dst,
                                           int lrow, int lslot) {
  using Tl = Tile<D, BF16>;
  const char* src;
  uint32_t stride;
  if (t < 2) {
    src = (t ? k1 : k0) + ((size_t)b * B * hkv + g) * Tl::kRowBytes;
    stride = (uint32_t)hkv * Tl::kRowBytes;
  } else {
    const int e = (t - 2) >> 1;
    src = ((t & 1) ? q1 : q0) + ((size_t)b * B * hq + (size_t)g * (hq / hkv) + e) * Tl::kRowBytes;
    stride = (uint32_t)hq * Tl::kRowBytes;
  }
#pragma unroll
  for (int i = 0; i < Tl::kCopies; ++i) {
    const int row = Tl::kRpi * i + lrow;
    const int srow = row < B ? row : B - 1;
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(src + srow * stride + 16 * swz(row, lslot)),
        (void __attribute__((address_space(3)))*)(dst + 1024 * i), 16, 0, kStreamPolicy);
  }
}

// kFull: a block of exactly 32 positions, known at compile time, so that the
// tile loop carries no code for padding keys and query rows. kG > 0: kG query
// heads per KV head and one KV group per wave (hkv == kWaves), so that every
// wave's tile sequence (K of both layers, then the Q tiles) is known at
// compile time.
// kSeqs > 1 (with kG > 0): the workgroup takes kSeqs consecutive sequences in
// one continuous tile stream, so that the next sequence's first tiles are in
// flight while one sequence's sums are reduced, and a launch of about one
// workgroup per CU streams without rounds of workgroups starting and ending.
// Measured at batch 1,024, outputs bitwise equal: 118.9 us with one sequence
// per workgroup, 109.6 with two, 105.3 with four (256 workgroups), 145.9 with
// eight (128 workgroups: half the CUs idle); seqs_per_workgroup picks the
// number. A last workgroup with fewer sequences repeats its last one (reads
// only, no second write), so the tile sequence stays fixed at compile time.
// kPair (with kFull): blocks of 16 positions, two per 32-position tile. Two
// consecutive blocks of 16 are laid out in memory exactly as one block of 32
// ([batch, 16, heads, D] is [batch / 2, 32, heads, D]), so the kernel runs on
// batch / 2 virtual sequences of 32 and keeps the two blocks apart: a query
// row's scores with the other block's keys are -inf before and after the
// pooling (so windows end at the blocks' edge, as at any block edge), and its
// softmax is over its own 16 keys. Rows 0-15 and keys 0-15 are the first
// block, 16-31 the second; lane (n, h) holds query n's keys 16h..16h+15, its
// own block's iff h == n / 16. The column sums, and the output and mask
// indices b * 32 + j, then fall on the two blocks' own positions. Without it
// a block of 16 pads every tile to 32 rows: 3.83 TB/s against 6.40 TB/s for
// blocks of 32, on the same bytes at batch 2,048.
template <int D, bool BF16, int R, int kWaves, bool kFull, int kG, int kSeqs = 1,
          bool kPair = false>
__global__ __launch_bounds__(64 * kWaves) void focus_delta_kernel(
    const char* __restrict__ q0, const char* __restrict__ k0, const char* __restrict__ q1,
    const char* __restrict__ k1, const uint8_t* __restrict__ decoded, float* __restrict__ out,
    int batch, int B, int hq, int hkv, int rt_r, float c) {
  static_assert(kSeqs == 1 || kG > 0, "several sequences per workgroup need the static tiles");
  static_assert(!kPair || kFull, "paired blocks of 16 run as full blocks of 32");
  if constexpr (kFull) B = 32;
  if constexpr (kG > 0) {
    hkv = kWaves;
    hq = kG * kWaves;
  }
  using Tl = Tile<D, BF16>;
  using Row = HalfRow<D, BF16>;
  // Two LDS stages per wave when they fit in 128 KB.
  constexpr int kStages = kWaves * 2 * Tl::kBytes <= 128 * 1024 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char ring[kWaves * kStages * Tl::kBytes];
  // per-wave column sums of a sequence; two buffers when sequences follow one another
  __shared__ float red[kSeqs > 1 ? 2 : 1][kWaves][2][32];

  const int b0 = blockIdx.x * kSeqs;
  // Sequence s of this workgroup (a last, partial workgroup repeats its last one).
  auto seq = [&](int s) { return b0 + s < batch ? b0 + s : batch - 1; };
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int G = kG > 0 ? kG : hq / hkv;
  const int kj = 16 * ((n >> 2) & 1) + (n & 3) + 4 * (n >> 3);
  const bool qvalid = n < B;
  char* wring = ring + w * kStages * Tl::kBytes;

  // Tile t of group gi (this wave's gi-th group): t = 0, 1 -> K of layer 0, 1;
  // t = 2 + 2e + l -> Q of head e of the group, layer l.
  const int ngroups = kG > 0 ? 1 : (hkv - w + kWaves - 1) / kWaves;
  const int per_group = 2 + 2 * G;
  // every tile of the workgroup's stream (kSeqs > 1: one group per sequence)
  const int ntiles = kSeqs * ngroups * per_group;
  const int lrow = lane / Tl::kChunks;
  const int lslot = lane % Tl::kChunks;
  float acc0[16], acc1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;

  // Tile `tile` of the stream: group gi of sequence 0 (kSeqs == 1), or the one
  // group of sequence gi (kSeqs > 1).
  auto issue = [&](int tile, int stage) __attribute__((always_inline)) {
    const int gi = tile / per_group;
    const int bs = kSeqs > 1 ? seq(gi) : b0;
    const int g = kSeqs > 1 ? w : w + gi * kWaves;
    issue_tile<D, BF16>(q0, k0, q1, k1, bs, B, hq, hkv, g, tile - gi * per_group,
                        wring + stage * Tl::kBytes, lrow, lslot);
  };
  Row K0, K1;
  if (ntiles > 0) issue(0, 0);
  if (kStages == 2 && ntiles > 1) issue(1, 1);
  auto step = [&](int tile) __attribute__((always_inline)) {
    const int stage = kStages == 2 ? (tile & 1) : 0;
    if (kStages == 2 && tile + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(Tl::kCopies));
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(0));
    }
    __builtin_amdgcn_wave_barrier();
    const char* src = wring + stage * Tl::kBytes;
    const int t = tile % per_group;
    // Each tile is read from LDS into registers first; as soon as those reads
    // have landed the stage is refilled kStages tiles ahead, so the copy is in
    // flight during this tile's MFMA and softmax work.
    auto refill = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_wave_barrier();
      if (tile + kStages < ntiles) issue(tile + kStages, stage);
    };
    if (t < 2) {
      if (t == 0) read_half<D, BF16>(K0, src, kj, h);
      else read_half<D, BF16>(K1, src, kj, h);
      refill();
    } else {
      Row Q;
      read_half<D, BF16>(Q, src, n, h);
      refill();
      f32x16 s;
      if (t & 1) s = score_tile<D, BF16>(K1, Q);
      else s = score_tile<D, BF16>(K0, Q);
      if (B < 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = (16 * h + r < B) ? s[r] : -INFINITY;
      }
      const bool own_half = !kPair || h == (n >> 4);
      if constexpr (kPair) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = own_half ? s[r] : -INFINITY;
      }
      if (t & 1) pool_softmax_accumulate<R, kPair>(s, h, rt_r, B, c, qvalid, acc1, own_half);
      else pool_softmax_accumulate<R, kPair>(s, h, rt_r, B, c, qvalid, acc0, own_half);
    }
  };
  // Sequence s's delta from this workgroup's column sums: the sum over the 32
  // query rows held by each lane half (fixed butterfly order), then over the
  // waves in LDS (fixed order). Clears the sums for the next sequence.
  auto finish = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int x = 1; x < 32; x <<= 1) {
        acc0[r] += __shfl_xor(acc0[r], x, kWave);
        acc1[r] += __shfl_xor(acc1[r], x, kWave);
      }
    }
    // Buffer s & 1: the buffer written here was last read before the previous
    // sequence's barrier, which every wave has passed.
    float(&rb)[kWaves][2][32] = red[kSeqs > 1 ? (s & 1) : 0];
    if (n == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        rb[w][0][16 * h + r] = acc0[r];
        rb[w][1][16 * h + r] = acc1[r];
      }
    }
    __syncthreads();
    if (threadIdx.x < B && b0 + s < batch) {
      const int j = threadIdx.x;
      const int b = b0 + s;
      float i0 = 0.f, i1 = 0.f;
      for (int v = 0; v < kWaves; ++v) {
        i0 += rb[v][0][j];
        i1 += rb[v][1][j];
      }
      out[(size_t)b * B + j] = decoded[(size_t)b * B + j] ? -INFINITY : i1 - i0;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
  };

  if constexpr (kG > 0) {
    // the 2 + 2G tiles of the wave's one group per sequence, unrolled: each
    // tile's kind is static
#pragma unroll
    for (int sq = 0; sq < kSeqs; ++sq) {
#pragma unroll
      for (int t = 0; t < 2 + 2 * kG; ++t) step(sq * (2 + 2 * kG) + t);
      finish(sq);
    }
  } else {
    for (int tile = 0; tile < ntiles; ++tile) step(tile);
    finish(0);
  }
}

// ---- Blocks of 33 to 64 positions -------------------------------------------
//
// The B keys of a row span two MFMA key tiles and the B query rows two query
// tiles. Key tile u feeds MFMA row m from block key
//   32*((m/4)%2) + 16*u + m%4 + 4*(m/8),
// so that lane l holds the 32 contiguous keys 32*(l/32) .. +31 of its query
// row: key 32*(l/32) + 16*u + r in register r of tile u's product. In LDS,
// row r of key tile u holds block key r + 16*(r >= 16) + 16*u, which keeps
// the operand read of the 32-key kernel (row pi(m)). Pooling, the row max,
// exp and the row sum stay in-lane, with the same boundary exchange as the
// 32-key kernel. A group's tiles run layer by layer (both key tiles, then the
// query tiles of each head, two row tiles per head), so only one layer's keys
// are held in registers; the column sums of a layer are folded into LDS at
// its last tile, in a fixed order.

// Pool, softmax and accumulate one query row of up to 64 keys: s[r] is the
// score with key 32*h + r (keys >= B already -inf); lanes l and l^32 together
// hold the row.
template <int R, bool kFull>
__device__ __forceinline__ void pool_softmax_accumulate_wide(const float (&s)[32], int h, int rt_r,
                                                             int B, float c, bool row_ok,
                                                             float (&acc)[32]) {
  float m = s[0];
#pragma unroll
  for (int r = 1; r < 32; ++r) m = fmaxf(m, s[r]);
  m = fmaxf(m, swap_halves(m));

  float p[32];
  if constexpr (R >= 0) {
    float ext[32 + 2 * R];
    if constexpr (R > 0) {
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const float recv = swap_halves(h ? s[t] : s[32 - R + t]);
        ext[t] = h ? recv : -INFINITY;                 // keys 32h - R + t
        ext[R + 32 + t] = h ? -INFINITY : recv;        // keys 32h + 32 + t
      }
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) ext[R + r] = s[r];
    sliding_max<R, 32>(ext, p);
  } else if (rt_r >= B - 1) {
    // The window of every key covers the whole row: each pooled value is the row max.
#pragma unroll
    for (int r = 0; r < 32; ++r) p[r] = m;
  } else {
    // Any other radius: rt_r rounds of a radius-1 max. Rounds compose exactly
    // (round t gives the max over [j - t, j + t]), and the lane pair trades one
    // edge key each per round.
#pragma unroll
    for (int r = 0; r < 32; ++r) p[r] = s[r];
    for (int it = 0; it < rt_r; ++it) {
      const float left = swap_halves(p[31]);       // key 31, for the upper half
      const float right = swap_halves(p[0]);       // key 32, for the lower half
      float q[32];
#pragma unroll
      for (int x = 0; x < 32; ++x) {
        const float lo = x > 0 ? p[x - 1] : (h ? left : -INFINITY);
        const float hi = x < 31 ? p[x + 1] : (h ? -INFINITY : right);
        q[x] = fmaxf(p[x], fmaxf(lo, hi));
      }
#pragma unroll
      for (int x = 0; x < 32; ++x) p[x] = q[x];
    }
  }
  if constexpr (!kFull) {
#pragma unroll
    for (int r = 0; r < 32; ++r) p[r] = (32 * h + r < B) ? p[r] : -INFINITY;
  }

  const float mc = m * c;
  float e[32];
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    e[r] = fast_exp2(fmaf(p[r], c, -mc));
    sum += e[r];
  }
  sum += swap_halves(sum);
  const float inv = row_ok ? 1.0f / sum : 0.0f;
#pragma unroll
  for (int r = 0; r < 32; ++r) acc[r] = fmaf(e[r], inv, acc[r]);
}

// Copies tile u of one layer's tiles of KV group g of sequence b into LDS at
// dst: u = 0, 1 -> key tile u of that layer (k); u = 2 + 2e + qt -> query rows
// 32*qt .. +31 of the group's query head e (q). Lane (lrow, lslot) copies as in
// issue_tile. Rows past the block repeat its last row (their scores are masked).
template <int D, bool BF16>
__device__ __forceinline__ void issue_tile_wide(const char* __restrict__ q,
                                                const char* __restrict__ k, int b, int B, int hq,
                                                int hkv, int g, int u, char* dst, int lrow,
                                                int lslot) {
  using Tl = Tile<D, BF16>;
  const char* src;
  uint32_t stride;
  int qt = 0;
  if (u < 2) {
    src = k + ((size_t)b * B * hkv + g) * Tl::kRowBytes;
    stride = (uint32_t)hkv * Tl::kRowBytes;
  } else {
    const int e = (u - 2) >> 1;
    qt = (u - 2) & 1;
    src = q + ((size_t)b * B * hq + (size_t)g * (hq / hkv) + e) * Tl::kRowBytes;
    stride = (uint32_t)hq * Tl::kRowBytes;
  }
#pragma unroll
  for (int i = 0; i < Tl::kCopies; ++i) {
    const int row = Tl::kRpi * i + lrow;
    const int brow = u < 2 ? row + 16 * (row >= 16) + 16 * u : 32 * qt + row;
    const int srow = brow < B ? brow : B - 1;
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(src + srow * stride + 16 * swz(row, lslot)),
        (void __attribute__((address_space(3)))*)(dst + 1024 * i), 16, 0, kStreamPolicy);
  }
}

// kFull: B = 64 at compile time. kG > 0: kG query heads per KV head and one
// group per wave (hkv == kWaves), so the tile sequence is static and unrolled.
template <int D, bool BF16, int R, int kWaves, bool kFull, int kG, int kSeqs = 1>
__global__ __launch_bounds__(64 * kWaves) void focus_delta_wide_kernel(
    const char* __restrict__ q0, const char* __restrict__ k0, const char* __restrict__ q1,
    const char* __restrict__ k1, const uint8_t* __restrict__ decoded, float* __restrict__ out,
    int batch, int B, int hq, int hkv, int rt_r, float c) {
  static_assert(kSeqs == 1 || kG > 0, "several sequences per workgroup need the static tiles");
  if constexpr (kFull) B = 64;
  if constexpr (kG > 0) {
    hkv = kWaves;
    hq = kG * kWaves;
  }
  using Tl = Tile<D, BF16>;
  using Row = HalfRow<D, BF16>;
  // One LDS stage per wave (a 64 KB ring at eight waves). Measured at batch 1,024,
  // block 64, one sequence per workgroup, in one process on three boxes: 214.8 / 219.1 /
  // 223.3 us against 220.0 / 224.4 / 224.4 us with two stages (outputs bitwise equal).
  // With several sequences per workgroup two stages would spill registers. The 32-key
  // kernel keeps two (one measured 4-5 % slower at batches 256 and 512).
  constexpr int kStages = 1;
  __shared__ __attribute__((aligned(16))) char ring[kWaves * kStages * Tl::kBytes];
  // per-wave column sums of a sequence; two buffers when sequences follow one another
  __shared__ float red[kSeqs > 1 ? 2 : 1][kWaves][2][64];

  // As in the 32-key kernel: kSeqs consecutive sequences per workgroup, a last
  // partial workgroup repeating its last one.
  const int b0 = blockIdx.x * kSeqs;
  auto seq = [&](int s) { return b0 + s < batch ? b0 + s : batch - 1; };
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  const int G = kG > 0 ? kG : hq / hkv;
  const int kj = 16 * ((n >> 2) & 1) + (n & 3) + 4 * (n >> 3);
  char* wring = ring + w * kStages * Tl::kBytes;

  // Tile t of group gi: layer l = t / per_layer, u = t % per_layer (u = 0, 1:
  // key tiles; u = 2 + 2e + qt: query tile qt of head e).
  const int ngroups = kG > 0 ? 1 : (hkv - w + kWaves - 1) / kWaves;
  const int per_layer = 2 + 2 * G;
  const int per_group = 2 * per_layer;
  const int ntiles = kSeqs * ngroups * per_group;
  const int lrow = lane / Tl::kChunks;
  const int lslot = lane % Tl::kChunks;
  float acc[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) acc[r] = 0.f;

  // Tile `tile` of the stream: group gi of sequence 0 (kSeqs == 1), or the one
  // group of sequence gi (kSeqs > 1).
  auto issue = [&](int tile, int stage) __attribute__((always_inline)) {
    const int gi = tile / per_group;
    const int t = tile - gi * per_group;
    const int l = t >= per_layer;
    const int bs = kSeqs > 1 ? seq(gi) : b0;
    const int g = kSeqs > 1 ? w : w + gi * kWaves;
    issue_tile_wide<D, BF16>(l ? q1 : q0, l ? k1 : k0, bs, B, hq, hkv, g, t - l * per_layer,
                             wring + stage * Tl::kBytes, lrow, lslot);
  };
  Row KA, KB;
  if (ntiles > 0) issue(0, 0);
  if (kStages == 2 && ntiles > 1) issue(1, 1);
  auto step = [&](int tile) __attribute__((always_inline)) {
    const int stage = kStages == 2 ? (tile & 1) : 0;
    if (kStages == 2 && tile + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(Tl::kCopies));
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(0));
    }
    __builtin_amdgcn_wave_barrier();
    const char* src = wring + stage * Tl::kBytes;
    const int gi = tile / per_group;
    const int t = tile - gi * per_group;
    const int l = t >= per_layer;
    const int u = t - l * per_layer;
    auto refill = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_wave_barrier();
      if (tile + kStages < ntiles) issue(tile + kStages, stage);
    };
    if (u < 2) {
      if (u == 0) read_half<D, BF16>(KA, src, kj, h);
      else read_half<D, BF16>(KB, src, kj, h);
      refill();
      return;
    }
    Row Q;
    read_half<D, BF16>(Q, src, n, h);
    refill();
    const f32x16 sa = score_tile<D, BF16>(KA, Q);
    const f32x16 sb = score_tile<D, BF16>(KB, Q);
    float s[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = sa[r];
      s[16 + r] = sb[r];
    }
    if constexpr (!kFull) {
#pragma unroll
      for (int r = 0; r < 32; ++r) s[r] = (32 * h + r < B) ? s[r] : -INFINITY;
    }
    const bool row_ok = kFull || 32 * ((u - 2) & 1) + n < B;
    pool_softmax_accumulate_wide<R, kFull>(s, h, rt_r, B, c, row_ok, acc);
    if (u == per_layer - 1) {
      // The layer's last tile: sum the 32 query rows of each lane half (fixed
      // butterfly order) and fold the group's column sums into LDS.
#pragma unroll
      for (int r = 0; r < 32; ++r) {
#pragma unroll
        for (int x = 1; x < 32; x <<= 1) acc[r] += __shfl_xor(acc[r], x, kWave);
      }
      // (kSeqs > 1: buffer gi & 1 for sequence gi; it was last read before the
      // previous sequence's barrier, which every wave has passed)
      if (n == 0) {
        const bool first = kSeqs > 1 || gi == 0;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          float* slot = &red[kSeqs > 1 ? (gi & 1) : 0][w][l][32 * h + r];
          *slot = first ? acc[r] : *slot + acc[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 32; ++r) acc[r] = 0.f;
    }
  };
  // Sequence s's delta from the waves' column sums in LDS (fixed order).
  auto finish = [&](int s) __attribute__((always_inline)) {
    __syncthreads();
    if (threadIdx.x < B && b0 + s < batch) {
      const int j = threadIdx.x;
      const int b = b0 + s;
      float(&rb)[kWaves][2][64] = red[kSeqs > 1 ? (s & 1) : 0];
      float i0 = 0.f, i1 = 0.f;
      for (int v = 0; v < kWaves; ++v) {
        i0 += rb[v][0][j];
        i1 += rb[v][1][j];
      }
      out[(size_t)b * B + j] = decoded[(size_t)b * B + j] ? -INFINITY : i1 - i0;
    }
  };
  if constexpr (kG > 0) {
#pragma unroll
    for (int sq = 0; sq < kSeqs; ++sq) {
#pragma unroll
      for (int t = 0; t < 2 * (2 + 2 * kG); ++t) step(sq * 2 * (2 + 2 * kG) + t);
      finish(sq);
    }
  } else {
    for (int tile = 0; tile < ntiles; ++tile) step(tile);
    finish(0);
  }
}

template <int D, bool BF16, int R, int kWaves>
hipError_t launch_wide_w(const void* q0, const void* k0, const void* q1, const void* k1,
                         const uint8_t* decoded, float* out, int batch, int B, int hq, int hkv,
                         int rt_r, float c, hipStream_t stream) {
  const char *a0 = (const char*)q0, *a1 = (const char*)k0, *a2 = (const char*)q1,
             *a3 = (const char*)k1;
  if constexpr (kWaves == 8 && R >= 0) {
    if (B == 64 && hkv == 8 && hq == 32) {
      // Sequences per workgroup as in the 32-key kernel (bf16 only).
      if constexpr (BF16) {
        const int per_wg = seqs_per_workgroup(batch);
        if (per_wg == 4) {
          hipLaunchKernelGGL((focus_delta_wide_kernel<D, BF16, R, kWaves, true, 4, 4>),
                             dim3((batch + 3) / 4), dim3(64 * kWaves), 0, stream, a0, a1, a2, a3,
                             decoded, out, batch, B, hq, hkv, rt_r, c);
          return hipGetLastError();
        }
        if (per_wg == 2) {
          hipLaunchKernelGGL((focus_delta_wide_kernel<D, BF16, R, kWaves, true, 4, 2>),
                             dim3((batch + 1) / 2), dim3(64 * kWaves), 0, stream, a0, a1, a2, a3,
                             decoded, out, batch, B, hq, hkv, rt_r, c);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((focus_delta_wide_kernel<D, BF16, R, kWaves, true, 4>), dim3(batch),
                         dim3(64 * kWaves), 0, stream, a0, a1, a2, a3, decoded, out, batch, B, hq,
                         hkv, rt_r, c);
      return hipGetLastError();
    }
  }
  if (B == 64)
    hipLaunchKernelGGL((focus_delta_wide_kernel<D, BF16, R, kWaves, true, 0>), dim3(batch),
                       dim3(64 * kWaves), 0, stream, a0, a1, a2, a3, decoded, out, batch, B, hq,
                       hkv, rt_r, c);
  else
    hipLaunchKernelGGL((focus_delta_wide_kernel<D, BF16, R, kWaves, false, 0>), dim3(batch),
                       dim3(64 * kWaves), 0, stream, a0, a1, a2, a3, decoded, out, batch, B, hq,
                       hkv, rt_r, c);
  return hipGetLastError();
}

// Blocks of exactly 32 positions (kPair: pairs of blocks of 16, as 32).
template <int D, bool BF16, int R, int kWaves, bool kPair>
hipError_t launch_full(const char* a0, const char* a1, const char* a2, const char* a3,
                       const uint8_t* decoded, float* out, int batch, int hq, int hkv, int rt_r,
                       float c, hipStream_t stream) {
  constexpr int B = 32;
  if constexpr (kWaves == 8) {
    if (hkv == 8 && hq == 32) {
      // Several sequences per workgroup in bf16 with a compile-time radius
      // only: the runtime-radius and fp32 variants would spill registers.
      if constexpr (BF16 && R >= 0) {
        const int per_wg = seqs_per_workgroup(batch);
        if (per_wg == 4) {
          hipLaunchKernelGGL((focus_delta_kernel<D, BF16, R, kWaves, true, 4, 4, kPair>),
                             dim3((batch + 3) / 4), dim3(64 * kWaves), 0, stream, a0, a1, a2, a3,
                             decoded, out, batch, B, hq, hkv, rt_r, c);
          return hipGetLastError();
        }
        if (per_wg == 2) {
          hipLaunchKernelGGL((focus_delta_kernel<D, BF16, R, kWaves, true, 4, 2, kPair>),
                             dim3((batch + 1) / 2), dim3(64 * kWaves), 0, stream, a0, a1, a2, a3,
                             decoded, out, batch, B, hq, hkv, rt_r, c);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((focus_delta_kernel<D, BF16, R, kWaves, true, 4, 1, kPair>), dim3(batch),
                         dim3(64 * kWaves), 0, stream, a0, a1, a2, a3, decoded, out, batch, B, hq,
                         hkv, rt_r, c);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((focus_delta_kernel<D, BF16, R, kWaves, true, 0, 1, kPair>), dim3(batch),
                     dim3(64 * kWaves), 0, stream, a0, a1, a2, a3, decoded, out, batch, B, hq, hkv,
                     rt_r, c);
  return hipGetLastError();
}

template <int D, bool BF16, int R, int kWaves>
hipError_t launch_w(const void* q0, const void* k0, const void* q1, const void* k1,
                    const uint8_t* decoded, float* out, int batch, int B, int hq, int hkv, int rt_r,
                    float c, hipStream_t stream) {
  const char *a0 = (const char*)q0, *a1 = (const char*)k0, *a2 = (const char*)q1,
             *a3 = (const char*)k1;
  if (B == 32)
    return launch_full<D, BF16, R, kWaves, false>(a0, a1, a2, a3, decoded, out, batch, hq, hkv,
                                                  rt_r, c, stream);
  if (B == 16 && batch >= 2) {
    // Blocks of 16 in pairs, as batch / 2 blocks of 32 (the same memory); an odd
    // last block runs on its own.
    hipError_t e = launch_full<D, BF16, R, kWaves, true>(a0, a1, a2, a3, decoded, out, batch / 2,
                                                         hq, hkv, rt_r, c, stream);
    if (e != hipSuccess || batch % 2 == 0) return e;
    const size_t es = BF16 ? 2 : 4;
    const size_t last = (size_t)(batch - 1) * 16;
    const size_t qo = last * hq * D * es, ko = last * hkv * D * es;
    return launch_w<D, BF16, R, kWaves>(a0 + qo, a1 + ko, a2 + qo, a3 + ko, decoded + last,
                                        out + last, 1, 16, hq, hkv, rt_r, c, stream);
  }
  hipLaunchKernelGGL((focus_delta_kernel<D, BF16, R, kWaves, false, 0>), dim3(batch),
                     dim3(64 * kWaves), 0, stream, a0, a1, a2, a3, decoded, out, batch, B, hq,
                     hkv, rt_r, c);
  return hipGetLastError();
}

// One wave per KV group, at most 8 (a wave loops over groups beyond that).
// fp32 rows of head dim 128 need more than the 256 VGPRs a wave may hold at two
// waves per SIMD (eight per workgroup): those take at most four waves.
template <int D, bool BF16, int R>
hipError_t launch_r(const void* q0, const void* k0, const void* q1, const void* k1,
                    const uint8_t* decoded, float* out, int batch, int B, int hq, int hkv, int rt_r,
                    float c, hipStream_t stream) {
  constexpr bool kWide = BF16 || D < 128;
  if (B > 32) {
    if (kWide && hkv >= 8) return launch_wide_w<D, BF16, R, kWide ? 8 : 4>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, rt_r, c, stream);
    if (hkv >= 4) return launch_wide_w<D, BF16, R, 4>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, rt_r, c, stream);
    if (hkv >= 2) return launch_wide_w<D, BF16, R, 2>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, rt_r, c, stream);
    return launch_wide_w<D, BF16, R, 1>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, rt_r, c, stream);
  }
  if (kWide && hkv >= 8) return launch_w<D, BF16, R, kWide ? 8 : 4>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, rt_r, c, stream);
  if (hkv >= 4) return launch_w<D, BF16, R, 4>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, rt_r, c, stream);
  if (hkv >= 2) return launch_w<D, BF16, R, 2>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, rt_r, c, stream);
  return launch_w<D, BF16, R, 1>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, rt_r, c, stream);
}

template <int D, bool BF16>
hipError_t launch_d(const void* q0, const void* k0, const void* q1, const void* k1,
                    const uint8_t* decoded, float* out, int batch, int B, int hq, int hkv, int r,
                    float c, hipStream_t stream) {
  switch (r) {
    case 0: return launch_r<D, BF16, 0>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, r, c, stream);
    case 1: return launch_r<D, BF16, 1>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, r, c, stream);
    case 2: return launch_r<D, BF16, 2>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, r, c, stream);
    case 3: return launch_r<D, BF16, 3>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, r, c, stream);
    default: return launch_r<D, BF16, -1>(q0, k0, q1, k1, decoded, out, batch, B, hq, hkv, r, c, stream);
  }
}

}  // namespace
}  // namespace bte

extern "C" int bte_focus_importance_delta(const void* q0, const void* k0, const void* q1,
                                          const void* k1, const uint8_t* decoded, float* delta_out,
                                          int batch, int block, int hq, int hkv, int head_dim,
                                          int pool_kernel, bte_dtype dtype, hipStream_t stream) {
  using namespace bte;
  if (!q0 || !k0 || !q1 || !k1 || !decoded || !delta_out) return BTE_ERR_NULL;
  if (batch <= 0 || hq <= 0 || hkv <= 0 || block < 1 || hq % hkv != 0) return BTE_ERR_DIM;
  if (block > 64) return BTE_ERR_DIM;
  if (head_dim != 64 && head_dim != 128) return BTE_ERR_UNSUPPORTED;
  if (pool_kernel < 1 || pool_kernel % 2 == 0) return BTE_ERR_UNSUPPORTED;
  if (dtype != BTE_F32 && dtype != BTE_BF16) return BTE_ERR_UNSUPPORTED;
  if (!aligned16(q0) || !aligned16(k0) || !aligned16(q1) || !aligned16(k1)) return BTE_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(delta_out) & 3u) != 0) return BTE_ERR_ALIGN;
  // Radii of a block's length or more are all equivalent to "whole row".
  const int r = (pool_kernel - 1) / 2 > 64 ? 64 : (pool_kernel - 1) / 2;
  const float c = (float)(1.4426950408889634 / sqrt((double)head_dim));
  hipError_t e;
  if (dtype == BTE_BF16) {
    e = head_dim == 128
            ? launch_d<128, true>(q0, k0, q1, k1, decoded, delta_out, batch, block, hq, hkv, r, c, stream)
            : launch_d<64, true>(q0, k0, q1, k1, decoded, delta_out, batch, block, hq, hkv, r, c, stream);
  } else {
    e = head_dim == 128
            ? launch_d<128, false>(q0, k0, q1, k1, decoded, delta_out, batch, block, hq, hkv, r, c, stream)
            : launch_d<64, false>(q0, k0, q1, k1, decoded, delta_out, batch, block, hq, hkv, r, c, stream);
  }
  return e == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}
