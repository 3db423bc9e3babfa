// Reduced-query GQA attention over prefix + block KV, gfx950.
//
// For kept row r of sequence b and query head h (KV head g = h / G):
//   o = softmax_j(scale * q[r,h] . K[seq_start[b] + j, g]) . V[...],  j < kv_len[b]
// (FOCUS paper Section 2 / Table 2, KV-cache attention over the exact cache;
// Section 4.2, later layers on the kept rows only with the evicted tokens as
// fixed reference KV; App. E.2.4, attention for ragged non-contiguous queries.
// ES-dLLM notes page, key design 2: survivors read the whole cached KV.)
//
// Work item: one workgroup per (sequence b, KV head g, group of 32*T query
// rows); the group's rows are the kept tokens' G query heads that share KV
// head g (row = token * G + head-in-group), so every K/V byte of the sequence
// is read once per KV head. The workgroup's waves (two, or four when there are
// few items: waves_for) split the key tiles (32 keys each) round-robin, each
// keeping a private flash-style state (reference max, sum and output), and the
// states are merged in LDS in a fixed order at the end: no HBM workspace and
// no second launch. When a sequence may have more than 64 rows per KV head,
// four-wave workgroups over 128-row groups split the rows instead (kQSplit):
// each wave holds 32 of them and sees every key tile, which the waves copy
// into one shared LDS ring.
//
// Per key tile: S^T = K . Q^T on the matrix cores (keys as MFMA rows fed in a
// permuted order so that lane l owns query column l%32 and the 16 contiguous
// keys 16*(l/32)..+15), online softmax in fp32 in-lane, then O^T += V^T . P^T
// on the matrix cores. K and V tiles are copied from HBM straight into LDS (no
// registers) into two stages per wave, so the next tile's 16 KB are in flight
// while the current one is being used; a stage's K half is refilled as soon as
// the scores are computed, its V half after P.V. 16-byte chunks are XOR-
// swizzled by row so that the K-operand reads and the transposing V reads are
// conflict-free.
//
// The softmax shift is a per-row reference max that only moves when a tile's
// max exceeds it by more than 2^8 in the exp2 domain (so every exponentiated
// score is at most 256): the shift cancels between numerator and denominator,
// bf16 keeps the same relative precision at any scale, and the accumulator
// rescale then runs about once per row instead of on most tiles.
#include <math.h>

#include "bte_device.h"

namespace bte {
namespace {

constexpr float kShiftSlack = 8.0f;   // log2 of the largest exponentiated score

template <int D, bool BF16, int kWaves>
struct Cfg {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int kRowBytes = D * ES;            // one head's K or V row
  static constexpr int kChunks = kRowBytes / 16;      // 16-byte chunks per row
  static constexpr int kHalf = kChunks / 2;           // chunks per lane half = loads per tile
  static constexpr int kRpi = 64 / kChunks;           // tile rows per coalesced load
  static constexpr int kTile = 32 * kRowBytes;        // LDS bytes of one K or V tile
  static constexpr int kOStride = D + 1;              // floats per row of the merge buffer
  static constexpr int kMerge = kWaves * 32 * kOStride * 4 + 2 * kWaves * 32 * 4;
  // LDS stages per wave (K + V tile each): two when all waves' stages fit in
  // 128 KB. (Three or four stages at one wave per workgroup measured slower:
  // the larger LDS share leaves fewer workgroups per CU.)
  static constexpr int kStages = kWaves * 2 * 2 * kTile <= 128 * 1024 ? 2 : 1;
  static constexpr int kStageBytes = 2 * kTile;
  static constexpr int kStage = kWaves * kStages * kStageBytes;
  static constexpr int kLds = kStage > kMerge ? kStage : kMerge;
  // Query split: the workgroup's waves share one ring of kRing stages.
  static constexpr int kRing = 4;
  static constexpr int kRingLds = kRing * kStageBytes > kMerge ? kRing * kStageBytes : kMerge;
};

// LDS placement of 16-byte chunk `c` of tile row `row`. K tiles: rows that the
// K-operand reads fetch together differ in their low 3 bits, so XOR-ing the
// chunk with them spreads a read over all banks. V tiles: the transpose reads
// fetch rows r..r+3 and r+16..r+19 together, so bit 4 of the row moves the
// chunk by 64 bytes.
__device__ __forceinline__ int kpos(int row, int c) { return c ^ (row & 7); }
__device__ __forceinline__ int vpos(int row, int c) { return c ^ (((row >> 4) & 1) << 2); }

// Transposing LDS read (gfx950): in each 16-lane group, lane i receives element
// i%4 of the 8 bytes addressed by group lanes i/4, i/4+4, i/4+8, i/4+12.
// Issued as inline asm so that the compiler does not order it behind the
// in-flight HBM->LDS copies of the other stage (it cannot prove they write
// elsewhere). The compiler does not track these reads: results may only be
// used after lds_wait_tr() has taken them as operands.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a) : "memory");
  return v;
}
// K operands are read with lds_read16 (inline asm, so that the compiler does not
// wait for the copies in flight before them), one chunk ahead of their MFMAs.
// lds_wait16 waits until v has arrived, with at most N (0 or 1) LDS reads
// issued after it still outstanding (LDS reads return in order).
template <int N>
__device__ __forceinline__ void lds_wait16(u32x4& v) {
  static_assert(N == 0 || N == 1, "one read in flight at most");
  if constexpr (N == 0)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v) : : "memory");
  else
    asm volatile("s_waitcnt lgkmcnt(1)" : "+v"(v) : : "memory");
}

// Page-table entry from its LDS copy, read as inline asm
// for the same reason (the value is waited for inside the asm).
__device__ __forceinline__ int lds_read_word(const int32_t* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int32_t*)p;
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}

// Waits for all outstanding LDS reads; the results are in/out operands, so no
// use of them can be scheduled before the wait.
template <int N>
__device__ __forceinline__ void lds_wait_tr(u32x2 (&v)[N]) {
  static_assert(N == 8 || N == 16, "one asm operand per read");
  if constexpr (N == 8) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                   "+v"(v[6]), "+v"(v[7])
                 :
                 : "memory");
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                   "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                   "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
                 :
                 : "memory");
  }
}

// Cache-policy operand of the HBM->LDS copies: non-temporal. Every byte of a
// K/V tile is read exactly once, so the lines need not stay in L2 or the MALL;
// the hint raises the streaming read rate by about a tenth on MI355X.
constexpr int kStreamPolicy = 2;

// Output stores use the sc0 sc1 nt policy (non-temporal, written through every
// cache level). Among the K/V read stream this costs less than the plain
// non-temporal store: the attention measured 1,722 against 1,740 us at batch
// 1,024 (outputs bit-identical; the load policies tried alongside changed
// nothing). The policy is reachable through buffer stores, so each workgroup
// builds a raw buffer resource based at its first output row; the offsets
// within it stay below 2^31 (the host limits k_max * hq * row bytes).
constexpr int kOutPolicy = 1 | 2 | 16;               // sc0 | nt | sc1
constexpr int kRsrcWord3 = 0x00020000;               // gfx9-family raw buffer: 32-bit data format

__device__ __forceinline__ void copy16_to_lds(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_dst, 16, 0,
                                   kStreamPolicy);
}

// Where sequence b's KV rows are: contiguous from seq_start[b], or (kPaged)
// logical position p in row block_table[b][p >> lg_page] * page + p % page of
// a page pool.
struct KvMap {
  const int64_t* seq_start;
  const int32_t* block_table;
  int max_pages;
  int lg_page;
};

// The fused KV scatter (kScatter): kept row t < count[b] of sequence b brings
// new K/V rows cu[b] + t of new_k/new_v, which belong at KV position
// pos_base[b] + idx[b, t] (idx ascending in [0, n)). The attention copies
// those positions' tile rows from new_k/new_v instead of the cache, and the
// workgroup of query row group 0 writes them from its LDS tiles into the
// cache once it has used them (so the scattered bytes are read from HBM once,
// by the attention). The cache rows written are never read by the launch, so
// the writes need no ordering against the reads.
struct KvScatter {
  const char* new_k;
  const char* new_v;
  const int32_t* idx;         // [batch, k_max]
  const int32_t* pos_base;    // [batch]
  char* cache_k;              // the caches again, writable
  char* cache_v;
  int n, k_max;
};
// Largest n: the kept set of a block is a 64-bit mask (bit j = block index j
// kept), and kept row t at index j is the number of kept indices below j.
constexpr int kScatterSpan = 64;

// Waits until at most `behind` tiles of kPerTile copies each are still in
// flight (s_waitcnt needs an immediate; behind <= kMax).
template <int kMax, int kPerTile>
__device__ __forceinline__ void wait_copies_behind(int behind) {
  static_assert(kMax * kPerTile <= 63, "vmcnt holds at most 63");
  if (kMax >= 3 && behind >= 3) {
    __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(kMax >= 3 ? 3 * kPerTile : 0));
  } else if (kMax >= 2 && behind >= 2) {
    __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(kMax >= 2 ? 2 * kPerTile : 0));
  } else if (kMax >= 1 && behind >= 1) {
    __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(kPerTile));
  } else {
    __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(0));
  }
}

// KV layouts: contiguous; paged with the sequence's page-table row staged in
// LDS at workgroup start (a page lookup is then an LDS read); paged with
// lookups from memory, for tables longer than the LDS copy. A lookup from
// memory in front of a copy needs an s_waitcnt vmcnt(0) to use its value,
// which also waits for every copy in flight: that variant is correct but
// serialises the pipeline, so it is a separate kernel and the host picks it
// only when a table has more than kPageCache entries.
enum { kContig = 0, kPagedLds = 1, kPagedMem = 2, kPagedBig = 3 };
// kPagedBig: the table in LDS and pages of at least 32 rows, so that every
// full key tile lies in one page (one lookup per tile, known at compile time).
template <int kPaged>
constexpr bool kLdsTable = kPaged == kPagedLds || kPaged == kPagedBig;
constexpr int kPageCache = 2048;

// Row block of query-split wave w (four waves): 0, 2, 1, 3. The map swaps the two
// bits of w, so it is its own inverse: block j belongs to wave qblock(j).
__device__ __forceinline__ int qblock(int w) { return (w >> 1) | ((w & 1) << 1); }

// One workgroup's work: sequence b, KV head g, the T 32-row query tiles from
// row0 on (each holding at least one real row).
// kQSplit = false: the waves share the query rows and take every kWaves-th key
// tile, their states merged at the end. kQSplit = true (four waves): wave w
// takes the 32*T query rows of row block qblock(w) and every key tile; the tiles
// go through one LDS ring shared by the waves, so each K/V byte is copied from
// HBM once per workgroup.
// kScatter: the KV positions [pb, pb + sc.n) may hold kept rows; bit j of
// `kept` marks block index j (position pb + j) as kept.
template <int D, bool BF16, int T, int kWaves, int kPaged, bool kQSplit, bool kScatter>
__device__ __forceinline__ void attn_body(
    char* __restrict__ smem, const int32_t* __restrict__ pages, const char* __restrict__ q,
    const int32_t* __restrict__ cu, const char* __restrict__ cache_k,
    const char* __restrict__ cache_v, const KvMap& map, const int32_t* __restrict__ kv_len,
    char* __restrict__ out, int hq, int hkv, float c, int b, int g, int rows, int row0,
    const KvScatter& sc, uint64_t kept, int pb) {
  using C = Cfg<D, BF16, kWaves>;
  constexpr int DT = D / 32;                           // 32-wide output column tiles
  const int G = hq / hkv;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int h = lane >> 5;
  // Query split: wave w holds the 32*T rows of row block qblock(w) of the group.
  // Waves 0 and 2 take the first two blocks: in a group of at most 64 rows the
  // busy waves are then 0 and 2, which measured faster than 0 and 1 (on the
  // extended step's selection: 1,889 against 1,966 us), presumably because the
  // busy waves of a CU's two workgroups then spread over more SIMDs.
  const int qrow0 = kQSplit ? row0 + 32 * T * qblock(w) : row0;   // this wave's first query row
  const int kt0 = kQSplit ? 0 : w;                       // this wave's first key tile
  constexpr int kStep = kQSplit ? 1 : kWaves;            // and its key-tile stride
  const int L = kv_len[b];
  const int cub = cu[b];
  const size_t kv_row = (size_t)hkv * C::kRowBytes;    // bytes per cache position
  const size_t seq_off = kPaged != kContig ? 0 : (size_t)map.seq_start[b] * kv_row;
  const char* kbase = cache_k + seq_off + (size_t)g * C::kRowBytes;
  const char* vbase = cache_v + seq_off + (size_t)g * C::kRowBytes;
  const int32_t* bt = kPaged != kContig ? map.block_table + (size_t)b * map.max_pages : nullptr;
  // Cache row (relative to the bases) of logical KV position p.
  auto kv_pos_row = [&](int p) -> size_t {
    if constexpr (kPaged == kContig) {
      return (size_t)p;
    } else {
      const int lg = map.lg_page;
      const int page = kLdsTable<kPaged> ? lds_read_word(pages + (p >> lg)) : bt[p >> lg];
      return ((size_t)page << lg) + (size_t)(p & ((1 << lg) - 1));
    }
  };
  const float thr = fminf(kShiftSlack / c, 3.0e38f);   // reference-max slack in score units

  // Query operands (B of S^T): lane (n, h) holds half h of query row n.
  u32x4 qop[T][C::kHalf];
#pragma unroll
  for (int tq = 0; tq < T; ++tq) {
    const int rho = qrow0 + 32 * tq + n;
    const bool ok = rho < rows;
    const int tok = ok ? rho / G : 0;
    const int head = g * G + (ok ? rho - tok * G : 0);
    const char* p = q + (((size_t)(cub + tok)) * hq + head) * C::kRowBytes + h * (C::kRowBytes / 2);
#pragma unroll
    // Unconditional loads (rows past the end read a valid row and are zeroed):
    // a branch around them would hide from the compiler that the prologue's
    // wait completes them, and it would then wait for every copy in the loop.
    for (int cc = 0; cc < C::kHalf; ++cc) {
      const u32x4 v = ld16(p + 16 * cc);
      qop[tq][cc] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m[T], lsum[T];
  f32x16 o[T][DT];
#pragma unroll
  for (int tq = 0; tq < T; ++tq) {
    m[tq] = -INFINITY;
    lsum[tq] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[tq][dt] = f32x16{};
  }

  const int ntiles = (L + 31) / 32;
  const int kj = 16 * ((n >> 2) & 1) + (n & 3) + 4 * (n >> 3);   // key fed as MFMA row n
  // Query split: the waves use the same key tiles, so they share one ring of
  // C::kRing stages; of every tile, wave w copies half w % 2 of the copies of
  // the K (w < 2) or V (w >= 2) tile. Key split: each wave has its own kStages
  // stages.
  constexpr bool kShared = kQSplit;
  static_assert(!kShared || (kWaves == 4 && BF16), "the shared ring takes four bf16 waves");
  constexpr int kParts = kShared ? 2 : 1;               // waves per tile half
  constexpr int kRing = kShared ? C::kRing : C::kStages;
  constexpr int kPer = C::kHalf / kParts;               // copies per wave and tile (shared ring)
  const int my_half = kShared ? w / kParts : 0;
  const int my_part = kShared ? w % kParts : 0;
  // A query-split wave whose rows all lie past the end copies and waits with
  // the others but computes nothing.
  const bool active = !kQSplit || qrow0 < rows;
  char* wave_lds = kShared ? smem : smem + w * C::kStages * C::kStageBytes;

  // Tile loads go straight from HBM into LDS (16 bytes per lane, no registers):
  // load i of a tile fills the 1 KB at i*1024, lane l writing byte 16*l of it, i.e.
  // tile row kRpi*i + l/kChunks, LDS chunk l%kChunks. Each lane therefore fetches
  // the global chunk that the swizzle maps to that LDS chunk. The tile base is
  // wave-uniform; the per-lane byte offsets within a full tile are fixed.
  const int lrow = lane / C::kChunks;
  const int lslot = lane % C::kChunks;
  const uint32_t lane_row_off = (uint32_t)(lrow * kv_row);
  // A full tile inside one page (contiguous cache, or pages of at least 32
  // rows, since tiles start at multiples of 32) is 32 consecutive cache rows
  // from the row of its first position: one page lookup serves all its copies,
  // K and V. Smaller pages take one lookup per copy.
  const bool tile_in_page = kPaged == kContig || kPaged == kPagedBig || map.lg_page >= 5;
  // Fused scatter: whether key tile kt holds positions of the block, and the
  // kept row at block index j (-1 if j is not kept or outside the block).
  auto in_block = [&](int kt) { return kt * 32 < pb + sc.n && kt * 32 + 32 > pb; };
  auto kept_slot = [&](int j) -> int {
    const bool hit = (unsigned)j < (unsigned)sc.n && ((kept >> (j & 63)) & 1ull);
    return hit ? (int)__popcll(kept & ((1ull << (j & 63)) - 1ull)) : -1;
  };
  // The writes of the kept rows: query row group 0 writes them, from the wave
  // that holds the tile (every wave holds every tile under the query split:
  // wave 0 there). write_kept copies the kept rows of the K (which = 0) or V
  // tile kt from LDS into the cache, 16 bytes per lane, once the tile has
  // been used and before its stage is refilled. Stores are counted by vmcnt
  // too, but loads complete in order among themselves, so the tile waits below
  // stay exact: an outstanding store can only make them wait longer.
  const bool writer = kScatter && row0 == 0 && (!kQSplit || w == 0);
  auto write_kept = [&](int kt, const char* tile, int which) {
    const int last = L - 1 - kt * 32;
    char* cbase = (which ? sc.cache_v : sc.cache_k) + seq_off + (size_t)g * C::kRowBytes;
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += C::kRpi) {
      const int row = r0 + lrow;
      const int p = kt * 32 + row;
      const bool hit = row <= last && kept_slot(p - pb) >= 0;
      if (__ballot(hit) == 0) continue;                  // wave-uniform
      if (hit) {
        const int s = which ? vpos(row, lslot) : kpos(row, lslot);
        u32x4 v = lds_read16(tile + row * C::kRowBytes + 16 * s);
        lds_wait16<0>(v);
        st16(cbase + kv_pos_row(p) * kv_row + 16 * lslot, v);
      }
    }
  };
  auto tile_row = [&](int kt) -> size_t {
    if constexpr (kPaged == kContig) {
      return (size_t)kt * 32;
    } else {
      const int p = kt * 32;
      const int lg = map.lg_page;
      const int page = __builtin_amdgcn_readfirstlane(
          kLdsTable<kPaged> ? lds_read_word(pages + (p >> lg)) : bt[p >> lg]);
      return ((size_t)page << lg) + (size_t)(p & ((1 << lg) - 1));
    }
  };
  // Copies the K (which = 0) or V (which = 1) half of key tile kt into `stage`;
  // trow = tile_row(kt) when tile_in_page. A full tile's copies each cover kRpi
  // consecutive rows that share one page (pages hold a multiple of kRpi rows),
  // so each copy has a wave-uniform base.
  auto issue_half = [&](int kt, int stage, int which, size_t trow, int part) {
    char* dst = wave_lds + stage * C::kStageBytes + which * C::kTile;
    const char* base = which ? vbase : kbase;
    if (kScatter && in_block(kt)) {
      // A tile holding positions that may be kept rows: each row comes from
      // its new K/V row when it is one, else from the cache (rows past the
      // sequence end repeat its last row, as below).
      const char* nbase = (which ? sc.new_v : sc.new_k) + (size_t)g * C::kRowBytes;
      const int last = L - 1 - kt * 32;
#pragma unroll
      for (int u = 0; u < C::kHalf / kParts; ++u) {
        const int i = part * (C::kHalf / kParts) + u;
        const int row = C::kRpi * i + lrow;
        const int p = kt * 32 + (row < last ? row : last);
        const int j = p - pb;
        const int t = kept_slot(j);
        const int chunk = which ? vpos(row, lslot) : kpos(row, lslot);
        const char* src = t >= 0 ? nbase + (size_t)(cub + t) * kv_row + 16 * chunk
                                 : base + kv_pos_row(p) * kv_row + 16 * chunk;
        copy16_to_lds(src, dst + 1024 * i);
      }
    } else if (kt * 32 + 32 <= L) {
#pragma unroll
      for (int u = 0; u < C::kHalf / kParts; ++u) {
        const int i = part * (C::kHalf / kParts) + u;
        const int row = C::kRpi * i + lrow;
        const size_t first = tile_in_page ? trow + C::kRpi * i : kv_pos_row(kt * 32 + C::kRpi * i);
        const size_t row_base = first * kv_row;                            // wave-uniform
        const int chunk = which ? vpos(row, lslot) : kpos(row, lslot);
        copy16_to_lds(base + row_base + (lane_row_off + 16 * chunk), dst + 1024 * i);
      }
    } else {
      // Last, partial tile: rows past the sequence end repeat its last row.
      // They get probability 0 below and a finite V row.
      const int last = L - 1 - kt * 32;
#pragma unroll
      for (int u = 0; u < C::kHalf / kParts; ++u) {
        const int i = part * (C::kHalf / kParts) + u;
        const int row = C::kRpi * i + lrow;
        const size_t prow = kv_pos_row(kt * 32 + (row < last ? row : last));
        const int chunk = which ? vpos(row, lslot) : kpos(row, lslot);
        copy16_to_lds(base + prow * kv_row + 16 * chunk, dst + 1024 * i);
      }
    }
  };
  auto issue_tile = [&](int kt, int stage) {
    const size_t trow = tile_in_page ? tile_row(kt) : 0;
    issue_half(kt, stage, 0, trow, 0);
    issue_half(kt, stage, 1, trow, 0);
  };

  // Lane part of the V^T transposing reads: k-slot (h, t) of P.V MFMA cc is
  // key 16h + 8cc + t; in a 16-lane group, lane gi reads row 16h + 8cc + 4sh + gi/4
  // at column 32dt + 16*((lane/16)%2) + 4*(gi%4).
  const int gi = lane & 15;                            // lane within its 16-lane group
  auto vt_off = [&](int dt, int cc, int sh) {
    const int row = 16 * h + 8 * cc + 4 * sh + (gi >> 2);
    const int byte = 2 * (32 * dt + 16 * ((lane >> 4) & 1) + 4 * (gi & 3));
    return row * C::kRowBytes + (vpos(row, byte >> 4) << 4) + (byte & 15);
  };

  // Prologue: this wave's first kStages tiles, one per stage. A wave with key
  // tiles always issues kStages of them (past its last tile it repeats that
  // tile into a stage the loop does not read), so that a fixed number of copies
  // follows the query loads. Waiting until only those copies are outstanding
  // completes the query loads while the copies stream; the compiler then knows
  // them complete and puts no wait for them into the tile loop, where it would
  // have to wait for every copy in flight.
  static_assert(C::kStages * 2 * C::kHalf <= 63, "vmcnt holds at most 63");
  static_assert((kRing - 1) * kPer <= 63, "vmcnt holds at most 63");
  if (kShared && ntiles > 0) {
    // Shared ring: this wave's part of tiles 0 .. kRing - 2 (repeating the last
    // tile past the end, into stages the loop does not read).
#pragma unroll
    for (int st = 0; st + 1 < kRing; ++st) {
      const int kt = min(st, ntiles - 1);
      issue_half(kt, st, my_half, tile_in_page ? tile_row(kt) : 0, my_part);
    }
    __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits((kRing - 1) * kPer));
  } else if (kt0 < ntiles) {
    const int last = kt0 + (ntiles - 1 - kt0) / kStep * kStep;    // this wave's last tile
#pragma unroll
    for (int st = 0; st < C::kStages; ++st) issue_tile(min(kt0 + st * kStep, last), st);
    __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(C::kStages * 2 * C::kHalf));
  } else {
    __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(0));
  }
  int stage = 0;
  for (int kt = kt0; kt < ntiles; kt += kStep) {
    // Wait for this tile's copies; those of the wave's later tiles already
    // issued (up to kStages - 1 tiles of 2 * kHalf copies) may stay in flight.
    if constexpr (kShared) {
      // This wave's part of tile kt has landed once only those of its later
      // tiles (up to kRing - 2) are in flight; the barrier then waits for the
      // other waves' parts, and every wave is past tile kt - 1, whose stage now
      // takes tile kt + kRing - 1.
      wait_copies_behind<kRing - 2, kPer>(min(kRing - 2, ntiles - 1 - kt));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int ahead = kt + kRing - 1;
      if (ahead < ntiles)
        issue_half(ahead, stage == 0 ? kRing - 1 : stage - 1, my_half,
                   tile_in_page ? tile_row(ahead) : 0, my_part);
      if (!active) {
        stage = stage + 1 == kRing ? 0 : stage + 1;
        continue;
      }
    } else {
      const int later = min(C::kStages - 1, (ntiles - 1 - kt) / kStep);
      wait_copies_behind<C::kStages - 1, 2 * C::kHalf>(later);
      __builtin_amdgcn_wave_barrier();
    }
    const char* kt_lds = wave_lds + stage * C::kStageBytes;
    const char* vt_lds = kt_lds + C::kTile;

    // S^T tiles: lane (n, h), register r = score of query row n with key kt*32 + 16h + r.
    f32x16 s[T];
#pragma unroll
    for (int tq = 0; tq < T; ++tq) s[tq] = f32x16{};
    // K operands, read one chunk ahead of the MFMAs that use them.
    const char* krow = kt_lds + kj * C::kRowBytes;
    u32x4 kop[C::kHalf];
    kop[0] = lds_read16(krow + (kpos(kj, h * C::kHalf) << 4));
#pragma unroll
    for (int cc = 0; cc < C::kHalf; ++cc) {
      if (cc + 1 < C::kHalf) {
        kop[cc + 1] = lds_read16(krow + (kpos(kj, h * C::kHalf + cc + 1) << 4));
        lds_wait16<1>(kop[cc]);
      } else {
        lds_wait16<0>(kop[cc]);
      }
      const u32x4 ka = kop[cc];
#pragma unroll
      for (int tq = 0; tq < T; ++tq) {
        if constexpr (BF16) {
          s[tq] = mfma_bf16(ka, qop[tq][cc], s[tq]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[tq] = mfma_f32(__uint_as_float(ka[e]), __uint_as_float(qop[tq][cc][e]), s[tq]);
        }
      }
    }

    if (writer && in_block(kt)) write_kept(kt, kt_lds, 0);

    // The K half of the stage is consumed: refill it with tile kt + kStages*kStep
    // now (the V half follows after P.V), once the operand reads have landed.
    const int refill = kt + C::kStages * kStep;
    size_t refill_row = 0;
    if (!kShared && refill < ntiles) {
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      refill_row = tile_in_page ? tile_row(refill) : 0;
      issue_half(refill, stage, 0, refill_row, 0);
    }

    // V^T operands, shared by the query tiles: k-slot (h, t) of MFMA cc is key
    // 16h + 8cc + t, for both operands.
    u32x2 vt[DT * 4];
    if constexpr (BF16) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int sh = 0; sh < 2; ++sh)
            vt[4 * dt + 2 * cc + sh] = lds_read_tr16(vt_lds + vt_off(dt, cc, sh));
    }

    // Keys of this lane half that exist. Padding rows of a partial tile repeat
    // the sequence's last key, so the row max is exact without masking; only
    // their probabilities are zeroed below.
    const int kvalid = L - (kt * 32 + 16 * h);
#pragma unroll
    for (int tq = 0; tq < T; ++tq) {
      float mt = fmaxf(s[tq][0], s[tq][1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mt = fmaxf(mt, s[tq][r]);
      mt = fmaxf(mt, swap_halves(mt));
      // Move the reference max only when this tile's max is more than the slack above it.
      const bool move = mt > m[tq] + thr;
      const float mnew = move ? mt : m[tq];
      if (__ballot(move && m[tq] != -INFINITY)) {       // rows with an earlier state
        const float alpha = move ? fast_exp2((m[tq] - mnew) * c) : 1.0f;
        lsum[tq] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[tq][dt][r] *= alpha;
      }
      m[tq] = mnew;
      const float mc = mnew * c;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(s[tq][r], c, -mc));
      if (kvalid < 16) {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = r < kvalid ? p[r] : 0.f;
      }
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ps += p[r];
      lsum[tq] += ps;

      if constexpr (BF16) {
        // P = P_hi + P_lo, both bf16: two products keep P.V accurate to about
        // 2^-16 relative instead of bf16's 2^-9 (V is exact in bf16).
        u32x4 ph[2], pl[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float x0 = p[8 * cc + 2 * u], x1 = p[8 * cc + 2 * u + 1];
            const uint32_t hi = pack_bf16x2(x0, x1);
            ph[cc][u] = hi;
            pl[cc][u] = pack_bf16x2(x0 - __uint_as_float(hi << 16),
                                    x1 - __uint_as_float(hi & 0xffff0000u));
          }
        if (tq == 0) lds_wait_tr(vt);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const u32x2 lo = vt[4 * dt + 2 * cc], hi = vt[4 * dt + 2 * cc + 1];
            const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
            o[tq][dt] = mfma_bf16(a, ph[cc], o[tq][dt]);
            o[tq][dt] = mfma_bf16(a, pl[cc], o[tq][dt]);
          }
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int byte = (32 * dt + n) * 4;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = 16 * h + i;
            const float a = *reinterpret_cast<const float*>(
                vt_lds + row * C::kRowBytes + (vpos(row, byte >> 4) << 4) + (byte & 15));
            o[tq][dt] = mfma_f32(a, p[i], o[tq][dt]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (writer && in_block(kt)) write_kept(kt, vt_lds, 1);
    // The V half is consumed too: refill it.
    if (!kShared && refill < ntiles) issue_half(refill, stage, 1, refill_row, 0);
    stage = stage + 1 == kRing ? 0 : stage + 1;
  }
  // Every copy has landed (the last tile's wait took all of them); the merge
  // below reuses the stage memory.
  __builtin_amdgcn_s_waitcnt(kVmcntNoLgkm | vmcnt_bits(0));

  // Output rows of this sequence, as a buffer resource (see kOutPolicy).
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      out + (size_t)__builtin_amdgcn_readfirstlane(cub) * hq * C::kRowBytes, (short)0, 0x7fffffff,
      kRsrcWord3);

  // Merge the 4 wave states: out = sum_w e^(m_w - M) O_w / sum_w e^(m_w - M) l_w.
  float* obuf = reinterpret_cast<float*>(smem);
  float* mbuf = obuf + kWaves * 32 * C::kOStride;
  float* lbuf = mbuf + kWaves * 32;
#pragma unroll
  for (int tq = 0; tq < T; ++tq) {
    __syncthreads();
    const float lt = lsum[tq] + swap_halves(lsum[tq]);
    if (h == 0) {
      mbuf[w * 32 + n] = m[tq];
      lbuf[w * 32 + n] = lt;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + 8 * (r >> 2) + 4 * h + (r & 3);
        obuf[(w * 32 + n) * C::kOStride + d] = o[tq][dt][r];
      }
    __syncthreads();
    // Output: thread t writes 16-byte chunk t % kChunks of a row, so one store
    // instruction covers whole rows (bf16, D = 128: four 256-byte rows, which
    // are the four query heads of one token, 1 KB contiguous), non-temporal and
    // written through (kOutPolicy). The output is 0.6 % of the bytes, but writes
    // that reach DRAM in the middle of the K/V read stream are costly: with
    // plain stores they took 10 % of the kernel's time (against 1 % for the
    // same stores kept in L2), with non-temporal stores 6 %.
    constexpr int kChunks = C::kRowBytes / 16;          // 16-byte chunks per output row
    constexpr int kElems = 16 / C::ES;                  // elements per chunk
    // Rows written for this tq: 32 merged ones (key split) or the 32 of each wave.
    constexpr int kOutRows = kQSplit ? 32 * kWaves : 32;
    constexpr int kRowsPerPass = 64 * kWaves / kChunks;
    static_assert(kRowsPerPass >= 1 && kOutRows % kRowsPerPass == 0, "passes tile the rows");
    const int chunk = threadIdx.x % kChunks;
#pragma unroll
    for (int r0 = 0; r0 < kOutRows; r0 += kRowsPerPass) {
      const int ro = r0 + threadIdx.x / kChunks;         // output row of this tq
      const int vq = kQSplit ? qblock(ro / 32) : 0;      // query split: the wave that owns it
      const int rr = ro % 32;                            // its row within the 32-row tile
      const int rho = row0 + (kQSplit ? 32 * T * (ro / 32) : 0) + 32 * tq + rr;
      if (rho < rows) {
        // Merge weights: one state per wave (key split), or the owner's own state.
        constexpr int kStates = kQSplit ? 1 : kWaves;
        const int v0 = kQSplit ? vq : 0;
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kStates; ++v) M = fmaxf(M, mbuf[(v0 + v) * 32 + rr]);
        float wgt[kStates];
        float Ls = 0.f;
#pragma unroll
        for (int v = 0; v < kStates; ++v) {
          wgt[v] = fast_exp2((mbuf[(v0 + v) * 32 + rr] - M) * c);
          Ls = fmaf(lbuf[(v0 + v) * 32 + rr], wgt[v], Ls);
        }
        const float inv = 1.0f / Ls;
        const int tok = rho / G;
        const int head = g * G + (rho - tok * G);
        const int voff = (tok * hq + head) * C::kRowBytes + 16 * chunk;
        float res[kElems];
#pragma unroll
        for (int i = 0; i < kElems; ++i) {
          const int d = chunk * kElems + i;
          float acc = 0.f;
#pragma unroll
          for (int v = 0; v < kStates; ++v)
            acc = fmaf(obuf[((v0 + v) * 32 + rr) * C::kOStride + d], wgt[v], acc);
          res[i] = acc * inv;
        }
        u32x4 val;
        if constexpr (BF16) {
#pragma unroll
          for (int u = 0; u < 4; ++u) val[u] = pack_bf16x2(res[2 * u], res[2 * u + 1]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) val[u] = __float_as_uint(res[u]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(val, orsrc, voff, 0, kOutPolicy);
      }
    }
  }
}

// Workgroup x runs on XCD x % 8 (MI355X dispatches workgroups round-robin over
// its 8 XCDs). The mapping below puts all KV heads of one sequence on one XCD,
// one after another, so the 256-byte head slices of each cache row are fetched
// together; sequences go round-robin over the XCDs in the given order.
// Query row groups past a sequence's kept rows exit at once. Such empty
// workgroups must not alternate with real ones at a period of 2 or 4 in an
// XCD's queue: that lines up with the dispatcher's round-robin inside the XCD
// and leaves part of its CUs without real work (measured: 43 % slower at two
// row groups, 160 % at four). With hkv >= 4 a sequence's row groups follow
// one another, each over all its KV heads (period 2 * hkv >= 8; a second row
// group then runs beside the first and finds part of its K/V in L2: 2 % faster
// than the alternative when 15 % of the sequences have one). With fewer KV
// heads the row group is the slowest grid dimension instead: every
// sequence's first row group, then the second ones, and so on.

// kQSplitOk (four waves): a row group spans 32*T*4 query rows, which the waves
// split (attn_body kQSplit); waves past the group's last real row only copy.
// The kernel's LDS is the shared ring (the key-split body is not built in).
// kFixed: 32 query heads over 8 KV heads, known at compile time (constant row
// strides and head mapping in the tile loop's address arithmetic).
template <int D, bool BF16, int T, int kWaves, int kPaged, bool kQSplitOk, bool kScatter,
          bool kFixed = false>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(T == 1 ? 2 : 1))) void attn_kernel(
    const char* __restrict__ q, const int32_t* __restrict__ count, const int32_t* __restrict__ cu,
    const char* __restrict__ cache_k, const char* __restrict__ cache_v, KvMap map,
    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ order, char* __restrict__ out,
    int batch, int hq, int hkv, int n_rg, int rg_inner, float c, KvScatter sc) {
  if constexpr (kFixed) {
    hq = 32;
    hkv = 8;
    rg_inner = 1;
  }
  static_assert(!kQSplitOk || kWaves == 4, "the query split takes four waves");
  __shared__ __attribute__((aligned(16))) char
      smem[kQSplitOk ? Cfg<D, BF16, kWaves>::kRingLds : Cfg<D, BF16, kWaves>::kLds];
  __shared__ int32_t pages[kLdsTable<kPaged> ? kPageCache : 1];
  int r, g, rg;                                        // r: position in the processing order
  if (rg_inner) {
    const int per_seq = hkv * n_rg;                    // workgroups per sequence
    const int s = blockIdx.x / kXcds;
    const int grp = s / per_seq;
    r = kXcds * grp + (int)(blockIdx.x % kXcds);
    const int j = s - grp * per_seq;
    rg = j / hkv;
    g = j - rg * hkv;
  } else {
    const int per_rg = (batch + kXcds - 1) / kXcds * kXcds * hkv;   // workgroups per row group
    rg = blockIdx.x / per_rg;
    const int x = blockIdx.x - rg * per_rg;
    const int s = x / kXcds;
    const int grp = s / hkv;
    r = kXcds * grp + x % kXcds;
    g = s - grp * hkv;
  }
  if (r >= batch) return;
  // Workgroups start in index order, so taking the sequences in the caller's
  // order (longest first) keeps long items out of the tail. An entry outside
  // [0, batch) is clamped: a bad order gives wrong results, never a stray access.
  const int b = order ? min(max(order[r], 0), batch - 1) : r;
  const int cnt = count[b];
  const int rows = cnt * (hq / hkv);
  constexpr int kSpan = kQSplitOk ? 32 * T * kWaves : 32 * T;   // query rows per row group
  const int row0 = rg * kSpan;
  if (row0 >= rows) return;
  if constexpr (kLdsTable<kPaged>) {
    const int n_pages = min((kv_len[b] + (1 << map.lg_page) - 1) >> map.lg_page, map.max_pages);
    const int32_t* bt = map.block_table + (size_t)b * map.max_pages;
    for (int i = threadIdx.x; i < n_pages; i += 64 * kWaves) pages[i] = bt[i];
    __syncthreads();
  }
  int pb = 0;
  uint64_t kept = 0;
  if constexpr (kScatter) {
    // The kept set as a mask, OR-ed over the wave from one index per lane (the
    // load is unconditional, index clamped into the row, so that it is issued
    // beside the other per-sequence loads). An index outside [0, n) marks
    // nothing (it breaks the device contract).
    const int lane = threadIdx.x & 63;
    const int j = sc.idx[(size_t)b * sc.k_max + min(lane, sc.k_max - 1)];
    unsigned long long bit = lane < cnt && j >= 0 && j < sc.n ? 1ull << j : 0ull;
#pragma unroll
    for (int x = 32; x > 0; x >>= 1) bit |= __shfl_xor(bit, x, kWave);
    kept = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(bit >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bit);
    pb = __builtin_amdgcn_readfirstlane(sc.pos_base[b]);
  }
  // Workgroup-uniform choices (every wave of the workgroup takes the same body,
  // so their barriers match): the query split in its own kernels; otherwise
  // skip query tiles that hold no real row.
  if constexpr (kQSplitOk) {
    attn_body<D, BF16, T, kWaves, kPaged, true, kScatter>(smem, pages, q, cu, cache_k, cache_v, map,
                                                          kv_len, out, hq, hkv, c, b, g, rows, row0,
                                                          sc, kept, pb);
  } else if (T == 2 && rows - row0 > 32) {
    attn_body<D, BF16, T, kWaves, kPaged, false, kScatter>(smem, pages, q, cu, cache_k, cache_v,
                                                           map, kv_len, out, hq, hkv, c, b, g,
                                                           rows, row0, sc, kept, pb);
  } else {
    attn_body<D, BF16, 1, kWaves, kPaged, false, kScatter>(smem, pages, q, cu, cache_k, cache_v,
                                                           map, kv_len, out, hq, hkv, c, b, g,
                                                           rows, row0, sc, kept, pb);
  }
}

struct AttnArgs {
  const void* q;
  const int32_t* count;
  const int32_t* cu;
  const void* ck;
  const void* cv;
  KvMap map;
  const int32_t* kl;
  const int32_t* order;
  void* out;
  int batch, k_max, hq, hkv;
  float c;
  KvScatter sc;               // used by the fused-scatter kernels only
};

template <int D, bool BF16, int T, int kWaves, int kPaged, bool kScatter, bool kQSplitOk = false>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  const long rows = (long)a.k_max * (a.hq / a.hkv);
  const long span = kQSplitOk ? 32L * T * kWaves : 32L * T;
  const long n_rg = (rows + span - 1) / span;
  const long grid = (long)((a.batch + kXcds - 1) / kXcds) * kXcds * a.hkv * n_rg;
  if (grid > 0x7fffffffL) return hipErrorInvalidValue;
  if constexpr (BF16 && D == 128 && !kScatter && (kPaged == kContig || kPaged == kPagedBig)) {
    if (a.hq == 32 && a.hkv == 8) {
      hipLaunchKernelGGL((attn_kernel<D, BF16, T, kWaves, kPaged, kQSplitOk, kScatter, true>),
                         dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, (const char*)a.q,
                         a.count, a.cu, (const char*)a.ck, (const char*)a.cv, a.map, a.kl,
                         a.order, (char*)a.out, a.batch, a.hq, a.hkv, (int)n_rg, 1, a.c, a.sc);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_kernel<D, BF16, T, kWaves, kPaged, kQSplitOk, kScatter>),
                     dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, (const char*)a.q, a.count,
                     a.cu, (const char*)a.ck, (const char*)a.cv, a.map, a.kl, a.order,
                     (char*)a.out, a.batch, a.hq, a.hkv, (int)n_rg, a.hkv >= 4 ? 1 : 0, a.c, a.sc);
  return hipGetLastError();
}

// Waves per workgroup. Several waves split one item's keys (merged in LDS);
// that shortens each item, which matters when there are few items or no
// longest-first order (long items would otherwise finish last). With many
// items, two waves per item stream best (batch 1,024, 8,192 items in
// longest-first order: 1,702 us against 1,717 us with one wave and 1,754 us
// with four).
inline int waves_for(long items, bool ordered) {
  return items >= (ordered ? 1024 : 2048) ? 2 : 4;
}

template <int D, int kPaged, bool kScatter>
hipError_t launch_bf16(const AttnArgs& a, hipStream_t stream) {
  const long rows = (long)a.k_max * (a.hq / a.hkv);
  const int T = rows > 32 ? 2 : 1;
  // More than 64 query rows per KV head possible: four-wave workgroups over
  // 128-row groups, whose waves split the rows (32 each) and share one LDS
  // ring. Past 64 rows the matrix-core work per K/V byte doubles; waves of 32
  // rows fit two per SIMD (LDS and registers), so one wave's softmax overlaps
  // another's products. At batch 1,024 with 80-128 rows per KV head: 2,061 us,
  // against 2,316 us for two waves of 64 rows that each copied every tile.
  if (rows > 64) return launch<D, true, 1, 4, kPaged, kScatter, true>(a, stream);
  const long items = (long)a.batch * a.hkv * ((rows + 32 * T - 1) / (32 * T));
  const int nw = waves_for(items, a.order != nullptr);
  if (T == 2)
    return nw == 2 ? launch<D, true, 2, 2, kPaged, kScatter>(a, stream)
                   : launch<D, true, 2, 4, kPaged, kScatter>(a, stream);
  return nw == 2 ? launch<D, true, 1, 2, kPaged, kScatter>(a, stream)
                 : launch<D, true, 1, 4, kPaged, kScatter>(a, stream);
}

// Shared by the contiguous and paged entry points, with and without the fused scatter.
template <int kPaged, bool kScatter = false>
int attention(const AttnArgs& a, int head_dim, bte_dtype dtype, hipStream_t stream) {
  hipError_t e;
  if (dtype == BTE_BF16)
    e = head_dim == 128 ? launch_bf16<128, kPaged, kScatter>(a, stream)
                        : launch_bf16<64, kPaged, kScatter>(a, stream);
  else  // fp32 operands take twice the registers: 32 query rows per workgroup only
    e = head_dim == 128 ? launch<128, false, 1, 4, kPaged, kScatter>(a, stream)
                        : launch<64, false, 1, 4, kPaged, kScatter>(a, stream);
  if (e == hipErrorInvalidValue) return BTE_ERR_DIM;
  return e == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

// Descending-work processing order. Work is the KV length, or with the kept
// counts the length times the 64-row query passes over the keys (a key-split
// wave holds 64 query rows; past 64 rows per KV head the query split's
// matrix-core work per key tile doubles). Sequence i's key is (work
// descending, index ascending) packed in 64 bits, so keys are distinct and the
// position of sequence i in the order is the number of keys below its own. A wave ranks
// kOrderPerWave sequences: its lanes take every 64th key (read straight from
// kv_len, a few KB that stay in L2) and compare it with each of them, then the
// counts are summed over the wave. A one-workgroup bitonic sort took 13 us at
// a batch of 1,024, a thread per sequence over all keys 26 us.
constexpr int kOrderThreads = 256;
constexpr int kOrderPerWave = 8;
constexpr int kOrderPerBlock = kOrderThreads / kWave * kOrderPerWave;
constexpr int kOrderMax = 16384;
// Keys per lane and pass: 16 for the length order (one pass up to a batch of
// 1,024: 4.4 against 5.9 us at 1,024, 7.4 against 13.4 us at 4,096), 8 when
// each key also reads a count (16 measured no faster there, and slower at 256).
template <bool kWork>
constexpr int kOrderKeys = kWork ? 8 : 16;

constexpr int kPassRows = 64;

// The loads are unconditional (index clamped into the batch) so that several
// can be in flight at once; positions past the batch get the padding key ~0,
// above every real key. Work saturates at 2^32 - 1.
template <bool kWork>
__device__ __forceinline__ uint64_t order_key(const int32_t* kv_len, const int32_t* count,
                                              int group, int i, int batch) {
  const int c = min(i, batch - 1);
  uint64_t work = (uint32_t)max(kv_len[c], 0);
  if constexpr (kWork) {
    const uint64_t rows = (uint64_t)(uint32_t)max(count[c], 0) * (uint32_t)group;
    const uint64_t passes = (rows + kPassRows - 1) / kPassRows;   // < 2^57
    work = passes > 0xffffffffull ? (work ? 0xffffffffull : 0ull)
                                  : min(work * passes, 0xffffffffull);   // < 2^63 before the cap
  }
  return i < batch ? ((uint64_t)(0xffffffffu - (uint32_t)work) << 32) | (uint32_t)i : ~0ull;
}

template <bool kWork>
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t* __restrict__ kv_len,
                                                             const int32_t* __restrict__ count,
                                                             int group, int batch,
                                                             int32_t* __restrict__ order) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i0 = blockIdx.x * kOrderPerBlock + (int)(threadIdx.x / kWave) * kOrderPerWave;
  if (i0 >= batch) return;                        // wave-uniform
  uint64_t mine[kOrderPerWave];
  int cnt[kOrderPerWave];
#pragma unroll
  for (int e = 0; e < kOrderPerWave; ++e) {
    mine[e] = order_key<kWork>(kv_len, count, group, i0 + e, batch);
    cnt[e] = 0;
  }
  // kOrderKeys keys per lane and pass, loaded together (one L2 round trip per
  // pass).
  constexpr int kKeys = kOrderKeys<kWork>;
  for (int j0 = lane; j0 < batch; j0 += kKeys * kWave) {
    uint64_t kj[kKeys];
#pragma unroll
    for (int u = 0; u < kKeys; ++u)
      kj[u] = order_key<kWork>(kv_len, count, group, j0 + u * kWave, batch);
#pragma unroll
    for (int u = 0; u < kKeys; ++u)
#pragma unroll
      for (int e = 0; e < kOrderPerWave; ++e) cnt[e] += kj[u] < mine[e] ? 1 : 0;
  }
#pragma unroll
  for (int e = 0; e < kOrderPerWave; ++e) {
#pragma unroll
    for (int x = kWave / 2; x > 0; x >>= 1) cnt[e] += __shfl_xor(cnt[e], x, kWave);
    if (lane == 0 && i0 + e < batch) order[cnt[e]] = i0 + e;
  }
}

}  // namespace
}  // namespace bte

extern "C" int bte_attention_order(const int32_t* kv_len, const int32_t* count, int group,
                                   int batch, int32_t* order_out, hipStream_t stream) {
  using namespace bte;
  if (!kv_len || !order_out) return BTE_ERR_NULL;
  if (batch <= 0 || batch > kOrderMax) return BTE_ERR_DIM;
  if (count && group <= 0) return BTE_ERR_DIM;
  const dim3 grid((batch + kOrderPerBlock - 1) / kOrderPerBlock);
  if (count)
    hipLaunchKernelGGL(order_kernel<true>, grid, dim3(kOrderThreads), 0, stream, kv_len, count,
                       group, batch, order_out);
  else
    hipLaunchKernelGGL(order_kernel<false>, grid, dim3(kOrderThreads), 0, stream, kv_len, count,
                       group, batch, order_out);
  return hipGetLastError() == hipSuccess ? BTE_OK : BTE_ERR_LAUNCH;
}

// Host-side checks common to both attention entry points.
static int attention_args_ok(const void* q, const int32_t* count, const int32_t* cu,
                             const void* cache_k, const void* cache_v, const int32_t* kv_len,
                             const void* out, int batch, int k_max, int hq, int hkv, int head_dim,
                             float scale, bte_dtype dtype) {
  using namespace bte;
  if (!q || !count || !cu || !cache_k || !cache_v || !kv_len || !out) return BTE_ERR_NULL;
  if (batch <= 0 || k_max < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return BTE_ERR_DIM;
  if (!(scale > 0.f) || !isfinite(scale)) return BTE_ERR_DIM;
  if (head_dim != 64 && head_dim != 128) return BTE_ERR_UNSUPPORTED;
  if (dtype != BTE_F32 && dtype != BTE_BF16) return BTE_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(cache_k) || !aligned16(cache_v) || !aligned16(out))
    return BTE_ERR_ALIGN;
  // one sequence's output rows are stored through a buffer resource of < 2^31 bytes
  if ((long long)k_max * hq * head_dim * (dtype == BTE_BF16 ? 2 : 4) > 0x7fffffffLL)
    return BTE_ERR_DIM;
  return BTE_OK;
}

extern "C" int bte_reduced_attention(const void* q, const int32_t* count, const int32_t* cu,
                                     const void* cache_k, const void* cache_v,
                                     const int64_t* seq_start, const int32_t* kv_len,
                                     const int32_t* order, void* out, int batch, int k_max, int hq,
                                     int hkv, int head_dim, float scale, bte_dtype dtype,
                                     hipStream_t stream) {
  using namespace bte;
  if (!seq_start) return BTE_ERR_NULL;
  const int st = attention_args_ok(q, count, cu, cache_k, cache_v, kv_len, out, batch, k_max, hq,
                                   hkv, head_dim, scale, dtype);
  if (st != BTE_OK || k_max == 0) return st;
  const AttnArgs a{q, count, cu, cache_k, cache_v, KvMap{seq_start, nullptr, 0, 0}, kv_len, order,
                   out, batch, k_max, hq, hkv, scale * kLog2e, {}};
  return attention<kContig>(a, head_dim, dtype, stream);
}

extern "C" int bte_reduced_attention_paged(const void* q, const int32_t* count, const int32_t* cu,
                                           const void* cache_k, const void* cache_v,
                                           const int32_t* block_table, int max_pages,
                                           int page_size, const int32_t* kv_len,
                                           const int32_t* order, void* out, int batch, int k_max,
                                           int hq, int hkv, int head_dim, float scale,
                                           bte_dtype dtype, hipStream_t stream) {
  using namespace bte;
  if (!block_table) return BTE_ERR_NULL;
  const int st = attention_args_ok(q, count, cu, cache_k, cache_v, kv_len, out, batch, k_max, hq,
                                   hkv, head_dim, scale, dtype);
  if (st != BTE_OK) return st;
  if (max_pages <= 0) return BTE_ERR_DIM;
  if (page_size < 8 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return BTE_ERR_UNSUPPORTED;
  if (k_max == 0) return BTE_OK;
  int lg = 0;
  while ((1 << lg) < page_size) ++lg;
  const AttnArgs a{q, count, cu, cache_k, cache_v, KvMap{nullptr, block_table, max_pages, lg},
                   kv_len, order, out, batch, k_max, hq, hkv, scale * kLog2e, {}};
  if (max_pages > kPageCache) return attention<kPagedMem>(a, head_dim, dtype, stream);
  return lg >= 5 ? attention<kPagedBig>(a, head_dim, dtype, stream)
                 : attention<kPagedLds>(a, head_dim, dtype, stream);
}

// Host-side checks of the fused scatter's own arguments.
static int scatter_args_ok(const int32_t* idx, int n, const int32_t* pos_base, const void* new_k,
                           const void* new_v) {
  using namespace bte;
  if (!idx || !pos_base || !new_k || !new_v) return BTE_ERR_NULL;
  if (n <= 0) return BTE_ERR_DIM;
  if (n > kScatterSpan) return BTE_ERR_UNSUPPORTED;
  if (!aligned16(new_k) || !aligned16(new_v)) return BTE_ERR_ALIGN;
  return BTE_OK;
}

extern "C" int bte_kv_scatter_attention(const void* q, const int32_t* count, const int32_t* cu,
                                        const int32_t* idx, int n, const int32_t* pos_base,
                                        const void* new_k, const void* new_v, void* cache_k,
                                        void* cache_v, const int64_t* seq_start,
                                        const int32_t* kv_len, const int32_t* order, void* out,
                                        int batch, int k_max, int hq, int hkv, int head_dim,
                                        float scale, bte_dtype dtype, hipStream_t stream) {
  using namespace bte;
  if (!seq_start) return BTE_ERR_NULL;
  int st = attention_args_ok(q, count, cu, cache_k, cache_v, kv_len, out, batch, k_max, hq, hkv,
                             head_dim, scale, dtype);
  if (st == BTE_OK) st = scatter_args_ok(idx, n, pos_base, new_k, new_v);
  if (st != BTE_OK || k_max == 0) return st;
  AttnArgs a{q, count, cu, cache_k, cache_v, KvMap{seq_start, nullptr, 0, 0}, kv_len, order,
             out, batch, k_max, hq, hkv, scale * kLog2e, {}};
  a.sc = KvScatter{(const char*)new_k, (const char*)new_v, idx, pos_base, (char*)cache_k,
                   (char*)cache_v, n, k_max};
  return attention<kContig, true>(a, head_dim, dtype, stream);
}

extern "C" int bte_kv_scatter_attention_paged(
    const void* q, const int32_t* count, const int32_t* cu, const int32_t* idx, int n,
    const int32_t* pos_base, const void* new_k, const void* new_v, void* cache_k, void* cache_v,
    const int32_t* block_table, int max_pages, int page_size, const int32_t* kv_len,
    const int32_t* order, void* out, int batch, int k_max, int hq, int hkv, int head_dim,
    float scale, bte_dtype dtype, hipStream_t stream) {
  using namespace bte;
  if (!block_table) return BTE_ERR_NULL;
  int st = attention_args_ok(q, count, cu, cache_k, cache_v, kv_len, out, batch, k_max, hq, hkv,
                             head_dim, scale, dtype);
  if (st == BTE_OK) st = scatter_args_ok(idx, n, pos_base, new_k, new_v);
  if (st != BTE_OK) return st;
  if (max_pages <= 0) return BTE_ERR_DIM;
  if (page_size < 8 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return BTE_ERR_UNSUPPORTED;
  if (k_max == 0) return BTE_OK;
  int lg = 0;
  while ((1 << lg) < page_size) ++lg;
  AttnArgs a{q, count, cu, cache_k, cache_v, KvMap{nullptr, block_table, max_pages, lg}, kv_len,
             order, out, batch, k_max, hq, hkv, scale * kLog2e, {}};
  a.sc = KvScatter{(const char*)new_k, (const char*)new_v, idx, pos_base, (char*)cache_k,
                   (char*)cache_v, n, k_max};
  if (max_pages > kPageCache) return attention<kPagedMem, true>(a, head_dim, dtype, stream);
  return lg >= 5 ? attention<kPagedBig, true>(a, head_dim, dtype, stream)
                 : attention<kPagedLds, true>(a, head_dim, dtype, stream);
}
