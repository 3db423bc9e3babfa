// Device-side helpers shared by the gfx950 kernels of libbte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bte.h"

namespace bte {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
// MI355X has 8 XCDs, each with its own L2; workgroup x of a grid is dispatched
// to XCD x % 8.
constexpr int kXcds = 8;

// XCD-grouped work mapping: a grid of ceil(batch / 8) * 8 * per workgroups,
// where workgroup i takes part s < per of sequence b. All parts of sequence b
// run on XCD b % 8, one after another in part order, and every XCD gets every
// eighth sequence. Returns false for the padding past the last sequence.
__device__ __forceinline__ bool xcd_seq_part(int batch, int per, int& b, int& s) {
  const int i = (int)blockIdx.x;
  const int grp = i / (kXcds * per);
  const int j = i - grp * kXcds * per;
  s = j / kXcds;
  b = kXcds * grp + (j - s * kXcds);
  return b < batch;
}
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two float32 -> two bfloat16 (round to nearest even, NaN stays NaN) packed
// into one word, `lo` in bits 15:0: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Streaming (read-once) load: hints the caches not to retain the line. Only
// for fully coalesced accesses; lines that other instructions of the wave still
// have to read must use ld16, or they are evicted before reuse.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Streaming store: the line is written once and not read again by the kernel.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// 32x32 output tile of one MFMA: lane l, register r holds row
// m = 8*(r/4) + 4*(l/32) + r%4 and column n = l%32.
__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Value of `v` held by lane (lane ^ 32) of the wave.
__device__ __forceinline__ float swap_halves(float v) { return __shfl_xor(v, 32, kWave); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS reads for kernels that keep HBM->LDS copies (global_load_lds) in flight.
// The compiler cannot tell which LDS bytes those copies write, so before a plain
// LDS load it waits for every copy in flight (s_waitcnt vmcnt(0)) and the copy
// pipeline drains. These reads are inline asm, which the compiler does not
// track: the kernel's own vmcnt waits must make the data land first, and a
// result may only be used after an asm s_waitcnt lgkmcnt that takes it as an
// in/out operand.
__device__ __forceinline__ u32x4 lds_read16(const void* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a) : "memory");
  return v;
}
// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima, i.e. not waited on. Used to wait for all but
// the newest N HBM->LDS copies of a wave.
constexpr int kVmcntNoLgkm = (0x7 << 4) | (0xF << 8);
constexpr int vmcnt_bits(int n) { return (n & 15) | ((n >> 4) << 14); }
// s_waitcnt immediate waiting for all LDS reads (lgkmcnt 0) and nothing else.
constexpr int kLgkm0 = 0xF | (0x7 << 4) | (0x3 << 14);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace bte
