// Shared device helpers of the matrix-core attention kernels (forward and
// backward): the bf16 operand types, the geometry and XOR swizzle of a
// 32-row LDS tile, the asynchronous global-to-LDS copy, and the wave-wide
// search of a sorted position table.  Header-only; every function inlines.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cpa {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int BN = 32;         // rows of one LDS tile (keys, or queries in the dK/dV pass)

template <int D>
struct Geo {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;  // one K or V tile
  static constexpr int KK = D / 16;                  // MFMA k-steps over d
  static constexpr int DB = D / 32;                  // 32-wide d blocks of O^T
  static_assert(TILE_BYTES % 1024 == 0, "a tile is a whole number of 1 KB copy instructions");
};

// Zigzag layout, closed form: rank r of nblk holds chunk r, then chunk
// 2nblk-1-r, C rows each.  Its local row u is global row (and position)
// zig_pos(r, u); zig_count_le counts its rows at positions <= x.
__device__ __forceinline__ int64_t zig_pos(int r, int64_t u, int64_t C, int nblk) {
  return u < C ? (int64_t)r * C + u : (int64_t)(2 * nblk - 1 - r) * C + (u - C);
}
__device__ __forceinline__ int64_t zig_count_le(int r, int nblk, int64_t C, int64_t x) {
  const int64_t lo = x - (int64_t)r * C + 1;
  const int64_t hi = x - (int64_t)(2 * nblk - 1 - r) * C + 1;
  return (lo < 0 ? 0 : (lo > C ? C : lo)) + (hi < 0 ? 0 : (hi > C ? C : hi));
}

// Number of entries <= x in the increasing array off[0, n); wave-cooperative
// 64-way search (every lane returns the same value).
__device__ inline int64_t count_le(const int64_t* __restrict__ off, int64_t n, int64_t x) {
  const int lane = threadIdx.x & 63;
  int64_t lo = 0, hi = n;
  while (hi - lo > 64) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t idx = lo + lane * step;
    const bool p = idx < hi && off[idx] <= x;
    const int c = __popcll(__ballot(p));
    if (c == 0) return lo;
    const int64_t nlo = lo + (int64_t)(c - 1) * step + 1;
    const int64_t probe_c = lo + (int64_t)c * step;
    hi = probe_c < hi ? probe_c : hi;
    lo = nlo;
  }
  const int64_t idx = lo + lane;
  const bool p = idx < hi && off[idx] <= x;
  return lo + __popcll(__ballot(p));
}

// Two floats rounded to bf16 (nearest even) and packed, lo in bits 0-15, as
// one v_cvt_pk_bf16_f32.  The empty asm makes the packed word opaque: without
// it the compiler rewrites later shifts and masks of the word into separate
// single-element conversions.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const bf16x2 pr = {(__bf16)lo, (__bf16)hi};
  uint32_t w = __builtin_bit_cast(uint32_t, pr);
  asm("" : "+v"(w));
  return w;
}

__device__ __forceinline__ float xhalf_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
// Inline asm: the instruction has no register result, and hiding it from the
// compiler keeps it from making unrelated LDS reads wait for it; completion is
// awaited explicitly (vmcnt) before the barrier that publishes the tile.
// `sbase` must be uniform across the wave; it is read from the first lane so
// that it always lands in SGPRs, whatever the compiler inferred.
__device__ __forceinline__ void copy16_saddr(uint32_t voff, const void* sbase, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const void* sb = (const void*)(uintptr_t)((hi << 32) | lo);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void copy16_vaddr(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order, so every older copy has landed).
template <int N>
__device__ __forceinline__ void wait_copies_but() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }


}  // namespace tile
}  // namespace cpa
