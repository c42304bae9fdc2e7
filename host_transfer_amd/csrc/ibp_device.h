// ibp_device.h -- device helpers shared by the IBP kernels (gfx950, wave64).
//
// Bit packing without a PEXT/PDEP instruction.  For a 32-bit selector `keep`
// (the non-invariant positions of one word), every kept bit at position p
// moves down by d(p) = number of unselected positions below p.  Writing d in
// binary, the moves are done in five stages of 1, 2, 4, 8 and 16 positions;
// stage s moves the bits whose d has bit s set.  Done in increasing order the
// stages never make two kept bits collide, and each stage is fully described
// by one "move mask" of the bits it moves (their positions before the stage).
// Expanding runs the stages backwards with the same masks.  This is the
// compress/expand construction of H. S. Warren, "Hacker's Delight", 2nd ed.,
// sections 7-4 and 7-5; the masks depend only on the Mask metadata, so they
// are computed once per kernel and each word then costs two operations per
// stage (a shift and a bit-field insert, v_bfi_b32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ibp {

constexpr int kWave = 64;

// Prefix XOR from bit 0 upwards: bit p of the result is the XOR of bits 0..p.
__host__ __device__ __forceinline__ uint32_t prefix_xor(uint32_t y) {
  y ^= y << 1;
  y ^= y << 2;
  y ^= y << 4;
  y ^= y << 8;
  y ^= y << 16;
  return y;
}

// Move masks of the five stages for selector `keep` (see the file header).
// `below` marks, at position p, an unselected position at p - 1; the parity
// of the unselected positions below each bit is then prefix_xor(below).
__host__ __device__ __forceinline__ void move_masks(uint32_t keep, uint32_t mv[5]) {
  uint32_t below = ~keep << 1;
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const uint32_t odd = prefix_xor(below);  // bit s of d(p) for every p
    const uint32_t moving = odd & keep;      // kept bits that move 2^s now
    mv[s] = moving;
    keep = (keep ^ moving) | (moving >> (1u << s));
    below &= ~odd;                           // halve the remaining distances
  }
}

// Bit-field insert: bits of `a` where m is set, bits of `b` elsewhere.
__host__ __device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  return (a & m) | (b & ~m);
}

// Packs the bits of x selected by `keep` into the low popcount(keep) bits.
__host__ __device__ __forceinline__ uint32_t pack_bits(uint32_t x, uint32_t keep, const uint32_t mv[5]) {
  x &= keep;
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const uint32_t t = x & mv[s];
    x = (x ^ t) | (t >> (1u << s));
  }
  return x;
}

// Inverse of pack_bits on the selected positions; the other positions hold
// leftovers and must be masked by the caller.  Bits of x above popcount(keep)
// never reach a selected position.
__host__ __device__ __forceinline__ uint32_t unpack_bits(uint32_t x, const uint32_t mv[5]) {
  x = bfi(mv[4], x << 16, x);
  x = bfi(mv[3], x << 8, x);
  x = bfi(mv[2], x << 4, x);
  x = bfi(mv[1], x << 2, x);
  x = bfi(mv[0], x << 1, x);
  return x;
}

// One v_bfi_b32 (left to itself the compiler splits the insert into four
// operations once several stages are chained).
__device__ __forceinline__ uint32_t bfi_op(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

// unpack_bits restricted to the stages set in `stages` (bit s = stage of
// 2^s positions).  `stages` must be uniform across the wave: a stage whose
// move mask is zero on every lane leaves x unchanged and is skipped.
__device__ __forceinline__ uint32_t unpack_stages(uint32_t x, const uint32_t mv[5],
                                                  uint32_t stages) {
  if (stages & 16u) x = bfi_op(mv[4], x << 16, x);
  if (stages & 8u) x = bfi_op(mv[3], x << 8, x);
  if (stages & 4u) x = bfi_op(mv[2], x << 4, x);
  if (stages & 2u) x = bfi_op(mv[1], x << 2, x);
  if (stages & 1u) x = bfi_op(mv[0], x << 1, x);
  return x;
}

// 32 bits of the LDS bit stream starting at bit `off` (two words and a funnel
// shift); the word after the last one read must be addressable.
__device__ __forceinline__ uint32_t window32(const uint32_t* pb32, uint32_t off) {
  const uint32_t d0 = pb32[off >> 5];
  const uint32_t d1 = pb32[(off >> 5) + 1];
  return __builtin_amdgcn_alignbit(d1, d0, off & 31u);
}

// Loads through a global-address-space pointer (device memory or mapped
// host memory).  A pointer the compiler cannot place is read with a flat
// instruction, which also counts against the LDS wait counter: every later
// wait for an LDS read would then wait for these loads as well.
// (The pointer goes through an integer: a direct cast of a generic pointer
// still compiles to a flat load.)
__device__ __forceinline__ uint64_t load_global(const uint64_t* p) {
  typedef __attribute__((address_space(1))) const uint64_t global_u64;
  return *(global_u64*)(uintptr_t)p;
}
__device__ __forceinline__ uint4 load_global(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
  const u32x4 v = *(global_u32x4*)(uintptr_t)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// MI355X has 8 XCDs, each with its own L2; workgroups are dispatched to them
// round robin (block b runs on XCD b % 8).  The XCD a row is routed to is
// chosen by a hash of its tensor index (Fibonacci hashing, top 3 bits), so all
// rows of one tensor meet in one L2.
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t xcd_of_tensor(int64_t id) {
  return (uint32_t)(((uint64_t)id * 0x9E3779B97F4A7C15ull) >> 61);
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Lane l's value of v (l wave-uniform).  The builtin returns a signed int:
// going through uint32_t keeps a later widening to 64 bits (an address, a
// row index) from sign-extending it.
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, uint32_t l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)l);
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, uint32_t l) {
  return ((uint64_t)lane_u32((uint32_t)(v >> 32), l) << 32) | (uint64_t)lane_u32((uint32_t)v, l);
}

// Orders LDS accesses among the lanes of one wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const uint32_t l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t u = __shfl_up(v, d, kWave);
    if (l >= (uint32_t)d) v += u;
  }
  return v;
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return __builtin_amdgcn_readfirstlane(v);
}

}  // namespace ibp
