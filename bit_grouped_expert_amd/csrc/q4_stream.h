// Device helpers of the 4-bit weight streams shared by the grouped GEMM engines that
// feed 128 + q to the matrix cores (resident-tile, tiled and wide-tile engines).
#pragma once

#include "common.h"

namespace moeq4 {

constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kNib = 0x000F000Fu;
constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 pair (1, 1)

// kMagic in a VGPR the compiler cannot constant-fold, so that (v & mask) | magic is
// one v_and_or_b32; only VALU instructions read it.
__device__ __forceinline__ uint32_t opaque_magic() {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "n"(kMagic));
  return v;
}

__device__ __forceinline__ u32x4_t unpack_word(uint32_t w, uint32_t magic) {
  u32x4_t b;
  b[0] = (w & kNib) | magic;
  b[1] = ((w >> 4) & kNib) | magic;
  b[2] = ((w >> 8) & kNib) | magic;
  b[3] = ((w >> 12) & kNib) | magic;
  return b;
}

template <typename T>
__device__ __forceinline__ T ld(const void* base, uint32_t byte_off) {
  return *(const T*)((const char*)base + byte_off);
}

// natural column c (0..7) of an 8-column run -> its position in the order 0,4,1,5,...
__device__ __forceinline__ int perm8(int c) { return ((c & 3) << 1) | (c >> 2); }

// Weights of one 256-K stage for one lane: for each of its two fragment rows and each
// 128-K half, the packed words 4q .. 4q+3 (one 16-byte load), and the scales and
// biases of the stage's four groups (8 bytes each).
struct StageW {
  u32x4_t c[2][2];  // [fragment][half]
  u32x2_t s[2], b[2];
};

// The two permlane32 swaps (word 0 <-> 2, word 1 <-> 3 between lanes l and l ^ 32) of a
// lane's word quad.  Before them quarter q holds words 4q .. 4q+3 of a 128-K half; after
// them MFMA steps 0, 1 draw every quarter's word from one scale group and steps 2, 3
// from the other.  The word a lane holds in each step is tracked by applying the same
// swaps to the word numbers, so nothing depends on the swap's direction.
__device__ __forceinline__ u32x4_t swap_quad(u32x4_t v) {
  const auto r0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  u32x4_t o;
  o[0] = r0[0];
  o[1] = r1[0];
  o[2] = r0[1];
  o[3] = r1[1];
  return o;
}

}  // namespace moeq4
