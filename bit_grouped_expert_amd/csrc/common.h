// Device helpers shared by the gfx950 kernels of the int4-g64 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA bf16 operand (8 per lane)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;      // 16x16 MFMA accumulator (4 per lane)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWave = 64;
constexpr int kGroup = 64;   // weights per (scale, bias) pair

// bf16 bits (low 16 bits of `b`) -> fp32, exact.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
// bf16 bits in the high 16 bits of `b` -> fp32, exact.
__device__ __forceinline__ float bf16hi_to_f32(uint32_t b) { return __uint_as_float(b & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 8 bf16 values (x0..x7, two per dword) -> the order x0,x4,x1,x5,x2,x6,x3,x7, in which
// a packed word of eight 4-bit codes unpacks.
__device__ __forceinline__ u32x4_t interleave8(u32x4_t d) {
  u32x4_t o;
  o[0] = (d[0] & 0xFFFFu) | (d[2] << 16);
  o[1] = (d[0] >> 16) | (d[2] & 0xFFFF0000u);
  o[2] = (d[1] & 0xFFFFu) | (d[3] << 16);
  o[3] = (d[1] >> 16) | (d[3] & 0xFFFF0000u);
  return o;
}

// Butterfly exchange with the lane `lane ^ mask` (ds_bpermute based).
__device__ __forceinline__ uint32_t xor_u32(uint32_t v, int mask) {
  int src = (lane_id() ^ mask) << 2;
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v);
}
__device__ __forceinline__ uint64_t xor_u64(uint64_t v, int mask) {
  uint32_t lo = xor_u32((uint32_t)v, mask), hi = xor_u32((uint32_t)(v >> 32), mask);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double xor_f64(double v, int mask) {
  return __longlong_as_double((long long)xor_u64((uint64_t)__double_as_longlong(v), mask));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Sum over the wave in a fixed butterfly order (every lane gets the same bits).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_f64(v, m);
  return v;
}

__device__ __forceinline__ uint32_t ldg_u32(const void* p) {
  return __builtin_nontemporal_load((const uint32_t*)p);
}

// s_waitcnt vmcnt(0) with the other counters unconstrained, fenced against reordering
__device__ __forceinline__ void wait_vmcnt0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS traffic: waits for this wavefront's LDS operations only, not
// for its in-flight global loads (__syncthreads() is a workgroup fence as well, and waits
// for every outstanding vector-memory operation, so a prefetch issued before it is drained
// at the barrier).  Enough wherever the barrier orders LDS accesses between the
// workgroup's threads and no global-memory access of one thread must be seen by another.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Device-scope (agent) accesses, coherent across the XCDs' L2 caches: what one
// workgroup writes this way and another reads this way within one launch is seen once a
// completed store is followed by a counter or flag that the reader observes.
__device__ __forceinline__ int atomic_add_agent(int32_t* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev16(void* p, u32x4_t v) {
  __hip_atomic_store((uint64_t*)p, (uint64_t)v[0] | ((uint64_t)v[1] << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store((uint64_t*)p + 1, (uint64_t)v[2] | ((uint64_t)v[3] << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4_t load_dev16(const void* p) {
  const uint64_t lo = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi =
      __hip_atomic_load((const uint64_t*)p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4_t{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

}  // namespace moeq4
