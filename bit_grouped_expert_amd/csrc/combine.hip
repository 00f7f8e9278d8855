// Weighted combine of the routed experts' outputs with the shared expert's.
//
// out[t] = bf16( S[t] + sum_j w[t, j] * Y[slot_row[t*k + j]] ), summed in fp32
// in slot order.  The pages (MarkTechPost, "Perplexity open sources Lily, a Rust +
// Metal inference engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph
// 4) name the shared expert that sees every token; applying the routing weight
// after the down projection and giving the shared expert unit weight are
// readings.  The kernel streams Y once with 128-bit loads: one workgroup per
// (token, 2048-column slice), eight columns per thread, up to eight slots' rows in
// flight.
#include "common.h"
#include "internal.h"

namespace moeq4 {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Y,
                                                      int64_t y_rows,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ S,
                                                      uint16_t* __restrict__ out, int D, int k) {
  const int t = blockIdx.x;
  const int d0 = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (d0 >= D) return;
  float acc[8];
  if (S) {
    const u32x4_t v = *(const u32x4_t*)(S + (int64_t)t * D + d0);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      acc[2 * h] = bf16lo_to_f32(v[h]);
      acc[2 * h + 1] = bf16hi_to_f32(v[h]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  }
  // slots in batches of eight: every row of a batch is loaded before any is added (in
  // slot order), so that eight loads are in flight
  for (int j0 = 0; j0 < k; j0 += 8) {
    u32x4_t v[8];
    float wj[8];
    bool okj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      const int32_t r = j < k ? slot_row[(int64_t)t * k + j] : -1;
      const bool ok = r >= 0 && r < y_rows;
      okj[u] = ok;
      wj[u] = ok ? w[(int64_t)t * k + j] : 0.f;
      v[u] = ok ? *(const u32x4_t*)(Y + (int64_t)r * D + d0) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (okj[u]) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] = fmaf(wj[u], bf16lo_to_f32(v[u][h]), acc[2 * h]);
          acc[2 * h + 1] = fmaf(wj[u], bf16hi_to_f32(v[u][h]), acc[2 * h + 1]);
        }
      }
    }
  }
  u32x4_t o;
#pragma unroll
  for (int h = 0; h < 4; ++h) o[h] = pack_bf16x2(acc[2 * h], acc[2 * h + 1]);
  *(u32x4_t*)(out + (int64_t)t * D + d0) = o;
}

void launch_combine(const uint16_t* Y, int64_t y_rows, const int32_t* slot_row, const float* w,
                    const uint16_t* S, uint16_t* out, int T, int D, int k, hipStream_t s) {
  dim3 grid(T, (D + 2047) / 2048), block(256);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, s, Y, y_rows, slot_row, w, S, out, D, k);
}

}  // namespace moeq4
