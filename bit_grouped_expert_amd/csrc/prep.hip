// The prepared copy of an activation matrix read by the resident-tile and wide-tile
// grouped GEMM engines.  A packed word of eight 4-bit codes unpacks (one AND-OR per
// pair of codes) into the k order 0,4,1,5,2,6,3,7, so every run of eight activation
// columns is stored in that order; the matrix-core operands of both sides then line up
// without any per-element shuffle inside the GEMM.  One zero row follows the last:
// gathered rows whose index falls outside [0, rows) read it.
#include "common.h"
#include "internal.h"

namespace moeq4 {

namespace {

// One wavefront per row; lane l copies the 16-byte chunks l, l + 64, ... of the row.
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ A, int rows, int K,
                                                   uint16_t* __restrict__ Ap) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (r > rows) return;  // row `rows` is the zero row
  const int nch = K >> 3;
  for (int c = l; c < nch; c += 64) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < rows) v = *(const u32x4_t*)(A + (int64_t)r * K + 8 * c);
    *(u32x4_t*)(Ap + (int64_t)r * K + 8 * c) = interleave8(v);
  }
}

}  // namespace

void launch_prep(const uint16_t* A, int rows, int K, uint16_t* Ap, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, dim3((rows + 1 + 3) / 4), dim3(256), 0, s, A, rows, K, Ap);
}

}  // namespace moeq4
