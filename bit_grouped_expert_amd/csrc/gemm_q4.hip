// Grouped GEMM over groupwise-affine 4-bit weights for gfx950 (MI355X).
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
// engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph 5 (4-bit weights,
// every group of 64 sharing a bf16 scale and bias, are reconstructed one tile at
// a time inside the grouped GEMM with FP32 accumulation, so the expanded weights
// never reach memory) and paragraph 6 (tile rows of one expert group; a block
// map drives one launch over uneven groups).  The Metal design there is prior
// art; this kernel is laid out for CDNA4 wavefronts and matrix cores.
//
// Arithmetic.  For one output row m, one weight row n and one 64-wide group g,
//   sum_c x[m,c] (q[n,c] s[n,g] + b[n,g])
//     = s[n,g] * P + (b[n,g] - 128 s[n,g]) * X,
//   P = sum_c x[m,c] (128 + q[n,c]),   X = sum_c x[m,c]   (c over group g).
// 128 + q is exactly the bf16 with bits 0x4300 | q, so a weight word's eight
// codes become four packed bf16 pairs with one AND-OR each (after a shift), and
// P is a plain bf16 matrix-core product with fp32 accumulation (every product
// x * (128 + q) is exact in fp32).  Scale and bias are applied once per group
// in fp32 to the group's partial accumulator.  Nothing is rounded to bf16 but
// the activations already in bf16 and the final output.
//
// Work decomposition.  A workgroup (4 wavefronts) takes one tile of <= 64 rows
// of one group (rows gathered through a row index) and a slice of output
// columns; the activation rows of the tile are staged in LDS in K chunks of
// 512, every wavefront streams its own 32 weight rows straight from HBM into
// registers with 128-bit loads (no LDS for weights), and issues
// v_mfma_f32_16x16x32_bf16 for each 16-row fragment of the tile.
//
// MFMA operand layout (16x16x32 bf16): lane l supplies row (l % 16) of A and
// column (l % 16) of B, each with eight k-slots belonging to quarter l / 16;
// the accumulator holds rows 4*(l/16)+i, column l%16.  Lanes of quarter q load
// words 4q..4q+3 of a 128-K block of their weight row; two permlane32 swaps
// regroup them so that each MFMA step's four quarters hold words of one 64-wide
// scale group.  The A fragment of each lane is read from the LDS column of the
// word it ended up with; that word index is tracked by applying the same swaps
// to the lanes' word numbers, so the pairing of A and B never depends on how
// the swap moves data.  Within an 8-element k-slot the codes come out in the
// order 0,4,1,5,2,6,3,7, and the LDS copy of the activations is stored in that
// same order.
#include "common.h"
#include "internal.h"

namespace moeq4 {

constexpr int KC = 512;         // K chunk staged in LDS
constexpr int LDA = KC + 8;     // LDS row stride in bf16 (16-byte pad against bank conflicts)
constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kMask = 0x000F000Fu;

// One packed word of eight codes -> MFMA operand holding 128 + q in the order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ u32x4_t unpack_word(uint32_t w) {
  u32x4_t b;
  b[0] = (w & kMask) | kMagic;
  b[1] = ((w >> 4) & kMask) | kMagic;
  b[2] = ((w >> 8) & kMask) | kMagic;
  b[3] = ((w >> 12) & kMask) | kMagic;
  return b;
}

__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

template <int NF, bool SWIGLU>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int g, int row0, int nrows,
                                          int slice, uint16_t* __restrict__ As,
                                          float* __restrict__ Xs) {
  constexpr int NR = NF * 16;  // rows staged
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int m = l & 15, q = l >> 4;
  const int N = p.N, K = p.K;
  const int KW = K >> 3;        // words per weight row
  const int KG = K >> 6;        // scale groups per weight row

  // columns of this wavefront
  int nrow0, nrow1, col0;
  bool active;
  if (SWIGLU) {
    const int F = N >> 1;
    col0 = slice * 64 + wave * 16;
    active = col0 < F;
    nrow0 = col0 + m;           // gate row
    nrow1 = F + col0 + m;       // up row
  } else {
    col0 = slice * 128 + wave * 32;
    active = col0 < N;
    nrow0 = col0 + m;
    nrow1 = col0 + 16 + m;
  }
  if (!active) nrow0 = nrow1 = 0;

  const bool in_main = g < p.n_main;
  const int gi = in_main ? g : 0;
  const uint32_t* qb = (in_main ? p.main.q : p.last.q) + (int64_t)gi * N * KW;
  const uint16_t* sb = (in_main ? p.main.s : p.last.s) + (int64_t)gi * N * KG;
  const uint16_t* bb = (in_main ? p.main.b : p.last.b) + (int64_t)gi * N * KG;
  const uint32_t* q0 = qb + (int64_t)nrow0 * KW;
  const uint32_t* q1 = qb + (int64_t)nrow1 * KW;
  const uint16_t* s0p = sb + (int64_t)nrow0 * KG;
  const uint16_t* s1p = sb + (int64_t)nrow1 * KG;
  const uint16_t* b0p = bb + (int64_t)nrow0 * KG;
  const uint16_t* b1p = bb + (int64_t)nrow1 * KG;
  const bool s_dword = (KG & 1) == 0;

  // word each lane holds in MFMA step s of a 128-K block (after the swaps)
  uint32_t widx[4] = {(uint32_t)(4 * q), (uint32_t)(4 * q + 1), (uint32_t)(4 * q + 2),
                      (uint32_t)(4 * q + 3)};
  swap32(widx[0], widx[2]);
  swap32(widx[1], widx[3]);

  f32x4_t acc[2][NF];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[nb][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < K; kc += KC) {
    const int kcl = min(KC, K - kc);
    const int cpr = kcl >> 3;  // 16-byte chunks per row
    __syncthreads();
    // ---- stage the tile's activation rows for this K chunk
    for (int u = tid; u < NR * cpr; u += 256) {
      const int r = u / cpr, cu = u - r * cpr;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (r < nrows) {
        const int gr = row0 + r;
        const int ar = p.a_row_index ? p.a_row_index[gr] : gr;
        if (ar >= 0 && ar < p.a_rows)
          v = *(const u32x4_t*)(p.A + (int64_t)ar * K + kc + cu * 8);
      }
      *(u32x4_t*)(As + r * LDA + cu * 8) = interleave8(v);
    }
    __syncthreads();
    // ---- per-group row sums of the activations
    const int ng = kcl >> 6;
    for (int u = tid; u < ng * NR; u += 256) {
      const int gl = u / NR, r = u - gl * NR;
      const u32x4_t* src = (const u32x4_t*)(As + r * LDA + gl * 64);
      float sum = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4_t v = src[c];
#pragma unroll
        for (int h = 0; h < 4; ++h) sum += bf16lo_to_f32(v[h]) + bf16hi_to_f32(v[h]);
      }
      Xs[gl * NR + r] = sum;
    }
    __syncthreads();
    if (!active) continue;

    // ---- 128-K blocks
    int kb = 0;
    for (; kb + 128 <= kcl; kb += 128) {
      const int wo = (kc + kb) >> 3;   // word offset of the block
      const int go = (kc + kb) >> 6;   // scale-group offset of the block
      u32x4_t c0 = *(const u32x4_t*)(q0 + wo + 4 * q);
      u32x4_t c1 = *(const u32x4_t*)(q1 + wo + 4 * q);
      uint32_t sw0, sw1, bw0, bw1;
      if (s_dword) {
        sw0 = *(const uint32_t*)(s0p + go);
        sw1 = *(const uint32_t*)(s1p + go);
        bw0 = *(const uint32_t*)(b0p + go);
        bw1 = *(const uint32_t*)(b1p + go);
      } else {
        sw0 = s0p[go] | ((uint32_t)s0p[go + 1] << 16);
        sw1 = s1p[go] | ((uint32_t)s1p[go + 1] << 16);
        bw0 = b0p[go] | ((uint32_t)b0p[go + 1] << 16);
        bw1 = b1p[go] | ((uint32_t)b1p[go + 1] << 16);
      }
      uint32_t w0[4] = {c0[0], c0[1], c0[2], c0[3]};
      uint32_t w1[4] = {c1[0], c1[1], c1[2], c1[3]};
      swap32(w0[0], w0[2]);
      swap32(w0[1], w0[3]);
      swap32(w1[0], w1[2]);
      swap32(w1[1], w1[3]);
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        f32x4_t P[2][NF];
#pragma unroll
        for (int st = 2 * grp; st < 2 * grp + 2; ++st) {
          const u32x4_t B0 = unpack_word(w0[st]);
          const u32x4_t B1 = unpack_word(w1[st]);
          const int acol = kb + 8 * (int)widx[st];
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const u32x4_t a = *(const u32x4_t*)(As + (f * 16 + m) * LDA + acol);
            if (st == 2 * grp) {
              P[0][f] = mfma16x16x32(a, B0, f32x4_t{0.f, 0.f, 0.f, 0.f});
              P[1][f] = mfma16x16x32(a, B1, f32x4_t{0.f, 0.f, 0.f, 0.f});
            } else {
              P[0][f] = mfma16x16x32(a, B0, P[0][f]);
              P[1][f] = mfma16x16x32(a, B1, P[1][f]);
            }
          }
        }
        // scale group of these two steps (words 0..7 -> first, 8..15 -> second), read off
        // the tracked word index so it never depends on the swap's direction
        const int gsel = __builtin_amdgcn_readfirstlane((int)(widx[2 * grp] >> 3));
        const float s0 = gsel ? bf16hi_to_f32(sw0) : bf16lo_to_f32(sw0);
        const float s1 = gsel ? bf16hi_to_f32(sw1) : bf16lo_to_f32(sw1);
        const float bp0 = fmaf(-128.f, s0, gsel ? bf16hi_to_f32(bw0) : bf16lo_to_f32(bw0));
        const float bp1 = fmaf(-128.f, s1, gsel ? bf16hi_to_f32(bw1) : bf16lo_to_f32(bw1));
        const int gl = (kb >> 6) + gsel;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const f32x4_t X = *(const f32x4_t*)(Xs + gl * NR + f * 16 + 4 * q);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[0][f][i] = fmaf(s0, P[0][f][i], fmaf(bp0, X[i], acc[0][f][i]));
            acc[1][f][i] = fmaf(s1, P[1][f][i], fmaf(bp1, X[i], acc[1][f][i]));
          }
        }
      }
    }
    // ---- a trailing 64-K block (K % 128 == 64): lanes of quarter q hold words 2q, 2q+1
    if (kb < kcl) {
      const int wo = (kc + kb) >> 3;
      const int go = (kc + kb) >> 6;
      const u32x2_t c0 = *(const u32x2_t*)(q0 + wo + 2 * q);
      const u32x2_t c1 = *(const u32x2_t*)(q1 + wo + 2 * q);
      f32x4_t P[2][NF];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4_t B0 = unpack_word(c0[st]);
        const u32x4_t B1 = unpack_word(c1[st]);
        const int acol = kb + 8 * (2 * q + st);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const u32x4_t a = *(const u32x4_t*)(As + (f * 16 + m) * LDA + acol);
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          P[0][f] = mfma16x16x32(a, B0, st ? P[0][f] : z);
          P[1][f] = mfma16x16x32(a, B1, st ? P[1][f] : z);
        }
      }
      const float s0 = bf16lo_to_f32(s0p[go]), s1 = bf16lo_to_f32(s1p[go]);
      const float bp0 = fmaf(-128.f, s0, bf16lo_to_f32(b0p[go]));
      const float bp1 = fmaf(-128.f, s1, bf16lo_to_f32(b1p[go]));
      const int gl = kb >> 6;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const f32x4_t X = *(const f32x4_t*)(Xs + gl * NR + f * 16 + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[0][f][i] = fmaf(s0, P[0][f][i], fmaf(bp0, X[i], acc[0][f][i]));
          acc[1][f][i] = fmaf(s1, P[1][f][i], fmaf(bp1, X[i], acc[1][f][i]));
        }
      }
    }
  }

  if (!active) return;
  // ---- epilogue and store (rows beyond the tile are not written)
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = f * 16 + 4 * q + i;
      if (r >= nrows) continue;
      uint16_t* crow = p.C + (int64_t)(row0 + r) * p.ldc;
      if (SWIGLU) {
        const float gte = acc[0][f][i], up = acc[1][f][i];
        const float h = gte / (1.f + __expf(-gte)) * up;
        crow[col0 + m] = to_bf16(h);
      } else {
        crow[col0 + m] = to_bf16(acc[0][f][i]);
        crow[col0 + 16 + m] = to_bf16(acc[1][f][i]);
      }
    }
}

template <int NFMAX, bool SWIGLU>
__global__ __launch_bounds__(256) void q4_gemm_rows_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[NFMAX * 16 * LDA];
  __shared__ __attribute__((aligned(16))) float Xs[(KC / 64) * NFMAX * 16];
  const int tile_id = blockIdx.x / p.n_slices;
  const int slice = blockIdx.x - tile_id * p.n_slices;
  if (tile_id >= *p.tile_count) return;
  const int4 t = p.tiles[tile_id];
  const int g = t.x, row0 = t.y, nrows = t.z;
  if (nrows <= 0) return;
  if (nrows <= 16)
    gemm_tile<1, SWIGLU>(p, g, row0, nrows, slice, As, Xs);
  else if (NFMAX == 2 || nrows <= 32)
    gemm_tile<2, SWIGLU>(p, g, row0, nrows, slice, As, Xs);
  else
    gemm_tile<NFMAX, SWIGLU>(p, g, row0, nrows, slice, As, Xs);
}

int gemm_q4_slices(int N, bool swiglu) {
  return swiglu ? ((N >> 1) + 63) / 64 : (N + 127) / 128;
}

void launch_gemm_q4(GemmParams p, int bm, bool swiglu, int64_t n_tiles_bound, hipStream_t s) {
  p.n_slices = gemm_q4_slices(p.N, swiglu);
  const int64_t blocks = n_tiles_bound * p.n_slices;
  if (blocks <= 0) return;
  dim3 grid((unsigned)blocks), block(256);
  if (bm <= 32) {
    if (swiglu) hipLaunchKernelGGL((q4_gemm_rows_kernel<2, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((q4_gemm_rows_kernel<2, false>), grid, block, 0, s, p);
  } else {
    if (swiglu) hipLaunchKernelGGL((q4_gemm_rows_kernel<4, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((q4_gemm_rows_kernel<4, false>), grid, block, 0, s, p);
  }
}

}  // namespace moeq4
