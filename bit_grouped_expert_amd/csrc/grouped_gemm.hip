// Grouped GEMM over groupwise-affine 4-bit weights for gfx950 (MI355X): one
// engine for every group size, from a few rows per expert (weight-streaming,
// HBM-bound) to thousands (matrix-core-bound).
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
// engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph 5 (4-bit weights,
// every 64 sharing one bf16 scale and one bf16 bias, reconstructed one tile at a
// time inside the grouped GEMM with FP32 accumulation, never expanded in memory)
// and paragraph 6 (tiles of expert rows driven by a block map; expert GEMMs are
// most of prefill).  The Metal design there is prior art; this one is laid out
// for CDNA4 wavefronts, matrix cores and XCDs.
//
// Arithmetic (exact up to fp32 rounding; no weight is ever rounded to bf16).
// For output row m, weight row n and one 64-wide scale group g with scale s and
// bias b:
//   sum_c x[m,c] (q[n,c] s + b) = s * P + c_nb * X,
//   P = sum_c x[m,c] (q[n,c] - 8),   X = sum_c x[m,c],   c_nb = b + 8 s.
// The matrix cores compute P as sum_c x[m,c] (128 + q[n,c]) starting from the
// accumulator value -136 X: 128 + q is exactly the bf16 with bits 0x4300 | q, so
// a packed word becomes four MFMA bf16 pairs with one AND-OR each, every product
// is exact, and the -136 X start (one fp32 product per row, shared by every
// weight row) removes the offset inside the fp32 accumulation.  The group's
// partial is then folded in with one FMA per output, acc += s * P, plus
// c_nb * X only when some weight row of the group has b != -8 s.  X (row sums of
// the activations per 64-wide group) is computed once per activation row by the
// producer of the activations, not per tile.
//
// Work decomposition.  A work item is a tile of up to 32 rows of one group
// (rows gathered through a row index) and a slice of weight rows: four
// wavefronts with 64 weight rows each (four 16-row fragments; for SwiGLU 32
// gate rows and the matching 32 up rows, i.e. 32 output columns per wave).
// K advances 128 at a time (two scale groups).  The tile's activation rows and
// row sums for the next 128 K are staged in a double-buffered LDS tile; each
// wavefront streams its own weight rows from HBM straight into VGPRs with
// 128-bit loads one stage ahead (weights never touch LDS) and issues
// v_mfma_f32_16x16x32_bf16 for each 16-row fragment of the tile.  The result
// tile goes back through LDS so that the global stores are 128-bit rows.
//
// MFMA layout (16x16x32 bf16): lane l supplies row (l % 16) of A and column
// (l % 16) of B, each with eight k-slots belonging to quarter l / 16; the
// accumulator holds rows 4*(l/16)+i, column l % 16.  Lanes of quarter q load
// words 4q..4q+3 of a 128-K block of their weight row; two permlane32 swaps
// regroup them so that each MFMA step's four quarters hold words of one scale
// group.  The word a lane holds in each step is tracked by applying the same
// swaps to the word numbers; the A fragment is read from the LDS column of that
// word, and the step's scale group is read off the tracked word number, so
// nothing depends on the swap's direction.  Within a k-slot the codes come out
// in the order 0,4,1,5,2,6,3,7 and the LDS copy of the activations is stored in
// that order.
//
// Scheduling: a persistent grid (a multiple of 8 workgroups).  Workgroups are
// dispatched round-robin over the 8 XCDs, so workgroup b runs on XCD b % 8; XCD
// x takes the x-th contiguous eighth of the device-side tile list and walks its
// (tile, slice) items tile-major, so the slices of one tile (which share its
// activation rows) run side by side in one L2.  No item depends on another.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moeq4 {

namespace {

constexpr int KS = 128;                 // K per stage: two scale groups
constexpr int LDA = KS + 8;             // LDS pitch in bf16 (272 B: conflict-free 16 B reads)
constexpr int BMX = 32;                 // most rows per tile
constexpr int A_BUF = BMX * LDA;        // bf16 elements per A buffer
constexpr int X_BUF = 2 * BMX;          // fp32 row sums per buffer (two groups)
constexpr int LDC_SWIGLU = 128 + 8;
constexpr int LDC_PLAIN = 256 + 8;
static_assert(BMX * LDC_PLAIN <= 2 * A_BUF, "output staging must fit the A buffers");
constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kNib = 0x000F000Fu;

// (v & mask) | magic.  `magic` is kept in a VGPR the compiler cannot constant-fold
// (see opaque_magic), so that this becomes one v_and_or_b32 with the mask in an SGPR
// instead of a separate AND and OR (a GFX9 VOP3 cannot encode two literals).
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t magic) {
  return (v & kNib) | magic;
}

// kMagic in a VGPR whose value the compiler does not know.  Written once per item by a
// plain v_mov; only VALU instructions (the AND-ORs above, which the compiler schedules
// and hazard-checks itself) read it, never a matrix instruction.
__device__ __forceinline__ uint32_t opaque_magic() {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "n"(kMagic));
  return v;
}

// One packed word of eight codes -> MFMA operand 128 + q in the order 0,4,1,5,2,6,3,7.
// `magic` holds kMagic in a VGPR.
__device__ __forceinline__ u32x4_t unpack_word(uint32_t w, uint32_t magic) {
  u32x4_t b;
  b[0] = and_or(w, magic);
  b[1] = and_or(w >> 4, magic);
  b[2] = and_or(w >> 8, magic);
  b[3] = and_or(w >> 12, magic);
  return b;
}

__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// the two permlane32 swaps (word 0 <-> 2, word 1 <-> 3) of one lane's word quad
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

// *(T*)(base + byte_off) with a 32-bit byte offset, so that the load can use a
// uniform 64-bit base and a 32-bit per-lane offset
template <typename T>
__device__ __forceinline__ T ld(const void* base, uint32_t byte_off) {
  return *(const T*)((const char*)base + byte_off);
}

// sum of the eight bf16 values in a 16-byte chunk, in fp32
__device__ __forceinline__ float sum8_bf16(u32x4_t v) {
  float s = 0.f;
#pragma unroll
  for (int h = 0; h < 4; ++h) s += bf16lo_to_f32(v[h]) + bf16hi_to_f32(v[h]);
  return s;
}

__device__ __forceinline__ float bf16_at(uint32_t pair, int hi) {
  return hi ? bf16hi_to_f32(pair) : bf16lo_to_f32(pair);
}

// Weight rows of this wave's four 16-row fragments: fragment j covers weight rows
// first[j] .. first[j] + 15 (lane m takes row first[j] + m).
struct WaveRows {
  int first[4];
  bool active;  // the wave has columns inside N
};

template <bool SWIGLU>
__device__ __forceinline__ WaveRows wave_rows(int N, int slice, int wave) {
  WaveRows r;
  if (SWIGLU) {
    const int F = N >> 1;
    const int c = slice * 128 + 32 * wave;
    r.active = c < F;
    const int cc = r.active ? c : 0;
    r.first[0] = cc;
    r.first[1] = cc + 16;
    r.first[2] = F + cc;
    r.first[3] = F + cc + 16;
  } else {
    const int c = slice * 256 + 64 * wave;
    r.active = c < N;
    const int cc = r.active ? c : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.first[j] = cc + 16 * j;
  }
  return r;
}

// Weights of one 128-K stage for this lane: a word quad of each fragment's row and the
// (scale, bias) pairs of the stage's two groups.
struct StageW {
  u32x4_t q[4];
  uint32_t s[4], b[4];
};

template <int NF, bool SWIGLU, bool SDW>
__device__ __forceinline__ void grouped_item(const GemmParams& p, int g, int row0, int nrows,
                                             int slice, uint16_t* __restrict__ As,
                                             float* __restrict__ Xs) {
  constexpr int BM = 16 * NF;
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int N = p.N, K = p.K, KW = K >> 3, KG = K >> 6;
  const int nfull = K / KS;          // full 128-K stages
  const bool tail = (K % KS) != 0;   // one trailing 64-K stage
  const uint32_t magic = opaque_magic();

  // uniform bases of this group's weights; per-lane offsets are 32-bit
  const bool in_main = g < p.n_main;
  const int gi = in_main ? g : 0;
  const uint32_t* qb = (in_main ? p.main.q : p.last.q) + (int64_t)gi * N * KW;
  const uint16_t* sb = (in_main ? p.main.s : p.last.s) + (int64_t)gi * N * KG;
  const uint16_t* bb = (in_main ? p.main.b : p.last.b) + (int64_t)gi * N * KG;
  const WaveRows wr = wave_rows<SWIGLU>(N, slice, wave);
  const bool active = wr.active;
  const uint32_t qlane = ((uint32_t)m * KW + 4 * q) * 4u;   // byte offset of this lane's quad
  const uint32_t slane = (uint32_t)m * KG * 2u;               // byte offset of this lane's row

  // weights of one full stage (rows of inactive waves are clamped to valid rows)
  auto load_w = [&](int stage) __attribute__((always_inline)) -> StageW {
    StageW w;
    const uint32_t wo = (uint32_t)stage * 16, go = (uint32_t)stage * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t* qr = qb + (uint32_t)wr.first[j] * KW + wo;
      const uint16_t* sr = sb + (uint32_t)wr.first[j] * KG + go;
      const uint16_t* br = bb + (uint32_t)wr.first[j] * KG + go;
      w.q[j] = ld<u32x4_t>(qr, qlane);
      if (SDW) {
        w.s[j] = ld<uint32_t>(sr, slane);
        w.b[j] = ld<uint32_t>(br, slane);
      } else {
        w.s[j] = ld<uint16_t>(sr, slane) | ((uint32_t)ld<uint16_t>(sr, slane + 2) << 16);
        w.b[j] = ld<uint16_t>(br, slane) | ((uint32_t)ld<uint16_t>(br, slane + 2) << 16);
      }
    }
    return w;
  };

  // ---- staging assignment: NF chunks of 8 activations per thread, one row sum for 2*BM threads
  const int akc = tid & 15;
  // byte offsets of this thread's chunk rows in A and of its row sum (A has fewer than
  // 2^31 elements, so byte offsets fit 32 bits); a row outside [0, a_rows) reads as zero
  uint32_t aoff[NF];
  bool aval[NF];
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int r = (tid + 256 * i) >> 4;
    int ar = -1;
    if (r < nrows) {
      const int gr = row0 + r;
      ar = p.a_row_index ? p.a_row_index[gr] : gr;
      if (ar < 0 || ar >= p.a_rows) ar = -1;
    }
    aval[i] = ar >= 0;
    aoff[i] = aval[i] ? ((uint32_t)ar * (uint32_t)K + 8u * akc) * 2u : 0u;
  }
  const int xr = tid < 2 * BM ? (tid % BM) : 0, xg = tid < 2 * BM ? tid / BM : 0;
  bool xval = false;
  uint32_t xoff = 0;
  if (tid < 2 * BM && xr < nrows) {
    const int gr = row0 + xr;
    const int ar = p.a_row_index ? p.a_row_index[gr] : gr;
    xval = ar >= 0 && ar < p.a_rows;
    if (xval) xoff = ((uint32_t)ar * (uint32_t)p.xsum_ld + xg) * 4u;
  }
  u32x4_t ra[NF];
  float rx = 0.f;
  auto load_act = [&](int stage, int groups) __attribute__((always_inline)) {
    const uint16_t* a0 = p.A + (uint32_t)stage * KS;
    const int kcl = 64 * groups;
#pragma unroll
    for (int i = 0; i < NF; ++i)
      ra[i] = (aval[i] && 8 * akc < kcl) ? ld<u32x4_t>(a0, aoff[i]) : u32x4_t{0u, 0u, 0u, 0u};
    rx = (xval && xg < groups) ? ld<float>(p.xsum + 2 * stage, xoff) : 0.f;
  };
  auto store_act = [&](int buf) __attribute__((always_inline)) {
    uint16_t* a = As + buf * A_BUF;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int r = (tid + 256 * i) >> 4;
      *(u32x4_t*)(a + r * LDA + 8 * akc) = interleave8(ra[i]);
    }
    if (tid < 2 * BM) Xs[buf * X_BUF + xg * BMX + xr] = rx;
  };

  // word each lane holds in MFMA step st of a 128-K block (after the swaps)
  uint32_t widx[4] = {(uint32_t)(4 * q), (uint32_t)(4 * q + 1), (uint32_t)(4 * q + 2),
                      (uint32_t)(4 * q + 3)};
  swap32(widx[0], widx[2]);
  swap32(widx[1], widx[3]);

  f32x4_t acc[NF][4];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // matrix-core work of one full stage from LDS buffer `buf`; the weight fragments are
  // taken in two halves to bound the live partial sums
  auto compute_full = [&](const StageW& w, int buf) __attribute__((always_inline)) {
    const uint16_t* a = As + buf * A_BUF;
    const float* xs = Xs + buf * X_BUF;
    u32x4_t wsw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wsw[j] = swap_quad(w.q[j]);
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const int gsel = __builtin_amdgcn_readfirstlane((int)(widx[2 * grp] >> 3));
      float sc[4], cb[4];
      bool cz = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = bf16_at(w.s[j], gsel);
        cb[j] = fmaf(8.f, sc[j], bf16_at(w.b[j], gsel));
        cz = cz && cb[j] == 0.f;
      }
      const bool all_cz = __all(cz);
      u32x4_t av[2][NF];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int acol = 8 * (int)widx[2 * grp + h];
#pragma unroll
        for (int f = 0; f < NF; ++f) av[h][f] = *(const u32x4_t*)(a + (16 * f + m) * LDA + acol);
      }
      f32x4_t C0[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const f32x4_t X = *(const f32x4_t*)(xs + gsel * BMX + 16 * f + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) C0[f][i] = -136.f * X[i];
      }
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        f32x4_t P[NF][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int st = 2 * grp + h;
          const u32x4_t B0 = unpack_word(wsw[2 * jh][st], magic);
          const u32x4_t B1 = unpack_word(wsw[2 * jh + 1][st], magic);
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            P[f][0] = mfma16x16x32(av[h][f], B0, h ? P[f][0] : C0[f]);
            P[f][1] = mfma16x16x32(av[h][f], B1, h ? P[f][1] : C0[f]);
          }
        }
        if (all_cz) {
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[f][2 * jh + jj][i] = fmaf(sc[2 * jh + jj], P[f][jj][i], acc[f][2 * jh + jj][i]);
        } else {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const f32x4_t X = *(const f32x4_t*)(xs + gsel * BMX + 16 * f + 4 * q);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[f][2 * jh + jj][i] =
                    fmaf(sc[2 * jh + jj], P[f][jj][i],
                         fmaf(cb[2 * jh + jj], X[i], acc[f][2 * jh + jj][i]));
          }
        }
      }
    }
  };

  __syncthreads();  // the previous item may still read the LDS
  if (nfull > 0) {
    // Stage s uses LDS buffer s % 2 and register set s % 2; stage s + 1 is loaded while
    // stage s computes.  Unrolled by two so that each register set stays put.
    StageW w0, w1;
    load_act(0, 2);
    w0 = load_w(0);
    store_act(0);
    __syncthreads();
    for (int s = 0;; s += 2) {
      const bool m1 = s + 1 < nfull;
      if (m1) {
        load_act(s + 1, 2);
        w1 = load_w(s + 1);
      }
      if (active) compute_full(w0, 0);
      if (m1) store_act(1);
      __syncthreads();
      if (!m1) break;
      const bool m2 = s + 2 < nfull;
      if (m2) {
        load_act(s + 2, 2);
        w0 = load_w(s + 2);
      }
      if (active) compute_full(w1, 1);
      if (m2) store_act(0);
      __syncthreads();
      if (!m2) break;
    }
  }
  if (tail) {
    // trailing 64-K stage: lanes of quarter q hold words 2q, 2q+1 (one scale group)
    const int stage = nfull;
    load_act(stage, 1);
    store_act(0);
    __syncthreads();
    if (active) {
      const uint32_t wo = (uint32_t)stage * 16, go = (uint32_t)stage * 2;
      const uint32_t qlane2 = ((uint32_t)m * KW + 2 * q) * 4u;
      u32x2_t c[4];
      float sc[4], cb[4];
      bool cz = true;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = ld<u32x2_t>(qb + (uint32_t)wr.first[j] * KW + wo, qlane2);
        const uint32_t so = (uint32_t)wr.first[j] * KG + go;
        sc[j] = bf16lo_to_f32(ld<uint16_t>(sb + so, slane));
        cb[j] = fmaf(8.f, sc[j], bf16lo_to_f32(ld<uint16_t>(bb + so, slane)));
        cz = cz && cb[j] == 0.f;
      }
      const bool all_cz = __all(cz);
      f32x4_t X[NF], C0[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        X[f] = *(const f32x4_t*)(Xs + 16 * f + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) C0[f][i] = -136.f * X[f][i];
      }
      f32x4_t P[NF][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4_t B[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) B[j] = unpack_word(c[j][h], magic);
        const int acol = 8 * (2 * q + h);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const u32x4_t av = *(const u32x4_t*)(As + (16 * f + m) * LDA + acol);
#pragma unroll
          for (int j = 0; j < 4; ++j) P[f][j] = mfma16x16x32(av, B[j], h ? P[f][j] : C0[f]);
        }
      }
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[f][j][i] = all_cz ? fmaf(sc[j], P[f][j][i], acc[f][j][i])
                                  : fmaf(sc[j], P[f][j][i], fmaf(cb[j], X[f][i], acc[f][j][i]));
    }
    __syncthreads();
  }

  // ---- epilogue: bf16 tile in LDS (A buffers are free), then 128-bit row stores
  uint16_t* Cs = As;
  if (SWIGLU) {
    if (active) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gte = acc[f][j][i], up = acc[f][j + 2][i];
            const float h = gte / (1.f + __expf(-gte)) * up;
            Cs[(16 * f + 4 * q + i) * LDC_SWIGLU + 32 * wave + 16 * j + m] = to_bf16(h);
          }
    }
    __syncthreads();
    const int F = N >> 1, c0 = slice * 128;
    for (int u = tid; u < BM * 16; u += 256) {
      const int r = u >> 4, ch = u & 15;
      if (r < nrows && c0 + 8 * ch < F)
        *(u32x4_t*)(p.C + (int64_t)(row0 + r) * p.ldc + c0 + 8 * ch) =
            *(const u32x4_t*)(Cs + r * LDC_SWIGLU + 8 * ch);
    }
    if (p.xsum_out) {
      // row sums of the rounded activations per 64-wide group (the next GEMM's X)
      const int r = tid >> 2, gg = (tid >> 1) & 1, half = tid & 1;
      float sum = 0.f;
      if (r < BM) {
        const u32x4_t* src = (const u32x4_t*)(Cs + r * LDC_SWIGLU + 64 * gg + 32 * half);
#pragma unroll
        for (int c = 0; c < 4; ++c) sum += sum8_bf16(src[c]);
      }
      sum += __shfl_xor(sum, 1);
      if (r < nrows && half == 0 && c0 + 64 * gg < F)
        p.xsum_out[(int64_t)(row0 + r) * p.xsum_out_ld + 2 * slice + gg] = sum;
    }
  } else {
    if (active) {
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Cs[(16 * f + 4 * q + i) * LDC_PLAIN + 64 * wave + 16 * j + m] = to_bf16(acc[f][j][i]);
    }
    __syncthreads();
    const int c0 = slice * 256;
    for (int u = tid; u < BM * 32; u += 256) {
      const int r = u >> 5, ch = u & 31;
      if (r < nrows && c0 + 8 * ch < N)
        *(u32x4_t*)(p.C + (int64_t)(row0 + r) * p.ldc + c0 + 8 * ch) =
            *(const u32x4_t*)(Cs + r * LDC_PLAIN + 8 * ch);
    }
  }
}

// SDW: the scale/bias arrays have an even number of groups per row, so the pair of a
// 128-K stage is one aligned dword
template <bool SWIGLU, bool SDW>
__global__ __launch_bounds__(256, 2) void q4_grouped_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2 * A_BUF];
  __shared__ __attribute__((aligned(16))) float Xs[2 * X_BUF];
  const int cnt = *p.tile_count;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const int t0 = (int)((int64_t)xcd * cnt / 8);
  const int t1 = (int)((int64_t)(xcd + 1) * cnt / 8);
  const int items = (t1 - t0) * p.n_slices;
  for (int w = slot; w < items; w += nslot) {
    const int tile = t0 + w / p.n_slices;
    const int slice = w - (tile - t0) * p.n_slices;
    const int4 t = p.tiles[tile];
    const int nrows = t.z;
    if (nrows <= 0) continue;
    if (nrows <= 16) grouped_item<1, SWIGLU, SDW>(p, t.x, t.y, nrows, slice, As, Xs);
    else grouped_item<2, SWIGLU, SDW>(p, t.x, t.y, nrows, slice, As, Xs);
  }
}

// Row sums per 64-wide group: out[r][g] = sum of A[r][64g .. 64g+63] (fp32).
// One wavefront per row; lane l sums groups l, l+64, ...
__global__ __launch_bounds__(256) void row_group_sums_kernel(const uint16_t* __restrict__ A,
                                                             int rows, int K,
                                                             float* __restrict__ out) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (r >= rows) return;
  const int KG = K >> 6;
  for (int g = l; g < KG; g += 64) {
    const u32x4_t* src = (const u32x4_t*)(A + (int64_t)r * K + 64 * g);
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) sum += sum8_bf16(src[c]);
    out[(int64_t)r * KG + g] = sum;
  }
}

}  // namespace

int grouped_slices(int N, bool swiglu) {
  return swiglu ? ((N >> 1) + 127) / 128 : (N + 255) / 256;
}

void launch_row_group_sums(const uint16_t* A, int rows, int K, float* out, hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(row_group_sums_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, A, rows, K,
                     out);
}

void launch_grouped(GemmParams p, bool swiglu, int64_t n_tiles_bound, int n_cu, hipStream_t s) {
  p.n_slices = grouped_slices(p.N, swiglu);
  const int64_t items = n_tiles_bound * p.n_slices;
  if (items <= 0) return;
  int64_t blocks = 2 * (int64_t)(n_cu > 0 ? n_cu : 256);
  if (blocks > items + 7) blocks = items + 7;
  blocks = (blocks + 7) / 8 * 8;
  dim3 grid((unsigned)blocks), block(256);
  const bool sdw = ((p.K >> 6) & 1) == 0;
  if (swiglu) {
    if (sdw) hipLaunchKernelGGL((q4_grouped_kernel<true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((q4_grouped_kernel<true, false>), grid, block, 0, s, p);
  } else {
    if (sdw) hipLaunchKernelGGL((q4_grouped_kernel<false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((q4_grouped_kernel<false, false>), grid, block, 0, s, p);
  }
}

}  // namespace moeq4
