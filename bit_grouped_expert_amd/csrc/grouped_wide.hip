// Wide-tile grouped GEMM over groupwise-affine 4-bit weights for gfx950 (MI355X): the
// engine for large groups (hundreds of rows per expert), where the layer is bound by
// the matrix cores and the vector work around them rather than by weight bytes.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
// engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph 5 (4-bit weights
// with one bf16 scale and bias per 64, reconstructed tile by tile inside the
// grouped GEMM, with fp32 accumulation).
//
// Arithmetic: as in the resident-tile engine (exact up to fp32 rounding): per 64-wide
// group, P' = sum x (128 + q) on the matrix cores from zero, acc += s P', and the bias
// term sum_g (b - 128 s) X.  Where K >= 1024 the bias term is formed once per block of
// weight rows, as bf16 matrix-core products with all 32 groups as k: b X and s X with
// X split exactly into three bf16 pieces (b and s are bf16 already, so every product is
// exact), then acc += b X - 128 (s X).  The lane's s and b words of the block are loaded
// at its first stage, and the product follows that stage once X is complete (every block
// after a workgroup's first), so that it does not delay the block's end.  Where K <= 512 (the down GEMM) the three pieces
// of X sit side by side in the 32-wide k (3 x 8 groups), so b X and s X are one MFMA
// each.  In between (K = 768) the bias stays a per-stage fp32 product
// (v_mfma_f32_16x16x4_f32, the stage's four groups as k); timing the engine without any
// bias term put that product at about 18% of gate_up and 14% of down at 8192 tokens.
//
// Work decomposition.  One workgroup per tile of up to 128 rows of one group (eight
// 16-row fragments); it walks every block of 256 weight rows (with SwiGLU: 128 gate
// rows and the matching 128 up rows) as one sequence of 256-K stages.  Each of the
// eight wavefronts owns two 16-row weight fragments of the block (SwiGLU: a gate
// fragment and its up fragment) for all eight row fragments, so that a packed word,
// unpacked once, feeds eight MFMAs, and the per-group fold costs two FMAs per MFMA.
// Weights stream from HBM into VGPRs as in the resident engine (16-byte loads of whole
// 128-byte row lines, two stages in flight, two permlane32 swaps per word quad).  The
// tile's activation rows go through two LDS buffers of one stage each, by direct
// global->LDS loads issued one stage ahead.  The two buffers are distinct LDS arrays
// addressed statically (the stage loop is unrolled by two), so the compiler can tell
// that a direct load into one does not feed the reads of the other and does not wait
// for it before them; each wavefront drains its loads before the stage's barrier,
// which costs little since they were issued a whole stage earlier.  The row sums X
// come from the first block's stages (activation fragments times ones) and stay in
// LDS for the later blocks.  Tiles of one group are adjacent and XCD b % 8 takes a
// contiguous run of tiles, so a group's weights are read from HBM about once per XCD.
// The tiles of an XCD's last, partial round go to one workgroup per unit of one or two
// blocks instead of one per tile, so that this round is spread over the XCD.
//
// Measured at 8192 tokens (uniform routing) gate_up takes about 545 us against 643 us
// on the resident engine.  Hardware counters put the matrix cores at 29% busy (bf16
// and the fp32 bias product together) and the cycles in which vector and matrix
// instructions execute together at about 2%: the two wavefronts of a SIMD go through
// their operand, MFMA and fold phases at the same time, so the folds and the unpacking
// add to the matrix time instead of hiding under it.  Timing variants agree: without
// any global load in the loop it still takes most of its time, and dropping the fold,
// the unpacking or the LDS activation reads alone changes little.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "q4_stream.h"

namespace moeq4 {

namespace {

constexpr int WBM = kWideBM;                 // rows per tile
constexpr int WKS = 256;                     // K per stage (four groups)
constexpr int A_BUF = (WBM / 16) * 32 * 256; // [fragment 8][16-byte chunk 32][row 16]: 64 KB
constexpr int XG = kWideMaxK / 64;           // 64-wide groups of the largest K (32)
constexpr int XP_PIECE = WBM * XG * 2;       // one bf16 piece of X: [128 rows][32 groups]
constexpr int XP_BYTES = 3 * XP_PIECE;       // X = hi + mid + lo, exactly: 24 KB
constexpr int STG_BYTES = 8 * 1024;          // epilogue staging, 1 KB per wavefront
static_assert(XG == 32, "one 16x16x32 MFMA covers every group of the largest K");
static_assert(2 * A_BUF + XP_BYTES + STG_BYTES <= 160 * 1024, "LDS budget");

struct WideLds {
  unsigned char* a[2];
  unsigned char* xp;
  unsigned char* stg;
};

// blocks of 256 weight rows per unit of a last round: enough for four 256-K stages, and a
// divisor of the tile's NB blocks
__host__ __device__ inline int wide_unit_blocks(int NB, int NK) {
  int ub = NK >= 4 ? 1 : (4 + NK - 1) / NK;
  if (ub > NB) ub = NB;
  while (NB % ub) --ub;
  return ub;
}

// BM (bias mode): 1, the bias term once per block as bf16 products with the 32 groups
// as k (K >= 1024); 2, once per block with the three pieces of X side by side in k (K
// <= 512: 3 x 8 groups fit one MFMA); 0, per stage as an fp32 product over the stage's
// four groups.
template <bool SWIGLU, int GS, int BM>
__device__ __forceinline__ void wide_body(const WideParams& p, const WideLds& lds) {
  constexpr bool BB = BM != 0;
  constexpr int D = 2;  // weight register sets: the next stage's in flight
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int N = p.N, K = p.K, KW = K >> 3, KG = K >> 6, NK = K / WKS;
  const int NB = SWIGLU ? (N >> 1) / 128 : N / 256;

  // ---- this workgroup's work: XCD b % 8 takes a contiguous run of `per` tiles, one
  // workgroup per tile in order (the hardware starts the next one wherever a compute unit
  // of the XCD frees up).  With xcd_cus set, the tiles of the XCD's last, partial round
  // (those past its whole rounds of xcd_cus tiles) get one workgroup per unit of UB
  // blocks of 256 weight rows instead (at least four stages each), so that this round
  // spreads over the compute units.
  const int cnt = *p.tile_count;
  const int per = (cnt + 7) >> 3;
  const int jx = blockIdx.x >> 3;
  const int UB = wide_unit_blocks(NB, NK), NUT = NB / UB;  // blocks per unit, units per tile
  int tile, blk0 = 0, nblk = NB;
  if (p.xcd_cus > 0) {
    const int full = per / p.xcd_cus * p.xcd_cus;  // tiles in whole rounds
    if (jx < full) {
      tile = (blockIdx.x & 7) * per + jx;
    } else {
      const int u = jx - full;
      if (u >= (per - full) * NUT) return;  // uniform, before any barrier
      tile = (blockIdx.x & 7) * per + full + u / NUT;
      blk0 = (u - (u / NUT) * NUT) * UB;
      nblk = UB;
    }
  } else {
    if (jx >= per) return;  // uniform, before any barrier
    tile = (blockIdx.x & 7) * per + jx;
  }
  if (tile >= cnt) return;
  const int UT = nblk * NK;  // stages of this workgroup: block blk0 + v / NK, stage v % NK
  const int4 tt = p.tiles[tile];
  const int grp = __builtin_amdgcn_readfirstlane(tt.x);
  const int row0 = __builtin_amdgcn_readfirstlane(tt.y);
  const int nrows = __builtin_amdgcn_readfirstlane(tt.z);
  const int nfv = (nrows + 15) >> 4;  // row fragments with rows (1..8)
  const bool in_main = grp < p.n_main;
  const int gi = in_main ? grp : 0;
  const uint32_t* Wq = (in_main ? p.main.q : p.last.q) + (int64_t)gi * N * KW;
  const uint16_t* Ws = (in_main ? p.main.s : p.last.s) + (int64_t)gi * N * KG;
  const uint16_t* Wb = (in_main ? p.main.b : p.last.b) + (int64_t)gi * N * KG;

  // ---- activation rows: wavefront w loads fragment w (rows 16 w + m); rows past the
  // tile repeat its last row, rows outside [0, a_rows) read row a_rows (zero)
  const uint16_t* asrc;
  {
    const int r = min(16 * wave + m, nrows - 1);
    int a = p.a_row_index ? p.a_row_index[row0 + r] : row0 + r;
    if (a < 0 || a >= p.a_rows) a = p.a_rows;
    asrc = p.A + (int64_t)a * K + 8 * q;
  }
  // stage st of the activations into buffer dst: chunks 4 cb .. 4 cb + 3 of fragment
  // `wave` per load (1 KB)
  auto issue_a = [&](int st, unsigned char* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      __builtin_amdgcn_global_load_lds(asrc + WKS * st + 32 * cb, dst + wave * 8192 + cb * 1024, 16, 0,
                                       0);
  };

  // ---- weight stream: flat stage index, past the end the last stage again
  int pf_v = 0;
  auto pf_load = [&](StageW& w) __attribute__((always_inline)) {
    const int v = min(pf_v, UT - 1);
    const int vb = v / NK, st = v - vb * NK, blk = blk0 + vb;
    int n0, n1;
    if (SWIGLU) {
      const int u = 8 * blk + wave;
      n0 = 16 * u + m;
      n1 = (N >> 1) + 16 * u + m;
    } else {
      n0 = 256 * blk + 32 * wave + m;
      n1 = n0 + 16;
    }
    const uint32_t co0 = ((uint32_t)n0 * KW + 4 * q) * 4u, co1 = ((uint32_t)n1 * KW + 4 * q) * 4u;
    const uint32_t so0 = (uint32_t)n0 * KG * 2u, so1 = (uint32_t)n1 * KG * 2u;
    const uint32_t* qs = Wq + 32 * st;
    w.c[0][0] = ld<u32x4_t>(qs, co0);
    w.c[0][1] = ld<u32x4_t>(qs + 16, co0);
    w.s[0] = ld<u32x2_t>(Ws + 4 * st, so0);
    w.b[0] = ld<u32x2_t>(Wb + 4 * st, so0);
    w.c[1][0] = ld<u32x4_t>(qs, co1);
    w.c[1][1] = ld<u32x4_t>(qs + 16, co1);
    w.s[1] = ld<u32x2_t>(Ws + 4 * st, so1);
    w.b[1] = ld<u32x2_t>(Wb + 4 * st, so1);
    ++pf_v;
  };

  const uint32_t magic = opaque_magic();
  const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  uint32_t widx[4] = {(uint32_t)(4 * q), (uint32_t)(4 * q + 1), (uint32_t)(4 * q + 2),
                      (uint32_t)(4 * q + 3)};
  {
    const auto r0 = __builtin_amdgcn_permlane32_swap(widx[0], widx[2], false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(widx[1], widx[3], false, false);
    widx[0] = r0[0];
    widx[2] = r0[1];
    widx[1] = r1[0];
    widx[3] = r1[1];
  }
  uint32_t a_step[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) a_step[t] = widx[t] * 256u + 16u * m;

  f32x4_t acc[8][2];  // [row fragment][weight fragment]
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      acc[f][0] = zero;
      acc[f][1] = zero;
    }
  };
  reset();

  // One 256-K stage in two 128-K halves (MFMA steps 2 (g ^ GS), 2 (g ^ GS) + 1 of a
  // half take its scale group g, as in the resident engine): per row fragment, P' of
  // both weight fragments and both groups from zero, then acc += s P'.  cbq (per-stage
  // bias only): the lane's (b - 128 s) of group q of the stage.
  auto compute = [&](const StageW& w, const unsigned char* abuf, float* cbq) __attribute__((always_inline)) {
    if constexpr (!BB) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t sw = (q & 2) ? w.s[j][1] : w.s[j][0];
        const uint32_t bw = (q & 2) ? w.b[j][1] : w.b[j][0];
        const float sq = (q & 1) ? bf16hi_to_f32(sw) : bf16lo_to_f32(sw);
        const float bq = (q & 1) ? bf16hi_to_f32(bw) : bf16lo_to_f32(bw);
        cbq[j] = fmaf(-128.f, sq, bq);
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const unsigned char* ab = abuf + hh * 4096;
      u32x4_t wsw[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) wsw[j] = swap_quad(w.c[j][hh]);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        u32x4_t B[2][2];  // [weight fragment][half step]
        float sc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int h = 0; h < 2; ++h) B[j][h] = unpack_word(wsw[j][2 * (g ^ GS) + h], magic);
          sc[j] = g == 0 ? bf16lo_to_f32(w.s[j][hh]) : bf16hi_to_f32(w.s[j][hh]);
        }
        // two row fragments at a time in three phases kept apart by scheduling barriers
        // (operands; the four MFMA chains; the folds), so that four independent chains
        // are in flight and no result is consumed before the chains are issued.  A pair
        // past the tile's last fragment computes rows it then drops.
#pragma unroll
        for (int fp = 0; fp < 4; ++fp) {
          if (2 * fp < nfv) {
            u32x4_t a[2][2];  // [fragment of the pair][half step]
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
              for (int h = 0; h < 2; ++h)
                a[e][h] = *(const u32x4_t*)(ab + (2 * fp + e) * 8192 + a_step[2 * (g ^ GS) + h]);
            __builtin_amdgcn_sched_barrier(0);
            f32x4_t P[2][2];  // [fragment of the pair][weight fragment]
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
              for (int j = 0; j < 2; ++j) P[e][j] = mfma16x16x32(a[e][0], B[j][0], zero);
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
              for (int j = 0; j < 2; ++j) P[e][j] = mfma16x16x32(a[e][1], B[j][1], P[e][j]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
              for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  acc[2 * fp + e][j][i] = fmaf(sc[j], P[e][j][i], acc[2 * fp + e][j][i]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  };
  // The same stage, branch-free and software-pipelined, for NP fragment pairs (the tile's
  // row fragments rounded up to pairs; rows past the tile repeat its last row and are
  // dropped): 4 NP units (half hh, group g, fragment pair fp).  During unit u the wavefront
  // issues the LDS reads of unit u + 1, the eight MFMAs of unit u and the folds of unit
  // u - 1, and during the last unit of a group it also unpacks the next group's words, so
  // that the LDS latency, the MFMA chains and the vector work overlap instead of following
  // each other.  Same arithmetic, in the same order per output, as `compute`.
  auto compute_pipe = [&](const StageW& w, const unsigned char* abuf, auto np_tag)
                          __attribute__((always_inline)) {
    constexpr int NP = decltype(np_tag)::value;
    constexpr int NU = 4 * NP;
    u32x4_t wsw[2];      // [weight fragment]: the current half's words after the swaps
    u32x4_t Bq[2][2][2]; // [buffer][weight fragment][half step]
    float sc[2][2];      // [buffer][weight fragment]
    u32x4_t A[2][2][2];  // [buffer][fragment of the pair][half step]
    f32x4_t P[2][2][2];  // [buffer][fragment of the pair][weight fragment]
    auto unpack_group = [&](int hh, int g, int bb) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) Bq[bb][j][h] = unpack_word(wsw[j][2 * (g ^ GS) + h], magic);
        sc[bb][j] = g == 0 ? bf16lo_to_f32(w.s[j][hh]) : bf16hi_to_f32(w.s[j][hh]);
      }
    };
    auto read_a = [&](int u, int ab) __attribute__((always_inline)) {
      const int gi = u / NP, hh = gi >> 1, g = gi & 1, fp = u - gi * NP;
      const unsigned char* base = abuf + hh * 4096;
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          A[ab][e][h] = *(const u32x4_t*)(base + (2 * fp + e) * 8192 + a_step[2 * (g ^ GS) + h]);
    };
#pragma unroll
    for (int j = 0; j < 2; ++j) wsw[j] = swap_quad(w.c[j][0]);
    unpack_group(0, 0, 0);
    read_a(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int gi = u / NP, fp = u - gi * NP, cb = u & 1, bb = gi & 1;
      if (u + 1 < NU) read_a(u + 1, cb ^ 1);
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < 2; ++j) P[cb][e][j] = mfma16x16x32(A[cb][e][0], Bq[bb][j][0], zero);
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < 2; ++j) P[cb][e][j] = mfma16x16x32(A[cb][e][1], Bq[bb][j][1], P[cb][e][j]);
      if (u > 0) {
        const int gq = (u - 1) / NP, fq = (u - 1) - gq * NP, pb = gq & 1;
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[2 * fq + e][j][i] = fmaf(sc[pb][j], P[cb ^ 1][e][j][i], acc[2 * fq + e][j][i]);
      }
      const bool unpack_next = fp == NP - 1 && u + 1 < NU;
      if (unpack_next) {
        const int gn = gi + 1;
        if ((gn >> 1) != (gi >> 1)) {
#pragma unroll
          for (int j = 0; j < 2; ++j) wsw[j] = swap_quad(w.c[j][1]);
        }
        unpack_group(gn >> 1, gn & 1, bb ^ 1);
      }
      // order inside the unit: the first MFMA (whose wait covers the reads issued a unit
      // earlier), then this unit's four reads for the next unit, then each further MFMA
      // followed by vector work (folds, and unpacking in a group's last unit)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (u + 1 < NU) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      if (unpack_next) {
#pragma unroll
        for (int r = 0; r < 7; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 7; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the folds of the last unit (fragment pair NP - 1 of group 3: buffer 1)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[2 * (NP - 1) + e][j][i] = fmaf(sc[1][j], P[(NU - 1) & 1][e][j][i], acc[2 * (NP - 1) + e][j][i]);
  };
  // X[row][group] of this wavefront's fragment for the stage's four groups: the product
  // of the group's two 32-K activation fragments with a fragment of ones (lanes of column
  // 0 hold it), stored as three bf16 pieces whose sum is X exactly (each takes the top
  // eight significant bits of what the previous ones left)
  unsigned char* xp = lds.xp;
  auto row_sums = [&](int st, const unsigned char* abuf) __attribute__((always_inline)) {
    if (wave < nfv) {
      const unsigned char* af = abuf + wave * 8192 + 16 * m;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x4_t a0 = *(const u32x4_t*)(af + (8 * g4 + q) * 256);
        const u32x4_t a1 = *(const u32x4_t*)(af + (8 * g4 + 4 + q) * 256);
        const f32x4_t X = mfma16x16x32(a1, ones, mfma16x16x32(a0, ones, zero));
        if (!BB && m == 0)
          *(f32x4_t*)((float*)xp + (4 * st + g4) * WBM + 16 * wave + 4 * q) = X;  // [group][row]
        if (BB && m == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t hi = __float_as_uint(X[i]) & 0xFFFF0000u;
            const float r1 = X[i] - __uint_as_float(hi);
            const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
            const float r2 = r1 - __uint_as_float(mid);
            const uint32_t lo = __float_as_uint(r2) & 0xFFFF0000u;
            const int off = (16 * wave + 4 * q + i) * (2 * XG) + 2 * (4 * st + g4);
            *(uint16_t*)(xp + off) = (uint16_t)(hi >> 16);
            *(uint16_t*)(xp + XP_PIECE + off) = (uint16_t)(mid >> 16);
            *(uint16_t*)(xp + 2 * XP_PIECE + off) = (uint16_t)(lo >> 16);
          }
        }
      }
    }
  };
  // The bias term of a finished block, sum over groups of (b - 128 s) X, exactly up to
  // fp32 rounding: b X and s X as bf16 products with the groups as k (v_mfma_f32_16x16x32:
  // lane (m, q) gives X of row m and groups 8q .. 8q+7, lane (n, q) b or s of column n and
  // the same groups), over the three pieces of X; then acc += b X - 128 (s X).  sb: this
  // lane's s and b words of groups 8q .. 8q+7, captured from the stages as they passed.
  // BM 1: the s and b words of the block that this lane feeds to the bias product
  // (groups 8q .. 8q+7), loaded at the block's first stage as two 8-byte halves; a half
  // past K is loaded again from the row's first groups and not used.  BM 2: groups 0 .. 7
  // on every lane, taken from the stages' words as they stream (capture_sb).
  const int sb_g0 = BM == 1 ? 8 * q : 0;
  const bool sb_lo = sb_g0 + 4 <= KG, sb_hi = sb_g0 + 8 <= KG;
  u32x2_t sbs[2][2], sbb[2][2];  // [weight fragment][half]
  auto load_sb = [&](int blk) __attribute__((always_inline)) {
    int n0, n1;
    if (SWIGLU) {
      const int u = 8 * blk + wave;
      n0 = 16 * u + m;
      n1 = (N >> 1) + 16 * u + m;
    } else {
      n0 = 256 * blk + 32 * wave + m;
      n1 = n0 + 16;
    }
    const uint32_t so[2] = {(uint32_t)n0 * KG * 2u, (uint32_t)n1 * KG * 2u};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t o0 = sb_lo ? so[j] + 2u * sb_g0 : so[j];
      const uint32_t o1 = sb_hi ? so[j] + 2u * sb_g0 + 8u : so[j];
      sbs[j][0] = ld<u32x2_t>(Ws, o0);
      sbs[j][1] = ld<u32x2_t>(Ws, o1);
      sbb[j][0] = ld<u32x2_t>(Wb, o0);
      sbb[j][1] = ld<u32x2_t>(Wb, o1);
    }
  };
  u32x4_t cs[2], cb[2];  // the words as MFMA operands (zero past K)
  auto clear_sb = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      cs[j] = u32x4_t{0u, 0u, 0u, 0u};
      cb[j] = cs[j];
    }
  };
  clear_sb();
  auto capture_sb = [&](int st, const StageW& w) __attribute__((always_inline)) {
    const bool lo_half = st == 0, hi_half = st == 1;  // groups 0 .. 3, 4 .. 7
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      cs[j][0] = lo_half ? w.s[j][0] : cs[j][0];
      cs[j][1] = lo_half ? w.s[j][1] : cs[j][1];
      cs[j][2] = hi_half ? w.s[j][0] : cs[j][2];
      cs[j][3] = hi_half ? w.s[j][1] : cs[j][3];
      cb[j][0] = lo_half ? w.b[j][0] : cb[j][0];
      cb[j][1] = lo_half ? w.b[j][1] : cb[j][1];
      cb[j][2] = hi_half ? w.b[j][0] : cb[j][2];
      cb[j][3] = hi_half ? w.b[j][1] : cb[j][3];
    }
  };
  auto take_sb = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      cs[j] = u32x4_t{sb_lo ? sbs[j][0][0] : 0u, sb_lo ? sbs[j][0][1] : 0u, sb_hi ? sbs[j][1][0] : 0u,
                      sb_hi ? sbs[j][1][1] : 0u};
      cb[j] = u32x4_t{sb_lo ? sbb[j][0][0] : 0u, sb_lo ? sbb[j][0][1] : 0u, sb_hi ? sbb[j][1][0] : 0u,
                      sb_hi ? sbb[j][1][1] : 0u};
    }
  };
  // Per stage (without BB): acc += (b - 128 s) X over the stage's four groups
  // (v_mfma_f32_16x16x4_f32: lane l gives A[row l % 16][k = l / 16] and B[k = l / 16]
  // [column l % 16], k = group), X fp32 [group][row] in the same LDS.
  auto bias_term = [&](int st, const float* cbq) __attribute__((always_inline)) {
    const float* xg = (const float*)xp + (4 * st + q) * WBM + m;
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfv) {
        const float xa = xg[16 * f];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, cbq[j], acc[f][j], 0, 0, 0);
      }
    }
  };
  // BM 2: k = 8 p + g takes piece p (0..2) of X and group g (0..7); b and s repeat
  // over p; quarter q = 3 gives zeros.  b X and s X are then one MFMA each.
  auto bias_block_packed = [&]() __attribute__((always_inline)) {
    const u32x4_t z4 = {0u, 0u, 0u, 0u};
    u32x4_t bq[2], sq[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bq[j] = q < 3 ? cb[j] : z4;
      sq[j] = q < 3 ? cs[j] : z4;
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfv) {
        u32x4_t xa = *(const u32x4_t*)(xp + (q < 3 ? q : 0) * XP_PIECE + (16 * f + m) * (2 * XG));
        if (q == 3) xa = z4;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4_t sx = mfma16x16x32(xa, sq[j], zero);
          acc[f][j] = mfma16x16x32(xa, bq[j], acc[f][j]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[f][j][i] = fmaf(-128.f, sx[i], acc[f][j][i]);
        }
      }
    }
  };
  auto bias_block = [&]() __attribute__((always_inline)) {
    take_sb();
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfv) {
        const unsigned char* xr = xp + (16 * f + m) * (2 * XG) + 16 * q;
        const u32x4_t x0 = *(const u32x4_t*)(xr);
        const u32x4_t x1 = *(const u32x4_t*)(xr + XP_PIECE);
        const u32x4_t x2 = *(const u32x4_t*)(xr + 2 * XP_PIECE);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4_t sx = mfma16x16x32(x2, cs[j], mfma16x16x32(x1, cs[j], mfma16x16x32(x0, cs[j], zero)));
          acc[f][j] = mfma16x16x32(x2, cb[j], mfma16x16x32(x1, cb[j], mfma16x16x32(x0, cb[j], acc[f][j])));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[f][j][i] = fmaf(-128.f, sx[i], acc[f][j][i]);
        }
      }
    }
  };
  // the finished block: bf16 rows through this wavefront's 1 KB of LDS staging
  unsigned char* stg = lds.stg + wave * 1024;
  auto epilogue = [&](int blk) __attribute__((always_inline)) {
    uint16_t* cs = (uint16_t*)stg;
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f < nfv) {
        if (SWIGLU) {
          const int col = p.c_perm ? ((m & 8) | perm8(m & 7)) : m;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gte = acc[f][0][i], up = acc[f][1][i];
            cs[(4 * q + i) * 16 + col] = to_bf16(gte / (1.f + __expf(-gte)) * up);
          }
          const int r = l >> 1, half = l & 1;
          const int u = 8 * blk + wave;
          if (l < 32 && 16 * f + r < nrows)
            *(u32x4_t*)(p.C + (int64_t)(row0 + 16 * f + r) * p.ldc + 16 * u + 8 * half) =
                *(const u32x4_t*)(cs + r * 16 + 8 * half);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) cs[(4 * q + i) * 32 + 16 * j + m] = to_bf16(acc[f][j][i]);
          const int r = l >> 2, piece = l & 3;
          if (16 * f + r < nrows)
            *(u32x4_t*)(p.C + (int64_t)(row0 + 16 * f + r) * p.ldc + 256 * blk + 32 * wave + 8 * piece) =
                *(const u32x4_t*)(cs + r * 32 + 8 * piece);
        }
      }
    }
  };

  // ---- prologue: the pieces of X zeroed (groups past K stay zero), stage 0's
  // activations and weights
  for (int o = 16 * tid; o < XP_BYTES; o += 16 * 512) *(u32x4_t*)(xp + o) = u32x4_t{0u, 0u, 0u, 0u};
  StageW W[D];
  issue_a(0, lds.a[0]);
  pf_load(W[0]);
  wait_vmcnt0();
  lds_barrier();

  // ---- stage loop: stage v in buffer v & 1 and register set v & 1.  The next stage's
  // activations and weights are issued first; after the matrix work every load has
  // landed and a barrier publishes the next buffer.  The bias term of stage v follows
  // the barrier (X of a first block's stage is formed during it); after a block's last
  // stage its outputs, then the accumulators start over.
  // The stage loop, one copy per stage form (NP > 0: the pipelined stage over NP fragment
  // pairs; 0: the generic stage), chosen once per tile so that each copy keeps its own
  // register allocation (a loop holding two forms spills).
  auto run = [&](auto np_tag) __attribute__((always_inline)) {
    constexpr int NP = decltype(np_tag)::value;
    auto step = [&](int v, const unsigned char* cur_a, unsigned char* next_a, StageW& cur,
                    StageW& fresh) __attribute__((always_inline)) {
      const int vb = v / NK, st = v - vb * NK, blk = blk0 + vb;
      const int vn = v + 1 < UT ? v + 1 : v;  // the last stage loads itself again
      issue_a(vn - (vn / NK) * NK, next_a);
      pf_load(fresh);
      if (BB && st == 0) load_sb(blk);
      float cbq[2];
      if constexpr (NP > 0) compute_pipe(cur, cur_a, np_tag);
      else compute(cur, cur_a, cbq);
      // BM 1: after the workgroup's first block X is in LDS, and the block's bias product
      // follows its first stage instead of delaying its end
      if (BM == 1 && vb > 0 && st == 0) bias_block();
      if (vb == 0) row_sums(st, cur_a);  // X during the first block of this workgroup
      wait_vmcnt0();
      lds_barrier();
      if (!BB) bias_term(st, cbq);
      if (st == NK - 1) {  // X of every group is in LDS from the first block's end
        if (BM == 1 && vb == 0) bias_block();
        if (BM == 2) {
          take_sb();
          bias_block_packed();
        }
        epilogue(blk);
        reset();
      }
    };
    int v = 0;
    for (; v + 2 <= UT; v += 2) {
      step(v, lds.a[0], lds.a[1], W[0], W[1]);
      step(v + 1, lds.a[1], lds.a[0], W[1], W[0]);
    }
    if (v < UT) step(v, lds.a[0], lds.a[1], W[0], W[1]);
  };
  // K >= 1024 (bias once per block over 32 groups): the pipelined stage; the other forms
  // (K <= 512, and the per-stage bias of K = 768) keep the generic stage, with which the
  // pipelined form spills
  if constexpr (BM == 1) {
    const int np = (nfv + 1) >> 1;
    if (np >= 4) run(std::integral_constant<int, 4>{});
    else if (np == 3) run(std::integral_constant<int, 3>{});
    else if (np == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 0>{});
  }
}

// GS: scale group of MFMA steps 0 and 1 after the word swaps, read off the swapped
// word numbers on entry (both orders compiled).
template <bool SWIGLU, int BM>
__global__ __launch_bounds__(512, 1) void q4_wide_kernel(WideParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char a0[A_BUF];
  __shared__ __attribute__((aligned(16))) unsigned char a1[A_BUF];
  __shared__ __attribute__((aligned(16))) unsigned char xp[XP_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char stg[STG_BYTES];
  const WideLds lds{{a0, a1}, xp, stg};
  const int l = threadIdx.x & 63;
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)(4 * (l >> 4)), (uint32_t)(4 * (l >> 4) + 2),
                                                  false, false);
  const int gs = __builtin_amdgcn_readfirstlane((int)(r[0] >> 3));
  if (gs) wide_body<SWIGLU, 1, BM>(p, lds);
  else wide_body<SWIGLU, 0, BM>(p, lds);
}

template <bool SWIGLU>
void launch_w(WideParams p, int64_t n_tiles_bound, int n_cu, hipStream_t s) {
  const int64_t bound = n_tiles_bound > 0 ? n_tiles_bound : 1;
  const int xc = n_cu / 8;
  const int NB = SWIGLU ? (p.N >> 1) / 128 : p.N / 256;
  const int NUT = NB / wide_unit_blocks(NB, p.K / WKS);  // units per tile of a last round
  // workgroups per XCD: at most per + (xcd_cus - 1) (NUT - 1) for any tile count up to
  // the bound (per <= ceil(bound / 8): whole rounds, then at most xcd_cus - 1 tiles of NUT)
  const int64_t per_b = (bound + 7) / 8;
  p.xcd_cus = xc >= 1 && per_b >= xc ? xc : 0;
  const int64_t per_xcd = p.xcd_cus ? per_b + (int64_t)(xc - 1) * (NUT - 1) : per_b;
  // the bias once per block: with the 32 groups as k from four stages (16 groups) up,
  // with the pieces of X side by side in k up to two stages (8 groups)
  const dim3 grid((unsigned)(8 * per_xcd)), block(512);
  if (p.K >= 4 * WKS) hipLaunchKernelGGL((q4_wide_kernel<SWIGLU, 1>), grid, block, 0, s, p);
  else if (p.K <= 2 * WKS) hipLaunchKernelGGL((q4_wide_kernel<SWIGLU, 2>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((q4_wide_kernel<SWIGLU, 0>), grid, block, 0, s, p);
}

}  // namespace

bool wide_supported(int N, int K, bool swiglu, int a_rows) {
  (void)swiglu;  // SwiGLU: 128 gate rows and 128 up rows per block, so N % 256 as well
  return a_rows >= 1 && K > 0 && K % WKS == 0 && K <= kWideMaxK && N > 0 && N % 256 == 0;
}

void launch_wide(WideParams p, bool swiglu, int64_t n_tiles_bound, int n_cu, hipStream_t s) {
  if (swiglu) launch_w<true>(p, n_tiles_bound, n_cu, s);
  else launch_w<false>(p, n_tiles_bound, n_cu, s);
}

}  // namespace moeq4
