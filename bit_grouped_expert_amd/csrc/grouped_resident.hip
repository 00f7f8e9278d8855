// Resident-tile grouped GEMM over groupwise-affine 4-bit weights for gfx950 (MI355X):
// the engine for small groups (a few to a few dozen rows per expert), where the
// layer is bound by streaming expert weights from HBM.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
// engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph 5 (4-bit weights
// with one bf16 scale and bias per 64, reconstructed tile by tile inside the
// grouped GEMM with FP32 accumulation) and paragraph 7 (with little weight reuse,
// memory bandwidth sets the ceiling).
//
// Arithmetic (exact up to fp32 rounding; no weight is rounded to bf16).  For output
// row m, weight row n and one 64-wide group g with scale s and bias b:
//   sum_c x[m,c] (s q[n,c] + b) = s * P' + (b - 128 s) * X,
//   P' = sum_c x[m,c] (128 + q[n,c]),   X = sum_c x[m,c].
// 128 + q is exactly the bf16 with bits 0x4300 | q (one AND-OR per pair of codes),
// so P' is a bf16 matrix-core product with exact products, and s * P' one FMA per
// output and group.  X comes from the same matrix cores (the activation fragment times
// a fragment of ones) and is kept in LDS as three bf16 pieces whose sum is X exactly;
// once per chunk the bias term is b X - 128 (s X), bf16 matrix-core products of those
// pieces with the chunk's s and b words (exact products), so it costs the same
// whatever the bias: with four stages per chunk it is the accumulators' starting value,
// formed while the chunk's first weight stage is in flight (the s and b words loaded
// with the chunk's prefetch setup); with fewer it is added at the chunk's end from the
// words the stages streamed.
//
// Work decomposition.  Tiles hold up to 32 rows of one group.  A tile's weight
// rows are cut into chunks of 128 or 256 rows; the list of (tile, chunk) pairs is
// split into equal contiguous ranges, one per workgroup, and the workgroups of one
// XCD (workgroup b runs on XCD b % 8) take adjacent ranges, so the chunks of one
// group run in one L2.  A workgroup walks its range tile by tile: it copies the
// tile's activation rows for the whole K into LDS once (direct global->LDS loads,
// rows gathered through the row index), then its eight wavefronts stream their
// weight rows from HBM straight into VGPRs with 16-byte loads, up to three stages of
// 256 K ahead, with no workgroup barrier inside the K loop.  A stage covers a whole
// 128-byte line of every weight row it touches.  With K >= 1024 the eight wavefronts are
// four column groups times two halves of K, and the halves are added through LDS
// at the end of each chunk; otherwise eight column groups each take the whole K.
// Each wavefront owns two 16-row weight fragments per chunk (SwiGLU: the gate
// fragment and the matching up fragment), so equal work lands on every wavefront.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16): lane l supplies row l % 16 of A and
// column l % 16 of B, each with the eight k-slots of quarter l / 16; the result
// holds rows 4 (l / 16) + i, column l % 16.  In each 128-K half of a stage, quarter q
// loads packed words 4q .. 4q+3 of its weight row; two permlane32 swaps between
// lanes l and l ^ 32 regroup them so that each pair of MFMA steps draws all four
// quarters' words from one scale group, and the A fragment of each step is read at
// the LDS column of the word the lane holds.  A word unpacks to the k order
// 0,4,1,5,2,6,3,7 and the activations are stored in that order.  LDS holds the activations as [fragment][16-byte
// chunk][16 rows], which makes every fragment read a contiguous 256 bytes per
// quarter-wave.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "q4_stream.h"

namespace moeq4 {

namespace {

constexpr int KS = 256;            // K per stage: four scale groups (two halves of 128)
constexpr int SEG_CAP = 48;        // most tiles one workgroup may touch (host-checked)
constexpr int PART_BYTES = 16384;  // partial sums / output staging
constexpr int kPairSpinLimit = 1 << 16;  // polls before a pair launch's wait gives up

__host__ __device__ constexpr int part_off(int K) { return 2 * (K / 8) * 256; }
// row sums X of the tile's activations per 64-wide group as three bf16 pieces whose sum
// is X exactly: [piece 3][32 rows][32 groups]
constexpr int XP_PIECE = 32 * 32 * 2;
__host__ __device__ constexpr int xs_off(int K) { return part_off(K) + PART_BYTES; }
__host__ __device__ constexpr int seg_off(int K) { return xs_off(K) + 3 * XP_PIECE; }
__host__ __device__ constexpr int idx_off(int K) { return seg_off(K) + SEG_CAP * 16; }
__host__ __device__ constexpr int lds_bytes(int K) { return idx_off(K) + SEG_CAP * 32 * 4; }
static_assert(lds_bytes(kResidentMaxK) <= 160 * 1024, "LDS budget");

template <bool SWIGLU, int NST, int GS>
__device__ __forceinline__ void resident_body(const ResidentParams& p, unsigned char* smem) {
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int N = p.N, K = p.K, KW = K >> 3, KG = K >> 6;
  const int S = p.ksplit;                 // 1 or 2 (host-chosen)
  const int CGN = 8 / S;                  // column groups
  const int cg = wave % CGN, kp = wave / CGN;
  const int CR = 32 * CGN;                // weight rows per chunk
  const int NCH = N / CR;
  constexpr int D = NST;  // register sets: the next D - 1 stages are in flight
  const int kbase = kp * NST;             // this wavefront's K stages: kbase .. kbase + NST - 1
  const int A_FRAG = KW * 256;
  unsigned char* part = smem + part_off(K);
  int4* segt = (int4*)(smem + seg_off(K));
  int* idxt = (int*)(smem + idx_off(K));

  // ---- this workgroup's (tile, chunk) pairs.  With few tiles per workgroup: an equal
  // contiguous range of the pairs, the workgroups of one XCD on adjacent ranges.  With
  // at least eight tiles per workgroup: XCD x takes the x-th eighth of the tiles and
  // deals them round robin to its workgroups, each taking whole tiles, so that at any
  // time an XCD works on a few consecutive groups whose weights its L2 shares.
  const int cnt = *p.tile_count;
  const int G = gridDim.x, WX = G >> 3;  // workgroups per XCD
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
  const bool dealt = cnt >= 8 * G;
  int c_begin, c_end, t_first, nseg, t_lo = 0;
  if (dealt) {
    t_lo = (int)((int64_t)cnt * xcd / 8);
    const int t_hi = (int)((int64_t)cnt * (xcd + 1) / 8);
    nseg = t_lo + jw < t_hi ? (t_hi - t_lo - jw + WX - 1) / WX : 0;
    c_begin = 0;
    c_end = nseg * NCH;
    t_first = 0;
  } else {
    const int rank = xcd * WX + jw;
    const int64_t total = (int64_t)cnt * NCH;
    c_begin = (int)(total * rank / G);
    c_end = (int)(total * (rank + 1) / G);
    if (p.pair_role == 2 && p.pair_wd > 0) {
      // down phase of a pair launch: split so that every workgroup's gate_up share plus its
      // down share weighs the same (a chunk weighs its weight rows times K): the down
      // prefix of rank r is the whole-launch share of r ranks less the gate_up chunks of
      // those ranks, in down chunks, rounded.  It stays within a few chunks of the gate_up
      // split and is increasing while a rank's down share exceeds the weight ratio + 2.
      const int64_t tu = (int64_t)cnt * p.ready_need, wu = p.pair_wu, wd = p.pair_wd;
      if (total * wd >= (int64_t)G * (wu + 2 * wd)) {
        auto prefix = [&](int64_t r) -> int64_t {
          const int64_t a = tu * r / G;
          return (2 * (r * (wu * tu + wd * total) - (int64_t)G * wu * a) + (int64_t)G * wd) /
                 (2 * (int64_t)G * wd);
        };
        c_begin = (int)prefix(rank);
        c_end = (int)prefix(rank + 1);
      }
    }
    t_first = c_begin / NCH;
    nseg = c_begin < c_end ? (c_end - 1) / NCH - t_first + 1 : 0;
  }
  if (c_begin >= c_end) return;  // uniform, before any barrier
  if (nseg > SEG_CAP) return;    // excluded by the host; never write past the table
  // a pair launch numbers chunks over the whole tile list (never dealt: excluded by the
  // host, and both phases see the same tile count, so neither waits on the other here)
  const int role = p.pair_role;
  if (role != 0 && dealt) {
    if (threadIdx.x == 0) atomic_add_agent(p.sync, 1);
    return;
  }
  // chunk i of this workgroup's sequence.  The down phase of a pair launch starts after
  // the tile it shares with the previous range (that range runs its gate_up part of the
  // tile last) and ends with it.
  const int n_ch = c_end - c_begin;
  int rot = 0;
  if (role == 2 && c_begin % NCH != 0) {
    const int first_full = (c_begin / NCH + 1) * NCH;
    if (first_full < c_end) rot = first_full - c_begin;
  }
  auto seq = [&](int i) -> int {
    const int j = i + rot;
    return c_begin + (j < n_ch ? j : j - n_ch);
  };
  // segment k's tile: the k-th of the range, or the k-th dealt to this workgroup
  auto tile_of = [&](int k) -> int { return dealt ? t_lo + jw + WX * k : t_first + k; };
  // tiles and activation row indices of every segment, before any weight load
  for (int e = tid; e < nseg * 32; e += 512) {
    const int k = e >> 5, rr = e & 31;
    const int4 t = p.tiles[tile_of(k)];
    if (rr == 0) segt[k] = t;
    const int row = t.y + (rr < t.z ? rr : t.z - 1);
    int a = p.a_row_index ? p.a_row_index[row] : row;
    if (a < 0 || a >= p.a_rows) a = p.a_rows;  // the zero row
    idxt[e] = a;
  }
  __syncthreads();

  auto seg_of = [&](int ch) -> int4 {
    const int k = ch / NCH - t_first;
    const int4 t = segt[k];
    return make_int4(__builtin_amdgcn_readfirstlane(t.x), __builtin_amdgcn_readfirstlane(t.y),
                     __builtin_amdgcn_readfirstlane(t.z), k);
  };

  // ---- weight prefetch cursor (stream of this wavefront's stages over its chunks)
  int pf_i = 0, pf_s = 0;
  const uint32_t* pf_q = nullptr;
  const uint16_t* pf_sc = nullptr;
  const uint16_t* pf_bi = nullptr;
  uint32_t pf_co[2], pf_so[2];
  // The s and b words of the prefetched chunk that this lane feeds to the chunk's bias
  // product: eight groups of this wavefront's 4 NST, from group sb_g0 (NST <= 2: groups
  // 0 .. 7; NST >= 3: groups 8 (q & 1) .. + 7), as two 8-byte halves; the second half
  // only where its groups exist (else it is loaded again from the first and not used).
  constexpr bool kStartBias = NST >= 3;  // else the product at the chunk's end
  const int sb_g0 = NST >= 3 ? 8 * (q & 1) : 0;
  const bool sb_hi = sb_g0 + 4 < 4 * NST;
  u32x2_t sb_s[2][2], sb_b[2][2];  // [weight fragment][half]
  auto pf_chunk = [&]() __attribute__((always_inline)) {
    const int pf_ch = seq(pf_i);
    const int4 t = seg_of(pf_ch);
    const int cin = pf_ch - (pf_ch / NCH) * NCH;
    const int g = t.x;
    const bool in_main = g < p.n_main;
    const int gi = in_main ? g : 0;
    pf_q = (in_main ? p.main.q : p.last.q) + (int64_t)gi * N * KW;
    pf_sc = (in_main ? p.main.s : p.last.s) + (int64_t)gi * N * KG;
    pf_bi = (in_main ? p.main.b : p.last.b) + (int64_t)gi * N * KG;
    int n0, n1;
    if (SWIGLU) {
      const int u = CGN * cin + cg;
      n0 = 16 * u + m;
      n1 = (N >> 1) + 16 * u + m;
    } else {
      n0 = CR * cin + 32 * cg + m;
      n1 = n0 + 16;
    }
    pf_co[0] = ((uint32_t)n0 * KW + 4 * q) * 4u;
    pf_co[1] = ((uint32_t)n1 * KW + 4 * q) * 4u;
    pf_so[0] = (uint32_t)n0 * KG * 2u;
    pf_so[1] = (uint32_t)n1 * KG * 2u;
#pragma unroll
    for (int j = 0; j < 2 && kStartBias; ++j) {
      const uint32_t o = pf_so[j] + (uint32_t)(4 * kbase + sb_g0) * 2u;
      const uint32_t o2 = sb_hi ? o + 8u : o;
      sb_s[j][0] = ld<u32x2_t>(pf_sc, o);
      sb_s[j][1] = ld<u32x2_t>(pf_sc, o2);
      sb_b[j][0] = ld<u32x2_t>(pf_bi, o);
      sb_b[j][1] = ld<u32x2_t>(pf_bi, o2);
    }
  };
  auto pf_load = [&](StageW& w) __attribute__((always_inline)) {
    const int st = kbase + pf_s;
    const uint32_t* qs = pf_q + 32 * st;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      w.c[j][0] = ld<u32x4_t>(qs, pf_co[j]);
      w.c[j][1] = ld<u32x4_t>(qs + 16, pf_co[j]);
      w.s[j] = ld<u32x2_t>(pf_sc + 4 * st, pf_so[j]);
      w.b[j] = ld<u32x2_t>(pf_bi + 4 * st, pf_so[j]);
    }
    if (++pf_s == NST) {
      pf_s = 0;
      if (++pf_i < n_ch) pf_chunk();
    }
  };

  const uint32_t magic = opaque_magic();
  const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  // word held in MFMA step t of a 128-K half, after the swaps
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
  // LDS byte offset of this lane's A fragment row for each step (chunk = word of the half)
  uint32_t a_step[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) a_step[t] = widx[t] * 256u + 16u * m;

  f32x4_t acc[2][2];  // [row fragment][weight fragment]

  // One 256-K stage in two 128-K halves.  In a half, MFMA steps 2 (g ^ GS) and
  // 2 (g ^ GS) + 1 take scale group g of the half (GS: the group order the swaps
  // produce, uniform and fixed by the hardware; both orders are compiled).  Each half
  // runs in three phases kept apart by scheduling barriers, so that matrix results are
  // consumed only after all of the half's chains are issued: operands (LDS reads and
  // unpacked weights), then the MFMA chains, then acc += s * P'.  The bias term
  // (b - 128 s) X is the accumulators' starting value (bias_init, NST >= 3) or added at
  // the chunk's end (bias_term, NST <= 2).
  auto compute = [&](const StageW& w, int st, auto nf_tag) __attribute__((always_inline)) {
    constexpr int NF = decltype(nf_tag)::value;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const unsigned char* ab = smem + ((uint32_t)st * 2 + hh) * 4096u;
      u32x4_t av[2][NF][2];  // [group][row fragment][half step]
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            av[g][f][h] = *(const u32x4_t*)(ab + f * A_FRAG + a_step[2 * (g ^ GS) + h]);
      u32x4_t B[2][2][2];  // [group][weight fragment][half step]
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t wsw = swap_quad(w.c[j][hh]);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int h = 0; h < 2; ++h) B[g][j][h] = unpack_word(wsw[2 * (g ^ GS) + h], magic);
      }
      float sc[2][2];  // [group][weight fragment]
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        sc[0][j] = bf16lo_to_f32(w.s[j][hh]);
        sc[1][j] = bf16hi_to_f32(w.s[j][hh]);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t P[2][2][NF];
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int j = 0; j < 2; ++j) P[g][j][f] = mfma16x16x32(av[g][f][0], B[g][j][0], zero);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int j = 0; j < 2; ++j) P[g][j][f] = mfma16x16x32(av[g][f][1], B[g][j][1], P[g][j][f]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[f][j][i] = fmaf(sc[g][j], P[g][j][f][i], acc[f][j][i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- weight register sets, D - 1 stages in flight from the prologue (issued with the
  // first tile below).  Every wavefront issues the same loads for every stage, also past
  // the end of its stream (those reload a valid stage and are never used), so that the
  // compiler's wait counts stay exact across the loop.
  StageW W[D];

  // The s and b words this lane feeds to the bias product, [weight fragment] x eight
  // groups of this wavefront's 4 NST: with NST <= 2 groups 0 .. 7 on every lane, with
  // NST >= 3 groups 8 (q & 1) .. 8 (q & 1) + 7.  Slots of groups past 4 NST stay zero.
  u32x4_t sw_s[2], sw_b[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    sw_s[j] = u32x4_t{0u, 0u, 0u, 0u};
    sw_b[j] = sw_s[j];
  }
  auto capture_sb = [&](int d, const StageW& w) __attribute__((always_inline)) {
    if constexpr (kStartBias) return;
    const int h = d & 1;  // groups 4 d .. 4 d + 3 of the wavefront: words 2 h, 2 h + 1
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (NST <= 2 || d < 2) {
        const bool take = NST <= 2 || (q & 1) == 0;
        sw_s[j][2 * h] = take ? w.s[j][0] : sw_s[j][2 * h];
        sw_s[j][2 * h + 1] = take ? w.s[j][1] : sw_s[j][2 * h + 1];
        sw_b[j][2 * h] = take ? w.b[j][0] : sw_b[j][2 * h];
        sw_b[j][2 * h + 1] = take ? w.b[j][1] : sw_b[j][2 * h + 1];
      } else {
        const bool take = (q & 1) == 1;
        sw_s[j][2 * h] = take ? w.s[j][0] : sw_s[j][2 * h];
        sw_s[j][2 * h + 1] = take ? w.s[j][1] : sw_s[j][2 * h + 1];
        sw_b[j][2 * h] = take ? w.b[j][0] : sw_b[j][2 * h];
        sw_b[j][2 * h + 1] = take ? w.b[j][1] : sw_b[j][2 * h + 1];
      }
    }
  };
  // One chunk: NST stages, stage s on register set s (D == NST, so the rotation starts
  // over with every chunk).  The loads stay outside the branch on the fragment count:
  // identical loads in both arms would be merged into the join block, after the matrix
  // work, which would turn the prefetch into load-then-wait.
  auto run_chunk = [&](int nfv) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      pf_load(W[(d + D - 1) % D]);
      if (nfv == 2) compute(W[d], kbase + d, std::integral_constant<int, 2>{});
      else compute(W[d], kbase + d, std::integral_constant<int, 1>{});
      capture_sb(d, W[d]);
    }
  };
  // acc starts as the chunk's bias term, sum over this wavefront's groups of
  // (b - 128 s) X, exactly up to fp32 rounding, formed while the chunk's first weight
  // stage is still in flight: bf16 matrix-core products (v_mfma_f32_16x16x32_bf16: lane
  // (m, q) gives k = 8 q .. 8 q + 7 of row m, lane (n, q) the same k of column n) of b
  // and s with the three pieces of X, then acc = b X - 128 (s X).  NST <= 2: k = 8 p + g,
  // piece p of X (quarter 3 zero), groups g 0 .. 7.  NST >= 3: first product quarters
  // (piece, group half) = (hi, 0), (hi, 1), (mid, 0), (mid, 1), second (lo, 0), (lo, 1),
  // zero.  Group slots past 4 NST have zero s and b.
  const unsigned char* xpb = smem + xs_off(K) + 8 * kbase;  // group 4 kbase, 2 bytes each
  auto bias_init = [&](int nfv) __attribute__((always_inline)) {
    const u32x4_t z4 = {0u, 0u, 0u, 0u};
    u32x4_t bw[2], sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bw[j] = u32x4_t{sb_b[j][0][0], sb_b[j][0][1], sb_hi ? sb_b[j][1][0] : 0u, sb_hi ? sb_b[j][1][1] : 0u};
      sw[j] = u32x4_t{sb_s[j][0][0], sb_s[j][0][1], sb_hi ? sb_s[j][1][0] : 0u, sb_hi ? sb_s[j][1][1] : 0u};
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (f < nfv) {
        const unsigned char* xr = xpb + (16 * f + m) * 64;
        if constexpr (NST <= 2) {
          u32x4_t xa = *(const u32x4_t*)(xr + (q < 3 ? q : 0) * XP_PIECE);
          if (q == 3) xa = z4;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const f32x4_t sx = mfma16x16x32(xa, sw[j], zero);
            acc[f][j] = mfma16x16x32(xa, bw[j], zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[f][j][i] = fmaf(-128.f, sx[i], acc[f][j][i]);
          }
        } else {
          const u32x4_t x1 = *(const u32x4_t*)(xr + (q >> 1) * XP_PIECE + 16 * (q & 1));
          u32x4_t x2 = *(const u32x4_t*)(xr + 2 * XP_PIECE + 16 * (q & 1));
          if (q >= 2) x2 = z4;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const f32x4_t sx = mfma16x16x32(x2, sw[j], mfma16x16x32(x1, sw[j], zero));
            acc[f][j] = mfma16x16x32(x2, bw[j], mfma16x16x32(x1, bw[j], zero));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[f][j][i] = fmaf(-128.f, sx[i], acc[f][j][i]);
          }
        }
      } else {
        acc[f][0] = zero;
        acc[f][1] = zero;
      }
    }
  };

  // acc += sum over this wavefront's groups of (b - 128 s) X, exactly up to fp32
  // rounding, as bf16 matrix-core products (v_mfma_f32_16x16x32_bf16: lane (m, q) gives
  // k = 8 q .. 8 q + 7 of row m, lane (n, q) the same k of column n): b X and s X over
  // the three pieces of X, then acc += b X - 128 (s X).  NST <= 2: k = 8 p + g, piece p
  // of X (quarter 3 zero), groups g 0 .. 7.  NST >= 3: first product quarters (piece,
  // group half) = (hi, 0), (hi, 1), (mid, 0), (mid, 1), second (lo, 0), (lo, 1), zero.
  auto bias_term = [&](int nfv) __attribute__((always_inline)) {
    const u32x4_t z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int f = 0; f < 2; ++f)
      if (f < nfv) {
        const unsigned char* xr = xpb + (16 * f + m) * 64;
        if constexpr (NST <= 2) {
          u32x4_t xa = *(const u32x4_t*)(xr + (q < 3 ? q : 0) * XP_PIECE);
          if (q == 3) xa = z4;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const u32x4_t bq = q < 3 ? sw_b[j] : z4, sq = q < 3 ? sw_s[j] : z4;
            const f32x4_t sx = mfma16x16x32(xa, sq, zero);
            acc[f][j] = mfma16x16x32(xa, bq, acc[f][j]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[f][j][i] = fmaf(-128.f, sx[i], acc[f][j][i]);
          }
        } else {
          const u32x4_t x1 = *(const u32x4_t*)(xr + (q >> 1) * XP_PIECE + 16 * (q & 1));
          u32x4_t x2 = *(const u32x4_t*)(xr + 2 * XP_PIECE + 16 * (q & 1));
          if (q >= 2) x2 = z4;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const f32x4_t sx = mfma16x16x32(x2, sw_s[j], mfma16x16x32(x1, sw_s[j], zero));
            acc[f][j] = mfma16x16x32(x2, sw_b[j], mfma16x16x32(x1, sw_b[j], acc[f][j]));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[f][j][i] = fmaf(-128.f, sx[i], acc[f][j][i]);
          }
        }
      }
  };

  // X of the tile: the product of each group's two 32-K activation fragments with a
  // fragment of ones, written by the lanes of column 0 as three bf16 pieces (each the top
  // eight significant bits of what the previous ones left); then a barrier
  auto tile_row_sums = [&](int nfv) __attribute__((always_inline)) {
    unsigned char* xw = smem + xs_off(K);
    const int KG4 = K >> 6;
    for (int pi = wave; pi < nfv * KG4; pi += 8) {
      const int f = pi / KG4, g = pi - f * KG4;
      const unsigned char* ab = smem + f * A_FRAG + (8 * g + 2 * q) * 256 + 16 * m;
      const u32x4_t a0 = *(const u32x4_t*)ab;
      const u32x4_t a1 = *(const u32x4_t*)(ab + 256);
      const f32x4_t X = mfma16x16x32(a1, ones, mfma16x16x32(a0, ones, zero));
      if (m == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t hi = __float_as_uint(X[i]) & 0xFFFF0000u;
          const float r1 = X[i] - __uint_as_float(hi);
          const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
          const uint32_t lo = __float_as_uint(r1 - __uint_as_float(mid)) & 0xFFFF0000u;
          const int off = (16 * f + 4 * q + i) * 64 + 2 * g;
          *(uint16_t*)(xw + off) = (uint16_t)(hi >> 16);
          *(uint16_t*)(xw + XP_PIECE + off) = (uint16_t)(mid >> 16);
          *(uint16_t*)(xw + 2 * XP_PIECE + off) = (uint16_t)(lo >> 16);
        }
      }
    }
    lds_barrier();
  };

  const int per_f = K >> 5;  // 1 KB pieces (32 K of 16 rows) per activation fragment
  // segment k's activation rows for the whole K: fragment f, 16-byte chunks 4 cb .. 4 cb + 3
  // of its 16 rows per direct load (1 KB of LDS); device-scope loads in the down phase of
  // a pair launch (rows written by other workgroups of the launch)
  auto gather = [&](int k, int nfv) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (f < nfv) {
        const int arow = idxt[k * 32 + 16 * f + m];
        const uint16_t* src = p.A + (int64_t)arow * K + 8 * q;
        if (role == 2) {
          for (int cb = wave; cb < per_f; cb += 8)
            __builtin_amdgcn_global_load_lds(src + 32 * cb, smem + f * A_FRAG + cb * 1024, 16, 0, 16);
        } else {
          for (int cb = wave; cb < per_f; cb += 8)
            __builtin_amdgcn_global_load_lds(src + 32 * cb, smem + f * A_FRAG + cb * 1024, 16, 0, 0);
        }
      }
    }
  };
  // pair launch, down phase: one wavefront waits until every gate_up chunk of `tile` has
  // been counted (bounded: past the limit it counts the failure in sync[0] and goes on)
  auto wait_tile = [&](int tile) __attribute__((always_inline)) {
    if (wave == 0) {
      const uint32_t* cnt = (const uint32_t*)(p.sync + kPairTileBase + tile);
      int spins = 0;
      while ((int)load_dev(cnt) < p.ready_need) {
        if (++spins > kPairSpinLimit) {
          if (l == 0) atomic_add_agent(p.sync, 1);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    lds_barrier();
  };

  int cur_seg;
  if (role == 2) {
    // the weight prologue first (it does not depend on the gate_up phase), then the wait,
    // then the first tile's activations
    const int c0 = seq(0);
    const int4 t = seg_of(c0);
    const int nf0 = t.z > 16 ? 2 : 1;
    pf_chunk();
#pragma unroll
    for (int d = 0; d < D - 1; ++d) pf_load(W[d]);
    for (int o = 16 * tid; o < 3 * XP_PIECE; o += 16 * 512)
      *(u32x4_t*)(smem + xs_off(K) + o) = u32x4_t{0u, 0u, 0u, 0u};
    wait_tile(c0 / NCH);
    gather(t.w, nf0);
    wait_vmcnt0();
    lds_barrier();
    tile_row_sums(nf0);
    cur_seg = t.w;
  } else {
    // the first tile's activation rows go through VGPRs, loaded before the weight
    // prologue: waiting for them then leaves the weight loads in flight (after direct
    // loads into LDS, the first LDS read would wait for every load issued before it)
    const int4 t = seg_of(seq(0));
    const int nf0 = t.z > 16 ? 2 : 1;
    u32x4_t a_first[2][8];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int arow = idxt[t.w * 32 + 16 * f + m];
      const uint16_t* src = p.A + (int64_t)arow * K + 8 * q;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int cb = wave + 8 * i;
        if (f < nf0 && cb < per_f) a_first[f][i] = *(const u32x4_t*)(src + 32 * cb);
      }
    }
    pf_chunk();
#pragma unroll
    for (int d = 0; d < D - 1; ++d) pf_load(W[d]);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int cb = wave + 8 * i;
        if (f < nf0 && cb < per_f) *(u32x4_t*)(smem + f * A_FRAG + cb * 1024 + 16 * l) = a_first[f][i];
      }
    // the pieces of X zeroed once (groups past K stay zero)
    for (int o = 16 * tid; o < 3 * XP_PIECE; o += 16 * 512)
      *(u32x4_t*)(smem + xs_off(K) + o) = u32x4_t{0u, 0u, 0u, 0u};
    lds_barrier();
    tile_row_sums(nf0);
    cur_seg = t.w;
  }
  int pend = -1;  // gate_up phase of a pair launch: tile of the chunk not yet counted
  for (int ci = 0; ci < n_ch; ++ci) {
    const int ch = seq(ci);
    const int4 t = seg_of(ch);
    const int k = t.w, row0 = t.y, nrows = t.z;
    const int nfv = nrows > 16 ? 2 : 1;
    const int cin = ch - (ch / NCH) * NCH;
    if (k != cur_seg) {
      lds_barrier();  // every wavefront is done with the previous tile
      if (role == 2) wait_tile(ch / NCH);
      gather(k, nfv);
      wait_vmcnt0();
      lds_barrier();
      tile_row_sums(nfv);
      cur_seg = k;
    }
    if constexpr (kStartBias) {
      bias_init(nfv);
      run_chunk(nfv);
    } else {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[f][j] = zero;
      run_chunk(nfv);
      bias_term(nfv);
    }

    if (role == 1) {
      // the previous chunk's outputs are complete: this chunk's last stage was loaded after
      // they were stored, and every wavefront has waited for that stage
      lds_barrier();
      if (tid == 0 && pend >= 0) atomic_add_agent(p.sync + kPairTileBase + pend, 1);
      pend = ch / NCH;
    }
    // ---- end of chunk: halves of K meet through LDS, then bf16 rows go out
    bool owner = true;
    unsigned char* stg = part + wave * 2048;
    if (S == 2) {
      f32x4_t* pw = (f32x4_t*)(part + cg * 4096) + l;
      lds_barrier();  // the previous chunk's partial sums have been consumed
      if (kp == 1) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
          if (f < nfv) {
            pw[(2 * f + 0) * 64] = acc[f][0];
            pw[(2 * f + 1) * 64] = acc[f][1];
          }
      }
      lds_barrier();
      owner = kp == 0;
      if (owner) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
          if (f < nfv) {
            const f32x4_t o0 = pw[(2 * f + 0) * 64], o1 = pw[(2 * f + 1) * 64];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[f][0][i] += o0[i];
              acc[f][1][i] += o1[i];
            }
          }
      }
      stg = part + cg * 4096;
    }
    if (owner) {
      uint16_t* cs = (uint16_t*)stg;
      if (SWIGLU) {
        // 16 output columns: silu(gate) * up, in the prepared column order if asked
        const int col = p.c_perm ? ((m & 8) | perm8(m & 7)) : m;
#pragma unroll
        for (int f = 0; f < 2; ++f)
          if (f < nfv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gte = acc[f][0][i], up = acc[f][1][i];
              const float h = gte / (1.f + __expf(-gte)) * up;
              cs[(16 * f + 4 * q + i) * 16 + col] = to_bf16(h);
            }
          }
        const int r = l >> 1, half = l & 1;
        const int u = CGN * cin + cg;
        if (r < nrows) {
          uint16_t* dst = p.C + (int64_t)(row0 + r) * p.ldc + 16 * u + 8 * half;
          const u32x4_t v = *(const u32x4_t*)(cs + r * 16 + 8 * half);
          if (role == 1) store_dev16(dst, v);
          else *(u32x4_t*)dst = v;
        }
      } else {
#pragma unroll
        for (int f = 0; f < 2; ++f)
          if (f < nfv) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                cs[(16 * f + 4 * q + i) * 32 + 16 * j + m] = to_bf16(acc[f][j][i]);
          }
        const int col0 = CR * cin + 32 * cg;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int r = (64 * pp + l) >> 2, piece = l & 3;
          if (r < nrows) {
            uint16_t* dst = p.C + (int64_t)(row0 + r) * p.ldc + col0 + 8 * piece;
            const u32x4_t v = *(const u32x4_t*)(cs + r * 32 + 8 * piece);
            if (role == 1) store_dev16(dst, v);
            else *(u32x4_t*)dst = v;
          }
        }
      }
    }
    // keeps the stores ahead of the next chunk's loads in program order
    asm volatile("" ::: "memory");
  }
  if (role == 1) {
    // the last chunk: wait for the stores themselves
    wait_vmcnt0();
    lds_barrier();
    if (tid == 0 && pend >= 0) atomic_add_agent(p.sync + kPairTileBase + pend, 1);
  }
}

}  // namespace

// GS: scale group of MFMA steps 0 and 1 after the word swaps (0 or 1), the same on
// every lane and every call; read off the swapped word numbers on entry, and both
// orders are compiled, so the result never depends on the swap's direction.
template <bool SWIGLU, int NST>
__global__ __launch_bounds__(512, 1) void q4_resident_kernel(ResidentParams p) {
  // sized for the largest K: every launch fits without a per-kernel attribute
  __shared__ __attribute__((aligned(16))) unsigned char smem_dyn[lds_bytes(kResidentMaxK)];
  const int l = threadIdx.x & 63;
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)(4 * (l >> 4)), (uint32_t)(4 * (l >> 4) + 2),
                                                  false, false);
  const int gs = __builtin_amdgcn_readfirstlane((int)(r[0] >> 3));
  if (gs) resident_body<SWIGLU, NST, 1>(p, smem_dyn);
  else resident_body<SWIGLU, NST, 0>(p, smem_dyn);
}

// gate_up (+ SwiGLU) then down in one launch: each workgroup runs its gate_up range, then
// its down range over the same tiles (the chunk counts per tile are equal at the layer's
// shapes, so both ranges cover about the same rows), so that the down weights start
// streaming as soon as a workgroup's gate_up share is done instead of after the slowest
// workgroup's.  Every workgroup must be resident at once: the grid is one workgroup per
// compute unit (the LDS of one takes a whole unit).
template <int NU, int ND>
__global__ __launch_bounds__(512, 1) void q4_resident_pair_kernel(ResidentParams up, ResidentParams dn) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_dyn[lds_bytes(kResidentMaxK)];
  const int l = threadIdx.x & 63;
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)(4 * (l >> 4)), (uint32_t)(4 * (l >> 4) + 2),
                                                  false, false);
  const int gs = __builtin_amdgcn_readfirstlane((int)(r[0] >> 3));
  if (gs) {
    resident_body<true, NU, 1>(up, smem_dyn);
    lds_barrier();
    resident_body<false, ND, 1>(dn, smem_dyn);
  } else {
    resident_body<true, NU, 0>(up, smem_dyn);
    lds_barrier();
    resident_body<false, ND, 0>(dn, smem_dyn);
  }
}

namespace {

template <int NU, int ND>
void launch_pair_one(const ResidentParams& up, const ResidentParams& dn, int grid, hipStream_t s) {
  hipLaunchKernelGGL((q4_resident_pair_kernel<NU, ND>), dim3(grid), dim3(512), 0, s, up, dn);
}

template <bool SWIGLU, int NST>
void launch_one(const ResidentParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((q4_resident_kernel<SWIGLU, NST>), dim3(grid), dim3(512), 0, s, p);
}

template <bool SWIGLU>
void launch_nst(const ResidentParams& p, int nst, int grid, hipStream_t s) {
  switch (nst) {
    case 1: launch_one<SWIGLU, 1>(p, grid, s); break;
    case 2: launch_one<SWIGLU, 2>(p, grid, s); break;
    case 3: launch_one<SWIGLU, 3>(p, grid, s); break;
    default: launch_one<SWIGLU, 4>(p, grid, s); break;
  }
}

}  // namespace

bool resident_plan(int N, int K, bool swiglu, int64_t n_tiles_bound, int n_cu, ResidentPlan* out) {
  (void)swiglu;
  if (K <= 0 || K % KS != 0 || K > kResidentMaxK || N <= 0) return false;
  const int KP = K / KS;  // 256-K stages
  int S = (KP % 2 == 0 && KP >= 4) ? 2 : 1;
  if (N % (32 * (8 / S)) != 0) {
    if (S == 1 && KP % 2 == 0 && N % 128 == 0) S = 2;
    else return false;
  }
  const int nst = KP / S;
  if (nst < 1 || nst > kResidentMaxStages) return false;
  int grid = (n_cu > 0 ? n_cu : 256) / 8 * 8;
  if (grid < 8) grid = 8;
  const int64_t NCH = N / (32 * (8 / S));
  const int64_t chunks = (n_tiles_bound > 0 ? n_tiles_bound : 1) * NCH;
  const int64_t per_wg = (chunks + grid - 1) / grid;
  const int64_t segs = (per_wg - 1) / NCH + 2;
  if (segs > SEG_CAP) return false;
  // tiles dealt round robin (at least eight per workgroup): an XCD's share over its
  // workgroups
  const int64_t tiles = n_tiles_bound > 0 ? n_tiles_bound : 1;
  if (((tiles + 7) / 8 + grid / 8 - 1) / (grid / 8) > SEG_CAP) return false;
  if (out) {
    out->ksplit = S;
    out->stages = nst;
    out->grid = grid;
  }
  return true;
}

void launch_resident(ResidentParams p, const ResidentPlan& plan, bool swiglu, hipStream_t s) {
  p.ksplit = plan.ksplit;
  if (swiglu) launch_nst<true>(p, plan.stages, plan.grid, s);
  else launch_nst<false>(p, plan.stages, plan.grid, s);
}

bool resident_pair_ok(const ResidentPlan& up, const ResidentPlan& down, int N_up, int K_up, int N_dn,
                      int K_dn, int64_t n_tiles_bound) {
  if (up.grid != down.grid || up.grid < 8) return false;
  if (up.stages != 2 && up.stages != 4) return false;
  if (down.stages != 1 && down.stages != 2) return false;
  // never the dealt mode (at least eight tiles per workgroup)
  if (n_tiles_bound <= 0 || n_tiles_bound >= 8 * (int64_t)up.grid) return false;
  // the weighted down split gives a workgroup at most its even share plus the weight ratio
  // plus two chunks: its tiles must fit the segment table
  const int64_t cr_up = 32 * (8 / up.ksplit), cr_dn = 32 * (8 / down.ksplit);
  const int64_t nch_dn = N_dn / cr_dn;
  const int64_t ratio = (cr_up * K_up + cr_dn * K_dn - 1) / (cr_dn * K_dn);
  const int64_t per_wg = (n_tiles_bound * nch_dn + up.grid - 1) / up.grid + ratio + 2;
  (void)N_up;
  return (per_wg - 1) / nch_dn + 2 <= SEG_CAP;
}

void launch_resident_pair(ResidentParams up, ResidentParams down, const ResidentPlan& pu,
                          const ResidentPlan& pd, int32_t* sync, hipStream_t s) {
  up.ksplit = pu.ksplit;
  down.ksplit = pd.ksplit;
  up.pair_role = 1;
  down.pair_role = 2;
  up.sync = down.sync = sync;
  up.ready_need = down.ready_need = 0;
  // a tile is ready for the down phase once all its gate_up chunks are counted
  down.ready_need = up.N / (32 * (8 / pu.ksplit));
  // chunk weights (weight rows times K) of the two phases, for the balanced down split
  down.pair_wu = 32 * (8 / pu.ksplit) * up.K;
  down.pair_wd = 32 * (8 / pd.ksplit) * down.K;
  if (pu.stages == 4) {
    if (pd.stages == 2) launch_pair_one<4, 2>(up, down, pu.grid, s);
    else launch_pair_one<4, 1>(up, down, pu.grid, s);
  } else {
    if (pd.stages == 2) launch_pair_one<2, 2>(up, down, pu.grid, s);
    else launch_pair_one<2, 1>(up, down, pu.grid, s);
  }
}

}  // namespace moeq4
