// Tiled grouped GEMM over groupwise-affine 4-bit weights for gfx950 (MI355X): the
// engine for large groups (hundreds of rows per expert), where the layer is bound by
// the matrix cores rather than by weight bytes.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
// engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph 5 (4-bit weights
// with one bf16 scale and bias per 64, reconstructed tile by tile inside the
// grouped GEMM, with fp32 accumulation).
//
// Arithmetic (exact up to fp32 rounding; no weight is rounded to bf16).  For token t,
// weight row n and one 64-wide group g with scale s and bias b:
//   sum_k x[t,k] (s q[n,k] + b) = s * P' + (b - 128 s) * X,
//   P' = sum_k x[t,k] (128 + q[n,k]),   X = sum_k x[t,k].
// 128 + q is exactly the bf16 with bits 0x4300 | q, so the LDS weight tile holds exact
// values (one AND-OR per pair of codes) and P' is a bf16 matrix-core product with
// exact products, formed per group from zero and added as acc += s * P'.  X comes
// from the same matrix cores (the activation fragments times a fragment of ones) and
// the bias term of four groups at a time is one fp32 matrix-core product
// (v_mfma_f32_16x16x4_f32, the groups as its k).
//
// Work decomposition.  One workgroup per tile of up to 128 rows of one group; it walks
// every block of 256 weight rows (with SwiGLU: 128 gate rows and the matching 128 up
// rows, so the epilogue finds both halves in the same registers) as one sequence of
// 64-K stages, so loads run ahead across block boundaries.  Tiles of one group are
// adjacent and XCD b % 8 takes a contiguous run of them, so a group's weights are
// read from HBM about once per XCD.  Every stage's activations (whole 128-byte lines
// per load instruction) and codes are loaded into VGPRs two stages ahead; while the
// matrix cores work on stage u in one LDS buffer, stage u + 1 is written into the
// other (codes unpacked on the way).  Plain loads rather than direct global->LDS
// loads keep the compiler's wait counts exact: it cannot tell a direct load's LDS
// target from the tile being read and would drain every load in flight before each
// LDS access.  Scales and biases come four groups at a time.  Eight wavefronts: two
// halves of the rows times four quarters of the block; each owns a 64 x 64 output
// block as 4 x 4 MFMA tiles.
//
// Measured at 8192 tokens this engine is no faster than the resident-tile engine: the
// unpacked weight tile is written to and read from LDS every stage, and LDS traffic
// (about 200 KB per compute unit per stage) bounds it.
//
// MFMA (v_mfma_f32_16x16x32_bf16) with the weights as the A operand and the
// activations as B: lane l supplies weight row l % 16 (A) and token l % 16 (B), each
// with the eight k-slots of quarter l / 16; the result holds weight rows
// 4 (l / 16) + i for token l % 16, so four adjacent output columns of one row sit in
// one lane.  A packed word unpacks to the k order 0,4,1,5,2,6,3,7; the activations
// come from the prepared copy stored in that order.  Both operands sit in LDS
// fragment-major: the 16 rows x 32 k of one fragment are one contiguous kilobyte,
// lane l's 16 bytes at 16 l, so every fragment read and every direct load is one
// contiguous kilobyte.
#include "common.h"
#include "internal.h"
#include "q4_stream.h"

namespace moeq4 {

namespace {

constexpr int TM = kTiledBM;             // rows per tile
constexpr int TN = 256;                  // weight rows per block
constexpr int TK = 64;                   // K per stage (one scale group)
constexpr int A_STAGE = TM * TK * 2;     // 16 KB
constexpr int B_STAGE = TN * TK * 2;     // 32 KB
constexpr int RING = 8;                  // stages of X kept
constexpr int OFF_B = 2 * A_STAGE;
constexpr int OFF_SB = OFF_B + 2 * B_STAGE;       // (s, b) bf16 pairs [2][4][TN]
constexpr int OFF_X = OFF_SB + 2 * 4 * TN * 4;    // X per token, fp32 [RING][TM]
constexpr int LDS_BYTES = OFF_X + RING * TM * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// What one lane loads for one stage.
struct StageData {
  u32x4_t a[2];   // activations: 16 bytes of two of the tile's rows (whole 128-byte lines
                  // per load instruction)
  u32x4_t c;      // packed words 4 h .. 4 h + 3 of the stage for this lane's weight row
  u32x2_t sb;     // every fourth stage: the row's scales (h = 0) or biases (h = 1) of the
                  // four stages' groups
};

template <bool SWIGLU>
__global__ __launch_bounds__(512, 1) void q4_tiled_kernel(TiledParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int N = p.N, K = p.K, KW = K >> 3, KG = K >> 6, NK = K / TK;
  const int NCB = SWIGLU ? (N >> 1) / (TN / 2) : N / TN;
  const int UT = NCB * NK;  // stages of the whole tile: block cb, stage st at cb * NK + st

  // ---- this workgroup's tile: XCD b % 8 takes a contiguous run of tiles
  const int cnt = *p.tile_count;
  const int per = (cnt + 7) >> 3;
  const int jx = blockIdx.x >> 3;
  if (jx >= per) return;  // uniform, before any barrier
  const int tile = (blockIdx.x & 7) * per + jx;
  if (tile >= cnt) return;
  const int4 tt = p.tiles[tile];
  const int grp = __builtin_amdgcn_readfirstlane(tt.x);
  const int row0 = __builtin_amdgcn_readfirstlane(tt.y);
  const int nrows = __builtin_amdgcn_readfirstlane(tt.z);
  const bool in_main = grp < p.n_main;
  const int gi = in_main ? grp : 0;
  const uint32_t* Wq = (in_main ? p.main.q : p.last.q) + (int64_t)gi * N * KW;
  const uint16_t* Ws = (in_main ? p.main.s : p.last.s) + (int64_t)gi * N * KG;
  const uint16_t* Wb = (in_main ? p.main.b : p.last.b) + (int64_t)gi * N * KG;

  // ---- activation lanes: rows 16 wave + 8 i + l / 8 (i = 0, 1), 16-byte chunk l % 8 of
  // the stage's 128 bytes; rows past the tile repeat its last row, rows outside
  // [0, a_rows) read row a_rows.  Byte offsets fit 32 bits (a_rows * K < 2^31).
  uint32_t aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = min(16 * wave + 8 * i + (l >> 3), nrows - 1);
    int a = p.a_row_index ? p.a_row_index[row0 + r] : row0 + r;
    if (a < 0 || a >= p.a_rows) a = p.a_rows;
    aoff[i] = ((uint32_t)a * (uint32_t)K + 8u * (l & 7)) * 2u;
  }
  // LDS place of row 8 i + l / 8 of fragment `wave`, step c / 4, quarter c % 4 (c = l % 8);
  // the second row is 8 rows (128 bytes) further
  const uint32_t adst = (uint32_t)((wave * 2 + ((l & 7) >> 2)) * 1024 + (16 * (l & 3) + (l >> 3)) * 16);
  const unsigned char* Abase = (const unsigned char*)p.A;
  // ---- unpacking lanes: weight row dn of the block, half dh of each stage
  const int dn = 32 * wave + (l & 31), dh = l >> 5;
  auto wrow_of = [&](int cb) -> int {
    if (SWIGLU) return dn < TN / 2 ? cb * (TN / 2) + dn : (N >> 1) + cb * (TN / 2) + (dn - TN / 2);
    return cb * TN + dn;
  };
  const uint32_t bdst = (uint32_t)(((dn >> 4) * 2 + dh) * 1024 + (dn & 15) * 16);
  const uint16_t* Wsb = dh ? Wb : Ws;

  // ---- computing lanes: rows 64 wm .., weight fragments jc[]
  const int wm = wave >> 2, wn = wave & 3;
  int jc[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    jc[jj] = SWIGLU ? (jj < 2 ? 2 * wn + jj : 8 + 2 * wn + (jj - 2)) : 4 * wn + jj;
  const int nfw = __builtin_amdgcn_readfirstlane(max(0, min(4, (nrows - 64 * wm + 15) >> 4)));

  uint32_t* SBl = (uint32_t*)(smem + OFF_SB);
  float* Xl = (float*)(smem + OFF_X);
  const uint32_t magic = opaque_magic();
  const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

  auto load = [&](StageData& d, int u) __attribute__((always_inline)) {
    const int cb = u / NK, st = u - cb * NK;
#pragma unroll
    for (int i = 0; i < 2; ++i) d.a[i] = *(const u32x4_t*)(Abase + aoff[i] + st * (TK * 2));
    const int wr = wrow_of(cb);
    d.c = *(const u32x4_t*)(Wq + (int64_t)wr * KW + 8 * st + 4 * dh);
    if ((st & 3) == 0) d.sb = *(const u32x2_t*)(Wsb + (int64_t)wr * KG + st);
  };
  // a stage into LDS buffer u & 1: activations as loaded, codes as 128 + q; every fourth
  // stage the (s, b) pairs of the next four groups (scale in the low half)
  auto store = [&](const StageData& d, int u) __attribute__((always_inline)) {
    const int buf = u & 1, st = u % NK;
#pragma unroll
    for (int i = 0; i < 2; ++i) *(u32x4_t*)(smem + buf * A_STAGE + adst + 128 * i) = d.a[i];
    unsigned char* dst = smem + OFF_B + buf * B_STAGE + bdst;
#pragma unroll
    for (int w = 0; w < 4; ++w) *(u32x4_t*)(dst + w * 256) = unpack_word(d.c[w], magic);
    if ((st & 3) == 0) {
      uint16_t* sbh = (uint16_t*)(SBl + ((u >> 2) & 1) * 4 * TN + dn) + dh;
#pragma unroll
      for (int g = 0; g < 4; ++g) sbh[2 * g * TN] = (uint16_t)(d.sb[g >> 1] >> (16 * (g & 1)));
    }
  };

  f32x4_t acc[4][4];
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[f][jj] = zero;
  };
  reset();

  // scales of stage u for this lane's output columns n = 16 jc + 4 q + i
  auto scales = [&](int u, f32x4_t* sv) __attribute__((always_inline)) {
    const uint32_t* sb = SBl + ((u >> 2) & 1) * 4 * TN + (u & 3) * TN;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const u32x4_t v = *(const u32x4_t*)(sb + 16 * jc[jj] + 4 * q);
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[jj][i] = bf16lo_to_f32(v[i]);
    }
  };

  // One stage: per token fragment, P' of the four weight fragments from zero over the
  // stage's 64 k, then acc += s * P'.  Wavefront (wm, wn) also forms X of
  // token fragment wn of its half for the bias term.
  auto compute = [&](int u) __attribute__((always_inline)) {
    const int buf = u & 1;
    const unsigned char* Ab = smem + buf * A_STAGE;
    const unsigned char* Bb = smem + OFF_B + buf * B_STAGE;
    u32x4_t bw[4][2];
    f32x4_t sv[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int h = 0; h < 2; ++h) bw[jj][h] = *(const u32x4_t*)(Bb + (jc[jj] * 2 + h) * 1024 + 16 * l);
    scales(u, sv);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (f < nfw) {
        const unsigned char* af = Ab + (4 * wm + f) * 2048 + 16 * l;
        const u32x4_t a0 = *(const u32x4_t*)af;
        const u32x4_t a1 = *(const u32x4_t*)(af + 1024);
        f32x4_t P[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) P[jj] = mfma16x16x32(bw[jj][0], a0, zero);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) P[jj] = mfma16x16x32(bw[jj][1], a1, P[jj]);
        if (f == wn) {
          const f32x4_t X = mfma16x16x32(ones, a1, mfma16x16x32(ones, a0, zero));
          Xl[(u % RING) * TM + 64 * wm + 16 * f + m] = X[0];
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[f][jj][i] = fmaf(sv[jj][i], P[jj][i], acc[f][jj][i]);
      }
    }
  };
  // acc += sum over the four stages u0 .. u0 + 3 of (b - 128 s) X: lane l gives
  // A[weight row l % 16][k = l / 16] and B[k = l / 16][token l % 16], k = stage - u0
  auto bias_term = [&](int u0) __attribute__((always_inline)) {
    const uint32_t* sb = SBl + ((u0 >> 2) & 1) * 4 * TN + q * TN;
    float cbv[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t v = sb[16 * jc[jj] + m];
      cbv[jj] = fmaf(-128.f, bf16lo_to_f32(v), bf16hi_to_f32(v));
    }
    const int slot = (u0 + q) % RING;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (f < nfw) {
        const float xv = Xl[slot * TM + 64 * wm + 16 * f + m];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[f][jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(cbv[jj], xv, acc[f][jj], 0, 0, 0);
      }
    }
  };
  // the finished block cb: each lane holds 4 adjacent columns of one row per MFMA tile
  auto epilogue = [&](int cb) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (f < nfw) {
        const int r = 64 * wm + 16 * f + m;
        uint16_t* crow = p.C + (int64_t)(row0 + r) * p.ldc;
        if (SWIGLU) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            float h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gte = acc[f][jj][i], up = acc[f][jj + 2][i];
              h[i] = gte / (1.f + __expf(-gte)) * up;
            }
            uint32_t o0 = pack_bf16x2(h[0], h[1]), o1 = pack_bf16x2(h[2], h[3]);
            if (p.c_perm) {
              // columns 0..3 (q even) and 4..7 (q odd) of a run of 8 go out in the order
              // 0,4,1,5 | 2,6,3,7: swap halves with the lane of the other parity
              const bool odd = q & 1;
              const uint32_t send = odd ? o0 : o1;
              const uint32_t recv = (uint32_t)__shfl_xor((int)send, 16);
              if (!odd) {
                const uint32_t a = o0;
                o0 = (a & 0xFFFFu) | (recv << 16);
                o1 = (a >> 16) | (recv & 0xFFFF0000u);
              } else {
                const uint32_t a = o1;
                o0 = (recv & 0xFFFFu) | (a << 16);
                o1 = (recv >> 16) | (a & 0xFFFF0000u);
              }
            }
            const int col = cb * (TN / 2) + 16 * (2 * wn + jj) + 4 * q;
            if (r < nrows) *(u32x2_t*)(crow + col) = u32x2_t{o0, o1};
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int col = cb * TN + 16 * (4 * wn + jj) + 4 * q;
            if (r < nrows)
              *(u32x2_t*)(crow + col) = u32x2_t{pack_bf16x2(acc[f][jj][0], acc[f][jj][1]),
                                                pack_bf16x2(acc[f][jj][2], acc[f][jj][3])};
          }
        }
      }
    }
  };

  // ---- prologue: stages 0 and 1 loaded, stage 0 stored
  StageData d0, d1;
  load(d0, 0);
  load(d1, 1);
  store(d0, 0);
  lds_barrier();
  // ---- stage loop over every block of the tile: stage u in buffer u & 1.  Stage u + 2
  // is loaded (the last stage is loaded again past the end, so the loop has no branch on
  // the loads), then stage u + 1 goes into the other buffer; at the end it holds the
  // same values a second time, which any wavefront still reading it sees unchanged.
  // After every fourth stage the bias term of those stages; after a block's last stage
  // its outputs, then the accumulators start over.  The two register sets alternate,
  // hence the unrolling by 2 (UT is a multiple of 4).
  auto step = [&](int u, StageData& next, StageData& fresh) __attribute__((always_inline)) {
    load(fresh, min(u + 2, UT - 1));
    compute(u);
    store(next, min(u + 1, UT - 1));
    lds_barrier();
    if ((u & 3) == 3) bias_term(u - 3);
    if (u % NK == NK - 1) {
      epilogue(u / NK);
      reset();
    }
  };
  for (int u = 0; u < UT; u += 2) {
    step(u, d1, d0);
    step(u + 1, d0, d1);
  }
}

template <bool SWIGLU>
void launch_t(const TiledParams& p, int64_t n_tiles_bound, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)q4_tiled_kernel<SWIGLU>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    attr = true;
  }
  const int64_t grid = ((n_tiles_bound > 0 ? n_tiles_bound : 1) + 7) / 8 * 8;
  hipLaunchKernelGGL((q4_tiled_kernel<SWIGLU>), dim3((unsigned)grid), dim3(512), LDS_BYTES, s, p);
}

}  // namespace

bool tiled_supported(int N, int K, bool swiglu, int a_rows) {
  (void)swiglu;  // SwiGLU: 128 gate rows and 128 up rows per unit, so N % 256 as well
  return a_rows >= 1 && K > 0 && K % (4 * TK) == 0 && N > 0 && N % TN == 0;
}

void launch_tiled(TiledParams p, bool swiglu, int64_t n_tiles_bound, hipStream_t s) {
  if (swiglu) launch_t<true>(p, n_tiles_bound, s);
  else launch_t<false>(p, n_tiles_bound, s);
}

}  // namespace moeq4
