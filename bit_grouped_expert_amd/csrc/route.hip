// Router of the MoE layer: fp32 logits, top-k selection and routing weights.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
// engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph 4 (a router
// scores 256 experts and picks eight, plus a shared expert that sees every
// token).  The weighting (softmax over the selected logits) and the tie rule
// (equal logits go to the lower expert id) are readings; the pages state neither.
//
// Logits.  L = x R^T with x bf16 [T, D] and R fp32 [E, D].  R is split once per
// call into three bf16 planes R = R0 + R1 + R2 (each the round-to-nearest-even of
// the remainder), which carries R's full 24-bit significand.  A product of a bf16
// x with a bf16 plane is exact in fp32, so three bf16 MFMAs with fp32
// accumulation give fp32-FMA accuracy at bf16 matrix-core speed.
//
// Selection.  One wavefront per token ranks the logits by a 64-bit key
// (order-preserving float bits, then the complemented expert id so equal logits
// rank the lower id higher) and extracts the k+1 best.  If the k-th and (k+1)-th
// fp32 logits are closer than `tau`, the experts at least tau above L_(k+1) keep
// their places, and every expert within tau of L_(k+1) is rescored exactly in fp64
// (bf16 x fp32 products are exact in fp64); the best of those, by fp64 logit, fill
// the remaining places.  As long as the fp32 error is under tau/2 the experts above
// are in the exact top k and those below are not, so the selection equals the
// exact (fp64) top-k; the places filled by rescoring are in exact order.
#include "common.h"
#include "internal.h"
#include "topk_select.h"

namespace moeq4 {

// ---------------------------------------------------------------------------- split
// The planes are written fragment-major: for each 16-expert tile `et` and 32-wide
// k-step `s`, the 64 lanes' 16-byte operands of v_mfma_f32_16x16x32_bf16 lie in one
// contiguous kilobyte, lane l = m + 16 q holding expert 16 et + m, k = 32 s + 8 q .. +7.
// Plane p starts at p * Epad * D (Epad = E rounded up to 16; padding experts are zero),
// so every operand load of the logits kernel reads one contiguous kilobyte.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ R,
                                                           uint16_t* __restrict__ Rs, int E, int D) {
  const int nsteps = D >> 5, ET = (E + 15) >> 4;
  const int64_t nfrag = (int64_t)ET * nsteps * 64, plane = (int64_t)ET * 16 * D;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nfrag; i += (int64_t)gridDim.x * 256) {
    const int l = (int)(i & 63);
    const int64_t ts = i >> 6;
    const int s = (int)(ts % nsteps), et = (int)(ts / nsteps);
    const int e = 16 * et + (l & 15), k0 = 32 * s + 8 * (l >> 4);
    float r[8];
    if (e < E) {
      const f32x4_t lo = *(const f32x4_t*)(R + (int64_t)e * D + k0);
      const f32x4_t hi = *(const f32x4_t*)(R + (int64_t)e * D + k0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[j] = lo[j];
        r[4 + j] = hi[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = 0.f;
    }
    uint32_t h[3][4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      uint32_t p0[3], p1[3];
      float a = r[j], b = r[j + 1];
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const uint16_t ha = to_bf16(a), hb = to_bf16(b);
        p0[pl] = ha;
        p1[pl] = hb;
        a -= bf16lo_to_f32(ha);
        b -= bf16lo_to_f32(hb);
      }
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) h[pl][j >> 1] = p0[pl] | (p1[pl] << 16);
    }
#pragma unroll
    for (int pl = 0; pl < 3; ++pl)
      *(u32x4_t*)(Rs + pl * plane + i * 8) = u32x4_t{h[pl][0], h[pl][1], h[pl][2], h[pl][3]};
  }
}

void launch_router_split(const float* R, uint16_t* Rs, int E, int D, hipStream_t s) {
  const int64_t nfrag = (int64_t)((E + 15) / 16) * (D / 32) * 64;
  int blocks = (int)((nfrag + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(router_split_kernel, dim3(blocks), dim3(256), 0, s, R, Rs, E, D);
}

// ---------------------------------------------------------------------------- logits
// Workgroup tile: 16 NTF tokens x 32 experts.  Its eight wavefronts are two 16-expert
// tiles times four quarters of D; each keeps one accumulator per R plane and token
// fragment (independent MFMA chains), and its loads are unconditional (rows past T or E
// are clamped to valid rows and their results dropped), so that the unrolled loop
// keeps several 32-wide k-steps of loads in flight.  The quarters are added through
// LDS.  NTF = 4 at large T shares each R fragment among four token fragments.
// v_mfma_f32_16x16x32_bf16 layout: lane l supplies row (l % 16) and the eight k-slots
// 8*(l/16)..+7; the accumulator holds rows 4*(l/16)+i, column l % 16.
//
// With `xprep` set, the workgroups of the first expert column also write the copy of x
// that the resident-tile GEMM reads (each run of 8 columns in the order
// 0,4,1,5,2,6,3,7, plus one zero row after the last token): their tile-0 wavefronts
// store each x fragment as they use it.
template <int NTF>
__global__ __launch_bounds__(512) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ Rs,
                                                            float* __restrict__ L, int T, int D,
                                                            int E, uint16_t* __restrict__ xprep) {
  __shared__ f32x4_t red[3][2][NTF][64];
  static_assert(NTF == 1 || NTF == 4, "token fragments");
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int m = l & 15, q = l >> 4;
  const int tile = wave & 1, kq = wave >> 1;
  const int t0 = blockIdx.x * 16 * NTF;
  const int nsteps = D >> 5, ET = (E + 15) >> 4;
  const int et = blockIdx.y * 2 + tile;
  const int e = 16 * et + m;
  const bool ev = e < E;
  const int64_t plane = (int64_t)ET * 16 * D;
  // fragment-major planes: step s of tile et is the kilobyte at (et * nsteps + s) * 512
  const uint16_t* rb = Rs + (int64_t)(et < ET ? et : ET - 1) * nsteps * 512 + 8 * l;
  const uint16_t* xa[NTF];
  bool tv[NTF];
#pragma unroll
  for (int f = 0; f < NTF; ++f) {
    const int t = t0 + 16 * f + m;
    tv[f] = t < T;
    xa[f] = x + (int64_t)(tv[f] ? t : T - 1) * D + 8 * q;
  }
  const int s0 = nsteps * kq / 4, s1 = nsteps * (kq + 1) / 4;
  f32x4_t a0[NTF], a1[NTF], a2[NTF];
#pragma unroll
  for (int f = 0; f < NTF; ++f) {
    a0[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    a1[f] = a0[f];
    a2[f] = a0[f];
  }
  // software pipeline over batches of BS k-steps: the loads of batch b + 1 are issued
  // before the matrix work of batch b; steps past s1 load the last valid step again
  // and skip the matrix work
  constexpr int BS = NTF == 1 ? 4 : 2;
  u32x4_t rv[2][BS][3], xv[2][BS][NTF];
  auto load = [&](int buf, int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < BS; ++i) {
      const int st = min(sb + i, s1 - 1), k0 = 32 * st;
      rv[buf][i][0] = *(const u32x4_t*)(rb + 512 * st);
      rv[buf][i][1] = *(const u32x4_t*)(rb + plane + 512 * st);
      rv[buf][i][2] = *(const u32x4_t*)(rb + 2 * plane + 512 * st);
#pragma unroll
      for (int f = 0; f < NTF; ++f) xv[buf][i][f] = *(const u32x4_t*)(xa[f] + k0);
    }
  };
  // the tile-0 waves of the first expert column store every x fragment they use,
  // permuted, into the GEMM's copy (each fragment is a 16-byte run of 8 columns)
  const bool prep = xprep != nullptr && blockIdx.y == 0 && tile == 0;
  uint16_t* xp[NTF];
#pragma unroll
  for (int f = 0; f < NTF; ++f) xp[f] = prep ? xprep + (int64_t)(t0 + 16 * f + m) * D + 8 * q : xprep;
  auto mma = [&](int buf, int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < BS; ++i)
      if (sb + i < s1) {
#pragma unroll
        for (int f = 0; f < NTF; ++f) {
          a0[f] = mfma16x16x32(xv[buf][i][f], rv[buf][i][0], a0[f]);
          a1[f] = mfma16x16x32(xv[buf][i][f], rv[buf][i][1], a1[f]);
          a2[f] = mfma16x16x32(xv[buf][i][f], rv[buf][i][2], a2[f]);
        }
        if (prep) {
#pragma unroll
          for (int f = 0; f < NTF; ++f)
            if (tv[f]) *(u32x4_t*)(xp[f] + 32 * (sb + i)) = interleave8(xv[buf][i][f]);
        }
      }
  };
  if (s0 < s1) {
    load(0, s0);
    for (int sb = s0; sb < s1; sb += 2 * BS) {
      load(1, sb + BS);
      mma(0, sb);
      load(0, sb + 2 * BS);
      mma(1, sb + BS);
    }
  }
  if (xprep && blockIdx.x == 0 && blockIdx.y == 0 && tile == 1) {
    // the zero row after the last token
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int c = kq * 64 + l; c < (D >> 3); c += 256)
      *(u32x4_t*)(xprep + (int64_t)T * D + 8 * c) = zero;
  }
  f32x4_t acc[NTF];
#pragma unroll
  for (int f = 0; f < NTF; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][i] = a0[f][i] + (a1[f][i] + a2[f][i]);
  if (kq > 0) {
#pragma unroll
    for (int f = 0; f < NTF; ++f) red[kq - 1][tile][f][l] = acc[f];
  }
  __syncthreads();
  if (kq == 0 && ev) {
#pragma unroll
    for (int f = 0; f < NTF; ++f) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const f32x4_t o = red[j][tile][f][l];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[f][i] += o[i];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = t0 + 16 * f + 4 * q + r;
        if (tt < T) L[(int64_t)tt * E + e] = acc[f][r];
      }
    }
  }
}

// Many tokens (T >= 2048, D % 256 == 0): workgroup tile of 64 tokens x 128 experts, its
// eight wavefronts one 16-expert tile each over the whole K, so that R (three planes)
// is read T / 64 times and x E / 128 times.  The tile's x rows go through LDS in chunks
// of 256 k: every thread loads 16-byte pieces of whole 512-byte row runs (line-whole,
// rows read once per workgroup) one chunk ahead, and writes them into the other buffer
// in fragment order.  A piece (fragment f, 32-k step s, quarter q, row m) sits at
// (8 f + s) * 1088 + (17 q + m) * 16 bytes: a wavefront's reads are conflict-free and
// its writes of one row's pieces at most two-way.  Each wavefront's R fragments for a
// step are loaded one chunk (eight steps) ahead.  The workgroups of the first expert
// column also write the prepared copy of x from the pieces they load.
constexpr int kWideTok = 64, kWideExp = 128, kWideKC = 256;
constexpr int kWideBlock = 1088;  // bytes per (fragment, step) block, padded
__global__ __launch_bounds__(512) void router_logits_wide_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Rs, float* __restrict__ L, int T,
    int D, int E, uint16_t* __restrict__ xprep) {
  __shared__ __attribute__((aligned(16))) unsigned char xs[2][4 * 8 * kWideBlock];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int m = l & 15, q = l >> 4;
  const int t0 = blockIdx.x * kWideTok;
  const int nsteps = D >> 5, ET = (E + 15) >> 4, nch = D / kWideKC;
  const int et = blockIdx.y * 8 + wave;
  const int e = 16 * et + m;
  const bool ev = e < E;
  const int64_t plane = (int64_t)ET * 16 * D;
  const uint16_t* rb = Rs + (int64_t)(et < ET ? et : ET - 1) * nsteps * 512 + 8 * l;
  // this thread's x pieces: rows (tid / 32) + 16 i, piece c = tid % 32 of each 512-byte run
  const int pc = tid & 31, pr = tid >> 5;
  const uint16_t* xsrc[4];
  bool tv[4];
  uint32_t xdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + pr + 16 * i;
    tv[i] = t < T;
    xsrc[i] = x + (int64_t)(tv[i] ? t : T - 1) * D + 8 * pc;
    xdst[i] = (uint32_t)((8 * i + (pc >> 2)) * kWideBlock + (17 * (pc & 3) + pr) * 16);
  }
  const bool prep = xprep != nullptr && blockIdx.y == 0;
  auto load_x = [&](u32x4_t* xr, int ch) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = *(const u32x4_t*)(xsrc[i] + ch * kWideKC);
  };
  auto store_x = [&](const u32x4_t* xr, int ch, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4_t*)(&xs[buf][xdst[i]]) = xr[i];
    if (prep) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tv[i])
          *(u32x4_t*)(xprep + (int64_t)(t0 + pr + 16 * i) * D + ch * kWideKC + 8 * pc) =
              interleave8(xr[i]);
    }
  };
  auto load_r = [&](u32x4_t* rv, int gs) __attribute__((always_inline)) {
    rv[0] = *(const u32x4_t*)(rb + 512 * gs);
    rv[1] = *(const u32x4_t*)(rb + plane + 512 * gs);
    rv[2] = *(const u32x4_t*)(rb + 2 * plane + 512 * gs);
  };
  f32x4_t a0[4], a1[4], a2[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    a0[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    a1[f] = a0[f];
    a2[f] = a0[f];
  }
  u32x4_t rv[8][3], xr[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) load_r(rv[s], s);
  load_x(xr, 0);
  store_x(xr, 0, 0);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    const int chn = ch + 1 < nch ? ch + 1 : ch;  // the last chunk loads itself again
    load_x(xr, chn);
    __builtin_amdgcn_sched_barrier(0);  // issued a chunk ahead of their store, not sunk to it
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4_t xa[4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
        xa[f] = *(const u32x4_t*)(&xs[buf][(8 * f + s) * kWideBlock + (17 * q + m) * 16]);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        a0[f] = mfma16x16x32(xa[f], rv[s][0], a0[f]);
        a1[f] = mfma16x16x32(xa[f], rv[s][1], a1[f]);
        a2[f] = mfma16x16x32(xa[f], rv[s][2], a2[f]);
      }
      // the step's fragments reloaded here, a whole chunk before their next use (left to
      // itself the scheduler sinks all of a chunk's reloads to its end)
      load_r(rv[s], 8 * chn + s);
      __builtin_amdgcn_sched_barrier(0);
    }
    // unconditional (after the last chunk it stores that chunk again into the unused
    // buffer), so that the compiler does not sink the loads of xr into a branch here
    store_x(xr, chn, buf ^ 1);
    __syncthreads();
  }
  if (xprep && blockIdx.x == 0 && blockIdx.y == 0 && wave == 0) {
    // the zero row after the last token
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int c = l; c < (D >> 3); c += 64) *(u32x4_t*)(xprep + (int64_t)T * D + 8 * c) = zero;
  }
  if (ev) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = t0 + 16 * f + 4 * q + r;
        if (tt < T) L[(int64_t)tt * E + e] = a0[f][r] + (a1[f][r] + a2[f][r]);
      }
  }
}

// Fewer tokens (D % 256 == 0): R itself, fp32, split in registers into three bf16 pieces
// that sum to it exactly, on the bf16 matrix cores (x is bf16 already, so every product
// is exact; an earlier form on the fp32 matrix cores, v_mfma_f32_16x16x4_f32, took 11.7
// against 10.3 us at 512 tokens).  Workgroup tile: 16 tokens x 32 experts; its sixteen
// wavefronts (four per SIMD, to hide the LDS and load latencies) are two 16-expert tiles
// times eight 32-K parts of each 256-K chunk, with two accumulators each, added through
// LDS at the end in a fixed order.  The chunk's R rows (1 KB each) and x rows go through
// padded LDS rows with line-whole loads, one chunk ahead in VGPRs.  A wavefront's 32 k
// of a chunk are one 16x16x32 step: lane (m, q) reads x of token m and R of expert m at
// k = 8 q .. 8 q + 7.  The workgroups of the first expert column also write the
// prepared copy of x from the x pieces they load.
constexpr int kF32KC = 256;
constexpr int kF32RRow = kF32KC * 4 + 16;  // padded LDS row of R, bytes
constexpr int kF32XRow = kF32KC * 2 + 16;  // padded LDS row of x, bytes
constexpr int kF32Threads = 1024;
__global__ __launch_bounds__(kF32Threads) void router_logits_f32_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ R, float* __restrict__ L, int T, int D,
    int E, uint16_t* __restrict__ xprep) {
  __shared__ __attribute__((aligned(16))) unsigned char rs[2][32 * kF32RRow];
  __shared__ __attribute__((aligned(16))) unsigned char xsh[2][16 * kF32XRow];
  __shared__ f32x4_t red[7][2][64];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int m = l & 15, q = l >> 4;
  const int tile = wave & 1, kq = wave >> 1;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 32;
  const int nch = D / kF32KC;
  // this thread's pieces: R rows (tid / 64) + 16 i, 16-byte piece tid % 64; x row tid / 32
  // (threads below 512), 16-byte piece tid % 32
  const float* rsrc[2];
  uint32_t rdst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (tid >> 6) + 16 * i;
    rsrc[i] = R + (int64_t)min(e0 + row, E - 1) * D + 4 * (tid & 63);
    rdst[i] = (uint32_t)(row * kF32RRow + 16 * (tid & 63));
  }
  const int xr = (tid >> 5) & 15, xc = tid & 31;
  const bool xl = tid < 512;  // loads and stores an x piece
  const bool xv = xl && t0 + xr < T;
  const uint16_t* xsrc = x + (int64_t)min(t0 + xr, T - 1) * D + 8 * xc;
  const uint32_t xdst = (uint32_t)(xr * kF32XRow + 16 * xc);
  const bool prep = xprep != nullptr && blockIdx.y == 0;
  // two register sets: chunk ch + 2 is loaded while ch is computed and ch + 1 is stored
  struct Piece {
    u32x4_t r[2], x;
  };
  auto load = [&](Piece& pc, int ch) __attribute__((always_inline)) {
    ch = min(ch, nch - 1);  // past the end: the last chunk again (never stored)
#pragma unroll
    for (int i = 0; i < 2; ++i) pc.r[i] = *(const u32x4_t*)(rsrc[i] + ch * kF32KC);
    if (xl) pc.x = *(const u32x4_t*)(xsrc + ch * kF32KC);
  };
  auto store = [&](const Piece& pc, int ch, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *(u32x4_t*)(&rs[buf][rdst[i]]) = pc.r[i];
    if (xl) *(u32x4_t*)(&xsh[buf][xdst]) = pc.x;
    if (prep && xv) *(u32x4_t*)(xprep + (int64_t)(t0 + xr) * D + ch * kF32KC + 8 * xc) = interleave8(pc.x);
  };
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  // The wavefront's 32 k of the chunk as one bf16 step (v_mfma_f32_16x16x32_bf16: lane
  // (m, q) gives x of token m and R of expert m at k = 8 q .. 8 q + 7): R split into
  // three bf16 pieces by truncation (hi, mid, lo: each the top eight significant bits of
  // what the previous ones left, so they sum to R exactly) and every product x R_piece
  // exact, accumulated in fp32.
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* rb = &rs[buf][(16 * tile + m) * kF32RRow + kq * 128 + 32 * q];
    const u32x4_t xa = *(const u32x4_t*)&xsh[buf][m * kF32XRow + kq * 64 + 16 * q];
    const f32x4_t r0 = *(const f32x4_t*)rb, r1 = *(const f32x4_t*)(rb + 16);
    const float r[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    uint32_t ph[8], pm[8], pl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ph[i] = __float_as_uint(r[i]) & 0xFFFF0000u;
      const float e1 = r[i] - __uint_as_float(ph[i]);
      pm[i] = __float_as_uint(e1) & 0xFFFF0000u;
      pl[i] = __float_as_uint(e1 - __uint_as_float(pm[i])) & 0xFFFF0000u;
    }
    u32x4_t bh, bm, bl;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      bh[w] = (ph[2 * w] >> 16) | ph[2 * w + 1];
      bm[w] = (pm[2 * w] >> 16) | pm[2 * w + 1];
      bl[w] = (pl[2 * w] >> 16) | pl[2 * w + 1];
    }
    acc0 = mfma16x16x32(xa, bh, acc0);
    acc1 = mfma16x16x32(xa, bm, acc1);
    acc0 = mfma16x16x32(xa, bl, acc0);
  };
  // chunk ch in buffer ch & 1; the other buffer was last read in the previous chunk,
  // before the last barrier
  auto step = [&](int ch, Piece& next, Piece& fresh) __attribute__((always_inline)) {
    load(fresh, ch + 2);
    compute(ch & 1);
    if (ch + 1 < nch) {
      store(next, ch + 1, (ch & 1) ^ 1);
      __syncthreads();
    }
  };
  Piece p0, p1;
  load(p0, 0);
  load(p1, 1);
  store(p0, 0, 0);
  __syncthreads();
  int ch = 0;
  for (; ch + 2 <= nch; ch += 2) {
    step(ch, p1, p0);
    step(ch + 1, p0, p1);
  }
  if (ch < nch) step(ch, p1, p0);
  if (xprep && blockIdx.x == 0 && blockIdx.y == 0 && wave == 0) {
    // the zero row after the last token
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int c = l; c < (D >> 3); c += 64) *(u32x4_t*)(xprep + (int64_t)T * D + 8 * c) = zero;
  }
  f32x4_t acc;
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = acc0[i] + acc1[i];
  if (kq > 0) red[kq - 1][tile][l] = acc;
  __syncthreads();
  const int e = e0 + 16 * tile + m;
  if (kq == 0 && e < E) {
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const f32x4_t o = red[j][tile][l];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += o[i];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = t0 + 4 * q + r;
      if (tt < T) L[(int64_t)tt * E + e] = acc[r];
    }
  }
}

constexpr int kSmallTok = 16;  // the one-wavefront-per-expert kernel serves T <= 16

bool router_small_ok(int T, int D) { return T <= kSmallTok && D % 256 == 0; }

bool router_uses_planes(int T, int D) {
  return !router_small_ok(T, D) && !(T < 2048 && D % kF32KC == 0);
}

void launch_router(const uint16_t* x, const float* R, uint16_t* Rs, float* L, int T, int D, int E,
                   uint16_t* xprep, hipStream_t s, bool planes_ready) {
  if (router_small_ok(T, D)) {
    launch_router_small(x, R, L, T, D, E, xprep, nullptr, 0, s);
    return;
  }
  if (T < 2048 && D % kF32KC == 0) {
    dim3 grid((T + 15) / 16, (E + 31) / 32);
    hipLaunchKernelGGL(router_logits_f32_kernel, grid, dim3(kF32Threads), 0, s, x, R, L, T, D, E,
                       xprep);
    return;
  }
  if (!planes_ready) launch_router_split(R, Rs, E, D, s);
  launch_router_logits(x, Rs, L, T, D, E, xprep, s);
}

void launch_router_logits(const uint16_t* x, const uint16_t* Rs, float* L, int T, int D, int E,
                          uint16_t* xprep, hipStream_t s) {
  dim3 block(512);
  if (T >= 2048 && D % kWideKC == 0) {
    dim3 grid((T + kWideTok - 1) / kWideTok, (E + kWideExp - 1) / kWideExp);
    hipLaunchKernelGGL(router_logits_wide_kernel, grid, block, 0, s, x, Rs, L, T, D, E, xprep);
  } else if (T >= 2048) {
    dim3 grid((T + 63) / 64, (E + 31) / 32);
    hipLaunchKernelGGL(router_logits_kernel<4>, grid, block, 0, s, x, Rs, L, T, D, E, xprep);
  } else {
    dim3 grid((T + 15) / 16, (E + 31) / 32);
    hipLaunchKernelGGL(router_logits_kernel<1>, grid, block, 0, s, x, Rs, L, T, D, E, xprep);
  }
}

// ---------------------------------------------------------------------------- top-k
// One wavefront per token; E <= 64 * MAXC.  The workgroups also clear n_zero words at
// `zero` (a later launch's counters).
template <int MAXC>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ L,
                                                   const uint16_t* __restrict__ x,
                                                   const float* __restrict__ R, int T, int D,
                                                   int E, int k, float tau,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ w_out,
                                                   int32_t* __restrict__ zero, int n_zero) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_zero; i += gridDim.x * 256) zero[i] = 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // no barriers below
  int e;
  float w;
  topk_token<MAXC, 8, 2>(L + (int64_t)t * E, x + (int64_t)t * D, R, D, E, k, tau, e, w);
  if (lane < k) {
    idx_out[(int64_t)t * k + lane] = e;
    w_out[(int64_t)t * k + lane] = w;
  }
}

void launch_topk(const float* L, const uint16_t* x, const float* R, int T, int D, int E, int k,
                 float tau, int32_t* idx, float* w, int32_t* zero, int n_zero, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  if (!zero) n_zero = 0;
  if (E <= 64)
    hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, L, x, R, T, D, E, k, tau, idx, w, zero, n_zero);
  else if (E <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, L, x, R, T, D, E, k, tau, idx, w, zero, n_zero);
  else
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, L, x, R, T, D, E, k, tau, idx, w, zero,
                       n_zero);
}

// ---------------------------------------------------------------------------- few tokens
// T <= 16 (decode): one wavefront per expert, four per workgroup, so that R (E * D * 4
// bytes, the bulk of the router's traffic) streams through every compute unit instead of
// the few workgroups a 16-token tile would give.  Lane l takes k = 256 s + 4 l .. + 3 of
// each 256-K step s: one 16-byte load of R and one 8-byte load of each token's x (TT
// tokens, T rounded up; rows past T re-read the last row and are dropped), all of a step
// issued before any is used (and a few steps at a time); the lane sums in fp32 in k order, then the wavefront sums in
// a fixed DPP order.  The workgroups also write the prepared copy of x (runs of 8 columns
// in the order 0,4,1,5,2,6,3,7, one zero row after the last token), and clear n_zero words
// at `zero` (the next kernel's counters and flags).
template <int TT>
__global__ __launch_bounds__(256) void router_logits_small_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ R, float* __restrict__ L, int T, int D,
    int E, uint16_t* __restrict__ xprep, int32_t* __restrict__ zero, int n_zero) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_zero; i += gridDim.x * 256) zero[i] = 0;
  if (xprep) {
    const int pieces = (T + 1) * (D >> 3);
    for (int pc = blockIdx.x * 256 + threadIdx.x; pc < pieces; pc += gridDim.x * 256) {
      const int row = pc / (D >> 3), c8 = pc - row * (D >> 3);
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < T) v = interleave8(*(const u32x4_t*)(x + (int64_t)row * D + 8 * c8));
      *(u32x4_t*)(xprep + (int64_t)row * D + 8 * c8) = v;
    }
  }
  if (e >= E) return;  // uniform per wavefront; no barriers
  const float* r = R + (int64_t)e * D + 4 * lane;
  const uint16_t* xr[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) xr[t] = x + (int64_t)min(t, T - 1) * D + 4 * lane;
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;
  constexpr int UN = TT <= 4 ? 8 : 2;  // steps whose loads are in flight together (d_model 2048 in one round)
  for (int k0 = 0; k0 < D; k0 += 256 * UN) {
    f32x4_t rv[UN];
    u32x2_t xw[UN][TT];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int kk = min(k0 + 256 * u, D - 256);  // past the end: a valid step, not summed
      rv[u] = *(const f32x4_t*)(r + kk);
#pragma unroll
      for (int t = 0; t < TT; ++t) xw[u][t] = *(const u32x2_t*)(xr[t] + kk);
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      if (k0 + 256 * u < D) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          acc[t] = fmaf(bf16lo_to_f32(xw[u][t][0]), rv[u][0], acc[t]);
          acc[t] = fmaf(bf16hi_to_f32(xw[u][t][0]), rv[u][1], acc[t]);
          acc[t] = fmaf(bf16lo_to_f32(xw[u][t][1]), rv[u][2], acc[t]);
          acc[t] = fmaf(bf16hi_to_f32(xw[u][t][1]), rv[u][3], acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (t < T) {
      const float v = wave_sum_f32(acc[t]);
      if (lane == 0) L[(int64_t)t * E + e] = v;
    }
  }
}

void launch_router_small(const uint16_t* x, const float* R, float* L, int T, int D, int E,
                         uint16_t* xprep, int32_t* zero, int n_zero, hipStream_t s) {
  const dim3 grid((E + 3) / 4), block(256);
  if (T <= 1)
    hipLaunchKernelGGL(router_logits_small_kernel<1>, grid, block, 0, s, x, R, L, T, D, E, xprep,
                       zero, n_zero);
  else if (T <= 4)
    hipLaunchKernelGGL(router_logits_small_kernel<4>, grid, block, 0, s, x, R, L, T, D, E, xprep,
                       zero, n_zero);
  else
    hipLaunchKernelGGL(router_logits_small_kernel<16>, grid, block, 0, s, x, R, L, T, D, E, xprep,
                       zero, n_zero);
}

}  // namespace moeq4
