// The MoE layer at decode sizes (T <= 16 tokens): a launch chain whose kernels spread the
// few touched experts' weights over every compute unit, with no permutation of token rows
// and no expert-output array in memory.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference engine for
// Qwen3.6-35B-A3B on Apple Silicon", body paragraph 7 (batch-1 decode reuses almost no
// weight, so memory bandwidth is the ceiling, and the engine cuts the number of sequential
// kernel stages) and paragraph 4 (eight of 256 experts per token plus a shared expert).
//
// Chain (after the router logits, computed by the one-wavefront-per-expert router kernel,
// which also writes the prepared copy of x with a zero row after the last token):
//   plan          one workgroup: the top k of every token (exact, the router's own
//                 selection code), the sorted list of distinct touched experts ("slots",
//                 the shared expert last), each slot's combine weight for each token, and
//                 the layer's routing outputs (top-k, group offsets, permuted rows);
//   gate_up       one workgroup per (slot, 16 weight rows of gate and the matching 16 of
//                 up): the 16-row fragment of all tokens (rows past T are the zero row)
//                 against those rows, K split over four wavefronts, SwiGLU, activations
//                 stored per slot;
//   down+combine  one workgroup per 16 output columns: every (slot, 64-wide group) unit
//                 of the down product for those columns, scaled by the slot's combine
//                 weight per token and summed in fp32 in a fixed order, so the expert
//                 outputs never leave registers.
//
// Arithmetic per 64-wide group g of one weight row (scale s, bias b): the matrix cores give
// P' = sum x (128 + q) with exact products (128 + q is the bf16 0x4300 | q) and the row sums
// X = sum x (activations times a fragment of ones); then acc += s P' + (b - 128 s) X in
// fp32.  The K order inside a group is a permutation shared by both operands: in MFMA step
// h of group g, quarter q of the lanes takes packed word 8 g + 2 q + h of its weight row
// and the matching eight activations, so each step stays inside one scale group and a lane
// loads its two words of a group with one 8-byte load.
#include "common.h"
#include "internal.h"
#include "q4_stream.h"
#include "topk_select.h"

namespace moeq4 {

namespace {

// the ws pieces of the plan
struct PlanPtrs {
  int32_t* n_slots;      // [1]
  int32_t* slot_expert;  // [max_slots]: expert id, -1 = the shared expert
  float* coef;           // [max_slots][16]: combine weight of the slot for token t
};

__host__ __device__ inline PlanPtrs plan_ptrs(void* plan) {
  PlanPtrs p;
  p.n_slots = (int32_t*)plan;
  p.slot_expert = p.n_slots + 4;
  p.coef = (float*)(p.slot_expert + ((kDecodeMaxSlots + 3) / 4) * 4);
  return p;
}

// ------------------------------------------------------------------------------- plan
template <int MAXC>
__global__ __launch_bounds__(1024) void decode_plan_kernel(
    const float* __restrict__ L, const uint16_t* __restrict__ x, const float* __restrict__ R, int T,
    int D, int E, int k, float tau, int has_shared, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_tok,
    int32_t* __restrict__ slot_row, PlanPtrs plan) {
  __shared__ int sel_e[kDecodeMaxT * kMaxTopK];
  __shared__ float sel_w[kDecodeMaxT * kMaxTopK];
  __shared__ uint32_t bits[32];      // touched experts, E <= 1024
  __shared__ int word_base[33];
  __shared__ int cnt[1024];
  __shared__ int scan_tmp[1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < 32) bits[tid] = 0u;
  cnt[tid] = 0;
  __syncthreads();
  if (wave < T) {
    int e;
    float w;
    topk_token<MAXC>(L + (int64_t)wave * E, x + (int64_t)wave * D, R, D, E, k, tau, e, w);
    if (lane < k) {
      sel_e[wave * k + lane] = e;
      sel_w[wave * k + lane] = w;
      idx_out[wave * k + lane] = e;
      w_out[wave * k + lane] = w;
      atomicOr(&bits[e >> 5], 1u << (e & 31));
      atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  // distinct experts in ascending order: slot of e = set bits below it
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < 32; ++i) {
      word_base[i] = acc;
      acc += __popc(bits[i]);
    }
    word_base[32] = acc;
    const int n = acc + (has_shared ? 1 : 0);
    *plan.n_slots = n;
    if (has_shared) plan.slot_expert[acc] = -1;
  }
  // exclusive scan of the per-expert counts (group offsets, as the grouped path's)
  {
    int v = tid < E ? cnt[tid] : 0;
    scan_tmp[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = tid >= off ? scan_tmp[tid - off] : 0;
      __syncthreads();
      scan_tmp[tid] += add;
      __syncthreads();
    }
    // scan_tmp[tid] is inclusive
    if (tid < E) offsets[tid] = scan_tmp[tid] - v;
    if (tid == 0) {
      offsets[E] = T * k;
      if (has_shared) offsets[E + 1] = T * k + T;
    }
  }
  __syncthreads();
  const int n_distinct = word_base[32];
  const int n_slots = n_distinct + (has_shared ? 1 : 0);
  // slot list and the combine weights (zero, then one entry per (token, slot) pair)
  for (int e = tid; e < E; e += 1024)
    if ((bits[e >> 5] >> (e & 31)) & 1u)
      plan.slot_expert[word_base[e >> 5] + __popc(bits[e >> 5] & ((1u << (e & 31)) - 1u))] = e;
  for (int i = tid; i < n_slots * 16; i += 1024) {
    const int s = i >> 4, t = i & 15;
    plan.coef[i] = (has_shared && s == n_distinct && t < T) ? 1.f : 0.f;
  }
  __syncthreads();
  if (tid < T * k) {
    const int t = tid / k;
    const int e = sel_e[tid];
    const int slot = word_base[e >> 5] + __popc(bits[e >> 5] & ((1u << (e & 31)) - 1u));
    plan.coef[slot * 16 + t] = sel_w[tid];
    // stable permuted row: the tokens before t that also picked e
    int rank = 0;
    for (int u = 0; u < t * k; ++u) rank += sel_e[u] == e ? 1 : 0;
    const int row = scan_tmp[e] - cnt[e] + rank;
    sorted_tok[row] = t;
    slot_row[tid] = row;
  }
  if (has_shared && tid < T) sorted_tok[T * k + tid] = tid;
}

// ------------------------------------------------------------------------------- staging
// Weights reach LDS through direct global->LDS loads of 16 bytes per lane: the 64 lanes of
// one instruction fill 1 KB of LDS, in lane order, from chunks that are contiguous in
// memory except where a region changes rows or experts.  Code rows are stored with their
// 16-byte chunks permuted: LDS chunk cs of staged row r holds the row's chunk
// cs ^ (r & mask) (mask: the largest power of two dividing the row's chunk count, at most
// 16, minus one).  The XOR stays inside an aligned block of chunks, so an instruction still
// covers whole lines, and the MFMA-layout reads of sixteen rows fall in distinct chunks.
__device__ __forceinline__ int chunk_mask(int cpr) {
  const int low = cpr & -cpr;
  return (low < 16 ? low : 16) - 1;
}

// nch chunks into LDS dst (chunk c at dst + 16 c), chunk c read from src(c); the
// instructions are dealt to nw wavefronts from `wave`.  Lanes past nch read chunk nch - 1
// again and write up to 1008 bytes past the region, which every region leaves as slack.
template <typename Src>
__device__ __forceinline__ void stage(unsigned char* dst, int nch, Src src, int wave, int nw,
                                      int lane) {
  const int n_ins = (nch + 63) >> 6;
  for (int k = wave; k < n_ins; k += nw) {
    int c = 64 * k + lane;
    if (c >= nch) c = nch - 1;
    __builtin_amdgcn_global_load_lds(src(c), dst + 1024 * k, 16, 0, 0);
  }
}

// the 8 bytes of words (w, w + 1) (w even) of staged code row r (cpr chunks per row)
__device__ __forceinline__ u32x2_t lds_words(const unsigned char* rows, int r, int cpr, int w) {
  const int c = w >> 2;
  return *(const u32x2_t*)(rows + (r * cpr + (c ^ (r & chunk_mask(cpr)))) * 16 + (w & 3) * 4);
}

// ------------------------------------------------------------------------------- gate_up
// One workgroup of eight wavefronts per (slot, slice of 16 gate rows and the 16 matching up
// rows).  The slice's codes (32 rows) and its scale and bias rows go to LDS first; while
// they land, wavefront w loads its activations for the 256-K stages w, w + 8, ... from the
// prepared x (rows past T read the zero row).  The eight partial sums meet through LDS (over
// the code area, once every wavefront is done with it) in a fixed order; wavefront 0 applies
// SwiGLU and stores the activations in the down kernel's fragment order:
// act[slot][group][step][lane 16 q + row][8] = the eight values of prepared word
// 8 group + 2 q + step of the row.
constexpr int kUpWaves = 8;
constexpr int kUpMaxD = 2048;
constexpr int kUpCodeBytes = 32 * kUpMaxD / 2 + 1024;     // 32 rows of codes + slack
constexpr int kUpSbBytes = 4 * 32 * (kUpMaxD / 64) + 1024;  // gate s, up s, gate b, up b
static_assert(kUpCodeBytes >= (int)sizeof(f32x4_t) * kUpWaves * 2 * 64, "reduction area");
__global__ __launch_bounds__(64 * kUpWaves) void decode_gate_up_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char codes[kUpCodeBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sb[kUpSbBytes];
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int F = p.F, D = p.D, NSL = F / 16;
  const int s = blockIdx.x / NSL, sl = blockIdx.x - s * NSL;
  const PlanPtrs plan = plan_ptrs(p.plan);
  const int n_slots = __builtin_amdgcn_readfirstlane(*plan.n_slots);
  if (s >= n_slots) return;  // uniform, before any barrier
  const int e = __builtin_amdgcn_readfirstlane(plan.slot_expert[s]);
  const Q4Ptrs& W = e >= 0 ? p.up_main : p.up_last;
  const int KW = D >> 3, KG = D >> 6, CPR = D >> 5;
  const int64_t base_row = (int64_t)(e >= 0 ? e : 0) * (2 * F);
  const int64_t gate0 = base_row + 16 * sl, up0 = base_row + F + 16 * sl;
  const int mask = chunk_mask(CPR);
  // staged rows 0..15: gate rows gate0 + r; 16..31: up rows up0 + r - 16
  stage(codes, 32 * CPR, [&](int c) {
    const int r = c / CPR, cs = c - r * CPR;
    const int64_t row = (r < 16 ? gate0 : up0 - 16) + r;
    return (const unsigned char*)(W.q + row * KW) + 16 * (cs ^ (r & mask));
  }, wave, kUpWaves, l);
  // four regions of 16 rows x KG bf16 (2 KG chunks each): gate s, up s, gate b, up b
  const int rch = 2 * KG;
  stage(sb, 4 * rch, [&](int c) {
    const int rg = c / rch, w = c - rg * rch;
    const uint16_t* base = (rg < 2 ? W.s : W.b) + ((rg & 1) ? up0 : gate0) * KG;
    return (const unsigned char*)base + 16 * w;
  }, (wave + 4) % kUpWaves, kUpWaves, l);
  // this wavefront's activations
  const uint16_t* xr = p.xprep + (int64_t)(m < p.T ? m : p.T) * D + 16 * q;  // row T is zero
  const int NST = D >> 8;
  constexpr int kMaxSt = kUpMaxD / 256 / kUpWaves;
  u32x4_t a[kMaxSt][4][2];
#pragma unroll
  for (int v = 0; v < kMaxSt; ++v) {
    const int st = wave + kUpWaves * v;
    if (st < NST) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) a[v][g][h] = *(const u32x4_t*)(xr + 256 * st + 64 * g + 8 * h);
    }
  }
  wait_vmcnt0();
  __syncthreads();
  const uint32_t magic = opaque_magic();
  const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc[2] = {zero, zero};
#pragma unroll
  for (int v = 0; v < kMaxSt; ++v) {
    const int st = wave + kUpWaves * v;
    if (st < NST) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t X = mfma16x16x32(a[v][g][1], ones, mfma16x16x32(a[v][g][0], ones, zero));
        const int so = (m * KG + 4 * st + g) * 2;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x2_t wd = lds_words(codes, 16 * j + m, CPR, 32 * st + 8 * g + 2 * q);
          const f32x4_t P = mfma16x16x32(a[v][g][1], unpack_word(wd[1], magic),
                                         mfma16x16x32(a[v][g][0], unpack_word(wd[0], magic), zero));
          const float sg = bf16lo_to_f32(*(const uint16_t*)(sb + j * 32 * KG + so));
          const float bg = bf16lo_to_f32(*(const uint16_t*)(sb + (2 + j) * 32 * KG + so));
          const float cg = fmaf(-128.f, sg, bg);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(sg, P[i], fmaf(cg, X[i], acc[j][i]));
        }
      }
    }
  }
  __syncthreads();  // every wavefront is past its code reads
  f32x4_t* part = (f32x4_t*)codes;  // [wave][2][64]
  part[(wave * 2 + 0) * 64 + l] = acc[0];
  part[(wave * 2 + 1) * 64 + l] = acc[1];
  __syncthreads();
  if (wave == 0) {
    f32x4_t g4 = part[l], u4 = part[64 + l];
#pragma unroll
    for (int w = 1; w < kUpWaves; ++w) {
      const f32x4_t gp = part[(2 * w) * 64 + l], up = part[(2 * w + 1) * 64 + l];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g4[i] += gp[i];
        u4[i] += up[i];
      }
    }
    // natural column c = 16 sl + m: prepared word w = c / 8, position perm8(c % 8); word w
    // is group w / 8, quarter (w % 8) / 2, step (w % 8) & 1 of the down kernel's fragments
    const int c = 16 * sl + m, w = c >> 3, pos = perm8(c & 7);
    const int g2 = w >> 3, qq = (w & 7) >> 1, hh = w & 1;
    uint16_t* dst = p.act + ((((int64_t)s * (F >> 6) + g2) * 2 + hh) * 64 + 16 * qq) * 8 + pos;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gte = g4[i];
      dst[(4 * q + i) * 8] = to_bf16(gte / (1.f + __expf(-gte)) * u4[i]);
    }
  }
}

// ------------------------------------------------------------------------------- down
// One workgroup of eight wavefronts per 16 output columns.  The slots' experts and combine
// weights go to LDS first; then, batch by batch of up to 12288 / F slots, the batch's
// 16-row code slices and scale and bias rows go to LDS, and the (slot, 256-K part) units
// are dealt to the wavefronts in turn: each unit loads its activation fragments (1 KB
// contiguous each) and adds coef[slot][t] (s P' + (b - 128 s) X) over its four groups to
// the wavefront's sums for its 16 columns and 16 token rows.  The eight partial sums meet
// through LDS in a fixed order, then one bf16 row piece per token goes out.
constexpr int kDownWaves = 8;
constexpr int kDownMaxF = 1024;
constexpr int kDownCodeArea = 96 * 1024;              // code slices of one batch
constexpr int kDownSbArea = kDownCodeArea / 8;        // their scales and biases
constexpr int kDownUnits = 4;                         // units' loads in flight per wavefront
__global__ __launch_bounds__(64 * kDownWaves) void decode_down_combine_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char codes[kDownCodeArea + 1024];
  __shared__ __attribute__((aligned(16))) unsigned char sbl[kDownSbArea + 1024];
  __shared__ float red[kDownWaves][16][17];
  __shared__ float scoef[kDecodeMaxSlots * 16];
  __shared__ int sexp[kDecodeMaxSlots];
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int F = p.F, D = p.D, n0 = 16 * blockIdx.x;
  const int KW = F >> 3, KG = F >> 6, CPR = F >> 5;
  const PlanPtrs plan = plan_ptrs(p.plan);
  const int n_slots = __builtin_amdgcn_readfirstlane(*plan.n_slots);
  for (int i = tid; i < n_slots * 16; i += 64 * kDownWaves) scoef[i] = plan.coef[i];
  for (int i = tid; i < n_slots; i += 64 * kDownWaves) sexp[i] = plan.slot_expert[i];
  __syncthreads();
  const int NP = (KG + 3) >> 2;  // 256-K parts
  const int per_batch = kDownCodeArea / (8 * F);  // 16 rows x F / 2 bytes per slot
  const int mask = chunk_mask(CPR);
  const uint32_t magic = opaque_magic();
  const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t out = zero;
  for (int s0 = 0; s0 < n_slots; s0 += per_batch) {
    const int nb = n_slots - s0 < per_batch ? n_slots - s0 : per_batch;
    if (s0 > 0) __syncthreads();  // the previous batch's LDS reads are done
    // codes: staged row r = 16 b + i is row n0 + i of slot s0 + b's expert
    stage(codes, nb * 16 * CPR, [&](int c) {
      const int r = c / CPR, cs = c - r * CPR, b = r >> 4;
      const int e = sexp[s0 + b];
      const Q4Ptrs& W = e >= 0 ? p.down_main : p.down_last;
      const int64_t row = (int64_t)(e >= 0 ? e : 0) * D + n0 + (r & 15);
      return (const unsigned char*)(W.q + row * KW) + 16 * (cs ^ (r & mask));
    }, wave, kDownWaves, l);
    // scales then biases of each slot's 16 rows (16 KG bf16, 2 KG chunks each)
    const int rch = 2 * KG;
    stage(sbl, nb * 2 * rch, [&](int c) {
      const int rg = c / rch, w = c - rg * rch, b = rg >> 1;
      const int e = sexp[s0 + b];
      const Q4Ptrs& W = e >= 0 ? p.down_main : p.down_last;
      const int64_t row = (int64_t)(e >= 0 ? e : 0) * D + n0;
      return (const unsigned char*)(((rg & 1) ? W.b : W.s) + row * KG) + 16 * w;
    }, (wave + 4) % kDownWaves, kDownWaves, l);
    wait_vmcnt0();
    __syncthreads();
    const int units = nb * NP;
    for (int u0 = wave; u0 < units; u0 += kDownWaves * kDownUnits) {
      u32x4_t a[kDownUnits][4][2];
#pragma unroll
      for (int k = 0; k < kDownUnits; ++k) {
        const int u = min(u0 + kDownWaves * k, units - 1);  // past the end: valid, not added
        const int b = u / NP, pt = u - b * NP;
        const uint16_t* af = p.act + (int64_t)(s0 + b) * KG * 2 * 512 + 8 * l;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int g = min(4 * pt + g4, KG - 1);  // past K: a valid group, not added
#pragma unroll
          for (int h = 0; h < 2; ++h) a[k][g4][h] = *(const u32x4_t*)(af + (2 * g + h) * 512);
        }
      }
#pragma unroll
      for (int k = 0; k < kDownUnits; ++k) {
        const int u = u0 + kDownWaves * k;
        if (u < units) {
          const int b = u / NP, pt = u - b * NP;
          f32x4_t y = zero;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int g = 4 * pt + g4;
            if (g < KG) {
              const u32x2_t wd = lds_words(codes, 16 * b + m, CPR, 8 * g + 2 * q);
              const f32x4_t X = mfma16x16x32(a[k][g4][1], ones, mfma16x16x32(a[k][g4][0], ones, zero));
              const f32x4_t P = mfma16x16x32(a[k][g4][1], unpack_word(wd[1], magic),
                                             mfma16x16x32(a[k][g4][0], unpack_word(wd[0], magic), zero));
              const int so = ((2 * b) * 16 * KG + m * KG + g) * 2;
              const float sg = bf16lo_to_f32(*(const uint16_t*)(sbl + so));
              const float bg = bf16lo_to_f32(*(const uint16_t*)(sbl + so + 32 * KG));
              const float cg = fmaf(-128.f, sg, bg);
#pragma unroll
              for (int i = 0; i < 4; ++i) y[i] = fmaf(sg, P[i], fmaf(cg, X[i], y[i]));
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = fmaf(scoef[(s0 + b) * 16 + 4 * q + i], y[i], out[i]);
        }
      }
    }
  }
  // out holds rows 4 q + i, column m
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * q + i][m] = out[i];
  __syncthreads();
  if (tid < 256) {
    const int t = tid >> 4, c = tid & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) v += red[w][t][c];
    if (t < p.T) p.out[(int64_t)t * D + n0 + c] = to_bf16(v);
  }
}

}  // namespace

bool decode_supported(int T, int D, int E, int k, int F) {
  return T >= 1 && T <= kDecodeMaxT && T * k <= kDecodeMaxPairs && E <= 1024 && D % 256 == 0 &&
         D <= kUpMaxD && F % 64 == 0 && F <= kDownMaxF;
}

size_t decode_plan_bytes() {
  return 16 + ((kDecodeMaxSlots + 3) / 4) * 16 + (size_t)kDecodeMaxSlots * 16 * 4;
}

void launch_decode_plan(const float* L, const uint16_t* x, const float* R, int T, int D, int E,
                        int k, float tau, bool has_shared, int32_t* idx, float* w,
                        int32_t* offsets, int32_t* sorted_tok, int32_t* slot_row, void* plan,
                        hipStream_t s) {
  const PlanPtrs pp = plan_ptrs(plan);
  const dim3 grid(1), block(1024);
  if (E <= 64)
    hipLaunchKernelGGL(decode_plan_kernel<1>, grid, block, 0, s, L, x, R, T, D, E, k, tau,
                       has_shared ? 1 : 0, idx, w, offsets, sorted_tok, slot_row, pp);
  else if (E <= 256)
    hipLaunchKernelGGL(decode_plan_kernel<4>, grid, block, 0, s, L, x, R, T, D, E, k, tau,
                       has_shared ? 1 : 0, idx, w, offsets, sorted_tok, slot_row, pp);
  else
    hipLaunchKernelGGL(decode_plan_kernel<16>, grid, block, 0, s, L, x, R, T, D, E, k, tau,
                       has_shared ? 1 : 0, idx, w, offsets, sorted_tok, slot_row, pp);
}

void launch_decode_gate_up(const DecodeParams& p, int max_slots, hipStream_t s) {
  hipLaunchKernelGGL(decode_gate_up_kernel, dim3(max_slots * (p.F / 16)), dim3(64 * kUpWaves), 0,
                     s, p);
}

void launch_decode_down_combine(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(decode_down_combine_kernel, dim3(p.D / 16), dim3(64 * kDownWaves), 0, s, p);
}

}  // namespace moeq4
