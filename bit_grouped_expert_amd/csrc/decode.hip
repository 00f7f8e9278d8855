// The MoE layer at decode sizes (T <= 16 tokens): one persistent launch after the router
// logits, whose workgroups stream the few touched experts' weights on every compute unit,
// with no permutation of token rows and no expert-output array in memory.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference engine for
// Qwen3.6-35B-A3B on Apple Silicon", body paragraph 7 (batch-1 decode reuses almost no
// weight, so memory bandwidth is the ceiling, and the engine cuts the number of sequential
// kernel stages by running independent kernels together) and paragraph 4 (eight of 256
// experts per token plus a shared expert).
//
// The launch (after the one-wavefront-per-expert router, which also writes the prepared
// copy of x and clears this launch's counters):
//   plan      every workgroup: the top k of every token (exact, the router's own selection
//             code), the sorted list of distinct touched experts ("slots", the shared
//             expert last), each slot's combine weight and token mask; workgroup 0 also
//             writes the layer's routing outputs (top-k, group offsets, permuted rows);
//   items     one per workgroup, in workgroup order, gate_up items first:
//     gate_up  (slot, 16 rows of gate and the matching 16 of up): the slot's tokens
//              against those rows, K over eight wavefronts, SwiGLU, activations stored
//              in the down step's fragment order; then the slot's counter is raised;
//     down     (16 output columns, group of consecutive slots): the group's down weights
//              are staged first, then the item waits for its slots' gate_up counters,
//              multiplies, scales by the combine weights and sums in fp32 in a fixed
//              order; with several groups the last one to arrive adds the groups'
//              partial sums in group order and writes the bf16 output.
// A down item waits only on gate_up items, all of lower workgroup index.  Workgroups are
// dispatched in index order, so those are running or done, and they never wait: every
// wait ends, whether or not the whole grid fits on the chip at once.  A wait is also
// bounded: past the limit it raises the error word and goes on.
//
// Cross-workgroup data (activations, the groups' partial sums) and the counters use
// device-scope loads and stores, which are coherent across the chiplets' L2 caches without
// cache-wide write-back or invalidation; a writer waits for its stores to complete before
// it raises a counter, and a reader loads only after it has seen the counter.  A single
// counter that every workgroup increments (a ticket queue) serialises at the memory and
// costs far more than a whole item, so items are not dealt that way.
//
// Arithmetic per 64-wide group g of one weight row (scale s, bias b): the matrix cores give
// P' = sum x (128 + q) with exact products (128 + q is the bf16 0x4300 | q) and the row sums
// X = sum x (activations times a fragment of ones); then acc += s P' + (b - 128 s) X in
// fp32.  The K order inside a group is a permutation shared by both operands: in MFMA step
// h of group g, quarter q of the lanes takes packed word 8 g + 2 q + h of its weight row
// and the matching eight activations, so each step stays inside one scale group.
#include "common.h"
#include "internal.h"
#include "q4_stream.h"
#include "topk_select.h"

namespace moeq4 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kUpMaxD = 2048;
constexpr int kMaxF = 1024;
constexpr int kGroupSlots = 10;                       // most slots of one down item
constexpr int kDownCodeArea = 40 * 1024;              // code slices of one down item
constexpr int kDownSbArea = kDownCodeArea / 8;        // their scales and biases
constexpr int kDownActArea = 16 * 1024;               // activation rows of one round
constexpr int kUpCodeBytes = 32 * kUpMaxD / 2;        // 32 code rows of one gate_up item
constexpr int kUpSbBytes = 4 * 32 * (kUpMaxD / 64);   // their scales and biases
constexpr int kSlack = 1024;                          // past-the-end writes of staging
constexpr int kUpArea = kUpCodeBytes + kSlack + kUpSbBytes + kSlack;
constexpr int kDownArea = kDownCodeArea + kSlack + kDownSbArea + kSlack + kDownActArea + kSlack;
constexpr int kArea = kUpArea > kDownArea ? kUpArea : kDownArea;
constexpr int kSpinLimit = 1 << 16;                   // polls before a wait gives up
static_assert((int)sizeof(f32x4_t) * kWaves * 2 * 64 <= kUpCodeBytes, "gate_up reduction");
static_assert((int)sizeof(float) * kWaves * 16 * 17 <= kDownCodeArea, "down reduction");
static_assert(kGroupSlots <= 16, "pair scan width");

// counters and flags, cleared before every launch: [0] error (waits that gave up);
// [kSyncCb + 32 cb] down groups done for column block cb, one 128-byte line each; then one
// done flag per gate_up item, slot-major, set by a plain store.  Many atomics on one line
// serialise at the memory, so nothing is counted that way on the critical path.
constexpr int kSyncCb = 32;
constexpr int kSyncPlan = 1;  // [1]: workgroup 0 has published the plan
__host__ __device__ inline int sync_flags_base(int n_cb) { return kSyncCb + 32 * n_cb; }

// the published plan (32-bit words): n_slots, slot_exp, rowmask, then coef
constexpr int kPubExp = 1, kPubMask = kPubExp + kDecodeMaxSlots, kPubCoef = kPubMask + kDecodeMaxSlots;
constexpr int kPubWords = kPubCoef + kDecodeMaxSlots * 16;

// the plan, in LDS, identical in every workgroup
struct Plan {
  float coef[kDecodeMaxSlots * 16];   // combine weight of slot s for token t (16-byte rows)
  int sel_e[kDecodeMaxPairs];
  float sel_w[kDecodeMaxPairs];
  uint32_t bits[32];  // touched experts, E <= 1024
  int word_base[33];
  int slot_exp[kDecodeMaxSlots];      // expert of each slot, -1 = the shared expert
  uint32_t rowmask[kDecodeMaxSlots];  // tokens of each slot
  int n_slots;
  int last;  // a down item completes its column block
  int pub_ok;  // the published plan was there
  // a down item's (slot, token) pairs: pair j of the group's slot b is pbase[b] + j, and
  // prow[pair] is its activation row (slot * 16 + token)
  int pbase[kGroupSlots + 1];
  int prow[kDecodeMaxPairs + kDecodeMaxT];
  int lrow[kGroupSlots * 16];  // staged row of (slot b, token t) in this round, or -1
};

__device__ __forceinline__ int slot_of(const Plan& pl, int e) {
  return pl.word_base[e >> 5] + __popc(pl.bits[e >> 5] & ((1u << (e & 31)) - 1u));
}

// inclusive prefix sum over the first n lanes of a wavefront (n <= 64, power of two)
__device__ __forceinline__ int wave_scan_incl(int v, int n) {
  const int lane = threadIdx.x & 63;
  for (int off = 1; off < n; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
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

// as stage(), with device-scope loads (data written by other workgroups of this launch)
template <typename Src>
__device__ __forceinline__ void stage_dev(unsigned char* dst, int nch, Src src, int wave, int nw,
                                          int lane) {
  const int n_ins = (nch + 63) >> 6;
  for (int k = wave; k < n_ins; k += nw) {
    int c = 64 * k + lane;
    if (c >= nch) c = nch - 1;
    __builtin_amdgcn_global_load_lds(src(c), dst + 1024 * k, 16, 0, 16 /* sc1: device scope */);
  }
}

// the 8 bytes of words (w, w + 1) (w even) of staged code row r (cpr chunks per row)
__device__ __forceinline__ u32x2_t lds_words(const unsigned char* rows, int r, int cpr, int w) {
  const int c = w >> 2;
  return *(const u32x2_t*)(rows + (r * cpr + (c ^ (r & chunk_mask(cpr)))) * 16 + (w & 3) * 4);
}

// ------------------------------------------------------------------------------- plan
// Every workgroup: waves take tokens t, t + 8 (one wavefront selects one token's top k).
// `writer` also stores the routing outputs: top-k ids and weights, group offsets (pairs
// with a lower expert), permuted rows (stable: a pair's rank among the earlier pairs with
// the same expert) and, with the shared expert, its T rows after the T k routed ones.
template <int MAXC>
__device__ void make_plan(const DecodeParams& p, Plan& pl, bool writer) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, E = p.E, k = p.k;
  if (tid < 32) pl.bits[tid] = 0u;
  for (int i = tid; i < kDecodeMaxSlots; i += kThreads) pl.rowmask[i] = 0u;
  __syncthreads();
  for (int t = wave; t < T; t += kWaves) {
    int e;
    float w;
    topk_token<MAXC>(p.logits + (int64_t)t * E, p.x + (int64_t)t * p.D, p.R, p.D, E, k, p.tau, e, w);
    if (lane < k) {
      pl.sel_e[t * k + lane] = e;
      pl.sel_w[t * k + lane] = w;
      atomicOr(&pl.bits[e >> 5], 1u << (e & 31));
      if (writer) {
        p.idx[t * k + lane] = e;
        p.w[t * k + lane] = w;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {  // slot of the first expert of each 32-expert word
    const int c = lane < 32 ? __popc(pl.bits[lane]) : 0;
    const int inc = wave_scan_incl(c, 32);
    if (lane < 32) pl.word_base[lane] = inc - c;
    if (lane == 31) {
      pl.word_base[32] = inc;
      pl.n_slots = inc + (p.has_shared ? 1 : 0);
    }
  }
  __syncthreads();
  const int n_distinct = pl.word_base[32], n_slots = pl.n_slots;
  for (int e = tid; e < E; e += kThreads)
    if ((pl.bits[e >> 5] >> (e & 31)) & 1u) pl.slot_exp[slot_of(pl, e)] = e;
  if (p.has_shared && tid == 0) {
    pl.slot_exp[n_distinct] = -1;
    pl.rowmask[n_distinct] = (T < 32 ? (1u << T) : 0u) - 1u;
  }
  for (int i = tid; i < n_slots * 16; i += kThreads) {
    const int s = i >> 4, t = i & 15;
    pl.coef[i] = (p.has_shared && s == n_distinct && t < T) ? 1.f : 0.f;
  }
  __syncthreads();
  const int pairs = T * k;
  if (tid < pairs) {
    const int t = tid / k, e = pl.sel_e[tid], s = slot_of(pl, e);
    pl.coef[s * 16 + t] = pl.sel_w[tid];
    atomicOr(&pl.rowmask[s], 1u << t);
    if (writer) {
      int below = 0, rank = 0;
      for (int u = 0; u < pairs; ++u) {
        const int eu = pl.sel_e[u];
        below += eu < e ? 1 : 0;
        rank += (u < tid && eu == e) ? 1 : 0;
      }
      p.sorted_tok[below + rank] = t;
      p.slot_row[tid] = below + rank;
    }
  }
  if (writer) {
    for (int e = tid; e <= E; e += kThreads) {
      int below = 0;
      for (int u = 0; u < pairs; ++u) below += pl.sel_e[u] < e ? 1 : 0;
      p.offsets[e] = below;
    }
    if (p.has_shared) {
      if (tid == 0) p.offsets[E + 1] = pairs + T;
      if (tid < T) p.sorted_tok[pairs + tid] = tid;
    }
  }
  __syncthreads();
}

// Workgroup 0 publishes the parts of the plan the items read (device-scope stores, complete
// before the flag is raised); a workgroup of a later round waits for the flag (bounded: if
// it does not come, the workgroup computes the plan itself) and loads them.
__device__ void publish_plan(const DecodeParams& p, const Plan& pl) {
  const int tid = threadIdx.x, n = pl.n_slots;
  for (int i = tid; i < n; i += kThreads) {
    store_dev(p.plan + kPubExp + i, (uint32_t)pl.slot_exp[i]);
    store_dev(p.plan + kPubMask + i, pl.rowmask[i]);
  }
  for (int i = tid; i < n * 16; i += kThreads) store_dev(p.plan + kPubCoef + i, __float_as_uint(pl.coef[i]));
  if (tid == 0) store_dev(p.plan, (uint32_t)n);
  wait_vmcnt0();
  __syncthreads();
  if (tid == 0) store_dev((uint32_t*)(p.sync + kSyncPlan), 1u);
}

__device__ bool load_plan(const DecodeParams& p, Plan& pl) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    int spins = 0, got = 0;
    for (;;) {
      if (__all(load_dev((const uint32_t*)(p.sync + kSyncPlan)) != 0u)) {
        got = 1;
        break;
      }
      if (++spins > kSpinLimit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (tid == 0) pl.pub_ok = got;
  }
  __syncthreads();
  if (!pl.pub_ok) return false;  // the same in every thread
  const int n = (int)load_dev(p.plan);
  for (int i = tid; i < n; i += kThreads) {
    pl.slot_exp[i] = (int)load_dev(p.plan + kPubExp + i);
    pl.rowmask[i] = load_dev(p.plan + kPubMask + i);
  }
  for (int i = tid; i < n * 16; i += kThreads) pl.coef[i] = __uint_as_float(load_dev(p.plan + kPubCoef + i));
  if (tid == 0) pl.n_slots = n;
  __syncthreads();
  return true;
}

// ------------------------------------------------------------------------------- gate_up
// Item (slot s, slice sl): 16 gate rows 16 sl .. and the matching 16 up rows.  The slice's
// codes (32 rows) and its scale and bias rows go to LDS first; while they land, wavefront
// w loads the slot's token rows of the prepared x for the 256-K stages w, w + 8, ...
// (other rows are zero).  The eight partial sums meet through LDS (over the code area, once
// every wavefront is done with it) in a fixed order; wavefront 0 applies SwiGLU, stores the
// slot's token rows (act[slot][token][F], columns in the prepared order of x, device-scope
// stores) and, once they are complete, sets the item's done flag.
__device__ void gate_up_item(const DecodeParams& p, const Plan& pl, unsigned char* area, int s,
                             int sl) {
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int F = p.F, D = p.D, KW = D >> 3, KG = D >> 6, CPR = D >> 5;
  const int e = __builtin_amdgcn_readfirstlane(pl.slot_exp[s]);
  const Q4Ptrs& W = e >= 0 ? p.up_main : p.up_last;
  const int64_t base_row = (int64_t)(e >= 0 ? e : 0) * (2 * F);
  const int64_t gate0 = base_row + 16 * sl, up0 = base_row + F + 16 * sl;
  const int mask = chunk_mask(CPR);
  unsigned char* codes = area;
  unsigned char* sb = area + kUpCodeBytes + kSlack;
  // staged rows 0..15: gate rows gate0 + r; 16..31: up rows up0 + r - 16
  stage(codes, 32 * CPR, [&](int c) {
    const int r = c / CPR, cs = c - r * CPR;
    const int64_t row = (r < 16 ? gate0 : up0 - 16) + r;
    return (const unsigned char*)(W.q + row * KW) + 16 * (cs ^ (r & mask));
  }, wave, kWaves, l);
  // four regions of 16 rows x KG bf16 (2 KG chunks each): gate s, up s, gate b, up b
  const int rch = 2 * KG;
  stage(sb, 4 * rch, [&](int c) {
    const int rg = c / rch, w = c - rg * rch;
    const uint16_t* base = (rg < 2 ? W.s : W.b) + ((rg & 1) ? up0 : gate0) * KG;
    return (const unsigned char*)base + 16 * w;
  }, (wave + 4) % kWaves, kWaves, l);
  // this wavefront's activations: the slot's token rows only
  const uint32_t rows = pl.rowmask[s];
  const bool mine = (rows >> m) & 1u;
  const uint16_t* xr = p.xprep + (int64_t)m * D + 16 * q;
  const int NST = D >> 8;
  constexpr int kMaxSt = kUpMaxD / 256 / kWaves;
  u32x4_t a[kMaxSt][4][2];
#pragma unroll
  for (int v = 0; v < kMaxSt; ++v) {
    const int st = wave + kWaves * v;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        a[v][g][h] = u32x4_t{0u, 0u, 0u, 0u};
        if (st < NST && mine) a[v][g][h] = *(const u32x4_t*)(xr + 256 * st + 64 * g + 8 * h);
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
    const int st = wave + kWaves * v;
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
  f32x4_t* part = (f32x4_t*)area;  // [wave][2][64]
  part[(wave * 2 + 0) * 64 + l] = acc[0];
  part[(wave * 2 + 1) * 64 + l] = acc[1];
  __syncthreads();
  if (wave == 0) {
    f32x4_t g4 = part[l], u4 = part[64 + l];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const f32x4_t gp = part[(2 * w) * 64 + l], up = part[(2 * w + 1) * 64 + l];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g4[i] += gp[i];
        u4[i] += up[i];
      }
    }
    // natural column c = 16 sl + m: prepared word w = c / 8, position perm8(c % 8); word w
    // is group w / 8, quarter (w % 8) / 2, step (w % 8) & 1 of the down step's fragments
    // natural column c = 16 sl + m sits at 8 (c / 8) + perm8(c % 8) of the prepared row.
    // Lanes m and m + 4 (m % 8 < 4) hold columns c and c + 4, positions 2 j and 2 j + 1:
    // the first stores both as one 32-bit word.
    const int c = 16 * sl + m;
    uint16_t* dst = p.act + (int64_t)s * 16 * F + 8 * (c >> 3) + perm8(c & 7);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * q + i;
      const float gte = g4[i];
      const uint32_t v = to_bf16(gte / (1.f + __expf(-gte)) * u4[i]);
      const uint32_t hi = (uint32_t)__shfl_down((int)v, 4, 64);
      if ((m & 4) == 0 && ((rows >> r) & 1u)) store_dev((uint32_t*)(dst + (int64_t)r * F), v | (hi << 16));
    }
    wait_vmcnt0();
    if (l == 0) store_dev((uint32_t*)(p.sync + sync_flags_base(p.n_cb) + s * (F >> 4) + sl), 1u);
  }
}

// ------------------------------------------------------------------------------- down
// Item (column block cb, slot group sg): 16 output columns n0 = 16 cb .. against the slots
// [s_lo, s_hi) of the group.  The slices' codes and scale and bias rows go to LDS first;
// meanwhile wavefront 0 reads the done flags of the group's gate_up items (all lanes at
// once) until every one is set.  Then, round by round, the group's (slot, token) rows of
// activations go to LDS (device-scope loads, only the rows the tokens routed), and the
// (slot, 256-K part) units are dealt to the wavefronts: a unit reads its A fragments from
// the staged rows (zero for tokens not in the round) and adds coef[slot][t] (s P' +
// (b - 128 s) X) over its four groups to the wavefront's sums for its 16 columns and 16
// token rows.  The eight partial sums meet through LDS in a fixed order.  One group: the
// bf16 row pieces go straight out.  Several: the group's sums go to `part`, and the last
// group to arrive (counter per column block) adds all groups' sums in group order and
// writes the output.
__device__ void down_item(const DecodeParams& p, Plan& pl, unsigned char* area, int cb, int sg,
                          int n_sg) {
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int F = p.F, D = p.D, n0 = 16 * cb;
  const int KW = F >> 3, KG = F >> 6, CPR = F >> 5, NSL = F >> 4;
  const int n_slots = pl.n_slots;
  const int s_lo = sg * n_slots / n_sg, s_hi = (sg + 1) * n_slots / n_sg, nb = s_hi - s_lo;
  const int mask = chunk_mask(CPR);
  unsigned char* codes = area;
  unsigned char* sbl = area + kDownCodeArea + kSlack;
  // activation area: one zero row (tokens a slot does not have read it), then the rows of
  // a round
  unsigned char* acts = sbl + kDownSbArea + kSlack;
  unsigned char* arows = acts + 2 * F;
  for (int i = tid; i < F / 8; i += kThreads) *(u32x4_t*)(acts + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
  // codes: staged row r = 16 b + i is row n0 + i of slot s_lo + b's expert
  stage(codes, nb * 16 * CPR, [&](int c) {
    const int r = c / CPR, cs = c - r * CPR;
    const int e = pl.slot_exp[s_lo + (r >> 4)];
    const Q4Ptrs& W = e >= 0 ? p.down_main : p.down_last;
    const int64_t row = (int64_t)(e >= 0 ? e : 0) * D + n0 + (r & 15);
    return (const unsigned char*)(W.q + row * KW) + 16 * (cs ^ (r & mask));
  }, wave, kWaves, l);
  // scales then biases of each slot's 16 rows (16 KG bf16, 2 KG chunks each)
  const int rch = 2 * KG;
  stage(sbl, nb * 2 * rch, [&](int c) {
    const int rg = c / rch, w = c - rg * rch;
    const int e = pl.slot_exp[s_lo + (rg >> 1)];
    const Q4Ptrs& W = e >= 0 ? p.down_main : p.down_last;
    const int64_t row = (int64_t)(e >= 0 ? e : 0) * D + n0;
    return (const unsigned char*)(((rg & 1) ? W.b : W.s) + row * KG) + 16 * w;
  }, (wave + 4) % kWaves, kWaves, l);
  if (wave == 0) {
    // the group's pairs: slot b's first at pbase[b]
    const int c = l < nb ? __popc(pl.rowmask[s_lo + l]) : 0;
    const int inc = wave_scan_incl(c, 16);  // nb <= kGroupSlots <= 16
    if (l < nb) pl.pbase[l] = inc - c;
    if (l == nb - 1) pl.pbase[nb] = inc;
    // the done flags of the group's gate_up items
    const int32_t* fl = p.sync + sync_flags_base(p.n_cb) + s_lo * NSL;
    const int nf = nb * NSL;
    int spins = 0;
    for (;;) {
      int ok = 1;
      for (int i = l; i < nf; i += 64) ok &= load_dev((const uint32_t*)(fl + i)) != 0u ? 1 : 0;
      if (__all(ok)) break;
      if (++spins > kSpinLimit) {
        if (l == 0) atomic_add_agent(p.sync, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  wait_vmcnt0();
  __syncthreads();
  if (tid < nb) {
    uint32_t mk = pl.rowmask[s_lo + tid];
    int j = pl.pbase[tid];
    while (mk) {
      pl.prow[j++] = (s_lo + tid) * 16 + __builtin_ctz(mk);
      mk &= mk - 1u;
    }
  }
  __syncthreads();
  const int npairs = pl.pbase[nb];
  const int R = kDownActArea / (2 * F) - 1;  // activation rows per round
  const int CPA = F >> 3;                 // 16-byte chunks per activation row
  const uint32_t magic = opaque_magic();
  const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  f32x4_t out = zero;
  for (int r0 = 0; r0 < npairs; r0 += R) {
    const int nr = npairs - r0 < R ? npairs - r0 : R;
    if (r0 > 0) __syncthreads();  // the previous round's reads are done
    stage_dev(arows, nr * CPA, [&](int c) {
      const int pr = c / CPA, w = c - pr * CPA;
      return (const unsigned char*)(p.act + (int64_t)pl.prow[r0 + pr] * F) + 16 * w;
    }, wave, kWaves, l);
    if (tid < nb * 16) {
      const int b = tid >> 4, t = tid & 15;
      const uint32_t mk = pl.rowmask[s_lo + b];
      const int pr = pl.pbase[b] + __popc(mk & ((1u << t) - 1u)) - r0;
      pl.lrow[tid] = ((mk >> t) & 1u) && pr >= 0 && pr < nr ? pr : -1;
    }
    wait_vmcnt0();
    __syncthreads();
    // Wavefront w: the 64-wide groups w, w + 8, ... of every slot, two slots per step as
    // straight-line code (a step past the last slot repeats it with a zero weight).  Per
    // slot b the LDS addresses move by fixed strides: code rows 16 b .. (same chunk order,
    // as the row's swizzle depends on the row modulo 16), scale and bias rows, weights.
    for (int g = wave; g < KG; g += kWaves) {
      const unsigned char* c0 = codes + (m * CPR + ((2 * g + (q >> 1)) ^ (m & mask))) * 16 + 8 * (q & 1);
      const unsigned char* s0 = sbl + (m * KG + g) * 2;
      const unsigned char* a0p = arows + 128 * g + 32 * q;
      auto slot = [&](int b, float wmul, f32x4_t& acc) __attribute__((always_inline)) {
        const unsigned char* ar = a0p + pl.lrow[b * 16 + m] * (2 * F);  // -1: the zero row
        const u32x4_t x0 = *(const u32x4_t*)ar;
        const u32x4_t x1 = *(const u32x4_t*)(ar + 16);
        const u32x2_t wd = *(const u32x2_t*)(c0 + b * 256 * CPR);
        const float sg = bf16lo_to_f32(*(const uint16_t*)(s0 + b * 64 * KG));
        const float bg = bf16lo_to_f32(*(const uint16_t*)(s0 + b * 64 * KG + 32 * KG));
        const f32x4_t cf = *(const f32x4_t*)&pl.coef[(s_lo + b) * 16 + 4 * q];
        const f32x4_t X = mfma16x16x32(x1, ones, mfma16x16x32(x0, ones, zero));
        const f32x4_t P = mfma16x16x32(x1, unpack_word(wd[1], magic),
                                       mfma16x16x32(x0, unpack_word(wd[0], magic), zero));
        const float ws = wmul * sg, wc = wmul * fmaf(-128.f, sg, bg);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(cf[i], fmaf(ws, P[i], wc * X[i]), acc[i]);
      };
      f32x4_t out2 = zero;
      for (int b = 0; b < nb; b += 2) {
        const bool two = b + 1 < nb;
        slot(b, 1.f, out);
        slot(two ? b + 1 : b, two ? 1.f : 0.f, out2);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] += out2[i];
    }
  }
  __syncthreads();  // every wavefront is past its LDS reads
  float* red = (float*)area;  // [wave][16][17]: out holds rows 4 q + i, column m
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * q + i) * 17 + m] = out[i];
  __syncthreads();
  const int t = tid >> 4, c = tid & 15;
  float v = 0.f;
  if (tid < 256) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * 16 + t) * 17 + c];
  }
  if (n_sg == 1) {
    if (tid < 256 && t < p.T) p.out[(int64_t)t * D + n0 + c] = to_bf16(v);
    return;
  }
  float* part = p.part + (int64_t)cb * 256;
  const int64_t gstride = (int64_t)p.n_cb * 256;
  if (tid < 256 && t < p.T) store_dev((uint32_t*)(part + sg * gstride + tid), __float_as_uint(v));
  wait_vmcnt0();
  __syncthreads();
  if (tid == 0) pl.last = atomic_add_agent(p.sync + kSyncCb + 32 * cb, 1) == n_sg - 1;
  __syncthreads();
  if (pl.last) {
    if (tid < 256 && t < p.T) {
      float sum = 0.f;
      for (int g = 0; g < n_sg; ++g)
        sum += __uint_as_float(load_dev((const uint32_t*)(part + g * gstride + tid)));
      p.out[(int64_t)t * D + n0 + c] = to_bf16(sum);
    }
  }
}

// ------------------------------------------------------------------------------- launch
// Two workgroups per compute unit (LDS and, for E <= 256, 128 registers per lane); the
// 1024-expert selection needs more registers and runs one per compute unit.
template <int MAXC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MAXC <= 4 ? 4 : 1)))
void decode_layer_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) Plan pl;
  __shared__ __attribute__((aligned(16))) unsigned char area[kArea];
  if ((int)blockIdx.x < p.early || !load_plan(p, pl)) make_plan<MAXC>(p, pl, blockIdx.x == 0);
  if (blockIdx.x == 0 && p.early < (int)gridDim.x) publish_plan(p, pl);
  const int n_slots = pl.n_slots, NSL = p.F >> 4;
  const int n_up = n_slots * NSL;
  const int n_sg = (n_slots + p.group_slots - 1) / p.group_slots;
  const int t = blockIdx.x;
  if (t < n_up) {
    gate_up_item(p, pl, area, t / NSL, t - (t / NSL) * NSL);
  } else if (t < n_up + p.n_cb * n_sg) {
    const int d = t - n_up, sg = d / p.n_cb;
    down_item(p, pl, area, d - sg * p.n_cb, sg, n_sg);
  }
}

}  // namespace

bool decode_supported(int T, int D, int E, int k, int F) {
  return T >= 1 && T <= kDecodeMaxT && T * k <= kDecodeMaxPairs && E <= 1024 && D % 256 == 0 &&
         D <= kUpMaxD && F % 64 == 0 && F <= kMaxF;
}

int decode_group_slots(int F) {
  const int by_area = kDownSbArea / F;  // nb F bytes of scales and biases, 8 nb F of codes
  return by_area < kGroupSlots ? by_area : kGroupSlots;
}

int decode_sync_ints(int D, int F, int max_slots) {
  return sync_flags_base(D / 16) + max_slots * (F / 16);
}

size_t decode_part_bytes(int D, int F, int max_slots) {
  const int gs = decode_group_slots(F);
  return (size_t)((max_slots + gs - 1) / gs) * (D / 16) * 256 * sizeof(float);
}

size_t decode_act_bytes(int F, int max_slots) { return (size_t)max_slots * 16 * F * 2; }

size_t decode_plan_bytes() { return (size_t)kPubWords * 4; }

void launch_decode_layer(const DecodeParams& p, int max_slots, hipStream_t s) {
  // the most items any routing can give; workgroups past the actual count return
  const int gs = decode_group_slots(p.F);
  const int64_t items = (int64_t)max_slots * (p.F / 16) + (int64_t)p.n_cb * ((max_slots + gs - 1) / gs);
  const dim3 grid((unsigned)items), block(kThreads);
  if (p.E <= 64)
    hipLaunchKernelGGL(decode_layer_kernel<1>, grid, block, 0, s, p);
  else if (p.E <= 256)
    hipLaunchKernelGGL(decode_layer_kernel<4>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(decode_layer_kernel<16>, grid, block, 0, s, p);
}

}  // namespace moeq4
