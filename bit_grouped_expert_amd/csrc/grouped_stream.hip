// Streamed grouped GEMM over groupwise-affine 4-bit weights for gfx950 (MI355X),
// for K a multiple of 128.  Same arithmetic and tiling as the grouped engine in
// grouped_gemm.hip; the difference is how the operands travel.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
// engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph 5 (4-bit weights
// with one bf16 scale and bias per 64, reconstructed tile by tile inside the
// grouped GEMM with FP32 accumulation) and paragraph 7 (with little weight reuse,
// bandwidth sets the ceiling).
//
// Operand stream.  Every operand of a 128-K stage reaches LDS through direct
// global->LDS loads (global_load_lds_dwordx4 / _dword), held in a ring of RING
// stage slots, so RING - 1 stages are in flight without holding a VGPR:
//   - each wavefront's own 64 weight rows: the packed codes (16 B per lane per
//     fragment) and one dword of two bf16 scales and one of two biases per row;
//   - the tile's activation rows, shared by the four wavefronts, taken from a
//     prepared copy in which every run of 8 columns is stored in the order
//     0,4,1,5,2,6,3,7 (the order in which a packed word unpacks), with the 16-byte
//     chunk index of row r XOR-ed with r % 16 so that matrix-operand reads are
//     free of bank conflicts without padding;
//   - per row and stage, the prepared (-136 X_lo, -136 X_hi, X_lo, X_hi) of the
//     stage's two scale groups (X = row sum of the activations over the group).
// The work items of a workgroup form one stream of stages, so the ring keeps
// filling across item boundaries.  Per stage a wavefront issues exactly
// 7 + NF vector-memory instructions, always, with addresses clamped to valid
// rows; before consuming stage s it waits until no more of its vector-memory
// operations are outstanding than those of the stages issued after s (they
// complete in order), then a workgroup barrier makes every wavefront's part of
// the stage visible and frees the slot of stage s - 1 for the next load.  The
// compiler does not order LDS reads after these loads by itself, hence the
// explicit waits.  Row indices of the next item are loaded one item ahead, so
// waiting for them never drains the ring.
//
// Matrix-core work per stage and wavefront: for each of the two scale groups and
// each 16-row fragment, P = sum_c x (128 + q) starting from -136 X on
// v_mfma_f32_16x16x32_bf16, then acc += s * P (+ (b + 8 s) X when b != -8 s).
// MFMA steps 0 and 1 take words 2q and 2q+1 of a row (first group), steps 2 and 3
// words 8+2q and 9+2q (second group), each pair one 8-byte LDS read.
//
// One workgroup of four wavefronts per compute unit; persistent, XCD-aware grid as
// in the grouped engine.  Tiles hold up to 16*NF rows (NF fixed per launch);
// fragments past a tile's last row are skipped.
#include "common.h"
#include "internal.h"

namespace moeq4 {

namespace {

constexpr int KS = 128;                      // K per stage
constexpr int RING = 4;                      // stage slots
constexpr int CODE_BYTES = 4 * 64 * 16;      // per wave: four fragments x 64 lanes x 16 B
constexpr int WAVE_BYTES = CODE_BYTES + 2 * 256;  // + scale and bias dwords of 64 rows
constexpr int XC_BYTES = 64 * 16;            // per wave: 16 rows (lanes duplicated 4x)
constexpr int LDC_SWIGLU = 128 + 8;
constexpr int LDC_PLAIN = 256 + 8;
constexpr int TABLE_CAP = 768;               // most items of one workgroup (host-enforced)
constexpr uint32_t kMagic = 0x43004300u;
constexpr uint32_t kNib = 0x000F000Fu;

template <int NF>
struct Lay {
  static constexpr int BM = 16 * NF;
  static constexpr int A_OFF = 0;                       // BM rows x 256 B
  static constexpr int XC_OFF = BM * 256;               // 4 waves x 1 KB
  static constexpr int W_OFF = XC_OFF + 4 * XC_BYTES;   // 4 waves x WAVE_BYTES
  static constexpr int SLOT = W_OFF + 4 * WAVE_BYTES;
  static constexpr int TABLE_OFF = RING * SLOT;          // this workgroup's tiles
  static constexpr int IDX_OFF = TABLE_OFF + TABLE_CAP * 8;  // [4 waves][2][64] row indices
  static constexpr int TOTAL = IDX_OFF + 4 * 2 * 64 * 4;
  static constexpr int DMA_PER_STAGE = 7 + NF;          // 4 codes + scale + bias + xc + NF rows
};
static_assert(Lay<4>::TOTAL <= 160 * 1024, "LDS budget");
static_assert(Lay<2>::TOTAL <= 160 * 1024, "LDS budget");
static_assert(Lay<4>::SLOT >= 64 * LDC_PLAIN * 2, "output staging fits a slot");
static_assert(Lay<2>::SLOT >= 32 * LDC_PLAIN * 2, "output staging fits a slot");

// kMagic in a VGPR whose value the compiler does not know, so that (v & mask) | magic
// becomes one v_and_or_b32 (only VALU instructions read it).
__device__ __forceinline__ uint32_t opaque_magic() {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "n"(kMagic));
  return v;
}

__device__ __forceinline__ u32x4_t unpack_word(uint32_t w, uint32_t magic) {
  u32x4_t b;
  b[0] = (w & kNib) | magic;
  b[1] = ((w >> 4) & kNib) | magic;
  b[2] = ((w >> 8) & kNib) | magic;
  b[3] = ((w >> 12) & kNib) | magic;
  return b;
}

__device__ __forceinline__ float sum8_bf16(u32x4_t v) {
  float s = 0.f;
#pragma unroll
  for (int h = 0; h < 4; ++h) s += bf16lo_to_f32(v[h]) + bf16hi_to_f32(v[h]);
  return s;
}

// s_waitcnt vmcnt(N), other counters unconstrained (GFX9 encoding), fenced so that
// no memory access is moved across it
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS traffic only: waits for this wavefront's LDS operations,
// not for its global memory operations (a __syncthreads() release fence would wait for
// every outstanding vector-memory operation, draining the operand ring).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// LDS reads whose result is complete when the statement ends, issued as inline
// assembly so that the compiler attaches no vector-memory wait to them (it cannot
// tell these tables apart from the targets of the in-flight direct loads)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ int2 lds_read_i2(const void* p) {
  int2 v;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(v)
               : "v"(lds_addr(p))
               : "memory");
  return v;
}
__device__ __forceinline__ int lds_read_i1(const void* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(v)
               : "v"(lds_addr(p))
               : "memory");
  return v;
}

// natural column c (0..7) of an 8-column run -> its position in the stored order 0,4,1,5,...
__device__ __forceinline__ int perm8(int c) { return ((c & 3) << 1) | (c >> 2); }

template <bool SWIGLU>
__device__ __forceinline__ void wave_rows(int N, int slice, int wave, int first[4], bool& active) {
  if (SWIGLU) {
    const int F = N >> 1;
    const int c = slice * 128 + 32 * wave;
    active = c < F;
    const int cc = active ? c : 0;
    first[0] = cc;
    first[1] = cc + 16;
    first[2] = F + cc;
    first[3] = F + cc + 16;
  } else {
    const int c = slice * 256 + 64 * wave;
    active = c < N;
    const int cc = active ? c : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) first[j] = cc + 16 * j;
  }
}

template <int NF, bool SWIGLU>
__device__ __forceinline__ void stream_body(const StreamParams& p, unsigned char* smem) {
  using LY = Lay<NF>;
  constexpr int BM = LY::BM;

  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int N = p.N, K = p.K, KW = K >> 3, KG = K >> 6, KP = K / KS;
  const int nst = KP;

  // ---- this workgroup's items: XCD x takes the x-th eighth of the tile list
  const int cnt = *p.tile_count;
  const int xcd = blockIdx.x & 7, slot0 = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  const int t0 = (int)((int64_t)xcd * cnt / 8);
  const int t1 = (int)((int64_t)(xcd + 1) * cnt / 8);
  const int n_items_x = (t1 - t0) * p.n_slices;
  const int n_items = n_items_x > slot0 ? (n_items_x - slot0 + nslot - 1) / nslot : 0;
  const int total = n_items * nst;
  if (total == 0) return;  // uniform; no barrier reached
  // The tiles of this workgroup's items go to an LDS table first: reading them later
  // from global memory would be a vector load whose wait drains the operand ring.
  // Entry: (first row, group | rows << 16); rows <= 64, group < 2^16.
  int2* table = (int2*)(smem + LY::TABLE_OFF);
  for (int k = tid; k < n_items && k < TABLE_CAP; k += 256) {
    const int w = slot0 + k * nslot;
    const int4 t = p.tiles[t0 + w / p.n_slices];
    table[k] = make_int2(t.y, t.x | (t.z << 16));
  }
  lds_barrier();
  auto item_tile = [&](int k, int& slice) -> int4 {
    const int w = slot0 + k * nslot;
    const int tile = t0 + w / p.n_slices;
    slice = w - (tile - t0) * p.n_slices;
    const int2 e = lds_read_i2(table + k);
    const int row0 = __builtin_amdgcn_readfirstlane(e.x);
    const int gz = __builtin_amdgcn_readfirstlane(e.y);
    return make_int4(gz & 0xFFFF, row0, gz >> 16, 0);
  };

  const uint32_t magic = opaque_magic();
  const int zero_row = p.a_rows;  // the prepared A has one zero row after the last

  // ---- producer: row indices of the current and next item, weight bases
  // lane rows: A chunk row of DMA i is 4 (NF wave + i) + q; xc row is 16 wave + m
  // Row indices of an item's tile reach LDS by a direct load too (lane l: tile row
  // min(l, rows - 1)), one item ahead, into a per-wavefront double buffer, so that
  // no vector-memory load in the loop writes a VGPR.  They are complete when read:
  // they were issued before the loads of the first stage of the previous item,
  // which the consumer has waited for by then (at least RING - 1 stages per item;
  // shorter items wait explicitly).
  int* idxbuf = (int*)(smem + LY::IDX_OFF) + wave * 128;
  int cur_ar[NF], cur_xr;
  auto fetch_rows = [&](int k) __attribute__((always_inline)) {
    if (!p.a_row_index) return;
    int sl;
    const int4 t = item_tile(k, sl);
    const int rr = t.y + (l < t.z ? l : t.z - 1);
    __builtin_amdgcn_global_load_lds(p.a_row_index + rr, idxbuf + (k & 1) * 64, 4, 0, 0);
  };
  auto row_of = [&](int k, int row0, int nrows, int r) __attribute__((always_inline)) -> int {
    if (r >= nrows) return zero_row;
    const int a = p.a_row_index ? lds_read_i1(idxbuf + (k & 1) * 64 + r) : row0 + r;
    return (a >= 0 && a < p.a_rows) ? a : zero_row;
  };
  int p_k = -1;
  const uint32_t* p_qb = nullptr;
  const uint16_t* p_sb = nullptr;
  const uint16_t* p_bb = nullptr;
  int p_first[4];
  bool p_active;
  auto produce = [&](int gs) __attribute__((always_inline)) {
    const int k = gs / nst, s = gs - k * nst;
    if (k != p_k) {
      p_k = k;
      if (k + 1 < n_items) fetch_rows(k + 1);
      int slice;
      const int4 t = item_tile(k, slice);
      if (p.a_row_index && nst < RING - 1 && k > 0) {
        // short items: the indices of item k may not have been waited for yet
        wait_vmcnt<0>();
      }
#pragma unroll
      for (int i = 0; i < NF; ++i) cur_ar[i] = row_of(k, t.y, t.z, 4 * (NF * wave + i) + q);
      cur_xr = row_of(k, t.y, t.z, 16 * wave + m);
      const int g = t.x;
      const bool in_main = g < p.n_main;
      const int gi = in_main ? g : 0;
      p_qb = (in_main ? p.main.q : p.last.q) + (int64_t)gi * N * KW;
      p_sb = (in_main ? p.main.s : p.last.s) + (int64_t)gi * N * KG;
      p_bb = (in_main ? p.main.b : p.last.b) + (int64_t)gi * N * KG;
      wave_rows<SWIGLU>(N, slice, wave, p_first, p_active);
    }
    unsigned char* sl = smem + (gs % RING) * LY::SLOT;
    unsigned char* wv = sl + LY::W_OFF + wave * WAVE_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(p_qb + (uint32_t)(p_first[j] + m) * KW + 16 * s + 4 * q,
                                       wv + j * 1024, 16, 0, 0);
    const int jr = q == 0 ? p_first[0] : q == 1 ? p_first[1] : q == 2 ? p_first[2] : p_first[3];
    const uint32_t srow = (uint32_t)(jr + m) * KG + 2 * s;
    __builtin_amdgcn_global_load_lds(p_sb + srow, wv + CODE_BYTES, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(p_bb + srow, wv + CODE_BYTES + 256, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(p.xc + (uint32_t)cur_xr * KP + s,
                                     sl + LY::XC_OFF + wave * XC_BYTES, 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int r = 4 * (NF * wave + i) + q;  // tile row of this lane's chunk
      const int c = m ^ (r & 15);             // logical 16-B chunk stored at position m
      __builtin_amdgcn_global_load_lds(p.A + (uint32_t)cur_ar[i] * K + KS * s + 8 * c,
                                       sl + LY::A_OFF + (NF * wave + i) * 1024, 16, 0, 0);
    }
  };

  // ---- consumer state of the current item
  int c_row0 = 0, c_nrows = 0, c_slice = 0, nfv = 0;
  bool c_active = false;
  f32x4_t acc[NF][4];
  auto begin_item = [&](int k) __attribute__((always_inline)) {
    const int4 t = item_tile(k, c_slice);
    c_row0 = t.y;
    c_nrows = t.z < 0 ? 0 : (t.z > BM ? BM : t.z);
    nfv = (c_nrows + 15) >> 4;
    int first[4];
    wave_rows<SWIGLU>(N, c_slice, wave, first, c_active);
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[f][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  auto compute = [&](int gs) __attribute__((always_inline)) {
    const unsigned char* sl = smem + (gs % RING) * LY::SLOT;
    const unsigned char* wv = sl + LY::W_OFF + wave * WAVE_BYTES;
    const uint16_t* a = (const uint16_t*)(sl + LY::A_OFF);
    u32x2_t w01[4], w23[4];
    uint32_t spair[4], bpair[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned char* sj = wv + j * 1024 + 16 * m + 8 * (q & 1);
      w01[j] = *(const u32x2_t*)(sj + 256 * (q >> 1));
      w23[j] = *(const u32x2_t*)(sj + 256 * (2 + (q >> 1)));
      spair[j] = *(const uint32_t*)(wv + CODE_BYTES + 4 * (16 * j + m));
      bpair[j] = *(const uint32_t*)(wv + CODE_BYTES + 256 + 4 * (16 * j + m));
    }
    // (C0_lo, C0_hi, X_lo, X_hi) of rows 16f + 4q + i: wave (f)'s xc block, lane 4q + i
    f32x4_t xc[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xc[f][i] = *(const f32x4_t*)(sl + LY::XC_OFF + f * XC_BYTES + 16 * (4 * q + i));
    // b == -8 s exactly for every row and both groups (a conservative bit test: a
    // normal, not huge scale s has -8 s = s with exponent + 3 and the sign set)
    bool cz = true;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e0 = (spair[j] >> 7) & 0xFFu, e1 = (spair[j] >> 23) & 0xFFu;
      cz = cz && bpair[j] == ((spair[j] + 0x01800180u) ^ 0x80008000u) && e0 != 0u && e1 != 0u &&
           e0 < 0xFCu && e1 < 0xFCu;
    }
    const bool all_cz = __all(cz);
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      float sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[j] = grp ? bf16hi_to_f32(spair[j]) : bf16lo_to_f32(spair[j]);
      u32x4_t av[2][NF];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int wd = grp ? 8 + 2 * q + h : 2 * q + h;  // logical 16-B chunk (word) index
#pragma unroll
        for (int f = 0; f < NF; ++f) av[h][f] = *(const u32x4_t*)(a + (16 * f + m) * 128 + 8 * (wd ^ m));
      }
      f32x4_t C0[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) C0[f][i] = xc[f][i][grp];
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        f32x4_t P[NF][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t wa = grp ? w23[2 * jh][h] : w01[2 * jh][h];
          const uint32_t wb = grp ? w23[2 * jh + 1][h] : w01[2 * jh + 1][h];
          const u32x4_t B0 = unpack_word(wa, magic);
          const u32x4_t B1 = unpack_word(wb, magic);
#pragma unroll
          for (int f = 0; f < NF; ++f)
            if (f < nfv) {
              P[f][0] = mfma16x16x32(av[h][f], B0, h ? P[f][0] : C0[f]);
              P[f][1] = mfma16x16x32(av[h][f], B1, h ? P[f][1] : C0[f]);
            }
        }
        if (all_cz) {
#pragma unroll
          for (int f = 0; f < NF; ++f)
            if (f < nfv) {
#pragma unroll
              for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  acc[f][2 * jh + jj][i] =
                      fmaf(sc[2 * jh + jj], P[f][jj][i], acc[f][2 * jh + jj][i]);
            }
        } else {
#pragma unroll
          for (int f = 0; f < NF; ++f)
            if (f < nfv) {
#pragma unroll
              for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * jh + jj;
                const float cb =
                    fmaf(8.f, sc[j], grp ? bf16hi_to_f32(bpair[j]) : bf16lo_to_f32(bpair[j]));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  acc[f][j][i] =
                      fmaf(sc[j], P[f][jj][i], fmaf(cb, xc[f][i][2 + grp], acc[f][j][i]));
              }
            }
        }
      }
    }
  };

  // epilogue of the current item; `cs` is the LDS slot just consumed (free after a barrier)
  auto epilogue = [&](unsigned char* cs_bytes) __attribute__((always_inline)) {
    uint16_t* Cs = (uint16_t*)cs_bytes;
    lds_barrier();  // every wavefront is done reading the slot
    if (SWIGLU) {
      if (c_active) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (f < nfv) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float gte = acc[f][j][i], up = acc[f][j + 2][i];
                const float h = gte / (1.f + __expf(-gte)) * up;
                int col = 32 * wave + 16 * j + m;
                if (p.c_perm) col = (col & ~7) | perm8(col & 7);
                Cs[(16 * f + 4 * q + i) * LDC_SWIGLU + col] = to_bf16(h);
              }
          }
      }
      lds_barrier();
      const int F = N >> 1, col0 = c_slice * 128;
      for (int u = tid; u < BM * 16; u += 256) {
        const int r = u >> 4, ch = u & 15;
        if (r < c_nrows && col0 + 8 * ch < F)
          *(u32x4_t*)(p.C + (int64_t)(c_row0 + r) * p.ldc + col0 + 8 * ch) =
              *(const u32x4_t*)(Cs + r * LDC_SWIGLU + 8 * ch);
      }
      if (p.xc_out) {
        // (C0, X) of the two 64-column groups of this slice, from the rounded outputs
        const int r = tid >> 2, gg = (tid >> 1) & 1, half = tid & 1;
        float sum = 0.f;
        if (r < BM) {
          const u32x4_t* src = (const u32x4_t*)(Cs + r * LDC_SWIGLU + 64 * gg + 32 * half);
#pragma unroll
          for (int c = 0; c < 4; ++c) sum += sum8_bf16(src[c]);
        }
        sum += __shfl_xor(sum, 1);
        if (r < c_nrows && half == 0 && col0 + 64 * gg < F) {
          float* o = (float*)(p.xc_out + (int64_t)(c_row0 + r) * p.xc_out_ld + c_slice);
          o[gg] = -136.f * sum;
          o[2 + gg] = sum;
        }
      }
    } else {
      if (c_active) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (f < nfv) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                Cs[(16 * f + 4 * q + i) * LDC_PLAIN + 64 * wave + 16 * j + m] =
                    to_bf16(acc[f][j][i]);
          }
      }
      lds_barrier();
      const int col0 = c_slice * 256;
      for (int u = tid; u < BM * 32; u += 256) {
        const int r = u >> 5, ch = u & 31;
        if (r < c_nrows && col0 + 8 * ch < N)
          *(u32x4_t*)(p.C + (int64_t)(c_row0 + r) * p.ldc + col0 + 8 * ch) =
              *(const u32x4_t*)(Cs + r * LDC_PLAIN + 8 * ch);
      }
    }
  };

  // ---- prologue
  fetch_rows(0);
  wait_vmcnt<0>();
  for (int gs = 0; gs < RING - 1; ++gs)
    if (gs < total) produce(gs);
  begin_item(0);

  for (int gs = 0; gs < total; ++gs) {
    const int k = gs / nst, s = gs - k * nst;
    // this wavefront's loads of stage gs are done once only the later stages issued so
    // far (gs + 1 .. gs + RING - 2) may be outstanding
    if (gs + RING - 2 < total) wait_vmcnt<LY::DMA_PER_STAGE * (RING - 2)>();
    else wait_vmcnt<0>();
    lds_barrier();  // every wavefront's part of stage gs is in; slot (gs - 1) % RING is free
    if (gs + RING - 1 < total) produce(gs + RING - 1);
    if (c_active && nfv > 0) compute(gs);
    if (s + 1 == nst) {
      epilogue(smem + (gs % RING) * LY::SLOT);
      if (k + 1 < n_items) begin_item(k + 1);
    }
  }
}

}  // namespace

template <int NF, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void q4_stream_kernel(StreamParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lay<NF>::TOTAL];
  stream_body<NF, SWIGLU>(p, smem);
}

namespace {

// ---- prepared activations: permuted copy plus (-136 X, X) per row and stage
// One wavefront per row.  Lane l handles 16-byte chunks l, l + 64, ...; the eight
// chunks of a 64-wide group sit in eight consecutive lanes.
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ A, int rows,
                                                   int K, uint16_t* __restrict__ Ap,
                                                   float4* __restrict__ xc) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (r > rows) return;  // row `rows` is the zero row
  const int nch = K >> 3, KP = K / KS;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + l;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (c < nch && r < rows) v = *(const u32x4_t*)(A + (int64_t)r * K + 8 * c);
    float sum = sum8_bf16(v);
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    if (c < nch) {
      *(u32x4_t*)(Ap + (int64_t)r * K + 8 * c) = interleave8(v);
      if (xc && (c & 7) == 0) {
        const int g = c >> 3;  // 64-wide group
        float* o4 = (float*)(xc + (int64_t)r * KP + (g >> 1));
        o4[g & 1] = -136.f * sum;
        o4[2 + (g & 1)] = sum;
      }
    }
  }
}

}  // namespace

bool stream_supported(int N, int K, int a_rows) { return K % KS == 0 && N % 64 == 0 && a_rows >= 1; }

int stream_slices(int N, bool swiglu) { return swiglu ? ((N >> 1) + 127) / 128 : (N + 255) / 256; }

void launch_prep(const uint16_t* A, int rows, int K, uint16_t* Ap, float4* xc, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, dim3((rows + 1 + 3) / 4), dim3(256), 0, s, A, rows, K, Ap, xc);
}

void launch_stream(StreamParams p, bool swiglu, int nf, int64_t n_tiles_bound, int n_cu,
                   hipStream_t s) {
  p.n_slices = stream_slices(p.N, swiglu);
  const int64_t items = n_tiles_bound * p.n_slices;
  if (items <= 0) return;
  int64_t blocks = n_cu > 0 ? n_cu : 256;
  if (blocks > items + 7) blocks = items + 7;
  // every workgroup keeps its items' tiles in LDS: at most TABLE_CAP of them
  const int64_t per_xcd = (n_tiles_bound / 8 + 1) * p.n_slices;
  const int64_t min_slots = (per_xcd + TABLE_CAP - 1) / TABLE_CAP;
  if (blocks < 8 * min_slots) blocks = 8 * min_slots;
  blocks = (blocks + 7) / 8 * 8;
  dim3 grid((unsigned)blocks), block(256);
  if (nf == 4) {
    if (swiglu) hipLaunchKernelGGL((q4_stream_kernel<4, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((q4_stream_kernel<4, false>), grid, block, 0, s, p);
  } else {
    if (swiglu) hipLaunchKernelGGL((q4_stream_kernel<2, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((q4_stream_kernel<2, false>), grid, block, 0, s, p);
  }
}

}  // namespace moeq4
