// Grouped-query decode attention: one query token against a bf16 KV cache, every query
// head of one KV head served by the same workgroups, so each cached row is read once.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference engine for
// Qwen3.6-35B-A3B on Apple Silicon", body paragraph 4 (full-attention layers with
// grouped-query attention: 16 query heads, two KV heads, a growing KV cache) and
// paragraph 8 (decode reads the key and value cache with coalesced loads; several query
// heads share one workgroup so that each KV row loads once).  Readings (the pages state
// neither): head dim 128, scale 1 / sqrt(head dim), query head h on KV head h / group.
//
// Split over the cache (the decode query is one row, so the work is the cache read):
//   partial   about one workgroup per compute unit, each over a run of 128-position chunks of
//             one KV head.  A chunk's key and value rows (whole lines) go to LDS with
//             direct loads when the run is one chunk, else through registers, loaded while
//             the previous chunk is computed; the value rows are
//             transposed on the matrix cores (a product with identity slices, exact) into a
//             second LDS copy; the group's query rows sit in registers.  Scores S = Q K^T on the matrix cores (the group's heads are the
//             rows, padded to 16), the chunk's softmax numerators exp(s - m) with its max m
//             and sum l per head, then O = P V on the matrix cores with P split into two
//             bf16 pieces (hi + lo carries P to about 2^-17, so the product is close to fp32
//             accuracy).  The chunks of a run are combined with a running maximum per head;
//             the unnormalised O, m and l of each head go to the workspace.
//   reduce    one workgroup per (query head, 16 dims): M = max m, L = sum e^(m - M) l,
//             out = sum e^(m - M) O / L, slices of the partials merged in a fixed pattern
//             (deterministic).
#include "common.h"
#include "internal.h"
#include "q4_stream.h"

namespace moeq4 {

namespace {

constexpr int kD = kAttnHeadDim;        // head dim
constexpr int kC = 128;                 // cached positions per workgroup
constexpr int kWaves = 8;               // 8 x 16 positions (scores), 8 x 16 dims (P V)
constexpr int kVtRow = 2 * kC + 16;     // bytes per transposed value row (one dim), padded
constexpr int kPRow = kC + 8;           // bf16 per row of P, padded
static_assert(kWaves * 16 == kC && kWaves * 16 == kD, "one 16-wide tile per wavefront");

__device__ __forceinline__ float row16_max(float v) {
  // within each row of 16 lanes: quad swaps, then rotations by 4 and 8
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
  return v;
}

// 16-byte pieces of one chunk per lane: kPieces key and kPieces value pieces (1 KB per
// wavefront each)
constexpr int kPieces = (kC * 16 / 64) / kWaves;

// vmcnt(n) with the other counters at their maximum (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt fits the low field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8) | N);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Workgroup (x, g): chunks x * per_part .. of KV head g, two buffers.  With one chunk per
// workgroup (DIRECT) its key and value rows go straight to LDS (direct loads).  With more,
// every chunk is loaded into registers while the one before it is computed and stored to
// LDS at that chunk's end: the barriers inside the loop order LDS traffic only, so those
// loads stay in flight across them (direct loads would not: the compiler waits for every
// outstanding one before the first LDS read that follows, in every iteration, once the
// kernel has issued any).  The chunks are combined with
// a running maximum per head (O and the sum rescaled when it rises), so the workgroup
// writes one partial.
template <bool DIRECT>
__global__ __launch_bounds__(64 * kWaves, 1) void gqa_partial_kernel(AttnParams p) {
  // per buffer: key rows (permuted chunks) for the scores, then the transposed value rows;
  // the value rows
  __shared__ __attribute__((aligned(16))) unsigned char kv[2][kD * kVtRow];
  __shared__ __attribute__((aligned(16))) unsigned char vs[2][kC * 2 * kD];
  __shared__ __attribute__((aligned(16))) uint16_t ph[16 * kPRow];         // P, high bf16 piece
  __shared__ __attribute__((aligned(16))) uint16_t pl[16 * kPRow];         // P, low bf16 piece
  __shared__ float red_m[kWaves][16], red_l[kWaves][16];
  static_assert(kD * kVtRow >= kC * 2 * kD, "the key rows fit the transposed value area");
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int x = blockIdx.x, g = blockIdx.y, G = p.group;
  const int c_first = x * p.per_part;
  const int c_last = min(c_first + p.per_part, p.n_chunks);  // > c_first (host-checked)
  const uint16_t* kb = p.k + (int64_t)g * p.kv_stride * kD;
  const uint16_t* vb = p.v + (int64_t)g * p.kv_stride * kD;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

  // key and value rows of chunk c: piece j of this lane is 16-byte slot I * 64 + l of the
  // chunk's rows, I = wave + kWaves j (positions 4 I .. 4 I + 3), stored at LDS bytes
  // 1024 I + 16 l of the buffer; the 16-byte chunk ch of position r sits at slot
  // ch ^ (r % 16), so that the sixteen positions a matrix-core step reads fall in distinct
  // bank groups.  Positions past the cache read the last cached row (finite values; their
  // weights are zero).
  u32x4_t kr[kPieces], vr[kPieces];
  auto fetch = [&](int c) __attribute__((always_inline)) {
    const int pos0 = c * kC;
    const int npos = p.ctx - pos0 < kC ? p.ctx - pos0 : kC;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int I = wave + kWaves * j;
      const int Gc = I * 64 + l, r = Gc >> 4, slot = Gc & 15;
      const int64_t off = (int64_t)(pos0 + (r < npos ? r : npos - 1)) * kD + 8 * (slot ^ (r & 15));
      kr[j] = *(const u32x4_t*)(kb + off);
      vr[j] = *(const u32x4_t*)(vb + off);
    }
  };
  auto put_direct = [&](int c, int b) __attribute__((always_inline)) {
    const int pos0 = c * kC;
    const int npos = p.ctx - pos0 < kC ? p.ctx - pos0 : kC;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int I = wave + kWaves * j;
      const int Gc = I * 64 + l, r = Gc >> 4, slot = Gc & 15;
      const int64_t off = (int64_t)(pos0 + (r < npos ? r : npos - 1)) * kD + 8 * (slot ^ (r & 15));
      __builtin_amdgcn_global_load_lds(kb + off, kv[b] + 1024 * I, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vb + off, vs[b] + 1024 * I, 16, 0, 0);
    }
  };
  auto put = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int I = wave + kWaves * j;
      *(u32x4_t*)(kv[b] + 1024 * I + 16 * l) = kr[j];
      *(u32x4_t*)(vs[b] + 1024 * I + 16 * l) = vr[j];
    }
  };
  // the group's query rows as matrix-core A fragments: lane (head m, quarter q), dims
  // 32 s + 8 q .. + 7; heads past the group are zero rows
  u32x4_t qa[4];
  const int64_t h0 = (int64_t)g * G;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qa[s] = m < G ? *(const u32x4_t*)(p.q + (h0 + m) * kD + 32 * s + 8 * q) : zero4;
  if constexpr (DIRECT) {
    put_direct(c_first, 0);  // c_last == c_first + 1 (host-chosen)
    wait_vmcnt<0>();
  } else {
    fetch(c_first);
    put(0);
    if (c_first + 1 < c_last) fetch(c_first + 1);
  }

  // the value-transposing identity slices: with A = the wavefront's 16 positions x 32 dims
  // (lane (position m, quarter q) holds dims 32 s + 8 q .. + 7) and B = the 32 x 16 slice t
  // of an identity (one 1.0 per column, at k = 16 t + column), D = those 16 dims of the 16
  // positions, exactly; lane (dim j, quarter q) then holds positions 4 q .. 4 q + 3 of dim
  // 32 s + 16 t + j, four bf16 that go to V^T[dim][position] as one 8-byte store.
  u32x4_t eye[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kk = m + 16 * t - 8 * q;  // this lane's k-slot holding the 1.0, if any
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const uint32_t lo = (kk == 2 * w2) ? 0x3F80u : 0u, hi = (kk == 2 * w2 + 1) ? 0x3F80u : 0u;
      eye[t][w2] = lo | (hi << 16);
    }
  }

  // running maximum and sum of heads 4 q + i, and O of heads 4 q + i at dim 16 wave + m
  float run_m[4], run_l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    run_m[i] = -__builtin_inff();
    run_l[i] = 0.f;
  }
  f32x4_t O = zero;
  const int r = 16 * wave + m;
  const int dcol = 16 * wave + m;
  for (int c = c_first; c < c_last; ++c) {
    const int b = (c - c_first) & 1;
    // this chunk's rows are in buffer b (the next chunk's loads may still be in flight)
    lds_barrier();
    const int pos0 = c * kC;
    const int npos = p.ctx - pos0 < kC ? p.ctx - pos0 : kC;
    const unsigned char* kvb = kv[b];
    const unsigned char* vsb = vs[b];

    // scores of wavefront w: positions 16 w .. 16 w + 15 (B columns), the heads (A rows)
    f32x4_t S = zero;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4_t kf = *(const u32x4_t*)(kvb + r * 2 * kD + 16 * ((4 * s + q) ^ (r & 15)));
      S = mfma16x16x32(qa[s], kf, S);
    }
    f32x4_t vtr[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4_t vf = *(const u32x4_t*)(vsb + r * 2 * kD + 16 * ((4 * s + q) ^ (r & 15)));
#pragma unroll
      for (int t = 0; t < 2; ++t) vtr[s][t] = mfma16x16x32(vf, eye[t], zero);
    }
    // S[i]: head 4 q + i, position r.  Chunk max per head: over the 16 lanes of the row,
    // then over the wavefronts through LDS.
    const bool valid = r < npos;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = valid ? S[i] * p.scale : -__builtin_inff();
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = row16_max(sv[i]);
    if (m == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red_m[wave][4 * q + i] = mx[i];
    }
    lds_barrier();  // also: every wavefront is past its key reads
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int dim = 32 * s + 16 * t + m;
        const uint32_t w0 = pack_bf16x2(vtr[s][t][0], vtr[s][t][1]);
        const uint32_t w1 = pack_bf16x2(vtr[s][t][2], vtr[s][t][3]);
        *(u32x2_t*)(kv[b] + dim * kVtRow + 2 * (16 * wave + 4 * q)) = u32x2_t{w0, w1};
      }
    // the new running maximum of each head; O and the sum scaled to it
    float e[4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = red_m[0][4 * q + i];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v = fmaxf(v, red_m[w][4 * q + i]);
      const float nm = fmaxf(run_m[i], v);  // finite: every chunk has a valid position
      alpha[i] = __expf(run_m[i] - nm);     // 0 on the first chunk
      run_m[i] = nm;
      e[i] = valid ? __expf(sv[i] - nm) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sum = row16_sum(e[i]);
      if (m == 0) red_l[wave][4 * q + i] = sum;
      const uint16_t hi = to_bf16(e[i]);
      const uint16_t lo = to_bf16(e[i] - bf16lo_to_f32(hi));
      ph[(4 * q + i) * kPRow + r] = hi;
      pl[(4 * q + i) * kPRow + r] = lo;
    }
    lds_barrier();
    // O = alpha O + P V: wavefront w takes dims 16 w .. 16 w + 15 (B columns), the heads A rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      O[i] *= alpha[i];
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) lsum += red_l[w][4 * q + i];
      run_l[i] = run_l[i] * alpha[i] + lsum;
    }
#pragma unroll
    for (int s = 0; s < kC / 32; ++s) {
      const int pp = 32 * s + 8 * q;  // positions of this lane's k-slots
      const u32x4_t ah = *(const u32x4_t*)(ph + m * kPRow + pp);
      const u32x4_t al = *(const u32x4_t*)(pl + m * kPRow + pp);
      const u32x4_t bv = *(const u32x4_t*)(kv[b] + dcol * kVtRow + 2 * pp);
      O = mfma16x16x32(al, bv, mfma16x16x32(ah, bv, O));
    }
    // the next chunk to buffer b ^ 1 (last read in the previous chunk, before this chunk's
    // first barrier), then the loads of the one after it
    if (!DIRECT && c + 1 < c_last) put(b ^ 1);
    if (!DIRECT && c + 2 < c_last) fetch(c + 2);
    // every wavefront is done with buffer b, P and the per-wavefront maxima and sums
    lds_barrier();
  }
  // O[i]: head 4 q + i, dim dcol
  const int64_t base = ((int64_t)g * p.n_part + x) * G;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q + i;
    if (h < G) p.part_o[(base + h) * kD + dcol] = O[i];
  }
  if (wave == 0 && m == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * q + i;
      if (h < G) {
        p.part_ml[(base + h) * 2] = run_m[i];
        p.part_ml[(base + h) * 2 + 1] = run_l[i];
      }
    }
  }
}

// One workgroup per (query head, 16 dims): 256 threads = 16 slices x 16 dims.  Slice s
// takes partials s, s + 16, ... in one pass (every load issued before any is used), with
// its own maximum M_s: acc_s = sum e^(m - M_s) O, L_s = sum e^(m - M_s) l.  Slices then
// merge pairwise, (M, acc, L) = (max, e^(Ma - M) acc_a + e^(Mb - M) acc_b, ...), which is
// symmetric in its two arguments, so both lanes of a pair get the same bits: the four
// slices of a wavefront (its rows of 16 lanes) through the lane swaps, the four
// wavefronts through LDS in a fixed order.
constexpr int kRedDims = 16;
constexpr int kRedSlices = 16;
constexpr int kRedUnroll = 8;
struct Part {
  float m, acc, l;
};
__device__ __forceinline__ Part merge_part(Part a, Part b) {
  const float M = fmaxf(a.m, b.m);
  const float wa = a.m == -__builtin_inff() ? 0.f : __expf(a.m - M);
  const float wb = b.m == -__builtin_inff() ? 0.f : __expf(b.m - M);
  return Part{M, wa * a.acc + wb * b.acc, wa * a.l + wb * b.l};
}
__global__ __launch_bounds__(kRedSlices * kRedDims) void gqa_reduce_kernel(AttnParams p) {
  __shared__ Part wpart[4][kRedDims];
  const int tid = threadIdx.x, h = blockIdx.x, G = p.group;
  const int g = h / G, hg = h - g * G;
  const int dd = tid & (kRedDims - 1), sl = tid / kRedDims;
  const int d = kRedDims * blockIdx.y + dd;
  const int np = p.n_part;
  const float* mlp = p.part_ml + ((int64_t)g * np * G + hg) * 2;     // partial c at + c G 2
  const float* op = p.part_o + ((int64_t)g * np * G + hg) * kD + d;  // partial c at + c G kD
  Part s{-__builtin_inff(), 0.f, 0.f};
  for (int c0 = sl; c0 < np; c0 += kRedSlices * kRedUnroll) {
    float mv[kRedUnroll], lv[kRedUnroll], ov[kRedUnroll];
#pragma unroll
    for (int u = 0; u < kRedUnroll; ++u) {
      const int c = c0 + kRedSlices * u;
      const int64_t cc = c < np ? c : c0;
      mv[u] = mlp[cc * G * 2];
      lv[u] = mlp[cc * G * 2 + 1];
      ov[u] = op[cc * G * kD];
    }
    float M = s.m;
#pragma unroll
    for (int u = 0; u < kRedUnroll; ++u)
      if (c0 + kRedSlices * u < np) M = fmaxf(M, mv[u]);
    const float r = s.m == -__builtin_inff() ? 0.f : __expf(s.m - M);
    float acc = s.acc * r, L = s.l * r;
#pragma unroll
    for (int u = 0; u < kRedUnroll; ++u)
      if (c0 + kRedSlices * u < np) {
        const float w = __expf(mv[u] - M);
        L = fmaf(w, lv[u], L);
        acc = fmaf(w, ov[u], acc);
      }
    s = Part{M, acc, L};
  }
  // the four slices of this wavefront: rows r and r ^ 1, then the halves
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    const uint32_t a0 = __float_as_uint(s.m), a1 = __float_as_uint(s.acc), a2 = __float_as_uint(s.l);
    Part o;
    if (step == 0) {
      const auto x0 = __builtin_amdgcn_permlane16_swap(a0, a0, false, false);
      const auto x1 = __builtin_amdgcn_permlane16_swap(a1, a1, false, false);
      const auto x2 = __builtin_amdgcn_permlane16_swap(a2, a2, false, false);
      s = Part{__uint_as_float(x0[0]), __uint_as_float(x1[0]), __uint_as_float(x2[0])};
      o = Part{__uint_as_float(x0[1]), __uint_as_float(x1[1]), __uint_as_float(x2[1])};
    } else {
      const auto x0 = __builtin_amdgcn_permlane32_swap(a0, a0, false, false);
      const auto x1 = __builtin_amdgcn_permlane32_swap(a1, a1, false, false);
      const auto x2 = __builtin_amdgcn_permlane32_swap(a2, a2, false, false);
      s = Part{__uint_as_float(x0[0]), __uint_as_float(x1[0]), __uint_as_float(x2[0])};
      o = Part{__uint_as_float(x0[1]), __uint_as_float(x1[1]), __uint_as_float(x2[1])};
    }
    s = merge_part(s, o);
  }
  const int w = tid >> 6;
  if ((tid & 63) < kRedDims) wpart[w][dd] = s;
  __syncthreads();
  if (tid < kRedDims) {
    const Part t = merge_part(merge_part(wpart[0][dd], wpart[1][dd]),
                              merge_part(wpart[2][dd], wpart[3][dd]));
    p.out[(int64_t)h * kD + d] = to_bf16(t.acc / t.l);
  }
}

}  // namespace

bool attn_supported(int n_q, int n_kv, int head_dim, int ctx, int64_t kv_stride) {
  return head_dim == kD && n_kv >= 1 && n_q >= n_kv && n_q % n_kv == 0 && n_q / n_kv <= 16 &&
         ctx >= 1 && kv_stride >= ctx;
}

int attn_chunks(int ctx) { return (ctx + kC - 1) / kC; }

size_t attn_workspace_bytes(int n_q, int n_kv, int ctx) {
  const size_t nch = (size_t)attn_chunks(ctx), G = (size_t)(n_q / n_kv);
  return (size_t)n_kv * nch * G * (kD + 2) * sizeof(float) + 256;
}

void attn_partition(AttnParams* p, int n_cu) {
  // about one workgroup per compute unit over all KV heads, each taking a run of chunks
  const int per_head = max(1, (n_cu > 0 ? n_cu : 256) / p->n_kv);
  p->per_part = (p->n_chunks + per_head - 1) / per_head;
  p->n_part = (p->n_chunks + p->per_part - 1) / p->per_part;
}

void launch_attention(const AttnParams& p, hipStream_t s) {
  if (p.per_part == 1)
    hipLaunchKernelGGL(gqa_partial_kernel<true>, dim3(p.n_part, p.n_kv), dim3(64 * kWaves), 0, s, p);
  else
    hipLaunchKernelGGL(gqa_partial_kernel<false>, dim3(p.n_part, p.n_kv), dim3(64 * kWaves), 0, s, p);
  hipLaunchKernelGGL(gqa_reduce_kernel, dim3(p.n_q, kD / kRedDims), dim3(kRedSlices * kRedDims), 0,
                     s, p);
}

}  // namespace moeq4
