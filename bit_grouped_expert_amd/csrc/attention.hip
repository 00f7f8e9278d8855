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
//   partial   one workgroup per (KV head, 128 cached positions).  The positions' key and
//             value rows go to LDS with direct 1 KB loads (whole lines); the value rows are
//             transposed on the matrix cores (a product with identity slices, exact) into a
//             second LDS copy; the group's query rows sit in registers.  Scores S = Q K^T on the matrix cores (the group's heads are the
//             rows, padded to 16), the chunk's softmax numerators exp(s - m) with its max m
//             and sum l per head, then O = P V on the matrix cores with P split into two
//             bf16 pieces (hi + lo carries P to about 2^-17, so the product is close to fp32
//             accuracy).  The unnormalised O, m and l of each head go to the workspace.
//   reduce    one workgroup per (query head, 16 dims): M = max m, L = sum e^(m - M) l,
//             out = sum e^(m - M) O / L over the chunks in a fixed order (deterministic).
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

__global__ __launch_bounds__(64 * kWaves) void gqa_partial_kernel(AttnParams p) {
  // kv: key rows (permuted chunks) for the scores, then the transposed value rows
  __shared__ __attribute__((aligned(16))) unsigned char kv[kD * kVtRow];
  __shared__ __attribute__((aligned(16))) unsigned char vs[kC * 2 * kD];   // value rows, permuted
  __shared__ __attribute__((aligned(16))) uint16_t ph[16 * kPRow];         // P, high bf16 piece
  __shared__ __attribute__((aligned(16))) uint16_t pl[16 * kPRow];         // P, low bf16 piece
  __shared__ float red_m[kWaves][16], red_l[kWaves][16];
  static_assert(kD * kVtRow >= kC * 2 * kD, "the key rows fit the transposed value area");
  const int tid = threadIdx.x, l = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = l & 15, q = l >> 4;
  const int c = blockIdx.x, g = blockIdx.y, G = p.group;
  const int pos0 = c * kC;
  const int npos = p.ctx - pos0 < kC ? p.ctx - pos0 : kC;  // >= 1
  const uint16_t* kb = p.k + (int64_t)g * p.kv_stride * kD;
  const uint16_t* vb = p.v + (int64_t)g * p.kv_stride * kD;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

  // key and value rows: load I fills LDS bytes 1024 I .. (positions 4 I .. 4 I + 3); the
  // 16-byte chunk ch of position r sits at slot ch ^ (r % 16), so that the sixteen positions
  // a matrix-core step reads fall in distinct bank groups.  Positions past the cache read the
  // last cached row (finite values; their weights are zero).
  for (int I = wave; I < kC * 16 / 64; I += kWaves) {
    const int Gc = I * 64 + l, r = Gc >> 4, slot = Gc & 15;
    const int64_t off = (int64_t)(pos0 + (r < npos ? r : npos - 1)) * kD + 8 * (slot ^ (r & 15));
    __builtin_amdgcn_global_load_lds(kb + off, kv + 1024 * I, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + off, vs + 1024 * I, 16, 0, 0);
  }
  // the group's query rows as matrix-core A fragments: lane (head m, quarter q), dims
  // 32 s + 8 q .. + 7; heads past the group are zero rows
  u32x4_t qa[4];
  const int64_t h0 = (int64_t)g * G;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qa[s] = m < G ? *(const u32x4_t*)(p.q + (h0 + m) * kD + 32 * s + 8 * q) : zero4;
  wait_vmcnt0();
  __syncthreads();

  // scores of wavefront w: positions 16 w .. 16 w + 15 (B columns), the group's heads (A rows)
  f32x4_t S = zero;
  const int r = 16 * wave + m;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4_t kf = *(const u32x4_t*)(kv + r * 2 * kD + 16 * ((4 * s + q) ^ (r & 15)));
    S = mfma16x16x32(qa[s], kf, S);
  }
  // the value rows transposed on the matrix cores: with A = the wavefront's 16 positions x 32
  // dims (lane (position m, quarter q) holds dims 32 s + 8 q .. + 7) and B = the 32 x 16 slice
  // t of an identity (one 1.0 per column, at k = 16 t + column), D = those 16 dims of the 16
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
  f32x4_t vtr[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4_t vf = *(const u32x4_t*)(vs + r * 2 * kD + 16 * ((4 * s + q) ^ (r & 15)));
#pragma unroll
    for (int t = 0; t < 2; ++t) vtr[s][t] = mfma16x16x32(vf, eye[t], zero);
  }
  // S[i]: head 4 q + i, position r.  Chunk max per head: over the 16 lanes of the row, then
  // over the wavefronts through LDS.
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
  __syncthreads();  // also: every wavefront is past its key reads
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int dim = 32 * s + 16 * t + m;
      const uint32_t w0 = pack_bf16x2(vtr[s][t][0], vtr[s][t][1]);
      const uint32_t w1 = pack_bf16x2(vtr[s][t][2], vtr[s][t][3]);
      *(u32x2_t*)(kv + dim * kVtRow + 2 * (16 * wave + 4 * q)) = u32x2_t{w0, w1};
    }
  float e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = red_m[0][4 * q + i];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v = fmaxf(v, red_m[w][4 * q + i]);
    e[i] = valid ? __expf(sv[i] - v) : 0.f;
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
  __syncthreads();

  // O = P V: wavefront w takes dims 16 w .. 16 w + 15 (B columns), the heads are A rows
  f32x4_t O = zero;
  const int dcol = 16 * wave + m;
#pragma unroll
  for (int s = 0; s < kC / 32; ++s) {
    const int pp = 32 * s + 8 * q;  // positions of this lane's k-slots
    const u32x4_t ah = *(const u32x4_t*)(ph + m * kPRow + pp);
    const u32x4_t al = *(const u32x4_t*)(pl + m * kPRow + pp);
    const u32x4_t bv = *(const u32x4_t*)(kv + dcol * kVtRow + 2 * pp);
    O = mfma16x16x32(al, bv, mfma16x16x32(ah, bv, O));
  }
  // O[i]: head 4 q + i, dim dcol
  const int64_t base = ((int64_t)g * p.n_chunks + c) * G;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q + i;
    if (h < G) p.part_o[(base + h) * kD + dcol] = O[i];
  }
  if (tid < G) {
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) lsum += red_l[w][tid];
    float mm = red_m[0][tid];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, red_m[w][tid]);
    p.part_ml[(base + tid) * 2] = mm;
    p.part_ml[(base + tid) * 2 + 1] = lsum;
  }
}

// one workgroup per (query head, 16 dims): 1024 threads = 64 slices of the chunks (slice s
// takes chunks s, s + 64, ...) x 16 dims.  The maximum over the chunks first, then each
// thread sums its slice four chunks at a time with every load of the four issued before any
// is used; the slices meet in LDS in slice order.
constexpr int kRedDims = 16;
constexpr int kRedSlices = 64;
__global__ __launch_bounds__(kRedSlices * kRedDims) void gqa_reduce_kernel(AttnParams p) {
  __shared__ float red[kRedSlices * kRedDims];
  __shared__ float accs[kRedSlices][kRedDims];
  __shared__ float ls[kRedSlices];
  const int tid = threadIdx.x, h = blockIdx.x, G = p.group;
  const int g = h / G, hg = h - g * G;
  const int dd = tid & (kRedDims - 1), sl = tid / kRedDims;
  const int d = kRedDims * blockIdx.y + dd;
  const int nch = p.n_chunks;
  const float* mlp = p.part_ml + ((int64_t)g * nch * G + hg) * 2;     // chunk c at + c G 2
  const float* op = p.part_o + ((int64_t)g * nch * G + hg) * kD + d;  // chunk c at + c G kD
  float mx = -__builtin_inff();
  for (int c = tid; c < nch; c += kRedSlices * kRedDims) mx = fmaxf(mx, mlp[(int64_t)c * G * 2]);
  red[tid] = mx;
  __syncthreads();
  for (int st = kRedSlices * kRedDims / 2; st > 0; st >>= 1) {
    if (tid < st) red[tid] = fmaxf(red[tid], red[tid + st]);
    __syncthreads();
  }
  const float M = red[0];
  float L = 0.f, acc = 0.f;
  int c = sl;
  for (; c + kRedSlices * 3 < nch; c += kRedSlices * 4) {
    float mv[4], lv[4], ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t cc = c + kRedSlices * u;
      mv[u] = mlp[cc * G * 2];
      lv[u] = mlp[cc * G * 2 + 1];
      ov[u] = op[cc * G * kD];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = __expf(mv[u] - M);
      L = fmaf(w, lv[u], L);
      acc = fmaf(w, ov[u], acc);
    }
  }
  for (; c < nch; c += kRedSlices) {
    const float w = __expf(mlp[(int64_t)c * G * 2] - M);
    L = fmaf(w, mlp[(int64_t)c * G * 2 + 1], L);
    acc = fmaf(w, op[(int64_t)c * G * kD], acc);
  }
  accs[sl][dd] = acc;
  if (dd == 0) ls[sl] = L;
  __syncthreads();
  if (sl == 0) {
    float a = 0.f, lt = 0.f;
    for (int u = 0; u < kRedSlices; ++u) {
      a += accs[u][dd];
      lt += ls[u];
    }
    p.out[(int64_t)h * kD + d] = to_bf16(a / lt);
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

void launch_attention(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL(gqa_partial_kernel, dim3(p.n_chunks, p.n_kv), dim3(64 * kWaves), 0, s, p);
  hipLaunchKernelGGL(gqa_reduce_kernel, dim3(p.n_q, kD / kRedDims), dim3(kRedSlices * kRedDims), 0,
                     s, p);
}

}  // namespace moeq4
