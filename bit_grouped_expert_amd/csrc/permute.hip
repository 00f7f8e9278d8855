// Histogram, prefix scan and stable scatter of routed (token, slot) pairs into
// contiguous per-expert groups, plus the tile map of the grouped GEMM.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
// engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraph 4 (routing gives
// uneven expert groups) and paragraph 6 (the routing histogram, prefix scan,
// scatter and block map stay on the GPU, with no CPU synchronisation inside the
// MoE layer).  Everything here is integer work sized from host-known bounds; the
// host never reads a count back.
//
// Stability: rows of an expert hold its tokens in ascending token order.  Tokens
// are cut into chunks of 256; a chunk's base row for expert e is offsets[e] plus
// the number of earlier-chunk pairs routed to e (column scan of per-chunk
// counts); inside a chunk each wavefront of 64 tokens sets one bit per token in a
// 64-bit mask per expert, and a token's rank is the popcount of the masks of the
// lower waves plus the bits of lower lanes in its own wave.
#include "common.h"
#include "internal.h"

namespace moeq4 {

// The k (<= 16) expert ids of token t, all loaded before any is used: one independent
// load per slot, so that they are in flight together (a load followed by its use in a
// loop is otherwise waited for one slot at a time).
__device__ __forceinline__ void load_slots(const int32_t* __restrict__ idx, int t, int k,
                                           int32_t (&e)[kMaxTopK]) {
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) e[j] = j < k ? idx[(int64_t)t * k + j] : -1;
}

// ---------------------------------------------------------------------------- count
__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                    int E, int32_t* __restrict__ chunk_cnt) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kChunkTokens + threadIdx.x;
  if (t < T) {
    int32_t ev[kMaxTopK];
    load_slots(idx, t, k, ev);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const int e = ev[j];
      if (j < k && e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_cnt[(int64_t)blockIdx.x * E + e] = hist[e];
}

void launch_count(const int32_t* idx, int T, int k, int E, int32_t* chunk_cnt, hipStream_t s) {
  hipLaunchKernelGGL(count_kernel, dim3(n_chunks(T)), dim3(256), E * sizeof(int32_t), s, idx, T, k,
                     E, chunk_cnt);
}

// ---------------------------------------------------------------------------- block scan
// Exclusive scan of one int per thread over a 1024-thread block; returns the
// exclusive prefix and writes the block total to *total.
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    int sv = wsum[w];
    if (w < wave) base += sv;
    tot += sv;
  }
  __syncthreads();  // wsum may be reused by the next call
  *total = tot;
  return base + incl - v;
}

__device__ void write_tiles(const int32_t* offs, int n_groups, int rows_total, int bm,
                            int4* __restrict__ tiles, int cap, int32_t* __restrict__ tile_count,
                            int* tab);

// ---------------------------------------------------------------------------- scan
// One workgroup of 1024 threads.  chunk_cnt [nchunks, E] is replaced by each
// chunk's exclusive base per expert; offsets[0..E] is the exclusive scan of the
// expert totals; if shared_rows >= 0, offsets[E+1] = offsets[E] + shared_rows.
// With tiles set, the same workgroup then writes the tile map of the E routed groups
// (and the shared one when shared_rows >= 0) from the offsets it holds, as
// build_tiles_kernel would from the written ones.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ chunk_cnt, int nchunks,
                                                    int E, int32_t* __restrict__ offsets,
                                                    int shared_rows, int rows_total, int bm,
                                                    int4* __restrict__ tiles, int cap,
                                                    int32_t* __restrict__ tile_count) {
  __shared__ int soff[kMaxTileGroups + 1];
  __shared__ int tab[3 * (kMaxTileGroups + 1)];
  const int e = threadIdx.x;
  int running = 0;
  if (e < E) {
    int c = 0;
    for (; c + 8 <= nchunks; c += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = chunk_cnt[(int64_t)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        chunk_cnt[(int64_t)(c + i) * E + e] = running;
        running += v[i];
      }
    }
    for (; c < nchunks; ++c) {
      int v = chunk_cnt[(int64_t)c * E + e];
      chunk_cnt[(int64_t)c * E + e] = running;
      running += v;
    }
  }
  int total;
  const int excl = block_exclusive_scan_1024(e < E ? running : 0, &total);
  if (e < E) offsets[e] = excl;
  if (threadIdx.x == 0) {
    offsets[E] = total;
    if (shared_rows >= 0) offsets[E + 1] = total + shared_rows;
  }
  if (tiles) {  // uniform: a kernel argument
    if (e < E) soff[e] = excl;
    if (threadIdx.x == 0) {
      soff[E] = total;
      if (shared_rows >= 0) soff[E + 1] = total + shared_rows;
    }
    // write_tiles starts with a barrier, after which soff is complete
    write_tiles(soff, shared_rows >= 0 ? E + 1 : E, rows_total, bm, tiles, cap, tile_count, tab);
  }
}

void launch_scan(int32_t* chunk_cnt, int nchunks, int E, int32_t* offsets, int shared_rows,
                 hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, chunk_cnt, nchunks, E, offsets,
                     shared_rows, 0, 1, nullptr, 0, nullptr);
}

void launch_scan_tiles(int32_t* chunk_cnt, int nchunks, int E, int32_t* offsets, int shared_rows,
                       int rows_total, int bm, int4* tiles, int32_t* tile_count, hipStream_t s) {
  const int n_groups = shared_rows >= 0 ? E + 1 : E;
  const int cap = (int)max_tiles(rows_total, n_groups, bm);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, chunk_cnt, nchunks, E, offsets,
                     shared_rows, rows_total, bm, tiles, cap, tile_count);
}

// ---------------------------------------------------------------------------- scatter
__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_tok,
    int32_t* __restrict__ slot_row, int shared_base) {
  extern __shared__ unsigned long long masks[];  // [4 waves][E]
  for (int i = threadIdx.x; i < 4 * E; i += 256) masks[i] = 0ull;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kChunkTokens + threadIdx.x;
  const unsigned long long bit = 1ull << lane;
  int32_t ev[kMaxTopK];
  if (t < T) {
    load_slots(idx, t, k, ev);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const int e = ev[j];
      if (j < k && e >= 0 && e < E) atomicOr(&masks[wave * E + e], bit);
    }
  }
  __syncthreads();
  if (t < T) {
    const int32_t* base = chunk_base + (int64_t)blockIdx.x * E;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      const int e = ev[j];
      int32_t row = -1;
      if (e >= 0 && e < E) {
        int rank = __popcll(masks[wave * E + e] & (bit - 1ull));
        for (int w = 0; w < wave; ++w) rank += __popcll(masks[w * E + e]);
        row = offsets[e] + base[e] + rank;
        if (row >= 0 && row < T * k) sorted_tok[row] = t;  // always true for consistent counts
        else row = -1;
      }
      slot_row[(int64_t)t * k + j] = row;
    }
    if (shared_base >= 0) sorted_tok[shared_base + t] = t;
  }
}

void launch_scatter(const int32_t* idx, int T, int k, int E, const int32_t* chunk_base,
                    const int32_t* offsets, int32_t* sorted_tok, int32_t* slot_row, int shared_base,
                    hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(n_chunks(T)), dim3(256),
                     4 * E * sizeof(unsigned long long), s, idx, T, k, E, chunk_base, offsets,
                     sorted_tok, slot_row, shared_base);
}

// ---------------------------------------------------------------------------- tile map
// Tiles of at most `bm` rows over every group, group by group, as (group, first row,
// rows, 0).  Offsets are clamped into [0, rows_total] so that no tile leaves C, and at
// most `cap` tiles are written (cap = the bound the grid was sized with), so malformed
// offsets cannot overrun the tile array.  Every thread of a 1024-thread workgroup
// calls it; `tab` is LDS scratch of at least 3 * (n_groups + 1) ints.  A scan gives
// each group its first tile, then tile t is written by thread t % 1024, which finds its
// group by binary search over the first tiles (consecutive threads write consecutive
// tiles).
__device__ void write_tiles(const int32_t* offs, int n_groups, int rows_total, int bm,
                            int4* __restrict__ tiles, int cap, int32_t* __restrict__ tile_count,
                            int* tab) {
  int* first = tab;                   // [n_groups + 1]
  int* glo = tab + n_groups + 1;      // [n_groups]
  int* ghi = glo + n_groups;          // [n_groups]
  __syncthreads();  // the caller may have used the scratch
  int running = 0;
  for (int g0 = 0; g0 < n_groups; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    int lo = 0, hi = 0;
    if (g < n_groups) {
      lo = min(max(offs[g], 0), rows_total);
      hi = min(max(offs[g + 1], lo), rows_total);
    }
    const int nt = (hi - lo + bm - 1) / bm;
    int total;
    const int f = running + block_exclusive_scan_1024(nt, &total);
    if (g < n_groups) {
      first[g] = f;
      glo[g] = lo;
      ghi[g] = hi;
    }
    running += total;
  }
  if (threadIdx.x == 0) first[n_groups] = running;
  __syncthreads();
  const int ntot = min(running, cap);
  for (int t = threadIdx.x; t < ntot; t += 1024) {
    // the last group whose first tile is <= t (empty groups share their successor's)
    int a = 0, b = n_groups - 1;
    while (a < b) {
      const int mid = (a + b + 1) >> 1;
      if (first[mid] <= t) a = mid;
      else b = mid - 1;
    }
    const int r0 = glo[a] + (t - first[a]) * bm;
    tiles[t] = make_int4(a, r0, min(bm, ghi[a] - r0), 0);
  }
  if (threadIdx.x == 0) *tile_count = ntot;
}

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int n_groups, int rows_total, int bm,
                                                           int4* __restrict__ tiles, int cap,
                                                           int32_t* __restrict__ tile_count) {
  __shared__ int tab[3 * (kMaxTileGroups + 1)];
  write_tiles(offsets, n_groups, rows_total, bm, tiles, cap, tile_count, tab);
}

void launch_build_tiles(const int32_t* offsets, int n_groups, int rows_total, int bm, int4* tiles,
                        int32_t* tile_count, hipStream_t s) {
  const int cap = (int)max_tiles(rows_total, n_groups, bm);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, offsets, n_groups, rows_total,
                     bm, tiles, cap, tile_count);
}

// ---------------------------------------------------------------------------- fused (T <= 1024)
constexpr size_t small_lds(int E) {
  return 16 * (size_t)E * 8 + 16 * (size_t)E * 4 + (size_t)(E + 2) * 4;
}
constexpr int kSmallMaxE = 768;  // above, the chunked kernels run
static_assert(small_lds(kSmallMaxE) + 64 <= 160 * 1024, "LDS budget");

// One workgroup of 1024 threads, thread t = token t: the histogram, the scan, the
// stable scatter and the tile map of a small batch in one launch.  Same ranking as
// the chunked kernels above: a token's rank among the tokens of expert e is the
// popcount of the lower waves' bit masks for e plus the bits of lower lanes in its
// own wave.  With shared_rows >= 0 the shared group's rows follow at T * k.
__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_tok, int32_t* __restrict__ slot_row, int shared_rows, int bm,
    int4* __restrict__ tiles, int cap, int32_t* __restrict__ tile_count) {
  // [16 waves][E] masks, then [16 waves][E] base rows (offset of the expert plus the
  // tokens of the lower waves), then offs[E + 2]
  __shared__ unsigned long long masks[small_lds(kSmallMaxE) / 8];  // sized for the largest E
  int32_t* base = (int32_t*)(masks + 16 * E);
  int32_t* offs = base + 16 * E;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 16 * E; i += 1024) masks[i] = 0ull;
  __syncthreads();
  const unsigned long long bit = 1ull << lane;
  int32_t ev[kMaxTopK];
  if (tid < T) {
    load_slots(idx, tid, k, ev);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const int e = ev[j];
      if (j < k && e >= 0 && e < E) atomicOr(&masks[wave * E + e], bit);
    }
  }
  __syncthreads();
  int cnt = 0;
  int pre[16];
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    pre[w] = cnt;
    if (tid < E) cnt += __popcll(masks[w * E + tid]);
  }
  int total;
  const int excl = block_exclusive_scan_1024(cnt, &total);
  if (tid < E) {
    offs[tid] = excl;
    offsets[tid] = excl;
#pragma unroll
    for (int w = 0; w < 16; ++w) base[w * E + tid] = excl + pre[w];
  }
  if (tid == 0) {
    offs[E] = total;
    offsets[E] = total;
    if (shared_rows >= 0) {
      offs[E + 1] = total + shared_rows;
      offsets[E + 1] = total + shared_rows;
    }
  }
  __syncthreads();
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      const int e = ev[j];
      int32_t row = -1;
      if (e >= 0 && e < E) {
        row = base[wave * E + e] + __popcll(masks[wave * E + e] & (bit - 1ull));
        if (row >= 0 && row < T * k) sorted_tok[row] = tid;  // always true for consistent counts
        else row = -1;
      }
      slot_row[(int64_t)tid * k + j] = row;
    }
    if (shared_rows >= 0) sorted_tok[T * k + tid] = tid;
  }
  const int n_groups = E + (shared_rows >= 0 ? 1 : 0);
  const int rows_total = T * k + (shared_rows >= 0 ? shared_rows : 0);
  // the masks are no longer needed: their space (16 E words) holds the tile scratch
  write_tiles(offs, n_groups, rows_total, bm, tiles, cap, tile_count, (int*)masks);
}


bool permute_small_ok(int T, int E) { return T >= 1 && T <= 1024 && E <= kSmallMaxE; }

void launch_permute_small(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_tok, int32_t* slot_row, int shared_rows, int bm,
                          int4* tiles, int32_t* tile_count, hipStream_t s) {
  const int n_groups = E + (shared_rows >= 0 ? 1 : 0);
  const int rows_total = T * k + (shared_rows >= 0 ? shared_rows : 0);
  const int cap = (int)max_tiles(rows_total, n_groups, bm);
  hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, s, idx, T, k, E, offsets,
                     sorted_tok, slot_row, shared_rows, bm, tiles, cap, tile_count);
}

// ---------------------------------------------------------------------------- expert-parallel
// Few routed pairs (T * k <= 8192): one workgroup of 256 threads per four experts, all
// independent.  Every workgroup loads all T * k expert ids (thread i holds the contiguous
// run of pairs i * per .. i * per + per - 1, so pair order is thread order) and histograms
// them in LDS; one packed scan of (rows, tiles) per group then gives every group's offset
// and first tile.  A workgroup places only the pairs of its own four experts: a packed
// scan of the per-thread counts of those experts (16 bits each) gives each thread the
// number of earlier pairs of each, so rows of an expert hold its tokens in ascending
// token order.  It also writes its experts' tiles; workgroup 0 writes the offsets, the
// tile count and slot_row = -1 for ids outside [0, E); the last workgroup writes the
// shared group's identity rows and tiles.  The results equal those of the kernels above.
constexpr int kEpThreads = 256;
constexpr int kEpPer = 32;      // pairs per thread
constexpr int kEpExperts = 4;   // experts per workgroup
constexpr int kEpMaxE = 1024;

// Inclusive scan over the wavefront with DPP row shifts (within rows of 16 lanes), then
// the row broadcasts of lanes 15 and 31.  Lanes a step does not update add 0.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive scan of one uint64 per thread over a 256-thread block, as two independent
// 32-bit scans of its halves (callers keep every 16- or 32-bit field below its width, so
// no carry crosses them).  *total = the block's sum.  Every thread must call it.
__device__ uint64_t block_exclusive_scan_u64_256(uint64_t v, uint64_t* total) {
  __shared__ uint32_t wsum[2 * (kEpThreads / 64)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t ilo = wave_incl_scan_u32(lo), ihi = wave_incl_scan_u32(hi);
  if (lane == 63) {
    wsum[wave] = ilo;
    wsum[kEpThreads / 64 + wave] = ihi;
  }
  __syncthreads();
  uint32_t blo = 0, bhi = 0, tlo = 0, thi = 0;
#pragma unroll
  for (int w = 0; w < kEpThreads / 64; ++w) {
    const uint32_t sl = wsum[w], sh = wsum[kEpThreads / 64 + w];
    if (w < wave) {
      blo += sl;
      bhi += sh;
    }
    tlo += sl;
    thi += sh;
  }
  __syncthreads();  // wsum may be reused by the next call
  *total = ((uint64_t)thi << 32) | tlo;
  return ((uint64_t)(bhi + ihi - hi) << 32) | (uint64_t)(blo + ilo - lo);
}

// PER: pairs per thread, a power of two with 256 * PER >= T * k (fixed at compile time,
// so that the per-pair loops carry no uniform branches)
template <int PER>
__global__ __launch_bounds__(kEpThreads) void permute_experts_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_tok, int32_t* __restrict__ slot_row, int shared_rows, int bm,
    int4* __restrict__ tiles, int cap, int32_t* __restrict__ tile_count) {
  __shared__ int cnt[kEpMaxE];
  __shared__ int offl[kEpMaxE + 1];
  __shared__ int ftl[kEpMaxE + 1];
  const int tid = threadIdx.x;
  const int n = T * k;
  constexpr int per = PER;
  const int f0 = tid * per;
  int32_t ev[PER];
  // 16-byte loads where four whole pairs are present (idx is 16-byte aligned, f0 % 4 == 0)
#pragma unroll
  for (int j = 0; j < PER; j += 4) {
    if (PER % 4 == 0 && f0 + j + 4 <= n) {
      const int4 v = *(const int4*)(idx + f0 + j);
      ev[j] = v.x;
      ev[j + 1] = v.y;
      ev[j + 2] = v.z;
      ev[j + 3] = v.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (j + u < PER) ev[j + u] = f0 + j + u < n ? idx[f0 + j + u] : -1;
    }
  }
  for (int g = tid; g < E; g += kEpThreads) cnt[g] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = ev[j];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // offsets and first tiles of the routed groups: thread i owns groups 4i .. 4i+3
  int c4[4], rsum = 0, tsum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int g = 4 * tid + u;
    c4[u] = g < E ? cnt[g] : 0;
    rsum += c4[u];
    tsum += (c4[u] + bm - 1) / bm;
  }
  uint64_t tot;
  const uint64_t ex =
      block_exclusive_scan_u64_256((uint64_t)(uint32_t)rsum | ((uint64_t)(uint32_t)tsum << 32), &tot);
  {
    int ro = (int)(uint32_t)ex, to = (int)(uint32_t)(ex >> 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = 4 * tid + u;
      if (g < E) {
        offl[g] = ro;
        ftl[g] = to;
      }
      ro += c4[u];
      to += (c4[u] + bm - 1) / bm;
    }
  }
  const int total = (int)(uint32_t)tot, ttot = (int)(uint32_t)(tot >> 32);
  if (tid == 0) {
    offl[E] = total;
    ftl[E] = ttot;
  }
  __syncthreads();

  if (blockIdx.x == 0) {
    for (int g = tid; g <= E; g += kEpThreads) offsets[g] = offl[g];
    if (tid == 0 && shared_rows >= 0) offsets[E + 1] = total + shared_rows;
    if (tid == 0 && tiles) {
      const int ns = shared_rows >= 0 ? (shared_rows + bm - 1) / bm : 0;
      *tile_count = min(ttot + ns, cap);
    }
  }

  // this workgroup's experts: ranks from a packed scan of the per-thread counts
  const int e0 = blockIdx.x * kEpExperts;
  uint64_t mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = ev[j], d = e - e0;
    if (d >= 0 && d < kEpExperts && e < E) mine += 1ull << (16 * d);
  }
  uint64_t unused;
  uint64_t run = block_exclusive_scan_u64_256(mine, &unused);
  int tok = f0 / k, slot = f0 - (f0 / k) * k;  // token and slot of pair f0 + j, stepped
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (f0 + j < n) {
      const int e = ev[j], d = e - e0;
      if (d >= 0 && d < kEpExperts && e < E) {
        int row = offl[e] + (int)((run >> (16 * d)) & 0xFFFFu);
        run += 1ull << (16 * d);
        if (row >= 0 && row < n) sorted_tok[row] = tok;  // always, for consistent counts
        else row = -1;
        slot_row[f0 + j] = row;
      } else if ((e < 0 || e >= E) && blockIdx.x == 0) {
        slot_row[f0 + j] = -1;
      }
    }
    if (++slot == k) {
      slot = 0;
      ++tok;
    }
  }

  if (tiles) {
#pragma unroll
    for (int d = 0; d < kEpExperts; ++d) {
      const int e = e0 + d;
      if (e < E) {
        const int c = cnt[e], nt = (c + bm - 1) / bm, ft = ftl[e], lo = offl[e];
        for (int u = tid; u < nt; u += kEpThreads) {
          const int t = ft + u;
          if (t < cap) tiles[t] = make_int4(e, lo + u * bm, min(bm, c - u * bm), 0);
        }
      }
    }
  }
  if (shared_rows >= 0 && blockIdx.x == gridDim.x - 1) {
    for (int t = tid; t < T; t += kEpThreads) sorted_tok[n + t] = t;
    if (tiles) {
      const int ns = (shared_rows + bm - 1) / bm;
      for (int u = tid; u < ns; u += kEpThreads) {
        const int t = ttot + u;
        if (t < cap) tiles[t] = make_int4(E, total + u * bm, min(bm, shared_rows - u * bm), 0);
      }
    }
  }
}

bool permute_experts_ok(int T, int k, int E) {
  return T >= 1 && k >= 1 && (int64_t)T * k <= (int64_t)kEpThreads * kEpPer && E >= 1 &&
         E <= kEpMaxE;
}

void launch_permute_experts(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                            int32_t* sorted_tok, int32_t* slot_row, int shared_rows, int bm,
                            int4* tiles, int32_t* tile_count, hipStream_t s) {
  int cap = 0;
  if (tiles) {
    const int n_groups = E + (shared_rows >= 0 ? 1 : 0);
    const int rows_total = T * k + (shared_rows >= 0 ? shared_rows : 0);
    cap = (int)max_tiles(rows_total, n_groups, bm);
  }
  const int grid = (E + kEpExperts - 1) / kEpExperts;
  const int need = (T * k + kEpThreads - 1) / kEpThreads;
#define MOEQ4_EP(P)                                                                           \
  hipLaunchKernelGGL(permute_experts_kernel<P>, dim3(grid), dim3(kEpThreads), 0, s, idx, T, k, \
                     E, offsets, sorted_tok, slot_row, shared_rows, bm, tiles, cap, tile_count)
  if (need <= 1) MOEQ4_EP(1);
  else if (need <= 2) MOEQ4_EP(2);
  else if (need <= 4) MOEQ4_EP(4);
  else if (need <= 8) MOEQ4_EP(8);
  else if (need <= 16) MOEQ4_EP(16);
  else MOEQ4_EP(32);
#undef MOEQ4_EP
}

}  // namespace moeq4
