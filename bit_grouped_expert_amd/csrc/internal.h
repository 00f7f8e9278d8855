// Internal launchers and workspace layout of libmoeq4 (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq4 {

// ---------------------------------------------------------------- routing
void launch_router_split(const float* R, uint16_t* Rs, int E, int D, hipStream_t s);
// xprep (nullable): also write the prepared copy of x ([T + 1, D], last row zero) read by
// the resident-tile GEMM
void launch_router_logits(const uint16_t* x, const uint16_t* Rs, float* L, int T, int D, int E,
                          uint16_t* xprep, hipStream_t s);
// Router logits L = x R^T (fp32): with T <= 16 one wavefront per expert; with T < 2048
// and D % 256 == 0 on the bf16 matrix cores with R split exactly in registers; otherwise
// R split into three bf16 planes (Rs, 3 * ceil(E/16) * 16 * D) and bf16 matrix cores.
// xprep as above.  planes_ready: Rs already holds the planes of this R (the split is
// skipped).
bool router_uses_planes(int T, int D);
// the one-wavefront-per-expert router (T <= 16, D % 256 == 0); its workgroups also clear
// n_zero words at `zero` for the kernel that follows
bool router_small_ok(int T, int D);
void launch_router_small(const uint16_t* x, const float* R, float* L, int T, int D, int E,
                         uint16_t* xprep, int32_t* zero, int n_zero, hipStream_t s);
void launch_router(const uint16_t* x, const float* R, uint16_t* Rs, float* L, int T, int D, int E,
                   uint16_t* xprep, hipStream_t s, bool planes_ready = false);
// also clears n_zero words at `zero` (nullable): a later launch's counters
void launch_topk(const float* L, const uint16_t* x, const float* R, int T, int D, int E, int k,
                 float tau, int32_t* idx, float* w, int32_t* zero, int n_zero, hipStream_t s);

// ---------------------------------------------------------------- permutation
constexpr int kChunkTokens = 256;  // tokens per histogram / scatter chunk
constexpr int kMaxTopK = 32;       // largest top_k the shape check accepts
inline int n_chunks(int T) { return (T + kChunkTokens - 1) / kChunkTokens; }
void launch_count(const int32_t* idx, int T, int k, int E, int32_t* chunk_cnt, hipStream_t s);
void launch_scan(int32_t* chunk_cnt, int nchunks, int E, int32_t* offsets, int shared_rows,
                 hipStream_t s);
void launch_scatter(const int32_t* idx, int T, int k, int E, const int32_t* chunk_base,
                    const int32_t* offsets, int32_t* sorted_tok, int32_t* slot_row, int shared_base,
                    hipStream_t s);
// launch_scan followed, in the same single-workgroup launch, by the tile map of the E
// routed groups (+ the shared group when shared_rows >= 0) over rows_total rows
void launch_scan_tiles(int32_t* chunk_cnt, int nchunks, int E, int32_t* offsets, int shared_rows,
                       int rows_total, int bm, int4* tiles, int32_t* tile_count, hipStream_t s);

// ---------------------------------------------------------------- grouped GEMM
struct Q4Ptrs {
  const uint32_t* q;
  const uint16_t* s;
  const uint16_t* b;
};

struct GemmParams {
  const uint16_t* A;          // bf16 [a_rows, K]
  const int32_t* a_row_index; // nullable: identity
  int32_t a_rows;
  Q4Ptrs main;                // groups 0..n_main-1, contiguous
  int32_t n_main;
  Q4Ptrs last;                // group n_main (if any)
  int32_t N, K;
  uint16_t* C;                // bf16 [rows, ldc]
  int32_t ldc;
  const int4* tiles;          // (group, row0, rows, 0)
  const int32_t* tile_count;
  int32_t n_slices;
  const float* xsum;          // [a_rows, xsum_ld] row sums of A per 64-wide K group
  int32_t xsum_ld;
  float* xsum_out;            // nullable; SwiGLU only: row sums of C per 64 columns
  int32_t xsum_out_ld;
};

constexpr int kMaxTileGroups = 1025;  // groups of a tile map: 1024 routed experts + the shared one
inline int64_t max_tiles(int64_t rows_total, int n_groups, int bm) {
  return (rows_total + bm - 1) / bm + n_groups;
}
void launch_build_tiles(const int32_t* offsets, int n_groups, int rows_total, int bm, int4* tiles,
                        int32_t* tile_count, hipStream_t s);
// Histogram, scan, stable scatter and tile map with one workgroup per four experts
// (T * k <= 8192, E <= 1024); with tiles == NULL no tile map is written.  Same results
// as launch_count + launch_scan + launch_scatter + launch_build_tiles.
bool permute_experts_ok(int T, int k, int E);
void launch_permute_experts(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                            int32_t* sorted_tok, int32_t* slot_row, int shared_rows, int bm,
                            int4* tiles, int32_t* tile_count, hipStream_t s);
// The same in one single-workgroup launch (T <= 1024).
bool permute_small_ok(int T, int E);
void launch_permute_small(const int32_t* idx, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_tok, int32_t* slot_row, int shared_rows, int bm,
                          int4* tiles, int32_t* tile_count, hipStream_t s);
// Grouped engine for every group size: tiles of up to 32 rows (tile map built with
// bm = 32), persistent XCD-aware grid of about 2 workgroups per compute unit.  Needs
// p.xsum (row sums of A per 64-wide group); with SwiGLU it can also write the row sums
// of its output (p.xsum_out) for the next GEMM.
constexpr int kGroupedBM = 32;
void launch_grouped(GemmParams p, bool swiglu, int64_t n_tiles_bound, int n_cu, hipStream_t s);
int grouped_slices(int N, bool swiglu);
// out[r][g] = sum of A[r][64g .. 64g+63] in fp32, A bf16 [rows, K]
void launch_row_group_sums(const uint16_t* A, int rows, int K, float* out, hipStream_t s);

// The prepared copy of A read by the resident and wide engines: every run of 8 columns
// stored in the order 0,4,1,5,2,6,3,7 (the order a packed word unpacks to), and one
// zero row after the last (row `rows`), which rows outside [0, rows) read instead.
void launch_prep(const uint16_t* A, int rows, int K, uint16_t* Ap, hipStream_t s);

// Resident-tile engine (grouped_resident.hip), for small groups: tiles of up to 32
// rows (tile map built with bm = 32) whose activation rows stay in LDS for the whole
// K.  A is the prepared copy (each run of 8 columns stored in the order
// 0,4,1,5,2,6,3,7) and row a_rows of A must be readable: rows that fall outside
// [0, a_rows) read it, so it must be zero where that can happen.  C rows are written with 16-byte stores (ldc % 8 == 0).
// With SwiGLU (N = 2F) and c_perm set, C is stored in the prepared column order.
constexpr int kResidentBM = 32;
constexpr int kResidentMaxK = 2048;
struct ResidentParams {
  const uint16_t* A;          // prepared bf16 [a_rows (+1), K]
  const int32_t* a_row_index; // nullable: identity
  int32_t a_rows;
  Q4Ptrs main;
  int32_t n_main;
  Q4Ptrs last;
  int32_t N, K;
  uint16_t* C;
  int32_t ldc;
  int32_t c_perm;
  const int4* tiles;
  const int32_t* tile_count;
  int32_t ksplit;             // set by launch_resident
  // One launch for gate_up then down (launch_resident_pair), else all zero.  Role 1 (the
  // gate_up phase): outputs go out with device-scope stores, and every finished chunk adds
  // one to sync[kPairTileBase + tile].  Role 2 (the down phase): before reading tile t's
  // activations (device-scope loads) it waits until that count reaches ready_need, and it
  // takes its chunk range starting after the tile it shares with the previous range.  A
  // wait that gives up adds one to sync[0].
  int32_t pair_role;
  int32_t ready_need;
  int32_t pair_wu, pair_wd;   // role 2: weights of a gate_up and a down chunk
  int32_t* sync;
};
constexpr int kResidentMaxStages = 4;  // 256-K stages per wavefront and chunk
constexpr int kPairTileBase = 64;      // sync words before the per-tile counters
struct ResidentPlan {
  int ksplit;  // 1: eight column groups over the whole K; 2: four column groups x two K halves
  int stages;  // 256-K stages per wavefront and chunk (K / 256 / ksplit)
  int grid;    // workgroups (a multiple of 8)
};
// false when the engine cannot take the shape (K % 256, K > kResidentMaxK, more than
// kResidentMaxStages stages per wavefront, N not a multiple of the chunk, or too many
// tiles per workgroup for n_tiles_bound)
bool resident_plan(int N, int K, bool swiglu, int64_t n_tiles_bound, int n_cu, ResidentPlan* out);
void launch_resident(ResidentParams p, const ResidentPlan& plan, bool swiglu, hipStream_t s);
// gate_up (+ SwiGLU) and down as one launch: every workgroup runs its gate_up range, then
// its down range, whose tiles wait on the gate_up chunks that write their activations.
// Needs sync[0 .. kPairTileBase + n_tiles_bound) zero at the launch.  resident_pair_ok is
// false where the pair does not apply: the two plans differ in grid, a stage count is not
// compiled for it, the tile bound reaches the dealt mode (8 tiles per workgroup), or a
// workgroup's down share could overflow its segment table.
bool resident_pair_ok(const ResidentPlan& up, const ResidentPlan& down, int N_up, int K_up, int N_dn,
                      int K_dn, int64_t n_tiles_bound);
void launch_resident_pair(ResidentParams up, ResidentParams down, const ResidentPlan& pu,
                          const ResidentPlan& pd, int32_t* sync, hipStream_t s);

// Parameters of the wide-tile engine.
struct WideParams {
  const uint16_t* A;          // prepared bf16 [a_rows (+1), K]
  const int32_t* a_row_index; // nullable: identity
  int32_t a_rows;
  Q4Ptrs main;
  int32_t n_main;
  Q4Ptrs last;
  int32_t N, K;
  uint16_t* C;
  int32_t ldc;
  int32_t c_perm;
  const int4* tiles;
  const int32_t* tile_count;
  int32_t xcd_cus;  // compute units per XCD (set by launch_wide; 0: one tile per workgroup)
};

// Wide-tile engine (grouped_wide.hip), for large groups: one workgroup per tile of up
// to 128 rows (tile map built with bm = kWideBM), weights streamed into VGPRs, the
// tile's activations through two LDS stage buffers.  Same A, C and c_perm conventions
// as the resident engine; needs K % 256 == 0, K <= kWideMaxK, N % 256 == 0 (SwiGLU:
// N = 2F with F % 128 == 0) and a_rows >= 1; C rows are written with 16-byte stores.
constexpr int kWideBM = 128;
constexpr int kWideMaxK = 2048;
bool wide_supported(int N, int K, bool swiglu, int a_rows);
void launch_wide(WideParams p, bool swiglu, int64_t n_tiles_bound, int n_cu, hipStream_t s);

// ---------------------------------------------------------------- decode-sized layer
// T <= 16 tokens (decode.hip): after the few-token router (which clears the counters),
// one launch whose workgroups each compute the plan (top-k, touched-expert slots, combine
// weights; workgroup 0 also the routing outputs) and then one item, in workgroup order:
// gate_up + SwiGLU per (slot, 16-row slice), then down fused with the combine per (16
// output columns, group of slots), each down item waiting on its slots' gate_up items.
constexpr int kDecodeMaxT = 16;
constexpr int kDecodeMaxPairs = 128;                  // T * k
constexpr int kDecodeMaxSlots = kDecodeMaxPairs + 1;  // distinct experts + the shared one
struct DecodeParams {
  int32_t T, D, E, k, F, has_shared;
  int32_t group_slots;  // most slots per down item
  int32_t n_cb;         // D / 16 output column blocks
  float tau;            // top-k refinement gap
  const float* logits;  // [T, E] fp32
  const uint16_t* x;    // [T, D] bf16 (the exact top-k rescoring)
  const float* R;       // [E, D] fp32
  const uint16_t* xprep;  // prepared x [T + 1, D], row T zero
  int32_t* idx;         // [T, k] routing outputs (written by workgroup 0)
  float* w;             // [T, k]
  int32_t* offsets;     // [E + 2]
  int32_t* sorted_tok;  // [T k + T]
  int32_t* slot_row;    // [T k]
  int32_t* sync;        // decode_sync_ints() counters and flags, zero at launch
  float* part;          // down partial sums [groups][n_cb][16][16]
  uint16_t* act;        // bf16 [max slots][16 tokens][F], prepared column order
  uint16_t* out;        // bf16 [T, D]
  Q4Ptrs up_main, up_last, down_main, down_last;  // experts [E, ...]; the shared expert
  // Workgroups from index `early` on (those that start only once earlier ones finish) take
  // the plan that workgroup 0 publishes to `plan` (decode_plan_bytes()) instead of
  // computing it, when it is there within a bounded wait; set early to the grid size or
  // more to have every workgroup compute it.
  int32_t early;
  uint32_t* plan;
};
bool decode_supported(int T, int D, int E, int k, int F);
size_t decode_plan_bytes();
int decode_group_slots(int F);
int decode_sync_ints(int D, int F, int max_slots);
size_t decode_part_bytes(int D, int F, int max_slots);
size_t decode_act_bytes(int F, int max_slots);
void launch_decode_layer(const DecodeParams& p, int max_slots, hipStream_t s);

// ---------------------------------------------------------------- decode attention
// Grouped-query attention of one query token over a bf16 KV cache (attention.hip): a
// partial launch over runs of 128-position chunks per KV head and a reduce launch per
// query head.
constexpr int kAttnHeadDim = 128;
struct AttnParams {
  int32_t n_q, n_kv, group, ctx, n_chunks;
  int32_t per_part, n_part;  // chunks per partial, partials per KV head (attn_partition)
  int64_t kv_stride;      // positions allocated per KV head
  float scale;            // 1 / sqrt(head dim)
  const uint16_t* q;      // bf16 [n_q, 128]
  const uint16_t* k;      // bf16 [n_kv, kv_stride, 128]
  const uint16_t* v;      // bf16 [n_kv, kv_stride, 128]
  float* part_o;          // [n_kv, n_part, group, 128] unnormalised partial outputs
  float* part_ml;         // [n_kv, n_part, group, 2] partial max and sum
  uint16_t* out;          // bf16 [n_q, 128]
};
bool attn_supported(int n_q, int n_kv, int head_dim, int ctx, int64_t kv_stride);
int attn_chunks(int ctx);
size_t attn_workspace_bytes(int n_q, int n_kv, int ctx);
void attn_partition(AttnParams* p, int n_cu);
void launch_attention(const AttnParams& p, hipStream_t s);

// ---------------------------------------------------------------- combine
void launch_combine(const uint16_t* Y, int64_t y_rows, const int32_t* slot_row, const float* w,
                    const uint16_t* S, uint16_t* out, int T, int D, int k, hipStream_t s);

}  // namespace moeq4
