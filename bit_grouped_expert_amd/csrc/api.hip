// C ABI of libmoeq4: host-side validation, workspace carving and launches.
// Every entry point validates on the host before it enqueues anything, then
// enqueues its kernels on the caller's stream and returns without waiting.
#include <stdlib.h>
#include <string.h>

#include "../../include/moeq4.h"
#include "internal.h"

using namespace moeq4;

namespace {

constexpr size_t kAlign = 256;
constexpr float kRefineGap = 1e-4f;
// average rows per group from which the wide-tile engine is the default (measured: at
// 8192 tokens, about 290 rows per group, 955 against 964 us for both GEMMs; at 32768,
// 3.06 against 3.29 ms)
constexpr int64_t kWideMinAvgRows = 192;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_NULL;
  if (s->T < 0 || s->d_model <= 0 || s->d_ff <= 0 || s->n_experts < 1 || s->n_experts > 1024 ||
      s->top_k < 1 || s->top_k > 32 || s->top_k > s->n_experts)
    return MOE_ERR_SHAPE;
  if (s->d_model % 64 != 0 || s->d_ff % 64 != 0) return MOE_ERR_SHAPE;
  const int64_t widest = s->d_model > 2 * (int64_t)s->d_ff ? s->d_model : 2 * (int64_t)s->d_ff;
  if ((int64_t)(s->top_k + 1) * s->T * widest >= (int64_t)1 << 31) return MOE_ERR_SHAPE;
  if ((int64_t)s->n_experts * s->d_model * 3 >= (int64_t)1 << 31) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// Which grouped-GEMM engine runs, and its tile rows.
//   resident (default wherever the shapes allow it): tiles of up to 32 rows whose
//            activations stay in LDS for the whole K while the weights stream
//            through VGPRs (measured faster than grouped at 512 and at 8192 tokens);
//   grouped  (default otherwise): register-prefetched grouped engine, tiles of 32 rows;
//   stream   (needs K % 128 == 0): operands streamed through an LDS ring by direct
//            global->LDS loads; tiles of 32 rows, or 64 when groups average at
//            least 48 rows;
//   rows:    the first register-streaming engine, one workgroup per tile and slice;
//   tiled    (K % 256 == 0, N % 256 == 0): tiles of 128 rows times blocks of 256
//            weight rows, both operands staged through LDS per 64-K stage, the
//            weights unpacked once per workgroup (measured no faster than resident
//            at 8192 tokens: bound by LDS traffic; not a default).
//   wide     (default when groups average at least 192 rows; K % 256 == 0,
//            K <= 2048, N % 256 == 0): tiles of 128 rows, weights streamed into VGPRs,
//            each packed word feeding eight row fragments, the activations through two
//            LDS stage buffers.
// The environment variable MOEQ4_GEMM=resident|stream|grouped|rows|tiled|wide forces one
// (for measurement and tests; an engine that cannot take the shapes falls back to
// grouped).
enum Engine { ENG_ROWS, ENG_GROUPED, ENG_STREAM, ENG_RESIDENT, ENG_TILED, ENG_WIDE };
struct GemmPlan {
  Engine eng;
  int bm;
};
GemmPlan plan_gemm(int64_t rows, int n_groups, bool stream_ok, bool resident_ok,
                   bool tiled_ok = false, bool wide_ok = false) {
  const int64_t g = n_groups > 0 ? n_groups : 1;
  const char* env = getenv("MOEQ4_GEMM");
  if (env && strcmp(env, "wide") == 0 && wide_ok) return GemmPlan{ENG_WIDE, kWideBM};
  if (env && strcmp(env, "tiled") == 0 && tiled_ok) return GemmPlan{ENG_TILED, kTiledBM};
  if (env && strcmp(env, "rows") == 0) return GemmPlan{ENG_ROWS, rows <= 64 * g ? 32 : 64};
  if (env && strcmp(env, "grouped") == 0) return GemmPlan{ENG_GROUPED, kGroupedBM};
  if (env && strcmp(env, "stream") == 0 && stream_ok)
    return GemmPlan{ENG_STREAM, rows >= 48 * g ? 64 : 32};
  if (env && strcmp(env, "resident") == 0 && resident_ok) return GemmPlan{ENG_RESIDENT, kResidentBM};
  if (!env && wide_ok && rows >= kWideMinAvgRows * g) return GemmPlan{ENG_WIDE, kWideBM};
  if (!env && resident_ok) return GemmPlan{ENG_RESIDENT, kResidentBM};
  return GemmPlan{ENG_GROUPED, kGroupedBM};
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Grouped GEMM launch with the plan's engine (the tile map is already built with plan.bm).
void run_gemm(GemmParams p, const GemmPlan& plan, bool swiglu, int64_t rows, int n_groups,
              hipStream_t stream) {
  const int64_t bound = max_tiles(rows, n_groups, plan.bm);
  if (plan.eng == ENG_GROUPED) launch_grouped(p, swiglu, bound, device_cu_count(), stream);
  else launch_gemm_q4(p, plan.bm, swiglu, bound, stream);
}

void run_stream(StreamParams p, const GemmPlan& plan, bool swiglu, int64_t rows, int n_groups,
                hipStream_t stream) {
  const int64_t bound = max_tiles(rows, n_groups, plan.bm);
  launch_stream(p, swiglu, plan.bm / 16, bound, device_cu_count(), stream);
}

struct Layout {
  size_t rsplit, logits, topk_idx, topk_w, chunk_cnt, offsets, sorted_tok, slot_row, tiles,
      tile_count, xsum_x, xsum_act, xprep, xc_x, xc_act, act, y, total;
};

// the streamed engine serves the layer when both GEMMs have K % 128 == 0
bool layer_stream_ok(const moe_shape* s) { return s->d_model % 128 == 0 && s->d_ff % 128 == 0; }

Layout make_layout(const moe_shape* s) {
  const int64_t T = s->T, D = s->d_model, E = s->n_experts, k = s->top_k, F = s->d_ff;
  const int64_t rows_ext = (k + 1) * T;
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.rsplit = take(3 * (size_t)((E + 15) / 16 * 16) * D * 2);
  L.logits = take(T * E * 4);
  L.topk_idx = take(T * k * 4);
  L.topk_w = take(T * k * 4);
  L.chunk_cnt = take((size_t)n_chunks((int)T) * E * 4);
  L.offsets = take((E + 2) * 4);
  L.sorted_tok = take(rows_ext * 4);
  L.slot_row = take(T * k * 4);
  L.tiles = take((size_t)max_tiles(rows_ext, (int)E + 1, 32) * sizeof(int4));
  L.tile_count = take(16);
  L.xsum_x = take(T * (D / 64) * 4);
  L.xsum_act = take(rows_ext * (F / 64) * 4);
  // prepared x (one zero row after the last) and the (-136 X, X) rows of x and act
  L.xprep = take((T + 1) * D * 2);
  L.xc_x = take((T + 1) * (D / 128) * 16);
  L.xc_act = take((rows_ext + 1) * (F / 128) * 16);
  L.act = take((rows_ext + 1) * F * 2);
  L.y = take(rows_ext * D * 2);
  L.total = o;
  return L;
}

bool q4_ok(const moe_q4& w) { return w.q && w.scale && w.bias; }
bool q4_aligned(const moe_q4& w) {
  return aligned16(w.q) && aligned16(w.scale) && aligned16(w.bias);
}

moe_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "invalid shape";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return make_layout(shape).total;
}

moe_status moe_workspace_layout(const moe_shape* shape, moe_ws_layout* layout) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!layout) return MOE_ERR_NULL;
  const Layout L = make_layout(shape);
  layout->topk_idx = L.topk_idx;
  layout->topk_w = L.topk_w;
  layout->offsets = L.offsets;
  layout->sorted_tok = L.sorted_tok;
  layout->slot_row = L.slot_row;
  layout->act = L.act;
  layout->y = L.y;
  layout->total = L.total;
  return MOE_OK;
}

namespace {
struct GemmWs {
  size_t tiles, tile_count, xsum, aprep, xc, total;
};
GemmWs gemm_ws(int32_t n_groups, int32_t rows_total, int32_t a_rows, int32_t K) {
  GemmWs w;
  w.tiles = 0;
  w.tile_count = align_up((size_t)max_tiles(rows_total, n_groups, 32) * sizeof(int4));
  w.xsum = w.tile_count + kAlign;
  w.aprep = w.xsum + align_up((size_t)a_rows * (size_t)(K / 64) * 4);
  // the prepared copy of A (resident, tiled and streamed engines)
  w.xc = w.aprep + align_up(((size_t)a_rows + 1) * (size_t)K * 2);
  w.total = w.xc;
  if (K % 128 == 0)  // the streamed engine's per-stage row sums
    w.total = w.xc + align_up(((size_t)a_rows + 1) * (size_t)(K / 128) * 16);
  return w;
}
}  // namespace

size_t moe_grouped_gemm_q4_workspace_bytes(int32_t n_groups, int32_t rows_total, int32_t a_rows,
                                           int32_t K) {
  if (n_groups < 1 || n_groups > kMaxTileGroups || rows_total < 0 || a_rows < 0 || K <= 0 || K % 64)
    return 0;
  return gemm_ws(n_groups, rows_total, a_rows, K).total;
}

static moe_status route_impl(const moe_shape* shape, const uint16_t* x, const float* router_w,
                             int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                             hipStream_t stream, float gap) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->T == 0) return MOE_OK;
  if (!x || !router_w || !topk_idx || !topk_w) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(topk_idx) || !aligned16(topk_w))
    return MOE_ERR_ALIGN;
  const Layout L = make_layout(shape);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  const int T = shape->T, D = shape->d_model, E = shape->n_experts, k = shape->top_k;
  uint16_t* Rs = at<uint16_t>(ws, L.rsplit);
  float* logits = at<float>(ws, L.logits);
  launch_router(x, router_w, Rs, logits, T, D, E, nullptr, stream);
  launch_topk(logits, x, router_w, T, D, E, k, gap, topk_idx, topk_w, stream);
  return launch_status();
}

moe_status moe_route(const moe_shape* shape, const uint16_t* x, const float* router_w,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  return route_impl(shape, x, router_w, topk_idx, topk_w, ws, ws_bytes, stream, kRefineGap);
}

moe_status moe_route_ex(const moe_shape* shape, const uint16_t* x, const float* router_w,
                        int32_t* topk_idx, float* topk_w, float refine_gap, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  if (!(refine_gap >= 0.f)) return MOE_ERR_SHAPE;
  return route_impl(shape, x, router_w, topk_idx, topk_w, ws, ws_bytes, stream, refine_gap);
}

// Chunked histogram, scan and scatter; with tiles set the scan launch also writes the
// tile map (bm rows per tile over rows_total rows).
static moe_status permute_impl(const moe_shape* shape, const int32_t* topk_idx, int32_t* offsets,
                               int32_t* sorted_tok, int32_t* slot_row, int32_t* chunk_cnt,
                               int shared_rows, hipStream_t stream, int4* tiles = nullptr,
                               int32_t* tile_count = nullptr, int rows_total = 0, int bm = 1) {
  const int T = shape->T, E = shape->n_experts, k = shape->top_k;
  const int nch = n_chunks(T);
  launch_count(topk_idx, T, k, E, chunk_cnt, stream);
  if (tiles)
    launch_scan_tiles(chunk_cnt, nch, E, offsets, shared_rows, rows_total, bm, tiles, tile_count,
                      stream);
  else
    launch_scan(chunk_cnt, nch, E, offsets, shared_rows, stream);
  launch_scatter(topk_idx, T, k, E, chunk_cnt, offsets, sorted_tok, slot_row,
                 shared_rows >= 0 ? T * k : -1, stream);
  return MOE_OK;
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, int32_t* offsets,
                       int32_t* sorted_tok, int32_t* slot_row, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  // with T == 0 only the offsets are written; the empty arrays may be NULL
  const bool empty = shape->T == 0;
  if (!offsets || (!empty && (!topk_idx || !sorted_tok || !slot_row))) return MOE_ERR_NULL;
  if (!aligned16(offsets) ||
      (!empty && (!aligned16(topk_idx) || !aligned16(sorted_tok) || !aligned16(slot_row))))
    return MOE_ERR_ALIGN;
  const Layout L = make_layout(shape);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  if (empty) {
    // empty routing still defines offsets (all zero): a scan over zero chunks
    launch_scan(at<int32_t>(ws, L.chunk_cnt), 0, shape->n_experts, offsets, -1, stream);
    return launch_status();
  }
  if (permute_experts_ok(shape->T, shape->top_k, shape->n_experts))
    launch_permute_experts(topk_idx, shape->T, shape->top_k, shape->n_experts, offsets, sorted_tok,
                           slot_row, -1, 1, nullptr, nullptr, stream);
  else
    permute_impl(shape, topk_idx, offsets, sorted_tok, slot_row, at<int32_t>(ws, L.chunk_cnt), -1,
                 stream);
  return launch_status();
}

moe_status moe_grouped_gemm_q4(int32_t n_groups, int32_t rows_total, int32_t N, int32_t K,
                               const uint16_t* A, int32_t a_rows, const int32_t* a_row_index,
                               const int32_t* offsets, moe_q4 W, int32_t epilogue, uint16_t* C,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_groups < 1 || n_groups > kMaxTileGroups || rows_total < 0 || a_rows < 0 || N <= 0 ||
      K <= 0 || N % 64 || K % 64 || (epilogue != 0 && epilogue != 1))
    return MOE_ERR_SHAPE;
  const int64_t widest = N > K ? N : K;
  if ((int64_t)rows_total * widest >= ((int64_t)1 << 31) ||
      (int64_t)a_rows * K >= ((int64_t)1 << 31))
    return MOE_ERR_SHAPE;
  if (rows_total == 0) return MOE_OK;
  if (!A || !offsets || !q4_ok(W) || !C) return MOE_ERR_NULL;
  if (!aligned16(A) || !aligned16(offsets) || !q4_aligned(W) || !aligned16(C) ||
      (a_row_index && !aligned16(a_row_index)))
    return MOE_ERR_ALIGN;
  const GemmWs gw = gemm_ws(n_groups, rows_total, a_rows, K);
  if (!ws || ws_bytes < gw.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;

  const int n_cu = device_cu_count();
  ResidentPlan rplan;
  const bool resident_ok =
      a_rows >= 1 &&
      resident_plan(N, K, epilogue == 1, max_tiles(rows_total, n_groups, kResidentBM), n_cu, &rplan);
  const GemmPlan plan = plan_gemm(rows_total, n_groups, stream_supported(N, K, a_rows), resident_ok,
                                  tiled_supported(N, K, epilogue == 1, a_rows),
                                  wide_supported(N, K, epilogue == 1, a_rows));
  int4* tiles = at<int4>(ws, gw.tiles);
  int32_t* tile_count = at<int32_t>(ws, gw.tile_count);
  float* xsum = at<float>(ws, gw.xsum);
  launch_build_tiles(offsets, n_groups, rows_total, plan.bm, tiles, tile_count, stream);
  if (plan.eng == ENG_TILED || plan.eng == ENG_WIDE) {
    // prepared copy of A (column order 0,4,1,5,... per run of 8, one zero row after the last)
    uint16_t* aprep = at<uint16_t>(ws, gw.aprep);
    launch_prep(A, a_rows, K, aprep, nullptr, stream);
    TiledParams tp;
    memset(&tp, 0, sizeof(tp));
    tp.A = aprep;
    tp.a_row_index = a_row_index;
    tp.a_rows = a_rows;
    tp.main = Q4Ptrs{W.q, W.scale, W.bias};
    tp.n_main = n_groups;
    tp.last = tp.main;
    tp.N = N;
    tp.K = K;
    tp.C = C;
    tp.ldc = epilogue == 1 ? N / 2 : N;
    tp.c_perm = 0;
    tp.tiles = tiles;
    tp.tile_count = tile_count;
    if (plan.eng == ENG_WIDE) launch_wide(tp, epilogue == 1, max_tiles(rows_total, n_groups, kWideBM), stream);
    else launch_tiled(tp, epilogue == 1, max_tiles(rows_total, n_groups, kTiledBM), stream);
    return launch_status();
  }
  if (plan.eng == ENG_RESIDENT) {
    // prepared copy of A (column order 0,4,1,5,... per run of 8, one zero row after the last)
    uint16_t* aprep = at<uint16_t>(ws, gw.aprep);
    launch_prep(A, a_rows, K, aprep, nullptr, stream);
    ResidentParams rp;
    memset(&rp, 0, sizeof(rp));
    rp.A = aprep;
    rp.a_row_index = a_row_index;
    rp.a_rows = a_rows;
    rp.main = Q4Ptrs{W.q, W.scale, W.bias};
    rp.n_main = n_groups;
    rp.last = rp.main;
    rp.N = N;
    rp.K = K;
    rp.C = C;
    rp.ldc = epilogue == 1 ? N / 2 : N;
    rp.c_perm = 0;
    rp.tiles = tiles;
    rp.tile_count = tile_count;
    launch_resident(rp, rplan, epilogue == 1, stream);
    return launch_status();
  }
  if (plan.eng == ENG_STREAM) {
    uint16_t* aprep = at<uint16_t>(ws, gw.aprep);
    float4* xc = at<float4>(ws, gw.xc);
    launch_prep(A, a_rows, K, aprep, xc, stream);
    StreamParams sp;
    memset(&sp, 0, sizeof(sp));
    sp.A = aprep;
    sp.xc = xc;
    sp.a_row_index = a_row_index;
    sp.a_rows = a_rows;
    sp.main = Q4Ptrs{W.q, W.scale, W.bias};
    sp.n_main = n_groups;
    sp.last = sp.main;
    sp.N = N;
    sp.K = K;
    sp.C = C;
    sp.ldc = epilogue == 1 ? N / 2 : N;
    sp.tiles = tiles;
    sp.tile_count = tile_count;
    run_stream(sp, plan, epilogue == 1, rows_total, n_groups, stream);
    return launch_status();
  }
  if (plan.eng == ENG_GROUPED) launch_row_group_sums(A, a_rows, K, xsum, stream);

  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A = A;
  p.a_row_index = a_row_index;
  p.a_rows = a_rows;
  p.main = Q4Ptrs{W.q, W.scale, W.bias};
  p.n_main = n_groups;
  p.last = p.main;
  p.N = N;
  p.K = K;
  p.C = C;
  p.ldc = epilogue == 1 ? N / 2 : N;
  p.tiles = tiles;
  p.tile_count = tile_count;
  p.xsum = xsum;
  p.xsum_ld = K / 64;
  run_gemm(p, plan, epilogue == 1, rows_total, n_groups, stream);
  return launch_status();
}

moe_status moe_combine(const moe_shape* shape, const uint16_t* y_sorted, const int32_t* slot_row,
                       const float* topk_w, const uint16_t* shared_out, uint16_t* out,
                       hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->T == 0) return MOE_OK;
  if (!y_sorted || !slot_row || !topk_w || !out) return MOE_ERR_NULL;
  if (!aligned16(y_sorted) || !aligned16(slot_row) || !aligned16(topk_w) || !aligned16(out) ||
      (shared_out && !aligned16(shared_out)))
    return MOE_ERR_ALIGN;
  const int T = shape->T, D = shape->d_model, k = shape->top_k;
  launch_combine(y_sorted, (int64_t)T * k, slot_row, topk_w, shared_out, out, T, D, k, stream);
  return launch_status();
}

static moe_status layer_impl(const moe_shape* shape, const uint16_t* x, const float* router_w,
                             const moe_q4_ffn* experts, const moe_q4_ffn* shared, uint16_t* out,
                             void* ws, size_t ws_bytes, hipEvent_t* events, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->T == 0) return MOE_OK;
  if (!x || !router_w || !experts || !out) return MOE_ERR_NULL;
  if (!q4_ok(experts->gate_up) || !q4_ok(experts->down)) return MOE_ERR_NULL;
  if (shared && (!q4_ok(shared->gate_up) || !q4_ok(shared->down))) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(out) ||
      !q4_aligned(experts->gate_up) || !q4_aligned(experts->down) ||
      (shared && (!q4_aligned(shared->gate_up) || !q4_aligned(shared->down))))
    return MOE_ERR_ALIGN;
  const Layout L = make_layout(shape);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;

  const int T = shape->T, D = shape->d_model, E = shape->n_experts, k = shape->top_k,
            F = shape->d_ff;
  const bool has_shared = shared != nullptr;
  const int n_groups = E + (has_shared ? 1 : 0);
  const int rows = T * k + (has_shared ? T : 0);

  int32_t* idx = at<int32_t>(ws, L.topk_idx);
  float* wts = at<float>(ws, L.topk_w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted_tok = at<int32_t>(ws, L.sorted_tok);
  int32_t* slot_row = at<int32_t>(ws, L.slot_row);
  int4* tiles = at<int4>(ws, L.tiles);
  int32_t* tile_count = at<int32_t>(ws, L.tile_count);
  uint16_t* act = at<uint16_t>(ws, L.act);
  uint16_t* y = at<uint16_t>(ws, L.y);
  float* xsum_x = at<float>(ws, L.xsum_x);
  float* xsum_act = at<float>(ws, L.xsum_act);

  auto mark = [&](int i) {
    if (events && events[i]) hipEventRecord(events[i], stream);
  };
  // the GEMM engine depends only on the shapes: chosen first, so that the router can
  // write the resident engine's copy of x on the way
  const int n_cu = device_cu_count();
  const int64_t rbound = max_tiles(rows, n_groups, kResidentBM);
  ResidentPlan rp_up, rp_down;
  const bool resident_ok = resident_plan(2 * F, D, true, rbound, n_cu, &rp_up) &&
                           resident_plan(D, F, false, rbound, n_cu, &rp_down);
  const bool tiled_ok = tiled_supported(2 * F, D, true, T) && tiled_supported(D, F, false, rows);
  const bool wide_ok = wide_supported(2 * F, D, true, T) && wide_supported(D, F, false, rows);
  const GemmPlan plan = plan_gemm(rows, n_groups, layer_stream_ok(shape), resident_ok, tiled_ok, wide_ok);
  // routing
  mark(0);
  uint16_t* Rs = at<uint16_t>(ws, L.rsplit);
  float* logits = at<float>(ws, L.logits);
  launch_router(x, router_w, Rs, logits, T, D, E,
                       plan.eng == ENG_RESIDENT || plan.eng == ENG_TILED || plan.eng == ENG_WIDE
                           ? at<uint16_t>(ws, L.xprep)
                           : nullptr,
                       stream);
  launch_topk(logits, x, router_w, T, D, E, k, kRefineGap, idx, wts, stream);
  mark(1);
  // histogram, scan, scatter (+ identity rows of the shared group), tile map
  if (permute_experts_ok(T, k, E)) {
    launch_permute_experts(idx, T, k, E, offsets, sorted_tok, slot_row, has_shared ? T : -1,
                           plan.bm, tiles, tile_count, stream);
  } else if (permute_small_ok(T, E)) {
    launch_permute_small(idx, T, k, E, offsets, sorted_tok, slot_row, has_shared ? T : -1,
                         plan.bm, tiles, tile_count, stream);
  } else {
    permute_impl(shape, idx, offsets, sorted_tok, slot_row, at<int32_t>(ws, L.chunk_cnt),
                 has_shared ? T : -1, stream, tiles, tile_count, (int)rows, plan.bm);
  }
  if (plan.eng == ENG_STREAM) launch_prep(x, T, D, at<uint16_t>(ws, L.xprep), at<float4>(ws, L.xc_x), stream);
  else if (plan.eng == ENG_GROUPED) launch_row_group_sums(x, T, D, xsum_x, stream);
  mark(2);

  if (plan.eng == ENG_TILED || plan.eng == ENG_WIDE) {
    // gate_up + SwiGLU over the prepared x rows gathered through sorted_tok -> act, stored
    // in the prepared column order so that the down GEMM reads it as is
    TiledParams tp;
    memset(&tp, 0, sizeof(tp));
    tp.A = at<uint16_t>(ws, L.xprep);
    tp.a_row_index = sorted_tok;
    tp.a_rows = T;
    tp.main = Q4Ptrs{experts->gate_up.q, experts->gate_up.scale, experts->gate_up.bias};
    tp.n_main = E;
    tp.last = has_shared ? Q4Ptrs{shared->gate_up.q, shared->gate_up.scale, shared->gate_up.bias}
                         : tp.main;
    tp.N = 2 * F;
    tp.K = D;
    tp.C = act;
    tp.ldc = F;
    tp.c_perm = 1;
    tp.tiles = tiles;
    tp.tile_count = tile_count;
    const bool wide = plan.eng == ENG_WIDE;
    const int64_t tbound = max_tiles(rows, n_groups, wide ? kWideBM : kTiledBM);
    if (wide) launch_wide(tp, true, tbound, stream);
    else launch_tiled(tp, true, tbound, stream);
    mark(3);
    // down: act rows in order -> y [rows, D]
    tp.A = act;
    tp.a_row_index = nullptr;
    tp.a_rows = rows;
    tp.main = Q4Ptrs{experts->down.q, experts->down.scale, experts->down.bias};
    tp.last = has_shared ? Q4Ptrs{shared->down.q, shared->down.scale, shared->down.bias} : tp.main;
    tp.N = D;
    tp.K = F;
    tp.C = y;
    tp.ldc = D;
    tp.c_perm = 0;
    if (wide) launch_wide(tp, false, tbound, stream);
    else launch_tiled(tp, false, tbound, stream);
    mark(4);
    launch_combine(y, (int64_t)T * k, slot_row, wts,
                   has_shared ? y + (int64_t)T * k * D : nullptr, out, T, D, k, stream);
    mark(5);
    return launch_status();
  }

  if (plan.eng == ENG_RESIDENT) {
    // gate_up + SwiGLU over the prepared x rows gathered through sorted_tok -> act, stored
    // in the prepared column order so that the down GEMM reads it as is
    ResidentParams rp;
    memset(&rp, 0, sizeof(rp));
    rp.A = at<uint16_t>(ws, L.xprep);
    rp.a_row_index = sorted_tok;
    rp.a_rows = T;
    rp.main = Q4Ptrs{experts->gate_up.q, experts->gate_up.scale, experts->gate_up.bias};
    rp.n_main = E;
    rp.last = has_shared ? Q4Ptrs{shared->gate_up.q, shared->gate_up.scale, shared->gate_up.bias}
                         : rp.main;
    rp.N = 2 * F;
    rp.K = D;
    rp.C = act;
    rp.ldc = F;
    rp.c_perm = 1;
    rp.tiles = tiles;
    rp.tile_count = tile_count;
    launch_resident(rp, rp_up, true, stream);
    mark(3);
    // down: act rows in order -> y [rows, D]
    rp.A = act;
    rp.a_row_index = nullptr;
    rp.a_rows = rows;
    rp.main = Q4Ptrs{experts->down.q, experts->down.scale, experts->down.bias};
    rp.last = has_shared ? Q4Ptrs{shared->down.q, shared->down.scale, shared->down.bias} : rp.main;
    rp.N = D;
    rp.K = F;
    rp.C = y;
    rp.ldc = D;
    rp.c_perm = 0;
    launch_resident(rp, rp_down, false, stream);
    mark(4);
    launch_combine(y, (int64_t)T * k, slot_row, wts,
                   has_shared ? y + (int64_t)T * k * D : nullptr, out, T, D, k, stream);
    mark(5);
    return launch_status();
  }

  if (plan.eng == ENG_STREAM) {
    // gate_up + SwiGLU over the prepared x rows gathered through sorted_tok -> act (stored
    // in the prepared column order, with its own (-136 X, X) rows for the down GEMM)
    StreamParams sp;
    memset(&sp, 0, sizeof(sp));
    sp.A = at<uint16_t>(ws, L.xprep);
    sp.xc = at<float4>(ws, L.xc_x);
    sp.a_row_index = sorted_tok;
    sp.a_rows = T;
    sp.main = Q4Ptrs{experts->gate_up.q, experts->gate_up.scale, experts->gate_up.bias};
    sp.n_main = E;
    sp.last = has_shared ? Q4Ptrs{shared->gate_up.q, shared->gate_up.scale, shared->gate_up.bias}
                         : sp.main;
    sp.N = 2 * F;
    sp.K = D;
    sp.C = act;
    sp.ldc = F;
    sp.c_perm = 1;
    sp.xc_out = at<float4>(ws, L.xc_act);
    sp.xc_out_ld = F / 128;
    sp.tiles = tiles;
    sp.tile_count = tile_count;
    run_stream(sp, plan, true, rows, n_groups, stream);
    mark(3);
    // down: act rows in order -> y [rows, D]
    sp.A = act;
    sp.xc = at<float4>(ws, L.xc_act);
    sp.a_row_index = nullptr;
    sp.a_rows = rows;
    sp.main = Q4Ptrs{experts->down.q, experts->down.scale, experts->down.bias};
    sp.last = has_shared ? Q4Ptrs{shared->down.q, shared->down.scale, shared->down.bias} : sp.main;
    sp.N = D;
    sp.K = F;
    sp.C = y;
    sp.ldc = D;
    sp.c_perm = 0;
    sp.xc_out = nullptr;
    run_stream(sp, plan, false, rows, n_groups, stream);
    mark(4);
    launch_combine(y, (int64_t)T * k, slot_row, wts,
                   has_shared ? y + (int64_t)T * k * D : nullptr, out, T, D, k, stream);
    mark(5);
    return launch_status();
  }

  // gate_up + SwiGLU: x rows gathered through sorted_tok -> act [rows, F]
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.A = x;
  p.a_row_index = sorted_tok;
  p.a_rows = T;
  p.main = Q4Ptrs{experts->gate_up.q, experts->gate_up.scale, experts->gate_up.bias};
  p.n_main = E;
  p.last = has_shared ? Q4Ptrs{shared->gate_up.q, shared->gate_up.scale, shared->gate_up.bias}
                      : p.main;
  p.N = 2 * F;
  p.K = D;
  p.C = act;
  p.ldc = F;
  p.tiles = tiles;
  p.tile_count = tile_count;
  p.xsum = xsum_x;          // gathered through sorted_tok like the rows of x
  p.xsum_ld = D / 64;
  p.xsum_out = xsum_act;    // row sums of act for the down GEMM
  p.xsum_out_ld = F / 64;
  run_gemm(p, plan, true, rows, n_groups, stream);
  mark(3);

  // down: act rows in order -> y [rows, D]
  p.A = act;
  p.a_row_index = nullptr;
  p.a_rows = rows;
  p.main = Q4Ptrs{experts->down.q, experts->down.scale, experts->down.bias};
  p.last = has_shared ? Q4Ptrs{shared->down.q, shared->down.scale, shared->down.bias} : p.main;
  p.N = D;
  p.K = F;
  p.C = y;
  p.ldc = D;
  p.xsum = xsum_act;
  p.xsum_ld = F / 64;
  p.xsum_out = nullptr;
  run_gemm(p, plan, false, rows, n_groups, stream);
  mark(4);

  // combine with the shared expert (rows T*k.. of y)
  launch_combine(y, (int64_t)T * k, slot_row, wts, has_shared ? y + (int64_t)T * k * D : nullptr,
                 out, T, D, k, stream);
  mark(5);
  return launch_status();
}

moe_status moe_layer_forward(const moe_shape* shape, const uint16_t* x, const float* router_w,
                             const moe_q4_ffn* experts, const moe_q4_ffn* shared, uint16_t* out,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_impl(shape, x, router_w, experts, shared, out, ws, ws_bytes, nullptr, stream);
}

moe_status moe_layer_forward_events(const moe_shape* shape, const uint16_t* x,
                                    const float* router_w, const moe_q4_ffn* experts,
                                    const moe_q4_ffn* shared, uint16_t* out, void* ws,
                                    size_t ws_bytes, hipEvent_t* events, hipStream_t stream) {
  return layer_impl(shape, x, router_w, experts, shared, out, ws, ws_bytes, events, stream);
}

}  // extern "C"
