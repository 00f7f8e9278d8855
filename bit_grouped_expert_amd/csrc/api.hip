// C ABI of libmoeq4: host-side validation, workspace carving and launches.
// Every entry point validates on the host before it enqueues anything, then
// enqueues its kernels on the caller's stream and returns without waiting.  Nothing
// here keeps state between calls: every decision is a function of the arguments and of
// the current device's compute-unit count.
#include <string.h>

#include <mutex>

#include "../../include/moeq4.h"
#include "internal.h"

using namespace moeq4;

namespace {

constexpr size_t kAlign = 256;
constexpr float kRefineGap = 1e-4f;
// average rows per group from which the wide-tile engine is the automatic choice.
// Measured on the layer's gate_up shape (N 1024, K 2048, 257 groups) with the same row
// count in every group: resident tiles are faster up to 32 rows per group (32: 118 against
// 149 us), wide tiles from 48 on (48: 170 against 194 us; 64: 188 against 211; 128: 284
// against 429).
constexpr int64_t kWideMinAvgRows = 40;

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

// The grouped-GEMM engines:
//   resident: tiles of up to 32 rows whose activations stay in LDS for the whole K while
//             the weights stream through VGPRs (K % 256 == 0, K <= 2048, N a multiple of
//             the chunk); the automatic choice for small groups;
//   wide:     tiles of 128 rows, each packed weight word feeding eight row fragments, the
//             activations through two LDS stage buffers (K % 256 == 0, K <= 2048,
//             N % 256 == 0); the automatic choice when groups average at least 192 rows;
//   grouped:  register-prefetched tiles of 32 rows for every shape (N % 64, K % 64); the
//             automatic choice where neither of the others can take the shape.
enum Engine { ENG_GROUPED, ENG_RESIDENT, ENG_WIDE };
struct GemmPlan {
  Engine eng;
  int bm;  // rows per tile of the tile map
};

// false when `forced` names an engine that cannot take the shape
bool plan_gemm(int32_t forced, int64_t rows, int n_groups, bool resident_ok, bool wide_ok,
               GemmPlan* out) {
  const int64_t g = n_groups > 0 ? n_groups : 1;
  switch (forced) {
    case MOE_ENGINE_GROUPED: *out = GemmPlan{ENG_GROUPED, kGroupedBM}; return true;
    case MOE_ENGINE_RESIDENT: *out = GemmPlan{ENG_RESIDENT, kResidentBM}; return resident_ok;
    case MOE_ENGINE_WIDE: *out = GemmPlan{ENG_WIDE, kWideBM}; return wide_ok;
    default: break;
  }
  if (wide_ok && rows >= kWideMinAvgRows * g) *out = GemmPlan{ENG_WIDE, kWideBM};
  else if (resident_ok) *out = GemmPlan{ENG_RESIDENT, kResidentBM};
  else *out = GemmPlan{ENG_GROUPED, kGroupedBM};
  return true;
}

bool engine_valid(int32_t e) { return e >= MOE_ENGINE_AUTO && e <= MOE_ENGINE_WIDE; }
bool layer_engine_valid(int32_t e) { return e >= MOE_ENGINE_AUTO && e <= MOE_ENGINE_DECODE; }

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

struct Layout {
  size_t rsplit, logits, topk_idx, topk_w, chunk_cnt, offsets, sorted_tok, slot_row, tiles,
      tile_count, xsum_x, xsum_act, xprep, act, y, sync, dec_part, dec_act, dec_plan, total;
  int32_t sync_words;  // cleared by the routing kernels of every call
};

// slots of the decode-sized chain: the distinct touched experts and the shared expert
int64_t decode_max_slots(const moe_shape* s) {
  const int64_t pairs = (int64_t)s->T * s->top_k;
  return (pairs < s->n_experts ? pairs : s->n_experts) + 1;
}
bool decode_ok(const moe_shape* s) {
  return decode_supported(s->T, s->d_model, s->n_experts, s->top_k, s->d_ff) &&
         router_small_ok(s->T, s->d_model);
}

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
  L.tiles = take((size_t)max_tiles(rows_ext, (int)E + 1, kResidentBM) * sizeof(int4));
  L.tile_count = take(16);
  L.xsum_x = take(T * (D / 64) * 4);
  L.xsum_act = take(rows_ext * (F / 64) * 4);
  L.xprep = take((T + 1) * D * 2);  // prepared x, one zero row after the last
  L.act = take((rows_ext + 1) * F * 2);
  L.y = take(rows_ext * D * 2);
  // the persistent launches' error word ([0]) and counters: the decode-sized chain's, or
  // one per tile of the resident pair launch
  int64_t words = kPairTileBase + max_tiles(rows_ext, (int)E + 1, kResidentBM);
  if (decode_ok(s)) {
    const int64_t dw = decode_sync_ints((int)D, (int)F, (int)decode_max_slots(s));
    words = dw > words ? dw : words;
  }
  L.sync_words = (int32_t)words;
  L.sync = take((size_t)words * 4);
  L.dec_part = L.dec_act = L.dec_plan = 0;
  if (decode_ok(s)) {
    const int ms = (int)decode_max_slots(s);
    L.dec_part = take(decode_part_bytes((int)D, (int)F, ms));
    L.dec_act = take(decode_act_bytes((int)F, ms));
    L.dec_plan = take(decode_plan_bytes());
  }
  L.total = o;
  return L;
}

bool q4_ok(const moe_q4& w) { return w.q && w.scale && w.bias; }
bool q4_aligned(const moe_q4& w) {
  return aligned16(w.q) && aligned16(w.scale) && aligned16(w.bias);
}
Q4Ptrs q4p(const moe_q4& w) { return Q4Ptrs{w.q, w.scale, w.bias}; }

moe_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

struct GemmWs {
  size_t tiles, tile_count, xsum, aprep, total;
};
GemmWs gemm_ws(int32_t n_groups, int32_t rows_total, int32_t a_rows, int32_t K) {
  GemmWs w;
  w.tiles = 0;
  w.tile_count = align_up((size_t)max_tiles(rows_total, n_groups, kResidentBM) * sizeof(int4));
  w.xsum = w.tile_count + kAlign;
  w.aprep = w.xsum + align_up((size_t)a_rows * (size_t)(K / 64) * 4);
  // the prepared copy of A (resident and wide engines), one zero row after the last
  w.total = w.aprep + align_up(((size_t)a_rows + 1) * (size_t)K * 2);
  return w;
}

// One grouped GEMM over an already-built tile map, with the plan's engine.  A is the
// prepared copy for the resident and wide engines and the plain rows (with their per-64
// row sums in xsum) for the grouped engine.
struct GemmCall {
  const uint16_t* A;
  const int32_t* a_row_index;
  int32_t a_rows;
  Q4Ptrs main;
  int32_t n_main;
  Q4Ptrs last;
  int32_t N, K;
  uint16_t* C;
  int32_t ldc;
  int32_t c_perm;       // resident and wide: store a SwiGLU output in the prepared order
  const float* xsum;    // grouped: row sums of A per 64
  float* xsum_out;      // grouped with SwiGLU: row sums of C per 64 (nullable)
  const int4* tiles;
  const int32_t* tile_count;
};

ResidentParams resident_params(const GemmCall& c) {
  ResidentParams p;
  memset(&p, 0, sizeof(p));
  p.A = c.A;
  p.a_row_index = c.a_row_index;
  p.a_rows = c.a_rows;
  p.main = c.main;
  p.n_main = c.n_main;
  p.last = c.last;
  p.N = c.N;
  p.K = c.K;
  p.C = c.C;
  p.ldc = c.ldc;
  p.c_perm = c.c_perm;
  p.tiles = c.tiles;
  p.tile_count = c.tile_count;
  return p;
}

void run_gemm(const GemmCall& c, const GemmPlan& plan, const ResidentPlan& rplan, bool swiglu,
              int64_t rows, int n_groups, int n_cu, hipStream_t stream) {
  const int64_t bound = max_tiles(rows, n_groups, plan.bm);
  if (plan.eng == ENG_WIDE) {
    WideParams p;
    memset(&p, 0, sizeof(p));
    p.A = c.A;
    p.a_row_index = c.a_row_index;
    p.a_rows = c.a_rows;
    p.main = c.main;
    p.n_main = c.n_main;
    p.last = c.last;
    p.N = c.N;
    p.K = c.K;
    p.C = c.C;
    p.ldc = c.ldc;
    p.c_perm = c.c_perm;
    p.tiles = c.tiles;
    p.tile_count = c.tile_count;
    launch_wide(p, swiglu, bound, n_cu, stream);
  } else if (plan.eng == ENG_RESIDENT) {
    launch_resident(resident_params(c), rplan, swiglu, stream);
  } else {
    GemmParams p;
    memset(&p, 0, sizeof(p));
    p.A = c.A;
    p.a_row_index = c.a_row_index;
    p.a_rows = c.a_rows;
    p.main = c.main;
    p.n_main = c.n_main;
    p.last = c.last;
    p.N = c.N;
    p.K = c.K;
    p.C = c.C;
    p.ldc = c.ldc;
    p.tiles = c.tiles;
    p.tile_count = c.tile_count;
    p.xsum = c.xsum;
    p.xsum_ld = c.K / 64;
    p.xsum_out = c.xsum_out;
    p.xsum_out_ld = c.N / 2 / 64;
    launch_grouped(p, swiglu, bound, n_cu, stream);
  }
}

// ---- scratch of moe_layer_forward_noalloc: a static device array (each GPU the library
// runs on holds its own copy until the process ends).  In host code `scratch` is only a
// stand-in for the symbol; its device address on the current device comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed to kernels.
constexpr size_t kNoallocScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];  // set once per device, then only read

// The current device's address of `scratch` (taken on the first call on that device, with
// that device current).
moe_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_DEVICE;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot]() {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    slot.ptr = slot.err == hipSuccess ? p : nullptr;
  });
  if (slot.err != hipSuccess || !slot.ptr) return MOE_ERR_DEVICE;
  *out = slot.ptr;
  return MOE_OK;
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
  layout->sync = L.sync;
  layout->total = L.total;
  return MOE_OK;
}

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
  launch_topk(logits, x, router_w, T, D, E, k, gap, topk_idx, topk_w, nullptr, 0, stream);
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
static void permute_chunked(const moe_shape* shape, const int32_t* topk_idx, int32_t* offsets,
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
    permute_chunked(shape, topk_idx, offsets, sorted_tok, slot_row, at<int32_t>(ws, L.chunk_cnt),
                    -1, stream);
  return launch_status();
}

moe_status moe_grouped_gemm_q4_ex(int32_t n_groups, int32_t rows_total, int32_t N, int32_t K,
                                  const uint16_t* A, int32_t a_rows, const int32_t* a_row_index,
                                  const int32_t* offsets, moe_q4 W, int32_t epilogue, uint16_t* C,
                                  void* ws, size_t ws_bytes, int32_t engine, hipStream_t stream) {
  if (n_groups < 1 || n_groups > kMaxTileGroups || rows_total < 0 || a_rows < 0 || N <= 0 ||
      K <= 0 || N % 64 || K % 64 || (epilogue != 0 && epilogue != 1) || !engine_valid(engine))
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

  const bool swiglu = epilogue == 1;
  const int n_cu = device_cu_count();
  ResidentPlan rplan;
  memset(&rplan, 0, sizeof(rplan));
  const bool resident_ok =
      a_rows >= 1 &&
      resident_plan(N, K, swiglu, max_tiles(rows_total, n_groups, kResidentBM), n_cu, &rplan);
  const bool wide_ok = wide_supported(N, K, swiglu, a_rows);
  GemmPlan plan;
  if (!plan_gemm(engine, rows_total, n_groups, resident_ok, wide_ok, &plan)) return MOE_ERR_SHAPE;
  int4* tiles = at<int4>(ws, gw.tiles);
  int32_t* tile_count = at<int32_t>(ws, gw.tile_count);
  launch_build_tiles(offsets, n_groups, rows_total, plan.bm, tiles, tile_count, stream);
  GemmCall c;
  memset(&c, 0, sizeof(c));
  c.a_row_index = a_row_index;
  c.a_rows = a_rows;
  c.main = q4p(W);
  c.n_main = n_groups;
  c.last = c.main;
  c.N = N;
  c.K = K;
  c.C = C;
  c.ldc = swiglu ? N / 2 : N;
  c.tiles = tiles;
  c.tile_count = tile_count;
  if (plan.eng == ENG_GROUPED) {
    float* xsum = at<float>(ws, gw.xsum);
    launch_row_group_sums(A, a_rows, K, xsum, stream);
    c.A = A;
    c.xsum = xsum;
  } else {
    uint16_t* aprep = at<uint16_t>(ws, gw.aprep);
    launch_prep(A, a_rows, K, aprep, stream);
    c.A = aprep;
  }
  run_gemm(c, plan, rplan, swiglu, rows_total, n_groups, n_cu, stream);
  return launch_status();
}

moe_status moe_grouped_gemm_q4(int32_t n_groups, int32_t rows_total, int32_t N, int32_t K,
                               const uint16_t* A, int32_t a_rows, const int32_t* a_row_index,
                               const int32_t* offsets, moe_q4 W, int32_t epilogue, uint16_t* C,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_grouped_gemm_q4_ex(n_groups, rows_total, N, K, A, a_rows, a_row_index, offsets, W,
                                epilogue, C, ws, ws_bytes, MOE_ENGINE_AUTO, stream);
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

// The grouped GEMMs of a prefill-sized layer: the engine (from the shapes and the average
// group size, or forced), the resident plans, and whether gate_up and down run as one
// launch.  False when a forced engine cannot take the shapes.
struct LayerGemmPlan {
  GemmPlan plan;
  ResidentPlan rp_up, rp_down;
  bool paired;
};
bool plan_layer_gemms(const moe_shape* s, bool has_shared, int32_t engine, int n_cu,
                      LayerGemmPlan* out) {
  const int T = s->T, D = s->d_model, E = s->n_experts, k = s->top_k, F = s->d_ff;
  const int n_groups = E + (has_shared ? 1 : 0);
  const int rows = T * k + (has_shared ? T : 0);
  const int64_t rbound = max_tiles(rows, n_groups, kResidentBM);
  memset(out, 0, sizeof(*out));
  const bool resident_ok = resident_plan(2 * F, D, true, rbound, n_cu, &out->rp_up) &&
                           resident_plan(D, F, false, rbound, n_cu, &out->rp_down);
  const bool wide_ok = wide_supported(2 * F, D, true, T) && wide_supported(D, F, false, rows);
  if (!plan_gemm(engine, rows, n_groups, resident_ok, wide_ok, &out->plan)) return false;
  out->paired = out->plan.eng == ENG_RESIDENT &&
                resident_pair_ok(out->rp_up, out->rp_down, 2 * F, D, D, F, rbound);
  return true;
}

// planes_ready: the workspace already holds the router's bf16 planes of router_w (a
// later chunk of moe_layer_forward_chunked)
static moe_status layer_impl(const moe_shape* shape, const uint16_t* x, const float* router_w,
                             const moe_q4_ffn* experts, const moe_q4_ffn* shared, uint16_t* out,
                             void* ws, size_t ws_bytes, const moe_layer_opts* opts,
                             hipStream_t stream, bool planes_ready = false) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const int32_t engine = opts ? opts->engine : MOE_ENGINE_AUTO;
  if (!layer_engine_valid(engine) || (opts && opts->reserved != 0)) return MOE_ERR_SHAPE;
  if (engine == MOE_ENGINE_DECODE && !decode_ok(shape)) return MOE_ERR_SHAPE;
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

  hipEvent_t* events = opts ? opts->events : nullptr;
  bool event_failed = false;
  auto mark = [&](int i) {
    if (events && events[i] && hipEventRecord(events[i], stream) != hipSuccess) event_failed = true;
  };
  auto finish = [&]() {
    const moe_status ls = launch_status();
    return ls != MOE_OK ? ls : (event_failed ? MOE_ERR_LAUNCH : MOE_OK);
  };

  if (engine == MOE_ENGINE_DECODE || (engine == MOE_ENGINE_AUTO && decode_ok(shape))) {
    // decode-sized chain: router logits (+ prepared x, + the counters cleared), then one
    // persistent launch: plan, gate_up + SwiGLU, down + combine
    int32_t* sync = at<int32_t>(ws, L.sync);
    mark(0);
    launch_router_small(x, router_w, at<float>(ws, L.logits), T, D, E, at<uint16_t>(ws, L.xprep),
                        sync, L.sync_words, stream);
    mark(1);
    mark(2);
    DecodeParams dp;
    memset(&dp, 0, sizeof(dp));
    dp.T = T;
    dp.D = D;
    dp.E = E;
    dp.k = k;
    dp.F = F;
    dp.has_shared = has_shared ? 1 : 0;
    dp.group_slots = decode_group_slots(F);
    dp.n_cb = D / 16;
    dp.tau = kRefineGap;
    dp.logits = at<float>(ws, L.logits);
    dp.x = x;
    dp.R = router_w;
    dp.xprep = at<uint16_t>(ws, L.xprep);
    dp.idx = at<int32_t>(ws, L.topk_idx);
    dp.w = at<float>(ws, L.topk_w);
    dp.offsets = at<int32_t>(ws, L.offsets);
    dp.sorted_tok = at<int32_t>(ws, L.sorted_tok);
    dp.slot_row = at<int32_t>(ws, L.slot_row);
    dp.sync = sync;
    dp.part = at<float>(ws, L.dec_part);
    dp.act = at<uint16_t>(ws, L.dec_act);
    dp.plan = at<uint32_t>(ws, L.dec_plan);
    // two workgroups per compute unit are resident at once: the later ones take the
    // plan workgroup 0 publishes
    dp.early = 2 * device_cu_count();
    dp.out = out;
    dp.up_main = q4p(experts->gate_up);
    dp.down_main = q4p(experts->down);
    dp.up_last = has_shared ? q4p(shared->gate_up) : dp.up_main;
    dp.down_last = has_shared ? q4p(shared->down) : dp.down_main;
    launch_decode_layer(dp, (int)decode_max_slots(shape) - (has_shared ? 0 : 1), stream);
    mark(3);
    mark(4);
    mark(5);
    return finish();
  }

  // the GEMM engine depends only on the shapes: chosen first, so that the router can
  // write the prepared copy of x on the way
  const int n_cu = device_cu_count();
  LayerGemmPlan lp;
  if (!plan_layer_gemms(shape, has_shared, engine, n_cu, &lp)) return MOE_ERR_SHAPE;
  const GemmPlan plan = lp.plan;
  const ResidentPlan rp_up = lp.rp_up, rp_down = lp.rp_down;
  const bool prepared = plan.eng != ENG_GROUPED;

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
  uint16_t* xprep = at<uint16_t>(ws, L.xprep);

  // routing (the router also writes the prepared copy of x)
  mark(0);
  launch_router(x, router_w, at<uint16_t>(ws, L.rsplit), at<float>(ws, L.logits), T, D, E,
                prepared ? xprep : nullptr, stream, planes_ready);
  int32_t* sync = at<int32_t>(ws, L.sync);
  const bool pair = lp.paired;
  launch_topk(at<float>(ws, L.logits), x, router_w, T, D, E, k, kRefineGap, idx, wts, sync,
              L.sync_words, stream);
  mark(1);
  // histogram, scan, scatter (+ identity rows of the shared group), tile map
  const int shared_rows = has_shared ? T : -1;
  if (permute_experts_ok(T, k, E))
    launch_permute_experts(idx, T, k, E, offsets, sorted_tok, slot_row, shared_rows, plan.bm, tiles,
                           tile_count, stream);
  else if (permute_small_ok(T, E))
    launch_permute_small(idx, T, k, E, offsets, sorted_tok, slot_row, shared_rows, plan.bm, tiles,
                         tile_count, stream);
  else
    permute_chunked(shape, idx, offsets, sorted_tok, slot_row, at<int32_t>(ws, L.chunk_cnt),
                    shared_rows, stream, tiles, tile_count, rows, plan.bm);
  if (!prepared) launch_row_group_sums(x, T, D, xsum_x, stream);
  mark(2);

  // gate_up + SwiGLU over the x rows gathered through sorted_tok -> act [rows, F]; the
  // resident and wide engines read the prepared x and store act in the prepared order,
  // so that the down GEMM reads it as is
  GemmCall c;
  memset(&c, 0, sizeof(c));
  c.A = prepared ? xprep : x;
  c.a_row_index = sorted_tok;
  c.a_rows = T;
  c.main = q4p(experts->gate_up);
  c.n_main = E;
  c.last = has_shared ? q4p(shared->gate_up) : c.main;
  c.N = 2 * F;
  c.K = D;
  c.C = act;
  c.ldc = F;
  c.c_perm = prepared ? 1 : 0;
  c.xsum = xsum_x;        // grouped: gathered through sorted_tok like the rows of x
  c.xsum_out = xsum_act;  // grouped: row sums of act for the down GEMM
  c.tiles = tiles;
  c.tile_count = tile_count;
  GemmCall cu = c;

  // down: act rows in order -> y [rows, D]
  c.A = act;
  c.a_row_index = nullptr;
  c.a_rows = rows;
  c.main = q4p(experts->down);
  c.last = has_shared ? q4p(shared->down) : c.main;
  c.N = D;
  c.K = F;
  c.C = y;
  c.ldc = D;
  c.c_perm = 0;
  c.xsum = xsum_act;
  c.xsum_out = nullptr;
  if (pair) {
    // both GEMMs in one launch (each workgroup's down share starts when its gate_up share
    // is done); the counters it waits on were cleared by the top-k launch
    launch_resident_pair(resident_params(cu), resident_params(c), rp_up, rp_down, sync, stream);
    mark(3);
  } else {
    run_gemm(cu, plan, rp_up, true, rows, n_groups, n_cu, stream);
    mark(3);
    run_gemm(c, plan, rp_down, false, rows, n_groups, n_cu, stream);
  }
  mark(4);

  // combine with the shared expert (rows T*k.. of y)
  launch_combine(y, (int64_t)T * k, slot_row, wts, has_shared ? y + (int64_t)T * k * D : nullptr,
                 out, T, D, k, stream);
  mark(5);
  return finish();
}

moe_status moe_layer_plan(const moe_shape* shape, int32_t engine, int32_t has_shared,
                          moe_layer_plan_info* info) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!info) return MOE_ERR_NULL;
  if (!layer_engine_valid(engine)) return MOE_ERR_SHAPE;
  if (engine == MOE_ENGINE_DECODE && !decode_ok(shape)) return MOE_ERR_SHAPE;
  memset(info, 0, sizeof(*info));
  if (engine == MOE_ENGINE_DECODE || (engine == MOE_ENGINE_AUTO && decode_ok(shape))) {
    info->gemm_engine = MOE_ENGINE_DECODE;
    return MOE_OK;
  }
  LayerGemmPlan lp;
  if (!plan_layer_gemms(shape, has_shared != 0, engine, device_cu_count(), &lp)) return MOE_ERR_SHAPE;
  info->gemm_engine = lp.plan.eng == ENG_WIDE       ? MOE_ENGINE_WIDE
                      : lp.plan.eng == ENG_RESIDENT ? MOE_ENGINE_RESIDENT
                                                    : MOE_ENGINE_GROUPED;
  info->paired = lp.paired ? 1 : 0;
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_shape* shape, const uint16_t* x, const float* router_w,
                             const moe_q4_ffn* experts, const moe_q4_ffn* shared, uint16_t* out,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_impl(shape, x, router_w, experts, shared, out, ws, ws_bytes, nullptr, stream);
}

moe_status moe_layer_forward_ex(const moe_shape* shape, const uint16_t* x, const float* router_w,
                                const moe_q4_ffn* experts, const moe_q4_ffn* shared, uint16_t* out,
                                void* ws, size_t ws_bytes, const moe_layer_opts* opts,
                                hipStream_t stream) {
  return layer_impl(shape, x, router_w, experts, shared, out, ws, ws_bytes, opts, stream);
}

moe_status moe_layer_forward_noalloc(const moe_shape* shape, const uint16_t* x,
                                     const float* router_w, const moe_q4_ffn* experts,
                                     const moe_q4_ffn* shared, uint16_t* out, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->T == 0) return MOE_OK;
  if (make_layout(shape).total > kNoallocScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != MOE_OK) return st;
  // nothing in the layer's workspace has to start at zero: every kernel writes what a later
  // one reads (the prepared copy of x and its zero row included) before it is read
  return layer_impl(shape, x, router_w, experts, shared, out, ws, kNoallocScratchBytes, nullptr,
                    stream);
}

size_t moe_chunked_workspace_bytes(const moe_shape* shape, int32_t chunk_tokens) {
  if (check_shape(shape) != MOE_OK || chunk_tokens < 1) return 0;
  moe_shape c = *shape;
  c.T = shape->T < chunk_tokens ? shape->T : chunk_tokens;
  return make_layout(&c).total;
}

moe_status moe_layer_forward_chunked(const moe_shape* shape, const uint16_t* x,
                                     const float* router_w, const moe_q4_ffn* experts,
                                     const moe_q4_ffn* shared, uint16_t* out, int32_t chunk_tokens,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (chunk_tokens < 1) return MOE_ERR_SHAPE;
  if (shape->T == 0) return MOE_OK;
  // every chunk's checks are those of the first (the layout grows with T), so a failure
  // is reported before anything is enqueued
  moe_shape c = *shape;
  c.T = shape->T < chunk_tokens ? shape->T : chunk_tokens;
  if (ws_bytes < make_layout(&c).total) return MOE_ERR_WORKSPACE;
  const int64_t D = shape->d_model;
  // the router's bf16 planes sit at the start of every chunk's layout: a chunk after one
  // that split R reuses them
  bool planes = false;
  for (int64_t t0 = 0; t0 < shape->T; t0 += chunk_tokens) {
    c.T = (int32_t)(shape->T - t0 < chunk_tokens ? shape->T - t0 : chunk_tokens);
    st = layer_impl(&c, x + t0 * D, router_w, experts, shared, out + t0 * D, ws, ws_bytes, nullptr,
                    stream, planes);
    if (st != MOE_OK) return st;
    planes = planes || router_uses_planes(c.T, c.d_model);
  }
  return MOE_OK;
}


size_t moe_gqa_decode_workspace_bytes(const moe_gqa_shape* s) {
  if (!s || !attn_supported(s->n_q_heads, s->n_kv_heads, s->head_dim, s->ctx_len, s->kv_stride))
    return 0;
  return attn_workspace_bytes(s->n_q_heads, s->n_kv_heads, s->ctx_len);
}

moe_status moe_gqa_decode_attention(const moe_gqa_shape* s, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!s) return MOE_ERR_NULL;
  if (!attn_supported(s->n_q_heads, s->n_kv_heads, s->head_dim, s->ctx_len, s->kv_stride))
    return MOE_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !out || !ws) return MOE_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(ws))
    return MOE_ERR_ALIGN;
  if (ws_bytes < attn_workspace_bytes(s->n_q_heads, s->n_kv_heads, s->ctx_len))
    return MOE_ERR_WORKSPACE;
  AttnParams p;
  p.n_q = s->n_q_heads;
  p.n_kv = s->n_kv_heads;
  p.group = s->n_q_heads / s->n_kv_heads;
  p.ctx = s->ctx_len;
  p.n_chunks = attn_chunks(s->ctx_len);
  p.kv_stride = s->kv_stride;
  p.scale = 1.0f / sqrtf((float)s->head_dim);
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  attn_partition(&p, device_cu_count());
  p.part_o = (float*)ws;
  p.part_ml = p.part_o + (size_t)p.n_kv * p.n_chunks * p.group * kAttnHeadDim;
  p.out = out;
  launch_attention(p, stream);
  return launch_status();
}

}  // extern "C"
