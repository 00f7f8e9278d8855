/*
 * moeq4.h -- C ABI of an MI355X (gfx950) mixture-of-experts layer with
 * groupwise-affine 4-bit expert weights.
 *
 * Pages the operations follow (cited by title and section):
 *   [MTP] MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference
 *         engine for Qwen3.6-35B-A3B on Apple Silicon", body paragraphs 4-7.
 *   [GF]  globalfeed.ai, "Perplexity open sources Lily, a Rust and Metal
 *         inference engine for Apple Silicon", sections "Requirements and model
 *         layout" and "Measurements".
 *
 * Conventions shared by every entry point
 *   - All tensors are row-major.  bf16 values travel as their raw uint16 bits.
 *   - Pointers are device pointers (hipMalloc / torch CUDA tensors) unless a
 *     comment says otherwise; the caller owns every buffer.  The library
 *     allocates nothing, keeps no pointer after a call returns and has no
 *     mutable global state (every launch decision is a function of the
 *     arguments and of the current device; the one exception is the device
 *     address of moe_layer_forward_noalloc's scratch array, taken once per
 *     device under std::call_once), so calls on different streams with
 *     different buffers are thread-safe.
 *   - Kernels whose workgroups wait on other workgroups (the paired GEMM launch,
 *     the decode-sized chain) bound every wait.  Work on other streams can only
 *     delay such a wait.  One that outlasts its bound (milliseconds) gives up:
 *     a decode-chain workgroup waiting for the published routing plan then
 *     computes the plan itself; any other such wait is counted in word 0 of the
 *     workspace's sync counters (moe_ws_layout.sync), and that call's output is
 *     not to be trusted.
 *   - Every compute call only enqueues work on `stream` (NULL = the legacy
 *     default stream) and never waits for the device; buffers must stay valid
 *     until the stream has passed the call.  No host synchronisation happens
 *     inside a call ([MTP] para. 6: routing stays on the GPU with no CPU sync
 *     inside the MoE layer).  No call enqueues a memset, so every compute call
 *     may be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     nonzero status means nothing was enqueued.  MOE_ERR_LAUNCH reports a
 *     launch failure seen by hipGetLastError (kernels already enqueued by the
 *     same call may still run).  Faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - Outputs must not alias inputs.  NaN/Inf inputs give unspecified results.
 *   - Required alignment: 16 bytes for every pointer.
 *
 * Weight format ([MTP] para. 5; [GF] "Requirements and model layout": 4-bit
 * weights, every group of 64 sharing one bf16 scale and one bf16 bias):
 *   A weight matrix W has N output rows and K inputs (K % 64 == 0).
 *     q     uint32 [groups, N, K/8]   eight 4-bit codes per word; nibble j
 *                                      (bits 4j..4j+3) of word w is input 8w+j
 *     scale bf16   [groups, N, K/64]
 *     bias  bf16   [groups, N, K/64]
 *   w[n][c] = q[n][c] * scale[n][c/64] + bias[n][c/64]   (q unsigned, 0..15)
 *   An expert FFN is SwiGLU: gate_up has N = 2F (rows 0..F-1 gate, F..2F-1 up)
 *   and K = D; down has N = D and K = F.
 */
#ifndef MOEQ4_H
#define MOEQ4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t, hipEvent_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* a size is out of range, breaks a divisibility rule, or an
                            option names an engine that cannot take the shape */
  MOE_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 4, /* the workspace is NULL or smaller than required */
  MOE_ERR_LAUNCH = 5,    /* a kernel launch failed (hipGetLastError) */
  MOE_ERR_DEVICE = 6     /* no usable gfx950 device / device query failed */
} moe_status;

/* Layer shape.  T tokens, D = d_model, E routed experts, k experts per token,
 * F = expert d_ff.  Rules: 0 <= T; D % 64 == 0; F % 64 == 0; 1 <= E <= 1024;
 * 1 <= k <= min(E, 32); (k+1) * T * max(D, 2F) < 2^31.
 * [MTP] para. 4 and [GF] "Requirements and model layout": 256 routed experts of
 * which eight are picked per token, plus one shared expert. */
typedef struct {
  int32_t T, d_model, n_experts, top_k, d_ff;
} moe_shape;

/* One packed 4-bit weight tensor (format above; [MTP] para. 5). */
typedef struct {
  const uint32_t* q;
  const uint16_t* scale;
  const uint16_t* bias;
} moe_q4;

/* The weights of a set of SwiGLU experts, stored contiguously group after group
 * ([MTP] para. 5: the expert weights of the model are 4-bit groupwise affine). */
typedef struct {
  moe_q4 gate_up; /* N = 2F, K = D */
  moe_q4 down;    /* N = D,  K = F */
} moe_q4_ffn;

/* Grouped-GEMM engine.  All compute the same result (see moe_grouped_gemm_q4); they
 * differ in how rows and weights are tiled ([MTP] para. 6: the expert GEMMs walk tiles
 * of expert rows through a block map).  AUTO picks from the shapes and the average
 * group size; a forced engine that cannot take the shape gives MOE_ERR_SHAPE. */
typedef enum {
  MOE_ENGINE_AUTO = 0,
  MOE_ENGINE_GROUPED = 1,  /* any N % 64, K % 64: tiles of up to 32 rows */
  MOE_ENGINE_RESIDENT = 2, /* K % 256 == 0, K <= 2048: tiles of up to 32 rows held in LDS
                              over the whole K while the weights stream (small groups); in
                              the layer calls gate_up and down run as one launch where
                              moe_layer_plan reports paired */
  MOE_ENGINE_WIDE = 3,     /* K % 256 == 0, K <= 2048, N % 256 == 0: tiles of up to 128
                              rows (large groups) */
  MOE_ENGINE_DECODE = 4    /* moe_layer_forward_ex only: the decode-sized chain (T <= 16,
                              T * k <= 128, E <= 1024, d_model % 256 == 0, d_model <= 2048,
                              d_ff <= 1024; the automatic choice there): the router, then
                              one persistent launch (plan, gate_up, down fused with the
                              combine); no permuted rows */
} moe_engine;

/* Options of moe_layer_forward_ex.  A NULL options pointer equals all fields zero. */
#define MOE_N_STAGE_EVENTS 6
typedef struct {
  int32_t engine;     /* moe_engine used by both grouped GEMMs */
  int32_t reserved;   /* must be 0 */
  hipEvent_t* events; /* NULL, or MOE_N_STAGE_EVENTS caller-created events (entries may be
                         NULL) recorded on `stream`: [0] before routing, [1] after routing
                         (logits, top-k), [2] after the permutation and tile map, [3] after
                         the grouped gate_up + SwiGLU, [4] after the grouped down, [5] after
                         the combine; when the two GEMMs run as one launch (moe_layer_plan's
                         paired), [3] and [4] both follow it */
} moe_layer_opts;

/* Byte offsets of the intermediates moe_layer_forward leaves in its workspace
 * (valid after the stream has passed the call, until the workspace is reused). */
typedef struct {
  size_t topk_idx;   /* int32 [T, k]   selected experts, descending logit */
  size_t topk_w;     /* fp32  [T, k]   routing weights */
  size_t offsets;    /* int32 [E + 2]  group row offsets; [E+1] = (k+1)T (shared group) */
  size_t sorted_tok; /* int32 [(k+1)T] token of each permuted row (tail: 0..T-1) */
  size_t slot_row;   /* int32 [T, k]   permuted row of pair (t, j) */
  size_t act;        /* bf16  [(k+1)T, F] SwiGLU activations, permuted rows (not written
                        by the decode-sized chain) */
  size_t y;          /* bf16  [(k+1)T, D] expert outputs; rows kT.. = shared expert (not
                        written by the decode-sized chain, which never stores them) */
  size_t sync;       /* int32 counters of the persistent launches (cleared by the call's
                        routing kernels); word 0 counts waits that gave up their bound,
                        and is 0 after every correct call */
  size_t total;      /* == moe_workspace_bytes */
} moe_ws_layout;

/* Human-readable name of a status (static string; never NULL). */
const char* moe_status_string(moe_status s);

/* Workspace bytes moe_layer_forward needs for `shape`; this also covers moe_route and
 * moe_permute.  Host-only, pure; 0 if the shape is invalid.  [MTP] para. 6: the
 * routing histogram, prefix scan, scatter and block map live in device memory that the
 * layer's own GPU work reads (here, the caller's workspace). */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Fills `layout` for `shape`.  Host-only.  Same passage as moe_workspace_bytes. */
moe_status moe_workspace_layout(const moe_shape* shape, moe_ws_layout* layout);

/* Workspace bytes moe_grouped_gemm_q4 needs (its tile map, the per-64 row sums of A and
 * a prepared copy of A).  Host-only, pure; 0 if the arguments are invalid.  [MTP]
 * para. 6: the grouped GEMM is driven by a block map of expert-row tiles. */
size_t moe_grouped_gemm_q4_workspace_bytes(int32_t n_groups, int32_t rows_total, int32_t a_rows,
                                           int32_t K);

/* Router: L = x R^T in fp32 (bf16 x split-exact against a three-way bf16 split
 * of R), top-k by descending logit with exact ties to the lower expert id;
 * when the k-th and (k+1)-th fp32 logits are closer than 1e-4 the logits of
 * every expert within 1e-4 of the boundary are recomputed exactly in fp64 and
 * the selection is redone.  Weights: softmax over the k selected logits.
 * [MTP] para. 4 (a router scores 256 experts and picks eight).
 *   x        bf16 [T, D];  router_w fp32 [E, D]
 *   topk_idx int32 [T, k] (descending logit);  topk_w fp32 [T, k]
 *   ws       >= moe_workspace_bytes(shape) bytes of scratch (caller-owned). */
moe_status moe_route(const moe_shape* shape, const uint16_t* x, const float* router_w,
                     int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* moe_route with an explicit near-tie threshold (moe_route uses 1e-4).  A larger
 * refine_gap sends more tokens through the exact fp64 rescoring (for testing);
 * refine_gap must be >= 0 (else MOE_ERR_SHAPE).  [MTP] para. 4. */
moe_status moe_route_ex(const moe_shape* shape, const uint16_t* x, const float* router_w,
                        int32_t* topk_idx, float* topk_w, float refine_gap, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* Histogram, exclusive prefix scan and stable scatter of the (token, slot)
 * pairs into contiguous per-expert groups ([MTP] paras. 4 and 6: uneven expert
 * groups; histogram, prefix scan and scatter stay on the GPU).
 *   topk_idx   int32 [T, k]; the k experts of a token must be distinct (else
 *              rows are unspecified, though always inside their group);
 *              entries outside [0, E) are ignored (their slot_row is set to -1
 *              and they are not counted)
 *   offsets    int32 [E + 1]: rows of expert e are offsets[e]..offsets[e+1]-1
 *   sorted_tok int32 [T*k]: token of each permuted row, ascending within a group
 *   slot_row   int32 [T*k]: slot_row[t*k + j] = permuted row of pair (t, j)
 *   ws         >= moe_workspace_bytes(shape) bytes.
 * With T == 0 only `offsets` (all zero) is written and the other arrays may be NULL. */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_idx, int32_t* offsets,
                       int32_t* sorted_tok, int32_t* slot_row, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Grouped GEMM over 4-bit weights ([MTP] para. 5: the 4-bit weights are
 * reconstructed tile by tile inside the grouped GEMM with fp32 accumulation,
 * never expanded in memory).  For each group g and row r in
 * offsets[g]..offsets[g+1]-1:
 *   H[r] = A[row(r)] W_g^T   (fp32),  row(r) = a_row_index ? a_row_index[r] : r
 *   epilogue 0: C[r][n] = bf16(H[r][n]),            C is [rows_total, N]
 *   epilogue 1: C[r][f] = bf16(silu(H[r][f]) * H[r][N/2 + f]), C is [rows_total, N/2]
 *   1 <= n_groups <= 1025;  N % 64 == 0;  K % 64 == 0;  rows_total >= 0
 *   A          bf16 [a_rows, K]; rows whose index is outside [0, a_rows) read as zero
 *   offsets    int32 [n_groups + 1] on the device, non-decreasing from 0;
 *              values are clamped to [0, rows_total]; C rows outside every
 *              group are not written
 *   W          q [n_groups, N, K/8], scale/bias [n_groups, N, K/64]
 *   ws         >= moe_grouped_gemm_q4_workspace_bytes(n_groups, rows_total, a_rows, K).
 * Arithmetic: no weight is rounded; each 64-wide group's partial sum is formed on
 * the matrix cores from the exact values 128 + q and scaled in fp32, and the bias
 * part (b - 128 s) X (X: the row's sum over the group) comes from exact products of
 * b, s and X (X split into three bf16 pieces that sum to it exactly, or X itself in
 * fp32), so H is the fp32-accumulated product with the exactly dequantized weights. */
moe_status moe_grouped_gemm_q4(int32_t n_groups, int32_t rows_total, int32_t N, int32_t K,
                               const uint16_t* A, int32_t a_rows, const int32_t* a_row_index,
                               const int32_t* offsets, moe_q4 W, int32_t epilogue,
                               uint16_t* C, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_grouped_gemm_q4 with an explicit engine (moe_engine; MOE_ENGINE_AUTO is what
 * moe_grouped_gemm_q4 uses).  Same results; an engine that cannot take the shape gives
 * MOE_ERR_SHAPE.  [MTP] para. 5 (in-GEMM dequantization) and para. 6 (tiles of expert
 * rows; 32-row tiles). */
moe_status moe_grouped_gemm_q4_ex(int32_t n_groups, int32_t rows_total, int32_t N, int32_t K,
                                  const uint16_t* A, int32_t a_rows, const int32_t* a_row_index,
                                  const int32_t* offsets, moe_q4 W, int32_t epilogue,
                                  uint16_t* C, void* ws, size_t ws_bytes, int32_t engine,
                                  hipStream_t stream);

/* Weighted combine: out[t] = bf16( S[t] + sum_j topk_w[t][j] * Y[slot_row[t*k+j]] ),
 * summed in fp32 (S = shared_out, or 0 when NULL).  slot_row entries outside
 * [0, T*k) are skipped.  [MTP] para. 4: each token's output joins its eight routed
 * experts and the shared expert that sees every token.
 *   y_sorted bf16 [T*k, D]; slot_row int32 [T*k]; topk_w fp32 [T*k];
 *   shared_out bf16 [T, D] or NULL; out bf16 [T, D]. */
moe_status moe_combine(const moe_shape* shape, const uint16_t* y_sorted, const int32_t* slot_row,
                       const float* topk_w, const uint16_t* shared_out, uint16_t* out,
                       hipStream_t stream);

/* The whole layer on one stream with no host synchronisation: route, permute,
 * grouped gate_up + SwiGLU over the E routed groups plus the shared expert as
 * one more group covering all T rows, grouped down, weighted combine.  [MTP] para. 6
 * (the routing stages stay in one GPU command stream with no CPU sync inside the MoE
 * layer; expert GEMMs are most of prefill) and paras. 4-5.
 *   x bf16 [T, D]; router_w fp32 [E, D];
 *   experts: E groups (q [E, 2F, D/8] ... as in the weight format);
 *   shared: one group, or NULL for no shared expert; out bf16 [T, D];
 *   ws >= moe_workspace_bytes(shape) bytes; its layout is moe_workspace_layout. */
moe_status moe_layer_forward(const moe_shape* shape, const uint16_t* x, const float* router_w,
                             const moe_q4_ffn* experts, const moe_q4_ffn* shared, uint16_t* out,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* What moe_layer_forward_ex does for `shape` with options engine `engine` and a shared
 * expert or not (has_shared 0/1), on the current device.  Host-only, pure.  [MTP] para. 6
 * (the expert GEMMs walk tiles of expert rows through a block map).
 *   gemm_engine: MOE_ENGINE_GROUPED, _RESIDENT or _WIDE for the grouped GEMMs, or
 *                MOE_ENGINE_DECODE for the decode-sized chain;
 *   paired:      1 when gate_up (+ SwiGLU) and down run as one launch (resident engine:
 *                each workgroup's down share starts when its gate_up share is done); the
 *                stage events [3] and [4] are then both recorded after that launch.
 * MOE_ERR_SHAPE where moe_layer_forward_ex would return it for the engine. */
typedef struct {
  int32_t gemm_engine;
  int32_t paired;
} moe_layer_plan_info;
moe_status moe_layer_plan(const moe_shape* shape, int32_t engine, int32_t has_shared,
                          moe_layer_plan_info* info);

/* moe_layer_forward with options (engine choice, stage events; NULL = defaults).  Same
 * validation and results; opts->reserved must be 0 and opts->engine a moe_engine (else
 * MOE_ERR_SHAPE).  [MTP] para. 6, as moe_layer_forward. */
moe_status moe_layer_forward_ex(const moe_shape* shape, const uint16_t* x, const float* router_w,
                                const moe_q4_ffn* experts, const moe_q4_ffn* shared, uint16_t* out,
                                void* ws, size_t ws_bytes, const moe_layer_opts* opts,
                                hipStream_t stream);

/* Workspace bytes moe_layer_forward_chunked needs: that of one chunk of
 * min(chunk_tokens, T) tokens.  Host-only, pure; 0 if the arguments are invalid. */
size_t moe_chunked_workspace_bytes(const moe_shape* shape, int32_t chunk_tokens);

/* The layer over T tokens in consecutive chunks of chunk_tokens (the last one shorter),
 * each chunk one moe_layer_forward on the same stream with the same workspace, so the
 * workspace is capped at one chunk's whatever T is ([MTP] para. 6: long prompts run in
 * bounded chunks).  Results equal those of moe_layer_forward over all T tokens (routing
 * and the expert FFNs act on each token alone).  chunk_tokens >= 1 (else MOE_ERR_SHAPE);
 * ws >= moe_chunked_workspace_bytes(shape, chunk_tokens). */
moe_status moe_layer_forward_chunked(const moe_shape* shape, const uint16_t* x,
                                     const float* router_w, const moe_q4_ffn* experts,
                                     const moe_q4_ffn* shared, uint16_t* out, int32_t chunk_tokens,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): moe_layer_forward with no workspace argument.  The
 * workspace is a static device array of MOE_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends (its address is taken once per device, on
 * the first call there); the call allocates nothing.  A shape whose moe_workspace_bytes
 * exceeds the array gives MOE_ERR_WORKSPACE (32 MiB: up to 580 tokens at d_model 2048,
 * 256 experts top-8, d_ff 512).  Every call on one GPU shares that GPU's array and leaves
 * its intermediates there: calls that overlap on one GPU (several streams or host
 * threads) race and give undefined results.  Results equal moe_layer_forward's. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_layer_forward_noalloc(const moe_shape* shape, const uint16_t* x,
                                     const float* router_w, const moe_q4_ffn* experts,
                                     const moe_q4_ffn* shared, uint16_t* out, hipStream_t stream);

/* ---- grouped-query decode attention ----------------------------------------------------
 * MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference engine for
 * Qwen3.6-35B-A3B on Apple Silicon", body paragraph 4 (full-attention layers with
 * grouped-query attention, 16 query heads and two KV heads, over a growing KV cache) and
 * paragraph 8 (decode reads the key and value cache; the query heads of one KV head share
 * a workgroup so that each cached row is loaded once).  One query token:
 *   out[h] = softmax_j(q[h] . k[g, j] / sqrt(head_dim)) . v[g, j],  j < ctx_len,
 *   g = h / (n_q_heads / n_kv_heads),
 * softmax and sums in fp32, output rounded to bf16.  Scale and head mapping are readings. */
typedef struct {
  int32_t n_q_heads;  /* query heads; a multiple of n_kv_heads, at most 16 per KV head */
  int32_t n_kv_heads; /* KV heads, >= 1 */
  int32_t head_dim;   /* 128 (the only size taken) */
  int32_t ctx_len;    /* cached positions attended, >= 1 */
  int64_t kv_stride;  /* positions allocated per KV head in each cache, >= ctx_len */
} moe_gqa_shape;

/* Workspace bytes of moe_gqa_decode_attention (partial outputs: n_kv_heads x
 * ceil(ctx_len / 128) x group x 130 floats); 0 for an unsupported shape. */
size_t moe_gqa_decode_workspace_bytes(const moe_gqa_shape* shape);

/* q: bf16 [n_q_heads, head_dim]; k_cache, v_cache: bf16 [n_kv_heads, kv_stride, head_dim]
 * (positions 0 .. ctx_len-1 are read, row-major, rows contiguous); out: bf16
 * [n_q_heads, head_dim]; all device pointers, 16-byte aligned, caller-owned; ws: device
 * workspace of at least moe_gqa_decode_workspace_bytes.  Two launches on `stream`, no
 * host synchronisation, no allocation.  Errors: MOE_ERR_SHAPE (unsupported shape),
 * MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH. */
moe_status moe_gqa_decode_attention(const moe_gqa_shape* shape, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    uint16_t* out, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ4_H */
