/*
 * moe.h - C ABI of the routed-expert MoE step on MI355X (gfx950).
 *
 * One layer of a Qwen3-Next-style sparse MoE FFN: a router picks the top-k of
 * E experts per token, each chosen expert is read from a fixed-stride packed
 * blob, its int4/int8 group-quantised gate/up/down weights are dequantised
 * inside a GEMV (decode) or grouped GEMM (prefill) with SwiGLU, and the
 * results are combined with the renormalised router weights plus an
 * always-resident, sigmoid-gated shared expert. An optional bounded HBM pool
 * with LFU + recency eviction holds hot experts while the full blob lives in
 * pinned host memory.
 *
 * Sources (web pages about the Swiftlet runtime):
 *  - routing 10 of 512 (80B) or 8 of 256 (35B) per layer; router and shared
 *    experts resident; fixed-stride .qpack blobs, one read per expert; bounded
 *    pool with LFU + recency; int4/int8 group quantisation; 64-bit offsets:
 *    cheshm.ai news article on Swiftlet, paragraphs on how it works and on the
 *    code base; paotong.dev commentary, paragraphs on the principle, the
 *    resident set, the fetch path and the bounded pool.
 *  - 48 layers; 480 experts (about 810 MiB) per token with no cache hit;
 *    --cache-gb budget filled lazily; renormalised top-k (norm_topk_prob):
 *    alphalab.site field test, sections on MoE expert streaming, on the 4.3 GB
 *    figure, on SSD reads and on the 35B correctness fix.
 *
 * Conventions for every function below:
 *  - Return value: moe_status (MOE_OK = 0, negative on error); functions that
 *    return a size return 0 on invalid input. No C++ exception crosses the ABI.
 *  - On error, moe_last_error() returns a message for the calling thread; it
 *    stays valid until that thread's next call into the library.
 *  - Arguments are validated before any HIP call is made.
 *  - "dev" pointers are device (HBM) memory on the current HIP device; "host"
 *    pointers are ordinary host memory. The caller owns every buffer it
 *    passes; the library never frees or retains caller pointers past the call.
 *  - Streams are hipStream_t passed as void*; NULL is the null stream. Work is
 *    enqueued on that stream; functions return once it is enqueued unless
 *    stated otherwise.
 *  - One model or pool must not be used from two host threads at once.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1, /* invalid argument or configuration */
  MOE_ENOMEM = -2, /* host or device allocation failed */
  MOE_EHIP = -3,   /* a HIP runtime call failed (message says which) */
  MOE_ESTATE = -4  /* wrong, destroyed or mismatched handle, or call out of order */
} moe_status;

/* Shapes of one model. Valid when: bits is 4 or 8; group == 64; hidden and
 * inter are powers of two in [64, 4096] with hidden*bits <= 16384 and
 * inter*bits <= 16384 (a code row holds at most 2048 bytes); shared_inter ==
 * inter; 1 <= n_experts <= 1024; 1 <= top_k <= min(n_experts, 16);
 * (top_k + 1) * inter <= 15360; 1 <= n_layers <= 4096; norm_topk is 0 or 1
 * (1: the top-k weights are renormalised to sum to 1). */
typedef struct {
  int32_t hidden;       /* H */
  int32_t n_experts;    /* E, routed experts per layer */
  int32_t top_k;        /* k */
  int32_t inter;        /* I, routed expert intermediate size */
  int32_t shared_inter; /* I_s, shared expert intermediate size */
  int32_t bits;         /* 4 or 8 */
  int32_t group;        /* 64 */
  int32_t n_layers;     /* L */
  int32_t norm_topk;    /* 1 = renormalise the selected weights */
} moe_config;

typedef struct {
  uint64_t accesses;        /* routed-expert lookups (k per token per layer) */
  uint64_t hits;
  uint64_t misses;
  uint64_t evictions;
  uint64_t h2d_bytes;       /* misses * record bytes copied host -> HBM */
  uint64_t requested_bytes; /* accesses * record bytes (logical reads) */
} moe_pool_stats_t;

typedef struct moe_model moe_model;
typedef struct moe_pool moe_pool;

/* ---------------------------------------------------------------- layout ---
 * Packed expert record (one expert, inter = I): gate codes [I][H] and up
 * codes [I][H], row-major; then the down matrix [H][I] in 16-byte tiles
 * [I*bits/128][H][16]: each row is cut into 16-byte tiles (32 int4 or 16 int8
 * codes) and tile t of every row precedes tile t+1 of any row, so an I-slice
 * of the whole matrix is contiguous. int4 stores element k of a row in byte
 * k>>1 (even k in the low nibble), int8 one unsigned byte per element. Then
 * (scale, bias) fp16 pairs per 64-element group along each row: gate
 * [I][H/64][2], up [I][H/64][2], and down group-major [I/64][H][2]. Then zero
 * bytes up to the stride = round_up(record bytes, 4096). The dequantised weight is
 * scale * code + bias. Global expert id gid = layer * E + e; record gid sits
 * at byte offset base + gid * stride (fixed-stride blob, one read of the
 * record bytes per expert: paotong.dev commentary, paragraph on the fetch
 * path). */

/* Bytes of one packed record with intermediate size `inter`
 * (3*H*inter*bits/8 + 3*(H*inter/64)*4), or 0 if the config is invalid.
 * Pass inter = cfg->inter for routed experts, cfg->shared_inter for the
 * shared expert. */
size_t moe_expert_bytes(const moe_config* cfg, int32_t inter);

/* round_up(moe_expert_bytes(cfg, inter), 4096), or 0 if invalid. */
size_t moe_expert_stride(const moe_config* cfg, int32_t inter);

/* base + gid * stride in 64-bit arithmetic (the 48-layer 80B blob exceeds
 * 2^32 bytes). */
uint64_t moe_blob_offset(uint64_t base, uint64_t gid, uint64_t stride);

/* Quantise and pack n experts on the host (multi-threaded).
 * w_gate, w_up: host fp32 [n][inter][H]; w_down: host fp32 [n][H][inter].
 * dst: host, receives n records at moe_expert_stride(cfg, inter) apart
 * (padding zeroed); dst_bytes must be >= n * stride.
 * Per row and 64-group, in IEEE fp32: lo, hi = min, max;
 * scale = fp16_rne((hi - lo) / (2^bits - 1)); bias = fp16_rne(lo);
 * code = clamp(rne((w - bias) / scale), 0, 2^bits - 1), 0 when scale == 0.
 * (The pages name MLX-style int4/int8 group quantisation, cheshm.ai article,
 * paragraph on the code base; this min/max grid is the reading taken.)
 * Errors: MOE_EINVAL for an invalid config or inter, n < 0, NULL pointers,
 * short dst, a non-finite weight, or a scale/bias that overflows fp16. */
moe_status moe_pack(const moe_config* cfg, int32_t inter, const float* w_gate, const float* w_up,
                    const float* w_down, int64_t n, void* dst, size_t dst_bytes);

/* Decode one record (host) for inspection: codes one byte per element in the
 * order gate [I][H], up [I][H], down [H][I] (3*H*inter bytes into q_out, the
 * down tiles put back into rows); fp16 bit patterns of the (scale, bias)
 * pairs as gate [I][H/64][2], up [I][H/64][2], down [H][I/64][2] into sc_out
 * (3*H*inter/64*2 uint16). */
moe_status moe_unpack(const moe_config* cfg, int32_t inter, const void* record, uint8_t* q_out,
                      uint16_t* sc_out);

/* ----------------------------------------------------------------- model ---*/

enum { MOE_STORE_DEVICE = 0, MOE_STORE_HOST = 1 };

/* Create a model on the current HIP device. Allocates the routed-expert
 * store (L*E records at the routed stride): in HBM for MOE_STORE_DEVICE, in
 * pinned host memory for MOE_STORE_HOST (the backing blob of a pool), plus
 * HBM for the resident dense part (routers, router biases, shared experts,
 * shared gates) and per-call scratch. Contents start zeroed/unset; fill them
 * with moe_model_set_layer and moe_model_set_experts (or write records
 * directly into moe_model_host_blob). Errors: MOE_EINVAL (config, storage),
 * MOE_ENOMEM, MOE_EHIP. */
moe_status moe_model_create(const moe_config* cfg, int32_t storage, moe_model** out);

/* Resident dense weights of one layer (all host pointers, copied in):
 * router_w fp32 [H][E]; router_bias fp32 [E] or NULL (zero); shared_record
 * one packed record of the shared expert (moe_expert_bytes(cfg,
 * shared_inter) bytes); shared_gate fp32 [H] (gate = sigmoid(x . g)).
 * Synchronous. Errors: MOE_EINVAL, MOE_ESTATE, MOE_EHIP. */
moe_status moe_model_set_layer(moe_model* m, int32_t layer, const float* router_w, const float* router_bias,
                               const void* shared_record, const float* shared_gate);

/* Copy n routed records (host, at the routed stride, in gid order starting
 * at first_gid) into the model's expert store. Synchronous.
 * Errors: MOE_EINVAL (range, NULL), MOE_ESTATE, MOE_EHIP. */
moe_status moe_model_set_experts(moe_model* m, int64_t first_gid, int64_t n, const void* records);

/* For MOE_STORE_HOST models: the pinned host blob (L*E*stride bytes) that
 * backs the pool; the caller may pack records straight into it. */
moe_status moe_model_host_blob(moe_model* m, void** ptr, size_t* bytes);

void moe_model_destroy(moe_model* m); /* NULL is a no-op; waits for the device */

/* --------------------------------------------------------------- forward ---*/

/* One MoE layer on n_tok tokens: out[t] = sum_j w[t,j] * expert_{idx[t,j]}(x_t)
 * + sigmoid(x_t . g_s) * shared(x_t), every token independent.
 * x: dev bf16 bit patterns [n_tok][H]; out: dev fp32 [n_tok][H]; stream: the
 * stream to run on. Batches of fewer than 8 tokens use the decode GEMV
 * kernels token by token; larger batches of int4 layers with H % 256 == 0
 * (and H, I <= 4096, E <= 1024) bucket the (token, expert) pairs and run the
 * MFMA grouped GEMM (other layers keep the GEMV path). The
 * batched path keeps a workspace sized for the largest batch seen so far; a
 * call that has to grow it synchronises the device and allocates (about
 * n_tok * (k + 1) * (4 H + 4 I + I / 16) bytes). Needs MOE_STORE_DEVICE.
 * n_tok == 0 is a no-op.
 * Errors: MOE_EINVAL (layer, n_tok < 0, NULL, n_tok > 65536), MOE_ESTATE, MOE_EHIP. */
moe_status moe_layer_forward(moe_model* m, int32_t layer, const uint16_t* x, int32_t n_tok, float* out,
                             void* stream);

/* Batch-1 decode of one layer over n_tok tokens processed strictly one after
 * another (each token's router -> top-k -> expert GEMV -> combine chain
 * completes before the next token starts). Same arguments and result as
 * moe_layer_forward; always the GEMV path. */
moe_status moe_layer_decode(moe_model* m, int32_t layer, const uint16_t* x, int32_t n_tok, float* out,
                            void* stream);

/* Batch-1 decode of the whole L-layer stack, tokens one at a time:
 * r_0 = x0; x_l = bf16_rne(r_l); r_{l+1} = r_l + layer_l(x_l); out = r_L.
 * pool == NULL: every expert must be resident (MOE_STORE_DEVICE).
 * pool != NULL: experts are served from the pool; on each (token, layer) the
 * host reads the top-k, looks the experts up in ascending expert order,
 * copies misses from the pinned blob into evicted slots with hipMemcpyAsync
 * on the pool's copy stream, and the expert kernels wait for those copies.
 * This call blocks the host until the last token is done when pool != NULL.
 * x0: dev bf16 [n_tok][H]; out: dev fp32 [n_tok][H].
 * Errors: MOE_EINVAL, MOE_ESTATE (pool of another model, host-store model
 * without a pool), MOE_EHIP. */
moe_status moe_stack_decode(moe_model* m, moe_pool* pool, const uint16_t* x0, int32_t n_tok, float* out,
                            void* stream);

/* Routing of the most recent forward/decode call: for each step (token-major,
 * then layer) the k selected experts in selection order (logit descending,
 * lower index first on ties) and their weights. Copies min(cap, steps) steps
 * into idx (int32 [cap][k]) and w (fp32 [cap][k]) on the host; *n_steps
 * receives the number of steps recorded. Synchronises the device. */
moe_status moe_debug_routing(moe_model* m, int32_t* idx, float* w, size_t cap, size_t* n_steps);

/* ------------------------------------------------------------------ pool ---*/

/* Bounded HBM expert pool for a MOE_STORE_HOST model: slots =
 * floor(budget_bytes / stride), allocated in HBM, starting empty (filled
 * lazily). LFU + recency: a hit bumps the slot's use count and last-use tick;
 * a miss takes the lowest empty slot, else evicts the slot with the smallest
 * (use count, last-use tick) that the current (token, layer) step does not
 * use. (cheshm.ai article, paragraph on how it works; paotong.dev commentary,
 * paragraph on the bounded pool; alphalab.site field test, section on the 4.3
 * GB figure, for the lazily filled --cache-gb budget.)
 * Errors: MOE_EINVAL (slots < top_k), MOE_ESTATE (device-store model),
 * MOE_ENOMEM, MOE_EHIP. */
moe_status moe_pool_create(moe_model* m, size_t budget_bytes, moe_pool** out);

/* Empty every slot and zero the statistics and trace. */
moe_status moe_pool_reset(moe_pool* p);

moe_status moe_pool_stats(const moe_pool* p, moe_pool_stats_t* out);

/* Per-access trace since creation/reset, in access order: hit[i] = 1/0 and
 * victim[i] = evicted gid or -1. Copies min(cap, n) entries; *n receives the
 * total count. Either output pointer may be NULL. */
moe_status moe_pool_trace(const moe_pool* p, uint8_t* hit, int64_t* victim, size_t cap, size_t* n);

void moe_pool_destroy(moe_pool* p); /* NULL is a no-op */

/* Host-only replay of the pool policy: n_slots slots, n_steps steps of k
 * gids each (gids [n_steps][k], visited in ascending order within a step).
 * Writes hit [n_steps*k] and victim [n_steps*k]. No GPU involved. */
moe_status moe_pool_simulate(int64_t n_slots, int32_t k, int64_t n_steps, const int64_t* gids, uint8_t* hit,
                             int64_t* victim);

/* ------------------------------------------------------------- profiling ---*/

typedef struct {
  char name[32];      /* kernel family: "router", "route", "gateup", "down", "prefill_*" */
  uint64_t launches;  /* launches recorded */
  double total_ms;    /* sum of per-launch durations (hipEvent pairs around each launch) */
} moe_kernel_time_t;

/* enable = 1: from now on record a hipEvent pair on the launch stream around
 * every kernel this model launches (adds two event records per launch);
 * enable = 0: stop recording. Errors: MOE_EINVAL, MOE_ESTATE. */
moe_status moe_profile_enable(moe_model* m, int32_t enable);

/* Wait for the recorded events, then return the per-kernel-family totals
 * accumulated since profiling was enabled (or last read) and reset them.
 * Copies min(cap, families) entries; *n receives the number of families. */
moe_status moe_profile_read(moe_model* m, moe_kernel_time_t* out, size_t cap, size_t* n);

/* --------------------------------------------------------------- errors ---*/
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
