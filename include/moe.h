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
  uint64_t storage_reads;   /* file-backed model: records read from the blob file */
  uint64_t storage_bytes;   /* bytes those reads took from storage (whole strides for direct I/O) */
  uint64_t direct_io;       /* 1 when the blob file bypasses the page cache (O_DIRECT) */
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
 * shared expert. This is the pages' expertSize, the bytes one read fetches
 * (paotong.dev commentary, paragraph on the fetch path; alphalab.site field
 * test, section on SSD reads, where 480 such reads come to about 810 MiB). */
size_t moe_expert_bytes(const moe_config* cfg, int32_t inter);

/* round_up(moe_expert_bytes(cfg, inter), 4096), or 0 if invalid: the pages'
 * expertStride, the fixed distance between records in the repacked blob
 * (paotong.dev commentary, paragraph on the fetch path; cheshm.ai article,
 * paragraph on how it works). */
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

enum { MOE_STORE_DEVICE = 0, MOE_STORE_HOST = 1, MOE_STORE_FILE = 2 };
enum { MOE_FILE_DIRECT = 1 };

/* Create a model on the current HIP device. Allocates the routed-expert
 * store (L*E records at the routed stride): in HBM for MOE_STORE_DEVICE, in
 * pinned host memory for MOE_STORE_HOST (the backing blob of a pool), or
 * none for MOE_STORE_FILE (the records stay in a blob file on storage, opened
 * with moe_model_open_blob and served through a pool), plus
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

/* For MOE_STORE_FILE models: open the blob file at `path` read-only. Record
 * gid is the moe_expert_bytes(cfg, inter) bytes at file offset base + gid *
 * stride; the file must hold base + L*E*stride bytes. A pool of this model
 * serves each miss with one pread of the record from the file into a pinned
 * staging buffer (the misses of a step read in parallel on up to 8 worker
 * threads) followed by the host->device copy into the slot (paotong.dev
 * commentary, paragraph on the fetch path: one pread of expertSize at
 * blobBase + expertIndex * expertStride; alphalab.site field test, section on
 * SSD reads: plain open() reads are served by the page cache when they hit).
 * flags = MOE_FILE_DIRECT asks for O_DIRECT, which bypasses the page cache
 * when the filesystem supports it and base is a multiple of 4096 (each read
 * then covers the whole stride); otherwise, or with flags = 0, reads are
 * buffered. moe_pool_stats reports which. The file is closed by
 * moe_model_destroy or by opening another. Errors: MOE_EINVAL (NULL path,
 * unknown flags, missing or short file), MOE_ESTATE (not a file-backed model). */
moe_status moe_model_open_blob(moe_model* m, const char* path, uint64_t base, int32_t flags);

void moe_model_destroy(moe_model* m); /* NULL is a no-op; waits for the device */

/* --------------------------------------------------------------- forward ---*/

/* One MoE layer on n_tok tokens: out[t] = sum_j w[t,j] * expert_{idx[t,j]}(x_t)
 * + sigmoid(x_t . g_s) * shared(x_t), every token independent. (Top-k routing
 * per layer and the resident shared expert: cheshm.ai article, paragraph on
 * how it works; paotong.dev commentary, paragraphs on the principle and the
 * resident set. Renormalised top-k weights: alphalab.site field test, section
 * on the 35B correctness fix. The pages' runtime has no batched prefill,
 * alphalab.site FAQ on long prompts; the batched path is this library's.)
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
 * moe_layer_forward; always the GEMV path. (The pages' decode loop handles one
 * token at a time: alphalab.site field test, method section and FAQ on
 * token-by-token processing; paotong.dev commentary, paragraph on the bounded
 * pool, on the loop being dispatch-bound.) */
moe_status moe_layer_decode(moe_model* m, int32_t layer, const uint16_t* x, int32_t n_tok, float* out,
                            void* stream);

/* Batch-1 decode of the whole L-layer stack, tokens one at a time (the 48
 * layers and 480 expert fetches per token: alphalab.site field test, sections
 * on MoE expert streaming and on SSD reads; the on-demand fetch into a bounded
 * pool: paotong.dev commentary, paragraphs on the fetch path and the pool):
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

/* moe_layer_forward's batched path (router GEMM, top-k, bucketing, grouped
 * GEMMs, combine) for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It calls no
 * hipMalloc, hipFree or other allocating routine: its workspace lives in one
 * static 64 MiB device array, of which each GPU holds its own copy from the
 * library's first use of this call on that GPU until the process ends. Same
 * arguments and arithmetic as moe_layer_forward on a batch of 8 or more
 * tokens (bit-identical results), for any 1 <= n_tok up to what the array
 * holds: about 108 KB per token for the 80B-shaped layer (H 2048, E 512,
 * k 10, I 512), so at most ~600 tokens per call; a larger n_tok returns
 * MOE_EINVAL with the limit in the message. Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads)
 * race and must be serialised by the caller. Each call rewrites everything it
 * reads, so nothing carries over from the previous call. The routing stays in
 * the array: moe_debug_routing reports no steps after this call. Needs an
 * int4 layer with H % 256 == 0 (MOE_EINVAL otherwise), MOE_STORE_DEVICE, and
 * the model's device current (MOE_ESTATE otherwise). */
moe_status moe_layer_forward_noalloc(moe_model* m, int32_t layer, const uint16_t* x, int32_t n_tok, float* out,
                                     void* stream);

/* Test support, not a step of the method. Routing of the most recent
 * forward/decode call: for each step (token-major, then layer) the k selected
 * experts in selection order (logit descending, lower index first on ties)
 * and their weights. Copies min(cap, steps) steps
 * into idx (int32 [cap][k]) and w (fp32 [cap][k]) on the host; *n_steps
 * receives the number of steps recorded. Synchronises the device. */
moe_status moe_debug_routing(moe_model* m, int32_t* idx, float* w, size_t cap, size_t* n_steps);

/* ------------------------------------------------------------------ pool ---*/

/* Bounded HBM expert pool for a MOE_STORE_HOST model, or a MOE_STORE_FILE
 * model whose blob file is open (which adds k pinned staging buffers of one
 * stride each and the read workers): slots =
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

/* Counters since creation/reset: lookups, hits, misses, evictions, the
 * bytes copied vs requested (the pages report 43-70% hit rates and ~810 MiB
 * of logical reads per token with no hit: paotong.dev commentary, paragraph
 * on the bounded pool; alphalab.site field test, section on SSD reads), and
 * for a file-backed model the reads taken from the blob file. */
moe_status moe_pool_stats(const moe_pool* p, moe_pool_stats_t* out);

/* Per-access trace since creation/reset, in access order: hit[i] = 1/0 and
 * victim[i] = evicted gid or -1. Copies min(cap, n) entries; *n receives the
 * total count. Either output pointer may be NULL. (The LFU + recency policy it
 * records: paotong.dev commentary, paragraph on the bounded pool; cheshm.ai
 * article, paragraph on how it works.) */
moe_status moe_pool_trace(const moe_pool* p, uint8_t* hit, int64_t* victim, size_t cap, size_t* n);

void moe_pool_destroy(moe_pool* p); /* NULL is a no-op */

/* Test support: host-only replay of the pool policy: n_slots slots, n_steps steps of k
 * gids each (gids [n_steps][k], visited in ascending order within a step).
 * Writes hit [n_steps*k] and victim [n_steps*k]. No GPU involved. */
moe_status moe_pool_simulate(int64_t n_slots, int32_t k, int64_t n_steps, const int64_t* gids, uint8_t* hit,
                             int64_t* victim);

/* ------------------------------------------------------ kernel variants ---*/

enum { MOE_KERNELS_FAST = 0, MOE_KERNELS_SCALAR = 1 };

/* Select the kernels the model's later forward and decode calls run.
 * MOE_KERNELS_SCALAR swaps in plainly written variants of the decode expert
 * kernel (route, gate/up + SwiGLU, weighted partial down rows: one thread per
 * value) and of the two grouped GEMMs of the batched path (one wave per
 * output tile, operands read from global memory right before each MFMA), which
 * repeat the fast kernels' arithmetic operation for operation and so give
 * bit-identical outputs, much more slowly: a reference on the GPU itself for
 * debugging the fast kernels (the pages' runtime keeps fast and scalar
 * kernels whose outputs must agree exactly: paotong.dev commentary,
 * paragraph on the test fixtures). The router, bucketing, reduce and combine
 * kernels are shared. A decode call on scalar kernels needs hidden <= 2048
 * (else MOE_EINVAL from that call) and resident experts (a pooled
 * moe_stack_decode returns MOE_EINVAL). Errors: MOE_EINVAL (unknown kernels),
 * MOE_ESTATE. */
moe_status moe_model_set_kernels(moe_model* m, int32_t kernels);

/* ------------------------------------------------------------- profiling ---*/

typedef struct {
  char name[32];      /* kernel family: "router", "route", "gateup", "down", "prefill_*" */
  uint64_t launches;  /* launches recorded */
  double total_ms;    /* sum of per-launch durations (each kernel's own begin/end timestamps) */
} moe_kernel_time_t;

/* Measurement support, not a step of the method. enable = 1: from now on
 * every kernel this model launches takes a hipEvent pair that the launch
 * fills with the kernel's own begin and end timestamps (hipExtLaunchKernel),
 * and decode sequences run as ordinary launches instead of replayed graphs;
 * enable = 0: stop recording. Errors: MOE_EINVAL, MOE_ESTATE. */
moe_status moe_profile_enable(moe_model* m, int32_t enable);

/* Wait for the recorded events, then return the per-kernel-family totals
 * accumulated since profiling was enabled (or last read) and reset them.
 * Copies min(cap, families) entries; *n receives the number of families. */
moe_status moe_profile_read(moe_model* m, moe_kernel_time_t* out, size_t cap, size_t* n);

/* ----------------------------------------------- Gated DeltaNet decode ---
 * The linear-attention step beside the MoE in 36 of the 80B model's 48
 * layers, whose recurrent state has a fixed size, about 72 MiB over those
 * layers (alphalab.site field test, section explaining MoE expert streaming;
 * cheshm.ai article, paragraph on the code base, for the Gated DeltaNet /
 * gated attention hybrid). The pages print no formula; the step is the
 * published gated delta rule in the decode form of the Qwen3-Next layer, per
 * value head h of key head h / (n_v_heads / n_k_heads), one token at a time:
 *   y = silu(causal 4-tap depthwise conv of the q, k, v channels);
 *   q = y_q / sqrt(|y_q|^2 + 1e-6) / sqrt(d_k), k = y_k / sqrt(|y_k|^2 + 1e-6);
 *   alpha = exp(-exp(A_log[h]) * softplus(a[h] + dt_bias[h])), beta = sigmoid(b[h]);
 *   S <- alpha S; u = beta (v - S^T k); S <- S + k u^T; o = S^T q;
 *   out = o / sqrt(mean(o^2) + 1e-6) * norm_w * silu(z).
 * The state S of a layer is fp32 [n_v_heads][d_v][d_k] in HBM (2 MiB at the
 * 80B shape, 36 layers 72 MiB), plus the last three conv inputs per channel. */
typedef struct {
  int32_t n_layers;
  int32_t n_k_heads;  /* query/key heads */
  int32_t n_v_heads;  /* value heads, a multiple of n_k_heads */
  int32_t d_k;        /* (d_k, d_v) is (32, 32), (64, 64) or (128, 128) */
  int32_t d_v;
} moe_gdn_config;
typedef struct moe_gdn moe_gdn;

/* Allocate parameters and zeroed state for n_layers layers on the current
 * device. Channels C = 2 * n_k_heads * d_k + n_v_heads * d_v (q, then k, then
 * v). Errors: MOE_EINVAL (config), MOE_ENOMEM. */
moe_status moe_gdn_create(const moe_gdn_config* cfg, moe_gdn** out);
/* Host fp32 parameters of one layer, copied in: conv_w [C][4] (tap 3 multiplies
 * the newest input), a_log [n_v_heads], dt_bias [n_v_heads], norm_w [d_v]. */
moe_status moe_gdn_set_layer(moe_gdn* g, int32_t layer, const float* conv_w, const float* a_log,
                             const float* dt_bias, const float* norm_w);
/* Zero every layer's state and conv history (synchronous). */
moe_status moe_gdn_reset(moe_gdn* g);
/* Decode n_tok tokens one after another through layers [first_layer,
 * first_layer + n_layers) (token-major: each token through every layer of the
 * range, then the next token), updating each layer's state in place. dev bf16
 * inputs qkv [n_tok][n_layers][C], z [n_tok][n_layers][n_v_heads * d_v], a, b
 * [n_tok][n_layers][n_v_heads]; dev fp32 out [n_tok][n_layers][n_v_heads *
 * d_v]. One kernel per (token, layer) (8 blocks per value head), which also
 * applies the previous step's gated norm, and one norm kernel after the
 * call's last step; sequences of 16 or more steps are captured once into a
 * HIP graph and replayed. The layers
 * of one call must have taken equally many tokens so far (MOE_ESTATE
 * otherwise). Errors: MOE_EINVAL, MOE_ESTATE, MOE_EHIP. */
moe_status moe_gdn_decode(moe_gdn* g, int32_t first_layer, int32_t n_layers, const uint16_t* qkv,
                          const uint16_t* z, const uint16_t* a, const uint16_t* b, int32_t n_tok, float* out,
                          void* stream);
/* Measurement support: enable = 1 makes every later step kernel take the
 * kernel's own begin/end timestamps (steps run as ordinary launches, not
 * graphs); each call first returns, in *total_ms and *launches (either may be
 * NULL), the time and count recorded since the previous call, waiting for
 * them, then sets recording per `enable`. */
moe_status moe_gdn_profile(moe_gdn* g, int32_t enable, double* total_ms, uint64_t* launches);
/* Test support: copy a layer's state (host fp32 [n_v_heads][d_v][d_k]) and conv
 * history (host fp32 [C][3], oldest first) out; either may be NULL.
 * Synchronises the device. */
moe_status moe_gdn_read_state(moe_gdn* g, int32_t layer, float* state, float* window);
void moe_gdn_destroy(moe_gdn* g); /* NULL is a no-op; waits for the device */

/* ------------------------------------ Gated attention decode, KV cache ---
 * The full-attention step of the 12 layers (of the 80B model's 48) that keep
 * a growing K/V cache, budgeted at 24 KiB per token in fp16 (alphalab.site
 * field test, section explaining MoE expert streaming; cheshm.ai article,
 * paragraph on the code base, for the gated attention / Gated DeltaNet
 * hybrid). The pages print no formula; the step is the decode form of the
 * Qwen3-Next gated attention layer, for the token at position p, query head h
 * of KV group h / (n_q_heads / n_kv_heads):
 *   q_h = rope(rms(q_h) * wq), k_g = rope(rms(k_g) * wk), rms(x) = x / sqrt(mean(x^2) + 1e-6);
 *   rope rotates the first rot_dim dims: pairs (i, i + rot_dim/2), angle p * 1e7^(-2i/rot_dim);
 *   K[p] = fp16(k_g), V[p] = fp16(v_g) (round to nearest even);
 *   out_h = softmax_j(q_h . K[j] / sqrt(d), j <= p) . V * sigmoid(gate_h).
 * Cache bytes per token and layer: 2 * n_kv_heads * head_dim * 2 (2 KiB at the
 * 80B shape: 2 KV heads of 256). On the device, K is [n_kv][max_pos][d] and V
 * is kept in tiles of 32 positions, [n_kv][span][d][32]. */
typedef struct {
  int32_t n_layers;
  int32_t n_q_heads;   /* query heads, n_kv_heads times 1, 2, 4, 8 or 16 */
  int32_t n_kv_heads;  /* <= 256 */
  int32_t head_dim;    /* 64, 128 or 256 */
  int32_t rot_dim;     /* rotated dims, even, <= head_dim */
  int32_t max_pos;     /* cache capacity in positions, <= 2^20 */
} moe_attn_config;
typedef struct moe_attn moe_attn;

/* Allocate the norm weights and a zeroed cache of max_pos positions for
 * n_layers layers on the current device. Errors: MOE_EINVAL (config),
 * MOE_ENOMEM. */
moe_status moe_attn_create(const moe_attn_config* cfg, moe_attn** out);
/* Host fp32 per-head RMS-norm weights of one layer, copied in: q_norm_w,
 * k_norm_w [head_dim]. */
moe_status moe_attn_set_layer(moe_attn* a, int32_t layer, const float* q_norm_w, const float* k_norm_w);
/* Write positions [first_pos, first_pos + n) of a layer's cache from host fp16
 * bits k, v [n_kv_heads][n][head_dim] (a prefilled context). Synchronous.
 * Errors: MOE_EINVAL (range), MOE_EHIP. */
moe_status moe_attn_write_cache(moe_attn* a, int32_t layer, int32_t first_pos, int32_t n, const uint16_t* k,
                                const uint16_t* v);
/* Test support: read positions [first_pos, first_pos + n) of a layer's cache
 * into host fp16 bits k, v [n_kv_heads][n][head_dim] (either may be NULL).
 * Synchronises the device. */
moe_status moe_attn_read_cache(moe_attn* a, int32_t layer, int32_t first_pos, int32_t n, uint16_t* k, uint16_t* v);
/* Decode n_tok tokens at positions pos0, pos0 + 1, ... through layers
 * [first_layer, first_layer + n_layers), token-major (each token through every
 * layer of the range, then the next). Each step writes the token's K/V row
 * at its position and attends over positions [0, p]; positions below pos0
 * must already hold the context. dev bf16 inputs q, gate
 * [n_tok][n_layers][n_q_heads * head_dim] and k, v [n_tok][n_layers][n_kv_heads
 * * head_dim] (the projections); dev fp32 out [n_tok][n_layers][n_q_heads *
 * head_dim] (before the output projection). Per (token, layer): a kernel
 * with one block per (KV head, 128 cached positions) producing softmax
 * partials, then their merge with the gate, which also prepares the next
 * step (its normed, rotated q, and its K/V row written into the cache); a
 * call's first step is prepared by a kernel of its own. Sequences of 16 or
 * more steps are captured once into a HIP graph and replayed. Errors: MOE_EINVAL, MOE_ESTATE (a layer
 * without moe_attn_set_layer), MOE_EHIP. */
moe_status moe_attn_decode(moe_attn* a, int32_t first_layer, int32_t n_layers, int32_t pos0, const uint16_t* q,
                           const uint16_t* gate, const uint16_t* k, const uint16_t* v, int32_t n_tok, float* out,
                           void* stream);
/* Measurement support: enable = 1 makes every later step take the kernels'
 * own begin/end timestamps (steps run as ordinary launches, not graphs); each
 * call first returns, in *split_ms (partials kernel), *combine_ms (merge
 * kernel) and *launches (steps; any may be NULL), what was recorded since the
 * previous call, waiting for it, then sets recording per `enable`. */
moe_status moe_attn_profile(moe_attn* a, int32_t enable, double* split_ms, double* combine_ms, uint64_t* launches);
void moe_attn_destroy(moe_attn* a); /* NULL is a no-op; waits for the device */

/* --------------------------------------------------------------- errors ---*/
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
