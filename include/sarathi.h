/*
 * sarathi.h — C ABI of the hybrid-batch decoder-layer library for AMD Instinct MI355X (gfx950).
 *
 * The library runs the forward pass of one LLaMA-style (or GPT-style) decoder layer over a HYBRID
 * BATCH: one prefill chunk of C tokens from one request plus B single-token decodes, each decode
 * request with its own KV cache (or, through the sarathi_multi_* entry points, several chunks of
 * different requests plus decodes).  The linear ops (QKV, O, gate/up, down) run as single GEMMs over the
 * C+B concatenated rows, so the decodes share the chunk's weight fetches; attention is split per
 * request: causal attention of the chunk over its cached prefix plus itself, and single-query
 * attention of each decode over its own cache plus its own new token.
 *   - Hybrid batch, fused linear ops, separate attention, in-place KV writes into caches allocated at
 *     maximum length: "SARATHI: Efficient LLM Inference by Piggybacking Decodes with Chunked
 *     Prefills", section 3, "Decode-Maximal Batching" and "Implementation" (KV cache
 *     pre-allocation).
 *   - Chunk mask (query at absolute position p sees keys 0..p): same page, "Chunked-Prefills",
 *     Figure 6.
 *   - A decode with S cached entries attends over S+1 keys: "Sarathi-Serve Guide: Chunked-Prefills &
 *     LLM Serving", "Deep Dive", "Attention Complexity Across Mixed Batches".
 *   - The caller advances prompt progress and decode lengths after the step (same guide, the
 *     co-scheduler's step update); the library never changes a length.
 *
 * Conventions for every entry point
 *   - Device pointers point to memory of the current HIP device; host pointers to host memory.
 *   - Matrices are row-major.  Weights are stored [out_features, in_features] (y = x W^T).
 *   - Storage type (weights, x, y, caches): float32 (SARATHI_F32) or bfloat16 (SARATHI_BF16), per
 *     the layer's dtype.  Norm gains/biases are always float32.  Arithmetic accumulates in float32.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only ENQUEUE work on it and return;
 *     they never synchronise the device.  All validation runs on the host before anything is
 *     enqueued; on any error nothing is launched and no buffer is written.
 *   - No C++ exception crosses this boundary.  Every failing call records a message readable with
 *     sarathi_last_error() (thread-local, valid until the thread's next failing call).
 */
#ifndef SARATHI_H
#define SARATHI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SARATHI_OK = 0,
    SARATHI_ERR_INVALID = -1,      /* bad argument: null pointer, negative size, aliasing, ... */
    SARATHI_ERR_UNSUPPORTED = -2,  /* valid but not supported shape (e.g. head_dim not 64/128) */
    SARATHI_ERR_CAPACITY = -3,     /* a position or write slot does not fit a cache / the RoPE table */
    SARATHI_ERR_HIP = -4,          /* a HIP runtime call failed */
    SARATHI_ERR_NOMEM = -5,        /* host or device allocation failed (create only) */
    SARATHI_ERR_WORKSPACE = -6,    /* workspace null, too small or misaligned */
    SARATHI_ERR_INTERNAL = -7
} sarathi_status;

typedef enum { SARATHI_F32 = 0, SARATHI_BF16 = 1 } sarathi_dtype;

/* LLAMA: RMSNorm, RoPE on Q and K (adjacent pairs (2j, 2j+1), angle pos * base^(-2j/head_dim)),
 *        SwiGLU FFN act = silu(x W_gate^T) * (x W_up^T).
 * GPT:   LayerNorm (biased variance) with bias, no RoPE, GELU MLP act = gelu(x W_up^T) (erf form). */
typedef enum { SARATHI_ARCH_LLAMA = 0, SARATHI_ARCH_GPT = 1 } sarathi_arch;

typedef struct {
    int32_t hidden;      /* H: model width; multiple of 64, at most 16384 */
    int32_t n_heads;     /* nh */
    int32_t head_dim;    /* d: 64 or 128.  Attention width A = nh*d; multiple of 64 */
    int32_t ffn;         /* F: FFN width; multiple of 64 in bf16 mode, of 16 in f32 mode */
    int32_t arch;        /* sarathi_arch */
    int32_t dtype;       /* sarathi_dtype */
    float norm_eps;      /* e.g. 1e-6 (RMSNorm) or 1e-5 (LayerNorm) */
    float rope_base;     /* e.g. 10000; unused for GPT */
    int32_t max_tokens;  /* largest C+B a forward call may pass */
    int32_t max_pos;     /* every position must be < max_pos (size of the RoPE table); at most 65536 */
} sarathi_layer_desc;

/* Device pointers to caller-owned weights, each 16-byte aligned.  A bf16 layer copies the five
 * projection weights at create (into its own k-tile-major layout, [in/32][out][32], which its GEMM
 * reads as whole 128-byte lines) and does not read the caller's projection buffers afterwards; the
 * norm weights, and every weight of a float32 layer, are referenced and must stay valid and
 * unchanged while the layer exists.
 *   w_qkv [3A, H]: rows [Q | K | V], each block head-major (head h = rows h*d .. h*d+d-1 of it)
 *   w_o [H, A];  w_gate [F, H] (LLAMA only; NULL for GPT);  w_up [F, H];  w_down [H, F]
 *   norm1_w, norm2_w: float32 [H];  norm1_b, norm2_b: float32 [H] (GPT only; NULL for LLAMA) */
typedef struct {
    const void *w_qkv, *w_o, *w_gate, *w_up, *w_down;
    const float *norm1_w, *norm1_b, *norm2_w, *norm2_b;
} sarathi_weights;

/* One request's KV cache: two device buffers, each [n_heads, capacity, head_dim] (head-major, one
 * contiguous [capacity, head_dim] slab per head), storage type = the layer's dtype.  K is stored
 * after RoPE.  Slot j holds the token at position j. */
typedef struct {
    void *k;
    void *v;
    int32_t capacity;
    int32_t reserved;    /* must be 0 */
} sarathi_kv;

/* One hybrid batch.  Rows 0..chunk_len-1 of x are the chunk, at positions chunk_offset+t; row
 * chunk_len+i is decode i, at position decode_len[i] (its cache already holds decode_len[i] entries).
 * The call writes: y; chunk K/V into chunk_kv slots [chunk_offset, chunk_offset+chunk_len); decode
 * i's K/V into its slot decode_len[i].  chunk_len == 0 is a decode-only batch (chunk_kv ignored);
 * n_decodes == 0 is a chunk-only batch.  chunk_len + n_decodes >= 1. */
typedef struct {
    int32_t chunk_len;          /* C >= 0 */
    int32_t chunk_offset;       /* entries already in the chunk request's cache, >= 0 */
    sarathi_kv chunk_kv;        /* device buffers; capacity >= chunk_offset + chunk_len */
    int32_t n_decodes;          /* B >= 0 */
    int32_t reserved;           /* must be 0 */
    const sarathi_kv *decode_kv;  /* HOST array [n_decodes]; capacity >= decode_len[i] + 1 */
    const int32_t *decode_len;    /* HOST array [n_decodes]; >= 0 */
    const void *x;              /* device [C+B, H] input hidden states, chunk rows first */
    void *y;                    /* device [C+B, H] output; must not overlap x, caches or workspace */
} sarathi_batch;

/* Device buffers, each float32 [C+B, width], that sarathi_layer_forward_debug fills with the layer's
 * intermediates (NULL entries are skipped):
 *   n1 [.,H] norm-1 output;  qkv [.,3A] projection before RoPE;  q_rot [.,A] rotated queries;
 *   attn [.,A] attention output (heads concatenated);  h1 [.,H] x + attn W_o^T;
 *   n2 [.,H] norm-2 output;  act [.,F] FFN activation (silu(gate)*up or gelu(up)). */
typedef struct {
    float *n1, *qkv, *q_rot, *attn, *h1, *n2, *act;
} sarathi_debug_dump;

typedef struct sarathi_layer sarathi_layer;   /* opaque, immutable after create */

/* Creates a layer handle for the current HIP device.  Copies *desc.  Allocates the device RoPE
 * cos/sin table [max_pos, head_dim/2] (LLAMA), built on the host in float64, and in bf16 mode one
 * device buffer holding the packed copies of the projection weights (as large as the five weights),
 * filled by kernels on the null stream before this call returns (the caller's weights must be
 * fully written when the call is made: the copy is ordered after earlier work on the null stream
 * only); float32 layers keep the weight pointers.  Errors: INVALID (null or misaligned weight
 * pointers, non-positive sizes), UNSUPPORTED (head_dim not 64/128, widths not multiples of 64, ffn
 * not a multiple of 16 in f32 mode, hidden above 16384, a bf16 weight of 2^31 or more elements),
 * NOMEM, HIP.  On error *out is set to NULL. */
sarathi_status sarathi_layer_create(const sarathi_layer_desc *desc, const sarathi_weights *weights,
                                    sarathi_layer **out);

/* Frees the handle, its RoPE table and its packed weights.  NULL is a no-op.  No call using the
 * handle may be in flight (the caller synchronises its streams first). */
void sarathi_layer_destroy(sarathi_layer *layer);

/* Host-only validation of a batch against a layer description (no HIP call).  Checks: C, B >= 0 and
 * C+B in [1, max_tokens]; non-null x, y, caches and host arrays; reserved fields 0; chunk_offset +
 * chunk_len <= chunk capacity; decode_len[i] + 1 <= capacity_i; every position < max_pos; no two
 * requests share a K or V buffer; y does not overlap x.  Returns OK, INVALID or CAPACITY. */
sarathi_status sarathi_batch_check(const sarathi_layer_desc *desc, const sarathi_batch *batch);

/* Bytes of device workspace sarathi_layer_forward needs for this batch (depends on C+B, the number
 * of decodes and their lengths).  Returns 0 if the batch fails sarathi_batch_check. */
size_t sarathi_workspace_size(const sarathi_layer_desc *desc, const sarathi_batch *batch);

/* Enqueues the layer's forward pass over the hybrid batch on `stream`.
 * workspace: caller-owned device buffer of ws_bytes >= sarathi_workspace_size(...), 256-byte aligned,
 * not shared with another call in flight.  Its contents on entry do not matter.
 * Errors (all before any launch): everything sarathi_batch_check reports, WORKSPACE, HIP. */
sarathi_status sarathi_layer_forward(sarathi_layer *layer, const sarathi_batch *batch,
                                     void *workspace, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): sarathi_layer_forward without a workspace argument.  It
 * runs the same kernels on a fixed scratch of 128 MiB (134217728 bytes) that the library holds in
 * device memory on every GPU it runs on until the process ends; it calls no allocating routine.
 * Batches whose sarathi_workspace_size exceeds 128 MiB are rejected with WORKSPACE before any
 * launch (with the llama-13b shape, a 512-row chunk plus 48 decodes of 1K context needs 119 MiB and
 * fits; a 512-row chunk at offset 7680 plus 48 decodes of 2K-8K context needs 176 MiB and does not:
 * use sarathi_layer_forward with a workspace there).  The scratch keeps the last call's contents;
 * no kernel needs it cleared.  Every call on one GPU uses that GPU's one scratch, so calls that
 * overlap on the same GPU (other streams, other threads, other layers) race: serialise them.  The
 * current device must be the layer's.  Errors (all before any launch): everything
 * sarathi_batch_check reports, WORKSPACE, INVALID (wrong device), HIP. */
sarathi_status sarathi_layer_forward_noalloc(sarathi_layer *layer, const sarathi_batch *batch,
                                             void *stream);

/* As sarathi_layer_forward, then also copies the intermediates named in *dump (float32 device
 * buffers of C+B rows) on the same stream.  dump may be NULL. */
sarathi_status sarathi_layer_forward_debug(sarathi_layer *layer, const sarathi_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           const sarathi_debug_dump *dump);

/* The fused linear op alone: out[M, N] = a[M, K] w[N, K]^T, in `dtype` storage with float32
 * accumulation (the GEMM each of the layer's projections runs over the C+B rows).  a, w, out are
 * device pointers, densely packed row-major.  M >= 1; in bf16 mode K must be a multiple of 64.
 * Errors: INVALID, UNSUPPORTED, HIP. */
sarathi_status sarathi_gemm(int32_t dtype, int32_t m, int32_t n, int32_t k, const void *a,
                            const void *w, void *out, void *stream);

/* The split attention alone, over caches that ALREADY hold this step's K/V rows (chunk slots
 * chunk_offset..chunk_offset+C-1 and decode slots decode_len[i]).  q: device [C+B, nh*d] queries
 * (after RoPE), out: device [C+B, nh*d].  Chunk row t attends to chunk keys 0..chunk_offset+t;
 * decode i attends to its keys 0..decode_len[i].  Scores are scaled by 1/sqrt(d).  batch->x and
 * batch->y are ignored.  workspace: as for the forward (sarathi_workspace_size of the same batch is
 * enough).  Errors: as sarathi_batch_check (x/y not required), WORKSPACE, HIP. */
sarathi_status sarathi_attention(const sarathi_layer_desc *desc, const sarathi_batch *batch,
                                 const void *q, void *out, void *workspace, size_t ws_bytes,
                                 void *stream);

/* ---- A stack of layers ------------------------------------------------------------------------
 * One hybrid batch through n_layers layers in sequence: layer l's output rows are layer l+1's input
 * rows, and every layer keeps its own KV caches.  This is how a prompt is prefilled chunk by chunk
 * with decodes riding along: each chunk passes through all layers, appending its K/V to each layer's
 * cache, before the next chunk (SARATHI: Efficient LLM Inference by Piggybacking Decodes with Chunked
 * Prefills, section 3, "Chunked-Prefills" and "Decode-Maximal Batching").  Layers must share hidden
 * size and storage type. */
typedef struct {
    int32_t chunk_len;          /* C >= 0 */
    int32_t chunk_offset;       /* entries already in the chunk request's caches (same in every layer) */
    const sarathi_kv *chunk_kv; /* HOST array [n_layers]: the chunk request's cache in layer l;
                                   may be NULL when chunk_len == 0 */
    int32_t n_decodes;          /* B >= 0 */
    int32_t reserved;           /* must be 0 */
    const sarathi_kv *decode_kv;  /* HOST array [n_layers * n_decodes], layer-major: decode i's
                                     cache in layer l is decode_kv[l * n_decodes + i] */
    const int32_t *decode_len;    /* HOST array [n_decodes], the same in every layer */
    const void *x;              /* device [C+B, H] input of layer 0, chunk rows first */
    void *y;                    /* device [C+B, H] output of the last layer; must not overlap x */
} sarathi_stack_batch;

/* Bytes of device workspace sarathi_stack_forward needs: the largest per-layer workspace plus two
 * [C+B, H] activation buffers for the hand-off between layers.  Returns 0 if any layer's batch fails
 * sarathi_batch_check or the layers do not share hidden size and storage type. */
size_t sarathi_stack_workspace_size(sarathi_layer *const *layers, int32_t n_layers,
                                    const sarathi_stack_batch *batch);

/* Enqueues all layers on `stream`.  Every layer's batch is validated before the first launch: on an
 * error nothing is written.  workspace as for sarathi_layer_forward, sized by
 * sarathi_stack_workspace_size.  Errors: INVALID, CAPACITY, UNSUPPORTED, WORKSPACE, HIP. */
sarathi_status sarathi_stack_forward(sarathi_layer *const *layers, int32_t n_layers,
                                     const sarathi_stack_batch *batch, void *workspace,
                                     size_t ws_bytes, void *stream);

/* ---- Batches with several prefill chunks -------------------------------------------------------
 * A token-budget batch: decodes plus SEVERAL prefill chunks, each from a different request (a
 * partially prefilled prompt and new prompts cut to fit the budget; junupark.xyz notes on
 * Sarathi-Serve, "Stall Free Batching" and its worked example 4 decodes + 30 + 66 tokens).  The
 * linear ops still run as single GEMMs over all rows; each chunk attends causally to its own
 * request's cached prefix plus itself, each decode to its own cache.  With one chunk (or none) the
 * result is bitwise that of sarathi_layer_forward on the equivalent sarathi_batch. */
#define SARATHI_MAX_CHUNKS 16

typedef struct {
    int32_t len;                /* rows of this chunk, >= 1 */
    int32_t offset;             /* entries already in this request's cache = position of row 0 */
    sarathi_kv kv;              /* device buffers; capacity >= offset + len */
} sarathi_chunk;

/* Rows of x: chunk 0's rows, then chunk 1's, ..., then decode 0..n_decodes-1.  Row r of chunk j
 * (batch row sum_{i<j} chunks[i].len + r) sits at position chunks[j].offset + r and writes cache
 * slot chunks[j].offset + r of chunks[j].kv. */
typedef struct {
    int32_t n_chunks;           /* 0 .. SARATHI_MAX_CHUNKS */
    int32_t reserved;           /* must be 0 */
    const sarathi_chunk *chunks;  /* HOST array [n_chunks]; may be NULL when n_chunks == 0 */
    int32_t n_decodes;          /* B >= 0 */
    int32_t reserved2;          /* must be 0 */
    const sarathi_kv *decode_kv;  /* HOST array [n_decodes]; capacity >= decode_len[i] + 1 */
    const int32_t *decode_len;    /* HOST array [n_decodes]; >= 0 */
    const void *x;              /* device [T, H], T = total chunk rows + n_decodes */
    void *y;                    /* device [T, H]; must not overlap x, caches or workspace */
} sarathi_multi_batch;

/* Host-only validation, as sarathi_batch_check, per chunk; also rejects n_chunks outside
 * [0, SARATHI_MAX_CHUNKS], a chunk with len < 1, and two chunks (or a chunk and a decode) that share
 * a cache.  Returns OK, INVALID or CAPACITY. */
sarathi_status sarathi_multi_batch_check(const sarathi_layer_desc *desc, const sarathi_multi_batch *batch);

/* Bytes of device workspace sarathi_multi_forward needs for this batch; 0 if the check fails. */
size_t sarathi_multi_workspace_size(const sarathi_layer_desc *desc, const sarathi_multi_batch *batch);

/* Enqueues the layer's forward over the batch (workspace rules as sarathi_layer_forward).
 * Errors (all before any launch): everything sarathi_multi_batch_check reports, WORKSPACE, HIP. */
sarathi_status sarathi_multi_forward(sarathi_layer *layer, const sarathi_multi_batch *batch,
                                     void *workspace, size_t ws_bytes, void *stream);

/* As sarathi_multi_forward plus the intermediates of sarathi_layer_forward_debug (dump may be NULL). */
sarathi_status sarathi_multi_forward_debug(sarathi_layer *layer, const sarathi_multi_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           const sarathi_debug_dump *dump);

/* ---- Paged KV caches ---------------------------------------------------------------------------
 * Instead of one buffer per request allocated at maximum length, every request's K/V rows live in
 * fixed-size pages of a pool shared by all requests of the layer, found through the request's block
 * table.  The pages call dynamic (vLLM-style) KV allocation complementary: it raises the number of
 * requests that fit, and so the number of decodes that can ride with each chunk (SARATHI: Efficient
 * LLM Inference by Piggybacking Decodes with Chunked Prefills, "System Optimizations from Prior
 * Work", memory management).  Everything else is as for sarathi_multi_forward.
 *
 * Layout: k_pool and v_pool are each [n_pages, n_heads, page_size, head_dim] in the layer's storage
 * type: page p holds, per head, page_size consecutive rows.  Token t of a request lives in pool page
 * pages[t / page_size] at row t % page_size.
 *
 * The block tables are DEVICE arrays the library only reads; their contents cannot be checked on the
 * host.  Every entry is clamped into [0, n_pages) before use, so a bad entry yields wrong values but
 * never an access outside the pools.  The pages a call WRITES (the slots of this step's rows) must
 * not be shared between requests; pages it only reads (a common prefix) may be. */
typedef struct {
    void *k_pool;               /* device [n_pages, n_heads, page_size, head_dim] */
    void *v_pool;               /* device, same shape; must not overlap k_pool */
    int32_t n_pages;            /* >= 1 */
    int32_t page_size;          /* tokens per page: a power of two in [1, 65536] (16 or 32 typical) */
} sarathi_page_pool;

typedef struct {
    const int32_t *pages;       /* DEVICE int32 [n_entries]: logical page i -> pool page */
    int32_t n_entries;          /* the request can hold n_entries * page_size tokens */
    int32_t reserved;           /* must be 0 */
} sarathi_page_table;

typedef struct {
    int32_t len;                /* rows of this chunk, >= 1 */
    int32_t offset;             /* tokens of this request already cached */
    sarathi_page_table table;   /* n_entries * page_size >= offset + len */
} sarathi_paged_chunk;

/* Rows of x as in sarathi_multi_batch: chunk rows in chunk order, then decodes. */
typedef struct {
    sarathi_page_pool pool;
    int32_t n_chunks;           /* 0 .. SARATHI_MAX_CHUNKS */
    int32_t reserved;           /* must be 0 */
    const sarathi_paged_chunk *chunks;          /* HOST array [n_chunks] */
    int32_t n_decodes;          /* >= 0 */
    int32_t reserved2;          /* must be 0 */
    const sarathi_page_table *decode_tables;    /* HOST array [n_decodes]; capacity > decode_len[i] */
    const int32_t *decode_len;                  /* HOST array [n_decodes] */
    const void *x;              /* device [T, H] */
    void *y;                    /* device [T, H]; must not overlap x or the pools */
} sarathi_paged_batch;

/* Host-only validation: as sarathi_multi_batch_check, plus the pool (non-null, page_size a power of
 * two, n_pages >= 1, K and V pools disjoint), each table (non-null, n_entries >= 1, capacity), and no
 * two requests passing the same table.  Returns OK, INVALID or CAPACITY. */
sarathi_status sarathi_paged_batch_check(const sarathi_layer_desc *desc, const sarathi_paged_batch *batch);

/* Bytes of device workspace sarathi_paged_forward needs; 0 if the check fails. */
size_t sarathi_paged_workspace_size(const sarathi_layer_desc *desc, const sarathi_paged_batch *batch);

/* Enqueues the forward over a paged batch.  Errors: as sarathi_paged_batch_check, WORKSPACE, HIP. */
sarathi_status sarathi_paged_forward(sarathi_layer *layer, const sarathi_paged_batch *batch,
                                     void *workspace, size_t ws_bytes, void *stream);

/* As sarathi_paged_forward plus the intermediates of sarathi_layer_forward_debug (dump may be NULL). */
sarathi_status sarathi_paged_forward_debug(sarathi_layer *layer, const sarathi_paged_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           const sarathi_debug_dump *dump);

/* ---- Per-stage timing (measurement only) ------------------------------------------------------
 * The layer's forward runs as the stages below, in this order (per-operation profile of a hybrid
 * iteration: preproj, attention, postproj, FFN; SARATHI: Efficient LLM Inference by Piggybacking
 * Decodes with Chunked Prefills, section 3, "Implementation" (per-operation profiling) and section 5,
 * per-operation runtime breakdown).  A stage with no work in a batch (e.g. chunk attention when
 * C == 0) is not counted. */
typedef enum {
    SARATHI_STAGE_NORM1 = 0,       /* norm 1 over the C+B rows */
    SARATHI_STAGE_QKV = 1,         /* QKV GEMM */
    SARATHI_STAGE_ROPE_APPEND = 2, /* RoPE + KV-cache append */
    SARATHI_STAGE_ATTN_CHUNK = 3,  /* chunk attention (prefix + causal chunk) */
    SARATHI_STAGE_ATTN_DECODE = 4, /* decode attention (split-KV partials); when the batch's chunk and
                                      decode attention run as one launch, that launch's time is
                                      recorded here and the chunk stage does not run */
    SARATHI_STAGE_ATTN_MERGE = 5,  /* merge of split partials */
    SARATHI_STAGE_O = 6,           /* O GEMM + residual */
    SARATHI_STAGE_NORM2 = 7,
    SARATHI_STAGE_FFN_UP = 8,      /* gate/up GEMM + SiLU*mul, or up GEMM + GELU */
    SARATHI_STAGE_FFN_DOWN = 9,    /* down GEMM + residual */
    SARATHI_N_STAGES = 10
} sarathi_stage;

typedef struct sarathi_timer sarathi_timer;   /* opaque */

/* Creates a timer able to hold the events of `capacity` forwards between two reads.  Only the stages
 * whose bit (1 << sarathi_stage) is set in stage_mask are timed: the forward records one HIP event
 * right before and one right after each of them (every recorded event adds a little to a forward,
 * so a measurement that must not be perturbed times one stage only).  It creates
 * 2 * capacity * (number of stages in the mask) HIP events on the current device.
 * Errors: INVALID (capacity <= 0, empty mask), HIP. */
sarathi_status sarathi_timer_create(int32_t capacity, uint32_t stage_mask, sarathi_timer **out);

/* Destroys the timer's events.  No forward recording into it may be in flight.  NULL is a no-op. */
void sarathi_timer_destroy(sarathi_timer *timer);

/* As sarathi_layer_forward, and records the timer's events on `stream` (no synchronisation).
 * Errors: as the forward; INVALID if the timer already holds `capacity` unread forwards (nothing is
 * enqueued then). */
sarathi_status sarathi_layer_forward_timed(sarathi_layer *layer, const sarathi_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           sarathi_timer *timer);

/* As sarathi_multi_forward, recording the timer's events (see sarathi_layer_forward_timed). */
sarathi_status sarathi_multi_forward_timed(sarathi_layer *layer, const sarathi_multi_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           sarathi_timer *timer);

/* As sarathi_paged_forward, recording the timer's events (see sarathi_layer_forward_timed). */
sarathi_status sarathi_paged_forward_timed(sarathi_layer *layer, const sarathi_paged_batch *batch,
                                           void *workspace, size_t ws_bytes, void *stream,
                                           sarathi_timer *timer);

/* Waits for the recorded events, writes each timed stage's elapsed milliseconds summed over the
 * recorded forwards into total_ms[s] and the number of forwards in which stage s ran into count[s]
 * (host arrays of SARATHI_N_STAGES entries, overwritten; untimed stages read 0), then empties the
 * timer.  Errors: INVALID, HIP. */
sarathi_status sarathi_timer_read(sarathi_timer *timer, double *total_ms, int32_t *count);

/* Enqueues on `stream` one kernel of 4096 single-wave workgroups spread over the compute units.  A
 * workgroup on compute unit u writes two 64-bit counters of that unit to the device buffer `out`
 * (uint64_t[4096], 2048 slots of two): out[2u] = the shader-clock timestamp counter (s_memtime),
 * out[2u+1] = the constant 100 MHz real-time counter (s_memrealtime), where u = 256 * XCD id + bits
 * 15:8 of the wave's HW_ID register (compute unit, shader array, shader engine).  Slots of units no
 * workgroup ran on are left unchanged (the caller zeroes the buffer first).  Each compute unit
 * counts on its own, so two samples taken around enqueued work give the average shader clock over
 * it for each unit present in both: 100 MHz x (delta out[2u]) / (delta out[2u+1]).  For
 * measurement only.  Errors: INVALID (out is NULL), HIP. */
sarathi_status sarathi_clock_sample(uint64_t *out, void *stream);

/* ---- Launch plan (inspection) -------------------------------------------------------------------
 * How a forward over a batch would run, computed on the host exactly as the forward computes it, with
 * no device work: for tests and tools.  The four linear ops run as one GEMM each over all C+B rows
 * and attention is split per request (SARATHI: Efficient LLM Inference by Piggybacking Decodes with
 * Chunked Prefills, "Decode-Maximal Batching"); the row tiles of those GEMMs are what the
 * same page's tile-quantization discussion ("Identifying the Ideal Chunk Size", Figure 7) is about. */
typedef struct {
    int32_t epilogue;    /* 0 bf16/f32 store, 1 float32 split-K partials, 2 SiLU*mul, 3 GELU */
    int32_t row_tiles;   /* workgroup tiles along the batch rows */
    int32_t col_tiles;   /* workgroup tiles along the output columns */
    int32_t k_splits;    /* split-K factor (partials summed in split order by the next kernel) */
    int32_t tile_cols;   /* output columns of one tile: 128, or 256 where row tiles of more than
                            288 rows are split into twice as many of at most 288 rows (batches of
                            more than 288 rows; a fused gate|up tile: 64 or 128 of each) */
} sarathi_gemm_plan;     /* 20 bytes */

typedef struct {
    int32_t rows;                                /* C + B */
    int32_t rows_alloc;                          /* rows of the activation buffers (multiple of 64) */
    int32_t n_chunks;
    int32_t fused_attention;                     /* 1: chunk and decode attention in one launch */
    int32_t chunk_splits[SARATHI_MAX_CHUNKS];    /* key-range splits of each chunk's query blocks */
    int32_t max_key_splits;                      /* split partials per row and head */
    int32_t chunk_query_blocks;                  /* 16-query blocks per wave of the chunk attention (1 or 2) */
    sarathi_gemm_plan qkv, o, up, down;          /* up: gate|up for LLAMA, up for GPT */
    sarathi_gemm_plan up_tail;                   /* all zero, or: up covers the first 256 weight stripes
                                                    (one round of fused tiles) and this split product
                                                    the remaining FFN columns */
    uint64_t workspace_bytes;                    /* as the matching *_workspace_size */
} sarathi_plan_info;     /* 200 bytes */

/* Fill *info for a forward over `batch`.  Errors: as the matching *_batch_check (without the x/y
 * requirement), or INVALID for a null info; *info is left unchanged then. */
sarathi_status sarathi_plan_describe(const sarathi_layer_desc *desc, const sarathi_batch *batch,
                                     sarathi_plan_info *info);
sarathi_status sarathi_multi_plan_describe(const sarathi_layer_desc *desc,
                                           const sarathi_multi_batch *batch, sarathi_plan_info *info);
sarathi_status sarathi_paged_plan_describe(const sarathi_layer_desc *desc,
                                           const sarathi_paged_batch *batch, sarathi_plan_info *info);

/* Static description of a status code. */
const char *sarathi_status_str(sarathi_status status);

/* Message of this thread's last failing call ("" if none). */
const char *sarathi_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SARATHI_H */
