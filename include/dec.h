/*
 * dec.h -- C ABI of the decoder forward pass on one AMD MI355X (gfx950).
 *
 * The library runs the forward pass of a pre-norm decoder with the Qwen3
 * switches: token ids -> tied embedding -> n_layers x [RMSNorm -> Q/K/V
 * projections (Q wider than the residual stream) -> per-head q/k RMSNorm ->
 * split-halves RoPE at absolute positions -> paged KV write -> causal
 * grouped-query attention -> output projection + residual -> RMSNorm ->
 * SwiGLU + residual] -> final RMSNorm -> tied LM head -> float32 logits.
 * Passages that define each step:
 *   - "Candle model runner (Llama + bigram, int4), Rust KV cache, sampler and
 *     PCG32", section 2.4 "The Llama forward, one step" (symbols table,
 *     RMSNorm / projection / attention / SwiGLU equations, paged KV
 *     placement, last-token LM head) and section 4 "The interface" (a step
 *     is a batch of sequences, each a run of new tokens at absolute
 *     positions; forward writes K and V into the blocks its table names; the
 *     caller allocates the blocks).
 *   - "A real model in our own decoder", section "Same design, bigger
 *     numbers, five switches" (head_dim, ff_hidden, rope_base, rope_split,
 *     qk_norm) and the qwen_config whitelist; section "Which channels rotate
 *     together" (channel j pairs with j + head_dim/2).
 *   - "Proving it's the same model", section "Every logit, every position"
 *     (logits at every position) and "Remove every source of noise first"
 *     (full path and cached path).
 *   - "Byte-identical: 1,000 tokens of proof", section "The bar we set"
 *     (uint4 weights W = (q - zp) * scale) and "The rope table that was too
 *     accurate" (angle pos * base^(-2j/head_dim)).
 *
 * Memory ownership. The caller allocates every device buffer (weights blob,
 * KV pool, workspace, logits, next-token ids) and keeps it alive until
 * dec_free. The library never frees or reallocates them. A dec_ctx owns only
 * host memory (a pinned staging ring for per-call metadata and the RoPE
 * table) and HIP events. Host arrays passed to a call are read during the
 * call only.
 *
 * Streams. `stream` is a hipStream_t passed as void* (NULL = the default
 * stream). Every call enqueues its work on that stream and returns without
 * waiting for it; the caller synchronises before reading results. One host
 * thread may use a ctx at a time. Calls on one ctx must be issued on one
 * stream, or the caller must order them: they share the ctx's workspace.
 *
 * Errors. Functions return DEC_OK (0) or a negative DEC_E_* code. Every
 * argument, size, token id, position and block id is validated on the host
 * before any work is enqueued, so a rejected call leaves the KV pool and the
 * outputs untouched ("Candle model runner", section 4, test
 * forward_refuses_bad_batches: a short block table or a position past the
 * context is an error; pitfall s21: token ids are checked against the
 * vocabulary). dec_last_error returns a message for the last failure.
 */
#ifndef DEC_H
#define DEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- codes ---------------------------------------------------------------------- */

#define DEC_OK 0
#define DEC_E_ARG (-1)         /* null pointer, non-positive count, misaligned buffer */
#define DEC_E_UNSUPPORTED (-2) /* configuration outside what the library runs */
#define DEC_E_CAPACITY (-3)    /* more rows/sequences than configured, buffer too small */
#define DEC_E_BLOCK (-4)       /* block id >= n_blocks, or block table too short */
#define DEC_E_POSITION (-5)    /* a position at or past max_context */
#define DEC_E_TOKEN (-6)       /* token id outside [0, vocab) */
#define DEC_E_HIP (-7)         /* a HIP runtime call failed */

/* storage formats */
#define DEC_F32 0
#define DEC_BF16 1
#define DEC_F16 2
#define DEC_UINT4_G32 3 /* 4-bit codes, bf16 scale and bf16 zero point per 32 input columns */
#define DEC_INT4_SYM_G32 4 /* signed 4-bit values, f16 scale per 32 input columns, no zero point */

/* which rows get logits */
#define DEC_LOGITS_ALL 0  /* every new row, in batch order: [sum n_new][vocab] */
#define DEC_LOGITS_LAST 1 /* each sequence's last new row: [n_seqs][vocab] */
#define DEC_LOGITS_NONE 2 /* no logits (KV cache is still written) */

/* ---- configuration ----------------------------------------------------------------- */

/*
 * Model and memory configuration. Accepted only with the switches of the
 * Qwen3 layout: rope_split = 1 (pairs j, j + head_dim/2), qk_norm = 1,
 * tie_embeddings = 1; anything else is refused at dec_init, never served
 * wrong ("Candle model runner" section 2.3; "A real model in our own
 * decoder", qwen_config). Size rules: d_model, n_heads*head_dim and ff_hidden
 * multiples of 64; head_dim in {32, 64, 128}; n_heads a multiple of
 * n_kv_heads; block_tokens in {16, 32, 64}.
 */
typedef struct dec_config {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ff_hidden;
  int32_t vocab;
  int32_t max_context; /* positions 0 .. max_context-1 are valid */
  float rms_eps;       /* used by all four norms (attention, q/k, ffn, final) */
  double rope_base;
  int32_t rope_split;     /* must be 1 */
  int32_t qk_norm;        /* must be 1 */
  int32_t tie_embeddings; /* must be 1 */
  int32_t weight_dtype;   /* DEC_F32 | DEC_BF16 | DEC_UINT4_G32 | DEC_INT4_SYM_G32 */
  int32_t kv_dtype;       /* DEC_F32 | DEC_F16 */
  int32_t block_tokens;   /* B: positions per KV block */
  int32_t n_blocks;       /* blocks in the KV pool */
  int32_t max_rows;       /* most new tokens in one call (sizes the workspace) */
  int32_t max_seqs;       /* most sequences in one call */
} dec_config;

/* Host-only check of a configuration; DEC_OK or DEC_E_UNSUPPORTED / DEC_E_ARG. */
int dec_check_config(const dec_config* cfg);

/* ---- memory layout ----------------------------------------------------------------- */

/*
 * Weights blob. One device buffer holding, at 256-byte aligned offsets, in this
 * order: E [vocab][d_model] (the tied embedding, also the LM head); for each
 * layer: attn_norm [d], W_q [H*D][d], W_k [Hkv*D][d], W_v [Hkv*D][d],
 * q_norm [D], k_norm [D], W_o [d][H*D], ffn_norm [d], W_gate [ff][d],
 * W_up [ff][d], W_down [d][ff]; then final_norm [d]. Matrices are [out][in]
 * row-major ("Candle model runner" 2.4: W stored [out, in], y = x W^T) in
 * weight_dtype; gains are float32. A DEC_UINT4_G32 matrix is three arrays:
 * codes uint8 [out][in/2] (column 2b in the low nibble, 2b+1 in the high
 * nibble, the order of "Candle model runner" 2.5), then scale bf16
 * [out][in/32], then zero point bf16 [out][in/32]; element (o, i) is
 * (code - zp[o][i/32]) * scale[o][i/32].
 * A DEC_INT4_SYM_G32 matrix is two arrays ("Candle model runner" 2.5, the
 * symmetric int4-g format): values uint8 [out][in/2], each nibble a 4-bit
 * two's complement integer q in [-8, 7] in the same column order, then scale
 * f16 [out][in/32]; element (o, i) is q * scale[o][i/32], exact in float32.
 * Its entries report zp_offset = 0.
 * The library only reads the blob.
 */
size_t dec_weight_bytes(const dec_config* cfg);

/* One entry of the blob, by index 0 .. dec_weight_count(cfg)-1 in the order above. */
typedef struct dec_weight_info {
  char name[32];      /* "embed", "attn_norm", "wq", ..., "final_norm" */
  int32_t layer;      /* -1 for embed / final_norm */
  int32_t dtype;      /* DEC_F32 (gains) or the config's weight_dtype (matrices) */
  int64_t rows, cols; /* logical shape; gains are [1][n] */
  size_t offset;      /* byte offset of the data (codes, for 4-bit formats) */
  size_t bytes;       /* bytes of the data (codes, for 4-bit formats) */
  size_t scale_offset, zp_offset; /* 4-bit formats: byte offsets of scale and zero point (0: none) */
  size_t group_bytes;             /* 4-bit formats: bytes of the scales (and of the zero points) */
} dec_weight_info;
int dec_weight_count(const dec_config* cfg);
int dec_weight_entry(const dec_config* cfg, int index, dec_weight_info* out);

/*
 * KV pool: [n_layers][2 (K, V)][n_blocks][n_kv_heads][block_tokens][head_dim]
 * of kv_dtype, so one block's slab of one layer's K is [H_kv][B][D] ("Candle
 * model runner" section 3, "Where a key lands": position j of a sequence is
 * block floor(j/B) of its table, slot j mod B, and KV head h's key starts at
 * element (h*B + slot)*D of the slab). f16 values are the round-to-nearest-
 * even conversion of the float32 key/value.
 */
size_t dec_kv_pool_bytes(const dec_config* cfg);

/* Scratch device memory for activations and per-call metadata (caller-owned). */
size_t dec_workspace_bytes(const dec_config* cfg);

/* ---- lifetime ---------------------------------------------------------------------- */

typedef struct dec_ctx dec_ctx;

/*
 * Bind a configuration to caller-owned device buffers: the runner's load step
 * ("Candle model runner", section 4, the ModelRunner interface: a runner is
 * built once from a model and its configuration, and a failure comes back as a
 * result rather than a crash). Here the model arrives as a packed weights blob,
 * and every device buffer belongs to the caller, as the pool's blocks do on
 * that page (the caller allocates the blocks the forward writes into).
 * Checks the config and that each buffer is at least the size above and
 * 256-byte aligned, builds the RoPE cos/sin table (angles in double precision,
 * stored float32) and uploads it into the workspace on `stream`. The weights
 * blob is not modified. On success *out is a new context; on failure *out is
 * NULL and dec_last_error(NULL) holds the reason.
 */
int dec_init(const dec_config* cfg, const void* weights, size_t weight_bytes, void* kv_pool,
             size_t kv_bytes, void* workspace, size_t workspace_bytes, void* stream,
             dec_ctx** out);

/*
 * End a context ("Candle model runner", section 4: the runner owns its own state;
 * the caller owns the blocks): releases the context's host memory and events.
 * Device buffers stay with the caller. NULL is a no-op.
 */
void dec_free(dec_ctx* ctx);

/*
 * Message of the last failure of a call on ctx (or, for ctx == NULL, of the
 * calling thread's last dec_init or context-free call). The runner's operations report invalid
 * dimensions, exhausted capacity, invalid block ids and format errors as
 * results ("Candle model runner", section 2.2); here the kind is the DEC_E_*
 * code returned by the call and this string names the check that failed. The
 * string stays valid until the next call on the same context.
 */
const char* dec_last_error(const dec_ctx* ctx);

/* ---- forward ----------------------------------------------------------------------- */

/*
 * One forward step over a batch of n_seqs sequences (prefill, chunked prefill
 * or a cached continuation). Sequence s brings n_new[s] >= 1 new tokens that
 * sit at absolute positions start[s] .. start[s]+n_new[s]-1; its keys and
 * values for positions < start[s] must already be in the pool (from earlier
 * calls), and this call writes those of the new positions. Rows are ordered
 * sequence by sequence (batch order).
 *   start, n_new:  host int32 [n_seqs]
 *   tokens:        host int32 [sum n_new], batch order
 *   block_tables:  host int32 [n_seqs][max_blocks], row-major; entries
 *                  0 .. ceil((start+n_new)/B)-1 of each row are used
 *   logits:        device float32 [sum n_new][vocab] (ALL), [n_seqs][vocab]
 *                  (LAST), or NULL (NONE)
 *   next_tokens:   device int32, one per logits row, or NULL: greedy choice,
 *                  the argmax of the row with ties to the lowest id ("Candle
 *                  model runner" section 2.6); needs logits.
 * A row's results do not depend on which other sequences share the call or
 * where it sits in the batch: bit for bit ("Candle model runner" 2.4,
 * batch invariance).
 */
int dec_prefill(dec_ctx* ctx, void* stream, int32_t n_seqs, const int32_t* start,
                const int32_t* n_new, const int32_t* tokens, const int32_t* block_tables,
                int32_t max_blocks, int32_t logits_mode, float* logits, int32_t* next_tokens);

/*
 * One decode step: one new token per sequence at position positions[s] (the
 * sequence's current length). Token ids come from host memory (tokens_host,
 * checked against the vocabulary) or from device memory (tokens_device, e.g.
 * the next_tokens of the previous step; exactly one of the two is non-NULL;
 * an out-of-range device id makes that row's logits NaN).
 *   logits:      device float32 [n_seqs][vocab], or NULL
 *   next_tokens: device int32 [n_seqs] or NULL: greedy choice, the argmax of
 *                the row with ties to the lowest id ("Candle model runner"
 *                section 2.6); needs logits != NULL.
 * As in dec_prefill, a row's results do not depend on the other sequences of
 * the call, bit for bit. The attention over a row with more than 4,096 keys
 * before its position is computed in 4,096-key segments merged in order; the
 * segmentation depends on that position alone.
 */
int dec_decode_step(dec_ctx* ctx, void* stream, int32_t n_seqs, const int32_t* tokens_host,
                    const int32_t* tokens_device, const int32_t* positions,
                    const int32_t* block_tables, int32_t max_blocks, float* logits,
                    int32_t* next_tokens);

/*
 * dec_decode_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). The same
 * kernels, arguments, checks and results as dec_decode_step, bit for bit, but the
 * step's per-call scratch (its uploaded metadata, the activations, the split
 * attention states and the greedy candidates) lives in a static device array of
 * DEC_STATIC_SCRATCH_BYTES that the library holds on each device until the
 * process ends, not in the ctx's workspace (the ctx's workspace still holds the
 * RoPE table). Nothing is allocated and nothing needs to start at zero.
 * Every call on one device shares that device's array: calls that overlap on a
 * device (on different streams, or from several ctxs or threads without
 * ordering) race and give wrong results. DEC_E_CAPACITY when the step needs more
 * than DEC_STATIC_SCRATCH_BYTES (the need grows with n_seqs, the model's widths
 * and max_context); DEC_E_HIP when the array's device address is unknown.
 */
#define DEC_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int dec_decode_step_static(dec_ctx* ctx, void* stream, int32_t n_seqs, const int32_t* tokens_host,
                           const int32_t* tokens_device, const int32_t* positions,
                           const int32_t* block_tables, int32_t max_blocks, float* logits,
                           int32_t* next_tokens);

/*
 * Host-only validation of a step, exactly as dec_prefill performs it before
 * enqueuing anything (for callers and tests without a GPU). For a decode step
 * pass n_new = NULL (one token each) and positions as start. tokens may be
 * NULL to skip the id check. Returns DEC_OK or the code dec_prefill would
 * return; `msg` (may be NULL) receives the message.
 */
int dec_check_step(const dec_config* cfg, int32_t n_seqs, const int32_t* start,
                   const int32_t* n_new, const int32_t* tokens, const int32_t* block_tables,
                   int32_t max_blocks, int32_t logits_mode, char* msg, size_t msg_len);

/*
 * Test hook: write weight entry `index` (a matrix) as float32 [rows][cols] to
 * device memory `out`, widened/dequantised by the same device code the
 * projections and the embedding use (uint4: t = f32(q) - f32(zp), then
 * w = t * f32(scale), no fused multiply-add).
 */
int dec_debug_dequant(dec_ctx* ctx, void* stream, int index, float* out);

/*
 * Quantise a float32 matrix to the DEC_INT4_SYM_G32 layout on the device (the
 * runner's quantise-at-load route, "Candle model runner" 2.5): per group of 32
 * columns s = f16(max |W| / 7) (rounded to nearest even), q = clamp(rint(W /
 * s), -8, 7) with the stored s, in float32; a group of zeros stores s = 0 and
 * q = 0 (W / s is undefined there).
 *   w:     device float32 [rows][cols], 16-byte aligned; cols % 32 == 0
 *   q:     device uint8 [rows][cols/2], 16-byte aligned (column 2b in the low
 *          nibble, 2b + 1 in the high nibble, 4-bit two's complement)
 *   scale: device f16 bits [rows][cols/32]
 * Asynchronous on `stream`. DEC_E_ARG for NULL, misaligned or misshaped
 * arguments (message: dec_last_error(NULL)).
 */
int dec_quantize_int4_sym(void* stream, const float* w, int64_t rows, int64_t cols, uint8_t* q, uint16_t* scale);

/* ---- seeded sampling ------------------------------------------------------------------ */

/* Sampling parameters of one sequence ("Candle model runner" section 2.6, SamplingParams). */
typedef struct dec_sampling {
  double temperature;        /* >= 0; 0 is greedy: the largest value, ties to the lowest id, no draw */
  double top_p;              /* in (0, 1]; 1 keeps every id */
  double min_p;              /* in [0, 1]; 0 keeps every id */
  double repetition_penalty; /* > 0; 1 leaves the logits as they are */
  double presence_penalty;   /* finite; 0 for none */
  double frequency_penalty;  /* finite; 0 for none */
  int32_t top_k;             /* >= 0; 0 keeps every id */
  int32_t reserved;          /* must be 0 */
} dec_sampling;

/* A sequence's history: its prompt ids and its output ids so far, as ranges of one id array. */
typedef struct dec_history {
  int32_t prompt_offset, prompt_len;
  int32_t output_offset, output_len;
} dec_history;

#define DEC_PURPOSE_SAMPLE 4       /* the purpose id of the sampling stream */
#define DEC_SAMPLE_MAX_NUCLEUS 1024 /* most ids the nucleus step orders one by one; beyond, its cut
                                       is found by a radix descent over the whole vocabulary */

/*
 * Host only: state_inc[0], state_inc[1] = the PCG32 state and increment of the
 * request stream stream(seed, purpose) ("Candle model runner" section 2.6):
 * pcg32_srandom_r(child_seed(seed, purpose), purpose) with child_seed(s, p) =
 * mix64(s + p * 0x9E3779B97F4A7C15), mix64 the splitmix64 finaliser. Pass
 * DEC_PURPOSE_SAMPLE for sampling; copy the pair into dec_sample's rng array.
 */
void dec_rng_stream(uint64_t seed, uint64_t purpose, uint64_t state_inc[2]);

/*
 * One token per sequence from a row of logits (for example dec_decode_step's
 * logits), drawn on the device in float64 in the order of "Candle model
 * runner" section 2.6: widen; repetition penalty over the distinct ids of
 * prompt and output (a positive value divided by it, any other multiplied);
 * presence and frequency penalties over the output only (an id seen c > 0
 * times loses frequency * c + presence); the logprob is log softmax of these
 * values; temperature 0 takes the largest value (ties to the lowest id) with no
 * draw; otherwise divide by the temperature, keep the top_k by (value
 * descending, id ascending), keep the nucleus (in that order, up to and
 * including the id whose cumulative probability reaches top_p), keep the ids
 * whose probability is at least min_p times the largest, take the softmax over
 * the kept ids in ascending id order, draw one uniform u from the sequence's
 * stream and return the first id in ascending order whose cumulative
 * probability exceeds u. The probabilities of the top-p and min-p steps are
 * over the ids top_k kept.
 *   logits:   device float32 [n_seqs][ld], ld >= vocab; row s for sequence s
 *   params:   host [n_seqs]
 *   history:  host [n_seqs]; ranges into ids: offset >= 0, len >= 0,
 *             offset + len <= n_ids
 *   ids:      device int32 [n_ids] (NULL when n_ids == 0); ids outside
 *             [0, vocab) are ignored
 *   rng:      device uint64 [n_seqs][2]: each sequence's PCG32 (state,
 *             increment), from dec_rng_stream; a sampled row advances it by one
 *             uniform (two outputs), a greedy row leaves it as it is
 *   next:     device int32 [n_seqs]
 *   logprob:  device float64 [n_seqs] or NULL
 * Sums over the at most DEC_SAMPLE_MAX_NUCLEUS ids of the nucleus path are
 * left-to-right in ascending id order; sums over the whole vocabulary run
 * left to right within fixed id ranges, then over the ranges in order (equal
 * to a left-to-right sum up to rounding). When top_k keeps more than
 * DEC_SAMPLE_MAX_NUCLEUS ids (top_k = 0 or top_k >= vocab keep all of them) and
 * top_p < 1, the nucleus's cumulative probability is taken over groups of ids
 * of equal leading key bits in a fixed order (equal to the walk's
 * left-to-right sum up to rounding); the same inputs always give the same
 * token. Uses the workspace: a count table per sequence that every call leaves
 * zero, so calls on one context must not overlap. Asynchronous on `stream`.
 * Errors (checked on the host before anything is enqueued): DEC_E_ARG (a
 * NULL pointer, a bad range, a parameter outside the ranges above),
 * DEC_E_CAPACITY (n_seqs > max_seqs), DEC_E_UNSUPPORTED (vocab > 262,144).
 */
int dec_sample(dec_ctx* ctx, void* stream, int32_t n_seqs, const float* logits, int64_t ld,
               const dec_sampling* params, const dec_history* history, const int32_t* ids,
               int64_t n_ids, uint64_t* rng, int32_t* next, double* logprob);

/* ---- KV block manager (host only) ------------------------------------------------------ */

/*
 * A manager of the pool's block ids ("Candle model runner" section 2.2, KvPool:
 * references per block, a prefix index, an LRU cache of released full blocks,
 * and the KvPool interface of section 4; tests kv_pool_bounds_and_cache_
 * lifecycle, kv_pool_evicts_the_oldest_cached_block, kv_pool_rejects_zero_
 * capacity). It keeps host state only and is independent of any dec_ctx;
 * callers pass the ids it hands out in their block tables. A block is FREE,
 * USED (reference count >= 1) or CACHED (released while registered, with
 * prefix caching on).
 *   create:   n_blocks >= 1 (a pool without blocks is refused), block_tokens
 *             >= 1; prefix_cache != 0 keeps released registered blocks
 *   alloc:    n blocks, all or nothing: free blocks lowest id first, then the
 *             oldest cached blocks (evicted from the index); each USED with
 *             reference 1 and fill 0; DEC_E_CAPACITY when free + cached < n
 *   retain / release: reference +1 / -1 of a USED block; at 0 a registered
 *             block becomes CACHED (newest in the LRU) when prefix caching is
 *             on, any other block FREE
 *   set_fill: tokens held by a USED block, 0 .. block_tokens (a registered
 *             block stays full)
 *   register: index a full USED block under a prefix key; when the key is
 *             already indexed to another block that block stays its entry and
 *             *canonical names it; a block registered under one key is refused
 *             another (DEC_E_ARG; the same key again is accepted)
 *   lookup:   *id = the block indexed under key (retained; a CACHED block is
 *             reacquired with reference 1), or -1; a FREE block is never returned
 * Errors: DEC_E_ARG, DEC_E_CAPACITY, DEC_E_BLOCK (an id that is not USED);
 * a failed call changes nothing. Not thread-safe: one caller at a time.
 */
typedef struct dec_block_pool dec_block_pool;
#define DEC_BLOCK_FREE 0
#define DEC_BLOCK_USED 1
#define DEC_BLOCK_CACHED 2
int dec_pool_create(int32_t n_blocks, int32_t block_tokens, int32_t prefix_cache, dec_block_pool** out);
void dec_pool_destroy(dec_block_pool* pool);
const char* dec_pool_last_error(const dec_block_pool* pool);
int dec_pool_alloc(dec_block_pool* pool, int32_t n, int32_t* ids);
int dec_pool_retain(dec_block_pool* pool, int32_t id);
int dec_pool_release(dec_block_pool* pool, int32_t id);
int dec_pool_set_fill(dec_block_pool* pool, int32_t id, int32_t n);
int dec_pool_register(dec_block_pool* pool, int32_t id, uint64_t key, int32_t* canonical);
int dec_pool_lookup(dec_block_pool* pool, uint64_t key, int32_t* id);
int dec_pool_block_info(const dec_block_pool* pool, int32_t id, int32_t* state, int32_t* ref, int32_t* fill);
void dec_pool_counts(const dec_block_pool* pool, int32_t* n_free, int32_t* n_used, int32_t* n_cached);

/*
 * Prefix key of a block: a 64-bit hash of the parent block's key (0 for the
 * first block) and the block's n token ids, so equal keys mean equal token
 * prefixes up to hash collisions (FNV-1a over the bytes, then the splitmix64
 * finaliser).
 */
uint64_t dec_prefix_key(uint64_t parent, const int32_t* tokens, int32_t n);

/*
 * Export / import of blocks' K and V data (the KvPool export/import of section
 * 4; test kv_pool_exports_and_imports_rust_owned_blocks). The envelope is a
 * header (magic "DECKVB01", n_layers, n_kv_heads, block_tokens, head_dim,
 * kv_dtype, n as int32), the n fills (int32), then per block and per layer its
 * K slab and its V slab ([H_kv][B][D] of the KV dtype each, the pool's own
 * bytes). Both calls copy between ctx's device pool and the host buffer on
 * `stream` and return after the copies are done.
 *   export: ids / fills host [n] (ids < n_blocks, fills <= block_tokens);
 *           buf of at least dec_kv_export_bytes(ctx, n) bytes
 *   import: buf as written by export for a pool of the same block format
 *           (else DEC_E_UNSUPPORTED); ids: host [n] destination blocks (the
 *           caller allocates them); fills (may be NULL): host [n], receives
 *           the envelope's fills
 */
size_t dec_kv_export_bytes(const dec_ctx* ctx, int32_t n);
int dec_kv_export(dec_ctx* ctx, void* stream, const int32_t* ids, const int32_t* fills, int32_t n, void* buf,
                  size_t buf_bytes);
int dec_kv_import(dec_ctx* ctx, void* stream, const void* buf, size_t buf_bytes, const int32_t* ids, int32_t n,
                  int32_t* fills);

/* ---- checkpoint loading (host only) ---------------------------------------------------- */

/*
 * config.json of a Qwen3 model -> the shape fields of *cfg (vocab, max_context
 * from max_position_embeddings, d_model, n_heads, n_layers, n_kv_heads,
 * head_dim, ff_hidden, rms_eps, rope_base; the three switches set to 1). The
 * settings "A real model in our own decoder" whitelists (qwen_config) must
 * hold: model_type "qwen3", hidden_act "silu", attention_bias false,
 * attention_dropout 0, rope_scaling null, use_sliding_window false,
 * tie_word_embeddings true, rms_norm_eps 1e-6; else DEC_E_UNSUPPORTED (refused
 * at load, never served wrong: "Candle model runner" 2.3). The memory fields
 * (dtypes, pool, rows) are left as the caller set them. `msg` (may be NULL)
 * receives the reason of a refusal.
 */
int dec_config_from_json(const char* json, size_t len, dec_config* cfg, char* msg, size_t msg_len);

/*
 * model.safetensors at `path` -> the weights blob in host memory (blob_bytes >=
 * dec_weight_bytes(cfg); the caller uploads it), for weight_dtype DEC_F32 or
 * DEC_BF16. The file is a little-endian u64 header length N, N bytes of JSON,
 * then the data buffer ("A real model in our own decoder", section "A
 * safetensors file is a JSON header and raw bytes"). Refused with DEC_E_ARG: N
 * outside [2, min(1e8, file size - 8)], a header that is not one object,
 * duplicate keys, metadata that is not strings, an unknown dtype, a byte count
 * that does not match the shape, ranges (from the start of the data buffer)
 * that overlap, leave a gap or do not end at the end of the file, a missing or
 * unexpected tensor, a shape mismatch, and an lm_head.weight whose values
 * differ from the embedding's (the tied matrix stored twice is accepted when
 * equal). F16 and BF16 tensors are widened to float32 ("Candle model runner"
 * 2.3); a bf16 blob stores BF16 tensors as they are and rounds others to
 * nearest even. Tensor names are Hugging Face's Qwen3 names
 * (model.embed_tokens.weight, model.layers.<l>.self_attn.q_proj.weight, ...,
 * model.norm.weight).
 */
int dec_load_safetensors(const char* path, const dec_config* cfg, void* blob, size_t blob_bytes, char* msg,
                         size_t msg_len);

/* ---- per-kernel timing (diagnostics) ------------------------------------------------ */

/* kernel classes */
#define DEC_K_EMBED 0
#define DEC_K_RMSNORM 1
#define DEC_K_GEMM_QKV 2
#define DEC_K_QK_ROPE_KV 3
#define DEC_K_ATTN_PREFILL 4 /* tile attention of prefill calls (f16 pool) */
#define DEC_K_ATTN_ROWS 5    /* split-key attention of decode steps (and float32-pool prefill) */
#define DEC_K_ATTN_COMBINE 6
#define DEC_K_GEMM_O 7
#define DEC_K_GEMM_GATEUP 8
#define DEC_K_GEMM_DOWN 9
#define DEC_K_GEMM_LMHEAD 10
#define DEC_K_ARGMAX 11
#define DEC_K_WIDEN 12 /* 4-bit weights widened to bf16 for a prefill call of many rows */
#define DEC_K_COUNT 13

/*
 * Bracket every later launch of the kernel classes in `class_mask` (bit k =
 * class k) with a pair of HIP events on the call's stream; 0 turns timing
 * off. Recorded launches accumulate until dec_timing_read.
 */
int dec_timing_enable(dec_ctx* ctx, uint32_t class_mask);

/*
 * Wait for the recorded launches of `kernel_class`, return the sum of their
 * durations in milliseconds and their count, and forget them.
 */
int dec_timing_read(dec_ctx* ctx, int kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* DEC_H */
