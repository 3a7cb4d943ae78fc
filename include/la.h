/*
 * la.h — C ABI of the MI355X (gfx950) lookahead decoding library.
 *
 * One call of la_step runs one lookahead decoding step, the method of
 * "Break the Sequential Dependency of LLM Inference Using Lookahead
 * Decoding" (Fu, Bailis, Stoica, Zhang 2024), summary page, sections Summary
 * and Key points ("Tuning knobs").  In this library's words: a single forward
 * pass carries the current token, W x (N-1) rows of Jacobi guesses (the
 * lookahead window, whose diagonals become new n-grams for a per-token
 * n-gram store) and up to G stored n-grams that start with the current token;
 * the longest candidate prefix that agrees with the model's own next-token
 * choices is accepted, so the emitted tokens are those of plain decoding.
 * A step forwards 1 + (W + G)(N - 1) rows.
 * The model is a LLaMA-style decoder (pre-norm RMSNorm, rotary embedding on
 * adjacent dimension pairs, grouped KV heads, SwiGLU, untied LM head).
 *
 * Conventions
 *   - Every pointer documented as "device" is HIP device memory; "host" is
 *     ordinary host memory.  The library never allocates or frees device
 *     memory: the caller passes one workspace of la_workspace_bytes() bytes
 *     and owns the weights, the workspace and the stream; all must outlive
 *     the context.  The library allocates three small pinned host buffers
 *     per context (two step-result slots, so that two submitted steps never
 *     share one, and a staging buffer for prompts, windows and inspection)
 *     and frees them in la_destroy.
 *   - Every call returns la_status; nothing aborts and no exception crosses
 *     the ABI.  Arguments are validated before any HIP call.  After a HIP
 *     failure the context is poisoned: every later call except la_destroy
 *     returns LA_ERR_STATE.  la_last_error() describes the last failure.
 *   - A context is not thread-safe; use one context per stream.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct la_ctx la_ctx;

typedef enum {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = -1,     /* bad argument or configuration */
  LA_ERR_STATE = -2,           /* call out of order, or context poisoned */
  LA_ERR_OUT_OF_CAPACITY = -3, /* KV cache (max_ctx) or workspace too small */
  LA_ERR_HIP = -4,             /* a HIP runtime call failed */
  LA_ERR_UNSUPPORTED = -5      /* valid but not supported by the kernels */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rope_theta; /* rotary base, e.g. 10000 */
  float rms_eps;    /* RMSNorm epsilon, e.g. 1e-5 */
  int32_t W;        /* lookahead window (columns), >= 0 */
  int32_t N;        /* n-gram size, 2..32 */
  int32_t G;        /* verification size = candidates per step = pool cap per key */
  int32_t max_ctx;  /* KV capacity in tokens (prompt + generated + one step's rows) */
  int32_t dtype;    /* la_dtype of weights, activations and KV cache */
  int32_t batch;    /* B independent sequences stepped together (0 reads as 1);
                       each has its own KV cache, window, pool and current
                       token, and a step forwards B blocks of rows at once */
} la_config;
/* Supported shapes.  LA_BF16: head_dim 128, d_model % 128 == 0 and
 * <= 8192, d_ffn % 64 == 0, vocab % 128 == 0, max_ctx <= 2^24.  LA_F32 (small models): head_dim even and
 * <= 256, d_model, d_ffn and vocab even, max_ctx <= 16384.  Both:
 * n_heads % n_kv_heads == 0 and B (1 + (W + G)(N - 1)) <= 256 (B = batch).
 * W = G = 0 gives the plain one-token greedy decode step.
 *
 * Batch.  Sequence b's rows are rows b*T .. b*T + T - 1 of a step (T = rows
 * per sequence, la_step_rows); every sequence attends only to its own cache
 * and block, so each sequence decodes exactly as it would alone.  Arrays
 * that the calls below describe "per sequence" are laid out sequence by
 * sequence (sequence 0 first). */

/* Result of one step (host struct). */
typedef struct {
  int32_t n_emitted;  /* tokens emitted this step, k + 1, in [1, N] */
  int32_t tokens[32]; /* emitted tokens; tokens[n_emitted-1] is the new current token */
  int32_t accepted;   /* k: candidate tokens accepted by verification */
  int32_t winner;     /* g*: index of the accepted candidate, -1 if the pool had none */
  int32_t n_candidates; /* candidates verified this step (<= G) */
  int32_t kv_len;     /* committed KV length after the step */
} la_step_result;

/* Weights: an array of 3 + 9 * n_layers DEVICE pointers, each a row-major
 * tensor of the config's dtype ([out_features][in_features] for matrices):
 *   [0] tok_emb [vocab][d_model]   [1] final_norm [d_model]
 *   [2] lm_head [vocab][d_model]
 *   then for layer l at 3 + 9 l:  +0 attn_norm [d_model],
 *   +1 wq [n_heads*head_dim][d_model], +2 wk [n_kv_heads*head_dim][d_model],
 *   +3 wv [n_kv_heads*head_dim][d_model], +4 wo [d_model][n_heads*head_dim],
 *   +5 ffn_norm [d_model], +6 w_gate [d_ffn][d_model],
 *   +7 w_up [d_ffn][d_model], +8 w_down [d_model][d_ffn]. */

/* Bytes of DEVICE workspace a context needs (0 for an invalid config).
 * Holds the repacked weights (bf16), the KV cache, the n-gram pool, the
 * activations and scratch. */
size_t la_workspace_bytes(const la_config *cfg);

/* Create a context.  Validates cfg, carves the workspace, repacks the
 * weights into the workspace (bf16: MFMA operand tiles, fused QKV and
 * interleaved gate/up; f32: fused QKV), clears the cache and captures the
 * step as a HIP graph.  hip_stream: the hipStream_t all work is queued on
 * (NULL = the null stream).  Blocks until set-up is done.
 * Errors: LA_ERR_INVALID_ARG (cfg, NULL pointers), LA_ERR_UNSUPPORTED
 * (shape), LA_ERR_OUT_OF_CAPACITY (workspace_bytes too small), LA_ERR_HIP. */
la_status la_create(const la_config *cfg, const void *const *weights,
                    void *workspace, size_t workspace_bytes, void *hip_stream,
                    la_ctx **out);

/* Prefill sequence 0: empty its cache and pool, run the prompt (host int32
 * [n_prompt], ids < vocab) causally in chunks, install the initial window
 * (host int32 [(N-1)*W], level 1 first, then level 2, ...; required when
 * W > 0, ignored otherwise) and return the first generated token (the
 * prompt's greedy next token) in *first_token (host).  The first token
 * becomes the current token of the next step.
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_OUT_OF_CAPACITY (n_prompt + step rows >
 * max_ctx), LA_ERR_STATE (poisoned), LA_ERR_HIP. */
la_status la_prefill(la_ctx *c, const int32_t *prompt, int32_t n_prompt,
                     const int32_t *init_window, int32_t *first_token);
/* The same for sequence seq (0 <= seq < batch); la_prefill is seq 0.  Only
 * that sequence's cache, pool, window and state are reset.
 * Errors: as la_prefill, and LA_ERR_INVALID_ARG for seq out of range. */
la_status la_prefill_seq(la_ctx *c, int32_t seq, const int32_t *prompt, int32_t n_prompt,
                         const int32_t *init_window, int32_t *first_token);

/* One lookahead step of every sequence (blocks until the results are on the
 * host): out is host la_step_result [batch], one per sequence.
 * Errors: LA_ERR_STATE (a sequence not prefilled, or poisoned),
 * LA_ERR_OUT_OF_CAPACITY (some sequence's kv_len + step rows > max_ctx; no
 * sequence steps), LA_ERR_INVALID_ARG (out NULL), LA_ERR_HIP. */
la_status la_step(la_ctx *c, la_step_result *out);

/* Pipelined stepping, for a serving loop that should keep the GPU busy
 * while it reads results: la_step_submit enqueues the next step of every
 * sequence on the context's stream and returns at once; la_step_collect
 * blocks until the oldest submitted step has finished and writes its
 * results (host la_step_result [batch]), exactly those la_step would have
 * returned for it.  A step only needs the device state the step before it
 * left, so submitting step k+1 before collecting step k is allowed; at most
 * two steps may be in flight.  While any is in flight every other call on
 * the context but la_destroy returns LA_ERR_STATE.  The capacity check of
 * a submit assumes each step in flight commits its maximum of N tokens.
 * Errors: la_step_submit: LA_ERR_STATE (two in flight, a sequence not
 * prefilled, poisoned), LA_ERR_OUT_OF_CAPACITY, LA_ERR_HIP;
 * la_step_collect: LA_ERR_STATE (none in flight, poisoned),
 * LA_ERR_INVALID_ARG (out NULL), LA_ERR_HIP. */
la_status la_step_submit(la_ctx *c);
la_status la_step_collect(la_ctx *c, la_step_result *out);

/* Seed the n-gram pool with every N-gram of a token sequence (host int32
 * [n], ids < vocab), in position order: key seq[p], tail seq[p+1 .. p+N-1]
 * for p = 0 .. n-N, each inserted with the pool's policy (distinct tails per
 * key, a repeat moves to the newest slot, the oldest of G is evicted).
 * "Break the Sequential Dependency of LLM Inference Using Lookahead
 * Decoding", Key points, "Ablation": n-grams taken from the prompt raise
 * the speedup.  Call after la_prefill (which empties the pool), typically
 * with the prompt.  Blocks until done.
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_STATE (before prefill or poisoned),
 * LA_ERR_HIP. */
la_status la_seed_pool(la_ctx *c, const int32_t *seq, int32_t n);
/* The same for the pool of sequence s (0 <= s < batch); la_seed_pool is
 * s = 0.  Errors: as la_seed_pool, LA_ERR_INVALID_ARG for s out of range. */
la_status la_seed_pool_seq(la_ctx *c, int32_t s, const int32_t *seq, int32_t n);

/* Sampling for sequence seq (0 <= seq < batch), from the next decision on
 * (a prefill's first token included); kept across la_prefill_seq.
 * temperature 0 (the state after la_create) selects the argmax (greedy
 * decoding); temperature > 0 draws every emitted token: the tokens ordered
 * by logit (descending, lower id first on ties), cut to the first top_k
 * (0: no cut), weighted by exp((logit - max) / temperature), cut to the
 * shortest prefix holding top_p (in (0, 1], 1: no cut) of the weight, and
 * the first token whose running weight exceeds u times the total is drawn.
 * u for the token at sequence position n (the prompt holds positions
 * 0..n_prompt-1) is the top 24 bits of word 0 of Philox4x32-10 with counter
 * (n low, n high, 0, 0) and key (seed low, seed high), times 2^-24.  A
 * candidate token is accepted when it equals the draw at its position, so
 * the output is exactly that of plain sampled decoding with the same seed
 * (the method's pages: sampling is supported and the output distribution
 * is unchanged; the scheme itself is this library's reading).  The
 * lookahead window keeps taking the argmax.  Needs vocab <= 32768 when
 * temperature > 0.
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED (vocab), LA_ERR_STATE,
 * LA_ERR_HIP. */
la_status la_set_sampling(la_ctx *c, int32_t seq, float temperature, int32_t top_k,
                          float top_p, uint64_t seed);

/* Destroy a context (NULL is fine).  Waits for the context's queued work. */
la_status la_destroy(la_ctx *c);

const char *la_status_string(la_status s);
const char *la_last_error(const la_ctx *c);

/* Rows forwarded per step and sequence: 1 + (W + G)(N - 1). */
int32_t la_step_rows(const la_ctx *c);

/* ---- profiling ----------------------------------------------------------
 * Run one step like la_step (same kernels, same state change) but launched
 * directly rather than from the captured graph, with a HIP event recorded
 * on the context's stream before and after every kernel launch.  ms[k]
 * (host float [LA_PROF_CLASSES]) receives the summed event time of kernel
 * class k and launches[k] (host int32) the number of launches.  The event
 * pairs add small gaps, so the step itself runs slower than la_step.  out:
 * host la_step_result [batch] as for la_step. */
enum {
  LA_PROF_QKV = 0,    /* fused QKV projection */
  LA_PROF_ATTN = 1,   /* masked attention (+ split merge) */
  LA_PROF_O = 2,      /* output projection */
  LA_PROF_GATEUP = 3, /* fused gate/up projection with the SwiGLU */
  LA_PROF_DOWN = 4,   /* down projection */
  LA_PROF_LMHEAD = 5, /* LM head (logits) */
  LA_PROF_REDUCE = 6, /* split-K sums with fused epilogues (RoPE + KV write,
                         residual + RMSNorm) and RMSNorm kernels */
  LA_PROF_OTHER = 7,  /* assembly, token selection, verification, KV compaction */
  LA_PROF_CLASSES = 8
};
la_status la_profile_step(la_ctx *c, float *ms, int32_t *launches,
                          la_step_result *out);

/* Mean duration of one launch of a single kernel class, without per-launch
 * event overhead: the kernel(s) of class klass (LA_PROF_QKV, LA_PROF_ATTN,
 * LA_PROF_O, LA_PROF_GATEUP or LA_PROF_DOWN) launched reps times back to
 * back (1..100000), launch i on layer i % n_layers, on the context's current
 * buffers, between two HIP events on the context's stream; *us_per_launch
 * (host) receives the mean in microseconds.
 * The decoding state is unchanged (only scratch buffers that every step
 * rewrites are written).  bf16 contexts only, after la_prefill.
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_STATE, LA_ERR_UNSUPPORTED, LA_ERR_HIP. */
la_status la_profile_kernel(la_ctx *c, int32_t klass, int32_t reps,
                            float *us_per_launch);

/* ---- inspection (tests, debugging); each synchronizes the stream ------- */

/* Logits of the last step's rows, host float [batch * rows][vocab]; n =
 * element count of the buffer (must be >= batch * rows * vocab). */
la_status la_debug_logits(la_ctx *c, float *host, size_t n);
/* Tokens and per-row decisions (argmax, or draw when sampling) of the last
 * step, host int32 [batch * rows]
 * each (either may be NULL). */
la_status la_debug_block(la_ctx *c, int32_t *tokens, int32_t *amax);
/* Current windows, host int32 [batch][(N-1)*W] (level 1 first). */
la_status la_debug_window(la_ctx *c, int32_t *win);
/* Pools: host int32 len [batch][vocab] and tails [batch][vocab][G][N-1]
 * (oldest first). */
la_status la_debug_pool(la_ctx *c, int32_t *len, int32_t *tails);
/* Insert one n-gram tail (host int32 [N-1]) under key into sequence 0's
 * pool, with the pool's policy (tests plant candidates with it);
 * la_debug_pool_insert_seq does it for sequence s. */
la_status la_debug_pool_insert(la_ctx *c, int32_t key, const int32_t *tail);
la_status la_debug_pool_insert_seq(la_ctx *c, int32_t s, int32_t key, const int32_t *tail);
/* Cached K and V of positions pos0..pos0+n-1 of one layer as host float
 * [batch][n_kv_heads][n][head_dim] each. */
la_status la_debug_kv(la_ctx *c, int32_t layer, int32_t pos0, int32_t n,
                      float *k, float *v);
/* Committed length and current token of each sequence, host int32 [batch]
 * each (either may be NULL). */
la_status la_debug_state(la_ctx *c, int32_t *kv_len, int32_t *current);

/* ---- one layer's masked attention on its own ---------------------------
 * The attention of a lookahead step ("Summary": both branches in one pass)
 * for the bf16 kernel: query rows in the step's row order (current token,
 * window rows level by level, candidate rows candidate by candidate); each
 * row sees cache positions 0..prefix_len-1 and the block rows the
 * lookahead/verification mask allows; block row r's key/value sit at cache
 * position prefix_len + r.
 *   q        DEVICE bf16 [rows][n_heads][128], rows = 1 + (W+G)(N-1)
 *   k_cache  DEVICE bf16 [n_kv_heads][ctx_stride][128]
 *   vt_cache DEVICE bf16 [n_kv_heads][128][ctx_stride] (V transposed)
 *   out      DEVICE bf16 [rows][n_heads][128]
 *   ctx_stride % 64 == 0 and prefix_len + rows <= ctx_stride.
 *   workspace: DEVICE, la_attention_workspace_bytes() bytes (split-KV
 *   partial results); stream: hipStream_t or NULL.  Asynchronous.
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED (head_dim != 128 or
 * ctx_stride > 2^24),
 * LA_ERR_OUT_OF_CAPACITY (workspace too small), LA_ERR_HIP. */
size_t la_attention_workspace_bytes(int32_t n_heads, int32_t head_dim,
                                    int32_t ctx_stride, int32_t W, int32_t N,
                                    int32_t G);
la_status la_attention(const void *q, const void *k_cache,
                       const void *vt_cache, void *out, int32_t n_heads,
                       int32_t n_kv_heads, int32_t head_dim,
                       int32_t prefix_len, int32_t ctx_stride, int32_t W,
                       int32_t N, int32_t G, void *workspace,
                       size_t workspace_bytes, void *stream);

/* The same call for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; the split-KV partials go to a scratch array the
 * library holds in device memory, LA_ATTENTION_NOALLOC_SCRATCH_BYTES per
 * GPU, for the life of the process.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (concurrent
 * streams, threads) race and must be serialized by the caller; nothing in
 * the array needs to start at zero.  Arguments, layouts and results as
 * la_attention.
 * Errors: as la_attention; LA_ERR_OUT_OF_CAPACITY when the call needs more
 * than LA_ATTENTION_NOALLOC_SCRATCH_BYTES (la_attention_workspace_bytes
 * larger), before any HIP call; LA_ERR_HIP if the array's address cannot be
 * resolved. */
#define LA_ATTENTION_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
la_status la_attention_noalloc(const void *q, const void *k_cache,
                               const void *vt_cache, void *out, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               int32_t prefix_len, int32_t ctx_stride, int32_t W,
                               int32_t N, int32_t G, void *stream);

/* ---- one draw per row on its own ---------------------------------------
 * The draw la_set_sampling describes (temperature > 0), for rows of
 * logits: out[r] = the token drawn from logits[r] with the uniform of
 * sequence position positions[r].  Queued on the hipStream_t stream (NULL:
 * the null stream), not waited for.
 *   logits     DEVICE float [rows][vocab], vocab <= 32768
 *   positions  DEVICE int64 [rows]
 *   out        DEVICE int32 [rows]
 * Errors: LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED (vocab), LA_ERR_HIP. */
la_status la_sample(const float *logits, int32_t rows, int32_t vocab, float temperature,
                    int32_t top_k, float top_p, uint64_t seed, const int64_t *positions,
                    int32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LA_H */
