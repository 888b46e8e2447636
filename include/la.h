/*
 * la.h -- C ABI of the MI355X lookahead decoding library (liblookahead.so).
 *
 * Exact Lookahead decoding as described on "M7.3 - Lookahead Decoding:
 * Jacobi Iterations, N-Gram Pools, and Parallel Verification" and in "Break
 * the Sequential Dependency of LLM Inference Using Lookahead Decoding":
 * one causal target forward per round updates a W-wide, (N-1)-level Jacobi
 * trajectory window and verifies up to G candidate n-grams, taken from a
 * keyed n-gram pool, against one committed prefix, then publishes exactly
 * the greedy (or exactly sampled) tokens.  The round follows the pages'
 * predict -> collect -> verify -> publish state machine (M7.3, 0x00 and
 * 0x03A lifecycle steps 1-8).
 *
 * Conventions for every function:
 *   - Return value: LA_OK (0) or a negative LA_E* code.  On error nothing is
 *     published: output tokens, committed K/V length, window and pool keep
 *     their previous contents (M7.3, 0x07 fail-closed publication).  A
 *     message is available from la_last_error(ctx) (ctx may be NULL for the
 *     context-free calls; the message is then per thread).
 *   - "device" pointers are HIP device addresses on the current device;
 *     "host" pointers are ordinary host memory and are only read/written
 *     during the call.  The library never frees caller memory; it borrows
 *     the device buffers passed to la_init until la_destroy.
 *   - stream: a hipStream_t (passed as void*); all device work of a call is
 *     ordered on it.  Calls that return host data synchronise that stream.
 *   - A context serves one request and is not thread-safe.
 *   - Token ids are int32 in [0, vocab).  Tensor layouts are row-major.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------------- errors */
#define LA_OK 0
#define LA_EINVAL (-1)    /* bad argument: N < 3 or not admitted, W < 1, G < 0, sizes out of range */
#define LA_ESTATE (-2)    /* call out of order, or an accept record from another round */
#define LA_EPLAN (-3)     /* publication plan fails validation (winner/h/emitted inconsistent) */
#define LA_EOVERFLOW (-4) /* K/V capacity, output capacity or a buffer too small */
#define LA_EDEVICE (-5)   /* a HIP call failed */

#define LA_MAX_N 16       /* N <= 16, so S = N - 1 <= 15 and a round emits <= N tokens */
#define LA_MAX_EMIT 32

enum { LA_DTYPE_F32 = 0, LA_DTYPE_BF16 = 1 };
enum { LA_VERIFY_GREEDY = 0, LA_VERIFY_SAMPLE = 1 };

/* ------------------------------------------------------------------ model */
/* Llama-style decoder: RMSNorm, RoPE (rotate-half, theta), grouped-query
 * attention, SwiGLU MLP, untied LM head, no biases. */
typedef struct la_model_dims {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ff, vocab;
  int32_t dtype;            /* LA_DTYPE_*: storage of weights, activations and K/V */
  float eps;                /* RMSNorm epsilon */
  float rope_theta;
} la_model_dims;

/* Device weight pointers (read-only, dtype of dims.dtype, nn.Linear layout
 * [out_features][in_features], layers stacked on the leading axis):
 *   embed      [V][d]                 lm_head [V][d]          final_norm [d]
 *   attn_norm  [L][d]                 mlp_norm [L][d]
 *   wqkv       [L][(H + 2 Hkv) dh][d] rows: q heads, then k heads, then v heads
 *   wo         [L][d][H dh]
 *   w_gate_up  [L][2 F][d]            rows: gate (F rows), then up (F rows)
 *   w_down     [L][d][F]
 *   packed     la_packed_weight_bytes(dims) bytes written by la_pack_weights
 *              from the five projections above.
 * la_init reads embed, the norms and packed; the plain projection pointers
 * are read only by la_pack_weights (they may be null for la_init). */
typedef struct la_model {
  const void* embed;
  const void* lm_head;
  const void* final_norm;
  const void* attn_norm;
  const void* wqkv;
  const void* wo;
  const void* mlp_norm;
  const void* w_gate_up;
  const void* w_down;
  const void* packed;
} la_model;

/* Packed projections.  A round streams every projection matrix once over the
 * packed rows ("M7.3", 0x05C), so the library keeps them in the order its
 * GEMM reads them: the 16-row MFMA operand slices one workgroup consumes per
 * step lie in one contiguous run.  When the QKV projection's K is not split,
 * its columns are packed pair-major inside each head (a 16-column tile holds
 * 8 dimensions and their rotary partners), so its GEMM rotates q and k and
 * places q, k and v itself.  la_packed_weight_bytes: size of that
 * buffer for dims (0 for bad dims).  la_pack_weights: fill it (device,
 * 256-byte aligned, caller-owned) from plain's wqkv, wo, w_gate_up, w_down
 * and lm_head, on stream; LA_EINVAL for bad dims or null pointers. */
uint64_t la_packed_weight_bytes(const la_model_dims* dims);
int la_pack_weights(const la_model_dims* dims, const la_model* plain, void* packed, void* stream);

/* ----------------------------------------------------------------- config */
typedef struct la_config {
  int32_t W;                /* window width (lookahead columns), >= 1 */
  int32_t N;                /* n-gram size; the pinned schedule admits integer N >= 3 */
  int32_t G;                /* max candidates verified per round, >= 0 */
  int32_t max_new;          /* tokens to generate (the first comes from prefill) */
  int32_t verify_mode;      /* LA_VERIFY_GREEDY | LA_VERIFY_SAMPLE */
  int32_t ar_only;          /* 1: plain autoregressive decoding (1 row per round) with the same kernels */
  double temperature;       /* sampling: p = softmax(logits / temperature) */
  uint64_t seed;            /* sampling: Philox4x32-10 key */
  int32_t max_prompt;       /* capacity planning: longest prompt passed to la_init */
  int32_t pool_from_prompt; /* 1: la_init inserts the prompt's observed N-grams into the pool
                               ("M7.3", 0x03A POOL_FROM_PROMPT): for i = 0, 1, ... while
                               i + N - 1 < prompt_len, key prompt[i] and suffix
                               prompt[i+1 .. i+N-1], by the per-key LRU rule (0x03B); 0: off */
  int32_t advance_by_accepted; /* 1: ALWAYS_FWD_ONE=False window schedule (0x03C alternative):
                               after the pinned one-column advance every level drops its first
                               h entries and its tail is refilled with the newest committed
                               token; 0: ALWAYS_FWD_ONE=True (pinned) */
  int32_t cap_full_match;   /* 1: the capped full-match convention ("M7.3", 0x05A names the
                               implementation's max_hit count beside the paper's full match plus
                               one extra target token): at most S - 1 candidate tokens are
                               accepted per round, so a round emits at most S tokens and copies
                               at most S - 1 K/V rows; 0: a full match of S tokens also emits the
                               target token read from its last row (S + 1 tokens).  The output
                               is exact either way; only accepted lengths differ */
  int32_t pool_from_output; /* 1: generated-prefix insertion ("M7.3", 0x06A names it, optional, in
                               the pool plan): the n-gram each generated token completes in the
                               text prompt + output (key the token N - 1 before it, suffix the
                               N - 1 tokens up to it) enters the pool by the per-key LRU rule, in
                               text order, after the round's trajectory n-grams -- the first
                               token's at la_init; a paused batch round inserts none.  With
                               pool_from_prompt the pool so sees every n-gram of the text;
                               0: off */
} la_config;

/* Buffer sizes for a (config, dims) pair.  The caller allocates
 *   kv    : kv_bytes    device bytes (K then V, each [L][Hkv][t_cap][dh])
 *   arena : arena_bytes device bytes (activations, workspace K/V, logits,
 *           row manifest, n-gram pool, window, verification scratch)
 * 256-byte aligned (torch allocations are). */
typedef struct la_sizes {
  uint64_t kv_bytes;
  uint64_t arena_bytes;
  int32_t t_cap;            /* K/V rows per layer and head */
  int32_t q_max;            /* most packed rows in one round */
  int32_t n_logit_max;      /* most logit rows in one round */
  int32_t reserved;
} la_sizes;

/* One verification result (M7.3, 0x06A publication plan, output part). */
typedef struct la_accept {
  int32_t round_id;         /* round the result belongs to */
  int32_t h;                /* accepted candidate tokens, 0..S */
  int32_t winner;           /* candidate whose first h rows are committed, -1 if h == 0 */
  int32_t n_emit;           /* h + 1 */
  int32_t emitted[LA_MAX_EMIT];
} la_accept;

/* Description of the round that la_predict compiled and ran. */
typedef struct la_round_info {
  int32_t round_id;
  int32_t p;                /* logical position of the ordinary row (= committed K/V rows) */
  int32_t Q;                /* packed rows */
  int32_t C;                /* candidates retrieved for the current token */
  int32_t n_inp;            /* rows of the deepest trajectory level */
  int32_t n_logit;          /* 1 + n_inp + C * S logit rows */
  int32_t warm;             /* window fully materialised (pool updates active) */
  int32_t reserved;
  const float* logits;      /* device [n_logit][vocab] fp32: out, inp (column order), guess ((c, s) order) */
} la_round_info;

typedef struct la_stats_t {
  int64_t rounds;
  int64_t tokens;           /* emitted, including the prefill token */
  int64_t candidates;       /* sum of C over rounds */
  int64_t accepted;         /* sum of h over rounds */
  int32_t hist[LA_MAX_EMIT];/* rounds by emitted count (index = n_emit) */
  int64_t paused;           /* rounds a batch ran without the lookahead branch (la_batch_step) */
} la_stats_t;

typedef struct la_state_t {
  int32_t round_id;
  int32_t kv_len;           /* committed K/V rows (= prompt + committed inputs) */
  int32_t n_out;            /* output tokens so far */
  int32_t R;                /* trajectory levels (N - 1) */
  int32_t level_sizes[LA_MAX_N];
  int32_t warm;
  int32_t win_stride;
} la_state_t;

typedef struct la_ctx la_ctx;

/* ------------------------------------------------------------- lifecycle */

/* Sizes of the caller-provided buffers for a (config, dims) pair ("M7.3",
 * 0x01A: the round's coordinate system and admission are fixed before any
 * state; 0x05C: rows per round, (W + G)(N - 1) when warm).  cfg, dims: host,
 * read only; out: host, written on success.  LA_EINVAL, with nothing
 * written, for an inadmissible config: N < 3 or N > LA_MAX_N, W < 1 or
 * W > 64, G < 0 or G > 64, bad dims, or a largest round the kernels do not
 * take (more than 256 packed rows, a branch reaching more than 64 positions
 * past the committed prefix, d_model beyond 2048 16-byte vectors a row). */
int la_query_sizes(const la_config* cfg, const la_model_dims* dims, la_sizes* out);

/* Create a request ("M7.3", 0x03A lifecycle step 1: window and pool set-up;
 * 0x06 loop set-up): validate and admit as la_query_sizes, clear the pool
 * (or seed it with the prompt's N-grams under pool_from_prompt), seed the
 * window from the prompt (level 0 holds the last W + N - 3 prompt tokens,
 * cyclically), prefill the prompt (one plain causal forward; its K/V land in
 * kv rows 0..P-1) and select the first output token from its last row.
 * weights: device pointers (la_model); kv/arena: device buffers of at least
 * la_query_sizes bytes, 256-byte aligned, borrowed until la_destroy; prompt:
 * host [prompt_len], 1 <= prompt_len <= cfg->max_prompt, tokens in
 * [0, vocab); *out receives the context (NULL on error).  LA_EINVAL for bad
 * arguments, LA_EDEVICE for a HIP failure (no context is created). */
int la_init(const la_config* cfg, const la_model_dims* dims, const la_model* weights, void* kv, void* arena,
            const int32_t* prompt, int32_t prompt_len, void* stream, la_ctx** out);
/* Release a context (its host state and events); the borrowed device
 * buffers stay the caller's.  NULL is ignored. */
void la_destroy(la_ctx* ctx);

/* One full round ("M7.3", 0x06 loop: predict, verify, publish): la_predict,
 * la_verify on the round's own logits, la_commit.  Writes the round's
 * emitted tokens (after truncation at max_new) to out_tokens (host, cap
 * entries); n_out receives their number (0 once max_new tokens exist).
 * LA_EOVERFLOW if cap < N; any error of the three steps is returned with
 * the round unpublished. */
int la_step(la_ctx* ctx, int32_t* out_tokens, int32_t cap, int32_t* n_out);

/* Run rounds ("M7.3", 0x06) until max_new tokens exist; out_tokens (host,
 * cap >= max_new entries, else LA_EOVERFLOW) receives the whole output,
 * first token included; n_out its length. */
int la_generate(la_ctx* ctx, int32_t* out_tokens, int32_t cap, int32_t* n_out);

/* ------------------------------------------------------- round, in steps */

/* Predict ("M7.3", 0x03A lifecycle steps 2-4; 0x04A row records and
 * visibility; 0x04C one causal forward over the uncached rows): look up
 * <= G suffixes for the current token (after warmup), compile the packed
 * rows, run the target forward and the LM head on the out / inp / guess
 * rows.  info (host, may be NULL) receives the round's description; its
 * logits pointer stays valid until the next la_predict.  Mutates nothing
 * that la_commit publishes.  LA_ESTATE if a predicted round is pending
 * commit or max_new tokens exist; LA_EOVERFLOW if the K/V capacity is
 * exhausted. */
int la_predict(la_ctx* ctx, la_round_info* info);

/* Verify ("M7.3", 0x05A greedy survivor matching, 0x05B exact one-hot
 * sampling; 0x06A the publication plan's output part), pure: no request
 * state changes.  logits: device
 * [1 + n_inp + C*S][vocab] fp32 laid out like la_round_info.logits, or NULL
 * for the pending round's own logits.  cand: host [C][S] suffixes in pool
 * order (NULL with logits == NULL: the pending round's candidates).
 * z (host, may be NULL) receives the argmax of the n_inp deepest-level rows.
 * Greedy or one-hot sampling per cfg->verify_mode; sampling draws use the
 * counter (round_id, offset, draw). */
int la_verify(la_ctx* ctx, const float* logits, int32_t n_inp, const int32_t* cand, int32_t C, la_accept* out,
              int32_t* z);

/* Publish one accepted path of the pending round ("M7.3", 0x06B output and
 * K/V frontiers, 0x06C compaction, 0x03B / 0x03C pool then window, 0x07
 * fail-closed publication).  The plan is
 * validated first (round_id of the pending round, 0 <= h <= hmax (S, or
 * S - 1 under cap_full_match), winner in
 * [0, C) iff h > 0, n_emit = h + 1, emitted[0..h-1] equal the winner's
 * suffix, tokens in range, K/V capacity); only then are the winner's h K/V
 * rows copied behind the ordinary row, the W new n-grams upserted into the
 * pool (pre-shift window + this round's z, column order), the window
 * advanced and the tokens appended.  LA_ESTATE / LA_EPLAN / LA_EOVERFLOW
 * leave every piece of state unchanged. */
int la_commit(la_ctx* ctx, const la_accept* acc);

/* ------------------------------------------------------------- batching */

/* Several requests decoded together ("Speculative Decoding" lesson, Chapter 7
 * "Speculation Meets the Batch": concurrent requests share one read of the
 * weights per step, and speculation may spend only the compute the batch's
 * own rows leave free, throttled per request; "M7.3", 0x03B: each request
 * keeps its own pool, window and K/V).  A batch owns the stacked activations
 * of up to max_rows (<= 256) rows; the requests are ordinary contexts
 * (la_init) created with the batch's dims and weights, on its stream.
 *
 * la_batch_bytes: device workspace bytes for max_rows rows (0 for bad dims
 * or max_rows outside [1, 256]).
 * la_batch_init: workspace (device, >= la_batch_bytes, 256-byte aligned) is
 * borrowed until la_batch_destroy; weights as for la_init.  The batch also
 * allocates a small pinned host buffer (the per-request argument tables of a
 * step, under 100 KB at max_rows = 256) and an event, freed by
 * la_batch_destroy.  LA_EINVAL for bad dims / max_rows / weights,
 * LA_EOVERFLOW for a short workspace, LA_EDEVICE if the pinned buffer or the
 * event cannot be created. */
typedef struct la_batch la_batch;
uint64_t la_batch_bytes(const la_model_dims* dims, int32_t max_rows);
int la_batch_init(const la_model_dims* dims, const la_model* weights, int32_t max_rows, void* workspace,
                  uint64_t bytes, void* stream, la_batch** out);
void la_batch_destroy(la_batch* batch);

/* The occupancy throttle (Chapter 7 above: the step's row budget is shared;
 * what the requests' own rows leave is spent on speculation, request by
 * request, down to none).  Host only, pure.  For n requests, base_rows[i] is
 * the rows of request i's round without candidates (its ordinary row plus
 * its lookahead branch; 0: the request is not in this step) and found[i] the
 * candidates its pool lookup returned.  Every request with base_rows > 0
 * keeps its base rows; if their sum exceeds row_budget, requests from the
 * last one backwards drop their lookahead branch (paused[i] = 1: one row)
 * until the sum fits.  The remaining budget is dealt in S-row candidate
 * blocks, one per request in turn in request order (request order is the
 * priority order), to requests that are not paused, up to found[i]:
 * cap[i] receives the candidates request i verifies.  Output arrays: host
 * [n].  LA_EOVERFLOW when more requests are active than row_budget rows;
 * LA_EINVAL for sizes out of range (n <= 256, 1 <= S < LA_MAX_N) or
 * negative inputs. */
int la_batch_plan(int32_t n, int32_t row_budget, int32_t S, const int32_t* base_rows, const int32_t* found,
                  int32_t* cap, int32_t* paused);

/* What one request's round did inside la_batch_step. */
typedef struct la_batch_round {
  int32_t Q;                /* packed rows (0: the request was finished) */
  int32_t found;            /* candidates its pool lookup returned */
  int32_t verified;         /* candidates verified (the throttle's cap) */
  int32_t paused;           /* 1: the round ran without the lookahead branch */
  int32_t h;                /* candidate tokens accepted */
  int32_t reserved[3];
} la_batch_round;

/* One round for each of n requests ("M7.3", 0x06 loop: predict, verify,
 * publish, per request) in one stacked forward.  ctx: host [n] distinct
 * contexts with no round pending, all of the batch's dims, weights and
 * stream and of one N (W, G and the other options may differ); requests
 * that already hold max_new tokens are skipped.
 * row_budget: the step's row budget (<= max_rows; <= 0: max_rows); the
 * requests' rows are planned with la_batch_plan's rule.  A paused round
 * verifies no candidates and leaves the window and the pool as they are;
 * outputs stay exact either way (only the accepted lengths change).  The
 * per-request arithmetic is that of the request's own la_step (the rows of a
 * request give bitwise the same logits whatever rows share the step), so
 * with a budget that throttles nothing every request's rounds are those of
 * la_step.  out_tokens: host [n][LA_MAX_EMIT], request i's emitted tokens
 * (after truncation at max_new) at row i; n_out: host [n] their counts;
 * rinfo: host [n] or NULL.  Errors before the forward (LA_EINVAL for
 * mismatched or repeated contexts, different N or a budget above max_rows, LA_ESTATE,
 * LA_EOVERFLOW from any request or the plan) leave every request as it
 * was; a failure while publishing leaves the requests before it published
 * (their n_out set) and the rest unchanged. */
int la_batch_step(la_batch* batch, la_ctx* const* ctx, int32_t n, int32_t row_budget, int32_t* out_tokens,
                  int32_t* n_out, la_batch_round* rinfo);

/* -------------------------------------------------------- pool and state */

/* Suffixes stored for key ("M7.3", 0x03 lookup of the live token's list,
 * 0x03B order), least recently used first (at most G).  out: host [G][S];
 * n (host) receives the count.  LA_EINVAL for a key outside [0, vocab). */
int la_pool_lookup(la_ctx* ctx, int32_t key, int32_t* out, int32_t* n);

/* Upsert n (key, suffix) pairs in order with the per-key LRU rule ("M7.3",
 * 0x03B).  keys: host [n], suffixes: host [n][S], tokens in [0, vocab);
 * 0 <= n <= 64 per call.  LA_EINVAL for bad tokens or sizes, LA_ESTATE
 * while a predicted round is pending (the pool may only change between
 * rounds, 0x03C). */
int la_pool_insert(la_ctx* ctx, const int32_t* keys, const int32_t* suffixes, int32_t n);

/* Host snapshot of the request state ("M7.3", 0x01A manifest: round id,
 * window, K/V length, output): st (host) receives the counters and level
 * sizes; window (host, may be NULL) receives [R][win_stride] tokens, output
 * (host, may be NULL) up to out_cap tokens. */
int la_get_state(la_ctx* ctx, la_state_t* st, int32_t* window, int32_t* output, int32_t out_cap);

/* Acceptance counters ("M7.3", 0x05: the step-compression statistics a
 * round produces): rounds, tokens, candidates, accepted and the histogram of
 * emitted counts.  out: host.  LA_EINVAL for NULL arguments. */
int la_stats(const la_ctx* ctx, la_stats_t* out);

/* Opt-in kernel timing (measurement of "M7.3", 0x05C's cost terms: weight
 * stream and attention per round): while enabled, every GEMM launch (projections, MLP,
 * LM head, with their split reductions) and every attention launch (with
 * its span merge) of the context's rounds is bracketed by HIP events on the
 * context's stream; elapsed times are accumulated at each verification sync,
 * together with the algorithmic bytes and flops of each launch (weights +
 * rows in + rows out for a GEMM; committed K/V read + branch K/V + Q + O
 * for attention).  la_profile(ctx, 1) clears the totals. */
typedef struct la_profile_t {
  double gemm_ms, gemm_bytes, gemm_flops;
  double attn_ms, attn_bytes, attn_flops;
  int64_t gemm_launches, attn_launches;
} la_profile_t;
int la_profile(la_ctx* ctx, int32_t enable);     /* LA_ESTATE while a round is pending */
int la_profile_read(const la_ctx* ctx, la_profile_t* out);
/* Message of the last error on ctx (or of this thread's last context-free
 * call when ctx is NULL); owned by the library, valid until the next call. */
const char* la_last_error(const la_ctx* ctx);

/* ------------------------------------------------ context-free operators */

/* Packed-row builder (M7.3, 0x04A row records and visibility).  desc
 * describes the round: levels[r] cells at columns starts[r].. (level 0 at
 * column 1, the ordinary row is column 0), C candidates of S tokens.
 * Rows are emitted in branch-major order: column j gives
 * [b_j, u_(1,j), ..., u_(d_j,j)], then candidate c gives [v_(c,0..S-1)].
 * out (device int32) receives, at the offsets reported in info:
 *   tok[Q] pos[Q] role[Q] (0 ordinary, 1 lookahead, 2 verify) level[Q]
 *   col[Q] cand[Q] off[Q] branch[Q] path[NB][maxp] path_len[NB]
 *   logit_rows[n_logit] mask[Q][mask_words] (bit k of row i: i sees k)
 *   tile_meta[T][64] tile_path[T][16][64]   (T = ceil(Q / 16) row tiles).
 * path[b][k] is the packed row (minus one) holding logical position
 * p + 1 + k on branch b.  For the row tile t (packed rows 16t .. 16t+15),
 * tile_meta[t][0] is the number n of distinct branches among its rows and
 * tile_meta[t][1 + i] (i < n) the i-th of them in row order (-1 after);
 * tile_path[t][i][k] is path[tile_meta[t][1 + i]][k] where k is below that
 * branch's path length and the value names a packed row other than the
 * ordinary one, else -1.  The attention kernel reads these per-tile tables
 * for the keys past the committed prefix.  window: device [R][win_stride] tokens; cand:
 * device [C][S].  la_rows_query fills info (host) without launching
 * anything; la_build_rows launches one kernel on stream and returns (out is
 * complete once the stream reaches it).  Errors: LA_EINVAL for a bad
 * descriptor (R or S outside 1..16, C outside 0..64, a level longer than
 * win_stride, levels not nested column by column, more than 1024 rows) or a
 * NULL pointer; LA_EOVERFLOW when the round's tables exceed the builder's
 * LDS. */
typedef struct la_rows_desc {
  int32_t p;                /* logical position of the ordinary row */
  int32_t R;                /* levels */
  int32_t sizes[LA_MAX_N];  /* cells per level, 0 = absent */
  int32_t starts[LA_MAX_N]; /* first column of levels r >= 1 (level 0 starts at 1) */
  int32_t C, S;
  int32_t x_t;              /* current token (ordinary row input) */
  int32_t win_stride;
} la_rows_desc;

typedef struct la_rows_info {
  int32_t Q, NB, maxp, n_logit, n_inp, n_cols, mask_words, total_words;
  int32_t off_tok, off_pos, off_role, off_level, off_col, off_cand, off_off, off_branch;
  int32_t off_path, off_path_len, off_logit_rows, off_mask, off_tile_meta, off_tile_path;
} la_rows_info;

int la_rows_query(const la_rows_desc* desc, la_rows_info* info);
int la_build_rows(const la_rows_desc* desc, const int32_t* window, const int32_t* cand, int32_t* out, void* stream,
                  la_rows_info* info);

/* Lookahead-mask attention for one layer (M7.3, 0x04A visibility; 0x07
 * three-region K/V).  q: device [Q][H][dh]; k_cache/v_cache: device
 * [Hkv][t_cap][dh] holding logical positions 0..shared_end-1; k_ws/v_ws:
 * device [Hkv][ws_cap][dh], packed row k at row k-1; rows: the device
 * buffer filled by la_build_rows with its info; out: device [Q][H][dh].
 * Row i attends positions 0..pos_i: those below shared_end from the cache,
 * the others through its branch path.  workspace: device scratch of
 * la_attention_workspace(Q, H, dh, max_pos, t_cap) bytes, max_pos =
 * shared_end - 1 + info->maxp (the largest position a row reaches): one
 * softmax state per row, head and key split.  A key split is a fixed run of
 * chunks of 32 positions whose length depends on t_cap and the head counts
 * only: max(4, ceil(chunks(t_cap) / min(8, 320 / H))) chunks.  Batch
 * invariant: a row's result does not depend on the other rows of the call
 * (its reduction tree is a function of key positions, t_cap and the head
 * counts only).  The call only launches (on stream).
 * Errors: LA_EINVAL for a NULL pointer, an unknown dtype, H not a multiple
 * of Hkv, shared_end outside [1, t_cap], ws_cap < Q - 1, or a shape the
 * kernel does not take (dh other than 64/128 in bf16 or 16/64 in fp32, a
 * row reaching more than 64 positions past shared_end); LA_EOVERFLOW for a
 * workspace smaller than la_attention_workspace; LA_EDEVICE for a failed
 * launch. */
size_t la_attention_workspace(int32_t Q, int32_t H, int32_t dh, int32_t max_pos, int32_t t_cap);
int la_attention(int32_t dtype, const void* q, const void* k_cache, const void* v_cache, int32_t t_cap,
                 const void* k_ws, const void* v_ws, int32_t ws_cap, int32_t H, int32_t Hkv, int32_t dh,
                 const int32_t* rows, const la_rows_info* info, int32_t shared_end, void* out, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Allocation-free la_attention, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results as la_attention (same
 * arguments minus the workspace), with the key splits' softmax states kept
 * in a library-owned device array of LA_NOALLOC_SCRATCH_BYTES per device
 * (allocated by the HIP runtime when the library's code is loaded, held
 * until the process ends).  The call allocates nothing; its first call on
 * a device looks up that device's array address.  Every call on one device
 * shares the array, so calls that overlap on one device (concurrent
 * streams, or host threads) race: order them on one stream.  LA_EOVERFLOW,
 * before anything is launched, when la_attention_workspace for the shape
 * exceeds LA_NOALLOC_SCRATCH_BYTES; otherwise the errors of la_attention. */
#define LA_NOALLOC_SCRATCH_BYTES (32u << 20)
int la_attention_noalloc(int32_t dtype, const void* q, const void* k_cache, const void* v_cache, int32_t t_cap,
                         const void* k_ws, const void* v_ws, int32_t ws_cap, int32_t H, int32_t Hkv, int32_t dh,
                         const int32_t* rows, const la_rows_info* info, int32_t shared_end, void* out, void* stream);

/* Token-wise linear layer of the target forward ("M7.3", 0x05C: the
 * projections and MLP run over every packed row), Y = epilogue(X W^T):
 *   LA_LINEAR_STORE    Y[M][N] = round(X W^T)
 *   LA_LINEAR_RESIDUAL Y[M][N] = round(R + X W^T)            (R may alias Y)
 *   LA_LINEAR_SWIGLU   W is [2N][K] (gate rows, then up rows);
 *                      Y[M][N] = round(silu(X Wg^T) * (X Wu^T))
 *   LA_LINEAR_F32      Y[M][N] = X W^T in fp32 (Y is float)
 * X: device [M][K], W: device [N or 2N][K] (nn.Linear layout), dtype of
 * X/W/R/Y (except F32's Y) is dtype; fp32 accumulation.  1 <= M <= 256,
 * K a multiple of 128 (bf16) or 64 (fp32), N a multiple of 16.  The K split
 * (and so every output bit) depends on (N, K) only, never on M: a row's
 * result is the same whatever other rows share the call.
 * workspace: device scratch of la_linear_workspace(...) bytes; la_linear
 * first writes the packed copy of W there (la_pack_linear), then runs
 * la_linear_packed.
 * la_pack_linear: W -> Wp (la_packed_linear_bytes bytes, device, 256-byte
 * aligned), the layout la_pack_weights uses; la_linear_packed: the same
 * product from a packed Wp, workspace as for la_linear (its first
 * la_packed_linear_bytes, rounded up to 256, are not used).  The calls only
 * launch (on stream).  Errors: LA_EINVAL for a NULL pointer, an unknown
 * dtype or epilogue, or a shape outside the bounds above; LA_EOVERFLOW for
 * a short workspace; LA_EDEVICE for a failed launch. */
enum { LA_LINEAR_STORE = 0, LA_LINEAR_RESIDUAL = 1, LA_LINEAR_SWIGLU = 2, LA_LINEAR_F32 = 3 };
size_t la_linear_workspace(int32_t dtype, int32_t epilogue, int32_t M, int32_t N, int32_t K);
int la_linear(int32_t dtype, int32_t epilogue, const void* X, const void* W, void* Y, const void* R, int32_t M,
              int32_t N, int32_t K, void* workspace, size_t workspace_bytes, void* stream);
size_t la_packed_linear_bytes(int32_t dtype, int32_t epilogue, int32_t N, int32_t K);
int la_pack_linear(int32_t dtype, int32_t epilogue, const void* W, int32_t N, int32_t K, void* Wp, void* stream);
int la_linear_packed(int32_t dtype, int32_t epilogue, const void* X, const void* Wp, void* Y, const void* R,
                     int32_t M, int32_t N, int32_t K, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LA_H */
