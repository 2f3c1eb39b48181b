/*
 * spec.h -- C ABI of libspec, an MI355X (gfx950) library for the hot path of
 * speculative decoding: one target forward pass over K+1 positions with the
 * weights streamed from HBM once, followed by the accept/reject rule, fed by
 * a draft-model loop.  All device work is hand-written HIP.
 *
 * Pages the operations come from (cited by title and section):
 *   [zh]  "在神諭塔當見習抄寫刺蝟…：推測解碼入門" (gu-log Lv-19, zh-tw)
 *   [en]  "Apprentice Scribe Hedgehog at the Oracle Tower … Speculative
 *          Decoding 101" (gu-log Lv-19, English)
 *   [int] "Speculative decoding internals" (tarrragon LLM notes, module 3)
 *
 * General conventions
 *   Return codes: every call returns SPEC_OK (0) or a negative SPEC_ERR_*.
 *   Argument errors are detected synchronously, before anything is enqueued.
 *   Device work is enqueued on the context's stream and the call returns
 *   without waiting; outputs are valid once that stream has drained
 *   (spec_sync, or any later call that synchronises).  A failed HIP call is
 *   reported as SPEC_ERR_HIP with its text in spec_last_error().
 *   No C++ exception crosses this interface.
 *
 *   Pointers: every *_dev argument is device memory owned by the caller; it
 *   must stay valid until the work that uses it has run.  The context owns
 *   the packed weights, KV caches, workspaces and graphs it creates.
 *   Host pointers are read before the call returns.
 *
 *   Layouts are row-major.  Token ids are int32 in [0, vocab).  Probability
 *   rows are fp32.  Weights are bf16, [out_features][in_features], stacked
 *   over layers.
 *
 *   Threading: one context per stream; a context is not thread-safe.
 *   Determinism: results depend only on weights, prompt, K and seed; device
 *   reductions use fixed orders (no floating-point atomics).
 */
#ifndef SPEC_H
#define SPEC_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_OK 0
#define SPEC_ERR_ARG (-1)        /* null pointer, bad size, unsupported shape */
#define SPEC_ERR_CAPACITY (-2)   /* a pass would write beyond max_seq */
#define SPEC_ERR_STATE (-3)      /* call out of order (e.g. commit with no verify) */
#define SPEC_ERR_OOM (-4)        /* device allocation failed */
#define SPEC_ERR_HIP (-5)        /* HIP runtime error; text in spec_last_error */

/* Largest K (drafted tokens per round) the model path supports: K+1 rows of
 * activations are carried as bf16 high and low halves in one 16-row MFMA
 * tile. */
#define SPEC_K_MAX 7
/* Largest K of the stateless accept/reject entry point. */
#define SPEC_AR_K_MAX 63

/* A Llama-style decoder: pre-norm RMSNorm blocks with rotate-half RoPE,
 * grouped-query causal attention and a SwiGLU feed-forward, final RMSNorm and
 * an LM head; the next-token distribution at every position is the softmax
 * of the logits at temperature 1 ([en] Floor 3: one pass scores every
 * position).  The pages fix no architecture; this is the one the workloads
 * name.
 * Shape rules: d_model % 64 == 0, d_ffn % 32 == 0, vocab % 16 == 0,
 * head_dim even, n_heads % n_kv_heads == 0, (n_heads*head_dim/2) % 8 == 0,
 * (n_kv_heads*head_dim/2) % 8 == 0, head_dim <= 256,
 * n_heads/n_kv_heads*(SPEC_K_MAX+1) <= 64. */
typedef struct spec_model_desc {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rope_theta, rms_eps;
  /* Device pointers to bf16 weights.  They are only read during spec_init
   * (copied and repacked into context-owned memory); the caller may free
   * them afterwards.  A draft whose embed or lm_head pointer equals the
   * target's shares the target's packed copy. */
  const void* embed;      /* [vocab][d_model] */
  const void* attn_norm;  /* [n_layers][d_model] */
  const void* wq;         /* [n_layers][n_heads*head_dim][d_model] */
  const void* wk;         /* [n_layers][n_kv_heads*head_dim][d_model] */
  const void* wv;         /* [n_layers][n_kv_heads*head_dim][d_model] */
  const void* wo;         /* [n_layers][d_model][n_heads*head_dim] */
  const void* ffn_norm;   /* [n_layers][d_model] */
  const void* wg;         /* [n_layers][d_ffn][d_model] */
  const void* wu;         /* [n_layers][d_ffn][d_model] */
  const void* wd;         /* [n_layers][d_model][d_ffn] */
  const void* final_norm; /* [d_model] */
  const void* lm_head;    /* [vocab][d_model] */
} spec_model_desc;

typedef struct spec_init_params {
  spec_model_desc target;
  spec_model_desc draft;     /* must have target.vocab ([en] Floor 6: shared vocabulary) */
  int32_t k_max;             /* 1..SPEC_K_MAX: largest K later calls may use */
  int32_t max_seq;           /* token capacity of each KV cache (>= n_prompt + k_max + 1) */
  int32_t greedy;            /* 1: greedy checking ([en] Floor 4); 0: sampling at T = 1 (Floor 5) */
  int32_t use_graphs;        /* 1: replay draft/verify from captured hipGraphs; 0: plain launches */
  int32_t profile_kernels;   /* 1: start with profiling on (see spec_set_profiling) */
  uint64_t stream_id;        /* Philox counter word c (0 in normal use) */
  void* hip_stream;          /* hipStream_t to enqueue on; NULL: the context creates one */
} spec_init_params;

typedef struct spec_ctx spec_ctx;

/* Creates a context: validates shapes, copies and packs the weights,
 * allocates the paged KV caches (block size 16) and workspaces, and runs the
 * prompt through both models.  prompt_host[0..n_prompt-2] is written into
 * the caches; prompt_host[n_prompt-1] becomes the pending token (emitted but
 * not yet in the target cache).  Synchronises before returning.
 * Errors: SPEC_ERR_ARG (shapes, n_prompt < 1, token ids), SPEC_ERR_CAPACITY,
 * SPEC_ERR_OOM, SPEC_ERR_HIP.  On error *out is NULL. */
int spec_init(const spec_init_params* p, const int32_t* prompt_host, int32_t n_prompt,
              spec_ctx** out);

/* Draft loop ([int] algorithm core, Step 1; [en] Floor 4 item 1): K
 * autoregressive draft-model steps.  Step s feeds the tokens the draft cache
 * lacks (the pending token, plus the last accepted draft after a round that
 * accepted all K) or d_s, and ends with the draft's softmax row D_{s+1}
 * written to D_dev[s] and its token d_{s+1} written to d_dev[s]: inverse CDF
 * on the 2^-40 grid with Philox word w0 at that token's position (seed,
 * stream_id), or the top token in greedy mode.
 *   d_dev: int32 [K];  D_dev: fp32 [K][vocab].
 * Errors: SPEC_ERR_ARG (K outside 1..k_max, null pointers), SPEC_ERR_CAPACITY,
 * SPEC_ERR_STATE (a verify is pending: drafting now would re-draft positions
 * whose decision awaits its commit and corrupt the draft cache). */
int spec_draft(spec_ctx* ctx, int32_t K, uint64_t seed, int32_t* d_dev, float* D_dev);

/* Prompt-lookup drafter ([en] Floor 6, [zh] Level 6: n-gram approaches such
 * as prompt lookup draft by searching the preceding text for a chunk likely
 * to repeat; verification is unchanged), run on the device with no draft
 * model.  The committed history hist[0..L] (hist[L] the pending token) is
 * searched for the latest earlier occurrence of its last n tokens, the
 * longest n <= n_max first; the K drafts are the tokens that followed it,
 * repeated with its period p = L - j when fewer than K follow, or the pending
 * token K times when nothing repeats.  D_dev receives one-hot rows (a
 * deterministic drafter), so spec_verify's rule accepts d_i with probability
 * T_i(d_i) and otherwise samples T_i without d_i.  The draft model's cache is
 * left as it is (a later spec_draft catches it up).
 *   d_dev: int32 [K]; D_dev: fp32 [K][vocab] (may be NULL in greedy mode).
 * Errors: SPEC_ERR_ARG (K outside 1..k_max, n_max outside 1..8, null
 * pointers), SPEC_ERR_STATE (a verify is pending). */
int spec_draft_ngram(spec_ctx* ctx, int32_t K, int32_t n_max, int32_t* d_dev, float* D_dev);

/* Multi-token-prediction heads as the drafter ("Speculative decoding
 * internals", variants: MTP -- the target carries extra output heads, head k
 * predicting the token k places ahead, and needs no separate drafter model).
 * The pages fix no head architecture; here head k maps the target's final
 * normed state h of the last position it processed to z_k = h + silu(W_k h)
 * and the target's own LM head scores z_k.  spec_heads_init packs the head
 * matrices into context-owned memory (the caller may free W_dev afterwards);
 * a second call replaces them.
 *   W_dev: bf16 [n_heads][d_model][d_model] (row-major, output-major) device
 *   memory of the target's width; n_heads in 1..7.
 * Synchronises the context stream.  Errors: SPEC_ERR_ARG (null pointers,
 * n_heads out of range), SPEC_ERR_STATE (a verify is pending), SPEC_ERR_OOM,
 * SPEC_ERR_HIP. */
int spec_heads_init(spec_ctx* ctx, const void* W_dev, int32_t n_heads);

/* K drafts from the heads: the state is the target's final residual at the
 * last committed position (kept by the prompt prefill and by every
 * spec_commit), so no draft model runs and the draft cache is left as it is.
 * The position after that state holds the pending token, so head k (k = 0..
 * K-1) drafts the token after it at position LT+1+k: D_dev[k] = softmax of
 * the LM head on z_k, d_dev[k] drawn from it by inverse CDF on the 2^-40 grid
 * with Philox word w0 at that position (seed, stream_id), or its top token in
 * greedy mode -- the same draw spec_draft makes.  Each D row depends on the
 * committed prefix only, not on the earlier drafts of the round; spec_verify
 * takes the pair unchanged.  Called after spec_draft in the same round, its
 * drafts replace the draft model's and the draft cache's committed length
 * stays where it was (the next spec_draft catches up over the committed
 * text).  Asynchronous on the context stream.
 *   d_dev: int32 [K]; D_dev: fp32 [K][vocab].
 * Errors: SPEC_ERR_ARG (K outside 1..min(n_heads, k_max), null pointers),
 * SPEC_ERR_STATE (no heads; a verify is pending; a one-token prompt and no
 * commit yet, so no position has been processed), SPEC_ERR_CAPACITY. */
int spec_draft_heads(spec_ctx* ctx, int32_t K, uint64_t seed, int32_t* d_dev, float* D_dev);

/* Verify pass plus accept/reject ([int] algorithm core, Steps 2-4; [en]
 * Floors 3-5).  One target pass over the K+1 rows [pending, d_1..d_K] at
 * positions L..L+K gives T_1..T_{K+1}; their keys/values are appended to the
 * target cache.  Then, sampling mode: draft i is accepted iff
 * r_i * D_i(d_i) < T_i(d_i) (r_i from Philox word w1 at the draft's
 * position); at the first reject the replacement is drawn from
 * max(0, fix(T_i) - fix(D_i)) by inverse CDF with word w2 (falling back to
 * T_i, then its argmax, if that residual is empty); if all K pass the bonus
 * token is drawn from T_{K+1} with w2.  Greedy mode: a draft passes iff it is
 * the lowest-index argmax of T_i; the first mismatch emits that argmax; the
 * bonus is the argmax of T_{K+1}.  Drafts may come from any source: D rows
 * are only read in sampling mode (one-hot rows describe a deterministic
 * drafter).  K = 0 is one step of plain decoding with the same kernels: a
 * one-row pass over the pending token and the next token drawn from T_1 (w2
 * at its position, or the argmax in greedy mode); d_dev and D_dev are not
 * read and may be NULL.
 *   d_dev: int32 [K]; D_dev: fp32 [K][vocab] (may be NULL in greedy mode);
 *   out_dev: int32 [K+1] receives the n_acc+1 emitted tokens, -1 after them;
 *   n_acc_dev: int32 [1] receives n_acc in 0..K, or -1 if an input that the
 *   rule read was invalid (a probability outside [0,1] or non-finite, or a
 *   draft id outside [0, vocab)) -- then out_dev is all -1;
 *   T_dev (nullable): fp32 [K+1][vocab] receives the target rows;
 *   logits_dev (nullable): fp32 [K+1][vocab] receives the target logits.
 * Errors: SPEC_ERR_ARG (K outside 0..k_max, null pointers), SPEC_ERR_CAPACITY
 * (L+K+1 > max_seq), SPEC_ERR_STATE (a verify is already awaiting its commit). */
int spec_verify(spec_ctx* ctx, int32_t K, uint64_t seed, const int32_t* d_dev, const float* D_dev,
                int32_t* out_dev, int32_t* n_acc_dev, float* T_dev, float* logits_dev);

/* Commit ([en] Floor 4: slips after a reject are torn up).  On the device:
 * the emitted tokens are appended to the committed history, the target
 * length advances by n_acc+1 (keys/values of the rejected rows stay in place
 * and are overwritten later), the last emitted token becomes the pending one,
 * and the draft length keeps only rows whose tokens were committed.  No host
 * synchronisation.  out_dev / n_acc_dev are the buffers given to the
 * preceding spec_verify (or equivalent values).  n_acc = -1 leaves the state
 * unchanged.  Errors: SPEC_ERR_ARG, SPEC_ERR_STATE (no verify pending). */
int spec_commit(spec_ctx* ctx, const int32_t* out_dev, const int32_t* n_acc_dev);

/* Releases everything the context owns.  NULL is accepted. */
int spec_destroy(spec_ctx* ctx);

/* Text of the last failure on ctx (or of the last failed spec_init /
 * stateless call on this thread when ctx is NULL).  Never NULL. */
const char* spec_last_error(const spec_ctx* ctx);

/* Waits for the context's stream. */
int spec_sync(spec_ctx* ctx);

/* The hipStream_t the context enqueues on. */
void* spec_stream(const spec_ctx* ctx);

typedef struct spec_state {
  int32_t target_len;   /* tokens in the target KV cache (pending token at this position) */
  int32_t draft_len;    /* tokens in the draft KV cache */
  int32_t pending;      /* pending token id */
  int32_t device_error; /* sticky device-side error bits (0 = none) */
  /* acceptance record: accept_counts[K][n] = committed verifies of K drafts
   * that accepted n of them (K = 0 counts plain decode steps).  The number of
   * accepted tokens per round and the per-position acceptance rates of the
   * pages' analysis ([int] "how many tokens per round") follow from it. */
  int32_t accept_counts[SPEC_K_MAX + 1][SPEC_K_MAX + 1];
} spec_state;

/* Synchronises and reads the device-side state. */
int spec_get_state(spec_ctx* ctx, spec_state* out);

/* Synchronises and copies committed tokens [0, n) (prompt included) to host. */
int spec_get_history(spec_ctx* ctx, int32_t* host_out, int32_t n);

/* With profiling on: durations in ms of the feed-forward gate/up GEMM
 * launches of the most recent spec_draft and spec_verify calls, in launch
 * order (draft launches first).  A duration is the launch's slice of the
 * back-to-back kernel stream: from the end of the O projection launched just
 * before it to its own end, each end being the latest of the per-workgroup
 * stamps the kernels write from the device wall clock.  It is therefore
 * measured inside the replayed graphs and includes the launch overhead.  -1
 * marks a launch whose stamps are missing.  Synchronises.  *n_out = count
 * written. */
int spec_kernel_times(spec_ctx* ctx, float* ms_out, int32_t cap, int32_t* n_out);

/* Profiling switch.  When on, spec_draft and spec_verify replay graphs
 * captured with the stamp slots of the gate/up GEMMs and the O projections
 * before them set (a separate graph cache from the plain one), after
 * resetting those slots on the stream; kernels and results are the same as
 * with profiling off.  Synchronises.
 * Also set at creation by spec_init_params.profile_kernels. */
int spec_set_profiling(spec_ctx* ctx, int32_t enable);

/* Measurement helper: the duration in ms of the LM head of the last
 * spec_verify run with profiling on, from the same per-workgroup end stamps
 * (the latest LM-head workgroup end minus the latest end of the last layer's
 * down projection, launch overhead included); -1 when that verify ran
 * without profiling.  Synchronises.  Errors: SPEC_ERR_ARG, SPEC_ERR_HIP. */
int spec_head_time(spec_ctx* ctx, float* ms_out);

/* A packed weight matrix multiplied by a batch of activation rows: the
 * verify pass's weight-streaming GEMM for M = B * (K+1) rows of B sequences
 * ([en] Floor 6, "crowded tower days": with a large batch every weight read
 * serves many rows, the work turns compute-bound and extra draft positions
 * stop being free).  The bytes streamed do not depend on M; the matrix-core
 * work grows with it.  Activations enter as bf16 high and low parts (as in
 * the verify pass), products accumulate in fp32.
 * spec_mat_create: packs W (device, bf16 [N][K], row-major; may be freed
 * after the call) into the stream layout; N % 16 == 0, K % 32 == 0.
 * Synchronises.  Errors: SPEC_ERR_ARG, SPEC_ERR_OOM, SPEC_ERR_HIP.
 * spec_mat_mul: Y = X W^T with X fp32 [M][K], Y fp32 [M][N] (device,
 * caller-owned), 1 <= M <= 128, enqueued on hip_stream (NULL: default).  The
 * matrix owns one activation workspace: calls on one matrix must not overlap
 * (keep them on one stream).  Errors: SPEC_ERR_ARG, SPEC_ERR_HIP.
 * spec_mat_destroy: synchronises the device and frees; NULL accepted. */
typedef struct spec_mat spec_mat;
int spec_mat_create(const void* W_dev, int32_t N, int32_t K, spec_mat** out);
int spec_mat_mul(spec_mat* m, const float* X_dev, int32_t M, float* Y_dev, void* hip_stream);
int spec_mat_destroy(spec_mat* m);

/* Batched verification: B sequences decoded together against one target
 * ([en] Floor 6, "crowded tower days"; [zh] Level 6: with many requests at
 * once every weight read serves B (K+1) rows, and the pass moves from memory
 * bound toward compute bound).  Each sequence keeps its own history,
 * positions and paged KV cache, and gets its own accept/reject decision;
 * sequence b draws its Philox words with sequence index s = b (counter
 * (p, b, stream_id, 0), the same words spec_verify uses for s = 0), so
 * sequence b's results are exactly those of a single-sequence verify of its
 * rows with that index.  Drafts come from the caller (any drafter) or from
 * spec_batch_draft_ngram.
 * Limits: 1 <= n_seq <= SPEC_BATCH_MAX_SEQ, 1 <= k_max <= SPEC_K_MAX,
 * n_seq * (k_max + 1) <= 128 activation rows; every prompt has n_prompt
 * tokens; the target follows spec_model_desc's shape rules with
 * d_model <= 8192. */
#define SPEC_BATCH_MAX_SEQ 32

typedef struct spec_batch_params {
  spec_model_desc target;
  int32_t n_seq;             /* B */
  int32_t k_max;             /* largest K later calls may use */
  int32_t max_seq;           /* token capacity of each sequence's cache (>= n_prompt + k_max + 1) */
  int32_t greedy;            /* 1: greedy checking; 0: sampling at T = 1 */
  int32_t use_graphs;        /* 1: replay the verify pass from captured hipGraphs */
  uint64_t stream_id;        /* Philox counter word c */
  void* hip_stream;          /* hipStream_t to enqueue on; NULL: the context creates one */
} spec_batch_params;

typedef struct spec_batch spec_batch;

/* Creates a batch context: packs the target weights (its own copy), allocates
 * B paged caches and the workspaces, and prefills prompts_host[b][0..n-2] of
 * every sequence; prompts_host[b][n-1] is sequence b's pending token.
 *   prompts_host: int32 [n_seq][n_prompt] (host).
 * Synchronises.  Errors: SPEC_ERR_ARG (shapes, limits, n_prompt < 1, token
 * ids), SPEC_ERR_CAPACITY, SPEC_ERR_OOM, SPEC_ERR_HIP.  On error *out is NULL. */
int spec_batch_init(const spec_batch_params* p, const int32_t* prompts_host, int32_t n_prompt,
                    spec_batch** out);

/* Prompt-lookup drafts for every sequence (the drafter of spec_draft_ngram,
 * applied to each sequence's own history).
 *   d_dev: int32 [n_seq][K]; D_dev: fp32 [n_seq][K][vocab] one-hot rows (may
 *   be NULL in greedy mode).
 * Errors: SPEC_ERR_ARG (K outside 1..k_max, n_max outside 1..8, null). */
int spec_batch_draft_ngram(spec_batch* bc, int32_t K, int32_t n_max, int32_t* d_dev, float* D_dev);

/* One target pass over the B (K+1) rows [pending_b, d_b1..d_bK] of every
 * sequence (weights streamed once for the whole batch), the row softmax, and
 * the rule per sequence, as spec_verify does for one sequence.
 *   d_dev: int32 [n_seq][K]; D_dev: fp32 [n_seq][K][vocab] (unused in greedy
 *   mode, may be NULL there); out_dev: int32 [n_seq][K+1]; n_acc_dev: int32
 *   [n_seq]; T_dev / logits_dev: optional fp32 [n_seq][K+1][vocab] copies of
 *   the target rows / logits (NULL: internal buffers).
 * Errors: SPEC_ERR_ARG (K outside 1..k_max, null pointers), SPEC_ERR_STATE (a
 * verify is pending), SPEC_ERR_CAPACITY (a sequence's positions would pass
 * max_seq). */
int spec_batch_verify(spec_batch* bc, int32_t K, uint64_t seed, const int32_t* d_dev,
                      const float* D_dev, int32_t* out_dev, int32_t* n_acc_dev, float* T_dev,
                      float* logits_dev);

/* Commits the last verify of every sequence from its outputs (same pointers
 * or copies): hist_b gets out[b][0..n_acc[b]], length L_b += n_acc[b] + 1;
 * the cache slots of rejected drafts are overwritten by the next pass.
 * Errors: SPEC_ERR_ARG (null), SPEC_ERR_STATE (no verify pending). */
int spec_batch_commit(spec_batch* bc, const int32_t* out_dev, const int32_t* n_acc_dev);

/* Waits for the context's stream. */
int spec_batch_sync(spec_batch* bc);
/* Synchronises, then copies every sequence's committed length L_b (the
 * pending token sits at hist_b[L_b]) and its sticky device error bits (1: a
 * token id out of range, 4: a position past max_seq); err_host may be NULL.
 *   len_host, err_host: int32 [n_seq]. */
int spec_batch_get_state(spec_batch* bc, int32_t* len_host, int32_t* err_host);
/* Synchronises, then copies hist_b[0..n) of sequence b into host_out. */
int spec_batch_get_history(spec_batch* bc, int32_t b, int32_t* host_out, int32_t n);
/* Last error message of the context (or of the thread's last failed call
 * when bc is NULL). */
const char* spec_batch_last_error(const spec_batch* bc);
/* Synchronises and frees everything the context owns; NULL accepted. */
int spec_batch_destroy(spec_batch* bc);

/* Choosing K from the measured acceptance rate (host-side helpers; no
 * context, no device work).
 * spec_expected_tokens: mean tokens one round yields when each of its K
 * drafts passes independently with probability alpha, 1 + alpha + ... +
 * alpha^K = (1 - alpha^(K+1)) / (1 - alpha) ([en] Floor 6; [zh] Level 6).
 * spec_alpha_from_tokens: the alpha at which that mean equals a measured
 * tokens-per-round figure for a given K (bisection; 0 at or below 1 token,
 * 1 at or above K+1).
 * spec_choose_k: the K in 1..k_max that maximises tokens per unit time,
 * spec_expected_tokens(alpha, K) / (K * t_draft_step + t_verify), with the
 * round cost of [int] "speedup" (K draft steps plus one target pass); ties go
 * to the smaller K.  Returns SPEC_ERR_ARG for alpha outside [0, 1], negative
 * times, both times 0, or k_max < 1. */
double spec_expected_tokens(double alpha, int32_t K);
double spec_alpha_from_tokens(double tokens_per_round, int32_t K);
int32_t spec_choose_k(double alpha, double t_draft_step, double t_verify, int32_t k_max);

/* Measurement helper, not a step of the method: the rate of a plain streaming
 * read (16-byte non-temporal loads, nothing else), the HBM ceiling that the
 * verify pass's GB/s is set against.  Reads bytes (a multiple of 16, at least
 * 1 MiB) of buf_dev reps times with 1, 2 and 4 workgroups per CU (each
 * workgroup one contiguous slice, 8 loads per lane in flight) and returns the
 * best rate in GB/s (1e9 bytes/s), timed with HIP events on hip_stream.
 * Synchronises the stream.  Errors: SPEC_ERR_ARG, SPEC_ERR_HIP. */
int spec_read_ceiling(const void* buf_dev, uint64_t bytes, int32_t reps, void* hip_stream,
                      double* gb_per_s);

/* Stateless accept/reject over a batch of independent sequences (the rule of
 * spec_verify without the forward pass).
 *   T_dev: fp32 [B][K+1][V]; D_dev: fp32 [B][K][V] (unused if greedy);
 *   d_dev: int32 [B][K]; pos_dev: uint64 [B], position of d_1 of each
 *   sequence; sequence b draws uniforms with counter (p, b, stream_id, 0);
 *   out_dev: int32 [B][K+1]; n_acc_dev: int32 [B] (-1 marks invalid input,
 *   as in spec_verify).
 *   hip_stream: hipStream_t (NULL = default stream).
 * Uses a library-owned workspace, allocated on first use and grown when a
 * larger B*V arrives (that call allocates).  Calls that overlap on one device
 * must not share it: serialise them on one stream.
 * Errors: SPEC_ERR_ARG (B < 0, K outside 1..SPEC_AR_K_MAX, V < 1, null
 * pointers), SPEC_ERR_OOM, SPEC_ERR_HIP. */
int spec_accept_reject(const float* T_dev, const float* D_dev, const int32_t* d_dev, int32_t B,
                       int32_t K, int32_t V, uint64_t seed, const uint64_t* pos_dev,
                       uint64_t stream_id, int32_t greedy, int32_t* out_dev, int32_t* n_acc_dev,
                       void* hip_stream);

/* spec_accept_reject for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, kernels and results, but the chunk
 * partials live in a fixed device array of SPEC_AR_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends.
 * No call allocates or frees device memory.  Every call on one device shares
 * that device's array and leaves its contents behind; calls that overlap on
 * one device (different streams, or with no ordering between them) race and
 * must be serialised by the caller.
 * Errors: those of spec_accept_reject, and SPEC_ERR_CAPACITY when B, K and V
 * need more scratch than the fixed size (B * chunks(B, V) * max(K + 2, 4)
 * 8-byte words, chunks(B, V) = min(ceil(512 / B), ceil(V / 1024), 512)
 * rounded up to whole 256-entry chunks; e.g. B = 64, K = 8, V = 32000 needs
 * 40 KiB). */
#define SPEC_AR_NOALLOC_SCRATCH_BYTES (2u << 20)
int spec_accept_reject_noalloc(const float* T_dev, const float* D_dev, const int32_t* d_dev,
                               int32_t B, int32_t K, int32_t V, uint64_t seed,
                               const uint64_t* pos_dev, uint64_t stream_id, int32_t greedy,
                               int32_t* out_dev, int32_t* n_acc_dev, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_H */
