/*
 * oracle.h -- plain CPU reference for speculative decoding (verify pass +
 * accept/reject rule).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU library never
 * links, calls or includes anything from here, and this file includes nothing
 * from the GPU library: the two share no code.
 *
 * Pages cited (by title and section):
 *   [zh]  "在神諭塔當見習抄寫刺蝟…：推測解碼入門" (gu-log Lv-19, zh-tw)
 *   [en]  "Apprentice Scribe Hedgehog at the Oracle Tower … Speculative
 *          Decoding 101" (gu-log Lv-19, English translation of [zh])
 *   [int] "Speculative decoding internals" (tarrragon LLM notes, module 3)
 *
 * Conventions
 *   - Probabilities are fp32 (the exchange type of the GPU library).  A value
 *     read by the rule is valid iff it is finite and 0 <= x <= 1 (-0.0 counts
 *     as 0).  Reading an invalid value is an error (ORC_EBADPROB).
 *   - Uniforms come from Philox4x64-10 keyed by (seed, 0) with counter
 *     (p, s, c, 0): p = absolute 0-based sequence position of the token being
 *     decided, s = sequence index, c = stream id.  Word w0 samples the draft
 *     token at p, w1 is the accept test of the draft at p, w2 samples the
 *     target at p, w3 is unused.  u24(w) = w >> 40, r = u24 * 2^-24.
 *   - The model forward runs in fp64 with bf16 weights widened exactly.
 */
#ifndef SPEC_ORACLE_H
#define SPEC_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_EBADPROB (-2)
#define ORC_ENOMEM (-3)
#define ORC_ECAPACITY (-4)

/* ---- counter-based uniforms -------------------------------------------- */
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);
void orc_uniform_words(uint64_t seed, uint64_t p, uint64_t s, uint64_t c, uint64_t w[4]);
uint32_t orc_u24(uint64_t w);

/* ---- sampler primitives ------------------------------------------------- */
/* fix(x) = floor(x * 2^40); returns ORC_OK or ORC_EBADPROB. */
int orc_fix(float x, uint64_t* out);
/* Smallest v with sum_{w<=v} q_w > floor(u24 * Z / 2^24), Z = sum q.  -1 if Z == 0. */
int32_t orc_sample_icdf(const uint64_t* q, int32_t V, uint32_t u24);
/* Smallest index attaining the fp32 maximum; -1 if V <= 0, -2 if a NaN is present. */
int32_t orc_argmax_low(const float* x, int32_t V);
/* Accept iff r*D < T evaluated exactly (fp32 x fp32 product is exact in fp64). */
int orc_accept(float r, float T, float D);

/* ---- accept / reject for one sequence ------------------------------------
 * T: [K+1][V], D: [K][V], d: [K].  P = position of the first new token (d_1).
 * out receives n_acc+1 tokens; *n_acc in 0..K.  Returns ORC_OK or an error
 * (then *n_acc = -1 and out[0..K] = -1). */
int orc_verify_sample(const float* T, const float* D, const int32_t* d, int32_t K, int32_t V,
                      uint64_t seed, uint64_t s, uint64_t c, uint64_t P,
                      int32_t* out, int32_t* n_acc);
/* Same rule with explicit u24 values instead of Philox: u_acc[i] for the
 * accept test of draft i (i = 0..K-1), u_smp for the one target sample. */
int orc_verify_sample_u(const float* T, const float* D, const int32_t* d, int32_t K, int32_t V,
                        const uint32_t* u_acc, uint32_t u_smp, int32_t* out, int32_t* n_acc);
int orc_verify_greedy(const float* T, const int32_t* d, int32_t K, int32_t V,
                      int32_t* out, int32_t* n_acc);
/* Batched form with the GPU library's stateless layout:
 * T [B][K+1][V], D [B][K][V], d [B][K], pos [B]; sequence b uses s = b.
 * Returns ORC_OK; per-sequence errors are n_acc[b] = -1, out[b][*] = -1. */
int orc_accept_reject_batch(const float* T, const float* D, const int32_t* d,
                            int32_t B, int32_t K, int32_t V, uint64_t seed,
                            const uint64_t* pos, uint64_t stream_id, int32_t greedy,
                            int32_t* out, int32_t* n_acc);
/* Draft token at position p from row Drow: inverse CDF on fix(D) with w0, or
 * argmax in greedy mode.  Returns the token, or a negative error. */
int32_t orc_draft_sample(const float* Drow, int32_t V, uint64_t seed, uint64_t p, uint64_t s,
                         uint64_t c, int32_t greedy);

/* ---- test helpers: exhaustive enumeration over the 2^24 grid ------------ */
/* counts[v] = #{u24 in [0,2^24) : sample_icdf(q, u24) == v} */
void orc_icdf_histogram(const uint64_t* q, int32_t V, uint64_t* counts);
/* #{u24 in [0,2^24) : accept(u24 * 2^-24, T, D)} */
uint64_t orc_accept_count(float T, float D);

/* ---- model (Llama-style pre-norm decoder, fp64) ------------------------- */
typedef struct orc_model {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  double rope_theta, rms_eps;
  /* bf16 bit patterns, stacked over layers, row-major [out][in]. */
  const uint16_t* embed;      /* [vocab][d] */
  const uint16_t* attn_norm;  /* [L][d] */
  const uint16_t* wq;         /* [L][n_heads*hd][d] */
  const uint16_t* wk;         /* [L][n_kv*hd][d] */
  const uint16_t* wv;         /* [L][n_kv*hd][d] */
  const uint16_t* wo;         /* [L][d][n_heads*hd] */
  const uint16_t* ffn_norm;   /* [L][d] */
  const uint16_t* wg;         /* [L][ffn][d] */
  const uint16_t* wu;         /* [L][ffn][d] */
  const uint16_t* wd;         /* [L][d][ffn] */
  const uint16_t* final_norm; /* [d] */
  const uint16_t* lm_head;    /* [vocab][d] */
} orc_model;

typedef struct orc_kv orc_kv;
orc_kv* orc_kv_new(const orc_model* m, int32_t max_seq);
void orc_kv_free(orc_kv* kv);

/* Runs n rows (tokens[r] at position pos0 + r) through the model, writing
 * their keys/values into kv.  If logits != NULL it receives [n][vocab] fp64
 * logits.  Rows attend to keys 0..pos0+r. */
int orc_forward(const orc_model* m, orc_kv* kv, const int32_t* tokens, int32_t n, int32_t pos0,
                double* logits);
/* orc_forward that also returns each row's final normed state
 * RMSNorm(x) * g_final ([n][d_model] fp64, nullable), the input of the LM head. */
int orc_forward_hidden(const orc_model* m, orc_kv* kv, const int32_t* tokens, int32_t n,
                       int32_t pos0, double* logits, double* hidden);
/* softmax of one fp64 logit row, rounded to fp32 */
void orc_softmax_f32(const double* logits, int32_t V, float* p);

/* ---- decode loops --------------------------------------------------------- */
typedef struct orc_spec_stats {
  int32_t rounds;
  int32_t target_passes;
  int32_t draft_passes;
  int64_t accepted;      /* sum of n_acc over rounds */
  int64_t emitted;       /* tokens emitted before truncation */
} orc_spec_stats;

/* Plain decode: prefill prompt[0..n-2], then n_new steps of forward(pending)
 * -> T -> argmax (greedy) or inverse CDF with w2 at the decided position. */
int orc_generate(const orc_model* m, const int32_t* prompt, int32_t n_prompt, int32_t n_new,
                 int32_t greedy, uint64_t seed, uint64_t c, int32_t* out);
/* Speculative decode: rounds of K draft steps, a (K+1)-row verify, the
 * accept/reject rule and commit, until >= n_new tokens, truncated to n_new.
 * nacc_per_round (nullable, capacity n_new) receives n_acc of each round. */
int orc_spec_generate(const orc_model* target, const orc_model* draft, const int32_t* prompt,
                      int32_t n_prompt, int32_t n_new, int32_t K, int32_t greedy, uint64_t seed,
                      uint64_t c, int32_t* out, int32_t* nacc_per_round, orc_spec_stats* st);

/* ---- primitives exposed for pinning ------------------------------------ */
void orc_rope(double* v, int32_t hd, int32_t pos, double theta);
void orc_rmsnorm(const double* x, int32_t d, const uint16_t* g, double eps, double* h);
/* one query head over n_keys keys/values stored [n_keys][hd] */
void orc_attend(const double* q, const double* k, const double* v, int32_t n_keys, int32_t hd,
                double* out);
/* out[b] = orc_draft_sample(D[b], ..., pos[b], s = b, c, greedy) */
int orc_draft_sample_batch(const float* D, int32_t B, int32_t V, uint64_t seed, const uint64_t* pos,
                           uint64_t c, int32_t greedy, int32_t* out);

/* ---- prompt-lookup (n-gram) drafter ---------------------------------------
 * [en] Floor 6 (and [zh] Level 6): n-gram approaches such as prompt lookup
 * draft by searching the preceding text for a chunk that repeats and
 * proposing what followed it; the verification rule is unchanged.
 * hist[0..L] is the committed text, hist[L] the pending token.  For
 * n = n_max down to 1 (n <= L), take the latest j in [n-1, L-1] with
 * hist[j-n+1..j] == hist[L-n+1..L]; the first n that has one is used.  The
 * draft is the text that followed, repeated with period p = L - j:
 * d[i] = hist[j + 1 + (i mod p)], i = 0..K-1.  Without any match,
 * d[i] = hist[L].  Returns the match length used (0: none) or ORC_EARG. */
int32_t orc_ngram_draft(const int32_t* hist, int32_t L, int32_t K, int32_t n_max, int32_t* d);

/* ---- choosing K from the acceptance rate --------------------------------
 * [en] Floor 6: with each draft passing independently with probability a, a
 * round yields (1 - a^(K+1)) / (1 - a) tokens on average (K + 1 at a = 1).
 * [int] "speedup": a round costs about K draft steps plus one target pass.
 * orc_choose_k returns the K in 1..k_max with the most tokens per unit of
 * round time, E(a, K) / (K t_draft + t_verify); ties go to the smaller K.
 * Returns ORC_EARG for a outside [0,1], negative times or k_max < 1. */
double orc_expected_tokens(double a, int32_t K);
int32_t orc_choose_k(double a, double t_draft, double t_verify, int32_t k_max);

/* ---- multi-token-prediction heads as the drafter -------------------------
 * [int] "variants" (MTP): the target carries K extra output heads, head k
 * predicting the token k places ahead; no separate drafter model.  Reading
 * (the pages fix no head architecture): head k maps the target's final normed
 * state h of the last position it processed to z_k = h + silu(W_k h), W_k a
 * [d][d] matrix (W_heads = [n_heads][d][d] bf16), scored by the target's LM
 * head: D_k = softmax(lm_head z_k).  The position after h holds the pending
 * token, already decided by the rule, so the K heads draft positions
 * P .. P+K-1 (P = position of d_1); d_k is drawn from D_k with word 0 at
 * P + k (argmax in greedy mode).  D: [K][V] fp32, d: [K].  K <= n_heads. */
int orc_heads_draft(const orc_model* m, const uint16_t* W_heads, int32_t n_heads, const double* h,
                    int32_t K, int32_t greedy, uint64_t seed, uint64_t P, uint64_t c, float* D,
                    int32_t* d);
/* Speculative decoding with the heads as the drafter (n_prompt >= 2: the
 * prefill must process at least one row).  Each round drafts from the kept
 * state, verifies K+1 rows, applies the rule and keeps the state of the last
 * committed row of the pass.  drafts_per_round (nullable, capacity n_new*K)
 * receives each round's drafts; the other outputs as in orc_spec_generate. */
int orc_spec_generate_heads(const orc_model* target, const uint16_t* W_heads, int32_t n_heads,
                            const int32_t* prompt, int32_t n_prompt, int32_t n_new, int32_t K,
                            int32_t greedy, uint64_t seed, uint64_t c, int32_t* out,
                            int32_t* nacc_per_round, int32_t* drafts_per_round,
                            orc_spec_stats* st);

int32_t orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
