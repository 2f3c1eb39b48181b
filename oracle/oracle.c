/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for speculative
 * decoding: the verify forward pass of a Llama-style decoder and the
 * accept/reject rule with its greedy variant.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Built with gcc -O2 -fopenmp
 * -ffp-contract=off, no fast-math.  OpenMP splits independent output features
 * only; every dot product is a sequential loop in index order, so results do
 * not depend on the thread count and a row's result does not depend on which
 * other rows are computed with it.
 *
 * Parity status of each part is stated at its definition:
 *   Philox, fix, sample_icdf, argmax_low, accept, verify_* -- pinned.
 *   Model forward -- the pages give no model equations, so it is pinned by
 *   the mathematics: invariants (causality, row invariance, GQA as MHA with
 *   repeated KV heads) and special cases of the whole pass computed another
 *   way (RoPE as complex rotation, scipy softmax and expit), which sixteen
 *   planted mistakes each fail (as fifteen planted in the rule, the sampler
 *   and Philox each fail their pins).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ======================================================================= */
/* Philox4x64-10.  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As  */
/* Easy as 1, 2, 3", SC'11: ten rounds of two 64x64->128 multiplies; the key */
/* is bumped by two Weyl constants between rounds.                           */
/* ======================================================================= */
static const uint64_t PHILOX_M0 = 0xD2E7470EE14C6C93ULL;
static const uint64_t PHILOX_M1 = 0xCA5A826395121157ULL;
static const uint64_t PHILOX_W0 = 0x9E3779B97F4A7C15ULL; /* golden ratio */
static const uint64_t PHILOX_W1 = 0xBB67AE8584CAA73BULL; /* sqrt(3) - 1 */

void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; round++) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    unsigned __int128 p0 = (unsigned __int128)PHILOX_M0 * c0;
    unsigned __int128 p1 = (unsigned __int128)PHILOX_M1 * c2;
    uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    uint64_t n0 = hi1 ^ c1 ^ k0;
    uint64_t n1 = lo1;
    uint64_t n2 = hi0 ^ c3 ^ k1;
    uint64_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The pages only say "r = uniform random in [0, 1]" ([int] algorithm core,
 * Step 3).  Reading adopted: r lies on the 2^-24 grid in [0, 1), drawn from a
 * counter keyed by the absolute position of the token being decided. */
void orc_uniform_words(uint64_t seed, uint64_t p, uint64_t s, uint64_t c, uint64_t w[4]) {
  const uint64_t ctr[4] = {p, s, c, 0};
  const uint64_t key[2] = {seed, 0};
  orc_philox4x64_10(ctr, key, w);
}

uint32_t orc_u24(uint64_t w) { return (uint32_t)(w >> 40); }

/* ======================================================================= */
/* Sampler primitives                                                        */
/* ======================================================================= */
static int prob_valid(float x) { return isfinite(x) && x >= 0.0f && x <= 1.0f; }

/* fix(x) = floor(x * 2^40).  x is fp32 in [0,1]: the scaling by a power of
 * two and the floor are exact in fp64. */
int orc_fix(float x, uint64_t* out) {
  if (!prob_valid(x)) return ORC_EBADPROB;
  double y = ldexp((double)x, 40);
  *out = (uint64_t)floor(y);
  return ORC_OK;
}

/* "Spin the wheel" ([zh] level 5, [en] Floor 5): each token owns a slice of
 * the wheel sized by its weight.  Reading adopted: inverse CDF over token ids
 * 0..V-1 in order; the needle t = floor(u24 * Z / 2^24) picks the first token
 * whose inclusive prefix sum exceeds t.  u24*Z can reach 2^86, so it is split
 * as u24*(Z>>24) + floor(u24*(Z mod 2^24) / 2^24), which is exact. */
int32_t orc_sample_icdf(const uint64_t* q, int32_t V, uint32_t u24) {
  uint64_t Z = 0;
  for (int32_t v = 0; v < V; v++) Z += q[v];
  if (Z == 0) return -1;
  uint64_t t = (uint64_t)u24 * (Z >> 24) + (((uint64_t)u24 * (Z & 0xFFFFFFULL)) >> 24);
  uint64_t acc = 0;
  for (int32_t v = 0; v < V; v++) {
    acc += q[v];
    if (acc > t) return v;
  }
  return -1; /* unreachable: t < Z */
}

/* Greedy "always pick the top-ranked word" ([en] Floor 4).  Ties go to the
 * lowest index (the pages do not say; numpy.argmax uses the same rule). */
int32_t orc_argmax_low(const float* x, int32_t V) {
  if (V <= 0) return -1;
  int32_t best = 0;
  if (isnan(x[0])) return -2;
  for (int32_t v = 1; v < V; v++) {
    if (isnan(x[v])) return -2;
    if (x[v] > x[best]) best = v;
  }
  return best;
}

/* Accept the draft iff r < min(1, T(d)/D(d)) ([int] algorithm core, Step 3;
 * [en] Floor 5 rule 2).  For D > 0 and r < 1 this equals r*D < T, which is
 * evaluated exactly: the product of two fp32 numbers fits in fp64.  D = 0
 * gives accept iff T > 0 (the limit T/D -> inf). */
int orc_accept(float r, float T, float D) {
  return (double)r * (double)D < (double)T;
}

/* ======================================================================= */
/* Accept / reject                                                           */
/* ======================================================================= */
static void fill_error(int32_t* out, int32_t K, int32_t* n_acc) {
  for (int32_t i = 0; i <= K; i++) out[i] = -1;
  *n_acc = -1;
}

/* q = fix(row) for a full row; ORC_EBADPROB if any value is invalid. */
static int fix_row(const float* row, int32_t V, uint64_t* q) {
  for (int32_t v = 0; v < V; v++)
    if (orc_fix(row[v], &q[v]) != ORC_OK) return ORC_EBADPROB;
  return ORC_OK;
}

/* Target sample from one row ("spin once", [en] Floor 5 last paragraph):
 * inverse CDF on fix(row), falling back to argmax if the row has no mass on
 * the 2^-40 grid. */
static int32_t sample_target_row(const float* row, int32_t V, uint32_t u24, uint64_t* q) {
  if (fix_row(row, V, q) != ORC_OK) return ORC_EBADPROB;
  int32_t tok = orc_sample_icdf(q, V, u24);
  if (tok < 0) tok = orc_argmax_low(row, V);
  return tok;
}

/* The core rule with explicit uniforms ([int] algorithm core, Steps 3-4;
 * [zh] level 5 rules 1-3; [en] Floor 5):
 *   for i = 1..K: accept d_i with probability min(1, T_i(d_i)/D_i(d_i));
 *   at the first reject, draw the replacement from normalize(max(0, T_i - D_i))
 *   and stop; if all K pass, draw the bonus token from T_{K+1}.
 * Readings: the residual is normalized implicitly by sampling the integer
 * weights fix(T_i) - fix(D_i) (saturating) with the inverse CDF; if the
 * residual has no mass (T_i == D_i on the grid) the replacement is drawn from
 * T_i, then argmax. */
int orc_verify_sample_u(const float* T, const float* D, const int32_t* d, int32_t K, int32_t V,
                        const uint32_t* u_acc, uint32_t u_smp, int32_t* out, int32_t* n_acc) {
  if (K < 1 || V < 1) return ORC_EARG;
  for (int32_t i = 0; i < K; i++)
    if (d[i] < 0 || d[i] >= V) { fill_error(out, K, n_acc); return ORC_EARG; }
  uint64_t* q = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)V);
  uint64_t* qd = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)V);
  if (!q || !qd) { free(q); free(qd); return ORC_ENOMEM; }
  int rc = ORC_OK;
  int32_t i;
  for (i = 0; i < K; i++) {
    const float* Ti = T + (size_t)i * V;
    const float* Di = D + (size_t)i * V;
    float t = Ti[d[i]], dd = Di[d[i]];
    if (!prob_valid(t) || !prob_valid(dd)) { rc = ORC_EBADPROB; break; }
    float r = (float)u_acc[i] * 0x1p-24f;
    if (orc_accept(r, t, dd)) {
      out[i] = d[i];
      continue;
    }
    /* first reject: residual max(0, T_i - D_i) on the 2^-40 grid */
    if (fix_row(Ti, V, q) != ORC_OK || fix_row(Di, V, qd) != ORC_OK) { rc = ORC_EBADPROB; break; }
    for (int32_t v = 0; v < V; v++) q[v] = q[v] > qd[v] ? q[v] - qd[v] : 0;
    int32_t tok = orc_sample_icdf(q, V, u_smp);
    if (tok < 0) tok = sample_target_row(Ti, V, u_smp, q);
    if (tok < 0) { rc = ORC_EBADPROB; break; }
    out[i] = tok;
    *n_acc = i;
    free(q); free(qd);
    return ORC_OK;
  }
  if (rc == ORC_OK) {
    /* all K accepted: bonus token from T_{K+1} */
    int32_t tok = sample_target_row(T + (size_t)K * V, V, u_smp, q);
    if (tok < 0) rc = ORC_EBADPROB;
    else { out[K] = tok; *n_acc = K; }
  }
  free(q); free(qd);
  if (rc != ORC_OK) fill_error(out, K, n_acc);
  return rc;
}

/* The same rule with Philox uniforms: draft i (1-based) sits at position
 * P+i-1; its accept test uses w1 there, and the single target sample uses w2
 * at the position of the token it decides (P+i-1 on a reject at i, P+K for
 * the bonus). */
int orc_verify_sample(const float* T, const float* D, const int32_t* d, int32_t K, int32_t V,
                      uint64_t seed, uint64_t s, uint64_t c, uint64_t P,
                      int32_t* out, int32_t* n_acc) {
  if (K < 1 || V < 1) return ORC_EARG;
  uint32_t* u_acc = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)K);
  if (!u_acc) return ORC_ENOMEM;
  uint64_t w[4];
  for (int32_t i = 0; i < K; i++) {
    orc_uniform_words(seed, P + (uint64_t)i, s, c, w);
    u_acc[i] = orc_u24(w[1]);
  }
  /* The target sample's position depends on where the first reject falls;
   * find it with the same exact test (no sampling yet). */
  int32_t j = K;
  for (int32_t i = 0; i < K; i++) {
    if (d[i] < 0 || d[i] >= V) { j = i; break; }
    float t = T[(size_t)i * V + d[i]], dd = D[(size_t)i * V + d[i]];
    if (!prob_valid(t) || !prob_valid(dd)) { j = i; break; }
    if (!orc_accept((float)u_acc[i] * 0x1p-24f, t, dd)) { j = i; break; }
  }
  orc_uniform_words(seed, P + (uint64_t)j, s, c, w);
  int rc = orc_verify_sample_u(T, D, d, K, V, u_acc, orc_u24(w[2]), out, n_acc);
  free(u_acc);
  return rc;
}

/* Greedy checking ([zh] level 4, [en] Floor 4): a draft passes if it equals
 * the target's top word; the first mismatch takes the target's word and ends
 * the round; if all K pass, the target's top word at the last slot is the
 * free extra.  Every row T_1..T_{K+1} is validated. */
int orc_verify_greedy(const float* T, const int32_t* d, int32_t K, int32_t V,
                      int32_t* out, int32_t* n_acc) {
  if (K < 1 || V < 1) return ORC_EARG;
  for (int32_t i = 0; i < K; i++)
    if (d[i] < 0 || d[i] >= V) { fill_error(out, K, n_acc); return ORC_EARG; }
  for (int32_t i = 0; i <= K; i++)
    for (int32_t v = 0; v < V; v++)
      if (!prob_valid(T[(size_t)i * V + v])) { fill_error(out, K, n_acc); return ORC_EBADPROB; }
  for (int32_t i = 0; i < K; i++) {
    int32_t a = orc_argmax_low(T + (size_t)i * V, V);
    out[i] = a;
    if (a != d[i]) { *n_acc = i; return ORC_OK; }
  }
  out[K] = orc_argmax_low(T + (size_t)K * V, V);
  *n_acc = K;
  return ORC_OK;
}

int orc_accept_reject_batch(const float* T, const float* D, const int32_t* d,
                            int32_t B, int32_t K, int32_t V, uint64_t seed,
                            const uint64_t* pos, uint64_t stream_id, int32_t greedy,
                            int32_t* out, int32_t* n_acc) {
  if (B < 0 || K < 1 || V < 1) return ORC_EARG;
  for (int32_t b = 0; b < B; b++) {
    const float* Tb = T + (size_t)b * (K + 1) * V;
    const float* Db = D + (size_t)b * K * V;
    const int32_t* db = d + (size_t)b * K;
    int32_t* ob = out + (size_t)b * (K + 1);
    for (int32_t i = 0; i <= K; i++) ob[i] = -1;
    if (greedy)
      orc_verify_greedy(Tb, db, K, V, ob, &n_acc[b]);
    else
      orc_verify_sample(Tb, Db, db, K, V, seed, (uint64_t)b, stream_id, pos[b], ob, &n_acc[b]);
  }
  return ORC_OK;
}

/* The draft "spins its own wheel" ([en] Floor 5 rule 1) with w0 at the
 * draft's position, or takes its top word in greedy mode. */
int32_t orc_draft_sample(const float* Drow, int32_t V, uint64_t seed, uint64_t p, uint64_t s,
                         uint64_t c, int32_t greedy) {
  if (V < 1) return ORC_EARG;
  for (int32_t v = 0; v < V; v++)
    if (!prob_valid(Drow[v])) return ORC_EBADPROB;
  if (greedy) return orc_argmax_low(Drow, V);
  uint64_t w[4];
  orc_uniform_words(seed, p, s, c, w);
  uint64_t* q = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)V);
  if (!q) return ORC_ENOMEM;
  int32_t tok = sample_target_row(Drow, V, orc_u24(w[0]), q);
  free(q);
  return tok;
}

void orc_icdf_histogram(const uint64_t* q, int32_t V, uint64_t* counts) {
  for (int32_t v = 0; v < V; v++) counts[v] = 0;
  for (uint32_t u = 0; u < (1u << 24); u++) {
    int32_t t = orc_sample_icdf(q, V, u);
    if (t >= 0) counts[t]++;
  }
}

uint64_t orc_accept_count(float T, float D) {
  uint64_t n = 0;
  for (uint32_t u = 0; u < (1u << 24); u++) n += (uint64_t)orc_accept((float)u * 0x1p-24f, T, D);
  return n;
}

/* ======================================================================= */
/* Model forward (fp64).  The pages name a "forward pass" that yields a     */
/* next-token distribution at every position ([en] Floor 3) but give no     */
/* equations.  The decoder below is the standard Llama-style pre-norm       */
/* block: RMSNorm, rotate-half RoPE, causal GQA attention, SwiGLU FFN,      */
/* final RMSNorm, untied LM head, softmax at T = 1; its pins are those of   */
/* the mathematics (header above).                                          */
/* ======================================================================= */
static double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

struct orc_kv {
  int32_t max_seq, n_layers, n_kv, hd;
  double* k; /* [L][max_seq][n_kv][hd] */
  double* v;
};

orc_kv* orc_kv_new(const orc_model* m, int32_t max_seq) {
  orc_kv* kv = (orc_kv*)calloc(1, sizeof(orc_kv));
  if (!kv) return NULL;
  kv->max_seq = max_seq;
  kv->n_layers = m->n_layers;
  kv->n_kv = m->n_kv_heads;
  kv->hd = m->head_dim;
  size_t n = (size_t)m->n_layers * max_seq * m->n_kv_heads * m->head_dim;
  kv->k = (double*)calloc(n ? n : 1, sizeof(double));
  kv->v = (double*)calloc(n ? n : 1, sizeof(double));
  if (!kv->k || !kv->v) { orc_kv_free(kv); return NULL; }
  return kv;
}

void orc_kv_free(orc_kv* kv) {
  if (!kv) return;
  free(kv->k);
  free(kv->v);
  free(kv);
}

/* y[r][o] = sum_k x[r][k] * W[o][k], each dot product sequential in k. */
static void matmul_rows(const double* x, int32_t n, int32_t in, const uint16_t* W, int32_t outf,
                        double* y) {
#pragma omp parallel for schedule(static)
  for (int32_t o = 0; o < outf; o++) {
    const uint16_t* w = W + (size_t)o * in;
    for (int32_t r = 0; r < n; r++) {
      const double* xr = x + (size_t)r * in;
      double acc = 0.0;
      for (int32_t k = 0; k < in; k++) acc += xr[k] * bf16_to_f64(w[k]);
      y[(size_t)r * outf + o] = acc;
    }
  }
}

/* h = x / sqrt(mean(x^2) + eps) * g */
static void rmsnorm_row(const double* x, int32_t d, const uint16_t* g, double eps, double* h) {
  double ss = 0.0;
  for (int32_t k = 0; k < d; k++) ss += x[k] * x[k];
  double inv = 1.0 / sqrt(ss / (double)d + eps);
  for (int32_t k = 0; k < d; k++) h[k] = x[k] * inv * bf16_to_f64(g[k]);
}

/* Rotate-half RoPE on one head vector: pairs (j, j + hd/2) turn by the angle
 * pos * theta^(-2j/hd). */
static void rope_head(double* v, int32_t hd, int32_t pos, double theta) {
  int32_t half = hd / 2;
  for (int32_t j = 0; j < half; j++) {
    double ang = (double)pos * pow(theta, -2.0 * (double)j / (double)hd);
    double c = cos(ang), s = sin(ang);
    double a = v[j], b = v[j + half];
    v[j] = a * c - b * s;
    v[j + half] = b * c + a * s;
  }
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* Causal attention of one query head over keys 0..n_keys-1 (key t at
 * kbase + t*stride): softmax(q.k_t / sqrt(hd)) with max subtraction, then the
 * probability-weighted sum of the values.  sc is scratch of n_keys doubles. */
static void attend_head(const double* qv, const double* kbase, const double* vbase, size_t stride,
                        int32_t n_keys, int32_t hd, double* sc, double* ov) {
  const double scale = 1.0 / sqrt((double)hd);
  double mx = -INFINITY;
  for (int32_t t = 0; t < n_keys; t++) {
    const double* kt = kbase + (size_t)t * stride;
    double s = 0.0;
    for (int32_t e = 0; e < hd; e++) s += qv[e] * kt[e];
    sc[t] = s * scale;
    if (sc[t] > mx) mx = sc[t];
  }
  double den = 0.0;
  for (int32_t t = 0; t < n_keys; t++) {
    sc[t] = exp(sc[t] - mx);
    den += sc[t];
  }
  for (int32_t e = 0; e < hd; e++) ov[e] = 0.0;
  for (int32_t t = 0; t < n_keys; t++) {
    const double* vt = vbase + (size_t)t * stride;
    const double p = sc[t] / den;
    for (int32_t e = 0; e < hd; e++) ov[e] += p * vt[e];
  }
}

/* The forward pass of n rows; `hidden` (nullable) receives each row's final
 * normed state RMSNorm(x) * g_final, the vector the LM head scores. */
static int forward_impl(const orc_model* m, orc_kv* kv, const int32_t* tokens, int32_t n,
                        int32_t pos0, double* logits, double* hidden) {
  if (n <= 0) return ORC_OK;
  if (pos0 < 0 || pos0 + n > kv->max_seq) return ORC_ECAPACITY;
  const int32_t d = m->d_model, H = m->n_heads, Hkv = m->n_kv_heads, hd = m->head_dim;
  const int32_t qd = H * hd, kvd = Hkv * hd, F = m->d_ffn, V = m->vocab;
  for (int32_t r = 0; r < n; r++)
    if (tokens[r] < 0 || tokens[r] >= V) return ORC_EARG;
  double* x = (double*)malloc(sizeof(double) * (size_t)n * d);
  double* h = (double*)malloc(sizeof(double) * (size_t)n * d);
  double* q = (double*)malloc(sizeof(double) * (size_t)n * qd);
  double* k = (double*)malloc(sizeof(double) * (size_t)n * kvd);
  double* v = (double*)malloc(sizeof(double) * (size_t)n * kvd);
  double* o = (double*)malloc(sizeof(double) * (size_t)n * qd);
  double* y = (double*)malloc(sizeof(double) * (size_t)n * d);
  double* g = (double*)malloc(sizeof(double) * (size_t)n * F);
  double* u = (double*)malloc(sizeof(double) * (size_t)n * F);
  double* sc = (double*)malloc(sizeof(double) * (size_t)(pos0 + n));
  if (!x || !h || !q || !k || !v || !o || !y || !g || !u || !sc) {
    free(x); free(h); free(q); free(k); free(v); free(o); free(y); free(g); free(u); free(sc);
    return ORC_ENOMEM;
  }
  for (int32_t r = 0; r < n; r++)
    for (int32_t c = 0; c < d; c++)
      x[(size_t)r * d + c] = bf16_to_f64(m->embed[(size_t)tokens[r] * d + c]);

  for (int32_t l = 0; l < m->n_layers; l++) {
    /* attention block */
    for (int32_t r = 0; r < n; r++)
      rmsnorm_row(x + (size_t)r * d, d, m->attn_norm + (size_t)l * d, m->rms_eps, h + (size_t)r * d);
    matmul_rows(h, n, d, m->wq + (size_t)l * qd * d, qd, q);
    matmul_rows(h, n, d, m->wk + (size_t)l * kvd * d, kvd, k);
    matmul_rows(h, n, d, m->wv + (size_t)l * kvd * d, kvd, v);
    for (int32_t r = 0; r < n; r++) {
      const int32_t pos = pos0 + r;
      for (int32_t hh = 0; hh < H; hh++) rope_head(q + (size_t)r * qd + (size_t)hh * hd, hd, pos, m->rope_theta);
      for (int32_t hh = 0; hh < Hkv; hh++) rope_head(k + (size_t)r * kvd + (size_t)hh * hd, hd, pos, m->rope_theta);
      double* kc = kv->k + (((size_t)l * kv->max_seq + pos) * Hkv) * hd;
      double* vc = kv->v + (((size_t)l * kv->max_seq + pos) * Hkv) * hd;
      memcpy(kc, k + (size_t)r * kvd, sizeof(double) * kvd);
      memcpy(vc, v + (size_t)r * kvd, sizeof(double) * kvd);
    }
    for (int32_t r = 0; r < n; r++) {
      const int32_t pos = pos0 + r;
      for (int32_t hh = 0; hh < H; hh++) {
        const int32_t kh = (int32_t)(((int64_t)hh * Hkv) / H); /* GQA group */
        const double* kb = kv->k + (((size_t)l * kv->max_seq) * Hkv + kh) * hd;
        const double* vb = kv->v + (((size_t)l * kv->max_seq) * Hkv + kh) * hd;
        attend_head(q + (size_t)r * qd + (size_t)hh * hd, kb, vb, (size_t)Hkv * hd, pos + 1, hd,
                    sc, o + (size_t)r * qd + (size_t)hh * hd);
      }
    }
    matmul_rows(o, n, qd, m->wo + (size_t)l * d * qd, d, y);
    for (size_t i = 0; i < (size_t)n * d; i++) x[i] += y[i];
    /* feed-forward block */
    for (int32_t r = 0; r < n; r++)
      rmsnorm_row(x + (size_t)r * d, d, m->ffn_norm + (size_t)l * d, m->rms_eps, h + (size_t)r * d);
    matmul_rows(h, n, d, m->wg + (size_t)l * F * d, F, g);
    matmul_rows(h, n, d, m->wu + (size_t)l * F * d, F, u);
    for (size_t i = 0; i < (size_t)n * F; i++) g[i] = silu(g[i]) * u[i];
    matmul_rows(g, n, F, m->wd + (size_t)l * d * F, d, y);
    for (size_t i = 0; i < (size_t)n * d; i++) x[i] += y[i];
  }
  if (logits || hidden) {
    for (int32_t r = 0; r < n; r++)
      rmsnorm_row(x + (size_t)r * d, d, m->final_norm, m->rms_eps, h + (size_t)r * d);
    if (hidden) memcpy(hidden, h, sizeof(double) * (size_t)n * d);
    if (logits) matmul_rows(h, n, d, m->lm_head, V, logits);
  }
  free(x); free(h); free(q); free(k); free(v); free(o); free(y); free(g); free(u); free(sc);
  return ORC_OK;
}

int orc_forward(const orc_model* m, orc_kv* kv, const int32_t* tokens, int32_t n, int32_t pos0,
                double* logits) {
  return forward_impl(m, kv, tokens, n, pos0, logits, NULL);
}

int orc_forward_hidden(const orc_model* m, orc_kv* kv, const int32_t* tokens, int32_t n,
                       int32_t pos0, double* logits, double* hidden) {
  return forward_impl(m, kv, tokens, n, pos0, logits, hidden);
}

/* Temperature-1 softmax with max subtraction, in fp64, rounded to fp32. */
void orc_softmax_f32(const double* logits, int32_t V, float* p) {
  double mx = -INFINITY;
  for (int32_t v = 0; v < V; v++)
    if (logits[v] > mx) mx = logits[v];
  double den = 0.0;
  for (int32_t v = 0; v < V; v++) den += exp(logits[v] - mx);
  for (int32_t v = 0; v < V; v++) p[v] = (float)(exp(logits[v] - mx) / den);
}

/* ======================================================================= */
/* Decode loops                                                              */
/* ======================================================================= */
/* One-token-per-pass decoding ([en] Floor 1): the pending token (last one
 * emitted) is fed back; the next token is decided at position pos+1. */
int orc_generate(const orc_model* m, const int32_t* prompt, int32_t n_prompt, int32_t n_new,
                 int32_t greedy, uint64_t seed, uint64_t c, int32_t* out) {
  if (n_prompt < 1 || n_new < 0) return ORC_EARG;
  const int32_t V = m->vocab;
  orc_kv* kv = orc_kv_new(m, n_prompt + n_new + 1);
  double* lg = (double*)malloc(sizeof(double) * (size_t)V);
  float* p = (float*)malloc(sizeof(float) * (size_t)V);
  uint64_t* q = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)V);
  int rc = (kv && lg && p && q) ? ORC_OK : ORC_ENOMEM;
  if (rc == ORC_OK && n_prompt > 1) rc = orc_forward(m, kv, prompt, n_prompt - 1, 0, NULL);
  int32_t pending = prompt[n_prompt - 1];
  for (int32_t i = 0; rc == ORC_OK && i < n_new; i++) {
    const int32_t pos = n_prompt - 1 + i;
    rc = orc_forward(m, kv, &pending, 1, pos, lg);
    if (rc != ORC_OK) break;
    orc_softmax_f32(lg, V, p);
    int32_t tok;
    if (greedy) {
      tok = orc_argmax_low(p, V);
    } else {
      uint64_t w[4];
      orc_uniform_words(seed, (uint64_t)pos + 1, 0, c, w);
      tok = sample_target_row(p, V, orc_u24(w[2]), q);
    }
    if (tok < 0) { rc = ORC_EBADPROB; break; }
    out[i] = tok;
    pending = tok;
  }
  orc_kv_free(kv);
  free(lg); free(p); free(q);
  return rc;
}

/* Speculative decoding rounds ([int] algorithm core Steps 1-4; [en] Boss
 * Level).  State: hist[0..L_T] holds every committed token; the target cache
 * holds positions 0..L_T-1 and hist[L_T] is the pending token.  The draft
 * cache holds positions 0..L_D-1 (L_D <= L_T).
 *   draft:  rows hist[L_D..L_T] then d_1..d_{K-1}, one step per token; the
 *           last row of each step gives D_{s+1} and d_{s+1} at L_T+s+1.
 *   verify: rows [hist[L_T], d_1..d_K] at positions L_T..L_T+K give
 *           T_1..T_{K+1}.
 *   commit: keep the pending token and the n accepted drafts ([en] Floor 4:
 *           slips after a reject are torn up); the emitted replacement or
 *           bonus becomes the next pending token. */
int orc_spec_generate(const orc_model* target, const orc_model* draft, const int32_t* prompt,
                      int32_t n_prompt, int32_t n_new, int32_t K, int32_t greedy, uint64_t seed,
                      uint64_t c, int32_t* out, int32_t* nacc_per_round, orc_spec_stats* st) {
  if (n_prompt < 1 || n_new < 0 || K < 1) return ORC_EARG;
  if (target->vocab != draft->vocab) return ORC_EARG; /* shared vocabulary ([en] Floor 6) */
  const int32_t V = target->vocab;
  const int32_t cap = n_prompt + n_new + K + 2;
  orc_kv* kvT = orc_kv_new(target, cap);
  orc_kv* kvD = orc_kv_new(draft, cap);
  int32_t* hist = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
  double* lgD = (double*)malloc(sizeof(double) * (size_t)cap * V);
  double* lgT = (double*)malloc(sizeof(double) * (size_t)(K + 1) * V);
  float* Dp = (float*)malloc(sizeof(float) * (size_t)K * V);
  float* Tp = (float*)malloc(sizeof(float) * (size_t)(K + 1) * V);
  int32_t* dr = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
  int32_t* ob = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
  orc_spec_stats s0 = {0, 0, 0, 0, 0};
  int rc = (kvT && kvD && hist && lgD && lgT && Dp && Tp && dr && rows && ob) ? ORC_OK : ORC_ENOMEM;
  if (rc == ORC_OK) {
    memcpy(hist, prompt, sizeof(int32_t) * (size_t)n_prompt);
    if (n_prompt > 1) rc = orc_forward(target, kvT, prompt, n_prompt - 1, 0, NULL);
    if (rc == ORC_OK && n_prompt > 1) rc = orc_forward(draft, kvD, prompt, n_prompt - 1, 0, NULL);
  }
  int32_t LT = n_prompt - 1, LD = n_prompt - 1, emitted = 0;
  while (rc == ORC_OK && emitted < n_new) {
    /* Step 1: K draft tokens and their distributions */
    for (int32_t s = 0; s < K && rc == ORC_OK; s++) {
      int32_t nrows, p0;
      const int32_t* toks;
      if (s == 0) { nrows = LT - LD + 1; p0 = LD; toks = hist + LD; }
      else { nrows = 1; p0 = LT + s; toks = &dr[s - 1]; }
      rc = orc_forward(draft, kvD, toks, nrows, p0, lgD);
      if (rc != ORC_OK) break;
      s0.draft_passes++;
      float* Ds = Dp + (size_t)s * V;
      orc_softmax_f32(lgD + (size_t)(nrows - 1) * V, V, Ds);
      int32_t t = orc_draft_sample(Ds, V, seed, (uint64_t)(LT + s + 1), 0, c, greedy);
      if (t < 0) { rc = ORC_EBADPROB; break; }
      dr[s] = t;
    }
    if (rc != ORC_OK) break;
    /* Step 2: one target pass over K+1 positions */
    rows[0] = hist[LT];
    for (int32_t i = 0; i < K; i++) rows[i + 1] = dr[i];
    rc = orc_forward(target, kvT, rows, K + 1, LT, lgT);
    if (rc != ORC_OK) break;
    s0.target_passes++;
    for (int32_t i = 0; i <= K; i++) orc_softmax_f32(lgT + (size_t)i * V, V, Tp + (size_t)i * V);
    /* Steps 3-4: accept/reject, replacement or bonus */
    int32_t n;
    if (greedy) rc = orc_verify_greedy(Tp, dr, K, V, ob, &n);
    else rc = orc_verify_sample(Tp, Dp, dr, K, V, seed, 0, c, (uint64_t)(LT + 1), ob, &n);
    if (rc != ORC_OK) break;
    /* commit */
    for (int32_t i = 0; i <= n; i++) hist[LT + 1 + i] = ob[i];
    LD = LT + (n + 1 < K ? n + 1 : K);
    LT += n + 1;
    if (nacc_per_round && s0.rounds < n_new) nacc_per_round[s0.rounds] = n;
    s0.rounds++;
    s0.accepted += n;
    s0.emitted += n + 1;
    for (int32_t i = 0; i <= n && emitted < n_new; i++) out[emitted++] = ob[i];
  }
  if (st) *st = s0;
  orc_kv_free(kvT); orc_kv_free(kvD);
  free(hist); free(lgD); free(lgT); free(Dp); free(Tp); free(dr); free(rows); free(ob);
  return rc;
}

/* ======================================================================= */
/* Multi-token-prediction heads as the drafter ([int] "variants": MTP gives  */
/* the target K extra output heads, head k predicting the token k places    */
/* ahead, so no separate drafter model is needed).  The pages fix no head   */
/* architecture; the reading used here: head k takes the target's final     */
/* normed state h of the last position it processed, z_k = h + silu(W_k h)  */
/* with its own [d][d] matrix, and scores z_k with the target's own LM head. */
/* The position right after h is the pending token, already decided by the  */
/* rule, so the K heads draft the K positions after it.                      */
/* ======================================================================= */
int orc_heads_draft(const orc_model* m, const uint16_t* W_heads, int32_t n_heads, const double* h,
                    int32_t K, int32_t greedy, uint64_t seed, uint64_t P, uint64_t c, float* D,
                    int32_t* d) {
  if (!m || !W_heads || !h || !D || !d || K < 1 || K > n_heads) return ORC_EARG;
  const int32_t dm = m->d_model, V = m->vocab;
  double* y = (double*)malloc(sizeof(double) * (size_t)dm);
  double* z = (double*)malloc(sizeof(double) * (size_t)dm);
  double* lg = (double*)malloc(sizeof(double) * (size_t)V);
  int rc = (y && z && lg) ? ORC_OK : ORC_ENOMEM;
  for (int32_t k = 0; rc == ORC_OK && k < K; k++) {
    matmul_rows(h, 1, dm, W_heads + (size_t)k * dm * dm, dm, y);
    for (int32_t i = 0; i < dm; i++) z[i] = h[i] + silu(y[i]);
    matmul_rows(z, 1, dm, m->lm_head, V, lg);
    float* Dk = D + (size_t)k * V;
    orc_softmax_f32(lg, V, Dk);
    /* d_k decides position P + k, drawn like any draft token (word 0) */
    const int32_t t = orc_draft_sample(Dk, V, seed, P + (uint64_t)k, 0, c, greedy);
    if (t < 0) rc = ORC_EBADPROB;
    else d[k] = t;
  }
  free(y); free(z); free(lg);
  return rc;
}

/* Speculative decoding with the heads as the drafter: the prompt prefill
 * keeps the normed state of its last row; each round drafts K tokens from
 * the kept state, runs the (K+1)-row verify pass and the rule, commits, and
 * keeps the state of the last committed row of the pass (row n_acc: the
 * pending token or the last accepted draft), whose successor is the new
 * pending token.  drafts_per_round (nullable, capacity n_new*K) receives
 * each round's drafts. */
int orc_spec_generate_heads(const orc_model* target, const uint16_t* W_heads, int32_t n_heads,
                            const int32_t* prompt, int32_t n_prompt, int32_t n_new, int32_t K,
                            int32_t greedy, uint64_t seed, uint64_t c, int32_t* out,
                            int32_t* nacc_per_round, int32_t* drafts_per_round,
                            orc_spec_stats* st) {
  if (n_prompt < 2 || n_new < 0 || K < 1 || K > n_heads || !W_heads) return ORC_EARG;
  const int32_t V = target->vocab, dm = target->d_model;
  const int32_t cap = n_prompt + n_new + K + 2;
  orc_kv* kvT = orc_kv_new(target, cap);
  int32_t* hist = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
  double* hid = (double*)malloc(sizeof(double) * (size_t)(n_prompt > K + 1 ? n_prompt : K + 1) * dm);
  double* hlast = (double*)malloc(sizeof(double) * (size_t)dm);
  double* lgT = (double*)malloc(sizeof(double) * (size_t)(K + 1) * V);
  float* Dp = (float*)malloc(sizeof(float) * (size_t)K * V);
  float* Tp = (float*)malloc(sizeof(float) * (size_t)(K + 1) * V);
  int32_t* dr = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
  int32_t* ob = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K + 1));
  orc_spec_stats s0 = {0, 0, 0, 0, 0};
  int rc = (kvT && hist && hid && hlast && lgT && Dp && Tp && dr && rows && ob) ? ORC_OK
                                                                                : ORC_ENOMEM;
  if (rc == ORC_OK) {
    memcpy(hist, prompt, sizeof(int32_t) * (size_t)n_prompt);
    rc = forward_impl(target, kvT, prompt, n_prompt - 1, 0, NULL, hid);
    if (rc == ORC_OK) memcpy(hlast, hid + (size_t)(n_prompt - 2) * dm, sizeof(double) * dm);
  }
  int32_t LT = n_prompt - 1, emitted = 0;
  while (rc == ORC_OK && emitted < n_new) {
    rc = orc_heads_draft(target, W_heads, n_heads, hlast, K, greedy, seed, (uint64_t)(LT + 1), c,
                         Dp, dr);
    if (rc != ORC_OK) break;
    s0.draft_passes++;
    if (drafts_per_round && s0.rounds < n_new)
      memcpy(drafts_per_round + (size_t)s0.rounds * K, dr, sizeof(int32_t) * K);
    rows[0] = hist[LT];
    for (int32_t i = 0; i < K; i++) rows[i + 1] = dr[i];
    rc = forward_impl(target, kvT, rows, K + 1, LT, lgT, hid);
    if (rc != ORC_OK) break;
    s0.target_passes++;
    for (int32_t i = 0; i <= K; i++) orc_softmax_f32(lgT + (size_t)i * V, V, Tp + (size_t)i * V);
    int32_t n;
    if (greedy) rc = orc_verify_greedy(Tp, dr, K, V, ob, &n);
    else rc = orc_verify_sample(Tp, Dp, dr, K, V, seed, 0, c, (uint64_t)(LT + 1), ob, &n);
    if (rc != ORC_OK) break;
    for (int32_t i = 0; i <= n; i++) hist[LT + 1 + i] = ob[i];
    memcpy(hlast, hid + (size_t)n * dm, sizeof(double) * dm);
    LT += n + 1;
    if (nacc_per_round && s0.rounds < n_new) nacc_per_round[s0.rounds] = n;
    s0.rounds++;
    s0.accepted += n;
    s0.emitted += n + 1;
    for (int32_t i = 0; i <= n && emitted < n_new; i++) out[emitted++] = ob[i];
  }
  if (st) *st = s0;
  orc_kv_free(kvT);
  free(hist); free(hid); free(hlast); free(lgT); free(Dp); free(Tp); free(dr); free(rows); free(ob);
  return rc;
}

int32_t orc_num_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- primitives exposed for pinning ------------------------------------ */
void orc_rope(double* v, int32_t hd, int32_t pos, double theta) { rope_head(v, hd, pos, theta); }

void orc_rmsnorm(const double* x, int32_t d, const uint16_t* g, double eps, double* h) {
  rmsnorm_row(x, d, g, eps, h);
}

void orc_attend(const double* q, const double* k, const double* v, int32_t n_keys, int32_t hd,
                double* out) {
  double* sc = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
  if (!sc) return;
  attend_head(q, k, v, (size_t)hd, n_keys, hd, sc, out);
  free(sc);
}

int orc_draft_sample_batch(const float* D, int32_t B, int32_t V, uint64_t seed, const uint64_t* pos,
                           uint64_t c, int32_t greedy, int32_t* out) {
  for (int32_t b = 0; b < B; b++)
    out[b] = orc_draft_sample(D + (size_t)b * V, V, seed, pos[b], (uint64_t)b, c, greedy);
  return ORC_OK;
}

/* ---- prompt-lookup (n-gram) drafter ([en] Floor 6: prompt lookup searches
 * the preceding text for a chunk likely to repeat and drafts what followed).
 * Longest key first, latest occurrence first: a plain double loop. */
int32_t orc_ngram_draft(const int32_t* hist, int32_t L, int32_t K, int32_t n_max, int32_t* d) {
  if (!hist || !d || L < 0 || K < 1 || n_max < 1) return ORC_EARG;
  for (int32_t n = n_max < L ? n_max : L; n >= 1; n--) {
    for (int32_t j = L - 1; j >= n - 1; j--) {
      int32_t same = 1;
      for (int32_t t = 0; t < n && same; t++) same = hist[j - t] == hist[L - t];
      if (same) {
        const int32_t p = L - j;
        for (int32_t i = 0; i < K; i++) d[i] = hist[j + 1 + i % p];
        return n;
      }
    }
  }
  for (int32_t i = 0; i < K; i++) d[i] = hist[L];
  return 0;
}

/* ---- K choice ([en] Floor 6 expected tokens; [int] "speedup" cost model) */
double orc_expected_tokens(double a, int32_t K) {
  /* the sum 1 + a + ... + a^K, term by term */
  double sum = 0.0, term = 1.0;
  for (int32_t j = 0; j <= K; j++) {
    sum += term;
    term *= a;
  }
  return sum;
}

int32_t orc_choose_k(double a, double t_draft, double t_verify, int32_t k_max) {
  if (!(a >= 0.0 && a <= 1.0) || !(t_draft >= 0.0) || !(t_verify >= 0.0) || k_max < 1 ||
      t_draft + t_verify <= 0.0)
    return ORC_EARG;
  int32_t best = 1;
  double best_rate = -1.0;
  for (int32_t K = 1; K <= k_max; K++) {
    const double rate = orc_expected_tokens(a, K) / (K * t_draft + t_verify);
    if (rate > best_rate) {
      best_rate = rate;
      best = K;
    }
  }
  return best;
}
