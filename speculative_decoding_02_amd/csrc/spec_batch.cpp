// spec_batch.cpp -- host side of the batched verify context (spec_batch_*).
//
// B sequences share one target: a pass carries R rows per sequence (K+1 for
// a verify, a prompt chunk for the prefill), M = B R activation rows in all,
// and streams every weight once for the whole batch through the rows GEMM.
// Per layer: norm_pack -> QKV GEMM -> qkv_post (RoPE, query fragments, KV
// append) -> batched attention -> O GEMM (+= residual) -> norm_pack ->
// gate/up GEMM -> silu_pack -> down GEMM (+= residual); then the final
// norm, the LM head, the row softmax and the rule for all B sequences in one
// launch pair.  GEMMs that split K leave their slices for the next kernel
// (norm_pack adds the residual GEMMs' slices to x, qkv_post sums QKV's).  The verify pass is captured as a hipGraph per (K, seed,
// pointers), as for a single sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "host_util.h"
#include "kernels.h"
#include "spec.h"

using namespace spec;
using spec_host::fmt;

namespace {

// one matrix packed for the rows GEMM (launch_pack layout, nb 1 or 2)
struct RMat {
  uint16_t* p = nullptr;
  int N = 0, K = 0, nb = 1;
};

struct BModel {
  int L = 0, d = 0, nq = 0, nkv = 0, hd = 0, F = 0, V = 0, qd = 0, kvd = 0;
  float theta = 10000.f, eps = 1e-5f;
  std::vector<RMat> qkv, o, gu, dn;
  RMat lm;
  uint16_t* arena = nullptr;
  uint16_t* embed = nullptr;
  uint16_t* norms = nullptr;  // attn [L][d], ffn [L][d], final [d]
  const uint16_t* attn_norm(int l) const { return norms + (size_t)l * d; }
  const uint16_t* ffn_norm(int l) const { return norms + (size_t)(L + l) * d; }
  const uint16_t* final_norm() const { return norms + (size_t)2 * L * d; }
};

}  // namespace

struct spec_batch {
  spec_batch_params p{};
  std::string err;
  hipStream_t stream = nullptr, cap_stream = nullptr;
  bool own_stream = false;
  int device = 0;
  int B = 0;
  BModel T;
  // per-sequence paged caches in one pool per layer: sequence b owns blocks
  // through its row of the block table
  int n_blocks = 0;       // blocks per sequence
  size_t kv_layer = 0;    // elements of one layer's key (= value) pool
  uint16_t *kcache = nullptr, *vcache = nullptr;
  int32_t* block_table = nullptr;  // [B][n_blocks]
  float2* rope = nullptr;
  // activations and workspaces (sized for kRowsMaxM rows)
  float *x = nullptr, *y = nullptr, *logits = nullptr, *Tbuf = nullptr;
  uint16_t* ap = nullptr;
  uint16_t* qf = nullptr;
  size_t qf_seq = 0;
  int max_chunks = 0;
  float* attn_wo = nullptr;
  float2* attn_ml = nullptr;
  float2* sm_part = nullptr;
  int sm_chunk = 0, sm_nchunks = 0;
  float* gemm_part = nullptr;  // split-K partials of the rows GEMM
  size_t gemm_part_elems = 0;
  uint64_t* ar_ws = nullptr;
  int ar_chunk = 0, ar_nchunks = 0;
  PassRows* rows = nullptr;
  uint64_t* pos_rule = nullptr;
  DevState* st = nullptr;
  int32_t* hist = nullptr;
  int hist_cap = 0;
  // host bookkeeping
  int LT_ub = 0;  // upper bound of every sequence's committed length
  bool verify_pending = false;
  int last_k = 0;
  bool graphs = true;
  std::map<std::vector<uint64_t>, hipGraphExec_t> graph_cache;
};

namespace {

int fail(spec_batch* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  spec_host::set_last_error(msg);
  return code;
}

#define BTRY(ctx, expr)                                                                         \
  do {                                                                                          \
    hipError_t e_ = (expr);                                                                     \
    if (e_ != hipSuccess)                                                                       \
      return fail(ctx, e_ == hipErrorOutOfMemory ? SPEC_ERR_OOM : SPEC_ERR_HIP,                 \
                  fmt("%s: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, __LINE__));     \
  } while (0)

template <typename T>
hipError_t dalloc(T** p, size_t n) {
  return hipMalloc((void**)p, std::max<size_t>(n, 1) * sizeof(T));
}

// the rows GEMM takes 16-column blocks in groups of nb = 2 when that divides
// a wide matrix, else 1
int rows_nb(int N) { return (N / 16 >= 384 && (N / 16) % 2 == 0) ? 2 : 1; }

int pack_mat(spec_batch* c, const std::vector<const uint16_t*>& rows, const RMat& m) {
  const uint16_t** drows = nullptr;
  BTRY(c, dalloc(&drows, rows.size()));
  hipError_t e = hipMemcpyAsync(drows, rows.data(), rows.size() * sizeof(void*),
                                hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = launch_pack(drows, m.K, m.nb, m.N / (16 * m.nb), 0, 0, m.p, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  (void)hipFree(drows);
  BTRY(c, e);
  return SPEC_OK;
}

// Packs the target for the rows GEMM.  QKV keeps its natural column order
// (q, k, v) and gate/up is [gate; up]: the kernels after each GEMM read
// plain rows.
int build_target(spec_batch* c, const spec_model_desc& md) {
  BModel& m = c->T;
  m.L = md.n_layers; m.d = md.d_model; m.nq = md.n_heads; m.nkv = md.n_kv_heads;
  m.hd = md.head_dim; m.F = md.d_ffn; m.V = md.vocab;
  m.qd = m.nq * m.hd; m.kvd = m.nkv * m.hd;
  m.theta = md.rope_theta; m.eps = md.rms_eps;
  const int L = m.L, d = m.d;
  auto mk = [](int N, int K) {
    RMat r;
    r.N = N; r.K = K; r.nb = rows_nb(N);
    return r;
  };
  m.qkv.assign(L, mk(m.qd + 2 * m.kvd, d));
  m.o.assign(L, mk(d, m.qd));
  m.gu.assign(L, mk(2 * m.F, d));
  m.dn.assign(L, mk(d, m.F));
  m.lm = mk(m.V, d);
  size_t total = (size_t)m.V * d;
  for (int l = 0; l < L; ++l)
    total += (size_t)(m.qd + 2 * m.kvd) * d + (size_t)d * m.qd + (size_t)2 * m.F * d +
             (size_t)d * m.F;
  BTRY(c, dalloc(&m.arena, total));
  size_t off = 0;
  auto place = [&](RMat& r) { r.p = m.arena + off; off += (size_t)r.N * r.K; };
  for (int l = 0; l < L; ++l) {
    place(m.qkv[l]); place(m.o[l]); place(m.gu[l]); place(m.dn[l]);
  }
  place(m.lm);
  const uint16_t* wq = (const uint16_t*)md.wq;
  const uint16_t* wk = (const uint16_t*)md.wk;
  const uint16_t* wv = (const uint16_t*)md.wv;
  const uint16_t* wo = (const uint16_t*)md.wo;
  const uint16_t* wg = (const uint16_t*)md.wg;
  const uint16_t* wu = (const uint16_t*)md.wu;
  const uint16_t* wdn = (const uint16_t*)md.wd;
  std::vector<const uint16_t*> rows;
  for (int l = 0; l < L; ++l) {
    rows.clear();
    for (int n = 0; n < m.qd; ++n) rows.push_back(wq + ((size_t)l * m.qd + n) * d);
    for (int n = 0; n < m.kvd; ++n) rows.push_back(wk + ((size_t)l * m.kvd + n) * d);
    for (int n = 0; n < m.kvd; ++n) rows.push_back(wv + ((size_t)l * m.kvd + n) * d);
    if (int r = pack_mat(c, rows, m.qkv[l])) return r;
    rows.clear();
    for (int n = 0; n < d; ++n) rows.push_back(wo + ((size_t)l * d + n) * m.qd);
    if (int r = pack_mat(c, rows, m.o[l])) return r;
    rows.clear();
    for (int n = 0; n < m.F; ++n) rows.push_back(wg + ((size_t)l * m.F + n) * d);
    for (int n = 0; n < m.F; ++n) rows.push_back(wu + ((size_t)l * m.F + n) * d);
    if (int r = pack_mat(c, rows, m.gu[l])) return r;
    rows.clear();
    for (int n = 0; n < d; ++n) rows.push_back(wdn + ((size_t)l * d + n) * m.F);
    if (int r = pack_mat(c, rows, m.dn[l])) return r;
  }
  rows.clear();
  for (int n = 0; n < m.V; ++n) rows.push_back((const uint16_t*)md.lm_head + (size_t)n * d);
  if (int r = pack_mat(c, rows, m.lm)) return r;
  BTRY(c, dalloc(&m.embed, (size_t)m.V * d));
  BTRY(c, hipMemcpyAsync(m.embed, md.embed, (size_t)m.V * d * 2, hipMemcpyDeviceToDevice, c->stream));
  BTRY(c, dalloc(&m.norms, (size_t)(2 * L + 1) * d));
  BTRY(c, hipMemcpyAsync(m.norms, md.attn_norm, (size_t)L * d * 2, hipMemcpyDeviceToDevice, c->stream));
  BTRY(c, hipMemcpyAsync(m.norms + (size_t)L * d, md.ffn_norm, (size_t)L * d * 2,
                         hipMemcpyDeviceToDevice, c->stream));
  BTRY(c, hipMemcpyAsync(m.norms + (size_t)2 * L * d, md.final_norm, (size_t)d * 2,
                         hipMemcpyDeviceToDevice, c->stream));
  BTRY(c, hipStreamSynchronize(c->stream));
  return SPEC_OK;
}

// With split != nullptr a split-K GEMM leaves its slices in gemm_part and
// *split says how many (0: Y holds the result); the next kernel sums them.
hipError_t gemm(spec_batch* c, const RMat& w, int M, float* Y, int ldy, int accumulate,
                hipStream_t s, int* split = nullptr) {
  RowsGemmArgs a{};
  a.Wp = w.p; a.N = w.N; a.K = w.K; a.nb = w.nb;
  a.X = nullptr; a.M = M; a.A = c->ap; a.Y = Y; a.ldy = ldy; a.accumulate = accumulate;
  a.P = c->gemm_part; a.P_elems = c->gemm_part_elems;
  a.defer_sum = split != nullptr; a.split_out = split;
  return launch_gemm_rows(a, s);
}

// RMSNorm of the residual rows into the packed operand; `split` slices of
// the residual GEMM before it are added to x first.
hipError_t norm_pack(spec_batch* c, int M, const uint16_t* gain, int split, hipStream_t s) {
  NormPackArgs a{};
  a.x = c->x; a.M = M; a.d = c->T.d; a.RT = rows_tiles(M); a.gain = gain; a.eps = c->T.eps;
  a.Ap = c->ap; a.P = c->gemm_part; a.S = split;
  return launch_norm_pack(a, s);
}

// One pass of R rows per sequence.  mode BEMB_VERIFY: rows [pending, drafts]
// at each sequence's length, then the LM head, softmax and rule; mode
// BEMB_PREFILL: prompt rows pos0..pos0+R-1 of every sequence, no head.
struct PassIO {
  int K = 0;
  uint64_t seed = 0;
  const int32_t* d = nullptr;
  const float* D = nullptr;
  int32_t* out = nullptr;
  int32_t* nacc = nullptr;
  float* Tb = nullptr;
  float* Lb = nullptr;
};

hipError_t enqueue_pass(spec_batch* c, hipStream_t s, int mode, int R, int pos0, const PassIO& io) {
  const BModel& m = c->T;
  const int B = c->B, M = B * R, RT = rows_tiles(M);
  BatchEmbedArgs em{};
  em.E = m.embed; em.d = m.d; em.vocab = m.V; em.max_seq = c->p.max_seq;
  em.st = c->st; em.hist = c->hist; em.hist_cap = c->hist_cap; em.dtok = io.d;
  em.mode = mode; em.B = B; em.R = R; em.pos0 = pos0;
  em.rows = c->rows; em.pos_rule = c->pos_rule; em.x = c->x;
  hipError_t e = launch_batch_embed(em, s);
  const int n_qkv = m.qd + 2 * m.kvd;
  int split = 0;  // slices of the last residual GEMM still to be added to x
  for (int l = 0; l < m.L && e == hipSuccess; ++l) {
    uint16_t* kc = c->kcache + (size_t)l * c->kv_layer;
    uint16_t* vc = c->vcache + (size_t)l * c->kv_layer;
    e = norm_pack(c, M, m.attn_norm(l), split, s);
    int qkv_split = 0;
    if (e == hipSuccess) e = gemm(c, m.qkv[l], M, c->y, n_qkv, 0, s, &qkv_split);
    if (e == hipSuccess) {
      QkvPostArgs q{};
      q.y = c->y; q.P = c->gemm_part; q.S = qkv_split;
      q.M = M; q.R = R; q.q_dim = m.qd; q.kv_dim = m.kvd; q.hd = m.hd; q.n_kv = m.nkv;
      q.max_seq = c->p.max_seq; q.rows = c->rows; q.rope = c->rope; q.qf = c->qf;
      q.qf_seq = c->qf_seq; q.k_cache = kc; q.v_cache = vc; q.block_table = c->block_table;
      q.n_blocks = c->n_blocks;
      e = launch_qkv_post(q, s);
    }
    if (e == hipSuccess) {
      AttnArgs at{};
      at.qf = c->qf; at.k_cache = kc; at.v_cache = vc; at.block_table = c->block_table;
      at.qf_bytes = (uint32_t)(c->qf_seq * 2); at.kv_layer_bytes = (uint32_t)(c->kv_layer * 2);
      at.rows = c->rows; at.n_q = m.nq; at.n_kv = m.nkv; at.hd = m.hd;
      at.max_chunks = c->max_chunks; at.n_blocks = c->n_blocks;
      at.ws_o = c->attn_wo; at.ws_ml = c->attn_ml;
      at.qg_max = (m.nq / m.nkv) * kMaxRows; at.Ap_out = c->ap;
      // one wave per chunk for both query tiles once the batch fills the chip
      // (measured: 11.55 -> 11.29 ms at B = 25; at B = 1 the halved wave count
      // is slower)
      at.n_seq = B; at.seq_rows = R; at.a_tiles = RT; at.qt_per_wave = B >= 4 ? 2 : 1;
      e = launch_attn(at, R, s);
    }
    if (e == hipSuccess) e = gemm(c, m.o[l], M, c->x, m.d, 1, s, &split);
    if (e == hipSuccess) e = norm_pack(c, M, m.ffn_norm(l), split, s);
    if (e == hipSuccess) e = gemm(c, m.gu[l], M, c->y, 2 * m.F, 0, s);
    if (e == hipSuccess) {
      SiluPackArgs sp{};
      sp.y = c->y; sp.M = M; sp.F = m.F; sp.RT = RT; sp.Ap = c->ap;
      e = launch_silu_pack(sp, s);
    }
    if (e == hipSuccess) e = gemm(c, m.dn[l], M, c->x, m.d, 1, s, &split);
  }
  // a prefill pass ends with the caches written (its residual is not needed)
  if (e != hipSuccess || mode != BEMB_VERIFY) return e;
  e = norm_pack(c, M, m.final_norm(), split, s);
  if (e == hipSuccess) e = gemm(c, m.lm, M, io.Lb, m.V, 0, s);
  if (e == hipSuccess) {
    RowSoftmaxArgs sm{};
    sm.logits = io.Lb; sm.M = M; sm.V = m.V; sm.chunk = c->sm_chunk; sm.n_chunks = c->sm_nchunks;
    sm.part = c->sm_part; sm.out = io.Tb;
    e = launch_row_softmax(sm, s);
  }
  if (e == hipSuccess) {
    ArArgs ar{};
    ar.T = io.Tb; ar.D = io.D; ar.d = io.d; ar.B = B; ar.K = io.K; ar.V = m.V;
    ar.seed = io.seed; ar.stream_id = c->p.stream_id; ar.pos = c->pos_rule; ar.st = nullptr;
    ar.pos_offset = 0; ar.greedy = c->p.greedy; ar.word = 2;
    ar.chunk = c->ar_chunk; ar.n_chunks = c->ar_nchunks;
    ar.out = io.out; ar.n_acc = io.nacc; ar.ws = c->ar_ws;
    e = launch_accept_reject(ar, s);
  }
  return e;
}

void destroy(spec_batch* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  for (auto& kv : c->graph_cache) (void)hipGraphExecDestroy(kv.second);
  c->graph_cache.clear();
  void* bufs[] = {c->T.arena, c->T.embed, c->T.norms, c->kcache, c->vcache, c->block_table,
                  c->rope, c->x, c->y, c->logits, c->Tbuf, c->ap, c->qf, c->attn_wo, c->attn_ml,
                  c->sm_part, c->gemm_part, c->ar_ws, c->rows, c->pos_rule, c->st, c->hist};
  for (void* b : bufs) (void)hipFree(b);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  if (c->own_stream && c->stream) (void)hipStreamDestroy(c->stream);
  delete c;
}

int init(spec_batch* c, const int32_t* prompts, int n_prompt) {
  const spec_batch_params& p = c->p;
  const int B = c->B;
  BTRY(c, hipGetDevice(&c->device));
  if (p.hip_stream) {
    c->stream = (hipStream_t)p.hip_stream;
  } else {
    BTRY(c, hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking));
    c->own_stream = true;
  }
  BTRY(c, hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
  if (int r = build_target(c, p.target)) return r;
  const BModel& m = c->T;
  // caches: B sequences x ceil(max_seq / 16) blocks; sequence b's logical
  // block i is physical block (b + 1) * n_blocks - 1 - i (any permutation works)
  c->n_blocks = (p.max_seq + kBlock - 1) / kBlock;
  c->kv_layer = (size_t)B * c->n_blocks * m.nkv * kBlock * 2 * m.hd;
  if (c->kv_layer * 2 >= (1ull << 31))
    return fail(c, SPEC_ERR_ARG, "one layer's KV pool must stay below 2 GiB (lower max_seq or n_seq)");
  BTRY(c, dalloc(&c->kcache, (size_t)m.L * c->kv_layer));
  BTRY(c, dalloc(&c->vcache, (size_t)m.L * c->kv_layer));
  // zero-filled: attention reads whole blocks and gives slots past the
  // length zero weight, which needs finite values there
  BTRY(c, hipMemsetAsync(c->kcache, 0, (size_t)m.L * c->kv_layer * 2, c->stream));
  BTRY(c, hipMemsetAsync(c->vcache, 0, (size_t)m.L * c->kv_layer * 2, c->stream));
  std::vector<int32_t> bt((size_t)B * c->n_blocks);
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < c->n_blocks; ++i) bt[(size_t)b * c->n_blocks + i] = (b + 1) * c->n_blocks - 1 - i;
  BTRY(c, dalloc(&c->block_table, bt.size()));
  BTRY(c, hipMemcpyAsync(c->block_table, bt.data(), bt.size() * 4, hipMemcpyHostToDevice, c->stream));
  BTRY(c, dalloc(&c->rope, (size_t)p.max_seq * (m.hd / 2)));
  BTRY(c, launch_rope_table(c->rope, p.max_seq, m.hd, (double)m.theta, c->stream));
  // activations
  const int Mmax = kRowsMaxM;
  const int kmax = std::max(std::max(m.d, m.qd), m.F);
  BTRY(c, dalloc(&c->x, (size_t)Mmax * m.d));
  BTRY(c, dalloc(&c->y, (size_t)Mmax * std::max(m.qd + 2 * m.kvd, 2 * m.F)));
  BTRY(c, dalloc(&c->ap, (size_t)(kmax / 32) * (Mmax / 8) * 64 * 8));
  // finite from the start: padding rows no producer writes are multiplied too
  // (their output rows are discarded)
  BTRY(c, hipMemsetAsync(c->ap, 0, (size_t)(kmax / 32) * (Mmax / 8) * 64 * 8 * 2, c->stream));
  size_t part = 0;
  for (const RMat* r : {&m.qkv[0], &m.o[0], &m.gu[0], &m.dn[0], &m.lm})
    part = std::max(part, rows_partials(Mmax, r->N, r->K));
  c->gemm_part_elems = part;
  BTRY(c, dalloc(&c->gemm_part, part));
  const size_t rows_out = (size_t)B * (p.k_max + 1) * m.V;
  BTRY(c, dalloc(&c->logits, rows_out));
  BTRY(c, dalloc(&c->Tbuf, rows_out));
  // attention: query fragments and chunk partials per sequence
  const int G = m.nq / m.nkv, n_es = (m.hd + 31) / 32, E16 = (m.hd + 15) / 16 * 16;
  c->qf_seq = (size_t)m.nkv * ((G + 1) / 2) * n_es * 2 * 64 * 8;
  BTRY(c, dalloc(&c->qf, (size_t)B * c->qf_seq));
  BTRY(c, hipMemsetAsync(c->qf, 0, (size_t)B * c->qf_seq * 2, c->stream));
  c->max_chunks = (p.max_seq + kAttnChunk - 1) / kAttnChunk;
  const size_t ws_ml = (size_t)B * m.nkv * c->max_chunks * G * kMaxRows;
  BTRY(c, dalloc(&c->attn_wo, ws_ml * E16));
  BTRY(c, dalloc(&c->attn_ml, ws_ml));
  // softmax: chunks of >= 2048 columns, at most 256 per row
  c->sm_chunk = std::max(2048, ((m.V + 255) / 256 + 255) / 256 * 256);
  c->sm_nchunks = (m.V + c->sm_chunk - 1) / c->sm_chunk;
  BTRY(c, dalloc(&c->sm_part, (size_t)Mmax * c->sm_nchunks));
  ar_choose_chunks(B, m.V, &c->ar_chunk, &c->ar_nchunks);
  BTRY(c, dalloc(&c->ar_ws, (size_t)B * c->ar_nchunks * ar_ws_words(p.k_max)));
  BTRY(c, dalloc(&c->rows, (size_t)B));
  BTRY(c, dalloc(&c->pos_rule, (size_t)B));
  // state and histories
  c->hist_cap = p.max_seq + p.k_max + 2;
  BTRY(c, dalloc(&c->hist, (size_t)B * c->hist_cap));
  BTRY(c, hipMemsetAsync(c->hist, 0, (size_t)B * c->hist_cap * 4, c->stream));
  std::vector<int32_t> h((size_t)B * c->hist_cap, 0);
  for (int b = 0; b < B; ++b)
    std::copy(prompts + (size_t)b * n_prompt, prompts + (size_t)(b + 1) * n_prompt,
              h.begin() + (size_t)b * c->hist_cap);
  BTRY(c, hipMemcpyAsync(c->hist, h.data(), h.size() * 4, hipMemcpyHostToDevice, c->stream));
  std::vector<DevState> hs(B);
  for (auto& s : hs) {
    s = DevState{};
    s.LT = s.LD = 0;
  }
  BTRY(c, dalloc(&c->st, (size_t)B));
  BTRY(c, hipMemcpyAsync(c->st, hs.data(), B * sizeof(DevState), hipMemcpyHostToDevice, c->stream));
  // prefill prompt[0..n-2] of every sequence, R rows per sequence per pass
  const int Rp = std::min(kMaxRows, kRowsMaxM / B);
  for (int p0 = 0; p0 < n_prompt - 1; p0 += Rp) {
    const int R = std::min(Rp, n_prompt - 1 - p0);
    BTRY(c, enqueue_pass(c, c->stream, BEMB_PREFILL, R, p0, PassIO{}));
  }
  for (auto& s : hs) s.LT = s.LD = n_prompt - 1;
  BTRY(c, hipMemcpyAsync(c->st, hs.data(), B * sizeof(DevState), hipMemcpyHostToDevice, c->stream));
  BTRY(c, hipStreamSynchronize(c->stream));
  c->LT_ub = n_prompt - 1;
  return SPEC_OK;
}

int read_state(spec_batch* c, std::vector<DevState>* hs) {
  hs->resize(c->B);
  BTRY(c, hipStreamSynchronize(c->stream));
  BTRY(c, hipMemcpy(hs->data(), c->st, c->B * sizeof(DevState), hipMemcpyDeviceToHost));
  return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_batch_init(const spec_batch_params* p, const int32_t* prompts_host, int32_t n_prompt,
                    spec_batch** out) {
  if (!out) return fail(nullptr, SPEC_ERR_ARG, "spec_batch_init: null output");
  *out = nullptr;
  if (!p || !prompts_host) return fail(nullptr, SPEC_ERR_ARG, "spec_batch_init: null argument");
  std::string why;
  if (!spec_host::valid_model(p->target, &why))
    return fail(nullptr, SPEC_ERR_ARG, "spec_batch_init: target: " + why);
  if (p->target.d_model > kNormPackMaxD)
    return fail(nullptr, SPEC_ERR_ARG, fmt("spec_batch_init: d_model above %d", kNormPackMaxD));
  const int B = p->n_seq;
  if (B < 1 || B > SPEC_BATCH_MAX_SEQ)
    return fail(nullptr, SPEC_ERR_ARG, fmt("spec_batch_init: n_seq=%d outside 1..%d", B, SPEC_BATCH_MAX_SEQ));
  if (p->k_max < 1 || p->k_max > SPEC_K_MAX || B * (p->k_max + 1) > kRowsMaxM)
    return fail(nullptr, SPEC_ERR_ARG,
                fmt("spec_batch_init: k_max=%d with n_seq=%d (need 1..%d and n_seq*(k_max+1) <= %d)",
                    p->k_max, B, SPEC_K_MAX, kRowsMaxM));
  if (n_prompt < 1) return fail(nullptr, SPEC_ERR_ARG, "spec_batch_init: n_prompt < 1");
  if (p->max_seq < n_prompt + p->k_max + 1 || p->max_seq > (1 << 24))
    return fail(nullptr, SPEC_ERR_CAPACITY, "spec_batch_init: max_seq < n_prompt + k_max + 1");
  for (size_t i = 0; i < (size_t)B * n_prompt; ++i)
    if (prompts_host[i] < 0 || prompts_host[i] >= p->target.vocab)
      return fail(nullptr, SPEC_ERR_ARG, fmt("spec_batch_init: token id %d out of range", prompts_host[i]));
  spec_batch* c = new spec_batch();
  c->p = *p;
  c->B = B;
  c->graphs = p->use_graphs != 0;
  if (int r = init(c, prompts_host, n_prompt)) {
    const std::string msg = c->err;
    destroy(c);
    spec_host::set_last_error(msg);
    return r;
  }
  *out = c;
  return SPEC_OK;
}

int spec_batch_draft_ngram(spec_batch* c, int32_t K, int32_t n_max, int32_t* d_dev, float* D_dev) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_batch_draft_ngram: null context");
  if (K < 1 || K > c->p.k_max) return fail(c, SPEC_ERR_ARG, fmt("K=%d outside 1..k_max", K));
  if (n_max < 1 || n_max > kNgramMaxN)
    return fail(c, SPEC_ERR_ARG, fmt("n_max=%d outside 1..%d", n_max, kNgramMaxN));
  if (!d_dev || (!D_dev && !c->p.greedy))
    return fail(c, SPEC_ERR_ARG, "spec_batch_draft_ngram: null output");
  if (c->verify_pending) return fail(c, SPEC_ERR_STATE, "a verify is pending: commit it first");
  BTRY(c, hipSetDevice(c->device));
  NgramArgs a{};
  a.st = c->st; a.hist = c->hist; a.hist_cap = c->hist_cap;
  a.K = K; a.n_max = n_max; a.V = c->T.V; a.d = d_dev; a.D = D_dev; a.B = c->B;
  BTRY(c, launch_ngram_draft(a, c->stream));
  return SPEC_OK;
}

int spec_batch_verify(spec_batch* c, int32_t K, uint64_t seed, const int32_t* d_dev,
                      const float* D_dev, int32_t* out_dev, int32_t* n_acc_dev, float* T_dev,
                      float* logits_dev) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_batch_verify: null context");
  if (K < 1 || K > c->p.k_max) return fail(c, SPEC_ERR_ARG, fmt("K=%d outside 1..k_max", K));
  if (!d_dev || !out_dev || !n_acc_dev || (!D_dev && !c->p.greedy))
    return fail(c, SPEC_ERR_ARG, "spec_batch_verify: null pointer");
  if (c->verify_pending) return fail(c, SPEC_ERR_STATE, "a verify is pending: commit it first");
  BTRY(c, hipSetDevice(c->device));
  if (c->LT_ub + K >= c->p.max_seq) {
    std::vector<DevState> hs;
    if (int r = read_state(c, &hs)) return r;
    int ub = 0;
    for (const DevState& s : hs) ub = std::max(ub, s.LT);
    c->LT_ub = ub;
    if (ub + K >= c->p.max_seq)
      return fail(c, SPEC_ERR_CAPACITY, "a sequence's positions would exceed max_seq");
  }
  PassIO io;
  io.K = K; io.seed = seed; io.d = d_dev; io.D = D_dev; io.out = out_dev; io.nacc = n_acc_dev;
  io.Tb = T_dev ? T_dev : c->Tbuf;
  io.Lb = logits_dev ? logits_dev : c->logits;
  auto body = [&](hipStream_t s) { return enqueue_pass(c, s, BEMB_VERIFY, K + 1, 0, io); };
  if (!c->graphs) {
    BTRY(c, body(c->stream));
  } else {
    const std::vector<uint64_t> key = {(uint64_t)K, seed, (uint64_t)(uintptr_t)d_dev,
                                       (uint64_t)(uintptr_t)D_dev, (uint64_t)(uintptr_t)out_dev,
                                       (uint64_t)(uintptr_t)n_acc_dev, (uint64_t)(uintptr_t)io.Tb,
                                       (uint64_t)(uintptr_t)io.Lb};
    auto it = c->graph_cache.find(key);
    if (it == c->graph_cache.end()) {
      hipGraphExec_t exec = nullptr;
      BTRY(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeRelaxed));
      hipError_t e = body(c->cap_stream);
      hipGraph_t g = nullptr;
      const hipError_t e2 = hipStreamEndCapture(c->cap_stream, &g);
      if (e == hipSuccess) e = e2;
      if (e == hipSuccess) e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
      if (g) (void)hipGraphDestroy(g);
      BTRY(c, e);
      it = c->graph_cache.emplace(key, exec).first;
    }
    BTRY(c, hipGraphLaunch(it->second, c->stream));
  }
  c->verify_pending = true;
  c->last_k = K;
  return SPEC_OK;
}

int spec_batch_commit(spec_batch* c, const int32_t* out_dev, const int32_t* n_acc_dev) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_batch_commit: null context");
  if (!out_dev || !n_acc_dev) return fail(c, SPEC_ERR_ARG, "spec_batch_commit: null pointer");
  if (!c->verify_pending) return fail(c, SPEC_ERR_STATE, "no verify to commit");
  BTRY(c, hipSetDevice(c->device));
  BatchCommitArgs a{};
  a.st = c->st; a.hist = c->hist; a.hist_cap = c->hist_cap; a.out = out_dev; a.n_acc = n_acc_dev;
  a.B = c->B; a.K = c->last_k;
  BTRY(c, launch_batch_commit(a, c->stream));
  c->verify_pending = false;
  c->LT_ub += c->last_k + 1;
  return SPEC_OK;
}

int spec_batch_sync(spec_batch* c) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_batch_sync: null context");
  BTRY(c, hipSetDevice(c->device));
  BTRY(c, hipStreamSynchronize(c->stream));
  return SPEC_OK;
}

int spec_batch_get_state(spec_batch* c, int32_t* len_host, int32_t* err_host) {
  if (!c || !len_host) return fail(c, SPEC_ERR_ARG, "spec_batch_get_state: null argument");
  BTRY(c, hipSetDevice(c->device));
  std::vector<DevState> hs;
  if (int r = read_state(c, &hs)) return r;
  for (int b = 0; b < c->B; ++b) {
    len_host[b] = hs[b].LT;
    if (err_host) err_host[b] = hs[b].err;
  }
  return SPEC_OK;
}

int spec_batch_get_history(spec_batch* c, int32_t b, int32_t* host_out, int32_t n) {
  if (!c || !host_out) return fail(c, SPEC_ERR_ARG, "spec_batch_get_history: null argument");
  if (b < 0 || b >= c->B || n < 0 || n > c->hist_cap)
    return fail(c, SPEC_ERR_ARG, "spec_batch_get_history: sequence or length out of range");
  BTRY(c, hipSetDevice(c->device));
  BTRY(c, hipStreamSynchronize(c->stream));
  BTRY(c, hipMemcpy(host_out, c->hist + (size_t)b * c->hist_cap, (size_t)n * 4, hipMemcpyDeviceToHost));
  return SPEC_OK;
}

const char* spec_batch_last_error(const spec_batch* c) {
  return c ? c->err.c_str() : spec_last_error(nullptr);
}

int spec_batch_destroy(spec_batch* c) {
  destroy(c);
  return SPEC_OK;
}

}  // extern "C"
