// spec_api.cpp -- host side of libspec: the C ABI declared in include/spec.h.
//
// A context owns two models (target, draft) with repacked weights, one paged
// KV cache per model, shared activation/workspace buffers, the device-side
// decoding state and the captured graphs.  Every step of the path runs in
// the HIP kernels; this file validates arguments, lays out memory, and
// enqueues launches (directly or through hipGraphs).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "host_util.h"
#include "kernels.h"
#include "spec.h"

using namespace spec;

namespace {
thread_local std::string g_err;
}  // namespace

namespace spec_host {

std::string fmt(const char* f, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

void set_last_error(const std::string& msg) { g_err = msg; }

bool valid_model(const spec_model_desc& m, std::string* why) {
  if (m.n_layers < 1 || m.d_model < 64 || m.n_heads < 1 || m.n_kv_heads < 1 || m.head_dim < 2 ||
      m.d_ffn < 32 || m.vocab < 16) {
    *why = "non-positive or too small dimension";
    return false;
  }
  if (m.d_model % 64 || m.d_ffn % 32 || m.vocab % 16 || m.head_dim % 2) {
    *why = "need d_model % 64 == 0, d_ffn % 32 == 0, vocab % 16 == 0, even head_dim";
    return false;
  }
  if (m.n_heads % m.n_kv_heads) {
    *why = "n_heads must be a multiple of n_kv_heads";
    return false;
  }
  if ((m.n_heads * m.head_dim / 2) % 8 || (m.n_kv_heads * m.head_dim / 2) % 8) {
    *why = "n_heads*head_dim/2 and n_kv_heads*head_dim/2 must be multiples of 8";
    return false;
  }
  if (m.head_dim > 256 || (m.n_heads / m.n_kv_heads) * kMaxRows > 64 || m.head_dim % 8) {
    *why = "head_dim must be a multiple of 8 and <= 256; n_heads/n_kv_heads <= 8";
    return false;
  }
  if ((m.n_heads * m.head_dim) % 32) {
    *why = "n_heads*head_dim must be a multiple of 32";
    return false;
  }
  if (!m.embed || !m.attn_norm || !m.wq || !m.wk || !m.wv || !m.wo || !m.ffn_norm || !m.wg ||
      !m.wu || !m.wd || !m.final_norm || !m.lm_head) {
    *why = "null weight pointer";
    return false;
  }
  if (!(m.rms_eps >= 0.0f) || !(m.rope_theta > 0.0f)) {
    *why = "rms_eps must be >= 0 and rope_theta > 0";
    return false;
  }
  return true;
}

}  // namespace spec_host

namespace {

using spec_host::fmt;
using spec_host::valid_model;

struct Mat {
  uint16_t* p = nullptr;  // packed (inside the model arena)
  GemmPlan plan;
  int K = 0, N = 0;
  size_t elems() const { return plan.packed_elems(); }
};

struct Model {
  int L = 0, d = 0, nq = 0, nkv = 0, hd = 0, F = 0, V = 0, qd = 0, kvd = 0;
  float theta = 10000.f, eps = 1e-5f;
  std::vector<Mat> qkv, o, gu, dn;
  Mat lm;
  bool lm_shared = false, embed_shared = false;
  uint16_t* arena = nullptr;      // packed matrices
  uint16_t* embed = nullptr;      // [V][d] (owned unless shared)
  uint16_t* norms = nullptr;      // attn [L][d], ffn [L][d], final [d]
  uint16_t* kcache = nullptr;     // [L][n_blocks][nkv][16][2 (hi, lo)][hd] bf16
  uint16_t* vcache = nullptr;
  int32_t* block_table = nullptr;
  float2* rope = nullptr;  // [max_seq][hd/2] (cos, sin)
  int n_blocks = 0;
  size_t kv_layer_elems() const { return (size_t)n_blocks * nkv * kBlock * 2 * hd; }
  const uint16_t* attn_norm(int l) const { return norms + (size_t)l * d; }
  const uint16_t* ffn_norm(int l) const { return norms + (size_t)(L + l) * d; }
  const uint16_t* final_norm() const { return norms + (size_t)2 * L * d; }
};

// First element of a graph-cache key: the kind of pass captured.
constexpr uint64_t kPassDraft = 1, kPassVerify = 2, kPassNgram = 3, kPassHeads = 4;

struct GraphEntry {
  hipGraphExec_t exec = nullptr;
};

}  // namespace

struct spec_ctx {
  spec_init_params p{};
  std::string err;
  hipStream_t stream = nullptr, cap_stream = nullptr;
  bool own_stream = false;
  int device = 0;
  Model T, D;
  // shared buffers (sized for the larger of the two models)
  float *x = nullptr, *ssq_a = nullptr, *ssq_b = nullptr;
  uint16_t* qf = nullptr;  // attention query fragments
  size_t qf_elems = 0;
  uint16_t *ap_x = nullptr, *ap_o = nullptr, *ap_a = nullptr;  // packed A operands
  float *logits = nullptr, *Tbuf = nullptr;
  float* attn_wo = nullptr;   // attention chunk partials: value sums
  float2* attn_ml = nullptr;  // attention chunk partials: (max, sum of exp)
  float2* lm_part = nullptr;
  uint64_t* ar_ws = nullptr;
  PassRows* rows = nullptr;
  DevState* st = nullptr;
  // multi-token-prediction heads (spec_heads_init): the stacked [n_heads*d][d]
  // matrices packed like any weight, and the state they draft from: the
  // target's final residual at the last committed position, kept by the
  // prompt prefill and by every commit
  Mat heads;
  uint16_t* heads_arena = nullptr;
  int n_heads = 0;
  float* h_last = nullptr;   // [T.d]
  float* hn = nullptr;       // [T.d] its normed form (heads pass)
  float* head_y = nullptr;   // [n_heads][T.d] head products
  bool h_valid = false;
  int32_t* hist = nullptr;
  int hist_cap = 0;
  int attn_max_chunks = 0;
  int ar_chunk = 0, ar_nchunks = 0;
  int sm_chunk = 0, sm_nchunks = 0;
  // host bookkeeping
  int LT_ub = 0, lag_ub = 0;
  int drafted_k = 0;
  bool verify_pending = false;
  int last_k = 0;
  bool graphs = true;
  std::map<std::vector<uint64_t>, GraphEntry> graph_cache;
  // profiling: each feed-forward gate/up GEMM and the O projection launched
  // just before it write per-workgroup end stamps (device wall clock) into
  // slot i of ts: [i][0][g] for the O projection, [i][1][g] for gate/up.  The
  // gate/up launch's duration is the latest gate/up end minus the latest O
  // end, i.e. its slice of the back-to-back stream, launch overhead
  // included.  Draft launches use slots [0, k_max * draft layers), verify
  // launches the target-layer slots after them.  Graphs are captured
  // separately with profiling on (the kernels are the same).
  bool profiling = false;
  unsigned long long* ts = nullptr;
  int ts_cap = 0;
  int ts_groups = 0;            // workgroups per stamp row (largest O / gate/up grid)
  int ts_next = 0;              // next slot while enqueueing a pass
  int prof_draft_n = 0, prof_verify_n = 0;  // slots written by the last calls
  // the verify pass's LM head: end stamps of the last layer's down GEMM
  // ([0][g]) and of the LM head ([1][g]); its duration is the latest LM-head
  // end minus the latest down end (same convention as the gate/up slots)
  unsigned long long* ts_head = nullptr;
  int ts_head_groups = 0;
  bool head_stamped = false;
  int wall_khz = 0;             // wall-clock counter rate
};

namespace {

int fail(spec_ctx* c, int code, const std::string& msg) {
  if (c) c->err = msg;
  g_err = msg;
  return code;
}

#define HIPTRY(ctx, expr)                                                                       \
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

// Packs one matrix from row pointers (host list, in the column order the
// epilogues number columns in, null past N) into m.p.  Column slices take the
// columns (or, for epilogues on column pairs, the pairs: columns w, w + 8 of a
// 16-column block) in consecutive runs, one per workgroup.
int pack_rows(spec_ctx* c, const std::vector<const uint16_t*>& virt, const Mat& m,
              bool paired = false) {
  const GemmPlan& pl = m.plan;
  const int nb = pl.shape.nb, cw = pl.shape.slice;
  const size_t n_slots = (size_t)pl.n_groups * nb * 16;
  std::vector<const uint16_t*> rows;
  if (!cw) {
    if (virt.size() != n_slots)
      return fail(c, SPEC_ERR_ARG, "internal: row list does not match the packing plan");
    rows = virt;
  } else {
    rows.assign(n_slots, nullptr);
    for (int g = 0; g < pl.n_groups; ++g)
      for (int j = 0; j < nb; ++j)
        for (int w = 0; w < 16; ++w) {
          size_t vc;
          if (paired) {
            const int lp = j * 8 + (w & 7);
            if (lp >= cw / 2) continue;
            const size_t P = (size_t)g * (cw / 2) + lp;
            vc = P / 8 * 16 + P % 8 + 8 * (w >> 3);
          } else {
            const int cc = j * 16 + w;
            if (cc >= cw) continue;
            vc = (size_t)g * cw + cc;
          }
          if (vc >= virt.size())
            return fail(c, SPEC_ERR_ARG, "internal: row list does not cover the column slices");
          rows[((size_t)g * nb + j) * 16 + w] = virt[vc];
        }
  }
  const uint16_t** drows = nullptr;
  HIPTRY(c, dalloc(&drows, rows.size()));
  hipError_t e = hipMemcpyAsync(drows, rows.data(), rows.size() * sizeof(void*),
                                hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess)
    e = launch_pack(drows, m.K, nb, pl.n_groups, cw, paired ? 1 : 0, m.p, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  (void)hipFree(drows);
  HIPTRY(c, e);
  return SPEC_OK;
}

int build_model(spec_ctx* c, const spec_model_desc& md, Model& m, const Model* share_from,
                const spec_model_desc* share_desc) {
  m.L = md.n_layers; m.d = md.d_model; m.nq = md.n_heads; m.nkv = md.n_kv_heads;
  m.hd = md.head_dim; m.F = md.d_ffn; m.V = md.vocab;
  m.qd = m.nq * m.hd; m.kvd = m.nkv * m.hd;
  m.theta = md.rope_theta; m.eps = md.rms_eps;
  const int L = m.L, d = m.d;
  int n_cu = 0;
  HIPTRY(c, hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, c->device));
  // half blocks only where the epilogue keeps each column on its own (O,
  // down); column slices by column there and by column pair for QKV and
  // gate/up; neither for the LM head
  auto mk = [n_cu](int N, int K, bool allow_half, int slice_kind) {
    Mat x;
    x.N = N; x.K = K;
    x.plan = plan_gemm(N, 1, K, n_cu, allow_half, slice_kind);
    return x;
  };
  m.qkv.assign(L, mk(m.qd + 2 * m.kvd, d, false, kSlicePairs));
  m.o.assign(L, mk(d, m.qd, true, kSliceCols));
  m.gu.assign(L, mk(2 * m.F, d, false, kSlicePairs));
  m.dn.assign(L, mk(d, m.F, true, kSliceCols));
  m.lm = mk(m.V, d, false, kSliceNone);
  m.lm_shared = share_from && share_desc && md.lm_head == share_desc->lm_head &&
                md.d_model == share_desc->d_model && md.vocab == share_desc->vocab;
  m.embed_shared = share_from && share_desc && md.embed == share_desc->embed &&
                   md.d_model == share_desc->d_model && md.vocab == share_desc->vocab;
  size_t total = 0;
  for (int l = 0; l < L; ++l)
    total += m.qkv[l].elems() + m.o[l].elems() + m.gu[l].elems() + m.dn[l].elems();
  if (!m.lm_shared) total += m.lm.elems();
  HIPTRY(c, dalloc(&m.arena, total));
  size_t off = 0;
  auto place = [&](Mat& x) { x.p = m.arena + off; off += x.elems(); };
  for (int l = 0; l < L; ++l) {
    place(m.qkv[l]); place(m.o[l]); place(m.gu[l]); place(m.dn[l]);
  }
  if (m.lm_shared) m.lm.p = share_from->lm.p;
  else place(m.lm);

  const uint16_t* wq = (const uint16_t*)md.wq;
  const uint16_t* wk = (const uint16_t*)md.wk;
  const uint16_t* wv = (const uint16_t*)md.wv;
  const uint16_t* wo = (const uint16_t*)md.wo;
  const uint16_t* wg = (const uint16_t*)md.wg;
  const uint16_t* wu = (const uint16_t*)md.wu;
  const uint16_t* wdn = (const uint16_t*)md.wd;
  const int half = m.hd / 2;
  std::vector<const uint16_t*> rows;
  for (int l = 0; l < L; ++l) {
    // QKV: q and k rows in pair-interleaved order (columns w, w+8 of a block
    // are the halves j, j+hd/2 of one RoPE pair), then v rows in order.
    auto slots = [](const Mat& x) {
      return x.plan.shape.slice ? (size_t)x.N : (size_t)x.plan.n_groups * x.plan.shape.nb * 16;
    };
    rows.assign(slots(m.qkv[l]), nullptr);
    for (int p = 0; p < m.qd + 2 * m.kvd; ++p) {
      const uint16_t* src;
      if (p < m.qd + m.kvd) {
        const bool is_q = p < m.qd;
        const int pl = is_q ? p : p - m.qd;
        const int b = pl / 16, w = pl % 16;
        const int pair = b * 8 + (w & 7), hf = w >> 3;
        const int head = pair / half, jj = pair % half;
        const int row = head * m.hd + jj + hf * half;
        src = is_q ? wq + ((size_t)l * m.qd + row) * d : wk + ((size_t)l * m.kvd + row) * d;
      } else {
        src = wv + ((size_t)l * m.kvd + (p - m.qd - m.kvd)) * d;
      }
      rows[p] = src;
    }
    if (int r = pack_rows(c, rows, m.qkv[l], true)) return r;
    rows.assign(slots(m.o[l]), nullptr);
    for (int n = 0; n < d; ++n) rows[n] = wo + ((size_t)l * d + n) * m.qd;
    if (int r = pack_rows(c, rows, m.o[l])) return r;
    // gate/up: 16-column block b holds the gate rows of features 8b..8b+7
    // in its columns 0-7 and the up rows of the same features in 8-15
    rows.assign(slots(m.gu[l]), nullptr);
    for (int n = 0; n < 2 * m.F; ++n) {
      const size_t f = (size_t)(n / 16) * 8 + (n % 8);
      rows[n] = ((n % 16) < 8 ? wg : wu) + ((size_t)l * m.F + f) * d;
    }
    if (int r = pack_rows(c, rows, m.gu[l], true)) return r;
    rows.assign(slots(m.dn[l]), nullptr);
    for (int n = 0; n < d; ++n) rows[n] = wdn + ((size_t)l * d + n) * m.F;
    if (int r = pack_rows(c, rows, m.dn[l])) return r;
  }
  if (!m.lm_shared) {
    rows.assign((size_t)m.lm.plan.n_groups * m.lm.plan.shape.nb * 16, nullptr);
    const uint16_t* lm = (const uint16_t*)md.lm_head;
    for (int n = 0; n < m.V; ++n) rows[n] = lm + (size_t)n * d;
    if (int r = pack_rows(c, rows, m.lm)) return r;
  }
  // embedding and norm gains (owned copies)
  if (m.embed_shared) {
    m.embed = share_from->embed;
  } else {
    HIPTRY(c, dalloc(&m.embed, (size_t)m.V * d));
    HIPTRY(c, hipMemcpyAsync(m.embed, md.embed, (size_t)m.V * d * 2, hipMemcpyDeviceToDevice,
                             c->stream));
  }
  HIPTRY(c, dalloc(&m.norms, (size_t)(2 * L + 1) * d));
  HIPTRY(c, hipMemcpyAsync(m.norms, md.attn_norm, (size_t)L * d * 2, hipMemcpyDeviceToDevice, c->stream));
  HIPTRY(c, hipMemcpyAsync(m.norms + (size_t)L * d, md.ffn_norm, (size_t)L * d * 2,
                           hipMemcpyDeviceToDevice, c->stream));
  HIPTRY(c, hipMemcpyAsync(m.norms + (size_t)2 * L * d, md.final_norm, (size_t)d * 2,
                           hipMemcpyDeviceToDevice, c->stream));
  // paged KV cache: blocks of 16 tokens; the block table maps logical block i
  // to physical block n_blocks-1-i (any permutation works).
  m.n_blocks = (c->p.max_seq + kBlock - 1) / kBlock;
  if (m.kv_layer_elems() * 2 >= (1ull << 31))
    return fail(c, SPEC_ERR_ARG, "one layer's KV cache must stay below 2 GiB (lower max_seq)");
  HIPTRY(c, dalloc(&m.kcache, (size_t)L * m.kv_layer_elems()));
  HIPTRY(c, dalloc(&m.vcache, (size_t)L * m.kv_layer_elems()));
  // zero-filled: attention reads whole blocks and relies on finite values in
  // slots it gives zero weight
  HIPTRY(c, hipMemsetAsync(m.kcache, 0, (size_t)L * m.kv_layer_elems() * 2, c->stream));
  HIPTRY(c, hipMemsetAsync(m.vcache, 0, (size_t)L * m.kv_layer_elems() * 2, c->stream));
  std::vector<int32_t> bt(m.n_blocks);
  for (int i = 0; i < m.n_blocks; ++i) bt[i] = m.n_blocks - 1 - i;
  HIPTRY(c, dalloc(&m.block_table, (size_t)m.n_blocks));
  HIPTRY(c, hipMemcpyAsync(m.block_table, bt.data(), bt.size() * 4, hipMemcpyHostToDevice, c->stream));
  HIPTRY(c, dalloc(&m.rope, (size_t)c->p.max_seq * half));
  HIPTRY(c, launch_rope_table(m.rope, c->p.max_seq, m.hd, (double)m.theta, c->stream));
  HIPTRY(c, hipStreamSynchronize(c->stream));
  return SPEC_OK;
}

void free_model(Model& m) {
  (void)hipFree(m.arena);
  if (!m.embed_shared) (void)hipFree(m.embed);
  (void)hipFree(m.norms);
  (void)hipFree(m.kcache);
  (void)hipFree(m.vcache);
  (void)hipFree(m.block_table);
  (void)hipFree(m.rope);
  m = Model();
}

// ------------------------------------------------------------ enqueuing --
GemmArgs gemm_base(spec_ctx* c, const Mat& w, const uint16_t* ap) {
  GemmArgs a{};
  a.Wp = w.p;
  a.n_groups = w.plan.n_groups;
  a.slice_cols = w.plan.shape.slice;
  a.Kb = w.plan.Kb;
  a.K = w.K;
  a.Ap = ap;
  a.rows = c->rows;
  return a;
}

// Per layer: QKV (norm scale, RoPE, KV append) -> attention -> O (+residual)
// -> gate/up (norm scale, SiLU*up) -> down (+residual).  The sums of squares
// for each RMSNorm alternate between two buffers so a producer never writes
// the partials its own consumer-to-be is still to read.  fixed_rows: the
// pass's row count when it is known as the launches are recorded (0: the
// kernels read it from the pass descriptor).
hipError_t enqueue_layers(spec_ctx* c, const Model& m, hipStream_t s, int n_rows, int fixed_rows,
                          bool profile, bool stamp_last_down = false) {
  hipError_t e = hipSuccess;
  int ssq_groups = m.d / 64;  // produced by the embedding
  float* ssq_in = c->ssq_a;
  float* ssq_other = c->ssq_b;
  for (int l = 0; l < m.L && e == hipSuccess; ++l) {
    // RMSNorm + QKV + RoPE + KV append
    GemmArgs a = gemm_base(c, m.qkv[l], c->ap_x);
    a.fixed_rows = fixed_rows;
    a.ssq = ssq_in; a.ssq_groups = ssq_groups; a.eps = m.eps;
    a.qf = c->qf;
    a.q_dim = m.qd; a.kv_dim = m.kvd; a.head_dim = m.hd; a.n_kv = m.nkv;
    a.k_cache = m.kcache + (size_t)l * m.kv_layer_elems();
    a.v_cache = m.vcache + (size_t)l * m.kv_layer_elems();
    a.block_table = m.block_table; a.rope = m.rope; a.max_seq = c->p.max_seq;
    e = launch_gemm(m.qkv[l].plan.shape, EPI_QKV, a, s);
    if (e != hipSuccess) break;
    // causal attention over the paged cache -> packed A of the O projection
    AttnArgs at{};
    at.qf = c->qf; at.k_cache = a.k_cache; at.v_cache = a.v_cache; at.block_table = m.block_table;
    at.qf_bytes = (uint32_t)(c->qf_elems * 2); at.kv_layer_bytes = (uint32_t)(m.kv_layer_elems() * 2);
    at.rows = c->rows; at.n_q = m.nq; at.n_kv = m.nkv; at.hd = m.hd;
    at.max_chunks = c->attn_max_chunks; at.n_blocks = m.n_blocks;
    at.ws_o = c->attn_wo; at.ws_ml = c->attn_ml;
    at.qg_max = (m.nq / m.nkv) * kMaxRows; at.Ap_out = c->ap_o;
    e = launch_attn(at, n_rows, s);
    if (e != hipSuccess) break;
    // O projection + residual; packs x * ffn_norm for gate/up
    GemmArgs b = gemm_base(c, m.o[l], c->ap_o);
    b.fixed_rows = fixed_rows;
    b.resid = c->x; b.ldr = m.d; b.gain_next = m.ffn_norm(l); b.Ap_out = c->ap_x;
    b.ssq_out = ssq_other;
    const bool stamp = profile && c->ts_next < c->ts_cap;
    if (stamp) b.ts_end = c->ts + (size_t)c->ts_next * 2 * c->ts_groups;
    e = launch_gemm(m.o[l].plan.shape, EPI_RESID, b, s);
    if (e != hipSuccess) break;
    std::swap(ssq_in, ssq_other);
    ssq_groups = m.o[l].plan.workgroups();
    // RMSNorm + gate/up + SiLU*mul -> packed A of the down projection
    GemmArgs g = gemm_base(c, m.gu[l], c->ap_x);
    g.fixed_rows = fixed_rows;
    g.ssq = ssq_in; g.ssq_groups = ssq_groups; g.eps = m.eps; g.Ap_out = c->ap_a;
    if (stamp) g.ts_end = c->ts + ((size_t)c->ts_next++ * 2 + 1) * c->ts_groups;
    e = launch_gemm(m.gu[l].plan.shape, EPI_SILU, g, s);
    if (e != hipSuccess) break;
    // down projection + residual; packs x * (next attn_norm or final norm)
    GemmArgs dn = gemm_base(c, m.dn[l], c->ap_a);
    dn.fixed_rows = fixed_rows;
    dn.resid = c->x; dn.ldr = m.d; dn.Ap_out = c->ap_x; dn.ssq_out = ssq_other;
    dn.gain_next = l + 1 < m.L ? m.attn_norm(l + 1) : m.final_norm();
    if (stamp_last_down && l == m.L - 1) dn.ts_end = c->ts_head;
    e = launch_gemm(m.dn[l].plan.shape, EPI_RESID, dn, s);
    std::swap(ssq_in, ssq_other);
    ssq_groups = m.dn[l].plan.workgroups();
  }
  return e;
}

// Sums of squares left by the last layer's down projection (each layer ends
// with them back in ssq_a) for the final RMSNorm.
int final_ssq_groups(const Model& m) { return m.dn[m.L - 1].plan.workgroups(); }
float* final_ssq(spec_ctx* c, const Model&) { return c->ssq_a; }

// final norm + LM head (+ logits partials) + softmax into `dst`
hipError_t enqueue_head(spec_ctx* c, const Model& m, hipStream_t s, int last_row_only, int n_rows,
                        int fixed_rows, float* logits_dst, float* dst, bool stamp = false) {
  GemmArgs a = gemm_base(c, m.lm, c->ap_x);
  a.fixed_rows = fixed_rows;
  if (stamp) a.ts_end = c->ts_head + c->ts_head_groups;
  a.ssq = final_ssq(c, m); a.ssq_groups = final_ssq_groups(m); a.eps = m.eps;
  a.last_row_only = last_row_only;
  a.out = logits_dst; a.ldo = m.V; a.lm_part = c->lm_part; a.n_valid = m.V;
  hipError_t e = launch_gemm(m.lm.plan.shape, EPI_LOGITS, a, s);
  if (e != hipSuccess) return e;
  SoftmaxArgs sm{};
  sm.logits = logits_dst; sm.part = c->lm_part; sm.G = m.lm.plan.workgroups(); sm.V = m.V;
  sm.rows = c->rows; sm.last_row_only = last_row_only; sm.out = dst; sm.chunk = c->sm_chunk;
  return launch_softmax(sm, c->sm_nchunks, last_row_only ? 1 : n_rows, s);
}

hipError_t enqueue_embed(spec_ctx* c, const Model& m, hipStream_t s, int mode, int n_rows, int pos0,
                         int step, const int32_t* dtok) {
  EmbedArgs a{};
  a.E = m.embed; a.d = m.d; a.vocab = m.V; a.max_seq = c->p.max_seq;
  a.st = c->st; a.hist = c->hist; a.dtok = dtok;
  a.mode = mode; a.n_rows = n_rows; a.pos0 = pos0; a.step = step;
  a.rows_out = c->rows; a.x = c->x; a.gain = m.attn_norm(0); a.Ap_out = c->ap_x;
  a.ssq = c->ssq_a;
  return launch_embed(a, s);
}

hipError_t enqueue_draft(spec_ctx* c, hipStream_t s, int K, uint64_t seed, int32_t* d, float* Dp) {
  const Model& m = c->D;
  hipError_t e = hipSuccess;
  for (int st = 0; st < K && e == hipSuccess; ++st) {
    e = enqueue_embed(c, m, s, st == 0 ? EMB_DRAFT0 : EMB_DRAFTS, 0, 0, st, d);
    // step 0 may carry catch-up rows; later steps have one row
    if (e == hipSuccess) e = enqueue_layers(c, m, s, st == 0 ? kMaxRows : 1, st == 0 ? 0 : 1, c->profiling);
    float* drow = Dp + (size_t)st * m.V;
    if (e == hipSuccess) e = enqueue_head(c, m, s, 1, 1, st == 0 ? 0 : 1, c->logits, drow);
    if (e == hipSuccess) {
      ArArgs ar{};
      ar.T = drow; ar.D = nullptr; ar.d = d; ar.B = 1; ar.K = 0; ar.V = m.V;
      ar.seed = seed; ar.stream_id = c->p.stream_id; ar.pos = nullptr; ar.st = c->st;
      ar.pos_offset = st + 1; ar.greedy = c->p.greedy; ar.word = 0;
      ar.chunk = c->ar_chunk; ar.n_chunks = c->ar_nchunks;
      ar.out = d + st; ar.n_acc = nullptr; ar.ws = c->ar_ws;
      e = launch_accept_reject(ar, s);
    }
  }
  return e;
}

hipError_t enqueue_verify(spec_ctx* c, hipStream_t s, int K, uint64_t seed, const int32_t* d,
                          const float* Dp, int32_t* out, int32_t* nacc, float* Tdst, float* Ldst) {
  const Model& m = c->T;
  float* Tb = Tdst ? Tdst : c->Tbuf;
  float* Lb = Ldst ? Ldst : c->logits;
  hipError_t e = enqueue_embed(c, m, s, EMB_VERIFY, K + 1, 0, 0, d);
  if (e == hipSuccess) e = enqueue_layers(c, m, s, K + 1, K + 1, c->profiling, c->profiling);
  if (e == hipSuccess) e = enqueue_head(c, m, s, 0, K + 1, K + 1, Lb, Tb, c->profiling);
  if (e == hipSuccess) {
    ArArgs ar{};
    ar.T = Tb; ar.D = Dp; ar.d = d; ar.B = 1; ar.K = K; ar.V = m.V;
    ar.seed = seed; ar.stream_id = c->p.stream_id; ar.pos = nullptr; ar.st = c->st;
    ar.pos_offset = 1; ar.greedy = c->p.greedy; ar.word = 2;
    ar.chunk = c->ar_chunk; ar.n_chunks = c->ar_nchunks;
    ar.out = out; ar.n_acc = nacc; ar.ws = c->ar_ws;
    e = launch_accept_reject(ar, s);
  }
  return e;
}

// Drafting heads: normed state -> stacked head GEMM (one row, the first K
// heads' columns) -> z_k rows -> LM head over K rows -> softmax into D ->
// one sampler per draft (word 0 at the draft's position, as for the draft
// model; argmax in greedy mode).
hipError_t enqueue_heads_draft(spec_ctx* c, hipStream_t s, int K, uint64_t seed, int32_t* d,
                               float* Dp) {
  const Model& m = c->T;
  HeadsArgs h{};
  h.h_last = c->h_last; h.g_final = m.final_norm(); h.d = m.d; h.eps = m.eps; h.hn = c->hn;
  h.Ap = c->ap_x; h.rows = c->rows; h.st = c->st; h.y = c->head_y; h.K = K;
  hipError_t e = launch_heads_prep(h, s);
  if (e != hipSuccess) return e;
  GemmArgs a = gemm_base(c, c->heads, c->ap_x);
  const int blocks = K * m.d / 16, nb = c->heads.plan.shape.nb;
  a.n_groups = (blocks + nb - 1) / nb;  // the first K heads' columns
  a.out = c->head_y; a.ldo = c->heads.N;
  e = launch_gemm(c->heads.plan.shape, EPI_STORE, a, s);
  if (e == hipSuccess) e = launch_heads_pack(h, s);
  if (e != hipSuccess) return e;
  GemmArgs lm = gemm_base(c, m.lm, c->ap_x);  // no norm: z_k is scored as it is
  lm.out = c->logits; lm.ldo = m.V; lm.lm_part = c->lm_part; lm.n_valid = m.V;
  e = launch_gemm(m.lm.plan.shape, EPI_LOGITS, lm, s);
  if (e != hipSuccess) return e;
  SoftmaxArgs sm{};
  sm.logits = c->logits; sm.part = c->lm_part; sm.G = m.lm.plan.workgroups(); sm.V = m.V;
  sm.rows = c->rows; sm.last_row_only = 0; sm.out = Dp; sm.chunk = c->sm_chunk;
  e = launch_softmax(sm, c->sm_nchunks, K, s);
  for (int k = 0; k < K && e == hipSuccess; ++k) {
    ArArgs ar{};
    ar.T = Dp + (size_t)k * m.V; ar.D = nullptr; ar.d = d; ar.B = 1; ar.K = 0; ar.V = m.V;
    ar.seed = seed; ar.stream_id = c->p.stream_id; ar.pos = nullptr; ar.st = c->st;
    ar.pos_offset = k + 1; ar.greedy = c->p.greedy; ar.word = 0;
    ar.chunk = c->ar_chunk; ar.n_chunks = c->ar_nchunks;
    ar.out = d + k; ar.n_acc = nullptr; ar.ws = c->ar_ws;
    e = launch_accept_reject(ar, s);
  }
  return e;
}

// Runs `body` either through a cached graph captured on the capture stream,
// or (no graphs) directly on the context stream.  With profiling on, the
// pass's timestamp slots [slot0, slot0 + n_slots) are reset on the stream
// first (outside any graph) and the graph is keyed separately.
template <typename F>
int run_pass(spec_ctx* c, std::vector<uint64_t> key, int slot0, int n_slots, F body) {
  if (c->profiling) {
    n_slots = std::min(n_slots, c->ts_cap - slot0);
    HIPTRY(c, hipMemsetAsync(c->ts + (size_t)slot0 * 2 * c->ts_groups, 0,
                             (size_t)n_slots * 2 * c->ts_groups * sizeof(unsigned long long),
                             c->stream));
    key.push_back(0x70726f66ull);  // separate graphs with the timestamp slots baked in
  }
  auto enqueue = [&](hipStream_t s) {
    c->ts_next = slot0;
    return body(s);
  };
  if (!c->graphs) {
    HIPTRY(c, enqueue(c->stream));
    return SPEC_OK;
  }
  auto it = c->graph_cache.find(key);
  if (it == c->graph_cache.end()) {
    GraphEntry ge;
    HIPTRY(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeRelaxed));
    hipError_t e = enqueue(c->cap_stream);
    hipGraph_t g = nullptr;
    hipError_t e2 = hipStreamEndCapture(c->cap_stream, &g);
    if (e == hipSuccess) e = e2;
    if (e == hipSuccess) e = hipGraphInstantiate(&ge.exec, g, nullptr, nullptr, 0);
    if (g) (void)hipGraphDestroy(g);
    HIPTRY(c, e);
    it = c->graph_cache.emplace(key, ge).first;
  }
  HIPTRY(c, hipGraphLaunch(it->second.exec, c->stream));
  return SPEC_OK;
}

int sync_state(spec_ctx* c, DevState* hs) {
  HIPTRY(c, hipStreamSynchronize(c->stream));
  HIPTRY(c, hipMemcpy(hs, c->st, sizeof(DevState), hipMemcpyDeviceToHost));
  return SPEC_OK;
}

// Prefill rows [pos0, pos0+n) of the committed history into model m.
int prefill(spec_ctx* c, const Model& m, int pos0, int n) {
  for (int p = pos0; p < pos0 + n; p += kMaxRows) {
    const int cnt = std::min(kMaxRows, pos0 + n - p);
    HIPTRY(c, enqueue_embed(c, m, c->stream, EMB_PREFILL, cnt, p, 0, nullptr));
    HIPTRY(c, enqueue_layers(c, m, c->stream, kMaxRows, 0, false));
  }
  return SPEC_OK;
}

void destroy_ctx(spec_ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  for (auto& kv : c->graph_cache)
    if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
  (void)hipFree(c->ts);
  free_model(c->D);
  free_model(c->T);
  void* bufs[] = {c->x,      c->qf,      c->ssq_a,  c->ssq_b, c->ap_x,  c->ap_o,
                  c->ap_a,   c->logits,  c->Tbuf,   c->attn_wo, c->attn_ml, c->lm_part,
                  c->ar_ws,  c->rows,    c->st,     c->hist,  c->heads_arena, c->h_last,
                  c->hn,     c->head_y,  c->ts_head};
  for (void* b : bufs) (void)hipFree(b);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  if (c->own_stream && c->stream) (void)hipStreamDestroy(c->stream);
  delete c;
}

}  // namespace

// ===================================================================== ABI ==
extern "C" {

int spec_init(const spec_init_params* p, const int32_t* prompt_host, int32_t n_prompt,
              spec_ctx** out) {
  if (!out) return fail(nullptr, SPEC_ERR_ARG, "spec_init: out is null");
  *out = nullptr;
  if (!p || !prompt_host) return fail(nullptr, SPEC_ERR_ARG, "spec_init: null argument");
  std::string why;
  if (!valid_model(p->target, &why)) return fail(nullptr, SPEC_ERR_ARG, "target: " + why);
  if (!valid_model(p->draft, &why)) return fail(nullptr, SPEC_ERR_ARG, "draft: " + why);
  if (p->draft.vocab != p->target.vocab)
    return fail(nullptr, SPEC_ERR_ARG, "draft and target must share the vocabulary");
  if (p->k_max < 1 || p->k_max > SPEC_K_MAX)
    return fail(nullptr, SPEC_ERR_ARG, fmt("k_max must be in 1..%d", SPEC_K_MAX));
  if (n_prompt < 1) return fail(nullptr, SPEC_ERR_ARG, "n_prompt must be >= 1");
  for (int i = 0; i < n_prompt; ++i)
    if (prompt_host[i] < 0 || prompt_host[i] >= p->target.vocab)
      return fail(nullptr, SPEC_ERR_ARG, fmt("prompt token %d out of range", i));
  if (p->max_seq < n_prompt + p->k_max + 1)
    return fail(nullptr, SPEC_ERR_CAPACITY, "max_seq must be >= n_prompt + k_max + 1");

  spec_ctx* c = new spec_ctx();
  c->p = *p;
  (void)hipGetDevice(&c->device);
  c->graphs = p->use_graphs != 0 && getenv("SPEC_NO_GRAPH") == nullptr;
  c->profiling = p->profile_kernels != 0;
  auto bail = [&](int rc) {
    std::string msg = c->err;
    destroy_ctx(c);
    g_err = msg;
    return rc;
  };
#define TRY(expr)                     \
  do {                                \
    int rc_ = (expr);                 \
    if (rc_ != SPEC_OK) return bail(rc_); \
  } while (0)
#define TRYH(expr)                                                                        \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return bail(fail(c, e_ == hipErrorOutOfMemory ? SPEC_ERR_OOM : SPEC_ERR_HIP,        \
                       fmt("%s: %s", #expr, hipGetErrorString(e_))));                      \
  } while (0)

  if (p->hip_stream) {
    c->stream = (hipStream_t)p->hip_stream;
  } else {
    TRYH(hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking));
    c->own_stream = true;
  }
  TRYH(hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));

  TRY(build_model(c, p->target, c->T, nullptr, nullptr));
  TRY(build_model(c, p->draft, c->D, &c->T, &p->target));

  const Model* ms[2] = {&c->T, &c->D};
  int dmax = 0, qmax = 0, fmax = 0, V = c->T.V, lm_groups = 0, ssq_groups = 0;
  size_t attn_wo = 0, attn_ml = 0, qf_elems = 0;
  c->attn_max_chunks = (p->max_seq + kAttnChunk - 1) / kAttnChunk;
  for (const Model* m : ms) {
    dmax = std::max(dmax, m->d);
    qmax = std::max(qmax, m->qd);
    fmax = std::max(fmax, m->F);
    lm_groups = std::max(lm_groups, m->lm.plan.workgroups());
    ssq_groups = std::max(ssq_groups, m->d / 64);
    for (int l = 0; l < m->L; ++l)
      ssq_groups = std::max({ssq_groups, m->o[l].plan.workgroups(), m->dn[l].plan.workgroups()});
    // every RMSNorm consumer must be able to fold its producer's partials
    auto cap = [](const Mat& x) { return x.plan.shape.waves * 64 / kMaxRows * kGemmMaxSsqPerThread; };
    bool ok = m->d / 64 <= cap(m->qkv[0]) && m->dn[m->L - 1].plan.workgroups() <= cap(m->lm);
    for (int l = 0; l < m->L; ++l) {
      ok = ok && m->o[l].plan.workgroups() <= cap(m->gu[l]);
      if (l > 0) ok = ok && m->dn[l - 1].plan.workgroups() <= cap(m->qkv[l]);
    }
    if (!ok) return bail(fail(c, SPEC_ERR_ARG, "d_model too large for the RMSNorm partial fold"));
    const int qg = (m->nq / m->nkv) * kMaxRows;
    attn_wo = std::max(attn_wo, (size_t)m->nkv * c->attn_max_chunks * qg * ((m->hd + 15) / 16 * 16));
    attn_ml = std::max(attn_ml, (size_t)m->nkv * c->attn_max_chunks * qg);
    qf_elems = std::max(qf_elems, (size_t)m->nkv * ((m->nq / m->nkv + 1) / 2) *
                                      ((m->hd + 31) / 32) * 2 * 512);
  }
  if (lm_groups > 8192)
    return bail(fail(c, SPEC_ERR_ARG, "vocabulary too large for the softmax partial fold"));
  ar_choose_chunks(1, V, &c->ar_chunk, &c->ar_nchunks);
  c->sm_chunk = 4096;
  c->sm_nchunks = (V + c->sm_chunk - 1) / c->sm_chunk;
  TRYH(dalloc(&c->x, (size_t)kMaxRows * dmax));
  if (qf_elems * 2 >= (1ull << 31))
    return bail(fail(c, SPEC_ERR_ARG, "attention query fragments exceed 2 GiB"));
  c->qf_elems = qf_elems;
  TRYH(dalloc(&c->qf, qf_elems));
  TRYH(hipMemsetAsync(c->qf, 0, qf_elems * 2, c->stream));
  TRYH(dalloc(&c->ssq_a, (size_t)kMaxRows * ssq_groups));
  TRYH(dalloc(&c->ssq_b, (size_t)kMaxRows * ssq_groups));
  // packed A operands: 16 bf16 rows (8 hi + 8 lo) per column
  TRYH(dalloc(&c->ap_x, (size_t)16 * dmax));
  TRYH(dalloc(&c->ap_o, (size_t)16 * qmax));
  TRYH(dalloc(&c->ap_a, (size_t)16 * fmax));
  TRYH(dalloc(&c->logits, (size_t)kMaxRows * V));
  TRYH(dalloc(&c->Tbuf, (size_t)kMaxRows * V));
  TRYH(dalloc(&c->attn_wo, attn_wo));
  TRYH(dalloc(&c->attn_ml, attn_ml));
  TRYH(dalloc(&c->lm_part, (size_t)lm_groups * kMaxRows));
  TRYH(dalloc(&c->ar_ws, (size_t)c->ar_nchunks * ar_ws_words(SPEC_K_MAX)));
  TRYH(dalloc(&c->rows, 1));
  TRYH(dalloc(&c->st, 1));
  c->ts_cap = p->k_max * c->D.L + c->T.L;
  for (const Model* m : ms)
    for (int l = 0; l < m->L; ++l)
      c->ts_groups = std::max({c->ts_groups, m->o[l].plan.workgroups(), m->gu[l].plan.workgroups()});
  TRYH(dalloc(&c->ts, (size_t)c->ts_cap * 2 * c->ts_groups));
  c->ts_head_groups = std::max(c->T.lm.plan.workgroups(), c->T.dn[c->T.L - 1].plan.workgroups());
  TRYH(dalloc(&c->ts_head, (size_t)2 * c->ts_head_groups));
  TRYH(hipDeviceGetAttribute(&c->wall_khz, hipDeviceAttributeWallClockRate, c->device));
  if (c->wall_khz <= 0) return bail(fail(c, SPEC_ERR_HIP, "device reports no wall-clock rate"));
  TRYH(hipMemsetAsync(c->ap_x, 0, (size_t)32 * dmax, c->stream));
  TRYH(hipMemsetAsync(c->ap_o, 0, (size_t)32 * qmax, c->stream));
  TRYH(hipMemsetAsync(c->ap_a, 0, (size_t)32 * fmax, c->stream));
  TRYH(dalloc(&c->h_last, (size_t)c->T.d));
  TRYH(dalloc(&c->hn, (size_t)c->T.d));
  c->hist_cap = p->max_seq + 16;
  TRYH(dalloc(&c->hist, (size_t)c->hist_cap));
  TRYH(hipMemsetAsync(c->x, 0, (size_t)kMaxRows * dmax * 4, c->stream));
  TRYH(hipMemsetAsync(c->hist, 0, (size_t)c->hist_cap * 4, c->stream));
  TRYH(hipMemcpyAsync(c->hist, prompt_host, (size_t)n_prompt * 4, hipMemcpyHostToDevice, c->stream));
  DevState hs{};
  TRYH(hipMemcpyAsync(c->st, &hs, sizeof hs, hipMemcpyHostToDevice, c->stream));
  TRYH(hipStreamSynchronize(c->stream));

  // prompt[0..n-2] into both caches; prompt[n-1] is the pending token
  TRY(prefill(c, c->T, 0, n_prompt - 1));
  if (n_prompt >= 2) {
    // the prefill's last row (position n_prompt - 2) sits at row (n_prompt - 2) % 8 of its chunk
    const int r = (n_prompt - 2) % kMaxRows;
    TRYH(hipMemcpyAsync(c->h_last, c->x + (size_t)r * c->T.d, (size_t)c->T.d * 4,
                        hipMemcpyDeviceToDevice, c->stream));
    c->h_valid = true;
  }
  TRY(prefill(c, c->D, 0, n_prompt - 1));
  hs.LT = n_prompt - 1;
  hs.LD = n_prompt - 1;
  TRYH(hipMemcpyAsync(c->st, &hs, sizeof hs, hipMemcpyHostToDevice, c->stream));
  TRYH(hipStreamSynchronize(c->stream));
  c->LT_ub = n_prompt - 1;
  c->lag_ub = 0;
  *out = c;
  return SPEC_OK;
#undef TRY
#undef TRYH
}

int spec_draft(spec_ctx* c, int32_t K, uint64_t seed, int32_t* d_dev, float* D_dev) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_draft: null context");
  if (K < 1 || K > c->p.k_max) return fail(c, SPEC_ERR_ARG, fmt("K=%d outside 1..k_max", K));
  if (!d_dev || !D_dev) return fail(c, SPEC_ERR_ARG, "spec_draft: null output");
  if (c->verify_pending) return fail(c, SPEC_ERR_STATE, "spec_draft: a verify is pending");
  HIPTRY(c, hipSetDevice(c->device));
  if (c->lag_ub > kMaxRows - 1 || c->LT_ub + K > c->p.max_seq) {
    DevState hs;
    if (int r = sync_state(c, &hs)) return r;
    c->LT_ub = hs.LT;
    if (hs.LT + K > c->p.max_seq)
      return fail(c, SPEC_ERR_CAPACITY, "draft positions would exceed max_seq");
    if (hs.LT - hs.LD > kMaxRows - 1) {
      // catch the draft cache up with the committed history, then continue
      if (int r = prefill(c, c->D, hs.LD, hs.LT - hs.LD)) return r;
      hs.LD = hs.LT;
      HIPTRY(c, hipMemcpyAsync(&c->st->LD, &hs.LD, 4, hipMemcpyHostToDevice, c->stream));
      HIPTRY(c, hipStreamSynchronize(c->stream));
    }
    c->lag_ub = hs.LT - hs.LD;
  }
  std::vector<uint64_t> key = {kPassDraft, (uint64_t)K, seed, (uint64_t)(uintptr_t)d_dev,
                               (uint64_t)(uintptr_t)D_dev};
  int r = run_pass(c, key, 0, K * c->D.L,
                   [&](hipStream_t s) { return enqueue_draft(c, s, K, seed, d_dev, D_dev); });
  if (r) return r;
  c->prof_draft_n = c->profiling ? std::min(K * c->D.L, c->ts_cap) : 0;
  c->drafted_k = K;
  return SPEC_OK;
}

int spec_draft_ngram(spec_ctx* c, int32_t K, int32_t n_max, int32_t* d_dev, float* D_dev) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_draft_ngram: null context");
  if (K < 1 || K > c->p.k_max) return fail(c, SPEC_ERR_ARG, fmt("K=%d outside 1..k_max", K));
  if (n_max < 1 || n_max > kNgramMaxN)
    return fail(c, SPEC_ERR_ARG, fmt("n_max=%d outside 1..%d", n_max, kNgramMaxN));
  if (!d_dev || (!D_dev && !c->p.greedy)) return fail(c, SPEC_ERR_ARG, "spec_draft_ngram: null output");
  if (c->verify_pending) return fail(c, SPEC_ERR_STATE, "spec_draft_ngram: a verify is pending");
  HIPTRY(c, hipSetDevice(c->device));
  std::vector<uint64_t> key = {kPassNgram, (uint64_t)K, (uint64_t)n_max, (uint64_t)(uintptr_t)d_dev,
                               (uint64_t)(uintptr_t)D_dev};
  int r = run_pass(c, key, 0, 0, [&](hipStream_t s) {
    NgramArgs a{};
    a.st = c->st; a.hist = c->hist; a.hist_cap = c->hist_cap;
    a.K = K; a.n_max = n_max; a.V = c->T.V; a.d = d_dev; a.D = D_dev;
    return launch_ngram_draft(a, s);
  });
  if (r) return r;
  c->drafted_k = 0;  // no draft-model rows were computed: the draft cache keeps its length
  c->prof_draft_n = 0;
  return SPEC_OK;
}

int spec_heads_init(spec_ctx* c, const void* W_dev, int32_t n_heads) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_heads_init: null context");
  if (!W_dev) return fail(c, SPEC_ERR_ARG, "spec_heads_init: null weights");
  if (n_heads < 1 || n_heads > SPEC_K_MAX)
    return fail(c, SPEC_ERR_ARG, fmt("n_heads=%d outside 1..%d", n_heads, SPEC_K_MAX));
  if (c->verify_pending) return fail(c, SPEC_ERR_STATE, "spec_heads_init: a verify is pending");
  HIPTRY(c, hipSetDevice(c->device));
  HIPTRY(c, hipStreamSynchronize(c->stream));
  // drop the previous heads and the graphs that captured them
  for (auto it = c->graph_cache.begin(); it != c->graph_cache.end();) {
    if (it->first[0] == kPassHeads) {
      if (it->second.exec) (void)hipGraphExecDestroy(it->second.exec);
      it = c->graph_cache.erase(it);
    } else {
      ++it;
    }
  }
  (void)hipFree(c->heads_arena);
  (void)hipFree(c->head_y);
  c->heads_arena = nullptr;
  c->head_y = nullptr;
  c->n_heads = 0;
  int n_cu = 0;
  HIPTRY(c, hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, c->device));
  const int d = c->T.d;
  Mat h;
  h.N = n_heads * d;
  h.K = d;
  h.plan = plan_gemm(h.N, 1, d, n_cu);
  HIPTRY(c, dalloc(&c->heads_arena, h.elems()));
  h.p = c->heads_arena;
  HIPTRY(c, dalloc(&c->head_y, (size_t)h.N));
  const uint16_t* W = (const uint16_t*)W_dev;
  std::vector<const uint16_t*> rows((size_t)h.plan.n_groups * h.plan.shape.nb * 16, nullptr);
  for (int n = 0; n < h.N; ++n) rows[n] = W + (size_t)n * d;  // row n: head n / d, output n % d
  if (int r = pack_rows(c, rows, h)) return r;
  c->heads = h;
  c->n_heads = n_heads;
  return SPEC_OK;
}

int spec_draft_heads(spec_ctx* c, int32_t K, uint64_t seed, int32_t* d_dev, float* D_dev) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_draft_heads: null context");
  if (c->n_heads < 1) return fail(c, SPEC_ERR_STATE, "spec_draft_heads: no heads (spec_heads_init)");
  if (K < 1 || K > c->n_heads || K > c->p.k_max)
    return fail(c, SPEC_ERR_ARG, fmt("K=%d outside 1..min(n_heads, k_max)", K));
  if (!d_dev || !D_dev) return fail(c, SPEC_ERR_ARG, "spec_draft_heads: null output");
  if (c->verify_pending) return fail(c, SPEC_ERR_STATE, "spec_draft_heads: a verify is pending");
  if (!c->h_valid)
    return fail(c, SPEC_ERR_STATE, "spec_draft_heads: no processed position yet (one-token prompt)");
  HIPTRY(c, hipSetDevice(c->device));
  if (c->LT_ub + K > c->p.max_seq) {
    DevState hs;
    if (int r = sync_state(c, &hs)) return r;
    c->LT_ub = hs.LT;
    if (hs.LT + K > c->p.max_seq)
      return fail(c, SPEC_ERR_CAPACITY, "draft positions would exceed max_seq");
  }
  std::vector<uint64_t> key = {kPassHeads, (uint64_t)K, seed, (uint64_t)(uintptr_t)d_dev,
                               (uint64_t)(uintptr_t)D_dev, (uint64_t)(uintptr_t)c->heads_arena};
  int r = run_pass(c, key, 0, 0,
                   [&](hipStream_t s) { return enqueue_heads_draft(c, s, K, seed, d_dev, D_dev); });
  if (r) return r;
  c->drafted_k = 0;  // the draft model computed none of these rows: its cache keeps its length
  c->prof_draft_n = 0;
  return SPEC_OK;
}

int spec_verify(spec_ctx* c, int32_t K, uint64_t seed, const int32_t* d_dev, const float* D_dev,
                int32_t* out_dev, int32_t* n_acc_dev, float* T_dev, float* logits_dev) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_verify: null context");
  if (K < 0 || K > c->p.k_max) return fail(c, SPEC_ERR_ARG, fmt("K=%d outside 0..k_max", K));
  if (!out_dev || !n_acc_dev || (K > 0 && (!d_dev || (!D_dev && !c->p.greedy))))
    return fail(c, SPEC_ERR_ARG, "spec_verify: null argument");
  if (K == 0) d_dev = nullptr, D_dev = nullptr;  // not read: a plain decode step
  if (c->verify_pending) return fail(c, SPEC_ERR_STATE, "spec_verify: previous verify not committed");
  HIPTRY(c, hipSetDevice(c->device));
  if (c->LT_ub + K + 1 > c->p.max_seq) {
    DevState hs;
    if (int r = sync_state(c, &hs)) return r;
    c->LT_ub = hs.LT;
    if (hs.LT + K + 1 > c->p.max_seq)
      return fail(c, SPEC_ERR_CAPACITY, "verify positions would exceed max_seq");
  }
  std::vector<uint64_t> key = {kPassVerify,
                               (uint64_t)K,
                               seed,
                               (uint64_t)(uintptr_t)d_dev,
                               (uint64_t)(uintptr_t)D_dev,
                               (uint64_t)(uintptr_t)out_dev,
                               (uint64_t)(uintptr_t)n_acc_dev,
                               (uint64_t)(uintptr_t)T_dev,
                               (uint64_t)(uintptr_t)logits_dev};
  const int vslot0 = c->p.k_max * c->D.L;
  if (c->profiling)
    HIPTRY(c, hipMemsetAsync(c->ts_head, 0, (size_t)2 * c->ts_head_groups * sizeof(unsigned long long),
                             c->stream));
  c->head_stamped = c->profiling;
  int r = run_pass(c, key, vslot0, c->T.L, [&](hipStream_t s) {
    return enqueue_verify(c, s, K, seed, d_dev, D_dev, out_dev, n_acc_dev, T_dev, logits_dev);
  });
  if (r) return r;
  c->prof_verify_n = c->profiling ? std::min(c->T.L, c->ts_cap - vslot0) : 0;
  c->verify_pending = true;
  c->last_k = K;
  return SPEC_OK;
}

int spec_commit(spec_ctx* c, const int32_t* out_dev, const int32_t* n_acc_dev) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_commit: null context");
  if (!out_dev || !n_acc_dev) return fail(c, SPEC_ERR_ARG, "spec_commit: null argument");
  if (!c->verify_pending) return fail(c, SPEC_ERR_STATE, "spec_commit: no verify pending");
  HIPTRY(c, hipSetDevice(c->device));
  HIPTRY(c, launch_commit(c->st, c->hist, c->hist_cap, out_dev, n_acc_dev, c->drafted_k, c->last_k,
                         c->x, c->T.d, c->h_last, c->stream));
  c->h_valid = true;
  c->LT_ub += c->last_k + 1;
  c->lag_ub = c->drafted_k > 0 ? 1 : c->lag_ub + c->last_k + 1;
  c->drafted_k = 0;
  c->verify_pending = false;
  return SPEC_OK;
}

int spec_destroy(spec_ctx* c) {
  destroy_ctx(c);
  return SPEC_OK;
}

const char* spec_last_error(const spec_ctx* c) { return c ? c->err.c_str() : g_err.c_str(); }

int spec_sync(spec_ctx* c) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_sync: null context");
  HIPTRY(c, hipStreamSynchronize(c->stream));
  return SPEC_OK;
}

void* spec_stream(const spec_ctx* c) { return c ? (void*)c->stream : nullptr; }

int spec_get_state(spec_ctx* c, spec_state* out) {
  if (!c || !out) return fail(c, SPEC_ERR_ARG, "spec_get_state: null argument");
  DevState hs;
  if (int r = sync_state(c, &hs)) return r;
  int32_t pend = -1;
  if (hs.LT >= 0 && hs.LT < c->hist_cap)
    HIPTRY(c, hipMemcpy(&pend, c->hist + hs.LT, 4, hipMemcpyDeviceToHost));
  out->target_len = hs.LT;
  out->draft_len = hs.LD;
  out->pending = pend;
  out->device_error = hs.err;
  static_assert(kAcceptBins == SPEC_K_MAX + 1, "acceptance record covers K = 0..SPEC_K_MAX");
  for (int k = 0; k < kAcceptBins; ++k)
    for (int n = 0; n < kAcceptBins; ++n) out->accept_counts[k][n] = hs.accept_counts[k][n];
  return SPEC_OK;
}

int spec_get_history(spec_ctx* c, int32_t* host_out, int32_t n) {
  if (!c || !host_out || n < 0 || n > c->hist_cap)
    return fail(c, SPEC_ERR_ARG, "spec_get_history: bad argument");
  HIPTRY(c, hipStreamSynchronize(c->stream));
  HIPTRY(c, hipMemcpy(host_out, c->hist, (size_t)n * 4, hipMemcpyDeviceToHost));
  return SPEC_OK;
}

int spec_kernel_times(spec_ctx* c, float* ms_out, int32_t cap, int32_t* n_out) {
  if (!c || !n_out || cap < 0 || (cap > 0 && !ms_out))
    return fail(c, SPEC_ERR_ARG, "spec_kernel_times: bad argument");
  HIPTRY(c, hipStreamSynchronize(c->stream));
  std::vector<unsigned long long> h((size_t)c->ts_cap * 2 * c->ts_groups);
  if (!h.empty())
    HIPTRY(c, hipMemcpy(h.data(), c->ts, h.size() * sizeof(unsigned long long),
                        hipMemcpyDeviceToHost));
  int n = 0;
  // a stamp of 0 is a workgroup that did not write (the slot was reset)
  auto take = [&](int slot0, int cnt, const Model& m, int layer0) {
    for (int i = slot0; i < slot0 + cnt; ++i) {
      const int l = (layer0 + i - slot0) % m.L;
      const unsigned long long* o = &h[(size_t)i * 2 * c->ts_groups];
      const unsigned long long* g = o + c->ts_groups;
      unsigned long long o_end = 0, g_end = 0;
      bool ok = true;
      for (int w = 0; w < m.o[l].plan.workgroups(); ++w) { ok = ok && o[w] != 0; o_end = std::max(o_end, o[w]); }
      for (int w = 0; w < m.gu[l].plan.workgroups(); ++w) { ok = ok && g[w] != 0; g_end = std::max(g_end, g[w]); }
      const float ms = ok && g_end > o_end ? (float)((double)(g_end - o_end) / c->wall_khz) : -1.0f;
      if (n < cap) ms_out[n] = ms;
      ++n;
    }
  };
  take(0, c->prof_draft_n, c->D, 0);
  take(c->p.k_max * c->D.L, c->prof_verify_n, c->T, 0);
  *n_out = std::min(n, cap);
  return SPEC_OK;
}

int spec_head_time(spec_ctx* c, float* ms_out) {
  if (!c || !ms_out) return fail(c, SPEC_ERR_ARG, "spec_head_time: null argument");
  *ms_out = -1.0f;
  if (!c->head_stamped) return SPEC_OK;
  HIPTRY(c, hipStreamSynchronize(c->stream));
  std::vector<unsigned long long> h((size_t)2 * c->ts_head_groups);
  HIPTRY(c, hipMemcpy(h.data(), c->ts_head, h.size() * sizeof(unsigned long long),
                      hipMemcpyDeviceToHost));
  const Model& m = c->T;
  unsigned long long d_end = 0, l_end = 0;
  bool ok = true;
  for (int w = 0; w < m.dn[m.L - 1].plan.workgroups(); ++w) { ok = ok && h[w] != 0; d_end = std::max(d_end, h[w]); }
  for (int w = 0; w < m.lm.plan.workgroups(); ++w) {
    const unsigned long long t = h[(size_t)c->ts_head_groups + w];
    ok = ok && t != 0;
    l_end = std::max(l_end, t);
  }
  if (ok && l_end > d_end) *ms_out = (float)((double)(l_end - d_end) / c->wall_khz);
  return SPEC_OK;
}

int spec_set_profiling(spec_ctx* c, int32_t enable) {
  if (!c) return fail(nullptr, SPEC_ERR_ARG, "spec_set_profiling: null context");
  HIPTRY(c, hipStreamSynchronize(c->stream));
  c->profiling = enable != 0;
  return SPEC_OK;
}

// ------------------------------------------- packed matrix, batched rows --
struct spec_mat {
  int device = 0;
  int N = 0, K = 0, nb = 1;
  uint16_t* Wp = nullptr;
  uint16_t* A = nullptr;  // activation workspace for up to kRowsMaxM rows
  float* P = nullptr;     // split-K partials for up to kRowsMaxM rows
  size_t P_elems = 0;
};

int spec_mat_create(const void* W_dev, int32_t N, int32_t K, spec_mat** out) {
  if (!out) return fail(nullptr, SPEC_ERR_ARG, "spec_mat_create: null output");
  *out = nullptr;
  if (!W_dev || N < 16 || K < 32 || N % 16 || K % 32)
    return fail(nullptr, SPEC_ERR_ARG, "spec_mat_create: need N % 16 == 0, K % 32 == 0");
  spec_mat* m = new spec_mat();
  m->N = N;
  m->K = K;
  const GemmPlan plan = plan_gemm(N, 1, K, 0);  // the rows GEMM takes nb 1 or 2
  m->nb = plan.shape.nb;
  hipError_t e = hipGetDevice(&m->device);
  std::vector<const uint16_t*> rows(N);
  for (int n = 0; n < N; ++n) rows[n] = (const uint16_t*)W_dev + (size_t)n * K;
  const uint16_t** drows = nullptr;
  if (e == hipSuccess) e = dalloc(&m->Wp, (size_t)N * K);
  if (e == hipSuccess) e = dalloc(&m->A, (size_t)(K / 32) * (kRowsMaxM / 8) * 64 * 8);
  m->P_elems = rows_partials(kRowsMaxM, N, K);
  if (e == hipSuccess) e = dalloc(&m->P, m->P_elems);
  if (e == hipSuccess) e = dalloc(&drows, (size_t)N);
  if (e == hipSuccess)
    e = hipMemcpy(drows, rows.data(), (size_t)N * sizeof(void*), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = launch_pack(drows, K, m->nb, N / (16 * m->nb), 0, 0, m->Wp, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipFree(drows);
  if (e != hipSuccess) {
    (void)hipFree(m->Wp);
    (void)hipFree(m->A);
    (void)hipFree(m->P);
    delete m;
    return fail(nullptr, e == hipErrorOutOfMemory ? SPEC_ERR_OOM : SPEC_ERR_HIP,
                fmt("spec_mat_create: %s", hipGetErrorString(e)));
  }
  *out = m;
  return SPEC_OK;
}

int spec_mat_mul(spec_mat* m, const float* X_dev, int32_t M, float* Y_dev, void* hip_stream) {
  if (!m || !X_dev || !Y_dev) return fail(nullptr, SPEC_ERR_ARG, "spec_mat_mul: null argument");
  if (M < 1 || M > kRowsMaxM)
    return fail(nullptr, SPEC_ERR_ARG, fmt("spec_mat_mul: M=%d outside 1..%d", M, kRowsMaxM));
  RowsGemmArgs a{};
  a.Wp = m->Wp; a.N = m->N; a.K = m->K; a.nb = m->nb;
  a.X = X_dev; a.M = M; a.A = m->A; a.Y = Y_dev; a.P = m->P; a.P_elems = m->P_elems;
  HIPTRY(nullptr, hipSetDevice(m->device));
  HIPTRY(nullptr, launch_gemm_rows(a, (hipStream_t)hip_stream));
  return SPEC_OK;
}

int spec_mat_destroy(spec_mat* m) {
  if (!m) return SPEC_OK;
  (void)hipSetDevice(m->device);
  (void)hipDeviceSynchronize();
  (void)hipFree(m->Wp);
  (void)hipFree(m->A);
  (void)hipFree(m->P);
  delete m;
  return SPEC_OK;
}

// ---------------------------------------------------------- choosing K --
// [en] Floor 6: mean tokens per round with iid acceptance; [int] "speedup":
// a round costs K draft steps plus one target pass.
double spec_expected_tokens(double alpha, int32_t K) {
  double total = 0.0, power = 1.0;  // alpha^j for j = 0..K
  for (int32_t j = 0; j <= K; ++j) {
    total += power;
    power *= alpha;
  }
  return total;
}

double spec_alpha_from_tokens(double tokens_per_round, int32_t K) {
  if (K < 1 || !(tokens_per_round > 1.0)) return 0.0;
  if (tokens_per_round >= K + 1.0) return 1.0;
  double lo = 0.0, hi = 1.0;  // spec_expected_tokens is increasing in alpha
  for (int it = 0; it < 100; ++it) {
    const double mid = 0.5 * (lo + hi);
    (spec_expected_tokens(mid, K) < tokens_per_round ? lo : hi) = mid;
  }
  return 0.5 * (lo + hi);
}

int32_t spec_choose_k(double alpha, double t_draft_step, double t_verify, int32_t k_max) {
  if (!(alpha >= 0.0 && alpha <= 1.0) || !(t_draft_step >= 0.0) || !(t_verify >= 0.0) ||
      t_draft_step + t_verify <= 0.0 || k_max < 1)
    return fail(nullptr, SPEC_ERR_ARG, "spec_choose_k: bad argument");
  int32_t best_k = 1;
  double best = -1.0;
  for (int32_t K = 1; K <= k_max; ++K) {
    const double per_time = spec_expected_tokens(alpha, K) / (K * t_draft_step + t_verify);
    if (per_time > best) {
      best = per_time;
      best_k = K;
    }
  }
  return best_k;
}

// -------------------------------------------------- stateless accept/reject --
namespace {
struct ArWorkspace {
  uint64_t* ws = nullptr;
  size_t ws_words = 0;
};
std::mutex g_ar_mu;
std::map<int, ArWorkspace> g_ar;

// Argument checks and the launch plan shared by both stateless entry points.
// Returns SPEC_OK and fills a (all but ws) and *words, or an error code.
int ar_prepare(const char* who, const float* T_dev, const float* D_dev, const int32_t* d_dev,
               int32_t B, int32_t K, int32_t V, uint64_t seed, const uint64_t* pos_dev,
               uint64_t stream_id, int32_t greedy, int32_t* out_dev, int32_t* n_acc_dev,
               ArArgs* a, size_t* words) {
  if (B < 0 || K < 1 || K > SPEC_AR_K_MAX || V < 1)
    return fail(nullptr, SPEC_ERR_ARG, fmt("%s: bad B, K or V", who));
  if (B > 0 && (!T_dev || !d_dev || !pos_dev || !out_dev || !n_acc_dev || (!greedy && !D_dev)))
    return fail(nullptr, SPEC_ERR_ARG, fmt("%s: null pointer", who));
  int chunk = 0, nch = 0;
  ar_choose_chunks(B, V, &chunk, &nch);
  if ((long long)B * nch > 0x7fffffffLL)
    return fail(nullptr, SPEC_ERR_ARG, fmt("%s: batch too large for one launch", who));
  *a = ArArgs{};
  a->T = T_dev; a->D = D_dev; a->d = d_dev; a->B = B; a->K = K; a->V = V;
  a->seed = seed; a->stream_id = stream_id; a->pos = pos_dev; a->st = nullptr; a->pos_offset = 0;
  a->greedy = greedy; a->word = 2; a->chunk = chunk; a->n_chunks = nch;
  a->out = out_dev; a->n_acc = n_acc_dev;
  *words = (size_t)B * nch * ar_ws_words(K);
  return SPEC_OK;
}
}  // namespace

int spec_accept_reject(const float* T_dev, const float* D_dev, const int32_t* d_dev, int32_t B,
                       int32_t K, int32_t V, uint64_t seed, const uint64_t* pos_dev,
                       uint64_t stream_id, int32_t greedy, int32_t* out_dev, int32_t* n_acc_dev,
                       void* hip_stream) {
  ArArgs a;
  size_t words = 0;
  if (int r = ar_prepare("spec_accept_reject", T_dev, D_dev, d_dev, B, K, V, seed, pos_dev,
                         stream_id, greedy, out_dev, n_acc_dev, &a, &words))
    return r;
  if (B == 0) return SPEC_OK;
  hipStream_t s = (hipStream_t)hip_stream;
  int dev = 0;
  HIPTRY(nullptr, hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_ar_mu);
  ArWorkspace& w = g_ar[dev];
  if (w.ws_words < words) {
    // the previous workspace may still be read by work queued on any stream
    HIPTRY(nullptr, hipDeviceSynchronize());
    (void)hipFree(w.ws);
    w.ws = nullptr;
    w.ws_words = 0;
    HIPTRY(nullptr, dalloc(&w.ws, words));
    w.ws_words = words;
  }
  a.ws = w.ws;
  HIPTRY(nullptr, launch_accept_reject(a, s));
  return SPEC_OK;
}

}  // extern "C"

// ------------------------------------- accept/reject without allocating --
// The chunk partials of spec_accept_reject_noalloc live in this file-scope
// device array: every device the library runs on holds one copy, from module
// load until the process ends.  In host code the name `scratch` is only a
// host-side stand-in for the symbol; its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is ever handed to a kernel.  Every word a finishing block reads is
// written by the partial kernel of the same call first, so nothing needs
// clearing between calls.
namespace {
constexpr size_t kNoAllocScratchWords = SPEC_AR_NOALLOC_SCRATCH_BYTES / sizeof(uint64_t);
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) uint64_t scratch[kNoAllocScratchWords];
std::mutex g_scratch_mu;
uint64_t* g_scratch_ptr[kNoAllocMaxDevices] = {};
}  // namespace

extern "C" {

int spec_accept_reject_noalloc(const float* T_dev, const float* D_dev, const int32_t* d_dev,
                               int32_t B, int32_t K, int32_t V, uint64_t seed,
                               const uint64_t* pos_dev, uint64_t stream_id, int32_t greedy,
                               int32_t* out_dev, int32_t* n_acc_dev, void* hip_stream) {
  ArArgs a;
  size_t words = 0;
  if (int r = ar_prepare("spec_accept_reject_noalloc", T_dev, D_dev, d_dev, B, K, V, seed, pos_dev,
                         stream_id, greedy, out_dev, n_acc_dev, &a, &words))
    return r;
  if (words > kNoAllocScratchWords)
    return fail(nullptr, SPEC_ERR_CAPACITY,
                fmt("spec_accept_reject_noalloc: B=%d, K=%d, V=%d needs %zu bytes of scratch, "
                    "more than the fixed %d",
                    B, K, V, words * sizeof(uint64_t), (int)SPEC_AR_NOALLOC_SCRATCH_BYTES));
  if (B == 0) return SPEC_OK;
  int dev = 0;
  HIPTRY(nullptr, hipGetDevice(&dev));
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(nullptr, SPEC_ERR_ARG, fmt("spec_accept_reject_noalloc: device %d unsupported", dev));
  uint64_t* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      HIPTRY(nullptr, hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      if (!p) return fail(nullptr, SPEC_ERR_HIP, "spec_accept_reject_noalloc: no scratch address");
      g_scratch_ptr[dev] = (uint64_t*)p;
    }
    ws = g_scratch_ptr[dev];
  }
  a.ws = ws;
  HIPTRY(nullptr, launch_accept_reject(a, (hipStream_t)hip_stream));
  return SPEC_OK;
}

int spec_read_ceiling(const void* buf_dev, uint64_t bytes, int32_t reps, void* hip_stream,
                      double* gb_per_s) {
  if (!buf_dev || !gb_per_s || bytes < (1u << 20) || bytes % 16 || reps < 1)
    return fail(nullptr, SPEC_ERR_ARG, "spec_read_ceiling: bad argument");
  hipStream_t s = (hipStream_t)hip_stream;
  int dev = 0, n_cu = 0;
  HIPTRY(nullptr, hipGetDevice(&dev));
  HIPTRY(nullptr, hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  uint32_t* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = dalloc(&sink, 1);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  double best = 0.0;
  for (int mult : {1, 2, 4}) {  // workgroups per CU
    const int grid = n_cu * mult;
    if (e == hipSuccess) e = launch_stream_read(buf_dev, bytes, grid, sink, s);  // warm-up
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch_stream_read(buf_dev, bytes, grid, sink, s);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && ms > 0.f) best = std::max(best, (double)bytes * reps / (ms * 1e-3) / 1e9);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(sink);
  HIPTRY(nullptr, e);
  *gb_per_s = best;
  return SPEC_OK;
}

}  // extern "C"
