// kernels.h -- launch-argument structs and host-side launchers of the HIP
// kernels (one translation unit per kernel family).  No kernel waits on, or
// synchronises with, another workgroup of the same launch: every cross-block
// reduction goes through a kernel boundary.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "k_gemm.h"

namespace spec {

// ------------------------------------------------------------- attention --
struct AttnArgs {
  const uint16_t* qf;        // query fragments (see qfrag_index)
  const uint16_t* k_cache;   // one layer, see kv_index
  const uint16_t* v_cache;   // one layer, see vt_index
  uint32_t qf_bytes;         // size of the fragment buffer (< 2^31)
  uint32_t kv_layer_bytes;   // size of one layer's key (= value) cache (< 2^31)
  const int32_t* block_table;
  const PassRows* rows;
  int n_q, n_kv, hd;
  int max_chunks;            // grid.x of the partial kernel: ceil(max_seq / kAttnChunk)
  int n_blocks;              // entries of block_table: ceil(max_seq / kBlock)
  float* ws_o;               // [n_kv][max_chunks][qg_max][ceil(hd/16)*16] unnormalised P V
  float2* ws_ml;             // [n_kv][max_chunks][qg_max] (max score, sum of exp)
  int qg_max;                // (n_q/n_kv) * kMaxRows
  uint16_t* Ap_out;          // packed attention output rows (K = n_q*hd) for the O projection
};
constexpr int kAttnChunk = 32;  // keys per partial (one wave), two cache blocks
// n_rows: rows the pass can have (bounds the merge grid); rows beyond
// rows->n_rows exit.
hipError_t launch_attn(const AttnArgs& a, int n_rows, hipStream_t s);

// ------------------------------------------------------------- embedding --
enum EmbedMode : int {
  EMB_VERIFY = 0,   // rows [hist[LT], d_0..d_{K-1}] at LT..LT+K
  EMB_DRAFT0 = 1,   // rows hist[LD..LT] at LD..
  EMB_DRAFTS = 2,   // row d_{step-1} at LT+step
  EMB_PREFILL = 3,  // rows hist[pos0..pos0+n-1]
};
struct EmbedArgs {
  const uint16_t* E;  // [vocab][d]
  int d, vocab, max_seq;
  DevState* st;
  const int32_t* hist;
  const int32_t* dtok;
  int mode, n_rows, pos0, step;
  PassRows* rows_out;
  float* x;               // [8][d]
  const uint16_t* gain;   // first RMSNorm gain [d]
  uint16_t* Ap_out;       // packed x * gain
  float* ssq;             // [d/64][8]
};
hipError_t launch_embed(const EmbedArgs& a, hipStream_t s);

// --------------------------------------------------------------- softmax --
struct SoftmaxArgs {
  const float* logits;   // [rows][V]
  const float2* part;    // [G][8]
  int G, V;
  const PassRows* rows;
  int last_row_only;
  float* out;            // [rows][V]
  int chunk;
};
// n_rows: rows the pass can have (grid.y); rows beyond rows->n_rows exit.
hipError_t launch_softmax(const SoftmaxArgs& a, int n_chunks, int n_rows, hipStream_t s);

// -------------------------------------------------------- accept/reject --
struct ArArgs {
  const float* T;        // [B][K+1][V]   (K = 0: one row to sample)
  const float* D;        // [B][K][V]
  const int32_t* d;      // [B][K]
  int B, K, V;
  uint64_t seed, stream_id;
  const uint64_t* pos;   // [B] position of d_1, or null: P = st->LT + pos_offset
  const DevState* st;
  int pos_offset;
  int greedy;
  int word;              // Philox word of the final sample (2 verify, 0 draft)
  int chunk, n_chunks;
  int32_t* out;          // [B][K+1]
  int32_t* n_acc;        // [B] or null
  uint64_t* ws;          // [B][n_chunks][ar_ws_words(K)] chunk partials
};
__host__ __device__ inline int ar_ws_words(int K) { return (K + 2) > 4 ? (K + 2) : 4; }
void ar_choose_chunks(int B, int V, int* chunk, int* n_chunks);
// Two launches: chunk partials, then one finishing block per sequence.
hipError_t launch_accept_reject(const ArArgs& a, hipStream_t s);

// --------------------------------------------- GEMM for a batch of rows --
constexpr int kRowsMaxM = 128;  // 16 row tiles of 8 activation rows (hi/lo)
struct RowsGemmArgs {
  const uint16_t* Wp;     // packed weights (launch_pack layout, NB = nb)
  int N, K, nb;
  const float* X;         // [M][K] fp32 activations
  int M;
  uint16_t* A;            // workspace: [K/32][ceil(M/8) rounded to a power of 2][64][8] bf16
  float* Y;               // [M][N] fp32
};
hipError_t launch_gemm_rows(const RowsGemmArgs& a, hipStream_t s);

// ------------------------------------------------------ n-gram drafter --
constexpr int kNgramMaxN = 8;   // longest key searched
constexpr int kNgramMaxK = 8;   // drafts per call (>= SPEC_K_MAX)
struct NgramArgs {
  const DevState* st;     // LT: position of the pending token
  const int32_t* hist;    // committed history [hist_cap]
  int hist_cap;
  int K, n_max, V;
  int32_t* d;             // [K] draft tokens
  float* D;               // [K][V] one-hot draft rows, or null
};
hipError_t launch_ngram_draft(const NgramArgs& a, hipStream_t s);

// ------------------------------------------------- multi-token heads --
struct HeadsArgs {
  const float* h_last;      // [d] final residual of the last committed position
  const uint16_t* g_final;  // [d] final RMSNorm gain (bf16)
  int d;
  float eps;
  float* hn;                // [d] normed state h (fp32)
  uint16_t* Ap;             // packed A operand (row 0: h; rows 0..K-1: z_k)
  PassRows* rows;           // pass descriptor of the head GEMM, then of the LM head
  const DevState* st;       // LT: position of the pending token
  const float* y;           // [K][d] head products W_k h (heads_pack)
  int K;                    // heads drafted, <= kMaxRows
};
hipError_t launch_heads_prep(const HeadsArgs& a, hipStream_t s);
hipError_t launch_heads_pack(const HeadsArgs& a, hipStream_t s);

// ---------------------------------------------------------------- commit --
// Also keeps the final residual row n_acc of the pass (x_rows, row stride d)
// in h_last: the state the drafting heads start from.
hipError_t launch_commit(DevState* st, int32_t* hist, int hist_cap, const int32_t* out,
                         const int32_t* n_acc, int drafted_k, int verified_k, const float* x_rows,
                         int d, float* h_last, hipStream_t s);
// Streaming read of `bytes` (a multiple of 16): `grid` workgroups of 512 threads, each reading one
// contiguous slice.
hipError_t launch_stream_read(const void* buf, size_t bytes, int grid, uint32_t* sink,
                              hipStream_t s);
// RoPE table: (cos, sin) of p * theta^(-2j/hd) for p < max_seq, j < hd/2,
// evaluated in fp64 and stored as fp32.
hipError_t launch_rope_table(float2* dst, int max_seq, int hd, double theta, hipStream_t s);

}  // namespace spec
