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
  // A batch of sequences in one launch (0 or 1: a single pass).  Sequence b
  // reads rows[b], block_table + b * n_blocks, the query fragments
  // qf + b * qf_bytes / 2 (qf_bytes is then one sequence's share), its own
  // workspace slice, and writes its rows as rows b * seq_rows + r of the
  // packed output, laid out in a_tiles row tiles (the rows GEMM's layout,
  // a_tiles >= 1); a_tiles = 0: a single pass, written in the skinny GEMM's
  // layout (apack_index).
  int n_seq, seq_rows, a_tiles;
  int qt_per_wave;           // 2: one wave scores both 16-query tiles of a chunk (0 or 1: one)
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
// Row tiles of the packed A operand for M rows: the smallest power of two
// RT with 8 RT >= M.
inline int rows_tiles(int M) {
  int RT = 1;
  while (8 * RT < M) RT *= 2;
  return RT;
}
// Packed A of the rows GEMM, [K/32][RT][64 lanes][8 bf16]: tile t holds the
// bf16 high parts of rows 8t..8t+7 in its MFMA rows 0-7 and their low parts
// in rows 8-15, lane-major within a tile (the single pass's skinny GEMM
// keeps each row's 32 values of a k-block contiguous instead: apack_index).
SPEC_DEVICE size_t apack_index_rt(int m, int part, int k, int RT) {
  const int kk = k & 31;
  const int lane = (m & 7) + 8 * part + 16 * (kk >> 3);
  return (((size_t)(k >> 5) * RT + (m >> 3)) * 64 + lane) * 8 + (kk & 7);
}
SPEC_DEVICE void apack_store8_rt(uint16_t* Ap, int m, int k0, const float* v, int RT) {
  uint16_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f32_to_bf16_rne(v[e]);
    l[e] = f32_to_bf16_rne(v[e] - bf16_to_f32(h[e]));
  }
  *(uint4*)(Ap + apack_index_rt(m, 0, k0, RT)) =
      make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                 pack_bf16x2(h[6], h[7]));
  *(uint4*)(Ap + apack_index_rt(m, 1, k0, RT)) =
      make_uint4(pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3]), pack_bf16x2(l[4], l[5]),
                 pack_bf16x2(l[6], l[7]));
}
struct RowsGemmArgs {
  const uint16_t* Wp;     // packed weights (launch_pack layout, NB = nb)
  int N, K, nb;
  const float* X;         // [M][K] fp32 activations, packed into A by the launch; or null:
                          // A already holds them (rows_tiles(M) tiles)
  int M;
  uint16_t* A;            // [K/32][rows_tiles(M)][64][8] bf16
  float* Y;               // [M][ldy] fp32 (ldy 0: N)
  int ldy;
  int accumulate;         // 1: Y += X W^T (a residual update); 0: Y = X W^T
  float* P;               // split-K partials of the wide kernel (may be null: no split)
  size_t P_elems;         // capacity of P in floats
  int defer_sum;          // 1: leave split partials in P for the next kernel to sum
  int* split_out;         // host, may be null: slices left in P (0: Y holds the result)
};
// More than 8 rows take the wide kernel when N is a multiple of
// kRowsWideCols: its waves split a workgroup's columns and share the
// activation tiles through LDS.  Narrow matrices split K over up to
// kRowsMaxSplit workgroups (partials summed by a second launch).
constexpr int kRowsWideCols = 128;
constexpr int kRowsMaxSplit = 8;
// K slices the wide kernel uses for an N x K matrix (1: no split): enough
// workgroups for about one per CU.  (Two per CU measured slower: the extra
// partial traffic and reduce launch cost more than the overlap gains.)
inline int rows_wide_split(int N, int K) {
  const int groups = N / kRowsWideCols, Kb = K / 32;
  if (groups >= 192) return 1;
  int S = 256 / (groups > 0 ? groups : 1);
  S = S < 1 ? 1 : (S > kRowsMaxSplit ? kRowsMaxSplit : S);
  while (S > 1 && Kb / S < 4) --S;  // at least four k-blocks per slice
  return S;
}
// Partial floats the wide kernel needs for M rows of an N x K matrix.
inline size_t rows_partials(int M, int N, int K) {
  const int S = rows_wide_split(N, K);
  return S > 1 ? (size_t)S * M * N : 0;
}
hipError_t launch_gemm_rows(const RowsGemmArgs& a, hipStream_t s);
// The wide kernel (k_gemm_wide.hip) for RT > 1 row tiles and N % kRowsWideCols == 0,
// with its slice sum unless a.defer_sum; the operand is already packed.
hipError_t launch_gemm_wide(const RowsGemmArgs& a, int RT, int ldy, hipStream_t s);

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
  int B;                  // sequences (0 or 1: one); sequence b uses st + b,
                          // hist + b * hist_cap, d + b * K, D + b * K * V
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

// ------------------------------------------------ batches of sequences --
// A batched pass carries R rows per sequence for B sequences: row m = b R + r
// of the activations is row r of sequence b, at position rows[b].pos0 + r.
enum BatchEmbedMode : int {
  BEMB_VERIFY = 0,   // rows [hist_b[LT_b], d_b0..d_b,R-2] at LT_b..
  BEMB_PREFILL = 1,  // rows hist_b[pos0 + r] at pos0..
};
struct BatchEmbedArgs {
  const uint16_t* E;      // [vocab][d]
  int d, vocab, max_seq;
  DevState* st;           // [B]
  const int32_t* hist;    // [B][hist_cap]
  int hist_cap;
  const int32_t* dtok;    // [B][R-1] drafts (verify)
  int mode, B, R, pos0;
  PassRows* rows;         // [B] written
  uint64_t* pos_rule;     // [B] written: position of row 1 (the first draft)
  float* x;               // [B R][d] written
};
hipError_t launch_batch_embed(const BatchEmbedArgs& a, hipStream_t s);

// h = x / sqrt(mean(x^2) + eps) * gain for rows m < M, packed (rows GEMM
// layout, RT tiles); rows M..8 RT-1 are written as zeros.  With S > 0 split
// partials P[s][m][:] of a residual GEMM are first added to x (in slice
// order) and x is written back.  d <= kNormPackMaxD.
constexpr int kNormPackMaxD = 8192;
struct NormPackArgs {
  float* x;               // [M][d]
  int M, d, RT;
  const uint16_t* gain;   // [d] bf16
  float eps;
  uint16_t* Ap;
  const float* P;         // [S][M][d] or null
  int S;
};
hipError_t launch_norm_pack(const NormPackArgs& a, hipStream_t s);

// QKV product rows [M][q_dim + 2 kv_dim] (q, k, v in natural order) -> RoPE
// on q and k at each row's position; q into the sequence's query fragments,
// k and v (high and low planes) into the paged cache through its block table.
struct QkvPostArgs {
  const float* y;              // [M][q_dim + 2 kv_dim], or with S > 0:
  const float* P;              // [S][M][q_dim + 2 kv_dim] split partials, summed in slice order
  int S;
  int M, R, q_dim, kv_dim, hd, n_kv, max_seq;
  const PassRows* rows;        // [B]
  const float2* rope;          // [max_seq][hd/2] (cos, sin)
  uint16_t* qf;                // [B][qf_seq] fragments
  size_t qf_seq;
  uint16_t* k_cache;           // one layer of the pool
  uint16_t* v_cache;
  const int32_t* block_table;  // [B][n_blocks]
  int n_blocks;
};
hipError_t launch_qkv_post(const QkvPostArgs& a, hipStream_t s);

// y [M][2F] (gate columns 0..F-1, up columns F..2F-1) -> silu(gate) * up,
// packed (RT tiles, K = F); rows M..8 RT-1 zero.
struct SiluPackArgs {
  const float* y;
  int M, F, RT;
  uint16_t* Ap;
};
hipError_t launch_silu_pack(const SiluPackArgs& a, hipStream_t s);

// Row softmax of logits [M][V] into out (max-subtracted, fp32), in two
// launches: per (chunk, row) (max, sum of exp) partials, then the
// normalisation, each block folding its row's partials in chunk order.
struct RowSoftmaxArgs {
  const float* logits;
  int M, V, chunk, n_chunks;   // n_chunks * chunk >= V, n_chunks <= 256
  float2* part;                // [M][n_chunks]
  float* out;
};
hipError_t launch_row_softmax(const RowSoftmaxArgs& a, hipStream_t s);

// Commit of a batched verify: per sequence b, hist_b[LT_b+1..LT_b+1+n] =
// out[b][0..n] with n = n_acc[b], then LT_b += n + 1.
struct BatchCommitArgs {
  DevState* st;
  int32_t* hist;
  int hist_cap;
  const int32_t* out;     // [B][K+1]
  const int32_t* n_acc;   // [B]
  int B, K;
};
hipError_t launch_batch_commit(const BatchCommitArgs& a, hipStream_t s);

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
