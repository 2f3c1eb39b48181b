// k_gemm.h -- launch arguments, launchers and launch plans of the
// weight-streaming skinny GEMM (k_gemm.hip).  Everything that decides the
// GEMM kernels' code and launch shapes lives in k_gemm.hip, this header and
// common.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "common.h"

namespace spec {

// ------------------------------------------------------------------ GEMM --
// Epilogue kinds of the skinny GEMM Y[m][n] = sum_k A[m][k] W[n][k].
enum Epi : int {
  EPI_STORE = 0,   // out[m][n] = y (fp32)
  EPI_RESID = 1,   // resid[m][n] += y; packed (resid * gain_next) for the next GEMM;
                   // per-workgroup sums of squares for the next RMSNorm
  EPI_SILU = 2,    // packed silu(gate) * up for the down projection (8 gate, 8 up columns per block)
  EPI_QKV = 3,     // RoPE on q/k; q -> attention query fragments, k/v -> paged KV cache
  EPI_LOGITS = 4,  // out[m][n] = logit; per-workgroup (max, sum exp) partials
};

struct GemmArgs {
  // packed weights: [n_groups][Kb][NB][64 lanes][8 bf16], or for column
  // slices [n_groups]{[Kb][NB-1][64 lanes][8 bf16], [Kb][live lanes][8 bf16]}
  const uint16_t* Wp;
  int n_groups;      // one workgroup per group of NB 16-column blocks
  int slice_cols;    // column slices: columns per workgroup (0: whole blocks)
  int Kb;            // K / 32
  int K;
  // A operand: packed rows (see apack_index) of length K
  const uint16_t* Ap;
  const PassRows* rows;
  // Rows of the pass when they are fixed at the time the launch is recorded
  // (a verify pass: K + 1; a later draft step: 1), so the kernel need not
  // wait for the pass descriptor before its first loads; 0: read n_rows from
  // the descriptor.  Only for passes whose descriptor would give the same
  // count (or 0 after a recorded error, when the pass's results are void).
  int fixed_rows;
  int last_row_only;  // use only row n_rows-1 (written as output row 0)
  // RMSNorm of the consumer: y[m][.] *= 1/sqrt(sum_g ssq[g][m] / K + eps)
  const float* ssq;   // [ssq_groups][8] or null (no norm)
  int ssq_groups;
  float eps;
  // epilogue
  float* out;
  int ldo;
  float* resid;       // EPI_RESID: fp32 residual rows [8][ldr]
  int ldr;
  const uint16_t* gain_next;  // EPI_RESID: gain of the next RMSNorm (bf16 [N])
  uint16_t* Ap_out;   // EPI_RESID / EPI_SILU: packed A rows for the next GEMM
  float* ssq_out;     // EPI_RESID: [n_groups][8]
  float2* lm_part;    // EPI_LOGITS: [n_groups][8]
  int n_valid;        // EPI_LOGITS: valid columns (vocab)
  // EPI_QKV: q -> query fragments, k/v -> paged caches
  uint16_t* qf;
  int q_dim, kv_dim, head_dim, n_kv;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* block_table;
  const float2* rope;      // [max_seq][head_dim/2] (cos, sin)
  int max_seq;
  // Optional end stamps: workgroup g writes the device wall clock to
  // ts_end[g] once all its threads have issued their last stores (a plain
  // store per workgroup, no atomics).  Null: off.
  unsigned long long* ts_end;
};

struct GemmShape {
  int nb;        // 16-column blocks per workgroup
  int waves;     // waves per workgroup, splitting K
  int half = 0;  // nb == 1 only: two workgroups per block, 8 columns each
  int slice = 0; // column slices: columns per workgroup, the last of the nb blocks partial
};

// Column slices.  A workgroup owns `slice` consecutive columns: nb - 1 whole
// 16-column blocks and a last block with t = slice - 16 (nb - 1) live
// columns.  For epilogues that pair columns (RoPE halves, gate/up) the unit
// is a pair -- column w and w + 8 of a block -- and the last block holds
// t / 2 pairs, columns w with (w & 7) < t / 2.  The last block is stored
// compacted, only its live lanes (4 per live column, one per 8-value k
// group), so every workgroup reads a contiguous span of exactly its bytes.
enum SliceKind : int { kSliceNone = 0, kSliceCols = 1, kSlicePairs = 2 };
constexpr int kSliceMaxNb = 4;
// Slices only for matrices of at least this many bytes per CU: below it the
// launch's fixed cost dominates and the extra CUs do not pay for the partial
// block's loads (measured: 31B-shaped QKV, O, gate/up and down at 0.23-1.8 MB
// per CU and the 4B-shaped down at 205 KB faster; the 8B-shaped QKV at 197 KB
// and smaller QKV and O projections slower).
constexpr double kSliceMinBytesPerCu = 200e3;

// Lane of the partial block: live, and its index in the compacted k-block.
__host__ __device__ inline bool slice_tail_lane(int lane, int t, bool paired, int* idx) {
  const int w = lane & 15, q = lane >> 4;
  if (paired) {
    const int tp = t >> 1;
    *idx = q * t + (w & 7) + (w >> 3) * tp;
    return (w & 7) < tp;
  }
  *idx = q * t + w;
  return w < t;
}
hipError_t launch_gemm(GemmShape sh, int epi, const GemmArgs& a, hipStream_t s);
// Norm partials each GEMM thread folds: ssq_groups <= waves * 64 / 8 * this.
constexpr int kGemmMaxSsqPerThread = 16;

// Packs a [N][K] bf16 matrix given as row pointers into the MFMA stream
// layout.  row_ptr[(g * nb + j) * 16 + w] (device array) is the row of column
// w of block j of workgroup g, or null (zero row); with column slices
// (slice_cols > 0, paired as the epilogue pairs columns) the dead columns of
// the last block are not stored.
hipError_t launch_pack(const uint16_t* const* row_ptr, int K, int nb, int n_groups, int slice_cols,
                       int paired, uint16_t* out, hipStream_t s);

// ------------------------------------------------------------ GEMM plans --
// One workgroup per group of `nb` 16-column blocks (or per half block),
// `waves` waves splitting K.
struct GemmPlan {
  GemmShape shape{1, 4};
  int n_groups = 0, Kb = 0;
  int workgroups() const { return n_groups * (shape.half ? 2 : 1); }
  // bf16 elements of the packed matrix
  size_t packed_elems() const {
    const size_t per_kb = shape.slice ? (size_t)(shape.nb - 1) * 512 + 32 * (shape.slice - 16 * (shape.nb - 1))
                                      : (size_t)shape.nb * 512;
    return (size_t)n_groups * Kb * per_kb;
  }
};

// Shapes measured on MI355X (graph-replayed sweeps over nb in {1,2,4,7} and
// waves in {4,8,16}, weights cold, with per-workgroup start/end stamps).
// A streaming GEMM is fastest when every CU gets the same number of weight
// bytes and all its workgroups are resident from the start: waves of one CU
// are served oldest first, so on CUs holding one workgroup more than others
// the last one streams alone at the end (896 gate/up workgroups of the 8B
// shape end between 14 and 39 us; 256 workgroups of 7 blocks all end
// together, 37.0 instead of 40.1 us).  So when the column blocks divide
// evenly over the CUs (n_cu > 0) a workgroup takes n_blocks / n_cu of them
// (2, 4, 5 or 7, eight waves from four blocks on).  Otherwise: two blocks per
// workgroup once that still leaves >= 192 workgroups, four waves, except
// for narrow matrices with a long K, where only eight waves per workgroup
// keep enough loads in flight.
//
// A matrix with at most n_cu / 2 column blocks would leave half the CUs
// idle, and one CU streams at most ~35 GB/s: with allow_half each block is
// split between two workgroups of 8 columns (each lane of a wave loads only
// the B-fragment slots of its own half, the others read as zero without a
// fetch), so every CU gets a share.  Not for epilogues that pair columns
// across the halves of a block (RoPE pairs w, w^8; gate/up pairs).
inline GemmPlan plan_gemm(int n_cols, int nb_min, int K, int n_cu, bool allow_half = false,
                          int slice_kind = kSliceNone) {
  GemmPlan p;
  const int n_blocks = n_cols / 16;
  p.Kb = K / 32;
  const int q = n_cu > 0 && n_blocks % n_cu == 0 ? n_blocks / n_cu : 0;
  if ((q == 2 || q == 4 || q == 5 || q == 7) && q >= nb_min) {
    p.shape.nb = q;
    p.n_groups = n_cu;
    p.shape.waves = q >= 4 ? 8 : 4;
    return p;
  }
  p.shape.nb = std::max(nb_min, (n_blocks >= 384 && n_blocks % 2 == 0) ? 2 : 1);
  p.n_groups = n_blocks / p.shape.nb;
  p.shape.waves = (p.n_groups <= 128 && p.Kb >= 256) ? 8 : 4;
  if (allow_half && p.shape.nb == 1 && n_cu > 0 && 2 * n_blocks <= n_cu) p.shape.half = 1;
  // More workgroups than CUs but not a whole number per CU: the CUs that
  // hold one more stream alone at the end.  One equal workgroup per CU on
  // fewer CUs is faster (each CU's share of the bandwidth grows as fewer
  // stream; 1.3B-shaped gate/up, 688 blocks: 344 two-block workgroups
  // 11.3 us, 172 four-block 10.3 us): take the smallest block count that
  // divides the blocks into at most one workgroup per CU.
  if (n_cu > 0 && !p.shape.half && p.workgroups() > n_cu && p.workgroups() % n_cu != 0) {
    for (const int nb : {2, 4, 5, 7}) {
      if (nb < nb_min || n_blocks % nb || n_blocks / nb > n_cu) continue;
      p.shape.nb = nb;
      p.n_groups = n_blocks / nb;
      p.shape.waves = nb >= 5 ? 8 : 4;  // five and seven blocks are built with eight waves only
      break;
    }
  }
  // Still not a whole number of workgroups per CU, and a large matrix:
  // column slices, r workgroups per CU with n_cols / (r n_cu) columns each,
  // the smallest r that keeps a workgroup within kSliceMaxNb blocks.
  if (slice_kind != kSliceNone && n_cu > 0 && p.workgroups() % n_cu != 0 &&
      2.0 * n_cols * K / n_cu >= kSliceMinBytesPerCu) {
    for (int r = 1; r <= 8; ++r) {
      const int G = r * n_cu;
      if (n_cols % G) continue;
      const int cw = n_cols / G;
      if (cw % 16 == 0 || (slice_kind == kSlicePairs && cw % 2)) continue;
      const int nb = (cw + 15) / 16;
      if (nb > kSliceMaxNb || nb < nb_min) continue;
      p.shape = GemmShape{nb, 4, 0, cw};
      p.n_groups = G;
      break;
    }
  }
  return p;
}

}  // namespace spec
