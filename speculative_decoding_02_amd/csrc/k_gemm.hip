// k_gemm.hip -- weight-streaming skinny GEMM for the verify pass on gfx950.
//
// Y[m][n] = sum_k A[m][k] * W[n][k] for up to 8 activation rows m (the K+1
// verify positions, or 1-2 draft rows) against a bf16 weight matrix W that is
// read from HBM exactly once.  A pass over K+1 positions costs about one
// weight read, the premise of the method ([en] Floor 3; [int] "why it is
// faster"): the work is bandwidth-bound, so the kernel is built around
// streaming W.
//
//  * W is repacked once (launch_pack) so that each 16-byte lane load of a
//    wave is one B fragment of v_mfma_f32_16x16x32_bf16 and a wave's k-range
//    is one contiguous span: [group][k-block][NB][64 lanes][8 bf16].
//  * A arrives already packed by its producer (see apack_index): bf16 high
//    and low halves of up to 8 fp32 rows in one 16-row MFMA tile, each row's
//    32 values of a k-block contiguous.  It is small and shared by every
//    workgroup, so it is read from L2; lanes of rows the pass does not use
//    are given an out-of-range buffer offset, which reads as zero without a
//    memory access.
//  * A workgroup owns NB 16-column blocks for the whole of K; its waves split
//    K and are reduced through LDS in wave order (deterministic, and no
//    workgroup ever waits for another).
//  * RMSNorm is folded in: the producer packs x * gain, and the row scale
//    1/sqrt(mean(x^2) + eps) multiplies Y here, from per-workgroup sums of
//    squares published by the producer.
#include <type_traits>

#include "k_gemm.h"

namespace spec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

SPEC_DEVICE bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// DPP move of a float within 16-lane rows (all lanes active, bound_ctrl on).
template <int CTRL>
SPEC_DEVICE float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

SPEC_DEVICE uint4 load_stream(const uint4* p) {
  // weights are read once per pass: non-temporal hint
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// HALF (NB == 1): workgroup 2b + h owns columns 8h .. 8h + 7 of block b.
// SLICE: workgroup g owns the column slice g (a.slice_cols columns, see
// GemmShape): NB - 1 whole blocks and a compacted partial block.
// Everything the first weight and activation loads need leads the arguments
// as scalars (preloaded in SGPRs with the wave instead of loaded from the
// argument segment), and the row count is one of them whenever the pass's
// row count is fixed when the launch is recorded (fixed_rows > 0; 0: read it
// from the pass descriptor).  In most instances the first batch of loads is
// issued before anything else, so it waits on no memory access; the norm
// partials and epilogue operands are fetched behind it and the partials are
// folded only after the main loop.
template <int NB, int W, int EPI, bool HALF, bool SLICE>
__global__ __launch_bounds__(W * 64) void gemm_skinny(const PassRows* rows, const uint16_t* Wp,
                                                     const uint16_t* Ap, const float* ssq, int Kb,
                                                     int fixed_rows, int ssq_groups, int slice_cols,
                                                     int last_row_only, GemmArgs a) {
  static_assert(!HALF || (NB == 1 && EPI != EPI_SILU && EPI != EPI_QKV),
                "half blocks split column pairs of the SiLU and RoPE epilogues");
  static_assert(!SLICE || (!HALF && (EPI == EPI_RESID || EPI == EPI_QKV || EPI == EPI_SILU)),
                "column slices for the residual, QKV and SiLU epilogues");
  constexpr int YW = HALF ? 8 : NB * 16;  // columns owned by the workgroup
  constexpr int U = NB == 1 ? 16 : (NB == 2 ? 8 : (NB <= 4 ? 4 : 2));  // k-blocks per batch
  __shared__ float s_red[W * NB * 128];
  __shared__ float s_y[(EPI == EPI_STORE || EPI == EPI_LOGITS) ? kMaxRows * YW : 1];
  __shared__ float s_ssq[W * kMaxRows];
  __shared__ float s_part[kMaxRows][(EPI == EPI_RESID && YW > 16) ? YW / 16 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = blockIdx.x;                 // workgroup: stamps and partial outputs
  const int gb = HALF ? g >> 1 : g;         // column group of the packed weights
  const int hc = HALF ? (g & 1) * 8 : 0;    // first column of the half within its block
  constexpr bool PAIRED = EPI == EPI_QKV || EPI == EPI_SILU;  // epilogues on column pairs
  constexpr int NBF = SLICE ? NB - 1 : NB;  // whole 16-column blocks of the workgroup
  const int cw = SLICE ? slice_cols : 0;    // columns of a slice
  const int tcols = SLICE ? cw - 16 * NBF : 0;  // live columns of its partial block
  // column c of the workgroup (block c / 16, MFMA column c % 16) holds an output
  auto live_col = [&](int c) -> bool {
    if constexpr (!SLICE) return true;
    else if constexpr (PAIRED) return (c >> 4) < NBF || (c & 7) < (tcols >> 1);
    else return c < cw;
  };
  // first pair (RoPE pair, gate/up feature) of the workgroup
  const int pair0 = SLICE ? g * (cw >> 1) : gb * NB * 8;
  int n_rows = fixed_rows;
  if (n_rows <= 0) n_rows = rows->n_rows;
  int row_base = 0;
  if (last_row_only) {
    row_base = n_rows - 1;
    n_rows = n_rows > 0 ? 1 : 0;
  }

  // ---- main-loop operands: this wave's share of K ------------------------
  const int kb0 = (Kb * wave) / W, kb1 = (Kb * (wave + 1)) / W;
  const int am = lane & 7;  // activation row of this lane (hi rows 0-7, lo rows 8-15)
  const bool aload = last_row_only ? (am == row_base) : (am < n_rows);
  // A through a range-checked buffer resource: lanes of rows the pass does not
  // use read at an out-of-range offset, which returns zero without a fetch.
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Ap), 0, Kb * 1024, 0x00020000);
  const uint32_t a_off = aload ? apack_lane_offset(lane) : 0x80000000u;
  // 16-byte units of one workgroup's weights
  const size_t g_u4 = SLICE ? (size_t)Kb * (NBF * 64 + 4 * tcols) : (size_t)Kb * NB * 64;
  const uint4* wp = (const uint4*)Wp + (size_t)(SLICE ? g : gb) * g_u4 + lane;
  // Half blocks: lanes of the other half's columns read at an out-of-range
  // offset of a buffer resource over the group's weights (zero, no fetch);
  // aux bit 1 is the non-temporal hint.
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(wp - lane), 0, HALF ? Kb * NB * 1024 : 0, 0x00020000);
  const uint32_t w_off = (unsigned)((lane & 15) - hc) < 8u ? (uint32_t)lane * 16 : 0x80000000u;
  // Slices: the partial block's k-blocks follow the whole blocks, 4 * tcols
  // lanes each; dead lanes read at an out-of-range offset (zero, no fetch).
  int t_ci = 0;
  const bool t_live = SLICE && slice_tail_lane(lane, tcols, PAIRED, &t_ci);
  const __amdgpu_buffer_rsrc_t rT = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(wp - lane + (size_t)Kb * NBF * 64), 0, SLICE ? Kb * 64 * tcols : 0, 0x00020000);
  const uint32_t t_off = t_live ? (uint32_t)t_ci * 16 : 0x80000000u;
  floatx4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Batches of k-blocks: all loads of a batch are issued before its first
  // MFMA (the scheduling barrier keeps the compiler from interleaving them),
  // so each wave keeps UB*NB KiB of weights in flight.
  auto load_batch = [&](auto ub_tag, int kb, uint4* av, uint4 (*wv)[NB]) {
    constexpr int UB = decltype(ub_tag)::value;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
          rA, (int)(aload ? a_off + (uint32_t)(kb + u) * 1024 : a_off), 0, 0);
      av[u] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if constexpr (HALF) {
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
              rW, (int)(w_off < 0x80000000u ? w_off + (uint32_t)((kb + u) * NB + j) * 1024 : w_off), 0,
              2);
          wv[u][j] = make_uint4(v.x, v.y, v.z, v.w);
        } else if (j < NBF) {
          wv[u][j] = load_stream(wp + ((size_t)(kb + u) * NBF + j) * 64);
        } else {
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
              rT, (int)(t_off < 0x80000000u ? t_off + (uint32_t)(kb + u) * 64 * tcols : t_off), 0, 2);
          wv[u][j] = make_uint4(v.x, v.y, v.z, v.w);
        }
      }
  };
  auto mma_batch = [&](auto ub_tag, const uint4* av, const uint4 (*wv)[NB]) {
    constexpr int UB = decltype(ub_tag)::value;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), as_bf16x8(wv[u][j]),
                                                         acc[j], 0, 0, 0);
    }
  };
  auto batch = [&](auto ub_tag, int kb) {
    constexpr int UB = decltype(ub_tag)::value;
    uint4 av[UB], wv[UB][NB];
    load_batch(ub_tag, kb, av, wv);
    __builtin_amdgcn_sched_barrier(0);
    mma_batch(ub_tag, av, wv);
  };
  // The first full batch is issued now, ahead of every other load (where
  // that is faster, see kPeel).
  uint4 av0[U], wv0[U][NB];
  // Issuing the first batch ahead of the prologue was measured per instance
  // (rocprofv3 kernel traces of graph-replayed rounds): it shortens the
  // half-block, the four-and-more-block and the one-block QKV launches by
  // 0.15-0.5 us and lengthens the whole-block residual launches with one block
  // (8B-shaped O and down, +2.2 us) and the two-block QKV (+0.4 us), which
  // therefore issue it in the loop as before.
  constexpr bool kPeel = HALF || NB >= 4 || (EPI == EPI_QKV && NB == 1);
  const bool peel = kPeel && kb0 + U <= kb1;  // wave-uniform
  if (peel) load_batch(std::integral_constant<int, U>{}, kb0, av0, wv0);
  __builtin_amdgcn_sched_barrier(0);

  // Row scale of the consumer's RMSNorm.  The producer's partial sums of
  // squares are spread over all threads (thread t: row t%8, partials
  // q = t/8, t/8 + P, ...), loaded here and folded in a fixed order after the
  // main loop.  The loads are unconditional (clamped indices) so they wait
  // for nothing; entries outside the pass are dropped when folded.
  constexpr int P = W * 64 / kMaxRows;
  constexpr int kMaxSsq = kGemmMaxSsqPerThread;  // ssq_groups <= P * kMaxSsq
  const int ssq_m = tid % kMaxRows, ssq_p0 = tid / kMaxRows;
  float ssq_v[kMaxSsq];
  if (ssq != nullptr) {
    const int mr = last_row_only ? row_base : ssq_m;  // row of the producer's partials
#pragma unroll
    for (int i = 0; i < kMaxSsq; ++i) {
      const int q = ssq_p0 + i * P;
      ssq_v[i] = ssq[(q < ssq_groups ? q : 0) * kMaxRows + (mr & (kMaxRows - 1))];
    }
  }

  // Epilogue operands that do not depend on the product, fetched now so their
  // latency hides behind the weight stream (the gains stay bf16 until used).
  const int col0 = SLICE ? g * cw : gb * NB * 16 + hc;
  // residual epilogue: item i = tid + i*W*64 is (row i / YW, column i % YW)
  constexpr int RI = EPI == EPI_RESID ? (kMaxRows * YW + W * 64 - 1) / (W * 64) : 1;
  float pre_x[RI];
  uint16_t pre_gn[RI];
#pragma unroll
  for (int i = 0; i < RI; ++i) {
    pre_x[i] = 0.0f;
    pre_gn[i] = 0;
    const int idx = tid + i * W * 64;
    if (EPI == EPI_RESID && idx < kMaxRows * YW && live_col(idx % YW)) {  // resid rows exist for all kMaxRows rows
      const int k = col0 + idx % YW;
      pre_x[i] = a.resid[(size_t)(idx / YW) * a.ldr + k];
      pre_gn[i] = a.gain_next[k];
    }
  }
  float2 pre_rope = make_float2(1.f, 0.f);
  int pre_blk = 0;
  if constexpr (EPI == EPI_QKV) {
    const int m = tid / YW, c = tid % YW;
    const int pos = rows->pos0 + m;
    const int P = pair0 + (c >> 4) * 8 + (c & 7);  // pair of the projection's q, k, v pairs
    const int q_pairs = a.q_dim / 2, qk_pairs = (a.q_dim + a.kv_dim) / 2, half_hd = a.head_dim / 2;
    if (m < kMaxRows && pos < a.max_seq) {
      pre_blk = a.block_table[pos / kBlock];
      if (P < qk_pairs && live_col(c)) pre_rope = a.rope[(size_t)pos * half_hd + (P < q_pairs ? P : P - q_pairs) % half_hd];
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- main loop -----------------------------------------------------------
  int kb = kb0;
  if (peel) {
    mma_batch(std::integral_constant<int, U>{}, av0, wv0);
    kb += U;
  }
  for (; kb + U <= kb1; kb += U) batch(std::integral_constant<int, U>{}, kb);
  for (; kb + 4 <= kb1; kb += 4) batch(std::integral_constant<int, 4>{}, kb);
  for (; kb < kb1; ++kb) batch(std::integral_constant<int, 1>{}, kb);

  float ssq_part = 0.0f;
  if (ssq != nullptr) {
#pragma unroll
    for (int i = 0; i < kMaxSsq; ++i)
      ssq_part += (ssq_p0 + i * P < ssq_groups && ssq_m < n_rows) ? ssq_v[i] : 0.0f;
  }

  // ---- hi + lo rows, then the waves' partial sums in wave order ----------
  // MFMA output: lane l, element r is (row 4*(l/16)+r, column l%16); lanes
  // 32-63 hold the low-part products of the rows of lanes 0-31.  Each lane
  // swaps its accumulators with lane l^32 (v_permlane32_swap) and lanes 0-31
  // publish hi + lo, so the cross-wave sum reads one value per wave.
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    float hl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float f = acc[j][r];  // bit_cast straight off a vector element reads element 0
      const uint32_t u = __builtin_bit_cast(uint32_t, f);
      const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      const uint32_t hi = p[0], lo = p[1];
      hl[r] = __builtin_bit_cast(float, hi) + __builtin_bit_cast(float, lo);
    }
    if (lane < 32)
      *(float4*)&s_red[((wave * NB + j) * 32 + lane) * 4] = make_float4(hl[0], hl[1], hl[2], hl[3]);
  }
  // sums of squares: lanes of one wave with the same row (lane % 8) first
  float sq = ssq_part;
  sq += __shfl_xor(sq, 8);
  sq += __shfl_xor(sq, 16);
  sq += __shfl_xor(sq, 32);
  if (lane < kMaxRows) s_ssq[wave * kMaxRows + lane] = sq;
  __syncthreads();

  // From here each thread produces its own outputs straight from the wave
  // partials: output row m (MFMA row mm, which differs only with
  // last_row_only) and column cb of the workgroup's NB*16 block columns.
  auto row_scale = [&](int m) -> float {
    if (ssq == nullptr || m >= n_rows) return 1.0f;
    float ss = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) ss += s_ssq[w * kMaxRows + m];
    return 1.0f / sqrtf(ss / (float)a.K + a.eps);
  };
  auto col_sum = [&](int mm, int cb) -> float {
    const int ln = (mm >> 2) * 16 + (cb & 15), r = mm & 3, j = cb >> 4;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += s_red[((w * NB + j) * 32 + ln) * 4 + r];
    return v;
  };
  auto src_row = [&](int m) { return last_row_only ? row_base : m; };

  // ---- epilogues -------------------------------------------------------------
  if constexpr (EPI == EPI_STORE || EPI == EPI_LOGITS) {
    for (int idx = tid; idx < n_rows * YW; idx += W * 64) {
      const int m = idx / YW, c = idx % YW;
      s_y[m * YW + c] = col_sum(src_row(m), c + hc) * row_scale(m);
    }
    __syncthreads();
  }
  if constexpr (EPI == EPI_STORE) {
    for (int idx = tid; idx < n_rows * YW; idx += W * 64) {
      const int m = idx / YW, c = idx % YW;
      a.out[(size_t)m * a.ldo + col0 + c] = s_y[m * YW + c];
    }
  } else if constexpr (EPI == EPI_LOGITS) {
    for (int idx = tid; idx < n_rows * YW; idx += W * 64) {
      const int m = idx / YW, c = idx % YW;
      if (col0 + c < a.n_valid) a.out[(size_t)m * a.ldo + col0 + c] = s_y[m * YW + c];
    }
    if (tid < kMaxRows) {
      const int m = tid;
      float M = -INFINITY, S = 0.0f;
      if (m < n_rows) {
        for (int c = 0; c < YW; ++c)
          if (col0 + c < a.n_valid) M = fmaxf(M, s_y[m * YW + c]);
        for (int c = 0; c < YW; ++c)
          if (col0 + c < a.n_valid) S += expf(s_y[m * YW + c] - M);
      }
      a.lm_part[g * kMaxRows + m] = make_float2(M, S);
    }
  } else if constexpr (EPI == EPI_RESID) {
    // x += y; next GEMM's packed A = x * gain_next; sums of squares of x.
    // One element per item: a row's elements sit on consecutive lanes, 16
    // (or, for half blocks, 8) to an aligned 16-lane DPP row.
    static_assert(YW == 8 || YW % 16 == 0, "rows fill whole DPP rows or half rows");
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const int idx = tid + i * W * 64, m = idx / YW, c = idx % YW;
      float sq = 0.0f;
      if (idx < kMaxRows * YW && m < n_rows && live_col(c)) {
        const float x = pre_x[i] + col_sum(src_row(m), c + hc) * row_scale(m);
        a.resid[(size_t)m * a.ldr + col0 + c] = x;
        apack_store1(a.Ap_out, m, col0 + c, x * bf16_to_f32(pre_gn[i]));
        sq = x * x;
      }
      // sum over the lanes of one row (up to 16), fixed order: quads, then
      // pairs of quads (row_half_mirror pairs quad 0 with 1 and 2 with 3),
      // then the two halves
      sq += dpp_f32<0xb1>(sq);   // quad_perm [1,0,3,2]: lane l^1
      sq += dpp_f32<0x4e>(sq);   // quad_perm [2,3,0,1]: lane l^2
      sq += dpp_f32<0x141>(sq);  // row_half_mirror: the other quad of the 8-lane half
      if constexpr (YW >= 16) sq += dpp_f32<0x128>(sq);  // row_ror:8: the other half
      if (idx < kMaxRows * YW && (c & 15) == 0) {
        if constexpr (YW <= 16) a.ssq_out[g * kMaxRows + m] = sq;
        else s_part[m][c >> 4] = sq;
      }
    }
    if constexpr (YW > 16) {
      __syncthreads();
      if (tid < kMaxRows) {
        float s2 = 0.0f;
        for (int q = 0; q < YW / 16; ++q) s2 += s_part[tid][q];
        a.ssq_out[g * kMaxRows + tid] = s2;
      }
    }
  } else if constexpr (EPI == EPI_SILU) {
    // block b = gb*NB + j: columns 0-7 are the gate and 8-15 the up outputs of
    // features 8b .. 8b+7; one feature per thread
    for (int idx = tid; idx < n_rows * NB * 8; idx += W * 64) {
      const int m = idx / (NB * 8), f = idx % (NB * 8), j = f >> 3, e = f & 7;
      if (SLICE && f >= (cw >> 1)) continue;
      const float sc = row_scale(m);
      const float gt = col_sum(src_row(m), j * 16 + e) * sc;
      const float up = col_sum(src_row(m), j * 16 + 8 + e) * sc;
      apack_store1(a.Ap_out, m, pair0 + f, gt / (1.0f + expf(-gt)) * up);
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int q_pairs = a.q_dim / 2, qk_pairs = (a.q_dim + a.kv_dim) / 2;
    const int half_hd = a.head_dim / 2;
    const int G = div_small(a.q_dim, rcp_small(a.kv_dim)), n_es = (a.head_dim + 31) / 32;
    const float inv_half = rcp_small(half_hd), inv_hd = rcp_small(a.head_dim), inv_G = rcp_small(G);
    const int pos0 = rows->pos0;
    for (int idx = tid; idx < n_rows * YW; idx += W * 64) {
      const int m = idx / YW, c = idx % YW;
      const int w = c & 15, hf = w >> 3;
      const int P = pair0 + (c >> 4) * 8 + (w & 7);
      const int pos = pos0 + m;
      if (pos >= a.max_seq || !live_col(c)) continue;
      const float sc = row_scale(m);
      const float mine = col_sum(src_row(m), c) * sc;
      if (P < qk_pairs) {
        // pair-interleaved block: columns w and w^8 are the two halves of one pair
        const bool is_q = P < q_pairs;
        const int pair = is_q ? P : P - q_pairs;
        const int head = div_small(pair, inv_half), jj = pair - head * half_hd;
        const float other = col_sum(src_row(m), c ^ 8) * sc;
        // (cos, sin) of pos * theta^(-2jj/hd); this thread's first item was prefetched
        const float2 r = idx == tid ? pre_rope : a.rope[(size_t)pos * half_hd + jj];
        const float lo = hf ? other : mine;
        const float hi = hf ? mine : other;
        const float val = hf ? hi * r.x + lo * r.y : lo * r.x - hi * r.y;
        const int dim = jj + hf * half_hd;
        if (is_q) {
          const int h_kv = div_small(head, inv_G), qi = m * G + (head - h_kv * G);
          const uint16_t hb = f32_to_bf16_rne(val);
          a.qf[qfrag_index(h_kv, G, n_es, qi, 0, dim)] = hb;
          a.qf[qfrag_index(h_kv, G, n_es, qi, 1, dim)] = f32_to_bf16_rne(val - bf16_to_f32(hb));
        } else {
          const int blk = idx == tid ? pre_blk : a.block_table[pos / kBlock];
          const uint16_t hb = f32_to_bf16_rne(val);
          a.k_cache[kv_index(blk, a.n_kv, head, pos % kBlock, a.head_dim, 0, dim)] = hb;
          a.k_cache[kv_index(blk, a.n_kv, head, pos % kBlock, a.head_dim, 1, dim)] =
              f32_to_bf16_rne(val - bf16_to_f32(hb));
        }
      } else {
        // v: pair pv covers features w and w + 8 of block pv / 8
        const int pv = P - qk_pairs;
        const int f0 = (pv >> 3) * 16 + (pv & 7) + 8 * hf;
        const int head = div_small(f0, inv_hd), dim = f0 - head * a.head_dim;
        const int blk = idx == tid ? pre_blk : a.block_table[pos / kBlock];
        const uint16_t hb = f32_to_bf16_rne(mine);
        a.v_cache[vt_index(blk, a.n_kv, head, 0, a.head_dim, dim, pos % kBlock)] = hb;
        a.v_cache[vt_index(blk, a.n_kv, head, 1, a.head_dim, dim, pos % kBlock)] =
            f32_to_bf16_rne(mine - bf16_to_f32(hb));
      }
    }
  }
  if (a.ts_end != nullptr) {
    __syncthreads();
    if (tid == 0) a.ts_end[g] = (unsigned long long)wall_clock64();
  }
}

template <int NB, int W, bool HALF = false, bool SLICE = false>
static hipError_t launch_epi(int epi, const GemmArgs& a, hipStream_t s) {
  const dim3 grid(a.n_groups * (HALF ? 2 : 1)), block(W * 64);
  if constexpr (SLICE) {
    switch (epi) {
      case EPI_RESID: hipLaunchKernelGGL((gemm_skinny<NB, W, EPI_RESID, false, true>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      case EPI_QKV: hipLaunchKernelGGL((gemm_skinny<NB, W, EPI_QKV, false, true>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      case EPI_SILU: hipLaunchKernelGGL((gemm_skinny<NB, W, EPI_SILU, false, true>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      default: return hipErrorInvalidValue;
    }
  } else if constexpr (HALF) {
    switch (epi) {
      case EPI_STORE: hipLaunchKernelGGL((gemm_skinny<1, W, EPI_STORE, true, false>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      case EPI_RESID: hipLaunchKernelGGL((gemm_skinny<1, W, EPI_RESID, true, false>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      case EPI_LOGITS: hipLaunchKernelGGL((gemm_skinny<1, W, EPI_LOGITS, true, false>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (epi) {
      case EPI_STORE: hipLaunchKernelGGL((gemm_skinny<NB, W, EPI_STORE, false, false>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      case EPI_RESID: hipLaunchKernelGGL((gemm_skinny<NB, W, EPI_RESID, false, false>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      case EPI_QKV: hipLaunchKernelGGL((gemm_skinny<NB, W, EPI_QKV, false, false>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      case EPI_LOGITS: hipLaunchKernelGGL((gemm_skinny<NB, W, EPI_LOGITS, false, false>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      case EPI_SILU: hipLaunchKernelGGL((gemm_skinny<NB, W, EPI_SILU, false, false>), grid, block, 0, s, a.rows, a.Wp, a.Ap, a.ssq, a.Kb, a.fixed_rows, a.ssq_groups, a.slice_cols, a.last_row_only, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm(GemmShape sh, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.slice_cols != sh.slice) return hipErrorInvalidValue;
  if (sh.slice) {
    // nb - 1 whole blocks and a partial one; pairs stay whole
    const bool paired = epi == EPI_QKV || epi == EPI_SILU;
    if (sh.half || sh.waves != 4 || sh.slice <= 16 * (sh.nb - 1) || sh.slice >= 16 * sh.nb ||
        (paired && sh.slice % 2))
      return hipErrorInvalidValue;
    if (sh.nb == 1) return launch_epi<1, 4, false, true>(epi, a, s);
    if (sh.nb == 2) return launch_epi<2, 4, false, true>(epi, a, s);
    if (sh.nb == 3) return launch_epi<3, 4, false, true>(epi, a, s);
    if (sh.nb == 4) return launch_epi<4, 4, false, true>(epi, a, s);
    return hipErrorInvalidValue;
  }
  if (sh.half) {
    if (sh.nb != 1) return hipErrorInvalidValue;
    if (sh.waves == 4) return launch_epi<1, 4, true>(epi, a, s);
    if (sh.waves == 8) return launch_epi<1, 8, true>(epi, a, s);
    return hipErrorInvalidValue;
  }
  if (sh.waves == 4) {
    if (sh.nb == 1) return launch_epi<1, 4>(epi, a, s);
    if (sh.nb == 2) return launch_epi<2, 4>(epi, a, s);
    if (sh.nb == 4) return launch_epi<4, 4>(epi, a, s);
  } else if (sh.waves == 8) {
    if (sh.nb == 1) return launch_epi<1, 8>(epi, a, s);
    if (sh.nb == 2) return launch_epi<2, 8>(epi, a, s);
    if (sh.nb == 4) return launch_epi<4, 8>(epi, a, s);
    if (sh.nb == 5) return launch_epi<5, 8>(epi, a, s);
    if (sh.nb == 7) return launch_epi<7, 8>(epi, a, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ pack --
// row_ptr lists the workgroups' column slots, (g * nb + j) * 16 + w; with
// column slices (cw > 0) the dead slots of the last block are not stored.
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* const* row_ptr, int K, int nb,
                                                   int n_groups, int cw, int paired, uint16_t* out) {
  const int Kb = K / 32;
  const size_t total = (size_t)n_groups * Kb * nb * 64;
  const int nbf = cw ? nb - 1 : nb, t = cw ? cw - 16 * nbf : 0;
  const size_t per_g = (size_t)Kb * (nbf * 64 + 4 * t);  // 16-byte units per workgroup
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx % 64);
    const int j = (int)((idx / 64) % nb);
    const int kb = (int)((idx / (64 * (size_t)nb)) % Kb);
    const size_t g = idx / (64 * (size_t)nb * Kb);
    const size_t n = (g * nb + j) * 16 + (lane & 15);
    const int k = kb * 32 + (lane >> 4) * 8;
    size_t dst;
    if (j < nbf) {
      dst = g * per_g + ((size_t)kb * nbf + j) * 64 + lane;
    } else {
      int ci;
      if (!slice_tail_lane(lane, t, paired != 0, &ci)) continue;
      dst = g * per_g + (size_t)Kb * nbf * 64 + (size_t)kb * 4 * t + ci;
    }
    const uint16_t* src = row_ptr[n];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src != nullptr) v = *(const uint4*)(src + k);
    ((uint4*)out)[dst] = v;
  }
}

hipError_t launch_pack(const uint16_t* const* row_ptr, int K, int nb, int n_groups, int slice_cols,
                       int paired, uint16_t* out, hipStream_t s) {
  if (slice_cols && (slice_cols <= 16 * (nb - 1) || slice_cols >= 16 * nb || (paired && slice_cols % 2)))
    return hipErrorInvalidValue;
  const size_t total = (size_t)n_groups * (K / 32) * nb * 64;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, row_ptr, K, nb, n_groups,
                     slice_cols, paired, out);
  return hipGetLastError();
}

}  // namespace spec
