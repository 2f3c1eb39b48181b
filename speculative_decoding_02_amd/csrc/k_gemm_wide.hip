// k_gemm_wide.hip -- the rows GEMM of a batched verify pass past 8
// activation rows (k_gemm_rows.hip covers up to 8 and packs the operand):
// Y[m][n] = sum_k X[m][k] W[n][k] against the same packed bf16 weight stream,
// the activations in the row tiles k_gemm_rows.hip describes.  Built with
// VGPR-form MFMAs (each accumulator stays in the VGPRs its MFMA writes), which
// keeps the compiler from copying the accumulators between register files at
// every k-block.
#include "kernels.h"

namespace spec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ wide kernel --
// For more than 8 rows the activation tiles outweigh the weights a
// workgroup streams (RT KiB of A per k-block against NB KiB of W), so here
// the four waves split the workgroup's 128 columns (two 16-column blocks
// each) and share the A tiles: the workgroup copies U k-blocks of tiles
// into LDS (double-buffered), every wave reads them from there, and streams
// only its own weight fragments, one stage ahead.  Each wave owns whole
// output columns, so no cross-wave reduction is needed.  In LDS the tiles
// are regrouped by pairs: the high parts of activation rows 16p .. 16p+15
// form one MFMA operand and their low parts another, and both multiply the
// same weight fragment into one accumulator -- the high and low halves are
// summed along K, not as separate output rows, which halves the
// accumulators per wave and leaves registers for a whole k-block of
// operands to be read from LDS before its MFMAs.  Workgroup
// (g, s) covers k-slice s; with S > 1 slices it writes fp32 partials P[s]
// and rows_reduce_kernel sums them in slice order.
constexpr int kWideCB = 2;       // 16-column blocks per wave
constexpr int kWideWaves = 4;
static_assert(kWideCB * 16 * kWideWaves == kRowsWideCols, "wide tile");

template <int RT>
struct WideStage {
  static constexpr int U = RT >= 16 ? 2 : (RT >= 8 ? 4 : 8);  // k-blocks per stage
  static constexpr int A16 = U * RT * 64;                     // 16-byte words of A per stage
  static constexpr int PER_THREAD = A16 / (kWideWaves * 64);
};

template <int RT>
__global__ __launch_bounds__(kWideWaves * 64) void gemm_wide_kernel(
    const uint16_t* Wp, int nb, const uint16_t* A, int Kb, int S, float* Y, int M, int ldy,
    int accumulate, float* P, int N) {
  using St = WideStage<RT>;
  constexpr int U = St::U;
  __shared__ u32x4_t s_a[2][St::A16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sl = blockIdx.y;
  const int kb0 = (Kb * sl) / S, kb1 = (Kb * (sl + 1)) / S;
  const int cb0 = blockIdx.x * (kWideCB * kWideWaves) + wave * kWideCB;
  const u32x4_t* wb[kWideCB];
#pragma unroll
  for (int j = 0; j < kWideCB; ++j) {
    const int cb = cb0 + j;
    wb[j] = (const u32x4_t*)Wp + ((size_t)(cb / nb) * Kb * nb + (cb % nb)) * 64 + lane;
  }
  const size_t wstep = (size_t)nb * 64;  // 16-byte words between k-blocks of one block
  const u32x4_t* ag = (const u32x4_t*)A;

  constexpr int RP = RT / 2;  // 16-row output tiles (tile pairs)
  static_assert(RT % 2 == 0, "row tiles come in pairs");
  floatx4 acc[RP][kWideCB];
#pragma unroll
  for (int t = 0; t < RP; ++t)
#pragma unroll
    for (int j = 0; j < kWideCB; ++j) acc[t][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // native vectors throughout (the uint4 struct would be copied through
  // private memory)
  constexpr int NW = 3;  // weight register sets: loads run two stages ahead
  u32x4_t areg[St::PER_THREAD];
  u32x4_t wr[NW][U][kWideCB];
  auto load_a = [&](int k) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < St::PER_THREAD; ++i) {
      const int w = tid + i * kWideWaves * 64;
      const int kk = min(k + w / (RT * 64), kb1 - 1);
      areg[i] = ag[(size_t)kk * RT * 64 + w % (RT * 64)];
    }
  };
  // Global word (k-block u, tile t, lane l) holds MFMA row i = l % 16 of
  // tile t (i < 8: high part of activation row 8t + i, else the low part of
  // row 8t + i - 8) for k group l / 16.  In LDS it goes to operand
  // (u, pair t / 2, high or low) at lane 16 (l / 16) + 8 (t % 2) + i % 8.
  auto store_a = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < St::PER_THREAD; ++i) {
      const int w = tid + i * kWideWaves * 64;
      const int l = w & 63, t = (w >> 6) % RT, u = w / (RT * 64);
      const int ri = l & 15, dst = (((u * RP + (t >> 1)) * 2 + (ri >> 3)) << 6) + (l & 48) + ((t & 1) << 3) + (ri & 7);
      s_a[buf][dst] = areg[i];
    }
  };
  auto load_w = [&](u32x4_t (&w)[U][kWideCB], int k) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < kWideCB; ++j) {
        const int kk = min(k + u, kb1 - 1);
        w[u][j] = __builtin_nontemporal_load(wb[j] + (size_t)kk * wstep);
      }
  };
  auto compute = [&](int buf, const u32x4_t (&w)[U][kWideCB], int nu) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4_t av[RP][2];  // the k-block's operands, all read before its MFMAs
#pragma unroll
      for (int p = 0; p < RP; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) av[p][h] = s_a[buf][((u * RP + p) * 2 + h) * 64 + lane];
      u32x4_t wz[kWideCB];
#pragma unroll
      for (int j = 0; j < kWideCB; ++j) wz[j] = u < nu ? w[u][j] : u32x4_t{0u, 0u, 0u, 0u};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int p = 0; p < RP; ++p)
#pragma unroll
          for (int j = 0; j < kWideCB; ++j)
            acc[p][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, av[p][h]), __builtin_bit_cast(bf16x8_t, wz[j]),
                acc[p][j], 0, 0, 0);
    }
  };

  // Stage s computes from LDS buffer s % 2 and weight set s % 3; it first
  // issues the activation tiles of stage s + 1 (copied into the idle buffer
  // after its MFMAs) and the weights of stage s + 2, so the weight stream runs
  // two stages ahead.  Loads are unconditional (past the slice they repeat
  // its last k-block), six stages per trip keep every register index static,
  // and all branches are uniform over the workgroup.
  load_w(wr[0], kb0);
  load_w(wr[1], kb0 + U);
  load_a(kb0);
  store_a(0);
  __syncthreads();
  int k = kb0;
  bool done = false;
  while (!done) {
#pragma unroll
    for (int p = 0; p < 6; ++p) {
      if (!done) {
        load_a(k + U);
        load_w(wr[(p + 2) % NW], k + 2 * U);
        __builtin_amdgcn_sched_barrier(0);  // loads go out before this stage computes
        compute(p % 2, wr[p % NW], min(U, kb1 - k));
        store_a((p + 1) % 2);
        __syncthreads();
        k += U;
        done = k >= kb1;
      }
    }
  }

  // MFMA output: lane l, element r is row 4 (l / 16) + r of the pair's 16
  // activation rows, column l % 16.
#pragma unroll
  for (int t = 0; t < RP; ++t)
#pragma unroll
    for (int j = 0; j < kWideCB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        {
          const float v = acc[t][j][r];
          const int m = 16 * t + 4 * (lane >> 4) + r;
          const int col = (cb0 + j) * 16 + (lane & 15);
          if (m < M) {
            if (S > 1) {
              P[((size_t)sl * M + m) * N + col] = v;
            } else {
              float* y = Y + (size_t)m * ldy + col;
              *y = accumulate ? *y + v : v;
            }
          }
        }
      }
}

// Y (=, +=) sum over slices of P[s], in slice order.
__global__ __launch_bounds__(256) void rows_reduce_kernel(const float* P, int S, int M, int N,
                                                          float* Y, int ldy, int accumulate) {
  const size_t total = (size_t)M * N;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    float v = P[i];
    for (int s = 1; s < S; ++s) v += P[(size_t)s * total + i];
    const int m = (int)(i / N), n = (int)(i % N);
    float* y = Y + (size_t)m * ldy + n;
    *y = accumulate ? *y + v : v;
  }
}

hipError_t launch_gemm_wide(const RowsGemmArgs& a, int RT, int ldy, hipStream_t s) {
  const int Kb = a.K / 32;
  int S = rows_wide_split(a.N, a.K);
  if (S > 1 && (a.P == nullptr || a.P_elems < (size_t)S * a.M * a.N)) S = 1;
  const dim3 grid(a.N / kRowsWideCols, S), block(kWideWaves * 64);
  switch (RT) {
    case 2: hipLaunchKernelGGL(gemm_wide_kernel<2>, grid, block, 0, s, a.Wp, a.nb, a.A, Kb, S, a.Y, a.M, ldy, a.accumulate, a.P, a.N); break;
    case 4: hipLaunchKernelGGL(gemm_wide_kernel<4>, grid, block, 0, s, a.Wp, a.nb, a.A, Kb, S, a.Y, a.M, ldy, a.accumulate, a.P, a.N); break;
    case 8: hipLaunchKernelGGL(gemm_wide_kernel<8>, grid, block, 0, s, a.Wp, a.nb, a.A, Kb, S, a.Y, a.M, ldy, a.accumulate, a.P, a.N); break;
    case 16: hipLaunchKernelGGL(gemm_wide_kernel<16>, grid, block, 0, s, a.Wp, a.nb, a.A, Kb, S, a.Y, a.M, ldy, a.accumulate, a.P, a.N); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (a.split_out) *a.split_out = S > 1 && a.defer_sum ? S : 0;
  if (e != hipSuccess || S == 1 || a.defer_sum) return e;
  const size_t total = (size_t)a.M * a.N;
  size_t blocks = (total + 255) / 256;
  blocks = blocks > 2048 ? 2048 : blocks;
  hipLaunchKernelGGL(rows_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.P, S, a.M,
                     a.N, a.Y, ldy, a.accumulate);
  return hipGetLastError();
}

}  // namespace spec
