// k_gemm_rows.hip -- the weight-streaming GEMM for a batch of verify passes:
// Y[m][n] = sum_k X[m][k] W[n][k] for M up to 128 activation rows (B
// sequences' K+1 rows each, M = B (K+1)), against the same packed bf16 weight
// stream as the single-pass GEMM.
//
// [en] Floor 6 ("crowded tower days"; [zh] Level 6): with many petitioners at
// once every weight read already serves a thick stack of rows, the work moves
// from memory-bound to compute-bound, and the extra draft positions stop
// being free.  This kernel is the instrument for that crossover: as M grows
// the bytes stay the same while the matrix-core work grows with M.
//
//  * Activations are packed per call into row tiles of the A operand of
//    v_mfma_f32_16x16x32_bf16, [Kb][RT][64 lanes][8 bf16]: tile t carries the
//    bf16 high parts of rows 8t..8t+7 in its rows 0-7 and their low parts
//    (x - hi) in rows 8-15, the same ~16-bit activation precision as the
//    verify pass.  Rows past M are zero.  A batched verify's producers
//    (norm, SiLU, attention merge) write this layout themselves, and the
//    residual updates accumulate into Y.
//  * A workgroup owns NB 16-column blocks for the whole of K; its W waves
//    split K; for every k-block a wave multiplies its NB weight fragments by
//    all RT row tiles, so each weight byte is read once whatever M is.  The
//    waves' partial tiles are reduced through LDS one row tile at a time, in
//    wave order (deterministic).
#include <type_traits>

#include "kernels.h"

namespace spec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// one thread per (k-block, tile, lane): 8 bf16 of one tile row
__global__ __launch_bounds__(256) void pack_rows_kernel(const float* X, int M, int K, int RT,
                                                        uint16_t* A) {
  const size_t total = (size_t)(K / 32) * RT * 64;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx % 64), t = (int)((idx / 64) % RT);
    const int kb = (int)(idx / (64 * (size_t)RT));
    const int l16 = lane & 15, grp = lane >> 4;
    const int row = 8 * t + (l16 & 7), part = l16 >> 3;
    const int k0 = 32 * kb + 8 * grp;
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = row < M ? X[(size_t)row * K + k0 + e] : 0.0f;
      const uint16_t hi = f32_to_bf16_rne(x);
      h[e] = part ? f32_to_bf16_rne(x - bf16_to_f32(hi)) : hi;
    }
    ((uint4*)A)[idx] = make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]),
                                  pack_bf16x2(h[4], h[5]), pack_bf16x2(h[6], h[7]));
  }
}

template <int NB, int W, int RT>
__global__ __launch_bounds__(W * 64) void gemm_rows_kernel(const uint16_t* Wp, const uint16_t* A,
                                                           int Kb, float* Y, int M, int ldy,
                                                           int accumulate) {
  constexpr int YW = NB * 16;
  constexpr int U = RT <= 2 ? 8 : (RT <= 4 ? 4 : 2);  // k-blocks per batch of loads
  __shared__ float s_red[W * NB * 256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x;
  const int kb0 = (Kb * wave) / W, kb1 = (Kb * (wave + 1)) / W;
  const uint4* wp = (const uint4*)Wp + (size_t)g * Kb * NB * 64 + lane;
  const uint4* ap = (const uint4*)A + lane;
  floatx4 acc[RT][NB];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[t][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto batch = [&](auto ub_tag, int kb) {
    constexpr int UB = decltype(ub_tag)::value;
    uint4 av[UB][RT], wv[UB][NB];
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int t = 0; t < RT; ++t) av[u][t] = ap[((size_t)(kb + u) * RT + t) * 64];
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const u32x4_t v =
            __builtin_nontemporal_load((const u32x4_t*)(wp + ((size_t)(kb + u) * NB + j) * 64));
        wv[u][j] = make_uint4(v.x, v.y, v.z, v.w);
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UB; ++u)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, av[u][t]), __builtin_bit_cast(bf16x8_t, wv[u][j]),
              acc[t][j], 0, 0, 0);
  };
  int kb = kb0;
  for (; kb + U <= kb1; kb += U) batch(std::integral_constant<int, U>{}, kb);
  for (; kb < kb1; ++kb) batch(std::integral_constant<int, 1>{}, kb);

  // per row tile: the waves' partials (high-part rows + low-part rows) in
  // wave order.  MFMA output: lane l, element r is row 4 (l / 16) + r, column
  // l % 16; rows 8-15 (lanes 32-63) are the low-part products of rows 0-7.
  const int col0 = g * YW;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
      *(float4*)&s_red[((wave * NB + j) * 64 + lane) * 4] =
          make_float4(acc[t][j][0], acc[t][j][1], acc[t][j][2], acc[t][j][3]);
    __syncthreads();
    for (int idx = tid; idx < NB * 128; idx += W * 64) {
      const int j = idx >> 7, ln = (idx >> 2) & 31, r = idx & 3;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w)
        v += s_red[((w * NB + j) * 64 + ln) * 4 + r] + s_red[((w * NB + j) * 64 + ln + 32) * 4 + r];
      const int m = 8 * t + 4 * (ln >> 4) + r;
      if (m < M) {
        float* y = Y + (size_t)m * ldy + col0 + j * 16 + (ln & 15);
        *y = accumulate ? *y + v : v;
      }
    }
    __syncthreads();
  }
}

template <int NB>
static hipError_t launch_rt(int RT, const uint16_t* Wp, const uint16_t* A, int Kb, int n_groups,
                            float* Y, int M, int ldy, int acc, hipStream_t s) {
  const dim3 grid(n_groups), block(4 * 64);
  switch (RT) {
    case 1: hipLaunchKernelGGL((gemm_rows_kernel<NB, 4, 1>), grid, block, 0, s, Wp, A, Kb, Y, M, ldy, acc); break;
    case 2: hipLaunchKernelGGL((gemm_rows_kernel<NB, 4, 2>), grid, block, 0, s, Wp, A, Kb, Y, M, ldy, acc); break;
    case 4: hipLaunchKernelGGL((gemm_rows_kernel<NB, 4, 4>), grid, block, 0, s, Wp, A, Kb, Y, M, ldy, acc); break;
    case 8: hipLaunchKernelGGL((gemm_rows_kernel<NB, 4, 8>), grid, block, 0, s, Wp, A, Kb, Y, M, ldy, acc); break;
    case 16: hipLaunchKernelGGL((gemm_rows_kernel<NB, 4, 16>), grid, block, 0, s, Wp, A, Kb, Y, M, ldy, acc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_rows(const RowsGemmArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > kRowsMaxM || a.K % 32 || (a.nb != 1 && a.nb != 2) || a.N % (16 * a.nb))
    return hipErrorInvalidValue;
  const int ldy = a.ldy > 0 ? a.ldy : a.N;
  if (ldy < a.N) return hipErrorInvalidValue;
  const int RT = rows_tiles(a.M);
  const int Kb = a.K / 32, n_groups = a.N / (16 * a.nb);
  if (a.X != nullptr) {
    const size_t total = (size_t)Kb * RT * 64;
    size_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.X, a.M, a.K,
                       RT, a.A);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.split_out) *a.split_out = 0;
  if (RT > 1 && a.N % kRowsWideCols == 0) return launch_gemm_wide(a, RT, ldy, s);
  if (a.nb == 1) return launch_rt<1>(RT, a.Wp, a.A, Kb, n_groups, a.Y, a.M, ldy, a.accumulate, s);
  return launch_rt<2>(RT, a.Wp, a.A, Kb, n_groups, a.Y, a.M, ldy, a.accumulate, s);
}

}  // namespace spec
