// k_heads.hip -- multi-token-prediction heads as the drafter.
//
// "Speculative decoding internals" (variants: MTP) describes targets that
// carry K extra output heads, head k predicting the token k places ahead, so
// that no separate drafter model is needed.  The pages fix no head
// architecture; the reading implemented here: head k takes the target's final
// normed state h of the last position it processed and forms
// z_k = h + silu(W_k h) with its own [d][d] matrix W_k; the target's own LM
// head scores z_k.  The position after h holds the pending token (already
// decided by the rule), so the K heads draft the K positions after it.
//
// A heads draft is: heads_prep (h from the kept final residual, packed as the
// A operand of the stacked head GEMM) -> head GEMM (all K matrices stacked,
// one row) -> heads_pack (z_k rows, packed as the A operand of the LM head)
// -> LM head over K rows -> softmax -> one sampler per draft.  The GEMM,
// softmax and sampler kernels are the verify pass's own.
#include "kernels.h"

namespace spec {

// One workgroup: h = x / sqrt(mean(x^2) + eps) * g, kept in fp32 for the
// residual of the heads and packed (bf16 high and low parts) as row 0 of the
// head GEMM's A operand; the pass descriptor then says one row.
__global__ __launch_bounds__(256) void heads_prep_kernel(HeadsArgs a) {
  __shared__ float s_red[16];
  const int tid = threadIdx.x, d = a.d;
  float ss = 0.0f;
  for (int i = tid; i < d; i += blockDim.x) ss += a.h_last[i] * a.h_last[i];
  ss = block_reduce(ss, s_red, [](float x, float y) { return x + y; });
  const float inv = 1.0f / sqrtf(ss / (float)d + a.eps);
  for (int k0 = tid * 8; k0 < d; k0 += blockDim.x * 8) {
    float g[8], v[8];
    load_gain8(a.g_final, k0, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = a.h_last[k0 + e] * inv * g[e];
      a.hn[k0 + e] = v[e];
    }
    apack_store8(a.Ap, 0, k0, v);
  }
  if (tid == 0) {
    a.rows->n_rows = 1;
    a.rows->pos0 = a.st->LT;
  }
}

// z_k = h + silu(y_k) for heads k < K, eight columns per thread, packed as
// row k of the LM head's A operand; the pass descriptor then says K rows
// (the drafts' positions start right after the pending token).
__global__ __launch_bounds__(256) void heads_pack_kernel(HeadsArgs a) {
  const int d = a.d;
  const int items = a.K * (d / 8);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < items; i += gridDim.x * blockDim.x) {
    const int k = i / (d / 8), c0 = (i % (d / 8)) * 8;
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = a.y[(size_t)k * d + c0 + e];
      z[e] = a.hn[c0 + e] + y / (1.0f + expf(-y));
    }
    apack_store8(a.Ap, k, c0, z);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.rows->n_rows = a.K;
    a.rows->pos0 = a.st->LT + 1;
  }
}

hipError_t launch_heads_prep(const HeadsArgs& a, hipStream_t s) {
  if (a.d % 8 || a.d <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(heads_prep_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_heads_pack(const HeadsArgs& a, hipStream_t s) {
  if (a.d % 8 || a.d <= 0 || a.K < 1 || a.K > kMaxRows) return hipErrorInvalidValue;
  const int items = a.K * (a.d / 8);
  const int grid = (items + 255) / 256;
  hipLaunchKernelGGL(heads_pack_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace spec
