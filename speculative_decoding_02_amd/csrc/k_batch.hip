// k_batch.hip -- the kernels a batched verify adds around the rows GEMM and
// the attention: B sequences' passes of R rows each in one set of launches
// (row m = b R + r is row r of sequence b).
//
// [en] Floor 6 ("crowded tower days"; [zh] Level 6): with many requests at
// once every weight read serves B (K+1) rows, so the pass moves from memory
// bound toward compute bound.  Each sequence still has its own history,
// positions, paged cache and accept/reject decision; only the weight stream
// is shared.
//
//   embed      -> rows of every sequence (its pending token and drafts, or a
//                 prompt chunk), pass descriptors and rule positions
//   norm_pack  -> RMSNorm of every row, packed as the rows GEMM's A operand
//   qkv_post   -> RoPE at each row's position; query fragments per sequence;
//                 keys and values appended through the sequence's block table
//   silu_pack  -> silu(gate) * up, packed
//   softmax    -> row softmax of the logits (two launches, fixed-order folds)
//   commit     -> per sequence: accepted tokens into its history, new length
#include "kernels.h"

namespace spec {

constexpr int kBatchThreads = 256;
constexpr uint32_t kBatchOOB = 0x80000000u;  // buffer offset past any range: reads zero, no fetch
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// --------------------------------------------------------------- embed --
__global__ __launch_bounds__(kBatchThreads) void batch_embed_kernel(BatchEmbedArgs a) {
  const int m = blockIdx.x, b = m / a.R, r = m % a.R, tid = threadIdx.x;
  DevState* st = a.st + b;
  const int32_t* hist = a.hist + (size_t)b * a.hist_cap;
  int LT = st->LT;
  if (LT < 0 || LT >= a.hist_cap) LT = 0;  // corrupt state: stay in bounds (flagged below)
  const int pos0 = a.mode == BEMB_VERIFY ? LT : a.pos0;
  const int pos = pos0 + r;
  int tok;
  if (a.mode == BEMB_VERIFY) {
    tok = r == 0 ? hist[LT] : a.dtok[(size_t)b * (a.R - 1) + r - 1];
  } else {
    tok = pos < a.hist_cap ? hist[pos] : -1;
  }
  const bool bad = tok < 0 || tok >= a.vocab;
  if (tid == 0) {
    int32_t err = 0;
    if (bad) err |= kErrBadToken;
    if (pos >= a.max_seq || st->LT != LT) err |= kErrCapacity;
    if (err) atomicOr(&st->err, err);
    if (r < kMaxRows) a.rows[b].tok[r] = bad ? 0 : tok;
    if (r == 0) {
      a.rows[b].n_rows = a.R;
      a.rows[b].pos0 = pos0;
      a.pos_rule[b] = (uint64_t)pos0 + 1;
    }
  }
  if (bad) tok = 0;
  const uint16_t* e = a.E + (size_t)tok * a.d;
  float* x = a.x + (size_t)m * a.d;
  for (int k0 = tid * 8; k0 < a.d; k0 += kBatchThreads * 8) {
    float v[8];
    load_gain8(e, k0, v);  // eight bf16 -> fp32
    *(float4*)(x + k0) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(x + k0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

hipError_t launch_batch_embed(const BatchEmbedArgs& a, hipStream_t s) {
  if (a.B < 1 || a.R < 1 || a.R > kMaxRows || a.B * a.R > kRowsMaxM || a.d % 8 ||
      (a.mode == BEMB_VERIFY && a.R > 1 && a.dtok == nullptr))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(batch_embed_kernel, dim3(a.B * a.R), dim3(kBatchThreads), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------- norm_pack --
// One workgroup per row; thread t owns the 8-element chunks t, t + 256, ...
// of its row in both passes (values kept in registers).
constexpr int kNormChunks = kNormPackMaxD / (kBatchThreads * 8);

__global__ __launch_bounds__(kBatchThreads) void norm_pack_kernel(NormPackArgs a) {
  __shared__ float s_red[16];
  const int m = blockIdx.x, tid = threadIdx.x, d = a.d;
  if (m >= a.M) {  // padding rows of the last tile
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = tid * 8; k0 < d; k0 += kBatchThreads * 8) apack_store8_rt(a.Ap, m, k0, z, a.RT);
    return;
  }
  float* x = a.x + (size_t)m * d;
  // split partials through a range-checked buffer: the loads of every slice
  // of a chunk are issued together (slices past S read zero without a fetch
  // and are not added), so a chunk costs one round trip, not one per slice
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.P), 0, a.S > 0 ? (int)((size_t)a.S * a.M * d * 4) : 0, 0x00020000);
  float v[kNormChunks][8];
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < kNormChunks; ++c) {
    const int k0 = (c * kBatchThreads + tid) * 8;
    if (k0 < d) {
      const float4 x0 = *(const float4*)(x + k0), x1 = *(const float4*)(x + k0 + 4);
      float r[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      if (a.S > 0) {
        f32x4_t p0[kRowsMaxSplit], p1[kRowsMaxSplit];
#pragma unroll
        for (int sl = 0; sl < kRowsMaxSplit; ++sl) {
          const uint32_t off = sl < a.S ? (uint32_t)((((size_t)sl * a.M + m) * d + k0) * 4) : kBatchOOB;
          p0[sl] = __builtin_amdgcn_raw_buffer_load_b128(rP, (int)off, 0, 0);
          p1[sl] = __builtin_amdgcn_raw_buffer_load_b128(rP, (int)(off == kBatchOOB ? off : off + 16), 0, 0);
        }
#pragma unroll
        for (int sl = 0; sl < kRowsMaxSplit; ++sl) {  // slice order, as a plain loop would add
          if (sl < a.S) {
            r[0] += p0[sl][0]; r[1] += p0[sl][1]; r[2] += p0[sl][2]; r[3] += p0[sl][3];
            r[4] += p1[sl][0]; r[5] += p1[sl][1]; r[6] += p1[sl][2]; r[7] += p1[sl][3];
          }
        }
        *(float4*)(x + k0) = make_float4(r[0], r[1], r[2], r[3]);
        *(float4*)(x + k0 + 4) = make_float4(r[4], r[5], r[6], r[7]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[c][e] = r[e];
        ss += r[e] * r[e];
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one chunk's loads in flight at a time (registers)
  }
  ss = block_reduce(ss, s_red, [](float p, float q) { return p + q; });
  const float inv = 1.0f / sqrtf(ss / (float)d + a.eps);
#pragma unroll
  for (int c = 0; c < kNormChunks; ++c) {
    const int k0 = (c * kBatchThreads + tid) * 8;
    if (k0 < d) {
      float g[8], h[8];
      load_gain8(a.gain, k0, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = v[c][e] * inv * g[e];
      apack_store8_rt(a.Ap, m, k0, h, a.RT);
    }
  }
}

hipError_t launch_norm_pack(const NormPackArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 8 * a.RT || a.RT > kRowsMaxM / 8 || a.d % 32 || a.d > kNormPackMaxD ||
      a.S < 0 || a.S > kRowsMaxSplit || (a.S > 0 && a.P == nullptr))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(norm_pack_kernel, dim3(8 * a.RT), dim3(kBatchThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ qkv_post --
__global__ __launch_bounds__(kBatchThreads) void qkv_post_kernel(QkvPostArgs a) {
  const int half = a.hd / 2;
  const int n_pairs = a.q_dim / 2 + a.kv_dim / 2;
  const int per_row = n_pairs + a.kv_dim;
  const int ldy = a.q_dim + 2 * a.kv_dim;
  const int G = a.q_dim / a.kv_dim, n_es = (a.hd + 31) / 32;
  const size_t total = (size_t)a.M * per_row;
  // column c of row m: the product, or the sum of its split partials in
  // slice order; every slice's load is issued before the first add (slices
  // past S read zero without a fetch through the range-checked buffer and
  // are not added)
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.P), 0, a.S > 0 ? (int)((size_t)a.S * a.M * ldy * 4) : 0, 0x00020000);
  auto yv = [&](int m, int c) -> float {
    if (a.S == 0) return a.y[(size_t)m * ldy + c];
    float p[kRowsMaxSplit];
#pragma unroll
    for (int sl = 0; sl < kRowsMaxSplit; ++sl) {
      const uint32_t off = sl < a.S ? (uint32_t)((((size_t)sl * a.M + m) * ldy + c) * 4) : kBatchOOB;
      p[sl] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rP, (int)off, 0, 0));
    }
    float v = 0.0f;
#pragma unroll
    for (int sl = 0; sl < kRowsMaxSplit; ++sl) v = sl < a.S ? v + p[sl] : v;
    return v;
  };
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(idx / per_row), i = (int)(idx % per_row);
    const int b = m / a.R, r = m % a.R;
    const int pos = a.rows[b].pos0 + r;
    if (pos < 0 || pos >= a.max_seq) continue;  // flagged by the embedding
    const int blk = a.block_table[(size_t)b * a.n_blocks + pos / kBlock];
    if (i < n_pairs) {
      // rotate-half RoPE on the pair (j, j + hd/2) of one head
      const bool is_q = i < a.q_dim / 2;
      const int pl = is_q ? i : i - a.q_dim / 2;
      const int head = pl / half, j = pl % half;
      const int c1 = (is_q ? 0 : a.q_dim) + head * a.hd + j;
      const float x1 = yv(m, c1), x2 = yv(m, c1 + half);
      const float2 cs = a.rope[(size_t)pos * half + j];
      const float v[2] = {x1 * cs.x - x2 * cs.y, x2 * cs.x + x1 * cs.y};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int dim = j + t * half;
        const uint16_t hb = f32_to_bf16_rne(v[t]);
        const uint16_t lb = f32_to_bf16_rne(v[t] - bf16_to_f32(hb));
        if (is_q) {
          uint16_t* qf = a.qf + (size_t)b * a.qf_seq;
          const int qi = r * G + head % G;
          qf[qfrag_index(head / G, G, n_es, qi, 0, dim)] = hb;
          qf[qfrag_index(head / G, G, n_es, qi, 1, dim)] = lb;
        } else {
          a.k_cache[kv_index(blk, a.n_kv, head, pos % kBlock, a.hd, 0, dim)] = hb;
          a.k_cache[kv_index(blk, a.n_kv, head, pos % kBlock, a.hd, 1, dim)] = lb;
        }
      }
    } else {
      const int f = i - n_pairs, head = f / a.hd, dim = f % a.hd;
      const float v = yv(m, a.q_dim + a.kv_dim + f);
      const uint16_t hb = f32_to_bf16_rne(v);
      a.v_cache[vt_index(blk, a.n_kv, head, 0, a.hd, dim, pos % kBlock)] = hb;
      a.v_cache[vt_index(blk, a.n_kv, head, 1, a.hd, dim, pos % kBlock)] =
          f32_to_bf16_rne(v - bf16_to_f32(hb));
    }
  }
}

hipError_t launch_qkv_post(const QkvPostArgs& a, hipStream_t s) {
  if (a.M < 1 || a.R < 1 || a.R > kMaxRows || a.M % a.R || a.hd % 2 || a.kv_dim <= 0 ||
      a.q_dim % a.kv_dim || a.S < 0 || a.S > kRowsMaxSplit || (a.S > 0 ? a.P == nullptr : a.y == nullptr))
    return hipErrorInvalidValue;
  const size_t total = (size_t)a.M * (a.q_dim / 2 + a.kv_dim / 2 + a.kv_dim);
  size_t blocks = (total + kBatchThreads - 1) / kBatchThreads;
  blocks = blocks > 2048 ? 2048 : blocks;
  hipLaunchKernelGGL(qkv_post_kernel, dim3((unsigned)blocks), dim3(kBatchThreads), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------- silu_pack --
__global__ __launch_bounds__(kBatchThreads) void silu_pack_kernel(SiluPackArgs a) {
  const int F8 = a.F / 8;
  const size_t total = (size_t)8 * a.RT * F8;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(idx / F8), k0 = (int)(idx % F8) * 8;
    float v[8];
    if (m < a.M) {
      const float* g = a.y + (size_t)m * 2 * a.F + k0;
      const float* u = g + a.F;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = g[e] / (1.0f + expf(-g[e])) * u[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    apack_store8_rt(a.Ap, m, k0, v, a.RT);
  }
}

hipError_t launch_silu_pack(const SiluPackArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 8 * a.RT || a.F % 32) return hipErrorInvalidValue;
  const size_t total = (size_t)8 * a.RT * (a.F / 8);
  size_t blocks = (total + kBatchThreads - 1) / kBatchThreads;
  blocks = blocks > 4096 ? 4096 : blocks;
  hipLaunchKernelGGL(silu_pack_kernel, dim3((unsigned)blocks), dim3(kBatchThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- softmax --
__global__ __launch_bounds__(kBatchThreads) void row_softmax_part_kernel(RowSoftmaxArgs a) {
  __shared__ float s_red[16];
  const int c = blockIdx.x, m = blockIdx.y, tid = threadIdx.x;
  const float* x = a.logits + (size_t)m * a.V;
  const int lo = c * a.chunk, hi = min(a.V, lo + a.chunk);
  float mx = -INFINITY;
  for (int v = lo + tid; v < hi; v += kBatchThreads) mx = fmaxf(mx, x[v]);
  mx = block_reduce(mx, s_red, [](float p, float q) { return fmaxf(p, q); });
  float sum = 0.0f;
  if (mx != -INFINITY)
    for (int v = lo + tid; v < hi; v += kBatchThreads) sum += expf(x[v] - mx);
  sum = block_reduce(sum, s_red, [](float p, float q) { return p + q; });
  if (tid == 0) a.part[(size_t)m * a.n_chunks + c] = make_float2(mx, sum);
}

__global__ __launch_bounds__(kBatchThreads) void row_softmax_norm_kernel(RowSoftmaxArgs a) {
  __shared__ float2 s_part[256];
  const int c = blockIdx.x, m = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < a.n_chunks; i += kBatchThreads) s_part[i] = a.part[(size_t)m * a.n_chunks + i];
  __syncthreads();
  float mx = -INFINITY;
  for (int i = 0; i < a.n_chunks; ++i) mx = fmaxf(mx, s_part[i].x);
  float den = 0.0f;
  for (int i = 0; i < a.n_chunks; ++i)
    den += s_part[i].x == -INFINITY ? 0.0f : s_part[i].y * expf(s_part[i].x - mx);
  const float inv = 1.0f / den;
  const float* x = a.logits + (size_t)m * a.V;
  float* out = a.out + (size_t)m * a.V;
  const int lo = c * a.chunk, hi = min(a.V, lo + a.chunk);
  for (int v = lo + tid; v < hi; v += kBatchThreads) out[v] = expf(x[v] - mx) * inv;
}

hipError_t launch_row_softmax(const RowSoftmaxArgs& a, hipStream_t s) {
  if (a.M < 1 || a.V < 1 || a.chunk < 1 || a.n_chunks < 1 || a.n_chunks > 256 ||
      (size_t)a.n_chunks * a.chunk < (size_t)a.V)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_softmax_part_kernel, dim3(a.n_chunks, a.M), dim3(kBatchThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_softmax_norm_kernel, dim3(a.n_chunks, a.M), dim3(kBatchThreads), 0, s, a);
  return hipGetLastError();
}

// -------------------------------------------------------------- commit --
__global__ __launch_bounds__(64) void batch_commit_kernel(BatchCommitArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  DevState* st = a.st + b;
  const int n = a.n_acc[b];
  if (n < 0 || n > a.K) return;
  const int LT = st->LT;
  if (LT < 0 || LT + 1 + n >= a.hist_cap) {
    if (tid == 0) atomicOr(&st->err, kErrCapacity);
    return;
  }
  int32_t* hist = a.hist + (size_t)b * a.hist_cap;
  for (int j = tid; j <= n; j += 64) hist[LT + 1 + j] = a.out[(size_t)b * (a.K + 1) + j];
  __syncthreads();
  if (tid == 0) {
    st->LT = LT + n + 1;
    st->LD = st->LT;
    if (a.K < kAcceptBins) st->accept_counts[a.K][n] += 1;
  }
}

hipError_t launch_batch_commit(const BatchCommitArgs& a, hipStream_t s) {
  if (a.B < 1 || a.K < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(batch_commit_kernel, dim3(a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace spec
