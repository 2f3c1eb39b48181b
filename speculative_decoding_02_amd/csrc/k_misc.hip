// k_misc.hip -- embedding gather, LM-head softmax normalisation, the commit
// and the RoPE table.
#include "kernels.h"

namespace spec {

// ============================================================ embedding ==
// Decides the rows of a pass from the device state (so captured graphs can be
// replayed whatever the previous round accepted), gathers their embedding
// rows into the fp32 residual stream, writes x * gain (first RMSNorm gain) as
// the packed A operand of the QKV projection, and publishes per-64-column
// sums of squares.  Grid: one block of 64 threads per 64 columns; thread t
// handles row t/8, columns 8*(t%8)..+7.
// Pointers of the first loads lead the arguments as scalars (preloaded in
// SGPRs) and replace the copies in the argument struct.
__global__ __launch_bounds__(64) void embed_kernel(DevState* st, const int32_t* hist,
                                                   const int32_t* dtok, const uint16_t* E,
                                                   EmbedArgs args) {
  EmbedArgs a = args;
  a.st = st; a.hist = hist; a.dtok = dtok; a.E = E;
  const int LT = a.st->LT, LD = a.st->LD;
  int n_rows = 0, pos0 = 0;
  int tok[kMaxRows];
  int err = 0;
  if (a.mode == EMB_VERIFY) {
    n_rows = a.n_rows;
    pos0 = LT;
    tok[0] = a.hist[LT];
    for (int r = 1; r < kMaxRows; ++r) tok[r] = r < n_rows ? a.dtok[r - 1] : 0;
  } else if (a.mode == EMB_DRAFT0) {
    n_rows = LT - LD + 1;
    pos0 = LD;
    if (n_rows > kMaxRows || n_rows < 1) {
      err |= kErrLag;
      n_rows = 0;
    }
    for (int r = 0; r < kMaxRows; ++r) tok[r] = r < n_rows ? a.hist[LD + r] : 0;
  } else if (a.mode == EMB_DRAFTS) {
    n_rows = 1;
    pos0 = LT + a.step;
    tok[0] = a.dtok[a.step - 1];
    for (int r = 1; r < kMaxRows; ++r) tok[r] = 0;
  } else {
    n_rows = a.n_rows;
    pos0 = a.pos0;
    for (int r = 0; r < kMaxRows; ++r) tok[r] = r < n_rows ? a.hist[pos0 + r] : 0;
  }
  if (n_rows > 0 && pos0 + n_rows > a.max_seq) {
    err |= kErrCapacity;
    n_rows = 0;
  }
  for (int r = 0; r < n_rows; ++r) {
    if (tok[r] < 0 || tok[r] >= a.vocab) {
      err |= kErrBadToken;
      tok[r] = 0;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.rows_out->n_rows = n_rows;
    a.rows_out->pos0 = pos0;
    for (int r = 0; r < kMaxRows; ++r) a.rows_out->tok[r] = tok[r];
    if (err) atomicOr(&a.st->err, err);
  }
  const int r = threadIdx.x >> 3, cg = threadIdx.x & 7;
  const int k0 = blockIdx.x * 64 + cg * 8;
  float sq = 0.0f;
  if (r < n_rows) {
    int tk = tok[0];
    for (int i = 1; i < kMaxRows; ++i)
      if (i == r) tk = tok[i];
    const uint4 ev = *(const uint4*)(a.E + (size_t)tk * a.d + k0);
    const uint32_t w[4] = {ev.x, ev.y, ev.z, ev.w};
    float x[8], gn[8], xg[8];
    load_gain8(a.gain, k0, gn);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = bf16_to_f32((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
      sq += x[e] * x[e];
      xg[e] = x[e] * gn[e];
    }
    float* px = a.x + (size_t)r * a.d + k0;
    *(float4*)px = make_float4(x[0], x[1], x[2], x[3]);
    *(float4*)(px + 4) = make_float4(x[4], x[5], x[6], x[7]);
    apack_store8(a.Ap_out, r, k0, xg);
  }
  // sum over the 8 threads of the row (fixed butterfly)
  sq += __shfl_xor(sq, 4);
  sq += __shfl_xor(sq, 2);
  sq += __shfl_xor(sq, 1);
  if (cg == 0) a.ssq[blockIdx.x * kMaxRows + r] = sq;
}

hipError_t launch_embed(const EmbedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(a.d / 64), dim3(64), 0, s, a.st, a.hist, a.dtok, a.E, a);
  return hipGetLastError();
}

// ============================================================== softmax ==
// T_i = softmax(logits_i) at temperature 1 ([en] Floor 5: the target's
// wheel).  The LM-head GEMM left per-workgroup (max, sum exp) partials; each
// block folds them in a fixed order, then normalises its chunk of the row.
// The chunk's logits and this thread's partials are loaded together at the
// start, so the block makes one round trip to memory.
constexpr int kSoftmaxThreads = 256;
constexpr int kSoftmaxVec = 4;          // float4 per thread per chunk: chunk = 4096
constexpr int kSoftmaxMaxPart = 32;     // partials per thread: G <= 8192

__global__ __launch_bounds__(kSoftmaxThreads) void softmax_kernel(const float* logits,
                                                                 const float2* part,
                                                                 const PassRows* rows,
                                                                 SoftmaxArgs args) {
  SoftmaxArgs a = args;
  a.logits = logits; a.part = part; a.rows = rows;
  __shared__ float s_m[16], s_s[16];
  const int r = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int lo = c * a.chunk;
  const float* lrow = a.logits + (size_t)r * a.V;
  float4 lv[kSoftmaxVec];
#pragma unroll
  for (int j = 0; j < kSoftmaxVec; ++j) {
    const int v = lo + (j * kSoftmaxThreads + tid) * 4;
    lv[j] = v < a.V ? *(const float4*)(lrow + v) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float2 pv[kSoftmaxMaxPart];
#pragma unroll
  for (int i = 0; i < kSoftmaxMaxPart; ++i) {
    const int g = i * kSoftmaxThreads + tid;
    pv[i] = g < a.G ? a.part[g * kMaxRows + r] : make_float2(-INFINITY, 0.0f);
  }
  int n_rows = a.rows->n_rows;
  if (a.last_row_only) n_rows = n_rows > 0 ? 1 : 0;
  if (r >= n_rows) return;
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSoftmaxMaxPart; ++i) M = fmaxf(M, pv[i].x);
  M = block_reduce(M, s_m, [](float x, float y) { return fmaxf(x, y); });
  float S = 0.0f;
#pragma unroll
  for (int i = 0; i < kSoftmaxMaxPart; ++i)
    if (pv[i].x != -INFINITY) S += pv[i].y * expf(pv[i].x - M);
  S = block_reduce(S, s_s, [](float x, float y) { return x + y; });
  const float inv = 1.0f / S;
  float* orow = a.out + (size_t)r * a.V;
#pragma unroll
  for (int j = 0; j < kSoftmaxVec; ++j) {
    const int v = lo + (j * kSoftmaxThreads + tid) * 4;
    if (v < a.V)
      *(float4*)(orow + v) = make_float4(expf(lv[j].x - M) * inv, expf(lv[j].y - M) * inv,
                                         expf(lv[j].z - M) * inv, expf(lv[j].w - M) * inv);
  }
}

hipError_t launch_softmax(const SoftmaxArgs& a, int n_chunks, int n_rows, hipStream_t s) {
  if (a.chunk != kSoftmaxThreads * kSoftmaxVec * 4 || a.G > kSoftmaxThreads * kSoftmaxMaxPart ||
      a.V % 4 != 0 || n_rows < 1 || n_rows > kMaxRows)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(softmax_kernel, dim3(n_chunks, n_rows), dim3(kSoftmaxThreads), 0, s, a.logits,
                     a.part, a.rows, a);
  return hipGetLastError();
}

// =============================================================== commit ==
// Keep the pending token and the n accepted drafts; the emitted token
// (replacement or bonus) becomes the next pending token ([en] Floor 4: slips
// after the first reject are torn up).  The draft cache keeps the rows whose
// tokens were committed: it processed [pending, d_1..d_{K-1}], so it is
// valid up to position LT + min(n, K-1).
// The verify's (K, n_acc) pair is counted in the state's acceptance record.
__global__ __launch_bounds__(256) void commit_kernel(DevState* st, int32_t* hist, int hist_cap,
                                                    const int32_t* out, const int32_t* n_acc,
                                                    int drafted_k, int verified_k,
                                                    const float* x_rows, int d, float* h_last) {
  if (blockIdx.x != 0) return;
  const int n = *n_acc;
  if (n < 0 || n > verified_k) return;
  const int LT = st->LT;
  if (LT + 1 + n >= hist_cap) {
    if (threadIdx.x == 0) atomicOr(&st->err, kErrCapacity);
    return;
  }
  // the state of the last committed position: row n of the pass
  if (h_last != nullptr)
    for (int i = threadIdx.x; i < d; i += blockDim.x) h_last[i] = x_rows[(size_t)n * d + i];
  if (threadIdx.x != 0) return;
  for (int i = 0; i <= n; ++i) hist[LT + 1 + i] = out[i];
  if (drafted_k > 0) st->LD = LT + (n + 1 < drafted_k ? n + 1 : drafted_k);
  st->LT = LT + n + 1;
  st->accept_counts[verified_k][n] += 1;
}

hipError_t launch_commit(DevState* st, int32_t* hist, int hist_cap, const int32_t* out,
                         const int32_t* n_acc, int drafted_k, int verified_k, const float* x_rows,
                         int d, float* h_last, hipStream_t s) {
  if (verified_k < 0 || verified_k >= kAcceptBins) return hipErrorInvalidValue;
  if (h_last != nullptr && (x_rows == nullptr || d <= 0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(256), 0, s, st, hist, hist_cap, out, n_acc,
                     drafted_k, verified_k, x_rows, d, h_last);
  return hipGetLastError();
}

// Plain streaming read of a buffer: the HBM read rate a kernel that does
// nothing else reaches, against which the verify pass's rate is read.
// Workgroup g reads the contiguous slice [n g / G, n (g+1) / G)
// of 16-byte words; its 512 lanes keep 8 non-temporal loads each in flight,
// the waves interleaved over 8 KiB steps.
constexpr int kReadThreads = 512;
constexpr int kReadDepth = 8;
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* p, size_t n,
                                                                  uint32_t* sink) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const size_t G = gridDim.x, g = blockIdx.x;
  const size_t b = n * g / G, e = n * (g + 1) / G;
  constexpr size_t step = kReadThreads;
  size_t i = b + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadDepth - 1) * step < e; i += kReadDepth * step) {
    u32x4_t v[kReadDepth];
#pragma unroll
    for (int u = 0; u < kReadDepth; ++u) v[u] = __builtin_nontemporal_load((const u32x4_t*)(p + i + u * step));
#pragma unroll
    for (int u = 0; u < kReadDepth; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < e; i += step) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the data must be used; this store almost never happens
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, int grid, uint32_t* sink,
                              hipStream_t s) {
  if (bytes % 16 || grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, s, (const uint4*)buf,
                     bytes / 16, sink);
  return hipGetLastError();
}

// RoPE rotation table ([cos, sin] of the angle pos * theta^(-2j/hd)), the
// angle and both functions evaluated in fp64 once per context.
__global__ void rope_table_kernel(float2* dst, int max_seq, int hd, double theta) {
  const int half = hd / 2;
  const size_t n = (size_t)max_seq * half;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int pos = (int)(i / half), j = (int)(i % half);
    const double ang = (double)pos * pow(theta, -2.0 * (double)j / (double)hd);
    double sn, cs;
    sincos(ang, &sn, &cs);
    dst[i] = make_float2((float)cs, (float)sn);
  }
}

hipError_t launch_rope_table(float2* dst, int max_seq, int hd, double theta, hipStream_t s) {
  const size_t n = (size_t)max_seq * (hd / 2);
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, max_seq, hd,
                     theta);
  return hipGetLastError();
}

}  // namespace spec
