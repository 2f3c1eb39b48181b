// k_misc.hip -- embedding gather, LM-head softmax normalisation, the
// accept/reject kernels (also used to sample draft tokens) and the commit.
#include "kernels.h"

namespace spec {

// ============================================================ embedding ==
// Decides the rows of a pass from the device state (so captured graphs can be
// replayed whatever the previous round accepted), gathers their embedding
// rows into the fp32 residual stream, writes x * gain (first RMSNorm gain) as
// the packed A operand of the QKV projection, and publishes per-64-column
// sums of squares.  Grid: one block of 64 threads per 64 columns; thread t
// handles row t/8, columns 8*(t%8)..+7.
__global__ __launch_bounds__(64) void embed_kernel(EmbedArgs a) {
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
  hipLaunchKernelGGL(embed_kernel, dim3(a.d / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ============================================================== softmax ==
// T_i = softmax(logits_i) at temperature 1 ([en] Floor 5: the target's
// wheel).  The LM-head GEMM left per-workgroup (max, sum exp) partials; each
// block folds them in a fixed order, then normalises its chunk of the row.
__global__ __launch_bounds__(256) void softmax_kernel(SoftmaxArgs a) {
  __shared__ float s_m[16], s_s[16];
  const int r = blockIdx.y, c = blockIdx.x;
  int n_rows = a.rows->n_rows;
  if (a.last_row_only) n_rows = n_rows > 0 ? 1 : 0;
  if (r >= n_rows) return;
  float M = -INFINITY;
  for (int g = threadIdx.x; g < a.G; g += blockDim.x) M = fmaxf(M, a.part[g * kMaxRows + r].x);
  M = block_reduce(M, s_m, [](float x, float y) { return fmaxf(x, y); });
  float S = 0.0f;
  for (int g = threadIdx.x; g < a.G; g += blockDim.x) {
    const float2 p = a.part[g * kMaxRows + r];
    if (p.x != -INFINITY) S += p.y * expf(p.x - M);
  }
  S = block_reduce(S, s_s, [](float x, float y) { return x + y; });
  const float inv = 1.0f / S;
  const float* l = a.logits + (size_t)r * a.V;
  float* o = a.out + (size_t)r * a.V;
  const int lo = c * a.chunk, hi = min(a.V, lo + a.chunk);
  for (int v = lo + threadIdx.x; v < hi; v += blockDim.x) o[v] = expf(l[v] - M) * inv;
}

hipError_t launch_softmax(const SoftmaxArgs& a, int n_chunks, hipStream_t s) {
  hipLaunchKernelGGL(softmax_kernel, dim3(n_chunks, kMaxRows), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ======================================================== accept/reject ==
// The rule of [int] algorithm core Steps 3-4 / [en] Floors 4-5, per
// sequence b, in two launches:
//  1. partial kernel, one block per (vocabulary chunk, sequence): decide the
//     K exact accept tests r_i * D_i(d_i) < T_i(d_i) (r_i = Philox w1 at the
//     draft's position); a wave ballot gives the first reject j (j = K:
//     none).  Then sum, over the chunk, the integer weights of the row to
//     sample from: the residual fix(T_j) - fix(D_j) (saturating, 2^-40 grid)
//     on a reject, else the bonus row fix(T_K); integer sums are order-free,
//     so the result does not depend on the reduction tree.  The fallbacks
//     (sum of fix(T_j), argmax of the row) are gathered in the same pass.
//  2. finish kernel, one block per sequence: repeat the accept tests, fold
//     the chunk partials in chunk order, find the chunk holding the
//     inverse-CDF needle floor(u24 * Z / 2^24) (u24 = Philox w2 at the
//     decided position), rescan that chunk and write the emitted tokens.
// Greedy mode replaces the sums by per-chunk argmaxes of every row.
// K = 0 samples one row (draft tokens, word w0).

// Accept tests and draft validation (wave 0).  Returns j (first reject, K if
// none; K in greedy mode) and whether the inputs read so far are invalid.
SPEC_DEVICE void decide_first_reject(const ArArgs& a, int b, uint64_t P, int* s_j, int* s_err) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    const int K = a.K, V = a.V;
    const float* Tb = a.T + (size_t)b * (K + 1) * V;
    const float* Db = a.D ? a.D + (size_t)b * K * V : nullptr;
    const int32_t* db = a.d + (size_t)b * K;
    bool bad_d = false, stop = false, invalid = false;
    if (lane < K) {
      const int di = db[lane];
      bad_d = di < 0 || di >= V;
      if (!a.greedy && !bad_d) {
        const float t = Tb[(size_t)lane * V + di];
        const float q = Db[(size_t)lane * V + di];
        invalid = !prob_valid(t) || !prob_valid(q);
        const uint32_t u = uniform_u24(a.seed, P + lane, b, a.stream_id, 1);
        const float rr = (float)u * 0x1p-24f;
        stop = invalid || !((double)rr * (double)q < (double)t);
      }
    }
    const uint64_t bd = __ballot(bad_d);
    const uint64_t st = __ballot(stop || bad_d);
    const int j = st ? __ffsll((long long)st) - 1 : K;
    const uint64_t inv = __ballot(invalid);
    if (lane == 0) {
      *s_j = a.greedy ? K : j;
      *s_err = (bd != 0) || (!a.greedy && j < K && ((inv >> j) & 1));
    }
  }
  __syncthreads();
}

SPEC_DEVICE uint64_t seq_pos(const ArArgs& a, int b) {
  return a.pos ? a.pos[b] : (uint64_t)(a.st->LT + a.pos_offset);
}

__global__ __launch_bounds__(256) void ar_partial_kernel(ArArgs a) {
  __shared__ int32_t s_j, s_err;
  __shared__ uint64_t s_u64[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, b = blockIdx.y;
  const int K = a.K, V = a.V;
  const uint64_t P = seq_pos(a, b);
  const float* Tb = a.T + (size_t)b * (K + 1) * V;
  const float* Db = a.D ? a.D + (size_t)b * K * V : nullptr;
  const int W = ar_ws_words(K);
  uint64_t* p = a.ws + ((size_t)b * a.n_chunks + c) * W;
  decide_first_reject(a, b, P, &s_j, &s_err);
  const int j = s_j;
  const int lo = c * a.chunk, hi = min(V, lo + a.chunk);

  if (!a.greedy) {
    uint64_t zr = 0, zt = 0, am = 0, bad = 0;
    if (!s_err) {
      const float* Tr = Tb + (size_t)j * V;
      const float* Dr = j < K ? Db + (size_t)j * V : nullptr;
      for (int v = lo + tid; v < hi; v += 256) {
        const float tv = Tr[v];
        if (!prob_valid(tv)) { bad = 1; continue; }
        const uint64_t ft = fix40(tv);
        am = max(am, argmax_key(tv, (uint32_t)v));
        if (Dr) {
          const float dv = Dr[v];
          if (!prob_valid(dv)) { bad = 1; continue; }
          const uint64_t fd = fix40(dv);
          zr += ft > fd ? ft - fd : 0;
          zt += ft;
        } else {
          zr += ft;
        }
      }
    }
    zr = wave_sum_u64(zr);
    zt = wave_sum_u64(zt);
    am = wave_max_u64(am);
    bad = wave_max_u64(bad);
    if (lane == 0) {
      s_u64[wave] = zr; s_u64[4 + wave] = zt; s_u64[8 + wave] = am; s_u64[12 + wave] = bad;
    }
    __syncthreads();
    if (tid == 0) {
      p[0] = s_u64[0] + s_u64[1] + s_u64[2] + s_u64[3];
      p[1] = s_u64[4] + s_u64[5] + s_u64[6] + s_u64[7];
      p[2] = max(max(s_u64[8], s_u64[9]), max(s_u64[10], s_u64[11]));
      p[3] = s_u64[12] | s_u64[13] | s_u64[14] | s_u64[15];
    }
  } else {
    // per-row argmax keys of this chunk, rows 0..K, and an invalid-value flag
    uint64_t bad_all = 0;
    for (int i = 0; i <= K; ++i) {
      const float* Tr = Tb + (size_t)i * V;
      uint64_t am = 0, bad = 0;
      for (int v = lo + tid; v < hi; v += 256) {
        const float tv = Tr[v];
        if (!prob_valid(tv)) { bad = 1; continue; }
        am = max(am, argmax_key(tv, (uint32_t)v));
      }
      am = wave_max_u64(am);
      bad = wave_max_u64(bad);
      if (lane == 0) { s_u64[wave] = am; s_u64[4 + wave] = bad; }
      __syncthreads();
      if (tid == 0) {
        p[i] = max(max(s_u64[0], s_u64[1]), max(s_u64[2], s_u64[3]));
        bad_all |= s_u64[4] | s_u64[5] | s_u64[6] | s_u64[7];
      }
      __syncthreads();
    }
    if (tid == 0) p[K + 1] = bad_all;
  }
}

__global__ __launch_bounds__(256) void ar_finish_kernel(ArArgs a) {
  __shared__ int32_t s_j, s_err, s_tok, s_c, s_bad;
  __shared__ uint64_t s_u64[4];
  __shared__ uint64_t s_before;
  __shared__ uint64_t s_scan[256];
  __shared__ int32_t s_am[64];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int K = a.K, V = a.V;
  const uint64_t P = seq_pos(a, b);
  const float* Tb = a.T + (size_t)b * (K + 1) * V;
  const float* Db = a.D ? a.D + (size_t)b * K * V : nullptr;
  const int32_t* db = a.d + (size_t)b * K;
  const int W = ar_ws_words(K);
  const uint64_t* ws_b = a.ws + (size_t)b * a.n_chunks * W;
  int32_t* ob = a.out + (size_t)b * (K + 1);
  decide_first_reject(a, b, P, &s_j, &s_err);
  const int j = s_j;

  if (a.greedy) {
    if (tid == 0) s_bad = 0;
    __syncthreads();
    for (int i = tid; i <= K + 1; i += 256) {
      uint64_t acc = 0;
      for (int cc = 0; cc < a.n_chunks; ++cc) {
        const uint64_t v = ws_b[(size_t)cc * W + i];
        acc = (i <= K) ? max(acc, v) : (acc | v);
      }
      if (i <= K) s_am[i] = (int32_t)argmax_key_index(acc);
      else if (acc) s_bad = 1;
    }
    __syncthreads();
    if (tid == 0) {
      const bool err = s_err || s_bad;
      int n = K;
      if (!err) {
        for (int i = 0; i < K; ++i) {
          if (s_am[i] != db[i]) { n = i; break; }
        }
      }
      for (int i = 0; i <= K; ++i) ob[i] = err ? -1 : (i < n ? db[i] : (i == n ? s_am[n] : -1));
      if (a.n_acc) a.n_acc[b] = err ? -1 : n;
    }
    return;
  }

  // sampling: fold chunk partials (fixed order)
  if (tid == 0) {
    uint64_t zr = 0, zt = 0, am = 0, bad = s_err;
    for (int cc = 0; cc < a.n_chunks; ++cc) {
      const uint64_t* p = ws_b + (size_t)cc * W;
      zr += p[0];
      zt += p[1];
      am = max(am, p[2]);
      bad |= p[3];
    }
    s_u64[0] = zr; s_u64[1] = zt; s_u64[2] = am; s_u64[3] = bad;
    s_tok = -1;
  }
  __syncthreads();
  const uint64_t zr = s_u64[0], zt = s_u64[1], am = s_u64[2], bad = s_u64[3];
  if (bad) {
    if (tid <= K) ob[tid] = -1;
    if (tid == 0 && a.n_acc) a.n_acc[b] = -1;
    return;
  }
  // which weights to sample: residual (or bonus row), else fix(T_j), else argmax
  const int use = zr > 0 ? 0 : ((j < K && zt > 0) ? 1 : 2);
  if (use < 2) {
    const uint32_t u = uniform_u24(a.seed, P + j, b, a.stream_id, a.word);
    const uint64_t Z = use == 0 ? zr : zt;
    const uint64_t t = icdf_needle(u, Z);
    if (tid == 0) {
      uint64_t cum = 0;
      int cs = a.n_chunks - 1;
      for (int cc = 0; cc < a.n_chunks; ++cc) {
        const uint64_t zc = ws_b[(size_t)cc * W + use];
        if (cum + zc > t) { cs = cc; break; }
        cum += zc;
      }
      s_c = cs;
      s_before = cum;
    }
    __syncthreads();
    const int cs = s_c;
    const uint64_t before = s_before;
    // rescan chunk cs: contiguous segment per thread, exclusive scan over threads
    const int clo = cs * a.chunk, chi = min(V, clo + a.chunk);
    const int per = (chi - clo + 255) / 256;
    const int slo = clo + tid * per, shi = min(chi, slo + per);
    const float* Tr = Tb + (size_t)j * V;
    const float* Dr = (j < K && use == 0) ? Db + (size_t)j * V : nullptr;
    uint64_t seg = 0;
    for (int v = slo; v < shi; ++v) {
      const uint64_t ft = fix40(Tr[v]);
      if (Dr) {
        const uint64_t fd = fix40(Dr[v]);
        seg += ft > fd ? ft - fd : 0;
      } else {
        seg += ft;
      }
    }
    s_scan[tid] = seg;
    __syncthreads();
    if (tid == 0) {
      uint64_t run = before;
      for (int i = 0; i < 256; ++i) {
        const uint64_t x = s_scan[i];
        s_scan[i] = run;
        run += x;
      }
    }
    __syncthreads();
    uint64_t run = s_scan[tid];
    if (run <= t && slo < shi) {
      for (int v = slo; v < shi; ++v) {
        const uint64_t ft = fix40(Tr[v]);
        uint64_t w = ft;
        if (Dr) {
          const uint64_t fd = fix40(Dr[v]);
          w = ft > fd ? ft - fd : 0;
        }
        run += w;
        if (run > t) {
          s_tok = v;
          break;
        }
      }
    }
    __syncthreads();
  } else {
    if (tid == 0) s_tok = (int32_t)argmax_key_index(am);
    __syncthreads();
  }
  if (tid == 0) {
    const int tok = s_tok;
    for (int i = 0; i <= K; ++i) ob[i] = i < j ? db[i] : (i == j ? tok : -1);
    if (a.n_acc) a.n_acc[b] = j;
  }
}

void ar_choose_chunks(int B, int V, int* chunk, int* n_chunks) {
  int want = (512 + (B > 0 ? B : 1) - 1) / (B > 0 ? B : 1);  // blocks per sequence
  int by_size = (V + 1023) / 1024;
  int C = want < by_size ? want : by_size;
  if (C < 1) C = 1;
  int ch = (V + C - 1) / C;
  ch = (ch + 255) / 256 * 256;
  *chunk = ch;
  *n_chunks = (V + ch - 1) / ch;
}

hipError_t launch_accept_reject(const ArArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ar_partial_kernel, dim3(a.n_chunks, a.B), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ar_finish_kernel, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

// =============================================================== commit ==
// Keep the pending token and the n accepted drafts; the emitted token
// (replacement or bonus) becomes the next pending token ([en] Floor 4: slips
// after the first reject are torn up).  The draft cache keeps the rows whose
// tokens were committed: it processed [pending, d_1..d_{K-1}], so it is
// valid up to position LT + min(n, K-1).
__global__ void commit_kernel(DevState* st, int32_t* hist, int hist_cap, const int32_t* out,
                              const int32_t* n_acc, int drafted_k) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const int n = *n_acc;
  if (n < 0) return;
  const int LT = st->LT;
  if (LT + 1 + n >= hist_cap) {
    atomicOr(&st->err, kErrCapacity);
    return;
  }
  for (int i = 0; i <= n; ++i) hist[LT + 1 + i] = out[i];
  if (drafted_k > 0) st->LD = LT + (n + 1 < drafted_k ? n + 1 : drafted_k);
  st->LT = LT + n + 1;
}

hipError_t launch_commit(DevState* st, int32_t* hist, int hist_cap, const int32_t* out,
                         const int32_t* n_acc, int drafted_k, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, s, st, hist, hist_cap, out, n_acc,
                     drafted_k);
  return hipGetLastError();
}

// RoPE inverse frequencies theta^(-2j/hd), j < hd/2, in fp64.
__global__ void inv_freq_kernel(double* dst, int hd, double theta) {
  const int j = threadIdx.x + blockIdx.x * blockDim.x;
  if (j < hd / 2) dst[j] = pow(theta, -2.0 * (double)j / (double)hd);
}

hipError_t launch_inv_freq(double* dst, int hd, double theta, hipStream_t s) {
  hipLaunchKernelGGL(inv_freq_kernel, dim3((hd / 2 + 255) / 256), dim3(256), 0, s, dst, hd, theta);
  return hipGetLastError();
}

}  // namespace spec
