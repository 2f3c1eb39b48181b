// k_accept.hip -- the accept/reject rule ([int] algorithm core Steps 3-4;
// [en] Floors 4-5), also used to sample draft tokens.
//
// Per sequence b, in two launches (no block waits on another):
//  1. partial kernel, one block per (vocabulary chunk, sequence): decide the
//     K exact accept tests r_i * D_i(d_i) < T_i(d_i) (r_i = Philox w1 at the
//     draft's position); a wave ballot gives the first reject j (j = K:
//     none).  Then sum, over the chunk, the integer weights of the row to
//     sample from: the residual fix(T_j) - fix(D_j) (saturating, 2^-40 grid)
//     on a reject, else the bonus row fix(T_K).  The fallbacks (sum of
//     fix(T_j), argmax of the row) are gathered in the same pass.
//  2. finish kernel, one block per sequence: repeat the accept tests, fold
//     the chunk partials, find the chunk holding the inverse-CDF needle
//     floor(u24 * Z / 2^24) (u24 = Philox w2 at the decided position) with a
//     block prefix sum, rescan that chunk and write the emitted tokens.
// Every sum is over 64-bit integers, so the result does not depend on the
// reduction order.  Greedy mode replaces the sums by per-chunk argmaxes of
// every row.  K = 0 samples one row (draft tokens, word w0).
#include "kernels.h"

namespace spec {

constexpr int kArThreads = 256;
constexpr int kArMaxChunks = 2 * kArThreads;  // the finish kernel scans 2 chunks per thread

// Accept tests and draft validation (wave 0).  Writes j (first reject, K if
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

SPEC_DEVICE uint64_t block_sum_u64(uint64_t v, uint64_t* lds) {
  v = wave_sum_u64(v);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint64_t r = lds[0] + lds[1] + lds[2] + lds[3];
  __syncthreads();
  return r;
}

SPEC_DEVICE uint64_t block_max_u64(uint64_t v, uint64_t* lds) {
  v = wave_max_u64(v);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint64_t r = max(max(lds[0], lds[1]), max(lds[2], lds[3]));
  __syncthreads();
  return r;
}

// weight of token v in the row being sampled: residual, or the row itself
SPEC_DEVICE uint64_t row_weight(const float* Tr, const float* Dr, int v) {
  const uint64_t ft = fix40(Tr[v]);
  if (!Dr) return ft;
  const uint64_t fd = fix40(Dr[v]);
  return ft > fd ? ft - fd : 0;
}

__global__ __launch_bounds__(kArThreads) void ar_partial_kernel(ArArgs a) {
  __shared__ int32_t s_j, s_err;
  __shared__ uint64_t s_red[4];
  const int tid = threadIdx.x;
  // one block per (chunk, sequence), flattened in x (grid.y is too narrow
  // for large batches)
  const int c = (int)(blockIdx.x % (unsigned)a.n_chunks), b = (int)(blockIdx.x / (unsigned)a.n_chunks);
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
      for (int v = lo + tid; v < hi; v += kArThreads) {
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
    zr = block_sum_u64(zr, s_red);
    zt = block_sum_u64(zt, s_red);
    am = block_max_u64(am, s_red);
    bad = block_max_u64(bad, s_red);
    if (tid == 0) {
      p[0] = zr; p[1] = zt; p[2] = am; p[3] = bad;
    }
  } else {
    // per-row argmax keys of this chunk, rows 0..K, and an invalid-value flag
    uint64_t bad = 0;
    for (int i = 0; i <= K; ++i) {
      const float* Tr = Tb + (size_t)i * V;
      uint64_t am = 0;
      for (int v = lo + tid; v < hi; v += kArThreads) {
        const float tv = Tr[v];
        if (!prob_valid(tv)) { bad = 1; continue; }
        am = max(am, argmax_key(tv, (uint32_t)v));
      }
      am = block_max_u64(am, s_red);
      if (tid == 0) p[i] = am;
    }
    bad = block_max_u64(bad, s_red);
    if (tid == 0) p[K + 1] = bad;
  }
}

__global__ __launch_bounds__(kArThreads) void ar_finish_kernel(ArArgs a) {
  __shared__ int32_t s_j, s_err, s_tok, s_c;
  __shared__ uint64_t s_red[4], s_before;
  __shared__ int32_t s_am[64];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int K = a.K, V = a.V, C = a.n_chunks;
  const uint64_t P = seq_pos(a, b);
  const float* Tb = a.T + (size_t)b * (K + 1) * V;
  const float* Db = a.D ? a.D + (size_t)b * K * V : nullptr;
  const int32_t* db = a.d + (size_t)b * K;
  const int W = ar_ws_words(K);
  const uint64_t* ws_b = a.ws + (size_t)b * C * W;
  int32_t* ob = a.out + (size_t)b * (K + 1);
  decide_first_reject(a, b, P, &s_j, &s_err);
  const int j = s_j;

  if (a.greedy) {
    uint64_t badv = 0;
    for (int cc = tid; cc < C; cc += kArThreads) badv |= ws_b[(size_t)cc * W + K + 1];
    const bool bad = block_max_u64(badv, s_red) != 0;
    for (int i = 0; i <= K; ++i) {
      uint64_t acc = 0;
      for (int cc = tid; cc < C; cc += kArThreads) acc = max(acc, ws_b[(size_t)cc * W + i]);
      acc = block_max_u64(acc, s_red);
      if (tid == 0) s_am[i] = (int32_t)argmax_key_index(acc);
    }
    __syncthreads();
    if (tid == 0) {
      const bool err = s_err || bad;
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

  // sampling: fold the chunk partials (integer sums / maxima: order-free)
  uint64_t zr = 0, zt = 0, am = 0, bad = 0;
  for (int cc = tid; cc < C; cc += kArThreads) {
    const uint64_t* p = ws_b + (size_t)cc * W;
    zr += p[0];
    zt += p[1];
    am = max(am, p[2]);
    bad |= p[3];
  }
  zr = block_sum_u64(zr, s_red);
  zt = block_sum_u64(zt, s_red);
  am = block_max_u64(am, s_red);
  bad = block_max_u64(bad, s_red);
  if (bad || s_err) {
    if (tid <= K) ob[tid] = -1;
    if (tid == 0 && a.n_acc) a.n_acc[b] = -1;
    return;
  }
  // weights to sample: residual (or bonus row), else fix(T_j), else the argmax
  const int use = zr > 0 ? 0 : ((j < K && zt > 0) ? 1 : 2);
  if (tid == 0) s_tok = (int32_t)argmax_key_index(am);
  if (use < 2) {
    const uint32_t u = uniform_u24(a.seed, P + j, b, a.stream_id, a.word);
    const uint64_t t = icdf_needle(u, use == 0 ? zr : zt);
    // chunk holding the needle: thread owns chunks 2*tid and 2*tid + 1
    const int c0 = 2 * tid, c1 = 2 * tid + 1;
    const uint64_t z0 = c0 < C ? ws_b[(size_t)c0 * W + use] : 0;
    const uint64_t z1 = c1 < C ? ws_b[(size_t)c1 * W + use] : 0;
    const uint64_t ex = block_exclusive_scan_u64_256(z0 + z1, s_red);
    if (ex <= t && t < ex + z0) {
      s_c = c0;
      s_before = ex;
    } else if (ex + z0 <= t && t < ex + z0 + z1) {
      s_c = c1;
      s_before = ex + z0;
    }
    __syncthreads();
    const int cs = s_c;
    const uint64_t before = s_before;
    // rescan chunk cs: one contiguous segment per thread, block prefix sum
    const int clo = cs * a.chunk, chi = min(V, clo + a.chunk);
    const int per = (chi - clo + kArThreads - 1) / kArThreads;
    const int slo = clo + tid * per, shi = min(chi, slo + per);
    const float* Tr = Tb + (size_t)j * V;
    const float* Dr = (j < K && use == 0) ? Db + (size_t)j * V : nullptr;
    uint64_t seg = 0;
    for (int v = slo; v < shi; ++v) seg += row_weight(Tr, Dr, v);
    uint64_t run = before + block_exclusive_scan_u64_256(seg, s_red);
    if (run <= t && t < run + seg) {
      for (int v = slo; v < shi; ++v) {
        run += row_weight(Tr, Dr, v);
        if (run > t) {
          s_tok = v;
          break;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int tok = s_tok;
    for (int i = 0; i <= K; ++i) ob[i] = i < j ? db[i] : (i == j ? tok : -1);
    if (a.n_acc) a.n_acc[b] = j;
  }
}

void ar_choose_chunks(int B, int V, int* chunk, int* n_chunks) {
  const int Bp = B > 0 ? B : 1;
  const int want = (512 + Bp - 1) / Bp;  // blocks per sequence
  const int by_size = (V + 1023) / 1024;
  int C = want < by_size ? want : by_size;
  if (C < 1) C = 1;
  if (C > kArMaxChunks) C = kArMaxChunks;
  int ch = (V + C - 1) / C;
  ch = (ch + 255) / 256 * 256;
  *chunk = ch;
  *n_chunks = (V + ch - 1) / ch;
}

hipError_t launch_accept_reject(const ArArgs& a, hipStream_t s) {
  if (a.n_chunks > kArMaxChunks || a.K > 63 || (long long)a.n_chunks * a.B > 0x7fffffffLL)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(ar_partial_kernel, dim3((unsigned)(a.n_chunks * a.B)), dim3(kArThreads), 0, s,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ar_finish_kernel, dim3(a.B), dim3(kArThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace spec
