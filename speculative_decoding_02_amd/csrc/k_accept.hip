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
//  2. finish kernel, one block per sequence: take the decision (and the
//     final sample's uniform, drawn with the accept tests) that the partial
//     blocks recorded beside their sums, fold the chunk partials, find the
//     chunk holding the inverse-CDF needle
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
// none; K in greedy mode), whether the inputs read so far are invalid, and
// (sampling mode) the uniform of the final sample at position P + j.  Lane
// i <= K evaluates Philox once at P + i: word 1 is its accept test, word
// a.word the final sample's draw should the decision land on i.
SPEC_DEVICE void decide_first_reject(const ArArgs& a, int b, uint64_t P, int* s_j, int* s_err,
                                     uint32_t* s_u) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    const int K = a.K, V = a.V;
    const bool sample = !a.greedy;
    const float* Tb = a.T + (size_t)b * (K + 1) * V;
    const float* Db = a.D ? a.D + (size_t)b * K * V : nullptr;
    const int32_t* db = a.d + (size_t)b * K;
    // draft ids, then the gathered T_i(d_i), D_i(d_i) (issued before the
    // Philox rounds so their latency overlaps them)
    const int di = lane < K ? db[lane] : 0;
    const bool bad_d = lane < K && (di < 0 || di >= V);
    const bool gather = sample && lane < K && !bad_d;
    const float t = gather ? Tb[(size_t)lane * V + di] : 0.0f;
    const float q = gather ? Db[(size_t)lane * V + di] : 0.0f;
    // one Philox evaluation per lane 0..K, all lanes in step
    uint32_t u_acc = 0, u_fin = 0;
    if (sample && lane <= K) {
      const U64x4 w = philox4x64_10(P + lane, b, a.stream_id, 0, a.seed, 0);
      u_acc = (uint32_t)(w.w[1] >> 40);
      // a select, not w.w[a.word]: a runtime index would put the four words
      // in per-thread LDS, whose address needs the work-group sizes read from
      // the dispatch packet, on this path's critical chain
      const uint64_t wf = a.word == 0 ? w.w[0] : a.word == 1 ? w.w[1] : a.word == 2 ? w.w[2] : w.w[3];
      u_fin = (uint32_t)(wf >> 40);
    }
    bool stop = false, invalid = false;
    if (gather) {
      invalid = !prob_valid(t) || !prob_valid(q);
      const float rr = (float)u_acc * 0x1p-24f;
      stop = invalid || !((double)rr * (double)q < (double)t);
    }
    const uint64_t bd = __ballot(bad_d);
    const uint64_t st = __ballot(stop || bad_d);
    const int j = st ? __ffsll((long long)st) - 1 : K;
    const uint64_t inv = __ballot(invalid);
    const uint32_t u_j = (uint32_t)__shfl((int)u_fin, j);
    if (lane == 0) {
      *s_j = a.greedy ? K : j;
      *s_err = (bd != 0) || (!a.greedy && j < K && ((inv >> j) & 1));
      *s_u = u_j;
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

SPEC_DEVICE uint64_t wave_or_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v |= shfl_xor_u64(v, m);
  return v;
}

// Four reductions in one exchange: sums of a and b, maximum of c, OR of d.
SPEC_DEVICE void block_sum2_max_or(uint64_t& a, uint64_t& b, uint64_t& c, uint64_t& d, uint64_t* lds) {
  a = wave_sum_u64(a);
  b = wave_sum_u64(b);
  c = wave_max_u64(c);
  d = wave_or_u64(d);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    lds[4 * w] = a; lds[4 * w + 1] = b; lds[4 * w + 2] = c; lds[4 * w + 3] = d;
  }
  __syncthreads();
  a = lds[0] + lds[4] + lds[8] + lds[12];
  b = lds[1] + lds[5] + lds[9] + lds[13];
  c = max(max(lds[2], lds[6]), max(lds[10], lds[14]));
  d = lds[3] | lds[7] | lds[11] | lds[15];
  __syncthreads();
}

// The decision word each partial block stores with its sums: bit 0 an
// invalid value in its scanned rows, bit 1 an invalid draft or gathered
// probability, bits 8..15 the first reject j, bits 32..55 (sampling mode)
// the uniform u24 of the final sample.  Every block computes the same word
// apart from bit 0, so the OR of all chunks' words holds them all.
SPEC_DEVICE uint64_t decision_word(uint64_t bad, int err, int j, uint32_t u24) {
  return (bad ? 1ull : 0ull) | (err ? 2ull : 0ull) | ((uint64_t)j << 8) | ((uint64_t)u24 << 32);
}

SPEC_DEVICE uint64_t block_max_u64(uint64_t v, uint64_t* lds) {
  v = wave_max_u64(v);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint64_t r = max(max(lds[0], lds[1]), max(lds[2], lds[3]));
  __syncthreads();
  return r;
}

// weight of a token in the row being sampled: residual fix(T) - fix(D)
// (saturating), or the row itself
SPEC_DEVICE uint64_t token_weight(float tv, float dv, bool residual) {
  const uint64_t ft = fix40(tv);
  if (!residual) return ft;
  const uint64_t fd = fix40(dv);
  return ft > fd ? ft - fd : 0;
}

// Rows are read in passes of kArPass elements: every thread issues all
// kArSeg loads of a pass before using any, through a buffer resource over
// the row (V floats), so an element past the chunk reads as 0 with no
// fetch.  Any row alignment works (dword loads).
constexpr int kArSeg = 16;
constexpr int kArPass = kArThreads * kArSeg;
constexpr uint32_t kArOOB = 0x80000000u;
SPEC_DEVICE __amdgpu_buffer_rsrc_t row_rsrc(const float* row, int V) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, V * 4, 0x00020000);
}
SPEC_DEVICE float row_at(__amdgpu_buffer_rsrc_t r, int v, bool in) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)(in ? (uint32_t)v * 4 : kArOOB), 0, 0));
}

// The rule's kernels take the pointers their first loads need as leading
// scalar arguments (preloaded in SGPRs) and use them in place of the copies
// in the argument struct.
__global__ __launch_bounds__(kArThreads) void ar_partial_kernel(const DevState* st,
                                                               const uint64_t* pos, const int32_t* dd,
                                                               const float* T, const float* D,
                                                               ArArgs args) {
  ArArgs a = args;
  a.st = st; a.pos = pos; a.d = dd; a.T = T; a.D = D;
  __shared__ int32_t s_j, s_err;
  __shared__ uint32_t s_u;
  __shared__ uint64_t s_red[16];
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
  decide_first_reject(a, b, P, &s_j, &s_err, &s_u);
  // uniform across the block: in scalar registers, so the row's buffer
  // descriptor is too (a descriptor the compiler cannot prove uniform costs
  // a serial loop around every load)
  const int j = __builtin_amdgcn_readfirstlane(s_j);
  const int lo = c * a.chunk, hi = min(V, lo + a.chunk);

  if (!a.greedy) {
    // the chunk of the row to sample from: T_j and D_j after a reject at j,
    // else the bonus row T_K; integer sums and maxima, so the element order
    // (strided over threads, pass by pass) changes nothing
    uint64_t zr = 0, zt = 0, am = 0, bad = 0;
    if (!s_err) {
      const bool res = j < K;
      const __amdgpu_buffer_rsrc_t rT = row_rsrc(Tb + (size_t)j * V, V);
      const __amdgpu_buffer_rsrc_t rD = res ? row_rsrc(Db + (size_t)j * V, V) : rT;
      for (int base = lo; base < hi; base += kArPass) {
        float tv[kArSeg], dv[kArSeg];
#pragma unroll
        for (int q = 0; q < kArSeg; ++q) {
          const int v = base + tid + q * kArThreads;
          tv[q] = row_at(rT, v, v < hi);
          dv[q] = res ? row_at(rD, v, v < hi) : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < kArSeg; ++q) {
          const int v = base + tid + q * kArThreads;
          if (v >= hi) continue;
          if (!prob_valid(tv[q]) || (res && !prob_valid(dv[q]))) {
            bad = 1;
            continue;
          }
          const uint64_t ft = fix40(tv[q]);
          am = max(am, argmax_key(tv[q], (uint32_t)v));
          zt += ft;
          if (res) {
            const uint64_t fd = fix40(dv[q]);
            zr += ft > fd ? ft - fd : 0;
          }
        }
      }
      if (!res) zr = zt;  // the bonus row samples from T_K itself
    }
    block_sum2_max_or(zr, zt, am, bad, s_red);
    if (tid == 0) {
      p[0] = zr; p[1] = zt; p[2] = am; p[3] = decision_word(bad, s_err, j, s_u);
    }
  } else {
    // per-row argmax keys of this chunk, rows 0..K, and an invalid-value flag
    uint64_t bad = 0;
    for (int i = 0; i <= K; ++i) {
      const __amdgpu_buffer_rsrc_t rT = row_rsrc(Tb + (size_t)i * V, V);
      uint64_t am = 0;
      for (int base = lo; base < hi; base += kArPass) {
        float tv[kArSeg];
#pragma unroll
        for (int q = 0; q < kArSeg; ++q) {
          const int v = base + tid + q * kArThreads;
          tv[q] = row_at(rT, v, v < hi);
        }
#pragma unroll
        for (int q = 0; q < kArSeg; ++q) {
          const int v = base + tid + q * kArThreads;
          if (v >= hi) continue;
          if (!prob_valid(tv[q])) {
            bad = 1;
            continue;
          }
          am = max(am, argmax_key(tv[q], (uint32_t)v));
        }
      }
      am = block_max_u64(am, s_red);
      if (tid == 0) p[i] = am;
    }
    bad = block_max_u64(bad, s_red);
    if (tid == 0) p[K + 1] = decision_word(bad, s_err, K, 0);
  }
}

__global__ __launch_bounds__(kArThreads) void ar_finish_kernel(const uint64_t* ws, const int32_t* dd,
                                                              const float* T, const float* D,
                                                              ArArgs args) {
  ArArgs a = args;
  a.ws = const_cast<uint64_t*>(ws); a.d = dd; a.T = T; a.D = D;
  __shared__ int32_t s_tok, s_c, s_found;
  __shared__ uint64_t s_red[16], s_before, s_total;
  __shared__ int32_t s_am[64];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int K = a.K, V = a.V, C = a.n_chunks;
  const float* Tb = a.T + (size_t)b * (K + 1) * V;
  const float* Db = a.D ? a.D + (size_t)b * K * V : nullptr;
  const int32_t* db = a.d + (size_t)b * K;
  const int W = ar_ws_words(K);
  const uint64_t* ws_b = a.ws + (size_t)b * C * W;
  int32_t* ob = a.out + (size_t)b * (K + 1);

  if (a.greedy) {
    uint64_t badv = 0;
    for (int cc = tid; cc < C; cc += kArThreads) badv |= ws_b[(size_t)cc * W + K + 1];
    badv = block_max_u64(badv, s_red);  // every chunk's word has the same bits 1..
    const bool bad = (badv & 3) != 0;
    for (int i = 0; i <= K; ++i) {
      uint64_t acc = 0;
      for (int cc = tid; cc < C; cc += kArThreads) acc = max(acc, ws_b[(size_t)cc * W + i]);
      acc = block_max_u64(acc, s_red);
      if (tid == 0) s_am[i] = (int32_t)argmax_key_index(acc);
    }
    __syncthreads();
    if (tid == 0) {
      const bool err = bad;
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
  // thread tid owns chunks 2 tid and 2 tid + 1 (C <= kArMaxChunks): their
  // partials serve both the fold and the needle's chunk search below
  const int c0 = 2 * tid, c1 = 2 * tid + 1;
  uint64_t q0[4] = {0, 0, 0, 0}, q1[4] = {0, 0, 0, 0};
  if (c0 < C) {
#pragma unroll
    for (int w = 0; w < 4; ++w) q0[w] = ws_b[(size_t)c0 * W + w];
  }
  if (c1 < C) {
#pragma unroll
    for (int w = 0; w < 4; ++w) q1[w] = ws_b[(size_t)c1 * W + w];
  }
  uint64_t zr = q0[0] + q1[0], zt = q0[1] + q1[1], am = max(q0[2], q1[2]), word = q0[3] | q1[3];
  block_sum2_max_or(zr, zt, am, word, s_red);
  const int j = __builtin_amdgcn_readfirstlane((int)((word >> 8) & 0xFF));
  const uint32_t u = (uint32_t)(word >> 32);
  if (word & 3) {
    if (tid <= K) ob[tid] = -1;
    if (tid == 0 && a.n_acc) a.n_acc[b] = -1;
    return;
  }
  // weights to sample: residual (or bonus row), else fix(T_j), else the argmax
  const int use = __builtin_amdgcn_readfirstlane(zr > 0 ? 0 : ((j < K && zt > 0) ? 1 : 2));
  if (tid == 0) {
    s_tok = (int32_t)argmax_key_index(am);
    s_found = 0;
  }
  if (use < 2) {
    const uint64_t t = icdf_needle(u, use == 0 ? zr : zt);
    // chunk holding the needle
    const uint64_t z0 = q0[use], z1 = q1[use];
    const uint64_t ex = block_exclusive_scan_u64_256(z0 + z1, s_red);
    if (ex <= t && t < ex + z0) {
      s_c = c0;
      s_before = ex;
    } else if (ex + z0 <= t && t < ex + z0 + z1) {
      s_c = c1;
      s_before = ex + z0;
    }
    __syncthreads();
    const int cs = __builtin_amdgcn_readfirstlane(s_c);
    uint64_t before = s_before;
    // rescan chunk cs in passes: thread tid owns the contiguous segment
    // [base + kArSeg tid, + kArSeg) of a pass, loaded whole into registers;
    // a block prefix sum over the segments locates the needle's segment and
    // its thread finds the token among its registers
    const int clo = cs * a.chunk, chi = min(V, clo + a.chunk);
    const bool res = j < K && use == 0;
    const __amdgpu_buffer_rsrc_t rT = row_rsrc(Tb + (size_t)j * V, V);
    const __amdgpu_buffer_rsrc_t rD = res ? row_rsrc(Db + (size_t)j * V, V) : rT;
    for (int base = clo; base < chi; base += kArPass) {  // uniform
      const int v0 = base + kArSeg * tid;
      float tv[kArSeg], dv[kArSeg];
#pragma unroll
      for (int q = 0; q < kArSeg; ++q) {
        tv[q] = row_at(rT, v0 + q, v0 + q < chi);
        dv[q] = res ? row_at(rD, v0 + q, v0 + q < chi) : 0.0f;
      }
      uint64_t w[kArSeg], seg = 0;
#pragma unroll
      for (int q = 0; q < kArSeg; ++q) {
        w[q] = v0 + q < chi ? token_weight(tv[q], dv[q], res) : 0;
        seg += w[q];
      }
      const uint64_t run0 = before + block_exclusive_scan_u64_256(seg, s_red);
      if (run0 <= t && t < run0 + seg) {
        uint64_t run = run0;
#pragma unroll
        for (int q = 0; q < kArSeg; ++q) {
          run += w[q];
          if (run > t) {
            s_tok = v0 + q;
            s_found = 1;
            break;
          }
        }
      }
      if (tid == kArThreads - 1) s_total = run0 - before + seg;
      __syncthreads();
      if (s_found) break;
      before += s_total;
      __syncthreads();
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
                     a.st, a.pos, a.d, a.T, a.D, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ar_finish_kernel, dim3(a.B), dim3(kArThreads), 0, s, (const uint64_t*)a.ws, a.d,
                     a.T, a.D, a);
  return hipGetLastError();
}

}  // namespace spec
