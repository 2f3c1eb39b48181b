// k_ngram.hip -- prompt-lookup (n-gram) drafter on the device.
//
// [en] Floor 6 ([zh] Level 6): n-gram approaches such as prompt lookup draft
// by searching the preceding text for a chunk that is likely to repeat and
// proposing what followed it; the verification rule is the same whatever the
// draft's source.  The committed history hist[0..L] (hist[L] the pending
// token) is searched for the latest earlier occurrence of its own last n
// tokens, the longest n <= n_max first; the draft is the text that followed
// that occurrence, repeated with its period p = L - j when it is shorter than
// K (the continuation of a repeating text), or the pending token when nothing
// repeats.  The drafter is deterministic, so its draft distributions are
// one-hot rows: with them the accept test passes a draft with probability
// T_i(d_i) and a reject samples T_i with d_i's mass removed.
//
// Every workgroup runs the (cheap) search itself, so no workgroup waits for
// another: each then writes its share of the one-hot rows, and workgroup 0
// the tokens.  A batch of sequences runs in one launch, grid.y indexing the
// sequence.
#include "kernels.h"

namespace spec {

constexpr int kNgramThreads = 256;
constexpr int kNgramTile = 4096;  // history tokens staged in LDS per pass

__global__ __launch_bounds__(kNgramThreads) void ngram_draft_kernel(NgramArgs a) {
  __shared__ int32_t s_hist[kNgramTile + kNgramMaxN];
  __shared__ int32_t s_key[kNgramMaxN];
  __shared__ unsigned long long s_best[kNgramThreads / 64];
  __shared__ int32_t s_d[kNgramMaxK];
  const int tid = threadIdx.x;
  {  // this workgroup's sequence
    const int b = blockIdx.y;
    a.st += b;
    a.hist += (size_t)b * a.hist_cap;
    a.d += (size_t)b * a.K;
    if (a.D != nullptr) a.D += (size_t)b * a.K * a.V;
  }
  int L = a.st->LT;
  if (L < 0 || L >= a.hist_cap) L = 0;  // a corrupt state is flagged elsewhere; stay in bounds
  const int nmax = min(a.n_max, L);
  if (tid < kNgramMaxN) s_key[tid] = tid <= L ? a.hist[L - tid] : -1;  // key[t] = hist[L - t]

  // best = (match length m, position j) maximised lexicographically, where
  // hist[j - t] == hist[L - t] for t < m, m <= nmax, j < L.
  unsigned long long best = 0;
  for (int t0 = 0; t0 < L; t0 += kNgramTile) {
    // stage hist[t0 - kNgramMaxN, t0 + kNgramTile) (clipped to [0, L))
    __syncthreads();
    for (int i = tid; i < kNgramTile + kNgramMaxN; i += kNgramThreads) {
      const int src = t0 - kNgramMaxN + i;
      s_hist[i] = (src >= 0 && src < L) ? a.hist[src] : -1;
    }
    __syncthreads();
    const int t1 = min(L, t0 + kNgramTile);
    for (int j = t0 + tid; j < t1; j += kNgramThreads) {
      int m = 0;
      while (m < nmax && m <= j && s_hist[j - m - t0 + kNgramMaxN] == s_key[m]) ++m;
      if (m > 0) {
        const unsigned long long key = ((unsigned long long)m << 32) | (unsigned)j;
        best = key > best ? key : best;
      }
    }
  }
  // block maximum
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if ((tid & 63) == 0) s_best[tid >> 6] = best;
  __syncthreads();
  best = s_best[0];
#pragma unroll
  for (int w = 1; w < kNgramThreads / 64; ++w) best = s_best[w] > best ? s_best[w] : best;
  const int n = (int)(best >> 32), j = (int)(best & 0xffffffffu);
  if (tid < a.K) {
    const int32_t tok = n > 0 ? a.hist[j + 1 + tid % (L - j)] : a.hist[L];
    s_d[tid] = tok;
    if (blockIdx.x == 0) a.d[tid] = tok;
  }
  __syncthreads();
  if (a.D != nullptr) {  // one-hot rows, float4 at a time (V % 4 == 0)
    const size_t n4 = (size_t)a.K * a.V / 4;
    for (size_t i = (size_t)blockIdx.x * kNgramThreads + tid; i < n4;
         i += (size_t)gridDim.x * kNgramThreads) {
      const size_t e = i * 4;
      const int row = (int)(e / a.V), col = (int)(e % a.V);
      const int t = s_d[row] - col;
      ((float4*)a.D)[i] = make_float4(t == 0 ? 1.f : 0.f, t == 1 ? 1.f : 0.f, t == 2 ? 1.f : 0.f,
                                      t == 3 ? 1.f : 0.f);
    }
  }
}

hipError_t launch_ngram_draft(const NgramArgs& a, hipStream_t s) {
  if (a.K < 1 || a.K > kNgramMaxK || a.n_max < 1 || a.n_max > kNgramMaxN || a.V % 4 != 0)
    return hipErrorInvalidValue;
  const size_t n4 = (size_t)a.K * a.V / 4;
  size_t blocks = (n4 + kNgramThreads * 4 - 1) / (kNgramThreads * 4);
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  const int B = a.B > 1 ? a.B : 1;
  hipLaunchKernelGGL(ngram_draft_kernel, dim3((unsigned)blocks, (unsigned)B), dim3(kNgramThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace spec
