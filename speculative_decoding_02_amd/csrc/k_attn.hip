// k_attn.hip -- causal attention of the pass's query rows against the paged
// KV cache.
//
// Row r (position pos0 + r) attends to keys 0..pos0+r: row i of the verify
// pass sees the context plus drafts d_1..d_{i-1}, which is what makes its
// output the target distribution T_i = T(. | x, d_1..d_{i-1}) ([int]
// algorithm core, Step 2).  Grouped-query heads: query head h reads KV head
// h / (n_q / n_kv); all query heads of a group and all rows share one read of
// each key/value chunk.
//
// Two launches, no inter-block waiting: (1) workgroup (chunk c, kv head h)
// handles 64 keys and writes, per query, (max score, sum of exp,
// unnormalised value sum); (2) one merge block per (kv head, slice) combines
// the chunks in chunk order (deterministic) and writes the output rows as the
// packed A operand of the O projection.
#include "kernels.h"

namespace spec {

size_t attn_lds_bytes(int hd, int qg_max) {
  return (size_t)2 * kAttnChunk * hd * sizeof(uint16_t)  // K, V chunk (bf16)
         + (size_t)qg_max * hd * sizeof(float)           // queries
         + (size_t)qg_max * kAttnChunk * sizeof(float);  // probabilities
}

constexpr int kMaxQPerWave = 16;

__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, h = blockIdx.y;
  const int hd = a.hd;
  const int G = a.n_q / a.n_kv;
  const int n_rows = a.rows->n_rows, pos0 = a.rows->pos0;
  const int n_keys = pos0 + n_rows;
  const int n_active = (n_keys + kAttnChunk - 1) / kAttnChunk;
  if (n_rows <= 0 || c >= n_active) return;
  const int QG = G * n_rows;  // query vectors: qi = r * G + gi

  uint16_t* Ks = (uint16_t*)lds;
  uint16_t* Vs = Ks + kAttnChunk * hd;
  float* Qs = (float*)(Vs + kAttnChunk * hd);
  float* Ps = Qs + (size_t)a.qg_max * hd;

  // ---- load the key/value chunk (16-byte vectors) and the queries ---------
  const int t0 = c * kAttnChunk;
  const int vec_per_row = hd / 8;
  for (int idx = tid; idx < kAttnChunk * vec_per_row; idx += 256) {
    const int i = idx / vec_per_row, e = (idx % vec_per_row) * 8;
    const int t = t0 + i;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (t < n_keys) {
      const int blk = a.block_table[t / kBlock];
      const size_t off = (((size_t)blk * a.n_kv + h) * kBlock + t % kBlock) * hd + e;
      kv = *(const uint4*)(a.k_cache + off);
      vv = *(const uint4*)(a.v_cache + off);
    }
    *(uint4*)(Ks + i * hd + e) = kv;
    *(uint4*)(Vs + i * hd + e) = vv;
  }
  for (int idx = tid; idx < QG * hd; idx += 256) {
    const int qi = idx / hd, e = idx % hd;
    const int r = qi / G, gi = qi % G;
    Qs[idx] = a.q[(size_t)r * a.n_q * hd + (size_t)(h * G + gi) * hd + e];
  }
  __syncthreads();

  // ---- scores: lane = key, wave = every 4th query -------------------------
  const float scale = 1.0f / sqrtf((float)hd);
  const int t = t0 + lane;
  float s[kMaxQPerWave];
#pragma unroll
  for (int qq = 0; qq < kMaxQPerWave; ++qq) s[qq] = 0.0f;
  for (int e = 0; e < hd; e += 8) {
    const uint4 kr = *(const uint4*)(Ks + lane * hd + e);
    const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
    float kf[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) kf[x] = bf16_to_f32((uint16_t)(kw[x >> 1] >> ((x & 1) * 16)));
#pragma unroll
    for (int qq = 0; qq < kMaxQPerWave; ++qq) {
      const int qi = wave + 4 * qq;
      if (qi < QG) {
        const float4 q0 = *(const float4*)(Qs + qi * hd + e);
        const float4 q1 = *(const float4*)(Qs + qi * hd + e + 4);
        s[qq] += q0.x * kf[0] + q0.y * kf[1] + q0.z * kf[2] + q0.w * kf[3] + q1.x * kf[4] +
                 q1.y * kf[5] + q1.z * kf[6] + q1.w * kf[7];
      }
    }
  }
  // softmax pieces of this chunk, per query
  float* my_ws = a.ws + ((size_t)h * a.max_chunks + c) * a.qg_max * (hd + 2);
#pragma unroll
  for (int qq = 0; qq < kMaxQPerWave; ++qq) {
    const int qi = wave + 4 * qq;
    if (qi < QG) {
      const int r = qi / G;
      const bool vis = t < n_keys && t <= pos0 + r;
      const float sc = vis ? s[qq] * scale : -INFINITY;
      const float mx = wave_max_f32(sc);
      const float p = (vis && mx != -INFINITY) ? expf(sc - mx) : 0.0f;
      const float l = wave_sum_f32(p);
      Ps[qi * kAttnChunk + lane] = p;
      if (lane == 0) {
        my_ws[(size_t)qi * (hd + 2) + 0] = mx;
        my_ws[(size_t)qi * (hd + 2) + 1] = l;
      }
    }
  }
  __syncthreads();

  // ---- unnormalised value sums of the chunk --------------------------------
  for (int idx = tid; idx < QG * hd; idx += 256) {
    const int qi = idx / hd, e = idx % hd;
    const float* pr = Ps + qi * kAttnChunk;
    float acc = 0.0f;
    for (int i = 0; i < kAttnChunk; ++i) acc += pr[i] * bf16_to_f32(Vs[i * hd + e]);
    my_ws[(size_t)qi * (hd + 2) + 2 + e] = acc;
  }
}

// Merge the chunks of kv head h in chunk order; each thread produces 8
// consecutive dims of one query vector and stores them packed (hi/lo bf16).
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int h = blockIdx.x;
  const int hd = a.hd, G = a.n_q / a.n_kv;
  const int n_rows = a.rows->n_rows, pos0 = a.rows->pos0;
  const int n_keys = pos0 + n_rows;
  const int n_active = (n_keys + kAttnChunk - 1) / kAttnChunk;
  if (n_rows <= 0) return;
  const int QG = G * n_rows, per = hd / 8;
  const int idx = blockIdx.y * blockDim.x + threadIdx.x;
  if (idx >= QG * per) return;
  const int qi = idx / per, e0 = (idx % per) * 8;
  const float* base = a.ws + (size_t)h * a.max_chunks * a.qg_max * (hd + 2) + (size_t)qi * (hd + 2);
  const size_t cstride = (size_t)a.qg_max * (hd + 2);
  float M = -INFINITY;
  for (int cc = 0; cc < n_active; ++cc) M = fmaxf(M, base[cc * cstride]);
  float L = 0.0f, O[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int cc = 0; cc < n_active; ++cc) {
    const float* pc = base + cc * cstride;
    const float m = pc[0];
    if (m == -INFINITY) continue;
    const float w = expf(m - M);
    L += pc[1] * w;
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] += pc[2 + e0 + e] * w;
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int e = 0; e < 8; ++e) O[e] *= inv;
  const int r = qi / G, gi = qi % G;
  apack_store8(a.Ap_out, r, (h * G + gi) * hd + e0, O);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_partial_kernel, dim3(a.max_chunks, a.n_kv), dim3(256),
                     attn_lds_bytes(a.hd, a.qg_max), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per_head = a.qg_max * (a.hd / 8);
  hipLaunchKernelGGL(attn_merge_kernel, dim3(a.n_kv, (per_head + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace spec
