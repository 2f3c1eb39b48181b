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
// Two launches, no inter-block waiting:
//  (1) partial kernel, workgroup (64-key chunk c, kv head h): scores and the
//      probability-weighted value sums on v_mfma_f32_16x16x32_bf16.  Queries
//      and probabilities enter as bf16 high/low row pairs, keys and values
//      as the cache's bf16 high/low planes (two MFMAs per fragment), so every
//      operand keeps ~16 mantissa bits.  Per query it writes (max score, sum
//      of exp, unnormalised value sum) for the chunk.
//  (2) merge kernel: combines the chunks in chunk order (deterministic) and
//      writes the output rows as the packed A operand of the O projection.
#include "kernels.h"

namespace spec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

SPEC_DEVICE bf16x8_t as_bf16x8_a(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS layout of the partial kernel (bf16 unless noted):
//   Kt [2][64 keys][E32 + 8]    keys (high, low planes), e padded to a
//                               multiple of 32 (+8 against bank conflicts)
//   Vt [2][E16][64 + 8]         values transposed (e-major), for B fragments
//   Qa [n_qt][n_es][64][8]      query A fragments (hi rows 0-7, lo rows 8-15);
//                               reused as S [qg_max][64] fp32 after the scores
//   Pa [n_qt][2][64][8]         probability A fragments
struct AttnLds {
  int E32, E16, n_es, n_et, n_qt, kstride, vstride;
  size_t kplane, vplane;  // elements per plane
  size_t off_v, off_q, off_p, bytes;
};

__host__ __device__ inline AttnLds attn_lds(int hd, int qg_max) {
  AttnLds L;
  L.E32 = (hd + 31) / 32 * 32;
  L.E16 = (hd + 15) / 16 * 16;
  L.n_es = L.E32 / 32;
  L.n_et = L.E16 / 16;
  L.n_qt = (qg_max + 7) / 8;
  L.kstride = L.E32 + 8;
  L.vstride = kAttnChunk + 8;
  L.kplane = (size_t)kAttnChunk * L.kstride;
  L.vplane = (size_t)L.E16 * L.vstride;
  const size_t qb = (size_t)L.n_qt * L.n_es * 1024;
  const size_t sb = (size_t)qg_max * kAttnChunk * 4;
  L.off_v = 2 * L.kplane * 2;
  L.off_q = L.off_v + 2 * L.vplane * 2;
  L.off_p = L.off_q + (qb > sb ? qb : sb);
  L.bytes = L.off_p + (size_t)L.n_qt * 2 * 1024;
  return L;
}

size_t attn_lds_bytes(int hd, int qg_max) { return attn_lds(hd, qg_max).bytes; }

// element index of (row m of 16, k of 32) inside one 1 KiB A fragment
SPEC_DEVICE int afrag_index(int row, int kk) { return (row + 16 * (kk >> 3)) * 8 + (kk & 7); }

__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = blockIdx.x, h = blockIdx.y;
  const int hd = a.hd;
  const int G = a.n_q / a.n_kv;
  const int n_rows = a.rows->n_rows, pos0 = a.rows->pos0;
  const int n_keys = pos0 + n_rows;
  const int n_active = (n_keys + kAttnChunk - 1) / kAttnChunk;
  if (n_rows <= 0 || c >= n_active) return;
  const int QG = G * n_rows;  // query vectors: qi = r * G + gi
  const AttnLds L = attn_lds(hd, a.qg_max);
  uint16_t* Kt = (uint16_t*)lds;
  uint16_t* Vt = (uint16_t*)(lds + L.off_v);
  uint16_t* Qa = (uint16_t*)(lds + L.off_q);
  float* S = (float*)(lds + L.off_q);  // aliases Qa after the scores
  uint16_t* Pa = (uint16_t*)(lds + L.off_p);

  // ---- stage keys (row-major), values (transposed), queries (hi/lo) -------
  const int t0 = c * kAttnChunk;
  const int vec_per_row = L.E32 / 8;
  for (int idx = tid; idx < 2 * kAttnChunk * vec_per_row; idx += 256) {
    const int part = idx / (kAttnChunk * vec_per_row);
    const int rest = idx % (kAttnChunk * vec_per_row);
    const int i = rest / vec_per_row, e = (rest % vec_per_row) * 8;
    const int t = t0 + i;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (t < n_keys && e < hd) {
      const int blk = a.block_table[t / kBlock];
      const size_t off = kv_index(blk, a.n_kv, h, t % kBlock, hd, part, e);
      kv = *(const uint4*)(a.k_cache + off);
      vv = *(const uint4*)(a.v_cache + off);
    }
    *(uint4*)(Kt + part * L.kplane + i * L.kstride + e) = kv;
    if (e < L.E16) {
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
      uint16_t* vp = Vt + part * L.vplane;
#pragma unroll
      for (int x = 0; x < 8; ++x)
        if (e + x < L.E16) vp[(e + x) * L.vstride + i] = (uint16_t)(w[x >> 1] >> ((x & 1) * 16));
    }
  }
  // query fragments: (q-tile qt, e-step es, lane) -> 8 e of one query, hi or lo
  for (int idx = tid; idx < L.n_qt * L.n_es * 64; idx += 256) {
    const int ln = idx & 63, es = (idx >> 6) % L.n_es, qt = (idx >> 6) / L.n_es;
    const int row = ln & 15, qi = qt * 8 + (row & 7), part = row >> 3;
    const int e0 = es * 32 + (ln >> 4) * 8;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (qi < QG) {
      const int r = qi / G, gi = qi % G;
      const float* qp = a.q + (size_t)r * a.n_q * hd + (size_t)(h * G + gi) * hd;
#pragma unroll
      for (int x = 0; x < 8; ++x) v[x] = e0 + x < hd ? qp[e0 + x] : 0.0f;
    }
    uint16_t hv[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const uint16_t hi = f32_to_bf16_rne(v[x]);
      hv[x] = part ? f32_to_bf16_rne(v[x] - bf16_to_f32(hi)) : hi;
    }
    *(uint4*)(Qa + (size_t)idx * 8) =
        make_uint4(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]), pack_bf16x2(hv[4], hv[5]),
                   pack_bf16x2(hv[6], hv[7]));
  }
  __syncthreads();

  // ---- scores S = Q K^T: wave w owns keys 16w..16w+15 ----------------------
  const int n_qt = (QG + 7) / 8;
  floatx4 sacc[8];
#pragma unroll
  for (int qt = 0; qt < 8; ++qt) sacc[qt] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int es = 0; es < L.n_es; ++es) {
    // B fragments: lane l -> key 16w + l%16, e = 32es + 8(l/16) .. +7, high
    // and low planes of the key
    const size_t koff = (size_t)(wave * 16 + (lane & 15)) * L.kstride + es * 32 + (lane >> 4) * 8;
    const uint4 kh = *(const uint4*)(Kt + koff);
    const uint4 kl = *(const uint4*)(Kt + L.kplane + koff);
#pragma unroll
    for (int qt = 0; qt < 8; ++qt)
      if (qt < n_qt) {
        const uint4 qa = *(const uint4*)(Qa + ((size_t)(qt * L.n_es + es) * 64 + lane) * 8);
        sacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_a(qa), as_bf16x8_a(kh),
                                                           sacc[qt], 0, 0, 0);
        sacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_a(qa), as_bf16x8_a(kl),
                                                           sacc[qt], 0, 0, 0);
      }
  }
  __syncthreads();  // Qa is about to be overwritten by S
  const float scale = 1.0f / sqrtf((float)hd);
#pragma unroll
  for (int qt = 0; qt < 8; ++qt)
    if (qt < n_qt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = sacc[qt][r] + __shfl_down(sacc[qt][r], 32);  // hi + lo rows
        const int qi = qt * 8 + 4 * ((lane >> 4) & 1) + r;
        const int key = wave * 16 + (lane & 15);
        if (lane < 32 && qi < QG) {
          const int t = t0 + key;
          const bool vis = t < n_keys && t <= pos0 + qi / G;
          S[qi * kAttnChunk + key] = vis ? v * scale : -INFINITY;
        }
      }
    }
  __syncthreads();

  // ---- softmax pieces per query (lane = key), probabilities as A fragments --
  float* my_ws = a.ws + ((size_t)h * a.max_chunks + c) * a.qg_max * (hd + 2);
  for (int qi = wave; qi < n_qt * 8; qi += 4) {
    float p = 0.0f;
    if (qi < QG) {
      const float sc = S[qi * kAttnChunk + lane];
      const float mx = wave_max_f32(sc);
      p = (sc != -INFINITY) ? expf(sc - mx) : 0.0f;
      const float l = wave_sum_f32(p);
      if (lane == 0) {
        my_ws[(size_t)qi * (hd + 2) + 0] = mx;
        my_ws[(size_t)qi * (hd + 2) + 1] = l;
      }
    }
    const uint16_t ph = f32_to_bf16_rne(p);
    const uint16_t pl = f32_to_bf16_rne(p - bf16_to_f32(ph));
    const int qt = qi / 8, m = qi % 8, ks = lane >> 5, kk = lane & 31;
    uint16_t* frag = Pa + (size_t)(qt * 2 + ks) * 512;
    frag[afrag_index(m, kk)] = ph;
    frag[afrag_index(m + 8, kk)] = pl;
  }
  __syncthreads();

  // ---- unnormalised value sums O = P V: wave w owns e-tiles w, w+4, ... ----
  for (int et = wave; et < L.n_et; et += 4) {
    // B fragments: lane l -> e = 16et + l%16, keys 32ks + 8(l/16) .. +7
    const uint16_t* vrow = Vt + (et * 16 + (lane & 15)) * L.vstride + (lane >> 4) * 8;
    const uint4 vh0 = *(const uint4*)(vrow);
    const uint4 vh1 = *(const uint4*)(vrow + 32);
    const uint4 vl0 = *(const uint4*)(vrow + L.vplane);
    const uint4 vl1 = *(const uint4*)(vrow + L.vplane + 32);
    for (int qt = 0; qt < n_qt; ++qt) {
      floatx4 o = floatx4{0.f, 0.f, 0.f, 0.f};
      const uint4 pa0 = *(const uint4*)(Pa + ((size_t)(qt * 2 + 0) * 64 + lane) * 8);
      const uint4 pa1 = *(const uint4*)(Pa + ((size_t)(qt * 2 + 1) * 64 + lane) * 8);
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_a(pa0), as_bf16x8_a(vh0), o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_a(pa1), as_bf16x8_a(vh1), o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_a(pa0), as_bf16x8_a(vl0), o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_a(pa1), as_bf16x8_a(vl1), o, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = o[r] + __shfl_down(o[r], 32);
        const int qi = qt * 8 + 4 * ((lane >> 4) & 1) + r;
        const int e = et * 16 + (lane & 15);
        if (lane < 32 && qi < QG && e < hd) my_ws[(size_t)qi * (hd + 2) + 2 + e] = v;
      }
    }
  }
}

// Merge the chunks of kv head h in chunk order.  Thread = (query, 8 dims);
// the chunk loop is unrolled so its loads are in flight together.
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
#pragma unroll 8
  for (int cc = 0; cc < n_active; ++cc) M = fmaxf(M, base[cc * cstride]);
  float L = 0.0f, O[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int cc = 0; cc < n_active; ++cc) {
    const float* pc = base + cc * cstride;
    const float m = pc[0];
    const float w = m == -INFINITY ? 0.0f : expf(m - M);
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

hipError_t attn_reserve_lds(size_t bytes) {
  return hipFuncSetAttribute((const void*)attn_partial_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
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
