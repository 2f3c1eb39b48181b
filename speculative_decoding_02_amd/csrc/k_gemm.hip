// k_gemm.hip -- weight-streaming skinny GEMM for the verify pass on gfx950.
//
// Y[m][n] = sum_k A[m][k] * W[n][k] for up to 8 activation rows m (the K+1
// verify positions, or 1-2 draft rows) against a bf16 weight matrix W that is
// read from HBM exactly once.  A pass over K+1 positions costs about one
// weight read, the premise of the method ([en] Floor 3; [int] "why it is
// faster"): the work is bandwidth-bound, so the kernel is built around
// streaming W.
//
//  * W is repacked once (launch_pack) so that each 16-byte lane load of a
//    wave is one B fragment of v_mfma_f32_16x16x32_bf16 and a wave's k-range
//    is one contiguous span: [group][k-block][NB][64 lanes][8 bf16].
//  * The A tile is 16 rows: rows 0-7 hold the bf16 high part of the fp32
//    activations, rows 8-15 the bf16 low part (x - hi), so one MFMA gives
//    ~16-bit-mantissa activations at no extra weight traffic.  It is staged in
//    LDS once per workgroup, with the RMSNorm of the consumer applied on the
//    fly from per-64-column sums of squares published by the producer.
//  * A workgroup = 4 waves; each wave owns NB 16-column blocks and the whole
//    k-range of its workgroup.  Column groups are split along K over `splits`
//    workgroups; partials go to a workspace and the last workgroup to arrive
//    sums them in split order (deterministic) and runs the epilogue.
#include "kernels.h"

namespace spec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

SPEC_DEVICE bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

SPEC_DEVICE uint4 load_stream(const uint4* p) {
  // weights are read once per pass: non-temporal hint
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

SPEC_DEVICE float4 load_nt_f4(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)p);
  return make_float4(v.x, v.y, v.z, v.w);
}

SPEC_DEVICE uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// Per-thread split of 8 fp32 values into bf16 (high or low part).
SPEC_DEVICE uint4 split8(const float* v, int part) {
  uint16_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t hi = f32_to_bf16_rne(v[e]);
    h[e] = part ? f32_to_bf16_rne(v[e] - bf16_to_f32(hi)) : hi;
  }
  return make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
}

constexpr int kUnroll = 8;

template <int NB, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny(GemmArgs a) {
  extern __shared__ uint4 lds_a[];  // [kcb][64]
  __shared__ float s_scale[kMaxRows];
  __shared__ float s_red[4][kMaxRows];
  __shared__ float s_red2[4][kMaxRows];
  __shared__ int32_t s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x % a.splits;
  const int wgg = blockIdx.x / a.splits;
  const int kb0 = split * a.kcb;
  const int kb1 = min(a.Kb, kb0 + a.kcb);
  const int nkb = kb1 - kb0;

  int n_rows = a.rows->n_rows;
  int row_base = 0;
  if (a.last_row_only) {
    row_base = n_rows - 1;
    n_rows = n_rows > 0 ? 1 : 0;
  }

  // ---- prologue: RMSNorm scale per row (fixed summation order) ----------
  if (tid < kMaxRows) {
    float sc = 1.0f;
    if (a.ssq != nullptr && tid < n_rows) {
      float ss = 0.0f;
      for (int g = 0; g < a.ssq_groups; ++g) ss += a.ssq[g * kMaxRows + row_base + tid];
      sc = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    }
    s_scale[tid] = sc;
  }
  __syncthreads();

  // ---- stage the A tile (hi rows 0-7, lo rows 8-15) ----------------------
  for (int idx = tid; idx < nkb * 64; idx += 256) {
    const int kbl = idx >> 6, l = idx & 63;
    const int row = l & 15, m = row & 7, part = row >> 3;
    uint4 packed = make_uint4(0, 0, 0, 0);
    if (m < n_rows) {
      const int k = (kb0 + kbl) * 32 + (l >> 4) * 8;
      const float* xr = a.X + (size_t)(row_base + m) * a.ldx + k;
      const float4 v0 = *(const float4*)xr;
      const float4 v1 = *(const float4*)(xr + 4);
      float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      if (a.ssq != nullptr) {
        const float sc = s_scale[m];
        const uint4 gv = *(const uint4*)(a.gain + k);
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = bf16_to_f32((uint16_t)(gw[e >> 1] >> ((e & 1) * 16)));
          v[e] = v[e] * sc * g;
        }
      }
      packed = split8(v, part);
    }
    lds_a[idx] = packed;
  }
  __syncthreads();

  // ---- main loop: stream W, MFMA against the staged A tile ----------------
  const int g = wgg * 4 + wave;
  floatx4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (g < a.n_groups) {
    const uint4* wp = (const uint4*)a.Wp + ((size_t)g * a.Kb + kb0) * NB * 64 + lane;
    int kb = 0;
    for (; kb + kUnroll <= nkb; kb += kUnroll) {
      uint4 b[kUnroll][NB];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < NB; ++j) b[u][j] = load_stream(wp + ((size_t)(kb + u) * NB + j) * 64);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const bf16x8_t av = as_bf16x8(lds_a[(kb + u) * 64 + lane]);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(b[u][j]), acc[j], 0, 0, 0);
      }
    }
    for (; kb < nkb; ++kb) {
      uint4 b[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) b[j] = load_stream(wp + ((size_t)kb * NB + j) * 64);
      const bf16x8_t av = as_bf16x8(lds_a[kb * 64 + lane]);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(b[j]), acc[j], 0, 0, 0);
    }
  }

  // ---- combine hi and lo rows: lane l < 32 gets rows 4*(l/16)+r ----------
  float y[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) y[j][r] = acc[j][r] + __shfl_down(acc[j][r], 32);

  // ---- split-K: publish partials, last workgroup reduces in split order ---
  if (a.splits > 1) {
    float* my = a.ws + ((size_t)(wgg * a.splits + split) * 4 + wave) * NB * 128;
    if (lane < 32) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        *(float4*)(my + j * 128 + lane * 4) = make_float4(y[j][0], y[j][1], y[j][2], y[j][3]);
    }
    __threadfence();
    if (!arrive_last(a.counters + wgg, a.splits, &s_flag)) return;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[j][r] = 0.0f;
    if (lane < 32) {
      for (int s = 0; s < a.splits; ++s) {
        const float* p = a.ws + ((size_t)(wgg * a.splits + s) * 4 + wave) * NB * 128;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const float4 v = load_nt_f4(p + j * 128 + lane * 4);
          y[j][0] += v.x; y[j][1] += v.y; y[j][2] += v.z; y[j][3] += v.w;
        }
      }
    }
  }

  // ---- epilogues ----------------------------------------------------------
  const int nl = lane & 15;           // column within the 16-block
  const int mrow0 = 4 * ((lane >> 4) & 1);  // first of the lane's 4 rows (lanes < 32)
  const bool lane_ok = lane < 32 && g < a.n_groups;

  if constexpr (EPI == EPI_STORE) {
    if (lane_ok) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mrow0 + r;
          if (m < n_rows) a.out[(size_t)m * a.ldo + (size_t)(g * NB + j) * 16 + nl] = y[j][r];
        }
    }
  } else if constexpr (EPI == EPI_SILU) {
    static_assert(NB == 2, "gate/up epilogue pairs two blocks");
    if (lane_ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mrow0 + r;
        if (m < n_rows) {
          const float gt = y[0][r], up = y[1][r];
          a.out[(size_t)m * a.ldo + (size_t)g * 16 + nl] = gt / (1.0f + expf(-gt)) * up;
        }
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    static_assert(NB == 1, "residual epilogue publishes 64-column norm partials");
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
    if (lane_ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mrow0 + r;
        if (m < n_rows) {
          float* px = a.resid + (size_t)m * a.ldr + (size_t)g * 16 + nl;
          const float nx = *px + y[0][r];
          *px = nx;
          sq[r] = nx * nx;
        }
      }
    }
    // sum over the 16 columns of the block (lanes sharing lane>>4), fixed tree
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int msk = 8; msk >= 1; msk >>= 1) sq[r] += __shfl_xor(sq[r], msk);
    }
    if (lane == 0 || lane == 16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s_red[wave][mrow0 + r] = sq[r];
    }
    __syncthreads();
    if (tid < kMaxRows)
      a.ssq_out[wgg * kMaxRows + tid] = ((s_red[0][tid] + s_red[1][tid]) + s_red[2][tid]) + s_red[3][tid];
  } else if constexpr (EPI == EPI_LOGITS) {
    float mx[4], sm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mrow0 + r;
      const int col = g * 16 + nl;
      const bool ok = lane_ok && m < n_rows && col < a.n_valid;
      if (ok) a.out[(size_t)m * a.ldo + col] = y[0][r];
      mx[r] = ok ? y[0][r] : -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int msk = 8; msk >= 1; msk >>= 1) mx[r] = fmaxf(mx[r], __shfl_xor(mx[r], msk));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mrow0 + r;
      const int col = g * 16 + nl;
      const bool ok = lane_ok && m < n_rows && col < a.n_valid;
      sm[r] = ok ? expf(y[0][r] - mx[r]) : 0.0f;
#pragma unroll
      for (int msk = 8; msk >= 1; msk >>= 1) sm[r] += __shfl_xor(sm[r], msk);
    }
    if (lane == 0 || lane == 16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s_red[wave][mrow0 + r] = mx[r];
        s_red2[wave][mrow0 + r] = sm[r];
      }
    }
    __syncthreads();
    if (tid < kMaxRows) {
      float M = s_red[0][tid];
      for (int w = 1; w < 4; ++w) M = fmaxf(M, s_red[w][tid]);
      float S = 0.0f;
      if (M != -INFINITY) {
        for (int w = 0; w < 4; ++w)
          if (s_red[w][tid] != -INFINITY) S += s_red2[w][tid] * expf(s_red[w][tid] - M);
      }
      a.lm_part[wgg * kMaxRows + tid] = make_float2(M, S);
    }
  } else if constexpr (EPI == EPI_QKV) {
    static_assert(NB == 1, "qkv epilogue works on single blocks");
    if (g < a.n_groups) {
      const int q_blocks = a.q_dim / 16, k_blocks = a.kv_dim / 16;
      const int half_hd = a.head_dim / 2;
      const int pos0 = a.rows->pos0;
      if (g < q_blocks + k_blocks) {
        // pair-interleaved block: columns w and w^8 are the two halves of one pair
        const bool is_q = g < q_blocks;
        const int bl = is_q ? g : g - q_blocks;
        const int pair = bl * 8 + (nl & 7), half = nl >> 3;
        const int head = pair / half_hd, jj = pair % half_hd;
        const double f = a.inv_freq[jj];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float mine = y[0][r];
          const float other = __shfl_xor(mine, 8);
          const int m = mrow0 + r;
          const int pos = pos0 + m;
          if (lane < 32 && m < n_rows && pos < a.max_seq) {
            double sn, cs;
            sincos((double)pos * f, &sn, &cs);
            const double lo = half ? (double)other : (double)mine;
            const double hi = half ? (double)mine : (double)other;
            const float val = (float)(half ? hi * cs + lo * sn : lo * cs - hi * sn);
            const int dim = jj + half * half_hd;
            if (is_q) {
              a.out[(size_t)m * a.ldo + (size_t)head * a.head_dim + dim] = val;
            } else {
              const int blk = a.block_table[pos / kBlock];
              a.k_cache[(((size_t)blk * a.n_kv + head) * kBlock + pos % kBlock) * a.head_dim + dim] =
                  f32_to_bf16_rne(val);
            }
          }
        }
      } else {
        const int f0 = (g - q_blocks - k_blocks) * 16 + nl;
        const int head = f0 / a.head_dim, dim = f0 % a.head_dim;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mrow0 + r;
          const int pos = pos0 + m;
          if (lane < 32 && m < n_rows && pos < a.max_seq) {
            const int blk = a.block_table[pos / kBlock];
            a.v_cache[(((size_t)blk * a.n_kv + head) * kBlock + pos % kBlock) * a.head_dim + dim] =
                f32_to_bf16_rne(y[0][r]);
          }
        }
      }
    }
  }
}

template <int NB, int EPI>
static hipError_t launch_one(const GemmArgs& a, hipStream_t s) {
  const int n_wgg = (a.n_groups + 3) / 4;
  hipLaunchKernelGGL((gemm_skinny<NB, EPI>), dim3(n_wgg * a.splits), dim3(256),
                     gemm_lds_bytes(a.kcb), s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int nb, int epi, const GemmArgs& a, hipStream_t s) {
  if (nb == 1) {
    switch (epi) {
      case EPI_STORE: return launch_one<1, EPI_STORE>(a, s);
      case EPI_RESID: return launch_one<1, EPI_RESID>(a, s);
      case EPI_QKV: return launch_one<1, EPI_QKV>(a, s);
      case EPI_LOGITS: return launch_one<1, EPI_LOGITS>(a, s);
      default: break;
    }
  } else if (nb == 2) {
    switch (epi) {
      case EPI_STORE: return launch_one<2, EPI_STORE>(a, s);
      case EPI_SILU: return launch_one<2, EPI_SILU>(a, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ pack --
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* const* row_ptr, int K, int nb,
                                                   int n_groups, uint16_t* out) {
  const int Kb = K / 32;
  const size_t total = (size_t)n_groups * Kb * nb * 64;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx % 64);
    const int j = (int)((idx / 64) % nb);
    const int kb = (int)((idx / (64 * (size_t)nb)) % Kb);
    const size_t g = idx / (64 * (size_t)nb * Kb);
    const size_t n = (g * nb + j) * 16 + (lane & 15);
    const int k = kb * 32 + (lane >> 4) * 8;
    const uint16_t* src = row_ptr[n];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src != nullptr) v = *(const uint4*)(src + k);
    ((uint4*)out)[idx] = v;
  }
}

hipError_t launch_pack(const uint16_t* const* row_ptr, int K, int nb, int n_groups, uint16_t* out,
                       hipStream_t s) {
  const size_t total = (size_t)n_groups * (K / 32) * nb * 64;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, row_ptr, K, nb, n_groups,
                     out);
  return hipGetLastError();
}

}  // namespace spec
