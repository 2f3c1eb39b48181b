// common.h -- device helpers and launch-argument structs shared by the HIP
// kernels of libspec (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SPEC_DEVICE __device__ __forceinline__

namespace spec {

constexpr int kWave = 64;
constexpr int kMaxRows = 8;       // activation rows per pass (K+1 <= 8)
constexpr int kBlock = 16;        // KV-cache block size in tokens

// ---------------------------------------------------------------- errors --
// Sticky device-side error bits (DevState::err).
enum : int32_t {
  kErrBadToken = 1,       // a token id outside [0, vocab) reached the embedding
  kErrLag = 2,            // draft cache lag larger than kMaxRows - 1
  kErrCapacity = 4,       // a position at or beyond max_seq
};

// Device-resident decoding state (one per context).
constexpr int kAcceptBins = kMaxRows;  // K = 0..7, n_acc = 0..7
struct DevState {
  int32_t LT;        // tokens in the target cache; hist[LT] is the pending token
  int32_t LD;        // tokens in the draft cache
  int32_t err;       // sticky error bits
  int32_t pad;
  // committed verifies by (K, n_acc): the acceptance record of the context
  int32_t accept_counts[kAcceptBins][kAcceptBins];
};

// Row descriptor of one forward pass, written by the embedding kernel and
// read by every later kernel of the pass.
struct PassRows {
  int32_t n_rows;    // 1..kMaxRows
  int32_t pos0;      // absolute position of row 0 (row r is at pos0 + r)
  int32_t tok[kMaxRows];
};

// ------------------------------------------------------------------ bf16 --
SPEC_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// floor(x / d) for 0 <= x < 2^21 and d >= 1, given inv = 1/d to within a
// relative 2^-23 (v_rcp_f32 is within one ulp): (x + 1/2)/d lies at least
// 1/(2d) from an integer, and inv's error plus the product's rounding move it
// by less than (x/d) * 2^-22 < 1/(2d), so the truncation is exact.  A few
// instructions instead of a software integer division.
SPEC_DEVICE float rcp_small(int d) { return __builtin_amdgcn_rcpf((float)d); }
SPEC_DEVICE int div_small(int x, float inv) { return (int)(((float)x + 0.5f) * inv); }

// fp32 -> bf16 with round-to-nearest-even (NaN stays a quiet NaN): the
// language conversion, which gfx950 carries out in one v_cvt_pk_bf16_f32.
SPEC_DEVICE uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two values at once, packed low half first (one instruction).
typedef float spec_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 spec_bf16x2 __attribute__((ext_vector_type(2)));
SPEC_DEVICE uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  const spec_bf16x2 v = __builtin_convertvector((spec_f32x2){lo, hi}, spec_bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------- KV cache --
// Paged caches of one layer, in blocks of 16 tokens.  Every key and value is
// kept as two bf16 planes: [0] the bf16 high part of the fp32 value, [1] the
// low part (x - hi).  Keeping ~16 mantissa bits matters: rounding keys and
// values to one bf16 is the largest error source of the pass (it compounds
// through the feed-forward blocks to ~1e-2 logit error on an 8B-shaped
// slice).
//   keys:   [block][kv head][16 tokens][2][head_dim]  -- a token's 8
//           consecutive dims are one 16-byte MFMA fragment row
//   values: [block][kv head][2][head_dim][16 tokens]  -- transposed, so 4
//           consecutive tokens of one dim are one 8-byte load
SPEC_DEVICE size_t kv_index(int blk, int n_kv, int head, int slot, int hd, int part, int dim) {
  return ((((size_t)blk * n_kv + head) * kBlock + slot) * 2 + part) * hd + dim;
}
SPEC_DEVICE size_t vt_index(int blk, int n_kv, int head, int part, int hd, int dim, int slot) {
  return ((((size_t)blk * n_kv + head) * 2 + part) * hd + dim) * kBlock + slot;
}

// Query fragments of the attention, written by the QKV epilogue:
// [n_kv][ceil(G/2)][n_es][2 parts][64 lanes][8 bf16] with G = n_q / n_kv and
// n_es = ceil(hd/32).  Query vector qi = row * G + g of kv head h (query head
// h*G + g) is column qi % 16 of tile qi / 16; part 0 holds its bf16 high
// parts, part 1 the low parts; lane l of e-step es holds dims
// 32 es + 8 (l / 16) .. + 7 of column l % 16 (the B operand layout of
// v_mfma_f32_16x16x32_bf16).
SPEC_DEVICE size_t qfrag_index(int h, int G, int n_es, int qi, int part, int dim) {
  const int lane = (qi & 15) + 16 * ((dim & 31) >> 3);
  const int n_qt = (G + 1) / 2;
  return (((((size_t)h * n_qt + (qi >> 4)) * n_es + (dim >> 5)) * 2 + part) * 64 + lane) * 8 +
         (dim & 7);
}

// ------------------------------------------------- packed MFMA A operand --
// Activations enter the skinny GEMM as the A operand of
// v_mfma_f32_16x16x32_bf16: 16 rows x 32 k per 1 KiB block, lane l taking 8
// bf16 of row l%16 at k = 32*kb + 8*(l/16) + 0..7.  Rows 0-7 carry the bf16
// high part of the fp32 activation rows 0-7, rows 8-15 the bf16 low part
// (x - hi), so products against bf16 weights keep ~16 mantissa bits.
// Within a block each row's 32 values are contiguous ([Kb][16 rows][32]
// bf16 per matrix): a pass over n rows touches 2n 64-byte runs per block
// (the four lanes of a row read one run), not every line of it.  Producers
// write this layout directly.
SPEC_DEVICE size_t apack_index(int m, int part, int k) {
  return ((size_t)(k >> 5) * 16 + (m + 8 * part)) * 32 + (k & 31);
}
// Byte offset of lane l's A fragment within a k-block of that layout.
SPEC_DEVICE uint32_t apack_lane_offset(int lane) {
  return (uint32_t)((lane & 15) * 64 + (lane >> 4) * 16);
}

SPEC_DEVICE uint32_t pack_bf16x2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Stores 8 consecutive activations of row m starting at k0 (k0 % 8 == 0) as
// their high and low bf16 parts: two 16-byte stores.
SPEC_DEVICE void apack_store8(uint16_t* Ap, int m, int k0, const float* v) {
  uint16_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f32_to_bf16_rne(v[e]);
    l[e] = f32_to_bf16_rne(v[e] - bf16_to_f32(h[e]));
  }
  *(uint4*)(Ap + apack_index(m, 0, k0)) =
      make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                 pack_bf16x2(h[6], h[7]));
  *(uint4*)(Ap + apack_index(m, 1, k0)) =
      make_uint4(pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3]), pack_bf16x2(l[4], l[5]),
                 pack_bf16x2(l[6], l[7]));
}

// Stores one activation of row m at column k as its high and low bf16 parts.
SPEC_DEVICE void apack_store1(uint16_t* Ap, int m, int k, float v) {
  const uint16_t h = f32_to_bf16_rne(v);
  Ap[apack_index(m, 0, k)] = h;
  Ap[apack_index(m, 1, k)] = f32_to_bf16_rne(v - bf16_to_f32(h));
}

// 8 bf16 gains starting at k0 -> fp32
SPEC_DEVICE void load_gain8(const uint16_t* g, int k0, float* out) {
  const uint4 v = *(const uint4*)(g + k0);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = bf16_to_f32((uint16_t)(w[e >> 1] >> ((e & 1) * 16)));
}

// ---------------------------------------------------------------- Philox --
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 64x64->128-bit multiplies, key bumped by two Weyl constants between rounds.
// The decode loop evaluates it at counter (position, sequence, stream, 0)
// with key (seed, 0) and uses word 0 for a draft sample, word 1 for the
// accept test and word 2 for the target's sample, each as its top 24 bits.
// Pick a word with constant indices or a select: a runtime index into w[]
// sends the array to per-thread LDS addressed through the dispatch packet.
struct U64x4 {
  uint64_t w[4];
};

SPEC_DEVICE U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  U64x4 o;
  o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
  return o;
}


// -------------------------------------------------------- probabilities --
SPEC_DEVICE bool prob_valid(float x) { return x >= 0.0f && x <= 1.0f; }  // false for NaN

// floor(x * 2^40) for a valid probability (exact: power-of-two scaling of an
// fp32 value, then truncation of a non-negative double).
SPEC_DEVICE uint64_t fix40(float x) { return (uint64_t)((double)x * 1099511627776.0); }

// Needle of the inverse CDF: floor(u24 * Z / 2^24) without 128-bit products.
SPEC_DEVICE uint64_t icdf_needle(uint32_t u24, uint64_t Z) {
  return (uint64_t)u24 * (Z >> 24) + (((uint64_t)u24 * (Z & 0xFFFFFFull)) >> 24);
}

// Key whose unsigned maximum is the largest fp32 value, ties to the lowest
// index.  Inputs are validated probabilities (>= 0); -0.0 is folded to +0.
SPEC_DEVICE uint64_t argmax_key(float x, uint32_t idx) {
  const uint32_t b = __float_as_uint(x == 0.0f ? 0.0f : x);
  return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
SPEC_DEVICE uint32_t argmax_key_index(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }

// ------------------------------------------------------ wave reductions --
SPEC_DEVICE uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
SPEC_DEVICE uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_u64(v, m);
  return v;
}
SPEC_DEVICE uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}
SPEC_DEVICE float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
SPEC_DEVICE float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Exclusive prefix sum of one uint64 per thread over a 256-thread block
// (integer addition: exact and order-free).  lds: >= 4 entries.
SPEC_DEVICE uint64_t block_exclusive_scan_u64_256(uint64_t v, uint64_t* lds) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)inc, d), hi = __shfl_up((uint32_t)(inc >> 32), d);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    if (lane >= d) inc += o;
  }
  if (lane == 63) lds[wid] = inc;
  __syncthreads();
  uint64_t base = 0;
  for (int w = 0; w < wid; ++w) base += lds[w];
  __syncthreads();
  return base + inc - v;
}

// Block-wide reductions through LDS (blockDim.x a multiple of 64, <= 1024).
// Fixed combination order: deterministic.
template <typename T, typename Op>
SPEC_DEVICE T block_reduce(T v, T* lds /* >= 16 */, Op op) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = op(v, __shfl_xor(v, m));
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  T r = lds[0];
  for (int i = 1; i < nw; ++i) r = op(r, lds[i]);
  __syncthreads();
  return r;
}

}  // namespace spec
