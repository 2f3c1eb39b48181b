// k_attn.hip -- causal attention of the pass's query rows against the paged
// KV cache.
//
// Row r (position pos0 + r) attends to keys 0..pos0+r: row i of the verify
// pass sees the context plus drafts d_1..d_{i-1}, which is what makes its
// output the target distribution T_i = T(. | x, d_1..d_{i-1}) ([int]
// algorithm core, Step 2).  Grouped-query heads: query head h*G + g reads KV
// head h; all G query heads of a group and all rows share one read of each
// key and value.
//
// Two launches, no inter-block waiting:
//  (1) partial kernel, one wave per (32-key chunk, kv head, 16-query tile):
//      the tiles of one chunk run as separate waves (on the same XCD, so the
//      second reads the chunk's keys and values from L2).  Everything
//      lives in registers: the wave issues all its loads at once (key
//      fragments, value fragments, query fragments), then
//        S^T = K Q^T  and  O^T = V^T P^T   on v_mfma_f32_16x16x32_bf16
//      over tiles of 16 query vectors.  Keys and values enter as the cache's
//      bf16 high/low planes, queries and probabilities as bf16 high/low
//      operands; the products hi*hi + hi*lo + lo*hi accumulate in one
//      register tile, so every product keeps ~16 mantissa bits (the lo*lo
//      term, ~2^-16 relative to the others, is left out).  The C layout of
//      S^T already gives each lane the 8 keys that form its slots of the P^T
//      operand, so lanes exchange data only for the max and the sum over
//      keys.  Per query it writes (max score, sum of exp, unnormalised value
//      sum) for the chunk.
//  (2) merge kernel, one workgroup per (query vector, kv head): all chunk
//      partials are loaded at once and combined with running-max rescaling,
//      per thread and then across threads in a fixed order (deterministic);
//      it writes the packed A operand of the O projection.
// A batch of sequences runs in the same two launches: the sequence index
// extends grid.z of the partial kernel and grid.y of the merge, and selects
// the sequence's pass descriptor, block table, query fragments and workspace.
#include <type_traits>

#include "kernels.h"

namespace spec {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

SPEC_DEVICE floatx4 mfma16(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Raw buffer resources (gfx9 descriptor word 3): loads at offsets >= size
// return zero.
constexpr uint32_t kOOB = 0x80000000u;
SPEC_DEVICE __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
SPEC_DEVICE uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
SPEC_DEVICE uint2 load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v.x, v.y);
}

// Cross-lane folds with gfx950's lane-swap instructions instead of the LDS
// permute unit: swapping a value with itself through v_permlane16_swap
// (odd and even 16-lane rows) or v_permlane32_swap (the wave's halves) gives
// every lane both its own value and that of lane l^16 (l^32).  Each lane
// computes op(x, y) on the same pair the xor shuffle would give it (op
// commutative), so results are unchanged.
template <class Op>
SPEC_DEVICE float fold_xor16(float v, Op op) {
  const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                                  __builtin_bit_cast(uint32_t, v), false, false);
  const uint32_t x = p[0], y = p[1];  // bit_cast straight off a vector element reads element 0
  return op(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}
template <class Op>
SPEC_DEVICE float fold_xor32(float v, Op op) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                                  __builtin_bit_cast(uint32_t, v), false, false);
  const uint32_t x = p[0], y = p[1];  // bit_cast straight off a vector element reads element 0
  return op(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}
struct OpMax {
  SPEC_DEVICE float operator()(float x, float y) const { return fmaxf(x, y); }
};
struct OpAdd {
  SPEC_DEVICE float operator()(float x, float y) const { return x + y; }
};

// Fragment layouts (lane l, l16 = l % 16, grp = l / 16):
//   A (16 x 32):  lane l holds row l16, k = 8 grp .. 8 grp + 7
//   B (32 x 16):  lane l holds column l16, k = 8 grp .. 8 grp + 7
//   C (16 x 16):  lane l holds rows 4 grp + r (r = 0..3) of column l16
// S^T tile (kt, qt): rows = keys 16 kt + 0..15 of the chunk, columns = query
// vectors 16 qt + 0..15.  The P^T operand's k slot 8 grp + j of lane l is
// key 16 (j / 4) + 4 grp + (j % 4) -- exactly the keys lane l holds in the C
// layouts of tiles kt = 0, 1; the V^T operand uses the same slot order (two
// 4-key runs of the transposed value cache).
// QTW query tiles per wave: with QTW = 2 one wave scores both tiles of a
// chunk from one load of its keys and values (the batched pass); with 1 the
// tiles run as separate waves.
// The pointers and sizes the first loads need lead the arguments as scalars
// (preloaded in SGPRs rather than loaded from the argument segment).
template <int NES, int QTW>
__global__ __launch_bounds__(64) void attn_partial_kernel(const PassRows* rows_all,
                                                          const int32_t* block_table,
                                                          const uint16_t* qf_all,
                                                          const uint16_t* k_cache,
                                                          const uint16_t* v_cache, uint32_t qf_bytes,
                                                          uint32_t kv_layer_bytes, AttnArgs a) {
  constexpr int NET = 2 * NES;            // e-tiles of 16 covering 32*NES dims
  const int lane = threadIdx.x, l16 = lane & 15, grp = lane >> 4;
  const int hd = a.hd, G = a.n_q / a.n_kv, n_kv = a.n_kv;
  const int n_qt_max = (G + 1) / 2;
  const int n_qw = (n_qt_max + QTW - 1) / QTW;  // waves per (chunk, kv head, sequence)
  // grid.x interleaves (chunk, kv head) with the head fastest: workgroup ids
  // congruent mod 8 share an XCD, so every chunk of a head runs on the XCD(s)
  // the head maps to, where the merge of that head reads their partials
  const int c = blockIdx.x / n_kv, h = blockIdx.x % n_kv, qw = blockIdx.z % n_qw;
  const int seq = blockIdx.z / n_qw;
  const int n_et = (hd + 15) / 16, E16 = n_et * 16, n_es = (hd + 31) / 32;
  const int key0 = c * kAttnChunk;
  const int32_t* table = block_table + (size_t)seq * a.n_blocks;
  const PassRows* rows = rows_all + seq;

  // Buffer loads: an offset at or past the resource's size reads as zero,
  // which masks padded dims and absent tiles without branches, so every load
  // of the wave is in flight at once.
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_cache, kv_layer_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_cache, kv_layer_bytes);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qf_all + (size_t)seq * (qf_bytes / 2), qf_bytes);
  // Query fragments of this wave's tile.  Columns beyond this pass's query
  // vectors hold finite values from earlier passes; their scores are masked
  // below.  Issued before the pass descriptor is read, with the chunk's two
  // cache blocks (the second clamped to the table).
  uint4 qf[QTW][NES][2];
#pragma unroll
  for (int q = 0; q < QTW; ++q) {
    const int qt = qw * QTW + q;
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      const bool ok = qt < n_qt_max && 32 * es + 8 * grp < hd;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t off =
            (uint32_t)((((((size_t)h * n_qt_max + qt) * n_es + es) * 2 + p) * 64 + lane) * 16);
        qf[q][es][p] = load16(rq, ok ? off : kOOB);
      }
    }
  }
  const int blk0 = table[2 * c];
  const int blk1_any = table[min(2 * c + 1, a.n_blocks - 1)];

  const int n_rows = rows->n_rows, pos0 = rows->pos0;
  const int n_keys = pos0 + n_rows;
  if (n_rows <= 0 || key0 >= n_keys) return;
  const int QG = G * n_rows, n_qt = (QG + 15) / 16;
  if (qw * QTW >= n_qt) return;
  const int blk1 = key0 + kBlock < n_keys ? blk1_any : blk0;
  const float scale = 1.0f / sqrtf((float)hd);
  const size_t hs = (size_t)seq * n_kv + h;  // (sequence, kv head) slice of the workspace
  float* wso = a.ws_o + (hs * a.max_chunks + c) * a.qg_max * E16;
  float2* wsml = a.ws_ml + (hs * a.max_chunks + c) * a.qg_max;

  uint4 kf[2][NES][2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = key0 + 16 * kt + l16;
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      const int e0 = 32 * es + 8 * grp;
      const bool ok = key < n_keys && e0 < hd;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t off = (uint32_t)(kv_index(kt ? blk1 : blk0, n_kv, h, l16, hd, p, e0) * 2);
        kf[kt][es][p] = load16(rk, ok ? off : kOOB);
      }
    }
  }
  uint4 vf[NET][2];
#pragma unroll
  for (int et = 0; et < NET; ++et) {
    const int e = 16 * et + l16;
    const bool ok = e < hd;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t o0 = (uint32_t)(vt_index(blk0, n_kv, h, p, hd, e, 4 * grp) * 2);
      const uint32_t o1 = (uint32_t)(vt_index(blk1, n_kv, h, p, hd, e, 4 * grp) * 2);
      const uint2 w0 = load8(rv, ok ? o0 : kOOB), w1 = load8(rv, ok ? o1 : kOOB);
      vf[et][p] = make_uint4(w0.x, w0.y, w1.x, w1.y);
    }
  }
  // Every key and value load is issued before the first MFMA waits on one:
  // left alone, the scheduler interleaves them with the score MFMAs and the
  // wave pays several dependent memory round trips instead of one.
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int q = 0; q < QTW; ++q) {
  const int qt = qw * QTW + q;
  if (qt >= n_qt) break;  // wave-uniform
  // ---- scores S^T = K Q^T for the 32 keys -----------------------------
  floatx4 s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    s[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int es = 0; es < NES; ++es) {
      s[kt] = mfma16(kf[kt][es][0], qf[q][es][0], s[kt]);
      s[kt] = mfma16(kf[kt][es][0], qf[q][es][1], s[kt]);
      s[kt] = mfma16(kf[kt][es][1], qf[q][es][0], s[kt]);
    }
  }
  const int qi = 16 * qt + l16;
  const int limit = pos0 + qi / G;  // last key row qi's position sees
  float sc[2][4];
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 16 * kt + 4 * grp + r;
      const bool vis = qi < QG && key < n_keys && key <= limit;
      sc[kt][r] = vis ? s[kt][r] * scale : -INFINITY;
      mx = fmaxf(mx, sc[kt][r]);
    }
  mx = fold_xor16(mx, OpMax{});
  mx = fold_xor32(mx, OpMax{});
  float lsum = 0.0f;
  float pv[8];
  uint32_t ph[4], pl[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = sc[j >> 2][j & 3];
    pv[j] = x == -INFINITY ? 0.0f : expf(x - mx);
    lsum += pv[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // high and low bf16 parts, two values per conversion
    ph[j] = f32x2_to_bf16x2_rne(pv[2 * j], pv[2 * j + 1]);
    pl[j] = f32x2_to_bf16x2_rne(pv[2 * j] - __uint_as_float(ph[j] << 16),
                                pv[2 * j + 1] - __uint_as_float(ph[j] & 0xffff0000u));
  }
  lsum = fold_xor16(lsum, OpAdd{});
  lsum = fold_xor32(lsum, OpAdd{});
  const uint4 pfh = make_uint4(ph[0], ph[1], ph[2], ph[3]);
  const uint4 pfl = make_uint4(pl[0], pl[1], pl[2], pl[3]);
  // ---- unnormalised value sums O^T = V^T P^T --------------------------
  // Every e-tile is computed (tiles past the head dimension read zeros), so
  // the NET independent chains overlap; only the stores are guarded.
  floatx4 o[NET];
#pragma unroll
  for (int et = 0; et < NET; ++et) {
    o[et] = mfma16(vf[et][0], pfh, floatx4{0.f, 0.f, 0.f, 0.f});
    o[et] = mfma16(vf[et][0], pfl, o[et]);
    o[et] = mfma16(vf[et][1], pfh, o[et]);
  }
  if (qi < QG) {
#pragma unroll
    for (int et = 0; et < NET; ++et) {
      const float4 v = make_float4(o[et][0], o[et][1], o[et][2], o[et][3]);
      if (et < n_et) *(float4*)(wso + (size_t)qi * E16 + 16 * et + 4 * grp) = v;
    }
  }
  if (grp == 0 && qi < QG) wsml[qi] = make_float2(mx, lsum);
  }  // query tiles
}

// Merge of the chunk partials of query vector qi of kv head h, one wave per
// (head, query vector): lane (chunk group cg, 8-dim group d8) takes chunks
// cg, cg + ncg, ... (ncg = 64 / n8 groups of n8 = hd/8 lanes).  Each batch of
// a lane's chunks is folded in two passes -- its maximum, then the weights
// exp(m_c - max), the running sums rescaled once per batch -- and the chunk
// groups are then brought to the wave's maximum and summed in a fixed order
// (deterministic), all inside the wave: no LDS and no barrier.
constexpr int kMergeBatch = 10;  // chunks per lane in flight at once

// v + (the value of lane l ^ OFF), by the cheapest exchange for that offset
template <int OFF>
SPEC_DEVICE float add_xor(float v) {
  if constexpr (OFF == 32) return fold_xor32(v, OpAdd{});
  else if constexpr (OFF == 16) return fold_xor16(v, OpAdd{});
  else if constexpr (OFF == 8)
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                      0x128, 0xf, 0xf, true));
  else if constexpr (OFF == 2)
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                      0x4e, 0xf, 0xf, true));
  else if constexpr (OFF == 1)
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                      0xb1, 0xf, 0xf, true));
  else return v + __shfl_xor(v, OFF);
}
template <int OFF>
SPEC_DEVICE void butterfly_add(float* v) {  // over lanes OFF, 2*OFF, ... < 64 apart
  if constexpr (OFF < 64) {
#pragma unroll
    for (int e = 0; e < 9; ++e) v[e] = add_xor<OFF>(v[e]);
    butterfly_add<2 * OFF>(v);
  }
}
// maximum over the wave (max is exact, so any exchange order gives the same value)
SPEC_DEVICE float wave_max_dpp(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 decltype(ctrl)::value, 0xf, 0xf, true));
  };
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0xb1>{}));   // lane l^1
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4e>{}));   // lane l^2
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));  // the other quad of the 8-lane half
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x128>{}));  // the other half of the 16-lane row
  v = fold_xor16(v, OpMax{});
  return fold_xor32(v, OpMax{});
}

// N8 > 0: hd / 8, a power of two known at compile time; 0: any hd (multiple of 8)
template <int N8>
__global__ __launch_bounds__(64) void attn_merge_kernel(const PassRows* rows, const float2* ws_ml,
                                                       const float* ws_o, AttnArgs a) {
  // one-dimensional grid, kv head fastest (the XCD its partials were written on)
  const int n_seq = a.n_seq > 1 ? a.n_seq : 1;
  const int qg_launch = gridDim.x / (a.n_kv * n_seq);  // query vectors per head in this launch
  const int h = blockIdx.x % a.n_kv, qi = (blockIdx.x / a.n_kv) % qg_launch;
  const int seq = blockIdx.x / (a.n_kv * qg_launch);
  const size_t hs = (size_t)seq * a.n_kv + h;  // (sequence, kv head) slice of the workspace
  const int hd = a.hd, G = a.n_q / a.n_kv;
  const int E16 = (hd + 15) / 16 * 16;
  const int n8 = N8 > 0 ? N8 : hd / 8, ncg = 64 / n8;
  const int lane = threadIdx.x;
  const int cg = lane / n8, d8 = lane % n8;
  const size_t cs_ml = (size_t)a.qg_max, cs_o = (size_t)a.qg_max * E16;
  const float2* ml = ws_ml + hs * a.max_chunks * a.qg_max + qi;
  const float* wo = ws_o + (hs * a.max_chunks * a.qg_max + qi) * E16 + d8 * 8;
  const bool worker = cg < ncg;

  float4 v0[kMergeBatch], v1[kMergeBatch];
  float2 mv[kMergeBatch];
  auto load = [&](int c0) {  // chunk indices clamped to the workspace
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const size_t cl = (size_t)min(c0 + u * ncg, a.max_chunks - 1);
      mv[u] = ml[cl * cs_ml];
      v0[u] = *(const float4*)(wo + cl * cs_o);
      v1[u] = *(const float4*)(wo + cl * cs_o + 4);
    }
  };
  // the first batch is issued before the pass descriptor is read
  load(worker ? cg : 0);

  const int n_rows = rows[seq].n_rows, pos0 = rows[seq].pos0;
  const int QG = G * n_rows;
  if (n_rows <= 0 || qi >= QG) return;
  const int n_keys = pos0 + n_rows;
  const int n_active = (n_keys + kAttnChunk - 1) / kAttnChunk;

  float mx = -INFINITY, l = 0.0f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.0f;
  for (int c0 = worker ? cg : n_active; c0 < n_active; c0 += kMergeBatch * ncg) {
    if (c0 != cg) load(c0);
    __builtin_amdgcn_sched_barrier(0);  // all loads of the batch in flight before any use
    // slots past the active chunks were loaded from clamped indices: their
    // workspace contents may be anything (not even finite), so they are
    // replaced, not weighted by zero; a chunk with no visible key has m = -inf
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (c0 + u * ncg < n_active) bm = fmaxf(bm, mv[u].x);
    const float mn = fmaxf(mx, bm);
    const float sa = mx == -INFINITY ? 0.0f : expf(mx - mn);
    l *= sa;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= sa;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const bool ok = c0 + u * ncg < n_active;
      const float m = ok ? mv[u].x : -INFINITY;
      const float w = m == -INFINITY ? 0.0f : expf(m - mn);
      const float ov[8] = {ok ? v0[u].x : 0.f, ok ? v0[u].y : 0.f, ok ? v0[u].z : 0.f,
                           ok ? v0[u].w : 0.f, ok ? v1[u].x : 0.f, ok ? v1[u].y : 0.f,
                           ok ? v1[u].z : 0.f, ok ? v1[u].w : 0.f};
      l += w * (ok ? mv[u].y : 0.0f);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += w * ov[e];
    }
    mx = mn;
  }
  // the wave's maximum, then every chunk group's sums at that scale
  const float M = wave_max_dpp(mx);
  const float sc = mx == -INFINITY ? 0.0f : expf(mx - M);
  float v[9];
  v[0] = l * sc;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[1 + e] = o[e] * sc;
  // sum over the chunk groups (lanes n8 apart): a butterfly when n8 is a
  // power of two, else lane d8 adds the groups one after another
  if constexpr (N8 > 0) {
    butterfly_add<N8>(v);
  } else {
    float acc[9];
#pragma unroll
    for (int e = 0; e < 9; ++e) acc[e] = v[e];
    for (int g = 1; g < ncg; ++g) {
#pragma unroll
      for (int e = 0; e < 9; ++e) acc[e] += __shfl(v[e], d8 + g * n8);
    }
#pragma unroll
    for (int e = 0; e < 9; ++e) v[e] = acc[e];
  }
  if (lane < n8) {
    const float inv = 1.0f / v[0];
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = v[1 + e] * inv;
    const int r = qi / G, gi = qi % G;
    if (a.a_tiles == 0)  // the single pass's GEMM layout
      apack_store8(a.Ap_out, r, (h * G + gi) * hd + lane * 8, out);
    else  // the rows GEMM's tiles (a batch of sequences)
      apack_store8_rt(a.Ap_out, seq * a.seq_rows + r, (h * G + gi) * hd + lane * 8, out, a.a_tiles);
  }
}

template <int NES>
static void launch_partial(const AttnArgs& a, int n_seq, hipStream_t s) {
  const int n_qt_max = (a.n_q / a.n_kv + 1) / 2;  // 16-query tiles of kMaxRows rows
  if (a.qt_per_wave == 2 && n_qt_max > 1) {
    hipLaunchKernelGGL((attn_partial_kernel<NES, 2>),
                       dim3(a.max_chunks * a.n_kv, 1, (n_qt_max + 1) / 2 * n_seq), dim3(64), 0, s, a.rows,
                       a.block_table, a.qf, a.k_cache, a.v_cache, a.qf_bytes, a.kv_layer_bytes, a);
  } else {
    hipLaunchKernelGGL((attn_partial_kernel<NES, 1>), dim3(a.max_chunks * a.n_kv, 1, n_qt_max * n_seq),
                       dim3(64), 0, s, a.rows, a.block_table, a.qf, a.k_cache, a.v_cache, a.qf_bytes,
                       a.kv_layer_bytes, a);
  }
}

hipError_t launch_attn(const AttnArgs& a, int n_rows, hipStream_t s) {
  if (n_rows < 1 || n_rows > kMaxRows) return hipErrorInvalidValue;
  const int n_seq = a.n_seq > 1 ? a.n_seq : 1;
  if (n_seq > 1 && (a.seq_rows < n_rows || n_seq * a.seq_rows > 8 * a.a_tiles))
    return hipErrorInvalidValue;
  switch ((a.hd + 31) / 32) {
    case 1: launch_partial<1>(a, n_seq, s); break;
    case 2: launch_partial<2>(a, n_seq, s); break;
    case 3: launch_partial<3>(a, n_seq, s); break;
    case 4: launch_partial<4>(a, n_seq, s); break;
    case 5: launch_partial<5>(a, n_seq, s); break;
    case 6: launch_partial<6>(a, n_seq, s); break;
    case 7: launch_partial<7>(a, n_seq, s); break;
    case 8: launch_partial<8>(a, n_seq, s); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.hd % 8 != 0 || a.hd / 8 > 64) return hipErrorInvalidValue;
  const dim3 mg(a.n_kv * (a.n_q / a.n_kv) * n_rows * n_seq), mb(64);
  switch (a.hd / 8) {
    case 2: hipLaunchKernelGGL(attn_merge_kernel<2>, mg, mb, 0, s, a.rows, a.ws_ml, a.ws_o, a); break;
    case 4: hipLaunchKernelGGL(attn_merge_kernel<4>, mg, mb, 0, s, a.rows, a.ws_ml, a.ws_o, a); break;
    case 8: hipLaunchKernelGGL(attn_merge_kernel<8>, mg, mb, 0, s, a.rows, a.ws_ml, a.ws_o, a); break;
    case 16: hipLaunchKernelGGL(attn_merge_kernel<16>, mg, mb, 0, s, a.rows, a.ws_ml, a.ws_o, a); break;
    case 32: hipLaunchKernelGGL(attn_merge_kernel<32>, mg, mb, 0, s, a.rows, a.ws_ml, a.ws_o, a); break;
    default: hipLaunchKernelGGL(attn_merge_kernel<0>, mg, mb, 0, s, a.rows, a.ws_ml, a.ws_o, a); break;
  }
  return hipGetLastError();
}

}  // namespace spec
