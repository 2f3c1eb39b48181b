// spec_run.cpp -- native driver of libspec: runs the decode loop (draft loop,
// verify pass, accept/reject, commit) on a synthetic model pair through the
// C ABI alone, with no Python or PyTorch in the process.
//
// It serves two purposes: a plain command-line runner of the library, and a
// small, self-contained process for hardware-counter collection (rocprofv3
// --pmc), where the kernels must run exactly as the benchmark runs them.
//
//   spec_run [--pair 8b|1.3b|toy] [--k K] [--prompt N] [--rounds R]
//            [--warmup W] [--greedy] [--no-graphs] [--copy-mib M]
//   spec_run --gemm-rows M1,M2,... [--gemm-matrix gate|down|qkv] [--rounds R]
//
// --gemm-rows runs the batched-verify GEMM (spec_mat_mul) instead of the
// decode loop: the 8B-shaped gate/up (28672 x 4096), down (4096 x 14336) and
// QKV (6144 x 4096) matrices, each in enough copies (>= 1 GiB) that every
// launch streams its weights from HBM, R launches per copy and row count M,
// one JSON line per (matrix, M) with the mean time per launch; --gemm-matrix
// keeps the matrices whose name contains the given word.
//
// Weights are random, N(0, 0.02) per element (Box-Muller over a counter
// hash), rounded to bf16; norm gains are 1; the prompt is uniform token ids.
// --copy-mib M first runs a plain copy kernel over M MiB (M MiB read and M MiB
// written per launch, three launches): the known-size reference that scales
// the memory counters.
//
// Prints one JSON line: tokens/s, ms per round, median draft-loop and
// verify-pass times (hipEvents on the context's stream).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "spec.h"

#define HCK(x)                                                                      \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "spec_run: %s failed: %s\n", #x, hipGetErrorString(e_));      \
      exit(1);                                                                      \
    }                                                                               \
  } while (0)

namespace {

struct Shape {
  int L, d, nh, nkv, hd, F, V;
  float theta;
};

// bf16 weights N(0, std) from a counter hash: element i of tensor `tag`.
__device__ inline uint64_t mix64(uint64_t z) {
  z += 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

__global__ void fill_normal_bf16(uint16_t* p, size_t n, uint64_t tag, float std_) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint64_t h = mix64(tag * 0x100000001b3ull + i);
    const float u1 = ((h >> 40) + 1) * (1.0f / 16777217.0f);  // (0, 1]
    const float u2 = ((h >> 16) & 0xFFFFFF) * (1.0f / 16777216.0f);
    const float z = sqrtf(-2.0f * logf(u1)) * cosf(6.28318530718f * u2) * std_;
    uint32_t b = __float_as_uint(z);
    b += 0x7FFF + ((b >> 16) & 1);  // round to nearest even
    p[i] = (uint16_t)(b >> 16);
  }
}

__global__ void fill_uniform_f32(float* p, size_t n, uint64_t tag) {  // (-1, 1)
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = (float)(mix64(tag * 0x100000001b3ull + i) >> 40) * (2.0f / 16777216.0f) - 1.0f;
}

__global__ void fill_const_bf16(uint16_t* p, size_t n, uint16_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// plain copy: n16 16-byte elements read and written
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

struct Weights {
  std::vector<void*> owned;
  spec_model_desc desc{};
};

void* dalloc(Weights& w, size_t bytes) {
  void* p = nullptr;
  HCK(hipMalloc(&p, bytes));
  w.owned.push_back(p);
  return p;
}

void* normal(Weights& w, size_t n, uint64_t tag) {
  uint16_t* p = (uint16_t*)dalloc(w, n * 2);
  hipLaunchKernelGGL(fill_normal_bf16, dim3(4096), dim3(256), 0, 0, p, n, tag, 0.02f);
  HCK(hipGetLastError());
  return p;
}

void* ones(Weights& w, size_t n) {
  uint16_t* p = (uint16_t*)dalloc(w, n * 2);
  hipLaunchKernelGGL(fill_const_bf16, dim3(256), dim3(256), 0, 0, p, n, (uint16_t)0x3F80);
  HCK(hipGetLastError());
  return p;
}

// share: 0 none, 1 embedding and head from `from`, 2 tied head (lm_head = embed)
void make_model(Weights& w, const Shape& s, uint64_t seed, int share, const spec_model_desc* from) {
  spec_model_desc& m = w.desc;
  m.n_layers = s.L; m.d_model = s.d; m.n_heads = s.nh; m.n_kv_heads = s.nkv; m.head_dim = s.hd;
  m.d_ffn = s.F; m.vocab = s.V; m.rope_theta = s.theta; m.rms_eps = 1e-5f;
  const size_t L = s.L, d = s.d, q = (size_t)s.nh * s.hd, kv = (size_t)s.nkv * s.hd, F = s.F;
  uint64_t tag = seed * 64;
  if (share == 1) {
    m.embed = from->embed;
    m.lm_head = from->lm_head;
  } else {
    m.embed = normal(w, (size_t)s.V * d, tag++);
    m.lm_head = share == 2 ? m.embed : normal(w, (size_t)s.V * d, tag++);
  }
  m.attn_norm = ones(w, L * d);
  m.wq = normal(w, L * q * d, tag++);
  m.wk = normal(w, L * kv * d, tag++);
  m.wv = normal(w, L * kv * d, tag++);
  m.wo = normal(w, L * d * q, tag++);
  m.ffn_norm = ones(w, L * d);
  m.wg = normal(w, L * F * d, tag++);
  m.wu = normal(w, L * F * d, tag++);
  m.wd = normal(w, L * d * F, tag++);
  m.final_norm = ones(w, d);
}

void usage() {
  fprintf(stderr,
          "usage: spec_run [--pair 8b|1.3b|toy] [--k K] [--prompt N] [--rounds R] [--warmup W]\n"
          "                [--greedy] [--no-graphs] [--copy-mib M]\n"
          "       spec_run --gemm-rows M1,M2,... [--gemm-matrix gate|down|qkv] [--rounds R]\n");
  exit(2);
}

int check(int rc, spec_ctx* ctx, const char* what) {
  if (rc != SPEC_OK) {
    fprintf(stderr, "spec_run: %s returned %d: %s\n", what, rc, spec_last_error(ctx));
    exit(1);
  }
  return rc;
}

// The batched-verify GEMM over row counts Ms (see the header).
int gemm_rows(const std::vector<int>& Ms, int reps, const std::string& only) {
  struct Shp { const char* name; int N, K; };
  const Shp shapes[] = {{"8b gate/up", 28672, 4096}, {"8b down", 4096, 14336}, {"8b qkv", 6144, 4096}};
  int max_m = 1;
  for (int M : Ms) max_m = std::max(max_m, M);
  float *X, *Y;
  HCK(hipMalloc(&X, (size_t)max_m * 14336 * sizeof(float)));
  HCK(hipMalloc(&Y, (size_t)max_m * 28672 * sizeof(float)));
  hipLaunchKernelGGL(fill_uniform_f32, dim3(1024), dim3(256), 0, 0, X, (size_t)max_m * 14336, 77);
  HCK(hipGetLastError());
  hipEvent_t e0, e1;
  HCK(hipEventCreate(&e0));
  HCK(hipEventCreate(&e1));
  for (const Shp& sh : shapes) {
    if (!only.empty() && std::string(sh.name).find(only) == std::string::npos) continue;
    const size_t bytes = (size_t)sh.N * sh.K * 2;
    const int copies = std::max<int>(2, (int)(((size_t)1 << 30) / bytes + 1));
    std::vector<uint16_t*> W(copies);
    std::vector<spec_mat*> mats(copies);
    for (int c = 0; c < copies; ++c) {
      HCK(hipMalloc(&W[c], bytes));
      hipLaunchKernelGGL(fill_normal_bf16, dim3(4096), dim3(256), 0, 0, W[c], bytes / 2, 500 + c, 0.02f);
      HCK(hipGetLastError());
      check(spec_mat_create(W[c], sh.N, sh.K, &mats[c]), nullptr, "spec_mat_create");
      HCK(hipFree(W[c]));  // the packed copy is the library's
    }
    for (int M : Ms) {
      for (int c = 0; c < copies; ++c) check(spec_mat_mul(mats[c], X, M, Y, nullptr), nullptr, "spec_mat_mul");
      HCK(hipEventRecord(e0, nullptr));
      const int n = reps * copies;
      for (int i = 0; i < n; ++i) check(spec_mat_mul(mats[i % copies], X, M, Y, nullptr), nullptr, "spec_mat_mul");
      HCK(hipEventRecord(e1, nullptr));
      HCK(hipEventSynchronize(e1));
      float ms = 0.0f;
      HCK(hipEventElapsedTime(&ms, e0, e1));
      printf("{\"matrix\": \"%s\", \"N\": %d, \"K\": %d, \"M\": %d, \"launches\": %d, \"us_per_launch\": %.2f}\n",
             sh.name, sh.N, sh.K, M, n, ms * 1e3f / n);
      fflush(stdout);
    }
    for (spec_mat* m : mats) check(spec_mat_destroy(m), nullptr, "spec_mat_destroy");
  }
  HCK(hipEventDestroy(e0));
  HCK(hipEventDestroy(e1));
  HCK(hipFree(X));
  HCK(hipFree(Y));
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  std::string pair = "8b";
  int K = 4, prompt_len = -1, rounds = 20, warmup = 3, greedy = 0, graphs = 1, copy_mib = 0;
  std::vector<int> gemm_ms;
  std::string gemm_only;
  for (int i = 1; i < argc; ++i) {
    const std::string a = argv[i];
    auto next = [&]() -> const char* {
      if (i + 1 >= argc) usage();
      return argv[++i];
    };
    if (a == "--pair") pair = next();
    else if (a == "--k") K = atoi(next());
    else if (a == "--prompt") prompt_len = atoi(next());
    else if (a == "--rounds") rounds = atoi(next());
    else if (a == "--warmup") warmup = atoi(next());
    else if (a == "--greedy") greedy = 1;
    else if (a == "--no-graphs") graphs = 0;
    else if (a == "--copy-mib") copy_mib = atoi(next());
    else if (a == "--gemm-rows") {
      for (const char* t = next(); *t;) {
        gemm_ms.push_back(atoi(t));
        while (*t && *t != ',') ++t;
        if (*t == ',') ++t;
      }
    } else if (a == "--gemm-matrix") gemm_only = next();
    else usage();
  }
  if (!gemm_ms.empty()) {
    for (int M : gemm_ms)
      if (M < 1 || M > 128) usage();
    if (rounds < 1) usage();
    HCK(hipSetDevice(0));
    return gemm_rows(gemm_ms, rounds, gemm_only);
  }
  Shape ts, ds;
  int dshare;
  if (pair == "8b") {
    ts = {32, 4096, 32, 8, 128, 14336, 128256, 500000.0f};
    ds = {16, 2048, 32, 8, 64, 8192, 128256, 500000.0f};
    dshare = 2;
  } else if (pair == "1.3b") {
    ts = {24, 2048, 16, 16, 128, 5504, 32000, 10000.0f};
    ds = {4, 2048, 16, 16, 128, 5504, 32000, 10000.0f};
    dshare = 1;
  } else if (pair == "toy") {
    ts = {2, 64, 4, 4, 16, 256, 256, 10000.0f};
    ds = {1, 64, 4, 4, 16, 256, 256, 10000.0f};
    dshare = 1;
  } else {
    usage();
  }
  if (prompt_len < 0) prompt_len = pair == "8b" ? 1024 : pair == "1.3b" ? 512 : 32;
  if (K < 1 || K > SPEC_K_MAX || prompt_len < 1 || rounds < 1 || warmup < 0 || copy_mib < 0) usage();
  HCK(hipSetDevice(0));

  if (copy_mib > 0) {
    const size_t bytes = (size_t)copy_mib << 20;
    uint4 *src, *dst;
    HCK(hipMalloc(&src, bytes));
    HCK(hipMalloc(&dst, bytes));
    HCK(hipMemset(src, 1, bytes));
    for (int r = 0; r < 3; ++r)
      hipLaunchKernelGGL(copy_kernel, dim3(8192), dim3(256), 0, 0, src, dst, bytes / 16);
    HCK(hipGetLastError());
    HCK(hipDeviceSynchronize());
    HCK(hipFree(src));
    HCK(hipFree(dst));
    fprintf(stderr, "spec_run: copy reference: 3 launches over %d MiB\n", copy_mib);
  }

  Weights tw, dw;
  make_model(tw, ts, 1001, 0, nullptr);
  make_model(dw, ds, 1002, dshare, &tw.desc);
  HCK(hipDeviceSynchronize());

  std::vector<int32_t> prompt(prompt_len);
  uint64_t st = 1002;
  for (auto& t : prompt) {
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    t = (int32_t)((st >> 33) % (uint64_t)ts.V);
  }
  spec_init_params p{};
  p.target = tw.desc;
  p.draft = dw.desc;
  p.k_max = K;
  p.max_seq = prompt_len + (K + 1) * (rounds + warmup) + 16;
  p.greedy = greedy;
  p.use_graphs = graphs;
  spec_ctx* ctx = nullptr;
  check(spec_init(&p, prompt.data(), prompt_len, &ctx), nullptr, "spec_init");
  fprintf(stderr, "spec_run: %s pair ready, prompt %d, K %d\n", pair.c_str(), prompt_len, K);

  const size_t V = ts.V;
  int32_t *d_dev, *out_dev, *nacc_dev;
  float* D_dev;
  HCK(hipMalloc(&d_dev, K * sizeof(int32_t)));
  HCK(hipMalloc(&out_dev, (K + 1) * sizeof(int32_t)));
  HCK(hipMalloc(&nacc_dev, sizeof(int32_t)));
  HCK(hipMalloc(&D_dev, K * V * sizeof(float)));
  hipStream_t s = (hipStream_t)spec_stream(ctx);
  const uint64_t seed = 1003;
  std::vector<hipEvent_t> ev(3 * rounds + 2);
  for (auto& e : ev) HCK(hipEventCreate(&e));

  auto round = [&](hipEvent_t e0, hipEvent_t e1, hipEvent_t e2) {
    if (e0) HCK(hipEventRecord(e0, s));
    check(spec_draft(ctx, K, seed, d_dev, D_dev), ctx, "spec_draft");
    if (e1) HCK(hipEventRecord(e1, s));
    check(spec_verify(ctx, K, seed, d_dev, greedy ? nullptr : D_dev, out_dev, nacc_dev, nullptr,
                      nullptr),
          ctx, "spec_verify");
    if (e2) HCK(hipEventRecord(e2, s));
    check(spec_commit(ctx, out_dev, nacc_dev), ctx, "spec_commit");
  };
  for (int r = 0; r < warmup; ++r) round(nullptr, nullptr, nullptr);
  spec_state s0{}, s1{};
  check(spec_get_state(ctx, &s0), ctx, "spec_get_state");
  HCK(hipEventRecord(ev[3 * rounds], s));
  for (int r = 0; r < rounds; ++r) round(ev[3 * r], ev[3 * r + 1], ev[3 * r + 2]);
  HCK(hipEventRecord(ev[3 * rounds + 1], s));
  check(spec_get_state(ctx, &s1), ctx, "spec_get_state");
  if (s1.device_error != 0) {
    fprintf(stderr, "spec_run: device error bits %d\n", s1.device_error);
    return 1;
  }
  float total = 0.0f;
  HCK(hipEventElapsedTime(&total, ev[3 * rounds], ev[3 * rounds + 1]));
  std::vector<float> dm(rounds), vm(rounds);
  for (int r = 0; r < rounds; ++r) {
    HCK(hipEventElapsedTime(&dm[r], ev[3 * r], ev[3 * r + 1]));
    HCK(hipEventElapsedTime(&vm[r], ev[3 * r + 1], ev[3 * r + 2]));
  }
  std::sort(dm.begin(), dm.end());
  std::sort(vm.begin(), vm.end());
  const int tokens = s1.target_len - s0.target_len;
  printf("{\"pair\": \"%s\", \"K\": %d, \"greedy\": %d, \"graphs\": %d, \"rounds\": %d, "
         "\"tokens\": %d, \"tokens_per_s\": %.2f, \"ms_per_round\": %.4f, "
         "\"draft_ms_median\": %.4f, \"verify_ms_median\": %.4f}\n",
         pair.c_str(), K, greedy, graphs, rounds, tokens, tokens / (total / 1e3), total / rounds,
         dm[rounds / 2], vm[rounds / 2]);
  check(spec_destroy(ctx), nullptr, "spec_destroy");
  for (void* q : tw.owned) HCK(hipFree(q));
  for (void* q : dw.owned) HCK(hipFree(q));
  for (auto& e : ev) HCK(hipEventDestroy(e));
  HCK(hipFree(d_dev));
  HCK(hipFree(out_dev));
  HCK(hipFree(nacc_dev));
  HCK(hipFree(D_dev));
  return 0;
}
