// A stand-alone driver of the library for hardware-counter runs (rocprofv3
// --pmc): no PyTorch and no other library kernels run in its process, only
// the layer's own launches and two calibration kernels.
//
//   moe_profile_driver layer <workload> <n_tokens> <calls> [slot|atomic]
//       Builds a seeded synthetic layer of one of the five workload shapes
//       with this file's own generator (the same shapes and distributions as
//       the Python workloads, other values), runs `calls` forward calls over
//       16 token batches, and prints one JSON line: the workload, the distinct
//       routed experts per call and the algorithmic bytes per launch of each
//       kernel (the expert weights it streams, as the benchmark counts them).
//   moe_profile_driver copy <MiB> <dispatches>
//       A plain device copy of MiB mebibytes per dispatch (16-byte loads and
//       stores): its FETCH_SIZE and WRITE_SIZE readings scale the counters.
//   moe_profile_driver read <MiB> <dispatches>
//       A plain read of MiB mebibytes per dispatch (a few bytes written).
//
// Expert weights are random valid encodings of each format (the kernels'
// traffic does not depend on the values); the router, its bias and the
// tokens follow the workloads' normal distributions, so the routing (and the
// number of distinct experts a call streams) is that of a random layer.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "moe_mi355x.h"

namespace {

#define HIP_OK(x)                                                                        \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) {                                                              \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(2);                                                                           \
    }                                                                                    \
  } while (0)

// splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014): one stream per tensor, seeded from (workload, tensor).
struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed) {}
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }  // [0, 1)
  double normal() {  // Box-Muller
    double u1 = uniform(), u2 = uniform();
    if (u1 < 1e-300) u1 = 1e-300;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
  }
  // a cheap near-normal for bulk expert weights (whose values do not shape
  // the traffic): the sum of four 16-bit uniforms, centred and scaled to unit
  // variance (Irwin-Hall with n = 4)
  float bulk_normal() {
    const uint64_t v = next();
    const float s = (float)(v & 0xFFFF) + (float)((v >> 16) & 0xFFFF) +
                    (float)((v >> 32) & 0xFFFF) + (float)(v >> 48);
    return (s * (1.0f / 65536.0f) - 2.0f) * 1.7320508f;
  }
};

uint16_t to_bf16(float f) {  // round to nearest even
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct Workload {
  const char* name;
  int H, I, E, k, I_s, scoring, renorm;
  float rsf;
  int routed_fmt, shared_fmt;  // moe_format (shared_fmt unused without a shared expert)
  double w_std, bias_std, zipf;
  int accum;
};

const Workload kWorkloads[] = {
    {"tiny_bf16", 256, 128, 8, 2, 128, MOE_SCORE_SOFTMAX, 1, 1.0f, MOE_FMT_BF16, MOE_FMT_BF16,
     0.02, 0.0, 0.0, MOE_ACCUM_SLOT},
    {"qwen3_30b_a3b_mxfp4", 2048, 768, 128, 8, 0, MOE_SCORE_SOFTMAX, 1, 1.0f, MOE_FMT_MXFP4,
     MOE_FMT_BF16, 0.02, 0.0, 0.0, MOE_ACCUM_ATOMIC_F32},
    {"deepseek_v3_nvfp4", 7168, 2048, 256, 8, 2048, MOE_SCORE_SIGMOID, 1, 2.5f, MOE_FMT_NVFP4,
     MOE_FMT_BF16, 0.02, 0.1, 0.0, MOE_ACCUM_ATOMIC_F32},
    {"grouped_fp8_h4096", 4096, 1536, 128, 8, 4096, MOE_SCORE_SOFTMAX, 1, 1.0f,
     MOE_FMT_FP8_ROWSCALE, MOE_FMT_FP8_ROWSCALE, 0.02, 0.0, 1.1, MOE_ACCUM_SLOT},
    {"prefill_bf16_h4096", 4096, 1536, 128, 8, 0, MOE_SCORE_SOFTMAX, 1, 1.0f, MOE_FMT_BF16,
     MOE_FMT_BF16, 1.0, 0.0, 0.0, MOE_ACCUM_SLOT},
};

// Bytes of one expert's projection of rows x cols: values, then scales.
void proj_bytes(int fmt, int rows, int cols, size_t* data, size_t* scales) {
  const size_t n = (size_t)rows * cols;
  switch (fmt) {
    case MOE_FMT_BF16: *data = 2 * n; *scales = 0; break;
    case MOE_FMT_FP8_ROWSCALE: *data = n; *scales = 4 * (size_t)rows; break;
    case MOE_FMT_MXFP4: *data = n / 2; *scales = n / 32; break;
    default: *data = n / 2; *scales = n / 16; break;  // NVFP4
  }
}

void* dev_upload(const void* host, size_t bytes) {
  void* d = nullptr;
  HIP_OK(hipMalloc(&d, bytes < 256 ? 256 : bytes));
  HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

// One projection of `count` experts with random valid encodings of the
// format, uploaded. BF16 values are near-normal with deviation std; FP8 bytes
// avoid the NaN codes and carry FP32 row scales; FP4 nibbles are all valid,
// their E8M0 block scales near 2^-7 and E4M3 block scales moderate, tensor
// scales 1.
moe_weight make_proj(Rng& g, int fmt, int count, int rows, int cols, double std) {
  size_t db, sb;
  proj_bytes(fmt, rows, cols, &db, &sb);
  moe_weight w{};
  w.format = fmt;
  w.rows = rows;
  w.cols = cols;
  w.count = count;
  w.data_bytes = db * count;
  w.scale_bytes = sb * count;
  std::vector<uint8_t> data(w.data_bytes), sc(w.scale_bytes);
  if (fmt == MOE_FMT_BF16) {
    uint16_t* p = reinterpret_cast<uint16_t*>(data.data());
    for (size_t i = 0; i < w.data_bytes / 2; ++i) p[i] = to_bf16(g.bulk_normal() * (float)std);
  } else {
    for (size_t i = 0; i < w.data_bytes; i += 8) {
      uint64_t v = g.next();
      memcpy(&data[i], &v, std::min<size_t>(8, w.data_bytes - i));
    }
    if (fmt == MOE_FMT_FP8_ROWSCALE)
      for (auto& b : data)
        if ((b & 0x7F) == 0x7F) b ^= 1;  // 0x7F / 0xFF are NaN in E4M3FN
  }
  if (fmt == MOE_FMT_FP8_ROWSCALE) {
    float* p = reinterpret_cast<float*>(sc.data());
    for (size_t i = 0; i < w.scale_bytes / 4; ++i) p[i] = (float)(std / 64.0);
  } else if (fmt == MOE_FMT_MXFP4) {
    for (auto& b : sc) b = (uint8_t)(120 + g.next() % 8);
  } else if (fmt == MOE_FMT_NVFP4) {
    for (auto& b : sc) b = (uint8_t)(0x20 + g.next() % 16);
  }
  w.data = dev_upload(data.data(), w.data_bytes);
  if (w.scale_bytes) w.scales = dev_upload(sc.data(), w.scale_bytes);
  if (fmt == MOE_FMT_NVFP4) {
    std::vector<float> ts(count, 1.0f);
    w.tensor_scale = static_cast<const float*>(dev_upload(ts.data(), 4 * (size_t)count));
  }
  return w;
}

int run_layer(const Workload& wl, int n, int calls, int accum) {
  const int H = wl.H, E = wl.E;
  Rng gr(1000 + (uint64_t)(&wl - kWorkloads));
  moe_cfg cfg{};
  cfg.hidden = H;
  cfg.inter = wl.I;
  cfg.num_experts = E;
  cfg.top_k = wl.k;
  cfg.shared_inter = wl.I_s;
  cfg.scoring = wl.scoring;
  cfg.norm_topk_prob = wl.renorm;
  cfg.routed_scaling_factor = wl.rsf;
  cfg.accum_mode = accum;
  cfg.path = MOE_PATH_AUTO;
  // router: N(0, 1/sqrt(H)) rows; with a Zipf skew, a seeded rank r_e of
  // each expert and the log-prior -s ln(r_e) in the last column, where
  // every token carries 1.0
  std::vector<uint16_t> wr((size_t)E * H);
  std::vector<int> rank(E);
  for (int e = 0; e < E; ++e) rank[e] = e + 1;
  for (int e = E - 1; e > 0; --e) std::swap(rank[e], rank[(int)(gr.next() % (uint64_t)(e + 1))]);
  for (int e = 0; e < E; ++e)
    for (int c = 0; c < H; ++c) {
      float v = (float)(gr.normal() / sqrt((double)H));
      if (wl.zipf > 0 && c == H - 1) v = (float)(-wl.zipf * log((double)rank[e]));
      wr[(size_t)e * H + c] = to_bf16(v);
    }
  moe_router router{};
  router.weight = dev_upload(wr.data(), wr.size() * 2);
  if (wl.bias_std > 0) {
    std::vector<float> b(E);
    for (auto& v : b) v = (float)(gr.normal() * wl.bias_std);
    router.bias = static_cast<const float*>(dev_upload(b.data(), 4 * (size_t)E));
  }
  moe_experts ex{}, sh{};
  ex.gate = make_proj(gr, wl.routed_fmt, E, wl.I, H, wl.w_std);
  ex.up = make_proj(gr, wl.routed_fmt, E, wl.I, H, wl.w_std);
  ex.down = make_proj(gr, wl.routed_fmt, E, H, wl.I, wl.w_std);
  if (wl.I_s > 0) {
    sh.gate = make_proj(gr, wl.shared_fmt, 1, wl.I_s, H, wl.w_std);
    sh.up = make_proj(gr, wl.shared_fmt, 1, wl.I_s, H, wl.w_std);
    sh.down = make_proj(gr, wl.shared_fmt, 1, H, wl.I_s, wl.w_std);
  }
  // 16 token batches, x ~ N(0, 1) (1.0 in the last column with a Zipf skew)
  constexpr int kBatches = 16;
  std::vector<void*> xs(kBatches);
  for (int bi = 0; bi < kBatches; ++bi) {
    std::vector<uint16_t> x((size_t)n * H);
    for (int t = 0; t < n; ++t)
      for (int c = 0; c < H; ++c)
        x[(size_t)t * H + c] = to_bf16(wl.zipf > 0 && c == H - 1 ? 1.0f : (float)gr.normal());
    xs[bi] = dev_upload(x.data(), x.size() * 2);
  }
  const size_t ws_bytes = moe_workspace_bytes(&cfg, n);
  if (ws_bytes == 0) {
    fprintf(stderr, "workspace: %s\n", moe_last_error());
    return 1;
  }
  void *ws = nullptr, *out = nullptr, *idx = nullptr;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemset(ws, 0, ws_bytes));
  HIP_OK(hipMalloc(&out, (size_t)n * H * 2));
  HIP_OK(hipMalloc(&idx, (size_t)calls * n * wl.k * 4));
  HIP_OK(hipDeviceSynchronize());
  for (int c = 0; c < calls; ++c) {
    moe_topk_out tk{};
    tk.idx = static_cast<uint32_t*>(idx) + (size_t)c * n * wl.k;
    const moe_status st = moe_forward(&cfg, &router, &ex, wl.I_s > 0 ? &sh : nullptr,
                                      xs[c % kBatches], n, out, &tk, ws, ws_bytes, nullptr,
                                      nullptr);
    if (st != MOE_OK) {
      fprintf(stderr, "moe_forward: %s: %s\n", moe_status_str(st), moe_last_error());
      return 1;
    }
  }
  HIP_OK(hipDeviceSynchronize());
  uint32_t err = 0;
  HIP_OK(hipMemcpy(&err, static_cast<char*>(ws) + 128, 4, hipMemcpyDeviceToHost));
  std::vector<uint32_t> hidx((size_t)calls * n * wl.k);
  HIP_OK(hipMemcpy(hidx.data(), idx, hidx.size() * 4, hipMemcpyDeviceToHost));
  // distinct routed experts per call, and the bytes each launch streams
  double u_sum = 0;
  for (int c = 0; c < calls; ++c) {
    std::vector<uint32_t> v(hidx.begin() + (size_t)c * n * wl.k,
                            hidx.begin() + (size_t)(c + 1) * n * wl.k);
    std::sort(v.begin(), v.end());
    u_sum += (double)(std::unique(v.begin(), v.end()) - v.begin());
  }
  const double U = u_sum / calls;
  size_t gd, gs, dd, ds, sgd = 0, sgs = 0, sdd = 0, sds = 0;
  proj_bytes(wl.routed_fmt, wl.I, H, &gd, &gs);
  proj_bytes(wl.routed_fmt, H, wl.I, &dd, &ds);
  if (wl.I_s > 0) {
    proj_bytes(wl.shared_fmt, wl.I_s, H, &sgd, &sgs);
    proj_bytes(wl.shared_fmt, H, wl.I_s, &sdd, &sds);
  }
  const double gu = U * 2.0 * (gd + gs) + 2.0 * (sgd + sgs);
  const double dn = U * (double)(dd + ds) + (double)(sdd + sds);
  const double rt = (double)E * H * 2;
  const int launches = moe_num_launches(&cfg, n);
  printf("{\"workload\": \"%s\", \"n\": %d, \"calls\": %d, \"accum\": \"%s\", "
         "\"launches_per_call\": %d, \"distinct_experts_mean\": %.3f, \"error_word\": %u, ",
         wl.name, n, calls, accum == MOE_ACCUM_SLOT ? "slot" : "atomic", launches, U, err);
  if (launches == 1)
    printf("\"alg_bytes_per_launch\": {\"k_moe_decode\": %.0f}}\n", gu + dn + rt);
  else
    printf("\"alg_bytes_per_launch\": {\"k_g_gate_up\": %.0f, \"k_g_down\": %.0f}}\n", gu, dn);
  return err == 0 ? 0 : 1;
}

__global__ void k_copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void k_read16(const uint4* __restrict__ src, size_t n, uint32_t* out) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;  // (practically never written)
}

int run_calibration(bool copy, int mib, int dispatches) {
  const size_t bytes = (size_t)mib << 20, n = bytes / 16;
  void *a = nullptr, *b = nullptr;
  HIP_OK(hipMalloc(&a, bytes));
  HIP_OK(hipMemset(a, 1, bytes));
  if (copy) HIP_OK(hipMalloc(&b, bytes));
  else HIP_OK(hipMalloc(&b, 4096 * 4));
  HIP_OK(hipDeviceSynchronize());
  for (int d = 0; d < dispatches; ++d) {
    if (copy)
      hipLaunchKernelGGL(k_copy16, dim3(4096), dim3(256), 0, nullptr,
                         static_cast<const uint4*>(a), static_cast<uint4*>(b), n);
    else
      hipLaunchKernelGGL(k_read16, dim3(4096), dim3(256), 0, nullptr,
                         static_cast<const uint4*>(a), n, static_cast<uint32_t*>(b));
    HIP_OK(hipGetLastError());
  }
  HIP_OK(hipDeviceSynchronize());
  printf("{\"calibration\": \"%s\", \"bytes_per_dispatch\": %zu, \"dispatches\": %d}\n",
         copy ? "copy" : "read", bytes, dispatches);
  return 0;
}

int usage() {
  fprintf(stderr,
          "usage: moe_profile_driver layer <workload> <n_tokens> <calls> [slot|atomic]\n"
          "       moe_profile_driver copy|read <MiB> <dispatches>\n");
  return 2;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) return usage();
  const std::string mode = argv[1];
  if ((mode == "copy" || mode == "read") && argc == 4) {
    const int mib = atoi(argv[2]), d = atoi(argv[3]);
    if (mib < 1 || mib > 4096 || d < 1 || d > 100) return usage();
    return run_calibration(mode == "copy", mib, d);
  }
  if (mode != "layer" || argc < 5) return usage();
  const Workload* wl = nullptr;
  for (const auto& w : kWorkloads)
    if (w.name == std::string(argv[2])) wl = &w;
  if (!wl) {
    fprintf(stderr, "unknown workload %s\n", argv[2]);
    return 2;
  }
  const int n = atoi(argv[3]), calls = atoi(argv[4]);
  if (n < 1 || n > MOE_MAX_TOKENS || calls < 1 || calls > 10000) return usage();
  int accum = wl->accum;
  if (argc > 5) {
    if (std::string(argv[5]) == "slot") accum = MOE_ACCUM_SLOT;
    else if (std::string(argv[5]) == "atomic") accum = MOE_ACCUM_ATOMIC_F32;
    else return usage();
  }
  return run_layer(*wl, n, calls, accum);
}
