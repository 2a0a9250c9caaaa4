// Attainable-bandwidth probe for the aggregation's HBM access pattern.
//
// The aggregation reads S = 9 source rows of a token and writes one output row
// (bf16, d = 7168): ~90% reads, ~10% writes, as 10 concurrent streams.  This
// program times the same pattern with trivial arithmetic (xor), plus plain
// streaming read / write / copy kernels, so the aggregation's achieved
// bandwidth can be compared with what the memory system delivers for this
// traffic mix on the same device.  Prints one JSON object.
//
//   pattern_bench [T] [d] [reps]
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 448;

#define CHECK(x)                                                                         \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) {                                                              \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                      \
    }                                                                                    \
  } while (0)

// One workgroup per token: 9 source rows in, one row out (or none).
template <bool kWrite>
__global__ void __launch_bounds__(kThreads)
token_pattern(const u32x4* __restrict__ src, int64_t T, int nvec, u32x4* __restrict__ out, unsigned* sink) {
  const int64_t t = blockIdx.x;
  u32x4 x[9][2];
#pragma unroll
  for (int s = 0; s < 9; ++s)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = v * kThreads + threadIdx.x;
      x[s][v] = idx < nvec ? __builtin_nontemporal_load(src + (s * T + t) * nvec + idx) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    u32x4 o = x[0][v];
#pragma unroll
    for (int s = 1; s < 9; ++s) o ^= x[s][v];
    const int idx = v * kThreads + threadIdx.x;
    if (kWrite) {
      if (idx < nvec) __builtin_nontemporal_store(o, out + t * nvec + idx);
    } else if ((o.x ^ o.y ^ o.z ^ o.w) == 0x9e3779b9u) {
      sink[0] = o.x;
    }
  }
}

// The fused step's pattern: 8 source rows + the partial row + the layer-output
// row in, the partial row written back in place and one output row out.
__global__ void __launch_bounds__(kThreads)
fused_pattern(u32x4* __restrict__ src, const u32x4* __restrict__ layer_out, int64_t T, int nvec,
              u32x4* __restrict__ out) {
  const int64_t t = blockIdx.x;
  u32x4 x[10][2];
#pragma unroll
  for (int s = 0; s < 10; ++s)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = v * kThreads + threadIdx.x;
      const u32x4* row = s < 9 ? src + (s * T + t) * nvec : layer_out + t * nvec;
      x[s][v] = idx < nvec ? __builtin_nontemporal_load(row + idx) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int idx = v * kThreads + threadIdx.x;
    const u32x4 p = x[8][v] ^ x[9][v];
    u32x4 o = p;
#pragma unroll
    for (int s = 0; s < 8; ++s) o ^= x[s][v];
    if (idx < nvec) {
      __builtin_nontemporal_store(p, src + (8 * T + t) * nvec + idx);
      __builtin_nontemporal_store(o, out + t * nvec + idx);
    }
  }
}

__global__ void __launch_bounds__(256) stream_read(const u32x4* __restrict__ a, int64_t n, unsigned* sink) {
  unsigned acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 1024) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * 256;
      v[u] = j < n ? __builtin_nontemporal_load(a + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

__global__ void __launch_bounds__(256) stream_write(u32x4* __restrict__ b, int64_t n) {
  const u32x4 v = {1u, 2u, 3u, 4u};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    __builtin_nontemporal_store(v, b + i);
}

}  // namespace

int main(int argc, char** argv) {
  const int64_t T = argc > 1 ? std::atoll(argv[1]) : 262144;
  const int64_t d = argc > 2 ? std::atoll(argv[2]) : 7168;
  const int reps = argc > 3 ? std::atoi(argv[3]) : 5;
  if (T <= 0 || T > 0x7fffffff || d <= 0 || d % 8 != 0 || d / 8 > 2 * kThreads || reps <= 0) {
    std::fprintf(stderr, "need T > 0, d a multiple of 8 up to %d, reps > 0\n", 16 * kThreads);
    return 2;
  }
  const int nvec = (int)(d / 8);
  const int64_t src_vecs = 9 * T * nvec, out_vecs = T * nvec;
  u32x4 *src = nullptr, *out = nullptr, *lout = nullptr;
  unsigned* sink = nullptr;
  CHECK(hipMalloc(&src, src_vecs * 16));
  CHECK(hipMalloc(&out, out_vecs * 16));
  CHECK(hipMalloc(&lout, out_vecs * 16));
  CHECK(hipMemset(lout, 2, out_vecs * 16));
  CHECK(hipMalloc(&sink, 64));
  CHECK(hipMemset(src, 1, src_vecs * 16));
  CHECK(hipMemset(out, 0, out_vecs * 16));
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  auto gbps = [&](double bytes, auto launch) {
    launch();
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0, 0));
    for (int i = 0; i < reps; ++i) launch();
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    return bytes / (ms / reps * 1e-3) / 1e9;
  };
  const double row = (double)T * d * 2.0;
  const int64_t grid = (int64_t)cus * 64;
  const double mixed = gbps(10 * row, [&] { token_pattern<true><<<T, kThreads>>>(src, T, nvec, out, sink); });
  const double ronly = gbps(9 * row, [&] { token_pattern<false><<<T, kThreads>>>(src, T, nvec, out, sink); });
  const double fused = gbps(12 * row, [&] { fused_pattern<<<T, kThreads>>>(src, lout, T, nvec, out); });
  const double rstream = gbps(9 * row, [&] { stream_read<<<grid, 256>>>(src, src_vecs, sink); });
  const double wstream = gbps(row, [&] { stream_write<<<grid, 256>>>(out, out_vecs); });
  std::printf("{\"T\": %lld, \"d\": %lld, \"reps\": %d, \"token_pattern_9r1w_gbps\": %.1f, "
              "\"token_pattern_9r_gbps\": %.1f, \"fused_pattern_10r2w_gbps\": %.1f, \"stream_read_gbps\": %.1f, "
              "\"stream_write_gbps\": %.1f}\n",
              (long long)T, (long long)d, reps, mixed, ronly, fused, rstream, wstream);
  CHECK(hipFree(lout));
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  CHECK(hipFree(sink));
  return 0;
}
