// Attainable-bandwidth probes for the aggregation's HBM access pattern.
//
// The aggregation reads S = 9 source rows of a token and writes one output row
// (bf16, d = 7168): ~90% reads, ~10% writes, as 10 concurrent streams; the
// fused step reads 10 rows and writes 2.  This program moves exactly those
// bytes with trivial arithmetic (xor), in several structures, so that the
// kernels' bandwidth can be set against what the memory system delivers for the
// same traffic on the same device:
//
//   token_*   one workgroup (448 lanes x 2 vectors) per token, every load of
//             the token issued at once -- the kernels' own structure, with
//             their token order (XCD x = workgroup % 8 takes runs of 32
//             consecutive tokens);
//   token_*_rr  the same, one token per XCD in turn (the order before runs);
//   chunk_*   one wave per 1 KiB chunk of every stream (64 lanes x 16 B), the
//             chunks in order, so that consecutive KiB go to different XCDs;
//             8 waves per CU (dynamic LDS caps the residency).  A per-token
//             kernel cannot take this shape without exchanging partial sums
//             across XCDs;
//   chunk_*_g128  the same with each XCD taking runs of 128 chunks;
//   stream_*  plain streams, one 16-byte vector per lane: read, write, copy.
//
// Prints one JSON object of GB/s (bytes moved / mean time over `reps` launches).
//
//   pattern_bench [T] [d] [reps]
//
// With a fourth argument `interblock`, it times instead the traffic of the
// two-phase schedule's inter-block pass when it closes a block by addition, for
// K = 3 .. 8 inter-block rows and B result rows: per token K rows and the layer
// output in; the closed row, B result rows and B x K float32 logits out -- one
// workgroup per token, every load issued at once, as the kernel does -- and
// prints the mean time per launch in microseconds for each K.
//
//   pattern_bench T d reps interblock [B]
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 448;
constexpr int kRunLog2 = 5;  // the kernels' XCD run: 32 tokens

#define CHECK(x)                                                                         \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) {                                                              \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                      \
    }                                                                                    \
  } while (0)

__device__ __forceinline__ u32x4 ld(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(u32x4 v, u32x4* p) { __builtin_nontemporal_store(v, p); }

// XCD b % 8 takes runs of 2^lg consecutive items (lg = 0: item b).
__device__ __forceinline__ int64_t xcd_item(int64_t b, int lg) {
  const int64_t x = b & 7, k = b >> 3;
  return ((((k >> lg) << 3) | x) << lg) | (k & ((INT64_C(1) << lg) - 1));
}

// One workgroup per token.  NR = 9: the 9 source rows; NR = 10: plus the layer
// output.  NW = 0: nothing written; 1: the output row; 2: also source row 8
// rewritten in place (the fused step's slot update).
template <int NR, int NW>
__global__ void __launch_bounds__(kThreads)
token_pattern(u32x4* __restrict__ src, const u32x4* __restrict__ lout, int64_t T, int nvec, u32x4* __restrict__ out,
              unsigned* sink, int lg) {
  const int64_t t = xcd_item(blockIdx.x, lg);
  if (t >= T) return;
  u32x4 x[NR][2];
#pragma unroll
  for (int s = 0; s < NR; ++s)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = v * kThreads + threadIdx.x;
      const u32x4* row = s < 9 ? src + (s * T + t) * nvec : lout + t * nvec;
      x[s][v] = idx < nvec ? ld(row + idx) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int idx = v * kThreads + threadIdx.x;
    u32x4 p = x[8][v];
    if (NR == 10) p ^= x[9][v];
    u32x4 o = p;
#pragma unroll
    for (int s = 0; s < 8; ++s) o ^= x[s][v];
    if (idx < nvec) {
      if (NW >= 1) st(o, out + t * nvec + idx);
      if (NW == 2) st(p, src + (8 * T + t) * nvec + idx);
    }
    if (NW == 0 && (o.x ^ o.y ^ o.z ^ o.w) == 0x9e3779b9u) sink[0] = o.x;
  }
}

// One wave per 1 KiB chunk: chunk c covers vectors [64 c, 64 c + 64) of every
// stream (the streams are n vectors long).  Same NR / NW meaning as above.
template <int NR, int NW>
__global__ void __launch_bounds__(64)
chunk_pattern(u32x4* __restrict__ src, const u32x4* __restrict__ lout, int64_t n, int64_t nchunks,
              u32x4* __restrict__ out, unsigned* sink, int lg) {
  const int64_t c = xcd_item(blockIdx.x, lg);
  if (c >= nchunks) return;
  const int64_t i = c * 64 + threadIdx.x;
  if (i >= n) return;
  u32x4 x[NR];
#pragma unroll
  for (int s = 0; s < NR; ++s) x[s] = ld((s < 9 ? src + s * n : lout) + i);
  u32x4 p = x[8];
  if (NR == 10) p ^= x[9];
  u32x4 o = p;
#pragma unroll
  for (int s = 0; s < 8; ++s) o ^= x[s];
  if (NW >= 1) st(o, out + i);
  if (NW == 2) st(p, src + 8 * n + i);
  if (NW == 0 && (o.x ^ o.y ^ o.z ^ o.w) == 0x9e3779b9u) sink[0] = o.x;
}

// Inter-block pass traffic at K rows, closing by addition: rows 0 .. K-1 of
// the token (row K-1 the open partial) and the layer output in; the partial
// written back with the layer output folded in, B result rows and the B x K
// logits out.
template <int K>
__global__ void __launch_bounds__(kThreads)
interblock_pattern(u32x4* __restrict__ src, const u32x4* __restrict__ lout, int64_t T, int nvec,
                   u32x4* __restrict__ inter, float* __restrict__ logits, int B) {
  const int64_t t = blockIdx.x;
  if (t >= T) return;
  u32x4 x[K + 1][2];
#pragma unroll
  for (int s = 0; s <= K; ++s)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = v * kThreads + threadIdx.x;
      const u32x4* row = s < K ? src + (s * T + t) * nvec : lout + t * nvec;
      x[s][v] = idx < nvec ? ld(row + idx) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int idx = v * kThreads + threadIdx.x;
    x[K - 1][v] ^= x[K][v];
    if (idx < nvec) st(x[K - 1][v], src + ((K - 1) * T + t) * nvec + idx);
  }
  u32x4 r[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    r[v] = x[0][v];
#pragma unroll
    for (int s = 1; s < K; ++s) r[v] ^= x[s][v];
  }
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int idx = v * kThreads + threadIdx.x;
      if (idx < nvec) st(r[v] ^ u32x4{(unsigned)b, 0, 0, 0}, inter + ((int64_t)b * T + t) * nvec + idx);
    }
  if (threadIdx.x < B * K)
    logits[((int64_t)(threadIdx.x / K) * T + t) * K + threadIdx.x % K] = __uint_as_float(r[0].x);
}

// Plain streams, one vector per lane: MODE 0 read, 1 write, 2 copy.
template <int MODE>
__global__ void __launch_bounds__(256) stream(const u32x4* __restrict__ a, u32x4* __restrict__ b, int64_t n,
                                              unsigned* sink) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  if (MODE == 0) {
    const u32x4 v = ld(a + i);
    if ((v.x ^ v.y ^ v.z ^ v.w) == 0x9e3779b9u) sink[0] = v.x;
  } else if (MODE == 1) {
    st(u32x4{1u, 2u, 3u, (unsigned)i}, b + i);
  } else {
    st(ld(a + i), b + i);
  }
}

}  // namespace

int interblock_main(int64_t T, int64_t d, int reps, int B);

int main(int argc, char** argv) {
  const int64_t T = argc > 1 ? std::atoll(argv[1]) : 262144;
  const int64_t d = argc > 2 ? std::atoll(argv[2]) : 7168;
  const int reps = argc > 3 ? std::atoi(argv[3]) : 5;
  if (T <= 0 || T > 0x7fffffff || d <= 0 || d % 8 != 0 || d / 8 > 2 * kThreads || reps <= 0) {
    std::fprintf(stderr, "need T > 0, d a multiple of 8 up to %d, reps > 0\n", 16 * kThreads);
    return 2;
  }
  if (argc > 4 && std::string(argv[4]) == "interblock") {
    const int B = argc > 5 ? std::atoi(argv[5]) : 12;
    if (B < 1 || B * 8 > kThreads) {
      std::fprintf(stderr, "need 1 <= B <= %d\n", kThreads / 8);
      return 2;
    }
    return interblock_main(T, d, reps, B);
  }
  const int nvec = (int)(d / 8);
  const int64_t n = T * nvec;                  // vectors per stream
  const int64_t nchunks = (n + 63) / 64;
  u32x4 *src = nullptr, *out = nullptr, *lout = nullptr;
  unsigned* sink = nullptr;
  CHECK(hipMalloc(&src, 9 * n * 16));
  CHECK(hipMalloc(&out, n * 16));
  CHECK(hipMalloc(&lout, n * 16));
  CHECK(hipMalloc(&sink, 64));
  CHECK(hipMemset(src, 1, 9 * n * 16));
  CHECK(hipMemset(out, 0, n * 16));
  CHECK(hipMemset(lout, 2, n * 16));
  int max_lds = 0;
  CHECK(hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, 0));
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
  const double row = (double)n * 16;
  // token grids: T rounded up to 8 runs (workgroups past T return)
  const int64_t run = INT64_C(1) << kRunLog2;
  const unsigned g_tok = (unsigned)((T + 8 * run - 1) / (8 * run) * (8 * run));
  const unsigned g_rr = (unsigned)T;
  // chunk grids: the fine order covers nchunks; runs of 128 round up to 8 runs
  const unsigned g_chunk = (unsigned)nchunks;
  const unsigned g_chunk128 = (unsigned)((nchunks + 8 * 128 - 1) / (8 * 128) * (8 * 128));
  const int lds8 = max_lds >= 20480 ? 20480 : 0;  // 160 KiB per CU / 20 KiB: 8 one-wave workgroups per CU
  const double t9r1w = gbps(10 * row, [&] { token_pattern<9, 1><<<g_tok, kThreads>>>(src, lout, T, nvec, out, sink, kRunLog2); });
  const double t9r = gbps(9 * row, [&] { token_pattern<9, 0><<<g_tok, kThreads>>>(src, lout, T, nvec, out, sink, kRunLog2); });
  const double t10r2w = gbps(12 * row, [&] { token_pattern<10, 2><<<g_tok, kThreads>>>(src, lout, T, nvec, out, sink, kRunLog2); });
  const double r9r1w = gbps(10 * row, [&] { token_pattern<9, 1><<<g_rr, kThreads>>>(src, lout, T, nvec, out, sink, 0); });
  const double r10r2w = gbps(12 * row, [&] { token_pattern<10, 2><<<g_rr, kThreads>>>(src, lout, T, nvec, out, sink, 0); });
  const double c9r1w = gbps(10 * row, [&] { chunk_pattern<9, 1><<<g_chunk, 64, lds8>>>(src, lout, n, nchunks, out, sink, 0); });
  const double c10r2w = gbps(12 * row, [&] { chunk_pattern<10, 2><<<g_chunk, 64, lds8>>>(src, lout, n, nchunks, out, sink, 0); });
  const double g9r1w = gbps(10 * row, [&] { chunk_pattern<9, 1><<<g_chunk128, 64, lds8>>>(src, lout, n, nchunks, out, sink, 7); });
  const double g10r2w = gbps(12 * row, [&] { chunk_pattern<10, 2><<<g_chunk128, 64, lds8>>>(src, lout, n, nchunks, out, sink, 7); });
  const unsigned g_st = (unsigned)((n + 255) / 256);
  const double sread = gbps(row, [&] { stream<0><<<g_st, 256>>>(src, out, n, sink); });
  const double swrite = gbps(row, [&] { stream<1><<<g_st, 256>>>(src, out, n, sink); });
  const double scopy = gbps(2 * row, [&] { stream<2><<<g_st, 256>>>(src, out, n, sink); });
  std::printf("{\"T\": %lld, \"d\": %lld, \"reps\": %d, "
              "\"token_pattern_9r1w_gbps\": %.1f, \"token_pattern_9r_gbps\": %.1f, \"fused_pattern_10r2w_gbps\": %.1f, "
              "\"token_rr_9r1w_gbps\": %.1f, \"token_rr_10r2w_gbps\": %.1f, "
              "\"chunk_9r1w_gbps\": %.1f, \"chunk_10r2w_gbps\": %.1f, "
              "\"chunk_g128_9r1w_gbps\": %.1f, \"chunk_g128_10r2w_gbps\": %.1f, "
              "\"stream_read_gbps\": %.1f, \"stream_write_gbps\": %.1f, \"stream_copy_gbps\": %.1f}\n",
              (long long)T, (long long)d, reps, t9r1w, t9r, t10r2w, r9r1w, r10r2w, c9r1w, c10r2w, g9r1w, g10r2w, sread,
              swrite, scopy);
  CHECK(hipFree(lout));
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  CHECK(hipFree(sink));
  return 0;
}

int interblock_main(int64_t T, int64_t d, int reps, int B) {
  constexpr int kMaxK = 8;
  const int nvec = (int)(d / 8);
  const int64_t n = T * nvec;  // vectors per row slab
  u32x4 *src = nullptr, *lout = nullptr, *inter = nullptr;
  float* logits = nullptr;
  CHECK(hipMalloc(&src, kMaxK * n * 16));
  CHECK(hipMalloc(&lout, n * 16));
  CHECK(hipMalloc(&inter, B * n * 16));
  CHECK(hipMalloc(&logits, (size_t)B * T * kMaxK * 4));
  CHECK(hipMemset(src, 1, kMaxK * n * 16));
  CHECK(hipMemset(lout, 2, n * 16));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  auto us = [&](auto launch) {
    launch();
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0, 0));
    for (int i = 0; i < reps; ++i) launch();
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    return ms / reps * 1e3;
  };
  const unsigned g = (unsigned)T;
  double t[kMaxK + 1] = {0};
  t[3] = us([&] { interblock_pattern<3><<<g, kThreads>>>(src, lout, T, nvec, inter, logits, B); });
  t[4] = us([&] { interblock_pattern<4><<<g, kThreads>>>(src, lout, T, nvec, inter, logits, B); });
  t[5] = us([&] { interblock_pattern<5><<<g, kThreads>>>(src, lout, T, nvec, inter, logits, B); });
  t[6] = us([&] { interblock_pattern<6><<<g, kThreads>>>(src, lout, T, nvec, inter, logits, B); });
  t[7] = us([&] { interblock_pattern<7><<<g, kThreads>>>(src, lout, T, nvec, inter, logits, B); });
  t[8] = us([&] { interblock_pattern<8><<<g, kThreads>>>(src, lout, T, nvec, inter, logits, B); });
  std::printf("{\"T\": %lld, \"d\": %lld, \"reps\": %d, \"B\": %d, \"interblock_pattern_us\": {", (long long)T,
              (long long)d, reps, B);
  for (int k = 3; k <= kMaxK; ++k) std::printf("%s\"%d\": %.1f", k > 3 ? ", " : "", k, t[k]);
  std::printf("}}\n");
  CHECK(hipFree(logits));
  CHECK(hipFree(inter));
  CHECK(hipFree(lout));
  CHECK(hipFree(src));
  return 0;
}
