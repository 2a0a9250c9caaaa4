// Partial-sum update of the current block (kimi.papertok.ai ch. 4 §4.3 eq 10;
// "Kimi K3技术详解系列（二）：AttnRes 与 Stable LatentMoE", §3): the block's
// layer outputs are summed into one block representation; the sum so far
// (up to the previous layer) is the partial source.
//
// partial <- round_bf16(f32(partial) + f32(layer_out)), one read-modify-write
// pass (3 streams of T*d elements), or partial <- layer_out for the first layer
// of a block (2 streams).  Closing a block moves no data: the slot simply
// becomes the block representation (kimi.papertok.ai §4.6: produced once at
// the boundary, then resident).  Element-wise and HBM-bound: 16-byte vectors,
// several independent vectors per lane to keep loads in flight, and one trip
// per workgroup: a grid that loops workgroups over the row keeps each trip's
// loads queued behind the previous trip's stores (16 workgroups per CU measured
// 6% slower at 3.76 GB per stream: 2.029 against 1.912 ms).
#include "device_common.h"
#include "internal.h"

namespace attnres {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // independent 16-byte vectors per lane per trip

template <bool kBf16, bool kCopy>
__global__ void __launch_bounds__(kThreads)
accumulate_kernel(const u32x4* partial, const u32x4* __restrict__ layer_out, u32x4* out, int64_t nvec) {
  const int64_t chunk = (int64_t)kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * chunk; base < nvec; base += (int64_t)gridDim.x * chunk) {
    u32x4 f[kUnroll], p[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      if (i < nvec) {
        f[u] = __builtin_nontemporal_load(layer_out + i);
        if constexpr (!kCopy) p[u] = __builtin_nontemporal_load(partial + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      if (i < nvec) {
        if constexpr (kCopy) {
          __builtin_nontemporal_store(f[u], out + i);
        } else {
          __builtin_nontemporal_store(add_rows(p[u], f[u], kBf16), out + i);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_accumulate(const AccumulateArgs& a, hipStream_t stream) {
  const int64_t nvec = a.elems / (a.bf16 ? 8 : 4);
  const int64_t chunk = (int64_t)kThreads * kUnroll;
  // one trip per workgroup up to the largest grid a launch takes (beyond it,
  // ~2^41 vectors, the workgroups loop)
  int64_t grid = (nvec + chunk - 1) / chunk;
  const int64_t cap = INT64_C(0x7fffffff);
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  const u32x4* p = static_cast<const u32x4*>(a.partial);
  const u32x4* f = static_cast<const u32x4*>(a.layer_out);
  u32x4* o = static_cast<u32x4*>(a.out != nullptr ? a.out : a.partial);
  if (a.copy) {
    hipLaunchKernelGGL((accumulate_kernel<true, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       p, f, o, nvec);
  } else if (a.bf16) {
    hipLaunchKernelGGL((accumulate_kernel<true, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       p, f, o, nvec);
  } else {
    hipLaunchKernelGGL((accumulate_kernel<false, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       p, f, o, nvec);
  }
  return hipGetLastError();
}

}  // namespace attnres
