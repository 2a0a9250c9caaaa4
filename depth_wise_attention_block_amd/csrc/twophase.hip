// Two-phase inference schedule of Block AttnRes (kimi.papertok.ai ch. 4 §4.4
// third benefit and §4.6 inference): within block n the inter-block sources
// h_0, b_1 .. b_{n-1} do not change, so one batched pass reads each of them
// once for all the block's layer queries; each layer then folds its growing
// partial sum in with an online-softmax merge.
//
// Phase 1, interblock_kernel (one launch per block).  Per token: load the K
// inter-block rows once (optionally closing the previous block first: its last
// layer output is added into the partial slot, which becomes b_{n-1}); for
// each of the B queries compute the K logits; softmax per query; and write
//     R_b = sum_s softmax_s(z_b) H_s          (bf16 row, one per query)
//     z_b,s                                     (float32 logits)
// R_0 is exactly the block's first-layer residual (no partial source yet).
// The B x K dot products and B weighted sums are the arithmetic of a small
// per-token contraction; the weighted sums use v_dot2_f32_bf16 on source pairs
// (the rows are transposed in registers into (source 2p, source 2p+1) element
// pairs once per token) with each weight split into bf16 hi + lo.
//
// Phase 2, merge_kernel (one launch per later layer of the block).  Per token:
// update the partial slot with the previous layer's output (copy or add, as in
// the stand-alone update), score it with this layer's query, and merge with
// the inter-block part by online softmax:
//     M = max(m_inter, z_p),  A = l_inter e^(m_inter - M),  P = e^(z_p - M)
//     r = (A R + P x_p) / (A + P)
// where m_inter, l_inter are recomputed from the stored logits.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace attnres {
namespace {

constexpr int kMaxInter = kMaxInterSources;   // inter-block sources per pass
constexpr int kMaxQueries = kMaxBlockQueries; // layer queries per pass
constexpr int kPairs = kMaxInter / 2;
constexpr int kNoClose = 0, kCloseCopy = 1, kCloseAdd = 2;

template <int kV>
constexpr int waves_per_simd2() { return kV == 1 ? 5 : kV == 2 ? 4 : 2; }

// Byte selectors of v_perm_b32 (result byte i <- selector byte i; 0-3 pick the
// second operand's bytes, 4-7 the first's): (a.lo, b.lo) and (a.hi, b.hi).
constexpr unsigned kSelLo = 0x05040100u, kSelHi = 0x07060302u;

__device__ __forceinline__ unsigned pack2(float a, float b) { return pack_bf16(a, b); }

template <int kV, int kClose>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(waves_per_simd2<kV>())))
interblock_kernel(u32x4* __restrict__ src, int K, int B, int64_t T, int nvec, int64_t src_stride_v,
                  const float* __restrict__ w, u32x4* __restrict__ inter, int64_t inter_stride_v,
                  float* __restrict__ logits, float* __restrict__ weights0, float eps, float inv_d,
                  const u32x4* __restrict__ layer_out) {
  __shared__ float red_ss[2][kMaxWaves][kMaxInter];
  __shared__ float red_dt[2][kMaxWaves][kMaxQueries][kMaxInter];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int s16 = lane & 15;

  int buf = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x, buf ^= 1) {
    u32x4* tok = src + t * (int64_t)nvec;

    // 1. the K inter-block rows (the last one formed here when closing)
    u32x4 x[kMaxInter][kV];
    u32x4 f[kV];
#pragma unroll
    for (int s = 0; s < kMaxInter; ++s) {
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int idx = v * nthr + tid;
        x[s][v] = u32x4{0, 0, 0, 0};
        if (s < K && idx < nvec) {
          if (kClose != kNoClose && s == K - 1) {
            if constexpr (kClose == kCloseCopy) {
              x[s][v] = __builtin_nontemporal_load(layer_out + t * (int64_t)nvec + idx);
            } else {
              f[v] = __builtin_nontemporal_load(layer_out + t * (int64_t)nvec + idx);
              x[s][v] = __builtin_nontemporal_load(tok + s * src_stride_v + idx);
            }
          } else {
            x[s][v] = __builtin_nontemporal_load(tok + s * src_stride_v + idx);
          }
        }
      }
    }
    if constexpr (kClose != kNoClose) {
#pragma unroll
      for (int s = 0; s < kMaxInter; ++s) {
        if (s == K - 1) {
#pragma unroll
          for (int v = 0; v < kV; ++v) {
            const int idx = v * nthr + tid;
            if (idx < nvec) {
              if constexpr (kClose == kCloseAdd) x[s][v] = add_rows(x[s][v], f[v], true);
              __builtin_nontemporal_store(x[s][v], tok + s * src_stride_v + idx);
            }
          }
        }
      }
    }

    // 2. sums of squares (shared by every query)
    float gss = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxInter; ++s) {
      if (s < K) {
        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < kV; ++v)
#pragma unroll
          for (int k = 0; k < 4; ++k) ss = dot2(x[s][v][k], x[s][v][k], ss);
        gss = put_lane(wave_sum(ss), s, gss, s16);
      }
    }
    if (lane < kMaxInter) red_ss[buf][wave][lane] = gss;

    // 3. w_b . x_s for every query b and source s
    for (int b = 0; b < B; ++b) {
      Query<true, kV> q;
      load_query<true, kV>(q, w + (int64_t)b * nvec * 8, nvec, tid, nthr);
      float gdt = 0.f;
#pragma unroll
      for (int s = 0; s < kMaxInter; ++s) {
        if (s < K) {
          float dt = 0.f;
#pragma unroll
          for (int v = 0; v < kV; ++v)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              dt = dot2(x[s][v][k], q.hi[v][k], dt);
              dt = dot2(x[s][v][k], q.lo[v][k], dt);
            }
          gdt = put_lane(wave_sum(dt), s, gdt, s16);
        }
      }
      if (lane < kMaxInter) red_dt[buf][wave][b][lane] = gdt;
    }
    __syncthreads();

    // 4. softmax per query: lane L handles query 8r + L/8, source L%8, r = 0, 1
    float a_r[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int b = 8 * r + (lane >> 3);
      const int s = lane & 7;
      const bool valid = b < B && s < K;
      float z = -INFINITY;
      if (valid) {
        float ss = 0.f, dt = 0.f;
        for (int k = 0; k < nwaves; ++k) {
          ss += red_ss[buf][k][s];
          dt += red_dt[buf][k][b][s];
        }
        z = dt / sqrtf(ss * inv_d + eps);
      }
      const float m = group_max8(z);
      const float p = valid ? expf(z - m) : 0.f;
      const float l = group_sum8(p);
      const float a = valid ? p / l : 0.f;
      if (valid && wave == 0) {
        logits[((int64_t)b * T + t) * K + s] = z;
        if (b == 0 && weights0 != nullptr) weights0[t * K + s] = a;
      }
      a_r[r] = a;
    }

    // 5. rows -> source-pair form: x[2p] holds (H_2p[j], H_2p+1[j]) for the even
    //    element j of every word, x[2p+1] the same for the odd element
#pragma unroll
    for (int p = 0; p < kPairs; ++p)
#pragma unroll
      for (int v = 0; v < kV; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const unsigned ea = x[2 * p][v][k], eb = x[2 * p + 1][v][k];
          x[2 * p][v][k] = __builtin_amdgcn_perm(eb, ea, kSelLo);
          x[2 * p + 1][v][k] = __builtin_amdgcn_perm(eb, ea, kSelHi);
        }

    // 6. R_b = sum_s a_b,s H_s for every query
    for (int b = 0; b < B; ++b) {
      const float ab = b < 8 ? a_r[0] : a_r[1];
      const int base = 8 * (b & 7);
      unsigned ahi[kPairs], alo[kPairs];
#pragma unroll
      for (int p = 0; p < kPairs; ++p) {
        const float a0 = (2 * p < K) ? lane_bcast(ab, base + 2 * p) : 0.f;
        const float a1 = (2 * p + 1 < K) ? lane_bcast(ab, base + 2 * p + 1) : 0.f;
        const __bf16 h0 = (__bf16)a0, h1 = (__bf16)a1;
        ahi[p] = __builtin_bit_cast(unsigned, bf16x2{h0, h1});
        alo[p] = pack2(a0 - (float)h0, a1 - (float)h1);
      }
      u32x4* row = inter + (int64_t)b * inter_stride_v + t * (int64_t)nvec;
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int idx = v * nthr + tid;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
          if (2 * p < K) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              acc[2 * k] = dot2(x[2 * p][v][k], ahi[p], acc[2 * k]);
              acc[2 * k] = dot2(x[2 * p][v][k], alo[p], acc[2 * k]);
              acc[2 * k + 1] = dot2(x[2 * p + 1][v][k], ahi[p], acc[2 * k + 1]);
              acc[2 * k + 1] = dot2(x[2 * p + 1][v][k], alo[p], acc[2 * k + 1]);
            }
          }
        }
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = pack_bf16(acc[2 * k], acc[2 * k + 1]);
        if (idx < nvec) __builtin_nontemporal_store(o, row + idx);
      }
    }
  }
}

template <int kV, bool kAdd>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(waves_per_simd2<kV>())))
merge_kernel(u32x4* __restrict__ slot, const u32x4* __restrict__ layer_out, const u32x4* inter,
             const float* __restrict__ logits, int K, int64_t T, int nvec, const float* __restrict__ w,
             u32x4* out, float* __restrict__ weights, float eps, float inv_d) {
  __shared__ float red[2][kMaxWaves][2];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int s16 = lane & 15;

  Query<true, kV> q;
  load_query<true, kV>(q, w, nvec, tid, nthr);

  int buf = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x, buf ^= 1) {
    const int64_t rowoff = t * (int64_t)nvec;
    u32x4 R[kV], xp[kV];
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int idx = v * nthr + tid;
      R[v] = u32x4{0, 0, 0, 0};
      xp[v] = u32x4{0, 0, 0, 0};
      if (idx < nvec) {
        R[v] = __builtin_nontemporal_load(inter + rowoff + idx);
        const u32x4 f = __builtin_nontemporal_load(layer_out + rowoff + idx);
        if constexpr (kAdd) {
          xp[v] = add_rows(__builtin_nontemporal_load(slot + rowoff + idx), f, true);
        } else {
          xp[v] = f;
        }
        __builtin_nontemporal_store(xp[v], slot + rowoff + idx);
      }
    }
    const float zi = (s16 < K) ? logits[t * K + s16] : -INFINITY;

    float ss = 0.f, dt = 0.f;
#pragma unroll
    for (int v = 0; v < kV; ++v)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ss = dot2(xp[v][k], xp[v][k], ss);
        dt = dot2(xp[v][k], q.hi[v][k], dt);
        dt = dot2(xp[v][k], q.lo[v][k], dt);
      }
    ss = wave_sum(ss);
    dt = wave_sum(dt);
    if (lane == 0) {
      red[buf][wave][0] = ss;
      red[buf][wave][1] = dt;
    }
    __syncthreads();
    float ssp = 0.f, dtp = 0.f;
    for (int k = 0; k < nwaves; ++k) {
      ssp += red[buf][k][0];
      dtp += red[buf][k][1];
    }
    const float zp = dtp / sqrtf(ssp * inv_d + eps);

    // inter-block statistics from the stored logits, then the online merge
    const float mi = row_max16(zi);
    const float li = row_sum16((s16 < K) ? expf(zi - mi) : 0.f);
    const float M = fmaxf(mi, zp);
    const float A = li * expf(mi - M);
    const float P = expf(zp - M);
    const float inv = 1.0f / (A + P);
    const float ca = A * inv, cp = P * inv;
    if (weights != nullptr && wave == 0) {
      if (lane < K) weights[t * (K + 1) + lane] = expf(zi - M) * inv;
      if (lane == K) weights[t * (K + 1) + K] = cp;
    }
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int idx = v * nthr + tid;
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[k] = pack_bf16(fmaf(cp, bf16_lo(xp[v][k]), ca * bf16_lo(R[v][k])),
                         fmaf(cp, bf16_hi(xp[v][k]), ca * bf16_hi(R[v][k])));
      }
      if (idx < nvec) __builtin_nontemporal_store(o, out + rowoff + idx);
    }
  }
}

template <int kV, int kClose>
hipError_t launch_prepare(const PrepareArgs& a, hipStream_t stream) {
  const int nvec = a.d / 8;
  hipLaunchKernelGGL((interblock_kernel<kV, kClose>), dim3((unsigned)a.grid), dim3(a.threads), 0, stream,
                     static_cast<u32x4*>(a.store), a.K, a.B, a.T, nvec, a.slot_stride / 8, a.w,
                     static_cast<u32x4*>(a.inter), a.inter_stride / 8, a.logits, a.weights0, a.eps,
                     1.0f / (float)a.d, static_cast<const u32x4*>(a.layer_out));
  return hipGetLastError();
}

template <int kV, bool kAdd>
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int nvec = a.d / 8;
  hipLaunchKernelGGL((merge_kernel<kV, kAdd>), dim3((unsigned)a.grid), dim3(a.threads), 0, stream,
                     static_cast<u32x4*>(a.slot), static_cast<const u32x4*>(a.layer_out),
                     static_cast<const u32x4*>(a.inter), a.logits, a.K, a.T, nvec, a.w,
                     static_cast<u32x4*>(a.out), a.weights, a.eps, 1.0f / (float)a.d);
  return hipGetLastError();
}

template <int kClose>
hipError_t prepare_v(const PrepareArgs& a, hipStream_t stream) {
  switch (a.vecs_per_lane) {
    case 1: return launch_prepare<1, kClose>(a, stream);
    case 2: return launch_prepare<2, kClose>(a, stream);
    case 3: return launch_prepare<3, kClose>(a, stream);
    case 4: return launch_prepare<4, kClose>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool kAdd>
hipError_t merge_v(const MergeArgs& a, hipStream_t stream) {
  switch (a.vecs_per_lane) {
    case 1: return launch_merge<1, kAdd>(a, stream);
    case 2: return launch_merge<2, kAdd>(a, stream);
    case 3: return launch_merge<3, kAdd>(a, stream);
    case 4: return launch_merge<4, kAdd>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_block_prepare(const PrepareArgs& a, hipStream_t stream) {
  switch (a.close) {
    case PrepareArgs::kNone: return prepare_v<kNoClose>(a, stream);
    case PrepareArgs::kCopy: return prepare_v<kCloseCopy>(a, stream);
    case PrepareArgs::kAdd: return prepare_v<kCloseAdd>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_block_merge(const MergeArgs& a, hipStream_t stream) {
  return a.add ? merge_v<true>(a, stream) : merge_v<false>(a, stream);
}

}  // namespace attnres
