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
// per-token contraction.  The dot products run on v_dot2_f32_bf16 with the
// queries pre-split into bf16 hi + lo (attnres_split_queries, once per set of
// frozen queries); the weighted sums run on the matrix cores
// (v_mfma_f32_4x4x4_16b_bf16): the rows are transposed in registers into
// (source 2p, source 2p+1) element pairs once per token, which is exactly the
// MFMA B operand, and each weight enters as bf16 hi + lo.
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
typedef short short4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int kV>
constexpr int waves_per_simd2() { return kV == 1 ? 5 : kV == 2 ? 4 : 2; }
// The inter-block pass holds kK rows of kV vectors per lane.  With 8 rows at
// kV = 2 it needs about 150 VGPRs: 3 waves per SIMD and no spills run faster
// than 4 waves with spills to scratch.  4 rows fit in 128 VGPRs (4 waves).
// (8 rows at kV = 4, d above 14336, cannot fit in 256 and spill a little.)
template <int kV, int kK>
constexpr int waves_per_simd_prepare() {
  return kV == 1 ? (kK <= 4 ? 5 : 4) : kV == 2 ? (kK <= 4 ? 4 : 3) : 2;
}

// Byte selectors of v_perm_b32 (result byte i <- selector byte i; 0-3 pick the
// second operand's bytes, 4-7 the first's): (a.lo, b.lo) and (a.hi, b.hi).
constexpr unsigned kSelLo = 0x05040100u, kSelHi = 0x07060302u;

__device__ __forceinline__ unsigned pack2(float a, float b) { return pack_bf16(a, b); }

template <int kV, int kClose, int kK>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(waves_per_simd_prepare<kV, kK>())))
interblock_kernel(u32x4* __restrict__ src, int K, int B, int64_t T, int nvec, int64_t src_stride_v,
                  const u32x4* __restrict__ w_split, u32x4* __restrict__ inter, int64_t inter_stride_v,
                  float* __restrict__ logits, float* __restrict__ weights0, float eps, float inv_d,
                  const u32x4* __restrict__ layer_out) {
  __shared__ float red_ss[2][kMaxWaves][kMaxInter];
  __shared__ float red_dt[2][kMaxWaves][kMaxQueries][kMaxInter];
  // per wave: every query's weights as bf16 pairs (sources 2p, 2p+1), hi and lo
  __shared__ unsigned a_pairs[kMaxWaves][2][kMaxQueries][kPairs];

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
    u32x4 x[kK][kV];
    u32x4 f[kV];
#pragma unroll
    for (int s = 0; s < kK; ++s) {
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
      for (int s = 0; s < kK; ++s) {
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
    for (int s = 0; s < kK; ++s) {
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
      u32x4 qhi[kV], qlo[kV];
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int idx = v * nthr + tid;
        qhi[v] = u32x4{0, 0, 0, 0};
        qlo[v] = u32x4{0, 0, 0, 0};
        if (idx < nvec) {
          qhi[v] = w_split[(int64_t)(2 * b) * nvec + idx];
          qlo[v] = w_split[(int64_t)(2 * b + 1) * nvec + idx];
        }
      }
      float gdt = 0.f;
#pragma unroll
      for (int s = 0; s < kK; ++s) {
        if (s < K) {
          float dt = 0.f;
#pragma unroll
          for (int v = 0; v < kV; ++v)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              dt = dot2(x[s][v][k], qhi[v][k], dt);
              dt = dot2(x[s][v][k], qlo[v][k], dt);
            }
          gdt = put_lane(wave_sum(dt), s, gdt, s16);
        }
      }
      if (lane < kMaxInter) red_dt[buf][wave][b][lane] = gdt;
    }
    __syncthreads();

    // 4. softmax per query: lane L handles query 8r + L/8, source L%8, r = 0, 1
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
      // lanes with an even source pack (a_s, a_s+1) as bf16 hi and lo words
      const float a_next = dpp<kDppXor1>(a, a);
      if ((s & 1) == 0 && b < kMaxQueries) {
        const __bf16 h0 = (__bf16)a, h1 = (__bf16)a_next;
        a_pairs[wave][0][b][s >> 1] = __builtin_bit_cast(unsigned, bf16x2{h0, h1});
        a_pairs[wave][1][b][s >> 1] = pack_bf16(a - (float)h0, a_next - (float)h1);
      }
    }

    __builtin_amdgcn_wave_barrier();  // this wave's weight pairs are in LDS

    // 5. rows -> source-pair form: x[2p] holds (H_2p[j], H_2p+1[j]) for the even
    //    element j of every word, x[2p+1] the same for the odd element
#pragma unroll
    for (int p = 0; p < kK / 2; ++p)
#pragma unroll
      for (int v = 0; v < kV; ++v)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const unsigned ea = x[2 * p][v][k], eb = x[2 * p + 1][v][k];
          x[2 * p][v][k] = __builtin_amdgcn_perm(eb, ea, kSelLo);
          x[2 * p + 1][v][k] = __builtin_amdgcn_perm(eb, ea, kSelHi);
        }

    // 6. R_b = sum_s a_b,s H_s for every query on the matrix cores:
    //    v_mfma_f32_4x4x4_16b_bf16 works on 16 blocks of 4 lanes; in a block,
    //    lane (base+m) gives row m of A (query q0+m's weights for 4 sources),
    //    lane (base+n) gives column n of B (its own element of those 4
    //    sources, i.e. two source-pair words) and gets D[m][n] = R_q0+m at its
    //    element.  Weights enter as bf16 hi + lo (two products per source).
    const int mq = lane & 3;
    const int nsg = (K + 3) >> 2;  // source groups of 4
    for (int q0 = 0; q0 < B; q0 += 4) {
      short4v ahi[kK / 4], alo[kK / 4];
#pragma unroll
      for (int sg = 0; sg < kK / 4; ++sg) {
        const int qq = min(q0 + mq, kMaxQueries - 1);
        ahi[sg] = __builtin_bit_cast(short4v, *reinterpret_cast<const u32x2*>(&a_pairs[wave][0][qq][2 * sg]));
        alo[sg] = __builtin_bit_cast(short4v, *reinterpret_cast<const u32x2*>(&a_pairs[wave][1][qq][2 * sg]));
      }
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int idx = v * nthr + tid;
        // the vector's 8 elements in two halves of 4; half 0's results wait as
        // packed bf16 words so that every query row goes out as one 16-byte
        // store (two 8-byte halves of a line written apart cost far more)
        u32x2 first[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 acc[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int sg = 0; sg < kK / 4; ++sg) {
            if (sg < nsg) {
#pragma unroll
              for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                  const int k = 2 * h + kk;
                  const u32x2 bw = {x[4 * sg + e][v][k], x[4 * sg + 2 + e][v][k]};
                  const short4v bop = __builtin_bit_cast(short4v, bw);
                  acc[2 * kk + e] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi[sg], bop, acc[2 * kk + e], 0, 0, 0);
                  acc[2 * kk + e] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo[sg], bop, acc[2 * kk + e], 0, 0, 0);
                }
            }
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x2 o = {pack_bf16(acc[0][m], acc[1][m]), pack_bf16(acc[2][m], acc[3][m])};
            if (h == 0) {
              first[m] = o;
            } else if (q0 + m < B && idx < nvec) {
              const u32x4 row = {first[m][0], first[m][1], o[0], o[1]};
              __builtin_nontemporal_store(row, inter + (int64_t)(q0 + m) * inter_stride_v + t * (int64_t)nvec + idx);
            }
          }
        }
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

__global__ void __launch_bounds__(256) split_queries_kernel(const float* __restrict__ w, int64_t n, int d,
                                                           unsigned short* __restrict__ out) {
  const int64_t total = n * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t q = i / d, j = i - q * d;
    const float x = w[i];
    const __bf16 hi = (__bf16)x;
    const __bf16 lo = (__bf16)(x - (float)hi);
    out[(2 * q) * d + j] = __builtin_bit_cast(unsigned short, hi);
    out[(2 * q + 1) * d + j] = __builtin_bit_cast(unsigned short, lo);
  }
}

template <int kV, int kClose, int kK>
hipError_t launch_prepare(const PrepareArgs& a, hipStream_t stream) {
  const int nvec = a.d / 8;
  hipLaunchKernelGGL((interblock_kernel<kV, kClose, kK>), dim3((unsigned)a.grid), dim3(a.threads), 0, stream,
                     static_cast<u32x4*>(a.store), a.K, a.B, a.T, nvec, a.slot_stride / 8,
                     static_cast<const u32x4*>(a.w_split),
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

// Register footprint follows the number of inter-block rows held: blocks with
// at most 4 of them use the smaller instance.
template <int kClose, int kK>
hipError_t prepare_vk(const PrepareArgs& a, hipStream_t stream) {
  switch (a.vecs_per_lane) {
    case 1: return launch_prepare<1, kClose, kK>(a, stream);
    case 2: return launch_prepare<2, kClose, kK>(a, stream);
    case 3: return launch_prepare<3, kClose, kK>(a, stream);
    case 4: return launch_prepare<4, kClose, kK>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int kClose>
hipError_t prepare_v(const PrepareArgs& a, hipStream_t stream) {
  return a.K <= 4 ? prepare_vk<kClose, 4>(a, stream) : prepare_vk<kClose, kMaxInter>(a, stream);
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

hipError_t launch_split_queries(const float* w, int64_t n, int d, void* out, hipStream_t stream) {
  int64_t grid = (n * d + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(split_queries_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w, n, d,
                     static_cast<unsigned short*>(out));
  return hipGetLastError();
}

hipError_t launch_block_merge(const MergeArgs& a, hipStream_t stream) {
  return a.add ? merge_v<true>(a, stream) : merge_v<false>(a, stream);
}

}  // namespace attnres
