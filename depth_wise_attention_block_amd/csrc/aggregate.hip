// Block AttnRes depth aggregation kernel for gfx950 (MI355X).
//
// For one token the method ("Kimi K3技术详解系列（二）：AttnRes 与 Stable
// LatentMoE", §2; kimi.papertok.ai ch. 4 §4.2 eq 8-9) computes, over S <= 9
// sources H_s:
//     z_s = w . H_s / sqrt(mean(H_s^2) + eps),  a = softmax(z),  r = sum_s a_s H_s
// Per source and token that is two reductions over d and one weighted sum --
// about 2.7 flop per byte moved, far below the fp32 ridge point, so the kernel
// is bound by HBM bandwidth and MFMA has nothing to do here.
//
// Design (one workgroup = one token; batches past the grid cap take several
// launches):
//   * the workgroup's lanes split the d-vector into 16-byte pieces; each lane
//     loads its V pieces of ALL S sources at once (S*V outstanding 16-byte
//     loads per lane), so every source row is read from HBM exactly once and
//     each workgroup keeps ~S*d*2 bytes in flight;
//   * bf16 statistics use v_dot2_f32_bf16 on the packed pairs straight from
//     memory: sum of squares as dot2(x, x), and w.x as dot2(x, w_hi) +
//     dot2(x, w_lo) with the float32 query split into two bf16 halves once per
//     workgroup -- no unpacking before the reductions;
//   * the query's float32 loads are issued with the rows' and converted to
//     bf16 hi + lo only after all of them are in flight, so that a token costs
//     one memory round trip (at decode sizes that round trip is the kernel);
//   * the 2*S per-lane sums reduced over each 16-lane row together by DPP
//     exchanges that halve the values a lane holds (a ninth source by two
//     plain row sums), one LDS exchange of every row's partials and ONE
//     barrier per token;
//   * logits, max, exponentials and the normaliser are computed by lanes
//     0..S-1 of each 16-lane row and broadcast with readlane; the softmax is
//     exact here because all S scores are known before the weighted sum.  (The
//     online-softmax merge of separately computed parts belongs to the
//     two-phase schedule, not to this single pass.);
//   * the weighted sum of the raw sources is formed in float32 registers and
//     rounded once to bf16 (round to nearest even, v_cvt_pk_bf16_f32).
//
// Fused update (kUpdate != 0): the last source is the current block's slot
// after this layer's output has been added to it (kimi.papertok.ai §4.3 eq 10:
// the next layer attends over the partial sum up to the previous layer, or over
// the block representation just closed).  The kernel reads the old slot row and
// the layer output, forms the new slot row exactly as the stand-alone partial
// update does, writes it back and uses it from registers -- one HBM pass less
// than update-then-aggregate, bit-identical results.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace attnres {
namespace {

constexpr int kMaxSrc = 9;  // ATTNRES_MAX_SOURCES
constexpr int kUpdateNone = 0, kUpdateCopy = 1, kUpdateAdd = 2;

// Waves per SIMD each instance is built for: two 7-wave workgroups per CU for
// the d = 7168 shape (V = 2), i.e. at most 128 VGPRs; wider rows get fewer.
template <int kV>
constexpr int waves_per_simd() { return kV == 1 ? 5 : kV == 2 ? 4 : 2; }

// Instances bounded at kSmallSrc (or 2) sources hold fewer rows per lane and
// are built for more waves per SIMD: with only a few rows per token, the bytes
// a CU keeps in flight come from more resident workgroups rather than from
// more rows.
constexpr int kSmallSrc = 4;
template <int kV, int kMaxS>
constexpr int waves_per_simd_s() {
  return kMaxS > kSmallSrc ? waves_per_simd<kV>() : kMaxS <= 2 ? (kV == 1 ? 8 : kV == 2 ? 8 : kV == 3 ? 5 : 4)
                                                  : kV == 1 ? 7 : kV == 2 ? 6 : kV == 3 ? 4 : 3;
}

template <bool kBf16, int kV, int kUpdate, int kMaxS>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(waves_per_simd_s<kV, kMaxS>())))
aggregate_kernel(u32x4* __restrict__ src, int S, int64_t T, int nvec, int64_t src_stride_v,
                 const float* __restrict__ w, u32x4* __restrict__ out, float* __restrict__ weights,
                 float eps, float inv_d, const u32x4* __restrict__ layer_out, int64_t b0, int run_log2) {
  // [statistic][part]: per 16-lane row of every wave (part 4 * wave + row),
  // the row's sum of each source's sum of squares (statistic s, or 2 kP for a
  // ninth source) and w.x (kP + s, or 2 kP + 1)
  constexpr int kP = kMaxS > 8 ? 8 : kMaxS > 2 ? 4 : 2;  // sources reduced together
  static_assert(kMaxS <= kP + 1, "at most one source beyond the reduced ones");
  constexpr int kParts = 4 * kMaxWaves;
  __shared__ __align__(16) float red[2 * kP + 2][kParts];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int s16 = lane & 15;  // source handled by this lane in the softmax step

  // virtual index b0 + blockIdx.x; past the end (T rounded up to whole XCD
  // runs) there is nothing to do
  const int64_t t = xcd_token(b0 + blockIdx.x, run_log2);
  if (t >= T) return;
  {
    QueryLoads<kBf16, kV> ql;
    issue_query<kBf16, kV>(ql, w, nvec, tid, nthr);
    u32x4* tok = src + t * (int64_t)nvec;
    const int s_upd = kUpdate != kUpdateNone ? S - 1 : kMaxS;  // the updated slot, if any

    // 1. issue every load of this token: S sources x V vectors per lane (for
    //    the updated slot: the layer output, and the old slot row when adding).
    //    Each row is read through a buffer resource of its own (the row's
    //    bytes; none for sources past S), so lanes past the row and sources
    //    past S read zeros without a branch: a load behind a branch makes the
    //    compiler wait for every load before it at the join.
    const int off = tid * kVecBytes;           // vector v at off + v * nthr * 16
    const int row_bytes = nvec * kVecBytes;
    const u32x4* lrow = layer_out + t * (int64_t)nvec;
    u32x4 x[kMaxS][kV];
    u32x4 f[kV];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      const u32x4* row = (kUpdate == kUpdateCopy && s == s_upd) ? lrow : tok + s * src_stride_v;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(row), (short)0,
                                                                         s < S ? row_bytes : 0, kBufferConfig);
#pragma unroll
      for (int v = 0; v < kV; ++v) x[s][v] = load_nt(r, off + v * nthr * kVecBytes);
    }
    if constexpr (kUpdate == kUpdateAdd) {
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(lrow), (short)0, row_bytes, kBufferConfig);
#pragma unroll
      for (int v = 0; v < kV; ++v) f[v] = load_nt(r, off + v * nthr * kVecBytes);
    }
    if constexpr (kUpdate != kUpdateNone) {
      // new slot row = old + layer output (or the layer output), written back
#pragma unroll
      for (int s = 0; s < kMaxS; ++s) {
        if (s == s_upd) {
          const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(tok + s * src_stride_v, (short)0,
                                                                             row_bytes, kBufferConfig);
#pragma unroll
          for (int v = 0; v < kV; ++v) {
            if constexpr (kUpdate == kUpdateAdd) x[s][v] = add_rows(x[s][v], f[v], kBf16);
            store_nt(x[s][v], r, off + v * nthr * kVecBytes);
          }
        }
      }
    }

    // 2. per-lane partial statistics, then row sums
    Query<kBf16, kV> q;
    finish_query<kBf16, kV>(q, ql);
    // the first kP sources' two sums per lane, reduced over each 16-lane row
    // together (lane i of a row ends with value i: source i's sum of squares,
    // then w.x of source i - kP); a ninth source takes two plain row sums
    float st[2 * kP];
    float ss9 = 0.f, dt9 = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      float ss = 0.f, dt = 0.f;
      if (s < S) {
#pragma unroll
        for (int v = 0; v < kV; ++v) {
          if constexpr (kBf16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              ss = dot2(x[s][v][k], x[s][v][k], ss);
              dt = dot2(x[s][v][k], q.hi[v][k], dt);
              dt = dot2(x[s][v][k], q.lo[v][k], dt);
            }
          } else {
            const f32x4 xf = __builtin_bit_cast(f32x4, x[s][v]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              ss = fmaf(xf[k], xf[k], ss);
              dt = fmaf(xf[k], q.f[v][k], dt);
            }
          }
        }
      }
      if (s < kP) {
        st[s] = ss;
        st[kP + s] = dt;
      } else {
        ss9 = ss;
        dt9 = dt;
      }
    }
    const float rs = row_sums<2 * kP>(st, lane);

    // 3. combine the rows of all waves: one LDS exchange, one barrier
    const int part = 4 * wave + (lane >> 4);
    if (s16 < 2 * kP) red[s16][part] = rs;
    if constexpr (kMaxS > kP) {
      if (S > kP) {
        ss9 = row_sum16(ss9);
        dt9 = row_sum16(dt9);
        if (s16 == 0) {
          red[2 * kP][part] = ss9;
          red[2 * kP + 1][part] = dt9;
        }
      }
    }
    __syncthreads();

    // 4. logits and softmax over depth, lanes s16 < S of every row
    float z = -INFINITY;
    if (s16 < S) {
      const int is = s16 < kP ? s16 : 2 * kP, id = s16 < kP ? kP + s16 : 2 * kP + 1;
      float ss = 0.f, dt = 0.f;
      for (int p = 0; p < 4 * nwaves; p += 4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&red[is][p]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&red[id][p]);
        ss += (a4[0] + a4[1]) + (a4[2] + a4[3]);
        dt += (d4[0] + d4[1]) + (d4[2] + d4[3]);
      }
      z = dt / sqrtf(ss * inv_d + eps);
    }
    const float m = row_max16(z);
    const float p = (s16 < S) ? expf(z - m) : 0.f;
    const float l = row_sum16(p);
    const float a = p / l;
    if (weights != nullptr && wave == 0 && lane < S) weights[t * S + lane] = a;

    // 5. weighted sum of the raw sources in float32, one rounding to the output
    float as[kMaxS];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) as[s] = (s < S) ? lane_bcast(a, s) : 0.f;

    const __amdgpu_buffer_rsrc_t orow =
        __builtin_amdgcn_make_buffer_rsrc(out + t * (int64_t)nvec, (short)0, row_bytes, kBufferConfig);
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      if constexpr (kBf16) {
        float acc[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] = as[0] * bf16_lo(x[0][v][k]);
          acc[2 * k + 1] = as[0] * bf16_hi(x[0][v][k]);
        }
#pragma unroll
        for (int s = 1; s < kMaxS; ++s) {
          if (s < S) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              acc[2 * k] = fmaf(as[s], bf16_lo(x[s][v][k]), acc[2 * k]);
              acc[2 * k + 1] = fmaf(as[s], bf16_hi(x[s][v][k]), acc[2 * k + 1]);
            }
          }
        }
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = pack_bf16(acc[2 * k], acc[2 * k + 1]);
        store_nt(o, orow, off + v * nthr * kVecBytes);
      } else {
        f32x4 acc = as[0] * __builtin_bit_cast(f32x4, x[0][v]);
#pragma unroll
        for (int s = 1; s < kMaxS; ++s) {
          if (s < S) {
            const f32x4 xf = __builtin_bit_cast(f32x4, x[s][v]);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = fmaf(as[s], xf[k], acc[k]);
          }
        }
        store_nt(__builtin_bit_cast(u32x4, acc), orow, off + v * nthr * kVecBytes);
      }
    }
  }
}

// ---- more than 9 sources: online softmax over batches ----------------------
//
// Full AttnRes (kimi.papertok.ai ch. 4 §4.2: every earlier layer output is a
// source, S up to L + 1) or sublayer granularity needs more rows than fit in
// registers at once.  The sources are taken in batches of kB; after each batch
// the running maximum m, normaliser l and float32 accumulator are rescaled by
// exp(m_old - m_new) before the batch's terms are added ([TUT] §4.4: online
// softmax merges partial results computed separately).  One barrier per batch.
// The logits are kept in LDS so the weights can be written once m and l are
// final.
//
// The traffic is nearly all reads (S rows in, one out), so what matters is
// keeping loads in flight: the rows go through two register buffers, and the
// next batch is loaded as soon as this one's statistics are formed, so that it
// arrives while this batch's barrier, merge and weighted sum run (the batch
// loop is unrolled by two so that each buffer keeps its registers).  Two
// 9-row buffers take ~230 VGPRs at V = 2: one workgroup per CU whose next batch
// is always in flight beats two that each drain between batches (smaller
// batches at two workgroups per CU were slower still: more barriers).  Wider
// rows take smaller batches.
template <int kV>
constexpr int many_batch() { return kV <= 2 ? 9 : kV == 3 ? 5 : 3; }
template <int kV>
constexpr int waves_per_simd_many() { return kV == 1 ? 3 : 2; }

template <bool kBf16, int kV>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(waves_per_simd_many<kV>())))
aggregate_many_kernel(const u32x4* __restrict__ src, int S, int64_t T, int nvec, int64_t src_stride_v,
                      const float* __restrict__ w, u32x4* __restrict__ out, float* __restrict__ weights,
                      float eps, float inv_d, int64_t span, int run_log2) {
  constexpr int kB = many_batch<kV>();
  // a batch's statistics reduced per 16-lane row as in aggregate_kernel: the
  // first kP sources together, one more by plain row sums; [buffer][statistic][part]
  constexpr int kP = kB > 8 ? 8 : kB > 4 ? 4 : 2;
  static_assert(kB == kP + 1, "one source beyond the reduced ones");
  __shared__ __align__(16) float red[2][2 * kP + 2][4 * kMaxWaves];
  __shared__ float zbuf[kMaxSourcesMany];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int s16 = lane & 15;

  Query<kBf16, kV> q;
  load_query<kBf16, kV>(q, w, nvec, tid, nthr);
  constexpr int kE = kBf16 ? 8 : 4;  // elements per 16-byte vector
  const int nbatches = (S + kB - 1) / kB;

  int buf = 0;
  // virtual indices blockIdx.x, + gridDim.x, ... below span (T rounded up to
  // whole XCD runs; the grid is a multiple of 8 with runs, so a workgroup
  // stays on its XCD's runs)
  for (int64_t vb = blockIdx.x; vb < span; vb += gridDim.x) {
    const int64_t t = xcd_token(vb, run_log2);
    if (t >= T) continue;
    const u32x4* tok = src + t * (int64_t)nvec;
    float m = -INFINITY, l = 0.f;
    float acc[kV][kE];
#pragma unroll
    for (int v = 0; v < kV; ++v)
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[v][e] = 0.f;

    // rows b*kB .. of this token into x (rows past S left zero)
    auto load_batch = [&](u32x4 (&x)[kB][kV], int b) {
      const int s0 = b * kB;
#pragma unroll
      for (int s = 0; s < kB; ++s) {
#pragma unroll
        for (int v = 0; v < kV; ++v) {
          const int idx = v * nthr + tid;
          x[s][v] = u32x4{0, 0, 0, 0};
          if (s0 + s < S && idx < nvec)
            x[s][v] = __builtin_nontemporal_load(tok + (int64_t)(s0 + s) * src_stride_v + idx);
        }
      }
    };

    // batch b from x; loads batch b + 1 into xn once x's statistics are formed
    auto batch = [&](u32x4 (&x)[kB][kV], u32x4 (&xn)[kB][kV], int b) {
      const int s0 = b * kB;
      const int nb = min(kB, S - s0);
      float st[2 * kP];
      float ssx = 0.f, dtx = 0.f;
#pragma unroll
      for (int s = 0; s < kB; ++s) {
        float ss = 0.f, dt = 0.f;
        if (s < nb) {
#pragma unroll
          for (int v = 0; v < kV; ++v) {
            if constexpr (kBf16) {
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                ss = dot2(x[s][v][k], x[s][v][k], ss);
                dt = dot2(x[s][v][k], q.hi[v][k], dt);
                dt = dot2(x[s][v][k], q.lo[v][k], dt);
              }
            } else {
              const f32x4 xf = __builtin_bit_cast(f32x4, x[s][v]);
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                ss = fmaf(xf[k], xf[k], ss);
                dt = fmaf(xf[k], q.f[v][k], dt);
              }
            }
          }
        }
        if (s < kP) {
          st[s] = ss;
          st[kP + s] = dt;
        } else {
          ssx = ss;
          dtx = dt;
        }
      }
      const float rs = row_sums<2 * kP>(st, lane);
      const bool extra = nb > kP;
      if (extra) {
        ssx = row_sum16(ssx);
        dtx = row_sum16(dtx);
      }
      if (b + 1 < nbatches) load_batch(xn, b + 1);
      const int part = 4 * wave + (lane >> 4);
      if (s16 < 2 * kP) red[buf][s16][part] = rs;
      if (extra && s16 == 0) {
        red[buf][2 * kP][part] = ssx;
        red[buf][2 * kP + 1][part] = dtx;
      }
      __syncthreads();
      float z = -INFINITY;
      if (s16 < nb) {
        const int is = s16 < kP ? s16 : 2 * kP, id = s16 < kP ? kP + s16 : 2 * kP + 1;
        float ss = 0.f, dt = 0.f;
        for (int p = 0; p < 4 * nwaves; p += 4) {
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(&red[buf][is][p]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&red[buf][id][p]);
          ss += (a4[0] + a4[1]) + (a4[2] + a4[3]);
          dt += (d4[0] + d4[1]) + (d4[2] + d4[3]);
        }
        z = dt / sqrtf(ss * inv_d + eps);
        if (wave == 0 && lane < 16) zbuf[s0 + s16] = z;
      }
      buf ^= 1;
      // online merge of this batch into (m, l, acc)
      const float m_new = fmaxf(m, row_max16(z));
      const float c = expf(m - m_new);  // 0 on the first batch (m = -inf)
      const float p = (s16 < nb) ? expf(z - m_new) : 0.f;
      l = l * c + row_sum16(p);
      m = m_new;
      float ps[kB];
#pragma unroll
      for (int s = 0; s < kB; ++s) ps[s] = (s < nb) ? lane_bcast(p, s) : 0.f;
#pragma unroll
      for (int v = 0; v < kV; ++v) {
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[v][e] *= c;
#pragma unroll
        for (int s = 0; s < kB; ++s) {
          if (s < nb) {
            if constexpr (kBf16) {
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                acc[v][2 * k] = fmaf(ps[s], bf16_lo(x[s][v][k]), acc[v][2 * k]);
                acc[v][2 * k + 1] = fmaf(ps[s], bf16_hi(x[s][v][k]), acc[v][2 * k + 1]);
              }
            } else {
              const f32x4 xf = __builtin_bit_cast(f32x4, x[s][v]);
#pragma unroll
              for (int k = 0; k < 4; ++k) acc[v][k] = fmaf(ps[s], xf[k], acc[v][k]);
            }
          }
        }
      }
    };

    u32x4 xa[kB][kV], xb[kB][kV];
    load_batch(xa, 0);
    for (int b = 0; b < nbatches; b += 2) {
      batch(xa, xb, b);
      if (b + 1 >= nbatches) break;
      batch(xb, xa, b + 1);
    }

    const float inv_l = 1.0f / l;
    u32x4* orow = out + t * (int64_t)nvec;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int idx = v * nthr + tid;
      u32x4 o;
      if constexpr (kBf16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = pack_bf16(acc[v][2 * k] * inv_l, acc[v][2 * k + 1] * inv_l);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = __float_as_uint(acc[v][k] * inv_l);
      }
      if (idx < nvec) __builtin_nontemporal_store(o, orow + idx);
    }
    if (weights != nullptr && wave == 0) {
      for (int s = lane; s < S; s += 64) weights[t * S + s] = expf(zbuf[s] - m) * inv_l;
    }
  }
}

template <bool kBf16, int kV>
hipError_t launch_many(const AggregateArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int epv = kBf16 ? 8 : 4;
  const int nvec = a.d / epv;
  const int run_log2 = __builtin_ctz((unsigned)a.xcd_run);
  const int64_t run8 = 8 * (int64_t)a.xcd_run;
  const int64_t span = a.xcd_run > 1 ? (a.T + run8 - 1) / run8 * run8 : a.T;
  if ((a.xcd_run & (a.xcd_run - 1)) != 0 || a.grid <= 0 || (a.xcd_run > 1 && a.grid % 8 != 0))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((aggregate_many_kernel<kBf16, kV>), dim3((unsigned)a.grid), dim3(a.threads), 0, stream,
                     static_cast<const u32x4*>(a.sources), a.S, a.T, nvec, a.src_stride / epv, a.w,
                     static_cast<u32x4*>(a.out), a.weights, a.eps, 1.0f / (float)a.d, span, run_log2);
  return hipGetLastError();
}

template <bool kBf16, int kV, int kUpdate, int kMaxS>
hipError_t launch_s(const AggregateArgs& a, hipStream_t stream) {
  const int epv = kBf16 ? 8 : 4;
  const int nvec = a.d / epv;
  const int run_log2 = __builtin_ctz((unsigned)a.xcd_run);
  // virtual indices [0, span): T, rounded up to whole runs on all 8 XCDs
  const int64_t span =
      a.xcd_run > 1 ? (a.T + 8 * (int64_t)a.xcd_run - 1) / (8 * (int64_t)a.xcd_run) * (8 * (int64_t)a.xcd_run) : a.T;
  if ((a.xcd_run & (a.xcd_run - 1)) != 0 || a.grid <= 0 || (a.xcd_run > 1 && a.grid % 8 != 0))
    return hipErrorInvalidValue;
  // one workgroup per token; at most a.grid per launch (a multiple of 8 with
  // XCD runs, so that every launch starts on XCD 0)
  for (int64_t b0 = 0; b0 < span; b0 += a.grid) {
    const int64_t n = span - b0 < a.grid ? span - b0 : a.grid;
    hipLaunchKernelGGL((aggregate_kernel<kBf16, kV, kUpdate, kMaxS>), dim3((unsigned)n), dim3(a.threads), 0,
                       stream, static_cast<u32x4*>(const_cast<void*>(a.sources)), a.S, a.T, nvec,
                       a.src_stride / epv, a.w, static_cast<u32x4*>(a.out), a.weights, a.eps, 1.0f / (float)a.d,
                       static_cast<const u32x4*>(a.layer_out), b0, run_log2);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool kBf16, int kV, int kUpdate>
hipError_t launch(const AggregateArgs& a, hipStream_t stream) {
  return a.S <= 2           ? launch_s<kBf16, kV, kUpdate, 2>(a, stream)
         : a.S <= kSmallSrc ? launch_s<kBf16, kV, kUpdate, kSmallSrc>(a, stream)
                            : launch_s<kBf16, kV, kUpdate, kMaxSrc>(a, stream);
}

hipError_t launch_many_v(const AggregateArgs& a, hipStream_t stream) {
  switch ((a.bf16 ? 0 : 8) + a.vecs_per_lane) {
    case 1: return launch_many<true, 1>(a, stream);
    case 2: return launch_many<true, 2>(a, stream);
    case 3: return launch_many<true, 3>(a, stream);
    case 4: return launch_many<true, 4>(a, stream);
    case 9: return launch_many<false, 1>(a, stream);
    case 10: return launch_many<false, 2>(a, stream);
    case 11: return launch_many<false, 3>(a, stream);
    case 12: return launch_many<false, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int kUpdate>
hipError_t launch_v(const AggregateArgs& a, hipStream_t stream) {
  switch ((a.bf16 ? 0 : 8) + a.vecs_per_lane) {
    case 1: return launch<true, 1, kUpdate>(a, stream);
    case 2: return launch<true, 2, kUpdate>(a, stream);
    case 3: return launch<true, 3, kUpdate>(a, stream);
    case 4: return launch<true, 4, kUpdate>(a, stream);
    case 9: return launch<false, 1, kUpdate>(a, stream);
    case 10: return launch<false, 2, kUpdate>(a, stream);
    case 11: return launch<false, 3, kUpdate>(a, stream);
    case 12: return launch<false, 4, kUpdate>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_aggregate(const AggregateArgs& a, hipStream_t stream) {
  if (a.S > kMaxSrc) {
    if (a.update != AggregateArgs::kNoUpdate || a.S > kMaxSourcesMany) return hipErrorInvalidValue;
    return launch_many_v(a, stream);
  }
  switch (a.update) {
    case AggregateArgs::kNoUpdate: return launch_v<kUpdateNone>(a, stream);
    case AggregateArgs::kCopyUpdate: return launch_v<kUpdateCopy>(a, stream);
    case AggregateArgs::kAddUpdate: return launch_v<kUpdateAdd>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attnres
