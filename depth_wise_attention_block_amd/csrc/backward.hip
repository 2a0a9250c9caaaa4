// Backward of the Block AttnRes depth aggregation for gfx950 (MI355X).
//
// The forward ("Kimi K3技术详解系列（二）：AttnRes 与 Stable LatentMoE", §2;
// kimi.papertok.ai ch. 4 §4.2 eq 8-9) is, per token over S sources H_s:
//     rho_s = sqrt(mean(H_s^2) + eps),  z_s = w . H_s / rho_s,
//     a = softmax(z),                    r = sum_s a_s H_s.
// Training recomputes it in the backward pass (kimi.papertok.ai §4.6: the
// aggregation sits inside activation checkpointing).  With g = dL/dr the
// derivative is, per token,
//     u_s = g . H_s,   delta_s = a_s (u_s - sum_s' a_s' u_s'),
//     dL/dH_s = a_s g + (delta_s / rho_s) w - (delta_s z_s / (d rho_s^2)) H_s,
//     dL/dw  += sum_s (delta_s / rho_s) H_s,
// the first term being the value path and the other two the softmax / query /
// key path of the gradient (llm-atlas.k1412.top/k3, study of the spike trajectory x backward path).
//
// One pass per token, like the forward: each lane loads its V 16-byte pieces
// of every source and of g at once; three reductions per source (sum of
// squares, w . H_s with w as bf16 hi + lo, g . H_s) share one LDS exchange and
// one barrier; lanes 0..S-1 of every 16-lane row form the softmax and the
// per-source coefficients, broadcast with readlane.  The float32 source
// gradients are then written (or added into, per source) one source at a
// time, the next source's old rows loading while the current one is formed.
// dL/dw is accumulated per lane over the workgroup's tokens and written as one
// float32 row per workgroup; reduce_rows_kernel sums those rows in a fixed
// order, so the result is deterministic for a given grid.  A caller that forms
// dL/dw itself gets every source's coefficients instead, and the grid is then
// one workgroup per token (no loop, so no token's loads wait behind the
// previous token's stores).
//
// Deferred sources (the inter-block sources every layer of a block shares)
// leave their gradient rows alone: the layer writes their coefficients
// (a_s, delta_s/rho_s, delta_s z_s/(d rho_s^2)) and block_backward_kernel
// applies all the block's layers at once, while block_dw_kernel (MFMA) adds
// their share of each layer's dL/dw.  When every source but the last is
// deferred, aggregate_backward_last_kernel streams the rows once and keeps
// only the last; the last source's (the partial sum's) share of dL/dw is then
// either summed there or formed per block by partial_dw_kernel from the
// coefficients.
//
// HBM bytes per token at S sources, bf16, all gradients accumulated:
//   2 S d (sources) + 2 d (g) + 8 S d (old and new float32 gradients)
//   (+ 2 d for the optional copy of the last source's gradient).
#include <math.h>

#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace attnres {
namespace {

constexpr int kMaxSrc = 9;  // ATTNRES_MAX_SOURCES

// Registers: all S sources, g and the query stay in registers for the whole
// token (~190 VGPRs at kV = 2), so one 7-wave workgroup fits per CU; 2 waves per
// SIMD is then the same occupancy as 3 and leaves room to avoid spills.
template <int kV>
constexpr int waves_per_simd_bwd() { return kV == 1 ? 4 : 2; }

// Elements of a 16-byte vector and the float32 gradient vectors it maps to.
template <bool kBf16>
struct Elems {
  static constexpr int kE = kBf16 ? 8 : 4;
  static constexpr int kG = kE / 4;  // f32x4 gradient vectors per source vector
};

template <bool kBf16>
__device__ __forceinline__ void unpack(u32x4 v, float (&e)[Elems<kBf16>::kE]) {
  if constexpr (kBf16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      e[2 * k] = bf16_lo(v[k]);
      e[2 * k + 1] = bf16_hi(v[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) e[k] = __uint_as_float(v[k]);
  }
}

// A float32 gradient row moves as kGv 16-byte pieces per lane, piece h of
// vector idx at (idx * kGv + h).  With kGv = 2 one instruction covers every
// other 16 bytes of its lines; non-temporal stores of the two halves of a line
// are not merged in L2 and each half goes to HBM as its own write (about twice
// the write traffic), while plain stores are merged there first.  The old row
// of a read-modify-write is read with plain loads as well, which measured
// faster than non-temporal ones.
template <int kGv>
__device__ __forceinline__ f32x4 load_grad_piece(const f32x4* p) {
  if constexpr (kGv == 1)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <int kGv>
__device__ __forceinline__ void store_grad_piece(f32x4 v, f32x4* p) {
  if constexpr (kGv == 1)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// dL/dw: each lane keeps its running sums for its own elements in LDS (one row
// of f32x4 per vector) and adds one token's share, summed in registers over the
// sources, per trip.
template <int kV, int kGv>
__device__ __forceinline__ void add_token_dw(f32x4 (*dw4)[64 * kMaxWaves], int tid, const float (&dtok)[kV][4 * kGv]) {
#pragma unroll
  for (int v = 0; v < kV; ++v)
#pragma unroll
    for (int h = 0; h < kGv; ++h) {
      f32x4 acc = dw4[v * kGv + h][tid];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += dtok[v][4 * h + c];
      dw4[v * kGv + h][tid] = acc;
    }
}

// kDw: dL/dw is formed here (per-lane sums over the workgroup's tokens, one
// row per workgroup); without it every source's coefficients are written
// instead and the grid is one workgroup per token.
template <bool kBf16, int kV, bool kDw>
__global__ void __launch_bounds__(64 * kMaxWaves)
__attribute__((amdgpu_waves_per_eu(waves_per_simd_bwd<kV>())))
aggregate_backward_kernel(const u32x4* __restrict__ src, int S, int64_t T, int nvec, int64_t src_stride_v,
                          const u32x4* __restrict__ last_src, const float* __restrict__ w,
                          const u32x4* __restrict__ gout,
                          f32x4* __restrict__ grad, int64_t grad_stride_v, unsigned acc_mask,
                          unsigned defer_mask, float* __restrict__ coef, int64_t coef_stride,
                          u32x4* __restrict__ grad_last, float* __restrict__ dw_rows, float eps, float inv_d) {
  using El = Elems<kBf16>;
  constexpr int kE = El::kE, kGv = El::kG;
  // [buffer][wave][sum of squares | w.x | g.x][source]
  __shared__ float red[2][kMaxWaves][3][16];
  // this lane's running dL/dw, [vector][lane] (each lane touches only its own)
  __shared__ f32x4 dw4[kDw ? kV * kGv : 1][64 * kMaxWaves];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int s16 = lane & 15;

  Query<kBf16, kV> q;
  load_query<kBf16, kV>(q, w, nvec, tid, nthr);
  if constexpr (kDw) {
#pragma unroll
    for (int k = 0; k < kV * kGv; ++k) dw4[k][tid] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int buf = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x, buf ^= 1) {
    const u32x4* tok = src + t * (int64_t)nvec;

    // 1. every source and g for this token, all loads at once
    u32x4 x[kMaxSrc][kV], g[kV];
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int idx = v * nthr + tid;
      g[v] = idx < nvec ? __builtin_nontemporal_load(gout + t * (int64_t)nvec + idx) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < kMaxSrc; ++s) {
      if (s < S) {
        // the last source may live elsewhere (a recomputed partial sum)
        const u32x4* row = (last_src != nullptr && s == S - 1) ? last_src + t * (int64_t)nvec
                                                               : tok + s * src_stride_v;
#pragma unroll
        for (int v = 0; v < kV; ++v) {
          const int idx = v * nthr + tid;
          x[s][v] = idx < nvec ? __builtin_nontemporal_load(row + idx) : u32x4{0, 0, 0, 0};
        }
      }
    }

    // 2. per source: sum of squares, w . H_s, g . H_s; wave sums
    float gss = 0.f, gdt = 0.f, gug = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSrc; ++s) {
      if (s < S) {
        float ss = 0.f, dt = 0.f, ug = 0.f;
#pragma unroll
        for (int v = 0; v < kV; ++v) {
          if constexpr (kBf16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              ss = dot2(x[s][v][k], x[s][v][k], ss);
              dt = dot2(x[s][v][k], q.hi[v][k], dt);
              dt = dot2(x[s][v][k], q.lo[v][k], dt);
              ug = dot2(x[s][v][k], g[v][k], ug);
            }
          } else {
            const f32x4 xf = __builtin_bit_cast(f32x4, x[s][v]);
            const f32x4 gf = __builtin_bit_cast(f32x4, g[v]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              ss = fmaf(xf[k], xf[k], ss);
              dt = fmaf(xf[k], q.f[v][k], dt);
              ug = fmaf(xf[k], gf[k], ug);
            }
          }
        }
        gss = put_lane(wave_sum(ss), s, gss, s16);
        gdt = put_lane(wave_sum(dt), s, gdt, s16);
        gug = put_lane(wave_sum(ug), s, gug, s16);
        __builtin_amdgcn_sched_barrier(0);  // three reductions in flight at a time
      }
    }
    if (lane < 16) {
      red[buf][wave][0][lane] = gss;
      red[buf][wave][1][lane] = gdt;
      red[buf][wave][2][lane] = gug;
    }
    __syncthreads();

    // 3. softmax and the per-source coefficients, lanes s16 < S of every row
    float z = -INFINITY, rho = 1.f, ug = 0.f;
    if (s16 < S) {
      float ss = 0.f, dt = 0.f;
      for (int k = 0; k < nwaves; ++k) {
        ss += red[buf][k][0][s16];
        dt += red[buf][k][1][s16];
        ug += red[buf][k][2][s16];
      }
      rho = sqrtf(ss * inv_d + eps);
      z = dt / rho;
    }
    const float m = row_max16(z);
    const float p = (s16 < S) ? expf(z - m) : 0.f;
    const float a = p / row_sum16(p);
    const float ubar = row_sum16(a * ug);            // g . r
    const float delta = a * (ug - ubar);             // dL/dz_s
    const float c1 = delta / rho;                    // coefficient of w (and of H_s in dL/dw)
    const float c3 = c1 * z * inv_d / rho;           // coefficient of H_s in dL/dH_s
    // deferred sources: their three coefficients go out instead of a gradient
    // row (every source's, when dL/dw is formed by the caller)
    if (wave == 0 && lane < S && (!kDw || ((defer_mask >> lane) & 1u))) {
      float* cf = coef + t * coef_stride + 3 * lane;
      cf[0] = a;
      cf[1] = c1;
      cf[2] = c3;
    }
    float as[kMaxSrc], c1s[kMaxSrc], c3s[kMaxSrc];
#pragma unroll
    for (int s = 0; s < kMaxSrc; ++s) {
      as[s] = s < S ? lane_bcast(a, s) : 0.f;
      c1s[s] = s < S ? lane_bcast(c1, s) : 0.f;
      c3s[s] = s < S ? lane_bcast(c3, s) : 0.f;
    }

    // 5. dL/dH_s = a_s g + c1_s w - c3_s H_s, written or added, source by
    //    source; the old rows of source s+1 load while source s is formed
    f32x4 old[2][kV][kGv];
    auto load_old = [&](int s, f32x4 (&o)[kV][kGv]) {
      const bool add = ((acc_mask & ~defer_mask) >> s) & 1u;
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int idx = v * nthr + tid;
#pragma unroll
        for (int h = 0; h < kGv; ++h) {
          o[v][h] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (add && idx < nvec)
            o[v][h] = load_grad_piece<kGv>(grad + s * grad_stride_v + (t * (int64_t)nvec + idx) * kGv + h);
        }
      }
    };
    load_old(0, old[0]);
    float dtok[kV][kE];
#pragma unroll
    for (int v = 0; v < kV; ++v)
#pragma unroll
      for (int e = 0; e < kE; ++e) dtok[v][e] = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSrc; ++s) {
      if (s < S) {
        if (s + 1 < S) load_old(s + 1, old[(s + 1) & 1]);
#pragma unroll
        for (int v = 0; v < kV; ++v) {
          const int idx = v * nthr + tid;
          // the query in float32 is hi + lo (exact) or w itself
          float xe[kE], ge[kE], wf[kE], r[kE];
          unpack<kBf16>(x[s][v], xe);
          unpack<kBf16>(g[v], ge);
          if constexpr (kBf16) {
            float lo[kE];
            unpack<true>(q.hi[v], wf);
            unpack<true>(q.lo[v], lo);
#pragma unroll
            for (int e = 0; e < kE; ++e) wf[e] += lo[e];
          } else {
#pragma unroll
            for (int e = 0; e < kE; ++e) wf[e] = q.f[v][e];
          }
#pragma unroll
          for (int e = 0; e < kE; ++e) r[e] = fmaf(as[s], ge[e], fmaf(c1s[s], wf[e], -c3s[s] * xe[e]));
          // this token's share of dL/dw: sum_s c1_s H_s for this lane's elements,
          // over the sources not deferred (the block pass adds the others')
          if (kDw && !((defer_mask >> s) & 1u)) {
#pragma unroll
            for (int e = 0; e < kE; ++e) dtok[v][e] = fmaf(c1s[s], xe[e], dtok[v][e]);
          }
#pragma unroll
          for (int h = 0; h < kGv; ++h) {
            f32x4 o = old[s & 1][v][h];
            o = f32x4{o[0] + r[4 * h], o[1] + r[4 * h + 1], o[2] + r[4 * h + 2], o[3] + r[4 * h + 3]};
            if (idx < nvec && !((defer_mask >> s) & 1u)) {
              store_grad_piece<kGv>(o, grad + s * grad_stride_v + (t * (int64_t)nvec + idx) * kGv + h);
              old[s & 1][v][h] = o;  // kept for the copy of the last source's gradient
            }
          }
        }
        if (grad_last != nullptr && s == S - 1) {
#pragma unroll
          for (int v = 0; v < kV; ++v) {
            const int idx = v * nthr + tid;
            u32x4 o;
            if constexpr (kBf16) {
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const f32x4 lo4 = old[s & 1][v][k >> 1];
                o[k] = pack_bf16(lo4[2 * (k & 1)], lo4[2 * (k & 1) + 1]);
              }
            } else {
              o = __builtin_bit_cast(u32x4, old[s & 1][v][0]);
            }
            if (idx < nvec) __builtin_nontemporal_store(o, grad_last + t * (int64_t)nvec + idx);
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // one source's rows in registers at a time
      }
    }
    if constexpr (kDw) add_token_dw<kV, kGv>(dw4, tid, dtok);
  }

  // 6. this workgroup's dL/dw row
  if constexpr (kDw) {
    float* row = dw_rows + (int64_t)blockIdx.x * nvec * kE;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int idx = v * nthr + tid;
      if (idx < nvec) {
#pragma unroll
        for (int h = 0; h < kGv; ++h) reinterpret_cast<f32x4*>(row)[idx * kGv + h] = dw4[v * kGv + h][tid];
      }
    }
  }
}

// The backward when every source but the last is deferred (each layer of a
// block defers the block's shared inter-block sources): only the last source's
// gradient row is formed, and only its share of dL/dw -- the deferred sources'
// shares are summed with their gradient rows in the block pass.  So after the
// statistics nothing but the last row is needed: the rows stream once through
// a three-row register ring, the last one is kept, and the kernel fits two
// workgroups per CU.  kDw as in aggregate_backward_kernel: without it the
// last source's coefficients are written too and nothing is summed over tokens.
template <bool kBf16, int kV, bool kDw>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(kV <= 2 ? 4 : 2)))
aggregate_backward_last_kernel(const u32x4* __restrict__ src, int S, int64_t T, int nvec, int64_t src_stride_v,
                               const u32x4* __restrict__ last_src, const float* __restrict__ w,
                               const u32x4* __restrict__ gout, f32x4* __restrict__ grad, int64_t grad_stride_v,
                               unsigned acc_mask, unsigned defer_mask, float* __restrict__ coef,
                               int64_t coef_stride, u32x4* __restrict__ grad_last, float* __restrict__ dw_rows,
                               float eps, float inv_d) {
  using El = Elems<kBf16>;
  constexpr int kE = El::kE, kGv = El::kG;
  constexpr int kRing = 3;
  __shared__ float red[2][kMaxWaves][3][16];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int s16 = lane & 15;
  const bool write_last = !((defer_mask >> (S - 1)) & 1u);

  Query<kBf16, kV> q;
  load_query<kBf16, kV>(q, w, nvec, tid, nthr);
  float dw[kV][kE];  // this lane's running share of dL/dw
#pragma unroll
  for (int v = 0; v < kV; ++v)
#pragma unroll
    for (int e = 0; e < kE; ++e) dw[v][e] = 0.f;

  int buf = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x, buf ^= 1) {
    const u32x4* tok = src + t * (int64_t)nvec;
    auto load_row = [&](int s, u32x4 (&xr)[kV]) {
      const u32x4* row = (last_src != nullptr && s == S - 1) ? last_src + t * (int64_t)nvec : tok + s * src_stride_v;
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int idx = v * nthr + tid;
        xr[v] = idx < nvec ? __builtin_nontemporal_load(row + idx) : u32x4{0, 0, 0, 0};
      }
    };

    u32x4 g[kV], xl[kV];
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int idx = v * nthr + tid;
      g[v] = idx < nvec ? __builtin_nontemporal_load(gout + t * (int64_t)nvec + idx) : u32x4{0, 0, 0, 0};
    }

    // 1. statistics, the rows streaming through the ring (kRing - 1 ahead)
    u32x4 ring[kRing][kV];
#pragma unroll
    for (int r = 0; r + 1 < kRing; ++r)
      if (r < S) load_row(r, ring[r]);
    float gss = 0.f, gdt = 0.f, gug = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSrc; ++s) {
      if (s < S) {
        if (s + kRing - 1 < S) load_row(s + kRing - 1, ring[(s + kRing - 1) % kRing]);
        const int slot = s % kRing;
        float ss = 0.f, dt = 0.f, ug = 0.f;
#pragma unroll
        for (int v = 0; v < kV; ++v) {
          if constexpr (kBf16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              ss = dot2(ring[slot][v][k], ring[slot][v][k], ss);
              dt = dot2(ring[slot][v][k], q.hi[v][k], dt);
              dt = dot2(ring[slot][v][k], q.lo[v][k], dt);
              ug = dot2(ring[slot][v][k], g[v][k], ug);
            }
          } else {
            const f32x4 xf = __builtin_bit_cast(f32x4, ring[slot][v]);
            const f32x4 gf = __builtin_bit_cast(f32x4, g[v]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              ss = fmaf(xf[k], xf[k], ss);
              dt = fmaf(xf[k], q.f[v][k], dt);
              ug = fmaf(xf[k], gf[k], ug);
            }
          }
          if (s == S - 1) xl[v] = ring[slot][v];
        }
        gss = put_lane(wave_sum(ss), s, gss, s16);
        gdt = put_lane(wave_sum(dt), s, gdt, s16);
        gug = put_lane(wave_sum(ug), s, gug, s16);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the last row's old gradient loads while the statistics are reduced
    f32x4 oldl[kV][kGv];
    {
      const bool add = write_last && ((acc_mask >> (S - 1)) & 1u);
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int idx = v * nthr + tid;
#pragma unroll
        for (int h = 0; h < kGv; ++h) {
          oldl[v][h] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (add && idx < nvec)
            oldl[v][h] =
                load_grad_piece<kGv>(grad + (S - 1) * grad_stride_v + (t * (int64_t)nvec + idx) * kGv + h);
        }
      }
    }
    if (lane < 16) {
      red[buf][wave][0][lane] = gss;
      red[buf][wave][1][lane] = gdt;
      red[buf][wave][2][lane] = gug;
    }
    __syncthreads();

    // 2. softmax and coefficients (as the general kernel)
    float z = -INFINITY, rho = 1.f, ug = 0.f;
    if (s16 < S) {
      float ss = 0.f, dt = 0.f;
      for (int k = 0; k < nwaves; ++k) {
        ss += red[buf][k][0][s16];
        dt += red[buf][k][1][s16];
        ug += red[buf][k][2][s16];
      }
      rho = sqrtf(ss * inv_d + eps);
      z = dt / rho;
    }
    const float m = row_max16(z);
    const float p = (s16 < S) ? expf(z - m) : 0.f;
    const float a = p / row_sum16(p);
    const float ubar = row_sum16(a * ug);
    const float delta = a * (ug - ubar);
    const float c1 = delta / rho;
    const float c3 = c1 * z * inv_d / rho;
    if (wave == 0 && lane < S && (!kDw || ((defer_mask >> lane) & 1u))) {
      float* cf = coef + t * coef_stride + 3 * lane;
      cf[0] = a;
      cf[1] = c1;
      cf[2] = c3;
    }

    // 3. the last source: its share of dL/dw, its gradient row and the copy
    if (write_last) {
      const float aL = lane_bcast(a, S - 1), c1L = lane_bcast(c1, S - 1), c3L = lane_bcast(c3, S - 1);
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        const int idx = v * nthr + tid;
        float xe[kE], ge[kE], wf[kE];
        unpack<kBf16>(xl[v], xe);
        unpack<kBf16>(g[v], ge);
        if constexpr (kBf16) {
          float lo[kE];
          unpack<true>(q.hi[v], wf);
          unpack<true>(q.lo[v], lo);
#pragma unroll
          for (int e = 0; e < kE; ++e) wf[e] += lo[e];
        } else {
#pragma unroll
          for (int e = 0; e < kE; ++e) wf[e] = q.f[v][e];
        }
        if constexpr (kDw) {
#pragma unroll
          for (int e = 0; e < kE; ++e) dw[v][e] = fmaf(c1L, xe[e], dw[v][e]);
        }
        f32x4 o[kGv];
#pragma unroll
        for (int h = 0; h < kGv; ++h) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int e = 4 * h + c;
            o[h][c] = oldl[v][h][c] + fmaf(aL, ge[e], fmaf(c1L, wf[e], -c3L * xe[e]));
          }
          if (idx < nvec)
            store_grad_piece<kGv>(o[h], grad + (S - 1) * grad_stride_v + (t * (int64_t)nvec + idx) * kGv + h);
        }
        if (grad_last != nullptr && idx < nvec) {
          u32x4 ob;
          if constexpr (kBf16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) ob[k] = pack_bf16(o[k >> 1][2 * (k & 1)], o[k >> 1][2 * (k & 1) + 1]);
          } else {
            ob = __builtin_bit_cast(u32x4, o[0]);
          }
          __builtin_nontemporal_store(ob, grad_last + t * (int64_t)nvec + idx);
        }
      }
    }
  }

  if constexpr (kDw) {
    float* row = dw_rows + (int64_t)blockIdx.x * nvec * kE;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int idx = v * nthr + tid;
      if (idx < nvec) {
#pragma unroll
        for (int h = 0; h < kGv; ++h)
          reinterpret_cast<f32x4*>(row)[idx * kGv + h] =
              f32x4{dw[v][4 * h], dw[v][4 * h + 1], dw[v][4 * h + 2], dw[v][4 * h + 3]};
      }
    }
  }
}

// Deferred gradients of a block's inter-block sources (the sources every layer
// of the block shares: h_0, b_1 .. b_{n-1}).  Each layer's backward wrote, per
// token and source, a_{l,s}, c1_{l,s} = delta/rho and c3_{l,s} =
// delta z/(d rho^2); here, per token and source,
//     G_s += sum_l (a_{l,s} g_l + c1_{l,s} w_l) - (sum_l c3_{l,s}) H_s,
// one read-modify-write of each gradient row per block instead of one per
// layer.  The coefficients of a token are staged in LDS and read as broadcasts;
// in memory layer l's triples start cls floats after layer l-1's (cls >= 3n:
// a layer's own last source may have its triple there too).
template <bool kBf16, int kV>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(kV <= 2 ? 4 : 2)))
block_backward_kernel(const u32x4* __restrict__ src, int n, int64_t T, int nvec, int64_t src_stride_v,
                      BlockRows rows, int B, const float* __restrict__ coef, int cls, f32x4* __restrict__ grad,
                      int64_t grad_stride_v, unsigned acc_mask, u32x4* __restrict__ grad_last) {
  using El = Elems<kBf16>;
  constexpr int kE = El::kE, kGv = El::kG;
  __shared__ float cf[2][kMaxBlockLayers * kMaxInterSources * 3];
  __shared__ float c3sum[2][kMaxInterSources];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int per_layer = n * 3;
  const int per_tok = B * per_layer;

  int buf = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x, buf ^= 1) {
    const float* ct = coef + t * (int64_t)(B * cls);
    for (int k = tid; k < per_tok; k += nthr) {
      const int l = k / per_layer;
      cf[buf][k] = ct[l * cls + (k - l * per_layer)];
    }
    __syncthreads();
    if (tid < n) {
      float c3 = 0.f;
      for (int l = 0; l < B; ++l) c3 += cf[buf][(l * n + tid) * 3 + 2];
      c3sum[buf][tid] = c3;
    }
    __syncthreads();
    const u32x4* tok = src + t * (int64_t)nvec;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const int idx = v * nthr + tid;
      if (idx >= nvec) continue;
      float acc[kMaxInterSources][kE];
#pragma unroll
      for (int s = 0; s < kMaxInterSources; ++s) {
        if (s < n) {
          float xe[kE];
          unpack<kBf16>(__builtin_nontemporal_load(tok + s * src_stride_v + idx), xe);
          const float c3 = c3sum[buf][s];
#pragma unroll
          for (int h = 0; h < kGv; ++h) {
            f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
            if ((acc_mask >> s) & 1u)
              o = load_grad_piece<kGv>(grad + s * grad_stride_v + (t * (int64_t)nvec + idx) * kGv + h);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[s][4 * h + c] = fmaf(-c3, xe[4 * h + c], o[c]);
          }
        }
      }
      // layer l's g and w rows, the next layer's loading meanwhile
      u32x4 gn = __builtin_nontemporal_load(static_cast<const u32x4*>(rows.g[0]) + t * (int64_t)nvec + idx);
      f32x4 wn[kGv];
#pragma unroll
      for (int h = 0; h < kGv; ++h) wn[h] = reinterpret_cast<const f32x4*>(rows.w[0])[idx * kGv + h];
      for (int l = 0; l < B; ++l) {
        float ge[kE], we[kE];
        unpack<kBf16>(gn, ge);
#pragma unroll
        for (int h = 0; h < kGv; ++h)
#pragma unroll
          for (int c = 0; c < 4; ++c) we[4 * h + c] = wn[h][c];
        if (l + 1 < B) {
          gn = __builtin_nontemporal_load(static_cast<const u32x4*>(rows.g[l + 1]) + t * (int64_t)nvec + idx);
#pragma unroll
          for (int h = 0; h < kGv; ++h) wn[h] = reinterpret_cast<const f32x4*>(rows.w[l + 1])[idx * kGv + h];
        }
#pragma unroll
        for (int s = 0; s < kMaxInterSources; ++s) {
          if (s < n) {
            const float a = cf[buf][(l * n + s) * 3], c1 = cf[buf][(l * n + s) * 3 + 1];
#pragma unroll
            for (int e = 0; e < kE; ++e) acc[s][e] = fmaf(a, ge[e], fmaf(c1, we[e], acc[s][e]));
          }
        }
      }
#pragma unroll
      for (int s = 0; s < kMaxInterSources; ++s) {
        if (s < n) {
#pragma unroll
          for (int h = 0; h < kGv; ++h)
            store_grad_piece<kGv>(f32x4{acc[s][4 * h], acc[s][4 * h + 1], acc[s][4 * h + 2], acc[s][4 * h + 3]},
                                  grad + s * grad_stride_v + (t * (int64_t)nvec + idx) * kGv + h);
          if (grad_last != nullptr && s == n - 1) {
            u32x4 o;
            if constexpr (kBf16) {
#pragma unroll
              for (int k = 0; k < 4; ++k) o[k] = pack_bf16(acc[s][2 * k], acc[s][2 * k + 1]);
            } else {
#pragma unroll
              for (int k = 0; k < 4; ++k) o[k] = __float_as_uint(acc[s][k]);
            }
            __builtin_nontemporal_store(o, grad_last + t * (int64_t)nvec + idx);
          }
        }
      }
    }
  }
}

// The deferred sources' share of each layer's dL/dw,
//     dw_l = sum over tokens t and inter-block sources s of c1_{t,l,s} H_s[t],
// is a dense contraction -- [layers] x [(token, source) pairs] x [d] -- and
// runs on the matrix cores as float32 MFMA 16x16x4: M = 16 layer slots, N = 16
// columns, K = 4 (token, source) pairs per step.  Lane L takes K slot L/16: it
// supplies the coefficient of layer L%16 (operand A) and 8 consecutive
// elements of that pair's source row (operand B of 8 column tiles: tile q
// holds columns col0 + 8 j + q, j = L%16).  The kN sources of a token take
// kNp slots (1, 2, 4 or 8; the padding slots read coefficient 0), so a lane's
// source is fixed -- or alternates between two, for kNp = 8 -- and only the
// token advances, by a uniform stride.  A workgroup of kDwWaves waves covers
// kDwWaves * 128 columns for one group of strided tokens (tg of ntg) and
// writes its partial rows to dw_part[tg][l][d] for a fixed-order sum.  A
// token's coefficients for layer l start at l * cls (cls >= 3 kN floats).
// Coefficients past the group's tokens or of layer slots past B come from a
// buffer load out of range (zero); rows are clamped to valid ones.  Every load
// is unconditional, so a ring of kDwRing steps stays in flight.
constexpr int kDwWaves = 4;
constexpr int kDwCols = 128;  // columns per wave
constexpr int kDwRing = 4;

template <bool kBf16, int kN>
__global__ void __launch_bounds__(64 * kDwWaves)
block_dw_kernel(const void* __restrict__ src, int64_t T, int d, int64_t src_stride, int B,
                const float* __restrict__ coef, int cls, float* __restrict__ dw_part, int ncolblocks) {
  constexpr int kNp = kN == 1 ? 1 : kN == 2 ? 2 : kN <= 4 ? 4 : 8;   // source slots per token
  constexpr int kTokPerStep = kNp <= 4 ? 4 / kNp : 1;
  constexpr int kStepsPerTok = kNp == 8 ? 2 : 1;
  static_assert(kDwRing % kStepsPerTok == 0, "a ring slot keeps its source");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = blockIdx.x % ncolblocks;
  const unsigned tg = blockIdx.x / ncolblocks;
  const unsigned ntg = gridDim.x / ncolblocks;
  const int j = lane & 15, kq = lane >> 4;
  const int col0 = (cb * kDwWaves + wave) * kDwCols;
  const bool col_ok = col0 + 8 * j < d;
  const int e = col_ok ? col0 + 8 * j : d - 8;          // clamped: such lanes write nothing
  const unsigned ntok = (unsigned)((T - tg + ntg - 1) / ntg);   // tokens of this group (tg < T)
  const unsigned per_tok = (unsigned)(B * cls);
  const unsigned tsub = kNp <= 4 ? kq / kNp : 0;        // token within a step
  const int slot = kNp <= 4 ? kq % kNp : kq;            // source slot (+4 on odd steps for kNp = 8)
  int64_t hbase[kStepsPerTok];
  unsigned cbase[kStepsPerTok];
  bool cval[kStepsPerTok];
#pragma unroll
  for (int p = 0; p < kStepsPerTok; ++p) {
    const int sp = slot + 4 * p;
    hbase[p] = (int64_t)(sp < kN ? sp : kN - 1) * src_stride + e;
    cbase[p] = (unsigned)(j * cls + sp * 3 + 1);
    cval[p] = sp < kN && j < B;
  }
  const unsigned steps =
      ((ntok + kTokPerStep - 1) / kTokPerStep * kStepsPerTok + kDwRing - 1) / kDwRing * kDwRing;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(coef), 0, (int)((unsigned)T * per_tok * 4u), 0x00020000);

  // operands of step i (parity p = i % kStepsPerTok, static in the ring), raw:
  // they are widened to float32 only when used, so the loads stay in flight
  constexpr int kW = kBf16 ? 1 : 2;   // 16-byte words of 8 elements
  auto load_step = [&](unsigned i, int p, unsigned& a, u32x4 (&hv)[kW]) {
    const unsigned tok = i / kStepsPerTok * kTokPerStep + tsub;
    const bool tv = tok < ntok;
    const unsigned t = tg + (tv ? tok : ntok - 1) * ntg;
    const unsigned coff = (tv && cval[p]) ? (t * per_tok + cbase[p]) * 4u : 0x80000000u;
    a = __builtin_amdgcn_raw_buffer_load_b32(crs, coff, 0, 0);
    const int64_t off = hbase[p] + (int64_t)((uint64_t)t * (unsigned)d);
    const u32x4* q = reinterpret_cast<const u32x4*>(static_cast<const char*>(src) + off * (kBf16 ? 2 : 4));
#pragma unroll
    for (int w = 0; w < kW; ++w) hv[w] = __builtin_nontemporal_load(q + w);
  };

  f32x4 acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  unsigned ra[kDwRing];
  u32x4 rh[kDwRing][kW];
#pragma unroll
  for (int r = 0; r < kDwRing; ++r) load_step(r, r % kStepsPerTok, ra[r], rh[r]);
  for (unsigned i0 = 0; i0 < steps; i0 += kDwRing) {
#pragma unroll
    for (int r = 0; r < kDwRing; ++r) {
      const float a = __uint_as_float(ra[r]);
      float h[8];
      if constexpr (kBf16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          h[2 * k] = bf16_lo(rh[r][0][k]);
          h[2 * k + 1] = bf16_hi(rh[r][0][k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = __uint_as_float(rh[r][k >> 2][k & 3]);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, h[q], acc[q], 0, 0, 0);
      // the slot is refilled after its last use, so the loads land in the
      // ring's own registers (no copy that would wait for them)
      __builtin_amdgcn_sched_barrier(0);
      load_step(i0 + r + kDwRing, r % kStepsPerTok, ra[r], rh[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // lane L holds rows 4 (L/16) + v of each tile, column j
  if (col_ok) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int l = 4 * kq + v;
      if (l < B) {
        float* row = dw_part + ((int64_t)tg * B + l) * d + col0 + 8 * j;
        *reinterpret_cast<f32x4*>(row) = f32x4{acc[0][v], acc[1][v], acc[2][v], acc[3][v]};
        *reinterpret_cast<f32x4*>(row + 4) = f32x4{acc[4][v], acc[5][v], acc[6][v], acc[7][v]};
      }
    }
  }
}

// out.p[l][j] (+)= sum over r < rows of in[l * layer_stride + r * row_stride + j]
// in a fixed order: slice k of 8 sums rows k, k+8, k+16, ... in turn, then the
// 8 slice sums are added in order.  A block covers 32 columns with 8 slices
// each; blockIdx.y is l.
__global__ void __launch_bounds__(256) reduce_rows_kernel(const float* __restrict__ in, int64_t rows,
                                                          int64_t row_stride, int64_t layer_stride, int n,
                                                          OutRows out, bool add) {
  __shared__ float part[8][32];
  const int col = threadIdx.x & 31, slice = threadIdx.x >> 5;
  const int j = blockIdx.x * 32 + col;
  const float* base = in + blockIdx.y * layer_stride + j;
  float acc = 0.f;
  if (j < n) {
    int64_t p = slice;
    for (; p + 24 < rows; p += 32) {       // four independent loads in flight
      const float a0 = base[p * row_stride], a1 = base[(p + 8) * row_stride], a2 = base[(p + 16) * row_stride],
                  a3 = base[(p + 24) * row_stride];
      acc = (((acc + a0) + a1) + a2) + a3;
    }
    for (; p < rows; p += 8) acc += base[p * row_stride];
  }
  part[slice][col] = acc;
  __syncthreads();
  if (slice == 0 && j < n) {
    float tot = part[0][col];
#pragma unroll
    for (int k = 1; k < 8; ++k) tot += part[k][col];
    float* o = out.p[blockIdx.y] + j;
    *o = add ? *o + tot : tot;
  }
}

// A layer's dL/dw share from a row of its own -- in the Block AttnRes backward
// the partial block sum that was the layer's last source, whose coefficient
// c1 = delta/rho the layer's backward wrote per token instead of summing it:
//     dw_part[tg][l][j] = sum over the tokens t = tg, tg + ntg, ... of c_l[t] X_l[t][j],
// tokens in increasing order, then reduce_rows_kernel sums the groups in a
// fixed order.  A workgroup covers kPartialDwThreads 16-byte vectors of one
// layer's row for one token group, kPdAhead tokens' vectors loading at once.
// A layer without a row gets zeros.
constexpr int kPdAhead = 8;

template <bool kBf16>
__global__ void __launch_bounds__(kPartialDwThreads)
partial_dw_kernel(DwRows rows, int64_t coef_stride, int64_t T, int nvec, int ncolblocks, int B,
                  float* __restrict__ dw_part) {
  using El = Elems<kBf16>;
  constexpr int kE = El::kE;
  const int l = blockIdx.y;
  const int cb = blockIdx.x % ncolblocks;
  const int64_t tg = blockIdx.x / ncolblocks;
  const int64_t ntg = gridDim.x / ncolblocks;
  const int idx = cb * kPartialDwThreads + threadIdx.x;
  const u32x4* __restrict__ x = static_cast<const u32x4*>(rows.x[l]);
  const float* __restrict__ c = rows.c[l];
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  if (x != nullptr && idx < nvec) {
    int64_t t = tg;
    for (; t + (kPdAhead - 1) * ntg < T; t += kPdAhead * ntg) {
      u32x4 xv[kPdAhead];
      float cv[kPdAhead];
#pragma unroll
      for (int k = 0; k < kPdAhead; ++k) {
        xv[k] = __builtin_nontemporal_load(x + (t + k * ntg) * (int64_t)nvec + idx);
        cv[k] = c[(t + k * ntg) * coef_stride];
      }
#pragma unroll
      for (int k = 0; k < kPdAhead; ++k) {
        float xe[kE];
        unpack<kBf16>(xv[k], xe);
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[e] = fmaf(cv[k], xe[e], acc[e]);
      }
    }
    for (; t < T; t += ntg) {
      float xe[kE];
      unpack<kBf16>(__builtin_nontemporal_load(x + t * (int64_t)nvec + idx), xe);
      const float cv = c[t * coef_stride];
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[e] = fmaf(cv, xe[e], acc[e]);
    }
  }
  if (idx < nvec) {
    f32x4* out = reinterpret_cast<f32x4*>(dw_part + ((int64_t)tg * B + l) * nvec * kE) + (int64_t)idx * (kE / 4);
#pragma unroll
    for (int h = 0; h < kE / 4; ++h) out[h] = f32x4{acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
  }
}

// The running partial sums of a block's layer outputs, formed exactly as the
// store forms them (each step one float32 addition, then for bf16 one rounding
// to nearest even): out[0] = F_0, out[k] = out[k-1] + F_k.  One pass: every
// layer output read once and every partial written once.
template <bool kBf16>
__global__ void __launch_bounds__(256) partial_sums_kernel(BlockRows rows, int count, int64_t nvec,
                                                           u32x4* __restrict__ out, int64_t out_stride_v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
    u32x4 f[kMaxBlockLayers];
#pragma unroll
    for (int k = 0; k < kMaxBlockLayers; ++k)
      if (k < count) f[k] = __builtin_nontemporal_load(static_cast<const u32x4*>(rows.g[k]) + i);
    u32x4 acc = f[0];
    __builtin_nontemporal_store(acc, out + i);
#pragma unroll
    for (int k = 1; k < kMaxBlockLayers; ++k) {
      if (k < count) {
        acc = add_rows(acc, f[k], kBf16);
        __builtin_nontemporal_store(acc, out + k * out_stride_v + i);
      }
    }
  }
}

template <bool kBf16, int kV>
hipError_t launch_bwd_v(const BackwardArgs& a, hipStream_t stream) {
  const int nvec = a.d / (kBf16 ? 8 : 4);
  if (a.T > 0) {
    auto kernel = a.form_dw ? (a.last_only ? aggregate_backward_last_kernel<kBf16, kV, true>
                                           : aggregate_backward_kernel<kBf16, kV, true>)
                            : (a.last_only ? aggregate_backward_last_kernel<kBf16, kV, false>
                                           : aggregate_backward_kernel<kBf16, kV, false>);
    hipLaunchKernelGGL(kernel, dim3((unsigned)a.grid), dim3(a.threads), 0, stream,
                       static_cast<const u32x4*>(a.sources), a.S, a.T, nvec, a.src_stride / (kBf16 ? 8 : 4),
                       static_cast<const u32x4*>(a.last_source), a.w,
                       static_cast<const u32x4*>(a.grad_out), reinterpret_cast<f32x4*>(a.grad_sources),
                       a.grad_stride / 4, a.acc_mask, a.defer_mask, a.coef, a.coef_stride,
                       static_cast<u32x4*>(a.grad_last), a.workspace, a.eps, 1.0f / (float)a.d);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!a.form_dw) return hipSuccess;
  OutRows out{};
  out.p[0] = a.grad_w;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)((a.d + 31) / 32)), dim3(256), 0, stream, a.workspace,
                     a.T > 0 ? a.grid : (int64_t)0, (int64_t)a.d, (int64_t)0, a.d, out, false);
  return hipGetLastError();
}

template <bool kBf16>
hipError_t launch_bwd(const BackwardArgs& a, hipStream_t stream) {
  switch (a.vecs_per_lane) {
    case 1: return launch_bwd_v<kBf16, 1>(a, stream);
    case 2: return launch_bwd_v<kBf16, 2>(a, stream);
    case 3: return launch_bwd_v<kBf16, 3>(a, stream);
    case 4: return launch_bwd_v<kBf16, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool kBf16, int kV>
hipError_t launch_block_v(const BlockBackwardArgs& a, hipStream_t stream) {
  const int nvec = a.d / (kBf16 ? 8 : 4);
  hipLaunchKernelGGL((block_backward_kernel<kBf16, kV>), dim3((unsigned)a.grid), dim3(a.threads), 0, stream,
                     static_cast<const u32x4*>(a.sources), a.n, a.T, nvec, a.src_stride / (kBf16 ? 8 : 4), a.rows,
                     a.B, a.coef, a.coef_layer, reinterpret_cast<f32x4*>(a.grad_sources), a.grad_stride / 4,
                     a.acc_mask, static_cast<u32x4*>(a.grad_last));
  return hipGetLastError();
}

template <bool kBf16>
hipError_t launch_block(const BlockBackwardArgs& a, hipStream_t stream) {
  hipError_t e;
  switch (a.vecs_per_lane) {
    case 1: e = launch_block_v<kBf16, 1>(a, stream); break;
    case 2: e = launch_block_v<kBf16, 2>(a, stream); break;
    case 3: e = launch_block_v<kBf16, 3>(a, stream); break;
    case 4: e = launch_block_v<kBf16, 4>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // the deferred sources' share of dL/dw, then its fixed-order sum into each layer's row
  const dim3 grid((unsigned)(a.dw_groups * a.dw_colblocks)), block(64 * kDwWaves);
  switch (a.n) {
#define ATTNRES_DW_CASE(N)                                                                                      \
  case N:                                                                                                       \
    hipLaunchKernelGGL((block_dw_kernel<kBf16, N>), grid, block, 0, stream, a.sources, a.T, a.d, a.src_stride, \
                       a.B, a.coef, a.coef_layer, a.workspace, a.dw_colblocks);                                \
    break;
    ATTNRES_DW_CASE(1) ATTNRES_DW_CASE(2) ATTNRES_DW_CASE(3) ATTNRES_DW_CASE(4)
    ATTNRES_DW_CASE(5) ATTNRES_DW_CASE(6) ATTNRES_DW_CASE(7) ATTNRES_DW_CASE(8)
#undef ATTNRES_DW_CASE
    default: return hipErrorInvalidValue;
  }
  static_assert(kMaxInterSources == 8, "one instance per source count");
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)((a.d + 31) / 32), (unsigned)a.B), dim3(256), 0, stream,
                     a.workspace, a.dw_groups, (int64_t)a.B * a.d, (int64_t)a.d, a.d, a.grad_w, true);
  return hipGetLastError();
}

static_assert(kDwWaves * kDwCols == kBlockDwCols, "columns per dL/dw workgroup");

}  // namespace

hipError_t launch_aggregate_backward(const BackwardArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_bwd<true>(a, stream) : launch_bwd<false>(a, stream);
}

// ---- static scratch for callers that cannot allocate -----------------------
//
// attnres_aggregate_backward_static keeps its per-workgroup dL/dw rows here
// instead of in a caller's workspace: 16 MiB, held on every GPU the library
// runs on until the process ends.  Every workgroup writes its whole row before
// the fixed-order sum reads it, so nothing needs clearing between calls; calls
// that overlap in time on one GPU race for it.  Host code never passes the
// array's name to a kernel -- in host code it is a stand-in, not a device
// address -- only the address resolved below.
namespace {
__device__ __align__(256) static float scratch[kStaticScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> hold(g_scratch_lock);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current: this GPU's copy
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

hipError_t launch_block_backward(const BlockBackwardArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  return a.bf16 ? launch_block<true>(a, stream) : launch_block<false>(a, stream);
}

hipError_t launch_partial_dw(const PartialDwArgs& a, hipStream_t stream) {
  // T = 0: no groups, and the sum of no rows writes zeros
  if (a.T > 0) {
    const int nvec = a.d / (a.bf16 ? 8 : 4);
    const dim3 grid((unsigned)(a.colblocks * a.groups), (unsigned)a.B);
    if (a.bf16)
      hipLaunchKernelGGL((partial_dw_kernel<true>), grid, dim3(kPartialDwThreads), 0, stream, a.rows,
                         a.coef_stride, a.T, nvec, a.colblocks, a.B, a.workspace);
    else
      hipLaunchKernelGGL((partial_dw_kernel<false>), grid, dim3(kPartialDwThreads), 0, stream, a.rows,
                         a.coef_stride, a.T, nvec, a.colblocks, a.B, a.workspace);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)((a.d + 31) / 32), (unsigned)a.B), dim3(256), 0, stream,
                     a.workspace, a.groups, (int64_t)a.B * a.d, (int64_t)a.d, a.d, a.out, false);
  return hipGetLastError();
}

hipError_t launch_partial_sums(const PartialSumsArgs& a, hipStream_t stream) {
  const int64_t nvec = a.elems / (a.bf16 ? 8 : 4);
  if (nvec == 0) return hipSuccess;
  // one trip per workgroup up to the largest grid a launch takes: a grid that
  // loops its workgroups over the rows queues each trip's loads behind the
  // previous trip's stores (8 workgroups per CU measured 14% slower for 11
  // rows of T = 32,768, d = 7168: 2.148 against 1.838 ms)
  int64_t grid = (nvec + 255) / 256;
  const int64_t cap = INT64_C(0x7fffffff);
  if (grid > cap) grid = cap;
  if (a.bf16)
    hipLaunchKernelGGL((partial_sums_kernel<true>), dim3((unsigned)grid), dim3(256), 0, stream, a.rows, a.count,
                       nvec, static_cast<u32x4*>(a.out), a.out_stride / 8);
  else
    hipLaunchKernelGGL((partial_sums_kernel<false>), dim3((unsigned)grid), dim3(256), 0, stream, a.rows, a.count,
                       nvec, static_cast<u32x4*>(a.out), a.out_stride / 4);
  return hipGetLastError();
}

}  // namespace attnres
