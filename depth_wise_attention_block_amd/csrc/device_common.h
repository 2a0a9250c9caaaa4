// Device helpers shared by the aggregation and accumulation kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace attnres {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two bf16 lanes of a 32-bit word: element 2i in the low half, 2i+1 in the high.
__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xFFFF0000u); }

// float32 pair -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, p);
}

// Partial-sum update of one 16-byte vector: per element one float32 addition,
// then (bf16) one rounding to nearest even.
__device__ __forceinline__ u32x4 add_rows(u32x4 p, u32x4 f, bool bf16) {
  u32x4 r;
  if (bf16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = pack_bf16(bf16_lo(p[k]) + bf16_lo(f[k]), bf16_hi(p[k]) + bf16_hi(f[k]));
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = __float_as_uint(__uint_as_float(p[k]) + __uint_as_float(f[k]));
  }
  return r;
}

// Token of virtual workgroup index b when each of the 8 XCDs (workgroup b runs
// on XCD b % 8) takes runs of 2^run_log2 consecutive tokens in turn.  A
// bijection of [0, T rounded up to 8 * 2^run_log2); run_log2 = 0 is b itself.
__device__ __forceinline__ int64_t xcd_token(int64_t b, int run_log2) {
  const int64_t x = b & 7, k = b >> 3;
  return ((((k >> run_log2) << 3) | x) << run_log2) | (k & ((INT64_C(1) << run_log2) - 1));
}

// Word 3 of a raw buffer resource on gfx9 (data format 32 bits; offsets at or
// past the resource's size read zeros and drop stores).
constexpr int kBufferConfig = 0x00020000;
constexpr int kCachePolicyNt = 2;  // buffer load / store cache policy: non-temporal

// 16-byte non-temporal load / store at byte offset off of a buffer resource.
__device__ __forceinline__ u32x4 load_nt(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyNt));
}
__device__ __forceinline__ void store_nt(u32x4 v, __amdgpu_buffer_rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCachePolicyNt);
}

// ---- DPP helpers (GFX9 data-parallel primitives inside one wave) -----------
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <- 7-i in 8
constexpr int kDppMirror = 0x140;     // row_mirror: lane i <- 15-i in 16
constexpr int kDppBcast15 = 0x142;    // row_bcast:15 -> next row
constexpr int kDppBcast31 = 0x143;    // row_bcast:31 -> rows 2,3
constexpr int kDppRor4 = 0x124;       // row_ror:4: rotate each 16-lane row by 4
constexpr int kDppRor8 = 0x128;       // row_ror:8: rotate each 16-lane row by 8

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp(float old, float src) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, src),
                                         kCtrl, kRowMask, 0xF, false));
}

// Every lane of each 16-lane row ends with that row's sum (bitwise equal
// across the row: each step adds the same two operands in either order).
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kDppXor1>(v, v);
  v += dpp<kDppXor2>(v, v);
  v += dpp<kDppHalfMirror>(v, v);
  v += dpp<kDppMirror>(v, v);
  return v;
}

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v, v));
  v = fmaxf(v, dpp<kDppXor2>(v, v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v, v));
  v = fmaxf(v, dpp<kDppMirror>(v, v));
  return v;
}

// Every lane of each 8-lane group ends with that group's sum / maximum.
__device__ __forceinline__ float group_sum8(float v) {
  v += dpp<kDppXor1>(v, v);
  v += dpp<kDppXor2>(v, v);
  v += dpp<kDppHalfMirror>(v, v);
  return v;
}

__device__ __forceinline__ float group_max8(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v, v));
  v = fmaxf(v, dpp<kDppXor2>(v, v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v, v));
  return v;
}

// Sum over all 64 lanes, returned wave-uniform.  Fixed order: rows, then
// row 0 + row 1 and row 2 + row 3, then the two halves.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += dpp<kDppBcast15, 0xA>(0.0f, v);  // rows 1,3 += lane 15 of the row below
  v += dpp<kDppBcast31, 0xC>(0.0f, v);  // rows 2,3 += lane 31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// One step of wave_sums: lane pairs (partner by kCtrl, differing in lane bit
// `bit`) halve the values each holds: a lane keeps the entries whose index has
// its own bit and adds the partner's copies of them.
template <int kCtrl, int M>
__device__ __forceinline__ void halve_values(const float (&cur)[2 * M], float (&nxt)[M], bool bit) {
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const float keep = bit ? cur[2 * j + 1] : cur[2 * j];
    const float send = bit ? cur[2 * j] : cur[2 * j + 1];
    nxt[j] = keep + dpp<kCtrl>(send, send);
  }
}

// Sums over each 16-lane row of N = 4, 8 or 16 values at once: lane L ends
// with its row's sum of v[L % N].  Exchanges across lane bits 0, 1 (quad
// permutes) and 2, 3 (rotations of the row) halve the values a lane holds, and
// plain sums cover the row's remaining bits: about 1.5 N operations where N
// separate row sums take 4 N.  The four rows of a wave are left apart (a
// caller combines them through LDS).  Fixed order, so deterministic.
template <int N>
__device__ __forceinline__ float row_sums(const float (&v)[N], int lane) {
  static_assert(N == 4 || N == 8 || N == 16, "4, 8 or 16 values");
  if constexpr (N == 16) {
    float a[8], b[4], c[2], e[1];
    halve_values<kDppXor1, 8>(v, a, lane & 1);
    halve_values<kDppXor2, 4>(a, b, lane & 2);
    halve_values<kDppRor4, 2>(b, c, lane & 4);
    halve_values<kDppRor8, 1>(c, e, lane & 8);
    return e[0];
  } else if constexpr (N == 8) {
    float a[4], b[2], c[1];
    halve_values<kDppXor1, 4>(v, a, lane & 1);
    halve_values<kDppXor2, 2>(a, b, lane & 2);
    halve_values<kDppRor4, 1>(b, c, lane & 4);
    return c[0] + dpp<kDppRor8>(c[0], c[0]);
  } else {
    float a[2], b[1];
    halve_values<kDppXor1, 2>(v, a, lane & 1);
    halve_values<kDppXor2, 1>(a, b, lane & 2);
    const float x = b[0] + dpp<kDppRor4>(b[0], b[0]);
    return x + dpp<kDppRor8>(x, x);
  }
}

__device__ __forceinline__ float lane_bcast(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Lane `lane` of every 16-lane row takes v; the other lanes keep old.
__device__ __forceinline__ float put_lane(float v, int lane, float old, int s16) {
  return s16 == lane ? v : old;
}

// ---- bf16 pair helpers -------------------------------------------------------
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned u) { return __builtin_bit_cast(bf16x2, u); }
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// Per-lane slice of the pseudo-query.  bf16 sources: w = hi + lo, both bf16
// pairs laid out like the source words (element 2i in the low half), so that
// w.x = dot2(x, hi) + dot2(x, lo) keeps ~16 significant bits of w.
template <bool kBf16, int kV>
struct Query {
  u32x4 hi[kV], lo[kV];  // bf16 path
  f32x4 f[kV];           // f32 path
};

template <bool kBf16, int kV>
__device__ __forceinline__ void load_query(Query<kBf16, kV>& q, const float* __restrict__ w, int nvec,
                                           int tid, int nthr) {
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    const int idx = v * nthr + tid;
    if constexpr (kBf16) {
      q.hi[v] = u32x4{0, 0, 0, 0};
      q.lo[v] = u32x4{0, 0, 0, 0};
      if (idx < nvec) {
        const f32x4* wp = reinterpret_cast<const f32x4*>(w) + 2 * (int64_t)idx;
        const f32x4 a = wp[0], b = wp[1];
        const float e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const __bf16 h0 = (__bf16)e[2 * k], h1 = (__bf16)e[2 * k + 1];
          const __bf16 l0 = (__bf16)(e[2 * k] - (float)h0), l1 = (__bf16)(e[2 * k + 1] - (float)h1);
          q.hi[v][k] = __builtin_bit_cast(unsigned, bf16x2{h0, h1});
          q.lo[v][k] = __builtin_bit_cast(unsigned, bf16x2{l0, l1});
        }
      }
    } else {
      q.f[v] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (idx < nvec) q.f[v] = reinterpret_cast<const f32x4*>(w)[idx];
    }
  }
}

// The same query in two steps, so that its loads can be in flight together
// with a token's row loads: issue_query starts the float32 loads (through a
// buffer resource over w, so that lanes past the row read zeros without a
// branch -- a load behind a branch makes the compiler wait for it at the
// join), and finish_query converts once they are needed.
template <bool kBf16, int kV>
struct QueryLoads {
  f32x4 raw[kV][kBf16 ? 2 : 1];
};

template <bool kBf16, int kV>
__device__ __forceinline__ void issue_query(QueryLoads<kBf16, kV>& ql, const float* __restrict__ w, int nvec,
                                            int tid, int nthr) {
  constexpr int kParts = kBf16 ? 2 : 1;  // 16-byte float32 loads per vector
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w), (short)0, nvec * 16 * kParts, kBufferConfig);
#pragma unroll
  for (int v = 0; v < kV; ++v)
#pragma unroll
    for (int p = 0; p < kParts; ++p)
      ql.raw[v][p] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ((v * nthr + tid) * kParts + p) * 16, 0, 0));
}

template <bool kBf16, int kV>
__device__ __forceinline__ void finish_query(Query<kBf16, kV>& q, const QueryLoads<kBf16, kV>& ql) {
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    if constexpr (kBf16) {
      const f32x4 a = ql.raw[v][0], b = ql.raw[v][1];
      const float e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const __bf16 h0 = (__bf16)e[2 * k], h1 = (__bf16)e[2 * k + 1];
        const __bf16 l0 = (__bf16)(e[2 * k] - (float)h0), l1 = (__bf16)(e[2 * k + 1] - (float)h1);
        q.hi[v][k] = __builtin_bit_cast(unsigned, bf16x2{h0, h1});
        q.lo[v][k] = __builtin_bit_cast(unsigned, bf16x2{l0, l1});
      }
    } else {
      q.f[v] = ql.raw[v][0];
    }
  }
}

}  // namespace attnres
