// Two-phase inference schedule of Block AttnRes (kimi.papertok.ai ch. 4 §4.4
// third benefit and §4.6 inference): within block n the inter-block sources
// h_0, b_1 .. b_{n-1} do not change, so one batched pass reads each of them
// once for all the block's layer queries; each layer then folds its growing
// partial sum in with an online-softmax merge.
//
// Phase 1, interblock_kernel (one launch per block, one workgroup per token;
// batches past the grid cap take several launches).  Per token: load the K
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

#include <utility>

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
// The inter-block pass holds kK rows of kV vectors per lane.  At kV = 2 both
// instances run at 4 waves per SIMD (two 7-wave workgroups per CU) and fit in
// 128 VGPRs without spilling (the 8-row one only as a straight-line one-token
// body, see interblock_kernel).  Wider rows (kV >= 3) get 2 waves per SIMD.
template <int kV, int kK>
constexpr int waves_per_simd_prepare() {
  return kV <= 2 ? 4 : 2;
}

// Byte selectors of v_perm_b32 (result byte i <- selector byte i; 0-3 pick the
// second operand's bytes, 4-7 the first's): (a.lo, b.lo) and (a.hi, b.hi).
constexpr unsigned kSelLo = 0x05040100u, kSelHi = 0x07060302u;


// Calls f(std::integral_constant<int, i>) for i = 0 .. kN-1 (compile-time i).
template <int kN, typename F, int... kIs>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, kIs...>) {
  (f(std::integral_constant<int, kIs>{}), ...);
}
template <int kN, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<kN>(f, std::make_integer_sequence<int, kN>{});
}

// Query chunks come through a raw buffer resource over the prepared queries
// ([G][hi, lo][chunk][4][8] bf16, see split_queries_kernel): lane n of a quad
// reads query 4 qg + n, so a quad's four loads are one 64-byte segment.  A
// read past the end returns zeros (the next group after the last one); a
// chunk past d reads some other chunk that only meets zero source chunks.  The
// loads are unconditional: a load behind a branch would make the compiler wait
// for every outstanding load at the join, which defeats the prefetch ring.

struct QueryRows {
  __amdgpu_buffer_rsrc_t rsrc;
  int plane_bytes;  // one hi or lo plane of a group: nvec * 64
  int lane_bytes;   // chunk cbase, query n of the group
};

__device__ __forceinline__ QueryRows query_rows(const u32x4* w_split, int B, int nvec, int cbase, int n) {
  QueryRows q;
  const int groups = (B + 3) >> 2;
  q.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(w_split), (short)0, groups * 2 * nvec * 64,
                                             kBufferConfig);
  q.plane_bytes = nvec * 64;
  q.lane_bytes = cbase * 64 + n * 16;
  return q;
}

// Chunk c(i) = cbase + 64 (i / 4) + i % 4 of group qg's hi and lo planes.
template <int kI>
__device__ __forceinline__ void load_query_chunk(u32x4& hi, u32x4& lo, const QueryRows& q, int qg) {
  const int off = 2 * qg * q.plane_bytes + q.lane_bytes + 4096 * (kI >> 2) + 64 * (kI & 3);
  hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q.rsrc, off, 0, 0));
  lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q.rsrc, off + q.plane_bytes, 0, 0));
}

// Quad layout of a token's inter-block rows.  Four consecutive lanes form a
// quad; quad j of wave w owns the 4 kV row chunks (16 bytes = 8 elements each)
//     c(4 k + r) = cbase + 64 k + r,   cbase = 64 kV w + 4 j,   k < kV, r < 4.
// The rows are read with lane r of the quad at chunks c(4 k + r) of every
// source (consecutive lanes, consecutive chunks) and moved through a per-wave
// LDS stage so that lane n holds sources n and n + 4 at all the quad's chunks.
// The four lanes of a quad then see the same positions for four different
// sources: the B operand of v_mfma_f32_4x4x4_16b_bf16 for the products
// w_b . x_s, with four queries b (lane n holding query 4 qg + n) as the A
// operand.  For the weighted sums the rows go back the same way, and the result
// rows leave as whole 64-byte segments.
template <int kV, int kClose, int kK>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(waves_per_simd_prepare<kV, kK>())))
interblock_kernel(u32x4* __restrict__ src, int K, int B, int64_t T, int64_t t0, int nvec, int64_t src_stride_v,
                  const u32x4* __restrict__ w_split, u32x4* __restrict__ inter, int64_t inter_stride_v,
                  float* __restrict__ logits, float* __restrict__ weights0, float eps, float inv_d,
                  const u32x4* __restrict__ layer_out) {
  constexpr int kG = kK / 4;          // source groups held per lane
  constexpr int kC = 4 * kV;          // chunks per quad
  // query-chunk ring: 4 slots (3 chunks ahead of use)
  constexpr int kRing = 4;
  static_assert(kC % kRing == 0, "ring slots must divide the chunks");
  constexpr int kParts = 4 * kMaxWaves;
  // partial sums: one per 16-lane row of every wave, summed in a fixed order
  __shared__ float red_ss[kMaxInter][kParts];
  __shared__ float red_dt[kMaxQueries][kMaxInter][kParts];
  __shared__ u32x4 stage[kMaxWaves][16][4][4];  // per wave: [quad][to lane][from lane]
  // per wave: every query's weights as bf16 pairs (sources 2p, 2p+1), hi and lo
  __shared__ unsigned a_pairs[kMaxWaves][2][kMaxQueries][kPairs];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int n = lane & 3;                    // lane in the quad
  const int j = lane >> 2;                   // quad in the wave
  const int cbase = 64 * kV * wave + 4 * j;  // c(i) = cbase + 64 (i / 4) + i % 4
  const bool writer = (lane & 12) == 0;      // one lane per (row, n) after the row sums
  const int part = 4 * wave + (lane >> 4);

  // One token per workgroup, t0 + blockIdx.x; the host splits larger batches
  // over several launches.
  auto token = [&](const int64_t t) {
    u32x4* tok = src + t * (int64_t)nvec;
    const u32x4* lo_tok = layer_out + t * (int64_t)nvec;

    // 1. the K inter-block rows, every source at this lane's chunks
    //    c(4 k + n) = cbase + 64 k + n (consecutive lanes read consecutive
    //    chunks); the last one is formed here when closing: the layer output
    //    alone, or added into the open partial, and written back
    u32x4 x[kG][kC];
    {
      u32x4 xr[kK][kV];
#pragma unroll
      for (int sr = 0; sr < kK; ++sr)
#pragma unroll
        for (int k = 0; k < kV; ++k) {
          const int c = cbase + 64 * k + n;
          xr[sr][k] = u32x4{0, 0, 0, 0};
          if (sr < K && c < nvec) {
            if (kClose == kCloseCopy && sr == K - 1) {
              xr[sr][k] = __builtin_nontemporal_load(lo_tok + c);
            } else {
              xr[sr][k] = __builtin_nontemporal_load(tok + sr * src_stride_v + c);
            }
          }
        }
      if constexpr (kClose != kNoClose) {
#pragma unroll
        for (int sr = 0; sr < kK; ++sr) {
          if (sr == K - 1) {
#pragma unroll
            for (int k = 0; k < kV; ++k) {
              const int c = cbase + 64 * k + n;
              if (c < nvec) {
                if constexpr (kClose == kCloseAdd)
                  xr[sr][k] = add_rows(xr[sr][k], __builtin_nontemporal_load(lo_tok + c), true);
                __builtin_nontemporal_store(xr[sr][k], tok + sr * src_stride_v + c);
              }
            }
          }
        }
      }
      // to quad layout through the wave's LDS stage: lane n of the quad takes
      // source 4 g + n at the quad's chunks c(4 k + r), r = 0..3
#pragma unroll
      for (int g = 0; g < kG; ++g)
#pragma unroll
        for (int k = 0; k < kV; ++k) {
#pragma unroll
          for (int to = 0; to < 4; ++to) stage[wave][j][to][n] = xr[4 * g + to][k];
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int from = 0; from < 4; ++from) x[g][4 * k + from] = stage[wave][j][n][from];
          __builtin_amdgcn_wave_barrier();
        }
    }

    // 2. sums of squares of this lane's sources; rows of 16 lanes reduced by
    //    rotations (lanes 4 and 8 apart hold the same source)
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < kC; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) ss = dot2(x[g][i][k], x[g][i][k], ss);
      ss += dpp<kDppRor4>(ss, ss);
      ss += dpp<kDppRor8>(ss, ss);
      if (writer) red_ss[4 * g + n][part] = ss;
    }

    // 3. w_b . x_s on the matrix cores, four queries at a time; each query
    //    enters as its bf16 hi and lo rows.  Query chunks stream through kRing
    //    register slots, kRing - 1 chunks ahead of use (into the next query
    //    group at the end of one), so that the L2 latency stays hidden.
    u32x4 qh[kRing], ql[kRing];
    const QueryRows qrows = query_rows(w_split, B, nvec, cbase, n);
    static_for<kRing - 1>([&](auto r) { load_query_chunk<r>(qh[r], ql[r], qrows, 0); });
    for (int qg = 0; 4 * qg < B; ++qg) {
      f32x4 acc[kG];
#pragma unroll
      for (int g = 0; g < kG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      static_for<kC>([&](auto ic) {
        constexpr int i = ic;
        // chunk i + kRing - 1 of this group, or of the next, into the slot
        // that chunk i - 1 has just freed
        constexpr int ahead = i + kRing - 1, slot = ahead % kRing;
        if constexpr (ahead < kC)
          load_query_chunk<ahead>(qh[slot], ql[slot], qrows, qg);
        else
          load_query_chunk<ahead - kC>(qh[slot], ql[slot], qrows, qg + 1);
        const u32x4 hq = qh[i % kRing], lq = ql[i % kRing];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const short4v ah = __builtin_bit_cast(short4v, u32x2{hq[2 * h], hq[2 * h + 1]});
          const short4v al = __builtin_bit_cast(short4v, u32x2{lq[2 * h], lq[2 * h + 1]});
#pragma unroll
          for (int g = 0; g < kG; ++g) {
            const short4v bx = __builtin_bit_cast(short4v, u32x2{x[g][i][2 * h], x[g][i][2 * h + 1]});
            acc[g] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ah, bx, acc[g], 0, 0, 0);
            acc[g] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(al, bx, acc[g], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep later loads from hoisting further
      });
      // lane (j, n), register m: query 4 qg + m against source 4 g + n
#pragma unroll
      for (int g = 0; g < kG; ++g)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float v = acc[g][m];
          v += dpp<kDppRor4>(v, v);
          v += dpp<kDppRor8>(v, v);
          if (writer) red_dt[4 * qg + m][4 * g + n][part] = v;
        }
    }
    __syncthreads();

    // 4. softmax per query: lane L handles query 8r + L/8, source L%8, r = 0, 1
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int bq = 8 * r + (lane >> 3);
      const int s = lane & 7;
      const bool valid = bq < B && s < K;
      float z = -INFINITY;
      if (valid) {
        float ss = 0.f, dt = 0.f;
        for (int p = 0; p < 4 * nwaves; p += 4) {
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(&red_ss[s][p]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&red_dt[bq][s][p]);
          ss += (a4[0] + a4[1]) + (a4[2] + a4[3]);
          dt += (d4[0] + d4[1]) + (d4[2] + d4[3]);
        }
        z = dt / sqrtf(ss * inv_d + eps);
      }
      const float m = group_max8(z);
      const float pexp = valid ? expf(z - m) : 0.f;
      const float l = group_sum8(pexp);
      const float a = valid ? pexp / l : 0.f;
      if (valid && wave == 0) {
        logits[((int64_t)bq * T + t) * K + s] = z;
        if (bq == 0 && weights0 != nullptr) weights0[t * K + s] = a;
      }
      // lanes with an even source pack (a_s, a_s+1) as bf16 hi and lo words
      const float a_next = dpp<kDppXor1>(a, a);
      if ((s & 1) == 0 && bq < kMaxQueries) {
        const __bf16 h0 = (__bf16)a, h1 = (__bf16)a_next;
        a_pairs[wave][0][bq][s >> 1] = __builtin_bit_cast(unsigned, bf16x2{h0, h1});
        a_pairs[wave][1][bq][s >> 1] = pack_bf16(a - (float)h0, a_next - (float)h1);
      }
    }

    // 5. quad layout -> every source at this lane's own chunks c(4 k + n),
    //    one (group, k) at a time through the wave's LDS stage; a wave's LDS
    //    operations complete in order, the wave barriers keep the compiler's
    //    order
    u32x4 xn[kK][kV];
#pragma unroll
    for (int g = 0; g < kG; ++g)
#pragma unroll
      for (int k = 0; k < kV; ++k) {
#pragma unroll
        for (int to = 0; to < 4; ++to) stage[wave][j][to][n] = x[g][4 * k + to];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int from = 0; from < 4; ++from) xn[4 * g + from][k] = stage[wave][j][n][from];
        __builtin_amdgcn_wave_barrier();
      }

    // 6. R_b = sum_s a_b,s H_s for every query on the matrix cores: in a quad,
    //    lane (base+m) gives row m of A (query q0+m's weights for 4 sources),
    //    lane (base+n) gives column n of B (its own element of those 4
    //    sources, i.e. two source-pair words) and gets D[m][n] = R_q0+m at its
    //    element.  Weights enter as bf16 hi + lo (two products per source).
    const int nsg = (K + 3) >> 2;  // source groups of 4
    for (int q0 = 0; q0 < B; q0 += 4) {
      // empty register barriers: the compiler must treat the rows as changed
      // here, so the pair-form perms below are not hoisted out of the loop
      // (that would keep a second copy of the rows live)
#pragma unroll
      for (int s = 0; s < kK; ++s)
#pragma unroll
        for (int e = 0; e < kV; ++e)
#pragma unroll
          for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(xn[s][e][k]));
      short4v ahi[kG], alo[kG];
#pragma unroll
      for (int sg = 0; sg < kG; ++sg) {
        const int qq = min(q0 + n, kMaxQueries - 1);
        ahi[sg] = __builtin_bit_cast(short4v, *reinterpret_cast<const u32x2*>(&a_pairs[wave][0][qq][2 * sg]));
        alo[sg] = __builtin_bit_cast(short4v, *reinterpret_cast<const u32x2*>(&a_pairs[wave][1][qq][2 * sg]));
      }
#pragma unroll
      for (int e = 0; e < kV; ++e) {
        const int c = cbase + 64 * e + n;
        // the chunk's 8 elements in two halves of 4; half 0's results wait as
        // packed bf16 words so that every query row goes out as one 16-byte
        // store (two 8-byte halves of a line written apart cost far more)
        u32x2 first[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 acc[4];
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) acc[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int sg = 0; sg < kG; ++sg) {
            if (sg < nsg) {
#pragma unroll
              for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ee = 0; ee < 2; ++ee) {
                  // B operand: (H_4sg[q], H_4sg+1[q]) and (H_4sg+2[q], H_4sg+3[q])
                  // for the even (ee = 0) or odd element q of word k, formed
                  // here so that no second copy of the rows stays live
                  const int k = 2 * h + kk;
                  const unsigned sel = ee ? kSelHi : kSelLo;
                  const u32x2 bw = {__builtin_amdgcn_perm(xn[4 * sg + 1][e][k], xn[4 * sg][e][k], sel),
                                    __builtin_amdgcn_perm(xn[4 * sg + 3][e][k], xn[4 * sg + 2][e][k], sel)};
                  const short4v bop = __builtin_bit_cast(short4v, bw);
                  acc[2 * kk + ee] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi[sg], bop, acc[2 * kk + ee], 0, 0, 0);
                  acc[2 * kk + ee] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo[sg], bop, acc[2 * kk + ee], 0, 0, 0);
                }
            }
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x2 o = {pack_bf16(acc[0][m], acc[1][m]), pack_bf16(acc[2][m], acc[3][m])};
            if (h == 0) {
              first[m] = o;
            } else {
              // through a buffer resource over query row q0 + m of this token
              // (empty past B; stores past the row end are dropped): the
              // address is a wave-uniform base and the lane's 32-bit offset,
              // so no 64-bit per-lane pointer is carried from token to token
              const u32x4 rowv = {first[m][0], first[m][1], o[0], o[1]};
              const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                  inter + (int64_t)(q0 + m) * inter_stride_v + t * (int64_t)nvec, (short)0,
                  q0 + m < B ? nvec * 16 : 0, kBufferConfig);
              store_nt(rowv, r, c * 16);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // one chunk's accumulators live at a time
      }
    }
  };
  if constexpr (kK > 4) {
    // straight-line: nothing is kept live from token to token, and the 8-row
    // instance fits in its registers without spilling
    const int64_t t = t0 + blockIdx.x;
    if (t < T) token(t);
  } else {
    // the same single trip as a loop the compiler cannot see through: it
    // schedules the 4-row body with more registers, measured 6% faster
    const int64_t t_end = t0 + (int64_t)gridDim.x < T ? t0 + (int64_t)gridDim.x : T;
    for (int64_t t = t0 + blockIdx.x; t < t_end; t += gridDim.x) token(t);
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

// The merge for small batches: one memory round trip per token (see
// merge_per_token in the launch policy for when each form is used).
template <int kV, bool kAdd>
__global__ void __launch_bounds__(64 * kMaxWaves) __attribute__((amdgpu_waves_per_eu(waves_per_simd2<kV>())))
merge_token_kernel(u32x4* __restrict__ slot, const u32x4* __restrict__ layer_out, const u32x4* inter,
             const float* __restrict__ logits, int K, int64_t T, int64_t t0, int nvec, const float* __restrict__ w,
             u32x4* out, float* __restrict__ weights, float eps, float inv_d) {
  __shared__ float red[kMaxWaves][2];

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  const int s16 = lane & 15;

  // one token per workgroup, t0 + blockIdx.x (the host splits larger batches
  // over several launches); every load of the token -- the query, the three
  // rows and the logits -- is issued before anything waits, each row through
  // a buffer resource of its own so that no load sits behind a branch.  The
  // arithmetic is merge_kernel's, in the same order: results are bit-identical.
  const int64_t t = t0 + blockIdx.x;
  if (t >= T) return;
  QueryLoads<true, kV> ql;
  issue_query<true, kV>(ql, w, nvec, tid, nthr);
  const int64_t rowoff = t * (int64_t)nvec;
  const int off = tid * kVecBytes;  // vector v at off + v * nthr * 16
  const int row_bytes = nvec * kVecBytes;
  auto rsrc = [&](const u32x4* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4*>(p + rowoff), (short)0, row_bytes, kBufferConfig);
  };
  const __amdgpu_buffer_rsrc_t r_inter = rsrc(inter), r_lo = rsrc(layer_out), r_slot = rsrc(slot);
  u32x4 R[kV], f[kV], xp[kV];
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    R[v] = load_nt(r_inter, off + v * nthr * kVecBytes);
    f[v] = load_nt(r_lo, off + v * nthr * kVecBytes);
    if constexpr (kAdd) xp[v] = load_nt(r_slot, off + v * nthr * kVecBytes);
  }
  const __amdgpu_buffer_rsrc_t r_logits =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(logits + t * K), (short)0, K * 4, kBufferConfig);
  const float zl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_logits, s16 * 4, 0, 0));
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    xp[v] = kAdd ? add_rows(xp[v], f[v], true) : f[v];
    store_nt(xp[v], r_slot, off + v * nthr * kVecBytes);
  }
  const float zi = (s16 < K) ? zl : -INFINITY;

  Query<true, kV> q;
  finish_query<true, kV>(q, ql);
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
    red[wave][0] = ss;
    red[wave][1] = dt;
  }
  __syncthreads();
  float ssp = 0.f, dtp = 0.f;
  for (int k = 0; k < nwaves; ++k) {
    ssp += red[k][0];
    dtp += red[k][1];
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
  const __amdgpu_buffer_rsrc_t r_out = rsrc(out);
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[k] = pack_bf16(fmaf(cp, bf16_lo(xp[v][k]), ca * bf16_lo(R[v][k])),
                       fmaf(cp, bf16_hi(xp[v][k]), ca * bf16_hi(R[v][k])));
    }
    store_nt(o, r_out, off + v * nthr * kVecBytes);
  }
}

// Prepared queries: groups of 4 queries, [G][plane: hi, lo][chunk][4][8] bf16,
// G = ceil(n / 4), queries past n zero.  One thread per (query, chunk).
__global__ void __launch_bounds__(256) split_queries_kernel(const float* __restrict__ w, int n, int nvec,
                                                            u32x4* __restrict__ out) {
  const int64_t groups = (n + 3) / 4;
  const int64_t total = groups * 4 * nvec;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t gq = i / nvec;  // global query slot 4 g + m
    const int c = (int)(i - gq * nvec);
    const int64_t g = gq >> 2;
    const int m = (int)(gq & 3);
    u32x4 hi = u32x4{0, 0, 0, 0}, lo = u32x4{0, 0, 0, 0};
    if (gq < n) {
      const f32x4* src = reinterpret_cast<const f32x4*>(w + gq * (int64_t)nvec * 8 + 8 * (int64_t)c);
      const f32x4 a = src[0], b = src[1];
      const float e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const __bf16 h0 = (__bf16)e[2 * k], h1 = (__bf16)e[2 * k + 1];
        hi[k] = __builtin_bit_cast(unsigned, bf16x2{h0, h1});
        lo[k] = pack_bf16(e[2 * k] - (float)h0, e[2 * k + 1] - (float)h1);
      }
    }
    out[((g * 2 + 0) * nvec + c) * 4 + m] = hi;
    out[((g * 2 + 1) * nvec + c) * 4 + m] = lo;
  }
}

template <int kV, int kClose, int kK>
hipError_t launch_prepare(const PrepareArgs& a, hipStream_t stream) {
  const int nvec = a.d / 8;
  if (a.grid <= 0) return hipErrorInvalidValue;
  // one workgroup per token, at most a.grid tokens per launch
  for (int64_t t0 = 0; t0 < a.T; t0 += a.grid) {
    const int64_t n = a.T - t0 < a.grid ? a.T - t0 : a.grid;
    hipLaunchKernelGGL((interblock_kernel<kV, kClose, kK>), dim3((unsigned)n), dim3(a.threads), 0, stream,
                       static_cast<u32x4*>(a.store), a.K, a.B, a.T, t0, nvec, a.slot_stride / 8,
                       static_cast<const u32x4*>(a.w_split),
                       static_cast<u32x4*>(a.inter), a.inter_stride / 8, a.logits, a.weights0, a.eps,
                       1.0f / (float)a.d, static_cast<const u32x4*>(a.layer_out));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int kV, bool kAdd>
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int nvec = a.d / 8;
  if (a.grid <= 0) return hipErrorInvalidValue;
  if (a.per_token) {
    // one workgroup per token, at most a.grid tokens per launch
    for (int64_t t0 = 0; t0 < a.T; t0 += a.grid) {
      const int64_t n = a.T - t0 < a.grid ? a.T - t0 : a.grid;
      hipLaunchKernelGGL((merge_token_kernel<kV, kAdd>), dim3((unsigned)n), dim3(a.threads), 0, stream,
                         static_cast<u32x4*>(a.slot), static_cast<const u32x4*>(a.layer_out),
                         static_cast<const u32x4*>(a.inter), a.logits, a.K, a.T, t0, nvec, a.w,
                         static_cast<u32x4*>(a.out), a.weights, a.eps, 1.0f / (float)a.d);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
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
  const int nvec = d / 8;
  int64_t grid = (((n + 3) / 4) * 4 * nvec + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(split_queries_kernel, dim3((unsigned)grid), dim3(256), 0, stream, w, (int)n, nvec,
                     static_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t launch_block_merge(const MergeArgs& a, hipStream_t stream) {
  return a.add ? merge_v<true>(a, stream) : merge_v<false>(a, stream);
}

}  // namespace attnres
