/*
 * attnres.h -- C ABI of libattnres.so: Block Attention-Residuals (Block AttnRes)
 * depth aggregation for AMD Instinct MI355X (gfx950).
 *
 * Method (pages cited by title and section):
 *   - "Kimi K3技术详解系列（二）：AttnRes 与 Stable LatentMoE", §2: a layer's
 *     residual is a softmax-weighted sum over depth sources, scored by a learned
 *     per-layer pseudo-query against RMS-normalised sources; §3: Block AttnRes
 *     keeps the embedding, one summary per completed block and the current
 *     block's partial sum.
 *   - kimi.papertok.ai tutorial, ch. 4 "Attention Residuals", §4.2 (eq 8-9:
 *     phi(q,k) = exp(q^T RMSNorm(k)), no temperature), §4.3 (eq 10: block
 *     representations and the partial sum; no partial entry for the first
 *     layer of a block), §4.6 (a block representation is produced once at the
 *     block boundary and then stays resident).
 *   - "Kimi K3 模型结构（6）：输入端与零件", loose model facts: RMSNorm eps 1e-5.
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are device memory on the current HIP device;
 *     the caller allocates and frees all of it.  The library never allocates,
 *     frees or synchronises, and keeps no pointer after a call returns.
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously on it; buffers must stay alive until it ends.
 *   - Return value: ATTNRES_OK or a negative status.  All argument checks run
 *     on the host before anything is enqueued; a failed check enqueues nothing.
 *     The only HIP calls a check may follow are the query of the current device
 *     and of its compute-unit count (cached per device), made by the entry
 *     points whose workspace size depends on them.  Nothing is thrown across
 *     the ABI.
 *   - Once its checks pass, a call reads (and so clears) the calling thread's
 *     HIP last-error state before it launches, so that ATTNRES_ELAUNCH
 *     reports its own launches only: a caller that wants the error of an
 *     earlier launch of its own reads hipGetLastError() before calling here.
 *   - Element layout is row-major; bf16 is IEEE binary32's top 16 bits.
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTNRES_API __attribute__((visibility("default")))

/* Most sources one aggregation takes: embedding + 8 block representations,
 * or embedding + 7 + the partial sum (kimi.papertok.ai ch. 4 §4.5). */
#define ATTNRES_MAX_SOURCES 9
/* Most sources attnres_aggregate takes in one call: Full AttnRes keeps every
 * earlier layer output as a source (kimi.papertok.ai ch. 4 §4.2), up to 94 for
 * K3's 93 layers, or about twice that at sublayer granularity. */
#define ATTNRES_MAX_SOURCES_FULL 256
/* Largest hidden size: 4 vectors of 16 bytes per lane, 512 lanes per token. */
#define ATTNRES_MAX_D_BF16 16384
#define ATTNRES_MAX_D_F32 8192

typedef enum { ATTNRES_BF16 = 0, ATTNRES_F32 = 1 } attnres_dtype;

enum {
  ATTNRES_OK = 0,
  ATTNRES_EINVAL = -1,       /* bad count, size, null pointer or flag        */
  ATTNRES_EUNSUPPORTED = -2, /* misaligned pointer/stride, d not a multiple of
                                the 16-byte vector, d above the maximum, or an
                                unknown dtype                                 */
  ATTNRES_EALIAS = -3,       /* an output overlaps an input                   */
  ATTNRES_ELAUNCH = -4,      /* the HIP runtime refused a launch              */
  ATTNRES_ESTATE = -5        /* source store full or its fields inconsistent  */
};

/* Library version, major*10000 + minor*100 + patch. */
ATTNRES_API int attnres_version(void);

/* Static text for a status code (never NULL). */
ATTNRES_API const char* attnres_strerror(int status);

/*
 * attnres_aggregate -- one depth aggregation for T tokens.
 *
 * For every token t:  k_s = H_s[t] / sqrt(mean_j H_s[t][j]^2 + eps)
 *                     z_s = w . k_s,    a_s = exp(z_s) / sum_s' exp(z_s')
 *                     out[t] = sum_s a_s H_s[t]          (raw sources as values)
 * ("Kimi K3技术详解系列（二）" §2 and its listing; kimi.papertok.ai §4.2 eq 8-9;
 * llm-atlas.k1412.top/k3 card 07.)  Each source row is read from HBM once;
 * sums, softmax and the weighted sum are formed in float32.  Up to 9 sources
 * are held in registers at once and the softmax is exact; beyond 9 (Full
 * AttnRes, kimi.papertok.ai §4.2) the sources are taken in batches of 9 and
 * merged by an online softmax (running max and normaliser, rescaled float32
 * accumulator; §4.4).
 *
 *   sources     device, [S][T][d] of dtype, source-major: source s, token t
 *               starts at element s*src_stride + t*d.  16-byte aligned.
 *   S           number of sources, 1..ATTNRES_MAX_SOURCES_FULL.
 *   T           tokens, >= 0.  T == 0 returns ATTNRES_OK with nothing enqueued.
 *   d           hidden size: a multiple of 8 (bf16) or 4 (f32), at most
 *               ATTNRES_MAX_D_BF16 / ATTNRES_MAX_D_F32.
 *   src_stride  elements between consecutive sources; 0 means T*d.  Must be a
 *               multiple of the 16-byte vector and >= T*d when S > 1.
 *   w           device, [d] float32 pseudo-query of the layer.
 *   out         device, [T][d] of dtype (bf16 rounded to nearest even).
 *   weights     device, [T][S] float32 depth weights, or NULL to skip them.
 *   eps         RMSNorm epsilon (the model uses 1e-5); finite and >= 0.
 *   dtype       ATTNRES_BF16 or ATTNRES_F32 (sources and out).
 *   stream      hipStream_t.
 * out and weights must not overlap sources, w or each other (ATTNRES_EALIAS).
 * Bitwise deterministic for a given device, shape and input.
 */
ATTNRES_API int attnres_aggregate(const void* sources, int32_t S, int64_t T, int32_t d,
                                  int64_t src_stride, const float* w, void* out,
                                  float* weights, float eps, int32_t dtype, void* stream);

/*
 * Source store: host-side bookkeeping for device slots [s_max][T][d].
 * Slot 0 holds the embedding h_0 (written by the caller); slot n holds block
 * representation b_n once block n is complete; slot 1 + n_completed holds the
 * running partial sum of the current block when partial_valid is set
 * ("Kimi K3技术详解系列（二）" §3 diagram order; kimi.papertok.ai §4.3 eq 10).
 * The live sources of the next aggregation are slots
 * [0, 1 + n_completed + partial_valid), contiguous at stride slot_stride.
 */
typedef struct attnres_store {
  void* base;            /* device, slot 0; 16-byte aligned                  */
  int64_t T;             /* tokens per slot                                  */
  int64_t slot_stride;   /* elements between slots, >= T*d                   */
  int32_t d;             /* hidden size                                      */
  int32_t s_max;         /* slots allocated, 2..ATTNRES_MAX_SOURCES          */
  int32_t dtype;         /* attnres_dtype                                    */
  int32_t n_completed;   /* completed block representations b_1..b_n         */
  int32_t partial_valid; /* 1 if slot 1 + n_completed holds a partial sum    */
  int32_t reserved;      /* zero                                             */
} attnres_store_t;

/*
 * attnres_store_init -- fill *st for caller-owned slots (host only, no HIP
 * call).  slot_stride 0 means T*d.  Counters start at zero: only h_0 is live.
 * Same size/alignment rules as attnres_aggregate; ATTNRES_EINVAL for s_max
 * outside 2..ATTNRES_MAX_SOURCES.  base may be NULL only when T = 0: an empty
 * store, whose calls update the counters and launch nothing.
 */
ATTNRES_API int attnres_store_init(attnres_store_t* st, void* base, int32_t s_max, int64_t T,
                                   int32_t d, int64_t slot_stride, int32_t dtype);

/* Number of live sources, 1 + n_completed + partial_valid, or a negative status
 * if *st is inconsistent (host only). */
ATTNRES_API int attnres_store_sources(const attnres_store_t* st);

/*
 * attnres_accumulate -- add one layer's output to the current block's partial
 * sum, and optionally close the block (kimi.papertok.ai §4.3 eq 10 and §4.6;
 * "Kimi K3技术详解系列（二）" §3).
 *
 *   slot = 1 + n_completed
 *   partial_valid ? slot = round(f32(slot) + f32(layer_out))   (one pass, RMW)
 *                 : slot = layer_out                           (first layer: copy)
 *   partial_valid = 1
 *   finalize_block: n_completed += 1, partial_valid = 0  -- the partial slot
 *                   becomes b_n in place; no data moves.
 * bf16: the sum is one float32 add rounded to bf16 (nearest even); f32: one
 * float32 add.  Bit-exact.
 *
 *   st             store (host struct, updated on success only).
 *   layer_out      device, [T][d] of st->dtype, 16-byte aligned; must not
 *                  overlap the store's slots (ATTNRES_EALIAS).
 *   finalize_block 0 or 1.
 * ATTNRES_ESTATE if slot would be >= s_max.  T == 0 updates the bookkeeping
 * and enqueues nothing.
 */
ATTNRES_API int attnres_accumulate(attnres_store_t* st, const void* layer_out,
                                   int32_t finalize_block, void* stream);

/*
 * attnres_accumulate_aggregate -- attnres_accumulate(st, layer_out,
 * finalize_block) followed by attnres_aggregate over the store's live sources
 * with the next layer's query w, in ONE kernel: the updated slot is formed in
 * registers from the old slot row and the layer output, written back, and used
 * as the last source without being read again (kimi.papertok.ai §4.3 eq 10: the
 * next layer sees the partial sum up to the previous layer, or the block
 * representation just closed).  Results (slot contents, out, weights, store
 * bookkeeping) are bit-identical to the two separate calls.
 *
 *   st, layer_out, finalize_block   as for attnres_accumulate.
 *   w, out, weights, eps            as for attnres_aggregate; the sources are
 *                                   slots [0, S) after the update, S =
 *                                   1 + n_completed + partial_valid (new values);
 *                                   weights is [T][S] or NULL.
 * out and weights must not overlap the store, layer_out, w or each other
 * (ATTNRES_EALIAS).  ATTNRES_ESTATE if the store has no slot left.  T == 0
 * updates the bookkeeping and enqueues nothing.  *st changes on success only.
 */
ATTNRES_API int attnres_accumulate_aggregate(attnres_store_t* st, const void* layer_out, int32_t finalize_block,
                                             const float* w, void* out, float* weights, float eps, void* stream);

/*
 * Two-phase schedule (kimi.papertok.ai ch. 4 §4.4, third benefit, and §4.6,
 * inference): inside block n the inter-block sources h_0, b_1 .. b_{n-1} stay
 * fixed, so one batched pass reads them once for all the block's layer
 * queries (attnres_block_prepare), and each later layer merges its partial
 * sum in by online softmax (attnres_block_merge).  bf16 stores only; at most
 * ATTNRES_MAX_INTER_SOURCES inter-block sources and ATTNRES_MAX_BLOCK_QUERIES
 * queries per pass.  Results equal attnres_aggregate over the same sources up
 * to one extra bf16 rounding of the inter-block part (the stored R rows).
 */
#define ATTNRES_MAX_INTER_SOURCES 8
#define ATTNRES_MAX_BLOCK_QUERIES 16

/*
 * attnres_split_queries -- pseudo-queries in the form the two-phase pass reads:
 * each float32 element becomes two bf16 values, hi = bf16(w) and lo =
 * bf16(w - hi) (both rounded to nearest even), so hi + lo keeps about 16
 * significant bits.  The queries are layer parameters, frozen after training
 * (kimi.papertok.ai §4.2), so this runs once, not per token.
 *   w         device, [n][d] float32, 16-byte aligned; d a multiple of 8.
 *   w_split   device, ATTNRES_PREPARED_QUERY_BYTES(n, d) bytes, 16-byte
 *             aligned: queries in groups of four, bf16
 *             [ceil(n/4)][2][d/8][4][8] -- group g, plane (0 hi, 1 lo), 8-element
 *             chunk c, query 4g+m, element 8c+e; queries past n are zero.
 * ATTNRES_EUNSUPPORTED for d % 8 != 0 or misaligned pointers.
 */
#define ATTNRES_PREPARED_QUERY_BYTES(n, d) ((((int64_t)(n) + 3) / 4) * 16 * (int64_t)(d))
ATTNRES_API int attnres_split_queries(const float* w, int32_t n, int32_t d, void* w_split, void* stream);

/*
 * attnres_block_prepare -- phase 1 for one block.
 *
 * If close_block, layer_out (the previous block's last layer output) is first
 * added into the partial slot and the block is closed, exactly as
 * attnres_accumulate(st, layer_out, 1) (copy when no partial is open);
 * otherwise no partial may be open (ATTNRES_ESTATE).  Then with K = 1 +
 * n_completed inter-block sources (slots [0, K)) and the B queries w_b (given
 * split, as attnres_split_queries writes them):
 *   z[b][t][s] = w_b . RMSNorm(H_s[t])          -> logits, float32 [B][T][K]
 *   R_b[t]     = sum_s softmax_s(z[b][t]) H_s[t] -> inter row b, bf16 [T][d]
 *   weights0[t][s] = softmax_s(z[0][t])         (optional, float32 [T][K])
 * R_0 is the residual of the block's first layer.
 *
 *   w_split       device, the B queries as attnres_split_queries prepares them
 *                 (ATTNRES_PREPARED_QUERY_BYTES(B, d) bytes), 16-byte aligned.
 *   B             1..ATTNRES_MAX_BLOCK_QUERIES.
 *   inter         device, B rows of [T][d] bf16, row b at element b*inter_stride
 *                 (0 means T*d); 16-byte aligned.
 *   logits        device, [B][T][K] float32.
 * No output may overlap the store, layer_out, w or another output
 * (ATTNRES_EALIAS).  *st is updated on success only.
 */
ATTNRES_API int attnres_block_prepare(attnres_store_t* st, const void* layer_out, int32_t close_block,
                                      const void* w_split, int32_t B, void* inter, int64_t inter_stride,
                                      float* logits, float* weights0, float eps, void* stream);

/*
 * attnres_block_merge -- phase 2 for one later layer of the block.
 *
 * Adds layer_out (the previous layer's output) into the partial slot (copy if
 * none is open; partial_valid becomes 1), scores the new partial with this
 * layer's query w, and merges it with the inter-block part of prepare's query
 * for this layer (inter row R and its logits [T][K], K = 1 + n_completed):
 *   M = max(max_s z_s, z_p),  A = sum_s e^(z_s - M),  P = e^(z_p - M)
 *   out = (A R + P x_p) / (A + P);  weights[t] = [e^(z_s - M), P] / (A + P)
 *
 *   out       device, [T][d] bf16; may be the inter row itself (in place).
 *   weights   device, [T][K+1] float32 (inter sources, then the partial), or NULL.
 */
ATTNRES_API int attnres_block_merge(attnres_store_t* st, const void* layer_out, const float* w,
                                    const void* inter, const float* logits, void* out, float* weights,
                                    float eps, void* stream);

/*
 * attnres_add_rows -- out = a + b element-wise over [T][d] (bf16: one float32
 * addition, then round to nearest even; f32: one addition), or out = b when a
 * is NULL: the partial-sum update of attnres_accumulate on plain rows, e.g. to
 * recompute a block's partial sums for the backward pass (kimi.papertok.ai
 * §4.6, recomputation).  out may be a (in place) but may not overlap b.
 */
ATTNRES_API int attnres_add_rows(const void* a, const void* b, void* out, int64_t T, int32_t d, int32_t dtype,
                                 void* stream);

/*
 * attnres_partial_sums -- the running partial sums of a block's layer outputs,
 * as the store forms them one update at a time: out[0] = F_0, out[k] =
 * out[k-1] + F_k (bf16: one float32 addition, then round to nearest even), in
 * one pass -- e.g. to recompute a block's partial sums for the backward pass
 * (kimi.papertok.ai §4.6).
 *   layer_outs  HOST array of count (1..16) device pointers, [T][d] in dtype,
 *               16-byte aligned.
 *   out         device, count rows [T][d] in dtype at out_stride elements (0
 *               means T*d); may not overlap the inputs.
 */
ATTNRES_API int attnres_partial_sums(const void* const* layer_outs, int32_t count, int64_t T, int32_t d, void* out,
                                     int64_t out_stride, int32_t dtype, void* stream);

/*
 * attnres_aggregate_backward -- gradients of one aggregation, recomputing its
 * forward (training wraps the aggregation in activation checkpointing,
 * kimi.papertok.ai §4.6).  With g = dL/dr for r = attnres_aggregate(sources, w):
 *   u_s = g . H_s,  delta_s = a_s (u_s - sum_s' a_s' u_s'),
 *   dL/dH_s = a_s g + (delta_s / rho_s) w - (delta_s z_s / (d rho_s^2)) H_s,
 *   dL/dw   = sum over tokens and sources of (delta_s / rho_s) H_s,
 * with rho_s = sqrt(mean(H_s^2) + eps) and z_s, a_s the forward's logits and
 * weights: the value path and the softmax / query / key path of the gradient
 * (llm-atlas.k1412.top/k3, study of the spike trajectory x backward path).
 *
 *   sources, S, T, d, src_stride, w, eps, dtype   as attnres_aggregate, S <= 9.
 *   last_source     device, [T][d] in dtype, or NULL: when given, source S-1 is
 *                   read here instead of at (S-1)*src_stride (a recomputed
 *                   partial sum next to the store's slots); sources may then be
 *                   NULL for S = 1.
 *   grad_out        device, [T][d] in dtype: dL/dr.
 *   grad_sources    device, S rows of [T][d] float32, row s at s*grad_stride
 *                   floats (0 means T*d); 16-byte aligned.  Row s is overwritten
 *                   with dL/dH_s, or, when bit s of accumulate_mask is set, has
 *                   it added (float32).
 *   defer_mask      bit s: leave grad row s alone and write source s's three
 *                   coefficients instead, (a_s, delta_s/rho_s, delta_s z_s/(d rho_s^2))
 *                   as float32 at coef[t*coef_stride + 3s .. 3s+2], for
 *                   attnres_block_backward to apply later (coef_stride >= 3S).
 *   grad_last       device, [T][d] in dtype (round to nearest even for bf16), or
 *                   NULL (required NULL when source S-1 is deferred): receives the
 *                   new value of grad row S-1 -- in a Block
 *                   AttnRes backward that is the finished gradient of the
 *                   previous layer's output.
 *   grad_w          device, [d] float32, overwritten with dL/dw summed over the
 *                   sources not in defer_mask (zero for T = 0); a deferred
 *                   source's share, sum over tokens of (delta_s/rho_s) H_s, is
 *                   added by attnres_block_backward with its gradient row.
 *                   Or NULL: dL/dw is left to the caller -- the three
 *                   coefficients of EVERY source are written to coef (coef
 *                   required, coef_stride >= 3S), gradient rows are formed as
 *                   usual, no workspace is used (it may be NULL), and each
 *                   workgroup takes one token; attnres_block_backward and
 *                   attnres_partial_dw then form dL/dw from the coefficients.
 *   workspace       device, at least attnres_aggregate_backward_workspace()
 *                   bytes, 16-byte aligned (NULL allowed for T = 0): one
 *                   float32 row of dL/dw per workgroup, summed in a fixed order,
 *                   so results are bitwise reproducible on one device.
 * Outputs may not overlap the inputs or each other (ATTNRES_EALIAS).  Unlike
 * the forward, T = 0 still launches (to zero grad_w; with grad_w NULL it
 * launches nothing).  coef_stride * T must stay below 2^40 (ATTNRES_EINVAL).
 */
ATTNRES_API int attnres_aggregate_backward(const void* sources, int32_t S, int64_t T, int32_t d, int64_t src_stride,
                                           const void* last_source, const float* w, const void* grad_out,
                                           float* grad_sources,
                                           int64_t grad_stride, uint32_t accumulate_mask, uint32_t defer_mask,
                                           float* coef, int64_t coef_stride, void* grad_last,
                                           float* grad_w, void* workspace, int64_t workspace_bytes, float eps,
                                           int32_t dtype, void* stream);

/*
 * attnres_aggregate_backward_static -- attnres_aggregate_backward without a
 * workspace, for callers that cannot allocate device memory: code under HIP
 * graph capture, training or serving loops, harnesses that forbid hipMalloc.
 * Allocates nothing.  The per-workgroup dL/dw rows go to a static device array
 * of ATTNRES_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends; the grid is capped at the rows it holds
 * (ATTNRES_STATIC_SCRATCH_BYTES / (4 d): 585 at d = 7168, 256 at d = 16384),
 * so with the same grid the results are bitwise those of
 * attnres_aggregate_backward.  Arguments, checks and outputs as there, minus
 * workspace; ATTNRES_EINVAL if one row of d floats exceeds the array (no d the
 * library supports does).  Every call on a GPU shares that GPU's array: calls
 * that overlap in time on one GPU (on different streams) race.  The first
 * call on a device resolves the array's address on it; make one call before
 * capturing a graph.
 */
#define ATTNRES_STATIC_SCRATCH_BYTES (16 << 20)
ATTNRES_API int attnres_aggregate_backward_static(const void* sources, int32_t S, int64_t T, int32_t d,
                                                  int64_t src_stride, const void* last_source, const float* w,
                                                  const void* grad_out, float* grad_sources, int64_t grad_stride,
                                                  uint32_t accumulate_mask, uint32_t defer_mask, float* coef,
                                                  int64_t coef_stride, void* grad_last, float* grad_w, float eps,
                                                  int32_t dtype, void* stream);

/*
 * attnres_block_backward -- the deferred gradients of a block's inter-block
 * sources.  In Block AttnRes the n sources h_0, b_1 .. b_{n-1} are shared by
 * every layer of block n (kimi.papertok.ai §4.3); when the B layers' backwards
 * defer them (attnres_aggregate_backward, defer_mask), this adds all their
 * contributions in one pass, per token and source:
 *   G_s += sum_l (a_{l,s} g_l + c1_{l,s} w_l) - (sum_l c3_{l,s}) H_s
 * and to each layer's dL/dw the deferred sources' share:
 *   dw_l += sum over tokens and s of c1_{l,s} H_s
 *
 *   sources       device, n rows [T][d] (dtype) at src_stride elements, n <= 8.
 *   B             layers, 1..16; grad_outs[l] (device [T][d] dtype, dL/dr_l),
 *                 queries[l] (device [d] float32) and grad_ws[l] (device [d]
 *                 float32, added to) are HOST arrays of B pointers.  A "layer"
 *                 may be any aggregation over these sources (e.g. the final
 *                 one of the network).
 *   coef          device float32 [T][B][m]: layer l's coefficients, as its
 *                 backward wrote them with coef = coef + m l, coef_stride m B;
 *                 its n triples (a, c1, c3) of the inter-block sources come
 *                 first, m = coef_layer_stride floats apart.
 *   coef_layer_stride  m >= 3n, or 0 for m = 3n.  A layer whose backward left
 *                 dL/dw to the caller also wrote the triple of its own last
 *                 source (its partial block sum) at 3n: m = 3(n + 1) keeps it
 *                 for attnres_partial_dw.
 *   grad_sources  device, n rows [T][d] float32 at grad_stride floats; rows whose
 *                 bit is set in accumulate_mask are added into, others written.
 *   grad_last     device [T][d] dtype, or NULL: the new gradient row n-1 (the
 *                 finished gradient of the previous block's last layer output).
 *   workspace     device, at least attnres_block_backward_workspace() bytes,
 *                 16-byte aligned: partial dL/dw rows, summed in a fixed order
 *                 (bitwise reproducible on one device).
 * Outputs may not overlap the inputs or each other (ATTNRES_EALIAS).  Needs d a
 * multiple of 8 and T*B*m*4 < 2^31 (else ATTNRES_EUNSUPPORTED).
 */
ATTNRES_API int attnres_block_backward(const void* sources, int32_t n, int64_t T, int32_t d, int64_t src_stride,
                                       int32_t B, const void* const* grad_outs, const float* const* queries,
                                       const float* coef, int64_t coef_layer_stride, float* grad_sources,
                                       int64_t grad_stride, uint32_t accumulate_mask, void* grad_last,
                                       float* const* grad_ws, void* workspace, int64_t workspace_bytes,
                                       int32_t dtype, void* stream);

/*
 * attnres_partial_dw -- each layer's dL/dw share from a source row of its own.
 * In Block AttnRes the last source of layer l's aggregation is the partial sum
 * of its block (kimi.papertok.ai §4.3), read by that layer only; when its
 * backward left dL/dw to the caller (attnres_aggregate_backward with grad_w
 * NULL), that source's share, sum over tokens of (delta/rho) H, is formed here
 * for up to 16 layers in one pass:
 *   grad_ws[l] = sum over tokens t of coef[t * coef_stride + l * coef_layer_stride] * rows[l][t]
 * (float32, summed in a fixed order: bitwise reproducible on one device).
 *   rows          HOST array of B pointers: device [T][d] in dtype, 16-byte
 *                 aligned, or NULL for a layer without such a row (its
 *                 grad_ws row is set to zero).
 *   coef          device float32; for layers written by
 *                 attnres_aggregate_backward with coef = base + m l and
 *                 coef_stride m B, pass base + 3 (S-1) + 1 (the c1 of the
 *                 last source), coef_stride m B and coef_layer_stride m.  May
 *                 be NULL when no row is given or T = 0.
 *   grad_ws       HOST array of B pointers: device [d] float32, overwritten
 *                 (zero for T = 0).
 *   workspace     device, at least attnres_partial_dw_workspace() bytes,
 *                 16-byte aligned (NULL allowed for T = 0).
 * Outputs may not overlap the inputs or each other (ATTNRES_EALIAS); strides
 * are non-negative with coef_stride * T and coef_layer_stride below 2^40
 * (ATTNRES_EINVAL).
 */
ATTNRES_API int attnres_partial_dw(const void* const* rows, int32_t B, int64_t T, int32_t d, const float* coef,
                                   int64_t coef_stride, int64_t coef_layer_stride, float* const* grad_ws,
                                   void* workspace, int64_t workspace_bytes, int32_t dtype, void* stream);

/* Workspace bytes attnres_partial_dw needs for T tokens of width d and B layers
 * on the current device (host only apart from a device-attribute query). */
ATTNRES_API int attnres_partial_dw_workspace(int64_t T, int32_t d, int32_t B, int32_t dtype, int64_t* bytes);

/* Workspace bytes attnres_block_backward needs for T tokens of width d and B
 * layers on the current device (host only apart from a device-attribute query). */
ATTNRES_API int attnres_block_backward_workspace(int64_t T, int32_t d, int32_t B, int32_t dtype, int64_t* bytes);

/* Workspace bytes attnres_aggregate_backward needs for T tokens of width d on
 * the current device (host only apart from a device-attribute query). */
ATTNRES_API int attnres_aggregate_backward_workspace(int64_t T, int32_t d, int32_t dtype, int64_t* bytes);

/* Launch shape the library picks for an aggregation (host only, no HIP call). */
typedef struct attnres_launch {
  int32_t threads;          /* threads per workgroup (multiple of 64)         */
  int32_t vecs_per_lane;    /* 16-byte vectors of one source row per lane     */
  int64_t grid;             /* workgroups                                     */
  int32_t tokens_per_group; /* tokens a workgroup handles (1)                 */
  int32_t xcd_run;          /* consecutive tokens each XCD takes in turn: the
                               workgroup of virtual index b (b = blockIdx, plus
                               grid per earlier launch when the batch needs
                               several launches of at most grid workgroups, or
                               per earlier trip of the workgroup for more than
                               9 sources) runs on XCD b % 8 and handles
                               token ((b / 8 / r) * 8 + b % 8) * r + (b / 8) % r
                               for r = xcd_run (1: token b); the virtual
                               indices cover T rounded up to 8 r             */
} attnres_launch_t;

/*
 * attnres_aggregate_config -- the launch attnres_aggregate would use for this
 * shape on a device with num_cus compute units (host only).  Same argument
 * checks as attnres_aggregate (without pointers).
 */
ATTNRES_API int attnres_aggregate_config(int32_t S, int64_t T, int32_t d, int32_t dtype,
                                         int32_t num_cus, attnres_launch_t* cfg);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
