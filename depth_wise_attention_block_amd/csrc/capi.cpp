// C ABI of libattnres.so: host-side argument checks, launch-shape policy and
// source-store bookkeeping.  Every check runs before any HIP call, so a
// rejected call has no side effect at all (and the checks work without a GPU).
#include <atomic>
#include <cmath>
#include <cstdint>
#include <vector>

#include "attnres.h"
#include "internal.h"
#include "launch_policy.h"

static_assert(ATTNRES_MAX_SOURCES_FULL == attnres::kMaxSourcesMany, "source limits disagree");
static_assert(ATTNRES_MAX_INTER_SOURCES == attnres::kMaxInterSources, "inter-source limits disagree");
static_assert(ATTNRES_MAX_BLOCK_QUERIES == attnres::kMaxBlockQueries, "query limits disagree");
static_assert(ATTNRES_STATIC_SCRATCH_BYTES == attnres::kStaticScratchBytes, "static scratch sizes disagree");

namespace {

constexpr int kVersion = 10000;  // 1.0.0

int elem_bytes(int32_t dtype) { return dtype == ATTNRES_BF16 ? 2 : 4; }
int elems_per_vec(int32_t dtype) { return attnres::kVecBytes / elem_bytes(dtype); }
bool known_dtype(int32_t dtype) { return dtype == ATTNRES_BF16 || dtype == ATTNRES_F32; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes of n prepared queries: ceil(n / 4) groups of [2][d / 8][4][8] bf16.
int64_t prepared_query_bytes(int64_t n, int d) { return ATTNRES_PREPARED_QUERY_BYTES(n, d); }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Shape checks shared by aggregate, its config query and the store.
int check_shape(int64_t T, int32_t d, int32_t dtype) {
  if (!known_dtype(dtype)) return ATTNRES_EUNSUPPORTED;
  if (T < 0 || d <= 0) return ATTNRES_EINVAL;
  if (d % elems_per_vec(dtype) != 0) return ATTNRES_EUNSUPPORTED;
  if (d > (dtype == ATTNRES_BF16 ? ATTNRES_MAX_D_BF16 : ATTNRES_MAX_D_F32)) return ATTNRES_EUNSUPPORTED;
  // keep every element offset far inside int64
  if (T > (INT64_C(1) << 40) / d) return ATTNRES_EINVAL;
  return ATTNRES_OK;
}

// Compute units of the current device, queried once per device.
int device_cus(int* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTNRES_ELAUNCH;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return ATTNRES_OK;
    }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return ATTNRES_ELAUNCH;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  *out = cus;
  return ATTNRES_OK;
}

int check_store(const attnres_store_t* st) {
  if (st == nullptr) return ATTNRES_EINVAL;
  int rc = check_shape(st->T, st->d, st->dtype);
  if (rc != ATTNRES_OK) return rc;
  if (st->base == nullptr && st->T > 0) return ATTNRES_EINVAL;  // an empty store holds no rows
  if (!aligned16(st->base)) return ATTNRES_EUNSUPPORTED;
  if (st->s_max < 2 || st->s_max > ATTNRES_MAX_SOURCES) return ATTNRES_EINVAL;
  if (st->slot_stride < st->T * st->d) return ATTNRES_EINVAL;
  if (st->slot_stride % elems_per_vec(st->dtype) != 0) return ATTNRES_EUNSUPPORTED;
  if (st->slot_stride > (INT64_C(1) << 40)) return ATTNRES_EINVAL;
  if (st->n_completed < 0 || (st->partial_valid != 0 && st->partial_valid != 1)) return ATTNRES_ESTATE;
  if (1 + st->n_completed + st->partial_valid > st->s_max) return ATTNRES_ESTATE;
  return ATTNRES_OK;
}

}  // namespace

extern "C" {

ATTNRES_API int attnres_version(void) { return kVersion; }

ATTNRES_API const char* attnres_strerror(int status) {
  switch (status) {
    case ATTNRES_OK: return "success";
    case ATTNRES_EINVAL: return "invalid argument (count, size, null pointer or flag)";
    case ATTNRES_EUNSUPPORTED: return "unsupported layout (alignment, vector multiple, hidden size or dtype)";
    case ATTNRES_EALIAS: return "an output buffer overlaps an input buffer";
    case ATTNRES_ELAUNCH: return "the HIP runtime refused the kernel launch";
    case ATTNRES_ESTATE: return "source store full or inconsistent";
    default: return "unknown status";
  }
}

ATTNRES_API int attnres_aggregate_config(int32_t S, int64_t T, int32_t d, int32_t dtype, int32_t num_cus,
                                         attnres_launch_t* cfg) {
  if (cfg == nullptr) return ATTNRES_EINVAL;
  if (S < 1 || S > ATTNRES_MAX_SOURCES_FULL) return ATTNRES_EINVAL;
  const int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  return pick_config(S, T, d, dtype, num_cus, cfg, true);
}

ATTNRES_API int attnres_aggregate(const void* sources, int32_t S, int64_t T, int32_t d, int64_t src_stride,
                                  const float* w, void* out, float* weights, float eps, int32_t dtype,
                                  void* stream) {
  if (S < 1 || S > ATTNRES_MAX_SOURCES_FULL) return ATTNRES_EINVAL;
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ATTNRES_EINVAL;
  const int64_t row = T * (int64_t)d;
  if (src_stride == 0) src_stride = row;
  if (src_stride < 0 || src_stride > (INT64_C(1) << 40)) return ATTNRES_EINVAL;
  if (S > 1 && src_stride < row) return ATTNRES_EINVAL;
  if (src_stride % elems_per_vec(dtype) != 0) return ATTNRES_EUNSUPPORTED;
  if (T == 0) return ATTNRES_OK;
  if (sources == nullptr || w == nullptr || out == nullptr) return ATTNRES_EINVAL;
  if (!aligned16(sources) || !aligned16(w) || !aligned16(out)) return ATTNRES_EUNSUPPORTED;
  if (weights != nullptr && (reinterpret_cast<uintptr_t>(weights) & 3u) != 0) return ATTNRES_EUNSUPPORTED;

  const int es = elem_bytes(dtype);
  const Range r_src = range(sources, ((int64_t)(S - 1) * src_stride + row) * es);
  const Range r_w = range(w, (int64_t)d * 4);
  const Range r_out = range(out, row * es);
  if (overlap(r_out, r_src) || overlap(r_out, r_w)) return ATTNRES_EALIAS;
  if (weights != nullptr) {
    const Range r_wt = range(weights, T * (int64_t)S * 4);
    if (overlap(r_wt, r_src) || overlap(r_wt, r_w) || overlap(r_wt, r_out)) return ATTNRES_EALIAS;
  }

  int cus = 0;
  rc = device_cus(&cus);
  if (rc != ATTNRES_OK) return rc;
  attnres_launch_t cfg;
  rc = pick_config(S, T, d, dtype, cus, &cfg, true);
  if (rc != ATTNRES_OK) return rc;

  attnres::AggregateArgs a;
  a.sources = sources;
  a.S = S;
  a.T = T;
  a.d = d;
  a.src_stride = src_stride;
  a.w = w;
  a.out = out;
  a.weights = weights;
  a.eps = eps;
  a.bf16 = dtype == ATTNRES_BF16;
  a.threads = cfg.threads;
  a.vecs_per_lane = cfg.vecs_per_lane;
  a.grid = cfg.grid;
  a.xcd_run = cfg.xcd_run;
  (void)hipGetLastError();  // start from a clean error state
  return attnres::launch_aggregate(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTNRES_OK
                                                                                      : ATTNRES_ELAUNCH;
}

// Workgroups of the backward pass: as many as fit on the device at once, each
// accumulating dL/dw over its tokens.  The general kernel holds every source
// row in registers: two workgroups per CU for d up to 4096, one above.  The
// kernel for the case where only the last row is written streams the rows and
// fits two per CU up to d = 8192.
int backward_per_cu(int v, bool last_only) { return (v == 1 || (last_only && v == 2)) ? 2 : 1; }

int64_t backward_grid(int64_t T, int cus, int per_cu) {
  const int64_t resident = (int64_t)cus * per_cu;
  return T < resident ? T : resident;
}

ATTNRES_API int attnres_aggregate_backward_workspace(int64_t T, int32_t d, int32_t dtype, int64_t* bytes) {
  if (bytes == nullptr) return ATTNRES_EINVAL;
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  if (T == 0) {
    *bytes = 0;
    return ATTNRES_OK;
  }
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != ATTNRES_OK) return rc;
  attnres_launch_t cfg;
  rc = pick_config(1, T, d, dtype, cus, &cfg);
  if (rc != ATTNRES_OK) return rc;
  *bytes = backward_grid(T, cus, backward_per_cu(cfg.vecs_per_lane, true)) * (int64_t)d * 4;
  return ATTNRES_OK;
}

}  // extern "C"

namespace {

// attnres_aggregate_backward, with its dL/dw rows either in the caller's
// workspace or (use_static) in the library's static device array, whose grid
// is then capped at the rows that fit.
int aggregate_backward_impl(const void* sources, int32_t S, int64_t T, int32_t d, int64_t src_stride,
                            const void* last_source, const float* w, const void* grad_out, float* grad_sources,
                            int64_t grad_stride, uint32_t accumulate_mask, uint32_t defer_mask, float* coef,
                            int64_t coef_stride, void* grad_last, float* grad_w, void* workspace,
                            int64_t workspace_bytes, bool use_static, float eps, int32_t dtype, void* stream) {
  if (S < 1 || S > ATTNRES_MAX_SOURCES) return ATTNRES_EINVAL;
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ATTNRES_EINVAL;
  const int64_t row = T * (int64_t)d;
  if (src_stride == 0) src_stride = row;
  if (grad_stride == 0) grad_stride = row;
  if (src_stride < 0 || src_stride > (INT64_C(1) << 40) || grad_stride < 0 || grad_stride > (INT64_C(1) << 40))
    return ATTNRES_EINVAL;
  if (S > 1 && (src_stride < row || grad_stride < row)) return ATTNRES_EINVAL;
  if (src_stride % elems_per_vec(dtype) != 0 || grad_stride % 4 != 0) return ATTNRES_EUNSUPPORTED;
  // without grad_w, dL/dw is left to the caller: every source's coefficients
  // are written, no workspace is used, and the grid is one workgroup per token
  const bool form_dw = grad_w != nullptr;
  if (form_dw && (reinterpret_cast<uintptr_t>(grad_w) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
  defer_mask &= (S >= 32) ? 0xFFFFFFFFu : ((1u << S) - 1u);
  if (defer_mask != 0 || !form_dw) {
    // every coefficient offset stays far inside int64 (as the element offsets do)
    if (coef == nullptr || coef_stride < 3 * (int64_t)S || coef_stride > (INT64_C(1) << 40) / (T > 0 ? T : 1))
      return ATTNRES_EINVAL;
    if ((reinterpret_cast<uintptr_t>(coef) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
    if (grad_last != nullptr && ((defer_mask >> (S - 1)) & 1u)) return ATTNRES_EINVAL;  // nothing to hand out
  }
  if (!form_dw) {
    workspace = nullptr;
    workspace_bytes = 0;
    use_static = false;
  }
  const int es = elem_bytes(dtype);
  const Range r_gw = form_dw ? range(grad_w, (int64_t)d * 4) : Range{0, 0};
  if (T > 0) {
    if ((sources == nullptr && !(S == 1 && last_source != nullptr)) || w == nullptr || grad_out == nullptr ||
        grad_sources == nullptr || (form_dw && !use_static && (workspace == nullptr || workspace_bytes <= 0)))
      return ATTNRES_EINVAL;
    if (!aligned16(sources) || !aligned16(w) || !aligned16(grad_out) || !aligned16(grad_sources) ||
        !aligned16(workspace) || (grad_last != nullptr && !aligned16(grad_last)) ||
        (last_source != nullptr && !aligned16(last_source)))
      return ATTNRES_EUNSUPPORTED;
    // rows read through the stride: all S, or S-1 when the last one is given apart
    const int strided = last_source != nullptr ? S - 1 : S;
    const Range r_src = strided > 0 ? range(sources, ((int64_t)(strided - 1) * src_stride + row) * es) : Range{0, 0};
    const Range r_last = last_source != nullptr ? range(last_source, row * es) : Range{0, 0};
    const Range r_w = range(w, (int64_t)d * 4);
    const Range r_g = range(grad_out, row * es);
    const Range r_gs = range(grad_sources, ((int64_t)(S - 1) * grad_stride + row) * 4);
    const Range r_gl = grad_last != nullptr ? range(grad_last, row * es) : Range{0, 0};
    const Range r_ws = form_dw ? range(workspace, workspace_bytes) : Range{0, 0};
    // coefficients are written for the deferred sources, up to the highest one
    // (for all S sources when dL/dw is left to the caller)
    const int top = !form_dw ? S : defer_mask != 0 ? 32 - __builtin_clz(defer_mask) : 0;
    const Range r_cf = top > 0 ? range(coef, ((T - 1) * coef_stride + 3 * (int64_t)top) * 4) : Range{0, 0};
    const Range outs[5] = {r_gs, r_gl, r_gw, r_ws, r_cf};
    const Range ins[4] = {r_src, r_w, r_g, r_last};
    for (int i = 0; i < 5; ++i) {
      for (int k = 0; k < 4; ++k)
        if (overlap(outs[i], ins[k])) return ATTNRES_EALIAS;
      for (int k = i + 1; k < 5; ++k)
        if (overlap(outs[i], outs[k])) return ATTNRES_EALIAS;
    }
  }
  if (!form_dw && T == 0) return ATTNRES_OK;  // no dL/dw to zero: nothing to launch
  const int64_t row_bytes = (int64_t)d * 4;
  if (use_static && row_bytes > attnres::kStaticScratchBytes) return ATTNRES_EINVAL;  // beyond the static array
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != ATTNRES_OK) return rc;
  attnres_launch_t cfg;
  rc = pick_config(S, T, d, dtype, cus, &cfg);
  if (rc != ATTNRES_OK) return rc;
  const unsigned all = S >= 32 ? 0xFFFFFFFFu : ((1u << S) - 1u);
  const bool last_only = ((~defer_mask & all) & ~(1u << (S - 1))) == 0;
  // with dL/dw formed here each workgroup sums it over the tokens it loops
  // over; without, a workgroup takes one token (a looping workgroup's loads
  // queue behind its previous token's stores: 9-13% slower per launch)
  int64_t grid = form_dw ? backward_grid(T, cus, backward_per_cu(cfg.vecs_per_lane, last_only))
                         : (T < INT64_C(0x7fffffff) ? T : INT64_C(0x7fffffff));
  if (use_static) {
    // the static array, resolved once per device, and no more rows than it holds
    if (attnres::static_scratch(&workspace) != hipSuccess) return ATTNRES_ELAUNCH;
    workspace_bytes = attnres::kStaticScratchBytes;
    const int64_t rows = workspace_bytes / row_bytes;
    if (grid > rows) grid = rows;
  }
  if (form_dw && T > 0 && workspace_bytes < grid * row_bytes) return ATTNRES_EINVAL;
  attnres::BackwardArgs a;
  a.sources = sources;
  a.S = S;
  a.T = T;
  a.d = d;
  a.src_stride = src_stride;
  a.last_source = last_source;
  a.w = w;
  a.grad_out = grad_out;
  a.grad_sources = grad_sources;
  a.grad_stride = grad_stride;
  a.acc_mask = accumulate_mask;
  a.defer_mask = defer_mask;
  a.coef = coef;
  a.coef_stride = coef_stride;
  a.grad_last = grad_last;
  a.grad_w = grad_w;
  a.workspace = static_cast<float*>(workspace);
  a.eps = eps;
  a.bf16 = dtype == ATTNRES_BF16;
  a.last_only = last_only;
  a.form_dw = form_dw;
  a.threads = cfg.threads;
  a.vecs_per_lane = cfg.vecs_per_lane;
  a.grid = grid;
  (void)hipGetLastError();
  return attnres::launch_aggregate_backward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTNRES_OK
                                                                                               : ATTNRES_ELAUNCH;
}

}  // namespace

extern "C" {

ATTNRES_API int attnres_aggregate_backward(const void* sources, int32_t S, int64_t T, int32_t d, int64_t src_stride,
                                           const void* last_source, const float* w, const void* grad_out,
                                           float* grad_sources,
                                           int64_t grad_stride, uint32_t accumulate_mask, uint32_t defer_mask,
                                           float* coef, int64_t coef_stride, void* grad_last,
                                           float* grad_w, void* workspace, int64_t workspace_bytes, float eps,
                                           int32_t dtype, void* stream) {
  return aggregate_backward_impl(sources, S, T, d, src_stride, last_source, w, grad_out, grad_sources, grad_stride,
                                 accumulate_mask, defer_mask, coef, coef_stride, grad_last, grad_w, workspace,
                                 workspace_bytes, false, eps, dtype, stream);
}

ATTNRES_API int attnres_aggregate_backward_static(const void* sources, int32_t S, int64_t T, int32_t d,
                                                  int64_t src_stride, const void* last_source, const float* w,
                                                  const void* grad_out, float* grad_sources, int64_t grad_stride,
                                                  uint32_t accumulate_mask, uint32_t defer_mask, float* coef,
                                                  int64_t coef_stride, void* grad_last, float* grad_w, float eps,
                                                  int32_t dtype, void* stream) {
  return aggregate_backward_impl(sources, S, T, d, src_stride, last_source, w, grad_out, grad_sources, grad_stride,
                                 accumulate_mask, defer_mask, coef, coef_stride, grad_last, grad_w, nullptr, 0, true,
                                 eps, dtype, stream);
}

// Token groups of the block pass's dL/dw contraction: about four workgroups per
// CU over the column blocks, and never more groups than tokens.
int64_t block_dw_groups(int64_t T, int d, int cus) {
  const int64_t colblocks = (d + attnres::kBlockDwCols - 1) / attnres::kBlockDwCols;
  const int64_t want = ((int64_t)cus * 4 + colblocks - 1) / colblocks;
  return T < want ? (T > 0 ? T : 1) : want;
}

ATTNRES_API int attnres_block_backward_workspace(int64_t T, int32_t d, int32_t B, int32_t dtype, int64_t* bytes) {
  if (bytes == nullptr || B < 1 || B > attnres::kMaxBlockLayers) return ATTNRES_EINVAL;
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  if (d % 8 != 0) return ATTNRES_EUNSUPPORTED;
  if (T == 0) {
    *bytes = 0;
    return ATTNRES_OK;
  }
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != ATTNRES_OK) return rc;
  *bytes = block_dw_groups(T, d, cus) * B * (int64_t)d * 4;
  return ATTNRES_OK;
}

ATTNRES_API int attnres_block_backward(const void* sources, int32_t n, int64_t T, int32_t d, int64_t src_stride,
                                       int32_t B, const void* const* grad_outs, const float* const* queries,
                                       const float* coef, int64_t coef_layer_stride, float* grad_sources,
                                       int64_t grad_stride, uint32_t accumulate_mask, void* grad_last,
                                       float* const* grad_ws, void* workspace, int64_t workspace_bytes,
                                       int32_t dtype, void* stream) {
  if (n < 1 || n > attnres::kMaxInterSources || B < 1 || B > attnres::kMaxBlockLayers) return ATTNRES_EINVAL;
  const int64_t cls = coef_layer_stride == 0 ? 3 * (int64_t)n : coef_layer_stride;
  if (cls < 3 * (int64_t)n) return ATTNRES_EINVAL;
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  const int64_t row = T * (int64_t)d;
  if (src_stride == 0) src_stride = row;
  if (grad_stride == 0) grad_stride = row;
  if (src_stride < 0 || grad_stride < 0 || src_stride > (INT64_C(1) << 40) || grad_stride > (INT64_C(1) << 40))
    return ATTNRES_EINVAL;
  if (n > 1 && (src_stride < row || grad_stride < row)) return ATTNRES_EINVAL;
  if (src_stride % elems_per_vec(dtype) != 0 || grad_stride % 4 != 0) return ATTNRES_EUNSUPPORTED;
  // the dL/dw contraction takes 8 columns per lane and addresses the
  // coefficients with 32-bit byte offsets: T * B * cls * 4 < 2^31
  if (d % 8 != 0 || (T > 0 && cls > ((INT64_C(1) << 31) - 1) / (4 * (int64_t)B * T))) return ATTNRES_EUNSUPPORTED;
  if (T == 0) return ATTNRES_OK;
  if (sources == nullptr || grad_outs == nullptr || queries == nullptr || coef == nullptr ||
      grad_sources == nullptr || grad_ws == nullptr || workspace == nullptr)
    return ATTNRES_EINVAL;
  const int es = elem_bytes(dtype);
  if (!aligned16(sources) || !aligned16(grad_sources) || !aligned16(workspace) ||
      (grad_last != nullptr && !aligned16(grad_last)) || (reinterpret_cast<uintptr_t>(coef) & 3u) != 0)
    return ATTNRES_EUNSUPPORTED;
  std::vector<Range> ins = {range(sources, ((int64_t)(n - 1) * src_stride + row) * es),
                            range(coef, (int64_t)T * B * cls * 4)};
  std::vector<Range> outs = {range(grad_sources, ((int64_t)(n - 1) * grad_stride + row) * 4),
                             grad_last != nullptr ? range(grad_last, row * es) : Range{0, 0},
                             range(workspace, workspace_bytes)};
  attnres::BlockBackwardArgs a;
  for (int l = 0; l < attnres::kMaxBlockLayers; ++l) {
    a.rows.g[l] = nullptr;
    a.rows.w[l] = nullptr;
    a.grad_w.p[l] = nullptr;
  }
  for (int l = 0; l < B; ++l) {
    if (grad_outs[l] == nullptr || queries[l] == nullptr || grad_ws[l] == nullptr) return ATTNRES_EINVAL;
    if (!aligned16(grad_outs[l]) || !aligned16(queries[l]) || !aligned16(grad_ws[l])) return ATTNRES_EUNSUPPORTED;
    ins.push_back(range(grad_outs[l], row * es));
    ins.push_back(range(queries[l], (int64_t)d * 4));
    outs.push_back(range(grad_ws[l], (int64_t)d * 4));
    a.rows.g[l] = grad_outs[l];
    a.rows.w[l] = queries[l];
    a.grad_w.p[l] = grad_ws[l];
  }
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ATTNRES_EALIAS;
    for (size_t k = i + 1; k < outs.size(); ++k)
      if (overlap(outs[i], outs[k])) return ATTNRES_EALIAS;
  }
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != ATTNRES_OK) return rc;
  attnres_launch_t cfg;
  rc = pick_config(n, T, d, dtype, cus, &cfg);
  if (rc != ATTNRES_OK) return rc;
  const int64_t groups = block_dw_groups(T, d, cus);
  if (workspace_bytes < groups * B * (int64_t)d * 4) return ATTNRES_EINVAL;
  a.sources = sources;
  a.n = n;
  a.T = T;
  a.d = d;
  a.src_stride = src_stride;
  a.B = B;
  a.coef = coef;
  a.coef_layer = (int)cls;
  a.grad_sources = grad_sources;
  a.grad_stride = grad_stride;
  a.acc_mask = accumulate_mask;
  a.grad_last = grad_last;
  a.workspace = static_cast<float*>(workspace);
  a.bf16 = dtype == ATTNRES_BF16;
  a.threads = cfg.threads;
  a.vecs_per_lane = cfg.vecs_per_lane;
  a.grid = cfg.grid;
  a.dw_colblocks = (d + attnres::kBlockDwCols - 1) / attnres::kBlockDwCols;
  a.dw_groups = groups;
  (void)hipGetLastError();
  return attnres::launch_block_backward(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTNRES_OK
                                                                                           : ATTNRES_ELAUNCH;
}

// Token groups of attnres_partial_dw: about 16 workgroups of two waves per CU
// over the B layers' column blocks, at most one group per token.
int64_t partial_dw_groups(int64_t T, int d, int32_t dtype, int B, int cus, int* colblocks) {
  const int64_t nvec = d / elems_per_vec(dtype);
  *colblocks = (int)((nvec + attnres::kPartialDwThreads - 1) / attnres::kPartialDwThreads);
  const int64_t per = (int64_t)*colblocks * B;
  const int64_t want = ((int64_t)cus * 16 + per - 1) / per;
  return T < want ? (T > 0 ? T : 1) : want;
}

ATTNRES_API int attnres_partial_dw_workspace(int64_t T, int32_t d, int32_t B, int32_t dtype, int64_t* bytes) {
  if (bytes == nullptr || B < 1 || B > attnres::kMaxBlockLayers) return ATTNRES_EINVAL;
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  if (T == 0) {
    *bytes = 0;
    return ATTNRES_OK;
  }
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != ATTNRES_OK) return rc;
  int colblocks = 0;
  *bytes = partial_dw_groups(T, d, dtype, B, cus, &colblocks) * B * (int64_t)d * 4;
  return ATTNRES_OK;
}

ATTNRES_API int attnres_partial_dw(const void* const* rows, int32_t B, int64_t T, int32_t d, const float* coef,
                                   int64_t coef_stride, int64_t coef_layer_stride, float* const* grad_ws,
                                   void* workspace, int64_t workspace_bytes, int32_t dtype, void* stream) {
  if (B < 1 || B > attnres::kMaxBlockLayers) return ATTNRES_EINVAL;
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  if (rows == nullptr || grad_ws == nullptr) return ATTNRES_EINVAL;
  // every coefficient offset t * coef_stride + l * coef_layer_stride far inside int64
  const int64_t lim = (INT64_C(1) << 40) / (T > 0 ? T : 1);
  if (coef_stride < 0 || coef_stride > lim || coef_layer_stride < 0 || coef_layer_stride > (INT64_C(1) << 40))
    return ATTNRES_EINVAL;
  const int64_t row = T * (int64_t)d;
  const int es = elem_bytes(dtype);
  bool any = false;  // a row to read (none for T = 0: the rows are only zeroed)
  for (int l = 0; l < B; ++l) any = any || (rows[l] != nullptr && T > 0);
  if (any) {
    if (coef == nullptr) return ATTNRES_EINVAL;
    if ((reinterpret_cast<uintptr_t>(coef) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
  }
  std::vector<Range> ins, outs;
  if (any) ins.push_back(range(coef, ((T - 1) * coef_stride + (int64_t)(B - 1) * coef_layer_stride + 1) * 4));
  attnres::PartialDwArgs a;
  for (int l = 0; l < attnres::kMaxBlockLayers; ++l) {
    a.rows.x[l] = nullptr;
    a.rows.c[l] = nullptr;
    a.out.p[l] = nullptr;
  }
  for (int l = 0; l < B; ++l) {
    if (grad_ws[l] == nullptr) return ATTNRES_EINVAL;
    if ((reinterpret_cast<uintptr_t>(grad_ws[l]) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
    outs.push_back(range(grad_ws[l], (int64_t)d * 4));
    a.out.p[l] = grad_ws[l];
    if (rows[l] == nullptr || T == 0) continue;
    if (!aligned16(rows[l])) return ATTNRES_EUNSUPPORTED;
    ins.push_back(range(rows[l], row * es));
    a.rows.x[l] = rows[l];
    a.rows.c[l] = coef + l * coef_layer_stride;
  }
  if (T > 0) {
    if (workspace == nullptr) return ATTNRES_EINVAL;
    if (!aligned16(workspace)) return ATTNRES_EUNSUPPORTED;
    outs.push_back(range(workspace, workspace_bytes));
  }
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ATTNRES_EALIAS;
    for (size_t k = i + 1; k < outs.size(); ++k)
      if (overlap(outs[i], outs[k])) return ATTNRES_EALIAS;
  }
  int cus = 0;
  rc = device_cus(&cus);
  if (rc != ATTNRES_OK) return rc;
  int colblocks = 0;
  const int64_t groups = T > 0 ? partial_dw_groups(T, d, dtype, B, cus, &colblocks) : 0;
  if (workspace_bytes < groups * B * (int64_t)d * 4) return ATTNRES_EINVAL;
  a.B = B;
  a.T = T;
  a.d = d;
  a.coef_stride = coef_stride;
  a.workspace = static_cast<float*>(workspace);
  a.bf16 = dtype == ATTNRES_BF16;
  a.colblocks = colblocks;
  a.groups = groups;
  (void)hipGetLastError();
  return attnres::launch_partial_dw(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTNRES_OK
                                                                                      : ATTNRES_ELAUNCH;
}

ATTNRES_API int attnres_partial_sums(const void* const* layer_outs, int32_t count, int64_t T, int32_t d, void* out,
                                     int64_t out_stride, int32_t dtype, void* stream) {
  if (count < 1 || count > attnres::kMaxBlockLayers) return ATTNRES_EINVAL;
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  const int64_t row = T * (int64_t)d;
  if (out_stride == 0) out_stride = row;
  if (out_stride < 0 || out_stride > (INT64_C(1) << 40) || (count > 1 && out_stride < row)) return ATTNRES_EINVAL;
  if (out_stride % elems_per_vec(dtype) != 0) return ATTNRES_EUNSUPPORTED;
  if (row == 0) return ATTNRES_OK;
  if (layer_outs == nullptr || out == nullptr) return ATTNRES_EINVAL;
  if (!aligned16(out)) return ATTNRES_EUNSUPPORTED;
  const int es = elem_bytes(dtype);
  const Range r_out = range(out, ((int64_t)(count - 1) * out_stride + row) * es);
  attnres::PartialSumsArgs a;
  for (int k = 0; k < count; ++k) {
    if (layer_outs[k] == nullptr) return ATTNRES_EINVAL;
    if (!aligned16(layer_outs[k])) return ATTNRES_EUNSUPPORTED;
    if (overlap(r_out, range(layer_outs[k], row * es))) return ATTNRES_EALIAS;
    a.rows.g[k] = layer_outs[k];
  }
  a.count = count;
  a.elems = row;
  a.out = out;
  a.out_stride = out_stride;
  a.bf16 = dtype == ATTNRES_BF16;
  (void)hipGetLastError();
  return attnres::launch_partial_sums(a, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTNRES_OK
                                                                                         : ATTNRES_ELAUNCH;
}

ATTNRES_API int attnres_accumulate_aggregate(attnres_store_t* st, const void* layer_out, int32_t finalize_block,
                                             const float* w, void* out, float* weights, float eps, void* stream) {
  int rc = check_store(st);
  if (rc != ATTNRES_OK) return rc;
  if (finalize_block != 0 && finalize_block != 1) return ATTNRES_EINVAL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ATTNRES_EINVAL;
  const int slot = 1 + st->n_completed;
  if (slot >= st->s_max) return ATTNRES_ESTATE;
  // bookkeeping after the update; the updated slot is the last live source
  const int n_after = st->n_completed + (finalize_block ? 1 : 0);
  const int p_after = finalize_block ? 0 : 1;
  const int S = 1 + n_after + p_after;
  const int64_t T = st->T;
  const int d = st->d;
  const int64_t row = T * (int64_t)d;
  if (row > 0) {
    if (layer_out == nullptr || w == nullptr || out == nullptr) return ATTNRES_EINVAL;
    if (!aligned16(layer_out) || !aligned16(w) || !aligned16(out)) return ATTNRES_EUNSUPPORTED;
    if (weights != nullptr && (reinterpret_cast<uintptr_t>(weights) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
    const int es = elem_bytes(st->dtype);
    const Range r_store = range(st->base, ((int64_t)(st->s_max - 1) * st->slot_stride + row) * es);
    const Range r_f = range(layer_out, row * es);
    const Range r_w = range(w, (int64_t)d * 4);
    const Range r_out = range(out, row * es);
    if (overlap(r_f, r_store) || overlap(r_out, r_store) || overlap(r_out, r_f) || overlap(r_out, r_w) ||
        overlap(r_w, r_store))
      return ATTNRES_EALIAS;
    if (weights != nullptr) {
      const Range r_wt = range(weights, T * (int64_t)S * 4);
      if (overlap(r_wt, r_store) || overlap(r_wt, r_f) || overlap(r_wt, r_w) || overlap(r_wt, r_out))
        return ATTNRES_EALIAS;
    }
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != ATTNRES_OK) return rc;
    attnres_launch_t cfg;
    rc = pick_config(S, T, d, st->dtype, cus, &cfg, true);
    if (rc != ATTNRES_OK) return rc;
    attnres::AggregateArgs a;
    a.sources = st->base;
    a.S = S;
    a.T = T;
    a.d = d;
    a.src_stride = st->slot_stride;
    a.w = w;
    a.out = out;
    a.weights = weights;
    a.eps = eps;
    a.bf16 = st->dtype == ATTNRES_BF16;
    a.threads = cfg.threads;
    a.vecs_per_lane = cfg.vecs_per_lane;
    a.grid = cfg.grid;
    a.xcd_run = cfg.xcd_run;
    a.update = st->partial_valid ? attnres::AggregateArgs::kAddUpdate : attnres::AggregateArgs::kCopyUpdate;
    a.layer_out = layer_out;
    (void)hipGetLastError();
    if (attnres::launch_aggregate(a, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTNRES_ELAUNCH;
  }
  st->n_completed = n_after;
  st->partial_valid = p_after;
  return ATTNRES_OK;
}

ATTNRES_API int attnres_split_queries(const float* w, int32_t n, int32_t d, void* w_split, void* stream) {
  if (n < 0 || n > (1 << 20) || d <= 0 || d > ATTNRES_MAX_D_BF16) return ATTNRES_EINVAL;
  if (n == 0) return ATTNRES_OK;
  if (w == nullptr || w_split == nullptr) return ATTNRES_EINVAL;
  if (d % 8 != 0 || !aligned16(w) || !aligned16(w_split)) return ATTNRES_EUNSUPPORTED;
  if (overlap(range(w, (int64_t)n * d * 4), range(w_split, prepared_query_bytes(n, d)))) return ATTNRES_EALIAS;
  (void)hipGetLastError();
  return attnres::launch_split_queries(w, n, d, w_split, static_cast<hipStream_t>(stream)) == hipSuccess
             ? ATTNRES_OK
             : ATTNRES_ELAUNCH;
}

ATTNRES_API int attnres_block_prepare(attnres_store_t* st, const void* layer_out, int32_t close_block,
                                      const void* w, int32_t B, void* inter, int64_t inter_stride, float* logits,
                                      float* weights0, float eps, void* stream) {
  int rc = check_store(st);
  if (rc != ATTNRES_OK) return rc;
  if (st->dtype != ATTNRES_BF16) return ATTNRES_EUNSUPPORTED;
  if (close_block != 0 && close_block != 1) return ATTNRES_EINVAL;
  if (B < 1 || B > attnres::kMaxBlockQueries) return ATTNRES_EINVAL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ATTNRES_EINVAL;
  if (close_block) {
    if (1 + st->n_completed >= st->s_max) return ATTNRES_ESTATE;
  } else if (st->partial_valid) {
    return ATTNRES_ESTATE;  // an open partial must be closed first
  }
  const int n_after = st->n_completed + close_block;
  const int K = 1 + n_after;
  if (K > attnres::kMaxInterSources) return ATTNRES_EUNSUPPORTED;
  const int64_t T = st->T;
  const int d = st->d;
  const int64_t row = T * (int64_t)d;
  if (inter_stride == 0) inter_stride = row;
  if (inter_stride < row || inter_stride % 8 != 0 || inter_stride > (INT64_C(1) << 40)) return ATTNRES_EINVAL;
  if (row > 0) {
    if (w == nullptr || inter == nullptr || logits == nullptr) return ATTNRES_EINVAL;
    if (close_block && layer_out == nullptr) return ATTNRES_EINVAL;
    if (!aligned16(w) || !aligned16(inter) || (close_block && !aligned16(layer_out))) return ATTNRES_EUNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(logits) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
    if (weights0 != nullptr && (reinterpret_cast<uintptr_t>(weights0) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
    const Range r_store = range(st->base, ((int64_t)(st->s_max - 1) * st->slot_stride + row) * 2);
    const Range r_w = range(w, prepared_query_bytes(B, d));
    const Range r_in = range(inter, ((int64_t)(B - 1) * inter_stride + row) * 2);
    const Range r_lg = range(logits, (int64_t)B * T * K * 4);
    const Range r_f = close_block ? range(layer_out, row * 2) : Range{0, 0};
    const Range r_w0 = weights0 != nullptr ? range(weights0, T * (int64_t)K * 4) : Range{0, 0};
    if (overlap(r_f, r_store) || overlap(r_w, r_store) || overlap(r_in, r_store) || overlap(r_in, r_w) ||
        overlap(r_in, r_f) || overlap(r_lg, r_store) || overlap(r_lg, r_w) || overlap(r_lg, r_in) ||
        overlap(r_lg, r_f) || overlap(r_w0, r_store) || overlap(r_w0, r_w) || overlap(r_w0, r_in) ||
        overlap(r_w0, r_lg) || overlap(r_w0, r_f))
      return ATTNRES_EALIAS;
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != ATTNRES_OK) return rc;
    attnres_launch_t cfg;
    rc = pick_config(K, T, d, st->dtype, cus, &cfg);
    if (rc != ATTNRES_OK) return rc;
    attnres::PrepareArgs a;
    a.store = st->base;
    a.slot_stride = st->slot_stride;
    a.K = K;
    a.B = B;
    a.T = T;
    a.d = d;
    a.w_split = w;
    a.inter = inter;
    a.inter_stride = inter_stride;
    a.logits = logits;
    a.weights0 = weights0;
    a.eps = eps;
    a.close = !close_block ? attnres::PrepareArgs::kNone
                           : (st->partial_valid ? attnres::PrepareArgs::kAdd : attnres::PrepareArgs::kCopy);
    a.layer_out = layer_out;
    a.threads = cfg.threads;
    a.vecs_per_lane = cfg.vecs_per_lane;
    a.grid = cfg.grid;
    (void)hipGetLastError();
    if (attnres::launch_block_prepare(a, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTNRES_ELAUNCH;
  }
  st->n_completed = n_after;
  st->partial_valid = 0;
  return ATTNRES_OK;
}

ATTNRES_API int attnres_block_merge(attnres_store_t* st, const void* layer_out, const float* w, const void* inter,
                                    const float* logits, void* out, float* weights, float eps, void* stream) {
  int rc = check_store(st);
  if (rc != ATTNRES_OK) return rc;
  if (st->dtype != ATTNRES_BF16) return ATTNRES_EUNSUPPORTED;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return ATTNRES_EINVAL;
  const int slot = 1 + st->n_completed;
  if (slot >= st->s_max) return ATTNRES_ESTATE;
  const int K = 1 + st->n_completed;
  if (K > attnres::kMaxInterSources) return ATTNRES_EUNSUPPORTED;
  const int64_t T = st->T;
  const int d = st->d;
  const int64_t row = T * (int64_t)d;
  if (row > 0) {
    if (layer_out == nullptr || w == nullptr || inter == nullptr || logits == nullptr || out == nullptr)
      return ATTNRES_EINVAL;
    if (!aligned16(layer_out) || !aligned16(w) || !aligned16(inter) || !aligned16(out)) return ATTNRES_EUNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(logits) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
    if (weights != nullptr && (reinterpret_cast<uintptr_t>(weights) & 3u) != 0) return ATTNRES_EUNSUPPORTED;
    const Range r_store = range(st->base, ((int64_t)(st->s_max - 1) * st->slot_stride + row) * 2);
    const Range r_f = range(layer_out, row * 2);
    const Range r_w = range(w, (int64_t)d * 4);
    const Range r_in = range(inter, row * 2);
    const Range r_lg = range(logits, T * (int64_t)K * 4);
    const Range r_out = range(out, row * 2);
    const Range r_wt = weights != nullptr ? range(weights, T * (int64_t)(K + 1) * 4) : Range{0, 0};
    // out may be the inter row itself (the merge is in place per element);
    // any other overlap is an error
    const bool in_place = out == inter;
    if (overlap(r_f, r_store) || overlap(r_w, r_store) || overlap(r_in, r_store) || overlap(r_lg, r_store) ||
        overlap(r_out, r_store) || overlap(r_out, r_f) || overlap(r_out, r_w) || overlap(r_out, r_lg) ||
        (!in_place && overlap(r_out, r_in)) || overlap(r_wt, r_store) || overlap(r_wt, r_f) ||
        overlap(r_wt, r_w) || overlap(r_wt, r_in) || overlap(r_wt, r_lg) || overlap(r_wt, r_out))
      return ATTNRES_EALIAS;
    int cus = 0;
    rc = device_cus(&cus);
    if (rc != ATTNRES_OK) return rc;
    attnres_launch_t cfg;
    rc = pick_config(2, T, d, st->dtype, cus, &cfg);
    if (rc != ATTNRES_OK) return rc;
    attnres::MergeArgs a;
    a.slot = static_cast<char*>(st->base) + (int64_t)slot * st->slot_stride * 2;
    a.layer_out = layer_out;
    a.add = st->partial_valid != 0;
    a.inter = inter;
    a.logits = logits;
    a.K = K;
    a.T = T;
    a.d = d;
    a.w = w;
    a.out = out;
    a.weights = weights;
    a.eps = eps;
    a.threads = cfg.threads;
    a.vecs_per_lane = cfg.vecs_per_lane;
    a.grid = cfg.grid;
    a.per_token = merge_per_token(T);
    (void)hipGetLastError();
    if (attnres::launch_block_merge(a, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTNRES_ELAUNCH;
  }
  st->partial_valid = 1;
  return ATTNRES_OK;
}

ATTNRES_API int attnres_store_init(attnres_store_t* st, void* base, int32_t s_max, int64_t T, int32_t d,
                                   int64_t slot_stride, int32_t dtype) {
  if (st == nullptr) return ATTNRES_EINVAL;
  attnres_store_t s;
  s.base = base;
  s.T = T;
  s.d = d;
  s.slot_stride = slot_stride == 0 ? T * (int64_t)d : slot_stride;
  s.s_max = s_max;
  s.dtype = dtype;
  s.n_completed = 0;
  s.partial_valid = 0;
  s.reserved = 0;
  const int rc = check_store(&s);
  if (rc != ATTNRES_OK) return rc;
  *st = s;
  return ATTNRES_OK;
}

ATTNRES_API int attnres_store_sources(const attnres_store_t* st) {
  const int rc = check_store(st);
  if (rc != ATTNRES_OK) return rc;
  return 1 + st->n_completed + st->partial_valid;
}

ATTNRES_API int attnres_add_rows(const void* a, const void* b, void* out, int64_t T, int32_t d, int32_t dtype,
                                 void* stream) {
  int rc = check_shape(T, d, dtype);
  if (rc != ATTNRES_OK) return rc;
  const int64_t row = T * (int64_t)d;
  if (row == 0) return ATTNRES_OK;
  if (b == nullptr || out == nullptr) return ATTNRES_EINVAL;
  if ((a != nullptr && !aligned16(a)) || !aligned16(b) || !aligned16(out)) return ATTNRES_EUNSUPPORTED;
  const int es = elem_bytes(dtype);
  const Range r_out = range(out, row * es);
  // out may be a itself (in place), not b, and no partial overlap with either
  if (overlap(r_out, range(b, row * es))) return ATTNRES_EALIAS;
  if (a != nullptr && a != out && overlap(r_out, range(a, row * es))) return ATTNRES_EALIAS;
  attnres::AccumulateArgs args;
  args.partial = const_cast<void*>(a);
  args.layer_out = b;
  args.out = out;
  args.elems = row;
  args.bf16 = dtype == ATTNRES_BF16;
  args.copy = a == nullptr;
  (void)hipGetLastError();
  return attnres::launch_accumulate(args, static_cast<hipStream_t>(stream)) == hipSuccess ? ATTNRES_OK
                                                                                          : ATTNRES_ELAUNCH;
}

ATTNRES_API int attnres_accumulate(attnres_store_t* st, const void* layer_out, int32_t finalize_block,
                                   void* stream) {
  int rc = check_store(st);
  if (rc != ATTNRES_OK) return rc;
  if (finalize_block != 0 && finalize_block != 1) return ATTNRES_EINVAL;
  const int slot = 1 + st->n_completed;
  if (slot >= st->s_max) return ATTNRES_ESTATE;
  const int es = elem_bytes(st->dtype);
  const int64_t row = st->T * (int64_t)st->d;
  if (row > 0) {
    if (layer_out == nullptr) return ATTNRES_EINVAL;
    if (!aligned16(layer_out)) return ATTNRES_EUNSUPPORTED;
    const Range r_store = range(st->base, ((int64_t)(st->s_max - 1) * st->slot_stride + row) * es);
    if (overlap(range(layer_out, row * es), r_store)) return ATTNRES_EALIAS;
    attnres::AccumulateArgs a;
    a.partial = static_cast<char*>(st->base) + (int64_t)slot * st->slot_stride * es;
    a.layer_out = layer_out;
    a.out = nullptr;
    a.elems = row;
    a.bf16 = st->dtype == ATTNRES_BF16;
    a.copy = st->partial_valid == 0;
    (void)hipGetLastError();
    if (attnres::launch_accumulate(a, static_cast<hipStream_t>(stream)) != hipSuccess) return ATTNRES_ELAUNCH;
  }
  st->partial_valid = 1;
  if (finalize_block) {
    st->n_completed += 1;
    st->partial_valid = 0;
  }
  return ATTNRES_OK;
}

}  // extern "C"
