// Internal interface between the C-ABI layer (capi.cpp) and the HIP kernels.
// Arguments reaching these launchers have already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

// Bytes per load/store vector: every global access is a 16-byte vector.
constexpr int kVecBytes = 16;
// Most waves (64 lanes each) one aggregation workgroup uses.
constexpr int kMaxWaves = 8;
// Most 16-byte vectors of one source row a lane holds.
constexpr int kMaxVecsPerLane = 4;
// Most sources one aggregation takes (batched online softmax beyond 9).
constexpr int kMaxSourcesMany = 256;
// Two-phase schedule: inter-block sources and layer queries per pass.
constexpr int kMaxInterSources = 8;
constexpr int kMaxBlockQueries = 16;

struct AggregateArgs {
  const void* sources;  // [S][T][d], source s at element offset s*src_stride
  int S;
  int64_t T;
  int d;
  int64_t src_stride;   // elements between sources
  const float* w;       // [d]
  void* out;            // [T][d]
  float* weights;       // [T][S] or nullptr
  float eps;
  bool bf16;
  int threads;          // multiple of 64, <= 64*kMaxWaves
  int vecs_per_lane;    // 1..kMaxVecsPerLane
  int64_t grid;         // a multiple of 8 when xcd_run > 1
  int xcd_run = 1;      // tokens per XCD run, a power of two (see xcd_token)
  // Fused partial-sum update of the last source (index S-1) before use:
  // kCopyUpdate: slot = layer_out; kAddUpdate: slot = slot + layer_out.
  enum Update { kNoUpdate = 0, kCopyUpdate = 1, kAddUpdate = 2 };
  Update update = kNoUpdate;
  const void* layer_out = nullptr;  // [T][d], with update only
};

// Enqueue one aggregation; returns the hipError_t of the launch.
hipError_t launch_aggregate(const AggregateArgs& a, hipStream_t stream);

struct AccumulateArgs {
  void* partial;        // [T][d] slot (read unless copy)
  const void* layer_out;// [T][d]
  void* out;            // [T][d] result; nullptr = in place over partial
  int64_t elems;        // T*d
  bool bf16;
  bool copy;            // true: partial = layer_out (first layer of a block)
};

hipError_t launch_accumulate(const AccumulateArgs& a, hipStream_t stream);

// Phase 1 of the two-phase schedule: one pass over a block's inter-block
// sources (bf16 store) for B layer queries.
struct PrepareArgs {
  void* store;          // slot 0
  int64_t slot_stride;  // elements
  int K;                // inter-block sources, slots [0, K)
  int B;                // queries
  int64_t T;
  int d;
  const void* w_split;  // [B][2][d] bf16: query b's hi row, then its lo row
  void* inter;          // [B] rows of [T][d] bf16 at inter_stride elements
  int64_t inter_stride;
  float* logits;        // [B][T][K]
  float* weights0;      // [T][K] or nullptr
  float eps;
  enum Close { kNone = 0, kCopy = 1, kAdd = 2 };
  Close close;          // form slot K-1 from layer_out first (closing a block)
  const void* layer_out;
  int threads, vecs_per_lane;
  int64_t grid;
};

hipError_t launch_block_prepare(const PrepareArgs& a, hipStream_t stream);

// Split float32 queries [n][d] into bf16 hi and lo rows [n][2][d], w ~ hi + lo.
hipError_t launch_split_queries(const float* w, int64_t n, int d, void* out, hipStream_t stream);

// Phase 2: one later layer of the block.
struct MergeArgs {
  void* slot;           // the partial slot [T][d]
  const void* layer_out;
  bool add;             // slot = slot + layer_out (else slot = layer_out)
  const void* inter;    // R row [T][d]
  const float* logits;  // [T][K]
  int K;
  int64_t T;
  int d;
  const float* w;       // [d]
  void* out;            // [T][d]; may be `inter` itself
  float* weights;       // [T][K+1] or nullptr
  float eps;
  int threads, vecs_per_lane;
  int64_t grid;
  bool per_token = false;  // one workgroup per token, every load issued up front
};

hipError_t launch_block_merge(const MergeArgs& a, hipStream_t stream);

// Backward of one aggregation: float32 source gradients (written or added per
// source), dL/dw via one float32 row per workgroup in `workspace` reduced in a
// fixed order, and optionally the last source's new gradient in the source
// dtype.
struct BackwardArgs {
  const void* sources;
  int S;
  int64_t T;
  int d;
  int64_t src_stride;     // elements
  const void* last_source;// source S-1 at this address instead, or nullptr
  const float* w;
  const void* grad_out;   // [T][d], source dtype
  float* grad_sources;    // S rows of [T][d] at grad_stride floats
  int64_t grad_stride;
  unsigned acc_mask;      // bit s: add into row s
  unsigned defer_mask;    // bit s: leave row s, write source s's coefficients instead
  float* coef;            // [T] x coef_stride floats: (a, c1, c3) of deferred source s at 3s
  int64_t coef_stride;
  void* grad_last;        // [T][d] source dtype, or nullptr
  float* grad_w;          // [d]
  float* workspace;       // grid rows of [d]
  float eps;
  bool bf16;
  bool last_only;         // every row but the last deferred: the streaming kernel
  bool form_dw;           // dL/dw summed here; else every source's coefficients
                          // are written and the grid is one workgroup per token
  int threads, vecs_per_lane;
  int64_t grid;
};

hipError_t launch_aggregate_backward(const BackwardArgs& a, hipStream_t stream);

// The dL/dw rows of attnres_aggregate_backward_static: a file-scope device array
// of this many bytes (ATTNRES_STATIC_SCRATCH_BYTES) in backward.hip.
constexpr int64_t kStaticScratchBytes = INT64_C(16) << 20;
// Its address on the current device: looked up once per device
// (hipGetSymbolAddress, with that device current) and kept.
hipError_t static_scratch(void** ptr);

// The deferred inter-block gradients of one block (see block_backward_kernel).
constexpr int kMaxBlockLayers = 16;
struct BlockRows {
  const void* g[kMaxBlockLayers];    // dL/dr of the block's layers, [T][d] source dtype
  const float* w[kMaxBlockLayers];   // their queries, [d] float32
};
// Output rows of a per-layer reduction (one [d] float32 row per layer).
struct OutRows {
  float* p[kMaxBlockLayers];
};

// The deferred sources' dL/dw share is an MFMA contraction over column blocks of
// kBlockDwCols and `dw_groups` strided token groups.
constexpr int kBlockDwCols = 512;

struct BlockBackwardArgs {
  const void* sources;    // n inter-block rows at src_stride elements
  int n;
  int64_t T;
  int d;
  int64_t src_stride;
  BlockRows rows;
  int B;
  const float* coef;      // [T][B][coef_layer]: layer l's n triples at l * coef_layer
  int coef_layer;         // floats per layer and token, >= 3n
  float* grad_sources;    // n rows of [T][d] float32 at grad_stride floats
  int64_t grad_stride;
  unsigned acc_mask;
  void* grad_last;        // [T][d] source dtype: the new row n-1, or nullptr
  OutRows grad_w;         // B rows [d] float32, each added to
  float* workspace;       // [dw_groups][B][d] float32
  bool bf16;
  int threads, vecs_per_lane;
  int64_t grid;           // workgroups of the gradient-row pass
  int dw_colblocks;       // ceil(d / kBlockDwCols)
  int64_t dw_groups;      // token groups of the dL/dw pass
};

hipError_t launch_block_backward(const BlockBackwardArgs& a, hipStream_t stream);

// Each layer's dL/dw share from a row of its own: x[l] ([T][d] source dtype, or
// nullptr for none) weighted per token by c[l][t * coef_stride].
struct DwRows {
  const void* x[kMaxBlockLayers];
  const float* c[kMaxBlockLayers];
};
// threads of a partial_dw workgroup: its column block is this many 16-byte vectors
constexpr int kPartialDwThreads = 128;
struct PartialDwArgs {
  DwRows rows;
  int B;
  int64_t T;
  int d;
  int64_t coef_stride;    // floats between consecutive tokens' coefficients
  OutRows out;            // B rows [d] float32, overwritten
  float* workspace;       // [groups][B][d] float32
  bool bf16;
  int colblocks;          // ceil(vectors per row / kPartialDwThreads)
  int64_t groups;         // strided token groups
};

hipError_t launch_partial_dw(const PartialDwArgs& a, hipStream_t stream);


// Running partial sums of up to kMaxBlockLayers rows (rows.g holds the inputs).
struct PartialSumsArgs {
  BlockRows rows;
  int count;
  int64_t elems;        // T*d
  void* out;            // count rows at out_stride elements
  int64_t out_stride;
  bool bf16;
};

hipError_t launch_partial_sums(const PartialSumsArgs& a, hipStream_t stream);


}  // namespace attnres
