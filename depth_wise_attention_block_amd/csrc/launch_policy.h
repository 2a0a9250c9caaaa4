// Launch policy of the per-token kernels (the aggregation, its fused update,
// the two-phase pair and the backward): threads, vectors per lane, grid and
// token order.  Host only; the C ABI layer (capi.cpp) calls it after its
// argument checks.  Kept apart from capi.cpp so that the aggregation's
// committed HBM counter bytes name exactly the files its launches depend on.
#pragma once

#include <stdint.h>

#include "attnres.h"
#include "internal.h"

namespace {

// Launch shape: each lane holds V 16-byte vectors of every source row; V is
// the smallest value that keeps the workgroup within kMaxWaves waves.  One
// token per workgroup at a time; the grid covers every token up to a cap.  Past
// the cap the aggregation and the inter-block pass take several launches of at
// most `grid` workgroups (each workgroup handles exactly one token); the other
// kernels loop over tokens.
//
// With xcd_runs (the aggregation kernels), workgroups are dispatched to the 8
// XCDs in turn, and each XCD takes runs of kXcdRun consecutive tokens instead
// of every 8th token: the HBM traffic of one XCD then moves in runs of
// kXcdRun rows of each source (measured at T = 262,144: 3% more bandwidth for
// the aggregation and the fused step; 2.5% for 94 sources at T = 32,768;
// results bit-identical).  Small batches keep one token per XCD in turn,
// where runs would leave workgroups idle.
constexpr int kXcdRunLog2 = 5;                  // runs of 32 tokens
constexpr int64_t kXcdRunMinTokens = 4096;      // from this batch size on
inline int pick_config(int32_t S, int64_t T, int32_t d, int32_t dtype, int32_t num_cus, attnres_launch_t* cfg,
                       bool xcd_runs = false) {
  const int nvec = d / (attnres::kVecBytes / (dtype == ATTNRES_BF16 ? 2 : 4));
  const int max_threads = 64 * attnres::kMaxWaves;
  const int v = (nvec + max_threads - 1) / max_threads;
  if (v < 1 || v > attnres::kMaxVecsPerLane) return ATTNRES_EUNSUPPORTED;
  const int lanes = (nvec + v - 1) / v;
  cfg->threads = (lanes + 63) / 64 * 64;
  cfg->vecs_per_lane = v;
  const int64_t cap = (int64_t)(num_cus > 0 ? num_cus : 256) * 4096;  // a multiple of 8
  cfg->xcd_run = (xcd_runs && T >= kXcdRunMinTokens) ? (1 << kXcdRunLog2) : 1;
  const int64_t span = cfg->xcd_run > 1 ? (T + 8 * cfg->xcd_run - 1) / (8 * cfg->xcd_run) * (8 * cfg->xcd_run) : T;
  cfg->grid = span < cap ? span : cap;
  cfg->tokens_per_group = 1;
  (void)S;
  return ATTNRES_OK;
}

// The merge of the two-phase schedule comes in two forms.  Up to this batch
// size each workgroup takes one token and issues every load of it (the
// query's, the three rows', the logits') before anything waits: one memory
// round trip where the looping form has three, and a decode pass 6-8% faster
// at T = 1..256.  From about 1,024 tokens on the looping form is as fast or
// faster (0.8% at 4,096, 1.6% at 16,384 per schedule pass, measured on one set
// of buffers).
constexpr int64_t kMergePerTokenMaxTokens = 512;
inline bool merge_per_token(int64_t T) { return T <= kMergePerTokenMaxTokens; }

}  // namespace
