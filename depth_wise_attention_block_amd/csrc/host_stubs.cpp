// Host-only build of the C ABI for sanitizer runs (AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU, no GPU).
//
// capi.cpp holds every argument check, the range/alias arithmetic and the
// store bookkeeping; it reaches the kernels only through these launchers.  In
// this build they launch nothing and report that no device is there, so a
// call whose checks pass ends as ATTNRES_ELAUNCH -- the same status a host
// without a GPU gets from the real library, whose device query fails first.
#include "internal.h"

namespace attnres {

hipError_t launch_aggregate(const AggregateArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_accumulate(const AccumulateArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_block_prepare(const PrepareArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_split_queries(const float*, int64_t, int, void*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_block_merge(const MergeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_aggregate_backward(const BackwardArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_block_backward(const BlockBackwardArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_partial_sums(const PartialSumsArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_partial_dw(const PartialDwArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t static_scratch(void**) { return hipErrorNoDevice; }

}  // namespace attnres
