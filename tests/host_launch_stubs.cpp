// Launch layer stand-in for host-only builds of the C ABI (tests/test_host_sanitizers.py):
// the argument checks, planning and workspace sizing of dcp_api.hip run for real, built
// with AddressSanitizer and UndefinedBehaviorSanitizer, and every kernel launch they
// reach returns an error instead of launching.  Test infrastructure only.
#include "dcp_internal.h"

namespace dcp {
namespace {
hipError_t no_launch() { return hipErrorNotSupported; }
}  // namespace
hipError_t launch_mla_partial(const PartialParams&, hipStream_t) { return no_launch(); }
hipError_t launch_gqa_partial(const PartialParams&, hipStream_t) { return no_launch(); }
hipError_t launch_split_reduce(const SplitReduceParams&, hipStream_t) { return no_launch(); }
hipError_t launch_merge_lse(const float*, int32_t, int64_t, float*, hipStream_t) { return no_launch(); }
hipError_t launch_rescale(const float*, const float*, const float*, int64_t, int32_t, bool, void*,
                          hipStream_t) { return no_launch(); }
hipError_t launch_sum_slice(const void*, bool, int32_t, int64_t, int32_t, int32_t, int32_t, float*,
                            hipStream_t) { return no_launch(); }
hipError_t launch_append(const void*, const void*, void*, void*, int64_t, const int32_t*, int32_t,
                         const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                         hipStream_t) { return no_launch(); }
hipError_t launch_merge(const float*, const float*, int32_t, int64_t, int32_t, float*, float*,
                        hipStream_t) { return no_launch(); }
hipError_t launch_shard_map(const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t*,
                            hipStream_t) { return no_launch(); }
hipError_t launch_zero_fill(void*, size_t, hipStream_t) { return no_launch(); }
hipError_t launch_local_block_table(const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t,
                                    int32_t*, int32_t, hipStream_t) { return no_launch(); }
}  // namespace dcp
