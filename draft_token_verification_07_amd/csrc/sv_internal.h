// sv_internal.h -- what the kernels add to sv_host.h: the HIP runtime and
// the launch functions of each path.  Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include "sv_host.h"

namespace sv {

hipError_t launch_greedy(const GreedyArgs &a, int dtype, hipStream_t st);
hipError_t launch_seq(const GreedyArgs &a, hipStream_t st);
hipError_t launch_lmhead(const LmheadArgs &a, hipStream_t st);
hipError_t launch_draft(const DraftArgs &a, int dtype, hipStream_t st);
hipError_t launch_count(const int32_t *accept_len, int32_t B, int32_t gamma, unsigned long long *counters,
                        hipStream_t st);
hipError_t launch_fanout(const FanoutArgs &a, hipStream_t st);
hipError_t launch_trim(const TrimArgs &a, hipStream_t st);
hipError_t launch_sample(const SampleArgs &a, int dt_t, int dt_d, hipStream_t st);

}  // namespace sv
