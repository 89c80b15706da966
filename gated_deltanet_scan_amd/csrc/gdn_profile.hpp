// gdn_profile.hpp -- launch hooks of the optional per-kernel timing.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace gdn {

// Kernel identifiers reported by gdn_profile_collect().
enum ProfKernel : int32_t {
    PROF_CHUNK_TABLE = 0,
    PROF_PREP = 1,
    PROF_SCAN = 2,
    PROF_DECODE = 3,
    PROF_SNAPSHOT = 4,
    PROF_NORM = 5,
    PROF_CONV = 6,
    PROF_CONV_STATE = 7,
    // which chunk-scan kernel a PROF_SCAN launch ran (each such launch also counts as PROF_SCAN)
    PROF_SCAN_ROWS = 8,    // gdn_chunk_scan_rows_kernel
    PROF_SCAN_WIDE = 9,    // gdn_chunk_scan_bf16_kernel
    PROF_SCAN_PLAIN = 10,  // gdn_chunk_scan_kernel
    PROF_SCAN_TFORM = 11,  // gdn_chunk_scan_tform_kernel
    PROF_SHORT = 12,       // gdn_short_prefill_kernel (token-recurrent prefill of short sequences)
};

// Start and stop events for one launch of `kernel`: both null while timing is
// off.  The launch sites pass them to hipExtLaunchKernelGGL, which stamps the
// kernel's own start and end (dispatch to completion) into them.
struct ProfEvents {
    hipEvent_t start, stop;
};
// `variant` (default: none) names the kernel behind a family identifier such as PROF_SCAN;
// gdn_profile_collect() of either identifier counts the launch.
ProfEvents prof_events(int32_t kernel, int32_t variant = -1);

}  // namespace gdn
