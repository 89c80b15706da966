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
};

void prof_begin(int32_t kernel, hipStream_t stream);
void prof_end(hipStream_t stream);

}  // namespace gdn
