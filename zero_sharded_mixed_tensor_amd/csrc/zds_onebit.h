// Launchers of the 1-bit codec kernels (arguments already validated).
#pragma once

#include "zds_internal.h"

namespace zds {

// chunk is 1024, 2048, 4096, 8192 or 16384; err may be null.
zds_status launch_onebit_encode(const float *x, float *err, int64_t n, int32_t chunk, uint32_t *words, float *scales,
                                hipStream_t s);
zds_status launch_onebit_decode(const uint32_t *const *words, const float *const *scales, int32_t npeers, int64_t n,
                                int32_t chunk, float *dst, bool accumulate, hipStream_t s);

}  // namespace zds
