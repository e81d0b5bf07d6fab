// Internal interface between the translation units of libstreamkl.so (not part
// of the C ABI and not exported from the library).
#ifndef STREAMKL_INTERNAL_H
#define STREAMKL_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace streamkl_internal {

// Enqueue the deterministic sum of n fp32 values (fixed reduction order, fp64
// accumulation) into the device scalar *out on stream s.
__attribute__((visibility("hidden"))) hipError_t launch_row_sum(const float *x, int64_t n, float *out,
                                                                hipStream_t s);

// True when the STREAMKL_LOG environment variable is set to anything but "0"
// (read once per process): every launch then prints its configuration and
// grid, one line on stderr.
__attribute__((visibility("hidden"))) bool log_enabled();

}  // namespace streamkl_internal

#endif  // STREAMKL_INTERNAL_H
