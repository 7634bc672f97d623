// Host-side launcher of the library's measurement helper (internal; the
// public C ABI is include/dsa_indexer.h).
#pragma once

#include <hip/hip_runtime.h>

namespace dsa {

// One launch of a pure FP8 MFMA loop (iters rounds per wave, two waves per
// SIMD); *flops = the FP8 operations it performs.
hipError_t launch_fp8_mfma_rate(int iters, double* flops, hipStream_t stream);

}  // namespace dsa
