// Host-side launchers of the library's measurement helpers (internal; the
// public C ABI is include/dsa_indexer.h).
#pragma once

#include <hip/hip_runtime.h>

namespace dsa {

// One launch of a pure FP8 MFMA loop (iters rounds per wave, two waves per
// SIMD); *flops = the FP8 operations it performs.
hipError_t launch_fp8_mfma_rate(int iters, double* flops, hipStream_t stream);

// One launch reading the n K pages whose ids are ids[0 .. n) whole (ids
// outside [0, num_pages) read nothing), three pages per wave, no compute.
hipError_t launch_page_read(const uint8_t* k_cache, int64_t num_pages,
                            const int32_t* ids, int64_t n, hipStream_t stream);

// Zeroes counts[0..2], then counts the FP8 code mismatches described at
// fp8_cvt_check_kernel / fp8_quotient_check_kernel (device counters).
hipError_t launch_fp8_code_check(unsigned long long* counts,
                                 hipStream_t stream);

}  // namespace dsa
