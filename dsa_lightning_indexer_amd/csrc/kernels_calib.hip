// Measurement helper of the gfx950 library (not a step of the indexer hot
// path): the FP8 matrix-core rate this device reaches at the clock it holds
// under a pure MFMA load.  The logits kernels' FP8 rate is then read against
// both the published dense peak and this measured one.
#include "dsa_calib.h"
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

// Results land here only so that the compiler keeps the loop; nobody reads
// them (concurrent launches may overwrite each other: harmless).
__device__ float g_calib_sink[64];

constexpr int kCalibChains = 8;       // independent accumulators per wave

// Every wave runs `iters` rounds of kCalibChains independent 16x16x128 FP8
// MFMAs on register operands: no memory traffic, no LDS, no dependency
// stalls (eight chains cover the instruction's latency).
__global__ __launch_bounds__(256) void fp8_mfma_rate_kernel(int iters) {
  const int lane = lane_id();
  // e4m3 code 0x20 is 0.125: products of 1/64 summed over 128 terms, so the
  // accumulators stay finite for any iteration count this helper accepts
  const int pat = 0x20202020 ^ (lane & 1);
  const i32x8 a = {pat, pat, pat, pat, pat, pat, pat, pat};
  const i32x8 b = {0x20202020, 0x20202020, 0x20202020, 0x20202020,
                   0x20202020, 0x20202020, 0x20202020, 0x20202020};
  f32x4 c[kCalibChains];
#pragma unroll
  for (int j = 0; j < kCalibChains; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kCalibChains; ++j) c[j] = mfma16x16x128_fp8(a, b, c[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kCalibChains; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  g_calib_sink[lane] = s;
}

hipError_t launch_fp8_mfma_rate(int iters, double* flops, hipStream_t stream) {
  // two 4-wave workgroups per compute unit: two waves on every SIMD
  const int64_t wgs = 2 * (int64_t)device_cu_count();
  hipLaunchKernelGGL(fp8_mfma_rate_kernel, dim3((unsigned)wgs), dim3(256), 0,
                     stream, iters);
  *flops = (double)wgs * 4.0 * (double)iters * kCalibChains * 2.0 * 16 * 16 *
           128;
  return hipGetLastError();
}

}  // namespace dsa
