// Measurement and check helpers of the gfx950 library (not steps of the
// indexer hot path): the FP8 matrix-core rate this device reaches at the
// clock it holds under a pure MFMA load, the time a bare read of a batch's K
// pages takes, and an exhaustive check of the FP8 code arithmetic the q
// quantisation's fast path relies on.  The logits kernels' rates are read against the published peaks
// and against these measured ones.
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

constexpr int kReadPagesPerWave = 3;

// Wave w reads pages ids[3 w .. 3 w + 2] whole (8448 bytes each: 8 loads of
// 1 KB contiguous per page, then its 256 scale bytes), all before the first
// result is used; an id outside [0, num_pages) reads nothing.  The words are
// folded into one value, kept only so that the loads are not dropped.
__global__ __launch_bounds__(64) void page_read_kernel(
    const uint8_t* __restrict__ k_cache, int64_t num_pages,
    const int32_t* __restrict__ ids, int64_t n) {
  const int lane = lane_id();
  const int64_t w = blockIdx.x;
  uint32_t acc = 0u;
  uint4 v[kReadPagesPerWave][8];
  uint32_t sc[kReadPagesPerWave];
#pragma unroll
  for (int q = 0; q < kReadPagesPerWave; ++q) {
    const int64_t i = w * kReadPagesPerWave + q;
    const int page = i < n ? load_uniform(ids, i) : -1;
    const bool ok = page >= 0 && (int64_t)page < num_pages;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        k_cache + (int64_t)(ok ? page : 0) * kPageBytes, ok ? kPageBytes : 0);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const auto x =
          __builtin_amdgcn_raw_buffer_load_b128(rs, 1024 * c + 16 * lane, 0, 0);
      v[q][c] = make_uint4(x[0], x[1], x[2], x[3]);
    }
    sc[q] = __builtin_amdgcn_raw_buffer_load_b32(rs, kPageKeyBytes + 4 * lane,
                                                 0, 0);
  }
#pragma unroll
  for (int q = 0; q < kReadPagesPerWave; ++q) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc ^= v[q][c].x ^ v[q][c].y ^ v[q][c].z ^ v[q][c].w;
    acc ^= sc[q];
  }
  if (acc == 0x9e3779b9u) g_calib_sink[lane] = (float)acc;
}

hipError_t launch_page_read(const uint8_t* k_cache, int64_t num_pages,
                            const int32_t* ids, int64_t n,
                            hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t waves = (n + kReadPagesPerWave - 1) / kReadPagesPerWave;
  hipLaunchKernelGGL(page_read_kernel, dim3((unsigned)waves), dim3(64), 0,
                     stream, k_cache, num_pages, ids, n);
  return hipGetLastError();
}

// FP8 code checks behind the q quantisation's fast path (counts[0..2]):
// [0] fp32 values with |x| < 464 (all a quotient q / s with |q| <= amax can
// round to) whose hardware e4m3 conversion differs from e4m3fn_encode;
// [1] bf16 pairs (q, amax), amax finite and positive, |q| <= amax, s =
// amax / 448 >= 2^-100, where div_by_scale differs from the IEEE quotient;
// [2] those pairs where the hardware code of div_by_scale differs from the
// integer code of the IEEE quotient (the one that matters).
// Thread t of workgroup b checks the 16 bit patterns base + 16 (256 b + t)
// + 0..15.
constexpr int kCvtPerThread = 16;
__global__ __launch_bounds__(256) void fp8_cvt_check_kernel(
    uint64_t base, unsigned long long* counts) {
  const uint64_t i0 = base + ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) *
                                 kCvtPerThread;
  unsigned long long n = 0;
  for (int k = 0; k < kCvtPerThread; ++k) {
    const uint64_t i = i0 + k;
    const uint32_t bits = (uint32_t)i;
    const uint32_t a = bits & 0x7fffffffu;
    if (i >= (1ull << 32) || a >= 0x43e80000u) continue;  // |x| >= 464, NaN
    const float x = __uint_as_float(bits);
    const uint32_t hw =
        (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xffu;
    n += hw != e4m3fn_encode(x) ? 1 : 0;
  }
  if (n) atomicAdd(&counts[0], n);
}

// Workgroup y: amax = bf16 bits (amax0 + y); thread t: q bits t, t + 256, ..
__global__ __launch_bounds__(256) void fp8_quotient_check_kernel(
    uint32_t amax0, unsigned long long* counts) {
  const uint32_t ah = amax0 + blockIdx.x;
  if (ah == 0u || ah > 0x7f7fu) return;                // positive finite
  const float amax = __uint_as_float(ah << 16);
  const float s = amax / kE4M3Max;
  if (!(s >= 0x1p-100f)) return;
  const float r = 1.0f / s;
  unsigned long long nq = 0, nc = 0;
  for (uint32_t qh = threadIdx.x; qh < 65536u; qh += 256u) {
    const float q = __uint_as_float(qh << 16);
    if (!(fabsf(q) <= amax)) continue;                 // also drops NaN
    const float ref = q / s;
    const float y = div_by_scale(q, s, r);
    nq += __float_as_uint(y) != __float_as_uint(ref) ? 1 : 0;
    const uint32_t hw =
        (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xffu;
    nc += hw != e4m3fn_encode(ref) ? 1 : 0;
  }
  if (nq) atomicAdd(&counts[1], nq);
  if (nc) atomicAdd(&counts[2], nc);
}

__global__ void zero_counts_kernel(unsigned long long* counts, int n) {
  if ((int)threadIdx.x < n) counts[threadIdx.x] = 0ull;
}

hipError_t launch_fp8_code_check(unsigned long long* counts,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, stream, counts,
                     3);
  const uint64_t chunk = 1ull << 30;
  for (uint64_t b = 0; b < (1ull << 32); b += chunk)
    hipLaunchKernelGGL(fp8_cvt_check_kernel,
                       dim3((unsigned)(chunk / (256 * kCvtPerThread))),
                       dim3(256), 0, stream, b, counts);
  hipLaunchKernelGGL(fp8_quotient_check_kernel, dim3(0x7f80u), dim3(256), 0,
                     stream, 0u, counts);
  return hipGetLastError();
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
