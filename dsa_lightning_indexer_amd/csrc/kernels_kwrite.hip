// gfx950 kernels for the indexer-K write path, the step before the hot
// path: the physical slot of every new token, and the per-token FP8
// quantisation of its key scattered into the paged cache.
//
// Slot (vLLM HBM-index notes, section 2.3): token of request r at position p
// lives at slot block_table[r, p / 64] * 64 + p % 64; the compressed
// variant of a DeepSeek-V4 cache is described at its kernel.  Write (GLM-5.3
// indexer-cache article, section on the indexer cache's write path, and the
// page layout of its eviction section): a token's 128 e4m3fn key bytes go to
// page slot / 64 at row slot % 64, its fp32 scale to byte 8192 + 4 * row of
// the same page; nothing is cleared, a write overwrites the slot.
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

__device__ unsigned g_err_kwrite = 0;

// One thread per token; the request by binary search over query_start_loc.
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ block_table, int64_t bt_stride,
    const int32_t* __restrict__ qsl, int R,
    const int32_t* __restrict__ positions, int64_t T,
    int64_t* __restrict__ slots) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int p = positions[t];
  int64_t slot = -1;
  if (p >= 0 && (int64_t)(p / kPageTokens) < bt_stride) {
    const int r = request_of_row(qsl, R, t);
    const int page = block_table[(int64_t)r * bt_stride + p / kPageTokens];
    if (page >= 0) slot = (int64_t)page * kPageTokens + p % kPageTokens;
  }
  slots[t] = slot;
}

// Compressed slots (vLLM HBM-index notes, sections 5.1-5.2, DeepSeek-V4):
// a token at position p has a slot only when (p + 1) % ratio == 0; it is
// entry c = p / ratio of its request, stored at block_table[r, c / bs] * bs
// + c % bs with bs the entries per storage block (host block / ratio); any
// other token gets -1.  Optionally also the last entry a row can see, the
// row's position in the compressed cache: (p + 1) / ratio - 1 (-1 for p < 0).
__global__ __launch_bounds__(256) void compressed_slot_mapping_kernel(
    const int32_t* __restrict__ block_table, int64_t bt_stride,
    const int32_t* __restrict__ qsl, int R,
    const int32_t* __restrict__ positions, int64_t T, int ratio, int bs,
    int64_t* __restrict__ slots, int32_t* __restrict__ positions_c) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int64_t p = positions[t];              // p + 1 may pass INT32_MAX
  int64_t slot = -1;
  if (p >= 0 && (p + 1) % ratio == 0) {
    const int64_t c = p / ratio;
    if (c / bs < bt_stride) {
      const int r = request_of_row(qsl, R, t);
      const int blk = block_table[(int64_t)r * bt_stride + c / bs];
      if (blk >= 0) slot = (int64_t)blk * bs + c % bs;
    }
  }
  slots[t] = slot;
  if (positions_c)
    positions_c[t] = p >= 0 ? (int32_t)((p + 1) / ratio - 1) : -1;
}

// 16 lanes per token, 8 bf16 values per lane (one 16-byte load):
//   amax = max |k|, s = amax / 448 (IEEE fp32 division), code = e4m3fn(k / s)
//   (round to nearest even, saturating; for a finite key with s >= 2^-100
//   from the reciprocal quotient and the hardware conversion, which give the
//   IEEE quotient's codes); an all-zero key stores s = 0 and zero codes.
// Lane i of the token's group writes key bytes 8 i .. 8 i + 7 (the group
// writes the 128-byte row in one coalesced store) and lane 0 the scale.  A
// negative slot writes nothing; a slot past the pool raises the page flag.
__global__ __launch_bounds__(256) void k_write_kernel(
    const uint16_t* __restrict__ k, int64_t N,
    const int64_t* __restrict__ slots, uint8_t* __restrict__ k_cache,
    int64_t num_pages) {
  const int64_t tok = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (tok >= N) return;                      // whole 16-lane groups exit
  const int64_t slot = slots[tok];
  const uint4 raw = *reinterpret_cast<const uint4*>(k + tok * kHeadDim + sub * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  float amax = 0.f;
  uint32_t abits = 0u;                       // largest |k| bit pattern
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    amax = fmaxf(amax, fabsf(f[i]));
    abits = max(abits, __float_as_uint(f[i]) & 0x7fffffffu);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    abits = max(abits, (uint32_t)__shfl_xor((int)abits, off, 16));
  }
  if (slot < 0) return;                      // padding token (group-uniform)
  if (slot >= num_pages * kPageTokens) {
    if (sub == 0) atomicOr(&g_err_kwrite, kErrPageOutOfRange);
    return;
  }
  const float s = amax / kE4M3Max;
  uint32_t lo = 0, hi = 0;
  if (abits < 0x7f800000u && s >= 0x1p-100f) {
    // finite key, scale not tiny: the reciprocal quotient and the hardware
    // conversion give the same codes as the IEEE quotient and the integer
    // encoder (dsa_fp8_code_check)
    const float r = 1.0f / s;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = div_by_scale(f[i], s, r);
    lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
        y[2], y[3], __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false),
        true);
    hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
        y[6], y[7], __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false),
        true);
  } else if (s > 0.f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3fn_encode(f[i] / s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3fn_encode(f[4 + i] / s) << (8 * i);
  }
  uint8_t* page = k_cache + (slot / kPageTokens) * kPageBytes;
  const int row = (int)(slot % kPageTokens);
  *reinterpret_cast<uint2*>(page + row * kHeadDim + sub * 8) = make_uint2(lo, hi);
  if (sub == 0)
    *reinterpret_cast<float*>(page + kPageKeyBytes + row * 4) = s;
}

hipError_t launch_slot_mapping(const int32_t* block_table, int64_t bt_stride,
                               const int32_t* qsl, int R,
                               const int32_t* positions, int64_t T,
                               int64_t* slots, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t grid = (T + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)grid), dim3(256), 0,
                     stream, block_table, bt_stride, qsl, R, positions, T,
                     slots);
  return hipGetLastError();
}

hipError_t launch_compressed_slot_mapping(
    const int32_t* block_table, int64_t bt_stride, const int32_t* qsl, int R,
    const int32_t* positions, int64_t T, int ratio, int block_size,
    int64_t* slots, int32_t* positions_c, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t grid = (T + 255) / 256;
  hipLaunchKernelGGL(compressed_slot_mapping_kernel, dim3((unsigned)grid),
                     dim3(256), 0, stream, block_table, bt_stride, qsl, R,
                     positions, T, ratio, block_size, slots, positions_c);
  return hipGetLastError();
}

hipError_t launch_k_write(const uint16_t* k, int64_t N, const int64_t* slots,
                          uint8_t* k_cache, int64_t num_pages,
                          hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const int64_t grid = (N + 15) / 16;
  hipLaunchKernelGGL(k_write_kernel, dim3((unsigned)grid), dim3(256), 0,
                     stream, k, N, slots, k_cache, num_pages);
  return hipGetLastError();
}

hipError_t read_kwrite_flags(unsigned* flags, bool reset) {
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_err_kwrite),
                                     sizeof(unsigned), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess || !reset) return e;
  const unsigned zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_err_kwrite), &zero, sizeof(unsigned),
                           0, hipMemcpyHostToDevice);
}

}  // namespace dsa
