// gfx950 kernels for the sparse-attention hand-off, the step after the hot
// path: the top-k rows (logical token positions, ascending, -1 padded) as
// physical cache slots, and as the additive score mask.
//
// Slots (vLLM HBM-index notes, section 2.3): position s of request r is
// slot block_table[r, s / 64] * 64 + s % 64, the slot the write path stored
// the token's key at.  Mask (msmodeling DeepseekV32 RFC, section 2.1.3,
// sparse MLA): 0 at the selected tokens, -inf at every other column of the
// score row, added to q k^T.
#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

// Grid (T, ceil(k / 256)): one thread per top-k entry.
__global__ __launch_bounds__(256) void topk_to_slots_kernel(
    const int32_t* __restrict__ topk, int k, int64_t topk_ld,
    const int32_t* __restrict__ block_table, int64_t bt_stride,
    const int32_t* __restrict__ qsl, int R, int64_t* __restrict__ slots) {
  const int64_t t = blockIdx.x;
  const int j = blockIdx.y * 256 + threadIdx.x;
  if (j >= k) return;
  const int r = request_of_row(qsl, R, t);
  const int idx = topk[t * topk_ld + j];
  int64_t slot = -1;
  if (idx >= 0 && (int64_t)(idx / kPageTokens) < bt_stride) {
    const int page = block_table[(int64_t)r * bt_stride + idx / kPageTokens];
    if (page >= 0) slot = (int64_t)page * kPageTokens + idx % kPageTokens;
  }
  slots[t * (int64_t)k + j] = slot;
}

constexpr int kMaskChunk = 16384;            // columns per workgroup
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int kMaskThreads = 256;

// Grid (T, ceil(ld / 16384)): the workgroup marks the row's selected
// columns that fall in its chunk in an LDS bitmap, then writes the chunk as
// 16-byte stores of 0 / -inf (every column written exactly once, no
// write-after-write between threads).
__global__ __launch_bounds__(kMaskThreads) void topk_mask_kernel(
    const int32_t* __restrict__ topk, int k, int64_t topk_ld,
    float* __restrict__ mask, int64_t ld) {
  __shared__ uint32_t bits[kMaskChunk / 32];
  const int64_t t = blockIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * kMaskChunk;
  const int tid = threadIdx.x;
  for (int w = tid; w < kMaskChunk / 32; w += kMaskThreads) bits[w] = 0u;
  __syncthreads();
  const int32_t* row = topk + t * topk_ld;
  for (int j = tid; j < k; j += kMaskThreads) {
    const int64_t c = (int64_t)row[j] - c0;
    if (row[j] >= 0 && c >= 0 && c < kMaskChunk)
      atomicOr(&bits[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  float* out = mask + t * ld + c0;
#pragma unroll 4
  for (int v = 0; v < kMaskChunk / (4 * kMaskThreads); ++v) {
    const int c = (v * kMaskThreads + tid) * 4;        // 4 columns
    if (c0 + c >= ld) break;                           // ld % 4 == 0
    const uint32_t b = (bits[c >> 5] >> (c & 31)) & 0xfu;
    const float4 val = make_float4((b & 1u) ? 0.f : -INFINITY,
                                   (b & 2u) ? 0.f : -INFINITY,
                                   (b & 4u) ? 0.f : -INFINITY,
                                   (b & 8u) ? 0.f : -INFINITY);
    // non-temporal: the mask is read by the attention later, not here, and
    // caching a stream of this size only displaces other lines (prefill
    // 1.34 GB: 0.295 -> 0.261 ms)
    const f4v nv = {val.x, val.y, val.z, val.w};
    __builtin_nontemporal_store(nv, reinterpret_cast<f4v*>(out + c));
  }
}

hipError_t launch_topk_to_slots(const int32_t* topk, int64_t T, int k,
                                int64_t topk_ld, const int32_t* block_table,
                                int64_t bt_stride, const int32_t* qsl, int R,
                                int64_t* slots, hipStream_t stream) {
  if (T <= 0 || k <= 0) return hipSuccess;
  const dim3 grid((unsigned)T, (unsigned)((k + 255) / 256));
  hipLaunchKernelGGL(topk_to_slots_kernel, grid, dim3(256), 0, stream, topk,
                     k, topk_ld, block_table, bt_stride, qsl, R, slots);
  return hipGetLastError();
}

hipError_t launch_topk_mask(const int32_t* topk, int64_t T, int k,
                            int64_t topk_ld, float* mask, int64_t ld,
                            hipStream_t stream) {
  if (T <= 0 || ld <= 0) return hipSuccess;
  const dim3 grid((unsigned)T, (unsigned)((ld + kMaskChunk - 1) / kMaskChunk));
  hipLaunchKernelGGL(topk_mask_kernel, grid, dim3(kMaskThreads), 0, stream,
                     topk, k, topk_ld, mask, ld);
  return hipGetLastError();
}

}  // namespace dsa
