// gfx950 kernel for the second half of the lightning-indexer hot path:
// per-row causal top-k over the fp32 logits, written into the shared int32
// index buffer (vLLM IndexCache practical guide, section 2: the indexer
// clears the buffer rows to -1 and scatters its top-k there; GLM-5.3
// cache-budget article, section on the top-k index buffer:
// [max_num_batched_tokens, index_topk] int32).
//
// Row t reads columns 0..p_t (n = p_t + 1 logits).  If n <= k the row is
// 0..n-1 followed by -1.  Otherwise the k largest logits are selected by a
// radix select on order-preserving 32-bit keys: 12 + 12 + 8 bit digits, each
// pass an LDS histogram (ds_add) followed by a workgroup scan that finds the
// digit holding the k-th largest key.  Keys equal to the final threshold are
// taken lowest index first.  The selected indices are then compacted in
// ascending index order with wave ballots, so every row of the buffer is
// deterministic and sorted by token position; slots [min(n,k), k) hold -1.
//
// One workgroup (16 waves) per row.  The row's keys are cached in LDS when
// they fit (dynamic shared memory sized by the host); longer rows are
// re-read from global memory (L2) in every pass.
#include <algorithm>

#include "dsa_common.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kHistBins = 4096;
constexpr int kMaxCachedKeys = 35840;          // 140 KiB of LDS

struct TopkShared {
  uint32_t hist[kHistBins];
  uint32_t wave_sum[kTopkWaves];
  uint32_t seg_gt[kTopkWaves];
  uint32_t seg_eq[kTopkWaves];
  uint32_t sel_digit, sel_above, sel_count;
};

// Exclusive prefix sum of one value per thread over the workgroup; also
// returns the total.  Contains barriers: call from all threads.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v,
                                                         uint32_t* wave_sum,
                                                         uint32_t* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_sum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t ws = lane < kTopkWaves ? wave_sum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kTopkWaves; off <<= 1) {
      const uint32_t y = __shfl_up(ws, off);
      if (lane >= off) ws += y;
    }
    if (lane < kTopkWaves) wave_sum[lane] = ws;        // inclusive
  }
  __syncthreads();
  const uint32_t before = wave ? wave_sum[wave - 1] : 0u;
  *total = wave_sum[kTopkWaves - 1];
  __syncthreads();
  return before + x - v;
}

// Reads key i of the row: from the LDS cache when i < cached, else global.
struct RowKeys {
  const float* row;
  const uint32_t* cache;
  int cached;
  __device__ __forceinline__ uint32_t operator()(int i) const {
    return i < cached ? cache[i] : float_to_ordered(row[i]);
  }
};

// One radix pass: histogram the digit at `shift` (nbins bins) of the keys
// that match `prefix` under `mask`, then find the digit where the count of
// larger keys first reaches k_rem.  Results land in sh.sel_*.
template <int NBINS>
__device__ void radix_pass(const RowKeys& keys, int n, uint32_t prefix,
                           uint32_t mask, int shift, uint32_t k_rem,
                           TopkShared& sh) {
  const int tid = threadIdx.x;
  for (int b = tid; b < NBINS; b += kTopkThreads) sh.hist[b] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = keys(i);
    if ((key & mask) == prefix)
      atomicAdd(&sh.hist[(key >> shift) & (NBINS - 1)], 1u);
  }
  __syncthreads();
  // Thread t owns BPT bins in descending order starting at the top.
  constexpr int BPT = NBINS >= kTopkThreads ? NBINS / kTopkThreads : 1;
  constexpr int ACTIVE = NBINS / BPT;
  uint32_t local = 0;
  if (tid < ACTIVE) {
#pragma unroll
    for (int j = 0; j < BPT; ++j) local += sh.hist[NBINS - 1 - (tid * BPT + j)];
  }
  uint32_t total;
  const uint32_t above0 = block_exclusive_scan(local, sh.wave_sum, &total);
  if (tid < ACTIVE && above0 < k_rem && above0 + local >= k_rem) {
    uint32_t above = above0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int bin = NBINS - 1 - (tid * BPT + j);
      const uint32_t c = sh.hist[bin];
      if (above + c >= k_rem) {
        sh.sel_digit = (uint32_t)bin;
        sh.sel_above = above;
        sh.sel_count = c;
        break;
      }
      above += c;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(
    const float* __restrict__ logits, int64_t ld,
    const int32_t* __restrict__ positions, int k, int32_t* __restrict__ out,
    int64_t out_ld, int cache_cap) {
  extern __shared__ uint32_t s_cache[];
  __shared__ TopkShared sh;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  int32_t* orow = out + t * out_ld;
  int p = positions[t];
  if (p >= ld) p = (int)ld - 1;              // logits past ld do not exist
  const int n = p + 1;                       // p < 0 -> empty row
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) orow[i] = i < n ? i : -1;
    return;
  }
  const float* row = logits + t * ld;
  const int cached = min(n, cache_cap);
  for (int i = tid; i < cached; i += kTopkThreads)
    s_cache[i] = float_to_ordered(row[i]);
  __syncthreads();
  const RowKeys keys{row, s_cache, cached};

  uint32_t prefix = 0u, mask = 0u, k_rem = (uint32_t)k;
  // pass 1: bits 31..20
  radix_pass<4096>(keys, n, prefix, mask, 20, k_rem, sh);
  prefix = sh.sel_digit << 20; mask = 0xfff00000u;
  k_rem -= sh.sel_above;
  bool done = sh.sel_count == k_rem;
  if (!done) {                               // pass 2: bits 19..8
    radix_pass<4096>(keys, n, prefix, mask, 8, k_rem, sh);
    prefix |= sh.sel_digit << 8; mask = 0xffffff00u;
    k_rem -= sh.sel_above;
    done = sh.sel_count == k_rem;
  }
  if (!done) {                               // pass 3: bits 7..0
    radix_pass<256>(keys, n, prefix, mask, 0, k_rem, sh);
    prefix |= sh.sel_digit; mask = 0xffffffffu;
    k_rem -= sh.sel_above;
  }
  // Selected: (key & mask) > prefix, or (key & mask) == prefix among the
  // first k_rem such keys in index order.  Contiguous per-wave segments.
  const int seg = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
  const int b0 = min(n, wave * seg), b1 = min(n, b0 + seg);
  uint32_t gt = 0, eq = 0;
  for (int i = b0 + lane; i < b1; i += 64) {
    const uint32_t km = keys(i) & mask;
    gt += km > prefix;
    eq += km == prefix;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) { sh.seg_gt[wave] = gt; sh.seg_eq[wave] = eq; }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) { gt_before += sh.seg_gt[w]; eq_before += sh.seg_eq[w]; }
  uint32_t pos = gt_before + min(eq_before, k_rem);
  uint32_t eq_seen = eq_before;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = b0; base < b1; base += 64) {
    const int i = base + lane;
    const bool in = i < b1;
    const uint32_t km = in ? (keys(i) & mask) : 0u;
    const bool is_gt = in && km > prefix;
    const bool is_eq = in && km == prefix;
    const uint64_t eq_mask = __ballot(is_eq);
    const uint32_t eq_rank = eq_seen + (uint32_t)__popcll(eq_mask & below);
    const bool sel = is_gt || (is_eq && eq_rank < k_rem);
    const uint64_t sel_mask = __ballot(sel);
    const uint32_t slot = pos + (uint32_t)__popcll(sel_mask & below);
    if (sel && slot < (uint32_t)k) orow[slot] = i;
    pos += (uint32_t)__popcll(sel_mask);
    eq_seen += (uint32_t)__popcll(eq_mask);
  }
}

size_t topk_workspace_bytes(int64_t T, int64_t ld, int k) {
  (void)T; (void)ld; (void)k;
  return 0;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  const int cap = (int)std::min<int64_t>(a.ld, kMaxCachedKeys);
  const size_t dyn = (size_t)cap * sizeof(uint32_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(topk_row_kernel),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)(kMaxCachedKeys * sizeof(uint32_t)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)a.T), dim3(kTopkThreads),
                     dyn, stream, a.logits, a.ld, a.positions, a.k, a.out,
                     a.out_ld, cap);
  return hipGetLastError();
}

}  // namespace dsa
