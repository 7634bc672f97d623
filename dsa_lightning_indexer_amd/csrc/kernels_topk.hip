// gfx950 kernel for the second half of the lightning-indexer hot path:
// per-row causal top-k over the fp32 logits, written into the shared int32
// index buffer (vLLM IndexCache practical guide, section 2: the indexer
// clears the buffer rows to -1 and scatters its top-k there; GLM-5.3
// cache-budget article, section on the top-k index buffer:
// [max_num_batched_tokens, index_topk] int32).
//
// Row t reads columns 0..p_t (n = p_t + 1 logits).  If n <= k the row is
// 0..n-1 followed by -1.  Otherwise the k largest logits are selected on
// order-preserving 32-bit keys (larger float -> larger key, -0 folded onto
// +0), ties at the k-th value taken lowest index first, and the selected
// indices are written in ascending index order, so every row is
// deterministic and sorted by token position.
//
// One workgroup (16 waves) per row:
//   1. one sweep over the row builds a 4096-bin LDS histogram of the top 12
//      key bits (and caches the keys in LDS while they fit);
//   2. a two-barrier workgroup scan finds the bin d holding the k-th largest
//      key;
//   3. a second sweep counts, per wave segment, the keys whose top bits
//      exceed d (all selected) and collects the keys of bin d (typically a
//      few dozen to a few hundred) into an LDS candidate list;
//   4. up to two more radix passes over the candidates only (bits 19..8,
//      then 7..0) find the exact threshold key T; candidates above T are
//      marked selected in an LDS bitmap, candidates equal to T marked as
//      ties, of which the lowest-index ones are taken;
//   5. each wave writes its segment's selected indices at the segment's
//      offset, compacted with ballots.
// When bin d holds more candidates than the list can take (heavy ties), or
// the row is longer than the bitmaps cover, the row falls back to a full
// 12+12+8-bit radix select over the row.
#include <algorithm>
#include <cmath>
#include <atomic>
#include <type_traits>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "dsa_score.h"
#include "dsa_topk_reg.h"

namespace dsa {

constexpr int kCandMax = 2048;
constexpr int kMaxRowForBitmap = 65536;        // bitmap of 2048 words
constexpr int kBitmapWords = kMaxRowForBitmap / 32;
constexpr int kMaxCachedHi = 48128;            // 94 KiB: top 16 key bits
constexpr int kMaxCachedFull = 23552;          // 92 KiB: whole 32-bit keys

// plim of a launch: ld, or the tighter bound the caller gives.
static int pos_limit(const TopkArgs& a) {
  const int64_t lim = a.pos_limit > 0 ? std::min(a.pos_limit, a.ld) : a.ld;
  return (int)std::min<int64_t>(lim, INT32_MAX);
}

struct TopkShared {
  uint32_t hist[kHistBins];                    // pass 1 and fallback passes
  uint32_t hist1[kHistBins];                   // candidate pass on bits 19..8
  uint32_t cand_key[kCandMax];
  uint32_t cand_idx[kCandMax];
  uint32_t selbits[kBitmapWords];              // candidate above threshold
  uint32_t tiebits[kBitmapWords];              // candidate equal to threshold
  uint32_t wave_sum[kTopkWaves];
  uint32_t seg_cnt[kTopkWaves];
  uint32_t seg_eq[kTopkWaves];
  uint32_t sel_digit, sel_above, sel_count, ncand;
};

// Strided sweep over [i0, i1) by all NT threads of the workgroup with U
// loads in flight per thread: fn(i, value) for every element.  Indices past
// the end are clamped to the last element, so every load is in bounds and
// unconditional (no branch between issue and use).
template <int U, int NT, typename Load, typename Fn>
__device__ __forceinline__ void block_sweep(int i0, int i1, Load load, Fn fn) {
  const int tid = threadIdx.x;
  for (int base = i0; base < i1; base += NT * U) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load(min(base + u * NT + tid, i1 - 1));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NT + tid;
      if (i < i1) fn(i, v[u]);
    }
  }
}

// In-order sweep of one wave's segment [s0, s1): U groups of 64 consecutive
// elements are loaded (clamped, unconditional) before any is used;
// fn(i, in_range, value) runs for every lane of every group (wave-uniform
// control flow, so fn may ballot).
template <int U, typename Load, typename Fn>
__device__ __forceinline__ void wave_sweep(int s0, int s1, Load load, Fn fn) {
  const int lane = lane_id();
  for (int base = s0; base < s1; base += 64 * U) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load(min(base + 64 * u + lane, s1 - 1));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + 64 * u + lane;
      fn(i, i < s1, v[u]);
    }
  }
}

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
    return (cache && i < cached) ? cache[i] : float_to_ordered(row[i]);
  }
};

// Given a filled histogram, find the bin where the count of larger keys
// first reaches k_rem (bins scanned from the top).  Results in sh.sel_*.
template <int NBINS>
__device__ void select_bin(uint32_t k_rem, TopkShared& sh) {
  const int tid = threadIdx.x;
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

// Histogram the digit at `shift` of the keys matching prefix under mask.
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
  select_bin<NBINS>(k_rem, sh);
}

// Fallback: full radix select from pass 2 on (pass 1 already in sh.sel_*),
// then ordered compaction taking equal keys lowest index first.
__device__ void topk_radix_rest(const RowKeys& keys, int n, int k,
                                int32_t* orow, TopkShared& sh) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  uint32_t prefix = sh.sel_digit << 20, mask = 0xfff00000u;
  uint32_t k_rem = (uint32_t)k - sh.sel_above;
  bool done = sh.sel_count == k_rem;
  __syncthreads();
  if (!done) {
    radix_pass<4096>(keys, n, prefix, mask, 8, k_rem, sh);
    prefix |= sh.sel_digit << 8; mask = 0xffffff00u;
    k_rem -= sh.sel_above;
    done = sh.sel_count == k_rem;
    __syncthreads();
  }
  if (!done) {
    radix_pass<256>(keys, n, prefix, mask, 0, k_rem, sh);
    prefix |= sh.sel_digit; mask = 0xffffffffu;
    k_rem -= sh.sel_above;
  }
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
  if (lane == 0) { sh.seg_cnt[wave] = gt; sh.seg_eq[wave] = eq; }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) { gt_before += sh.seg_cnt[w]; eq_before += sh.seg_eq[w]; }
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

// KEY32: rows short enough to cache whole keys in LDS (no reload of the
// candidates' keys); otherwise the top 16 key bits are cached.
template <bool KEY32>
__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(
    const float* __restrict__ logits, int64_t ld,
    const int32_t* __restrict__ positions, int k, int32_t* __restrict__ out,
    int64_t out_ld, int cache_cap, int plim) {
  using CacheT = typename std::conditional<KEY32, uint32_t, uint16_t>::type;
  extern __shared__ __align__(16) unsigned char s_raw[];
  CacheT* s_hi = reinterpret_cast<CacheT*>(s_raw);
  constexpr int kDigShift = KEY32 ? 20 : 4;   // digit = top 12 key bits
  __shared__ TopkShared sh;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  int32_t* orow = out + t * out_ld;
  // p < 0 or p >= plim (a position the logits call does not score):
  // empty row, all -1
  const int n = row_len_of(positions[t], plim);
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) orow[i] = i < n ? i : -1;
    return;
  }
  const float* row = logits + t * ld;
  const int cached = min(n, cache_cap);

  // 0. clear
  for (int b = tid; b < kHistBins; b += kTopkThreads) {
    sh.hist[b] = 0u;
    sh.hist1[b] = 0u;
  }
  for (int b = tid; b < kBitmapWords; b += kTopkThreads) {
    sh.selbits[b] = 0u;
    sh.tiebits[b] = 0u;
  }
  if (tid < kTopkWaves) { sh.seg_cnt[tid] = 0u; sh.seg_eq[tid] = 0u; }
  if (tid == 0) sh.ncand = 0u;
  __syncthreads();
  // 1. histogram of the top 12 key bits; cache the top 16 bits
  block_sweep<8, kTopkThreads>(
      0, n, [&](int i) { return float_to_ordered(row[i]); },
      [&](int i, uint32_t key) {
        if (i < cached) s_hi[i] = (CacheT)(KEY32 ? key : key >> 16);
        atomicAdd(&sh.hist[key >> 20], 1u);
      });
  __syncthreads();
  // 2. the bin holding the k-th largest key
  topk_select_bin<kHistBins, kTopkThreads>(sh.hist, (uint32_t)k, sh);
  const uint32_t d = sh.sel_digit;
  const uint32_t k_rem = (uint32_t)k - sh.sel_above;
  const uint32_t c = sh.sel_count;
  if (c > (uint32_t)kCandMax || n > kMaxRowForBitmap) {
    const RowKeys keys{row, nullptr, 0};       // full keys from global
    topk_radix_rest(keys, n, k, orow, sh);     // heavy ties or very long row
    return;
  }
  // 3. per-segment counts of keys above bin d; collect the indices of bin d
  const int seg = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
  const int b0 = min(n, wave * seg), b1 = min(n, b0 + seg);
  uint32_t gt = 0;
  auto lds_hi = [&](int i) { return (uint32_t)s_hi[i]; };
  auto glb_hi = [&](int i) {
    return KEY32 ? float_to_ordered(row[i]) : float_to_ordered(row[i]) >> 16;
  };
  const int bm = min(max(b0, cached), b1);   // [b0, bm) cached, [bm, b1) not
  auto collect = [&](int i, bool in, uint32_t hi) {
    if (!in) return;
    const uint32_t dig = hi >> kDigShift;
    gt += dig > d;
    if (dig == d) {
      const uint32_t slot = atomicAdd(&sh.ncand, 1u);
      if (slot < (uint32_t)kCandMax) {
        sh.cand_idx[slot] = (uint32_t)i;
        if (KEY32) sh.cand_key[slot] = hi;
      }
    }
  };
  wave_sweep<8>(b0, bm, lds_hi, collect);
  wave_sweep<8>(bm, b1, glb_hi, collect);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) gt += __shfl_xor(gt, off);
  if (lane == 0) atomicAdd(&sh.seg_cnt[wave], gt);
  __syncthreads();
  // full keys of the candidates, all loads in flight together
  if (!KEY32) {
    const uint32_t ncl = min(sh.ncand, (uint32_t)kCandMax);
    const uint32_t j0 = tid, j1 = tid + kTopkThreads;
    const float f0 = row[j0 < ncl ? sh.cand_idx[j0] : 0];
    const float f1 = row[j1 < ncl ? sh.cand_idx[j1] : 0];
    if (j0 < ncl) sh.cand_key[j0] = float_to_ordered(f0);
    if (j1 < ncl) sh.cand_key[j1] = float_to_ordered(f1);
  }
  __syncthreads();
  // 4. exact threshold among the candidates: (key & mask) > thr is taken,
  //    (key & mask) == thr is a tie, k_tie of the ties are taken by index.
  const uint32_t nc = min(sh.ncand, (uint32_t)kCandMax);
  uint32_t mask = 0u, thr = 0u, k_tie = k_rem;  // all candidates tie
  if (k_rem < nc) {
    for (uint32_t j = tid; j < nc; j += kTopkThreads)
      atomicAdd(&sh.hist1[(sh.cand_key[j] >> 8) & 0xfffu], 1u);
    for (int b = tid; b < 256; b += kTopkThreads) sh.hist[b] = 0u;
    __syncthreads();
    topk_select_bin<kHistBins, kTopkThreads>(sh.hist1, k_rem, sh);
    const uint32_t p24 = (d << 12) | sh.sel_digit;
    const uint32_t k2 = k_rem - sh.sel_above;
    mask = 0xffffff00u; thr = p24 << 8; k_tie = k2;
    if (sh.sel_count != k2) {
      for (uint32_t j = tid; j < nc; j += kTopkThreads) {
        const uint32_t key = sh.cand_key[j];
        if ((key >> 8) == p24) atomicAdd(&sh.hist[key & 0xffu], 1u);
      }
      __syncthreads();
      topk_select_bin<256, kTopkThreads>(sh.hist, k2, sh);
      mask = 0xffffffffu; thr = (p24 << 8) | sh.sel_digit;
      k_tie = k2 - sh.sel_above;
    }
  }
  for (uint32_t j = tid; j < nc; j += kTopkThreads) {
    const uint32_t km = sh.cand_key[j] & mask, ij = sh.cand_idx[j];
    if (km > thr) {
      atomicOr(&sh.selbits[ij >> 5], 1u << (ij & 31));
      atomicAdd(&sh.seg_cnt[ij / (uint32_t)seg], 1u);
    } else if (km == thr) {
      atomicOr(&sh.tiebits[ij >> 5], 1u << (ij & 31));
      atomicAdd(&sh.seg_eq[ij / (uint32_t)seg], 1u);
    }
  }
  __syncthreads();
  // 5. ordered write of this wave's segment
  uint32_t pos = 0, tie_seen = 0;
  for (int w = 0; w < wave; ++w) { pos += sh.seg_cnt[w]; tie_seen += sh.seg_eq[w]; }
  pos += min(tie_seen, k_tie);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto emit = [&](int i, bool in, uint32_t hi) {
    bool sel = false, tie = false;
    if (in) {
      const uint32_t dig = hi >> kDigShift;
      sel = dig > d;
      if (dig == d) {
        sel = (sh.selbits[i >> 5] >> (i & 31)) & 1u;
        tie = (sh.tiebits[i >> 5] >> (i & 31)) & 1u;
      }
    }
    const uint64_t tie_mask = __ballot(tie);
    const uint32_t tie_rank = tie_seen + (uint32_t)__popcll(tie_mask & below);
    sel = sel || (tie && tie_rank < k_tie);
    const uint64_t sel_mask = __ballot(sel);
    const uint32_t slot = pos + (uint32_t)__popcll(sel_mask & below);
    if (sel && slot < (uint32_t)k) orow[slot] = i;
    pos += (uint32_t)__popcll(sel_mask);
    tie_seen += (uint32_t)__popcll(tie_mask);
  };
  wave_sweep<8>(b0, bm, lds_hi, emit);
  wave_sweep<8>(bm, b1, glb_hi, emit);
}


constexpr int kRegSlice = 4 * kTopkThreads;     // columns per slice
constexpr int kRegMaxSlices = 12;
constexpr int kRegMaxRow = kRegSlice * kRegMaxSlices;   // 49152

// Rows t = blockIdx.x, blockIdx.x + gridDim.x, ...: one workgroup of 1024
// threads per compute unit (the keys fill the registers), so the loads of a
// row would otherwise leave HBM idle while the previous row is selected.
// The next row's keys are loaded into registers before the current row is
// processed and only converted when its turn comes.  BITMAP selects the
// column-bitmap emit (sparse selections: prefill-length rows) instead of
// the per-slice scans, whose cost does not grow with the number of keys
// taken (dense selections: a quarter or more of a decode row).
// NT threads; PF: the next row's keys are loaded into registers while the
// current row is selected (one resident workgroup per compute unit).
// Without PF the workgroup is smaller and two share a compute unit, each
// one's loads and barrier waits overlapping the other's work.
template <int S, bool BITMAP, int NT, bool PF>
__global__ __launch_bounds__(NT, 4) void topk_reg_kernel(
    const float* __restrict__ logits, int64_t ld,
    const int32_t* __restrict__ positions, int k, int32_t* __restrict__ out,
    int64_t out_ld, int64_t T, int plim) {
  static_assert(S >= 1 && S * 4 * NT <= kRegMaxRow, "slices");
  constexpr int kSlice = 4 * NT;
  __shared__ RegTopkShared<NT, S> sh;
  const int tid = threadIdx.x;
  // n = p + 1 columns (p < 0 or p >= plim: empty row)
  auto row_len = [&](int64_t t) {
    return row_len_of(load_uniform(positions, t), plim);
  };
  // buffer loads over the row (one offset register for all slices; reads
  // past the row's n columns return 0 and are masked out anyway)
  auto issue = [&](int64_t t, int n, float4 (&v)[S]) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(logits + t * ld, n > k ? n * 4 : 0);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const auto x =
          __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * tid, s * kSlice * 4, 0);
      v[s] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                         __uint_as_float(x[2]), __uint_as_float(x[3]));
    }
  };
  auto select = [&](int64_t t, int n, const float4 (&v)[S]) {
    int32_t* orow = out + t * out_ld;
    if (n <= k) {
      topk_row_short<NT>(n, k, orow);
      return;
    }
    reg_clear(sh);
    RegKeys<S, NT> r;
    r.n = n;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      r.key[s][0] = float_to_ordered(v[s].x);
      r.key[s][1] = float_to_ordered(v[s].y);
      r.key[s][2] = float_to_ordered(v[s].z);
      r.key[s][3] = float_to_ordered(v[s].w);
    }
    __syncthreads();
    uint32_t mask, thr, k_tie, n_eq;
    reg_threshold<NT, S>(r, k, sh, mask, thr, k_tie, BITMAP ? &n_eq : nullptr);
    if (BITMAP)
      // the usual case (distinct values at the threshold): every tied key
      // is selected and the bitmaps carry no tie words
      reg_emit_columns<NT, S>(r, k, mask, thr, k_tie, orow, sh,
                              k_tie == n_eq);
    else
      reg_emit<NT, S>(r, k, mask, thr, k_tie, orow, sh,
                      [](int, int, int pos) { return pos; });
  };
  int64_t t = blockIdx.x;
  if (t >= T) return;
  int n = row_len(t);
  float4 cur[S];
  issue(t, n, cur);
  for (;;) {
    const int64_t tn = t + gridDim.x;
    const int nn = tn < T ? row_len(tn) : 0;
    if (PF) {
      float4 nxt[S];
      issue(tn < T ? tn : t, tn < T ? nn : 0, nxt);
      select(t, n, cur);
#pragma unroll
      for (int s = 0; s < S; ++s) cur[s] = nxt[s];
    } else {
      select(t, n, cur);
      if (tn < T) issue(tn, nn, cur);
    }
    if (tn >= T) break;
    t = tn;
    n = nn;
  }
}

// ---------------------------------------------------------------------------
// Multi-workgroup top-k for long rows (n > kMaxRowForBitmap, e.g. a 1M-token
// context).  Each row is cut into chunks of kMwChunk keys, one 256-thread
// workgroup per (chunk, row):
//   pass 1  histogram of the top 12 key bits per chunk (LDS), added into a
//           per-row global histogram; the last workgroup of the row to finish
//           (a device-scope counter) finds the bin d of the k-th largest key;
//   pass 2  per chunk: count the keys above bin d, append the keys of bin d
//           to a per-row candidate list; the last workgroup resolves the
//           exact threshold key T and the number of ties at T to take (two
//           LDS radix passes over the candidates), adds the candidates above
//           T to their chunks' counts, and scans the chunk counts into
//           offsets;
//   write   per chunk: keys > T and the lowest-index ties, written in
//           ascending index order at the chunk's offset.
// All cross-workgroup hand-offs are device-scope atomics with fences on
// both sides; nothing waits on another workgroup.  A candidate list that
// overflows (heavy ties) is resolved by the last workgroup sweeping the row.
// ---------------------------------------------------------------------------
constexpr int kMwThreads = 256;
constexpr int kMwWaves = kMwThreads / 64;
constexpr int kMwChunk = 16384;
constexpr int kMwCandCap = 32768;

struct MwState {
  uint32_t d1, above1, count1, thr, k_tie, pad[3];
};

struct MwWorkspace {
  uint32_t* hist;     // [T][4096]
  uint32_t* done1;    // [T]
  uint32_t* done2;    // [T]
  uint32_t* ncand;    // [T]
  MwState* state;     // [T]
  uint32_t* ccnt;     // [T][C] keys > T per chunk (then exclusive prefix)
  uint32_t* ctie;     // [T][C] keys == T per chunk (then exclusive prefix)
  uint32_t* cand_key; // [T][cap]
  uint32_t* cand_idx; // [T][cap]
  int64_t C;          // chunks per row
  int plim;           // positions >= plim: empty row
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool use_multi_wg(int64_t ld) { return ld > kMaxRowForBitmap; }

static MwWorkspace carve(void* base, int64_t T, int64_t ld, size_t* total) {
  MwWorkspace w{};
  const int64_t C = (ld + kMwChunk - 1) / kMwChunk;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) { char* q = p ? p + off : nullptr; off += align256(bytes); return q; };
  w.hist = reinterpret_cast<uint32_t*>(take((size_t)T * kHistBins * 4));
  w.done1 = reinterpret_cast<uint32_t*>(take((size_t)T * 4));
  w.done2 = reinterpret_cast<uint32_t*>(take((size_t)T * 4));
  w.ncand = reinterpret_cast<uint32_t*>(take((size_t)T * 4));
  w.ccnt = reinterpret_cast<uint32_t*>(take((size_t)T * C * 4));
  w.ctie = reinterpret_cast<uint32_t*>(take((size_t)T * C * 4));
  const size_t zero_bytes = off;                 // everything above starts at 0
  w.state = reinterpret_cast<MwState*>(take((size_t)T * sizeof(MwState)));
  w.cand_key = reinterpret_cast<uint32_t*>(take((size_t)T * kMwCandCap * 4));
  w.cand_idx = reinterpret_cast<uint32_t*>(take((size_t)T * kMwCandCap * 4));
  w.C = C;
  if (total) *total = off;
  (void)zero_bytes;
  return w;
}

static size_t mw_zero_bytes(int64_t T, int64_t ld) {
  const int64_t C = (ld + kMwChunk - 1) / kMwChunk;
  return align256((size_t)T * kHistBins * 4) + 3 * align256((size_t)T * 4) +
         2 * align256((size_t)T * C * 4);
}

__global__ void mw_clear_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// Block-level bin search for a 256-thread workgroup over an LDS histogram:
// the bin where the count of larger keys first reaches k_rem.  Thread i owns
// BPL bins starting at the top.  Two barriers.
template <int NBINS>
__device__ void mw_select(const uint32_t* hist, uint32_t k_rem,
                          uint32_t* wave_sum, uint32_t* out /*digit,above,count*/) {
  constexpr int BPL = NBINS >= kMwThreads ? NBINS / kMwThreads : 1;
  constexpr int ACTIVE = NBINS / BPL;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const bool active = tid < ACTIVE;
  const int top = NBINS - 1 - tid * BPL;
  uint32_t local = 0;
  if (active)
    for (int j = 0; j < BPL; ++j) local += hist[top - j];
  uint32_t incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  uint32_t above = incl - local;
  for (int w = 0; w < wave; ++w) above += wave_sum[w];
  if (active && above < k_rem && above + local >= k_rem) {
    for (int j = 0; j < BPL; ++j) {
      const uint32_t c = hist[top - j];
      if (above + c >= k_rem) {
        out[0] = (uint32_t)(top - j);
        out[1] = above;
        out[2] = c;
        break;
      }
      above += c;
    }
  }
  __syncthreads();
}

constexpr int kMwLocalCand = 1024;

struct MwShared {
  uint32_t hist[kHistBins];
  uint32_t wave_sum[kMwWaves];
  uint32_t sel[3];
  uint32_t last;
  uint32_t wcnt[kMwWaves], wtie[kMwWaves];
  uint32_t lkey[kMwLocalCand], lidx[kMwLocalCand];
  uint32_t nloc, base;
};

__device__ __forceinline__ int row_len(const int32_t* positions, int64_t t,
                                       int plim) {
  return row_len_of(positions[t], plim);
}

// Becomes true in exactly one workgroup per row: the last of `parts`
// workgroups to call it.  Publishes this workgroup's earlier global writes.
__device__ bool mw_arrive_last(uint32_t* counter, uint32_t parts, MwShared& sh) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(counter, 1u);
    sh.last = (old == parts - 1) ? 1u : 0u;
  }
  __syncthreads();
  const bool last = sh.last != 0;
  if (last) __threadfence();
  return last;
}

__global__ __launch_bounds__(kMwThreads) void mw_pass1_kernel(
    const float* __restrict__ logits, int64_t ld, const int32_t* positions,
    int k, MwWorkspace ws) {
  __shared__ MwShared sh;
  const int64_t t = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int n = row_len(positions, t, ws.plim);
  if (n <= k) return;
  const uint32_t parts = (uint32_t)((n + kMwChunk - 1) / kMwChunk);
  if (c >= parts) return;
  const int tid = threadIdx.x;
  for (int b = tid; b < kHistBins; b += kMwThreads) sh.hist[b] = 0u;
  __syncthreads();
  const float* row = logits + t * ld;
  const int i0 = (int)c * kMwChunk, i1 = min(n, i0 + kMwChunk);
  block_sweep<8, kMwThreads>(
      i0, i1, [&](int i) { return float_to_ordered(row[i]); },
      [&](int, uint32_t key) { atomicAdd(&sh.hist[key >> 20], 1u); });
  __syncthreads();
  uint32_t* gh = ws.hist + t * kHistBins;
  for (int b = tid; b < kHistBins; b += kMwThreads)
    if (sh.hist[b]) atomicAdd(&gh[b], sh.hist[b]);
  if (!mw_arrive_last(&ws.done1[t], parts, sh)) return;
  for (int b = tid; b < kHistBins; b += kMwThreads)
    sh.hist[b] = __atomic_load_n(&gh[b], __ATOMIC_RELAXED);
  __syncthreads();
  mw_select<kHistBins>(sh.hist, (uint32_t)k, sh.wave_sum, sh.sel);
  if (tid == 0) {
    ws.state[t].d1 = sh.sel[0];
    ws.state[t].above1 = sh.sel[1];
    ws.state[t].count1 = sh.sel[2];
  }
}

// Last workgroup of pass 2: exact threshold among the keys of bin d1.
// Candidate source: the candidate list, or (overflow) the whole row.
__device__ void mw_resolve(const float* row, int n, int k, const MwState st,
                           const uint32_t* ck, const uint32_t* ci, uint32_t nc,
                           bool from_row, int64_t t, MwWorkspace& ws,
                           MwShared& sh) {
  const int tid = threadIdx.x;
  const uint32_t d1 = st.d1;
  uint32_t k_rem = (uint32_t)k - st.above1;
  const uint32_t total = from_row ? st.count1 : nc;
  auto for_each = [&](auto&& fn) {
    if (from_row) {
      for (int i = tid; i < n; i += kMwThreads) {
        const uint32_t key = float_to_ordered(row[i]);
        if ((key >> 20) == d1) fn(key, (uint32_t)i);
      }
    } else {
      for (uint32_t j = tid; j < nc; j += kMwThreads) fn(ck[j], ci[j]);
    }
  };
  uint32_t mask = 0xfff00000u, thr = d1 << 20, k_tie = k_rem;
  if (k_rem < total) {
    for (int b = tid; b < kHistBins; b += kMwThreads) sh.hist[b] = 0u;
    __syncthreads();
    for_each([&](uint32_t key, uint32_t) {
      atomicAdd(&sh.hist[(key >> 8) & 0xfffu], 1u);
    });
    __syncthreads();
    mw_select<kHistBins>(sh.hist, k_rem, sh.wave_sum, sh.sel);
    const uint32_t p24 = (d1 << 12) | sh.sel[0];
    const uint32_t k2 = k_rem - sh.sel[1];
    mask = 0xffffff00u; thr = p24 << 8; k_tie = k2;
    if (sh.sel[2] != k2) {
      __syncthreads();
      for (int b = tid; b < 256; b += kMwThreads) sh.hist[b] = 0u;
      __syncthreads();
      for_each([&](uint32_t key, uint32_t) {
        if ((key >> 8) == p24) atomicAdd(&sh.hist[key & 0xffu], 1u);
      });
      __syncthreads();
      mw_select<256>(sh.hist, k2, sh.wave_sum, sh.sel);
      mask = 0xffffffffu; thr = (p24 << 8) | sh.sel[0];
      k_tie = k2 - sh.sel[1];
    }
  }
  // keys of bin d1 above the threshold join their chunk's count; ties
  // at the threshold are counted per chunk
  uint32_t* ccnt = ws.ccnt + t * ws.C;
  uint32_t* ctie = ws.ctie + t * ws.C;
  for_each([&](uint32_t key, uint32_t idx) {
    const uint32_t km = key & mask;
    if (km > thr) atomicAdd(&ccnt[idx / kMwChunk], 1u);
    else if (km == thr) atomicAdd(&ctie[idx / kMwChunk], 1u);
  });
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    ws.state[t].thr = thr;
    ws.state[t].k_tie = k_tie;
    ws.state[t].pad[0] = mask;
    // exclusive prefixes over the chunks (few dozen)
    const int parts = (n + kMwChunk - 1) / kMwChunk;
    uint32_t a = 0, b = 0;
    for (int q = 0; q < parts; ++q) {
      const uint32_t x = __atomic_load_n(&ccnt[q], __ATOMIC_RELAXED);
      const uint32_t y = __atomic_load_n(&ctie[q], __ATOMIC_RELAXED);
      ccnt[q] = a; ctie[q] = b;
      a += x; b += y;
    }
  }
}

__global__ __launch_bounds__(kMwThreads) void mw_pass2_kernel(
    const float* __restrict__ logits, int64_t ld, const int32_t* positions,
    int k, MwWorkspace ws) {
  __shared__ MwShared sh;
  const int64_t t = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int n = row_len(positions, t, ws.plim);
  if (n <= k) return;
  const uint32_t parts = (uint32_t)((n + kMwChunk - 1) / kMwChunk);
  if (c >= parts) return;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const MwState st = ws.state[t];
  const float* row = logits + t * ld;
  const int i0 = (int)c * kMwChunk, i1 = min(n, i0 + kMwChunk);
  uint32_t* ck = ws.cand_key + t * kMwCandCap;
  uint32_t* ci = ws.cand_idx + t * kMwCandCap;
  if (tid == 0) sh.nloc = 0u;
  __syncthreads();
  // keys above bin d1 are counted; keys in bin d1 are gathered in LDS and
  // appended to the row's list with one global atomic per workgroup
  uint32_t gt = 0;
  block_sweep<8, kMwThreads>(
      i0, i1, [&](int i) { return float_to_ordered(row[i]); },
      [&](int i, uint32_t key) {
        const uint32_t dig = key >> 20;
        gt += dig > st.d1;
        if (dig == st.d1) {
          const uint32_t slot = atomicAdd(&sh.nloc, 1u);
          if (slot < (uint32_t)kMwLocalCand) {
            sh.lkey[slot] = key;
            sh.lidx[slot] = (uint32_t)i;
          } else {                                 // rare: straight to global
            const uint32_t g = atomicAdd(&ws.ncand[t], 1u);
            if (g < (uint32_t)kMwCandCap) { ck[g] = key; ci[g] = (uint32_t)i; }
          }
        }
      });
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) gt += __shfl_xor(gt, off);
  if (lane == 0) sh.wcnt[wave] = gt;
  __syncthreads();
  const uint32_t nl = min(sh.nloc, (uint32_t)kMwLocalCand);
  if (tid == 0) {
    uint32_t s = 0;
    for (int w = 0; w < kMwWaves; ++w) s += sh.wcnt[w];
    atomicAdd(&ws.ccnt[t * ws.C + c], s);
    sh.base = nl ? atomicAdd(&ws.ncand[t], nl) : 0u;
  }
  __syncthreads();
  for (uint32_t j = tid; j < nl; j += kMwThreads) {
    const uint32_t g = sh.base + j;
    if (g < (uint32_t)kMwCandCap) { ck[g] = sh.lkey[j]; ci[g] = sh.lidx[j]; }
  }
  if (!mw_arrive_last(&ws.done2[t], parts, sh)) return;
  const uint32_t nc = __atomic_load_n(&ws.ncand[t], __ATOMIC_RELAXED);
  const bool overflow = nc > (uint32_t)kMwCandCap;
  mw_resolve(row, n, k, st, ck, ci, overflow ? 0u : nc, overflow, t, ws, sh);
}

__global__ __launch_bounds__(kMwThreads) void mw_write_kernel(
    const float* __restrict__ logits, int64_t ld, const int32_t* positions,
    int k, int32_t* __restrict__ out, int64_t out_ld, MwWorkspace ws) {
  __shared__ MwShared sh;
  const int64_t t = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int n = row_len(positions, t, ws.plim);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  int32_t* orow = out + t * out_ld;
  if (n <= k) {
    if (c == 0)
      for (int i = tid; i < k; i += kMwThreads) orow[i] = i < n ? i : -1;
    return;
  }
  const int parts = (n + kMwChunk - 1) / kMwChunk;
  if (c >= parts) return;
  const MwState st = ws.state[t];
  const uint32_t mask = st.pad[0], thr = st.thr, k_tie = st.k_tie;
  const float* row = logits + t * ld;
  const int i0 = (int)c * kMwChunk, i1 = min(n, i0 + kMwChunk);
  constexpr int kSub = kMwChunk / kMwWaves;
  const int s0 = min(i1, i0 + wave * kSub), s1 = min(i1, s0 + kSub);
  uint32_t gt = 0, eq = 0;
  auto load = [&](int i) { return float_to_ordered(row[i]) & mask; };
  wave_sweep<8>(s0, s1, load, [&](int, bool in, uint32_t km) {
    gt += in && km > thr;
    eq += in && km == thr;
  });
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) { sh.wcnt[wave] = gt; sh.wtie[wave] = eq; }
  __syncthreads();
  uint32_t gt_before = ws.ccnt[t * ws.C + c], tie_seen = ws.ctie[t * ws.C + c];
  for (int w = 0; w < wave; ++w) { gt_before += sh.wcnt[w]; tie_seen += sh.wtie[w]; }
  uint32_t pos = gt_before + min(tie_seen, k_tie);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  wave_sweep<8>(s0, s1, load, [&](int i, bool in, uint32_t km) {
    const bool is_gt = in && km > thr;
    const bool is_eq = in && km == thr;
    const uint64_t eq_mask = __ballot(is_eq);
    const uint32_t eq_rank = tie_seen + (uint32_t)__popcll(eq_mask & below);
    const bool sel = is_gt || (is_eq && eq_rank < k_tie);
    const uint64_t sel_mask = __ballot(sel);
    const uint32_t slot = pos + (uint32_t)__popcll(sel_mask & below);
    if (sel && slot < (uint32_t)k) orow[slot] = i;
    pos += (uint32_t)__popcll(sel_mask);
    tie_seen += (uint32_t)__popcll(eq_mask);
  });
}

// ---------------------------------------------------------------------------
// Sample-select top-k for long rows (16384 < n, rows of up to 16M columns).
// A key below the k-th largest can never be selected, so any lower bound
// T_lo of the k-th largest key turns the row into a short candidate list
// {key >= T_lo} that still holds the whole answer:
//   sample   16 workgroups per row read the row's 16384 keys at jittered
//            stride n / 16384 (scattered 4-byte reads: spread over many
//            compute units, since one unit alone is limited by its own L2
//            bandwidth for 16384 separate lines) into a contiguous buffer;
//            then one 1024-thread workgroup per row reads them back
//            coalesced and takes the m-th largest as T_lo, m = k * 16384 /
//            n + 4 sqrt(k * 16384 / n) + 16: about m n / 16384 keys of the
//            row (k plus a few standard deviations) are then at or above
//            T_lo;
//   collect  one 256-thread workgroup per 16384-key chunk writes its keys
//            >= T_lo, in column order, to the chunk's slot of 512 (one
//            fully coalesced pass over the row, the HBM-bound part);
//   select   one 1024-thread workgroup per row gathers the candidates (a scan
//            of the chunk counts, a binary search per item) into registers
//            and runs the register top-k on them, writing their columns in
//            ascending order.
// The sample decides only the speed, never the result: when the candidates
// number fewer than k (T_lo above the k-th key) or more than 16384, or a
// chunk overflows its slot (heavy ties), the select workgroup runs an exact
// radix select over the whole row instead.
// ---------------------------------------------------------------------------
constexpr int kSsSample = 16384;
constexpr int kSsThreads = 256;
constexpr int kSsChunk = 16384;
constexpr int kSsChunkCap = 512;
constexpr int kSsCandMax = 4 * 4 * kTopkThreads;   // 16384 (RegKeys<4>)
constexpr int64_t kSsMaxChunks = 1024;             // rows up to 16M columns

struct SsWorkspace {
  uint32_t* samp;     // [T][kSsSample] sampled keys (ordered)
  uint32_t* thr;      // [T] T_lo
  uint32_t* count;    // [T][C] candidates per chunk (> cap: overflow)
  uint2* cand;        // [T][C][cap] (key, column)
  int64_t C;
  int plim;           // positions >= plim: empty row
};

static bool use_sample_select(int64_t ld) {
  return ld > kMaxRowForBitmap &&
         (ld + kSsChunk - 1) / kSsChunk <= kSsMaxChunks;
}

static SsWorkspace ss_carve(void* base, int64_t T, int64_t ld,
                            size_t* total) {
  SsWorkspace w{};
  const int64_t C = (ld + kSsChunk - 1) / kSsChunk;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += align256(bytes);
    return q;
  };
  w.samp = reinterpret_cast<uint32_t*>(take((size_t)T * kSsSample * 4));
  w.thr = reinterpret_cast<uint32_t*>(take((size_t)T * 4));
  w.count = reinterpret_cast<uint32_t*>(take((size_t)T * C * 4));
  w.cand = reinterpret_cast<uint2*>(take((size_t)T * C * kSsChunkCap * 8));
  w.C = C;
  if (total) *total = off;
  return w;
}

__device__ __forceinline__ uint32_t ss_hash(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu;
  return x ^ (x >> 16);
}

constexpr int kSsGatherWgs = 16;                        // per row
constexpr int kSsGatherPerThread = kSsSample / (kSsGatherWgs * kSsThreads);

// Grid (16, T): sample q (0..16383) of row t is column q * stride +
// hash(q) % stride (< n, stride = n / 16384 >= 1), stored as its ordered key
// at samp[t][q]; workgroup g takes q in [1024 g, 1024 g + 1024).
__global__ __launch_bounds__(kSsThreads) void ss_gather_kernel(
    const float* __restrict__ logits, int64_t ld, const int32_t* positions,
    int k, SsWorkspace ws) {
  const int64_t t = blockIdx.y;
  const int n = row_len(positions, t, ws.plim);
  if (n <= kSsCandMax || n <= k) return;
  const float* row = logits + t * ld;
  const uint32_t stride = (uint32_t)n / kSsSample;     // >= 1
  uint32_t* out = ws.samp + t * kSsSample;
  uint32_t key[kSsGatherPerThread];
#pragma unroll
  for (int j = 0; j < kSsGatherPerThread; ++j) {
    const uint32_t q = (uint32_t)((blockIdx.x * kSsGatherPerThread + j) *
                                  kSsThreads + threadIdx.x);
    key[j] = float_to_ordered(row[q * stride + ss_hash(q) % stride]);
  }
#pragma unroll
  for (int j = 0; j < kSsGatherPerThread; ++j)
    out[(blockIdx.x * kSsGatherPerThread + j) * kSsThreads + threadIdx.x] =
        key[j];
}

// One workgroup per row: the m-th largest of the row's 16384 samples.
__global__ __launch_bounds__(kTopkThreads) void ss_sample_kernel(
    const float* __restrict__ logits, int64_t ld, const int32_t* positions,
    int k, SsWorkspace ws) {
  __shared__ RegTopkShared<kTopkThreads, 4> sh;
  const int64_t t = blockIdx.x;
  const int n = row_len(positions, t, ws.plim);
  if (n <= kSsCandMax || n <= k) return;
  const int tid = threadIdx.x;
  reg_clear(sh);
  const uint32_t* samp = ws.samp + t * kSsSample;
  RegKeys<4> r;
  r.n = kSsSample;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint4 v = *reinterpret_cast<const uint4*>(
        samp + s * 4 * kTopkThreads + 4 * tid);
    r.key[s][0] = v.x;
    r.key[s][1] = v.y;
    r.key[s][2] = v.z;
    r.key[s][3] = v.w;
  }
  __syncthreads();
  const float e = (float)k * (float)kSsSample / (float)n;
  const int m = min(kSsSample - 1, (int)(e + 4.f * sqrtf(e)) + 16);
  uint32_t mask, thr, k_tie;
  reg_threshold<kTopkThreads, 4>(r, m, sh, mask, thr, k_tie);
  if (tid == 0) ws.thr[t] = thr & mask;
}

__global__ __launch_bounds__(kSsThreads) void ss_collect_kernel(
    const float* __restrict__ logits, int64_t ld, const int32_t* positions,
    int k, SsWorkspace ws) {
  constexpr int kWaves = kSsThreads / 64;
  constexpr int kSlices = kSsChunk / (4 * kSsThreads);   // 16
  __shared__ uint32_t s_tot[kSlices * kWaves];
  const int64_t t = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int n = row_len(positions, t, ws.plim);
  if (n <= kSsCandMax || n <= k) return;
  const int parts = (n + kSsChunk - 1) / kSsChunk;
  if (c >= parts) return;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t thr = ws.thr[t];
  const float* row = logits + t * ld;
  const int i0 = (int)c * kSsChunk;
  if (thr == 0u) {
    // every key qualifies: the candidate list would be the whole row, which
    // the select kernel handles by its exact path (flagged as an overflow)
    if (tid == 0) ws.count[t * ws.C + c] = kSsChunkCap + 1;
    return;
  }
  uint32_t key[kSlices][4];
  // all 16 loads in flight before any is used (interleaving them with the
  // scans below makes every slice a separate round trip to HBM); buffer
  // loads over the chunk's columns below n share one offset register, and
  // reads past n return 0 (masked out below)
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(row + i0, min(n - i0, kSsChunk) * 4);
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(
        rs, 16 * tid, s * 4 * kSsThreads * 4, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) key[s][j] = x[j];           // fp32 bits
  }
  // a slice's count and in-wave scan are recomputed after the barrier
  // rather than kept, and a column at or past n gets key 0, below thr >= 1
  // (only the 64 keys stay live: fewer registers, more workgroups resident
  // per compute unit)
  auto count = [&](int s) {
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) m += key[s][j] >= thr ? 1u : 0u;
    return m;
  };
  const int n_here = n - i0;                 // columns of this chunk below n
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t kk = float_to_ordered(__uint_as_float(key[s][j]));
      key[s][j] = s * 4 * kSsThreads + 4 * tid + j < n_here ? kk : 0u;
    }
    const uint32_t incl = wave_inclusive_scan(count(s));
    if (lane == 63) s_tot[s * kWaves + wave] = incl;
  }
  __syncthreads();
  if (wave == 0) {                           // 64 (slice, wave) totals
    const uint32_t v = s_tot[lane];
    const uint32_t sc = wave_inclusive_scan(v);
    s_tot[lane] = sc - v;
    if (lane == 63 && tid == 63)
      ws.count[t * ws.C + c] = sc;            // may exceed the slot: overflow
  }
  __syncthreads();
  uint2* slot = ws.cand + (t * ws.C + c) * kSsChunkCap;
#pragma unroll
  for (int s = 0; s < kSlices; ++s) {
    const uint32_t m = count(s);
    uint32_t o = s_tot[s * kWaves + wave] + wave_inclusive_scan(m) - m;
    const int c0 = i0 + s * 4 * kSsThreads + 4 * tid;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (key[s][j] >= thr) {
        if (o < (uint32_t)kSsChunkCap)
          slot[o] = make_uint2(key[s][j], (uint32_t)(c0 + j));
        ++o;
      }
    }
  }
}

union SsSelectShared {
  RegTopkShared<kTopkThreads, 4> reg;
  TopkShared full;
};

__global__ __launch_bounds__(kTopkThreads) void ss_select_kernel(
    const float* __restrict__ logits, int64_t ld, const int32_t* positions,
    int k, int32_t* __restrict__ out, int64_t out_ld, SsWorkspace ws) {
  __shared__ SsSelectShared sh;
  __shared__ uint32_t s_pre[kSsMaxChunks + 1];
  __shared__ uint32_t s_flag[2];
  const int64_t t = blockIdx.x;
  const int n = row_len(positions, t, ws.plim);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  int32_t* orow = out + t * out_ld;
  if (n <= k) {
    topk_row_short<kTopkThreads>(n, k, orow);
    return;
  }
  const float* row = logits + t * ld;
  if (n <= kSsCandMax) {                     // the whole row fits
    topk_row_registers<kTopkThreads, 4>(row, ld, n, k, orow, sh.reg);
    return;
  }
  // candidates per chunk -> exclusive prefix (at most 1024 chunks)
  const int parts = (n + kSsChunk - 1) / kSsChunk;
  const uint32_t cc = tid < parts ? ws.count[t * ws.C + tid] : 0u;
  if (tid == 0) { s_flag[0] = 0u; s_flag[1] = 0u; }
  __syncthreads();
  if (cc > (uint32_t)kSsChunkCap) s_flag[0] = 1u;           // overflow
  const uint32_t wi = wave_inclusive_scan(cc);
  if (lane == 63) sh.reg.wave_sum[wave] = wi;
  __syncthreads();
  uint32_t before = wi - cc;
  for (int w = 0; w < wave; ++w) before += sh.reg.wave_sum[w];
  if (tid < parts) s_pre[tid] = before;
  if (tid == parts - 1) { s_pre[parts] = before + cc; s_flag[1] = before + cc; }
  __syncthreads();
  const uint32_t total = s_flag[1];
  const bool exact_path = s_flag[0] != 0u || total < (uint32_t)k ||
                          total > (uint32_t)kSsCandMax;
  __syncthreads();
  if (exact_path) {
    // exact radix select over the whole row (keys from global)
    const RowKeys keys{row, nullptr, 0};
    radix_pass<kHistBins>(keys, n, 0u, 0u, 20, (uint32_t)k, sh.full);
    topk_radix_rest(keys, n, k, orow, sh.full);
    return;
  }
  reg_clear(sh.reg);
  // gather: item x (list order = column order) lives in chunk q with
  // s_pre[q] <= x < s_pre[q + 1]
  RegKeys<4> r;
  r.n = (int)total;
  uint32_t col[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = (uint32_t)(s * 4 * kTopkThreads + 4 * tid + j);
      r.key[s][j] = 0u;
      col[s][j] = 0u;
      if (x < total) {
        int lo = 0, hi = parts - 1;           // last chunk with s_pre <= x
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_pre[mid] <= x) lo = mid; else hi = mid - 1;
        }
        const uint2 e = ws.cand[(t * ws.C + lo) * kSsChunkCap + (x - s_pre[lo])];
        r.key[s][j] = e.x;
        col[s][j] = e.y;
      }
    }
  }
  __syncthreads();
  uint32_t mask, thr, k_tie;
  reg_threshold<kTopkThreads, 4>(r, k, sh.reg, mask, thr, k_tie);
  reg_emit<kTopkThreads, 4>(r, k, mask, thr, k_tie, orow, sh.reg,
                            [&](int s, int j, int) { return (int)col[s][j]; });
}

// ---------------------------------------------------------------------------
// Fused forward: logits and exact top-k without the [T, ld] logits buffer
// (the GLM-5.3 cache-budget article's logits budget, section on SGLang's
// logits budget: a score buffer of rows x columns fp32 that grows with the
// context; here the rows never materialise).  The same lower-bound idea as
// the sample select above, with the sample scored instead of read:
//   sample    the tile kernel scores every SS-th page of each row (SS >= 16)
//             into a compact buffer (logits_tile16_kernel, page_stride);
//   threshold one workgroup per row takes the m-th largest sampled key as
//             T_lo, m = e + 4 sqrt(e) + 16 with e = k n_s / n the expected
//             number of sampled keys among the row's k largest (n_s sampled
//             visible columns);
//   score     the tile kernel scores every page again and appends every
//             logit >= T_lo, as (key, column), to its (row, split) slot in
//             ascending column order, with the slot's count
//             (logits_tile16_kernel, CAND);
//   select    one workgroup per row gathers its slots (column order) into
//             registers and runs the register top-k on them;
//   rescue    rows whose candidates cannot hold the answer (fewer than k,
//             a slot overflowed, more than 16384) are re-scored whole into
//             a per-workgroup scratch row with the tile kernel's arithmetic
//             and ranked by the exact radix select.
// Every key above the k-th largest is >= T_lo once the candidates number k
// or more, and every key equal to it is a candidate too, so the selection
// (ties lowest column first) is the exact top-k of the row's logits: the
// sample decides the speed only.  The logits themselves are those of the
// default tiled kernel bit for bit (same operations per logit), so the
// result equals dsa_indexer_forward's for such a batch.
// ---------------------------------------------------------------------------
constexpr int kFusedMaxSplits = 2048;
constexpr int kFusedCandMax = 4 * 4 * kTopkThreads;    // RegKeys<4>
constexpr int kFusedMinStride = 16;
constexpr int kFusedMaxSampledPages = 256;             // n_s <= 16384
constexpr int kFusedRescueSlots = 64;

// One sample workgroup of NT threads per row (up to 16 NT sampled
// columns): T_lo[t] (0xffffffff for a row of at most k columns: nothing to
// collect); workgroup 0 also clears the rescue count.
template <int NT, int S>
__global__ __launch_bounds__(NT) void fused_threshold_kernel(
    const float* __restrict__ samp, int64_t ld_s,
    const int32_t* __restrict__ positions, int plim, int SS, int k,
    uint32_t* __restrict__ tlo, uint32_t* __restrict__ fail) {
  __shared__ RegTopkShared<NT, S> sh;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  if (t == 0 && tid == 0) fail[0] = 0u;
  const int n = row_len_of(positions[t], plim);
  if (n <= k) {
    if (tid == 0) tlo[t] = 0xffffffffu;
    return;
  }
  // logical pages 0..lp-1 hold real pages 0, SS, 2 SS, ..: all full but
  // the last, whose real page may be the row's partial one
  const int lp = ((n - 1) >> 6) / SS + 1;
  const int ns = kPageTokens * lp;
  const int nreal =
      kPageTokens * (lp - 1) + min(kPageTokens, n - kPageTokens * (lp - 1) * SS);
  const float e = (float)k * (float)nreal / (float)n;
  const int m = min(nreal - 1, (int)(e + 4.f * sqrtf(e)) + 16);
  if (m < 1) {                               // take every logit
    if (tid == 0) tlo[t] = 0u;
    return;
  }
  reg_clear(sh);
  RegKeys<S, NT> r;
  r.n = ns;                                  // the -inf tail ranks last
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(samp + t * ld_s, ns * 4);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(
        rs, 16 * tid, s * 16 * NT, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r.key[s][j] = float_to_ordered(__uint_as_float(v[j]));
  }
  __syncthreads();
  uint32_t mask, thr, k_tie;
  reg_threshold<NT, S>(r, m, sh, mask, thr, k_tie);
  if (tid == 0) tlo[t] = thr & mask;
}

// One workgroup per row: the row's candidate slots -> top-k, or the row
// goes on the rescue list.
__global__ __launch_bounds__(kTopkThreads) void fused_select_kernel(
    const int32_t* __restrict__ positions, const int32_t* __restrict__ qsl,
    int R, int plim, int k,
    int32_t* __restrict__ out, int64_t out_ld,
    const uint32_t* __restrict__ count, const uint2* __restrict__ cand,
    int gx, int cap, int force_rescue, uint32_t* __restrict__ fail) {
  __shared__ RegTopkShared<kTopkThreads, 4> sh;
  __shared__ uint32_t s_pre[kFusedMaxSplits + 1];
  __shared__ uint32_t s_flag[2];
  const int64_t t = blockIdx.x;
  // a row outside query_start_loc's rows is in no tile: a row of -1
  const bool in_batch =
      t >= load_uniform(qsl, 0) && t < load_uniform(qsl, R);
  const int n = in_batch ? row_len_of(positions[t], plim) : 0;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  int32_t* orow = out + t * out_ld;
  if (n <= k) {
    topk_row_short<kTopkThreads>(n, k, orow);
    return;
  }
  // slot counts -> exclusive prefix over the gx splits (two per thread)
  const uint32_t* crow = count + t * gx;
  const uint32_t c0 = 2 * tid < gx ? crow[2 * tid] : 0u;
  const uint32_t c1 = 2 * tid + 1 < gx ? crow[2 * tid + 1] : 0u;
  if (tid == 0) { s_flag[0] = 0u; s_flag[1] = 0u; }
  __syncthreads();
  if (c0 > (uint32_t)cap || c1 > (uint32_t)cap) s_flag[0] = 1u;  // overflow
  const uint32_t cc = c0 + c1;
  const uint32_t wi = wave_inclusive_scan(cc);
  if (lane == 63) sh.wave_sum[wave] = wi;
  __syncthreads();
  uint32_t before = wi - cc;
  for (int w = 0; w < wave; ++w) before += sh.wave_sum[w];
  if (2 * tid < gx) s_pre[2 * tid] = before;
  if (2 * tid + 1 < gx) s_pre[2 * tid + 1] = before + c0;
  if (tid == kTopkThreads - 1) s_flag[1] = before + cc;
  __syncthreads();
  const uint32_t total = s_flag[1];
  const bool rescue = force_rescue || s_flag[0] != 0u ||
                      total < (uint32_t)k || total > (uint32_t)kFusedCandMax;
  if (rescue) {
    if (tid == 0) fail[1 + atomicAdd(fail, 1u)] = (uint32_t)t;
    return;
  }
  reg_clear(sh);
  // item x (list order = column order) lives in split q with s_pre[q] <= x
  // < s_pre[q + 1]; every count is <= cap, so x - s_pre[q] < cap
  RegKeys<4> r;
  r.n = (int)total;
  uint32_t col[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = (uint32_t)(s * 4 * kTopkThreads + 4 * tid + j);
      r.key[s][j] = 0u;
      col[s][j] = 0u;
      if (x < total) {
        int lo = 0, hi = gx - 1;              // last split with s_pre <= x
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_pre[mid] <= x) lo = mid; else hi = mid - 1;
        }
        const uint2 e =
            cand[(t * gx + lo) * (int64_t)cap + (x - s_pre[lo])];
        r.key[s][j] = e.x;
        col[s][j] = e.y;
      }
    }
  }
  __syncthreads();
  uint32_t mask, thr, k_tie;
  reg_threshold<kTopkThreads, 4>(r, k, sh, mask, thr, k_tie);
  reg_emit<kTopkThreads, 4>(r, k, mask, thr, k_tie, orow, sh,
                            [&](int s, int j, int) { return (int)col[s][j]; });
}

// ---------------------------------------------------------------------------
// One wave per row (sample thresholds and candidate lists of up to a few
// thousand items): the items in registers, item x = 64 j + lane (j < KPL),
// and a radix select with 8-bit digits over a 256-bin LDS histogram of the
// wave's own -- no workgroup barrier, and a few hundred bytes of LDS per
// row, so a compute unit holds many rows at once.
// ---------------------------------------------------------------------------
constexpr int kWaveRowsPerWg = 4;
constexpr int kWaveMaxSplits = 16;

// The k-th largest of the n valid items' keys (1 <= k <= n): thr, and
// k_tie, how many of the items equal to it belong to the k largest (the
// lowest-x ones).  Each round bins the keys of the items still in play by
// (key - lo) >> s over [lo, hi], their smallest and largest key, in at most
// 256 bins of a 256-bin LDS histogram of the wave's own (bins follow the
// keys' actual spread, so few items share an LDS address: atomics to one
// address serialise); the bin holding the k-th largest becomes the next
// range, narrowed again to its items' smallest and largest key.
template <int KPL>
__device__ __forceinline__ void wave_kth_key(const uint32_t (&key)[KPL], int n, uint32_t k,
                             uint32_t* hist, uint32_t& thr, uint32_t& k_tie) {
  const int lane = lane_id();
  const int jn = (n + 63) >> 6;
  uint32_t lo = 0u, hi = 0xffffffffu, k_rem = k;
#pragma unroll 1
  for (int round = 0; round < 8; ++round) {
    uint32_t a = 0xffffffffu, z = 0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (j >= jn) continue;
      if (64 * j + lane < n && key[j] - lo <= hi - lo) {
        a = min(a, key[j]);
        z = max(z, key[j]);
      }
    }
    lo = wave_umin(a);
    hi = wave_umax(z);
    thr = lo; k_tie = k_rem;
    if (lo == hi) return;                      // every item in play is equal
    const uint32_t range = hi - lo;
    const int s = max(0, 24 - __builtin_clz(range));   // range >> s < 256
    // (LDS accesses of one wave take effect in program order)
    *reinterpret_cast<uint4*>(&hist[4 * lane]) = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (j >= jn) continue;
      if (64 * j + lane < n && key[j] - lo <= range)
        atomicAdd(&hist[(key[j] - lo) >> s], 1u);
    }
    // lane l holds bins 255 - 4 l down to 252 - 4 l
    const uint4 h = *reinterpret_cast<const uint4*>(&hist[252 - 4 * lane]);
    const uint32_t c[4] = {h.w, h.z, h.y, h.x};
    const uint32_t local = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_inclusive_scan(local);
    const int ls = __builtin_ctzll(__ballot(incl >= k_rem));
    uint32_t acc = incl - local, ab = 0u, cn = 0u;
    int jj = 0;
    bool found = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!found && acc + c[q] >= k_rem) {
        found = true;
        jj = q;
        ab = acc;
        cn = c[q];
      }
      acc += c[q];
    }
    const uint32_t b = 255u - 4u * (uint32_t)ls -
                       (uint32_t)__builtin_amdgcn_readlane(jj, ls);
    const uint32_t above = __builtin_amdgcn_readlane(ab, ls);
    const uint32_t count = __builtin_amdgcn_readlane(cn, ls);
    k_rem -= above;
    const uint32_t blo = lo + (b << s);
    const uint32_t bhi = s == 0 ? blo : min(hi, blo + ((1u << s) - 1u));
    if (count == k_rem) {
      // the whole bin is taken: keys > thr, and all k_rem ties at thr
      // ... expressed with the bin's smallest key as thr
      lo = blo; hi = bhi;
      uint32_t a2 = 0xffffffffu;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        if (j >= jn) continue;
        if (64 * j + lane < n && key[j] - lo <= hi - lo) a2 = min(a2, key[j]);
      }
      thr = wave_umin(a2);
      // items equal to thr are all in the bin: all of them are taken
      k_tie = k_rem;
      return;
    }
    lo = blo; hi = bhi;
  }
}

// Writes the selected items' col_of(j, taken) in item order (ascending x;
// of the items equal to thr the k_tie lowest-x ones) to orow[0..k).
// col_of is called for every j in turn, on every lane (taken: whether this
// lane's item is written).
template <int KPL, typename ColOf>
__device__ __forceinline__ void wave_emit(const uint32_t (&key)[KPL], int n, uint32_t thr,
                          uint32_t k_tie, int k, int32_t* orow, ColOf col_of) {
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1ull;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(orow, k * 4);
  uint32_t pos = 0u, eq_seen = 0u;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    if (64 * j >= n) continue;
    const bool ok = 64 * j + lane < n;
    const bool gt = ok && key[j] > thr;
    const bool eq = ok && key[j] == thr;
    const uint64_t eqm = __ballot(eq);
    const uint32_t er = eq_seen + (uint32_t)__popcll(eqm & below);
    const bool take = gt || (eq && er < k_tie);
    const uint64_t tm = __ballot(take);
    const uint32_t slot = pos + (uint32_t)__popcll(tm & below);
    const uint32_t col = (uint32_t)col_of(j, take);
    __builtin_amdgcn_raw_buffer_store_b32(col, ro,
                                          take ? (int)(4 * slot) : 4 * k, 0,
                                          0);
    pos += (uint32_t)__popcll(tm);
    eq_seen += (uint32_t)__popcll(eqm);
  }
}

// Sample thresholds, one wave per row (rows of at most 64 KPL sampled
// columns); see fused_threshold_kernel.  Only a lower bound of the m-th
// largest sample is needed, found on the values: a 256-bin histogram over
// [min, max] of the finite samples, a second one over the bin holding the
// m-th largest, and the smallest sample of the sub-bin holding it (the bin
// of a value is a non-decreasing function of the value, so that sub-bin's
// smallest sample is at most the m-th largest).
template <int KPL>
__global__ __launch_bounds__(64 * kWaveRowsPerWg) void fused_threshold_wave_kernel(
    const float* __restrict__ samp, int64_t ld_s,
    const int32_t* __restrict__ positions, int64_t T, int plim, int SS, int k,
    uint32_t* __restrict__ tlo, uint32_t* __restrict__ fail) {
  __shared__ __align__(16) uint32_t s_hist[kWaveRowsPerWg][256];
  const int lane = lane_id();
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int64_t t = (int64_t)blockIdx.x * kWaveRowsPerWg + wave;
  if (blockIdx.x == 0 && threadIdx.x == 0) fail[0] = 0u;
  if (t >= T) return;
  const int n = row_len_of(load_uniform(positions, t), plim);
  if (n <= k) {
    if (lane == 0) tlo[t] = 0xffffffffu;
    return;
  }
  const int lp = ((n - 1) >> 6) / SS + 1;
  const int ns = kPageTokens * lp;
  const int nreal =
      kPageTokens * (lp - 1) + min(kPageTokens, n - kPageTokens * (lp - 1) * SS);
  const float e = (float)k * (float)nreal / (float)n;
  const int m = min(nreal - 1, (int)(e + 4.f * sqrtf(e)) + 16);
  // the sample order does not matter here: 16-byte loads, item (j4, q) =
  // column 256 j4 + 4 lane + q; columns past ns count as -inf
  const int j4n = (ns + 255) >> 8;
  float v[KPL];
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(samp + t * ld_s, ns * 4);
#pragma unroll
  for (int j4 = 0; j4 < KPL / 4; ++j4) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane,
                                                         j4 * 1024, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[4 * j4 + q] = 256 * j4 + 4 * lane + q < ns ? __uint_as_float(x[q])
                                                   : -INFINITY;
  }
  uint32_t* hist = s_hist[wave];
  float mx = -INFINITY, mn = INFINITY;
  uint32_t nfin = 0u;
  bool nan = false;
#pragma unroll
  for (int j4 = 0; j4 < KPL / 4; ++j4) {
    if (j4 >= j4n) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float y = v[4 * j4 + q];
      nan |= y != y;
      if (fabsf(y) <= 3.402823466e38f) {
        mx = fmaxf(mx, y);
        mn = fminf(mn, y);
        ++nfin;
      }
    }
  }
  nfin = __builtin_amdgcn_readlane(wave_inclusive_scan(nfin), 63);
  // (ordered keys: a max / min over them is one over the values)
  const uint32_t kmx = wave_umax(float_to_ordered(mx));
  const uint32_t kmn = wave_umin(float_to_ordered(mn));
  if (m < 1 || __ballot(nan) != 0ull || (uint32_t)m >= nfin) {
    if (lane == 0) tlo[t] = 0u;                 // take every logit
    return;
  }
  if (kmx == kmn) {                             // all finite samples equal
    if (lane == 0) tlo[t] = kmn;
    return;
  }
  mx = ordered_to_float(kmx);
  mn = ordered_to_float(kmn);
  const float scale = 256.f / (mx - mn);       // 0 if the span overflows
  auto bin1 = [&](float y) { return min(255, (int)((y - mn) * scale)); };
  uint32_t k_rem = (uint32_t)m, above = 0u;
  int b1 = 0;
  // pass 1 over the finite samples, pass 2 over those of bin b1
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    *reinterpret_cast<uint4*>(&hist[4 * lane]) = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j4 = 0; j4 < KPL / 4; ++j4) {
      if (j4 >= j4n) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float y = v[4 * j4 + q];
        if (!(fabsf(y) <= 3.402823466e38f)) continue;
        const int c1 = bin1(y);
        if (pass == 0) {
          atomicAdd(&hist[c1], 1u);
        } else if (c1 == b1) {
          const int c2 =
              min(255, max(0, (int)(((y - mn) * scale - (float)b1) * 256.f)));
          atomicAdd(&hist[c2], 1u);
        }
      }
    }
    const uint4 h = *reinterpret_cast<const uint4*>(&hist[252 - 4 * lane]);
    const uint32_t c[4] = {h.w, h.z, h.y, h.x};
    const uint32_t local = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_inclusive_scan(local);
    const int ls = __builtin_ctzll(__ballot(incl >= k_rem));
    uint32_t acc = incl - local, ab = 0u;
    int jj = 0;
    bool found = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!found && acc + c[q] >= k_rem) {
        found = true;
        jj = q;
        ab = acc;
      }
      acc += c[q];
    }
    const int b = 255 - 4 * ls - __builtin_amdgcn_readlane(jj, ls);
    above = __builtin_amdgcn_readlane(ab, ls);
    k_rem -= above;
    if (pass == 0) {
      b1 = b;
    } else {
      // the smallest sample of sub-bin b of bin b1
      float lowest = INFINITY;
#pragma unroll
      for (int j4 = 0; j4 < KPL / 4; ++j4) {
        if (j4 >= j4n) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float y = v[4 * j4 + q];
          if (!(fabsf(y) <= 3.402823466e38f) || bin1(y) != b1) continue;
          const int c2 =
              min(255, max(0, (int)(((y - mn) * scale - (float)b1) * 256.f)));
          if (c2 == b) lowest = fminf(lowest, y);
        }
      }
      const uint32_t kl = wave_umin(float_to_ordered(lowest));
      if (lane == 0) tlo[t] = kl;
    }
  }
}

// Candidate item x of a row: in split q, the last q with pre[q] <= x (a
// fixed four-step search over at most 16 splits).
static_assert(kWaveMaxSplits <= 16, "four search steps");
__device__ __forceinline__ const uint2* wave_item(const uint2* crow,
                                                  const uint32_t* pre, int gx,
                                                  int cap, uint32_t x) {
  int q = 0;
#pragma unroll
  for (int st = 8; st >= 1; st >>= 1)
    if (q + st < gx && pre[q + st] <= x) q += st;
  return crow + (int64_t)q * cap + (x - pre[q]);
}

// Candidate select, one wave per row (candidate lists of at most 64 KPL
// items, at most kWaveMaxSplits splits); see fused_select_kernel.
template <int KPL>
__global__ __launch_bounds__(64 * kWaveRowsPerWg) void fused_select_wave_kernel(
    const int32_t* __restrict__ positions, const int32_t* __restrict__ qsl,
    int R, int64_t T, int plim, int k, int32_t* __restrict__ out,
    int64_t out_ld, const uint32_t* __restrict__ count,
    const uint2* __restrict__ cand, int gx, int cap, int force_rescue,
    uint32_t* __restrict__ fail) {
  __shared__ __align__(16) uint32_t s_hist[kWaveRowsPerWg][256];
  __shared__ uint32_t s_pre[kWaveRowsPerWg][kWaveMaxSplits + 1];
  const int lane = lane_id();
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int64_t t = (int64_t)blockIdx.x * kWaveRowsPerWg + wave;
  if (t >= T) return;
  const bool in_batch =
      t >= load_uniform(qsl, 0) && t < load_uniform(qsl, R);
  const int n = in_batch ? row_len_of(load_uniform(positions, t), plim) : 0;
  int32_t* orow = out + t * out_ld;
  if (n <= k) {
    for (int i = lane; i < k; i += 64) orow[i] = i < n ? i : -1;
    return;
  }
  // slot counts -> prefix (lane l: splits 4 l .. 4 l + 3)
  uint32_t c[4], local = 0u;
  bool over = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int x = 4 * lane + q;
    c[q] = x < gx ? count[t * gx + x] : 0u;
    over |= c[q] > (uint32_t)cap;
    local += c[q];
  }
  const uint32_t incl = wave_inclusive_scan(local);
  uint32_t run = incl - local;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (4 * lane + q < gx) s_pre[wave][4 * lane + q] = run;
    run += c[q];
  }
  const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
  if (force_rescue || __ballot(over) != 0ull || total < (uint32_t)k ||
      total > 64u * KPL) {
    if (lane == 0) fail[1 + atomicAdd(fail, 1u)] = (uint32_t)t;
    return;
  }
  // (a taken item's column could be read again at the end instead of kept
  // in registers: measured slower, the reads then wait one by one)
  const uint2* crow = cand + t * gx * (int64_t)cap;
  const uint32_t* pre = s_pre[wave];
  uint32_t key[KPL], col[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const uint32_t x = (uint32_t)(64 * j + lane);
    key[j] = 0u;
    col[j] = 0u;
    if (x < total) {
      const uint2 e = *wave_item(crow, pre, gx, cap, x);
      key[j] = e.x;
      col[j] = e.y;
    }
  }
  uint32_t thr, k_tie;
  wave_kth_key<KPL>(key, (int)total, (uint32_t)k, s_hist[wave], thr, k_tie);
  wave_emit<KPL>(key, (int)total, thr, k_tie, k, orow,
                 [&](int j, bool) { return col[j]; });
}

// Rescue: workgroup b takes rows fail[1 + b], fail[1 + b + gridDim.x], ..
// of the list's fail[0].  Each of its 16 waves scores pages w, w + 16, ..
// of the row into the workgroup's scratch row with the operations the
// 16-row tile kernel applies to that row.  The row's place in its tile
// (wave w of the tile, w = row - tile start, tiles of 16 rows from the
// request's first row) fixes the order of the N-tiles in the head
// reduction; the linear term's MFMA gets the same A operand as in the tile
// -- the pieces of all four rows of the row's group of four (rows of the
// tile past its end, or with a position the tile does not score, are zero
// there as in the tile), since its outputs are not bit-independent of the
// other A rows.  Then the exact radix select over the scratch row.
template <int MT, bool FULL>
__global__ __launch_bounds__(kTopkThreads) void fused_rescue_kernel(
    LogitsArgs a, int plim, int k, int32_t* __restrict__ out, int64_t out_ld,
    const uint32_t* __restrict__ fail, float* __restrict__ scratch) {
  __shared__ TopkShared sh;
  __shared__ __align__(16) uint8_t s_alin[2048];
  __shared__ __align__(16) float s_asc[4][kLinPieces];
  __shared__ float s_lv[kTopkWaves][kPageTokens];
  const uint32_t nf = fail[0];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = wave_uniform(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  float* srow = scratch + (int64_t)blockIdx.x * a.ld;
  for (uint32_t i = blockIdx.x; i < nf; i += gridDim.x) {
    const int64_t t = wave_uniform((int)fail[1 + i]);
    int32_t* orow = out + t * out_ld;
    const int n = row_len_of(a.positions[t], plim);
    // the request holding row t: the last r with qsl[r] <= t
    int lo = 0, hi = a.R - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (load_uniform(a.qsl, mid) <= t) lo = mid; else hi = mid - 1;
    }
    const int q0 = load_uniform(a.qsl, lo);
    const int q1 = load_uniform(a.qsl, lo + 1);
    if (n <= k || t < q0 || t >= q1) {
      // not a row the tile kernel scores: no candidates to rank
      for (int j = tid; j < k; j += kTopkThreads) orow[j] = -1;
      continue;
    }
    const int p = n - 1;
    const int64_t row0 = q0 + (t - q0) / kTileRows * kTileRows;
    const int tw = (int)(t - row0);            // the row's wave in its tile
    const int wq = tw & 3;
    // the group's linear-term operand: waves 0..3 split the pieces of rows
    // 4 (tw / 4) + wave of the tile
    if (tid < 128)
      *reinterpret_cast<uint4*>(&s_alin[16 * tid]) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    if (wave < 4) {
      const int gw = (tw & ~3) + wave;
      const int64_t tg = row0 + gw;
      bool valid = gw < q1 - row0 && tg < a.T;
      if (valid) {
        const int pg = load_uniform(a.positions, tg);
        valid = !(pg < 0 || pg >= a.ld || (int64_t)(pg >> 6) >= a.bt_stride);
      }
      if (valid) {
        i32x8 qg[MT];
        load_q_frags_cm<MT, FULL>(a.q8 + tg * a.H * kHeadDim, a.H, qg);
        float wa[MT];
        load_a_weights<MT, FULL>(a.weights + tg * a.H, a.q_scale + tg * a.H,
                                 a.H, wa);
        const float2 ql = row_qlin<MT>(qg, wa);
        split_pieces(ql.x, ql.y, wave, &s_alin[0], &s_asc[wave][0]);
      }
    }
    __syncthreads();
    i32x8 alin;
    {
      const uint4 x = *reinterpret_cast<const uint4*>(&s_alin[16 * lane]);
      const uint4 y = *reinterpret_cast<const uint4*>(&s_alin[16 * lane + 1024]);
      alin = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                   (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    }
    const float4 lsc = *reinterpret_cast<const float4*>(&s_asc[wq][0]);
    i32x8 qa[MT];
    load_q_frags_cm<MT, FULL>(a.q8 + t * a.H * kHeadDim, a.H, qa);
    float w[MT][4];
    load_head_weights<MT, FULL>(a.weights + t * a.H, a.q_scale + t * a.H,
                                a.H, w);
    const int tok = 16 * ((wq + g) & 3) + i16;
    const int32_t* bt = a.block_table + (int64_t)lo * a.bt_stride;
    for (int jp = wave; jp <= (p >> 6); jp += kTopkWaves) {
      const int page = load_uniform(bt, jp);
      const bool ok = page >= 0 && (int64_t)page < a.num_pages;
      const uint8_t* pg = a.k_cache + (int64_t)(ok ? page : 0) * kPageBytes;
      // N-tile (wq + nt) mod 4 in turn (a rolled loop: few registers live);
      // its head sum, the same FMA chain as head_reduce_abs, into v[nt]
      float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
#pragma unroll 1
      for (int nt = 0; nt < 4; ++nt) {
        const int nn = (wq + nt) & 3;
        const uint8_t* src = pg + (16 * nn + i16) * kHeadDim + 16 * g;
        const uint4 x = *reinterpret_cast<const uint4*>(src);
        const uint4 y = *reinterpret_cast<const uint4*>(src + 64);
        const i32x8 kb = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                               (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        float vv = 0.f;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const f32x4 acc =
              mfma16x16x128_fp8(qa[m], kb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int j = 0; j < 4; ++j) vv = fmaf(w[m][j], fabsf(acc[j]), vv);
        }
        const f32x4 lin =
            mfma16x16x128_fp8(alin, kb, f32x4{0.f, 0.f, 0.f, 0.f});
        const float lval = fmaf(lsc.w, lin[3],
                           fmaf(lsc.z, lin[2],
                           fmaf(lsc.y, lin[1], lsc.x * lin[0])));
        if (g == wq) s_lv[wave][16 * nn + i16] = lval;
        v0 = nt == 0 ? vv : v0;
        v1 = nt == 1 ? vv : v1;
        v2 = nt == 2 ? vv : v2;
        v3 = nt == 3 ? vv : v3;
      }
      const float tot = reduce_scatter4(v0, v1, v2, v3);
      const float lv = s_lv[wave][tok];
      const float ks =
          ok ? *reinterpret_cast<const float*>(pg + kPageKeyBytes + 4 * tok)
             : 0.f;
      const int s = jp * kPageTokens + tok;
      srow[s] = (s <= p && ok) ? (tot + lv) * ks : -INFINITY;
    }
    // the row's logits, written by every wave, become visible to all
    __threadfence();
    __syncthreads();
    const RowKeys keys{srow, nullptr, 0};
    radix_pass<kHistBins>(keys, n, 0u, 0u, 20, (uint32_t)k, sh);
    topk_radix_rest(keys, n, k, orow, sh);
    __syncthreads();
  }
}

// Workspace of the fused forward after the q codes and scales.
struct FusedLayout {
  int64_t gxm;          // page splits per tile the slots are sized for
  int64_t ld_s;         // sampled columns per row
  int cap;              // candidates per (row, split) slot
  int slots;            // rescue scratch rows
  size_t samp, tlo, count, cand, fail, scr, total;    // byte offsets
};

static FusedLayout fused_layout(int64_t T, int64_t ld, int k) {
  FusedLayout L{};
  const int64_t P = ld / kPageTokens;
  const int64_t rt = (T + kTileRows - 1) / kTileRows;
  // the candidate pass's splits never exceed this (tile grid rule)
  L.gxm = std::max<int64_t>(
      1, std::min<int64_t>((2048 + rt - 1) / rt, (P + 63) / 64));
  L.ld_s = (int64_t)kPageTokens *
           std::min<int64_t>(kFusedMaxSampledPages,
                             (P + kFusedMinStride - 1) / kFusedMinStride);
  // a split covers at least 64 pages; a row's candidates number about k
  // plus a few standard deviations, all of them in one split for a row no
  // longer than it
  const int64_t split_cols =
      (int64_t)kPageTokens * std::max<int64_t>(64, (P + L.gxm - 1) / L.gxm);
  const int64_t want = std::max<int64_t>(2048, ((2 * (int64_t)k + 255) / 256) * 256);
  // (more than kFusedCandMax candidates in a row go to the rescue anyway)
  L.cap = (int)std::min<int64_t>(std::min<int64_t>(split_cols, want),
                                 kFusedCandMax);
  L.slots = (int)std::min<int64_t>(T, kFusedRescueSlots);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.samp = take((size_t)T * L.ld_s * 4);
  L.tlo = take((size_t)T * 4);
  L.count = take((size_t)T * L.gxm * 4);
  L.cand = take((size_t)T * L.gxm * L.cap * 8);
  L.fail = take((size_t)(T + 1) * 4);
  L.scr = take((size_t)L.slots * ld * 4);
  L.total = off;
  return L;
}

size_t fused_workspace_bytes(int64_t T, int64_t ld, int k) {
  if (T <= 0 || ld <= 0) return 0;
  return fused_layout(T, ld, k).total;
}

hipError_t launch_forward_fused(const ForwardArgs& f, void* ws,
                                hipStream_t stream) {
  const LogitsArgs& a = f.lg;
  const int64_t T = a.T;
  if (T <= 0) return hipSuccess;
  const int k = f.tk.k;
  const FusedLayout L = fused_layout(T, a.ld, k);
  char* base = static_cast<char*>(ws);
  float* samp = reinterpret_cast<float*>(base + L.samp);
  uint32_t* tlo = reinterpret_cast<uint32_t*>(base + L.tlo);
  uint32_t* count = reinterpret_cast<uint32_t*>(base + L.count);
  uint2* cand = reinterpret_cast<uint2*>(base + L.cand);
  uint32_t* fail = reinterpret_cast<uint32_t*>(base + L.fail);
  float* scr = reinterpret_cast<float*>(base + L.scr);
  const Options o = options();
  const int64_t max_pages = std::min<int64_t>(a.bt_stride, a.ld / kPageTokens);
  // every 32nd page unless set: about 1/32 of the scoring, and about
  // k + 48 * 32 candidates per long row (the sample rule below)
  int64_t SS = o.fused_sample_stride > 0 ? o.fused_sample_stride
                                         : 2 * kFusedMinStride;
  SS = std::max<int64_t>(SS, (max_pages + kFusedMaxSampledPages - 1) /
                                 kFusedMaxSampledPages);
  const int64_t gx = fused_candidate_splits(a);
  if (gx < 1 || gx > L.gxm) return hipErrorInvalidValue;
  int cap = L.cap;
  if (o.fused_cand_cap > 0) cap = std::min(cap, o.fused_cand_cap);
  const int plim = pos_limit(f.tk);

  hipError_t e = launch_quantize_q(f.q_bf16, T * a.H, f.q8, f.q_scale, stream);
  if (e == hipSuccess)
    e = launch_logits_sample(a, (int)SS, samp, L.ld_s, stream);
  if (e != hipSuccess) return e;
  const unsigned wgs = (unsigned)((T + kWaveRowsPerWg - 1) / kWaveRowsPerWg);
  // sampled columns of the longest row: 64 * ceil(max_pages / SS)
  const int64_t ns_max =
      (int64_t)kPageTokens * ((max_pages + SS - 1) / SS);
#define DSA_THR_WAVE(KPL)                                                     \
    hipLaunchKernelGGL(fused_threshold_wave_kernel<KPL>, dim3(wgs),           \
                       dim3(64 * kWaveRowsPerWg), 0, stream, samp, L.ld_s,    \
                       a.positions, T, plim, (int)SS, k, tlo, fail);
  if (ns_max <= 64 * 16) { DSA_THR_WAVE(16) }
  else if (ns_max <= 64 * 40) { DSA_THR_WAVE(40) }
  else if (ns_max <= 64 * 64) { DSA_THR_WAVE(64) }
#undef DSA_THR_WAVE
  else
    hipLaunchKernelGGL((fused_threshold_kernel<kTopkThreads, 4>),
                       dim3((unsigned)T), dim3(kTopkThreads), 0, stream, samp,
                       L.ld_s, a.positions, plim, (int)SS, k, tlo, fail);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  FusedTile ft;
  ft.tlo = tlo;
  ft.cand = cand;
  ft.count = count;
  ft.cap = cap;
  if ((e = launch_logits_candidates(a, ft, gx, stream)) != hipSuccess)
    return e;
  // a row's candidates number about k + (4 sqrt(k / SS) + 16) SS (the
  // sample rule; 4 standard deviations and more below the wave kernels'
  // capacity)
  const double c_est =
      k + (4.0 * std::sqrt((double)k / (double)SS) + 16.0) * (double)SS;
  const int force = o.fused_force_rescue ? 1 : 0;
  // one wave per row (its items found by a four-step search over at most
  // 16 splits) when the list fits 80 % of its capacity, else the
  // 1024-thread workgroup (measured on the prefill chunk: 0.12-0.16 ms
  // against 0.27 ms; a 256-thread workgroup per row with the wave kernel's
  // range-adaptive digits measured 0.24 ms)
  const int qsel = o.fused_select;
  const bool wave_ok = gx <= kWaveMaxSplits;
  if (wave_ok && (qsel == 1 || (qsel == 0 && c_est <= 0.8 * 64 * 64)))
    hipLaunchKernelGGL(fused_select_wave_kernel<64>, dim3(wgs),
                       dim3(64 * kWaveRowsPerWg), 0, stream, a.positions,
                       a.qsl, a.R, T, plim, k, f.tk.out, f.tk.out_ld, count,
                       cand, (int)gx, cap, force, fail);
  else if (wave_ok && (qsel == 2 || (qsel == 0 && c_est <= 0.8 * 64 * 80)))
    hipLaunchKernelGGL(fused_select_wave_kernel<80>, dim3(wgs),
                       dim3(64 * kWaveRowsPerWg), 0, stream, a.positions,
                       a.qsl, a.R, T, plim, k, f.tk.out, f.tk.out_ld, count,
                       cand, (int)gx, cap, force, fail);
  else
    hipLaunchKernelGGL(fused_select_kernel, dim3((unsigned)T),
                       dim3(kTopkThreads), 0, stream, a.positions, a.qsl, a.R,
                       plim, k, f.tk.out, f.tk.out_ld, count, cand, (int)gx,
                       cap, force, fail);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 rg((unsigned)L.slots);
  auto rescue = [&](auto mt, auto full) {
    constexpr int MT = decltype(mt)::value;
    constexpr bool FULL = decltype(full)::value;
    hipLaunchKernelGGL((fused_rescue_kernel<MT, FULL>), rg,
                       dim3(kTopkThreads), 0, stream, a, plim, k, f.tk.out,
                       f.tk.out_ld, fail, scr);
  };
  switch (a.H) {
    case 16: rescue(std::integral_constant<int, 1>(), std::true_type()); break;
    case 32: rescue(std::integral_constant<int, 2>(), std::true_type()); break;
    case 48: rescue(std::integral_constant<int, 3>(), std::true_type()); break;
    case 64: rescue(std::integral_constant<int, 4>(), std::true_type()); break;
    default:
      switch ((a.H + 15) / 16) {
        case 1: rescue(std::integral_constant<int, 1>(), std::false_type()); break;
        case 2: rescue(std::integral_constant<int, 2>(), std::false_type()); break;
        case 3: rescue(std::integral_constant<int, 3>(), std::false_type()); break;
        default: rescue(std::integral_constant<int, 4>(), std::false_type()); break;
      }
  }
  return hipGetLastError();
}

size_t topk_workspace_bytes(int64_t T, int64_t ld, int k) {
  (void)k;
  if (T <= 0 || !use_multi_wg(ld)) return 0;
  // room for either long-row path (the option can switch between them)
  size_t mw = 0, ss = 0;
  carve(nullptr, T, ld, &mw);
  if (use_sample_select(ld)) ss_carve(nullptr, T, ld, &ss);
  return std::max(mw, ss);
}

template <bool KEY32>
static hipError_t launch_topk_single_t(const TopkArgs& a, hipStream_t stream,
                                       int max_cache, size_t elem) {
  const int cap = (int)std::min<int64_t>(a.ld, max_cache);
  const size_t dyn = (size_t)cap * elem;
  // the dynamic-LDS limit is a per-device attribute of the kernel: set once
  // on each device the library launches on (setting it twice is harmless)
  static std::atomic<bool> attr_set[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !attr_set[dev].load()) {
    e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(topk_row_kernel<KEY32>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)(max_cache * elem));
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) attr_set[dev].store(true);
  }
  hipLaunchKernelGGL(topk_row_kernel<KEY32>, dim3((unsigned)a.T),
                     dim3(kTopkThreads), dyn, stream, a.logits, a.ld,
                     a.positions, a.k, a.out, a.out_ld, cap, pos_limit(a));
  return hipGetLastError();
}

// Compute units of the current device (queried once per device).
int device_cu_count() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return 256;
  int n = cached[dev].load();
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n);
  }
  return n;
}

template <int S>
static hipError_t launch_topk_reg_t(const TopkArgs& a, hipStream_t stream) {
  // one resident workgroup per compute unit; each loops over its rows
  const int64_t grid = std::min<int64_t>(a.T, device_cu_count());
  // the bitmap emit when the longest rows take fewer than 1/8 of their keys
  if ((int64_t)a.k * 8 < a.ld)
    hipLaunchKernelGGL((topk_reg_kernel<S, true, kTopkThreads, true>),
                       dim3((unsigned)grid), dim3(kTopkThreads), 0, stream,
                       a.logits, a.ld, a.positions, a.k, a.out, a.out_ld, a.T,
                       pos_limit(a));
  else
    hipLaunchKernelGGL((topk_reg_kernel<S, false, kTopkThreads, true>),
                       dim3((unsigned)grid), dim3(kTopkThreads), 0, stream,
                       a.logits, a.ld, a.positions, a.k, a.out, a.out_ld, a.T,
                       pos_limit(a));
  return hipGetLastError();
}

// 512-thread workgroups without the register prefetch, two per compute
// unit.  A row's selection is a chain of histogram passes and barriers that
// leaves one 1024-thread workgroup waiting about half its cycles; with two
// workgroups each one's loads and waits overlap the other's work.
constexpr int kReg2Threads = 512;
template <int S, bool BITMAP = true>
static hipError_t launch_topk_reg2_t(const TopkArgs& a, hipStream_t stream) {
  const int64_t grid = std::min<int64_t>(a.T, 2 * (int64_t)device_cu_count());
  hipLaunchKernelGGL((topk_reg_kernel<S, BITMAP, kReg2Threads, false>),
                     dim3((unsigned)grid), dim3(kReg2Threads), 0, stream,
                     a.logits, a.ld, a.positions, a.k, a.out, a.out_ld, a.T,
                       pos_limit(a));
  return hipGetLastError();
}

// dense selections (rows of up to 8 slices of 2048 columns)
constexpr int kReg2DenseMaxRow = 8 * 4 * kReg2Threads;    // 16384
static hipError_t launch_topk_reg2_dense(const TopkArgs& a,
                                         hipStream_t stream) {
  constexpr int kSl = 4 * kReg2Threads;
  switch ((a.ld + kSl - 1) / kSl) {
#define DSA_REG2D(N) case N: return launch_topk_reg2_t<N, false>(a, stream);
    DSA_REG2D(1) DSA_REG2D(2) DSA_REG2D(3) DSA_REG2D(4) DSA_REG2D(5)
    DSA_REG2D(6) DSA_REG2D(7)
#undef DSA_REG2D
    default: return launch_topk_reg2_t<8, false>(a, stream);
  }
}

static hipError_t launch_topk_reg2(const TopkArgs& a, hipStream_t stream) {
  constexpr int kSl = 4 * kReg2Threads;
  switch ((a.ld + kSl - 1) / kSl) {
#define DSA_REG2(N) case N: return launch_topk_reg2_t<N>(a, stream);
    DSA_REG2(1) DSA_REG2(2) DSA_REG2(3) DSA_REG2(4) DSA_REG2(5) DSA_REG2(6)
    DSA_REG2(7) DSA_REG2(8) DSA_REG2(9) DSA_REG2(10) DSA_REG2(11)
    DSA_REG2(12) DSA_REG2(13) DSA_REG2(14) DSA_REG2(15) DSA_REG2(16)
    DSA_REG2(17) DSA_REG2(18) DSA_REG2(19) DSA_REG2(20) DSA_REG2(21)
    DSA_REG2(22) DSA_REG2(23)
#undef DSA_REG2
    default: return launch_topk_reg2_t<24>(a, stream);
  }
}

static hipError_t launch_topk_reg(const TopkArgs& a, hipStream_t stream) {
  // more rows than compute units: two 512-thread workgroups per compute
  // unit (measured: prefill rows 0.46 -> 0.39 ms; 384 / 1024 dense decode
  // rows of 8192 columns 11.6 -> 9.5 / 22.6 -> 17.6 us); otherwise one
  // 1024-thread workgroup per row, faster when every row has a compute unit
  // to itself (64 rows: 6.5 against 6.9 us).  Option 1 / 4 force either.
  const int opt = options().topk_kernel;
  const bool two =
      opt == 4 || (opt != 1 && a.T > (int64_t)device_cu_count());
  if (two && (int64_t)a.k * 8 < a.ld) return launch_topk_reg2(a, stream);
  if (two && a.ld <= kReg2DenseMaxRow) return launch_topk_reg2_dense(a, stream);
  switch ((a.ld + kRegSlice - 1) / kRegSlice) {
    case 1: return launch_topk_reg_t<1>(a, stream);
    case 2: return launch_topk_reg_t<2>(a, stream);
    case 3: return launch_topk_reg_t<3>(a, stream);
    case 4: return launch_topk_reg_t<4>(a, stream);
    case 5: return launch_topk_reg_t<5>(a, stream);
    case 6: return launch_topk_reg_t<6>(a, stream);
    case 7: return launch_topk_reg_t<7>(a, stream);
    case 8: return launch_topk_reg_t<8>(a, stream);
    case 9: return launch_topk_reg_t<9>(a, stream);
    case 10: return launch_topk_reg_t<10>(a, stream);
    case 11: return launch_topk_reg_t<11>(a, stream);
    default: return launch_topk_reg_t<12>(a, stream);
  }
}

static hipError_t launch_topk_single(const TopkArgs& a, hipStream_t stream) {
  // register-resident kernel unless disabled (option 2) or the row is too
  // long for it; it needs 16-byte aligned rows (ld is a multiple of 256)
  const bool aligned = (reinterpret_cast<uintptr_t>(a.logits) & 15u) == 0;
  if (options().topk_kernel != 2 && a.ld <= kRegMaxRow && aligned)
    return launch_topk_reg(a, stream);
  if (a.ld <= kMaxCachedFull)
    return launch_topk_single_t<true>(a, stream, kMaxCachedFull, 4);
  return launch_topk_single_t<false>(a, stream, kMaxCachedHi, 2);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  if (!use_multi_wg(a.ld)) return launch_topk_single(a, stream);
  const bool aligned = (reinterpret_cast<uintptr_t>(a.logits) & 15u) == 0;
  if (use_sample_select(a.ld) && aligned && options().topk_kernel != 3) {
    SsWorkspace ss = ss_carve(a.workspace, a.T, a.ld, nullptr);
    ss.plim = pos_limit(a);
    hipLaunchKernelGGL(ss_gather_kernel, dim3(kSsGatherWgs, (unsigned)a.T),
                       dim3(kSsThreads), 0, stream, a.logits, a.ld,
                       a.positions, a.k, ss);
    hipLaunchKernelGGL(ss_sample_kernel, dim3((unsigned)a.T),
                       dim3(kTopkThreads), 0, stream, a.logits, a.ld,
                       a.positions, a.k, ss);
    hipLaunchKernelGGL(ss_collect_kernel, dim3((unsigned)ss.C, (unsigned)a.T),
                       dim3(kSsThreads), 0, stream, a.logits, a.ld,
                       a.positions, a.k, ss);
    hipLaunchKernelGGL(ss_select_kernel, dim3((unsigned)a.T),
                       dim3(kTopkThreads), 0, stream, a.logits, a.ld,
                       a.positions, a.k, a.out, a.out_ld, ss);
    return hipGetLastError();
  }
  MwWorkspace ws = carve(a.workspace, a.T, a.ld, nullptr);
  ws.plim = pos_limit(a);
  const size_t zb = mw_zero_bytes(a.T, a.ld);
  const size_t n16 = zb / 16;
  hipLaunchKernelGGL(mw_clear_kernel,
                     dim3((unsigned)std::min<size_t>((n16 + 255) / 256, 1024)),
                     dim3(256), 0, stream, static_cast<uint4*>(a.workspace), n16);
  const dim3 grid((unsigned)ws.C, (unsigned)a.T);
  hipLaunchKernelGGL(mw_pass1_kernel, grid, dim3(kMwThreads), 0, stream,
                     a.logits, a.ld, a.positions, a.k, ws);
  hipLaunchKernelGGL(mw_pass2_kernel, grid, dim3(kMwThreads), 0, stream,
                     a.logits, a.ld, a.positions, a.k, ws);
  hipLaunchKernelGGL(mw_write_kernel, grid, dim3(kMwThreads), 0, stream,
                     a.logits, a.ld, a.positions, a.k, a.out, a.out_ld, ws);
  return hipGetLastError();
}

}  // namespace dsa
