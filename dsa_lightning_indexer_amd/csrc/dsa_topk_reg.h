// Register-resident exact top-k of one row per workgroup, shared by the
// top-k kernels and the one-launch decode forward: order-preserving keys in
// registers, up to three LDS histogram passes (top 12 key bits, bits 19..8
// inside the boundary bin, bits 7..0 inside the 24-bit prefix) and an emit
// of the selected columns in ascending order, ties at the k-th value taken
// lowest column first.
#pragma once

#include "dsa_common.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kHistBins = 4096;

// Columns a row ranks: n = p + 1, or 0 (a row of -1) for a position the
// logits call leaves unscored -- p < 0, or p >= plim (past the logits row,
// or past the rows' block-table entries in the forward pass).
__device__ __forceinline__ int row_len_of(int p, int plim) {
  return (p < 0 || p >= plim) ? 0 : p + 1;
}

// Bin search on an LDS histogram: the bin where the count of larger keys
// first reaches k_rem, scanning from the top.  4096 bins: thread tid owns
// 4096/NT consecutive bins from 4095 - (4096/NT) tid down; a DPP scan in
// each wave and the per-wave totals in LDS give every thread the count
// above its bins (two barriers).  256 bins: wave 0 alone, 4 per lane.
// Results in sh.sel_digit / sel_above / sel_count.  Call from all threads.
template <int NBINS, int NT, typename Shared>
__device__ void topk_select_bin(const uint32_t* hist, uint32_t k_rem,
                                Shared& sh) {
  static_assert(NBINS == 4096 || NBINS == 256, "bins");
  static_assert(NBINS == 256 || NBINS % NT == 0, "threads");
  constexpr int B = (NBINS == 4096) ? 4096 / NT : 4;
  constexpr int NW = NT / 64;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const bool active = NBINS == 4096 || wave == 0;
  const int top = (NBINS == 4096) ? 4095 - B * (int)threadIdx.x
                                  : 255 - 4 * lane;
  uint32_t c[B];
  uint32_t local = 0u;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    c[j] = active ? hist[top - j] : 0u;
    local += c[j];
  }
  const uint32_t incl = wave_inclusive_scan(local);
  uint32_t above_w = 0u;
  if (NBINS == 4096 && NW > 1) {
    if (lane == 63) sh.wave_sum[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave; ++w) above_w += sh.wave_sum[w];
  }
  uint32_t above = above_w + incl - local;
  if (active && above < k_rem && above + local >= k_rem) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
      if (above + c[j] >= k_rem) {
        sh.sel_digit = (uint32_t)(top - j);
        sh.sel_above = above;
        sh.sel_count = c[j];
        break;
      }
      above += c[j];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Register-resident top-k for rows of up to kRegMaxRow columns (decode rows,
// prefill rows): one workgroup of 1024 threads per row, the row's keys in
// registers.
// ---------------------------------------------------------------------------
template <int NT, int S>
struct RegTopkShared {
  __align__(16) uint32_t hist[kHistBins];
  __align__(16) uint32_t hist2[kHistBins];
  __align__(16) uint32_t hist3[256];           // pass 3 (bits 7..0)
  uint32_t tot[S * (NT / 64)];                 // packed per (slice, wave)
  uint32_t wave_sum[NT / 64];
  uint32_t sel_digit, sel_above, sel_count;
  // column bitmaps of the keys above the threshold and of the ties
  uint32_t selw[S * NT / 8];
  uint32_t tiew[S * NT / 8];
};

// Keys held in registers: item s * 4 NT + 4 tid + j of a list in key[s][j]
// (slice s, j = 0..3, NT threads), valid when that item index is below n
// (no per-key mask registers).
template <int S, int NT = kTopkThreads>
struct RegKeys {
  uint32_t key[S][4];
  int n;
  // written as (per-lane offset) < (uniform bound) so that only 4 *
  // threadIdx.x + j lives in vector registers
  __device__ __forceinline__ bool ok(int s, int j) const {
    return 4 * (int)threadIdx.x + j < n - s * 4 * NT;
  }
};

// Clears the three histograms reg_threshold expects zero (16-byte stores);
// the caller then passes a barrier before calling it.
template <int NT, int S>
__device__ __forceinline__ void reg_clear(RegTopkShared<NT, S>& sh) {
  for (int b = 4 * (int)threadIdx.x; b < kHistBins; b += 4 * NT) {
    *reinterpret_cast<uint4*>(&sh.hist[b]) = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(&sh.hist2[b]) = make_uint4(0u, 0u, 0u, 0u);
  }
  if (4 * (int)threadIdx.x < 256)
    *reinterpret_cast<uint4*>(&sh.hist3[4 * threadIdx.x]) =
        make_uint4(0u, 0u, 0u, 0u);
}

// The bin of the k_rem-th largest key of a 4096-bin histogram (bins taken
// from the top), found by every wave itself after one barrier: thread t
// owns bins 4095 - B t down to 4096 - B (t + 1) (B = 4096 / NT); each wave
// scans its bins and publishes its total; after the barrier every wave
// scans the totals, finds the wave that owns the bin, reads that wave's
// bins from LDS and scans them again -- so the result (d, the count of keys
// above it, its count) is in registers of every wave without a second
// barrier.  k_rem must not exceed the histogram's total.
template <int NT>
__device__ __forceinline__ void select_bin_all(const uint32_t* hist,
                                               uint32_t k_rem,
                                               uint32_t* wave_sum, uint32_t& d,
                                               uint32_t& above,
                                               uint32_t& count) {
  constexpr int B = kHistBins / NT;
  constexpr int NW = NT / 64;
  static_assert(B * NT == kHistBins && NW <= 64, "bins per thread");
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  uint32_t local = 0u;
  {
    const int top = kHistBins - 1 - B * (int)threadIdx.x;
#pragma unroll
    for (int j = 0; j < B; ++j) local += hist[top - j];
  }
  const uint32_t incl = wave_inclusive_scan(local);
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  const uint32_t wt = lane < NW ? wave_sum[lane] : 0u;
  const uint32_t wincl = wave_inclusive_scan(wt);
  const int ws =
      __builtin_ctzll(__ballot(lane < NW && wincl >= k_rem));
  const uint32_t above_w =
      __builtin_amdgcn_readlane(wincl - wt, ws);
  uint32_t c[B];
  uint32_t l2 = 0u;
  const int top = kHistBins - 1 - B * (64 * ws + lane);
#pragma unroll
  for (int j = 0; j < B; ++j) {
    c[j] = hist[top - j];
    l2 += c[j];
  }
  const uint32_t i2 = wave_inclusive_scan(l2);
  uint32_t a = above_w + i2 - l2;
  const int ls = __builtin_ctzll(__ballot(a < k_rem && a + l2 >= k_rem));
  int jj = 0;
  uint32_t ab = 0u, cn = 0u;
  bool found = false;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    if (!found && a + c[j] >= k_rem) {
      found = true;
      jj = j;
      ab = a;
      cn = c[j];
    }
    a += c[j];
  }
  d = (uint32_t)(kHistBins - 1 - B * (64 * ws + ls) -
                 __builtin_amdgcn_readlane(jj, ls));
  above = __builtin_amdgcn_readlane(ab, ls);
  count = __builtin_amdgcn_readlane(cn, ls);
}

// Threshold of the k largest valid keys (k < number of valid keys): a key
// is selected when (key & mask) > thr, or (key & mask) == thr and it is
// among the k_tie lowest-position such keys.  Up to three LDS histograms
// (top 12 key bits over the list; bits 19..8 over the keys of the chosen
// bin; bits 7..0 over the keys matching the 24-bit prefix), each its own
// array, so none is cleared while a wave may still read it.  The first
// bin search is select_bin_all (one barrier) for instances of up to 4
// slices; wider ones keep their registers for the keys and use the
// two-barrier search throughout.  reg_clear and a barrier must precede the
// call.  Call from all NT threads.  n_eq (optional) receives the number of
// valid keys equal to thr under mask; k_tie == n_eq means every tied key is
// selected.
template <int NT, int S>
__device__ void reg_threshold(const RegKeys<S, NT>& r, int k,
                              RegTopkShared<NT, S>& sh, uint32_t& mask,
                              uint32_t& thr, uint32_t& k_tie,
                              uint32_t* n_eq = nullptr) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (r.ok(s, j)) atomicAdd(&sh.hist[r.key[s][j] >> 20], 1u);
  __syncthreads();
  uint32_t d, above, count;
  if constexpr (S <= 4) {
    select_bin_all<NT>(sh.hist, (uint32_t)k, sh.wave_sum, d, above, count);
  } else {
    topk_select_bin<kHistBins, NT>(sh.hist, (uint32_t)k, sh);
    d = sh.sel_digit;
    above = sh.sel_above;
    count = sh.sel_count;
  }
  const uint32_t k_rem = (uint32_t)k - above;
  mask = 0xfff00000u; thr = d << 20; k_tie = k_rem;
  if (n_eq) *n_eq = count;
  if (k_rem < count) {
    // pass 2: bits 19..8 of the keys in bin d (hist2; hist may still be
    // read by waves finishing the first bin search, so pass 3 has its own
    // histogram)
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (r.ok(s, j) && (r.key[s][j] >> 20) == d)
          atomicAdd(&sh.hist2[(r.key[s][j] >> 8) & 0xfffu], 1u);
    __syncthreads();
    topk_select_bin<kHistBins, NT>(sh.hist2, k_rem, sh);
    const uint32_t p24 = (d << 12) | sh.sel_digit;
    const uint32_t k2 = k_rem - sh.sel_above;
    const uint32_t c2 = sh.sel_count;
    mask = 0xffffff00u; thr = p24 << 8; k_tie = k2;
    if (n_eq) *n_eq = c2;
    if (k2 < c2) {
      // pass 3: bits 7..0 of the keys matching the 24-bit prefix
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (r.ok(s, j) && (r.key[s][j] >> 8) == p24)
            atomicAdd(&sh.hist3[r.key[s][j] & 0xffu], 1u);
      __syncthreads();
      topk_select_bin<256, NT>(sh.hist3, k2, sh);
      mask = 0xffffffffu; thr = (p24 << 8) | sh.sel_digit;
      k_tie = k2 - sh.sel_above;
      if (n_eq) *n_eq = sh.sel_count;
    }
  }
}

// Largest / smallest of x over the wave (DPP within rows of 16 lanes, then
// the four row results).
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xf, 0xf, false));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)x, 0),
                 (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)x, 32),
                 (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
  return ~wave_umax(~x);
}

// Writes the selected items in list order: the output slot of an item is
// the number of selected items before it, from packed (above, tie) counts
// per thread and slice, a DPP scan within the wave and a scan of the
// per-wave totals; orow[slot] = index_of(s, j, position in the list).
template <int NT, int S, typename IndexOf>
__device__ void reg_emit(const RegKeys<S, NT>& r, int k, uint32_t mask,
                         uint32_t thr, uint32_t k_tie, int32_t* orow,
                         RegTopkShared<NT, S>& sh, IndexOf index_of) {
  constexpr int NW = NT / 64;
  constexpr int kSlice = 4 * NT;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  // packed per-slice counts: above in bits 0..15, ties in bits 16..31; only
  // the exclusive prefix within the wave is kept
  uint32_t excl[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    uint32_t c = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = r.ok(s, j);
      const uint32_t km = r.key[s][j] & mask;
      c += (ok && km > thr) ? 1u : 0u;
      c += (ok && km == thr) ? 0x10000u : 0u;
    }
    const uint32_t incl = wave_inclusive_scan(c);
    excl[s] = incl - c;
    if (lane == 63) sh.tot[s * NW + wave] = incl;
  }
  __syncthreads();
  // every wave scans the S * NW (slice, wave) totals itself (exclusive, in
  // (slice, wave) order; lane l holds entries kPer l ..), then takes the
  // entry of (s, its wave) from the lane holding it: no second barrier
  constexpr int kPer = (S * NW + 63) / 64;
  uint32_t ex[kPer];
  {
    uint32_t v[kPer], local = 0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = lane * kPer + i;
      v[i] = idx < S * NW ? sh.tot[idx] : 0u;
      local += v[i];
    }
    uint32_t run = wave_inclusive_scan(local) - local;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      ex[i] = run;
      run += v[i];
    }
  }
  auto base_of = [&](int s) {
    const int idx = s * NW + wave;            // wave-uniform
    uint32_t x = ex[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i)
      if (idx % kPer == i) x = ex[i];
    return __builtin_amdgcn_readlane(x, idx / kPer);
  };
  // 4 tid through an empty asm: the column indices below are then computed
  // where they are used instead of being hoisted out of a caller's row loop
  // as S x 4 loop-invariant registers
  int tid4 = 4 * tid;
  asm volatile("" : "+v"(tid4));
  // Branch-free: a key above the threshold, or one of the first k_tie keys
  // equal to it, goes to slot gt_b + min(eq_b, k_tie) (for a taken tie
  // eq_b < k_tie, so this is gt_b + eq_b); every key issues a store, and
  // one not taken is pushed past the end of the row's k-slot buffer and
  // dropped.  Slots are < k by construction; the buffer bound keeps a
  // row's writes inside the row whatever the counts.
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(orow, k * 4);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint32_t before = base_of(s) + excl[s];
    uint32_t gt_b = before & 0xffffu, eq_b = before >> 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = r.ok(s, j);
      const uint32_t km = r.key[s][j] & mask;
      const int pos = s * kSlice + tid4 + j;
      const bool gt = ok && km > thr;
      const bool eq = ok && km == thr;
      const bool take = gt || (eq && eq_b < k_tie);
      const uint32_t slot = gt_b + min(eq_b, k_tie);
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)index_of(s, j, pos), ro,
                                            take ? (int)(4 * slot) : 4 * k, 0,
                                            0);
      gt_b += gt ? 1u : 0u;
      eq_b += eq ? 1u : 0u;
    }
  }
}

// The same output for a list whose item index is its column: the selected
// and tied keys go into column bitmaps (a thread's 4 keys of slice s are the
// nibble 4 (tid % 8) of word s NT / 8 + tid / 8; 8 lanes OR-combine their
// nibbles with DPP and one writes the word, so every word of the row is
// written once, no atomics), one workgroup scan over the words' packed
// (selected, tie) counts gives every word its first slot, and each lane
// expands only the set bits of its words.  Ties are taken lowest column
// first up to k_tie.
template <int NT, int S>
__device__ void reg_emit_columns(const RegKeys<S, NT>& r, int k, uint32_t mask,
                                 uint32_t thr, uint32_t k_tie, int32_t* orow,
                                 RegTopkShared<NT, S>& sh,
                                 bool all_ties = false) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  auto or8 = [](uint32_t x) {
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false);
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false);
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xf, 0xf, false);
    return x;
  };
  const int sh4 = 4 * (tid & 7);
  if (all_ties) {
    // every tied key taken: one bitmap of the keys at or above the
    // threshold, no tie words.  thr is zero below the bits mask keeps, so
    // (key & mask) >= thr is key >= thr; a thread's valid keys of a slice
    // are a prefix of its four
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int lim = r.n - s * 4 * NT - 4 * tid;
      const uint32_t valid =
          lim >= 4 ? 0xfu : (lim <= 0 ? 0u : (1u << lim) - 1u);
      uint32_t sel = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) sel |= r.key[s][j] >= thr ? (1u << j) : 0u;
      sel = or8((sel & valid) << sh4);
      if ((tid & 7) == 0) sh.selw[s * (NT / 8) + (tid >> 3)] = sel;
    }
  } else {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      uint32_t sel = 0u, tie = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = r.ok(s, j);
        const uint32_t km = r.key[s][j] & mask;
        sel |= (ok && km > thr) ? (1u << j) : 0u;
        tie |= (ok && km == thr) ? (1u << j) : 0u;
      }
      sel = or8(sel << sh4);
      tie = or8(tie << sh4);
      if ((tid & 7) == 0) {
        sh.selw[s * (NT / 8) + (tid >> 3)] = sel;
        sh.tiew[s * (NT / 8) + (tid >> 3)] = tie;
      }
    }
  }
  __syncthreads();
  // thread tid owns words WPT tid .. WPT tid + WPT - 1 of the row's
  // ceil(n / 32) (S NT / 8 words in all; at least 2 per thread)
  constexpr int WPT = (S * NT / 8 + NT - 1) / NT > 2
                          ? (S * NT / 8 + NT - 1) / NT : 2;
  const int nw = (r.n + 31) >> 5;
  const int w0 = WPT * tid;
  uint32_t sw_[WPT], tw_[WPT];
  uint32_t n_sel = 0u, n_tie = 0u;
#pragma unroll
  for (int h = 0; h < WPT; ++h) {
    sw_[h] = 0u;
    tw_[h] = 0u;
    if (w0 + h < nw) {
      sw_[h] = sh.selw[w0 + h];
      tw_[h] = all_ties ? 0u : sh.tiew[w0 + h];
    }
    n_sel += (uint32_t)__builtin_popcount(sw_[h]);
    n_tie += (uint32_t)__builtin_popcount(tw_[h]);
  }
  const uint32_t c = n_sel | (n_tie << 16);
  const uint32_t incl = wave_inclusive_scan(c);
  if (lane == 63) sh.wave_sum[wave] = incl;
  __syncthreads();
  uint32_t before = incl - c;
  for (int w = 0; w < wave; ++w) before += sh.wave_sum[w];
  uint32_t gt_b = before & 0xffffu, eq_b = before >> 16;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(orow, k * 4);
#pragma unroll
  for (int h = 0; h < WPT; ++h) {
    const uint32_t sw = sw_[h], tw = tw_[h];
    uint32_t any = sw | tw;
    while (any) {
      const int b = __builtin_ctz(any);
      any &= any - 1u;
      const bool is_sel = (sw >> b) & 1u;
      const bool take = is_sel || eq_b < k_tie;
      const uint32_t slot = gt_b + min(eq_b, k_tie);
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(32 * (w0 + h) + b), ro,
                                            take ? (int)(4 * slot) : 4 * k, 0,
                                            0);
      gt_b += is_sel ? 1u : 0u;
      eq_b += is_sel ? 0u : 1u;
    }
  }
}

// Top-k of row[0..n) (k < n <= S * 4 * NT <= ld) into orow[0..k), in
// ascending column order.  Thread tid holds columns s * 4 NT + 4 tid + j in
// registers: one 16-byte load per slice, no LDS copy of the row.  `row`
// must be 16-byte aligned and ld a multiple of 4.  Call from all NT
// threads.
template <int NT, int S>
__device__ void topk_row_registers(const float* row, int64_t ld, int n, int k,
                                   int32_t* orow, RegTopkShared<NT, S>& sh) {
  constexpr int kSlice = 4 * NT;
  const int tid = threadIdx.x;
  reg_clear(sh);
  RegKeys<S, NT> r;
  r.n = n;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c0 = s * kSlice + 4 * tid;
    r.key[s][0] = r.key[s][1] = r.key[s][2] = r.key[s][3] = 0u;
    if (s * kSlice < n) {                     // workgroup-uniform
      const float4 v =
          *reinterpret_cast<const float4*>(row + min(c0, (int)ld - 4));
      r.key[s][0] = float_to_ordered(v.x);
      r.key[s][1] = float_to_ordered(v.y);
      r.key[s][2] = float_to_ordered(v.z);
      r.key[s][3] = float_to_ordered(v.w);
    }
  }
  __syncthreads();
  uint32_t mask, thr, k_tie;
  reg_threshold<NT, S>(r, k, sh, mask, thr, k_tie);
  reg_emit<NT, S>(r, k, mask, thr, k_tie, orow, sh,
                  [](int, int, int pos) { return pos; });
}

// Row with n <= k columns: 0..n-1, then -1 (n <= 0: all -1).
template <int NT>
__device__ __forceinline__ void topk_row_short(int n, int k, int32_t* orow) {
  for (int i = threadIdx.x; i < k; i += NT) orow[i] = i < n ? i : -1;
}

}  // namespace dsa
