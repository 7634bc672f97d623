// gfx950 kernels for the first half of the lightning-indexer hot path:
//   * q quantisation (bf16 -> e4m3fn codes + one fp32 scale per 128 block),
//   * paged FP8 logits: per-head FP8 MFMA dot products q_h . k_s, ReLU, the
//     per-head weighted sum, the K scale and the causal bound.
//
// Score: for query row t at position p and cached token s <= p,
//   logit[t, s] = sum_h w[t,h] * max(qhat[t,h,:] . khat[s,:], 0)
// (the DeepSeek Sparse Attention lightning-indexer score of DeepSeek-V3.2,
// arXiv:2512.02556, which the GLM-5.3 cache-budget article cites; the pages
// name the indexer and an fp8_index operator -- Ascend msmodeling DeepSeek-V3.2
// RFC, section 2.1.3 -- but print no formula).  With qhat = code_q * s_q and
// khat = code_k * s_k, s_q, s_k >= 0, this equals
//   s_k[s] * sum_h (w[t,h] * s_q[t,h]) * max(code_q[t,h,:] . code_k[s,:], 0),
// so the MFMA contracts raw FP8 codes and both scales are applied in the
// fp32 epilogue.
//
// Paging (vLLM HBM-index notes, section 2.3; GLM-5.3 article, SGLang
// buffer-shape section): token s of request r lives in physical page
// block_table[r, s / 64], slot s % 64; the page holds 64 x 128 key bytes and
// then 64 fp32 scales.
#include <algorithm>
#include <type_traits>

#include "dsa_common.h"
#include "dsa_launch.h"
#include "dsa_score.h"

namespace dsa {

__device__ unsigned g_err_logits = 0;

__device__ __forceinline__ void raise_flag(unsigned f) {
  atomicOr(&g_err_logits, f);
}

// ---------------------------------------------------------------------------
// q quantisation: 16 lanes per (t, h) block of 128 bf16 values, 8 per lane.
//   amax = max |q|;  s = amax / 448 (IEEE fp32 division; s = 1 if amax == 0)
//   code = e4m3fn(q / s) (IEEE fp32 division, RNE, saturating)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void quantize_q_blocks(
    const uint16_t* __restrict__ q, int64_t blocks, uint8_t* __restrict__ q8,
    float* __restrict__ q_scale, int64_t wg) {
  const int64_t blk = wg * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (blk >= blocks) return;                 // whole 16-lane groups exit
  const uint4 raw = *reinterpret_cast<const uint4*>(q + blk * 128 + sub * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  float amax = 0.f;
  uint32_t abits = 0u;                       // largest |x| bit pattern
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
  const float s = (amax == 0.f) ? 1.0f : amax / kE4M3Max;
  uint32_t lo = 0, hi = 0;
  if (abits < 0x7f800000u && s >= 0x1p-100f) {
    // all finite, scale not tiny: q / s from the reciprocal with one FMA
    // correction and the hardware e4m3 conversion -- the same code as the
    // IEEE quotient and the integer encoder below for every pair of bf16
    // values |q| <= amax (dsa_fp8_code_check), at a fraction of the
    // instructions
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
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3fn_encode(f[i] / s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3fn_encode(f[4 + i] / s) << (8 * i);
  }
  *reinterpret_cast<uint2*>(q8 + blk * 128 + sub * 8) = make_uint2(lo, hi);
  if (sub == 0) q_scale[blk] = s;
}

__global__ __launch_bounds__(256) void quantize_q_kernel(
    const uint16_t* __restrict__ q, int64_t blocks, uint8_t* __restrict__ q8,
    float* __restrict__ q_scale) {
  quantize_q_blocks(q, blocks, q8, q_scale, blockIdx.x);
}


// ---------------------------------------------------------------------------
// Request of row t: the number of requests r < R with qsl[r] <= t, minus 1
// (query_start_loc is non-decreasing), and 0 for a row before qsl[0] (no
// request holds it: a caller error, kept in bounds as request_of_row
// does).  64 entries per wave-wide load and ballot, so the lookup costs one
// memory round trip for R <= 64.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int request_of_row_wave(const int32_t* qsl, int R,
                                                   int64_t t) {
  const int lane = lane_id();
  int count = 0;
  for (int c = 0; c < R; c += 64) {
    const int i = c + lane;
    const bool le = i < R && (int64_t)qsl[i] <= t;
    const uint64_t m = __ballot(le);
    count += __popcll(m);
    if (m != ~0ull) break;                     // later entries are > t
  }
  return max(count - 1, 0);
}

// ---------------------------------------------------------------------------
// Row-wise logits (decode shape: few query rows per request).  Grid:
// x = query row, y = page group; 4 waves per workgroup, each wave scores
// `ppw` consecutive pages of its row straight from HBM into MFMA registers
// (each K byte is used by exactly one row, so there is nothing to share
// through LDS).  Every load that does not depend on the page list (q
// fragments, weights, the row's position and request) is issued before the
// block-table lookup, and the next page is prefetched while the current one
// is scored.  Lane l stores the logit of token l of the page: one coalesced
// 256-byte store per page.
// ---------------------------------------------------------------------------
template <int MT, bool FULL, bool PREFETCH>
__device__ __forceinline__ void logits_row_body(const LogitsArgs& a, int ppw) {
  const int64_t t = blockIdx.x;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int lane = lane_id();
  const int i16 = lane & 15, g = lane >> 4;
  const int j0 = (blockIdx.y * 4 + wave) * ppw;

  // Everything below is issued before any of it is waited on: the q
  // fragments, the weights, the position, the request lookup and -- on the
  // guess that row t belongs to request t (one query row per request, the
  // decode layout) -- the block-table entries of this wave's pages.
  i32x8 qa[MT];
  load_q_frags<MT, FULL>(a.q8 + t * a.H * kHeadDim, a.H, qa);
  float w[MT][4];
  load_head_weights<MT, FULL>(a.weights + t * a.H, a.q_scale + t * a.H, a.H,
                              w);
  const int p = a.positions[t];
  const int r_guess = (int)min<int64_t>(t, a.R - 1);
  const bool in_row = lane < ppw && (int64_t)(j0 + lane) < a.bt_stride;
  int my_page = in_row ? a.block_table[(int64_t)r_guess * a.bt_stride + j0 + lane]
                       : -1;
  const int r = wave_uniform(request_of_row_wave(a.qsl, a.R, t));

  if (p < 0 || p >= a.ld || (int64_t)(p >> 6) >= a.bt_stride) {
    if (threadIdx.x == 0 && blockIdx.y == 0) raise_flag(kErrPositionOutOfRange);
    return;
  }
  const int npages = (p >> 6) + 1;
  if (j0 >= npages) return;
  const int j1 = min(j0 + ppw, npages);
  if (r != r_guess)                           // rows are not one per request
    my_page = in_row ? a.block_table[(int64_t)r * a.bt_stride + j0 + lane] : -1;
  float* out = a.logits + t * a.ld;

  auto load_page = [&](int page, i32x8 (&kb)[4], float& ks) {
    const uint8_t* pg = a.k_cache + (int64_t)page * kPageBytes;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      kb[nt] = load_frag_global(pg + (16 * nt + i16) * kHeadDim + 32 * g);
    ks = reinterpret_cast<const float*>(pg + kPageKeyBytes)[lane];
  };
  auto page_at = [&](int jp) {
    return __builtin_amdgcn_readlane(my_page, jp - j0);
  };
  auto valid = [&](int page) {
    return page >= 0 && (int64_t)page < a.num_pages;
  };

  i32x8 kb[4];
  float ks = 0.f;
  int cur = page_at(j0);
  if (valid(cur)) load_page(cur, kb, ks);
  for (int jp = j0; jp < j1; ++jp) {
    i32x8 nb[4];
    float nks = 0.f;
    int nxt = -1;
    if (PREFETCH && jp + 1 < j1) {
      nxt = page_at(jp + 1);
      if (valid(nxt)) load_page(nxt, nb, nks);
    }
    const int s = jp * kPageTokens + lane;
    if (!valid(cur)) {
      if (lane == 0) raise_flag(kErrPageOutOfRange);
      out[s] = -INFINITY;
    } else {
      float v[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[m] = mfma16x16x128_fp8(qa[m], kb[nt], f32x4{0.f, 0.f, 0.f, 0.f});
        v[nt] = head_reduce<MT>(acc, w);
      }
      const float tot = reduce_scatter4(v[0], v[1], v[2], v[3]);
      out[s] = (s <= p) ? tot * ks : -INFINITY;
    }
    if (jp + 1 < j1) {
      if (PREFETCH) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) kb[nt] = nb[nt];
        ks = nks;
        cur = nxt;
      } else {
        cur = page_at(jp + 1);
        if (valid(cur)) load_page(cur, kb, ks);
      }
    }
  }
}

// One page per wave: at most 128 VGPRs so four waves share each SIMD.
template <int MT, bool FULL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void logits_row_kernel(LogitsArgs a, int ppw) {
  logits_row_body<MT, FULL, false>(a, ppw);
}

// Several pages per wave with the next page prefetched.
template <int MT, bool FULL>
__global__ __launch_bounds__(256)
void logits_row_prefetch_kernel(LogitsArgs a, int ppw) {
  logits_row_body<MT, FULL, true>(a, ppw);
}

// ---------------------------------------------------------------------------
// Balanced row-wise logits for small decode batches (T <= 128 rows).  With
// few rows of very different lengths, a grid of (row, page group) leaves
// some compute units with several long groups and others idle, and a
// compute unit's share of the bytes sets the kernel time.  Here the visible
// pages of the whole batch are dealt out evenly: every wave (one per
// workgroup) reads the positions of all rows with scalar loads, computes
// P = the number of visible pages, a per-wave budget
// ppw = max(D, ceil(P / waves in the grid)), gives row t ceil(n_t / ppw)
// waves, and takes its own contiguous page range of one row from a prefix
// sum over the rows.  Page ids and the request check are scalar loads too,
// so the K loads are issued after two scalar round trips and never queue
// behind vector loads.  K pages are read with buffer loads whose size is
// zero for pages outside the range (no traffic, no branch), which keeps the
// hardware wait counts exact: page q is scored as soon as its bytes arrive
// while later pages are still in flight.
// ---------------------------------------------------------------------------
constexpr int kBalancedMaxRows = 128;

// Positions of rows c0 .. c0+63 in lanes 0..63 (rows >= T repeat row T-1).
__device__ __forceinline__ int positions_to_lanes(const int32_t* pos, int c0,
                                                  int64_t T) {
  int x[64];
  if ((int64_t)c0 + 64 <= T) {
    typedef int i32x16 __attribute__((ext_vector_type(16)));
    typedef __attribute__((address_space(4))) const i32x16 const_i32x16;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const i32x16 v = ((const_i32x16*)(pos + c0))[k];
#pragma unroll
      for (int j = 0; j < 16; ++j) x[16 * k + j] = v[j];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i)
      x[i] = load_uniform(pos, min<int64_t>(c0 + i, T - 1));
  }
  int v = 0;
#pragma unroll
  for (int i = 0; i < 64; ++i)
    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(x[i]), "i"(i));
  return v;
}

struct RowSpan {
  int row, jb, je, p;
};

// The page range [jb, je) of row `row` owned by wave li of XCD x; row = -1
// when the wave has no work.  Workgroups are dealt to the 8 XCDs
// round-robin, so wave (one workgroup) w runs on XCD w % 8: the flattened
// page list (rows in order) is cut into 8 contiguous parts, part x goes to
// the waves of XCD x, and a row's q is then fetched into one or two of the
// XCD L2 caches instead of all eight.  Within a part every row fragment of f
// pages gets ceil(f / ppw) waves, ppw = max(D, ceil(ceil(P / 8) /
// per_xcd)), so a part needs at most per_xcd + T waves: the grid is 8
// (per_xcd + T) waves.  Rows whose position is out of range own no pages
// (the row is left untouched and wave 0 raises the flag).
template <int NCH>
__device__ __forceinline__ RowSpan balanced_span(const LogitsArgs& a, int D,
                                                 int per_xcd, int wv,
                                                 int head_pages) {
  const int lane = lane_id();
  int pl[NCH], n[NCH];
  uint32_t incl[NCH];                         // page prefix over the batch
  uint32_t total = 0u;
  bool bad = false;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    pl[c] = positions_to_lanes(a.positions, 64 * c, a.T);
    const bool in = 64 * c + lane < a.T;
    const bool ok = pl[c] >= 0 && pl[c] < a.ld &&
                    (int64_t)(pl[c] >> 6) < a.bt_stride;
    bad |= in && !ok;
    n[c] = (in && ok) ? max(0, (pl[c] >> 6) + 1 - head_pages) : 0;
    incl[c] = total + wave_inclusive_scan((uint32_t)n[c]);
    total = __builtin_amdgcn_readlane(incl[c], 63);
  }
  if (wv == 0 && __ballot(bad) != 0ull && lane == 0)
    raise_flag(kErrPositionOutOfRange);
  const uint32_t x = (uint32_t)wv & 7u, li = (uint32_t)wv >> 3;
  const uint32_t lo_x = (uint32_t)((uint64_t)total * x / 8u);
  const uint32_t hi_x = (uint32_t)((uint64_t)total * (x + 1u) / 8u);
  const uint32_t part = (total + 7u) / 8u;
  const int ppw =
      max(D, (int)((part + (uint32_t)per_xcd - 1) / (uint32_t)per_xcd));
  RowSpan sp{-1, 0, 0, 0};
  uint32_t base = 0u;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    // this row's fragment in part x: pages [lo, hi) of the flattened list
    const uint32_t ex_pages = incl[c] - (uint32_t)n[c];
    const uint32_t lo = max(ex_pages, lo_x), hi = min(incl[c], hi_x);
    const uint32_t f = hi > lo ? hi - lo : 0u;
    const uint32_t cnt = (f + ppw - 1) / (uint32_t)ppw;
    const uint32_t wincl = wave_inclusive_scan(cnt);
    const uint64_t m = __ballot(li < base + wincl);
    if (sp.row < 0 && m != 0ull) {
      const int l = __builtin_ctzll(m);
      const int ex = (int)(base + __builtin_amdgcn_readlane(wincl - cnt, l));
      const int cl = __builtin_amdgcn_readlane((int)cnt, l);
      const int fl = __builtin_amdgcn_readlane((int)f, l);
      const int first = __builtin_amdgcn_readlane((int)(lo - ex_pages), l);
      // fl = cl * qd + rm: the first rm waves of the fragment take qd + 1
      const int i = (int)li - ex, qd = fl / cl, rm = fl - qd * cl;
      sp.row = 64 * c + l;
      sp.jb = first + i * qd + min(i, rm);
      sp.je = sp.jb + qd + (i < rm ? 1 : 0);
      sp.p = __builtin_amdgcn_readlane(pl[c], l);
    }
    base += __builtin_amdgcn_readlane(wincl, 63);
  }
  sp.row = wave_uniform(sp.row);
  sp.jb = wave_uniform(sp.jb) + head_pages;
  sp.je = wave_uniform(sp.je) + head_pages;
  sp.p = wave_uniform(sp.p);
  return sp;
}

// ---------------------------------------------------------------------------
// Decode page schedule, built once per batch.  The balanced waves' spans
// depend only on the positions, query_start_loc and block table, which a
// forward pass shares with every F layer of an IndexCache run, so they are
// computed ahead of the logits launch -- by extra workgroups of the
// q-quantisation launch, whose own work is latency-bound -- and a logits
// wave then issues its K loads after one scalar load of its entry instead of
// a chain of three metadata round trips (positions, spans, block table).
// Entry of logits wave w, kSchedInts int32: row (-1: no work), position,
// first page, end page, request, physical pages of its first kSchedPages
// pages (-1 past the range).  The spans are balanced_span's without head
// waves, so each (row, page) is scored by the same code as without the
// schedule: the logits are bit-identical.
// ---------------------------------------------------------------------------
constexpr int kSchedInts = 8;
constexpr int kSchedPages = 3;

template <int NCH>
__global__ __launch_bounds__(256) void quantize_q_sched_kernel(
    const uint16_t* __restrict__ q, int64_t blocks, uint8_t* __restrict__ q8,
    float* __restrict__ q_scale, int qgrid, LogitsArgs a, int D, int per_xcd,
    int nwaves, int32_t* __restrict__ sched) {
  if ((int)blockIdx.x < qgrid) {
    quantize_q_blocks(q, blocks, q8, q_scale, blockIdx.x);
    return;
  }
  const int w = ((int)blockIdx.x - qgrid) * 4 + (int)(threadIdx.x >> 6);
  if (w >= nwaves) return;
  const int lane = lane_id();
  // query_start_loc of the first 64 requests, loaded while the span is
  // computed from the positions: the request of a row among them then
  // needs no further round trip before the block-table load
  const int q_first = lane < a.R ? a.qsl[lane] : 0;
  const RowSpan sp = balanced_span<NCH>(a, D, per_xcd, w, 0);
  int v = -1;
  if (sp.row >= 0) {
    const uint64_t le = __ballot(lane < a.R && q_first <= sp.row);
    const int r = wave_uniform(le != ~0ull
                                   ? max(__popcll(le) - 1, 0)
                                   : request_of_row_wave(a.qsl, a.R, sp.row));
    const int last = (int)a.bt_stride - 1;
    const int j = sp.jb + (lane - 5);
    const int page = a.block_table[(int64_t)r * a.bt_stride +
                                   min(max(j, 0), last)];
    v = lane == 0 ? sp.row : lane == 1 ? sp.p : lane == 2 ? sp.jb
        : lane == 3 ? sp.je : lane == 4 ? r : (j < sp.je ? page : -1);
  }
  if (lane < kSchedInts) sched[(int64_t)w * kSchedInts + lane] = v;
}

// head_waves > 0: the first head_waves workgroups are head waves: wave
// (t, i) = (b / HW, b % HW) takes pages [i D, i D + D) of row t, known
// without the positions, so its block-table, q and position loads go out
// together and its K loads one round trip before the balanced waves'
// (which first need every row's position); the balanced waves share the
// pages from HW D on.  head_waves is a multiple of 8 (XCD parity).
//
// SCHED: the spans come from the page schedule (no head waves): wave b
// reads entry b -- row, position, range, request and its first pages -- in
// one scalar load and issues its K loads right after it.
template <int MT, bool FULL, int D, int NCH, bool SCHED>
__global__ __launch_bounds__(64) void logits_balanced_kernel(
    LogitsArgs a, int per_xcd, int hw, int head_waves,
    const int32_t* __restrict__ sched) {
  static_assert(!SCHED || D <= kSchedPages, "schedule holds 3 pages");
  const int lane = lane_id();
  const bool head = !SCHED && (int)blockIdx.x < head_waves;
  RowSpan sp;
  int sched_r = 0;
  int sched_pages[kSchedPages];
  if (SCHED) {
    typedef __attribute__((address_space(4))) const i32x8 const_i32x8;
    const i32x8 e = ((const_i32x8*)(sched))[blockIdx.x];
    sp = RowSpan{e[0], e[2], e[3], e[1]};
    // an entry the builder did not write for this batch (a knob changed
    // in between) must still keep every access in bounds
    if (sp.row < 0 || sp.row >= a.T || sp.p < 0 || sp.p >= a.ld ||
        (int64_t)(sp.p >> 6) >= a.bt_stride || sp.jb < 0)
      return;
    sp.je = min(sp.je, (sp.p >> 6) + 1);
    if (sp.jb >= sp.je) return;
    sched_r = min(max(e[4], 0), a.R - 1);
    sched_pages[0] = e[5];
    sched_pages[1] = e[6];
    sched_pages[2] = e[7];
  } else if (head) {
    const int hb = (int)blockIdx.x;
    sp = RowSpan{hb / hw, (hb % hw) * D, (hb % hw) * D + D, 0};
    if (sp.row >= a.T) return;
  } else {
    sp = balanced_span<NCH>(a, D, per_xcd, (int)blockIdx.x - head_waves,
                            hw * D);
    if (sp.row < 0) return;
  }
  const int64_t t = sp.row;
  int p = sp.p, je = sp.je;
  const int jb = sp.jb;
  if (head) p = load_uniform(a.positions, t);

  // request guess r = t (one query row per request), checked below; the
  // page ids of the first chunk are fetched with it (the schedule has both)
  int r = SCHED ? sched_r : (int)min<int64_t>(t, a.R - 1);
  const int q0 = SCHED ? 0 : load_uniform(a.qsl, r);
  const int q1 = SCHED ? 1 : load_uniform(a.qsl, r + 1);
  const int32_t* btr = a.block_table + (int64_t)r * a.bt_stride;
  const int last = (int)a.bt_stride - 1;
  int pages[D];
#pragma unroll
  for (int q = 0; q < D; ++q)
    pages[q] = SCHED ? sched_pages[q] : load_uniform(btr, min(jb + q, last));
  i32x8 qa[MT];
  load_q_frags<MT, FULL>(a.q8 + t * a.H * kHeadDim, a.H, qa);
  float w[MT][4];
  load_head_weights<MT, FULL>(a.weights + t * a.H, a.q_scale + t * a.H, a.H,
                              w);
  if (head) {
    // the position arrived with the other loads: clip the range, or leave
    // (a bad position is flagged by the balanced wave that reads them all)
    if (p < 0 || p >= a.ld || (int64_t)(p >> 6) >= a.bt_stride) return;
    je = min(je, (p >> 6) + 1);
    if (jb >= je) return;
  }
  if (!SCHED && !(q0 <= t && t < q1)) {      // rows are not one per request
    r = wave_uniform(request_of_row_wave(a.qsl, a.R, t));
    btr = a.block_table + (int64_t)r * a.bt_stride;
#pragma unroll
    for (int q = 0; q < D; ++q) pages[q] = load_uniform(btr, min(jb + q, last));
  }
  float* out = a.logits + t * a.ld;
  bool bad_page = false;
  for (int c = jb; c < je; c += D) {
    if (c != jb) {
#pragma unroll
      for (int q = 0; q < D; ++q) pages[q] = load_uniform(btr, min(c + q, last));
    }
    i32x8 kb[D][4];
    float ks[D];
    bool ok[D];
#pragma unroll
    for (int q = 0; q < D; ++q) {
      ok[q] = c + q < je && pages[q] >= 0 && (int64_t)pages[q] < a.num_pages;
      bad_page |= c + q < je && !ok[q];
      load_k_page_regs(
          make_rsrc(a.k_cache + (int64_t)(ok[q] ? pages[q] : 0) * kPageBytes,
                    ok[q] ? kPageBytes : 0),
          kb[q], ks[q]);
    }
    // keep every load of the chunk ahead of the first MFMA
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < D; ++q) {
      const int jp = c + q;
      float res = -INFINITY;
      if (ok[q]) {
        const float tot = decode_page_sum<MT>(qa, kb[q], w);
        if (jp * kPageTokens + lane <= p) res = tot * ks[q];
      }
      // device-scope (sc1) store: written through this XCD's L2, so the
      // end of the launch has no dirty logits lines left to write back
      // before the top-k launch reads them from another XCD (measured
      // 0.15-0.2 us faster per decode forward; non-temporal stores were
      // 0.25 us slower)
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(
          out + (int64_t)min(jp, last) * kPageTokens,
          jp < je ? kPageTokens * 4 : 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res), ro, 4 * lane,
                                            0, 16);
    }
  }
  if (bad_page && lane == 0) raise_flag(kErrPageOutOfRange);
}

// ---------------------------------------------------------------------------
// Tiled logits (several query rows of one request share every K page: the
// prefill chunk and the long-context tail).  A workgroup of 8 waves owns a
// tile of 16 consecutive rows of one request and a range of pages; each
// page (8192 key bytes + 256 scale bytes) is read from HBM once per tile with
// fully coalesced 16-byte loads, staged in LDS (double-buffered, rows padded
// to 144 bytes so the MFMA-layout reads are bank-conflict free) and used by
// all 8 waves; wave w scores rows 2w and 2w+1.  Grid: x = page split,
// y = tile (tiles of request r are numbered after those of requests < r).
// ---------------------------------------------------------------------------
constexpr int kTileWaves = 8;
constexpr int kLdsRow = 144;

// Tile y -> (request, first row, rows).  One wave scans query_start_loc.
__device__ void find_tile(const int32_t* qsl, int R, int y, int* s_info) {
  const int lane = lane_id();
  int base = 0;
  for (int c = 0; c < R; c += 64) {
    const int r = c + lane;
    int n = 0;
    if (r < R) n = (qsl[r + 1] - qsl[r] + kTileRows - 1) / kTileRows;
    if (n < 0) n = 0;
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int excl = incl - n;
    if (r < R && y >= base + excl && y < base + incl) {
      s_info[0] = r;
      s_info[1] = qsl[r] + (y - base - excl) * kTileRows;
      s_info[2] = min(kTileRows, qsl[r + 1] - s_info[1]);
    }
    base += __shfl(incl, 63);
  }
}

template <int MT, bool FULL>
__global__ __launch_bounds__(512) void logits_tile_kernel(LogitsArgs a,
                                                          int pages_per_split) {
  __shared__ __align__(16) uint8_t s_keys[2][kPageTokens * kLdsRow];
  __shared__ __align__(16) float s_scale[2][kPageTokens];
  __shared__ int s_ok[2];
  __shared__ int s_info[4];
  __shared__ int s_pos[kTileRows];

  const int tid = threadIdx.x;
  const int wave = wave_uniform(tid >> 6);
  const int lane = lane_id();
  if (tid == 0) { s_info[0] = -1; s_info[1] = 0; s_info[2] = 0; }
  __syncthreads();
  if (wave == 0) find_tile(a.qsl, a.R, blockIdx.y, s_info);
  __syncthreads();
  const int r = s_info[0];
  if (r < 0) return;                         // grid bound beyond last tile
  const int64_t row0 = s_info[1];
  const int nrows = s_info[2];
  if (tid < kTileRows) {
    int p = -1;
    if (tid < nrows && row0 + tid >= 0 && row0 + tid < a.T) {
      p = a.positions[row0 + tid];
      if (p < 0 || p >= a.ld || (int64_t)(p >> 6) >= a.bt_stride) {
        raise_flag(kErrPositionOutOfRange);
        p = -1;
      }
    }
    s_pos[tid] = p;
  }
  __syncthreads();
  int maxp = -1;
#pragma unroll
  for (int i = 0; i < kTileRows; ++i) maxp = max(maxp, s_pos[i]);
  const int npages = (maxp >> 6) + 1;        // 0 when no valid row
  const int jb = blockIdx.x * pages_per_split;
  const int je = min(jb + pages_per_split, npages);
  if (jb >= je) return;

  const int32_t* bt = a.block_table + (int64_t)r * a.bt_stride;
  const int i16 = lane & 15, g = lane >> 4;

  // This wave's two rows.
  int prow[2];
  i32x8 qa[2][MT];
  float w[2][MT][4];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int lr = 2 * wave + rr;
    prow[rr] = s_pos[lr];
    if (prow[rr] >= 0) {
      const int64_t t = row0 + lr;
      load_q_frags<MT, FULL>(a.q8 + t * a.H * kHeadDim, a.H, qa[rr]);
      load_head_weights<MT, FULL>(a.weights + t * a.H, a.q_scale + t * a.H,
                                  a.H, w[rr]);
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        qa[rr][m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) w[rr][m][j] = 0.f;
      }
    }
  }

  // Cooperative page copy: thread i moves key bytes [16 i, 16 i + 16)
  // (token i / 8, chunk i % 8); threads 0..15 also move the 256 scale bytes.
  const int ctok = tid >> 3, cchunk = tid & 7;
  auto fetch = [&](int jp, uint4& kreg, uint4& sreg, bool& ok) {
    const int page = bt[jp];
    ok = page >= 0 && (int64_t)page < a.num_pages;
    if (!ok) {
      kreg = make_uint4(0, 0, 0, 0);
      sreg = make_uint4(0, 0, 0, 0);
      return;
    }
    const uint8_t* pg = a.k_cache + (int64_t)page * kPageBytes;
    kreg = *reinterpret_cast<const uint4*>(pg + tid * 16);
    if (tid < 16) sreg = *reinterpret_cast<const uint4*>(pg + kPageKeyBytes + tid * 16);
  };
  auto stash = [&](int buf, const uint4& kreg, const uint4& sreg, bool ok) {
    *reinterpret_cast<uint4*>(&s_keys[buf][ctok * kLdsRow + cchunk * 16]) = kreg;
    if (tid < 16) *reinterpret_cast<uint4*>(&s_scale[buf][tid * 4]) = sreg;
    if (tid == 0) s_ok[buf] = ok;
  };

  uint4 kreg, sreg = make_uint4(0, 0, 0, 0);
  bool ok;
  fetch(jb, kreg, sreg, ok);
  if (!ok && tid == 0) raise_flag(kErrPageOutOfRange);
  stash(0, kreg, sreg, ok);

  for (int jp = jb; jp < je; ++jp) {
    const int buf = (jp - jb) & 1;
    const bool more = jp + 1 < je;
    if (more) {
      fetch(jp + 1, kreg, sreg, ok);
      if (!ok && tid == 0) raise_flag(kErrPageOutOfRange);
    }
    __syncthreads();
    const uint8_t* kb_lds = s_keys[buf];
    const bool page_ok = s_ok[buf] != 0;
#pragma unroll
    for (int ntp = 0; ntp < 2; ++ntp) {
      i32x8 kb[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint8_t* src = kb_lds + (16 * (2 * ntp + q) + i16) * kLdsRow + 32 * g;
        const uint4 x = *reinterpret_cast<const uint4*>(src);
        const uint4 y = *reinterpret_cast<const uint4*>(src + 16);
        kb[q] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                      (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      }
      float v[2][2];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          f32x4 acc[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[m] = mfma16x16x128_fp8(qa[rr][m], kb[q], f32x4{0.f, 0.f, 0.f, 0.f});
          v[rr][q] = head_reduce<MT>(acc, w[rr]);
        }
      // lane group g ends with (row g >> 1, N-tile 2*ntp + (g & 1))
      const float tot = reduce_scatter4(v[0][0], v[0][1], v[1][0], v[1][1]);
      const int rr = g >> 1;
      const int tok = 16 * (2 * ntp + (g & 1)) + i16;
      const int pr = rr ? prow[1] : prow[0];
      if (pr >= 0 && jp <= (pr >> 6)) {        // the row's own pages only
        const int s = jp * kPageTokens + tok;
        const float val = (s <= pr && page_ok) ? tot * s_scale[buf][tok]
                                               : -INFINITY;
        a.logits[(row0 + 2 * wave + rr) * a.ld + s] = val;
      }
    }
    if (more) stash(buf ^ 1, kreg, sreg, ok);
  }
}


// ---------------------------------------------------------------------------
// Tiled logits, one row per wave.  A workgroup of 16 waves owns a tile of 16
// consecutive rows of one request and a range of pages; wave w scores row
// w.  With one row per wave a wave holds 16 heads x 128 q codes (32 VGPRs)
// instead of two rows, so it fits in 128 VGPRs and four waves share each
// SIMD: the MFMAs of one wave overlap the VALU work of the others.
//
// A tile's pages are cut into gridDim.x equal ranges (at least 64 pages),
// so all splits of a tile take the same time and the last wave of
// workgroups does not leave compute units idle.  Pages are staged in LDS PP
// at a time (double-buffered, one barrier per step) by direct-to-LDS buffer
// loads: no staging registers, no LDS store instructions.  A page's keys sit in LDS chunk-major: 16-byte chunk
// (N-tile n, half r, chunk g, token t) at n * 2048 + r * 1024 + g * 256 +
// t * 16, holding bytes [64 r + 16 g, + 16) of token 16 n + t.  The B
// operand of N-tile n is then two fully contiguous 1 KB reads (lane l at
// n * 2048 + r * 1024 + 16 l), which the LDS serves at full rate; the
// padded token-row layout costs ~1.7x that in bank conflicts.  q uses the
// same permutation of the reduction index (load_q_frags_cm).  A page
// outside the pool is a zero-size buffer: its loads touch no memory and its
// logits are -inf.  Each page: 4 N-tiles x MT MFMAs, the head reduction in
// registers, one reduce-scatter across the 4 lane groups, one 256-byte
// logit store.
//
// LIN: the epilogue is w * |dot| (one FMA per output) and the linear part L
// comes from the shared MFMA described above: wave 4 G + i computes it for
// N-tile i of every page for rows 4 G .. 4 G + 3 and leaves it in LDS; the
// logits of a page pair are completed and stored in the next pass of the
// loop, after the barrier that publishes L.
// ---------------------------------------------------------------------------
constexpr int kT16Waves = 16;
constexpr int kT16Threads = 64 * kT16Waves;

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Direct-to-LDS buffer loads (lane l's SIZE bytes from base + voff land at
// LDS address lds + SIZE * l) through the compiler's builtin, which sets m0
// itself.  (An earlier inline-assembly version wrote m0 behind the
// compiler's back; the builtin measured as fast, logits bit-identical.)  The
// caller makes the data visible itself (vmcnt(0), then a barrier).  base,
// bytes and lds are wave-uniform; reads at or past `bytes` return 0.
template <int SIZE>
__device__ __forceinline__ void lds_copy(const void* base, int bytes,
                                         const void* lds, int voff) {
  static_assert(SIZE == 4 || SIZE == 16, "copy size");
  typedef __attribute__((address_space(3))) void lds_void;
  lds_void* dst = (lds_void*)(const lds_u8*)lds;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, bytes);
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, 0, 0, 0);
}

//
// a.page_stride > 1 (the fused forward's sample pass, LIN only): the tile's
// pages are the logical pages j = 0, 1, .. of real page j * page_stride; a
// row sees logical page j when j * page_stride <= p / 64, its logits go to
// columns 64 j .. of row t at a.logits + t * a.out_ld.
// CAND (LIN only): no logits are written; every visible logit of row t at
// or above ft.tlo[t] (as an ordered key) is appended as (key, column) to
// this workgroup's slot of the row in ascending column order, and the
// count to ft.count (FusedTile).
template <int MT, bool FULL, bool LIN, int PP, bool PF, bool CAND>
__global__ __launch_bounds__(kT16Threads) void logits_tile16_kernel(
    LogitsArgs a, int pages_per_split, int min_pages, FusedTile ft) {
  static_assert(PP == 2 || PP == 4, "pages per step");
  static_assert(LIN || !CAND, "candidate mode has the linear-term epilogue");
  constexpr int kLs = PP * kPageTokens + 16;     // s_lin row stride (banks)
  // two key buffers [page of the step][8192 key bytes, chunk-major], as two
  // objects so the compiler can tell the reads of one from the direct-to-LDS
  // copy into the other (it would otherwise wait for the copy before every
  // read); the scales have a third buffer: a step's scales are still read
  // after the barrier that lets the next-but-one step's copy start
  __shared__ __align__(16) uint8_t s_keys0[PP][kPageKeyBytes];
  __shared__ __align__(16) uint8_t s_keys1[PP][kPageKeyBytes];
  __shared__ __align__(16) float s_scale[3][PP][kPageTokens];
  __shared__ __align__(16) uint8_t s_alin[LIN ? kTileRows / 4 : 1][2048];
  __shared__ __align__(16) float s_ascale[LIN ? kTileRows : 1][kLinPieces];
  __shared__ __align__(16) float s_lin[2][LIN ? kTileRows : 1][kLs];
  __shared__ int s_info[4];
  __shared__ int s_pos[kTileRows];

  const int tid = threadIdx.x;
  const int wave = wave_uniform(tid >> 6);
  const int lane = lane_id();
  if (tid == 0) { s_info[0] = -1; s_info[1] = 0; s_info[2] = 0; }
  __syncthreads();
  if (wave == 0) find_tile(a.qsl, a.R, blockIdx.y, s_info);
  __syncthreads();
  const int r = s_info[0];
  if (r < 0) return;                         // grid bound beyond last tile
  const int64_t row0 = s_info[1];
  const int nrows = s_info[2];
  if (tid < kTileRows) {
    int p = -1;
    if (tid < nrows && row0 + tid >= 0 && row0 + tid < a.T) {
      p = a.positions[row0 + tid];
      if (p < 0 || p >= a.ld || (int64_t)(p >> 6) >= a.bt_stride) {
        raise_flag(kErrPositionOutOfRange);
        p = -1;
      }
    }
    s_pos[tid] = p;
  }
  __syncthreads();
  const int SSt = LIN ? a.page_stride : 1;
  int maxp = -1;
#pragma unroll
  for (int i = 0; i < kTileRows; ++i) maxp = max(maxp, s_pos[i]);
  // (logical) pages of the tile; 0 when no valid row
  const int npages = maxp < 0 ? 0 : (maxp >> 6) / SSt + 1;
  // pages_per_split > 0: fixed ranges; otherwise this tile's pages are cut
  // into gridDim.x equal ranges of at least min_pages (the splits of a
  // tile then take the same time whatever its length)
  const int per = pages_per_split > 0
                      ? pages_per_split
                      : max(min_pages, (npages + (int)gridDim.x - 1) / (int)gridDim.x);
  const int jb = blockIdx.x * per;
  const int je = min(jb + per, npages);
  if (jb >= je) {
    // a split past the tile's pages: its rows found no candidates here
    if (CAND && tid < kTileRows && s_pos[tid] >= 0)
      ft.count[(row0 + tid) * gridDim.x + blockIdx.x] = 0u;
    return;
  }

  const int32_t* bt = a.block_table + (int64_t)r * a.bt_stride;
  const int i16 = lane & 15, g = lane >> 4;
  const int prow = wave_uniform(s_pos[wave]);
  const int64_t t = row0 + wave;

  // Page copy of a step, issued right after the barrier that frees the
  // buffer: wave w moves LDS chunks 64 (w & 7) .. + 63 of pages (w >> 3) +
  // 2 k of the step (lane l -> chunk q = 64 (w & 7) + l: N-tile q >> 7,
  // half (q >> 6) & 1, chunk (q >> 4) & 3, token q & 15); waves 0 and 8
  // also move those pages' 64 scales.
  const int half = wave_uniform(wave >> 3);
  const int cq = 64 * (wave & 7) + lane;
  const int csrc = (16 * (cq >> 7) + (cq & 15)) * kHeadDim +
                   64 * ((cq >> 6) & 1) + 16 * ((cq >> 4) & 3);
  bool bad_page = false;
  const int last = (int)a.bt_stride - 1;
  auto page_id = [&](int jp) {
    const int page = load_uniform(bt, min(jp * SSt, last));
    return jp < je ? page : -1;
  };
  auto fetch = [&](int jp, auto buf_, int sbuf) {
    constexpr int B = decltype(buf_)::value;
    auto& keys = *(B ? &s_keys1 : &s_keys0);
#pragma unroll
    for (int k = 0; k < PP / 2; ++k) {
      const int ph = half + 2 * k;
      const int page = page_id(jp + ph);
      const bool ok = page >= 0 && (int64_t)page < a.num_pages;
      bad_page |= jp + ph < je && !ok;
      const uint8_t* pg = a.k_cache + (int64_t)(ok ? page : 0) * kPageBytes;
      const int bytes = ok ? kPageBytes : 0;
      lds_copy<16>(pg, bytes, &keys[ph][64 * 16 * (wave & 7)], csrc);
      if ((wave & 7) == 0)
        lds_copy<4>(pg, bytes, &s_scale[sbuf][ph][0], kPageKeyBytes + 4 * lane);
    }
  };

  i32x8 qa[MT];
  if (prow >= 0) {
    load_q_frags_cm<MT, FULL>(a.q8 + t * a.H * kHeadDim, a.H, qa);
  } else {
#pragma unroll
    for (int m = 0; m < MT; ++m) qa[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  fetch(jb, std::integral_constant<int, 0>(), 0);

  // Shared linear part: this wave's qlin pieces to LDS, then the A operand
  // of its group (rows 4 G .. 4 G + 3, G = wave / 4).  The piece scales of
  // the row a lane group receives are read from LDS where they are used.
  const int G = wave >> 2;
  auto load_alin = [&]() {
    const uint8_t* src = &s_alin[G][16 * lane];
    const uint4 x = *reinterpret_cast<const uint4*>(src);
    const uint4 y = *reinterpret_cast<const uint4*>(src + 1024);
    return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                 (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  };
  i32x8 alin = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  if (LIN) {
    float wa[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) wa[m] = 0.f;
    if (prow >= 0)
      load_a_weights<MT, FULL>(a.weights + t * a.H, a.q_scale + t * a.H, a.H,
                               wa);
    const float2 ql = row_qlin<MT>(qa, wa);
    split_pieces(ql.x, ql.y, wave & 3, &s_alin[G][0], &s_ascale[wave][0]);
    __syncthreads();
    alin = load_alin();
  }
  float w[MT][4];
  if (prow >= 0) {
    load_head_weights<MT, FULL>(a.weights + t * a.H, a.q_scale + t * a.H,
                                a.H, w);
  } else {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) w[m][j] = 0.f;
  }
  float* orow = a.logits + t * (a.out_ld > 0 ? a.out_ld : a.ld);
  // candidate mode: this row's threshold and slot, the running count
  const uint32_t cthr =
      (CAND && prow >= 0) ? load_uniform(reinterpret_cast<const int32_t*>(
                                             ft.tlo), t)
                          : 0u;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(
      CAND ? ft.cand + (t * gridDim.x + blockIdx.x) * (int64_t)ft.cap
           : nullptr,
      CAND && prow >= 0 ? ft.cap * 8 : 0);
  uint32_t cbase = 0u;

  // LIN: wave 4 G + wq takes the N-tiles of a page in the order wq, wq + 1,
  // ... (mod 4), so the tile it computes L for is always its first one and
  // the loop carries no wave-dependent branch; lane group g then ends with
  // N-tile (wq + g) mod 4.  The head sums of a step wait in registers for L
  // until after the next barrier, and take their k-scales then.
  const int wq = LIN ? (wave & 3) : 0;
  const int tok = 16 * ((wq + g) & 3) + i16;
  float pt[PP];
  bool pok[PP];
#pragma unroll
  for (int h = 0; h < PP; ++h) { pt[h] = 0.f; pok[h] = false; }
  int pjp = -1, pbuf = 0, psbuf = 0;
  auto complete = [&]() {
#pragma unroll
    for (int h = 0; h < PP; ++h) {
      const int pj = pjp + h;
      const int s = pj * SSt * kPageTokens + tok;      // real column
      const float lv = s_lin[pbuf][wave][kPageTokens * h + tok];
      const float ks = s_scale[psbuf][h][tok];
      const float val = (s <= prow && pok[h]) ? (pt[h] + lv) * ks : -INFINITY;
      if (CAND) {
        // lane group g holds token group (wq + g) & 3: rotating the lane
        // mask by 16 wq bits gives the mask in token order, so a lane's
        // slot is the number of selected tokens before its own
        const bool vis = prow >= 0 && pj < je && s <= prow;
        const uint32_t key = float_to_ordered(val);
        const bool sel = vis && key >= (uint32_t)cthr;
        const uint64_t lm = __ballot(sel);
        if (lm) {
          const uint64_t tm = __builtin_rotateleft64(lm, 16 * wq);
          const uint32_t rank =
              (uint32_t)__popcll(tm & ((1ull << tok) - 1ull));
          const uint32_t slot = cbase + rank;
          // slots past cap fall outside the buffer and are dropped
          const int off = sel && slot < (uint32_t)ft.cap ? (int)slot * 8
                                                          : ft.cap * 8;
          typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{key, (uint32_t)s}, crs,
                                                off, 0, 0);
          cbase += (uint32_t)__popcll(lm);
        }
        continue;
      }
      // the page's 64 logits as a buffer, empty for a padding row, a page
      // past the range or past the row's own last page (a shorter row of
      // the tile): an unconditional store, no 64-bit address math;
      // non-temporal (nt), so the logits stream does not fill the caches
      // with lines the kernel never reads (measured 1-2 % faster on the
      // prefill chunk and the 1M-token tail)
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(
          orow + (int64_t)min(pj, npages - 1) * kPageTokens,
          prow >= 0 && pj < je && pj * SSt <= (prow >> 6) ? kPageTokens * 4
                                                           : 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ro, 4 * tok,
                                            0, 2);
    }
  };

  // B operand of N-tile (wq + nt) mod 4 of page h of a step: two contiguous
  // 1 KB reads (chunk-major layout)
  auto load_kb = [&](auto& keys, int h, int nt) {
    const int n = (wq + nt) & 3;
    const uint8_t* src = &keys[h][0] + 2048 * n + 16 * lane;
    const uint4 x = *reinterpret_cast<const uint4*>(src);
    const uint4 y = *reinterpret_cast<const uint4*>(src + 1024);
    return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                 (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  };
  // One step: the pages [jp, jp + PP) from key buffer B, the next step's
  // copy into the other one.  The loop below alternates B = 0, 1 so that
  // each buffer is a fixed object in each half.
  auto step = [&](int jp, int si, auto buf_) {
    constexpr int buf = decltype(buf_)::value;
    auto& keys = *(buf ? &s_keys1 : &s_keys0);
    const int sbuf = si % 3;
    const bool more = jp + PP < je;
    // this wave's copy of the step has landed in LDS (the direct loads
    // count in vmcnt); the barrier then publishes every wave's copy
    __builtin_amdgcn_s_waitcnt(0x0f70);        // vmcnt(0)
    __syncthreads();
    if (LIN && jp != jb) complete();
    if (more)
      fetch(jp + PP, std::integral_constant<int, buf ^ 1>(),
            sbuf == 2 ? 0 : sbuf + 1);
    i32x8 kb_next;
    if (PF) kb_next = load_kb(keys, 0, 0);
#pragma unroll
    for (int h = 0; h < PP; ++h) {
      const int pj = jp + h;
      float v[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        // B operand of this N-tile; with PF the next N-tile's is read from
        // LDS before this one's MFMAs are issued
        i32x8 kb;
        if (PF) {
          kb = kb_next;
          if (!(h == PP - 1 && nt == 3))
            kb_next = load_kb(keys, nt == 3 ? h + 1 : h, (nt + 1) & 3);
        } else {
          kb = load_kb(keys, h, nt);
        }
        f32x4 acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[m] = mfma16x16x128_fp8(qa[m], kb, f32x4{0.f, 0.f, 0.f, 0.f});
        if (LIN) {
          v[nt] = head_reduce_abs<MT>(acc, w);
          if (nt == 0) {
            // L of rows 4 G + g, keys of N-tile wq
            const f32x4 lin = mfma16x16x128_fp8(alin, kb, f32x4{0.f, 0.f, 0.f, 0.f});
            const float4 lsc =
                *reinterpret_cast<const float4*>(&s_ascale[4 * G + g][0]);
            const float lval = fmaf(lsc.w, lin[3],
                               fmaf(lsc.z, lin[2],
                               fmaf(lsc.y, lin[1], lsc.x * lin[0])));
            s_lin[buf][4 * G + g][kPageTokens * h + 16 * wq + i16] = lval;
          }
        } else {
          v[nt] = head_reduce<MT>(acc, w);
        }
      }
      // lane group g ends with N-tile (wq + g) mod 4: token tok of the page
      const float tot = reduce_scatter4(v[0], v[1], v[2], v[3]);
      const int s = pj * kPageTokens + tok;
      // a page outside the pool scores -inf
      const int page = page_id(pj);
      const bool page_ok = page >= 0 && (int64_t)page < a.num_pages;
      if (LIN) {
        pt[h] = tot;
        pok[h] = page_ok;
      } else {
        const float val = (s <= prow && page_ok) ? tot * s_scale[sbuf][h][tok]
                                                 : -INFINITY;
        if (prow >= 0 && pj < je && pj <= (prow >> 6)) orow[s] = val;
      }
    }
    if (LIN) { pjp = jp; pbuf = buf; psbuf = sbuf; }
  };
  for (int jp = jb, si = 0;;) {
    step(jp, si, std::integral_constant<int, 0>());
    jp += PP; ++si;
    if (jp >= je) break;
    step(jp, si, std::integral_constant<int, 1>());
    jp += PP; ++si;
    if (jp >= je) break;
  }
  if (LIN) {
    __syncthreads();
    complete();
  }
  if (CAND && prow >= 0 && lane == 0)
    ft.count[t * gridDim.x + blockIdx.x] = cbase;
  // each half of the workgroup checks the pages it copies
  if (bad_page && lane == 0) raise_flag(kErrPageOutOfRange);
}

// ---------------------------------------------------------------------------
// Tiled logits without LDS staging: the same 16-row tile and page split,
// but every wave streams the pages itself (16-byte loads straight into MFMA
// B registers, next page prefetched); the 8 waves of a tile read the same
// page within a few hundred cycles, so HBM sees it once and L2 serves the
// rest.  No workgroup barrier inside the page loop, so the waves drift
// apart and one wave's MFMAs overlap another's epilogue.
// ---------------------------------------------------------------------------
template <int MT, bool FULL>
__global__ __launch_bounds__(512) void logits_tile_direct_kernel(
    LogitsArgs a, int pages_per_split) {
  __shared__ int s_info[4];
  __shared__ int s_pos[kTileRows];
  const int tid = threadIdx.x;
  const int wave = wave_uniform(tid >> 6);
  const int lane = lane_id();
  if (tid == 0) { s_info[0] = -1; s_info[1] = 0; s_info[2] = 0; }
  __syncthreads();
  if (wave == 0) find_tile(a.qsl, a.R, blockIdx.y, s_info);
  __syncthreads();
  const int r = s_info[0];
  if (r < 0) return;
  const int64_t row0 = s_info[1];
  const int nrows = s_info[2];
  if (tid < kTileRows) {
    int p = -1;
    if (tid < nrows && row0 + tid >= 0 && row0 + tid < a.T) {
      p = a.positions[row0 + tid];
      if (p < 0 || p >= a.ld || (int64_t)(p >> 6) >= a.bt_stride) {
        raise_flag(kErrPositionOutOfRange);
        p = -1;
      }
    }
    s_pos[tid] = p;
  }
  __syncthreads();
  int maxp = -1;
#pragma unroll
  for (int i = 0; i < kTileRows; ++i) maxp = max(maxp, s_pos[i]);
  const int npages = (maxp >> 6) + 1;
  const int jb = blockIdx.x * pages_per_split;
  const int je = min(jb + pages_per_split, npages);
  if (jb >= je) return;
  const int prow0 = s_pos[2 * wave], prow1 = s_pos[2 * wave + 1];
  if (prow0 < 0 && prow1 < 0) return;        // this wave has no rows
  // pages past both rows' positions are not needed by this wave
  const int my_je = min(je, (max(prow0, prow1) >> 6) + 1);
  if (jb >= my_je) return;

  const int32_t* bt = a.block_table + (int64_t)r * a.bt_stride;
  const int i16 = lane & 15, g = lane >> 4;
  i32x8 qa[2][MT];
  float w[2][MT][4];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int pr = rr ? prow1 : prow0;
    const int64_t t = row0 + 2 * wave + rr;
    if (pr >= 0) {
      load_q_frags<MT, FULL>(a.q8 + t * a.H * kHeadDim, a.H, qa[rr]);
      load_head_weights<MT, FULL>(a.weights + t * a.H, a.q_scale + t * a.H,
                                  a.H, w[rr]);
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        qa[rr][m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) w[rr][m][j] = 0.f;
      }
    }
  }

  auto valid = [&](int page) {
    return page >= 0 && (int64_t)page < a.num_pages;
  };
  // B fragments of one page plus the two k-scales this lane applies (token
  // 16*(2*ntp + (g & 1)) + i16 for ntp = 0, 1).
  auto load_page = [&](int page, i32x8 (&kb)[4], float (&ks)[2]) {
    const uint8_t* pg = a.k_cache + (int64_t)page * kPageBytes;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      kb[nt] = load_frag_global(pg + (16 * nt + i16) * kHeadDim + 32 * g);
    const float* sc = reinterpret_cast<const float*>(pg + kPageKeyBytes);
    ks[0] = sc[16 * (g & 1) + i16];
    ks[1] = sc[16 * (2 + (g & 1)) + i16];
  };

  i32x8 kb[4];
  float ks[2] = {0.f, 0.f};
  int cur = wave_uniform(bt[jb]);
  if (valid(cur)) load_page(cur, kb, ks);
  else if (lane == 0) raise_flag(kErrPageOutOfRange);
  const int rr_out = g >> 1;
  const int pr_out = rr_out ? prow1 : prow0;
  float* orow = a.logits + (row0 + 2 * wave + rr_out) * a.ld;

  for (int jp = jb; jp < my_je; ++jp) {
    i32x8 nb[4];
    float nks[2] = {0.f, 0.f};
    int nxt = -1;
    if (jp + 1 < my_je) {
      nxt = wave_uniform(bt[jp + 1]);
      if (valid(nxt)) load_page(nxt, nb, nks);
      else if (lane == 0) raise_flag(kErrPageOutOfRange);
    }
    const bool ok = valid(cur);
#pragma unroll
    for (int ntp = 0; ntp < 2; ++ntp) {
      float v[2][2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          f32x4 acc[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[m] = mfma16x16x128_fp8(qa[rr][m], kb[2 * ntp + q],
                                       f32x4{0.f, 0.f, 0.f, 0.f});
          v[rr][q] = head_reduce<MT>(acc, w[rr]);
        }
      }
      // lane group g ends with (row g >> 1, N-tile 2*ntp + (g & 1))
      const float tot = reduce_scatter4(v[0][0], v[0][1], v[1][0], v[1][1]);
      if (pr_out >= 0 && jp <= (pr_out >> 6)) {  // the row's own pages only
        const int s = jp * kPageTokens + 16 * (2 * ntp + (g & 1)) + i16;
        orow[s] = (s <= pr_out && ok) ? tot * ks[ntp] : -INFINITY;
      }
    }
    if (jp + 1 < my_je) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) kb[nt] = nb[nt];
      ks[0] = nks[0]; ks[1] = nks[1];
      cur = nxt;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_quantize_q(const uint16_t* q_bf16, int64_t blocks,
                             uint8_t* q8, float* q_scale, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  const int64_t grid = (blocks + 15) / 16;
  hipLaunchKernelGGL(quantize_q_kernel, dim3((unsigned)grid), dim3(256), 0,
                     stream, q_bf16, blocks, q8, q_scale);
  return hipGetLastError();
}

LogitsPlan logits_plan(int64_t T, int R) {
  const Options& o = options();
  bool tiled = T > 2 * (int64_t)R;
  if (o.logits_kernel == 1 || o.logits_kernel == 4) tiled = false;
  if (o.logits_kernel == 2 || o.logits_kernel == 3 || o.logits_kernel == 5 ||
      o.logits_kernel == 6)
    tiled = true;
  if (tiled) return LogitsPlan::Tiled;
  return T <= kBalancedMaxRows && o.logits_kernel != 4 ? LogitsPlan::Balanced
                                                       : LogitsPlan::Rowwise;
}

// Grid of the balanced decode kernel: D pages per wave; enough waves that a
// batch whose rows all reach max_pages still gets about D pages per wave;
// with the page schedule no head waves.
struct BalancedGeometry {
  int D;
  int64_t per_xcd;
  int hw;                 // head waves per row
  int64_t head_waves;
  int64_t waves;          // grid size (one wave per workgroup)
};

static BalancedGeometry balanced_geometry(int64_t T, int64_t max_pages,
                                          const Options& o, bool sched) {
  BalancedGeometry g{};
  int D = o.row_pages_per_wave;
  D = D <= 0 ? 3 : std::min(D, 4);
  if (D == 1) D = 2;
  g.D = D;
  const int64_t pmax = T * max_pages;
  const int64_t part = (pmax + 7) / 8;
  g.per_xcd =
      std::max<int64_t>(1, std::min<int64_t>((part + D - 1) / D, 1 << 13));
  // one head wave per row (measured: 10.54 -> 10.39 us on the decode
  // batch; more head waves gain nothing, the balanced waves' chain of three
  // round trips still ends the kernel); option value 1 + n sets n.  The
  // schedule removes that chain: no head waves.
  g.hw = sched ? 0 : (o.row_head_waves > 0 ? o.row_head_waves - 1 : 1);
  g.head_waves = g.hw ? (T * g.hw + 7) / 8 * 8 : 0;
  g.waves = g.head_waves + 8 * (g.per_xcd + T);
  return g;
}

// The page schedule serves decode launches of the balanced class whose D
// fits an entry.
static bool schedule_applies(int64_t T, int64_t max_pages, const Options& o) {
  return T >= 1 && T <= kBalancedMaxRows &&
         balanced_geometry(T, max_pages, o, true).D <= kSchedPages;
}

size_t logits_schedule_bytes(int64_t T, int64_t ld) {
  if (T < 1 || T > kBalancedMaxRows || ld < 1) return 0;
  // the most waves any option value gives: D = 2, max_pages = ld / 64
  Options o{};
  o.row_pages_per_wave = 2;
  const int64_t w = balanced_geometry(T, (ld + 63) / 64, o, true).waves;
  return (size_t)w * kSchedInts * sizeof(int32_t);
}

// Grid of the tiled logits kernels: gx page splits per tile (the 16-row
// kernel re-cuts each tile's own pages into gx equal ranges unless the
// split size is forced: pps16 > 0), tiles workgroup rows (an upper bound:
// grid rows past the last tile exit at once).
struct TileGeometry {
  int64_t gx, tiles;
  int pps, pps16;
  bool deep;                    // four pages per copy step
};

static TileGeometry tile_geometry(int64_t T, int R, int64_t max_pages,
                                  const Options& o) {
  TileGeometry g{};
  g.tiles = (T + kTileRows - 1) / kTileRows + R;
  int pps = o.tile_pages_per_split;
  if (pps <= 0) {
    const int64_t real_tiles = (T + kTileRows - 1) / kTileRows;
    int64_t splits = (2048 + real_tiles - 1) / real_tiles;
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, max_pages));
    // at least 64 pages per workgroup: a 16-wave workgroup has a
    // noticeable start (tile lookup, q fragments, first page pair); the
    // 1M-token tail (one tile) measured best at 64 (256 workgroups)
    pps = (int)std::max<int64_t>(64, (max_pages + splits - 1) / splits);
    // One 16-wave workgroup fills a compute unit, so the grid runs in
    // rounds of `cus` workgroups and a last round that is barely used
    // costs a whole round (a 103-tile launch with 10 splits is 4 rounds
    // and 6 workgroups).  Among 1/2 .. 1 times the splits chosen above,
    // take the one with the fewest rounds per unit of work, the nearest
    // to that choice on a tie.
    const int64_t g0 = (max_pages + pps - 1) / pps;
    const int64_t cus = device_cu_count();
    int64_t best = g0, br = (g0 * real_tiles + cus - 1) / cus;
    for (int64_t g = g0 - 1; g >= (g0 + 1) / 2; --g) {
      const int64_t r = (g * real_tiles + cus - 1) / cus;
      if (r * best < br * g) { best = g; br = r; }   // r / g < br / best
    }
    if (best != g0) pps = (int)((max_pages + best - 1) / best);
  }
  g.pps = pps;
  g.gx = std::max<int64_t>(1, (max_pages + pps - 1) / pps);
  g.pps16 = o.tile_pages_per_split > 0 ? pps : 0;
  // four pages per copy step (twice the lookahead) when the workgroups
  // take more than two rounds of the compute units: measured faster on
  // the prefill chunk (8 rounds); on the 1M tail (2 rounds) the step was
  // slower
  g.deep = o.tile_pages_per_step == 4 ||
           (o.tile_pages_per_step == 0 &&
            g.gx * g.tiles > 2 * (int64_t)device_cu_count());
  return g;
}

template <int MT, bool FULL>
static hipError_t launch_logits_mt(const LogitsArgs& a, hipStream_t stream,
                                   LogitsPlan plan, int64_t max_pages,
                                   const int32_t* sched) {
  const Options& o = options();
  const bool tiled = plan == LogitsPlan::Tiled;
  if (plan == LogitsPlan::Balanced && a.T <= kBalancedMaxRows) {
    const bool use_sched = sched && schedule_applies(a.T, max_pages, o);
    const BalancedGeometry bg = balanced_geometry(a.T, max_pages, o, use_sched);
    const dim3 grid((unsigned)bg.waves);
    const bool two = a.T > 64;
    const int per_xcd = (int)bg.per_xcd, hw = bg.hw, hwv = (int)bg.head_waves;
#define DSA_BAL(DD, SC)                                                      \
    if (two) hipLaunchKernelGGL((logits_balanced_kernel<MT, FULL, DD, 2, SC>),\
                                grid, dim3(64), 0, stream, a, per_xcd, hw,    \
                                hwv, sched);                                  \
    else hipLaunchKernelGGL((logits_balanced_kernel<MT, FULL, DD, 1, SC>),    \
                            grid, dim3(64), 0, stream, a, per_xcd, hw, hwv,   \
                            sched);
    if (use_sched) {
      if (bg.D == 2) { DSA_BAL(2, true) } else { DSA_BAL(3, true) }
    } else if (bg.D == 2) { DSA_BAL(2, false) }
    else if (bg.D == 3) { DSA_BAL(3, false) }
    else { DSA_BAL(4, false) }
#undef DSA_BAL
  } else if (!tiled) {
    int ppw = o.row_pages_per_wave;
    if (ppw <= 0) {
      // about 512 workgroups of 4 waves: enough waves in flight to keep
      // HBM busy, few enough that each streams several pages with the next
      // one prefetched (measured best on the decode batch)
      const int64_t pages = a.T * max_pages;
      ppw = (int)std::max<int64_t>(1, std::min<int64_t>(8, pages / (4 * 512)));
    }
    if (ppw > 64) ppw = 64;
    const int64_t gy = (max_pages + 4 * ppw - 1) / (4 * ppw);
    if (ppw > 1)
      hipLaunchKernelGGL((logits_row_prefetch_kernel<MT, FULL>),
                         dim3((unsigned)a.T, (unsigned)gy), dim3(256), 0,
                         stream, a, ppw);
    else
      hipLaunchKernelGGL((logits_row_kernel<MT, FULL>),
                         dim3((unsigned)a.T, (unsigned)gy), dim3(256), 0,
                         stream, a, ppw);
  } else {
    const TileGeometry tg = tile_geometry(a.T, a.R, max_pages, o);
    const int64_t tiles = tg.tiles, gx = tg.gx;
    const int pps = tg.pps, pps16 = tg.pps16;
    const bool deep = tg.deep;
    const dim3 g3((unsigned)gx, (unsigned)tiles);
    if (o.logits_kernel == 5)
      hipLaunchKernelGGL((logits_tile16_kernel<MT, FULL, false, 2, false, false>),
                         g3, dim3(kT16Threads), 0, stream, a, pps16, 64,
                         FusedTile{});
    else if (o.logits_kernel != 2 && o.logits_kernel != 3 && deep)
      hipLaunchKernelGGL((logits_tile16_kernel<MT, FULL, true, 4, true, false>),
                         g3, dim3(kT16Threads), 0, stream, a, pps16, 64,
                         FusedTile{});
    else if (o.logits_kernel != 2 && o.logits_kernel != 3)
      hipLaunchKernelGGL((logits_tile16_kernel<MT, FULL, true, 2, true, false>),
                         g3, dim3(kT16Threads), 0, stream, a, pps16, 64,
                         FusedTile{});
    else if (o.logits_kernel == 3)
      hipLaunchKernelGGL((logits_tile_direct_kernel<MT, FULL>),
                         dim3((unsigned)gx, (unsigned)tiles),
                         dim3(kTileWaves * 64), 0, stream, a, pps);
    else
      hipLaunchKernelGGL((logits_tile_kernel<MT, FULL>),
                         dim3((unsigned)gx, (unsigned)tiles),
                         dim3(kTileWaves * 64), 0, stream, a, pps);
  }
  return hipGetLastError();
}

static int64_t logits_max_pages(const LogitsArgs& a) {
  return std::min<int64_t>(a.bt_stride, a.ld / kPageTokens);
}

hipError_t launch_logits(const LogitsArgs& a, hipStream_t stream,
                         LogitsPlan plan, const int32_t* sched) {
  if (a.T <= 0) return hipSuccess;
  const int64_t max_pages = logits_max_pages(a);
  if (plan == LogitsPlan::Auto) plan = logits_plan(a.T, a.R);
  switch (a.H) {
    case 16: return launch_logits_mt<1, true>(a, stream, plan, max_pages, sched);
    case 32: return launch_logits_mt<2, true>(a, stream, plan, max_pages, sched);
    case 48: return launch_logits_mt<3, true>(a, stream, plan, max_pages, sched);
    case 64: return launch_logits_mt<4, true>(a, stream, plan, max_pages, sched);
    default: break;
  }
  switch ((a.H + 15) / 16) {
    case 1: return launch_logits_mt<1, false>(a, stream, plan, max_pages, sched);
    case 2: return launch_logits_mt<2, false>(a, stream, plan, max_pages, sched);
    case 3: return launch_logits_mt<3, false>(a, stream, plan, max_pages, sched);
    default: return launch_logits_mt<4, false>(a, stream, plan, max_pages, sched);
  }
}

// ---------------------------------------------------------------------------
// Tile passes of the fused forward (the default 16-row class with the
// linear-term epilogue, whatever logits_kernel says).
// ---------------------------------------------------------------------------
template <typename F>
static hipError_t with_heads(int H, F f) {
  switch (H) {
    case 16: return f(std::integral_constant<int, 1>(), std::true_type());
    case 32: return f(std::integral_constant<int, 2>(), std::true_type());
    case 48: return f(std::integral_constant<int, 3>(), std::true_type());
    case 64: return f(std::integral_constant<int, 4>(), std::true_type());
    default: break;
  }
  switch ((H + 15) / 16) {
    case 1: return f(std::integral_constant<int, 1>(), std::false_type());
    case 2: return f(std::integral_constant<int, 2>(), std::false_type());
    case 3: return f(std::integral_constant<int, 3>(), std::false_type());
    default: return f(std::integral_constant<int, 4>(), std::false_type());
  }
}

int64_t fused_candidate_splits(const LogitsArgs& a) {
  return tile_geometry(a.T, a.R, logits_max_pages(a), options()).gx;
}

hipError_t launch_logits_sample(const LogitsArgs& a, int page_stride,
                                float* samp, int64_t ld_s,
                                hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  LogitsArgs s = a;
  s.logits = samp;
  s.out_ld = ld_s;
  s.page_stride = page_stride;
  const int64_t lp = (logits_max_pages(a) + page_stride - 1) / page_stride;
  const int64_t real_tiles = (a.T + kTileRows - 1) / kTileRows;
  // about two workgroups per compute unit, at least two logical pages each
  const int64_t cus = device_cu_count();
  const int64_t gx = std::max<int64_t>(
      1, std::min<int64_t>((2 * cus + real_tiles - 1) / real_tiles,
                           (lp + 1) / 2));
  const dim3 g3((unsigned)gx, (unsigned)(real_tiles + a.R));
  return with_heads(a.H, [&](auto mt, auto full) {
    constexpr int MT = decltype(mt)::value;
    constexpr bool FULL = decltype(full)::value;
    hipLaunchKernelGGL((logits_tile16_kernel<MT, FULL, true, 2, true, false>),
                       g3, dim3(kT16Threads), 0, stream, s, 0, 2, FusedTile{});
    return hipGetLastError();
  });
}

hipError_t launch_logits_candidates(const LogitsArgs& a, const FusedTile& ft,
                                    int64_t gx, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  const TileGeometry tg =
      tile_geometry(a.T, a.R, logits_max_pages(a), options());
  if (tg.gx != gx) return hipErrorInvalidValue;   // options changed between
  const dim3 g3((unsigned)tg.gx, (unsigned)tg.tiles);
  return with_heads(a.H, [&](auto mt, auto full) {
    constexpr int MT = decltype(mt)::value;
    constexpr bool FULL = decltype(full)::value;
    if (tg.deep)
      hipLaunchKernelGGL((logits_tile16_kernel<MT, FULL, true, 4, true, true>),
                         g3, dim3(kT16Threads), 0, stream, a, tg.pps16, 64,
                         ft);
    else
      hipLaunchKernelGGL((logits_tile16_kernel<MT, FULL, true, 2, true, true>),
                         g3, dim3(kT16Threads), 0, stream, a, tg.pps16, 64,
                         ft);
    return hipGetLastError();
  });
}

// q quantisation plus, in the same launch, the decode page schedule of the
// logits launch that follows (extra 4-wave workgroups, one wave per entry).
static hipError_t launch_quantize_q_sched(const ForwardArgs& f,
                                          int64_t max_pages,
                                          hipStream_t stream) {
  const int64_t blocks = f.lg.T * f.lg.H;
  const int64_t qgrid = (blocks + 15) / 16;
  const BalancedGeometry bg =
      balanced_geometry(f.lg.T, max_pages, options(), true);
  const int64_t sgrid = (bg.waves + 3) / 4;
  const dim3 grid((unsigned)(qgrid + sgrid));
  if (f.lg.T > 64)
    hipLaunchKernelGGL(quantize_q_sched_kernel<2>, grid, dim3(256), 0, stream,
                       f.q_bf16, blocks, f.q8, f.q_scale, (int)qgrid, f.lg,
                       bg.D, (int)bg.per_xcd, (int)bg.waves, f.sched);
  else
    hipLaunchKernelGGL(quantize_q_sched_kernel<1>, grid, dim3(256), 0, stream,
                       f.q_bf16, blocks, f.q8, f.q_scale, (int)qgrid, f.lg,
                       bg.D, (int)bg.per_xcd, (int)bg.waves, f.sched);
  return hipGetLastError();
}

// The page schedule alone (dsa_logits_schedule): the builder workgroups of
// the launch above, no quantisation.
hipError_t launch_logits_schedule(const LogitsArgs& a, int32_t* sched,
                                  hipStream_t stream) {
  if (a.T <= 0 || a.T > kBalancedMaxRows) return hipSuccess;
  const BalancedGeometry bg =
      balanced_geometry(a.T, logits_max_pages(a), options(), true);
  const dim3 grid((unsigned)((bg.waves + 3) / 4));
  if (a.T > 64)
    hipLaunchKernelGGL(quantize_q_sched_kernel<2>, grid, dim3(256), 0, stream,
                       nullptr, (int64_t)0, nullptr, nullptr, 0, a, bg.D,
                       (int)bg.per_xcd, (int)bg.waves, sched);
  else
    hipLaunchKernelGGL(quantize_q_sched_kernel<1>, grid, dim3(256), 0, stream,
                       nullptr, (int64_t)0, nullptr, nullptr, 0, a, bg.D,
                       (int)bg.per_xcd, (int)bg.waves, sched);
  return hipGetLastError();
}

// One layer's hot path: q quantisation, logits, top-k.  A decode batch of
// the balanced class with a schedule buffer builds its page schedule in the
// quantisation launch (build_sched; otherwise the buffer already holds the
// schedule of the same positions, query_start_loc and block table) and the
// logits launch reads it.
hipError_t launch_forward(const ForwardArgs& f, hipStream_t stream) {
  if (f.lg.T <= 0) return hipSuccess;
  const int64_t max_pages = logits_max_pages(f.lg);
  const LogitsPlan plan = logits_plan(f.lg.T, f.lg.R);
  const bool sched = f.sched && plan == LogitsPlan::Balanced &&
                     schedule_applies(f.lg.T, max_pages, options());
  hipError_t e;
  if (sched && f.build_sched)
    e = launch_quantize_q_sched(f, max_pages, stream);
  else
    e = launch_quantize_q(f.q_bf16, f.lg.T * f.lg.H, f.q8, f.q_scale, stream);
  if (e == hipSuccess)
    e = launch_logits(f.lg, stream, plan, sched ? f.sched : nullptr);
  if (e == hipSuccess) e = launch_topk(f.tk, stream);
  return e;
}

hipError_t read_logits_flags(unsigned* flags, bool reset) {
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_err_logits),
                                     sizeof(unsigned), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess || !reset) return e;
  const unsigned zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_err_logits), &zero, sizeof(unsigned), 0,
                           hipMemcpyHostToDevice);
}

}  // namespace dsa
