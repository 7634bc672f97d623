// Scoring building blocks shared by the logits kernels and the fused
// forward's rescue path: the FP8 MFMA operand loads (row-major and
// chunk-major reduction order), the folded head weights, the per-output
// head reduction, and the shared linear term of the tile kernels (qlin
// split into e4m3 pieces).  Each logit's arithmetic is fixed by these
// functions, so two kernels that call them in the same order for a (row,
// page) produce the same bits.
#pragma once

#include "dsa_common.h"

namespace dsa {

// ---------------------------------------------------------------------------
// MFMA operand layout used below (v_mfma_f32_16x16x128_f8f6f4, wave64):
//   A (16 x 128): lane l holds row (l % 16), 32 bytes of K-chunk (l / 16);
//   B (128 x 16): lane l holds column (l % 16), the same 32-byte K-chunk;
//   C (16 x 16):  lane l holds rows 4*(l/16) + j, j = 0..3, column (l % 16).
// A and B place the 128-long reduction index identically, so loading q rows
// and K rows with the same byte pattern gives the exact dot products.
// Rows of A are heads (16 per M-tile), columns of B are tokens (16 per
// N-tile); a 64-token page is 4 N-tiles.
// ---------------------------------------------------------------------------
__device__ __forceinline__ i32x8 load_frag_global(const uint8_t* row32) {
  const uint4 x = *reinterpret_cast<const uint4*>(row32);
  const uint4 y = *reinterpret_cast<const uint4*>(row32 + 16);
  i32x8 v = {(int)x.x, (int)x.y, (int)x.z, (int)x.w,
             (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  return v;
}

// A fragments of one query row (MT M-tiles of 16 heads; heads >= H are 0).
// FULL (H == 16 * MT): plain loads.  Otherwise the head index is clamped so
// every load stays in bounds and is issued unconditionally (no divergent
// branch, so the loads overlap), and padded heads are zeroed afterwards.
template <int MT, bool FULL>
__device__ __forceinline__ void load_q_frags(const uint8_t* q8_row, int H,
                                             i32x8 (&qa)[MT]) {
  const int lane = lane_id();
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int head = 16 * m + i16;
    const int hh = FULL ? head : min(head, H - 1);
    qa[m] = load_frag_global(q8_row + hh * kHeadDim + 32 * g);
    if (!FULL && head >= H) qa[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// The same fragments in the chunk-major K order of the 16-row tile kernel:
// lane l holds bytes [16 (l / 16), + 16) and [64 + 16 (l / 16), + 16) of its
// row (a permutation of the 128-long reduction index; A and B use the same
// one, so the dot products are unchanged).
template <int MT, bool FULL>
__device__ __forceinline__ void load_q_frags_cm(const uint8_t* q8_row, int H,
                                                i32x8 (&qa)[MT]) {
  const int lane = lane_id();
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int head = 16 * m + i16;
    const int hh = FULL ? head : min(head, H - 1);
    const uint8_t* row = q8_row + hh * kHeadDim + 16 * g;
    const uint4 x = *reinterpret_cast<const uint4*>(row);
    const uint4 y = *reinterpret_cast<const uint4*>(row + 64);
    qa[m] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                  (int)y.x, (int)y.y, (int)y.z, (int)y.w};
    if (!FULL && head >= H) qa[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// Per-lane effective head weights w[h] * s_q[h] / 2 for the C rows this
// lane holds: head 16*m + 4*(lane/16) + j, j = 0..3 (4 consecutive heads,
// one 16-byte load each when FULL).  The 1/2 belongs to head_reduce's ReLU.
template <int MT, bool FULL>
__device__ __forceinline__ void load_head_weights(const float* w_row,
                                                  const float* s_row, int H,
                                                  float (&w)[MT][4]) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (FULL) {
      const float4 wv = *reinterpret_cast<const float4*>(w_row + 16 * m + 4 * g);
      const float4 sv = *reinterpret_cast<const float4*>(s_row + 16 * m + 4 * g);
      w[m][0] = 0.5f * (wv.x * sv.x); w[m][1] = 0.5f * (wv.y * sv.y);
      w[m][2] = 0.5f * (wv.z * sv.z); w[m][3] = 0.5f * (wv.w * sv.w);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int head = 16 * m + 4 * g + j;
        const int hh = min(head, H - 1);
        const float x = 0.5f * (w_row[hh] * s_row[hh]);
        w[m][j] = head < H ? x : 0.f;
      }
    }
  }
}

// sum over this lane's heads of w * ReLU(dot) for one N-tile.  ReLU is
// written as (x + |x|) / 2 with the 1/2 folded into the weights: one add
// with an abs source modifier and one FMA per MFMA output (a plain fmaxf
// costs an extra NaN-canonicalising max on gfx950).
template <int MT>
__device__ __forceinline__ float head_reduce(const f32x4 (&acc)[MT],
                                             const float (&w_half)[MT][4]) {
  float v = 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v = fmaf(w_half[m][j], acc[m][j] + fabsf(acc[m][j]), v);
  return v;
}

// The same sum without the linear part: sum over this lane's heads of
// w * |dot| (one FMA with an abs source modifier per MFMA output).  The
// tile kernels add sum_h w * dot, computed once for four rows, afterwards.
template <int MT>
__device__ __forceinline__ float head_reduce_abs(const f32x4 (&acc)[MT],
                                                 const float (&w_half)[MT][4]) {
  float v = 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) v = fmaf(w_half[m][j], fabsf(acc[m][j]), v);
  return v;
}

// ---------------------------------------------------------------------------
// One 64-token page of the decode kernels, K read straight into the MFMA B
// operand: N-tile nt (tokens 16 nt .. 16 nt + 15) of lane l is token 16 nt
// + l % 16, bytes 32 (l / 16) .. + 31 of its key; lane l also takes the
// scale of token l.  rs covers the page's 8448 bytes (zero size for a page
// that is not scored: every load returns 0 without touching memory).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load_k_page_regs(__amdgpu_buffer_rsrc_t rs,
                                                 i32x8 (&kb)[4], float& ks) {
  const int lane = lane_id();
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int off = (16 * nt + i16) * kHeadDim + 32 * g;
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    const auto y = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0);
    kb[nt] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                   (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  }
  ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      rs, kPageKeyBytes + 4 * lane, 0, 0));
}

// Head-weighted ReLU sum of one page for one query row, before the K scale:
// lane l ends with token l's sum over the H heads (16 MFMAs for H = 64, the
// head reduction of each N-tile, then the lane-group reduce-scatter).
template <int MT>
__device__ __forceinline__ float decode_page_sum(const i32x8 (&qa)[MT],
                                                 const i32x8 (&kb)[4],
                                                 const float (&w)[MT][4]) {
  float v[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      acc[m] = mfma16x16x128_fp8(qa[m], kb[nt], f32x4{0.f, 0.f, 0.f, 0.f});
    v[nt] = head_reduce<MT>(acc, w);
  }
  return reduce_scatter4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------------------
// Linear part of the head reduction, shared by four rows (tile kernel).
// With ReLU written as (x + |x|) / 2 and the 1/2 folded into the weights,
//   sum_h w_h (x_h + |x_h|) = L + sum_h w_h |x_h|,
//   L = sum_h w_h x_h = qlin . code_k,   qlin = sum_h w_h code_q[h, :],
// so the per-output epilogue is a single FMA, and L costs one more FP8
// MFMA per 16 keys for four rows together.  qlin (fp32) is split into
// kLinPieces FP8 pieces, qlin ~= sum_p s_p c_p: s_p an fp32 scale, c_p the
// e4m3 rounding of what the earlier pieces left over.  Each piece shrinks
// the largest residual at least 28-fold (half an e4m3 step at the top of
// the range is 1/28 of it), so four pieces leave at most ~1.6e-6 max|qlin|
// per element, far inside the fp32 accumulation error of the dot products.
// The A operand of that MFMA has rows 4 q + p = (row q of the group, piece
// p), so lane group q of its output holds the four pieces of row q.
// ---------------------------------------------------------------------------
constexpr int kLinPieces = 4;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// One reduce-scatter step over v[0..N): lanes paired by the DPP pattern
// CTRL differ in `bit`; a lane keeps half `bit` of the list and adds the
// partner's copy of that half.
template <int CTRL, int N>
__device__ __forceinline__ void rs_step(float* v, bool bit) {
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const float send = bit ? v[j] : v[j + N / 2];
    const float keep = bit ? v[j + N / 2] : v[j];
    v[j] = keep + dpp_f<CTRL>(send);
  }
}

// Maximum over the wave of x >= 0 (wave-uniform result).
__device__ __forceinline__ float wave_max_nonneg(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));   // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));   // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// qlin of one row from its chunk-major A fragments (lane l: head 16 m +
// l % 16; byte j of qa[m] is dim 16 (l / 16) + j for j < 16 and 64 + 16 (l
// / 16) + j - 16 after; wa[m] the folded weight of that head), summed over
// the 16 lanes of each lane row by a reduce-scatter (row_mirror,
// row_half_mirror, then two quad permutations): lane l ends with bytes
// 2 (l % 16) and + 1 of that list.  The hardware fp8 -> f32 conversion
// decodes e4m3fn exactly.
template <int MT>
__device__ __forceinline__ float2 row_qlin(const i32x8 (&qa)[MT],
                                           const float (&wa)[MT]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  float v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(qa[m][k], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(qa[m][k], true);
      v[4 * k + 0] = fmaf(wa[m], lo[0], v[4 * k + 0]);
      v[4 * k + 1] = fmaf(wa[m], lo[1], v[4 * k + 1]);
      v[4 * k + 2] = fmaf(wa[m], hi[0], v[4 * k + 2]);
      v[4 * k + 3] = fmaf(wa[m], hi[1], v[4 * k + 3]);
    }
  const int i16 = lane_id() & 15;
  rs_step<0x140, 32>(v, (i16 >> 3) & 1);
  rs_step<0x141, 16>(v, (i16 >> 2) & 1);
  rs_step<0x4E, 8>(v, (i16 >> 1) & 1);
  rs_step<0xB1, 4>(v, i16 & 1);
  return make_float2(v[0], v[1]);
}

// Splits qlin (this lane's dims d, d + 1 as left by row_qlin) into
// kLinPieces e4m3 pieces, A row a = 4 q + p of the group's operand (q = the
// row within the group), stored chunk-major like the keys: byte d of A row
// a at group[(d / 64) * 1024 + (d / 16 % 4) * 256 + a * 16 + d % 16], so
// lane l reads its fragment at group + 16 l (+ 1024).  The scale of piece p
// goes to scales[p].  qlin is first brought to max|qlin| in [1, 2) by a
// power of two (exact), so a residual below 2^-60 -- nothing left that
// matters -- ends the split without dividing by a denormal.
__device__ __forceinline__ void split_pieces(float r0, float r1, int q,
                                             uint8_t* group, float* scales) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int lane = lane_id();
  const int i16 = lane & 15, g = lane >> 4;
  const int d = (i16 < 8 ? 16 * g : 64 + 16 * g - 16) + 2 * i16;
  const float amax0 = wave_max_nonneg(fmaxf(fabsf(r0), fabsf(r1)));
  int e = 0;
  if (amax0 > 0.f) (void)frexpf(amax0, &e);
  const int E = amax0 > 0.f ? 1 - e : 0;          // amax0 * 2^E in [1, 2)
  r0 = __builtin_amdgcn_ldexpf(r0, E);
  r1 = __builtin_amdgcn_ldexpf(r1, E);
#pragma unroll
  for (int p = 0; p < kLinPieces; ++p) {
    const float amax = wave_max_nonneg(fmaxf(fabsf(r0), fabsf(r1)));
    const bool live = amax > 0x1p-60f;
    const float inv = live ? kE4M3Max / amax : 0.f;
    const float sc = live ? amax / kE4M3Max : 0.f;
    const uint32_t c0 = e4m3fn_encode(r0 * inv);
    const uint32_t c1 = e4m3fn_encode(r1 * inv);
    const uint32_t pk = c0 | (c1 << 8);
    const f32x2 dec = __builtin_amdgcn_cvt_pk_f32_fp8((int)pk, false);
    r0 = fmaf(-sc, dec[0], r0);
    r1 = fmaf(-sc, dec[1], r1);
    *reinterpret_cast<uint16_t*>(group + (d >> 6) * 1024 + ((d >> 4) & 3) * 256 +
                                 (4 * q + p) * 16 + (d & 15)) = (uint16_t)pk;
    if (lane == 0) scales[p] = __builtin_amdgcn_ldexpf(sc, -E);
  }
}

// Folded weights w[h] * s_q[h] / 2 of the A-fragment heads of this lane:
// head 16 m + l % 16 (0 for heads >= H).
template <int MT, bool FULL>
__device__ __forceinline__ void load_a_weights(const float* w_row,
                                               const float* s_row, int H,
                                               float (&wa)[MT]) {
  const int i16 = lane_id() & 15;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int head = 16 * m + i16;
    const int hh = FULL ? head : min(head, H - 1);
    const float x = 0.5f * (w_row[hh] * s_row[hh]);
    wa[m] = (FULL || head < H) ? x : 0.f;
  }
}

}  // namespace dsa
