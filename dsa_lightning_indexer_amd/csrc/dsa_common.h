// Device-side building blocks shared by the gfx950 kernels of the DSA
// lightning-indexer library: fixed layout constants, the FP8 e4m3fn encoder,
// the FP8 MFMA wrapper and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Indexer-K cache layout (GLM-5.3 KV/indexer cache budget article, SGLang
// buffer-shape section and the IndexKeyCache.move comment in the eviction
// section): one 128-dim K per token, FP8 e4m3fn, plus one fp32 scale per
// 128-element block; a 64-token page stores 64 x 128 key bytes first, then
// 64 x 4 scale bytes: 8448 bytes.
constexpr int kPageTokens = 64;
constexpr int kHeadDim = 128;
constexpr int kPageKeyBytes = kPageTokens * kHeadDim;       // 8192
constexpr int kPageBytes = kPageKeyBytes + kPageTokens * 4;  // 8448
constexpr int kMaxHeads = 64;
// Rows of a tile of the tiled logits kernels: tiles of 16 consecutive rows
// from each request's first row.
constexpr int kTileRows = 16;
constexpr float kE4M3Max = 448.0f;

// Device error flags (sticky, cleared by dsa_device_error_flags(reset=1)).
constexpr unsigned kErrPageOutOfRange = 1u;   // block_table entry not in pool
constexpr unsigned kErrPositionOutOfRange = 2u;  // p < 0, p >= ld or page past bt
constexpr unsigned kErrCandidateOverflow = 4u;   // internal top-k list full

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16x16x128 FP8 (e4m3) x FP8 (e4m3) -> fp32 matrix FMA.  Operand format 0 on
// both sides selects e4m3; zero scale operands make the compiler emit the
// unscaled v_mfma_f32_16x16x128_f8f6f4.
__device__ __forceinline__ f32x4 mfma16x16x128_fp8(const i32x8& a,
                                                    const i32x8& b,
                                                    const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0,
                                                          0, 0);
}

// float -> OCP e4m3fn byte: round to nearest, ties to even mantissa,
// magnitudes >= 448 saturate to 448, NaN -> 0x7F.  Integer arithmetic on the
// fp32 bit pattern.
__device__ __forceinline__ uint32_t e4m3fn_encode(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;               // NaN
  uint32_t code;
  if (a >= 0x43e00000u) {                          // |x| >= 448
    code = 0x7eu;
  } else if (a < 0x3c800000u) {                    // |x| < 2^-6: subnormal
    // value = m * 2^-9; scaling by 2^9 is exact, rint rounds half to even
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    const uint32_t e = (a >> 23) - 120u;           // rebias 127 -> 7
    const uint32_t mant = a & 0x7fffffu;
    code = (e << 3) | (mant >> 20);
    const uint32_t rem = mant & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;
    if (code > 0x7eu) code = 0x7eu;
  }
  return code | sign;
}

// q / s for an FP8 block scale s (= amax / 448) and r = 1 / s, both IEEE
// float32: the reciprocal product with one FMA correction -- y = q r, then
// e = q - s y (exact), y + e r; y itself when e = 0 (keeps the sign of a
// zero).  For a finite block of bf16 values with s >= 2^-100 its FP8 code
// (hardware e4m3 conversion) equals the integer encoder's code of the IEEE
// quotient q / s for every q with |q| <= amax: dsa_fp8_code_check counts the
// pairs where it does not (none on gfx950).
__device__ __forceinline__ float div_by_scale(float q, float s, float r) {
  const float y0 = q * r;
  const float e = fmaf(-y0, s, q);
  return e == 0.f ? y0 : fmaf(e, r, y0);
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger
// key); -0 is folded onto +0 first so the two compare equal.
__device__ __forceinline__ uint32_t float_to_ordered(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of float_to_ordered (-0 comes back as +0).
__device__ __forceinline__ float ordered_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The value of a wave-uniform expression, held in a scalar register.
__device__ __forceinline__ int wave_uniform(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP: four
// row_shr steps within each 16-lane row, then row_bcast:15 / row_bcast:31
// carry the row totals into the later rows.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false); // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false); // row_bcast:31
  return x;
}

// Read-only metadata (positions, query_start_loc, block table) through the
// constant address space: a wave-uniform index becomes a scalar load, which
// travels on the scalar cache path instead of queueing behind the vector
// loads in flight on the compute unit.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int load_uniform(const int32_t* p, int64_t i) {
  return ((const_i32*)(p))[i];
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero without touching memory and stores past the end are dropped, so a
// load or store can be issued unconditionally and switched off by its size.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes,
                                           0x00020000);
}

// Row -> request index by binary search over query_start_loc[0..R].
__device__ __forceinline__ int request_of_row(const int32_t* qsl, int R,
                                              int64_t t) {
  int lo = 0, hi = R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Sum over the 4 lane groups (lanes l, l^16, l^32, l^48) of four partial
// values, scattered so that lane group g ends with the total of value g.
// gfx950's permlane swaps do the exchange in VALU: the 32-lane swap of
// (v0, v2) leaves lanes < 32 with v0 of lanes l and l + 32 and lanes >= 32
// with v2 of lanes l - 32 and l (likewise (v1, v3)); the 16-lane swap of the
// two sums then pairs 16-lane rows 0/1 and 2/3.  Each total is the same two
// additions in the same order as an exchange through lane shuffles.
__device__ __forceinline__ float reduce_scatter4(float v0, float v1, float v2,
                                                 float v3) {
  const auto p02 = __builtin_amdgcn_permlane32_swap(
      __float_as_uint(v0), __float_as_uint(v2), false, false);
  const auto p13 = __builtin_amdgcn_permlane32_swap(
      __float_as_uint(v1), __float_as_uint(v3), false, false);
  const float a = __uint_as_float(p02[0]) + __uint_as_float(p02[1]);
  const float b = __uint_as_float(p13[0]) + __uint_as_float(p13[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a),
                                                  __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

}  // namespace dsa
