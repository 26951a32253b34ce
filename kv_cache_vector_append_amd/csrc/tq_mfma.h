// Building blocks of the matrix-core (MFMA) decode on gfx950.
//
// The decode contractions -- query x decoded keys for the GQA group, and
// softmax weights x decoded values -- run on v_mfma_scale_f32_16x16x128_f8f6f4
// with one operand in fp4 (e2m1) and the other in fp8 (e4m3, OCP encoding):
//
//  * Every code bit-plane is a +-1 matrix: a symmetric Lloyd-Max codebook is
//    an odd function of the code's sign bits s_k = 1 - 2 bit_k,
//    c[idx] = sum over odd subsets S of a_S prod_{k in S} s_k, so a dot
//    product with decoded codes is a weighted sum of +-1 plane products, and
//    the QJL bits are +-1 already.  Key bits turn into fp4 operands with one
//    ALU operation per 8 values through an affine encoding
//    (bits_to_fp4_affine); value bits, whose products are summed over many
//    tokens, keep a centred encoding, +-6 (bits_to_fp4_pm6_dwords): an affine
//    offset there grows with the token count while the result does not, and
//    costs accuracy in the matrix-core sums.
//  * The fp32 operand (rotated query, softmax weight) is split into four fp8
//    parts x = sum_p 16^-p x_p held in four operand rows; the fp32 accumulator
//    then carries about 2^-17 relative precision, far below the fp32 -> fp64
//    parity tolerance.
//
// Register layouts of the 16x16x128 f8f6f4 MFMA on gfx950 (lane l, group
// g = l / 16, index r = l % 16; measured on the device):
//   fp8 operand:  32 bytes per lane; byte e holds K index 16g + e (e < 16) or
//                 64 + 16g + (e - 16) (e >= 16); row/column r.
//   fp4 operand:  16 bytes per lane; nibble e (low nibble first) holds K index
//                 32g + e; row/column r.
//   result:       4 floats per lane; float i holds row 4g + i, column r.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqi {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0;
constexpr int kFmtFp4 = 4;
constexpr int kScaleOne = 127;  // E8M0 exponent of 1.0

// Operand scales are E8M0 exponents (2^(s - 127)) held per lane: lane l
// scales row (A) or column (B) l % 16 over its own K group l / 16 (measured on
// the device), so a per-row or per-column power of two costs nothing.

// acc += (A(fp8) * 2^(scale_a - 127)) x B(fp4)
__device__ __forceinline__ v4f mfma_f8_f4(const v8i& a, const v8i& b, v4f acc, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, kFmtFp8, kFmtFp4, 0, scale_a, 0, kScaleOne);
}

// acc += A(fp4) x (B(fp8) * 2^(scale_b - 127))
__device__ __forceinline__ v4f mfma_f4_f8(const v8i& a, const v8i& b, v4f acc, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, kFmtFp4, kFmtFp8, 0, kScaleOne, 0, scale_b);
}

// 32 code bits -> 32 fp4 values, one ALU operation per 8 values.  Dword j
// takes the bits 4n + j of w (n = 0..7) in place, so fp4 element e = 8j + n
// comes from bit 4(e % 8) + e / 8, and a set bit reads as 0.5, 1.0 or 2.0 for
// j = 0, 1, 2 (clear: 0) and as -1.0 for j = 3 (clear: +1.0).  With
// s = 1 - 2 bit, the +-1 sign of a bit is s = 1 + f_j v for j < 3 and s = v
// for j = 3, where v is the fp4 value and f_j = -4, -2, -1; so
//   sum_c x_c s_c = sum_{c : j(c) < 3} x_c + sum_c (f_j(c) x_c) v_c,
// i.e. the other operand carries the factor f_j and a per-row constant is
// added to the product.
__device__ __forceinline__ v8i bits_to_fp4_affine(uint32_t w) {
  // dword 3 = (w & 0x88888888) | 0x22222222 in one bitop3
  const v4i lo = {int(w & 0x11111111u), int(w & 0x22222222u), int(w & 0x44444444u),
                  int(__builtin_amdgcn_bitop3_b32(w, 0x88888888u, 0x22222222u, 0xEA))};
  // an fp4 operand occupies the low four registers; the upper four are not read
  return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1);
}

// v_bitop3_b32 truth tables (operands a, b, c stand for 0xF0, 0xCC, 0xAA)
constexpr int kAndOr = 0xEA;  // (a & b) | c
constexpr int kXor3 = 0x96;   // a ^ b ^ c

// 32 sign bits -> 32 fp4 values +-6 (bit set -> -6.0), same element order as
// bits_to_fp4_affine, one shift-or per dword: dword j = (w << (3 - j)) |
// 0x77777777.  The OR forces both exponent bits and the mantissa bit of every
// nibble to one (e2m1 0111 = 6.0), so whatever bits the shift brings into
// those places, only the sign bit -- bit 4n + j of w -- carries data.
constexpr uint32_t kPm6Fill = 0x77777777u;
constexpr float kPm6 = 6.f;
__device__ __forceinline__ v4i bits_to_fp4_pm6_dwords(uint32_t w) {
  return v4i{int((w << 3) | kPm6Fill), int((w << 2) | kPm6Fill), int((w << 1) | kPm6Fill), int(w | kPm6Fill)};
}
// The +-6 encoding of the XOR of three bit words: XOR of their encodings (the
// 0111 magnitude bits of three operands XOR back to 0111, the signs multiply).
__device__ __forceinline__ v4i fp4_pm6_product3(const v4i& a, const v4i& b, const v4i& c) {
  return v4i{int(__builtin_amdgcn_bitop3_b32(uint32_t(a[0]), uint32_t(b[0]), uint32_t(c[0]), kXor3)),
             int(__builtin_amdgcn_bitop3_b32(uint32_t(a[1]), uint32_t(b[1]), uint32_t(c[1]), kXor3)),
             int(__builtin_amdgcn_bitop3_b32(uint32_t(a[2]), uint32_t(b[2]), uint32_t(c[2]), kXor3)),
             int(__builtin_amdgcn_bitop3_b32(uint32_t(a[3]), uint32_t(b[3]), uint32_t(c[3]), kXor3))};
}
// an fp4 operand occupies the low four registers; the upper four are not read
__device__ __forceinline__ v8i fp4_operand(const v4i& lo) {
  return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1);
}

// Operand factor f_j for the element group j = (bit position) % 4 of the above.
__host__ __device__ constexpr float fp4_affine_factor(int j) {
  return j == 0 ? -4.f : j == 1 ? -2.f : j == 2 ? -1.f : 1.f;
}

// Bit position inside a 32-bit source word of fp4 element e (inverse of the above).
__host__ __device__ constexpr int fp4_elem_bit(int e) { return 4 * (e % 8) + e / 8; }

// K index held by byte e of an fp8 operand in lane group g.
__host__ __device__ constexpr int fp8_elem_k(int g, int e) { return e < 16 ? 16 * g + e : 64 + 16 * g + (e - 16); }

// Four-part fp8 split of x (|x| <= 448): bytes p0 | p1 << 8 | p2 << 16 | p3 << 24
// with x ~= p0 + p1/16 + p2/256 + p3/4096, each part rounded to nearest even.
__device__ __forceinline__ uint32_t fp8_split4(float x) {
  uint32_t out = 0;
  float r = x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(r, 0.0f, 0, false);
    const float back = __builtin_amdgcn_cvt_f32_fp8(packed, 0);
    out |= uint32_t(packed & 0xff) << (8 * p);
    r = (r - back) * 16.0f;
  }
  return out;
}

// The same four-part split for two values at once with the gfx950 scaled
// conversions (fp8(r / s) one way, fp8 * s back, s a power of two): part p of x
// is fp8(r_p 16^p) with r_0 = x and r_{p+1} = r_p - part_p 16^-p.  Byte order:
// lo = x0 | y0 << 8 | x1 << 16 | y1 << 24, hi likewise with parts 2 and 3.
// Both words of lo and hi are written, so they start from any caller values
// (seed_lo, seed_hi): registers that are dead anyway avoid two moves.
typedef short v2s __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp8_split4_pair(float x, float y, uint32_t seed_lo, uint32_t seed_hi, uint32_t& lo,
                                                uint32_t& hi) {
  v2s a = __builtin_bit_cast(v2s, seed_lo), b = __builtin_bit_cast(v2s, seed_hi);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(a, x, y, 1.0f, false);
  v2f r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(__builtin_bit_cast(uint32_t, a), 1.0f, false);
  x -= r.x;
  y -= r.y;
  a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(a, x, y, 0.0625f, true);
  r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(__builtin_bit_cast(uint32_t, a), 0.0625f, true);
  x -= r.x;
  y -= r.y;
  b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(b, x, y, 0.00390625f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(__builtin_bit_cast(uint32_t, b), 0.00390625f, false);
  x -= r.x;
  y -= r.y;
  b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(b, x, y, 0.000244140625f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

}  // namespace tqi
