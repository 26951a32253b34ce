// Device-side helpers shared by the kernels: element loads, fp16 conversion,
// wavefront (64-lane) reductions and the in-wavefront Walsh-Hadamard transform.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tqi {

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ float f16_bits_to_float(uint16_t b) {
  return float(__builtin_bit_cast(_Float16, b));
}

// Round to nearest even, as the IEEE conversion does.
__device__ __forceinline__ uint16_t float_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ __forceinline__ float load_elem(const void* base, int dtype, size_t i) {
  if (dtype == TQ_F32) return static_cast<const float*>(base)[i];
  const uint16_t b = static_cast<const uint16_t*>(base)[i];
  return dtype == TQ_BF16 ? bf16_bits_to_float(b) : f16_bits_to_float(b);
}

// Debug capacity check: ORs `bits` into the caller's status word (when one
// was given) from every lane where `bad` holds.
__device__ __forceinline__ void report(uint32_t* status, bool bad, uint32_t bits) {
  if (status != nullptr && bad) atomicOr(status, bits);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Word offset of 32-coordinate group g inside a key token row (each group
// holds its half's code planes, then its QJL plane when there is one).
__device__ __forceinline__ int key_group_word(const Codec& k, int g, int D) {
  const int hg = D / (2 * kGroup), lo = k.kbits[0] + k.qjl;
  return g < hg ? g * lo : hg * lo + (g - hg) * (k.kbits[1] + k.qjl);
}

// Word offset of coordinate pair i (coordinates 2i, 2i + 1) inside a value block.
__device__ __forceinline__ int value_pair_word(const Codec& k, int i, int D) {
  const int hp = D / 4;
  return i < hp ? i * k.vbits[0] : hp * k.vbits[0] + (i - hp) * k.vbits[1];
}

// Negate v when bit `bit` of the sign word is set (the Rademacher stage D).
__device__ __forceinline__ float apply_sign(float v, uint32_t bit) {
  return __uint_as_float(__float_as_uint(v) ^ (bit << 31));
}

// Sign bit (1 = negative) of coordinate c for a sign role in the parameter blob.
__device__ __forceinline__ uint32_t sign_bit(const uint8_t* params, int role, int c) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(params + kOffSigns + role * kSignRoleBytes);
  return (w[c >> 5] >> (c & 31)) & 1u;
}

// Unnormalised Sylvester-order Walsh-Hadamard transform of a d = 64*R vector
// spread over one wavefront: lane l holds coordinates r*64 + l, r < R.  The
// butterfly of half-width s pairs coordinate i (bit s clear) with i + s and
// maps (a, b) -> (a + b, a - b).
template <int R>
__device__ __forceinline__ void wave_fwht(float (&v)[R], int lane) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const bool upper = (lane & s) != 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float p = __shfl_xor(v[r], s);
      v[r] = upper ? (p - v[r]) : (v[r] + p);
    }
  }
#pragma unroll
  for (int s = 1; s < R; s <<= 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!(r & s)) {
        const float x = v[r], y = v[r + s];
        v[r] = x + y;
        v[r + s] = x - y;
      }
    }
  }
}

// Same transform for G vectors of length d stored row-major in LDS,
// performed by a whole workgroup (caller synchronises before and after).
__device__ __forceinline__ void block_fwht(float* buf, int G, int d, int tid, int nthreads) {
  for (int hs = 1; hs < d; hs <<= 1) {
    for (int b = tid; b < G * (d / 2); b += nthreads) {
      const int g = b / (d / 2), k = b % (d / 2);
      const int i = (k / hs) * 2 * hs + (k % hs);
      float* row = buf + g * d;
      const float x = row[i], y = row[i + hs];
      row[i] = x + y;
      row[i + hs] = x - y;
    }
    __syncthreads();
  }
}

}  // namespace tqi
