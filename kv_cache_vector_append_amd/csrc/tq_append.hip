// Quantize-append kernel.
//
// Per post-RoPE key / value head vector ([Reconstruction] = "Mathematical
// Reconstruction, Lineage, and Accuracy Limits of TurboQuant and TurboVec",
// section 5 steps 1-5 and section 6; [Design Study] = "TurboQuant Family Design
// Study for CPU and Browser WASM KV Caches", "CPU and WASM kernel design":
// append-time key kernel):
//   nu = ||x||;  y = T (x / nu);  idx_i = #{j : t_j < y_i}
//   keys:   e = y - c[idx], gamma = ||e||, z = [S e < 0]
//   pack the bit-planes into page block_table[slot][pos / 16], slot pos % 16,
//   and copy the last `window` tokens to the fp16 ring.
//
// Three kernels:
//  * append_tok_kernel (FWHT rotation, d = 64 or 128, appends of 32 or more
//    tokens per sequence): a lane per token, everything in registers; see the
//    comment above it.
//  * append_dense_kernel (dense rotation, d = 128 or 256): GEMMs of 64-token
//    tiles on the matrix cores; see the comment above it.
//  * append_kernel (d = 256 FWHT, dense d = 64, and short appends): two
//    64-lane wavefronts per (sequence, kv head, part), one for the keys and
//    one for the values; the part strides over the pages the sequence's new
//    tokens touch, so a page is only ever written by one workgroup in a call.
//    Lanes hold coordinates (lane l owns coordinates r*64 + l), so the
//    Walsh-Hadamard butterflies are cross-lane shuffles, the dense products
//    read rows of the transposed matrices, the norms are wavefront reductions,
//    and each key bit-plane row is one wavefront ballot.  Value bit-planes are
//    stored per coordinate (16 token bits), which each lane accumulates in
//    registers over the page's tokens and writes once.
#include "tq_device.h"

namespace tqi {
namespace {

constexpr float kZeroNorm = 1e-7f;

template <int D>
struct Codebooks {
  float kc[8], kt[7], vc[16], vt[15];
};

// x <- scale * M x for a wavefront-resident vector (lane l holds coordinates
// r*64 + l) and a d x d matrix given transposed (mt = M^T, row-major): lane l
// computes outputs R l .. R l + R - 1 from an R-wide slice of each row of M^T,
// so the wavefront's loads of one step are one contiguous row; x and the
// outputs pass through the wavefront's own LDS (no other wavefront touches it,
// and one wavefront's LDS accesses complete in order).
template <int D>
__device__ __forceinline__ void rotate_dense_t(float (&x)[D / 64], const float* mt, float* lds, int lane,
                                               float scale) {
  constexpr int R = D / 64;
  typedef float vecR __attribute__((ext_vector_type(R)));
#pragma unroll
  for (int r = 0; r < R; ++r) lds[r * 64 + lane] = x[r];
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  const vecR* col = reinterpret_cast<const vecR*>(mt) + lane;
  vecR acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = vecR{};
#pragma unroll 4
  for (int j = 0; j < D; j += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += col[size_t(j + u) * (D / R)] * lds[j + u];
  }
  const vecR o = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int k = 0; k < R; ++k) lds[R * lane + k] = o[k];
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = lds[r * 64 + lane] * scale;
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// The value of lane l ^ S (every lane active): DPP moves inside each row of
// 16 lanes below S = 16 (xor 4 = half-row mirror, then quad reversal; xor 8 =
// row mirror, then half-row mirror), the LDS crossbar at 16 and 32.  A chain
// of such exchanges (the transforms and sums of one token) then waits on the
// crossbar only for its last two steps.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int S>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (S == 1) return dpp_mov<0xB1>(v);
  else if constexpr (S == 2) return dpp_mov<0x4E>(v);
  else if constexpr (S == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(v));
  else if constexpr (S == 8) return dpp_mov<0x141>(dpp_mov<0x140>(v));
  else return __shfl_xor(v, S);
}
// sum over the wavefront, pairs combined in the order of wave_sum
__device__ __forceinline__ float wave_sum_x(float v) {
  v += lane_xor<32>(v);
  v += lane_xor<16>(v);
  v += lane_xor<8>(v);
  v += lane_xor<4>(v);
  v += lane_xor<2>(v);
  v += lane_xor<1>(v);
  return v;
}
// one butterfly stage of wave_fwht (half-width S across lanes)
template <int S, int R>
__device__ __forceinline__ void fwht_stage(float (&v)[R], int lane) {
  const bool upper = (lane & S) != 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float p = lane_xor<S>(v[r]);
    v[r] = upper ? (p - v[r]) : (v[r] + p);
  }
}
// wave_fwht with the exchanges above (the same butterflies in the same order)
template <int R>
__device__ __forceinline__ void wave_fwht_x(float (&v)[R], int lane) {
  fwht_stage<1>(v, lane);
  fwht_stage<2>(v, lane);
  fwht_stage<4>(v, lane);
  fwht_stage<8>(v, lane);
  fwht_stage<16>(v, lane);
  fwht_stage<32>(v, lane);
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

// FWHT rotation with the role's sign bits already in registers (as masks on
// the float sign bit): x <- scale * H D x.
template <int R>
__device__ __forceinline__ void fwht_rotate(float (&x)[R], const uint32_t (&sm)[R], int lane, float scale) {
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = __uint_as_float(__float_as_uint(x[r]) ^ sm[r]);
  wave_fwht_x<R>(x, lane);
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] *= scale;
}

__device__ __forceinline__ int quantize(float y, const float* t, int n_thr) {
  int idx = 0;
  for (int j = 0; j < n_thr; ++j) idx += (t[j] < y) ? 1 : 0;
  return idx;
}

// Two wavefronts per (sequence, kv head, part): wavefront 0 quantizes the keys
// (norm, rotation, codes, residual, QJL sketch, key words and norms, key ring
// rows), wavefront 1 the values (norm, rotation, codes, value words and norms,
// value ring rows), each over the same tokens; the two never wait for each
// other.
template <int D, int ROT>
__global__ __launch_bounds__(128) void append_kernel(AppendArgs a) {
  constexpr int R = D / 64;
  constexpr int P = 16;
  __shared__ float lds_all[2][D];
  const int lane = threadIdx.x & 63;
  const bool values = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)) != 0;  // this wavefront's role
  float* lds = lds_all[values ? 1 : 0];
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads;
  int unit = blockIdx.x;
  const int part = unit % a.parts;
  unit /= a.parts;
  const int h = unit % H;
  const int s = unit / H;
  if (s >= a.num_seqs) return;
  const int slot = a.seq_slots[s];
  if (slot < 0 || slot >= cv.max_seqs) {
    report(cv.status, true, TQ_STATUS_BAD_SLOT);
    return;
  }
  const int start = a.ctx_len_before[s];
  const int b0 = a.cu_new_tokens[s];
  const int n = a.cu_new_tokens[s + 1] - b0;
  if (n <= 0 || start < 0) return;
  const int new_len = start + n;
  const int W = cv.window;

  const int mk = a.key_mse_bits, bv = a.value_bits;
  const int nkt = (1 << mk) - 1, nvt = (1 << bv) - 1;
  // this role's codebook (keys: centroids and thresholds; values: thresholds)
  const float* kc = reinterpret_cast<const float*>(a.params + kOffKeyCentroids);
  const float* thr = reinterpret_cast<const float*>(a.params + (values ? kOffValueThresholds : kOffKeyThresholds));
  float kcr[8], tr[15];
#pragma unroll
  for (int j = 0; j < 8; ++j) kcr[j] = kc[j];
#pragma unroll
  for (int j = 0; j < 15; ++j) tr[j] = thr[j];
  const float rot_scale = (ROT == TQ_ROT_FWHT) ? rsqrtf(float(D)) : 1.0f;
  // FWHT variant: this role's sign bits, requested with the other parameters
  // rather than after the page stores (which the compiler cannot move them past)
  uint32_t sgn_a[R], sgn_b[R], sgn_c[R];
  if constexpr (ROT == TQ_ROT_FWHT) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sgn_a[r] = sign_bit(a.params, values ? kRoleValueRot : kRoleKeyRot, r * 64 + lane) << 31;
      sgn_b[r] = sign_bit(a.params, kRoleSketch1, r * 64 + lane) << 31;
      sgn_c[r] = sign_bit(a.params, kRoleSketch2, r * 64 + lane) << 31;
    }
  }
  const float* rot_t = reinterpret_cast<const float*>(a.params + dense_t_offset(D, values ? 3 : 0));
  const float* g_t = reinterpret_cast<const float*>(a.params + dense_t_offset(D, 2));
  const void* rows = values ? a.v_new : a.k_new;
  uint16_t* ring = values ? cv.v_window : cv.k_window;

  const size_t plane_bytes = size_t(P) * D / 8;
  for (int pg = start / P + part; pg * P < new_len; pg += a.parts) {
    if (pg >= cv.max_pages_per_seq) {
      report(cv.status, true, TQ_STATUS_CAPACITY);
      break;
    }
    const int phys = cv.block_table[size_t(slot) * cv.max_pages_per_seq + pg];
    const bool page_ok = phys >= 0 && phys < cv.num_pages;
    report(cv.status, !page_ok, TQ_STATUS_BAD_PAGE);
    const int lo = max(start, pg * P), hi = min(new_len, (pg + 1) * P);
    uint8_t* kb = cv.k_pages + (size_t(phys) * H + h) * cv.key_block;
    uint8_t* vb = cv.v_pages + (size_t(phys) * H + h) * cv.value_block;
    uint32_t vmask[4][R];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int r = 0; r < R; ++r) vmask[p][r] = 0;
    // value words of a page that already holds tokens: requested now, merged
    // after the last token (no other wavefront writes this page in this call)
    const uint32_t keep16 = (1u << (lo - pg * P)) - 1u;
    uint32_t old[4][R];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        old[p][r] = 0u;
        if (values && page_ok && keep16 != 0u && p < bv && !(lane & 1))
          old[p][r] = reinterpret_cast<const uint32_t*>(vb)[((r * 64 + lane) / 2) * bv + p];
      }

    for (int pos = lo; pos < hi; ++pos) {
      const size_t tok = size_t(b0) + (pos - start);
      const int t = pos - pg * P;
      const size_t base = (tok * H + h) * D;
      const bool in_window = W > 0 && pos >= new_len - W;
      float x[R], xin[R];
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) xin[r] = load_elem(rows, a.dtype, base + r * 64 + lane);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        x[r] = xin[r];
        ss = fmaf(x[r], x[r], ss);
      }
      ss = wave_sum_x(ss);
      const float nu = sqrtf(ss);
      const bool zero = !(nu >= kZeroNorm);
      const float inv = zero ? 0.f : 1.0f / nu;
      if constexpr (ROT == TQ_ROT_FWHT) fwht_rotate<R>(x, sgn_a, lane, rot_scale * inv);
      else rotate_dense_t<D>(x, rot_t, lds, lane, rot_scale * inv);
      if (!values) {
        // ---------------- key
        int idx[R];
        float e[R];
        float es = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          idx[r] = zero ? 0 : quantize(x[r], tr, nkt);
          float c = kcr[0];
#pragma unroll
          for (int j = 1; j < 8; ++j) c = (idx[r] == j) ? kcr[j] : c;
          e[r] = zero ? 0.f : x[r] - c;
          es = fmaf(e[r], e[r], es);
        }
        es = wave_sum_x(es);
        const float gamma = sqrtf(es);
        // QJL projection w = S e: FWHT variant S = H D2 H_n D1, dense variant S = G
        if constexpr (ROT == TQ_ROT_FWHT) {
          fwht_rotate<R>(e, sgn_b, lane, rsqrtf(float(D)));
          fwht_rotate<R>(e, sgn_c, lane, 1.0f);
        } else {
          rotate_dense_t<D>(e, g_t, lds, lane, 1.0f);
        }
        if (page_ok) {
          // token row: for each 32-coordinate group, the words of all planes
          uint32_t words[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) words[p] = 0;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            if (p > mk) break;
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const bool bit = (p < mk) ? (((idx[r] >> p) & 1) != 0) : (!zero && e[r] < 0.f);
              const uint64_t m = __ballot(bit);
              if ((lane >> 1) == r) words[p] = (lane & 1) ? uint32_t(m >> 32) : uint32_t(m);
            }
          }
          if (lane < D / 32) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(kb + size_t(t) * (D / 32) * (mk + 1) * 4) + lane * (mk + 1);
            for (int p = 0; p <= mk; ++p) dst[p] = words[p];
          }
          if (lane == 0) {
            float* norms = reinterpret_cast<float*>(kb + size_t(mk + 1) * plane_bytes) + 2 * t;
            norms[0] = zero ? 0.f : nu;
            norms[1] = zero ? 0.f : gamma;
          }
        }
      } else {
        // ---------------- value
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int vi = zero ? 0 : quantize(x[r], tr, nvt);
#pragma unroll
          for (int p = 0; p < 4; ++p) vmask[p][r] |= uint32_t((vi >> p) & 1) << t;
        }
        if (page_ok && lane == 0) {
          float* norms = reinterpret_cast<float*>(vb + size_t(bv) * plane_bytes);
          norms[t] = zero ? 0.f : nu;
        }
      }
      if (in_window) {
        uint16_t* rw = ring + ((size_t(slot) * H + h) * W + (pos % W)) * D;
#pragma unroll
        for (int r = 0; r < R; ++r) rw[r * 64 + lane] = float_to_f16_bits(xin[r]);
      }
    }
    if (values && page_ok) {
      // token bits below `lo` were written by earlier calls; keep them.  Value
      // words pair coordinates 2i (low half) and 2i + 1 (high half).
      const uint32_t keep = keep16 | (keep16 << 16);
      uint32_t* words = reinterpret_cast<uint32_t*>(vb);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p >= bv) break;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t mine = vmask[p][r];
          const uint32_t other = __shfl_xor(mine, 1);
          if (!(lane & 1)) {
            const int c = r * 64 + lane;
            words[(c / 2) * bv + p] = (old[p][r] & keep) | mine | (other << 16);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Token-per-lane append (FWHT rotation, d = 64 or 128).
//
// One wavefront takes 64 consecutive positions (four pages) of one
// (sequence, kv head); lane l owns position P0 + l and holds its whole head
// vector in registers, so the Walsh-Hadamard butterflies, the norms and the
// code decisions involve no other lane.  Instead of scaling d coordinates by
// 1 / (sqrt(d) nu), each lane scales its thresholds and centroids by
// sqrt(d) nu and works on z = H D x directly: y > t  <=>  z > t sqrt(d) nu,
// and the QJL signs of S e do not change under the positive factor.  Key
// bit-plane words are built by shifting the comparison bits in; value planes,
// stored per coordinate with the page's 16 token slots in a word, come from
// the comparisons' lane masks (one mask = 64 tokens of one coordinate),
// handed to the lane that stores that coordinate pair.
typedef const uint32_t __attribute__((address_space(4))) const_u32;
typedef const int32_t __attribute__((address_space(4))) const_i32;
typedef const float __attribute__((address_space(4))) const_f32;

template <int N>
__device__ __forceinline__ void fwht_regs(float (&x)[N]) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int i = 0; i < N; i += 2 * h)
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float u = x[j], v = x[j + h];
        x[j] = u + v;
        x[j + h] = u - v;
      }
}

// One exchange step of a 16 x 16 bit transpose over the 16 lanes of a row,
// done on both 16-bit halves of the word at once.  Lane l swaps, with lane
// l ^ S, the bits c of its half-words with (c & S) != (l & S): the lane with
// bit S clear keeps the bits with (c & S) == 0 and takes the partner's other
// bits moved down by S (a rotation), the other lane the converse.  Steps 8, 4,
// 2 and 1 together move bit c of lane l to bit l of lane c.
template <int S>
__device__ __forceinline__ uint32_t transpose16_step(uint32_t a, int lane) {
  constexpr uint32_t kHi = S == 8 ? 0xff00ff00u : S == 4 ? 0xf0f0f0f0u : S == 2 ? 0xccccccccu : 0xaaaaaaaau;
  // ds_swizzle in bit mode: partner = lane ^ S within each 32-lane half
  const uint32_t p = uint32_t(__builtin_amdgcn_ds_swizzle(int(a), 0x1f | (S << 10)));
  const bool hi = (lane & S) != 0;
  const uint32_t r = __builtin_amdgcn_alignbit(p, p, hi ? S : 32 - S);  // rotate right
  const uint32_t keep = hi ? kHi : ~kHi;
  return (a & keep) | (r & ~keep);
}

// Keeps the scheduler from moving work across phases (loads of the next phase
// hoisted over a long computation would hold its registers throughout).
__device__ __forceinline__ void phase() { __builtin_amdgcn_sched_barrier(0); }

// x <- D x for the sign vector of one role: bit c % 32 of word c / 32 set
// means -1.  The words are uniform (scalar loads), so each coordinate's sign
// mask is formed on the scalar unit and applied with one XOR of the float's
// sign bit -- bit for bit the product with -1.0 or +1.0, with no table and no
// registers held for it.
template <int N>
__device__ __forceinline__ void flip_signs(float (&x)[N], const const_u32* sw) {
  uint32_t w[N / 32];
#pragma unroll
  for (int q = 0; q < N / 32; ++q) w[q] = sw[q];
#pragma unroll
  for (int c = 0; c < N; ++c) {
    const uint32_t m = (w[c >> 5] << (31 - (c & 31))) & 0x80000000u;
    x[c] = __uint_as_float(__float_as_uint(x[c]) ^ m);
  }
}

// Row `row` of a [rows][N] input of the given dtype, as fp32.
template <int N>
__device__ __forceinline__ void load_row(const void* src, int dtype, size_t row, float (&x)[N]) {
  if (dtype == TQ_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + row * N);
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const float4 f = p[q];
      x[4 * q] = f.x; x[4 * q + 1] = f.y; x[4 * q + 2] = f.z; x[4 * q + 3] = f.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + row * N);
    uint32_t w[N / 2];
#pragma unroll
    for (int q = 0; q < N / 8; ++q) {
      const uint4 u = p[q];
      w[4 * q] = u.x; w[4 * q + 1] = u.y; w[4 * q + 2] = u.z; w[4 * q + 3] = u.w;
    }
    if (dtype == TQ_BF16) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        x[2 * i] = f16_bits_to_float(uint16_t(w[i] & 0xffffu));
        x[2 * i + 1] = f16_bits_to_float(uint16_t(w[i] >> 16));
      }
    }
  }
}

// fp16 copy of a row into the ring
template <int N>
__device__ __forceinline__ void store_f16_row(uint16_t* dst, const float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N / 8; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = uint32_t(float_to_f16_bits(x[8 * q + 2 * i])) | (uint32_t(float_to_f16_bits(x[8 * q + 2 * i + 1])) << 16);
    reinterpret_cast<uint4*>(dst)[q] = uint4{w[0], w[1], w[2], w[3]};
  }
}

// Codes of z for an odd codebook of L = 2^M levels, in sign-bit form.  The
// host builds the codebook odd (c[L-1-j] = -c[j]), so the fp32 thresholds are
// odd too and the middle one is 0: idx = #{t_j < z} has top bit [z > 0] and
// lower bits equal to the magnitude index m = #{tu_k < |z|} over the upper
// thresholds tu = t[L/2 .. L-2], complemented when z < 0 (up to ties, which
// sit inside any rounding band).  Every decision is kept as the sign bit of a
// float: bit j of m is the sign of d_j = tu_(...) - |z| (a binary search), the
// code's top bit is NOT sign(z), and its bit j < M-1 is sign(d_j) XOR sign(z).  Bits
// are shifted into words with v_alignbit and selections use masks built from
// sign bits, so no comparison result has to stay alive as a lane mask.
__device__ __forceinline__ uint32_t sign_mask(float d) { return uint32_t(int32_t(__float_as_uint(d)) >> 31); }
__device__ __forceinline__ float pick(uint32_t m, float if_set, float if_clear) {
  return __uint_as_float((__float_as_uint(if_set) & m) | (__float_as_uint(if_clear) & ~m));
}
// w <- (w << 1) | sign bit of v
__device__ __forceinline__ uint32_t shift_in_sign(uint32_t w, uint32_t v) { return __builtin_amdgcn_alignbit(w, v, 31); }

// d[j] for the magnitude bits j = 0 .. M-2 of |z| = a (entries >= M-1 unused)
template <int M>
__device__ __forceinline__ void magnitude_signs(float a, const float* tu, float (&d)[4]) {
  if constexpr (M == 2) {
    d[0] = tu[0] - a;
  } else if constexpr (M == 3) {
    d[1] = tu[1] - a;
    d[0] = pick(sign_mask(d[1]), tu[2], tu[0]) - a;
  } else if constexpr (M == 4) {
    d[2] = tu[3] - a;
    const uint32_t m2 = sign_mask(d[2]);
    d[1] = pick(m2, tu[5], tu[1]) - a;
    const uint32_t m1 = sign_mask(d[1]);
    d[0] = pick(m2, pick(m1, tu[6], tu[4]), pick(m1, tu[2], tu[0])) - a;
  }
}

// |c[idx]| from the magnitude bits (odd codebook: c[idx] = +-cu[m])
template <int M>
__device__ __forceinline__ float centroid_mag(const float* cu, const float (&d)[4]) {
  if constexpr (M == 1) {
    return cu[0];
  } else if constexpr (M == 2) {
    return pick(sign_mask(d[0]), cu[1], cu[0]);
  } else {
    const uint32_t m1 = sign_mask(d[1]), m0 = sign_mask(d[0]);
    return pick(m1, pick(m0, cu[3], cu[2]), pick(m0, cu[1], cu[0]));
  }
}

// Two wavefronts per SIMD: the kernel is bound by its ALU work, and a second
// wavefront hides the latencies of the butterfly chains (a head vector of
// d = 128 floats per lane fits in the 256 registers each then has).
template <int D, int MK, int BV>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void append_tok_kernel(AppendArgs a) {
  constexpr int P = 16, NG = D / 32;
  // upper thresholds and centroids of the odd codebooks (at least one entry)
  constexpr int NKT = (1 << (MK - 1)) - 1 > 0 ? (1 << (MK - 1)) - 1 : 1, NKC = 1 << (MK - 1);
  constexpr int NVT = (1 << (BV - 1)) - 1 > 0 ? (1 << (BV - 1)) - 1 : 1;
  constexpr int KWORDS = NG * (MK + 1);
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads, W = cv.window;
  int unit = blockIdx.x;
  const int chunk = unit % a.parts;
  unit /= a.parts;
  const int h = unit % H;
  const int s = unit / H;
  if (s >= a.num_seqs) return;
  const int slot = a.seq_slots[s];
  if (slot < 0 || slot >= cv.max_seqs) {
    report(cv.status, true, TQ_STATUS_BAD_SLOT);
    return;
  }
  const int start = a.ctx_len_before[s];
  const int b0 = a.cu_new_tokens[s];
  const int n = a.cu_new_tokens[s + 1] - b0;
  if (n <= 0 || start < 0) return;
  const int new_len = start + n;
  // chunks chunk, chunk + parts, ...: every 64-position chunk of the new
  // tokens is written whatever max_new_per_seq the launch was sized with
  for (int P0 = (start / 64 + chunk) * 64; P0 < new_len; P0 += a.parts * 64) {
    // lane-derived values are recomputed in every chunk (hoisted out of the
    // loop they would stay live in registers across the whole body)
    int lane = threadIdx.x;
    asm volatile("" : "+v"(lane));
    const int pos = P0 + lane;
    const bool valid = pos >= start && pos < new_len;
    const int g = lane >> 4, t = lane & 15;

    // the four pages of this chunk (uniform ids through the scalar cache)
    const const_i32* bt = (const const_i32*)(cv.block_table + size_t(slot) * cv.max_pages_per_seq);
    int phys[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pg = P0 / P + j;
      const int ph = pg < cv.max_pages_per_seq ? bt[pg] : -1;
      phys[j] = (ph >= 0 && ph < cv.num_pages) ? ph : -1;
      if (cv.status != nullptr && lane == 0 && pg * P < new_len && (pg + 1) * P > start && phys[j] < 0)
        report(cv.status, true, pg < cv.max_pages_per_seq ? TQ_STATUS_BAD_PAGE : TQ_STATUS_CAPACITY);
    }
    int my_phys = phys[0];
    my_phys = g == 1 ? phys[1] : my_phys;
    my_phys = g == 2 ? phys[2] : my_phys;
    my_phys = g == 3 ? phys[3] : my_phys;
    const bool page_ok = valid && my_phys >= 0;
    const bool in_window = valid && W > 0 && pos >= new_len - W;
    const size_t row = (size_t(b0) + (pos - start)) * H + h;

    // the parameters are re-addressed in every chunk: hoisting their loads out
    // of the chunk loop would hold them (dense: the matrix operands) in
    // registers across the whole body
    const uint8_t* params = a.params;
    asm volatile("" : "+s"(params));
    const const_f32* prm = (const const_f32*)params;
    // the four sign vectors (roles KR, KS1, KS2, VR), read through the scalar cache
    const const_u32* sgn_words = (const const_u32*)(params + kOffSigns);
    auto sgn = [&](int role) { return sgn_words + role * (kSignRoleBytes / 4); };
    const float sqd = sqrtf(float(D));
    const size_t plane_bytes = size_t(P) * D / 8;

    float x[D];
    // ------------------------------------------------------------------ key
    if (valid) {
      load_row<D>(a.k_new, a.dtype, row, x);
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) x[c] = 0.f;
    }
    if (in_window) store_f16_row<D>(cv.k_window + ((size_t(slot) * H + h) * W + (pos % W)) * D, x);
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) ss = fmaf(x[c], x[c], ss);
    const float nu = sqrtf(ss);
    const bool zero = !(nu >= kZeroNorm);
    const float kscale = zero ? 0.f : sqd * nu;
    float tk[NKT], ck[NKC];
#pragma unroll
    for (int j = 0; j < NKT; ++j) tk[j] = prm[kOffKeyThresholds / 4 + (1 << (MK - 1)) + j] * kscale;
#pragma unroll
    for (int j = 0; j < NKC; ++j) ck[j] = prm[kOffKeyCentroids / 4 + (1 << (MK - 1)) + j] * kscale;
    phase();
    flip_signs<D>(x, sgn(kRoleKeyRot));
    fwht_regs<D>(x);
    phase();
    // codes, residual e = z - c[idx] (in place), its norm
    uint32_t kw[MK + 1][NG];
    float es = 0.f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
#pragma unroll
      for (int p = 0; p <= MK; ++p) kw[p][gg] = 0u;
#pragma unroll
      for (int k = 31; k >= 0; --k) {
        const int c = 32 * gg + k;
        const float z = x[c];
        const uint32_t zb = __float_as_uint(z);
        float dm[4];
        magnitude_signs<MK>(fabsf(z), tk, dm);
        // sign(z) and sign(d_p) alone; the XOR and the inversion follow per word
        kw[MK - 1][gg] = shift_in_sign(kw[MK - 1][gg], zb);
#pragma unroll
        for (int p = 0; p + 1 < MK; ++p) kw[p][gg] = shift_in_sign(kw[p][gg], __float_as_uint(dm[p]));
        const float e = z - __builtin_copysignf(centroid_mag<MK>(ck, dm), z);
        x[c] = e;
        es = fmaf(e, e, es);
        // keep the words and the sum current here (the compiler would otherwise
        // defer them and hold every z and e alive)
#pragma unroll
        for (int p = 0; p < MK; ++p) asm volatile("" : "+v"(kw[p][gg]));
        asm volatile("" : "+v"(es));
      }
#pragma unroll
      for (int p = 0; p + 1 < MK; ++p) kw[p][gg] ^= kw[MK - 1][gg];
      kw[MK - 1][gg] = ~kw[MK - 1][gg];
    }
    const float gamma = sqrtf(es) * (zero ? 0.f : 1.f / kscale);
    phase();
    // QJL: z = [S e < 0] with S = H D2 H_n D1 (the positive factors drop out)
    flip_signs<D>(x, sgn(kRoleSketch1));
    fwht_regs<D>(x);
    flip_signs<D>(x, sgn(kRoleSketch2));
    fwht_regs<D>(x);
    phase();
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      uint32_t q = 0u;
#pragma unroll
      for (int k = 31; k >= 0; --k) {
        q = shift_in_sign(q, __float_as_uint(x[32 * gg + k]));
        asm volatile("" : "+v"(q));
      }
      kw[MK][gg] = zero ? 0u : q;
    }
    if (zero) {
#pragma unroll
      for (int p = 0; p < MK; ++p)
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) kw[p][gg] = 0u;
    }
    uint8_t* kb = page_ok ? cv.k_pages + (size_t(my_phys) * H + h) * cv.key_block : nullptr;
    if (page_ok) {
      // token row: for each 32-coordinate group, the words of all planes
      uint32_t wr[KWORDS];
#pragma unroll
      for (int gg = 0; gg < NG; ++gg)
#pragma unroll
        for (int p = 0; p <= MK; ++p) wr[gg * (MK + 1) + p] = kw[p][gg];
      uint32_t* dst = reinterpret_cast<uint32_t*>(kb + size_t(t) * KWORDS * 4);
      if constexpr (KWORDS % 4 == 0) {
#pragma unroll
        for (int q = 0; q < KWORDS / 4; ++q)
          reinterpret_cast<uint4*>(dst)[q] = uint4{wr[4 * q], wr[4 * q + 1], wr[4 * q + 2], wr[4 * q + 3]};
      } else {
#pragma unroll
        for (int q = 0; q < KWORDS / 2; ++q) reinterpret_cast<uint2*>(dst)[q] = uint2{wr[2 * q], wr[2 * q + 1]};
      }
      *reinterpret_cast<float2*>(kb + size_t(MK + 1) * plane_bytes + 8 * t) =
          make_float2(zero ? 0.f : nu, gamma);
    }

    // ------------------------------------------------------------------ value
    phase();
    if (valid) {
      load_row<D>(a.v_new, a.dtype, row, x);
    } else {
#pragma unroll
      for (int c = 0; c < D; ++c) x[c] = 0.f;
    }
    if (in_window) store_f16_row<D>(cv.v_window + ((size_t(slot) * H + h) * W + (pos % W)) * D, x);
    ss = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) ss = fmaf(x[c], x[c], ss);
    const float vnu = sqrtf(ss);
    const bool vzero = !(vnu >= kZeroNorm);
    const float vscale = vzero ? 0.f : sqd * vnu;
    float tv[NVT];
#pragma unroll
    for (int j = 0; j < NVT; ++j) tv[j] = prm[kOffValueThresholds / 4 + (1 << (BV - 1)) + j] * vscale;
    phase();
    flip_signs<D>(x, sgn(kRoleValueRot));
    fwht_regs<D>(x);
    phase();
    // Value bits in the page layout (per coordinate pair, the 16 token bits of
    // each coordinate) without ballots.  Each lane packs its own token's bits
    // of a 32-coordinate group into one word per plane, even coordinates in the
    // low half and odd ones in the high half: bit k of a half is coordinate pair
    // k.  The 16 lanes of a page then transpose both 16 x 16 bit matrices at
    // once (transpose16_step), after which lane t holds the word of coordinate
    // pair 16 w + t of group w: coordinate 2 i in the low half, 2 i + 1 in the
    // high half, token bits in lane order.  The top bit is NOT sign(z) and bit p
    // below it sign(d_p) XOR sign(z), formed on the words.
    const bool vbit_ok = valid && !vzero;
    uint32_t vw[BV][NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      uint32_t ev[BV], od[BV];
#pragma unroll
      for (int p = 0; p < BV; ++p) ev[p] = od[p] = 0u;
#pragma unroll
      for (int k = 15; k >= 0; --k) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          const float z = x[32 * gg + 2 * k + par];
          float dm[4];
          magnitude_signs<BV>(fabsf(z), tv, dm);
          uint32_t(&acc)[BV] = par ? od : ev;
          acc[BV - 1] = shift_in_sign(acc[BV - 1], __float_as_uint(z));
#pragma unroll
          for (int q = 0; q + 1 < BV; ++q) acc[q] = shift_in_sign(acc[q], __float_as_uint(dm[q]));
        }
      }
#pragma unroll
      for (int p = 0; p < BV; ++p) vw[p][gg] = (od[p] << 16) | ev[p];
#pragma unroll
      for (int p = 0; p + 1 < BV; ++p) vw[p][gg] ^= vw[BV - 1][gg];
      vw[BV - 1][gg] = ~vw[BV - 1][gg];
#pragma unroll
      for (int p = 0; p < BV; ++p) {
        uint32_t w = vbit_ok ? vw[p][gg] : 0u;
        w = transpose16_step<8>(w, lane);
        w = transpose16_step<4>(w, lane);
        w = transpose16_step<2>(w, lane);
        vw[p][gg] = transpose16_step<1>(w, lane);
      }
    }
    if (page_ok) *reinterpret_cast<float*>(cv.v_pages + (size_t(my_phys) * H + h) * cv.value_block +
                                           size_t(BV) * plane_bytes + 4 * t) = vzero ? 0.f : vnu;
    // lane t of page g stores the words of coordinate pairs 16 w + t of that page
    const int pg0 = (P0 / P + g) * P;
    const uint32_t keep16 = start > pg0 ? (start - pg0 >= P ? 0xffffu : (1u << (start - pg0)) - 1u) : 0u;
    if (my_phys >= 0 && pg0 < new_len && keep16 != 0xffffu) {  // the page holds a new token
      const uint32_t keep = keep16 | (keep16 << 16);
      uint32_t* base = reinterpret_cast<uint32_t*>(cv.v_pages + (size_t(my_phys) * H + h) * cv.value_block);
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        uint32_t* dst = base + (16 * gg + t) * BV;
        uint32_t wv[BV];
#pragma unroll
        for (int p = 0; p < BV; ++p) wv[p] = keep ? (dst[p] & keep) | vw[p][gg] : vw[p][gg];
        if constexpr (BV == 4) {
          *reinterpret_cast<uint4*>(dst) = uint4{wv[0], wv[1], wv[2], wv[3]};
        } else if constexpr (BV == 2) {
          *reinterpret_cast<uint2*>(dst) = uint2{wv[0], wv[1]};
        } else {
#pragma unroll
          for (int p = 0; p < BV; ++p) dst[p] = wv[p];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Dense-rotation append on the matrix cores (d = 128 or 256).
//
// One workgroup of four wavefronts takes 64 consecutive positions (four pages)
// of one (sequence, kv head).  The three products of the dense variant,
// y = Pi_K x / nu, the QJL projection w = G e and y_V = Pi_V v / nu_V, are
// GEMMs over the 64 tokens, out[n][t] = sum_k M[n][k] X[t][k], on
// v_mfma_f32_16x16x32_f16: A = rows of M (wavefront q owns the output
// coordinates q d/4 .. (q+1) d/4 - 1 and reads them from the fp16 split in the
// parameter blob, so every matrix entry is read once per tile), B = the token
// rows staged in LDS.  fp32 accuracy from fp16 operands: both sides are split
// hi + lo and hi*hi + hi*lo + lo*hi are accumulated in fp32 (the dropped lo*lo
// term is below 2^-22 of each product).  The matrix cores flush fp16
// subnormals, so the operands are scaled until only negligible lo pieces fall
// below 2^-14: token rows by 2^10 / nu and the rotations by 2^10, so the
// products are 2^20 y (thresholds and centroids scaled alike); the residual
// enters the sketch as 2^12 e and G as 2^8 G (signs only come out).
//
// One [64 tokens][d] LDS block holds in turn: the token rows as fp16 pieces
// ([8 hi][8 lo] per 8 coordinates), the fp32 products, the residuals as fp16
// pieces (each written over its own fp32 source), the fp32 projections, and
// the same for the values.  Between the GEMMs each wavefront takes a token per
// lane over its quarter of the coordinates and makes the same code decisions
// as the token-per-lane kernel.
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr float kRowScale = 1024.f;                 // token rows: 2^10 x / nu
constexpr float kOutScale = 1024.f * 1024.f;        // rotation products: 2^20 y
constexpr float kResidualScale = 1.f / 256.f;       // sketch operand: 2^12 e
template <int D>
struct DenseTile {
  static constexpr int T = 64;             // positions per workgroup
  static constexpr int ROWB = D * 4 + 16;  // bytes per LDS row, padded against bank conflicts
  static constexpr int Q = D / 4;          // coordinates per wavefront
  static constexpr int CT = Q / 16;        // 16-coordinate tiles per wavefront
  static constexpr int KS = D / 32;        // K steps of the GEMM
};

// out[n][t] for the wavefront's coordinates and all 64 tokens, accumulated in
// acc[ct][tt] (lane l, element i: coordinate q d/4 + 16 ct + 4 (l / 16) + i,
// token 16 tt + l % 16).  A and B place K index 32 ks + 8 g + e at element e of
// lane group g, so the pairing holds whatever the instruction's K order.
// The matrix pieces are read through global-address-space pointers: a
// uniform base plus a 32-bit lane offset and immediate offsets per K step, so
// no 64-bit address arithmetic and no flat accesses (which would also count
// against the LDS reads' waits).
typedef const h8v __attribute__((address_space(1))) g_h8v;
typedef const uint8_t __attribute__((address_space(1))) g_u8;
// ONE: only 16-token tile tt0 holds new tokens (short appends), so only its
// products are formed; the other tiles' outputs are zero.
template <int D, bool ONE = false>
__device__ __forceinline__ void dense_gemm(const _Float16* mhi, const _Float16* mlo, const uint8_t* buf, int q,
                                           int lane, f4v (&acc)[DenseTile<D>::CT][4], int tt0 = 0) {
  using DT = DenseTile<D>;
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < DT::CT; ++ct)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[ct][tt] = f4v{0.f, 0.f, 0.f, 0.f};
  if constexpr (ONE) {
    f4v a1[DT::CT];
#pragma unroll
    for (int ct = 0; ct < DT::CT; ++ct) a1[ct] = f4v{0.f, 0.f, 0.f, 0.f};
    const g_u8* ghi = (const g_u8*)mhi;
    const g_u8* glo = (const g_u8*)mlo;
    const uint32_t lane_off = uint32_t(((q * DT::Q + r16) * D + 8 * g) * 2);
    const uint8_t* brow = buf + (16 * tt0 + r16) * DT::ROWB;
    // the matrix pieces of NB K steps in flight: each step's slot is refilled
    // with step ks + NB once its products are issued (the scheduling barriers
    // keep the compiler from moving the loads next to their first use, which
    // would wait out one memory round trip per K step)
    constexpr int NB = DT::KS < 3 ? DT::KS : 3;
    h8v ah[NB][DT::CT], al[NB][DT::CT];
    auto load_a = [&](int ks) {
#pragma unroll
      for (int ct = 0; ct < DT::CT; ++ct) {
        const uint32_t off = lane_off + uint32_t((16 * ct * D + 32 * ks) * 2);
        ah[ks % NB][ct] = *reinterpret_cast<g_h8v*>(ghi + off);
        al[ks % NB][ct] = *reinterpret_cast<g_h8v*>(glo + off);
      }
    };
#pragma unroll
    for (int ks = 0; ks < NB; ++ks) load_a(ks);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < DT::KS; ++ks) {
      const h8v bh = *reinterpret_cast<const h8v*>(brow + (4 * ks + g) * 32);
      const h8v bl = *reinterpret_cast<const h8v*>(brow + (4 * ks + g) * 32 + 16);
#pragma unroll
      for (int ct = 0; ct < DT::CT; ++ct) {
        a1[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks % NB][ct], bh, a1[ct], 0, 0, 0);
        a1[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks % NB][ct], bl, a1[ct], 0, 0, 0);
        a1[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[ks % NB][ct], bh, a1[ct], 0, 0, 0);
      }
      if (ks + NB < DT::KS) load_a(ks + NB);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ct = 0; ct < DT::CT; ++ct)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        if (tt == tt0) acc[ct][tt] = a1[ct];
    return;
  }
  h8v ah[2][DT::CT], al[2][DT::CT];
  const g_u8* ghi = (const g_u8*)mhi;
  const g_u8* glo = (const g_u8*)mlo;
  const uint32_t lane_off = uint32_t(((q * DT::Q + r16) * D + 8 * g) * 2);
  auto load_a = [&](int ks, int slot) {
#pragma unroll
    for (int ct = 0; ct < DT::CT; ++ct) {
      const uint32_t off = lane_off + uint32_t((16 * ct * D + 32 * ks) * 2);
      ah[slot][ct] = *reinterpret_cast<g_h8v*>(ghi + off);
      al[slot][ct] = *reinterpret_cast<g_h8v*>(glo + off);
    }
  };
  load_a(0, 0);
#pragma unroll
  for (int ks = 0; ks < DT::KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < DT::KS) load_a(ks + 1, cur ^ 1);
    h8v bh[4], bl[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint8_t* p = buf + (16 * tt + r16) * DT::ROWB + (4 * ks + g) * 32;
      bh[tt] = *reinterpret_cast<const h8v*>(p);
      bl[tt] = *reinterpret_cast<const h8v*>(p + 16);
    }
#pragma unroll
    for (int ct = 0; ct < DT::CT; ++ct)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[cur][ct], bh[tt], acc[ct][tt], 0, 0, 0);
        acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[cur][ct], bl[tt], acc[ct][tt], 0, 0, 0);
        acc[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[cur][ct], bh[tt], acc[ct][tt], 0, 0, 0);
      }
  }
}

// The products as fp32 rows [token][coordinate] of the LDS block.
template <int D>
__device__ __forceinline__ void dense_store(const f4v (&acc)[DenseTile<D>::CT][4], uint8_t* buf, int q, int lane) {
  using DT = DenseTile<D>;
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < DT::CT; ++ct)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      *reinterpret_cast<f4v*>(buf + (16 * tt + r16) * DT::ROWB + (q * DT::Q + 16 * ct + 4 * g) * 4) = acc[ct][tt];
}

// 8 values as fp16 pieces [8 hi][8 lo] at p (32 bytes).  Each value is pinned
// as the fp32 number it is first: otherwise the product that produced it can
// be contracted into the lo computation, whose hi would then be rounded from
// the exact product while the stored hi is rounded from the fp32 one.
__device__ __forceinline__ void store_pieces(uint8_t* p, const float (&v)[8]) {
#pragma clang fp contract(off)
  h8v hi, lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = v[e];
    asm volatile("" : "+v"(x));
    hi[e] = _Float16(x);
    lo[e] = _Float16(x - float(hi[e]));
  }
  *reinterpret_cast<h8v*>(p) = hi;
  *reinterpret_cast<h8v*>(p + 16) = lo;
}

__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// SHORT (appends of at most 16 tokens per sequence, such as decode steps):
// a chunk whose new tokens fall in one 16-token tile forms only that tile's
// products.  (A separate instantiation: the extra path in the long-append
// kernel cost it 3%.)
template <int D, int MK, int BV, bool SHORT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void append_dense_kernel(AppendArgs a) {
  using DT = DenseTile<D>;
  constexpr int P = 16, T = DT::T, Q = DT::Q, LPT = D / 8, TPP = 64 / LPT;
  constexpr int NKT = (1 << (MK - 1)) - 1 > 0 ? (1 << (MK - 1)) - 1 : 1, NKC = 1 << (MK - 1);
  constexpr int NVT = (1 << (BV - 1)) - 1 > 0 ? (1 << (BV - 1)) - 1 : 1;
  constexpr int NGQ = Q / 32;            // 32-coordinate key groups per wavefront
  constexpr int KWORDS = (D / 32) * (MK + 1);
  __shared__ __attribute__((aligned(16))) uint8_t buf[T * DT::ROWB];
  __shared__ float nrm[T], esum[4][T];
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads, W = cv.window;
  int unit = blockIdx.x;
  const int chunk = unit % a.parts;
  unit /= a.parts;
  const int h = unit % H;
  const int s = unit / H;
  if (s >= a.num_seqs) return;
  const int slot = a.seq_slots[s];
  if (slot < 0 || slot >= cv.max_seqs) {
    report(cv.status, true, TQ_STATUS_BAD_SLOT);
    return;
  }
  const int start = a.ctx_len_before[s];
  const int b0 = a.cu_new_tokens[s];
  const int n = a.cu_new_tokens[s + 1] - b0;
  if (n <= 0 || start < 0) return;
  const int new_len = start + n;
  // chunks chunk, chunk + parts, ... (uniform per workgroup): every chunk of
  // the new tokens is written whatever max_new_per_seq the launch was sized with
  for (int P0 = (start / T + chunk) * T; P0 < new_len; P0 += a.parts * T) {
    // thread-derived values are recomputed in every chunk (hoisted out of the
    // loop they would stay live in registers across the whole body)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, q = tid >> 6;
    const const_i32* bt = (const const_i32*)(cv.block_table + size_t(slot) * cv.max_pages_per_seq);
    int phys[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pg = P0 / P + j;
      const int ph = pg < cv.max_pages_per_seq ? bt[pg] : -1;
      phys[j] = (ph >= 0 && ph < cv.num_pages) ? ph : -1;
      if (cv.status != nullptr && lane == 0 && pg * P < new_len && (pg + 1) * P > start && phys[j] < 0)
        report(cv.status, true, pg < cv.max_pages_per_seq ? TQ_STATUS_BAD_PAGE : TQ_STATUS_CAPACITY);
    }
    // the parameters are re-addressed in every chunk: hoisting their loads out
    // of the chunk loop would hold them (dense: the matrix operands) in
    // registers across the whole body
    const uint8_t* params = a.params;
    asm volatile("" : "+s"(params));
    const const_f32* prm = (const const_f32*)params;
    const _Float16* m16 = reinterpret_cast<const _Float16*>(params + dense16_offset(D, 0));
    const size_t mm = size_t(D) * D;  // halves per fp16 matrix
    const size_t plane_bytes = size_t(P) * D / 8;

    // token rows [P0, P0 + 64) of src into the LDS block as fp16 pieces of
    // 2^10 x / nu; norms to nrm (0 outside [start, new_len)); fp16 ring copies of
    // window rows.  Wavefront q stages tokens 16 q .. 16 q + 15, LPT lanes per row.
    auto stage = [&](const void* src, uint16_t* ring) {
      constexpr int NP = 16 / TPP;  // passes
      // every pass's 8 elements first (one uniform dtype branch), so that the
      // loads are in flight together
      uint32_t raw[NP][8];
#pragma unroll
      for (int pass = 0; pass < NP; ++pass) {
        const int t = 16 * q + pass * TPP + lane / LPT, sub = lane % LPT;
        const int pos = P0 + t;
        const size_t e0 = ((size_t(b0) + (pos - start)) * H + h) * D + 8 * sub;
        const bool valid = pos >= start && pos < new_len;
        if (a.dtype == TQ_F32) {
          const uint4* p4 = reinterpret_cast<const uint4*>(static_cast<const float*>(src) + e0);
          const uint4 u = valid ? p4[0] : uint4{0u, 0u, 0u, 0u}, v = valid ? p4[1] : uint4{0u, 0u, 0u, 0u};
          raw[pass][0] = u.x; raw[pass][1] = u.y; raw[pass][2] = u.z; raw[pass][3] = u.w;
          raw[pass][4] = v.x; raw[pass][5] = v.y; raw[pass][6] = v.z; raw[pass][7] = v.w;
        } else {
          const uint4 u = valid ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + e0)
                                : uint4{0u, 0u, 0u, 0u};
          raw[pass][0] = u.x; raw[pass][1] = u.y; raw[pass][2] = u.z; raw[pass][3] = u.w;
        }
      }
#pragma unroll
      for (int pass = 0; pass < NP; ++pass) {
        const int t = 16 * q + pass * TPP + lane / LPT, sub = lane % LPT;
        const int pos = P0 + t;
        const bool valid = pos >= start && pos < new_len;
        float x[8];
        if (a.dtype == TQ_F32) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(raw[pass][e]);
        } else if (a.dtype == TQ_BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(raw[pass][i] << 16);
            x[2 * i + 1] = __uint_as_float(raw[pass][i] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[2 * i] = f16_bits_to_float(uint16_t(raw[pass][i] & 0xffffu));
            x[2 * i + 1] = f16_bits_to_float(uint16_t(raw[pass][i] >> 16));
          }
        }
        if (valid && W > 0 && pos >= new_len - W) {
          uint32_t w4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w4[i] = uint32_t(float_to_f16_bits(x[2 * i])) | (uint32_t(float_to_f16_bits(x[2 * i + 1])) << 16);
          *reinterpret_cast<uint4*>(ring + ((size_t(slot) * H + h) * W + (pos % W)) * D + 8 * sub) =
              uint4{w4[0], w4[1], w4[2], w4[3]};
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
        for (int o = 1; o < LPT; o <<= 1) ss += __shfl_xor(ss, o);
        const float nu = sqrtf(ss);
        const float sc = nu >= kZeroNorm ? kRowScale / nu : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= sc;
        store_pieces(buf + t * DT::ROWB + 32 * sub, x);
        if (sub == 0) nrm[t] = valid && nu >= kZeroNorm ? nu : 0.f;
      }
    };
    // SHORT: the 16-token tiles of this chunk that hold new tokens
    const int tt_first = max(start - P0, 0) / 16, tt_last = (min(new_len - P0, T) - 1) / 16;
    auto gemm_to_rows = [&](int m) {
      f4v acc[DT::CT][4];
      block_barrier();  // rows staged
      if (SHORT && tt_first == tt_last)
        dense_gemm<D, SHORT>(m16 + size_t(m) * 2 * mm, m16 + size_t(m) * 2 * mm + mm, buf, q, lane, acc, tt_first);
      else
        dense_gemm<D>(m16 + size_t(m) * 2 * mm, m16 + size_t(m) * 2 * mm + mm, buf, q, lane, acc);
      block_barrier();  // every wavefront has read the rows
      dense_store<D>(acc, buf, q, lane);
      block_barrier();  // products visible
    };
    // this lane's token, 32 coordinates of this wavefront's quarter
    float z[32];
    auto read_group = [&](int gg) {
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const float4 v = *reinterpret_cast<const float4*>(buf + lane * DT::ROWB + (q * Q + 32 * gg + c) * 4);
        z[c] = v.x; z[c + 1] = v.y; z[c + 2] = v.z; z[c + 3] = v.w;
      }
    };

    const int t = lane, pos = P0 + t;
    const bool valid = pos >= start && pos < new_len;
    const int pj = t >> 4, ts = t & 15;
    const bool page_ok = valid && phys[pj] >= 0;

    // ------------------------------------------------------------------ key
    stage(a.k_new, cv.k_window);
    gemm_to_rows(0);
    const float nu = nrm[t];
    const bool zero = !(nu > 0.f);
    float tk[NKT], ck[NKC];
#pragma unroll
    for (int j = 0; j < NKT; ++j) tk[j] = prm[kOffKeyThresholds / 4 + (1 << (MK - 1)) + j] * kOutScale;
#pragma unroll
    for (int j = 0; j < NKC; ++j) ck[j] = prm[kOffKeyCentroids / 4 + (1 << (MK - 1)) + j] * kOutScale;
    uint32_t kw[MK + 1][NGQ];
    float es = 0.f;
#pragma unroll
    for (int gg = 0; gg < NGQ; ++gg) {
      read_group(gg);
#pragma unroll
      for (int p = 0; p <= MK; ++p) kw[p][gg] = 0u;
#pragma unroll
      for (int k = 31; k >= 0; --k) {
        const int c = k;
        const float zz = z[c];
        const uint32_t zb = __float_as_uint(zz);
        float dm[4];
        magnitude_signs<MK>(fabsf(zz), tk, dm);
        // sign(z) and sign(d_p) alone; the XOR and the inversion follow per word
        kw[MK - 1][gg] = shift_in_sign(kw[MK - 1][gg], zb);
#pragma unroll
        for (int p = 0; p + 1 < MK; ++p) kw[p][gg] = shift_in_sign(kw[p][gg], __float_as_uint(dm[p]));
        const float e = zz - __builtin_copysignf(centroid_mag<MK>(ck, dm), zz);
        z[c] = e;
        es = fmaf(e, e, es);
        // keep the words and the sum current (deferred, every decision would stay live)
#pragma unroll
        for (int p = 0; p < MK; ++p) asm volatile("" : "+v"(kw[p][gg]));
        asm volatile("" : "+v"(es));
        if ((k & 7) == 0) {  // the 8 residuals of this block (as 2^12 e), over their fp32 source
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = z[c + i] * kResidualScale;
          store_pieces(buf + t * DT::ROWB + (q * Q + 32 * gg + c) * 4, v);
        }
      }
#pragma unroll
      for (int p = 0; p + 1 < MK; ++p) kw[p][gg] ^= kw[MK - 1][gg];
      kw[MK - 1][gg] = ~kw[MK - 1][gg];
    }
    esum[q][t] = es;
    // QJL: signs of w = G e
    gemm_to_rows(1);
#pragma unroll
    for (int gg = 0; gg < NGQ; ++gg) {
      read_group(gg);
      uint32_t qb = 0u;
#pragma unroll
      for (int k = 31; k >= 0; --k) qb = shift_in_sign(qb, __float_as_uint(z[k]));
      kw[MK][gg] = qb;
    }
    if (page_ok) {
      uint8_t* kb = cv.k_pages + (size_t(phys[pj]) * H + h) * cv.key_block;
      uint32_t* dst = reinterpret_cast<uint32_t*>(kb + size_t(ts) * KWORDS * 4) + q * NGQ * (MK + 1);
#pragma unroll
      for (int gg = 0; gg < NGQ; ++gg)
#pragma unroll
        for (int p = 0; p <= MK; ++p) dst[gg * (MK + 1) + p] = zero ? 0u : kw[p][gg];
      if (q == 0) {
        const float gamma = zero ? 0.f : sqrtf(esum[0][t] + esum[1][t] + esum[2][t] + esum[3][t]) * (1.f / kOutScale);
        *reinterpret_cast<float2*>(kb + size_t(MK + 1) * plane_bytes + 8 * ts) = make_float2(zero ? 0.f : nu, gamma);
      }
    }
    block_barrier();  // key products consumed, norms read

    // ------------------------------------------------------------------ value
    stage(a.v_new, cv.v_window);
    gemm_to_rows(2);
    const float vnu = nrm[t];
    const bool vbit_ok = valid && vnu > 0.f;
    float tv[NVT];
#pragma unroll
    for (int j = 0; j < NVT; ++j) tv[j] = prm[kOffValueThresholds / 4 + (1 << (BV - 1)) + j] * kOutScale;
    // value bits packed per lane and transposed across each page's 16 lanes, as
    // in the token-per-lane kernel: after the transpose, lane ts of page pj
    // holds the word of coordinate pair q Q / 2 + 16 gg + ts of that page
    uint32_t vw[BV][NGQ];
#pragma unroll
    for (int gg = 0; gg < NGQ; ++gg) {
      read_group(gg);
      uint32_t ev[BV], od[BV];
#pragma unroll
      for (int p = 0; p < BV; ++p) ev[p] = od[p] = 0u;
#pragma unroll
      for (int k = 15; k >= 0; --k) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
          const float zz = z[2 * k + par];
          float dm[4];
          magnitude_signs<BV>(fabsf(zz), tv, dm);
          uint32_t(&acc)[BV] = par ? od : ev;
          acc[BV - 1] = shift_in_sign(acc[BV - 1], __float_as_uint(zz));
#pragma unroll
          for (int r = 0; r + 1 < BV; ++r) acc[r] = shift_in_sign(acc[r], __float_as_uint(dm[r]));
        }
      }
#pragma unroll
      for (int p = 0; p < BV; ++p) vw[p][gg] = (od[p] << 16) | ev[p];
#pragma unroll
      for (int p = 0; p + 1 < BV; ++p) vw[p][gg] ^= vw[BV - 1][gg];
      vw[BV - 1][gg] = ~vw[BV - 1][gg];
#pragma unroll
      for (int p = 0; p < BV; ++p) {
        uint32_t w = vbit_ok ? vw[p][gg] : 0u;
        w = transpose16_step<8>(w, lane);
        w = transpose16_step<4>(w, lane);
        w = transpose16_step<2>(w, lane);
        vw[p][gg] = transpose16_step<1>(w, lane);
      }
    }
    if (page_ok && q == 0)
      *reinterpret_cast<float*>(cv.v_pages + (size_t(phys[pj]) * H + h) * cv.value_block + size_t(BV) * plane_bytes +
                                4 * ts) = vbit_ok ? vnu : 0.f;
    const int pg0 = (P0 / P + pj) * P;
    const uint32_t keep16 = start > pg0 ? (start - pg0 >= P ? 0xffffu : (1u << (start - pg0)) - 1u) : 0u;
    if (phys[pj] >= 0 && pg0 < new_len && keep16 != 0xffffu) {  // the page holds a new token
      const uint32_t keep = keep16 | (keep16 << 16);
      uint32_t* base = reinterpret_cast<uint32_t*>(cv.v_pages + (size_t(phys[pj]) * H + h) * cv.value_block);
#pragma unroll
      for (int gg = 0; gg < NGQ; ++gg) {
        uint32_t* dst = base + (q * Q / 2 + 16 * gg + ts) * BV;
#pragma unroll
        for (int p = 0; p < BV; ++p) dst[p] = keep ? (dst[p] & keep) | vw[p][gg] : vw[p][gg];
      }
    }
    block_barrier();  // LDS rows and norms are rewritten by the next chunk
  }
}

template <int D, int MK>
hipError_t launch_dense_bv(const AppendArgs& a, int units, hipStream_t st, bool short_append) {
#define TQ_DENSE(BV_)                                                                                   \
  case BV_:                                                                                             \
    if (short_append) hipLaunchKernelGGL((append_dense_kernel<D, MK, BV_, true>), dim3(units), dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((append_dense_kernel<D, MK, BV_, false>), dim3(units), dim3(256), 0, st, a); \
    break;
  switch (a.value_bits) {
    TQ_DENSE(1) TQ_DENSE(2) TQ_DENSE(3) TQ_DENSE(4)
    default: return hipErrorInvalidValue;
  }
#undef TQ_DENSE
  return hipGetLastError();
}

// appends of at most this many tokens per sequence take the SHORT kernel
constexpr int kDenseShortMaxNew = 16;

template <int D>
hipError_t launch_dense(const AppendArgs& a, int units, hipStream_t st, int max_new) {
  const bool short_append = max_new <= kDenseShortMaxNew;
  switch (a.key_mse_bits) {
    case 1: return launch_dense_bv<D, 1>(a, units, st, short_append);
    case 2: return launch_dense_bv<D, 2>(a, units, st, short_append);
    case 3: return launch_dense_bv<D, 3>(a, units, st, short_append);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int MK>
hipError_t launch_tok_bv(const AppendArgs& a, int units, hipStream_t st) {
  switch (a.value_bits) {
    case 1: hipLaunchKernelGGL((append_tok_kernel<D, MK, 1>), dim3(units), dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((append_tok_kernel<D, MK, 2>), dim3(units), dim3(64), 0, st, a); break;
    case 3: hipLaunchKernelGGL((append_tok_kernel<D, MK, 3>), dim3(units), dim3(64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((append_tok_kernel<D, MK, 4>), dim3(units), dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_tok(const AppendArgs& a, int units, hipStream_t st) {
  switch (a.key_mse_bits) {
    case 1: return launch_tok_bv<D, 1>(a, units, st);
    case 2: return launch_tok_bv<D, 2>(a, units, st);
    case 3: return launch_tok_bv<D, 3>(a, units, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int ROT>
hipError_t launch(const AppendArgs& a, int units, hipStream_t st) {
  hipLaunchKernelGGL((append_kernel<D, ROT>), dim3(units), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// Below this many new tokens per sequence (decode-time appends) a wavefront
// per token has the shorter latency: one lane would otherwise do a whole head
// vector alone while the other 63 idle.
constexpr int kTokenLaneMinNew = 32;
// Dense rotation: the matrix-core kernel at any append size.  A single token's
// 64-token tile (38 us at head_dim 256) still beats the wavefront-per-token
// kernel, whose one wavefront per role streams each d x d matrix with only a
// few row loads in flight (137 us for a one-token-per-sequence step at
// head_dim 256, with coalesced rows of the transposed matrices).
constexpr int kDenseMatrixMinNew = 1;

int launch_append(const tq_config& cfg, const AppendArgs& args, int num_seqs, int max_new, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool dense = cfg.rotation == TQ_ROT_DENSE;
  AppendArgs a = args;
  const long long H = cfg.num_kv_heads;
  if (dense && (cfg.head_dim == 128 || cfg.head_dim == 256) && max_new >= kDenseMatrixMinNew) {
    // matrix-core kernel: one workgroup per 64-position chunk a sequence's new tokens touch
    a.parts = (max_new + 63) / 64 + 1;
    const long long units = (long long)num_seqs * H * a.parts;
    if (units > 0x7fffffffLL) return hipErrorInvalidValue;
    return cfg.head_dim == 128 ? launch_dense<128>(a, int(units), st, max_new)
                               : launch_dense<256>(a, int(units), st, max_new);
  }
  if (!dense && (cfg.head_dim == 64 || cfg.head_dim == 128) && max_new >= kTokenLaneMinNew) {
    // token-per-lane kernel: one wavefront per 64-position chunk a sequence's new tokens touch
    a.parts = (max_new + 63) / 64 + 1;
    const long long units = (long long)num_seqs * H * a.parts;
    if (units > 0x7fffffffLL) return hipErrorInvalidValue;
    return cfg.head_dim == 64 ? launch_tok<64>(a, int(units), st) : launch_tok<128>(a, int(units), st);
  }
  // wavefront-per-token kernel: one wavefront per page, capped for huge prefills
  int parts = (max_new + cfg.page_tokens - 1) / cfg.page_tokens + 1;
  if (parts > 4096) parts = 4096;
  a.parts = parts;
  const long long units = (long long)num_seqs * H * parts;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (cfg.head_dim) {
    case 64: return dense ? launch<64, TQ_ROT_DENSE>(a, int(units), st) : launch<64, TQ_ROT_FWHT>(a, int(units), st);
    case 128: return dense ? launch<128, TQ_ROT_DENSE>(a, int(units), st) : launch<128, TQ_ROT_FWHT>(a, int(units), st);
    case 256: return dense ? launch<256, TQ_ROT_DENSE>(a, int(units), st) : launch<256, TQ_ROT_FWHT>(a, int(units), st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqi
