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
// Work decomposition: one 64-lane wavefront per (sequence, kv head, part);
// the part strides over the pages the sequence's new tokens touch, so a page
// is only ever written by one wavefront in a call.  Lanes hold coordinates
// (lane l owns coordinates r*64 + l), so the Walsh-Hadamard butterflies are
// cross-lane shuffles, the norms are wavefront reductions, and each key
// bit-plane row is one wavefront ballot.  Value bit-planes are stored per
// coordinate (16 token bits), which each lane accumulates in registers over
// the page's tokens and writes once.
#include "tq_device.h"

namespace tqi {
namespace {

constexpr float kZeroNorm = 1e-7f;

template <int D>
struct Codebooks {
  float kc[8], kt[7], vc[16], vt[15];
};

// Rotation of a wavefront-resident vector: FWHT variant y = H D x * scale,
// dense variant y = M x * scale (M row-major d x d in global memory, x staged
// through LDS).
template <int D, int ROT>
__device__ __forceinline__ void rotate(float (&x)[D / 64], const uint8_t* params, int role,
                                       const float* dense, float* lds, int lane, float scale) {
  constexpr int R = D / 64;
  if (ROT == TQ_ROT_FWHT) {
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = apply_sign(x[r], sign_bit(params, role, r * 64 + lane));
    wave_fwht<R>(x, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] *= scale;
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) lds[r * 64 + lane] = x[r];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float* row = dense + size_t(r * 64 + lane) * D;
      float acc = 0.f;
      for (int j = 0; j < D; j += 4) {
        const float4 m = *reinterpret_cast<const float4*>(row + j);
        acc = fmaf(m.x, lds[j], acc);
        acc = fmaf(m.y, lds[j + 1], acc);
        acc = fmaf(m.z, lds[j + 2], acc);
        acc = fmaf(m.w, lds[j + 3], acc);
      }
      x[r] = acc * scale;
    }
    __syncthreads();
  }
}

// QJL projection w = S e: FWHT variant S = H D2 H_n D1, dense variant S = G.
template <int D, int ROT>
__device__ __forceinline__ void sketch(float (&e)[D / 64], const uint8_t* params, float* lds, int lane) {
  constexpr int R = D / 64;
  if (ROT == TQ_ROT_FWHT) {
    rotate<D, ROT>(e, params, kRoleSketch1, nullptr, lds, lane, rsqrtf(float(D)));
    rotate<D, ROT>(e, params, kRoleSketch2, nullptr, lds, lane, 1.0f);
  } else {
    const float* g = reinterpret_cast<const float*>(params + kOffDense) + size_t(D) * D;
    rotate<D, ROT>(e, params, 0, g, lds, lane, 1.0f);
  }
  (void)R;
}

__device__ __forceinline__ int quantize(float y, const float* t, int n_thr) {
  int idx = 0;
  for (int j = 0; j < n_thr; ++j) idx += (t[j] < y) ? 1 : 0;
  return idx;
}

template <int D, int ROT>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  constexpr int R = D / 64;
  constexpr int P = 16;
  __shared__ float lds[D];
  const int lane = threadIdx.x;
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads;
  int unit = blockIdx.x;
  const int part = unit % a.parts;
  unit /= a.parts;
  const int h = unit % H;
  const int s = unit / H;
  if (s >= a.num_seqs) return;
  const int slot = a.seq_slots[s];
  if (slot < 0 || slot >= cv.max_seqs) return;
  const int start = a.ctx_len_before[s];
  const int b0 = a.cu_new_tokens[s];
  const int n = a.cu_new_tokens[s + 1] - b0;
  if (n <= 0 || start < 0) return;
  const int new_len = start + n;
  const int W = cv.window;

  const int mk = a.key_mse_bits, bv = a.value_bits;
  const int nkt = (1 << mk) - 1, nvt = (1 << bv) - 1;
  const float* kc = reinterpret_cast<const float*>(a.params + kOffKeyCentroids);
  const float* kt = reinterpret_cast<const float*>(a.params + kOffKeyThresholds);
  const float* vt = reinterpret_cast<const float*>(a.params + kOffValueThresholds);
  float kcr[8], ktr[7], vtr[15];
#pragma unroll
  for (int j = 0; j < 8; ++j) kcr[j] = kc[j];
#pragma unroll
  for (int j = 0; j < 7; ++j) ktr[j] = kt[j];
#pragma unroll
  for (int j = 0; j < 15; ++j) vtr[j] = vt[j];
  const float* pik = reinterpret_cast<const float*>(a.params + kOffDense);
  const float* piv = pik + size_t(2) * D * D;
  const float rot_scale = (ROT == TQ_ROT_FWHT) ? rsqrtf(float(D)) : 1.0f;

  const size_t plane_bytes = size_t(P) * D / 8;
  for (int pg = start / P + part; pg * P < new_len; pg += a.parts) {
    if (pg >= cv.max_pages_per_seq) break;
    const int phys = cv.block_table[size_t(slot) * cv.max_pages_per_seq + pg];
    const bool page_ok = phys >= 0 && phys < cv.num_pages;
    const int lo = max(start, pg * P), hi = min(new_len, (pg + 1) * P);
    uint8_t* kb = cv.k_pages + (size_t(phys) * H + h) * cv.key_block;
    uint8_t* vb = cv.v_pages + (size_t(phys) * H + h) * cv.value_block;
    uint32_t vmask[4][R];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int r = 0; r < R; ++r) vmask[p][r] = 0;

    for (int pos = lo; pos < hi; ++pos) {
      const size_t tok = size_t(b0) + (pos - start);
      const int t = pos - pg * P;
      const size_t base = (tok * H + h) * D;
      const bool in_window = W > 0 && pos >= new_len - W;
      // ---------------- key
      float x[R], xin[R];
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        xin[r] = load_elem(a.k_new, a.dtype, base + r * 64 + lane);
        x[r] = xin[r];
        ss = fmaf(x[r], x[r], ss);
      }
      ss = wave_sum(ss);
      const float nu = sqrtf(ss);
      const bool zero = !(nu >= kZeroNorm);
      const float inv = zero ? 0.f : 1.0f / nu;
      rotate<D, ROT>(x, a.params, kRoleKeyRot, pik, lds, lane, rot_scale * inv);
      int idx[R];
      float e[R];
      float es = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        idx[r] = zero ? 0 : quantize(x[r], ktr, nkt);
        float c = kcr[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) c = (idx[r] == j) ? kcr[j] : c;
        e[r] = zero ? 0.f : x[r] - c;
        es = fmaf(e[r], e[r], es);
      }
      es = wave_sum(es);
      const float gamma = sqrtf(es);
      sketch<D, ROT>(e, a.params, lds, lane);
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
      if (in_window) {
        uint16_t* kw = cv.k_window + ((size_t(slot) * H + h) * W + (pos % W)) * D;
#pragma unroll
        for (int r = 0; r < R; ++r) kw[r * 64 + lane] = float_to_f16_bits(xin[r]);
      }
      // ---------------- value
      ss = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        xin[r] = load_elem(a.v_new, a.dtype, base + r * 64 + lane);
        x[r] = xin[r];
        ss = fmaf(x[r], x[r], ss);
      }
      ss = wave_sum(ss);
      const float vnu = sqrtf(ss);
      const bool vzero = !(vnu >= kZeroNorm);
      const float vinv = vzero ? 0.f : 1.0f / vnu;
      rotate<D, ROT>(x, a.params, kRoleValueRot, piv, lds, lane, rot_scale * vinv);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int vi = vzero ? 0 : quantize(x[r], vtr, nvt);
#pragma unroll
        for (int p = 0; p < 4; ++p) vmask[p][r] |= uint32_t((vi >> p) & 1) << t;
      }
      if (page_ok && lane == 0) {
        float* norms = reinterpret_cast<float*>(vb + size_t(bv) * plane_bytes);
        norms[t] = vzero ? 0.f : vnu;
      }
      if (in_window) {
        uint16_t* vw = cv.v_window + ((size_t(slot) * H + h) * W + (pos % W)) * D;
#pragma unroll
        for (int r = 0; r < R; ++r) vw[r * 64 + lane] = float_to_f16_bits(xin[r]);
      }
    }
    if (page_ok) {
      // token bits below `lo` were written by earlier calls; keep them.  Value
      // words pair coordinates 2i (low half) and 2i + 1 (high half).
      const uint32_t keep16 = (1u << (lo - pg * P)) - 1u;
      const uint32_t keep = keep16 | (keep16 << 16);
      uint32_t* words = reinterpret_cast<uint32_t*>(vb);
      for (int p = 0; p < bv; ++p) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t mine = vmask[p][r];
          const uint32_t other = __shfl_xor(mine, 1);
          if (!(lane & 1)) {
            const int c = r * 64 + lane;
            uint32_t* w = words + (c / 2) * bv + p;
            const uint32_t old = keep ? *w : 0u;
            *w = (old & keep) | mine | (other << 16);
          }
        }
      }
    }
  }
}

template <int D, int ROT>
hipError_t launch(const AppendArgs& a, int units, hipStream_t st) {
  hipLaunchKernelGGL((append_kernel<D, ROT>), dim3(units), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int launch_append(const tq_config& cfg, const AppendArgs& a, int total_units, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool dense = cfg.rotation == TQ_ROT_DENSE;
  switch (cfg.head_dim) {
    case 64: return dense ? launch<64, TQ_ROT_DENSE>(a, total_units, st) : launch<64, TQ_ROT_FWHT>(a, total_units, st);
    case 128: return dense ? launch<128, TQ_ROT_DENSE>(a, total_units, st) : launch<128, TQ_ROT_FWHT>(a, total_units, st);
    case 256: return dense ? launch<256, TQ_ROT_DENSE>(a, total_units, st) : launch<256, TQ_ROT_FWHT>(a, total_units, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqi
