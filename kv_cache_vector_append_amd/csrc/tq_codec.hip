// The generic path: quantize-append, decode attention and reconstruction for
// every stored format a configuration describes (Codec, built on the host):
// the default one, and the extended ones
//   * mixed-channel rates: the upper half d/2 .. d-1 of the rotated
//     coordinates has its own bit count and Lloyd-Max codebook ([Design
//     Study] = "TurboQuant Family Design Study for CPU and Browser WASM KV
//     Caches", "Packed format and complete bit accounting");
//   * scale-corrected keys: all key bits to the code and one scale s instead
//     of the QJL bit, est = s <qt, c[idx]>, s = nu / <y, yhat> or
//     nu <y, yhat> / ||yhat||^2 ([Reconstruction] = "Mathematical
//     Reconstruction, Lineage, and Accuracy Limits of TurboQuant and
//     TurboVec", "The DRIVE/EDEN Mathematical Critique" and "12. TurboVec
//     Additions and Divergences");
//   * the key outlier sidecar: the largest-magnitude coordinates of each key
//     kept as (index, fp16 value) and removed before quantization ([Design
//     Study], body item 5 of the packed format; [Reconstruction] section 11);
//   * group-quantized values: per 32 coordinates an fp16 scale and zero,
//     uniform codes, no rotation ([README] = "TurboQuant: KV Cache Compression
//     for LLM Inference", "How It Works" item 4).
//
// append_codec_kernel: one wavefront per (sequence, kv head, part), striding
//   over the pages the new tokens touch; lanes hold coordinates (lane l owns
//   r * 64 + l), so rotations are cross-lane butterflies (or a matrix-vector
//   product through LDS), norms and sums are wavefront reductions, the
//   sidecar is picked by wavefront arg-max and key bit-planes are ballots.
// decode_codec_split_kernel / decode_codec_combine_kernel: one workgroup of
//   four wavefronts per (sequence, kv head, context split), one lane per token
//   for the scores (codebook lookups per coordinate), one thread per
//   coordinate for the values; a log-sum-exp merge and the inverse value
//   rotation per query head.  Used where the matrix-core kernels
//   (tq_decode_mfma.hip) do not apply: group-quantized values, head_dim 64,
//   GQA groups above 4.
// dequant_codec_kernel: one wavefront per (token, kv head).
#include "tq_device.h"

namespace tqi {
namespace {

constexpr float kZeroNorm = 1e-7f;
constexpr float kQjlConst = 1.2533141373155003f;  // sqrt(pi / 2)
constexpr int kPage = 16;

// ------------------------------------------------------------------ format
// Tables of the parameter blob: kind 0 key centroids, 1 key thresholds,
// 2 value centroids, 3 value thresholds; half 0 lower, 1 upper.
__host__ __device__ constexpr int table_offset(int kind, int half) {
  return (kind == 0 ? kOffKeyCentroids : kind == 1 ? kOffKeyThresholds : kind == 2 ? kOffValueCentroids
                                                                                   : kOffValueThresholds) +
         (half ? kOffUpperHalf : 0);
}

// idx = #{j : t_j < y} over the n thresholds (ties to the lower cell)
__device__ __forceinline__ int code_of(float y, const float* t, int n) {
  int idx = 0;
  for (int j = 0; j < n; ++j) idx += t[j] < y ? 1 : 0;
  return idx;
}

// The eight codebook tables, staged in LDS by the whole block.
__device__ __forceinline__ void load_tables(const uint8_t* params, float (&tab)[8][16], int tid, int nthreads) {
  for (int i = tid; i < 128; i += nthreads) {
    const int tb = i / 16;
    tab[tb][i % 16] = reinterpret_cast<const float*>(params + table_offset(tb / 2, tb & 1))[i % 16];
  }
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = uint32_t(__shfl_xor(int(uint32_t(v)), o));
    const uint32_t hi = uint32_t(__shfl_xor(int(uint32_t(v >> 32)), o));
    const uint64_t p = (uint64_t(hi) << 32) | lo;
    v = p > v ? p : v;
  }
  return v;
}

// ------------------------------------------------------------------ transforms of a wavefront-resident vector
// x <- scale * H D_role x (FWHT variant)
template <int R>
__device__ __forceinline__ void fwht_rotate(float (&x)[R], const uint8_t* params, int role, int lane, float scale) {
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = apply_sign(x[r], sign_bit(params, role, r * 64 + lane));
  wave_fwht<R>(x, lane);
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] *= scale;
}

// x <- scale * D_role H x (the transpose of the above, H being symmetric)
template <int R>
__device__ __forceinline__ void fwht_rotate_t(float (&x)[R], const uint8_t* params, int role, int lane, float scale) {
  wave_fwht<R>(x, lane);
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = apply_sign(x[r] * scale, sign_bit(params, role, r * 64 + lane));
}

// x <- scale * M x (TRANS: M^T x) for a row-major d x d matrix, x staged through LDS
template <int D, bool TRANS>
__device__ __forceinline__ void matvec(float (&x)[D / 64], const float* m, float* lds, int lane, float scale) {
  constexpr int R = D / 64;
#pragma unroll
  for (int r = 0; r < R; ++r) lds[r * 64 + lane] = x[r];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = r * 64 + lane;
    float acc = 0.f;
    for (int j = 0; j < D; ++j) acc = fmaf(TRANS ? m[size_t(j) * D + i] : m[size_t(i) * D + j], lds[j], acc);
    x[r] = acc * scale;
  }
  __syncthreads();
}

__device__ __forceinline__ const float* dense_matrix(const uint8_t* params, int which, int D) {
  return reinterpret_cast<const float*>(params + kOffDense) + size_t(which) * D * D;
}

// ------------------------------------------------------------------ append
template <int D, int ROT>
__global__ __launch_bounds__(64) void append_codec_kernel(AppendArgs a) {
  constexpr int R = D / 64;
  constexpr int P = kPage;
  __shared__ float lds[D];
  __shared__ float tab[8][16];
  const int lane = threadIdx.x;
  const CacheView& cv = a.cache;
  const Codec& k = cv.codec;
  const int H = cv.num_kv_heads, W = cv.window;
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
  load_tables(a.params, tab, lane, 64);
  __syncthreads();
  const bool group_values = k.value_mode == TQ_VALUE_GROUP;
  const float rot_scale = ROT == TQ_ROT_FWHT ? rsqrtf(float(D)) : 1.0f;
  // the half, and so the bit counts, of this lane's coordinates
  int hf[R];
#pragma unroll
  for (int r = 0; r < R; ++r) hf[r] = r * 64 + lane >= D / 2 ? 1 : 0;

  for (int pg = start / P + part; pg * P < new_len; pg += a.parts) {
    if (pg >= cv.max_pages_per_seq) {
      report(cv.status, true, TQ_STATUS_CAPACITY);
      break;
    }
    const int phys = cv.block_table[size_t(slot) * cv.max_pages_per_seq + pg];
    const bool page_ok = phys >= 0 && phys < cv.num_pages;
    report(cv.status, !page_ok, TQ_STATUS_BAD_PAGE);
    const int lo = max(start, pg * P), hi = min(new_len, (pg + 1) * P);
    uint8_t* kb = cv.k_pages + (size_t(max(phys, 0)) * H + h) * cv.key_block;
    uint8_t* vb = cv.v_pages + (size_t(max(phys, 0)) * H + h) * cv.value_block;
    uint32_t* vwords = reinterpret_cast<uint32_t*>(vb);
    // value planes, per coordinate: the page's 16 token bits; a partly filled
    // page's earlier tokens are kept (no other wavefront writes this page)
    const uint32_t keep16 = (1u << (lo - pg * P)) - 1u;
    uint32_t vmask[4][R], old[4][R];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        vmask[p][r] = 0u;
        old[p][r] = 0u;
        if (page_ok && keep16 != 0u && p < k.vbits[hf[r]] && !(lane & 1))
          old[p][r] = vwords[value_pair_word(k, (r * 64 + lane) / 2, D) + p];
      }

    for (int pos = lo; pos < hi; ++pos) {
      const int t = pos - pg * P;
      const size_t base = ((size_t(b0) + (pos - start)) * H + h) * D;
      const bool in_window = W > 0 && pos >= new_len - W;
      float x[R], vin[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        x[r] = load_elem(a.k_new, a.dtype, base + r * 64 + lane);
        vin[r] = load_elem(a.v_new, a.dtype, base + r * 64 + lane);
      }
      if (in_window) {
        uint16_t* kw = cv.k_window + ((size_t(slot) * H + h) * W + (pos % W)) * D;
        uint16_t* vw = cv.v_window + ((size_t(slot) * H + h) * W + (pos % W)) * D;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          kw[r * 64 + lane] = float_to_f16_bits(x[r]);
          vw[r * 64 + lane] = float_to_f16_bits(vin[r]);
        }
      }
      // ---------------- key outlier sidecar: repeated wavefront arg-max of
      // |x| (ties to the lower coordinate), each winner removed from x
      int side_idx[kMaxOutliers];
      float side_val[kMaxOutliers];
      int side_cnt = 0;
      bool done = false;
#pragma unroll
      for (int j = 0; j < kMaxOutliers; ++j) {
        side_idx[j] = 0;
        side_val[j] = 0.f;
        if (j < k.outliers && !done) {
          uint64_t best = 0;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint64_t key = (uint64_t(__float_as_uint(fabsf(x[r]))) << 32) | uint32_t(~uint32_t(r * 64 + lane));
            best = key > best ? key : best;
          }
          best = wave_max_u64(best);
          if (uint32_t(best >> 32) == 0u) {
            done = true;  // no nonzero coordinate left
          } else {
            const int coord = int(~uint32_t(best));
            float v = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r)
              if (r * 64 + lane == coord) {
                v = x[r];
                x[r] = 0.f;
              }
            side_val[j] = __shfl(v, coord & 63);
            side_idx[j] = coord;
            side_cnt = j + 1;
          }
        }
      }
      // ---------------- key: norm, rotation, codes
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) ss = fmaf(x[r], x[r], ss);
      const float nu = sqrtf(wave_sum(ss));
      const bool zero = !(nu >= kZeroNorm);
      const float inv = zero ? 0.f : 1.0f / nu;
      if constexpr (ROT == TQ_ROT_FWHT) fwht_rotate<R>(x, a.params, kRoleKeyRot, lane, rot_scale * inv);
      else matvec<D, false>(x, dense_matrix(a.params, 0, D), lds, lane, inv);
      int idx[R];
      float yh[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        idx[r] = zero ? 0 : code_of(x[r], tab[2 + hf[r]], (1 << k.kbits[hf[r]]) - 1);
        yh[r] = tab[hf[r]][idx[r]];
      }
      float aux = 0.f;
      bool zbit[R];
      if (k.qjl) {
        float e[R], es = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          e[r] = zero ? 0.f : x[r] - yh[r];
          es = fmaf(e[r], e[r], es);
        }
        aux = sqrtf(wave_sum(es));
        // w = S e: FWHT variant S = H D2 H_n D1, dense variant the Gaussian G
        if constexpr (ROT == TQ_ROT_FWHT) {
          fwht_rotate<R>(e, a.params, kRoleSketch1, lane, rsqrtf(float(D)));
          fwht_rotate<R>(e, a.params, kRoleSketch2, lane, 1.0f);
        } else {
          matvec<D, false>(e, dense_matrix(a.params, 1, D), lds, lane, 1.0f);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) zbit[r] = !zero && e[r] < 0.f;
      } else {
        float ip = 0.f, nn = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          ip = fmaf(zero ? 0.f : x[r], yh[r], ip);
          nn = fmaf(yh[r], yh[r], nn);
          zbit[r] = false;
        }
        ip = wave_sum(ip);
        nn = wave_sum(nn);
        aux = zero ? 0.f : (k.key_mode == TQ_KEY_SCALED_UNBIASED ? nu / ip : nu * ip / nn);
      }
      if (page_ok) {
        // lane g < d/32 gathers the words of 32-coordinate group g (ballots of
        // 64 coordinates cover groups 2r and 2r + 1)
        uint32_t words[5];
#pragma unroll
        for (int p = 0; p < 5; ++p) {
          words[p] = 0u;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const bool bit = p < 4 ? (p < k.kbits[hf[r]] && ((idx[r] >> p) & 1)) : zbit[r];
            const uint64_t m = __ballot(bit);
            if ((lane >> 1) == r) words[p] = (lane & 1) ? uint32_t(m >> 32) : uint32_t(m);
          }
        }
        if (lane < D / kGroup) {
          const int mg = k.kbits[lane >= D / (2 * kGroup) ? 1 : 0];
          uint32_t* dst = reinterpret_cast<uint32_t*>(kb) + t * k.key_row_words + key_group_word(k, lane, D);
#pragma unroll
          for (int p = 0; p < 4; ++p)
            if (p < mg) dst[p] = words[p];
          if (k.qjl) dst[mg] = words[4];
        }
        if (lane == 0) {
          *reinterpret_cast<float2*>(kb + k.key_norm_off + 8 * t) = make_float2(zero ? 0.f : nu, aux);
          if (k.outliers) {
            uint8_t* rec = kb + k.key_side_off + t * k.side_bytes;
            rec[0] = uint8_t(side_cnt);
#pragma unroll
            for (int j = 0; j < kMaxOutliers; ++j)
              if (j < k.outliers) {
                rec[1 + j] = uint8_t(j < side_cnt ? side_idx[j] : 0);
                reinterpret_cast<uint16_t*>(rec + k.side_val_off)[j] =
                    j < side_cnt ? float_to_f16_bits(side_val[j]) : uint16_t(0);
              }
          }
        }
      }
      // ---------------- value
#pragma unroll
      for (int r = 0; r < R; ++r) x[r] = vin[r];
      if (group_values) {
        // per 32-coordinate group (a half wavefront for each r): fp16 scale and
        // zero, codes decided in fp32
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float mn = x[r], mx = x[r];
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) {
            mn = fminf(mn, __shfl_xor(mn, o));
            mx = fmaxf(mx, __shfl_xor(mx, o));
          }
          const int b = k.vbits[hf[r]];
          const float levels = float((1 << b) - 1);
          const uint16_t s16 = float_to_f16_bits((mx - mn) / levels);
          const uint16_t z16 = float_to_f16_bits(mn);
          const float sf = f16_bits_to_float(s16), zf = f16_bits_to_float(z16);
          const int code = sf > 0.f ? int(fminf(fmaxf(rintf((x[r] - zf) / sf), 0.f), levels)) : 0;
#pragma unroll
          for (int p = 0; p < 4; ++p) vmask[p][r] |= uint32_t((code >> p) & 1) << t;
          if (page_ok && (lane & (kGroup - 1)) == 0) {
            const int g = (r * 64 + lane) / kGroup;
            reinterpret_cast<uint32_t*>(vb + k.value_tail_off)[t * (D / kGroup) + g] =
                uint32_t(s16) | (uint32_t(z16) << 16);
          }
        }
      } else {
        ss = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) ss = fmaf(x[r], x[r], ss);
        const float vnu = sqrtf(wave_sum(ss));
        const bool vzero = !(vnu >= kZeroNorm);
        const float vinv = vzero ? 0.f : 1.0f / vnu;
        if constexpr (ROT == TQ_ROT_FWHT) fwht_rotate<R>(x, a.params, kRoleValueRot, lane, rot_scale * vinv);
        else matvec<D, false>(x, dense_matrix(a.params, 2, D), lds, lane, vinv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int vi = vzero ? 0 : code_of(x[r], tab[6 + hf[r]], (1 << k.vbits[hf[r]]) - 1);
#pragma unroll
          for (int p = 0; p < 4; ++p) vmask[p][r] |= uint32_t((vi >> p) & 1) << t;
        }
        if (page_ok && lane == 0) reinterpret_cast<float*>(vb + k.value_tail_off)[t] = vzero ? 0.f : vnu;
      }
    }
    if (page_ok) {
      // value words pair coordinates 2i (low half) and 2i + 1 (high half)
      const uint32_t keep = keep16 | (keep16 << 16);
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t mine = vmask[p][r];
          const uint32_t other = __shfl_xor(mine, 1);
          if (!(lane & 1) && p < k.vbits[hf[r]])
            vwords[value_pair_word(k, (r * 64 + lane) / 2, D) + p] = (old[p][r] & keep) | mine | (other << 16);
        }
    }
  }
}

// ------------------------------------------------------------------ decode
constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kMaxGroup = 8;

// rows of buf (G vectors of length D in LDS) <- scale * T rows, by the block
template <int D, int ROT>
__device__ void rotate_rows(float* buf, int G, const uint8_t* params, int role, const float* dense, float* tmp,
                            float scale, int tid) {
  if (ROT == TQ_ROT_FWHT) {
    for (int i = tid; i < G * D; i += kThreads) buf[i] = apply_sign(buf[i], sign_bit(params, role, i % D));
    __syncthreads();
    block_fwht(buf, G, D, tid, kThreads);
    for (int i = tid; i < G * D; i += kThreads) buf[i] *= scale;
    __syncthreads();
  } else {
    for (int i = tid; i < G * D; i += kThreads) {
      const int g = i / D, c = i % D;
      const float* row = dense + size_t(c) * D;
      const float* x = buf + g * D;
      float acc = 0.f;
      for (int j = 0; j < D; ++j) acc = fmaf(row[j], x[j], acc);
      tmp[i] = acc * scale;
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += kThreads) buf[i] = tmp[i];
    __syncthreads();
  }
}

// est = nu (<qt, yhat> + gamma sqrt(pi/2)/d <qh, 1 - 2z>) or s <qt, yhat>,
// plus the sidecar's sum_j q[idx_j] val_j, for one stored key and one head
template <int D>
__device__ __forceinline__ float key_estimate(const Codec& k, const uint32_t* row, const float* aux2,
                                              const uint8_t* side, const float* qr, const float* qs, const float* qraw,
                                              const float (&tab)[8][16]) {
  float mse = 0.f, qjl = 0.f;
#pragma unroll
  for (int g = 0; g < D / kGroup; ++g) {
    const int half = g >= D / (2 * kGroup) ? 1 : 0;
    const int mg = k.kbits[half];
    const uint32_t* gw = row + key_group_word(k, g, D);
    uint32_t w[5];
#pragma unroll
    for (int p = 0; p < 5; ++p) w[p] = p < mg + k.qjl ? gw[p] : 0u;
    const uint32_t zw = k.qjl ? w[min(mg, 4)] : 0u;
    for (int b = 0; b < kGroup; ++b) {
      int idx = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if (p < mg) idx |= int((w[p] >> b) & 1u) << p;
      mse = fmaf(qr[g * kGroup + b], tab[half][idx], mse);
      if (k.qjl) qjl += ((zw >> b) & 1u) ? -qs[g * kGroup + b] : qs[g * kGroup + b];
    }
  }
  float est = k.qjl ? aux2[0] * (mse + aux2[1] * (kQjlConst / float(D)) * qjl) : aux2[1] * mse;
  if (k.outliers) {
    const int cnt = side[0];
    const uint16_t* vals = reinterpret_cast<const uint16_t*>(side + k.side_val_off);
    for (int j = 0; j < cnt && j < k.outliers; ++j) est = fmaf(qraw[side[1 + j]], f16_bits_to_float(vals[j]), est);
  }
  return est;
}

template <int D, int ROT>
__global__ __launch_bounds__(kThreads) void decode_codec_split_kernel(DecodeArgs a) {
  constexpr int P = kPage;
  constexpr int HPT = (D * kMaxGroup + kThreads - 1) / kThreads;  // (coordinate, head) pairs per thread
  __shared__ float q_rot[kMaxGroup * D];
  __shared__ float q_sk[kMaxGroup * D];
  __shared__ float q_raw[kMaxGroup * D];
  __shared__ float tmp[kMaxGroup * D];
  __shared__ float w_tile[kMaxGroup][kTile];
  __shared__ float vnu_tile[kTile];
  __shared__ float m_run[kMaxGroup], l_run[kMaxGroup], alpha[kMaxGroup];
  __shared__ float tab[8][16];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const CacheView& cv = a.cache;
  const Codec& k = cv.codec;
  const int H = cv.num_kv_heads, W = cv.window;
  const int G = a.num_q_heads / H;
  const int s = blockIdx.x / H, h = blockIdx.x % H;
  const int split = blockIdx.y;
  const bool group_values = k.value_mode == TQ_VALUE_GROUP;

  const int slot = a.seq_slots[s];
  int L = a.ctx_len[s];
  if (cv.status != nullptr && split == 0 && tid == 0) {
    report(cv.status, slot < 0 || slot >= cv.max_seqs, TQ_STATUS_BAD_SLOT);
    report(cv.status, L < 0 || L > min(cv.max_pages_per_seq * P, a.max_ctx), TQ_STATUS_CAPACITY);
  }
  if (slot < 0 || slot >= cv.max_seqs || L < 0) L = 0;
  if (L > cv.max_pages_per_seq * P) L = cv.max_pages_per_seq * P;
  if (L > a.max_ctx) L = a.max_ctx;
  const int nc = W > 0 ? max(0, L - W) : L;
  const int t_begin = split * a.split_tokens;
  const int t_end = min(nc, t_begin + a.split_tokens);
  const bool do_window = (split == a.splits - 1) && W > 0 && L > nc;

  load_tables(a.params, tab, tid, kThreads);
  if (tid < kMaxGroup) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.f;
  }
  for (int i = tid; i < G * D; i += kThreads) {
    const float v = load_elem(a.q, a.q_dtype, (size_t(s) * a.num_q_heads + h * G) * D + i);
    q_raw[i] = v;
    q_rot[i] = v;
  }
  __syncthreads();

  const float* pik = dense_matrix(a.params, 0, D);
  // qt = T_K q;  qh = S qt (QJL mode)
  rotate_rows<D, ROT>(q_rot, G, a.params, kRoleKeyRot, pik, tmp, ROT == TQ_ROT_FWHT ? rsqrtf(float(D)) : 1.0f, tid);
  if (k.qjl) {
    for (int i = tid; i < G * D; i += kThreads) q_sk[i] = q_rot[i];
    __syncthreads();
    if (ROT == TQ_ROT_FWHT) {
      rotate_rows<D, ROT>(q_sk, G, a.params, kRoleSketch1, nullptr, tmp, rsqrtf(float(D)), tid);
      rotate_rows<D, ROT>(q_sk, G, a.params, kRoleSketch2, nullptr, tmp, 1.0f, tid);
    } else {
      rotate_rows<D, ROT>(q_sk, G, a.params, 0, dense_matrix(a.params, 1, D), tmp, 1.0f, tid);
    }
  }

  // value accumulators: thread owns coordinate c and heads g = g0, g0 + gstep, ...
  // (acc_rot in the rotated domain; acc_win unrotated: the window and the
  // group-quantized values)
  const int c_own = tid % D;
  const int g0 = tid / D;
  const int gstep = kThreads / D > 0 ? kThreads / D : 1;
  const int c_half = c_own >= D / 2 ? 1 : 0;
  const int c_bits = k.vbits[c_half];
  const int c_word = value_pair_word(k, c_own / 2, D);
  float acc_rot[HPT], acc_win[HPT];
#pragma unroll
  for (int kk = 0; kk < HPT; ++kk) acc_rot[kk] = acc_win[kk] = 0.f;
  float* logits = a.logits;

  // ------------------------------------------------ compressed tokens
  for (int tb = t_begin; tb < t_end; tb += kTile) {
    // scores: thread -> token j = lane, heads g = wv, wv + 4, ...
    {
      const int j = lane;
      const int pos = tb + j;
      const bool valid = pos < t_end;
      bool page_ok = false;
      const uint8_t* kb = nullptr;
      int t = 0;
      if (valid) {
        const int phys = cv.block_table[size_t(slot) * cv.max_pages_per_seq + pos / P];
        page_ok = phys >= 0 && phys < cv.num_pages;
        report(cv.status, !page_ok, TQ_STATUS_BAD_PAGE);
        t = pos % P;
        if (page_ok) {
          kb = cv.k_pages + (size_t(phys) * H + h) * cv.key_block;
          if (wv == 0) {
            const uint8_t* vb = cv.v_pages + (size_t(phys) * H + h) * cv.value_block;
            vnu_tile[j] = group_values ? 1.f : reinterpret_cast<const float*>(vb + k.value_tail_off)[t];
          }
        }
      }
      if (!page_ok && wv == 0) vnu_tile[j] = 0.f;
      for (int g = wv; g < G; g += kThreads / 64) {
        float score = -INFINITY;
        if (page_ok) {
          const uint32_t* row = reinterpret_cast<const uint32_t*>(kb) + t * k.key_row_words;
          const float* aux2 = reinterpret_cast<const float*>(kb + k.key_norm_off) + 2 * t;
          const uint8_t* side = kb + k.key_side_off + t * k.side_bytes;
          score = a.scale * key_estimate<D>(k, row, aux2, side, q_rot + g * D, q_sk + g * D, q_raw + g * D, tab);
          if (logits) logits[(size_t(s) * a.num_q_heads + h * G + g) * a.max_ctx + pos] = score;
        }
        w_tile[g][j] = score;
      }
    }
    __syncthreads();
    // online softmax per head: wavefront wv handles heads wv, wv + 4, ...
    for (int g = wv; g < G; g += kThreads / 64) {
      const float sc = w_tile[g][lane];
      const float tmax = wave_max(sc);
      const float m_old = m_run[g];
      const float m_new = fmaxf(m_old, tmax);
      const float p = (m_new == -INFINITY) ? 0.f : __expf(sc - m_new);
      const float psum = wave_sum(p);
      const float al = (m_new == -INFINITY) ? 1.f : __expf(m_old - m_new);
      w_tile[g][lane] = p * vnu_tile[lane];
      if (lane == 0) {
        l_run[g] = l_run[g] * al + psum;
        m_run[g] = m_new;
        alpha[g] = al;
      }
    }
    __syncthreads();
    // values
    {
      const int ntok = min(kTile, t_end - tb);
#pragma unroll
      for (int kk = 0; kk < HPT; ++kk) {
        const int g = g0 + kk * gstep;
        const float al = g < G ? alpha[g] : 1.f;
        acc_rot[kk] *= al;
        acc_win[kk] *= al;
      }
      for (int pgs = 0; pgs < ntok; pgs += P) {
        const int pos0 = tb + pgs;
        const int phys = cv.block_table[size_t(slot) * cv.max_pages_per_seq + pos0 / P];
        if (phys < 0 || phys >= cv.num_pages) continue;
        const uint8_t* vb = cv.v_pages + (size_t(phys) * H + h) * cv.value_block;
        uint32_t masks[4];
        const uint32_t* vw = reinterpret_cast<const uint32_t*>(vb) + c_word;
#pragma unroll
        for (int p = 0; p < 4; ++p) masks[p] = p < c_bits ? (vw[p] >> (16 * (c_own & 1))) & 0xffffu : 0u;
        const uint32_t* sz = reinterpret_cast<const uint32_t*>(vb + k.value_tail_off) + c_own / kGroup;
        const int nt = min(P, ntok - pgs);
        for (int t = 0; t < nt; ++t) {
          int idx = 0;
#pragma unroll
          for (int p = 0; p < 4; ++p) idx |= int((masks[p] >> t) & 1u) << p;
          if (group_values) {
            const uint32_t pair = sz[t * (D / kGroup)];
            const float val = fmaf(f16_bits_to_float(uint16_t(pair & 0xffffu)), float(idx),
                                   f16_bits_to_float(uint16_t(pair >> 16)));
#pragma unroll
            for (int kk = 0; kk < HPT; ++kk) {
              const int g = g0 + kk * gstep;
              if (g < G) acc_win[kk] = fmaf(w_tile[g][pgs + t], val, acc_win[kk]);
            }
          } else {
            const float val = tab[4 + c_half][idx];
#pragma unroll
            for (int kk = 0; kk < HPT; ++kk) {
              const int g = g0 + kk * gstep;
              if (g < G) acc_rot[kk] = fmaf(w_tile[g][pgs + t], val, acc_rot[kk]);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------ fp16 window (exact)
  if (do_window) {
    const uint16_t* kwin = cv.k_window + (size_t(slot) * H + h) * W * D;
    const uint16_t* vwin = cv.v_window + (size_t(slot) * H + h) * W * D;
    for (int tb = nc; tb < L; tb += kTile) {
      const int j = lane;
      const int pos = tb + j;
      const bool valid = pos < L;
      for (int g = wv; g < G; g += kThreads / 64) {
        float score = -INFINITY;
        if (valid) {
          const uint16_t* kr = kwin + size_t(pos % W) * D;
          const float* qr = q_raw + g * D;
          float dot = 0.f;
          for (int c = 0; c < D; ++c) dot = fmaf(qr[c], f16_bits_to_float(kr[c]), dot);
          score = a.scale * dot;
          if (logits) logits[(size_t(s) * a.num_q_heads + h * G + g) * a.max_ctx + pos] = score;
        }
        w_tile[g][j] = score;
      }
      __syncthreads();
      for (int g = wv; g < G; g += kThreads / 64) {
        const float sc = w_tile[g][lane];
        const float tmax = wave_max(sc);
        const float m_old = m_run[g];
        const float m_new = fmaxf(m_old, tmax);
        const float p = (m_new == -INFINITY) ? 0.f : __expf(sc - m_new);
        const float psum = wave_sum(p);
        const float al = (m_new == -INFINITY) ? 1.f : __expf(m_old - m_new);
        w_tile[g][lane] = p;
        if (lane == 0) {
          l_run[g] = l_run[g] * al + psum;
          m_run[g] = m_new;
          alpha[g] = al;
        }
      }
      __syncthreads();
      const int ntok = min(kTile, L - tb);
#pragma unroll
      for (int kk = 0; kk < HPT; ++kk) {
        const int g = g0 + kk * gstep;
        const float al = g < G ? alpha[g] : 1.f;
        acc_rot[kk] *= al;
        acc_win[kk] *= al;
      }
      for (int t = 0; t < ntok; ++t) {
        const float v = f16_bits_to_float(vwin[size_t((tb + t) % W) * D + c_own]);
#pragma unroll
        for (int kk = 0; kk < HPT; ++kk) {
          const int g = g0 + kk * gstep;
          if (g < G) acc_win[kk] = fmaf(w_tile[g][t], v, acc_win[kk]);
        }
      }
      __syncthreads();
    }
  }

  // ------------------------------------------------ partial results
  const int rec = 2 + 2 * D;
#pragma unroll
  for (int kk = 0; kk < HPT; ++kk) {
    const int g = g0 + kk * gstep;
    if (g < G) {
      float* ws = a.workspace + ((size_t(s) * a.num_q_heads + h * G + g) * a.splits + split) * rec;
      ws[2 + c_own] = acc_rot[kk];
      ws[2 + D + c_own] = acc_win[kk];
      if (c_own == 0) {
        ws[0] = m_run[g];
        ws[1] = l_run[g];
      }
    }
  }
}

// Merge the splits of one (sequence, query head) by log-sum-exp, rotate the
// rotated-domain value sum back once, add the unrotated one, normalise.
template <int D, int ROT>
__global__ __launch_bounds__(D) void decode_codec_combine_kernel(DecodeArgs a) {
  __shared__ float buf[D];
  const int c = threadIdx.x;
  const size_t row = blockIdx.x;  // s * H_q + hq
  const int rec = 2 + 2 * D;
  const float* ws = a.workspace + row * a.splits * rec;
  float M = -INFINITY;
  for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, ws[sp * rec]);
  float l = 0.f, ar = 0.f, aw = 0.f;
  if (M != -INFINITY) {
    for (int sp = 0; sp < a.splits; ++sp) {
      const float m = ws[sp * rec];
      if (m == -INFINITY) continue;
      const float f = __expf(m - M);
      l = fmaf(ws[sp * rec + 1], f, l);
      ar = fmaf(ws[sp * rec + 2 + c], f, ar);
      aw = fmaf(ws[sp * rec + 2 + D + c], f, aw);
    }
  }
  float o = 0.f;
  if (a.cache.codec.value_mode != TQ_VALUE_GROUP) {  // group-quantized values are accumulated unrotated
    buf[c] = ar;
    __syncthreads();
    if (ROT == TQ_ROT_FWHT) {
      block_fwht(buf, 1, D, c, D);
      o = apply_sign(buf[c] * rsqrtf(float(D)), sign_bit(a.params, kRoleValueRot, c));
    } else {
      const float* piv = dense_matrix(a.params, 2, D);
      for (int j = 0; j < D; ++j) o = fmaf(piv[size_t(j) * D + c], buf[j], o);
    }
  }
  a.out[row * D + c] = l > 0.f ? (o + aw) / l : 0.f;
}

// ------------------------------------------------------------------ dequantize
// k~ = nu T_K^T (c[idx] + gamma sqrt(pi/2)/d S^T (1 - 2z)) (QJL mode) or
// s T_K^T c[idx] (scaled modes), plus the sidecar entries; v~ = nu T_V^T c[idx]
// or zero + scale * code.  <q, k~> equals the decode-time score estimate.
template <int D, int ROT>
__global__ __launch_bounds__(64) void dequant_codec_kernel(DequantArgs a) {
  constexpr int R = D / 64;
  constexpr int P = kPage;
  __shared__ float lds[D];
  __shared__ float tab[8][16];
  const int lane = threadIdx.x;
  const CacheView& cv = a.cache;
  const Codec& k = cv.codec;
  const int H = cv.num_kv_heads;
  const int i = blockIdx.x / H, h = blockIdx.x % H;
  const int pos = a.tok_begin + i;
  float* ko = a.k_out + (size_t(i) * H + h) * D;
  float* vo = a.v_out + (size_t(i) * H + h) * D;
  const int pg = pos / P, t = pos % P;
  const int phys = (pg < cv.max_pages_per_seq) ? cv.block_table[size_t(a.seq_slot) * cv.max_pages_per_seq + pg] : -1;
  if (phys < 0 || phys >= cv.num_pages) {
    report(cv.status, lane == 0, TQ_STATUS_BAD_PAGE);
#pragma unroll
    for (int r = 0; r < R; ++r) ko[r * 64 + lane] = vo[r * 64 + lane] = 0.f;
    return;
  }
  load_tables(a.params, tab, lane, 64);
  __syncthreads();
  const uint8_t* kb = cv.k_pages + (size_t(phys) * H + h) * cv.key_block;
  const uint8_t* vb = cv.v_pages + (size_t(phys) * H + h) * cv.value_block;

  // ---------------- key
  const uint32_t* row = reinterpret_cast<const uint32_t*>(kb) + t * k.key_row_words;
  float yr[R], sg[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = r * 64 + lane, g = c / kGroup, half = c >= D / 2 ? 1 : 0, mg = k.kbits[half];
    const uint32_t* gw = row + key_group_word(k, g, D);
    int idx = 0;
    for (int p = 0; p < mg; ++p) idx |= int((gw[p] >> (c % kGroup)) & 1u) << p;
    yr[r] = tab[half][idx];
    sg[r] = k.qjl && ((gw[mg] >> (c % kGroup)) & 1u) ? -1.f : 1.f;
  }
  const float* aux2 = reinterpret_cast<const float*>(kb + k.key_norm_off) + 2 * t;
  float kscale = aux2[1];
  if (k.qjl) {
    // S^T s: FWHT variant S^T = D1 H_n D2 H; dense variant G^T
    if constexpr (ROT == TQ_ROT_FWHT) {
      fwht_rotate_t<R>(sg, a.params, kRoleSketch2, lane, 1.0f);
      fwht_rotate_t<R>(sg, a.params, kRoleSketch1, lane, rsqrtf(float(D)));
    } else {
      matvec<D, true>(sg, dense_matrix(a.params, 1, D), lds, lane, 1.0f);
    }
    const float qc = aux2[1] * kQjlConst / float(D);
#pragma unroll
    for (int r = 0; r < R; ++r) yr[r] = fmaf(qc, sg[r], yr[r]);
    kscale = aux2[0];
  }
  if constexpr (ROT == TQ_ROT_FWHT) fwht_rotate_t<R>(yr, a.params, kRoleKeyRot, lane, rsqrtf(float(D)));
  else matvec<D, true>(yr, dense_matrix(a.params, 0, D), lds, lane, 1.0f);
#pragma unroll
  for (int r = 0; r < R; ++r) yr[r] *= kscale;
  if (k.outliers) {
    const uint8_t* side = kb + k.key_side_off + t * k.side_bytes;
    const uint16_t* vals = reinterpret_cast<const uint16_t*>(side + k.side_val_off);
    const int cnt = side[0];
    for (int j = 0; j < cnt && j < k.outliers; ++j) {
      const int c = side[1 + j];
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (c == r * 64 + lane) yr[r] += f16_bits_to_float(vals[j]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) ko[r * 64 + lane] = yr[r];

  // ---------------- value
  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = r * 64 + lane, half = c >= D / 2 ? 1 : 0, b = k.vbits[half];
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(vb) + value_pair_word(k, c / 2, D);
    int idx = 0;
    for (int p = 0; p < b; ++p) idx |= int((vw[p] >> (16 * (c & 1) + t)) & 1u) << p;
    if (k.value_mode == TQ_VALUE_GROUP) {
      const uint32_t pair = reinterpret_cast<const uint32_t*>(vb + k.value_tail_off)[t * (D / kGroup) + c / kGroup];
      v[r] = fmaf(f16_bits_to_float(uint16_t(pair & 0xffffu)), float(idx), f16_bits_to_float(uint16_t(pair >> 16)));
    } else {
      v[r] = tab[4 + half][idx];
    }
  }
  if (k.value_mode != TQ_VALUE_GROUP) {
    const float vnu = reinterpret_cast<const float*>(vb + k.value_tail_off)[t];
    if constexpr (ROT == TQ_ROT_FWHT) fwht_rotate_t<R>(v, a.params, kRoleValueRot, lane, rsqrtf(float(D)));
    else matvec<D, true>(v, dense_matrix(a.params, 2, D), lds, lane, 1.0f);
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] *= vnu;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) vo[r * 64 + lane] = v[r];
}

template <int D, int ROT>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
  const int H = a.cache.num_kv_heads;
  hipLaunchKernelGGL((decode_codec_split_kernel<D, ROT>), dim3(a.num_seqs * H, a.splits), dim3(kThreads), 0, st,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_codec_combine_kernel<D, ROT>), dim3(a.num_seqs * a.num_q_heads), dim3(D), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int launch_append_codec(const tq_config& cfg, const AppendArgs& args, int num_seqs, int max_new, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  AppendArgs a = args;
  // one wavefront per page the new tokens touch (plus one for a partial first
  // page), capped for huge prefills; each strides over the pages
  int parts = (max_new + cfg.page_tokens - 1) / cfg.page_tokens + 1;
  if (parts > 4096) parts = 4096;
  a.parts = parts;
  const long long units = (long long)num_seqs * cfg.num_kv_heads * parts;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  const bool dense = cfg.rotation == TQ_ROT_DENSE;
#define TQ_LAUNCH(D_)                                                                                            \
  if (cfg.head_dim == D_) {                                                                                      \
    if (dense) hipLaunchKernelGGL((append_codec_kernel<D_, TQ_ROT_DENSE>), dim3(units), dim3(64), 0, st, a);     \
    else hipLaunchKernelGGL((append_codec_kernel<D_, TQ_ROT_FWHT>), dim3(units), dim3(64), 0, st, a);            \
    return hipGetLastError();                                                                                    \
  }
  TQ_LAUNCH(64) TQ_LAUNCH(128) TQ_LAUNCH(256)
#undef TQ_LAUNCH
  return hipErrorInvalidValue;
}

int launch_decode_codec(const tq_config& cfg, const DecodeArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool dense = cfg.rotation == TQ_ROT_DENSE;
  switch (cfg.head_dim) {
    case 64: return dense ? launch_decode_d<64, TQ_ROT_DENSE>(a, st) : launch_decode_d<64, TQ_ROT_FWHT>(a, st);
    case 128: return dense ? launch_decode_d<128, TQ_ROT_DENSE>(a, st) : launch_decode_d<128, TQ_ROT_FWHT>(a, st);
    case 256: return dense ? launch_decode_d<256, TQ_ROT_DENSE>(a, st) : launch_decode_d<256, TQ_ROT_FWHT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

int launch_dequantize_codec(const tq_config& cfg, const DequantArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int n = a.tok_end - a.tok_begin;
  if (n <= 0) return 0;
  const dim3 grid(unsigned(n) * cfg.num_kv_heads);
  const bool dense = cfg.rotation == TQ_ROT_DENSE;
#define TQ_LAUNCH(D_)                                                                                  \
  if (cfg.head_dim == D_) {                                                                            \
    if (dense) hipLaunchKernelGGL((dequant_codec_kernel<D_, TQ_ROT_DENSE>), grid, dim3(64), 0, st, a); \
    else hipLaunchKernelGGL((dequant_codec_kernel<D_, TQ_ROT_FWHT>), grid, dim3(64), 0, st, a);        \
    return hipGetLastError();                                                                          \
  }
  TQ_LAUNCH(64) TQ_LAUNCH(128) TQ_LAUNCH(256)
#undef TQ_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace tqi
