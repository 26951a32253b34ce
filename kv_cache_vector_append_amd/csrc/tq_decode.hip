// Decode attention over the compressed cache.
//
// [Design Study] = "TurboQuant Family Design Study for CPU and Browser WASM KV
// Caches": "Capacity model" (the query is moved into the keys' rotated basis,
// q.k = (Tq).(Tk)), "CPU and WASM kernel design" (decode-time key scan over
// packed pages with no history-sized dequant buffer, value scan accumulating in
// FP32, inverse transform of the final head output only).
// [Reconstruction] = "Mathematical Reconstruction, Lineage, and Accuracy Limits
// of TurboQuant and TurboVec", section 6 "The Asymmetric Unbiased Estimator".
//
//   qt = T_K q,  qh = S qt
//   est_t = nu_t (<qt, c[idx_t]> + gamma_t sqrt(pi/2)/d <qh, 1 - 2 z_t>)
//   online softmax over scale * est (window tokens: scale * <q, k_w>, exact)
//   acc_rot = sum_t p_t nu_V,t c_V[idx_t]   (rotated domain)
//   acc_win = sum_w p_w v_w
//   out = (T_V^T acc_rot + acc_win) / l
//
// decode_split_kernel: one workgroup (4 wavefronts) per (sequence, kv head,
// context split); it serves all query heads of the GQA group so every packed
// byte is read once per group.  decode_combine_kernel merges the splits by
// log-sum-exp and applies the inverse value rotation once per query head.
#include "tq_device.h"

namespace tqi {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kMaxGroup = 8;
constexpr float kQjlConst = 1.2533141373155003f;  // sqrt(pi / 2)

template <int D, int ROT>
__device__ void rotate_rows(float* buf, int G, const uint8_t* params, int role, const float* dense,
                            float* tmp, float scale, int tid) {
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

template <int D, int ROT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int P = 16;
  constexpr int HPT = (D * kMaxGroup + kThreads - 1) / kThreads;  // (coordinate, head) pairs per thread
  __shared__ float q_rot[kMaxGroup * D];
  __shared__ float q_sk[kMaxGroup * D];
  __shared__ float q_raw[kMaxGroup * D];
  __shared__ float tmp[kMaxGroup * D];
  __shared__ float w_tile[kMaxGroup][kTile];
  __shared__ float vnu_tile[kTile];
  __shared__ float m_run[kMaxGroup], l_run[kMaxGroup], alpha[kMaxGroup];
  __shared__ float kcs[8], vcs[16];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads, W = cv.window;
  const int G = a.num_q_heads / H;
  const int s = blockIdx.x / H, h = blockIdx.x % H;
  const int split = blockIdx.y;
  const int mk = a.key_mse_bits, bv = a.value_bits;
  const size_t plane_bytes = size_t(P) * D / 8;

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

  if (tid < 8) kcs[tid] = reinterpret_cast<const float*>(a.params + kOffKeyCentroids)[tid];
  if (tid < 16) vcs[tid] = reinterpret_cast<const float*>(a.params + kOffValueCentroids)[tid];
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

  const float* pik = reinterpret_cast<const float*>(a.params + kOffDense);
  // qt = T_K q
  rotate_rows<D, ROT>(q_rot, G, a.params, kRoleKeyRot, pik, tmp,
                      ROT == TQ_ROT_FWHT ? rsqrtf(float(D)) : 1.0f, tid);
  // qh = S qt
  for (int i = tid; i < G * D; i += kThreads) q_sk[i] = q_rot[i];
  __syncthreads();
  if (ROT == TQ_ROT_FWHT) {
    rotate_rows<D, ROT>(q_sk, G, a.params, kRoleSketch1, nullptr, tmp, rsqrtf(float(D)), tid);
    rotate_rows<D, ROT>(q_sk, G, a.params, kRoleSketch2, nullptr, tmp, 1.0f, tid);
  } else {
    rotate_rows<D, ROT>(q_sk, G, a.params, 0, pik + size_t(D) * D, tmp, 1.0f, tid);
  }

  // value accumulators: thread owns coordinate c and heads g = g0, g0 + gstep, ...
  const int c_own = tid % D;
  const int g0 = tid / D;
  const int gstep = kThreads / D > 0 ? kThreads / D : 1;
  float acc_rot[HPT], acc_win[HPT];
#pragma unroll
  for (int k = 0; k < HPT; ++k) acc_rot[k] = acc_win[k] = 0.f;

  const float qjl_scale = kQjlConst / float(D);
  float* logits = a.logits;

  // ------------------------------------------------ compressed tokens
  for (int tb = t_begin; tb < t_end; tb += kTile) {
    // scores: thread -> token j = lane, heads g = wv, wv + 4, ...
    {
      const int j = lane;
      const int pos = tb + j;
      const bool valid = pos < t_end;
      uint32_t words[4][D / 32];
      float knu = 0.f, kgam = 0.f;
      bool page_ok = false;
      if (valid) {
        const int phys = cv.block_table[size_t(slot) * cv.max_pages_per_seq + pos / P];
        page_ok = phys >= 0 && phys < cv.num_pages;
        report(cv.status, !page_ok, TQ_STATUS_BAD_PAGE);
        if (page_ok) {
          const uint8_t* kb = cv.k_pages + (size_t(phys) * H + h) * cv.key_block;
          const int t = pos % P;
          const uint32_t* row = reinterpret_cast<const uint32_t*>(kb) + size_t(t) * (D / 32) * (mk + 1);
          for (int p = 0; p <= mk; ++p) {
#pragma unroll
            for (int wi = 0; wi < D / 32; ++wi) words[p][wi] = row[wi * (mk + 1) + p];
          }
          const float* norms = reinterpret_cast<const float*>(kb + size_t(mk + 1) * plane_bytes) + 2 * t;
          knu = norms[0];
          kgam = norms[1];
          if (wv == 0) {
            const uint8_t* vb = cv.v_pages + (size_t(phys) * H + h) * cv.value_block;
            vnu_tile[j] = reinterpret_cast<const float*>(vb + size_t(bv) * plane_bytes)[t];
          }
        } else if (wv == 0) {
          vnu_tile[j] = 0.f;
        }
      } else if (wv == 0) {
        vnu_tile[j] = 0.f;
      }
      for (int g = wv; g < G; g += kThreads / 64) {
        float score = -INFINITY;
        if (valid && page_ok) {
          const float* qr = q_rot + g * D;
          const float* qs = q_sk + g * D;
          float mse = 0.f, qjl = 0.f;
#pragma unroll
          for (int wi = 0; wi < D / 32; ++wi) {
            for (int b = 0; b < 32; ++b) {
              int idx = 0;
              for (int p = 0; p < mk; ++p) idx |= int((words[p][wi] >> b) & 1u) << p;
              mse = fmaf(qr[wi * 32 + b], kcs[idx], mse);
              const float sv = ((words[mk][wi] >> b) & 1u) ? -qs[wi * 32 + b] : qs[wi * 32 + b];
              qjl += sv;
            }
          }
          score = a.scale * knu * (mse + kgam * qjl_scale * qjl);
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
    // value accumulation in the rotated domain
    {
      const int ntok = min(kTile, t_end - tb);
      float al[HPT];
#pragma unroll
      for (int k = 0; k < HPT; ++k) {
        const int g = g0 + k * gstep;
        al[k] = g < G ? alpha[g] : 1.f;
        acc_rot[k] *= al[k];
        acc_win[k] *= al[k];
      }
      for (int pgs = 0; pgs < ntok; pgs += P) {
        const int pos0 = tb + pgs;
        const int phys = cv.block_table[size_t(slot) * cv.max_pages_per_seq + pos0 / P];
        if (phys < 0 || phys >= cv.num_pages) continue;
        const uint8_t* vb = cv.v_pages + (size_t(phys) * H + h) * cv.value_block;
        uint32_t masks[4];
        const uint32_t* vw = reinterpret_cast<const uint32_t*>(vb) + (c_own / 2) * bv;
        for (int p = 0; p < bv; ++p) masks[p] = (vw[p] >> (16 * (c_own & 1))) & 0xffffu;
        const int nt = min(P, ntok - pgs);
        for (int t = 0; t < nt; ++t) {
          int idx = 0;
          for (int p = 0; p < bv; ++p) idx |= int((masks[p] >> t) & 1u) << p;
          const float val = vcs[idx];
#pragma unroll
          for (int k = 0; k < HPT; ++k) {
            const int g = g0 + k * gstep;
            if (g < G) acc_rot[k] = fmaf(w_tile[g][pgs + t], val, acc_rot[k]);
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
      for (int k = 0; k < HPT; ++k) {
        const int g = g0 + k * gstep;
        const float al = g < G ? alpha[g] : 1.f;
        acc_rot[k] *= al;
        acc_win[k] *= al;
      }
      for (int t = 0; t < ntok; ++t) {
        const float v = f16_bits_to_float(vwin[size_t((tb + t) % W) * D + c_own]);
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
          const int g = g0 + k * gstep;
          if (g < G) acc_win[k] = fmaf(w_tile[g][t], v, acc_win[k]);
        }
      }
      __syncthreads();
    }
  }

  // ------------------------------------------------ partial results
  const int rec = 2 + 2 * D;
#pragma unroll
  for (int k = 0; k < HPT; ++k) {
    const int g = g0 + k * gstep;
    if (g < G) {
      float* ws = a.workspace + ((size_t(s) * a.num_q_heads + h * G + g) * a.splits + split) * rec;
      ws[2 + c_own] = acc_rot[k];
      ws[2 + D + c_own] = acc_win[k];
      if (c_own == 0) {
        ws[0] = m_run[g];
        ws[1] = l_run[g];
      }
    }
  }
}

template <int D, int ROT>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
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
  buf[c] = ar;
  __syncthreads();
  float o;
  if (ROT == TQ_ROT_FWHT) {
    block_fwht(buf, 1, D, c, D);
    o = apply_sign(buf[c] * rsqrtf(float(D)), sign_bit(a.params, kRoleValueRot, c));
  } else {
    const float* piv = reinterpret_cast<const float*>(a.params + kOffDense) + size_t(2) * D * D;
    o = 0.f;
    for (int j = 0; j < D; ++j) o = fmaf(piv[size_t(j) * D + c], buf[j], o);
  }
  a.out[row * D + c] = l > 0.f ? (o + aw) / l : 0.f;
}

template <int D, int ROT>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  const int H = a.cache.num_kv_heads;
  hipLaunchKernelGGL((decode_split_kernel<D, ROT>), dim3(a.num_seqs * H, a.splits), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D, ROT>), dim3(a.num_seqs * a.num_q_heads), dim3(D), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int launch_decode(const tq_config& cfg, const DecodeArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool dense = cfg.rotation == TQ_ROT_DENSE;
  switch (cfg.head_dim) {
    case 64: return dense ? launch<64, TQ_ROT_DENSE>(a, st) : launch<64, TQ_ROT_FWHT>(a, st);
    case 128: return dense ? launch<128, TQ_ROT_DENSE>(a, st) : launch<128, TQ_ROT_FWHT>(a, st);
    case 256: return dense ? launch<256, TQ_ROT_DENSE>(a, st) : launch<256, TQ_ROT_FWHT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tqi
