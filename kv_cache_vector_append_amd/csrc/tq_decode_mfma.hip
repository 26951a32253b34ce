// Decode attention over the compressed cache on the matrix cores (gfx950).
//
// Same computation as the plain kernel in tq_decode.hip ([Design Study] =
// "TurboQuant Family Design Study for CPU and Browser WASM KV Caches",
// "Capacity model" and "CPU and WASM kernel design"; [Reconstruction] =
// "Mathematical Reconstruction, Lineage, and Accuracy Limits of TurboQuant and
// TurboVec", section 6 "The Asymmetric Unbiased Estimator"):
//   est_t = nu_t (<qt, c_K[idx_t]> + gamma_t sqrt(pi/2)/d <qh, 1 - 2 z_t>)
//   acc_rot = sum_t softmax_t nu_V,t c_V[idx_V,t],  out = T_V^T acc_rot (+ window)
// with both contractions on v_mfma_scale_f32_16x16x128_f8f6f4 (tq_mfma.h):
//
//   scores^T [16 (head, part) x 16 tokens] = Q [16 x 128 coords, fp8] x planes [128 coords x 16 tokens, fp4]
//     for every key bit-plane product (the codebook's odd multilinear terms,
//     weighted through Q) and for the QJL bits; one page per MFMA;
//   values^T [16 coords x 16 (head, part)] = planes^T [16 coords x 128 tokens, fp4] x W [128 tokens x 16, fp8]
//     for every value bit-plane product; 128 tokens (8 pages) per MFMA.
//
// decode_mfma_kernel: one workgroup of NW wavefronts per (sequence, kv head,
// context split), serving the whole GQA group so every packed byte is read
// once.  Per block of 128 tokens the wavefronts score disjoint pages, agree on
// the block maximum through LDS, write the fp8 parts of the softmax weights to
// LDS in the value operand's order, and each accumulates its coordinate
// blocks of the value tiles.  decode_window_combine merges the splits by
// log-sum-exp, adds the recent-token window exactly, and applies the inverse
// value rotation once per head.
#include "tq_device.h"
#include "tq_mfma.h"

namespace tqi {
namespace {

constexpr float kQjlConst = 1.2533141373155003f;  // sqrt(pi / 2)
constexpr int kBlock = 128;                      // tokens per block (8 pages)
constexpr int kPage = 16;
constexpr int kMaxG = 4;                         // query heads per kv head on this path

// Odd subsets of `bits` code bits (bitmasks), in plane order.
__host__ __device__ constexpr int odd_subset(int bits, int i) {
  return bits == 1 ? 1
       : bits == 2 ? (i == 0 ? 1 : 2)
       : bits == 3 ? (i < 3 ? (1 << i) : 7)
       : (i < 4 ? (1 << i) : (i == 4 ? 7 : i == 5 ? 11 : i == 6 ? 13 : 14));
}
__host__ __device__ constexpr int num_planes(int bits) { return 1 << (bits - 1); }

template <int BITS>
__device__ __forceinline__ uint32_t plane_word(const uint32_t (&w)[4], int i) {
  const int sub = odd_subset(BITS, i);
  uint32_t x = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b)
    if ((sub >> b) & 1) x ^= w[b];
  return x;
}

__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// power of two f with max_abs * f in (128, 256]; 1 when max_abs == 0
__device__ __forceinline__ float fp8_range_scale(float max_abs) {
  if (!(max_abs > 0.f)) return 1.f;
  int e;
  frexpf(max_abs, &e);
  return ldexpf(1.f, 8 - e);
}

// n consecutive 16-bit masks (n in 2, 4, 8, 16; 4 n-byte aligned) as one vector load
template <int N>
__device__ __forceinline__ void load_masks(const uint16_t* row, bool ok, uint32_t (&out)[N]) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "mask count");
  uint32_t w[N / 2];
  if (N == 2) {
    w[0] = ok ? *reinterpret_cast<const uint32_t*>(row) : 0u;
  } else if (N == 4) {
    const uint2 v = ok ? *reinterpret_cast<const uint2*>(row) : uint2{0u, 0u};
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < N / 8; ++q) {
      const uint4 v = ok ? reinterpret_cast<const uint4*>(row)[q] : uint4{0u, 0u, 0u, 0u};
      w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
  }
#pragma unroll
  for (int c = 0; c < N; ++c) out[c] = (w[c / 2] >> (16 * (c & 1))) & 0xffffu;
}

// fp4 element e of a converted word comes from bit fp4_elem_bit(e); inverse:
__host__ __device__ constexpr int fp4_bit_elem(int b) { return 8 * (b % 4) + b / 4; }

template <int D, int MK, int BV, int NW, int ROT>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int KP = num_planes(MK);   // key plane products
  constexpr int VP = num_planes(BV);   // value plane products
  constexpr int KH = D / 128;          // 128-coordinate halves of the score contraction
  constexpr int NCB = D / 16;          // 16-coordinate blocks of the value contraction
  constexpr int CBW = NCB / NW;        // coordinate blocks per wavefront
  constexpr int PPW = 8 / NW;          // pages scored per wavefront per block
  constexpr int THREADS = 64 * NW;
  static_assert(NCB % NW == 0 && 8 % NW == 0, "wavefront split");

  __shared__ float q_rot[kMaxG * D];
  __shared__ float q_sk[kMaxG * D];
  __shared__ __attribute__((aligned(16))) uint8_t q_parts[(KP + 1) * KH * 16 * 128];
  __shared__ __attribute__((aligned(16))) uint8_t w_parts[16 * 128];
  __shared__ float red[NW][8];
  __shared__ float coef_k[16], coef_v[16];
  __shared__ float qscale[2 * kMaxG];
  __shared__ float fin[NW][kMaxG];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads;
  const int G = a.num_q_heads / H;
  const int s = blockIdx.x / H, hk = blockIdx.x % H;
  const int split = blockIdx.y;
  const size_t plane_bytes = size_t(kPage) * D / 8;
  const int W = cv.window;

  const int slot = a.seq_slots[s];
  int L = a.ctx_len[s];
  if (slot < 0 || slot >= cv.max_seqs || L < 0) L = 0;
  if (L > cv.max_pages_per_seq * kPage) L = cv.max_pages_per_seq * kPage;
  if (L > a.max_ctx) L = a.max_ctx;
  const int nc = W > 0 ? max(0, L - W) : L;
  const int t_begin = split * a.split_tokens;
  const int t_end = min(nc, t_begin + a.split_tokens);

  // ------------------------------------------------------------ query preparation
  if (tid < 16) {
    coef_k[tid] = reinterpret_cast<const float*>(a.params + kOffKeyPlaneCoef)[tid];
    coef_v[tid] = reinterpret_cast<const float*>(a.params + kOffValuePlaneCoef)[tid];
  }
  for (int i = tid; i < kMaxG * D; i += THREADS) {
    const int g = i / D;
    q_rot[i] = g < G ? load_elem(a.q, a.q_dtype, (size_t(s) * a.num_q_heads + hk * G) * D + i) : 0.f;
  }
  __syncthreads();
  if (ROT == TQ_ROT_FWHT) {
    // qt = H_n D_K q;  qh = H D2 H_n D1 qt
    for (int i = tid; i < kMaxG * D; i += THREADS) q_rot[i] = apply_sign(q_rot[i], sign_bit(a.params, kRoleKeyRot, i % D));
    __syncthreads();
    block_fwht(q_rot, kMaxG, D, tid, THREADS);
    for (int i = tid; i < kMaxG * D; i += THREADS) {
      q_rot[i] *= rsqrtf(float(D));
      q_sk[i] = apply_sign(q_rot[i], sign_bit(a.params, kRoleSketch1, i % D));
    }
    __syncthreads();
    block_fwht(q_sk, kMaxG, D, tid, THREADS);
    for (int i = tid; i < kMaxG * D; i += THREADS)
      q_sk[i] = apply_sign(q_sk[i] * rsqrtf(float(D)), sign_bit(a.params, kRoleSketch2, i % D));
    __syncthreads();
    block_fwht(q_sk, kMaxG, D, tid, THREADS);
  } else {
    // qt = Pi_K q;  qh = G qt
    const float* pik = reinterpret_cast<const float*>(a.params + kOffDense);
    for (int i = tid; i < kMaxG * D; i += THREADS) {
      const float* row = pik + size_t(i % D) * D;
      const float* x = q_rot + (i / D) * D;
      float acc = 0.f;
      for (int j = 0; j < D; ++j) acc = fmaf(row[j], x[j], acc);
      q_sk[i] = acc;
    }
    __syncthreads();
    for (int i = tid; i < kMaxG * D; i += THREADS) q_rot[i] = q_sk[i];
    __syncthreads();
    const float* gm = pik + size_t(D) * D;
    for (int i = tid; i < kMaxG * D; i += THREADS) {
      const float* row = gm + size_t(i % D) * D;
      const float* x = q_rot + (i / D) * D;
      float acc = 0.f;
      for (int j = 0; j < D; ++j) acc = fmaf(row[j], x[j], acc);
      q_sk[i] = acc;
    }
    __syncthreads();
  }
  // per-head power-of-two scales bringing the largest fp8 operand into (128, 256]
  if (tid < kMaxG) {
    float cmax = 0.f;
    for (int i = 0; i < KP; ++i) cmax = fmaxf(cmax, fabsf(coef_k[odd_subset(MK, i)]));
    float qm = 0.f, qh = 0.f;
    for (int c = 0; c < D; ++c) {
      qm = fmaxf(qm, fabsf(q_rot[tid * D + c]));
      qh = fmaxf(qh, fabsf(q_sk[tid * D + c]));
    }
    qscale[tid] = fp8_range_scale(qm * cmax);
    qscale[kMaxG + tid] = fp8_range_scale(qh);
  }
  __syncthreads();
  // fp8 parts of a_S * qt (key planes) and of qh (QJL), laid out as
  // q_parts[plane][half][row = 4 h + part][k].  Coordinate c sits in 32-bit
  // key word c / 32 at bit c % 32; word wd feeds half (KH == 2 ? wd & 1 : 0)
  // at K group (KH == 2 ? wd >> 1 : wd), fp4 element fp4_bit_elem(c % 32).
  for (int i = tid; i < (KP + 1) * kMaxG * D; i += THREADS) {
    const int pl = i / (kMaxG * D), rem = i % (kMaxG * D), h = rem / D, c = rem % D;
    const float x = pl < KP ? q_rot[h * D + c] * coef_k[odd_subset(MK, pl)] * qscale[h]
                            : q_sk[h * D + c] * qscale[kMaxG + h];
    const uint32_t parts = fp8_split4(x);
    const int wd = c / 32;
    const int hf = KH == 2 ? (wd & 1) : 0;
    const int kg = KH == 2 ? (wd >> 1) : wd;
    const int k = 32 * kg + fp4_bit_elem(c % 32);
    uint8_t* dst = q_parts + size_t((pl * KH + hf) * 16) * 128;
#pragma unroll
    for (int p = 0; p < 4; ++p) dst[(h * 4 + p) * 128 + k] = uint8_t(parts >> (8 * p));
  }
  __syncthreads();
  // fp8 operands: lane (row r16, group g4) holds K indices fp8_elem_k(g4, e)
  v8i qa[KP + 1][KH];
#pragma unroll
  for (int pl = 0; pl <= KP; ++pl)
#pragma unroll
    for (int hf = 0; hf < KH; ++hf) {
      const uint8_t* src = q_parts + size_t((pl * KH + hf) * 16 + r16) * 128;
      const uint4 lo = *reinterpret_cast<const uint4*>(src + 16 * g4);
      const uint4 hi = *reinterpret_cast<const uint4*>(src + 64 + 16 * g4);
      qa[pl][hf] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
  // score layout: lane (token r16 of the page, head g4)
  const bool head_ok = g4 < G;
  const float inv_sm = 1.f / qscale[g4], inv_sq = 1.f / qscale[kMaxG + g4];
  const float qjl_c = kQjlConst / float(D);

  v4f acc[VP][CBW];
#pragma unroll
  for (int p = 0; p < VP; ++p)
#pragma unroll
    for (int c = 0; c < CBW; ++c) acc[p][c] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running maximum of head g4 (same in every lane of the head)
  float l_part = 0.f;       // this lane's share of head g4's denominator, relative to m_run
  float sig_run = 0.f;      // power-of-two factor the accumulators carry (0 = nothing yet)

  const int* bt = cv.block_table + size_t(slot) * cv.max_pages_per_seq;

  for (int tb = t_begin; tb < t_end; tb += kBlock) {
    // ---------------------------------------------- scores of this wavefront's pages
    float sc[PPW], vnu[PPW];
    float loc_max = -INFINITY, loc_vmax = 0.f;
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const int pos0 = tb + (wv * PPW + j) * kPage;
      const int pos = pos0 + r16;
      const int phys = pos0 < t_end ? bt[pos0 / kPage] : -1;
      const bool ok = phys >= 0 && phys < cv.num_pages;
      const uint8_t* kb = cv.k_pages + (size_t(ok ? phys : 0) * H + hk) * cv.key_block;
      const uint8_t* vb = cv.v_pages + (size_t(ok ? phys : 0) * H + hk) * cv.value_block;
      v4f dm = {0.f, 0.f, 0.f, 0.f}, dq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hf = 0; hf < KH; ++hf) {
        const int wd = KH == 2 ? 2 * g4 + hf : g4;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        uint32_t wq = 0u;
        if (ok) {
#pragma unroll
          for (int b = 0; b < MK; ++b)
            w[b] = reinterpret_cast<const uint32_t*>(kb + size_t(b) * plane_bytes + size_t(r16) * (D / 8))[wd];
          wq = reinterpret_cast<const uint32_t*>(kb + size_t(MK) * plane_bytes + size_t(r16) * (D / 8))[wd];
        }
#pragma unroll
        for (int pl = 0; pl < KP; ++pl) {
          v8i bop = {0, 0, 0, 0, 0, 0, 0, 0};
          bits_to_fp4_pm1(plane_word<MK>(w, pl), bop);
          dm = mfma_f8_f4(qa[pl][hf], bop, dm);
        }
        v8i bq = {0, 0, 0, 0, 0, 0, 0, 0};
        bits_to_fp4_pm1(wq, bq);
        dq = mfma_f8_f4(qa[KP][hf], bq, dq);
      }
      float knu = 0.f, kgam = 0.f, vn = 0.f;
      if (ok) {
        const float* kn = reinterpret_cast<const float*>(kb + size_t(MK + 1) * plane_bytes);
        knu = kn[r16];
        kgam = kn[kPage + r16];
        vn = reinterpret_cast<const float*>(vb + size_t(BV) * plane_bytes)[r16];
      }
      // dm[i], dq[i]: part i of head g4 for token r16
      const float msum = fmaf(fmaf(fmaf(dm[3], 0.0625f, dm[2]), 0.0625f, dm[1]), 0.0625f, dm[0]);
      const float qsum = fmaf(fmaf(fmaf(dq[3], 0.0625f, dq[2]), 0.0625f, dq[1]), 0.0625f, dq[0]);
      const float est = knu * fmaf(kgam * qjl_c, qsum * inv_sq, msum * inv_sm);
      const bool tok_ok = ok && pos < t_end;
      const bool valid = tok_ok && head_ok;
      sc[j] = valid ? a.scale * est : -INFINITY;
      vnu[j] = tok_ok ? vn : 0.f;
      if (valid && a.logits) a.logits[(size_t(s) * a.num_q_heads + hk * G + g4) * a.max_ctx + pos] = sc[j];
      loc_max = fmaxf(loc_max, sc[j]);
      loc_vmax = fmaxf(loc_vmax, vnu[j]);
    }
    // ---------------------------------------------- block maximum, weight range
    loc_max = max16(loc_max);
    loc_vmax = wave_max(loc_vmax);
    if (r16 == 0) red[wv][g4] = loc_max;
    if (lane == 0) red[wv][4] = loc_vmax;
    __syncthreads();
    float blk_max = -INFINITY, blk_vmax = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
      blk_max = fmaxf(blk_max, red[w2][g4]);
      blk_vmax = fmaxf(blk_vmax, red[w2][4]);
    }
    const float m_new = fmaxf(m_run, blk_max);
    const float sig_blk = fp8_range_scale(blk_vmax);
    const float sig_new = sig_run > 0.f ? fminf(sig_run, sig_blk) : sig_blk;
    const float al_s = (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
    l_part *= al_s;
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const float p = (m_new == -INFINITY) ? 0.f : __expf(sc[j] - m_new);
      l_part += p;
      const uint32_t parts = fp8_split4(p * vnu[j] * sig_new);
      const int t = (wv * PPW + j) * kPage + r16;
      const int k = 32 * (t / 32) + fp4_bit_elem(t % 32);
#pragma unroll
      for (int p4 = 0; p4 < 4; ++p4) w_parts[(g4 * 4 + p4) * 128 + k] = uint8_t(parts >> (8 * p4));
    }
    // accumulator rescale (value layout: column r16 = (head r16 / 4, part r16 % 4))
    const int src_lane = (r16 >> 2) * 16;
    const float mo = __shfl(m_run, src_lane), mn = __shfl(m_new, src_lane);
    float alpha = (mn == -INFINITY) ? 1.f : __expf(mo - mn);
    if (sig_run > 0.f) alpha *= sig_new / sig_run;
    m_run = m_new;
    sig_run = sig_new;
#pragma unroll
    for (int p = 0; p < VP; ++p)
#pragma unroll
      for (int c = 0; c < CBW; ++c) acc[p][c] *= alpha;
    __syncthreads();
    // ---------------------------------------------- value tiles of this wavefront
    {
      const uint8_t* src = w_parts + r16 * 128;
      const uint4 lo = *reinterpret_cast<const uint4*>(src + 16 * g4);
      const uint4 hi = *reinterpret_cast<const uint4*>(src + 64 + 16 * g4);
      const v8i wop = {int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      // lane group g4 reads pages 2 g4 and 2 g4 + 1 of the block; operand row r16
      // of coordinate block cb is coordinate NCB * r16 + cb
      uint32_t masks[2][BV][CBW];
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        const int pos0 = tb + (2 * g4 + hp) * kPage;
        const int phys = pos0 < t_end ? bt[pos0 / kPage] : -1;
        const bool ok = phys >= 0 && phys < cv.num_pages;
        const uint8_t* vb = cv.v_pages + (size_t(ok ? phys : 0) * H + hk) * cv.value_block;
#pragma unroll
        for (int b = 0; b < BV; ++b) {
          const uint16_t* row = reinterpret_cast<const uint16_t*>(vb + size_t(b) * plane_bytes) + NCB * r16 + CBW * wv;
          load_masks<CBW>(row, ok, masks[hp][b]);
        }
      }
#pragma unroll
      for (int c = 0; c < CBW; ++c) {
        uint32_t wb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < BV; ++b) wb[b] = masks[0][b][c] | (masks[1][b][c] << 16);
#pragma unroll
        for (int p = 0; p < VP; ++p) {
          v8i aop = {0, 0, 0, 0, 0, 0, 0, 0};
          bits_to_fp4_pm1(plane_word<BV>(wb, p), aop);
          acc[p][c] = mfma_f4_f8(aop, wop, acc[p][c]);
        }
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ partial results
  // denominator: sum l_part over the 16 lanes of head g4 in every wavefront
  const float l_w = sum16(l_part);
  if (r16 == 0) fin[wv][g4] = l_w;
  __syncthreads();
  const int rec = 2 + D;
  if (wv == 0 && r16 == 0 && head_ok) {
    float l = 0.f;
    for (int w2 = 0; w2 < NW; ++w2) l += fin[w2][g4];
    float* ws = a.workspace + ((size_t(s) * a.num_q_heads + hk * G + g4) * a.splits + split) * rec;
    ws[0] = m_run;
    ws[1] = l;
  }
  // values: planes combine in-lane, parts across the lane quad (columns 4h..4h+3)
  const int ch = r16 >> 2, cp = r16 & 3;
  const float part_w = cp == 0 ? 1.f : cp == 1 ? 0.0625f : cp == 2 ? 0.00390625f : 0.000244140625f;
  const float inv_sig = sig_run > 0.f ? 1.f / sig_run : 0.f;
  float* wsh = a.workspace + ((size_t(s) * a.num_q_heads + hk * G + ch) * a.splits + split) * rec + 2;
#pragma unroll
  for (int c = 0; c < CBW; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int p = 0; p < VP; ++p) v = fmaf(coef_v[odd_subset(BV, p)], acc[p][c][i], v);
      v *= part_w;
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      const int coord = NCB * (4 * g4 + i) + CBW * wv + c;
      if (cp == 0 && ch < G) wsh[coord] = v * inv_sig;
    }
}

// Merge the splits of one (sequence, kv head), add the window tokens exactly,
// rotate the value accumulator back once per head, normalise and store.
template <int D, int ROT>
__global__ __launch_bounds__(256) void decode_window_combine(DecodeArgs a) {
  constexpr int kT = 256;
  __shared__ float accr[kMaxG * D];
  __shared__ float qraw[kMaxG * D];
  __shared__ float wsc[kMaxG][1024];
  __shared__ float mM[kMaxG], lL[kMaxG], fM[kMaxG];
  const int tid = threadIdx.x;
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads, W = cv.window;
  const int G = a.num_q_heads / H;
  const int s = blockIdx.x / H, hk = blockIdx.x % H;
  const int slot = a.seq_slots[s];
  int L = a.ctx_len[s];
  if (slot < 0 || slot >= cv.max_seqs || L < 0) L = 0;
  if (L > cv.max_pages_per_seq * kPage) L = cv.max_pages_per_seq * kPage;
  if (L > a.max_ctx) L = a.max_ctx;
  const int nc = W > 0 ? max(0, L - W) : L;
  const int nw = L - nc;
  const int rec = 2 + D;
  const float* ws0 = a.workspace + (size_t(s) * a.num_q_heads + hk * G) * a.splits * rec;

  if (tid < G) {
    float M = -INFINITY;
    for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, ws0[(size_t(tid) * a.splits + sp) * rec]);
    float l = 0.f;
    if (M != -INFINITY)
      for (int sp = 0; sp < a.splits; ++sp) {
        const float* r = ws0 + (size_t(tid) * a.splits + sp) * rec;
        if (r[0] != -INFINITY) l = fmaf(r[1], __expf(r[0] - M), l);
      }
    mM[tid] = M;
    lL[tid] = l;
  }
  for (int i = tid; i < G * D; i += kT)
    qraw[i] = load_elem(a.q, a.q_dtype, (size_t(s) * a.num_q_heads + hk * G) * D + i);
  __syncthreads();
  for (int i = tid; i < G * D; i += kT) {
    const int g = i / D, c = i % D;
    float v = 0.f;
    if (mM[g] != -INFINITY)
      for (int sp = 0; sp < a.splits; ++sp) {
        const float* r = ws0 + (size_t(g) * a.splits + sp) * rec;
        if (r[0] != -INFINITY) v = fmaf(r[2 + c], __expf(r[0] - mM[g]), v);
      }
    accr[i] = v;
  }
  // exact window scores
  const uint16_t* kwin = W > 0 ? cv.k_window + (size_t(slot) * H + hk) * W * D : nullptr;
  const uint16_t* vwin = W > 0 ? cv.v_window + (size_t(slot) * H + hk) * W * D : nullptr;
  for (int i = tid; i < G * nw; i += kT) {
    const int g = i / nw, t = i % nw;
    const int pos = nc + t;
    const uint16_t* kr = kwin + size_t(pos % W) * D;
    float dot = 0.f;
    for (int c = 0; c < D; ++c) dot = fmaf(qraw[g * D + c], f16_bits_to_float(kr[c]), dot);
    wsc[g][t] = a.scale * dot;
    if (a.logits) a.logits[(size_t(s) * a.num_q_heads + hk * G + g) * a.max_ctx + pos] = wsc[g][t];
  }
  __syncthreads();
  if (tid < G) {
    float M2 = mM[tid];
    for (int t = 0; t < nw; ++t) M2 = fmaxf(M2, wsc[tid][t]);
    float l = (mM[tid] == -INFINITY) ? 0.f : lL[tid] * __expf(mM[tid] - M2);
    for (int t = 0; t < nw; ++t) {
      const float p = __expf(wsc[tid][t] - M2);
      wsc[tid][t] = p;
      l += p;
    }
    fM[tid] = (mM[tid] == -INFINITY || M2 == -INFINITY) ? 0.f : __expf(mM[tid] - M2);
    lL[tid] = l;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kT) accr[i] *= fM[i / D];
  __syncthreads();
  if (ROT == TQ_ROT_FWHT) {
    block_fwht(accr, G, D, tid, kT);
    for (int i = tid; i < G * D; i += kT)
      accr[i] = apply_sign(accr[i] * rsqrtf(float(D)), sign_bit(a.params, kRoleValueRot, i % D));
    __syncthreads();
  } else {
    const float* piv = reinterpret_cast<const float*>(a.params + kOffDense) + size_t(2) * D * D;
    for (int i = tid; i < G * D; i += kT) {
      const int g = i / D, c = i % D;
      float o = 0.f;
      for (int j = 0; j < D; ++j) o = fmaf(piv[size_t(j) * D + c], accr[g * D + j], o);
      qraw[i] = o;  // query no longer needed
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += kT) accr[i] = qraw[i];
    __syncthreads();
  }
  for (int i = tid; i < G * D; i += kT) {
    const int g = i / D, c = i % D;
    float o = accr[i];
    for (int t = 0; t < nw; ++t) o = fmaf(wsc[g][t], f16_bits_to_float(vwin[size_t((nc + t) % W) * D + c]), o);
    const float l = lL[g];
    a.out[(size_t(s) * a.num_q_heads + hk * G + g) * D + c] = l > 0.f ? o / l : 0.f;
  }
}

template <int D, int MK, int BV, int ROT>
hipError_t launch_mfma(const DecodeArgs& a, hipStream_t st) {
  constexpr int tiles = num_planes(BV) * (D / 16);
  constexpr int NW = tiles <= 16 ? 1 : tiles <= 32 ? 2 : tiles <= 64 ? 4 : 8;
  const int H = a.cache.num_kv_heads;
  hipLaunchKernelGGL((decode_mfma_kernel<D, MK, BV, NW, ROT>), dim3(a.num_seqs * H, a.splits), dim3(64 * NW), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_window_combine<D, ROT>), dim3(a.num_seqs * H), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int ROT>
hipError_t dispatch_bits(const DecodeArgs& a, hipStream_t st) {
  const int mk = a.key_mse_bits, bv = a.value_bits;
#define TQ_CASE(MK_, BV_) \
  if (mk == MK_ && bv == BV_) return launch_mfma<D, MK_, BV_, ROT>(a, st);
  TQ_CASE(1, 1) TQ_CASE(1, 2) TQ_CASE(1, 3) TQ_CASE(1, 4)
  TQ_CASE(2, 1) TQ_CASE(2, 2) TQ_CASE(2, 3) TQ_CASE(2, 4)
  TQ_CASE(3, 1) TQ_CASE(3, 2) TQ_CASE(3, 3) TQ_CASE(3, 4)
#undef TQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_mfma_supported(const tq_config& cfg) {
  return (cfg.head_dim == 128 || cfg.head_dim == 256) && cfg.num_q_heads / cfg.num_kv_heads <= kMaxG &&
         cfg.page_tokens == kPage && cfg.window <= 1024;
}

int launch_decode_mfma(const tq_config& cfg, const DecodeArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool dense = cfg.rotation == TQ_ROT_DENSE;
  if (cfg.head_dim == 128) return dense ? dispatch_bits<128, TQ_ROT_DENSE>(a, st) : dispatch_bits<128, TQ_ROT_FWHT>(a, st);
  if (cfg.head_dim == 256) return dense ? dispatch_bits<256, TQ_ROT_DENSE>(a, st) : dispatch_bits<256, TQ_ROT_FWHT>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace tqi
