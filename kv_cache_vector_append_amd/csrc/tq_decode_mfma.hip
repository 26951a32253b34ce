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
// Three launches:
//   decode_prep: per (sequence, kv head), rotate and sketch the GQA group's
//     queries and store their fp8 operand rows in the workspace;
//   decode_split: one workgroup of NW wavefronts per (sequence, kv head,
//     context split).  Per block of 128 tokens the wavefronts score disjoint
//     pages, agree on the block maximum, write the fp8 parts of the softmax
//     weights to LDS in the value operand's order and each accumulates its
//     coordinate blocks of the value tiles.  The next block's page data is
//     requested as soon as the current block's registers are consumed.  One
//     extra split per (sequence, kv head) attends the fp16 recent window
//     exactly;
//   decode_combine: per (sequence, query head), merge the splits by
//     log-sum-exp, rotate the compressed part back once, add the window part,
//     normalise and store.
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

// bytes of one (sequence, kv head) entry of the query-operand region
__host__ __device__ constexpr int prep_stride(int d, int mk) { return (num_planes(mk) + 1) * (d / 128) * 2048 + 64; }

template <int BITS>
__device__ __forceinline__ uint32_t plane_word(const uint32_t* w, int i) {
  const int sub = odd_subset(BITS, i);
  uint32_t x = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b)
    if ((sub >> b) & 1) x ^= w[b];
  return x;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// reductions over the 16 lanes of a row: quad butterflies, then half-row and row mirrors
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}
__device__ __forceinline__ float row_value(float v, int row) {  // value held by row `row` (uniform within rows)
  const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return row == 0 ? a0 : row == 1 ? a1 : row == 2 ? a2 : a3;
}

// power of two f with max_abs * f in (128, 256]; 1 when max_abs == 0
__device__ __forceinline__ float fp8_range_scale(float max_abs) {
  if (!(max_abs > 0.f)) return 1.f;
  int e;
  frexpf(max_abs, &e);
  return ldexpf(1.f, 8 - e);
}

// fp4 element e of a converted word comes from bit fp4_elem_bit(e); inverse:
__host__ __device__ constexpr int fp4_bit_elem(int b) { return 8 * (b % 4) + b / 4; }

// N consecutive dwords from global memory (N-dword aligned), zeros when !ok
template <int N>
__device__ __forceinline__ void load_dwords(const uint32_t* p, bool ok, uint32_t* out) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const uint4 v = ok ? reinterpret_cast<const uint4*>(p)[q] : uint4{0u, 0u, 0u, 0u};
      out[4 * q] = v.x; out[4 * q + 1] = v.y; out[4 * q + 2] = v.z; out[4 * q + 3] = v.w;
    }
  } else if constexpr (N == 2) {
    const uint2 v = ok ? *reinterpret_cast<const uint2*>(p) : uint2{0u, 0u};
    out[0] = v.x; out[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q) out[q] = ok ? p[q] : 0u;
  }
}

__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

template <int NW>
__device__ __forceinline__ void block_sync() {
  if constexpr (NW > 1) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS traffic done; global loads may stay in flight
    __builtin_amdgcn_s_barrier();
  }
  lds_fence();
}

// ---------------------------------------------------------------------------- query operands
template <int D, int MK, int ROT>
__global__ __launch_bounds__(256) void decode_prep_kernel(DecodeArgs a) {
  constexpr int KP = num_planes(MK), KH = D / 128, T = 256;
  __shared__ float q_rot[kMaxG * D];
  __shared__ float q_sk[kMaxG * D];
  __shared__ float coef_k[16], qscale[2 * kMaxG];
  const int tid = threadIdx.x;
  const int H = a.cache.num_kv_heads;
  const int G = a.num_q_heads / H;
  const int s = blockIdx.x / H, hk = blockIdx.x % H;
  uint8_t* dst = reinterpret_cast<uint8_t*>(a.workspace) + size_t(blockIdx.x) * prep_stride(D, MK);
  if (tid < 16) coef_k[tid] = reinterpret_cast<const float*>(a.params + kOffKeyPlaneCoef)[tid];
  for (int i = tid; i < kMaxG * D; i += T) {
    const int g = i / D;
    q_rot[i] = g < G ? load_elem(a.q, a.q_dtype, (size_t(s) * a.num_q_heads + hk * G) * D + i) : 0.f;
  }
  __syncthreads();
  if (ROT == TQ_ROT_FWHT) {
    // qt = H_n D_K q;  qh = H D2 H_n D1 qt
    for (int i = tid; i < kMaxG * D; i += T) q_rot[i] = apply_sign(q_rot[i], sign_bit(a.params, kRoleKeyRot, i % D));
    __syncthreads();
    block_fwht(q_rot, kMaxG, D, tid, T);
    for (int i = tid; i < kMaxG * D; i += T) {
      q_rot[i] *= rsqrtf(float(D));
      q_sk[i] = apply_sign(q_rot[i], sign_bit(a.params, kRoleSketch1, i % D));
    }
    __syncthreads();
    block_fwht(q_sk, kMaxG, D, tid, T);
    for (int i = tid; i < kMaxG * D; i += T)
      q_sk[i] = apply_sign(q_sk[i] * rsqrtf(float(D)), sign_bit(a.params, kRoleSketch2, i % D));
    __syncthreads();
    block_fwht(q_sk, kMaxG, D, tid, T);
  } else {
    // qt = Pi_K q;  qh = G qt
    const float* pik = reinterpret_cast<const float*>(a.params + kOffDense);
    for (int i = tid; i < kMaxG * D; i += T) {
      const float* row = pik + size_t(i % D) * D;
      const float* x = q_rot + (i / D) * D;
      float acc = 0.f;
      for (int j = 0; j < D; ++j) acc = fmaf(row[j], x[j], acc);
      q_sk[i] = acc;
    }
    __syncthreads();
    for (int i = tid; i < kMaxG * D; i += T) q_rot[i] = q_sk[i];
    __syncthreads();
    const float* gm = pik + size_t(D) * D;
    for (int i = tid; i < kMaxG * D; i += T) {
      const float* row = gm + size_t(i % D) * D;
      const float* x = q_rot + (i / D) * D;
      float acc = 0.f;
      for (int j = 0; j < D; ++j) acc = fmaf(row[j], x[j], acc);
      q_sk[i] = acc;
    }
    __syncthreads();
  }
  // per-head power-of-two scales bringing the largest operand entry into (128, 256]
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
    reinterpret_cast<float*>(dst + (KP + 1) * KH * 2048)[tid] = 1.f / qscale[tid];
    reinterpret_cast<float*>(dst + (KP + 1) * KH * 2048)[kMaxG + tid] = 1.f / qscale[kMaxG + tid];
  }
  __syncthreads();
  // fp8 parts of a_S * qt (key planes) and of qh (QJL) as operand rows
  // [plane][half][row = 4 h + part][k].  Coordinate c sits in key word c / 32
  // at bit c % 32; word wd feeds half (KH == 2 ? wd & 1 : 0) at K group
  // (KH == 2 ? wd >> 1 : wd), fp4 element fp4_bit_elem(c % 32).
  for (int i = tid; i < (KP + 1) * kMaxG * D; i += T) {
    const int pl = i / (kMaxG * D), rem = i % (kMaxG * D), h = rem / D, c = rem % D;
    const float x = pl < KP ? q_rot[h * D + c] * coef_k[odd_subset(MK, pl)] * qscale[h]
                            : q_sk[h * D + c] * qscale[kMaxG + h];
    const uint32_t parts = fp8_split4(x);
    const int wd = c / 32;
    const int hf = KH == 2 ? (wd & 1) : 0;
    const int kg = KH == 2 ? (wd >> 1) : wd;
    const int k = 32 * kg + fp4_bit_elem(c % 32);
    uint8_t* row0 = dst + size_t((pl * KH + hf) * 16) * 128;
#pragma unroll
    for (int p = 0; p < 4; ++p) row0[(h * 4 + p) * 128 + k] = uint8_t(parts >> (8 * p));
  }
}

// ---------------------------------------------------------------------------- window split
// Positions [nc, L) from the fp16 ring: wavefront wv serves heads wv, wv + NW, ...
// with lanes holding coordinates r * 64 + lane.  Writes (max, denominator,
// sum_w p_w v_w) in the value's own (unrotated) basis.
template <int D, int NW>
__device__ void window_split(const DecodeArgs& a, float* ws, int s, int hk, int G, int slot, int nc, int L) {
  constexpr int R = D / 64;
  __shared__ float wsc[kMaxG][1024];
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads, W = cv.window;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = L - nc;
  const int rec = 2 + D, nrec = a.splits + 1;
  const uint16_t* kwin = cv.k_window + (size_t(slot) * H + hk) * W * D;
  const uint16_t* vwin = cv.v_window + (size_t(slot) * H + hk) * W * D;
  for (int g = wv; g < G; g += NW) {
    float q[R];
#pragma unroll
    for (int r = 0; r < R; ++r) q[r] = load_elem(a.q, a.q_dtype, (size_t(s) * a.num_q_heads + hk * G + g) * D + r * 64 + lane);
    float m = -INFINITY;
    for (int t = 0; t < nw; ++t) {
      const uint16_t* kr = kwin + size_t((nc + t) % W) * D;
      float dot = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) dot = fmaf(q[r], f16_bits_to_float(kr[r * 64 + lane]), dot);
      dot = wave_sum(dot) * a.scale;
      if (lane == 0) {
        wsc[g][t] = dot;
        if (a.logits) a.logits[(size_t(s) * a.num_q_heads + hk * G + g) * a.max_ctx + nc + t] = dot;
      }
      m = fmaxf(m, dot);
    }
    float l = 0.f, acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    for (int t = 0; t < nw; ++t) {
      const float p = __expf(wsc[g][t] - m);
      l += p;
      const uint16_t* vr = vwin + size_t((nc + t) % W) * D;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = fmaf(p, f16_bits_to_float(vr[r * 64 + lane]), acc[r]);
    }
    float* w0 = ws + ((size_t(s) * a.num_q_heads + hk * G + g) * nrec + a.splits) * rec;
    if (lane == 0) {
      w0[0] = nw > 0 ? m : -INFINITY;
      w0[1] = l;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) w0[2 + r * 64 + lane] = acc[r];
  }
}

// ---------------------------------------------------------------------------- split kernel
template <int N>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* out) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[q];
      out[4 * q] = v.x; out[4 * q + 1] = v.y; out[4 * q + 2] = v.z; out[4 * q + 3] = v.w;
    }
  } else if constexpr (N == 3) {
    const uint3 v = *reinterpret_cast<const uint3*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z;
  } else if constexpr (N == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = v.x; out[1] = v.y;
  } else if constexpr (N == 6) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    const uint4 w = *reinterpret_cast<const uint4*>(p + 8);
    out[0] = v.x; out[1] = v.y; out[2] = w.x; out[3] = w.y; out[4] = w.z; out[5] = w.w;
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q) out[q] = reinterpret_cast<const uint32_t*>(p)[q];
  }
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int D, int MK, int BV, int NW>
__global__ __launch_bounds__(64 * NW, 2) void decode_split_kernel(DecodeArgs a, size_t part_offset) {
  constexpr int KP = num_planes(MK);   // key plane products
  constexpr int VP = num_planes(BV);   // value plane products
  constexpr int KH = D / 128;          // 128-coordinate halves of the score contraction
  constexpr int NCB = D / 16;          // 16-coordinate blocks of the value contraction
  constexpr int CBW = NCB / NW;        // coordinate blocks per wavefront
  constexpr int PPW = 8 / NW;          // pages scored per wavefront per block
  constexpr int KW = (MK + 1) * KH;    // key words per lane per page
  constexpr int VW = (CBW / 2) * BV;   // value words per lane per page
  static_assert(NCB % NW == 0 && 8 % NW == 0 && CBW % 2 == 0, "wavefront split");

  __shared__ __attribute__((aligned(16))) uint8_t w_parts[16 * 128];
  __shared__ float red[NW][8];
  __shared__ float fin[NW][kMaxG];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads;
  const int G = a.num_q_heads / H;
  const int s = blockIdx.x / H, hk = blockIdx.x % H;
  const int split = blockIdx.y;
  const size_t plane_bytes = size_t(kPage) * D / 8;
  const size_t kcode_bytes = (MK + 1) * plane_bytes;
  const size_t vcode_bytes = BV * plane_bytes;
  const int W = cv.window;

  const int slot = a.seq_slots[s];
  int L = a.ctx_len[s];
  if (slot < 0 || slot >= cv.max_seqs || L < 0) L = 0;
  if (L > cv.max_pages_per_seq * kPage) L = cv.max_pages_per_seq * kPage;
  if (L > a.max_ctx) L = a.max_ctx;
  const int nc = W > 0 ? max(0, L - W) : L;
  const int rec = 2 + D, nrec = a.splits + 1;
  float* ws = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.workspace) + part_offset);
  if (split == a.splits) {
    // the recent-token window, exactly: fp16 keys and values from the ring
    window_split<D, NW>(a, ws, s, hk, G, slot, nc, L);
    return;
  }
  const int t_begin = split * a.split_tokens;
  const int t_end = min(nc, t_begin + a.split_tokens);

  // query operands of this (sequence, kv head): lane (row r16, group g4)
  const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.workspace) + size_t(blockIdx.x) * prep_stride(D, MK);
  v8i qa[KP + 1][KH];
#pragma unroll
  for (int pl = 0; pl <= KP; ++pl)
#pragma unroll
    for (int hf = 0; hf < KH; ++hf) {
      const uint8_t* src = qp + size_t((pl * KH + hf) * 16 + r16) * 128;
      const uint4 lo = *reinterpret_cast<const uint4*>(src + 16 * g4);
      const uint4 hi = *reinterpret_cast<const uint4*>(src + 64 + 16 * g4);
      qa[pl][hf] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
  const float* qinv = reinterpret_cast<const float*>(qp + (KP + 1) * KH * 2048);
  const bool head_ok = g4 < G;
  const float inv_sm = qinv[g4], inv_sq = qinv[kMaxG + g4];
  const float qjl_c = kQjlConst / float(D);

  // page addressing: uniform page base + constant per-lane offsets
  const uint8_t* kbase = cv.k_pages + size_t(hk) * cv.key_block;
  const uint8_t* vbase = cv.v_pages + size_t(hk) * cv.value_block;
  const size_t kstride = size_t(H) * cv.key_block, vstride = size_t(H) * cv.value_block;
  const uint32_t k_off = uint32_t((r16 * (D / 32) + KH * g4) * (MK + 1) * 4);
  const uint32_t kn_off = uint32_t(kcode_bytes + 8 * r16);
  const uint32_t vn_off = uint32_t(vcode_bytes + 4 * r16);
  const uint32_t v_off = uint32_t(((NCB * r16 + CBW * wv) / 2) * BV * 4);
  const int* bt = cv.block_table + size_t(slot) * cv.max_pages_per_seq;
  auto page_id = [&](int pos0) {  // uniform physical page of the page starting at pos0 (0 if outside)
    int ph = pos0 < t_end ? bt[pos0 / kPage] : 0;
    ph = (ph >= 0 && ph < cv.num_pages) ? ph : 0;
    return uniform(ph);
  };
  auto page_ok = [&](int pos0) {
    if (pos0 >= t_end) return false;
    const int ph = bt[pos0 / kPage];
    return ph >= 0 && ph < cv.num_pages;
  };

  v4f acc[VP][CBW];
#pragma unroll
  for (int p = 0; p < VP; ++p)
#pragma unroll
    for (int c = 0; c < CBW; ++c) acc[p][c] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running maximum of head g4 (score layout)
  float l_part = 0.f;       // this lane's share of head g4's denominator, relative to m_run
  float sig_run = 0.f;      // power-of-two factor carried by the accumulators (0 = none yet)

  uint32_t kw[PPW][KW];
  float2 kn[PPW];
  float vn[PPW];
  uint32_t vw[2][VW];
  auto load_keys = [&](int tb) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      const uint8_t* kb = kbase + size_t(page_id(tb + (wv * PPW + j) * kPage)) * kstride;
      const uint8_t* vb = vbase + size_t(page_id(tb + (wv * PPW + j) * kPage)) * vstride;
      load_words<KW>(kb + k_off, kw[j]);
      kn[j] = *reinterpret_cast<const float2*>(kb + kn_off);
      vn[j] = *reinterpret_cast<const float*>(vb + vn_off);
    }
  };
  auto load_values = [&](int tb) {
    // lane group g4 reads pages 2 g4 and 2 g4 + 1 of the block
    int ph[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ph[j] = page_id(tb + j * kPage);
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const int mine = g4 == 0 ? ph[hp] : g4 == 1 ? ph[2 + hp] : g4 == 2 ? ph[4 + hp] : ph[6 + hp];
      load_words<VW>(vbase + size_t(mine) * vstride + v_off, vw[hp]);
    }
  };

  if (t_begin < t_end) {
    load_keys(t_begin);
    load_values(t_begin);
  }
  for (int tb = t_begin; tb < t_end; tb += kBlock) {
    const bool more = tb + kBlock < t_end;
    // ---------------------------------------------- scores of this wavefront's pages
    float sc[PPW], vnu[PPW];
    float loc_max = -INFINITY, loc_vmax = 0.f;
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      v4f dm = {0.f, 0.f, 0.f, 0.f}, dq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hf = 0; hf < KH; ++hf) {
        const uint32_t* w = kw[j] + hf * (MK + 1);
#pragma unroll
        for (int pl = 0; pl < KP; ++pl) {
          v8i bop = {0, 0, 0, 0, 0, 0, 0, 0};
          bits_to_fp4_pm1(plane_word<MK>(w, pl), bop);
          dm = mfma_f8_f4(qa[pl][hf], bop, dm);
        }
        v8i bq = {0, 0, 0, 0, 0, 0, 0, 0};
        bits_to_fp4_pm1(w[MK], bq);
        dq = mfma_f8_f4(qa[KP][hf], bq, dq);
      }
      const int pos0 = tb + (wv * PPW + j) * kPage;
      const int pos = pos0 + r16;
      // dm[i], dq[i]: part i of head g4 for token r16
      const float msum = fmaf(fmaf(fmaf(dm[3], 0.0625f, dm[2]), 0.0625f, dm[1]), 0.0625f, dm[0]);
      const float qsum = fmaf(fmaf(fmaf(dq[3], 0.0625f, dq[2]), 0.0625f, dq[1]), 0.0625f, dq[0]);
      const float est = kn[j].x * fmaf(kn[j].y * qjl_c, qsum * inv_sq, msum * inv_sm);
      const bool tok_ok = pos < t_end && page_ok(pos0);
      const bool valid = tok_ok && head_ok;
      sc[j] = valid ? a.scale * est : -INFINITY;
      vnu[j] = tok_ok ? vn[j] : 0.f;
      if (a.logits && valid) a.logits[(size_t(s) * a.num_q_heads + hk * G + g4) * a.max_ctx + pos] = sc[j];
      loc_max = fmaxf(loc_max, sc[j]);
      loc_vmax = fmaxf(loc_vmax, vnu[j]);
    }
    if (more) load_keys(tb + kBlock);
    // ---------------------------------------------- block maximum, weight range
    loc_max = max16(loc_max);
    loc_vmax = max16(loc_vmax);
    loc_vmax = fmaxf(fmaxf(row_value(loc_vmax, 0), row_value(loc_vmax, 1)),
                     fmaxf(row_value(loc_vmax, 2), row_value(loc_vmax, 3)));
    float blk_max = loc_max, blk_vmax = loc_vmax;
    if constexpr (NW > 1) {
      if (r16 == 0) red[wv][g4] = loc_max;
      if (lane == 0) red[wv][4] = loc_vmax;
      block_sync<NW>();
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        blk_max = fmaxf(blk_max, red[w2][g4]);
        blk_vmax = fmaxf(blk_vmax, red[w2][4]);
      }
    }
    const float m_new = fmaxf(m_run, blk_max);
    const float sig_blk = fp8_range_scale(blk_vmax);
    const float sig_new = sig_run > 0.f ? fminf(sig_run, sig_blk) : sig_blk;
    if (m_new != m_run) l_part *= (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
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
    // accumulator rescale, only when some head's maximum or the range moved
    // (value layout: column r16 = (head r16 / 4, part r16 % 4))
    if (__any((m_new != m_run) || (sig_new != sig_run && sig_run > 0.f))) {
      const float mo = row_value(m_run, r16 >> 2), mn = row_value(m_new, r16 >> 2);
      float alpha = (mn == -INFINITY || mo == mn) ? 1.f : __expf(mo - mn);
      if (sig_run > 0.f) alpha *= sig_new / sig_run;
#pragma unroll
      for (int p = 0; p < VP; ++p)
#pragma unroll
        for (int c = 0; c < CBW; ++c) acc[p][c] *= alpha;
    }
    m_run = m_new;
    sig_run = sig_new;
    block_sync<NW>();
    // ---------------------------------------------- value tiles of this wavefront
    {
      const uint8_t* src = w_parts + r16 * 128;
      const uint4 lo = *reinterpret_cast<const uint4*>(src + 16 * g4);
      const uint4 hi = *reinterpret_cast<const uint4*>(src + 64 + 16 * g4);
      const v8i wop = {int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      // operand row r16 of coordinate block CBW wv + c is coordinate NCB r16 + CBW wv + c
#pragma unroll
      for (int cp = 0; cp < CBW / 2; ++cp) {
        uint32_t we[4] = {0u, 0u, 0u, 0u}, wo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < BV; ++b) {
          const uint32_t A = vw[0][cp * BV + b], B = vw[1][cp * BV + b];
          we[b] = __builtin_amdgcn_perm(B, A, 0x05040100u);  // A.lo | B.lo << 16 (even coordinate)
          wo[b] = __builtin_amdgcn_perm(B, A, 0x07060302u);  // A.hi | B.hi << 16 (odd coordinate)
        }
#pragma unroll
        for (int p = 0; p < VP; ++p) {
          v8i ae = {0, 0, 0, 0, 0, 0, 0, 0}, ao = {0, 0, 0, 0, 0, 0, 0, 0};
          bits_to_fp4_pm1(plane_word<BV>(we, p), ae);
          bits_to_fp4_pm1(plane_word<BV>(wo, p), ao);
          acc[p][2 * cp] = mfma_f4_f8(ae, wop, acc[p][2 * cp]);
          acc[p][2 * cp + 1] = mfma_f4_f8(ao, wop, acc[p][2 * cp + 1]);
        }
      }
    }
    if (more) load_values(tb + kBlock);
    block_sync<NW>();
  }

  // ------------------------------------------------------------ partial results
  const float* coef_v = reinterpret_cast<const float*>(a.params + kOffValuePlaneCoef);
  const float l_w = sum16(l_part);
  float l = l_w;
  if constexpr (NW > 1) {
    if (r16 == 0) fin[wv][g4] = l_w;
    block_sync<NW>();
    l = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) l += fin[w2][g4];
  }
  if (wv == 0 && r16 == 0 && head_ok) {
    float* w0 = ws + ((size_t(s) * a.num_q_heads + hk * G + g4) * nrec + split) * rec;
    w0[0] = m_run;
    w0[1] = l;
  }
  // values: planes combine in-lane, parts across the lane quad (columns 4h..4h+3)
  const int ch = r16 >> 2, cq = r16 & 3;
  const float part_w = cq == 0 ? 1.f : cq == 1 ? 0.0625f : cq == 2 ? 0.00390625f : 0.000244140625f;
  const float inv_sig = sig_run > 0.f ? 1.f / sig_run : 0.f;
  float* wsh = ws + ((size_t(s) * a.num_q_heads + hk * G + ch) * nrec + split) * rec + 2;
  float cvals[VP];
#pragma unroll
  for (int p = 0; p < VP; ++p) cvals[p] = coef_v[odd_subset(BV, p)];
#pragma unroll
  for (int c = 0; c < CBW; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int p = 0; p < VP; ++p) v = fmaf(cvals[p], acc[p][c][i], v);
      v *= part_w;
      v += dpp<0xB1>(v);
      v += dpp<0x4E>(v);
      const int coord = NCB * (4 * g4 + i) + CBW * wv + c;
      if (cq == 0 && ch < G) wsh[coord] = v * inv_sig;
    }
}

// Merge the compressed splits of one (sequence, query head) by log-sum-exp,
// rotate their value sum back once, add the window's (already unrotated) sum,
// normalise and store.
template <int D, int ROT>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a, size_t part_offset) {
  __shared__ float buf[D];
  const int c = threadIdx.x;
  const size_t row = blockIdx.x;  // s * H_q + h
  const int rec = 2 + D, nrec = a.splits + 1;
  const float* ws = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.workspace) + part_offset) +
                    row * nrec * rec;
  float Mc = -INFINITY;
  for (int sp = 0; sp < a.splits; ++sp) Mc = fmaxf(Mc, ws[sp * rec]);
  const float Mw = ws[a.splits * rec];
  const float M = fmaxf(Mc, Mw);
  float l = 0.f, ar = 0.f, aw = 0.f;
  if (M != -INFINITY) {
    for (int sp = 0; sp < a.splits; ++sp) {
      const float m = ws[sp * rec];
      if (m == -INFINITY) continue;
      const float f = __expf(m - M);
      l = fmaf(ws[sp * rec + 1], f, l);
      ar = fmaf(ws[sp * rec + 2 + c], f, ar);
    }
    if (Mw != -INFINITY) {
      const float f = __expf(Mw - M);
      l = fmaf(ws[a.splits * rec + 1], f, l);
      aw = ws[a.splits * rec + 2 + c] * f;
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

template <int D, int MK, int BV, int ROT>
hipError_t launch_mfma(const DecodeArgs& a, hipStream_t st) {
  // one wavefront per work item unless its value tiles exceed 32 (128 accumulators)
  constexpr int tiles = num_planes(BV) * (D / 16);
  constexpr int NW = tiles <= 32 ? 1 : tiles <= 64 ? 2 : 4;
  const int H = a.cache.num_kv_heads;
  const size_t part_offset = decode_prep_bytes(D, a.num_seqs, H);
  hipLaunchKernelGGL((decode_prep_kernel<D, MK, ROT>), dim3(a.num_seqs * H), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_split_kernel<D, MK, BV, NW>), dim3(a.num_seqs * H, a.splits + 1), dim3(64 * NW), 0, st,
                     a, part_offset);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D, ROT>), dim3(a.num_seqs * a.num_q_heads), dim3(D), 0, st, a,
                     part_offset);
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

size_t decode_prep_bytes(int d, int num_seqs, int num_kv_heads) {
  // sized for the largest key bit width, 256-byte aligned
  const size_t b = size_t(num_seqs) * num_kv_heads * prep_stride(d, 3);
  return (b + 255) & ~size_t(255);
}

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
