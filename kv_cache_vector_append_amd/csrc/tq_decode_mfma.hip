// Decode attention over the compressed cache on the matrix cores (gfx950).
//
// Same computation as the plain kernel in tq_codec.hip ([Design Study] =
// "TurboQuant Family Design Study for CPU and Browser WASM KV Caches",
// "Capacity model" and "CPU and WASM kernel design"; [Reconstruction] =
// "Mathematical Reconstruction, Lineage, and Accuracy Limits of TurboQuant and
// TurboVec", section 6 "The Asymmetric Unbiased Estimator"):
//   est_t = nu_t (<qt, c_K[idx_t]> + gamma_t sqrt(pi/2)/d <qh, 1 - 2 z_t>)
//   acc_rot = sum_t softmax_t nu_V,t c_V[idx_V,t],  out = T_V^T acc_rot (+ window)
// The EXT variants take the extended stored formats with Lloyd-Max values
// (a Codec describes them): per-half bit counts and codebooks ([Design Study]
// "Packed format and complete bit accounting"), keys scored as
// s <qt, c_K[idx]> without the QJL plane ([Reconstruction] "The DRIVE/EDEN
// Mathematical Critique", "12. TurboVec Additions and Divergences"), and the
// key outlier sidecar, whose sum_j q[idx_j] val_j joins each score.
// with both contractions on v_mfma_scale_f32_16x16x128_f8f6f4 (tq_mfma.h):
//
//   scores^T [16 (head, part) x 16 tokens] = Q [16 x 128 coords, fp8] x planes [128 coords x 16 tokens, fp4]
//     for every key bit-plane product (the codebook's odd multilinear terms,
//     weighted through Q) and for the QJL bits; one page per MFMA;
//   values^T [16 coords x 16 (head, part)] = planes^T [16 coords x 128 tokens, fp4] x W [128 tokens x 16, fp8]
//     for every value bit-plane product; 128 tokens (8 pages) per MFMA.
//
// Launches:
//   decode_prep: per (sequence, kv head), rotate and sketch the GQA group's
//     queries and store their fp8 operand rows in the workspace (skipped
//     with the FWHT rotation and few splits per (sequence, kv head): each
//     split work item then builds its query operands itself, in LDS);
//   decode_split: one workgroup of NW wavefronts per (sequence, kv head,
//     context split).  Per block of 128 tokens the wavefronts score
//     disjoint pages, agree on the block maximum, write the fp8 parts of the
//     softmax weights to LDS in the value operand's order and each
//     accumulates its coordinate blocks of the value tiles.  The next block's
//     page data is requested as soon as the current block's registers are
//     consumed.  Up to four extra work items per (sequence, kv head) attend
//     the fp16 recent window exactly;
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

// bytes of one (sequence, kv head) entry of the query-operand region: the
// operand images, 256 bytes of scales and constants, and (EXT) the unrotated
// query of each head for the sidecar entries, as floats in logit units
__host__ __device__ constexpr int prep_stride(int d, int mk, bool ext) {
  return (num_planes(mk) + 1) * (d / 128) * 2048 + 256 + (ext ? 4 * kMaxG * d : 0);
}

template <int BITS>
__device__ __forceinline__ uint32_t plane_word(const uint32_t* w, int i) {
  const int sub = odd_subset(BITS, i);
  if (__builtin_popcount(sub) == 3) {
    const int b0 = __builtin_ctz(sub), b1 = __builtin_ctz(sub & (sub - 1)), b2 = 31 - __builtin_clz(sub);
    return __builtin_amdgcn_bitop3_b32(w[b0], w[b1], w[b2], kXor3);
  }
  uint32_t x = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b)
    if ((sub >> b) & 1) x ^= w[b];
  return x;
}

// The value operands of all plane products for one coordinate row: the
// single-bit planes converted once, the three-bit products as XORs of those.
template <int BITS>
__device__ __forceinline__ void value_operands(const uint32_t (&w)[4], v8i (&op)[num_planes(BITS)]) {
  v4i f[BITS];
#pragma unroll
  for (int b = 0; b < BITS; ++b) f[b] = bits_to_fp4_pm6_dwords(w[b]);
#pragma unroll
  for (int p = 0; p < num_planes(BITS); ++p) {
    const int sub = odd_subset(BITS, p);
    if (__builtin_popcount(sub) == 1) {
      op[p] = fp4_operand(f[__builtin_ctz(sub)]);
    } else {
      const int b0 = __builtin_ctz(sub), b1 = __builtin_ctz(sub & (sub - 1)), b2 = 31 - __builtin_clz(sub);
      op[p] = fp4_operand(fp4_pm6_product3(f[b0], f[b1], f[b2]));
    }
  }
}

// value of another lane of the same row (every pattern used reads inside the
// row, so the bound control never applies); folds into the consuming add/max
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
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

// exponent e of the power of two 2^e with max_abs 2^e in (128, 256] (0 when
// max_abs == 0), at most 114 so that 127 - e - 12 stays a valid E8M0 scale
__device__ __forceinline__ int fp8_range_exp(float max_abs) {
  if (!(max_abs > 0.f)) return 0;
  int e;
  frexpf(max_abs, &e);
  return min(8 - e, 114);
}

// fp4 element e of a converted word comes from bit fp4_elem_bit(e); inverse:
__host__ __device__ constexpr int fp4_bit_elem(int b) { return 8 * (b % 4) + b / 4; }

// Byte offset of row/column r, K index k inside a 2048-byte lane-major image of
// an fp8 operand: bytes 0..15 of every lane first (lane = 16 g + r, 16 bytes
// each), then bytes 16..31, so each half loads as one conflict-free 16-byte
// read per lane.
__host__ __device__ constexpr int fp8_image_offset(int r, int k) {
  return (k < 64 ? 0 : 1024) + (16 * ((k % 64) / 16) + r) * 16 + (k % 16);
}

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

// N consecutive dwords from global memory at a 4-byte aligned address (the
// extended layouts place groups and pairs at any word)
template <int N>
__device__ __forceinline__ void load_words_a4(const uint8_t* p, uint32_t* out) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4), aligned(4)));
  typedef uint32_t u2 __attribute__((ext_vector_type(2), aligned(4)));
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    const u4 v = *reinterpret_cast<const u4*>(p + 16 * q);
    out[4 * q] = v.x; out[4 * q + 1] = v.y; out[4 * q + 2] = v.z; out[4 * q + 3] = v.w;
  }
  constexpr int Q = N / 4 * 4;
  if constexpr (N % 4 >= 2) {
    const u2 v = *reinterpret_cast<const u2*>(p + 4 * Q);
    out[Q] = v.x; out[Q + 1] = v.y;
  }
  if constexpr (N % 2 == 1) out[N - 1] = *reinterpret_cast<const uint32_t*>(p + 4 * (N - 1));
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

// ---------------------------------------------------------------------------- debug capacity checks
// Reports, in the caller's status word, a slot outside the table, a length
// the call clamps, and every block-table entry outside the pool among the
// pages the compressed part of sequence s reads.  Run by the query-preparation
// workgroup of the sequence's first kv head, and only when a status word was
// given, so the split kernel carries no bookkeeping.
__device__ void check_sequence(const DecodeArgs& a, int s, int tid, int nthreads) {
  const CacheView& cv = a.cache;
  const int slot = a.seq_slots[s];
  const int L = a.ctx_len[s];
  const bool slot_ok = slot >= 0 && slot < cv.max_seqs;
  if (tid == 0) {
    report(cv.status, !slot_ok, TQ_STATUS_BAD_SLOT);
    report(cv.status, L < 0 || L > min(cv.max_pages_per_seq * kPage, a.max_ctx), TQ_STATUS_CAPACITY);
  }
  if (!slot_ok) return;
  const int Lc = max(0, min(L, min(cv.max_pages_per_seq * kPage, a.max_ctx)));
  const int nc = cv.window > 0 ? max(0, Lc - cv.window) : Lc;
  const int32_t* bt = cv.block_table + size_t(slot) * cv.max_pages_per_seq;
  for (int pg = tid; pg * kPage < nc; pg += nthreads) report(cv.status, uint32_t(bt[pg]) >= uint32_t(cv.num_pages),
                                                            TQ_STATUS_BAD_PAGE);
}

// ---------------------------------------------------------------------------- query operands
// Operand region of one (sequence, kv head): the lane-major fp8 images
// [plane][half] (rows 4 h + part), then a 256-byte tail of 32-bit words:
// [0, 16) the E8M0 scales of rows 4 h + p, [16, 20) the key-plane constants,
// [20, 24) the QJL constants of heads 0-3, [24, 28) each head's operand scale
// (used while the images are built).
template <int D, int MK>
__host__ __device__ constexpr int image_bytes() { return (num_planes(MK) + 1) * (D / 128) * 2048; }

// Rotated query qt = H_n D_K q of head h of the GQA group and its sketch
// qh = H D2 H_n D1 qt ([Reconstruction] section 6; H_n the orthonormal
// Walsh-Hadamard transform), in base-2 logit units (the softmax scale times
// log2(e), and the sketch also the QJL constant sqrt(pi/2)/d), to LDS rows
// q_rot[h] and q_sk[h]: zeros past the group, and no sketch for keys without
// the QJL plane.  EXT also keeps the unrotated query in logit units in raw[h]
// for the sidecar entries.  One wavefront per head, in two steps: the loads
// (query row and the three sign masks), then the transforms, so that a
// caller can issue other loads in between.
template <int D>
struct QueryRegs {
  float x[D / 64];
  uint32_t sgk[D / 64], sg1[D / 64], sg2[D / 64];
};
template <int D>
__device__ __forceinline__ void query_load(const DecodeArgs& a, size_t qrow0, int G, int h, int lane, QueryRegs<D>& q) {
  constexpr int R = D / 64;
  const size_t qb = (qrow0 + h) * D + lane;
  // one uniform dtype branch, every load in flight together
  if (h >= G) {
#pragma unroll
    for (int r = 0; r < R; ++r) q.x[r] = 0.f;
  } else if (a.q_dtype == TQ_F32) {
#pragma unroll
    for (int r = 0; r < R; ++r) q.x[r] = static_cast<const float*>(a.q)[qb + r * 64];
  } else {
    uint16_t qbits[R];
#pragma unroll
    for (int r = 0; r < R; ++r) qbits[r] = static_cast<const uint16_t*>(a.q)[qb + r * 64];
    const bool bf = a.q_dtype == TQ_BF16;
#pragma unroll
    for (int r = 0; r < R; ++r) q.x[r] = bf ? bf16_bits_to_float(qbits[r]) : f16_bits_to_float(qbits[r]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = r * 64 + lane;
    q.sgk[r] = sign_bit(a.params, kRoleKeyRot, c);
    q.sg1[r] = sign_bit(a.params, kRoleSketch1, c);
    q.sg2[r] = sign_bit(a.params, kRoleSketch2, c);
  }
}
template <int D, bool EXT>
__device__ __forceinline__ void query_finish(const DecodeArgs& a, QueryRegs<D>& q, int h, int lane, bool qjl, float* q_rot,
                                             float* q_sk, float* raw) {
  constexpr int R = D / 64;
  const float s2 = a.scale * 1.4426950408889634f;
  const float s2q = s2 * kQjlConst / float(D);
  float* x = q.x;
  float y[R];
  if constexpr (EXT) {
#pragma unroll
    for (int r = 0; r < R; ++r) raw[h * D + r * 64 + lane] = x[r] * s2;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = apply_sign(x[r], q.sgk[r]);
  wave_fwht<R>(q.x, lane);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    x[r] *= rsqrtf(float(D));
    y[r] = apply_sign(x[r], q.sg1[r]);
  }
  if (qjl) {
    wave_fwht<R>(y, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) y[r] = apply_sign(y[r] * rsqrtf(float(D)), q.sg2[r]);
    wave_fwht<R>(y, lane);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) y[r] = 0.f;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    q_rot[h * D + r * 64 + lane] = x[r] * s2;
    q_sk[h * D + r * 64 + lane] = y[r] * s2q;
  }
}
template <int D, bool EXT>
__device__ __forceinline__ void query_fwht(const DecodeArgs& a, size_t qrow0, int G, int h, int lane, bool qjl,
                                           float* q_rot, float* q_sk, float* raw) {
  QueryRegs<D> q;
  query_load<D>(a, qrow0, G, h, lane, q);
  query_finish<D, EXT>(a, q, h, lane, qjl, q_rot, q_sk, raw);
}

// Head h's operand constants (one wavefront): one power of two 2^e bringing
// the larger of its key-plane and QJL operands' largest entry into (128, 256]
// (the smaller operand keeps the four parts' precision far below the
// tolerance), undone by the score MFMA's per-row operand scale together with
// the part weight 16^-p; and the constants of the affine fp4 encoding of the
// key bits (coordinate c falls in element group c % 4): the sums of the
// operands over the coordinates with c % 4 < 3, which seed the accumulators.
// coef: the key-plane coefficients (EXT: lower half [0, 16), upper [16, 32));
// tail: the region's tail words.
// EXT: each half of the coordinates takes its own plane coefficients (zero
// for products of planes the half does not store).
template <int D, int MK, bool EXT>
__device__ __forceinline__ void head_constants(const float* q_rot, const float* q_sk, const float* coef, int h,
                                               int lane, uint32_t* tail) {
  constexpr int KP = num_planes(MK), R = D / 64;
  // per half (one half unless EXT): the sum and the largest magnitude of the
  // plane coefficients
  float csum[2] = {0.f, 0.f}, cmax[2] = {0.f, 0.f};
#pragma unroll
  for (int hf = 0; hf < (EXT ? 2 : 1); ++hf)
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const float cf = coef[16 * hf + odd_subset(MK, i)];
      csum[hf] += cf;
      cmax[hf] = fmaxf(cmax[hf], fabsf(cf));
    }
  float qm = 0.f, qh = 0.f, sm = 0.f, sh = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = r * 64 + lane;
    const int hf = EXT && c >= D / 2 ? 1 : 0;
    const float f = fabsf(fp4_affine_factor(c & 3));
    const float xr = q_rot[h * D + c], xs = q_sk[h * D + c];
    qm = fmaxf(qm, f * fabsf(xr) * (EXT ? cmax[hf] : 1.f));
    qh = fmaxf(qh, f * fabsf(xs));
    if ((c & 3) != 3) {
      sm += EXT ? xr * csum[hf] : xr;
      sh += xs;
    }
  }
  qm = wave_max(qm);
  qh = wave_max(qh);
  sm = wave_sum(sm);
  sh = wave_sum(sh);
  const int e = fp8_range_exp(fmaxf(EXT ? qm : qm * cmax[0], qh));
  if (lane < 4) tail[4 * h + lane] = uint32_t(kScaleOne - e - 4 * lane);
  if (lane == 0) {
    tail[16 + h] = __float_as_uint(EXT ? sm : sm * csum[0]);
    tail[16 + kMaxG + h] = __float_as_uint(sh);
    tail[16 + 2 * kMaxG + h] = __float_as_uint(ldexpf(1.f, e));
  }
}

// The operand images [plane][half], rows 4 h + part, from q_rot and q_sk
// with T threads.  Coordinate c sits in key word wd = c / 32 at bit c % 32;
// the word feeds half (KH == 2 ? wd & 1 : 0) at K group
// (KH == 2 ? wd >> 1 : wd), fp4 element fp4_bit_elem(c % 32).  Coordinates c
// and c + 4 (c % 8 < 4) land on adjacent bytes, so each thread splits such a
// pair at once and stores 16 bits per part row.
template <int D, int MK, bool EXT, int T>
__device__ __forceinline__ void build_images(const float* q_rot, const float* q_sk, const float* coef,
                                             const uint32_t* tail, uint8_t* img, int tid) {
  constexpr int KP = num_planes(MK), KH = D / 128;
  for (int i = tid; i < (KP + 1) * kMaxG * (D / 2); i += T) {
    const int pl = i / (kMaxG * D / 2), rem = i % (kMaxG * D / 2), h = rem / (D / 2), cp = rem % (D / 2);
    const int c = 8 * (cp >> 2) + (cp & 3);
    const float* src = (pl < KP ? q_rot : q_sk) + h * D;
    const int chf = EXT && c >= D / 2 ? 16 : 0;
    const float mul = fp4_affine_factor(c & 3) * __uint_as_float(tail[16 + 2 * kMaxG + h]) *
                      (pl < KP ? coef[chf + odd_subset(MK, pl)] : 1.f);
    uint32_t lo, hi;
    fp8_split4_pair(src[c] * mul, src[c + 4] * mul, 0u, 0u, lo, hi);
    const int wd = c / 32;
    const int hf = KH == 2 ? (wd & 1) : 0;
    const int kg = KH == 2 ? (wd >> 1) : wd;
    uint16_t* im = reinterpret_cast<uint16_t*>(img + (pl * KH + hf) * 2048 +
                                               fp8_image_offset(4 * h, 32 * kg + fp4_bit_elem(c % 32)));
    im[0] = uint16_t(lo);
    im[8] = uint16_t(lo >> 16);
    im[16] = uint16_t(hi);
    im[24] = uint16_t(hi >> 16);
  }
}

// One workgroup per (sequence, kv head): the GQA group's rotated queries and
// sketches (FWHT: a wavefront per head; dense: the products qt = Pi_K q and
// qh = G Pi_K q of the whole group over 1024 threads), the heads' constants
// and the operand images, built in LDS and copied to the workspace in 16-byte
// pieces.  EXT stores the unrotated query after the tail for the sidecar
// entries.
template <int ROT>
__host__ __device__ constexpr int prep_threads() { return ROT == TQ_ROT_DENSE ? 1024 : 256; }
template <int D, int MK, int ROT, bool EXT>
__global__ __launch_bounds__(prep_threads<ROT>()) void decode_prep_kernel(DecodeArgs a) {
  // dense: 1024 threads, so that the matrix-vector products have enough
  // wavefronts to hide latency
  constexpr int T = prep_threads<ROT>();
  static_assert(T >= 64 * kMaxG, "a wavefront per query head of the group");
  constexpr int KQ = T / D;  // dense: slices of the contraction per output row
  // operand images and tail; before them (dense) the products' partial sums per slice
  constexpr int kImgBytes = image_bytes<D, MK>() + 256;
  constexpr int kRedBytes = ROT == TQ_ROT_DENSE ? 2 * KQ * kMaxG * D * 4 : 0;
  __shared__ __attribute__((aligned(16))) uint8_t img[kImgBytes > kRedBytes ? kImgBytes : kRedBytes];
  float* red = reinterpret_cast<float*>(img);
  uint32_t* tail = reinterpret_cast<uint32_t*>(img + image_bytes<D, MK>());
  __shared__ __attribute__((aligned(16))) float q_rot[kMaxG * D];
  __shared__ __attribute__((aligned(16))) float q_sk[kMaxG * D];
  __shared__ float coef_k[EXT ? 32 : 16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.cache.num_kv_heads;
  const int G = a.num_q_heads / H;
  const int s = blockIdx.x / H, hk = blockIdx.x % H;
  uint8_t* dst = reinterpret_cast<uint8_t*>(a.workspace) + size_t(blockIdx.x) * prep_stride(D, MK, EXT);
  float* dst_raw = reinterpret_cast<float*>(dst + kImgBytes);  // EXT only
  const bool qjl = !EXT || a.cache.codec.qjl;
  if (tid < (EXT ? 32 : 16))
    coef_k[tid] = reinterpret_cast<const float*>(a.params + kOffKeyPlaneCoef + (tid >= 16 ? kOffUpperHalf : 0))[tid % 16];
  if (a.cache.status != nullptr && hk == 0) check_sequence(a, s, tid, T);
  const size_t qrow0 = size_t(s) * a.num_q_heads + size_t(hk) * G;
  if constexpr (ROT == TQ_ROT_FWHT) {
    if (wv < kMaxG) query_fwht<D, EXT>(a, qrow0, G, wv, lane, qjl, q_rot, q_sk, dst_raw);
    __syncthreads();
  } else {
    // scores come out in base-2 logits: the softmax scale times log2(e) rides
    // on both query operands, and the QJL constant sqrt(pi/2)/d on the sketch
    // one.  qt and qh in one pass over q, from the transposed matrices Pi_K^T
    // and (G Pi_K)^T: thread (i, k) sums slice k of the products for output
    // coordinate i of the whole group, so that the threads of a wavefront read
    // consecutive entries of a matrix row (each entry is read once); the
    // slices meet in LDS.
    const float s2 = a.scale * 1.4426950408889634f;
    const float s2q = s2 * kQjlConst / float(D);
    for (int i = tid; i < kMaxG * D; i += T) {
      const int g = i / D;
      q_rot[i] = g < G ? load_elem(a.q, a.q_dtype, qrow0 * D + i) : 0.f;
      if constexpr (EXT) dst_raw[i] = q_rot[i] * s2;
    }
    __syncthreads();
    constexpr int J = D / KQ;  // contraction slice per thread
    const int i = tid % D, k = tid / D, k0 = k * J;
    const float* m0 = reinterpret_cast<const float*>(a.params + dense_t_offset(D, 0)) + size_t(k0) * D + i;
    const float* m1 = reinterpret_cast<const float*>(a.params + dense_t_offset(D, 1)) + size_t(k0) * D + i;
    float ar[kMaxG] = {0.f, 0.f, 0.f, 0.f}, as[kMaxG] = {0.f, 0.f, 0.f, 0.f};
    if (qjl) {
#pragma unroll 16
      for (int j = 0; j < J; ++j) {
        const float u = m0[size_t(j) * D], v = m1[size_t(j) * D];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
          const float x = q_rot[h * D + k0 + j];
          ar[h] = fmaf(u, x, ar[h]);
          as[h] = fmaf(v, x, as[h]);
        }
      }
    } else {
#pragma unroll 16
      for (int j = 0; j < J; ++j) {
        const float u = m0[size_t(j) * D];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) ar[h] = fmaf(u, q_rot[h * D + k0 + j], ar[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      red[(k * kMaxG + h) * D + i] = ar[h];
      red[((KQ + k) * kMaxG + h) * D + i] = as[h];
    }
    __syncthreads();
    for (int o = tid; o < kMaxG * D; o += T) {
      float vr = 0.f, vs = 0.f;
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        vr += red[q * kMaxG * D + o];
        vs += red[(KQ + q) * kMaxG * D + o];
      }
      q_rot[o] = vr * s2;
      q_sk[o] = vs * s2q;
    }
    __syncthreads();
  }
  if (wv < kMaxG) head_constants<D, MK, EXT>(q_rot, q_sk, coef_k, wv, lane, tail);
  __syncthreads();
  build_images<D, MK, EXT, T>(q_rot, q_sk, coef_k, tail, img, tid);
  __syncthreads();
  for (int i = tid; i < kImgBytes / 16; i += T)
    reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(img)[i];
}

// ---------------------------------------------------------------------------- recent-token window
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Positions [nc, L) from the fp16 ring, exactly: window item wi (of
// a.window_items) takes the 16-token blocks wi, wi + window_items, ... on
// one wavefront, with an online softmax over its blocks, and writes (max,
// denominator, sum_t p_t v_t) per query head, in the value's own (unrotated)
// basis, to record splits + wi.
//   scores: v_mfma_f32_16x16x32_f16 with rows 2h + part holding the query of
//     head h as two fp16 parts (hi + lo, after a power-of-two scale) and
//     columns the ring's fp16 keys of 16 tokens, so every product is exact and
//     sums carry fp32 precision;
//   values: lanes over coordinates, the block's weights broadcast through
//     `pbuf` (64 floats of LDS).
// Both score operands place coordinate 32 kc + 8 g + e at element e of lane
// group g of chunk kc, which pairs the same coordinate on both sides whatever
// the instruction's internal K order.  A block's ring rows are requested DP
// blocks ahead.
template <int D, int DP>
__device__ void window_part(const DecodeArgs& a, float* ws, int s, int hk, int G, int slot, int nc, int L,
                            int wi, float* pbuf) {
  constexpr int KC = D / 32, NP = D / 128;
  const int kStep = 16 * a.window_items;  // tokens between this item's blocks
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads, W = cv.window;
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
  const int nw = L - nc;
  const int rec = 2 + D, nrec = a.splits + kWindowRecords;
  const size_t qrow0 = size_t(s) * a.num_q_heads + size_t(hk) * G;
  float m[kMaxG], l[kMaxG], acc[kMaxG][2 * NP];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 2 * NP; ++j) acc[h][j] = 0.f;
  }
  if (nw > 16 * wi) {
    const uint16_t* kwin = cv.k_window + (size_t(slot) * H + hk) * W * D;
    const uint16_t* vwin = cv.v_window + (size_t(slot) * H + hk) * W * D;
    // query operand: row r16 = 2 h + part
    const int qh = r16 >> 1, part = r16 & 1;
    const bool qrow_ok = qh < G;
    float qv[KC][8];
    float qmax = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[kc][e] = qrow_ok ? load_elem(a.q, a.q_dtype, (qrow0 + qh) * D + 32 * kc + 8 * g4 + e) : 0.f;
        qmax = fmaxf(qmax, fabsf(qv[kc][e]));
      }
    qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
    qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
    // power of two bringing the head's largest entry into [256, 512)
    float qs = 1.f;
    if (qmax > 0.f) {
      int e;
      frexpf(qmax, &e);
      qs = ldexpf(1.f, 9 - e);
    }
    v8h qa[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qv[kc][e] * qs;
        const _Float16 hi = _Float16(x);
        qa[kc][e] = part == 0 ? hi : _Float16(x - float(hi));
      }
    // result lane (token r16, group g4 < 2): rows 4 g4 + i = heads 2 g4 + i / 2, parts i % 2
    const int h0 = 2 * g4;
    const float sc0 = a.scale / __shfl(qs, 2 * h0 & 15);  // rows 2 h hold head h's scale
    const float sc1 = a.scale / __shfl(qs, 2 * (h0 + 1) & 15);
    const bool ok0 = g4 < 2 && h0 < G, ok1 = g4 < 2 && h0 + 1 < G;

    // ring of DP blocks in registers: block b lives in slot b % DP and is
    // requested DP blocks before it is used (each step waits for the oldest
    // requests only)
    uint4 kb[DP][KC];
    uint32_t vv[DP][16][NP];
    // ring slot of window offset p < nw: (nc + p) mod W without a division
    // (nc mod W < W and p < W)
    const int s0 = nc % W;
    auto ring_row = [&](int p) { const int r = s0 + p; return r >= W ? r - W : r; };
    auto load_block = [&](int d, int t0) {  // rows past the window repeat its last row
      const uint16_t* kr = kwin + size_t(ring_row(min(t0 + r16, nw - 1))) * D + 8 * g4;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kb[d][kc] = *reinterpret_cast<const uint4*>(kr + 32 * kc);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint32_t* vr = reinterpret_cast<const uint32_t*>(vwin + size_t(ring_row(min(t0 + u, nw - 1))) * D);
#pragma unroll
        for (int c = 0; c < NP; ++c) vv[d][u][c] = vr[64 * c + lane];
      }
    };
#pragma unroll
    for (int d = 0; d < DP; ++d) load_block(d, 16 * wi + d * kStep);
    for (int tb = 16 * wi; tb < nw; tb += DP * kStep) {
#pragma unroll
      for (int d = 0; d < DP; ++d) {
        const int t0 = tb + d * kStep;
        if (t0 >= nw) break;
        v4f sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kc], __builtin_bit_cast(v8h, kb[d][kc]), sacc, 0, 0, 0);
        const int t = t0 + r16;
        const bool tok = t < nw;
        const float s0 = ok0 && tok ? (sacc[0] + sacc[1]) * sc0 : -INFINITY;
        const float s1 = ok1 && tok ? (sacc[2] + sacc[3]) * sc1 : -INFINITY;
        if (a.logits) {
          if (ok0 && tok) a.logits[(qrow0 + h0) * a.max_ctx + nc + t] = s0;
          if (ok1 && tok) a.logits[(qrow0 + h0 + 1) * a.max_ctx + nc + t] = s1;
        }
        // block maxima per head (rows 0 and 1 hold heads 0, 1 and 2, 3)
        const float b0 = max16(s0), b1 = max16(s1);
        const float bm[kMaxG] = {row_value(b0, 0), row_value(b1, 0), row_value(b0, 1), row_value(b1, 1)};
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
          const float mn = fmaxf(m[h], bm[h]);
          const float r = mn == m[h] ? 1.f : __expf(m[h] - mn);
          l[h] *= r;
#pragma unroll
          for (int j = 0; j < 2 * NP; ++j) acc[h][j] *= r;
          m[h] = mn;
        }
        const float m0 = g4 == 0 ? m[0] : m[2], m1 = g4 == 0 ? m[1] : m[3];
        const float p0 = s0 == -INFINITY ? 0.f : __expf(s0 - m0);
        const float p1 = s1 == -INFINITY ? 0.f : __expf(s1 - m1);
        if (g4 < 2) {
          pbuf[r16 * kMaxG + h0] = p0;
          pbuf[r16 * kMaxG + h0 + 1] = p1;
        }
        const float q0 = sum16(p0), q1 = sum16(p1);
        l[0] += row_value(q0, 0);
        l[1] += row_value(q1, 0);
        l[2] += row_value(q0, 1);
        l[3] += row_value(q1, 1);
        lds_fence();
        float4 pw[16];  // the block's weights, all requested before the first use
#pragma unroll
        for (int u = 0; u < 16; ++u) pw[u] = *reinterpret_cast<const float4*>(pbuf + u * kMaxG);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float4 p = pw[u];
          const float ph[kMaxG] = {p.x, p.y, p.z, p.w};
#pragma unroll
          for (int c = 0; c < NP; ++c) {
            const float v0 = f16_bits_to_float(uint16_t(vv[d][u][c] & 0xffffu));
            const float v1 = f16_bits_to_float(uint16_t(vv[d][u][c] >> 16));
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
              acc[h][2 * c] = fmaf(ph[h], v0, acc[h][2 * c]);
              acc[h][2 * c + 1] = fmaf(ph[h], v1, acc[h][2 * c + 1]);
            }
          }
        }
        lds_fence();
        // slot d is consumed: request this item's block DP steps ahead
        // (unconditional; past the window it repeats rows already read)
        load_block(d, min(t0 + DP * kStep, nw - 1));
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h >= G) break;
    float* w0 = ws + ((qrow0 + h) * nrec + a.splits + wi) * rec;
    if (lane == 0) {
      w0[0] = m[h];
      w0[1] = l[h];
    }
#pragma unroll
    for (int c = 0; c < NP; ++c)
      *reinterpret_cast<float2*>(w0 + 2 + 128 * c + 2 * lane) = make_float2(acc[h][2 * c], acc[h][2 * c + 1]);
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

// Registers per lane a split-kernel variant needs (estimate): value
// accumulators, query operands unless they sit in LDS, the next block's key
// words and norms, current and next value words, key-plane staging, and a
// working margin (scores, addresses) calibrated on the compiled kernels.
// Two wavefronts per SIMD leave 256.
constexpr int kRegBudget = 256;
constexpr int kRegMargin = 68;
// fmt: 0 the default format, 1 an extended one (EXT adds two sidecar words per
// scored page, the lanes' word offsets and the format's runtime fields), 2
// group-quantized values (GV adds each scored page's scale and zero words, kept
// twice, a tile's value words instead of a pair's, and the group sums).
constexpr int kExtMargin = 40;
__host__ __device__ constexpr int split_regs(int D, int MK, int BV, int NW, bool q_in_lds, int fmt = 0) {
  return num_planes(BV) * (D / 16 / NW) * 4 + (q_in_lds ? 0 : (num_planes(MK) + 1) * (D / 128) * 8) +
         (8 / NW) * ((MK + 1) * (D / 128) + 3) + (D / 16 / NW) * BV + num_planes(MK) * (D / 128) * 4 + kRegMargin +
         (fmt ? 2 * (8 / NW) + kExtMargin + (MK == 4 ? kExtMargin : 0) : 0) +
         (fmt == 2 ? 2 * (8 / NW) * (D / 32) + (D / 16 / NW) * BV + 2 * (D / 32) : 0);
}
__host__ __device__ constexpr bool split_shape_ok(int D, int NW) {
  return (D / 16) % NW == 0 && 8 % NW == 0 && ((D / 16) / NW) % 2 == 0;
}
__host__ __device__ constexpr bool split_fits(int D, int MK, int BV, int NW, bool q_in_lds, int fmt = 0) {
  return split_shape_ok(D, NW) && split_regs(D, MK, BV, NW, q_in_lds, fmt) <= kRegBudget;
}
// Wavefronts resident per SIMD.  With three or four value bits at d = 128 the
// work of a block divides over four wavefronts that each fit in 168 registers
// (query operands read from LDS), so three share a SIMD and hide each other's
// latencies.  The other variants need up to 256 registers and run two per
// SIMD: at d = 128 with at most two value bits one wavefront per work item
// measured faster than four at four per SIMD, whose recent-token window then
// runs on one of the four.
__host__ __device__ constexpr int split_occupancy(int D, int MK, int BV, int fmt = 0) {
  return D == 128 && BV > 2 && !fmt ? 3 : 2;
}
// Variants where the estimate above is too optimistic (the compiled loop
// spills at the estimated count) and the wavefront count that compiles clean;
// and the default format at d = 256 with 2-bit key codes and 2-bit values,
// where four wavefronts per item (half the items, each twice as long)
// measured 5% faster than the two that fit.
__host__ __device__ constexpr int split_waves_override(int D, int MK, int BV, int fmt = 0) {
  return split_occupancy(D, MK, BV, fmt) > 2 ? 4
       : D == 256 && MK == 1 && BV == 3       ? 4
       : D == 256 && MK == 2 && BV == 4       ? 8
       : D == 256 && MK == 2 && BV == 2 && !fmt ? 4
                                              : 0;
}
// wavefronts per work item: the fewest whose registers fit two wavefronts per SIMD
__host__ __device__ constexpr int split_waves(int D, int MK, int BV, int fmt = 0) {
  return split_waves_override(D, MK, BV, fmt) ? split_waves_override(D, MK, BV, fmt)
       : split_fits(D, MK, BV, 1, true, fmt) ? 1 : split_fits(D, MK, BV, 2, true, fmt) ? 2
       : split_fits(D, MK, BV, 4, true, fmt) || !split_shape_ok(D, 8) ? 4 : 8;
}
// query operands stay in registers when they fit, else each MFMA reads them from LDS
__host__ __device__ constexpr bool split_q_in_lds(int D, int MK, int BV, int fmt = 0) {
  return split_occupancy(D, MK, BV, fmt) > 2 ? true : !split_fits(D, MK, BV, split_waves(D, MK, BV, fmt), false, fmt);
}

// With the FWHT rotation and few splits per (sequence, kv head) the split
// work items build their query operands themselves: the transforms then cost
// less than a launch and its workspace traffic.  With many splits per
// (sequence, kv head) every one would repeat them, on SIMDs the score and
// value work already keeps busy, so one preparation launch serves them all;
// the dense rotation's products read two d x d matrices and always take that
// launch.
constexpr int kFusedQueryMaxSplits = 4;
__host__ __device__ constexpr bool split_builds_query(int rot, int splits) {
  return rot == TQ_ROT_FWHT && splits <= kFusedQueryMaxSplits;
}

// Re-base a head's reference maximum only when a block's maximum exceeds it by
// more than this (weights stay below e^20; fp32 sums keep their range).
constexpr float kRebase = 28.f;  // base-2 logits: weights stay below 2^28 of the reference
constexpr float kLn2 = 0.6931471805599453f;

// EXT (the extended formats with Lloyd-Max values; MK and BV are the larger
// half's bit counts): lanes read their key groups and value pairs at the
// Codec's word offsets, lanes of the lower half (lane groups 0-1 of the
// scores, coordinate rows 0-7 of the values) ignore the planes they do not
// store (their plane coefficients are zero), the QJL plane is each group's
// last, scale-corrected keys skip it, and sidecar records are staged in LDS
// and added to the scores.
//
// GV (group-quantized values, with EXT): a value tile's 16 operand rows are 16
// consecutive coordinates, so that a tile lies in one 32-coordinate group and
// takes that group's weight operand p_t scale_{t,g}; codes are linear in their
// bits, so only the single-bit planes are multiplied:
//   sum_t p_t v_{t,c} = sum_t p_t zero_{t,g} + (2^b - 1)/2 sum_t p_t scale_{t,g}
//                       - sum_j 2^(j-1) sum_t p_t scale_{t,g} s_{j,t,c},  s = 1 - 2 bit,
// the first two sums kept per (head, group) in registers; the result stays in
// the value's own basis (no inverse rotation in the merge).
template <int D, int MK, int BV, int NW, bool QL, int OCC, bool EXT, bool GV, bool FQ>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC))) void decode_split_kernel(DecodeArgs a, size_t part_offset) {
  static_assert(!GV || EXT, "group-quantized values are an extended format");
  constexpr int KP = num_planes(MK);   // key plane products
  constexpr int VP = GV ? BV : num_planes(BV);  // value plane products (GV: single planes)
  constexpr int KH = D / 128;          // 128-coordinate halves of the score contraction
  constexpr int NCB = D / 16;          // 16-coordinate blocks of the value contraction
  constexpr int CBW = NCB / NW;        // coordinate blocks per wavefront
  constexpr int PPW = 8 / NW;          // pages scored per wavefront per block
  constexpr int KW = (MK + 1) * KH;    // key words per lane per page
  constexpr int VW = (GV ? CBW : CBW / 2) * BV;  // value words per lane per page pair
  constexpr int NG = D / kGroup;       // GV: scale / zero groups per token
  // scheduling fences between page pairs of the scores, only where the extra
  // pages in flight would spill (d = 256, 3 key MSE bits, 2 value bits);
  // elsewhere the compiler interleaves more pages across the chained MFMAs
  constexpr bool kPageFence = D == 256 && MK == 3 && BV == 2;
  constexpr bool kPlaneOuter = QL && PPW <= 4;  // eight pages of accumulators would spill
  constexpr bool kRollKeys = !kPlaneOuter;  // key pages re-requested one by one
  static_assert(NCB % NW == 0 && 8 % NW == 0 && CBW % 2 == 0, "wavefront split");

  __shared__ __attribute__((aligned(16))) uint8_t w_img[GV ? NG * 2048 : 2048];   // softmax-weight operand(s)
  __shared__ float gsum[GV ? NW * kMaxG * NG * 2 : 1];  // GV: per-wavefront zero and scale sums
  // query operands (FQ: with their tail, built here from the rotated queries and sketches)
  __shared__ __attribute__((aligned(16))) uint8_t q_img[QL || FQ ? image_bytes<D, MK>() + (FQ ? 256 : 0) : 16];
  __shared__ __attribute__((aligned(16))) float q_rs[FQ ? 2 * kMaxG * D : 1];
  __shared__ float coef_k[FQ ? 32 : 1];
  __shared__ float red[NW][8];
  __shared__ float fin[NW][kMaxG];
  constexpr int kSideWords = 8;  // record stride in LDS: two words per lane group
  static_assert((1 + kMaxOutliers + 1 + 2 * kMaxOutliers + 3) / 4 <= kSideWords, "sidecar record");
  __shared__ float q_raw[EXT ? kMaxG * D : 1];                        // unrotated queries (sidecar)
  __shared__ uint32_t side_lds[EXT ? 8 * kPage * kSideWords : 1];     // the block's sidecar records

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wvu = NW > 1 ? uniform(wv) : 0;  // wavefront index as a scalar
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
  const int rec = 2 + D, nrec = a.splits + kWindowRecords;
  float* ws = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.workspace) + part_offset);
  const int t_begin = split * a.split_tokens;
  const int t_end = min(nc, t_begin + a.split_tokens);
  // the window_items items after the last split attend the recent-token
  // window, exactly, from the fp16 ring (first wavefront, in the weight
  // operand's LDS), so that it runs beside the compressed splits instead of
  // after one of them
  if (split >= a.splits) {
    // ring depth: as many 16-token blocks in flight as the registers allow
    constexpr int kWinDepth = D == 128 && OCC == 2 ? 2 : 1;
    if (wv == 0)
      window_part<D, kWinDepth>(a, ws, s, hk, G, slot, nc, L, split - a.splits, reinterpret_cast<float*>(w_img));
    return;
  }

  // query operands of this (sequence, kv head), lane-major images with their
  // tail: built here (FQ) or read from the workspace
  const Codec& cd = cv.codec;
  const bool qjl = !EXT || cd.qjl;
  const int n_side = EXT ? cd.outliers : 0;          // sidecar entries per record
  const int side_words = EXT ? cd.side_bytes / 4 : 0;
  // FQ: the group's query rows, sign masks and plane coefficients are
  // requested here, the first block's pages after them, and the operands are
  // built while the pages are in flight (a wavefront per head)
  constexpr int HPW = (kMaxG + NW - 1) / NW;  // query heads per wavefront
  QueryRegs<D> qreg[FQ ? HPW : 1];
  float coef_r = 0.f;
  const uint8_t* qp;
  if constexpr (FQ) {
    const size_t qrow0 = size_t(s) * a.num_q_heads + size_t(hk) * G;
    if (tid < (EXT ? 32 : 16))
      coef_r = reinterpret_cast<const float*>(a.params + kOffKeyPlaneCoef + (tid >= 16 ? kOffUpperHalf : 0))[tid % 16];
#pragma unroll
    for (int i = 0; i < HPW; ++i)
      if (wvu + i * NW < kMaxG) query_load<D>(a, qrow0, G, wvu + i * NW, lane, qreg[i]);
    qp = q_img;
  } else {
    qp = reinterpret_cast<const uint8_t*>(a.workspace) + size_t(blockIdx.x) * prep_stride(D, MK, EXT);
  }
  v8i qa[QL ? 1 : KP + 1][QL ? 1 : KH];
  auto qop = [&](int pl, int hf) -> v8i {
    if constexpr (QL) {
      const uint8_t* img = q_img + (pl * KH + hf) * 2048;
      const uint4 lo = reinterpret_cast<const uint4*>(img)[lane];
      const uint4 hi = reinterpret_cast<const uint4*>(img + 1024)[lane];
      return v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    } else {
      return qa[pl][hf];
    }
  };
  // per-row operand scales of the query images (lane r16 scales row r16) and
  // the affine constants of head g4, which seed the score accumulators (read
  // once the operands are in place)
  const bool head_ok = g4 < G;
  int sa = 0;
  float k_m = 0.f, k_q = 0.f;

  // page addressing: uniform page base + constant per-lane offsets.  Page ids
  // come through the scalar data cache (uniform addresses in the constant
  // address space), so waiting for them never waits for page data in flight.
  const uint8_t* kbase = cv.k_pages + size_t(hk) * cv.key_block;
  const uint8_t* vbase = cv.v_pages + size_t(hk) * cv.value_block;
  const size_t kstride = size_t(H) * cv.key_block, vstride = size_t(H) * cv.value_block;
  uint32_t k_off = uint32_t((r16 * (D / 32) + KH * g4) * (MK + 1) * 4);
  uint32_t k_off1 = k_off + (MK + 1) * 4;  // second 32-coordinate group of the lane (d = 256)
  uint32_t kn_off = uint32_t(kcode_bytes + 8 * r16);
  uint32_t vn_off = uint32_t(vcode_bytes + 4 * r16);
  uint32_t v_off = uint32_t(((NCB * r16 + CBW * wvu) / 2) * BV * 4);
  uint32_t v_pair = 0;      // EXT: bytes between the lane's consecutive value pairs
  int q_word = MK;          // EXT: the lane's QJL word among its group's words
  uint32_t side_off = 0;    // EXT: this lane's word of its token's sidecar record
  uint32_t gv_off[GV ? CBW : 1];  // GV: the words of this lane's coordinate pair in each of its tiles
  if constexpr (EXT) {
    const int kh = g4 >= 2 ? 1 : 0;  // score lane groups 2-3 hold upper-half coordinates
    const int vh = r16 >= 8 ? 1 : 0;  // value rows 8-15 likewise
    k_off = uint32_t((r16 * cd.key_row_words + key_group_word(cd, KH * g4, D)) * 4);
    k_off1 = uint32_t((r16 * cd.key_row_words + key_group_word(cd, KH * g4 + (KH - 1), D)) * 4);
    kn_off = uint32_t(cd.key_norm_off + 8 * r16);
    vn_off = uint32_t(cd.value_tail_off + 4 * r16);
    v_off = uint32_t(value_pair_word(cd, (NCB * r16 + CBW * wvu) / 2, D) * 4);
    v_pair = uint32_t(cd.vbits[vh] * 4);
    q_word = cd.kbits[kh];
    side_off = uint32_t(cd.key_side_off + r16 * cd.side_bytes + 4 * g4);
    if constexpr (GV) {
      // tile CBW wv + c holds coordinates 16 (CBW wv + c) + row; the lane's row is r16
#pragma unroll
      for (int c = 0; c < CBW; ++c)
        gv_off[c] = uint32_t(value_pair_word(cd, (16 * (CBW * wvu + c) + r16) / 2, D) * 4);
      vn_off = uint32_t(cd.value_tail_off + r16 * NG * 4);  // the token's (scale, zero) pairs
    }
  }
  typedef const int __attribute__((address_space(4))) const_int;
  const const_int* bt = (const const_int*)(cv.block_table + size_t(slot) * cv.max_pages_per_seq);
  // Physical pages of the 8 pages of the block starting at tb (-1 outside
  // [t_begin, t_end) or when invalid): one 32-byte scalar load when the
  // block-table row holds 8 entries from there, else entry by entry.
  int nid[8], nkid[PPW];
  auto fetch_ids = [&](int tb) {
    const int p0 = tb / kPage;
    if (p0 + 8 <= cv.max_pages_per_seq) {
      typedef int ids8 __attribute__((ext_vector_type(8), aligned(4)));
      typedef const ids8 __attribute__((address_space(4))) const_ids8;
      const ids8 v = *(const const_ids8*)(bt + p0);
#pragma unroll
      for (int j = 0; j < 8; ++j) nid[j] = v[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) nid[j] = p0 + j < cv.max_pages_per_seq ? bt[p0 + j] : -1;
    }
    // this wavefront's scored pages (its own scalar load: selecting from nid
    // by wavefront would become a table in scratch memory)
    if constexpr (NW == 1) {
#pragma unroll
      for (int j = 0; j < PPW; ++j) nkid[j] = nid[j];
    } else {
      const int q0 = p0 + wvu * PPW;
#pragma unroll
      for (int j = 0; j < PPW; ++j) nkid[j] = q0 + j < cv.max_pages_per_seq ? bt[q0 + j] : -1;
    }
  };
  // validity, applied where the ids are first used (so that the scalar loads
  // stay in flight through the scores); pages past the split's end need no
  // test here, their tokens fail the position test
  auto checked = [&](int id) { return uint32_t(id) < uint32_t(cv.num_pages) ? id : -1; };

  v4f acc[VP][CBW];
#pragma unroll
  for (int p = 0; p < VP; ++p)
#pragma unroll
    for (int c = 0; c < CBW; ++c) acc[p][c] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -1e30f;     // reference maximum of head g4 (score layout, base-2 logits); finite so
                            // that exp2(-inf - m_ref) = 0
  float l_part = 0.f;       // this lane's share of head g4's denominator, relative to m_ref
  // GV: this lane's shares of sum_t p_t zero_{t,g} and sum_t p_t scale_{t,g} for head g4
  float zacc[GV ? NG : 1], sacc[GV ? NG : 1];
#pragma unroll
  for (int g = 0; g < (GV ? NG : 1); ++g) zacc[g] = sacc[g] = 0.f;

  int kid[PPW];  // page ids of the scored pages of the block being loaded
  uint32_t kw[PPW][KW];
  float2 kn[PPW];
  float vn[PPW];
  uint32_t sw[EXT ? PPW : 1][2];  // EXT: sidecar words g4 and g4 + 4 of the lane's token record
  uint32_t gsz[GV ? PPW : 1][GV ? NG : 1];  // GV: the lane's token's (fp16 scale, fp16 zero) per group
  uint32_t vw[2][VW];  // value words of the block
  auto load_key_page = [&](int j) {
    kid[j] = checked(nkid[j]);
    const int ph = max(kid[j], 0);
    const uint8_t* kb = kbase + size_t(ph) * kstride;
    const uint8_t* vb = vbase + size_t(ph) * vstride;
    // uniform base + 32-bit lane offset, kept inside the loop so that the
    // loads take the scalar-base addressing form (no 64-bit vector adds)
    uint32_t ko = k_off, kno = kn_off, vno = vn_off;
    asm volatile("" : "+v"(ko), "+v"(kno), "+v"(vno));
    if constexpr (EXT) {
      uint32_t ko1 = k_off1, so = side_off;
      asm volatile("" : "+v"(ko1), "+v"(so));
      load_words_a4<MK + 1>(kb + ko, kw[j]);
      if constexpr (KH == 2) load_words_a4<MK + 1>(kb + ko1, kw[j] + (MK + 1));
      if (n_side > 0) {
        sw[j][0] = g4 < side_words ? *reinterpret_cast<const uint32_t*>(kb + so) : 0u;
        sw[j][1] = g4 + 4 < side_words ? *reinterpret_cast<const uint32_t*>(kb + so + 16) : 0u;
      }
    } else {
      load_words<KW>(kb + ko, kw[j]);
    }
    kn[j] = *reinterpret_cast<const float2*>(kb + kno);
    if constexpr (GV) load_words<NG>(vb + vno, gsz[j]);
    else vn[j] = *reinterpret_cast<const float*>(vb + vno);
  };
  // The lane's QJL word among the words of its group (EXT: after the
  // half's own planes), selected with per-lane masks (a select on the word's
  // index would become an indexed load from scratch memory)
  uint32_t q_mask[EXT ? MK + 1 : 1];
  if constexpr (EXT) {
#pragma unroll
    for (int p = 0; p <= MK; ++p) {
      q_mask[p] = q_word == p ? ~0u : 0u;
      asm volatile("" : "+v"(q_mask[p]));
    }
  }
  auto qjl_word = [&](const uint32_t* w) -> uint32_t {
    if constexpr (!EXT) {
      return w[MK];
    } else {
      uint32_t z = w[0] & q_mask[0];
#pragma unroll
      for (int p = 1; p <= MK; ++p) z |= w[p] & q_mask[p];
      return z;
    }
  };
  // sum_j q[idx_j] val_j over the sidecar record of token r16 of page j of the
  // wavefront, for head g4 (logit units), from the records staged in LDS
  auto side_term = [&](int j) -> float {
    const uint8_t* rec =
        reinterpret_cast<const uint8_t*>(side_lds + ((wvu * PPW + j) * kPage + r16) * kSideWords);
    const int cnt = rec[0];
    float acc = 0.f;
    for (int e = 0; e < n_side; ++e) {
      const int c = rec[1 + e] & (D - 1);
      const float v = f16_bits_to_float(*reinterpret_cast<const uint16_t*>(rec + cd.side_val_off + 2 * e));
      acc = e < cnt ? fmaf(q_raw[g4 * D + c], v, acc) : acc;
    }
    return acc;
  };
  auto load_keys = [&]() {
#pragma unroll
    for (int j = 0; j < PPW; ++j) load_key_page(j);
  };
  auto load_values = [&]() {
    // lane group g4 reads pages 2 g4 and 2 g4 + 1 of the block
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const int p0 = max(checked(nid[hp]), 0);
      const int p1 = max(checked(nid[2 + hp]), 0);
      const int p2 = max(checked(nid[4 + hp]), 0);
      const int p3 = max(checked(nid[6 + hp]), 0);
      int mine = p0;
      mine = g4 == 1 ? p1 : mine;
      mine = g4 == 2 ? p2 : mine;
      mine = g4 == 3 ? p3 : mine;
      if constexpr (GV) {
        const uint8_t* vb = vbase + size_t(mine) * vstride;
#pragma unroll
        for (int c = 0; c < CBW; ++c) load_words_a4<BV>(vb + gv_off[c], vw[hp] + c * BV);
      } else if constexpr (EXT) {
        const uint8_t* vb = vbase + size_t(mine) * vstride + v_off;
#pragma unroll
        for (int cp = 0; cp < CBW / 2; ++cp) load_words_a4<BV>(vb + cp * v_pair, vw[hp] + cp * BV);
      } else {
        load_words<VW>(vbase + size_t(mine) * vstride + v_off, vw[hp]);
      }
    }
  };

  if (t_begin < t_end) {
    fetch_ids(t_begin);
    load_keys();
    load_values();
  }
  // the query operands, while the first block's pages are in flight (the
  // barriers wait for LDS traffic only)
  if constexpr (FQ) {
    if (tid < (EXT ? 32 : 16)) coef_k[tid] = coef_r;
    float* q_sk = q_rs + kMaxG * D;
    uint32_t* tail = reinterpret_cast<uint32_t*>(q_img + image_bytes<D, MK>());
#pragma unroll
    for (int i = 0; i < HPW; ++i)
      if (wvu + i * NW < kMaxG) query_finish<D, EXT>(a, qreg[i], wvu + i * NW, lane, qjl, q_rs, q_sk, q_raw);
    block_sync<NW>();
#pragma unroll
    for (int i = 0; i < HPW; ++i)
      if (wvu + i * NW < kMaxG) head_constants<D, MK, EXT>(q_rs, q_sk, coef_k, wvu + i * NW, lane, tail);
    block_sync<NW>();
    build_images<D, MK, EXT, 64 * NW>(q_rs, q_sk, coef_k, tail, q_img, tid);
    block_sync<NW>();
    if (cv.status != nullptr && hk == 0 && split == 0) check_sequence(a, s, tid, 64 * NW);
  } else {
    if constexpr (EXT) {
      if (n_side > 0) {
        const float* src = reinterpret_cast<const float*>(qp + image_bytes<D, MK>() + 256);
        for (int i = tid; i < kMaxG * D; i += 64 * NW) q_raw[i] = src[i];
      }
    }
    if constexpr (QL) {
      for (int i = tid; i < image_bytes<D, MK>() / 16; i += 64 * NW)
        reinterpret_cast<uint4*>(q_img)[i] = reinterpret_cast<const uint4*>(qp)[i];
    }
    if constexpr (QL || EXT) __syncthreads();
  }
  if constexpr (!QL) {
#pragma unroll
    for (int pl = 0; pl <= KP; ++pl)
#pragma unroll
      for (int hf = 0; hf < KH; ++hf) {
        const uint8_t* img = qp + (pl * KH + hf) * 2048;
        const uint4 lo = reinterpret_cast<const uint4*>(img)[lane];
        const uint4 hi = reinterpret_cast<const uint4*>(img + 1024)[lane];
        qa[pl][hf] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
  }
  {
    const int32_t* tail_i = reinterpret_cast<const int32_t*>(qp + image_bytes<D, MK>());
    const float* tail_f = reinterpret_cast<const float*>(tail_i + 16);
    sa = tail_i[r16];
    k_m = tail_f[g4];
    k_q = tail_f[kMaxG + g4];
  }
  // wait here once for everything requested so far, so that the loop's own
  // waits only ever cover loads issued inside the loop
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // Blocks of 128 tokens.  A block's key words and norms are requested as soon
  // as the previous block's scores are done, its value words as soon as the
  // previous block's value tiles are; the requests are unconditional (past
  // the split's end they fall on page 0 and are not used), so that no wait
  // depends on a branch.
  for (int tb = t_begin; tb < t_end; tb += kBlock) {
    fetch_ids(tb + kBlock);  // the next block's pages; their waits fall after the scores
    // ---------------------------------------------- scores of this wavefront's pages
    float sc[PPW], vnu[PPW];
    uint32_t gcur[GV ? PPW : 1][GV ? NG : 1];  // GV: this block's (scale, zero) pairs, kept past the reload
    bool kok[PPW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) kok[j] = kid[j] >= 0;
    float loc_max = -INFINITY, loc_vmax = 0.f;
    if constexpr (EXT) {
      // this block's sidecar records to LDS (each wavefront its own pages;
      // read back by the same wavefront, in order)
      if (n_side > 0) {
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
          uint32_t* rec = side_lds + ((wvu * PPW + j) * kPage + r16) * kSideWords;
          rec[g4] = sw[j][0];
          rec[g4 + 4] = sw[j][1];
        }
      }
    }
    // plane products x pages: with the query operands in LDS, each operand is
    // read once per block and feeds one independent MFMA per page; with them
    // in registers, page by page (pages interleave across the chains)
    v4f dm[PPW], dq[PPW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      dm[j] = v4f{k_m, 0.f, 0.f, 0.f};
      dq[j] = v4f{k_q, 0.f, 0.f, 0.f};
    }
    if constexpr (kPlaneOuter) {
#pragma unroll
      for (int hf = 0; hf < KH; ++hf)
#pragma unroll
        for (int pl = 0; pl <= KP; ++pl) {
          if (pl == KP && !qjl) break;
          const v8i qo = qop(pl, hf);
#pragma unroll
          for (int j = 0; j < PPW; ++j) {
            const uint32_t* w = kw[j] + hf * (MK + 1);
            if (pl < KP)
              dm[j] = mfma_f8_f4(qo, bits_to_fp4_affine(plane_word<MK>(w, pl)), dm[j], sa);
            else
              dq[j] = mfma_f8_f4(qo, bits_to_fp4_affine(qjl_word(w)), dq[j], sa);
          }
        }
    }
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      float2 knj = kn[j];
      float vnj;
      if constexpr (GV) {  // the token's largest group scale bounds its weights
        vnj = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          gcur[j][g] = gsz[j][g];
          vnj = fmaxf(vnj, f16_bits_to_float(uint16_t(gsz[j][g] & 0xffffu)));
        }
      } else {
        vnj = vn[j];
      }
      if constexpr (!kPlaneOuter) {
#pragma unroll
        for (int hf = 0; hf < KH; ++hf) {
          const uint32_t* w = kw[j] + hf * (MK + 1);
#pragma unroll
          for (int pl = 0; pl < KP; ++pl)
            dm[j] = mfma_f8_f4(qop(pl, hf), bits_to_fp4_affine(plane_word<MK>(w, pl)), dm[j], sa);
          if (qjl) dq[j] = mfma_f8_f4(qop(KP, hf), bits_to_fp4_affine(qjl_word(w)), dq[j], sa);
        }
        // this page's registers are consumed: request the next block's page
        // now, so that the wavefront's key requests stay spread over the
        // block instead of leaving in one burst
        if constexpr (kRollKeys) load_key_page(j);
      }
      const int pos = tb + (wvu * PPW + j) * kPage + r16;
      // dm[i], dq[i]: part i of head g4 for token r16, already in logit units
      const float msum = (dm[j][0] + dm[j][1]) + (dm[j][2] + dm[j][3]);
      const float qsum = (dq[j][0] + dq[j][1]) + (dq[j][2] + dq[j][3]);
      float est = knj.x * fmaf(knj.y, qsum, msum);
      if constexpr (EXT) {
        if (!qjl) est = knj.y * msum;  // s <qt, c[idx]>
        if (n_side > 0) est += side_term(j);
      }
      const bool tok_ok = pos < t_end && kok[j];
      const bool valid = tok_ok && head_ok;
      sc[j] = valid ? est : -INFINITY;
      vnu[j] = tok_ok ? vnj : 0.f;
      loc_max = fmaxf(loc_max, sc[j]);
      loc_vmax = fmaxf(loc_vmax, vnu[j]);
      if constexpr (kPageFence && !kPlaneOuter) {
        if (j % 2 == 1) __builtin_amdgcn_sched_barrier(0);  // bounds the pages in flight
      }
    }
    if (a.logits) {  // optional score dump (tests); one uniform branch per block
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        const int pos = tb + (wvu * PPW + j) * kPage + r16;
        if (sc[j] != -INFINITY) a.logits[(size_t(s) * a.num_q_heads + hk * G + g4) * a.max_ctx + pos] = sc[j] * kLn2;
      }
    }
    if constexpr (!kRollKeys) load_keys();
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
    // re-base the reference maximum (rare): weights stay below e^kRebase
    const bool rebase = blk_max > m_ref + kRebase;
    if (__any(rebase)) {
      const float m_new = rebase ? blk_max : m_ref;
      const float r = m_new == m_ref ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      l_part *= r;
#pragma unroll
      for (int g = 0; g < (GV ? NG : 1); ++g) {
        zacc[g] *= r;
        sacc[g] *= r;
      }
      // value layout: column r16 = (head r16 / 4, part r16 % 4)
      const float rv = row_value(r, r16 >> 2);
#pragma unroll
      for (int p = 0; p < VP; ++p)
#pragma unroll
        for (int c = 0; c < CBW; ++c) acc[p][c] *= rv;
      m_ref = m_new;
    }
    // power of two bringing the block's largest weight into (128, 256] as fp8;
    // the value MFMAs undo it through their E8M0 operand scale
    const float hd = blk_max - m_ref;  // <= kRebase, -inf for heads without tokens
    const float hmax = fmaxf(fmaxf(row_value(hd, 0), row_value(hd, 1)), fmaxf(row_value(hd, 2), row_value(hd, 3)));
    const float bound = blk_vmax * __builtin_amdgcn_exp2f(hmax);
    int e8 = 0;
    if (bound > 0.f) {
      frexpf(bound, &e8);
      e8 = min(max(8 - e8, -120), 115);
    }
    const float wscale = ldexpf(1.f, e8);
    const int scale_b = kScaleOne - e8;
    // fp8 parts of the weights, two pages at a time, to rows 4 g4 + part of
    // the weight image
#pragma unroll
    for (int j = 0; j < PPW; j += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sc[j] - m_ref);  // 0 for sc = -inf
      const float p1 = j + 1 < PPW ? __builtin_amdgcn_exp2f(sc[j + 1] - m_ref) : 0.f;
      l_part += p0 + p1;
      // weight image g holds p_t scale_{t,g} (GV); the single image p_t nu_t otherwise
#pragma unroll
      for (int g = 0; g < (GV ? NG : 1); ++g) {
        float x0, x1;
        if constexpr (GV) {
          const float s0 = f16_bits_to_float(uint16_t(gcur[j][g] & 0xffffu));
          const float z0 = f16_bits_to_float(uint16_t(gcur[j][g] >> 16));
          const float s1 = j + 1 < PPW ? f16_bits_to_float(uint16_t(gcur[j + 1][g] & 0xffffu)) : 0.f;
          const float z1 = j + 1 < PPW ? f16_bits_to_float(uint16_t(gcur[j + 1][g] >> 16)) : 0.f;
          zacc[g] = fmaf(p0, z0, fmaf(p1, z1, zacc[g]));
          sacc[g] = fmaf(p0, s0, fmaf(p1, s1, sacc[g]));
          x0 = p0 * s0 * wscale;
          x1 = p1 * s1 * wscale;
        } else {
          x0 = p0 * vnu[j] * wscale;
          x1 = j + 1 < PPW ? p1 * vnu[j + 1] * wscale : 0.f;
        }
        uint32_t lo, hi;
        fp8_split4_pair(x0, x1, __builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), lo, hi);
#pragma unroll
        for (int u = 0; u < 2 && j + u < PPW; ++u) {
          const int t = (wvu * PPW + j + u) * kPage + r16;
          uint8_t* o = w_img + g * 2048 + fp8_image_offset(g4 * 4, 32 * (t / 32) + fp4_bit_elem(t % 32));
          uint32_t l8 = lo >> (8 * u), h8 = hi >> (8 * u);
          if (u) asm volatile("" : "+v"(l8), "+v"(h8));  // keeps the >> 16 below a byte-2 store
          o[0] = uint8_t(l8);
          o[16] = uint8_t(l8 >> 16);
          o[32] = uint8_t(h8);
          o[48] = uint8_t(h8 >> 16);
        }
      }
    }
    block_sync<NW>();
    // ---------------------------------------------- value tiles of this wavefront
    if constexpr (GV) {
      // operand row r16 of tile CBW wv + c is coordinate 16 (CBW wv + c) + r16: its
      // bits are the low (even r16) or high half of its pair's words
      const uint32_t sel = (r16 & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
      for (int c = 0; c < CBW; c += 2) {
        const uint8_t* wi = w_img + ((CBW * wvu + c) / 2) * 2048;  // the tiles' group
        const uint4 lo = reinterpret_cast<const uint4*>(wi)[lane];
        const uint4 hi = reinterpret_cast<const uint4*>(wi + 1024)[lane];
        const v8i wop = {int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int b = 0; b < BV; ++b) {
            const uint32_t w = __builtin_amdgcn_perm(vw[1][(c + u) * BV + b], vw[0][(c + u) * BV + b], sel);
            acc[b][c + u] = mfma_f4_f8(fp4_operand(bits_to_fp4_pm6_dwords(w)), wop, acc[b][c + u], scale_b);
          }
      }
    } else {
      const uint4 lo = reinterpret_cast<const uint4*>(w_img)[lane];
      const uint4 hi = reinterpret_cast<const uint4*>(w_img + 1024)[lane];
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
        // even coordinate's planes, then the odd one's (keeps half the operands live)
        {
          v8i op[VP];
          value_operands<BV>(we, op);
#pragma unroll
          for (int p = 0; p < VP; ++p) acc[p][2 * cp] = mfma_f4_f8(op[p], wop, acc[p][2 * cp], scale_b);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          v8i op[VP];
          value_operands<BV>(wo, op);
#pragma unroll
          for (int p = 0; p < VP; ++p) acc[p][2 * cp + 1] = mfma_f4_f8(op[p], wop, acc[p][2 * cp + 1], scale_b);
        }
      }
    }
    load_values();
    block_sync<NW>();
  }

  // ------------------------------------------------------------ partial results
  // (EXT: lane groups 2-3 hold upper-half coordinates, with their own coefficients)
  const float* coef_v =
      reinterpret_cast<const float*>(a.params + kOffValuePlaneCoef + (EXT && g4 >= 2 ? kOffUpperHalf : 0));
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
    w0[0] = l > 0.f ? m_ref * kLn2 : -INFINITY;  // natural-log units for the merge
    w0[1] = l;
  }
  // values: planes combine in-lane, parts across the lane quad (columns 4h..4h+3)
  const int ch = r16 >> 2, cq = r16 & 3;
  const float part_w = cq == 0 ? 1.f : cq == 1 ? 0.0625f : cq == 2 ? 0.00390625f : 0.000244140625f;
  float* wsh = ws + ((size_t(s) * a.num_q_heads + hk * G + ch) * nrec + split) * rec + 2;
  if constexpr (GV) {
    // the per-(head, group) sums of this wavefront's tokens, to LDS
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float zs = sum16(zacc[g]), ss = sum16(sacc[g]);
      if (r16 == 0) {
        gsum[((wv * kMaxG + g4) * NG + g) * 2] = zs;
        gsum[((wv * kMaxG + g4) * NG + g) * 2 + 1] = ss;
      }
    }
    block_sync<NW>();  // (one wavefront reads its own LDS writes in order)
  }
  float cvals[VP];
  if constexpr (!GV) {
#pragma unroll
    for (int p = 0; p < VP; ++p) cvals[p] = coef_v[odd_subset(BV, p)] * (1.f / kPm6);  // planes read +-6
  }
#pragma unroll
  for (int c = 0; c < CBW; ++c) {
    float half_const = 0.f;  // GV: (2^b - 1) / 2 for the tile's half
    if constexpr (GV) {
      // plane j carries -2^(j-1) s_j, read as +-6
      const int bits = cd.vbits[16 * (CBW * wv + c) >= D / 2 ? 1 : 0];
#pragma unroll
      for (int p = 0; p < VP; ++p) cvals[p] = p < bits ? -float(1 << p) / (2.f * kPm6) : 0.f;
      half_const = 0.5f * float((1 << bits) - 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int p = 0; p < VP; ++p) v = fmaf(cvals[p], acc[p][c][i], v);
      v *= part_w;
      v += dpp<0xB1>(v);
      v += dpp<0x4E>(v);
      const int coord = GV ? 16 * (CBW * wv + c) + 4 * g4 + i : NCB * (4 * g4 + i) + CBW * wv + c;
      if (cq == 0 && ch < G) {
        if constexpr (GV) {
          const int g = coord / kGroup;
          float zs = 0.f, ss = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) {
            zs += gsum[((w2 * kMaxG + ch) * NG + g) * 2];
            ss += gsum[((w2 * kMaxG + ch) * NG + g) * 2 + 1];
          }
          v += fmaf(half_const, ss, zs);
        }
        wsh[coord] = v;
      }
    }
  }
}

// Merge the compressed splits of one (sequence, query head) by log-sum-exp,
// rotate their value sum back once, add the window's (already unrotated) sum,
// normalise and store.  FWHT variant: one wavefront per row, four rows per
// workgroup -- the splits' maxima and denominators across lanes, the value
// sums per coordinate (D / 64 per lane) with several loads in flight, the
// inverse FWHT in registers.  Dense variant: one row per workgroup of 1024
// threads, D per slice: each slice sums every KQ-th split for its coordinate,
// then multiplies its share of the rows of Pi_V^T, the slices meeting in LDS
// (enough wavefronts to hide the loads' latency).  With few rows (WIDE, FWHT only) one row takes a whole
// workgroup instead: each wavefront sums a quarter of the splits, the partial
// sums meet in LDS and the first wavefront finishes the row, so that a short
// list of rows still spreads its record loads over many CUs.
template <int ROT>
__host__ __device__ constexpr int combine_rows(int) { return ROT == TQ_ROT_DENSE ? 1 : 4; }
constexpr int kWideCombineRows = 512;
template <int N>
struct Count {
  static constexpr int value = N;
};  // FWHT rows up to this many: a workgroup per row
template <int ROT>
__host__ __device__ constexpr int combine_threads() { return ROT == TQ_ROT_DENSE ? 1024 : 256; }
template <int D, int ROT, bool WIDE>
__global__ __launch_bounds__(combine_threads<ROT>()) void decode_combine_kernel(DecodeArgs a, size_t part_offset) {
  static_assert(!WIDE || ROT == TQ_ROT_FWHT, "the wide combine is the FWHT variant's");
  constexpr int R = D / 64;
  constexpr int RPB = WIDE ? 1 : combine_rows<ROT>(0);
  constexpr int KQ = combine_threads<ROT>() / D;  // dense: slices of the sums per coordinate
  __shared__ float buf[ROT == TQ_ROT_DENSE ? (KQ + 1) * D : (WIDE ? 4 * D : 1)];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t row = size_t(blockIdx.x) * RPB + (RPB > 1 ? wv : 0);  // s * H_q + h
  if (RPB > 1 && row >= size_t(a.num_seqs) * a.num_q_heads) return;  // whole wavefronts; no barrier on this path
  const int s = int(row / a.num_q_heads);
  const int rec = 2 + D, nrec = a.splits + kWindowRecords;
  const float* ws = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(a.workspace) + part_offset) +
                    row * nrec * rec;
  // compressed splits that hold tokens of this sequence (the rest are empty)
  const CacheView& cv = a.cache;
  // group-quantized values are accumulated in their own basis: no inverse rotation
  const bool rotated = cv.codec.value_mode != TQ_VALUE_GROUP;
  const int slot = a.seq_slots[s];
  int L = a.ctx_len[s];
  if (slot < 0 || slot >= cv.max_seqs || L < 0) L = 0;
  L = min(L, min(cv.max_pages_per_seq * kPage, a.max_ctx));
  const int nc = cv.window > 0 ? max(0, L - cv.window) : L;
  const int ns = min(a.splits, (nc + a.split_tokens - 1) / a.split_tokens);
  // records in merge order: the ns compressed splits, then the window's
  const int NWR = a.window_items;
  auto rec_of = [&](int sp) { return ws + size_t(sp < ns ? sp : a.splits + (sp - ns)) * rec; };
  // maximum and denominator over the records (every wavefront of the row
  // alike).  In the wide and the dense forms with at most 128 records, lane t
  // keeps the weights of records t and t + 64, and the weights are broadcast
  // from the lanes instead of being read again (every caller's record index
  // is uniform across its wavefront).
  const bool in_lanes = (WIDE || ROT == TQ_ROT_DENSE) && ns + NWR <= 128;
  // this thread's coordinates of the window records' sums, requested first so
  // that they arrive with the records' maxima (FWHT: r * 64 + lane; dense:
  // tid % D, used by the first slice)
  constexpr int NWC = ROT == TQ_ROT_DENSE ? 1 : R;
  float wvals[kWindowRecords][NWC];
#pragma unroll
  for (int j = 0; j < kWindowRecords; ++j)
#pragma unroll
    for (int r = 0; r < NWC; ++r) {
      const int c = ROT == TQ_ROT_DENSE ? tid % D : r * 64 + lane;
      wvals[j][r] = j < NWR ? rec_of(ns + j)[2 + c] : 0.f;
    }
  float M = -INFINITY, l = 0.f, wl[2] = {0.f, 0.f};
  if (in_lanes) {
    // lane t holds records t and t + 64
    float m[2] = {-INFINITY, -INFINITY}, lr[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (lane + 64 * i < ns + NWR) {
        const float* r = rec_of(lane + 64 * i);
        m[i] = r[0];
        lr[i] = r[1];
      }
    M = wave_max(fmaxf(m[0], m[1]));
#pragma unroll
    for (int i = 0; i < 2; ++i) wl[i] = m[i] == -INFINITY ? 0.f : __expf(m[i] - M);
    l = wave_sum(fmaf(wl[0], lr[0], wl[1] * lr[1]));
  } else {
    for (int sp = lane; sp < ns + NWR; sp += 64) M = fmaxf(M, rec_of(sp)[0]);
    M = wave_max(M);
    for (int sp = lane; sp < ns + NWR; sp += 64) {
      const float m = rec_of(sp)[0];
      if (m != -INFINITY) l = fmaf(__expf(m - M), rec_of(sp)[1], l);
    }
    l = wave_sum(l);
  }
  // weight of record sp in merge order (compressed splits below ns); sp is
  // uniform across the calling wavefront
  auto weight = [&](int sp) {
    if (in_lanes)
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sp < 64 ? wl[0] : wl[1]), sp & 63));
    const float m = rec_of(sp)[0];
    return m == -INFINITY ? 0.f : __expf(m - M);
  };
  float fw[kWindowRecords];
#pragma unroll
  for (int j = 0; j < kWindowRecords; ++j) fw[j] = j < NWR ? weight(ns + j) : 0.f;
  // the window records' weighted value sum at this thread's coordinate i
  // (index into wvals)
  auto window_sum = [&](int i) {
    float aw = 0.f;
#pragma unroll
    for (int j = 0; j < kWindowRecords; ++j) aw = fmaf(fw[j], wvals[j][i], aw);
    return aw;
  };
  if constexpr (ROT == TQ_ROT_FWHT) {
    // compressed value sums, coordinates r * 64 + lane
    float ar[R];
#pragma unroll
    for (int r = 0; r < R; ++r) ar[r] = 0.f;
    constexpr int B = (WIDE ? 64 : 32) / R;  // splits per batch: loads in flight per lane
    const int sp_beg = WIDE ? (wv * ns) / 4 : 0, sp_end = WIDE ? ((wv + 1) * ns) / 4 : ns;
    // NB splits from sp0 with every load issued at once; past the end the
    // last split again, with weight 0
    auto batch = [&](auto nb, int sp0) {
      constexpr int NB = decltype(nb)::value;
      float f[NB], v[NB][R];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int sp = min(sp0 + u, sp_end - 1);
        f[u] = sp0 + u < sp_end ? weight(sp) : 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) v[u][r] = ws[size_t(sp) * rec + 2 + r * 64 + lane];
      }
#pragma unroll
      for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) ar[r] = fmaf(f[u], v[u][r], ar[r]);
    };
    int sp0 = sp_beg;
    for (; sp0 + B <= sp_end; sp0 += B) batch(Count<B>{}, sp0);
    const int rem = sp_end - sp0;
    if constexpr (WIDE) {  // the rest in one batch of the next power of two
      if (rem > B / 2) batch(Count<B>{}, sp0);
      else if (rem > B / 4) batch(Count<B / 2>{}, sp0);
      else if (rem > B / 8) batch(Count<B / 4>{}, sp0);
      else if (rem > 2) batch(Count<4>{}, sp0);
      else if (rem == 2) batch(Count<2>{}, sp0);
      else if (rem == 1) batch(Count<1>{}, sp0);
    } else {  // many rows in flight: the rest one split at a time
      for (int sp = sp0; sp < sp_end; ++sp) batch(Count<1>{}, sp);
    }
    if constexpr (WIDE) {
#pragma unroll
      for (int r = 0; r < R; ++r) buf[wv * D + r * 64 + lane] = ar[r];
      __syncthreads();
      if (wv != 0) return;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int c = r * 64 + lane;
        ar[r] = (buf[c] + buf[D + c]) + (buf[2 * D + c] + buf[3 * D + c]);
      }
    }
    if (rotated) wave_fwht<R>(ar, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = r * 64 + lane;
      const float o = rotated ? apply_sign(ar[r] * rsqrtf(float(D)), sign_bit(a.params, kRoleValueRot, c)) : ar[r];
      const float aw = window_sum(r);
      a.out[row * D + c] = l > 0.f ? (o + aw) / l : 0.f;
    }
  } else {
    // thread (c, k): coordinate c, slice k of the splits and then of the
    // rows of Pi_V; the slices meet in LDS (buf[k D + c]; the merged sum at
    // buf[KQ D + c])
    const int c = tid % D, k = tid / D;
    constexpr int J = D / KQ;
    // this thread's share of Pi_V^T, requested before the merge so that its
    // loads overlap the merge's
    const float* piv = reinterpret_cast<const float*>(a.params + kOffDense) + size_t(2) * D * D + size_t(k * J) * D + c;
    float pv[J];
    if (rotated) {
#pragma unroll
      for (int j = 0; j < J; ++j) pv[j] = piv[size_t(j) * D];
    }
    float ar = 0.f;
    {
      int sp = k;
      for (; sp + 3 * KQ < ns; sp += 4 * KQ) {
        float f[4], v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          f[u] = weight(sp + u * KQ);
          v[u] = ws[size_t(sp + u * KQ) * rec + 2 + c];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) ar = fmaf(f[u], v[u], ar);
      }
      for (; sp < ns; sp += KQ) ar = fmaf(weight(sp), ws[size_t(sp) * rec + 2 + c], ar);
    }
    buf[k * D + c] = ar;
    __syncthreads();
    if (k == 0) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < KQ; ++q) v += buf[q * D + c];
      buf[KQ * D + c] = v;
    }
    __syncthreads();
    const float* sum = buf + KQ * D + k * J;
    float o4[4] = {0.f, 0.f, 0.f, 0.f};
    if (rotated) {
#pragma unroll
      for (int j = 0; j < J; ++j) o4[j % 4] = fmaf(pv[j], sum[j], o4[j % 4]);
    } else if (k == 0) {
      o4[0] = buf[KQ * D + c];
    }
    __syncthreads();  // every read of the slices above is done
    buf[k * D + c] = (o4[0] + o4[1]) + (o4[2] + o4[3]);
    __syncthreads();
    if (k == 0) {
      float o = 0.f;
#pragma unroll
      for (int q = 0; q < KQ; ++q) o += buf[q * D + c];
      const float aw = window_sum(0);
      a.out[row * D + c] = l > 0.f ? (o + aw) / l : 0.f;
    }
  }
}

constexpr int kSimds = 1024;  // 256 CUs x 4 SIMDs

template <int D, int ROT>
hipError_t launch_combine(const DecodeArgs& a, size_t part_offset, hipStream_t st) {
  const int rows = a.num_seqs * a.num_q_heads, rpb = combine_rows<ROT>(0);
  if constexpr (ROT == TQ_ROT_FWHT) {
    if (rows <= kWideCombineRows) {
      hipLaunchKernelGGL((decode_combine_kernel<D, ROT, true>), dim3(rows), dim3(256), 0, st, a, part_offset);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_combine_kernel<D, ROT, false>), dim3((rows + rpb - 1) / rpb), dim3(combine_threads<ROT>()), 0, st, a,
                     part_offset);
  return hipGetLastError();
}

template <int D, int MK, int BV, int ROT, bool EXT, bool GV>
hipError_t launch_mfma(const DecodeArgs& a, size_t part_offset, hipStream_t st) {
  constexpr int FMT = GV ? 2 : EXT ? 1 : 0;
  constexpr int NW = split_waves(D, MK, BV, FMT);
  constexpr bool QL = split_q_in_lds(D, MK, BV, FMT);
  constexpr int OCC = split_occupancy(D, MK, BV, FMT);
  const int H = a.cache.num_kv_heads;
  // one work item per (sequence, kv head, split), plus window_items per (sequence, kv head) for the window
  const dim3 grid(a.num_seqs * H, a.splits + a.window_items);
  hipError_t e;
  // Latency-bound launches (fewer wavefronts than SIMDs, FWHT): four
  // wavefronts per work item, which build the query operands themselves, one
  // query head each; every item's block then divides over four SIMDs.
  constexpr bool kWideOk = ROT == TQ_ROT_FWHT && NW < 4 && split_shape_ok(D, 4);
  if constexpr (kWideOk) {
    if (size_t(grid.x) * grid.y * NW < size_t(kSimds)) {
      constexpr bool QLW = !split_fits(D, MK, BV, 4, false, FMT);
      hipLaunchKernelGGL((decode_split_kernel<D, MK, BV, 4, QLW, OCC, EXT, GV, true>), grid, dim3(256), 0, st, a,
                         part_offset);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_combine<D, ROT>(a, part_offset, st);
    }
  }
  if (ROT == TQ_ROT_FWHT && split_builds_query(ROT, a.splits)) {
    hipLaunchKernelGGL((decode_split_kernel<D, MK, BV, NW, QL, OCC, EXT, GV, ROT == TQ_ROT_FWHT>), grid, dim3(64 * NW), 0, st,
                       a, part_offset);
  } else {
    hipLaunchKernelGGL((decode_prep_kernel<D, MK, ROT, EXT>), dim3(a.num_seqs * H), dim3(prep_threads<ROT>()), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_split_kernel<D, MK, BV, NW, QL, OCC, EXT, GV, false>), grid, dim3(64 * NW), 0, st, a, part_offset);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine<D, ROT>(a, part_offset, st);
}

// Key and value bit counts the kernels are built for: the larger half's
// (the default format has one count per role).
struct Bits {
  int mk, bv;
};
Bits kernel_bits(const tq_config& cfg) {
  const Codec k = make_codec(cfg);
  return {k.kbits[0] > k.kbits[1] ? k.kbits[0] : k.kbits[1], k.vbits[0] > k.vbits[1] ? k.vbits[0] : k.vbits[1]};
}

template <int D, int ROT, bool EXT, bool GV>
hipError_t dispatch_bits(const DecodeArgs& a, Bits b, size_t part_offset, hipStream_t st) {
#define TQ_CASE(MK_, BV_) \
  if (b.mk == MK_ && b.bv == BV_) return launch_mfma<D, MK_, BV_, ROT, EXT, GV>(a, part_offset, st);
  TQ_CASE(1, 1) TQ_CASE(1, 2) TQ_CASE(1, 3) TQ_CASE(1, 4)
  TQ_CASE(2, 1) TQ_CASE(2, 2) TQ_CASE(2, 3) TQ_CASE(2, 4)
  TQ_CASE(3, 1) TQ_CASE(3, 2) TQ_CASE(3, 3) TQ_CASE(3, 4)
  if constexpr (EXT) {  // all four key bits to the codebook (scale-corrected keys)
    TQ_CASE(4, 1) TQ_CASE(4, 2) TQ_CASE(4, 3) TQ_CASE(4, 4)
  }
#undef TQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace

int decode_mfma_items(const tq_config& cfg) {
  const Bits b = kernel_bits(cfg);
  const int d = cfg.head_dim;
  if (b.mk < 1 || b.mk > 4 || b.bv < 1 || b.bv > 4 || (d != 128 && d != 256)) return 2048;
  // work items that fill every SIMD once: SIMDs x resident wavefronts / wavefronts per item
  const int fmt = cfg.value_mode == TQ_VALUE_GROUP ? 2 : make_codec(cfg).ext ? 1 : 0;
  return kSimds * split_occupancy(d, b.mk, b.bv, fmt) / split_waves(d, b.mk, b.bv, fmt);
}

size_t decode_prep_bytes(const tq_config& cfg, int num_seqs) {
  // the default format's region is sized for its largest key bit width; an
  // extended format's for the bits its kernels are built for; 256-byte aligned
  const int d = cfg.head_dim;
  const size_t stride = make_codec(cfg).ext ? prep_stride(d, kernel_bits(cfg).mk, true) : prep_stride(d, 3, false);
  const size_t b = size_t(num_seqs) * cfg.num_kv_heads * stride;
  return (b + 255) & ~size_t(255);
}

// The matrix-core path takes head_dim 128 and 256, GQA groups up to 4, and
// every stored format.
bool decode_mfma_supported(const tq_config& cfg) {
  return (cfg.head_dim == 128 || cfg.head_dim == 256) && cfg.num_q_heads / cfg.num_kv_heads <= kMaxG &&
         cfg.page_tokens == kPage && cfg.window <= 1024;
}

int launch_decode_mfma(const tq_config& cfg, const DecodeArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool dense = cfg.rotation == TQ_ROT_DENSE;
  const bool ext = make_codec(cfg).ext != 0;
  const bool gv = cfg.value_mode == TQ_VALUE_GROUP;
  const Bits b = kernel_bits(cfg);
  const size_t part_offset = decode_prep_bytes(cfg, a.num_seqs);
#define TQ_DISPATCH(D_)                                                                                   \
  if (cfg.head_dim == D_) {                                                                               \
    if (gv) return dense ? dispatch_bits<D_, TQ_ROT_DENSE, true, true>(a, b, part_offset, st)             \
                         : dispatch_bits<D_, TQ_ROT_FWHT, true, true>(a, b, part_offset, st);             \
    if (ext) return dense ? dispatch_bits<D_, TQ_ROT_DENSE, true, false>(a, b, part_offset, st)           \
                          : dispatch_bits<D_, TQ_ROT_FWHT, true, false>(a, b, part_offset, st);           \
    return dense ? dispatch_bits<D_, TQ_ROT_DENSE, false, false>(a, b, part_offset, st)                   \
                 : dispatch_bits<D_, TQ_ROT_FWHT, false, false>(a, b, part_offset, st);                   \
  }
  TQ_DISPATCH(128) TQ_DISPATCH(256)
#undef TQ_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace tqi
