// Reconstruction of page-resident keys and values ([Reconstruction] =
// "Mathematical Reconstruction, Lineage, and Accuracy Limits of TurboQuant and
// TurboVec", section 5 "Step 5: Code Assignment, Packing, and Reconstruction":
// centroid lookup, inverse rotation, scaling by the stored norm; section 6 "The
// Asymmetric Unbiased Estimator": the final dot product combines the MSE
// reconstruction and the QJL residual term).
//   k~ = nu T_K^T (c_K[idx] + gamma sqrt(pi/2)/d S^T (1 - 2z))
//   v~ = nu_V T_V^T c_V[idx]
// so <q, k~> equals the decode-time score estimate.  Used by tests; decode
// never materialises these vectors.
#include "tq_device.h"

namespace tqi {
namespace {

constexpr float kQjlConst = 1.2533141373155003f;  // sqrt(pi / 2)

// y = M^T x for a row-major d x d matrix M, x staged through LDS.
template <int D>
__device__ __forceinline__ void dense_t(float (&x)[D / 64], const float* m, float* lds, int lane) {
  constexpr int R = D / 64;
#pragma unroll
  for (int r = 0; r < R; ++r) lds[r * 64 + lane] = x[r];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = r * 64 + lane;
    float acc = 0.f;
    for (int j = 0; j < D; ++j) acc = fmaf(m[size_t(j) * D + c], lds[j], acc);
    x[r] = acc;
  }
  __syncthreads();
}

// x <- D_role H x * scale (the transpose of H D_role is D_role H, H symmetric).
template <int D>
__device__ __forceinline__ void fwht_then_sign(float (&x)[D / 64], const uint8_t* params, int role, int lane,
                                               float scale) {
  constexpr int R = D / 64;
  wave_fwht<R>(x, lane);
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = apply_sign(x[r] * scale, sign_bit(params, role, r * 64 + lane));
}

template <int D, int ROT>
__global__ __launch_bounds__(64) void dequant_kernel(DequantArgs a) {
  constexpr int R = D / 64;
  constexpr int P = 16;
  __shared__ float lds[D];
  const int lane = threadIdx.x;
  const CacheView& cv = a.cache;
  const int H = cv.num_kv_heads;
  const int i = blockIdx.x / H, h = blockIdx.x % H;
  const int pos = a.tok_begin + i;
  const int mk = a.key_mse_bits, bv = a.value_bits;
  const size_t plane_bytes = size_t(P) * D / 8;
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
  const float* kc = reinterpret_cast<const float*>(a.params + kOffKeyCentroids);
  const float* vc = reinterpret_cast<const float*>(a.params + kOffValueCentroids);
  const float* dense = reinterpret_cast<const float*>(a.params + kOffDense);
  const uint8_t* kb = cv.k_pages + (size_t(phys) * H + h) * cv.key_block;
  const uint8_t* vb = cv.v_pages + (size_t(phys) * H + h) * cv.value_block;

  // ---------------- key
  float yr[R], sg[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = r * 64 + lane;
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(kb) + (size_t(t) * (D / 32) + c / 32) * (mk + 1);
    int idx = 0;
    for (int p = 0; p < mk; ++p) idx |= int((kw[p] >> (c % 32)) & 1u) << p;
    yr[r] = kc[idx];
    sg[r] = ((kw[mk] >> (c % 32)) & 1u) ? -1.f : 1.f;
  }
  const float* knorm = reinterpret_cast<const float*>(kb + size_t(mk + 1) * plane_bytes) + 2 * t;
  const float nu = knorm[0], gamma = knorm[1];
  // S^T s: FWHT variant S^T = D1 H_n D2 H; dense variant G^T
  if (ROT == TQ_ROT_FWHT) {
    fwht_then_sign<D>(sg, a.params, kRoleSketch2, lane, 1.0f);
    fwht_then_sign<D>(sg, a.params, kRoleSketch1, lane, rsqrtf(float(D)));
  } else {
    dense_t<D>(sg, dense + size_t(D) * D, lds, lane);
  }
  const float qc = gamma * kQjlConst / float(D);
#pragma unroll
  for (int r = 0; r < R; ++r) yr[r] = fmaf(qc, sg[r], yr[r]);
  if (ROT == TQ_ROT_FWHT) {
    fwht_then_sign<D>(yr, a.params, kRoleKeyRot, lane, rsqrtf(float(D)));
  } else {
    dense_t<D>(yr, dense, lds, lane);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) ko[r * 64 + lane] = nu * yr[r];

  // ---------------- value
  const uint32_t* vwords = reinterpret_cast<const uint32_t*>(vb);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = r * 64 + lane;
    int idx = 0;
    for (int p = 0; p < bv; ++p) idx |= int((vwords[(c / 2) * bv + p] >> (16 * (c & 1) + t)) & 1u) << p;
    yr[r] = vc[idx];
  }
  const float vnu = reinterpret_cast<const float*>(vb + size_t(bv) * plane_bytes)[t];
  if (ROT == TQ_ROT_FWHT) {
    fwht_then_sign<D>(yr, a.params, kRoleValueRot, lane, rsqrtf(float(D)));
  } else {
    dense_t<D>(yr, dense + size_t(2) * D * D, lds, lane);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) vo[r * 64 + lane] = vnu * yr[r];
}

template <int D, int ROT>
hipError_t launch(const DequantArgs& a, hipStream_t st) {
  const int n = a.tok_end - a.tok_begin;
  hipLaunchKernelGGL((dequant_kernel<D, ROT>), dim3(n * a.cache.num_kv_heads), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int launch_dequantize(const tq_config& cfg, const DequantArgs& a, void* stream) {
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
