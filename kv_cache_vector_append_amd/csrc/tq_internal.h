// Internal definitions shared by the host code and the HIP kernels of the
// library: the parameter-blob layout and the argument blocks of each launch.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "tq.h"

namespace tqi {

// ---------------------------------------------------------------------------
// Parameter blob (written by tq_init_codebooks, read by every kernel).
//   [0, 64)        header (int32/uint64 fields below)
//   [64, 128)      key centroids, float[16] ascending (2^(key_bits-1) used)
//   [128, 192)     key thresholds, float[16] (midpoints; unused = +inf)
//   [192, 256)     value centroids, float[16]
//   [256, 320)     value thresholds, float[16]
//   [320, 384)     key bit-plane coefficients, float[16] (see below)
//   [384, 448)     value bit-plane coefficients, float[16]
//   [448, 832)     the same six tables for the upper coordinate half d/2 .. d-1
//                  (key_bits_hi / value_bits_hi; copies of the lower ones
//                  when the rate is uniform)
//   [1024, 1280)   Rademacher sign words, 4 roles x 64 bytes (coordinate i of a
//                  role is bit i % 32 of uint32 word i / 32; 1 means -1)
//   [2048, ...)    dense variant: Pi_K, G, Pi_V as float[d*d] row-major each,
//                  then for each of them (same order) fp16 hi and lo copies,
//                  row-major [d][d] each, of s*M with s = 1024 for Pi_K and
//                  Pi_V and 256 for G: hi = fp16(s M), lo = fp16(s M - hi), the
//                  operands of the matrix-core append (the scales keep every lo
//                  piece that matters out of the fp16 subnormal range)
//
// Bit-plane coefficients: a symmetric (odd) codebook c over b-bit codes is a
// multilinear function of the signs s_k = 1 - 2*bit_k(idx):
//   c[idx] = sum_{S odd} a_S prod_{k in S} s_k,   a_S = 2^-b sum_idx c[idx] prod_{k in S} s_k.
// a_S is stored at index S (bitmask); even subsets are zero.
// ---------------------------------------------------------------------------
constexpr uint32_t kParamsMagic = 0x31505154u;  // "TQP1"
constexpr int kOffKeyCentroids = 64;
constexpr int kOffKeyThresholds = 128;
constexpr int kOffValueCentroids = 192;
constexpr int kOffValueThresholds = 256;
constexpr int kOffKeyPlaneCoef = 320;
constexpr int kOffValuePlaneCoef = 384;
constexpr int kOffUpperHalf = 384;  // add to a lower-half table offset for its upper-half copy
constexpr int kOffSigns = 1024;
constexpr int kSignRoleBytes = 64;
constexpr int kOffDense = 2048;

enum SignRole { kRoleKeyRot = 0, kRoleSketch1 = 1, kRoleSketch2 = 2, kRoleValueRot = 3 };

struct ParamsHeader {
  uint32_t magic;
  uint32_t version;
  int32_t head_dim;
  int32_t key_mse_bits;
  int32_t value_bits;
  int32_t rotation;
  uint64_t seed;
  uint32_t total_bytes;
  int32_t key_mse_bits_hi, value_bits_hi, key_mode, value_mode, key_outliers;
  uint32_t reserved[2];
};
static_assert(sizeof(ParamsHeader) == 64, "header is 64 bytes");

// Dense variant after the header tables: Pi_K, G, Pi_V as fp32 row-major;
// their fp16 hi / lo splits; then, as fp32 row-major, Pi_K^T and (G Pi_K)^T
// (the decode's query preparation: both products of the query in one pass)
// and G^T, Pi_V^T (the short appends' products): a wavefront's loads of one
// step of a product read one contiguous row.
inline size_t params_bytes(int d, int rotation) {
  return kOffDense + (rotation == TQ_ROT_DENSE ? size_t(d) * d * (3 * sizeof(float) + 3 * 2 * sizeof(uint16_t) +
                                                                  4 * sizeof(float))
                                               : 0);
}
// byte offset of the fp16 split of dense matrix m (0 Pi_K, 1 G, 2 Pi_V); lo follows hi
constexpr size_t dense16_offset(int d, int m) { return kOffDense + size_t(3) * d * d * 4 + size_t(m) * d * d * 4; }
// byte offset of the transposed fp32 matrix m (0 Pi_K^T, 1 (G Pi_K)^T, 2 G^T, 3 Pi_V^T)
constexpr size_t dense_t_offset(int d, int m) { return kOffDense + size_t(6) * d * d * 4 + size_t(m) * d * d * 4; }
constexpr float kDense16Scale[3] = {1024.f, 256.f, 1024.f};

// ---------------------------------------------------------------------------
// Stored format of one configuration (built on the host from tq_config).
// Coordinates d/2 .. d-1 form the upper half, with their own bit counts.
// ---------------------------------------------------------------------------
constexpr int kGroup = 32;         // coordinates per key word and per value scale/zero group
constexpr int kMaxOutliers = 8;
struct Codec {
  int32_t ext;                     // any feature beyond the default format
  int32_t key_mode, value_mode;    // tq_key_mode, tq_value_mode
  int32_t kbits[2];                // key Lloyd-Max bits of the lower / upper half
  int32_t vbits[2];                // value bits of the lower / upper half
  int32_t qjl;                     // 1: a QJL plane per key group
  int32_t outliers;                // key sidecar entries per vector
  int32_t key_row_words;           // code words per token in a key block
  int32_t key_norm_off;            // bytes: (nu, gamma or s) pairs
  int32_t key_side_off;            // bytes: sidecar records
  int32_t side_bytes;              // bytes per sidecar record
  int32_t side_val_off;            // bytes: fp16 values inside a record
  int32_t value_words;             // code words in a value block
  int32_t value_tail_off;          // bytes: nu[] or the (scale, zero) pairs
  int32_t key_block, value_block;  // bytes
};
Codec make_codec(const tq_config& cfg);
inline size_t key_block_bytes(const tq_config& cfg) { return size_t(make_codec(cfg).key_block); }
inline size_t value_block_bytes(const tq_config& cfg) { return size_t(make_codec(cfg).value_block); }

// ---------------------------------------------------------------------------
// Launch argument blocks.
// ---------------------------------------------------------------------------
struct CacheView {
  uint8_t* k_pages;
  uint8_t* v_pages;
  const int32_t* block_table;
  uint16_t* k_window;  // fp16 bits
  uint16_t* v_window;
  int32_t num_pages, max_seqs, max_pages_per_seq;
  int32_t num_kv_heads, page_tokens, window;
  int32_t key_block, value_block;  // bytes
  uint32_t* status;                // optional TQ_STATUS_* word
  Codec codec;
};

struct AppendArgs {
  CacheView cache;
  const uint8_t* params;
  const void* k_new;
  const void* v_new;
  const int32_t* seq_slots;
  const int32_t* ctx_len_before;
  const int32_t* cu_new_tokens;
  int32_t num_seqs, dtype, key_mse_bits, value_bits;
  int32_t parts;  // workers per (sequence, kv head), set by launch_append
};

// Decode partial records per (sequence, query head) beyond the splits': one
// per work item of the recent-token window.
constexpr int kWindowRecords = 4;

struct DecodeArgs {
  CacheView cache;
  const uint8_t* params;
  const void* q;
  const int32_t* seq_slots;
  const int32_t* ctx_len;
  float* out;
  float* workspace;   // plain path: [num_seqs][H_q][splits][2 + 2d]; matrix-core path: query
                      // operands (decode_prep_bytes), then [num_seqs][H_q][splits + kWindowRecords][2 + d]
  float* logits;      // optional [num_seqs][H_q][max_ctx]
  int32_t num_seqs, num_q_heads, q_dtype, key_mse_bits, value_bits;
  int32_t splits, split_tokens, max_ctx;
  int32_t window_items;  // matrix-core path: 1 .. kWindowRecords
  float scale;
};

struct DequantArgs {
  CacheView cache;
  const uint8_t* params;
  float* k_out;
  float* v_out;
  int32_t seq_slot, tok_begin, tok_end, key_mse_bits, value_bits;
};

// Decode split sizing shared by the workspace query and the launch.
struct SplitPlan {
  int splits;
  int split_tokens;
  int window_items;  // matrix-core path: work items of the recent-token window per (sequence, KV head)
};
// At most kMaxSplits context splits per (sequence, KV head).
constexpr int kMaxSplits = 2048;
SplitPlan plan_splits(const tq_config& cfg, int num_seqs, int max_ctx);

// Host-side parameter construction (tq_host.cpp).
void build_params(const tq_config& cfg, uint8_t* blob);

// Kernel launchers (one per .hip file); return hipError_t as int.
int launch_append(const tq_config& cfg, const AppendArgs& a, int num_seqs, int max_new, void* stream);
// the generic path (tq_codec.hip): every stored format, one wavefront per page
// of append, a per-lane scoring decode, and the reconstruction
int launch_append_codec(const tq_config& cfg, const AppendArgs& a, int num_seqs, int max_new, void* stream);
int launch_decode_codec(const tq_config& cfg, const DecodeArgs& a, void* stream);
bool decode_mfma_supported(const tq_config& cfg);
int decode_mfma_items(const tq_config& cfg);  // (sequence, KV head, split) work items that fill the GPU once
size_t decode_prep_bytes(const tq_config& cfg, int num_seqs);  // query-operand region at the workspace start
int launch_decode_mfma(const tq_config& cfg, const DecodeArgs& a, void* stream);
int launch_dequantize_codec(const tq_config& cfg, const DequantArgs& a, void* stream);

// Device address of the current GPU's library-owned decode workspace of
// TQ_STATIC_WORKSPACE_BYTES (tq_scratch.hip); returns hipError_t as int.
int static_workspace(void** ptr);

}  // namespace tqi
