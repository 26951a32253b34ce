/*
 * tq.h -- C ABI of a TurboQuant-style compressed KV cache for AMD Instinct
 * MI355X (gfx950): online quantize-append of post-RoPE key/value head vectors
 * into fixed-size pages, and decode attention computed directly over the
 * packed pages.
 *
 * Sources (cited by page title and section):
 *   [Design Study]   "TurboQuant Family Design Study for CPU and Browser WASM
 *                    KV Caches".
 *   [Reconstruction] "Mathematical Reconstruction, Lineage, and Accuracy
 *                    Limits of TurboQuant and TurboVec".
 *   [README]         "TurboQuant: KV Cache Compression for LLM Inference".
 *
 * Conventions shared by every entry point
 *   - All pointers named *_dev, and every pointer inside tq_cache, are device
 *     pointers on the current HIP device; the caller allocates and owns them.
 *     The library never allocates, frees or keeps device memory, and holds no
 *     state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued on it asynchronously; only tq_init_codebooks synchronises.
 *   - Device pointers must be 16-byte aligned; int32 arrays 4-byte aligned.
 *   - Errors found on the host are returned as a tq_status before anything is
 *     enqueued; tq_last_error() then describes the problem.  A launch failure
 *     reported by the HIP runtime returns TQ_ERR_HIP.  Kernels skip (never
 *     write through) page ids outside [0, num_pages), sequence slots outside
 *     [0, max_seqs) and positions beyond max_pages_per_seq * page_tokens; when
 *     tq_cache.status is set they also report each such skip there (device-side
 *     capacity checks, [Design Study] "Paging, lifecycle, and cache identity":
 *     partial pages must not silently corrupt the cache).
 *   - Keys and values are [tokens, num_kv_heads, head_dim] row-major; queries
 *     are [num_seqs, num_q_heads, head_dim]; query head h reads KV head
 *     h / (num_q_heads / num_kv_heads).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARGUMENT = 1,
  TQ_ERR_UNSUPPORTED = 2,
  TQ_ERR_CAPACITY = 3,
  TQ_ERR_HIP = 4
} tq_status;

/* Rotation family ([Design Study] "Dense and structured transform comparison";
 * [Reconstruction] section 5 "Step 2: Random Rotation" and section 9).
 * FWHT: y = H_n D u with seeded Rademacher D and Sylvester-order Hadamard
 * H_n = H / sqrt(d); the QJL projection is S = H D2 H_n D1.
 * DENSE: y = Pi u with Pi the positive-diagonal QR factor of a seeded
 * Gaussian matrix; the QJL projection is an i.i.d. N(0,1) matrix G. */
typedef enum { TQ_ROT_FWHT = 0, TQ_ROT_DENSE = 1 } tq_rotation;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/* Key codec.  QJL: key_bits-1 Lloyd-Max bits plus one QJL sign bit per
 * coordinate, score nu (<Tq, c[idx]> + gamma sqrt(pi/2)/d <STq, 1-2z>)
 * ([Reconstruction] section 6 "The Asymmetric Unbiased Estimator").
 * SCALED_*: all key_bits go to the Lloyd-Max code and one per-vector scale s
 * replaces the residual bit, score s <Tq, c[idx]> ([Reconstruction] "The
 * DRIVE/EDEN Mathematical Critique"; "12. TurboVec Additions and Divergences"
 * item 2): UNBIASED s = nu / <y, c[idx]> (TurboVec's length renormalization,
 * EDEN's unbiased scale), MSE s = nu <y, c[idx]> / ||c[idx]||^2 (EDEN's
 * MSE-optimal scale). */
typedef enum { TQ_KEY_QJL = 0, TQ_KEY_SCALED_UNBIASED = 1, TQ_KEY_SCALED_MSE = 2 } tq_key_mode;

/* Value codec.  LLOYD: rotated Lloyd-Max codes and the fp32 norm.  GROUP: no
 * rotation; per token and 32-coordinate group an fp16 scale and zero (min),
 * uniform codes rint((v - zero) / scale) clamped to [0, 2^b - 1], decided in
 * fp32 ([README] "How It Works" item 4; [Design Study] "Candidate key and
 * value algorithms": the per-token value control arm). */
typedef enum { TQ_VALUE_LLOYD = 0, TQ_VALUE_GROUP = 1 } tq_value_mode;

typedef struct {
  int32_t head_dim;      /* 64, 128 or 256 */
  int32_t num_q_heads;
  int32_t num_kv_heads;  /* num_q_heads % num_kv_heads == 0 */
  int32_t key_bits;      /* bits per key coordinate: TQ_KEY_QJL 2..4 (key_bits-1 Lloyd-Max bits
                            + 1 QJL bit, [Reconstruction] section 6 "The Residual and
                            Bit-Splitting"); scaled key modes 1..4 Lloyd-Max bits */
  int32_t value_bits;    /* 1..4 bits per value coordinate, no QJL */
  int32_t page_tokens;   /* tokens per page; 16 */
  int32_t window;        /* FP16 recent-window tokens: 0 or a multiple of 16 up to 1024
                            ([Design Study] "Packed format and complete bit accounting") */
  int32_t rotation;      /* tq_rotation */
  uint64_t seed;         /* identifies the signs / matrices ([Design Study] "Paging, lifecycle,
                            and cache identity") */
  /* Extended formats ([Design Study] "Packed format and complete bit accounting").  All zero
     selects the default format above. */
  int32_t key_mode;      /* tq_key_mode */
  int32_t value_mode;    /* tq_value_mode */
  int32_t key_bits_hi;   /* 0, or the key_bits of rotated coordinates d/2 .. d-1 (a mixed-channel
                            rate: key_bits 3 and key_bits_hi 4 give 3.5 bits per channel) */
  int32_t value_bits_hi; /* 0, or the value_bits of coordinates d/2 .. d-1 */
  int32_t key_outliers;  /* 0..8 entries of the key outlier sidecar: the coordinates of largest
                            magnitude of each key, kept as (u8 index, fp16 value) with a count
                            byte and removed from the vector before it is quantized
                            ([Design Study] body item 5; [Reconstruction] section 11) */
  int32_t reserved[3];   /* zero */
} tq_config;

/* The paged cache.  Page layout per (page, KV head) block, all little-endian
 * ([Design Study] "Packed format and complete bit accounting";
 * [Reconstruction] section 8 "Bit Accounting and Memory Formulas").  Codes
 * are bit-sliced, lowest code bit first, in 32-bit words; m_g = the Lloyd-Max
 * bits of 32-coordinate group g (key_bits - 1 in the QJL mode, key_bits in
 * the scaled modes, from key_bits_hi for the groups of coordinates >= d/2);
 * b_i = the value bits of coordinate pair i, likewise:
 *   key block   = for token slot t, for group g, for plane j in 0..m_g-1: one
 *                 word whose bit k belongs to coordinate 32g+k, then in the
 *                 QJL mode the group's QJL sign word;
 *                 then (nu_t, gamma_t) float32 pairs for t = 0..page_tokens-1
 *                 (input norm, then the residual norm or the scale s);
 *                 then, with key_outliers = k > 0, per token a record
 *                 [count u8][index u8 x k][pad to even][fp16 value x k][pad to 4].
 *   value block = for coordinate pair i, for plane j in 0..b_i-1: one word
 *                 whose bits 0..15 are plane j of slots 0..15 of coordinate 2i
 *                 and bits 16..31 the same for coordinate 2i+1;
 *                 then nu[page_tokens] float32 (LLOYD), or per token and
 *                 32-coordinate group an (fp16 scale, fp16 zero) pair (GROUP).
 * A QJL bit is 1 where the projected residual is negative.  Bytes of slots at
 * or beyond a sequence's length are unspecified. */
typedef struct {
  void* k_pages;                /* [num_pages][num_kv_heads][tq_key_block_bytes] */
  void* v_pages;                /* [num_pages][num_kv_heads][tq_value_block_bytes] */
  const int32_t* block_table;   /* [max_seqs][max_pages_per_seq] physical page ids, any order */
  void* k_window;               /* fp16 [max_seqs][num_kv_heads][window][head_dim], slot pos % window;
                                   NULL when window == 0 */
  void* v_window;               /* same shape as k_window */
  int32_t num_pages;
  int32_t max_seqs;
  int32_t max_pages_per_seq;
  int32_t reserved;
  uint32_t* status;             /* optional device word (NULL = no reporting); kernels OR in
                                   TQ_STATUS_* bits for work they skipped.  The caller clears
                                   and reads it; the library never resets it. */
} tq_cache;

/* Bits of tq_cache.status. */
enum {
  TQ_STATUS_BAD_SLOT = 1u,   /* a sequence slot outside [0, max_seqs): that sequence was skipped */
  TQ_STATUS_BAD_PAGE = 2u,   /* a block-table entry outside [0, num_pages) where a position was to be
                                written or read: those tokens were skipped */
  TQ_STATUS_CAPACITY = 4u    /* a position at or beyond max_pages_per_seq * page_tokens (append: not
                                written), or a decode length above that or above max_ctx (clamped) */
};

/* Bytes of the parameter blob (codebooks, thresholds, signs or dense
 * matrices) that tq_init_codebooks writes.  0 for an invalid config. */
size_t tq_params_bytes(const tq_config* cfg);

/* Bytes of one (page, KV head) key / value block.  0 for an invalid config. */
size_t tq_key_block_bytes(const tq_config* cfg);
size_t tq_value_block_bytes(const tq_config* cfg);

/* Build the parameter blob on the host and copy it to params_dev
 * (tq_params_bytes(cfg) bytes, caller-owned device memory).
 *   Lloyd-Max codebooks for key_bits-1 and value_bits bits on the exact
 *   rotated-coordinate density f_d(x) ~ (1-x^2)^((d-3)/2) ([Reconstruction]
 *   section 5 "Step 2" and "Step 4: Lloyd-Max Boundaries and Centroids"),
 *   thresholds at centroid midpoints, and the seeded transforms.
 * If params_host_or_null is not NULL the same bytes are also written there;
 * params_dev may then be NULL, which builds the blob on the host only (no
 * device is touched).  Synchronises `stream` before returning. */
tq_status tq_init_codebooks(const tq_config* cfg, void* params_dev, void* params_host_or_null,
                            void* stream);

/* Quantize and append new tokens of num_seqs sequences
 * ([Design Study] "CPU and WASM kernel design": append-time key kernel;
 * [Reconstruction] section 5 steps 1-5 and section 6).
 * For sequence i, tokens cu_new_tokens[i] .. cu_new_tokens[i+1]-1 of k_new /
 * v_new ([total_new][num_kv_heads][head_dim], dtype `dtype`, post-RoPE) take
 * positions ctx_len_before[i] + 0, 1, ... of cache row seq_slots[i].  Every
 * token-head is norm-split, rotated, Lloyd-Max quantized (keys: plus the
 * residual norm and QJL signs) and packed into page
 * block_table[slot][pos / page_tokens], slot pos % page_tokens.  When
 * window > 0 the tokens with pos >= ctx_len_before[i] + n_i - window are also
 * written, as fp16, to ring slot pos % window.
 *   seq_slots, ctx_len_before: device int32[num_seqs];
 *   cu_new_tokens: device int32[num_seqs + 1], cu_new_tokens[0] == 0,
 *   cu_new_tokens[num_seqs] == total_new;
 *   max_new_per_seq: host upper bound on any sequence's new-token count, used
 *   only to size the launch (any value >= 1 gives correct results).
 * The caller must have mapped pages for every position written.  Sequences
 * in one call must use distinct slots. */
tq_status tq_quantize_append(const tq_config* cfg, const void* params_dev, const tq_cache* cache,
                             const void* k_new, const void* v_new, tq_dtype dtype,
                             const int32_t* seq_slots, const int32_t* ctx_len_before,
                             const int32_t* cu_new_tokens, int32_t num_seqs, int32_t total_new,
                             int32_t max_new_per_seq, void* stream);

/* Longest context a decode call accepts (max_ctx); larger values are
 * rejected with TQ_ERR_CAPACITY (and a zero workspace size). */
#define TQ_MAX_CONTEXT (1 << 30)

/* Workspace bytes tq_decode_attention needs for num_seqs sequences whose
 * lengths are at most max_ctx (0 for an invalid config or max_ctx outside
 * [0, TQ_MAX_CONTEXT]). */
size_t tq_decode_workspace_bytes(const tq_config* cfg, int32_t num_seqs, int32_t max_ctx);

/* Decode attention over the compressed cache, one query per sequence
 * ([Design Study] "Capacity model": the query is moved into the keys' rotated
 * basis after RoPE; "CPU and WASM kernel design": decode-time key scan over
 * packed pages and value scan with FP32 accumulation, inverse transform of the
 * final head output only; [Reconstruction] "The Asymmetric Unbiased
 * Estimator").  For sequence i with L = ctx_len[i]:
 *   positions < L - window (all when window == 0) are scored from the packed
 *   pages with est = nu * (<Tq, c[idx]> + gamma * sqrt(pi/2)/d * <S T q, 1-2z>),
 *   positions >= L - window use the fp16 ring exactly;
 *   out = softmax(softmax_scale * scores) . values, values reconstructed in
 *   the rotated domain and rotated back once per head.
 *   q: device [num_seqs][num_q_heads][head_dim] of q_dtype (post-RoPE);
 *   out: device float32 [num_seqs][num_q_heads][head_dim];
 *   workspace: device, >= tq_decode_workspace_bytes(cfg, num_seqs, max_ctx);
 *   logits_or_null: if not NULL, device float32
 *   [num_seqs][num_q_heads][max_ctx] receives softmax_scale * score for
 *   positions < L (debug; slows the call).
 * softmax_scale <= 0 selects 1/sqrt(head_dim).  Rows with L == 0 get zeros.
 * Lengths above max_ctx or above the slot's page capacity are clamped. */
tq_status tq_decode_attention(const tq_config* cfg, const void* params_dev, const tq_cache* cache,
                              const void* q, tq_dtype q_dtype, const int32_t* seq_slots,
                              const int32_t* ctx_len, int32_t num_seqs, int32_t max_ctx,
                              float softmax_scale, float* out, void* workspace,
                              size_t workspace_bytes, float* logits_or_null, void* stream);

/* Bytes of the library-owned decode workspace tq_decode_attention_static
 * uses (one copy per GPU, held until the process ends). */
#define TQ_STATIC_WORKSPACE_BYTES (64u << 20)

/* tq_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, results and errors as
 * tq_decode_attention, except that the workspace is a library-owned device
 * array of TQ_STATIC_WORKSPACE_BYTES per GPU: calls whose
 * tq_decode_workspace_bytes(cfg, num_seqs, max_ctx) exceeds it return
 * TQ_ERR_CAPACITY before anything is enqueued.  Allocates and frees nothing.
 * All calls on one GPU share that array (each call writes every part of it
 * it reads, so nothing needs clearing), so calls that overlap on one GPU --
 * on different streams, or from different threads -- race and must not be
 * issued.  The array's address on the current GPU is looked up on the first
 * call there (tq_init_codebooks does it too, so that a caller that captures
 * the call in a graph can resolve it beforehand). */
tq_status tq_decode_attention_static(const tq_config* cfg, const void* params_dev, const tq_cache* cache,
                                     const void* q, tq_dtype q_dtype, const int32_t* seq_slots,
                                     const int32_t* ctx_len, int32_t num_seqs, int32_t max_ctx,
                                     float softmax_scale, float* out, float* logits_or_null, void* stream);

/* Reconstruct the page-resident keys and values of positions
 * [tok_begin, tok_end) of cache row seq_slot ([Reconstruction] "Step 5":
 * centroid lookup, inverse rotation, scaling by the stored norm; keys also add
 * gamma * sqrt(pi/2)/d * S^T (1-2z), so <q, k~> equals the decode estimate).
 * k_out, v_out: device float32 [tok_end-tok_begin][num_kv_heads][head_dim].
 * For tests and inspection; decode never calls it. */
tq_status tq_dequantize(const tq_config* cfg, const void* params_dev, const tq_cache* cache,
                        int32_t seq_slot, int32_t tok_begin, int32_t tok_end, float* k_out,
                        float* v_out, void* stream);

const char* tq_status_string(tq_status status);

/* Human-readable detail of the last error returned on the calling thread. */
const char* tq_last_error(void);

/* Hash of the sources (include/ and the library's csrc/) this binary was
 * built from, so that a loaded library can be matched to its source tree. */
const char* tq_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
