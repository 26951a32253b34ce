// The exported C ABI: argument validation on the host, then one launcher call.
// No device memory is allocated or freed here.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "tq_internal.h"

#ifndef TQ_SOURCE_HASH
#error "TQ_SOURCE_HASH (hash of the library sources) must be defined by the build"
#endif

namespace {

thread_local char g_last_error[512] = "";

tq_status fail(tq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

tq_status hip_fail(int err, const char* what) {
  return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(err)));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

tq_status check_config(const tq_config* c) {
  if (!c) return fail(TQ_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(TQ_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128, 256)", c->head_dim);
  if (c->num_kv_heads <= 0 || c->num_q_heads <= 0 || c->num_q_heads % c->num_kv_heads)
    return fail(TQ_ERR_INVALID_ARGUMENT, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                c->num_q_heads, c->num_kv_heads);
  if (c->num_q_heads / c->num_kv_heads > 8)
    return fail(TQ_ERR_UNSUPPORTED, "GQA group of %d query heads per kv head (max 8)",
                c->num_q_heads / c->num_kv_heads);
  if (c->key_mode != TQ_KEY_QJL && c->key_mode != TQ_KEY_SCALED_UNBIASED && c->key_mode != TQ_KEY_SCALED_MSE)
    return fail(TQ_ERR_INVALID_ARGUMENT, "key_mode %d unknown", c->key_mode);
  if (c->value_mode != TQ_VALUE_LLOYD && c->value_mode != TQ_VALUE_GROUP)
    return fail(TQ_ERR_INVALID_ARGUMENT, "value_mode %d unknown", c->value_mode);
  const int kmin = c->key_mode == TQ_KEY_QJL ? 2 : 1;
  if (c->key_bits < kmin || c->key_bits > 4)
    return fail(TQ_ERR_UNSUPPORTED, "key_bits %d not in %d..4", c->key_bits, kmin);
  if (c->key_bits_hi != 0 && (c->key_bits_hi < kmin || c->key_bits_hi > 4))
    return fail(TQ_ERR_UNSUPPORTED, "key_bits_hi %d not 0 or in %d..4", c->key_bits_hi, kmin);
  if (c->value_bits < 1 || c->value_bits > 4)
    return fail(TQ_ERR_UNSUPPORTED, "value_bits %d not in 1..4", c->value_bits);
  if (c->value_bits_hi < 0 || c->value_bits_hi > 4)
    return fail(TQ_ERR_UNSUPPORTED, "value_bits_hi %d not 0 or in 1..4", c->value_bits_hi);
  if (c->key_outliers < 0 || c->key_outliers > tqi::kMaxOutliers)
    return fail(TQ_ERR_UNSUPPORTED, "key_outliers %d not in 0..%d", c->key_outliers, tqi::kMaxOutliers);
  if (c->reserved[0] || c->reserved[1] || c->reserved[2])
    return fail(TQ_ERR_INVALID_ARGUMENT, "reserved config fields must be zero");
  if (c->page_tokens != 16) return fail(TQ_ERR_UNSUPPORTED, "page_tokens %d not supported (16)", c->page_tokens);
  if (c->window < 0 || c->window > 1024 || c->window % 16)
    return fail(TQ_ERR_UNSUPPORTED, "window %d must be 0 or a multiple of 16 up to 1024", c->window);
  if (c->rotation != TQ_ROT_FWHT && c->rotation != TQ_ROT_DENSE)
    return fail(TQ_ERR_INVALID_ARGUMENT, "rotation %d unknown", c->rotation);
  return TQ_OK;
}

tq_status check_cache(const tq_config* c, const tq_cache* k) {
  if (!k) return fail(TQ_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!k->k_pages || !k->v_pages || !k->block_table)
    return fail(TQ_ERR_INVALID_ARGUMENT, "cache pages / block table are NULL");
  if (!aligned16(k->k_pages) || !aligned16(k->v_pages) || !aligned4(k->block_table))
    return fail(TQ_ERR_INVALID_ARGUMENT, "cache pointers misaligned");
  if (k->num_pages <= 0 || k->max_seqs <= 0 || k->max_pages_per_seq <= 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "cache sizes must be positive");
  if ((long long)k->max_pages_per_seq * c->page_tokens > TQ_MAX_CONTEXT)
    return fail(TQ_ERR_CAPACITY, "max_pages_per_seq %d x %d tokens above %d", k->max_pages_per_seq, c->page_tokens,
                TQ_MAX_CONTEXT);
  if (c->window > 0 && (!k->k_window || !k->v_window || !aligned16(k->k_window) || !aligned16(k->v_window)))
    return fail(TQ_ERR_INVALID_ARGUMENT, "window > 0 needs 16-byte aligned k_window / v_window");
  if (k->status && !aligned4(k->status)) return fail(TQ_ERR_INVALID_ARGUMENT, "status word misaligned");
  return TQ_OK;
}

tqi::CacheView view(const tq_config* c, const tq_cache* k) {
  tqi::CacheView v{};
  v.k_pages = static_cast<uint8_t*>(k->k_pages);
  v.v_pages = static_cast<uint8_t*>(k->v_pages);
  v.block_table = k->block_table;
  v.k_window = static_cast<uint16_t*>(k->k_window);
  v.v_window = static_cast<uint16_t*>(k->v_window);
  v.num_pages = k->num_pages;
  v.max_seqs = k->max_seqs;
  v.max_pages_per_seq = k->max_pages_per_seq;
  v.num_kv_heads = c->num_kv_heads;
  v.page_tokens = c->page_tokens;
  v.window = c->window;
  v.codec = tqi::make_codec(*c);
  v.key_block = v.codec.key_block;
  v.value_block = v.codec.value_block;
  v.status = k->status;
  return v;
}

}  // namespace

extern "C" {

size_t tq_params_bytes(const tq_config* cfg) {
  if (check_config(cfg) != TQ_OK) return 0;
  return tqi::params_bytes(cfg->head_dim, cfg->rotation);
}

size_t tq_key_block_bytes(const tq_config* cfg) {
  if (check_config(cfg) != TQ_OK) return 0;
  return tqi::key_block_bytes(*cfg);
}

size_t tq_value_block_bytes(const tq_config* cfg) {
  if (check_config(cfg) != TQ_OK) return 0;
  return tqi::value_block_bytes(*cfg);
}

tq_status tq_init_codebooks(const tq_config* cfg, void* params_dev, void* params_host_or_null, void* stream) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (!params_dev && !params_host_or_null) return fail(TQ_ERR_INVALID_ARGUMENT, "no destination for params");
  if (params_dev && !aligned16(params_dev)) return fail(TQ_ERR_INVALID_ARGUMENT, "params_dev misaligned");
  const size_t n = tqi::params_bytes(cfg->head_dim, cfg->rotation);
  std::vector<uint8_t> blob(n);
  tqi::build_params(*cfg, blob.data());
  if (params_host_or_null) std::memcpy(params_host_or_null, blob.data(), n);
  if (!params_dev) return TQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(params_dev, blob.data(), n, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(params)");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  // resolve this GPU's library-owned decode workspace now, outside any graph capture
  void* ws = nullptr;
  const int we = tqi::static_workspace(&ws);
  if (we != 0) return hip_fail(we, "library-owned workspace lookup");
  return TQ_OK;
}

tq_status tq_quantize_append(const tq_config* cfg, const void* params_dev, const tq_cache* cache, const void* k_new,
                             const void* v_new, tq_dtype dtype, const int32_t* seq_slots,
                             const int32_t* ctx_len_before, const int32_t* cu_new_tokens, int32_t num_seqs,
                             int32_t total_new, int32_t max_new_per_seq, void* stream) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != TQ_OK) return st;
  if (!params_dev || !aligned16(params_dev)) return fail(TQ_ERR_INVALID_ARGUMENT, "params_dev NULL or misaligned");
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return fail(TQ_ERR_INVALID_ARGUMENT, "bad dtype");
  if (num_seqs < 0 || total_new < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "negative sizes");
  if (num_seqs == 0 || total_new == 0) return TQ_OK;
  if (!k_new || !v_new || !seq_slots || !ctx_len_before || !cu_new_tokens)
    return fail(TQ_ERR_INVALID_ARGUMENT, "NULL input pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned4(seq_slots) || !aligned4(ctx_len_before) ||
      !aligned4(cu_new_tokens))
    return fail(TQ_ERR_INVALID_ARGUMENT, "input pointers misaligned");
  if (max_new_per_seq < 1) max_new_per_seq = 1;
  tqi::AppendArgs a{};
  a.cache = view(cfg, cache);
  a.params = static_cast<const uint8_t*>(params_dev);
  a.k_new = k_new;
  a.v_new = v_new;
  a.seq_slots = seq_slots;
  a.ctx_len_before = ctx_len_before;
  a.cu_new_tokens = cu_new_tokens;
  a.num_seqs = num_seqs;
  a.dtype = dtype;
  a.key_mse_bits = cfg->key_bits - 1;
  a.value_bits = cfg->value_bits;
  if ((long long)num_seqs * cfg->num_kv_heads * ((max_new_per_seq + 15) / 16 + 1) > 0x7fffffffLL)
    return fail(TQ_ERR_CAPACITY, "append launch too large");
  const int e = a.cache.codec.ext ? tqi::launch_append_codec(*cfg, a, num_seqs, max_new_per_seq, stream)
                                  : tqi::launch_append(*cfg, a, num_seqs, max_new_per_seq, stream);
  if (e != 0) return hip_fail(e, "append launch");
  return TQ_OK;
}

size_t tq_decode_workspace_bytes(const tq_config* cfg, int32_t num_seqs, int32_t max_ctx) {
  if (check_config(cfg) != TQ_OK || num_seqs <= 0 || max_ctx < 0 || max_ctx > TQ_MAX_CONTEXT) return 0;
  const tqi::SplitPlan p = tqi::plan_splits(*cfg, num_seqs, max_ctx > 0 ? max_ctx : 1);
  const size_t partials =
      size_t(num_seqs) * cfg->num_q_heads * (p.splits + tqi::kWindowRecords) * (2 + 2 * size_t(cfg->head_dim)) *
      sizeof(float);
  return tqi::decode_prep_bytes(*cfg, num_seqs) + partials;
}

}  // extern "C"

namespace {

// Validation and launch shared by tq_decode_attention and
// tq_decode_attention_static; `workspace` NULL selects the library-owned one.
tq_status decode(const tq_config* cfg, const void* params_dev, const tq_cache* cache, const void* q,
                 tq_dtype q_dtype, const int32_t* seq_slots, const int32_t* ctx_len, int32_t num_seqs,
                 int32_t max_ctx, float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                 float* logits_or_null, void* stream, bool library_workspace) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != TQ_OK) return st;
  if (!params_dev || !aligned16(params_dev)) return fail(TQ_ERR_INVALID_ARGUMENT, "params_dev NULL or misaligned");
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return fail(TQ_ERR_INVALID_ARGUMENT, "bad dtype");
  if (num_seqs < 0 || max_ctx < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "negative sizes");
  if (max_ctx > TQ_MAX_CONTEXT) return fail(TQ_ERR_CAPACITY, "max_ctx %d above %d", max_ctx, TQ_MAX_CONTEXT);
  if (num_seqs == 0) return TQ_OK;
  if (!q || !seq_slots || !ctx_len || !out || (!library_workspace && !workspace))
    return fail(TQ_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!aligned16(q) || !aligned16(out) || (!library_workspace && !aligned16(workspace)) || !aligned4(seq_slots) ||
      !aligned4(ctx_len))
    return fail(TQ_ERR_INVALID_ARGUMENT, "pointers misaligned");
  if (logits_or_null && !aligned4(logits_or_null)) return fail(TQ_ERR_INVALID_ARGUMENT, "logits misaligned");
  const int mc = max_ctx > 0 ? max_ctx : 1;
  const size_t need = tq_decode_workspace_bytes(cfg, num_seqs, mc);
  if (library_workspace) {
    if (need > TQ_STATIC_WORKSPACE_BYTES)
      return fail(TQ_ERR_CAPACITY, "decode needs %zu workspace bytes, above the library-owned %u", need,
                  unsigned(TQ_STATIC_WORKSPACE_BYTES));
    const int e = tqi::static_workspace(&workspace);
    if (e != 0) return hip_fail(e, "library-owned workspace lookup");
    workspace_bytes = TQ_STATIC_WORKSPACE_BYTES;
  }
  if (workspace_bytes < need)
    return fail(TQ_ERR_CAPACITY, "workspace %zu bytes < %zu required", workspace_bytes, need);
  const tqi::SplitPlan p = tqi::plan_splits(*cfg, num_seqs, mc);
  tqi::DecodeArgs a{};
  a.cache = view(cfg, cache);
  a.params = static_cast<const uint8_t*>(params_dev);
  a.q = q;
  a.seq_slots = seq_slots;
  a.ctx_len = ctx_len;
  a.out = out;
  a.workspace = static_cast<float*>(workspace);
  a.logits = logits_or_null;
  a.num_seqs = num_seqs;
  a.num_q_heads = cfg->num_q_heads;
  a.q_dtype = q_dtype;
  a.key_mse_bits = cfg->key_bits - 1;
  a.value_bits = cfg->value_bits;
  a.splits = p.splits;
  a.split_tokens = p.split_tokens;
  a.window_items = p.window_items;
  a.max_ctx = mc;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(cfg->head_dim));
  const int e = tqi::decode_mfma_supported(*cfg) ? tqi::launch_decode_mfma(*cfg, a, stream)
                                                 : tqi::launch_decode_codec(*cfg, a, stream);
  if (e != 0) return hip_fail(e, "decode launch");
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_decode_attention(const tq_config* cfg, const void* params_dev, const tq_cache* cache, const void* q,
                              tq_dtype q_dtype, const int32_t* seq_slots, const int32_t* ctx_len,
                              int32_t num_seqs, int32_t max_ctx, float softmax_scale, float* out,
                              void* workspace, size_t workspace_bytes, float* logits_or_null, void* stream) {
  return decode(cfg, params_dev, cache, q, q_dtype, seq_slots, ctx_len, num_seqs, max_ctx, softmax_scale, out,
                workspace, workspace_bytes, logits_or_null, stream, false);
}

tq_status tq_decode_attention_static(const tq_config* cfg, const void* params_dev, const tq_cache* cache,
                                     const void* q, tq_dtype q_dtype, const int32_t* seq_slots,
                                     const int32_t* ctx_len, int32_t num_seqs, int32_t max_ctx,
                                     float softmax_scale, float* out, float* logits_or_null, void* stream) {
  return decode(cfg, params_dev, cache, q, q_dtype, seq_slots, ctx_len, num_seqs, max_ctx, softmax_scale, out,
                nullptr, 0, logits_or_null, stream, true);
}

tq_status tq_dequantize(const tq_config* cfg, const void* params_dev, const tq_cache* cache, int32_t seq_slot,
                        int32_t tok_begin, int32_t tok_end, float* k_out, float* v_out, void* stream) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if ((st = check_cache(cfg, cache)) != TQ_OK) return st;
  if (!params_dev || !aligned16(params_dev)) return fail(TQ_ERR_INVALID_ARGUMENT, "params_dev NULL or misaligned");
  if (seq_slot < 0 || seq_slot >= cache->max_seqs) return fail(TQ_ERR_INVALID_ARGUMENT, "seq_slot out of range");
  if (tok_begin < 0 || tok_end < tok_begin) return fail(TQ_ERR_INVALID_ARGUMENT, "bad token range");
  if ((long long)tok_end > (long long)cache->max_pages_per_seq * cfg->page_tokens)
    return fail(TQ_ERR_CAPACITY, "token range beyond the sequence's page capacity");
  if (tok_end == tok_begin) return TQ_OK;
  if (!k_out || !v_out || !aligned16(k_out) || !aligned16(v_out))
    return fail(TQ_ERR_INVALID_ARGUMENT, "outputs NULL or misaligned");
  tqi::DequantArgs a{};
  a.cache = view(cfg, cache);
  a.params = static_cast<const uint8_t*>(params_dev);
  a.k_out = k_out;
  a.v_out = v_out;
  a.seq_slot = seq_slot;
  a.tok_begin = tok_begin;
  a.tok_end = tok_end;
  a.key_mse_bits = cfg->key_bits - 1;
  a.value_bits = cfg->value_bits;
  const int e = tqi::launch_dequantize_codec(*cfg, a, stream);
  if (e != 0) return hip_fail(e, "dequantize launch");
  return TQ_OK;
}

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARGUMENT: return "TQ_ERR_INVALID_ARGUMENT";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_CAPACITY: return "TQ_ERR_CAPACITY";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
  }
  return "TQ_UNKNOWN";
}

const char* tq_last_error(void) { return g_last_error; }

const char* tq_build_id(void) { return TQ_SOURCE_HASH; }

}  // extern "C"
