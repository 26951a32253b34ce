"""ctypes binding of the C ABI in include/tq.h (argument marshalling only).

Every step of the quantize-append / decode path runs in the HIP library
``libtq_hip.so``; this module only converts torch tensors to device pointers,
torch streams to hipStream_t, and status codes to exceptions.  There is no
fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq_hip.so")

TQ_OK = 0
TQ_ROT_FWHT, TQ_ROT_DENSE = 0, 1
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
_ROT = {"fwht": TQ_ROT_FWHT, "dense": TQ_ROT_DENSE}
_KEY_MODE = {"qjl": 0, "scaled_unbiased": 1, "scaled_mse": 2}
_VALUE_MODE = {"lloyd": 0, "group": 1}
_DTYPE = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}


class _Config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("key_bits", ctypes.c_int32), ("value_bits", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("window", ctypes.c_int32), ("rotation", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("key_mode", ctypes.c_int32), ("value_mode", ctypes.c_int32), ("key_bits_hi", ctypes.c_int32),
                ("value_bits_hi", ctypes.c_int32), ("key_outliers", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 3)]


class _Cache(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("k_window", ctypes.c_void_p), ("v_window", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("status", ctypes.c_void_p)]


class TQError(RuntimeError):
    pass


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libtq_hip.so (built by ``python -m kv_cache_vector_append_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise TQError(f"{LIB_PATH} is missing; build it with `python -m kv_cache_vector_append_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    cfgp, cachep = ctypes.POINTER(_Config), ctypes.POINTER(_Cache)
    sig = {
        "tq_params_bytes": (SZ, [cfgp]),
        "tq_key_block_bytes": (SZ, [cfgp]),
        "tq_value_block_bytes": (SZ, [cfgp]),
        "tq_init_codebooks": (I32, [cfgp, P, P, P]),
        "tq_quantize_append": (I32, [cfgp, P, cachep, P, P, I32, P, P, P, I32, I32, I32, P]),
        "tq_decode_workspace_bytes": (SZ, [cfgp, I32, I32]),
        "tq_decode_attention": (I32, [cfgp, P, cachep, P, I32, P, P, I32, I32, F32, P, P, SZ, P, P]),
        "tq_decode_attention_static": (I32, [cfgp, P, cachep, P, I32, P, P, I32, I32, F32, P, P, P]),
        "tq_dequantize": (I32, [cfgp, P, cachep, I32, I32, I32, P, P, P]),
        "tq_status_string": (ctypes.c_char_p, [I32]),
        "tq_last_error": (ctypes.c_char_p, []),
        "tq_build_id": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return ["tq_params_bytes", "tq_key_block_bytes", "tq_value_block_bytes", "tq_init_codebooks",
            "tq_quantize_append", "tq_decode_workspace_bytes", "tq_decode_attention", "tq_decode_attention_static",
            "tq_dequantize",
            "tq_status_string", "tq_last_error", "tq_build_id"]


def _check(status: int, what: str):
    if status != TQ_OK:
        lib = load_library()
        raise TQError(f"{what}: {lib.tq_status_string(status).decode()}: {lib.tq_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    return int(t)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclass(frozen=True)
class Config:
    head_dim: int
    num_q_heads: int
    num_kv_heads: int
    key_bits: int
    value_bits: int
    page_tokens: int = 16
    window: int = 0
    rotation: str = "fwht"
    seed: int = 42
    key_mode: str = "qjl"            # "qjl" | "scaled_unbiased" | "scaled_mse"
    value_mode: str = "lloyd"        # "lloyd" | "group"
    key_bits_hi: int = 0             # mixed-channel rate: bits of coordinates d/2.. (0 = key_bits)
    value_bits_hi: int = 0
    key_outliers: int = 0            # key sidecar entries per vector

    def c(self) -> _Config:
        return _Config(self.head_dim, self.num_q_heads, self.num_kv_heads, self.key_bits, self.value_bits,
                       self.page_tokens, self.window, _ROT[self.rotation], self.seed, _KEY_MODE[self.key_mode],
                       _VALUE_MODE[self.value_mode], self.key_bits_hi, self.value_bits_hi, self.key_outliers)


TQ_STATUS_BAD_SLOT, TQ_STATUS_BAD_PAGE, TQ_STATUS_CAPACITY = 1, 2, 4
TQ_MAX_CONTEXT = 1 << 30
TQ_STATIC_WORKSPACE_BYTES = 64 << 20


def build_id() -> str:
    return load_library().tq_build_id().decode()


def params_bytes(cfg: Config) -> int:
    return load_library().tq_params_bytes(ctypes.byref(cfg.c()))


def key_block_bytes(cfg: Config) -> int:
    return load_library().tq_key_block_bytes(ctypes.byref(cfg.c()))


def value_block_bytes(cfg: Config) -> int:
    return load_library().tq_value_block_bytes(ctypes.byref(cfg.c()))


def decode_workspace_bytes(cfg: Config, num_seqs: int, max_ctx: int) -> int:
    return load_library().tq_decode_workspace_bytes(ctypes.byref(cfg.c()), num_seqs, max_ctx)


@dataclass
class CacheBuffers:
    """Device buffers of one paged cache (owned by the caller through torch)."""
    k_pages: torch.Tensor       # uint8 [num_pages, H_kv, key_block]
    v_pages: torch.Tensor       # uint8 [num_pages, H_kv, value_block]
    block_table: torch.Tensor   # int32 [max_seqs, max_pages_per_seq]
    k_window: torch.Tensor | None
    v_window: torch.Tensor | None
    status: torch.Tensor | None = None   # optional int32 [1]: TQ_STATUS_* bits of skipped work

    def c(self) -> _Cache:
        return _Cache(_ptr(self.k_pages), _ptr(self.v_pages), _ptr(self.block_table),
                      _ptr(self.k_window), _ptr(self.v_window), self.k_pages.shape[0],
                      self.block_table.shape[0], self.block_table.shape[1], 0, _ptr(self.status))


def allocate_cache(cfg: Config, num_pages: int, block_table: torch.Tensor, device="cuda") -> CacheBuffers:
    kb, vb = key_block_bytes(cfg), value_block_bytes(cfg)
    H, d = cfg.num_kv_heads, cfg.head_dim
    bt = block_table.to(device=device, dtype=torch.int32).contiguous()
    W = cfg.window
    kw = torch.zeros((bt.shape[0], H, W, d), dtype=torch.float16, device=device) if W else None
    vw = torch.zeros_like(kw) if W else None
    return CacheBuffers(torch.zeros((num_pages, H, kb), dtype=torch.uint8, device=device),
                        torch.zeros((num_pages, H, vb), dtype=torch.uint8, device=device), bt, kw, vw)


def init_codebooks(cfg: Config, params_dev, params_host=None, stream=None):
    """Build the parameter blob; params_dev may be None to fill only params_host (a writable
    uint8 numpy array of params_bytes(cfg) bytes)."""
    host_ptr = None
    if params_host is not None:
        host_ptr = params_host.ctypes.data if hasattr(params_host, "ctypes") else params_host.data_ptr()
    st = _stream(stream) if params_dev is not None else None
    _check(load_library().tq_init_codebooks(ctypes.byref(cfg.c()), _ptr(params_dev), host_ptr, st),
           "tq_init_codebooks")


def quantize_append(cfg: Config, params_dev, cache: CacheBuffers, k_new, v_new, seq_slots, ctx_len_before,
                    cu_new_tokens, max_new_per_seq: int, stream=None):
    cc = cache.c()
    _check(load_library().tq_quantize_append(
        ctypes.byref(cfg.c()), _ptr(params_dev), ctypes.byref(cc), _ptr(k_new), _ptr(v_new), _DTYPE[k_new.dtype],
        _ptr(seq_slots), _ptr(ctx_len_before), _ptr(cu_new_tokens), int(seq_slots.shape[0]), int(k_new.shape[0]),
        int(max_new_per_seq), _stream(stream)), "tq_quantize_append")


def decode_attention(cfg: Config, params_dev, cache: CacheBuffers, q, seq_slots, ctx_len, max_ctx: int, out,
                     workspace, scale: float = 0.0, logits=None, stream=None):
    cc = cache.c()
    _check(load_library().tq_decode_attention(
        ctypes.byref(cfg.c()), _ptr(params_dev), ctypes.byref(cc), _ptr(q), _DTYPE[q.dtype], _ptr(seq_slots),
        _ptr(ctx_len), int(q.shape[0]), int(max_ctx), float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(logits), _stream(stream)), "tq_decode_attention")


def decode_attention_static(cfg: Config, params_dev, cache: CacheBuffers, q, seq_slots, ctx_len, max_ctx: int, out,
                            scale: float = 0.0, logits=None, stream=None):
    """decode_attention with the library-owned workspace (no allocation anywhere)."""
    cc = cache.c()
    _check(load_library().tq_decode_attention_static(
        ctypes.byref(cfg.c()), _ptr(params_dev), ctypes.byref(cc), _ptr(q), _DTYPE[q.dtype], _ptr(seq_slots),
        _ptr(ctx_len), int(q.shape[0]), int(max_ctx), float(scale), _ptr(out), _ptr(logits), _stream(stream)),
        "tq_decode_attention_static")


def dequantize(cfg: Config, params_dev, cache: CacheBuffers, seq_slot: int, tok_begin: int, tok_end: int,
               k_out, v_out, stream=None):
    cc = cache.c()
    _check(load_library().tq_dequantize(
        ctypes.byref(cfg.c()), _ptr(params_dev), ctypes.byref(cc), int(seq_slot), int(tok_begin), int(tok_end),
        _ptr(k_out), _ptr(v_out), _stream(stream)), "tq_dequantize")
