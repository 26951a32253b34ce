"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle scripts.

This module only *describes* workloads and draws their inputs (keys, values,
queries, page orders) from seeded generators.  It holds none of the
quantisation arithmetic: no rotation, codebook, packing or attention code
lives here, so the HIP library and the CPU oracle can both consume the same
inputs without sharing any of the method's code.

Shapes follow the workloads the pages discuss: head_dim 128 and 256 with a
16-token page and a 128-token FP16 recent window ("TurboQuant Family Design
Study for CPU and Browser WASM KV Caches", section "Packed format and complete
bit accounting"), GQA with 8 KV heads, and contexts from 1k to 131k tokens
("TurboQuant: KV Cache Compression for LLM Inference", baseline context table).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np
import torch

# Tokens per generator block.  Every block of keys/values has its own seed, so a
# sampled subset of a long context can be regenerated without drawing the rest.
GEN_BLOCK = 1024


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    key_bits: int          # total key bits per coordinate (MSE bits + 1 QJL bit)
    value_bits: int        # value bits per coordinate (MSE only)
    page_tokens: int
    window: int            # FP16 recent-window tokens (0 = none)
    rotation: str          # "fwht" or "dense"
    input_dtype: str       # "f32" or "bf16"
    decode_seqs: int       # sequences attended by the decode call
    decode_ctx: int        # cached tokens per decode sequence
    prefill_seqs: int = 0  # sequences re-appended inside one step (0 = decode-time append of 1 token)
    prefill_tokens: int = 0
    k_dist: str = "normal"     # "normal" | "normal_head_scale" | "normal_outlier"
    v_dist: str = "normal"     # "normal" | "normal_head_scale" | "student_t3"
    input_seed: int = 1001
    method_seed: int = 42
    outlier_channels: int = 4
    outlier_scale: float = 20.0
    # stored format beyond the default (mixed-channel rates, scaled keys, key
    # outlier sidecar, group-quantized values); see the library's tq_config
    key_mode: str = "qjl"
    value_mode: str = "lloyd"
    key_bits_hi: int = 0
    value_bits_hi: int = 0
    key_outliers: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self):
        return torch.float32 if self.input_dtype == "f32" else torch.bfloat16

    def pages_per_seq(self, ctx: int | None = None) -> int:
        ctx = self.decode_ctx if ctx is None else ctx
        return -(-ctx // self.page_tokens)


WORKLOADS: dict[str, Workload] = {}


def _register(w: Workload) -> Workload:
    WORKLOADS[w.name] = w
    return w


TINY_REF = _register(Workload(
    name="tiny_ref",
    description="1 KV head, d=128, 1024 cached tokens, 1 query; fp32 N(0,1); 3-bit keys / 2-bit values; FWHT; no window",
    num_q_heads=1, num_kv_heads=1, head_dim=128, key_bits=3, value_bits=2,
    page_tokens=16, window=0, rotation="fwht", input_dtype="f32",
    decode_seqs=1, decode_ctx=1024, input_seed=1001))

GQA_DECODE = _register(Workload(
    name="gqa_decode",
    description="batch 1, 32 q / 8 KV heads, d=128, 8192 ctx, bf16 N(0,1) x per-head scale U(0.5,2); 3/2-bit; 16-token pages; FP16 window 128",
    num_q_heads=32, num_kv_heads=8, head_dim=128, key_bits=3, value_bits=2,
    page_tokens=16, window=128, rotation="fwht", input_dtype="bf16",
    decode_seqs=1, decode_ctx=8192, k_dist="normal_head_scale", v_dist="normal_head_scale",
    input_seed=1002))

HD256_DENSE_32 = _register(Workload(
    name="hd256_long_dense_3_2",
    description="batch 8, 16 q / 4 KV heads, d=256, 32768 ctx, bf16 N(0,1); 3/2-bit; dense random orthogonal rotation",
    num_q_heads=16, num_kv_heads=4, head_dim=256, key_bits=3, value_bits=2,
    page_tokens=16, window=128, rotation="dense", input_dtype="bf16",
    decode_seqs=8, decode_ctx=32768, input_seed=1003))

HD256_DENSE_44 = _register(HD256_DENSE_32.replace(
    name="hd256_long_dense_4_4",
    description="batch 8, 16 q / 4 KV heads, d=256, 32768 ctx, bf16 N(0,1); 4/4-bit; dense random orthogonal rotation",
    key_bits=4, value_bits=4))

HD256_FWHT_32 = _register(HD256_DENSE_32.replace(
    name="hd256_long_fwht_3_2",
    description="batch 8, 16 q / 4 KV heads, d=256, 32768 ctx, bf16 N(0,1); 3/2-bit; FWHT rotation (comparison arm)",
    rotation="fwht"))

HD256_DENSE_PREFILL = _register(HD256_DENSE_32.replace(
    name="hd256_dense_prefill",
    description="the head_dim=256 dense 3/2-bit cache written by one append (8 seqs x 32768 tokens, 4 KV heads), "
                "then decoded; the dense rotation's matrix-core workload",
    prefill_seqs=8, prefill_tokens=32768))

OUTLIER_STRESS = _register(Workload(
    name="outlier_stress",
    description="batch 4, 32 q / 8 KV heads, d=128, 131072 ctx; K bf16 N(0,1) with 4 fixed channels per head x20; V Student-t(3); 4/4-bit; FWHT",
    num_q_heads=32, num_kv_heads=8, head_dim=128, key_bits=4, value_bits=4,
    page_tokens=16, window=128, rotation="fwht", input_dtype="bf16",
    decode_seqs=4, decode_ctx=131072, k_dist="normal_outlier", v_dist="student_t3",
    input_seed=1004))

MIXED_SERVING = _register(Workload(
    name="mixed_serving",
    description="append 64 seqs x 4096 new tokens, then decode 256 seqs x 4096 ctx; 32 q / 8 KV heads, d=128, bf16 N(0,1); 3/2-bit; shuffled pages",
    num_q_heads=32, num_kv_heads=8, head_dim=128, key_bits=3, value_bits=2,
    page_tokens=16, window=128, rotation="fwht", input_dtype="bf16",
    decode_seqs=256, decode_ctx=4096, prefill_seqs=64, prefill_tokens=4096,
    input_seed=1005))


# --------------------------------------------------------------------------
# seeded draws


def _gen(seed: int, *stream: int) -> torch.Generator:
    """A CPU generator keyed by (seed, stream...) through a fixed integer hash."""
    with np.errstate(over="ignore"):
        h = np.uint64(seed) * np.uint64(0x9E3779B97F4A7C15)
        for s in stream:
            h = (h ^ np.uint64(s + 0x632BE59BD9B4E019)) * np.uint64(0xBF58476D1CE4E5B9)
            h ^= h >> np.uint64(29)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(h & np.uint64((1 << 63) - 1)))
    return g


_STREAM_K, _STREAM_V, _STREAM_Q, _STREAM_PAGES, _STREAM_HEAD = 1, 2, 3, 4, 5


def head_scales(w: Workload, which: str) -> torch.Tensor:
    """Per-KV-head multipliers ~ U(0.5, 2), drawn separately for keys and values."""
    g = _gen(w.input_seed, _STREAM_HEAD, 0 if which == "k" else 1)
    return 0.5 + 1.5 * torch.rand(w.num_kv_heads, generator=g, dtype=torch.float64)


def outlier_channels(w: Workload) -> torch.Tensor:
    """[H_kv, n] channel indices scaled in every key of that head (fixed across tokens and batch)."""
    g = _gen(w.input_seed, _STREAM_HEAD, 7)
    rows = [torch.randperm(w.head_dim, generator=g)[: w.outlier_channels] for _ in range(w.num_kv_heads)]
    return torch.stack(rows)


def _draw(w: Workload, which: str, shape, g: torch.Generator, device="cpu") -> torch.Tensor:
    """float64 draws [n, H_kv, d] with the workload's distribution for keys or values."""
    dist = w.k_dist if which == "k" else w.v_dist
    x = torch.randn(shape, generator=g, dtype=torch.float64, device=device)
    if dist == "normal_head_scale":
        x = x * head_scales(w, which).to(device).view(1, -1, 1)
    elif dist == "normal_outlier":
        ch = outlier_channels(w)
        scale = torch.ones(w.num_kv_heads, w.head_dim, dtype=torch.float64)
        scale.scatter_(1, ch, w.outlier_scale)
        x = x * scale.to(device).view(1, w.num_kv_heads, w.head_dim)
    elif dist == "student_t3":
        chi2 = (torch.randn((3,) + tuple(shape), generator=g, dtype=torch.float64, device=device) ** 2).sum(0)
        x = x / torch.sqrt(chi2 / 3.0)
    elif dist != "normal":
        raise ValueError(dist)
    return x


def _block(w: Workload, which: str, seq: int, blk: int) -> torch.Tensor:
    """One GEN_BLOCK x H_kv x d float64 block of raw draws for sequence `seq`."""
    g = _gen(w.input_seed, _STREAM_K if which == "k" else _STREAM_V, seq, blk)
    return _draw(w, which, (GEN_BLOCK, w.num_kv_heads, w.head_dim), g)


def kv_tokens(w: Workload, which: str, seq: int, start: int, count: int) -> torch.Tensor:
    """Keys or values for positions [start, start+count) of sequence `seq`.

    Returns a CPU tensor [count, H_kv, d] in the workload's input dtype.  The
    draw for a position does not depend on which range was requested.
    """
    if count <= 0:
        return torch.empty((0, w.num_kv_heads, w.head_dim), dtype=w.torch_dtype)
    b0, b1 = start // GEN_BLOCK, (start + count - 1) // GEN_BLOCK
    parts = [_block(w, which, seq, b) for b in range(b0, b1 + 1)]
    x = torch.cat(parts, 0)[start - b0 * GEN_BLOCK: start - b0 * GEN_BLOCK + count]
    return x.to(w.torch_dtype).contiguous()


def queries(w: Workload, seq: int, step: int = 0) -> torch.Tensor:
    """Query [H_q, d] for sequence `seq` (post-RoPE, N(0,1)) in the input dtype."""
    g = _gen(w.input_seed, _STREAM_Q, seq, step)
    return torch.randn((w.num_q_heads, w.head_dim), generator=g, dtype=torch.float64).to(w.torch_dtype)


def page_permutation(w: Workload, num_pages: int, salt: int = 0) -> torch.Tensor:
    """A seeded random permutation of physical page ids (shuffled page order)."""
    g = _gen(w.input_seed, _STREAM_PAGES, salt)
    return torch.randperm(num_pages, generator=g).to(torch.int32)


def block_table(w: Workload, num_seqs: int, pages_per_seq: int, salt: int = 0) -> torch.Tensor:
    """[num_seqs, pages_per_seq] int32 physical ids, every page used once, in shuffled order."""
    perm = page_permutation(w, num_seqs * pages_per_seq, salt)
    return perm.view(num_seqs, pages_per_seq).contiguous()


def device_generator(w: Workload, salt: int, device) -> torch.Generator:
    """A seeded generator on `device` for benchmark-scale draws."""
    g = torch.Generator(device=device)
    g.manual_seed(int(w.input_seed) * 1000003 + salt)
    return g


def device_kv(w: Workload, which: str, num_tokens: int, g: torch.Generator, device) -> torch.Tensor:
    """Benchmark-scale keys or values [num_tokens, H_kv, d] drawn on the device.

    Same distribution recipe as ``kv_tokens`` (a different random stream), so
    gigabytes of inputs never pass through host memory.
    """
    x = _draw(w, which, (num_tokens, w.num_kv_heads, w.head_dim), g, device)
    return x.to(w.torch_dtype).contiguous()


def device_queries(w: Workload, num_seqs: int, g: torch.Generator, device) -> torch.Tensor:
    x = torch.randn((num_seqs, w.num_q_heads, w.head_dim), generator=g, dtype=torch.float64, device=device)
    return x.to(w.torch_dtype).contiguous()


# Extended stored formats ([Design Study] "Packed format and complete bit
# accounting", "Final recommendation and expected gains"; [Reconstruction]
# "The DRIVE/EDEN Mathematical Critique", "12. TurboVec Additions and
# Divergences", section 11; [README] "How It Works" item 4), on the decode
# shape of the mixed serving step (256 sequences x 4096 tokens, 32 q / 8 KV
# heads, d = 128, bf16 N(0,1)) unless stated.
_EXT_BASE = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_tokens=16, window=128, rotation="fwht",
                 input_dtype="bf16", decode_seqs=256, decode_ctx=4096, input_seed=1006)

MIXED_DECODE = _register(Workload(
    name="mixed_3p5_2p5_decode",
    description="256 x 4096 ctx, 32 q / 8 KV heads, d=128, bf16 N(0,1); mixed-channel rates: keys 3.5 bpc "
                "(64 channels at 2+1 bits, 64 at 3+1), values 2.5 bpc (64 at 2, 64 at 3); FWHT",
    key_bits=3, key_bits_hi=4, value_bits=2, value_bits_hi=3, **_EXT_BASE))

SCALED_DECODE = _register(Workload(
    name="scaled_unbiased_3p5_3_decode",
    description="256 x 4096 ctx, 32 q / 8 KV heads, d=128, bf16 N(0,1); the recommended first product mode: "
                "keys 3.5 bpc all Lloyd-Max with the length-renormalized scale, values 3.0 bpc; FWHT",
    key_mode="scaled_unbiased", key_bits=3, key_bits_hi=4, value_bits=3, **_EXT_BASE))

GROUP_DECODE = _register(Workload(
    name="group_values_decode",
    description="256 x 4096 ctx, 32 q / 8 KV heads, d=128, bf16 N(0,1); 3-bit QJL keys, 2-bit group-quantized "
                "values (fp16 scale and zero per 32 coordinates, no rotation); FWHT",
    key_bits=3, value_bits=2, value_mode="group", **_EXT_BASE))

SIDECAR_DECODE = _register(OUTLIER_STRESS.replace(
    name="outlier_sidecar_decode",
    description="the outlier-stress workload (batch 4, 131072 ctx, 4 fixed channels per head x20, V Student-t(3), "
                "4/4-bit, FWHT) with a 4-entry key outlier sidecar",
    key_outliers=4))
