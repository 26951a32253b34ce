"""CPU-side checks of the C ABI library: it loads, exports every symbol that
include/tq.h declares, builds its parameter blob on the host exactly like the
oracle's independent construction, and rejects bad arguments before touching a
device."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import codebook, layout
from oracle.rotation import Transforms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _tqa():
    import kv_cache_vector_append_amd as tqa
    return tqa


def test_library_exports_every_declared_symbol():
    tqa = _tqa()
    lib = tqa.load_library()
    header = open(os.path.join(ROOT, "include", "tq.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\**(tq_[a-z_0-9]+)\s*\(", header, re.M))
    assert declared == set(tqa.exported_symbols())
    for name in declared:
        assert hasattr(lib, name), name


CASES = [(128, 3, 2, "fwht"), (128, 4, 4, "fwht"), (256, 3, 2, "dense"), (256, 4, 4, "dense"), (64, 2, 1, "fwht")]


@pytest.mark.parametrize("d,kb,vb,rot", CASES)
def test_host_params_match_oracle(d, kb, vb, rot):
    tqa = _tqa()
    cfg = tqa.Config(d, 8, 2, kb, vb, 16, 128, rot, 42)
    blob = np.zeros(tqa.params_bytes(cfg), np.uint8)
    tqa.init_codebooks(cfg, None, blob)
    f = blob.view(np.float32)
    head = blob[:64].view(np.int32)
    assert head[0] == 0x31505154 and head[2] == d and head[3] == kb - 1 and head[4] == vb
    for off, bits in ((16, kb - 1), (48, vb)):
        L = 1 << bits
        c = codebook.lloyd_max(d, bits)
        assert np.abs(f[off:off + L] - c).max() <= 2e-7 * np.abs(c).max()
        t = codebook.thresholds(c)
        assert np.abs(f[off + 16:off + 16 + L - 1] - t).max() <= 2e-7 * np.abs(c).max()
        assert np.all(np.isinf(f[off + 16 + L - 1:off + 32]))
    # bit-plane coefficients reproduce the codebook: c[idx] = sum_S a_S prod_{k in S} s_k
    for off_c, off_a, bits in ((16, 80, kb - 1), (48, 96, vb)):
        L = 1 << bits
        coef = f[off_a:off_a + 16].astype(np.float64)
        c = f[off_c:off_c + L].astype(np.float64)
        for idx in range(L):
            val = 0.0
            for S in range(L):
                sgn = np.prod([(-1.0 if (idx >> k) & 1 else 1.0) for k in range(bits) if (S >> k) & 1])
                val += coef[S] * sgn
            assert abs(val - c[idx]) < 1e-6 * np.abs(c).max()
    T = Transforms(d, rot, 42)
    if rot == "fwht":
        w = blob[1024:1280].view(np.uint32).reshape(4, 16)
        for r, arr in enumerate([T.dk, T.ds1, T.ds2, T.dv]):
            bits = (w[r][np.arange(d) // 32] >> (np.arange(d) % 32).astype(np.uint32)) & 1
            assert np.array_equal(np.where(bits == 1, -1.0, 1.0), arr)
    else:
        M = f[512:512 + 3 * d * d].reshape(3, d, d)
        assert np.abs(M[0] - T.pk).max() < 1e-6
        assert np.abs(M[1] - T.g).max() < 1e-5
        assert np.abs(M[2] - T.pv).max() < 1e-6
        # fp16 hi/lo operands of the matrix-core append: hi + lo = s M to fp32 precision
        h16 = blob[2048 + 12 * d * d:2048 + 24 * d * d].view(np.float16).reshape(3, 2, d, d).astype(np.float64)
        for m, s in enumerate((1024.0, 256.0, 1024.0)):
            ref = s * M[m].astype(np.float64)
            assert np.array_equal(h16[m, 0], ref.astype(np.float16).astype(np.float64))
            assert np.abs(h16[m, 0] + h16[m, 1] - ref).max() <= 2.0 ** -20 * np.abs(ref).max()
        # the decode's query preparation: Pi_K^T and (G Pi_K)^T in fp32
        Mt = f[(2048 + 24 * d * d) // 4:(2048 + 32 * d * d) // 4].reshape(2, d, d).astype(np.float64)
        assert np.abs(Mt[0] - T.pk.T).max() < 1e-6
        gp = (T.g @ T.pk).T
        assert np.abs(Mt[1] - gp).max() <= 2.0 ** -23 * np.abs(gp).max() * 2
        # G^T and Pi_V^T for the short appends: exact transposes of the fp32 matrices
        Mt2 = f[(2048 + 32 * d * d) // 4:(2048 + 40 * d * d) // 4].reshape(2, d, d)
        assert np.array_equal(Mt2[0], M[1].T) and np.array_equal(Mt2[1], M[2].T)


def test_size_queries_match_layout():
    tqa = _tqa()
    for d, kb, vb, rot in CASES:
        cfg = tqa.Config(d, 8, 2, kb, vb, 16, 128, rot, 1)
        from oracle import tq
        f = tq.Config(d, 8, 2, kb, vb)
        assert tqa.key_block_bytes(cfg) == layout.key_block_bytes(f)
        assert tqa.value_block_bytes(cfg) == layout.value_block_bytes(f)
        assert tqa.params_bytes(cfg) == 2048 + (40 * d * d if rot == "dense" else 0)
        ws = tqa.decode_workspace_bytes(cfg, 3, 1000)
        # at least one partial record (max, denominator, d sums) per (sequence, query head)
        # for the compressed part and one for the window, in float32
        assert ws % 4 == 0 and ws >= 2 * 3 * 8 * (2 + d) * 4
        assert tqa.decode_workspace_bytes(cfg, 3, 100000) > ws


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(key_bits=5), dict(value_bits=0), dict(page_tokens=32),
                                 dict(window=100), dict(num_q_heads=12, num_kv_heads=8), dict(num_q_heads=80)])
def test_invalid_configs_are_rejected(bad):
    tqa = _tqa()
    base = dict(head_dim=128, num_q_heads=32, num_kv_heads=8, key_bits=3, value_bits=2, page_tokens=16,
                window=128, rotation="fwht", seed=1)
    base.update(bad)
    cfg = tqa.Config(**base)
    assert tqa.params_bytes(cfg) == 0
    with pytest.raises(tqa.TQError):
        tqa.init_codebooks(cfg, None, np.zeros(4096, np.uint8))


def test_calls_validate_before_touching_a_device():
    tqa = _tqa()
    lib = tqa.load_library()
    cfg = tqa.Config(128, 32, 8, 3, 2, 16, 128, "fwht", 1).c()
    # NULL cache, NULL params, misaligned pointers, too-small workspace: all host-side errors
    assert lib.tq_quantize_append(ctypes.byref(cfg), None, None, None, None, 1, None, None, None, 1, 1, 1, None) == 1
    cache = tqa._lib._Cache(16, 16, 16, 16, 16, 4, 1, 4, 0, None)
    assert lib.tq_quantize_append(ctypes.byref(cfg), 16, ctypes.byref(cache), 17, 16, 1, 16, 16, 16, 1, 1, 1,
                                  None) == 1
    assert lib.tq_decode_attention(ctypes.byref(cfg), 16, ctypes.byref(cache), 16, 1, 16, 16, 1, 100, 0.0, 16, 16,
                                   0, None, None) == 3  # workspace too small
    assert b"workspace" in lib.tq_last_error()
    assert lib.tq_dequantize(ctypes.byref(cfg), 16, ctypes.byref(cache), 5, 0, 1, 16, 16, None) == 1
    assert lib.tq_dequantize(ctypes.byref(cfg), 16, ctypes.byref(cache), 0, 0, 1000, 16, 16, None) == 3
    assert lib.tq_status_string(2) == b"TQ_ERR_UNSUPPORTED"
    # empty work is a no-op that succeeds without a device
    assert lib.tq_quantize_append(ctypes.byref(cfg), 16, ctypes.byref(cache), 16, 16, 1, 16, 16, 16, 0, 0, 1,
                                  None) == 0


def test_build_id_matches_the_sources():
    """The loaded library was built from the sources in this tree."""
    from kv_cache_vector_append_amd import build
    assert _tqa().build_id() == build.source_hash()


def test_context_limit_is_rejected_on_the_host():
    tqa = _tqa()
    lib = tqa.load_library()
    cfg = tqa.Config(128, 32, 8, 3, 2, 16, 128, "fwht", 1)
    # the split plan is computed in 64 bits up to the limit, and refused beyond it
    assert tqa.decode_workspace_bytes(cfg, 2, tqa.TQ_MAX_CONTEXT) > 0
    assert tqa.decode_workspace_bytes(cfg, 2, tqa.TQ_MAX_CONTEXT + 1) == 0
    assert tqa.decode_workspace_bytes(cfg, 2, 2 ** 31 - 1) == 0
    c = cfg.c()
    cache = tqa._lib._Cache(16, 16, 16, 16, 16, 4, 1, 4, 0, None)
    assert lib.tq_decode_attention(ctypes.byref(c), 16, ctypes.byref(cache), 16, 1, 16, 16, 1, 2 ** 31 - 1, 0.0,
                                   16, 16, 1 << 40, None, None) == 3
    assert b"max_ctx" in lib.tq_last_error()
    # a cache whose pages per sequence exceed the limit is refused as well
    big = tqa._lib._Cache(16, 16, 16, 16, 16, 4, 1, (1 << 26) + 1, 0, None)
    assert lib.tq_dequantize(ctypes.byref(c), 16, ctypes.byref(big), 0, 0, 1, 16, 16, None) == 3
    # a misaligned status word is an argument error
    odd = tqa._lib._Cache(16, 16, 16, 16, 16, 4, 1, 4, 0, 18)
    assert lib.tq_dequantize(ctypes.byref(c), 16, ctypes.byref(odd), 0, 0, 1, 16, 16, None) == 1
