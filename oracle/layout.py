"""Byte layout of one (page, KV head) block (oracle side).

[Design Study] "Packed format and complete bit accounting": fixed-token pages
with token-major append order and head-major inner layout; the body holds key
norms, the key main-code stream, the key residual sign stream, value norms and
the value main-code stream, padded to 16 bytes.  [Reconstruction] section 8
"Bit Accounting and Memory Formulas": per vector, TurboQuant_prod stores a
float32 input norm, a float32 residual norm, (b-1) d bits of codes and d sign
bits; TurboQuant_mse stores a float32 norm and b d bits.

READING (bit arrangement, which the pages leave open): codes are stored
bit-sliced, LSB plane first, in 32-bit little-endian words.

Key block, m = key_bits - 1 MSE bits, P tokens, d coordinates:
    for token t, for 32-coordinate group g, for plane j in 0..m: one word whose
    bit k belongs to coordinate 32 g + k; planes 0..m-1 are the code bits,
    plane m the QJL sign bits;  (P * d/32 * (m+1) words)
    then for token t: nu_t, gamma_t as float32 pairs.
Value block, b = value_bits:
    for coordinate pair i (coordinates 2i, 2i+1), for plane j in 0..b-1: one
    word whose bit s is the plane bit of token slot s for coordinate 2i and bit
    16 + s the same for coordinate 2i + 1;  (d/2 * b words, P = 16)
    then nu[P] float32.

A QJL bit is 1 where the projected residual is negative (sign bit convention).
Slots beyond a sequence's length hold unspecified bytes.
"""
import numpy as np


def key_block_bytes(d: int, key_bits: int, P: int = 16) -> int:
    return key_bits * P * d // 8 + 8 * P


def value_block_bytes(d: int, value_bits: int, P: int = 16) -> int:
    return value_bits * P * d // 8 + 4 * P


def _bits_to_words(bits):
    """[..., 32] 0/1 -> [...] uint32, element k at bit k."""
    w = np.zeros(bits.shape[:-1], dtype=np.uint64)
    for k in range(32):
        w |= np.asarray(bits[..., k], dtype=np.uint64) << np.uint64(k)
    return w.astype(np.uint32)


def _words_to_bits(w):
    w = np.asarray(w, dtype=np.uint32)
    return ((w[..., None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8)


def pack_key_block(codes, z, nu, gamma, mse_bits: int):
    """codes [..., P, d] ints in [0, 2^m), z [..., P, d] bool, nu/gamma [..., P] -> uint8 [..., bytes]."""
    codes = np.asarray(codes, dtype=np.int64)
    lead, (P, d) = codes.shape[:-2], codes.shape[-2:]
    m = mse_bits
    planes = [(codes >> j) & 1 for j in range(m)] + [np.asarray(z, dtype=np.int64)]
    # [..., P, d] -> [..., P, d/32, 32] -> words [..., P, d/32]
    words = np.stack([_bits_to_words(pl.reshape(lead + (P, d // 32, 32))) for pl in planes], axis=-1)
    code_bytes = words.astype("<u4").view(np.uint8).reshape(lead + (P * (d // 32) * (m + 1) * 4,))
    norms = np.stack([np.asarray(nu, dtype="<f4"), np.asarray(gamma, dtype="<f4")], axis=-1)
    norm_bytes = norms.view(np.uint8).reshape(lead + (8 * P,))
    return np.concatenate([code_bytes, norm_bytes], axis=-1)


def unpack_key_block(buf, d: int, mse_bits: int, P: int = 16):
    """Inverse of pack_key_block: returns codes [..., P, d] int64, z bool, nu f32, gamma f32."""
    buf = np.asarray(buf, dtype=np.uint8)
    lead = buf.shape[:-1]
    m = mse_bits
    nbytes = P * (d // 32) * (m + 1) * 4
    words = np.ascontiguousarray(buf[..., :nbytes]).view("<u4").reshape(lead + (P, d // 32, m + 1))
    bits = _words_to_bits(words)                       # [..., P, d/32, m+1, 32]
    bits = np.moveaxis(bits, -2, 0)                    # [m+1, ..., P, d/32, 32]
    bits = bits.reshape((m + 1,) + lead + (P, d))
    codes = np.zeros(lead + (P, d), dtype=np.int64)
    for j in range(m):
        codes |= bits[j].astype(np.int64) << j
    z = bits[m].astype(bool)
    norms = np.ascontiguousarray(buf[..., nbytes:nbytes + 8 * P]).view("<f4").reshape(lead + (P, 2))
    return codes, z, norms[..., 0].copy(), norms[..., 1].copy()


def pack_value_block(codes, nu, bits: int):
    codes = np.asarray(codes, dtype=np.int64)
    lead, (P, d) = codes.shape[:-2], codes.shape[-2:]
    assert P == 16, "value masks pack 16 token slots per coordinate"
    out = np.zeros(lead + (d // 2, bits), dtype=np.uint32)
    slots = np.arange(P, dtype=np.uint64)
    for j in range(bits):
        plane = ((codes >> j) & 1).astype(np.uint64)          # [..., P, d]
        masks = (plane << slots[:, None]).sum(axis=-2)        # [..., d] 16-bit masks
        masks = masks.reshape(lead + (d // 2, 2))
        out[..., j] = (masks[..., 0] | (masks[..., 1] << np.uint64(16))).astype(np.uint32)
    code_bytes = out.astype("<u4").view(np.uint8).reshape(lead + (d * bits * 2,))
    nu_bytes = np.asarray(nu, dtype="<f4").view(np.uint8).reshape(lead + (4 * P,))
    return np.concatenate([code_bytes, nu_bytes], axis=-1)


def unpack_value_block(buf, d: int, bits: int, P: int = 16):
    buf = np.asarray(buf, dtype=np.uint8)
    lead = buf.shape[:-1]
    nbytes = d * bits * 2
    words = np.ascontiguousarray(buf[..., :nbytes]).view("<u4").reshape(lead + (d // 2, bits))
    masks = np.stack([words & 0xFFFF, words >> 16], axis=-2)   # [..., d/2, 2, bits]
    masks = masks.reshape(lead + (d, bits))
    slot_bits = (masks[..., None, :] >> np.arange(P, dtype=np.uint32)[:, None]) & 1   # [..., d, P, bits]
    codes = np.zeros(lead + (P, d), dtype=np.int64)
    for j in range(bits):
        codes |= np.swapaxes(slot_bits[..., j], -1, -2).astype(np.int64) << j
    nu = np.ascontiguousarray(buf[..., nbytes:nbytes + 4 * P]).view("<f4").reshape(lead + (P,))
    return codes, nu
