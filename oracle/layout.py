"""Byte layout of one (page, KV head) block (oracle side).

[Design Study] "Packed format and complete bit accounting": fixed-token pages
with token-major append order and head-major inner layout; the body holds key
norms, the key main-code stream, the key residual sign stream, value norms and
the value main-code stream, padded to 16 bytes.  [Reconstruction] section 8
"Bit Accounting and Memory Formulas": per vector, TurboQuant_prod stores a
float32 input norm, a float32 residual norm, (b-1) d bits of codes and d sign
bits; TurboQuant_mse stores a float32 norm and b d bits.

READING (bit order, which the pages leave open): codes are stored bit-sliced,
one plane per code bit, LSB first.

Key block, m = key_bits - 1 MSE bits, P tokens, d coordinates:
    m code planes, then 1 QJL sign plane; each plane is P rows of d/8 bytes,
    row t holding bit j of coordinate i at byte i // 8, bit i % 8 (so in a
    little-endian 32-bit word w, coordinate 32 w + k sits at bit k);
    then nu[P] float32, then gamma[P] float32.
Value block, b = value_bits:
    b code planes; each plane is d rows of P/8 bytes, row i holding, at bit t,
    the plane bit of token slot t for coordinate i;
    then nu[P] float32.

A QJL bit is 1 where the projected residual is negative (sign bit convention).
Slots beyond a sequence's length hold unspecified bytes.
"""
import numpy as np


def key_block_bytes(d: int, key_bits: int, P: int = 16) -> int:
    return key_bits * P * d // 8 + 8 * P


def value_block_bytes(d: int, value_bits: int, P: int = 16) -> int:
    return value_bits * P * d // 8 + 4 * P


def _bits_to_bytes(bits):
    """[..., n] 0/1 -> [..., n/8] uint8, LSB first."""
    return np.packbits(np.asarray(bits, dtype=np.uint8), axis=-1, bitorder="little")


def _bytes_to_bits(b, n):
    return np.unpackbits(np.asarray(b, dtype=np.uint8), axis=-1, bitorder="little", count=n)


def pack_key_block(codes, z, nu, gamma, mse_bits: int):
    """codes [..., P, d] ints in [0, 2^m), z [..., P, d] bool, nu/gamma [..., P] -> uint8 [..., bytes]."""
    codes = np.asarray(codes, dtype=np.int64)
    lead, (P, d) = codes.shape[:-2], codes.shape[-2:]
    parts = []
    for j in range(mse_bits):
        parts.append(_bits_to_bytes((codes >> j) & 1).reshape(lead + (P * d // 8,)))
    parts.append(_bits_to_bytes(np.asarray(z, dtype=np.uint8)).reshape(lead + (P * d // 8,)))
    parts.append(np.asarray(nu, dtype="<f4").view(np.uint8).reshape(lead + (4 * P,)))
    parts.append(np.asarray(gamma, dtype="<f4").view(np.uint8).reshape(lead + (4 * P,)))
    return np.concatenate(parts, axis=-1)


def unpack_key_block(buf, d: int, mse_bits: int, P: int = 16):
    """Inverse of pack_key_block: returns codes [..., P, d] int64, z bool, nu f32, gamma f32."""
    buf = np.asarray(buf, dtype=np.uint8)
    lead = buf.shape[:-1]
    plane = P * d // 8
    codes = np.zeros(lead + (P, d), dtype=np.int64)
    for j in range(mse_bits):
        raw = buf[..., j * plane:(j + 1) * plane].reshape(lead + (P, d // 8))
        codes |= _bytes_to_bits(raw, d).astype(np.int64) << j
    raw = buf[..., mse_bits * plane:(mse_bits + 1) * plane].reshape(lead + (P, d // 8))
    z = _bytes_to_bits(raw, d).astype(bool)
    off = (mse_bits + 1) * plane
    nu = np.ascontiguousarray(buf[..., off:off + 4 * P]).view("<f4").reshape(lead + (P,))
    gamma = np.ascontiguousarray(buf[..., off + 4 * P:off + 8 * P]).view("<f4").reshape(lead + (P,))
    return codes, z, nu, gamma


def pack_value_block(codes, nu, bits: int):
    codes = np.asarray(codes, dtype=np.int64)
    lead, (P, d) = codes.shape[:-2], codes.shape[-2:]
    parts = []
    for j in range(bits):
        plane = (codes >> j) & 1                       # [..., P, d]
        plane_t = np.swapaxes(plane, -1, -2)           # [..., d, P]
        parts.append(_bits_to_bytes(plane_t).reshape(lead + (d * P // 8,)))
    parts.append(np.asarray(nu, dtype="<f4").view(np.uint8).reshape(lead + (4 * P,)))
    return np.concatenate(parts, axis=-1)


def unpack_value_block(buf, d: int, bits: int, P: int = 16):
    buf = np.asarray(buf, dtype=np.uint8)
    lead = buf.shape[:-1]
    plane = P * d // 8
    codes = np.zeros(lead + (P, d), dtype=np.int64)
    for j in range(bits):
        raw = buf[..., j * plane:(j + 1) * plane].reshape(lead + (d, P // 8))
        bt = _bytes_to_bits(raw, P)                      # [..., d, P]
        codes |= np.swapaxes(bt, -1, -2).astype(np.int64) << j
    off = bits * plane
    nu = np.ascontiguousarray(buf[..., off:off + 4 * P]).view("<f4").reshape(lead + (P,))
    return codes, nu
