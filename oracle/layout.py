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

Extended formats (see tq.py): the code planes of a 32-coordinate key group,
or of a value coordinate pair, number the bits of that coordinate's half (a
mixed-channel rate gives the upper half d/2 .. d-1 its own count); the scaled
key modes have no QJL plane and store (nu, s) in place of (nu, gamma); the
key outlier sidecar adds, per token after the norms, a record of
[count u8][index u8 x k][pad to even][fp16 value x k][pad to 4];
group-quantized values store, after the code words, per token and
32-coordinate group an (fp16 scale, fp16 zero) pair in place of nu.

The functions take `fmt`, any object with the format attributes of
tq.Config: head_dim, page_tokens, key_mse_bits, key_mse_bits_hi, qjl,
key_outliers, value_bits, value_bits_hi_, value_mode.
"""
import numpy as np

GROUP = 32


def _key_plane_counts(fmt):
    """Planes per 32-coordinate key group (code bits, plus the QJL plane)."""
    ng = fmt.head_dim // 32
    q = 1 if fmt.qjl else 0
    return [(fmt.key_mse_bits if g < ng // 2 or ng == 1 else fmt.key_mse_bits_hi) + q for g in range(ng)]


def _value_plane_counts(fmt):
    """Planes per value coordinate pair."""
    npair = fmt.head_dim // 2
    return [fmt.value_bits if i < npair // 2 else fmt.value_bits_hi_ for i in range(npair)]


def sidecar_bytes(k: int) -> int:
    if k == 0:
        return 0
    head = 1 + k + ((1 + k) & 1)
    return (head + 2 * k + 3) // 4 * 4


def key_block_bytes(fmt, P: int = 16) -> int:
    return 4 * P * sum(_key_plane_counts(fmt)) + 8 * P + P * sidecar_bytes(fmt.key_outliers)


def value_block_bytes(fmt, P: int = 16) -> int:
    tail = P * (fmt.head_dim // GROUP) * 4 if fmt.value_mode == "group" else 4 * P
    return 4 * sum(_value_plane_counts(fmt)) + tail


def _bits_to_words(bits):
    """[..., 32] 0/1 -> [...] uint32, element k at bit k."""
    w = np.zeros(bits.shape[:-1], dtype=np.uint64)
    for k in range(32):
        w |= np.asarray(bits[..., k], dtype=np.uint64) << np.uint64(k)
    return w.astype(np.uint32)


def _words_to_bits(w):
    w = np.asarray(w, dtype=np.uint32)
    return ((w[..., None] >> np.arange(32, dtype=np.uint32)) & 1).astype(np.uint8)


def pack_key_block(fmt, codes, z, nu, gamma, side_idx=None, side_val=None, side_cnt=None):
    """codes [..., P, d] ints, z [..., P, d] bool, nu/gamma [..., P], sidecar
    [..., P, k] -> uint8 [..., key_block_bytes]."""
    codes = np.asarray(codes, dtype=np.int64)
    lead, (P, d) = codes.shape[:-2], codes.shape[-2:]
    counts = _key_plane_counts(fmt)
    q = 1 if fmt.qjl else 0
    zz = np.asarray(z, dtype=np.int64)
    words = []
    for g, npl in enumerate(counts):
        cg = codes[..., 32 * g:32 * (g + 1)]
        for j in range(npl - q):
            words.append(_bits_to_words((cg >> j) & 1))
        if q:
            words.append(_bits_to_words(zz[..., 32 * g:32 * (g + 1)]))
    code_bytes = np.stack(words, axis=-1).astype("<u4").view(np.uint8).reshape(lead + (P * sum(counts) * 4,))
    norms = np.stack([np.asarray(nu, dtype="<f4"), np.asarray(gamma, dtype="<f4")], axis=-1)
    parts = [code_bytes, norms.view(np.uint8).reshape(lead + (8 * P,))]
    k = fmt.key_outliers
    if k:
        sb = sidecar_bytes(k)
        rec = np.zeros(lead + (P, sb), np.uint8)
        rec[..., 0] = np.asarray(side_cnt, np.uint8)
        rec[..., 1:1 + k] = np.asarray(side_idx, np.uint8)
        voff = 1 + k + ((1 + k) & 1)
        rec[..., voff:voff + 2 * k] = np.ascontiguousarray(np.asarray(side_val, "<f2")).view(np.uint8).reshape(
            lead + (P, 2 * k))
        parts.append(rec.reshape(lead + (P * sb,)))
    return np.concatenate(parts, axis=-1)


def unpack_key_block(fmt, buf):
    """Inverse of pack_key_block: codes [..., P, d] int64, z bool, nu f32, gamma f32,
    side_idx u8 [..., P, k], side_val f16, side_cnt u8."""
    buf = np.asarray(buf, dtype=np.uint8)
    lead = buf.shape[:-1]
    P, d = fmt.page_tokens, fmt.head_dim
    counts = _key_plane_counts(fmt)
    q = 1 if fmt.qjl else 0
    nw = sum(counts)
    words = np.ascontiguousarray(buf[..., :P * nw * 4]).view("<u4").reshape(lead + (P, nw))
    codes = np.zeros(lead + (P, d), dtype=np.int64)
    z = np.zeros(lead + (P, d), dtype=bool)
    off = 0
    for g, npl in enumerate(counts):
        for j in range(npl - q):
            codes[..., 32 * g:32 * (g + 1)] |= _words_to_bits(words[..., off + j]).astype(np.int64) << j
        if q:
            z[..., 32 * g:32 * (g + 1)] = _words_to_bits(words[..., off + npl - 1]).astype(bool)
        off += npl
    nb = P * nw * 4
    norms = np.ascontiguousarray(buf[..., nb:nb + 8 * P]).view("<f4").reshape(lead + (P, 2))
    k = fmt.key_outliers
    side_idx = np.zeros(lead + (P, k), np.uint8)
    side_val = np.zeros(lead + (P, k), np.float16)
    side_cnt = np.zeros(lead + (P,), np.uint8)
    if k:
        sb = sidecar_bytes(k)
        rec = np.ascontiguousarray(buf[..., nb + 8 * P:nb + 8 * P + P * sb]).reshape(lead + (P, sb))
        side_cnt = rec[..., 0].copy()
        side_idx = rec[..., 1:1 + k].copy()
        voff = 1 + k + ((1 + k) & 1)
        side_val = np.ascontiguousarray(rec[..., voff:voff + 2 * k]).view("<f2").reshape(lead + (P, k)).copy()
    return codes, z, norms[..., 0].copy(), norms[..., 1].copy(), side_idx, side_val, side_cnt


def pack_value_block(fmt, codes, nu, scale=None, zero=None):
    codes = np.asarray(codes, dtype=np.int64)
    lead, (P, d) = codes.shape[:-2], codes.shape[-2:]
    assert P == 16, "value masks pack 16 token slots per coordinate"
    slots = np.arange(P, dtype=np.uint64)
    words = []
    for i, b in enumerate(_value_plane_counts(fmt)):
        for j in range(b):
            plane = ((codes[..., 2 * i:2 * i + 2] >> j) & 1).astype(np.uint64)     # [..., P, 2]
            masks = (plane << slots[:, None]).sum(axis=-2)                          # [..., 2]
            words.append((masks[..., 0] | (masks[..., 1] << np.uint64(16))).astype(np.uint32))
    code_bytes = np.stack(words, axis=-1).astype("<u4").view(np.uint8).reshape(lead + (4 * len(words),))
    if fmt.value_mode == "group":
        tail = np.stack([np.asarray(scale, "<f2"), np.asarray(zero, "<f2")], axis=-1)     # [..., P, d/32, 2]
        tail = np.ascontiguousarray(tail).view(np.uint8).reshape(lead + (P * (d // GROUP) * 4,))
    else:
        tail = np.asarray(nu, dtype="<f4").view(np.uint8).reshape(lead + (4 * P,))
    return np.concatenate([code_bytes, tail], axis=-1)


def unpack_value_block(fmt, buf):
    """Inverse of pack_value_block: codes [..., P, d] int64, nu f32 [..., P],
    scale / zero f16 [..., P, d/32] (zeros in the mode that does not store them)."""
    buf = np.asarray(buf, dtype=np.uint8)
    lead = buf.shape[:-1]
    P, d = fmt.page_tokens, fmt.head_dim
    counts = _value_plane_counts(fmt)
    nw = sum(counts)
    words = np.ascontiguousarray(buf[..., :4 * nw]).view("<u4").reshape(lead + (nw,))
    codes = np.zeros(lead + (P, d), dtype=np.int64)
    slot = np.arange(P, dtype=np.uint32)
    off = 0
    for i, b in enumerate(counts):
        for j in range(b):
            w = words[..., off + j]
            for h in range(2):
                bits = ((w[..., None] >> (slot + np.uint32(16 * h))) & 1).astype(np.int64)      # [..., P]
                codes[..., 2 * i + h] |= bits << j
        off += b
    nb = 4 * nw
    nu = np.zeros(lead + (P,), np.float32)
    scale = np.zeros(lead + (P, d // GROUP), np.float16)
    zero = np.zeros(lead + (P, d // GROUP), np.float16)
    if fmt.value_mode == "group":
        t = np.ascontiguousarray(buf[..., nb:nb + P * (d // GROUP) * 4]).view("<f2").reshape(lead + (P, d // GROUP, 2))
        scale, zero = t[..., 0].copy(), t[..., 1].copy()
    else:
        nu = np.ascontiguousarray(buf[..., nb:nb + 4 * P]).view("<f4").reshape(lead + (P,)).copy()
    return codes, nu, scale, zero
