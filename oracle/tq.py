"""The method, step by step, in float64 (oracle side).

Append, per post-RoPE key or value head vector x ([Design Study] "Capacity
model": keys are quantised after RoPE and the query is moved into the same
basis since q.k = (Tq).(Tk); [Reconstruction] sections 5 and 6):

  1. norm separation: nu = ||x||, u = x / nu          ("Step 1: Norm Separation")
  2. rotation: y = T u                                 ("Step 2: Random Rotation")
  3. scalar quantisation per coordinate with the Lloyd-Max codebook of the
     rotated marginal: idx_i = #{j : t_j < y_i}, yhat = c[idx]
                                                       ("Step 4", "Step 5")
  4. keys only, TurboQuant_prod: b-1 MSE bits, residual e = y - yhat, its norm
     gamma = ||e||, and one QJL bit per coordinate z = [S e < 0]
                                                       ("The Residual and Bit-Splitting",
                                                        "The 1-Bit QJL Transform")
  5. bit packing into fixed-size pages (see ``layout``), and the last W tokens
     also kept in FP16 ([Design Study] "Packed format and complete bit
     accounting": last W = 128 tokens remain FP16 for K and V).

Decode ([Design Study] "CPU and WASM kernel design": transform the live query
once, score packed key codes without a history-sized dequant buffer, then
stream value pages and accumulate in FP32, inverse-transforming only the final
head output; [Reconstruction] "The Asymmetric Unbiased Estimator"):

  qt = T_K q,  qh = S qt
  est_t = nu_t * ( <qt, c_K[idx_t]> + gamma_t * sqrt(pi/2) / d * <qh, 1 - 2 z_t> )
  logits = scale * est (window tokens: scale * <q, k_w>), softmax,
  out = T_V^T ( sum_t p_t nu_V,t c_V[idx_V,t] ) + sum_w p_w v_w.

Extended modes (the next items the pages rank after the method above):

  * mixed-channel rates ([Design Study] "Packed format and complete bit
    accounting": a fractional nominal rate is an exact split of the channels,
    e.g. 3.5 bits per channel = 64 channels at 3 bits + 64 at 4 bits at
    d = 128, with no entropy coding).  READING: after the random rotation all
    coordinates are exchangeable, so the split is positional: rotated
    coordinates 0 .. d/2 - 1 use the lower rate (key_bits, value_bits) and
    d/2 .. d - 1 the upper one (key_bits_hi, value_bits_hi), each with the
    Lloyd-Max codebook of its own bit count; the QJL bit, when present,
    covers every coordinate;
  * scale-corrected keys instead of the QJL bit ([Reconstruction] "The
    DRIVE/EDEN Mathematical Critique"; "12. TurboVec Additions and
    Divergences" item 2, length-renormalized scoring): all key bits go to the
    Lloyd-Max code and one per-vector scale replaces the norm in the score,
    est = s <qt, yhat>.  key_mode "scaled_unbiased": s = nu / <y, yhat>
    (TurboVec's correction, which is also EDEN's unbiased scale: E[s yhat]
    reconstructs y); "scaled_mse": s = nu <y, yhat> / ||yhat||^2 (EDEN's
    MSE-optimal scale).  The formulas are images on the page; READING: these
    are the scales that restore unbiasedness and minimise the squared error
    respectively, and with them the page's asymptotic 1-bit variances
    (QJL pi/2 against EDEN pi/2 - 1, the "2.75x") are reproduced by the pins;
  * key outlier sidecar ([Design Study] "Packed format and complete bit
    accounting", body item 5: repeated (u8 index, fp16 value) pairs plus a
    count byte; [Reconstruction] "11. Finite-Dimension and Adversarial
    Analysis": outlier channels skew the rotated distribution).  READING: a
    fixed capacity of key_outliers entries per key vector; the entries are the
    coordinates of largest magnitude of the post-RoPE key (ties to the lower
    index), their values kept in fp16 and removed (set to zero) from the
    vector that is then norm-split, rotated and quantized; the count is the
    number of those coordinates that are nonzero.  The score adds
    sum_j q[idx_j] val_j;
  * group-quantized values as the control arm ([README] "How It Works" item 4:
    per-group scales and zeros; [Design Study] "Candidate key and value
    algorithms": a per-token value baseline).  READING: per token, groups of
    32 coordinates, no rotation; in float32: scale = (max - min) / (2^b - 1)
    and zero = min, both rounded to fp16, code = clamp(rint((v - zero) /
    scale), 0, 2^b - 1) (a group whose fp16 scale is 0 stores code 0);
    v~ = zero + scale * code.  The decisions are made in float32, the
    precision the kernel makes them in.

READINGS (the estimator formula is an image on the page):
  * the QJL constant is sqrt(pi/2)/m with m = d sketch rows, the value that
    makes the estimator unbiased for Gaussian rows, E[sign(g.e) g.q] =
    sqrt(2/pi) <e, q> / ||e||;
  * every token is compressed when appended; the FP16 ring additionally holds
    the last W tokens, and decode reads positions >= len - W from the ring;
  * a vector with nu < 1e-7 is stored as nu = 0, gamma = 0, all codes and bits 0
    ([Reconstruction] section 13 pseudocode zero-norm guard);
  * the softmax scale is 1/sqrt(d) unless given.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import codebook, layout
from .rotation import Transforms

QJL_CONST = np.sqrt(np.pi / 2.0)
ZERO_NORM = 1e-7


KEY_MODES = ("qjl", "scaled_unbiased", "scaled_mse")
VALUE_MODES = ("lloyd", "group")
GROUP = 32          # coordinates per scale/zero group of the group-quantized values


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
    key_mode: str = "qjl"
    value_mode: str = "lloyd"
    key_bits_hi: int = 0          # 0: key_bits on every coordinate
    value_bits_hi: int = 0        # 0: value_bits on every coordinate
    key_outliers: int = 0         # key sidecar entries per vector

    @property
    def qjl(self) -> bool:
        return self.key_mode == "qjl"

    @property
    def key_mse_bits(self) -> int:
        """Lloyd-Max bits of the lower coordinate half (the QJL bit excluded)."""
        return self.key_bits - 1 if self.qjl else self.key_bits

    @property
    def key_mse_bits_hi(self) -> int:
        b = self.key_bits_hi or self.key_bits
        return b - 1 if self.qjl else b

    @property
    def value_bits_hi_(self) -> int:
        return self.value_bits_hi or self.value_bits

    def key_bits_of(self, d: int):
        """Lloyd-Max bits per coordinate [d]."""
        return np.where(np.arange(d) >= d // 2, self.key_mse_bits_hi, self.key_mse_bits)

    def value_bits_of(self, d: int):
        return np.where(np.arange(d) >= d // 2, self.value_bits_hi_, self.value_bits)


class Params:
    """Codebooks and transforms of one configuration (the a0 init step).

    kc / kt and vc / vt are the codebooks of the lower coordinate half; kc_hi
    and friends those of the upper half (the same arrays for a uniform rate).
    """

    def __init__(self, cfg: Config):
        d = cfg.head_dim
        self.cfg = cfg
        self.kc = codebook.lloyd_max(d, cfg.key_mse_bits)
        self.kt = codebook.thresholds(self.kc)
        self.kc_hi = codebook.lloyd_max(d, cfg.key_mse_bits_hi)
        self.kt_hi = codebook.thresholds(self.kc_hi)
        self.vc = codebook.lloyd_max(d, cfg.value_bits)
        self.vt = codebook.thresholds(self.vc)
        self.vc_hi = codebook.lloyd_max(d, cfg.value_bits_hi_)
        self.vt_hi = codebook.thresholds(self.vc_hi)
        self.T = Transforms(d, cfg.rotation, cfg.seed)

    def key_thresholds_of(self, i, d):
        return self.kt_hi if i >= d // 2 else self.kt

    def value_thresholds_of(self, i, d):
        return self.vt_hi if i >= d // 2 else self.vt


def quantize(y, t):
    """idx = number of thresholds strictly below y (ties go to the lower cell)."""
    return np.searchsorted(t, y, side="left")


def _halves(y, lo, hi, fn):
    """fn(lower half, lo) | fn(upper half, hi) along the last axis."""
    d = y.shape[-1]
    return np.concatenate([fn(y[..., :d // 2], lo), fn(y[..., d // 2:], hi)], axis=-1)


def quantize_halves(y, t_lo, t_hi):
    return _halves(y, t_lo, t_hi, quantize)


def centroids_halves(codes, c_lo, c_hi):
    codes = np.asarray(codes, dtype=np.int64)
    return _halves(codes, c_lo, c_hi, lambda i, c: c[i])


def key_centroids(P: Params, codes):
    return centroids_halves(codes, P.kc, P.kc_hi)


def value_centroids(P: Params, codes):
    return centroids_halves(codes, P.vc, P.vc_hi)


def split_outliers(x, k):
    """The outlier sidecar: the k coordinates of largest |x| per row (ties to the
    lower index), their fp16 values, how many of them are nonzero, and x with
    those coordinates set to zero."""
    x = np.array(x, dtype=np.float64, copy=True)
    n, d = x.shape
    idx = np.zeros((n, max(k, 1)), np.int64)[:, :k]
    val = np.zeros((n, k), np.float16)
    if k == 0:
        return x, idx.astype(np.uint8), val, np.zeros(n, np.uint8)
    order = np.argsort(-np.abs(x), axis=-1, kind="stable")[:, :k]
    nz = np.abs(np.take_along_axis(x, order, axis=-1)) > 0
    count = nz.sum(axis=-1)
    # nonzero entries first, in magnitude order; unused slots hold index 0, value 0
    idx = np.where(nz, order, 0)
    val = np.where(nz, np.take_along_axis(x, order, axis=-1), 0.0).astype(np.float16)
    rows = np.arange(n)[:, None]
    x[rows, order] = np.where(nz, 0.0, x[rows, order])
    return x, idx.astype(np.uint8), val, count.astype(np.uint8)


def encode_keys(P: Params, x):
    """Keys [N, d] -> dict(codes, z, nu, gamma, side_idx, side_val, side_count, y, w, e).

    gamma is the residual norm in the QJL mode and the score scale s in the
    scaled modes (the second fp32 of each token's pair); y and w are kept for
    band accounting.
    """
    cfg = P.cfg
    x = np.asarray(x, dtype=np.float64)
    x, side_idx, side_val, side_count = split_outliers(x, cfg.key_outliers)
    nu = np.linalg.norm(x, axis=-1)
    zero = nu < ZERO_NORM
    u = x / np.where(zero, 1.0, nu)[:, None]
    y = P.T.rot_key(u)
    idx = quantize_halves(y, P.kt, P.kt_hi)
    yhat = key_centroids(P, idx)
    e = y - yhat
    if cfg.qjl:
        gamma = np.linalg.norm(e, axis=-1)
        w = P.T.sketch(e)
        z = w < 0
    else:
        ip = (y * yhat).sum(-1)
        if cfg.key_mode == "scaled_unbiased":
            gamma = nu / np.where(zero, 1.0, ip)
        else:
            gamma = nu * ip / np.where(zero, 1.0, (yhat * yhat).sum(-1))
        w = np.zeros_like(y)
        z = np.zeros(y.shape, bool)
    nu = np.where(zero, 0.0, nu)
    gamma = np.where(zero, 0.0, gamma)
    idx = np.where(zero[:, None], 0, idx)
    z = np.where(zero[:, None], False, z)
    return dict(codes=idx.astype(np.uint8), z=z, nu=nu, gamma=gamma, side_idx=side_idx, side_val=side_val,
                side_count=side_count, y=y, w=w, e=e)


def group_quantize(x, bits_of):
    """The group-quantized value codec in float32: per GROUP coordinates,
    scale = fp16((max - min) / (2^b - 1)), zero = fp16(min),
    code = clamp(rint((v - zero) / scale), 0, 2^b - 1)."""
    x32 = np.asarray(x, dtype=np.float32)
    n, d = x32.shape
    g = x32.reshape(n, d // GROUP, GROUP)
    levels = (np.left_shift(1, np.asarray(bits_of).reshape(d // GROUP, GROUP)[:, 0]) - 1).astype(np.float32)
    mn, mx = g.min(-1), g.max(-1)
    scale16 = ((mx - mn) / levels[None, :]).astype(np.float16)
    zero16 = mn.astype(np.float16)
    s32, z32 = scale16.astype(np.float32), zero16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - z32[..., None]) / s32[..., None]
    code = np.clip(np.rint(t), 0, levels[None, :, None])
    code = np.where(s32[..., None] > 0, code, 0).astype(np.uint8).reshape(n, d)
    return code, scale16, zero16


def encode_values(P: Params, x):
    cfg = P.cfg
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if cfg.value_mode == "group":
        code, scale16, zero16 = group_quantize(x, cfg.value_bits_of(d))
        return dict(codes=code, nu=np.zeros(len(x)), scale=scale16, zero=zero16, y=None)
    nu = np.linalg.norm(x, axis=-1)
    zero = nu < ZERO_NORM
    u = x / np.where(zero, 1.0, nu)[:, None]
    y = P.T.rot_value(u)
    idx = quantize_halves(y, P.vt, P.vt_hi)
    nu = np.where(zero, 0.0, nu)
    idx = np.where(zero[:, None], 0, idx)
    return dict(codes=idx.astype(np.uint8), nu=nu, y=y)


def sidecar_scores(q, side_idx, side_val, side_count):
    """sum_j q[idx_j] val_j over each token's nonzero sidecar entries: [G, N]."""
    q = np.asarray(q, dtype=np.float64)
    k = side_idx.shape[-1] if side_idx is not None and side_idx.ndim == 2 else 0
    if k == 0:
        return 0.0
    used = np.arange(k)[None, :] < np.asarray(side_count)[:, None]
    vals = np.where(used, np.asarray(side_val, np.float64), 0.0)
    return np.einsum("gnk,nk->gn", q[:, np.asarray(side_idx, np.int64)], vals)


def estimate_scores(P: Params, q, kcodes, kz, knu, kgamma, side_idx=None, side_val=None, side_count=None):
    """Compressed-domain score estimates est[h, t] for queries q [G, d] against N stored keys.

    QJL mode:    est = nu (<qt, yhat> + gamma sqrt(pi/2)/d <qh, 1 - 2z>)
    scaled modes: est = s <qt, yhat>          (kgamma holds s)
    plus the sidecar's exact part sum_j q[idx_j] val_j.
    """
    d = P.cfg.head_dim
    qt = P.T.rot_key(np.asarray(q, dtype=np.float64))
    mse = qt @ key_centroids(P, kcodes).T
    if P.cfg.qjl:
        qh = P.T.sketch(qt)
        qjl = qh @ (1.0 - 2.0 * kz.astype(np.float64)).T
        est = np.asarray(knu, np.float64)[None, :] * (
            mse + np.asarray(kgamma, np.float64)[None, :] * (QJL_CONST / d) * qjl)
    else:
        est = np.asarray(kgamma, np.float64)[None, :] * mse
    if P.cfg.key_outliers:
        est = est + sidecar_scores(q, side_idx, side_val, side_count)
    return est


def sidecar_vectors(side_idx, side_val, side_count, d):
    """The sidecar entries scattered into dense [N, d] vectors."""
    n, k = side_idx.shape
    out = np.zeros((n, d))
    for j in range(k):
        used = j < np.asarray(side_count)
        out[np.arange(n)[used], np.asarray(side_idx, np.int64)[used, j]] = np.asarray(side_val, np.float64)[used, j]
    return out


def dequantize_keys(P: Params, codes, z, nu, gamma, side_idx=None, side_val=None, side_count=None):
    """The key whose inner product with any q equals the score estimate:
    QJL mode k~ = nu T_K^T (yhat + gamma sqrt(pi/2)/d S^T (1 - 2z)), scaled
    modes k~ = s T_K^T yhat; plus the sidecar entries."""
    d = P.cfg.head_dim
    yhat = key_centroids(P, codes)
    if P.cfg.qjl:
        s = 1.0 - 2.0 * np.asarray(z, dtype=np.float64)
        yr = yhat + np.asarray(gamma, np.float64)[:, None] * (QJL_CONST / d) * P.T.sketch_t(s)
        k = np.asarray(nu, np.float64)[:, None] * P.T.unrot_key(yr)
    else:
        k = np.asarray(gamma, np.float64)[:, None] * P.T.unrot_key(yhat)
    if P.cfg.key_outliers:
        k = k + sidecar_vectors(side_idx, side_val, side_count, d)
    return k


def dequantize_values(P: Params, codes, nu, scale=None, zero=None):
    """Lloyd mode: v~ = nu T_V^T c[idx] ([Reconstruction] "Step 5": centroid
    lookup, inverse rotation, norm).  Group mode: v~ = zero + scale * code per
    group of GROUP coordinates."""
    if P.cfg.value_mode == "group":
        codes = np.asarray(codes, np.float64)
        n, d = codes.shape
        s = np.repeat(np.asarray(scale, np.float64), GROUP, axis=-1)
        z = np.repeat(np.asarray(zero, np.float64), GROUP, axis=-1)
        return z + s * codes
    return np.asarray(nu, np.float64)[:, None] * P.T.unrot_value(value_centroids(P, codes))


def exact_attention(q, K, V, scale):
    """softmax(scale q K^T) V in float64; q [G, d], K/V [N, d]."""
    q, K, V = (np.asarray(a, dtype=np.float64) for a in (q, K, V))
    s = scale * (q @ K.T)
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ V


class Cache:
    """Oracle model of the paged cache, kept unpacked (per page, per KV head, per slot).

    ``key_bytes`` / ``value_bytes`` / ``load_bytes`` convert to and from the
    byte layout of ``layout``, so pages written by another implementation can
    be decoded here.  k_gamma holds each key's second fp32 (the residual norm,
    or the score scale of the scaled key modes); the sidecar and the group
    scales exist in the modes that use them.
    """

    def __init__(self, cfg: Config, num_pages: int, block_table):
        P, d, H = cfg.page_tokens, cfg.head_dim, cfg.num_kv_heads
        self.cfg = cfg
        self.block_table = np.asarray(block_table, dtype=np.int64)
        max_seqs = self.block_table.shape[0]
        k = cfg.key_outliers
        self.k_codes = np.zeros((num_pages, H, P, d), np.uint8)
        self.k_z = np.zeros((num_pages, H, P, d), bool)
        self.k_nu = np.zeros((num_pages, H, P), np.float32)
        self.k_gamma = np.zeros((num_pages, H, P), np.float32)
        self.k_side_idx = np.zeros((num_pages, H, P, k), np.uint8)
        self.k_side_val = np.zeros((num_pages, H, P, k), np.float16)
        self.k_side_cnt = np.zeros((num_pages, H, P), np.uint8)
        self.v_codes = np.zeros((num_pages, H, P, d), np.uint8)
        self.v_nu = np.zeros((num_pages, H, P), np.float32)
        self.v_scale = np.zeros((num_pages, H, P, d // GROUP), np.float16)
        self.v_zero = np.zeros((num_pages, H, P, d // GROUP), np.float16)
        W = max(cfg.window, 1)
        self.k_window = np.zeros((max_seqs, H, W, d), np.float16)
        self.v_window = np.zeros((max_seqs, H, W, d), np.float16)

    # byte conversion -------------------------------------------------------
    def key_bytes(self):
        return layout.pack_key_block(self.cfg, self.k_codes, self.k_z, self.k_nu, self.k_gamma,
                                     self.k_side_idx, self.k_side_val, self.k_side_cnt)

    def value_bytes(self):
        return layout.pack_value_block(self.cfg, self.v_codes, self.v_nu, self.v_scale, self.v_zero)

    def load_bytes(self, k_pages, v_pages, k_window=None, v_window=None):
        c = self.cfg
        (self.k_codes, self.k_z, self.k_nu, self.k_gamma, self.k_side_idx, self.k_side_val,
         self.k_side_cnt) = layout.unpack_key_block(c, k_pages)
        self.k_codes = self.k_codes.astype(np.uint8)
        self.v_codes, self.v_nu, self.v_scale, self.v_zero = layout.unpack_value_block(c, v_pages)
        self.v_codes = self.v_codes.astype(np.uint8)
        if k_window is not None:
            self.k_window = np.asarray(k_window, np.float16)
            self.v_window = np.asarray(v_window, np.float16)

    # addressing ------------------------------------------------------------
    def locate(self, slot: int, positions):
        P = self.cfg.page_tokens
        positions = np.asarray(positions, dtype=np.int64)
        return self.block_table[slot, positions // P], positions % P

    def gather(self, slot: int, positions):
        """Stored fields for the given positions of one sequence: arrays [n, H, ...]."""
        pg, t = self.locate(slot, positions)
        return dict(k_codes=self.k_codes[pg, :, t], k_z=self.k_z[pg, :, t],
                    k_nu=self.k_nu[pg, :, t], k_gamma=self.k_gamma[pg, :, t],
                    k_side_idx=self.k_side_idx[pg, :, t], k_side_val=self.k_side_val[pg, :, t],
                    k_side_cnt=self.k_side_cnt[pg, :, t],
                    v_codes=self.v_codes[pg, :, t], v_nu=self.v_nu[pg, :, t],
                    v_scale=self.v_scale[pg, :, t], v_zero=self.v_zero[pg, :, t])


def key_fields(f, g):
    """estimate_scores / dequantize_keys keyword fields of kv head g from a gather()."""
    return dict(side_idx=f["k_side_idx"][:, g], side_val=f["k_side_val"][:, g], side_count=f["k_side_cnt"][:, g])


def append(P: Params, cache: Cache, k_new, v_new, seq_slots, ctx_len_before, cu_new_tokens):
    """Quantize-append new tokens of several sequences (a1-a5 for every token-head).

    k_new, v_new: [total_new, H_kv, d] (any float dtype; read as float64).
    Returns per-token encode records (for band accounting in the parity tests).
    """
    cfg = cache.cfg
    H, d, W = cfg.num_kv_heads, cfg.head_dim, cfg.window
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    total = k_new.shape[0]
    ek = encode_keys(P, k_new.reshape(total * H, d))
    ev = encode_values(P, v_new.reshape(total * H, d))
    rec = dict(k=ek, v=ev)
    k = cfg.key_outliers
    fields = dict(
        k_codes=ek["codes"].reshape(total, H, d), k_z=ek["z"].reshape(total, H, d),
        k_nu=ek["nu"].reshape(total, H).astype(np.float32), k_gamma=ek["gamma"].reshape(total, H).astype(np.float32),
        k_side_idx=ek["side_idx"].reshape(total, H, k), k_side_val=ek["side_val"].reshape(total, H, k),
        k_side_cnt=ek["side_count"].reshape(total, H),
        v_codes=ev["codes"].reshape(total, H, d), v_nu=ev["nu"].reshape(total, H).astype(np.float32))
    if cfg.value_mode == "group":
        fields.update(v_scale=ev["scale"].reshape(total, H, d // GROUP), v_zero=ev["zero"].reshape(total, H, d // GROUP))
    for s in range(len(seq_slots)):
        slot = int(seq_slots[s])
        a, b = int(cu_new_tokens[s]), int(cu_new_tokens[s + 1])
        n = b - a
        if n <= 0:
            continue
        start = int(ctx_len_before[s])
        pos = np.arange(start, start + n)
        pg, t = cache.locate(slot, pos)
        for name, arr in fields.items():
            getattr(cache, name)[pg, :, t] = arr[a:b]
        if W > 0:
            new_len = start + n
            keep = pos >= new_len - W
            ring = pos[keep] % W
            cache.k_window[slot][:, ring] = np.swapaxes(k_new[a:b][keep], 0, 1).astype(np.float16)
            cache.v_window[slot][:, ring] = np.swapaxes(v_new[a:b][keep], 0, 1).astype(np.float16)
    return rec


def compressed_count(cfg: Config, length: int) -> int:
    return length if cfg.window == 0 else max(0, length - cfg.window)


def decode(P: Params, cache: Cache, q, seq_slots, ctx_len, scale=None, return_logits=False):
    """Decode attention for one query per sequence over the compressed cache.

    q: [num_seqs, H_q, d].  Returns out [num_seqs, H_q, d] float64 (and, when
    asked, a list of per-sequence logits [H_q, len]).
    """
    cfg = cache.cfg
    d, H, Hq, W = cfg.head_dim, cfg.num_kv_heads, cfg.num_q_heads, cfg.window
    G = Hq // H
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros((q.shape[0], Hq, d))
    all_logits = []
    for s in range(q.shape[0]):
        slot, L = int(seq_slots[s]), int(ctx_len[s])
        nc = compressed_count(cfg, L)
        f = cache.gather(slot, np.arange(nc))
        wpos = np.arange(nc, L)
        logits_s = np.zeros((Hq, L))
        for g in range(H):
            qg = q[s, g * G:(g + 1) * G]
            est = estimate_scores(P, qg, f["k_codes"][:, g], f["k_z"][:, g], f["k_nu"][:, g], f["k_gamma"][:, g],
                                  **key_fields(f, g))
            kw = cache.k_window[slot, g, wpos % W].astype(np.float64) if W else np.zeros((0, d))
            vw = cache.v_window[slot, g, wpos % W].astype(np.float64) if W else np.zeros((0, d))
            lg = scale * np.concatenate([est, qg @ kw.T], axis=1)
            logits_s[g * G:(g + 1) * G] = lg
            if L == 0:
                continue
            m = lg.max(axis=1, keepdims=True)
            p = np.exp(lg - m)
            l = p.sum(axis=1, keepdims=True)
            acc_win = p[:, nc:] @ vw
            if cfg.value_mode == "group":
                vt = dequantize_values(P, f["v_codes"][:, g], None, f["v_scale"][:, g], f["v_zero"][:, g])
                out[s, g * G:(g + 1) * G] = (p[:, :nc] @ vt + acc_win) / l
            else:
                vrot = f["v_nu"][:, g].astype(np.float64)[:, None] * value_centroids(P, f["v_codes"][:, g])
                acc_rot = p[:, :nc] @ vrot
                out[s, g * G:(g + 1) * G] = (P.T.unrot_value(acc_rot) + acc_win) / l
        all_logits.append(logits_s)
    return (out, all_logits) if return_logits else out


def dequantize(P: Params, cache: Cache, slot: int, tok_begin: int, tok_end: int):
    """Reconstructed keys and values [n, H_kv, d] for page-resident positions [tok_begin, tok_end)."""
    cfg = cache.cfg
    H, d = cfg.num_kv_heads, cfg.head_dim
    pos = np.arange(tok_begin, tok_end)
    f = cache.gather(slot, pos)
    n = len(pos)
    kk = cfg.key_outliers
    k = dequantize_keys(P, f["k_codes"].reshape(n * H, d), f["k_z"].reshape(n * H, d),
                        f["k_nu"].reshape(-1), f["k_gamma"].reshape(-1), f["k_side_idx"].reshape(n * H, kk),
                        f["k_side_val"].reshape(n * H, kk), f["k_side_cnt"].reshape(-1)).reshape(n, H, d)
    v = dequantize_values(P, f["v_codes"].reshape(n * H, d), f["v_nu"].reshape(-1),
                          f["v_scale"].reshape(n * H, d // GROUP), f["v_zero"].reshape(n * H, d // GROUP)).reshape(n, H, d)
    return k, v


def attention_over_dequantized(P: Params, cache: Cache, q, seq_slots, ctx_len, scale=None):
    """Exact softmax attention over dequantize() output plus the FP16 window (decode-algebra check)."""
    cfg = cache.cfg
    d, H, Hq, W = cfg.head_dim, cfg.num_kv_heads, cfg.num_q_heads, cfg.window
    G = Hq // H
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros((q.shape[0], Hq, d))
    for s in range(q.shape[0]):
        slot, L = int(seq_slots[s]), int(ctx_len[s])
        if L == 0:
            continue
        nc = compressed_count(cfg, L)
        k, v = dequantize(P, cache, slot, 0, nc)
        wpos = np.arange(nc, L)
        for g in range(H):
            kk = np.concatenate([k[:, g], cache.k_window[slot, g, wpos % max(W, 1)].astype(np.float64)]) if W else k[:, g]
            vv = np.concatenate([v[:, g], cache.v_window[slot, g, wpos % max(W, 1)].astype(np.float64)]) if W else v[:, g]
            out[s, g * G:(g + 1) * G] = exact_attention(q[s, g * G:(g + 1) * G], kk, vv, scale)
    return out
