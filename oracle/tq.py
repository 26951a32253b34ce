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

    @property
    def key_mse_bits(self) -> int:
        return self.key_bits - 1


class Params:
    """Codebooks and transforms of one configuration (the a0 init step)."""

    def __init__(self, cfg: Config):
        d = cfg.head_dim
        self.cfg = cfg
        self.kc = codebook.lloyd_max(d, cfg.key_mse_bits)
        self.kt = codebook.thresholds(self.kc)
        self.vc = codebook.lloyd_max(d, cfg.value_bits)
        self.vt = codebook.thresholds(self.vc)
        self.T = Transforms(d, cfg.rotation, cfg.seed)


def quantize(y, t):
    """idx = number of thresholds strictly below y (ties go to the lower cell)."""
    return np.searchsorted(t, y, side="left")


def encode_keys(P: Params, x):
    """Keys [N, d] -> dict(codes, z, nu, gamma, y, w); y and w are kept for band accounting."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    nu = np.linalg.norm(x, axis=-1)
    zero = nu < ZERO_NORM
    u = x / np.where(zero, 1.0, nu)[:, None]
    y = P.T.rot_key(u)
    idx = quantize(y, P.kt)
    e = y - P.kc[idx]
    gamma = np.linalg.norm(e, axis=-1)
    w = P.T.sketch(e)
    z = w < 0
    nu = np.where(zero, 0.0, nu)
    gamma = np.where(zero, 0.0, gamma)
    idx = np.where(zero[:, None], 0, idx)
    z = np.where(zero[:, None], False, z)
    return dict(codes=idx.astype(np.uint8), z=z, nu=nu, gamma=gamma, y=y, w=w, e=e)


def encode_values(P: Params, x):
    x = np.asarray(x, dtype=np.float64)
    nu = np.linalg.norm(x, axis=-1)
    zero = nu < ZERO_NORM
    u = x / np.where(zero, 1.0, nu)[:, None]
    y = P.T.rot_value(u)
    idx = quantize(y, P.vt)
    nu = np.where(zero, 0.0, nu)
    idx = np.where(zero[:, None], 0, idx)
    return dict(codes=idx.astype(np.uint8), nu=nu, y=y)


def estimate_scores(P: Params, q, kcodes, kz, knu, kgamma):
    """Compressed-domain score estimates est[h, t] for queries q [G, d] against N stored keys."""
    d = P.cfg.head_dim
    qt = P.T.rot_key(np.asarray(q, dtype=np.float64))
    qh = P.T.sketch(qt)
    mse = qt @ P.kc[kcodes].T
    qjl = qh @ (1.0 - 2.0 * kz.astype(np.float64)).T
    return np.asarray(knu, np.float64)[None, :] * (
        mse + np.asarray(kgamma, np.float64)[None, :] * (QJL_CONST / d) * qjl)


def dequantize_keys(P: Params, codes, z, nu, gamma):
    """k~ = nu T_K^T (c[idx] + gamma sqrt(pi/2)/d S^T (1 - 2z)), so <q, k~> equals the score estimate."""
    d = P.cfg.head_dim
    s = 1.0 - 2.0 * np.asarray(z, dtype=np.float64)
    yr = P.kc[codes] + np.asarray(gamma, np.float64)[:, None] * (QJL_CONST / d) * P.T.sketch_t(s)
    return np.asarray(nu, np.float64)[:, None] * P.T.unrot_key(yr)


def dequantize_values(P: Params, codes, nu):
    """v~ = nu T_V^T c[idx] ([Reconstruction] "Step 5": centroid lookup, inverse rotation, norm)."""
    return np.asarray(nu, np.float64)[:, None] * P.T.unrot_value(P.vc[codes])


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
    be decoded here.
    """

    def __init__(self, cfg: Config, num_pages: int, block_table):
        P, d, H = cfg.page_tokens, cfg.head_dim, cfg.num_kv_heads
        self.cfg = cfg
        self.block_table = np.asarray(block_table, dtype=np.int64)
        max_seqs = self.block_table.shape[0]
        self.k_codes = np.zeros((num_pages, H, P, d), np.uint8)
        self.k_z = np.zeros((num_pages, H, P, d), bool)
        self.k_nu = np.zeros((num_pages, H, P), np.float32)
        self.k_gamma = np.zeros((num_pages, H, P), np.float32)
        self.v_codes = np.zeros((num_pages, H, P, d), np.uint8)
        self.v_nu = np.zeros((num_pages, H, P), np.float32)
        W = max(cfg.window, 1)
        self.k_window = np.zeros((max_seqs, H, W, d), np.float16)
        self.v_window = np.zeros((max_seqs, H, W, d), np.float16)

    # byte conversion -------------------------------------------------------
    def key_bytes(self):
        return layout.pack_key_block(self.k_codes, self.k_z, self.k_nu, self.k_gamma, self.cfg.key_mse_bits)

    def value_bytes(self):
        return layout.pack_value_block(self.v_codes, self.v_nu, self.cfg.value_bits)

    def load_bytes(self, k_pages, v_pages, k_window=None, v_window=None):
        c = self.cfg
        self.k_codes, self.k_z, self.k_nu, self.k_gamma = layout.unpack_key_block(
            k_pages, c.head_dim, c.key_mse_bits, c.page_tokens)
        self.k_codes = self.k_codes.astype(np.uint8)
        self.v_codes, self.v_nu = layout.unpack_value_block(v_pages, c.head_dim, c.value_bits, c.page_tokens)
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
                    v_codes=self.v_codes[pg, :, t], v_nu=self.v_nu[pg, :, t])


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
    codes_k = ek["codes"].reshape(total, H, d)
    z_k = ek["z"].reshape(total, H, d)
    nu_k = ek["nu"].reshape(total, H).astype(np.float32)
    g_k = ek["gamma"].reshape(total, H).astype(np.float32)
    codes_v = ev["codes"].reshape(total, H, d)
    nu_v = ev["nu"].reshape(total, H).astype(np.float32)
    for s in range(len(seq_slots)):
        slot = int(seq_slots[s])
        a, b = int(cu_new_tokens[s]), int(cu_new_tokens[s + 1])
        n = b - a
        if n <= 0:
            continue
        start = int(ctx_len_before[s])
        pos = np.arange(start, start + n)
        pg, t = cache.locate(slot, pos)
        cache.k_codes[pg, :, t] = codes_k[a:b]
        cache.k_z[pg, :, t] = z_k[a:b]
        cache.k_nu[pg, :, t] = nu_k[a:b]
        cache.k_gamma[pg, :, t] = g_k[a:b]
        cache.v_codes[pg, :, t] = codes_v[a:b]
        cache.v_nu[pg, :, t] = nu_v[a:b]
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
            est = estimate_scores(P, qg, f["k_codes"][:, g], f["k_z"][:, g], f["k_nu"][:, g], f["k_gamma"][:, g])
            kw = cache.k_window[slot, g, wpos % W].astype(np.float64) if W else np.zeros((0, d))
            vw = cache.v_window[slot, g, wpos % W].astype(np.float64) if W else np.zeros((0, d))
            lg = scale * np.concatenate([est, qg @ kw.T], axis=1)
            logits_s[g * G:(g + 1) * G] = lg
            if L == 0:
                continue
            m = lg.max(axis=1, keepdims=True)
            p = np.exp(lg - m)
            l = p.sum(axis=1, keepdims=True)
            vrot = f["v_nu"][:, g].astype(np.float64)[:, None] * P.vc[f["v_codes"][:, g]]
            acc_rot = p[:, :nc] @ vrot
            acc_win = p[:, nc:] @ vw
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
    k = dequantize_keys(P, f["k_codes"].reshape(n * H, d), f["k_z"].reshape(n * H, d),
                        f["k_nu"].reshape(-1), f["k_gamma"].reshape(-1)).reshape(n, H, d)
    v = dequantize_values(P, f["v_codes"].reshape(n * H, d), f["v_nu"].reshape(-1)).reshape(n, H, d)
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
