"""Pins for the oracle's append / decode / dequantize (the method itself).

Checks: QJL unbiasedness (Theorem 2 as validated in [README]), the MSE
shrinkage bias ([Reconstruction] section 6), decode == exact attention over the
dequantized cache, reductions to plain attention, needle retrieval, rank
metrics against the README's thresholds, and brute force on the tiny workload.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import codebook, tq
from oracle.rotation import Transforms
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")
README = json.load(open(os.path.join(GOLD, "readme_validation.json")))


def _params(d=128, kb=3, vb=2, rot="fwht", W=0, hq=4, hkv=1, seed=42):
    cfg = tq.Config(head_dim=d, num_q_heads=hq, num_kv_heads=hkv, key_bits=kb, value_bits=vb,
                    page_tokens=16, window=W, rotation=rot, seed=seed)
    return cfg, tq.Params(cfg)


def _relative_bias(P, d, rot, seeds, per_seed, rng_seed=0):
    g = np.random.default_rng(rng_seed)
    num = den = 0.0
    for s in seeds:
        P.T = Transforms(d, rot, int(s))
        k = g.standard_normal((per_seed, d))
        e = tq.encode_keys(P, k)
        est = tq.estimate_scores(P, k, e["codes"], e["z"], e["nu"], e["gamma"])
        num += np.diag(est).sum() - (k * k).sum()
        den += (k * k).sum()
    return num / den


@pytest.mark.parametrize("kb", [3, 4])
def test_qjl_estimator_unbiased_fwht(kb):
    # [README] "Paper Validation": relative bias < 0.1 % (Theorem 2), q = k.
    d = 128
    cfg, P = _params(d, kb)
    bias = _relative_bias(P, d, "fwht", range(1500), 64)
    assert abs(bias) < README["thm2_relative_bias_max"]


def test_qjl_estimator_unbiased_dense():
    d = 64
    cfg, P = _params(d, 3, rot="dense")
    bias = _relative_bias(P, d, "dense", range(400), 256)
    assert abs(bias) < README["thm2_relative_bias_max"]


def test_mse_only_estimate_shrinks_by_one_minus_distortion():
    # [Reconstruction] section 6: <q, yhat> underestimates <q, y> because the
    # Lloyd-Max reconstruction shrinks the norm; on average by 1 - D_b/... per
    # unit vector: E <y, yhat> = 1 - D_b(d) / 1 (centroid condition).
    d = 128
    cfg, P = _params(d, 3)
    k = np.random.default_rng(5).standard_normal((20000, d))
    e = tq.encode_keys(P, k)
    yhat = P.kc[e["codes"]]
    ratio = (e["y"] * yhat).sum(1).mean()
    assert abs(ratio - (1 - codebook.distortion(P.kc, d))) < 2e-3


def _build_cache(cfg, P, lens, rng_seed=0, dtype=np.float32, shuffle=True, chunks=1):
    g = np.random.default_rng(rng_seed)
    H, d, Pt = cfg.num_kv_heads, cfg.head_dim, cfg.page_tokens
    nseq = len(lens)
    mpp = max(1, -(-max(lens) // Pt))
    perm = g.permutation(nseq * mpp) if shuffle else np.arange(nseq * mpp)
    cache = tq.Cache(cfg, nseq * mpp, perm.reshape(nseq, mpp))
    K = [g.standard_normal((n, H, d)).astype(dtype) for n in lens]
    V = [g.standard_normal((n, H, d)).astype(dtype) for n in lens]
    # append in `chunks` calls to exercise partially filled pages
    done = [0] * nseq
    for c in range(chunks):
        ks, vs, cu, before = [], [], [0], []
        for s, n in enumerate(lens):
            hi = n if c == chunks - 1 else (n * (c + 1)) // chunks
            ks.append(K[s][done[s]:hi]); vs.append(V[s][done[s]:hi])
            before.append(done[s]); cu.append(cu[-1] + hi - done[s]); done[s] = hi
        tq.append(P, cache, np.concatenate(ks), np.concatenate(vs), np.arange(nseq), before, cu)
    return cache, K, V


@pytest.mark.parametrize("rot,W,chunks", [("fwht", 0, 1), ("fwht", 32, 3), ("dense", 16, 2)])
def test_decode_equals_attention_over_dequantized(rot, W, chunks):
    cfg, P = _params(64, 3, 2, rot=rot, W=W, hq=8, hkv=2)
    lens = [0, 1, 17, 100]
    cache, K, V = _build_cache(cfg, P, lens, chunks=chunks)
    q = np.random.default_rng(9).standard_normal((len(lens), 8, 64))
    out = tq.decode(P, cache, q, np.arange(len(lens)), lens)
    ref = tq.attention_over_dequantized(P, cache, q, np.arange(len(lens)), lens)
    assert np.abs(out[1:] - ref[1:]).max() < 1e-12
    assert np.all(out[0] == 0)                     # empty context -> zero output


def test_window_covering_context_is_plain_fp16_attention():
    cfg, P = _params(64, 3, 2, W=128, hq=4, hkv=1)
    lens = [100]
    cache, K, V = _build_cache(cfg, P, lens)
    q = np.random.default_rng(2).standard_normal((1, 4, 64))
    out = tq.decode(P, cache, q, [0], lens)
    k16 = torch.tensor(K[0][:, 0].astype(np.float16).astype(np.float64))
    v16 = torch.tensor(V[0][:, 0].astype(np.float16).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q[0])[None], k16[None], v16[None]).numpy()[0]
    assert np.abs(out[0] - ref).max() < 1e-12


def test_single_token_and_identical_keys():
    cfg, P = _params(128, 4, 4, hq=2, hkv=1)
    cache, K, V = _build_cache(cfg, P, [1])
    q = np.random.default_rng(3).standard_normal((1, 2, 128))
    out = tq.decode(P, cache, q, [0], [1])
    k, v = tq.dequantize(P, cache, 0, 0, 1)
    assert np.allclose(out[0], v[0, 0][None], atol=1e-13)
    # identical keys: uniform attention -> mean of reconstructed values
    g = np.random.default_rng(4)
    kk = np.repeat(g.standard_normal((1, 1, 128)), 40, axis=0)
    vv = g.standard_normal((40, 1, 128))
    cache2 = tq.Cache(cfg, 3, np.array([[2, 0, 1]]))
    tq.append(P, cache2, kk, vv, [0], [0], [0, 40])
    out2 = tq.decode(P, cache2, q, [0], [40])
    _, v2 = tq.dequantize(P, cache2, 0, 0, 40)
    assert np.allclose(out2[0], v2[:, 0].mean(0)[None], atol=1e-12)


def test_zero_vector_is_stored_as_zero():
    cfg, P = _params(128, 3, 2, hq=1, hkv=1)
    x = np.zeros((2, 128)); x[1, 0] = 1.0
    e = tq.encode_keys(P, x)
    assert e["nu"][0] == 0 and e["gamma"][0] == 0 and not e["z"][0].any() and not e["codes"][0].any()
    assert np.isfinite(e["y"]).all()
    k = tq.dequantize_keys(P, e["codes"], e["z"], e["nu"], e["gamma"])
    assert np.all(k[0] == 0)


def test_needle_and_rank_metrics():
    # [README] "Paper Validation": needle retrieval passes; Recall@8 >= 0.40 at
    # N = 4096 (3-bit); Spearman rho > 0.85 at N = 2048.
    d = 128
    cfg, P = _params(d, 3)
    g = np.random.default_rng(6)
    keys = g.standard_normal((4096, d))
    e = tq.encode_keys(P, keys)
    for j in (0, 1234, 4095):
        est = tq.estimate_scores(P, 8.0 * keys[j][None], e["codes"], e["z"], e["nu"], e["gamma"])[0]
        assert np.argmax(est) == j
    qs = g.standard_normal((16, d))
    est = tq.estimate_scores(P, qs, e["codes"], e["z"], e["nu"], e["gamma"])
    true = qs @ keys.T
    rec = np.mean([len(set(np.argsort(-true[i])[:8]) & set(np.argsort(-est[i])[:8])) / 8 for i in range(16)])
    assert rec >= README["recall_at_8_threshold"]
    from scipy.stats import spearmanr
    rho = np.mean([spearmanr(true[i, :2048], est[i, :2048]).statistic for i in range(16)])
    assert rho > README["spearman_rho_min_N2048"]


def test_tiny_reference_workload_against_exact_attention():
    # Brute force on the tiny workload: compressed decode vs exact attention on
    # the raw fp32 keys/values (quality, not parity).
    w = workloads.TINY_REF
    cfg = tq.Config(w.head_dim, w.num_q_heads, w.num_kv_heads, w.key_bits, w.value_bits,
                    w.page_tokens, w.window, w.rotation, w.method_seed)
    P = tq.Params(cfg)
    K = workloads.kv_tokens(w, "k", 0, 0, w.decode_ctx).numpy()
    V = workloads.kv_tokens(w, "v", 0, 0, w.decode_ctx).numpy()
    q = workloads.queries(w, 0).numpy()
    cache = tq.Cache(cfg, w.pages_per_seq(), np.arange(w.pages_per_seq())[None])
    tq.append(P, cache, K, V, [0], [0], [0, w.decode_ctx])
    out, logits = tq.decode(P, cache, q[None], [0], [w.decode_ctx], return_logits=True)
    ref = tq.exact_attention(q, K[:, 0], V[:, 0], 1 / np.sqrt(128))
    cos = (out[0] * ref).sum() / np.linalg.norm(out[0]) / np.linalg.norm(ref)
    assert cos > 0.8
    ltrue = (q @ K[:, 0].T) / np.sqrt(128)
    pt = np.exp(ltrue - ltrue.max()); pt /= pt.sum()
    pe = np.exp(logits[0] - logits[0].max()); pe /= pe.sum()
    kl = float((pt * np.log(pt / pe)).sum())
    assert kl < 0.1


def test_encode_matches_plain_definitions():
    # Code assignment is nearest-centroid and the QJL bit is the sign of S e.
    cfg, P = _params(128, 4, 2)
    x = np.random.default_rng(8).standard_normal((50, 128))
    e = tq.encode_keys(P, x)
    y = P.T.key_matrix() @ (x / np.linalg.norm(x, axis=1, keepdims=True)).T
    assert np.allclose(e["y"], y.T, atol=1e-13)
    nearest = np.argmin(np.abs(e["y"][..., None] - P.kc), axis=-1)
    assert np.array_equal(e["codes"], nearest)
    w = (P.T.sketch_matrix() @ (e["y"] - P.kc[nearest]).T).T
    assert np.array_equal(e["z"], w < 0)


@pytest.mark.parametrize("d,kb,vb,rot", [(128, 3, 4, "fwht"), (256, 3, 4, "dense"), (128, 4, 2, "dense"),
                                         (256, 4, 2, "fwht"), (128, 2, 3, "fwht")])
def test_value_codec_distortion_and_cosine_closed_forms(d, kb, vb, rot):
    """encode_values / dequantize_values at the configured value bits.

    For a uniformly rotated unit vector every coordinate follows f_d, so the
    per-vector squared error of the Lloyd-Max codec is D_b(d) / d per
    coordinate on average (Thm 1 in expectation: E||u - u~||^2 = D_b), and the
    centroid condition gives E cos(v, v~) = sqrt(1 - D_b) to first order
    (0.9402 at 2 bits and head_dim 256, the [README] "TQ Quantization
    Quality" value).  The key codebook here has a different bit count, so a
    key/value codebook swap or a wrong bit count fails.
    """
    cfg, P = _params(d, kb, vb, rot)
    g = np.random.default_rng(100 + d + vb)
    n = 6000
    x = g.standard_normal((n, d)) * g.uniform(0.5, 3.0, (n, 1))
    ev = tq.encode_values(P, x)
    assert ev["codes"].max() == (1 << vb) - 1 and ev["codes"].min() == 0
    assert np.allclose(ev["nu"], np.linalg.norm(x, axis=1), rtol=1e-15)
    vt = tq.dequantize_values(P, ev["codes"], ev["nu"])
    D = codebook.distortion(codebook.lloyd_max(d, vb), d)
    Dk = codebook.distortion(codebook.lloyd_max(d, kb - 1), d)
    err = ((x - vt) ** 2).sum(1) / ev["nu"] ** 2
    se = err.std() / np.sqrt(n)
    assert abs(err.mean() - D) < 5 * se, (err.mean(), D)
    assert abs(err.mean() - Dk) > 20 * se          # distinguishable from the key codebook
    cos = (x * vt).sum(1) / np.linalg.norm(x, axis=1) / np.linalg.norm(vt, axis=1)
    # first order in D (Jensen's gap is O(Var D)): allow 2% of D on top of the sampling error
    assert abs(cos.mean() - np.sqrt(1 - D)) < 5 * cos.std() / np.sqrt(n) + 0.02 * D
    if d == 256 and vb == 2:
        assert abs(cos.mean() - README["value_cos_2bit_head_dim256"]) < 2e-3
