"""GPU parity at the full benchmark sizes, in the launch configuration bench.py
times.

The caches are filled by bench.py's own setup functions (same appends, same
decode split plan); the seeded device generator is then replayed to recover
the inputs at sampled positions.  The oracle cannot redo these sizes whole, so
it checks what it can compute piece by piece:

  * append: sampled token-heads (first and last positions, page edges, the
    window boundary, random positions) re-encoded by the oracle from their
    inputs: codes and QJL bits bit-exact up to the threshold band, norms at
    NORM_RTOL;
  * decode: for one kv head of one sequence, the oracle decodes the GPU's own
    bytes of every token of that head (a cache holding that head alone) and
    the GPU's output for the head's query group must agree within DECODE_TOL;
    the logits the kernel dumps are checked at sampled positions of every
    query head against the oracle's estimate from the same bytes;
  * on the outlier workload, that head's output cosine, and the Spearman rank
    correlation and Recall@8 of its logits, against the oracle (agreement) and
    against exact attention over the raw keys and values (quality).

Workloads: outlier stress (4 x 131072, d = 128, 4/4-bit, FWHT), head_dim 256
(8 x 32768, dense rotation, 3/2- and 4/4-bit) and the mixed serving step
(64 x 4096 appended, 256 x 4096 decoded).
"""
import numpy as np
import pytest
import torch

import bench
import workloads
from harness import BAND, DECODE_TOL, NORM_RTOL, decode_error, key_aux, near_threshold, oracle_config
from oracle import tq

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _ocfg(w, num_q_heads=None, num_kv_heads=None):
    return oracle_config(w, num_q_heads=num_q_heads or w.num_q_heads, num_kv_heads=num_kv_heads or w.num_kv_heads)


def _sample_positions(w, L, rng, extra=24):
    P, W = w.page_tokens, w.window
    pos = {0, 1, P - 1, P, L - 1, L - 2}
    if W:
        pos |= {max(0, L - W - 1), max(0, L - W), L - W + 1}
    pos |= set(int(x) for x in rng.integers(0, L, extra))
    return np.array(sorted(p for p in pos if 0 <= p < L), dtype=np.int64)


def _gpu_blocks(cache, bt_row, positions, page):
    """Key and value blocks of the pages holding `positions`, as an oracle cache
    over just those pages (block table remapped)."""
    pages = np.unique(bt_row[positions // page])
    kb = cache.k_pages[torch.from_numpy(pages).to(DEV)].cpu().numpy()
    vb = cache.v_pages[torch.from_numpy(pages).to(DEV)].cpu().numpy()
    return pages, kb, vb


def _check_append(w, P, cache, bt, samples, inputs):
    """samples: {slot: positions}; inputs: {slot: (k rows, v rows)} float64 [n, H, d]."""
    d, H = w.head_dim, w.num_kv_heads
    cfg = _ocfg(w)
    flips = 0
    for slot, pos in samples.items():
        pages, kb, vb = _gpu_blocks(cache, bt[slot], pos, w.page_tokens)
        remap = {int(p): i for i, p in enumerate(pages)}
        c = tq.Cache(cfg, len(pages), np.zeros((1, 1), np.int64))
        c.load_bytes(kb, vb)
        pg = np.array([remap[int(p)] for p in bt[slot][pos // w.page_tokens]])
        t = pos % w.page_tokens
        kx, vx = inputs[slot]
        ek = tq.encode_keys(P, kx.reshape(-1, d))
        ev = tq.encode_values(P, vx.reshape(-1, d))
        gk = c.k_codes[pg, :, t].reshape(-1, d).astype(np.int64)
        gz = c.k_z[pg, :, t].reshape(-1, d)
        mism = gk != ek["codes"]
        near = near_threshold(ek["y"], P.kt, P.kt_hi)
        assert not (mism & ~near).any(), f"slot {slot}: key codes differ away from a threshold"
        flips += int(mism.sum())
        oaux, wv = key_aux(P, ek["y"], gk, ek["nu"])
        if cfg.qjl:
            zexp = wv < 0
            zexp[ek["nu"] == 0] = False
            zm = gz != zexp
            assert not (zm & ~(np.abs(wv) / np.sqrt(d) < BAND)).any(), f"slot {slot}: QJL bits differ"
        if cfg.key_outliers:
            assert np.array_equal(c.k_side_cnt[pg, :, t].reshape(-1), ek["side_count"])
            used = np.arange(cfg.key_outliers)[None, :] < ek["side_count"][:, None]
            gi = c.k_side_idx[pg, :, t].reshape(-1, cfg.key_outliers)
            gsv = c.k_side_val[pg, :, t].reshape(-1, cfg.key_outliers).view(np.uint16)
            assert not ((gi != ek["side_idx"]) & used).any() and not ((gsv != ek["side_val"].view(np.uint16)) & used).any()
        gnu = c.k_nu[pg, :, t].reshape(-1).astype(np.float64)
        gaux = c.k_gamma[pg, :, t].reshape(-1).astype(np.float64)
        assert np.all(np.abs(gnu - ek["nu"]) <= NORM_RTOL * np.maximum(ek["nu"], 1e-30))
        assert np.all(np.abs(gaux - oaux) <= NORM_RTOL * np.maximum(np.abs(oaux), 1e-30))
        gv = c.v_codes[pg, :, t].reshape(-1, d).astype(np.int64)
        if cfg.value_mode == "group":
            assert np.array_equal(gv, ev["codes"]), f"slot {slot}: group value codes differ"
            assert np.array_equal(c.v_scale[pg, :, t].reshape(ev["scale"].shape).view(np.uint16),
                                  ev["scale"].view(np.uint16))
            assert np.array_equal(c.v_zero[pg, :, t].reshape(ev["zero"].shape).view(np.uint16),
                                  ev["zero"].view(np.uint16))
        else:
            vm = gv != ev["codes"]
            assert not (vm & ~near_threshold(ev["y"], P.vt, P.vt_hi)).any(), f"slot {slot}: value codes differ"
            flips += int(vm.sum())
            gvn = c.v_nu[pg, :, t].reshape(-1).astype(np.float64)
            assert np.all(np.abs(gvn - ev["nu"]) <= NORM_RTOL * np.maximum(ev["nu"], 1e-30))
    return flips


def _check_decode_head(w, cache, bt, slot, hk, L, q, out_gpu):
    """Oracle decode of one kv head of one sequence over the GPU's bytes of that
    head, against the GPU output of the head's query group.  Returns the error,
    the oracle's output rows [G, d] and its logits [G, L]."""
    G, d, W = w.gqa, w.head_dim, w.window
    cfg1 = _ocfg(w, num_q_heads=G, num_kv_heads=1)
    P1 = tq.Params(cfg1)
    npg = -(-L // w.page_tokens)
    pages = torch.from_numpy(bt[slot][:npg].astype(np.int64)).to(DEV)
    kb = cache.k_pages[pages, hk:hk + 1].cpu().numpy()
    vb = cache.v_pages[pages, hk:hk + 1].cpu().numpy()
    c = tq.Cache(cfg1, npg, np.arange(npg, dtype=np.int64)[None])
    kwin = vwin = None
    if W:
        kwin = cache.k_window[slot, hk:hk + 1].cpu().numpy().view(np.float16)[None]
        vwin = cache.v_window[slot, hk:hk + 1].cpu().numpy().view(np.float16)[None]
    c.load_bytes(kb, vb, kwin, vwin)
    qg = q[slot, hk * G:(hk + 1) * G].double().cpu().numpy()[None]
    ref, lg = tq.decode(P1, c, qg, [0], [L], return_logits=True)
    return decode_error(out_gpu[slot, hk * G:(hk + 1) * G][None], ref), ref[0], lg[0]


def _rank_metrics(a, b, k=8):
    """Per row: cosine of two outputs is computed elsewhere; here Spearman rho of
    two logit rows and the overlap of their top-k positions (Recall@k)."""
    from scipy.stats import spearmanr
    rho = [spearmanr(x, y).correlation for x, y in zip(a, b)]
    rec = [len(set(np.argsort(-x)[:k]) & set(np.argsort(-y)[:k])) / k for x, y in zip(a, b)]
    return float(np.mean(rho)), float(np.min(rho)), float(np.mean(rec)), float(np.min(rec))


def _cos(a, b):
    return (a * b).sum(-1) / np.linalg.norm(a, axis=-1) / np.linalg.norm(b, axis=-1)


def _decode(S, cache, logits=None):
    import kv_cache_vector_append_amd as tqa
    tqa.decode_attention(S.cfg, S.params, cache, S.q, S.dec_slots, S.dec_lens, S.max_ctx, S.out, S.ws,
                         0.0, logits)
    torch.cuda.synchronize()
    return S.out.cpu().double().numpy()


def _logit_samples(w, S, cache, bt, slot, rng):
    """Dumped logits at sampled positions of every query head of `slot`, against
    the oracle's estimate from the same bytes (window positions: q . k / sqrt(d))."""
    L, d, H, G = S.lens[slot], w.head_dim, w.num_kv_heads, w.gqa
    logits = torch.full((len(S.lens), w.num_q_heads, S.max_ctx), float("nan"), device=DEV)
    _decode(S, cache, logits)
    lg = logits[slot].cpu().double().numpy()
    pos = _sample_positions(w, L, rng, extra=64)
    nc = tq.compressed_count(_ocfg(w), L)
    pos_c = pos[pos < nc]
    pages, kb, vb = _gpu_blocks(cache, bt[slot], pos_c, w.page_tokens)
    remap = {int(p): i for i, p in enumerate(pages)}
    c = tq.Cache(_ocfg(w), len(pages), np.zeros((1, 1), np.int64))
    c.load_bytes(kb, vb)
    pg = np.array([remap[int(p)] for p in bt[slot][pos_c // w.page_tokens]])
    t = pos_c % w.page_tokens
    P = tq.Params(_ocfg(w))
    q = S.q[slot].double().cpu().numpy()
    worst = 0.0
    for g in range(H):
        est = tq.estimate_scores(P, q[g * G:(g + 1) * G], c.k_codes[pg, g, t], c.k_z[pg, g, t], c.k_nu[pg, g, t],
                                 c.k_gamma[pg, g, t], c.k_side_idx[pg, g, t], c.k_side_val[pg, g, t],
                                 c.k_side_cnt[pg, g, t]) / np.sqrt(d)
        got = lg[g * G:(g + 1) * G][:, pos_c]
        scale = np.abs(est).max()
        worst = max(worst, float(np.abs(got - est).max() / scale))
    assert worst <= 1e-4, worst
    return worst


def _full_size_decode(name, head, logit_slot, quality=False):
    """The decode workload `name` at full size in bench.py's launch
    configuration: sampled append token-heads, one kv head decoded over all its
    tokens from the GPU's bytes, sampled logits; with `quality`, also the rank
    and output agreement of that head with the oracle and with exact attention
    over its raw keys and values."""
    import kv_cache_vector_append_amd as tqa
    w = workloads.WORKLOADS[name]
    torch.cuda.set_device(DEV)
    S = bench.build_decode_setup(w, tqa, torch, DEV)
    nseq, ctx = w.decode_seqs, w.decode_ctx
    hs, hk = head
    # the timed step: append token ctx - 1 of every sequence, decode over ctx tokens
    tqa.quantize_append(S.cfg, S.params, S.cache, S.step_k, S.step_v, *S.app_args)
    out = _decode(S, S.cache)
    assert np.isfinite(out).all()
    # replay the device generator for the inputs at sampled positions
    rng = np.random.default_rng(20241)
    samples = {s: _sample_positions(w, ctx, rng) for s in range(nseq)}
    inputs = {s: ([], []) for s in range(nseq)}
    head_k, head_v = [], []
    g = workloads.device_generator(w, 1, DEV)
    chunk = 16384
    for start in range(0, ctx - 1, chunk):
        n = min(chunk, ctx - 1 - start)
        k = workloads.device_kv(w, "k", nseq * n, g, DEV)
        v = workloads.device_kv(w, "v", nseq * n, g, DEV)
        for s in range(nseq):
            sel = samples[s][(samples[s] >= start) & (samples[s] < start + n)]
            rows = torch.from_numpy(s * n + sel - start).to(DEV)
            inputs[s][0].append(k[rows].double().cpu().numpy())
            inputs[s][1].append(v[rows].double().cpu().numpy())
        if quality:
            head_k.append(k[hs * n:(hs + 1) * n, hk].double().cpu().numpy())
            head_v.append(v[hs * n:(hs + 1) * n, hk].double().cpu().numpy())
        del k, v
    step_k = workloads.device_kv(w, "k", nseq, g, DEV)
    step_v = workloads.device_kv(w, "v", nseq, g, DEV)
    q = workloads.device_queries(w, nseq, g, DEV)
    assert torch.equal(step_k, S.step_k) and torch.equal(q, S.q), "device generator replay diverged"
    for s in range(nseq):
        if samples[s][-1] == ctx - 1:
            inputs[s][0].append(step_k[s:s + 1].double().cpu().numpy())
            inputs[s][1].append(step_v[s:s + 1].double().cpu().numpy())
        inputs[s] = (np.concatenate(inputs[s][0]), np.concatenate(inputs[s][1]))
    bt = S.cache.block_table.cpu().numpy()
    P = tq.Params(_ocfg(w))
    flips = _check_append(w, P, S.cache, bt, samples, inputs)
    err, ref, lg_ref = _check_decode_head(w, S.cache, bt, hs, hk, ctx, S.q, out)
    worst = _logit_samples(w, S, S.cache, bt, logit_slot, rng)
    print(f"[full size] {name}: {sum(len(p) for p in samples.values()) * w.num_kv_heads} sampled "
          f"token-heads ({flips} band flips), decode err {err:.3g} (seq {hs}, kv head {hk}, {ctx} tokens), "
          f"logit rel err {worst:.3g}", flush=True)
    assert err <= DECODE_TOL
    if not quality:
        return
    G, d = w.gqa, w.head_dim
    logits = torch.full((nseq, w.num_q_heads, S.max_ctx), float("nan"), device=DEV)
    _decode(S, S.cache, logits)
    lg_gpu = logits[hs, hk * G:(hk + 1) * G].double().cpu().numpy()
    o_gpu = out[hs, hk * G:(hk + 1) * G]
    Kh = np.concatenate(head_k + [step_k[hs:hs + 1, hk].double().cpu().numpy()])
    Vh = np.concatenate(head_v + [step_v[hs:hs + 1, hk].double().cpu().numpy()])
    qh = S.q[hs, hk * G:(hk + 1) * G].double().cpu().numpy()
    lg_exact = qh @ Kh.T / np.sqrt(d)
    o_exact = tq.exact_attention(qh, Kh, Vh, 1 / np.sqrt(d))
    vs_oracle = (float(_cos(o_gpu, ref).min()),) + _rank_metrics(lg_gpu, lg_ref)
    vs_exact = (float(_cos(o_gpu, o_exact).min()),) + _rank_metrics(lg_gpu, lg_exact)
    for what, m in (("oracle", vs_oracle), ("exact attention", vs_exact)):
        print(f"[full size] {name} vs {what}: cos_sim min {m[0]:.6f}; Spearman rho mean {m[1]:.5f} min {m[2]:.5f}; "
              f"Recall@8 mean {m[3]:.3f} min {m[4]:.3f} (seq {hs}, kv head {hk}, {G} query heads, {ctx} tokens)",
              flush=True)
    # against the oracle: the same computation, so the same ranking
    assert vs_oracle[0] > 1 - 1e-5 and vs_oracle[2] > 0.9999 and vs_oracle[4] >= 7 / 8
    # against exact attention: quality, at the bars [README] "Paper Validation" sets
    assert vs_exact[1] > 0.85 and vs_exact[3] >= 0.40


def test_full_size_outlier_stress_decode():
    """4 x 131072 tokens, 32 q / 8 KV heads, 4/4-bit, FWHT: the default bench workload."""
    _full_size_decode("outlier_stress", head=(2, 5), logit_slot=1, quality=True)


@pytest.mark.parametrize("name", ["hd256_long_dense_3_2", "hd256_long_dense_4_4"])
def test_full_size_head_dim_256_dense_decode(name):
    """8 x 32768 tokens, 16 q / 4 KV heads, head_dim 256, dense rotation (matrix-core append)."""
    _full_size_decode(name, head=(5, 3), logit_slot=6)


def test_full_size_mixed_serving_step():
    """64 x 4096-token append into shuffled pages, then decode of 256 x 4096."""
    import kv_cache_vector_append_amd as tqa
    w = workloads.WORKLOADS["mixed_serving"]
    torch.cuda.set_device(DEV)
    S = bench.build_mixed_setup(w, tqa, torch, DEV)
    nseq, ctx, npre, ntok = w.decode_seqs, w.decode_ctx, w.prefill_seqs, w.prefill_tokens
    tqa.quantize_append(S.cfg, S.params, S.cache, S.step_k, S.step_v, *S.app_args)
    out = _decode(S, S.cache)
    assert np.isfinite(out).all()
    rng = np.random.default_rng(20242)
    # samples: two prefilled sequences and two of the timed append
    pick = [npre, nseq - 1, 0, npre - 1]
    samples = {s: _sample_positions(w, ctx, rng) for s in pick}
    inputs = {}
    g = workloads.device_generator(w, 1, DEV)
    group = 32
    for s0 in range(npre, nseq, group):
        ns = min(group, nseq - s0)
        k = workloads.device_kv(w, "k", ns * ctx, g, DEV)
        v = workloads.device_kv(w, "v", ns * ctx, g, DEV)
        for s in pick:
            if s0 <= s < s0 + ns:
                rows = torch.from_numpy((s - s0) * ctx + samples[s]).to(DEV)
                inputs[s] = (k[rows].double().cpu().numpy(), v[rows].double().cpu().numpy())
        del k, v
    step_k = workloads.device_kv(w, "k", npre * ntok, g, DEV)
    step_v = workloads.device_kv(w, "v", npre * ntok, g, DEV)
    assert torch.equal(step_k, S.step_k), "device generator replay diverged"
    for s in pick:
        if s < npre:
            rows = torch.from_numpy(s * ntok + samples[s]).to(DEV)
            inputs[s] = (step_k[rows].double().cpu().numpy(), step_v[rows].double().cpu().numpy())
    bt = S.cache.block_table.cpu().numpy()
    P = tq.Params(_ocfg(w))
    flips = _check_append(w, P, S.cache, bt, samples, inputs)
    errs = [_check_decode_head(w, S.cache, bt, s, hk, ctx, S.q, out)[0] for s, hk in ((3, 0), (200, 7))]
    worst = _logit_samples(w, S, S.cache, bt, 17, rng)
    print(f"[full size] mixed_serving: {sum(len(p) for p in samples.values()) * w.num_kv_heads} sampled "
          f"token-heads ({flips} band flips), decode err {max(errs):.3g}, logit rel err {worst:.3g}", flush=True)
    assert max(errs) <= DECODE_TOL


@pytest.mark.parametrize("name", ["mixed_3p5_2p5_decode", "scaled_unbiased_3p5_3_decode", "group_values_decode",
                                  "outlier_sidecar_decode"])
def test_full_size_extended_formats(name):
    """The extended stored formats at their benchmark sizes (256 x 4096, or the
    outlier workload's 4 x 131072 with a key sidecar), in bench.py's launch
    configuration; the sidecar workload also reports its quality against exact
    attention, on the same head as the outlier workload without it."""
    _full_size_decode(name, head=(2, 5), logit_slot=1, quality=name == "outlier_sidecar_decode")
