"""GPU parity: the HIP library against the float64 oracle, through the C ABI.

Each workload is run at a reduced size that the oracle finishes in seconds but
that still spans several pages, several 64-token tiles, ragged lengths, a
partially filled last page, the FP16 window boundary and (with chunked
appends) pages filled across several calls.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import tq

from harness import (DECODE_TOL, NORM_RTOL, aligned_oracle_cache, compare_append, decode_error,
                     gpu_cache_as_oracle, gpu_decode, make_run, oracle_config, queries)

pytestmark = pytest.mark.gpu

def _ragged(n, top, spread, step=37):
    """n lengths, the first equal to `top` (the decode's max_ctx), the rest ragged below it."""
    return [top] + [top - (s * step) % spread for s in range(1, n)]


# case name -> (workload, lengths, append calls)
CASES = {
    "tiny_ref": ("tiny_ref", [1024], 1),
    "gqa_decode": ("gqa_decode", [700, 129, 1000], 1),
    "hd256_long_dense_3_2": ("hd256_long_dense_3_2", [300, 77], 1),
    "hd256_long_dense_4_4": ("hd256_long_dense_4_4", [300, 77], 2),
    "hd256_long_fwht_3_2": ("hd256_long_fwht_3_2", [257, 31], 1),
    # head_dim 256 with enough sequences that the decode's split plan gives
    # every split several 128-token blocks (2, 8 and 2 per split): the online
    # softmax re-base, the next-block prefetch and the cross-wavefront merge
    # run across blocks
    "hd256_dense_3_2_multiblock": ("hd256_long_dense_3_2", _ragged(64, 1024, 200), 1),
    "hd256_dense_4_4_multiblock": ("hd256_long_dense_4_4", _ragged(16, 4096, 700), 2),
    "hd256_fwht_3_2_multiblock": ("hd256_long_fwht_3_2", _ragged(64, 1024, 300), 1),
    "outlier_stress": ("outlier_stress", [520, 260, 1], 1),
    "mixed_serving": ("mixed_serving", [400, 3, 160, 0], 3),
    # shapes outside the matrix-core kernel (head_dim 64, GQA group of 8) use the plain kernels
    "plain_hd64_gqa8": ("plain_hd64_gqa8", [300, 130], 2),
    "plain_hd128_gqa8": ("plain_hd128_gqa8", [200, 50], 1),
    # dense rotation, appends of a few tokens per call (partial matrix-core tiles)
    "dense_short_appends": ("dense_short_appends", [40, 13], 8),
    # dense rotation at head_dim 64 (the wavefront-per-token kernel)
    "dense_hd64": ("dense_hd64", [100, 37], 3),
    # extended formats, on the generic path
    "mixed_3p5_2p5": ("mixed_3p5_2p5", [700, 129, 300], 2),
    "mixed_dense_hd256": ("mixed_dense_hd256", [300, 77], 1),
    "scaled_unbiased_3p5_3": ("scaled_unbiased_3p5_3", [520, 33, 257], 2),
    "scaled_mse_dense_hd256": ("scaled_mse_dense_hd256", [300, 77], 1),
    "outlier_sidecar": ("outlier_sidecar", [520, 260, 1], 1),
    "group_values": ("group_values", [400, 3, 160, 0], 3),
    "group_values_dense_hd256": ("group_values_dense_hd256", [300, 77], 1),
    "every_feature_hd64_gqa8": ("every_feature_hd64_gqa8", [300, 130], 2),
    # FWHT decode, where the query operands come from three places: a launch
    # whose narrow kernel (one or two wavefronts per work item) would have
    # fewer wavefronts than the GPU has SIMDs takes four wavefronts per item
    # that build them (most small cases, among them mixed_3p5_2p5_fewsplits and
    # the two manysplits cases); otherwise the split work items build them when
    # a (sequence, kv head) has at most four splits (scaled_unbiased and
    # outlier_sidecar fewsplits, whose kernels have four wavefronts), and a
    # preparation launch does with more (the manyunits cases, outlier_stress)
    "mixed_3p5_2p5_fewsplits": ("mixed_3p5_2p5", [500, 129, 300], 2),
    "scaled_unbiased_3p5_3_fewsplits": ("scaled_unbiased_3p5_3", [500, 33, 257], 2),
    "outlier_sidecar_fewsplits": ("outlier_sidecar", [500, 260, 1], 1),
    "group_values_manysplits": ("group_values", [1000, 3, 160, 0], 3),
    "hd256_fwht_3_2_manysplits": ("hd256_long_fwht_3_2", [1100, 31], 1),
    # dense rotation with fp32 inputs
    "dense_f32_inputs": ("dense_f32_hd256", [300, 77], 1),
    "gqa_decode_manyunits": ("gqa_decode", [800] + _ragged(39, 200, 160), 1),
    "mixed_3p5_2p5_manyunits": ("mixed_3p5_2p5", [800] + _ragged(39, 200, 160), 1),
    "group_values_manyunits": ("group_values", [800] + _ragged(39, 200, 160), 1),
}

import workloads as _w
_w.WORKLOADS.setdefault("plain_hd64_gqa8", _w.GQA_DECODE.replace(
    name="plain_hd64_gqa8", num_q_heads=16, num_kv_heads=2, head_dim=64, key_bits=3, value_bits=3, window=32))
_w.WORKLOADS.setdefault("dense_hd64", _w.GQA_DECODE.replace(
    name="dense_hd64", num_q_heads=8, num_kv_heads=2, head_dim=64, key_bits=3, value_bits=2, window=32,
    rotation="dense"))
_w.WORKLOADS.setdefault("dense_short_appends", _w.HD256_DENSE_32.replace(name="dense_short_appends", window=16))
_w.WORKLOADS.setdefault("plain_hd128_gqa8", _w.GQA_DECODE.replace(
    name="plain_hd128_gqa8", num_q_heads=16, num_kv_heads=2, key_bits=4, value_bits=2, window=48,
    rotation="dense"))
for _name in ("mixed_3p5_2p5", "scaled_unbiased_3p5_3", "outlier_sidecar", "group_values"):
    _w.WORKLOADS.setdefault(_name, _w.WORKLOADS[_name + "_decode"].replace(
        name=_name, num_q_heads=8, num_kv_heads=2))
_w.WORKLOADS.setdefault("mixed_dense_hd256", _w.HD256_DENSE_32.replace(
    name="mixed_dense_hd256", key_bits=3, key_bits_hi=4, value_bits=2, value_bits_hi=4))
_w.WORKLOADS.setdefault("scaled_mse_dense_hd256", _w.HD256_DENSE_32.replace(
    name="scaled_mse_dense_hd256", key_mode="scaled_mse", key_bits=2, value_bits=2))
_w.WORKLOADS.setdefault("group_values_dense_hd256", _w.HD256_DENSE_44.replace(
    name="group_values_dense_hd256", value_mode="group"))
_w.WORKLOADS.setdefault("dense_f32_hd256", _w.HD256_DENSE_32.replace(name="dense_f32_hd256", input_dtype="f32"))
_w.WORKLOADS.setdefault("every_feature_hd64_gqa8", _w.GQA_DECODE.replace(
    name="every_feature_hd64_gqa8", num_q_heads=16, num_kv_heads=2, head_dim=64, key_mode="scaled_unbiased",
    key_bits=2, key_bits_hi=3, value_mode="group", value_bits=2, value_bits_hi=3, key_outliers=3, window=32,
    k_dist="normal_outlier"))

_RUNS = {}
_PARAMS = {}


def _run(name):
    if name not in _RUNS:
        wname, lens, chunks = CASES[name]
        w = workloads.WORKLOADS[wname]
        print(f"[parity] append {name} lens={lens} chunks={chunks}", flush=True)
        key = oracle_config(w)
        run = make_run(w, lens, chunks=chunks, P=_PARAMS.get(key))
        _PARAMS[key] = run.P
        _RUNS[name] = run
    return _RUNS[name]


@pytest.mark.parametrize("name", list(CASES))
def test_append_parity(name):
    run = _run(name)
    rep = compare_append(run)
    print(f"[parity] {name}: {rep}", flush=True)
    assert rep.unexcused == 0
    assert rep.window_mismatch == 0
    assert rep.max_nu_rel < NORM_RTOL and rep.max_gamma_rel < NORM_RTOL


@pytest.mark.parametrize("name", list(CASES))
def test_decode_parity(name):
    run = _run(name)
    nseq = len(run.lens)
    q = queries(run.w, nseq)
    print(f"[parity] decode {name}", flush=True)
    o_gpu, logits = gpu_decode(run, q, want_logits=True)
    gc = gpu_cache_as_oracle(run)
    qn = q.double().numpy()
    o_on_gpu_bytes, lg_ref = tq.decode(run.P, gc, qn, np.arange(nseq), run.lens, return_logits=True)
    oc, adjusted = aligned_oracle_cache(run, gc)
    o_end_to_end = tq.decode(run.P, oc, qn, np.arange(nseq), run.lens)
    e1 = decode_error(o_gpu, o_on_gpu_bytes)
    e2 = decode_error(o_gpu, o_end_to_end)
    print(f"[parity] {name}: decode err over GPU bytes {e1:.3g}, end to end {e2:.3g} "
          f"({adjusted} token-heads with near-threshold decisions aligned)", flush=True)
    assert e1 <= DECODE_TOL and e2 <= DECODE_TOL
    for s, n in enumerate(run.lens):
        if n:
            assert np.allclose(logits[s, :, :n], lg_ref[s], rtol=1e-4, atol=1e-4 * np.abs(lg_ref[s]).max())
    for s, n in enumerate(run.lens):
        if n == 0:
            assert np.all(o_gpu[s] == 0)


@pytest.mark.parametrize("name", ["gqa_decode", "hd256_long_dense_4_4", "outlier_stress", "mixed_dense_hd256",
                                  "scaled_unbiased_3p5_3", "outlier_sidecar", "group_values",
                                  "every_feature_hd64_gqa8"])
def test_dequantize_parity(name):
    import kv_cache_vector_append_amd as tqa
    run = _run(name)
    gc = gpu_cache_as_oracle(run)
    H, d = run.w.num_kv_heads, run.w.head_dim
    for s, n in enumerate(run.lens):
        if n == 0:
            continue
        k = torch.empty((n, H, d), device="cuda")
        v = torch.empty((n, H, d), device="cuda")
        tqa.dequantize(run.cfg, run.params, run.cache, s, 0, n, k, v)
        torch.cuda.synchronize()
        kr, vr = tq.dequantize(run.P, gc, s, 0, n)
        for got, ref in ((k, kr), (v, vr)):
            err = np.abs(got.cpu().double().numpy() - ref).max() / np.abs(ref).max()
            assert err < 1e-5, err


@pytest.mark.parametrize("name", ["gqa_decode", "scaled_unbiased_3p5_3", "outlier_sidecar"])
def test_decode_matches_attention_over_gpu_dequantized(name):
    # invariant: compressed-domain decode == exact attention over the dequantized cache
    import kv_cache_vector_append_amd as tqa
    run = _run(name)
    H, d, G = run.w.num_kv_heads, run.w.head_dim, run.w.gqa
    q = queries(run.w, len(run.lens))
    o_gpu, _ = gpu_decode(run, q)
    gc = gpu_cache_as_oracle(run)
    for s, n in enumerate(run.lens):
        nc = max(0, n - run.w.window)
        k = torch.empty((nc, H, d), device="cuda")
        v = torch.empty((nc, H, d), device="cuda")
        tqa.dequantize(run.cfg, run.params, run.cache, s, 0, nc, k, v)
        torch.cuda.synchronize()
        k, v = k.cpu().double().numpy(), v.cpu().double().numpy()
        wpos = np.arange(nc, n) % run.w.window
        for g in range(H):
            kk = np.concatenate([k[:, g], gc.k_window[s, g, wpos].astype(np.float64)])
            vv = np.concatenate([v[:, g], gc.v_window[s, g, wpos].astype(np.float64)])
            ref = tq.exact_attention(q[s, g * G:(g + 1) * G].double().numpy(), kk, vv, 1 / np.sqrt(d))
            assert decode_error(o_gpu[s, g * G:(g + 1) * G], ref) < DECODE_TOL


def test_append_is_deterministic():
    w = workloads.GQA_DECODE
    a = make_run(w, [333, 50], oracle_append=False)
    b = make_run(w, [333, 50], oracle_append=False, P=a.P)
    for s, n in enumerate([333, 50]):
        ga, gb = gpu_cache_as_oracle(a).gather(s, np.arange(n)), gpu_cache_as_oracle(b).gather(s, np.arange(n))
        for key in ga:
            assert np.array_equal(ga[key], gb[key]), key


def test_edge_cases_single_tokens_and_page_edges():
    # lengths 1, 16, 17 and 33 appended in two calls: single tokens, a full
    # page, one token past a page edge, pages completed across calls
    w = workloads.TINY_REF.replace(num_q_heads=2, num_kv_heads=1, window=16, input_dtype="f32")
    run = make_run(w, [1, 16, 17, 33], chunks=2)
    rep = compare_append(run)
    assert rep.unexcused == 0 and rep.window_mismatch == 0
    q = queries(w, 4)
    o_gpu, _ = gpu_decode(run, q)
    o_ref = tq.decode(run.P, gpu_cache_as_oracle(run), q.double().numpy(), np.arange(4), run.lens)
    assert decode_error(o_gpu, o_ref) <= DECODE_TOL


def test_zero_vector_append():
    import kv_cache_vector_append_amd as tqa
    w = workloads.TINY_REF.replace(input_dtype="f32")
    run = make_run(w, [20])
    kz = torch.zeros((1, 1, 128), device="cuda")
    vz = torch.zeros((1, 1, 128), device="cuda")
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    tqa.quantize_append(run.cfg, run.params, run.cache, kz, vz, i32([0]), i32([20]), i32([0, 1]), 1)
    torch.cuda.synchronize()
    g = gpu_cache_as_oracle(run).gather(0, [20])
    assert g["k_nu"][0, 0] == 0 and g["k_gamma"][0, 0] == 0 and g["v_nu"][0, 0] == 0
    assert not g["k_codes"].any() and not g["k_z"].any() and not g["v_codes"].any()
    q = queries(w, 1)
    o_gpu, _ = gpu_decode(run, q, lens=[21])
    assert np.isfinite(o_gpu).all()


@pytest.mark.parametrize("value_bits", [2, 4])
def test_zero_rows_inside_long_appends(monkeypatch, value_bits):
    """Zero key or value rows inside appends of 100 and 70 tokens, which take the
    token-per-lane kernel: each zero row stores nu = gamma = 0 and all-zero bits,
    while its neighbours in the same wavefront keep their codes bit for bit."""
    zero_rows = {"k": (3, 40, 77), "v": (5, 40, 64)}
    orig = workloads.kv_tokens

    def with_zero_rows(w, which, seq, start, count):
        x = orig(w, which, seq, start, count).clone()
        for r in zero_rows[which]:
            if start <= r < start + count:
                x[r - start] = 0
        return x

    monkeypatch.setattr(workloads, "kv_tokens", with_zero_rows)
    w = workloads.GQA_DECODE.replace(num_q_heads=8, num_kv_heads=2, window=16, value_bits=value_bits,
                                     key_bits=4 if value_bits == 4 else 3)
    run = make_run(w, [100, 70])
    rep = compare_append(run)
    assert rep.tokens == 170 * w.num_kv_heads and rep.unexcused == 0 and rep.window_mismatch == 0
    gc = gpu_cache_as_oracle(run)
    for s, n in enumerate(run.lens):
        g = gc.gather(s, [r for r in zero_rows["k"] if r < n])
        assert not g["k_nu"].any() and not g["k_gamma"].any()
        assert not g["k_codes"].any() and not g["k_z"].any()
        g = gc.gather(s, [r for r in zero_rows["v"] if r < n])
        assert not g["v_nu"].any() and not g["v_codes"].any()
    q = queries(w, 2)
    o_gpu, _ = gpu_decode(run, q)
    o_ref = tq.decode(run.P, gc, q.double().numpy(), np.arange(2), run.lens)
    assert decode_error(o_gpu, o_ref) <= DECODE_TOL


@pytest.mark.parametrize("wname,max_new", [("hd256_long_dense_3_2", 1), ("gqa_decode", 32), ("outlier_stress", 40)])
def test_understated_launch_bound_still_writes_every_token(wname, max_new):
    """max_new_per_seq only sizes the launch: 200- and 130-token appends with a
    bound of 1 (dense matrix-core kernel, two chunk workers per sequence) or 32
    and 40 (token-per-lane kernel) must still write every position."""
    w = workloads.WORKLOADS[wname]
    w = w.replace(num_q_heads=w.num_q_heads // w.num_kv_heads * 2, num_kv_heads=2)
    print(f"[parity] understated bound {wname} max_new={max_new}", flush=True)
    run = make_run(w, [200, 130], max_new=max_new)
    rep = compare_append(run)
    print(f"[parity] {rep}", flush=True)
    assert rep.tokens == 330 * 2 and rep.unexcused == 0 and rep.window_mismatch == 0
    assert rep.max_nu_rel < NORM_RTOL and rep.max_gamma_rel < NORM_RTOL


@pytest.mark.parametrize("wname", ["gqa_decode", "hd256_long_dense_3_2"])
def test_status_word_reports_skipped_work(wname):
    """Debug capacity checks: a block-table entry outside the pool, a slot
    outside the table and a position beyond the table's pages are skipped and
    reported in the caller's status word, and every other token is written
    exactly as the oracle writes it."""
    import kv_cache_vector_append_amd as tqa
    from harness import lib_config, oracle_config
    w = workloads.WORKLOADS[wname]
    w = w.replace(num_q_heads=w.num_q_heads // w.num_kv_heads * 2, num_kv_heads=2)
    cfg, ocfg = lib_config(w), oracle_config(w)
    dev = "cuda"
    lens, mpp = [300, 90], 20
    bt = workloads.block_table(w, 2, mpp).numpy().copy()
    bad_page = 4                                   # positions 64..79 of sequence 0, outside the window
    bt[0, bad_page] = 2 * mpp + 7                  # outside the 2 * mpp pages of the pool
    params = torch.empty(tqa.params_bytes(cfg), dtype=torch.uint8, device=dev)
    tqa.init_codebooks(cfg, params)
    cache = tqa.allocate_cache(cfg, 2 * mpp, torch.from_numpy(bt), dev)
    cache.status = torch.zeros(1, dtype=torch.int32, device=dev)
    K = [workloads.kv_tokens(w, "k", s, 0, n) for s, n in enumerate(lens)]
    V = [workloads.kv_tokens(w, "v", s, 0, n) for s, n in enumerate(lens)]
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    kn, vn = torch.cat(K).to(dev), torch.cat(V).to(dev)
    cu = [0, lens[0], lens[0] + lens[1]]
    for max_new in (300, 8):                       # two launch shapes (and, for FWHT, two kernels)
        cache.status.zero_()
        tqa.quantize_append(cfg, params, cache, kn, vn, i32([0, 1]), i32([0, 0]), i32(cu), max_new)
        torch.cuda.synchronize()
        assert int(cache.status.item()) == tqa.TQ_STATUS_BAD_PAGE
    # every position outside the bad page is bit-exact (up to the threshold band)
    P = tq.Params(ocfg)
    from harness import Run, compare_append as cmp
    run = Run(w, lens, cfg, params, cache, ocfg, P, tq.Cache(ocfg, 2 * mpp, np.where(bt >= 2 * mpp, 0, bt)), K, V,
              np.where(bt >= 2 * mpp, 0, bt))
    keep = [np.array([p for p in range(lens[0]) if p // w.page_tokens != bad_page]), np.arange(lens[1])]
    rep = cmp(run, positions=keep)
    assert rep.tokens == (lens[0] - 16 + lens[1]) * 2 and rep.unexcused == 0
    # a slot outside the table, and positions past the table's pages
    cache.status.zero_()
    tqa.quantize_append(cfg, params, cache, kn[:10], vn[:10], i32([5]), i32([0]), i32([0, 10]), 10)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == tqa.TQ_STATUS_BAD_SLOT
    cache.status.zero_()
    tqa.quantize_append(cfg, params, cache, kn[:40], vn[:40], i32([1]), i32([mpp * 16 - 8]), i32([0, 40]), 40)
    torch.cuda.synchronize()
    assert int(cache.status.item()) == tqa.TQ_STATUS_CAPACITY
    # decode over the bad page: reported, and the output stays finite
    cache.status.zero_()
    q = queries(w, 2)
    o_gpu, _ = gpu_decode(run, q)
    torch.cuda.synchronize()
    assert int(cache.status.item()) & tqa.TQ_STATUS_BAD_PAGE
    assert np.isfinite(o_gpu).all()
