"""Benchmark of the compressed-KV hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the whole hot path over one batch: quantize-append of
the step's new tokens (decode workloads: one new token per sequence; the mixed
serving workload: a 64 x 4096-token prefill) followed by decode attention over
every sequence's full context.  Inputs are seeded, synthetic and resident in
HBM before timing starts.  Prints one JSON line.

value = decoded cached tokens per second over the whole step (sum of context
lengths attended per step / step time).  The `roofline` object covers the
dominant call, timed live with HIP events on the stream the library launches
on; `quality_vs_exact` compares one head's output and logit ranking with exact
attention over its raw keys and values; `other_workloads` repeats the step for
the other workloads (mixed serving, head_dim 256 at both bit widths, the dense
append, GQA decode); `cpu_baseline` times the float64 oracle on a bounded
sample of the same workload on the host's cores (before the GPU is used).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_F16_TFLOPS = 2500.0   # dense fp16 matrix-core peak (no sparsity)
DENSE_SPLIT_PASSES = 3          # hi*hi + hi*lo + lo*hi fp16 products per contraction
DEFAULT_WORKLOAD = "outlier_stress"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def record_bytes(w):
    """Stored bytes per token-head: key = code bits (+ d/8 QJL signs) + the two
    fp32 of the key (+ the sidecar record); value = code bits + nu (or the fp16
    scale/zero pairs of group-quantized values)."""
    d = w.head_dim
    kb = (w.key_bits + (w.key_bits_hi or w.key_bits)) * d // 16        # each half at its own rate
    key = kb + 8
    if w.key_outliers:
        head = 1 + w.key_outliers + ((1 + w.key_outliers) & 1)
        key += (head + 2 * w.key_outliers + 3) // 4 * 4
    value = (w.value_bits + (w.value_bits_hi or w.value_bits)) * d // 16
    value += d // 32 * 4 if w.value_mode == "group" else 4
    return key, value


def dense_append_flops(w, counts):
    """Algorithmic flops of the dense-rotation append: three d x d products per
    new token-head (Pi_K x, G e, Pi_V v), 2 d^2 flops each."""
    return sum(counts) * w.num_kv_heads * 3 * 2 * w.head_dim ** 2


def in_bytes(w):
    return 4 if w.input_dtype == "f32" else 2


def decode_algorithmic_bytes(w, lens):
    """Bytes the decode call must move: packed records of compressed token-heads,
    fp16 window K/V, the block-table entries, the query and the fp32 output."""
    kr, vr = record_bytes(w)
    H, d, W = w.num_kv_heads, w.head_dim, w.window
    tot = 0
    for L in lens:
        nc = max(0, L - W) if W else L
        tot += H * (nc * (kr + vr) + (L - nc) * 2 * d * 2)
        tot += 4 * math.ceil(L / w.page_tokens)
    tot += len(lens) * w.num_q_heads * d * (in_bytes(w) + 4)
    return tot


def append_algorithmic_bytes(w, counts, lens_after):
    """Bytes the append call must move: the new K/V rows, their packed records,
    and the fp16 copies of tokens landing in the window."""
    kr, vr = record_bytes(w)
    H, d, W = w.num_kv_heads, w.head_dim, w.window
    tot = 0
    for n, L in zip(counts, lens_after):
        tot += n * H * (2 * d * in_bytes(w) + kr + vr)
        if W:
            tot += min(n, W) * H * 2 * d * 2
    return tot


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Sources each call's kernels are built from (the traffic entry is only used
# while they are unchanged) and the kernels one call launches.
_CSRC = "kv_cache_vector_append_amd/csrc/"
SOURCES = {
    "decode": [_CSRC + f for f in ("tq_decode_mfma.hip", "tq_mfma.h", "tq_codec.hip", "tq_device.h",
                                   "tq_internal.h")],
    "append": [_CSRC + f for f in ("tq_append.hip", "tq_device.h", "tq_internal.h")],
}
KERNELS = {
    "decode": "tq_decode_attention (decode_split + decode_combine, after decode_prep where that launch builds "
              "the query operands)",
    "append": "tq_quantize_append (append_tok_kernel, append_dense_kernel or append_kernel)",
}
# rocprofv3 kernel names of each call's kernels (an append launches one of the
# alternatives); groups in OPTIONAL_KERNELS may be absent (the split work items
# build the query operands themselves)
KERNEL_MATCH = {"decode": (("decode_prep_kernel",), ("decode_split_kernel",), ("decode_combine_kernel",)),
                "append": (("append_tok_kernel", "append_dense_kernel", "append_kernel<"),)}
OPTIONAL_KERNELS = {("decode_prep_kernel",)}
CALIBRATION_BYTES = 1 << 30


def hbm_reference():
    """Streaming rates plain torch kernels reach on this GPU in the same run, as
    context for the decode's rate: a read-only reduction and an elementwise
    read + write pass over four rotating 1 GiB fp32 buffers (so that no pass
    finds its data in the last-level cache), each timed with one event pair
    over 8 passes after 2 untimed ones."""
    import torch
    n = CALIBRATION_BYTES // 4
    bufs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(4)]
    out = torch.empty(n, dtype=torch.float32, device="cuda:0")
    acc = torch.empty((), dtype=torch.float32, device="cuda:0")

    def rate(fn, bytes_per_pass):
        for i in range(2):
            fn(bufs[i % 4])
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(8):
            fn(bufs[(i + 2) % 4])
        e.record()
        e.synchronize()
        return bytes_per_pass * 8 / (s.elapsed_time(e) / 1e3) / 1e9

    read = rate(lambda b: torch.sum(b, dim=0, out=acc), CALIBRATION_BYTES)
    read_write = rate(lambda b: torch.neg(b, out=out), 2 * CALIBRATION_BYTES)
    del bufs, out, acc
    torch.cuda.empty_cache()
    return {"read_GBs": round(read, 1), "read_write_GBs": round(read_write, 1),
            "method": "torch.sum (read) and torch.neg (read + write) over four rotating 1 GiB fp32 buffers, "
                      "8 timed passes each"}


def calibration_copy():
    """One plain device-to-device copy of CALIBRATION_BYTES (read once, written
    once), whose FETCH_SIZE / WRITE_SIZE calibrate the counters' units."""
    import torch
    a = torch.zeros(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    # an elementwise kernel with a name nothing else in the run has (a plain
    # memcpy may run on a DMA engine, which the counters do not see)
    torch.bitwise_not(a, out=b)
    torch.cuda.synchronize()
    del a, b


def _counter_sums(path, counter):
    """Per-dispatch values of `counter` from a rocprofv3 counter_collection.csv:
    {kernel name: [(dispatch id, value), ...] in dispatch order}."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append((int(row["Dispatch_Id"]), float(row["Counter_Value"])))
    for v in out.values():
        v.sort()
    return out


# dispatches of each kernel group taken from a counter run: the last ones, i.e.
# the timed steps (the runs use --steps 2 --warmup 1; prefill dispatches come first)
TRAFFIC_LAST_DISPATCHES = 2


def write_traffic(fetch_csv, write_csv, workload):
    fetch = _counter_sums(fetch_csv, "FETCH_SIZE")
    write = _counter_sums(write_csv, "WRITE_SIZE")

    def copy_kib(d):
        # the calibration kernel is the run's only bitwise-not
        cands = [max(x for _, x in v) for k, v in d.items() if "bitwise_not" in k.lower() or "bitwisenot" in k.lower()]
        return max(cands) if cands else None

    fk, wk = copy_kib(fetch), copy_kib(write)
    f_scale = CALIBRATION_BYTES / fk if fk else None   # bytes per counted unit
    w_scale = CALIBRATION_BYTES / wk if wk else None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data["_calibration"] = {"copy_bytes": CALIBRATION_BYTES, "fetch_units": fk, "write_units": wk,
                            "fetch_bytes_per_unit": f_scale, "write_bytes_per_unit": w_scale}
    for call, groups in KERNEL_MATCH.items():
        per_kernel = {}
        for alts in groups:
            # the group's last dispatches, whichever alternative they ran (the
            # timed calls come after the prefill)
            fv = sorted((i, v, n) for n in alts for k, vals in fetch.items() if n in k for i, v in vals)
            wv = sorted((i, v, n) for n in alts for k, vals in write.items() if n in k for i, v in vals)
            if fv and wv:
                fl, wl = fv[-TRAFFIC_LAST_DISPATCHES:], wv[-TRAFFIC_LAST_DISPATCHES:]
                per_kernel[fl[-1][2]] = (float(np.median([v for _, v, _ in fl])), float(np.median([v for _, v, _ in wl])))
        required = [g for g in groups if g not in OPTIONAL_KERNELS]
        found = {n for alts in groups for n in alts if any(n in k for k in per_kernel)}
        if any(not any(n in found for n in alts) for alts in required) or not f_scale or not w_scale:
            continue
        fb = sum(v[0] for v in per_kernel.values()) * f_scale
        wb = sum(v[1] for v in per_kernel.values()) * w_scale
        data[f"{call}:{workload}"] = {
            "hbm_bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb), "write_bytes": int(wb),
            "per_kernel_median_units": per_kernel, "source_hash": source_hash(SOURCES[call])}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps(data, indent=1, sort_keys=True))
    return 0


def measured_traffic(kernel_key, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- GPU side

class Setup:
    pass


def library_config(w, tqa):
    """The library's tq_config of a workload, stored format included."""
    return tqa.Config(w.head_dim, w.num_q_heads, w.num_kv_heads, w.key_bits, w.value_bits, w.page_tokens,
                      w.window, w.rotation, w.method_seed, key_mode=w.key_mode, value_mode=w.value_mode,
                      key_bits_hi=w.key_bits_hi, value_bits_hi=w.value_bits_hi, key_outliers=w.key_outliers)


def build_decode_setup(w, tqa, torch, dev, keep_head=None):
    """Cache filled with decode_ctx - 1 tokens per sequence; the step appends token
    decode_ctx - 1 of every sequence and decodes over decode_ctx tokens.
    keep_head = (seq, kv head): also keep that head's raw keys and values of all
    decode_ctx positions on the device (S.head_k, S.head_v), for quality metrics."""
    import workloads
    S = Setup()
    nseq, ctx = w.decode_seqs, w.decode_ctx
    mpp = w.pages_per_seq(ctx)
    S.cfg = library_config(w, tqa)
    S.params = torch.empty(tqa.params_bytes(S.cfg), dtype=torch.uint8, device=dev)
    tqa.init_codebooks(S.cfg, S.params)
    bt = workloads.block_table(w, nseq, mpp)
    S.cache = tqa.allocate_cache(S.cfg, nseq * mpp, bt, dev)
    g = workloads.device_generator(w, 1, dev)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    slots = i32(list(range(nseq)))
    chunk = 16384
    hk_parts, hv_parts = [], []
    for start in range(0, ctx - 1, chunk):
        n = min(chunk, ctx - 1 - start)
        k = workloads.device_kv(w, "k", nseq * n, g, dev)
        v = workloads.device_kv(w, "v", nseq * n, g, dev)
        tqa.quantize_append(S.cfg, S.params, S.cache, k, v, slots, i32([start] * nseq),
                            i32([i * n for i in range(nseq + 1)]), n)
        if keep_head is not None:
            hs, hh = keep_head
            hk_parts.append(k[hs * n:(hs + 1) * n, hh].clone())
            hv_parts.append(v[hs * n:(hs + 1) * n, hh].clone())
        del k, v
    torch.cuda.synchronize()
    log(f"prefilled {nseq} x {ctx - 1} tokens")
    S.step_k = workloads.device_kv(w, "k", nseq, g, dev)
    S.step_v = workloads.device_kv(w, "v", nseq, g, dev)
    if keep_head is not None:
        hs, hh = keep_head
        S.keep_head = keep_head
        S.head_k = torch.cat(hk_parts + [S.step_k[hs:hs + 1, hh]])
        S.head_v = torch.cat(hv_parts + [S.step_v[hs:hs + 1, hh]])
    S.app_args = (slots, i32([ctx - 1] * nseq), i32(list(range(nseq + 1))), 1)
    S.q = workloads.device_queries(w, nseq, g, dev)
    S.dec_slots, S.dec_lens = slots, i32([ctx] * nseq)
    S.lens = [ctx] * nseq
    S.max_ctx = ctx
    S.app_counts, S.app_lens_after = [1] * nseq, [ctx] * nseq
    S.ws = torch.empty(tqa.decode_workspace_bytes(S.cfg, nseq, ctx) // 4 + 4, dtype=torch.float32, device=dev)
    S.out = torch.empty((nseq, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    return S


def build_mixed_setup(w, tqa, torch, dev):
    """256 sequences of 4096 tokens; the step re-appends all 4096 tokens of
    sequences 0..63 (a prefill) and decodes all 256 sequences."""
    import workloads
    S = Setup()
    nseq, ctx, npre, ntok = w.decode_seqs, w.decode_ctx, w.prefill_seqs, w.prefill_tokens
    mpp = w.pages_per_seq(ctx)
    S.cfg = library_config(w, tqa)
    S.params = torch.empty(tqa.params_bytes(S.cfg), dtype=torch.uint8, device=dev)
    tqa.init_codebooks(S.cfg, S.params)
    bt = workloads.block_table(w, nseq, mpp)
    S.cache = tqa.allocate_cache(S.cfg, nseq * mpp, bt, dev)
    g = workloads.device_generator(w, 1, dev)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    group = 32
    for s0 in range(npre, nseq, group):
        ns = min(group, nseq - s0)
        k = workloads.device_kv(w, "k", ns * ctx, g, dev)
        v = workloads.device_kv(w, "v", ns * ctx, g, dev)
        tqa.quantize_append(S.cfg, S.params, S.cache, k, v, i32(list(range(s0, s0 + ns))), i32([0] * ns),
                            i32([i * ctx for i in range(ns + 1)]), ctx)
        del k, v
    torch.cuda.synchronize()
    log(f"prefilled sequences {npre}..{nseq - 1} x {ctx} tokens")
    S.step_k = workloads.device_kv(w, "k", npre * ntok, g, dev)
    S.step_v = workloads.device_kv(w, "v", npre * ntok, g, dev)
    S.app_args = (i32(list(range(npre))), i32([0] * npre), i32([i * ntok for i in range(npre + 1)]), ntok)
    S.q = workloads.device_queries(w, nseq, g, dev)
    S.dec_slots, S.dec_lens = i32(list(range(nseq))), i32([ctx] * nseq)
    S.lens = [ctx] * nseq
    S.max_ctx = ctx
    S.app_counts, S.app_lens_after = [ntok] * npre, [ntok] * npre
    S.ws = torch.empty(tqa.decode_workspace_bytes(S.cfg, nseq, ctx) // 4 + 4, dtype=torch.float32, device=dev)
    S.out = torch.empty((nseq, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    return S


def replicate_cache(S, tqa, w, copies):
    """Independent copies of the filled cache (pages and fp16 rings), so that
    consecutive steps never find the previous step's pages in the 256 MB
    last-level cache."""
    c = S.cache
    S.caches = [c] + [tqa.CacheBuffers(c.k_pages.clone(), c.v_pages.clone(), c.block_table,
                                       None if c.k_window is None else c.k_window.clone(),
                                       None if c.v_window is None else c.v_window.clone())
                      for _ in range(copies - 1)]


def run_gpu(w, steps, warmup, copies, keep_head=None):
    import torch
    import kv_cache_vector_append_amd as tqa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S = (build_mixed_setup(w, tqa, torch, dev) if w.prefill_seqs
         else build_decode_setup(w, tqa, torch, dev, keep_head=keep_head))
    if copies <= 0:
        copies = 4 if decode_algorithmic_bytes(w, S.lens) < 2 ** 30 else 1
    replicate_cache(S, tqa, w, copies)
    torch.cuda.synchronize()
    log(f"{copies} cache copies rotated across steps")
    stream = torch.cuda.current_stream()

    def append(i):
        tqa.quantize_append(S.cfg, S.params, S.caches[i % copies], S.step_k, S.step_v, *S.app_args, stream=stream)

    def decode(i):
        tqa.decode_attention(S.cfg, S.params, S.caches[i % copies], S.q, S.dec_slots, S.dec_lens, S.max_ctx, S.out,
                             S.ws, stream=stream)

    for i in range(warmup):
        append(i)
        decode(i)
    torch.cuda.synchronize()
    # the step, steps times: append then decode, each call between a pair of
    # events on its stream (their durations are the calls' launch durations;
    # the pair around the loop times the steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        append(warmup + i)
        ev[i][1].record(stream)
        decode(warmup + i)
        ev[i][2].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    app_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    if not torch.isfinite(S.out).all():
        raise RuntimeError("non-finite decode output")
    log(f"{steps} steps: {total_ms:.3f} ms on the stream ({wall * 1e3:.1f} ms wall); "
        f"append {app_ms * 1e3:.1f} us, decode {dec_ms * 1e3:.1f} us per call")
    return dict(total_ms=total_ms, app_ms=app_ms, dec_ms=dec_ms, lens=S.lens, app_counts=S.app_counts,
                app_lens_after=S.app_lens_after, copies=copies, setup=S)


def step_summary(w, r, steps):
    """Per-step throughput and each call's achieved HBM rate for one workload."""
    ms = r["total_ms"] / steps
    dec_bytes = decode_algorithmic_bytes(w, r["lens"])
    app_bytes = append_algorithmic_bytes(w, r["app_counts"], r["app_lens_after"])
    out = {"ms_per_step": round(ms, 5), "value": round(sum(r["lens"]) / (ms / 1e3), 1), "unit": "cached tokens/s"}
    for call, b, t in (("decode", dec_bytes, r["dec_ms"]), ("append", app_bytes, r["app_ms"])):
        gbs = b / (t / 1e3) / 1e9
        out[call] = {"avg_launch_ms": round(t, 5), "algorithmic_bytes_per_launch": int(b),
                     "achieved_GBs": round(gbs, 2), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    if w.rotation == "dense" and w.prefill_seqs:
        tflops = dense_append_flops(w, r["app_counts"]) / (r["app_ms"] / 1e3) / 1e12
        out["append"].update({"bound": "mfma", "achieved_TFLOPs": round(tflops, 2),
                              "frac_of_fp16_mfma_peak": round(tflops / PEAK_MFMA_F16_TFLOPS, 4)})
    return out


def quality_vs_exact(w, S):
    """Output cosine, and the Spearman rank correlation and Recall@8 of the
    logits, of one kv head's query group against exact softmax attention over
    that head's raw keys and values (fp32 on the device: a measurement, not
    part of the library's path)."""
    import torch
    import kv_cache_vector_append_amd as tqa
    hs, hh = S.keep_head
    G, d, L = w.gqa, w.head_dim, S.lens[hs]
    logits = torch.full((len(S.lens), w.num_q_heads, S.max_ctx), float("nan"), device=S.q.device)
    tqa.decode_attention(S.cfg, S.params, S.cache, S.q, S.dec_slots, S.dec_lens, S.max_ctx, S.out, S.ws,
                         logits=logits)
    torch.cuda.synchronize()
    q = S.q[hs, hh * G:(hh + 1) * G].float()
    K, V = S.head_k.float(), S.head_v.float()
    exact_logits = (q @ K.T) / math.sqrt(d)
    o_exact = torch.softmax(exact_logits, dim=-1) @ V
    o = S.out[hs, hh * G:(hh + 1) * G]
    cos = torch.nn.functional.cosine_similarity(o, o_exact, dim=-1)
    est = logits[hs, hh * G:(hh + 1) * G, :L]

    def ranks(x):
        r = torch.empty_like(x)
        r.scatter_(-1, torch.argsort(x, dim=-1), torch.arange(x.shape[-1], device=x.device, dtype=x.dtype).expand_as(x))
        return r

    ra, rb = ranks(est.double()), ranks(exact_logits.double())
    ra, rb = ra - ra.mean(-1, keepdim=True), rb - rb.mean(-1, keepdim=True)
    rho = (ra * rb).sum(-1) / (ra.norm(dim=-1) * rb.norm(dim=-1))
    top_a = torch.topk(est, 8, dim=-1).indices
    top_b = torch.topk(exact_logits, 8, dim=-1).indices
    recall = (top_a[:, :, None] == top_b[:, None, :]).any(-1).float().mean(-1)
    return {"against": "exact fp32 softmax attention over the raw bf16 keys and values",
            "head": f"sequence {hs}, kv head {hh}, {G} query heads, {L} tokens",
            "cos_sim_min": round(float(cos.min()), 6), "cos_sim_mean": round(float(cos.mean()), 6),
            "spearman_rho_mean": round(float(rho.mean()), 5), "spearman_rho_min": round(float(rho.min()), 5),
            "recall_at_8_mean": round(float(recall.mean()), 4), "recall_at_8_min": round(float(recall.min()), 4)}


# ----------------------------------------------------------------------------- CPU oracle baseline

# One oracle work unit: one (sequence, kv head) of the workload -- append
# UNIT_CTX tokens of that kv head, then decode its query group over them.
# Built in the parent before any worker is forked (and before the GPU is
# touched); the workers only run numpy.
UNIT_CTX = 8192
MAX_WORKERS = 16          # the host's CPU share per GPU
_UNIT = {}


def _unit_setup(w):
    import workloads
    from oracle import tq
    G = w.gqa
    cfg1 = tq.Config(w.head_dim, G, 1, w.key_bits, w.value_bits, w.page_tokens, w.window, w.rotation,
                     w.method_seed)
    ctx = min(UNIT_CTX, w.decode_ctx)
    _UNIT.update(cfg=cfg1, P=tq.Params(cfg1), ctx=ctx,
                 K=workloads.kv_tokens(w, "k", 0, 0, ctx)[:, 0:1].double().numpy(),
                 V=workloads.kv_tokens(w, "v", 0, 0, ctx)[:, 0:1].double().numpy(),
                 q=workloads.queries(w, 0)[:G].double().numpy()[None])


def _unit_run(_=None):
    """(append seconds, decode seconds) of one unit, on one thread."""
    from threadpoolctl import threadpool_limits
    from oracle import tq
    u = _UNIT
    with threadpool_limits(1):
        mpp = math.ceil(u["ctx"] / u["cfg"].page_tokens)
        c = tq.Cache(u["cfg"], mpp, np.arange(mpp)[None])
        t0 = time.perf_counter()
        tq.append(u["P"], c, u["K"], u["V"], [0], [0], [0, u["ctx"]])
        t1 = time.perf_counter()
        tq.decode(u["P"], c, u["q"], [0], [u["ctx"]])
        t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def cpu_baseline(w, reps=4):
    """The float64 oracle, as it stands, on a bounded sample of the workload:
    (sequence, kv head) units timed on one core, then on N worker processes
    at once (N = the host's cores, at most MAX_WORKERS), scaled to the step's
    appended token-heads and cached token-heads.  Call before the GPU is used
    (the workers are forked)."""
    import multiprocessing as mp
    _unit_setup(w)
    _unit_run()                                                    # warm-up
    one = [_unit_run() for _ in range(reps)]
    t_app = float(np.median([a for a, _ in one])) / _UNIT["ctx"]   # seconds per appended token-head
    t_dec = float(np.median([d for _, d in one])) / _UNIT["ctx"]   # seconds per cached token-head (query group)
    cores = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = cores
    n = max(1, min(cores, avail, MAX_WORKERS))
    with mp.get_context("fork").Pool(n) as pool:
        pool.map(_unit_run, range(n))                              # warm-up in every worker
        t0 = time.perf_counter()
        pool.map(_unit_run, range(n * reps), chunksize=1)
        wall = time.perf_counter() - t0
    speedup = (n * reps / wall) * (t_app + t_dec) * _UNIT["ctx"]
    H = w.num_kv_heads
    cached_th = w.decode_seqs * w.decode_ctx * H
    appended_th = (w.prefill_seqs * w.prefill_tokens if w.prefill_seqs else w.decode_seqs) * H
    t_step_1 = appended_th * t_app + cached_th * t_dec
    tokens = w.decode_seqs * w.decode_ctx
    return {"value": round(tokens / (t_step_1 / speedup), 1), "unit": "cached tokens/s", "cores": n,
            "kind": "oracle", "value_1core": round(tokens / t_step_1, 1), "speedup_over_1core": round(speedup, 2),
            "os_cpu_count": cores,
            "sample": f"oracle (float64 numpy, one thread per process) on (sequence, kv head) units of "
                      f"{_UNIT['ctx']} tokens: append of the unit's tokens "
                      f"({t_app * _UNIT['ctx']:.3f} s) and decode of its {w.gqa} query heads over them "
                      f"({t_dec * _UNIT['ctx']:.3f} s), median of {reps} on 1 core; {n * reps} units on {n} "
                      f"processes in {wall:.2f} s; scaled to the step's {appended_th} appended and {cached_th} "
                      f"cached token-heads"}


# ----------------------------------------------------------------------------- main

# Workloads timed after the headline one and reported in the same line: the
# mixed serving step (append-heavy), the head_dim-256 decode at both bit
# widths, the dense rotation's matrix-core append, and the latency-bound GQA
# decode.
EXTRA_WORKLOADS = ("mixed_serving", "hd256_long_dense_3_2", "hd256_long_dense_4_4", "hd256_dense_prefill",
                   "gqa_decode",
                   # extended stored formats: mixed-channel rates, scaled keys, group-quantized
                   # values, and the outlier workload with a key sidecar
                   "mixed_3p5_2p5_decode", "scaled_unbiased_3p5_3_decode", "group_values_decode",
                   "outlier_sidecar_decode")
# (sequence, kv head) whose query group the quality metrics cover (the same
# head with and without the key sidecar)
QUALITY_HEAD = {"outlier_stress": (2, 5), "outlier_sidecar_decode": (2, 5)}
# what the decode arithmetic is: scores and value sums on the matrix cores with
# the fp32 query / softmax weights carried as four fp8 parts against fp4 code
# bit-planes, accumulated in fp32
DTYPE = "fp8x4*fp4->f32"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=60,
                    help="untimed steps first: the decode call runs ~10%% slower for its first ~40 calls on a box")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="time only --workload")
    ap.add_argument("--copies", type=int, default=0,
                    help="cache copies rotated across steps (0: 4 when the decode working set is under 1 GiB)")
    ap.add_argument("--traffic-from", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "WORKLOAD"),
                    help="turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) of a bench run "
                         "with --calibrate-copy into profiles/traffic.json entries, then exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy, whose counters calibrate the byte counts")
    args = ap.parse_args(argv)
    if args.traffic_from:
        return write_traffic(*args.traffic_from)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        return 2
    import workloads
    w = workloads.WORKLOADS[args.workload]
    baseline = None
    if not args.no_cpu_baseline:
        # first: the oracle's workers are forked, which must happen before the GPU is touched
        log("timing the oracle on the host")
        baseline = cpu_baseline(w)
    if args.calibrate_copy:
        calibration_copy()
    r = run_gpu(w, args.steps, args.warmup, args.copies, keep_head=QUALITY_HEAD.get(w.name))
    ms = r["total_ms"] / args.steps
    cached = sum(r["lens"])
    value = cached / (ms / 1e3)
    dec_bytes = decode_algorithmic_bytes(w, r["lens"])
    app_bytes = append_algorithmic_bytes(w, r["app_counts"], r["app_lens_after"])
    calls = {"decode": dict(ms=r["dec_ms"], bytes=dec_bytes, src=SOURCES["decode"]),
             "append": dict(ms=r["app_ms"], bytes=app_bytes, src=SOURCES["append"])}
    dom = max(calls, key=lambda k: calls[k]["ms"])
    c = calls[dom]
    achieved = c["bytes"] / (c["ms"] / 1e3) / 1e9
    src_hash = source_hash(c["src"])
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(f"{dom}:{w.name}", src_hash),
                "kernel": KERNELS[dom],
                "algorithmic_bytes_per_launch": int(c["bytes"]), "avg_launch_ms": round(c["ms"], 5),
                "source_hash": src_hash}
    if dom == "append" and w.rotation == "dense":
        # the dense rotation's append is a GEMM on the matrix cores
        flops = dense_append_flops(w, r["app_counts"])
        tflops = flops / (c["ms"] / 1e3) / 1e12
        roofline.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_F16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
                         "algorithmic_flops_per_launch": int(flops),
                         "executed_frac": round(DENSE_SPLIT_PASSES * tflops / PEAK_MFMA_F16_TFLOPS, 4),
                         "hbm_achieved_GBs": round(achieved, 2)})
    other = [k for k in calls if k != dom][0]
    oc = calls[other]
    import kv_cache_vector_append_amd as tqa
    line = {
        "metric": "decode-attn cached tokens/s over TQ-packed KV; achieved HBM GB/s % of peak",
        "value": round(value, 1), "unit": "cached tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": w.name, "description": w.description, "decode_seqs": w.decode_seqs,
                   "decode_ctx": w.decode_ctx, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "key_bits": w.key_bits, "value_bits": w.value_bits,
                   "rotation": w.rotation, "window": w.window, "page_tokens": w.page_tokens},
        "roofline": roofline,
        "cache_copies": r["copies"],
        f"{other}_call": {"avg_launch_ms": round(oc["ms"], 5), "algorithmic_bytes_per_launch": int(oc["bytes"]),
                          "achieved_GBs": round(oc["bytes"] / (oc["ms"] / 1e3) / 1e9, 2)},
        "library_build_id": tqa.build_id(),
    }
    # (not in counter runs: its logit dump would be counted as the last decode's traffic)
    if w.name in QUALITY_HEAD and not args.calibrate_copy:
        line["quality_vs_exact"] = quality_vs_exact(w, r["setup"])
    del r
    if not args.calibrate_copy:
        ref = hbm_reference()
        dec_rate = calls["decode"]["bytes"] / (calls["decode"]["ms"] / 1e3) / 1e9
        ref["decode_frac_of_read"] = round(dec_rate / ref["read_GBs"], 4)
        ref["decode_frac_of_read_write"] = round(dec_rate / ref["read_write_GBs"], 4)
        line["hbm_reference"] = ref
    if not args.no_extra:
        import torch
        extra = {}
        for name in EXTRA_WORKLOADS:
            if name == w.name:
                continue
            torch.cuda.empty_cache()
            ew = workloads.WORKLOADS[name]
            er = run_gpu(ew, 10, args.warmup, 0, keep_head=QUALITY_HEAD.get(name))
            extra[name] = step_summary(ew, er, 10)
            extra[name]["format"] = {"key_mode": ew.key_mode, "key_bits": [ew.key_bits, ew.key_bits_hi or ew.key_bits],
                                     "value_mode": ew.value_mode,
                                     "value_bits": [ew.value_bits, ew.value_bits_hi or ew.value_bits],
                                     "key_outliers": ew.key_outliers, "rotation": ew.rotation}
            if name in QUALITY_HEAD:
                extra[name]["quality_vs_exact"] = quality_vs_exact(ew, er["setup"])
            del er
        line["other_workloads"] = extra
    if baseline is not None:
        line["cpu_baseline"] = baseline
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
