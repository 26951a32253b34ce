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
on; `cpu_baseline` times the float64 oracle on a bounded sample of the same
workload on the host.
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
    d = w.head_dim
    key = w.key_bits * d // 8 + 8          # (b-1) d/8 codes + d/8 QJL signs + nu + gamma
    value = w.value_bits * d // 8 + 4      # b d/8 codes + nu
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
    "decode": [_CSRC + f for f in ("tq_decode_mfma.hip", "tq_mfma.h", "tq_decode.hip", "tq_device.h",
                                   "tq_internal.h")],
    "append": [_CSRC + f for f in ("tq_append.hip", "tq_device.h", "tq_internal.h")],
}
KERNELS = {
    "decode": "tq_decode_attention (decode_prep + decode_split + decode_combine)",
    "append": "tq_quantize_append (append_tok_kernel, append_dense_kernel or append_kernel)",
}
# rocprofv3 kernel names of each call's kernels (an append launches one of the two)
KERNEL_MATCH = {"decode": (("decode_prep_kernel",), ("decode_split_kernel",), ("decode_combine_kernel",)),
                "append": (("append_tok_kernel", "append_dense_kernel", "append_kernel<"),)}
CALIBRATION_BYTES = 1 << 30


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
        if len(per_kernel) != len(groups) or not f_scale or not w_scale:
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


def build_decode_setup(w, tqa, torch, dev):
    """Cache filled with decode_ctx - 1 tokens per sequence; the step appends token
    decode_ctx - 1 of every sequence and decodes over decode_ctx tokens."""
    import workloads
    S = Setup()
    nseq, ctx = w.decode_seqs, w.decode_ctx
    mpp = w.pages_per_seq(ctx)
    S.cfg = tqa.Config(w.head_dim, w.num_q_heads, w.num_kv_heads, w.key_bits, w.value_bits, w.page_tokens,
                       w.window, w.rotation, w.method_seed)
    S.params = torch.empty(tqa.params_bytes(S.cfg), dtype=torch.uint8, device=dev)
    tqa.init_codebooks(S.cfg, S.params)
    bt = workloads.block_table(w, nseq, mpp)
    S.cache = tqa.allocate_cache(S.cfg, nseq * mpp, bt, dev)
    g = workloads.device_generator(w, 1, dev)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    slots = i32(list(range(nseq)))
    chunk = 16384
    for start in range(0, ctx - 1, chunk):
        n = min(chunk, ctx - 1 - start)
        k = workloads.device_kv(w, "k", nseq * n, g, dev)
        v = workloads.device_kv(w, "v", nseq * n, g, dev)
        tqa.quantize_append(S.cfg, S.params, S.cache, k, v, slots, i32([start] * nseq),
                            i32([i * n for i in range(nseq + 1)]), n)
        del k, v
    torch.cuda.synchronize()
    log(f"prefilled {nseq} x {ctx - 1} tokens")
    S.step_k = workloads.device_kv(w, "k", nseq, g, dev)
    S.step_v = workloads.device_kv(w, "v", nseq, g, dev)
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
    S.cfg = tqa.Config(w.head_dim, w.num_q_heads, w.num_kv_heads, w.key_bits, w.value_bits, w.page_tokens,
                       w.window, w.rotation, w.method_seed)
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


def run_gpu(w, steps, warmup, copies):
    import torch
    import kv_cache_vector_append_amd as tqa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S = build_mixed_setup(w, tqa, torch, dev) if w.prefill_seqs else build_decode_setup(w, tqa, torch, dev)
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
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
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
                app_lens_after=S.app_lens_after, copies=copies)


# ----------------------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(w, budget_s=20.0):
    """Time the float64 oracle (as it stands) on a bounded sample of the workload
    and scale to decoded cached tokens per second for the whole step."""
    import torch
    import workloads
    from oracle import tq
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    ocfg = tq.Config(w.head_dim, w.num_q_heads, w.num_kv_heads, w.key_bits, w.value_bits, w.page_tokens,
                     w.window, w.rotation, w.method_seed)
    P = tq.Params(ocfg)
    sample_ctx = min(w.decode_ctx, 8192)
    mpp = math.ceil(sample_ctx / w.page_tokens)
    cache = tq.Cache(ocfg, mpp, np.arange(mpp)[None])
    K = workloads.kv_tokens(w, "k", 0, 0, sample_ctx).double().numpy()
    V = workloads.kv_tokens(w, "v", 0, 0, sample_ctx).double().numpy()
    t = time.perf_counter()
    tq.append(P, cache, K, V, [0], [0], [0, sample_ctx])
    t_app = time.perf_counter() - t
    app_rate = sample_ctx / t_app                                  # tokens (all KV heads) per second
    q = workloads.queries(w, 0).double().numpy()[None]
    t = time.perf_counter()
    reps = 0
    while True:
        tq.decode(P, cache, q, [0], [sample_ctx])
        reps += 1
        if time.perf_counter() - t > min(budget_s / 2, 5.0) or reps >= 20:
            break
    t_dec = (time.perf_counter() - t) / reps
    dec_rate = sample_ctx / t_dec                                  # cached tokens (all heads) per second
    step_tokens = w.decode_seqs * w.decode_ctx
    appended = w.prefill_seqs * w.prefill_tokens if w.prefill_seqs else w.decode_seqs
    t_step = appended / app_rate + step_tokens / dec_rate
    return {"value": step_tokens / t_step, "unit": "cached tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle append of {sample_ctx} tokens x {w.num_kv_heads} KV heads ({t_app:.2f} s) and "
                      f"{reps} decodes of 1 sequence x {w.num_q_heads} query heads over {sample_ctx} tokens "
                      f"({t_dec:.2f} s each), scaled to {appended} appended tokens + {step_tokens} cached tokens "
                      f"per step"}


# ----------------------------------------------------------------------------- main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    if args.calibrate_copy:
        calibration_copy()
    r = run_gpu(w, args.steps, args.warmup, args.copies)
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
    line = {
        "metric": "decode-attn cached tokens/s over TQ-packed KV; achieved HBM GB/s % of peak",
        "value": round(value, 1), "unit": "cached tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": w.name, "description": w.description, "decode_seqs": w.decode_seqs,
                   "decode_ctx": w.decode_ctx, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "key_bits": w.key_bits, "value_bits": w.value_bits,
                   "rotation": w.rotation, "window": w.window, "page_tokens": w.page_tokens},
        "roofline": roofline,
        "cache_copies": r["copies"],
        f"{other}_call": {"avg_launch_ms": round(oc["ms"], 5), "algorithmic_bytes_per_launch": int(oc["bytes"]),
                          "achieved_GBs": round(oc["bytes"] / (oc["ms"] / 1e3) / 1e9, 2)},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
