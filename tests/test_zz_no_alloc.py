"""The decode entry point that allocates nothing: tq_decode_attention_static,
whose workspace is a library-owned device array, against tq_decode_attention
with a caller workspace, through the C ABI, on two calls in a row (the second
smaller), plus its size limit."""
import numpy as np
import pytest
import torch

import workloads
from harness import DECODE_TOL, decode_error, gpu_cache_as_oracle, gpu_decode, make_run, queries
from oracle import tq

pytestmark = pytest.mark.gpu


def _static_decode(run, q, lens, want_logits=False):
    import kv_cache_vector_append_amd as tqa
    dev = run.params.device
    nseq = q.shape[0]
    max_ctx = max(max(lens), 1)
    out = torch.full((nseq, run.w.num_q_heads, run.w.head_dim), float("nan"), dtype=torch.float32, device=dev)
    logits = torch.full((nseq, run.w.num_q_heads, max_ctx), float("nan"), device=dev) if want_logits else None
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    tqa.decode_attention_static(run.cfg, run.params, run.cache, q.to(dev).contiguous(), i32(list(range(nseq))),
                                i32(list(lens)), max_ctx, out, 0.0, logits)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), (logits.cpu().double().numpy() if want_logits else None)


@pytest.mark.parametrize("name", ["gqa_decode", "hd256_long_dense_4_4"])
def test_static_workspace_decode_matches_caller_workspace(name):
    w = workloads.WORKLOADS[name]
    lens = [700, 129, 1000, 333]
    print(f"[no-alloc] {name} lens={lens}", flush=True)
    run = make_run(w, lens, oracle_append=False)
    q = queries(w, len(lens))
    # first call: all four sequences, with the logits dump
    o_ref, lg_ref = gpu_decode(run, q, want_logits=True)
    o_st, lg_st = _static_decode(run, q, lens, want_logits=True)
    assert np.array_equal(o_st, o_ref)
    assert np.array_equal(np.nan_to_num(lg_st, nan=7.0), np.nan_to_num(lg_ref, nan=7.0))
    o_ora = tq.decode(run.P, gpu_cache_as_oracle(run), q.double().numpy(), np.arange(len(lens)), lens)
    assert decode_error(o_st, o_ora) <= DECODE_TOL
    # second call, smaller: two sequences over shorter prefixes of their contexts,
    # so a different split plan reuses the array the first call wrote
    small = [300, 64]
    o_ref2, _ = gpu_decode(run, q[:2], lens=small)
    o_st2, _ = _static_decode(run, q[:2], small)
    assert np.array_equal(o_st2, o_ref2)
    o_ora2 = tq.decode(run.P, gpu_cache_as_oracle(run), q[:2].double().numpy(), np.arange(2), small)
    assert decode_error(o_st2, o_ora2) <= DECODE_TOL
    print(f"[no-alloc] {name}: bit-identical to the caller-workspace call on both calls; "
          f"oracle err {decode_error(o_st, o_ora):.3g}, {decode_error(o_st2, o_ora2):.3g}", flush=True)


def test_static_workspace_rejects_calls_above_its_size():
    import kv_cache_vector_append_amd as tqa
    w = workloads.WORKLOADS["gqa_decode"]
    run = make_run(w, [100], oracle_append=False)
    nseq = 4096                      # far more records than the library-owned array holds
    assert tqa.decode_workspace_bytes(run.cfg, nseq, 65536) > tqa.TQ_STATIC_WORKSPACE_BYTES
    dev = run.params.device
    q = torch.zeros((nseq, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((nseq, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    i32 = torch.zeros(nseq, dtype=torch.int32, device=dev)
    with pytest.raises(tqa.TQError, match="TQ_ERR_CAPACITY"):
        tqa.decode_attention_static(run.cfg, run.params, run.cache, q, i32, i32, 65536, out)
