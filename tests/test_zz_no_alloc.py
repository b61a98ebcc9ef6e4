"""kvq_attn_decode_static (the entry point that allocates nothing: split partials in the
library's static device scratch) against kvq_attn_decode, through the C ABI.

Two calls in a row, the second with a smaller input (fewer sequences and a shorter cache), each
checked against the existing entry point on the same cache and query; a call whose partials would
not fit the scratch is refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import workloads as W
from kvq_testlib import MAX_ABS_TOL, REL_L2_TOL, Case, max_abs, rel_l2

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _compare(case, li, batch, label):
    wl = case.wl
    q = W.gen_q(wl, case.layers[li], 3, batch=batch).to("cuda")
    ref = torch.full((batch, wl.n_q_heads, 128), float("nan"), device="cuda")
    got = torch.full_like(ref, float("nan"))
    case.cache.attn_decode(li, q, ref)
    case.cache.attn_decode_static(li, q, got)
    torch.cuda.synchronize()
    r, m = rel_l2(got.cpu().numpy(), ref.cpu().numpy()), max_abs(got.cpu().numpy(), ref.cpu().numpy())
    _say(f"  {label}: rel_l2={r:.2e} max_abs={m:.2e} bit-identical={torch.equal(got, ref)}")
    assert np.isfinite(got.cpu().numpy()).all()
    assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (label, r, m)
    assert torch.equal(got, ref), label  # same kernels and split plan: the same bits


def test_static_scratch_decode_two_calls_second_smaller():
    wl = W.DENSE27B_120K_KVARN  # 40 query heads, batch 4
    _say("case: static-scratch decode,", wl.name)
    case = Case(wl, 3000, layers=[0], batch=4)
    case.prefill(0)
    _compare(case, 0, 4, "call 1: batch 4, 3000 tokens")
    small = Case(W.LLAMA3B_32K_KVARN, 700, layers=[0], batch=1)
    small.prefill(0)
    _compare(small, 0, 1, "call 2: batch 1, 700 tokens")
    _compare(case, 0, 2, "call 3: batch 2 of the first cache")


def test_static_scratch_refuses_oversized_partials():
    import quantized_decode_attention_kvq_amd as K
    wl = W.LLAMA3B_32K_KVARN
    # 64 sequences x 24 query heads at 4096 tokens in splits of 64 tokens: 64 splits per
    # (sequence, kv head), 64 x 24 x 64 x 528 B = 51.9 MB of partials, beyond the 32 MiB scratch
    case = Case(wl, 4096, layers=[0], batch=64)
    case.prefill(0)
    case.cache.set_option(1, 64)
    q = W.gen_q(wl, 0, 0, batch=64).to("cuda")
    out = torch.full((64, wl.n_q_heads, 128), 5.0, device="cuda")
    with pytest.raises(K.KvqError) as e:
        case.cache.attn_decode_static(0, q, out)
    assert e.value.name == "KVQ_ERR_SCRATCH"
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
    case.cache.attn_decode(0, q, out)  # the cache's own workspace takes it
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
