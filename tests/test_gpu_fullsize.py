"""GPU parity at the full sizes of the benchmarked workloads, in bench.py's launch configuration.

Each case builds the cache at the workload's full context and batch, with bulk prefill of every
token. It uses the automatic decode path and split planning, as bench.py does. Inputs are
generated on the device by the seeded generators and copied back for the oracle. The oracle then:

- rebuilds the planes of sampled (layer, sequence, kv head) from those inputs;
- checks them bit-exact against the device bytes;
- computes fp64 attention for sampled kv heads (all their query heads).

The bar is 2e-3 relative L2 and 1e-2 max-abs per sampled block of the output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from kvq_testlib import MAX_ABS_TOL, REL_L2_TOL, Case, compare_plane, max_abs, rel_l2

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run(wl, layers, seqs, plane_heads, attn_heads, batch=None):
    B = wl.batch if batch is None else batch
    _say(f"case: {wl.name} full context {wl.context}, batch {B}, layers {layers}")
    case = Case(wl, wl.context, layers=layers, batch=B, gen_device="cuda")
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    G = wl.group
    for li, layer in enumerate(layers):
        case.prefill(li)
        q = W.gen_q(wl, layer, 0, device="cuda", batch=B)
        out = torch.full((B, wl.n_q_heads, 128), float("nan"), device="cuda")
        case.cache.attn_decode(li, q, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        qn = q.float().cpu().numpy()
        for b in seqs:
            worst = (0.0, 0.0)
            for h in sorted(set(plane_heads) | set(attn_heads)):
                row = []
                for tensor in (0, 1):
                    tb = case.oracle_tables(li, h, tensor, mu, theta)
                    p, _ = case.oracle_plane(li, b, h, tensor, tb)
                    if h in plane_heads:
                        compare_plane(case.device_plane(li, b, h, tensor), p,
                                      f"layer {layer} seq {b} head {h} tensor {tensor}")
                    row += [p, tb]
                if h in attn_heads:
                    ref = oracle.attention(row[0], row[2], row[1], row[3], qn[b, h * G:(h + 1) * G])
                    blk = got[b, h * G:(h + 1) * G]
                    r, m = rel_l2(blk, ref), max_abs(blk, ref)
                    worst = (max(worst[0], r), max(worst[1], m))
                    assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (layer, b, h, r, m)
            _say(f"  layer {layer} seq {b}: planes bit-exact for heads {plane_heads}; attention "
                 f"heads {attn_heads} rel_l2<={worst[0]:.2e} max_abs<={worst[1]:.2e}")
        del out
        case.inputs.clear()
        torch.cuda.empty_cache()


ALL8 = list(range(8))


def test_fullsize_llama3b_32k_kvarn():
    _run(W.LLAMA3B_32K_KVARN, layers=[0, 27], seqs=[0], plane_heads=ALL8, attn_heads=ALL8)


def test_fullsize_llama3b_32k_turbo_qjl():
    _run(W.LLAMA3B_32K_TURBO, layers=[0, 27], seqs=[0], plane_heads=[0, 4, 7], attn_heads=[0, 4, 7])


def test_fullsize_llama3b_32k_turbo_asym():
    _run(W.LLAMA3B_32K_TURBO_ASYM, layers=[0, 27], seqs=[0], plane_heads=[0, 4, 7],
         attn_heads=[0, 4, 7])


def test_fullsize_llama3b_128k_progressive_b1():
    _run(W.LLAMA3B_128K_PROGRESSIVE, layers=[0, 27], seqs=[0], plane_heads=ALL8,
         attn_heads=[0, 3, 7])


def test_fullsize_llama3b_128k_progressive_b8():
    _run(W.LLAMA3B_128K_PROGRESSIVE, layers=[0], seqs=[0, 7], plane_heads=[0, 7], attn_heads=[0, 7],
         batch=8)


@pytest.mark.parametrize("wl", [W.DENSE27B_120K_KVARN, W.DENSE27B_120K_U8], ids=lambda w: w.name)
def test_fullsize_dense27b_120k_b4(wl):
    _run(wl, layers=[0, 63], seqs=[0, 3], plane_heads=[0, 7], attn_heads=[0, 7])


@pytest.mark.parametrize("wl", [W.LLAMA8B_32K_Q8_0_TURBO25_V, W.LLAMA8B_32K_Q8_0_TURBO35_V],
                         ids=lambda w: w.name)
def test_fullsize_llama8b_32k_turbo_split_v(wl):
    _run(wl, layers=[0, 31], seqs=[0], plane_heads=[0, 4, 7], attn_heads=[0, 4, 7])
