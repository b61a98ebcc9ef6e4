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


@pytest.mark.parametrize("wl", [W.LLAMA8B_32K_TURBO25_KV, W.LLAMA8B_32K_TURBO35_KV], ids=lambda w: w.name)
def test_fullsize_llama8b_32k_turbo_split_kv(wl):
    _run(wl, layers=[0, 31], seqs=[0], plane_heads=[0, 4, 7], attn_heads=[0, 4, 7])


def _fused_steps(wl, layers, seqs, heads, batch=None):
    """kvq_append_attn_decode, the call bench.py times, at the workload's full context: one step
    on the matrix-core path (the automatic choice, with the automatic split plan) and one on the
    vector-ALU path, each checked against the oracle: the planes (the appended token's codes,
    scales and window slot included) bit-exact and the output of every query head of the sampled
    kv heads within tolerance."""
    B = wl.batch if batch is None else batch
    _say(f"case: fused append+decode, {wl.name} full context {wl.context}, batch {B}, layers {layers}")
    case = Case(wl, wl.context, layers=layers, batch=B, gen_device="cuda", extra_tokens=2)
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    G = wl.group
    cap = case.cache.cfg.max_context
    for li, layer in enumerate(layers):
        case.prefill(li)
        src = case.kv(layer)
        orc = {}  # (b, h, tensor) -> (plane, tables), grown by one token per step
        for b in seqs:
            for h in heads:
                for tensor in (0, 1):
                    tb = case.oracle_tables(li, h, tensor, mu, theta)
                    scheme = wl.k_scheme if tensor == 0 else wl.v_scheme
                    bits = wl.k_bits if tensor == 0 else wl.v_bits
                    rot = (wl.rotate_k if tensor == 0 else wl.rotate_v) or W.is_turbo(scheme)
                    sink = wl.sinkhorn_iters > 0 and not W.is_turbo(scheme)
                    p = oracle.Plane(scheme, bits, rot, sink, wl.window, tensor, cap)
                    p.append(src[tensor][b, :, h].float().cpu().numpy(), tb)
                    orc[(b, h, tensor)] = (p, tb)
        case.inputs.clear()
        del src
        for s, path in enumerate((0, 1)):  # 0: automatic (matrix cores), 1: vector ALU
            case.cache.set_option(2, path)
            k, v = W.gen_step_kv(wl, layer, s, device="cuda", batch=B)
            q = W.gen_q(wl, layer, 1 + s, device="cuda", batch=B)
            out = torch.full((B, wl.n_q_heads, 128), float("nan"), device="cuda")
            case.cache.append_attn_decode(li, k, v, q, out)
            torch.cuda.synchronize()
            assert case.cache.length(li, 0) == wl.context + 1 + s
            got = out.cpu().numpy()
            assert np.isfinite(got).all()
            kn, vn, qn = k.float().cpu().numpy(), v.float().cpu().numpy(), q.float().cpu().numpy()
            worst = (0.0, 0.0)
            for b in seqs:
                for h in heads:
                    for tensor, x in ((0, kn), (1, vn)):
                        p, tb = orc[(b, h, tensor)]
                        p.append(x[b, h], tb)
                        compare_plane(case.device_plane(li, b, h, tensor), p,
                                      f"layer {layer} seq {b} head {h} tensor {tensor} path {path}")
                    pk, tk = orc[(b, h, 0)]
                    pv, tv = orc[(b, h, 1)]
                    ref = oracle.attention(pk, pv, tk, tv, qn[b, h * G:(h + 1) * G])
                    blk = got[b, h * G:(h + 1) * G]
                    r, m = rel_l2(blk, ref), max_abs(blk, ref)
                    worst = (max(worst[0], r), max(worst[1], m))
                    assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (layer, path, b, h, r, m)
            _say(f"  layer {layer} path {path} n={wl.context + 1 + s}: planes bit-exact, attention "
                 f"rel_l2<={worst[0]:.2e} max_abs<={worst[1]:.2e}")
        case.cache.set_option(2, 0)
        torch.cuda.empty_cache()


def test_fullsize_fused_llama3b_32k_kvarn():
    # the benchmarked workload and call: 32K WHT + Sinkhorn U4, first and last layer
    _fused_steps(W.LLAMA3B_32K_KVARN, layers=[0, 27], seqs=[0], heads=ALL8)


def test_fullsize_fused_llama3b_128k_progressive_b1():
    # 128K progressive: the new token lands in the FP32 window, owned by the window workgroup
    _fused_steps(W.LLAMA3B_128K_PROGRESSIVE, layers=[0, 27], seqs=[0], heads=[0, 3, 7])


@pytest.mark.parametrize("wl", [W.LLAMA3B_32K_U8_K_U3_V, W.LLAMA3B_32K_KVARN_U3], ids=lambda w: w.name)
def test_fullsize_llama3b_32k_uniform3(wl):
    # 3-bit uniform group packing at full size: V only (K 8-bit), and K and V behind WHT + Sinkhorn
    _run(wl, layers=[0, 27], seqs=[0], plane_heads=[0, 4, 7], attn_heads=[0, 4, 7])
