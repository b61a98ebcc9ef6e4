"""GPU parity of the prefill-chunk attention (kvq_attn_prefill) against the oracle's prefix
attention: the n_q newest tokens of each sequence are the queries, query i at position
len - n_q + i sees tokens 0 .. len - n_q + i of the cache as it stands.

Bar: 2e-3 relative L2 and 1e-2 max-abs per (sequence, query token) output [Hq x 128].
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from kvq_testlib import MAX_ABS_TOL, REL_L2_TOL, Case, max_abs, rel_l2

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run(wl, n0, B, nb, ne, n_q, seed=0, workspace="auto"):
    """Every sequence gets n0 tokens; the first nb of them ne more in a second call (ragged
    lengths); then n_q queries per sequence over the cache as it stands."""
    case = Case(wl, n0, layers=[0], batch=B, max_context=n0 + ne)
    case.prefill(0)
    streams = {b: [x[b].float().cpu().numpy() for x in case.kv(0)] for b in range(B)}
    if nb:
        k = W.gen_kv(wl, 900 + seed, 0, ne, batch=nb)
        v = W.gen_kv(wl, 900 + seed, 1, ne, batch=nb)
        case.cache.prefill_quantize(0, k.to("cuda"), v.to("cuda"))
        for b in range(nb):
            streams[b][0] = np.concatenate([streams[b][0], k[b].float().numpy()])
            streams[b][1] = np.concatenate([streams[b][1], v[b].float().numpy()])
    g = torch.Generator().manual_seed(1234 + seed)
    q = torch.randn((B, n_q, wl.n_q_heads, 128), generator=g)
    if wl.dtype == "bf16":
        q = q.to(torch.bfloat16)
    out = torch.full((B, n_q, wl.n_q_heads, 128), float("nan"), device="cuda")
    ws = workspace
    if isinstance(ws, int):
        ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
    case.cache.attn_prefill(0, q.to("cuda"), out, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    qn = q.float().numpy()
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    cap = case.cache.cfg.max_context
    G = wl.group
    worst = (0.0, 0.0)
    for b in range(B):
        n = streams[b][0].shape[0]
        assert case.cache.length(0, b) == n
        planes = []
        for h in range(wl.n_kv_heads):
            row = []
            for tensor in (0, 1):
                scheme = wl.k_scheme if tensor == 0 else wl.v_scheme
                bits = wl.k_bits if tensor == 0 else wl.v_bits
                rot = (wl.rotate_k if tensor == 0 else wl.rotate_v) or W.is_turbo(scheme)
                sink = wl.sinkhorn_iters > 0 and not W.is_turbo(scheme)
                tb = case.oracle_tables(0, h, tensor, mu, theta)
                pl = oracle.Plane(scheme, bits, rot, sink, wl.window, tensor, cap)
                pl.append(streams[b][tensor][:, h], tb)
                row += [pl, tb]
            planes.append(row)
        for i in range(n_q):
            pos = n - n_q + i
            ref = np.zeros((wl.n_q_heads, 128))
            for h in range(wl.n_kv_heads):
                pk, tk, pv, tv = planes[h]
                ref[h * G:(h + 1) * G] = oracle.attention_prefix(pk, pv, tk, tv, qn[b, i, h * G:(h + 1) * G], pos + 1)
            r, m = rel_l2(got[b, i], ref), max_abs(got[b, i], ref)
            worst = (max(worst[0], r), max(worst[1], m))
            assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (b, i, pos, r, m)
    _say(f"  {wl.name} batch {B} n_q {n_q}: rel_l2 <= {worst[0]:.2e}, max_abs <= {worst[1]:.2e}")
    return case, got, q


@pytest.mark.parametrize("n_q", [1, 37, 130])
def test_prefill_attention_kvarn(n_q):
    _say("case: prefill attention, KVarN U4, n_q", n_q)
    _run(W.LLAMA3B_32K_KVARN, n0=220, B=2, nb=1, ne=40, n_q=n_q)


@pytest.mark.parametrize("wl", [W.DENSE27B_120K_U8, W.DENSE27B_120K_KVARN, W.DENSE27B_120K_Q8_0],
                         ids=lambda w: w.name)
def test_prefill_attention_dense27b_gqa5_bf16(wl):
    _say("case: prefill attention,", wl.name)
    _run(wl, n0=150, B=3, nb=2, ne=33, n_q=70, seed=1)


@pytest.mark.parametrize("wl", [W.LLAMA3B_32K_TURBO_ASYM, W.LLAMA3B_32K_Q8_0_TURBO_V, W.LLAMA3B_32K_Q8_0_TURBO4_V,
                                W.LLAMA3B_32K_TURBO_ASYM.with_(name="llama3b-u4-k-turbomse-v", k_bits=4),
                                W.LLAMA8B_32K_Q8_0_TURBO25_V, W.LLAMA8B_32K_Q8_0_TURBO35_V],
                         ids=lambda w: w.name)
def test_prefill_attention_turbo_mse_v(wl):
    # TurboQuant-MSE values (3- and 4-bit codes, and the outlier split at 2.5 / 3.5 bits; rotated
    # domain, inverse rotation and un-permutation at the end) under uniform or q8_0 keys: the
    # cache types of the application rule K = Q8, V = Turbo
    _say("case: prefill attention,", wl.name)
    _run(wl, n0=300, B=2, nb=1, ne=37, n_q=90, seed=5)


@pytest.mark.parametrize("wl", [W.LLAMA3B_32K_Q8_0_TURBO4_V, W.LLAMA8B_32K_Q8_0_TURBO25_V], ids=lambda w: w.name)
def test_prefill_attention_turbo_v_key_splits(wl):
    # a long context, so that the keys are split over workgroups and the merge un-rotates V
    _say("case: prefill attention with key splits,", wl.name)
    case, _, _ = _run(wl, n0=3000, B=1, nb=0, ne=0, n_q=64, seed=6)
    assert case.cache.attn_prefill_workspace(0, 64, 1) > 0


@pytest.mark.parametrize("n0,nb,ne,n_q", [(500, 1, 37, 150), (90, 0, 0, 40), (64, 1, 100, 60)])
def test_prefill_attention_progressive_window(n0, nb, ne, n_q):
    # quantcpp's progressive cache (4-bit codes, newest 128 tokens in FP32): a query sees the
    # window tokens of the cache as it stands with their original values, older ones from the
    # codes; queries on both sides of the window start, whole caches inside the window, and a
    # ragged batch whose sequences have different window starts
    wl = W.LLAMA3B_3970_PROGRESSIVE
    _say("case: prefill attention, progressive window, n0", n0, "n_q", n_q)
    _run(wl, n0=n0, B=2, nb=nb, ne=ne, n_q=n_q, seed=7)


def test_prefill_attention_progressive_128k_shape_key_splits():
    wl = W.LLAMA3B_128K_PROGRESSIVE
    _say("case: prefill attention,", wl.name, "3000 tokens, key splits")
    case, _, _ = _run(wl, n0=3000, B=1, nb=0, ne=0, n_q=64, seed=8)
    assert case.cache.attn_prefill_workspace(0, 64, 1) > 0


def test_prefill_attention_asym_bits_and_long_chunk():
    # 8-bit K with 4-bit V (uniform, no rotation), a chunk longer than the two-tile boundary
    wl = W.LLAMA3B_3970_PROGRESSIVE.with_(window=0, k_bits=8)
    _say("case: prefill attention, U8 K / U4 V, n_q 200")
    _run(wl, n0=520, B=1, nb=0, ne=0, n_q=200, seed=2)


@pytest.mark.parametrize("ws", ["auto", None, 16], ids=["auto", "cache-workspace", "one-split"])
def test_prefill_attention_split_plans(ws):
    # the caller's workspace (several key splits + merge), the cache's own, and one too small for
    # any partials (the attention kernel finishes the rows itself) all meet the oracle
    wl = W.LLAMA3B_32K_KVARN
    _say("case: prefill attention split plan", ws)
    case, got, q = _run(wl, n0=4000, B=1, nb=0, ne=0, n_q=64, seed=4, workspace=ws)
    need = case.cache.attn_prefill_workspace(0, 64, 1)
    _say("  workspace bytes for the fastest plan:", need)
    assert need > 0  # 192 rows per kv head over 63 key chunks: key splits fill the chip


def test_prefill_attention_last_token_equals_decode():
    wl = W.LLAMA3B_32K_KVARN
    case, got, q = _run(wl, n0=333, B=1, nb=0, ne=0, n_q=1, seed=3)
    out = torch.empty((1, wl.n_q_heads, 128), device="cuda")
    case.cache.attn_decode(0, q[:, 0].contiguous().to("cuda"), out)
    torch.cuda.synchronize()
    assert rel_l2(got[0, 0], out.cpu().numpy()[0]) <= REL_L2_TOL


def test_prefill_attention_refusals():
    import quantized_decode_attention_kvq_amd as K
    # n_q beyond a length; a caller workspace smaller than the window copy that a progressive
    # cache beside rotated and balanced codes needs (nothing is written in either case)
    for wl, n, nq, ws, name in ((W.LLAMA3B_32K_KVARN, 200, 201, None, "KVQ_ERR_INVALID_ARG"),
                                (W.LLAMA3B_32K_KVARN.with_(window=128), 200, 10, 16, "KVQ_ERR_BUFFER_TOO_SMALL")):
        case = Case(wl, n, layers=[0], batch=1)
        case.prefill(0)
        q = torch.zeros((1, nq, wl.n_q_heads, 128), device="cuda")
        out = torch.full((1, nq, wl.n_q_heads, 128), 5.0, device="cuda")
        wst = None if ws is None else torch.empty(ws, dtype=torch.uint8, device="cuda")
        with pytest.raises(K.KvqError) as e:
            case.cache.attn_prefill(0, q, out, workspace=wst)
        assert e.value.name == name
        torch.cuda.synchronize()
        assert bool((out == 5.0).all())


QJL = W.LLAMA3B_32K_TURBO


@pytest.mark.parametrize("wl", [QJL, QJL.with_(name="llama3b-turboqjl-k-u8-v", v_bits=8),
                                QJL.with_(name="llama3b-turboqjl-k-u3-v", v_bits=3),
                                QJL.with_(name="llama3b-turboqjl-k-turbomse-v", v_scheme=W.TURBO_MSE, v_bits=3,
                                          rotate_v=True),
                                QJL.with_(name="llama3b-turboqjl-k-turbo4mse-v", v_scheme=W.TURBO_MSE, v_bits=4,
                                          rotate_v=True),
                                W.LLAMA8B_32K_Q8_0_TURBO25_V.with_(name="llama8b-turboqjl-k-turbo2.5split-v",
                                                                   k_scheme=W.TURBO_QJL, k_bits=3)],
                         ids=lambda w: w.name)
def test_prefill_attention_turbo_qjl_keys(wl):
    # TurboQuant-QJL keys (3-bit Lloyd-Max codes + 1-bit QJL of the residual): the score is the
    # oracle's n <R q, mu[code]> + gamma sqrt(pi/2) / 128 sum_i sign_i (S R q)_i, beside every
    # value kind (uniform 4 / 8 / 3 bits, TurboQuant-MSE 3 / 4 bits, the 2.5-bit split)
    _say("case: prefill attention,", wl.name)
    _run(wl, n0=300, B=2, nb=1, ne=37, n_q=90, seed=12)


def test_prefill_attention_turbo_qjl_keys_splits():
    _say("case: prefill attention,", QJL.name, "3000 tokens, key splits")
    case, _, _ = _run(QJL, n0=3000, B=1, nb=0, ne=0, n_q=64, seed=13)
    assert case.cache.attn_prefill_workspace(0, 64, 1) > 0


PROG = 128  # the quantcpp progressive window


@pytest.mark.parametrize("wl", [
    W.LLAMA3B_32K_KVARN.with_(name="llama3b-wht-sinkhorn-u4-progressive", window=PROG),
    W.LLAMA3B_3970_PROGRESSIVE.with_(name="llama3b-wht-k-u4-progressive", rotate_k=True),
    QJL.with_(name="llama3b-turboqjl-k-u4-v-progressive", window=PROG),
    W.LLAMA3B_32K_Q8_0_TURBO_V.with_(name="llama3b-q8_0-k-turbomse-v-progressive", window=PROG),
    W.LLAMA3B_32K_Q8_0_TURBO4_V.with_(name="llama3b-q8_0-k-turbo4mse-v-progressive", window=PROG),
    W.LLAMA8B_32K_Q8_0_TURBO35_V.with_(name="llama8b-q8_0-k-turbo3.5split-v-progressive", window=PROG),
    W.LLAMA3B_32K_KVARN_U3.with_(name="llama3b-wht-sinkhorn-u3-progressive", window=PROG),
    QJL.with_(name="llama3b-turboqjl-k-turbomse-v-progressive", v_scheme=W.TURBO_MSE, v_bits=3, rotate_v=True,
              window=PROG),
    W.DENSE27B_120K_KVARN.with_(name="dense27b-wht-sinkhorn-u4-progressive", window=PROG)],
    ids=lambda w: w.name)
def test_prefill_attention_window_in_code_domain(wl):
    # an FP32 window beside rotated, balanced or TurboQuant codes: the window tokens' originals
    # are mapped into their codes' domain (R(x) ./ c, R(x), the split's permuted 64-point
    # rotations) and meet the oracle, which reads them as they are; queries on both sides of the
    # window start, a ragged batch with different window starts
    _say("case: prefill attention, window in the code domain,", wl.name)
    _run(wl, n0=500, B=2, nb=1, ne=37, n_q=150, seed=14)


@pytest.mark.parametrize("n0,nb,ne,n_q,ws", [(90, 0, 0, 40, "auto"), (64, 1, 100, 60, None),
                                              (3000, 0, 0, 64, "auto"), (3000, 0, 0, 64, None)],
                         ids=["inside-window", "ragged-cache-workspace", "key-splits", "key-splits-cache-workspace"])
def test_prefill_attention_window_in_code_domain_edges(n0, nb, ne, n_q, ws):
    # whole caches inside the window, a ragged batch on the cache's own workspace (window copy
    # ahead of the partials there), and long caches whose keys are split over workgroups
    wl = W.LLAMA3B_32K_KVARN.with_(name="llama3b-wht-sinkhorn-u4-progressive", window=PROG)
    _say("case: prefill attention, KVarN progressive, n0", n0, "n_q", n_q, "workspace", ws)
    case, _, _ = _run(wl, n0=n0, B=2 if nb else 1, nb=nb, ne=ne, n_q=n_q, seed=15, workspace=ws)
    assert case.cache.attn_prefill_workspace(0, n_q, 1) >= 8 * 2 * 128 * 128 * 4


@pytest.mark.parametrize("wl", [W.LLAMA3B_32K_U8_K_U3_V, W.LLAMA3B_32K_KVARN_U3,
                                W.DENSE27B_120K_KVARN.with_(name="dense27b-wht-sinkhorn-u3", k_bits=3, v_bits=3),
                                W.LLAMA3B_32K_KVARN_U3.with_(name="llama3b-kvarn-u3-k-u4-v", v_bits=4),
                                W.LLAMA3B_32K_TURBO_ASYM.with_(name="llama3b-u3-k-turbomse-v", k_bits=3)],
                         ids=lambda w: w.name)
def test_prefill_attention_uniform3(wl):
    # 3-bit uniform keys and / or values (bit planes, fp16 scale and zero per 32 channels)
    _say("case: prefill attention,", wl.name)
    _run(wl, n0=300, B=2, nb=1, ne=37, n_q=90, seed=9)


def test_prefill_attention_uniform3_window_and_key_splits():
    # a progressive 3-bit cache (window tokens overwrite 3-bit values dequantized by the value
    # units), and a long 3-bit KVarN cache whose keys are split over workgroups
    wl = W.LLAMA3B_3970_PROGRESSIVE.with_(name="llama3b-u3-progressive", k_bits=3, v_bits=3)
    _say("case: prefill attention,", wl.name)
    _run(wl, n0=500, B=2, nb=1, ne=37, n_q=150, seed=10)
    case, _, _ = _run(W.LLAMA3B_32K_KVARN_U3, n0=3000, B=1, nb=0, ne=0, n_q=64, seed=11)
    assert case.cache.attn_prefill_workspace(0, 64, 1) > 0


@pytest.mark.parametrize("wl", [W.LLAMA3B_32K_KVARN.with_(name="llama3b-wht-sinkhorn-u4-f16", dtype="f16"),
                                QJL.with_(name="llama3b-turboqjl-k-u4-v-progressive-f16", dtype="f16", window=PROG)],
                         ids=lambda w: w.name)
def test_prefill_attention_f16_inputs(wl):
    # KVQ_F16 queries (and cache sources): widened exactly on load
    _say("case: prefill attention,", wl.name)
    _run(wl, n0=300, B=2, nb=1, ne=37, n_q=90, seed=16)


@pytest.mark.parametrize("wl", [W.LLAMA8B_32K_TURBO25_KV, W.LLAMA8B_32K_TURBO35_KV,
                                W.LLAMA8B_32K_TURBO25_KV.with_(name="llama8b-turbo2.5split-k-u4-v", v_scheme=W.UNIFORM,
                                                               v_bits=4, rotate_v=False),
                                W.LLAMA8B_32K_TURBO35_KV.with_(name="llama8b-turbo3.5split-kv-progressive", window=PROG)],
                         ids=lambda w: w.name)
def test_prefill_attention_split_keys(wl):
    # keys at 2.5 / 3.5 bits: the unit's half picks its norm, code width and codebook, the QJL
    # term as for TurboQuant keys; q' is the split domain of q; window tokens mapped the same way
    _say("case: prefill attention,", wl.name)
    _run(wl, n0=300, B=2, nb=1, ne=37, n_q=90, seed=17)
