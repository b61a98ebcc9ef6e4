"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: packed codes, fp16 scales/zeros, norms, QJL bits, window bytes and tables are bit-exact;
attention outputs are within 2e-3 relative L2 and 1e-2 max-abs of the oracle's fp64 attention on
the same dequantized cache.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from kvq_testlib import (MAX_ABS_TOL, REL_L2_TOL, Case, compare_plane, max_abs,
                         oracle_attention_case, rel_l2)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _check_all_planes(case, li, heads=None, seqs=None):
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    planes = {}
    for b in (seqs if seqs is not None else range(case.batch)):
        for h in (heads if heads is not None else range(case.wl.n_kv_heads)):
            row = []
            for tensor in (0, 1):
                tb = case.oracle_tables(li, h, tensor, mu, theta)
                p, _ = case.oracle_plane(li, b, h, tensor, tb)
                compare_plane(case.device_plane(li, b, h, tensor), p, f"layer {li} seq {b} head {h} tensor {tensor}")
                row += [p, tb]
            planes[(b, h)] = row
    return planes


def _paths(wl):
    return (1, 2)  # vector-ALU kernel, matrix-core kernel


def _decode_and_compare(case, li, planes=None, step=0, seqs=None):
    wl = case.wl
    q = W.gen_q(wl, case.layers[li], step, batch=case.batch).to(case.device)
    qn = q.float().cpu().numpy()
    refs = {}
    outs = {}
    for path in _paths(wl):
        case.cache.set_option(2, path)
        out = torch.full((case.batch, wl.n_q_heads, 128), float("nan"), dtype=torch.float32,
                         device=case.device)
        case.cache.attn_decode(li, q, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        worst = (0.0, 0.0)
        for b in (seqs if seqs is not None else range(case.batch)):
            if b not in refs:
                pl = None
                if planes is not None:
                    pl = {h: planes[(b, h)] for h in range(wl.n_kv_heads)}
                refs[b] = oracle_attention_case(case, li, b, qn[b], planes=pl)
            ref = refs[b]
            r, m = rel_l2(got[b], ref), max_abs(got[b], ref)
            worst = (max(worst[0], r), max(worst[1], m))
            assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (path, b, r, m)
        _say(f"  path {path}: attention rel_l2={worst[0]:.2e} max_abs={worst[1]:.2e}")
        outs[path] = got
    case.cache.set_option(2, 0)
    return outs[_paths(wl)[-1]]


def test_progressive_3970_full():
    wl = W.LLAMA3B_3970_PROGRESSIVE
    _say("case:", wl.name)
    case = Case(wl, wl.context)
    case.prefill(0)
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0)
    _decode_and_compare(case, 0, planes)


@pytest.mark.parametrize("wl", [W.LLAMA3B_3970_PROGRESSIVE, W.LLAMA3B_32K_TURBO, W.LLAMA3B_32K_TURBO_ASYM,
                                W.LLAMA3B_32K_Q8_0_TURBO_V, W.DENSE27B_120K_Q8_0, W.LLAMA3B_32K_Q8_0_TURBO4_V,
                                W.LLAMA8B_32K_Q8_0_TURBO25_V, W.LLAMA8B_32K_Q8_0_TURBO35_V,
                                W.LLAMA3B_32K_U8_K_U3_V, W.LLAMA3B_32K_KVARN_U3, W.LLAMA8B_32K_TURBO25_KV,
                                W.LLAMA8B_32K_TURBO35_KV],
                         ids=lambda w: w.name)
def test_prefill_equals_appends_bytewise(wl):
    _say("case: prefill == appends,", wl.name, "n=300")
    a = Case(wl, 300, layers=[0])
    b = Case(wl, 300, layers=[0])
    a.prefill(0, chunks=[1, 63, 100, 7, 129])
    b.append_all(0)
    torch.cuda.synchronize()
    for h in range(wl.n_kv_heads):
        for t in (0, 1):
            da, db = a.device_plane(0, 0, h, t), b.device_plane(0, 0, h, t)
            for x, y in zip(da, db):
                if x is not None:
                    assert np.array_equal(x, y), (h, t)
    _check_all_planes(a, 0, heads=[0, 5])


# (sequences, tokens) of successive prefill calls: ragged starts per sequence, partial octets at
# both ends of the bulk calls (>= 16 tokens) and single-octet calls below that
RAGGED_CALLS = [(3, 21), (1, 5), (2, 3), (3, 37), (1, 16), (3, 130)]


@pytest.mark.parametrize("wl", [W.LLAMA3B_3970_PROGRESSIVE, W.LLAMA3B_32K_KVARN, W.LLAMA3B_32K_TURBO,
                                W.LLAMA3B_32K_TURBO_ASYM, W.DENSE27B_120K_U8, W.DENSE27B_120K_Q8_0,
                                W.LLAMA3B_32K_Q8_0_TURBO_V, W.LLAMA3B_32K_Q8_0_TURBO4_V,
                                W.LLAMA8B_32K_Q8_0_TURBO25_V, W.LLAMA8B_32K_Q8_0_TURBO35_V,
                                W.LLAMA3B_32K_U8_K_U3_V, W.LLAMA3B_32K_KVARN_U3, W.LLAMA8B_32K_TURBO35_KV],
                         ids=lambda w: w.name)
def test_prefill_ragged_batch_bytewise(wl):
    """Prefill calls over a batch whose sequences start at different lengths leave exactly the
    bytes the oracle builds from each sequence's own token stream."""
    n_max = sum(t for _, t in RAGGED_CALLS)
    _say("case: ragged-batch prefill,", wl.name, RAGGED_CALLS)
    case = Case(wl, n_max, layers=[0], batch=3)
    streams = {b: ([], []) for b in range(3)}
    for ci, (nb, nt) in enumerate(RAGGED_CALLS):
        k = W.gen_kv(wl, 1000 + ci, 0, nt, batch=nb)
        v = W.gen_kv(wl, 1000 + ci, 1, nt, batch=nb)
        case.cache.prefill_quantize(0, k.to("cuda"), v.to("cuda"))
        for b in range(nb):
            streams[b][0].append(k[b].float().numpy())
            streams[b][1].append(v[b].float().numpy())
    torch.cuda.synchronize()
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    cap = case.cache.cfg.max_context
    for b in range(3):
        assert case.cache.length(0, b) == sum(x.shape[0] for x in streams[b][0])
        for h in range(wl.n_kv_heads):
            for tensor in (0, 1):
                X = np.concatenate(streams[b][tensor])[:, h]
                scheme = wl.k_scheme if tensor == 0 else wl.v_scheme
                bits = wl.k_bits if tensor == 0 else wl.v_bits
                rot = (wl.rotate_k if tensor == 0 else wl.rotate_v) or W.is_turbo(scheme)
                sink = wl.sinkhorn_iters > 0 and not W.is_turbo(scheme)
                tb = case.oracle_tables(0, h, tensor, mu, theta)
                pl = oracle.Plane(scheme, bits, rot, sink, wl.window, tensor, cap)
                pl.append(X, tb)
                compare_plane(case.device_plane(0, b, h, tensor), pl, f"seq {b} head {h} tensor {tensor}")
    _say("  planes bit-exact for 3 sequences x", wl.n_kv_heads, "heads")


def test_kvarn_rotation_sinkhorn_small():
    wl = W.LLAMA3B_32K_KVARN
    _say("case:", wl.name, "2 layers, 1000 tokens")
    case = Case(wl, 1000, layers=[0, 13])
    for li in range(2):
        case.prefill(li)
    torch.cuda.synchronize()
    # Sinkhorn tables bit-exact
    for li, layer in enumerate(case.layers):
        c_dev = case.cache.table("c", 2 * 8 * 2 * 128).cpu().numpy().reshape(2, 8, 2, 128)
        ic_dev = case.cache.table("inv_c", 2 * 8 * 2 * 128).cpu().numpy().reshape(2, 8, 2, 128)
        for h in range(8):
            for t in (0, 1):
                tb = case.oracle_tables(li, h, t)
                assert np.array_equal(c_dev[li, h, t].view(np.uint32), tb.arrays["c"].view(np.uint32)), (li, h, t)
                assert np.array_equal(ic_dev[li, h, t].view(np.uint32), tb.arrays["inv_c"].view(np.uint32))
    for li in range(2):
        planes = _check_all_planes(case, li)
        _decode_and_compare(case, li, planes)


def test_turbo_qjl_small():
    wl = W.LLAMA3B_32K_TURBO
    _say("case:", wl.name, "1 layer, 700 tokens")
    case = Case(wl, 700, layers=[3])
    case.prefill(0)
    torch.cuda.synchronize()
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    mu_dev = case.cache.table("mu", 8).cpu().numpy()
    th_dev = case.cache.table("theta", 7).cpu().numpy()
    assert np.array_equal(mu_dev.view(np.uint32), mu.view(np.uint32))
    assert np.array_equal(th_dev.view(np.uint32), theta.view(np.uint32))
    planes = _check_all_planes(case, 0)
    _decode_and_compare(case, 0, planes)


def test_turbo_asym_u8k_msev_small():
    wl = W.LLAMA3B_32K_TURBO_ASYM
    _say("case:", wl.name, "1 layer, 777 tokens")
    case = Case(wl, 777, layers=[5])
    case.prefill(0)
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0)
    _decode_and_compare(case, 0, planes)


def test_q8_0_k_turbo4_mse_v_small():
    # the application rule K = Q8, V = TurboQuant 4-bit: the device's 16-level codebook equals the
    # oracle's bit for bit, the planes byte for byte (appends and a bulk prefill), and attention
    wl = W.LLAMA3B_32K_Q8_0_TURBO4_V
    _say("case:", wl.name, "1 layer, 300 prefill + 40 appends")
    case = Case(wl, 340, layers=[1])
    k, v = case.kv(1)
    case.cache.prefill_quantize(0, k[:, :300].contiguous(), v[:, :300].contiguous())
    for t in range(300, 340):
        case.cache.append(0, k[:, t].contiguous(), v[:, t].contiguous())
    torch.cuda.synchronize()
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS, 16)
    assert np.array_equal(case.cache.table("mu16", 16).cpu().numpy().view(np.uint32), mu.view(np.uint32))
    assert np.array_equal(case.cache.table("theta16", 15).cpu().numpy().view(np.uint32), theta.view(np.uint32))
    planes = _check_all_planes(case, 0)
    _decode_and_compare(case, 0, planes)  # both decode paths


@pytest.mark.parametrize("wl", [W.LLAMA8B_32K_Q8_0_TURBO25_V, W.LLAMA8B_32K_Q8_0_TURBO35_V],
                         ids=lambda w: w.name)
def test_turbo_split_v_small(wl):
    # TurboQuant's fractional bit widths (outlier-channel split): the device's outlier choice per
    # kv head equals the oracle's from the same calibration block, its N(0, 1/64) codebooks equal
    # the oracle's bit for bit, the planes byte for byte (bulk prefill and appends), and attention
    _say("case:", wl.name, "2 layers, 300 prefill + 45 appends")
    case = Case(wl, 345, layers=[0, 7])
    for li, layer in enumerate(case.layers):
        k, v = case.kv(layer)
        case.cache.prefill_quantize(li, k[:, :300].contiguous(), v[:, :300].contiguous())
        for t in range(300, 345):
            case.cache.append(li, k[:, t].contiguous(), v[:, t].contiguous())
    torch.cuda.synchronize()
    perm = case.cache.table("perm", 2 * 8 * 128).cpu().numpy().reshape(2, 8, 128)
    for li, layer in enumerate(case.layers):
        for h in range(8):
            ref = oracle.select_outliers(case.calib[layer][1][:, h, :])
            assert np.array_equal(perm[li, h], ref), (li, h)
    mu64 = case.cache.table("mu64", 28).cpu().numpy()
    th64 = case.cache.table("theta64", 28).cpu().numpy()
    for levels in (4, 8, 16):
        _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS, levels, 64)
        o = levels - 4
        assert np.array_equal(mu64[o:o + levels].view(np.uint32), mu.view(np.uint32)), levels
        assert np.array_equal(th64[o:o + levels - 1].view(np.uint32), theta.view(np.uint32)), levels
    for li in range(2):
        planes = _check_all_planes(case, li)
        _decode_and_compare(case, li, planes)  # both decode paths


def test_turbo_split_v_bf16_window_batch():
    # bf16 sources (calibration included), two sequences, and the progressive FP32 window beside a
    # split V: planes and rings byte-exact, decode (window tokens in FP32) against the oracle
    wl = W.LLAMA8B_32K_Q8_0_TURBO35_V.with_(name="llama8b-split3.5-bf16-window", dtype="bf16", window=128)
    _say("case:", wl.name, "1 layer, 2 seqs, 250 prefill + 50 appends")
    case = Case(wl, 300, layers=[3], batch=2)
    k, v = case.kv(3)
    case.cache.prefill_quantize(0, k[:, :250].contiguous(), v[:, :250].contiguous())
    for t in range(250, 300):
        case.cache.append(0, k[:, t].contiguous(), v[:, t].contiguous())
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0, heads=[0, 3, 7])
    _decode_and_compare(case, 0, None)


def test_turbo_split_v_requires_calibration():
    # appending to a split V before kvq_calibrate has chosen its outlier channels is refused
    wl = W.LLAMA8B_32K_Q8_0_TURBO25_V
    import quantized_decode_attention_kvq_amd as K
    cache = K.KvCache(device="cuda", **wl.kvq_config(max_context=128))
    cache.set_random_tables(torch.from_numpy(np.ascontiguousarray(W.rotation_signs(wl))).cuda(),
                            torch.from_numpy(W.qjl_projection(wl)).cuda())
    k = W.gen_kv(wl, 0, 0, 4).cuda()
    v = W.gen_kv(wl, 0, 1, 4).cuda()
    with pytest.raises(K.KvqError) as e:
        cache.prefill_quantize(0, k, v)
    assert e.value.name == "KVQ_ERR_NOT_READY"
    with pytest.raises(K.KvqError) as e:  # the split takes its outliers from V's block
        cache.calibrate(0, W.gen_calib(wl, 0, 0, device="cuda"), None)
    assert e.value.name == "KVQ_ERR_INVALID_ARG"
    assert cache.length(0, 0) == 0


def test_q8_0_k_turbo_mse_v_small():
    # the application rule K = Q8 (symmetric q8_0), V = TurboQuant 3-bit, appended token by token
    wl = W.LLAMA3B_32K_Q8_0_TURBO_V
    _say("case:", wl.name, "1 layer, 401 appends")
    case = Case(wl, 401, layers=[2])
    case.append_all(0)
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0)
    _decode_and_compare(case, 0, planes)


@pytest.mark.parametrize("wl", [W.DENSE27B_120K_U8, W.DENSE27B_120K_KVARN, W.DENSE27B_120K_Q8_0],
                         ids=lambda w: w.name)
def test_dense27b_bf16_gqa5_small(wl):
    _say("case:", wl.name, "1 layer, 2 seqs, 650 tokens")
    case = Case(wl, 650, layers=[63], batch=2)
    case.prefill(0)
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0, heads=[0, 3, 7])
    _decode_and_compare(case, 0, None)


def test_progressive_batch_ragged_lengths():
    # two sequences of different lengths: append to seq 0 only (batch=1 calls) after a shared prefill
    wl = W.LLAMA3B_128K_PROGRESSIVE
    _say("case:", wl.name, "batch 2, ragged")
    case = Case(wl, 500, layers=[0], batch=2, extra_tokens=64)
    case.prefill(0)
    k, v = W.gen_step_kv(wl, 0, 0, batch=1)
    case.cache.append(0, k.to("cuda"), v.to("cuda"))
    torch.cuda.synchronize()
    assert case.cache.length(0, 0) == 501 and case.cache.length(0, 1) == 500
    q = W.gen_q(wl, 0, 0, batch=2).to("cuda")
    qn = q.float().cpu().numpy()
    gots = []
    for path in (1, 2):
        case.cache.set_option(2, path)
        out = torch.empty((2, 24, 128), device="cuda")
        case.cache.attn_decode(0, q, out)
        torch.cuda.synchronize()
        gots.append(out.cpu().numpy())
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    for b in (0, 1):
        ref = np.zeros((24, 128))
        for h in range(8):
            pk, tk = case.oracle_plane(0, b, h, 0, case.oracle_tables(0, h, 0))
            pv, tv = case.oracle_plane(0, b, h, 1, case.oracle_tables(0, h, 1))
            if b == 0:
                pk.append(k[0, h].float().numpy(), tk)
                pv.append(v[0, h].float().numpy(), tv)
                compare_plane(case.device_plane(0, 0, h, 0), pk, f"seq0 head {h} K")
                compare_plane(case.device_plane(0, 0, h, 1), pv, f"seq0 head {h} V")
            ref[h * 3:h * 3 + 3] = oracle.attention(pk, pv, tk, tv, qn[b, h * 3:h * 3 + 3])
        for got in gots:
            assert rel_l2(got[b], ref) <= REL_L2_TOL and max_abs(got[b], ref) <= MAX_ABS_TOL


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("wl", [W.LLAMA3B_3970_PROGRESSIVE, W.LLAMA3B_32K_TURBO, W.LLAMA3B_32K_TURBO_ASYM,
                                W.LLAMA8B_32K_TURBO25_KV],
                         ids=lambda w: w.name)
def test_split_count_invariance_and_determinism(wl, path):
    _say("case: split invariance", wl.name, "path", path)
    case = Case(wl, 3970, layers=[0])
    case.prefill(0)
    case.cache.set_option(2, path)
    q = W.gen_q(wl, 0, 0).to("cuda")
    outs = {}
    for st in (0, 64, 256, 1024, 4096):
        case.cache.set_option(1, st)
        o1 = torch.empty((1, wl.n_q_heads, 128), device="cuda")
        o2 = torch.empty((1, wl.n_q_heads, 128), device="cuda")
        case.cache.attn_decode(0, q, o1)
        case.cache.attn_decode(0, q, o2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), st  # run-to-run bit identity at a fixed split count
        outs[st] = o1.cpu().numpy()
    for st, o in outs.items():
        assert rel_l2(o, outs[0]) < 1e-5, st


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("wl", [W.LLAMA3B_32K_KVARN, W.LLAMA8B_32K_TURBO25_KV], ids=lambda w: w.name)
def test_decode_batch_with_an_empty_sequence(wl, path):
    # one decode call over a batch whose last sequence is empty: the empty sequence's splits all
    # hold m = -inf, l = 0 and the merge writes zeros for it (l = 0), while the others match the
    # oracle (lengths 700 and 130, built by a batch-2 and a batch-1 prefill call)
    _say("case: batch with an empty sequence,", wl.name, "path", path)
    case = Case(wl, 700, layers=[0], batch=3)
    case.cache.set_option(2, path)
    streams = {b: ([], []) for b in range(2)}
    for ci, (nb, nt) in enumerate([(2, 130), (1, 570)]):
        k = W.gen_kv(wl, 2000 + ci, 0, nt, batch=nb)
        v = W.gen_kv(wl, 2000 + ci, 1, nt, batch=nb)
        case.cache.prefill_quantize(0, k.to("cuda"), v.to("cuda"))
        for b in range(nb):
            streams[b][0].append(k[b].float().numpy())
            streams[b][1].append(v[b].float().numpy())
    q = W.gen_q(wl, 0, 0, batch=3).to("cuda")
    out = torch.full((3, wl.n_q_heads, 128), 7.0, device="cuda")
    case.cache.attn_decode(0, q, out)
    torch.cuda.synchronize()
    assert [case.cache.length(0, b) for b in range(3)] == [700, 130, 0]
    got = out.cpu().numpy()
    assert np.count_nonzero(got[2]) == 0
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    cap = case.cache.cfg.max_context
    qn = q.float().cpu().numpy()
    G = wl.group
    for b in range(2):
        ref = np.zeros((wl.n_q_heads, 128))
        for h in range(wl.n_kv_heads):
            pl = []
            for tensor in (0, 1):
                scheme = wl.k_scheme if tensor == 0 else wl.v_scheme
                bits = wl.k_bits if tensor == 0 else wl.v_bits
                rot = (wl.rotate_k if tensor == 0 else wl.rotate_v) or W.is_turbo(scheme)
                sink = wl.sinkhorn_iters > 0 and not W.is_turbo(scheme)
                tb = case.oracle_tables(0, h, tensor, mu, theta)
                pln = oracle.Plane(scheme, bits, rot, sink, wl.window, tensor, cap)
                pln.append(np.concatenate(streams[b][tensor])[:, h], tb)
                pl.append((pln, tb))
            ref[h * G:(h + 1) * G] = oracle.attention(pl[0][0], pl[1][0], pl[0][1], pl[1][1], qn[b, h * G:(h + 1) * G])
        e, m = rel_l2(got[b], ref), max_abs(got[b], ref)
        _say(f"  seq {b}: rel_l2={e:.2e} max_abs={m:.2e}")
        assert e <= REL_L2_TOL and m <= MAX_ABS_TOL, (b, e, m)


@pytest.mark.parametrize("path", [1, 2])
def test_empty_and_single_token(path):
    wl = W.LLAMA3B_32K_KVARN
    _say("case: empty / single token, path", path)
    case = Case(wl, 1, layers=[0], extra_tokens=10)
    case.cache.set_option(2, path)
    q = W.gen_q(wl, 0, 0).to("cuda")
    out = torch.full((1, 24, 128), 7.0, device="cuda")
    case.cache.attn_decode(0, q, out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    case.prefill(0)
    case.cache.attn_decode(0, q, out)
    torch.cuda.synchronize()
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    for h in range(8):
        pv, tv = case.oracle_plane(0, 0, h, 1, case.oracle_tables(0, h, 1))
        ref = pv.dequant(0, tv)
        for g in range(3):
            assert rel_l2(out[0, 3 * h + g].cpu().numpy(), ref) < 1e-5


def test_capacity_and_batch_limits_leave_state_unchanged():
    """A call past max_context or max_batch fails with its status before anything is enqueued:
    lengths, planes and the output buffer are left as they were."""
    wl = W.LLAMA3B_3970_PROGRESSIVE
    case = Case(wl, 90, layers=[0], batch=2, max_context=100)
    K = case.K
    case.prefill(0)
    torch.cuda.synchronize()
    before = [case.device_plane(0, b, 0, 0) for b in (0, 1)]
    k = W.gen_kv(wl, 7, 0, 11, batch=2).to("cuda")
    v = W.gen_kv(wl, 7, 1, 11, batch=2).to("cuda")
    with pytest.raises(K.KvqError) as e:
        case.cache.prefill_quantize(0, k, v)  # 90 + 11 > 100
    assert e.value.name == "KVQ_ERR_CAPACITY"
    k3 = W.gen_kv(wl, 7, 0, 1, batch=3).to("cuda")
    v3 = W.gen_kv(wl, 7, 1, 1, batch=3).to("cuda")
    with pytest.raises(ValueError):  # the binding refuses batch 3 > max_batch 2 ...
        case.cache.prefill_quantize(0, k3, v3)
    lib = K._kvq.load()  # ... and so does the library itself, called directly
    st = lib.kvq_prefill_quantize(case.cache.handle, 0, k3.data_ptr(), v3.data_ptr(), 0, 1, 3, None)
    assert st == 1  # KVQ_ERR_INVALID_ARG
    q3 = W.gen_q(wl, 0, 0, batch=3).to("cuda")
    out3 = torch.full((3, 24, 128), 3.0, device="cuda")
    with pytest.raises(ValueError):
        case.cache.attn_decode(0, q3, out3)
    assert lib.kvq_attn_decode(case.cache.handle, 0, q3.data_ptr(), 0, out3.data_ptr(), 3, 0.0, None) == 1
    torch.cuda.synchronize()
    assert case.cache.length(0, 0) == 90 and case.cache.length(0, 1) == 90
    assert bool((out3 == 3.0).all())
    for b in (0, 1):
        for x, y in zip(before[b], case.device_plane(0, b, 0, 0)):
            if x is not None:
                assert np.array_equal(x, y)
    # filling the cache exactly to max_context is allowed
    k10 = W.gen_kv(wl, 8, 0, 10, batch=2).to("cuda")
    v10 = W.gen_kv(wl, 8, 1, 10, batch=2).to("cuda")
    case.cache.prefill_quantize(0, k10, v10)
    torch.cuda.synchronize()
    assert case.cache.length(0, 0) == 100


@pytest.mark.parametrize("path", [1, 2])
def test_max_batch_64_sequences(path):
    """The largest batch a call takes (64 sequences, ragged lengths): planes of sampled
    sequences are bit-exact and their attention matches the oracle."""
    wl = W.LLAMA3B_32K_KVARN
    B = 64
    _say("case: batch 64, path", path)
    case = Case(wl, 160, layers=[0], batch=B, extra_tokens=40)
    case.prefill(0)
    # ragged: the first 17 sequences get 23 more tokens
    k = W.gen_kv(wl, 500, 0, 23, batch=17).to("cuda")
    v = W.gen_kv(wl, 500, 1, 23, batch=17).to("cuda")
    case.cache.prefill_quantize(0, k, v)
    case.cache.set_option(2, path)
    q = W.gen_q(wl, 0, 0, batch=B).to("cuda")
    out = torch.full((B, 24, 128), float("nan"), device="cuda")
    case.cache.attn_decode(0, q, out)
    torch.cuda.synchronize()
    assert case.cache.length(0, 0) == 183 and case.cache.length(0, 63) == 160
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    qn = q.float().cpu().numpy()
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    cap = case.cache.cfg.max_context
    base_k, base_v = case.kv(0)
    for b in (0, 16, 17, 63):
        ref = np.zeros((24, 128))
        for h in range(8):
            pl = []
            for tensor, base, extra in ((0, base_k, k), (1, base_v, v)):
                X = base[b, :, h].float().cpu().numpy()
                if b < 17:
                    X = np.concatenate([X, extra[b, :, h].float().cpu().numpy()])
                tb = case.oracle_tables(0, h, tensor, mu, theta)
                p = oracle.Plane(W.UNIFORM, 4, True, True, 0, tensor, cap)
                p.append(X, tb)
                if h in (0, 7):
                    compare_plane(case.device_plane(0, b, h, tensor), p, f"seq {b} head {h} tensor {tensor}")
                pl += [p, tb]
            ref[h * 3:h * 3 + 3] = oracle.attention(pl[0], pl[2], pl[1], pl[3], qn[b, h * 3:h * 3 + 3])
        r, m = rel_l2(got[b], ref), max_abs(got[b], ref)
        assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (b, r, m)


def _planes_equal(a, b, li, batch, n_heads):
    for s in range(batch):
        for h in range(n_heads):
            for t in (0, 1):
                for x, y in zip(a.device_plane(li, s, h, t), b.device_plane(li, s, h, t)):
                    if x is not None:
                        assert np.array_equal(x, y), (s, h, t)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("wl,n", [(W.LLAMA3B_3970_PROGRESSIVE, 1000), (W.LLAMA3B_3970_PROGRESSIVE, 0),
                                  (W.LLAMA3B_32K_KVARN, 1023), (W.LLAMA3B_32K_TURBO, 700),
                                  (W.LLAMA3B_32K_TURBO_ASYM, 64), (W.DENSE27B_120K_KVARN, 500),
                                  (W.LLAMA3B_32K_Q8_0_TURBO_V, 130), (W.DENSE27B_120K_Q8_0, 65),
                                  (W.LLAMA3B_32K_Q8_0_TURBO4_V, 200), (W.LLAMA8B_32K_Q8_0_TURBO25_V, 190),
                                  (W.LLAMA8B_32K_Q8_0_TURBO35_V, 64), (W.LLAMA3B_32K_U8_K_U3_V, 257),
                                  (W.LLAMA3B_32K_KVARN_U3, 100)],
                         ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_fused_append_decode_equals_separate_calls(wl, n, path):
    # kvq_append_attn_decode == kvq_append + kvq_attn_decode: byte-identical planes and
    # bit-identical outputs over consecutive steps, with ragged lengths in the batch
    _say("case: fused append+decode", wl.name, "n", n, "path", path)
    B = 2
    a = Case(wl, max(n, 1), layers=[0], batch=B, extra_tokens=8)
    b = Case(wl, max(n, 1), layers=[0], batch=B, extra_tokens=8)
    for c in (a, b):
        c.cache.set_option(2, path)
        if n > 0:
            c.prefill(0)
    k0, v0 = W.gen_step_kv(wl, 0, 99, batch=1)
    for c in (a, b):  # sequence 0 one token longer than sequence 1
        c.cache.append(0, k0.to("cuda"), v0.to("cuda"))
    for step in range(3):
        k, v = W.gen_step_kv(wl, 0, step, batch=B)
        q = W.gen_q(wl, 0, step, batch=B).to("cuda")
        k, v = k.to("cuda"), v.to("cuda")
        oa = torch.full((B, wl.n_q_heads, 128), float("nan"), device="cuda")
        ob = torch.full_like(oa, float("nan"))
        a.cache.append(0, k, v)
        a.cache.attn_decode(0, q, oa)
        b.cache.append_attn_decode(0, k, v, q, ob)
        torch.cuda.synchronize()
        assert a.cache.length(0, 0) == b.cache.length(0, 0) == n + 2 + step
        assert torch.equal(oa, ob), step
        _planes_equal(a, b, 0, B, wl.n_kv_heads)


def test_fused_append_decode_matches_oracle():
    wl = W.LLAMA3B_3970_PROGRESSIVE
    _say("case: fused append+decode vs oracle", wl.name)
    n = 777
    case = Case(wl, n + 1, layers=[0])
    k_all, v_all = case.kv(0)
    case.cache.prefill_quantize(0, k_all[:, :n].contiguous(), v_all[:, :n].contiguous())
    q = W.gen_q(wl, 0, 5).to("cuda")
    out = torch.empty((1, wl.n_q_heads, 128), device="cuda")
    case.cache.append_attn_decode(0, k_all[:, n].contiguous(), v_all[:, n].contiguous(), q, out)
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0)
    ref = oracle_attention_case(case, 0, 0, q.float().cpu().numpy()[0],
                                planes={h: planes[(0, h)] for h in range(wl.n_kv_heads)})
    got = out.cpu().numpy()[0]
    assert rel_l2(got, ref) <= REL_L2_TOL and max_abs(got, ref) <= MAX_ABS_TOL


# Progressive caches at the edges of the FP32 window: every token in the ring (n <= 128), the
# first token read from the codes (n = 129), and a few beyond.  Plain, rotated + balanced, and
# TurboQuant-QJL keys beside the window.
WINDOW_EDGE_NS = [1, 2, 64, 127, 128, 129, 130, 192, 257]


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("wl", [W.LLAMA3B_3970_PROGRESSIVE,
                                W.LLAMA3B_32K_KVARN.with_(name="llama3b-kvarn-u4-window", window=128),
                                W.LLAMA3B_32K_TURBO.with_(name="llama3b-turboqjl-k-window", window=128),
                                W.LLAMA8B_32K_TURBO25_KV.with_(name="llama8b-split2.5-kv-window", window=128)],
                         ids=lambda w: w.name)
def test_window_edges_decode_and_fused(wl, path):
    """At each n the cache holds tokens 0 .. n - 2 (bulk prefill and appends), token n - 1 comes
    through kvq_append_attn_decode, then kvq_attn_decode runs on the same cache: planes and ring
    bit-exact, both outputs against the oracle."""
    _say("case: window edges,", wl.name, "path", path, WINDOW_EDGE_NS)
    n_max = max(WINDOW_EDGE_NS)
    case = Case(wl, n_max, layers=[0])
    case.cache.set_option(2, path)
    k_all, v_all = case.kv(0)
    done = 0
    for n in WINDOW_EDGE_NS:
        if n - 1 > done:
            case.cache.prefill_quantize(0, k_all[:, done:n - 1].contiguous(), v_all[:, done:n - 1].contiguous())
            done = n - 1
        q = W.gen_q(wl, 0, n).to("cuda")
        o_fused = torch.full((1, wl.n_q_heads, 128), float("nan"), device="cuda")
        case.cache.append_attn_decode(0, k_all[:, n - 1].contiguous(), v_all[:, n - 1].contiguous(), q, o_fused)
        done = n
        o_dec = torch.full_like(o_fused, float("nan"))
        case.cache.attn_decode(0, q, o_dec)
        torch.cuda.synchronize()
        assert case.cache.length(0, 0) == n
        _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
        planes = {}
        for h in range(wl.n_kv_heads):
            row = []
            for tensor in (0, 1):
                tb = case.oracle_tables(0, h, tensor, mu, theta)
                p, _ = case.oracle_plane(0, 0, h, tensor, tb, n=n)
                if h in (0, 7):
                    compare_plane(case.device_plane(0, 0, h, tensor), p, f"n {n} head {h} tensor {tensor}")
                row += [p, tb]
            planes[h] = row
        ref = oracle_attention_case(case, 0, 0, q.float().cpu().numpy()[0], planes=planes)
        for label, o in (("fused", o_fused), ("decode", o_dec)):
            got = o.cpu().numpy()[0]
            r, m = rel_l2(got, ref), max_abs(got, ref)
            assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (n, label, r, m)
        _say(f"  n={n}: planes bit-exact, fused and decode within tolerance")


# Five query heads per kv head (the 27B shape) with the value coders whose matrix-core kernels
# take the two-head-block form: 4-bit TurboQuant-MSE V and the split V at 2.5 / 3.5 bits.
G5_TURBO_V = [
    W.DENSE27B_120K_Q8_0.with_(name="dense27b-q8_0-k-turbo4mse-v", v_scheme=W.TURBO_MSE, v_bits=4,
                               rotate_v=True),
    W.DENSE27B_120K_Q8_0.with_(name="dense27b-q8_0-k-turbo2.5split-v", v_scheme=W.TURBO_SPLIT, v_bits=3,
                               rotate_v=True, calib_tokens=512),
    W.DENSE27B_120K_Q8_0.with_(name="dense27b-q8_0-k-turbo3.5split-v", v_scheme=W.TURBO_SPLIT, v_bits=4,
                               rotate_v=True, calib_tokens=512),
]


@pytest.mark.parametrize("wl", G5_TURBO_V, ids=lambda w: w.name)
def test_gqa5_turbo_values_both_paths(wl):
    _say("case:", wl.name, "2 seqs, 300 prefill + 44 appends + 1 fused step")
    case = Case(wl, 345, layers=[0], batch=2)
    k, v = case.kv(0)
    case.cache.prefill_quantize(0, k[:, :300].contiguous(), v[:, :300].contiguous())
    for t in range(300, 344):
        case.cache.append(0, k[:, t].contiguous(), v[:, t].contiguous())
    q = W.gen_q(wl, 0, 9, batch=2).to("cuda")
    out = torch.full((2, wl.n_q_heads, 128), float("nan"), device="cuda")
    case.cache.append_attn_decode(0, k[:, 344].contiguous(), v[:, 344].contiguous(), q, out)
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0, heads=[0, 7])
    qn = q.float().cpu().numpy()
    for b in (0, 1):
        ref = oracle_attention_case(case, 0, b, qn[b])
        r, m = rel_l2(out.cpu().numpy()[b], ref), max_abs(out.cpu().numpy()[b], ref)
        assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (b, r, m)
    _decode_and_compare(case, 0, None)  # both decode paths


# Uniform 3-bit group packing (codes as three bit planes, fp16 scale and zero per 32 channels):
# K 8-bit / V 3-bit, WHT + Sinkhorn 3-bit K and V, the same with five query heads per kv head and
# bf16 sources, and a progressive 3-bit cache with the FP32 window.
U3_CASES = [
    W.LLAMA3B_32K_U8_K_U3_V,
    W.LLAMA3B_32K_KVARN_U3,
    W.DENSE27B_120K_KVARN.with_(name="dense27b-wht-sinkhorn-u3", k_bits=3, v_bits=3),
    W.LLAMA3B_128K_PROGRESSIVE.with_(name="llama3b-u3-progressive", k_bits=3, v_bits=3),
]


@pytest.mark.parametrize("wl", U3_CASES, ids=lambda w: w.name)
def test_uniform3_planes_and_decode(wl):
    _say("case:", wl.name, "2 seqs, 300 prefill + 44 appends + 1 fused step")
    case = Case(wl, 345, layers=[0], batch=2)
    k, v = case.kv(0)
    case.cache.prefill_quantize(0, k[:, :300].contiguous(), v[:, :300].contiguous())
    for t in range(300, 344):
        case.cache.append(0, k[:, t].contiguous(), v[:, t].contiguous())
    q = W.gen_q(wl, 0, 9, batch=2).to("cuda")
    out = torch.full((2, wl.n_q_heads, 128), float("nan"), device="cuda")
    case.cache.append_attn_decode(0, k[:, 344].contiguous(), v[:, 344].contiguous(), q, out)
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0)
    qn = q.float().cpu().numpy()
    for b in (0, 1):
        pl = {h: planes[(b, h)] for h in range(wl.n_kv_heads)}
        ref = oracle_attention_case(case, 0, b, qn[b], planes=pl)
        r, m = rel_l2(out.cpu().numpy()[b], ref), max_abs(out.cpu().numpy()[b], ref)
        _say(f"  fused step seq {b}: rel_l2={r:.2e} max_abs={m:.2e}")
        assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (b, r, m)
    _decode_and_compare(case, 0, planes)  # both decode paths


F16_CASES = [
    W.LLAMA3B_32K_KVARN.with_(name="llama3b-wht-sinkhorn-u4-f16", dtype="f16"),
    W.LLAMA3B_32K_TURBO.with_(name="llama3b-turboqjl-k-u4-v-f16", dtype="f16"),
    W.LLAMA8B_32K_Q8_0_TURBO25_V.with_(name="llama8b-q8_0-k-turbo2.5split-v-f16", dtype="f16"),
    W.LLAMA3B_3970_PROGRESSIVE.with_(name="llama3b-u4-progressive-f16", dtype="f16"),
    W.DENSE27B_120K_KVARN.with_(name="dense27b-wht-sinkhorn-u4-f16", dtype="f16"),
]


@pytest.mark.parametrize("wl", F16_CASES, ids=lambda w: w.name)
def test_f16_inputs_planes_and_decode(wl):
    # KVQ_F16 inputs (K, V, q and the calibration block rounded to fp16): the library widens them
    # exactly, so planes, tables and attention meet the oracle fed the same values in fp32 --
    # bulk prefill, per-token appends, a fused step and both decode paths
    _say("case:", wl.name, "2 seqs, 300 prefill + 20 appends + 1 fused step")
    case = Case(wl, 321, layers=[0], batch=2)
    k, v = case.kv(0)
    assert k.dtype == torch.float16
    case.cache.prefill_quantize(0, k[:, :300].contiguous(), v[:, :300].contiguous())
    for t in range(300, 320):
        case.cache.append(0, k[:, t].contiguous(), v[:, t].contiguous())
    q = W.gen_q(wl, 0, 5, batch=2).to("cuda")
    out = torch.full((2, wl.n_q_heads, 128), float("nan"), device="cuda")
    case.cache.append_attn_decode(0, k[:, 320].contiguous(), v[:, 320].contiguous(), q, out)
    torch.cuda.synchronize()
    planes = _check_all_planes(case, 0)
    qn = q.float().cpu().numpy()
    for b in (0, 1):
        pl = {h: planes[(b, h)] for h in range(wl.n_kv_heads)}
        ref = oracle_attention_case(case, 0, b, qn[b], planes=pl)
        r, m = rel_l2(out.cpu().numpy()[b], ref), max_abs(out.cpu().numpy()[b], ref)
        _say(f"  fused step seq {b}: rel_l2={r:.2e} max_abs={m:.2e}")
        assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (b, r, m)
    _decode_and_compare(case, 0, planes)


SPLIT_KV = [W.LLAMA8B_32K_TURBO25_KV, W.LLAMA8B_32K_TURBO35_KV,
            W.LLAMA8B_32K_TURBO25_KV.with_(name="llama8b-turbo2.5split-k-u4-v", v_scheme=W.UNIFORM, v_bits=4,
                                           rotate_v=False),
            W.LLAMA8B_32K_TURBO35_KV.with_(name="llama8b-turbo3.5split-k-progressive", window=128),
            W.LLAMA8B_32K_TURBO25_KV.with_(name="llama8b-turbo2.5split-kv-g5", n_q_heads=40),
            W.LLAMA8B_32K_TURBO35_KV.with_(name="llama8b-turbo3.5split-k-turbomse-v-bf16", v_scheme=W.TURBO_MSE,
                                           v_bits=3, dtype="bf16")]


@pytest.mark.parametrize("wl", SPLIT_KV, ids=lambda w: w.name)
def test_split_keys_planes_and_decode(wl):
    # keys at 2.5 / 3.5 bits (split MSE codes + QJL): bulk prefill (the per-token quantizer for the
    # key plane), appends and a fused step (matrix-core path) leave the oracle's bytes, and both
    # decode paths meet the oracle's split-key score
    _say("case:", wl.name, "2 seqs, 300 prefill + 20 appends + 1 fused step")
    case = Case(wl, 321, layers=[0], batch=2)
    k, v = case.kv(0)
    case.cache.prefill_quantize(0, k[:, :300].contiguous(), v[:, :300].contiguous())
    for t in range(300, 320):
        case.cache.append(0, k[:, t].contiguous(), v[:, t].contiguous())
    q = W.gen_q(wl, 0, 5, batch=2).to("cuda")
    out = torch.full((2, wl.n_q_heads, 128), float("nan"), device="cuda")
    case.cache.append_attn_decode(0, k[:, 320].contiguous(), v[:, 320].contiguous(), q, out)
    torch.cuda.synchronize()
    perm_k = case.cache.table("perm_k", 8 * 128).cpu().numpy().reshape(8, 128)
    for h in range(8):
        assert np.array_equal(perm_k[h], oracle.select_outliers(case.calib[0][0][:, h, :])), h
    planes = _check_all_planes(case, 0)
    qn = q.float().cpu().numpy()
    for b in (0, 1):
        pl = {h: planes[(b, h)] for h in range(wl.n_kv_heads)}
        ref = oracle_attention_case(case, 0, b, qn[b], planes=pl)
        r, m = rel_l2(out.cpu().numpy()[b], ref), max_abs(out.cpu().numpy()[b], ref)
        _say(f"  fused step seq {b}: rel_l2={r:.2e} max_abs={m:.2e}")
        assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (b, r, m)
    _decode_and_compare(case, 0, planes)  # both decode paths


@pytest.mark.parametrize("wl", [W.LLAMA3B_32K_TURBO, W.LLAMA3B_32K_KVARN, W.LLAMA8B_32K_TURBO25_KV],
                         ids=lambda w: w.name)
def test_seeded_random_tables(wl):
    # kvq_set_random_tables_seeded: the device holds exactly the oracle's draw from the seed (signs
    # and S; the transposed copy the kernels read shows in the QJL bits and scores), and the planes
    # and attention built on them match the oracle's, on both decode paths
    seed = 20261202
    _say("case:", wl.name, "seeded tables, 2 layers, 300 prefill + 10 appends")
    case = Case(wl, 310, layers=[0, 1], seed=seed)
    L, H = 2, wl.n_kv_heads
    sg = case.cache.table("signs", L * H * 2 * 128).cpu().numpy().reshape(L, H, 2, 128)
    S = case.cache.table("qjl_S", 128 * 128).cpu().numpy().reshape(128, 128)
    assert np.array_equal(sg.view(np.uint32), case.signs.view(np.uint32))
    assert np.array_equal(S.view(np.uint32), case.S.view(np.uint32))
    for li in range(2):
        k, v = case.kv(li)
        case.cache.prefill_quantize(li, k[:, :300].contiguous(), v[:, :300].contiguous())
        for t in range(300, 310):
            case.cache.append(li, k[:, t].contiguous(), v[:, t].contiguous())
    torch.cuda.synchronize()
    for li in range(2):
        planes = _check_all_planes(case, li, heads=[0, 5, 7])
        _decode_and_compare(case, li, None)
