"""Host-only checks of libkvq: it loads, exports every symbol include/kvq.h declares, plans the
buffer layout with the byte counts the format implies, and rejects bad arguments before touching
the device.  No compute call is made (no GPU here)."""
import ctypes
import os
import re

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
K = pytest.importorskip("quantized_decode_attention_kvq_amd._kvq")


def _header_symbols():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = K.load()
    syms = _header_symbols()
    assert len(syms) >= 14
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(K.EXPORTS) == syms


def _cfg(wl, **over):
    d = wl.kvq_config()
    d.update(over)
    return K.make_config(**d)


def test_required_bytes_match_format():
    # 4-bit K and V: 64 B codes + 16 B meta per token-head (the "6.4x" of the quantcpp article);
    # the 32K KVarN workload is 28 layers x 8 heads x 32768 tokens x 160 B plus small tables.
    wl = W.LLAMA3B_32K_KVARN
    n = K.kvq_cache_required_bytes(_cfg(wl))
    planes = 28 * 8 * 32768 * 160
    assert planes <= n <= planes + 16 * 2 ** 20
    # 8-bit: 128 + 16 B per token-head
    wl8 = W.DENSE27B_120K_U8
    n8 = K.kvq_cache_required_bytes(_cfg(wl8))
    p8 = 64 * 4 * 8 * 122880 * 144 * 2
    assert p8 <= n8 <= p8 + 64 * 2 ** 20
    # TurboQuant K: 48 B codes + 4 B norms + 16 B QJL bits = 68 B; uniform 4-bit V: 80 B
    wlt = W.LLAMA3B_32K_TURBO
    nt = K.kvq_cache_required_bytes(_cfg(wlt))
    pt = 28 * 8 * 32768 * (68 + 80)
    assert pt <= nt <= pt + 16 * 2 ** 20
    # progressive window: 128 x 128 fp32 per (layer, seq, head, tensor) on top of the codes
    wlp = W.LLAMA3B_128K_PROGRESSIVE
    npg = K.kvq_cache_required_bytes(_cfg(wlp))
    pp = 28 * 8 * (131072 * 160 + 2 * 128 * 512)
    assert pp <= npg <= pp + 16 * 2 ** 20
    # 3-bit uniform: 48 B of bit planes + 16 B meta = 64 B per token-head (K 8-bit: 144 B)
    wl3 = W.LLAMA3B_32K_U8_K_U3_V
    n3 = K.kvq_cache_required_bytes(_cfg(wl3))
    p3 = 28 * 8 * 32768 * (144 + 64)
    assert p3 <= n3 <= p3 + 16 * 2 ** 20
    n33 = K.kvq_cache_required_bytes(_cfg(W.LLAMA3B_32K_KVARN_U3))
    p33 = 28 * 8 * 32768 * (64 + 64)
    assert p33 <= n33 <= p33 + 16 * 2 ** 20
    # split V (2.5 / 3.5 bits): 40 / 56 B codes + 4 B norms per token-head, K q8_0 at 144 B
    for wls, vb in ((W.LLAMA8B_32K_Q8_0_TURBO25_V, 44), (W.LLAMA8B_32K_Q8_0_TURBO35_V, 60)):
        ns = K.kvq_cache_required_bytes(_cfg(wls))
        ps = 32 * 8 * 32768 * (144 + vb)
        assert ps <= ns <= ps + 16 * 2 ** 20
    # split K (2.5 / 3.5 bits): 24 / 40 B split codes + 16 B QJL signs + 8 B norms and gamma,
    # beside split V at 44 / 60 B
    for wls, kb, vb in ((W.LLAMA8B_32K_TURBO25_KV, 48, 44), (W.LLAMA8B_32K_TURBO35_KV, 64, 60)):
        ns = K.kvq_cache_required_bytes(_cfg(wls))
        ps = 32 * 8 * 32768 * (kb + vb)
        assert ps <= ns <= ps + 16 * 2 ** 20


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), 2), (dict(group_size=64), 2), (dict(k_bits=5), 2), (dict(v_bits=2), 2),
    (dict(fp32_window=64), 2), (dict(n_q_heads=25), 1), (dict(n_q_heads=8 * 9), 2),
    (dict(max_batch=65), 2), (dict(max_batch=0), 1), (dict(k_scheme=2), 2), (dict(v_scheme=1), 2),
    (dict(rotate_k=2), 1), (dict(n_layers=0), 1), (dict(sinkhorn_iters=5, calib_tokens=1), 2),
    # the outlier split takes 3 or 4 outlier bits and needs a calibration block, on either tensor
    (dict(k_scheme=4, k_bits=3), 2), (dict(k_scheme=4, k_bits=5, calib_tokens=512), 2),
    (dict(k_scheme=4, k_bits=2, calib_tokens=512), 2), (dict(v_scheme=4, v_bits=2, calib_tokens=512), 2),
    (dict(v_scheme=4, v_bits=5, calib_tokens=512), 2), (dict(v_scheme=4, v_bits=3, calib_tokens=0), 2),
])
def test_invalid_configs_rejected(over, status):
    with pytest.raises(K.KvqError) as e:
        K.kvq_cache_required_bytes(_cfg(W.LLAMA3B_3970_PROGRESSIVE, **over))
    assert e.value.status == status


def test_create_argument_checks_before_device():
    lib = K.load()
    cfg = _cfg(W.LLAMA3B_3970_PROGRESSIVE)
    need = K.kvq_cache_required_bytes(cfg)
    h = ctypes.c_void_p()
    assert lib.kvq_cache_create(ctypes.byref(cfg), None, need, None, ctypes.byref(h)) == 1
    assert lib.kvq_cache_create(ctypes.byref(cfg), ctypes.c_void_p(0x10010), need, None,
                                ctypes.byref(h)) == 6
    assert lib.kvq_cache_create(ctypes.byref(cfg), ctypes.c_void_p(0x10000), need - 1, None,
                                ctypes.byref(h)) == 5
    assert lib.kvq_cache_create(ctypes.byref(cfg), ctypes.c_void_p(0x10000), need, None, None) == 1
    assert not h.value


def test_null_handle_calls_rejected():
    lib = K.load()
    assert lib.kvq_append(None, 0, None, None, 0, 1, None) == 1
    assert lib.kvq_attn_decode(None, 0, None, 0, None, 1, 0.0, None) == 1
    assert lib.kvq_calibrate(None, 0, None, None, 0, 512, None) == 1
    assert lib.kvq_get_length(None, 0, 0) == -1
    assert lib.kvq_cache_destroy(None) == 1
    assert lib.kvq_set_timing_events(None, None, None) == 1
    assert lib.kvq_set_option(None, 1, 0) == 1
    assert K.kvq_status_str(0) == "ok" and K.kvq_status_str(3) == "context capacity exceeded"


def test_binding_refuses_bad_tensors_before_c():
    """The binding checks every tensor against the handle's shapes, the call's dtype rules and
    device residency before a pointer reaches C (which takes no sizes).  A fake handle is
    registered with the binding only: no call below may reach the library."""
    import torch
    h = ctypes.c_void_p(0x5000)
    K._SHAPES[h.value] = {"n_layers": 2, "n_q_heads": 24, "n_kv_heads": 8, "max_batch": 2}
    try:
        q, out = torch.zeros(1, 24, 128), torch.zeros(1, 24, 128)
        with pytest.raises(TypeError, match="device"):
            K.kvq_attn_decode(h, 0, q, out)  # host tensors
        with pytest.raises(ValueError, match="shape"):
            K.kvq_attn_decode(h, 0, torch.zeros(1, 23, 128), out)  # head count
        with pytest.raises(ValueError, match="shape"):
            K.kvq_attn_decode(h, 0, q, torch.zeros(1, 24, 64))  # undersized out
        with pytest.raises(TypeError, match="dtype"):
            K.kvq_attn_decode(h, 0, q, torch.zeros(1, 24, 128, dtype=torch.bfloat16))  # out not fp32
        with pytest.raises(TypeError, match="dtype"):
            K.kvq_attn_decode(h, 0, q.double(), out)  # unsupported input dtype
        with pytest.raises(ValueError, match="batch"):
            K.kvq_attn_decode(h, 0, torch.zeros(3, 24, 128), torch.zeros(3, 24, 128))  # > max_batch
        k32, v32 = torch.zeros(1, 8, 128), torch.zeros(1, 8, 128)
        with pytest.raises(TypeError, match="one dtype"):
            K.kvq_append_attn_decode(h, 0, k32, v32, q.bfloat16(), out)  # mixed input dtypes
        with pytest.raises(ValueError, match="shape"):
            K.kvq_append_attn_decode(h, 0, torch.zeros(2, 8, 128), torch.zeros(2, 8, 128), q, out)
        with pytest.raises(ValueError, match="shape"):
            K.kvq_prefill_quantize(h, 0, torch.zeros(1, 5, 8, 128), torch.zeros(1, 4, 8, 128))
        with pytest.raises(ValueError, match="shape"):
            K.kvq_append(h, 0, torch.zeros(1, 7, 128), torch.zeros(1, 7, 128))  # kv head count
        with pytest.raises(ValueError, match="shape"):
            K.kvq_set_random_tables(h, torch.zeros(3, 8, 2, 128))  # layer count
        with pytest.raises(ValueError, match="shape"):
            K.kvq_attn_prefill(h, 0, torch.zeros(1, 4, 24, 128), torch.zeros(1, 4, 24, 127))
        with pytest.raises(TypeError, match="dtype"):
            K.kvq_calibrate(h, 0, torch.zeros(512, 8, 128), torch.zeros(512, 8, 128).bfloat16())
        with pytest.raises(ValueError, match="unknown kvq handle"):
            K.kvq_attn_decode(ctypes.c_void_p(0x6000), 0, q, out)
    finally:
        K._SHAPES.pop(h.value)


def test_f16_inputs_are_kvq_f16():
    # KVQ_F16 = 2 in the header and the binding; fp16 tensors pass the dtype rules (the fake
    # handle's call then stops at the residency check), fp64 does not
    import torch
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    assert re.search(r"KVQ_F16\s*=\s*2", text)
    assert K.KVQ_F16 == 2 and K._dtype(torch.zeros(1, dtype=torch.float16)) == 2
    with pytest.raises(TypeError, match="unsupported dtype"):
        K._dtype(torch.zeros(1, dtype=torch.float64))
    h = ctypes.c_void_p(0x5100)
    K._SHAPES[h.value] = {"n_layers": 2, "n_q_heads": 24, "n_kv_heads": 8, "max_batch": 2}
    try:
        q16, out = torch.zeros(1, 24, 128, dtype=torch.float16), torch.zeros(1, 24, 128)
        with pytest.raises(TypeError, match="device"):
            K.kvq_attn_decode(h, 0, q16, out)
        k16 = torch.zeros(1, 8, 128, dtype=torch.float16)
        with pytest.raises(TypeError, match="device"):
            K.kvq_append_attn_decode(h, 0, k16, k16, q16, out)
        with pytest.raises(TypeError, match="one dtype"):
            K.kvq_append_attn_decode(h, 0, k16, k16, q16.float(), out)
    finally:
        K._SHAPES.pop(h.value)


@pytest.mark.parametrize("seed", [0, 1, 123456789, 2**63 + 11, 2**64 - 1])
def test_seeded_tables_equal_the_oracle_draw(seed):
    # host-only: the library's SplitMix64 / Box-Muller draw, written separately from the oracle's
    # from the same definition, gives the same signs and projection bit for bit
    import numpy as np

    import oracle
    signs, S = K.kvq_derive_random_tables(seed, 3, 5)
    osigns, oS = oracle.derive_random_tables(seed, 3, 5)
    assert np.array_equal(signs.view(np.uint32), osigns.view(np.uint32))
    assert np.array_equal(S.view(np.uint32), oS.view(np.uint32))


def test_seeded_tables_arguments():
    lib = K.load()
    assert lib.kvq_derive_random_tables(1, 0, 8, ctypes.c_void_p(0x10000), None) == 1
    assert lib.kvq_derive_random_tables(1, 2, 0, ctypes.c_void_p(0x10000), None) == 1
    assert lib.kvq_derive_random_tables(1, 0, 0, None, None) == 0  # nothing asked, nothing drawn
    assert lib.kvq_set_random_tables_seeded(None, 1, None) == 1
