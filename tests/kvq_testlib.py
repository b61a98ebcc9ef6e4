"""Helpers shared by the GPU parity tests and smoke(): build a device cache through the C ABI,
build the oracle's planes from the same inputs, and compare them.

Inputs come only from ``workloads`` (seeded generators); expected values only from ``oracle``.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

REL_L2_TOL = 2e-3
MAX_ABS_TOL = 1e-2


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


class Case:
    """One workload instance on the device plus everything the oracle needs."""

    def __init__(self, wl: W.Workload, n_tokens: int, layers=None, batch=None, max_context=None,
                 device="cuda", gen_device=None, extra_tokens=0, seed=None):
        """seed: install the random tables with kvq_set_random_tables_seeded (the oracle then
        uses its own draw from the same seed) instead of passing the workload's tables."""
        import quantized_decode_attention_kvq_amd as K
        self.K = K
        self.wl = wl
        self.n = n_tokens
        self.layers = list(range(wl.n_layers)) if layers is None else list(layers)
        self.batch = wl.batch if batch is None else batch
        self.device = device
        self.gen_device = gen_device or "cpu"
        cfg = wl.kvq_config(max_context=max_context or (n_tokens + extra_tokens),
                            max_batch=self.batch)
        cfg["n_layers"] = len(self.layers)
        self.cache = K.KvCache(device=device, **cfg)
        if seed is not None:
            # the cache's layers are 0 .. len(layers) - 1, and so are the seeded tables'
            self.signs, self.S = oracle.derive_random_tables(seed, len(self.layers), wl.n_kv_heads)
            self.cache.set_random_tables_seeded(seed)
        else:
            self.signs = W.rotation_signs(wl)[self.layers]  # [L][Hkv][2][128]
            self.S = W.qjl_projection(wl)
        needs_signs = wl.rotate_k or wl.rotate_v or W.is_turbo(wl.k_scheme) or W.is_turbo(wl.v_scheme)
        if seed is None and (needs_signs or wl.k_scheme == W.TURBO_QJL):
            self.cache.set_random_tables(
                torch.from_numpy(np.ascontiguousarray(self.signs)).to(device),
                torch.from_numpy(self.S).to(device))
        self.calib = {}
        if wl.sinkhorn_iters > 0 or wl.v_scheme == W.TURBO_SPLIT or wl.k_scheme == W.TURBO_SPLIT:
            for li, layer in enumerate(self.layers):
                kc = W.gen_calib(wl, layer, 0, device=self.gen_device).to(device)
                vc = W.gen_calib(wl, layer, 1, device=self.gen_device).to(device)
                self.cache.calibrate(li, kc, vc)
                self.calib[layer] = (kc.float().cpu().numpy(), vc.float().cpu().numpy())
        self.inputs = {}

    # -- inputs ---------------------------------------------------------------------------------
    def kv(self, layer):
        if layer not in self.inputs:
            k = W.gen_kv(self.wl, layer, 0, self.n, device=self.gen_device, batch=self.batch)
            v = W.gen_kv(self.wl, layer, 1, self.n, device=self.gen_device, batch=self.batch)
            self.inputs[layer] = (k.to(self.device), v.to(self.device))
        return self.inputs[layer]

    def prefill(self, li, chunks=None):
        layer = self.layers[li]
        k, v = self.kv(layer)
        if chunks is None:
            self.cache.prefill_quantize(li, k, v)
        else:
            pos = 0
            for c in chunks:
                self.cache.prefill_quantize(li, k[:, pos:pos + c].contiguous(), v[:, pos:pos + c].contiguous())
                pos += c
            assert pos == self.n

    def append_all(self, li):
        layer = self.layers[li]
        k, v = self.kv(layer)
        for t in range(self.n):
            self.cache.append(li, k[:, t].contiguous(), v[:, t].contiguous())

    # -- oracle ---------------------------------------------------------------------------------
    def oracle_tables(self, li, head, tensor, mu=None, theta=None):
        wl = self.wl
        layer = self.layers[li]
        scheme = wl.k_scheme if tensor == 0 else wl.v_scheme
        rotate = (wl.rotate_k if tensor == 0 else wl.rotate_v) or W.is_turbo(scheme)
        kw = {}
        if rotate:
            kw["signs"] = self.signs[li, head, tensor]
        if wl.sinkhorn_iters > 0 and not W.is_turbo(scheme):
            X = self.calib[layer][tensor][:, head, :]
            c, inv_c = oracle.sinkhorn(X, kw.get("signs"), wl.sinkhorn_iters)
            kw["c"], kw["inv_c"] = c, inv_c
        if scheme == W.TURBO_SPLIT:
            # outlier split: channels from the tensor's calibration block, codebooks of
            # N(0, 1/64) -- V: bo / bo - 1 bits; K (b): b - 1 / b - 2 bits and the QJL projection
            bo = wl.v_bits if tensor == 1 else wl.k_bits - 1
            kw["perm"] = oracle.select_outliers(self.calib[layer][tensor][:, head, :])
            _, kw["mu"], kw["theta"], _ = _codebook64(1 << bo)
            _, kw["mu2"], kw["theta2"], _ = _codebook64(1 << (bo - 1))
            if tensor == 0:
                kw["S"] = self.S
        elif W.is_turbo(scheme):
            bits = wl.k_bits if tensor == 0 else wl.v_bits
            if bits == 4:  # 4-bit TurboQuant-MSE V: the 16-level codebook
                _, mu, theta, _ = _codebook16()
            elif mu is None:
                _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
            kw["mu"], kw["theta"] = mu, theta
            kw["S"] = self.S
        return oracle.TableSet(**kw)

    def oracle_plane(self, li, b, head, tensor, tables=None, n=None):
        wl = self.wl
        scheme = wl.k_scheme if tensor == 0 else wl.v_scheme
        bits = wl.k_bits if tensor == 0 else wl.v_bits
        rotate = (wl.rotate_k if tensor == 0 else wl.rotate_v) or W.is_turbo(scheme)
        sink = wl.sinkhorn_iters > 0 and not W.is_turbo(scheme)
        cap = self.cache.cfg.max_context
        p = oracle.Plane(scheme, bits, rotate, sink, wl.window, tensor, cap)
        tb = tables or self.oracle_tables(li, head, tensor)
        X = self.kv(self.layers[li])[tensor][b, : (n or self.n), head].float().cpu().numpy()
        p.append(X, tb)
        return p, tb

    def device_plane(self, li, b, head, tensor):
        return [None if t is None else t.cpu().numpy() for t in
                self.cache.plane_bytes(li, b, head, tensor)]


def compare_plane(dev, orc: oracle.Plane, label=""):
    codes, meta, qjl, win = dev
    assert np.array_equal(codes, orc.codes), f"{label}: codes differ at {np.flatnonzero(codes != orc.codes)[:8]}"
    assert np.array_equal(meta, orc.meta), f"{label}: meta differ at {np.flatnonzero(meta != orc.meta)[:8]}"
    if qjl is not None:
        assert np.array_equal(qjl, orc.qjl[: qjl.size]), f"{label}: qjl bits differ"
    if win is not None:
        w = win.view(np.float32)
        assert np.array_equal(w.view(np.uint32), orc.ring.view(np.uint32)), f"{label}: window differs"


_CB16 = None
_CB64 = {}


def _codebook64(levels):
    if levels not in _CB64:
        _CB64[levels] = oracle.lloyd_max(oracle.LLOYD_ITERS, levels, 64)
    return _CB64[levels]


def _codebook16():
    global _CB16
    if _CB16 is None:
        _CB16 = oracle.lloyd_max(oracle.LLOYD_ITERS, 16)
    return _CB16


def oracle_attention_case(case: Case, li, b, q_np, n=None, planes=None):
    """Oracle output [Hq][128] for sequence b of layer li (planes rebuilt from the inputs)."""
    wl = case.wl
    G = wl.group
    out = np.zeros((wl.n_q_heads, 128))
    _, mu, theta, _ = oracle.lloyd_max(oracle.LLOYD_ITERS)
    for h in range(wl.n_kv_heads):
        if planes is not None:
            pk, tk, pv, tv = planes[h]
        else:
            pk, tk = case.oracle_plane(li, b, h, 0, case.oracle_tables(li, h, 0, mu, theta), n)
            pv, tv = case.oracle_plane(li, b, h, 1, case.oracle_tables(li, h, 1, mu, theta), n)
        out[h * G:(h + 1) * G] = oracle.attention(pk, pv, tk, tv, q_np[h * G:(h + 1) * G])
    return out
