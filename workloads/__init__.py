"""Seeded synthetic workloads for the compressed-KV decode path.

This module only draws random numbers and shapes them; it holds none of the method's
arithmetic.  Both the HIP path (tests, bench) and the CPU oracle take their inputs from here, and
the random tables the method draws (rotation signs, the QJL projection) are drawn here too and
passed to both sides as inputs.

Workloads are named for what they are (model shape, context, cache scheme).  The pages measure on
real models and text (quantcpp article: Llama 3.2 3B at 3970 tokens and 16K-128K contexts; KVarN
post: a 27B dense model at 120K context); these synthetic stand-ins keep those shapes and lengths
with the value distributions described per workload.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

UNIFORM, TURBO_QJL, TURBO_MSE, Q8_0, TURBO_SPLIT = 0, 1, 2, 3, 4
D = 128


def is_turbo(scheme: int) -> bool:
    """TurboQuant planes (rotation implied, Lloyd-Max codes); the others use the uniform layout."""
    return scheme in (TURBO_QJL, TURBO_MSE, TURBO_SPLIT)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    batch: int
    context: int
    k_scheme: int
    v_scheme: int
    k_bits: int
    v_bits: int
    window: int
    rotate_k: bool
    rotate_v: bool
    sinkhorn_iters: int
    calib_tokens: int
    dtype: str  # "f32", "bf16" or "f16" (values rounded to the 16-bit type, RN)
    data: str  # value recipe, see gen_kv
    seed: int

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw):
        return dataclasses.replace(self, **kw)

    def kvq_config(self, max_context: Optional[int] = None, max_batch: Optional[int] = None):
        """Field values of the library's kvq_config for this workload."""
        return dict(n_layers=self.n_layers, n_q_heads=self.n_q_heads, n_kv_heads=self.n_kv_heads,
                    head_dim=D, max_batch=max_batch or self.batch,
                    max_context=max_context or self.context, k_scheme=self.k_scheme,
                    v_scheme=self.v_scheme, k_bits=self.k_bits, v_bits=self.v_bits, group_size=32,
                    fp32_window=self.window, rotate_k=int(self.rotate_k),
                    rotate_v=int(self.rotate_v), sinkhorn_iters=self.sinkhorn_iters,
                    calib_tokens=self.calib_tokens)


# Llama-3.2-3B attention shape: 24 query heads, 8 KV heads, head_dim 128, 28 layers.
LLAMA3B_3970_PROGRESSIVE = Workload(
    "llama3b-1layer-3970-u4-progressive", 1, 24, 8, 1, 3970, UNIFORM, UNIFORM, 4, 4, 128,
    False, False, 0, 0, "f32", "outliers4x10", 1001)
LLAMA3B_32K_KVARN = Workload(
    "llama3b-28layer-32k-wht-sinkhorn-u4", 28, 24, 8, 1, 32768, UNIFORM, UNIFORM, 4, 4, 0,
    True, True, 5, 512, "f32", "loguniform_std", 1002)
LLAMA3B_32K_TURBO = Workload(
    "llama3b-28layer-32k-turboqjl-k-u4-v", 28, 24, 8, 1, 32768, TURBO_QJL, UNIFORM, 3, 4, 0,
    True, False, 0, 0, "f32", "outliers8x8", 1003)
LLAMA3B_32K_TURBO_ASYM = Workload(
    "llama3b-28layer-32k-u8-k-turbomse-v", 28, 24, 8, 1, 32768, UNIFORM, TURBO_MSE, 8, 3, 0,
    False, True, 0, 0, "f32", "outliers8x8", 1003)
LLAMA3B_128K_PROGRESSIVE = Workload(
    "llama3b-28layer-128k-u4-progressive", 28, 24, 8, 1, 131072, UNIFORM, UNIFORM, 4, 4, 128,
    False, False, 0, 0, "f32", "ar1_drift", 1004)
DENSE27B_120K_KVARN = Workload(
    "dense27b-64layer-120k-b4-wht-sinkhorn-u4", 64, 40, 8, 4, 122880, UNIFORM, UNIFORM, 4, 4, 0,
    True, True, 5, 512, "bf16", "student_t4", 1005)
DENSE27B_120K_U8 = Workload(
    "dense27b-64layer-120k-b4-u8", 64, 40, 8, 4, 122880, UNIFORM, UNIFORM, 8, 8, 0,
    False, False, 0, 0, "bf16", "student_t4", 1005)
# the KVarN post's q8_0 cache baseline on the 27B shape, and the survey page's application rule
# (K kept at Q8, only V cut to TurboQuant 3-bit)
DENSE27B_120K_Q8_0 = Workload(
    "dense27b-64layer-120k-b4-q8_0", 64, 40, 8, 4, 122880, Q8_0, Q8_0, 8, 8, 0,
    False, False, 0, 0, "bf16", "student_t4", 1005)
LLAMA3B_32K_Q8_0_TURBO_V = Workload(
    "llama3b-28layer-32k-q8_0-k-turbomse-v", 28, 24, 8, 1, 32768, Q8_0, TURBO_MSE, 8, 3, 0,
    False, True, 0, 0, "f32", "outliers8x8", 1003)
LLAMA3B_32K_Q8_0_TURBO4_V = Workload(
    "llama3b-28layer-32k-q8_0-k-turbo4mse-v", 28, 24, 8, 1, 32768, Q8_0, TURBO_MSE, 8, 4, 0,
    False, True, 0, 0, "f32", "outliers8x8", 1003)
# TurboQuant's fractional bit widths on the Llama-3.1-8B attention shape (32 layers, 32 query
# heads, 8 KV heads): V with the outlier-channel split at 2.5 bits (3 on the 64 outlier channels,
# 2 on the rest) and 3.5 bits (4 / 3), K kept at Q8; the outlier channels come from a 512-token
# calibration block of the same per-channel distribution
LLAMA8B_32K_Q8_0_TURBO25_V = Workload(
    "llama8b-32layer-32k-q8_0-k-turbo2.5split-v", 32, 32, 8, 1, 32768, Q8_0, TURBO_SPLIT, 8, 3, 0,
    False, True, 0, 512, "f32", "outliers8x8", 1006)
LLAMA8B_32K_Q8_0_TURBO35_V = Workload(
    "llama8b-32layer-32k-q8_0-k-turbo3.5split-v", 32, 32, 8, 1, 32768, Q8_0, TURBO_SPLIT, 8, 4, 0,
    False, True, 0, 512, "f32", "outliers8x8", 1006)

# 3-bit uniform group packing: the asymmetric variant with V cut to 3 bits (K kept at 8-bit
# groups), and the KVarN rotation + balancing in front of 3-bit K and V
LLAMA3B_32K_U8_K_U3_V = Workload(
    "llama3b-28layer-32k-u8-k-u3-v", 28, 24, 8, 1, 32768, UNIFORM, UNIFORM, 8, 3, 0,
    False, False, 0, 0, "f32", "outliers8x8", 1003)
LLAMA3B_32K_KVARN_U3 = Workload(
    "llama3b-28layer-32k-wht-sinkhorn-u3", 28, 24, 8, 1, 32768, UNIFORM, UNIFORM, 3, 3, 0,
    True, True, 5, 512, "f32", "loguniform_std", 1002)

# TurboQuant's 2.5 / 3.5-bit figures are for the whole KV cache: the outlier split on both
# tensors (K: split MSE codes + 1-bit QJL; V: split MSE codes), Llama-3.1-8B attention shape
LLAMA8B_32K_TURBO25_KV = Workload(
    "llama8b-32layer-32k-turbo2.5split-kv", 32, 32, 8, 1, 32768, TURBO_SPLIT, TURBO_SPLIT, 3, 3, 0,
    True, True, 0, 512, "f32", "outliers8x8", 1006)
LLAMA8B_32K_TURBO35_KV = Workload(
    "llama8b-32layer-32k-turbo3.5split-kv", 32, 32, 8, 1, 32768, TURBO_SPLIT, TURBO_SPLIT, 4, 4, 0,
    True, True, 0, 512, "f32", "outliers8x8", 1006)

ALL = [LLAMA3B_3970_PROGRESSIVE, LLAMA3B_32K_KVARN, LLAMA3B_32K_TURBO, LLAMA3B_32K_TURBO_ASYM,
       LLAMA3B_128K_PROGRESSIVE, DENSE27B_120K_KVARN, DENSE27B_120K_U8, DENSE27B_120K_Q8_0,
       LLAMA3B_32K_Q8_0_TURBO_V, LLAMA3B_32K_Q8_0_TURBO4_V, LLAMA8B_32K_Q8_0_TURBO25_V,
       LLAMA8B_32K_Q8_0_TURBO35_V, LLAMA3B_32K_U8_K_U3_V, LLAMA3B_32K_KVARN_U3, LLAMA8B_32K_TURBO25_KV,
       LLAMA8B_32K_TURBO35_KV]
BY_NAME = {w.name: w for w in ALL}

TAGS = {"kv": 1, "calib": 2, "q": 3, "signs": 4, "qjl": 5, "chan": 6, "step": 7}


def _seed(wl: Workload, tag: str, *idx: int) -> int:
    ss = np.random.SeedSequence([wl.seed, TAGS[tag], *[int(i) for i in idx]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _dtype(wl):
    return {"bf16": torch.bfloat16, "f16": torch.float16}.get(wl.dtype, torch.float32)


# ----------------------------------------------------------------------------------------------
# random tables the method draws (passed to both sides as inputs)
# ----------------------------------------------------------------------------------------------

def rotation_signs(wl: Workload) -> np.ndarray:
    """[n_layers][n_kv_heads][2 (K, V)][128] of +-1.0 (fp32), independent per (layer, head,
    tensor)."""
    rng = np.random.default_rng(_seed(wl, "signs"))
    bits = rng.integers(0, 2, size=(wl.n_layers, wl.n_kv_heads, 2, D))
    return np.where(bits == 1, -1.0, 1.0).astype(np.float32)


def qjl_projection(wl: Workload) -> np.ndarray:
    """[128][128] i.i.d. N(0,1) fp32: one QJL projection per cache."""
    return np.random.default_rng(_seed(wl, "qjl")).standard_normal((D, D)).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# K / V values
# ----------------------------------------------------------------------------------------------

def _channel_params(wl: Workload, layer: int, tensor: int):
    """Per-(head, channel) multiplier [n_kv_heads][128] for the recipe."""
    rng = np.random.default_rng(_seed(wl, "chan", layer, tensor))
    m = np.ones((wl.n_kv_heads, D), np.float64)
    if wl.data in ("outliers4x10", "outliers8x8"):
        k, f = (4, 10.0) if wl.data == "outliers4x10" else (8, 8.0)
        for h in range(wl.n_kv_heads):
            m[h, rng.choice(D, size=k, replace=False)] = f
    elif wl.data == "loguniform_std":
        m = np.exp(rng.uniform(math.log(0.1), math.log(10.0), size=(wl.n_kv_heads, D)))
    return m


def _ar1(eta: torch.Tensor, d0: torch.Tensor, rho: float, chunk: int = 512) -> torch.Tensor:
    """d_t = rho d_{t-1} + sqrt(1 - rho^2) eta_t along dim 1 of eta [B, T, ...], with d_{-1} = d0
    (a chunked linear scan: a lower-triangular Toeplitz product inside each chunk)."""
    B, T = eta.shape[0], eta.shape[1]
    rest = eta.shape[2:]
    cols = int(np.prod(rest)) if rest else 1
    c = math.sqrt(1.0 - rho * rho)
    k = torch.arange(chunk, device=eta.device, dtype=torch.float64)
    M = torch.tril(rho ** (k[:, None] - k[None, :]).clamp(min=0)) * c
    M = M.to(torch.float32)
    pw = (rho ** (k + 1)).to(torch.float32)[:, None]
    out = torch.empty_like(eta)
    prev = d0.reshape(B, cols).to(torch.float32)
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        L = e - s
        blk = eta[:, s:e].reshape(B, L, cols)
        val = torch.matmul(M[:L, :L], blk) + pw[:L] * prev[:, None, :]
        out[:, s:e] = val.reshape(B, L, *rest)
        prev = val[:, L - 1]
    return out


def gen_kv(wl: Workload, layer: int, tensor: int, n_tokens: Optional[int] = None,
           device="cpu", batch: Optional[int] = None) -> torch.Tensor:
    """Source K (tensor 0) or V (tensor 1) for one layer: [batch][n_tokens][n_kv_heads][128] in
    the workload's source dtype."""
    n = wl.context if n_tokens is None else n_tokens
    B = wl.batch if batch is None else batch
    g = _gen(device, _seed(wl, "kv", layer, tensor))
    shape = (B, n, wl.n_kv_heads, D)
    mult = torch.tensor(_channel_params(wl, layer, tensor), dtype=torch.float32, device=device)
    if wl.data == "student_t4":
        z = torch.randn(shape, generator=g, device=device)
        u1 = torch.rand(shape, generator=g, device=device).clamp_(min=1e-30)
        u2 = torch.rand(shape, generator=g, device=device).clamp_(min=1e-30)
        chi2 = -2.0 * torch.log(u1 * u2)
        x = z / torch.sqrt(chi2 / 4.0)
    elif wl.data == "ar1_drift":
        z = torch.randn(shape, generator=g, device=device)
        eta = torch.randn(shape, generator=g, device=device)
        d0 = torch.randn((B, wl.n_kv_heads, D), generator=g, device=device)
        x = z + _ar1(eta, d0, 0.99)
    else:
        x = torch.randn(shape, generator=g, device=device) * mult
    return x.to(_dtype(wl))


def gen_calib(wl: Workload, layer: int, tensor: int, device="cpu") -> torch.Tensor:
    """Separate 512-token calibration block [calib_tokens][n_kv_heads][128] from the same
    per-channel distribution as gen_kv."""
    n = wl.calib_tokens or 512
    g = _gen(device, _seed(wl, "calib", layer, tensor))
    mult = torch.tensor(_channel_params(wl, layer, tensor), dtype=torch.float32, device=device)
    shape = (n, wl.n_kv_heads, D)
    if wl.data == "student_t4":
        z = torch.randn(shape, generator=g, device=device)
        u1 = torch.rand(shape, generator=g, device=device).clamp_(min=1e-30)
        u2 = torch.rand(shape, generator=g, device=device).clamp_(min=1e-30)
        x = z / torch.sqrt(-2.0 * torch.log(u1 * u2) / 4.0)
    else:
        x = torch.randn(shape, generator=g, device=device) * mult
    return x.to(_dtype(wl))


def gen_step_kv(wl: Workload, layer: int, step: int, device="cpu", batch=None):
    """New K and V for one decode step: two [batch][n_kv_heads][128] tensors."""
    B = wl.batch if batch is None else batch
    g = _gen(device, _seed(wl, "step", layer, step))
    mk = torch.tensor(_channel_params(wl, layer, 0), dtype=torch.float32, device=device)
    mv = torch.tensor(_channel_params(wl, layer, 1), dtype=torch.float32, device=device)
    k = torch.randn((B, wl.n_kv_heads, D), generator=g, device=device) * mk
    v = torch.randn((B, wl.n_kv_heads, D), generator=g, device=device) * mv
    return k.to(_dtype(wl)), v.to(_dtype(wl))


def gen_q(wl: Workload, layer: int, step: int = 0, device="cpu", batch=None) -> torch.Tensor:
    """Decode queries [batch][n_q_heads][128] ~ N(0,1) in the workload's source dtype."""
    B = wl.batch if batch is None else batch
    g = _gen(device, _seed(wl, "q", layer, step))
    return torch.randn((B, wl.n_q_heads, D), generator=g, device=device).to(_dtype(wl))
