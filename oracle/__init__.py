"""CPU oracle for the compressed-KV decode path (ctypes binding of kvq_oracle.c).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package.  The HIP library never imports, links or calls it,
and the two share no code.

Parity notes: every function here is pinned by ``tests/test_oracle_pins.py`` except the
Sinkhorn calibration's agreement with KVarN itself (the pages give no values), which is
"parity unpinned" beyond the invariants tested there.  The outlier split (TURBO_SPLIT) is pinned
by the 64-point Sylvester matrix, brute-force outlier ranking with ties, nearest-centroid codes,
the textbook 4-level codebook and distortions, and hand-derived layout words.  Uniform 3-bit
planes (three bit planes in the TurboQuant 3-bit byte layout, uniform fp16 scale/zero meta) are
pinned by the quantizer's error bound, brute-force nearest level and grid-point recovery at
L = 7, hand-derived K and V words, round trips, and lossless-grid attention against the textbook.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "libkvq_oracle.so")

UNIFORM, TURBO_QJL, TURBO_MSE, Q8_0, TURBO_SPLIT = 0, 1, 2, 3, 4
TENSOR_K, TENSOR_V = 0, 1
D = 128

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"], cwd=HERE)
        os.replace(tmp, LIB)
    return LIB


class PlaneCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("scheme", "bits", "rotate", "sinkhorn", "window", "tensor", "capacity")]


class Tables(ctypes.Structure):
    _fields_ = [(n, ctypes.POINTER(ctypes.c_float)) for n in
                ("signs", "c", "inv_c", "S", "mu", "theta", "mu2", "theta2")] + \
               [("perm", ctypes.POINTER(ctypes.c_int))]


_lib = None
_F = ctypes.POINTER(ctypes.c_float)
_Dp = ctypes.POINTER(ctypes.c_double)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_U16 = ctypes.POINTER(ctypes.c_uint16)
_I32 = ctypes.POINTER(ctypes.c_int)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        L.orc_f32_to_f16_rn.restype = ctypes.c_uint16
        L.orc_f32_to_f16_rn.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16_rd.restype = ctypes.c_uint16
        L.orc_f32_to_f16_rd.argtypes = [ctypes.c_float]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_rotate_f32.argtypes = [_F, _F, _F]
        L.orc_rotate_f64.argtypes = [_Dp, _F, _Dp]
        L.orc_unrotate_f64.argtypes = [_Dp, _F, _Dp]
        L.orc_sinkhorn.argtypes = [_F, ctypes.c_int, _F, ctypes.c_int, _F, _F, _Dp, _Dp]
        L.orc_quant_group.argtypes = [_F, ctypes.c_int, _U8, _U16, _U16]
        L.orc_quant_group_sym8.argtypes = [_F, _U8, _U16, _U16]
        L.orc_lloyd_max.argtypes = [ctypes.c_int, _Dp, _F, _F, _Dp]
        L.orc_lloyd_max_levels.argtypes = [ctypes.c_int, ctypes.c_int, _Dp, _F, _F, _Dp]
        L.orc_turbo_encode.argtypes = [_F, ctypes.POINTER(Tables), ctypes.c_int, _F, _U8, _U16,
                                       _U16, _U8, _F]
        L.orc_turbo_encode_bits.argtypes = [_F, ctypes.POINTER(Tables), ctypes.c_int, ctypes.c_int,
                                            _F, _U8, _U16, _U16, _U8, _F]
        L.orc_tree_sum_sq.restype = ctypes.c_float
        L.orc_tree_sum_sq.argtypes = [_F]
        L.orc_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.orc_stream_key.restype = ctypes.c_uint64
        L.orc_stream_draw.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.orc_stream_draw.restype = ctypes.c_uint64
        L.orc_box_muller.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.orc_box_muller.restype = ctypes.c_double
        L.orc_derive_tables.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, _F, _F]
        L.orc_lloyd_max_dim.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _Dp, _F, _F, _Dp]
        L.orc_rotate64_f32.argtypes = [_F, _F, _F]
        L.orc_unrotate64_f64.argtypes = [_Dp, _F, _Dp]
        L.orc_tree_sum_sq64.restype = ctypes.c_float
        L.orc_tree_sum_sq64.argtypes = [_F]
        L.orc_select_outliers.argtypes = [_F, ctypes.c_int, _I32]
        L.orc_split_encode.argtypes = [_F, ctypes.POINTER(Tables), ctypes.c_int, _U8, _U16]
        L.orc_split_qjl_encode.argtypes = [_F, ctypes.POINTER(Tables), ctypes.c_int, _U8, _U16, _U16, _U8]
        L.orc_split_rotate_f64.argtypes = [_Dp, ctypes.POINTER(Tables), _Dp]
        L.orc_split_score.restype = ctypes.c_double
        L.orc_split_score.argtypes = [ctypes.POINTER(PlaneCfg), ctypes.POINTER(Tables), _U8, _U8, _U8,
                                      ctypes.c_int, _Dp, _Dp]
        for f in ("orc_codes_bytes", "orc_meta_bytes", "orc_qjl_bytes", "orc_ring_floats"):
            getattr(L, f).restype = ctypes.c_size_t
            getattr(L, f).argtypes = [ctypes.POINTER(PlaneCfg)]
        L.orc_plane_append.argtypes = [ctypes.POINTER(PlaneCfg), ctypes.POINTER(Tables), _F,
                                       ctypes.c_int, ctypes.c_int, _U8, _U8, _U8, _F]
        L.orc_plane_read.argtypes = [ctypes.POINTER(PlaneCfg), _U8, _U8, _U8, ctypes.c_int, _U8,
                                     _U16, _U8]
        L.orc_dequant_token.argtypes = [ctypes.POINTER(PlaneCfg), ctypes.POINTER(Tables), _U8,
                                        _U8, ctypes.c_int, _Dp]
        L.orc_turbo_score.restype = ctypes.c_double
        L.orc_turbo_score.argtypes = [ctypes.POINTER(Tables), _U8, _U8, _U8, ctypes.c_int, _Dp,
                                      _Dp]
        L.orc_attention.argtypes = [ctypes.POINTER(PlaneCfg), ctypes.POINTER(PlaneCfg),
                                    ctypes.POINTER(Tables), ctypes.POINTER(Tables), _U8, _U8, _U8,
                                    _F, _U8, _U8, _F, ctypes.c_int, ctypes.c_int, _F,
                                    ctypes.c_double, _Dp]
        L.orc_attention_prefix.argtypes = [ctypes.POINTER(PlaneCfg), ctypes.POINTER(PlaneCfg),
                                           ctypes.POINTER(Tables), ctypes.POINTER(Tables), _U8,
                                           _U8, _U8, _F, _U8, _U8, _F, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, _F, ctypes.c_double, _Dp]
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t) if a is not None else None


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ----------------------------------------------------------------------------------------------
# scalar / vector helpers
# ----------------------------------------------------------------------------------------------

def f32_to_f16_rn(x: float) -> int:
    return int(lib().orc_f32_to_f16_rn(float(np.float32(x))))


def f32_to_f16_rd(x: float) -> int:
    return int(lib().orc_f32_to_f16_rd(float(np.float32(x))))


def f16_to_f32(h: int) -> float:
    return float(lib().orc_f16_to_f32(int(h)))


def rotate_f32(x, signs):
    x, s = _f32(x), _f32(signs)
    y = np.empty(D, np.float32)
    lib().orc_rotate_f32(_p(x, _F), _p(s, _F), _p(y, _F))
    return y


def rotate_f64(x, signs):
    x, s = np.ascontiguousarray(x, np.float64), _f32(signs)
    y = np.empty(D, np.float64)
    lib().orc_rotate_f64(_p(x, _Dp), _p(s, _F), _p(y, _Dp))
    return y


def unrotate_f64(y, signs):
    y, s = np.ascontiguousarray(y, np.float64), _f32(signs)
    x = np.empty(D, np.float64)
    lib().orc_unrotate_f64(_p(y, _Dp), _p(s, _F), _p(x, _Dp))
    return x


def sinkhorn(X, signs=None, iters=5, want_internals=False):
    X = _f32(X)
    n = X.shape[0]
    c = np.empty(D, np.float32)
    inv_c = np.empty(D, np.float32)
    A = np.empty((n, D), np.float64) if want_internals else None
    C = np.empty(D, np.float64) if want_internals else None
    s = _f32(signs) if signs is not None else None
    lib().orc_sinkhorn(_p(X, _F), n, _p(s, _F), iters, _p(c, _F), _p(inv_c, _F), _p(A, _Dp),
                       _p(C, _Dp))
    if want_internals:
        return c, inv_c, A, C
    return c, inv_c


def quant_group(y, bits):
    y = _f32(y)
    codes = np.empty(32, np.uint8)
    s16 = np.zeros(1, np.uint16)
    z16 = np.zeros(1, np.uint16)
    lib().orc_quant_group(_p(y, _F), bits, _p(codes, _U8), _p(s16, _U16), _p(z16, _U16))
    return codes, int(s16[0]), int(z16[0])


def quant_group_sym8(y):
    """Symmetric 8-bit ("q8_0") group quantizer: (codes q + 128, fp16 bits of d, of -128 d)."""
    y = _f32(y)
    codes = np.empty(32, np.uint8)
    d16 = np.zeros(1, np.uint16)
    z16 = np.zeros(1, np.uint16)
    lib().orc_quant_group_sym8(_p(y, _F), _p(codes, _U8), _p(d16, _U16), _p(z16, _U16))
    return codes, int(d16[0]), int(z16[0])


def lloyd_max(iters=2000, levels=8, dim=128):
    """Lloyd-Max codebook of N(0,1) with `levels` (4, 8 or 16) levels: (mu*, mu = mu*/sqrt(dim) in
    fp32, thresholds in fp32, last change of the iteration)."""
    mu_star = np.empty(levels, np.float64)
    mu = np.empty(levels, np.float32)
    theta = np.empty(levels - 1, np.float32)
    ch = np.zeros(1, np.float64)
    lib().orc_lloyd_max_dim(levels, dim, iters, _p(mu_star, _Dp), _p(mu, _F), _p(theta, _F), _p(ch, _Dp))
    return mu_star, mu, theta, float(ch[0])


def rotate64_f32(x, signs):
    x, s = _f32(x), _f32(signs)
    y = np.empty(64, np.float32)
    lib().orc_rotate64_f32(_p(x, _F), _p(s, _F), _p(y, _F))
    return y


def unrotate64_f64(y, signs):
    y, s = np.ascontiguousarray(y, np.float64), _f32(signs)
    x = np.empty(64, np.float64)
    lib().orc_unrotate64_f64(_p(y, _Dp), _p(s, _F), _p(x, _Dp))
    return x


def tree_sum_sq64(v):
    v = _f32(v)
    return float(lib().orc_tree_sum_sq64(_p(v, _F)))


def select_outliers(X):
    """Outlier split permutation of calibration tokens X [n][128]: the 64 channels of largest
    energy ascending, then the other 64 ascending (int32 [128])."""
    X = _f32(X).reshape(-1, D)
    perm = np.empty(D, np.int32)
    lib().orc_select_outliers(_p(X, _F), X.shape[0], _p(perm, _I32))
    return perm


def split_encode(x, tables: "TableSet", bits_o):
    """Split token code: (codes by position [128], (n_outlier, n_rest) fp16 bits)."""
    x = _f32(x)
    codes = np.empty(D, np.uint8)
    n16 = np.zeros(2, np.uint16)
    lib().orc_split_encode(_p(x, _F), tables.ref, int(bits_o), _p(codes, _U8), _p(n16, _U16))
    return codes, (int(n16[0]), int(n16[1]))


def split_qjl_encode(x, tables: "TableSet", b):
    """Split key code at b = 3 / 4: codes by position, (n_outlier, n_rest), gamma (fp16 bits) and
    the 128 QJL bits of the residual."""
    x = _f32(x)
    codes = np.empty(D, np.uint8)
    n16 = np.zeros(2, np.uint16)
    g16 = np.zeros(1, np.uint16)
    bits = np.zeros(D, np.uint8)
    lib().orc_split_qjl_encode(_p(x, _F), tables.ref, int(b), _p(codes, _U8), _p(n16, _U16),
                               _p(g16, _U16), _p(bits, _U8))
    return dict(codes=codes, n16=(int(n16[0]), int(n16[1])), g16=int(g16[0]), bits=bits)


def split_rotate_f64(q, tables: "TableSet"):
    """The split domain of q in binary64 (position 64h + j = R64(q[perm[64h + .]])_j)."""
    q = np.ascontiguousarray(q, np.float64)
    y = np.empty(D, np.float64)
    lib().orc_split_rotate_f64(_p(q, _Dp), tables.ref, _p(y, _Dp))
    return y


def split_score(plane: "Plane", tables: "TableSet", t, rho_q, s_rho_q):
    """Split-key score estimate of token t of a split K plane (unscaled, fp64)."""
    rq = np.ascontiguousarray(rho_q, np.float64)
    sq = np.ascontiguousarray(s_rho_q, np.float64)
    return float(lib().orc_split_score(plane.ref, tables.ref, _p(plane.codes, _U8), _p(plane.meta, _U8),
                                       _p(plane.qjl, _U8), int(t), _p(rq, _Dp), _p(sq, _Dp)))


LLOYD_ITERS = 2000  # fixed iteration count of the codebook (same count on the device side)


class TableSet:
    """Keeps numpy arrays alive behind an orc_tables struct."""

    def __init__(self, signs=None, c=None, inv_c=None, S=None, mu=None, theta=None, mu2=None,
                 theta2=None, perm=None):
        self.arrays = {}
        self.struct = Tables()
        for name, val in (("signs", signs), ("c", c), ("inv_c", inv_c), ("S", S), ("mu", mu),
                          ("theta", theta), ("mu2", mu2), ("theta2", theta2)):
            if val is not None:
                a = _f32(val).ravel()
                self.arrays[name] = a
                setattr(self.struct, name, _p(a, _F))
        if perm is not None:
            a = np.ascontiguousarray(perm, np.int32).ravel()
            assert a.size == D and np.array_equal(np.sort(a), np.arange(D)), "perm must permute 0..127"
            self.arrays["perm"] = a
            self.struct.perm = _p(a, _I32)

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def turbo_encode(x, tables: TableSet, with_qjl=True, bits=3):
    x = _f32(x)
    rho = np.empty(D, np.float32)
    resid = np.empty(D, np.float32)
    codes = np.empty(D, np.uint8)
    qbits = np.zeros(D, np.uint8)
    n16 = np.zeros(1, np.uint16)
    g16 = np.zeros(1, np.uint16)
    lib().orc_turbo_encode_bits(_p(x, _F), tables.ref, int(bits), int(with_qjl), _p(rho, _F),
                                _p(codes, _U8), _p(n16, _U16), _p(g16, _U16), _p(qbits, _U8),
                                _p(resid, _F))
    return dict(rho=rho, codes=codes, n16=int(n16[0]), g16=int(g16[0]), bits=qbits, resid=resid)


def tree_sum_sq(v):
    v = _f32(v)
    return float(lib().orc_tree_sum_sq(_p(v, _F)))


# ----------------------------------------------------------------------------------------------
# planes
# ----------------------------------------------------------------------------------------------

class Plane:
    """One (layer, sequence, kv head, tensor) plane: code bytes, meta bytes, QJL bytes, ring."""

    def __init__(self, scheme, bits, rotate, sinkhorn, window, tensor, capacity):
        self.cfg = PlaneCfg(scheme, bits, int(rotate or scheme in (TURBO_QJL, TURBO_MSE, TURBO_SPLIT)), int(sinkhorn), window,
                            tensor, capacity)
        L = lib()
        r = ctypes.byref(self.cfg)
        self.codes = np.zeros(L.orc_codes_bytes(r), np.uint8)
        self.meta = np.zeros(L.orc_meta_bytes(r), np.uint8)
        self.qjl = np.zeros(max(1, L.orc_qjl_bytes(r)), np.uint8)
        self.ring = np.zeros(max(1, L.orc_ring_floats(r)), np.float32)
        self.length = 0

    @property
    def ref(self):
        return ctypes.byref(self.cfg)

    def append(self, X, tables: TableSet):
        X = _f32(X).reshape(-1, D)
        n = X.shape[0]
        if self.length + n > self.cfg.capacity:
            raise ValueError("oracle plane capacity exceeded")
        lib().orc_plane_append(self.ref, tables.ref, _p(X, _F), self.length, n,
                               _p(self.codes, _U8), _p(self.meta, _U8), _p(self.qjl, _U8),
                               _p(self.ring, _F))
        self.length += n

    def read(self, t):
        code = np.empty(D, np.uint8)
        meta8 = np.empty(8, np.uint16)
        bits = np.zeros(D, np.uint8)
        lib().orc_plane_read(self.ref, _p(self.codes, _U8), _p(self.meta, _U8), _p(self.qjl, _U8),
                             t, _p(code, _U8), _p(meta8, _U16), _p(bits, _U8))
        return code, meta8, bits

    def dequant(self, t, tables: TableSet):
        out = np.empty(D, np.float64)
        lib().orc_dequant_token(self.ref, tables.ref, _p(self.codes, _U8), _p(self.meta, _U8), t,
                                _p(out, _Dp))
        return out

    def turbo_score(self, t, tables: TableSet, rho_q, s_rho_q):
        rq = np.ascontiguousarray(rho_q, np.float64)
        srq = np.ascontiguousarray(s_rho_q, np.float64)
        return float(lib().orc_turbo_score(tables.ref, _p(self.codes, _U8), _p(self.meta, _U8),
                                           _p(self.qjl, _U8), t, _p(rq, _Dp), _p(srq, _Dp)))


def attention(kplane: Plane, vplane: Plane, ktables: TableSet, vtables: TableSet, q, n=None,
              scale=None):
    """fp64 decode attention of G = q.shape[0] query heads over one kv head's planes."""
    q = _f32(q).reshape(-1, D)
    G = q.shape[0]
    n = kplane.length if n is None else n
    scale = 1.0 / np.sqrt(128.0) if scale is None or scale <= 0 else float(scale)
    out = np.empty((G, D), np.float64)
    lib().orc_attention(kplane.ref, vplane.ref, ktables.ref, vtables.ref,
                        _p(kplane.codes, _U8), _p(kplane.meta, _U8), _p(kplane.qjl, _U8),
                        _p(kplane.ring, _F), _p(vplane.codes, _U8), _p(vplane.meta, _U8),
                        _p(vplane.ring, _F), n, G, _p(q, _F), scale, _p(out, _Dp))
    return out


def attention_prefix(kplane: Plane, vplane: Plane, ktables: TableSet, vtables: TableSet, q,
                     n_vis, scale=None):
    """fp64 attention of G = q.shape[0] query heads over tokens 0 .. n_vis - 1 of the cache as it
    stands (the FP32 window is chosen by the cache length): one query of a prefill chunk."""
    q = _f32(q).reshape(-1, D)
    G = q.shape[0]
    scale = 1.0 / np.sqrt(128.0) if scale is None or scale <= 0 else float(scale)
    out = np.empty((G, D), np.float64)
    lib().orc_attention_prefix(kplane.ref, vplane.ref, ktables.ref, vtables.ref,
                               _p(kplane.codes, _U8), _p(kplane.meta, _U8), _p(kplane.qjl, _U8),
                               _p(kplane.ring, _F), _p(vplane.codes, _U8), _p(vplane.meta, _U8),
                               _p(vplane.ring, _F), kplane.length, int(n_vis), G, _p(q, _F), scale,
                               _p(out, _Dp))
    return out


# ---- seeded random tables (counter-based SplitMix64 + Box-Muller; see kvq_oracle.c) ----------
def stream_key(seed: int, tag: int, layer: int, head: int, tensor: int) -> int:
    return int(lib().orc_stream_key(seed, tag, layer, head, tensor))


def stream_draw(key: int, i: int) -> int:
    return int(lib().orc_stream_draw(key, i))


def box_muller(x1: int, x2: int) -> float:
    return float(lib().orc_box_muller(x1, x2))


def derive_random_tables(seed: int, n_layers: int, n_kv_heads: int):
    """(signs [n_layers][n_kv_heads][2][128] of +-1, S [128][128]) float32 from a 64-bit seed."""
    signs = np.zeros((n_layers, n_kv_heads, 2, D), np.float32)
    S = np.zeros((D, D), np.float32)
    lib().orc_derive_tables(seed, n_layers, n_kv_heads, _p(signs, _F), _p(S, _F))
    return signs, S
