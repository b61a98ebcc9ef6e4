"""ctypes binding of libkvq (include/kvq.h): argument marshalling only.

Every function keeps the C name.  Tensors are PyTorch device tensors; only their data pointers,
shapes and dtypes cross into C.  Streams default to torch's current stream.  A non-OK status
raises KvqError.  Importing this module fails loudly when libkvq.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_F32, KVQ_BF16, KVQ_F16 = 0, 1, 2
KVQ_UNIFORM, KVQ_TURBO_QJL, KVQ_TURBO_MSE, KVQ_Q8_0, KVQ_TURBO_SPLIT = 0, 1, 2, 3, 4
KVQ_OPT_SPLIT_TOKENS, KVQ_OPT_DECODE_PATH = 1, 2
STATUS = {0: "KVQ_OK", 1: "KVQ_ERR_INVALID_ARG", 2: "KVQ_ERR_UNSUPPORTED", 3: "KVQ_ERR_CAPACITY",
          4: "KVQ_ERR_NOT_READY", 5: "KVQ_ERR_BUFFER_TOO_SMALL", 6: "KVQ_ERR_MISALIGNED",
          7: "KVQ_ERR_HOST_ALLOC", 8: "KVQ_ERR_DEVICE", 9: "KVQ_ERR_SCRATCH"}
KVQ_STATIC_SCRATCH_BYTES = 32 << 20
EXPORTS = ["kvq_cache_required_bytes", "kvq_cache_create", "kvq_cache_destroy",
           "kvq_set_random_tables", "kvq_derive_random_tables", "kvq_set_random_tables_seeded",
           "kvq_calibrate", "kvq_prefill_quantize", "kvq_append",
           "kvq_attn_decode", "kvq_get_layout", "kvq_get_tables", "kvq_set_option",
           "kvq_set_timing_events", "kvq_append_attn_decode", "kvq_attn_prefill",
           "kvq_attn_prefill_workspace", "kvq_attn_decode_static",
           "kvq_get_length", "kvq_status_str", "kvq_last_hip_error"]


class KvqError(RuntimeError):
    def __init__(self, status, fn=""):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{fn}: {self.name}")


class kvq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "max_batch", "max_context",
        "k_scheme", "v_scheme", "k_bits", "v_bits", "group_size", "fp32_window", "rotate_k",
        "rotate_v", "sinkhorn_iters", "calib_tokens")]


class kvq_layout(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p), ("qjl", ctypes.c_void_p),
                ("window", ctypes.c_void_p), ("codes_bytes", ctypes.c_size_t),
                ("meta_bytes", ctypes.c_size_t), ("qjl_bytes", ctypes.c_size_t),
                ("window_bytes", ctypes.c_size_t), ("length", ctypes.c_int)]


class kvq_tables(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("signs", "c", "inv_c", "qjl_S", "mu", "theta", "mu16",
                                              "theta16", "perm", "mu64", "theta64", "perm_k")]


_lib = None


def load():
    """Load libkvq.so (raises ImportError if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python quantized_decode_attention_kvq_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int
    sig = {
        "kvq_cache_required_bytes": [ctypes.POINTER(kvq_config), ctypes.POINTER(ctypes.c_size_t)],
        "kvq_cache_create": [ctypes.POINTER(kvq_config), vp, ctypes.c_size_t, vp,
                             ctypes.POINTER(vp)],
        "kvq_cache_destroy": [vp],
        "kvq_set_random_tables": [vp, vp, vp, vp],
        "kvq_derive_random_tables": [ctypes.c_ulonglong, i, i, vp, vp],
        "kvq_set_random_tables_seeded": [vp, ctypes.c_ulonglong, vp],
        "kvq_calibrate": [vp, i, vp, vp, i, i, vp],
        "kvq_prefill_quantize": [vp, i, vp, vp, i, i, i, vp],
        "kvq_append": [vp, i, vp, vp, i, i, vp],
        "kvq_attn_decode": [vp, i, vp, i, vp, i, f, vp],
        "kvq_attn_decode_static": [vp, i, vp, i, vp, i, f, vp],
        "kvq_append_attn_decode": [vp, i, vp, vp, vp, i, vp, i, f, vp],
        "kvq_attn_prefill": [vp, i, vp, i, vp, i, i, f, vp, ctypes.c_size_t, vp],
        "kvq_attn_prefill_workspace": [vp, i, i, i, ctypes.POINTER(ctypes.c_size_t)],
        "kvq_get_layout": [vp, i, i, i, i, ctypes.POINTER(kvq_layout)],
        "kvq_get_tables": [vp, ctypes.POINTER(kvq_tables)],
        "kvq_set_option": [vp, i, i],
        "kvq_set_timing_events": [vp, vp, vp],
        "kvq_get_length": [vp, i, i],
        "kvq_status_str": [i],
        "kvq_last_hip_error": [vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "kvq_status_str" else st
    _lib = L
    return L


def _check(status, fn):
    if status != 0:
        raise KvqError(status, fn)


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t):
    import torch
    if t.dtype == torch.float32:
        return KVQ_F32
    if t.dtype == torch.bfloat16:
        return KVQ_BF16
    if t.dtype == torch.float16:
        return KVQ_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


# Shapes each handle was created with: the C ABI takes raw pointers and no sizes, so the binding
# checks every tensor against them before a pointer crosses into C (a wrong shape or dtype would
# otherwise make a kernel read or write past the tensor).
_SHAPES = {}


def _dims(h):
    key = h.value if isinstance(h, ctypes.c_void_p) else h
    d = _SHAPES.get(key)
    if d is None:
        raise ValueError("unknown kvq handle (not created through this binding, or destroyed)")
    return d


def _tensor(t, name, shape, dtypes):
    """Checks one tensor argument's shape (None = any extent) and dtype."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dim() != len(shape) or any(e is not None and t.shape[i] != e for i, e in enumerate(shape)):
        want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    return t


def _resident(**named):
    """Every given tensor lives in device memory and is contiguous (the last check before C)."""
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError(f"{name} must be a device (cuda) tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _inputs():
    import torch
    return (torch.float32, torch.bfloat16, torch.float16)


def _same_dtype(*ts):
    ts = [t for t in ts if t is not None]
    if any(t.dtype != ts[0].dtype for t in ts):
        raise TypeError("all inputs of one call must share one dtype: " + ", ".join(str(t.dtype) for t in ts))


def _batch(h, B):
    if not 1 <= B <= _dims(h)["max_batch"]:
        raise ValueError(f"batch {B} outside 1 .. max_batch = {_dims(h)['max_batch']}")


def make_config(**kw) -> kvq_config:
    c = kvq_config()
    for k, v in kw.items():
        setattr(c, k, int(v))
    return c


def kvq_cache_required_bytes(cfg: kvq_config) -> int:
    n = ctypes.c_size_t(0)
    _check(load().kvq_cache_required_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "kvq_cache_required_bytes")
    return n.value


def kvq_cache_create(cfg: kvq_config, buf, stream=None):
    h = ctypes.c_void_p()
    nbytes = buf.numel() * buf.element_size()
    _resident(buf=buf)
    _check(load().kvq_cache_create(ctypes.byref(cfg), _ptr(buf), nbytes, _stream(stream),
                                   ctypes.byref(h)), "kvq_cache_create")
    _SHAPES[h.value] = {"n_layers": cfg.n_layers, "n_q_heads": cfg.n_q_heads,
                        "n_kv_heads": cfg.n_kv_heads, "max_batch": cfg.max_batch}
    return h


def kvq_cache_destroy(h):
    _check(load().kvq_cache_destroy(h), "kvq_cache_destroy")
    _SHAPES.pop(h.value if isinstance(h, ctypes.c_void_p) else h, None)


def kvq_set_random_tables(h, signs=None, qjl_S=None, stream=None):
    """signs: [n_layers][n_kv_heads][2][128] fp32; qjl_S: [128][128] fp32 (either may be None)."""
    import torch
    d = _dims(h)
    if signs is not None:
        _tensor(signs, "signs", (d["n_layers"], d["n_kv_heads"], 2, 128), (torch.float32,))
    if qjl_S is not None:
        _tensor(qjl_S, "qjl_S", (128, 128), (torch.float32,))
    _resident(signs=signs, qjl_S=qjl_S)
    _check(load().kvq_set_random_tables(h, _ptr(signs), _ptr(qjl_S), _stream(stream)),
           "kvq_set_random_tables")


def kvq_derive_random_tables(seed, n_layers, n_kv_heads):
    """Host-side draw of (signs [n_layers][n_kv_heads][2][128], S [128][128]) float32 numpy arrays
    from a 64-bit seed (no device work)."""
    import numpy as np
    signs = np.zeros((n_layers, n_kv_heads, 2, 128), np.float32)
    S = np.zeros((128, 128), np.float32)
    _check(load().kvq_derive_random_tables(seed, n_layers, n_kv_heads, signs.ctypes.data_as(ctypes.c_void_p),
                                           S.ctypes.data_as(ctypes.c_void_p)), "kvq_derive_random_tables")
    return signs, S


def kvq_set_random_tables_seeded(h, seed, stream=None):
    _check(load().kvq_set_random_tables_seeded(h, seed, _stream(stream)), "kvq_set_random_tables_seeded")


def kvq_calibrate(h, layer, Kc=None, Vc=None, stream=None):
    """Kc, Vc: [n_tokens][n_kv_heads][128] calibration tokens of one dtype (either may be None)."""
    d = _dims(h)
    if Kc is None and Vc is None:
        raise ValueError("kvq_calibrate needs Kc or Vc")
    for name, t in (("Kc", Kc), ("Vc", Vc)):
        if t is not None:
            _tensor(t, name, (None, d["n_kv_heads"], 128), _inputs())
    _same_dtype(Kc, Vc)
    if Kc is not None and Vc is not None and Kc.shape[0] != Vc.shape[0]:
        raise ValueError("Kc and Vc must hold the same number of tokens")
    _resident(Kc=Kc, Vc=Vc)
    t = Kc if Kc is not None else Vc
    _check(load().kvq_calibrate(h, layer, _ptr(Kc), _ptr(Vc), _dtype(t), t.shape[0],
                                _stream(stream)), "kvq_calibrate")


def kvq_prefill_quantize(h, layer, K, V, stream=None):
    """K, V: [batch][n_tokens][n_kv_heads][128], one dtype."""
    d = _dims(h)
    _tensor(K, "K", (None, None, d["n_kv_heads"], 128), _inputs())
    _tensor(V, "V", tuple(K.shape), _inputs())
    _same_dtype(K, V)
    _batch(h, K.shape[0])
    _resident(K=K, V=V)
    _check(load().kvq_prefill_quantize(h, layer, _ptr(K), _ptr(V), _dtype(K), K.shape[1],
                                       K.shape[0], _stream(stream)), "kvq_prefill_quantize")


def kvq_append(h, layer, k, v, stream=None):
    """k, v: [batch][n_kv_heads][128], one dtype."""
    d = _dims(h)
    _tensor(k, "k", (None, d["n_kv_heads"], 128), _inputs())
    _tensor(v, "v", tuple(k.shape), _inputs())
    _same_dtype(k, v)
    _batch(h, k.shape[0])
    _resident(k=k, v=v)
    _check(load().kvq_append(h, layer, _ptr(k), _ptr(v), _dtype(k), k.shape[0],
                             _stream(stream)), "kvq_append")


def _check_q_out(h, q, out, lead):
    import torch
    d = _dims(h)
    _tensor(q, "q", (*lead, d["n_q_heads"], 128), _inputs())
    _tensor(out, "out", tuple(q.shape), (torch.float32,))
    _batch(h, q.shape[0])


def kvq_attn_decode(h, layer, q, out, softmax_scale=0.0, stream=None):
    """q: [batch][n_q_heads][128]; out: [batch][n_q_heads][128] fp32."""
    _check_q_out(h, q, out, (None,))
    _resident(q=q, out=out)
    _check(load().kvq_attn_decode(h, layer, _ptr(q), _dtype(q), _ptr(out), q.shape[0],
                                  float(softmax_scale), _stream(stream)), "kvq_attn_decode")


def kvq_attn_decode_static(h, layer, q, out, softmax_scale=0.0, stream=None):
    """kvq_attn_decode with the split partials in the library's static device scratch."""
    _check_q_out(h, q, out, (None,))
    _resident(q=q, out=out)
    _check(load().kvq_attn_decode_static(h, layer, _ptr(q), _dtype(q), _ptr(out), q.shape[0],
                                         float(softmax_scale), _stream(stream)), "kvq_attn_decode_static")


def kvq_attn_prefill(h, layer, q, out, softmax_scale=0.0, workspace=None, stream=None):
    """q: [batch][n_q][Hq][128] (f32 or bf16), out: [batch][n_q][Hq][128] f32; workspace: a
    device tensor (any dtype, contiguous) or None for the cache's own."""
    _check_q_out(h, q, out, (None, None))
    _resident(q=q, out=out, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kvq_attn_prefill(h, layer, _ptr(q), _dtype(q), _ptr(out), q.shape[1], q.shape[0],
                                   float(softmax_scale), _ptr(workspace), ws_bytes, _stream(stream)),
           "kvq_attn_prefill")


def kvq_attn_prefill_workspace(h, layer, n_q, batch) -> int:
    n = ctypes.c_size_t(0)
    _check(load().kvq_attn_prefill_workspace(h, layer, n_q, batch, ctypes.byref(n)),
           "kvq_attn_prefill_workspace")
    return n.value


def kvq_append_attn_decode(h, layer, k, v, q, out, softmax_scale=0.0, stream=None):
    """k, v: [batch][n_kv_heads][128]; q: [batch][n_q_heads][128]; out: fp32 like q."""
    d = _dims(h)
    _check_q_out(h, q, out, (None,))
    _tensor(k, "k", (q.shape[0], d["n_kv_heads"], 128), _inputs())
    _tensor(v, "v", tuple(k.shape), _inputs())
    _same_dtype(k, v, q)
    _resident(k=k, v=v, q=q, out=out)
    _check(load().kvq_append_attn_decode(h, layer, _ptr(k), _ptr(v), _ptr(q), _dtype(q), _ptr(out),
                                         q.shape[0], float(softmax_scale), _stream(stream)),
           "kvq_append_attn_decode")


def kvq_get_layout(h, layer, seq, kv_head, tensor) -> kvq_layout:
    out = kvq_layout()
    _check(load().kvq_get_layout(h, layer, seq, kv_head, tensor, ctypes.byref(out)),
           "kvq_get_layout")
    return out


def kvq_get_tables(h) -> kvq_tables:
    out = kvq_tables()
    _check(load().kvq_get_tables(h, ctypes.byref(out)), "kvq_get_tables")
    return out


def kvq_set_option(h, option, value):
    _check(load().kvq_set_option(h, option, value), "kvq_set_option")


def kvq_set_timing_events(h, ev_start=None, ev_stop=None):
    """Events are torch.cuda.Event objects (their raw handles are passed) or None."""
    raw = [None if e is None else ctypes.c_void_p(e.cuda_event) for e in (ev_start, ev_stop)]
    _check(load().kvq_set_timing_events(h, *raw), "kvq_set_timing_events")


def kvq_get_length(h, layer, seq) -> int:
    return int(load().kvq_get_length(h, layer, seq))


def kvq_status_str(status) -> str:
    return load().kvq_status_str(status).decode()


def kvq_last_hip_error(h) -> int:
    return int(load().kvq_last_hip_error(h))
