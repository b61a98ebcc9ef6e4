"""MI355X-native compressed KV cache with fused decode attention (Python side of libkvq).

The compute path is the HIP library libkvq.so behind the C ABI in include/kvq.h; this package
only marshals arguments (``_kvq``) and offers ``KvCache``, a small owner of the device buffer and
the handle.  It raises ImportError when libkvq.so is missing; there is no CPU fallback.
"""
from __future__ import annotations

import torch

from . import _kvq
from ._kvq import *  # noqa: F401,F403  (the C-named functions and structs)
from ._kvq import KvqError, kvq_config, kvq_layout, make_config

_kvq.load()

__all__ = list(_kvq.EXPORTS) + ["KvCache", "KvqError", "make_config", "kvq_config", "kvq_layout"]


class KvCache:
    """Owns one device buffer (a torch uint8 tensor) and the kvq_cache handle bound to it."""

    def __init__(self, device="cuda", stream=None, **cfg):
        self.cfg = make_config(**{"head_dim": 128, "group_size": 32, **cfg})
        self.nbytes = _kvq.kvq_cache_required_bytes(self.cfg)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.handle = _kvq.kvq_cache_create(self.cfg, self.buf, stream)

    def close(self):
        if self.handle is not None:
            _kvq.kvq_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # thin forwards -----------------------------------------------------------------------------
    def set_random_tables(self, signs=None, qjl_S=None, stream=None):
        _kvq.kvq_set_random_tables(self.handle, signs, qjl_S, stream)

    def set_random_tables_seeded(self, seed, stream=None):
        _kvq.kvq_set_random_tables_seeded(self.handle, seed, stream)

    def calibrate(self, layer, Kc=None, Vc=None, stream=None):
        _kvq.kvq_calibrate(self.handle, layer, Kc, Vc, stream)

    def prefill_quantize(self, layer, K, V, stream=None):
        _kvq.kvq_prefill_quantize(self.handle, layer, K, V, stream)

    def append(self, layer, k, v, stream=None):
        _kvq.kvq_append(self.handle, layer, k, v, stream)

    def attn_decode(self, layer, q, out, softmax_scale=0.0, stream=None):
        _kvq.kvq_attn_decode(self.handle, layer, q, out, softmax_scale, stream)

    def attn_decode_static(self, layer, q, out, softmax_scale=0.0, stream=None):
        _kvq.kvq_attn_decode_static(self.handle, layer, q, out, softmax_scale, stream)

    def append_attn_decode(self, layer, k, v, q, out, softmax_scale=0.0, stream=None):
        _kvq.kvq_append_attn_decode(self.handle, layer, k, v, q, out, softmax_scale, stream)

    def attn_prefill(self, layer, q, out, softmax_scale=0.0, stream=None, workspace="auto"):
        """workspace: "auto" (a device buffer of kvq_attn_prefill_workspace bytes, kept on this
        object and grown when a call needs more), None (the cache's own), or a device tensor."""
        if isinstance(workspace, str):
            need = _kvq.kvq_attn_prefill_workspace(self.handle, layer, q.shape[1], q.shape[0])
            ws = getattr(self, "_prefill_ws", None)
            if need and (ws is None or ws.numel() < need):
                import torch
                ws = torch.empty(need, dtype=torch.uint8, device=self.buf.device)
                self._prefill_ws = ws
            workspace = ws if need else None
        _kvq.kvq_attn_prefill(self.handle, layer, q, out, softmax_scale, workspace, stream)

    def attn_prefill_workspace(self, layer, n_q, batch):
        return _kvq.kvq_attn_prefill_workspace(self.handle, layer, n_q, batch)

    def set_option(self, option, value):
        _kvq.kvq_set_option(self.handle, option, value)

    def set_timing_events(self, ev_start=None, ev_stop=None):
        """torch.cuda.Event objects that already exist on the device (record each once first)."""
        _kvq.kvq_set_timing_events(self.handle, ev_start, ev_stop)

    def length(self, layer, seq=0):
        return _kvq.kvq_get_length(self.handle, layer, seq)

    # views of device memory (for inspection and tests) ------------------------------------------
    def _slice(self, ptr, nbytes):
        off = ptr - self.buf.data_ptr()
        return self.buf[off:off + nbytes]

    def plane_bytes(self, layer, seq, kv_head, tensor):
        """(codes, meta, qjl, window) uint8 device tensors of one plane (qjl/window may be None)."""
        lay = _kvq.kvq_get_layout(self.handle, layer, seq, kv_head, tensor)
        codes = self._slice(lay.codes, lay.codes_bytes)
        meta = self._slice(lay.meta, lay.meta_bytes)
        qjl = self._slice(lay.qjl, lay.qjl_bytes) if lay.qjl_bytes else None
        win = self._slice(lay.window, lay.window_bytes) if lay.window_bytes else None
        return codes, meta, qjl, win

    def table(self, name, count):
        """Device view of one table: fp32 for signs, c, inv_c, qjl_S, mu, theta, mu16, theta16, mu64,
        theta64; int32 for perm and perm_k (the split V's / K's position -> channel maps)."""
        t = _kvq.kvq_get_tables(self.handle)
        return self._slice(getattr(t, name), 4 * count).view(torch.int32 if name in ("perm", "perm_k") else torch.float32)
