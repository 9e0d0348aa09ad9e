"""Python binding of libgsa, the MI355X Global Sparse Attention forward library.

Argument marshalling only: every function forwards device pointers, sizes and
the current HIP stream to the C ABI declared in ``include/gsa.h`` and raises
``GSAError`` on a non-zero status.  All arithmetic runs in the library's HIP
kernels; there is no fallback path.  If ``libgsa.so`` has not been built the
import fails.

Tensors may be torch tensors (their ``data_ptr()`` is passed) or raw integer
device addresses.  ``stream=None`` means torch's current stream on the current
device.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libgsa.so not found at {LIB_PATH}; build it with "
                      "`python sparse_global_attention_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

GSA_OK, GSA_ERR_INVALID_ARG, GSA_ERR_SHAPE, GSA_ERR_UNSUPPORTED, GSA_ERR_WORKSPACE, GSA_ERR_HIP = range(6)
GSA_BF16, GSA_F32 = 0, 1
GSA_OP_FORWARD, GSA_OP_SPECIAL, GSA_OP_SELECT, GSA_OP_DENSE, GSA_OP_COMPRESSED, GSA_OP_BACKWARD = range(6)
GSA_MAX_CTX_FRAMES = 16

EXPORTS = ("gsa_workspace_size", "gsa_pool", "gsa_compressed_attn_topk", "gsa_select_attn",
           "gsa_special_attn", "gsa_gate_combine", "gsa_forward", "gsa_dense_attn", "gsa_frame_attn",
           "gsa_descriptor_count", "gsa_descriptor_set", "gsa_descriptor_attn", "gsa_backward",
           "gsa_train_state_size", "gsa_forward_train", "gsa_backward_train", "gsa_forward_noalloc",
           "gsa_status_string")
GSA_NOALLOC_SCRATCH_BYTES = 256 << 20


class GSAConfig(ctypes.Structure):
    _fields_ = [("n_frames", ctypes.c_int32), ("n_special", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("pool", ctypes.c_int32), ("topk", ctypes.c_int32), ("n_ctx_frames", ctypes.c_int32),
                ("ctx_frames", ctypes.c_int32 * GSA_MAX_CTX_FRAMES), ("ctx_exclude_from_topk", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]

    @classmethod
    def make(cls, n_frames, n_special, grid_h, grid_w, n_heads, head_dim, pool, topk, dtype=GSA_BF16,
             ctx_frames=(), ctx_exclude_from_topk=1, scale=0.0):
        c = cls()
        c.n_frames, c.n_special, c.grid_h, c.grid_w = n_frames, n_special, grid_h, grid_w
        c.n_heads, c.head_dim, c.pool, c.topk = n_heads, head_dim, pool, topk
        if len(ctx_frames) > GSA_MAX_CTX_FRAMES:
            raise ValueError("at most 16 context frames")
        c.n_ctx_frames = len(ctx_frames)
        for i, f in enumerate(ctx_frames):
            c.ctx_frames[i] = f
        c.ctx_exclude_from_topk = ctx_exclude_from_topk
        c.scale = scale
        c.dtype = dtype
        return c

    @classmethod
    def from_shape(cls, sh, **overrides):
        """From any object with the GSA shape attributes (n_frames, n_special, ...)."""
        kw = dict(n_frames=sh.n_frames, n_special=sh.n_special, grid_h=sh.grid_h, grid_w=sh.grid_w,
                  n_heads=sh.n_heads, head_dim=sh.head_dim, pool=sh.pool, topk=sh.topk, dtype=sh.dtype,
                  ctx_frames=tuple(sh.ctx_frames), ctx_exclude_from_topk=sh.ctx_exclude)
        kw.update(overrides)
        return cls.make(**kw)


class GSAError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {gsa_status_string(status)}")


_P = ctypes.c_void_p
_CFG = ctypes.POINTER(GSAConfig)
_sig = {
    "gsa_workspace_size": [_CFG, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)],
    "gsa_pool": [_CFG, _P, _P, _P, _P, _P, _P, _P],
    "gsa_compressed_attn_topk": [_CFG, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "gsa_select_attn": [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "gsa_special_attn": [_CFG, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "gsa_gate_combine": [_CFG, _P, _P, _P, _P, _P, _P, _P],
    "gsa_forward": [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "gsa_dense_attn": [_CFG, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "gsa_frame_attn": [_CFG, _P, _P, _P, _P, _P],
    "gsa_descriptor_count": [_CFG, ctypes.POINTER(ctypes.c_int64)],
    "gsa_descriptor_set": [_CFG, _P, _P, _P, _P, _P],
    "gsa_descriptor_attn": [_CFG, _P, _P, _P, _P, _P],
    "gsa_backward": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "gsa_train_state_size": [_CFG, ctypes.POINTER(ctypes.c_size_t)],
    "gsa_forward_train": [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P],
    "gsa_backward_train": [_CFG, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                           _P],
    "gsa_forward_noalloc": [_CFG, _P, _P, _P, _P, _P, _P],
}
for _name, _args in _sig.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = ctypes.c_int
_lib.gsa_status_string.argtypes = [ctypes.c_int]
_lib.gsa_status_string.restype = ctypes.c_char_p


def gsa_status_string(status: int) -> str:
    return _lib.gsa_status_string(status).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _nbytes(x):
    if x is None:
        return 0
    return x.numel() * x.element_size()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, fn: str):
    if status != GSA_OK:
        raise GSAError(status, fn)


def gsa_workspace_size(cfg: GSAConfig, op: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.gsa_workspace_size(ctypes.byref(cfg), op, ctypes.byref(out)), "gsa_workspace_size")
    return out.value


def gsa_pool(cfg, q, k, v, qc, kc, vc, stream=None):
    _check(_lib.gsa_pool(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(qc), _ptr(kc), _ptr(vc),
                         _stream(stream)), "gsa_pool")


def gsa_compressed_attn_topk(cfg, qc, kc, vc, oc, topk_idx, topk_score, ws, ws_bytes=None, stream=None):
    wsb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(_lib.gsa_compressed_attn_topk(ctypes.byref(cfg), _ptr(qc), _ptr(kc), _ptr(vc), _ptr(oc),
                                         _ptr(topk_idx), _ptr(topk_score), _ptr(ws), wsb, _stream(stream)),
           "gsa_compressed_attn_topk")


def gsa_select_attn(cfg, q, k, v, topk_idx, o_sel, ws, ws_bytes=None, stream=None):
    wsb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(_lib.gsa_select_attn(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(o_sel),
                                _ptr(ws), wsb, _stream(stream)), "gsa_select_attn")


def gsa_special_attn(cfg, q, k, v, o, ws, ws_bytes=None, stream=None):
    wsb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(_lib.gsa_special_attn(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(ws), wsb,
                                 _stream(stream)), "gsa_special_attn")


def gsa_gate_combine(cfg, q, wg, gate, oc, o_sel, o, stream=None):
    _check(_lib.gsa_gate_combine(ctypes.byref(cfg), _ptr(q), _ptr(wg), _ptr(gate), _ptr(oc), _ptr(o_sel),
                                 _ptr(o), _stream(stream)), "gsa_gate_combine")


def gsa_forward(cfg, q, k, v, wg, o, ws, ws_bytes=None, stream=None):
    wsb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(_lib.gsa_forward(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(wg), _ptr(o), _ptr(ws), wsb,
                            _stream(stream)), "gsa_forward")


def gsa_dense_attn(cfg, q, k, v, o, ws=None, ws_bytes=None, stream=None):
    wsb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(_lib.gsa_dense_attn(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(ws), wsb,
                               _stream(stream)), "gsa_dense_attn")


def gsa_frame_attn(cfg, q, k, v, o, stream=None):
    _check(_lib.gsa_frame_attn(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _stream(stream)),
           "gsa_frame_attn")


def gsa_descriptor_count(cfg) -> int:
    out = ctypes.c_int64(0)
    _check(_lib.gsa_descriptor_count(ctypes.byref(cfg), ctypes.byref(out)), "gsa_descriptor_count")
    return out.value


def gsa_descriptor_set(cfg, k, v, kd, vd, stream=None):
    _check(_lib.gsa_descriptor_set(ctypes.byref(cfg), _ptr(k), _ptr(v), _ptr(kd), _ptr(vd), _stream(stream)),
           "gsa_descriptor_set")


def gsa_descriptor_attn(cfg, q, kd, vd, o, stream=None):
    _check(_lib.gsa_descriptor_attn(ctypes.byref(cfg), _ptr(q), _ptr(kd), _ptr(vd), _ptr(o), _stream(stream)),
           "gsa_descriptor_attn")


def gsa_backward(cfg, q, k, v, wg, topk_idx, d_o, dq, dk, dv, dwg, ws, ws_bytes=None, stream=None):
    wsb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(_lib.gsa_backward(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(wg), _ptr(topk_idx), _ptr(d_o),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dwg), _ptr(ws), wsb, _stream(stream)),
           "gsa_backward")


def gsa_train_state_size(cfg) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.gsa_train_state_size(ctypes.byref(cfg), ctypes.byref(out)), "gsa_train_state_size")
    return out.value


def gsa_forward_train(cfg, q, k, v, wg, o, state, ws, ws_bytes=None, stream=None, state_bytes=None):
    wsb = _nbytes(ws) if ws_bytes is None else ws_bytes
    stb = _nbytes(state) if state_bytes is None else state_bytes
    _check(_lib.gsa_forward_train(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(wg), _ptr(o), _ptr(state),
                                  stb, _ptr(ws), wsb, _stream(stream)), "gsa_forward_train")


def gsa_backward_train(cfg, q, k, v, wg, state, d_o, dq, dk, dv, dwg, ws, ws_bytes=None, stream=None,
                       state_bytes=None):
    wsb = _nbytes(ws) if ws_bytes is None else ws_bytes
    stb = _nbytes(state) if state_bytes is None else state_bytes
    _check(_lib.gsa_backward_train(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(wg), _ptr(state), stb,
                                   _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dwg), _ptr(ws), wsb, _stream(stream)),
           "gsa_backward_train")


def gsa_forward_noalloc(cfg, q, k, v, wg, o, stream=None):
    _check(_lib.gsa_forward_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(wg), _ptr(o),
                                    _stream(stream)), "gsa_forward_noalloc")


def call_status(fn: str, *args) -> int:
    """Raw status of a C entry point (used by the argument-validation tests)."""
    return getattr(_lib, fn)(*args)
