"""GSA forward oracle -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``gsa_oracle.c``: a plain, double-precision,
step-by-step CPU implementation of the Global Sparse Attention forward pass
(Paper-Notes page "Speed3R: Sparse Feed-forward 3D Reconstruction Models",
sections "全局稀疏注意力（GSA）核心设计", "压缩分支", "选择分支", "门控聚合",
"Speed3R-VGGT 适配"), the frame attention it alternates with (section
"整体框架"), the gradients of the GSA layer (for end-to-end training), and the
descriptor attention of the Paper-Notes page "FlashVGGT:
Efficient and Scalable Visual Geometry Transformers with Compressed Descriptor
Attention" (section "关键设计").  Only ``tests/``, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg use it.  It shares no code with the HIP library and
imports nothing from it.

Each function below calls exactly one oracle step; ``forward`` composes them
in the pages' order for workloads small enough to run in full.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


class OrcCfg(ctypes.Structure):
    _fields_ = [("n_frames", ctypes.c_int), ("n_special", ctypes.c_int), ("grid_h", ctypes.c_int),
                ("grid_w", ctypes.c_int), ("n_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("pool", ctypes.c_int), ("topk", ctypes.c_int), ("n_ctx", ctypes.c_int),
                ("ctx_frames", ctypes.c_int * 16), ("ctx_exclude", ctypes.c_int),
                ("scale", ctypes.c_double), ("dtype", ctypes.c_int)]


def build() -> None:
    """Compile liboracle.so with gcc: -O2, OpenMP, no FMA contraction, no fast-math."""
    src = os.path.join(_HERE, "gsa_oracle.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", src, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        cfgp = ctypes.POINTER(OrcCfg)
        lib.orc_pool.argtypes = [cfgp, P, P]
        lib.orc_special.argtypes = [cfgp, P, P, P, P, I64, P]
        lib.orc_frame.argtypes = [cfgp, P, P, P, P, I64, P]
        lib.orc_dense.argtypes = [cfgp, P, P, P, P, I64, P]
        lib.orc_backward.argtypes = [cfgp, P, P, P, P, P, ctypes.c_int, P, P, P, P, P]
        lib.orc_backward_dq_rows.argtypes = [cfgp, P, P, P, P, P, ctypes.c_int, P, P, I64, P]
        lib.orc_backward_dkdv_rows.argtypes = [cfgp, P, P, P, P, P, ctypes.c_int, P, P, I64, P, P]
        lib.orc_descriptor_count.argtypes = [cfgp]
        lib.orc_descriptor_count.restype = I64
        lib.orc_descriptor_set.argtypes = [cfgp, P, P]
        lib.orc_descriptor_attn.argtypes = [cfgp, P, P, P, I64, P, I64, P]
        lib.orc_compressed.argtypes = [cfgp, P, P, P, P, I64, P, P, P, P]
        lib.orc_guide_scores.argtypes = [cfgp, P, P, P, I64, P, ctypes.c_int, P]
        lib.orc_select.argtypes = [cfgp, P, P, P, P, I64, P, ctypes.c_int, P]
        lib.orc_gate_combine.argtypes = [cfgp, P, P, P, P, I64, P, P, P]
        lib.orc_window_token.argtypes = [cfgp, I64, ctypes.c_int]
        lib.orc_window_token.restype = I64
        for f in ("orc_pool", "orc_special", "orc_frame", "orc_dense", "orc_backward", "orc_backward_dq_rows",
                  "orc_backward_dkdv_rows", "orc_descriptor_set", "orc_descriptor_attn", "orc_compressed", "orc_guide_scores", "orc_select",
                  "orc_gate_combine"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def cfg_of(sh, scale: float = 0.0, topk: Optional[int] = None) -> OrcCfg:
    c = OrcCfg()
    c.n_frames, c.n_special, c.grid_h, c.grid_w = sh.n_frames, sh.n_special, sh.grid_h, sh.grid_w
    c.n_heads, c.head_dim, c.pool = sh.n_heads, sh.head_dim, sh.pool
    c.topk = sh.topk if topk is None else topk
    c.n_ctx = len(sh.ctx_frames)
    for i, f in enumerate(sh.ctx_frames):
        c.ctx_frames[i] = f
    c.ctx_exclude = sh.ctx_exclude
    c.scale = scale
    c.dtype = sh.dtype
    return c


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def pool(sh, x: np.ndarray) -> np.ndarray:
    """s x s average pooling -> float32 [M'][H][d] (values in the input precision)."""
    out = np.empty((sh.n_windows, sh.n_heads, sh.head_dim), np.float32)
    _load().orc_pool(ctypes.byref(cfg_of(sh)), _p(x), _p(out))
    return out


def special(sh, q, k, v, rows: np.ndarray) -> np.ndarray:
    """Dense attention of the listed special rows over all tokens -> [n][H][d] float64."""
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, sh.n_heads, sh.head_dim), np.float64)
    _load().orc_special(ctypes.byref(cfg_of(sh)), _p(q), _p(k), _p(v), _p(rows), rows.size, _p(out))
    return out


def dense(sh, q, k, v, rows: np.ndarray) -> np.ndarray:
    """Dense global attention of the listed token rows (special or image) over all tokens
    -> [n][H][d] float64 (the benchmark comparator's definition)."""
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, sh.n_heads, sh.head_dim), np.float64)
    _load().orc_dense(ctypes.byref(cfg_of(sh)), _p(q), _p(k), _p(v), _p(rows), rows.size, _p(out))
    return out


def backward(sh, q, k, v, wg, idx: np.ndarray, d_o):
    """Gradients of sum(d_o * forward(q, k, v, wg)) with the top-k window sets fixed at
    idx [M'][H][k] -> (dq, dk, dv [N][T_f][H][d] float64, dwg [H][d] float64).
    Whole workload; small shapes only."""
    idx = np.ascontiguousarray(idx, np.int32)
    shp = (sh.n_frames, sh.tokens_per_frame, sh.n_heads, sh.head_dim)
    dq, dk, dv = (np.empty(shp, np.float64) for _ in range(3))
    dwg = np.empty((sh.n_heads, sh.head_dim), np.float64)
    _load().orc_backward(ctypes.byref(cfg_of(sh)), _p(q), _p(k), _p(v), _p(wg), _p(idx), idx.shape[-1],
                         _p(np.ascontiguousarray(d_o)), _p(dq), _p(dk), _p(dv), _p(dwg))
    return dq, dk, dv, dwg


def backward_dq_rows(sh, q, k, v, wg, idx: np.ndarray, d_o, rows: np.ndarray) -> np.ndarray:
    """dq of the listed token rows (backward with the top-k sets fixed at idx), one row at a
    time, for workloads too large for the whole layer -> [n][H][d] float64."""
    idx = np.ascontiguousarray(idx, np.int32)
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, sh.n_heads, sh.head_dim), np.float64)
    _load().orc_backward_dq_rows(ctypes.byref(cfg_of(sh)), _p(q), _p(k), _p(v), _p(wg), _p(idx), idx.shape[-1],
                                 _p(np.ascontiguousarray(d_o)), _p(rows), rows.size, _p(out))
    return out


def backward_dkdv_rows(sh, q, k, v, wg, idx: np.ndarray, d_o, rows: np.ndarray):
    """dK and dV of the listed token rows (backward with the top-k sets fixed at idx), per
    key row, for workloads too large for the whole layer; query rows whose incoming
    gradient is exactly zero are skipped (they contribute exactly zero), so the cost
    follows the non-zero rows of d_o -> ([n][H][d], [n][H][d]) float64."""
    idx = np.ascontiguousarray(idx, np.int32)
    rows = np.ascontiguousarray(rows, np.int64)
    assert np.unique(rows).size == rows.size, "rows must be distinct"
    dk = np.empty((rows.size, sh.n_heads, sh.head_dim), np.float64)
    dv = np.empty_like(dk)
    _load().orc_backward_dkdv_rows(ctypes.byref(cfg_of(sh)), _p(q), _p(k), _p(v), _p(wg), _p(idx), idx.shape[-1],
                                   _p(np.ascontiguousarray(d_o)), _p(rows), rows.size, _p(dk), _p(dv))
    return dk, dv


def frame(sh, q, k, v, rows: np.ndarray) -> np.ndarray:
    """Frame attention (each token over the T_f tokens of its own frame) of the listed
    token rows -> [n][H][d] float64."""
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, sh.n_heads, sh.head_dim), np.float64)
    _load().orc_frame(ctypes.byref(cfg_of(sh)), _p(q), _p(k), _p(v), _p(rows), rows.size, _p(out))
    return out


def descriptor_set(sh, x: np.ndarray) -> np.ndarray:
    """FlashVGGT key/value set of x: bilinear r x r descriptors (r = pool) of every frame, then
    the auxiliary tokens (frame 0 and the keyframes ctx_frames whole, the other frames'
    special tokens) -> float32 [n_set][H][d] (values in the input precision)."""
    cfg = cfg_of(sh)
    n = _load().orc_descriptor_count(ctypes.byref(cfg))
    out = np.empty((n, sh.n_heads, sh.head_dim), np.float32)
    _load().orc_descriptor_set(ctypes.byref(cfg), _p(x), _p(out))
    return out


def descriptor_attn(sh, q, kd: np.ndarray, vd: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Descriptor attention of the listed token rows over the set kd/vd -> [n][H][d] float64."""
    rows = np.ascontiguousarray(rows, np.int64)
    kd = np.ascontiguousarray(kd, np.float32)
    vd = np.ascontiguousarray(vd, np.float32)
    out = np.empty((rows.size, sh.n_heads, sh.head_dim), np.float64)
    _load().orc_descriptor_attn(ctypes.byref(cfg_of(sh)), _p(q), _p(kd), _p(vd), kd.shape[0], _p(rows),
                                rows.size, _p(out))
    return out


def compressed(sh, qc, kc, vc, wins: np.ndarray, topk: Optional[int] = None):
    """Compressed attention + guide-score top-k for the listed windows.

    Returns (oc [n][H][d] f64, topk_idx [n][H][k] i32, topk_scores [n][H][k+1] f64,
    s_absmax [n][H] f64).
    """
    wins = np.ascontiguousarray(wins, np.int64)
    k = sh.topk if topk is None else topk
    n, H, d = wins.size, sh.n_heads, sh.head_dim
    oc = np.empty((n, H, d), np.float64)
    idx = np.empty((n, H, k), np.int32)
    sc = np.empty((n, H, k + 1), np.float64)
    amax = np.empty((n, H), np.float64)
    _load().orc_compressed(ctypes.byref(cfg_of(sh, topk=k)), _p(qc), _p(kc), _p(vc), _p(wins), n,
                           _p(oc), _p(idx), _p(sc), _p(amax))
    return oc, idx, sc, amax


def guide_scores(sh, qc, kc, wins: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """S_ij = Q_comp_i . K_comp_j for the given [n][H][k] window ids (NaN where id < 0)."""
    wins = np.ascontiguousarray(wins, np.int64)
    idx = np.ascontiguousarray(idx, np.int32)
    out = np.empty(idx.shape, np.float64)
    _load().orc_guide_scores(ctypes.byref(cfg_of(sh)), _p(qc), _p(kc), _p(wins), wins.size,
                             _p(idx), idx.shape[-1], _p(out))
    return out


def select(sh, q, k, v, wins: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Selection attention of the listed windows' queries -> [n][s*s][H][d] float64."""
    wins = np.ascontiguousarray(wins, np.int64)
    idx = np.ascontiguousarray(idx, np.int32)
    s2 = sh.pool * sh.pool
    out = np.empty((wins.size, s2, sh.n_heads, sh.head_dim), np.float64)
    _load().orc_select(ctypes.byref(cfg_of(sh)), _p(q), _p(k), _p(v), _p(wins), wins.size, _p(idx),
                       idx.shape[-1], _p(out))
    return out


def gate_combine(sh, q, wg, wins, oc_rows, osel, gate=None) -> np.ndarray:
    """g * upsample(O'_comp) + (1-g) * O_sel for the listed windows -> [n][s*s][H][d]."""
    wins = np.ascontiguousarray(wins, np.int64)
    oc_rows = np.ascontiguousarray(oc_rows, np.float64)
    osel = np.ascontiguousarray(osel, np.float64)
    out = np.empty_like(osel)
    g = None if gate is None else np.ascontiguousarray(gate, np.float64)
    _load().orc_gate_combine(ctypes.byref(cfg_of(sh)), _p(q), None if wg is None else _p(wg),
                             None if g is None else _p(g), _p(wins), wins.size, _p(oc_rows),
                             _p(osel), _p(out))
    return out


def window_tokens(sh, wins: np.ndarray) -> np.ndarray:
    """Token rows [n][s*s] of the pixels of the listed windows (row-major in the window)."""
    lib, c = _load(), cfg_of(sh)
    s2 = sh.pool * sh.pool
    return np.array([[lib.orc_window_token(ctypes.byref(c), int(j), qq) for qq in range(s2)]
                     for j in wins], dtype=np.int64)


def forward(sh, q, k, v, wg, gate=None):
    """Full GSA forward for a workload small enough to run whole.

    Steps in the pages' order: split, pool, special attention, compressed
    attention with guide-score top-k, selection attention, upsample + gate.
    Returns a dict with O [N][T_f][H][d] float64 and every intermediate.
    """
    wins = np.arange(sh.n_windows, dtype=np.int64)
    qc, kc, vc = pool(sh, q), pool(sh, k), pool(sh, v)
    rows = np.arange(sh.m_spec, dtype=np.int64)
    o = np.zeros(sh.qkv_shape, np.float64).reshape(sh.m_tokens, sh.n_heads, sh.head_dim)
    if sh.m_spec:
        ospec = special(sh, q, k, v, rows)
        tf = sh.tokens_per_frame
        tok = (rows // sh.n_special) * tf + rows % sh.n_special
        o[tok] = ospec
    oc, idx, sc, amax = compressed(sh, qc, kc, vc, wins)
    osel = select(sh, q, k, v, wins, idx)
    oimg = gate_combine(sh, q, None if gate is not None else wg, wins, oc, osel, gate)
    toks = window_tokens(sh, wins)
    o[toks.reshape(-1)] = oimg.reshape(-1, sh.n_heads, sh.head_dim)
    return {"o": o.reshape(sh.qkv_shape), "qc": qc, "kc": kc, "vc": vc, "oc": oc, "topk": idx,
            "topk_scores": sc, "s_absmax": amax, "osel": osel, "oimg": oimg, "win_tokens": toks}
