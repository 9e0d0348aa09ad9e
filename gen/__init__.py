"""Seeded synthetic GSA inputs shared by the oracle tests, the GPU tests and the bench.

The C generator (``gsa_gen.c``) is counter based: each element depends only on
(seed, stream, flat index), so inputs are reproducible at any thread count and
can be regenerated for any sub-range.  This package holds no attention
arithmetic; it draws numbers, names the workload shapes and writes tensors in
the token layout ``[N][P + h*w][H][d]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import CONFIGS, GSAShape, config_by_name  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libgsagen.so")
_lib = None

BF16, F32 = 0, 1
STREAM_Q, STREAM_K, STREAM_V, STREAM_WG = 1, 2, 3, 4
STREAM_KCEN, STREAM_VCEN, STREAM_KVMAP, STREAM_QMAP = 5, 6, 7, 8
STREAM_SAMPLE_WIN, STREAM_SAMPLE_SPEC = 9, 10
STREAM_DO = 11


def build() -> None:
    """Compile libgsagen.so with gcc (OpenMP, no fast-math)."""
    src = os.path.join(_HERE, "gsa_gen.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           src, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.gen_normal.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_double, ctypes.c_int64]
        lib.gen_normal.restype = None
        lib.gen_clustered.argtypes = [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_int] * 7 + [
            ctypes.c_uint64] * 4 + [ctypes.c_int, ctypes.c_double]
        lib.gen_clustered.restype = None
        lib.gen_mix64.argtypes = [ctypes.c_uint64]
        lib.gen_mix64.restype = ctypes.c_uint64
        lib.gen_normal_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.gen_normal_at.restype = ctypes.c_double
        _lib = lib
    return _lib


def np_dtype(dtype: int):
    """Storage dtype: bf16 is carried as raw uint16 bits, fp32 as float32."""
    return np.uint16 if dtype == BF16 else np.float32


def normal(shape, dtype: int, seed: int, stream: int, std: float = 1.0, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np_dtype(dtype))
    _load().gen_normal(out.ctypes.data, out.size, dtype, seed, stream, std, offset)
    return out


def clustered(sh: GSAShape, seed: int, stream_noise: int, stream_centroid: int, stream_map: int,
              n_clusters: int = 64, noise_std: float = 0.1) -> np.ndarray:
    out = np.empty(sh.qkv_shape, dtype=np_dtype(sh.dtype))
    _load().gen_clustered(out.ctypes.data, sh.dtype, sh.n_frames, sh.n_special, sh.grid_h, sh.grid_w,
                          sh.n_heads, sh.head_dim, sh.pool, seed, stream_noise, stream_centroid,
                          stream_map, n_clusters, noise_std)
    return out


def mix64(z: int) -> int:
    return int(_load().gen_mix64(z))


def normal_at(seed: int, stream: int, i: int) -> float:
    return float(_load().gen_normal_at(seed, stream, i))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f32(x: np.ndarray, dtype: int) -> np.ndarray:
    return bf16_bits_to_f32(x) if dtype == BF16 else x.astype(np.float32, copy=False)


def make_inputs(sh: GSAShape, seed: int | None = None):
    """Q, K, V, W_g host arrays for a workload, following its input recipe.

    * ``normal`` recipe: Q, K, V ~ N(0,1); W_g ~ N(0, 1/d).
    * ``clustered`` recipe: K and V tokens are window-cluster centroids plus
      0.1 N(0,1) noise (64 clusters, K and V share the window->cluster map),
      Q is drawn from the K centroid table with its own map, special tokens
      are N(0,1), W_g ~ N(0, 1/d).
    """
    seed = sh.seed if seed is None else seed
    wg = normal((sh.n_heads, sh.head_dim), sh.dtype, seed, STREAM_WG, std=sh.head_dim ** -0.5)
    if sh.recipe == "clustered":
        q = clustered(sh, seed, STREAM_Q, STREAM_KCEN, STREAM_QMAP)
        k = clustered(sh, seed, STREAM_K, STREAM_KCEN, STREAM_KVMAP)
        v = clustered(sh, seed, STREAM_V, STREAM_VCEN, STREAM_KVMAP)
    else:
        q = normal(sh.qkv_shape, sh.dtype, seed, STREAM_Q)
        k = normal(sh.qkv_shape, sh.dtype, seed, STREAM_K)
        v = normal(sh.qkv_shape, sh.dtype, seed, STREAM_V)
    return q, k, v, wg


def make_output_grad(sh: GSAShape, seed: int | None = None) -> np.ndarray:
    """Output gradient dO [N][T_f][H][d] ~ N(0, 1) in the workload's dtype."""
    seed = sh.seed if seed is None else seed
    return normal(sh.qkv_shape, sh.dtype, seed, STREAM_DO)


def sample_windows(sh: GSAShape, n: int, seed: int | None = None) -> np.ndarray:
    """n distinct window ids (sorted), always including the first and last."""
    seed = sh.seed if seed is None else seed
    m = sh.n_windows
    if n >= m:
        return np.arange(m, dtype=np.int64)
    rng = np.random.default_rng([seed, STREAM_SAMPLE_WIN])
    pick = rng.choice(np.arange(1, m - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, m - 1], pick]).astype(np.int64))


def sample_special(sh: GSAShape, n: int, seed: int | None = None) -> np.ndarray:
    """n distinct special-row ids (sorted), always including the first and last."""
    seed = sh.seed if seed is None else seed
    m = sh.m_spec
    if n >= m:
        return np.arange(m, dtype=np.int64)
    rng = np.random.default_rng([seed, STREAM_SAMPLE_SPEC])
    pick = rng.choice(np.arange(1, m - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, m - 1], pick]).astype(np.int64))
