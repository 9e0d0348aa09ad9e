"""Workload shapes of the GSA layer used by the tests and the bench.

Each workload is named for what it is.  The token layout of Q/K/V/O is
``[N][T_f][H][d]`` with ``T_f = P + h*w`` (P special tokens first, then the
image tokens of the h x w grid, row-major).
"""
from __future__ import annotations

import dataclasses
from typing import Tuple


@dataclasses.dataclass(frozen=True)
class GSAShape:
    name: str
    n_frames: int
    n_special: int
    grid_h: int
    grid_w: int
    n_heads: int
    head_dim: int
    pool: int
    topk: int
    dtype: int  # 0 = bf16, 1 = fp32
    ctx_frames: Tuple[int, ...] = ()
    ctx_exclude: int = 1
    recipe: str = "normal"
    seed: int = 1000

    # derived sizes -------------------------------------------------------
    @property
    def tokens_per_frame(self) -> int:
        return self.n_special + self.grid_h * self.grid_w

    @property
    def m_tokens(self) -> int:
        return self.n_frames * self.tokens_per_frame

    @property
    def m_spec(self) -> int:
        return self.n_frames * self.n_special

    @property
    def m_img(self) -> int:
        return self.n_frames * self.grid_h * self.grid_w

    @property
    def windows_per_frame(self) -> int:
        return (self.grid_h // self.pool) * (self.grid_w // self.pool)

    @property
    def n_windows(self) -> int:
        return self.n_frames * self.windows_per_frame

    @property
    def qkv_shape(self):
        return (self.n_frames, self.tokens_per_frame, self.n_heads, self.head_dim)

    @property
    def n_candidates(self) -> int:
        if self.ctx_exclude and self.ctx_frames:
            return (self.n_frames - len(self.ctx_frames)) * self.windows_per_frame
        return self.n_windows

    @property
    def topk_eff(self) -> int:
        return min(self.topk, self.n_candidates)

    def replace(self, **kw) -> "GSAShape":
        return dataclasses.replace(self, **kw)

    # algorithmic work (one layer) ----------------------------------------
    def flops(self) -> dict:
        d, h = self.head_dim, self.n_heads
        ctx = len(self.ctx_frames) * self.tokens_per_frame
        keys_sel = self.topk_eff * self.pool * self.pool + ctx
        return {
            "special": 4.0 * self.m_spec * self.m_tokens * d * h,
            "compressed": 4.0 * self.n_windows ** 2 * d * h,
            "selection": 4.0 * self.m_img * keys_sel * d * h,
            "dense": 4.0 * self.m_tokens ** 2 * d * h,
            "frame": 4.0 * self.n_frames * self.tokens_per_frame ** 2 * d * h,
        }


BF16, F32 = 0, 1

TINY_F32 = GSAShape("tiny-fp32 4f-8x8-s2-k4", 4, 1, 8, 8, 1, 64, 2, 4, F32, seed=1000)
SMALL_BF16 = GSAShape("32f-32x32-h16-s4-k16", 32, 5, 32, 32, 16, 64, 4, 16, BF16, seed=1001)
VGGT_CTX = GSAShape("vggt-ctx 128f-36x36-h16-s4-k32+ctx{0,100}", 128, 5, 36, 36, 16, 64, 4, 32,
                    BF16, ctx_frames=(0, 100), seed=1002)
PI3_LONG = GSAShape("pi3-long 1000f-36x36-h16-s4-k32", 1000, 5, 36, 36, 16, 64, 4, 32, BF16,
                    seed=1003)
PEAKY = GSAShape("peaky 1024f-36x36-h16-s4-k32", 1024, 5, 36, 36, 16, 64, 4, 32, BF16,
                 recipe="clustered", seed=1004)

CONFIGS = [TINY_F32, SMALL_BF16, VGGT_CTX, PI3_LONG, PEAKY]


def config_by_name(name: str) -> GSAShape:
    for c in CONFIGS:
        if c.name == name or c.name.split()[0] == name:
            return c
    raise KeyError(name)
