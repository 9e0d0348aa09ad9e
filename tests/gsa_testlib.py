"""Shared helpers of the GPU parity tests: device marshalling of the seeded
inputs, the HIP calls through the C ABI, and the comparison rules.

Comparison rules (floating point): bf16 inputs with fp32 accumulation must stay
within max-abs 2e-2 and mean-abs 2e-3 of the oracle; fp32 inputs within
max-abs 1e-5.  Top-k: index sets must equal the oracle's unless the oracle's
k-th / (k+1)-th guide-score gap is below the tie band
delta = 1e-4 * max(|s_k|, |s_k+1|) + 1e-6 * max_j |S_ij|; inside the band the
GPU set must contain every window scoring above s_k + delta and only windows
scoring at least s_k - delta.
"""
from __future__ import annotations

import numpy as np
import torch

import gen
import oracle
import sparse_global_attention_amd as gsa

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-5
TIE_REL, TIE_ABS = 1e-4, 1e-6

DEV = "cuda"


def to_dev(x: np.ndarray, dtype: int) -> torch.Tensor:
    if dtype == gen.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 values widened exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def empty(shape, dtype: int) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == gen.BF16 else torch.float32, device=DEV)


def workspace(cfg, op) -> torch.Tensor:
    n = gsa.gsa_workspace_size(cfg, op)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)


class Case:
    """Seeded inputs of one workload, on the host and on the device."""

    def __init__(self, sh, q=None, k=None, v=None, wg=None):
        self.sh = sh
        gq, gk, gv, gw = gen.make_inputs(sh)
        self.q = gq if q is None else q
        self.k = gk if k is None else k
        self.v = gv if v is None else v
        self.wg = gw if wg is None else wg
        self.cfg = gsa.GSAConfig.from_shape(sh)
        self.dq, self.dk, self.dv = (to_dev(x, sh.dtype) for x in (self.q, self.k, self.v))
        self.dwg = to_dev(self.wg, sh.dtype)

    # ---- HIP path, through the C ABI ----
    def pool(self):
        sh = self.sh
        shp = (sh.n_windows, sh.n_heads, sh.head_dim)
        qc, kc, vc = empty(shp, sh.dtype), empty(shp, sh.dtype), empty(shp, sh.dtype)
        gsa.gsa_pool(self.cfg, self.dq, self.dk, self.dv, qc, kc, vc)
        return qc, kc, vc

    def compressed(self, qc, kc, vc, with_scores=True):
        sh = self.sh
        oc = torch.empty((sh.n_windows, sh.n_heads, sh.head_dim), dtype=torch.float32, device=DEV)
        idx = torch.empty((sh.n_windows, sh.n_heads, sh.topk), dtype=torch.int32, device=DEV)
        sc = torch.empty((sh.n_windows, sh.n_heads, sh.topk), dtype=torch.float32, device=DEV) if with_scores else None
        ws = workspace(self.cfg, gsa.GSA_OP_COMPRESSED)
        gsa.gsa_compressed_attn_topk(self.cfg, qc, kc, vc, oc, idx, sc, ws)
        return oc, idx, sc

    def select(self, idx):
        sh = self.sh
        osel = torch.empty((sh.m_img, sh.n_heads, sh.head_dim), dtype=torch.float32, device=DEV)
        ws = workspace(self.cfg, gsa.GSA_OP_SELECT)
        gsa.gsa_select_attn(self.cfg, self.dq, self.dk, self.dv, idx, osel, ws)
        return osel

    def special(self, o=None):
        sh = self.sh
        o = torch.zeros(sh.qkv_shape, dtype=self.dq.dtype, device=DEV) if o is None else o
        ws = workspace(self.cfg, gsa.GSA_OP_SPECIAL)
        gsa.gsa_special_attn(self.cfg, self.dq, self.dk, self.dv, o, ws)
        return o

    def forward(self, o=None):
        sh = self.sh
        o = torch.zeros(sh.qkv_shape, dtype=self.dq.dtype, device=DEV) if o is None else o
        ws = workspace(self.cfg, gsa.GSA_OP_FORWARD)
        gsa.gsa_forward(self.cfg, self.dq, self.dk, self.dv, self.dwg, o, ws)
        return o

    def frame(self):
        sh = self.sh
        o = torch.zeros(sh.qkv_shape, dtype=self.dq.dtype, device=DEV)
        gsa.gsa_frame_attn(self.cfg, self.dq, self.dk, self.dv, o)
        return o

    def descriptor_set(self):
        sh = self.sh
        n = gsa.gsa_descriptor_count(self.cfg)
        kd, vd = empty((n, sh.n_heads, sh.head_dim), sh.dtype), empty((n, sh.n_heads, sh.head_dim), sh.dtype)
        gsa.gsa_descriptor_set(self.cfg, self.dk, self.dv, kd, vd)
        return kd, vd

    def descriptor_attn(self, kd, vd):
        sh = self.sh
        o = torch.zeros(sh.qkv_shape, dtype=self.dq.dtype, device=DEV)
        gsa.gsa_descriptor_attn(self.cfg, self.dq, kd, vd, o)
        return o

    def dense(self):
        sh = self.sh
        o = torch.zeros(sh.qkv_shape, dtype=self.dq.dtype, device=DEV)
        gsa.gsa_dense_attn(self.cfg, self.dq, self.dk, self.dv, o)
        return o


# ---- geometry (the test's own, from reshapes) ----
def window_token_ids(sh) -> np.ndarray:
    s = sh.pool
    grid = np.arange(sh.m_tokens, dtype=np.int64).reshape(sh.n_frames, sh.tokens_per_frame)
    img = grid[:, sh.n_special:].reshape(sh.n_frames, sh.grid_h // s, s, sh.grid_w // s, s)
    return img.transpose(0, 1, 3, 2, 4).reshape(-1, s * s)


def window_image_ids(sh) -> np.ndarray:
    s = sh.pool
    img = np.arange(sh.m_img, dtype=np.int64).reshape(sh.n_frames, sh.grid_h // s, s, sh.grid_w // s, s)
    return img.transpose(0, 1, 3, 2, 4).reshape(-1, s * s)


def special_token_ids(sh) -> np.ndarray:
    grid = np.arange(sh.m_tokens, dtype=np.int64).reshape(sh.n_frames, sh.tokens_per_frame)
    return grid[:, :sh.n_special].reshape(-1)


# ---- comparisons ----
def assert_close(got: np.ndarray, ref: np.ndarray, dtype: int, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    if dtype == gen.BF16:
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, f"{what}: max {mx:.3g} mean {mean:.3g} relL2 {rel:.3g}"
    else:
        assert mx <= F32_MAX_ABS, f"{what}: max {mx:.3g} mean {mean:.3g} relL2 {rel:.3g}"
    return mx, mean, rel


def check_topk(sh, gpu_idx: np.ndarray, orc_idx: np.ndarray, orc_sc: np.ndarray, absmax: np.ndarray,
               gpu_s: np.ndarray) -> int:
    """Tie-band comparison of GPU top-k sets with the oracle's; returns the number of in-band rows.

    gpu_idx, orc_idx: [n][H][k]; orc_sc: [n][H][k+1] sorted oracle scores; absmax: [n][H];
    gpu_s: [n][H][k] the oracle's guide scores of the GPU's windows.
    """
    kp = sh.topk_eff
    ncand = sh.n_candidates
    banded = 0
    n, H, _ = gpu_idx.shape
    assert np.all(gpu_idx[..., kp:] == -1), "slots past k' must be -1"
    # every pick is a candidate window: in range and, when the context frames
    # are excluded, not one of their windows (checked for every row, in or out
    # of the tie band)
    cand = candidate_windows(sh)
    picks = gpu_idx[..., :kp]
    assert np.all((picks >= 0) & (picks < sh.n_windows)), "window id out of range"
    assert np.all(cand[picks]), "a pick is not a candidate window (excluded context frame)"
    for i in range(n):
        for h in range(H):
            g = gpu_idx[i, h, :kp]
            assert np.all(g >= 0) and len(set(g.tolist())) == kp, (i, h, g)
            o = orc_idx[i, h, :kp]
            if kp == ncand:
                assert set(g.tolist()) == set(o.tolist()), (i, h)
                continue
            tau, taup = orc_sc[i, h, kp - 1], orc_sc[i, h, kp]
            delta = TIE_REL * max(abs(tau), abs(taup)) + TIE_ABS * absmax[i, h]
            if tau - taup >= delta:
                assert set(g.tolist()) == set(o.tolist()), (i, h, sorted(g), sorted(o))
            else:
                banded += 1
                must = {int(j) for j, s in zip(orc_idx[i, h, :kp], orc_sc[i, h, :kp]) if s > tau + delta}
                assert must <= set(g.tolist()), (i, h)
                assert np.all(gpu_s[i, h, :kp] >= tau - delta), (i, h)
            # the GPU list is sorted by score (within the band)
            s = gpu_s[i, h, :kp]
            assert np.all(np.diff(s) <= TIE_REL * np.abs(s[:-1]) + TIE_ABS * absmax[i, h] + 1e-12), (i, h, s)
    return banded


def candidate_windows(sh) -> np.ndarray:
    """[M'] mask of the top-k candidate windows: all windows, minus those of the
    context frames when they are excluded (section "Speed3R-VGGT 适配": the
    dynamic top-k comes from the non-reference frames)."""
    cand = np.ones(sh.n_windows, bool)
    if sh.ctx_exclude:
        for f in sh.ctx_frames:
            cand[f * sh.windows_per_frame:(f + 1) * sh.windows_per_frame] = False
    return cand


def same_sets(gpu_idx: np.ndarray, orc_idx: np.ndarray) -> np.ndarray:
    """[n][H] mask of the (window, head) rows whose GPU top-k set equals the oracle's.

    Only those rows have a unique expected selection output; the others hold a
    different, valid choice inside the tie band (checked by check_topk)."""
    return np.all(np.sort(gpu_idx, axis=-1) == np.sort(orc_idx, axis=-1), axis=-1)


def assert_close_rows(got: np.ndarray, ref: np.ndarray, rows: np.ndarray, dtype: int, what: str):
    """assert_close on the (window, head) rows selected by rows [n][H], for
    per-window outputs [n][s*s][H][d]."""
    mask = np.broadcast_to(rows[:, None, :, None], got.shape)
    return assert_close(got[mask], ref[mask], dtype, what)
