"""Parity of the HIP backward (gsa_backward, through the C ABI) with the CPU
oracle's gradients, element by element, on seeded inputs and output
gradients.  The top-k window sets both sides hold fixed come from the
oracle's own top-k of the same inputs (or, at full size, from a seeded
generator), so no oracle input comes from the GPU.  At the full workload
sizes (too large for the whole-layer oracle) dq is checked on sampled rows
the oracle evaluates one by one, dK/dV on listed rows for an output gradient
that is non-zero on a few rows only (the oracle then evaluates those rows one
by one too), and through properties that hold at any size: sum_t dV_t =
sum_t dO_t and sum_t dK_t = 0 per head and channel; plus finite values and
determinism.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_global_attention_amd as gsa
from gen.configs import BF16, F32, PI3_LONG, TINY_F32, VGGT_CTX, GSAShape
from gsa_testlib import DEV, to_dev, workspace

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny_f32": TINY_F32,
    "odd_bf16": GSAShape("odd 3f-12x8-h3-s4-k5", 3, 2, 12, 8, 3, 64, 4, 5, BF16, seed=21),
    "odd_f32": GSAShape("odd 3f-12x8-h3-s4-k5 fp32", 3, 2, 12, 8, 3, 64, 4, 5, F32, seed=22),
    "mid_bf16": GSAShape("mid 8f-16x16-h4-s4-k8", 8, 5, 16, 16, 4, 64, 4, 8, BF16, seed=40),
    "s8": GSAShape("s8 3f-16x16-h2-s8-k3", 3, 1, 16, 16, 2, 64, 8, 3, BF16, seed=23),
    "s1": GSAShape("s1 2f-6x5-h2-s1-k7", 2, 1, 6, 5, 2, 64, 1, 7, BF16, seed=24),
    "s2": GSAShape("s2 4f-8x8-h2-s2-k4", 4, 3, 8, 8, 2, 64, 2, 4, BF16, seed=25),
    "s5": GSAShape("s5 2f-10x10-h2-s5-k3", 2, 2, 10, 10, 2, 64, 5, 3, BF16, seed=33),
    # 9 keys in 16 slots and 49 in 56 (padding slots; windows straddle 32-slot chunks)
    "s3": GSAShape("s3 3f-9x12-h2-s3-k4", 3, 1, 9, 12, 2, 64, 3, 4, BF16, seed=70),
    "s7": GSAShape("s7 2f-14x14-h2-s7-k3", 2, 1, 14, 14, 2, 64, 7, 3, BF16, seed=71),
    "s6_f32": GSAShape("s6 3f-12x12-h2-s6-k3 fp32", 3, 1, 12, 12, 2, 64, 6, 3, F32, seed=34),
    "p0": GSAShape("p0 4f-8x12-h2-s4-k3", 4, 0, 8, 12, 2, 64, 4, 3, BF16, seed=26),
    "ctx": GSAShape("ctx 6f-8x8-h2-s4-k3+ctx{0,3}", 6, 2, 8, 8, 2, 64, 4, 3, BF16, ctx_frames=(0, 3), seed=27),
    "ctx_f32": GSAShape("ctx 5f-8x8-h1-s2-k6+ctx{4}", 5, 1, 8, 8, 1, 64, 2, 6, F32, ctx_frames=(4,), seed=28),
    "k_clamp": GSAShape("kclamp 2f-8x8-h2-s4-k64", 2, 1, 8, 8, 2, 64, 4, 64, BF16, seed=29),
    "k40": GSAShape("k40 10f-16x16-h2-s4-k40", 10, 1, 16, 16, 2, 64, 4, 40, BF16, seed=32),
}

# Gradients are sums of many products; errors are stated relative to the
# largest reference magnitude of each tensor.  bf16: operands of every
# matrix-core product (q, k, v, dO, P, dS) are bf16 (relative rounding 2^-9),
# the accumulation is fp32.  fp32: the exp2 and the fp32 accumulation.
BF16_MAX_REL, BF16_MEAN_REL = 2e-2, 2e-3
F32_MAX_REL = 1e-5


def assert_grad_close(got, ref, dtype, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got - ref) / scale
    mx, mean = float(err.max()), float(err.mean())
    if dtype == BF16:
        assert mx <= BF16_MAX_REL and mean <= BF16_MEAN_REL, f"{what}: max {mx:.3g} mean {mean:.3g} (of {scale:.3g})"
    else:
        assert mx <= F32_MAX_REL, f"{what}: max {mx:.3g} mean {mean:.3g} (of {scale:.3g})"
    return mx, mean


def oracle_topk(sh, q, k):
    """The oracle's top-k of the workload (its own pooling and guide scores)."""
    qc, kc = oracle.pool(sh, q), oracle.pool(sh, k)
    vc = np.zeros_like(qc)
    return oracle.compressed(sh, qc, kc, vc, np.arange(sh.n_windows))[1]


def gpu_backward(sh, q, k, v, wg, idx, d_o):
    cfg = gsa.GSAConfig.from_shape(sh)
    dq_, dk_, dv_ = (torch.empty(sh.qkv_shape, dtype=torch.float32, device=DEV) for _ in range(3))
    dwg_ = torch.empty((sh.n_heads, sh.head_dim), dtype=torch.float32, device=DEV)
    ws = workspace(cfg, gsa.GSA_OP_BACKWARD)
    gsa.gsa_backward(cfg, to_dev(q, sh.dtype), to_dev(k, sh.dtype), to_dev(v, sh.dtype), to_dev(wg, sh.dtype),
                     torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(DEV), to_dev(d_o, sh.dtype),
                     dq_, dk_, dv_, dwg_, ws)
    torch.cuda.synchronize()
    return dq_, dk_, dv_, dwg_


@pytest.mark.parametrize("name", list(SHAPES))
def test_backward_matches_oracle(name):
    sh = SHAPES[name]
    q, k, v, wg = gen.make_inputs(sh)
    d_o = gen.make_output_grad(sh)
    idx = oracle_topk(sh, q, k)
    got = [x.cpu().numpy() for x in gpu_backward(sh, q, k, v, wg, idx, d_o)]
    ref = oracle.backward(sh, q, k, v, wg, idx, d_o)
    for g_, r_, what in zip(got, ref, ("dq", "dk", "dv", "dwg")):
        mx, mean = assert_grad_close(g_.reshape(r_.shape), r_, sh.dtype, f"{name} {what}")
        print(f"{name} {what}: max {mx:.3g} mean {mean:.3g} of the largest |ref|")


def test_backward_is_deterministic():
    sh = SHAPES["mid_bf16"]
    q, k, v, wg = gen.make_inputs(sh)
    d_o = gen.make_output_grad(sh)
    idx = oracle_topk(sh, q, k)
    a = gpu_backward(sh, q, k, v, wg, idx, d_o)
    b = gpu_backward(sh, q, k, v, wg, idx, d_o)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("sh", [VGGT_CTX, PI3_LONG], ids=["vggt_ctx", "pi3_long"])
def test_backward_full_size(sh):
    """At the full sizes, with seeded window sets (any fixed sets define the
    backward; the same sets on both sides): dq of sampled special and image rows
    against the oracle evaluated row by row; column sums of dV equal those of dO
    and those of dK vanish (per head and channel: softmax weights sum to one,
    each query's score gradients sum to zero); finite values; a second call is
    bitwise identical."""
    from gsa_testlib import Case
    rng = np.random.default_rng(sh.seed + 11)
    idx = rng.integers(0, sh.n_windows, size=(sh.n_windows, sh.n_heads, sh.topk)).astype(np.int32)
    c = Case(sh)
    d_o_h = gen.make_output_grad(sh)
    d_o = to_dev(d_o_h, sh.dtype)
    didx = torch.from_numpy(idx).to(DEV)
    cfg = c.cfg
    dq_, dk_, dv_ = (torch.empty(sh.qkv_shape, dtype=torch.float32, device=DEV) for _ in range(3))
    dwg_ = torch.empty((sh.n_heads, sh.head_dim), dtype=torch.float32, device=DEV)
    ws = workspace(cfg, gsa.GSA_OP_BACKWARD)
    gsa.gsa_backward(cfg, c.dq, c.dk, c.dv, c.dwg, didx, d_o, dq_, dk_, dv_, dwg_, ws)
    torch.cuda.synchronize()
    shp = (sh.m_tokens, sh.n_heads, sh.head_dim)
    for x in (dq_, dk_, dv_, dwg_):
        assert torch.isfinite(x).all()
    # sampled dq rows: a few special rows, image rows spread over the sequence
    tf = sh.tokens_per_frame
    frames = rng.choice(sh.n_frames, 4, replace=False)
    spec_rows = frames * tf + rng.integers(0, sh.n_special, 4)
    img_rows = rng.choice(sh.n_frames, 32) * tf + sh.n_special + rng.integers(0, sh.grid_h * sh.grid_w, 32)
    rows = np.unique(np.concatenate([spec_rows, img_rows]))
    got = dq_.view(shp).index_select(0, torch.from_numpy(rows).to(DEV)).cpu().numpy()
    ref = oracle.backward_dq_rows(sh, c.q, c.k, c.v, c.wg, idx, d_o_h, rows)
    mx, mean = assert_grad_close(got, ref, sh.dtype, f"{sh.name} sampled dq")
    print(f"{sh.name}: sampled dq ({rows.size} rows) max {mx:.3g} mean {mean:.3g} of the largest |ref|")
    # Each column sum adds ~1e6 terms whose matrix-core operands (P, dS, dO_sel)
    # were rounded to bf16 (relative 2^-9, independent signs): the deviation is
    # a random sum of size ~2^-9 sqrt(sum of squared terms).  Allow 8x that with
    # 2^-8 per term; a dropped or mis-scaled branch moves a sum by orders more.
    G = d_o.float().view(shp).double()
    sig_v = (dv_.view(shp).double().pow(2).sum(0) + G.pow(2).sum(0)).sqrt()
    sig_k = dk_.view(shp).double().pow(2).sum(0).sqrt()
    err_v = (dv_.view(shp).double().sum(0) - G.sum(0)).abs() / sig_v
    err_k = dk_.view(shp).double().sum(0).abs() / sig_k
    print(f"{sh.name}: |sum dV - sum dO| / sqrt(sum sq) max {err_v.max().item():.3g}, "
          f"|sum dK| / sqrt(sum sq) max {err_k.max().item():.3g}")
    assert err_v.max().item() <= 8 * 2.0 ** -8
    assert err_k.max().item() <= 8 * 2.0 ** -8
    first = [x.clone() for x in (dq_, dk_, dv_, dwg_)]
    gsa.gsa_backward(cfg, c.dq, c.dk, c.dv, c.dwg, didx, d_o, dq_, dk_, dv_, dwg_, ws)
    torch.cuda.synchronize()
    for x, y in zip(first, (dq_, dk_, dv_, dwg_)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


@pytest.mark.slow
@pytest.mark.timeout(1100)
@pytest.mark.parametrize("sh", [VGGT_CTX, PI3_LONG], ids=["vggt_ctx", "pi3_long"])
def test_backward_full_size_dkdv_rows(sh):
    """dK and dV rows at the full sizes.  The output gradient is the seeded one on
    a few rows (6 special tokens and every token of 24 windows) and zero
    elsewhere: the backward is linear in dO, so every key row's gradient is
    still defined, and the oracle evaluates listed key rows one by one from
    the non-zero rows only.  Listed rows: every token of the windows that the
    top-k sets of two of those windows select (all heads; they receive the
    selection-branch gradients through the inverse top-k lists), tokens of the
    context frames, special tokens and random rows -- so a contribution routed
    to a wrong key row shows up.  Seeded window sets, the same on both sides."""
    from gsa_testlib import Case
    rng = np.random.default_rng(sh.seed + 21)
    idx = rng.integers(0, sh.n_windows, size=(sh.n_windows, sh.n_heads, sh.topk)).astype(np.int32)
    if sh.ctx_frames and sh.ctx_exclude:  # candidates only (any sets define the backward; keep them valid)
        wpf = sh.windows_per_frame
        bad = np.isin(idx // wpf, sh.ctx_frames)
        idx[bad] = (idx[bad] + wpf) % sh.n_windows
        assert not np.isin(idx // wpf, sh.ctx_frames).any()
    c = Case(sh)
    tf = sh.tokens_per_frame
    grid = np.arange(sh.m_tokens).reshape(sh.n_frames, tf)
    wtok = grid[:, sh.n_special:].reshape(sh.n_frames, sh.grid_h // sh.pool, sh.pool, sh.grid_w // sh.pool, sh.pool)
    wtok = wtok.transpose(0, 1, 3, 2, 4).reshape(sh.n_windows, sh.pool ** 2)
    wins = rng.choice(sh.n_windows, 24, replace=False)
    keep = np.zeros(sh.m_tokens, bool)
    keep[wtok[wins].reshape(-1)] = True
    keep[rng.choice(sh.n_frames, 6, replace=False) * tf + rng.integers(0, sh.n_special, 6)] = True
    d_o_h = gen.make_output_grad(sh).reshape(sh.m_tokens, -1).copy()
    d_o_h[~keep] = 0
    d_o_h = d_o_h.reshape(sh.qkv_shape)
    d_o = to_dev(d_o_h, sh.dtype)
    dq_, dk_, dv_ = (torch.empty(sh.qkv_shape, dtype=torch.float32, device=DEV) for _ in range(3))
    dwg_ = torch.empty((sh.n_heads, sh.head_dim), dtype=torch.float32, device=DEV)
    ws = workspace(c.cfg, gsa.GSA_OP_BACKWARD)
    gsa.gsa_backward(c.cfg, c.dq, c.dk, c.dv, c.dwg, torch.from_numpy(idx).to(DEV), d_o, dq_, dk_, dv_, dwg_, ws)
    torch.cuda.synchronize()
    del ws
    selected = np.unique(idx[wins[:2]].reshape(-1))
    parts = [wtok[selected].reshape(-1), rng.choice(sh.m_tokens, 512, replace=False),
             grid[:, :sh.n_special].reshape(-1)[:64], wtok[wins[:2]].reshape(-1)]
    for f in sh.ctx_frames:
        parts.append(f * tf + rng.choice(tf, 128, replace=False))
    rows = np.unique(np.concatenate(parts))
    shp = (sh.m_tokens, sh.n_heads, sh.head_dim)
    sel = torch.from_numpy(rows).to(DEV)
    got_k = dk_.view(shp).index_select(0, sel).cpu().numpy()
    got_v = dv_.view(shp).index_select(0, sel).cpu().numpy()
    ref_k, ref_v = oracle.backward_dkdv_rows(sh, c.q, c.k, c.v, c.wg, idx, d_o_h, rows)
    for got, ref, what in ((got_k, ref_k, "dK"), (got_v, ref_v, "dV")):
        mx, mean = assert_grad_close(got, ref, sh.dtype, f"{sh.name} sampled {what} rows")
        nz = int((np.abs(ref).max(axis=(1, 2)) > 0).sum())
        print(f"{sh.name}: {what} of {rows.size} rows ({nz} with non-zero gradients) max {mx:.3g} "
              f"mean {mean:.3g} of the largest |ref|")


# ---- the training pair: forward saving its state, backward reading it ----------

TRAIN_SHAPES = ["tiny_f32", "odd_bf16", "mid_bf16", "s8", "s5", "p0", "ctx", "ctx_f32", "k40"]


def train_pair(sh, q, k, v, wg, d_o):
    cfg = gsa.GSAConfig.from_shape(sh)
    dq, dk, dv, dw = (to_dev(x, sh.dtype) for x in (q, k, v, wg))
    o = torch.zeros(sh.qkv_shape, dtype=dq.dtype, device=DEV)
    state = torch.empty(gsa.gsa_train_state_size(cfg), dtype=torch.uint8, device=DEV)
    gsa.gsa_forward_train(cfg, dq, dk, dv, dw, o, state, workspace(cfg, gsa.GSA_OP_FORWARD))
    grads = [torch.empty(sh.qkv_shape, dtype=torch.float32, device=DEV) for _ in range(3)]
    grads.append(torch.empty((sh.n_heads, sh.head_dim), dtype=torch.float32, device=DEV))
    gsa.gsa_backward_train(cfg, dq, dk, dv, dw, state, to_dev(d_o, sh.dtype), *grads,
                           workspace(cfg, gsa.GSA_OP_BACKWARD))
    torch.cuda.synchronize()
    idx = state[:sh.n_windows * sh.n_heads * sh.topk * 4].view(torch.int32).view(sh.n_windows, sh.n_heads, sh.topk)
    return o, idx, grads


@pytest.mark.parametrize("name", TRAIN_SHAPES)
def test_training_pair(name):
    """gsa_forward_train writes gsa_forward's output bit for bit and the top-k sets
    of gsa_compressed_attn_topk; gsa_backward_train equals gsa_backward on those
    sets (the only difference: the compressed output and its log-sum-exp come
    from the forward's bound sweep instead of a plain sweep, a rounding-level
    change); and, where the forward's sets equal the oracle's for every
    (window, head), the gradients match the oracle's."""
    from gsa_testlib import Case, same_sets
    sh = SHAPES[name]
    q, k, v, wg = gen.make_inputs(sh)
    d_o = gen.make_output_grad(sh)
    o, idx, grads = train_pair(sh, q, k, v, wg, d_o)
    c = Case(sh, q=q, k=k, v=v, wg=wg)
    assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                       (lambda x: x.view(torch.int16) if x.dtype == torch.bfloat16 else x)(c.forward()))
    qc, kc, vc = c.pool()
    _, idx_c, _ = c.compressed(qc, kc, vc, with_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_c)
    gidx = idx.cpu().numpy()
    ref_gpu = gpu_backward(sh, q, k, v, wg, gidx, d_o)
    for g_, r_, what in zip(grads, ref_gpu, ("dq", "dk", "dv", "dwg")):
        g_, r_ = g_.cpu().numpy().astype(np.float64), r_.cpu().numpy().astype(np.float64)
        scale = max(np.abs(r_).max(), 1e-30)
        tol = 1e-5 if sh.dtype == F32 else 2e-3
        assert np.abs(g_ - r_).max() <= tol * scale, (name, what, np.abs(g_ - r_).max() / scale)
    oidx = oracle_topk(sh, q, k)
    if not same_sets(gidx, oidx).all():
        pytest.skip(f"{name}: the forward's top-k sets differ from the oracle's within the tie band")
    ref = oracle.backward(sh, q, k, v, wg, oidx, d_o)
    for g_, r_, what in zip(grads, ref, ("dq", "dk", "dv", "dwg")):
        assert_grad_close(g_.cpu().numpy().reshape(r_.shape), r_, sh.dtype, f"{name} train {what}")


def test_backward_with_repeated_and_missing_windows():
    """Caller-supplied top-k lists may repeat a window (its keys then enter the
    softmax twice, as in the forward) and hold -1 or out-of-range entries
    (skipped); the key side's inverse lists keep both copies.  Both sides get the
    same lists."""
    sh = SHAPES["odd_bf16"]
    q, k, v, wg = gen.make_inputs(sh)
    d_o = gen.make_output_grad(sh)
    idx = oracle_topk(sh, q, k).copy()
    idx[:, :, 1] = idx[:, :, 0]        # a repeated window in every list
    idx[::2, :, 3] = -1                # missing entries
    idx[1::3, 0, 4] = sh.n_windows + 7  # out of range: skipped
    ref_idx = np.where(idx >= sh.n_windows, -1, idx).astype(np.int32)
    got = [x.cpu().numpy() for x in gpu_backward(sh, q, k, v, wg, idx, d_o)]
    ref = oracle.backward(sh, q, k, v, wg, ref_idx, d_o)
    for g_, r_, what in zip(got, ref, ("dq", "dk", "dv", "dwg")):
        assert_grad_close(g_.reshape(r_.shape), r_, sh.dtype, f"repeated/missing {what}")


@pytest.mark.parametrize("sh", [
    GSAShape("longlists 10f-16x16-h2-s4-k8", 10, 1, 16, 16, 2, 64, 4, 8, BF16, seed=43),
    GSAShape("longlists 9f-16x16-h1-s1-k4", 9, 1, 16, 16, 1, 64, 1, 4, BF16, seed=44),
], ids=["lists160", "lists2304"])
def test_backward_long_inverse_lists(sh):
    """Every image key row identical: all guide scores tie, every query window
    selects the k lowest windows, and each of those is on the inverse list of
    every query window -- 160 entries (sorted in LDS) or 2304 (beyond the LDS
    sort, ranked), where the seeded lists hold about k."""
    q, k, v, wg = gen.make_inputs(sh)
    K = k.reshape(sh.n_frames, sh.tokens_per_frame, -1)
    K[:, sh.n_special:] = K[0, sh.n_special]
    k = K.reshape(sh.qkv_shape)
    d_o = gen.make_output_grad(sh)
    idx = oracle_topk(sh, q, k)
    assert np.all(idx[..., :sh.topk] == np.arange(sh.topk))
    got = [x.cpu().numpy() for x in gpu_backward(sh, q, k, v, wg, idx, d_o)]
    ref = oracle.backward(sh, q, k, v, wg, idx, d_o)
    for g_, r_, what in zip(got, ref, ("dq", "dk", "dv", "dwg")):
        assert_grad_close(g_.reshape(r_.shape), r_, sh.dtype, f"{sh.name} {what}")
