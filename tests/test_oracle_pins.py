"""Pins of the CPU oracle against facts fixed by the pages' definitions.

The pages print no worked GSA example, so every pin here is a special case,
a closed form, brute force or a library routine reached by a different route
than the oracle's own loops (numpy reshapes for the window geometry, torch's
scaled_dot_product_attention in float64 for softmax attention, masks instead
of gathers, lexsort for ordering).  Each test names the pin and the passage
(Paper-Notes page "Speed3R: Sparse Feed-forward 3D Reconstruction Models")
it follows.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gen.configs import BF16, F32, GSAShape


def shape(**kw):
    base = dict(name="pin", n_frames=2, n_special=1, grid_h=8, grid_w=8, n_heads=2, head_dim=16,
                pool=2, topk=3, dtype=F32, seed=7)
    base.update(kw)
    return GSAShape(**base)


def f64(x, sh):
    return gen.to_f32(x, sh.dtype).astype(np.float64)


# ---- independent geometry: numpy reshapes, not the oracle's index arithmetic ----

def token_grid(sh):
    return np.arange(sh.m_tokens, dtype=np.int64).reshape(sh.n_frames, sh.tokens_per_frame)


def window_token_ids(sh):
    """[M'][s*s] token rows of each window, from reshapes of the token grid."""
    s, gh, gw = sh.pool, sh.grid_h, sh.grid_w
    img = token_grid(sh)[:, sh.n_special:].reshape(sh.n_frames, gh // s, s, gw // s, s)
    return img.transpose(0, 1, 3, 2, 4).reshape(-1, s * s)


def image_token_ids(sh):
    return token_grid(sh)[:, sh.n_special:].reshape(-1)


def special_token_ids(sh):
    return token_grid(sh)[:, :sh.n_special].reshape(-1)


def sdpa(qrows, krows, vrows, scale, mask=None):
    """softmax(scale q k^T [+mask]) v in float64 via torch's library routine."""
    q = torch.from_numpy(np.ascontiguousarray(qrows))[None]
    k = torch.from_numpy(np.ascontiguousarray(krows))[None]
    v = torch.from_numpy(np.ascontiguousarray(vrows))[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0].numpy()


def flat(x, sh):
    return f64(x, sh).reshape(sh.m_tokens, sh.n_heads, sh.head_dim)


# ---------------------------------------------------------------------------
# P1 -- pooling is the window mean (section "压缩分支", s x s average pooling)

@pytest.mark.parametrize("s", [1, 2, 4])
def test_pool_integer_inputs_equal_window_mean(s):
    sh = shape(pool=s, grid_h=8, grid_w=8)
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 9, size=sh.qkv_shape).astype(np.float32)
    got = oracle.pool(sh, x)
    ref = x.astype(np.float64).reshape(sh.m_tokens, sh.n_heads, sh.head_dim)[window_token_ids(sh)].mean(1)
    np.testing.assert_array_equal(got.astype(np.float64), ref)  # small integers: exact


def test_pool_constant_window_and_identity():
    sh = shape(pool=1)
    q, _, _, _ = gen.make_inputs(sh)
    np.testing.assert_array_equal(oracle.pool(sh, q), f64(q, sh)[:, 1:].reshape(-1, 2, 16))
    sh4 = shape(pool=4)
    x = np.full(sh4.qkv_shape, 0.3, np.float32)
    np.testing.assert_array_equal(oracle.pool(sh4, x), np.float32(0.3) * np.ones((sh4.n_windows, 2, 16)))


def test_pool_bf16_rounds_the_fp32_mean():
    sh = shape(pool=4, dtype=BF16)
    x, _, _, _ = gen.make_inputs(sh)
    got = oracle.pool(sh, x).astype(np.float64)
    ref = flat(x, sh)[window_token_ids(sh)].mean(1)
    # the stored value is a bf16 number within half a bf16 ulp (plus fp32 sum error) of the mean
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)
    bits = got.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


# ---------------------------------------------------------------------------
# P5 -- special tokens: dense softmax attention over all M tokens
# (section "全局稀疏注意力（GSA）核心设计", special-token equation)

@pytest.mark.parametrize("dtype", [F32, BF16])
def test_special_equals_dense_attention(dtype):
    sh = shape(n_special=3, dtype=dtype)
    q, k, v, _ = gen.make_inputs(sh)
    rows = np.arange(sh.m_spec)
    got = oracle.special(sh, q, k, v, rows)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    for h in range(sh.n_heads):
        ref = sdpa(Q[special_token_ids(sh), h], K[:, h], V[:, h], sh.head_dim ** -0.5)
        np.testing.assert_allclose(got[:, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_dense_rows_equal_sdpa_over_all_tokens(dtype):
    """Dense global attention (the benchmark comparator's definition) of listed
    rows, special and image, in any order: float64 SDPA over every token."""
    sh = shape(n_special=2, dtype=dtype)
    q, k, v, _ = gen.make_inputs(sh)
    rows = np.random.default_rng(4).permutation(sh.m_tokens)[:40]
    got = oracle.dense(sh, q, k, v, rows)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    for h in range(sh.n_heads):
        ref = sdpa(Q[rows, h], K[:, h], V[:, h], sh.head_dim ** -0.5)
        np.testing.assert_allclose(got[:, h], ref, rtol=0, atol=1e-12)
    # the special rows equal the special-token attention's
    spec = special_token_ids(sh)
    np.testing.assert_allclose(oracle.dense(sh, q, k, v, spec), oracle.special(sh, q, k, v, np.arange(sh.m_spec)),
                               rtol=0, atol=1e-14)


def test_special_custom_scale_is_applied():
    sh = shape(n_special=2)
    q, k, v, _ = gen.make_inputs(sh)
    rows = np.arange(sh.m_spec)
    c = oracle.cfg_of(sh, scale=0.5)
    out = np.empty((rows.size, sh.n_heads, sh.head_dim))
    oracle._load().orc_special(oracle.ctypes.byref(c), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                               rows.astype(np.int64).ctypes.data, rows.size, out.ctypes.data)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    ref = sdpa(Q[special_token_ids(sh), 1], K[:, 1], V[:, 1], 0.5)
    np.testing.assert_allclose(out[:, 1], ref, atol=1e-12)


# ---------------------------------------------------------------------------
# Compressed attention (section "压缩分支": O'_comp = Attention(Q_comp, K_comp, V_comp))

def test_compressed_attention_equals_dense_on_pooled():
    sh = shape(pool=2)
    q, k, v, _ = gen.make_inputs(sh)
    qc, kc, vc = oracle.pool(sh, q), oracle.pool(sh, k), oracle.pool(sh, v)
    wins = np.arange(sh.n_windows)
    oc, _, _, _ = oracle.compressed(sh, qc, kc, vc, wins)
    for h in range(sh.n_heads):
        ref = sdpa(qc[:, h].astype(np.float64), kc[:, h].astype(np.float64), vc[:, h].astype(np.float64),
                   sh.head_dim ** -0.5)
        np.testing.assert_allclose(oc[:, h], ref, atol=1e-12)


# ---------------------------------------------------------------------------
# P8 -- top-k over the guide scores S = Q_comp K_comp^T (section "压缩分支"
# guide-score equation; section "选择分支" TopKSelect), ties to the lower index

def _int_pooled(sh, seed):
    rng = np.random.default_rng(seed)
    shp = (sh.n_windows, sh.n_heads, sh.head_dim)
    return [rng.integers(-3, 4, size=shp).astype(np.float32) for _ in range(3)]


@pytest.mark.parametrize("topk", [1, 3, 16])
def test_topk_equals_full_sort(topk):
    sh = shape(topk=topk, head_dim=8)
    qc, kc, vc = _int_pooled(sh, 3)  # integer scores: exact in double, so ties are real ties
    wins = np.arange(sh.n_windows)
    _, idx, sc, _ = oracle.compressed(sh, qc, kc, vc, wins)
    for h in range(sh.n_heads):
        S = qc[:, h].astype(np.float64) @ kc[:, h].astype(np.float64).T
        for i in range(sh.n_windows):
            order = np.lexsort((np.arange(sh.n_windows), -S[i]))  # score desc, then index asc
            np.testing.assert_array_equal(idx[i, h], order[:topk])
            np.testing.assert_array_equal(sc[i, h, :topk], S[i, order[:topk]])
            assert sc[i, h, topk] == S[i, order[topk]]


def test_topk_ties_go_to_lower_index():
    sh = shape(topk=2, head_dim=8)
    qc, kc, vc = _int_pooled(sh, 4)
    kc[:] = kc[5]  # every key window identical -> every score tied
    _, idx, _, _ = oracle.compressed(sh, qc, kc, vc, np.arange(sh.n_windows))
    assert np.all(idx == np.array([0, 1], np.int32))


def test_topk_clamps_and_excludes_context_windows():
    sh = shape(topk=100, ctx_frames=(1,), n_frames=3)
    qc, kc, vc = _int_pooled(sh, 5)
    _, idx, sc, _ = oracle.compressed(sh, qc, kc, vc, np.arange(sh.n_windows))
    wpf = sh.windows_per_frame
    ncand = 2 * wpf
    assert np.all(idx[..., ncand:] == -1)
    real = idx[..., :ncand]
    assert np.all((real // wpf) != 1)  # context frame windows are never candidates
    assert np.all(np.sort(real, axis=-1) == np.concatenate([np.arange(wpf), np.arange(2 * wpf, 3 * wpf)]))
    assert np.all(np.isnan(sc[..., ncand + 1:]))


# ---------------------------------------------------------------------------
# Selection branch (section "选择分支"; fixed context: section "Speed3R-VGGT 适配")

def _selection_mask(sh, idx_h):
    """[M_img][M] additive mask of the keys each image query may attend, built from window sets."""
    wt = window_token_ids(sh)
    img = image_token_ids(sh)
    pos = {int(t): r for r, t in enumerate(img)}
    mask = np.full((sh.m_img, sh.m_tokens), -np.inf)
    for i in range(sh.n_windows):
        keys = np.concatenate([wt[j] for j in idx_h[i] if j >= 0] +
                              [token_grid(sh)[f] for f in sh.ctx_frames])
        for t in wt[i]:
            mask[pos[int(t)], keys] = 0.0
    return mask


@pytest.mark.parametrize("ctx", [(), (1,)])
def test_selection_equals_masked_dense_attention(ctx):
    sh = shape(n_frames=3, topk=3, ctx_frames=ctx)
    q, k, v, _ = gen.make_inputs(sh)
    qc, kc, vc = oracle.pool(sh, q), oracle.pool(sh, k), oracle.pool(sh, v)
    wins = np.arange(sh.n_windows)
    _, idx, _, _ = oracle.compressed(sh, qc, kc, vc, wins)
    osel = oracle.select(sh, q, k, v, wins, idx)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    img = image_token_ids(sh)
    wt = window_token_ids(sh)
    pos = {int(t): r for r, t in enumerate(img)}
    for h in range(sh.n_heads):
        ref = sdpa(Q[img, h], K[:, h], V[:, h], sh.head_dim ** -0.5, _selection_mask(sh, idx[:, h]))
        got = np.empty_like(ref)
        for i in range(sh.n_windows):
            for qq, t in enumerate(wt[i]):
                got[pos[int(t)]] = osel[i, qq, h]
        np.testing.assert_allclose(got, ref, atol=1e-12)


def test_P2_topk_covering_all_windows_is_dense_image_attention():
    sh = shape(topk=10 ** 6)
    q, k, v, _ = gen.make_inputs(sh)
    wins = np.arange(sh.n_windows)
    idx = np.tile(np.arange(sh.n_windows, dtype=np.int32), (sh.n_windows, sh.n_heads, 1))
    osel = oracle.select(sh, q, k, v, wins, idx)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    wt = window_token_ids(sh)
    img = image_token_ids(sh)
    for h in range(sh.n_heads):
        ref = sdpa(Q[wt.reshape(-1), h], K[img, h], V[img, h], sh.head_dim ** -0.5)
        np.testing.assert_allclose(osel[:, :, h].reshape(-1, sh.head_dim), ref, atol=1e-12)


def test_P9_context_every_frame_is_dense_attention_over_all_tokens():
    sh = shape(n_frames=2, topk=4, ctx_frames=(0, 1))
    q, k, v, _ = gen.make_inputs(sh)
    qc, kc, vc = oracle.pool(sh, q), oracle.pool(sh, k), oracle.pool(sh, v)
    wins = np.arange(sh.n_windows)
    _, idx, _, _ = oracle.compressed(sh, qc, kc, vc, wins)
    assert np.all(idx == -1)  # no candidates left
    osel = oracle.select(sh, q, k, v, wins, idx)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    wt = window_token_ids(sh)
    for h in range(sh.n_heads):
        ref = sdpa(Q[wt.reshape(-1), h], K[:, h], V[:, h], sh.head_dim ** -0.5)
        np.testing.assert_allclose(osel[:, :, h].reshape(-1, sh.head_dim), ref, atol=1e-12)


# ---------------------------------------------------------------------------
# Upsample + gate (section "压缩分支" upsampling; section "门控聚合")

def test_P4_explicit_gates_select_one_branch():
    sh = shape()
    q, k, v, wg = gen.make_inputs(sh)
    wins = np.arange(sh.n_windows)
    rng = np.random.default_rng(0)
    oc = rng.standard_normal((sh.n_windows, sh.n_heads, sh.head_dim))
    osel = rng.standard_normal((sh.n_windows, 4, sh.n_heads, sh.head_dim))
    g0 = np.zeros((sh.n_windows, 4, sh.n_heads))
    np.testing.assert_array_equal(oracle.gate_combine(sh, q, None, wins, oc, osel, g0), osel)
    g1 = np.ones_like(g0)
    np.testing.assert_array_equal(oracle.gate_combine(sh, q, None, wins, oc, osel, g1),
                                  np.broadcast_to(oc[:, None], osel.shape))
    # W_g = 0 gives g = 1/2 exactly: the midpoint
    mid = oracle.gate_combine(sh, q, np.zeros_like(wg), wins, oc, osel)
    np.testing.assert_allclose(mid, 0.5 * (oc[:, None] + osel), atol=1e-15)


def test_gate_direction_large_logit_picks_compressed_branch():
    sh = shape()
    q, _, _, wg = gen.make_inputs(sh)
    q = np.abs(q)  # q . W_g > 0 everywhere when W_g >= 0 ...
    wg = np.full_like(wg, 50.0)  # ... and very large, so g = sigmoid(.) ~ 1
    wins = np.arange(sh.n_windows)
    rng = np.random.default_rng(1)
    oc = rng.standard_normal((sh.n_windows, sh.n_heads, sh.head_dim))
    osel = rng.standard_normal((sh.n_windows, 4, sh.n_heads, sh.head_dim))
    out = oracle.gate_combine(sh, q, wg, wins, oc, osel)
    np.testing.assert_allclose(out, np.broadcast_to(oc[:, None], osel.shape), atol=1e-12)
    out = oracle.gate_combine(sh, q, -wg, wins, oc, osel)
    np.testing.assert_allclose(out, osel, atol=1e-12)


def test_forward_upsample_gate_one_gives_each_token_its_window_output():
    sh = shape()
    q, k, v, wg = gen.make_inputs(sh)
    g1 = np.ones((sh.n_windows, 4, sh.n_heads))
    res = oracle.forward(sh, q, k, v, wg, gate=g1)
    qc, kc, vc = oracle.pool(sh, q), oracle.pool(sh, k), oracle.pool(sh, v)
    O = res["o"].reshape(sh.m_tokens, sh.n_heads, sh.head_dim)
    wt = window_token_ids(sh)
    for h in range(sh.n_heads):
        comp = sdpa(qc[:, h].astype(np.float64), kc[:, h].astype(np.float64),
                    vc[:, h].astype(np.float64), sh.head_dim ** -0.5)
        for i in range(sh.n_windows):
            np.testing.assert_allclose(O[wt[i], h], np.broadcast_to(comp[i], (4, sh.head_dim)), atol=1e-12)


# ---------------------------------------------------------------------------
# P3, P6, P7 -- whole-forward special cases

def test_P3_pool1_all_windows_any_gate_is_dense_image_attention():
    sh = shape(pool=1, topk=10 ** 6, n_special=2)
    q, k, v, wg = gen.make_inputs(sh)
    gate = np.random.default_rng(2).random((sh.n_windows, 1, sh.n_heads))
    res = oracle.forward(sh, q, k, v, wg, gate=gate)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    O = res["o"].reshape(sh.m_tokens, sh.n_heads, sh.head_dim)
    img = image_token_ids(sh)
    for h in range(sh.n_heads):
        ref = sdpa(Q[img, h], K[img, h], V[img, h], sh.head_dim ** -0.5)
        np.testing.assert_allclose(O[img, h], ref, atol=1e-12)


@pytest.mark.parametrize("ctx", [(), (0,)])
def test_P6_constant_values_give_constant_output(ctx):
    sh = shape(n_frames=3, ctx_frames=ctx, n_special=2)
    q, k, _, wg = gen.make_inputs(sh)
    c = np.random.default_rng(3).standard_normal((sh.n_heads, sh.head_dim)).astype(np.float32)
    v = np.broadcast_to(c, sh.qkv_shape).copy()
    res = oracle.forward(sh, q, k, v, wg)
    np.testing.assert_allclose(res["o"], np.broadcast_to(c.astype(np.float64), sh.qkv_shape), atol=1e-12)


def test_P7_single_window():
    sh = shape(n_frames=1, grid_h=4, grid_w=4, pool=4, topk=32, n_special=1)
    q, k, v, wg = gen.make_inputs(sh)
    res = oracle.forward(sh, q, k, v, wg)
    assert sh.n_windows == 1
    assert res["topk"].tolist() == [[[0] + [-1] * 31] * sh.n_heads]
    np.testing.assert_allclose(res["oc"][0], res["vc"][0].astype(np.float64), atol=1e-12)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    img = image_token_ids(sh)
    for h in range(sh.n_heads):
        ref = sdpa(Q[img, h], K[img, h], V[img, h], sh.head_dim ** -0.5)
        np.testing.assert_allclose(res["osel"][0, :, h], ref, atol=1e-12)


# ---------------------------------------------------------------------------
# generator sanity (not the method: the inputs' recipe)

def test_generator_is_deterministic_and_standard_normal():
    a = gen.normal((1 << 18,), F32, 11, 1)
    b = gen.normal((1 << 18,), F32, 11, 1)
    np.testing.assert_array_equal(a, b)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    c = gen.normal((1000,), F32, 11, 1, offset=500)
    np.testing.assert_array_equal(c[:500], a[500:1000])
    assert not np.array_equal(a[:1000], gen.normal((1000,), F32, 11, 2))
    bf = gen.normal((1000,), BF16, 11, 1)
    np.testing.assert_allclose(gen.to_f32(bf, BF16), a[:1000], rtol=2 ** -8)


def test_clustered_recipe_windows_share_a_centroid():
    sh = shape(recipe="clustered", pool=4, n_heads=2, head_dim=16)
    k = gen.to_f32(gen.clustered(sh, 5, 2, 5, 7), F32).astype(np.float64)
    K = k.reshape(sh.m_tokens, sh.n_heads, sh.head_dim)
    wt = window_token_ids(sh)
    spread = K[wt].std(axis=1)  # within-window spread = the 0.1 noise
    assert 0.06 < spread.mean() < 0.14
    assert K[special_token_ids(sh)].std() > 0.7


def test_guide_scores_are_the_raw_dot_products():
    """S_ij = Q_comp_i . K_comp_j, unscaled (section "压缩分支", guide-score equation);
    integer-valued pooled rows make the products exact, so equality is exact."""
    sh = shape(head_dim=8, topk=5)
    qc, kc, _ = _int_pooled(sh, 9)
    wins = np.array([0, 3, sh.n_windows - 1])
    idx = np.array([[[1, 0, 7, -1, 5]] * sh.n_heads] * 3, np.int32)
    got = oracle.guide_scores(sh, qc, kc, wins, idx)
    for a, i in enumerate(wins):
        for h in range(sh.n_heads):
            for t, j in enumerate(idx[a, h]):
                if j < 0:
                    assert np.isnan(got[a, h, t])
                else:
                    assert got[a, h, t] == float(qc[i, h].astype(np.int64) @ kc[j, h].astype(np.int64))


# ---------------------------------------------------------------------------
# P10 -- frame attention, the local step that alternates with GSA (section
# "整体框架"): dense attention restricted to each frame, i.e. all-token
# attention under a block-diagonal mask whose blocks are the frames.

@pytest.mark.parametrize("dtype,n_special", [(F32, 0), (F32, 2), (BF16, 3)])
def test_frame_attention_equals_block_diagonal_masked_attention(dtype, n_special):
    sh = shape(n_frames=3, n_special=n_special, grid_h=6, grid_w=4, dtype=dtype)
    q, k, v, _ = gen.make_inputs(sh)
    rows = np.arange(sh.m_tokens)
    got = oracle.frame(sh, q, k, v, rows)
    frame_of = np.repeat(np.arange(sh.n_frames), sh.tokens_per_frame)  # from the token grid's rows
    mask = np.where(frame_of[:, None] == frame_of[None, :], 0.0, -np.inf)
    Q, K, V = flat(q, sh), flat(k, sh), flat(v, sh)
    for h in range(sh.n_heads):
        ref = sdpa(Q[:, h], K[:, h], V[:, h], sh.head_dim ** -0.5, mask)
        np.testing.assert_allclose(got[:, h], ref, rtol=0, atol=1e-12)


def test_frame_attention_of_one_frame_is_the_special_rows_dense_attention():
    """With a single frame every token's frame is the whole sequence, so the special
    rows' frame attention is the special-token attention over all M tokens."""
    sh = shape(n_frames=1, n_special=3)
    q, k, v, _ = gen.make_inputs(sh)
    got = oracle.frame(sh, q, k, v, special_token_ids(sh))
    ref = oracle.special(sh, q, k, v, np.arange(sh.m_spec))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_frame_attention_equal_keys_average_the_frame_values():
    """Equal keys inside each frame give uniform weights: every output row is the mean
    of its own frame's value rows (catches a key range off by one token or frame)."""
    sh = shape(n_frames=3, n_special=1, grid_h=4, grid_w=6)
    q, _, v, _ = gen.make_inputs(sh)
    k = np.broadcast_to(np.float32(0.25), sh.qkv_shape).copy()
    got = oracle.frame(sh, q, k, v, np.arange(sh.m_tokens))
    V = flat(v, sh).reshape(sh.n_frames, sh.tokens_per_frame, sh.n_heads, sh.head_dim)
    ref = np.repeat(V.mean(1), sh.tokens_per_frame, axis=0)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# P11 -- FlashVGGT descriptor attention (Paper-Notes page "FlashVGGT: Efficient
# and Scalable Visual Geometry Transformers with Compressed Descriptor
# Attention", section "关键设计"; auxiliary tokens from "关键发现").  The
# downsampling factor r is the config's pool field, the keyframes its
# ctx_frames.

def _image_planes(x64, sh):
    """[N][T_f][H][d] -> torch [N, H*d, h, w] of the image tokens (float64)."""
    img = x64.reshape(sh.n_frames, sh.tokens_per_frame, sh.n_heads * sh.head_dim)[:, sh.n_special:]
    img = img.reshape(sh.n_frames, sh.grid_h, sh.grid_w, -1).transpose(0, 3, 1, 2)
    return torch.from_numpy(np.ascontiguousarray(img))


def _torch_descriptors(x64, sh):
    r = sh.pool
    out = torch.nn.functional.interpolate(_image_planes(x64, sh), size=(sh.grid_h // r, sh.grid_w // r),
                                          mode="bilinear", align_corners=False)
    return out.permute(0, 2, 3, 1).reshape(-1, sh.n_heads, sh.head_dim).numpy()


def _aux_token_ids(sh, keyframes):
    grid = token_grid(sh)
    full = [0] + [f for f in keyframes if f != 0]
    rest = [f for f in range(sh.n_frames) if f not in full]
    return np.concatenate([grid[full].reshape(-1), grid[rest, :sh.n_special].reshape(-1)])


@pytest.mark.parametrize("r", [1, 2, 3, 4])
def test_descriptors_equal_torch_bilinear_resampling(r):
    sh = shape(n_frames=2, n_special=2, grid_h=12, grid_w=12, pool=r)
    _, k, _, _ = gen.make_inputs(sh)
    got = oracle.descriptor_set(sh, k).astype(np.float64)
    nd = sh.n_frames * (sh.grid_h // r) * (sh.grid_w // r)
    ref = _torch_descriptors(f64(k, sh), sh)
    # four weighted corners summed in float: at most 3 roundings of partial
    # sums bounded by the sum of the terms' magnitudes
    bound = 3 * 2.0 ** -24 * _torch_descriptors(np.abs(f64(k, sh)), sh)
    assert np.all(np.abs(got[:nd] - ref) <= bound + 1e-30)
    if r % 2 == 1:  # odd r samples one pixel exactly
        np.testing.assert_array_equal(got[:nd], ref)


def test_descriptors_r4_are_the_mean_of_the_central_2x2():
    """Half-pixel centres at r = 4 sample between rows 4y+1 and 4y+2 (weights 1/2 each)."""
    sh = shape(n_frames=2, n_special=1, grid_h=8, grid_w=12, pool=4)
    rng = np.random.default_rng(4)
    x = rng.integers(-8, 9, size=sh.qkv_shape).astype(np.float32)
    got = oracle.descriptor_set(sh, x)
    img = x.astype(np.float64).reshape(sh.n_frames, sh.tokens_per_frame, -1)[:, 1:]
    img = img.reshape(sh.n_frames, 2, 4, 3, 4, sh.n_heads, sh.head_dim)
    ref = img[:, :, 1:3, :, 1:3].mean(axis=(2, 4)).reshape(-1, sh.n_heads, sh.head_dim)
    np.testing.assert_array_equal(got[:ref.shape[0]].astype(np.float64), ref)  # small integers: exact


def test_descriptor_set_bf16_rounds_and_carries_the_auxiliary_tokens():
    sh = shape(n_frames=5, n_special=3, grid_h=8, grid_w=8, pool=4, dtype=BF16, ctx_frames=(3, 0))
    _, _, v, _ = gen.make_inputs(sh)
    got = oracle.descriptor_set(sh, v)
    nd = sh.n_frames * 4
    aux = _aux_token_ids(sh, (3, 0))
    assert got.shape[0] == nd + aux.size == nd + 2 * sh.tokens_per_frame + 3 * sh.n_special
    np.testing.assert_array_equal(got[nd:].astype(np.float64), flat(v, sh)[aux])
    ref = _torch_descriptors(f64(v, sh), sh)
    assert np.all(np.abs(got[:nd] - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)
    assert np.all(got[:nd].view(np.uint32) & 0xFFFF == 0)


@pytest.mark.parametrize("keyframes", [(), (2,)])
def test_descriptor_attention_equals_attention_over_the_set(keyframes):
    sh = shape(n_frames=4, n_special=2, grid_h=8, grid_w=8, pool=4, ctx_frames=keyframes)
    q, k, v, _ = gen.make_inputs(sh)
    rows = np.arange(sh.m_tokens)
    kd, vd = oracle.descriptor_set(sh, k), oracle.descriptor_set(sh, v)
    got = oracle.descriptor_attn(sh, q, kd, vd, rows)
    # the set rebuilt from torch's resampling and numpy indexing
    aux = _aux_token_ids(sh, keyframes)
    K = np.concatenate([_torch_descriptors(f64(k, sh), sh), flat(k, sh)[aux]])
    V = np.concatenate([_torch_descriptors(f64(v, sh), sh), flat(v, sh)[aux]])
    Q = flat(q, sh)
    for h in range(sh.n_heads):
        ref = sdpa(Q[:, h], K[:, h], V[:, h], sh.head_dim ** -0.5)
        np.testing.assert_allclose(got[:, h], ref, rtol=0, atol=2e-6)


# ---------------------------------------------------------------------------
# P12 -- the backward: gradients of sum(dO * O) with the top-k sets fixed
# (trained end to end: Paper-Notes page, sections "研究背景与动机", "训练策略").
# Pins: torch autograd (float64) through a forward rebuilt from masks and
# reshapes; central differences of the oracle's own forward steps on dyadic
# inputs (every pooled mean exact); the identities sum_t dV = sum_t dO and
# sum_t dK = 0 that every softmax attention obeys.

def _fixed_topk(sh, seed):
    """A valid top-k set per (window, head): distinct candidate windows, -1 padded."""
    rng = np.random.default_rng(seed)
    wpf = (sh.grid_h // sh.pool) * (sh.grid_w // sh.pool)
    cand = np.array([j for j in range(sh.n_windows) if not (sh.ctx_exclude and j // wpf in sh.ctx_frames)])
    kk = min(sh.topk, cand.size)
    idx = np.full((sh.n_windows, sh.n_heads, sh.topk), -1, np.int32)
    for i in range(sh.n_windows):
        for h in range(sh.n_heads):
            idx[i, h, :kk] = rng.choice(cand, kk, replace=False)
    return idx


def _torch_forward(sh, Q, K, V, W, idx):
    """GSA forward in float64 torch ops: pooling by reshape-mean, attention by SDPA
    under masks built from the window sets."""
    H, d, sc = sh.n_heads, sh.head_dim, sh.head_dim ** -0.5
    M, tf = sh.m_tokens, sh.tokens_per_frame
    wt = torch.from_numpy(window_token_ids(sh))            # [M'][s^2] token rows
    Qc, Kc, Vc = (X[wt].mean(1) for X in (Q, K, V))        # [M'][H][d]
    out = torch.zeros(M, H, d, dtype=torch.float64)
    spec = torch.from_numpy(special_token_ids(sh))
    img = wt.reshape(-1)                                    # image tokens, window-major
    win_of = torch.arange(sh.n_windows).repeat_interleave(sh.pool ** 2)
    frame_of_tok = torch.arange(M) // tf
    sdp = torch.nn.functional.scaled_dot_product_attention
    rows = []
    for h in range(H):
        o_h = torch.zeros(M, d, dtype=torch.float64)
        if spec.numel():
            o_h = o_h.index_put((spec,), sdp(Q[spec, h][None], K[:, h][None], V[:, h][None], scale=sc)[0])
        oc = sdp(Qc[:, h][None], Kc[:, h][None], Vc[:, h][None], scale=sc)[0]
        allowed = np.zeros((sh.n_windows, M), bool)
        for i in range(sh.n_windows):
            for j in idx[i, h]:
                if j >= 0:
                    allowed[i, window_token_ids(sh)[j]] = True
            for f in sh.ctx_frames:
                allowed[i, f * tf:(f + 1) * tf] = True
        mask = torch.from_numpy(np.where(allowed, 0.0, -np.inf))[win_of]
        osel = sdp(Q[img, h][None], K[:, h][None], V[:, h][None], attn_mask=mask[None], scale=sc)[0]
        g = torch.sigmoid(Q[img, h] @ W[h])[:, None]
        o_h = o_h.index_put((img,), g * oc[win_of] + (1 - g) * osel)
        rows.append(o_h)
    return torch.stack(rows, 1)


@pytest.mark.parametrize("kw", [dict(), dict(n_special=0, pool=4, topk=2), dict(ctx_frames=(1,), topk=2)])
def test_backward_equals_torch_autograd(kw):
    sh = shape(**kw)
    q, k, v, wg = gen.make_inputs(sh)
    d_o = gen.make_output_grad(sh)
    idx = _fixed_topk(sh, 5)
    dq, dk, dv, dwg = oracle.backward(sh, q, k, v, wg, idx, d_o)
    Q, K, V = (torch.from_numpy(flat(x, sh)).requires_grad_() for x in (q, k, v))
    W = torch.from_numpy(f64(wg, sh).reshape(sh.n_heads, sh.head_dim)).requires_grad_()
    out = _torch_forward(sh, Q, K, V, W, idx)
    (out * torch.from_numpy(flat(d_o, sh))).sum().backward()
    # the oracle's pooled rows are rounded to float, the torch means are not
    for got, ref in ((dq, Q.grad), (dk, K.grad), (dv, V.grad), (dwg, W.grad)):
        ref = ref.numpy().reshape(got.shape)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-6 * max(1.0, np.abs(ref).max()))


def _dyadic_inputs(sh, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.integers(-16, 17, size=sh.qkv_shape).astype(np.float32) / 16 for _ in range(3))
    wg = rng.integers(-4, 5, size=(sh.n_heads, sh.head_dim)).astype(np.float32) / 16
    d_o = rng.integers(-8, 9, size=sh.qkv_shape).astype(np.float32) / 8
    return q, k, v, wg, d_o


def _loss(sh, q, k, v, wg, idx, d_o):
    """sum(dO * O) from the oracle's forward steps with the top-k sets fixed."""
    wins = np.arange(sh.n_windows)
    qc, kc, vc = oracle.pool(sh, q), oracle.pool(sh, k), oracle.pool(sh, v)
    oc = oracle.compressed(sh, qc, kc, vc, wins)[0]
    osel = oracle.select(sh, q, k, v, wins, idx)
    oimg = oracle.gate_combine(sh, q, wg, wins, oc, osel)
    G = d_o.astype(np.float64).reshape(sh.m_tokens, sh.n_heads, sh.head_dim)
    L = float((G[window_token_ids(sh).reshape(-1)] * oimg.reshape(-1, sh.n_heads, sh.head_dim)).sum())
    if sh.m_spec:
        L += float((G[special_token_ids(sh)] * oracle.special(sh, q, k, v, np.arange(sh.m_spec))).sum())
    return L


def test_backward_matches_central_differences():
    sh = shape(n_frames=2, n_special=1, grid_h=4, grid_w=4, pool=2, topk=2, head_dim=8)
    q, k, v, wg, d_o = _dyadic_inputs(sh, 3)
    idx = _fixed_topk(sh, 6)
    grads = oracle.backward(sh, q, k, v, wg, idx, d_o)
    eps = 2.0 ** -10
    rng = np.random.default_rng(7)
    checked = 0
    for which, arr in enumerate((q, k, v, wg)):
        for _ in range(6):
            pos = tuple(int(rng.integers(0, n)) for n in arr.shape)
            if which < 3 and _ == 0:
                pos = (0, 0) + pos[2:]  # a special token
            plus, minus = arr.copy(), arr.copy()
            plus[pos] += eps
            minus[pos] -= eps
            args = [q, k, v, wg]
            args[which] = plus
            lp = _loss(sh, *args, idx, d_o)
            args[which] = minus
            lm = _loss(sh, *args, idx, d_o)
            fd = (lp - lm) / (2 * eps)
            g = grads[which][pos]
            assert abs(fd - g) <= 1e-5 * max(1.0, abs(g)), (which, pos, fd, g)
            checked += 1
    assert checked == 24


@pytest.mark.parametrize("kw", [dict(), dict(ctx_frames=(0,), topk=2, dtype=BF16)])
def test_backward_sum_identities(kw):
    """sum_t dV_t = sum_t dO_t and sum_t dK_t = 0 per head and channel: softmax weights
    sum to one and the score gradients of each query sum to zero."""
    sh = shape(**kw)
    q, k, v, wg = gen.make_inputs(sh)
    d_o = gen.make_output_grad(sh)
    dq, dk, dv, dwg = oracle.backward(sh, q, k, v, wg, _fixed_topk(sh, 8), d_o)
    G = flat(d_o, sh)
    np.testing.assert_allclose(dv.reshape(G.shape).sum(0), G.sum(0), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk.reshape(G.shape).sum(0), 0.0, rtol=0, atol=1e-10)


@pytest.mark.parametrize("kw", [dict(), dict(ctx_frames=(1,), topk=2, dtype=BF16), dict(n_special=0, pool=4, topk=2)])
def test_backward_dq_rows_equal_the_whole_layer_backward(kw):
    """The per-row dq (for full-size checks) is the whole-layer backward's dq,
    which the autograd and difference pins above fix."""
    sh = shape(**kw)
    q, k, v, wg = gen.make_inputs(sh)
    d_o = gen.make_output_grad(sh)
    idx = _fixed_topk(sh, 9)
    dq = oracle.backward(sh, q, k, v, wg, idx, d_o)[0].reshape(sh.m_tokens, sh.n_heads, sh.head_dim)
    rows = np.arange(sh.m_tokens)
    got = oracle.backward_dq_rows(sh, q, k, v, wg, idx, d_o, rows)
    np.testing.assert_allclose(got, dq[rows], rtol=0, atol=1e-12 * max(1.0, np.abs(dq).max()))


def _sparse_output_grad(sh, d_o, seed):
    """d_o with most rows set to zero: a few special rows and the tokens of a
    few windows keep their seeded values."""
    rng = np.random.default_rng(seed)
    keep = np.zeros(sh.m_tokens, bool)
    tf = sh.tokens_per_frame
    if sh.n_special:
        keep[rng.choice(sh.n_frames, 2) * tf + rng.integers(0, sh.n_special, 2)] = True
    img = np.arange(sh.m_tokens).reshape(sh.n_frames, tf)[:, sh.n_special:]
    keep[rng.choice(img.reshape(-1), 5, replace=False)] = True
    out = d_o.copy().reshape(sh.m_tokens, -1)
    out[~keep] = 0
    return out.reshape(d_o.shape)


@pytest.mark.parametrize("kw", [dict(), dict(ctx_frames=(1,), topk=2, dtype=BF16), dict(n_special=0, pool=4, topk=2),
                                dict(n_frames=3, ctx_frames=(0, 2), ctx_exclude=0, topk=3)])
@pytest.mark.parametrize("sparse", [False, True])
def test_backward_dkdv_rows_equal_the_whole_layer_backward(kw, sparse):
    """The per-row dK/dV (for full-size checks) are the whole-layer backward's,
    which the autograd and difference pins above fix, for a dense output
    gradient and for one that is zero on most rows (the per-row version skips
    queries with a zero incoming gradient); rows listed in a shuffled order.
    With ctx_exclude = 0 a context frame's windows may also be selected, so a
    key can sit twice in one selection set."""
    sh = shape(**kw)
    q, k, v, wg = gen.make_inputs(sh)
    d_o = gen.make_output_grad(sh)
    if sparse:
        d_o = _sparse_output_grad(sh, d_o, 13)
    idx = _fixed_topk(sh, 10)
    _, dk, dv, _ = oracle.backward(sh, q, k, v, wg, idx, d_o)
    dk = dk.reshape(sh.m_tokens, sh.n_heads, sh.head_dim)
    dv = dv.reshape(sh.m_tokens, sh.n_heads, sh.head_dim)
    rows = np.random.default_rng(3).permutation(sh.m_tokens)
    gk, gv = oracle.backward_dkdv_rows(sh, q, k, v, wg, idx, d_o, rows)
    np.testing.assert_allclose(gk, dk[rows], rtol=0, atol=1e-12 * max(1.0, np.abs(dk).max()))
    np.testing.assert_allclose(gv, dv[rows], rtol=0, atol=1e-12 * max(1.0, np.abs(dv).max()))
    if sparse:
        assert np.abs(dk).max() > 0 and np.abs(dv).max() > 0
