"""Parity at the full workload sizes, in the launch configuration the bench
times (gsa_forward), checked on sampled outputs the oracle computes one by one:

* pooled Q/K/V: every element, bit for bit;
* compressed attention and top-k: sampled query windows x all heads
  (tie-band rule for the index sets);
* the forward's image rows of those windows (oracle selection over the
  oracle's own index sets, then upsample + gate), on every (window, head)
  whose GPU set equals the oracle's (the others: valid tie-band choices, at
  most the tie-band count); and every sampled (window, head) through the
  selection and gate calls driven by the oracle's own sets in those rows;
* the forward's special rows: sampled special tokens x all heads;
* determinism: a second forward is bitwise identical;
* frame attention (the per-frame step beside GSA): sampled tokens x all heads;
* FlashVGGT descriptor attention (r = s, keyframes = the context frames): the
  key/value set bit for bit, sampled tokens x all heads.

Workloads: VGGT-style 128 frames with fixed context {0, 100}; the pi^3-style
1000-frame sequence; the peaky clustered 1024-frame sequence; an fp32
32-frame sequence with two context frames, large enough (4 096 query blocks x
heads) that one workgroup sweeps both context frames, as in the bf16
VGGT-style workload.
"""
import sys
import time

import numpy as np
import pytest
import torch

import gen
import oracle
from gen.configs import F32, PEAKY, PI3_LONG, VGGT_CTX, GSAShape
import sparse_global_attention_amd as gsa
from gsa_testlib import (Case, assert_close, assert_close_rows, check_topk, same_sets, special_token_ids, to_host,
                         window_token_ids, workspace)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CTX_F32 = GSAShape("ctx-f32 32f-32x32-h16-s4-k16+ctx{17,3}", 32, 1, 32, 32, 16, 64, 4, 16, F32,
                   ctx_frames=(17, 3), seed=1005)
WORKLOADS = {"vggt_ctx": (VGGT_CTX, 1024), "pi3_long": (PI3_LONG, 512), "peaky": (PEAKY, 512),
             "ctx_f32": (CTX_F32, 512)}
N_SPECIAL_ROWS = 64


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.timeout(1100)
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size_sampled_parity(name):
    sh, n_win = WORKLOADS[name]
    t0 = time.time()
    log(f"[{name}] {sh.name}: generating inputs")
    c = Case(sh)
    log(f"[{name}] inputs on device ({time.time() - t0:.0f} s); forward + pool + top-k on the GPU")
    out = c.forward()
    fr_rows = np.unique(np.concatenate([np.arange(sh.tokens_per_frame),
                                        np.arange(sh.m_tokens - sh.tokens_per_frame, sh.m_tokens),
                                        np.random.default_rng(sh.seed + 5).choice(sh.m_tokens, 256, replace=False)]))
    fr = c.frame()
    o_frame = to_host(fr.view(sh.m_tokens, sh.n_heads, sh.head_dim).index_select(
        0, torch.from_numpy(fr_rows).cuda()))
    del fr
    kd, vd = c.descriptor_set()
    de = c.descriptor_attn(kd, vd)
    de_rows = np.unique(np.concatenate([[0, sh.m_tokens - 1],
                                        np.random.default_rng(sh.seed + 6).choice(sh.m_tokens, 30, replace=False)]))
    o_desc = to_host(de.view(sh.m_tokens, sh.n_heads, sh.head_dim).index_select(0, torch.from_numpy(de_rows).cuda()))
    g_set = [x.float().cpu().numpy() for x in (kd, vd)]
    del de, kd, vd
    qc, kc, vc = c.pool()
    oc, idx, _ = c.compressed(qc, kc, vc, with_scores=False)
    again = c.forward()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "forward is not deterministic"
    del again

    wins = gen.sample_windows(sh, n_win)
    rows = gen.sample_special(sh, N_SPECIAL_ROWS)
    wtok = torch.from_numpy(window_token_ids(sh)[wins].reshape(-1)).cuda()
    stok = torch.from_numpy(special_token_ids(sh)[rows]).cuda()
    o_img = to_host(out.view(sh.m_tokens, sh.n_heads, sh.head_dim).index_select(0, wtok))
    o_spec = to_host(out.view(sh.m_tokens, sh.n_heads, sh.head_dim).index_select(0, stok))
    gidx = idx.index_select(0, torch.from_numpy(wins).cuda()).cpu().numpy()
    goc = to_host(oc.index_select(0, torch.from_numpy(wins).cuda()))
    gpooled = [x.float().cpu().numpy() for x in (qc, kc, vc)]
    idx_full, oc_full = idx, oc  # kept for the selection + gate calls with the oracle's sets
    del out, qc, kc, vc
    torch.cuda.empty_cache()

    log(f"[{name}] oracle: pooling ({time.time() - t0:.0f} s)")
    pooled = [oracle.pool(sh, x) for x in (c.q, c.k, c.v)]
    for g, o, what in zip(gpooled, pooled, "QKV"):
        assert np.array_equal(g.view(np.uint32), o.view(np.uint32)), f"{name}: pooled {what} differs"
    qc_h, kc_h, vc_h = pooled

    log(f"[{name}] oracle: compressed attention + top-k for {len(wins)} windows ({time.time() - t0:.0f} s)")
    ooc, oidx, osc, amax = oracle.compressed(sh, qc_h, kc_h, vc_h, wins)
    assert_close(goc, ooc, sh.dtype, f"{name} O'_comp")
    gs = oracle.guide_scores(sh, qc_h, kc_h, wins, gidx)
    banded = check_topk(sh, gidx, oidx, osc, amax, gs)
    log(f"[{name}] top-k: {banded} of {gidx.shape[0] * gidx.shape[1]} (window, head) rows in the tie band")

    log(f"[{name}] oracle: selection + gate ({time.time() - t0:.0f} s)")
    # (1) the fused forward, on the rows where the GPU's set is the oracle's
    # (rows with another valid tie-band set have no unique expected output);
    # every other row must be in the tie band
    same = same_sets(gidx, oidx)
    assert (~same).sum() <= banded, f"{name}: {(~same).sum()} rows with other sets, {banded} in the band"
    osel = oracle.select(sh, c.q, c.k, c.v, wins, oidx)
    oimg = oracle.gate_combine(sh, c.q, c.wg, wins, ooc, osel)
    mx, mean, rel = assert_close_rows(o_img.reshape(oimg.shape), oimg, same, sh.dtype, f"{name} O_img (sampled)")
    log(f"[{name}] fused forward O_img: max-abs {mx:.2e} mean-abs {mean:.2e} rel-L2 {rel:.2e} on "
        f"{same.sum()} of {same.size} (window, head) rows ({(~same).sum()} rows with another tie-band set)")
    # (2) every sampled row: the selection and gate calls on the GPU, driven by
    # the oracle's own sets in the sampled windows' rows (the GPU's sets
    # elsewhere), against the oracle's selection + gate over the same sets
    idx_mix = idx_full.clone()
    idx_mix[torch.from_numpy(wins).cuda()] = torch.from_numpy(oidx.astype(np.int32)).cuda()
    osel_g = torch.empty((sh.m_img, sh.n_heads, sh.head_dim), dtype=torch.float32, device="cuda")
    ws_sel = workspace(c.cfg, gsa.GSA_OP_SELECT)
    gsa.gsa_select_attn(c.cfg, c.dq, c.dk, c.dv, idx_mix, osel_g, ws_sel)
    del ws_sel, idx_mix
    o_all = torch.zeros(sh.qkv_shape, dtype=c.dq.dtype, device="cuda")
    gsa.gsa_gate_combine(c.cfg, c.dq, c.dwg, None, oc_full, osel_g, o_all)
    torch.cuda.synchronize()
    o_img2 = to_host(o_all.view(sh.m_tokens, sh.n_heads, sh.head_dim).index_select(0, wtok))
    del osel_g, o_all
    mx, mean, rel = assert_close(o_img2.reshape(oimg.shape), oimg, sh.dtype, f"{name} O_img, oracle sets (sampled)")
    log(f"[{name}] O_img with the oracle's sets: max-abs {mx:.2e} mean-abs {mean:.2e} rel-L2 {rel:.2e} on all "
        f"{same.size} sampled (window, head) rows")

    log(f"[{name}] oracle: special attention for {len(rows)} rows ({time.time() - t0:.0f} s)")
    ospec = oracle.special(sh, c.q, c.k, c.v, rows)
    mx, mean, rel = assert_close(o_spec, ospec, sh.dtype, f"{name} O_spec (sampled)")
    log(f"[{name}] O_spec: max-abs {mx:.2e} mean-abs {mean:.2e} rel-L2 {rel:.2e}")

    log(f"[{name}] oracle: frame attention for {len(fr_rows)} rows ({time.time() - t0:.0f} s)")
    ofr = oracle.frame(sh, c.q, c.k, c.v, fr_rows)
    mx, mean, rel = assert_close(o_frame, ofr, sh.dtype, f"{name} frame attention (sampled)")
    log(f"[{name}] frame: max-abs {mx:.2e} mean-abs {mean:.2e} rel-L2 {rel:.2e}")

    log(f"[{name}] oracle: descriptor set and attention for {len(de_rows)} rows ({time.time() - t0:.0f} s)")
    o_set = [oracle.descriptor_set(sh, x) for x in (c.k, c.v)]
    for g, o, what in zip(g_set, o_set, "KV"):
        assert np.array_equal(g.view(np.uint32), o.view(np.uint32)), f"{name}: descriptor {what} set differs"
    ode = oracle.descriptor_attn(sh, c.q, o_set[0], o_set[1], de_rows)
    mx, mean, rel = assert_close(o_desc, ode, sh.dtype, f"{name} descriptor attention (sampled)")
    log(f"[{name}] descriptor: max-abs {mx:.2e} mean-abs {mean:.2e} rel-L2 {rel:.2e}; done in {time.time() - t0:.0f} s")


@pytest.mark.timeout(900)
def test_dense_comparator_full_size_rows():
    """The dense global-attention comparator that the bench times at the
    1000-frame workload (its ratio to GSA is reported): 64 sampled rows (the
    first and last token, special and image rows) x all heads against the
    oracle's dense attention over all 1.3 M tokens."""
    sh = PI3_LONG
    t0 = time.time()
    c = Case(sh)
    log(f"[dense] {sh.name}: gsa_dense_attn on the GPU ({time.time() - t0:.0f} s)")
    out = c.dense()
    torch.cuda.synchronize()
    rng = np.random.default_rng(sh.seed + 7)
    spec = special_token_ids(sh)
    rows = np.unique(np.concatenate([[0, sh.m_tokens - 1], rng.choice(spec, 8, replace=False),
                                     rng.choice(sh.m_tokens, 54, replace=False)]))
    got = to_host(out.view(sh.m_tokens, sh.n_heads, sh.head_dim).index_select(0, torch.from_numpy(rows).cuda()))
    del out
    log(f"[dense] oracle: {rows.size} rows over all tokens ({time.time() - t0:.0f} s)")
    ref = oracle.dense(sh, c.q, c.k, c.v, rows)
    mx, mean, rel = assert_close(got, ref, sh.dtype, "dense comparator (sampled)")
    log(f"[dense] {rows.size} rows: max-abs {mx:.2e} mean-abs {mean:.2e} rel-L2 {rel:.2e} ({time.time() - t0:.0f} s)")
