"""Host-only checks of the C ABI: the library loads, exports every entry point
that include/gsa.h declares, and rejects bad arguments on the host without
touching a device (each case below fails validation before any launch)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    so = os.path.join(ROOT, "sparse_global_attention_amd", "libgsa.so")
    if not os.path.exists(so):
        from sparse_global_attention_amd import build as b  # noqa: F401  (import fails without the .so)
    import sparse_global_attention_amd as g
    return g


def header_functions():
    text = open(os.path.join(ROOT, "include", "gsa.h")).read()
    return sorted(set(re.findall(r"^(?:const char\*|gsa_status)\s+(gsa_\w+)\(", text, re.M)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for want in ("gsa_pool", "gsa_compressed_attn_topk", "gsa_select_attn", "gsa_special_attn",
                 "gsa_gate_combine", "gsa_forward", "gsa_dense_attn", "gsa_frame_attn", "gsa_workspace_size",
                 "gsa_descriptor_count", "gsa_descriptor_set", "gsa_descriptor_attn", "gsa_backward",
                 "gsa_train_state_size", "gsa_forward_train", "gsa_backward_train", "gsa_forward_noalloc",
                 "gsa_status_string"):
        assert want in fns


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, re.M))
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    assert set(lib.EXPORTS) == set(header_functions())


def test_status_strings(lib):
    assert lib.gsa_status_string(0) == "GSA_OK"
    for s in range(1, 6):
        assert lib.gsa_status_string(s).startswith("GSA_ERR_")
    assert "unknown" in lib.gsa_status_string(99)


def cfg(lib, **kw):
    base = dict(n_frames=4, n_special=1, grid_h=8, grid_w=8, n_heads=2, head_dim=64, pool=2, topk=4,
                dtype=lib.GSA_BF16)
    base.update(kw)
    return lib.GSAConfig.make(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(grid_h=9), 2), (dict(grid_w=6, pool=4), 2), (dict(n_frames=0), 2), (dict(n_heads=0), 2),
    (dict(head_dim=128), 3), (dict(pool=16, grid_h=16, grid_w=16), 3), (dict(topk=129), 3), (dict(dtype=7), 3),
    (dict(topk=0), 1), (dict(ctx_frames=(4,)), 1), (dict(ctx_frames=(1, 1)), 1), (dict(scale=-1.0), 1),
    (dict(scale=float("nan")), 1), (dict(ctx_exclude_from_topk=2), 1),
    # key positions are int32 inside the kernels: M = 64 N tokens must stay below 2^31 - 64
    (dict(n_frames=(2**31 - 64) // 64, n_special=0, n_heads=1), 2),
    (dict(n_frames=(2**31 - 64) // 64 - 1, n_special=0, n_heads=1), 0),
    # a window's s grid rows are read at 32-bit byte offsets: s w H d 4 < 2^31 - 4096
    (dict(n_frames=1, n_special=0, grid_h=8, grid_w=1 << 15, n_heads=32, pool=8), 2),
    (dict(n_frames=1, n_special=0, grid_h=8, grid_w=1 << 13, n_heads=32, pool=8), 0),
])
def test_config_validation(lib, kw, status):
    size = ctypes.c_size_t()
    assert lib.call_status("gsa_workspace_size", ctypes.byref(cfg(lib, **kw)), 0, ctypes.byref(size)) == status


def test_null_config_and_bad_op(lib):
    size = ctypes.c_size_t()
    assert lib.call_status("gsa_workspace_size", None, 0, ctypes.byref(size)) == 1
    assert lib.call_status("gsa_workspace_size", ctypes.byref(cfg(lib)), 9, ctypes.byref(size)) == 1
    assert lib.call_status("gsa_workspace_size", ctypes.byref(cfg(lib)), 0, None) == 1


def test_workspace_sizes(lib):
    c = cfg(lib, n_frames=32, n_special=5, grid_h=32, grid_w=32, n_heads=16, pool=4, topk=16)
    fw = lib.gsa_workspace_size(c, lib.GSA_OP_FORWARD)
    sel = lib.gsa_workspace_size(c, lib.GSA_OP_SELECT)
    spec = lib.gsa_workspace_size(c, lib.GSA_OP_SPECIAL)
    assert lib.gsa_workspace_size(c, lib.GSA_OP_DENSE) == 0
    mw, H, d = 32 * 64, 16, 64
    pooled = mw * H * d * 2
    assert sel == 0  # bf16 gathers K and V rows from the token layout
    assert fw >= 3 * pooled + mw * H * d * 4 + mw * H * 16 * 4 + spec
    assert spec > 0
    # fp32 gathers V from a blocked, transposed copy: 16 slots per window
    c32 = cfg(lib, n_frames=32, n_special=5, grid_h=32, grid_w=32, n_heads=16, pool=4, topk=16, dtype=lib.GSA_F32)
    assert lib.gsa_workspace_size(c32, lib.GSA_OP_SELECT) == mw * H * 16 * d * 4
    ctx = cfg(lib, n_frames=8, ctx_frames=(0, 5))
    assert lib.gsa_workspace_size(ctx, lib.GSA_OP_SELECT) > lib.gsa_workspace_size(cfg(lib, n_frames=8),
                                                                                    lib.GSA_OP_SELECT)


# Addresses that are never dereferenced: every call below fails validation first.
A = 0x10000
MISALIGNED = 0x10004


def test_pointer_validation(lib):
    c = ctypes.byref(cfg(lib))
    assert lib.call_status("gsa_pool", c, None, A, A, A, A, A, None) == 1
    assert lib.call_status("gsa_pool", c, MISALIGNED, A, A, A, A, A, None) == 1
    assert lib.call_status("gsa_compressed_attn_topk", c, A, A, A, A, None, None, A, 1 << 30, None) == 1
    assert lib.call_status("gsa_compressed_attn_topk", c, A, A, A, A, A, MISALIGNED, A, 1 << 30, None) == 1
    assert lib.call_status("gsa_gate_combine", c, A, None, None, A, A, A + 64, None) == 1  # no wg and no gate
    assert lib.call_status("gsa_forward", c, A, A, A, A, A, A, 1 << 30, None) == 1  # o aliases q
    assert lib.call_status("gsa_special_attn", c, A, A, A, A, A, 1 << 30, None) == 1  # o aliases q
    assert lib.call_status("gsa_dense_attn", c, A, A + 16, A + 32, A, None, 0, None) == 1  # o aliases q
    assert lib.call_status("gsa_frame_attn", c, A, A + 16, A + 32, A + 32, None) == 1  # o aliases v
    assert lib.call_status("gsa_frame_attn", c, A, None, A + 32, A + 48, None) == 1
    assert lib.call_status("gsa_frame_attn", c, A, A + 16, MISALIGNED, A + 48, None) == 1
    assert lib.call_status("gsa_descriptor_set", c, A, A + 16, A + 16, A + 48, None) == 1  # kd aliases v
    assert lib.call_status("gsa_descriptor_set", c, A, A + 16, A + 32, A + 32, None) == 1  # kd aliases vd
    assert lib.call_status("gsa_descriptor_set", c, A, A + 16, None, A + 48, None) == 1
    assert lib.call_status("gsa_descriptor_attn", c, A, A + 16, A + 32, A + 16, None) == 1  # o aliases kd
    assert lib.call_status("gsa_descriptor_attn", c, MISALIGNED, A + 16, A + 32, A + 48, None) == 1
    assert lib.call_status("gsa_descriptor_count", c, None) == 1
    # gsa_backward(cfg, q, k, v, wg, idx, d_o, dq, dk, dv, dwg, ws, ws_bytes, stream)
    bw = [A, A + 16, A + 32, A + 48, A + 64, A + 80, A + 96, A + 112, A + 128, A + 144]
    # rejected on the host before any launch: an output aliasing an input or
    # another output, a null or misaligned pointer
    for i, bad in ((6, A), (7, A + 96), (9, A + 128), (3, None), (8, MISALIGNED)):
        args = list(bw)
        args[i] = bad
        assert lib.call_status("gsa_backward", c, *args, A + 256, 1 << 40, None) == 1, (i, bad)


def test_workspace_validation(lib):
    cc = cfg(lib)
    c = ctypes.byref(cc)
    need = lib.gsa_workspace_size(cc, lib.GSA_OP_FORWARD)
    o = A + (1 << 20)
    assert lib.call_status("gsa_forward", c, A, A, A, A, o, A, need - 1, None) == 4
    assert lib.call_status("gsa_forward", c, A, A, A, A, o, None, need, None) == 1
    assert lib.call_status("gsa_forward", c, A, A, A, A, o, A + 16, need, None) == 1  # ws not 256-aligned
    # (bf16 selection needs no workspace without context frames; fp32 does)
    c32 = cfg(lib, dtype=lib.GSA_F32)
    need = lib.gsa_workspace_size(c32, lib.GSA_OP_SELECT)
    assert need > 0
    assert lib.call_status("gsa_select_attn", ctypes.byref(c32), A, A, A, A, o, A, need - 256, None) == 4
    need = lib.gsa_workspace_size(cc, lib.GSA_OP_SPECIAL)
    assert lib.call_status("gsa_special_attn", c, A, A, A, o, A, need - 1, None) == 4
    need = lib.gsa_workspace_size(cc, lib.GSA_OP_COMPRESSED)
    assert need > 0
    assert lib.call_status("gsa_compressed_attn_topk", c, A, A, A, o, o + 4096, None, A, need - 1, None) == 4
    need = lib.gsa_workspace_size(cc, lib.GSA_OP_BACKWARD)
    bw = [A + 16 * i for i in range(6)] + [o, o + 4096, o + 8192, o + 12288]
    assert lib.call_status("gsa_backward", c, *bw, A, need - 1, None) == 4
    assert lib.call_status("gsa_backward", c, *bw, None, need, None) == 1
    # the training pair: a null, misaligned, aliased or undersized state is
    # rejected before any launch
    need_f = lib.gsa_workspace_size(cc, lib.GSA_OP_FORWARD)
    sb = lib.gsa_train_state_size(cc)
    st = A + (1 << 24)
    assert lib.call_status("gsa_forward_train", c, A, A, A, A, o, None, sb, A, need_f, None) == 1
    assert lib.call_status("gsa_forward_train", c, A, A, A, A, o, st + 16, sb, A, need_f, None) == 1
    assert lib.call_status("gsa_forward_train", c, A, A, A, A, o, o, sb, A, need_f, None) == 1
    assert lib.call_status("gsa_forward_train", c, A, A, A, A, o, st, sb, A, need_f - 1, None) == 4
    assert lib.call_status("gsa_forward_train", c, A, A, A, A, o, st, sb - 1, A, need_f, None) == 4
    assert lib.call_status("gsa_forward_train", c, A, A, A, A, o, st, 0, A, need_f, None) == 4
    tr = [A, A + 16, A + 32, A + 48, st, sb, A + 64, o, o + 4096, o + 8192, o + 12288]
    assert lib.call_status("gsa_backward_train", c, *tr, A, need - 1, None) == 4
    tr[5] = sb - 1
    assert lib.call_status("gsa_backward_train", c, *tr, A, need, None) == 4
    tr[5] = sb
    tr[4] = None
    assert lib.call_status("gsa_backward_train", c, *tr, A, need, None) == 1
    tr[4] = o  # the state aliasing dq
    assert lib.call_status("gsa_backward_train", c, *tr, A, need, None) == 1
    n = ctypes.c_size_t(0)
    assert lib.call_status("gsa_train_state_size", c, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.call_status("gsa_compressed_attn_topk", c, A, A, A, o, o + 4096, None, None, need, None) == 1


def test_noalloc_forward_validation(lib):
    """The allocation-free forward rejects, on the host, configs whose forward
    workspace exceeds its static scratch, and bad pointers, before any launch."""
    small = cfg(lib)
    assert lib.gsa_workspace_size(small, lib.GSA_OP_FORWARD) <= lib.GSA_NOALLOC_SCRATCH_BYTES
    mid = cfg(lib, n_frames=32, n_special=5, grid_h=32, grid_w=32, n_heads=16, pool=4, topk=16)
    assert lib.gsa_workspace_size(mid, lib.GSA_OP_FORWARD) <= lib.GSA_NOALLOC_SCRATCH_BYTES
    big = cfg(lib, n_frames=128, n_special=5, grid_h=36, grid_w=36, n_heads=16, pool=4, topk=32)
    assert lib.gsa_workspace_size(big, lib.GSA_OP_FORWARD) > lib.GSA_NOALLOC_SCRATCH_BYTES
    o = A + (1 << 20)
    assert lib.call_status("gsa_forward_noalloc", ctypes.byref(big), A, A, A, A, o, None) == 4
    c = ctypes.byref(small)
    assert lib.call_status("gsa_forward_noalloc", c, None, A, A, A, o, None) == 1
    assert lib.call_status("gsa_forward_noalloc", c, A, A, A, A + 8, o, None) == 1  # wg misaligned
    assert lib.call_status("gsa_forward_noalloc", c, A, A, A, A, A, None) == 1  # o aliases q
    assert lib.call_status("gsa_forward_noalloc", ctypes.byref(cfg(lib, grid_h=7)), A, A, A, A, o, None) == 2


def test_window_count_limit(lib):
    """Per-head rows of window bounds are addressed with 32-bit byte offsets,
    so M' must stay below 2^29 windows: the boundary is rejected on the host."""
    at = cfg(lib, n_frames=1, n_special=0, grid_h=1 << 14, grid_w=1 << 15, n_heads=1, pool=1, topk=4)
    assert lib.call_status("gsa_workspace_size", ctypes.byref(at), lib.GSA_OP_FORWARD,
                           ctypes.byref(ctypes.c_size_t(0))) == lib.GSA_ERR_SHAPE
    below = cfg(lib, n_frames=1, n_special=0, grid_h=(1 << 14) - 1, grid_w=1 << 15, n_heads=1, pool=1, topk=4)
    assert lib.gsa_workspace_size(below, lib.GSA_OP_COMPRESSED) > 0


def test_binding_raises_gsa_error(lib):
    with pytest.raises(lib.GSAError) as e:
        lib.gsa_workspace_size(cfg(lib, grid_h=7), lib.GSA_OP_FORWARD)
    assert e.value.status == lib.GSA_ERR_SHAPE


def test_descriptor_count_matches_the_set_layout(lib):
    """N (h/r)(w/r) descriptors + frame 0 and the keyframes whole + the other frames' specials."""
    n = ctypes.c_int64(0)
    c = lib.GSAConfig.make(10, 5, 36, 36, 16, 64, 4, 32)
    assert lib.call_status("gsa_descriptor_count", ctypes.byref(c), ctypes.byref(n)) == 0
    assert n.value == 10 * 81 + 1301 + 9 * 5
    c = lib.GSAConfig.make(10, 5, 36, 36, 16, 64, 4, 32, ctx_frames=(0, 7, 3))
    assert lib.call_status("gsa_descriptor_count", ctypes.byref(c), ctypes.byref(n)) == 0
    assert n.value == 10 * 81 + 3 * 1301 + 7 * 5
    c = lib.GSAConfig.make(4, 0, 8, 12, 2, 64, 2, 3)
    assert lib.call_status("gsa_descriptor_count", ctypes.byref(c), ctypes.byref(n)) == 0
    assert n.value == 4 * 4 * 6 + 96
