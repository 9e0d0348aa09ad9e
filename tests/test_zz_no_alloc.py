"""The allocation-free forward (gsa_forward_noalloc: workspace in a static
device array) against gsa_forward with a caller-allocated workspace, through
the C ABI: two calls in a row on one device, the second with a smaller input
than the first (so stale contents of the shared array from the first call
must not leak into the second), then the first shape again.  Both entry
points run the same kernels, so their outputs must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import gen
import sparse_global_attention_amd as gsa
from gen.configs import BF16, F32, GSAShape
from gsa_testlib import DEV, to_dev

pytestmark = pytest.mark.gpu

LARGER = GSAShape("32f-32x32-h16-s4-k16", 32, 5, 32, 32, 16, 64, 4, 16, BF16, seed=1001)
SMALLER = GSAShape("5f-16x12-h3-s4-k6+ctx{2}", 5, 2, 16, 12, 3, 64, 4, 6, BF16, ctx_frames=(2,), seed=61)
SMALL_F32 = GSAShape("3f-8x8-h2-s2-k5 fp32", 3, 1, 8, 8, 2, 64, 2, 5, F32, seed=62)


def run_both(sh):
    q, k, v, wg = gen.make_inputs(sh)
    dq, dk, dv, dwg = (to_dev(x, sh.dtype) for x in (q, k, v, wg))
    cfg = gsa.GSAConfig.from_shape(sh)
    need = gsa.gsa_workspace_size(cfg, gsa.GSA_OP_FORWARD)
    assert need <= gsa.GSA_NOALLOC_SCRATCH_BYTES
    ref = torch.full_like(dq, float("nan"))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    gsa.gsa_forward(cfg, dq, dk, dv, dwg, ref, ws)
    got = torch.full_like(dq, float("nan"))
    gsa.gsa_forward_noalloc(cfg, dq, dk, dv, dwg, got)
    torch.cuda.synchronize()
    print(f"no-alloc forward {sh.name}: workspace {need / 2**20:.1f} MiB", flush=True)
    a, b = ref.cpu(), got.cpu()
    assert torch.isfinite(b.float()).all()
    assert torch.equal(a.view(torch.int16) if sh.dtype == BF16 else a.view(torch.int32),
                       b.view(torch.int16) if sh.dtype == BF16 else b.view(torch.int32)), sh.name


def test_noalloc_matches_forward_twice_then_smaller():
    run_both(LARGER)
    run_both(SMALLER)
    run_both(SMALL_F32)
    run_both(LARGER)


def test_noalloc_rejects_oversized_config():
    sh = GSAShape("128f-36x36-h16-s4-k32", 128, 5, 36, 36, 16, 64, 4, 32, BF16)
    cfg = gsa.GSAConfig.from_shape(sh)
    assert gsa.gsa_workspace_size(cfg, gsa.GSA_OP_FORWARD) > gsa.GSA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    o = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gsa.GSAError) as e:
        gsa.gsa_forward_noalloc(cfg, x, x, x, x, o)
    assert e.value.status == gsa.GSA_ERR_WORKSPACE
