"""GSA-layer benchmark on one MI355X.

One step = one gsa_forward over the whole layer (pooling, special-token
attention, compressed attention with the guide-score top-k, selection attention
with the fused upsample + gate) on seeded synthetic inputs already resident in
HBM.
Default workload: the pi^3-style long sequence, 1000 frames x (36x36 image + 5
special tokens), 16 heads, d = 64, bf16, s = 4, k = 32.

Prints ONE JSON line.  Besides the throughput it reports, for the dominant
stage (the compressed attention + top-k call), a roofline object (algorithmic
work per launch / its average duration from HIP events on its stream), the
per-stage times, per-kernel fractions from the committed kernel trace, the
shader clock and run metadata, the dense global-attention comparator at the
same shape, and the CPU oracle timed on a bounded sample of the same workload
(a baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 matrix/vector peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "GSA-layer image tokens/s + % bf16 MFMA peak at 1000 frames x 1296 tok, 1 GPU"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="pi3-long", help="workload name (see gen/configs.py)")
    ap.add_argument("--topk", type=int, default=None, help="override the workload's k (test-time top-k)")
    ap.add_argument("--pool", type=int, default=None, help="override the workload's window size s")
    ap.add_argument("--special", type=int, default=None, help="override the special tokens per frame P")
    ap.add_argument("--grid", type=int, nargs=2, default=None, metavar=("H", "W"), help="override the image grid")
    ap.add_argument("--ctx", type=int, nargs="*", default=None, metavar="FRAME",
                    help="override the fixed context frames (none: --ctx with no frames)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparator")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the frame attention, descriptor attention and backward timings")
    ap.add_argument("--cpu-windows", type=int, default=128)
    ap.add_argument("--cpu-special", type=int, default=32)
    ap.add_argument("--forward-only", action="store_true",
                    help="time only the forward steps (no stage calls or extras; for kernel profiles)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates HBM byte counters) and exit")
    ap.add_argument("--gemm-probe", type=int, default=0, metavar="N",
                    help="only time a library bf16 GEMM (N x N x N, torch.matmul) with the shader clock "
                         "sampled, as a reference for what the matrix cores sustain, and exit")
    return ap.parse_args()


def copy_probe(mib: int):
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}))


_COMMON = ("gsa_device.h", "gsa_kernels.h")
KERNEL_SOURCES = {
    "flash_kernel<bf16,4,partial>": ("flash.hip", "flash_frag.h") + _COMMON,
    "flash_kernel<bf16,4,bound>": ("flash.hip", "flash_frag.h") + _COMMON,
    "flash_kernel<bf16,4,final>": ("flash.hip", "flash_frag.h") + _COMMON,
    "threshold_kernel<64>": ("topk.hip", "flash_frag.h") + _COMMON,
    "hot_group_kernel<bf16,8>": ("topk.hip", "flash_frag.h") + _COMMON,
    "rank_kernel": ("topk.hip", "flash_frag.h") + _COMMON,
    "refine_kernel<bf16,4,64>": ("topk.hip", "flash_frag.h") + _COMMON,
    "select_kernel<bf16,1>": ("select.hip", "select_frag.h", "flash_frag.h") + _COMMON,
    "pool_kernel<bf16>": ("pool.hip",) + _COMMON,
    "combine_kernel<bf16>": ("select.hip", "select_frag.h", "flash_frag.h") + _COMMON,
    "merge_kernel<bf16>": ("flash.hip", "flash_frag.h") + _COMMON,
    "flash_kernel<bf16,4,partial>,rloop": ("flash.hip", "flash_frag.h") + _COMMON,
    "descriptor_kernel": ("descriptor.hip",) + _COMMON,
}
# the backward's kernels (all in backward.hip)
KERNEL_SOURCES.update({k: ("backward.hip", "flash_frag.h", "select_frag.h") + _COMMON for k in (
    "flash_bwd_kernel<bf16,4,dq>", "flash_bwd_kernel<bf16,4,dkdv>", "sel_dq_kernel", "sel_dkdv_kernel",
    "gate_bwd_kernel", "dwg_slice_kernel", "dwg_total_kernel", "inv_zero_kernel", "inv_count_kernel",
    "scan_blocks_kernel", "scan_sums_kernel", "scan_add_kernel", "inv_fill_kernel", "inv_sort_kernel",
    "order_count_kernel", "order_fill_kernel", "reduce_kernel", "fill_kernel")})
# the kernels of gsa_compressed_attn_topk, in launch order
COMPRESSED_KERNELS = ("flash_kernel<bf16,4,bound>", "threshold_kernel<64>", "hot_group_kernel<bf16,8>",
                      "rank_kernel", "refine_kernel<bf16,4,64>")


def kernel_sources_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "sparse_global_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _profile_rows(path: str, ncells: int):
    """Rows of the markdown table in a committed profile summary whose last cell
    is the kernel's source hash and matches the current sources."""
    if not os.path.exists(path):
        return {}
    rows = {}
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == ncells and cells[0] in KERNEL_SOURCES and cells[-1] == kernel_sources_hash(cells[0]):
            rows[cells[0]] = cells
    return rows


def measured_traffic(kernels, workload: str):
    """HBM bytes per launch (fetched + written, summed over `kernels`) from the
    committed rocprofv3 counter summary profiles/hbm_traffic_<workload>.md, or
    None when a row is absent or was taken on other kernel sources."""
    rows = _profile_rows(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload.split()[0]}.md"), 7)
    if not all(k in rows for k in kernels):
        return None
    return round(sum((float(rows[k][4]) + float(rows[k][5])) * 1e9 for k in kernels))


def traced_ms(workload: str):
    """Average duration (ms) of each forward kernel in the committed kernel trace
    profiles/gsa_forward_<workload>_kernel_trace.md (rows with matching sources)."""
    rows = _profile_rows(os.path.join(ROOT, "profiles", f"gsa_forward_{workload.split()[0]}_kernel_trace.md"), 7)
    return {k: float(v[2]) for k, v in rows.items()}


def run_metadata():
    """ROCm version, device name and the host CPU model."""
    meta = {}
    try:
        meta["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        meta["rocm"] = None
    try:
        import torch
        meta["torch_hip"] = torch.version.hip
        meta["device"] = torch.cuda.get_device_properties(0).name
        meta["gcn_arch"] = getattr(torch.cuda.get_device_properties(0), "gcnArchName", None)
    except Exception:  # noqa: BLE001  (metadata only)
        pass
    meta["cpu_model"] = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                meta["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    meta["host_threads"] = os.cpu_count()
    return meta


class ClockSampler:
    """Samples the shader clock (MHz) from the amdgpu sysfs DPM table while the
    timed region runs (the level marked '*'); None where sysfs is not readable."""

    def __init__(self, period_s: float = 0.02):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        for line in open(path):
            if line.rstrip().endswith("*"):
                return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        return None

    def _run(self):
        while not self._stop.is_set():
            for p in self.paths:
                try:
                    v = self._read(p)
                except (OSError, ValueError, IndexError):
                    v = None
                if v:
                    self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.paths:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return {"source": "sysfs pp_dpm_sclk", "readable": bool(self.paths), "samples": 0}
        xs = sorted(self.samples)
        return {"source": "sysfs pp_dpm_sclk", "samples": len(xs), "mean_mhz": round(sum(xs) / len(xs), 1),
                "min_mhz": xs[0], "max_mhz": xs[-1]}


def gemm_probe(n: int, seconds: float = 1.5):
    """A library bf16 GEMM (random N(0,1) operands, fp32 accumulation) timed
    over ~`seconds` with the shader clock sampled: the rate the matrix cores
    sustain on dense work at this part's power limit, beside the published peak."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(7)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    c = a @ b
    e1.record()
    torch.cuda.synchronize()
    reps = max(3, int(seconds * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
    with ClockSampler() as cs:
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    print(json.dumps({"gemm_probe": {"n": n, "dtype": "bf16", "reps": reps, "ms_each": round(ms, 4),
                                     "tflops": round(tflops, 1), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                                     "shader_clock": cs.summary()}}))


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gemm_probe:
        gemm_probe(args.gemm_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import sparse_global_attention_amd as gsa
    from gen.configs import config_by_name

    sh = config_by_name(args.config)
    over = {k: v for k, v in (("topk", args.topk), ("pool", args.pool), ("n_special", args.special)) if v is not None}
    if args.grid:
        over.update(grid_h=args.grid[0], grid_w=args.grid[1])
    if args.ctx is not None:
        over.update(ctx_frames=tuple(args.ctx))
    if over:
        import dataclasses
        sh = dataclasses.replace(sh, **over)
        ctx = "+ctx{" + ",".join(map(str, sh.ctx_frames)) + "}" if sh.ctx_frames else ""
        sh = dataclasses.replace(sh, name=f"{sh.name.split()[0]}-variant {sh.n_frames}f-{sh.grid_h}x{sh.grid_w}-"
                                           f"h{sh.n_heads}-s{sh.pool}-k{sh.topk}-P{sh.n_special}{ctx}")
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    t0 = time.time()
    q, k, v, wg = gen.make_inputs(sh)
    t_gen = time.time() - t0

    def to_dev(x):
        if sh.dtype == gen.BF16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    dq, dk, dv, dwg = (to_dev(x) for x in (q, k, v, wg))
    cfg = gsa.GSAConfig.from_shape(sh)
    o = torch.empty_like(dq)
    ws = torch.empty(gsa.gsa_workspace_size(cfg, gsa.GSA_OP_FORWARD), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        gsa.gsa_forward(cfg, dq, dk, dv, dwg, o, ws, stream=stream)

    # ---- whole-layer throughput -------------------------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clock:
        t_wall = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
    ms_step = ev0.elapsed_time(ev1) / args.steps
    value = sh.m_img / (ms_step * 1e-3)
    fl = sh.flops()
    gsa_flops = fl["special"] + fl["compressed"] + fl["selection"]
    eff_tflops = gsa_flops / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if sh.dtype == gen.BF16 else PEAK_F32_TFLOPS

    if args.forward_only:
        print(json.dumps({"metric": METRIC, "value": round(value, 1), "unit": "image tokens/s", "n_gpus": 1,
                          "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
                          "mode": "forward-only (profiling)", "config": {"workload": sh.name},
                          "shader_clock": clock.summary()}))
        return

    # ---- per-stage launches (public entry points), HIP events on the same stream ----
    H, d = sh.n_heads, sh.head_dim
    shp = (sh.n_windows, H, d)
    qc, kc, vc = (torch.empty(shp, dtype=dq.dtype, device=dev) for _ in range(3))
    oc = torch.empty(shp, dtype=torch.float32, device=dev)
    idx = torch.empty((sh.n_windows, H, sh.topk), dtype=torch.int32, device=dev)
    osel = torch.empty((sh.m_img, H, d), dtype=torch.float32, device=dev)
    ws_spec = torch.empty(max(256, gsa.gsa_workspace_size(cfg, gsa.GSA_OP_SPECIAL)), dtype=torch.uint8, device=dev)
    ws_sel = torch.empty(max(256, gsa.gsa_workspace_size(cfg, gsa.GSA_OP_SELECT)), dtype=torch.uint8, device=dev)
    ws_cmp = torch.empty(max(256, gsa.gsa_workspace_size(cfg, gsa.GSA_OP_COMPRESSED)), dtype=torch.uint8, device=dev)
    o2 = torch.empty_like(dq)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(2, args.steps)
    st = {}
    st["pool"] = timed(lambda: gsa.gsa_pool(cfg, dq, dk, dv, qc, kc, vc, stream=stream), reps)
    st["compressed_topk"] = timed(lambda: gsa.gsa_compressed_attn_topk(cfg, qc, kc, vc, oc, idx, None, ws_cmp, stream=stream), reps)
    st["special"] = timed(lambda: gsa.gsa_special_attn(cfg, dq, dk, dv, o2, ws_spec, stream=stream), reps)
    st["select_standalone"] = timed(lambda: gsa.gsa_select_attn(cfg, dq, dk, dv, idx, osel, ws_sel, stream=stream), reps)
    st["gate_combine"] = timed(lambda: gsa.gsa_gate_combine(cfg, dq, dwg, None, oc, osel, o2, stream=stream), reps)

    # Roofline of the dominant stage, the compressed step (gsa_compressed_attn_topk:
    # the attention sweep with its score bounds, then the top-k kernels), timed by
    # HIP events on its stream, against its algorithmic work alone (4 M'^2 d H
    # FLOP of compressed attention; the top-k re-scoring is overhead, not work).
    esz = 2 if sh.dtype == gen.BF16 else 4
    achieved = fl["compressed"] / (st["compressed_topk"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(COMPRESSED_KERNELS, sh.name),
                "kernel": "+".join(COMPRESSED_KERNELS),
                "what": "compressed attention + guide-score top-k (gsa_compressed_attn_topk), the dominant stage",
                "work_per_launch_flop": fl["compressed"], "avg_launch_ms": round(st["compressed_topk"], 4)}

    # Algorithmic bytes of the memory-bound steps: bytes per unit (window, head,
    # channel or token) times the units one launch processes
    pool_bytes = 3 * sh.m_img * H * d * esz + 3 * sh.n_windows * H * d * esz
    gather_bytes = sh.n_windows * H * sh.topk_eff * sh.pool ** 2 * 2 * d * esz
    sb = (sh.pool ** 2 + 7) // 8 * 8
    idx_bytes = sh.n_windows * H * sh.topk * 4
    # standalone selection: q rows in, the gathers, the index lists, O_sel (fp32) out
    select_bytes = gather_bytes + sh.m_img * H * d * (esz + 4) + idx_bytes
    # its overhead: fp32 builds a blocked V^T copy first (V read, copy written);
    # bf16 gathers V rows from the token layout and builds none
    select_copy_bytes = 0 if esz == 2 else sh.m_img * H * d * esz + sh.n_windows * H * sb * d * esz
    # the forward's fused selection launch: q in, gathers, lists, O'_comp in, o out
    select_fused_bytes = gather_bytes + 2 * sh.m_img * H * d * esz + idx_bytes + sh.n_windows * H * d * 4
    combine_bytes = sh.m_img * H * d * (esz + 4 + esz) + sh.n_windows * H * d * 4

    # per-kernel fractions from the committed kernel trace of the forward (same sources only)
    tr = traced_ms(sh.name)
    kernel_work = {
        "flash_kernel<bf16,4,bound>": ("mfma", fl["compressed"], "compressed attention sweep (+ score bounds)"),
        "flash_kernel<bf16,4,partial>": ("mfma", fl["special"], "special-token attention partials"),
        "select_kernel<bf16,1>": ("hbm", select_fused_bytes, "selection attention + fused upsample/gate (forward)"),
        "pool_kernel<bf16>": ("hbm", pool_bytes, "pooling of Q, K and V"),
        "hot_group_kernel<bf16,8>": ("overhead", None, "top-k: re-scoring of the hot key groups"),
        "threshold_kernel<64>": ("overhead", None, "top-k: theta and hot-group masks"),
        "rank_kernel": ("overhead", None, "top-k: ranking of the candidate lists"),
    }
    kernels = []
    for kn, (bound, work, what) in kernel_work.items():
        if kn not in tr:
            continue
        ms = tr[kn]
        row = {"kernel": kn, "what": what, "trace_ms": ms}
        if bound == "mfma":
            row.update(bound="mfma", flop=work, tflops=round(work / (ms * 1e-3) / 1e12, 1),
                       frac=round(work / (ms * 1e-3) / 1e12 / peak, 4))
        elif bound == "hbm":
            row.update(bound="hbm", bytes=work, gbs=round(work / (ms * 1e-3) / 1e9, 1),
                       frac=round(work / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
        kernels.append(row)

    detail = {
        "stage_ms": {k_: round(v_, 4) for k_, v_ in st.items()},
        "effective_tflops": round(eff_tflops, 2),
        "frac_bf16_mfma_peak": round(eff_tflops / peak, 4),
        "gsa_flops": gsa_flops,
        "flops": fl,
        "special_step": {"kernels": ["flash_kernel<bf16,4,partial>", "merge_kernel<bf16>"],
                         "ms": round(st["special"], 4), "flop": fl["special"],
                         "tflops": round(fl["special"] / (st["special"] * 1e-3) / 1e12, 2),
                         "frac": round(fl["special"] / (st["special"] * 1e-3) / 1e12 / peak, 4),
                         "traffic": measured_traffic(("flash_kernel<bf16,4,partial>",), sh.name),
                         "kv_bytes": 2 * sh.m_tokens * H * d * esz},
        "kernels_from_trace": {"source": f"profiles/gsa_forward_{sh.name.split()[0]}_kernel_trace.md",
                               "rows": kernels},
        "pool_hbm_gbs": round(pool_bytes / (st["pool"] * 1e-3) / 1e9, 1),
        "pool_frac_hbm": round(pool_bytes / (st["pool"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "select_gather_bytes": gather_bytes,
        # the standalone selection call: algorithmic bytes (q rows in, gathers,
        # lists, O_sel out) over the entry point's time; the blocked V^T copy an
        # fp32 call builds first is overhead, reported beside (0 for bf16)
        "select_bytes": select_bytes,
        "select_copy_overhead_bytes": select_copy_bytes,
        "select_hbm_gbs": round(select_bytes / (st["select_standalone"] * 1e-3) / 1e9, 1),
        "select_frac_hbm": round(select_bytes / (st["select_standalone"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "combine_hbm_gbs": round(combine_bytes / (st["gate_combine"] * 1e-3) / 1e9, 1),
        "combine_frac_hbm": round(combine_bytes / (st["gate_combine"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "compressed_step": {"kernels": list(COMPRESSED_KERNELS),
                            "ms": round(st["compressed_topk"], 4),
                            "flop": fl["compressed"],
                            "tflops": round(fl["compressed"] / (st["compressed_topk"] * 1e-3) / 1e12, 2),
                            "frac": round(fl["compressed"] / (st["compressed_topk"] * 1e-3) / 1e12 / peak, 4)},
        "shader_clock": clock.summary(),
        "run": run_metadata(),
        "wall_s_timed_region": round(t_wall, 3),
        "input_gen_s": round(t_gen, 1),
    }
    if not args.no_extras:
        # Frame attention, the dense per-frame step that alternates with GSA in the
        # aggregation transformer: its time and one alternating pair (frame + GSA).
        t_frame = timed(lambda: gsa.gsa_frame_attn(cfg, dq, dk, dv, o2, stream=stream), reps)
        # one alternating pair as in the aggregation blocks: frame attention, then
        # GSA, back to back on one stream, timed as one region.  In a block the
        # two are separated by projections (weights the pages do not give), so
        # GSA takes inputs of the workload's statistics rather than the frame
        # output itself (whose small values would make a different top-k).
        o3 = torch.empty_like(dq)

        def pair():
            gsa.gsa_frame_attn(cfg, dq, dk, dv, o2, stream=stream)
            gsa.gsa_forward(cfg, dq, dk, dv, dwg, o3, ws, stream=stream)

        t_pair = timed(pair, reps)
        del o3
        detail["frame_attention"] = {
            "kernel": "flash_kernel<bf16,4,final>" if sh.dtype == gen.BF16 else "flash_kernel<f32,4,final>",
            "ms": round(t_frame, 4), "flop": fl["frame"],
            "tflops": round(fl["frame"] / (t_frame * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(fl["frame"] / (t_frame * 1e-3) / 1e12 / peak, 4),
            "alternating_pair_ms": round(t_pair, 4),
            "alternating_pair_note": "gsa_frame_attn then gsa_forward on one stream, one event-timed "
                                     "region per pair"}
        # FlashVGGT descriptor attention at the same shape (r = s, keyframes = the
        # context frames): building the key/value set, then every token over it.
        n_set = gsa.gsa_descriptor_count(cfg)
        kd, vd = (torch.empty((n_set, H, d), dtype=dq.dtype, device=dev) for _ in range(2))
        t_dset = timed(lambda: gsa.gsa_descriptor_set(cfg, dk, dv, kd, vd, stream=stream), reps)
        t_datt = timed(lambda: gsa.gsa_descriptor_attn(cfg, dq, kd, vd, o2, stream=stream), max(2, reps // 4))
        datt_flop = 4.0 * sh.m_tokens * n_set * d * H
        dset_bytes = (2 * sh.n_frames * (sh.grid_h // sh.pool) * (sh.grid_w // sh.pool) * 4
                      + 2 * (n_set - sh.n_frames * (sh.grid_h // sh.pool) * (sh.grid_w // sh.pool))
                      + 2 * n_set) * H * d * esz
        detail["descriptor_attention"] = {
            "kernels": ["descriptor_kernel", "flash_kernel<bf16,4,final>" if sh.dtype == gen.BF16 else
                        "flash_kernel<f32,4,final>"],
            "n_set": n_set, "set_ms": round(t_dset, 4), "set_hbm_gbs": round(dset_bytes / (t_dset * 1e-3) / 1e9, 1),
            "attn_ms": round(t_datt, 4), "attn_flop": datt_flop,
            "attn_tflops": round(datt_flop / (t_datt * 1e-3) / 1e12, 2),
            "attn_frac_mfma_peak": round(datt_flop / (t_datt * 1e-3) / 1e12 / peak, 4)}
        del kd, vd
        # Backward of the layer (gradients of q, k, v and W_g for a seeded dO, the
        # top-k sets of the compressed step above held fixed).  Algorithmic work:
        # 2.5x the forward attention FLOPs (recomputed scores, dP, dV, dQ, dK).
        d_o = to_dev(gen.make_output_grad(sh))
        gq, gk, gv = (torch.empty(sh.qkv_shape, dtype=torch.float32, device=dev) for _ in range(3))
        gw = torch.empty((H, d), dtype=torch.float32, device=dev)
        ws_bwd = torch.empty(max(256, gsa.gsa_workspace_size(cfg, gsa.GSA_OP_BACKWARD)), dtype=torch.uint8, device=dev)
        t_bwd = timed(lambda: gsa.gsa_backward(cfg, dq, dk, dv, dwg, idx, d_o, gq, gk, gv, gw, ws_bwd, stream=stream),
                      max(2, reps // 2))
        # the training pair: the forward saves its state, the backward reads it
        state = torch.empty(gsa.gsa_train_state_size(cfg), dtype=torch.uint8, device=dev)
        t_ftr = timed(lambda: gsa.gsa_forward_train(cfg, dq, dk, dv, dwg, o2, state, ws, stream=stream), reps)
        t_btr = timed(lambda: gsa.gsa_backward_train(cfg, dq, dk, dv, dwg, state, d_o, gq, gk, gv, gw, ws_bwd,
                                                     stream=stream), max(2, reps // 2))
        bwd_flop = 2.5 * gsa_flops
        detail["backward"] = {"ms": round(t_bwd, 4), "flop": bwd_flop,
                              "tflops": round(bwd_flop / (t_bwd * 1e-3) / 1e12, 2),
                              "frac_mfma_peak": round(bwd_flop / (t_bwd * 1e-3) / 1e12 / peak, 4),
                              "workspace_gb": round(ws_bwd.numel() / 1e9, 2),
                              "train_pair": {"forward_train_ms": round(t_ftr, 4), "backward_train_ms": round(t_btr, 4),
                                             "step_ms": round(t_ftr + t_btr, 4),
                                             "backward_tflops": round(bwd_flop / (t_btr * 1e-3) / 1e12, 2),
                                             "state_gb": round(state.numel() / 1e9, 2)}}
        del d_o, gq, gk, gv, gw, ws_bwd, state
    del ws_spec, ws_sel, ws_cmp, o2, osel

    # ---- dense comparator at the same shape --------------------------------------
    if not args.no_dense:
        od = torch.empty_like(dq)
        t_dense = timed(lambda: gsa.gsa_dense_attn(cfg, dq, dk, dv, od, stream=stream), 1)
        detail["dense_ms"] = round(t_dense, 2)
        detail["dense_tflops"] = round(fl["dense"] / (t_dense * 1e-3) / 1e12, 2)
        detail["speedup_vs_dense"] = round(t_dense / ms_step, 2)
        del od

    # ---- CPU oracle baseline on a bounded sample -----------------------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(sh, q, k, v, wg, args.cpu_windows, args.cpu_special)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "image tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == gen.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": sh.name, "frames": sh.n_frames, "special_per_frame": sh.n_special,
                   "grid": [sh.grid_h, sh.grid_w], "heads": H, "head_dim": d, "pool": sh.pool,
                   "topk": sh.topk, "ctx_frames": list(sh.ctx_frames), "image_tokens": sh.m_img,
                   "recipe": sh.recipe},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out))


def cpu_baseline(sh, q, k, v, wg, n_win, n_spec):
    """The oracle (as it stands) on a bounded sample of the workload, extrapolated to the layer.

    Full pooling of Q/K/V, then every step for n_win sampled query windows (all
    heads) and the special attention of n_spec sampled special rows (all heads).
    Layer estimate = pool + (M'/n_win) * window part + (M_spec/n_spec) * special part.
    """
    import numpy as np

    import gen
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    wins = gen.sample_windows(sh, n_win)
    rows = gen.sample_special(sh, n_spec)
    t0 = time.perf_counter()
    qc, kc, vc = oracle.pool(sh, q), oracle.pool(sh, k), oracle.pool(sh, v)
    t_pool = time.perf_counter() - t0
    t0 = time.perf_counter()
    oc, idx, _, _ = oracle.compressed(sh, qc, kc, vc, wins)
    osel = oracle.select(sh, q, k, v, wins, idx)
    oracle.gate_combine(sh, q, wg, wins, oc, osel)
    t_win = time.perf_counter() - t0
    t0 = time.perf_counter()
    if sh.m_spec:
        oracle.special(sh, q, k, v, rows)
    t_spec = time.perf_counter() - t0
    est = t_pool + t_win * sh.n_windows / len(wins) + (t_spec * sh.m_spec / len(rows) if sh.m_spec else 0.0)
    return {"value": round(sh.m_img / est, 3), "unit": "image tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"full pooling of Q/K/V ({t_pool:.1f} s) + all steps for {len(wins)} of {sh.n_windows} "
                       f"query windows x {sh.n_heads} heads ({t_win:.1f} s) + special attention for "
                       f"{len(rows)} of {sh.m_spec} special rows x {sh.n_heads} heads ({t_spec:.1f} s); "
                       f"linear extrapolation to the layer = {est:.0f} s"),
            "measured_s": round(t_pool + t_win + t_spec, 2)}


if __name__ == "__main__":
    main()
