// C ABI of libgsa: argument validation, workspace layout and launch sequences.
// The operations are those of the Paper-Notes page "Speed3R: Sparse
// Feed-forward 3D Reconstruction Models" (sections "全局稀疏注意力（GSA）核心设计",
// "压缩分支", "选择分支", "门控聚合", "Speed3R-VGGT 适配"); see gsa.h for each
// entry point's contract.
#include <algorithm>
#include <math.h>
#include <mutex>
#include <string.h>

#include "gsa.h"
#include "gsa_device.h"
#include "gsa_kernels.h"

using namespace gsa;

namespace {

constexpr int64_t kAlign = 256;
// Workgroups of the attention kernels resident at once on a gfx950 part:
// 256 compute units, four 256-thread workgroups each.
constexpr int64_t kWorkgroupSlots = 256 * 4;

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Call {
  Geometry g;
  int dtype;
  int64_t esz;  // bytes per element of q/k/v/o
  float scale;
  int topk;
  int n_ctx;
  int ctx[GSA_MAX_CTX_FRAMES];
  int exclude;
};

gsa_status check_cfg(const gsa_config* c, Call* out) {
  if (!c) return GSA_ERR_INVALID_ARG;
  if (c->dtype != GSA_BF16 && c->dtype != GSA_F32) return GSA_ERR_UNSUPPORTED;
  if (c->n_frames < 1 || c->n_special < 0 || c->grid_h < 1 || c->grid_w < 1 || c->n_heads < 1 || c->pool < 1)
    return GSA_ERR_SHAPE;
  if (c->head_dim != kHeadDim) return GSA_ERR_UNSUPPORTED;
  if (c->pool > 8) return GSA_ERR_UNSUPPORTED;
  if (c->grid_h % c->pool != 0 || c->grid_w % c->pool != 0) return GSA_ERR_SHAPE;
  if (c->topk < 1) return GSA_ERR_INVALID_ARG;
  if (c->topk > 128) return GSA_ERR_UNSUPPORTED;
  if (c->n_ctx_frames < 0 || c->n_ctx_frames > GSA_MAX_CTX_FRAMES) return GSA_ERR_INVALID_ARG;
  for (int i = 0; i < c->n_ctx_frames; ++i) {
    if (c->ctx_frames[i] < 0 || c->ctx_frames[i] >= c->n_frames) return GSA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (c->ctx_frames[j] == c->ctx_frames[i]) return GSA_ERR_INVALID_ARG;
  }
  if (c->ctx_exclude_from_topk != 0 && c->ctx_exclude_from_topk != 1) return GSA_ERR_INVALID_ARG;
  if (!(c->scale >= 0.0f) || isinf(c->scale)) return GSA_ERR_INVALID_ARG;

  Geometry& g = out->g;
  g.n_frames = c->n_frames;
  g.n_special = c->n_special;
  g.grid_h = c->grid_h;
  g.grid_w = c->grid_w;
  g.n_heads = c->n_heads;
  g.pool = c->pool;
  g.tf = (int64_t)c->n_special + (int64_t)c->grid_h * c->grid_w;
  g.m_tokens = g.n_frames * g.tf;
  g.m_spec = g.n_frames * g.n_special;
  g.m_img = g.n_frames * g.grid_h * g.grid_w;
  g.wx = g.grid_w / g.pool;
  g.wpf = (g.grid_h / g.pool) * g.wx;
  g.n_windows = g.n_frames * g.wpf;
  g.sb = (g.pool * g.pool + 7) / 8 * 8;
  // window ids are int32 in topk_idx, key positions inside a kernel's key range
  // are int32, and every element count stays well inside int64
  // (per-head rows of window bounds are addressed with 32-bit byte offsets:
  // M' * 4 < 2^31; the selection reads a window's rows at 32-bit byte offsets
  // from its first row: s grid rows of tokens stay below 2^31 bytes)
  if (g.n_windows >= ((int64_t)1 << 29) || g.m_tokens > INT32_MAX - 64 ||
      g.m_tokens > ((int64_t)1 << 40) / (g.n_heads * kHeadDim) ||
      g.pool * g.grid_w * g.n_heads * kHeadDim * 4 >= (int64_t)INT32_MAX - 4096)
    return GSA_ERR_SHAPE;

  out->dtype = c->dtype;
  out->esz = c->dtype == GSA_BF16 ? 2 : 4;
  out->scale = c->scale > 0.0f ? c->scale : 1.0f / sqrtf((float)kHeadDim);
  out->topk = c->topk;
  out->n_ctx = c->n_ctx_frames;
  for (int i = 0; i < c->n_ctx_frames; ++i) out->ctx[i] = c->ctx_frames[i];
  out->exclude = c->ctx_exclude_from_topk;
  return GSA_OK;
}

bool ptr_ok(const void* p) { return p != nullptr && ((uintptr_t)p & 15) == 0; }

// FlashVGGT key/value set: r = the pool field, keyframes = the context frames.
DescParams descriptor_plan(const Call& c) {
  DescParams d;
  memset(&d, 0, sizeof(d));
  const Geometry& g = c.g;
  d.g = g;
  d.r = (int)g.pool;
  d.n_desc = g.n_frames * (g.grid_h / g.pool) * (g.grid_w / g.pool);
  d.full[d.n_full++] = 0;
  for (int i = 0; i < c.n_ctx; ++i)
    if (c.ctx[i] != 0) d.full[d.n_full++] = c.ctx[i];
  for (int i = 0; i < d.n_full; ++i) d.full_sorted[i] = d.full[i];
  for (int i = 1; i < d.n_full; ++i)
    for (int j = i; j > 0 && d.full_sorted[j - 1] > d.full_sorted[j]; --j) {
      const int t = d.full_sorted[j];
      d.full_sorted[j] = d.full_sorted[j - 1];
      d.full_sorted[j - 1] = t;
    }
  d.n_set = d.n_desc + d.n_full * g.tf + (g.n_frames - d.n_full) * g.n_special;
  return d;
}

// ---- workspace layout ----------------------------------------------------------
struct Plan {
  int n_split;  // special-attention key splits
  int64_t qc, kc, vc, oc, topk, kblk, vblk, spec_o, spec_lse, ctx_o, ctx_lse, total;
  int n_groups, group_tiles;  // compressed step: key-tile groups of the score bounds
  int n_words, cap, n_chunks;  // top-k: hot-mask words, list entries per query, query chunks
  int64_t gbound, gerr, theta, hot, cnt, cand;
  // backward
  int ctx_qsplits;  // query splits of the context frames' key-side pass
  int64_t qblk, qT, kT, vrow, lse_c, spec_o32, spec_l2, spec_dd, osel, l2sel, doblk, doT, l2blk, dblk,
      dzblk, dosel_img, dsel_img, doc, dc, l2c, dwg_part, dwg_slices, dqc, dkc, dvc;
  int64_t inv_off, inv_bsum, inv_raw, inv_list, inv_order, inv_ccnt, inv_cbsum, ctx_dq, ctx_dkdv;
};

// Training state saved by gsa_forward_train for gsa_backward_train.
struct TrainState {
  int64_t topk, oc, lse_c, spec_o32, spec_l2, osel, l2sel, total;
};
TrainState state_plan(const Call& c) {
  const Geometry& g = c.g;
  TrainState t;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    int64_t at = off;
    off += align_up(bytes);
    return at;
  };
  t.topk = take(g.n_windows * g.n_heads * (int64_t)c.topk * 4);
  t.oc = take(g.n_windows * g.n_heads * kHeadDim * 4);
  t.lse_c = take(g.n_windows * g.n_heads * 4);
  t.spec_o32 = take(g.m_spec * g.n_heads * kHeadDim * 4);
  t.spec_l2 = take(g.m_spec * g.n_heads * 4);
  t.osel = take(g.m_img * g.n_heads * kHeadDim * 4);
  t.l2sel = take(g.m_img * g.n_heads * 4);
  t.total = off;
  return t;
}

// Query splits of the key-side backward pass over one context frame: enough
// workgroups to fill the resident slots, at most one per query tile.
int ctx_query_splits(const Call& c) {
  const Geometry& g = c.g;
  const int64_t per = ((g.tf + 127) / 128) * g.n_heads;
  int64_t z = (kWorkgroupSlots * 2 + per - 1) / per;
  const int64_t n_qt = (g.m_img + 31) / 32;
  if (z > n_qt) z = n_qt;
  if (z < 1) z = 1;
  return (int)z;
}

// Groups of key tiles for the score bounds: at most topk_groups_for_k(k)
// groups, so that the k-th best group bound sits close to the k-th best score
// and about k groups per query are hot.
void bound_groups(const Call& c, int* n_groups, int* group_tiles) {
  const int64_t tiles = (c.g.n_windows + 31) / 32;
  const int64_t target = topk_groups_for_k(c.topk);
  int64_t gt = (tiles + target - 1) / target;
  if (gt < 1) gt = 1;
  *group_tiles = (int)gt;
  *n_groups = (int)((tiles + gt - 1) / gt);
}
// Query chunks of the hot-group pass: a chunk's query rows (128 bytes each in
// bf16) stay within about 2 MB, so the workgroups of one (head, chunk) that
// run together on an XCD share them through its L2, and the grid holds at
// least 4096 workgroups.
int hot_chunks(const Call& c, int n_groups) {
  int64_t nc = (c.g.n_windows + 16383) / 16384;
  const int64_t fill = (4096 + c.g.n_heads * n_groups - 1) / (c.g.n_heads * n_groups);
  if (nc < fill) nc = fill;
  if (nc > c.g.n_windows) nc = c.g.n_windows;
  return (int)(nc < 1 ? 1 : nc);
}

// Key splits of the special-token attention.  Every workgroup of a split
// sweeps 1/n of the keys, so with W = per_split * n workgroups running
// kWorkgroupSlots at a time the sweep takes about ceil(W / slots) / n of the
// unsplit time: n is chosen to minimise that (the smallest such n), i.e. to
// fill the last round of workgroups, with at least 4 key tiles per split.
int special_splits(const Call& c) {
  const Geometry& g = c.g;
  if (g.m_spec == 0) return 1;
  const int64_t per_split = g.n_heads * ((g.m_spec + 127) / 128);
  int64_t max_n = (g.m_tokens + 4 * 32 - 1) / (4 * 32);
  if (max_n > kMaxRanges) max_n = kMaxRanges;
  int best = 1;
  double best_t = 0.0;
  for (int64_t n = 1; n <= max_n; ++n) {
    const double t = (double)((per_split * n + kWorkgroupSlots - 1) / kWorkgroupSlots) / (double)n;
    if (n == 1 || t < best_t * (1.0 - 1e-9)) {
      best = (int)n;
      best_t = t;
    }
  }
  return best;
}
// Context frames' partials: one sweep per query block over every context
// frame (one partial) when the query blocks alone fill the chip several
// times over, else one split and one partial per frame.
bool ctx_range_loop(const Call& c) {
  const int64_t n_qt = (c.g.m_img + 127) / 128;
  return c.n_ctx > 1 && n_qt * c.g.n_heads >= 4096;
}
int ctx_parts(const Call& c) { return c.n_ctx == 0 ? 0 : ctx_range_loop(c) ? 1 : c.n_ctx; }


Plan make_plan(const Call& c, gsa_op op) {
  const Geometry& g = c.g;
  Plan p;
  memset(&p, 0, sizeof(p));
  p.n_split = special_splits(c);
  bound_groups(c, &p.n_groups, &p.group_tiles);
  p.n_words = (p.n_groups + 31) / 32;
  p.cap = topk_list_cap(c.topk);
  p.n_chunks = hot_chunks(c, p.n_groups);
  const int64_t pooled = g.n_windows * g.n_heads * kHeadDim * c.esz;
  const int64_t blk = g.n_windows * g.n_heads * g.sb * kHeadDim * c.esz;
  const int64_t spec_o = (int64_t)p.n_split * g.m_spec * g.n_heads * kHeadDim * 4;
  const int64_t spec_lse = (int64_t)p.n_split * g.m_spec * g.n_heads * 4;
  const int64_t ctx_o = (int64_t)ctx_parts(c) * g.m_img * g.n_heads * kHeadDim * 4;
  const int64_t ctx_lse = (int64_t)ctx_parts(c) * g.m_img * g.n_heads * 4;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    int64_t at = off;
    off += align_up(bytes);
    return at;
  };
  if (op == GSA_OP_FORWARD) {
    p.qc = take(pooled);
    p.kc = take(pooled);
    p.vc = take(pooled);
    p.oc = take(g.n_windows * g.n_heads * kHeadDim * 4);
    p.topk = take(g.n_windows * g.n_heads * (int64_t)c.topk * 4);
  }
  if (op == GSA_OP_FORWARD || op == GSA_OP_COMPRESSED) {
    const int64_t qh = g.n_heads * g.n_windows;
    p.gbound = take((int64_t)p.n_groups * qh * 4);
    p.gerr = take(qh * 4);
    p.theta = take(qh * 4);
    p.hot = take((int64_t)p.n_words * qh * 4);
    p.cnt = take(qh * 4);
    p.cand = take(qh * p.cap * 8);
  }
  // transposed V blocks for the selection gathers: fp32 only (bf16 gathers
  // V rows and transposes them in LDS)
  const int64_t vt_blk = c.dtype == GSA_BF16 ? 0 : blk;
  if (op == GSA_OP_FORWARD || op == GSA_OP_SELECT) {
    p.vblk = take(vt_blk);
    p.ctx_o = take(ctx_o);
    p.ctx_lse = take(ctx_lse);
  }
  if (op == GSA_OP_FORWARD || op == GSA_OP_SPECIAL) {
    p.spec_o = take(spec_o);
    p.spec_lse = take(spec_lse);
  }
  if (op == GSA_OP_BACKWARD) {
    const int64_t wf = g.n_windows * g.n_heads * kHeadDim * 4;  // float [M'][H][d]
    const int64_t wl = g.n_windows * g.n_heads * 4;             // float [M'][H]
    const int64_t bl = g.n_windows * g.n_heads * g.sb * 4;      // float [M'][H][sb]
    const int64_t imgf = g.m_img * g.n_heads * kHeadDim * 4;
    const int64_t segs = g.n_windows * g.n_heads;
    const int64_t entries = segs * c.topk;
    p.ctx_qsplits = ctx_query_splits(c);
    p.qc = take(pooled);
    p.kc = take(pooled);
    p.vc = take(pooled);
    const int64_t tblk = c.dtype == GSA_BF16 ? 0 : blk;  // transposed copies: fp32 only
    p.qblk = take(blk);
    p.qT = take(tblk);
    p.kblk = take(blk);
    p.kT = take(tblk);
    p.vrow = take(blk);
    p.vblk = take(vt_blk);
    p.oc = take(wf);
    p.lse_c = take(wl);
    p.spec_o = take(spec_o);
    p.spec_lse = take(spec_lse);
    p.spec_o32 = take(g.m_spec * g.n_heads * kHeadDim * 4);
    p.spec_l2 = take(g.m_spec * g.n_heads * 4);
    p.spec_dd = take(g.m_spec * g.n_heads * 4);
    p.ctx_o = take(ctx_o);
    p.ctx_lse = take(ctx_lse);
    p.osel = take(imgf);
    p.l2sel = take(g.m_img * g.n_heads * 4);
    p.doblk = take(blk);
    p.doT = take(tblk);
    p.l2blk = take(bl);
    p.dblk = take(bl);
    p.dzblk = take(bl);
    if (c.n_ctx) {
      p.dosel_img = take(g.m_img * g.n_heads * kHeadDim * c.esz);
      p.dsel_img = take(g.m_img * g.n_heads * 4);
      p.ctx_dq = take(c.n_ctx > 1 ? c.n_ctx * imgf : 0);
      p.ctx_dkdv = take(p.ctx_qsplits > 1 ? 2 * (int64_t)p.ctx_qsplits * g.tf * g.n_heads * kHeadDim * 4 : 0);
    }
    p.doc = take(g.n_windows * g.n_heads * kHeadDim * c.esz);
    p.dc = take(wl);
    p.l2c = take(wl);
    p.dwg_part = take(wf);
    p.dwg_slices = take((int64_t)kDwgSlices * g.n_heads * kHeadDim * 4);
    p.dqc = take(wf);
    p.dkc = take(wf);
    p.dvc = take(wf);
    p.inv_off = take((segs + 1) * 4);
    p.inv_bsum = take(((segs + 1 + 1023) / 1024) * 4);
    p.inv_raw = take(entries * 4);
    p.inv_list = take(entries * 4);
    const int64_t oblk = (segs + 1023) / 1024;
    p.inv_order = take(segs * 4);
    p.inv_ccnt = take(8 * oblk * 4);
    p.inv_cbsum = take(((8 * oblk + 1023) / 1024) * 4);
  }
  p.total = off;
  return p;
}

gsa_status check_ws(const Plan& pl, void* ws, size_t ws_bytes) {
  if (pl.total == 0) return GSA_OK;
  if (ws == nullptr || ((uintptr_t)ws & (kAlign - 1)) != 0) return GSA_ERR_INVALID_ARG;
  if ((int64_t)ws_bytes < pl.total) return GSA_ERR_WORKSPACE;
  return GSA_OK;
}

char* at(void* ws, int64_t off) { return static_cast<char*>(ws) + off; }

gsa_status hip_status(hipError_t e) { return e == hipSuccess ? GSA_OK : GSA_ERR_HIP; }

// ---- launch sequences --------------------------------------------------------------
FlashParams flash_base(const Call& c, const void* q, const void* k, const void* v) {
  FlashParams f;
  memset(&f, 0, sizeof(f));
  f.q = q;
  f.k = k;
  f.v = v;
  f.row_stride = c.g.n_heads * kHeadDim;
  f.n_heads = (int)c.g.n_heads;
  f.scale_log2 = c.scale * kLog2e;
  f.n_batch = 1;
  return f;
}

void set_rows_identity(FlashParams& f, int64_t n) {
  f.n_q = n;
  f.qa = n > 0 ? n : 1;
  f.qb = 0;
  f.qc = 0;
}

hipError_t run_special(const Call& c, const Plan& pl, const void* q, const void* k, const void* v, void* o,
                       void* ws, hipStream_t st, float* o32 = nullptr, float* l2 = nullptr) {
  const Geometry& g = c.g;
  if (g.m_spec == 0) return hipSuccess;
  FlashParams f = flash_base(c, q, k, v);
  f.n_q = g.m_spec;
  f.qa = g.n_special;
  f.qb = g.tf;
  f.qc = 0;
  // even split of the M keys into n_split ranges (multiples of 32 keys)
  const int ns = pl.n_split;
  const int64_t tiles = (g.m_tokens + 31) / 32;
  f.n_splits = ns;
  for (int s = 0; s < ns; ++s) {
    f.kbeg[s] = tiles * s / ns * 32;
    f.kend[s] = s + 1 == ns ? g.m_tokens : tiles * (s + 1) / ns * 32;
  }
  f.part_o = reinterpret_cast<float*>(at(ws, pl.spec_o));
  f.part_lse = reinterpret_cast<float*>(at(ws, pl.spec_lse));
  hipError_t e = launch_flash(c.dtype, kFlashPartial, f, st);
  if (e != hipSuccess) return e;
  MergeParams m;
  memset(&m, 0, sizeof(m));
  m.part_o = f.part_o;
  m.part_lse = f.part_lse;
  m.n_splits = ns;
  m.n_q = g.m_spec;
  m.qa = g.n_special;
  m.qb = g.tf;
  m.qc = 0;
  m.n_heads = (int)g.n_heads;
  m.row_stride = g.n_heads * kHeadDim;
  m.o = o;
  m.o32 = o32;
  m.l2 = l2;
  return launch_merge(c.dtype, m, st);
}

// Compressed attention + exact top-k (k <= kTopkMaxK = 128):
//  1. flash attention over all M' windows, also writing per-group score bounds;
//  2. launch_topk: theta and the hot groups from the bounds, the hot groups'
//     keys >= theta as candidates, ranking -> topk (with a full score sweep
//     for the query tiles whose candidate lists overflow).
hipError_t run_compressed(const Call& c, const Plan& pl, const void* qc, const void* kc, const void* vc, float* oc,
                          int32_t* idx, float* score, void* ws, hipStream_t st, float* lse = nullptr) {
  const Geometry& g = c.g;
  if (g.n_windows == 0) return hipSuccess;
  FlashParams f = flash_base(c, qc, kc, vc);
  set_rows_identity(f, g.n_windows);
  f.n_splits = 1;
  f.kbeg[0] = 0;
  f.kend[0] = g.n_windows;
  f.oc = oc;
  f.part_lse = lse;
  // the windows of excluded frames as ascending, merged key ranges
  f.n_excl = 0;
  if (c.exclude && c.n_ctx > 0) {
    int fr[kMaxExcl];
    for (int i = 0; i < c.n_ctx; ++i) fr[i] = c.ctx[i];
    std::sort(fr, fr + c.n_ctx);
    for (int i = 0; i < c.n_ctx; ++i) {
      const int b = (int)(fr[i] * g.wpf), e = (int)((fr[i] + 1) * g.wpf);
      if (f.n_excl > 0 && b <= f.excl_end[f.n_excl - 1]) {
        f.excl_end[f.n_excl - 1] = std::max(f.excl_end[f.n_excl - 1], e);
      } else {
        f.excl_beg[f.n_excl] = b;
        f.excl_end[f.n_excl] = e;
        ++f.n_excl;
      }
    }
  }
  f.gbound = reinterpret_cast<float*>(at(ws, pl.gbound));
  f.gerr = reinterpret_cast<float*>(at(ws, pl.gerr));
  f.n_groups = pl.n_groups;
  f.group_tiles = pl.group_tiles;
  hipError_t e = launch_flash(c.dtype, kFlashBound, f, st);
  if (e != hipSuccess) return e;

  TopkParams r;
  memset(&r, 0, sizeof(r));
  r.q = qc;
  r.k = kc;
  r.row_stride = f.row_stride;
  r.n_heads = f.n_heads;
  r.n_q = g.n_windows;
  r.gbound = f.gbound;
  r.gerr = f.gerr;
  r.n_groups = pl.n_groups;
  r.group_tiles = pl.group_tiles;
  r.topk = c.topk;
  r.theta = reinterpret_cast<float*>(at(ws, pl.theta));
  r.hot = reinterpret_cast<uint32_t*>(at(ws, pl.hot));
  r.n_words = pl.n_words;
  r.cnt = reinterpret_cast<int32_t*>(at(ws, pl.cnt));
  r.cand = reinterpret_cast<uint2*>(at(ws, pl.cand));
  r.cap = pl.cap;
  r.n_chunks = pl.n_chunks;
  r.n_excl = f.n_excl;
  for (int i = 0; i < f.n_excl; ++i) {
    r.excl_beg[i] = f.excl_beg[i];
    r.excl_end[i] = f.excl_end[i];
  }
  r.topk_idx = idx;
  r.topk_score = score;
  return launch_topk(c.dtype, r, st);
}

// Context frames' part of the selection softmax: image queries over all T_f tokens of each context frame.
hipError_t run_context(const Call& c, const Plan& pl, const void* q, const void* k, const void* v, void* ws,
                       hipStream_t st) {
  const Geometry& g = c.g;
  FlashParams f = flash_base(c, q, k, v);
  f.n_q = g.m_img;
  f.qa = g.grid_h * g.grid_w;
  f.qb = g.tf;
  f.qc = g.n_special;
  f.n_splits = c.n_ctx;  // one split per context frame
  f.range_loop = ctx_range_loop(c) ? 1 : 0;
  for (int i = 0; i < c.n_ctx; ++i) {
    f.kbeg[i] = (int64_t)c.ctx[i] * g.tf;
    f.kend[i] = f.kbeg[i] + g.tf;
  }
  f.part_o = reinterpret_cast<float*>(at(ws, pl.ctx_o));
  f.part_lse = reinterpret_cast<float*>(at(ws, pl.ctx_lse));
  return launch_flash(c.dtype, kFlashPartial, f, st);
}

PoolParams pool_base(const Call& c) {
  PoolParams p;
  memset(&p, 0, sizeof(p));
  p.g = c.g;
  p.inv_area = 1.0f / (float)(c.g.pool * c.g.pool);
  return p;
}

SelectParams select_base(const Call& c, const Plan& pl, const void* q, const void* k, const void* v,
                         const int32_t* idx, void* ws) {
  SelectParams s;
  memset(&s, 0, sizeof(s));
  s.q = q;
  s.k = k;
  s.v = v;
  s.vblk = c.dtype == GSA_BF16 ? nullptr : at(ws, pl.vblk);
  s.topk_idx = idx;
  s.topk = c.topk;
  s.g = c.g;
  s.scale_log2 = c.scale * kLog2e;
  s.n_ctx = ctx_parts(c);
  if (c.n_ctx) {
    s.ctx_o = reinterpret_cast<const float*>(at(ws, pl.ctx_o));
    s.ctx_lse = reinterpret_cast<const float*>(at(ws, pl.ctx_lse));
  }
  return s;
}

}  // namespace

extern "C" {

const char* gsa_status_string(gsa_status s) {
  switch (s) {
    case GSA_OK: return "GSA_OK";
    case GSA_ERR_INVALID_ARG: return "GSA_ERR_INVALID_ARG: null, misaligned or aliasing pointer, or invalid argument value";
    case GSA_ERR_SHAPE: return "GSA_ERR_SHAPE: grid not divisible by the pool size, non-positive or oversized shape";
    case GSA_ERR_UNSUPPORTED: return "GSA_ERR_UNSUPPORTED: head_dim != 64, pool > 8, topk > 128 or unknown dtype";
    case GSA_ERR_WORKSPACE: return "GSA_ERR_WORKSPACE: workspace smaller than gsa_workspace_size()";
    case GSA_ERR_HIP: return "GSA_ERR_HIP: a HIP kernel launch failed";
  }
  return "unknown gsa_status";
}

gsa_status gsa_workspace_size(const gsa_config* cfg, gsa_op op, size_t* bytes) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!bytes) return GSA_ERR_INVALID_ARG;
  if (op < GSA_OP_FORWARD || op > GSA_OP_BACKWARD) return GSA_ERR_INVALID_ARG;
  *bytes = (size_t)make_plan(c, op).total;
  return GSA_OK;
}

gsa_status gsa_pool(const gsa_config* cfg, const void* q, const void* k, const void* v, void* qc, void* kc,
                    void* vc, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(qc) || !ptr_ok(kc) || !ptr_ok(vc)) return GSA_ERR_INVALID_ARG;
  PoolParams p = pool_base(c);
  p.src[0] = q;
  p.src[1] = k;
  p.src[2] = v;
  p.dst[0] = qc;
  p.dst[1] = kc;
  p.dst[2] = vc;
  p.first_tensor = 0;
  return hip_status(launch_pool(c.dtype, p, 3, static_cast<hipStream_t>(stream)));
}

gsa_status gsa_compressed_attn_topk(const gsa_config* cfg, const void* qc, const void* kc, const void* vc, float* oc,
                                    int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(qc) || !ptr_ok(kc) || !ptr_ok(vc) || !ptr_ok(oc) || !ptr_ok(topk_idx)) return GSA_ERR_INVALID_ARG;
  if (topk_score && !ptr_ok(topk_score)) return GSA_ERR_INVALID_ARG;
  Plan pl = make_plan(c, GSA_OP_COMPRESSED);
  if ((s = check_ws(pl, ws, ws_bytes)) != GSA_OK) return s;
  return hip_status(run_compressed(c, pl, qc, kc, vc, oc, topk_idx, topk_score, ws, static_cast<hipStream_t>(stream)));
}

gsa_status gsa_select_attn(const gsa_config* cfg, const void* q, const void* k, const void* v,
                           const int32_t* topk_idx, float* o_sel, void* ws, size_t ws_bytes, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(topk_idx) || !ptr_ok(o_sel)) return GSA_ERR_INVALID_ARG;
  Plan pl = make_plan(c, GSA_OP_SELECT);
  if ((s = check_ws(pl, ws, ws_bytes)) != GSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // fp32: the transposed V blocks the selection gathers (bf16 gathers K and V
  // rows from k and v themselves)
  hipError_t e = hipSuccess;
  if (c.dtype != GSA_BF16) {
    PoolParams pp = pool_base(c);
    pp.src[2] = v;
    pp.trans[2] = at(ws, pl.vblk);
    pp.first_tensor = 2;
    e = launch_pool(c.dtype, pp, 1, st);
  }
  if (e == hipSuccess && c.n_ctx) e = run_context(c, pl, q, k, v, ws, st);
  if (e != hipSuccess) return GSA_ERR_HIP;
  SelectParams sp = select_base(c, pl, q, k, v, topk_idx, ws);
  sp.osel = o_sel;
  return hip_status(launch_select(c.dtype, sp, st));
}

gsa_status gsa_special_attn(const gsa_config* cfg, const void* q, const void* k, const void* v, void* o, void* ws,
                            size_t ws_bytes, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o)) return GSA_ERR_INVALID_ARG;
  if (o == q || o == k || o == v) return GSA_ERR_INVALID_ARG;
  Plan pl = make_plan(c, GSA_OP_SPECIAL);
  if ((s = check_ws(pl, ws, ws_bytes)) != GSA_OK) return s;
  return hip_status(run_special(c, pl, q, k, v, o, ws, static_cast<hipStream_t>(stream)));
}

gsa_status gsa_gate_combine(const gsa_config* cfg, const void* q, const void* wg, const float* gate, const float* oc,
                            const float* o_sel, void* o, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(q) || !ptr_ok(oc) || !ptr_ok(o_sel) || !ptr_ok(o)) return GSA_ERR_INVALID_ARG;
  if (wg == nullptr && gate == nullptr) return GSA_ERR_INVALID_ARG;
  if ((wg && !ptr_ok(wg)) || (!wg && !ptr_ok(gate))) return GSA_ERR_INVALID_ARG;
  if (o == q) return GSA_ERR_INVALID_ARG;
  CombineParams p;
  p.q = q;
  p.wg = wg;
  p.gate = gate;
  p.oc = oc;
  p.osel = o_sel;
  p.o = o;
  p.g = c.g;
  return hip_status(launch_combine(c.dtype, p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// gsa_forward and gsa_forward_train (state: the training state, or null).
gsa_status forward_impl(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg, void* o,
                        void* state, size_t state_bytes, void* ws, size_t ws_bytes, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(wg) || !ptr_ok(o)) return GSA_ERR_INVALID_ARG;
  if (o == q || o == k || o == v) return GSA_ERR_INVALID_ARG;
  if (state && (((uintptr_t)state & (kAlign - 1)) != 0 || state == q || state == k || state == v || state == o))
    return GSA_ERR_INVALID_ARG;
  Plan pl = make_plan(c, GSA_OP_FORWARD);
  if ((s = check_ws(pl, ws, ws_bytes)) != GSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const TrainState ts = state_plan(c);
  if (state && (int64_t)state_bytes < ts.total) return GSA_ERR_WORKSPACE;
  auto saved = [&](int64_t off) { return state ? reinterpret_cast<float*>(at(state, off)) : nullptr; };

  // 1. pooling of Q/K/V (fp32: plus the transposed V blocks for the gather)
  PoolParams pp = pool_base(c);
  pp.src[0] = q;
  pp.src[1] = k;
  pp.src[2] = v;
  pp.dst[0] = at(ws, pl.qc);
  pp.dst[1] = at(ws, pl.kc);
  pp.dst[2] = at(ws, pl.vc);
  pp.trans[2] = c.dtype == GSA_BF16 ? nullptr : at(ws, pl.vblk);
  pp.first_tensor = 0;
  hipError_t e = launch_pool(c.dtype, pp, 3, st);
  // 2. special tokens over all tokens
  if (e == hipSuccess) e = run_special(c, pl, q, k, v, o, ws, st, saved(ts.spec_o32), saved(ts.spec_l2));
  // 3. compressed attention + top-k
  float* oc = state ? saved(ts.oc) : reinterpret_cast<float*>(at(ws, pl.oc));
  int32_t* idx = reinterpret_cast<int32_t*>(state ? at(state, ts.topk) : at(ws, pl.topk));
  if (e == hipSuccess)
    e = run_compressed(c, pl, pp.dst[0], pp.dst[1], pp.dst[2], oc, idx, nullptr, ws, st, saved(ts.lse_c));
  // 4. fixed-context partial
  if (e == hipSuccess && c.n_ctx) e = run_context(c, pl, q, k, v, ws, st);
  // 5. selection + upsample + gate
  if (e == hipSuccess) {
    SelectParams sp = select_base(c, pl, q, k, v, idx, ws);
    sp.wg = wg;
    sp.oc = oc;
    sp.o = o;
    sp.osel = saved(ts.osel);
    sp.l2 = saved(ts.l2sel);
    e = launch_select(c.dtype, sp, st);
  }
  return hip_status(e);
}

}  // namespace

extern "C" {

gsa_status gsa_forward(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg, void* o,
                       void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(cfg, q, k, v, wg, o, nullptr, 0, ws, ws_bytes, stream);
}

gsa_status gsa_train_state_size(const gsa_config* cfg, size_t* bytes) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!bytes) return GSA_ERR_INVALID_ARG;
  *bytes = (size_t)state_plan(c).total;
  return GSA_OK;
}

gsa_status gsa_forward_train(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg,
                             void* o, void* state, size_t state_bytes, void* ws, size_t ws_bytes, void* stream) {
  if (state == nullptr) return GSA_ERR_INVALID_ARG;
  return forward_impl(cfg, q, k, v, wg, o, state, state_bytes, ws, ws_bytes, stream);
}

gsa_status gsa_dense_attn(const gsa_config* cfg, const void* q, const void* k, const void* v, void* o, void* ws,
                          size_t ws_bytes, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  (void)ws;
  (void)ws_bytes;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o)) return GSA_ERR_INVALID_ARG;
  if (o == q || o == k || o == v) return GSA_ERR_INVALID_ARG;
  FlashParams f = flash_base(c, q, k, v);
  set_rows_identity(f, c.g.m_tokens);
  f.n_splits = 1;
  f.kbeg[0] = 0;
  f.kend[0] = c.g.m_tokens;
  f.o = o;
  return hip_status(launch_flash(c.dtype, kFlashFinal, f, static_cast<hipStream_t>(stream)));
}

gsa_status gsa_frame_attn(const gsa_config* cfg, const void* q, const void* k, const void* v, void* o,
                          void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(o)) return GSA_ERR_INVALID_ARG;
  if (o == q || o == k || o == v) return GSA_ERR_INVALID_ARG;
  // one batch per frame: its T_f query rows over its own T_f keys
  FlashParams f = flash_base(c, q, k, v);
  set_rows_identity(f, c.g.tf);
  f.n_splits = 1;
  f.kbeg[0] = 0;
  f.kend[0] = c.g.tf;
  f.n_batch = c.g.n_frames;
  f.q_bstride = c.g.tf;
  f.k_bstride = c.g.tf;
  f.o = o;
  return hip_status(launch_flash(c.dtype, kFlashFinal, f, static_cast<hipStream_t>(stream)));
}

gsa_status gsa_descriptor_count(const gsa_config* cfg, int64_t* n_set) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!n_set) return GSA_ERR_INVALID_ARG;
  *n_set = descriptor_plan(c).n_set;
  return GSA_OK;
}

gsa_status gsa_descriptor_set(const gsa_config* cfg, const void* k, const void* v, void* kd, void* vd,
                              void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(k) || !ptr_ok(v) || !ptr_ok(kd) || !ptr_ok(vd)) return GSA_ERR_INVALID_ARG;
  if (kd == k || kd == v || vd == k || vd == v || kd == vd) return GSA_ERR_INVALID_ARG;
  DescParams d = descriptor_plan(c);
  if (d.n_set > INT32_MAX - 64) return GSA_ERR_SHAPE;
  d.src[0] = k;
  d.src[1] = v;
  d.dst[0] = kd;
  d.dst[1] = vd;
  return hip_status(launch_descriptor(c.dtype, d, static_cast<hipStream_t>(stream)));
}

gsa_status gsa_descriptor_attn(const gsa_config* cfg, const void* q, const void* kd, const void* vd, void* o,
                               void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(q) || !ptr_ok(kd) || !ptr_ok(vd) || !ptr_ok(o)) return GSA_ERR_INVALID_ARG;
  if (o == q || o == kd || o == vd) return GSA_ERR_INVALID_ARG;
  const int64_t n_set = descriptor_plan(c).n_set;
  if (n_set > INT32_MAX - 64) return GSA_ERR_SHAPE;
  // every token over the n_set rows of the set (same row stride as q)
  FlashParams f = flash_base(c, q, kd, vd);
  set_rows_identity(f, c.g.m_tokens);
  f.n_splits = 1;
  f.kbeg[0] = 0;
  f.kend[0] = n_set;
  f.o = o;
  return hip_status(launch_flash(c.dtype, kFlashFinal, f, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// gsa_backward (state null: the forward quantities are recomputed) and
// gsa_backward_train (top-k sets and forward quantities read from the state).
gsa_status backward_impl(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg,
                         const int32_t* topk_idx, const void* state, size_t state_bytes, const void* d_o, float* dq,
                         float* dk, float* dv, float* dwg, void* ws, size_t ws_bytes, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  const TrainState ts = state_plan(c);
  if (state) {
    if (((uintptr_t)state & (kAlign - 1)) != 0) return GSA_ERR_INVALID_ARG;
    if ((int64_t)state_bytes < ts.total) return GSA_ERR_WORKSPACE;
    topk_idx = reinterpret_cast<const int32_t*>(at(const_cast<void*>(state), ts.topk));
  }
  auto saved = [&](int64_t off) { return reinterpret_cast<float*>(at(const_cast<void*>(state), off)); };
  const void* in[6] = {q, k, v, wg, topk_idx, d_o};
  const void* out[4] = {dq, dk, dv, dwg};
  for (const void* x : in)
    if (!ptr_ok(x)) return GSA_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i) {
    if (!ptr_ok(out[i])) return GSA_ERR_INVALID_ARG;
    for (const void* x : in)
      if (x == out[i]) return GSA_ERR_INVALID_ARG;
    for (int j = 0; j < i; ++j)
      if (out[j] == out[i]) return GSA_ERR_INVALID_ARG;
    if (state && out[i] == state) return GSA_ERR_INVALID_ARG;
  }
  const Geometry& g = c.g;
  if (g.n_windows * g.n_heads * (int64_t)c.topk > INT32_MAX) return GSA_ERR_SHAPE;
  Plan pl = make_plan(c, GSA_OP_BACKWARD);
  if ((s = check_ws(pl, ws, ws_bytes)) != GSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t H = g.n_heads;
  hipError_t e = hipSuccess;
  auto ok = [&](hipError_t x) { if (e == hipSuccess) e = x; return e == hipSuccess; };

  // 1. pooled Q/K/V and the window-blocked copies the selection passes gather
  PoolParams pp = pool_base(c);
  pp.src[0] = q;
  pp.src[1] = k;
  pp.src[2] = v;
  pp.dst[0] = at(ws, pl.qc);
  pp.dst[1] = at(ws, pl.kc);
  pp.dst[2] = at(ws, pl.vc);
  // (bf16: the selection backward transposes Q and K chunks in LDS)
  pp.rows[0] = at(ws, pl.qblk);
  pp.trans[0] = c.dtype == GSA_BF16 ? nullptr : at(ws, pl.qT);
  pp.rows[1] = at(ws, pl.kblk);
  pp.trans[1] = c.dtype == GSA_BF16 ? nullptr : at(ws, pl.kT);
  pp.rows[2] = at(ws, pl.vrow);
  // V^T only for an fp32 selection recompute
  pp.trans[2] = state || c.dtype == GSA_BF16 ? nullptr : at(ws, pl.vblk);
  ok(launch_pool(c.dtype, pp, 3, st));

  // 2. forward quantities: compressed output + log-sum-exp (one split)
  float* oc = state ? saved(ts.oc) : reinterpret_cast<float*>(at(ws, pl.oc));
  float* lse_c = state ? saved(ts.lse_c) : reinterpret_cast<float*>(at(ws, pl.lse_c));
  if (g.n_windows && !state) {
    FlashParams f = flash_base(c, at(ws, pl.qc), at(ws, pl.kc), at(ws, pl.vc));
    set_rows_identity(f, g.n_windows);
    f.n_splits = 1;
    f.kbeg[0] = 0;
    f.kend[0] = g.n_windows;
    f.part_o = oc;
    f.part_lse = lse_c;
    ok(launch_flash(c.dtype, kFlashPartial, f, st));
  }
  //    special rows: merged output in float, L2 and D = dO . O
  float* spec_o32 = state ? saved(ts.spec_o32) : reinterpret_cast<float*>(at(ws, pl.spec_o32));
  float* spec_l2 = state ? saved(ts.spec_l2) : reinterpret_cast<float*>(at(ws, pl.spec_l2));
  float* spec_dd = reinterpret_cast<float*>(at(ws, pl.spec_dd));
  FlashParams fs = flash_base(c, q, k, v);
  if (g.m_spec && state) {
    // the split layout of the key-range sweep, and D = dO . O from the saved rows
    // (a one-part merge: weight 1, the part itself)
    const int ns = pl.n_split;
    const int64_t tiles = (g.m_tokens + 31) / 32;
    fs.n_splits = ns;
    for (int i = 0; i < ns; ++i) {
      fs.kbeg[i] = tiles * i / ns * 32;
      fs.kend[i] = i + 1 == ns ? g.m_tokens : tiles * (i + 1) / ns * 32;
    }
    MergeParams m;
    memset(&m, 0, sizeof(m));
    m.part_o = spec_o32;
    m.part_lse = spec_l2;
    m.n_splits = 1;
    m.n_q = g.m_spec;
    m.qa = g.n_special;
    m.qb = g.tf;
    m.qc = 0;
    m.n_heads = (int)H;
    m.row_stride = H * kHeadDim;
    m.d_o = d_o;
    m.dd = spec_dd;
    ok(launch_merge(c.dtype, m, st));
  } else if (g.m_spec) {
    fs.n_q = g.m_spec;
    fs.qa = g.n_special;
    fs.qb = g.tf;
    fs.qc = 0;
    const int ns = pl.n_split;
    const int64_t tiles = (g.m_tokens + 31) / 32;
    fs.n_splits = ns;
    for (int i = 0; i < ns; ++i) {
      fs.kbeg[i] = tiles * i / ns * 32;
      fs.kend[i] = i + 1 == ns ? g.m_tokens : tiles * (i + 1) / ns * 32;
    }
    fs.part_o = reinterpret_cast<float*>(at(ws, pl.spec_o));
    fs.part_lse = reinterpret_cast<float*>(at(ws, pl.spec_lse));
    ok(launch_flash(c.dtype, kFlashPartial, fs, st));
    MergeParams m;
    memset(&m, 0, sizeof(m));
    m.part_o = fs.part_o;
    m.part_lse = fs.part_lse;
    m.n_splits = ns;
    m.n_q = g.m_spec;
    m.qa = g.n_special;
    m.qb = g.tf;
    m.qc = 0;
    m.n_heads = (int)H;
    m.row_stride = H * kHeadDim;
    m.o32 = spec_o32;
    m.l2 = spec_l2;
    m.d_o = d_o;
    m.dd = spec_dd;
    ok(launch_merge(c.dtype, m, st));
  }
  //    selection output and joint L2 (context partials first)
  float* osel = state ? saved(ts.osel) : reinterpret_cast<float*>(at(ws, pl.osel));
  float* l2sel = state ? saved(ts.l2sel) : reinterpret_cast<float*>(at(ws, pl.l2sel));
  if (!state) {
    if (c.n_ctx && e == hipSuccess) ok(run_context(c, pl, q, k, v, ws, st));
    SelectParams sp = select_base(c, pl, q, k, v, topk_idx, ws);
    sp.osel = osel;
    sp.l2 = l2sel;
    ok(launch_select(c.dtype, sp, st));
  }

  // 3. gate: dz (the selection backward stores dq = dz W_g + ...), dO_sel blocks,
  //    dO_comp, dW_g partials
  GateBwdParams gp;
  memset(&gp, 0, sizeof(gp));
  gp.q = q;
  gp.wg = wg;
  gp.d_o = d_o;
  gp.oc = oc;
  gp.osel = osel;
  gp.l2sel = l2sel;
  gp.g = g;
  gp.dzblk = reinterpret_cast<float*>(at(ws, pl.dzblk));
  gp.doblk = at(ws, pl.doblk);
  gp.doT = c.dtype == GSA_BF16 ? nullptr : at(ws, pl.doT);
  gp.l2blk = reinterpret_cast<float*>(at(ws, pl.l2blk));
  gp.dblk = reinterpret_cast<float*>(at(ws, pl.dblk));
  if (c.n_ctx) {
    gp.dosel_img = at(ws, pl.dosel_img);
    gp.dsel_img = reinterpret_cast<float*>(at(ws, pl.dsel_img));
  }
  gp.doc = at(ws, pl.doc);
  gp.dc = reinterpret_cast<float*>(at(ws, pl.dc));
  gp.lse_c = lse_c;
  gp.l2c = reinterpret_cast<float*>(at(ws, pl.l2c));
  gp.dwg_part = reinterpret_cast<float*>(at(ws, pl.dwg_part));
  ok(launch_gate_bwd(c.dtype, gp, st));
  DwgParams dp;
  dp.part = gp.dwg_part;
  dp.n_windows = g.n_windows;
  dp.n_heads = (int)H;
  dp.slices = reinterpret_cast<float*>(at(ws, pl.dwg_slices));
  dp.dwg = dwg;
  ok(launch_dwg_reduce(dp, st));

  FlashBwdParams b0;
  memset(&b0, 0, sizeof(b0));
  b0.row_stride = H * kHeadDim;
  b0.n_heads = (int)H;
  b0.scale = c.scale;
  b0.scale_log2 = c.scale * kLog2e;
  b0.n_splits = 1;
  b0.n_qsplits = 1;

  // 4. special tokens over all tokens: dq of the special rows, dk / dv of every row
  if (g.m_spec) {
    FlashBwdParams b = b0;
    b.q = q;
    b.k = k;
    b.v = v;
    b.d_o = d_o;
    b.n_q = g.m_spec;
    b.qa = g.n_special;
    b.qb = g.tf;
    b.qc = 0;
    b.do_mapped = 1;
    b.lse = spec_l2;
    b.lse_mul = 1.0f;
    b.dd = spec_dd;
    b.n_splits = fs.n_splits;
    for (int i = 0; i < fs.n_splits; ++i) {
      b.kbeg[i] = fs.kbeg[i];
      b.kend[i] = fs.kend[i];
    }
    b.dq = dq;
    b.part = reinterpret_cast<float*>(at(ws, pl.spec_o));  // the merged partials are no longer needed
    ok(launch_flash_bwd(c.dtype, kBwdDQ, b, st));
    if (b.n_splits > 1) {
      ReduceParams r;
      r.part = b.part;
      r.n_parts = b.n_splits;
      r.part_stride = g.m_spec * H * kHeadDim;
      r.n_rows = g.m_spec;
      r.n_heads = (int)H;
      r.qa = g.n_special;
      r.qb = g.tf;
      r.qc = 0;
      r.out = dq;
      r.accumulate = 0;
      ok(launch_reduce(r, st));
    }
    FlashBwdParams kv = b;
    kv.n_splits = 1;
    kv.kbeg[0] = 0;
    kv.kend[0] = g.m_tokens;
    kv.dk = dk;
    kv.dv = dv;
    kv.accumulate = 0;
    ok(launch_flash_bwd(c.dtype, kBwdDKDV, kv, st));
  } else {
    ok(launch_fill(dk, g.m_tokens * H * kHeadDim, st));
    ok(launch_fill(dv, g.m_tokens * H * kHeadDim, st));
  }

  // 5. compressed attention over the pooled windows
  float* dqc = reinterpret_cast<float*>(at(ws, pl.dqc));
  float* dkc = reinterpret_cast<float*>(at(ws, pl.dkc));
  float* dvc = reinterpret_cast<float*>(at(ws, pl.dvc));
  {
    FlashBwdParams b = b0;
    b.q = at(ws, pl.qc);
    b.k = at(ws, pl.kc);
    b.v = at(ws, pl.vc);
    b.d_o = gp.doc;
    b.n_q = g.n_windows;
    b.qa = g.n_windows > 0 ? g.n_windows : 1;
    b.qb = 0;
    b.qc = 0;
    b.do_mapped = 0;
    b.lse = gp.l2c;
    b.lse_mul = 1.0f;
    b.dd = gp.dc;
    b.kbeg[0] = 0;
    b.kend[0] = g.n_windows;
    b.dq = dqc;
    b.dk = dkc;
    b.dv = dvc;
    ok(launch_flash_bwd(c.dtype, kBwdDQ, b, st));
    ok(launch_flash_bwd(c.dtype, kBwdDKDV, b, st));
  }

  // 6. selection: inverse top-k lists, then the query and key sides (their
  //    stores also add each window token's pooled-row gradient / s^2)
  InvParams ip;
  ip.topk_idx = topk_idx;
  ip.topk = c.topk;
  ip.n_windows = g.n_windows;
  ip.n_heads = (int)H;
  ip.off = reinterpret_cast<int32_t*>(at(ws, pl.inv_off));
  ip.bsum = reinterpret_cast<int32_t*>(at(ws, pl.inv_bsum));
  ip.raw = reinterpret_cast<int32_t*>(at(ws, pl.inv_raw));
  ip.list = reinterpret_cast<int32_t*>(at(ws, pl.inv_list));
  ip.order = reinterpret_cast<int32_t*>(at(ws, pl.inv_order));
  ip.ccnt = reinterpret_cast<int32_t*>(at(ws, pl.inv_ccnt));
  ip.cbsum = reinterpret_cast<int32_t*>(at(ws, pl.inv_cbsum));
  ok(launch_inverse_index(ip, st));
  SelBwdParams sb;
  sb.qblk = at(ws, pl.qblk);
  sb.qT = at(ws, pl.qT);
  sb.kblk = at(ws, pl.kblk);
  sb.kT = at(ws, pl.kT);
  sb.vrow = at(ws, pl.vrow);
  sb.doblk = gp.doblk;
  sb.doT = gp.doT;
  sb.l2blk = gp.l2blk;
  sb.dblk = gp.dblk;
  sb.dzblk = gp.dzblk;
  sb.wg = wg;
  sb.topk_idx = topk_idx;
  sb.topk = c.topk;
  sb.inv_off = ip.off;
  sb.inv_list = ip.list;
  sb.order = ip.order;
  sb.g = g;
  sb.scale = c.scale;
  sb.scale_log2 = c.scale * kLog2e;
  sb.dqc = dqc;
  sb.dkc = dkc;
  sb.dvc = dvc;
  sb.inv_area = 1.0f / (float)(g.pool * g.pool);
  sb.dq = dq;
  sb.dk = dk;
  sb.dv = dv;
  ok(launch_sel_bwd(c.dtype, sb, st));

  // 7. context frames (one joint softmax with the selection): image queries over each frame
  if (c.n_ctx) {
    FlashBwdParams b = b0;
    b.q = q;
    b.k = k;
    b.v = v;
    b.d_o = gp.dosel_img;
    b.n_q = g.m_img;
    b.qa = g.grid_h * g.grid_w;
    b.qb = g.tf;
    b.qc = g.n_special;
    b.do_mapped = 0;
    b.lse = l2sel;
    b.lse_mul = 1.0f;
    b.dd = gp.dsel_img;
    b.n_splits = c.n_ctx;
    for (int i = 0; i < c.n_ctx; ++i) {
      b.kbeg[i] = (int64_t)c.ctx[i] * g.tf;
      b.kend[i] = b.kbeg[i] + g.tf;
    }
    b.dq = dq;
    b.accumulate = 1;
    b.part = reinterpret_cast<float*>(at(ws, pl.ctx_dq));
    ok(launch_flash_bwd(c.dtype, kBwdDQ, b, st));
    if (c.n_ctx > 1) {
      ReduceParams r;
      r.part = b.part;
      r.n_parts = c.n_ctx;
      r.part_stride = g.m_img * H * kHeadDim;
      r.n_rows = g.m_img;
      r.n_heads = (int)H;
      r.qa = g.grid_h * g.grid_w;
      r.qb = g.tf;
      r.qc = g.n_special;
      r.out = dq;
      r.accumulate = 1;
      ok(launch_reduce(r, st));
    }
    for (int i = 0; i < c.n_ctx; ++i) {
      FlashBwdParams kv = b;
      kv.n_splits = 1;
      kv.kbeg[0] = (int64_t)c.ctx[i] * g.tf;
      kv.kend[0] = kv.kbeg[0] + g.tf;
      kv.n_qsplits = pl.ctx_qsplits;
      kv.dk = dk;
      kv.dv = dv;
      kv.accumulate = 1;
      kv.part = reinterpret_cast<float*>(at(ws, pl.ctx_dkdv));
      ok(launch_flash_bwd(c.dtype, kBwdDKDV, kv, st));
      if (kv.n_qsplits > 1) {
        ReduceParams r;
        r.n_parts = kv.n_qsplits;
        r.part_stride = g.tf * H * kHeadDim;
        r.n_rows = g.tf;
        r.n_heads = (int)H;
        r.qa = g.tf;
        r.qb = 0;
        r.qc = kv.kbeg[0];
        r.accumulate = 1;
        r.part = kv.part;
        r.out = dk;
        ok(launch_reduce(r, st));
        r.part = kv.part + (int64_t)kv.n_qsplits * g.tf * H * kHeadDim;
        r.out = dv;
        ok(launch_reduce(r, st));
      }
    }
  }

  return hip_status(e);
}

}  // namespace

extern "C" {

gsa_status gsa_backward(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg,
                        const int32_t* topk_idx, const void* d_o, float* dq, float* dk, float* dv, float* dwg,
                        void* ws, size_t ws_bytes, void* stream) {
  return backward_impl(cfg, q, k, v, wg, topk_idx, nullptr, 0, d_o, dq, dk, dv, dwg, ws, ws_bytes, stream);
}

gsa_status gsa_backward_train(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg,
                              const void* state, size_t state_bytes, const void* d_o, float* dq, float* dk, float* dv,
                              float* dwg, void* ws, size_t ws_bytes, void* stream) {
  if (state == nullptr) return GSA_ERR_INVALID_ARG;
  return backward_impl(cfg, q, k, v, wg, nullptr, state, state_bytes, d_o, dq, dk, dv, dwg, ws, ws_bytes, stream);
}

}  // extern "C"

// ---- gsa_forward_noalloc: the forward's workspace in a static device array ----
// Every device the library runs on holds its own copy of `scratch` from the
// first launch on that device until the process ends.  In host code the name
// is only a stand-in: the device address comes from hipGetSymbolAddress, once
// per device, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[GSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on first use).
gsa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GSA_OK;
}

}  // namespace

extern "C" {

gsa_status gsa_forward_noalloc(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg,
                               void* o, void* stream) {
  Call c;
  gsa_status s = check_cfg(cfg, &c);
  if (s != GSA_OK) return s;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(wg) || !ptr_ok(o)) return GSA_ERR_INVALID_ARG;
  if (o == q || o == k || o == v) return GSA_ERR_INVALID_ARG;
  const int64_t need = make_plan(c, GSA_OP_FORWARD).total;
  if (need > (int64_t)GSA_NOALLOC_SCRATCH_BYTES) return GSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != GSA_OK) return s;
  return forward_impl(cfg, q, k, v, wg, o, nullptr, 0, ws, (size_t)GSA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
