// Tiled softmax attention on the gfx950 matrix cores, in three output modes:
//
//  * kFlashFinal    dense attention, normalised rows written in the input
//                   dtype (the dense comparator: all M queries over all M keys);
//  * kFlashPartial  split-K partials (normalised o and log-sum-exp) merged by
//                   merge_kernel: the special-token attention of the
//                   Paper-Notes page "Speed3R: Sparse Feed-forward 3D
//                   Reconstruction Models", section "全局稀疏注意力（GSA）核心设计"
//                   (M_spec queries over all M keys), and the fixed-context
//                   part of the selection branch (section "Speed3R-VGGT 适配");
//  * kFlashBound     compressed attention over the pooled windows (section
//                   "压缩分支") that also leaves, per group of key tiles, a
//                   lower bound of each query's best raw guide score
//                   S = Qc Kc^T; refine_kernel below turns them into the exact
//                   top-k (section "选择分支").  S is never written out.
//
// Work decomposition: a workgroup of WAVES wavefronts owns 32*WAVES query
// rows of one head and one key split; each wavefront owns 32 query rows.  Key
// tiles of 32 keys are staged once per workgroup in LDS (K as rows, V
// transposed so the PV operand is a contiguous read) and shared by all its
// waves.  Per tile and wave:
//   S^T[32 keys x 32 q] = K Q^T       4 x v_mfma_f32_32x32x16_bf16 (K=d=64)
//   online softmax on S^T             exp2 of log2e-scaled logits, lazy rescale
//   O^T[64 dv x 32 q] += V^T P^T      4 x v_mfma_f32_32x32x16_bf16
// Lane l holds query l%32 and 16 of the tile's keys; the other 16 keys of the
// same query sit in lane l^32.
//
#include <math.h>

#include <type_traits>

#include "flash_frag.h"
#include "gsa_device.h"
#include "gsa_kernels.h"

namespace gsa {

constexpr float kLazyRescale = 8.0f; // rescale only when the max grows by > 2^8
// Attention modes without a per-tile max: a tile is redone after a rescale
// only when its weights against the running reference sum to 2^64 or more.
constexpr float kSumLimit = 0x1p64f;

// ---- the kernel ---------------------------------------------------------------
// The ring of bf16 K/V tile buffers: two buffers of two 32-key tiles each
// (separate arrays, so the compiler can tell which buffer a global-to-LDS
// load writes).  Only the kernels that use them get them allocated.
__shared__ __attribute__((aligned(16))) __bf16 ring64a[kKT * kHeadDim * 4];
__shared__ __attribute__((aligned(16))) __bf16 ring64b[kKT * kHeadDim * 4];

// The bf16 bound mode asks for four workgroups per CU (at most 128 VGPRs),
// the occupancy of the plain attention modes.
template <typename T, int WAVES, int MODE, bool RLOOP = false>
__global__ __launch_bounds__(WAVES * 64, MODE == kFlashBound && sizeof(T) == 2 ? 4 : 1) void flash_kernel(FlashParams p) {
  using TL = Tile<T>;
  using F = Frag32<T>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // bf16 key tiles go from global memory straight into LDS (a ring of three
  // static buffers, below); fp32 tiles are staged through registers into two
  // buffers in the dynamic LDS.
  constexpr bool DMA = sizeof(T) == 2;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 31, hf = lane >> 5;

  constexpr int QW = WAVES * 32;
  const int64_t n_qt = (p.n_q + QW - 1) / QW;
  const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t qt = w % n_qt;
  const int64_t hs = w / n_qt;
  const int h = (int)(hs % p.n_heads);
  const int64_t sb = hs / p.n_heads;
  // RLOOP (kFlashPartial, range_loop set): the workgroup sweeps every split
  // in turn into one partial (index 0); otherwise the grid holds one split each.
  static_assert(!RLOOP || MODE == kFlashPartial, "range loop: partial mode only");
  constexpr bool rloop = RLOOP;
  const int grid_splits = rloop ? 1 : p.n_splits;
  const int split = (int)(sb % grid_splits);
  const int64_t batch = sb / grid_splits;
  const int part = rloop ? 0 : split;

  const int64_t qrow = qt * QW + wv * 32 + r;
  const bool qvalid = qrow < p.n_q;
  // A wave whose 32 query rows all lie past the end (the last query tile of a
  // batch, e.g. 21 of a frame's 128-row tail tile) still loads its share of
  // every key tile and meets the others at each barrier, but skips the
  // matrix-core and softmax work, leaving its SIMD to the other workgroups.
  // Not in the split-K partial sweeps: there the 40-odd query tiles of a key
  // range stream the same K/V tiles through L2 together, and the faster tail
  // workgroup among them raised the special attention's HBM fetch from 10.7
  // to 39 GB per launch at 1000 frames (and its time by ~3 %).
  const bool wave_live = MODE == kFlashPartial || wave_any(qvalid);
  const int64_t hoff = (int64_t)h * kHeadDim;
  const int64_t qtok = batch * p.q_bstride + (qrow / p.qa) * p.qb + p.qc + qrow % p.qa;
  const T* K = static_cast<const T*>(p.k);
  const T* V = static_cast<const T*>(p.v);
  typename F::Q qf = F::load_q(qvalid ? static_cast<const T*>(p.q) + qtok * p.row_stride + hoff : nullptr, hf);
  // Let the query fragment land before any tile prefetch is issued, so the
  // loop never has to drain the prefetch queue to be sure of it.
  __builtin_amdgcn_s_waitcnt(0);

  f32x16 o[2] = {{}, {}};
  float m_run = -INFINITY, l_run = 0.0f;
  bool first = true;
  const float c = p.scale_log2;
  const float rc = 1.0f / c;

  // kFlashBound: running max over the current group of fl(tile max u + m),
  // the largest |m| seen in the group, the group's last tile and its index.
  // The bounds are written with buffer stores: scalar base (the group's row
  // of this head, 64-bit pointer arithmetic), one per-lane offset (the query
  // row; the host keeps n_q * 4 below 2^31).
  // gbu: this lane's max of u since the reference m_run last changed (so
  // fl(gbu + m_run) is the max of fl(u + m_run), adding m being monotonic);
  // emax: the largest error term of the query's finite group bounds.
  float gb = -INFINITY, gbu = -INFINITY, gm_abs = 0.0f, emax = 0.0f;
  int gend = p.group_tiles - 1, gi = 0;
  const int gb_off = (int)(qrow * 4);

  // Key tiles of split rs: tile t covers keys kb + 32t .. kb + 32t + 31.
  // Prefetches past the last tile re-read the last tile (never used), so the
  // load/store pattern has no branches and the compiler can keep two tiles of
  // loads in flight across the barriers.
  // Positions inside the range are int32 (the host keeps token counts below
  // 2^31 - 64), so the per-tile bookkeeping is scalar 32-bit arithmetic.
  // Between two splits of a range loop the tile buffers are free: every wave
  // has passed the last barrier after its last read, and a wave's loads
  // still in flight write only the LDS chunks that wave loads.
  const int rs_end = rloop ? p.n_splits : split + 1;
  for (int rs = rloop ? 0 : split; rs < rs_end; ++rs) {
  const int64_t kb = p.kbeg[rs] + batch * p.k_bstride;
  const int nk = (int)(p.kend[rs] - p.kbeg[rs]);
  const int n_tiles = (nk + kKT - 1) / kKT, n_full = nk / kKT;
  if (gend > n_tiles - 1) gend = n_tiles - 1;
  auto tile_rel = [&](int t) { return (t < n_tiles ? t : n_tiles - 1) * kKT; };
  ExclCursor excl;  // kFlashBound: the excluded key ranges (single range from key 0)

  // One tile t from the K/V tile at kt (V follows K).  A step past the last
  // tile (the loops below run in whole unrolled rounds) sees only masked keys.
  auto compute = [&](int t, const T* kt) __attribute__((always_inline)) {
    if (!wave_live) return;
    const int64_t cur0 = kb + (int64_t)t * kKT;
    const T* vt = kt + TL::K_ELEMS;
    f32x16 s = F::qk(kt, r, hf, qf);
    if (t >= n_full) {
      const int lim = nk - t * kKT - 4 * hf;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i / 4) + (i % 4) >= lim) s[i] = -INFINITY;
    }
    if (first) {
      // the running max starts at the first tile's max (every tile holds a valid key)
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, xor_lane(mx, 32));
      m_run = mx * c;
      first = false;
    }
    // u = shifted log2-domain logits; every max below is taken on u, which the
    // compiler knows to be canonical, so the reductions are bare v_max3 ops
    f32x16 u;
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = fmaf(s[i], c, -m_run);
    if constexpr (MODE == kFlashFinal || MODE == kFlashPartial) {
      // No per-tile max.  The weights are formed against the running
      // reference m_run (the first tile's max, raised only here) and summed;
      // only a tile whose weights sum to 2^64 or more (or overflow) is redone,
      // after moving the reference to the tile's max.  Below that every
      // weight, the row sum (at most 2^31 keys) and the products with V stay
      // finite, and since the reference never exceeds the true max, no weight
      // that matters underflows: the result is the same softmax.
      f32x16 pw;
#pragma unroll
      for (int i = 0; i < 16; ++i) pw[i] = fast_exp2(u[i]);
      float ts = 0.0f;
      typename F::P pp = F::to_p(pw, ts);
      if (wave_any(!(ts < kSumLimit))) {
        const float m0 = max3(u[0], u[1], u[2]), m1 = max3(u[3], u[4], u[5]), m2 = max3(u[6], u[7], u[8]);
        const float m3 = max3(u[9], u[10], u[11]), m4 = max3(u[12], u[13], u[14]);
        float mt = max3(max3(m0, m1, m2), max3(m3, m4, u[15]), u[15]);
        // both halves of the query, and never downwards (a fully masked
        // tile's max is -inf)
        mt = fmaxf(fmaxf(mt, xor_lane(mt, 32)), 0.0f);
        const float alpha = fast_exp2(-mt);
        m_run += mt;
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[n][i] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) pw[i] = fast_exp2(u[i] - mt);
        ts = 0.0f;
        pp = F::to_p(pw, ts);
      }
      l_run += ts;
      F::pv(vt, lane, pp, o);
      return;
    }
    float mu;
    {
      const float m0 = max3(u[0], u[1], u[2]), m1 = max3(u[3], u[4], u[5]), m2 = max3(u[6], u[7], u[8]);
      const float m3 = max3(u[9], u[10], u[11]), m4 = max3(u[12], u[13], u[14]);
      mu = max3(max3(m0, m1, m2), max3(m3, m4, u[15]), u[15]);
    }
    // mu is this lane's max over its 16 keys; the query's other 16 keys are in
    // lane l^32.  The hot path needs no cross-lane step: whether any query of
    // the wave must rescale is the same test on either half, and only the
    // (cold) rescale combines the halves.
    if constexpr (MODE == kFlashBound) {
      // Lower bound of the tile's best candidate score, recovered from u and
      // the running max before any rescale: |fl(fl(u + m) / c) - s| stays
      // below 2^-22 |s| + 2^-24 |m / c|, so subtracting 2^-20 (|a| + |m / c|)
      // gives a true lower bound.  Windows of excluded frames do not count.
      // gb runs per lane; the halves are combined when the group is written.
      // The reference is added only when it changes (a rescale) and at the
      // group's end, and so is |m| folded into gm_abs.
      float mt = mu;
      const uint32_t em = p.n_excl ? excl.mask(p, (int)cur0) : 0u;
      if (em) {
        float x = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!((em >> (8 * (i / 4) + 4 * hf + (i % 4))) & 1u)) x = fmaxf(x, u[i]);
        mt = x;
      }
      gbu = fmaxf(gbu, mt);
      if (t == gend) {
        gb = fmaxf(gb, gbu + m_run);
        gm_abs = fmaxf(gm_abs, fabsf(m_run));
        const float gq = fmaxf(gb, xor_lane(gb, 32));  // uniform branch: every lane takes part
        const float a = gq * rc;
        const float e = ldexpf(fabsf(a) + gm_abs * rc, -20);
        if (a > -INFINITY) emax = fmaxf(emax, e);  // a group of excluded keys only has no bound
        if (hf == 0 && qvalid) {
          const __amdgpu_buffer_rsrc_t gbr = __builtin_amdgcn_make_buffer_rsrc(
              p.gbound + ((int64_t)h * p.n_groups + gi) * p.n_q, (short)0, (int)(p.n_q * 4), 0x00020000);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a - e), gbr, gb_off, 0, 0);
        }
        gb = -INFINITY;
        gbu = -INFINITY;
        gm_abs = 0.0f;
        gend = min(gend + p.group_tiles, n_tiles - 1);
        ++gi;
      }
    }
    // lazy rescale: only when the max has grown by more than 2^kLazyRescale
    if (wave_any(mu > kLazyRescale)) {
      mu = fmaxf(mu, xor_lane(mu, 32));
      if (mu > kLazyRescale) {
        if constexpr (MODE == kFlashBound) {
          gb = fmaxf(gb, gbu + m_run);
          gm_abs = fmaxf(gm_abs, fabsf(m_run));
          gbu = -INFINITY;
        }
        const float alpha = fast_exp2(-mu);
        m_run += mu;
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[n][i] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) u[i] -= mu;
      }
    }
    f32x16 pw;
#pragma unroll
    for (int i = 0; i < 16; ++i) pw[i] = fast_exp2(u[i]);
    const typename F::P pp = F::to_p(pw, l_run);
    F::pv(vt, lane, pp, o);
  };

  if constexpr (DMA) {
    // Two buffers of two tiles (64 keys).  Step u issues the loads of tiles
    // 2u+2 and 2u+3 into the buffer step u-1 used (every wave left it at the
    // last barrier), computes tiles 2u and 2u+1 (those past the last are
    // skipped), waits for its own loads and meets the other waves at a
    // barrier, after which the next pair is complete in LDS: one barrier per
    // 64 keys with two tiles' compute to cover the loads (a ring of three
    // 32-key tiles, the same prefetch distance, was 0.3 ms slower on the
    // compressed step at 1000 frames).
    // A tile is 512 16-byte chunks: K chunks 0..255, then V.  This wave
    // loads NDMA of them, lane l chunk 64 (WAVES j + wave) + l into the same
    // LDS chunk, which holds chunk c' of key row (chunk % 256) / 8 of its
    // operand, i.e. that row's global chunk c' ^ swz(row).
    constexpr int NDMA = (2 * kKT * kHeadDim / 8) / (WAVES * 64);
    static_assert(NDMA >= 1 && NDMA * WAVES * 64 == 2 * kKT * kHeadDim / 8, "tile must split evenly over the waves");
    constexpr int TE = kKT * kHeadDim * 2;  // elements of one tile (K, then V)
    const int wu = __builtin_amdgcn_readfirstlane(wv);
    int goff[NDMA];
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int ch = (64 * (WAVES * j + wu) + lane) & 255, row = ch >> 3;
      goff[j] = (int)(row * p.row_stride * 2 + (((ch & 7) ^ TL::swz(row)) << 4));
    }
    auto dma_tile = [&](__bf16* buf, int t) __attribute__((always_inline)) {
      const int rel = tile_rel(t), valid = min(nk - rel, kKT);
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(K, p.row_stride, hoff, kb + rel, valid);
      const __amdgpu_buffer_rsrc_t rv = tile_rsrc(V, p.row_stride, hoff, kb + rel, valid);
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const int c0 = 64 * (WAVES * j + wu);  // first chunk of this wave's load (the operand is uniform)
        lds_load16(c0 < 256 ? rk : rv, buf + 8 * c0, goff[j]);
      }
    };
    auto dma_pair = [&](__bf16* buf, int u) __attribute__((always_inline)) {
      dma_tile(buf, 2 * u);
      dma_tile(buf + TE, 2 * u + 1);
    };
    // Wait for this wave's loads and every LDS read, then meet at the
    // barrier.  No memory fence (the waits cover it); the compiler barriers
    // keep every memory access on its side.
    auto pair_barrier = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x70);  // vmcnt(0) lgkmcnt(0), expcnt untouched
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    dma_pair(ring64a, 0);
    pair_barrier();
    auto step = [&](int u, const __bf16* cur, __bf16* fill) __attribute__((always_inline)) {
      dma_pair(fill, u + 1);
      if (2 * u < n_tiles) compute(2 * u, cur);
      if (2 * u + 1 < n_tiles) compute(2 * u + 1, cur + TE);
      pair_barrier();
    };
    for (int u = 0; 2 * u < n_tiles; u += 2) {
      step(u, ring64a, ring64b);
      step(u + 1, ring64b, ring64a);
    }
    // (the last barrier waited for every load, so the LDS can be handed on)
  } else {
    // two LDS buffers fed from two register stages: compute tile t from
    // buffer t%2, move tile t+1 from stage `nxt` into the other buffer and
    // reuse `nxt` for tile t+3 (unrolled by two so the stages swap roles
    // without register copies, which would wait for the loads in flight)
    T* const kbuf0 = reinterpret_cast<T*>(smem);
    T* const kbuf1 = reinterpret_cast<T*>(smem + TL::BYTES);
    auto load_tile = [&](TileLoader<T, WAVES * 64>& ld, int t) {
      const int rel = tile_rel(t);
      ld.load(K, V, p.row_stride, hoff, kb + rel, min(nk - rel, kKT), tid);
    };
    TileLoader<T, WAVES * 64> sa, sb;
    load_tile(sa, 0);
    load_tile(sb, 1);
    sa.store(kbuf0, kbuf0 + TL::K_ELEMS, tid);
    load_tile(sa, 2);
    lds_barrier();
    auto step = [&](int t, TileLoader<T, WAVES * 64>& nxt) __attribute__((always_inline)) {
      compute(t, (t & 1) ? kbuf1 : kbuf0);
      T* kn = (t & 1) ? kbuf0 : kbuf1;
      nxt.store(kn, kn + TL::K_ELEMS, tid);
      load_tile(nxt, t + 3);
      lds_barrier();
    };
    for (int t = 0; t < n_tiles; t += 2) {
      step(t, sb);
      step(t + 1, sa);
    }
  }
  }  // splits of the range loop

  // ---- epilogue ----
  const float l = l_run + xor_lane(l_run, 32);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (qvalid) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dv0 = 32 * n + 8 * a + 4 * hf;
        f32x4 v4 = {o[n][4 * a] * inv, o[n][4 * a + 1] * inv, o[n][4 * a + 2] * inv, o[n][4 * a + 3] * inv};
        if constexpr (MODE == kFlashFinal) {
          T* dst = static_cast<T*>(p.o) + qtok * p.row_stride + hoff + dv0;
          if constexpr (sizeof(T) == 2) {
            bf16x4 b4 = {(__bf16)v4[0], (__bf16)v4[1], (__bf16)v4[2], (__bf16)v4[3]};
            *reinterpret_cast<bf16x4*>(dst) = b4;
          } else {
            *reinterpret_cast<f32x4*>(dst) = v4;
          }
        } else if constexpr (MODE == kFlashPartial) {
          float* dst = p.part_o + ((part * p.n_q + qrow) * p.n_heads + h) * kHeadDim + dv0;
          *reinterpret_cast<f32x4*>(dst) = v4;
        } else {
          float* dst = p.oc + (qrow * p.n_heads + h) * kHeadDim + dv0;
          *reinterpret_cast<f32x4*>(dst) = v4;
        }
      }
    }
    // log-sum-exp of the row (natural log); the compressed sweep writes it
    // only when asked (training state)
    if constexpr (MODE == kFlashPartial || MODE == kFlashBound) {
      if (hf == 0 && (MODE == kFlashPartial || p.part_lse))
        p.part_lse[(part * p.n_q + qrow) * p.n_heads + h] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    }
    // The true best score of a group lies within 1.25 e (+ an ulp) of its
    // stored bound a - e (|fl(fl(u + m) / c) - s| <= 2^-22 |s| + 2^-24 |m / c|);
    // 4 e also covers the rounding of theta - E when the hot groups are picked.
    if constexpr (MODE == kFlashBound) {
      if (hf == 0) p.gerr[(int64_t)h * p.n_q + qrow] = 4.0f * emax;
    }
  }

}

// Combine split partials: o = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - max).
template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t qh = gid / 16;
  const int chunk = (int)(gid % 16);
  if (qh >= p.n_q * p.n_heads) return;
  const int64_t q = qh / p.n_heads;
  const int h = (int)(qh % p.n_heads);
  float mx = -INFINITY;
  for (int s = 0; s < p.n_splits; ++s) mx = fmaxf(mx, p.part_lse[(s * p.n_q + q) * p.n_heads + h]);
  float den = 0.0f;
  f32x4 acc = {0, 0, 0, 0};
  for (int s = 0; s < p.n_splits; ++s) {
    const float lse = p.part_lse[(s * p.n_q + q) * p.n_heads + h];
    const float wgt = lse == -INFINITY ? 0.0f : expf(lse - mx);
    den += wgt;
    f32x4 x = *reinterpret_cast<const f32x4*>(p.part_o + ((s * p.n_q + q) * p.n_heads + h) * kHeadDim + 4 * chunk);
    acc += wgt * x;
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const int64_t tok = (q / p.qa) * p.qb + p.qc + q % p.qa;
  const f32x4 res = acc * inv;
  if (p.o) {
    T* dst = static_cast<T*>(p.o) + tok * p.row_stride + (int64_t)h * kHeadDim + 4 * chunk;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(res[e]);
  }
  if (p.o32) *reinterpret_cast<f32x4*>(p.o32 + (q * p.n_heads + h) * kHeadDim + 4 * chunk) = res;
  if (p.l2 && chunk == 0) p.l2[q * p.n_heads + h] = den > 0.0f ? mx * kLog2e + log2f(den) : INFINITY;
  if (p.dd) {
    // D = d_o . o over the 16 threads (4 channels each) of this (query, head)
    const T* g = static_cast<const T*>(p.d_o) + tok * p.row_stride + (int64_t)h * kHeadDim + 4 * chunk;
    float x = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) x += to_f32(g[e]) * res[e];
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) x += xor_lane(x, m);
    if (chunk == 0) p.dd[q * p.n_heads + h] = x;
  }
}

template <typename T, int WAVES, int MODE, bool RLOOP = false>
static hipError_t launch_flash_t(const FlashParams& p, hipStream_t stream) {
  const int64_t n_qt = (p.n_q + WAVES * 32 - 1) / (WAVES * 32);
  const int64_t grid_splits = RLOOP ? 1 : p.n_splits;
  const int64_t blocks = n_qt * p.n_heads * grid_splits * p.n_batch;
  if (blocks == 0) return hipSuccess;
  if (p.n_batch < 1 || (p.n_batch > 1 && MODE != kFlashFinal) || p.range_loop != (RLOOP ? 1 : 0) ||
      blocks > 0xffffffffLL)
    return hipErrorInvalidValue;
  size_t lds = sizeof(T) == 2 ? 0 : 2 * (size_t)Tile<T>::BYTES;  // bf16 tiles live in static LDS
  const void* fn = reinterpret_cast<const void*>(&flash_kernel<T, WAVES, MODE, RLOOP>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((flash_kernel<T, WAVES, MODE, RLOOP>), dim3((unsigned)blocks), dim3(WAVES * 64), lds, stream, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_flash_dt(int mode, const FlashParams& p, hipStream_t stream) {
  if (mode == kFlashFinal) return launch_flash_t<T, 4, kFlashFinal>(p, stream);
  if (mode == kFlashPartial)
    return p.range_loop ? launch_flash_t<T, 4, kFlashPartial, true>(p, stream) : launch_flash_t<T, 4, kFlashPartial>(p, stream);
  if (mode == kFlashBound) return launch_flash_t<T, 4, kFlashBound>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_flash(int dtype, int mode, const FlashParams& p, hipStream_t stream) {
  return dtype == kBF16 ? launch_flash_dt<__bf16>(mode, p, stream) : launch_flash_dt<float>(mode, p, stream);
}

hipError_t launch_merge(int dtype, const MergeParams& p, hipStream_t stream) {
  const int64_t threads = p.n_q * p.n_heads * 16;
  if (threads == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(merge_kernel<__bf16>, dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<float>, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gsa
