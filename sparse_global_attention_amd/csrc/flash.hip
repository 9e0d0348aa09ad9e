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

// ---- candidates of the exact top-k ------------------------------------------
struct Cand {
  float s;
  int j;
};

// Excluded keys of a 32-key tile as a bit mask (bit i = key key0 + i),
// uniform across the wave.  Tiles are visited in increasing key order, so a
// cursor passes the ranges that end before the tile once and a tile usually
// tests no range at all (scalar 32-bit arithmetic: key counts are int32).
struct ExclCursor {
  int x = 0;
  template <typename P>
  __device__ __forceinline__ uint32_t mask(const P& p, int key0) {
    while (x < p.n_excl && p.excl_end[x] <= key0) ++x;
    uint32_t m = 0;
    for (int y = x; y < p.n_excl && p.excl_beg[y] < key0 + kKT; ++y) {
      const int lo = max(p.excl_beg[y] - key0, 0), hi = min(p.excl_end[y] - key0, kKT);
      m |= (hi - lo == kKT ? 0xffffffffu : (1u << (hi - lo)) - 1u) << lo;
    }
    return m;
  }
};

// ---- the kernel ---------------------------------------------------------------
// The ring of bf16 K/V tile buffers (three separate arrays, so the compiler
// can tell which buffer a global-to-LDS load writes and wait only for that).
// Only the kernels that use them get them allocated.
__shared__ __attribute__((aligned(16))) __bf16 ring0[kKT * kHeadDim * 2];
__shared__ __attribute__((aligned(16))) __bf16 ring1[kKT * kHeadDim * 2];
__shared__ __attribute__((aligned(16))) __bf16 ring2[kKT * kHeadDim * 2];

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
  // The bounds of this head are written with buffer stores: scalar base (the
  // head's slab) and group offset, one per-lane offset (the query row).
  // gbu: this lane's max of u since the reference m_run last changed (so
  // fl(gbu + m_run) is the max of fl(u + m_run), adding m being monotonic)
  float gb = -INFINITY, gbu = -INFINITY, gm_abs = 0.0f;
  int gend = p.group_tiles - 1, gi = 0;
  const int64_t slab = MODE == kFlashBound ? (int64_t)p.n_groups * p.n_q * 4 : 0;
  const __amdgpu_buffer_rsrc_t gbr = __builtin_amdgcn_make_buffer_rsrc(
      MODE == kFlashBound ? p.gbound + (int64_t)h * p.n_groups * p.n_q : nullptr, (short)0,
      (int)(slab < 0x7fffffff ? slab : 0x7fffffff), 0x00020000);
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
        if (hf == 0 && qvalid) {
          const float a = gq * rc;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a - ldexpf(fabsf(a) + gm_abs * rc, -20)), gbr, gb_off,
                                                (int)((int64_t)gi * p.n_q * 4), 0);
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
    // Ring of three tile buffers.  Step t issues the loads of tile t+2 into
    // the buffer tile t-1 used (every wave left it at the last barrier),
    // computes tile t, waits for its own loads of tile t+1 (only tile t+2's
    // stay in flight: loads complete in order) and meets the other waves at
    // a barrier, after which tile t+1 is complete in LDS.
    // A tile is 512 16-byte chunks: K chunks 0..255, then V.  This wave
    // loads NDMA of them, lane l chunk 64 (WAVES j + wave) + l into the same
    // LDS chunk, which holds chunk c' of key row (chunk % 256) / 8 of its
    // operand, i.e. that row's global chunk c' ^ swz(row).
    constexpr int NDMA = (2 * kKT * kHeadDim / 8) / (WAVES * 64);
    static_assert(NDMA >= 1 && NDMA * WAVES * 64 == 2 * kKT * kHeadDim / 8, "tile must split evenly over the waves");
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
    // Wait until at most the NDMA loads of the newest tile are in flight
    // and every LDS read has returned, then meet at the barrier.  No memory
    // fence: a workgroup release fence would also wait for the newest tile's
    // loads.  The compiler barriers keep every memory access on its side.
    auto ring_barrier = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x70 | NDMA);  // vmcnt(NDMA) lgkmcnt(0), expcnt untouched
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    dma_tile(ring0, 0);
    dma_tile(ring1, 1);
    ring_barrier();
    auto step = [&](int t, const __bf16* cur, __bf16* fill) __attribute__((always_inline)) {
      dma_tile(fill, t + 2);
      compute(t, cur);
      ring_barrier();
    };
    for (int t = 0; t < n_tiles; t += 3) {
      step(t, ring0, ring2);
      step(t + 1, ring1, ring0);
      step(t + 2, ring2, ring1);
    }
    // the last prefetches (re-reads of the last tile) must land before the
    // workgroup's LDS can be handed to another workgroup
    __builtin_amdgcn_s_waitcnt(0x70);  // vmcnt(0) lgkmcnt(0)
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
  }

}

// ---- exact top-k from the group bounds ---------------------------------------
// Order-preserving map of floats to unsigned keys and back.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// The next float above x (x finite or -inf): "y > x" is "y >= next_up(x)".
// (both zeros map to +0 first, so the result is the smallest positive value)
__device__ __forceinline__ float next_up(float x) { return key_value(order_key(x == 0.0f ? 0.0f : x) + 1u); }


// theta = the k-th largest of the query's group bounds.  Each group bound is
// at most the score of one distinct candidate key, so the k-th best candidate
// score is >= theta, and every top-k key scores >= theta.  Radix select over
// the order keys, bit by bit from the top; the two lanes of a query hold the
// even and the odd groups (n_groups <= 2 * kMaxGroupsPerLane).  Returns -inf
// when there are fewer than k finite bounds (then every candidate qualifies).
template <int kMaxGroupsPerLane>
__device__ float kth_bound(const RefineParams& p, int64_t qrow, int h, int hf, bool qvalid) {
  const int NG = p.n_groups;
  const int per = (NG - hf + 1) / 2;
  const float* src = p.gbound + (int64_t)h * NG * p.n_q + (qvalid ? qrow : 0);
  uint32_t kv[kMaxGroupsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxGroupsPerLane; ++i) {
    // clamped, unconditional loads; out-of-range slots become key 0, which no
    // candidate key below reaches (every candidate key has a bit set)
    const int g = min(2 * i + hf, NG - 1);
    const float x = src[(int64_t)g * p.n_q];
    kv[i] = (qvalid && i < per) ? order_key(x) : 0u;
  }
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kMaxGroupsPerLane; ++i) cnt += kv[i] >= cand ? 1 : 0;
    cnt = sum_halves(cnt);
    if (cnt >= p.topk) T = cand;
  }
  return T > order_key(-INFINITY) ? key_value(T) : -INFINITY;
}

__device__ __forceinline__ bool cand_better(Cand a, Cand b) { return a.s > b.s || (a.s == b.s && a.j < b.j); }

// Candidate slots of one wave in LDS: slot i of query r at buf[i * 32 + r],
// kRefineSlots slots per query.  The even lane of a query fills slots upwards
// from 0 (its entries are [0, lo)), the odd lane downwards from the top (its
// entries are (hi, kRefineSlots)); the slots between are free.  Within each
// lane's range the entries are in ascending key order.
struct CandSlots {
  Cand* buf;
  int r, hf;
  int fp;      // this lane's next free slot (even lane: lo, odd lane: hi)
  int dir;     // +1 for the even lane, -1 for the odd lane
  int nslots;  // slots per query (a compile-time constant of the kernel)
  __device__ __forceinline__ int count() const { return hf ? nslots - 1 - fp : fp; }
  __device__ __forceinline__ int slot(int i) const { return hf ? nslots - 1 - i : i; }  // i-th own entry
};

// Keep only the k best candidates (score desc, index asc) of every query of the
// wave; returns the k-th best score (-inf if fewer than k).  Radix select on the
// order keys of the scores; ties at the cut are decided by the lowest indices
// with a second select on the index bits.  Entries move only inside their own
// lane's range (a lane reads slot i before writing slot <= i), so the
// compaction is done in place.  Every lane of the wave must call it.
__device__ float compact_slots(CandSlots& cs, int K, bool& cut) {
  const int c = cs.count();
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int cnt = 0;
    for (int i = 0; i < c; ++i) cnt += order_key(cs.buf[cs.slot(i) * 32 + cs.r].s) >= cand ? 1 : 0;
    cnt = sum_halves(cnt);
    if (cnt >= K) T = cand;
  }
  // entries strictly above the cut score, and those equal to it
  int gt = 0, eq = 0;
  for (int i = 0; i < c; ++i) {
    const uint32_t k = order_key(cs.buf[cs.slot(i) * 32 + cs.r].s);
    gt += k > T ? 1 : 0;
    eq += k == T ? 1 : 0;
  }
  gt = sum_halves(gt);
  eq = sum_halves(eq);
  // among the entries equal to the cut score keep the (K - gt) lowest indices:
  // J = the largest index kept (smallest J with #{equal, index <= J} >= K - gt)
  uint32_t J = 0xffffffffu;
  const bool straddle = gt < K && gt + eq > K;
  if (wave_any(straddle)) {
    uint32_t lowJ = 0;  // build the answer from the top bit: count(index < lowJ + bit) < need -> set bit
    for (int b = 31; b >= 0; --b) {
      const uint32_t probe = lowJ | (1u << b);
      int cnt = 0;
      for (int i = 0; i < c; ++i) {
        const Cand x = cs.buf[cs.slot(i) * 32 + cs.r];
        cnt += (order_key(x.s) == T && (uint32_t)x.j < probe) ? 1 : 0;
      }
      cnt = sum_halves(cnt);
      if (cnt < K - gt) lowJ = probe;
    }
    if (straddle) J = lowJ;
  }
  // squeeze the kept entries of this lane's range towards its end
  int w = 0;
  for (int i = 0; i < c; ++i) {
    const Cand x = cs.buf[cs.slot(i) * 32 + cs.r];
    const uint32_t k = order_key(x.s);
    if (k > T || (k == T && (uint32_t)x.j <= J)) {
      cs.buf[cs.slot(w) * 32 + cs.r] = x;
      ++w;
    }
  }
  cs.fp = cs.slot(w);
  cut = gt + eq >= K;
  return cut ? key_value(T) : -INFINITY;
}

// One workgroup: WAVES x 32 queries of one head against all M' keys.  Key
// tiles are staged in LDS, RSUB tiles of 32 keys at a time, and only
// S^T = K Q^T is formed.  Keys with score >= theta are
// appended to the query's LDS slots; when the slots run low, the query keeps
// only its current k best (so the slots never overflow) and from then on a key
// must beat the k-th best score strictly (an equal score loses: it has a
// higher index than every kept key).  At the end the candidates are ranked and
// the first k written, sorted.  Requires k <= kRefineMaxK.
// One LDS stage of RSUB key tiles: the waves test all RSUB tiles, meet at a
// barrier, store the next stage (loaded into registers during the tests) and
// meet again.  A wave's candidate work varies from tile to tile, and every
// wave waits for the slowest at a barrier; four tiles per test phase average
// that out better than two tiles per barrier with two stages (which LDS
// allows only up to two tiles: the candidate slots take 64 KB).
constexpr int RSUB = 4;
template <typename T, int WAVES, int SLOTS>
__global__ __launch_bounds__(WAVES * 64) void refine_kernel(RefineParams p) {
  constexpr int kRefineSlots = SLOTS;
  using TL = Tile<T>;
  using F = Frag32<T>;
  using Loader = TileLoader<T, WAVES * 64>;
  constexpr int KBYTES = TL::K_ELEMS * (int)sizeof(T);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // the stage buffer: RSUB key tiles, then the candidate slots
  auto tile_buf = [&](int j) { return reinterpret_cast<T*>(smem + j * KBYTES); };

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 31, hf = lane >> 5;
  CandSlots cs;
  cs.buf = reinterpret_cast<Cand*>(smem + RSUB * KBYTES) + wv * kRefineSlots * 32;
  cs.r = r;
  cs.hf = hf;
  cs.nslots = kRefineSlots;
  cs.fp = hf ? kRefineSlots - 1 : 0;
  cs.dir = hf ? -1 : 1;
  constexpr int QW = WAVES * 32;
  const int64_t n_qt = (p.n_q + QW - 1) / QW;
  const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t qt = w % n_qt;
  const int h = (int)(w / n_qt);
  const int64_t qrow = qt * QW + wv * 32 + r;
  const bool qvalid = qrow < p.n_q;
  const int64_t hoff = (int64_t)h * kHeadDim;
  const int Kk = p.topk;
  const T* K = static_cast<const T*>(p.k);
  typename F::Q qf = F::load_q(qvalid ? static_cast<const T*>(p.q) + qrow * p.row_stride + hoff : nullptr, hf);
  // a key is a candidate when its score is >= tlo: theta at first, then just
  // above the k-th best kept score (an equal score loses to the kept keys,
  // which all have lower indices)
  float tlo = kth_bound<kRefineGroups(SLOTS) / 2>(p, qrow, h, hf, qvalid);
  if (!qvalid) tlo = INFINITY;
  int ntot = 0;  // candidates held for this lane's query (both lanes)
  __builtin_amdgcn_s_waitcnt(0);
  // compare raw scores as integers when every threshold of the wave is
  // positive (order-preserving on the bit patterns then), else as floats;
  // thresholds only grow, so the choice stays valid
  const bool as_int = !wave_any(!(tlo > 0.0f));

  const int nk = (int)p.n_q;  // window counts are int32 (checked on the host)
  const int n_tiles = (nk + kKT - 1) / kKT, n_full = nk / kKT;
  const int n_steps = (n_tiles + RSUB - 1) / RSUB;
  auto tile_key = [&](int t) { return (t < n_tiles ? t : n_tiles - 1) * kKT; };
  ExclCursor excl;
  struct Stage {
    Loader l[RSUB];
  };
  auto stage_load = [&](Stage& st, int u) {
#pragma unroll
    for (int j = 0; j < RSUB; ++j) {
      const int key0 = tile_key(u * RSUB + j);
      st.l[j].load_k(K, p.row_stride, hoff, key0, min(nk - key0, kKT), tid);
    }
  };
  auto stage_store = [&](const Stage& st) {
#pragma unroll
    for (int j = 0; j < RSUB; ++j) st.l[j].store_k(tile_buf(j), tid);
  };
  Stage st;
  stage_load(st, 0);
  stage_store(st);
  stage_load(st, 1);
  lds_barrier();

  // The sweep, compiled once for integer and once for float comparisons.
  auto sweep = [&](auto int_tag) {
    constexpr bool AS_INT = decltype(int_tag)::value;
    // candidates of one 32-key tile t, from its scores s (S^T)
    auto tile = [&](int t, f32x16 s) {
      const int cur0 = t * kKT;
      if (t >= n_full) {
        const int lim = nk - cur0 - 4 * hf;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i / 4) + (i % 4) >= lim) s[i] = -INFINITY;
      }
      // a score passes when >= tlo (and is not -inf: keys past the end)
      const int tlo_bits = __float_as_int(tlo);
      auto pass = [&](float x) {
        if constexpr (AS_INT) return __float_as_int(x) >= tlo_bits;
        else return x >= tlo && x != -INFINITY;
      };
      // 4-key group maxima first (the exact per-key test follows)
      bool g[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if constexpr (AS_INT) {
          const int m = max(max(__float_as_int(s[4 * a]), __float_as_int(s[4 * a + 1])),
                            max(__float_as_int(s[4 * a + 2]), __float_as_int(s[4 * a + 3])));
          g[a] = m >= tlo_bits;
        } else {
          const float m = fmaxf(fmaxf(s[4 * a], s[4 * a + 1]), fmaxf(s[4 * a + 2], s[4 * a + 3]));
          g[a] = m >= tlo && m != -INFINITY;
        }
      }
      if (!wave_any(g[0] || g[1] || g[2] || g[3])) return;
      // groups with a passing key in some lane of the wave (uniform)
      const unsigned gany = (wave_any(g[0]) ? 1u : 0u) | (wave_any(g[1]) ? 2u : 0u) |
                            (wave_any(g[2]) ? 4u : 0u) | (wave_any(g[3]) ? 8u : 0u);
      // excluded keys of the tile, as this lane's bits (bit 4a+e = key 8a+4hf+e)
      unsigned ex = 0;
      if (p.n_excl) {
        const uint32_t em = excl.mask(p, cur0);
#pragma unroll
        for (int a = 0; a < 4; ++a) ex |= ((em >> (8 * a + 4 * hf)) & 15u) << (4 * a);
      }
      auto key_of = [&](int a, int e) { return (int)(cur0 + 8 * a + 4 * hf + e); };
      // exact tests of group a: bit e = key 8a+4hf+e is a candidate
      auto group_keep = [&](int a) {
        unsigned gm = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) gm |= (pass(s[4 * a + e]) ? 1u : 0u) << e;
        return gm & ~(ex >> (4 * a)) & 15u;
      };
      // Whole group: every lane writes the group's 4 keys, its kept keys
      // compacted at its fill pointer and the others at pointer + e.  A kept
      // key's slot is at most its own e, so a later kept key may overwrite an
      // earlier dropped one but never the reverse; the dropped keys land in
      // free slots (needs >= 8 free, so the two ends never meet).
      auto append_group = [&](int a, unsigned gm) {
        int kb = 0;  // kept keys of the group so far
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool kept = (gm >> e) & 1u;
          cs.buf[(cs.fp + cs.dir * (kept ? kb : e)) * 32 + r] = Cand{s[4 * a + e], key_of(a, e)};
          kb += kept ? 1 : 0;
        }
        cs.fp += cs.dir * kb;
      };
      // a passing group adds at most 8 candidates to a query (4 per lane)
      if (!wave_any(ntot + 8 * __builtin_popcount(gany) + 8 > kRefineSlots)) {
        // common case: room for whole groups, test and append in one pass
        int need = 0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          if ((gany >> a) & 1u) {
            const unsigned gm = group_keep(a);
            append_group(a, gm);
            need += __builtin_popcount(gm);
          }
        }
        ntot += sum_halves(need);  // outside any condition: every lane takes part
        return;
      }
      // slots running low: one group at a time, keeping the k best first when
      // the group might not fit (a group adds at most 8; k + 8 + 8 <= slots)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if ((gany >> a) & 1u) {
          unsigned gm = group_keep(a);
          int need = sum_halves(__builtin_popcount(gm));  // the query's new candidates
          if (wave_any(ntot + need + 8 > kRefineSlots)) {
            bool cut;
            const float kth = compact_slots(cs, Kk, cut);
            if (cut) {
              tlo = next_up(kth);
              ntot = Kk;
            }
            gm = group_keep(a);
            need = sum_halves(__builtin_popcount(gm));
          }
          append_group(a, gm);
          ntot += need;
        }
      }
    };

    // stage u: scores two tiles at a time (the second tile's matrix-core
    // work runs while the first is tested), then the stage swap
    for (int u = 0; u < n_steps; ++u) {
#pragma unroll
      for (int j = 0; j < RSUB; j += 2) {
        const f32x16 s0 = F::qk(tile_buf(j), r, hf, qf);
        const f32x16 s1 = F::qk(tile_buf(j + 1), r, hf, qf);
        tile(u * RSUB + j, s0);
        tile(u * RSUB + j + 1, s1);
      }
      lds_barrier();
      stage_store(st);
      stage_load(st, u + 2);
      lds_barrier();
    }
  };
  if (as_int)
    sweep(std::integral_constant<bool, true>{});
  else
    sweep(std::integral_constant<bool, false>{});

  // rank this lane's candidates against all of the query's and write the first k
  const int c_me = cs.count(), c_ot = xor_lane(c_me, 32);
  const int n = c_me + c_ot;
  if (qvalid) {
    int32_t* di = p.topk_idx + (qrow * p.n_heads + h) * Kk;
    float* ds = p.topk_score ? p.topk_score + (qrow * p.n_heads + h) * Kk : nullptr;
    const int lo0 = hf ? c_ot : c_me;  // the even lane's entries are slots [0, lo0)
    for (int i0 = 0; i0 < c_me; i0 += 16) {
      Cand x[16];
      int rk[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        x[j] = i0 + j < c_me ? cs.buf[cs.slot(i0 + j) * 32 + r] : Cand{-INFINITY, 0x7fffffff};
        rk[j] = 0;
      }
      for (int y = 0; y < n; ++y) {
        const int sl = y < lo0 ? y : kRefineSlots - 1 - (y - lo0);
        const Cand cy = cs.buf[sl * 32 + r];
#pragma unroll
        for (int j = 0; j < 16; ++j) rk[j] += cand_better(cy, x[j]) ? 1 : 0;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (i0 + j < c_me && rk[j] < Kk) {
          di[rk[j]] = x[j].j;
          if (ds) ds[rk[j]] = x[j].s;
        }
      }
    }
    for (int t = n + hf; t < Kk; t += 2) {
      di[t] = -1;
      if (ds) ds[t] = -INFINITY;
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

template <typename T, int SLOTS>
static hipError_t launch_refine_s(const RefineParams& p, hipStream_t stream) {
  constexpr int WAVES = 4;
  const int64_t blocks = (p.n_q + WAVES * 32 - 1) / (WAVES * 32) * p.n_heads;
  if (blocks == 0) return hipSuccess;
  const size_t lds = RSUB * (size_t)Tile<T>::K_ELEMS * sizeof(T) + (size_t)WAVES * SLOTS * 32 * sizeof(Cand);
  const void* fn = reinterpret_cast<const void*>(&refine_kernel<T, WAVES, SLOTS>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((refine_kernel<T, WAVES, SLOTS>), dim3((unsigned)blocks), dim3(WAVES * 64), lds, stream, p);
  return hipGetLastError();
}
template <typename T>
static hipError_t launch_refine_t(const RefineParams& p, hipStream_t stream) {
  if (p.topk <= kRefineSlotsSmall - 16) return launch_refine_s<T, kRefineSlotsSmall>(p, stream);
  return launch_refine_s<T, kRefineSlotsLarge>(p, stream);
}

hipError_t launch_refine(int dtype, const RefineParams& p, hipStream_t stream) {
  return dtype == kBF16 ? launch_refine_t<__bf16>(p, stream) : launch_refine_t<float>(p, stream);
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
