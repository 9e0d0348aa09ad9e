// Exact top-k of the compressed branch (Paper-Notes page "Speed3R: Sparse
// Feed-forward 3D Reconstruction Models", section "选择分支": TopKSelect over
// the guide scores S_guide = Q_comp K_comp^T of section "压缩分支"; section
// "高效 Triton Kernel 实现": the score matrix is never stored).
//
// Input: the lower bounds that the compressed-attention sweep
// (flash_kernel<kFlashBound>) leaves per (head, group of key tiles, query),
// and per query a bound E on how far a group's best score can lie above its
// stored bound.  Every score below is the raw score of the same four
// v_mfma_f32_32x32x16 steps (Frag32::qk) the sweep used, so it equals the
// sweep's score bit for bit.
//
//  threshold_kernel  theta = the k-th largest group bound.  The k groups
//                    behind it each hold a distinct key scoring >= theta, so
//                    the k-th best score is >= theta and every top-k key
//                    scores >= theta.  A group can hold such a key only if its
//                    bound is >= theta - E: those groups are the query's hot
//                    groups (about k of them), kept as a bit mask.
//  hot_group_kernel  one workgroup per (head, group, query chunk) holds the
//                    group's key tiles in LDS; each wave scans the chunk's
//                    queries for those the group is hot for, gathers their
//                    rows 32 at a time and scores them against the group, and
//                    appends keys >= theta to the query's candidate list (one
//                    atomic per lane that has any, so list order varies from
//                    run to run, list contents do not).
//  rank_kernel       ranks each list under (score desc, key asc) -- a total
//                    order, so the sorted top-k is deterministic.
//  refine_kernel     fallback for query tiles holding a query whose list would
//                    overflow (or whose theta is -inf: fewer than k finite
//                    bounds, e.g. k beyond the candidate count): the full
//                    score-only sweep of every key, compacting to the k best
//                    whenever the LDS slots run low, exact for any input.
#include <math.h>

#include "flash_frag.h"
#include "gsa_device.h"
#include "gsa_kernels.h"

namespace gsa {

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

struct Cand {
  float s;
  int j;
};

// x + (x of the lane with index ^1 / ^2 in its group of four), by DPP.
__device__ __forceinline__ int quad_xor1(int x) { return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int quad_xor2(int x) { return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); }

// ---- theta and the hot groups ------------------------------------------------------
// Four lanes per (head, query); lane li holds groups [li * VPL, li * VPL + VPL)
// as order keys (groups past n_groups as key 0, below every real key).  Radix
// select of the k-th largest key, bit by bit from the top, counts summed over
// the four lanes.  Hot: bound >= fl(theta - E) (the key one step below the
// threshold's, so -0 and +0 compare as equal floats do).
template <int VPL>
__global__ __launch_bounds__(256) void threshold_kernel(TopkParams p) {
  const int li = threadIdx.x & 3;
  const int64_t n_qh = (int64_t)p.n_heads * p.n_q;
  const int64_t qh0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 2;
  const bool valid = qh0 < n_qh;
  const int64_t qh = valid ? qh0 : n_qh - 1;
  const int64_t h = qh / p.n_q, q = qh - h * p.n_q;
  const int NG = p.n_groups;
  const float* src = p.gbound + h * NG * p.n_q + q;
  const int g0 = li * VPL;
  // The keys' top 31 bits (the lowest dropped): the difference of two such
  // keys is negative exactly when the first is below, so a count is the sign
  // bits shifted into a mask (one v_alignbit per key) and a popcount per 32
  // keys.  theta may then come out one key step low, still a lower bound of
  // the k-th largest bound (which only admits candidates), and the hot test
  // below, at the same resolution, keeps a superset of the groups.
  uint32_t kv[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int g = min(g0 + i, NG - 1);  // clamped, unconditional loads
    const uint32_t x = order_key(src[(int64_t)g * p.n_q]);
    kv[i] = (g0 + i < NG ? x : 0u) >> 1;
  }
  uint32_t T = 0;
  for (int b = 30; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int below = 0;
#pragma unroll
    for (int w = 0; w < VPL / 32; ++w) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) m = __builtin_amdgcn_alignbit(m, kv[32 * w + i] - cand, 31);
      below += __builtin_popcount(m);
    }
    int cnt = VPL - below;
    cnt += quad_xor1(cnt);
    cnt += quad_xor2(cnt);
    if (cnt >= p.topk) T = cand;
  }
  const uint32_t k_ninf = order_key(-INFINITY);
  const bool fin = (T << 1) > k_ninf;
  const float theta = fin ? key_value(T << 1) : -INFINITY;
  const uint32_t thr = fin ? (order_key(theta - p.gerr[qh]) - 1u) >> 1 : 0x7fffffffu;
  if (valid) {
#pragma unroll
    for (int w = 0; w < VPL / 32; ++w) {
      const int word = g0 / 32 + w;
      if (word < p.n_words) {
        uint32_t bits = 0;
#pragma unroll
        for (int b = 0; b < 32; ++b)
          bits |= (kv[32 * w + b] >= thr && kv[32 * w + b] > (k_ninf >> 1) ? 1u : 0u) << b;
        p.hot[(h * p.n_words + word) * p.n_q + q] = bits;
      }
    }
    if (li == 0) {
      p.theta[qh] = theta;
      p.cnt[qh] = fin ? 0 : p.cap + 1;
    }
  }
}

// ---- candidates from the hot groups ---------------------------------------------------
// LDS: the group's key tiles (at most kHotTiles<T> at a time), then per wave a
// 16-float slab per lane (the scores of a tile with candidates, read back by
// index) and a ring of 128 query ids.  A wave scans its share of the chunk 256
// queries at a time (four coalesced loads of hot words per lane), appends the
// hot ones to its ring and scores 32 of them at a time: lane (r, hf) holds
// ring query r and, per tile, keys 8(i/4) + 4hf + i%4 in element i.
template <typename T>
constexpr int kHotTiles = sizeof(T) == 2 ? 16 : 8;
constexpr int kHotRing = 128;

template <typename T>
__device__ __forceinline__ int k_chunk_elem(int row, int c) {
  if constexpr (sizeof(T) == 2) return Tile<T>::chunk(row, c);
  else return row * Tile<T>::KSTRIDE + c * Tile<T>::VE;
}

template <typename T, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void hot_group_kernel(TopkParams p) {
  using TL = Tile<T>;
  using F = Frag32<T>;
  constexpr int KBYTES = TL::K_ELEMS * (int)sizeof(T);
  constexpr int VPR = kHeadDim / TL::VE;  // 16-byte chunks per key row
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 31, hf = lane >> 5;
  const int NG = p.n_groups;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int g = (int)(wid % NG);
  const int64_t hc = wid / NG;
  const int chunk = (int)(hc % p.n_chunks);
  const int h = (int)(hc / p.n_chunks);
  const int nk = (int)p.n_q;  // window counts are int32 (checked on the host)
  const int n_tiles = (nk + kKT - 1) / kKT, n_full = nk / kKT;
  const int gt0 = g * p.group_tiles, gt1 = min(gt0 + p.group_tiles, n_tiles);
  const int64_t hoff = (int64_t)h * kHeadDim;
  const T* K = static_cast<const T*>(p.k);
  const T* Q = static_cast<const T*>(p.q);

  const int sub_max = min(p.group_tiles, kHotTiles<T>);
  float* stash = reinterpret_cast<float*>(smem + sub_max * KBYTES) + (wv * 64 + lane) * 16;
  int* ring = reinterpret_cast<int*>(smem + sub_max * KBYTES + WAVES * 64 * 16 * 4) + wv * kHotRing;

  // this wave's queries: a contiguous share of the chunk
  const int64_t c0 = p.n_q * chunk / p.n_chunks, c1 = p.n_q * (chunk + 1) / p.n_chunks;
  const int64_t w0 = c0 + (c1 - c0) * wv / WAVES, w1 = c0 + (c1 - c0) * (wv + 1) / WAVES;
  const uint32_t* hot = p.hot + ((int64_t)h * p.n_words + g / 32) * p.n_q;
  const uint32_t gbit = 1u << (g & 31);
  const int64_t hq = (int64_t)h * p.n_q;

  for (int s0 = gt0; s0 < gt1; s0 += sub_max) {
    const int s1 = min(s0 + sub_max, gt1), nt = s1 - s0;
    // stage the tiles (rows past the last key as zeros; their scores are masked)
    if (s0 != gt0) __syncthreads();  // every wave is done with the previous tiles
    for (int c = tid; c < nt * kKT * VPR; c += WAVES * 64) {
      const int t = c / (kKT * VPR), row = (c / VPR) % kKT, ch = c % VPR;
      const int key = (s0 + t) * kKT + row;
      const uint4 x = key < nk ? ld16(K + (int64_t)key * p.row_stride + hoff + ch * TL::VE) : make_uint4(0, 0, 0, 0);
      st16(reinterpret_cast<T*>(smem + t * KBYTES) + k_chunk_elem<T>(row, ch), x);
    }
    __syncthreads();

    // score ring entries [head, head + n) (n <= 32) against the staged tiles
    auto batch = [&](uint32_t head, int n) {
      const int qi = r < n ? ring[(head + r) & (kHotRing - 1)] : -1;
      const typename F::Q qf = F::load_q(qi >= 0 ? Q + (int64_t)qi * p.row_stride + hoff : nullptr, hf);
      const int64_t qh = hq + (qi >= 0 ? qi : 0);
      const float th = qi >= 0 ? p.theta[qh] : INFINITY;
      // Up to four candidates per lane wait in registers; list slots are
      // taken with one atomic per four (or at the end of the batch), not per
      // tile, so the atomic's round trip is rarely on the tile loop's path.
      uint2 pend0 = {}, pend1 = {}, pend2 = {}, pend3 = {};
      int np = 0;
      auto flush = [&]() __attribute__((always_inline)) {
        if (np > 0) {
          const int slot = atomicAdd(p.cnt + qh, np);
          uint2* dst = p.cand + qh * p.cap;
          if (slot < p.cap) dst[slot] = pend0;
          if (np > 1 && slot + 1 < p.cap) dst[slot + 1] = pend1;
          if (np > 2 && slot + 2 < p.cap) dst[slot + 2] = pend2;
          if (np > 3 && slot + 3 < p.cap) dst[slot + 3] = pend3;
          np = 0;
        }
      };
      ExclCursor excl;
      for (int t = 0; t < nt; ++t) {
        f32x16 s = F::qk(reinterpret_cast<const T*>(smem + t * KBYTES), r, hf, qf);
        const int key0 = (s0 + t) * kKT;
        if (s0 + t >= n_full) {
          const int lim = nk - key0 - 4 * hf;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (8 * (i / 4) + (i % 4) >= lim) s[i] = -INFINITY;
        }
        // bit i: s[i] >= th, i.e. the sign bit of s[i] - th clear (th is finite
        // for a hot query, +inf for an empty lane; masked keys are -inf), shifted
        // in from the top with one v_alignbit per key
        uint32_t m = 0;
#pragma unroll
        for (int i = 15; i >= 0; --i) m = __builtin_amdgcn_alignbit(m, __float_as_uint(s[i] - th), 31);
        m = ~m & 0xffffu;
        if (p.n_excl) {
          const uint32_t em = excl.mask(p, key0);
#pragma unroll
          for (int a = 0; a < 4; ++a) m &= ~(((em >> (8 * a + 4 * hf)) & 15u) << (4 * a));
        }
        if (wave_any(m != 0)) {
          if (m != 0) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
              *reinterpret_cast<f32x4*>(stash + 4 * a) = f32x4{s[4 * a], s[4 * a + 1], s[4 * a + 2], s[4 * a + 3]};
            while (m != 0) {
              const int i = __builtin_ctz(m);
              m &= m - 1;
              if (np == 4) flush();
              const uint2 e = make_uint2(__float_as_uint(stash[i]), (uint32_t)(key0 + 8 * (i >> 2) + 4 * hf + (i & 3)));
              pend0 = np == 0 ? e : pend0;
              pend1 = np == 1 ? e : pend1;
              pend2 = np == 2 ? e : pend2;
              pend3 = np == 3 ? e : pend3;
              ++np;
            }
          }
        }
      }
      flush();
    };

    uint32_t head = 0, tail = 0;  // wave-uniform ring positions
    for (int64_t qb = w0; qb < w1; qb += 256) {
      uint32_t x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t q = qb + 64 * u + lane;
        x[u] = hot[q < w1 ? q : w1 - 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t q = qb + 64 * u + lane;
        const bool is_hot = q < w1 && (x[u] & gbit) != 0;
        const uint64_t mask = __builtin_amdgcn_ballot_w64(is_hot);
        if (is_hot) {
          const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
          ring[(tail + below) & (kHotRing - 1)] = (int)q;
        }
        tail += (uint32_t)__builtin_popcountll(mask);
        while (tail - head >= 32) {
          batch(head, 32);
          head += 32;
        }
      }
    }
    if (tail != head) batch(head, (int)(tail - head));
  }
}

// ---- ranking -------------------------------------------------------------------------
// One wave per (head, query): the list goes to LDS, each lane ranks its
// entries against all of them and writes those that rank below k.
__global__ __launch_bounds__(256) void rank_kernel(TopkParams p) {
  __shared__ uint2 buf[4][2 * kTopkMaxK + 64];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t qh = (int64_t)blockIdx.x * 4 + wv;
  if (qh >= (int64_t)p.n_heads * p.n_q) return;
  const int n = p.cnt[qh];
  if (n > p.cap) return;  // refine_kernel writes this query
  const uint2* src = p.cand + qh * p.cap;
  for (int i = lane; i < n; i += 64) buf[wv][i] = src[i];
  const int64_t h = qh / p.n_q, q = qh - h * p.n_q;
  const int K = p.topk;
  int32_t* di = p.topk_idx + (q * p.n_heads + h) * K;
  float* ds = p.topk_score ? p.topk_score + (q * p.n_heads + h) * K : nullptr;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const uint2 xe = buf[wv][i < n ? i : 0];
    const Cand x{__uint_as_float(xe.x), (int)xe.y};
    int rk = 0;
    for (int j = 0; j < n; ++j) {
      const uint2 ye = buf[wv][j];
      const float ys = __uint_as_float(ye.x);
      rk += (ys > x.s || (ys == x.s && (int)ye.y < x.j)) ? 1 : 0;
    }
    if (i < n && rk < K) {
      di[rk] = x.j;
      if (ds) ds[rk] = x.s;
    }
  }
  for (int t = n + lane; t < K; t += 64) {
    di[t] = -1;
    if (ds) ds[t] = -INFINITY;
  }
}

// ---- fallback: the full score-only sweep ---------------------------------------------
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
// the first k written, sorted.  Requires k <= kTopkMaxK.
// One LDS stage of RSUB key tiles: the waves test all RSUB tiles, meet at a
// barrier, store the next stage (loaded into registers during the tests) and
// meet again.  A wave's candidate work varies from tile to tile, and every
// wave waits for the slowest at a barrier; four tiles per test phase average
// that out better than two tiles per barrier with two stages (which LDS
// allows only up to two tiles: the candidate slots take 64 KB).
constexpr int RSUB = 4;
template <typename T, int WAVES, int SLOTS>
__global__ __launch_bounds__(WAVES * 64) void refine_kernel(TopkParams p) {
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
  // Only query tiles holding a query whose candidate list overflowed (or whose
  // theta is -inf) are swept; the others leave at once, all waves together.
  // (the flags borrow the first bytes of the LDS before the first tile is stored)
  {
    int* any_overflow = reinterpret_cast<int*>(smem);
    const bool mine = qvalid && p.cnt[(int64_t)h * p.n_q + qrow] > p.cap;
    const bool wave_has = wave_any(mine);
    if (lane == 0) any_overflow[wv] = wave_has ? 1 : 0;
    __syncthreads();
    int n_over = 0;
#pragma unroll
    for (int i = 0; i < WAVES; ++i) n_over += any_overflow[i];
    __syncthreads();
    if (n_over == 0) return;
  }
  const T* K = static_cast<const T*>(p.k);
  typename F::Q qf = F::load_q(qvalid ? static_cast<const T*>(p.q) + qrow * p.row_stride + hoff : nullptr, hf);
  // a key is a candidate when its score is >= tlo: theta at first, then just
  // above the k-th best kept score (an equal score loses to the kept keys,
  // which all have lower indices)
  float tlo = qvalid ? p.theta[(int64_t)h * p.n_q + qrow] : INFINITY;
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

template <typename T, int WAVES, int SLOTS>
static hipError_t launch_refine_s(const TopkParams& p, hipStream_t stream) {
  constexpr size_t lds = RSUB * (size_t)Tile<T>::K_ELEMS * sizeof(T) + (size_t)WAVES * SLOTS * 32 * sizeof(Cand);
  static_assert(lds <= 160 * 1024, "refine_kernel: LDS of a gfx950 CU exceeded");
  const int64_t blocks = (p.n_q + WAVES * 32 - 1) / (WAVES * 32) * p.n_heads;
  if (blocks == 0) return hipSuccess;
  const void* fn = reinterpret_cast<const void*>(&refine_kernel<T, WAVES, SLOTS>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((refine_kernel<T, WAVES, SLOTS>), dim3((unsigned)blocks), dim3(WAVES * 64), lds, stream, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_topk_t(const TopkParams& p, hipStream_t stream) {
  const int64_t n_qh = (int64_t)p.n_heads * p.n_q;
  if (n_qh == 0) return hipSuccess;
  if (p.n_groups < 1 || p.n_groups > kTopkMaxGroups || p.topk < 1 || p.topk > kTopkMaxK || p.cap < 2 * p.topk ||
      p.cap > 2 * kTopkMaxK + 64 || p.n_words != (p.n_groups + 31) / 32 || p.n_chunks < 1)
    return hipErrorInvalidValue;
  // 1. theta, hot masks, list counters
  const unsigned tblocks = (unsigned)((n_qh * 4 + 255) / 256);
  const int vpl = (p.n_groups + 3) / 4;
  if (vpl <= 32)
    hipLaunchKernelGGL(threshold_kernel<32>, dim3(tblocks), dim3(256), 0, stream, p);
  else if (vpl <= 64)
    hipLaunchKernelGGL(threshold_kernel<64>, dim3(tblocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(threshold_kernel<128>, dim3(tblocks), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. candidates from the hot groups
  {
    constexpr int WAVES = 8;
    const int sub = p.group_tiles < kHotTiles<T> ? p.group_tiles : kHotTiles<T>;
    const size_t lds = (size_t)sub * Tile<T>::K_ELEMS * sizeof(T) + (size_t)WAVES * (64 * 16 * 4 + kHotRing * 4);
    const int64_t blocks = (int64_t)p.n_heads * p.n_chunks * p.n_groups;
    if (blocks > 0xffffffffLL) return hipErrorInvalidValue;
    const void* fn = reinterpret_cast<const void*>(&hot_group_kernel<T, WAVES>);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((hot_group_kernel<T, WAVES>), dim3((unsigned)blocks), dim3(WAVES * 64), lds, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 3. ranking
  hipLaunchKernelGGL(rank_kernel, dim3((unsigned)((n_qh + 3) / 4)), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 4. fallback sweep of the tiles with an overflowed list
  if (p.topk <= kRefineSlotsSmall - 16) return launch_refine_s<T, 4, kRefineSlotsSmall>(p, stream);
  // fp32 tiles are twice as large: two waves per workgroup keep the slots within the LDS
  if constexpr (sizeof(T) == 4) return launch_refine_s<T, 2, kRefineSlotsLarge>(p, stream);
  else return launch_refine_s<T, 4, kRefineSlotsLarge>(p, stream);
}

hipError_t launch_topk(int dtype, const TopkParams& p, hipStream_t stream) {
  return dtype == kBF16 ? launch_topk_t<__bf16>(p, stream) : launch_topk_t<float>(p, stream);
}

}  // namespace gsa
