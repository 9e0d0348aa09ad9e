// Backward of the GSA layer on the gfx950 matrix cores: the gradients of q, k,
// v and W_g given the output gradient dO, with the top-k window sets of the
// forward held fixed (GSA is trained end to end by distillation: Paper-Notes
// page "Speed3R: Sparse Feed-forward 3D Reconstruction Models", sections
// "研究背景与动机" and "训练策略").
//
// Every attention branch uses the softmax backward with the forward's log2
// denominators L2 (P = exp2(c s - L2), c = scale log2 e) and D = dO . O:
//   dP = dO . v,  dS = P (dP - D),  dq = scale sum dS k,  dk = scale sum dS q,
//   dv = sum P dO.
// Kernels:
//  * flash_bwd_kernel   dense branches (special tokens over all tokens, the
//                       compressed windows over all windows, image queries
//                       over the context frames): one kernel for the query
//                       side (dQ) and one for the key side (dK, dV), both on
//                       the 32x32 fragments of the forward flash kernel;
//  * gate_bwd_kernel    the gate and the split of dO into the selection and
//                       compressed branches, one wave per (window, head);
//  * sel_dq_kernel / sel_dkdv_kernel   the selection branch, gathering whole
//                       windows from blocked copies: the query side walks a
//                       window's top-k list, the key side walks the inverse
//                       list (the query windows that selected it); bf16 chunks
//                       are transposed in LDS, fp32 ones gathered twice;
//  * inverse-index, reduction and dW_g kernels.  The pooling backward (each
//    window token gets its pooled row's gradient / s^2) is folded into the
//    selection kernels' stores, which touch the same token rows.
// All sums run in a fixed order, so the gradients are deterministic.
#include <math.h>

#include <algorithm>

#include "flash_frag.h"
#include "gsa_device.h"
#include "gsa_kernels.h"
#include "select_frag.h"

namespace gsa {

// ---- 32x32 fragments: P / dS as the contraction operand ----------------------
template <typename T>
struct BwdOp;
template <>
struct BwdOp<__bf16> {
  __device__ static Frag32<__bf16>::P make(const f32x16& x) {
    Frag32<__bf16>::P r;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) r.v[m][e] = (__bf16)x[8 * m + e];
    return r;
  }
};
template <>
struct BwdOp<float> {
  __device__ static Frag32<float>::P make(const f32x16& x) { return Frag32<float>::P{x}; }
};

// ---- tile staging of the backward flash kernels ------------------------------
// Two 32-row operands A and B per tile (dQ side: K and V of a key range; key
// side: Q and dO of 32 queries, rows gathered through the query map).  bf16
// tiles are stored in the swizzled row layout only (the transposing reads of
// the pv fragment serve both products); fp32 tiles also get a transposed copy.
template <typename T, int NT>
struct BwdStage {
  using TL = Tile<T>;
  static constexpr int VE = TL::VE;
  static constexpr int VPR = kHeadDim / VE;
  static constexpr int NV = kKT * VPR / NT;
  static_assert(NV >= 1 && NV * NT == kKT * VPR, "tile must split evenly over the workgroup");
  uint4 a[NV], b[NV];
  float l2v, ddv;

  static __device__ uint4 buf16(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
  // rows row0 .. row0 + 31 (rows from `valid` on read as zeros)
  __device__ void load_range(const T* A, const T* B, int64_t stride, int64_t hoff, int64_t row0, int valid,
                             int tid) {
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc(A, stride, hoff, row0, valid);
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc(B, stride, hoff, row0, valid);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + i * NT, row = idx / VPR, c = idx % VPR;
      const int off = (int)(((int64_t)row * stride + c * VE) * (int64_t)sizeof(T));
      a[i] = buf16(ra, off);
      b[i] = buf16(rb, off);
    }
  }
  // queries r0 .. r0 + 31 (r < n_q): Q rows through the query map, dO rows
  // through the map or by index, and their L2 / D
  __device__ void load_queries(const FlashBwdParams& p, int64_t hoff, int h, int64_t r0, int tid) {
    const T* Q = static_cast<const T*>(p.q);
    const T* G = static_cast<const T*>(p.d_o);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + i * NT, row = idx / VPR, c = idx % VPR;
      const int64_t r = r0 + row;
      if (r < p.n_q) {
        // query rows and the map's period are below 2^31 (checked on the host):
        // 32-bit division instead of the long 64-bit sequence, once per tile
        const uint32_t ru = (uint32_t)r, qa = (uint32_t)p.qa, fr = ru / qa;
        const int64_t tok = (int64_t)fr * p.qb + p.qc + (ru - fr * qa);
        const int64_t gtok = p.do_mapped ? tok : r;
        a[i] = ld16(Q + tok * p.row_stride + hoff + c * VE);
        b[i] = ld16(G + gtok * p.row_stride + hoff + c * VE);
      } else {
        a[i] = make_uint4(0, 0, 0, 0);
        b[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < kKT) {
      const int64_t r = r0 + tid;
      l2v = r < p.n_q ? p.lse[r * p.n_heads + h] * p.lse_mul : INFINITY;
      ddv = r < p.n_q ? p.dd[r * p.n_heads + h] : 0.0f;
    }
  }
  __device__ void store(T* a_rows, T* a_tr, T* b_rows, T* b_tr, float* l2s, float* dds, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + i * NT, row = idx / VPR, c = idx % VPR;
      if constexpr (sizeof(T) == 2) {
        st16(a_rows + TL::chunk(row, c), a[i]);
        st16(b_rows + TL::chunk(row, c), b[i]);
      } else {
        st16(a_rows + row * TL::KSTRIDE + c * VE, a[i]);
        st16(b_rows + row * TL::KSTRIDE + c * VE, b[i]);
        const T* xa = reinterpret_cast<const T*>(&a[i]);
        const T* xb = reinterpret_cast<const T*>(&b[i]);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          if (a_tr) a_tr[(c * VE + e) * TL::VSTRIDE + row] = xa[e];
          if (b_tr) b_tr[(c * VE + e) * TL::VSTRIDE + row] = xb[e];
        }
      }
    }
    if (l2s && tid < kKT) {
      l2s[tid] = l2v;
      dds[tid] = ddv;
    }
  }
};

template <typename T>
struct BwdLds {
  using TL = Tile<T>;
  static constexpr int A_EL = TL::K_ELEMS;
  static constexpr int T_EL = sizeof(T) == 2 ? 0 : TL::V_ELEMS;
  static constexpr int STAGE_BYTES = 2 * (A_EL + T_EL) * (int)sizeof(T) + 2 * kKT * 4;
  T *a_rows, *a_tr, *b_rows, *b_tr;
  float *l2s, *dds;
  __device__ BwdLds(char* base) {
    a_rows = reinterpret_cast<T*>(base);
    a_tr = sizeof(T) == 2 ? a_rows : a_rows + A_EL;
    b_rows = a_rows + A_EL + T_EL;
    b_tr = sizeof(T) == 2 ? b_rows : b_rows + A_EL;
    l2s = reinterpret_cast<float*>(base + 2 * (A_EL + T_EL) * sizeof(T));
    dds = l2s + kKT;
  }
};

// bf16 dQ pass: a ring of three (K, V) tile buffers fed by global-to-LDS
// loads, as in the forward flash kernel (separate arrays, so the compiler can
// tell which buffer a load writes).
__shared__ __attribute__((aligned(16))) __bf16 bq_ring0[kKT * kHeadDim * 2];
__shared__ __attribute__((aligned(16))) __bf16 bq_ring1[kKT * kHeadDim * 2];
__shared__ __attribute__((aligned(16))) __bf16 bq_ring2[kKT * kHeadDim * 2];

// bf16 key-side pass: the same ring over (Q, dO) query tiles, and beside
// each buffer every wave's own copy of the tile's L2 and D values (64 floats
// each, of which the tile uses the first 32).  Every buffer is an array of
// its own: the compiler then knows that reading one does not wait for the
// loads still filling another.
constexpr int kBkvQT = 2;                         // 32-query sub-tiles per ring tile
constexpr int kBkvTQ = kBkvQT * kKT;               // query rows per ring tile
constexpr int kBkvQdoElems = kBkvTQ * kHeadDim * 2;  // Q rows, then dO rows
constexpr int kBkvRowVals = 64;                   // L2 / D values one wave loads (>= kBkvTQ)
constexpr int kBkvVals = 2 * 4 * kBkvRowVals;     // L2 of 4 waves, then D of 4 waves
__shared__ __attribute__((aligned(16))) __bf16 bk_ring0[kBkvQdoElems];
__shared__ __attribute__((aligned(16))) __bf16 bk_ring1[kBkvQdoElems];
__shared__ __attribute__((aligned(16))) __bf16 bk_ring2[kBkvQdoElems];
__shared__ __attribute__((aligned(16))) float bk_vals0[kBkvVals];
__shared__ __attribute__((aligned(16))) float bk_vals1[kBkvVals];
__shared__ __attribute__((aligned(16))) float bk_vals2[kBkvVals];

__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t rs, void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

template <typename T, int WAVES, int KIND>
__global__ __launch_bounds__(WAVES * 64) void flash_bwd_kernel(FlashBwdParams p) {
  using F = Frag32<T>;
  using L = BwdLds<T>;
  constexpr int NT = WAVES * 64;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 31, hf = lane >> 5;
  const float c = p.scale_log2;
  const int64_t H = p.n_heads;
  const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
  // LDS stage i % 2 (pointers computed, not indexed, so nothing spills)
  auto buf = [&](int64_t i) __attribute__((always_inline)) { return L(smem + (i & 1) * L::STAGE_BYTES); };
  BwdStage<T, NT> st;

  if constexpr (KIND == kBwdDQ) {
    const int64_t n_qt = (p.n_q + NT / 2 - 1) / (NT / 2);
    const int64_t qt = w % n_qt, hs = w / n_qt;
    const int h = (int)(hs % H);
    const int split = (int)(hs / H);
    const int64_t hoff = (int64_t)h * kHeadDim;
    const int64_t qrow = qt * (NT / 2) + wv * 32 + r;
    const bool qvalid = qrow < p.n_q;
    const int64_t qtok = (qrow / p.qa) * p.qb + p.qc + qrow % p.qa;
    const int64_t gtok = p.do_mapped ? qtok : qrow;
    const typename F::Q qf = F::load_q(qvalid ? static_cast<const T*>(p.q) + qtok * p.row_stride + hoff : nullptr, hf);
    const typename F::Q gf = F::load_q(qvalid ? static_cast<const T*>(p.d_o) + gtok * p.row_stride + hoff : nullptr, hf);
    const float L2 = qvalid ? p.lse[qrow * H + h] * p.lse_mul : INFINITY;
    const float D = qvalid ? p.dd[qrow * H + h] : 0.0f;
    const T* K = static_cast<const T*>(p.k);
    const T* V = static_cast<const T*>(p.v);
    const int64_t kb = p.kbeg[split];
    const int nk = (int)(p.kend[split] - kb);
    const int n_tiles = (nk + kKT - 1) / kKT, n_full = nk / kKT;
    f32x16 acc[2] = {{}, {}};
    // one 32-key tile: dS = P (dO . v - D), acc^T += K^T dS^T
    auto tile_dq = [&](int t, const T* kt, const T* vt) __attribute__((always_inline)) {
      f32x16 s = F::qk(kt, r, hf, qf);
      if (t >= n_full) {
        const int lim = nk - t * kKT - 4 * hf;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i / 4) + (i % 4) >= lim) s[i] = -INFINITY;
      }
      f32x16 pm;
#pragma unroll
      for (int i = 0; i < 16; ++i) pm[i] = fast_exp2(fmaf(s[i], c, -L2));
      const f32x16 dp = F::qk(vt, r, hf, gf);
      f32x16 ds;
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = pm[i] * (dp[i] - D);
      F::pv(kt, lane, BwdOp<T>::make(ds), acc);
    };

    if constexpr (sizeof(T) == 2) {
      // Ring of three 32-key tile buffers fed by global-to-LDS loads: step t
      // loads tile t+2 into the buffer tile t-1 used, computes tile t, waits
      // for its own loads of tile t+1 and meets the other waves at a barrier
      // (no fence).  Tiles past the last one re-read it (their keys are
      // masked).  (The forward flash kernel's two 64-key buffers were
      // slightly slower for this pass.)
      constexpr int NDMA = (2 * kKT * kHeadDim / 8) / (WAVES * 64);
      static_assert(NDMA >= 1 && NDMA * WAVES * 64 == 2 * kKT * kHeadDim / 8, "tile must split evenly");
      using TL = Tile<T>;
      const int wu = __builtin_amdgcn_readfirstlane(wv);
      int goff[NDMA];
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const int ch = (64 * (WAVES * j + wu) + lane) & 255, row = ch >> 3;
        goff[j] = (int)(row * p.row_stride * 2 + (((ch & 7) ^ TL::swz(row)) << 4));
      }
      auto dma_tile = [&](__bf16* b, int t) __attribute__((always_inline)) {
        const int rel = (t < n_tiles ? t : n_tiles - 1) * kKT, valid = min(nk - rel, kKT);
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(K, p.row_stride, hoff, kb + rel, valid);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(V, p.row_stride, hoff, kb + rel, valid);
#pragma unroll
        for (int j = 0; j < NDMA; ++j) {
          const int c0 = 64 * (WAVES * j + wu);
          lds_load16(c0 < 256 ? rk : rv, b + 8 * c0, goff[j]);
        }
      };
      auto ring_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x70 | NDMA);  // vmcnt(NDMA) lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      };
      // the query and dO fragments land before any tile load is issued, so
      // the loop never drains the load queue to be sure of them
      __builtin_amdgcn_s_waitcnt(0);
      dma_tile(bq_ring0, 0);
      dma_tile(bq_ring1, 1);
      ring_barrier();
      auto step = [&](int t, const __bf16* cur, __bf16* fill) __attribute__((always_inline)) {
        dma_tile(fill, t + 2);
        tile_dq(t, cur, cur + TL::K_ELEMS);
        ring_barrier();
      };
      for (int t = 0; t < n_tiles; t += 3) {
        step(t, bq_ring0, bq_ring2);
        step(t + 1, bq_ring1, bq_ring0);
        step(t + 2, bq_ring2, bq_ring1);
      }
      __builtin_amdgcn_s_waitcnt(0x70);  // the last prefetches land before the LDS is handed on
    } else {
    st.load_range(K, V, p.row_stride, hoff, kb, min(nk, kKT), tid);
    {
      const L b0 = buf(0);
      st.store(b0.a_rows, b0.a_tr, b0.b_rows, nullptr, nullptr, nullptr, tid);
    }
    lds_barrier();
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) st.load_range(K, V, p.row_stride, hoff, kb + (int64_t)(t + 1) * kKT,
                                         min(nk - (t + 1) * kKT, kKT), tid);
      const L cur = buf(t);
      // fp32: K rows, V rows and K transposed (the PV operand) in LDS
      {
        f32x16 s = F::qk(cur.a_rows, r, hf, qf);
        if (t >= n_full) {
          const int lim = nk - t * kKT - 4 * hf;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (8 * (i / 4) + (i % 4) >= lim) s[i] = -INFINITY;
        }
        f32x16 pm;
#pragma unroll
        for (int i = 0; i < 16; ++i) pm[i] = fast_exp2(fmaf(s[i], c, -L2));
        const f32x16 dp = F::qk(cur.b_rows, r, hf, gf);
        f32x16 ds;
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = pm[i] * (dp[i] - D);
        F::pv(cur.a_tr, lane, BwdOp<T>::make(ds), acc);
      }
      if (t + 1 < n_tiles) {
        const L nx = buf(t + 1);
        st.store(nx.a_rows, nx.a_tr, nx.b_rows, nullptr, nullptr, nullptr, tid);
      }
      lds_barrier();
    }
    }
    if (qvalid) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int ch = 32 * n + 8 * a + 4 * hf;
          const f32x4 v4 = {acc[n][4 * a] * p.scale, acc[n][4 * a + 1] * p.scale, acc[n][4 * a + 2] * p.scale,
                            acc[n][4 * a + 3] * p.scale};
          float* dst = p.n_splits > 1 ? p.part + ((split * p.n_q + qrow) * H + h) * kHeadDim + ch
                                      : p.dq + qtok * p.row_stride + hoff + ch;
          f32x4* d4 = reinterpret_cast<f32x4*>(dst);
          *d4 = (p.accumulate && p.n_splits == 1) ? *d4 + v4 : v4;
        }
    }
  } else {
    const int64_t nk = p.kend[0] - p.kbeg[0];
    const int64_t n_kt = (nk + NT / 2 - 1) / (NT / 2);
    const int64_t kt = w % n_kt, hs = w / n_kt;
    const int h = (int)(hs % H);
    const int z = (int)(hs / H);
    const int64_t hoff = (int64_t)h * kHeadDim;
    const int64_t key = kt * (NT / 2) + wv * 32 + r;
    const bool kvalid = key < nk;
    const int64_t ktok = p.kbeg[0] + key;
    const typename F::Q kf = F::load_q(kvalid ? static_cast<const T*>(p.k) + ktok * p.row_stride + hoff : nullptr, hf);
    const typename F::Q vf = F::load_q(kvalid ? static_cast<const T*>(p.v) + ktok * p.row_stride + hoff : nullptr, hf);
    const int64_t n_qt = (p.n_q + kKT - 1) / kKT;
    const int64_t t0 = n_qt * z / p.n_qsplits, t1 = n_qt * (z + 1) / p.n_qsplits;
    f32x16 dk[2] = {{}, {}}, dv[2] = {{}, {}};
    // one 32-query tile: P^T and dS^T for this wave's 32 keys, dV += P^T dO, dK += dS^T Q
    auto tile_kv = [&](const T* qt, const T* qtr, const T* gt, const T* gtr, const float* l2s, const float* dds)
        __attribute__((always_inline)) {
      // element i: query row 8 (i/4) + 4 hf + i%4 of the tile, key r of this wave
      const f32x16 s = F::qk(qt, r, hf, kf);
      const f32x16 dp = F::qk(gt, r, hf, vf);
      f32x16 pm, ds;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(l2s + 8 * a + 4 * hf);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dds + 8 * a + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pm[4 * a + e] = fast_exp2(fmaf(s[4 * a + e], c, -l4[e]));
          ds[4 * a + e] = pm[4 * a + e] * (dp[4 * a + e] - d4[e]);
        }
      }
      F::pv(gtr, lane, BwdOp<T>::make(pm), dv);
      F::pv(qtr, lane, BwdOp<T>::make(ds), dk);
    };

    if constexpr (sizeof(T) == 2) {
      // Ring of three (Q, dO, L2, D) buffers as in the query-side pass, over
      // tiles of kBkvTQ queries (kBkvQT sub-tiles of 32, whose score
      // products are issued together so the matrix cores have independent
      // work while the exponentials of the other sub-tile run): step t loads
      // tile t+2 into the buffer tile t-1 used, computes tile t (tiles past
      // the split are loaded, not computed), waits for its own loads of tile
      // t+1 and meets the other waves at a barrier.  Lane l loads chunk l % 8
      // of query rows 32 j + 8 w + l / 8 (sub-tile j) of both Q and dO; it
      // follows those rows through the query map with running (frame,
      // remainder) pairs, so no tile needs a division.  Offsets are relative
      // to the wave's first row (the host bounds them below 2^31); rows from
      // n_q on get an offset past the buffer's limit and read as zeros, as do
      // their L2 and D, and such a row adds nothing (P = 1 but dO = 0 and
      // dP - D = 0).  The L2 values are log2 denominators (lse_mul = 1,
      // checked on the host).
      constexpr int QT = kBkvQT, TQ = kBkvTQ;
      constexpr int NDMA = 2 * QT + 2;  // Q and dO chunks per sub-tile, L2 values, D values
      static_assert(TQ <= kBkvRowVals, "one L2 / D load covers the tile");
      using TL = Tile<T>;
      const int64_t n_ut = (p.n_q + TQ - 1) / TQ;
      const int64_t u0 = n_ut * z / p.n_qsplits, u1 = n_ut * (z + 1) / p.n_qsplits;
      const int wu = __builtin_amdgcn_readfirstlane(wv);
      const int rowl = 8 * wu + (lane >> 3);
      const uint32_t cbyte = (uint32_t)(((lane & 7) ^ TL::swz(rowl)) << 4);
      const uint32_t qa = (uint32_t)p.qa, qb = (uint32_t)p.qb;
      const uint32_t df = (uint32_t)kKT / qa, dr = (uint32_t)kKT % qa;
      const uint32_t nq = (uint32_t)p.n_q;
      const uint32_t stride_b = (uint32_t)(p.row_stride * 2);
      uint32_t rr = (uint32_t)(u0 * TQ) + (uint32_t)rowl;  // this lane's sub-tile 0 row in the next tile loaded
      uint32_t fr = rr / qa, rem = rr - fr * qa;
      // (frame, remainder) of the row kKT further on
      auto adv = [&](uint32_t& f, uint32_t& m) __attribute__((always_inline)) {
        f += df;
        m += dr;
        if (m >= qa) {
          m -= qa;
          f += 1;
        }
      };
      const T* Qb = static_cast<const T*>(p.q) + p.qc * p.row_stride + hoff;
      const T* Gb = static_cast<const T*>(p.d_o) + (p.do_mapped ? p.qc * p.row_stride : 0) + hoff;
      const uint32_t lane_lin = (uint32_t)(lane >> 3) * stride_b + cbyte;  // dO rows by index
      const uint32_t lrow_off = (uint32_t)lane * (uint32_t)H * 4u;
      auto dma_tile = [&](__bf16* b, float* bv, int64_t t) __attribute__((always_inline)) {
        const uint32_t fr0 = __builtin_amdgcn_readfirstlane(fr), rem0 = __builtin_amdgcn_readfirstlane(rem);
        const bool valid0 = (uint32_t)(t * TQ) + (uint32_t)(8 * wu) < nq;
        const int64_t tok0 = valid0 ? (int64_t)fr0 * qb + rem0 : 0;
        const int64_t r_first = valid0 ? t * TQ + 8 * wu : 0;
        const __amdgpu_buffer_rsrc_t rq =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Qb + tok0 * p.row_stride), (short)0, 0x7fffffff, 0x00020000);
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(Gb + (p.do_mapped ? tok0 : r_first) * p.row_stride), (short)0, 0x7fffffff, 0x00020000);
        uint32_t f = fr, m = rem, rj = rr;
#pragma unroll
        for (int j = 0; j < QT; ++j) {
          const bool valid = rj < nq;
          const uint32_t rows = (f - fr0) * qb + m - rem0;  // token rows past the wave's first
          const uint32_t oq = valid ? rows * stride_b + cbyte : 0x80000000u;
          const uint32_t og = valid ? (p.do_mapped ? oq : lane_lin + 32u * j * stride_b) : 0x80000000u;
          lds_load16(rq, b + kKT * kHeadDim * j + 512 * wu, (int)oq);
          lds_load16(rg, b + TQ * kHeadDim + kKT * kHeadDim * j + 512 * wu, (int)og);
          if (j + 1 < QT) {
            rj += kKT;
            adv(f, m);
          }
        }
        const int64_t r0 = t * TQ;
        const int nrec = r0 < p.n_q ? (int)(((p.n_q - r0 - 1) * H + 1) * 4) : 0;
        const int64_t lo = r0 < p.n_q ? r0 * H + h : 0;
        const __amdgpu_buffer_rsrc_t rl =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.lse + lo), (short)0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t rd =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.dd + lo), (short)0, nrec, 0x00020000);
        lds_load4(rl, bv + kBkvRowVals * wu, (int)lrow_off);
        lds_load4(rd, bv + kBkvRowVals * (4 + wu), (int)lrow_off);
        // the next tile's rows
        rr += TQ;
#pragma unroll
        for (int j = 0; j < QT; ++j) adv(fr, rem);
      };
      auto ring_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x70 | NDMA);  // vmcnt(NDMA) lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      };
      // one ring tile: every sub-tile's score and dO . v products first, then
      // per sub-tile the softmax gradient and the two accumulations
      auto tile_all = [&](const __bf16* cur, const float* curv) __attribute__((always_inline)) {
        f32x16 sc[QT], dpv[QT];
#pragma unroll
        for (int j = 0; j < QT; ++j) {
          sc[j] = F::qk(cur + kKT * kHeadDim * j, r, hf, kf);
          dpv[j] = F::qk(cur + TQ * kHeadDim + kKT * kHeadDim * j, r, hf, vf);
        }
#pragma unroll
        for (int j = 0; j < QT; ++j) {
          const float* l2s = curv + kBkvRowVals * wu + kKT * j;
          const float* dds = l2s + 4 * kBkvRowVals;
          f32x16 pm, ds;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(l2s + 8 * a + 4 * hf);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dds + 8 * a + 4 * hf);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pm[4 * a + e] = fast_exp2(fmaf(sc[j][4 * a + e], c, -l4[e]));
              ds[4 * a + e] = pm[4 * a + e] * (dpv[j][4 * a + e] - d4[e]);
            }
          }
          F::pv(cur + TQ * kHeadDim + kKT * kHeadDim * j, lane, BwdOp<T>::make(pm), dv);
          F::pv(cur + kKT * kHeadDim * j, lane, BwdOp<T>::make(ds), dk);
        }
      };
      auto step = [&](int64_t t, const __bf16* cur, const float* curv, __bf16* fill, float* fillv)
          __attribute__((always_inline)) {
        dma_tile(fill, fillv, t + 2);
        if (t < u1) tile_all(cur, curv);
        ring_barrier();
      };
      if (u0 < u1) {
        // the key and value fragments land before any tile load is issued
        __builtin_amdgcn_s_waitcnt(0);
        dma_tile(bk_ring0, bk_vals0, u0);
        dma_tile(bk_ring1, bk_vals1, u0 + 1);
        ring_barrier();
        for (int64_t t = u0; t < u1; t += 3) {
          step(t, bk_ring0, bk_vals0, bk_ring2, bk_vals2);
          step(t + 1, bk_ring1, bk_vals1, bk_ring0, bk_vals0);
          step(t + 2, bk_ring2, bk_vals2, bk_ring1, bk_vals1);
        }
        __builtin_amdgcn_s_waitcnt(0x70);  // the last prefetches land before the LDS is handed on
      }
    } else {
    if (t0 < t1) {
      st.load_queries(p, hoff, h, t0 * kKT, tid);
      const L b0 = buf(0);
      st.store(b0.a_rows, b0.a_tr, b0.b_rows, b0.b_tr, b0.l2s, b0.dds, tid);
      lds_barrier();
    }
    for (int64_t t = t0; t < t1; ++t) {
      if (t + 1 < t1) st.load_queries(p, hoff, h, (t + 1) * kKT, tid);
      const L cur = buf(t - t0);
      tile_kv(cur.a_rows, cur.a_tr, cur.b_rows, cur.b_tr, cur.l2s, cur.dds);
      if (t + 1 < t1) {
        const L nx = buf(t + 1 - t0);
        st.store(nx.a_rows, nx.a_tr, nx.b_rows, nx.b_tr, nx.l2s, nx.dds, tid);
      }
      lds_barrier();
    }
    }
    if (kvalid) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int ch = 32 * n + 8 * a + 4 * hf;
          const f32x4 k4 = {dk[n][4 * a] * p.scale, dk[n][4 * a + 1] * p.scale, dk[n][4 * a + 2] * p.scale,
                            dk[n][4 * a + 3] * p.scale};
          const f32x4 v4 = {dv[n][4 * a], dv[n][4 * a + 1], dv[n][4 * a + 2], dv[n][4 * a + 3]};
          if (p.n_qsplits > 1) {
            *reinterpret_cast<f32x4*>(p.part + ((z * nk + key) * H + h) * kHeadDim + ch) = k4;
            *reinterpret_cast<f32x4*>(p.part + (((p.n_qsplits + z) * nk + key) * H + h) * kHeadDim + ch) = v4;
          } else {
            f32x4* dk4 = reinterpret_cast<f32x4*>(p.dk + ktok * p.row_stride + hoff + ch);
            f32x4* dv4 = reinterpret_cast<f32x4*>(p.dv + ktok * p.row_stride + hoff + ch);
            *dk4 = p.accumulate ? *dk4 + k4 : k4;
            *dv4 = p.accumulate ? *dv4 + v4 : v4;
          }
        }
    }
  }
}

template <typename T, int KIND>
static hipError_t launch_flash_bwd_t(const FlashBwdParams& p, hipStream_t stream) {
  constexpr int WAVES = 4;
  int64_t blocks;
  if (KIND == kBwdDQ) {
    blocks = (p.n_q + WAVES * 32 - 1) / (WAVES * 32) * p.n_heads * p.n_splits;
  } else {
    const int64_t nk = p.kend[0] - p.kbeg[0];
    blocks = (nk + WAVES * 32 - 1) / (WAVES * 32) * p.n_heads * p.n_qsplits;
  }
  if (blocks == 0) return hipSuccess;
  if (blocks > 0xffffffffLL || p.n_splits < 1 || p.n_qsplits < 1) return hipErrorInvalidValue;
  if (KIND == kBwdDKDV && sizeof(T) == 2) {
    // the key-side tile ring: log2 denominators, a query map whose rows never
    // go back (consecutive queries move at most qb token rows), 32-bit row
    // counters and per-wave byte offsets below 2^31
    const int64_t span = (kBkvTQ - kKT + 7) * std::max<int64_t>(p.qb, 1) * p.row_stride * 2 + 128;
    if (p.lse_mul != 1.0f || p.qa < 1 || (p.qb == 0 ? p.n_q > p.qa : p.qb < p.qa) ||
        p.n_q + 4 * kBkvTQ > INT32_MAX || p.n_q * p.n_heads * 4 > INT32_MAX || span > INT32_MAX)
      return hipErrorInvalidValue;
  }
  // (the bf16 passes use the static tile rings instead)
  const size_t lds = sizeof(T) == 2 ? 0 : 2 * (size_t)BwdLds<T>::STAGE_BYTES;
  const void* fn = reinterpret_cast<const void*>(&flash_bwd_kernel<T, WAVES, KIND>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((flash_bwd_kernel<T, WAVES, KIND>), dim3((unsigned)blocks), dim3(WAVES * 64), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_flash_bwd(int dtype, int kind, const FlashBwdParams& p, hipStream_t stream) {
  if (kind == kBwdDQ)
    return dtype == kBF16 ? launch_flash_bwd_t<__bf16, kBwdDQ>(p, stream) : launch_flash_bwd_t<float, kBwdDQ>(p, stream);
  if (kind == kBwdDKDV)
    return dtype == kBF16 ? launch_flash_bwd_t<__bf16, kBwdDKDV>(p, stream)
                          : launch_flash_bwd_t<float, kBwdDKDV>(p, stream);
  return hipErrorInvalidValue;
}

// ---- partial sums ------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = (int64_t)p.n_heads * (kHeadDim / 4);
  if (gid >= p.n_rows * per_row) return;
  const int64_t r = gid / per_row, rem = gid - r * per_row;
  f32x4 acc = {0, 0, 0, 0};
  for (int i = 0; i < p.n_parts; ++i) acc += *reinterpret_cast<const f32x4*>(p.part + i * p.part_stride + 4 * gid);
  const int64_t row = (r / p.qa) * p.qb + p.qc + r % p.qa;
  f32x4* dst = reinterpret_cast<f32x4*>(p.out + row * p.n_heads * kHeadDim + 4 * rem);
  *dst = p.accumulate ? *dst + acc : acc;
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream) {
  const int64_t threads = p.n_rows * p.n_heads * (kHeadDim / 4);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_kernel(float* x, int64_t n) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < n) x[gid] = 0.0f;
}

hipError_t launch_fill(float* x, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x, n);
  return hipGetLastError();
}

// ---- gate backward -----------------------------------------------------------
// One wave per (window, head); 16 lanes per token (4 channels each), four
// tokens per step.  Per image token t (window i, in-window index kk):
//   g = sigmoid(W_g . q),  dO_sel = (1 - g) dO,  D_sel = dO_sel . O_sel,
//   dz = (dO . (O'_i - O_sel)) g (1 - g) (stored; the selection backward
//   writes the token's dq = dz W_g + ...),
// and per window: dO_comp = sum_t g dO, D_comp = dO_comp . O'_i, the dW_g
// partial sum_t dz q, and the compressed attention's log2 denominator.
template <typename T>
__device__ __forceinline__ f32x4 load4(const T* x) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(x);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
  } else {
    return *reinterpret_cast<const f32x4*>(x);
  }
}
template <typename T>
__device__ __forceinline__ void store4(T* x, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(x) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  } else {
    *reinterpret_cast<f32x4*>(x) = v;
  }
}
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x += xor_lane(x, m);
  return x;
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

template <typename T>
__global__ __launch_bounds__(256) void gate_bwd_kernel(GateBwdParams p) {
  const Geometry& geo = p.g;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int cl = lane & 15, tg = lane >> 4;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  if (item >= geo.n_windows * geo.n_heads) return;  // whole waves
  const int64_t H = geo.n_heads;
  const int64_t win = item / H, h = item % H;
  const int s2 = (int)(geo.pool * geo.pool);
  const int64_t sb = geo.sb;
  const int ch = 4 * cl;
  const f32x4 w4 = load4(static_cast<const T*>(p.wg) + h * kHeadDim + ch);
  const f32x4 oc4 = *reinterpret_cast<const f32x4*>(p.oc + (win * H + h) * kHeadDim + ch);
  const T* Q = static_cast<const T*>(p.q);
  const T* G = static_cast<const T*>(p.d_o);
  T* doblk = static_cast<T*>(p.doblk) + (win * H + h) * sb * kHeadDim;
  T* doT = p.doT ? static_cast<T*>(p.doT) + (win * H + h) * kHeadDim * sb : nullptr;
  f32x4 acc_doc = {0, 0, 0, 0}, acc_dwg = {0, 0, 0, 0};
  for (int it = 0; 4 * it < sb; ++it) {
    const int kk = 4 * it + tg;
    const bool valid = kk < s2;
    const int64_t tok = window_token(geo, win, valid ? kk : 0);
    const int64_t u = window_image_index(geo, win, valid ? kk : 0);
    const f32x4 zero = {0, 0, 0, 0};
    const f32x4 q4 = valid ? load4(Q + (tok * H + h) * kHeadDim + ch) : zero;
    const f32x4 g4 = valid ? load4(G + (tok * H + h) * kHeadDim + ch) : zero;
    const f32x4 os4 = valid ? *reinterpret_cast<const f32x4*>(p.osel + (u * H + h) * kHeadDim + ch) : zero;
    const float z = sum16(dot4(q4, w4));
    const float g = 1.0f / (1.0f + expf(-z));
    const float dg = sum16(dot4(g4, oc4 - os4));
    const float dz = dg * g * (1.0f - g);
    const f32x4 ds4 = (1.0f - g) * g4;
    const float dsel = sum16(dot4(ds4, os4));
    if (valid) {
      acc_dwg += dz * q4;
      acc_doc += g * g4;
      if (p.dosel_img) {
        store4(static_cast<T*>(p.dosel_img) + (u * H + h) * kHeadDim + ch, ds4);
        if (cl == 0) p.dsel_img[u * H + h] = dsel;
      }
    }
    // blocked copies (padding slots get zeros, L2 = +inf)
    store4(doblk + kk * kHeadDim + ch, ds4);
    if (p.doT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) doT[(ch + e) * sb + kk] = from_f32<T>(ds4[e]);
    }
    if (cl == 0) {
      p.l2blk[(win * H + h) * sb + kk] = valid ? p.l2sel[u * H + h] : INFINITY;
      p.dblk[(win * H + h) * sb + kk] = valid ? dsel : 0.0f;
      p.dzblk[(win * H + h) * sb + kk] = valid ? dz : 0.0f;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc_doc[e] += xor_lane(acc_doc[e], 16);
    acc_doc[e] += xor_lane(acc_doc[e], 32);
    acc_dwg[e] += xor_lane(acc_dwg[e], 16);
    acc_dwg[e] += xor_lane(acc_dwg[e], 32);
  }
  const float dc = sum16(dot4(acc_doc, oc4));
  if (tg == 0) {
    store4(static_cast<T*>(p.doc) + (win * H + h) * kHeadDim + ch, acc_doc);
    *reinterpret_cast<f32x4*>(p.dwg_part + (win * H + h) * kHeadDim + ch) = acc_dwg;
    if (cl == 0) {
      p.dc[win * H + h] = dc;
      p.l2c[win * H + h] = p.lse_c[win * H + h] * kLog2e;
    }
  }
}

hipError_t launch_gate_bwd(int dtype, const GateBwdParams& p, hipStream_t stream) {
  const int64_t items = p.g.n_windows * p.g.n_heads;
  if (items == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  if (dtype == kBF16)
    hipLaunchKernelGGL(gate_bwd_kernel<__bf16>, dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(gate_bwd_kernel<float>, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// dW_g[h] = sum over windows of the partials, in a fixed order: the windows
// are cut into kDwgSlices contiguous slices; a workgroup per (slice, head)
// sums its slice (four interleaved runs, then in order), and one workgroup
// per head then sums the slice totals.
__global__ __launch_bounds__(256) void dwg_slice_kernel(DwgParams p) {
  __shared__ float red[4][kHeadDim];
  const int sl = blockIdx.x, h = blockIdx.y, e = threadIdx.x & 63, sub = threadIdx.x >> 6;
  const int64_t per = (p.n_windows + kDwgSlices - 1) / kDwgSlices;
  const int64_t j0 = sl * per, j1 = j0 + per < p.n_windows ? j0 + per : p.n_windows;
  float acc = 0.0f;
  for (int64_t j = j0 + sub; j < j1; j += 4) acc += p.part[(j * p.n_heads + h) * kHeadDim + e];
  red[sub][e] = acc;
  __syncthreads();
  if (sub == 0) p.slices[((int64_t)sl * p.n_heads + h) * kHeadDim + e] = red[0][e] + red[1][e] + red[2][e] + red[3][e];
}
__global__ __launch_bounds__(256) void dwg_total_kernel(DwgParams p) {
  __shared__ float red[4][kHeadDim];
  const int h = blockIdx.x, e = threadIdx.x & 63, sub = threadIdx.x >> 6;
  float acc = 0.0f;
  for (int sl = sub; sl < kDwgSlices; sl += 4) acc += p.slices[((int64_t)sl * p.n_heads + h) * kHeadDim + e];
  red[sub][e] = acc;
  __syncthreads();
  if (sub == 0) p.dwg[h * kHeadDim + e] = red[0][e] + red[1][e] + red[2][e] + red[3][e];
}

hipError_t launch_dwg_reduce(const DwgParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(dwg_slice_kernel, dim3(kDwgSlices, (unsigned)p.n_heads), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(dwg_total_kernel, dim3((unsigned)p.n_heads), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ---- inverse top-k lists -------------------------------------------------------
__global__ __launch_bounds__(256) void inv_zero_kernel(int32_t* x, int64_t n) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < n) x[gid] = 0;
}
// Counts per (head, window) list; the count an entry's atomic returns is its
// rank in the list (in arrival order), parked in `list` until the scatter.
__global__ __launch_bounds__(256) void inv_count_kernel(InvParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = p.n_windows * p.n_heads * p.topk;
  if (gid >= n) return;
  const int32_t j = p.topk_idx[gid];
  const int64_t h = (gid / p.topk) % p.n_heads;
  if (j >= 0 && j < p.n_windows) p.list[gid] = atomicAdd(&p.off[h * p.n_windows + j], 1);
}
// Exclusive scan of off[0 .. n) in blocks of 1024 (4 per thread), block sums
// scanned by one workgroup, then added back.
constexpr int kScanBlock = 1024;
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* tmp, int32_t& total) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int32_t x = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += x;
    __syncthreads();
  }
  total = tmp[255];
  const int32_t incl = tmp[t];
  __syncthreads();
  return incl - v;
}
__global__ __launch_bounds__(256) void scan_blocks_kernel(int32_t* x, int64_t n, int32_t* bsum) {
  __shared__ int32_t tmp[256];
  const int64_t base = (int64_t)blockIdx.x * kScanBlock + 4 * threadIdx.x;
  int32_t v[4];
  for (int e = 0; e < 4; ++e) v[e] = base + e < n ? x[base + e] : 0;
  const int32_t s = v[0] + v[1] + v[2] + v[3];
  int32_t total;
  int32_t run = block_exclusive_scan(s, tmp, total);
  for (int e = 0; e < 4; ++e) {
    if (base + e < n) x[base + e] = run;
    run += v[e];
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}
__global__ __launch_bounds__(256) void scan_sums_kernel(int32_t* bsum, int64_t nb) {
  __shared__ int32_t tmp[256];
  int32_t carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += 256) {
    const int64_t b = b0 + threadIdx.x;
    const int32_t v = b < nb ? bsum[b] : 0;
    int32_t total;
    const int32_t ex = block_exclusive_scan(v, tmp, total);
    if (b < nb) bsum[b] = carry + ex;
    carry += total;
  }
}
__global__ __launch_bounds__(256) void scan_add_kernel(int32_t* x, int64_t n, const int32_t* bsum) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < n) x[gid] += bsum[gid / kScanBlock];
}
// Each entry to its list at the scanned offset + its rank (no atomics).
__global__ __launch_bounds__(256) void inv_fill_kernel(InvParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = p.n_windows * p.n_heads * p.topk;
  if (gid >= n) return;
  const int32_t j = p.topk_idx[gid];
  const int64_t i = gid / p.topk / p.n_heads, h = (gid / p.topk) % p.n_heads;
  if (j < 0 || j >= p.n_windows) return;
  p.raw[p.off[h * p.n_windows + j] + p.list[gid]] = (int32_t)i;
}
// One wave per list: each element's position is its rank (ties by fill
// position, so repeated entries keep distinct slots); the result does not
// depend on the order the fill kernel's atomics took.
// Lists of 65 .. kSortMax entries are sorted by a bitonic network in a
// wave-private LDS buffer (padded to a power of two); shorter and longer
// lists by rank: the list is compared in chunks of 64 entries (one per
// lane, loaded once) whose values are broadcast lane by lane (n^2 / 64
// register compares per lane).  Equal entries are equal values, so every
// method gives the same list.
constexpr int kSortMax = 2048;
__shared__ int32_t sort_buf[4][kSortMax];
__global__ __launch_bounds__(256) void inv_sort_kernel(InvParams p) {
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= p.n_windows * p.n_heads) return;  // whole waves
  const int lane = lane_id();
  const int32_t b = p.off[seg], n = p.off[seg + 1] - b;
  if (n > 64 && n <= kSortMax) {
    int32_t* a = sort_buf[threadIdx.x >> 6];
    int N = 128;
    while (N < n) N <<= 1;
    for (int i = lane; i < N; i += 64) a[i] = i < n ? p.raw[b + i] : INT32_MAX;
    // the wave's LDS operations complete in order; the waits keep the
    // compiler from moving a stage's reads above the previous stage's writes
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    for (int k = 2; k <= N; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int t = lane; t < N / 2; t += 64) {
          const int i = 2 * j * (t / j) + t % j, l = i + j;  // i has bit j clear
          const int32_t x = a[i], y = a[l];
          if ((x > y) == ((i & k) == 0)) {
            a[i] = y;
            a[l] = x;
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
      }
    }
    for (int i = lane; i < n; i += 64) p.list[b + i] = a[i];
    return;
  }
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int e = e0 + lane;
    const int32_t x = e < n ? p.raw[b + e] : 0;
    int32_t rank = 0;
    for (int c0 = 0; c0 < n; c0 += 64) {
      const int32_t y = c0 + lane < n ? p.raw[b + c0 + lane] : INT32_MAX;
      const int m = n - c0 < 64 ? n - c0 : 64;
      for (int f = 0; f < m; ++f) {
        const int32_t yf = __builtin_amdgcn_readlane(y, f);
        rank += (yf < x || (yf == x && c0 + f < e)) ? 1 : 0;
      }
    }
    if (e < n) p.list[b + rank] = x;
  }
}

// Processing order of the key side of the selection backward: the (head,
// window) lists by length class, longest first (class 0: 512 entries or
// more, then one class per power of two, class 7: under 8), in list order
// within a class, so the long lists do not start last and leave a tail.  A
// counting sort: per block of 1024 lists the class counts, an exclusive scan
// of the class-major counts, then each block writes its lists at the
// scanned positions.
constexpr int kOrdClasses = 8;
constexpr int kOrdBlock = 1024;
__device__ __forceinline__ int list_class(int32_t n) {
  const int bits = 32 - __builtin_clz((uint32_t)n | 1u);
  const int c = 10 - bits;
  return c < 0 ? 0 : (c > kOrdClasses - 1 ? kOrdClasses - 1 : c);
}
__global__ __launch_bounds__(256) void order_count_kernel(InvParams p) {
  __shared__ int32_t cnt[kOrdClasses];
  const int64_t segs = p.n_windows * p.n_heads;
  const int64_t nblk = (segs + kOrdBlock - 1) / kOrdBlock;
  if (threadIdx.x < kOrdClasses) cnt[threadIdx.x] = 0;
  __syncthreads();
  for (int e = 0; e < kOrdBlock / 256; ++e) {
    const int64_t seg = (int64_t)blockIdx.x * kOrdBlock + e * 256 + threadIdx.x;
    if (seg < segs) atomicAdd(&cnt[list_class(p.off[seg + 1] - p.off[seg])], 1);
  }
  __syncthreads();
  if (threadIdx.x < kOrdClasses) p.ccnt[threadIdx.x * nblk + blockIdx.x] = cnt[threadIdx.x];
}
__global__ __launch_bounds__(256) void order_fill_kernel(InvParams p) {
  __shared__ int32_t wcnt[kOrdBlock / 64][kOrdClasses];  // per 64-list group, in list order
  const int64_t segs = p.n_windows * p.n_heads;
  const int64_t nblk = (segs + kOrdBlock - 1) / kOrdBlock;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  int cls[kOrdBlock / 256];
  uint64_t below[kOrdBlock / 256];
  for (int e = 0; e < kOrdBlock / 256; ++e) {
    const int64_t seg = (int64_t)blockIdx.x * kOrdBlock + e * 256 + threadIdx.x;
    cls[e] = seg < segs ? list_class(p.off[seg + 1] - p.off[seg]) : -1;
    uint64_t mine = 0;
    for (int c = 0; c < kOrdClasses; ++c) {
      const uint64_t m = __ballot(cls[e] == c);
      if (cls[e] == c) mine = m;
      if (lane == 0) wcnt[e * 4 + wv][c] = __builtin_popcountll(m);
    }
    below[e] = mine & ((1ull << lane) - 1);
  }
  __syncthreads();
  for (int e = 0; e < kOrdBlock / 256; ++e) {
    if (cls[e] < 0) continue;
    const int c = cls[e], grp = e * 4 + wv;
    int32_t pos = p.ccnt[c * nblk + blockIdx.x] + __builtin_popcountll(below[e]);
    for (int g = 0; g < grp; ++g) pos += wcnt[g][c];
    p.order[pos] = (int32_t)((int64_t)blockIdx.x * kOrdBlock + e * 256 + threadIdx.x);
  }
}

hipError_t launch_inverse_index(const InvParams& p, hipStream_t stream) {
  const int64_t segs = p.n_windows * p.n_heads;
  const int64_t n = segs + 1;
  const int64_t entries = segs * p.topk;
  if (segs == 0) return hipSuccess;
  const unsigned gz = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(inv_zero_kernel, dim3(gz), dim3(256), 0, stream, p.off, n);
  const unsigned ge = (unsigned)((entries + 255) / 256);
  hipLaunchKernelGGL(inv_count_kernel, dim3(ge), dim3(256), 0, stream, p);
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  hipLaunchKernelGGL(scan_blocks_kernel, dim3((unsigned)nb), dim3(256), 0, stream, p.off, n, p.bsum);
  hipLaunchKernelGGL(scan_sums_kernel, dim3(1), dim3(256), 0, stream, p.bsum, nb);
  hipLaunchKernelGGL(scan_add_kernel, dim3(gz), dim3(256), 0, stream, p.off, n, (const int32_t*)p.bsum);
  hipLaunchKernelGGL(inv_fill_kernel, dim3(ge), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(inv_sort_kernel, dim3((unsigned)((segs + 3) / 4)), dim3(256), 0, stream, p);
  if (p.order) {
    const int64_t ob = (segs + kOrdBlock - 1) / kOrdBlock, nc = kOrdClasses * ob;
    const int64_t ncb = (nc + kScanBlock - 1) / kScanBlock;
    hipLaunchKernelGGL(order_count_kernel, dim3((unsigned)ob), dim3(256), 0, stream, p);
    hipLaunchKernelGGL(scan_blocks_kernel, dim3((unsigned)ncb), dim3(256), 0, stream, p.ccnt, nc, p.cbsum);
    hipLaunchKernelGGL(scan_sums_kernel, dim3(1), dim3(256), 0, stream, p.cbsum, ncb);
    hipLaunchKernelGGL(scan_add_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, stream, p.ccnt, nc,
                       (const int32_t*)p.cbsum);
    hipLaunchKernelGGL(order_fill_kernel, dim3((unsigned)ob), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

// ---- selection backward ------------------------------------------------------
// Window-blocked gathers in the layout of the forward selection kernel: a
// chunk is 32 slots of concatenated windows (sb slots each); lane l = 16 g + ql.
template <typename T>
struct BwdChunk {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int KV = 16 / VE;  // 16-byte loads per 16 channels of a row
  static constexpr int VV = 8 / VE;   // 16-byte loads per 8 slots of a transposed row
  uint4 x[2][KV];  // score operand rows, tiles tau = 0, 1
  uint4 y[2][KV];  // second score operand rows
  uint4 t[4][VV];  // contraction operand (transposed), slots 8g .. 8g+7
  uint4 u[4][VV];  // second contraction operand (key side only)
  float l2[8], dd[8];  // key side: L2 and D of slots 8g .. 8g+7
  int jv, kkv0;    // window and first in-window slot of this lane's 8 slots
};

// rows of the blocked [M'][H][sb][d] tensor X for A row ql of both tiles
template <typename T>
__device__ __forceinline__ void load_rows(uint4 (&dst)[2][BwdChunk<T>::KV], const T* X, int ja, int64_t kka,
                                          int64_t h, int64_t H, int64_t sb, int g) {
  using C = BwdChunk<T>;
  const T* b = X + (((int64_t)(ja < 0 ? 0 : ja) * H + h) * sb + kka) * kHeadDim + 16 * g;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int x = 0; x < C::KV; ++x) dst[tau][x] = ld16(b + 4 * tau * kHeadDim + x * C::VE);
}
// 8 slots from kk0 of channel rows 16m + ql of the blocked [M'][H][d][sb] tensor X
template <typename T>
__device__ __forceinline__ void load_trans(uint4 (&dst)[4][BwdChunk<T>::VV], const T* X, int j, int64_t kk0,
                                           int64_t h, int64_t H, int64_t sb, int ql) {
  using C = BwdChunk<T>;
  const T* b = X + ((int64_t)(j < 0 ? 0 : j) * H + h) * kHeadDim * sb + kk0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int x = 0; x < C::VV; ++x) dst[m][x] = ld16(b + (16 * m + ql) * sb + x * C::VE);
}

__shared__ __attribute__((aligned(16))) __bf16 sel_slab[4][2][kSlabElems];

// Query side: one wave per (window, head, group of QB blocks of 16 queries);
// per chunk of the window's top-k slots: S^T = K Q^T, P, dP^T = V dO^T,
// dS, dq^T += K^T dS.  Stores dz W_g + scale * dq + the pooled row's gradient / s^2
// into the query rows (their first store).
template <typename T, int QB>
__global__ __launch_bounds__(256) void sel_dq_kernel(SelBwdParams p) {
  using F = Frag16<T>;
  using C = BwdChunk<T>;
  const Geometry& geo = p.g;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int ql = lane & 15, g = lane >> 4;
  const int s2 = (int)(geo.pool * geo.pool);
  const int n_grp = ((s2 + 15) / 16 + QB - 1) / QB;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  if (item >= geo.n_windows * geo.n_heads * n_grp) return;
  const int qg = (int)(item % n_grp);
  const int64_t h = item / n_grp / geo.n_windows;
  const int64_t win = item / n_grp % geo.n_windows;
  const int64_t H = geo.n_heads, sb = geo.sb;
  const int K = p.topk;
  const float c = p.scale_log2;
  const int32_t* trow = p.topk_idx + (win * H + h) * K;
  const int tr0 = lane < K ? trow[lane] : -1;
  const int tr1 = lane + 64 < K ? trow[lane + 64] : -1;
  const int n_chunks = (int)((K * sb + 31) / 32);

  typename F::Q qfs[QB], gfs[QB];
  float l2s[QB], dds[QB], dzs[QB];
  f32x4 acc[QB][4];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int kq = (QB * qg + b) * 16 + ql;
    const bool qvalid = kq < s2;
    const int64_t row = (win * H + h) * sb + (qvalid ? kq : 0);
    qfs[b] = F::load_q(qvalid ? static_cast<const T*>(p.qblk) + row * kHeadDim : nullptr, g);
    gfs[b] = F::load_q(qvalid ? static_cast<const T*>(p.doblk) + row * kHeadDim : nullptr, g);
    l2s[b] = qvalid ? p.l2blk[row] : INFINITY;
    dds[b] = qvalid ? p.dblk[row] : 0.0f;
    dzs[b] = qvalid ? p.dzblk[row] : 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[b][m] = f32x4{0, 0, 0, 0};
  }
  auto load = [&](C& ch, int ci) __attribute__((always_inline)) {
    const int64_t ga = (int64_t)ci * 32 + 8 * (ql >> 2);
    const int ja = topk_entry(tr0, tr1, (int)(ga / sb), K, geo.n_windows);
    const int64_t kka = ga % sb + (ql & 3);
    load_rows<T>(ch.x, static_cast<const T*>(p.kblk), ja, kka, h, H, sb, g);
    load_rows<T>(ch.y, static_cast<const T*>(p.vrow), ja, kka, h, H, sb, g);
    const int64_t gv = (int64_t)ci * 32 + 8 * g;
    ch.jv = topk_entry(tr0, tr1, (int)(gv / sb), K, geo.n_windows);
    ch.kkv0 = (int)(gv % sb);
    if constexpr (sizeof(T) == 2)
      transpose_chunk(ch.x, ch.t, sel_slab[wv][0], ql, g);
    else
      load_trans<T>(ch.t, static_cast<const T*>(p.kT), ch.jv, ch.kkv0, h, H, sb, ql);
  };
  auto process = [&](const C& ch) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const f32x4 s0 = F::qk(ch.x[0], qfs[b]), s1 = F::qk(ch.x[1], qfs[b]);
      const f32x4 d0 = F::qk(ch.y[0], gfs[b]), d1 = F::qk(ch.y[1], gfs[b]);
      f32x4 ds0, ds1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool v0 = ch.jv >= 0 && ch.kkv0 + e < s2;
        const bool v1 = ch.jv >= 0 && ch.kkv0 + 4 + e < s2;
        const float p0 = v0 ? fast_exp2(fmaf(s0[e], c, -l2s[b])) : 0.0f;
        const float p1 = v1 ? fast_exp2(fmaf(s1[e], c, -l2s[b])) : 0.0f;
        ds0[e] = p0 * (d0[e] - dds[b]);
        ds1[e] = p1 * (d1[e] - dds[b]);
      }
      F::pv(ch.t, ds0, ds1, acc[b]);
    }
  };
  C A, B;
  load(A, 0);
  if (n_chunks > 1) load(B, 1);
  int ci = 0;
  for (; ci + 3 < n_chunks; ci += 2) {
    process(A);
    load(A, ci + 2);
    process(B);
    load(B, ci + 3);
  }
  process(A);
  if (ci + 2 < n_chunks) load(A, ci + 2);
  if (ci + 1 < n_chunks) process(B);
  if (ci + 2 < n_chunks) process(A);

#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int kq = (QB * qg + b) * 16 + ql;
    if (kq >= s2) continue;
    const int64_t tok = window_token(geo, win, kq);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // the gate's dz W_g, + this branch's gradient, + the pooled row's
      // gradient / s^2 (the pooling backward): the first store of the row
      const f32x4 w4 = load4(static_cast<const T*>(p.wg) + h * kHeadDim + 16 * m + 4 * g);
      const f32x4 pooled = *reinterpret_cast<const f32x4*>(p.dqc + (win * H + h) * kHeadDim + 16 * m + 4 * g);
      f32x4* dst = reinterpret_cast<f32x4*>(p.dq + (tok * H + h) * kHeadDim + 16 * m + 4 * g);
      *dst = dzs[b] * w4 + acc[b][m] * p.scale + pooled * p.inv_area;
    }
  }
}

// Key side: one wave per (key window, head, group of KB blocks of 16 keys);
// per chunk of the inverse list's query slots: S^T = Q K^T, P, dP^T = dO V^T,
// dS, dv^T += dO^T P, dk^T += Q^T dS.  Adds scale * dk and dv, and the pooled
// rows' gradients / s^2, into the key rows.
template <typename T, int KB>
__global__ __launch_bounds__(256) void sel_dkdv_kernel(SelBwdParams p) {
  using F = Frag16<T>;
  using C = BwdChunk<T>;
  const Geometry& geo = p.g;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int kl = lane & 15, g = lane >> 4;
  const int s2 = (int)(geo.pool * geo.pool);
  const int n_grp = ((s2 + 15) / 16 + KB - 1) / KB;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  if (item >= geo.n_windows * geo.n_heads * n_grp) return;
  const int kg = (int)(item % n_grp);
  // (head, window) lists in the longest-first order when one is given
  const int64_t seg = p.order ? p.order[item / n_grp] : item / n_grp;
  const int64_t h = seg / geo.n_windows;
  const int64_t win = seg % geo.n_windows;
  const int64_t H = geo.n_heads, sb = geo.sb;
  const float c = p.scale_log2;
  const int32_t lb = p.inv_off[h * geo.n_windows + win];
  const int32_t n_list = p.inv_off[h * geo.n_windows + win + 1] - lb;
  const int32_t* list = p.inv_list + lb;
  const int n_chunks = (int)(((int64_t)n_list * sb + 31) / 32);

  typename F::Q kfs[KB], vfs[KB];
  f32x4 dk[KB][4], dv[KB][4];
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int kk = (KB * kg + b) * 16 + kl;
    const bool kvalid = kk < s2;
    const int64_t row = (win * H + h) * sb + (kvalid ? kk : 0);
    kfs[b] = F::load_q(kvalid ? static_cast<const T*>(p.kblk) + row * kHeadDim : nullptr, g);
    vfs[b] = F::load_q(kvalid ? static_cast<const T*>(p.vrow) + row * kHeadDim : nullptr, g);
#pragma unroll
    for (int m = 0; m < 4; ++m) dk[b][m] = dv[b][m] = f32x4{0, 0, 0, 0};
  }
  // The list is read 64 entries at a time into one register per lane; the
  // chunks then take their window ids from it with a lane permute (a chunk's
  // windows never straddle two batches: 64 sb slots is a multiple of 32), so
  // the gathers do not wait on a dependent global load.
  int lent = -1;
  auto entry = [&](int64_t w) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_bpermute((int)(w & 63) << 2, lent);
  };
  auto load = [&](C& ch, int ci) __attribute__((always_inline)) {
    const int64_t ga = (int64_t)ci * 32 + 8 * (kl >> 2);
    const int ja = entry(ga / sb);
    const int64_t kka = ga % sb + (kl & 3);
    load_rows<T>(ch.x, static_cast<const T*>(p.qblk), ja, kka, h, H, sb, g);
    load_rows<T>(ch.y, static_cast<const T*>(p.doblk), ja, kka, h, H, sb, g);
    const int64_t gv = (int64_t)ci * 32 + 8 * g;
    ch.jv = entry(gv / sb);
    ch.kkv0 = (int)(gv % sb);
    if constexpr (sizeof(T) == 2) {
      transpose_chunk(ch.y, ch.t, sel_slab[wv][0], kl, g);
      transpose_chunk(ch.x, ch.u, sel_slab[wv][1], kl, g);
    } else {
      load_trans<T>(ch.t, static_cast<const T*>(p.doT), ch.jv, ch.kkv0, h, H, sb, kl);
      load_trans<T>(ch.u, static_cast<const T*>(p.qT), ch.jv, ch.kkv0, h, H, sb, kl);
    }
    const int64_t lrow = ((int64_t)(ch.jv < 0 ? 0 : ch.jv) * H + h) * sb + ch.kkv0;
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(p.l2blk + lrow + e);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(p.dblk + lrow + e);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        ch.l2[e + x] = ch.jv < 0 ? INFINITY : l4[x];
        ch.dd[e + x] = ch.jv < 0 ? 0.0f : d4[x];
      }
    }
  };
  auto process = [&](const C& ch) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const f32x4 s0 = F::qk(ch.x[0], kfs[b]), s1 = F::qk(ch.x[1], kfs[b]);
      const f32x4 d0 = F::qk(ch.y[0], vfs[b]), d1 = F::qk(ch.y[1], vfs[b]);
      f32x4 p0, p1, ds0, ds1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p0[e] = fast_exp2(fmaf(s0[e], c, -ch.l2[e]));
        p1[e] = fast_exp2(fmaf(s1[e], c, -ch.l2[4 + e]));
        ds0[e] = p0[e] * (d0[e] - ch.dd[e]);
        ds1[e] = p1[e] * (d1[e] - ch.dd[4 + e]);
      }
      F::pv(ch.t, p0, p1, dv[b]);
      F::pv(ch.u, ds0, ds1, dk[b]);
    }
  };
  // One chunk in registers at a time (148 VGPRs, three waves per SIMD): the
  // other waves' gathers hide each wave's load latency; two chunks in flight
  // per wave would cost the occupancy (one wave per SIMD, 45 % slower).
  int batch = -1;
  for (int ci = 0; ci < n_chunks; ++ci) {
    const int b = (int)(((int64_t)ci * 32 / sb) >> 6);
    if (b != batch) {  // uniform across the wave
      batch = b;
      const int64_t w = (int64_t)b * 64 + lane;
      lent = w < n_list ? list[w] : -1;
    }
    C A;
    load(A, ci);
    process(A);
  }

#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int kk = (KB * kg + b) * 16 + kl;
    if (kk >= s2) continue;
    const int64_t tok = window_token(geo, win, kk);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // + the pooled rows' gradients / s^2 (the pooling backward)
      const int64_t pr = (win * H + h) * kHeadDim + 16 * m + 4 * g;
      const f32x4 pk = *reinterpret_cast<const f32x4*>(p.dkc + pr);
      const f32x4 pv = *reinterpret_cast<const f32x4*>(p.dvc + pr);
      f32x4* k4 = reinterpret_cast<f32x4*>(p.dk + (tok * H + h) * kHeadDim + 16 * m + 4 * g);
      f32x4* v4 = reinterpret_cast<f32x4*>(p.dv + (tok * H + h) * kHeadDim + 16 * m + 4 * g);
      *k4 = *k4 + dk[b][m] * p.scale + pk * p.inv_area;
      *v4 = *v4 + dv[b][m] + pv * p.inv_area;
    }
  }
}

template <typename T, int QB>
static void launch_sel_pair(const SelBwdParams& p, unsigned blocks, hipStream_t stream) {
  hipLaunchKernelGGL((sel_dq_kernel<T, QB>), dim3(blocks), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((sel_dkdv_kernel<T, QB>), dim3(blocks), dim3(256), 0, stream, p);
}
template <typename T>
static void launch_sel_t(const SelBwdParams& p, int n_sub, unsigned blocks, hipStream_t stream) {
  if (n_sub == 1) launch_sel_pair<T, 1>(p, blocks, stream);
  else if (n_sub == 2) launch_sel_pair<T, 2>(p, blocks, stream);
  else if (n_sub == 3) launch_sel_pair<T, 3>(p, blocks, stream);
  else launch_sel_pair<T, 4>(p, blocks, stream);
}

hipError_t launch_sel_bwd(int dtype, const SelBwdParams& p, hipStream_t stream) {
  // one wave per (window, head) serves all of the window's blocks of 16
  const int n_sub = (int)((p.g.pool * p.g.pool + 15) / 16);
  const int64_t items = p.g.n_windows * p.g.n_heads;
  if (items == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  if (dtype == kBF16) launch_sel_t<__bf16>(p, n_sub, blocks, stream);
  else launch_sel_t<float>(p, n_sub, blocks, stream);
  return hipGetLastError();
}

}  // namespace gsa
