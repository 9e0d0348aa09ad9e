// Tiles and matrix-core fragments shared by the forward and backward
// attention kernels (gfx950, v_mfma_f32_32x32x16_bf16 / _f32).
//
// A tile is 32 rows (keys, or queries in the backward key-side pass) of one
// head, staged in LDS and read by the fragments below:
//   qk(tile, frag)   S^T[32 tile rows x 32 frag rows] = tile . frag^T over d;
//                    lane l holds fragment row l%32 and tile rows
//                    8*(i/4) + 4*(l/32) + i%4 in element i;
//   pv(tile, P, acc) acc^T[64 d x 32 frag rows] += tile^T . P^T, contracting
//                    the tile rows; the P operand of a lane is its own 16
//                    S^T-layout values (the contraction order is permuted to
//                    match, so no shuffles are needed).
#pragma once

#include <math.h>

#include "gsa_device.h"
#include "gsa_kernels.h"

namespace gsa {

constexpr int kKT = 32;              // keys per tile
// LDS tile of 32 keys.
// bf16: K and V are stored row-major (one 128-byte row per key) with the
// 16-byte chunks of row r permuted as c -> c ^ swz(r), no padding.  Two rows
// share one 256-byte line of the 64 LDS banks (row parity picks the half), so
// swz(r) = bit-reverse of (r >> 1) % 8: the same chunk read by 16 consecutive
// rows (the K operand) lands on 16 different 16-byte bank groups, and the
// transposing V reads (4 rows x 4 chunks per 32 lanes) see rows r and r + 2
// in different 64-byte halves.
// fp32: K rows padded by 16 bytes; V stored transposed (channel rows) since
// there is no transposing read for 32-bit data.
template <typename T>
struct Tile;

template <>
struct Tile<__bf16> {
  static constexpr int VE = 8;
  static constexpr int K_ELEMS = kKT * kHeadDim;
  static constexpr int V_ELEMS = kKT * kHeadDim;
  static constexpr int BYTES = (K_ELEMS + V_ELEMS) * 2;
  // element offset of 16-byte chunk c of key row `key`
  __device__ static int swz(int key) {
    const int x = (key >> 1) & 7;
    return ((x & 1) << 2) | (x & 2) | (x >> 2);
  }
  __device__ static int chunk(int key, int c) { return key * kHeadDim + ((c ^ swz(key)) << 3); }
};

template <>
struct Tile<float> {
  static constexpr int VE = 4;
  static constexpr int KSTRIDE = kHeadDim + VE;
  static constexpr int VSTRIDE = kKT + 4;
  static constexpr int K_ELEMS = kKT * KSTRIDE;
  static constexpr int V_ELEMS = kHeadDim * VSTRIDE;
  static constexpr int BYTES = (K_ELEMS + V_ELEMS) * 4;
};

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i%4 of the 8-byte chunks addressed by lanes 4e + i/4 (e = 0..3) of its group.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// ---- matrix-core fragments (32x32 family) ----------------------------------
template <typename T>
struct Frag32;

template <>
struct Frag32<__bf16> {
  using TL = Tile<__bf16>;
  struct Q {
    bf16x8 v[4];
  };
  // Q^T operand: lane (q, hf) holds d = 32*hf + 8*ks + [0, 8) for ks = 0..3.
  __device__ static Q load_q(const __bf16* row, int hf) {
    Q f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (row) {
        f.v[ks] = *reinterpret_cast<const bf16x8*>(row + 32 * hf + 8 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[ks][e] = (__bf16)0.0f;
      }
    }
    return f;
  }
  // S^T = K Q^T over d (the same d order on both operands).
  __device__ static f32x16 qk(const __bf16* kt, int r, int hf, const Q& q) {
    bf16x8 a[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(kt + TL::chunk(r, 4 * hf + ks));
    f32x16 s = {};
    // raised wave priority while the matrix-core ops issue, so a wave that has
    // them ready goes first and the others' VALU work fills in behind
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s = mfma32(a[ks], q.v[ks], s);
    __builtin_amdgcn_s_setprio(0);
    return s;
  }
  // P operand: the bf16 values of the lane's S^T elements; the row sum adds
  // exactly these rounded values, so numerator and denominator agree.
  struct P {
    bf16x8 v[2];
  };
  __device__ static P to_p(const f32x16& p, float& psum) {
    P r;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) r.v[m][e] = (__bf16)p[8 * m + e];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) psum = add_pair(bf16x2{r.v[m][2 * e], r.v[m][2 * e + 1]}, psum);
    return r;
  }
  // O^T += V^T P^T.  The P operand of lane (q, hf) for key group m is its own
  // S^T elements 8m..8m+7, i.e. keys 16m + 8*(e/4) + 4*hf + e%4; the V^T
  // operand of lane (dv, hf) needs the same keys for channel dv.  With V rows
  // in LDS, lane j of each 16-lane group G addresses key 16m + 8c + 4(G/2) + j/4,
  // channels 32n + 16(G%2) + 4(j%4) .. +3; the transposing read then hands
  // lane l exactly V[16m + 8c + 4hf + e'][32n + l%32] for e' = 0..3.
  __device__ static void pv(const __bf16* vt, int lane, const P& p, f32x16 o[2]) {
    __builtin_amdgcn_s_setprio(1);
    const int G = lane >> 4, j = lane & 15;
    const int krow = 4 * (G >> 1) + (j >> 2);      // + 16m + 8c
    const int dv = 16 * (G & 1) + 4 * (j & 3);     // + 32n
    // chunk swizzles of the rows this lane reads (16m + 8c + krow: 16m keeps
    // swz, +8 flips its low bit)
    const int sw_lo = TL::swz(krow), sw_hi = TL::swz(krow + 8);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int off_lo = (((4 * n + (dv >> 3)) ^ sw_lo) << 3) + (dv & 7);
        const int off_hi = (((4 * n + (dv >> 3)) ^ sw_hi) << 3) + (dv & 7);
        const __bf16* q0 = vt + (16 * m + krow) * kHeadDim;
        bf16x4 lo = lds_read_tr16(q0 + off_lo);
        bf16x4 hi = lds_read_tr16(q0 + 8 * kHeadDim + off_hi);
        bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[n] = mfma32(a, p.v[m], o[n]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
};

template <>
struct Frag32<float> {
  using TL = Tile<float>;
  struct Q {
    float v[32];
  };
  // lane (q, hf) holds d = 32*hf + i for i = 0..31; MFMA i contracts that d.
  __device__ static Q load_q(const float* row, int hf) {
    Q f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 x = row ? *reinterpret_cast<const f32x4*>(row + 32 * hf + 4 * i) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) f.v[4 * i + e] = x[e];
    }
    return f;
  }
  __device__ static f32x16 qk(const float* kt, int r, int hf, const Q& q) {
    const float* base = kt + r * TL::KSTRIDE + 32 * hf;
    f32x16 s = {};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4 a = *reinterpret_cast<const f32x4*>(base + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma32(a[e], q.v[4 * i + e], s);
    }
    return s;
  }
  struct P {
    f32x16 v;
  };
  __device__ static P to_p(const f32x16& p, float& psum) {
#pragma unroll
    for (int i = 0; i < 16; ++i) psum += p[i];
    return P{p};
  }
  // element i of lane (q, hf) is key 8*(i/4) + 4*hf + i%4; one MFMA per i.
  __device__ static void pv(const float* vt, int lane, const P& p, f32x16 o[2]) {
    const int r = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 x = *reinterpret_cast<const f32x4*>(vt + (32 * n + r) * TL::VSTRIDE + 8 * a4 + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[n] = mfma32(x[e], p.v[4 * a4 + e], o[n]);
      }
    }
  }
};

// ---- cooperative K/V tile staging ------------------------------------------
// A tile is rows key0 .. key0+31 of one head, read with buffer loads whose
// (scalar) base is the tile's first row: the per-thread byte offsets are the
// same for every tile, and rows from `valid` (0..32) on lie beyond the
// buffer's byte limit, which the hardware returns as zeros (those keys are
// masked: -inf scores, weight 0).  The limit is 32-bit scalar arithmetic
// (32 rows of a token row stride).
template <typename T>
__device__ __amdgpu_buffer_rsrc_t tile_rsrc(const T* X, int64_t stride, int64_t hoff, int64_t key0, int valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(X + key0 * stride + hoff), (short)0,
                                           valid * (int)(stride * (int64_t)sizeof(T)), 0x00020000);
}

template <typename T, int NT>
struct TileLoader {
  using TL = Tile<T>;
  static constexpr int VE = TL::VE;
  static constexpr int VPR = kHeadDim / VE;
  static constexpr int NV = kKT * VPR / NT;
  static_assert(NV >= 1 && NV * NT == kKT * VPR, "tile must split evenly over the workgroup");
  uint4 kr[NV], vr[NV];

  // The loads are unconditional, so the compiler can count the loads in
  // flight and wait only for the oldest tile.
  static __device__ int chunk_offset(int64_t stride, int idx) {
    const int key = idx / VPR, c = idx % VPR;
    return (int)(((int64_t)key * stride + c * VE) * (int64_t)sizeof(T));
  }
  static __device__ uint4 buf16(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
  __device__ void load(const T* K, const T* V, int64_t stride, int64_t hoff, int64_t key0, int valid,
                       int tid) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(K, stride, hoff, key0, valid);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(V, stride, hoff, key0, valid);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int off = chunk_offset(stride, tid + i * NT);
      kr[i] = buf16(rk, off);
      vr[i] = buf16(rv, off);
    }
  }
  // K only (score-only sweep)
  __device__ void load_k(const T* K, int64_t stride, int64_t hoff, int64_t key0, int valid, int tid) {
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(K, stride, hoff, key0, valid);
#pragma unroll
    for (int i = 0; i < NV; ++i) kr[i] = buf16(rk, chunk_offset(stride, tid + i * NT));
  }
  __device__ void store_k(T* kt, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int idx = tid + i * NT;
      int key = idx / VPR, c = idx % VPR;
      if constexpr (sizeof(T) == 2)
        st16(kt + TL::chunk(key, c), kr[i]);
      else
        st16(kt + key * TL::KSTRIDE + c * VE, kr[i]);
    }
  }
  __device__ void store(T* kt, T* vt, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int idx = tid + i * NT;
      int key = idx / VPR, c = idx % VPR;
      if constexpr (sizeof(T) == 2) {
        st16(kt + TL::chunk(key, c), kr[i]);
        st16(vt + TL::chunk(key, c), vr[i]);
      } else {
        st16(kt + key * TL::KSTRIDE + c * VE, kr[i]);
        const T* x = reinterpret_cast<const T*>(&vr[i]);
#pragma unroll
        for (int e = 0; e < VE; ++e) vt[(c * VE + e) * TL::VSTRIDE + key] = x[e];
      }
    }
  }
};

// Excluded keys of a 32-key tile as a bit mask (bit i = key key0 + i),
// uniform across the wave, for parameter blocks holding the excluded key
// ranges n_excl, excl_beg, excl_end (FlashParams, TopkParams).  Tiles are
// visited in increasing key order, so a cursor passes the ranges that end
// before the tile once and a tile usually tests no range at all (scalar
// 32-bit arithmetic: key counts are int32).
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

}  // namespace gsa
