// Matrix-core fragments of the selection kernels (gfx950,
// v_mfma_f32_16x16x32_bf16 / 16x16x4f32), shared by the forward and backward
// gathers.  A chunk is 32 key (or query) slots; lane l = 16 g + ql holds
// fragment row ql and slots 8g .. 8g+7 of the chunk:
//   qk(rows, frag)      S^T[16 slots x 16 frag rows] for one tile tau of the
//                       chunk, A row ql of tile tau = slot 8 (ql / 4) + 4 tau + ql % 4,
//                       so element e of tile tau is slot 8 g + 4 tau + e;
//   pv(trans, p0, p1)   acc^T[16 channels x 16 frag rows] per block m of 16
//                       channels += trans . P over the chunk's slots, with the
//                       lane's own 8 values as the P operand.
#pragma once

#include "flash_frag.h"
#include "gsa_device.h"

namespace gsa {

template <typename T>
struct Frag16;

template <>
struct Frag16<__bf16> {
  struct Q {
    bf16x8 v[2];
  };
  // lane (q, g) holds d = 16 g + 8 ks + [0, 8)
  __device__ static Q load_q(const __bf16* row, int g) {
    Q f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (row) {
        f.v[ks] = *reinterpret_cast<const bf16x8*>(row + 16 * g + 8 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[ks][e] = (__bf16)0.0f;
      }
    }
    return f;
  }
  __device__ static float q_dot(const Q& f, const __bf16* w, int g) {
    float z = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) z += (float)f.v[ks][e] * (float)w[16 * g + 8 * ks + e];
    return z;
  }
  __device__ static f32x4 qk(const uint4 (&k)[2], const Q& q) {
    f32x4 s = {0, 0, 0, 0};
    s = mfma16(__builtin_bit_cast(bf16x8, k[0]), q.v[0], s);
    s = mfma16(__builtin_bit_cast(bf16x8, k[1]), q.v[1], s);
    return s;
  }
  __device__ static void pv(const uint4 (&v)[4][1], const f32x4& p0, const f32x4& p1, f32x4 o[4]) {
    bf16x8 b = {(__bf16)p0[0], (__bf16)p0[1], (__bf16)p0[2], (__bf16)p0[3],
                (__bf16)p1[0], (__bf16)p1[1], (__bf16)p1[2], (__bf16)p1[3]};
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = mfma16(__builtin_bit_cast(bf16x8, v[m][0]), b, o[m]);
  }
};

template <>
struct Frag16<float> {
  struct Q {
    float v[16];
  };
  // lane (q, g) holds d = 16 g + i; MFMA i contracts that d.
  __device__ static Q load_q(const float* row, int g) {
    Q f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 x = row ? *reinterpret_cast<const f32x4*>(row + 16 * g + 4 * i) : f32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) f.v[4 * i + e] = x[e];
    }
    return f;
  }
  __device__ static float q_dot(const Q& f, const float* w, int g) {
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) z += f.v[i] * w[16 * g + i];
    return z;
  }
  __device__ static f32x4 qk(const uint4 (&k)[4], const Q& q) {
    f32x4 s = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 a = __builtin_bit_cast(f32x4, k[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma16(a[e], q.v[4 * i + e], s);
    }
    return s;
  }
  // slot 8g + 4 tau + e <-> S_tau[e] (B) and v element 4 tau + e (A)
  __device__ static void pv(const uint4 (&v)[4][2], const f32x4& p0, const f32x4& p1, f32x4 o[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f32x4 lo = __builtin_bit_cast(f32x4, v[m][0]);
      f32x4 hi = __builtin_bit_cast(f32x4, v[m][1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[m] = mfma16(lo[e], p0[e], o[m]);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[m] = mfma16(hi[e], p1[e], o[m]);
    }
  }
};

// bf16: the transposed operand of a chunk (slots contiguous per channel, as a
// product contracting over the slots needs) is built from its rows, already in
// registers, through a wave-private LDS slab instead of a gather of a
// transposed copy.  Lane (ql, g) holds rows 8 (ql/4) + 4 tau + ql%4 (tau = 0,
// 1), channels 16 g .. 16 g + 15; the transposing read (ds_read_b64_tr_b16: within a 16-lane group, lane
// i gets element i%4 of the 8-byte chunks addressed by lanes 4e + i/4) hands
// lane i of group g channel 16 m + i of rows 8 g .. 8 g + 7 when lane j of the
// group addresses row 8 g + j/4 (then + 4), channels 16 m + 4 (j%4).
constexpr int kSlabStride = kHeadDim + 8;  // bf16 per slab row: 16-byte aligned rows, shifted banks
constexpr int kSlabElems = 32 * kSlabStride;
__device__ __forceinline__ void transpose_chunk(const uint4 (&rows)[2][2], uint4 (&tr)[4][1], __bf16* slab, int ql,
                                                int g) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      st16(slab + (8 * (ql >> 2) + 4 * tau + (ql & 3)) * kSlabStride + 16 * g + 8 * x, rows[tau][x]);
  // a wave's LDS operations complete in order; the wait keeps the compiler from
  // moving the transposing reads above the stores
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  const __bf16* r0 = slab + (8 * g + (ql >> 2)) * kSlabStride + 4 * (ql & 3);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const bf16x4 lo = lds_read_tr16(r0 + 16 * m);
    const bf16x4 hi = lds_read_tr16(r0 + 4 * kSlabStride + 16 * m);
    tr[m][0] = __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// Window id of top-k entry t, from the two registers holding entries lane and
// lane+64.  Entries past k, negative or not below M' read as -1 (skipped).
__device__ __forceinline__ int topk_entry(int tr0, int tr1, int t, int K, int64_t n_windows) {
  int a = __builtin_amdgcn_ds_bpermute((t & 63) << 2, tr0);
  int b = __builtin_amdgcn_ds_bpermute((t & 63) << 2, tr1);
  int j = t < 64 ? a : b;
  return (t >= K || j < 0 || j >= n_windows) ? -1 : j;
}

}  // namespace gsa
