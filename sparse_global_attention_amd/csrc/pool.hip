// s x s average pooling of the image Q/K/V (Paper-Notes page "Speed3R: Sparse
// Feed-forward 3D Reconstruction Models", section "压缩分支": Q_comp, K_comp,
// V_comp from s x s non-overlapping average pooling, M' = M_img / s^2).
//
// HBM-bound.  One thread owns one (window, head, 16-byte channel chunk): the
// 128 threads of a 2 KB token row (16 heads x 64 channels of bf16) read it
// with consecutive 16-byte loads.  The s^2 window values are summed in fp32
// in row-major order from +0, multiplied by 1/s^2 and rounded to the dtype,
// so the pooled tensors are reproducible bit for bit.
//
// While a tensor's windows are in registers the kernel can also write the
// copies the selection kernels gather from, one contiguous block per
// (window, head):
//   rows  [M'][H][sb][d]  rows in window-local order (zero padded to sb tokens),
//                         the layout of a score-product operand;
//   trans [M'][H][d][sb]  transposed (tokens contiguous per channel), the
//                         layout of an operand that contracts over tokens.
// The fp32 forward uses V transposed (bf16 transposes V in LDS and needs no
// copy); the backward uses Q, K and V rows (fp32 also Q and K transposed).
#include <type_traits>

#include "gsa_device.h"
#include "gsa_kernels.h"

namespace gsa {

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  constexpr int VE = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int CPH = kHeadDim / VE;        // chunks per head row
  const Geometry& g = p.g;
  const int tensor = p.first_tensor + blockIdx.y;
  const int64_t per_window = g.n_heads * CPH;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= g.n_windows * per_window) return;
  const int64_t j = gid / per_window;
  const int64_t rem = gid - j * per_window;
  const int64_t h = rem / CPH;
  const int c = (int)(rem - h * CPH);
  const int64_t row = g.n_heads * kHeadDim;
  const int64_t col = h * kHeadDim + c * VE;
  const T* src = static_cast<const T*>(p.src[tensor]);
  const int s2 = (int)(g.pool * g.pool);

  T* kb = p.rows[tensor] ? static_cast<T*>(p.rows[tensor]) + (j * g.n_heads + h) * g.sb * kHeadDim : nullptr;
  T* vb = p.trans[tensor] ? static_cast<T*>(p.trans[tensor]) + (j * g.n_heads + h) * kHeadDim * g.sb : nullptr;

  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.0f;

  // Walk the window's keys KS at a time (sb is a multiple of 8): 16 when sb
  // allows, so each channel's 32-byte row of the transposed copy is stored
  // whole (two halves stored one pass apart were evicted from L2 separately:
  // the copy's HBM writes doubled).
  auto walk = [&](auto ks_tag) __attribute__((always_inline)) {
    constexpr int KS = decltype(ks_tag)::value;
    for (int k0 = 0; k0 < g.sb; k0 += KS) {
      uint4 chunk[KS];
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const int kk = k0 + t;
        chunk[t] = kk < s2 ? ld16(src + window_token(g, j, kk) * row + col) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        if (k0 + t < s2) {
          const T* x = reinterpret_cast<const T*>(&chunk[t]);
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[e] += to_f32(x[e]);
        }
      }
      if (kb) {
#pragma unroll
        for (int t = 0; t < KS; ++t) st16(kb + (k0 + t) * kHeadDim + c * VE, chunk[t]);
      }
      if (vb) {
        // channel c*VE+e gets keys k0 .. k0+KS-1: KS consecutive elements
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          T colk[KS];
#pragma unroll
          for (int t = 0; t < KS; ++t) colk[t] = reinterpret_cast<const T*>(&chunk[t])[e];
          T* d = vb + (c * VE + e) * g.sb + k0;
#pragma unroll
          for (int q = 0; q < KS * (int)sizeof(T) / 16; ++q)
            st16(d + q * VE, *reinterpret_cast<const uint4*>(colk + q * VE));
        }
      }
    }
  };
  if (g.sb % 16 == 0)
    walk(std::integral_constant<int, 16>{});
  else
    walk(std::integral_constant<int, 8>{});

  T* dst = static_cast<T*>(p.dst[tensor]);
  if (dst) {
    T out[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) out[e] = from_f32<T>(acc[e] * p.inv_area);
    st16(dst + (j * g.n_heads + h) * kHeadDim + c * VE, *reinterpret_cast<const uint4*>(out));
  }
}

hipError_t launch_pool(int dtype, const PoolParams& p, int n_tensors, hipStream_t stream) {
  const int ve = dtype == kBF16 ? 8 : 4;
  const int64_t threads = p.g.n_windows * p.g.n_heads * (kHeadDim / ve);
  if (threads == 0 || n_tensors == 0) return hipSuccess;
  dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_tensors);
  if (dtype == kBF16)
    hipLaunchKernelGGL(pool_kernel<__bf16>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(pool_kernel<float>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gsa
