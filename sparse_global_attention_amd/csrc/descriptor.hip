// Key/value set of FlashVGGT descriptor attention (Paper-Notes page "FlashVGGT:
// Efficient and Scalable Visual Geometry Transformers with Compressed
// Descriptor Attention", section "关键设计": each frame's spatial tokens are
// bilinearly resampled from (h, w) to (h/r, w/r); section "关键发现": the
// auxiliary descriptor tokens are the first frame's full tokens, keyframes
// and camera tokens).
//
// Rows of the set, in order: the descriptors of every frame (frame-major,
// row-major), every token of frame 0 and of each keyframe, then the special
// tokens of every other frame.  HBM-bound: one thread owns one (row, head,
// 16-byte channel chunk), so a token row is read and written with
// consecutive 16-byte accesses.
//
// A descriptor samples the image at ((y + 0.5) r - 0.5, (x + 0.5) r - 0.5)
// (half-pixel centres).  With an integer r that point is an integer or a
// half-integer, so each row and column weight is 1, 1/2 or 0 and every
// weighted value is exact; the four corners are added in float in the order
// (y0,x0), (y0,x1), (y1,x0), (y1,x1) with explicitly rounded operations and
// the sum is rounded to the dtype, so the set is reproducible bit for bit.
#include "gsa_device.h"
#include "gsa_kernels.h"

namespace gsa {

template <typename T>
__global__ __launch_bounds__(256) void descriptor_kernel(DescParams p) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int CPH = kHeadDim / VE;
  const Geometry& g = p.g;
  const int tensor = blockIdx.y;
  const int64_t per_row = g.n_heads * CPH;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= p.n_set * per_row) return;
  const int64_t row = gid / per_row;
  const int64_t rem = gid - row * per_row;
  const int64_t col = (rem / CPH) * kHeadDim + (rem % CPH) * VE;
  const int64_t stride = g.n_heads * kHeadDim;
  const T* src = static_cast<const T*>(p.src[tensor]);
  T* dst = static_cast<T*>(p.dst[tensor]) + row * stride + col;

  if (row >= p.n_desc) {
    // auxiliary token: a plain copy of its row
    int64_t a = row - p.n_desc, tok;
    const int64_t full_rows = (int64_t)p.n_full * g.tf;
    if (a < full_rows) {
      tok = (int64_t)p.full[a / g.tf] * g.tf + a % g.tf;
    } else {
      a -= full_rows;
      // the (a / P)-th frame outside the full ones (full_sorted ascending)
      int64_t f = a / g.n_special;
      for (int i = 0; i < p.n_full; ++i) f += p.full_sorted[i] <= f ? 1 : 0;
      tok = f * g.tf + a % g.n_special;
    }
    st16(dst, ld16(src + tok * stride + col));
    return;
  }

  const int r = p.r;
  const int64_t dh = g.grid_h / r, dw = g.grid_w / r;
  const int64_t f = row / (dh * dw);
  const int y = (int)((row / dw) % dh), x = (int)(row % dw);
  // twice the sample coordinate: (2y + 1) r - 1 >= 0
  const int ny = (2 * y + 1) * r - 1, nx = (2 * x + 1) * r - 1;
  const int y0 = ny >> 1, x0 = nx >> 1;
  const int y1 = min(y0 + 1, (int)g.grid_h - 1), x1 = min(x0 + 1, (int)g.grid_w - 1);
  const float fy = (ny & 1) ? 0.5f : 0.0f, fx = (nx & 1) ? 0.5f : 0.0f;
  const float wy[2] = {1.0f - fy, fy}, wx[2] = {1.0f - fx, fx};
  const int ys[2] = {y0, y1}, xs[2] = {x0, x1};
  const T* base = src + (f * g.tf + g.n_special) * stride + col;

  uint4 c[4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) c[2 * a + b] = ld16(base + ((int64_t)ys[a] * g.grid_w + xs[b]) * stride);
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float w = __fmul_rn(wy[a], wx[b]);
      const T* v = reinterpret_cast<const T*>(&c[2 * a + b]);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = __fadd_rn(acc[e], __fmul_rn(w, to_f32(v[e])));
    }
  T out[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) out[e] = from_f32<T>(acc[e]);
  st16(dst, *reinterpret_cast<const uint4*>(out));
}

hipError_t launch_descriptor(int dtype, const DescParams& p, hipStream_t stream) {
  const int ve = dtype == kBF16 ? 8 : 4;
  const int64_t threads = p.n_set * p.g.n_heads * (kHeadDim / ve);
  if (threads == 0) return hipSuccess;
  dim3 grid((unsigned)((threads + 255) / 256), 2u);
  if (dtype == kBF16)
    hipLaunchKernelGGL(descriptor_kernel<__bf16>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(descriptor_kernel<float>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gsa
