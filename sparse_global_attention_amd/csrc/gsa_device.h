// Device-side building blocks shared by the libgsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsa {

constexpr int kHeadDim = 64;  // d; the only head dimension the kernels are built for

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// log2(e): softmax exponentials are evaluated as exp2 of log2e-scaled logits.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Value of `x` held by lane (lane ^ mask) of the same wave.
__device__ __forceinline__ float xor_lane(float x, int mask) {
  int src = (lane_id() ^ mask) << 2;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x)));
}
__device__ __forceinline__ int xor_lane(int x, int mask) {
  int src = (lane_id() ^ mask) << 2;
  return __builtin_amdgcn_ds_bpermute(src, x);
}

// x + (x of lane l ^ 32), through v_permlane32_swap: a VALU lane exchange
// between the two halves of the wave, no LDS round trip.  Each lane ends up
// with its own value and its partner's (in some order), so the sum does not
// depend on which is which.  Every lane of the wave must be active.
__device__ __forceinline__ int sum_halves(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (int)(r[0] + r[1]);
}

// max(x, x of lane l ^ 32) and max(x, x of lane l ^ 16) with the VALU lane
// swaps (v_permlane32_swap: the two 32-lane halves; v_permlane16_swap: the
// odd and even 16-lane rows): each lane gets its own value and its partner's,
// in some order, so the max does not depend on which is which.  Every lane of
// the wave must be active.
__device__ __forceinline__ float max_halves32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Global-to-LDS load of 16 bytes per lane (buffer load with the LDS flag):
// lane l's bytes at byte offset `voff` of the buffer land at lds + 16 l;
// lanes past the buffer's byte limit write zeros.  `lds` must be the same
// for the whole wave.  Completion is counted by vmcnt like other loads.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// fences global memory, which makes every wave wait for its in-flight global
// loads (the tile prefetch) at the barrier; this one does not.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw hardware exp2 (v_exp_f32): denormal results flush to zero, which only
// drops softmax weights below 2^-126.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Three-way max.  On values the compiler knows to be canonical (results of
// ordinary float arithmetic) this lowers to a bare v_max3_f32.
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// a + x.lo + x.hi for a pair of bf16 values (v_dot2c_f32_bf16 against 1.0).
__device__ __forceinline__ float add_pair(bf16x2 x, float a) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(x, one, a, false);
}

// ---- MFMA wrappers (gfx950) ----------------------------------------------
// 32x32 family: D[32x32] += A[32xK] B[Kx32]; lane l holds A row l%32, B column
// l%32, and D column l%32 with rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// 16x16 family: lane l holds A row l%16, B column l%16, and D column l%16
// with rows 4*(l/16) + r for r = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- element conversions -----------------------------------------------------
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

// 16-byte vector load/store through uint4.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// ---- XCD-aware block order -------------------------------------------------
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2.  Remap so that each XCD receives a contiguous range of
// logical work ids: neighbouring work items (which share K/V tiles) then run
// on the same L2.  The map is a bijection on [0, n).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t n) {
  constexpr int64_t kXcd = 8;
  int64_t full = n / kXcd * kXcd;
  if (bid >= full) return bid;
  return (bid % kXcd) * (full / kXcd) + bid / kXcd;
}

}  // namespace gsa
