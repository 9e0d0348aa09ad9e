// Selection-branch attention and the upsample + gate epilogue.
//
// Paper-Notes page "Speed3R: Sparse Feed-forward 3D Reconstruction Models":
//  * section "选择分支": every image query attends the full-resolution K/V of
//    its window's top-k windows; the s^2 queries of one window share one KV
//    set, so one wavefront serves one (window, head) and gathers each selected
//    window once;
//  * section "Speed3R-VGGT 适配": optional fixed context (all tokens of the
//    reference frames) joins the same softmax; its part is computed by the
//    dense flash kernel as a partial (o, lse) and merged here;
//  * section "压缩分支" (nearest-neighbour upsampling) and section "门控聚合"
//    (g = sigmoid(W_g q), O = g O_comp + (1 - g) O_sel): fused epilogue.
//
// Gather-bound.  The K and V rows of a selected (window, head) are read
// straight from the token layout.  K lands directly in matrix-core operand
// layout (a lane reads 32 bytes of one 128-byte row).  V's product contracts
// over the slots, so its operand needs them contiguous per channel: bf16 V
// rows go by global-to-LDS loads into a wave-private slab and are read back
// transposed (ds_read_b64_tr_b16); fp32, which has no such read, gathers V
// from the transposed block [d][sb] the pooling pass writes.  No barriers:
// waves are independent.
// A chunk is 32 key slots (two windows at s = 4); the next chunk's loads are
// issued before the current chunk's matrix-core work.
//   S^T[32 slots x 16 q] : 2 tiles x 2 x v_mfma_f32_16x16x32_bf16 (K = d)
//   O^T[64 dv x 16 q]   += V^T P^T : 4 x v_mfma_f32_16x16x32_bf16 (K = 32 slots)
// Lane l = 16 g + ql holds query ql and slots 8g..8g+7 of the chunk.
#include <math.h>

#include "gsa_device.h"
#include "gsa_kernels.h"
#include "select_frag.h"

namespace gsa {

template <typename T>
struct SelChunk {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int KV = 16 / VE;  // 16-byte loads per 16 channels of a K row
  static constexpr int VV = 8 / VE;   // fp32: 16-byte loads per 8 slots of a V^T row
  static constexpr bool kSlabV = sizeof(T) == 2;  // bf16: V rows in an LDS slab
  uint4 k[2][KV];
  uint4 v[kSlabV ? 1 : 4][kSlabV ? 1 : VV];  // fp32: the V^T operand
  int jv;    // window of this lane's 8 S^T slots (-1: none)
  int kkv0;  // window-local key of the first of them
};

// Token row of the first (top-left) token of top-k entry t's window, from
// the two registers holding that of entries lane and lane+64 (-1: skipped).
__device__ __forceinline__ int64_t topk_base(int64_t tb0, int64_t tb1, int t) {
  const int lo0 = __builtin_amdgcn_ds_bpermute((t & 63) << 2, (int)tb0);
  const int hi0 = __builtin_amdgcn_ds_bpermute((t & 63) << 2, (int)(tb0 >> 32));
  const int lo1 = __builtin_amdgcn_ds_bpermute((t & 63) << 2, (int)tb1);
  const int hi1 = __builtin_amdgcn_ds_bpermute((t & 63) << 2, (int)(tb1 >> 32));
  const int lo = t < 64 ? lo0 : lo1, hi = t < 64 ? hi0 : hi1;
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Token row of window j's first token (-1 for a skipped entry).
__device__ __forceinline__ int64_t window_base(const Geometry& g, int j) {
  if (j < 0) return -1;
  const int64_t f = j / g.wpf, r = j - f * g.wpf;
  const int64_t wy = r / g.wx, wxx = r - wy * g.wx;
  return f * g.tf + g.n_special + wy * g.pool * g.grid_w + wxx * g.pool;
}

// bf16 V slab of a chunk: 32 rows (the chunk's slots) of 128 bytes, the
// 16-byte pieces of row r permuted (position x holds channels 8 (x ^ vswz(r))
// onward) so that the 16 rows one transposing read touches (32 bytes each)
// spread over the banks: rows 8g + {0, 2} and 8g + {1, 3} of the four lane
// groups g get four different 32-byte positions.
__device__ __forceinline__ int vswz(int r) { return (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1; }

// Slabs of chunks A and B, one per wave: two arrays, so that the compiler
// tells the reads of one from the global-to-LDS loads into the other.
__shared__ __attribute__((aligned(16))) __bf16 sel_vslab_a[4][32 * kHeadDim];
__shared__ __attribute__((aligned(16))) __bf16 sel_vslab_b[4][32 * kHeadDim];

__device__ __forceinline__ const void* wave_uniform(const void* ptr) {
  const uint64_t x = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

template <typename T>
__device__ __forceinline__ void load_chunk(SelChunk<T>& ch, const SelectParams& p, int64_t h, int c, int ql,
                                           int g, int tr0, int tr1, int64_t tb0, int64_t tb1, __bf16* vslab) {
  using C = SelChunk<T>;
  const int64_t sb = p.g.sb, H = p.g.n_heads;
  const int s = (int)p.g.pool, s2 = s * s;
  const T* K = static_cast<const T*>(p.k);
  const T* vblk = static_cast<const T*>(p.vblk);
  // Slot positions are multiples of 8 below k sb <= 8192 and sb is a multiple
  // of 8 up to 64, so entry and key follow from u = position / 8 < 1024 and
  // sb / 8 <= 8 by one multiply: (u * msb) >> 16 = u / (sb / 8) exactly.
  const int sb8 = (int)(sb >> 3), msb = (65536 + sb8 - 1) / sb8;
  // K operand: A-row ql of tile tau is slot 8*(ql/4) + 4*tau + ql%4 of the
  // chunk, i.e. key kka + 4 tau (row-major in the s x s window) of top-k
  // entry ea; keys past s^2 (padding slots) read the window's first token
  // instead -- their scores are masked below.
  const int ua = c * 4 + (ql >> 2), ea = (ua * msb) >> 16;
  const int64_t base = topk_base(tb0, tb1, ea);
  const int kka = 8 * (ua - ea * sb8) + (ql & 3);
  const int64_t row0 = base < 0 ? 0 : base;
  const int m16 = (65536 + s - 1) / s;  // kk / s = (kk * m16) >> 16 exactly for kk < 64, s <= 8
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const int kk = kka + 4 * tau < s2 ? kka + 4 * tau : 0;
    const int dy = (kk * m16) >> 16, dx = kk - dy * s;
    const T* kb = K + ((row0 + dy * p.g.grid_w + dx) * H + h) * kHeadDim + 16 * g;
#pragma unroll
    for (int x = 0; x < C::KV; ++x) ch.k[tau][x] = ld16(kb + x * C::VE);
  }
  // S^T rows of this lane: slots 8g .. 8g+7 of the chunk
  const int uv = c * 4 + g, ev = (uv * msb) >> 16;
  ch.jv = topk_entry(tr0, tr1, ev, p.topk, p.g.n_windows);
  ch.kkv0 = 8 * (uv - ev * sb8);
  if constexpr (C::kSlabV) {
    // V rows into the slab: load i fills rows 8i .. 8i+7 (the same window,
    // sb being a multiple of 8), lane l row 8i + l/8 at position l%8, from a
    // buffer whose base is the window's first row of this head; padding keys
    // and skipped entries read past the buffer's limit, i.e. zeros.
    const int lane = 16 * g + ql;
    const T* V = static_cast<const T*>(p.v);
    // The slab's previous chunk must be read out first: a global-to-LDS write
    // is not ordered after earlier LDS reads of the wave, so wait for them.
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = c * 4 + i, e = (u * msb) >> 16;
      const int64_t wb = topk_base(tb0, tb1, e);  // the same in every lane
      const int kk = 8 * (u - e * sb8) + (lane >> 3);
      const int dy = (kk * m16) >> 16, dx = kk - dy * s;
      const int r = 8 * i + (lane >> 3);
      const uint32_t voff = wb >= 0 && kk < s2
                                ? (uint32_t)((dy * p.g.grid_w + dx) * (int)H * kHeadDim + 8 * ((lane & 7) ^ vswz(r))) * 2u
                                : 0x80000000u;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<void*>(wave_uniform(V + ((wb < 0 ? 0 : wb) * H + h) * kHeadDim)), (short)0, 0x7fffffff,
          0x00020000);
      lds_load16(rs, vslab + 512 * i, (int)voff);
    }
  } else {
    // V^T operand: channel 16 m + ql of the same slots
    const T* vb = vblk + ((int64_t)(ch.jv < 0 ? 0 : ch.jv) * H + h) * kHeadDim * sb + ch.kkv0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int x = 0; x < C::VV; ++x) ch.v[m][x] = ld16(vb + (16 * m + ql) * sb + x * C::VE);
  }
}

// bf16: the V^T operand of a chunk from its slab.  Lane j of group g addresses
// row 8 g + j/4 (then + 4), channels 16 m + 4 (j%4) .. + 3; the transposing
// read hands lane i of the group channel 16 m + i of rows 8 g .. 8 g + 7
// (within a 16-lane group, lane i gets element i%4 of the 8-byte pieces
// addressed by lanes 4e + i/4).
__device__ __forceinline__ void slab_vt(const __bf16* vslab, int ql, int g, uint4 (&vt)[4][1]) {
  const int r = 8 * g + (ql >> 2), sw = vswz(r);  // row r + 4 has the same permutation
  // The second row's offset is kept opaque: folded into the read as an
  // immediate, the read loses the compiler's record of which slab it reads
  // and then waits for every global-to-LDS load in flight, the next chunk's
  // included.
  const int off_lo = r * kHeadDim + 4 * (ql & 1);
  int off_hi = off_lo + 4 * kHeadDim;
  asm volatile("" : "+v"(off_hi));
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int x = (2 * m + ((ql >> 1) & 1)) ^ sw;
    const bf16x4 lo = lds_read_tr16(vslab + off_lo + 8 * x);
    const bf16x4 hi = lds_read_tr16(vslab + off_hi + 8 * x);
    vt[m][0] = __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// bf16 with one block of 16 queries per window (s <= 4) fits in 128 VGPRs
// without spills: four waves per SIMD (the compiler alone picks more registers
// and three).
template <typename T, int QB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QB == 1 && sizeof(T) == 2 ? 4 : 1)))
void select_kernel(SelectParams p) {
  using F = Frag16<T>;
  const Geometry& geo = p.g;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  const int ql = lane & 15, g = lane >> 4;
  // One wave per (head, window, group of QB blocks of 16 of the window's s^2
  // queries); every gathered chunk serves the QB blocks from registers, so a
  // window's K/V is gathered once (QB = the number of blocks, 1 for s <= 4).
  // Head-major order: all waves in flight gather from the same head's K/V
  // blocks (M' x 4 KB), a working set the 256 MB Infinity Cache can hold a
  // large part of, instead of all heads' blocks at once.
  const int s2 = (int)(geo.pool * geo.pool);
  const int n_grp = ((s2 + 15) / 16 + QB - 1) / QB;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  if (item >= geo.n_windows * geo.n_heads * n_grp) return;
  const int qg = (int)(item % n_grp);
  const int64_t h = item / n_grp / geo.n_windows;
  const int64_t win = item / n_grp % geo.n_windows;
  const int64_t H = geo.n_heads;
  const int K = p.topk;
  const float c = p.scale_log2;

  const int32_t* trow = p.topk_idx + (win * geo.n_heads + h) * K;
  const int tr0 = lane < K ? trow[lane] : -1;
  const int tr1 = lane + 64 < K ? trow[lane + 64] : -1;
  // first token of each entry's window (entries outside [0, M') skipped)
  const int64_t tb0 = window_base(geo, tr0 < geo.n_windows ? tr0 : -1);
  const int64_t tb1 = window_base(geo, tr1 < geo.n_windows ? tr1 : -1);
  const int n_chunks = (int)((K * geo.sb + 31) / 32);

  {
    // block b: window-local queries (QB qg + b) * 16 + ql
    typename F::Q qfs[QB];
    f32x4 os[QB][4];
    float m_runs[QB], l_runs[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int kq = (QB * qg + b) * 16 + ql;
      const bool qvalid = kq < s2;
      const int64_t tok = window_token(geo, win, qvalid ? kq : 0);
      qfs[b] = F::load_q(qvalid ? static_cast<const T*>(p.q) + (tok * H + h) * kHeadDim : nullptr, g);
#pragma unroll
      for (int m = 0; m < 4; ++m) os[b][m] = f32x4{0, 0, 0, 0};
      m_runs[b] = -INFINITY;
      l_runs[b] = 0.0f;
    }

    // One chunk: scores of 32 key slots, online softmax, PV, for each block.
    auto process = [&](const SelChunk<T>& ch, const __bf16* vslab) __attribute__((always_inline)) {
      uint4 vt[4][1];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
      const typename F::Q& qf = qfs[b];
      f32x4 (&o)[4] = os[b];
      float& m_run = m_runs[b];
      float& l_run = l_runs[b];
      f32x4 s0 = F::qk(ch.k[0], qf);
      f32x4 s1 = F::qk(ch.k[1], qf);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool v0 = ch.jv >= 0 && ch.kkv0 + e < s2;
        const bool v1 = ch.jv >= 0 && ch.kkv0 + 4 + e < s2;
        if (!v0) s0[e] = -INFINITY;
        if (!v1) s1[e] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                       fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
      mx = max_halves32(max_rows16(mx));  // the query's four lanes ql + 16 g
      const float mnew = mx * c;
      if (mnew > m_run) {  // few chunks per window: rescale eagerly
        const float alpha = fast_exp2(m_run - mnew);
        m_run = mnew;
        l_run *= alpha;
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] *= alpha;
      }
      f32x4 p0, p1;
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p0[e] = m_run == -INFINITY ? 0.0f : fast_exp2(fmaf(s0[e], c, -m_run));
        p1[e] = m_run == -INFINITY ? 0.0f : fast_exp2(fmaf(s1[e], c, -m_run));
        ps += p0[e] + p1[e];
      }
      l_run += ps;
      if constexpr (SelChunk<T>::kSlabV) {
        // after the first block's scores, so that V's loads have had their time
        if (b == 0) slab_vt(vslab, ql, g, vt);
        F::pv(vt, p0, p1, o);
      } else {
        F::pv(ch.v, p0, p1, o);
      }
      }
    };

    // Two chunk buffers alternate so that two chunks of gathers are always in
    // flight; no register copies (a copy would wait for its loads).
    SelChunk<T> A, B;
    __bf16* sa = nullptr;
    __bf16* sbb = nullptr;
    if constexpr (SelChunk<T>::kSlabV) {
      const int wu = __builtin_amdgcn_readfirstlane(wv);
      sa = sel_vslab_a[wu];
      sbb = sel_vslab_b[wu];
    }
    load_chunk<T>(A, p, h, 0, ql, g, tr0, tr1, tb0, tb1, sa);
    load_chunk<T>(B, p, h, 1, ql, g, tr0, tr1, tb0, tb1, sbb);
    int ci = 0;
    for (; ci + 3 < n_chunks; ci += 2) {
      process(A, sa);
      load_chunk<T>(A, p, h, ci + 2, ql, g, tr0, tr1, tb0, tb1, sa);
      process(B, sbb);
      load_chunk<T>(B, p, h, ci + 3, ql, g, tr0, tr1, tb0, tb1, sbb);
    }
    process(A, sa);
    if (ci + 2 < n_chunks) load_chunk<T>(A, p, h, ci + 2, ql, g, tr0, tr1, tb0, tb1, sa);
    if (ci + 1 < n_chunks) process(B, sbb);
    if (ci + 2 < n_chunks) process(A, sa);

#pragma unroll
    for (int b = 0; b < QB; ++b) {
    if ((QB * qg + b) * 16 >= s2) continue;  // a block past the window's queries (uniform)
    const int kq = (QB * qg + b) * 16 + ql;
    const bool qvalid = kq < s2;
    const int64_t tok = window_token(geo, win, qvalid ? kq : 0);
    const typename F::Q& qf = qfs[b];
    const f32x4 (&o)[4] = os[b];
    const float m_run = m_runs[b], l_run = l_runs[b];
    float l = l_run + xor_lane(l_run, 16);
    l = l + xor_lane(l, 32);

    const int64_t u = window_image_index(geo, win, qvalid ? kq : 0);
    // join the context frames' partials (o_c normalised, lse_c natural log) into
    // the same softmax: weights 2^(m_run - M) for the gathered part and
    // 2^(lse_c log2 e - M) for each context part, M the largest exponent.
    float mm = m_run;
    for (int x = 0; x < p.n_ctx; ++x) mm = fmaxf(mm, p.ctx_lse[(x * geo.m_img + u) * H + h] * kLog2e);
    const float wsel = m_run == -INFINITY ? 0.0f : fast_exp2(m_run - mm);
    f32x4 res[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) res[m] = o[m] * wsel;
    float den = l * wsel;
    for (int x = 0; x < p.n_ctx; ++x) {
      const float lc = p.ctx_lse[(x * geo.m_img + u) * H + h] * kLog2e;
      const float wc = lc == -INFINITY ? 0.0f : fast_exp2(lc - mm);
      den += wc;
      const float* oc_row = p.ctx_o + ((x * geo.m_img + u) * H + h) * kHeadDim + 4 * g;
#pragma unroll
      for (int m = 0; m < 4; ++m) res[m] += wc * *reinterpret_cast<const f32x4*>(oc_row + 16 * m);
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) res[m] *= inv;

    if (p.o) {
      // fused upsample + gate + blend
      const float z0 = F::q_dot(qf, static_cast<const T*>(p.wg) + h * kHeadDim, g);
      float z = z0 + xor_lane(z0, 16);
      z = z + xor_lane(z, 32);
      const float gate = 1.0f / (1.0f + expf(-z));
      if (qvalid) {
        T* dst = static_cast<T*>(p.o) + (tok * H + h) * kHeadDim;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int dv0 = 16 * m + 4 * g;
          f32x4 ocv = *reinterpret_cast<const f32x4*>(p.oc + (win * H + h) * kHeadDim + dv0);
          // one rounding order whatever the register allocation: (1 - g) O_sel
          // fused onto the rounded g O'_comp
          f32x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = fmaf(1.0f - gate, res[m][e], gate * ocv[e]);
          if constexpr (sizeof(T) == 2) {
            bf16x4 b4 = {(__bf16)out[0], (__bf16)out[1], (__bf16)out[2], (__bf16)out[3]};
            *reinterpret_cast<bf16x4*>(dst + dv0) = b4;
          } else {
            *reinterpret_cast<f32x4*>(dst + dv0) = out;
          }
        }
      }
    }
    if (p.osel && qvalid) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        *reinterpret_cast<f32x4*>(p.osel + (u * H + h) * kHeadDim + 16 * m + 4 * g) = res[m];
    }
    // log2 of the joint denominator: sum of exp2(c s) over all keys = den 2^mm
    if (p.l2 && g == 0 && qvalid) p.l2[u * H + h] = den > 0.0f ? mm + log2f(den) : INFINITY;
    }
  }
}

// Standalone upsample + gate + blend: 8 lanes per (image token, head), each
// owning 8 channels; the gate dot product is reduced across the 8 lanes.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const Geometry& geo = p.g;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t uh = gid >> 3;
  const int part = (int)(gid & 7);
  const bool active = uh < geo.m_img * geo.n_heads;
  const int64_t uu = active ? uh : 0;
  const int64_t u = uu / geo.n_heads, h = uu % geo.n_heads, H = geo.n_heads;
  const int64_t hw = geo.grid_h * geo.grid_w;
  const int64_t f = u / hw, pix = u % hw, y = pix / geo.grid_w, x = pix % geo.grid_w;
  const int64_t tok = f * geo.tf + geo.n_special + pix;
  const int64_t win = f * geo.wpf + (y / geo.pool) * geo.wx + x / geo.pool;
  const T* qrow = static_cast<const T*>(p.q) + (tok * H + h) * kHeadDim + 8 * part;
  float gate;
  if (p.wg) {
    const T* w = static_cast<const T*>(p.wg) + h * kHeadDim + 8 * part;
    float z = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) z += to_f32(qrow[e]) * to_f32(w[e]);
    z += __shfl_xor(z, 1);
    z += __shfl_xor(z, 2);
    z += __shfl_xor(z, 4);
    gate = 1.0f / (1.0f + expf(-z));
  } else {
    gate = p.gate[u * H + h];
  }
  if (!active) return;
  const float* ocr = p.oc + (win * H + h) * kHeadDim + 8 * part;
  const float* osr = p.osel + (u * H + h) * kHeadDim + 8 * part;
  T* dst = static_cast<T*>(p.o) + (tok * H + h) * kHeadDim + 8 * part;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = from_f32<T>(fmaf(1.0f - gate, osr[e], gate * ocr[e]));
}

hipError_t launch_select(int dtype, const SelectParams& p, hipStream_t stream) {
  // one wave per (window, head) serves all of the window's blocks of 16
  // queries (s <= 8: at most 4 blocks)
  const int n_sub = (int)((p.g.pool * p.g.pool + 15) / 16);
  const int64_t items = p.g.n_windows * p.g.n_heads;
  if (items == 0) return hipSuccess;
  // bf16 V rows are addressed by 32-bit byte offsets from their window's first
  // row: s token rows of the grid must stay below 2^31 bytes
  if (dtype == kBF16 && p.g.pool * p.g.grid_w * p.g.n_heads * kHeadDim * 2 >= INT32_MAX - 4096)
    return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  if (dtype == kBF16) {
    if (n_sub == 1) hipLaunchKernelGGL((select_kernel<__bf16, 1>), dim3(blocks), dim3(256), 0, stream, p);
    else if (n_sub == 2) hipLaunchKernelGGL((select_kernel<__bf16, 2>), dim3(blocks), dim3(256), 0, stream, p);
    else if (n_sub == 3) hipLaunchKernelGGL((select_kernel<__bf16, 3>), dim3(blocks), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((select_kernel<__bf16, 4>), dim3(blocks), dim3(256), 0, stream, p);
  } else {
    if (n_sub == 1) hipLaunchKernelGGL((select_kernel<float, 1>), dim3(blocks), dim3(256), 0, stream, p);
    else if (n_sub == 2) hipLaunchKernelGGL((select_kernel<float, 2>), dim3(blocks), dim3(256), 0, stream, p);
    else if (n_sub == 3) hipLaunchKernelGGL((select_kernel<float, 3>), dim3(blocks), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((select_kernel<float, 4>), dim3(blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const CombineParams& p, hipStream_t stream) {
  const int64_t threads = p.g.m_img * p.g.n_heads * 8;
  if (threads == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(combine_kernel<__bf16>, dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gsa
