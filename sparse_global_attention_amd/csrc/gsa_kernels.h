// Kernel parameter blocks and launchers of libgsa (host and device visible).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsa {

enum Dtype { kBF16 = 0, kF32 = 1 };

// Token / window geometry of one GSA call (derived from gsa_config).
struct Geometry {
  int64_t n_frames, n_special, grid_h, grid_w, n_heads, pool;
  int64_t tf;         // tokens per frame, P + h*w
  int64_t m_tokens;   // N * tf
  int64_t m_spec;     // N * P
  int64_t m_img;      // N * h * w
  int64_t wx;         // windows per window-row, w / s
  int64_t wpf;        // windows per frame
  int64_t n_windows;  // M'
  int64_t sb;         // key slots per window in the blocked K/V copies: s*s rounded up to 8
};

// Token row of the kk-th pixel (row-major inside the window) of window j.
__host__ __device__ __forceinline__ int64_t window_token(const Geometry& g, int64_t j, int64_t kk) {
  int64_t f = j / g.wpf, r = j - f * g.wpf;
  int64_t wy = r / g.wx, wxx = r - wy * g.wx;
  int64_t dy = kk / g.pool, dx = kk - dy * g.pool;
  return f * g.tf + g.n_special + (wy * g.pool + dy) * g.grid_w + wxx * g.pool + dx;
}
// Image-token index u = f*h*w + y*w + x of the kk-th pixel of window j.
__host__ __device__ __forceinline__ int64_t window_image_index(const Geometry& g, int64_t j, int64_t kk) {
  int64_t f = j / g.wpf, r = j - f * g.wpf;
  int64_t wy = r / g.wx, wxx = r - wy * g.wx;
  int64_t dy = kk / g.pool, dx = kk - dy * g.pool;
  return (f * g.grid_h + wy * g.pool + dy) * g.grid_w + wxx * g.pool + dx;
}

// ---- pooling (+ optional blocked K / transposed-V copies) -------------------
struct PoolParams {
  const void* src[3];  // q, k, v in the token layout
  void* dst[3];        // pooled [M'][H][d] (an entry may be null: no mean written)
  void* kblk;          // optional [M'][H][sb][d] copy of K, window-local key order
  void* vblk;          // optional [M'][H][d][sb] transposed copy of V
  Geometry g;
  float inv_area;      // 1.0f / (s*s)
  int first_tensor;    // grid.y enumerates tensors first_tensor .. first_tensor+grid.y-1
};
hipError_t launch_pool(int dtype, const PoolParams& p, int n_tensors, hipStream_t stream);

// ---- tiled flash attention (special / dense / context / compressed+top-k) ----
constexpr int kMaxRanges = 64;
constexpr int kMaxExcl = 16;
// kFlashBound: compressed attention that also records, per group of key
// tiles, a lower bound of the group's best candidate score (input of
// refine_kernel, which turns them into the exact top-k, k <= kRefineMaxK).
enum FlashMode { kFlashFinal = 0, kFlashPartial = 1, kFlashBound = 3 };
// refine_kernel: LDS candidate slots per query.  64 slots (80 KB per
// workgroup, two per CU) serve k <= 48; 144 slots (the whole 160 KB, one
// workgroup per CU) serve k <= 128.  A query needs its k best + one 4-key
// group of each lane (8) + 8 spare slots for whole-group writes.
constexpr int kRefineSlotsSmall = 64;
constexpr int kRefineSlotsLarge = 144;
constexpr int kRefineMaxK = kRefineSlotsLarge - 16;
// Groups of key tiles for the score bounds (at most; fewer when there are
// fewer tiles).  The threshold is the k-th largest group bound, so it needs
// groups well beyond k: 128 for k <= 48, 512 for larger k.
constexpr int kRefineGroups(int slots) { return slots == kRefineSlotsSmall ? 128 : 512; }
inline int refine_groups_for_k(int k) { return kRefineGroups(k <= kRefineSlotsSmall - 16 ? kRefineSlotsSmall : kRefineSlotsLarge); }

struct FlashParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t row_stride;  // elements between consecutive rows of q/k/v (H*d)
  int n_heads;
  // query rows r in [0, n_q) map to token rows (r / qa) * qb + qc + r % qa
  int64_t n_q, qa, qb, qc;
  // key splits: split s covers the non-empty contiguous key range [kbeg[s], kend[s])
  int n_splits;
  int64_t kbeg[kMaxRanges], kend[kMaxRanges];
  // independent batches (kFlashFinal only; 1 otherwise): batch b shifts every
  // query token row by b * q_bstride and every key range by b * k_bstride
  int64_t n_batch, q_bstride, k_bstride;
  float scale_log2;  // softmax scale * log2(e)
  // kFlashFinal: normalised output in the input dtype at rows token(r) of o
  void* o;
  // kFlashPartial: part_o [split][n_q][H][d] (normalised), part_lse [split][n_q][H] (natural log)
  float* part_o;
  float* part_lse;
  // kFlashBound: oc [n_q][H][d] fp32
  float* oc;
  int64_t wins_per_frame;
  int n_excl;                 // frames whose windows are not top-k candidates
  int excl_frames[kMaxExcl];
  // kFlashBound: gbound [H][n_groups][n_q]; group g covers key tiles
  // [g*group_tiles, (g+1)*group_tiles) of the single key range
  float* gbound;
  int n_groups, group_tiles;
};
hipError_t launch_flash(int dtype, int mode, const FlashParams& p, hipStream_t stream);

// Exact top-k from the group bounds: theta = k-th best bound per query; a
// score-only sweep keeps the candidate keys with score >= theta in LDS
// (compacting to the current k best when the slots run low) and ranks them.
struct RefineParams {
  const void* q;
  const void* k;
  int64_t row_stride;
  int n_heads;
  int64_t n_q;      // queries = keys = M'
  const float* gbound;
  int n_groups;
  int topk;
  int64_t wins_per_frame;
  int n_excl;
  int excl_frames[kMaxExcl];
  int32_t* topk_idx;
  float* topk_score;
};
hipError_t launch_refine(int dtype, const RefineParams& p, hipStream_t stream);

// Combine split partials into the final rows of o (input dtype).
struct MergeParams {
  const float* part_o;
  const float* part_lse;
  int n_splits;
  int64_t n_q, qa, qb, qc;
  int n_heads;
  int64_t row_stride;
  void* o;
};
hipError_t launch_merge(int dtype, const MergeParams& p, hipStream_t stream);

// ---- selection attention over gathered top-k windows ------------------------
struct SelectParams {
  const void* q;        // token layout
  const void* kblk;     // [M'][H][sb][d]
  const void* vblk;     // [M'][H][d][sb]
  const int32_t* topk_idx;  // [M'][H][topk]
  int topk;
  Geometry g;
  float scale_log2;
  int n_ctx;            // context partials (one per context frame), 0 if none
  const float* ctx_o;   // [n_ctx][M_img][H][d] (normalised)
  const float* ctx_lse; // [n_ctx][M_img][H] log-sum-exp
  float* osel;          // standalone output [M_img][H][d]
  const void* wg;       // fused epilogue: gate projection [H][d]
  const float* oc;      // fused epilogue: compressed output [M'][H][d]
  void* o;              // fused epilogue: output rows in the token layout
};
hipError_t launch_select(int dtype, const SelectParams& p, hipStream_t stream);

// ---- FlashVGGT descriptor set (bilinear descriptors + auxiliary tokens) -------
struct DescParams {
  const void* src[2];  // k, v in the token layout
  void* dst[2];        // [n_set][H][d]
  Geometry g;
  int r;               // downsampling factor (divides h and w)
  int64_t n_desc;      // N * (h/r) * (w/r) descriptor rows
  int64_t n_set;       // n_desc + auxiliary rows
  int n_full;          // frames whose every token is in the set: frame 0, then the keyframes
  int full[kMaxExcl + 1];         // in set order
  int full_sorted[kMaxExcl + 1];  // ascending
};
hipError_t launch_descriptor(int dtype, const DescParams& p, hipStream_t stream);

// ---- standalone upsample + gate + blend ----------------------------------------
struct CombineParams {
  const void* q;
  const void* wg;      // [H][d] or null
  const float* gate;   // [M_img][H], used when wg is null
  const float* oc;     // [M'][H][d]
  const float* osel;   // [M_img][H][d]
  void* o;
  Geometry g;
};
hipError_t launch_combine(int dtype, const CombineParams& p, hipStream_t stream);

}  // namespace gsa
