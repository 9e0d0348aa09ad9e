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
  // optional blocked copies of each tensor's windows, window-local token order
  // (zero padded to sb tokens): rows [M'][H][sb][d] and transposed [M'][H][d][sb]
  void* rows[3];
  void* trans[3];
  Geometry g;
  float inv_area;      // 1.0f / (s*s)
  int first_tensor;    // grid.y enumerates tensors first_tensor .. first_tensor+grid.y-1
};
hipError_t launch_pool(int dtype, const PoolParams& p, int n_tensors, hipStream_t stream);

// ---- tiled flash attention (special / dense / context / compressed+top-k) ----
constexpr int kMaxRanges = 64;
constexpr int kMaxExcl = 16;
// kFlashBound: compressed attention that also records, per group of key
// tiles, a lower bound of the group's best candidate score (input of the
// exact top-k kernels below, k <= kTopkMaxK).
enum FlashMode { kFlashFinal = 0, kFlashPartial = 1, kFlashBound = 3 };
// refine_kernel (the fallback sweep for queries whose candidate list
// overflowed): LDS candidate slots per query.  64 slots (80 KB per
// workgroup, two per CU) serve k <= 48; 144 slots (the whole 160 KB, one
// workgroup per CU) serve k <= 128.  A query needs its k best + one 4-key
// group of each lane (8) + 8 spare slots for whole-group writes.
constexpr int kRefineSlotsSmall = 64;
constexpr int kRefineSlotsLarge = 144;
constexpr int kTopkMaxK = kRefineSlotsLarge - 16;
// Groups of key tiles for the score bounds (at most; fewer when there are
// fewer tiles).  The threshold is the k-th largest group bound, so groups
// must well outnumber k; the more groups, the fewer keys each hot group
// holds.  8k groups, between 128 and 512.
inline int topk_groups_for_k(int k) { return k * 8 < 128 ? 128 : k * 8 > 512 ? 512 : k * 8; }
constexpr int kTopkMaxGroups = 512;
// Candidate list entries per query: about k + k^2/(2 * groups) keys reach the
// threshold on unstructured inputs; lists that overflow go to refine_kernel.
inline int topk_list_cap(int k) {
  const int c = (2 * k + 32 + 31) / 32 * 32;
  return c < 64 ? 64 : c;
}

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
  // kFlashPartial: part_o [split][n_q][H][d] (normalised), part_lse [split][n_q][H] (natural log);
  // with range_loop = 1 one workgroup sweeps all splits and writes one partial (index 0)
  int range_loop;
  float* part_o;
  float* part_lse;
  // kFlashBound: oc [n_q][H][d] fp32 (and, if part_lse is set, the rows' log-sum-exp there)
  float* oc;
  // keys (windows) that are not top-k candidates: n_excl ranges
  // [excl_beg[i], excl_end[i]), ascending, disjoint and not touching
  int n_excl;
  int excl_beg[kMaxExcl], excl_end[kMaxExcl];
  // kFlashBound: gbound [H][n_groups][n_q]; group g covers key tiles
  // [g*group_tiles, (g+1)*group_tiles) of the single key range; gerr [H][n_q]
  // receives 4x the largest error term of the query's finite bounds
  float* gbound;
  float* gerr;
  int n_groups, group_tiles;
};
hipError_t launch_flash(int dtype, int mode, const FlashParams& p, hipStream_t stream);

// Exact top-k of the compressed step, from the group bounds of the bound sweep:
//  threshold_kernel  theta = the k-th largest group bound of each query (every
//                    top-k key scores >= theta), a bit mask of the query's hot
//                    groups (those whose bound comes within the bound error of
//                    theta: only they can hold a key scoring >= theta), and
//                    the list counters (cap + 1 marks a query for the fallback);
//  hot_group_kernel  per (head, key group): every query for which the group is
//                    hot is scored against the group's keys; keys >= theta are
//                    appended to the query's candidate list;
//  rank_kernel       ranks each list (score desc, key asc), writes the top-k;
//  refine_kernel     fallback for the query tiles holding a query whose list
//                    overflowed or whose theta is -inf (fewer than k finite
//                    bounds): the full score-only sweep with compaction.
struct TopkParams {
  const void* q;
  const void* k;
  int64_t row_stride;
  int n_heads;
  int64_t n_q;          // queries = keys = M'
  const float* gbound;  // [H][n_groups][n_q] lower bounds of each group's best score
  const float* gerr;    // [H][n_q] bound on |bound - group max| + rounding slack
  int n_groups, group_tiles;
  int topk;
  float* theta;         // [H][n_q]
  uint32_t* hot;        // [H][n_words][n_q], bit g%32 of word g/32: group g is hot
  int n_words;          // ceil(n_groups / 32)
  int32_t* cnt;         // [H][n_q] list lengths (> cap: fallback)
  uint2* cand;          // [H][n_q][cap] (score bits, key)
  int cap;
  int n_chunks;         // hot_group_kernel: query chunks per (head, group)
  int n_excl;           // excluded key ranges, as in FlashParams
  int excl_beg[kMaxExcl], excl_end[kMaxExcl];
  int32_t* topk_idx;    // [n_q][H][topk]
  float* topk_score;    // [n_q][H][topk] or null
};
hipError_t launch_topk(int dtype, const TopkParams& p, hipStream_t stream);

// Combine split partials into the final rows of o (input dtype).
struct MergeParams {
  const float* part_o;
  const float* part_lse;
  int n_splits;
  int64_t n_q, qa, qb, qc;
  int n_heads;
  int64_t row_stride;
  void* o;              // merged rows in the input dtype at token rows (or null)
  // optional backward inputs: o32 [n_q][H][d] merged rows in float, l2
  // [n_q][H] log2 of the softmax denominator; with d_o (token rows, dtype)
  // also dd [n_q][H] = d_o . o
  float* o32;
  float* l2;
  const void* d_o;
  float* dd;
};
hipError_t launch_merge(int dtype, const MergeParams& p, hipStream_t stream);

// ---- selection attention over gathered top-k windows ------------------------
struct SelectParams {
  const void* q;        // token layout
  const void* k;        // token layout (K rows are gathered from it directly)
  const void* v;        // token layout (bf16: V rows are gathered from it directly)
  const void* vblk;     // fp32: [M'][H][d][sb] transposed V blocks
  const int32_t* topk_idx;  // [M'][H][topk]
  int topk;
  Geometry g;
  float scale_log2;
  int n_ctx;            // context partials (one per context frame, or one for all), 0 if none
  const float* ctx_o;   // [n_ctx][M_img][H][d] (normalised)
  const float* ctx_lse; // [n_ctx][M_img][H] log-sum-exp
  float* osel;          // standalone output [M_img][H][d]; fused path: optional copy of O_sel
  float* l2;            // optional: [M_img][H] log2 of the joint softmax denominator
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

// ---- backward ------------------------------------------------------------------
// Softmax attention backward with the log2 denominators L2 (P = exp2(c s - L2),
// c = scale log2 e) and D = dO . O given per query:
//   kBwdDQ    a workgroup owns 32*WAVES query rows and sweeps one key range:
//             dQ = scale sum_j dS_j k_j, dS_j = P_j (dO . v_j - D);
//   kBwdDKDV  a workgroup owns 32*WAVES keys of range 0 and sweeps the queries
//             (a contiguous part of them per query split):
//             dK_j = scale sum_i dS_ij q_i, dV_j = sum_i P_ij dO_i.
enum BwdKind { kBwdDQ = 0, kBwdDKDV = 1 };
struct FlashBwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  int64_t row_stride;  // elements between rows of q/k/v/d_o and of the float outputs (H*d)
  int n_heads;
  int64_t n_q, qa, qb, qc;  // query r -> token row (r / qa) * qb + qc + r % qa of q
  int do_mapped;            // 1: d_o rows follow that map; 0: d_o row = r
  const float* lse;         // [n_q][H]; L2 = lse * lse_mul
  float lse_mul;
  const float* dd;          // [n_q][H]
  int n_splits;             // kBwdDQ: one split per key range (partials when > 1)
  int64_t kbeg[kMaxRanges], kend[kMaxRanges];
  int n_qsplits;            // kBwdDKDV: query splits (partials when > 1)
  float scale, scale_log2;
  float* dq;                // kBwdDQ, one split: rows by the query map
  float* dk;                // kBwdDKDV, one query split: rows kbeg[0] + key
  float* dv;
  float* part;              // partials: kBwdDQ [split][n_q][H][d]; kBwdDKDV dk [z][nk][H][d] then dv
  int accumulate;           // add into dq / dk / dv instead of storing
};
hipError_t launch_flash_bwd(int dtype, int kind, const FlashBwdParams& p, hipStream_t stream);

// out[row(r)] (+)= sum over n_parts of part[i * part_stride + r*H*d ...]
struct ReduceParams {
  const float* part;
  int n_parts;
  int64_t part_stride;  // elements between consecutive partials
  int64_t n_rows;
  int n_heads;
  int64_t qa, qb, qc;   // row r -> output row (r / qa) * qb + qc + r % qa
  float* out;
  int accumulate;
};
hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream);

// Gate backward, one wave per (window, head): g, dz, the selection and
// compressed output gradients and the blocked copies the selection backward
// gathers.
struct GateBwdParams {
  const void* q;
  const void* wg;
  const void* d_o;
  const float* oc;     // [M'][H][d]
  const float* osel;   // [M_img][H][d]
  const float* l2sel;  // [M_img][H]
  Geometry g;
  float* dzblk;        // [M'][H][sb] dz = dO . (O'_i - O_sel) g (1 - g) (0 on padding)
  void* doblk;         // [M'][H][sb][d] dO_sel rows (dtype)
  void* doT;           // [M'][H][d][sb] dO_sel transposed (dtype), or null (bf16: transposed in LDS)
  float* l2blk;        // [M'][H][sb] (+inf on padding)
  float* dblk;         // [M'][H][sb] D_sel = dO_sel . O_sel (0 on padding)
  void* dosel_img;     // optional [M_img][H][d] (dtype)
  float* dsel_img;     // optional [M_img][H]
  void* doc;           // [M'][H][d] dO_comp (dtype)
  float* dc;           // [M'][H] dO_comp . O'_comp
  const float* lse_c;  // [M'][H] natural log-sum-exp of the compressed attention
  float* l2c;          // [M'][H] the same as a log2 denominator (lse_c log2 e)
  float* dwg_part;     // [M'][H][d]
};
hipError_t launch_gate_bwd(int dtype, const GateBwdParams& p, hipStream_t stream);

// Inverse top-k lists: for head h and window j, the query windows whose
// top-k holds j, ascending.  off [H*M' + 1] (exclusive scan of the counts).
struct InvParams {
  const int32_t* topk_idx;
  int topk;
  int64_t n_windows;
  int n_heads;
  int32_t* off;     // [H*M' + 1]: counts, then offsets
  int32_t* bsum;    // scan block sums
  int32_t* raw;     // [H*M'*k] lists in fill order
  int32_t* list;    // [H*M'*k] lists, ascending (before: each entry's rank in its list)
  int32_t* order;   // optional [H*M']: (head, window) lists, longest length class first
  int32_t* ccnt;    // [8 * ceil(H*M' / 1024)] class counts per block, then their scan
  int32_t* cbsum;   // scan block sums of ccnt
};
hipError_t launch_inverse_index(const InvParams& p, hipStream_t stream);

struct SelBwdParams {
  const void* qblk;  // [M'][H][sb][d]
  const void* qT;    // [M'][H][d][sb]
  const void* kblk;
  const void* kT;
  const void* vrow;  // [M'][H][sb][d]
  const void* doblk;
  const void* doT;
  const float* l2blk;
  const float* dblk;
  const float* dzblk;  // [M'][H][sb] the gate's dz per query slot
  const void* wg;      // [H][d] W_g (dtype)
  const int32_t* topk_idx;
  int topk;
  const int32_t* inv_off;
  const int32_t* inv_list;
  const int32_t* order;  // optional processing order of the key side (head * M' + window)
  Geometry g;
  float scale, scale_log2;
  const float* dqc;  // [M'][H][d] gradients of the pooled rows (the compressed branch's)
  const float* dkc;
  const float* dvc;
  float inv_area;    // 1 / s^2
  float* dq;  // token rows (float): image rows stored = dz W_g + selection gradient + pooled row's / s^2
  float* dk;
  float* dv;
};
hipError_t launch_sel_bwd(int dtype, const SelBwdParams& p, hipStream_t stream);

constexpr int kDwgSlices = 512;  // window slices of the dW_g reduction
struct DwgParams {
  const float* part;  // [M'][H][d]
  int64_t n_windows;
  int n_heads;
  float* slices;      // [kDwgSlices][H][d] slice totals (scratch)
  float* dwg;         // [H][d]
};
hipError_t launch_dwg_reduce(const DwgParams& p, hipStream_t stream);
hipError_t launch_fill(float* x, int64_t n, hipStream_t stream);

}  // namespace gsa
