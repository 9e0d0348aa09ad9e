/*
 * libgsa -- Global Sparse Attention (GSA) forward on AMD Instinct MI355X (gfx950).
 *
 * GSA is the sparse replacement for dense global attention introduced by
 * "Speed3R: Sparse Feed-forward 3D Reconstruction Models" (CVPR 2026,
 * arXiv 2603.08055).  Citations below name the Paper-Notes page
 * "Speed3R: Sparse Feed-forward 3D Reconstruction Models" and its sections.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes: N frames, P special tokens per frame, an h x w image-token grid per
 * frame, T_f = P + h*w tokens per frame, M = N*T_f tokens, M_spec = N*P,
 * M_img = N*h*w, H heads of dimension d (d must be 64), pool size s (h and w
 * divisible by s), M' = M_img / s^2 windows, top-k k.
 *
 * Layouts (row-major, contiguous, element type = cfg->dtype unless stated):
 *   q, k, v, o   [N][T_f][H][d]. Token p < P of a frame is special; token
 *                p >= P is image pixel (y, x) = divmod(p - P, w).
 *   qc, kc, vc   [M'][H][d]; window j = f*(h/s)*(w/s) + wy*(w/s) + wx
 *                (frame-major, then window row, then window column).
 *   oc           float [M'][H][d].
 *   topk_idx     int32 [M'][H][k], per (window, head) sorted by guide score
 *                descending, ties to the lower window index; slots past the
 *                number of candidate windows hold -1.
 *   topk_score   float [M'][H][k] raw guide scores of those windows (or NULL).
 *   o_sel        float [M_img][H][d], image token u = f*h*w + y*w + x.
 *   gate         float [M_img][H].
 *   wg           [H][d] gate projection W_g (one scalar gate per token and head).
 *
 * Ownership: every tensor pointer is a DEVICE pointer owned by the caller and
 * must be 16-byte aligned; the workspace must be 256-byte aligned.  libgsa
 * never allocates device memory; gsa_workspace_size states the scratch it
 * needs.  Outputs must not alias inputs.
 *
 * Execution: every call validates its arguments on the host first; on any
 * validation error it returns that status without touching the device.
 * Otherwise it enqueues kernels on `stream` (a hipStream_t; NULL = the
 * default stream) of the current device and returns GSA_OK without
 * synchronising.  A failed kernel launch returns GSA_ERR_HIP.  Results are
 * bitwise deterministic for a given configuration and device.  The only
 * mutable global state is the per-device address table of the static scratch
 * used by gsa_forward_noalloc (filled once, under a lock), so calls from
 * several threads are safe (gsa_forward_noalloc: see its contract).
 */
#ifndef GSA_H_
#define GSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GSA_OK = 0,
  GSA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad k, bad context frame, aliasing */
  GSA_ERR_SHAPE = 2,       /* h or w not divisible by s, non-positive sizes, size overflow
                              (M' >= 2^29 windows, M >= 2^31 - 64 tokens, M*H*d > 2^40,
                              s*w*H*d*4 >= 2^31 - 4096 bytes) */
  GSA_ERR_UNSUPPORTED = 3, /* d != 64, s > 8, k > 128, unknown dtype */
  GSA_ERR_WORKSPACE = 4,   /* workspace smaller than gsa_workspace_size() */
  GSA_ERR_HIP = 5          /* a HIP launch failed */
} gsa_status;

typedef enum { GSA_BF16 = 0, GSA_F32 = 1 } gsa_dtype;

typedef enum {
  GSA_OP_FORWARD = 0, /* gsa_forward */
  GSA_OP_SPECIAL = 1, /* gsa_special_attn */
  GSA_OP_SELECT = 2,  /* gsa_select_attn */
  GSA_OP_DENSE = 3,   /* gsa_dense_attn */
  GSA_OP_COMPRESSED = 4, /* gsa_compressed_attn_topk */
  GSA_OP_BACKWARD = 5    /* gsa_backward */
} gsa_op;

#define GSA_MAX_CTX_FRAMES 16

typedef struct {
  int32_t n_frames;  /* N >= 1 */
  int32_t n_special; /* P >= 0 (P = 0: no special tokens) */
  int32_t grid_h;    /* h >= 1 */
  int32_t grid_w;    /* w >= 1 */
  int32_t n_heads;   /* H >= 1 */
  int32_t head_dim;  /* d, must be 64 */
  int32_t pool;      /* s in [1, 8], divides h and w */
  int32_t topk;      /* k in [1, 128]; clamped internally to the candidate count */
  int32_t n_ctx_frames;                   /* number of fixed-context frames, 0..16 */
  int32_t ctx_frames[GSA_MAX_CTX_FRAMES]; /* distinct frame ids in [0, N) */
  int32_t ctx_exclude_from_topk;          /* 1: context frames' windows are not top-k candidates */
  float scale;                            /* softmax scale; 0 means 1/sqrt(d) */
  int32_t dtype;                          /* gsa_dtype of q/k/v/o/wg/qc/kc/vc */
} gsa_config;

/* Device scratch (bytes) needed by the entry point `op` for this config. */
gsa_status gsa_workspace_size(const gsa_config* cfg, gsa_op op, size_t* bytes);

/*
 * s x s non-overlapping average pooling of the image Q/K/V into qc/kc/vc
 * (section "压缩分支": Q_comp, K_comp, V_comp in R^{M' x d}, M' = M_img/s^2).
 * Each pooled value is the float sum of the s^2 window values taken in
 * row-major order, times 1/s^2, rounded to the dtype (nearest even).
 */
gsa_status gsa_pool(const gsa_config* cfg, const void* q, const void* k, const void* v, void* qc,
                    void* kc, void* vc, void* stream);

/*
 * Compressed attention and the top-k over the guide scores (section "压缩分支":
 * O'_comp = Attention(Q_comp, K_comp, V_comp) and S_guide = Q_comp K_comp^T;
 * section "选择分支": TopKSelect of the most relevant windows; section
 * "高效 Triton Kernel 实现": the top-k is found from score tiles on chip, the
 * M' x M' score matrix is never stored).  Softmax over all M' windows with
 * the config scale; top-k over the raw scores of the candidate windows (all
 * windows, minus the context frames' windows when ctx_exclude_from_topk is
 * set), per head.  Writes oc, topk_idx and, if not NULL, topk_score.
 * The attention sweep also records a lower bound of the best score in each
 * group of key tiles; theta = the query's k-th best bound is at most its k-th
 * best score.  Only the groups whose bound comes within the bound's error of
 * theta can hold a key scoring >= theta; those keys are re-scored, collected
 * and ranked.  Exact for any input: query tiles where a query's candidate
 * list would overflow (e.g. many tied scores), or with fewer than k finite
 * bounds, are re-swept over every key, keeping the k best so far whenever the
 * slots fill up.  Workspace: GSA_OP_COMPRESSED bytes.
 */
gsa_status gsa_compressed_attn_topk(const gsa_config* cfg, const void* qc, const void* kc,
                                    const void* vc, float* oc, int32_t* topk_idx,
                                    float* topk_score, void* ws, size_t ws_bytes, void* stream);

/*
 * Selection-branch attention (section "选择分支": each image query attends the
 * full-resolution K/V of its window's top-k windows, the s^2 queries of a
 * window share one KV set; section "Speed3R-VGGT 适配": plus all T_f tokens
 * of each fixed-context frame, in one joint softmax).  topk_idx entries < 0
 * or >= M' are skipped.  Writes o_sel.  Workspace: GSA_OP_SELECT bytes (none
 * for bf16 without context frames).
 */
gsa_status gsa_select_attn(const gsa_config* cfg, const void* q, const void* k, const void* v,
                           const int32_t* topk_idx, float* o_sel, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Special-token attention (section "全局稀疏注意力（GSA）核心设计":
 * O_spec = softmax(Q_spec K^T / sqrt(d_k)) V over all M tokens).  Writes the
 * special rows of o only.  Workspace: GSA_OP_SPECIAL bytes.
 */
gsa_status gsa_special_attn(const gsa_config* cfg, const void* q, const void* k, const void* v,
                            void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * Nearest-neighbour upsampling and gated aggregation (section "压缩分支":
 * O_comp = Upsample(O'_comp); section "门控聚合": g = sigmoid(W_g Q_img),
 * O_img = g O_comp + (1 - g) O_sel).  If wg is NULL the gate is taken from
 * `gate` instead (explicit gates, e.g. exactly 0 or 1).  Writes the image
 * rows of o only.
 */
gsa_status gsa_gate_combine(const gsa_config* cfg, const void* q, const void* wg,
                            const float* gate, const float* oc, const float* o_sel, void* o,
                            void* stream);

/*
 * The whole GSA forward: pooling, special attention, compressed attention with
 * top-k, selection attention with the fused upsample + gate epilogue.  Writes
 * every row of o.  Workspace: GSA_OP_FORWARD bytes.
 */
gsa_status gsa_forward(const gsa_config* cfg, const void* q, const void* k, const void* v,
                       const void* wg, void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of the GSA layer (GSA is trained end to end by distillation from
 * the dense model: sections "研究背景与动机", "训练策略", "亮点与创新").
 * Given the gradient d_o ([N][T_f][H][d], dtype) of a loss with respect to
 * the output of gsa_forward(q, k, v, wg), writes the gradients of that loss
 * with respect to the inputs: dq, dk, dv float [N][T_f][H][d] (every row) and
 * dwg float [H][d].  The top-k window sets are held fixed at topk_idx
 * ([M'][H][k], as written by gsa_compressed_attn_topk for these inputs; the
 * selection is an index choice and is not differentiated; entries < 0 or
 * >= M' are skipped).  The pooled Q/K/V are used rounded to the dtype, as in
 * the forward, and the rounding is passed through as the identity (each
 * token of a window receives 1/s^2 of its pooled row's gradient).  The
 * forward quantities (pooled rows, the three attention outputs and their
 * softmax denominators, the gate) are recomputed inside the call.
 * Outputs must not alias inputs or each other.  GSA_ERR_SHAPE if M' H k >=
 * 2^31.  Workspace: GSA_OP_BACKWARD bytes.
 */
gsa_status gsa_backward(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg,
                        const int32_t* topk_idx, const void* d_o, float* dq, float* dk, float* dv, float* dwg,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * Training pair: the forward saves what the backward needs, so the backward
 * recomputes only the pooled rows.  The state (gsa_train_state_size bytes,
 * device memory owned by the caller, 256-byte aligned) holds, in this order
 * at 256-byte aligned offsets: topk_idx int32 [M'][H][k], O'_comp float
 * [M'][H][d] and its log-sum-exp float [M'][H] (natural log), the special rows'
 * outputs float [M_spec][H][d] and log2 softmax denominators float [M_spec][H],
 * O_sel float [M_img][H][d] and its log2 joint denominators float [M_img][H].
 * gsa_forward_train writes o exactly as gsa_forward does, plus the state
 * (workspace: GSA_OP_FORWARD bytes).  gsa_backward_train computes what
 * gsa_backward computes for the state's top-k sets, from the saved
 * quantities (workspace: GSA_OP_BACKWARD bytes; the state must come from
 * gsa_forward_train on the same inputs and config).  Both calls take the
 * state's size in bytes and return GSA_ERR_WORKSPACE, without touching the
 * device, when it is smaller than gsa_train_state_size.
 */
gsa_status gsa_train_state_size(const gsa_config* cfg, size_t* bytes);
gsa_status gsa_forward_train(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg,
                             void* o, void* state, size_t state_bytes, void* ws, size_t ws_bytes, void* stream);
gsa_status gsa_backward_train(const gsa_config* cfg, const void* q, const void* k, const void* v, const void* wg,
                              const void* state, size_t state_bytes, const void* d_o, float* dq, float* dk,
                              float* dv, float* dwg, void* ws, size_t ws_bytes, void* stream);

/*
 * Dense global attention of all M tokens over all M tokens at the same shape
 * (the attention GSA replaces; benchmark comparator).  Writes every row of o.
 */
gsa_status gsa_dense_attn(const gsa_config* cfg, const void* q, const void* k, const void* v,
                          void* o, void* ws, size_t ws_bytes, void* stream);

/*
 * Frame attention, the dense per-frame step that the aggregation transformer
 * alternates with GSA (section "整体框架": blocks alternate intra-frame
 * attention and global sparse attention).  Every token (special and image)
 * attends, in one softmax with the config scale, to the T_f tokens of its own
 * frame.  Uses n_frames, n_special, grid_h, grid_w, n_heads, head_dim, scale
 * and dtype of cfg (the other fields are validated as for every entry point).
 * Writes every row of o.  No workspace.
 */
gsa_status gsa_frame_attn(const gsa_config* cfg, const void* q, const void* k, const void* v, void* o,
                          void* stream);

/*
 * FlashVGGT descriptor attention (Paper-Notes page "FlashVGGT: Efficient and
 * Scalable Visual Geometry Transformers with Compressed Descriptor
 * Attention", section "关键设计": compressed descriptor tokens and descriptor
 * cross-attention; section "关键发现": auxiliary descriptor tokens).  These
 * three calls use the config's pool field as the downsampling factor r and
 * its ctx_frames as the keyframes (chosen by the caller); ctx_exclude_from_topk
 * and topk are validated but unused.
 *
 * The key/value set has n_set rows [n_set][H][d] (dtype), in this order:
 *   - descriptors: each frame's h x w image grid bilinearly resampled to
 *     (h/r) x (w/r) with half-pixel centres (output (y, x) samples the input
 *     at ((y + 0.5) r - 0.5, (x + 0.5) r - 0.5)), frame-major, row-major; the
 *     four weighted corners are summed in float in the order (y0,x0), (y0,x1),
 *     (y1,x0), (y1,x1) and rounded to the dtype (nearest even);
 *   - every token of frame 0 and of each keyframe (list order, frame 0 once);
 *   - the P special (camera) tokens of every other frame, frame-major.
 * n_set = N (h/r)(w/r) + n_full T_f + (N - n_full) P with n_full = the number
 * of distinct frames among {0} and the keyframes.
 */
gsa_status gsa_descriptor_count(const gsa_config* cfg, int64_t* n_set);

/* Builds the key set kd and the value set vd from k and v.  GSA_ERR_SHAPE if
 * n_set >= 2^31 - 64.  No workspace. */
gsa_status gsa_descriptor_set(const gsa_config* cfg, const void* k, const void* v, void* kd, void* vd,
                              void* stream);

/* Every token of q (full resolution, special and image) attends, in one
 * softmax with the config scale, to the n_set rows of kd/vd.  Writes every
 * row of o ([N][T_f][H][d]).  No workspace. */
gsa_status gsa_descriptor_attn(const gsa_config* cfg, const void* q, const void* kd, const void* vd, void* o,
                               void* stream);

/*
 * The forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and result as gsa_forward, with the workspace taken from a
 * static device array of GSA_NOALLOC_SCRATCH_BYTES (256 MiB) that each device
 * holds from the first call until the process ends.  The call allocates
 * nothing and frees nothing; q, k, v, wg and o are as for gsa_forward.
 * Returns GSA_ERR_WORKSPACE when the config's GSA_OP_FORWARD workspace is
 * larger than the array (e.g. 32 frames of 32 x 32 tokens with 16 heads,
 * s = 4, k = 16 fit; 128 frames of 36 x 36 do not).  Every call on a device
 * shares that device's array and no kernel relies on its previous contents:
 * calls that overlap on one device (several streams or host threads) race
 * and must be serialised by the caller.
 */
#define GSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
gsa_status gsa_forward_noalloc(const gsa_config* cfg, const void* q, const void* k, const void* v,
                               const void* wg, void* o, void* stream);

/* Static description of a status code. */
const char* gsa_status_string(gsa_status status);

#ifdef __cplusplus
}
#endif

#endif /* GSA_H_ */
