/*
 * GSA forward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, step-by-step CPU implementation of the Global Sparse
 * Attention (GSA) forward pass of "Speed3R: Sparse Feed-forward 3D
 * Reconstruction Models" (CVPR 2026, arXiv 2603.08055), as described on the
 * Paper-Notes page "Speed3R: Sparse Feed-forward 3D Reconstruction Models"
 * (sections "全局稀疏注意力（GSA）核心设计", "压缩分支", "选择分支",
 * "门控聚合", "Speed3R-VGGT 适配"), of the frame attention that alternates
 * with it (section "整体框架"), and of the descriptor attention of the
 * Paper-Notes page "FlashVGGT: Efficient and Scalable Visual Geometry
 * Transformers with Compressed Descriptor Attention".  Only the tests, the package smoke check
 * and the benchmark's CPU-baseline leg may call it; the HIP library never
 * does, and the two share no code.
 *
 * Arithmetic: inputs (bf16 bits or fp32) are widened exactly to double and
 * every dot product, exponential, sum and division is done in double.  The
 * single rounding inside the definition is the pooled tensors, which are
 * stored in the input precision (reading: average pooling of a bf16 tensor
 * gives a bf16 tensor).  Build with -ffp-contract=off and without fast-math.
 *
 * Layouts (all host memory, row-major):
 *   q, k, v       [N][T_f][H][d], T_f = P + h*w; token p < P of a frame is a
 *                 special token, token p >= P is image pixel (y, x) =
 *                 divmod(p - P, w).
 *   pooled        [M'][H][d] as float (values exactly representable in the
 *                 input precision); window j = f*(h/s)*(w/s) + wy*(w/s) + wx.
 *   per-window    rows follow the window's s*s tokens in row-major order
 *   outputs       (dy outer, dx inner).
 *
 * Readings of points the pages leave open (each is also listed with the
 * design notes of the library):
 *   - every step is per head; top-k is chosen per head;
 *   - the scale 1/sqrt(d) is used in all three attentions; the guide score
 *     used for selection is the raw product Q_comp K_comp^T;
 *   - top-k order is (score descending, window index ascending); ties go to
 *     the lower window index; k' = min(k, #candidates), slots past k' = -1;
 *   - image queries attend only image tokens of the selected windows, plus,
 *     when fixed-context frames are given, all T_f tokens of those frames in
 *     one joint softmax; context-frame windows are not top-k candidates when
 *     ctx_exclude is set;
 *   - the gate is g = sigmoid(W_g[h] . q) with W_g of shape [H][d], no bias.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int n_frames, n_special, grid_h, grid_w;
  int n_heads, head_dim, pool, topk;
  int n_ctx;
  int ctx_frames[16];
  int ctx_exclude;
  double scale; /* 0 -> 1/sqrt(head_dim) */
  int dtype;    /* 0: bf16 bits (uint16), 1: fp32 */
} orc_cfg;

/* ---- element access and rounding ------------------------------------- */

static double elem(const void* p, int dtype, int64_t i) {
  if (dtype == 1) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a float to bf16 (nearest, ties to even) and widen back to float. */
static float round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return f;
  u += 0x7FFFu + ((u >> 16) & 1u);
  u &= 0xFFFF0000u;
  memcpy(&f, &u, 4);
  return f;
}

static double scale_of(const orc_cfg* c) {
  return c->scale != 0.0 ? c->scale : 1.0 / sqrt((double)c->head_dim);
}

/* ---- token and window indexing (the split of X into spec/img rows) ------ */

static int64_t tokens_per_frame(const orc_cfg* c) {
  return (int64_t)c->n_special + (int64_t)c->grid_h * c->grid_w;
}
static int64_t n_tokens(const orc_cfg* c) { return (int64_t)c->n_frames * tokens_per_frame(c); }
static int64_t windows_x(const orc_cfg* c) { return c->grid_w / c->pool; }
static int64_t windows_per_frame(const orc_cfg* c) {
  return (int64_t)(c->grid_h / c->pool) * windows_x(c);
}
static int64_t n_windows(const orc_cfg* c) { return (int64_t)c->n_frames * windows_per_frame(c); }

/* Token row of the kk-th pixel (row-major inside the s x s window) of window j. */
static int64_t window_token(const orc_cfg* c, int64_t j, int kk) {
  int64_t f = j / windows_per_frame(c), r = j % windows_per_frame(c);
  int64_t wy = r / windows_x(c), wx = r % windows_x(c);
  int64_t y = wy * c->pool + kk / c->pool, x = wx * c->pool + kk % c->pool;
  return f * tokens_per_frame(c) + c->n_special + y * c->grid_w + x;
}

static int is_ctx_frame(const orc_cfg* c, int64_t f) {
  for (int i = 0; i < c->n_ctx; ++i)
    if (c->ctx_frames[i] == f) return 1;
  return 0;
}

/* Row (token t, head h) of a [M][H][d] tensor. */
static int64_t row_off(const orc_cfg* c, int64_t t, int h) {
  return (t * c->n_heads + h) * (int64_t)c->head_dim;
}

/* ---- plain softmax attention of one query row over a list of key rows ---- */

/* out[0..d) = sum_t softmax_t(scale * q.k_t) v_t over the n listed tokens. */
static void attend_tokens(const orc_cfg* c, const double* qrow, const void* k, const void* v,
                          const int64_t* toks, int64_t n, int h, double* logits, double* out) {
  const int d = c->head_dim;
  const double sc = scale_of(c);
  double mx = -INFINITY;
  for (int64_t t = 0; t < n; ++t) {
    int64_t o = row_off(c, toks[t], h);
    double s = 0.0;
    for (int e = 0; e < d; ++e) s += qrow[e] * elem(k, c->dtype, o + e);
    logits[t] = sc * s;
    if (logits[t] > mx) mx = logits[t];
  }
  double den = 0.0;
  for (int e = 0; e < d; ++e) out[e] = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    double w = exp(logits[t] - mx);
    den += w;
    int64_t o = row_off(c, toks[t], h);
    for (int e = 0; e < d; ++e) out[e] += w * elem(v, c->dtype, o + e);
  }
  for (int e = 0; e < d; ++e) out[e] /= den;
}

/* ======================================================================== */
/* Compression branch, pooling: s x s non-overlapping average pooling of the
 * image Q/K/V into [M'][H][d], M' = M_img / s^2.  (Paper-Notes page, section
 * "压缩分支": Q_comp, K_comp, V_comp from s x s non-overlapping average
 * pooling.)  The s^2 values are summed in float in row-major order starting
 * from +0, multiplied by 1/s^2 (a float computed once) and rounded to the
 * input precision. */
void orc_pool(const orc_cfg* c, const void* x, float* out) {
  const int64_t nw = n_windows(c);
  const int H = c->n_heads, d = c->head_dim, s2 = c->pool * c->pool;
  const float inv_area = 1.0f / (float)s2;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nw; ++j)
    for (int h = 0; h < H; ++h)
      for (int e = 0; e < d; ++e) {
        float acc = 0.0f;
        for (int kk = 0; kk < s2; ++kk)
          acc += (float)elem(x, c->dtype, row_off(c, window_token(c, j, kk), h) + e);
        float m = acc * inv_area;
        out[(j * H + h) * d + e] = c->dtype == 1 ? m : round_bf16(m);
      }
}

/* ======================================================================== */
/* Special tokens: dense softmax attention of each special query over all M
 * tokens, O_spec = softmax(Q_spec K^T / sqrt(d_k)) V.  (Paper-Notes page,
 * section "全局稀疏注意力（GSA）核心设计", the special-token equation.)
 * rows[i] is a special-row id r in [0, N*P): frame r / P, token r % P.
 * out: [n][H][d]. */
void orc_special(const orc_cfg* c, const void* q, const void* k, const void* v,
                 const int64_t* rows, int64_t n, double* out) {
  const int H = c->n_heads, d = c->head_dim;
  const int64_t M = n_tokens(c), tf = tokens_per_frame(c);
#pragma omp parallel
  {
    int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * M);
    double* logits = (double*)malloc(sizeof(double) * M);
    double* qrow = (double*)malloc(sizeof(double) * d);
    for (int64_t t = 0; t < M; ++t) toks[t] = t;
#pragma omp for schedule(dynamic, 1)
    for (int64_t ih = 0; ih < n * H; ++ih) {
      int64_t i = ih / H;
      int h = (int)(ih % H);
      int64_t t = (rows[i] / c->n_special) * tf + rows[i] % c->n_special;
      for (int e = 0; e < d; ++e) qrow[e] = elem(q, c->dtype, row_off(c, t, h) + e);
      attend_tokens(c, qrow, k, v, toks, M, h, logits, out + (i * H + h) * d);
    }
    free(toks);
    free(logits);
    free(qrow);
  }
}

/* ======================================================================== */
/* Compressed attention, guide scores and top-k selection, for the listed
 * query windows (all heads).
 *   S_ij  = Q_comp_i . K_comp_j (raw, unscaled)       -- section "压缩分支",
 *           guide-score equation;
 *   O'_i  = softmax_j(scale * S_ij) V_comp_j over all M' windows -- same
 *           section, compressed-attention equation;
 *   TopK_i = first k' windows of the candidate set sorted by (S_ij desc,
 *           j asc)                                   -- section "选择分支".
 * Inputs qc, kc, vc: pooled [M'][H][d] floats.
 * Outputs (n = number of listed windows):
 *   oc        [n][H][d]     O'_comp rows;
 *   topk_idx  [n][H][k]     k' sorted window ids then -1;
 *   topk_sc   [n][H][k+1]   the k'+1 best guide scores (NaN when absent);
 *   s_absmax  [n][H]        max_j |S_ij| over the candidates.
 * Any of the outputs may be NULL. */
typedef struct {
  double s;
  int64_t j;
} scored;

static int by_score_desc_index_asc(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

void orc_compressed(const orc_cfg* c, const float* qc, const float* kc, const float* vc,
                    const int64_t* wins, int64_t n, double* oc, int32_t* topk_idx,
                    double* topk_sc, double* s_absmax) {
  const int H = c->n_heads, d = c->head_dim, K = c->topk;
  const int64_t nw = n_windows(c), wpf = windows_per_frame(c);
  const double sc = scale_of(c);
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * nw);
    scored* cand = (scored*)malloc(sizeof(scored) * nw);
#pragma omp for schedule(dynamic, 1)
    for (int64_t ih = 0; ih < n * H; ++ih) {
      int64_t i = wins[ih / H];
      int h = (int)(ih % H);
      const float* qi = qc + (i * H + h) * d;
      /* guide scores S_ij */
      for (int64_t j = 0; j < nw; ++j) {
        const float* kj = kc + (j * H + h) * d;
        double s = 0.0;
        for (int e = 0; e < d; ++e) s += (double)qi[e] * (double)kj[e];
        S[j] = s;
      }
      /* compressed attention O'_i */
      if (oc) {
        double mx = -INFINITY, den = 0.0;
        double* o = oc + (ih / H * H + h) * d;
        for (int64_t j = 0; j < nw; ++j)
          if (sc * S[j] > mx) mx = sc * S[j];
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        for (int64_t j = 0; j < nw; ++j) {
          double w = exp(sc * S[j] - mx);
          den += w;
          const float* vj = vc + (j * H + h) * d;
          for (int e = 0; e < d; ++e) o[e] += w * (double)vj[e];
        }
        for (int e = 0; e < d; ++e) o[e] /= den;
      }
      /* top-k over the candidate windows */
      int64_t nc = 0;
      double amax = 0.0;
      for (int64_t j = 0; j < nw; ++j) {
        if (c->ctx_exclude && is_ctx_frame(c, j / wpf)) continue;
        cand[nc].s = S[j];
        cand[nc].j = j;
        ++nc;
        if (fabs(S[j]) > amax) amax = fabs(S[j]);
      }
      qsort(cand, (size_t)nc, sizeof(scored), by_score_desc_index_asc);
      int64_t kk = nc < K ? nc : K;
      int64_t base = ih / H * H + h;
      if (topk_idx)
        for (int t = 0; t < K; ++t) topk_idx[base * K + t] = t < kk ? (int32_t)cand[t].j : -1;
      if (topk_sc)
        for (int t = 0; t <= K; ++t) topk_sc[base * (K + 1) + t] = t < nc && t <= kk ? cand[t].s : NAN;
      if (s_absmax) s_absmax[base] = amax;
    }
    free(S);
    free(cand);
  }
}

/* Guide scores S_ij for given (window i, head h, window j) triples laid out as
 * idx [n][H][k] for the listed windows; out [n][H][k] (NaN where idx < 0). */
void orc_guide_scores(const orc_cfg* c, const float* qc, const float* kc, const int64_t* wins,
                      int64_t n, const int32_t* idx, int k, double* out) {
  const int H = c->n_heads, d = c->head_dim;
#pragma omp parallel for schedule(static)
  for (int64_t ih = 0; ih < n * H; ++ih) {
    int64_t i = wins[ih / H];
    int h = (int)(ih % H);
    for (int t = 0; t < k; ++t) {
      int32_t j = idx[ih * k + t];
      if (j < 0) {
        out[ih * k + t] = NAN;
        continue;
      }
      double s = 0.0;
      for (int e = 0; e < d; ++e)
        s += (double)qc[(i * H + h) * d + e] * (double)kc[((int64_t)j * H + h) * d + e];
      out[ih * k + t] = s;
    }
  }
}

/* ======================================================================== */
/* Selection branch: each image query of window i attends, in one softmax,
 * the full-resolution image tokens of the windows in TopK_i (the s^2 queries
 * of a window share one KV set) -- section "选择分支" -- together with all
 * T_f tokens of every fixed-context frame -- section "Speed3R-VGGT 适配".
 * idx: [n][H][k] window ids for the listed windows (entries < 0 ignored).
 * out: [n][s*s][H][d]. */
void orc_select(const orc_cfg* c, const void* q, const void* k, const void* v, const int64_t* wins,
                int64_t n, const int32_t* idx, int kcols, double* out) {
  const int H = c->n_heads, d = c->head_dim, s2 = c->pool * c->pool;
  const int64_t tf = tokens_per_frame(c);
  const int64_t cap = (int64_t)kcols * s2 + (int64_t)c->n_ctx * tf;
#pragma omp parallel
  {
    int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * cap);
    double* logits = (double*)malloc(sizeof(double) * cap);
    double* qrow = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t ih = 0; ih < n * H; ++ih) {
      int64_t i = wins[ih / H];
      int h = (int)(ih % H);
      int64_t nt = 0;
      for (int t = 0; t < kcols; ++t) {
        int32_t j = idx[ih * kcols + t];
        if (j < 0) continue;
        for (int kk = 0; kk < s2; ++kk) toks[nt++] = window_token(c, j, kk);
      }
      for (int cf = 0; cf < c->n_ctx; ++cf)
        for (int64_t p = 0; p < tf; ++p) toks[nt++] = (int64_t)c->ctx_frames[cf] * tf + p;
      for (int qq = 0; qq < s2; ++qq) {
        int64_t tq = window_token(c, i, qq);
        for (int e = 0; e < d; ++e) qrow[e] = elem(q, c->dtype, row_off(c, tq, h) + e);
        attend_tokens(c, qrow, k, v, toks, nt, h, logits,
                      out + (((ih / H) * s2 + qq) * H + h) * d);
      }
    }
    free(toks);
    free(logits);
    free(qrow);
  }
}

/* ======================================================================== */
/* Upsampling and gated aggregation for the listed windows:
 *   O_comp = nearest-neighbour upsampling of O'_comp  -- section "压缩分支";
 *   g = sigmoid(W_g . q), O_img = g O_comp + (1 - g) O_sel -- section
 *   "门控聚合".
 * wg: [H][d] in the input precision, or NULL to use gate [n][s*s][H].
 * oc: [n][H][d] (the windows' O'_comp rows); osel, out: [n][s*s][H][d]. */
void orc_gate_combine(const orc_cfg* c, const void* q, const void* wg, const double* gate,
                      const int64_t* wins, int64_t n, const double* oc, const double* osel,
                      double* out) {
  const int H = c->n_heads, d = c->head_dim, s2 = c->pool * c->pool;
#pragma omp parallel for schedule(static)
  for (int64_t iw = 0; iw < n; ++iw)
    for (int qq = 0; qq < s2; ++qq) {
      int64_t tq = window_token(c, wins[iw], qq);
      for (int h = 0; h < H; ++h) {
        double g;
        if (wg) {
          double z = 0.0;
          for (int e = 0; e < d; ++e)
            z += elem(wg, c->dtype, (int64_t)h * d + e) * elem(q, c->dtype, row_off(c, tq, h) + e);
          g = 1.0 / (1.0 + exp(-z));
        } else {
          g = gate[(iw * s2 + qq) * H + h];
        }
        for (int e = 0; e < d; ++e) {
          int64_t o = ((iw * s2 + qq) * H + h) * d + e;
          out[o] = g * oc[(iw * H + h) * d + e] + (1.0 - g) * osel[o];
        }
      }
    }
}

/* ======================================================================== */
/* Backward of the GSA layer.  Given the gradient dO [M][H][d] of a loss with
 * respect to the layer output o, the gradients dq, dk, dv [M][H][d] and dwg
 * [H][d] of that loss (equivalently of sum(dO * o)) with respect to the
 * inputs, with the top-k window sets held fixed at idx [M'][H][kcols] (the
 * selection is an index choice and is not differentiated; entries < 0 are
 * ignored).  The pages train GSA end to end by distillation from the dense
 * model (Paper-Notes page, sections "研究背景与动机", "训练策略" and
 * "亮点与创新"), which needs exactly these gradients of the forward above.
 *
 * Softmax attention of one query q over keys k_j, values v_j, weights
 * P_j = softmax_j(scale q.k_j), output O = sum_j P_j v_j:
 *   dP_j = dO . v_j,   D = sum_j P_j dP_j (= dO . O),   dS_j = P_j (dP_j - D),
 *   dq += scale sum_j dS_j k_j,   dk_j += scale dS_j q,   dv_j += P_j dO.
 * Gate g = sigmoid(z), z = W_g[h] . q, O_img = g O_comp + (1 - g) O_sel:
 *   dO_comp += g dO,  dO_sel = (1 - g) dO,  dz = (dO . (O_comp - O_sel)) g (1 - g),
 *   dq += dz W_g[h],  dW_g[h] += dz q.
 * Nearest upsampling sums dO_comp over the s^2 tokens of each window; the
 * compressed attention is the softmax attention of pooled rows over all M'
 * pooled rows; the pooled tensors are rounded as in the forward and the
 * rounding is passed through as the identity, so a pooled row's gradient
 * reaches each of its s^2 token rows times 1/s^2.
 * Every quantity is a double; this is the plain definition, for workloads
 * small enough to run whole. */

static double dot_d(const double* a, const double* b, int d) {
  double s = 0.0;
  for (int e = 0; e < d; ++e) s += a[e] * b[e];
  return s;
}

/* Softmax weights of query row qrow over the listed rows of K (a double
 * [rows][H][d] array, head h) into P[0..n). */
static void softmax_weights(int d, int H, int h, double sc, const double* qrow, const double* K,
                            const int64_t* rows, int64_t n, double* P) {
  double mx = -INFINITY, den = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    P[t] = sc * dot_d(qrow, K + (rows[t] * H + h) * d, d);
    if (P[t] > mx) mx = P[t];
  }
  for (int64_t t = 0; t < n; ++t) {
    P[t] = exp(P[t] - mx);
    den += P[t];
  }
  for (int64_t t = 0; t < n; ++t) P[t] /= den;
}

/* out[0..d) = sum_t P_t V[rows[t]] */
static void weighted_values(int d, int H, int h, const double* V, const int64_t* rows, int64_t n,
                            const double* P, double* out) {
  for (int e = 0; e < d; ++e) out[e] = 0.0;
  for (int64_t t = 0; t < n; ++t)
    for (int e = 0; e < d; ++e) out[e] += P[t] * V[(rows[t] * H + h) * d + e];
}

/* Attention backward of one query (weights recomputed): adds to dq_row[d]
 * and to the rows of dK, dV (double [rows][H][d]). */
static void attention_backward(int d, int H, int h, double sc, const double* qrow, const double* K,
                               const double* V, const int64_t* rows, int64_t n, const double* dorow,
                               double* P, double* dP, double* dq_row, double* dK, double* dV) {
  softmax_weights(d, H, h, sc, qrow, K, rows, n, P);
  double D = 0.0;
  for (int64_t t = 0; t < n; ++t) {
    dP[t] = dot_d(dorow, V + (rows[t] * H + h) * d, d);
    D += P[t] * dP[t];
  }
  for (int64_t t = 0; t < n; ++t) {
    const double ds = P[t] * (dP[t] - D);
    const double* kr = K + (rows[t] * H + h) * d;
    double* dkr = dK + (rows[t] * H + h) * d;
    double* dvr = dV + (rows[t] * H + h) * d;
    for (int e = 0; e < d; ++e) {
      dq_row[e] += sc * ds * kr[e];
      dkr[e] += sc * ds * qrow[e];
      dvr[e] += P[t] * dorow[e];
    }
  }
}

void orc_backward(const orc_cfg* c, const void* q, const void* k, const void* v, const void* wg,
                  const int32_t* idx, int kcols, const void* d_o, double* dq, double* dk, double* dv,
                  double* dwg) {
  const int H = c->n_heads, d = c->head_dim, s2 = c->pool * c->pool;
  const int64_t M = n_tokens(c), tf = tokens_per_frame(c), nw = n_windows(c);
  const double sc = scale_of(c);
  const size_t nel = (size_t)M * H * d, nwel = (size_t)nw * H * d;
  double* Q = (double*)malloc(sizeof(double) * nel);
  double* K = (double*)malloc(sizeof(double) * nel);
  double* V = (double*)malloc(sizeof(double) * nel);
  double* G = (double*)malloc(sizeof(double) * nel);
  for (size_t i = 0; i < nel; ++i) {
    Q[i] = elem(q, c->dtype, (int64_t)i);
    K[i] = elem(k, c->dtype, (int64_t)i);
    V[i] = elem(v, c->dtype, (int64_t)i);
    G[i] = elem(d_o, c->dtype, (int64_t)i);
    dq[i] = dk[i] = dv[i] = 0.0;
  }
  /* pooled rows, rounded as in the forward */
  float* pooled = (float*)malloc(sizeof(float) * nwel);
  double* Qc = (double*)malloc(sizeof(double) * nwel);
  double* Kc = (double*)malloc(sizeof(double) * nwel);
  double* Vc = (double*)malloc(sizeof(double) * nwel);
  double* dQc = (double*)calloc(nwel, sizeof(double));
  double* dKc = (double*)calloc(nwel, sizeof(double));
  double* dVc = (double*)calloc(nwel, sizeof(double));
  double* dOc = (double*)calloc(nwel, sizeof(double));
  double* Oc = (double*)malloc(sizeof(double) * nwel);
  const void* src[3] = {q, k, v};
  double* dstp[3] = {Qc, Kc, Vc};
  for (int x = 0; x < 3; ++x) {
    orc_pool(c, src[x], pooled);
    for (size_t i = 0; i < nwel; ++i) dstp[x][i] = pooled[i];
  }
  free(pooled);

  const int64_t cap = (M > nw ? M : nw) + (int64_t)kcols * s2;
#pragma omp parallel for schedule(static, 1)
  for (int h = 0; h < H; ++h) {
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * cap);
    double* P = (double*)malloc(sizeof(double) * cap);
    double* dP = (double*)malloc(sizeof(double) * cap);
    double osel[512], dosel[512], dorow[512];
    for (int e = 0; e < d; ++e) dwg[h * d + e] = 0.0;

    /* special rows: attention over all M tokens */
    for (int64_t t = 0; t < M; ++t) rows[t] = t;
    for (int64_t f = 0; f < c->n_frames; ++f)
      for (int p = 0; p < c->n_special; ++p) {
        const int64_t t = f * tf + p;
        attention_backward(d, H, h, sc, Q + (t * H + h) * d, K, V, rows, M, G + (t * H + h) * d, P, dP,
                           dq + (t * H + h) * d, dk, dv);
      }

    /* compressed attention output of every window */
    for (int64_t j = 0; j < nw; ++j) rows[j] = j;
    for (int64_t i = 0; i < nw; ++i) {
      softmax_weights(d, H, h, sc, Qc + (i * H + h) * d, Kc, rows, nw, P);
      weighted_values(d, H, h, Vc, rows, nw, P, Oc + (i * H + h) * d);
    }

    /* image rows: gate, selection attention (+ context), compressed-branch gradient */
    for (int64_t i = 0; i < nw; ++i) {
      int64_t nt = 0;
      for (int t = 0; t < kcols; ++t) {
        const int32_t j = idx[(i * H + h) * kcols + t];
        if (j < 0) continue;
        for (int kk = 0; kk < s2; ++kk) rows[nt++] = window_token(c, j, kk);
      }
      for (int cf = 0; cf < c->n_ctx; ++cf)
        for (int64_t p = 0; p < tf; ++p) rows[nt++] = (int64_t)c->ctx_frames[cf] * tf + p;
      const double* oc = Oc + (i * H + h) * d;
      for (int qq = 0; qq < s2; ++qq) {
        const int64_t t = window_token(c, i, qq);
        const double* qrow = Q + (t * H + h) * d;
        const double* g_o = G + (t * H + h) * d;
        softmax_weights(d, H, h, sc, qrow, K, rows, nt, P);
        weighted_values(d, H, h, V, rows, nt, P, osel);
        double z = 0.0;
        for (int e = 0; e < d; ++e) z += elem(wg, c->dtype, (int64_t)h * d + e) * qrow[e];
        const double g = 1.0 / (1.0 + exp(-z));
        double dg = 0.0;
        for (int e = 0; e < d; ++e) {
          dg += g_o[e] * (oc[e] - osel[e]);
          dOc[(i * H + h) * d + e] += g * g_o[e];
          dosel[e] = (1.0 - g) * g_o[e];
        }
        const double dz = dg * g * (1.0 - g);
        for (int e = 0; e < d; ++e) {
          dq[(t * H + h) * d + e] += dz * elem(wg, c->dtype, (int64_t)h * d + e);
          dwg[h * d + e] += dz * qrow[e];
        }
        attention_backward(d, H, h, sc, qrow, K, V, rows, nt, dosel, P, dP, dq + (t * H + h) * d, dk, dv);
      }
    }

    /* compressed attention backward over the pooled rows */
    for (int64_t j = 0; j < nw; ++j) rows[j] = j;
    for (int64_t i = 0; i < nw; ++i) {
      for (int e = 0; e < d; ++e) dorow[e] = dOc[(i * H + h) * d + e];
      attention_backward(d, H, h, sc, Qc + (i * H + h) * d, Kc, Vc, rows, nw, dorow, P, dP,
                         dQc + (i * H + h) * d, dKc, dVc);
    }

    /* pooling backward: each token of window j gets its pooled row's gradient / s^2 */
    for (int64_t j = 0; j < nw; ++j)
      for (int kk = 0; kk < s2; ++kk) {
        const int64_t t = window_token(c, j, kk);
        for (int e = 0; e < d; ++e) {
          dq[(t * H + h) * d + e] += dQc[(j * H + h) * d + e] / s2;
          dk[(t * H + h) * d + e] += dKc[(j * H + h) * d + e] / s2;
          dv[(t * H + h) * d + e] += dVc[(j * H + h) * d + e] / s2;
        }
      }
    free(rows);
    free(P);
    free(dP);
  }
  free(Q);
  free(K);
  free(V);
  free(G);
  free(Qc);
  free(Kc);
  free(Vc);
  free(dQc);
  free(dKc);
  free(dVc);
  free(dOc);
  free(Oc);
}

/* dq contribution of one query row (head h) attending the listed token rows
 * of k/v (dtype arrays): adds scale * sum_j P_j (dO . v_j - D) k_j to o. */
static void dq_over_rows(const orc_cfg* c, const void* k, const void* v, int h, double sc, const double* qrow,
                         const double* dorow, const int64_t* rows, int64_t n, double* P, double* dP, double* o) {
  const int d = c->head_dim;
  double mx = -INFINITY, den = 0.0, D = 0.0;
  for (int64_t u = 0; u < n; ++u) {
    double s = 0.0;
    for (int e = 0; e < d; ++e) s += qrow[e] * elem(k, c->dtype, row_off(c, rows[u], h) + e);
    P[u] = sc * s;
    if (P[u] > mx) mx = P[u];
  }
  for (int64_t u = 0; u < n; ++u) {
    P[u] = exp(P[u] - mx);
    den += P[u];
  }
  for (int64_t u = 0; u < n; ++u) {
    P[u] /= den;
    double dp = 0.0;
    for (int e = 0; e < d; ++e) dp += dorow[e] * elem(v, c->dtype, row_off(c, rows[u], h) + e);
    dP[u] = dp;
    D += P[u] * dp;
  }
  for (int64_t u = 0; u < n; ++u) {
    const double ds = P[u] * (dP[u] - D);
    for (int e = 0; e < d; ++e) o[e] += sc * ds * elem(k, c->dtype, row_off(c, rows[u], h) + e);
  }
}

/* dq of the listed token rows only (the same definition as orc_backward,
 * evaluated per row, for workloads too large for the whole layer): a
 * special row's attention backward over all M tokens; an image row's gate
 * term, its selection backward (with fixed idx and the context frames), and
 * 1/s^2 of its window's row of the compressed-attention backward (dO_comp of
 * the window summed from its s^2 tokens).  rows are token ids; out: [n][H][d]. */
void orc_backward_dq_rows(const orc_cfg* c, const void* q, const void* k, const void* v, const void* wg,
                          const int32_t* idx, int kcols, const void* d_o, const int64_t* rows, int64_t n,
                          double* out) {
  const int H = c->n_heads, d = c->head_dim, s2 = c->pool * c->pool;
  const int64_t M = n_tokens(c), tf = tokens_per_frame(c), nw = n_windows(c);
  const double sc = scale_of(c);
  const size_t nwel = (size_t)nw * H * d;
  /* pooled rows, rounded as in the forward, widened to double */
  float* pooled = (float*)malloc(sizeof(float) * nwel);
  double* pq[3];
  const void* src[3] = {q, k, v};
  for (int x = 0; x < 3; ++x) {
    pq[x] = (double*)malloc(sizeof(double) * nwel);
    orc_pool(c, src[x], pooled);
    for (size_t i = 0; i < nwel; ++i) pq[x][i] = pooled[i];
  }
  free(pooled);
  const int64_t cap = (M > nw ? M : nw) + (int64_t)kcols * s2;
#pragma omp parallel
  {
    int64_t* krows = (int64_t*)malloc(sizeof(int64_t) * cap);
    double* P = (double*)malloc(sizeof(double) * cap);
    double* dP = (double*)malloc(sizeof(double) * cap);
    double qrow[512], grow[512], osel[512], oc[512], doc[512], dqc[512], dosel[512];
#pragma omp for schedule(dynamic, 1)
    for (int64_t ih = 0; ih < n * H; ++ih) {
      const int64_t t = rows[ih / H];
      const int h = (int)(ih % H);
      double* o = out + ih * d;
      for (int e = 0; e < d; ++e) {
        qrow[e] = elem(q, c->dtype, row_off(c, t, h) + e);
        grow[e] = elem(d_o, c->dtype, row_off(c, t, h) + e);
        o[e] = 0.0;
      }
      const int64_t f = t / tf, p = t % tf;
      if (p < c->n_special) {  /* special row: attention over all M tokens */
        for (int64_t u = 0; u < M; ++u) krows[u] = u;
        dq_over_rows(c, k, v, h, sc, qrow, grow, krows, M, P, dP, o);
        continue;
      }
      /* image row of window i */
      const int64_t pix = p - c->n_special, y = pix / c->grid_w, x = pix % c->grid_w;
      const int64_t i = f * windows_per_frame(c) + (y / c->pool) * windows_x(c) + x / c->pool;
      /* O'_comp of window i, the gates of its tokens, dO_comp of window i */
      for (int64_t j = 0; j < nw; ++j) krows[j] = j;
      softmax_weights(d, H, h, sc, pq[0] + (i * H + h) * d, pq[1], krows, nw, P);
      weighted_values(d, H, h, pq[2], krows, nw, P, oc);
      double g_t = 0.0;
      for (int e = 0; e < d; ++e) doc[e] = 0.0;
      for (int kk = 0; kk < s2; ++kk) {
        const int64_t tt = window_token(c, i, kk);
        double z = 0.0;
        for (int e = 0; e < d; ++e)
          z += elem(wg, c->dtype, (int64_t)h * d + e) * elem(q, c->dtype, row_off(c, tt, h) + e);
        const double g = 1.0 / (1.0 + exp(-z));
        if (tt == t) g_t = g;
        for (int e = 0; e < d; ++e) doc[e] += g * elem(d_o, c->dtype, row_off(c, tt, h) + e);
      }
      /* row i of the compressed-attention backward: dQc_i (P still holds row i's weights) */
      for (int e = 0; e < d; ++e) dqc[e] = 0.0;
      double D = 0.0;
      for (int64_t j = 0; j < nw; ++j) {
        dP[j] = dot_d(doc, pq[2] + (j * H + h) * d, d);
        D += P[j] * dP[j];
      }
      for (int64_t j = 0; j < nw; ++j) {
        const double ds = P[j] * (dP[j] - D);
        for (int e = 0; e < d; ++e) dqc[e] += sc * ds * pq[1][(j * H + h) * d + e];
      }
      /* the row's selection set (+ context) and O_sel */
      int64_t nt = 0;
      for (int tt = 0; tt < kcols; ++tt) {
        const int32_t j = idx[(i * H + h) * kcols + tt];
        if (j < 0) continue;
        for (int kk = 0; kk < s2; ++kk) krows[nt++] = window_token(c, j, kk);
      }
      for (int cf = 0; cf < c->n_ctx; ++cf)
        for (int64_t pp = 0; pp < tf; ++pp) krows[nt++] = (int64_t)c->ctx_frames[cf] * tf + pp;
      attend_tokens(c, qrow, k, v, krows, nt, h, P, osel);
      /* gate term, pooled term, selection term */
      double dg = 0.0;
      for (int e = 0; e < d; ++e) dg += grow[e] * (oc[e] - osel[e]);
      const double dz = dg * g_t * (1.0 - g_t);
      for (int e = 0; e < d; ++e) {
        o[e] += dz * elem(wg, c->dtype, (int64_t)h * d + e) + dqc[e] / s2;
        dosel[e] = (1.0 - g_t) * grow[e];
      }
      dq_over_rows(c, k, v, h, sc, qrow, dosel, krows, nt, P, dP, o);
    }
    free(krows);
    free(P);
    free(dP);
  }
  for (int x = 0; x < 3; ++x) free(pq[x]);
}

/* dK and dV of the listed token rows only (the same definition as
 * orc_backward, evaluated per key row, for workloads too large for the whole
 * layer).  A key/value row t collects, for head h:
 *   - from every special query i: scale P_it (dP_it - D_i) q_i and P_it dO_i
 *     (softmax of q_i over all M tokens, dP_it = dO_i . v_t, D_i = sum_u P_iu dP_iu);
 *   - from every window i as a compressed query, when t is an image token of
 *     window j: 1/s^2 of scale P_ij (dP_ij - D_i) Qc_i and of P_ij dOc_i
 *     (softmax of Qc_i over all M' pooled rows, dOc_i = sum of g dO over the
 *     tokens of window i, dP_ij = dOc_i . Vc_j);
 *   - from every image query u whose selection set (the tokens of its
 *     window's top-k windows, then every token of the context frames) holds
 *     t, once per occurrence: scale P_ut (dP_ut - D_u) q_u and P_ut dOsel_u
 *     (dOsel_u = (1 - g_u) dO_u).
 * A query whose incoming gradient (dO_i, dOc_i or dOsel_u) is exactly zero
 * contributes exactly zero and is skipped, so the cost follows the rows where
 * d_o is non-zero.  rows are distinct token ids; dk_out, dv_out: [n][H][d]. */
/* g = sigmoid(W_g[h] . q_t) of token row t, head h. */
static double gate_of(const orc_cfg* c, const void* q, const void* wg, int64_t t, int h) {
  const int d = c->head_dim;
  double z = 0.0;
  for (int e = 0; e < d; ++e) z += elem(wg, c->dtype, (int64_t)h * d + e) * elem(q, c->dtype, row_off(c, t, h) + e);
  return 1.0 / (1.0 + exp(-z));
}

void orc_backward_dkdv_rows(const orc_cfg* c, const void* q, const void* k, const void* v, const void* wg,
                            const int32_t* idx, int kcols, const void* d_o, const int64_t* rows, int64_t n,
                            double* dk_out, double* dv_out) {
  const int H = c->n_heads, d = c->head_dim, s2 = c->pool * c->pool;
  const int64_t M = n_tokens(c), tf = tokens_per_frame(c), nw = n_windows(c);
  const double sc = scale_of(c);
  const size_t nwel = (size_t)nw * H * d;
  /* listed[t] = position of token t in rows, or -1 */
  int64_t* listed = (int64_t*)malloc(sizeof(int64_t) * M);
  for (int64_t t = 0; t < M; ++t) listed[t] = -1;
  for (int64_t r = 0; r < n; ++r) listed[rows[r]] = r;
  for (size_t i = 0; i < (size_t)n * H * d; ++i) dk_out[i] = dv_out[i] = 0.0;
  /* pooled rows, rounded as in the forward, widened to double */
  float* pooled = (float*)malloc(sizeof(float) * nwel);
  double* pq[3];
  const void* src[3] = {q, k, v};
  for (int x = 0; x < 3; ++x) {
    pq[x] = (double*)malloc(sizeof(double) * nwel);
    orc_pool(c, src[x], pooled);
    for (size_t i = 0; i < nwel; ++i) pq[x][i] = pooled[i];
  }
  free(pooled);
  const int64_t cap = (M > nw ? M : nw) + (int64_t)kcols * s2 + (int64_t)c->n_ctx * tf;
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < H; ++h) {
    int64_t* krows = (int64_t*)malloc(sizeof(int64_t) * cap);
    double* P = (double*)malloc(sizeof(double) * cap);
    double* dP = (double*)malloc(sizeof(double) * cap);
    double qrow[512], grow[512], doc[512], dosel[512];
    /* 1. special queries over all M tokens */
    for (int64_t f = 0; f < c->n_frames; ++f)
      for (int pp = 0; pp < c->n_special; ++pp) {
        const int64_t i = f * tf + pp;
        int nz = 0;
        for (int e = 0; e < d; ++e) {
          qrow[e] = elem(q, c->dtype, row_off(c, i, h) + e);
          grow[e] = elem(d_o, c->dtype, row_off(c, i, h) + e);
          nz |= grow[e] != 0.0;
        }
        if (!nz) continue;
        double mx = -INFINITY, den = 0.0, D = 0.0;
        for (int64_t t = 0; t < M; ++t) {
          double sdot = 0.0, gdot = 0.0;
          for (int e = 0; e < d; ++e) {
            sdot += qrow[e] * elem(k, c->dtype, row_off(c, t, h) + e);
            gdot += grow[e] * elem(v, c->dtype, row_off(c, t, h) + e);
          }
          P[t] = sc * sdot;
          dP[t] = gdot;
          if (P[t] > mx) mx = P[t];
        }
        for (int64_t t = 0; t < M; ++t) {
          P[t] = exp(P[t] - mx);
          den += P[t];
        }
        for (int64_t t = 0; t < M; ++t) {
          P[t] /= den;
          D += P[t] * dP[t];
        }
        for (int64_t r = 0; r < n; ++r) {
          const int64_t t = rows[r];
          const double ds = P[t] * (dP[t] - D);
          for (int e = 0; e < d; ++e) {
            dk_out[(r * H + h) * d + e] += sc * ds * qrow[e];
            dv_out[(r * H + h) * d + e] += P[t] * grow[e];
          }
        }
      }
    /* 2. windows as compressed queries over all M' pooled rows */
    for (int64_t j = 0; j < nw; ++j) krows[j] = j;
    for (int64_t i = 0; i < nw; ++i) {
      int nz = 0;
      for (int e = 0; e < d; ++e) doc[e] = 0.0;
      for (int kk = 0; kk < s2; ++kk) {
        const int64_t tt = window_token(c, i, kk);
        const double g = gate_of(c, q, wg, tt, h);
        for (int e = 0; e < d; ++e) doc[e] += g * elem(d_o, c->dtype, row_off(c, tt, h) + e);
      }
      for (int e = 0; e < d; ++e) nz |= doc[e] != 0.0;
      if (!nz) continue;
      softmax_weights(d, H, h, sc, pq[0] + (i * H + h) * d, pq[1], krows, nw, P);
      double D = 0.0;
      for (int64_t j = 0; j < nw; ++j) {
        dP[j] = dot_d(doc, pq[2] + (j * H + h) * d, d);
        D += P[j] * dP[j];
      }
      for (int64_t r = 0; r < n; ++r) {
        const int64_t t = rows[r], f = t / tf, p = t % tf;
        if (p < c->n_special) continue;
        const int64_t pix = p - c->n_special, y = pix / c->grid_w, x = pix % c->grid_w;
        const int64_t j = f * windows_per_frame(c) + (y / c->pool) * windows_x(c) + x / c->pool;
        const double ds = P[j] * (dP[j] - D);
        for (int e = 0; e < d; ++e) {
          dk_out[(r * H + h) * d + e] += sc * ds * pq[0][(i * H + h) * d + e] / s2;
          dv_out[(r * H + h) * d + e] += P[j] * doc[e] / s2;
        }
      }
    }
    /* 3. image queries over their selection sets (+ context) */
    for (int64_t i = 0; i < nw; ++i) {
      int64_t nt = 0;
      for (int tt = 0; tt < kcols; ++tt) {
        const int32_t j = idx[(i * H + h) * kcols + tt];
        if (j < 0 || j >= nw) continue;
        for (int kk = 0; kk < s2; ++kk) krows[nt++] = window_token(c, j, kk);
      }
      for (int cf = 0; cf < c->n_ctx; ++cf)
        for (int64_t pp = 0; pp < tf; ++pp) krows[nt++] = (int64_t)c->ctx_frames[cf] * tf + pp;
      for (int qq = 0; qq < s2; ++qq) {
        const int64_t u = window_token(c, i, qq);
        int nz = 0;
        for (int e = 0; e < d; ++e) {
          grow[e] = elem(d_o, c->dtype, row_off(c, u, h) + e);
          nz |= grow[e] != 0.0;
        }
        if (!nz) continue;
        const double g = gate_of(c, q, wg, u, h);
        for (int e = 0; e < d; ++e) {
          qrow[e] = elem(q, c->dtype, row_off(c, u, h) + e);
          dosel[e] = (1.0 - g) * grow[e];
        }
        double mx = -INFINITY, den = 0.0, D = 0.0;
        for (int64_t e2 = 0; e2 < nt; ++e2) {
          double sdot = 0.0, gdot = 0.0;
          for (int e = 0; e < d; ++e) {
            sdot += qrow[e] * elem(k, c->dtype, row_off(c, krows[e2], h) + e);
            gdot += dosel[e] * elem(v, c->dtype, row_off(c, krows[e2], h) + e);
          }
          P[e2] = sc * sdot;
          dP[e2] = gdot;
          if (P[e2] > mx) mx = P[e2];
        }
        for (int64_t e2 = 0; e2 < nt; ++e2) {
          P[e2] = exp(P[e2] - mx);
          den += P[e2];
        }
        for (int64_t e2 = 0; e2 < nt; ++e2) {
          P[e2] /= den;
          D += P[e2] * dP[e2];
        }
        for (int64_t e2 = 0; e2 < nt; ++e2) {
          const int64_t r = listed[krows[e2]];
          if (r < 0) continue;
          const double ds = P[e2] * (dP[e2] - D);
          for (int e = 0; e < d; ++e) {
            dk_out[(r * H + h) * d + e] += sc * ds * qrow[e];
            dv_out[(r * H + h) * d + e] += P[e2] * dosel[e];
          }
        }
      }
    }
    free(krows);
    free(P);
    free(dP);
  }
  for (int x = 0; x < 3; ++x) free(pq[x]);
  free(listed);
}

/* Dense global attention, the attention GSA replaces (Paper-Notes page,
 * section "研究背景与动机"): each listed token (special or image) attends,
 * in one softmax with the config scale, to all M tokens.  rows are token
 * ids t in [0, M); out: [n][H][d].  (For the benchmark comparator's
 * sampled rows.) */
void orc_dense(const orc_cfg* c, const void* q, const void* k, const void* v, const int64_t* rows, int64_t n,
               double* out) {
  const int H = c->n_heads, d = c->head_dim;
  const int64_t M = n_tokens(c);
#pragma omp parallel
  {
    int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * M);
    double* logits = (double*)malloc(sizeof(double) * M);
    double* qrow = (double*)malloc(sizeof(double) * d);
    for (int64_t t = 0; t < M; ++t) toks[t] = t;
#pragma omp for schedule(dynamic, 1)
    for (int64_t ih = 0; ih < n * H; ++ih) {
      const int64_t i = ih / H;
      const int h = (int)(ih % H);
      for (int e = 0; e < d; ++e) qrow[e] = elem(q, c->dtype, row_off(c, rows[i], h) + e);
      attend_tokens(c, qrow, k, v, toks, M, h, logits, out + (i * H + h) * d);
    }
    free(toks);
    free(logits);
    free(qrow);
  }
}

/* ======================================================================== */
/* Frame attention: the local step that alternates with GSA in the
 * aggregation transformer (Paper-Notes page, section "整体框架": blocks
 * alternate intra-frame attention and global sparse attention).  Each token
 * attends, in one softmax with the config scale, to every token of its own
 * frame (special and image, T_f keys); frames do not see each other.
 * rows[i] is a token id t in [0, M); out: [n][H][d]. */
void orc_frame(const orc_cfg* c, const void* q, const void* k, const void* v,
               const int64_t* rows, int64_t n, double* out) {
  const int H = c->n_heads, d = c->head_dim;
  const int64_t tf = tokens_per_frame(c);
#pragma omp parallel
  {
    int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * tf);
    double* logits = (double*)malloc(sizeof(double) * tf);
    double* qrow = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t ih = 0; ih < n * H; ++ih) {
      int64_t i = ih / H;
      int h = (int)(ih % H);
      int64_t t = rows[i], first = (t / tf) * tf;
      for (int64_t j = 0; j < tf; ++j) toks[j] = first + j;
      for (int e = 0; e < d; ++e) qrow[e] = elem(q, c->dtype, row_off(c, t, h) + e);
      attend_tokens(c, qrow, k, v, toks, tf, h, logits, out + (i * H + h) * d);
    }
    free(toks);
    free(logits);
    free(qrow);
  }
}

/* ======================================================================== */
/* FlashVGGT descriptor attention (Paper-Notes page "FlashVGGT: Efficient and
 * Scalable Visual Geometry Transformers with Compressed Descriptor
 * Attention", section "关键设计": spatially compressed descriptor tokens,
 * descriptor attention, and the auxiliary descriptor tokens of "关键发现").
 * The downsampling factor r is the config's pool field and the keyframes are
 * its ctx_frames list.
 *
 * The key/value set, in this order:
 *   1. descriptors: each frame's h x w image grid bilinearly resampled to
 *      (h/r) x (w/r), half-pixel centres: output (y, x) samples the input at
 *      ((y + 0.5) r - 0.5, (x + 0.5) r - 0.5); frame-major, then row-major;
 *   2. every token (special and image) of frame 0 and of each listed
 *      keyframe (list order, frame 0 not repeated);
 *   3. the special (camera) tokens of every other frame, frame-major. */

static int is_full_aux(const orc_cfg* c, int64_t f) { return f == 0 || is_ctx_frame(c, f); }

int64_t orc_descriptor_count(const orc_cfg* c) {
  const int r = c->pool;
  int64_t n = (int64_t)c->n_frames * (c->grid_h / r) * (c->grid_w / r);
  for (int64_t f = 0; f < c->n_frames; ++f)
    n += is_full_aux(c, f) ? tokens_per_frame(c) : c->n_special;
  return n;
}

/* One bilinear sample (a float, before rounding to the input precision):
 * the corner weights are the products of the row and column weights, the
 * four weighted values are added in the order (y0,x0), (y0,x1), (y1,x0),
 * (y1,x1) in float; a coordinate past the last row or column is clamped. */
static float bilinear_sample(const orc_cfg* c, const void* x, int64_t f, int y, int xx, int h, int e) {
  const int r = c->pool;
  const double sy = (y + 0.5) * r - 0.5, sx = (xx + 0.5) * r - 0.5;
  int y0 = (int)floor(sy), x0 = (int)floor(sx);
  const float fy = (float)(sy - y0), fx = (float)(sx - x0);
  int y1 = y0 + 1 < c->grid_h ? y0 + 1 : c->grid_h - 1;
  int x1 = x0 + 1 < c->grid_w ? x0 + 1 : c->grid_w - 1;
  const int64_t base = f * tokens_per_frame(c) + c->n_special;
  const int ys[2] = {y0, y1}, xs[2] = {x0, x1};
  const float wy[2] = {1.0f - fy, fy}, wx[2] = {1.0f - fx, fx};
  float acc = 0.0f;
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b) {
      const float w = wy[a] * wx[b];
      const float v = (float)elem(x, c->dtype, row_off(c, base + (int64_t)ys[a] * c->grid_w + xs[b], h) + e);
      acc = acc + w * v;
    }
  return acc;
}

/* The key (or value) set of x as float [n][H][d] (values exactly
 * representable in the input precision: descriptors are rounded to it). */
void orc_descriptor_set(const orc_cfg* c, const void* x, float* out) {
  const int r = c->pool, H = c->n_heads, d = c->head_dim;
  const int dh = c->grid_h / r, dw = c->grid_w / r;
  const int64_t tf = tokens_per_frame(c);
  const int64_t nd = (int64_t)c->n_frames * dh * dw;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nd; ++i) {
    const int64_t f = i / ((int64_t)dh * dw);
    const int y = (int)((i / dw) % dh), xx = (int)(i % dw);
    for (int h = 0; h < H; ++h)
      for (int e = 0; e < d; ++e) {
        const float m = bilinear_sample(c, x, f, y, xx, h, e);
        out[(i * H + h) * d + e] = c->dtype == 1 ? m : round_bf16(m);
      }
  }
  int64_t row = nd;
  int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (c->n_frames + 1));
  int n_full = 0;
  order[n_full++] = 0;
  for (int i = 0; i < c->n_ctx; ++i)
    if (c->ctx_frames[i] != 0) order[n_full++] = c->ctx_frames[i];
  for (int i = 0; i < n_full; ++i)
    for (int64_t t = 0; t < tf; ++t, ++row)
      for (int h = 0; h < H; ++h)
        for (int e = 0; e < d; ++e)
          out[(row * H + h) * d + e] = (float)elem(x, c->dtype, row_off(c, order[i] * tf + t, h) + e);
  for (int64_t f = 0; f < c->n_frames; ++f) {
    if (is_full_aux(c, f)) continue;
    for (int64_t t = 0; t < c->n_special; ++t, ++row)
      for (int h = 0; h < H; ++h)
        for (int e = 0; e < d; ++e)
          out[(row * H + h) * d + e] = (float)elem(x, c->dtype, row_off(c, f * tf + t, h) + e);
  }
  free(order);
}

/* Descriptor attention of the listed token rows: each query (any token, full
 * resolution) attends, in one softmax with the config scale, to all n_set
 * rows of the key/value set kd/vd (float [n_set][H][d]).  out: [n][H][d]. */
void orc_descriptor_attn(const orc_cfg* c, const void* q, const float* kd, const float* vd, int64_t n_set,
                         const int64_t* rows, int64_t n, double* out) {
  const int H = c->n_heads, d = c->head_dim;
  orc_cfg cf = *c;
  cf.dtype = 1; /* the set is float */
#pragma omp parallel
  {
    int64_t* toks = (int64_t*)malloc(sizeof(int64_t) * n_set);
    double* logits = (double*)malloc(sizeof(double) * n_set);
    double* qrow = (double*)malloc(sizeof(double) * d);
    for (int64_t t = 0; t < n_set; ++t) toks[t] = t;
#pragma omp for schedule(dynamic, 1)
    for (int64_t ih = 0; ih < n * H; ++ih) {
      int64_t i = ih / H;
      int h = (int)(ih % H);
      for (int e = 0; e < d; ++e) qrow[e] = elem(q, c->dtype, row_off(c, rows[i], h) + e);
      attend_tokens(&cf, qrow, kd, vd, toks, n_set, h, logits, out + (i * H + h) * d);
    }
    free(toks);
    free(logits);
    free(qrow);
  }
}

/* Token row of the qq-th pixel of window j (exported for the test harness,
 * which scatters per-window rows back into the token layout). */
int64_t orc_window_token(const orc_cfg* c, int64_t j, int qq) { return window_token(c, j, qq); }
