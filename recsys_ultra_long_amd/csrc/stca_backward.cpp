// stca_backward.cpp -- the training step's backward (include/stca.h,
// stca_backward): gradients of a loss through z for every STCA weight and
// every embedding row the forward read.
//
// Sequence (everything on the caller's stream, nothing kept between calls):
//   1. forward recompute: stca_forward on the staged path, keeping each
//      layer's o, attention output, scaled Q, K/V rows and softmax lse;
//   2. z head: [o_1..o_M | x_t] W_Z -> SwiGLU (+LN), backward to dW_Z, the
//      z FFN's weights, and the upstream gradients of every o_i and of x_t;
//   3. per layer, last to first: W_O (da, dW_O); the attention backward
//      (dQ per target, dK | dV per history item); the query side recomputed
//      from [o_1..o_{i-1} | x_t] (or x_t) and differentiated back through
//      W_Q, LN, SwiGLU and W_C into the o's of earlier layers and x_t; the
//      history side recomputed from the gathered rows X and differentiated
//      back through W_K | W_V, LN and SwiGLU into dX (summed over layers,
//      since every layer reads the same X) and the weight gradients;
//   4. per-item row gradients scattered into the table gradient.
// Every product is one call of the strided GEMM (grad_gemm.hip); the
// element-wise and row-wise derivatives are in grad_ops.hip; the attention
// backward in attn_bwd.hip.  ([Review] 核心公式 for the layer and the fusion,
// [Notes] §STCA for the history side reading the raw rows at every layer.)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <vector>

#include "grad_internal.h"
#include "stca.h"

using namespace stca;

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += up(bytes);
    return o;
  }
};

constexpr int kBwdChunkBlocks = 32;  // 1024 keys per attention-backward workgroup

struct BwdLayout {
  size_t fws = 0, fws_bytes = 0;
  size_t z = 0, o = 0, attn = 0, q = 0, kv = 0, lse = 0;
  size_t plan = 0;
  size_t xt = 0, ocat = 0, docat = 0, dxt = 0;
  size_t c = 0, h13 = 0, g = 0, y = 0, st = 0, qln = 0, dy = 0, dg = 0, dh13 = 0, dc = 0, da = 0, dq = 0;
  size_t da_lo = 0, dsum = 0, part_dq = 0;
  size_t X = 0, H13 = 0, G = 0, Y = 0, ST = 0, XT = 0, dKV = 0, dXT = 0, dY = 0, dG = 0, dH13 = 0, dX = 0;
  size_t ln_part = 0, gemm_part = 0;
  int64_t max_chunks = 0;
  // STCA_FLAG_DEDUP: the history backward runs over Rh = drows unique rows
  bool dedup = false;
  int64_t Rh = 0;
  size_t keys0 = 0, keys1 = 0, vals0 = 0, vals1 = 0, hist = 0, seg = 0, poff = 0, moff = 0, ppart = 0, dKVu = 0;
  size_t total = 0;
};

stca_config forward_cfg(const stca_config *c) {
  stca_config f = *c;
  f.path = STCA_PATH_STAGED;  // STCA_FLAG_DEDUP is kept: the recompute then encodes unique rows
  return f;
}

// Split-K choice: weight gradients (K = rows) aim at 2048 workgroups (the
// rows may be capped on the device, leaving only part of them live); a
// product over rows with few output tiles is split too (K = the width).
int split_weight_grad(int64_t m, int64_t n, int64_t k) { return gemm_split_for(m, n, k, 2048, 256); }
int split_rows(int64_t m, int64_t n, int64_t k) { return gemm_split_for(m, n, k, 512, 64); }

// Largest split-K partial buffer any product of the backward asks for (its
// GEMM refuses a split that would need more).
int64_t part_floats_needed(int64_t d, int64_t h, int64_t M, int64_t R, int64_t T) {
  int64_t best = 0;
  auto need = [&](int64_t m, int64_t n, int64_t k, bool wg) {
    const int sp = wg ? split_weight_grad(m, n, k) : split_rows(m, n, k);
    best = std::max(best, gemm_part_floats(m, n, sp));
  };
  for (int64_t rows : {R, T}) {  // weight gradients over the history items / targets
    need(d, h, rows, true);
    need(h, d, rows, true);
    need(d, d, rows, true);
  }
  for (int64_t k = 1; k <= M; ++k) {  // fusion and z maps: [o_1..o_k] blocks of width k d
    need(k * d, d, T, true);
    need(T, d, k * d, false);
    need(T, k * d, d, false);
  }
  // the query side's FFN and projections over the T target rows
  need(T, h, d, false);
  need(T, d, h, false);
  need(T, d, d, false);
  return best;
}

int make_layout(const stca_config *cfg, const stca_batch *b, BwdLayout &L) {
  const stca_config fc = forward_cfg(cfg);
  size_t fws = 0;
  int r = stca_workspace_size(&fc, b, &fws);
  if (r) return r;
  const int64_t d = cfg->d, h = cfg->hidden, M = cfg->M, H = cfg->H, dh = d / H;
  const int64_t T = b->n_tgt, R = b->n_hist;
  L.dedup = (cfg->flags & STCA_FLAG_DEDUP) && R > 0;
  const int64_t Rh = L.dedup ? dedup_rows(R) : R;  // rows of the history backward
  L.Rh = Rh;
  Carver cv;
  L.fws_bytes = fws;
  L.fws = cv.take(fws);
  L.z = cv.take(T * d * 4);
  L.o = cv.take(M * T * d * 4);
  L.attn = cv.take(M * T * d * 4);
  L.q = cv.take(M * T * d * 2);
  L.kv = cv.take(L.dedup ? 0 : M * 2 * R * d * 2);  // dedup: K/V read through the unique rows
  L.lse = cv.take(M * T * H * 4);
  L.plan = cv.take(4 * sizeof(int) * (size_t)(cfg->B + 1));
  L.xt = cv.take(T * d * 4);
  L.ocat = cv.take(T * M * d * 4);
  L.docat = cv.take(T * M * d * 4);
  L.dxt = cv.take(T * d * 4);
  L.c = cv.take(T * d * 4);
  L.h13 = cv.take(T * 2 * h * 4);
  L.g = cv.take(T * h * 4);
  L.y = cv.take(T * d * 4);
  L.st = cv.take(T * 2 * 4);
  L.qln = cv.take(T * d * 4);
  L.dy = cv.take(T * d * 4);
  L.dg = cv.take(T * h * 4);
  L.dh13 = cv.take(T * 2 * h * 4);
  L.dc = cv.take(T * d * 4);
  L.da = cv.take(T * d * 4);
  L.dq = cv.take(T * d * 4);
  L.da_lo = cv.take(T * d * 2);
  L.dsum = cv.take(T * H * 4);
  L.max_chunks = max_chunks(R, cfg->B, kBwdChunkBlocks);
  L.part_dq = cv.take((size_t)attn_bwd_part_floats(L.max_chunks, (int)H, (int)dh) * 4);
  L.dKV = cv.take(R * 2 * d * 2);
  L.X = cv.take(Rh * d * 2);
  L.H13 = cv.take(Rh * 2 * h * 4);
  L.G = cv.take(Rh * h * 2);
  L.Y = cv.take(Rh * d * 4);
  L.ST = cv.take(Rh * 2 * 4);
  L.XT = cv.take(Rh * d * 2);
  L.dXT = cv.take(Rh * d * 4);
  L.dY = cv.take(Rh * d * 2);
  L.dG = cv.take(Rh * h * 4);
  L.dH13 = cv.take(Rh * 2 * h * 2);
  L.dX = cv.take(Rh * d * 4);
  if (L.dedup) {
    L.keys0 = cv.take(R * 4);
    L.keys1 = cv.take(R * 4);
    L.vals0 = cv.take(R * 4);
    L.vals1 = cv.take(R * 4);
    L.hist = cv.take((size_t)radix_hist_ints(R) * 4);
    L.seg = cv.take((size_t)(Rh + 1) * 4);
    L.poff = cv.take((size_t)(Rh + 1) * 4);
    L.moff = cv.take((size_t)(Rh + 1) * 4);
    L.ppart = cv.take((size_t)agg_max_partials(R) * 2 * d * 4);
    L.dKVu = cv.take(Rh * 2 * d * 2);
  }
  L.ln_part = cv.take((size_t)2 * ln_part_rows(std::max(Rh, T)) * d * 4);
  L.gemm_part = cv.take((size_t)part_floats_needed(d, h, M, Rh, T) * 4);
  L.total = cv.off;
  return STCA_OK;
}

int validate(const stca_config *c, const stca_batch *b, const stca_weights *w, const float *dz, const stca_grads *g) {
  if (!c) return api_error(STCA_ERR_INVALID_ARG, "config is NULL");
  if (!b) return api_error(STCA_ERR_INVALID_ARG, "batch is NULL");
  if (c->dtype != STCA_BF16) return api_error(STCA_ERR_UNSUPPORTED, "stca_backward is bf16 only");
  if (c->qmode != STCA_Q_FUSION) return api_error(STCA_ERR_UNSUPPORTED, "stca_backward needs STCA_Q_FUSION");
  if (c->encoder != STCA_ENC_SWIGLU)
    return api_error(STCA_ERR_UNSUPPORTED, "stca_backward needs the SwiGLU history encoder");
  if (c->head_map || b->key_mask)
    return api_error(STCA_ERR_UNSUPPORTED, "stca_backward does not take Cross-Mask key_mask / head_map");
  if (c->H <= 0 || c->d % c->H) return api_error(STCA_ERR_INVALID_ARG, "d %% H != 0");
  const int dh = c->d / c->H;
  if (dh != 32 && dh != 64) return api_error(STCA_ERR_UNSUPPORTED, "stca_backward needs d_h 32 or 64 (got %d)", dh);
  if (b->max_tgt_per_user > 64)
    return api_error(STCA_ERR_UNSUPPORTED, "stca_backward serves at most 64 targets per user (got %d)",
                     b->max_tgt_per_user);
  if (!g) return api_error(STCA_ERR_INVALID_ARG, "grads is NULL");
  if (b->n_tgt > 0 && !dz) return api_error(STCA_ERR_INVALID_ARG, "dz is NULL");
  if (dz && !aligned16(dz)) return api_error(STCA_ERR_INVALID_ARG, "dz not 16-byte aligned");
  if (!w || !w->layers) return api_error(STCA_ERR_INVALID_ARG, "weights NULL");
  if (!g->layers) return api_error(STCA_ERR_INVALID_ARG, "grads->layers is NULL");
  const bool kvln = c->flags & STCA_FLAG_KV_LN, zln = c->flags & STCA_FLAG_Z_LN;
  auto ffn_ok = [&](const stca_ffn_grad &f, bool ln) {
    return f.w1 && f.w3 && f.w2 && (!ln || (f.ln_g && f.ln_b));
  };
  for (int i = 0; i < c->M; ++i) {
    const stca_layer_grad &l = g->layers[i];
    if (!ffn_ok(l.kv, kvln) || !ffn_ok(l.q, true) || !l.wk || !l.wv || !l.wq || !l.wo || (i > 0 && !l.wc))
      return api_error(STCA_ERR_INVALID_ARG, "gradient buffer NULL (layer %d)", i);
  }
  if (!ffn_ok(g->z, zln) || !g->wz) return api_error(STCA_ERR_INVALID_ARG, "z gradient buffer NULL");
  if ((c->flags & STCA_FLAG_DEDUP) && g->d_hist)
    return api_error(STCA_ERR_UNSUPPORTED,
                     "d_hist is not available with STCA_FLAG_DEDUP (the history backward runs per unique row)");
  const void *p16[] = {g->table, g->d_hist, g->d_tgt, g->z_out, g->dq_dump, g->da_dump, g->dkv_dump};
  for (const void *p : p16)
    if (p && !aligned16(p)) return api_error(STCA_ERR_INVALID_ARG, "gradient output %p not 16-byte aligned", p);
  return STCA_OK;
}

template <typename T> T *at(void *ws, size_t off) { return reinterpret_cast<T *>((char *)ws + off); }

}  // namespace

extern "C" {

int stca_backward_workspace_size(const stca_config *cfg, const stca_batch *batch, size_t *bytes) {
  api_clear_error();
  if (!bytes) return api_error(STCA_ERR_INVALID_ARG, "bytes is NULL");
  if (!cfg || !batch) return api_error(STCA_ERR_INVALID_ARG, "config or batch is NULL");
  if (cfg->encoder != STCA_ENC_SWIGLU)
    return api_error(STCA_ERR_UNSUPPORTED, "stca_backward needs the SwiGLU history encoder");
  BwdLayout L;
  int r = make_layout(cfg, batch, L);
  if (r) return r;
  *bytes = L.total;
  return STCA_OK;
}

int stca_backward(const stca_config *cfg, const stca_batch *batch, const stca_weights *w, const float *dz,
                  const stca_grads *gr, void *ws, size_t ws_bytes, void *stream) {
  api_clear_error();
  int r = validate(cfg, batch, w, dz, gr);
  if (r) return r;
  BwdLayout L;
  if ((r = make_layout(cfg, batch, L))) return r;
  if (!ws && L.total > 0) return api_error(STCA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (ws_bytes < L.total) return api_error(STCA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, L.total);
  if (ws && !aligned16(ws)) return api_error(STCA_ERR_INVALID_ARG, "workspace not 16-byte aligned");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int B = cfg->B, d = cfg->d, H = cfg->H, M = cfg->M, h = cfg->hidden, dh = d / H;
  const int64_t T = batch->n_tgt, R = batch->n_hist;
  const float qscale = 1.0f / std::sqrt((float)dh);
  const bool kvln = cfg->flags & STCA_FLAG_KV_LN, zln = cfg->flags & STCA_FLAG_Z_LN;
  hipError_t e = hipSuccess;
  auto hip_err = [&](const char *what) { return api_error(STCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e)); };
  if (gr->n_stage_events < 0 || (gr->n_stage_events > 0 && !gr->stage_events))
    return api_error(STCA_ERR_INVALID_ARG, "stage_events inconsistent with n_stage_events");
  auto rec = [&](int k) -> hipError_t {
    if (k < gr->n_stage_events && gr->stage_events[k])
      return hipEventRecord(reinterpret_cast<hipEvent_t>(gr->stage_events[k]), s);
    return hipSuccess;
  };

  // ---- 1. forward recompute (arguments checked before anything is enqueued)
  const stca_config fc = forward_cfg(cfg);
  stca_outputs fo;
  std::memset(&fo, 0, sizeof(fo));
  float *z = gr->z_out ? gr->z_out : at<float>(ws, L.z);
  float *o_all = at<float>(ws, L.o), *a_all = at<float>(ws, L.attn), *lse_all = at<float>(ws, L.lse);
  bf16_t *q_all = at<bf16_t>(ws, L.q), *kv_all = at<bf16_t>(ws, L.kv);
  fo.z = z;
  fo.o_layers = o_all;
  fo.attn = a_all;
  fo.q_dump = q_all;
  fo.kv_dump = L.dedup ? nullptr : kv_all;
  fo.lse = cfg->score == STCA_SCORE_SOFTMAX ? lse_all : nullptr;
  fo.dev_status = gr->dev_status;
  ForwardInternals fi;
  if ((r = forward_check(&fc, batch, w))) return r;
  if ((e = rec(0))) return hip_err("stage event");
  if ((r = forward_with_internals(&fc, batch, w, &fo, at<void>(ws, L.fws), L.fws_bytes, stream, &fi))) return r;
  if ((e = rec(1))) return hip_err("stage event");
  const int64_t Rh = L.Rh;
  const int *hdev = L.dedup ? fi.n_unique : nullptr;  // device cap on the history backward's rows

  float *dX = gr->d_hist ? gr->d_hist : at<float>(ws, L.dX);
  float *dxt = gr->d_tgt ? gr->d_tgt : at<float>(ws, L.dxt);
  float *gpart = at<float>(ws, L.gemm_part);
  const int64_t gpart_cap = part_floats_needed(d, h, M, L.Rh, T);
  float *lnpart = at<float>(ws, L.ln_part);
  if (T == 0 || B == 0) {  // nothing reads the history: every gradient is zero
    if (gr->d_hist && R > 0) {  // K = 0 product: writes beta * C = 0
      GemmArgs z0;
      std::memset(&z0, 0, sizeof(z0));
      z0.M = R;
      z0.N = d;
      z0.A = dX;
      z0.sak = 1;
      z0.B = dX;
      z0.sbk = 1;
      z0.C = dX;
      z0.scm = d;
      z0.scn = 1;
      z0.alpha = 1.f;
      if ((e = launch_gemm(z0, s))) return hip_err("zero d_hist");
    }
    return STCA_OK;
  }

  // ---- GEMM helper: C = alpha * A B + beta * C with explicit strides
  const int *gdev = nullptr;  // device cap applied by gemm(): rows (M) or, for split products, K
  // kind: kWgrad = a weight gradient (K = rows, split along K); kTgt = a
  // product over the target rows (split along the width when it has few
  // output tiles); kHist = a product over the history rows (never split:
  // thousands of tiles, and a device row cap under dedup)
  enum { kHist = 0, kWgrad = 1, kTgt = 2 };
  auto gemm = [&](int64_t Mm, int64_t Nn, int64_t Kk, const void *A, bool abf, int64_t sam, int64_t sak,
                  const void *Bp, bool bbf, int64_t sbk, int64_t sbn, float *C, int64_t scm, int64_t scn, float alpha,
                  float beta, int kind) -> hipError_t {
    GemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.M = Mm;
    g.N = Nn;
    g.K = Kk;
    g.A = A;
    g.sam = sam;
    g.sak = sak;
    g.a_bf16 = abf;
    g.B = Bp;
    g.sbk = sbk;
    g.sbn = sbn;
    g.b_bf16 = bbf;
    g.C = C;
    g.scm = scm;
    g.scn = scn;
    g.alpha = alpha;
    g.beta = beta;
    g.split = kind == kWgrad ? split_weight_grad(Mm, Nn, Kk) : kind == kTgt ? split_rows(Mm, Nn, Kk) : 1;
    g.part = gpart;
    g.part_cap = gpart_cap;
    g.dev_rows = gdev;
    g.dev_dim = gdev ? (kind == kWgrad ? 2 : 1) : 0;
    return launch_gemm(g, s);
  };
  // ---- 2. planner for the attention backward (its own chunking)
  Plan plan;
  plan.hoff = at<int>(ws, L.plan);
  plan.toff = plan.hoff + (B + 1);
  plan.pblk = plan.toff + (B + 1);
  plan.coff = plan.pblk + (B + 1);
  plan.prow = nullptr;
  if ((e = launch_plan(batch->hist_offsets, batch->tgt_offsets, B, R, T, batch->max_tgt_per_user, kBwdChunkBlocks, 1,
                       plan, gr->dev_status, s)))
    return hip_err("planner");

  const bf16_t *table = (const bf16_t *)batch->table;
  float *xt = at<float>(ws, L.xt), *ocat = at<float>(ws, L.ocat), *docat = at<float>(ws, L.docat);
  float *c = at<float>(ws, L.c), *h13 = at<float>(ws, L.h13), *g = at<float>(ws, L.g), *y = at<float>(ws, L.y);
  float *st = at<float>(ws, L.st), *qln = at<float>(ws, L.qln), *dy = at<float>(ws, L.dy), *dg = at<float>(ws, L.dg);
  float *dh13 = at<float>(ws, L.dh13), *dc = at<float>(ws, L.dc), *da = at<float>(ws, L.da), *dq = at<float>(ws, L.dq);
  const int64_t MD = (int64_t)M * d;
  if ((e = launch_gather_rows(table, cfg->table_rows, batch->tgt_ids, T, d, xt, false, s))) return hip_err("x_t");
  if ((e = launch_concat_layers(o_all, M, T, d, ocat, s))) return hip_err("concat");

  // SwiGLU FFN (+LN) forward over n rows of x (fp32) with bf16 weights f:
  // h13 = x [W1 | W3], g = SiLU(h1) h3, y = g W2, out = LN(y) (or y).
  auto ffn_fwd = [&](int64_t n, const float *x, const stca_ffn &f, bool ln, float *out) -> hipError_t {
    hipError_t er;
    if ((er = gemm(n, h, d, x, false, d, 1, f.w1, true, h, 1, h13, 2 * h, 1, 1.f, 0.f, kTgt))) return er;
    if ((er = gemm(n, h, d, x, false, d, 1, f.w3, true, h, 1, h13 + h, 2 * h, 1, 1.f, 0.f, kTgt))) return er;
    if ((er = launch_swiglu_fwd(h13, n, h, g, false, s))) return er;
    if ((er = gemm(n, d, h, g, false, h, 1, f.w2, true, d, 1, y, d, 1, 1.f, 0.f, kTgt))) return er;
    if (ln) return launch_ln_fwd(y, n, d, f.ln_g, f.ln_b, out, false, st, s);
    return hipSuccess;
  };
  // its backward from dout [n, d] to dx [n, d] (overwritten), weight grads +=
  auto ffn_bwd = [&](int64_t n, const float *x, const stca_ffn &f, const stca_ffn_grad &fg, bool ln, const float *dout,
                     float *dx) -> hipError_t {
    hipError_t er;
    const float *dyv = dout;
    if (ln) {
      if ((er = launch_ln_bwd(dout, y, st, n, d, f.ln_g, dy, false, fg.ln_g, fg.ln_b, lnpart, s))) return er;
      dyv = dy;
    }
    // dG = dY W2^T; dW2 += G^T dY
    if ((er = gemm(n, h, d, dyv, false, d, 1, f.w2, true, 1, d, dg, h, 1, 1.f, 0.f, kTgt))) return er;
    if ((er = gemm(h, d, n, g, false, 1, h, dyv, false, d, 1, fg.w2, d, 1, 1.f, 1.f, kWgrad))) return er;
    if ((er = launch_swiglu_bwd(dg, h13, n, h, dh13, false, s))) return er;
    // dW1 += x^T dH1, dW3 += x^T dH3
    if ((er = gemm(d, h, n, x, false, 1, d, dh13, false, 2 * h, 1, fg.w1, h, 1, 1.f, 1.f, kWgrad))) return er;
    if ((er = gemm(d, h, n, x, false, 1, d, dh13 + h, false, 2 * h, 1, fg.w3, h, 1, 1.f, 1.f, kWgrad))) return er;
    // dx = dH1 W1^T + dH3 W3^T
    if ((er = gemm(n, d, h, dh13, false, 2 * h, 1, f.w1, true, 1, h, dx, d, 1, 1.f, 0.f, kTgt))) return er;
    return gemm(n, d, h, dh13 + h, false, 2 * h, 1, f.w3, true, 1, h, dx, d, 1, 1.f, 1.f, kTgt);
  };

  // ---- 3. z head: cz = [o_1..o_M | x_t] W_Z, z = SwiGLU_Z(cz) (+LN)
  {
    if ((e = gemm(T, d, MD, ocat, false, MD, 1, w->wz, true, d, 1, c, d, 1, 1.f, 0.f, kTgt))) return hip_err("z");
    if ((e = gemm(T, d, d, xt, false, d, 1, (const bf16_t *)w->wz + MD * d, true, d, 1, c, d, 1, 1.f, 1.f, kTgt)))
      return hip_err("z");
    if ((e = ffn_fwd(T, c, w->z, zln, qln))) return hip_err("z ffn");
    if ((e = ffn_bwd(T, c, w->z, gr->z, zln, dz, dc))) return hip_err("z backward");
    // dW_Z += [o | x_t]^T dcz; d[o | x_t] = dcz W_Z^T
    if ((e = gemm(MD, d, T, ocat, false, 1, MD, dc, false, d, 1, gr->wz, d, 1, 1.f, 1.f, kWgrad))) return hip_err("dWz");
    if ((e = gemm(d, d, T, xt, false, 1, d, dc, false, d, 1, gr->wz + MD * d, d, 1, 1.f, 1.f, kWgrad)))
      return hip_err("dWz");
    if ((e = gemm(T, MD, d, dc, false, d, 1, w->wz, true, 1, d, docat, MD, 1, 1.f, 0.f, kTgt))) return hip_err("do");
    if ((e = gemm(T, d, d, dc, false, d, 1, (const bf16_t *)w->wz + MD * d, true, 1, d, dxt, d, 1, 1.f, 0.f, kTgt)))
      return hip_err("dx_t");
  }

  // ---- history rows, gathered once (every layer reads the same raw X)
  bf16_t *X = at<bf16_t>(ws, L.X);
  float *H13 = at<float>(ws, L.H13), *Y = at<float>(ws, L.Y), *ST = at<float>(ws, L.ST), *dXT = at<float>(ws, L.dXT);
  float *dG = at<float>(ws, L.dG);
  bf16_t *G = at<bf16_t>(ws, L.G), *XT = at<bf16_t>(ws, L.XT), *dY = at<bf16_t>(ws, L.dY);
  bf16_t *dH13 = at<bf16_t>(ws, L.dH13);
  const int *hids = L.dedup ? fi.uniq_rows : batch->hist_ids;
  if (R > 0 && (e = launch_gather_rows(table, cfg->table_rows, hids, Rh, d, X, true, s, hdev)))
    return hip_err("history gather");
  UniqueSumArgs ua;
  std::memset(&ua, 0, sizeof(ua));
  if (L.dedup) {  // items in (unique row, item) order, once for every layer
    ua.n = R;
    ua.max_u = Rh;
    ua.tok2u = fi.tok2u;
    ua.n_unique = fi.n_unique;
    ua.keys[0] = at<int>(ws, L.keys0);
    ua.keys[1] = at<int>(ws, L.keys1);
    ua.vals[0] = at<int>(ws, L.vals0);
    ua.vals[1] = at<int>(ws, L.vals1);
    ua.hist = at<int>(ws, L.hist);
    ua.seg = at<int>(ws, L.seg);
    ua.poff = at<int>(ws, L.poff);
    ua.moff = at<int>(ws, L.moff);
    ua.d2 = 2 * d;
    ua.ppart = at<float>(ws, L.ppart);
    ua.out = at<bf16_t>(ws, L.dKVu);
    if ((e = launch_unique_sort(ua, s))) return hip_err("unique sort");
  }
  if ((e = rec(2))) return hip_err("stage event");

  // ---- 4. layers, last to first
  for (int i = M - 1; i >= 0; --i) {
    const stca_layer &lw = w->layers[i];
    const stca_layer_grad &lg = gr->layers[i];
    const float *a_i = a_all + (size_t)i * T * d;
    float *do_i = docat + (size_t)i * d;
    // W_O: da = do W_O^T, dW_O += a^T do
    if ((e = gemm(T, d, d, do_i, false, MD, 1, lw.wo, true, 1, d, da, d, 1, 1.f, 0.f, kTgt))) return hip_err("da");
    if ((e = gemm(d, d, T, a_i, false, 1, d, do_i, false, MD, 1, lg.wo, d, 1, 1.f, 1.f, kWgrad))) return hip_err("dWo");
    if (gr->da_dump && (e = launch_add_rows(da, d, gr->da_dump + (size_t)i * T * d, d, T, d, false, s)))
      return hip_err("da dump");
    // attention backward
    bf16_t *dkv = gr->dkv_dump ? (bf16_t *)gr->dkv_dump + (size_t)i * R * 2 * d : at<bf16_t>(ws, L.dKV);
    {
      AttnBwdArgs ab;
      std::memset(&ab, 0, sizeof(ab));
      ab.d = d;
      ab.H = H;
      ab.dh = dh;
      ab.score = cfg->score;
      ab.B = B;
      ab.n_hist = R;
      ab.n_tgt = T;
      ab.nb = kBwdChunkBlocks;
      ab.plan = plan;
      ab.max_chunks = L.max_chunks;
      ab.q = q_all + (size_t)i * T * d;
      if (L.dedup) {
        ab.k = fi.ukv + (size_t)2 * i * fi.ukv_layer_elems;
        ab.v = fi.vrows + (size_t)i * fi.drows * d;
        ab.tok2u = fi.tok2u;
      } else {
        ab.k = kv_all + (size_t)i * 2 * R * d;
        ab.v = ab.k + (size_t)R * d;
      }
      ab.a = a_i;
      ab.da = da;
      ab.lse = lse_all + (size_t)i * T * H;
      ab.da_lo = at<bf16_t>(ws, L.da_lo);
      ab.dsum = at<float>(ws, L.dsum);
      ab.part_dq = at<float>(ws, L.part_dq);
      ab.dq = dq;
      ab.dkv = dkv;
      if ((e = launch_attn_bwd(ab, s))) return hip_err("attention backward");
    }
    if (gr->dq_dump && (e = launch_add_rows(dq, d, gr->dq_dump + (size_t)i * T * d, d, T, d, false, s)))
      return hip_err("dq dump");
    const int ev = 3 + 3 * (M - 1 - i);
    if ((e = rec(ev))) return hip_err("stage event");
    // query side of layer i, recomputed: c = x_t (i = 0) or [o_1..o_i-1 | x_t] W_C
    const float *cin = xt;
    if (i > 0) {
      const int64_t K1 = (int64_t)i * d;
      if ((e = gemm(T, d, K1, ocat, false, MD, 1, lw.wc, true, d, 1, c, d, 1, 1.f, 0.f, kTgt))) return hip_err("wc");
      if ((e = gemm(T, d, d, xt, false, d, 1, (const bf16_t *)lw.wc + K1 * d, true, d, 1, c, d, 1, 1.f, 1.f, kTgt)))
        return hip_err("wc");
      cin = c;
    }
    if ((e = ffn_fwd(T, cin, lw.q, true, qln))) return hip_err("query ffn");
    // Q = q W_Q / sqrt(d_h): dW_Q += q^T dQ / sqrt(d_h), dq = dQ W_Q^T / sqrt(d_h)
    if ((e = gemm(d, d, T, qln, false, 1, d, dq, false, d, 1, lg.wq, d, 1, qscale, 1.f, kWgrad))) return hip_err("dWq");
    if ((e = gemm(T, d, d, dq, false, d, 1, lw.wq, true, 1, d, qln, d, 1, qscale, 0.f, kTgt))) return hip_err("dq");
    if ((e = ffn_bwd(T, cin, lw.q, lg.q, true, qln, dc))) return hip_err("query backward");
    if (i > 0) {
      const int64_t K1 = (int64_t)i * d;
      if ((e = gemm(K1, d, T, ocat, false, 1, MD, dc, false, d, 1, lg.wc, d, 1, 1.f, 1.f, kWgrad))) return hip_err("dWc");
      if ((e = gemm(d, d, T, xt, false, 1, d, dc, false, d, 1, lg.wc + K1 * d, d, 1, 1.f, 1.f, kWgrad)))
        return hip_err("dWc");
      if ((e = gemm(T, K1, d, dc, false, d, 1, lw.wc, true, 1, d, docat, MD, 1, 1.f, 1.f, kTgt))) return hip_err("do");
      if ((e = gemm(T, d, d, dc, false, d, 1, (const bf16_t *)lw.wc + K1 * d, true, 1, d, dxt, d, 1, 1.f, 1.f, kTgt)))
        return hip_err("dx_t");
    } else {
      if ((e = launch_add_rows(dc, d, dxt, d, T, d, true, s))) return hip_err("dx_t");
    }
    if ((e = rec(ev + 1))) return hip_err("stage event");
    // history side of layer i, over the history items or (dedup) the unique
    // rows with each row's dK | dV summed over its items
    if (R > 0) {
      const bf16_t *dkvh = dkv;
      if (L.dedup) {
        ua.dkv = dkv;
        if ((e = launch_unique_sums(ua, s))) return hip_err("unique sums");
        dkvh = ua.out;
      }
      const stca_ffn &f = lw.kv;
      const stca_ffn_grad &fg = lg.kv;
      gdev = hdev;
      if ((e = gemm(Rh, h, d, X, true, d, 1, f.w1, true, h, 1, H13, 2 * h, 1, 1.f, 0.f, kHist))) return hip_err("h1");
      if ((e = gemm(Rh, h, d, X, true, d, 1, f.w3, true, h, 1, H13 + h, 2 * h, 1, 1.f, 0.f, kHist))) return hip_err("h3");
      if ((e = launch_swiglu_fwd(H13, Rh, h, G, true, s, hdev))) return hip_err("swiglu");
      if ((e = gemm(Rh, d, h, G, true, h, 1, f.w2, true, d, 1, Y, d, 1, 1.f, 0.f, kHist))) return hip_err("y");
      if ((e = launch_ln_fwd(Y, Rh, d, kvln ? f.ln_g : nullptr, f.ln_b, XT, true, ST, s, hdev))) return hip_err("ln");
      // dXt = dK W_K^T + dV W_V^T; dW_K += Xt^T dK, dW_V += Xt^T dV
      if ((e = gemm(Rh, d, d, dkvh, true, 2 * d, 1, lw.wk, true, 1, d, dXT, d, 1, 1.f, 0.f, kHist))) return hip_err("dxt");
      if ((e = gemm(Rh, d, d, dkvh + d, true, 2 * d, 1, lw.wv, true, 1, d, dXT, d, 1, 1.f, 1.f, kHist)))
        return hip_err("dxt");
      if ((e = gemm(d, d, Rh, XT, true, 1, d, dkvh, true, 2 * d, 1, lg.wk, d, 1, 1.f, 1.f, kWgrad))) return hip_err("dWk");
      if ((e = gemm(d, d, Rh, XT, true, 1, d, dkvh + d, true, 2 * d, 1, lg.wv, d, 1, 1.f, 1.f, kWgrad)))
        return hip_err("dWv");
      if ((e = launch_ln_bwd(dXT, Y, ST, Rh, d, kvln ? f.ln_g : nullptr, dY, true, fg.ln_g, fg.ln_b, lnpart, s, hdev)))
        return hip_err("ln backward");
      // dG = dY W2^T, dW2 += G^T dY
      if ((e = gemm(Rh, h, d, dY, true, d, 1, f.w2, true, 1, d, dG, h, 1, 1.f, 0.f, kHist))) return hip_err("dg");
      if ((e = gemm(h, d, Rh, G, true, 1, h, dY, true, d, 1, fg.w2, d, 1, 1.f, 1.f, kWgrad))) return hip_err("dW2");
      if ((e = launch_swiglu_bwd(dG, H13, Rh, h, dH13, true, s, hdev))) return hip_err("swiglu backward");
      if ((e = gemm(d, h, Rh, X, true, 1, d, dH13, true, 2 * h, 1, fg.w1, h, 1, 1.f, 1.f, kWgrad))) return hip_err("dW1");
      if ((e = gemm(d, h, Rh, X, true, 1, d, dH13 + h, true, 2 * h, 1, fg.w3, h, 1, 1.f, 1.f, kWgrad)))
        return hip_err("dW3");
      const float beta0 = i == M - 1 ? 0.f : 1.f;
      if ((e = gemm(Rh, d, h, dH13, true, 2 * h, 1, f.w1, true, 1, h, dX, d, 1, 1.f, beta0, kHist)))
        return hip_err("dx");
      if ((e = gemm(Rh, d, h, dH13 + h, true, 2 * h, 1, f.w3, true, 1, h, dX, d, 1, 1.f, 1.f, kHist)))
        return hip_err("dx");
      gdev = nullptr;
    }
    if ((e = rec(ev + 2))) return hip_err("stage event");
  }

  // ---- 5. row gradients into the table
  if (gr->table) {
    if (R > 0 && (e = launch_scatter_add(dX, hids, Rh, d, gr->table, cfg->table_rows, s, hdev)))
      return hip_err("scatter");
    if ((e = launch_scatter_add(dxt, batch->tgt_ids, T, d, gr->table, cfg->table_rows, s))) return hip_err("scatter");
  }
  if ((e = rec(3 + 3 * M))) return hip_err("stage event");
  return STCA_OK;
}

}  // extern "C"
