// stca_api.cpp -- the C ABI (include/stca.h): argument validation, workspace
// planning and the per-layer launch sequence of the STCA forward.
//
// Launch sequence of stca_forward (bf16 shown; fp32 is the same without the
// weight preparation):
//   1. weight preparation: every matrix re-laid as W^T in MFMA fragment order
//      (one batched launch) so each operand fragment is one contiguous 1 KB load;
//   2. planner: CSR validation, padded block offsets, split-L chunk offsets;
//   3. history side of every layer (gather -> SwiGLU FFN -> LN -> W_K | W_V)
//      into the blocked K/V buffers.  The history side never depends on the
//      query ([Notes] §STCA: each layer's FFN reads the raw rows), so all M
//      layers are encoded before the query chain starts -- for bf16 at
//      d <= 256 in one launch that gathers each tile once for all layers;
//   4. per layer: query (q1 from x_t, or the fusion of [o_1..o_i | x_t]),
//      Q = q W_Q / sqrt(d_h); attention partials and merge; o = attn W_O;
//   5. z = SwiGLU([o_1 | .. | o_M | x_t] W_Z) [+ LN]   (linear mode: z = O_M).
// On the fused path (bf16) step 3 disappears: per layer, after the query, one
// persistent kernel gathers, encodes and attends tile by tile, and no K/V
// buffer exists; the merge and W_O follow as above.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "grad_internal.h"
#include "stca.h"
#include "stca_internal.h"

using namespace stca;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(STCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace stca {
int api_error(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}
void api_clear_error() { g_err[0] = 0; }
}  // namespace stca

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += up(bytes);
    return o;
  }
};

// Offsets (elements) of the prepared (fragment-packed) bf16 weights of one layer.
struct PrepLayer {
  size_t kv_w1, kv_w3, kv_w2, wkv, q_w1, q_w3, q_w2, wq, wo, wc, r;
};

struct Layout {
  bool fused = false;
  int nb = 1;              // blocks per chunk
  int64_t max_blocks = 0;  // host bound
  int64_t max_chunks = 0;
  int tile_blocks = 1;     // users padded to this many 32-key blocks (fused: its tile)
  int64_t max_tiles = 0;   // fused: key tiles (host bound)
  int fused_grid = 0;      // fused: partial buffers hold this many workgroups
  size_t esize = 2;
  size_t prow = 0;         // staged bf16: padded-row id map (0 = none)
  bool dedup = false;      // STCA_FLAG_DEDUP: encoder over the unique ids
  int64_t drows = 0, dslots = 0;
  size_t d_keys = 0, d_slot = 0, d_bcnt = 0, d_boff = 0, d_uniq = 0, d_tok2u = 0, d_small = 0, d_sort = 0;
  size_t ukv = 0, ukv_layer = 0, vrows = 0;
  size_t plan = 0, prep = 0, kv = 0, kv_layer = 0, part_ml = 0, part_acc = 0, part_cnt = 0, fstate = 0;
  size_t xt = 0, ocat = 0, qs = 0, attn32 = 0, attnlo = 0, qcur = 0, total = 0;
  size_t hy_mp = 0, hy_g = 0, hy_h13 = 0, hy_gg = 0, hy_out = 0, hy_qcat = 0, hy_qmix = 0, hy_o32 = 0;
  size_t hy_pool = 0, hy_part = 0;
  int64_t hy_part_floats = 0;
  size_t bias = 0;         // score bias, blocked like K (0 = none)
  std::vector<PrepLayer> pl;
  size_t z_w1 = 0, z_w3 = 0, z_w2 = 0, wz = 0, prep_elems = 0;
};

// 32-key blocks per attention scheduling unit.  Units only set how finely
// the persistent grid's ranges can be cut (the partial count is set by the
// grid, not by the unit), so they are small: 128 keys.
int choose_nb(int chunk_keys) { return chunk_keys > 0 ? chunk_keys / 32 : 4; }

// Partial slots of the streaming attention: (grid cap + B H) x groups slots
// (one per segment of a workgroup and a (user, group, head) pair, or of a
// (user, head) pair and each of its groups), each with room for the targets of
// one group.
size_t partial_slots(int64_t B, int H, int max_tgt) {
  const int groups = (max_tgt + 63) / 64;
  const int tgs = groups > 1 ? 64 : max_tgt;
  return (size_t)(kAttnMaxGrid + B * H) * groups * tgs;
}

int validate_cfg(const stca_config *c) {
  if (!c) return fail(STCA_ERR_INVALID_ARG, "cfg is NULL");
  if (c->B < 0) return fail(STCA_ERR_INVALID_ARG, "B must be >= 0 (got %d)", c->B);
  if (c->H <= 0 || c->d <= 0 || c->d % c->H)
    return fail(STCA_ERR_INVALID_ARG, "d (%d) must be a positive multiple of H (%d)", c->d, c->H);
  const int dh = c->d / c->H;
  if (dh != 32 && dh != 64) return fail(STCA_ERR_UNSUPPORTED, "d_h = %d unsupported (32 or 64)", dh);
  if (c->M < 1 || c->M > 16) return fail(STCA_ERR_INVALID_ARG, "M = %d outside 1..16", c->M);
  if (c->dtype != STCA_F32 && c->dtype != STCA_BF16)
    return fail(STCA_ERR_INVALID_ARG, "dtype %d unknown", c->dtype);
  if (c->score != STCA_SCORE_SOFTMAX && c->score != STCA_SCORE_RELU)
    return fail(STCA_ERR_INVALID_ARG, "score %d unknown", c->score);
  if (c->qmode != STCA_Q_FUSION && c->qmode != STCA_Q_LINEAR && c->qmode != STCA_Q_HYFORMER)
    return fail(STCA_ERR_INVALID_ARG, "qmode %d unknown", c->qmode);
  if (c->qmode == STCA_Q_HYFORMER) {
    if (c->dtype != STCA_BF16) return fail(STCA_ERR_UNSUPPORTED, "STCA_Q_HYFORMER is bf16 only");
    if (c->path != STCA_PATH_STAGED) return fail(STCA_ERR_UNSUPPORTED, "STCA_Q_HYFORMER needs the staged path");
    if (c->n_ns < 0) return fail(STCA_ERR_INVALID_ARG, "n_ns %d < 0", c->n_ns);
    if (c->q_hidden <= 0 || c->q_hidden % 32)
      return fail(STCA_ERR_UNSUPPORTED, "q_hidden %d must be a positive multiple of 32", c->q_hidden);
  }
  if (c->path != STCA_PATH_STAGED && c->path != STCA_PATH_FUSED)
    return fail(STCA_ERR_INVALID_ARG, "path %d unknown", c->path);
  if (c->flags & ~(STCA_FLAG_KV_LN | STCA_FLAG_Z_LN | STCA_FLAG_DEDUP))
    return fail(STCA_ERR_INVALID_ARG, "unknown flag bits 0x%x", c->flags);
  if (c->chunk_keys < 0 || c->chunk_keys % 32)
    return fail(STCA_ERR_INVALID_ARG, "chunk_keys %d must be a multiple of 32", c->chunk_keys);
  if (c->table_rows <= 0 || c->table_rows >= (1ll << 31))
    return fail(STCA_ERR_INVALID_ARG, "table_rows %lld outside [1, 2^31)", (long long)c->table_rows);
  if (c->dtype == STCA_BF16) {
    if (c->d != 128 && c->d != 256 && c->d != 512)
      return fail(STCA_ERR_UNSUPPORTED, "bf16 supports d in {128, 256, 512} (got %d)", c->d);
    if (c->hidden <= 0 || c->hidden % 128)
      return fail(STCA_ERR_UNSUPPORTED, "bf16 needs hidden a positive multiple of 128 (got %d)", c->hidden);
  } else {
    if (c->d > 512 || c->d % 32)
      return fail(STCA_ERR_UNSUPPORTED, "fp32 supports d a multiple of 32 up to 512 (got %d)", c->d);
    if (c->hidden <= 0 || c->hidden % 32)
      return fail(STCA_ERR_UNSUPPORTED, "fp32 needs hidden a positive multiple of 32 (got %d)", c->hidden);
  }
  if (c->encoder != STCA_ENC_SWIGLU && c->encoder != STCA_ENC_LONGER)
    return fail(STCA_ERR_INVALID_ARG, "encoder %d unknown", c->encoder);
  if (c->encoder == STCA_ENC_LONGER) {
    if (c->dtype != STCA_BF16) return fail(STCA_ERR_UNSUPPORTED, "STCA_ENC_LONGER is bf16 only");
    if (c->path != STCA_PATH_STAGED) return fail(STCA_ERR_UNSUPPORTED, "STCA_ENC_LONGER needs the staged path");
    if (c->score != STCA_SCORE_SOFTMAX) return fail(STCA_ERR_UNSUPPORTED, "STCA_ENC_LONGER uses softmax scores");
    if (c->flags & STCA_FLAG_DEDUP) return fail(STCA_ERR_UNSUPPORTED, "STCA_ENC_LONGER is not available with STCA_FLAG_DEDUP");
    if (c->head_map) return fail(STCA_ERR_UNSUPPORTED, "STCA_ENC_LONGER is not available with Cross-Mask maps");
    if (c->l_short < 1 || c->l_short > 4096)
      return fail(STCA_ERR_INVALID_ARG, "l_short %d outside 1..4096", c->l_short);
  }
  return STCA_OK;
}

// What the fused kernel is built for.
int validate_dedup(const stca_config *c) {
  if (!(c->flags & STCA_FLAG_DEDUP)) return STCA_OK;
  if (c->dtype != STCA_BF16) return fail(STCA_ERR_UNSUPPORTED, "STCA_FLAG_DEDUP is bf16 only");
  if (c->path != STCA_PATH_STAGED) return fail(STCA_ERR_UNSUPPORTED, "STCA_FLAG_DEDUP needs the staged path");
  return STCA_OK;
}

int validate_map(const int32_t *map, int H) {
  if (!map) return STCA_OK;
  if (H > 16) return fail(STCA_ERR_UNSUPPORTED, "head_map supports at most 16 heads (got %d)", H);
  for (int h = 0; h < H; ++h)
    if (map[h] < 0 || map[h] >= H) return fail(STCA_ERR_INVALID_ARG, "head_map[%d] = %d outside [0, %d)", h, map[h], H);
  return STCA_OK;
}

// Cross-Mask masks and maps, and the score bias: the staged bf16 attention
// implements them
int validate_cross_mask(const stca_config *c, const stca_batch *b) {
  const bool any = c->head_map || (b && (b->key_mask || b->score_bias));
  if (!any) return STCA_OK;
  if (c->dtype != STCA_BF16) return fail(STCA_ERR_UNSUPPORTED, "key_mask / head_map / score_bias need bf16");
  if (c->path != STCA_PATH_STAGED)
    return fail(STCA_ERR_UNSUPPORTED, "key_mask / head_map / score_bias need the staged path");
  if (b && b->key_mask && ((reinterpret_cast<uintptr_t>(b->key_mask) & 15u)))
    return fail(STCA_ERR_INVALID_ARG, "key_mask not 16-byte aligned");
  if (b && b->score_bias && ((reinterpret_cast<uintptr_t>(b->score_bias) & 15u)))
    return fail(STCA_ERR_INVALID_ARG, "score_bias not 16-byte aligned");
  if (b && b->score_bias && c->H > 16) return fail(STCA_ERR_UNSUPPORTED, "score_bias supports at most 16 heads");
  return validate_map(c->head_map, c->H);
}

int validate_fused(const stca_config *c, const stca_batch *b) {
  if (c->path != STCA_PATH_FUSED) return STCA_OK;
  const int dh = c->d / c->H;
  if (c->dtype != STCA_BF16) return fail(STCA_ERR_UNSUPPORTED, "fused path is bf16 only");
  if (!((c->d == 256 && (dh == 32 || dh == 64)) || (c->d == 128 && dh == 32)))
    return fail(STCA_ERR_UNSUPPORTED, "fused path supports d = 256 (d_h 32, 64) or d = 128 (d_h 32); got d = %d, d_h = %d",
                c->d, dh);
  if (!(c->flags & STCA_FLAG_KV_LN))
    return fail(STCA_ERR_UNSUPPORTED, "fused path needs STCA_FLAG_KV_LN (LN after the history FFN)");
  if (b && b->max_tgt_per_user > 64)
    return fail(STCA_ERR_UNSUPPORTED, "fused path serves at most 64 targets per user (got %d)", b->max_tgt_per_user);
  return STCA_OK;
}

int validate_batch(const stca_config *c, const stca_batch *b) {
  if (!b) return fail(STCA_ERR_INVALID_ARG, "batch is NULL");
  if (b->n_hist < 0 || b->n_hist >= (1ll << 31))
    return fail(STCA_ERR_INVALID_ARG, "n_hist %lld outside [0, 2^31)", (long long)b->n_hist);
  if (b->n_tgt < 0 || b->n_tgt >= (1ll << 31))
    return fail(STCA_ERR_INVALID_ARG, "n_tgt %lld outside [0, 2^31)", (long long)b->n_tgt);
  if (b->max_tgt_per_user < 1 || b->max_tgt_per_user > 4096)
    return fail(STCA_ERR_INVALID_ARG, "max_tgt_per_user %d outside 1..4096", b->max_tgt_per_user);
  if (c->B == 0 && (b->n_hist || b->n_tgt))
    return fail(STCA_ERR_INVALID_ARG, "B = 0 with n_hist = %lld, n_tgt = %lld", (long long)b->n_hist,
                (long long)b->n_tgt);
  if (c->B > 0 && (!b->hist_offsets || !b->tgt_offsets))
    return fail(STCA_ERR_INVALID_ARG, "hist_offsets / tgt_offsets must not be NULL");
  if (b->n_hist > 0 && !b->hist_ids) return fail(STCA_ERR_INVALID_ARG, "hist_ids is NULL");
  if (!b->table) return fail(STCA_ERR_INVALID_ARG, "table is NULL");
  if (c->qmode == STCA_Q_FUSION && b->n_tgt > 0 && !b->tgt_ids)
    return fail(STCA_ERR_INVALID_ARG, "tgt_ids is NULL (fusion mode)");
  if (c->qmode == STCA_Q_LINEAR && b->n_tgt > 0 && !b->q0)
    return fail(STCA_ERR_INVALID_ARG, "q0 is NULL (linear mode)");
  if (c->qmode == STCA_Q_HYFORMER) {
    const int m = b->max_tgt_per_user, T = m + c->n_ns;
    if (b->n_tgt != (int64_t)c->B * m)
      return fail(STCA_ERR_INVALID_ARG, "STCA_Q_HYFORMER: n_tgt %lld != B * max_tgt_per_user (%d * %d)",
                  (long long)b->n_tgt, c->B, m);
    if (c->d % T) return fail(STCA_ERR_UNSUPPORTED, "STCA_Q_HYFORMER: m + n_ns = %d must divide d = %d", T, c->d);
    if (c->n_ns > 0 && b->n_tgt > 0 && !b->ns_feats) return fail(STCA_ERR_INVALID_ARG, "ns_feats is NULL");
    if (b->ns_feats && !aligned16(b->ns_feats)) return fail(STCA_ERR_INVALID_ARG, "ns_feats not 16-byte aligned");
  }
  const void *ptrs[] = {b->hist_offsets, b->hist_ids, b->tgt_offsets, b->tgt_ids, b->q0, b->table};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return fail(STCA_ERR_INVALID_ARG, "batch pointer %p not 16-byte aligned", p);
  if (c->encoder == STCA_ENC_LONGER && b->key_mask)
    return fail(STCA_ERR_UNSUPPORTED, "STCA_ENC_LONGER is not available with Cross-Mask masks");
  if (c->encoder == STCA_ENC_LONGER && b->score_bias)
    return fail(STCA_ERR_UNSUPPORTED, "STCA_ENC_LONGER is not available with a score bias");
  int r = validate_dedup(c);
  if (r) return r;
  if ((r = validate_cross_mask(c, b))) return r;
  return validate_fused(c, b);
}

int check_ffn(const stca_ffn &f, bool ln, const char *name, int layer) {
  if (!f.w1 || !f.w3 || !f.w2) return fail(STCA_ERR_INVALID_ARG, "%s FFN matrix NULL (layer %d)", name, layer);
  if (ln && (!f.ln_g || !f.ln_b)) return fail(STCA_ERR_INVALID_ARG, "%s LN params NULL (layer %d)", name, layer);
  const void *ptrs[] = {f.w1, f.w3, f.w2, f.ln_g, f.ln_b};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return fail(STCA_ERR_INVALID_ARG, "%s weight not 16-byte aligned (layer %d)", name, layer);
  return STCA_OK;
}

int validate_weights(const stca_config *c, const stca_weights *w) {
  if (!w || !w->layers) return fail(STCA_ERR_INVALID_ARG, "weights / weights->layers is NULL");
  const bool kvln = c->flags & STCA_FLAG_KV_LN;
  for (int i = 0; i < c->M; ++i) {
    const stca_layer &l = w->layers[i];
    int r = STCA_OK;
    if (c->encoder == STCA_ENC_LONGER) {  // the history FFN is not used
      const void *em[] = {l.enc_wq, l.enc_wk, l.enc_wv, l.enc_wo};
      for (const void *p : em)
        if (!p || !aligned16(p)) return fail(STCA_ERR_INVALID_ARG, "encoder weight NULL or misaligned (layer %d)", i);
    } else if ((r = check_ffn(l.kv, kvln, "kv", i))) {
      return r;
    }
    const void *mats[] = {l.wk, l.wv, l.wq, l.wo};
    for (const void *p : mats) {
      if (!p) return fail(STCA_ERR_INVALID_ARG, "W_K/W_V/W_Q/W_O NULL (layer %d)", i);
      if (!aligned16(p)) return fail(STCA_ERR_INVALID_ARG, "layer %d weight not 16-byte aligned", i);
    }
    if (c->qmode == STCA_Q_FUSION) {
      if ((r = check_ffn(l.q, true, "q", i))) return r;
      if (i > 0 && !l.wc) return fail(STCA_ERR_INVALID_ARG, "W_C NULL (layer %d)", i);
      if (l.wc && !aligned16(l.wc)) return fail(STCA_ERR_INVALID_ARG, "W_C not aligned (layer %d)", i);
    } else if (c->qmode == STCA_Q_LINEAR && i + 1 < c->M) {
      if (!l.r) return fail(STCA_ERR_INVALID_ARG, "R NULL (layer %d, linear mode)", i);
      if (!aligned16(l.r)) return fail(STCA_ERR_INVALID_ARG, "R not aligned (layer %d)", i);
    }
  }
  if (c->qmode == STCA_Q_HYFORMER) {
    const void *qm[] = {w->qgen_w1, w->qgen_w3, w->qgen_w2};
    for (const void *p : qm)
      if (!p || !aligned16(p)) return fail(STCA_ERR_INVALID_ARG, "query-generation weight NULL or misaligned");
    for (int i = 0; i < c->M; ++i) {
      const stca_layer &l = w->layers[i];
      const void *bm[] = {l.boost_w1, l.boost_w3, l.boost_w2};
      for (const void *p : bm)
        if (!p || !aligned16(p)) return fail(STCA_ERR_INVALID_ARG, "boosting weight NULL or misaligned (layer %d)", i);
    }
  }
  if (c->qmode == STCA_Q_FUSION) {
    int r = check_ffn(w->z, c->flags & STCA_FLAG_Z_LN, "z", c->M);
    if (r) return r;
    if (!w->wz) return fail(STCA_ERR_INVALID_ARG, "W_Z is NULL");
    if (!aligned16(w->wz)) return fail(STCA_ERR_INVALID_ARG, "W_Z not aligned");
  }
  return STCA_OK;
}

// Split-K of the HyFormer query FFN products: n problems of [M x N] over K,
// aiming at ~512 workgroups in all.
int hy_split(int64_t n, int64_t M, int64_t N, int64_t K) {
  return gemm_split_for(M, N, K, std::max<int64_t>(1, 512 / std::max<int64_t>(n, 1)), 128);
}
int64_t hy_part_floats(int64_t n, int64_t M, int64_t N, int64_t K) {
  const int sp = hy_split(n, M, N, K);
  return sp > 1 ? n * sp * M * N : 0;
}

Layout make_layout(const stca_config *c, const stca_batch *b) {
  Layout L;
  const int64_t d = c->d, h = c->hidden, T = b->n_tgt;
  const int dh = c->d / c->H;
  L.esize = c->dtype == STCA_BF16 ? 2 : 4;
  L.fused = c->path == STCA_PATH_FUSED;
  L.nb = choose_nb(c->chunk_keys);
  L.tile_blocks = L.fused ? fused_tile_blocks(c->d) : 1;
  L.max_blocks = max_blocks(b->n_hist, c->B, L.tile_blocks);
  L.max_chunks = max_chunks(b->n_hist, c->B, L.nb);
  L.max_tiles = fused_max_tiles(b->n_hist, c->B, L.fused ? L.tile_blocks : 2);
  L.fused_grid = (int)fused_grid_bound(L.max_tiles);
  Carver cv;
  L.plan = cv.take(4 * sizeof(int) * (size_t)(c->B + 1));
  L.dedup = (c->flags & STCA_FLAG_DEDUP) && b->n_hist > 0;
  if (c->dtype == STCA_BF16 && !L.fused && b->n_hist > 0 && !L.dedup)
    L.prow = cv.take(sizeof(int) * (size_t)prow_rows(L.max_blocks));
  if (L.dedup) {
    L.drows = dedup_rows(b->n_hist);
    L.dslots = dedup_slots(b->n_hist);
    L.d_keys = cv.take(sizeof(int) * (size_t)L.dslots);
    L.d_slot = cv.take(sizeof(int) * (size_t)L.dslots);
    L.d_bcnt = cv.take(sizeof(int) * (size_t)(L.dslots / 256));
    L.d_boff = cv.take(sizeof(int) * (size_t)(L.dslots / 256));
    L.d_uniq = cv.take(sizeof(int) * (size_t)L.drows);
    L.d_tok2u = cv.take(sizeof(int) * (size_t)b->n_hist);
    L.d_small = cv.take(sizeof(int) * 8);
    L.d_sort = cv.take(sizeof(int) * (size_t)L.drows * 6 + sizeof(int) * (size_t)radix_hist_ints(L.drows));
    L.ukv_layer = (size_t)L.drows * d * 2;  // K or V of the unique rows, one layer
    L.ukv = cv.take(2 * L.ukv_layer * c->M);
    L.vrows = cv.take(L.ukv_layer * c->M);  // each layer's unique V, row-major
  }
  if (c->dtype == STCA_BF16) {
    size_t e = 0;
    L.pl.resize(c->M);
    for (int i = 0; i < c->M; ++i) {
      PrepLayer &p = L.pl[i];
      p.kv_w1 = e; e += h * d;
      p.kv_w3 = e; e += h * d;
      p.kv_w2 = e; e += h * d;
      p.wkv = e; e += 2 * d * d;
      p.wq = e; e += d * d;
      p.wo = e; e += d * d;
      if (c->qmode == STCA_Q_FUSION) {
        p.q_w1 = e; e += h * d;
        p.q_w3 = e; e += h * d;
        p.q_w2 = e; e += h * d;
        if (i > 0) { p.wc = e; e += d * (i + 1) * d; }
      } else if (c->qmode == STCA_Q_LINEAR) {
        p.r = e; e += d * d;
      }
    }
    if (c->qmode == STCA_Q_FUSION) {
      L.z_w1 = e; e += h * d;
      L.z_w3 = e; e += h * d;
      L.z_w2 = e; e += h * d;
      L.wz = e; e += d * (c->M + 1) * d;
    }
    L.prep_elems = e;
    L.prep = cv.take(e * 2);
  }
  // staged: blocked K/V of every layer; fused: none (the point of that path)
  L.kv_layer = L.fused ? 0 : (size_t)L.max_blocks * 32 * d * L.esize;  // K or V of one layer
  L.kv = cv.take(2 * L.kv_layer * c->M);
  if (b->score_bias && b->n_hist > 0) L.bias = cv.take((size_t)L.max_blocks * c->H * 32 * sizeof(float));
  size_t np = partial_slots(c->B, c->H, b->max_tgt_per_user);
  if (L.fused)  // one slot per (workgroup, user): independent of the history length
    np = (size_t)(L.fused_grid + c->B) * c->H * b->max_tgt_per_user;
  L.part_ml = cv.take(np * 2 * sizeof(float));
  L.part_acc = cv.take(np * dh * sizeof(float));
  L.part_cnt = cv.take(np * sizeof(int));
  if (L.fused) L.fstate = cv.take(fused_state_bytes(c->d, dh, L.fused_grid));
  L.xt = cv.take(T * d * L.esize);
  L.ocat = cv.take(T * d * c->M * L.esize);
  L.qs = cv.take(T * d * L.esize);
  L.attn32 = cv.take(T * d * sizeof(float));
  L.attnlo = cv.take(T * d * L.esize);
  L.qcur = cv.take(T * d * L.esize);
  if (c->qmode == STCA_Q_HYFORMER) {  // query generation and boosting (fp32)
    const int64_t m = b->max_tgt_per_user, Tk = m + c->n_ns, hq = c->q_hidden, Bu = c->B;
    const int64_t stack = std::max(m, Tk) * Bu;
    L.hy_mp = cv.take(Bu * d * 4);
    L.hy_g = cv.take(Bu * (c->n_ns + 1) * d * 4);
    L.hy_h13 = cv.take(stack * 2 * hq * 4);
    L.hy_gg = cv.take(stack * hq * 4);
    L.hy_out = cv.take(stack * d * 4);
    L.hy_qcat = cv.take(Bu * Tk * d * 4);
    L.hy_qmix = cv.take(Bu * Tk * d * 4);
    L.hy_o32 = cv.take(T * d * 4);
    L.hy_pool = cv.take((size_t)mean_pool_part_floats(c->B, (int)d) * 4);
    const int64_t din = (int64_t)(c->n_ns + 1) * d;
    int64_t pf = std::max({hy_part_floats(m, Bu, hq, din), hy_part_floats(Tk, Bu, hq, d),
                           hy_part_floats(m, Bu, d, hq), hy_part_floats(Tk, Bu, d, hq)});
    L.hy_part_floats = pf;
    L.hy_part = cv.take((size_t)pf * 4);
  }
  L.total = cv.off;
  return L;
}

template <typename T> T *at(void *ws, size_t off) { return reinterpret_cast<T *>((char *)ws + off); }

// LONGER-style encoding ([HyFormer] eq. (6), (8)): workspace of the pre-pass
// that turns every layer's raw history into its short rows H_l.  The forward
// proper then runs over the short rows (a batch whose history is the short
// sequences and whose "table" is the stack of H_l), after this area.
struct LongerLayout {
  int64_t nS = 0;             // host bound on the short rows: min(n_hist, B * l_short)
  int64_t mb = 0, mc = 0;     // raw history: max 32-key blocks, chunks
  int nb = 4;
  size_t plan = 0, soff = 0, sids = 0, iota = 0, prep = 0, kv = 0, kvl = 0;
  size_t ml = 0, acc = 0, cnt = 0, qe = 0, a32 = 0, alo = 0, htab = 0, total = 0;
};

LongerLayout make_longer_layout(const stca_config *c, const stca_batch *b) {
  LongerLayout LL;
  const int64_t d = c->d;
  LL.nS = std::min<int64_t>(b->n_hist, (int64_t)c->B * c->l_short);
  LL.nb = choose_nb(c->chunk_keys);
  LL.mb = max_blocks(b->n_hist, c->B, 1);
  LL.mc = max_chunks(b->n_hist, c->B, LL.nb);
  const size_t rows = (size_t)std::max<int64_t>(LL.nS, 1);
  Carver cv;
  LL.plan = cv.take(4 * sizeof(int) * (size_t)(c->B + 1));
  LL.soff = cv.take(sizeof(int) * (size_t)(c->B + 1));
  LL.sids = cv.take(sizeof(int) * rows);
  LL.iota = cv.take(sizeof(int) * rows);
  LL.prep = cv.take((size_t)c->M * 4 * d * d * 2);  // per layer: W'_Q, W'_K | W'_V, W'_O (packed bf16)
  LL.kvl = (size_t)LL.mb * 32 * d * 2;
  LL.kv = cv.take(2 * LL.kvl);
  const size_t np = partial_slots(c->B, c->H, c->l_short);
  LL.ml = cv.take(np * 2 * sizeof(float));
  LL.acc = cv.take(np * (d / c->H) * sizeof(float));
  LL.cnt = cv.take(np * sizeof(int));
  LL.qe = cv.take(rows * d * 2);
  LL.a32 = cv.take(rows * d * 4);
  LL.alo = cv.take(rows * d * 2);
  LL.htab = cv.take((size_t)c->M * rows * d * 2);
  LL.total = cv.off;
  return LL;
}

// What the forward over the short rows needs of the caller's batch.
struct LongerInner {
  const stca_batch *raw;   // the caller's batch (raw history, targets, table)
  Plan raw_plan;           // offsets of the raw history (HyFormer mean pool)
  int64_t raw_table_rows;  // rows of the caller's table
  int64_t layer_rows;      // short rows per layer in the stacked table
};

// The configuration and batch of the forward over the short rows.  Pointers
// into `ws` (which may be NULL when only sizes are wanted).
void longer_inner(const stca_config *c, const stca_batch *b, const LongerLayout &LL, void *ws,
                  stca_config &c2, stca_batch &b2) {
  c2 = *c;
  c2.encoder = STCA_ENC_SWIGLU;
  c2.flags &= ~STCA_FLAG_KV_LN;
  c2.table_rows = std::max<int64_t>(LL.nS, 1);
  b2 = *b;
  b2.hist_offsets = at<int>(ws, LL.soff);
  b2.hist_ids = at<int>(ws, LL.iota);
  b2.n_hist = LL.nS;
  b2.table = at<void>(ws, LL.htab);
  b2.key_mask = nullptr;
  b2.score_bias = nullptr;
}

}  // namespace

extern "C" {

int stca_version(void) { return 100; }

const char *stca_status_string(int s) {
  switch (s) {
    case STCA_OK: return "STCA_OK";
    case STCA_ERR_INVALID_ARG: return "STCA_ERR_INVALID_ARG";
    case STCA_ERR_UNSUPPORTED: return "STCA_ERR_UNSUPPORTED";
    case STCA_ERR_WORKSPACE: return "STCA_ERR_WORKSPACE";
    case STCA_ERR_HIP: return "STCA_ERR_HIP";
    default: return "STCA_ERR_UNKNOWN";
  }
}

const char *stca_last_error(void) { return g_err; }

int stca_workspace_size(const stca_config *cfg, const stca_batch *batch, size_t *bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(STCA_ERR_INVALID_ARG, "bytes is NULL");
  int r = validate_cfg(cfg);
  if (r) return r;
  if ((r = validate_batch(cfg, batch))) return r;
  if (cfg->encoder == STCA_ENC_LONGER) {
    const LongerLayout LL = make_longer_layout(cfg, batch);
    stca_config c2;
    stca_batch b2;
    longer_inner(cfg, batch, LL, nullptr, c2, b2);
    *bytes = LL.total + make_layout(&c2, &b2).total;
    return STCA_OK;
  }
  *bytes = make_layout(cfg, batch).total;
  return STCA_OK;
}

}  // extern "C"

namespace stca {

int forward_body(const stca_config *cfg, const stca_batch *batch, const stca_weights *w, const stca_outputs *out,
                 void *ws, size_t ws_bytes, void *stream, ForwardInternals *fi, const LongerInner *li);
int longer_forward(const stca_config *cfg, const stca_batch *batch, const stca_weights *w, const stca_outputs *out,
                   void *ws, size_t ws_bytes, void *stream);

int forward_check(const stca_config *cfg, const stca_batch *batch, const stca_weights *w) {
  int r = validate_cfg(cfg);
  if (r) return r;
  if ((r = validate_batch(cfg, batch))) return r;
  return validate_weights(cfg, w);
}

// Where the forward leaves its unique-row buffers in `ws` (STCA_FLAG_DEDUP).
void set_internals(const Layout &L, void *ws, ForwardInternals *fi) {
  std::memset(fi, 0, sizeof(*fi));
  if (!L.dedup) return;
  fi->dedup = true;
  fi->tok2u = at<int>(ws, L.d_tok2u);
  fi->uniq_rows = at<int>(ws, L.d_uniq);
  fi->n_unique = at<int>(ws, L.d_small);
  fi->drows = L.drows;
  fi->ukv = at<bf16_t>(ws, L.ukv);
  fi->ukv_layer_elems = L.ukv_layer / 2;
  fi->vrows = at<bf16_t>(ws, L.vrows);
}

void forward_internals(const stca_config *cfg, const stca_batch *batch, void *ws, ForwardInternals *fi) {
  set_internals(make_layout(cfg, batch), ws, fi);
}

int forward_with_internals(const stca_config *cfg, const stca_batch *batch, const stca_weights *w,
                           const stca_outputs *out, void *ws, size_t ws_bytes, void *stream, ForwardInternals *fi) {
  g_err[0] = 0;
  if (fi) std::memset(fi, 0, sizeof(*fi));
  int r = validate_cfg(cfg);
  if (r) return r;
  if ((r = validate_batch(cfg, batch))) return r;
  if ((r = validate_weights(cfg, w))) return r;
  if (!out) return fail(STCA_ERR_INVALID_ARG, "outputs is NULL");
  if (!out->z && batch->n_tgt > 0) return fail(STCA_ERR_INVALID_ARG, "outputs->z is required");
  {
    const void *ptrs[] = {out->z, out->o_layers, out->attn, out->active, out->q_dump, out->kv_dump,
                          out->x_dump, out->dev_status, out->lse};
    for (const void *p : ptrs)
      if (p && (reinterpret_cast<uintptr_t>(p) & 3u)) return fail(STCA_ERR_INVALID_ARG, "output pointer %p misaligned", p);
    const void *p16[] = {out->z, out->o_layers, out->attn, out->q_dump, out->x_dump};
    for (const void *p : p16)
      if (p && !aligned16(p)) return fail(STCA_ERR_INVALID_ARG, "output pointer %p not 16-byte aligned", p);
  }
  if ((cfg->flags & STCA_FLAG_DEDUP) && out->x_dump)
    return fail(STCA_ERR_UNSUPPORTED, "x_dump is not available with STCA_FLAG_DEDUP (the encoder gathers unique rows)");
  if (cfg->path == STCA_PATH_FUSED && out->kv_dump)
    return fail(STCA_ERR_UNSUPPORTED, "kv_dump needs the staged path (the fused path keeps no K/V)");
  if (cfg->encoder == STCA_ENC_LONGER) {
    if (fi) return fail(STCA_ERR_UNSUPPORTED, "the backward of STCA_ENC_LONGER is not available");
    if (out->x_dump || out->kv_dump)
      return fail(STCA_ERR_UNSUPPORTED, "x_dump / kv_dump are not available with STCA_ENC_LONGER");
    return longer_forward(cfg, batch, w, out, ws, ws_bytes, stream);
  }
  return forward_body(cfg, batch, w, out, ws, ws_bytes, stream, fi, nullptr);
}

// The forward after validation.  li != NULL: the history of `batch` is the
// short rows of a LONGER-style encoding (its table the stacked H_l, one block
// of rows per layer, already encoded); target-side gathers and the HyFormer
// mean pool read the caller's raw table and history through li.
int forward_body(const stca_config *cfg, const stca_batch *batch, const stca_weights *w, const stca_outputs *out,
                 void *ws, size_t ws_bytes, void *stream, ForwardInternals *fi, const LongerInner *li) {
  const Layout L = make_layout(cfg, batch);
  if (!ws && L.total > 0) return fail(STCA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (ws_bytes < L.total)
    return fail(STCA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, L.total);
  if (ws && !aligned16(ws)) return fail(STCA_ERR_INVALID_ARG, "workspace not 16-byte aligned");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int B = cfg->B, d = cfg->d, H = cfg->H, M = cfg->M, dh = d / H;
  if (out->n_stage_events < 0 || (out->n_stage_events > 0 && !out->stage_events))
    return fail(STCA_ERR_INVALID_ARG, "stage_events inconsistent with n_stage_events");
  auto rec = [&](int k) -> hipError_t {
    if (k < out->n_stage_events && out->stage_events[k])
      return hipEventRecord(reinterpret_cast<hipEvent_t>(out->stage_events[k]), s);
    return hipSuccess;
  };
  const int64_t T = batch->n_tgt;
  const bool bf = cfg->dtype == STCA_BF16;
  const size_t es = L.esize;
  const bool fusion = cfg->qmode == STCA_Q_FUSION;
  const float qscale = 1.0f / std::sqrt((float)dh);
  hipError_t e = hipSuccess;

  Plan plan;
  plan.hoff = at<int>(ws, L.plan);
  plan.toff = plan.hoff + (B + 1);
  plan.pblk = plan.toff + (B + 1);
  plan.coff = plan.pblk + (B + 1);
  plan.prow = L.prow ? at<int>(ws, L.prow) : nullptr;

  if (!li && (e = rec(0))) return hip_fail(e, "stage event");
  // bf16, d <= 256: all layers' history encoding in one launch that gathers
  // each tile once (the 128-row encoders, hist_bf16.hip / hist128_bf16.hip)
  const bool multi = bf && d <= 256 && !L.fused && batch->n_hist > 0 && M <= kMaxLayers && !li;
  // ---- 1. weight preparation (bf16): fragment-packed W^T into the workspace
  bf16_t *prep = bf ? at<bf16_t>(ws, L.prep) : nullptr;
  if (bf) {
    PackBatch pb;
    int n = 0;
    // W [K, N] -> packed W^T fragments at `dst` (+ row tile offset)
    auto add = [&](const void *src, int K, int N, size_t dst, int tile0, int fmt = 0) -> hipError_t {
      pb.m[n++] = PackDesc{(const bf16_t *)src, prep + dst, K, N, tile0, fmt};
      if (n == kMaxPacks) {
        hipError_t er = launch_pack_batch(pb, n, s);
        n = 0;
        return er;
      }
      return hipSuccess;
    };
    const int hd = cfg->hidden;
    for (int i = 0; i < M; ++i) {
      const stca_layer &l = w->layers[i];
      const PrepLayer &p = L.pl[i];
      // the 128-row history encoders (d = 256 staged and fused, d = 128 staged)
      // read W1 / W3 as 16-row tiles and W_K, W_V block-interleaved
      const bool enc128 = d == 256 || (d == 128 && multi);
      const int f13 = enc128 ? 1 : 0;
      if (!li) {  // short rows are encoded already: no history FFN
        if ((e = add(l.kv.w1, d, hd, p.kv_w1, 0, f13))) break;
        if ((e = add(l.kv.w3, d, hd, p.kv_w3, 0, f13))) break;
        if ((e = add(l.kv.w2, hd, d, p.kv_w2, 0))) break;
      }
      if (enc128 && !li) {
        if ((e = add(l.wk, d, d, p.wkv, 0, 4))) break;
        if ((e = add(l.wv, d, d, p.wkv, 0, 5))) break;
      } else {
        if ((e = add(l.wk, d, d, p.wkv, 0))) break;
        if ((e = add(l.wv, d, d, p.wkv, d / 32))) break;
      }
      if ((e = add(l.wq, d, d, p.wq, 0))) break;
      if ((e = add(l.wo, d, d, p.wo, 0))) break;
      if (fusion) {
        if ((e = add(l.q.w1, d, hd, p.q_w1, 0))) break;
        if ((e = add(l.q.w3, d, hd, p.q_w3, 0))) break;
        if ((e = add(l.q.w2, hd, d, p.q_w2, 0))) break;
        if (i > 0 && (e = add(l.wc, (i + 1) * d, d, p.wc, 0))) break;
      } else if (cfg->qmode == STCA_Q_LINEAR && i + 1 < M) {
        if ((e = add(l.r, d, d, p.r, 0))) break;
      }
    }
    if (!e && fusion) {
      e = add(w->z.w1, d, hd, L.z_w1, 0);
      if (!e) e = add(w->z.w3, d, hd, L.z_w3, 0);
      if (!e) e = add(w->z.w2, hd, d, L.z_w2, 0);
      if (!e) e = add(w->wz, (M + 1) * d, d, L.wz, 0);
    }
    if (!e && n) e = launch_pack_batch(pb, n, s);
    if (e) return hip_fail(e, "weight preparation");
  }

  // ---- 2. planner
  if (B > 0) {
    // short rows: n_hist is only a bound on the device-side total
    e = launch_plan(batch->hist_offsets, batch->tgt_offsets, B, li ? -1 : batch->n_hist, T,
                    batch->max_tgt_per_user, L.nb, L.tile_blocks, plan, out->dev_status, s);
    if (e) return hip_fail(e, "planner");
    if (plan.prow) {
      e = launch_padded_ids(plan, B, batch->hist_ids, cfg->table_rows, L.max_blocks, out->dev_status, s);
      if (e) return hip_fail(e, "padded ids");
    }
    if (L.bias) {  // the score bias in the blocked layout the attention reads
      e = launch_bias_relayout(batch->score_bias, at<float>(ws, L.bias), plan, B, L.max_blocks, H, s);
      if (e) return hip_fail(e, "score bias relayout");
    }
  }
  if ((e = rec(1))) return hip_fail(e, "stage event");
  if (B == 0 || (batch->n_hist == 0 && T == 0)) return STCA_OK;

  auto chain = [&](const ChainArgs &a) { return bf ? launch_chain_bf16(a, s) : launch_chain_f32(a, s); };
  auto base_args = [&]() {
    ChainArgs a;
    std::memset(&a, 0, sizeof(a));
    a.d = d;
    a.hidden = cfg->hidden;
    a.table = li ? li->raw->table : batch->table;
    a.table_rows = li ? li->raw_table_rows : cfg->table_rows;
    a.plan = plan;
    a.B = B;
    a.H = H;
    a.scale = 1.0f;
    a.status = out->dev_status;
    return a;
  };

  const bool kvln = cfg->flags & STCA_FLAG_KV_LN;
  // history-side chain arguments of layer i (gather -> FFN -> LN -> W_K | W_V)
  auto hist_args = [&](int i) {
    const stca_layer &l = w->layers[i];
    ChainArgs a = base_args();
    a.in_mode = IN_GATHER_CSR;
    a.out_mode = L.fused ? OUT_FUSED : OUT_KV;
    a.ffn = !li;
    a.ln = kvln && !li;
    a.proj = true;
    if (li) {  // layer i's block of short rows
      a.table = (const char *)batch->table + (size_t)i * li->layer_rows * d * L.esize;
      a.table_rows = li->layer_rows;
    }
    a.n_rows = L.max_blocks * 32;
    a.ids = batch->hist_ids;
    a.in_dump = i == 0 ? out->x_dump : nullptr;
    if (bf) {
      const PrepLayer &p = L.pl[i];
      a.w1 = prep + p.kv_w1;
      a.w3 = prep + p.kv_w3;
      a.w2 = prep + p.kv_w2;
      a.wp = prep + p.wkv;
    } else {
      a.w1 = l.kv.w1;
      a.w3 = l.kv.w3;
      a.w2 = l.kv.w2;
      a.wp = l.wk;
      a.wp2 = l.wv;
    }
    a.ln_g = l.kv.ln_g;
    a.ln_b = l.kv.ln_b;
    a.pn = 2 * d;
    return a;
  };
  auto attn_args = [&](int i, const void *q) {
    AttnArgs at_;
    std::memset(&at_, 0, sizeof(at_));
    at_.dtype = cfg->dtype;
    at_.score = cfg->score;
    at_.d = d;
    at_.H = H;
    at_.dh = dh;
    at_.nb = L.nb;
    at_.max_tgt = batch->max_tgt_per_user;
    attn_shape(at_, L.max_chunks);
    at_.fused = L.fused ? 1 : 0;
    at_.tile_blocks = L.tile_blocks;
    at_.max_grid = L.fused_grid;
    at_.plan = plan;
    at_.q = q;
    at_.n_tgt = T;
    at_.part_ml = at<float>(ws, L.part_ml);
    at_.part_acc = at<float>(ws, L.part_acc);
    at_.part_cnt = at<int>(ws, L.part_cnt);
    at_.fstate = L.fused ? at<float>(ws, L.fstate) : nullptr;
    at_.attn = out->attn ? out->attn + (size_t)i * T * d : at<float>(ws, L.attn32);
    at_.attn_lo = at<void>(ws, L.attnlo);
    at_.active = out->active ? out->active + (size_t)i * T * H : nullptr;
    at_.lse = (out->lse && cfg->score == STCA_SCORE_SOFTMAX) ? out->lse + (size_t)i * T * H : nullptr;
    at_.key_mask = batch->key_mask;
    at_.bias_blk = L.bias ? at<float>(ws, L.bias) : nullptr;
    if (cfg->head_map) {
      at_.has_map = 1;
      for (int hh = 0; hh < H; ++hh) at_.head_map[hh] = cfg->head_map[hh];
    }
    at_.B = B;
    if (batch->n_hist == 0) at_.max_units = 0;
    return at_;
  };

  if (L.fused) {
    // no separate history stage: its events mark the same instant
    for (int i = 0; i < M; ++i)
      if ((e = rec(2 + i))) return hip_fail(e, "stage event");
    if (T == 0) {  // nothing attends; only the optional input dump is produced
      if (out->x_dump && batch->n_hist > 0) {
        AttnArgs at_ = attn_args(0, nullptr);
        ChainArgs a = hist_args(0);
        e = d == 256 ? launch_fused256(a, at_, L.max_tiles, s) : launch_fused(a, at_, L.max_tiles, s);
        if (e) return hip_fail(e, "fused encoding");
      }
      return STCA_OK;
    }
  }

  // ---- 3. history side of every layer -> blocked K/V (staged path)
  char *kvbase = at<char>(ws, L.kv);
  auto kbuf = [&](int i) { return (void *)(kvbase + (size_t)(2 * i) * L.kv_layer); };
  auto vbuf = [&](int i) { return (void *)(kvbase + (size_t)(2 * i + 1) * L.kv_layer); };
  // STCA_FLAG_DEDUP: the encoder runs over the batch's distinct ids (a
  // one-user plan whose padded rows are those ids); each layer's token K/V is
  // then expanded from the unique rows
  Plan uplan = plan;
  int *n_unique = nullptr, *tok2u = nullptr;
  char *ukvbase = L.dedup ? at<char>(ws, L.ukv) : nullptr;
  auto ukbuf = [&](int i) { return (void *)(ukvbase + (size_t)(2 * i) * L.ukv_layer); };
  auto uvbuf = [&](int i) { return (void *)(ukvbase + (size_t)(2 * i + 1) * L.ukv_layer); };
  if (L.dedup) {
    int *small = at<int>(ws, L.d_small);
    DedupArgs da;
    std::memset(&da, 0, sizeof(da));
    da.ids = batch->hist_ids;
    da.n_hist = batch->n_hist;
    da.table_rows = cfg->table_rows;
    da.keys = at<int>(ws, L.d_keys);
    da.slot_uid = at<int>(ws, L.d_slot);
    da.mask = (uint32_t)(L.dslots - 1);
    da.block_cnt = at<int>(ws, L.d_bcnt);
    da.block_off = at<int>(ws, L.d_boff);
    da.uniq_rows = at<int>(ws, L.d_uniq);
    da.tok2u = at<int>(ws, L.d_tok2u);
    da.n_unique = small;
    da.uplan_hoff = small + 1;
    da.uplan_toff = small + 3;
    da.uplan_pblk = small + 5;
    da.status = out->dev_status;
    {
      int *sb = at<int>(ws, L.d_sort);
      const size_t nr = (size_t)L.drows;
      da.sort_in = sb;
      da.sort_keys[0] = sb + nr;
      da.sort_keys[1] = sb + 2 * nr;
      da.sort_vals[0] = sb + 3 * nr;
      da.sort_vals[1] = sb + 4 * nr;
      da.perm = sb + 5 * nr;
      da.sort_hist = sb + 6 * nr;
    }
    if ((e = launch_dedup(da, s))) return hip_fail(e, "id dedup");
    uplan.hoff = da.uplan_hoff;
    uplan.toff = da.uplan_toff;
    uplan.pblk = da.uplan_pblk;
    uplan.coff = da.uplan_toff;
    uplan.prow = da.uniq_rows;
    n_unique = da.n_unique;
    tok2u = da.tok2u;
    if (fi) set_internals(L, ws, fi);
  }
  // the encoder's view of the rows: the batch, or the unique ids
  auto enc_args = [&](int i) {
    ChainArgs a = hist_args(i);
    if (L.dedup) {
      a.plan = uplan;
      a.B = 1;
      a.n_rows = L.drows;
      a.in_dump = nullptr;
    }
    return a;
  };
  auto enc_k = [&](int i) { return L.dedup ? ukbuf(i) : kbuf(i); };
  auto enc_v = [&](int i) { return L.dedup ? uvbuf(i) : vbuf(i); };
  auto vrows = [&](int i) { return at<bf16_t>(ws, L.vrows) + (size_t)i * L.drows * d; };
  auto finish_layer = [&](int i) -> hipError_t {  // dedup V rows, K/V dump, stage event
    hipError_t er = hipSuccess;
    if (L.dedup) {
      er = launch_vrows((const bf16_t *)uvbuf(i), vrows(i), n_unique, L.drows, d, H, s);
      if (!er && out->kv_dump)  // the dump is per token: expand the unique rows
        er = launch_expand_kv((const bf16_t *)ukbuf(i), vrows(i), (bf16_t *)kbuf(i), (bf16_t *)vbuf(i), tok2u,
                              plan, B, L.max_blocks, d, H, s);
    }
    if (!er && out->kv_dump) {
      char *kd = (char *)out->kv_dump + (size_t)i * 2 * batch->n_hist * d * es;
      char *vd = kd + (size_t)batch->n_hist * d * es;
      er = launch_kv_relayout(cfg->dtype, kd, vd, kbuf(i), vbuf(i), plan, B, L.max_blocks, d, H, false, s);
    }
    if (!er) er = rec(2 + i);
    return er;
  };

  if (multi) {
    ChainArgs a = enc_args(0);
    HistLayers hl;
    std::memset(&hl, 0, sizeof(hl));
    hl.M = M;
    hl.clock = reinterpret_cast<unsigned long long *>(out->clock_probe);
    hl.persistent = L.dedup ? 1 : 0;  // the unique rows are counted on the device
    for (int i = 0; i < M; ++i) {
      const PrepLayer &p = L.pl[i];
      hl.w1[i] = prep + p.kv_w1;
      hl.w3[i] = prep + p.kv_w3;
      hl.w2[i] = prep + p.kv_w2;
      hl.wp[i] = prep + p.wkv;
      hl.ln_g[i] = w->layers[i].kv.ln_g;
      hl.ln_b[i] = w->layers[i].kv.ln_b;
      hl.kbuf[i] = enc_k(i);
      hl.vbuf[i] = enc_v(i);
    }
    e = d == 256 ? launch_hist256(a, hl, s) : launch_hist128(a, hl, s);
    if (e) return hip_fail(e, "history encoding");
    for (int i = 0; i < M; ++i)
      if ((e = finish_layer(i))) return hip_fail(e, "history K/V");
  }
  for (int i = 0; i < M && batch->n_hist > 0 && !L.fused && !multi; ++i) {
    ChainArgs a = enc_args(i);
    a.kbuf = enc_k(i);
    a.vbuf = enc_v(i);
    if ((e = chain(a))) return hip_fail(e, "history encoding");
    if ((e = finish_layer(i))) return hip_fail(e, "history K/V");
  }
  if (T == 0) return STCA_OK;

  // ---- 4. query chain and attention, layer by layer
  void *xt = at<void>(ws, L.xt);
  char *ocat = at<char>(ws, L.ocat);
  void *qs = at<void>(ws, L.qs);
  void *qcur = at<void>(ws, L.qcur);
  void *attnlo = at<void>(ws, L.attnlo);
  // HyFormer queries: one strided GEMM per step, batched over the m query
  // FFNs (or the T boosting FFNs), with the SwiGLU row kernel between
  const bool hyf = cfg->qmode == STCA_Q_HYFORMER;
  const int hm = batch->max_tgt_per_user, hT = hm + cfg->n_ns, hq = cfg->q_hidden;
  float *hy_h13 = hyf ? at<float>(ws, L.hy_h13) : nullptr, *hy_gg = hyf ? at<float>(ws, L.hy_gg) : nullptr;
  float *hy_out = hyf ? at<float>(ws, L.hy_out) : nullptr;
  // n FFNs (w1, w3 [n, din, hq], w2 [n, hq, d]) on n stacked [B, din] inputs
  // (a_batch_stride 0: one shared input) -> hy_out [n][B][d]
  auto ffn_stack = [&](int n, const float *a, int64_t din, int64_t a_bs, const void *w1, const void *w3,
                       const void *w2) -> hipError_t {
    GemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.M = B;
    g.N = hq;
    g.K = din;
    g.A = a;
    g.sam = din;
    g.sak = 1;
    g.B = w1;
    g.sbk = hq;
    g.sbn = 1;
    g.b_bf16 = true;
    g.C = hy_h13;
    g.scm = 2 * hq;
    g.scn = 1;
    g.alpha = 1.f;
    g.split = 1;
    g.batch = n;
    g.bsa = a_bs;
    g.bsb = din * hq;
    g.bsc = (int64_t)B * 2 * hq;
    g.part = at<float>(ws, L.hy_part);
    g.part_cap = L.hy_part_floats;
    g.split = hy_split(n, B, hq, din);
    hipError_t er = launch_gemm(g, s);
    if (er) return er;
    g.B = w3;
    g.C = hy_h13 + hq;
    if ((er = launch_gemm(g, s))) return er;
    if ((er = launch_swiglu_fwd(hy_h13, (int64_t)n * B, hq, hy_gg, false, s))) return er;
    g.A = hy_gg;
    g.sam = hq;
    g.K = hq;
    g.bsa = (int64_t)B * hq;
    g.B = w2;
    g.sbk = d;
    g.N = d;
    g.bsb = (int64_t)hq * d;
    g.C = hy_out;
    g.scm = d;
    g.bsc = (int64_t)B * d;
    g.split = hy_split(n, B, d, hq);
    return launch_gemm(g, s);
  };
  if (hyf) {  // q_u,n = FFN_n([F_u | MeanPool(rows of u)])
    float *mp = at<float>(ws, L.hy_mp), *gi = at<float>(ws, L.hy_g);
    if (li)  // MeanPool over the raw history, not the short rows
      e = launch_mean_pool((const bf16_t *)li->raw->table, li->raw_table_rows, li->raw->hist_ids, li->raw_plan, B, d,
                           mp, at<float>(ws, L.hy_pool), s);
    else
      e = launch_mean_pool((const bf16_t *)batch->table, cfg->table_rows, batch->hist_ids, plan, B, d, mp,
                           at<float>(ws, L.hy_pool), s);
    if (!e) e = launch_global_info((const bf16_t *)batch->ns_feats, mp, B, cfg->n_ns, d, gi, s);
    const int64_t din = (int64_t)(cfg->n_ns + 1) * d;
    if (!e) e = ffn_stack(hm, gi, din, 0, w->qgen_w1, w->qgen_w3, w->qgen_w2);
    if (!e) e = launch_queries_from_stack(hy_out, hm, B, d, (bf16_t *)qcur, s);
    if (e) return hip_fail(e, "query generation");
  }
  for (int i = 0; i < M; ++i) {
    const stca_layer &l = w->layers[i];
    const PrepLayer *p = bf ? &L.pl[i] : nullptr;
    void *qdst = out->q_dump ? (void *)((char *)out->q_dump + (size_t)i * T * d * es) : qs;
    {  // Q = q W_Q / sqrt(d_h)
      ChainArgs a = base_args();
      a.out_mode = OUT_ROWS;
      a.proj = true;
      a.n_rows = T;
      a.pn = d;
      a.scale = qscale;
      a.wp = bf ? (const void *)(prep + p->wq) : l.wq;
      a.out = qdst;
      a.ldo = d;
      if (fusion) {
        a.ffn = true;
        a.ln = true;
        a.ln_g = l.q.ln_g;
        a.ln_b = l.q.ln_b;
        a.w1 = bf ? (const void *)(prep + p->q_w1) : l.q.w1;
        a.w3 = bf ? (const void *)(prep + p->q_w3) : l.q.w3;
        a.w2 = bf ? (const void *)(prep + p->q_w2) : l.q.w2;
        if (i == 0) {  // q1 = LN(SwiGLU(x_t)); x_t kept for the fusion concat
          a.in_mode = IN_GATHER_IDS;
          a.ids = batch->tgt_ids;
          a.in_dump = xt;
        } else {  // q = LN(SwiGLU([o_1..o_i | x_t] W_C))
          a.in_mode = IN_PREGEMM;
          a.a = ocat;
          a.lda = M * d;
          a.k1 = i * d;
          a.a2 = xt;
          a.lda2 = d;
          a.k2 = d;
          a.wpre = bf ? (const void *)(prep + p->wc) : l.wc;
        }
      } else {
        a.in_mode = IN_DENSE;
        a.a = (i == 0 && !hyf) ? batch->q0 : qcur;
        a.lda = d;
      }
      if ((e = chain(a))) return hip_fail(e, "query");
    }
    if ((e = rec(2 + M + 4 * i))) return hip_fail(e, "stage event");
    {  // attention partials (fused: with the history encoding) + merge
      AttnArgs at_ = attn_args(i, qdst);
      if (L.fused) {
        if (batch->n_hist > 0) {
          ChainArgs a = hist_args(i);
          e = d == 256 ? launch_fused256(a, at_, L.max_tiles, s) : launch_fused(a, at_, L.max_tiles, s);
          if (e) return hip_fail(e, "fused encoding + attention");
        }
      } else {
        at_.kbuf = L.dedup ? ukbuf(i) : kbuf(i);
        at_.vbuf = vbuf(i);
        if (L.dedup) {  // K/V through the token -> unique row map
          at_.tok2u = tok2u;
          at_.vrows = vrows(i);
        }
        if ((e = launch_attn_partial(at_, s))) return hip_fail(e, "attention");
      }
      if ((e = rec(3 + M + 4 * i))) return hip_fail(e, "stage event");
      if ((e = launch_attn_merge(at_, s))) return hip_fail(e, "attention merge");
      if ((e = rec(4 + M + 4 * i))) return hip_fail(e, "stage event");
    }
    const bool last = i + 1 == M;
    {  // o = attn W_O -> fp32 output and the concat buffer
      ChainArgs a = base_args();
      a.in_mode = IN_DENSE;
      a.out_mode = OUT_ROWS;
      a.proj = true;
      a.n_rows = T;
      a.a = attnlo;
      a.lda = d;
      a.pn = d;
      a.wp = bf ? (const void *)(prep + p->wo) : l.wo;
      a.out = ocat + (size_t)i * d * es;
      a.ldo = M * d;
      if (out->o_layers) {
        a.out32 = out->o_layers + (size_t)i * T * d;
        a.ldo32 = d;
      } else if (hyf) {  // the boosting reads o in fp32
        a.out32 = at<float>(ws, L.hy_o32);
        a.ldo32 = d;
      } else if (!fusion && last) {
        a.out32 = out->z;
        a.ldo32 = d;
      }
      if ((e = chain(a))) return hip_fail(e, "output projection");
      if (!fusion && !hyf && last && out->o_layers) {  // z = O_M
        e = hipMemcpy2DAsync(out->z, d * sizeof(float), out->o_layers + (size_t)i * T * d,
                             d * sizeof(float), d * sizeof(float), T, hipMemcpyDeviceToDevice, s);
        if (e) return hip_fail(e, "z copy");
      }
    }
    if (hyf) {  // Q_boost = [o | F] + FFN'(mix([o | F])); first m tokens -> next queries (or z)
      const float *o32 = out->o_layers ? out->o_layers + (size_t)i * T * d : at<float>(ws, L.hy_o32);
      float *qcat = at<float>(ws, L.hy_qcat), *qmix = at<float>(ws, L.hy_qmix);
      e = launch_boost_input(o32, (const bf16_t *)batch->ns_feats, B, hm, cfg->n_ns, d, qcat, qmix, s);
      if (!e) e = ffn_stack(hT, qmix, d, (int64_t)B * d, l.boost_w1, l.boost_w3, l.boost_w2);
      if (!e) e = launch_boost_output(qcat, hy_out, B, hm, cfg->n_ns, d, (bf16_t *)qcur, last ? out->z : nullptr, s);
      if (e) return hip_fail(e, "query boosting");
    } else if (!fusion && !last) {  // Q_{i+1} = O_i R_i
      ChainArgs a = base_args();
      a.in_mode = IN_DENSE;
      a.out_mode = OUT_ROWS;
      a.proj = true;
      a.n_rows = T;
      a.a = ocat + (size_t)i * d * es;
      a.lda = M * d;
      a.pn = d;
      a.wp = bf ? (const void *)(prep + p->r) : l.r;
      a.out = qcur;
      a.ldo = d;
      if ((e = chain(a))) return hip_fail(e, "next-query map");
    }
    if ((e = rec(5 + M + 4 * i))) return hip_fail(e, "stage event");
  }

  // ---- 5. z = SwiGLU([o_1 .. o_M | x_t] W_Z) [+ LN]
  if (fusion) {
    ChainArgs a = base_args();
    a.in_mode = IN_PREGEMM;
    a.out_mode = OUT_ROWS;
    a.ffn = true;
    a.ln = cfg->flags & STCA_FLAG_Z_LN;
    a.proj = false;
    a.n_rows = T;
    a.a = ocat;
    a.lda = M * d;
    a.k1 = M * d;
    a.a2 = xt;
    a.lda2 = d;
    a.k2 = d;
    a.wpre = bf ? (const void *)(prep + L.wz) : w->wz;
    a.w1 = bf ? (const void *)(prep + L.z_w1) : w->z.w1;
    a.w3 = bf ? (const void *)(prep + L.z_w3) : w->z.w3;
    a.w2 = bf ? (const void *)(prep + L.z_w2) : w->z.w2;
    a.ln_g = w->z.ln_g;
    a.ln_b = w->z.ln_b;
    a.out32 = out->z;
    a.ldo32 = d;
    if ((e = chain(a))) return hip_fail(e, "final z");
  }
  if ((e = rec(2 + 5 * M))) return hip_fail(e, "stage event");
  return STCA_OK;
}

// LONGER-style encoding ([HyFormer] §3.4.1, eq. (6) then (8)).  Per layer l:
//   H_l = CrossAttn(S_short, S, S) = softmax_h((S_short W'_Q)(S W'_K)^T / sqrt(d_h)) (S W'_V) W'_O,
// S the user's raw rows, S_short the last min(L_u, l_short) of them; the
// layer's K/V are then H_l W_K, H_l W_V.  The pre-pass reuses the row chain
// (projections without FFN) and the split-L attention with the short rows as
// its targets, and writes every layer's H_l into a stacked table; the forward
// then runs over the short rows as its history.
int longer_forward(const stca_config *cfg, const stca_batch *batch, const stca_weights *w, const stca_outputs *out,
                   void *ws, size_t ws_bytes, void *stream) {
  const LongerLayout LL = make_longer_layout(cfg, batch);
  stca_config c2;
  stca_batch b2;
  longer_inner(cfg, batch, LL, ws, c2, b2);
  const size_t inner = make_layout(&c2, &b2).total;
  if (!ws) return fail(STCA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", LL.total + inner);
  if (ws_bytes < LL.total + inner)
    return fail(STCA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, LL.total + inner);
  if (!aligned16(ws)) return fail(STCA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  if (out->n_stage_events < 0 || (out->n_stage_events > 0 && !out->stage_events))
    return fail(STCA_ERR_INVALID_ARG, "stage_events inconsistent with n_stage_events");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int B = cfg->B, d = cfg->d, H = cfg->H, M = cfg->M;
  hipError_t e = hipSuccess;
  auto rec = [&](int k) -> hipError_t {
    if (k < out->n_stage_events && out->stage_events[k])
      return hipEventRecord(reinterpret_cast<hipEvent_t>(out->stage_events[k]), s);
    return hipSuccess;
  };
  const int ev0 = 3 + 5 * M;  // the pre-pass events follow the forward's own
  if ((e = rec(0))) return hip_fail(e, "stage event");

  // encoder weights, packed as the row chain reads them: W'_Q, W'_K | W'_V, W'_O
  bf16_t *prep = at<bf16_t>(ws, LL.prep);
  const size_t dd = (size_t)d * d;
  {
    PackBatch pb;
    int n = 0;
    for (int i = 0; i < M && !e; ++i) {
      const stca_layer &l = w->layers[i];
      bf16_t *base = prep + (size_t)i * 4 * dd;
      const PackDesc ds[4] = {{(const bf16_t *)l.enc_wq, base, d, d, 0, 0},
                              {(const bf16_t *)l.enc_wk, base + dd, d, d, 0, 0},
                              {(const bf16_t *)l.enc_wv, base + dd, d, d, d / 32, 0},
                              {(const bf16_t *)l.enc_wo, base + 3 * dd, d, d, 0, 0}};
      for (const PackDesc &pd : ds) {
        pb.m[n++] = pd;
        if (n == kMaxPacks) {
          e = launch_pack_batch(pb, n, s);
          n = 0;
          if (e) break;
        }
      }
    }
    if (!e && n) e = launch_pack_batch(pb, n, s);
    if (e) return hip_fail(e, "encoder weight preparation");
  }

  // short sequences and the raw plan (the short rows are the raw history's targets)
  Plan P;
  P.hoff = at<int>(ws, LL.plan);
  P.toff = P.hoff + (B + 1);
  P.pblk = P.toff + (B + 1);
  P.coff = P.pblk + (B + 1);
  P.prow = nullptr;
  int *soff = at<int>(ws, LL.soff), *sids = at<int>(ws, LL.sids);
  const int64_t rows = std::max<int64_t>(LL.nS, 1);
  if (B > 0) {
    e = launch_short_seq(batch->hist_offsets, batch->hist_ids, B, batch->n_hist, cfg->l_short, rows, soff, sids,
                         at<int>(ws, LL.iota), s);
    if (!e) e = launch_plan(batch->hist_offsets, soff, B, batch->n_hist, -1, cfg->l_short, LL.nb, 1, P,
                            out->dev_status, s);
    if (e) return hip_fail(e, "short sequences");
  }
  if ((e = rec(ev0))) return hip_fail(e, "stage event");

  if (B > 0 && batch->n_hist > 0) {
    const int dh = d / H;
    void *kb = at<void>(ws, LL.kv), *vb = at<char>(ws, LL.kv) + LL.kvl;
    for (int i = 0; i < M; ++i) {
      const bf16_t *base = prep + (size_t)i * 4 * dd;
      ChainArgs a;
      std::memset(&a, 0, sizeof(a));
      a.d = d;
      a.hidden = cfg->hidden;
      a.table = batch->table;
      a.table_rows = cfg->table_rows;
      a.plan = P;
      a.B = B;
      a.H = H;
      a.scale = 1.0f;
      a.status = out->dev_status;
      a.proj = true;
      {  // S W'_K, S W'_V over the raw rows -> blocked K/V
        ChainArgs k = a;
        k.in_mode = IN_GATHER_CSR;
        k.out_mode = OUT_KV;
        k.n_rows = LL.mb * 32;
        k.ids = batch->hist_ids;
        k.wp = base + dd;
        k.pn = 2 * d;
        k.kbuf = kb;
        k.vbuf = vb;
        if ((e = launch_chain_bf16(k, s))) return hip_fail(e, "encoder K/V");
        if ((e = rec(ev0 + 1 + 4 * i))) return hip_fail(e, "stage event");
      }
      bf16_t *qe = at<bf16_t>(ws, LL.qe);
      {  // S_short W'_Q / sqrt(d_h)
        ChainArgs q = a;
        q.in_mode = IN_GATHER_IDS;
        q.out_mode = OUT_ROWS;
        q.n_rows = rows;
        q.ids = sids;
        q.wp = base;
        q.pn = d;
        q.scale = 1.0f / std::sqrt((float)dh);
        q.out = qe;
        q.ldo = d;
        if ((e = launch_chain_bf16(q, s))) return hip_fail(e, "encoder queries");
        if ((e = rec(ev0 + 2 + 4 * i))) return hip_fail(e, "stage event");
      }
      {  // per-head softmax attention of each short row over the user's raw rows
        AttnArgs at_;
        std::memset(&at_, 0, sizeof(at_));
        at_.dtype = STCA_BF16;
        at_.score = STCA_SCORE_SOFTMAX;
        at_.d = d;
        at_.H = H;
        at_.dh = dh;
        at_.nb = LL.nb;
        at_.max_tgt = cfg->l_short;
        attn_shape(at_, LL.mc);
        at_.tile_blocks = 1;
        at_.plan = P;
        at_.q = qe;
        at_.n_tgt = rows;
        at_.kbuf = kb;
        at_.vbuf = vb;
        at_.part_ml = at<float>(ws, LL.ml);
        at_.part_acc = at<float>(ws, LL.acc);
        at_.part_cnt = at<int>(ws, LL.cnt);
        at_.attn = at<float>(ws, LL.a32);
        at_.attn_lo = at<void>(ws, LL.alo);
        at_.B = B;
        if ((e = launch_attention(at_, s))) return hip_fail(e, "encoder attention");
        if ((e = rec(ev0 + 3 + 4 * i))) return hip_fail(e, "stage event");
      }
      {  // H_l = attn W'_O -> layer i's block of the stacked table
        ChainArgs o = a;
        o.in_mode = IN_DENSE;
        o.out_mode = OUT_ROWS;
        o.n_rows = rows;
        o.a = at<void>(ws, LL.alo);
        o.lda = d;
        o.wp = base + 3 * dd;
        o.pn = d;
        o.out = at<bf16_t>(ws, LL.htab) + (size_t)i * rows * d;
        o.ldo = d;
        if ((e = launch_chain_bf16(o, s))) return hip_fail(e, "encoder output projection");
        if ((e = rec(ev0 + 4 + 4 * i))) return hip_fail(e, "stage event");
      }
    }
  }

  LongerInner li;
  li.raw = batch;
  li.raw_plan = P;
  li.raw_table_rows = cfg->table_rows;
  li.layer_rows = rows;
  return forward_body(&c2, &b2, w, out, (char *)ws + LL.total, ws_bytes - LL.total, stream, nullptr, &li);
}

}  // namespace stca

extern "C" {

int stca_forward(const stca_config *cfg, const stca_batch *batch, const stca_weights *w,
                 const stca_outputs *out, void *ws, size_t ws_bytes, void *stream) {
  return forward_with_internals(cfg, batch, w, out, ws, ws_bytes, stream, nullptr);
}

// ---------------------------------------------------------------- attention only
static int attn_validate(const stca_attn_args *a) {
  if (!a) return fail(STCA_ERR_INVALID_ARG, "args is NULL");
  if (a->B < 0) return fail(STCA_ERR_INVALID_ARG, "B must be >= 0");
  if (a->H <= 0 || a->d <= 0 || a->d % a->H) return fail(STCA_ERR_INVALID_ARG, "d must be a multiple of H");
  const int dh = a->d / a->H;
  if (dh != 32 && dh != 64) return fail(STCA_ERR_UNSUPPORTED, "d_h = %d unsupported", dh);
  if (a->dtype != STCA_F32 && a->dtype != STCA_BF16) return fail(STCA_ERR_INVALID_ARG, "dtype unknown");
  if (a->score != STCA_SCORE_SOFTMAX && a->score != STCA_SCORE_RELU)
    return fail(STCA_ERR_INVALID_ARG, "score unknown");
  if (a->chunk_keys < 0 || a->chunk_keys % 32) return fail(STCA_ERR_INVALID_ARG, "chunk_keys must be a multiple of 32");
  if (a->n_hist < 0 || a->n_hist >= (1ll << 31) || a->n_tgt < 0 || a->n_tgt >= (1ll << 31))
    return fail(STCA_ERR_INVALID_ARG, "n_hist / n_tgt outside [0, 2^31)");
  if (a->max_tgt_per_user < 1 || a->max_tgt_per_user > 4096)
    return fail(STCA_ERR_INVALID_ARG, "max_tgt_per_user outside 1..4096");
  if (a->B > 0 && (!a->hist_offsets || !a->tgt_offsets)) return fail(STCA_ERR_INVALID_ARG, "offsets NULL");
  if (a->n_tgt > 0 && (!a->q || !a->attn)) return fail(STCA_ERR_INVALID_ARG, "q / attn NULL");
  if (a->n_hist > 0 && (!a->k || !a->v)) return fail(STCA_ERR_INVALID_ARG, "k / v NULL");
  const void *ptrs[] = {a->hist_offsets, a->tgt_offsets, a->q, a->k, a->v, a->attn, a->active, a->key_mask,
                        a->score_bias};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return fail(STCA_ERR_INVALID_ARG, "pointer %p not 16-byte aligned", p);
  if ((a->key_mask || a->head_map || a->score_bias) && a->dtype != STCA_BF16)
    return fail(STCA_ERR_UNSUPPORTED, "key_mask / head_map / score_bias need bf16");
  if (a->score_bias && a->H > 16) return fail(STCA_ERR_UNSUPPORTED, "score_bias supports at most 16 heads");
  return validate_map(a->head_map, a->H);
}

struct AttnLayout {
  int nb;
  int64_t mb, mc;
  size_t plan, kv, kvl, ml, acc, cnt, bias, total;
};

static AttnLayout attn_layout(const stca_attn_args *a) {
  AttnLayout L;
  const size_t es = a->dtype == STCA_BF16 ? 2 : 4;
  L.nb = choose_nb(a->chunk_keys);
  L.mb = max_blocks(a->n_hist, a->B);
  L.mc = max_chunks(a->n_hist, a->B, L.nb);
  Carver cv;
  L.plan = cv.take(4 * sizeof(int) * (size_t)(a->B + 1));
  L.kvl = (size_t)L.mb * 32 * a->d * es;
  L.kv = cv.take(2 * L.kvl);
  const size_t np = partial_slots(a->B, a->H, a->max_tgt_per_user);
  L.ml = cv.take(np * 2 * sizeof(float));
  L.acc = cv.take(np * (a->d / a->H) * sizeof(float));
  L.cnt = cv.take(np * sizeof(int));
  L.bias = (a->score_bias && a->n_hist > 0) ? cv.take((size_t)L.mb * a->H * 32 * sizeof(float)) : 0;
  L.total = cv.off;
  return L;
}

int stca_attention_workspace_size(const stca_attn_args *a, size_t *bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(STCA_ERR_INVALID_ARG, "bytes is NULL");
  int r = attn_validate(a);
  if (r) return r;
  *bytes = attn_layout(a).total;
  return STCA_OK;
}

int stca_attention(const stca_attn_args *a, void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  int r = attn_validate(a);
  if (r) return r;
  const AttnLayout L = attn_layout(a);
  if (ws_bytes < L.total || (!ws && L.total))
    return fail(STCA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, L.total);
  if (ws && !aligned16(ws)) return fail(STCA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  if (a->B == 0 || a->n_tgt == 0) return STCA_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Plan plan;
  plan.hoff = at<int>(ws, L.plan);
  plan.toff = plan.hoff + (a->B + 1);
  plan.pblk = plan.toff + (a->B + 1);
  plan.coff = plan.pblk + (a->B + 1);
  plan.prow = nullptr;
  hipError_t e = launch_plan(a->hist_offsets, a->tgt_offsets, a->B, a->n_hist, a->n_tgt,
                             a->max_tgt_per_user, L.nb, 1, plan, a->dev_status, s);
  if (e) return hip_fail(e, "planner");
  char *kv = at<char>(ws, L.kv);
  if (a->n_hist > 0) {
    e = launch_kv_relayout(a->dtype, a->k, a->v, kv, kv + L.kvl, plan, a->B, L.mb, a->d, a->H, true, s);
    if (e) return hip_fail(e, "relayout");
    if (L.bias) {
      e = launch_bias_relayout(a->score_bias, at<float>(ws, L.bias), plan, a->B, L.mb, a->H, s);
      if (e) return hip_fail(e, "score bias relayout");
    }
  }
  AttnArgs at_;
  std::memset(&at_, 0, sizeof(at_));
  at_.dtype = a->dtype;
  at_.score = a->score;
  at_.d = a->d;
  at_.H = a->H;
  at_.dh = a->d / a->H;
  at_.nb = L.nb;
  at_.max_tgt = a->max_tgt_per_user;
  attn_shape(at_, L.mc);
  if (a->n_hist == 0) at_.max_units = 0;
  at_.plan = plan;
  at_.kbuf = kv;
  at_.vbuf = kv + L.kvl;
  at_.q = a->q;
  at_.n_tgt = a->n_tgt;
  at_.part_ml = at<float>(ws, L.ml);
  at_.part_acc = at<float>(ws, L.acc);
  at_.part_cnt = at<int>(ws, L.cnt);
  at_.attn = a->attn;
  at_.active = a->active;
  at_.B = a->B;
  at_.key_mask = a->key_mask;
  at_.bias_blk = L.bias ? at<float>(ws, L.bias) : nullptr;
  if (a->head_map) {
    at_.has_map = 1;
    for (int hh = 0; hh < a->H; ++hh) at_.head_map[hh] = a->head_map[hh];
  }
  if ((e = launch_attention(at_, s))) return hip_fail(e, "attention");
  return STCA_OK;
}

}  // extern "C"
