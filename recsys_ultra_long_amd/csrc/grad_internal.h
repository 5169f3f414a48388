// grad_internal.h -- launchers of the backward pass (training step) kernels.
// Not part of the public ABI.
#pragma once

#include "stca.h"
#include "stca_internal.h"

namespace stca {

// ------------------------------------------------------------ forward internals
// stca_forward with, when STCA_FLAG_DEDUP is set, the location of its
// unique-row buffers (valid until the workspace is reused):
//   tok2u[n_hist]       unique index of every history item
//   uniq_rows[drows]    table id of every unique row (-1: padding / out of range)
//   n_unique            device int: the number of unique rows
//   ukv                 layer i: K of the unique rows at ukv + 2 i ukv_layer_elems,
//                       blocked [row / 32][H][32][d_h]
//   vrows               layer i: V of the unique rows at vrows + i drows d, [row][d]
struct ForwardInternals {
  bool dedup;
  const int *tok2u, *uniq_rows, *n_unique;
  int64_t drows;
  const bf16_t *ukv;
  size_t ukv_layer_elems;
  const bf16_t *vrows;
};
// The forward's synchronous argument checks (config, batch, weights).
int forward_check(const stca_config *cfg, const stca_batch *batch, const stca_weights *w);
int forward_with_internals(const stca_config *cfg, const stca_batch *batch, const stca_weights *w,
                           const stca_outputs *out, void *ws, size_t ws_bytes, void *stream, ForwardInternals *fi);
// The internals a forward of (cfg, batch) leaves in ws, without running it.
void forward_internals(const stca_config *cfg, const stca_batch *batch, void *ws, ForwardInternals *fi);

// ------------------------------------------------------------ generic GEMM
// C(m, n) = alpha * sum_k A(m, k) B(k, n) + beta * C(m, n)
// with A(m, k) = A[m * sam + k * sak], B(k, n) = B[k * sbk + n * sbn],
// C(m, n) = C[m * scm + n * scn].  Either stride of A and of B must be 1.
// Operands are fp32 or bf16 (converted to bf16 for the MFMA), accumulation
// fp32, C fp32.  split > 1 cuts K into that many ranges, each writing a
// partial [M, N] into `part` (split * M * N floats), folded in range order.
// dev_rows (optional): a device count that caps M (dev_dim 1: row tiles past
// it exit, their C rows are left as they are) or K (dev_dim 2: the sum stops
// there), for products over rows whose number is only known on the device.
struct GemmArgs {
  int64_t M, N, K;
  const void *A;
  int64_t sam, sak;
  bool a_bf16;
  const void *B;
  int64_t sbk, sbn;
  bool b_bf16;
  float *C;
  int64_t scm, scn;
  float alpha, beta;
  int split;
  float *part;
  int64_t part_cap;  // floats in `part`: a split needing more is refused
  const int *dev_rows;
  int dev_dim;
  // batch > 1: `batch` problems whose A, B, C start z * bsa, z * bsb, z * bsc
  // elements further (with split > 1 the partials are [batch][split][M][N])
  int batch;
  int64_t bsa, bsb, bsc;
  // optional second output: columns n >= n_split go to C2 (column n - n_split,
  // same strides), e.g. two weight gradients with one shared operand as one
  // product (no batching with it)
  float *C2;
  int64_t n_split;
};
hipError_t launch_gemm(const GemmArgs &g, hipStream_t s);
// Split factor for a long-K product (weight gradients), and the partial
// buffer it needs (floats).
int gemm_split_for(int64_t M, int64_t N, int64_t K, int64_t target = 1024, int64_t min_chunk = 128);
inline int64_t gemm_part_floats(int64_t M, int64_t N, int split) { return split > 1 ? (int64_t)split * M * N : 0; }

// ------------------------------------------------------------ row kernels
// out[r, :] = table[ids[r], :] for valid ids, zero rows otherwise (bf16 in;
// bf16 or fp32 out).
// Every row kernel takes an optional device count `dev_rows` that caps R.
hipError_t launch_gather_rows(const bf16_t *table, int64_t table_rows, const int *ids, int64_t R, int d,
                              void *out, bool out_bf16, hipStream_t s, const int *dev_rows = nullptr);
// G = SiLU(H1) * H3 with H13 = [H1 | H3] ([R, 2h] fp32); G bf16 or fp32.
hipError_t launch_swiglu_fwd(const float *h13, int64_t R, int h, void *g, bool g_bf16, hipStream_t s,
                             const int *dev_rows = nullptr);
// dH1 = dG * H3 * SiLU'(H1), dH3 = dG * SiLU(H1) into [R, 2h] (bf16 or fp32).
hipError_t launch_swiglu_bwd(const float *dg, const float *h13, int64_t R, int h, void *dh13, bool out_bf16,
                             hipStream_t s, const int *dev_rows = nullptr);
// LayerNorm over rows of Y [R, d] (fp32): out = xhat * g + b (bf16 or fp32);
// per-row (mean, rstd) into stats [R, 2].  g == nullptr: out = Y, no stats.
hipError_t launch_ln_fwd(const float *y, int64_t R, int d, const float *g, const float *b, void *out, bool out_bf16,
                         float *stats, hipStream_t s, const int *dev_rows = nullptr);
// Backward of the LN above: dY (bf16 or fp32) from dOut [R, d] fp32; dg, db
// accumulated (+=) over the rows through per-block partials `part`
// (2 * ln_part_rows(R) * d floats).  g == nullptr: dY = dOut.
int64_t ln_part_rows(int64_t R);
// dg, db += the sums over nblk per-block partials [nblk, 2, d] (gain, then
// bias) in `part`, folded in a fixed order; `part` holds 2 * (nblk + 64) * d
// floats (the fold's slices follow the partials).
hipError_t launch_ln_fold(float *part, int64_t nblk, int d, float *dg, float *db, hipStream_t s);
hipError_t launch_ln_bwd(const float *dout, const float *y, const float *stats, int64_t R, int d, const float *g,
                         void *dy, bool dy_bf16, float *dg, float *db, float *part, hipStream_t s,
                         const int *dev_rows = nullptr);
// dst[r, :] (+)= src[r, :] over a [R, d] block with row strides.
hipError_t launch_add_rows(const float *src, int64_t lds, float *dst, int64_t ldd, int64_t R, int d, bool accumulate,
                           hipStream_t s);
// dst[t, s*d + f] = src[s][t][f]: layer-major [S][R][d] -> row-major [R][S*d].
hipError_t launch_concat_layers(const float *src, int S, int64_t R, int d, float *dst, hipStream_t s);
// table[ids[r], :] += rows[r, :] (rows lds apart, lds = 0: d; d a multiple
// of 4, rows and table 16-byte aligned), ids outside the table skipped;
// atomic unless `unique` (no id repeats among the rows).
hipError_t launch_scatter_add(const float *rows, const int *ids, int64_t R, int d, float *table, int64_t table_rows,
                              hipStream_t s, const int *dev_rows = nullptr, int64_t lds = 0, bool unique = false);

// ------------------------------------------------------------ history backward (d = 256)
// One layer of the history encoder's backward on 128-row tiles in one launch
// (hist_bwd_bf16.hip): the forward recomputed from the rows X, then
// dX~ = dK W_K^T + dV W_V^T, the LN backward, dG = dY W2^T, the SwiGLU
// backward and dX (+)= dH1 W1^T + dH3 W3^T.  It writes the operands of the
// weight-gradient products (X~, G, dY, dH1 | dH3, bf16, row-major) and, with
// LN, per-tile partial sums of the LN gain and bias gradients.
struct HistBwdArgs {
  int64_t R;              // rows (host bound)
  const int *dev_rows;    // optional device count capping R
  int hidden;             // multiple of 128
  bool ln;
  const bf16_t *x;        // [R, 256] the rows X
  const bf16_t *dkv;      // [R, 512] dK | dV
  // packed operands (launch_pack_batch): W1, W3 fmt 1 (K 256, N hidden);
  // W2 fmt 0 (K hidden, N 256); W_K^T | W_V^T fmt 4 / 5 from transposed
  // sources (K = N = 256); W2^T fmt 1 from a transposed source (K 256,
  // N hidden); W1^T | W3^T fmt 4 / 5 from transposed sources (K hidden, N 256)
  const bf16_t *w1p, *w3p, *w2p, *wkvt, *w2t, *w13t;
  const float *ln_g, *ln_b;
  bf16_t *xt;             // [R, 256] X~ = LN(Y)
  bf16_t *g;              // [R, hidden] G
  bf16_t *dy;             // [R, 256] dY
  bf16_t *dh13;           // [R, 2 hidden] dH1 | dH3
  bf16_t *hs;             // scratch: hist_bwd_scratch_elems(R, hidden)
  float *dx;              // [R, 256] fp32
  bool dx_acc;            // dX += (else dX =)
  float *ln_part;         // [hist_bwd_tiles(R), 2, 256] (with LN)
};
inline bool hist_bwd256_ok(int d, int hidden) { return d == 256 && hidden >= 128 && hidden % 128 == 0; }
inline int64_t hist_bwd_tiles(int64_t R) { return (R + 127) / 128; }
inline int64_t hist_bwd_scratch_elems(int64_t R, int hidden) { return hist_bwd_tiles(R) * 128 * 2 * (int64_t)hidden; }
// Elements of one layer's packed operands.
inline int64_t hist_bwd_pack_elems(int d, int hidden) { return 6 * (int64_t)d * hidden + 2 * (int64_t)d * d; }
hipError_t launch_hist_bwd256(const HistBwdArgs &a, hipStream_t s);

// ------------------------------------------------------------ attention backward
// Inputs per layer, all token-indexed: Q (scaled, bf16 [T, d]), K and V rows
// (bf16 [n_hist, d]), the attention output a (fp32 [T, d]), its upstream
// gradient dA (fp32 [T, d]) and, for softmax, the natural-log softmax
// denominators lse [T, H].  Outputs: dQ (gradient w.r.t. the scaled Q, fp32
// [T, d]) and dK | dV (bf16 [n_hist, 2d] rows, dK in columns [0, d)).
struct AttnBwdArgs {
  int d, H, dh, score;
  int B;
  int64_t n_hist, n_tgt;
  int nb;  // 32-key blocks per chunk
  int max_tgt;  // host bound on any user's targets (the planner zeroes users past it)
  Plan plan;
  int64_t max_chunks;
  const bf16_t *q, *k, *v;
  const float *a, *da, *lse;
  bf16_t *da_lo;    // [T, d] scratch: dA in bf16
  float *dsum;      // [T, H] scratch: D = rowsum(dA * a) per head
  float *part_dq;   // [max_chunks * H * 4 * 64 * dh] scratch
  float *dq;
  bf16_t *dkv;
  // optional: K and V through the unique rows (STCA_FLAG_DEDUP): k is the
  // unique rows' blocked K [row / 32][H][32][d_h], v their V rows [row][d],
  // tok2u[n_hist] the unique row of every history item
  const int *tok2u;
};
int64_t attn_bwd_part_floats(int64_t max_chunks, int H, int dh);
hipError_t launch_attn_bwd(const AttnBwdArgs &a, hipStream_t s);

// ------------------------------------------------------------ HyFormer queries
// mp[u, :] = mean of the table rows of user u's history (zero when empty);
// part: mean_pool_part_floats(B, d) floats of scratch
int64_t mean_pool_part_floats(int B, int d);
hipError_t launch_mean_pool(const bf16_t *table, int64_t table_rows, const int *hist_ids, const Plan &plan, int B,
                            int d, float *mp, float *part, hipStream_t s);
// g[u] = [F_u,1 .. F_u,n_ns | mp[u]] (fp32, [B, (n_ns + 1) d]) from bf16 F
hipError_t launch_global_info(const bf16_t *ns, const float *mp, int B, int n_ns, int d, float *g, hipStream_t s);
// qcur[u m + n] = bf16(src[n][u]) for src [m][B][d] fp32
hipError_t launch_queries_from_stack(const float *src, int m, int B, int d, bf16_t *qcur, hipStream_t s);
// qcat[u][t] = o[u m + t] (t < m), F_u,t-m (t >= m); qmix[h][u] = mixed token h
// of user u (T = m + n_ns tokens, subspaces of width d / T)
hipError_t launch_boost_input(const float *o, const bf16_t *ns, int B, int m, int n_ns, int d, float *qcat,
                              float *qmix, hipStream_t s);
// Q_boost[u][t] = qcat[u][t] + ffn[t][u]; its first m tokens -> qcur (bf16)
// and, when z is given, -> z (fp32)
hipError_t launch_boost_output(const float *qcat, const float *ffn, int B, int m, int n_ns, int d, bf16_t *qcur,
                               float *z, hipStream_t s);

// ------------------------------------------------------------ per-unique sums
// out[u] = sum over the items j with tok2u[j] = u, in item order, of dkv[j]
// (fp32 accumulation, bf16 out), u < *n_unique.
struct UniqueSumArgs {
  int64_t n;              // history items
  int64_t max_u;          // host bound on the unique rows
  const int *tok2u;       // [n]
  const int *n_unique;    // device count
  int *keys[2], *vals[2]; // [n] ints each (scratch)
  int *hist;              // sort_hist_ints(n) ints (scratch)
  int *seg;               // [max_u + 1] ints (scratch): run starts
  const bf16_t *dkv;      // [n, d2]
  int d2;                 // 2d, at most 1024
  float *ppart;           // [agg_partial_floats(n, d2)] (scratch)
  bf16_t *out;            // [max_u, d2]
  const int *sorted_items;  // set by launch_unique_sort (points into vals)
  const int *sorted_keys;   // set by launch_unique_sort (points into keys)
};
int64_t agg_partial_floats(int64_t n, int d2);
// Once per batch: the items sorted by (unique row, item) and the run starts;
// then per layer: the sums of that layer's dkv.
hipError_t launch_unique_sort(UniqueSumArgs &a, hipStream_t s);
hipError_t launch_unique_sums(const UniqueSumArgs &a, hipStream_t s);

}  // namespace stca
