// grad_internal.h -- launchers of the backward pass (training step) kernels.
// Not part of the public ABI.
#pragma once

#include "stca_internal.h"

namespace stca {

// ------------------------------------------------------------ generic GEMM
// C(m, n) = alpha * sum_k A(m, k) B(k, n) + beta * C(m, n)
// with A(m, k) = A[m * sam + k * sak], B(k, n) = B[k * sbk + n * sbn],
// C(m, n) = C[m * scm + n * scn].  Either stride of A and of B must be 1.
// Operands are fp32 or bf16 (converted to bf16 for the MFMA), accumulation
// fp32, C fp32.  split > 1 cuts K into that many ranges, each writing a
// partial [M, N] into `part` (split * M * N floats), folded in range order.
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
};
hipError_t launch_gemm(const GemmArgs &g, hipStream_t s);
// Split factor for a long-K product (weight gradients), and the partial
// buffer it needs (floats).
int gemm_split_for(int64_t M, int64_t N, int64_t K);
inline int64_t gemm_part_floats(int64_t M, int64_t N, int split) { return split > 1 ? (int64_t)split * M * N : 0; }

// ------------------------------------------------------------ row kernels
// out[r, :] = table[ids[r], :] for valid ids, zero rows otherwise (bf16 in;
// bf16 or fp32 out).
hipError_t launch_gather_rows(const bf16_t *table, int64_t table_rows, const int *ids, int64_t R, int d,
                              void *out, bool out_bf16, hipStream_t s);
// G = SiLU(H1) * H3 with H13 = [H1 | H3] ([R, 2h] fp32); G bf16 or fp32.
hipError_t launch_swiglu_fwd(const float *h13, int64_t R, int h, void *g, bool g_bf16, hipStream_t s);
// dH1 = dG * H3 * SiLU'(H1), dH3 = dG * SiLU(H1) into [R, 2h] (bf16 or fp32).
hipError_t launch_swiglu_bwd(const float *dg, const float *h13, int64_t R, int h, void *dh13, bool out_bf16,
                             hipStream_t s);
// LayerNorm over rows of Y [R, d] (fp32): out = xhat * g + b (bf16 or fp32);
// per-row (mean, rstd) into stats [R, 2].  g == nullptr: out = Y, no stats.
hipError_t launch_ln_fwd(const float *y, int64_t R, int d, const float *g, const float *b, void *out, bool out_bf16,
                         float *stats, hipStream_t s);
// Backward of the LN above: dY (bf16 or fp32) from dOut [R, d] fp32; dg, db
// accumulated (+=) over the rows through per-block partials `part`
// (2 * ln_part_rows(R) * d floats).  g == nullptr: dY = dOut.
int64_t ln_part_rows(int64_t R);
hipError_t launch_ln_bwd(const float *dout, const float *y, const float *stats, int64_t R, int d, const float *g,
                         void *dy, bool dy_bf16, float *dg, float *db, float *part, hipStream_t s);
// dst[r, :] (+)= src[r, :] over a [R, d] block with row strides.
hipError_t launch_add_rows(const float *src, int64_t lds, float *dst, int64_t ldd, int64_t R, int d, bool accumulate,
                           hipStream_t s);
// dst[t, s*d + f] = src[s][t][f]: layer-major [S][R][d] -> row-major [R][S*d].
hipError_t launch_concat_layers(const float *src, int S, int64_t R, int d, float *dst, hipStream_t s);
// table[ids[r], :] += rows[r, :] (atomic), ids outside the table skipped.
hipError_t launch_scatter_add(const float *rows, const int *ids, int64_t R, int d, float *table, int64_t table_rows,
                              hipStream_t s);

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
  Plan plan;
  int64_t max_chunks;
  const bf16_t *q, *k, *v;
  const float *a, *da, *lse;
  bf16_t *da_lo;    // [T, d] scratch: dA in bf16
  float *dsum;      // [T, H] scratch: D = rowsum(dA * a) per head
  float *part_dq;   // [max_chunks * H * 4 * 64 * dh] scratch
  float *dq;
  bf16_t *dkv;
};
int64_t attn_bwd_part_floats(int64_t max_chunks, int H, int dh);
hipError_t launch_attn_bwd(const AttnBwdArgs &a, hipStream_t s);

}  // namespace stca
