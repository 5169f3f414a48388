// hyformer.hip -- the data movement of HyFormer query generation and query
// boosting ([HyFormer] §3.3.2 eq. (3)-(4), §3.5 eq. (10)-(15)); the FFNs
// themselves are batched strided GEMMs (grad_gemm.hip) and the SwiGLU row
// kernel (grad_ops.hip).
//
//   MeanPool(Seq): per user, the mean of the raw history rows (one pass over
//     the history: 16 interleaved row chunks per user, partial sums folded
//     in a fixed order);
//   GlobalInfo = Concat(F_1..F_M, MeanPool(Seq)) per user;
//   boosting input: Q = [decoded queries | F] per user (T = m + n_ns tokens),
//     and its mixed form, grouped by mixed token so that each token's FFN is
//     one GEMM over the users: mixed token h of user u is the concatenation
//     over t of token t's h-th subspace (width d / T);
//   boosting output: Q_boost = Q + FFN(mix(Q)) position by position; its
//     first m tokens are the next layer's queries.
#include "grad_internal.h"

namespace stca {
namespace {

constexpr int kT = 256;

// Partial sums of user u's rows in chunk c (rows c, c + kPoolChunks, ..):
// four waves x four rows in flight, folded in wave order; then the chunks
// are folded in order.  The order depends on the lengths alone.
constexpr int kPoolChunks = 16;

__global__ __launch_bounds__(kT) void mean_pool_part_kernel(const bf16_t *__restrict__ table, int64_t table_rows,
                                                            const int *__restrict__ ids, Plan P, int B, int d,
                                                            float *part) {
  // 8 consecutive features per lane (one 16-byte load per row), 512 per wave
  __shared__ float sm[4][512];
  const int u = blockIdx.x / kPoolChunks, c = blockIdx.x % kPoolChunks;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int f0 = blockIdx.y * 512 + lane * 8;
  if (u >= B) return;
  const int h0 = P.hoff[u], L = P.hoff[u + 1] - h0;
  // this wave's rows: j = c + kPoolChunks * (w + 4 k), k = 0, 1, ..
  constexpr int S = 4 * kPoolChunks;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto row = [&](int id) -> bf16x8 {
    bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    return (id >= 0 && (int64_t)id < table_rows) ? ld8(table + (int64_t)id * d + f0) : z;
  };
  if (f0 < d) {
    int j = c + kPoolChunks * w;
    for (; j + 3 * S < L; j += 4 * S) {
      int id[4];
      bf16x8 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) id[q] = ids[h0 + j + q * S];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = row(id[q]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += bf2f((bf16_t)v[q][e]);
    }
    for (; j < L; j += S) {
      const bf16x8 v = row(ids[h0 + j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += bf2f((bf16_t)v[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm[w][lane * 8 + e] = s[e];
  __syncthreads();
  if (w == 0 && f0 < d) {
    const int64_t o = ((int64_t)u * kPoolChunks + c) * d + f0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int x = lane * 8 + e;
      part[o + e] = ((sm[0][x] + sm[1][x]) + sm[2][x]) + sm[3][x];
    }
  }
}

__global__ __launch_bounds__(kT) void mean_pool_fold_kernel(const float *__restrict__ part, Plan P, int B, int d,
                                                            float *mp) {
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (e >= (int64_t)B * d) return;
  const int64_t u = e / d, f = e % d;
  const int L = P.hoff[u + 1] - P.hoff[u];
  float s = 0.f;
  for (int c = 0; c < kPoolChunks; ++c) s += part[(u * kPoolChunks + c) * d + f];
  mp[e] = L > 0 ? s / L : 0.f;
}

__global__ __launch_bounds__(kT) void global_info_kernel(const bf16_t *__restrict__ ns, const float *__restrict__ mp,
                                                         int B, int n_ns, int d, float *g) {
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  const int64_t w = (int64_t)(n_ns + 1) * d;
  if (e >= (int64_t)B * w) return;
  const int64_t u = e / w, c = e % w;
  g[e] = c < (int64_t)n_ns * d ? bf2f(ns[u * n_ns * d + c]) : mp[u * d + (c - (int64_t)n_ns * d)];
}

__global__ __launch_bounds__(kT) void queries_from_stack_kernel(const float *__restrict__ src, int m, int B, int d,
                                                                bf16_t *qcur) {
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;  // over [m][B][d]
  if (e >= (int64_t)m * B * d) return;
  const int64_t n = e / ((int64_t)B * d), rem = e % ((int64_t)B * d);
  const int64_t u = rem / d, f = rem % d;
  qcur[(u * m + n) * d + f] = f2bf(src[e]);
}

__global__ __launch_bounds__(kT) void boost_input_kernel(const float *__restrict__ o, const bf16_t *__restrict__ ns,
                                                         int B, int m, int n_ns, int d, float *qcat, float *qmix) {
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;  // over [B][T][d] of qcat
  const int T = m + n_ns;
  if (e >= (int64_t)B * T * d) return;
  const int64_t u = e / ((int64_t)T * d), rem = e % ((int64_t)T * d);
  const int t = (int)(rem / d), c = (int)(rem % d);
  const float v = t < m ? o[(u * m + t) * d + c] : bf2f(ns[(u * n_ns + (t - m)) * d + c]);
  qcat[e] = v;
  // value c of token t lies in subspace h = c / w at offset c % w; it goes to
  // mixed token h, at position t * w + c % w
  const int w = d / T, h = c / w;
  qmix[((int64_t)h * B + u) * d + (int64_t)t * w + (c % w)] = v;
}

__global__ __launch_bounds__(kT) void boost_output_kernel(const float *__restrict__ qcat,
                                                          const float *__restrict__ ffn, int B, int m, int n_ns,
                                                          int d, bf16_t *qcur, float *z) {
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;  // over [B][m][d]: the query tokens
  const int T = m + n_ns;
  if (e >= (int64_t)B * m * d) return;
  const int64_t u = e / ((int64_t)m * d), rem = e % ((int64_t)m * d);
  const int t = (int)(rem / d), c = (int)(rem % d);
  const float v = qcat[(u * T + t) * d + c] + ffn[((int64_t)t * B + u) * d + c];
  qcur[e] = f2bf(v);  // row u m + t
  if (z) z[e] = v;
}

unsigned blocks(int64_t n) { return (unsigned)((n + kT - 1) / kT); }

}  // namespace

int64_t mean_pool_part_floats(int B, int d) { return (int64_t)B * kPoolChunks * d; }

hipError_t launch_mean_pool(const bf16_t *table, int64_t table_rows, const int *hist_ids, const Plan &plan, int B,
                            int d, float *mp, float *part, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (d % 8) return hipErrorInvalidValue;  // 16-byte row pieces
  hipLaunchKernelGGL(mean_pool_part_kernel, dim3((unsigned)(B * kPoolChunks), (unsigned)((d + 511) / 512)), dim3(kT),
                     0, s, table, table_rows, hist_ids, plan, B, d, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mean_pool_fold_kernel, dim3(blocks((int64_t)B * d)), dim3(kT), 0, s, part, plan, B, d, mp);
  return hipGetLastError();
}

hipError_t launch_global_info(const bf16_t *ns, const float *mp, int B, int n_ns, int d, float *g, hipStream_t s) {
  const int64_t n = (int64_t)B * (n_ns + 1) * d;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(global_info_kernel, dim3(blocks(n)), dim3(kT), 0, s, ns, mp, B, n_ns, d, g);
  return hipGetLastError();
}

hipError_t launch_queries_from_stack(const float *src, int m, int B, int d, bf16_t *qcur, hipStream_t s) {
  const int64_t n = (int64_t)m * B * d;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(queries_from_stack_kernel, dim3(blocks(n)), dim3(kT), 0, s, src, m, B, d, qcur);
  return hipGetLastError();
}

hipError_t launch_boost_input(const float *o, const bf16_t *ns, int B, int m, int n_ns, int d, float *qcat,
                              float *qmix, hipStream_t s) {
  const int64_t n = (int64_t)B * (m + n_ns) * d;
  if (n <= 0) return hipSuccess;
  if (d % (m + n_ns)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(boost_input_kernel, dim3(blocks(n)), dim3(kT), 0, s, o, ns, B, m, n_ns, d, qcat, qmix);
  return hipGetLastError();
}

hipError_t launch_boost_output(const float *qcat, const float *ffn, int B, int m, int n_ns, int d, bf16_t *qcur,
                               float *z, hipStream_t s) {
  const int64_t n = (int64_t)B * m * d;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(boost_output_kernel, dim3(blocks(n)), dim3(kT), 0, s, qcat, ffn, B, m, n_ns, d, qcur, z);
  return hipGetLastError();
}

}  // namespace stca
