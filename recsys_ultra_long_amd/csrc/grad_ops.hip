// grad_ops.hip -- row-wise and element-wise steps of the backward pass.
//
// The derivatives written out here are those of the forward's blocks:
//   SwiGLU  y = (SiLU(x W1) * (x W3)) W2,  SiLU(u) = u * sigmoid(u),
//           SiLU'(u) = sigmoid(u) * (1 + u * (1 - sigmoid(u)));
//   LayerNorm y = xhat * g + b, xhat = (x - mean) * rstd (biased variance,
//           eps 1e-5): dx = rstd * (gy - mean(gy) - xhat * mean(gy * xhat))
//           with gy = dy * g; dg = sum over rows of dy * xhat, db = sum dy.
// ([Notes] §STCA names the SwiGLU FFN + LN block of every layer; the forms
// above are the readings the forward uses.)  Column sums over rows (dg, db)
// go through per-block partials folded in block order: no atomics decide a
// floating-point result here, except the table scatter, whose adds into a
// shared row are atomic by nature.
#include "grad_internal.h"

namespace stca {
namespace {

constexpr int kT = 256;
constexpr float kLnEps = 1e-5f;

DEV float sigm(float u) { return 1.0f / (1.0f + expf(-u)); }

template <typename T> DEV void store(void *p, int64_t i, float v) { ((T *)p)[i] = from_f<T>(v); }

__global__ __launch_bounds__(kT) void gather_kernel(const bf16_t *__restrict__ table, int64_t table_rows,
                                                    const int *__restrict__ ids, int64_t R, int d, void *out,
                                                    bool out_bf16, const int *dev_rows) {
  if (dev_rows) R = min(R, (int64_t)*dev_rows);
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (e >= R * d) return;
  const int64_t r = e / d;
  const int f = (int)(e % d);
  const int id = ids[r];
  const float v = (id >= 0 && (int64_t)id < table_rows) ? bf2f(table[(int64_t)id * d + f]) : 0.f;
  if (out_bf16) store<bf16_t>(out, e, v);
  else store<float>(out, e, v);
}

__global__ __launch_bounds__(kT) void swiglu_fwd_kernel(const float *__restrict__ h13, int64_t R, int h, void *g,
                                                        bool g_bf16, const int *dev_rows) {
  if (dev_rows) R = min(R, (int64_t)*dev_rows);
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (e >= R * h) return;
  const int64_t r = e / h;
  const int j = (int)(e % h);
  const float u = h13[r * 2 * h + j], v = h13[r * 2 * h + h + j];
  const float y = u * sigm(u) * v;
  if (g_bf16) store<bf16_t>(g, e, y);
  else store<float>(g, e, y);
}

__global__ __launch_bounds__(kT) void swiglu_bwd_kernel(const float *__restrict__ dg, const float *__restrict__ h13,
                                                        int64_t R, int h, void *dh13, bool out_bf16,
                                                        const int *dev_rows) {
  if (dev_rows) R = min(R, (int64_t)*dev_rows);
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (e >= R * h) return;
  const int64_t r = e / h;
  const int j = (int)(e % h);
  const float u = h13[r * 2 * h + j], v = h13[r * 2 * h + h + j];
  const float sg = sigm(u);
  const float gg = dg[e];
  const float d1 = gg * v * sg * (1.0f + u * (1.0f - sg));
  const float d3 = gg * u * sg;
  const int64_t o1 = r * 2 * h + j, o3 = o1 + h;
  if (out_bf16) {
    store<bf16_t>(dh13, o1, d1);
    store<bf16_t>(dh13, o3, d3);
  } else {
    store<float>(dh13, o1, d1);
    store<float>(dh13, o3, d3);
  }
}

// One wave per row (d <= 1024: each lane handles d / 64 features).
constexpr int kLnRowsPerBlock = 4;

__global__ __launch_bounds__(kT) void ln_fwd_kernel(const float *__restrict__ y, int64_t R, int d,
                                                    const float *__restrict__ g, const float *__restrict__ b, void *out,
                                                    bool out_bf16, float *stats, const int *dev_rows) {
  if (dev_rows) R = min(R, (int64_t)*dev_rows);
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kLnRowsPerBlock + (threadIdx.x >> 6);
  if (r >= R) return;
  const float *yr = y + r * d;
  float s = 0.f;
  for (int f = lane; f < d; f += 64) s += yr[f];
  const float mu = wave_sum(s) / d;
  float q = 0.f;
  for (int f = lane; f < d; f += 64) {
    const float c = yr[f] - mu;
    q += c * c;
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) / d + kLnEps);
  for (int f = lane; f < d; f += 64) {
    const float v = (yr[f] - mu) * rstd * g[f] + b[f];
    if (out_bf16) store<bf16_t>(out, r * d + f, v);
    else store<float>(out, r * d + f, v);
  }
  if (lane == 0) {
    stats[2 * r] = mu;
    stats[2 * r + 1] = rstd;
  }
}

__global__ __launch_bounds__(kT) void copy_rows_kernel(const float *__restrict__ y, int64_t n, void *out,
                                                       bool out_bf16, const int *dev_rows, int d) {
  if (dev_rows) n = min(n, (int64_t)*dev_rows * d);
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (e >= n) return;
  if (out_bf16) store<bf16_t>(out, e, y[e]);
  else store<float>(out, e, y[e]);
}

// Rows per LN-backward block (each block leaves one partial row of dg, db):
// a few thousand rows (the targets) in blocks of 8, so that the launch fills
// the chip, more in blocks of 64.
constexpr int kFoldSlices = 64;  // first fold stage: partial rows cut into this many slices
int ln_bwd_rows(int64_t R) { return R <= 16384 ? 8 : 64; }

__global__ __launch_bounds__(kT) void ln_bwd_kernel(const float *__restrict__ dout, const float *__restrict__ y,
                                                    const float *__restrict__ stats, int64_t R, int d, int rows,
                                                    const float *__restrict__ g, void *dy, bool dy_bf16,
                                                    float *part, const int *dev_rows) {
  if (dev_rows) R = min(R, (int64_t)*dev_rows);
  // block: `rows` rows, one wave per row at a time; per-lane column
  // partials of dg, db kept in LDS [4 waves][d] and folded in wave order.
  // A row's values (d <= 512: up to 8 per lane) are loaded before any is used.
  extern __shared__ float sm[];
  float *pg = sm, *pb = sm + 4 * d;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int f = lane; f < d; f += 64) {
    pg[w * d + f] = 0.f;
    pb[w * d + f] = 0.f;
  }
  const int64_t rb = (int64_t)blockIdx.x * rows;
  for (int i = w; i < rows; i += 4) {
    const int64_t r = rb + i;
    if (r >= R) break;
    const float mu = stats[2 * r], rstd = stats[2 * r + 1];
    const float *dr = dout + r * d, *yr = y + r * d;
    float dv[8], yv[8], gv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int f = k * 64 + lane;
      if (f < d) {
        dv[k] = dr[f];
        yv[k] = yr[f];
        gv[k] = g[f];
      }
    }
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int f = k * 64 + lane;
      if (f < d) {
        const float xh = (yv[k] - mu) * rstd, gy = dv[k] * gv[k];
        s1 += gy;
        s2 += gy * xh;
        pg[w * d + f] += dv[k] * xh;
        pb[w * d + f] += dv[k];
      }
    }
    s1 = wave_sum(s1) / d;
    s2 = wave_sum(s2) / d;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int f = k * 64 + lane;
      if (f < d) {
        const float xh = (yv[k] - mu) * rstd, gy = dv[k] * gv[k];
        const float v = rstd * (gy - s1 - xh * s2);
        if (dy_bf16) store<bf16_t>(dy, r * d + f, v);
        else store<float>(dy, r * d + f, v);
      }
    }
  }
  __syncthreads();
  for (int f = threadIdx.x; f < d; f += kT) {
    float a = 0.f, c = 0.f;
    for (int k = 0; k < 4; ++k) {
      a += pg[k * d + f];
      c += pb[k * d + f];
    }
    part[(int64_t)blockIdx.x * 2 * d + f] = a;
    part[(int64_t)blockIdx.x * 2 * d + d + f] = c;
  }
}

// Two-stage fold of the per-block partials [nblk][2d], fixed order: stage 1,
// block (column group of 64, slice) sums its slice of partial rows (4 waves
// interleaved, then in wave order) into part2[slice][2d]; stage 2 sums the
// slices in order.  Columns are read 64 at a time by a wave: coalesced.
__global__ __launch_bounds__(kT) void ln_fold1_kernel(const float *__restrict__ part, int64_t nblk, int d,
                                                      float *part2) {
  __shared__ float sm[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int f = blockIdx.x * 64 + lane;
  const int64_t per = (nblk + kFoldSlices - 1) / kFoldSlices;
  const int64_t b0 = (int64_t)blockIdx.y * per, b1 = b0 + per < nblk ? b0 + per : nblk;
  float s = 0.f;
  if (f < 2 * d)
    for (int64_t b = b0 + w; b < b1; b += 4) s += part[b * 2 * d + f];
  sm[w][lane] = s;
  __syncthreads();
  if (w == 0 && f < 2 * d) part2[(int64_t)blockIdx.y * 2 * d + f] = ((sm[0][lane] + sm[1][lane]) + sm[2][lane]) + sm[3][lane];
}

__global__ __launch_bounds__(kT) void ln_fold2_kernel(const float *__restrict__ part2, int d, float *dg, float *db) {
  const int f = blockIdx.x * kT + threadIdx.x;
  if (f >= 2 * d) return;
  float s = 0.f;
  for (int i = 0; i < kFoldSlices; ++i) s += part2[(int64_t)i * 2 * d + f];
  if (f < d) dg[f] += s;
  else db[f - d] += s;
}

__global__ __launch_bounds__(kT) void add_rows_kernel(const float *__restrict__ src, int64_t lds, float *dst,
                                                      int64_t ldd, int64_t R, int d, bool accumulate) {
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (e >= R * d) return;
  const int64_t r = e / d;
  const int f = (int)(e % d);
  const float v = src[r * lds + f];
  dst[r * ldd + f] = accumulate ? dst[r * ldd + f] + v : v;
}

__global__ __launch_bounds__(kT) void concat_kernel(const float *__restrict__ src, int S, int64_t R, int d,
                                                    float *dst) {
  const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (e >= (int64_t)S * R * d) return;
  const int64_t sidx = e / (R * d), rem = e % (R * d);
  const int64_t r = rem / d;
  const int f = (int)(rem % d);
  dst[r * S * d + sidx * d + f] = src[e];
}

// Four features per thread, grid-stride over the live rows (the grid is
// sized for the host bound, capped).
template <bool UNIQUE>
__global__ __launch_bounds__(kT) void scatter_kernel(const float *__restrict__ rows, int64_t lds,
                                                     const int *__restrict__ ids, int64_t R, int d, float *table,
                                                     int64_t table_rows, const int *dev_rows) {
  if (dev_rows) R = min(R, (int64_t)*dev_rows);
  const int d4 = d / 4;
  const int64_t n = R * d4, step = (int64_t)gridDim.x * kT;
  for (int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x; e < n; e += step) {
    const int64_t r = e / d4;
    const int f = (int)(e % d4) * 4;
    const int id = ids[r];
    if (id < 0 || (int64_t)id >= table_rows) continue;
    const float4 v = *reinterpret_cast<const float4 *>(rows + r * lds + f);
    float *t = table + (int64_t)id * d + f;
    if (UNIQUE) {  // no other row of this launch touches the table row
      float4 o = *reinterpret_cast<float4 *>(t);
      o.x += v.x;
      o.y += v.y;
      o.z += v.z;
      o.w += v.w;
      *reinterpret_cast<float4 *>(t) = o;
    } else {
      atomicAdd(t, v.x);
      atomicAdd(t + 1, v.y);
      atomicAdd(t + 2, v.z);
      atomicAdd(t + 3, v.w);
    }
  }
}

unsigned blocks(int64_t n) { return (unsigned)((n + kT - 1) / kT); }

}  // namespace

hipError_t launch_gather_rows(const bf16_t *table, int64_t table_rows, const int *ids, int64_t R, int d, void *out,
                              bool out_bf16, hipStream_t s, const int *dev_rows) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(blocks(R * d)), dim3(kT), 0, s, table, table_rows, ids, R, d, out, out_bf16,
                     dev_rows);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const float *h13, int64_t R, int h, void *g, bool g_bf16, hipStream_t s,
                             const int *dev_rows) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(blocks(R * h)), dim3(kT), 0, s, h13, R, h, g, g_bf16, dev_rows);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float *dg, const float *h13, int64_t R, int h, void *dh13, bool out_bf16,
                             hipStream_t s, const int *dev_rows) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(blocks(R * h)), dim3(kT), 0, s, dg, h13, R, h, dh13, out_bf16, dev_rows);
  return hipGetLastError();
}

hipError_t launch_ln_fwd(const float *y, int64_t R, int d, const float *g, const float *b, void *out, bool out_bf16,
                         float *stats, hipStream_t s, const int *dev_rows) {
  if (R <= 0) return hipSuccess;
  if (!g) {
    hipLaunchKernelGGL(copy_rows_kernel, dim3(blocks(R * d)), dim3(kT), 0, s, y, R * d, out, out_bf16, dev_rows, d);
  } else {
    const unsigned nb = (unsigned)((R + kLnRowsPerBlock - 1) / kLnRowsPerBlock);
    hipLaunchKernelGGL(ln_fwd_kernel, dim3(nb), dim3(kT), 0, s, y, R, d, g, b, out, out_bf16, stats, dev_rows);
  }
  return hipGetLastError();
}

int64_t ln_part_rows(int64_t R) { return (R + ln_bwd_rows(R) - 1) / ln_bwd_rows(R) + kFoldSlices; }

hipError_t launch_ln_bwd(const float *dout, const float *y, const float *stats, int64_t R, int d, const float *g,
                         void *dy, bool dy_bf16, float *dg, float *db, float *part, hipStream_t s,
                         const int *dev_rows) {
  if (R <= 0) return hipSuccess;
  if (!g) {
    hipLaunchKernelGGL(copy_rows_kernel, dim3(blocks(R * d)), dim3(kT), 0, s, dout, R * d, dy, dy_bf16, dev_rows, d);
    return hipGetLastError();
  }
  if (d > 512) return hipErrorInvalidValue;  // up to 8 values per lane
  const int rows = ln_bwd_rows(R);
  const int64_t nblk = (R + rows - 1) / rows;
  hipLaunchKernelGGL(ln_bwd_kernel, dim3((unsigned)nblk), dim3(kT), 8 * d * sizeof(float), s, dout, y, stats, R, d,
                     rows, g, dy, dy_bf16, part, dev_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float *part2 = part + nblk * 2 * d;  // ln_part_rows() leaves room for the slices
  hipLaunchKernelGGL(ln_fold1_kernel, dim3((unsigned)((2 * d + 63) / 64), kFoldSlices), dim3(kT), 0, s, part, nblk,
                     d, part2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ln_fold2_kernel, dim3(blocks(2 * d)), dim3(kT), 0, s, part2, d, dg, db);
  return hipGetLastError();
}

hipError_t launch_ln_fold(float *part, int64_t nblk, int d, float *dg, float *db, hipStream_t s) {
  if (nblk <= 0) return hipSuccess;
  float *part2 = part + nblk * 2 * d;
  hipLaunchKernelGGL(ln_fold1_kernel, dim3((unsigned)((2 * d + 63) / 64), kFoldSlices), dim3(kT), 0, s, part, nblk,
                     d, part2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ln_fold2_kernel, dim3(blocks(2 * d)), dim3(kT), 0, s, part2, d, dg, db);
  return hipGetLastError();
}

hipError_t launch_add_rows(const float *src, int64_t lds, float *dst, int64_t ldd, int64_t R, int d, bool accumulate,
                           hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(add_rows_kernel, dim3(blocks(R * d)), dim3(kT), 0, s, src, lds, dst, ldd, R, d, accumulate);
  return hipGetLastError();
}

hipError_t launch_concat_layers(const float *src, int S, int64_t R, int d, float *dst, hipStream_t s) {
  if (R <= 0 || S <= 0) return hipSuccess;
  hipLaunchKernelGGL(concat_kernel, dim3(blocks((int64_t)S * R * d)), dim3(kT), 0, s, src, S, R, d, dst);
  return hipGetLastError();
}

hipError_t launch_scatter_add(const float *rows, const int *ids, int64_t R, int d, float *table, int64_t table_rows,
                              hipStream_t s, const int *dev_rows, int64_t lds, bool unique) {
  if (R <= 0) return hipSuccess;
  if (d % 4) return hipErrorInvalidValue;
  const unsigned g = std::min(blocks(R * (d / 4)), 4096u);
  const int64_t ld = lds > 0 ? lds : (int64_t)d;
  if (unique)
    hipLaunchKernelGGL(scatter_kernel<true>, dim3(g), dim3(kT), 0, s, rows, ld, ids, R, d, table, table_rows, dev_rows);
  else
    hipLaunchKernelGGL(scatter_kernel<false>, dim3(g), dim3(kT), 0, s, rows, ld, ids, R, d, table, table_rows,
                       dev_rows);
  return hipGetLastError();
}

}  // namespace stca
