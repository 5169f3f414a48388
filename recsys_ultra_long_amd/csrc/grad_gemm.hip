// grad_gemm.hip -- one strided GEMM for the products of the backward pass.
//
// The backward's dense products are plain GEMMs of three shapes: weight
// gradients (A^T B with K = the number of rows, up to the whole history),
// input gradients (A W^T), and the small query-side products over the
// targets.  One kernel serves all of them: a 128 x 128 output tile per
// 4-wave workgroup, each wave a 64 x 64 quadrant on 32x32x16 bf16 MFMA with
// fp32 accumulation.  Operands are staged through LDS in [row][k] order
// whatever their layout in memory (k-contiguous rows load as 16-byte runs;
// row-contiguous operands load 8 rows at one k and are written transposed),
// and fp32 operands are rounded to bf16 on the way.  Long K is split over
// blockIdx.z into partials folded in order by a second kernel, so results do
// not depend on scheduling.
#include "grad_internal.h"

namespace stca {
namespace {

constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 8;

template <typename T> DEV void load8(const T *p, float (&v)[8]);
template <> DEV void load8<bf16_t>(const bf16_t *p, float (&v)[8]) {
  const bf16x8 x = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = bf2f((bf16_t)x[e]);
}
template <> DEV void load8<float>(const float *p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = a[e];
    v[4 + e] = b[e];
  }
}

// Stage a [128 rows x 32 k] tile of an operand into S[row * LDK + k] (bf16).
// Rows r0 .. r0+127 of R, k0 .. k0+31 of [k0, ke).  KC: the k stride is 1
// (else the row stride is 1).  vec: 8-element runs along the contiguous
// dimension may be loaded as vectors (aligned, and the other stride a
// multiple of 8).
template <typename T, bool KC>
DEV void stage(const T *__restrict__ p, int64_t sr, int64_t sk, int64_t r0, int64_t R, int64_t k0, int64_t ke,
               bool vec, bf16_t *S, int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + 256 * j;
    if (KC) {
      const int r = c >> 2, kc = (c & 3) * 8;
      const int64_t gr = r0 + r, gk = k0 + kc;
      float v[8];
      if (gr < R && vec && gk + 8 <= ke) {
        load8<T>(p + gr * sr + gk, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (gr < R && gk + e < ke) ? to_f<T>(p[gr * sr + gk + e]) : 0.f;
      }
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf2(v[2 * e], v[2 * e + 1]);
      *reinterpret_cast<u32x4 *>(S + r * LDK + kc) = w;
    } else {
      const int k = c >> 4, rc = (c & 15) * 8;
      const int64_t gk = k0 + k, gr = r0 + rc;
      float v[8];
      if (gk < ke && vec && gr + 8 <= R) {
        load8<T>(p + gk * sk + gr, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (gk < ke && gr + e < R) ? to_f<T>(p[gk * sk + gr + e]) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) S[(rc + e) * LDK + k] = f2bf(v[e]);
    }
  }
}

template <typename TA, typename TB, bool AKC, bool BKC, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g, int64_t kchunk, bool va, bool vb) {
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int64_t m0 = (int64_t)blockIdx.x * BM, n0 = (int64_t)blockIdx.y * BN;
  int64_t kb = 0, ke = g.K;
  if (SPLIT) {
    kb = (int64_t)blockIdx.z * kchunk;
    ke = kb + kchunk < g.K ? kb + kchunk : g.K;
  }
  const TA *A = (const TA *)g.A;
  const TB *B = (const TB *)g.B;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int64_t k0 = kb; k0 < ke; k0 += BK) {
    stage<TA, AKC>(A, g.sam, g.sak, m0, g.M, k0, ke, va, As, tid);
    stage<TB, BKC>(B, g.sbn, g.sbk, n0, g.N, k0, ke, vb, Bs, tid);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = ld8(As + (wm * 64 + i * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = ld8(Bs + (wn * 64 + j * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + c32_row(lane, r);
        if (m >= g.M) continue;
        if (SPLIT) {
          g.part[((int64_t)blockIdx.z * g.M + m) * g.N + n] = acc[i][j][r];
        } else {
          float *c = g.C + m * g.scm + n * g.scn;
          const float v = g.alpha * acc[i][j][r];
          *c = g.beta != 0.f ? v + g.beta * *c : v;
        }
      }
    }
}

__global__ __launch_bounds__(256) void split_reduce_kernel(GemmArgs g, int split) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= g.M * g.N) return;
  const int64_t m = e / g.N, n = e % g.N;
  float s = 0.f;
  for (int z = 0; z < split; ++z) s += g.part[(int64_t)z * g.M * g.N + e];
  float *c = g.C + m * g.scm + n * g.scn;
  const float v = g.alpha * s;
  *c = g.beta != 0.f ? v + g.beta * *c : v;
}

template <typename TA, typename TB, bool AKC, bool BKC>
hipError_t run(const GemmArgs &g, hipStream_t s) {
  const int64_t es_a = g.a_bf16 ? 2 : 4, es_b = g.b_bf16 ? 2 : 4;
  // vector loads: 16-byte aligned base, and the non-unit stride a multiple of 8
  const bool va = (reinterpret_cast<uintptr_t>(g.A) % 16 == 0) && ((AKC ? g.sam : g.sak) % 8 == 0) && es_a > 0;
  const bool vb = (reinterpret_cast<uintptr_t>(g.B) % 16 == 0) && ((BKC ? g.sbn : g.sbk) % 8 == 0) && es_b > 0;
  const unsigned gx = (unsigned)((g.M + BM - 1) / BM), gy = (unsigned)((g.N + BN - 1) / BN);
  if (g.split > 1) {
    int64_t kchunk = (g.K + g.split - 1) / g.split;
    kchunk = (kchunk + BK - 1) / BK * BK;
    const int split = (int)((g.K + kchunk - 1) / kchunk);
    hipLaunchKernelGGL((gemm_kernel<TA, TB, AKC, BKC, true>), dim3(gx, gy, split), dim3(256), 0, s, g, kchunk, va,
                       vb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = g.M * g.N;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, split);
  } else {
    hipLaunchKernelGGL((gemm_kernel<TA, TB, AKC, BKC, false>), dim3(gx, gy, 1), dim3(256), 0, s, g, g.K, va, vb);
  }
  return hipGetLastError();
}

template <typename TA, typename TB>
hipError_t run_layout(const GemmArgs &g, hipStream_t s) {
  const bool akc = g.sak == 1, bkc = g.sbk == 1;
  if (akc && bkc) return run<TA, TB, true, true>(g, s);
  if (akc) return run<TA, TB, true, false>(g, s);
  if (bkc) return run<TA, TB, false, true>(g, s);
  return run<TA, TB, false, false>(g, s);
}

}  // namespace

int gemm_split_for(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int64_t split = 1;
  // aim at ~1024 workgroups, each with at least 512 of K
  while (tiles * split < 1024 && K / (split * 2) >= 512) split *= 2;
  return (int)split;
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (!((g.sak == 1 || g.sam == 1) && (g.sbk == 1 || g.sbn == 1))) return hipErrorInvalidValue;
  if (g.K <= 0) {  // empty sum: C = beta * C
    GemmArgs z = g;
    z.split = 1;
    z.K = 0;
    const int64_t n = g.M * g.N;
    if (g.beta == 1.f) return hipSuccess;
    // reuse the reduce kernel with zero partials: write alpha * 0 + beta * C
    z.part = nullptr;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, z, 0);
    return hipGetLastError();
  }
  if (g.a_bf16 && g.b_bf16) return run_layout<bf16_t, bf16_t>(g, s);
  if (g.a_bf16) return run_layout<bf16_t, float>(g, s);
  if (g.b_bf16) return run_layout<float, bf16_t>(g, s);
  return run_layout<float, float>(g, s);
}

}  // namespace stca
