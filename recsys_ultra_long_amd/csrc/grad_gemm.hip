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

// A [128 rows x 32 k] tile of an operand, as each thread holds it between
// its global load and its LDS store: two runs of 8 elements along the
// contiguous dimension (KC: along k; else along rows).  Rows r0 .. r0+127 of
// R, k in [k0, k0 + 32) within [.., ke).  vec: an 8-element run may be loaded
// as vectors (aligned, and the other stride a multiple of 8).
struct Frag {
  float v[2][8];
};

template <typename T, bool KC>
DEV void tile_load(const T *__restrict__ p, int64_t sr, int64_t sk, int64_t r0, int64_t R, int64_t k0, int64_t ke,
                   bool vec, Frag &f, int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + 256 * j;
    if (KC) {
      const int64_t gr = r0 + (c >> 2), gk = k0 + (c & 3) * 8;
      if (gr < R && vec && gk + 8 <= ke) {
        load8<T>(p + gr * sr + gk, f.v[j]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[j][e] = (gr < R && gk + e < ke) ? to_f<T>(p[gr * sr + gk + e]) : 0.f;
      }
    } else {
      const int64_t gk = k0 + (c >> 4), gr = r0 + (c & 15) * 8;
      if (gk < ke && vec && gr + 8 <= R) {
        load8<T>(p + gk * sk + gr, f.v[j]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[j][e] = (gk < ke && gr + e < R) ? to_f<T>(p[gk * sk + gr + e]) : 0.f;
      }
    }
  }
}

// ... into S[row * LDK + k] (bf16, rounded to nearest even)
template <bool KC>
DEV void tile_store(const Frag &f, bf16_t *S, int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + 256 * j;
    if (KC) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf2(f.v[j][2 * e], f.v[j][2 * e + 1]);
      *reinterpret_cast<u32x4 *>(S + (c >> 2) * LDK + (c & 3) * 8) = w;
    } else {
      const int k = c >> 4, rc = (c & 15) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) S[(rc + e) * LDK + k] = f2bf(f.v[j][e]);
    }
  }
}

// Double-buffered: tile k+1 is loaded into registers while tile k is
// multiplied out of LDS, then stored into the other buffer; one barrier per
// k-tile.
template <typename TA, typename TB, bool AKC, bool BKC, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g, int64_t kchunk, bool va, bool vb) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int64_t m0 = (int64_t)blockIdx.x * BM, n0 = (int64_t)blockIdx.y * BN;
  int64_t kb = 0, ke = g.K, Meff = g.M;
  int bz = blockIdx.z;  // batch index (and, split, K range: z = batch * ranges + range)
  if (SPLIT) {
    const int ranges = (int)((g.K + kchunk - 1) / kchunk);
    bz = (int)blockIdx.z / ranges;
    kb = (int64_t)(blockIdx.z % ranges) * kchunk;
    ke = kb + kchunk < g.K ? kb + kchunk : g.K;
  }
  if (g.dev_rows) {
    const int64_t lim = *g.dev_rows;
    if (g.dev_dim == 1) {
      Meff = lim < g.M ? lim : g.M;
      if (m0 >= Meff) return;  // the whole workgroup: before any barrier
    } else if (g.dev_dim == 2 && lim < ke) {
      ke = lim;
      if (SPLIT && kb >= ke) return;  // a range past the device count: the fold skips it
    }
  }
  const TA *A = (const TA *)g.A;
  const TB *B = (const TB *)g.B;
  float *Cb = g.C;
  if (g.batch > 1) {
    A += (int64_t)bz * g.bsa;
    B += (int64_t)bz * g.bsb;
    Cb += (int64_t)bz * g.bsc;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  Frag fa, fb;
  if (kb < ke) {
    tile_load<TA, AKC>(A, g.sam, g.sak, m0, Meff, kb, ke, va, fa, tid);
    tile_load<TB, BKC>(B, g.sbn, g.sbk, n0, g.N, kb, ke, vb, fb, tid);
    tile_store<AKC>(fa, As[0], tid);
    tile_store<BKC>(fb, Bs[0], tid);
  }
  __syncthreads();
  int cur = 0;
  for (int64_t k0 = kb; k0 < ke; k0 += BK) {
    const bool more = k0 + BK < ke;
    if (more) {
      tile_load<TA, AKC>(A, g.sam, g.sak, m0, Meff, k0 + BK, ke, va, fa, tid);
      tile_load<TB, BKC>(B, g.sbn, g.sbk, n0, g.N, k0 + BK, ke, vb, fb, tid);
    }
    const bf16_t *as = As[cur], *bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = ld8(as + (wm * 64 + i * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = ld8(bs + (wn * 64 + j * 32 + (lane & 31)) * LDK + kk + 8 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (more) {
      tile_store<AKC>(fa, As[cur ^ 1], tid);
      tile_store<BKC>(fb, Bs[cur ^ 1], tid);
    }
    __syncthreads();
    cur ^= 1;
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
        if (m >= Meff) continue;
        if (SPLIT) {
          g.part[((int64_t)blockIdx.z * g.M + m) * g.N + n] = acc[i][j][r];
        } else {
          float *c = Cb + m * g.scm + n * g.scn;
          const float v = g.alpha * acc[i][j][r];
          *c = g.beta != 0.f ? v + g.beta * *c : v;
        }
      }
    }
}

// Folds the K ranges in order; with a device cap on K only the ranges that
// start below it were written.  Partials: [batch][split][M][N].
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmArgs g, int split, int64_t kchunk) {
  const int64_t MN = g.M * g.N;
  const int nb = g.batch > 1 ? g.batch : 1;
  const int64_t ei = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (ei >= MN * nb) return;
  const int64_t b = ei / MN, e = ei % MN;
  const int stride = split;
  if (g.dev_rows && g.dev_dim == 2 && kchunk > 0) {
    const int64_t lim = *g.dev_rows;
    const int64_t live = (lim + kchunk - 1) / kchunk;
    if (live < split) split = (int)live;
  }
  const int64_t m = e / g.N, n = e % g.N;
  float s = 0.f;
  for (int z = 0; z < split; ++z) s += g.part[((int64_t)b * stride + z) * MN + e];
  float *c = g.C + b * g.bsc + m * g.scm + n * g.scn;
  const float v = g.alpha * s;
  *c = g.beta != 0.f ? v + g.beta * *c : v;
}

template <typename TA, typename TB, bool AKC, bool BKC>
hipError_t run(const GemmArgs &g, hipStream_t s) {
  // vector loads: 16-byte aligned base, and the non-unit stride a multiple of 8
  const bool bat = g.batch > 1;
  const bool va = (reinterpret_cast<uintptr_t>(g.A) % 16 == 0) && ((AKC ? g.sam : g.sak) % 8 == 0) &&
                  (!bat || g.bsa % 8 == 0);
  const bool vb = (reinterpret_cast<uintptr_t>(g.B) % 16 == 0) && ((BKC ? g.sbn : g.sbk) % 8 == 0) &&
                  (!bat || g.bsb % 8 == 0);
  const unsigned gx = (unsigned)((g.M + BM - 1) / BM), gy = (unsigned)((g.N + BN - 1) / BN);
  if (g.split > 1) {
    int64_t kchunk = (g.K + g.split - 1) / g.split;
    kchunk = (kchunk + BK - 1) / BK * BK;
    const int split = (int)((g.K + kchunk - 1) / kchunk);
    const int nb = g.batch > 1 ? g.batch : 1;
    if (!g.part || (int64_t)nb * split * g.M * g.N > g.part_cap) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_kernel<TA, TB, AKC, BKC, true>), dim3(gx, gy, (unsigned)(split * nb)), dim3(256), 0, s,
                       g, kchunk, va, vb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = g.M * g.N * nb;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, split, kchunk);
  } else {
    const unsigned gz = g.batch > 1 ? (unsigned)g.batch : 1u;
    hipLaunchKernelGGL((gemm_kernel<TA, TB, AKC, BKC, false>), dim3(gx, gy, gz), dim3(256), 0, s, g, g.K, va, vb);
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

int gemm_split_for(int64_t M, int64_t N, int64_t K, int64_t target, int64_t min_chunk) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int64_t split = 1;
  // aim at `target` workgroups, each with at least min_chunk of K
  while (tiles * split < target && K / (split * 2) >= min_chunk) split *= 2;
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
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, z, 0, (int64_t)0);
    return hipGetLastError();
  }
  if (g.a_bf16 && g.b_bf16) return run_layout<bf16_t, bf16_t>(g, s);
  if (g.a_bf16) return run_layout<bf16_t, float>(g, s);
  if (g.b_bf16) return run_layout<float, bf16_t>(g, s);
  return run_layout<float, float>(g, s);
}

}  // namespace stca
