// grad_gemm.hip -- one strided GEMM for the products of the backward pass.
//
// The backward's dense products are plain GEMMs of three shapes: weight
// gradients (A^T B with K = the number of rows, up to the whole history),
// input gradients (A W^T), and the small query-side products over the
// targets.  One kernel serves all of them: a 128 x 128 output tile per
// 4-wave workgroup, each wave a 64 x 64 quadrant on 32x32x16 bf16 MFMA with
// fp32 accumulation, 64-wide k tiles double-buffered in LDS.  Each operand
// keeps its memory layout in LDS: a k-contiguous operand as [row][k] (its
// MFMA fragments are single 16-byte reads), a row-contiguous one as [k][row]
// (fragments from two transposing 8-byte LDS reads), so staging is a copy
// of 16-byte runs either way; fp32 operands are rounded to bf16 on the way.
// Long K is split over blockIdx.z into partials folded in order by a second
// kernel, so results do not depend on scheduling.
#include "grad_internal.h"

namespace stca {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;   // [row][k] tiles: 144-byte rows (4 banks apart)
constexpr int LDR = BM + 16;  // [k][row] tiles: 288-byte rows (8 banks apart)
constexpr int kTile = BM * LDK > BK * LDR ? BM * LDK : BK * LDR;
static_assert(BM == BN, "one [k][row] stride serves both operands");

// 8 consecutive elements as bf16 (rounded to nearest even).
template <typename T> DEV u32x4 load8_bf(const T *p);
template <> DEV u32x4 load8_bf<bf16_t>(const bf16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
template <> DEV u32x4 load8_bf<float>(const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  return u32x4{pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3])};
}

// One operand's share of a [128 rows x 64 k] tile: four runs of 8 elements
// along its contiguous dimension.  KC (k-contiguous): run c is row c / 8,
// k 8 (c % 8) ..; otherwise run c is k c / 16, rows 8 (c % 16) ...  Rows
// r0 .. r0+127 of R, k in [k0, k0 + 64) within [.., ke); outside reads 0.
// EDGE = false: every run lies wholly inside or wholly outside the operand
// and may be loaded as one vector (the host checks alignment, strides and
// that the contiguous extent is a multiple of 8); EDGE = true takes any
// shape element by element.
struct Runs {
  u32x4 v[4];
};

template <typename T, bool KC, bool EDGE>
DEV void tile_load(const T *__restrict__ p, int64_t sr, int64_t sk, int64_t r0, int64_t R, int64_t k0, int64_t ke,
                   bool vec, Runs &f, int tid) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    int64_t gr, gk;
    bool full, any;
    if (KC) {
      gr = r0 + (c >> 3);
      gk = k0 + (c & 7) * 8;
      full = gr < R && gk + 8 <= ke;
      any = gr < R && gk < ke;
    } else {
      gk = k0 + (c >> 4);
      gr = r0 + (c & 15) * 8;
      full = gk < ke && gr + 8 <= R;
      any = gk < ke && gr < R;
    }
    const T *q = p + gr * sr + gk * sk;
    if (!EDGE) {
      f.v[j] = any ? load8_bf<T>(q) : u32x4{0u, 0u, 0u, 0u};
    } else if (full && vec) {
      f.v[j] = load8_bf<T>(q);
    } else {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in = KC ? (any && gk + e < ke) : (any && gr + e < R);
        x[e] = in ? to_f<T>(KC ? q[e * sk] : q[e * sr]) : 0.f;
      }
      f.v[j] = u32x4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])};
    }
  }
}

template <bool KC>
DEV void tile_store(const Runs &f, bf16_t *S, int tid) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    bf16_t *d = KC ? S + (c >> 3) * LDK + (c & 7) * 8 : S + (c >> 4) * LDR + (c & 15) * 8;
    *reinterpret_cast<u32x4 *>(d) = f.v[j];
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The 32x32x16 operand fragment of rows base .. base+31 at k = kk .. kk+15:
// lane l holds row base + l % 32, k = kk + 8 (l / 32) .. + 7.  From a
// [k][row] tile the LDS transposing read does it in two steps: within each
// 16-lane group, lane 4q + r receives element r of the 8-byte runs that
// lanes 4e + q address (e = 0..3), so lane (e, q) addresses row k = .. + e,
// rows .. + 4q, and two reads cover the 8 k values.
template <bool KC>
DEV bf16x8 frag(const bf16_t *S, int base, int kk, int lane) {
  if (KC) return ld8(S + (base + (lane & 31)) * LDK + kk + 8 * (lane >> 5));
  const int g = lane >> 4, e = (lane & 15) >> 2, q = lane & 3;
  const bf16_t *p = S + (kk + 8 * (g >> 1) + e) * LDR + base + 16 * (g & 1) + 4 * q;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 4 * LDR));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Double-buffered: tile k+1 is loaded into registers while tile k is
// multiplied out of LDS, then stored into the other buffer; one barrier per
// k-tile.
template <typename TA, typename TB, bool AKC, bool BKC, bool SPLIT, bool EDGE>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g, int64_t kchunk, bool va, bool vb) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kTile];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kTile];
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
  Runs fa, fb;
  if (kb < ke) {
    tile_load<TA, AKC, EDGE>(A, g.sam, g.sak, m0, Meff, kb, ke, va, fa, tid);
    tile_load<TB, BKC, EDGE>(B, g.sbn, g.sbk, n0, g.N, kb, ke, vb, fb, tid);
    tile_store<AKC>(fa, As[0], tid);
    tile_store<BKC>(fb, Bs[0], tid);
  }
  __syncthreads();
  int cur = 0;
  for (int64_t k0 = kb; k0 < ke; k0 += BK) {
    const bool more = k0 + BK < ke;
    if (more) {
      tile_load<TA, AKC, EDGE>(A, g.sam, g.sak, m0, Meff, k0 + BK, ke, va, fa, tid);
      tile_load<TB, BKC, EDGE>(B, g.sbn, g.sbk, n0, g.N, k0 + BK, ke, vb, fb, tid);
    }
    const bf16_t *as = As[cur], *bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = frag<AKC>(as, wm * 64 + i * 32, kk, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = frag<BKC>(bs, wn * 64 + j * 32, kk, lane);
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
          float *c = g.C2 && n >= g.n_split ? g.C2 + m * g.scm + (n - g.n_split) * g.scn : Cb + m * g.scm + n * g.scn;
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
  float *c = g.C2 && n >= g.n_split ? g.C2 + m * g.scm + (n - g.n_split) * g.scn : g.C + b * g.bsc + m * g.scm + n * g.scn;
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
  // whole 8-element runs: a device cap must not cut the contiguous extent
  const bool capk = g.dev_rows && g.dev_dim == 2, capm = g.dev_rows && g.dev_dim == 1;
  const bool runs_a = va && (AKC ? g.K % 8 == 0 && !capk : g.M % 8 == 0 && !capm);
  const bool runs_b = vb && (BKC ? g.K % 8 == 0 && !capk : g.N % 8 == 0);
  const bool edge = !(runs_a && runs_b);
  if (g.split > 1) {
    int64_t kchunk = (g.K + g.split - 1) / g.split;
    kchunk = (kchunk + BK - 1) / BK * BK;
    const int split = (int)((g.K + kchunk - 1) / kchunk);
    const int nb = g.batch > 1 ? g.batch : 1;
    if (!g.part || (int64_t)nb * split * g.M * g.N > g.part_cap) return hipErrorInvalidValue;
    if (edge)
      hipLaunchKernelGGL((gemm_kernel<TA, TB, AKC, BKC, true, true>), dim3(gx, gy, (unsigned)(split * nb)), dim3(256),
                         0, s, g, kchunk, va, vb);
    else
      hipLaunchKernelGGL((gemm_kernel<TA, TB, AKC, BKC, true, false>), dim3(gx, gy, (unsigned)(split * nb)), dim3(256),
                         0, s, g, kchunk, va, vb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = g.M * g.N * nb;
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g, split, kchunk);
  } else {
    const unsigned gz = g.batch > 1 ? (unsigned)g.batch : 1u;
    if (edge)
      hipLaunchKernelGGL((gemm_kernel<TA, TB, AKC, BKC, false, true>), dim3(gx, gy, gz), dim3(256), 0, s, g, g.K, va, vb);
    else
      hipLaunchKernelGGL((gemm_kernel<TA, TB, AKC, BKC, false, false>), dim3(gx, gy, gz), dim3(256), 0, s, g, g.K, va,
                         vb);
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
  if (g.C2 && (g.batch > 1 || g.n_split <= 0 || g.n_split >= g.N)) return hipErrorInvalidValue;
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
