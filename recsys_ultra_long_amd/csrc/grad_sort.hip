// grad_sort.hip -- per-unique-row sums of the history items' K/V gradients.
//
// With unique-id dedup the history backward runs once per distinct id: a
// row's K/V depend on its id alone, and the history side's backward is
// linear in (dK, dV) for a fixed row, so the gradients of all items that
// carry one id can be summed first.  The sum has to be in a fixed order for
// the result not to depend on scheduling, so the items are put in (unique
// index, item index) order by a stable LSD radix sort on the unique index,
// and each unique row's run is summed front to back:
//   1. radix sort (8-bit digits; per pass: block histograms, one scan,
//      stable scatter that ranks equal digits inside a wave with ballots);
//   2. run starts seg[u] (every unique index has at least one item);
//   3. runs cut into pieces of at most kPiece items, one wave per piece;
//      a run of one piece is written directly, longer runs through per-piece
//      partials folded in piece order.
#include "grad_internal.h"

namespace stca {
namespace {

constexpr int kT = 256;
constexpr int kIPT = 8;                // items per thread per sort block
constexpr int kIPB = kT * kIPT;        // items per sort block
constexpr int kPiece = 256;            // items per aggregation piece
static_assert(kPiece % 64 == 0, "whole groups of 64 item ids per piece");

__global__ __launch_bounds__(kT) void iota_kernel(int *v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i < n) v[i] = (int)i;
}

__global__ __launch_bounds__(kT) void sort_hist_kernel(const int *__restrict__ keys, int64_t n, int shift, int *hist,
                                                       int nblk) {
  __shared__ int c[256];
  c[threadIdx.x] = 0;
  __syncthreads();
  const int64_t b0 = (int64_t)blockIdx.x * kIPB;
  for (int r = 0; r < kIPT; ++r) {
    const int64_t i = b0 + r * kT + threadIdx.x;
    if (i < n) atomicAdd(&c[(keys[i] >> shift) & 255], 1);
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = c[threadIdx.x];
}

// Exclusive scan of n ints in place, in three coalesced steps: each block
// scans 1024 consecutive values (4 per thread) and leaves its total; one
// workgroup scans the totals; each block adds its offset.
constexpr int kScanB = 1024;

DEV int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// exclusive scan of the 256 threads' values of a block; returns the block total
DEV int block_excl_scan(int x, int &excl, int *sh) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int inc = wave_incl_scan(x, lane);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  int off = 0;
  for (int k = 0; k < w; ++k) off += sh[k];
  const int total = sh[0] + sh[1] + sh[2] + sh[3];
  excl = off + inc - x;
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kT) void scan_local_kernel(int *v, int64_t n, int *totals) {
  __shared__ int sh[4];
  const int64_t i0 = (int64_t)blockIdx.x * kScanB + 4 * threadIdx.x;
  int x[4], s = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = i0 + e < n ? v[i0 + e] : 0;
    s += x[e];
  }
  int excl;
  const int total = block_excl_scan(s, excl, sh);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (i0 + e < n) v[i0 + e] = excl;
    excl += x[e];
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = total;
}

__global__ __launch_bounds__(kT) void scan_add_kernel(int *v, int64_t n, const int *offs) {
  const int64_t i0 = (int64_t)blockIdx.x * kScanB + 4 * threadIdx.x;
  const int o = offs[blockIdx.x];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (i0 + e < n) v[i0 + e] += o;
}

// exclusive scan of a short array (one workgroup, chunk per thread)
__global__ __launch_bounds__(1024) void scan_small_kernel(int *v, int64_t n) {
  __shared__ int sh[1024];
  const int t = threadIdx.x;
  const int64_t C = (n + 1023) / 1024;
  const int64_t i0 = (int64_t)t * C, i1 = i0 + C < n ? i0 + C : n;
  int sum = 0;
  for (int64_t i = i0; i < i1; ++i) sum += v[i];
  sh[t] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int y = t >= o ? sh[t - o] : 0;
    __syncthreads();
    sh[t] += y;
    __syncthreads();
  }
  int run = sh[t] - sum;
  for (int64_t i = i0; i < i1; ++i) {
    const int x = v[i];
    v[i] = run;
    run += x;
  }
}

__global__ __launch_bounds__(kT) void sort_scatter_kernel(const int *__restrict__ kin, const int *__restrict__ vin,
                                                          int *kout, int *vout, int64_t n, int shift,
                                                          const int *__restrict__ hist, int nblk) {
  __shared__ int base[256];
  __shared__ int wcnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  base[tid] = hist[(int64_t)tid * nblk + blockIdx.x];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t b0 = (int64_t)blockIdx.x * kIPB;
  for (int r = 0; r < kIPT; ++r) {
    for (int k = lane; k < 256; k += 64) wcnt[w][k] = 0;
    const int64_t i = b0 + r * kT + tid;
    const bool valid = i < n;
    const int key = valid ? kin[i] : 0;
    const int dig = (key >> shift) & 255;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (dig >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & lt);
    __syncthreads();
    if (valid && rank == 0) wcnt[w][dig] = __popcll(m);
    __syncthreads();
    if (valid) {
      int pos = base[dig] + rank;
      for (int x = 0; x < w; ++x) pos += wcnt[x][dig];
      kout[pos] = key;
      vout[pos] = vin[i];
    }
    __syncthreads();
    base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

// run start of every unique index in the sorted keys; seg[U] = n
__global__ __launch_bounds__(kT) void seg_kernel(const int *__restrict__ skeys, int64_t n, const int *n_unique,
                                                 int *seg) {
  const int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i == 0) seg[*n_unique] = (int)n;
  if (i >= n) return;
  const int k = skeys[i];
  if (i == 0 || skeys[i - 1] != k) seg[k] = (int)i;
}

// pieces per unique row (all, and those of rows with more than one piece)
__global__ __launch_bounds__(kT) void pieces_kernel(const int *__restrict__ seg, const int *n_unique, int64_t max_u,
                                                    int *np, int *mp) {
  const int64_t u = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (u > max_u) return;
  int a = 0, b = 0;
  if (u < *n_unique) {
    const int len = seg[u + 1] - seg[u];
    a = (len + kPiece - 1) / kPiece;
    b = a > 1 ? a : 0;
  }
  np[u] = a;
  mp[u] = b;
}

// The unique row of every piece, and a zero count of finished pieces per row.
__global__ __launch_bounds__(kT) void p2u_kernel(const int *__restrict__ poff, const int *n_unique, int64_t max_u,
                                                 int *p2u, int *cnt) {
  const int64_t u = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (u >= max_u) return;
  cnt[u] = 0;
  if (u >= *n_unique) return;
  for (int p = poff[u]; p < poff[u + 1]; ++p) p2u[p] = (int)u;
}

// One wave per piece: the fp32 sum of its items' dK | dV rows (2d bf16
// values per row, 8 per lane per 512-value chunk), in item order.  A row of
// one piece is written at once; a row of several leaves one partial per
// piece, and the wave that finishes the row's last piece (a per-row count,
// after a device-scope fence) folds them in piece order and clears the count.
__global__ __launch_bounds__(kT) void agg_kernel(const bf16_t *__restrict__ dkv, const int *__restrict__ stok,
                                                 const int *__restrict__ seg, const int *__restrict__ poff,
                                                 const int *__restrict__ moff, const int *__restrict__ p2u,
                                                 const int *n_unique, int d2, int64_t max_pieces, bf16_t *out,
                                                 float *ppart, int *cnt) {
  const int lane = threadIdx.x & 63;
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int U = *n_unique;
  if (p >= max_pieces || p >= poff[U]) return;
  const int u = p2u[p];
  const int k = (int)(p - poff[u]);
  const int npu = poff[u + 1] - poff[u];
  const int i0 = seg[u] + k * kPiece;
  const int n = min(i0 + kPiece, seg[u + 1]) - i0;  // items of this piece, 1 .. kPiece
  // The piece's item ids, kPiece / 64 per lane, loaded together (ids past
  // the piece repeat its last one); row q of a group then comes from lane q
  // by a lane shuffle, so that 16 row loads go out at once.
  constexpr int PL = kPiece / 64;
  int tok[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) tok[j] = stok[i0 + min(j * 64 + lane, n - 1)];
  // every lane runs the loop (the shuffles read all lanes); lanes past the
  // row's 2d values read column 0 and store nothing
  for (int c0 = 0; c0 < d2; c0 += 512) {
    const int f0 = c0 + lane * 8;
    const bool on = f0 < d2;
    const int fc = on ? f0 : 0;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int m = min(n - j * 64, 64);  // items of this group of 64
      for (int b = 0; b < m; b += 16) {
        bf16x8 x[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = ld8(dkv + (int64_t)__shfl(tok[j], min(b + q, m - 1)) * d2 + fc);
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (b + q < m) {  // in item order
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += bf2f((bf16_t)x[q][e]);
          }
      }
    }
    if (!on) continue;
    if (npu == 1) {
      u32x4 wv;
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[e] = pack_bf2(acc[2 * e], acc[2 * e + 1]);
      *reinterpret_cast<u32x4 *>(out + (int64_t)u * d2 + f0) = wv;
    } else {
      float *pp = ppart + (int64_t)(moff[u] + k) * d2 + f0;
#pragma unroll
      for (int e = 0; e < 8; ++e) pp[e] = acc[e];
    }
  }
  if (npu == 1) return;
  __threadfence();  // this piece's partial is visible device-wide
  int done = 0;
  if (lane == 0) done = atomicAdd(&cnt[u], 1);
  done = __shfl(done, 0);
  if (done != npu - 1) return;
  __threadfence();
  // the row's last piece: fold all of its partials in piece order (loads
  // that bypass this CU's cache: other workgroups wrote them)
  for (int f0 = lane * 8; f0 < d2; f0 += 512) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < npu; ++q) {
      const float *pp = ppart + (int64_t)(moff[u] + q) * d2 + f0;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __hip_atomic_load(pp + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    u32x4 wv;
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] = pack_bf2(acc[2 * e], acc[2 * e + 1]);
    *reinterpret_cast<u32x4 *>(out + (int64_t)u * d2 + f0) = wv;
  }
  if (lane == 0) cnt[u] = 0;  // ready for the next layer's sums
}

int bits_for(int64_t n) {
  int b = 1;
  while (b < 31 && (int64_t(1) << b) < n) ++b;
  return b;
}

}  // namespace

int64_t agg_max_pieces(int64_t n, int64_t max_u) { return max_u + n / kPiece + 1; }
int64_t agg_max_partials(int64_t n) { return 2 * (n / kPiece) + 2; }

// scratch of excl_scan over n values: one total per block (the block totals
// of any scan of up to 256 * n / kIPB + n values fit after the histogram)
hipError_t excl_scan(int *v, int64_t n, int *tmp, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t nb = (n + kScanB - 1) / kScanB;
  hipLaunchKernelGGL(scan_local_kernel, dim3((unsigned)nb), dim3(kT), 0, s, v, n, tmp);
  hipLaunchKernelGGL(scan_small_kernel, dim3(1), dim3(1024), 0, s, tmp, nb);
  hipLaunchKernelGGL(scan_add_kernel, dim3((unsigned)nb), dim3(kT), 0, s, v, n, (const int *)tmp);
  return hipGetLastError();
}

// histogram (256 per sort block) followed by room for the block totals of
// the scans that use it as scratch
int64_t radix_hist_ints(int64_t n) {
  const int64_t h = 256 * ((n + kIPB - 1) / kIPB);
  return h + (h + n + 2) / kScanB + 2;
}
int radix_bits(int64_t max_key) { return bits_for(max_key + 1); }

hipError_t launch_radix_sort(const int *kin, const int *vin, int64_t n, int bits, int *keys[2], int *vals[2],
                             int *hist, RadixResult *res, hipStream_t s) {
  res->keys = kin;
  res->vals = vin;
  if (n <= 0) return hipSuccess;
  const int nblk = (int)((n + kIPB - 1) / kIPB);
  int *scan_tmp = hist + (int64_t)256 * nblk;  // block totals of the histogram scan
  hipError_t e = hipSuccess;
  if (!vin) {  // values: the item indices
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)((n + kT - 1) / kT)), dim3(kT), 0, s, vals[0], n);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    vin = vals[0];
  }
  int cur = 0;
  for (int shift = 0; shift < bits; shift += 8) {
    // never write the buffer being read: keys alternate 0, 1, ..; values
    // alternate away from wherever they are
    int *kout = keys[cur];
    int *vout = (vin == vals[0]) ? vals[1] : vals[0];
    hipLaunchKernelGGL(sort_hist_kernel, dim3(nblk), dim3(kT), 0, s, kin, n, shift, hist, nblk);
    if ((e = excl_scan(hist, (int64_t)256 * nblk, scan_tmp, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(nblk), dim3(kT), 0, s, kin, vin, kout, vout, n, shift, hist, nblk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    kin = kout;
    vin = vout;
    cur ^= 1;
  }
  res->keys = kin;
  res->vals = vin;
  return hipSuccess;
}

hipError_t launch_unique_sort(UniqueSumArgs &a, hipStream_t s) {
  const int64_t n = a.n;
  if (n <= 0) return hipSuccess;
  const unsigned g = (unsigned)((n + kT - 1) / kT);
  RadixResult rr;
  hipError_t e = launch_radix_sort(a.tok2u, nullptr, n, radix_bits(a.max_u), a.keys, a.vals, a.hist, &rr, s);
  if (e != hipSuccess) return e;
  a.sorted_items = rr.vals;
  hipLaunchKernelGGL(seg_kernel, dim3(g), dim3(kT), 0, s, rr.keys, n, a.n_unique, a.seg);
  const unsigned gu = (unsigned)((a.max_u + 1 + kT - 1) / kT);
  hipLaunchKernelGGL(pieces_kernel, dim3(gu), dim3(kT), 0, s, a.seg, a.n_unique, a.max_u, a.poff, a.moff);
  if ((e = excl_scan(a.poff, a.max_u + 1, a.hist, s)) != hipSuccess) return e;
  if ((e = excl_scan(a.moff, a.max_u + 1, a.hist, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(p2u_kernel, dim3((unsigned)((a.max_u + kT - 1) / kT)), dim3(kT), 0, s, a.poff, a.n_unique,
                     a.max_u, a.p2u, a.cnt);
  return hipGetLastError();
}

hipError_t launch_unique_sums(const UniqueSumArgs &a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const int64_t maxp = agg_max_pieces(a.n, a.max_u);
  hipLaunchKernelGGL(agg_kernel, dim3((unsigned)((maxp + 3) / 4)), dim3(kT), 0, s, a.dkv, a.sorted_items, a.seg,
                     a.poff, a.moff, a.p2u, a.n_unique, a.d2, maxp, a.out, a.ppart, a.cnt);
  return hipGetLastError();
}

}  // namespace stca
