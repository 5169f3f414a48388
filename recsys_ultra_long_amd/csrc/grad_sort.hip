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
//   3. the sorted items cut into spans of kSpan, one wave per span, which
//      sums each run (or the part of it inside the span) front to back: a
//      run inside the span is written directly, one that crosses a span
//      boundary leaves one partial per span, and a second launch folds them
//      in span order.
#include "grad_internal.h"

namespace stca {
namespace {

constexpr int kT = 256;
constexpr int kIPT = 8;                // items per thread per sort block
constexpr int kIPB = kT * kIPT;        // items per sort block
constexpr int kSpan = 128;             // sorted items per wave of the run sums (two per lane)

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

// One wave per span of kSpan consecutive items in (unique row, item) order:
// the fp32 sum of each run's dK | dV rows over the span (2d bf16 values per
// row, 8 per lane per 512-value block), in item order.  Rows are loaded 16 at
// a time across run boundaries (item ids and run keys one per lane, passed
// round by lane shuffles).  A run that lies inside the span is written as
// bf16 at once; one that continues from the previous span leaves its partial
// in slot 2w, one that starts here and continues in slot 2w + 1.
__global__ __launch_bounds__(kT) void span_sum_kernel(const bf16_t *__restrict__ dkv, const int *__restrict__ skey,
                                                      const int *__restrict__ stok, int64_t n, int d2, bf16_t *out,
                                                      float *ppart) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t j0 = w * kSpan;
  if (j0 >= n) return;
  const int m = (int)min((int64_t)kSpan, n - j0);  // items of this span, 1 .. kSpan
  const int ia = min(lane, m - 1), ib = min(64 + lane, m - 1);
  const int key0 = skey[j0 + ia], key1 = skey[j0 + ib];
  const int tok0 = stok[j0 + ia], tok1 = stok[j0 + ib];
  const int prev = j0 > 0 ? skey[j0 - 1] : -1;     // the run before the span
  const int next = j0 + m < n ? skey[j0 + m] : -1;  // the run after it
  // every lane runs the loops (the shuffles read all lanes); lanes past the
  // row's 2d values read column 0 and store nothing
  for (int c0 = 0; c0 < d2; c0 += 512) {
    const int f0 = c0 + lane * 8;
    const bool on = f0 < d2;
    const int fc = on ? f0 : 0;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int cur = __shfl(key0, 0), start = 0;  // the current run and its first item in the span
    auto flush = [&](bool cont_next) {
      const bool cont_prev = start == 0 && cur == prev;
      if (!on) return;
      if (!cont_prev && !cont_next) {
        u32x4 wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = pack_bf2(acc[2 * e], acc[2 * e + 1]);
        *reinterpret_cast<u32x4 *>(out + (int64_t)cur * d2 + f0) = wv;
      } else {
        float *pp = ppart + (2 * w + (cont_prev ? 0 : 1)) * d2 + f0;
        *reinterpret_cast<float4 *>(pp) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4 *>(pp + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
      }
    };
    for (int b = 0; b < m; b += 16) {
      bf16x8 x[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int j = min(b + q, m - 1);
        x[q] = ld8(dkv + (int64_t)__shfl(j < 64 ? tok0 : tok1, j & 63) * d2 + fc);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int j = b + q;
        if (j < m) {
          const int k = __shfl(j < 64 ? key0 : key1, j & 63);
          if (k != cur) {  // the run ended at item j - 1
            flush(false);
            cur = k;
            start = j;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += bf2f((bf16_t)x[q][e]);
        }
      }
    }
    flush(cur == next);
  }
}

// One workgroup per span w whose last run starts in span w and continues past
// it: that run's partials (slot 2w + 1, then slot 2c of each later span c it
// reaches) summed in span order -- eight waves over fixed consecutive groups
// of them, the group sums then in wave order -- and written as bf16.
constexpr int kFoldT = 512;
__global__ __launch_bounds__(kFoldT) void span_fold_kernel(const int *__restrict__ skey, const int *__restrict__ seg,
                                                           int64_t n, int d2, const float *__restrict__ ppart,
                                                           bf16_t *out) {
  __shared__ float red[kFoldT / 64][1024];
  const int64_t w = blockIdx.x;
  const int64_t j1 = (w + 1) * kSpan;  // first item after the span
  if (j1 >= n) return;                 // the last span: nothing continues
  const int u = skey[j1 - 1];
  if (skey[j1] != u) return;           // its last run ends inside it
  if (seg[u] < w * kSpan) return;      // the run started earlier: folded there
  const int k = (int)((seg[u + 1] - 1) / kSpan - w + 1);  // spans the run reaches
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = (k + kFoldT / 64 - 1) / (kFoldT / 64);
  const int q0 = min(wave * G, k), q1 = min(q0 + G, k);
  for (int f0 = lane * 4; f0 < d2; f0 += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int qb = q0; qb < q1; qb += 8) {
      float4 x[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int q = min(qb + r, q1 - 1);
        const int64_t slot = q == 0 ? 2 * w + 1 : 2 * (w + q);
        x[r] = *reinterpret_cast<const float4 *>(ppart + slot * d2 + f0);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (qb + r < q1) {
          acc.x += x[r].x;
          acc.y += x[r].y;
          acc.z += x[r].z;
          acc.w += x[r].w;
        }
    }
    *reinterpret_cast<float4 *>(&red[wave][f0]) = acc;
  }
  __syncthreads();
  for (int f = 2 * threadIdx.x; f < d2; f += 2 * kFoldT) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int g = 0; g < kFoldT / 64; ++g) {
      a0 += red[g][f];
      a1 += red[g][f + 1];
    }
    *reinterpret_cast<uint32_t *>(out + (int64_t)u * d2 + f) = pack_bf2(a0, a1);
  }
}

int bits_for(int64_t n) {
  int b = 1;
  while (b < 31 && (int64_t(1) << b) < n) ++b;
  return b;
}

}  // namespace

int64_t agg_partial_floats(int64_t n, int d2) { return 2 * ((n + kSpan - 1) / kSpan) * (int64_t)d2; }

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
  a.sorted_keys = rr.keys;
  hipLaunchKernelGGL(seg_kernel, dim3(g), dim3(kT), 0, s, rr.keys, n, a.n_unique, a.seg);
  return hipGetLastError();
}

hipError_t launch_unique_sums(const UniqueSumArgs &a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (a.d2 > 1024 || a.d2 % 8) return hipErrorInvalidValue;
  const int64_t spans = (a.n + kSpan - 1) / kSpan;
  hipLaunchKernelGGL(span_sum_kernel, dim3((unsigned)((spans + 3) / 4)), dim3(kT), 0, s, a.dkv, a.sorted_keys,
                     a.sorted_items, a.n, a.d2, a.out, a.ppart);
  hipLaunchKernelGGL(span_fold_kernel, dim3((unsigned)spans), dim3(kFoldT), 0, s, a.sorted_keys, a.seg, a.n, a.d2,
                     (const float *)a.ppart, a.out);
  return hipGetLastError();
}

}  // namespace stca
