// plan.hip -- batch planner (a1): validates the CSR offsets on the device and
// builds the padded K/V block offsets and the split-L chunk offsets.
//
// Each user's history is padded to whole 32-key blocks so that a block never
// mixes users ([Notes] §RLB: a user's encoding is shared by all of that
// user's targets and by no one else).  Chunks group `nb` consecutive blocks of
// one user; every (chunk, head, target group) is one attention workgroup.
#include "stca_internal.h"

namespace stca {

namespace {

constexpr int kPlanThreads = 1024;

__device__ int block_exclusive_scan(int v, int *sh, int &total) {
  // Hillis-Steele inclusive scan in shared memory, then shift to exclusive.
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int o = 1; o < kPlanThreads; o <<= 1) {
    int x = (t >= o) ? sh[t - o] : 0;
    __syncthreads();
    sh[t] += x;
    __syncthreads();
  }
  int incl = sh[t];
  total = sh[kPlanThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int *__restrict__ hist_off, const int *__restrict__ tgt_off, int B, long long n_hist,
    long long n_tgt, int max_tgt, int nb, int align, Plan plan, int *status) {
  __shared__ int sh[kPlanThreads];
  __shared__ int bad_h, bad_t;
  const int t = threadIdx.x;
  if (t == 0) {
    // a negative total means the offsets were built on the device and the
    // host holds only an upper bound (the LONGER short sequences)
    bad_h = (hist_off[0] != 0) || (n_hist >= 0 ? (long long)hist_off[B] != n_hist : false);
    bad_t = (tgt_off[0] != 0) || (n_tgt >= 0 ? (long long)tgt_off[B] != n_tgt : false);
  }
  __syncthreads();
  for (int u = t; u < B; u += kPlanThreads) {
    int lh = hist_off[u + 1] - hist_off[u];
    int lt = tgt_off[u + 1] - tgt_off[u];
    if (lh < 0) atomicOr(&bad_h, 1);
    if (lt < 0 || lt > max_tgt) atomicOr(&bad_t, 1);
  }
  __syncthreads();
  const bool bh = bad_h != 0, bt = bad_t != 0;
  if (t == 0) {
    if (bh) set_status(status, 1);
    if (bt) set_status(status, 2);
  }
  int carry_b = 0, carry_c = 0;
  for (int base = 0; base <= B; base += kPlanThreads) {
    const int u = base + t;
    int nbk = 0, nch = 0;
    if (u < B) {
      int lh = bh ? 0 : hist_off[u + 1] - hist_off[u];
      nbk = (lh + 32 * align - 1) / (32 * align) * align;
      nch = (nbk + nb - 1) / nb;
    }
    int tb, tc;
    int eb = block_exclusive_scan(nbk, sh, tb);
    int ec = block_exclusive_scan(nch, sh, tc);
    if (u <= B) {
      plan.pblk[u] = carry_b + eb;
      plan.coff[u] = carry_c + ec;
      plan.hoff[u] = bh ? 0 : hist_off[u];
      plan.toff[u] = bt ? 0 : tgt_off[u];
    }
    carry_b += tb;
    carry_c += tc;
  }
}

// One thread per padded row: which user's block, which item, which id.
__global__ __launch_bounds__(256) void padded_ids_kernel(Plan plan, int B, const int *__restrict__ ids,
                                                         long long table_rows, long long rows,
                                                         int *status) {
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  int id = -1;
  const int blk = (int)(r >> 5);
  if (blk < plan.pblk[B]) {
    const int u = upper_index(plan.pblk, B, blk);
    const int j = (int)(r - (long long)plan.pblk[u] * 32);
    if (j < plan.hoff[u + 1] - plan.hoff[u]) {
      id = ids[plan.hoff[u] + j];
      if (id < 0 || (long long)id >= table_rows) {
        set_status(status, 4);
        id = -1;
      }
    }
  }
  plan.prow[r] = id;
}

// Short sequences of the LONGER-style encoding ([HyFormer] eq. (6)): user u
// keeps its last ls_u = min(L_u, l_short) items.  One block: ls_u and its
// exclusive scan into short_off (all users empty when hist_off is
// inconsistent, as in the planner).
__global__ __launch_bounds__(kPlanThreads) void short_off_kernel(const int *__restrict__ hist_off, int B,
                                                                 long long n_hist, int l_short, int *short_off) {
  __shared__ int sh[kPlanThreads];
  __shared__ int bad;
  const int t = threadIdx.x;
  if (t == 0) bad = (hist_off[0] != 0) || ((long long)hist_off[B] != n_hist);
  __syncthreads();
  for (int u = t; u < B; u += kPlanThreads)
    if (hist_off[u + 1] - hist_off[u] < 0) atomicOr(&bad, 1);
  __syncthreads();
  int carry = 0;
  for (int base = 0; base <= B; base += kPlanThreads) {
    const int u = base + t;
    int ls = 0;
    if (u < B && !bad) ls = min(hist_off[u + 1] - hist_off[u], l_short);
    int tot;
    const int ex = block_exclusive_scan(ls, sh, tot);
    if (u <= B) short_off[u] = carry + ex;
    carry += tot;
  }
}

// One block per user: the table ids of its short items (in history order),
// then every block fills its share of the identity map and pads short_ids up
// to the host bound with id 0 (rows past the device count are computed by
// bound-sized launches and discarded; they must still gather a valid row).
__global__ __launch_bounds__(256) void short_ids_kernel(const int *__restrict__ hist_off,
                                                        const int *__restrict__ hist_ids, int B,
                                                        const int *__restrict__ short_off, long long bound,
                                                        int *short_ids, int *iota) {
  const int u = blockIdx.x;
  const int s0 = short_off[u], ls = short_off[u + 1] - s0;
  const int end = hist_off[u + 1];
  for (int r = threadIdx.x; r < ls; r += 256) short_ids[s0 + r] = hist_ids[end - ls + r];
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < bound; i += stride) {
    iota[i] = (int)i;
    if (i >= short_off[B]) short_ids[i] = 0;
  }
}

}  // namespace

hipError_t launch_short_seq(const int *hist_off, const int *hist_ids, int B, int64_t n_hist, int l_short,
                            int64_t bound, int *short_off, int *short_ids, int *iota, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(short_off_kernel, dim3(1), dim3(kPlanThreads), 0, s, hist_off, B, (long long)n_hist, l_short,
                     short_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || bound <= 0) return e;
  hipLaunchKernelGGL(short_ids_kernel, dim3((unsigned)B), dim3(256), 0, s, hist_off, hist_ids, B, short_off,
                     (long long)bound, short_ids, iota);
  return hipGetLastError();
}

hipError_t launch_padded_ids(const Plan &plan, int B, const int *hist_ids, int64_t table_rows,
                             int64_t max_blocks, int *status, hipStream_t s) {
  const int64_t rows = prow_rows(max_blocks);
  hipLaunchKernelGGL(padded_ids_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, plan, B,
                     hist_ids, (long long)table_rows, (long long)rows, status);
  return hipGetLastError();
}

hipError_t launch_plan(const int *hist_off, const int *tgt_off, int B, int64_t n_hist,
                       int64_t n_tgt, int max_tgt, int nb, int align, Plan plan, int *status,
                       hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, hist_off, tgt_off, B,
                     (long long)n_hist, (long long)n_tgt, max_tgt, nb, align, plan, status);
  return hipGetLastError();
}

}  // namespace stca
