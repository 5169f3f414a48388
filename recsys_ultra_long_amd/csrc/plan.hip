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
    bad_h = (hist_off[0] != 0) || ((long long)hist_off[B] != n_hist);
    bad_t = (tgt_off[0] != 0) || ((long long)tgt_off[B] != n_tgt);
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

}  // namespace

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
