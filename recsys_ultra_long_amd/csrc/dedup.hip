// dedup.hip -- unique-id deduplication of the history encoding.
//
// A history row's encoding depends on its table id alone (every layer's FFN
// reads the raw embedding row, [Notes] §STCA), so each layer's K/V need only
// be computed once per distinct id of the batch and copied to every token
// that carries it.  Under Zipf-distributed ids that is a fraction of the rows
// (the HyFormer page reports about a quarter unique, §3.8.1).
//
// Steps (all on the device, no host round trip):
//   1. open-addressing hash set of the batch's ids (ids outside the table
//      all become one entry, id -1, which gathers a zero row as before);
//   2. unique numbering in slot order: per-block counts, one scan, per-slot
//      index -- deterministic, no atomics decide the order;
//   3. the encoder's input: the unique ids padded to whole 128-row tiles, as
//      a one-user plan whose padded-row id map is that list;
//   4. token -> unique index map;
//   5. after the encoder: the unique rows' V re-laid row-major (the attention
//      then reads every token's K/V through the token -> unique map); the
//      per-token blocked K/V is only expanded when the caller dumps it.
#include "stca_internal.h"

namespace stca {
namespace {

constexpr int kT = 256;
constexpr int kEmpty = INT32_MIN;  // free slot (ids are >= -1 once clamped)

DEV uint32_t hash_id(int id) {
  // splitmix-style 32-bit finaliser
  uint32_t x = (uint32_t)id;
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

DEV int clamp_id(int id, long long table_rows) { return (id < 0 || (long long)id >= table_rows) ? -1 : id; }

// Probe for `id`; inserts it when `insert`.  Returns its slot (or -1 if absent).
DEV int probe(int *keys, uint32_t mask, int id, bool insert) {
  uint32_t h = hash_id(id) & mask;
  for (uint32_t n = 0; n <= mask; ++n) {
    const int k = keys[h];
    if (k == id) return (int)h;
    if (k == kEmpty) {
      if (!insert) return -1;
      const int prev = atomicCAS(&keys[h], kEmpty, id);
      if (prev == kEmpty || prev == id) return (int)h;
    }
    h = (h + 1) & mask;
  }
  return -1;  // unreachable: the table holds at least twice the tokens
}

__global__ __launch_bounds__(kT) void clear_kernel(int *keys, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (i < n) keys[i] = kEmpty;
}

// Ids repeat heavily (Zipf: the most frequent one fills ~10% of a batch), and
// thousands of threads racing to insert one id into one global slot would
// serialise on it.  Each workgroup first dedups its 256 ids in an LDS set; one
// thread per distinct id then inserts it into the global set.
constexpr int kLocal = 512;  // LDS set size (2 x the workgroup)
__global__ __launch_bounds__(kT) void insert_kernel(DedupArgs d) {
  __shared__ int lk[kLocal];
  for (int i = threadIdx.x; i < kLocal; i += kT) lk[i] = kEmpty;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (t >= d.n_hist) return;
  int id = d.ids[t];
  if (id < 0 || (long long)id >= d.table_rows) {
    set_status(d.status, 4);
    id = -1;
  }
  uint32_t h = hash_id(id) & (kLocal - 1);
  for (int n = 0; n < kLocal; ++n) {  // at most 256 distinct ids: always finds room
    const int prev = atomicCAS(&lk[h], kEmpty, id);
    if (prev == id) return;                            // another thread carries it
    if (prev == kEmpty) break;                         // this thread carries it
    h = (h + 1) & (kLocal - 1);
  }
  probe(d.keys, d.mask, id, true);
}

// Occupied slots per 256-slot block.
__global__ __launch_bounds__(kT) void count_kernel(DedupArgs d) {
  __shared__ int c;
  if (threadIdx.x == 0) c = 0;
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (d.keys[s] != kEmpty) atomicAdd(&c, 1);
  __syncthreads();
  if (threadIdx.x == 0) d.block_cnt[blockIdx.x] = c;
}

// Exclusive scan of the block counts (one workgroup); writes the unique count
// and the one-user plan of the unique rows (blocks of 32 padded to tiles).
__global__ __launch_bounds__(1024) void scan_kernel(DedupArgs d, int nblk) {
  __shared__ int sh[1024];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nblk; base += 1024) {
    const int i = base + threadIdx.x;
    const int v = i < nblk ? d.block_cnt[i] : 0;
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int x = threadIdx.x >= o ? sh[threadIdx.x - o] : 0;
      __syncthreads();
      sh[threadIdx.x] += x;
      __syncthreads();
    }
    if (i < nblk) d.block_off[i] = carry + sh[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 0) carry += sh[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int U = carry;
    d.uplan_hoff[0] = 0;
    d.uplan_hoff[1] = U;
    d.uplan_pblk[0] = 0;
    d.uplan_pblk[1] = (U + 127) / 128 * 4;  // whole 128-row tiles
    d.uplan_toff[0] = 0;
    d.uplan_toff[1] = 0;
    *d.n_unique = U;
  }
}

// Unique index of every occupied slot (slot order), and the unique id list.
__global__ __launch_bounds__(kT) void assign_kernel(DedupArgs d) {
  __shared__ int sh[kT];
  const int64_t s = (int64_t)blockIdx.x * kT + threadIdx.x;
  const int occ = d.keys[s] != kEmpty ? 1 : 0;
  sh[threadIdx.x] = occ;
  __syncthreads();
  for (int o = 1; o < kT; o <<= 1) {
    const int x = threadIdx.x >= o ? sh[threadIdx.x - o] : 0;
    __syncthreads();
    sh[threadIdx.x] += x;
    __syncthreads();
  }
  if (occ) {
    const int u = d.block_off[blockIdx.x] + sh[threadIdx.x] - 1;
    d.slot_uid[s] = u;
    d.uniq_rows[u] = d.keys[s];
  }
}

// Padding of the unique id list up to whole tiles (rows the encoder reads).
__global__ __launch_bounds__(kT) void pad_kernel(DedupArgs d, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (r < rows && r >= *d.n_unique) d.uniq_rows[r] = -1;
}

// Sort keys of the unique rows: id + 1 (the out-of-range entry, id -1, sorts
// first), padding rows after every id.
__global__ __launch_bounds__(kT) void sortkey_kernel(DedupArgs d, int64_t rows, int pad_key) {
  const int64_t r = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (r < rows) d.sort_in[r] = r < *d.n_unique ? d.uniq_rows[r] + 1 : pad_key;
}

// Row r of the id order was row perm^-1(r) of the slot order.
__global__ __launch_bounds__(kT) void renumber_kernel(DedupArgs d, int64_t rows, const int *skeys,
                                                      const int *svals) {
  const int64_t r = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (r >= rows) return;
  if (r < *d.n_unique) {
    d.perm[svals[r]] = (int)r;
    d.uniq_rows[r] = skeys[r] - 1;
  } else {
    d.uniq_rows[r] = -1;
  }
}

__global__ __launch_bounds__(kT) void slot_renumber_kernel(DedupArgs d) {
  const int64_t s = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (d.keys[s] != kEmpty) d.slot_uid[s] = d.perm[d.slot_uid[s]];
}

__global__ __launch_bounds__(kT) void map_kernel(DedupArgs d) {
  const int64_t t = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (t >= d.n_hist) return;
  const int id = clamp_id(d.ids[t], d.table_rows);
  const int sl = probe(d.keys, d.mask, id, false);  // present: inserted above
  d.tok2u[t] = sl >= 0 ? d.slot_uid[sl] : 0;
}

// The encoder writes V transposed per 32-row block (V[blk][h][d_h][row]);
// the expansion wants whole rows: V^T blocks of the unique rows -> row-major
// [rows][d], one workgroup per block through LDS.
constexpr int kMaxD = 512;
__global__ __launch_bounds__(kT) void vrows_kernel(const bf16_t *__restrict__ uv, bf16_t *__restrict__ vr,
                                                   const int *__restrict__ n_unique, int d, int H) {
  __shared__ bf16_t t[32][kMaxD + 8];
  const int ub = blockIdx.x;
  if (ub * 32 >= *n_unique) return;
  const int DH = d / H;
  for (int e = threadIdx.x; e < d * 32; e += kT) {  // (h, dh, row), row fastest
    const int f = e / 32, r = e % 32;
    t[r][f] = uv[((int64_t)ub * d + f) * 32 + r];  // [blk][h][dh][row] = [blk][f][row]
  }
  __syncthreads();
  const int C8 = d / 8;
  for (int e = threadIdx.x; e < 32 * C8; e += kT) {
    const int r = e / C8, c = (e % C8) * 8;
    *reinterpret_cast<u32x4 *>(vr + ((int64_t)ub * 32 + r) * d + c) = *reinterpret_cast<const u32x4 *>(&t[r][c]);
  }
  (void)DH;
}

// Blocked K/V of the tokens from the unique rows: one workgroup per padded
// 32-key block.  K rows are copied in 16-byte pieces from the unique K blocks
// (same layout); V rows are gathered into LDS and written transposed.
__global__ __launch_bounds__(kT) void expand_kernel(const bf16_t *__restrict__ uk, const bf16_t *__restrict__ vr,
                                                    bf16_t *__restrict__ k, bf16_t *__restrict__ v,
                                                    const int *__restrict__ tok2u, Plan P, int B, int d, int H) {
  __shared__ bf16_t t[32][kMaxD + 8];
  __shared__ int s_u[32];
  const int b = blockIdx.x;
  if (b >= P.pblk[B]) return;
  const int DH = d / H;
  const int u = upper_index(P.pblk, B, b);
  const int L = P.hoff[u + 1] - P.hoff[u];
  const int j0 = (b - P.pblk[u]) * 32;
  if (threadIdx.x < 32) s_u[threadIdx.x] = j0 + (int)threadIdx.x < L ? tok2u[P.hoff[u] + j0 + threadIdx.x] : -1;
  __syncthreads();
  // K: [blk][h][key][d_h]
  const int C8h = DH / 8;
  for (int e = threadIdx.x; e < H * 32 * C8h; e += kT) {
    const int h = e / (32 * C8h), key = (e / C8h) % 32, c = (e % C8h) * 8;
    const int ui = s_u[key];
    u32x4 val = {0u, 0u, 0u, 0u};
    if (ui >= 0) val = *reinterpret_cast<const u32x4 *>(uk + (((int64_t)(ui >> 5) * H + h) * 32 + (ui & 31)) * DH + c);
    *reinterpret_cast<u32x4 *>(k + (((int64_t)b * H + h) * 32 + key) * DH + c) = val;
  }
  // V rows -> LDS, then V^T: [blk][h][d_h][key]
  const int C8 = d / 8;
  for (int e = threadIdx.x; e < 32 * C8; e += kT) {
    const int key = e / C8, c = (e % C8) * 8;
    const int ui = s_u[key];
    u32x4 val = {0u, 0u, 0u, 0u};
    if (ui >= 0) val = *reinterpret_cast<const u32x4 *>(vr + (int64_t)ui * d + c);
    *reinterpret_cast<u32x4 *>(&t[key][c]) = val;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < d * 4; e += kT) {  // (f = h d_h + dh, 8 keys), 16 bytes per store
    const int f = e / 4, k0 = (e % 4) * 8;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)t[k0 + 2 * i][f] | ((uint32_t)t[k0 + 2 * i + 1][f] << 16);
    *reinterpret_cast<u32x4 *>(v + ((int64_t)b * d + f) * 32 + k0) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

}  // namespace

hipError_t launch_dedup(DedupArgs &d, hipStream_t s) {
  if (d.n_hist <= 0) return hipSuccess;
  const unsigned g = (unsigned)((d.n_hist + kT - 1) / kT);
  const int64_t slots = (int64_t)d.mask + 1;
  const unsigned gs = (unsigned)(slots / kT);
  hipLaunchKernelGGL(clear_kernel, dim3(gs), dim3(kT), 0, s, d.keys, slots);
  hipLaunchKernelGGL(insert_kernel, dim3(g), dim3(kT), 0, s, d);
  hipLaunchKernelGGL(count_kernel, dim3(gs), dim3(kT), 0, s, d);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, d, (int)gs);
  hipLaunchKernelGGL(assign_kernel, dim3(gs), dim3(kT), 0, s, d);
  const int64_t rows = dedup_rows(d.n_hist);
  hipLaunchKernelGGL(pad_kernel, dim3((unsigned)((rows + kT - 1) / kT)), dim3(kT), 0, s, d, rows);
  // number the unique rows in increasing id order
  const int bits = radix_bits(d.table_rows + 1);  // keys 0 .. table_rows, and the padding key
  const int pad_key = (int)((1ll << bits) - 1);
  const unsigned gr = (unsigned)((rows + kT - 1) / kT);
  hipLaunchKernelGGL(sortkey_kernel, dim3(gr), dim3(kT), 0, s, d, rows, pad_key);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RadixResult rr;
  if ((e = launch_radix_sort(d.sort_in, nullptr, rows, bits, d.sort_keys, d.sort_vals, d.sort_hist, &rr, s)))
    return e;
  hipLaunchKernelGGL(renumber_kernel, dim3(gr), dim3(kT), 0, s, d, rows, rr.keys, rr.vals);
  hipLaunchKernelGGL(slot_renumber_kernel, dim3(gs), dim3(kT), 0, s, d);
  hipLaunchKernelGGL(map_kernel, dim3(g), dim3(kT), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_vrows(const bf16_t *uv, bf16_t *vrows, const int *n_unique, int64_t max_unique, int d, int H,
                        hipStream_t s) {
  if (max_unique <= 0) return hipSuccess;
  if (d > kMaxD || d % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vrows_kernel, dim3((unsigned)((max_unique + 31) / 32)), dim3(kT), 0, s, uv, vrows, n_unique, d,
                     H);
  return hipGetLastError();
}

hipError_t launch_expand_kv(const bf16_t *uk, const bf16_t *vrows, bf16_t *k, bf16_t *v, const int *tok2u,
                            const Plan &plan, int B, int64_t max_blocks, int d, int H, hipStream_t s) {
  if (max_blocks <= 0) return hipSuccess;
  if (d > kMaxD || d % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)max_blocks), dim3(kT), 0, s, uk, vrows, k, v, tok2u, plan, B,
                     d, H);
  return hipGetLastError();
}

}  // namespace stca
