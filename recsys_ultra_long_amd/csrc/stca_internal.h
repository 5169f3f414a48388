// stca_internal.h -- host-side launcher interface between the C ABI layer
// (stca_api.cpp) and the HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace stca {

// Thread-local error message of the C ABI (stca_last_error); returns `code`.
int api_error(int code, const char *fmt, ...);
void api_clear_error();

// Device-side batch plan written by the planner kernel (all int32):
//   hoff[B+1]  sanitised history offsets (all zero when the CSR is bad)
//   toff[B+1]  sanitised target offsets
//   pblk[B+1]  first 32-key block of each user in the padded K/V layout
//   coff[B+1]  first split-L chunk of each user
//   prow[]     optional (staged bf16 history): per padded row, the table id
//              of its history item, or -1 for padding and for ids outside the
//              table (prow_rows(max_blocks) entries)
struct Plan {
  int *hoff, *toff, *pblk, *coff;
  int *prow;
};

// Upper bound (host) on the padded blocks / chunks of a batch.
inline int64_t max_blocks(int64_t n_hist, int B, int align = 1) {
  return (n_hist + 31) / 32 + (int64_t)B * align;
}
inline int64_t max_chunks(int64_t n_hist, int B, int nb) {
  return (max_blocks(n_hist, B) + nb - 1) / nb + B;
}

// Padded-row id map (Plan::prow) after the planner: entries for every row of
// the 64-row tiles over max_blocks blocks.  Ids outside [0, table_rows) set
// status bit 4 and read as -1.
inline int64_t prow_rows(int64_t max_blocks) { return (max_blocks + 4) * 32; }
hipError_t launch_padded_ids(const Plan &plan, int B, const int *hist_ids, int64_t table_rows,
                             int64_t max_blocks, int *status, hipStream_t s);

// LONGER-style encoding: short_off [B+1] of the users' last min(L_u, l_short)
// items, their table ids (short_ids, padded with 0 up to `bound`) and the
// identity map iota [bound].  bound >= the device total.
hipError_t launch_short_seq(const int *hist_off, const int *hist_ids, int B, int64_t n_hist, int l_short,
                            int64_t bound, int *short_off, int *short_ids, int *iota, hipStream_t s);

// align: every user is padded to a multiple of `align` 32-key blocks (2 on
// the fused path, whose tiles hold 64 keys).  n_hist / n_tgt < 0: the host
// holds only a bound, and the offsets' totals are not checked against it.
hipError_t launch_plan(const int *hist_off, const int *tgt_off, int B, int64_t n_hist,
                       int64_t n_tgt, int max_tgt, int nb, int align, Plan plan, int *status,
                       hipStream_t s);

// ------------------------------------------------------------ row chain
// One launch computes, for a set of rows,
//   input -> [SwiGLU FFN] -> [LN] -> [projection (scaled)] -> output
// Input modes:
enum InMode { IN_GATHER_CSR = 0, IN_GATHER_IDS = 1, IN_DENSE = 2, IN_PREGEMM = 3 };
// Output modes:
enum OutMode { OUT_KV = 0, OUT_ROWS = 1, OUT_FUSED = 2 };

struct ChainArgs {
  int in_mode, out_mode;
  bool ffn, ln, proj;
  int d, hidden;
  int64_t n_rows;           // IN_GATHER_IDS / DENSE / PREGEMM: rows; CSR: max blocks * 32
  // gather
  const void *table;
  int64_t table_rows;
  const int *ids;           // per-row ids (IDS) or history ids (CSR)
  Plan plan;
  int B;
  // dense / pre-GEMM input (config dtype)
  const void *a;            // dense rows, or pre-GEMM segment 1
  int lda;
  const void *a2;           // pre-GEMM segment 2 (x_t rows)
  int lda2;
  int k1, k2;               // pre-GEMM segment widths (multiples of 32)
  const void *wpre;         // pre-GEMM weight [k1+k2, d] (bf16: packed W^T)
  void *in_dump;            // optional copy of the input rows (IDS: [n_rows, d]; CSR: per token)
  // FFN (bf16: packed W^T fragments, see PackDesc)
  const void *w1, *w3, *w2;
  const float *ln_g, *ln_b;
  // projection
  const void *wp;           // [d, pn] (bf16: packed; OUT_KV: W_K then W_V tiles)
  const void *wp2;          // fp32 OUT_KV: W_V (wp is W_K)
  int pn;
  float scale;
  // outputs
  void *out;                // OUT_ROWS, config dtype [n_rows, ldo]
  int ldo;
  float *out32;             // OUT_ROWS optional fp32 copy [n_rows, ldo32]
  int ldo32;
  void *kbuf, *vbuf;        // OUT_KV blocked layout
  int H;
  int *status;
  int pf_stride;            // history tiles: touch the rows of tile + pf_stride (0: off)
};

hipError_t launch_chain_bf16(const ChainArgs &a, hipStream_t s);

// All M layers' history encodings in one launch (bf16, d 128 or 256,
// 128-row tiles): the gathered rows of a tile are reused by every layer.  `a` carries the batch,
// plan, flags and in_dump; the per-layer weights and K/V buffers come from hl.
constexpr int kMaxLayers = 16;
struct HistLayers {
  const void *w1[kMaxLayers], *w3[kMaxLayers], *w2[kMaxLayers], *wp[kMaxLayers];
  const float *ln_g[kMaxLayers], *ln_b[kMaxLayers];
  void *kbuf[kMaxLayers], *vbuf[kMaxLayers];
  int M;
  unsigned long long *clock;  // optional [8][4]: start / end clock counters of workgroups 0..7
  int persistent;             // d = 256: about one workgroup per CU looping over the tiles (n_rows an upper bound)
};
// d = 256: 128-row tiles on 8 waves (W1, W3 packed with fmt 1).
hipError_t launch_hist256(const ChainArgs &a, const HistLayers &hl, hipStream_t s);
// The same 128-row encoder at d = 128 (hist128_bf16.hip).
hipError_t launch_hist128(const ChainArgs &a, const HistLayers &hl, hipStream_t s);
hipError_t launch_chain_f32(const ChainArgs &a, hipStream_t s);

// Weight preparation (bf16): a matrix W [K, N] (row-major, y = x W) is stored
// as W^T in MFMA fragment order.  Rows of W^T (outputs n) are grouped in
// tiles of 32, k in blocks of 32; the 2 KB of a (tile, k block) hold the two
// 32x32x16 operand fragments (half h = 0, 1) lane by lane:
//   element (n, k) -> ((rt * NK + kb) * 2 + h) * 512 + lane * 8 + e
//   rt = n / 32, kb = k / 32, lane = 32 * ((k % 32) / 16) + n % 32,
//   h = (k % 16) / 8, e = k % 8, NK = K / 32.
// so one fragment load is a single contiguous 1 KB read.  row_tile0 places
// the matrix at a tile offset of the destination (W_K and W_V share one).
// fmt 4 / 5 pack W_K / W_V of one layer (d = 256) into one array whose k
// blocks alternate between the two matrices, so that one wave's K and V
// fragments of a k block are adjacent:
//   element (n, k) -> (((rt * NK + kb) * 2 + m) * 2 + h) * 512 + lane * 8 + e,
//   m = 0 for W_K (fmt 4), 1 for W_V (fmt 5), the rest as fmt 0.
// fmt 1 packs for the 16x16x32 A operand instead (16-row tiles):
//   element (n, k) -> ((n / 16 * NK + kb) * 64 + lane) * 8 + e,
//   lane = 16 * ((k % 32) / 8) + n % 16,  e = k % 8.
// src_t = 1: the source holds W^T instead ([N, K] row-major: element (n, k)
// at src[n K + k]), for operands that are the transpose of a stored weight.
struct PackDesc {
  const bf16_t *src;
  bf16_t *dst;
  int K, N, row_tile0;
  int fmt;
  int src_t;
};
constexpr int kMaxPacks = 48;
struct PackBatch {
  PackDesc m[kMaxPacks];
};
hipError_t launch_pack_batch(const PackBatch &pb, int n, hipStream_t s);

// Offset (elements) of the lane's half-h fragment of (tile rt, block kb).
__host__ __device__ inline int64_t frag_off(int rt, int kb, int nk, int h, int lane) {
  return (((int64_t)rt * nk + kb) * 2 + h) * 512 + lane * 8;
}

// ------------------------------------------------------------ attention
struct AttnArgs {
  int dtype;                // 0 fp32, 1 bf16
  int score;                // 0 softmax, 1 relu
  int d, H, dh;
  int nb;                   // 32-key blocks per scheduling unit
  int max_tgt;
  int groups;               // target groups of 64 (1 when max_tgt <= 64)
  int tgs;                  // target slots per partial (max_tgt if one group, else 64)
  int64_t max_units;        // host bound on units (chunks x H x groups); 0: nothing to do
  int grid;                 // persistent workgroups (set by the partial launch)
  int share;                // set by the partial launch: units are (user, head) x keys and
                            // the partials are per (segment, group); 0: (user, group, head)
  int max_grid;             // fused: bound on the grid the partial buffers hold
  int fused;                // partials come from the fused kernel (slot = workgroup + user)
  int tile_blocks;          // fused: 32-key blocks per tile (2: d = 128, 4: d = 256)
  Plan plan;
  const void *kbuf, *vbuf;  // blocked K/V of one layer
  const void *q;            // [n_tgt, d] scaled queries
  int64_t n_tgt;
  float *part_ml;           // [units, tgs, 2]
  float *part_acc;          // [units, tgs, dh]
  int *part_cnt;            // [units, tgs]
  float *fstate;            // fused: per-workgroup attention state between tiles
  const int *tok2u;         // dedup: token -> unique row (kbuf = unique rows' blocked K)
  const void *vrows;        // dedup: unique rows' V, row-major [rows][d]
  float *attn;              // [n_tgt, d] fp32 (required)
  void *attn_lo;            // [n_tgt, d] config dtype copy (optional)
  int *active;              // [n_tgt, H] (optional)
  float *lse;               // [n_tgt, H] (optional, softmax): max + ln(sum of weights)
  int B;
  // Cross-Mask ([WeChat] §3.2-3.3): key_mask[token] bit h = the key is visible
  // to head h (NULL: all visible); head_map[h] = the head whose Q/K columns
  // give head h's scores (has_map; V and the output stay head h's own)
  const uint32_t *key_mask;
  int has_map;
  int head_map[16];
  // Context-similarity score bias ([WeChat] §2.2.3), blocked like K:
  // bias_blk[(b * H + h) * 32 + key] is added to the score of key `key` of
  // padded block b for head h (0 on padding rows).  NULL: no bias.
  const float *bias_blk;
};

// Partials + merge.  launch_attn_partial fills a.grid, which the merge reads.
hipError_t launch_attention(AttnArgs &a, hipStream_t s);
hipError_t launch_attn_partial(AttnArgs &a, hipStream_t s);
hipError_t launch_attn_merge(const AttnArgs &a, hipStream_t s);

inline void attn_shape(AttnArgs &a, int64_t max_chunks) {
  a.groups = (a.max_tgt + 63) / 64;
  a.tgs = a.groups > 1 ? 64 : a.max_tgt;
  a.max_units = max_chunks * a.H * a.groups;
}

// ------------------------------------------------------------ fused path
// History chain + attention of one layer in one persistent kernel (bf16;
// d 128 or 256 with d_h 32, or d 256 with d_h 64; LN after the history FFN;
// at most 64 targets per user).  Users are padded to 64-key tiles (planner
// align = 2).  Partials: one slot per (workgroup, user), H heads x max_tgt
// targets each, at most fused_grid_bound(tiles) + B slots; between tiles each
// workgroup keeps its heads' state in fused_state_bytes / grid bytes of
// at.fstate.  Sets at.grid.
constexpr int kFusedMaxGrid = 512;
// Streaming attention: cap on its persistent grid (MI355X launches 256 CUs x 2
// workgroups).  Its partials live in slots (logical workgroup + global pair):
// each workgroup's range of units covers an ordered run of pairs, so the slots
// of different (workgroup, pair) segments are distinct, and their number is
// bounded by the cap plus the pairs, whatever the history length.
constexpr int kAttnMaxGrid = 1024;
// d = 256 runs 128-key tiles on 8 waves (launch_fused256), d = 128 64-key
// tiles on 4 waves (launch_fused); users are padded to whole tiles.
inline int fused_tile_blocks(int d) { return d == 256 ? 4 : 2; }
inline int64_t fused_max_tiles(int64_t n_hist, int B, int tile_blocks) {
  const int64_t keys = 32 * (int64_t)tile_blocks;
  return (n_hist + keys - 1) / keys + B;
}
inline int64_t fused_grid_bound(int64_t max_tiles) {
  return max_tiles < kFusedMaxGrid ? max_tiles : kFusedMaxGrid;
}
// Per workgroup: every wave keeps one record of at most 11 f32x4 per lane per
// head it serves (o for <= 64 targets, then m, l, count).
inline size_t fused_state_bytes(int d, int dh, int64_t grid) {
  const int waves = d == 256 ? 8 : 4;
  const int heads_per_wave = d == 256 ? 1 : (d / 4) / dh;
  return (size_t)grid * waves * heads_per_wave * 11 * 64 * 16;
}
hipError_t launch_fused(const ChainArgs &a, AttnArgs &at, int64_t max_tiles, hipStream_t s);
hipError_t launch_fused256(const ChainArgs &a, AttnArgs &at, int64_t max_tiles, hipStream_t s);

// ------------------------------------------------------------ id dedup
// Unique-id deduplication of the history encoding (dedup.hip).  The encoder
// then runs on a one-user plan over the unique ids (uplan_*, prow =
// uniq_rows, padded with -1 to whole 128-row tiles), and each layer's K/V of
// the tokens is expanded from the unique rows.
// ------------------------------------------------------------ radix sort
// Stable LSD radix sort (8-bit digits) of n (key, value) pairs by the low
// `bits` bits of the keys (keys >= 0).  vin == nullptr: the values are the
// item indices.  keys[2], vals[2]: [n] ints each, hist: radix_hist_ints(n)
// ints (scratch).  The sorted pairs are at res->keys / res->vals (inside
// the scratch, or the inputs when bits == 0).
struct RadixResult {
  const int *keys, *vals;
};
int64_t radix_hist_ints(int64_t n);
int radix_bits(int64_t max_key);  // bits that cover keys 0 .. max_key
hipError_t launch_radix_sort(const int *kin, const int *vin, int64_t n, int bits, int *keys[2], int *vals[2],
                             int *hist, RadixResult *res, hipStream_t s);

struct DedupArgs {
  const int *ids;
  int64_t n_hist, table_rows;
  int *keys, *slot_uid;      // hash set: [mask + 1] slots
  uint32_t mask;
  int *block_cnt, *block_off;  // [(mask + 1) / 256]
  int *uniq_rows;            // [dedup_rows(n_hist)]
  int *tok2u;                // [n_hist]
  int *n_unique;             // [1]
  int *uplan_hoff, *uplan_toff, *uplan_pblk;  // [2] each
  int *status;
  // renumbering of the unique rows in increasing id order (the slot order a
  // concurrent insert leaves is not reproducible), dedup_rows(n_hist) ints
  // each, and radix_hist_ints(dedup_rows(n_hist)) for the histogram
  int *sort_in, *sort_keys[2], *sort_vals[2], *sort_hist, *perm;
};
inline int64_t dedup_rows(int64_t n_hist) { return ((n_hist + 127) / 128 + 1) * 128; }
inline int64_t dedup_slots(int64_t n_hist) {
  int64_t s = 256;
  while (s < 2 * n_hist) s <<= 1;
  return s;
}
hipError_t launch_dedup(DedupArgs &d, hipStream_t s);
// The unique rows' V (blocked, transposed per 32 rows) -> row-major [rows][d].
hipError_t launch_vrows(const bf16_t *uv, bf16_t *vrows, const int *n_unique, int64_t max_unique, int d, int H,
                        hipStream_t s);
// Token K/V (blocked, per the batch plan) from the unique rows (for K/V dumps).
hipError_t launch_expand_kv(const bf16_t *uk, const bf16_t *vrows, bf16_t *k, bf16_t *v, const int *tok2u,
                            const Plan &plan, int B, int64_t max_blocks, int d, int H, hipStream_t s);

// Row-major K, V ([n_hist, d]) -> blocked K/V layout (for stca_attention) and
// the reverse (for kv_dump).
hipError_t launch_kv_relayout(int dtype, const void *k, const void *v, void *kbuf, void *vbuf,
                              Plan plan, int B, int64_t max_blocks, int d, int H, bool to_blocked,
                              hipStream_t s);

// Caller's score bias [n_hist, H] -> the blocked layout of AttnArgs.bias_blk
// (max_blocks * H * 32 floats).
hipError_t launch_bias_relayout(const float *bias, float *out, const Plan &plan, int B, int64_t max_blocks, int H,
                                hipStream_t s);

hipError_t launch_copy_rows(int dtype, const void *src, int lds, void *dst, int ldd,
                            int64_t rows, int cols, hipStream_t s);

}  // namespace stca
