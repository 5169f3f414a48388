// hist_common.h -- pieces shared by the 128-row history encoders
// (hist_bf16.hip at d = 256, hist128_bf16.hip at d = 128): the register ring
// through which the weight fragments stream, one weight phase over that ring,
// and the gather of a tile's table rows into LDS.
#pragma once

#include "stca_internal.h"

namespace stca {
namespace enc {

// Two 16-byte fragments per k block: (W1, W3) of a 16-row tile in the G
// phase, the two k halves of a 32-row tile elsewhere.
struct Src {
  const bf16_t *p0, *p1;
  int stride;  // elements per k block
};
struct Ring {
  bf16x8 v[4][2];
};
DEV void ring_load(Ring &r, int slot, const Src &s, int kb) {
  r.v[slot][0] = ldg8(s.p0 + kb * s.stride);
  r.v[slot][1] = ldg8(s.p1 + kb * s.stride);
}

// The NK blocks of one phase; `mma(kb, slot)` does the block's matrix work.
// Block kb + 3 is loaded while block kb is used (from the next phase once this
// one runs out; `more` = whether there is a next phase).
template <int NK, class F>
DEV void run_phase(Ring &ring, const Src &cur, const Src &nxt, bool more, F mma) {
  static_assert(NK % 4 == 0, "phase length must be a multiple of 4 blocks");
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    const int nb = kb + 3;
    if (nb < NK) ring_load(ring, nb % 4, cur, nb);
    else if (more) ring_load(ring, nb % 4, nxt, nb - NK);
    __builtin_amdgcn_sched_barrier(0);
    mma(kb, kb % 4);
    // the last block's products may overlap the epilogue that follows
    if (kb + 1 < NK) __builtin_amdgcn_sched_barrier(0);
  }
}

template <int N>
DEV void zero4(f32x4 (&a)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}
template <int N>
DEV void zero16(f32x16 (&a)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) a[i][e] = 0.f;
}

// Gather the R table rows (width D) of a tile into xs (row stride XRLD;
// zeros for padding rows and for ids outside the table), with the optional
// copy by history token.  `use_prow`: take the planner's padded-row ids when
// present.  NT threads; ends synchronised.
template <int D, int R, int XRLD, int NT>
DEV void gather_tile(const ChainArgs &a, bf16_t *xs, int *s_id, int *s_tok, int64_t row0, int total_blocks,
                     int tid, bool use_prow) {
  if (tid < R) {
    const int64_t p = row0 + tid;
    int id = -1, tok = -1;
    const int blk = (int)(p >> 5);
    if (use_prow && a.plan.prow && !a.in_dump) {
      id = a.plan.prow[p];  // planner-validated id of this padded row
    } else if (blk < total_blocks) {
      const int u = upper_index(a.plan.pblk, a.B, blk);
      const int j = (int)(p - (int64_t)a.plan.pblk[u] * 32);
      if (j < a.plan.hoff[u + 1] - a.plan.hoff[u]) {
        tok = a.plan.hoff[u] + j;
        id = a.ids[tok];
        if (id < 0 || (int64_t)id >= a.table_rows) {
          set_status(a.status, 4);
          id = -1;
        }
      }
    }
    s_id[tid] = id;
    s_tok[tid] = tok;
  }
  __syncthreads();
  const bf16_t *table = (const bf16_t *)a.table;
  constexpr int C8 = D / 8;
  constexpr int NL = R * C8 / NT;
  static_assert(NL * NT == R * C8, "whole 16-byte pieces per thread");
  // Every row load is issued before any is used (rows without a valid id
  // read table row 0 and are replaced by zeros), so that all of them are in
  // flight together rather than one round trip each.
  u32x4 v[NL];
  if (a.table_rows > 0) {
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int e = tid + k * NT, r = e / C8, c = (e % C8) * 8;
      const int id = s_id[r];
      v[k] = *reinterpret_cast<const u32x4 *>(table + (int64_t)(id >= 0 ? id : 0) * D + c);
    }
  }
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int e = tid + k * NT, r = e / C8, c = (e % C8) * 8;
    const uint32_t keep = s_id[r] >= 0 ? 0xffffffffu : 0u;  // (all ids invalid when the table is empty)
    const u32x4 val = v[k] & keep;
    *reinterpret_cast<u32x4 *>(xs + r * XRLD + c) = val;
    if (a.in_dump && s_tok[r] >= 0)
      *reinterpret_cast<u32x4 *>((bf16_t *)a.in_dump + (int64_t)s_tok[r] * D + c) = val;
  }
  __syncthreads();
}

}  // namespace enc
}  // namespace stca
