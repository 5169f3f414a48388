// attn.hip -- m-target multi-head cross attention over a user's history
// (a8), split along the history and merged in a fixed order.
//
// Per user u, target t of u and head eta ([Review] formula for alpha and o;
// [WeChat] §1.2 for the ReLU-scored form):
//   s_j = Q_t[eta] . K_j[eta]   (Q rows already carry 1/sqrt(d_h))
//   softmax: o = sum_j exp(s_j - max) V_j[eta] / sum_j exp(s_j - max)
//   relu:    o = sum_j max(0, s_j) V_j[eta],   active = #{j : s_j > 0}
//
// Request Level Batching ([Notes] §RLB): a workgroup streams a user's K/V
// blocks once and serves up to 64 of the user's targets with them.
//
// Scheduling ("stream-K"): the work is the sequence of units
//   ((user, target group, head), 128-key unit)      in that order,
// and a persistent grid (one workgroup per occupancy slot) takes equal
// contiguous ranges of it.  A workgroup carries the online-softmax state
// across the units of one (user, group, head) and writes one partial
// (running max, running sum, accumulator) when that pair ends or its range
// ends -- the single-GPU form of the per-device partial attention of [WeChat]
// §1.1, with the blocked tiling of [WeChat] §3.3.1.  Ragged histories stay
// balanced, and the partial traffic is set by the grid, not by the length.
// A second pass folds a pair's partials in workgroup order: no float atomics,
// so results do not depend on scheduling.
//
// K/V layout (written by the history chain): per 32-key block b and head h,
//   K[b][h][key 0..31][d_h]   (row of a key contiguous)
//   V[b][h][d_h][key 0..31]   (transposed: a feature's 32 keys contiguous)
// so every MFMA operand fragment is one 16-byte load.
#include <algorithm>
#include <type_traits>

#include "attn_block.h"
#include "stca_internal.h"

namespace stca {
namespace {

constexpr float kLog2e = kAttnLog2e;
constexpr float kNegBig = kAttnNegBig;
DEV float ex2(float x) { return attn_ex2(x); }

// Position of global unit `unit` in the sequence: user u, pair index within
// the user (group * H + head), first unit of the pair, units of the pair.
struct UnitPos {
  int u, pair, first, nc;
};
DEV UnitPos decode_unit(const Plan &P, int B, int HG, int unit) {
  UnitPos r;
  r.u = upper_index(P.coff, B, unit / HG);
  r.nc = P.coff[r.u + 1] - P.coff[r.u];
  const int rem = unit - P.coff[r.u] * HG;
  r.pair = rem / r.nc;
  r.first = P.coff[r.u] * HG + r.pair * r.nc;
  return r;
}

// Units per workgroup of the persistent grid.
DEV int units_per_wg(int total, int grid) { return (total + grid - 1) / grid; }

// Logical workgroup of hardware workgroup b.  Workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2); this order gives every
// XCD a contiguous share of the logical ranges, so neighbouring ranges (the
// target groups of one user and head, when a user has more than 64 targets)
// read the same K/V through one L2.  Identity when n is not a multiple of 8.
DEV int xcd_order(int b, int n) { return (n & 7) ? b : (b & 7) * (n >> 3) + (b >> 3); }

// ------------------------------------------------------------------ bf16 / MFMA
// S^T = K Q^T (16 keys x 16 targets per MFMA), online softmax in registers,
// O^T += V^T P^T (16 features x 16 targets per MFMA).  The key order inside a
// 32-key block is permuted when K is loaded so that the score tile's lane
// layout is exactly the B-operand layout P^T needs: lane l (g = l/16) holds the
// scores of keys 8g..8g+7 for target l%16.  The four waves of a workgroup take
// alternate blocks of a pair's range and merge in LDS when the pair ends.
//
// IND (unique-id dedup): K/V are not per token but per distinct history id;
// a token's row is found through a.tok2u.  K rows are read from the unique
// rows' blocked K (16 bytes per lane, as above); the V rows of a block are
// read row-major (a.vrows) and written transposed into a wave-private LDS
// tile, from which the V^T fragments are read.
//
// MASK (Cross-Mask vertical masks, [WeChat] §3.2, and the context-similarity
// score bias, [WeChat] §2.2.3): each lane also loads the mask word of key
// lane % 32 of a block (in the same pipeline stage as K/V; all ones without
// a mask), and one ballot turns the head's bit of the 32 words into the
// block's visibility word; with a bias it loads the bias of its eight keys of
// the block (two 16-byte loads from the blocked copy) and the block step adds
// them to the scores.  A head map (a.has_map) takes head h's scores from the
// Q / K columns of head a.head_map[h] ([WeChat] §3.3.1: heads sharing one
// attention map under different masks); V, the bias and the output stay
// head h's.
//
// SHARE (two to four target groups): the units are (user, head) x 128 keys,
// each wave serves one group over every block, and a block's K/V go from HBM
// through a workgroup-wide LDS ring (see below) instead of to every wave.
template <int DH, int NT, int SCORE, bool IND, bool MASK, bool SHARE>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = DH / 32;  // k-steps of the score MFMA
  constexpr int DT = DH / 16;  // feature tiles of the output
  constexpr int TG = NT * 16;  // targets per group
  constexpr int LDT = 32 + 8;  // row stride of the transposed V tile
  __shared__ float sm_m[4][TG], sm_l[4][TG];
  __shared__ int sm_c[4][TG];
  __shared__ __attribute__((aligned(16))) float sm_o[4][TG][DH + 1];
  __shared__ __attribute__((aligned(16))) bf16_t sm_vt[IND ? 4 : 1][IND ? DH * LDT : 8];

  const Plan P = a.plan;
  const int H = a.H, G = a.groups, HG = SHARE ? H : H * G;  // pairs per user: heads, or (group, head)
  const int total = P.coff[a.B] * HG;
  const int per = units_per_wg(total, gridDim.x);
  const int wgl = xcd_order(blockIdx.x, gridDim.x);  // logical workgroup
  int unit = wgl * per;
  const int unit_end = min(total, unit + per);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g16 = lane >> 4, c16 = lane & 15;
  const bf16_t *Q = (const bf16_t *)a.q;
  const bf16_t *Kb = (const bf16_t *)a.kbuf, *Vb = (const bf16_t *)a.vbuf;
  const int kr0 = attn_key_row(lane);  // permuted key row of score tile 0

  while (unit < unit_end) {
    const UnitPos pos = decode_unit(P, a.B, HG, unit);
    const int seg_end = min(unit_end, pos.first + pos.nc);
    // SHARE (at most 4 groups): wave w serves target group w over every
    // block of the segment (waves past the user's groups have no targets);
    // otherwise the four waves split the blocks of the workgroup's group
    const int u = pos.u, grp = SHARE ? w : pos.pair / H, h = SHARE ? pos.pair : pos.pair % H;
    const int hq = a.has_map ? a.head_map[h] : h;  // the head whose Q / K give the scores
    const int tbase = P.toff[u];
    const int m_u = P.toff[u + 1] - tbase;
    const int t0 = grp * TG;
    if constexpr (SHARE) {
      // Each block of the segment is read from HBM once per workgroup: the
      // 256 threads load it cooperatively (16 bytes x DH / 32 each, two
      // blocks ahead in registers), write it one block ahead into a 3-slot LDS
      // ring over sm_o (used only after the loop), and every wave reads its
      // MFMA fragments from there.  The 16-byte pieces of a row are permuted
      // by row bits so that the 16 lanes of a fragment read hit 16 distinct
      // bank groups.  Waves without targets still load and synchronise.
      const bool act = t0 < m_u;
      const int L = P.hoff[u + 1] - P.hoff[u];
      const int cl = unit - pos.first;
      const int b0 = P.pblk[u] + cl * a.nb;
      const int b1 = min(P.pblk[u + 1], P.pblk[u] + (cl + seg_end - unit) * a.nb);
      AttnState<DH, NT> st;
      attn_reset(st);
      if (act) attn_load_q(st, Q, a.d, hq, tbase, t0, m_u, lane);
      constexpr int NP = DH / 32;      // 16-byte pieces per thread per block
      constexpr int BLK = 64 * DH;     // bf16 of one head's K and V in a block
      constexpr int KP = DH / 8;       // 16-byte pieces per K row (one key)
      bf16_t *ring = reinterpret_cast<bf16_t *>(&sm_o[0][0][0]);
      static_assert(sizeof(sm_o) >= 3 * BLK * sizeof(bf16_t), "K/V ring exceeds sm_o");
      auto kswz = [](int r) {  // K row r: piece permutation
        return DH == 64 ? (((r >> 1) & 1) | (((r >> 3) & 3) << 1)) : ((r >> 3) & 3);
      };
      auto vswz = [](int r) { return (r >> 2) & 3; };  // V row r (one feature, 32 keys)
      auto gload = [&](int b, bf16x8 (&g)[NP]) {
        const bf16_t *kb = Kb + ((int64_t)b * H + hq) * 32 * DH;
        const bf16_t *vb = Vb + ((int64_t)b * H + h) * DH * 32;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          const int pc = tid + 256 * j;
          const bf16_t *src = pc < 4 * DH ? kb + pc * 8 : vb + (pc - 4 * DH) * 8;
          g[j] = ldnt8(src);
        }
      };
      auto swrite = [&](int b, const bf16x8 (&g)[NP]) {
        bf16_t *dst = ring + (b % 3) * BLK;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          const int pc = tid + 256 * j;
          int off;
          if (pc < 4 * DH) {
            const int r = pc / KP, c = pc % KP;
            off = r * DH + ((c ^ kswz(r)) << 3);
          } else {
            const int q = pc - 4 * DH, r = q >> 2, c = q & 3;
            off = 32 * DH + r * 32 + ((c ^ vswz(r)) << 3);
          }
          *reinterpret_cast<bf16x8 *>(dst + off) = g[j];
        }
      };
      bf16x8 ga[NP], gb[NP];
      if (b0 < b1) {
        gload(b0, ga);
        swrite(b0, ga);
      }
      if (b0 + 1 < b1) gload(b0 + 1, gb);
      __syncthreads();
      auto step = [&](const int b, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        if (b + 2 < b1) gload(b + 2, ga);
        if (b + 1 < b1) swrite(b + 1, gb);
        __syncthreads();  // block b + 1 written; every wave is past block b - 2 (its slot)
        if (act) {
          const bf16_t *kl = ring + (b % 3) * BLK, *vl = kl + 32 * DH;
          bf16x8 kf[2][KS], vf[DT];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const int r = kr0 + 4 * kt;
#pragma unroll
            for (int k = 0; k < KS; ++k) kf[kt][k] = ld8(kl + r * DH + (((4 * k + g16) ^ kswz(r)) << 3));
          }
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            const int r = t * 16 + c16;
            vf[t] = ld8(vl + r * 32 + ((g16 ^ vswz(r)) << 3));
          }
          attn_block<DH, NT, SCORE, FULL, true>(st, kf, vf, L - (b - P.pblk[u]) * 32, 0xffffffffu, lane);
        }
#pragma unroll
        for (int j = 0; j < NP; ++j) gb[j] = ga[j];
      };
      const int bfull = min(b1, P.pblk[u] + L / 32);
      int b = b0;
      for (; b < bfull; ++b) step(b, std::true_type{});
      for (; b < b1; ++b) step(b, std::false_type{});
      __syncthreads();  // the ring (over sm_o) is read no more
      if (act) {  // this wave's partial, through its own LDS rows
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          int cn = st.cnt[n];
          cn = isum_x16(cn);
          cn = isum_x32(cn);
          if (g16 == 0) {
            sm_m[w][n * 16 + c16] = st.mrun[n];
            sm_l[w][n * 16 + c16] = st.l[n][0];
            sm_c[w][n * 16 + c16] = cn;
          }
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm_o[w][n * 16 + c16][t * 16 + 4 * g16 + r] = st.o[t][n][r];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const int64_t pw = ((int64_t)(wgl + u * H + h) * G + grp) * a.tgs;  // slot (workgroup + pair), group
        for (int e = lane; e < TG * DH; e += 64) {
          const int tl = e / DH, dh = e % DH;
          if (t0 + tl >= m_u) continue;
          a.part_acc[(pw + tl) * DH + dh] = sm_o[w][tl][dh];
          if (dh == 0) {
            if (SCORE == 0) {
              a.part_ml[(pw + tl) * 2] = sm_m[w][tl];
              a.part_ml[(pw + tl) * 2 + 1] = sm_l[w][tl];
            } else {
              a.part_cnt[pw + tl] = sm_c[w][tl];
            }
          }
        }
      }
      __syncthreads();  // sm_o is the next segment's ring
    } else if (t0 < m_u) {
      const int L = P.hoff[u + 1] - P.hoff[u];
      const int cl = unit - (pos.first);  // first unit of this segment within the pair
      const int b0 = P.pblk[u] + cl * a.nb;
      const int b1 = min(P.pblk[u + 1], P.pblk[u] + (cl + seg_end - unit) * a.nb);

      AttnState<DH, NT> st;
      attn_reset(st);
      attn_load_q(st, Q, a.d, hq, tbase, t0, m_u, lane);
      bf16x8 kf[2][KS], vf[DT];
      // IND: the V rows of a block come as DT 16-byte chunks per lane: chunk
      // lane + 64 i = (key, part) with DH / 8 parts of 8 features per key
      constexpr int PARTS = DH / 8;
      const int64_t tok0 = (int64_t)P.hoff[u] - (int64_t)P.pblk[u] * 32;  // token of padded row 0
      auto uid_of = [&](int b, int key) -> int {  // unique row of key `key` of block b (-1: padding)
        const int j = (b - P.pblk[u]) * 32 + key;
        return j < L ? a.tok2u[tok0 + (int64_t)b * 32 + key] : -1;
      };
      // IND: the unique rows of this lane's keys in a block (K: 2, V: DT),
      // looked up one pipeline stage before the rows themselves are loaded
      struct Uids {
        int k[2], v[DT];
      };
      auto load_uids = [&](int b, Uids &U) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) U.k[kt] = uid_of(b, kr0 + 4 * kt);
#pragma unroll
        for (int i = 0; i < DT; ++i) U.v[i] = uid_of(b, (lane + 64 * i) / PARTS);
      };
      Uids U8;  // uids of the block two ahead of the one in use
      auto load_kv = [&](int b, bf16x8 (&kk)[2][KS], bf16x8 (&vv)[DT]) {
        if constexpr (IND) {
          const bf16_t *Vr = (const bf16_t *)a.vrows;
          Uids U;
          if (b < b0 + w + 8) load_uids(b, U);  // pipeline start
          else U = U8;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const int ui = U.k[kt];
#pragma unroll
            for (int k = 0; k < KS; ++k) {
              bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
              kk[kt][k] = ui < 0 ? z
                                 : ld8(Kb + ((((int64_t)(ui >> 5)) * H + hq) * 32 + (ui & 31)) * DH + k * 32 + g16 * 8);
            }
          }
#pragma unroll
          for (int i = 0; i < DT; ++i) {
            const int part = (lane + 64 * i) % PARTS;
            const int ui = U.v[i];
            bf16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
            vv[i] = ui < 0 ? z : ld8(Vr + (int64_t)ui * a.d + h * DH + part * 8);
          }
        } else {
          const bf16_t *kb = Kb + ((int64_t)b * H + hq) * 32 * DH;
          const bf16_t *vb = Vb + ((int64_t)b * H + h) * DH * 32;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int k = 0; k < KS; ++k) kk[kt][k] = ldnt8(kb + (kr0 + 4 * kt) * DH + k * 32 + g16 * 8);
#pragma unroll
          for (int t = 0; t < DT; ++t) vv[t] = ldnt8(vb + (t * 16 + c16) * 32 + g16 * 8);
        }
      };
      // IND: V row chunks -> transposed wave-private tile -> V^T fragments
      auto v_fragments = [&](const bf16x8 (&raw)[DT], bf16x8 (&out)[DT]) {
        if constexpr (IND) {
          bf16_t *vt = sm_vt[w];
#pragma unroll
          for (int i = 0; i < DT; ++i) {
            const int c = lane + 64 * i, key = c / PARTS, part = c % PARTS;
#pragma unroll
            for (int e = 0; e < 8; ++e) vt[(part * 8 + e) * LDT + key] = (bf16_t)raw[i][e];
          }
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int t = 0; t < DT; ++t) out[t] = ld8(vt + (t * 16 + c16) * LDT + g16 * 8);
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
        } else {
#pragma unroll
          for (int t = 0; t < DT; ++t) out[t] = raw[t];
        }
      };
      // MASK: the mask word of key lane % 32 of block b (0 past the history,
      // all ones without a mask)
      auto load_mask = [&](int b) -> uint32_t {
        const int key = lane & 31, j = (b - P.pblk[u]) * 32 + key;
        if (j >= L) return 0u;
        return a.key_mask ? a.key_mask[tok0 + (int64_t)b * 32 + key] : 0xffffffffu;
      };
      // MASK: this lane's eight keys' bias of block b for head h (0 without a bias)
      auto load_bias = [&](int b, f32x4 (&bb)[2]) {
        if (a.bias_blk) {
          const float *src = a.bias_blk + ((int64_t)b * H + h) * 32 + 8 * g16;
          bb[0] = ldg4(src);
          bb[1] = ldg4(src + 4);
        } else {
          bb[0] = bb[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      };
      uint32_t mk = 0, mk1 = 0;
      f32x4 bz[2], bz1[2];
      bz[0] = bz[1] = bz1[0] = bz1[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      // two blocks of this wave in flight ahead of the one being used: the
      // loads, not the arithmetic, set the pace once the block step is lean
      bf16x8 k1[2][KS], v1[DT];
      if (b0 + w < b1) {
        load_kv(b0 + w, kf, vf);
        if (MASK) {
          mk = load_mask(b0 + w);
          load_bias(b0 + w, bz);
        }
      }
      if (b0 + w + 4 < b1) {
        load_kv(b0 + w + 4, k1, v1);
        if (MASK) {
          mk1 = load_mask(b0 + w + 4);
          load_bias(b0 + w + 4, bz1);
        }
      }
      if (IND && b0 + w + 8 < b1) load_uids(b0 + w + 8, U8);
      // one block of this wave; FULL: every key of the block is visible
      auto step = [&](const int b, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        bf16x8 k2[2][KS], v2[DT];
        Uids U12;
        // uids first: waiting for them later does not wait for the rows below
        if (IND && b + 12 < b1) load_uids(b + 12, U12);
        uint32_t mk2 = 0;
        f32x4 bz2[2];
        bz2[0] = bz2[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (b + 8 < b1) {
          load_kv(b + 8, k2, v2);
          if (MASK) {
            mk2 = load_mask(b + 8);
            load_bias(b + 8, bz2);
          }
        }
        if (IND) U8 = U12;
        __builtin_amdgcn_sched_barrier(0);
        // keys of this lane: 8g + 4kt + r; valid while below the user's length
        bf16x8 vuse[DT];
        v_fragments(vf, vuse);
        uint32_t kvis = 0xffffffffu;
        if (MASK) kvis = (uint32_t)__ballot((mk >> h) & 1u);  // lanes 0..31: keys 0..31
        attn_block<DH, NT, SCORE, FULL, false, MASK>(st, kf, vuse, L - (b - P.pblk[u]) * 32, kvis, lane, bz);
        mk = mk1;
        mk1 = mk2;
        if constexpr (MASK) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            bz[i] = bz1[i];
            bz1[i] = bz2[i];
          }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            kf[kt][k] = k1[kt][k];
            k1[kt][k] = k2[kt][k];
          }
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          vf[t] = v1[t];
          v1[t] = v2[t];
        }
      };
      // the user's full blocks first, then its partial last block (and any
      // padding); with Cross-Mask masks every block takes the masked step.
      // Two loops over one pipeline: a branch per block would keep both
      // bodies' registers live at once.
      const int bfull = MASK ? b0 : min(b1, P.pblk[u] + L / 32);
      int b = b0 + w;
      for (; b < bfull; b += 4) step(b, std::true_type{});
      for (; b < b1; b += 4) step(b, std::false_type{});

      // ---- merge the four waves in LDS, write this segment's partial
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float l = st.l[n][0];  // already the whole block range's sum
        int cn = st.cnt[n];
        cn = isum_x16(cn);
        cn = isum_x32(cn);
        if (g16 == 0) {
          sm_m[w][n * 16 + c16] = st.mrun[n];
          sm_l[w][n * 16 + c16] = l;
          sm_c[w][n * 16 + c16] = cn;
        }
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) sm_o[w][n * 16 + c16][t * 16 + 4 * g16 + r] = st.o[t][n][r];
      }
      __syncthreads();
      const int64_t pbase = (int64_t)(wgl + u * HG + pos.pair) * a.tgs;  // slot: workgroup + pair
      for (int e = tid; e < TG * DH; e += 256) {
        const int tl = e / DH, dh = e % DH;
        if (t0 + tl >= m_u) continue;
        if (SCORE == 0) {
          const float M = fmaxf(fmaxf(sm_m[0][tl], sm_m[1][tl]), fmaxf(sm_m[2][tl], sm_m[3][tl]));
          float acc = 0.f, l = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float f = ex2((sm_m[q][tl] - M) * kLog2e);
            acc += sm_o[q][tl][dh] * f;
            l += sm_l[q][tl] * f;
          }
          a.part_acc[(pbase + tl) * DH + dh] = acc;
          if (dh == 0) {
            a.part_ml[(pbase + tl) * 2] = M;
            a.part_ml[(pbase + tl) * 2 + 1] = l;
          }
        } else {
          a.part_acc[(pbase + tl) * DH + dh] =
              sm_o[0][tl][dh] + sm_o[1][tl][dh] + sm_o[2][tl][dh] + sm_o[3][tl][dh];
          if (dh == 0) a.part_cnt[pbase + tl] = sm_c[0][tl] + sm_c[1][tl] + sm_c[2][tl] + sm_c[3][tl];
        }
      }
      __syncthreads();  // LDS reused by the next segment
    }
    unit = seg_end;
  }
}

// ------------------------------------------------------------------ fp32
// One wave per workgroup, lane = target, keys streamed one at a time over the
// same unit ranges.  The fp32 configuration is the precision reference of the
// library (small shapes), so scores and sums are accumulated in fp64: the
// ReLU-scored sum is unnormalised and cancels heavily, and fp32 accumulation
// alone would cost most of a 1e-5 error budget.
template <int DH, int SCORE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const Plan P = a.plan;
  const int H = a.H, G = a.groups, HG = H * G;
  const int total = P.coff[a.B] * HG;
  const int per = units_per_wg(total, gridDim.x);
  int unit = blockIdx.x * per;
  const int unit_end = min(total, unit + per);
  const float *Q = (const float *)a.q;
  const float *Kb = (const float *)a.kbuf, *Vb = (const float *)a.vbuf;
  while (unit < unit_end) {
    const UnitPos pos = decode_unit(P, a.B, HG, unit);
    const int seg_end = min(unit_end, pos.first + pos.nc);
    const int u = pos.u, grp = pos.pair / H, h = pos.pair % H;
    const int tbase = P.toff[u];
    const int m_u = P.toff[u + 1] - tbase;
    const int tl = grp * 64 + threadIdx.x;
    if (grp * 64 < m_u) {
      const bool act = tl < m_u;
      const int L = P.hoff[u + 1] - P.hoff[u];
      const int cl = unit - pos.first;
      const int b0 = P.pblk[u] + cl * a.nb;
      const int b1 = min(P.pblk[u + 1], P.pblk[u] + (cl + seg_end - unit) * a.nb);
      double q[DH], acc[DH];
#pragma unroll
      for (int i = 0; i < DH; ++i) {
        q[i] = act ? (double)Q[(int64_t)(tbase + tl) * a.d + h * DH + i] : 0.0;
        acc[i] = 0.0;
      }
      double mrun = -1.0e300, lrun = 0.0;
      int cnt = 0;
      for (int b = b0; b < b1; ++b) {
        const float *kb = Kb + ((int64_t)b * H + h) * 32 * DH;
        const float *vb = Vb + ((int64_t)b * H + h) * DH * 32;
        const int nvalid = min(32, L - (b - P.pblk[u]) * 32);
        for (int j = 0; j < nvalid; ++j) {
          double sc = 0.0;
#pragma unroll
          for (int i = 0; i < DH; ++i) sc = fma(q[i], (double)kb[j * DH + i], sc);
          double p;
          if (SCORE == 0) {
            const double mnew = fmax(mrun, sc);
            const double corr = exp(mrun - mnew);
            p = exp(sc - mnew);
            lrun = lrun * corr + p;
#pragma unroll
            for (int i = 0; i < DH; ++i) acc[i] *= corr;
            mrun = mnew;
          } else {
            p = sc > 0.0 ? sc : 0.0;
            cnt += sc > 0.0 ? 1 : 0;
          }
#pragma unroll
          for (int i = 0; i < DH; ++i) acc[i] = fma(p, (double)vb[i * 32 + j], acc[i]);
        }
      }
      if (act) {
        const int64_t pi = (int64_t)(blockIdx.x + u * HG + pos.pair) * a.tgs + (tl - grp * 64);
        // softmax partials are stored normalised by their own running sum
        // (a convex combination, no cancellation), the sum separately
        if (SCORE == 0) {
          const double inv = lrun > 0.0 ? 1.0 / lrun : 0.0;
#pragma unroll
          for (int i = 0; i < DH; ++i) a.part_acc[pi * DH + i] = (float)(acc[i] * inv);
          a.part_ml[pi * 2] = (float)mrun;
          a.part_ml[pi * 2 + 1] = (float)lrun;
        } else {
#pragma unroll
          for (int i = 0; i < DH; ++i) a.part_acc[pi * DH + i] = (float)acc[i];
          a.part_cnt[pi] = cnt;
        }
      }
    }
    unit = seg_end;
  }
}

// ------------------------------------------------------------------ merge
// One thread per (target, 4 consecutive features of one head): fold the
// partials of the target's (user, group, head) in workgroup order.
//   softmax: attn = sum_w acc_w e^{m_w - M} / sum_w l_w e^{m_w - M};  ReLU: sums.
// Streaming partials: a workgroup's segment of a pair is stored at the
// segment's first unit.  Fused partials (one per workgroup and user, all
// heads): slot workgroup + user, units = the user's key tiles.
template <int SCORE>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int d = a.d, DH = a.dh, H = a.H, G = a.groups, HG = H * G;
  const int d4 = d >> 2;  // d = H d_h, d_h 32 or 64
  const int64_t e4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n4 = a.n_tgt * d4;
  if (e4 >= n4) return;
  int t, f;
  if (n4 <= 0x7fffffff) {
    const unsigned q = (unsigned)e4 / (unsigned)d4;
    t = (int)q;
    f = ((int)e4 - (int)q * d4) * 4;
  } else {
    t = (int)(e4 / d4);
    f = (int)(e4 % d4) * 4;
  }
  const int hs = DH == 64 ? 6 : 5;
  const int h = f >> hs, dh = f & (DH - 1);
  const Plan P = a.plan;
  f32x4 out = {0.f, 0.f, 0.f, 0.f};
  float lse_v = 0.f;
  int cnt = 0;
  if (t < P.toff[a.B] && a.grid > 0) {
    const int u = upper_index(P.toff, a.B, t);
    const int tl = t - P.toff[u];
    const int grp = G > 1 ? tl / 64 : 0;
    const int tg = tl - grp * 64;
    int first, nu, per;
    if (a.fused) {
      const int tb = a.tile_blocks;
      first = P.pblk[u] / tb;
      nu = (P.pblk[u + 1] - P.pblk[u]) / tb;
      per = units_per_wg(P.pblk[a.B] / tb, a.grid);
    } else {
      nu = P.coff[u + 1] - P.coff[u];
      const int hg = a.share ? H : HG;  // pairs per user of the partial kernel's units
      first = P.coff[u] * hg + (a.share ? h : grp * H + h) * nu;
      per = units_per_wg(P.coff[a.B] * hg, a.grid);
    }
    // slot of the segment of workgroup wg: wg + the pair's global index
    const int64_t gp = a.share ? (int64_t)u * H + h : (int64_t)u * HG + grp * H + h;
    auto pidx = [&](int wg) -> int64_t {
      if (a.fused) return partial_index(wg + u, H, h, a.tgs, tg);
      return (a.share ? (wg + gp) * G + grp : wg + gp) * a.tgs + tg;
    };
    if (nu > 0) {
      const int w0 = first / per, w1 = (first + nu - 1) / per;
      if (SCORE == 0 && a.dtype) {
        float M = kNegBig;
        for (int wg = w0; wg <= w1; ++wg) M = fmaxf(M, a.part_ml[pidx(wg) * 2]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float l = 0.f;
        for (int wg = w0; wg <= w1; ++wg) {
          const int64_t pi = pidx(wg);
          const float fct = ex2((a.part_ml[pi * 2] - M) * kLog2e);
          const f32x4 pa = ldg4(a.part_acc + pi * DH + dh);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] += pa[c] * fct;
          l += a.part_ml[pi * 2 + 1] * fct;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) out[c] = l > 0.f ? acc[c] / l : 0.f;
        lse_v = l > 0.f ? M + logf(l) : 0.f;
      } else if (SCORE == 0) {  // fp32 path: normalised partials, fp64 fold
        double M = -1.0e300;
        for (int wg = w0; wg <= w1; ++wg) M = fmax(M, (double)a.part_ml[pidx(wg) * 2]);
        double acc[4] = {0.0, 0.0, 0.0, 0.0}, l = 0.0;
        for (int wg = w0; wg <= w1; ++wg) {
          const int64_t pi = pidx(wg);
          const double wgt = (double)a.part_ml[pi * 2 + 1] * exp((double)a.part_ml[pi * 2] - M);
          const f32x4 pa = ldg4(a.part_acc + pi * DH + dh);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] += (double)pa[c] * wgt;
          l += wgt;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) out[c] = l > 0.0 ? (float)(acc[c] / l) : 0.f;
        lse_v = l > 0.0 ? (float)(M + log(l)) : 0.f;
      } else {
        double acc[4] = {0.0, 0.0, 0.0, 0.0};
        for (int wg = w0; wg <= w1; ++wg) {
          const int64_t pi = pidx(wg);
          const f32x4 pa = ldg4(a.part_acc + pi * DH + dh);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] += (double)pa[c];
          if (dh == 0) cnt += a.part_cnt[pi];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) out[c] = (float)acc[c];
      }
    }
  }
  if (SCORE == 0 && a.lse && dh == 0) a.lse[(int64_t)t * H + h] = lse_v;
  const int64_t e = e4 * 4;
  *reinterpret_cast<f32x4 *>(a.attn + e) = out;
  if (a.attn_lo) {
    if (a.dtype) {
      const uint32_t lo = pack_bf2(out[0], out[1]), hi = pack_bf2(out[2], out[3]);
      *reinterpret_cast<uint2 *>((bf16_t *)a.attn_lo + e) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<f32x4 *>((float *)a.attn_lo + e) = out;
    }
  }
  if (SCORE == 1 && a.active && dh == 0) a.active[(int64_t)t * H + h] = cnt;
}

// ------------------------------------------------------------------ relayout
template <typename T>
__global__ void relayout_kernel(const T *k, const T *v, T *kb, T *vb, Plan P, int B, int d, int H,
                                bool to_blocked) {
  const int b = blockIdx.x;
  if (b >= P.pblk[B]) return;
  const int DH = d / H;
  const int u = upper_index(P.pblk, B, b);
  const int L = P.hoff[u + 1] - P.hoff[u];
  const int j0 = (b - P.pblk[u]) * 32;
  for (int e = threadIdx.x; e < 32 * d; e += blockDim.x) {
    const int key = e / d, f = e % d;
    const int h = f / DH, dh = f % DH;
    const bool valid = j0 + key < L;
    const int64_t row = (int64_t)P.hoff[u] + j0 + key;
    const int64_t ki = (((int64_t)b * H + h) * 32 + key) * DH + dh;
    const int64_t vi = (((int64_t)b * H + h) * DH + dh) * 32 + key;
    if (to_blocked) {
      kb[ki] = valid ? k[row * d + f] : (T)0;
      vb[vi] = valid ? v[row * d + f] : (T)0;
    } else if (valid) {
      ((T *)k)[row * d + f] = kb[ki];
      ((T *)v)[row * d + f] = vb[vi];
    }
  }
}

// One workgroup per padded block: out[(b * H + h) * 32 + key] = the caller's
// bias[token, h] of the block's key, 0 on padding rows.
__global__ __launch_bounds__(256) void bias_relayout_kernel(const float *bias, float *out, Plan P, int B, int H) {
  const int b = blockIdx.x;
  if (b >= P.pblk[B]) return;
  const int u = upper_index(P.pblk, B, b);
  const int L = P.hoff[u + 1] - P.hoff[u];
  const int j0 = (b - P.pblk[u]) * 32;
  for (int e = threadIdx.x; e < 32 * H; e += blockDim.x) {
    const int h = e >> 5, key = e & 31;
    const int64_t row = (int64_t)P.hoff[u] + j0 + key;
    out[((int64_t)b * H + h) * 32 + key] = j0 + key < L ? bias[row * H + h] : 0.f;
  }
}

template <typename K>
int persistent_grid(K kernel, int threads, int64_t units) {
  int dev = 0, cus = 256, per_cu = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return (int)std::max<int64_t>(1, std::min<int64_t>({units, (int64_t)cus * per_cu, (int64_t)kAttnMaxGrid}));
}

template <int DH, int SCORE, bool IND, bool MASK>
hipError_t launch_bf16(AttnArgs &a, hipStream_t s) {
  const int nt = a.groups > 1 ? 4 : (a.max_tgt + 15) / 16;
  const dim3 block(256);
#define GO(NT, SH)                                                                     \
  {                                                                                    \
    auto k = attn_bf16_kernel<DH, NT, SCORE, IND, MASK, SH>;                           \
    a.grid = persistent_grid(k, 256, a.max_units);                                     \
    hipLaunchKernelGGL(k, dim3(a.grid), block, 0, s, a);                               \
  }
  if constexpr (!IND && !MASK) {
    if (a.groups > 1 && a.groups <= 4) {  // units are (user, head) x 128 keys; each wave one group
      a.share = 1;
      auto k = attn_bf16_kernel<DH, 4, SCORE, IND, MASK, true>;
      a.grid = persistent_grid(k, 256, a.max_units / a.groups);
      hipLaunchKernelGGL(k, dim3(a.grid), block, 0, s, a);
      return hipGetLastError();
    }
  }
  if (nt >= 4) GO(4, false) else if (nt == 3) GO(3, false) else if (nt == 2) GO(2, false) else GO(1, false)
#undef GO
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_partial(AttnArgs &a, hipStream_t s) {
  a.grid = 0;
  a.share = 0;
  if (a.max_units <= 0 || a.n_tgt <= 0) return hipSuccess;
  if (a.dtype == 1) {
#define SEL(IND, MASK)                                                                                      \
  {                                                                                                         \
    if (a.dh == 32) return a.score ? launch_bf16<32, 1, IND, MASK>(a, s) : launch_bf16<32, 0, IND, MASK>(a, s); \
    if (a.dh == 64) return a.score ? launch_bf16<64, 1, IND, MASK>(a, s) : launch_bf16<64, 0, IND, MASK>(a, s); \
    return hipErrorInvalidValue;                                                                            \
  }
    const bool mod = a.key_mask || a.bias_blk;  // masks and / or a score bias
    if (a.tok2u) {
      if (mod) SEL(true, true) else SEL(true, false)
    }
    if (mod) SEL(false, true) else SEL(false, false)
#undef SEL
  }
  if (a.key_mask || a.has_map || a.bias_blk) return hipErrorInvalidValue;  // fp32: no Cross-Mask, no bias
#define GO(DH, SC)                                                   \
  {                                                                  \
    auto k = attn_f32_kernel<DH, SC>;                                \
    a.grid = persistent_grid(k, 64, a.max_units);                    \
    hipLaunchKernelGGL(k, dim3(a.grid), dim3(64), 0, s, a);          \
  }
  if (a.dh == 32) {
    if (a.score) GO(32, 1) else GO(32, 0)
  } else if (a.dh == 64) {
    if (a.score) GO(64, 1) else GO(64, 0)
  } else {
    return hipErrorInvalidValue;
  }
#undef GO
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs &a, hipStream_t s) {
  if (a.n_tgt <= 0) return hipSuccess;
  if ((a.dh != 32 && a.dh != 64) || a.d % 4) return hipErrorInvalidValue;
  const int64_t n = a.n_tgt * (a.d / 4);  // threads: 4 features each
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (a.score) hipLaunchKernelGGL(merge_kernel<1>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<0>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bias_relayout(const float *bias, float *out, const Plan &plan, int B, int64_t max_blocks, int H,
                                hipStream_t s) {
  if (max_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(bias_relayout_kernel, dim3((unsigned)max_blocks), dim3(256), 0, s, bias, out, plan, B, H);
  return hipGetLastError();
}

hipError_t launch_attention(AttnArgs &a, hipStream_t s) {
  hipError_t e = launch_attn_partial(a, s);
  if (e != hipSuccess) return e;
  return launch_attn_merge(a, s);
}

hipError_t launch_kv_relayout(int dtype, const void *k, const void *v, void *kbuf, void *vbuf,
                              Plan plan, int B, int64_t max_blocks, int d, int H, bool to_blocked,
                              hipStream_t s) {
  if (max_blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)max_blocks), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(relayout_kernel<bf16_t>, grid, block, 0, s, (const bf16_t *)k, (const bf16_t *)v,
                       (bf16_t *)kbuf, (bf16_t *)vbuf, plan, B, d, H, to_blocked);
  else
    hipLaunchKernelGGL(relayout_kernel<float>, grid, block, 0, s, (const float *)k, (const float *)v,
                       (float *)kbuf, (float *)vbuf, plan, B, d, H, to_blocked);
  return hipGetLastError();
}

}  // namespace stca
