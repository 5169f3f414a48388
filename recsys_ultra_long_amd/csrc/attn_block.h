// attn_block.h -- one 32-key block of the m-target cross attention for one
// head, on 16x16x32 bf16 MFMA (shared by the streaming kernel in attn.hip and
// the fused kernel in chain_bf16.hip).
//
// Per target t and key j of the block ([Review] formula for alpha and o;
// [WeChat] §1.2 for the ReLU form):  s = Q_t . K_j  (Q already carries
// 1/sqrt(d_h));  softmax: online update of (running max, running sum, sum of
// p V);  relu: w = max(0, s), sum of w V, count of s > 0.
//
// Lane layout: lane l = 16 g + c.  S^T = K Q^T is computed with the key order
// inside the block permuted at load time (lane c loads key row
// 8 (c / 4) + (c % 4) + 4 kt for score tile kt), so that the score tile's
// registers are exactly the B operand P^T of O^T += V^T P^T: lane l holds the
// scores of keys 8g .. 8g+7 for target c (+16 n for target tile n).
#pragma once

#include "common.h"

namespace stca {

constexpr float kAttnLog2e = 1.4426950408889634f;
constexpr float kAttnNegBig = -1.0e30f;

DEV float attn_ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DH, int NT>
struct AttnState {
  static constexpr int KS = DH / 32;  // k-steps of the score MFMA
  static constexpr int DT = DH / 16;  // feature tiles of the output
  bf16x8 qf[NT][KS];
  float mrun[NT];  // running max (natural units) the weights are taken against
  f32x4 l[NT];     // softmax: running sum of the (rounded) weights, in every row
  int cnt[NT];     // relu: keys with a positive score (this lane's share)
  f32x4 o[DT][NT];
};

// key row this lane loads for score tile 0 (add 4 for tile 1)
DEV int attn_key_row(int lane) {
  const int c = lane & 15;
  return 8 * (c >> 2) + (c & 3);
}

template <int DH, int NT>
DEV void attn_reset(AttnState<DH, NT> &s) {
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    s.mrun[n] = kAttnNegBig;
    s.l[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    s.cnt[n] = 0;
#pragma unroll
    for (int t = 0; t < AttnState<DH, NT>::DT; ++t) s.o[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Q fragments (B operand of the score MFMA) of targets t0 .. t0 + 16 NT of one
// user; rows beyond m_u are zero.
template <int DH, int NT>
DEV void attn_load_q(AttnState<DH, NT> &s, const bf16_t *Q, int d, int h, int64_t tbase, int t0,
                     int m_u, int lane) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int tl = t0 + n * 16 + c;
#pragma unroll
    for (int k = 0; k < AttnState<DH, NT>::KS; ++k) {
      if (tl < m_u) {
        s.qf[n][k] = ld8(Q + (tbase + tl) * d + h * DH + k * 32 + g * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) s.qf[n][k][e] = 0;
      }
    }
  }
}

// Softmax weights are taken against a running max that is only raised when
// some target's block max exceeds it by more than kAttnLazy (natural units,
// a factor 2^8): weights then stay below 256, well inside bf16 and fp32, and
// o and l are always scaled against the same max, so the normalised result
// is unchanged -- only the rescaling work is skipped for most blocks.
constexpr float kAttnLazy = 8.0f / kAttnLog2e;

// One block: kf = K fragments (score tiles 0/1, k-steps), vf = V^T fragments
// (feature tiles); keys at or beyond nvalid (block-local) are masked, and so
// is every key j whose bit j of kvis is clear (a Cross-Mask vertical mask,
// [WeChat] §3.2: the head attends only to the rows its feature-domain
// condition selects).  Masked keys take weight 0 and no part in the max.
// FULL: the caller has checked that every key is visible (the code for
// masking is then left out; left in, the compiler turns it into selects on
// every score of every block).  SWAP: the block max crosses lanes with lane
// swaps (VALU) instead of LDS permutes, for launches bound by the block
// step's latency rather than by memory.  BIAS: bias[kt][r] is added to the
// score of key 8g + 4kt + r (this lane's keys) for every target before the
// softmax or the ReLU (the context-similarity bias of [WeChat] §2.2.3).
template <int DH, int NT, int SCORE, bool FULL = false, bool SWAP = false, bool BIAS = false>
DEV void attn_block(AttnState<DH, NT> &s, const bf16x8 (&kf)[2][DH / 32], const bf16x8 (&vf)[DH / 16],
                    int nvalid, uint32_t kvis, int lane, const f32x4 *bias = nullptr) {
  constexpr int KS = DH / 32, DT = DH / 16;
  const int g = lane >> 4;
  // uniform: only a user's last block is partial, and masks are per block
  const bool full = FULL || (nvalid >= 32 && kvis == 0xffffffffu);
  auto visible = [&](int j) { return j < nvalid && ((kvis >> j) & 1u); };
  f32x4 st[2][NT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      st[kt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) st[kt][n] = mfma16(kf[kt][k], s.qf[n][k], st[kt][n]);
      if constexpr (BIAS) st[kt][n] += bias[kt];
    }
  bf16x8 pk[NT];
  if (SCORE == 0) {
    if (!full) {  // masked keys score -inf
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!visible(8 * g + 4 * kt + r)) st[kt][n][r] = kAttnNegBig;
    }
    float mx[NT];
    bool raise = false;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float m = fmaxf(fmaxf(fmaxf(st[0][n][0], st[0][n][1]), fmaxf(st[0][n][2], st[0][n][3])),
                      fmaxf(fmaxf(st[1][n][0], st[1][n][1]), fmaxf(st[1][n][2], st[1][n][3])));
      if constexpr (SWAP) {
        m = max_x32(max_x16(m));
      } else {
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
      }
      mx[n] = m;
      raise |= m > s.mrun[n] + kAttnLazy;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float mnew = fmaxf(s.mrun[n], mx[n]);
        const float corr = attn_ex2((s.mrun[n] - mnew) * kAttnLog2e);
        s.mrun[n] = mnew;
        s.l[n] *= corr;
#pragma unroll
        for (int t = 0; t < DT; ++t) s.o[t][n] *= corr;
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float mb = s.mrun[n] * kAttnLog2e;
      float pv[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[4 * kt + r] = attn_ex2(fmaf(st[kt][n][r], kAttnLog2e, -mb));
      if (!full) {  // exactly 0, also while no visible key has raised the max yet
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!visible(8 * g + 4 * kt + r)) pv[4 * kt + r] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t pr = pack_bf2(pv[e], pv[e + 1]);
        pk[n][e] = (short)(pr & 0xffff);
        pk[n][e + 1] = (short)(pr >> 16);
      }
    }
  } else {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float pv[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = st[kt][n][r];
          const bool on = (full || visible(8 * g + 4 * kt + r)) && sc > 0.f;
          s.cnt[n] += on ? 1 : 0;
          pv[4 * kt + r] = on ? sc : 0.f;
        }
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t pr = pack_bf2(pv[e], pv[e + 1]);
        pk[n][e] = (short)(pr & 0xffff);
        pk[n][e + 1] = (short)(pr >> 16);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) s.o[t][n] = mfma16(vf[t], pk[n], s.o[t][n]);
  if (SCORE == 0) {
    // l += sum of this block's weights as rounded for the PV product: an
    // all-ones A operand makes every output row that column sum
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (short)0x3f80;  // bf16 1.0
#pragma unroll
    for (int n = 0; n < NT; ++n) s.l[n] = mfma16(ones, pk[n], s.l[n]);
  }
}

// Partial-slot indexing shared by the attention kernels and the merge: the
// partial of pair P written by workgroup wg lives in slot wg + P (pairs are
// visited in order and each workgroup's range is contiguous, so (wg, P)
// pairs map to distinct slots in [0, grid + pairs)).  A slot holds `heads`
// heads (1 for the streaming kernel, whose pairs include the head; H for the
// fused kernel) of `tgs` targets.
DEV int64_t partial_index(int slot, int heads, int hh, int tgs, int tl) {
  return ((int64_t)slot * heads + hh) * tgs + tl;
}

}  // namespace stca
