// attn_bwd.hip -- backward of the m-target cross attention, one user's keys
// against all of that user's targets per head ([Review] "核心公式": the
// single-layer attention alpha = softmax(q W_Q (X~ W_K)^T / sqrt(d_h)),
// o = alpha X~ W_V; [WeChat] §1.2 for the ReLU-scored form), with the
// softmax weights recomputed from the forward's log-sum-exp:
//
//   s = Q K^T (Q already carries 1/sqrt(d_h)),  p = exp(s - lse)  | max(0, s)
//   dP = dA V^T,  dS = p * (dP - D) with D = rowsum(dA * a)  | dP * [s > 0]
//   dV = P^T dA,  dK = dS^T Q,  dQ = dS K.
//
// Work split: a workgroup takes one split-L chunk of one user and one head;
// its four waves take 32-key blocks in turn.  Everything a block needs is on
// the 32x32x16 bf16 MFMA:
//   S^T, dP^T [keys x targets]:  A = K / V rows (16-byte runs of d_h),
//                                 B = Q / dA rows;
//   dQ [targets x d_h] += dS K:  A = dS straight from the S^T accumulator
//                                 (lane = target; its 16 key rows form two
//                                 16-deep k-steps in the accumulator's row
//                                 order), B = K^T from a wave-private LDS copy
//                                 read in that same key order;
//   dK, dV [keys x d_h]:         A = dS^T / P^T re-read from wave-private LDS
//                                 as [key][target], B = Q^T / dA^T (LDS).
// dQ is accumulated per wave over its blocks and written as a partial; a
// second kernel folds a target's partials in (chunk, wave) order.
#include "grad_internal.h"

namespace stca {
namespace {

constexpr int kMaxTgt = 64;
constexpr int LT = kMaxTgt + 8;  // row stride of [.][target] LDS tiles
constexpr int LK = 32 + 8;       // row stride of [.][key] LDS tiles
// p = e^(s - lse) on the hardware base-2 exponential (a few ulp in fp32;
// p and dS feed bf16 products)
constexpr float kLog2e = 1.4426950408889634f;

__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(AttnBwdArgs a) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (target, head)
  if (e >= a.n_tgt * a.H) return;
  const int64_t t = e / a.H;
  const int h = (int)(e % a.H);
  const int64_t base = t * a.d + (int64_t)h * a.dh;
  // D = sum_j p_j dP_j = dA . a, taken with the bf16 dA the dP product
  // uses: a component shared by every V row (the LN bias mapped through W_V)
  // then cancels exactly in dP_j - D instead of leaving dA's rounding behind
  float s = 0.f;
  for (int n = 0; n < a.dh; ++n) {
    const bf16_t g = f2bf(a.da[base + n]);
    s += bf2f(g) * a.a[base + n];
    a.da_lo[base + n] = g;
  }
  a.dsum[e] = s;
}

DEV void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int DH, int SCORE, bool DD>
__global__ __launch_bounds__(256) void attn_bwd_kernel(AttnBwdArgs a) {
  constexpr int KS = DH / 16;  // 16-deep k-steps over d_h
  constexpr int NN = DH / 32;  // 32-wide output tiles over d_h
  __shared__ __attribute__((aligned(16))) bf16_t sQ[kMaxTgt * (DH + 8)];
  __shared__ __attribute__((aligned(16))) bf16_t sdA[kMaxTgt * (DH + 8)];
  __shared__ __attribute__((aligned(16))) bf16_t sQT[DH * LT];
  __shared__ __attribute__((aligned(16))) bf16_t sdAT[DH * LT];
  __shared__ __attribute__((aligned(16))) bf16_t sKT[4][DH * LK];
  __shared__ __attribute__((aligned(16))) bf16_t sP[4][32 * LT];
  __shared__ __attribute__((aligned(16))) bf16_t sdS[4][32 * LT];
  __shared__ float slse[kMaxTgt], sD[kMaxTgt];

  const Plan P = a.plan;
  const int c = blockIdx.x, eta = blockIdx.y;
  if (c >= P.coff[a.B]) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int u = upper_index(P.coff, a.B, c);
  const int ci = c - P.coff[u];
  const int64_t h0 = P.hoff[u];
  const int L = P.hoff[u + 1] - P.hoff[u];
  const int k_begin = ci * a.nb * 32;
  const int k_end = min(L, k_begin + a.nb * 32);
  const int64_t t0 = P.toff[u];
  const int m = min(P.toff[u + 1] - P.toff[u], kMaxTgt);
  const int NT = (m + 31) / 32;
  const int d = a.d;
  const int64_t col0 = (int64_t)eta * DH;

  // the user's Q and dA rows of this head, in 16-byte pieces (all loads in
  // flight together; rows past m read target 0 and are zeroed)
  constexpr int PER = DH / 8;
  static_assert((kMaxTgt * PER) % 256 == 0, "whole pieces per thread");
#pragma unroll
  for (int e0 = 0; e0 < kMaxTgt * PER; e0 += 256) {
    const int e = e0 + tid, t = e / PER, n0 = (e % PER) * 8;
    u32x4 q = {0u, 0u, 0u, 0u}, gq = q;
    if (m > 0) {  // (uniform)
      const int64_t row = (t0 + (t < m ? t : 0)) * d + col0 + n0;
      q = *reinterpret_cast<const u32x4 *>(a.q + row);
      gq = *reinterpret_cast<const u32x4 *>(a.da_lo + row);
      const uint32_t keep = t < m ? 0xffffffffu : 0u;
      q &= keep;
      gq &= keep;
    }
    *reinterpret_cast<u32x4 *>(sQ + t * (DH + 8) + n0) = q;
    *reinterpret_cast<u32x4 *>(sdA + t * (DH + 8) + n0) = gq;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sQT[(n0 + k) * LT + t] = (bf16_t)(q[k >> 1] >> (16 * (k & 1)));
      sdAT[(n0 + k) * LT + t] = (bf16_t)(gq[k >> 1] >> (16 * (k & 1)));
    }
  }
  if (tid < kMaxTgt) {
    slse[tid] = (SCORE == 0 && tid < m) ? a.lse[(t0 + tid) * a.H + eta] : 0.f;
    sD[tid] = tid < m ? a.dsum[(t0 + tid) * a.H + eta] : 0.f;
  }
  __syncthreads();

  f32x16 dq[2][NN];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[nt][nn][r] = 0.f;

  bf16_t *kt_w = sKT[w], *p_w = sP[w], *ds_w = sdS[w];
  const bf16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  // The K / V rows of a wave's next block are loaded while the current one
  // is worked on (and before its dK | dV stores, which share the in-order
  // memory counter); with dedup the row ids are fetched one block further
  // ahead.  Loads are unconditional: keys past the chunk read its last key,
  // and their rows are zeroed where they are used.
  auto row_id = [&](int kb) -> int {  // DD (dedup): the key's unique row; else the key
    const int key = min(kb + l32, k_end - 1);
    return DD ? a.tok2u[h0 + key] : key;
  };
  auto load_kv = [&](int id, bf16x8(&kf)[KS], bf16x8(&vf)[KS]) {
    const bf16_t *kr, *vr;
    if (DD) {  // blocked K, row-major V of the unique rows
      kr = a.k + ((((int64_t)(id >> 5)) * a.H + eta) * 32 + (id & 31)) * DH;
      vr = a.v + (int64_t)id * d + col0;
    } else {
      kr = a.k + (h0 + id) * d + col0;
      vr = a.v + (h0 + id) * d + col0;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = ld8(kr + 16 * s + 8 * g);
      vf[s] = ld8(vr + 16 * s + 8 * g);
    }
  };
  // (the block loop runs per wave: its counter is kept wave-uniform, so that
  // the loop is not a divergent one; it is unrolled by two, the prefetched
  // rows alternating between two register sets, so that none is copied and
  // each is waited for only where it is used)
  const int kb0 = k_begin + 32 * __builtin_amdgcn_readfirstlane(w);
  bf16x8 kr0[KS], vr0[KS], kr1[KS], vr1[KS];  // the two register sets
  int idn = 0;  // the row id of the block after the next
  if (kb0 < k_end) {
    load_kv(row_id(kb0), kr0, vr0);
    idn = row_id(kb0 + 128);
  }
  auto block = [&](const int kb, const bf16x8(&kc)[KS], const bf16x8(&vc)[KS], bf16x8(&kn)[KS],
                   bf16x8(&vn)[KS]) {
    const int key = kb + l32;
    const bool kval = key < k_end;
    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = kval ? kc[s] : zero8;
      vf[s] = kval ? vc[s] : zero8;
    }
    // the next block (past the chunk's end: its last key again, unused)
    load_kv(idn, kn, vn);
    idn = row_id(kb + 256);
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) kt_w[(16 * s + 8 * g + e) * LK + l32] = (bf16_t)kf[s][e];
    wave_sync();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (nt >= NT) break;
      f32x16 st, dpt;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[r] = 0.f;
        dpt[r] = 0.f;
      }
      const int t = nt * 32 + l32;  // this lane's target (accumulator column)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        st = mfma32(kf[s], ld8(sQ + t * (DH + 8) + 16 * s + 8 * g), st);
        dpt = mfma32(vf[s], ld8(sdA + t * (DH + 8) + 16 * s + 8 * g), dpt);
      }
      const bool tval = t < m;
      const float lse = slse[t], D = sD[t];
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = c32_row(lane, r);  // key row within the block
        const bool ok = tval && kb + kr < k_end;
        float p, dsv;
        if (SCORE == 0) {
          p = ok ? __builtin_amdgcn_exp2f((st[r] - lse) * kLog2e) : 0.f;
          dsv = p * (dpt[r] - D);
        } else {
          const bool pos = ok && st[r] > 0.f;
          p = pos ? st[r] : 0.f;
          dsv = pos ? dpt[r] : 0.f;
        }
        ds[r] = dsv;
        p_w[kr * LT + t] = f2bf(p);
        ds_w[kr * LT + t] = f2bf(dsv);
      }
      // dQ[targets of nt] += dS K over this block's 32 keys
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 af;
#pragma unroll
        for (int e = 0; e < 8; ++e) af[e] = (short)f2bf(ds[8 * ks + e]);
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
          const bf16_t *row = kt_w + (nn * 32 + l32) * LK + 16 * ks + 4 * g;
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(row);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(row + 8);
          u32x4 bw = {lo[0], lo[1], hi[0], hi[1]};
          dq[nt][nn] = mfma32(af, __builtin_bit_cast(bf16x8, bw), dq[nt][nn]);
        }
      }
    }
    wave_sync();
    // dK^T = Q^T dS, dV^T = dA^T P over this user's targets (16 per k-step):
    // features as accumulator rows, keys as columns, so that each lane ends
    // up with 16 consecutive features of one key for 16-byte stores
    f32x16 dk[NN], dv[NN];
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[nn][r] = 0.f;
        dv[nn][r] = 0.f;
      }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (kt >= 2 * NT) break;
      const bf16x8 dsa = ld8(ds_w + l32 * LT + 16 * kt + 8 * g);
      const bf16x8 pa = ld8(p_w + l32 * LT + 16 * kt + 8 * g);
#pragma unroll
      for (int nn = 0; nn < NN; ++nn) {
        dk[nn] = mfma32(ld8(sQT + (nn * 32 + l32) * LT + 16 * kt + 8 * g), dsa, dk[nn]);
        dv[nn] = mfma32(ld8(sdAT + (nn * 32 + l32) * LT + 16 * kt + 8 * g), pa, dv[nn]);
      }
    }
    wave_sync();
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
      u32x4 k0, k1, v0, v1;
      halves16(dk[nn], g, k0, k1);  // lane (key l32, g): features 16 g .. 16 g + 15 of the tile
      halves16(dv[nn], g, v0, v1);
      if (key < k_end) {
        bf16_t *row = a.dkv + (h0 + key) * 2 * d + col0 + nn * 32 + 16 * g;
        *reinterpret_cast<u32x4 *>(row) = k0;
        *reinterpret_cast<u32x4 *>(row + 8) = k1;
        *reinterpret_cast<u32x4 *>(row + d) = v0;
        *reinterpret_cast<u32x4 *>(row + d + 8) = v1;
      }
    }
  };
  for (int kb = kb0; kb < k_end; kb += 256) {
    block(kb, kr0, vr0, kr1, vr1);
    if (kb + 128 >= k_end) break;
    block(kb + 128, kr1, vr1, kr0, vr0);
  }
  // this wave's dQ partial: [64 targets][d_h]
  float *pd = a.part_dq + (((int64_t)c * a.H + eta) * 4 + w) * kMaxTgt * DH;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
#pragma unroll
      for (int r = 0; r < 16; ++r) pd[(nt * 32 + c32_row(lane, r)) * DH + nn * 32 + l32] = dq[nt][nn][r];
}

// The same backward for users of at most 16 targets at d_h = 32 (the training
// workload's shape), on tiles that match it instead of 32-target tiles with
// half their columns empty.  Per 32-key block and wave:
//   S^T, dP^T [keys x targets]:  two 16x16x32 tiles each (keys 0-15, 16-31;
//                                 k = d_h), A = K / V rows, B = Q / dA rows;
//   dQ [targets x d_h] += dS K:  16x16x32 per 16 features, A = dS straight
//                                 from the S^T tiles (lane = target; its 8
//                                 keys, 4 of each tile, form the k-group in
//                                 that order), B = K^T from a wave-private LDS
//                                 copy read in the same key order;
//   dK^T, dV^T [d_h x keys]:     one 32x32x16 each over the 16 targets, A =
//                                 Q^T / dA^T, B = dS^T / P^T re-read from
//                                 wave-private LDS as [key][target].
constexpr int kT16 = 16;
constexpr int LT16 = kT16 + 8;  // row stride of [.][target] tiles (48 bytes)

template <int SCORE, bool DD>
__global__ __launch_bounds__(256) void attn_bwd16_kernel(AttnBwdArgs a) {
  constexpr int DH = 32;
  __shared__ __attribute__((aligned(16))) bf16_t sQ[kT16 * (DH + 8)];
  __shared__ __attribute__((aligned(16))) bf16_t sdA[kT16 * (DH + 8)];
  __shared__ __attribute__((aligned(16))) bf16_t sQT[DH * LT16];
  __shared__ __attribute__((aligned(16))) bf16_t sdAT[DH * LT16];
  __shared__ __attribute__((aligned(16))) bf16_t sKT[4][DH * LK];
  __shared__ __attribute__((aligned(16))) bf16_t sP[4][32 * LT16];
  __shared__ __attribute__((aligned(16))) bf16_t sdS[4][32 * LT16];
  __shared__ float slse[kT16], sD[kT16];

  const Plan P = a.plan;
  const int c = blockIdx.x, eta = blockIdx.y;
  if (c >= P.coff[a.B]) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;  // 16x16 operand lanes: row / column, k-group
  const int l32 = lane & 31, g2 = lane >> 5;  // 32x32 operand lanes
  const int u = upper_index(P.coff, a.B, c);
  const int ci = c - P.coff[u];
  const int64_t h0 = P.hoff[u];
  const int L = P.hoff[u + 1] - P.hoff[u];
  const int k_begin = ci * a.nb * 32;
  const int k_end = min(L, k_begin + a.nb * 32);
  const int64_t t0 = P.toff[u];
  const int m = min(P.toff[u + 1] - P.toff[u], kT16);
  const int d = a.d;
  const int64_t col0 = (int64_t)eta * DH;

  // the user's Q and dA rows of this head (16 targets x 4 pieces of 8; rows
  // past m read target 0 and are zeroed)
  if (tid < kT16 * (DH / 8)) {
    const int t = tid >> 2, n0 = (tid & 3) * 8;
    u32x4 q = {0u, 0u, 0u, 0u}, gq = q;
    if (m > 0) {
      const int64_t row = (t0 + (t < m ? t : 0)) * d + col0 + n0;
      q = *reinterpret_cast<const u32x4 *>(a.q + row);
      gq = *reinterpret_cast<const u32x4 *>(a.da_lo + row);
      const uint32_t keep = t < m ? 0xffffffffu : 0u;
      q &= keep;
      gq &= keep;
    }
    *reinterpret_cast<u32x4 *>(sQ + t * (DH + 8) + n0) = q;
    *reinterpret_cast<u32x4 *>(sdA + t * (DH + 8) + n0) = gq;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sQT[(n0 + k) * LT16 + t] = (bf16_t)(q[k >> 1] >> (16 * (k & 1)));
      sdAT[(n0 + k) * LT16 + t] = (bf16_t)(gq[k >> 1] >> (16 * (k & 1)));
    }
  }
  if (tid < kT16) {
    slse[tid] = (SCORE == 0 && tid < m) ? a.lse[(t0 + tid) * a.H + eta] : 0.f;
    sD[tid] = tid < m ? a.dsum[(t0 + tid) * a.H + eta] : 0.f;
  }
  __syncthreads();

  f32x4 dq[2];
#pragma unroll
  for (int nn = 0; nn < 2; ++nn)
#pragma unroll
    for (int r = 0; r < 4; ++r) dq[nn][r] = 0.f;

  bf16_t *kt_w = sKT[w], *p_w = sP[w], *ds_w = sdS[w];
  const bf16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  // Lane l loads, for tile t, key 16 t + l % 16 of the block, features
  // 8 (l / 16) .. + 7: the 16x16x32 A operand as it comes from memory.  The
  // next block's rows are loaded while the current one is worked on (with
  // dedup the row ids one block further ahead); loads are unconditional
  // (keys past the chunk read its last key, zeroed where used).
  auto row_ids = [&](int kb, int (&id)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = min(kb + 16 * t + l16, k_end - 1);
      id[t] = DD ? a.tok2u[h0 + key] : key;
    }
  };
  auto load_kv = [&](const int (&id)[2], bf16x8(&kf)[2], bf16x8(&vf)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16_t *kr, *vr;
      if (DD) {  // blocked K, row-major V of the unique rows
        kr = a.k + ((((int64_t)(id[t] >> 5)) * a.H + eta) * 32 + (id[t] & 31)) * DH;
        vr = a.v + (int64_t)id[t] * d + col0;
      } else {
        kr = a.k + (h0 + id[t]) * d + col0;
        vr = a.v + (h0 + id[t]) * d + col0;
      }
      kf[t] = ld8(kr + 8 * g4);
      vf[t] = ld8(vr + 8 * g4);
    }
  };
  const int kb0 = k_begin + 32 * __builtin_amdgcn_readfirstlane(w);
  bf16x8 kr0[2], vr0[2], kr1[2], vr1[2];  // the two register sets
  int idn[2] = {0, 0};                    // the row ids of the block after the next
  if (kb0 < k_end) {
    int id0[2];
    row_ids(kb0, id0);
    load_kv(id0, kr0, vr0);
    row_ids(kb0 + 128, idn);
  }
  const bf16x8 qb = ld8(sQ + l16 * (DH + 8) + 8 * g4);   // B of S^T: Q[target l16][k-group g4]
  const bf16x8 gb = ld8(sdA + l16 * (DH + 8) + 8 * g4);  // B of dP^T
  const bool tval = l16 < m;
  const float lse = slse[l16], D = sD[l16];
  auto block = [&](const int kb, const bf16x8(&kc)[2], const bf16x8(&vc)[2], bf16x8(&kn)[2], bf16x8(&vn)[2]) {
    bf16x8 kf[2], vf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool kval = kb + 16 * t + l16 < k_end;
      kf[t] = kval ? kc[t] : zero8;
      vf[t] = kval ? vc[t] : zero8;
    }
    // the next block (past the chunk's end: its last key again, unused)
    load_kv(idn, kn, vn);
    row_ids(kb + 256, idn);
    // K^T [feature][key] for dQ's B operand
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) kt_w[(8 * g4 + e) * LK + 16 * t + l16] = (bf16_t)kf[t][e];
    wave_sync();
    float ds[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 st = {0.f, 0.f, 0.f, 0.f}, dpt = st;
      st = mfma16(kf[t], qb, st);
      dpt = mfma16(vf[t], gb, dpt);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = 16 * t + 4 * g4 + r;  // key row within the block
        const bool ok = tval && kb + kr < k_end;
        float p, dsv;
        if (SCORE == 0) {
          p = ok ? __builtin_amdgcn_exp2f((st[r] - lse) * kLog2e) : 0.f;
          dsv = p * (dpt[r] - D);
        } else {
          const bool pos = ok && st[r] > 0.f;
          p = pos ? st[r] : 0.f;
          dsv = pos ? dpt[r] : 0.f;
        }
        ds[t][r] = dsv;
        p_w[kr * LT16 + l16] = f2bf(p);
        ds_w[kr * LT16 + l16] = f2bf(dsv);
      }
    }
    // dQ[targets] += dS K over the block's 32 keys: the lane's k-group g4 is
    // keys 4 g4 .. + 3 then 16 + 4 g4 .. + 3
    {
      bf16x8 af;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        af[r] = (short)f2bf(ds[0][r]);
        af[4 + r] = (short)f2bf(ds[1][r]);
      }
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const bf16_t *row = kt_w + (nn * 16 + l16) * LK + 4 * g4;
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(row);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(row + 16);
        u32x4 bw = {lo[0], lo[1], hi[0], hi[1]};
        dq[nn] = mfma16(af, __builtin_bit_cast(bf16x8, bw), dq[nn]);
      }
    }
    wave_sync();
    // dK^T = Q^T dS, dV^T = dA^T P over the 16 targets: features as rows,
    // keys as columns, so each lane ends up with 16 consecutive features of
    // one key for 16-byte stores
    f32x16 dk, dv;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[r] = 0.f;
      dv[r] = 0.f;
    }
    dk = mfma32(ld8(sQT + l32 * LT16 + 8 * g2), ld8(ds_w + l32 * LT16 + 8 * g2), dk);
    dv = mfma32(ld8(sdAT + l32 * LT16 + 8 * g2), ld8(p_w + l32 * LT16 + 8 * g2), dv);
    wave_sync();
    u32x4 k0, k1, v0, v1;
    halves16(dk, g2, k0, k1);  // lane (key l32, g2): features 16 g2 .. 16 g2 + 15
    halves16(dv, g2, v0, v1);
    const int key = kb + l32;
    if (key < k_end) {
      bf16_t *row = a.dkv + (h0 + key) * 2 * d + col0 + 16 * g2;
      *reinterpret_cast<u32x4 *>(row) = k0;
      *reinterpret_cast<u32x4 *>(row + 8) = k1;
      *reinterpret_cast<u32x4 *>(row + d) = v0;
      *reinterpret_cast<u32x4 *>(row + d + 8) = v1;
    }
  };
  for (int kb = kb0; kb < k_end; kb += 256) {
    block(kb, kr0, vr0, kr1, vr1);
    if (kb + 128 >= k_end) break;
    block(kb + 128, kr1, vr1, kr0, vr0);
  }
  // this wave's dQ partial: targets 0..15 of the [64 targets][d_h] slot (the
  // fold reads no target past the user's count)
  float *pd = a.part_dq + (((int64_t)c * a.H + eta) * 4 + w) * kMaxTgt * DH;
#pragma unroll
  for (int nn = 0; nn < 2; ++nn)
#pragma unroll
    for (int r = 0; r < 4; ++r) pd[(4 * g4 + r) * DH + nn * 16 + l16] = dq[nn][r];
}

__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= a.n_tgt * a.d) return;
  const int64_t t = e / a.d;
  const int f = (int)(e % a.d);
  const Plan P = a.plan;
  float s = 0.f;
  if (t < P.toff[a.B]) {
    const int u = upper_index(P.toff, a.B, (int)t);
    const int tl = (int)(t - P.toff[u]);
    const int h = f / a.dh, n = f % a.dh;
    if (tl < kMaxTgt)
      for (int c = P.coff[u]; c < P.coff[u + 1]; ++c)
        for (int w = 0; w < 4; ++w) s += a.part_dq[((((int64_t)c * a.H + h) * 4 + w) * kMaxTgt + tl) * a.dh + n];
  }
  a.dq[e] = s;
}

}  // namespace

int64_t attn_bwd_part_floats(int64_t max_chunks, int H, int dh) { return max_chunks * H * 4 * kMaxTgt * dh; }

hipError_t launch_attn_bwd(const AttnBwdArgs &a, hipStream_t s) {
  if (a.n_tgt > 0) {
    const int64_t n = a.n_tgt * a.H;
    hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.max_chunks > 0 && a.n_hist > 0) {
    const dim3 grid((unsigned)a.max_chunks, (unsigned)a.H);
#define AB(DH, SC)                                                                        \
  do {                                                                                    \
    if (a.tok2u) hipLaunchKernelGGL((attn_bwd_kernel<DH, SC, true>), grid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((attn_bwd_kernel<DH, SC, false>), grid, dim3(256), 0, s, a);       \
  } while (0)
#define AB16(SC)                                                                                  \
  do {                                                                                            \
    if (a.tok2u) hipLaunchKernelGGL((attn_bwd16_kernel<SC, true>), grid, dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((attn_bwd16_kernel<SC, false>), grid, dim3(256), 0, s, a);        \
  } while (0)
    if (a.dh == 32 && a.max_tgt <= kT16) {  // every user has at most 16 targets
      if (a.score) AB16(1);
      else AB16(0);
    } else if (a.dh == 32) {
      if (a.score) AB(32, 1);
      else AB(32, 0);
    } else if (a.dh == 64) {
      if (a.score) AB(64, 1);
      else AB(64, 0);
    } else {
      return hipErrorInvalidValue;
    }
#undef AB
#undef AB16
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_tgt > 0) {
    const int64_t n = a.n_tgt * a.d;
    hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace stca
