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

template <int DH, int SCORE>
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

  for (int e = tid; e < kMaxTgt * DH; e += 256) {
    const int t = e / DH, n = e % DH;
    bf16_t q = 0, gq = 0;
    if (t < m) {
      q = a.q[(t0 + t) * d + col0 + n];
      gq = a.da_lo[(t0 + t) * d + col0 + n];
    }
    sQ[t * (DH + 8) + n] = q;
    sdA[t * (DH + 8) + n] = gq;
    sQT[n * LT + t] = q;
    sdAT[n * LT + t] = gq;
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
  for (int kb = k_begin + 32 * w; kb < k_end; kb += 128) {
    const int key = kb + l32;
    const bool kval = key < k_end;
    bf16x8 kf[KS], vf[KS];
    if (a.tok2u) {  // the item's unique row: blocked K, row-major V
      const int ui = kval ? a.tok2u[h0 + key] : 0;
      const bf16_t *kr = a.k + ((((int64_t)(ui >> 5)) * a.H + eta) * 32 + (ui & 31)) * DH;
      const bf16_t *vr = a.v + (int64_t)ui * d + col0;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kf[s] = kval ? ld8(kr + 16 * s + 8 * g) : zero8;
        vf[s] = kval ? ld8(vr + 16 * s + 8 * g) : zero8;
      }
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        kf[s] = kval ? ld8(a.k + (h0 + key) * d + col0 + 16 * s + 8 * g) : zero8;
        vf[s] = kval ? ld8(a.v + (h0 + key) * d + col0 + 16 * s + 8 * g) : zero8;
      }
    }
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
          p = ok ? expf(st[r] - lse) : 0.f;
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
    // dK = dS^T Q, dV = P^T dA over this user's targets (16 per k-step)
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
        dk[nn] = mfma32(dsa, ld8(sQT + (nn * 32 + l32) * LT + 16 * kt + 8 * g), dk[nn]);
        dv[nn] = mfma32(pa, ld8(sdAT + (nn * 32 + l32) * LT + 16 * kt + 8 * g), dv[nn]);
      }
    }
    wave_sync();
#pragma unroll
    for (int nn = 0; nn < NN; ++nn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = kb + c32_row(lane, r);
        if (kk < k_end) {
          bf16_t *row = a.dkv + (h0 + kk) * 2 * d + col0 + nn * 32 + l32;
          row[0] = f2bf(dk[nn][r]);
          row[d] = f2bf(dv[nn][r]);
        }
      }
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
    if (a.dh == 32) {
      if (a.score) hipLaunchKernelGGL((attn_bwd_kernel<32, 1>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attn_bwd_kernel<32, 0>), grid, dim3(256), 0, s, a);
    } else if (a.dh == 64) {
      if (a.score) hipLaunchKernelGGL((attn_bwd_kernel<64, 1>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attn_bwd_kernel<64, 0>), grid, dim3(256), 0, s, a);
    } else {
      return hipErrorInvalidValue;
    }
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
