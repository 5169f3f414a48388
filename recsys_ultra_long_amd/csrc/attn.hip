// attn.hip -- m-target multi-head cross attention over a user's history
// (a8), split along the history and merged in a fixed order.
//
// Per user u, target t of u and head eta ([Review] formula for alpha and o;
// [WeChat] §1.2 for the ReLU-scored form):
//   s_j = Q_t[eta] . K_j[eta]   (Q rows already carry 1/sqrt(d_h))
//   softmax: o = sum_j exp(s_j - max) V_j[eta] / sum_j exp(s_j - max)
//   relu:    o = sum_j max(0, s_j) V_j[eta],   active = #{j : s_j > 0}
//
// Request Level Batching ([Notes] §RLB): one workgroup streams a chunk of the
// user's K/V blocks once and serves up to 64 of the user's targets with it.
// The history is split into chunks of `nb` 32-key blocks (the single-GPU form
// of the per-device partial attention of [WeChat] §1.1; the blocked tiling
// follows the SRAM tiling idea of [WeChat] §3.3.1): each chunk writes a
// partial (running max, running sum, accumulator) per (target, head), and a
// second pass merges a user's partials in chunk order -- no float atomics, so
// results do not depend on scheduling.
//
// K/V layout (written by the history chain): per 32-key block b and head h,
//   K[b][h][key 0..31][d_h]   (row of a key contiguous)
//   V[b][h][d_h][key 0..31]   (transposed: a feature's 32 keys contiguous)
// so every MFMA operand fragment is one 16-byte load.
#include "stca_internal.h"

namespace stca {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

DEV float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ bf16 / MFMA
// S^T = K Q^T (16 keys x 16 targets per MFMA), online softmax in registers,
// O^T += V^T P^T (16 features x 16 targets per MFMA).  The key order inside a
// 32-key block is permuted when K is loaded so that the score tile's lane
// layout is exactly the B-operand layout P^T needs: lane l (g = l/16) holds the
// scores of keys 8g..8g+7 for target l%16.
template <int DH, int NT, int SCORE>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KS = DH / 32;  // k-steps of the score MFMA
  constexpr int DT = DH / 16;  // feature tiles of the output
  constexpr int TG = NT * 16;  // targets per workgroup
  __shared__ float sm_m[4][TG], sm_l[4][TG];
  __shared__ int sm_c[4][TG];
  __shared__ float sm_o[4][TG][DH + 1];

  const int c = blockIdx.x, h = blockIdx.y;
  const Plan P = a.plan;
  if (c >= P.coff[a.B]) return;
  const int u = upper_index(P.coff, a.B, c);
  const int tbase = P.toff[u];
  const int m_u = P.toff[u + 1] - tbase;
  const int t0 = blockIdx.z * TG;
  if (t0 >= m_u) return;
  const int L = P.hoff[u + 1] - P.hoff[u];
  const int cl = c - P.coff[u];
  const int b_begin = P.pblk[u] + cl * a.nb;
  const int b_end = min(P.pblk[u + 1], b_begin + a.nb);
  const int key0 = cl * a.nb * 32;  // user-local index of the chunk's first key

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int H = a.H;
  const bf16_t *Q = (const bf16_t *)a.q;
  const bf16_t *Kb = (const bf16_t *)a.kbuf, *Vb = (const bf16_t *)a.vbuf;

  bf16x8 qf[NT][KS];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int tl = t0 + n * 16 + c16;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (tl < m_u) {
        qf[n][k] = ld8(Q + (int64_t)(tbase + tl) * a.d + h * DH + k * 32 + g * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[n][k][e] = 0;
      }
    }
  }
  float mrun[NT], lrun[NT];
  int cnt[NT];
  f32x4 o[DT][NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    mrun[n] = kNegBig;
    lrun[n] = 0.f;
    cnt[n] = 0;
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // key row this lane loads for score tile kt (a permutation of the block)
  const int kr0 = 8 * (c16 >> 2) + (c16 & 3);

  for (int b = b_begin + w; b < b_end; b += 4) {
    const bf16_t *kb = Kb + ((int64_t)b * H + h) * 32 * DH;
    const bf16_t *vb = Vb + ((int64_t)b * H + h) * DH * 32;
    bf16x8 kf[2][KS], vf[DT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int k = 0; k < KS; ++k) kf[kt][k] = ld8(kb + (kr0 + 4 * kt) * DH + k * 32 + g * 8);
#pragma unroll
    for (int t = 0; t < DT; ++t) vf[t] = ld8(vb + (t * 16 + c16) * 32 + g * 8);

    f32x4 st[2][NT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        st[kt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; ++k) st[kt][n] = mfma16(kf[kt][k], qf[n][k], st[kt][n]);
      }
    // keys of this lane: 8g + 4kt + r; valid while below the user's length
    const int nvalid = L - (key0 + (b - b_begin) * 32);
    bf16x8 pk[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (SCORE == 0) {
        float mx = kNegBig;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (8 * g + 4 * kt + r < nvalid) mx = fmaxf(mx, st[kt][n][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrun[n], mx);
        const float corr = ex2((mrun[n] - mnew) * kLog2e);
        mrun[n] = mnew;
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float p = 0.f;
            if (8 * g + 4 * kt + r < nvalid) p = ex2((st[kt][n][r] - mnew) * kLog2e);
            const bf16_t pb = f2bf(p);
            psum += bf2f(pb);
            pk[n][4 * kt + r] = (short)pb;
          }
        lrun[n] = lrun[n] * corr + psum;
#pragma unroll
        for (int t = 0; t < DT; ++t) o[t][n] *= corr;
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = st[kt][n][r];
            const bool on = (8 * g + 4 * kt + r < nvalid) && s > 0.f;
            cnt[n] += on ? 1 : 0;
            pk[n][4 * kt + r] = (short)f2bf(on ? s : 0.f);
          }
      }
    }
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int n = 0; n < NT; ++n) o[t][n] = mfma16(vf[t], pk[n], o[t][n]);
  }

  // ---- merge the four waves in LDS, then write this chunk's partial
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float l = lrun[n];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    int cn = cnt[n];
    cn += __shfl_xor(cn, 16);
    cn += __shfl_xor(cn, 32);
    if (g == 0) {
      sm_m[w][n * 16 + c16] = mrun[n];
      sm_l[w][n * 16 + c16] = l;
      sm_c[w][n * 16 + c16] = cn;
    }
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[w][n * 16 + c16][t * 16 + 4 * g + r] = o[t][n][r];
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)c * H + h) * a.max_tgt + t0;
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
}

// ------------------------------------------------------------------ fp32
// One wave per (chunk, head, 64 targets); lane = target; keys streamed one at
// a time.  The fp32 configuration is the precision reference of the library
// (small shapes), so scores and sums are accumulated in fp64: the ReLU-scored
// sum is unnormalised and cancels heavily, and fp32 accumulation alone would
// cost most of a 1e-5 error budget.
template <int DH, int SCORE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int c = blockIdx.x, h = blockIdx.y;
  const Plan P = a.plan;
  if (c >= P.coff[a.B]) return;
  const int u = upper_index(P.coff, a.B, c);
  const int tbase = P.toff[u];
  const int m_u = P.toff[u + 1] - tbase;
  const int t0 = blockIdx.z * 64;
  if (t0 >= m_u) return;
  const int L = P.hoff[u + 1] - P.hoff[u];
  const int cl = c - P.coff[u];
  const int b_begin = P.pblk[u] + cl * a.nb;
  const int b_end = min(P.pblk[u + 1], b_begin + a.nb);
  const int key0 = cl * a.nb * 32;
  const int H = a.H;
  const int tl = t0 + threadIdx.x;
  const bool act = tl < m_u;
  const float *Q = (const float *)a.q;
  const float *Kb = (const float *)a.kbuf, *Vb = (const float *)a.vbuf;
  double q[DH], acc[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) {
    q[i] = act ? (double)Q[(int64_t)(tbase + tl) * a.d + h * DH + i] : 0.0;
    acc[i] = 0.0;
  }
  double mrun = -1.0e300, lrun = 0.0;
  int cnt = 0;
  for (int b = b_begin; b < b_end; ++b) {
    const float *kb = Kb + ((int64_t)b * H + h) * 32 * DH;
    const float *vb = Vb + ((int64_t)b * H + h) * DH * 32;
    const int nvalid = min(32, L - (key0 + (b - b_begin) * 32));
    for (int j = 0; j < nvalid; ++j) {
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < DH; ++i) s = fma(q[i], (double)kb[j * DH + i], s);
      double p;
      if (SCORE == 0) {
        const double mnew = fmax(mrun, s);
        const double corr = exp(mrun - mnew);
        p = exp(s - mnew);
        lrun = lrun * corr + p;
#pragma unroll
        for (int i = 0; i < DH; ++i) acc[i] *= corr;
        mrun = mnew;
      } else {
        p = s > 0.0 ? s : 0.0;
        cnt += s > 0.0 ? 1 : 0;
      }
#pragma unroll
      for (int i = 0; i < DH; ++i) acc[i] = fma(p, (double)vb[i * 32 + j], acc[i]);
    }
  }
  if (!act) return;
  const int64_t pi = ((int64_t)c * H + h) * a.max_tgt + tl;
  // fp32 partials: the softmax accumulator is stored normalised by its own
  // running sum (a convex combination, no cancellation), the sum separately.
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

// ------------------------------------------------------------------ merge
// One thread per (target, feature): fold the user's chunk partials in chunk
// order.  attn = sum_c acc_c e^{m_c - M} / sum_c l_c e^{m_c - M}; ReLU: sums.
template <int SCORE>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int d = a.d, DH = a.dh, H = a.H;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= a.n_tgt * d) return;
  const int t = (int)(e / d), f = (int)(e % d);
  const int h = f / DH, dh = f % DH;
  const Plan P = a.plan;
  float out = 0.f;
  int cnt = 0;
  if (t < P.toff[a.B]) {
    const int u = upper_index(P.toff, a.B, t);
    const int tl = t - P.toff[u];
    const int c0 = P.coff[u], c1 = P.coff[u + 1];
    if (SCORE == 0 && a.dtype) {
      float M = kNegBig;
      for (int c = c0; c < c1; ++c) M = fmaxf(M, a.part_ml[(((int64_t)c * H + h) * a.max_tgt + tl) * 2]);
      float acc = 0.f, l = 0.f;
      for (int c = c0; c < c1; ++c) {
        const int64_t pi = ((int64_t)c * H + h) * a.max_tgt + tl;
        const float fct = ex2((a.part_ml[pi * 2] - M) * kLog2e);
        acc += a.part_acc[pi * DH + dh] * fct;
        l += a.part_ml[pi * 2 + 1] * fct;
      }
      out = l > 0.f ? acc / l : 0.f;
    } else if (SCORE == 0) {  // fp32 path: normalised partials, fp64 fold
      double M = -1.0e300;
      for (int c = c0; c < c1; ++c)
        M = fmax(M, (double)a.part_ml[(((int64_t)c * H + h) * a.max_tgt + tl) * 2]);
      double acc = 0.0, l = 0.0;
      for (int c = c0; c < c1; ++c) {
        const int64_t pi = ((int64_t)c * H + h) * a.max_tgt + tl;
        const double wgt = (double)a.part_ml[pi * 2 + 1] * exp((double)a.part_ml[pi * 2] - M);
        acc += (double)a.part_acc[pi * DH + dh] * wgt;
        l += wgt;
      }
      out = l > 0.0 ? (float)(acc / l) : 0.f;
    } else if (a.dtype) {
      for (int c = c0; c < c1; ++c) {
        const int64_t pi = ((int64_t)c * H + h) * a.max_tgt + tl;
        out += a.part_acc[pi * DH + dh];
        if (dh == 0) cnt += a.part_cnt[pi];
      }
    } else {
      double acc = 0.0;
      for (int c = c0; c < c1; ++c) {
        const int64_t pi = ((int64_t)c * H + h) * a.max_tgt + tl;
        acc += (double)a.part_acc[pi * DH + dh];
        if (dh == 0) cnt += a.part_cnt[pi];
      }
      out = (float)acc;
    }
  }
  a.attn[e] = out;
  if (a.attn_lo) {
    if (a.dtype) ((bf16_t *)a.attn_lo)[e] = f2bf(out);
    else ((float *)a.attn_lo)[e] = out;
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

template <int DH, int SCORE>
hipError_t launch_bf16(const AttnArgs &a, hipStream_t s) {
  const int groups = (a.max_tgt + 63) / 64;
  const int nt = a.max_tgt >= 64 ? 4 : (a.max_tgt + 15) / 16;
  const dim3 block(256);
  if (nt == 4 || groups > 1) {
    hipLaunchKernelGGL((attn_bf16_kernel<DH, 4, SCORE>), dim3(a.grid_chunks, a.H, groups), block, 0, s, a);
  } else if (nt == 3) {
    hipLaunchKernelGGL((attn_bf16_kernel<DH, 3, SCORE>), dim3(a.grid_chunks, a.H, 1), block, 0, s, a);
  } else if (nt == 2) {
    hipLaunchKernelGGL((attn_bf16_kernel<DH, 2, SCORE>), dim3(a.grid_chunks, a.H, 1), block, 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_bf16_kernel<DH, 1, SCORE>), dim3(a.grid_chunks, a.H, 1), block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_partial(const AttnArgs &a, hipStream_t s) {
  if (a.grid_chunks <= 0 || a.n_tgt <= 0) return hipSuccess;
  if (a.dtype == 1) {
    if (a.dh == 32) return a.score ? launch_bf16<32, 1>(a, s) : launch_bf16<32, 0>(a, s);
    if (a.dh == 64) return a.score ? launch_bf16<64, 1>(a, s) : launch_bf16<64, 0>(a, s);
    return hipErrorInvalidValue;
  }
  const dim3 grid(a.grid_chunks, a.H, (a.max_tgt + 63) / 64), block(64);
  if (a.dh == 32) {
    if (a.score) hipLaunchKernelGGL((attn_f32_kernel<32, 1>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_f32_kernel<32, 0>), grid, block, 0, s, a);
  } else if (a.dh == 64) {
    if (a.score) hipLaunchKernelGGL((attn_f32_kernel<64, 1>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_f32_kernel<64, 0>), grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs &a, hipStream_t s) {
  if (a.n_tgt <= 0) return hipSuccess;
  const int64_t n = a.n_tgt * a.d;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (a.score) hipLaunchKernelGGL(merge_kernel<1>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<0>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
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
