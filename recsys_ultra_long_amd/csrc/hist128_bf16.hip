// hist128_bf16.hip -- history encoder for d = 128 (bf16): every layer's
//   X~ = [LN](SwiGLU(X)) = [LN]((SiLU(X W1) * (X W3)) W2),  K = X~ W_K, V = X~ W_V
// ([Notes] §STCA; [Review] architecture tree) over 128-row tiles of the
// padded history, all M layers per launch on one gathered tile.
//
// The d = 256 encoder's shape (hist_bf16.hip) at half the width: one
// workgroup of 8 waves (one per CU, two per SIMD) takes 128 rows, so each
// weight fragment feeds more rows than the 64-row row chain does.
//   G   = SiLU(X W1) * (X W3)  : wave w owns hidden units 16w .. 16w+15 of each
//                                128-unit chunk, all 128 rows (16x16x32 MFMA)
//   Y^T += W2^T G^T            : wave w owns features 32 (w & 3) .. + 31 of
//                                rows 64 (w >> 2) .. + 63 (32x32x16 MFMA)
//   K^T  = W_K^T X~^T, V = X~ W_V : the same feature tile and row half
// At d = 128 the 128 output features are four 32-wide MFMA tiles, so the
// waves split the rows of the Y and projection phases in two halves (each of
// those weight fragments feeds 64 rows); the G phase keeps all 128 rows per
// fragment.  LN statistics of a row are merged over the four waves of its
// row half.  Weights stream through the shared register ring (hist_common.h)
// three blocks ahead across phases and layers.  LDS: the raw rows (kept for
// all layers) and two G chunk buffers, the first of which holds the LN output
// for the projection.
#include <algorithm>

#include "hist_common.h"
#include "stca_internal.h"

namespace stca {
namespace {

using enc::Ring;
using enc::Src;
using enc::ring_load;
using enc::run_phase;
using enc::zero16;
using enc::zero4;

constexpr int kD = 128;
constexpr int kT = 512;          // threads: 8 waves
constexpr int kR = 128;          // rows per tile
constexpr int kHC = 128;         // hidden units per chunk (16 per wave)
constexpr int kXLD = kD + 8;     // LDS row stride of X~ (read as the 32x32x16 operand)
constexpr int kXRLD = kD + 16;   // LDS row stride of the raw rows (16x16x32 operand of the G phase)
constexpr int kGLD = kHC + 8;    // LDS row stride of a G chunk (32x32x16 operand)

struct Smem {
  __attribute__((aligned(16))) bf16_t xs[kR * kXRLD];
  __attribute__((aligned(16))) bf16_t gs[2][kR * kGLD];
  float red[2][4][kR];
  int s_id[kR], s_tok[kR];
};
static_assert(sizeof(Smem::gs[0]) >= sizeof(bf16_t) * kR * kXLD, "LN output must fit the first G buffer");

struct Layer {
  const bf16_t *w1, *w3, *w2, *wp;
  const float *ln_g, *ln_b;
  bf16_t *kb, *vb;
};
// W1 / W3: 16-row tiles of the 16x16x32 A operand (tile hc * 8 + w).
DEV Src src_g(const Layer &L, int hc, int w, int lane) {
  const int64_t o = (int64_t)((hc * 8 + w) * (kD / 32)) * 512 + lane * 8;
  return Src{L.w1 + o, L.w3 + o, 512};
}
// W2^T: 32-feature tile ft of the 32x32x16 A operand, hidden chunk hc.
DEV Src src_y(const Layer &L, int hc, int ft, int lane, int nkh) {
  const bf16_t *p = L.w2 + frag_off(ft, hc * (kHC / 32), nkh, 0, lane);
  return Src{p, p + 512, 1024};
}
// W_K | W_V of feature tile ft, k blocks interleaved (K0, V0, K1, V1, ..).
DEV Src src_kv(const Layer &L, int ft, int lane) {
  const bf16_t *p = L.wp + (int64_t)ft * (kD / 32) * 2048 + lane * 8;
  return Src{p, p + 512, 1024};
}

// SwiGLU FFN [+ LN] of one layer over the 128 rows in sm.xs; X~ goes to
// sm.gs[0] (row stride kXLD) and the raw rows survive for the next layer.
// The ring enters holding the first blocks of G chunk 0 and leaves holding
// those of `after`; X~ is visible to every thread on return.
template <bool LN>
DEV void ffn_ln(Ring &ring, const Layer &L, Smem &sm, int w, int lane, int nkh, int nchunk, const Src &after) {
  const int l32 = lane & 31, hi = lane >> 5;
  const int c16 = lane & 15, g16 = lane >> 4;
  const int ft = w & 3, rh = w >> 2;  // Y / projection: feature tile, row half
  const bf16_t *const xrow = sm.xs + c16 * kXRLD + g16 * 8;  // G-phase operand base
  f32x16 y[2];  // Y^T: features 32 ft .., tokens 32 (2 rh + j) + l32
  zero16(y);
  f32x4 acc[2][8];  // G^T of one chunk: W1 and W3 rows of this wave's 16 units x 128 tokens
  auto g_mma = [&](int hc, const Src &nxt) {
    zero4(acc[0]);
    zero4(acc[1]);
    run_phase<kD / 32>(ring, src_g(L, hc, w, lane), nxt, true, [&](int kb, int slot) {
#pragma unroll
      for (int t0 = 0; t0 < 8; t0 += 4) {  // four row tiles at a time
        bf16x8 bx[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) bx[t] = ld8(xrow + (t0 + t) * 16 * kXRLD + kb * 32);
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[f][t0 + t] = mfma16(ring.v[slot][f], bx[t], acc[f][t0 + t]);
      }
    });
  };
  // lane: hidden rows 4 g16 + i of token 16 t + c16
  auto silu_store = [&](bf16_t *g, int t) {
    float gv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) gv[i] = silu_fast(acc[0][t][i]) * acc[1][t][i];
    u32x2 v = {pack_bf2(gv[0], gv[1]), pack_bf2(gv[2], gv[3])};
    *reinterpret_cast<u32x2 *>(g + (t * 16 + c16) * kGLD + w * 16 + 4 * g16) = v;
  };
  // Y^T += W2^T[feature tile ft, chunk hc] G^T[chunk, row half rh]; with
  // `gnext`, also the SiLU epilogue of the chunk in acc (two row tiles per block)
  auto y_mma = [&](int hc, const Src &nxt, bf16_t *gnext) {
    const bf16_t *g = sm.gs[hc & 1];
    run_phase<kHC / 32>(ring, src_y(L, hc, ft, lane, nkh), nxt, true, [&](int kb, int slot) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 bg[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bg[j] = ld8(g + ((2 * rh + j) * 32 + l32) * kGLD + kb * 32 + hi * 16 + h * 8);
#pragma unroll
        for (int j = 0; j < 2; ++j) y[j] = mfma32(ring.v[slot][h], bg[j], y[j]);
      }
      if (gnext) {
        silu_store(gnext, 2 * kb);
        silu_store(gnext, 2 * kb + 1);
      }
    });
  };
  static_assert(kHC / 32 * 2 == 8, "two row tiles of the SiLU epilogue per Y block");
  // software-pipelined over hidden chunks: G0 | G1, Y0 (+ SiLU of G1) | .. | Y(last)
  g_mma(0, nchunk > 1 ? src_g(L, 1, w, lane) : src_y(L, 0, ft, lane, nkh));
#pragma unroll
  for (int t = 0; t < 8; ++t) silu_store(sm.gs[0], t);
  __syncthreads();
#pragma unroll 1
  for (int hc = 1; hc < nchunk; ++hc) {
    g_mma(hc, src_y(L, hc - 1, ft, lane, nkh));
    y_mma(hc - 1, hc + 1 < nchunk ? src_g(L, hc + 1, w, lane) : src_y(L, hc, ft, lane, nkh), sm.gs[hc & 1]);
    __syncthreads();
  }
  y_mma(nchunk - 1, after, nullptr);

  // ------------------------------------------------------------ LayerNorm
  // lane: features 32 ft + (8q + 4hi + r) of token 32 (2 rh + j) + l32
  float mean[2], rstd[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    mean[j] = 0.f;
    rstd[j] = 1.f;
  }
  if (LN) {
    // each lane's 16 values give a partial (mean, sum of squared deviations),
    // merged with the other half-wave, then over the four waves of the row
    // half through LDS: M2 = sum M2_q + n sum_q (mean_q - mean)^2, n = 32
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float s1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s1 += y[j][i];
      const float m16 = s1 * (1.0f / 16);
      float m2 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m2 += (y[j][i] - m16) * (y[j][i] - m16);
      uint32_t ma = __float_as_uint(m16), mb = ma, qa = __float_as_uint(m2), qb = qa;
      swap32(ma, mb);  // ma: lower half-wave's partial, mb: upper's
      swap32(qa, qb);
      const float dm = __uint_as_float(ma) - __uint_as_float(mb);
      if (hi == 0) {
        const int t = (2 * rh + j) * 32 + l32;
        sm.red[0][ft][t] = 0.5f * (__uint_as_float(ma) + __uint_as_float(mb));
        sm.red[1][ft][t] = __uint_as_float(qa) + __uint_as_float(qb) + 8.0f * dm * dm;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = (2 * rh + j) * 32 + l32;
      float mq[4], tot = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mq[q] = sm.red[0][q][t];
        tot += mq[q];
      }
      const float mu = tot * (1.0f / 4);
      float m2 = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) m2 += sm.red[1][q][t] + 32.0f * (mq[q] - mu) * (mq[q] - mu);
      mean[j] = mu;
      rstd[j] = rsqrtf(m2 * (1.0f / kD) + 1e-5f);
    }
  } else {
    __syncthreads();  // every wave is done reading the last G chunk
  }
  bf16_t *const xt = &sm.gs[0][0];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = ft * 32 + 8 * q + 4 * hi;
    f32x4 gg = {1.f, 1.f, 1.f, 1.f}, bb = {0.f, 0.f, 0.f, 0.f};
    if (LN) {
      gg = ldg4(L.ln_g + f);
      bb = ldg4(L.ln_b + f);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = y[j][4 * q + r];
        if (LN) v[r] = (v[r] - mean[j]) * rstd[j] * gg[r] + bb[r];
      }
      u32x2 pv = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
      *reinterpret_cast<u32x2 *>(xt + ((2 * rh + j) * 32 + l32) * kXLD + f) = pv;
    }
  }
  __syncthreads();
}

template <bool LN>
__global__ __launch_bounds__(kT, 1) void hist128_kernel(ChainArgs a, HistLayers hl) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * kR;
  const int total_blocks = a.plan.pblk[a.B];
  if (row0 >= (int64_t)total_blocks * 32) return;
  const int nkh = a.hidden / 32, nchunk = a.hidden / kHC;
  const int H = a.H, DH = kD / a.H;
  // optional clock probe: shader-clock and 100 MHz counters at start and end
  if (hl.clock && blockIdx.x < 8 && tid == 0) {
    hl.clock[blockIdx.x * 4] = __builtin_amdgcn_s_memtime();
    hl.clock[blockIdx.x * 4 + 1] = __builtin_amdgcn_s_memrealtime();
  }
  auto layer = [&](int i) {
    Layer L;
    L.w1 = (const bf16_t *)hl.w1[i];
    L.w3 = (const bf16_t *)hl.w3[i];
    L.w2 = (const bf16_t *)hl.w2[i];
    L.wp = (const bf16_t *)hl.wp[i];
    L.ln_g = hl.ln_g[i];
    L.ln_b = hl.ln_b[i];
    L.kb = (bf16_t *)hl.kbuf[i];
    L.vb = (bf16_t *)hl.vbuf[i];
    return L;
  };

  Ring ring;
  {
    const Layer L0 = layer(0);
    const Src s0 = src_g(L0, 0, w, lane);
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) ring_load(ring, kb, s0, kb);
  }

  enc::gather_tile<kD, kR, kXRLD, kT>(a, sm.xs, sm.s_id, sm.s_tok, row0, total_blocks, tid, true);

  const bf16_t *const xt = &sm.gs[0][0];  // LN output, row stride kXLD
#pragma unroll 1
  for (int li = 0; li < hl.M; ++li) {
    // lane quantities re-derived per layer so none is held across layers
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    const int lane = ltid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int ft = w & 3, rh = w >> 2;
    Layer L = layer(li);
    // the weight addresses stay loop-variant (no hoisting across layers)
    asm volatile("" : "+s"(L.w1), "+s"(L.w3), "+s"(L.w2), "+s"(L.wp), "+s"(L.ln_g), "+s"(L.ln_b));
    if (li > 0) __syncthreads();  // the previous layer's projection is done with X~

    ffn_ln<LN>(ring, L, sm, w, lane, nkh, nchunk, src_kv(L, ft, lane));

    // ------------------------------------------------------------ W_K | W_V
    // K^T = W_K^T X~^T and V = X~ W_V of feature tile ft and row half rh in one
    // pass over the interleaved weight stream: the X~ operand of a k block is
    // read once, for both products.  After the exchange each lane holds 16
    // consecutive features of one key (K) or 16 consecutive keys of one
    // feature (V), stored as two 16-byte runs.
    {
      f32x16 ka[2], va[2];
      zero16(ka);
      zero16(va);
      bf16x8 bx[2][2];
      const bool more = li + 1 < hl.M;
      Src nxt = src_kv(L, ft, lane);  // any valid address when nothing follows
      if (more) {
        const Layer Ln = layer(li + 1);
        nxt = src_g(Ln, 0, w, lane);
      }
      run_phase<2 * kD / 32>(ring, src_kv(L, ft, lane), nxt, more, [&](int b, int slot) {
        const int kb = b >> 1;
        if ((b & 1) == 0) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              bx[h][j] = ld8(xt + ((2 * rh + j) * 32 + l32) * kXLD + kb * 32 + hi * 16 + h * 8);
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 2; ++j) ka[j] = mfma32(ring.v[slot][h], bx[h][j], ka[j]);
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 2; ++j) va[j] = mfma32(bx[h][j], ring.v[slot][h], va[j]);
        }
      });
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int blk = (int)(row0 >> 5) + 2 * rh + j;
        if (blk >= total_blocks) continue;
        u32x4 o0, o1;
        halves16(ka[j], hi, o0, o1);
        const int f = ft * 32 + 16 * hi;
        const int h = f / DH, dh = f % DH;
        bf16_t *dst = L.kb + (((int64_t)blk * H + h) * 32 + l32) * DH + dh;
        stnt16(dst, o0);
        stnt16(dst + 8, o1);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int blk = (int)(row0 >> 5) + 2 * rh + j;
        if (blk >= total_blocks) continue;
        u32x4 o0, o1;
        halves16(va[j], hi, o0, o1);
        const int f = ft * 32 + l32;
        const int h = f / DH, dh = f % DH;
        bf16_t *dst = L.vb + (((int64_t)blk * H + h) * DH + dh) * 32 + 16 * hi;
        stnt16(dst, o0);
        stnt16(dst + 8, o1);
      }
    }
  }
  if (hl.clock && blockIdx.x < 8 && tid == 0) {
    hl.clock[blockIdx.x * 4 + 2] = __builtin_amdgcn_s_memtime();
    hl.clock[blockIdx.x * 4 + 3] = __builtin_amdgcn_s_memrealtime();
  }
}

}  // namespace

hipError_t launch_hist128(const ChainArgs &a, const HistLayers &hl, hipStream_t s) {
  if (a.n_rows <= 0 || hl.M <= 0) return hipSuccess;
  if (a.d != kD || hl.M > kMaxLayers || a.hidden % kHC || a.in_mode != IN_GATHER_CSR)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.n_rows + kR - 1) / kR)), block(kT);
  if (a.ln) hipLaunchKernelGGL(hist128_kernel<true>, grid, block, 0, s, a, hl);
  else hipLaunchKernelGGL(hist128_kernel<false>, grid, block, 0, s, a, hl);
  return hipGetLastError();
}

}  // namespace stca
