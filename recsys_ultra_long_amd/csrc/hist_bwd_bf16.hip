// hist_bwd_bf16.hip -- backward of one layer of the d = 256 history encoder
// (bf16) on 128-row tiles, in one launch ([Notes] §STCA history encoding,
// each step's derivative written out):
//   recompute   H1 = X W1, H3 = X W3, G = SiLU(H1) * H3, Y = G W2,
//               X~ = LN(Y) (x^ = (Y - mean) rstd, X~ = x^ gain + bias)
//   dX~ = dK W_K^T + dV W_V^T
//   LN          dY = rstd (gain dX~ - mean_f(gain dX~) - x^ mean_f(gain dX~ x^)),
//               per-tile sums over the rows of dX~ x^ (gain) and dX~ (bias)
//   SwiGLU      dG = dY W2^T, dH1 = dG H3 SiLU'(H1), dH3 = dG SiLU(H1)
//   rows        dX (+)= dH1 W1^T + dH3 W3^T
// X~, G, dY and dH1 | dH3 go to HBM as the operands of the weight-gradient
// products (sums over all rows, run afterwards as split-K GEMMs).
//
// Shape (the encoder's, hist_bf16.hip): 8 waves split the *outputs* of every
// contraction so that each weight fragment a wave streams from L2 feeds all
// 128 rows; weights are consumed as one chain of phases through the 4-slot
// register ring.  Per tile:
//   A  the encoder's FFN over hidden chunks of 128 (wave w: units 16w.. of a
//      chunk on 16x16x32; Y^T on 32x32x16, features 32w..), LN statistics;
//      H1, H3 to a scratch in lane order (they come back in phase C);
//   B  dX~^T = [W_K | W_V] [dK | dV]^T from the dK | dV rows staged in LDS
//      (wave w: features 32w.., the same lanes as Y), then the LN backward
//      in registers; dY staged in LDS;
//   C  per hidden chunk: dG^T (16x16x32, the lanes of phase A's H), the
//      SwiGLU derivative, dH1 | dH3 staged in LDS, dX^T += (32x32x16).
// LDS: region P (X, then dY) and region Q (two G chunks, then the dH chunk);
// the dK | dV rows span both.  Phase C cannot keep X as well (P + Q + X is
// over the 160 KB), hence H1, H3 through the scratch instead of a recompute.
#include <algorithm>

#include "grad_internal.h"
#include "hist_common.h"

namespace stca {
namespace {

using enc::Ring;
using enc::Src;
using enc::ring_load;
using enc::run_phase;
using enc::zero16;
using enc::zero4;

constexpr int kD = 256;
constexpr int kT = 512;          // 8 waves
constexpr int kR = 128;          // rows per tile
constexpr int kHC = 128;         // hidden units per chunk (16 per wave)
// LDS row strides (elements) by read pattern, as in the encoder: rows read as
// the 16x16x32 B operand at 544 bytes, as the 32x32x16 B operand at 16 mod
// 256 bytes.
constexpr int kXRLD = kD + 16;     // X
constexpr int kGLD = kHC + 8;      // G chunk
constexpr int kKVLD = 2 * kD + 8;  // dK | dV
constexpr int kYLD = kD + 16;      // dY
constexpr int kHLD = 2 * kHC + 8;  // dH1 | dH3 chunk

constexpr int kRegionP = kR * kXRLD * 2;     // bytes
constexpr int kRegionQ = 2 * kR * kGLD * 2;
static_assert(kR * kYLD * 2 <= kRegionP, "dY fits region P");
static_assert(kR * kHLD * 2 <= kRegionQ, "the dH chunk fits region Q");
static_assert(kR * kKVLD * 2 <= kRegionP + kRegionQ, "dK | dV fit P and Q");

struct Smem {
  __attribute__((aligned(16))) unsigned char pq[kRegionP + kRegionQ];
  float red[2][8][kR];
  __attribute__((aligned(16))) float lnp[2][kD];  // LN gain, bias
};

typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const u32x2 gu32x2;

// Per-wave weight streams of each phase (layouts: grad_internal.h).
struct Ops {
  const bf16_t *w1, *w3, *w2, *wkv, *w2t, *w13;
};
// A: W1, W3 rows of the wave's 16 units of chunk hc, k blocks of 32 features
DEV Src src_g(const Ops &L, int hc, int w, int lane) {
  const int64_t o = (int64_t)((hc * 8 + w) * (kD / 32)) * 512 + lane * 8;
  return Src{L.w1 + o, L.w3 + o, 512};
}
// A: W2^T rows of features 32w.., k blocks of chunk hc's units
DEV Src src_y(const Ops &L, int hc, int w, int lane, int nkh) {
  const bf16_t *p = L.w2 + frag_off(w, hc * (kHC / 32), nkh, 0, lane);
  return Src{p, p + 512, 1024};
}
// B: W_K, W_V rows of features 32w.., their k blocks interleaved (16 blocks)
DEV Src src_b(const Ops &L, int w, int lane) {
  const bf16_t *p = L.wkv + (int64_t)w * (kD / 32) * 2048 + lane * 8;
  return Src{p, p + 512, 1024};
}
// C: W2 rows of the wave's 16 units of chunk hc, two k blocks per ring slot
DEV Src src_dg(const Ops &L, int hc, int w, int lane) {
  const bf16_t *p = L.w2t + (int64_t)((hc * 8 + w) * (kD / 32)) * 512 + lane * 8;
  return Src{p, p + 512, 1024};
}
// C: W1, W3 rows of features 32w.., chunk hc's unit blocks, W1 / W3 alternating
DEV Src src_dx(const Ops &L, int hc, int w, int lane, int nkh) {
  const bf16_t *p = L.w13 + (((int64_t)w * nkh + hc * (kHC / 32)) * 2) * 1024 + lane * 8;
  return Src{p, p + 512, 1024};
}

// Rows row0 .. row0 + 127 of a [*, W] bf16 matrix into LDS (row stride LD),
// zeros past nrows (row0 < nrows).  Every load is issued unconditionally
// (rows past the end read row0 and are replaced by zeros afterwards), so that
// all of them are in flight together.  All threads; the caller synchronises.
template <int W>
struct Rows {
  static constexpr int C8 = W / 8, N = kR * C8 / kT;
  static_assert(N * kT == kR * C8, "whole 16-byte pieces per thread");
  u32x4 v[N];
  DEV void load(const bf16_t *src, int64_t row0, int64_t nrows, int tid) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int e = tid + k * kT, r = e / C8, c = (e % C8) * 8;
      const int64_t row = row0 + r < nrows ? row0 + r : row0;
      v[k] = *(gu32x4 *)(src + row * W + c);
    }
  }
  template <int LD>
  DEV void store(bf16_t *dst, int64_t row0, int64_t nrows, int tid) const {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int e = tid + k * kT, r = e / C8, c = (e % C8) * 8;
      const uint32_t keep = row0 + r < nrows ? 0xffffffffu : 0u;
      *reinterpret_cast<u32x4 *>(dst + r * LD + c) = v[k] & keep;
    }
  }
};
template <int W, int LD>
DEV void load_rows(const bf16_t *src, bf16_t *dst, int64_t row0, int64_t nrows, int tid) {
  Rows<W> rw;
  rw.load(src, row0, nrows, tid);
  rw.template store<LD>(dst, row0, nrows, tid);
}

DEV float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Sum over the 32 lanes of each half-wave, in every lane: four DPP steps
// within rows of 16 (pairs, quads, half-row and row mirrors) and one swap
// between the rows -- VALU only, no LDS round trips.
DEV float dpp_add(float v, int ctrl) {
  switch (ctrl) {  // the control must be a constant of the builtin
    case 0xB1: return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    case 0x4E: return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    case 0x141: return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    default: return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
  }
}
DEV float sum32_lanes(float v) {
  v = dpp_add(v, 0xB1);   // quad_perm [1,0,3,2]: pairs
  v = dpp_add(v, 0x4E);   // quad_perm [2,3,0,1]: quads
  v = dpp_add(v, 0x141);  // row_half_mirror: 8 lanes
  v = dpp_add(v, 0x140);  // row_mirror: 16 lanes
  return sum_x16(v);      // with the other row of the half-wave
}

template <bool LN>
__global__ __launch_bounds__(kT, 1) void hist_bwd256_kernel(HistBwdArgs a) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, w = tid >> 6;
  // Lane roles (32x32: l32, hi; 16x16: c16, g16), re-derived at each phase
  // boundary through an opaque copy of the thread index, so that no address
  // computed from them is held across phases (the live ranges of the
  // accumulators leave no room for it).
  int lane, l32, hi, c16, g16;
  auto roles = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    lane = t & 63;
    l32 = lane & 31;
    hi = lane >> 5;
    c16 = lane & 15;
    g16 = lane >> 4;
  };
  roles();
  const int tile = blockIdx.x;
  const int64_t row0 = (int64_t)tile * kR;
  int64_t nrows = a.R;
  if (a.dev_rows) nrows = min(nrows, (int64_t)*a.dev_rows);
  float *const part = LN ? a.ln_part + (int64_t)tile * 2 * kD : nullptr;
  if (row0 >= nrows) {  // past the device count: a zero partial for the fold
    if (LN) part[tid] = 0.f;
    return;
  }
  const int h = a.hidden, nkh = h / 32, nchunk = h / kHC;
  const Ops L{a.w1p, a.w3p, a.w2p, a.wkvt, a.w2t, a.w13t};
  bf16_t *const regP = reinterpret_cast<bf16_t *>(sm.pq);
  bf16_t *const regQ = reinterpret_cast<bf16_t *>(sm.pq + kRegionP);
  bf16_t *const xs = regP;
  auto gs = [&](int hc) { return regQ + (hc & 1) * kR * kGLD; };  // G chunk buffers
  bf16_t *const kvs = regP;  // spans P and Q
  bf16_t *const dys = regP;
  bf16_t *const dhs = regQ;
  bf16_t *const hs_tile = a.hs + (int64_t)tile * nchunk * (8 * 8 * 512);

  Ring ring;
  {
    const Src s0 = src_g(L, 0, w, lane);
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) ring_load(ring, kb, s0, kb);
  }
  load_rows<kD, kXRLD>(a.x, xs, row0, nrows, tid);
  if (LN) sm.lnp[tid >> 8][tid & 255] = (tid < kD ? a.ln_g : a.ln_b)[tid & 255];
  __syncthreads();

  // ================================================================ A
  // Y^T: lane holds features 32w + c32_row(lane, i) of tokens 32j + l32
  f32x16 y[4];
  zero16(y);
  {
    const bf16_t *const xrow = xs + c16 * kXRLD + g16 * 8;
    f32x4 acc[2][8];  // H1^T, H3^T of one chunk: the wave's 16 units x 128 tokens
    auto g_mma = [&](int hc, const Src &nxt) {
      zero4(acc[0]);
      zero4(acc[1]);
      run_phase<kD / 32>(ring, src_g(L, hc, w, lane), nxt, true, [&](int kb, int slot) {
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += 4) {
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
    // lane: units 4 g16 + i of the wave's 16, token 16 t + c16.  G to LDS
    // (for Y; copy_g takes it on to HBM); H1, H3 to the scratch in lane order.
    auto silu_store = [&](int hc, int t) {
      float gv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gv[i] = silu_fast(acc[0][t][i]) * acc[1][t][i];
      const u32x2 gp = {pack_bf2(gv[0], gv[1]), pack_bf2(gv[2], gv[3])};
      const int tok = t * 16 + c16;
      *reinterpret_cast<u32x2 *>(gs(hc) + tok * kGLD + w * 16 + 4 * g16) = gp;
      bf16_t *hp = hs_tile + ((hc * 8 + w) * 8 + t) * 512 + lane * 4;
      const u32x2 h1 = {pack_bf2(acc[0][t][0], acc[0][t][1]), pack_bf2(acc[0][t][2], acc[0][t][3])};
      const u32x2 h3 = {pack_bf2(acc[1][t][0], acc[1][t][1]), pack_bf2(acc[1][t][2], acc[1][t][3])};
      *reinterpret_cast<u32x2 *>(hp) = h1;
      *reinterpret_cast<u32x2 *>(hp + 256) = h3;
    };
    // Y^T += W2^T[features 32w.., chunk hc] G^T[chunk, tokens]; with
    // hn >= 0, also chunk hn's SiLU epilogue (two row tiles per block)
    auto y_mma = [&](int hc, const Src &nxt, int hn) {
      const bf16_t *g = gs(hc);
      run_phase<kHC / 32>(ring, src_y(L, hc, w, lane, nkh), nxt, true, [&](int kb, int slot) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 bg[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) bg[j] = ld8(g + (j * 32 + l32) * kGLD + kb * 32 + hi * 16 + hh * 8);
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = mfma32(ring.v[slot][hh], bg[j], y[j]);
        }
        if (hn >= 0) {
          silu_store(hn, 2 * kb);
          silu_store(hn, 2 * kb + 1);
        }
      });
    };
    // a staged G chunk to HBM for dW2: 16-byte pieces of whole 256-byte rows
    auto copy_g = [&](int hc) {
      const bf16_t *g = gs(hc);
      int ti = tid;  // opaque: no address of the copy is held across the loop
      asm volatile("" : "+v"(ti));
#pragma unroll
      for (int k = 0; k < kR * (kHC / 8) / kT; ++k) {
        const int e = ti + k * kT, r = e / (kHC / 8), c = (e % (kHC / 8)) * 8;
        if (row0 + r < nrows)
          *reinterpret_cast<u32x4 *>(a.g + (row0 + r) * h + hc * kHC + c) =
              *reinterpret_cast<const u32x4 *>(g + r * kGLD + c);
      }
    };
    g_mma(0, nchunk > 1 ? src_g(L, 1, w, lane) : src_y(L, 0, w, lane, nkh));
#pragma unroll
    for (int t = 0; t < 8; ++t) silu_store(0, t);
    __syncthreads();
    copy_g(0);
#pragma unroll 1
    for (int hc = 1; hc < nchunk; ++hc) {
      roles();
      g_mma(hc, src_y(L, hc - 1, w, lane, nkh));
      y_mma(hc - 1, hc + 1 < nchunk ? src_g(L, hc + 1, w, lane) : src_y(L, hc, w, lane, nkh), hc);
      __syncthreads();
      copy_g(hc);
    }
    y_mma(nchunk - 1, src_b(L, w, lane), -1);
  }
  // the tile's dK | dV rows: loads issued now (after the weight stream's last
  // loads of phase A), stored to LDS once every wave is done with X and G
  Rows<2 * kD> kvrows;
  kvrows.load(a.dkv, row0, nrows, tid);

  roles();
  // LN statistics (the encoder's single exchange: per-lane partial mean and
  // squared deviations, merged pairwise across the half-waves and waves)
  float mean[4], rstd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mean[j] = 0.f;
    rstd[j] = 1.f;
  }
  if (LN) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s1 += y[j][i];
      const float m16 = s1 * (1.0f / 16);
      float m2 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m2 += (y[j][i] - m16) * (y[j][i] - m16);
      uint32_t ma = __float_as_uint(m16), mb = ma, qa = __float_as_uint(m2), qb = qa;
      swap32(ma, mb);
      swap32(qa, qb);
      const float dm = __uint_as_float(ma) - __uint_as_float(mb);
      if (hi == 0) {
        sm.red[0][w][j * 32 + l32] = 0.5f * (__uint_as_float(ma) + __uint_as_float(mb));
        sm.red[1][w][j * 32 + l32] = __uint_as_float(qa) + __uint_as_float(qb) + 8.0f * dm * dm;
      }
    }
  }
  __syncthreads();  // (also: every wave is done with X and the G chunks)
  kvrows.store<kKVLD>(kvs, row0, nrows, tid);  // over P and Q
  if (LN) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = j * 32 + l32;
      float mq[8], tot = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        mq[q] = sm.red[0][q][t];
        tot += mq[q];
      }
      const float mu = tot * (1.0f / 8);
      float m2 = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) m2 += sm.red[1][q][t] + 32.0f * (mq[q] - mu) * (mq[q] - mu);
      mean[j] = mu;
      rstd[j] = rsqrtf(m2 * (1.0f / kD) + 1e-5f);
    }
  }
  // X~ to HBM; y becomes x^ (LN) for the backward
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = w * 32 + 8 * q + 4 * hi;
    f32x4 gg = {1.f, 1.f, 1.f, 1.f}, bb = {0.f, 0.f, 0.f, 0.f};
    if (LN) {
      gg = *reinterpret_cast<const f32x4 *>(&sm.lnp[0][f]);
      bb = *reinterpret_cast<const f32x4 *>(&sm.lnp[1][f]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (LN) y[j][4 * q + r] = (y[j][4 * q + r] - mean[j]) * rstd[j];
        v[r] = LN ? y[j][4 * q + r] * gg[r] + bb[r] : y[j][4 * q + r];
      }
      const int64_t row = row0 + j * 32 + l32;
      if (row < nrows)
        *reinterpret_cast<u32x2 *>(a.xt + row * kD + f) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
    }
  }
  __syncthreads();  // dK | dV staged

  // ================================================================ B
  roles();
  // dX~^T: lane holds features 32w + c32_row(lane, i) of tokens 32j + l32
  f32x16 dxt[4];
  zero16(dxt);
  run_phase<2 * kD / 32>(ring, src_b(L, w, lane), src_dg(L, 0, w, lane), true, [&](int b, int slot) {
    const int col = (b & 1) * kD + (b >> 1) * 32 + hi * 16;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      bf16x8 bk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bk[j] = ld8(kvs + (j * 32 + l32) * kKVLD + col + hh * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) dxt[j] = mfma32(ring.v[slot][hh], bk[j], dxt[j]);
    }
  });

  // LN backward (y holds x^): dY = rstd (gy - mean_f gy - x^ mean_f(gy x^)),
  // gy = gain dX~; gain / bias partials of the tile
  if (LN) {
    float gam[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 gg = *reinterpret_cast<const f32x4 *>(&sm.lnp[0][w * 32 + 8 * q + 4 * hi]);
#pragma unroll
      for (int r = 0; r < 4; ++r) gam[4 * q + r] = gg[r];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float p1 = 0.f, p2 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float gy = dxt[j][i] * gam[i];
        p1 += gy;
        p2 += gy * y[j][i];
      }
      p1 = sum_x32(p1);  // with the other 16 features of the wave's 32
      p2 = sum_x32(p2);
      if (hi == 0) {
        sm.red[0][w][j * 32 + l32] = p1;
        sm.red[1][w][j * 32 + l32] = p2;
      }
    }
    // gain and bias sums over the tile's 128 tokens (lanes l32, then j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float pg = 0.f, pb = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pg += dxt[j][i] * y[j][i];
        pb += dxt[j][i];
      }
      pg = sum32_lanes(pg);
      pb = sum32_lanes(pb);
      if (l32 == 0) {
        const int f = w * 32 + c32_row(lane, i);
        part[f] = pg;
        part[kD + f] = pb;
      }
    }
  }
  __syncthreads();  // the statistics are in; every wave is done with dK | dV
  float s1[4] = {0.f, 0.f, 0.f, 0.f}, s2[4] = {0.f, 0.f, 0.f, 0.f};
  if (LN) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = j * 32 + l32;
      float a1 = 0.f, a2 = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        a1 += sm.red[0][q][t];
        a2 += sm.red[1][q][t];
      }
      s1[j] = a1 * (1.0f / kD);
      s2[j] = a2 * (1.0f / kD);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = w * 32 + 8 * q + 4 * hi;
    f32x4 gg = {1.f, 1.f, 1.f, 1.f};
    if (LN) gg = *reinterpret_cast<const f32x4 *>(&sm.lnp[0][f]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float dv = dxt[j][4 * q + r];
        v[r] = LN ? rstd[j] * (dv * gg[r] - s1[j] - y[j][4 * q + r] * s2[j]) : dv;
      }
      const u32x2 pv = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
      const int tok = j * 32 + l32;
      *reinterpret_cast<u32x2 *>(dys + tok * kYLD + f) = pv;
      if (row0 + tok < nrows) *reinterpret_cast<u32x2 *>(a.dy + (row0 + tok) * kD + f) = pv;
    }
  }
  __syncthreads();  // dY staged

  // ================================================================ C
  roles();
  // dX^T: lane holds features 32w + c32_row(lane, i) of tokens 32j + l32
  f32x16 dx[4];
  zero16(dx);
  const bf16_t *const yrow = dys + c16 * kYLD + g16 * 8;
  // H1, H3 of the wave's units of a chunk, as phase A left them; loaded a
  // chunk ahead
  u32x2 hv[8][2];
  auto load_h = [&](int hc) {
    const bf16_t *hp = hs_tile + ((hc * 8 + w) * 8) * 512 + lane * 4;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      hv[t][0] = *(gu32x2 *)(hp + t * 512);
      hv[t][1] = *(gu32x2 *)(hp + t * 512 + 256);
    }
  };
  load_h(0);
#pragma unroll 1
  for (int hc = 0; hc < nchunk; ++hc) {
    roles();
    // dG^T = W2[units, :] dY^T (lanes as H)
    f32x4 dg[8];
    zero4(dg);
    run_phase<kD / 64>(ring, src_dg(L, hc, w, lane), src_dx(L, hc, w, lane, nkh), true, [&](int s, int slot) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += 4) {
          bf16x8 by[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) by[t] = ld8(yrow + (t0 + t) * 16 * kYLD + (2 * s + kk) * 32);
#pragma unroll
          for (int t = 0; t < 4; ++t) dg[t0 + t] = mfma16(ring.v[slot][kk], by[t], dg[t0 + t]);
        }
    });
    if (hc > 0) __syncthreads();  // every wave is done reading the previous dH chunk
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float d1[4], d3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w1 = hv[t][0][i >> 1], w3 = hv[t][1][i >> 1];
        const float u = __uint_as_float((i & 1) ? (w1 & 0xffff0000u) : (w1 << 16));
        const float v = __uint_as_float((i & 1) ? (w3 & 0xffff0000u) : (w3 << 16));
        const float sg = sigmoid_fast(u);
        d1[i] = dg[t][i] * v * sg * (1.0f + u * (1.0f - sg));
        d3[i] = dg[t][i] * u * sg;
      }
      const u32x2 p1 = {pack_bf2(d1[0], d1[1]), pack_bf2(d1[2], d1[3])};
      const u32x2 p3 = {pack_bf2(d3[0], d3[1]), pack_bf2(d3[2], d3[3])};
      const int tok = t * 16 + c16, u0 = w * 16 + 4 * g16;
      *reinterpret_cast<u32x2 *>(dhs + tok * kHLD + u0) = p1;
      *reinterpret_cast<u32x2 *>(dhs + tok * kHLD + kHC + u0) = p3;
      if (row0 + tok < nrows) {
        bf16_t *dst = a.dh13 + (row0 + tok) * 2 * h + hc * kHC + u0;
        *reinterpret_cast<u32x2 *>(dst) = p1;
        *reinterpret_cast<u32x2 *>(dst + h) = p3;
      }
    }
    if (hc + 1 < nchunk) load_h(hc + 1);
    __syncthreads();  // the dH chunk is staged
    // dX^T += [W1 | W3][features, chunk units] [dH1 | dH3]^T
    const bool more = hc + 1 < nchunk;
    const Src nxt = more ? src_dg(L, hc + 1, w, lane) : src_dx(L, hc, w, lane, nkh);
    run_phase<2 * kHC / 32>(ring, src_dx(L, hc, w, lane, nkh), nxt, more, [&](int b, int slot) {
      const int col = (b & 1) * kHC + (b >> 1) * 32 + hi * 16;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 bh[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bh[j] = ld8(dhs + (j * 32 + l32) * kHLD + col + hh * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) dx[j] = mfma32(ring.v[slot][hh], bh[j], dx[j]);
      }
    });
  }
  // dX rows (fp32): 16-byte pieces, 128 bytes of a row per wave; with
  // accumulation every old value is loaded first (rows past the end read
  // row0 and are not written)
  f32x4 old[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) old[j][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.dx_acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = row0 + j * 32 + l32 < nrows ? row0 + j * 32 + l32 : row0;
#pragma unroll
      for (int q = 0; q < 4; ++q) old[j][q] = ldg4(a.dx + row * kD + w * 32 + 8 * q + 4 * hi);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t row = row0 + j * 32 + l32;
    if (row >= nrows) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = {dx[j][4 * q] + old[j][q][0], dx[j][4 * q + 1] + old[j][q][1],
                       dx[j][4 * q + 2] + old[j][q][2], dx[j][4 * q + 3] + old[j][q][3]};
      *reinterpret_cast<f32x4 *>(a.dx + row * kD + w * 32 + 8 * q + 4 * hi) = v;
    }
  }
}

}  // namespace

hipError_t launch_hist_bwd256(const HistBwdArgs &a, hipStream_t s) {
  if (a.R <= 0) return hipSuccess;
  if (!hist_bwd256_ok(kD, a.hidden) || !a.x || !a.dkv || !a.hs || !a.dx || (a.ln && (!a.ln_part || !a.ln_g)))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)hist_bwd_tiles(a.R)), block(kT);
  if (a.ln) hipLaunchKernelGGL(hist_bwd256_kernel<true>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(hist_bwd256_kernel<false>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace stca
