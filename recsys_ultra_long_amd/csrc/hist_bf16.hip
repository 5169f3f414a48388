// hist_bf16.hip -- history encoder for d = 256 (bf16): every layer's
//   X~ = [LN](SwiGLU(X)) = [LN]((SiLU(X W1) * (X W3)) W2),  K = X~ W_K, V = X~ W_V
// ([Notes] §STCA; [Review] architecture tree) over 128-row tiles of the
// padded history, all M layers per launch on one gathered tile.
//
// Why this shape.  The encoder's weights (1 MB per layer) do not fit on chip,
// so every row tile streams all of them from L2; with 64-row tiles that
// stream is the bound (the vector-memory data path, not the matrix cores).
// Here a workgroup of 8 waves (one per CU, two per SIMD) takes 128 rows and
// splits the *outputs* of each contraction over its waves, so every weight
// fragment a wave loads feeds all 128 rows:
//   G   = SiLU(X W1) * (X W3)  : wave w owns hidden units 16w .. 16w+15 of each
//                                128-unit chunk (16x16x32 MFMA, 8 row tiles)
//   Y^T += W2^T G^T            : wave w owns features 32w .. 32w+31 (32x32x16)
//   K^T  = W_K^T X~^T, V = X~ W_V : wave w owns features 32w .. 32w+31
// Weights are consumed as a fixed chain of phases whose 32-wide k blocks
// stream through a 4-slot register ring kept three blocks ahead, across phase
// (and layer) boundaries.  LDS: the raw rows (kept for all layers), two G
// chunk buffers which, after the FFN, hold the LN output for the projection.
#include <algorithm>

#include "attn_block.h"
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

constexpr int kD = 256;
constexpr int kT = 512;          // threads: 8 waves
constexpr int kR = 128;          // rows per tile
constexpr int kHC = 128;         // hidden units per chunk (16 per wave)
constexpr int kXLD = kD + 8;     // LDS row stride of X~ (elements)
// Row strides are chosen per read pattern: on gfx950 16-byte LDS reads of
// 16 rows x 4 column groups (the 16x16x32 B operand) are conflict-free at a
// 544-byte stride but not at 528; 32 rows x 2 groups (32x32x16) the reverse.
constexpr int kXRLD = kD + 16;   // LDS row stride of the raw rows X (G phase)
constexpr int kGLD = kHC + 8;    // LDS row stride of a G chunk

struct Smem {
  __attribute__((aligned(16))) bf16_t xs[kR * kXRLD];
  __attribute__((aligned(16))) bf16_t gs[2][kR * kGLD];
  float red[2][8][kR];
  int s_id[kR], s_tok[kR];
};
static_assert(sizeof(Smem::gs) >= sizeof(bf16_t) * kR * kXLD, "LN output must fit the G buffers");

// Per-wave weight sources of each phase.  W1/W3 are packed for the 16x16x32
// A operand (frag16), W2 and W_K|W_V for the 32x32x16 A operand (frag_off).
struct Layer {
  const bf16_t *w1, *w3, *w2, *wp;
  const float *ln_g, *ln_b;
  bf16_t *kb, *vb;
};
DEV Src src_g(const Layer &L, int hc, int w, int lane) {
  const int64_t o = (int64_t)((hc * 8 + w) * (kD / 32)) * 512 + lane * 8;
  return Src{L.w1 + o, L.w3 + o, 512};
}
DEV Src src_y(const Layer &L, int hc, int w, int lane, int nkh) {
  const bf16_t *p = L.w2 + frag_off(w, hc * (kHC / 32), nkh, 0, lane);
  return Src{p, p + 512, 1024};
}
// W_K and W_V are packed with their k blocks interleaved (K0, V0, K1, V1, ..
// for each 32-feature tile): one stream for both, or every other block.
DEV Src src_kv(const Layer &L, int w, int lane) {
  const bf16_t *p = L.wp + (int64_t)w * (kD / 32) * 2048 + lane * 8;
  return Src{p, p + 512, 1024};
}
DEV Src src_k(const Layer &L, int w, int lane) {
  const bf16_t *p = L.wp + (int64_t)w * (kD / 32) * 2048 + lane * 8;
  return Src{p, p + 512, 2048};
}
DEV Src src_v(const Layer &L, int w, int lane) {
  const bf16_t *p = L.wp + (int64_t)w * (kD / 32) * 2048 + 1024 + lane * 8;
  return Src{p, p + 512, 2048};
}

// Gather the 128 table rows of a tile into sm.xs (see enc::gather_tile).
DEV void gather_tile(const ChainArgs &a, Smem &sm, int64_t row0, int total_blocks, int tid, bool use_prow) {
  enc::gather_tile<kD, kR, kXRLD, kT>(a, sm.xs, sm.s_id, sm.s_tok, row0, total_blocks, tid, use_prow);
}

// SwiGLU FFN [+ LN] of one layer over the 128 rows in sm.xs; X~ goes to
// `xt` (row stride kXLD: over the rows themselves, or into the G buffers when
// the rows must survive for another layer).  The ring enters holding the
// first blocks of G chunk 0 and leaves holding those of `after` (the
// projection's weight stream); X~ is visible to every thread on return.
template <bool LN, bool PIPE>
DEV void ffn_ln(Ring &ring, const Layer &L, Smem &sm, bf16_t *xt, int w, int lane, int nkh, int nchunk,
                const Src &after) {
  const int l32 = lane & 31, hi = lane >> 5;
  const int c16 = lane & 15, g16 = lane >> 4;
  const bf16_t *const xrow = sm.xs + c16 * kXRLD + g16 * 8;  // G-phase operand base
  // ------------------------------------------------------------ SwiGLU FFN
  // PIPE: software-pipelined over hidden chunks: the products of chunk hc's
  // G tiles, then chunk hc - 1's Y products with chunk hc's SiLU epilogue
  // (VALU) interleaved among them, then one barrier.  Order of weight
  // phases: G0 | G1, Y0 | G2, Y1 | ... | Y(last).  Otherwise (fewer live
  // registers, for the fused kernel): G(hc), its SiLU, a barrier, Y(hc).
  f32x16 y[4];  // Y^T: features 32w .., tokens 32j + l32
  zero16(y);
  f32x4 acc[2][8];  // G^T of one chunk: W1 and W3 rows of this wave's 16 units x 128 tokens
  // Operands from LDS in groups of four fragments: one group is read while
  // the other group's products run.  `opa` holds the first group of a phase;
  // a phase's last block reads the first group of the phase that follows
  // (code `nf`: 0 = a G phase, 1 + c = the Y phase of chunk c; -1 = none),
  // so that no phase starts on an LDS round trip.
  bf16x8 opa[4], opb[4];
  auto load_first = [&](int nf) {
    if (nf == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) opa[t] = ld8(xrow + t * 16 * kXRLD);
    } else if (nf > 0) {
      const bf16_t *g = sm.gs[(nf - 1) & 1] + l32 * kGLD + hi * 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) opa[j] = ld8(g + j * 32 * kGLD);
    }
  };
  // G: row tiles 0..3 (opa) and 4..7 (opb) of each k block
  auto g_mma = [&](int hc, const Src &nxt, bool have, int nf) {
    zero4(acc[0]);
    zero4(acc[1]);
    constexpr int NK = kD / 32;
    if constexpr (!PIPE) {  // (the fused kernel: no registers to spare)
      run_phase<NK>(ring, src_g(L, hc, w, lane), nxt, true, [&](int kb, int slot) {
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += 4) {
#pragma unroll
          for (int t = 0; t < 4; ++t) opa[t] = ld8(xrow + (t0 + t) * 16 * kXRLD + kb * 32);
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[f][t0 + t] = mfma16(ring.v[slot][f], opa[t], acc[f][t0 + t]);
        }
      });
      return;
    }
    if (!have) load_first(0);
    run_phase<NK>(ring, src_g(L, hc, w, lane), nxt, true, [&](int kb, int slot) {
#pragma unroll
      for (int t = 0; t < 4; ++t) opb[t] = ld8(xrow + (4 + t) * 16 * kXRLD + kb * 32);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[f][t] = mfma16(ring.v[slot][f], opa[t], acc[f][t]);
      if (kb + 1 < NK) {
#pragma unroll
        for (int t = 0; t < 4; ++t) opa[t] = ld8(xrow + t * 16 * kXRLD + (kb + 1) * 32);
      } else {
        load_first(nf);
      }
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[f][4 + t] = mfma16(ring.v[slot][f], opb[t], acc[f][4 + t]);
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
  // Y^T += W2^T[features 32w.., chunk hc] G^T[chunk, tokens]: the two k
  // halves of each block (opa, opb); with `gnext`, also the SiLU epilogue of
  // the chunk in acc (two row tiles per block)
  auto y_mma = [&](int hc, const Src &nxt, bf16_t *gnext, bool have, int nf) {
    constexpr int NK = kHC / 32;
    const bf16_t *g = sm.gs[hc & 1] + l32 * kGLD + hi * 16;
    if constexpr (!PIPE) {
      run_phase<NK>(ring, src_y(L, hc, w, lane, nkh), nxt, true, [&](int kb, int slot) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int j = 0; j < 4; ++j) opa[j] = ld8(g + j * 32 * kGLD + kb * 32 + h * 8);
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = mfma32(ring.v[slot][h], opa[j], y[j]);
        }
      });
      return;
    }
    if (!have) load_first(1 + hc);
    run_phase<NK>(ring, src_y(L, hc, w, lane, nkh), nxt, true, [&](int kb, int slot) {
#pragma unroll
      for (int j = 0; j < 4; ++j) opb[j] = ld8(g + j * 32 * kGLD + kb * 32 + 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = mfma32(ring.v[slot][0], opa[j], y[j]);
      if (kb + 1 < NK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) opa[j] = ld8(g + j * 32 * kGLD + (kb + 1) * 32);
      } else {
        load_first(nf);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = mfma32(ring.v[slot][1], opb[j], y[j]);
      if (gnext) {
        silu_store(gnext, 2 * kb);
        silu_store(gnext, 2 * kb + 1);
      }
    });
  };
  static_assert(kHC / 32 * 2 == 8, "two row tiles of the SiLU epilogue per Y block");
  if (PIPE) {
    // G(hc) reads the first group of Y(hc - 1) (written before the last
    // barrier); Y(hc - 1) that of G(hc + 1) (the raw rows never change).
    g_mma(0, nchunk > 1 ? src_g(L, 1, w, lane) : src_y(L, 0, w, lane, nkh), false, nchunk > 1 ? 0 : -1);
#pragma unroll
    for (int t = 0; t < 8; ++t) silu_store(sm.gs[0], t);
    __syncthreads();
#pragma unroll 1
    for (int hc = 1; hc < nchunk; ++hc) {
      g_mma(hc, src_y(L, hc - 1, w, lane, nkh), true, hc);
      y_mma(hc - 1, hc + 1 < nchunk ? src_g(L, hc + 1, w, lane) : src_y(L, hc, w, lane, nkh), sm.gs[hc & 1], true,
            hc + 1 < nchunk ? 0 : -1);
      __syncthreads();
    }
    y_mma(nchunk - 1, after, nullptr, false, -1);
  } else {
#pragma unroll 1
    for (int hc = 0; hc < nchunk; ++hc) {
      g_mma(hc, src_y(L, hc, w, lane, nkh), false, -1);
#pragma unroll
      for (int t = 0; t < 8; ++t) silu_store(sm.gs[hc & 1], t);
      __syncthreads();
      y_mma(hc, hc + 1 < nchunk ? src_g(L, hc + 1, w, lane) : after, nullptr, false, -1);
    }
  }

  // ------------------------------------------------------------ LayerNorm
  // lane: features 32w + c32_row(lane, i) of tokens 32j + l32
  float mean[4], rstd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mean[j] = 0.f;
    rstd[j] = 1.f;
  }
  if (LN) {
    // Row statistics in one exchange: each lane's 16 values give a partial
    // (mean, sum of squared deviations), merged with the other half-wave and
    // then across the 8 waves by the pairwise formula
    //   M2 = M2_a + M2_b + (mean_a - mean_b)^2 n_a n_b / (n_a + n_b).
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
      swap32(ma, mb);  // ma: lower half-wave's partial, mb: upper's
      swap32(qa, qb);
      const float dm = __uint_as_float(ma) - __uint_as_float(mb);
      if (hi == 0) {
        sm.red[0][w][j * 32 + l32] = 0.5f * (__uint_as_float(ma) + __uint_as_float(mb));
        sm.red[1][w][j * 32 + l32] = __uint_as_float(qa) + __uint_as_float(qb) + 8.0f * dm * dm;
      }
    }
    __syncthreads();
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
  } else {
    __syncthreads();  // every wave is done reading the last G chunk
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = w * 32 + 8 * q + 4 * hi;
    f32x4 gg = {1.f, 1.f, 1.f, 1.f}, bb = {0.f, 0.f, 0.f, 0.f};
    if (LN) {
      gg = ldg4(L.ln_g + f);
      bb = ldg4(L.ln_b + f);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = y[j][4 * q + r];
        if (LN) v[r] = (v[r] - mean[j]) * rstd[j] * gg[r] + bb[r];
      }
      u32x2 pv = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
      *reinterpret_cast<u32x2 *>(xt + (j * 32 + l32) * kXLD + f) = pv;
    }
  }
  __syncthreads();

}

template <bool LN, bool PERSIST>
__global__ __launch_bounds__(kT, 1) void hist256_kernel(ChainArgs a, HistLayers hl) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;     // 32x32 operand / output roles
  const int c16 = lane & 15, g16 = lane >> 4;    // 16x16 roles
  const int total_blocks = a.plan.pblk[a.B];
  const int tiles = (total_blocks + 3) / 4;
  // Work units.  One workgroup per tile with all of its layers; or, PERSIST
  // (a grid of about one workgroup per CU, sized from an upper bound of the
  // rows: the unique rows of a batch are counted on the device), workgroups
  // looping over the units, a unit being one tile with all of its layers or,
  // when that would leave the last round of workgroups mostly idle, one
  // (tile, layer) pair.  Every row's arithmetic is the same in all three forms.
  int units = tiles, stride = tiles;
  bool split = false;
  if (PERSIST) {
    const int G = (int)gridDim.x;
    const int64_t r_all = (int64_t)((tiles + G - 1) / G) * hl.M, r_split = ((int64_t)tiles * hl.M + G - 1) / G;
    split = r_split < r_all;
    units = split ? tiles * hl.M : tiles;
    stride = G;
  }
  if ((int)blockIdx.x >= units) return;
  const int nkh = a.hidden / 32, nchunk = a.hidden / kHC;
  const int H = a.H, DH = kD / a.H;
  // optional clock probe: shader-clock and 100 MHz counters at start and end
  // (written at once, so that nothing is held across the layers)
  const bool probe = hl.clock && blockIdx.x < 8 && tid == 0;
  if (probe) {
    const unsigned long long clk0 = __builtin_amdgcn_s_memtime(), rt0 = __builtin_amdgcn_s_memrealtime();
    hl.clock[blockIdx.x * 4] = clk0;
    hl.clock[blockIdx.x * 4 + 1] = rt0;
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

  bf16_t *const xt = &sm.gs[0][0];  // LN output, row stride kXLD
  auto unit = [&](const int64_t row0, const int l0, const int l1) {
  Ring ring;
  {
    const Layer L0 = layer(l0);
    const Src s0 = src_g(L0, 0, w, lane);
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) ring_load(ring, kb, s0, kb);
  }

  gather_tile(a, sm, row0, total_blocks, tid, true);

#pragma unroll 1
  for (int li = l0; li < l1; ++li) {
    // lane quantities re-derived per layer so none is held across layers
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    const int lane = ltid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int c16 = lane & 15, g16 = lane >> 4;
    Layer L = layer(li);
    // the weight addresses stay loop-variant (no hoisting across layers)
    asm volatile("" : "+s"(L.w1), "+s"(L.w3), "+s"(L.w2), "+s"(L.wp), "+s"(L.ln_g), "+s"(L.ln_b));
    if (li > l0) __syncthreads();  // the previous layer's projection is done with X~

    ffn_ln<LN, true>(ring, L, sm, xt, w, lane, nkh, nchunk, src_kv(L, w, lane));

    // ------------------------------------------------------------ W_K | W_V
    // K^T = W_K^T X~^T and V = X~ W_V in one pass over the interleaved weight
    // stream (K0, V0, K1, V1, ..): the X~ operand of a k block is read once,
    // for both products.  After the exchange each lane holds 16 consecutive
    // features of one key (K) or 16 consecutive keys of one feature (V).
    {
      f32x16 ka[4], va[4];
      zero16(ka);
      zero16(va);
      bf16x8 bx[2][4];
      const bool more = li + 1 < l1;
      Src nxt = src_kv(L, w, lane);  // any valid address when nothing follows
      if (more) {
        const Layer Ln = layer(li + 1);
        nxt = src_g(Ln, 0, w, lane);
      }
      // X~ operands of k block kb + 1 are read while block kb's V products
      // run (each half once its V products are issued).
      const bf16_t *xo = xt + l32 * kXLD + hi * 16;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) bx[h][j] = ld8(xo + j * 32 * kXLD + h * 8);
      run_phase<2 * kD / 32>(ring, src_kv(L, w, lane), nxt, more, [&](int b, int slot) {
        const int kb = b >> 1;
        if ((b & 1) == 0) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) ka[j] = mfma32(ring.v[slot][h], bx[h][j], ka[j]);
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 4; ++j) va[j] = mfma32(bx[h][j], ring.v[slot][h], va[j]);
            if (kb + 1 < kD / 32) {
#pragma unroll
              for (int j = 0; j < 4; ++j) bx[h][j] = ld8(xo + j * 32 * kXLD + (kb + 1) * 32 + h * 8);
            }
          }
        }
      });
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = (int)(row0 >> 5) + j;
        if (blk >= total_blocks) continue;
        u32x4 o0, o1;
        halves16(ka[j], hi, o0, o1);
        const int f = w * 32 + 16 * hi;
        const int h = f / DH, dh = f % DH;
        bf16_t *dst = L.kb + (((int64_t)blk * H + h) * 32 + l32) * DH + dh;
        stnt16(dst, o0);
        stnt16(dst + 8, o1);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = (int)(row0 >> 5) + j;
        if (blk >= total_blocks) continue;
        u32x4 o0, o1;
        halves16(va[j], hi, o0, o1);
        const int f = w * 32 + l32;
        const int h = f / DH, dh = f % DH;
        bf16_t *dst = L.vb + (((int64_t)blk * H + h) * DH + dh) * 32 + 16 * hi;
        stnt16(dst, o0);
        stnt16(dst + 8, o1);
      }
    }
  }
  };
  if (!PERSIST) {
    unit((int64_t)blockIdx.x * kR, 0, hl.M);
  } else {
#pragma unroll 1
    for (int u = (int)blockIdx.x; u < units; u += stride) {
      if (u != (int)blockIdx.x) __syncthreads();  // the previous unit is done with the LDS
      const int l0 = split ? u / tiles : 0;
      unit((int64_t)(split ? u % tiles : u) * kR, l0, split ? l0 + 1 : hl.M);
    }
  }
  if (hl.clock && blockIdx.x < 8 && tid == 0) {
    const unsigned long long clk1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
    hl.clock[blockIdx.x * 4 + 2] = clk1;
    hl.clock[blockIdx.x * 4 + 3] = rt1;
  }
}


// ---------------------------------------------------------------- fused path
// "Lookup while computing" ([WeChat] §1.1) on the same 128-row structure: a
// persistent workgroup (one per CU) walks a contiguous range of 128-key tiles
// (users padded to whole tiles).  Per tile: gather, SwiGLU FFN, LN (over the
// rows), W_K into LDS over the G buffers (K rows padded), W_V into LDS over
// the rows once every wave has read them (V^T rows of 128 keys, the 16-byte
// chunks of row f XOR-swizzled by f mod 16 so that 16 consecutive features
// read at one key offset hit different banks), then each wave folds the
// tile's keys into the online-softmax (or ReLU) state of one head: d_h = 32,
// wave w = head w, all targets; d_h = 64, waves 2h and 2h + 1 = head h,
// targets 0..31 and 32..63.  No K/V tensor exists in HBM.  Between tiles of
// one user the state goes through the workgroup's state area (each lane reads
// back only what it wrote); at the user's last tile in the range it becomes a
// partial in slot (workgroup + user) -- distinct slots, fewer than grid + B,
// because ranges are contiguous and users ordered.
template <int DH, int NT, int SCORE, bool LN>
__global__ __launch_bounds__(kT, 1) void fused256_kernel(ChainArgs a, AttnArgs at) {
  constexpr int H = kD / DH;
  constexpr int WPH = 8 / H;            // waves per head
  constexpr int TPW = 64 / WPH;         // targets per wave
  constexpr int KS = DH / 32, DT = DH / 16;
  constexpr int REC = DT * NT + 3;      // f32x4 per lane: o, then m, l, count
  static_assert(NT * 16 <= TPW, "target tiles exceed the wave's share");
  __shared__ Smem sm;
  const int tid = threadIdx.x, w = tid >> 6;
  const Plan P = at.plan;
  const int tiles = P.pblk[at.B] / 4;
  const int per = (tiles + (int)gridDim.x - 1) / (int)gridDim.x;
  int tile = (int)blockIdx.x * per;
  const int tend = min(tiles, tile + per);
  const int nkh = a.hidden / 32, nchunk = a.hidden / kHC;
  const int head = w / WPH, t0 = (w % WPH) * TPW;
  const bf16_t *Q = (const bf16_t *)at.q;
  Ring ring;
  if (tile < tend) {
    Layer L0{(const bf16_t *)a.w1, (const bf16_t *)a.w3, (const bf16_t *)a.w2, (const bf16_t *)a.wp,
             a.ln_g, a.ln_b, nullptr, nullptr};
    const Src s0 = src_g(L0, 0, w, tid & 63);
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) ring_load(ring, kb, s0, kb);
  }
  int cur_u = -1;
  for (; tile < tend; ++tile) {
    const int u = upper_index(P.pblk, at.B, tile * 4);
    const int tbase = P.toff[u];
    const int m_u = P.toff[u + 1] - tbase;
    // a user without targets needs no K/V (only the optional input dump)
    if (m_u == 0 && !a.in_dump) continue;
    const bool first = u != cur_u;                                   // user's first tile here
    const bool last = tile + 1 == tend || (tile + 1) * 4 >= P.pblk[u + 1];  // ... and last
    cur_u = u;
    // per-tile lane quantities and weight addresses (nothing held across tiles)
    int ltid = tid;
    asm volatile("" : "+v"(ltid));
    const int lane = ltid & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int c16 = lane & 15, g16 = lane >> 4;
    Layer L{(const bf16_t *)a.w1, (const bf16_t *)a.w3, (const bf16_t *)a.w2, (const bf16_t *)a.wp,
            a.ln_g, a.ln_b, nullptr, nullptr};
    asm volatile("" : "+s"(L.w1), "+s"(L.w3), "+s"(L.w2), "+s"(L.wp), "+s"(L.ln_g), "+s"(L.ln_b));
    __syncthreads();  // the previous tile's attention is done with the staging
    const int64_t row0 = (int64_t)tile * kR;
    gather_tile(a, sm, row0, P.pblk[at.B], ltid, false);
    ffn_ln<LN, false>(ring, L, sm, sm.xs, w, lane, nkh, nchunk, src_k(L, w, lane));

    bf16_t *const kst = &sm.gs[0][0];  // K: [key][feature], row stride kXLD
    bf16_t *const vst = sm.xs;         // V^T: [feature][128 keys], swizzled chunks
    {  // K^T = W_K^T X~^T
      f32x16 acc[4];
      zero16(acc);
      const Src cur = src_k(L, w, lane), nxt = src_v(L, w, lane);
      run_phase<kD / 32>(ring, cur, nxt, true, [&](int kb, int slot) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 bx[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) bx[j] = ld8(sm.xs + (j * 32 + l32) * kXLD + kb * 32 + hi * 16 + h * 8);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] = mfma32(ring.v[slot][h], bx[j], acc[j]);
        }
      });
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = w * 32 + 8 * q + 4 * hi;
          u32x2 v = {pack_bf2(acc[j][4 * q], acc[j][4 * q + 1]), pack_bf2(acc[j][4 * q + 2], acc[j][4 * q + 3])};
          *reinterpret_cast<u32x2 *>(kst + (j * 32 + l32) * kXLD + f) = v;
        }
    }
    {  // V = X~ W_V, keys as MFMA rows
      f32x16 acc[4];
      zero16(acc);
      const bool more = tile + 1 < tend;  // then the next tile's first G blocks follow
      const Src cur = src_v(L, w, lane), nxt = src_g(L, 0, w, lane);
      run_phase<kD / 32>(ring, cur, nxt, more, [&](int kb, int slot) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 bx[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) bx[j] = ld8(sm.xs + (j * 32 + l32) * kXLD + kb * 32 + hi * 16 + h * 8);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] = mfma32(bx[j], ring.v[slot][h], acc[j]);
        }
      });
      __syncthreads();  // every wave has read X~: V^T goes over it
      const int f = w * 32 + l32;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int chunk = (j * 4 + q) ^ (f & 15);
          u32x2 v = {pack_bf2(acc[j][4 * q], acc[j][4 * q + 1]), pack_bf2(acc[j][4 * q + 2], acc[j][4 * q + 3])};
          *reinterpret_cast<u32x2 *>(vst + f * kR + chunk * 8 + 4 * hi) = v;
        }
    }
    __syncthreads();  // the tile's K and V are staged
    if (m_u == 0 || t0 >= m_u) continue;

    const int Lu = P.hoff[u + 1] - P.hoff[u];
    const int kbase = (tile * 4 - P.pblk[u]) * 32;  // user-local index of the tile's first key
    const int kr0 = attn_key_row(lane);
    f32x4 *const rec = reinterpret_cast<f32x4 *>(at.fstate) + ((int64_t)blockIdx.x * 8 + w) * REC * 64 + lane;
    AttnState<DH, NT> st;
    if (first) {
      attn_reset(st);
    } else {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n) st.o[t][n] = rec[(t * NT + n) * 64];
      const f32x4 m4 = rec[(DT * NT) * 64], l4 = rec[(DT * NT + 1) * 64], c4 = rec[(DT * NT + 2) * 64];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        st.mrun[n] = m4[n];
        st.l[n] = f32x4{l4[n], l4[n], l4[n], l4[n]};
        st.cnt[n] = __float_as_int(c4[n]);
      }
    }
    attn_load_q(st, Q, at.d, head, tbase, t0, m_u, lane);
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int nvalid = Lu - (kbase + blk * 32);
      if (nvalid <= 0) break;
      bf16x8 kf[2][KS], vf[DT];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int k = 0; k < KS; ++k)
          kf[kt][k] = ld8(kst + (blk * 32 + kr0 + 4 * kt) * kXLD + head * DH + k * 32 + g16 * 8);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int f = head * DH + t * 16 + c16;
        vf[t] = ld8(vst + f * kR + (((blk * 4 + g16) ^ (f & 15)) * 8));
      }
      attn_block<DH, NT, SCORE>(st, kf, vf, nvalid, 0xffffffffu, lane);
    }
    if (!last) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n) rec[(t * NT + n) * 64] = st.o[t][n];
      f32x4 m4 = {0.f, 0.f, 0.f, 0.f}, l4 = m4, c4 = m4;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        m4[n] = st.mrun[n];
        l4[n] = st.l[n][0];
        c4[n] = __int_as_float(st.cnt[n]);
      }
      rec[(DT * NT) * 64] = m4;
      rec[(DT * NT + 1) * 64] = l4;
      rec[(DT * NT + 2) * 64] = c4;
      continue;
    }
    // the user's last tile in this range: write the partial
    const int slot = (int)blockIdx.x + u;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      int cn = st.cnt[n];
      cn = isum_x16(cn);
      cn = isum_x32(cn);
      const int tl = t0 + n * 16 + c16;
      if (tl < m_u) {
        const int64_t idx = partial_index(slot, H, head, at.tgs, tl);
        if (g16 == 0) {
          if (SCORE == 0) {
            at.part_ml[idx * 2] = st.mrun[n];
            at.part_ml[idx * 2 + 1] = st.l[n][0];
          } else {
            at.part_cnt[idx] = cn;
          }
        }
#pragma unroll
        for (int t = 0; t < DT; ++t)
          *reinterpret_cast<f32x4 *>(at.part_acc + idx * DH + t * 16 + 4 * g16) = st.o[t][n];
      }
    }
  }
}

template <int DH, int NT, int SCORE>
hipError_t launch_fused256_t(const ChainArgs &a, AttnArgs &at, int64_t max_tiles, hipStream_t s) {
  auto k = a.ln ? fused256_kernel<DH, NT, SCORE, true> : fused256_kernel<DH, NT, SCORE, false>;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  int64_t g = std::min<int64_t>(max_tiles, (int64_t)cus);
  g = std::max<int64_t>(1, std::min<int64_t>(g, at.max_grid));
  at.grid = (int)g;
  hipLaunchKernelGGL(k, dim3(at.grid), dim3(kT), 0, s, a, at);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fused256(const ChainArgs &a, AttnArgs &at, int64_t max_tiles, hipStream_t s) {
  at.grid = 0;
  if (max_tiles <= 0 || (at.n_tgt <= 0 && !a.in_dump)) return hipSuccess;
  if (a.d != kD || at.max_tgt > 64 || at.max_grid < 1 || a.hidden % kHC) return hipErrorInvalidValue;
  const int mt = at.max_tgt;
  if (at.dh == 32) {
    const int nt = (mt + 15) / 16;
    if (at.score) {
      if (nt <= 1) return launch_fused256_t<32, 1, 1>(a, at, max_tiles, s);
      if (nt <= 2) return launch_fused256_t<32, 2, 1>(a, at, max_tiles, s);
      return launch_fused256_t<32, 4, 1>(a, at, max_tiles, s);
    }
    if (nt <= 1) return launch_fused256_t<32, 1, 0>(a, at, max_tiles, s);
    if (nt <= 2) return launch_fused256_t<32, 2, 0>(a, at, max_tiles, s);
    return launch_fused256_t<32, 4, 0>(a, at, max_tiles, s);
  }
  if (at.dh == 64) {  // each wave of a head's pair serves up to 32 targets
    const int nt = (std::min(mt, 32) + 15) / 16;
    if (at.score) {
      if (nt <= 1) return launch_fused256_t<64, 1, 1>(a, at, max_tiles, s);
      return launch_fused256_t<64, 2, 1>(a, at, max_tiles, s);
    }
    if (nt <= 1) return launch_fused256_t<64, 1, 0>(a, at, max_tiles, s);
    return launch_fused256_t<64, 2, 0>(a, at, max_tiles, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_hist256(const ChainArgs &a, const HistLayers &hl, hipStream_t s) {
  if (a.n_rows <= 0 || hl.M <= 0) return hipSuccess;
  if (a.d != kD || hl.M > kMaxLayers || a.hidden % kHC || a.in_mode != IN_GATHER_CSR)
    return hipErrorInvalidValue;
  int64_t nwg = (a.n_rows + kR - 1) / kR;
  if (hl.persistent) {  // one workgroup per CU (the LDS allows no more)
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    nwg = std::min<int64_t>(nwg, std::max(cus, 1));
  }
  const dim3 grid((unsigned)nwg), block(kT);
  if (hl.persistent) {
    if (a.ln) hipLaunchKernelGGL((hist256_kernel<true, true>), grid, block, 0, s, a, hl);
    else hipLaunchKernelGGL((hist256_kernel<false, true>), grid, block, 0, s, a, hl);
  } else {
    if (a.ln) hipLaunchKernelGGL((hist256_kernel<true, false>), grid, block, 0, s, a, hl);
    else hipLaunchKernelGGL((hist256_kernel<false, false>), grid, block, 0, s, a, hl);
  }
  return hipGetLastError();
}

}  // namespace stca
