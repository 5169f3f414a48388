// chain_bf16.hip -- the row chain on bf16 MFMA (gfx950):
//
//   rows -> [SwiGLU FFN d->h->d] -> [LayerNorm] -> [projection d->pn, scaled]
//
// Used for the history side of every layer (gather of embedding rows, then
// Xt = LN(SwiGLU(X)), K = Xt W_K, V = Xt W_V; [Notes] §STCA, [HyFormer]
// eq. (7)-(8)) and for the query side (q1 = LN(SwiGLU(x_t)), the fusion
// q_{i+1} = LN(SwiGLU([o_1|..|o_i|x_t] W_C)), Q = q W_Q / sqrt(d_h), o = attn W_O,
// z = SwiGLU([o_1|..|o_M|x_t] W_Z); [Review] architecture tree and 核心公式).
//
// One workgroup = 4 waves = 64 rows.  The gathered rows stay in LDS for the
// whole chain; the hidden activations are produced 128 columns at a time
// (double-buffered in LDS) and immediately contracted with W2, so the
// [64 x h] activation block never exists in full.  Weights are read as
// prepared transposes ([out, in], k contiguous) straight from L2 into MFMA
// operand registers.  All contractions are 32x32x16 bf16 MFMA with fp32
// accumulation; LN statistics are fp32.
#include "stca_internal.h"

namespace stca {
namespace {

constexpr int kRows = 64;     // rows per workgroup
constexpr int kThreads = 256; // 4 waves
constexpr int kHC = 128;      // hidden columns per chunk
constexpr int kPad = 8;       // bf16 elements of row padding in LDS (16 bytes)

// acc[i][j] += A(rows of tile i) * B(cols of tile j)^T over k in [0, K).
// ar[i] / br[j] point at the lane's row (A) / column (B) already offset by
// the lane's 16-element k group; each 32-wide k block is two MFMAs.
template <int RT, int CT>
DEV void mma(f32x16 (&acc)[RT][CT], const bf16_t *const (&ar)[RT], const bf16_t *const (&br)[CT],
             int K) {
#pragma unroll 1
  for (int k0 = 0; k0 < K; k0 += 32) {
    bf16x8 a[RT][2], b[CT][2];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      a[i][0] = ld8(ar[i] + k0);
      a[i][1] = ld8(ar[i] + k0 + 8);
    }
#pragma unroll
    for (int j = 0; j < CT; ++j) {
      b[j][0] = ld8(br[j] + k0);
      b[j][1] = ld8(br[j] + k0 + 8);
    }
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        acc[i][j] = mfma32(a[i][0], b[j][0], acc[i][j]);
        acc[i][j] = mfma32(a[i][1], b[j][1], acc[i][j]);
      }
  }
}

template <int RT, int CT>
DEV void zero(f32x16 (&acc)[RT][CT]) {
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

template <int D, int IN, bool FFN, bool LN, bool PROJ, int OUT>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
  constexpr int XLD = D + kPad;
  constexpr int GLD = kHC + kPad;
  constexpr int CTY = D / 128;  // 32-col tiles per wave for d-wide outputs
  __shared__ __attribute__((aligned(16))) bf16_t xs[kRows * XLD];
  __shared__ __attribute__((aligned(16))) bf16_t gs[FFN ? 2 : 1][FFN ? kRows * GLD : 8];
  __shared__ float red[2][4][kRows];
  __shared__ int s_id[kRows], s_tok[kRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int kg = (lane >> 5) * 16;  // lane's k offset inside a 32-wide k block
  const int64_t row0 = (int64_t)blockIdx.x * kRows;
  const bf16_t *table = (const bf16_t *)a.table;

  int total_blocks = 0;
  if (IN == IN_GATHER_CSR) {
    total_blocks = a.plan.pblk[a.B];
    if (row0 >= (int64_t)total_blocks * 32) return;
  } else {
    if (row0 >= a.n_rows) return;
  }

  // ------------------------------------------------------------ input rows
  if (IN == IN_GATHER_CSR || IN == IN_GATHER_IDS) {
    if (tid < kRows) {
      int id = -1, tok = -1;
      const int64_t p = row0 + tid;
      if (IN == IN_GATHER_CSR) {
        const int blk = (int)(p >> 5);
        if (blk < total_blocks) {
          const int u = upper_index(a.plan.pblk, a.B, blk);
          const int j = (int)(p - (int64_t)a.plan.pblk[u] * 32);
          if (j < a.plan.hoff[u + 1] - a.plan.hoff[u]) {
            tok = a.plan.hoff[u] + j;
            id = a.ids[tok];
          }
        }
      } else if (p < a.n_rows) {
        tok = (int)p;
        id = a.ids[p];
      }
      if (tok >= 0 && (id < 0 || (int64_t)id >= a.table_rows)) {
        set_status(a.status, 4);
        id = -1;
      }
      s_id[tid] = id;
      s_tok[tid] = tok;
    }
    __syncthreads();
    constexpr int C8 = D / 8;
    for (int e = tid; e < kRows * C8; e += kThreads) {
      const int r = e / C8, c = (e % C8) * 8;
      const int id = s_id[r];
      u32x4 v = {0u, 0u, 0u, 0u};
      if (id >= 0) v = *reinterpret_cast<const u32x4 *>(table + (int64_t)id * D + c);
      *reinterpret_cast<u32x4 *>(xs + r * XLD + c) = v;
      if (a.in_dump && s_tok[r] >= 0)
        *reinterpret_cast<u32x4 *>((bf16_t *)a.in_dump + (int64_t)s_tok[r] * D + c) = v;
    }
  } else if (IN == IN_DENSE) {
    constexpr int C8 = D / 8;
    const bf16_t *src = (const bf16_t *)a.a;
    for (int e = tid; e < kRows * C8; e += kThreads) {
      const int r = e / C8, c = (e % C8) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row0 + r < a.n_rows) v = *reinterpret_cast<const u32x4 *>(src + (row0 + r) * a.lda + c);
      *reinterpret_cast<u32x4 *>(xs + r * XLD + c) = v;
    }
  } else {  // IN_PREGEMM: xs = bf16([seg1 | seg2] W_pre)
    f32x16 acc[2][CTY];
    zero(acc);
    const bf16_t *wpre = (const bf16_t *)a.wpre;
    const int kt = a.k1 + a.k2;
    const bf16_t *br[CTY];
#pragma unroll
    for (int j = 0; j < CTY; ++j) br[j] = wpre + (int64_t)(w * (D / 4) + j * 32 + l32) * kt + kg;
    const bf16_t *ar[2];
    int64_t rr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rr[i] = row0 + i * 32 + l32;
      if (rr[i] >= a.n_rows) rr[i] = a.n_rows - 1;  // clamp: result discarded
    }
    if (a.k1 > 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) ar[i] = (const bf16_t *)a.a + rr[i] * a.lda + kg;
      mma<2, CTY>(acc, ar, br, a.k1);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) ar[i] = (const bf16_t *)a.a2 + rr[i] * a.lda2 + kg;
#pragma unroll
    for (int j = 0; j < CTY; ++j) br[j] += a.k1;
    mma<2, CTY>(acc, ar, br, a.k2);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < CTY; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          xs[(i * 32 + c32_row(lane, e)) * XLD + w * (D / 4) + j * 32 + l32] = f2bf(acc[i][j][e]);
  }
  __syncthreads();

  // ------------------------------------------------------------ SwiGLU FFN
  if (FFN) {
    f32x16 y[2][CTY];
    zero(y);
    const bf16_t *w1 = (const bf16_t *)a.w1, *w3 = (const bf16_t *)a.w3, *w2 = (const bf16_t *)a.w2;
    const bf16_t *ax[2] = {xs + l32 * XLD + kg, xs + (32 + l32) * XLD + kg};
    const int nchunk = a.hidden / kHC;
    for (int hc = 0; hc < nchunk; ++hc) {
      bf16_t *g = gs[hc & 1];
      {  // g = SiLU(X W1) * (X W3) for this wave's 32 hidden columns
        f32x16 acc[2][2];
        zero(acc);
        const int col = hc * kHC + w * 32 + l32;
        const bf16_t *br[2] = {w1 + (int64_t)col * D + kg, w3 + (int64_t)col * D + kg};
        mma<2, 2>(acc, ax, br, D);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            g[(i * 32 + c32_row(lane, e)) * GLD + w * 32 + l32] =
                f2bf(silu_fast(acc[i][0][e]) * acc[i][1][e]);
      }
      __syncthreads();
      {  // y += g W2[chunk rows]
        const bf16_t *ag[2] = {g + l32 * GLD + kg, g + (32 + l32) * GLD + kg};
        const bf16_t *br[CTY];
#pragma unroll
        for (int j = 0; j < CTY; ++j)
          br[j] = w2 + (int64_t)(w * (D / 4) + j * 32 + l32) * a.hidden + hc * kHC + kg;
        mma<2, CTY>(y, ag, br, kHC);
      }
    }
    // -------------------------------------------------------- LayerNorm
    float mean[2][16], rstd[2][16];
    if (LN) {
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        float s[2][16];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float v = 0.f;
#pragma unroll
            for (int j = 0; j < CTY; ++j) {
              const float x = y[i][j][e];
              v += pass == 0 ? x : (x - mean[i][e]) * (x - mean[i][e]);
            }
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o);
            s[i][e] = v;
          }
        if (l32 == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[pass][w][i * 32 + c32_row(lane, e)] = s[i][e];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = i * 32 + c32_row(lane, e);
            const float t = red[pass][0][r] + red[pass][1][r] + red[pass][2][r] + red[pass][3][r];
            if (pass == 0) mean[i][e] = t * (1.0f / D);
            else rstd[i][e] = rsqrtf(t * (1.0f / D) + 1e-5f);
          }
      }
    }
    // normalised (or plain) FFN output -> xs (bf16) or straight to out32
#pragma unroll
    for (int j = 0; j < CTY; ++j) {
      const int c = w * (D / 4) + j * 32 + l32;
      const float gg = LN ? a.ln_g[c] : 1.f, bb = LN ? a.ln_b[c] : 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = i * 32 + c32_row(lane, e);
          float v = y[i][j][e];
          if (LN) v = (v - mean[i][e]) * rstd[i][e] * gg + bb;
          if (PROJ) {
            xs[r * XLD + c] = f2bf(v);
          } else if (row0 + r < a.n_rows) {
            if (a.out32) a.out32[(row0 + r) * a.ldo32 + c] = v;
            if (a.out) ((bf16_t *)a.out)[(row0 + r) * a.ldo + c] = f2bf(v);
          }
        }
    }
    if (!PROJ) return;
    __syncthreads();
  }

  // ------------------------------------------------------------ projection
  if (PROJ) {
    const bf16_t *wp = (const bf16_t *)a.wp;
    const bf16_t *bx[2] = {xs + l32 * XLD + kg, xs + (32 + l32) * XLD + kg};
    if (OUT == OUT_KV) {
      const int H = a.H;
      constexpr int DH_LOG_MIN = 5;
      (void)DH_LOG_MIN;
      const int DH = D / H;
      bf16_t *kb = (bf16_t *)a.kbuf, *vb = (bf16_t *)a.vbuf;
      {  // K^T = W_K^T Xt^T: lane gets 4 consecutive features of one token
        f32x16 acc[CTY][2];
        zero(acc);
        const bf16_t *ar[CTY];
#pragma unroll
        for (int i = 0; i < CTY; ++i) ar[i] = wp + (int64_t)(w * (D / 4) + i * 32 + l32) * D + kg;
        mma<CTY, 2>(acc, ar, bx, D);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int blk = (int)(row0 >> 5) + t;
          if (blk >= total_blocks) continue;
#pragma unroll
          for (int i = 0; i < CTY; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int f = w * (D / 4) + i * 32 + 8 * q + 4 * (lane >> 5);
              const int h = f / DH, dh = f % DH;
              u32x2 v = {pack_bf2(acc[i][t][4 * q], acc[i][t][4 * q + 1]),
                         pack_bf2(acc[i][t][4 * q + 2], acc[i][t][4 * q + 3])};
              *reinterpret_cast<u32x2 *>(kb + (((int64_t)blk * H + h) * 32 + l32) * DH + dh) = v;
            }
        }
      }
      {  // V = Xt W_V: lane gets 4 consecutive tokens of one feature -> V^T rows
        f32x16 acc[2][CTY];
        zero(acc);
        const bf16_t *br[CTY];
#pragma unroll
        for (int j = 0; j < CTY; ++j) br[j] = wp + (int64_t)(D + w * (D / 4) + j * 32 + l32) * D + kg;
        mma<2, CTY>(acc, bx, br, D);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int blk = (int)(row0 >> 5) + t;
          if (blk >= total_blocks) continue;
#pragma unroll
          for (int j = 0; j < CTY; ++j) {
            const int f = w * (D / 4) + j * 32 + l32;
            const int h = f / DH, dh = f % DH;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int key = 8 * q + 4 * (lane >> 5);
              u32x2 v = {pack_bf2(acc[t][j][4 * q], acc[t][j][4 * q + 1]),
                         pack_bf2(acc[t][j][4 * q + 2], acc[t][j][4 * q + 3])};
              *reinterpret_cast<u32x2 *>(vb + (((int64_t)blk * H + h) * DH + dh) * 32 + key) = v;
            }
          }
        }
      }
    } else {  // OUT_ROWS: out^T = Wp^T Xt^T, pn/4 features per wave in tiles of 32
      const int per_wave = a.pn / 4;
      for (int f0 = 0; f0 < per_wave; f0 += 32 * CTY) {
        f32x16 acc[CTY][2];
        zero(acc);
        const bf16_t *ar[CTY];
#pragma unroll
        for (int i = 0; i < CTY; ++i) {
          int f = w * per_wave + f0 + i * 32 + l32;
          if (f0 + i * 32 >= per_wave) f = w * per_wave;  // beyond this wave's slice: dummy
          ar[i] = wp + (int64_t)f * D + kg;
        }
        mma<CTY, 2>(acc, ar, bx, D);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int64_t row = row0 + t * 32 + l32;
          if (row >= a.n_rows) continue;
#pragma unroll
          for (int i = 0; i < CTY; ++i) {
            if (f0 + i * 32 >= per_wave) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int f = w * per_wave + f0 + i * 32 + 8 * q + 4 * (lane >> 5);
              const float v0 = acc[i][t][4 * q] * a.scale, v1 = acc[i][t][4 * q + 1] * a.scale;
              const float v2 = acc[i][t][4 * q + 2] * a.scale, v3 = acc[i][t][4 * q + 3] * a.scale;
              if (a.out) {
                u32x2 v = {pack_bf2(v0, v1), pack_bf2(v2, v3)};
                *reinterpret_cast<u32x2 *>((bf16_t *)a.out + row * a.ldo + f) = v;
              }
              if (a.out32) {
                f32x4 v = {v0, v1, v2, v3};
                *reinterpret_cast<f32x4 *>(a.out32 + row * a.ldo32 + f) = v;
              }
            }
          }
        }
      }
    }
  }
}

template <int D>
hipError_t dispatch_d(const ChainArgs &a, hipStream_t s) {
  int64_t rows = a.n_rows;
  const dim3 grid((unsigned)((rows + kRows - 1) / kRows)), block(kThreads);
#define CH(IN, FFN, LN, PROJ, OUT) \
  hipLaunchKernelGGL((chain_kernel<D, IN, FFN, LN, PROJ, OUT>), grid, block, 0, s, a)
  const bool f = a.ffn, l = a.ln, p = a.proj;
  switch (a.in_mode) {
    case IN_GATHER_CSR:  // history: FFN (+LN) then K/V
      if (!(f && p && a.out_mode == OUT_KV)) return hipErrorInvalidValue;
      if (l) CH(IN_GATHER_CSR, true, true, true, OUT_KV);
      else CH(IN_GATHER_CSR, true, false, true, OUT_KV);
      break;
    case IN_GATHER_IDS:  // first query: FFN + LN + W_Q
      if (!(f && l && p)) return hipErrorInvalidValue;
      CH(IN_GATHER_IDS, true, true, true, OUT_ROWS);
      break;
    case IN_DENSE:  // projections only (W_Q, W_O, R)
      if (f || l || !p) return hipErrorInvalidValue;
      CH(IN_DENSE, false, false, true, OUT_ROWS);
      break;
    case IN_PREGEMM:  // fusion (FFN + LN + W_Q) or z (FFN [+LN], no projection)
      if (!f) return hipErrorInvalidValue;
      if (p && l) CH(IN_PREGEMM, true, true, true, OUT_ROWS);
      else if (!p && l) CH(IN_PREGEMM, true, true, false, OUT_ROWS);
      else if (!p && !l) CH(IN_PREGEMM, true, false, false, OUT_ROWS);
      else return hipErrorInvalidValue;
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef CH
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void transpose_batch_kernel(TransposeBatch tb) {
  const TransposeDesc &t = tb.m[blockIdx.y];
  const int tiles_c = (t.cols + 31) / 32;
  const int tile = blockIdx.x;
  if (tile >= tiles_c * ((t.rows + 31) / 32)) return;
  __shared__ bf16_t sh[32][33];
  const int bx = (tile % tiles_c) * 32, by = (tile / tiles_c) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int j = ty; j < 32; j += 8) {
    const int r = by + j, c = bx + tx;
    sh[j][tx] = (r < t.rows && c < t.cols) ? t.src[(int64_t)r * t.cols + c] : (bf16_t)0;
  }
  __syncthreads();
  for (int j = ty; j < 32; j += 8) {
    const int r = bx + j, c = by + tx;  // dst[src col][src row]
    if (r < t.cols && c < t.rows) t.dst[(int64_t)r * t.ld_dst + t.dst_col0 + c] = sh[tx][j];
  }
}

}  // namespace

hipError_t launch_chain_bf16(const ChainArgs &a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  switch (a.d) {
    case 128: return dispatch_d<128>(a, s);
    case 256: return dispatch_d<256>(a, s);
    case 512: return dispatch_d<512>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_transpose_batch(const TransposeBatch &tb, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int max_tiles = 1;
  for (int i = 0; i < n; ++i) {
    const int t = ((tb.m[i].rows + 31) / 32) * ((tb.m[i].cols + 31) / 32);
    if (t > max_tiles) max_tiles = t;
  }
  hipLaunchKernelGGL(transpose_batch_kernel, dim3(max_tiles, n), dim3(256), 0, s, tb);
  return hipGetLastError();
}

}  // namespace stca
