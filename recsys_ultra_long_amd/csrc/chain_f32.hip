// chain_f32.hip -- the row chain in fp32 (plain FMA; the fp32 configuration
// of the library).  Same stages and semantics as chain_bf16.hip:
//   rows -> [SwiGLU FFN] -> [LayerNorm] -> [projection, scaled] -> output
// but with weights read in their stored [in, out] layout, 16 rows per
// workgroup held in LDS, and one thread per output element.
#include "stca_internal.h"

namespace stca {
namespace {

constexpr int kR = 16;        // rows per workgroup
constexpr int kT = 256;       // threads
constexpr int kHC = 32;       // hidden columns per chunk
constexpr int kMaxD = 512;

template <int IN, bool FFN, bool LN, bool PROJ, int OUT>
__global__ __launch_bounds__(kT) void chain_f32_kernel(ChainArgs a) {
  __shared__ float xs[kR][kMaxD];
  __shared__ float ys[kR][kMaxD];
  __shared__ float gs[kR][kHC];
  __shared__ int s_id[kR], s_tok[kR];
  const int D = a.d;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * kR;
  const float *table = (const float *)a.table;

  int total_blocks = 0;
  if (IN == IN_GATHER_CSR) {
    total_blocks = a.plan.pblk[a.B];
    if (row0 >= (int64_t)total_blocks * 32) return;
  } else if (row0 >= a.n_rows) {
    return;
  }

  if (IN == IN_GATHER_CSR || IN == IN_GATHER_IDS) {
    if (tid < kR) {
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
    for (int e = tid; e < kR * D; e += kT) {
      const int r = e / D, c = e % D;
      const float v = s_id[r] >= 0 ? table[(int64_t)s_id[r] * D + c] : 0.f;
      xs[r][c] = v;
      if (a.in_dump && s_tok[r] >= 0) ((float *)a.in_dump)[(int64_t)s_tok[r] * D + c] = v;
    }
  } else if (IN == IN_DENSE) {
    for (int e = tid; e < kR * D; e += kT) {
      const int r = e / D, c = e % D;
      xs[r][c] = row0 + r < a.n_rows ? ((const float *)a.a)[(row0 + r) * a.lda + c] : 0.f;
    }
  } else {  // IN_PREGEMM
    const float *wpre = (const float *)a.wpre;
    for (int e = tid; e < kR * D; e += kT) {
      const int r = e / D, c = e % D;
      float acc = 0.f;
      if (row0 + r < a.n_rows) {
        const float *s1 = (const float *)a.a + (row0 + r) * a.lda;
        const float *s2 = (const float *)a.a2 + (row0 + r) * a.lda2;
        for (int k = 0; k < a.k1; ++k) acc = fmaf(s1[k], wpre[(int64_t)k * D + c], acc);
        for (int k = 0; k < a.k2; ++k) acc = fmaf(s2[k], wpre[(int64_t)(a.k1 + k) * D + c], acc);
      }
      xs[r][c] = acc;
    }
  }
  __syncthreads();

  if (FFN) {
    const float *w1 = (const float *)a.w1, *w3 = (const float *)a.w3, *w2 = (const float *)a.w2;
    for (int e = tid; e < kR * D; e += kT) ys[e / D][e % D] = 0.f;
    for (int h0 = 0; h0 < a.hidden; h0 += kHC) {
      for (int e = tid; e < kR * kHC; e += kT) {
        const int r = e / kHC, c = e % kHC;
        float a1 = 0.f, a3 = 0.f;
        for (int k = 0; k < D; ++k) {
          const float x = xs[r][k];
          a1 = fmaf(x, w1[(int64_t)k * a.hidden + h0 + c], a1);
          a3 = fmaf(x, w3[(int64_t)k * a.hidden + h0 + c], a3);
        }
        gs[r][c] = silu_exact(a1) * a3;
      }
      __syncthreads();
      for (int e = tid; e < kR * D; e += kT) {
        const int r = e / D, c = e % D;
        float acc = ys[r][c];
        for (int k = 0; k < kHC; ++k) acc = fmaf(gs[r][k], w2[(int64_t)(h0 + k) * D + c], acc);
        ys[r][c] = acc;
      }
      __syncthreads();
    }
    for (int r = w; r < kR; r += 4) {
      float mean = 0.f, rstd = 1.f;
      if (LN) {
        float s = 0.f;
        for (int c = lane; c < D; c += 64) s += ys[r][c];
        mean = wave_sum(s) / D;
        float v = 0.f;
        for (int c = lane; c < D; c += 64) v += (ys[r][c] - mean) * (ys[r][c] - mean);
        rstd = 1.0f / sqrtf(wave_sum(v) / D + 1e-5f);
      }
      for (int c = lane; c < D; c += 64) {
        float y = ys[r][c];
        if (LN) y = (y - mean) * rstd * a.ln_g[c] + a.ln_b[c];
        if (PROJ) {
          xs[r][c] = y;
        } else if (row0 + r < a.n_rows) {
          if (a.out32) a.out32[(row0 + r) * a.ldo32 + c] = y;
          if (a.out) ((float *)a.out)[(row0 + r) * a.ldo + c] = y;
        }
      }
    }
    if (!PROJ) return;
    __syncthreads();
  }

  if (PROJ) {
    if (OUT == OUT_KV) {
      const int H = a.H, DH = D / H;
      float *kb = (float *)a.kbuf, *vb = (float *)a.vbuf;
      for (int e = tid; e < kR * 2 * D; e += kT) {
        const int r = e / (2 * D), c = e % (2 * D);
        const int64_t p = row0 + r;
        const int blk = (int)(p >> 5), key = (int)(p & 31);
        if (blk >= total_blocks) continue;
        const bool isv = c >= D;
        const int f = isv ? c - D : c;
        const float *W = (const float *)(isv ? a.wp2 : a.wp);
        float acc = 0.f;
        for (int k = 0; k < D; ++k) acc = fmaf(xs[r][k], W[(int64_t)k * D + f], acc);
        const int h = f / DH, dh = f % DH;
        if (isv) vb[(((int64_t)blk * H + h) * DH + dh) * 32 + key] = acc;
        else kb[(((int64_t)blk * H + h) * 32 + key) * DH + dh] = acc;
      }
    } else {
      const float *W = (const float *)a.wp;
      for (int e = tid; e < kR * a.pn; e += kT) {
        const int r = e / a.pn, c = e % a.pn;
        if (row0 + r >= a.n_rows) continue;
        float acc = 0.f;
        for (int k = 0; k < D; ++k) acc = fmaf(xs[r][k], W[(int64_t)k * a.pn + c], acc);
        acc *= a.scale;
        if (a.out) ((float *)a.out)[(row0 + r) * a.ldo + c] = acc;
        if (a.out32) a.out32[(row0 + r) * a.ldo32 + c] = acc;
      }
    }
  }
}

}  // namespace

hipError_t launch_chain_f32(const ChainArgs &a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.d > kMaxD || a.d % 32 || a.hidden % kHC) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.n_rows + kR - 1) / kR)), block(kT);
#define CH(IN, FFN, LN, PROJ, OUT) \
  hipLaunchKernelGGL((chain_f32_kernel<IN, FFN, LN, PROJ, OUT>), grid, block, 0, s, a)
  const bool f = a.ffn, l = a.ln, p = a.proj;
  switch (a.in_mode) {
    case IN_GATHER_CSR:
      if (!(f && p && a.out_mode == OUT_KV)) return hipErrorInvalidValue;
      if (l) CH(IN_GATHER_CSR, true, true, true, OUT_KV);
      else CH(IN_GATHER_CSR, true, false, true, OUT_KV);
      break;
    case IN_GATHER_IDS:
      if (!(f && l && p)) return hipErrorInvalidValue;
      CH(IN_GATHER_IDS, true, true, true, OUT_ROWS);
      break;
    case IN_DENSE:
      if (f || l || !p) return hipErrorInvalidValue;
      CH(IN_DENSE, false, false, true, OUT_ROWS);
      break;
    case IN_PREGEMM:
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

}  // namespace stca
