// common.h -- device helpers shared by the STCA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define DEV __device__ __forceinline__

typedef uint16_t bf16_t;  // raw bf16 bits

typedef short bf16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

static constexpr int kWave = 64;
static constexpr int kBlockKeys = 32;  // keys per K/V block of the staged layout

// ---------------------------------------------------------------- bf16
DEV float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16, round to nearest, ties to even: the gfx950 conversion
// instruction (v_cvt_pk_bf16_f32, RNE under the default rounding mode; NaN
// stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

DEV uint32_t pack_bf2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> DEV float to_f(T x);
template <> DEV float to_f<float>(float x) { return x; }
template <> DEV float to_f<bf16_t>(bf16_t x) { return bf2f(x); }
template <typename T> DEV T from_f(float x);
template <> DEV float from_f<float>(float x) { return x; }
template <> DEV bf16_t from_f<bf16_t>(float x) { return f2bf(x); }

// ---------------------------------------------------------------- MFMA
// 32x32x16 bf16 -> fp32.  Lane l supplies A[row l%32][8 k-values of group l/32]
// and B[same 8 k-values][col l%32]; the k order inside a block only has to
// agree between A and B.  Output: lane l holds column l%32, rows
// 8*(i/4) + 4*(l/32) + (i%4) for i = 0..15.
DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 -> fp32.  Lane l supplies A[row l%16][8 k-values of group l/16]
// and B[same k][col l%16]; output lane l holds column l%16, rows 4*(l/16)+i.
DEV f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

DEV int c32_row(int lane, int i) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// A 32x32 accumulator holds, in lane (c, hi), rows 8q + 4hi + r (q, r < 4)
// of column c.  Exchanged with lane c + 32(1 - 2hi), each lane ends up with
// 16 consecutive rows as bf16: rows 0..15 for hi = 0, 16..31 for hi = 1.
DEV void halves16(const f32x16 &acc, int hi, u32x4 &o0, u32x4 &o1) {
  u32x2 p[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) p[q] = u32x2{pack_bf2(acc[4 * q], acc[4 * q + 1]), pack_bf2(acc[4 * q + 2], acc[4 * q + 3])};
  const u32x2 s0 = hi ? p[0] : p[2], s1 = hi ? p[1] : p[3];
  u32x2 r0, r1;
  r0[0] = __shfl_xor((int)s0[0], 32);
  r0[1] = __shfl_xor((int)s0[1], 32);
  r1[0] = __shfl_xor((int)s1[0], 32);
  r1[1] = __shfl_xor((int)s1[1], 32);
  if (hi) {
    o0 = u32x4{r0[0], r0[1], p[2][0], p[2][1]};
    o1 = u32x4{r1[0], r1[1], p[3][0], p[3][1]};
  } else {
    o0 = u32x4{p[0][0], p[0][1], r0[0], r0[1]};
    o1 = u32x4{p[1][0], p[1][1], r1[0], r1[1]};
  }
}

DEV bf16x8 ld8(const bf16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Loads through pointers known to address global memory.  A pointer whose
// origin the optimiser cannot see (for instance one passed through an empty
// asm to keep address arithmetic inside a loop) otherwise becomes a flat
// access, which also counts against the LDS wait counter: every wait for an
// LDS operand would then drain the weight prefetches as well.
typedef __attribute__((address_space(1))) const bf16x8 gbf16x8;
typedef __attribute__((address_space(1))) const f32x4 gf32x4;
DEV bf16x8 ldg8(const bf16_t *p) { return *(gbf16x8 *)p; }
DEV f32x4 ldg4(const float *p) { return *(gf32x4 *)p; }

// Streaming (non-temporal) access for data touched once: K/V written by the
// history encoder and read once per layer by the attention.  Neither side
// then leaves K/V lines in the memory-side cache, where dirty ones would
// otherwise be written back during the next kernels' reads.
DEV bf16x8 ldnt8(const bf16_t *p) { return __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p)); }
DEV void stnt16(bf16_t *p, const u32x4 &v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p)); }

// ---------------------------------------------------------------- misc
DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

DEV float silu_fast(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
DEV float silu_exact(float x) { return x / (1.0f + expf(-x)); }

// Largest u with off[u] <= key (off ascending, off[0] = 0), over [0, n).
DEV int upper_index(const int *off, int n, int key) {
  int lo = 0, hi = n;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (off[mid] <= key) lo = mid; else hi = mid;
  }
  return lo;
}

DEV void set_status(int *st, int bits) {
  if (st) atomicOr(st, bits);
}
