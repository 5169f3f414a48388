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

// Cross-lane exchanges through the VALU (gfx950 v_permlane32_swap /
// v_permlane16_swap) rather than an LDS permute.  swap32: a <- [a lanes 0-31,
// b lanes 0-31], b <- [a lanes 32-63, b lanes 32-63].  swap16, per row of 16
// lanes r0..r3: a <- [a.r0, b.r0, a.r2, b.r2], b <- [a.r1, b.r1, a.r3, b.r3].
DEV void swap32(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
DEV void swap16(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
// v(lane) op v(lane ^ 32) and v(lane) op v(lane ^ 16), for commutative ops.
DEV float sum_x32(float v) {
  uint32_t a = __float_as_uint(v), b = a;
  swap32(a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
DEV float max_x32(float v) {
  uint32_t a = __float_as_uint(v), b = a;
  swap32(a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
DEV float max_x16(float v) {
  uint32_t a = __float_as_uint(v), b = a;
  swap16(a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
DEV float sum_x16(float v) {
  uint32_t a = __float_as_uint(v), b = a;
  swap16(a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
DEV int isum_x32(int v) {
  uint32_t a = (uint32_t)v, b = a;
  swap32(a, b);
  return (int)(a + b);
}
DEV int isum_x16(int v) {
  uint32_t a = (uint32_t)v, b = a;
  swap16(a, b);
  return (int)(a + b);
}

// A 32x32 accumulator holds, in lane (c, hi), rows 8q + 4hi + r (q, r < 4)
// of column c.  Exchanged with lane c + 32(1 - 2hi), each lane ends up with
// 16 consecutive rows as bf16: rows 0..15 for hi = 0, 16..31 for hi = 1
// (lanes of the lower half keep their rows 8q + r of q = 0, 1 and take the
// partner's 8q + 4 + r; the upper half the same for q = 2, 3).
DEV void halves16(const f32x16 &acc, int hi, u32x4 &o0, u32x4 &o1) {
  uint32_t p[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p[q][0] = pack_bf2(acc[4 * q], acc[4 * q + 1]);
    p[q][1] = pack_bf2(acc[4 * q + 2], acc[4 * q + 3]);
  }
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    swap32(p[0][e], p[2][e]);
    swap32(p[1][e], p[3][e]);
  }
  o0 = u32x4{p[0][0], p[0][1], p[2][0], p[2][1]};
  o1 = u32x4{p[1][0], p[1][1], p[3][0], p[3][1]};
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
  v = max_x16(max_x32(v));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
DEV float wave_sum(float v) {
  v = sum_x32(v);
  v = sum_x16(v);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o);
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
