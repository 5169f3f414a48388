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
