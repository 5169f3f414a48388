// peak.hip -- a measurement aid, not a step of the method: a kernel that
// does nothing but dense bf16 MFMA from registers, so the matrix cores'
// attainable rate at the clock the chip holds under that load can be quoted
// beside the nominal figure the rooflines are priced against.
#include "stca.h"
#include "stca_internal.h"

namespace stca {
namespace {

// Each wave: `iters` rounds of 8 independent 32x32x16 bf16 products
// (8 x 32,768 flop per round); one checksum per wave keeps the work live.
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float *out, unsigned long long *clock) {
  const int lane = threadIdx.x & 63;
  if (clock && blockIdx.x == 0 && threadIdx.x == 0) {
    clock[0] = __builtin_amdgcn_s_memtime();
    clock[1] = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (short)(0x3c00 + ((lane + e) & 7));  // small positive bf16 values
    b[e] = (short)(0x3c00 + ((lane * 3 + e) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
  if (clock && blockIdx.x == 0 && threadIdx.x == 0) {
    clock[2] = __builtin_amdgcn_s_memtime();
    clock[3] = __builtin_amdgcn_s_memrealtime();
  }
}

// The same product stream with operands whose bits vary like real data:
// every lane holds four A and four B fragments of random signs, exponents
// (magnitudes 2^-7 .. 2^-3) and mantissas, and consecutive products take
// different ones, so the matrix cores switch as many operand bits as they do
// on activations and weights (the chip's clock under MFMA load depends on it).
// Random bits from the lowbias32 integer hash (C. Wellons) of
// (block, lane, element).
DEV uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__global__ __launch_bounds__(256) void mfma_peak_mixed_kernel(int iters, float *out, unsigned long long *clock) {
  const int lane = threadIdx.x & 63;
  if (clock && blockIdx.x == 0 && threadIdx.x == 0) {
    clock[0] = __builtin_amdgcn_s_memtime();
    clock[1] = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 a[4], b[4];
  const uint32_t seed = ((uint32_t)blockIdx.x * 256u + threadIdx.x) * 64u;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t ha = hash32(seed + 16u * i + e), hb = hash32(seed + 16u * i + 8u + e);
      a[i][e] = (short)((ha & 0x807fu) | (0x3c00u + ((ha >> 16) & 3u) * 0x80u));
      b[i][e] = (short)((hb & 0x807fu) | (0x3c00u + ((hb >> 16) & 3u) * 0x80u));
    }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma32(a[j & 3], b[(j + (j >> 2)) & 3], acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
  if (clock && blockIdx.x == 0 && threadIdx.x == 0) {
    clock[2] = __builtin_amdgcn_s_memtime();
    clock[3] = __builtin_amdgcn_s_memrealtime();
  }
}

// Each thread reads four 16-byte words per round, one grid stride apart.
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4 *p, int64_t n, uint32_t *out) {
  uint32_t x = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride * 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * stride;
      v[u] = j < n ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (x == 0x5a17c0deu) out[0] = x;
}

}  // namespace
}  // namespace stca

extern "C" int stca_peak_hbm_read(const void *buf, int64_t bytes, int32_t blocks, uint32_t *out,
                                  void *hip_stream) {
  using namespace stca;
  api_clear_error();
  if (!buf || !out || bytes <= 0 || bytes % 16 || blocks <= 0)
    return api_error(STCA_ERR_INVALID_ARG, "buf, out non-NULL; bytes > 0 and a multiple of 16; blocks > 0");
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream,
                     (const u32x4 *)buf, bytes / 16, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return api_error(STCA_ERR_HIP, "hbm read launch: %s", hipGetErrorString(e));
  return STCA_OK;
}

extern "C" int stca_peak_mfma_bf16(int32_t blocks, int32_t iters, float *out, uint64_t *clock, void *hip_stream) {
  using namespace stca;
  api_clear_error();
  // iters < 0: the mixed-operand variant, |iters| rounds
  if (blocks <= 0 || iters == 0 || !out) return api_error(STCA_ERR_INVALID_ARG, "blocks > 0, iters != 0, out non-NULL");
  if (iters > 0)
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream, (int)iters,
                       out, reinterpret_cast<unsigned long long *>(clock));
  else
    hipLaunchKernelGGL(mfma_peak_mixed_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream,
                       (int)-iters, out, reinterpret_cast<unsigned long long *>(clock));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return api_error(STCA_ERR_HIP, "mfma peak launch: %s", hipGetErrorString(e));
  return STCA_OK;
}
