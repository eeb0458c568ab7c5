// Device/host helpers shared by the gfx950 kernels of the GPT training step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage type for bfloat16 (raw bits)

#define GPT_WAVE 64

// ---------------------------------------------------------------------------
// bfloat16 <-> float (round to nearest even; NaN kept quiet)

__device__ __host__ inline float bf2f(bf16_t v) {
  uint32_t u = ((uint32_t)v) << 16;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

__device__ __host__ inline bf16_t f2bf(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ inline uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// ---------------------------------------------------------------------------
// wave reductions (wave64)

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// 8x8 transpose of 16-bit elements held as 8 uint4 rows.
// in[j] holds row j (8 elements); out[r] holds column r (element j = in[j][r]).
__device__ inline void transpose8x8_b16(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* s = reinterpret_cast<const uint32_t*>(in);
  uint32_t* d = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t x = s[(2 * t) * 4 + (r >> 1)];      // element r of row 2t
      uint32_t y = s[(2 * t + 1) * 4 + (r >> 1)];  // element r of row 2t+1
      uint32_t lo = (r & 1) ? (x >> 16) : (x & 0xffffu);
      uint32_t hi = (r & 1) ? (y & 0xffff0000u) : (y << 16);
      d[r * 4 + t] = lo | hi;
    }
  }
}

__device__ inline f32x16_t mfma32x32x16_bf16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32 f32 accumulator layout (for lane l, register r):
//   column = l % 32, row = (r / 4) * 8 + (l / 32) * 4 + (r % 4)
__device__ inline int acc_row(int lane, int r) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

#define HIP_CHECK_RET(x)                                   \
  do {                                                     \
    hipError_t e_ = (x);                                   \
    if (e_ != hipSuccess) return GPT_ERR_HIP;              \
  } while (0)
