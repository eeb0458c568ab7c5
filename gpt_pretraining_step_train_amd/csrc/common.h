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
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(bf16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: round to nearest even
#else
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
#endif
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> two bfloat16 (lo in the low half), one v_cvt_pk_bf16_f32
__device__ inline uint32_t pack_bf2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// x as a bf16 store rounds it.  Rounding to nearest is monotonic and odd, so the largest
// magnitude among stored bf16 values is bf16_round of the largest fp32 magnitude: a
// producer's running max of |value| gives the amax its stored tensor has.
__device__ inline float bf16_round(float x) { return bf2f(f2bf(x)); }

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

// IEEE binary16 (fp16): same MFMA rate and operand layout as bf16, 11 significant bits
typedef _Float16 f16_t;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ inline f32x16_t mfma32x32x16_f16(const f16x8_t& a, const f16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 32x32 f32 accumulator layout (for lane l, register r):
//   column = l % 32, row = (r / 4) * 8 + (l / 32) * 4 + (r % 4)
__device__ inline int acc_row(int lane, int r) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

// ---------------------------------------------------------------------------
// LDS transpose reads (ds_read_b64_tr_b16).  In each group of 16 lanes, lane i
// supplies the address of 4 consecutive 16-bit elements M[i][0..3]; it receives
// M[i/4][i%4], M[i/4+4][i%4], M[i/4+8][i%4], M[i/4+12][i%4].

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ inline i16x4_t lds_read_tr16(const bf16_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lds_ptr);
}

// MFMA operand whose reduction index runs down the rows of a row-major LDS tile
// T (row stride ld elements): lane l (hl = l/32) receives column c0 + l%32 at rows
// r0 + 4hl + {0,1,2,3} (k = 0..3) and r0 + 8 + 4hl + {0,1,2,3} (k = 4..7).  That
// is the row order in which a 32x32 accumulator holds rows r0..r0+15 of a lane's
// column (registers 4..7 of a 16-row group follow registers 0..3 at +8 rows).
__device__ inline bf16x8_t tr_operand(const bf16_t* T, int ld, int r0, int c0, int lane) {
  const int i = lane & 15;
  const bf16_t* p = T + (r0 + 4 * (lane >> 5) + (i >> 2)) * ld + c0 + ((lane >> 4) & 1) * 16 + 4 * (i & 3);
  const i16x4_t a = lds_read_tr16(p);
  const i16x4_t b = lds_read_tr16(p + 8 * ld);
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

#define HIP_CHECK_RET(x)                                   \
  do {                                                     \
    hipError_t e_ = (x);                                   \
    if (e_ != hipSuccess) return GPT_ERR_HIP;              \
  } while (0)
