// Bandwidth-bound kernels of the GPT step: embedding gather and deterministic
// scatter-add, RMSNorm forward/backward, RoPE + QK-norm, fused softmax
// cross-entropy, and the elementwise pieces of Muon.  One wave per row for the
// per-row kernels, float4 accesses across the 64 lanes.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace {

template <typename T>
__device__ inline void st(T* p, float v);
template <>
__device__ inline void st<float>(float* p, float v) { *p = v; }
template <>
__device__ inline void st<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }
template <typename T>
__device__ inline float ld(const T* p);
template <>
__device__ inline float ld<float>(const float* p) { return *p; }
template <>
__device__ inline float ld<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <>
__device__ inline void st<f16_t>(f16_t* p, float v) { *p = (f16_t)v; }
template <>
__device__ inline float ld<f16_t>(const f16_t* p) { return (float)*p; }

template <typename T>
__device__ inline void st4(T* p, float4 v) {
  st<T>(p, v.x); st<T>(p + 1, v.y); st<T>(p + 2, v.z); st<T>(p + 3, v.w);
}
template <>
__device__ inline void st4<float>(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
template <>
__device__ inline void st4<f16_t>(f16_t* p, float4 v) {
  typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));
  const f16x4v h = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
  *reinterpret_cast<f16x4v*>(p) = h;
}
template <>
__device__ inline void st4<bf16_t>(bf16_t* p, float4 v) {
  uint2 u = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
  *reinterpret_cast<uint2*>(p) = u;
}

template <typename T>
__device__ inline float4 ld4(const T* p) { return make_float4(ld<T>(p), ld<T>(p + 1), ld<T>(p + 2), ld<T>(p + 3)); }
template <>
__device__ inline float4 ld4<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <>
__device__ inline float4 ld4<bf16_t>(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

// the magnitude m as a store of type T holds it (see bf16_round)
template <typename T>
__device__ inline float round_act(float m) { return m; }
template <>
__device__ inline float round_act<bf16_t>(float m) { return bf16_round(m); }
__device__ inline float max4abs(const float4& v) { return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))); }

constexpr int ROWS_PER_BLOCK = 4;  // one wave per row, 256 threads
constexpr int MAXV4 = 8;           // float4 per lane -> d <= 2048

// ---------------------------------------------------------------------------
// embedding gather: h[n] = E[tok[n]]

__global__ void __launch_bounds__(256) embed_gather_kernel(const int32_t* __restrict__ tok,
                                                           const float* __restrict__ E, float* __restrict__ h,
                                                           int N, int d, int V, int* err) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const int t = tok[row];
  const bool ok = (t >= 0 && t < V);
  if (!ok && lane == 0) atomicOr(err, 1);
  const float4* src = reinterpret_cast<const float4*>(E + (long)(ok ? t : 0) * d);
  float4* dst = reinterpret_cast<float4*>(h + (long)row * d);
  for (int i = lane; i < d / 4; i += 64) dst[i] = ok ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// RMSNorm (no gain): y = x / sqrt(mean(x^2) + eps)

// amax_part (or null): amax_part[row] = max |y[row][:]| as stored (an fp8 quantiser's amax
// without a pass of its own)
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_fwd_kernel(const float* __restrict__ x, T* __restrict__ y,
                                                          float* __restrict__ rstd, int N, int d, float eps,
                                                          float* __restrict__ amax_part) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const float4* xr = reinterpret_cast<const float4*>(x + (long)row * d);
  const int n4 = d / 4;
  float4 v[MAXV4];
  float ss = 0.f, ma = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    v[j] = i < n4 ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ma = fmaxf(ma, max4abs(v[j]));
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  T* yr = y + (long)row * d;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    if (i < n4) st4<T>(yr + 4 * i, make_float4(v[j].x * r, v[j].y * r, v[j].z * r, v[j].w * r));
  }
  if (lane == 0) rstd[row] = r;
  if (amax_part) {  // max over j of |v_j| r is the rounded product of the largest |v_j| (r > 0)
    ma = wave_max(ma);
    if (lane == 0) amax_part[row] = round_act<T>(ma * r);
  }
}

// dx = dres + r * (dy - y * mean(dy * y)),  y = x * r
// HAT: x is the forward's stored output y = x rstd (type T: the bf16 copy the step keeps
// for its Linear), read in place of the fp32 input and its product with rstd (2 bytes per
// element less; y then carries that store's rounding)
template <typename T, bool HAT>
__global__ void __launch_bounds__(256) rmsnorm_bwd_kernel(const float* __restrict__ dy, const void* __restrict__ x,
                                                          const float* __restrict__ rstd, const float* __restrict__ dres,
                                                          float* __restrict__ dx, T* __restrict__ dxa, int N, int d,
                                                          float* __restrict__ amax_part) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const long off = (long)row * d;
  const float4* gr = reinterpret_cast<const float4*>(dy + off);
  const int n4 = d / 4;
  const float r = rstd[row];
  float4 yv[MAXV4], gv[MAXV4];
  float dot = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f), g = y;
    if (i < n4) {
      g = gr[i];
      if constexpr (HAT) {
        y = ld4<T>(reinterpret_cast<const T*>(x) + off + 4 * i);
      } else {
        const float4 a = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off)[i];
        y = make_float4(a.x * r, a.y * r, a.z * r, a.w * r);
      }
    }
    yv[j] = y;
    gv[j] = g;
    dot += g.x * yv[j].x + g.y * yv[j].y + g.z * yv[j].z + g.w * yv[j].w;
  }
  dot = wave_sum(dot) / (float)d;
  float mo = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    if (i >= n4) continue;
    float4 o;
    o.x = r * (gv[j].x - yv[j].x * dot);
    o.y = r * (gv[j].y - yv[j].y * dot);
    o.z = r * (gv[j].z - yv[j].z * dot);
    o.w = r * (gv[j].w - yv[j].w * dot);
    if (dres) {
      const float4 q = reinterpret_cast<const float4*>(dres + off)[i];
      o.x += q.x; o.y += q.y; o.z += q.z; o.w += q.w;
    }
    reinterpret_cast<float4*>(dx + off)[i] = o;
    if (dxa) st4<T>(dxa + off + 4 * i, o);
    mo = fmaxf(mo, max4abs(o));
  }
  if (amax_part) {  // amax_part[row] = max |dxa[row][:]| as stored
    mo = wave_max(mo);
    if (lane == 0) amax_part[row] = round_act<T>(mo);
  }
}

// ---------------------------------------------------------------------------
// Extras: per-layer residual scaling, smear and backout.  Their scalars live in the
// parameter vector on the device; a coefficient is mul * (*p), or mul when p is null.

__device__ inline float coef(const float* p, float mul) { return p ? mul * *p : mul; }

// m = a x + b z (z may be null when b = 0), stored fp32, then y = m / rms(m) as in
// rmsnorm_fwd
template <typename T>
__global__ void __launch_bounds__(256) mix_rmsnorm_fwd_kernel(const float* __restrict__ x, const float* __restrict__ z,
                                                              const float* pa, float ma, const float* pb, float mb,
                                                              float* __restrict__ m, T* __restrict__ y,
                                                              float* __restrict__ rstd, int N, int d, float eps) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const float a = coef(pa, ma), b = z ? coef(pb, mb) : 0.f;
  const long off = (long)row * d;
  const float4* xr = reinterpret_cast<const float4*>(x + off);
  const float4* zr = reinterpret_cast<const float4*>(z ? z + off : x + off);
  float4* mr = reinterpret_cast<float4*>(m + off);
  const int n4 = d / 4;
  float4 v[MAXV4];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n4) {
      const float4 p = xr[i], q = zr[i];
      v[j] = make_float4(a * p.x + b * q.x, a * p.y + b * q.y, a * p.z + b * q.z, a * p.w + b * q.w);
      mr[i] = v[j];
    }
    ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  T* yr = y + off;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    if (i < n4) st4<T>(yr + 4 * i, make_float4(v[j].x * r, v[j].y * r, v[j].z * r, v[j].w * r));
  }
  if (lane == 0) rstd[row] = r;
}

// Backward of a norm whose input m = a x_a + b x_b was mixed:
//   g = dres + rstd (dy - ym mean(dy ym)), ym = m rstd      (d loss / d m)
//   out = a g + add1 + add2 (+ b g when b_to_out), fp32 and the activation copy
//   acc += b g (when acc is given and not b_to_out)
//   dots_a[row] = sa (g . x_a), dots_b[row] = sb (g . x_b)  (the scale gradients' rows)
template <typename T>
__global__ void __launch_bounds__(256) rmsnorm_mix_bwd_kernel(
    const float* __restrict__ dy, const float* __restrict__ mx, const float* __restrict__ rstd,
    const float* __restrict__ dres, const float* pa, float ma, const float* pb, float mb, int b_to_out,
    const float* __restrict__ add1, const float* __restrict__ add2, float* __restrict__ acc,
    const float* __restrict__ xa, float* __restrict__ dots_a, float sa, const float* __restrict__ xb,
    float* __restrict__ dots_b, float sb, float* __restrict__ out, T* __restrict__ outa, int N, int d) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const float a = coef(pa, ma), b = coef(pb, mb);
  const long off = (long)row * d;
  const int n4 = d / 4;
  const float r = rstd[row];
  float4 yv[MAXV4], gv[MAXV4];
  float dot = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f), g = v;
    if (i < n4) {
      v = reinterpret_cast<const float4*>(mx + off)[i];
      g = reinterpret_cast<const float4*>(dy + off)[i];
    }
    yv[j] = make_float4(v.x * r, v.y * r, v.z * r, v.w * r);
    gv[j] = g;
    dot += g.x * yv[j].x + g.y * yv[j].y + g.z * yv[j].z + g.w * yv[j].w;
  }
  dot = wave_sum(dot) / (float)d;
  const float ao = b_to_out ? a + b : a;
  float da = 0.f, db = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    if (i >= n4) continue;
    float4 g;
    g.x = r * (gv[j].x - yv[j].x * dot);
    g.y = r * (gv[j].y - yv[j].y * dot);
    g.z = r * (gv[j].z - yv[j].z * dot);
    g.w = r * (gv[j].w - yv[j].w * dot);
    if (dres) {
      const float4 q = reinterpret_cast<const float4*>(dres + off)[i];
      g.x += q.x; g.y += q.y; g.z += q.z; g.w += q.w;
    }
    if (xa) {
      const float4 q = reinterpret_cast<const float4*>(xa + off)[i];
      da += g.x * q.x + g.y * q.y + g.z * q.z + g.w * q.w;
    }
    if (xb) {
      const float4 q = reinterpret_cast<const float4*>(xb + off)[i];
      db += g.x * q.x + g.y * q.y + g.z * q.z + g.w * q.w;
    }
    if (acc && !b_to_out) {
      float4 q = reinterpret_cast<float4*>(acc + off)[i];
      q.x += b * g.x; q.y += b * g.y; q.z += b * g.z; q.w += b * g.w;
      reinterpret_cast<float4*>(acc + off)[i] = q;
    }
    float4 o = make_float4(ao * g.x, ao * g.y, ao * g.z, ao * g.w);
    if (add1) {
      const float4 q = reinterpret_cast<const float4*>(add1 + off)[i];
      o.x += q.x; o.y += q.y; o.z += q.z; o.w += q.w;
    }
    if (add2) {
      const float4 q = reinterpret_cast<const float4*>(add2 + off)[i];
      o.x += q.x; o.y += q.y; o.z += q.z; o.w += q.w;
    }
    reinterpret_cast<float4*>(out + off)[i] = o;
    if (outa) st4<T>(outa + off + 4 * i, o);
  }
  if (xa) da = wave_sum(da);
  if (xb) db = wave_sum(db);
  if (lane == 0) {
    if (xa) dots_a[row] = sa * da;
    if (xb) dots_b[row] = sb * db;
  }
}

constexpr int SMEAR_CH = 24;  // channels of the current position the smear gate reads

__device__ inline float sigmoidf_(float z) { return 1.f / (1.f + expf(-z)); }

// the smear-gate weights a lane < 6 pairs with its channels 4 lane .. 4 lane + 3 (ws sits
// at an odd float pair inside the parameter vector, so it is read by scalars)
__device__ inline float4 smear_w4(const float* __restrict__ ws, int lane) {
  return make_float4(ws[4 * lane], ws[4 * lane + 1], ws[4 * lane + 2], ws[4 * lane + 3]);
}

// gate logit of row n: ws . e[n, 0:24] (lanes 0..5 hold channels 0..23 in v0)
__device__ inline float smear_logit(const float4& v0, const float* __restrict__ ws, int lane) {
  float z = 0.f;
  if (lane < SMEAR_CH / 4) {
    const float4 w = smear_w4(ws, lane);
    z = v0.x * w.x + v0.y * w.y + v0.z * w.z + v0.w * w.w;
  }
  return wave_sum(z);
}

// x[n] = e[n] + ls sigmoid(ws . e[n, :24]) e[n-1]; nothing is added at the first
// position of each sequence (n % T == 0)
__global__ void __launch_bounds__(256) smear_fwd_kernel(const float* __restrict__ e, const float* __restrict__ pls,
                                                        const float* __restrict__ ws, float* __restrict__ x, int N,
                                                        int T, int d) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const long off = (long)row * d;
  const int n4 = d / 4;
  const float4* er = reinterpret_cast<const float4*>(e + off);
  float4* xr = reinterpret_cast<float4*>(x + off);
  // channels 0..23 sit in lanes 0..5 (d >= 24); lanes past the row load nothing
  const float4 v0 = lane < n4 ? er[lane] : make_float4(0.f, 0.f, 0.f, 0.f);
  const float gl = smear_logit(v0, ws, lane);
  const bool first = row % T == 0;
  const float g = first ? 0.f : *pls * sigmoidf_(gl);
  const float4* pr = reinterpret_cast<const float4*>(e + off - (first ? 0 : d));
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    if (i >= n4) continue;
    const float4 c = er[i];
    const float4 q = first ? make_float4(0.f, 0.f, 0.f, 0.f) : pr[i];
    xr[i] = make_float4(c.x + g * q.x, c.y + g * q.y, c.z + g * q.z, c.w + g * q.w);
  }
}

// backward of the smear for row n, dx = d loss / d x:
//   de[n] = dx[n] + gate[n+1] dx[n+1] (same sequence) + dz[n] ws (channels < 24)
//   dgate[n] = dx[n] . e[n-1],  dz[n] = dgate[n] ls s'(z[n]),  s = sigmoid
//   part_ls[n] = dgate[n] s(z[n]),  part_ws[c][n] = dz[n] e[n, c]
__global__ void __launch_bounds__(256) smear_bwd_kernel(const float* __restrict__ dx, const float* __restrict__ e,
                                                        const float* __restrict__ pls, const float* __restrict__ ws,
                                                        float* __restrict__ de, float* __restrict__ part_ls,
                                                        float* __restrict__ part_ws, int N, int T, int d) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const long off = (long)row * d;
  const int n4 = d / 4;
  const float ls = *pls;
  const bool first = row % T == 0, last = (row + 1) % T == 0;  // row + 1 < N unless last
  const float4* gr = reinterpret_cast<const float4*>(dx + off);
  const float4* er = reinterpret_cast<const float4*>(e + off);
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 e0 = lane < n4 ? er[lane] : zero4;
  const float zn = smear_logit(e0, ws, lane);
  const float sn = sigmoidf_(zn);
  float gnext = 0.f;
  if (!last) {
    const float4 en = lane < n4 ? reinterpret_cast<const float4*>(e + off + d)[lane] : zero4;
    gnext = ls * sigmoidf_(smear_logit(en, ws, lane));
  }
  float dg = 0.f;
  float4 o[MAXV4];
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    o[j] = zero4;
    if (i >= n4) continue;
    const float4 g = gr[i];
    o[j] = g;
    if (!first) {
      const float4 q = reinterpret_cast<const float4*>(e + off - d)[i];
      dg += g.x * q.x + g.y * q.y + g.z * q.z + g.w * q.w;
    }
    if (!last) {
      const float4 q = reinterpret_cast<const float4*>(dx + off + d)[i];
      o[j].x += gnext * q.x; o[j].y += gnext * q.y; o[j].z += gnext * q.z; o[j].w += gnext * q.w;
    }
  }
  dg = wave_sum(dg);
  const float dz = dg * ls * sn * (1.f - sn);
  if (lane < SMEAR_CH / 4) {
    const float4 w = smear_w4(ws, lane);
    o[0].x += dz * w.x; o[0].y += dz * w.y; o[0].z += dz * w.z; o[0].w += dz * w.w;
    part_ws[(long)(4 * lane + 0) * N + row] = dz * e0.x;
    part_ws[(long)(4 * lane + 1) * N + row] = dz * e0.y;
    part_ws[(long)(4 * lane + 2) * N + row] = dz * e0.z;
    part_ws[(long)(4 * lane + 3) * N + row] = dz * e0.w;
  }
  float4* dr = reinterpret_cast<float4*>(de + off);
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i = lane + j * 64;
    if (i < n4) dr[i] = o[j];
  }
  if (lane == 0) part_ls[row] = dg * sn;
}

// dS[j] = sum over rows of part[j][row] (fixed order, fp64), for the entries of the
// extras that are switched on; the other entries get 0.  accumulate: added to dS.
__global__ void __launch_bounds__(256) extras_reduce_kernel(const float* __restrict__ part, int N, int L, int mask,
                                                            float* __restrict__ dS, int accumulate) {
  const int j = blockIdx.x;
  const bool on = j < 2 * L ? (mask & 1) : j == 2 * L + 1 ? (mask & 4) : (mask & 2);
  __shared__ double red[256];
  double s = 0.0;
  if (on)
    for (int n = threadIdx.x; n < N; n += 256) s += (double)part[(long)j * N + n];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dS[j] = (float)(accumulate ? (double)dS[j] + red[0] : red[0]);
}

// S at its identity: residual scales 1, every other entry 0
__global__ void extras_init_kernel(float* S, int L, int n) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n) S[j] = j < L ? 1.f : 0.f;
}

// ---------------------------------------------------------------------------
// Value embeddings: v[n, h] += 3 sigmoid(Wg[h] . a[n, 0:24]) VE[tok[n], h] for each key/
// value head h, in place in the qkv rows [q (H hd) | k (Hkv hd) | v (Hkv hd)].  One wave
// per (token, head); lanes 0..23 form the gate logit, then each lane owns pairs of
// adjacent values (64 lanes cover 128 of them per pass).

constexpr int VE_CH = 24;  // channels of the normed block input the gate reads

template <typename T>
__device__ inline float ve_gate_logit(const T* __restrict__ a_row, const float* __restrict__ wg_row, int lane) {
  return wave_sum(lane < VE_CH ? ld<T>(a_row + lane) * wg_row[lane] : 0.f);
}

// two adjacent act-typed values (4- or 8-byte aligned pairs: hd and every row offset even)
template <typename T>
__device__ inline float2 ld2(const T* p);
template <>
__device__ inline float2 ld2<float>(const float* p) { return *reinterpret_cast<const float2*>(p); }
template <>
__device__ inline float2 ld2<bf16_t>(const bf16_t* p) {
  const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(bf2f((bf16_t)(u & 0xffffu)), bf2f((bf16_t)(u >> 16)));
}
template <typename T>
__device__ inline void st2(T* p, float2 v);
template <>
__device__ inline void st2<float>(float* p, float2 v) { *reinterpret_cast<float2*>(p) = v; }
template <>
__device__ inline void st2<bf16_t>(bf16_t* p, float2 v) { *reinterpret_cast<uint32_t*>(p) = pack_bf2(v.x, v.y); }

template <typename T>
__global__ void __launch_bounds__(256) ve_fwd_kernel(T* __restrict__ qkv, const T* __restrict__ a,
                                                     const int32_t* __restrict__ tok, const float* __restrict__ ve,
                                                     const float* __restrict__ wg, float* __restrict__ vg, int N,
                                                     int V, int H, int Hkv, int hd, int d) {
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, head)
  const int lane = threadIdx.x & 63;
  if (w >= (long)N * Hkv) return;
  const int n = (int)(w / Hkv), h = (int)(w % Hkv), t = tok[n];
  const float g = 3.f * sigmoidf_(ve_gate_logit<T>(a + (long)n * d, wg + h * VE_CH, lane));
  if (lane == 0) vg[w] = g;
  if (t < 0 || t >= V) return;  // the gather flags the id; the step then fails
  const float* er = ve + (long)t * Hkv * hd + (long)h * hd;
  T* vr = qkv + (long)n * (H + 2 * Hkv) * hd + (long)(H + Hkv + h) * hd;
  for (int j = 2 * lane; j < hd; j += 128) {
    const float2 v = ld2<T>(vr + j), e = *reinterpret_cast<const float2*>(er + j);
    st2<T>(vr + j, make_float2(v.x + g * e.x, v.y + g * e.y));
  }
}

// backward, from dv = d loss / d v' (v' = v + g ve, g = 3 sigmoid(z)):
//   dve[n, h] = g dv (rows for the table's scatter), dz[n, h] = (dv . ve) g (1 - g / 3),
//   part[n][h * 24 + c] = dz a[n, c] (rows of the gate weights' gradient)
template <typename T>
__global__ void __launch_bounds__(256) ve_bwd_kernel(const T* __restrict__ dqkv, const T* __restrict__ a,
                                                     const int32_t* __restrict__ tok, const float* __restrict__ ve,
                                                     const float* __restrict__ vg, float* __restrict__ dve,
                                                     float* __restrict__ dz, float* __restrict__ part, int N, int V,
                                                     int H, int Hkv, int hd, int d) {
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= (long)N * Hkv) return;
  const int n = (int)(w / Hkv), h = (int)(w % Hkv), t = tok[n];
  const float g = vg[w];
  const float* er = ve + (long)(t < 0 || t >= V ? 0 : t) * Hkv * hd + (long)h * hd;  // bad ids: flagged
  const T* dr = dqkv + (long)n * (H + 2 * Hkv) * hd + (long)(H + Hkv + h) * hd;
  float* out = dve + (long)n * Hkv * hd + (long)h * hd;
  float dot = 0.f;
  for (int j = 2 * lane; j < hd; j += 128) {
    const float2 dv = ld2<T>(dr + j), e = *reinterpret_cast<const float2*>(er + j);
    *reinterpret_cast<float2*>(out + j) = make_float2(g * dv.x, g * dv.y);
    dot += dv.x * e.x + dv.y * e.y;
  }
  const float z = wave_sum(dot) * g * (1.f - g / 3.f);
  if (lane < VE_CH) part[(long)n * Hkv * VE_CH + h * VE_CH + lane] = z * ld<T>(a + (long)n * d + lane);
  if (lane == 0) dz[w] = z;
}

// da[n, c] += sum_h dz[n, h] Wg[h, c] for c < 24 (the gate's path into the block input)
__global__ void __launch_bounds__(256) ve_da_kernel(float* __restrict__ da, const float* __restrict__ dz,
                                                    const float* __restrict__ wg, int N, int Hkv, int d) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)N * VE_CH) return;
  const int n = (int)(i / VE_CH), c = (int)(i % VE_CH);
  float s = 0.f;
  for (int h = 0; h < Hkv; ++h) s += dz[(long)n * Hkv + h] * wg[h * VE_CH + c];
  da[(long)n * d + c] += s;
}

// Column sums of part [N][R] in a fixed order (fp64): stage 1, block (column group of 64,
// row chunk) -> chunk sums; stage 2, per column, the chunk sums in chunk order.
constexpr int CS_CHUNKS = 256;
__global__ void __launch_bounds__(256) colsum_chunk_kernel(const float* __restrict__ part, int N, int R,
                                                           double* __restrict__ chunk) {
  __shared__ double sm[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane, c = blockIdx.y;
  const int per = (N + CS_CHUNKS - 1) / CS_CHUNKS, n0 = c * per, n1 = min(N, n0 + per);
  double s = 0.0;
  if (j < R)
    for (int n = n0 + wave; n < n1; n += 4) s += (double)part[(long)n * R + j];
  sm[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && j < R) chunk[(long)c * R + j] = (sm[0][lane] + sm[1][lane]) + (sm[2][lane] + sm[3][lane]);
}

__global__ void __launch_bounds__(256) colsum_final_kernel(const double* __restrict__ chunk, int R,
                                                           float* __restrict__ out, int accumulate) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= R) return;
  double s = 0.0;
  for (int c = 0; c < CS_CHUNKS; ++c) s += chunk[(long)c * R + j];
  out[j] = (float)(accumulate ? (double)out[j] + s : s);
}

// ---------------------------------------------------------------------------
// RoPE table: cs[t][i] = (cos, sin)(t * base^(-2i/hd)), angles in double precision

__global__ void rope_table_kernel(float* cs, int T, int hd, float base) {
  const int half = hd / 2;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= T * half) return;
  const int t = e / half, i = e % half;
  const double ang = (double)t * pow((double)base, -2.0 * (double)i / (double)hd);
  cs[2 * e] = (float)cos(ang);
  cs[2 * e + 1] = (float)sin(ang);
}

// q and k of every (token, head): rotate half-split pairs, then RMS-normalise the
// head vector; in place in the qkv buffer [B*T][(H + 2 Hkv) hd] (q heads, then Hkv
// k heads, then Hkv v heads).  A "slot" s < H + Hkv names one head vector to
// normalise: s < H is query head s, s >= H key head s - H; it starts at column s hd.
template <typename F>
__device__ inline F* rstd_slot(F* rq, F* rk, long n, int s, int H, int Hkv) {
  return s < H ? rq + n * H + s : rk + n * Hkv + (s - H);
}

template <typename T>
__global__ void __launch_bounds__(256) rope_qknorm_fwd_kernel(T* __restrict__ qkv, const float* __restrict__ cs,
                                                              float* __restrict__ rq, float* __restrict__ rk, int N,
                                                              int Tlen, int H, int Hkv, int hd, float eps) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, slot)
  const int lane = threadIdx.x & 63;
  const int S = H + Hkv;
  if (w >= N * S) return;
  const int n = w / S, sl = w % S;
  const int t = n % Tlen, half = hd / 2;
  T* p = qkv + (long)n * (H + 2 * Hkv) * hd + (long)sl * hd;
  float y1[2], y2[2];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + 64 * j;
    y1[j] = y2[j] = 0.f;
    if (i < half) {
      const float x1 = ld<T>(p + i), x2 = ld<T>(p + i + half);
      const float c = cs[2 * (t * half + i)], s = cs[2 * (t * half + i) + 1];
      y1[j] = x1 * c - x2 * s;
      y2[j] = x1 * s + x2 * c;
      ss += y1[j] * y1[j] + y2[j] * y2[j];
    }
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + 64 * j;
    if (i < half) {
      st<T>(p + i, y1[j] * r);
      st<T>(p + i + half, y2[j] * r);
    }
  }
  if (lane == 0) *rstd_slot(rq, rk, n, sl, H, Hkv) = r;
}

// backward: dz = r (dy - y mean(dy y)) in the rotated frame, then rotate by -angle
template <typename T>
__global__ void __launch_bounds__(256) rope_qknorm_bwd_kernel(T* __restrict__ dqkv, const T* __restrict__ qkv,
                                                              const float* __restrict__ cs, const float* __restrict__ rq,
                                                              const float* __restrict__ rk, int N, int Tlen, int H,
                                                              int Hkv, int hd) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int S = H + Hkv;
  if (w >= N * S) return;
  const int n = w / S, sl = w % S;
  const int t = n % Tlen, half = hd / 2;
  const long off = (long)n * (H + 2 * Hkv) * hd + (long)sl * hd;
  T* dp = dqkv + off;
  const T* yp = qkv + off;
  const float r = *rstd_slot(rq, rk, n, sl, H, Hkv);
  float g1[2], g2[2], a1[2], a2[2];
  float dot = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + 64 * j;
    g1[j] = g2[j] = a1[j] = a2[j] = 0.f;
    if (i < half) {
      g1[j] = ld<T>(dp + i); g2[j] = ld<T>(dp + i + half);
      a1[j] = ld<T>(yp + i); a2[j] = ld<T>(yp + i + half);
      dot += g1[j] * a1[j] + g2[j] * a2[j];
    }
  }
  dot = wave_sum(dot) / (float)hd;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + 64 * j;
    if (i < half) {
      const float z1 = r * (g1[j] - a1[j] * dot), z2 = r * (g2[j] - a2[j] * dot);
      const float c = cs[2 * (t * half + i)], s = cs[2 * (t * half + i) + 1];
      st<T>(dp + i, z1 * c + z2 * s);
      st<T>(dp + i + half, -z1 * s + z2 * c);
    }
  }
}

// bf16 versions with 16-byte accesses: a group of HD/16 lanes owns one head vector;
// lane j holds elements 8j..8j+7 of the first half and their pair partners
// HD/2+8j..HD/2+8j+7, and the group reduces the squared norm with shuffles.

__device__ inline void unpack8(const uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf2f((bf16_t)(w[i] & 0xffffu));
    f[2 * i + 1] = bf2f((bf16_t)(w[i] >> 16));
  }
}
__device__ inline uint4 pack8f(const float (&f)[8]) {
  return make_uint4(pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]), pack_bf2(f[6], f[7]));
}

template <int HD>
__device__ inline float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < HD / 16; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int HD>
__global__ void __launch_bounds__(256) rope_qknorm_fwd_vec_kernel(bf16_t* __restrict__ qkv, const float* __restrict__ cs,
                                                                  float* __restrict__ rq, float* __restrict__ rk, int N,
                                                                  int Tlen, int H, int Hkv, float eps) {
  constexpr int G = HD / 16, HALF = HD / 2;
  const long gid = ((long)blockIdx.x * 256 + threadIdx.x) / G;  // (token, slot), slots fastest
  const int j = threadIdx.x % G;
  const int S = H + Hkv;
  if (gid >= (long)N * S) return;  // whole groups leave together (G divides 64)
  const int n = (int)(gid / S), sl = (int)(gid % S);
  bf16_t* p = qkv + (long)n * (H + 2 * Hkv) * HD + (long)sl * HD;
  float x1[8], x2[8];
  unpack8(*reinterpret_cast<const uint4*>(p + 8 * j), x1);
  unpack8(*reinterpret_cast<const uint4*>(p + HALF + 8 * j), x2);
  const float4* c4 = reinterpret_cast<const float4*>(cs + 2 * ((long)(n % Tlen) * HALF + 8 * j));
  float y1[8], y2[8], ss = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 cc = c4[q];  // (cos, sin) of pairs 2q and 2q+1
    const float c[2] = {cc.x, cc.z}, sn[2] = {cc.y, cc.w};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * q + e;
      y1[i] = x1[i] * c[e] - x2[i] * sn[e];
      y2[i] = x1[i] * sn[e] + x2[i] * c[e];
      ss += y1[i] * y1[i] + y2[i] * y2[i];
    }
  }
  ss = group_sum<HD>(ss);
  const float r = 1.0f / sqrtf(ss / (float)HD + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) { y1[i] *= r; y2[i] *= r; }
  *reinterpret_cast<uint4*>(p + 8 * j) = pack8f(y1);
  *reinterpret_cast<uint4*>(p + HALF + 8 * j) = pack8f(y2);
  if (j == 0) *rstd_slot(rq, rk, n, sl, H, Hkv) = r;
}

template <int HD>
__global__ void __launch_bounds__(256) rope_qknorm_bwd_vec_kernel(bf16_t* __restrict__ dqkv,
                                                                  const bf16_t* __restrict__ qkv,
                                                                  const float* __restrict__ cs,
                                                                  const float* __restrict__ rq,
                                                                  const float* __restrict__ rk, int N, int Tlen, int H,
                                                                  int Hkv, float* __restrict__ amax_part) {
  constexpr int G = HD / 16, HALF = HD / 2;
  const long gid = ((long)blockIdx.x * 256 + threadIdx.x) / G;
  const int j = threadIdx.x % G;
  const int S = H + Hkv;
  // amax_part (or null): one entry per wave, max |dq|, |dk| as stored (whole waves stay to
  // reduce it; a thread group is wholly inside or past the end)
  float mo = 0.f;
  if (gid < (long)N * S) {
  const int n = (int)(gid / S), sl = (int)(gid % S);
  const long off = (long)n * (H + 2 * Hkv) * HD + (long)sl * HD;
  bf16_t* dp = dqkv + off;
  const bf16_t* yp = qkv + off;
  float g1[8], g2[8], a1[8], a2[8];
  unpack8(*reinterpret_cast<const uint4*>(dp + 8 * j), g1);
  unpack8(*reinterpret_cast<const uint4*>(dp + HALF + 8 * j), g2);
  unpack8(*reinterpret_cast<const uint4*>(yp + 8 * j), a1);
  unpack8(*reinterpret_cast<const uint4*>(yp + HALF + 8 * j), a2);
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) dot += g1[i] * a1[i] + g2[i] * a2[i];
  dot = group_sum<HD>(dot) / (float)HD;
  const float r = *rstd_slot(rq, rk, n, sl, H, Hkv);
  const float4* c4 = reinterpret_cast<const float4*>(cs + 2 * ((long)(n % Tlen) * HALF + 8 * j));
  float o1[8], o2[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 cc = c4[q];
    const float c[2] = {cc.x, cc.z}, sn[2] = {cc.y, cc.w};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * q + e;
      const float z1 = r * (g1[i] - a1[i] * dot), z2 = r * (g2[i] - a2[i] * dot);
      o1[i] = z1 * c[e] + z2 * sn[e];
      o2[i] = -z1 * sn[e] + z2 * c[e];
    }
  }
  *reinterpret_cast<uint4*>(dp + 8 * j) = pack8f(o1);
  *reinterpret_cast<uint4*>(dp + HALF + 8 * j) = pack8f(o2);
#pragma unroll
  for (int i = 0; i < 8; ++i) mo = fmaxf(mo, fmaxf(fabsf(o1[i]), fabsf(o2[i])));
  }
  if (amax_part) {
    mo = wave_max(mo);
    if ((threadIdx.x & 63) == 0) amax_part[blockIdx.x * 4 + (threadIdx.x >> 6)] = bf16_round(mo);
  }
}

// ---------------------------------------------------------------------------
// fused softmax cross-entropy over a vocabulary row held in registers.
// row_loss[n] = lse - z[y]; dz = (softmax - onehot) * inv_n; argmax (lowest index)

__device__ inline void blk_argmax(float& v, int& idx, float* sv, int* si) {
  // wave level
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
  }
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) { sv[w] = v; si[w] = idx; }
  __syncthreads();
  v = sv[0]; idx = si[0];
  for (int k = 1; k < (int)(blockDim.x >> 6); ++k) {
    if (sv[k] > v || (sv[k] == v && si[k] < idx)) { v = sv[k]; idx = si[k]; }
  }
  __syncthreads();
}

__device__ inline float blk_sum(float v, float* sv) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sv[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int k = 0; k < (int)(blockDim.x >> 6); ++k) s += sv[k];
  __syncthreads();
  return s;
}

// dz_part (or null): dz_part[4 n + wave] = max |dz| over the wave's part of row n, as stored
template <typename T, int C>  // C float4 per thread, 256 threads -> V = 1024*C
__global__ void __launch_bounds__(256) ce_kernel(const float* __restrict__ z, const int32_t* __restrict__ tgt,
                                                 T* __restrict__ dz, float* __restrict__ row_loss,
                                                 int32_t* __restrict__ amax, int V, float inv_n, int* err,
                                                 float* __restrict__ dz_part) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const long n = blockIdx.x;
  const float4* zr = reinterpret_cast<const float4*>(z + n * V);
  float4 v[C];
  float mx = -INFINITY;
  int mi = 0x7fffffff;
  bool bad = false;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int i4 = threadIdx.x + c * 256;
    v[c] = zr[i4];
    const float e[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bad |= !isfinite(e[k]);
      if (e[k] > mx) { mx = e[k]; mi = 4 * i4 + k; }
    }
  }
  blk_argmax(mx, mi, sv, si);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    v[c].x = __expf(v[c].x - mx); v[c].y = __expf(v[c].y - mx);
    v[c].z = __expf(v[c].z - mx); v[c].w = __expf(v[c].w - mx);
    s += (v[c].x + v[c].y) + (v[c].z + v[c].w);
  }
  s = blk_sum(s, sv);
  const int y = tgt[n];
  const bool yok = (y >= 0 && y < V);
  const float inv = 1.f / s;
  const float sc = inv * inv_n;
  T* dr = dz + n * V;
  float mp = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int i4 = threadIdx.x + c * 256;
    float4 p = make_float4(v[c].x * sc, v[c].y * sc, v[c].z * sc, v[c].w * sc);
    if (yok && (y >> 2) == i4) {
      const int k = y & 3;
      if (k == 0) p.x -= inv_n; else if (k == 1) p.y -= inv_n; else if (k == 2) p.z -= inv_n; else p.w -= inv_n;
    }
    st4<T>(dr + 4 * i4, p);
    mp = fmaxf(mp, max4abs(p));
  }
  if (dz_part) {
    mp = wave_max(mp);
    if ((threadIdx.x & 63) == 0) dz_part[n * 4 + (threadIdx.x >> 6)] = round_act<T>(mp);
  }
  if (threadIdx.x == 0) {
    const float zy = yok ? z[n * V + y] : 0.f;
    row_loss[n] = (mx + logf(s)) - zy;
    amax[n] = mi;
    if (!yok) atomicOr(err, 1);
  }
  if (bad) atomicOr(err, 2);
}

// V a multiple of 4096: two passes over the row with few registers, so that two rows
// share a CU and one row's reductions and stores overlap the other's loads (the
// register-resident ce_kernel holds a whole row per CU at 256 VGPRs, one wave per SIMD,
// and its load, reduce and store phases leave HBM idle in turn).  Pass 1 streams the row
// in groups of CE_G float4 per thread with an online maximum and sum of exponentials
// (the per-thread sum is rescaled when a group raises the maximum), and the lowest-index
// argmax; the per-thread sums are combined at the row maximum.  Pass 2 re-reads the row,
// which the first pass has just brought into the caches (the launch reserves LDS so that
// at most two rows are in flight per CU), and writes dz.
constexpr int CE_G = 16;
constexpr int CE_LDS_RESERVE = 56 * 1024;  // three would exceed the CU's 160 KB
template <typename T>
__global__ void __launch_bounds__(256) ce_stream_kernel(const float* __restrict__ z, const int32_t* __restrict__ tgt,
                                                        T* __restrict__ dz, float* __restrict__ row_loss,
                                                        int32_t* __restrict__ amax, int V, float inv_n, int* err,
                                                        float* __restrict__ dz_part) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const long n = blockIdx.x;
  const float4* zr = reinterpret_cast<const float4*>(z + n * V);
  const int ng = V / (1024 * CE_G);  // groups per thread
  float mx = -INFINITY, ts = 0.f;    // running maximum and sum of exp(x - mx) of the thread
  int mi = 0x7fffffff;
  bool bad = false;
  for (int gi = 0; gi < ng; ++gi) {
    float4 v[CE_G];
#pragma unroll
    for (int c = 0; c < CE_G; ++c) v[c] = zr[threadIdx.x + (gi * CE_G + c) * 256];
    float gm = mx;
#pragma unroll
    for (int c = 0; c < CE_G; ++c) {
      const int i4 = threadIdx.x + (gi * CE_G + c) * 256;
      const float e[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        bad |= !isfinite(e[k]);
        if (e[k] > gm) { gm = e[k]; mi = 4 * i4 + k; }
      }
    }
    if (gm > mx) { ts *= __expf(mx - gm); mx = gm; }  // exp(-inf) = 0 before the first group
#pragma unroll
    for (int c = 0; c < CE_G; ++c)
      ts += (__expf(v[c].x - mx) + __expf(v[c].y - mx)) + (__expf(v[c].z - mx) + __expf(v[c].w - mx));
  }
  float rm = mx;
  int ri = mi;
  blk_argmax(rm, ri, sv, si);
  const float s = blk_sum(ts * __expf(mx - rm), sv);
  const int y = tgt[n];
  const bool yok = (y >= 0 && y < V);
  const float sc = (1.f / s) * inv_n;
  T* dr = dz + n * V;
  float mp = 0.f;
  for (int gi = 0; gi < ng; ++gi) {
    float4 v[CE_G];
#pragma unroll
    for (int c = 0; c < CE_G; ++c) v[c] = zr[threadIdx.x + (gi * CE_G + c) * 256];
#pragma unroll
    for (int c = 0; c < CE_G; ++c) {
      const int i4 = threadIdx.x + (gi * CE_G + c) * 256;
      float4 p = make_float4(__expf(v[c].x - rm) * sc, __expf(v[c].y - rm) * sc, __expf(v[c].z - rm) * sc,
                             __expf(v[c].w - rm) * sc);
      if (yok && (y >> 2) == i4) {
        const int k = y & 3;
        if (k == 0) p.x -= inv_n; else if (k == 1) p.y -= inv_n; else if (k == 2) p.z -= inv_n; else p.w -= inv_n;
      }
      st4<T>(dr + 4 * i4, p);
      mp = fmaxf(mp, max4abs(p));
    }
  }
  if (dz_part) {
    mp = wave_max(mp);
    if ((threadIdx.x & 63) == 0) dz_part[n * 4 + (threadIdx.x >> 6)] = round_act<T>(mp);
  }
  if (threadIdx.x == 0) {
    const float zy = yok ? z[n * V + y] : 0.f;
    row_loss[n] = (rm + logf(s)) - zy;
    amax[n] = ri;
    if (!yok) atomicOr(err, 1);
  }
  if (bad) atomicOr(err, 2);
}

// any V: three passes over the row from memory
template <typename T>
__global__ void __launch_bounds__(256) ce_generic_kernel(const float* __restrict__ z, const int32_t* __restrict__ tgt,
                                                         T* __restrict__ dz, float* __restrict__ row_loss,
                                                         int32_t* __restrict__ amax, int V, float inv_n, int* err,
                                                         float* __restrict__ dz_part) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const long n = blockIdx.x;
  const float* zr = z + n * V;
  float mx = -INFINITY;
  int mi = 0x7fffffff;
  bool bad = false;
  for (int i = threadIdx.x; i < V; i += 256) {
    const float e = zr[i];
    bad |= !isfinite(e);
    if (e > mx) { mx = e; mi = i; }
  }
  blk_argmax(mx, mi, sv, si);
  float s = 0.f;
  for (int i = threadIdx.x; i < V; i += 256) s += __expf(zr[i] - mx);
  s = blk_sum(s, sv);
  const int y = tgt[n];
  const bool yok = (y >= 0 && y < V);
  const float inv = 1.f / s;
  float mp = 0.f;
  for (int i = threadIdx.x; i < V; i += 256) {
    float p = __expf(zr[i] - mx) * inv * inv_n;
    if (i == y) p -= inv_n;
    st<T>(dz + n * V + i, p);
    mp = fmaxf(mp, fabsf(p));
  }
  if (dz_part) {
    mp = wave_max(mp);
    if ((threadIdx.x & 63) == 0) dz_part[n * 4 + (threadIdx.x >> 6)] = round_act<T>(mp);
  }
  if (threadIdx.x == 0) {
    row_loss[n] = (mx + logf(s)) - (yok ? zr[y] : 0.f);
    amax[n] = mi;
    if (!yok) atomicOr(err, 1);
  }
  if (bad) atomicOr(err, 2);
}

// deterministic sum of n floats into one double (one block, fixed order)
__global__ void __launch_bounds__(256) sum_rows_kernel(const float* __restrict__ x, int n, double* out) {
  __shared__ double sd[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += (double)x[i];
  sd[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sd[threadIdx.x] += sd[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = sd[0];
}

// ---------------------------------------------------------------------------
// deterministic embedding backward
//   1 per-chunk histograms  table[p][v] (chunks of 1024 positions)
//   2 per token: exclusive prefix over chunks, total count
//   3 exclusive scan of counts over the vocabulary -> offsets
//   4 stable fill: sorted[offsets[v] + table[p][v] + rank within chunk] = n
//   5 segment sums: fixed segments of 64 sorted entries, one partial per run
//   6 per token: sum its runs' partials in order (zero rows for absent ids)

constexpr int SC_CHUNK = 1024;
constexpr int SC_SEG = 64;

__global__ void __launch_bounds__(SC_CHUNK) sc_hist_kernel(const int32_t* tok, int N, int V, int* table) {
  const int n = blockIdx.x * SC_CHUNK + threadIdx.x;
  if (n < N) {
    const int t = tok[n];
    if (t >= 0 && t < V) atomicAdd(&table[(long)blockIdx.x * V + t], 1);
  }
}

__global__ void __launch_bounds__(256) sc_colscan_kernel(int* table, int P, int V, int* counts) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= V) return;
  int run = 0;
  for (int p = 0; p < P; ++p) {
    const int c = table[(long)p * V + v];
    table[(long)p * V + v] = run;
    run += c;
  }
  counts[v] = run;
}

__global__ void __launch_bounds__(1024) sc_vscan_kernel(const int* counts, int V, int* offsets) {
  __shared__ int part[1024];
  const int per = (V + 1023) / 1024;
  const int b = threadIdx.x * per;
  int s = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < V) s += counts[b + i];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan of 1024 partial sums
  for (int o = 1; o < 1024; o <<= 1) {
    const int add = (int)threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;
  for (int i = 0; i < per; ++i)
    if (b + i < V) { offsets[b + i] = run; run += counts[b + i]; }
  if (threadIdx.x == 1023) offsets[V] = part[1023];
}

__global__ void __launch_bounds__(SC_CHUNK) sc_fill_kernel(const int32_t* tok, int N, int V, const int* table,
                                                           const int* offsets, int* sorted) {
  __shared__ int st_tok[SC_CHUNK];
  const int base = blockIdx.x * SC_CHUNK;
  const int n = base + threadIdx.x;
  const int t = n < N ? tok[n] : -1;
  st_tok[threadIdx.x] = t;
  __syncthreads();
  if (n >= N || t < 0 || t >= V) return;
  int rank = 0;
  for (int m = 0; m < (int)threadIdx.x; ++m) rank += (st_tok[m] == t);
  sorted[offsets[t] + table[(long)blockIdx.x * V + t] + rank] = n;
}

// segments of SC_SEG sorted entries x column chunks of 256 floats (64 lanes x float4)
__global__ void __launch_bounds__(64) sc_segsum_kernel(const int32_t* tok, const int* sorted, const int* nsorted_p,
                                                       const float* dh, int d, float* partial) {
  const int nsorted = *nsorted_p;  // positions with a valid id (the rest of sorted is unfilled)
  const int s0 = blockIdx.x * SC_SEG;
  const int c = blockIdx.y * 256 + threadIdx.x * 4;
  const bool on = c < d;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int run_start = s0;
  const int s1 = min(s0 + SC_SEG, nsorted);
  for (int i = s0; i < s1; ++i) {
    const int row = sorted[i];
    if (on) {
      const float4 x = *reinterpret_cast<const float4*>(dh + (long)row * d + c);
      acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
    const bool last = (i + 1 == s1) || (tok[sorted[i + 1]] != tok[row]);
    if (last) {
      if (on) *reinterpret_cast<float4*>(partial + (long)run_start * d + c) = acc;
      acc = make_float4(0.f, 0.f, 0.f, 0.f);
      run_start = i + 1;
    }
  }
}

__global__ void __launch_bounds__(64) sc_combine_kernel(const int* offsets, const float* partial, int d, float* dE,
                                                        int accumulate) {
  const int v = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x * 4;
  if (c >= d) return;
  const int b = offsets[v], e = offsets[v + 1];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (e > b) {
    for (int s = b / SC_SEG; s <= (e - 1) / SC_SEG; ++s) {
      const int start = max(b, s * SC_SEG);
      const float4 x = *reinterpret_cast<const float4*>(partial + (long)start * d + c);
      acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
    }
  }
  float4* out = reinterpret_cast<float4*>(dE + (long)v * d + c);
  if (accumulate) {
    const float4 o = *out;
    acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
  }
  *out = acc;
}

// ---------------------------------------------------------------------------
// misc

template <typename T>
__global__ void cast_kernel(const float* __restrict__ x, T* __restrict__ y, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    st<T>(y + i, x[i]);
}

__global__ void zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

__device__ inline uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// counter-based N(0, std^2): SplitMix64 on (seed, stream, index) -> Box-Muller
__global__ void fill_normal_kernel(float* w, size_t n, uint64_t seed, uint64_t sid, float stddev) {
  const uint64_t key = splitmix64(seed ^ splitmix64(sid + 0x632BE59BD9B4E019ull));
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const uint64_t r1 = splitmix64(key + 2 * i), r2 = splitmix64(key + 2 * i + 1);
    const double u1 = ((double)(r1 >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    const double u2 = (double)(r2 >> 11) * (1.0 / 9007199254740992.0);
    w[i] = (float)(stddev * sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
  }
}


// AdamW on one flat fp32 tensor: m, v moments; rbc1 = 1 / (1 - b1^t), rbc2 = 1 / (1 - b2^t);
// the decay acts on the weight before the step; wa (optional) receives the new weight
// in the activation type
template <typename T>
__global__ void __launch_bounds__(256) adamw_kernel(float* __restrict__ w, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v, T* __restrict__ wa,
                                                    size_t n, float lr, float b1, float b2, float eps, float wd,
                                                    float rbc1, float rbc2) {
  auto one = [&](float& wi, float gi, float& mi, float& vi) {
    mi = b1 * mi + (1.f - b1) * gi;
    vi = b2 * vi + (1.f - b2) * gi * gi;
    wi = wi - lr * wd * wi - lr * (mi * rbc1) / (sqrtf(vi * rbc2) + eps);
  };
  const size_t stride = (size_t)gridDim.x * blockDim.x, t = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t n4 = n / 4;
  for (size_t i = t; i < n4; i += stride) {
    float4 w4 = reinterpret_cast<float4*>(w)[i], m4 = reinterpret_cast<float4*>(m)[i],
           v4 = reinterpret_cast<float4*>(v)[i];
    const float4 g4 = reinterpret_cast<const float4*>(g)[i];
    one(w4.x, g4.x, m4.x, v4.x);
    one(w4.y, g4.y, m4.y, v4.y);
    one(w4.z, g4.z, m4.z, v4.z);
    one(w4.w, g4.w, m4.w, v4.w);
    reinterpret_cast<float4*>(w)[i] = w4;
    reinterpret_cast<float4*>(m)[i] = m4;
    reinterpret_cast<float4*>(v)[i] = v4;
    if (wa) {
      st<T>(wa + 4 * i, w4.x);
      st<T>(wa + 4 * i + 1, w4.y);
      st<T>(wa + 4 * i + 2, w4.z);
      st<T>(wa + 4 * i + 3, w4.w);
    }
  }
  for (size_t i = n4 * 4 + t; i < n; i += stride) {
    one(w[i], g[i], m[i], v[i]);
    if (wa) st<T>(wa + i, w[i]);
  }
}


// heavy-ball momentum m = mu m + g on every block matrix, and the per-part sums of the
// new m^2 (fp64) for the Frobenius norms, in one pass; matrices start at multiples of
// 4 floats, each part covers whole float4s (the last part also the scalar tail)
__global__ void __launch_bounds__(256) momentum_sumsq_kernel(float* __restrict__ m, const float* __restrict__ g,
                                                             float mu, const long* offs, const long* sizes, int parts,
                                                             double* partial) {
  __shared__ double sd[4];
  const int mat = blockIdx.y, part = blockIdx.x;
  float* mp = m + offs[mat];
  const float* gp = g + offs[mat];
  const long n = sizes[mat], n4 = n / 4;
  const long per = (n4 + parts - 1) / parts;
  const long b = part * per, e = min(n4, b + per);
  double s = 0.0;
  // four float4 of each operand per thread in flight before any is used
  for (long i0 = b + threadIdx.x; i0 < e; i0 += 4 * 256) {
    float4 a[4], q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long i = i0 + k * 256;
      if (i < e) { a[k] = reinterpret_cast<float4*>(mp)[i]; q[k] = reinterpret_cast<const float4*>(gp)[i]; }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long i = i0 + k * 256;
      if (i >= e) break;
      float4 v = a[k];
      v.x = mu * v.x + q[k].x; v.y = mu * v.y + q[k].y; v.z = mu * v.z + q[k].z; v.w = mu * v.w + q[k].w;
      reinterpret_cast<float4*>(mp)[i] = v;
      s += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
    }
  }
  if (part == parts - 1)
    for (long i = n4 * 4 + threadIdx.x; i < n; i += 256) {
      mp[i] = mu * mp[i] + gp[i];
      s += (double)mp[i] * mp[i];
    }
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) sd[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) partial[(long)mat * parts + part] = (sd[0] + sd[1]) + (sd[2] + sd[3]);
}

__global__ void sumsq_final_kernel(const double* partial, int parts, int nmat, double* out) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= nmat) return;
  double s = 0.0;
  for (int k = 0; k < parts; ++k) s += partial[(long)m * parts + k];
  out[m] = s;
}

// X = src / (sqrt(sumsq) + eps), written transposed ([cols][rows]) when asked; 32x32 LDS tiles
template <typename T>
__device__ inline void st_hilo(T* hi, T* lo, long o, float v) {
  st<T>(hi + o, v);
  if (lo) st<T>(lo + o, v - ld<T>(hi + o));
}

template <typename T>
__global__ void __launch_bounds__(256) ns_normalize_kernel(const float* __restrict__ src, const double* sumsq, int mat,
                                                           float eps, int rows, int cols, int transpose,
                                                           float* __restrict__ xf, T* __restrict__ xa,
                                                           T* __restrict__ xlo) {
  __shared__ float tile[32][33];
  const float scale = (float)(1.0 / (sqrt(sumsq[mat]) + (double)eps));
  const int tr = blockIdx.y * 32, tc = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  if (!transpose) {
    for (int i = ty; i < 32; i += 8) {
      const int r = tr + i, c = tc + tx;
      if (r < rows && c < cols) {
        const float v = src[(long)r * cols + c] * scale;
        xf[(long)r * cols + c] = v;
        st_hilo<T>(xa, xlo, (long)r * cols + c, v);
      }
    }
    return;
  }
  for (int i = ty; i < 32; i += 8) {
    const int r = tr + i, c = tc + tx;
    tile[i][tx] = (r < rows && c < cols) ? src[(long)r * cols + c] * scale : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = tc + i, r = tr + tx;  // output row c, column r of the [cols][rows] matrix
    if (r < rows && c < cols) {
      const float v = tile[tx][i];
      xf[(long)c * rows + r] = v;
      st_hilo<T>(xa, xlo, (long)c * rows + r, v);
    }
  }
}

// The transposed form on 64 x 64 tiles (rows and cols multiples of 64): 16 lanes per
// 256-byte row with float4 accesses on both sides of the transpose; the tile's row
// stride of 65 floats puts the lanes of every LDS access in 64 different banks
template <typename T>
__global__ void __launch_bounds__(256) ns_normalize_t64_kernel(const float* __restrict__ src, const double* sumsq,
                                                               int mat, float eps, int rows, int cols,
                                                               float* __restrict__ xf, T* __restrict__ xa,
                                                               T* __restrict__ xlo) {
  __shared__ float tile[64][65];
  const float scale = (float)(1.0 / (sqrt(sumsq[mat]) + (double)eps));
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x, q = (t & 15) * 4, i0 = t >> 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {  // rows r0 + i of src, columns c0 + q .. + 3
    const int i = i0 + 16 * p;
    const float4 a = *reinterpret_cast<const float4*>(src + (long)(r0 + i) * cols + c0 + q);
    tile[i][q] = a.x * scale;
    tile[i][q + 1] = a.y * scale;
    tile[i][q + 2] = a.z * scale;
    tile[i][q + 3] = a.w * scale;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p) {  // output row c0 + c ([cols][rows]), elements r0 + q .. + 3
    const int c = i0 + 16 * p;
    const float4 v = make_float4(tile[q][c], tile[q + 1][c], tile[q + 2][c], tile[q + 3][c]);
    const long o = (long)(c0 + c) * rows + r0 + q;
    *reinterpret_cast<float4*>(xf + o) = v;
    st4<T>(xa + o, v);
    if (xlo) {
      const float4 h = make_float4(ld<T>(xa + o), ld<T>(xa + o + 1), ld<T>(xa + o + 2), ld<T>(xa + o + 3));
      st4<T>(xlo + o, make_float4(v.x - h.x, v.y - h.y, v.z - h.z, v.w - h.w));
    }
  }
}

// the same without a transpose, four consecutive elements per thread (n % 4 == 0)
template <typename T>
__global__ void __launch_bounds__(256) ns_normalize_vec_kernel(const float* __restrict__ src, const double* sumsq,
                                                               int mat, float eps, long n4, float* __restrict__ xf,
                                                               T* __restrict__ xa, T* __restrict__ xlo) {
  const float scale = (float)(1.0 / (sqrt(sumsq[mat]) + (double)eps));
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    const float4 a = reinterpret_cast<const float4*>(src)[i];
    const float4 v = make_float4(a.x * scale, a.y * scale, a.z * scale, a.w * scale);
    reinterpret_cast<float4*>(xf)[i] = v;
    st4<T>(xa + 4 * i, v);
    if (xlo) {
      const float4 h = make_float4(ld<T>(xa + 4 * i), ld<T>(xa + 4 * i + 1), ld<T>(xa + 4 * i + 2),
                                   ld<T>(xa + 4 * i + 3));
      st4<T>(xlo + 4 * i, make_float4(v.x - h.x, v.y - h.y, v.z - h.z, v.w - h.w));
    }
  }
}

// the same over many matrices in one launch: blockIdx.y picks the job
template <typename T>
__global__ void __launch_bounds__(256) ns_normalize_batched_kernel(const float* __restrict__ src,
                                                                   const double* sumsq, float eps,
                                                                   const MuonVecJob* __restrict__ jobs,
                                                                   float* __restrict__ xf, T* __restrict__ xa,
                                                                   T* __restrict__ xlo) {
  const MuonVecJob jb = jobs[blockIdx.y];
  const float scale = (float)(1.0 / (sqrt(sumsq[jb.mat]) + (double)eps));
  const float4* s4 = reinterpret_cast<const float4*>(src + jb.src);
  float4* f4 = reinterpret_cast<float4*>(xf + jb.dst);
  T* a = xa + jb.dst;
  T* lo = xlo ? xlo + jb.dst : nullptr;
  const long n4 = jb.n / 4, stride = (long)gridDim.x * 256;
  for (long i0 = blockIdx.x * 256L + threadIdx.x; i0 < n4; i0 += 4 * stride) {
    float4 u[4];  // four loads in flight before the first store
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i0 + k * stride < n4) u[k] = s4[i0 + k * stride];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long i = i0 + k * stride;
      if (i >= n4) break;
      const float4 v = make_float4(u[k].x * scale, u[k].y * scale, u[k].z * scale, u[k].w * scale);
      f4[i] = v;
      st4<T>(a + 4 * i, v);
      if (lo) {
        const float4 h = make_float4(ld<T>(a + 4 * i), ld<T>(a + 4 * i + 1), ld<T>(a + 4 * i + 2), ld<T>(a + 4 * i + 3));
        st4<T>(lo + 4 * i, make_float4(v.x - h.x, v.y - h.y, v.z - h.z, v.w - h.w));
      }
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(256) muon_apply_batched_kernel(float* __restrict__ w, T* __restrict__ wa,
                                                                 const float* __restrict__ x, float lr,
                                                                 const MuonVecJob* __restrict__ jobs,
                                                                 const float* __restrict__ row_scale) {
  const MuonVecJob jb = jobs[blockIdx.y];
  float4* w4 = reinterpret_cast<float4*>(w + jb.src);
  const float4* x4 = reinterpret_cast<const float4*>(x + jb.dst);
  T* a = wa ? wa + jb.wact : nullptr;
  const float* rs = row_scale ? row_scale + jb.srow : nullptr;
  const long n4 = jb.n / 4, stride = (long)gridDim.x * 256;
  for (long i0 = blockIdx.x * 256L + threadIdx.x; i0 < n4; i0 += 4 * stride) {
    float4 v[4], q[4];  // four of each in flight before the first store
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i0 + k * stride < n4) { v[k] = w4[i0 + k * stride]; q[k] = x4[i0 + k * stride]; }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long i = i0 + k * stride;
      if (i >= n4) break;
      const float f = rs ? lr * rs[4 * i / jb.cols] : lr;  // cols % 4 == 0: one row
      float4 o = v[k];
      o.x -= f * q[k].x; o.y -= f * q[k].y; o.z -= f * q[k].z; o.w -= f * q[k].w;
      w4[i] = o;
      if (a) st4<T>(a + 4 * i, o);
    }
  }
}

// W -= lr * X without a transpose, four consecutive elements per thread
template <typename T>
__global__ void __launch_bounds__(256) muon_apply_vec_kernel(float* __restrict__ w, T* __restrict__ wa,
                                                             const float* __restrict__ x, float lr, long n4,
                                                             const float* __restrict__ row_scale, int cols) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    float4 a = reinterpret_cast<float4*>(w)[i];
    const float4 q = reinterpret_cast<const float4*>(x)[i];
    const float f = row_scale ? lr * row_scale[4 * i / cols] : lr;  // cols % 4 == 0: one row
    a.x -= f * q.x; a.y -= f * q.y; a.z -= f * q.z; a.w -= f * q.w;
    reinterpret_cast<float4*>(w)[i] = a;
    if (wa) st4<T>(wa + 4 * i, a);
  }
}

// W -= lr * s[r] * X (X stored [cols][rows] when transposed; s the optional per-row scale);
// refresh the act copy of W
template <typename T>
__global__ void __launch_bounds__(256) muon_apply_kernel(float* __restrict__ w, T* __restrict__ wa,
                                                         const float* __restrict__ x, float lr, int rows, int cols,
                                                         int transposed, const float* __restrict__ row_scale) {
  __shared__ float tile[32][33];
  const int tr = blockIdx.y * 32, tc = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  if (transposed) {
    for (int i = ty; i < 32; i += 8) {  // read X^T tile rows (columns of W)
      const int c = tc + i, r = tr + tx;
      tile[i][tx] = (r < rows && c < cols) ? x[(long)c * rows + r] : 0.f;
    }
    __syncthreads();
  }
  for (int i = ty; i < 32; i += 8) {
    const int r = tr + i, c = tc + tx;
    if (r < rows && c < cols) {
      const float xv = transposed ? tile[tx][i] : x[(long)r * cols + c];
      const float nw = w[(long)r * cols + c] - (row_scale ? lr * row_scale[r] : lr) * xv;
      w[(long)r * cols + c] = nw;
      if (wa) st<T>(wa + (long)r * cols + c, nw);
    }
  }
}

// The transposed apply on 64 x 64 tiles (rows and cols multiples of 64): X^T rows (the
// columns of W) staged through LDS, then W rows updated with float4 accesses (same tile
// layout as ns_normalize_t64_kernel)
template <typename T>
__global__ void __launch_bounds__(256) muon_apply_t64_kernel(float* __restrict__ w, T* __restrict__ wa,
                                                             const float* __restrict__ x, float lr, int rows,
                                                             int cols, const float* __restrict__ row_scale) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x, q = (t & 15) * 4, i0 = t >> 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {  // X^T row c0 + c, elements r0 + q .. + 3
    const int c = i0 + 16 * p;
    const float4 a = *reinterpret_cast<const float4*>(x + (long)(c0 + c) * rows + r0 + q);
    tile[c][q] = a.x;
    tile[c][q + 1] = a.y;
    tile[c][q + 2] = a.z;
    tile[c][q + 3] = a.w;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p) {  // W row r0 + r, columns c0 + q .. + 3
    const int r = i0 + 16 * p;
    const long o = (long)(r0 + r) * cols + c0 + q;
    const float s = row_scale ? lr * row_scale[r0 + r] : lr;
    const float4 wv = *reinterpret_cast<const float4*>(w + o);
    const float4 nw = make_float4(wv.x - s * tile[q][r], wv.y - s * tile[q + 1][r], wv.z - s * tile[q + 2][r],
                                  wv.w - s * tile[q + 3][r]);
    *reinterpret_cast<float4*>(w + o) = nw;
    if (wa) st4<T>(wa + o, nw);
  }
}

// ---------------------------------------------------------------------------
// fp8 e4m3fn (OCP): 1 sign, 4 exponent (bias 7), 3 mantissa bits; max 448, no
// infinities, 0x7F / 0xFF are NaN.  Round to nearest even, saturate to +-448.

__device__ inline uint8_t f32_to_e4m3(float x) {
  const uint8_t sign = (uint8_t)((__float_as_uint(x) >> 24) & 0x80);
  const float a = fabsf(x);
  if (!(a == a)) return 0x7F;
  if (a >= 448.f) return sign | 0x7E;
  if (a < 0.015625f) return sign | (uint8_t)rintf(a * 512.f);  // subnormals, step 2^-9 (8 -> min normal)
  int e = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;      // 2^e <= a < 2^(e+1), e in [-6, 8]
  int mant = (int)rintf((ldexpf(a, -e) - 1.f) * 8.f);
  if (mant == 8) { mant = 0; ++e; }
  int code = ((e + 7) << 3) | mant;
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}

template <typename T>
__global__ void __launch_bounds__(256) amax_kernel(const T* __restrict__ x, long rows, long cols, long ldx,
                                                   unsigned* amax_bits) {
  __shared__ float sm[4];
  float m = 0.f;
  const long n = rows * cols;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long r = i / cols, c = i - r * cols;
    m = fmaxf(m, fabsf(ld<T>(x + r * ldx + c)));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    atomicMax(amax_bits, __float_as_uint(m));
  }
}

// 64x64 tiles through LDS so both the row-major and the transposed copies are coalesced
template <typename T>
__global__ void __launch_bounds__(256) quant_e4m3_kernel(const T* __restrict__ x, int rows, int cols, long ldx,
                                                         const unsigned* amax_bits, uint8_t* __restrict__ q,
                                                         long ldq, uint8_t* __restrict__ qt, long ldqt,
                                                         float* inv_scale) {
  __shared__ uint8_t tile[64][65];
  const float amax = __uint_as_float(*amax_bits);
  const float s = amax > 0.f ? 448.f / amax : 1.f;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *inv_scale = 1.f / s;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    uint8_t b = 0;
    if (r < rows && c < cols) {
      b = f32_to_e4m3(ld<T>(x + (long)r * ldx + c) * s);
      if (q) q[(long)r * ldq + c] = b;
    }
    tile[i][tx] = b;
  }
  if (!qt) return;
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) qt[(long)c * ldqt + r] = tile[tx][i];
  }
}

// 16-byte versions (cols and the leading dimension multiples of 8).  The e4m3 code is
// produced by v_cvt_pk_fp8_f32 (round to nearest even) on values first clamped to
// +-448, which is the saturating encode above.

// eight consecutive elements as loaded; widened to fp32 only where they are used, so
// that a thread can hold several chunks in flight in their stored width
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16_t> {
  uint4 u;
  __device__ inline void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ inline void get(float (&f)[8]) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Raw8<float> {
  float4 a, b;
  __device__ inline void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ inline void get(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

template <typename T>
__device__ inline void load8f(const T* p, float (&f)[8]) {
  Raw8<T> r;
  r.load(p);
  r.get(f);
}

__device__ inline uint2 e4m3x8(const float (&f)[8], float s) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(f[i] * s, -448.f), 448.f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// contiguous rows are one flat range of 8-element chunks, four loads in flight per
// lane; strided rows go row by row (no index division either way)
template <typename T>
__global__ void __launch_bounds__(256) amax_vec_kernel(const T* __restrict__ x, long rows, long cols8, long ldx,
                                                       unsigned* amax_bits) {
  __shared__ float sm[4];
  float m = 0.f;
  auto take = [&](const T* p) {
    float f[8];
    load8f<T>(p, f);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[k]));
  };
  if (ldx == cols8 * 8) {
    const long n = rows * cols8, stride = (long)gridDim.x * 256;
    long i = blockIdx.x * 256L + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
      float f[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8f<T>(x + (i + u * stride) * 8, f[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[u][k]));
    }
    for (; i < n; i += stride) take(x + i * 8);
  } else {
    for (long r = blockIdx.x; r < rows; r += gridDim.x)
      for (long c = threadIdx.x; c < cols8; c += 256) take(x + r * ldx + c * 8);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    atomicMax(amax_bits, __float_as_uint(m));
  }
}

// two-stage form: each block's max into partials[blockIdx.x] (plain stores), then one
// block folds the partials into the slot with a single atomic.  Thousands of atomics on
// one address from every XCD serialise; this keeps the pass bandwidth-bound.
template <typename T>
__global__ void __launch_bounds__(256) amax_part_kernel(const T* __restrict__ x, long rows, long cols8, long ldx,
                                                        float* __restrict__ partials) {
  __shared__ float sm[4];
  float m = 0.f;
  auto take = [&](const T* p) {
    float f[8];
    load8f<T>(p, f);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[k]));
  };
  if (ldx == cols8 * 8) {
    const long n = rows * cols8, stride = (long)gridDim.x * 256;
    long i = blockIdx.x * 256L + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
      float f[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8f<T>(x + (i + u * stride) * 8, f[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(f[u][k]));
    }
    for (; i < n; i += stride) take(x + i * 8);
  } else {
    for (long r = blockIdx.x; r < rows; r += gridDim.x)
      for (long c = threadIdx.x; c < cols8; c += 256) take(x + r * ldx + c * 8);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
}

__global__ void __launch_bounds__(1024) amax_final_kernel(const float* __restrict__ partials, int n,
                                                          unsigned* amax_bits) {
  __shared__ float sm[16];
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) m = fmaxf(m, partials[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w) m = fmaxf(m, sm[w]);
    m = fmaxf(m, sm[0]);
    atomicMax(amax_bits, __float_as_uint(m));
  }
}

// the slot (zeroed) <- max of n non-negative partials: up to 64 blocks over strided chunks,
// one atomic each (max is order-free, so the result is exact and repeatable)
__global__ void __launch_bounds__(256) amax_fold_kernel(const float* __restrict__ part, int n,
                                                        unsigned* amax_bits) {
  __shared__ float sm[4];
  float m = 0.f;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) m = fmaxf(m, part[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(amax_bits, __float_as_uint(fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]))));
}

// a 128x128 tile per block: rows of q and of qt leave as whole 128-byte lines.  Each
// thread converts eight 8-wide row chunks (16 threads per row); qt is read back from
// LDS by columns, eight lanes per 128-byte line of qt.  FULL: the tile lies inside the
// matrix and qt rows are 16-byte aligned, so no chunk or store needs a bounds check
template <typename T, bool FULL>
__global__ void __launch_bounds__(256) quant_e4m3_t128_kernel(const T* __restrict__ x, int rows, int cols, long ldx,
                                                              const unsigned* amax_bits, uint8_t* __restrict__ q,
                                                              long ldq, uint8_t* __restrict__ qt, long ldqt,
                                                              float* inv_scale) {
  // LDS row stride in bytes (8-byte aligned rows); each group of 16 rows is shifted by a
  // further 8 bytes, so the eight row groups that one column read touches start in
  // different banks (544 dwords apart they shared two)
  constexpr int TS = 136;
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * TS + 7 * 8];
  auto lrow = [](int rl) { return rl * TS + (rl >> 4) * 8; };
  const int r0 = blockIdx.y * 128, c0 = blockIdx.x * 128;
  const int t = threadIdx.x, c8 = (t & 15) * 8;
  // the thread's eight chunks are all loaded, in their stored width, before the first is
  // converted (a chunk outside the matrix reads element 0 and is zeroed), so that eight
  // loads per thread are in flight instead of one load-convert-store chain at a time
  Raw8<T> raw[8];
  bool ok[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = r0 + (t >> 4) + 16 * j, c = c0 + c8;
    ok[j] = FULL || (r < rows && c < cols);
    raw[j].load(x + (ok[j] ? (long)r * ldx + c : 0L));
  }
  const float amax = __uint_as_float(*amax_bits);
  const float s = amax > 0.f ? 448.f / amax : 1.f;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *inv_scale = 1.f / s;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rl = (t >> 4) + 16 * j, r = r0 + rl, c = c0 + c8;
    uint2 b = make_uint2(0, 0);
    if (ok[j]) {
      float f[8];
      raw[j].get(f);
      b = e4m3x8(f, s);
      if (q) *reinterpret_cast<uint2*>(q + (long)r * ldq + c) = b;
    }
    if (qt) *reinterpret_cast<uint2*>(tile + lrow(rl) + c8) = b;
  }
  if (!qt) return;
  __syncthreads();
  // qt row c (tile column cl) is the tile's 128 rows: eight lanes write it as one whole
  // 128-byte line, 16 rows each, so that a wave's store covers eight lines (lanes writing
  // 16 bytes into 64 different rows left every line partial)
  const int ch = t & 7, rs = ch * 16, rb = r0 + rs;
  const bool vec = FULL || (rb + 16 <= rows && (ldqt % 16) == 0);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int cl = it * 32 + (t >> 3), c = c0 + cl;
    if (!FULL && (c >= cols || rb >= rows)) continue;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t v = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) v |= (uint32_t)tile[lrow(rs + 4 * k + e) + cl] << (8 * e);
      w[k] = v;
    }
    uint8_t* dst = qt + (long)c * ldqt + rb;
    if (vec) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      for (int e = 0; e < 16 && rb + e < rows; ++e) dst[e] = (uint8_t)(w[e / 4] >> (8 * (e % 4)));
    }
  }
}

// a 64x64 tile per block: each thread converts two 8-wide row chunks; the transposed
// copy is read back from LDS by columns, 16 bytes per thread
template <typename T>
__global__ void __launch_bounds__(256) quant_e4m3_vec_kernel(const T* __restrict__ x, int rows, int cols, long ldx,
                                                             const unsigned* amax_bits, uint8_t* __restrict__ q,
                                                             long ldq, uint8_t* __restrict__ qt, long ldqt,
                                                             float* inv_scale) {
  constexpr int TS = 72;  // LDS row stride in bytes (8-byte aligned rows)
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * TS];
  const float amax = __uint_as_float(*amax_bits);
  const float s = amax > 0.f ? 448.f / amax : 1.f;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *inv_scale = 1.f / s;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x, c8 = (t & 7) * 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rl = (t >> 3) + 32 * j, r = r0 + rl, c = c0 + c8;
    uint2 b = make_uint2(0, 0);
    if (r < rows && c < cols) {
      float f[8];
      load8f<T>(x + (long)r * ldx + c, f);
      b = e4m3x8(f, s);
      if (q) *reinterpret_cast<uint2*>(q + (long)r * ldq + c) = b;
    }
    *reinterpret_cast<uint2*>(tile + rl * TS + c8) = b;
  }
  if (!qt) return;
  __syncthreads();
  const int cl = t >> 2, rs = (t & 3) * 16, c = c0 + cl, rb = r0 + rs;
  if (c >= cols || rb >= rows) return;
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) v |= (uint32_t)tile[(rs + 4 * k + e) * TS + cl] << (8 * e);
    w[k] = v;
  }
  uint8_t* dst = qt + (long)c * ldqt + rb;
  if (rb + 16 <= rows && (ldqt % 16) == 0 && (rb % 16) == 0) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    for (int e = 0; e < 16 && rb + e < rows; ++e) dst[e] = (uint8_t)(w[e / 4] >> (8 * (e % 4)));
  }
}

inline int grid_for(size_t n, int block = 256, int cap = 65536) {
  size_t g = (n + block - 1) / block;
  if (g > (size_t)cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

void launch_embed_gather(const int32_t* tok, const float* E, float* h, int N, int d, int V, int* err,
                         hipStream_t st) {
  hipLaunchKernelGGL(embed_gather_kernel, dim3((N + 3) / 4), dim3(256), 0, st, tok, E, h, N, d, V, err);
}

int launch_rmsnorm_fwd(const float* x, void* y, int yt, float* rstd, int N, int d, float eps, hipStream_t st,
                       float* amax_part, long amax_cap) {
  dim3 g((N + 3) / 4), b(256);
  if (!amax_part || N > amax_cap) amax_part = nullptr;
  if (yt == ACT_BF16)
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16_t>, g, b, 0, st, x, (bf16_t*)y, rstd, N, d, eps, amax_part);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<float>, g, b, 0, st, x, (float*)y, rstd, N, d, eps, amax_part);
  return amax_part ? N : 0;
}

int launch_rmsnorm_bwd(const float* dy, const float* x, const float* rstd, const float* dres, float* dx,
                       void* dxa, int at, int N, int d, float eps, hipStream_t st, float* amax_part, long amax_cap,
                       const void* y) {
  (void)eps;
  dim3 g((N + 3) / 4), b(256);
  if (!amax_part || !dxa || N > amax_cap) amax_part = nullptr;
  if (at == ACT_BF16) {
    if (y)
      hipLaunchKernelGGL((rmsnorm_bwd_kernel<bf16_t, true>), g, b, 0, st, dy, y, rstd, dres, dx, (bf16_t*)dxa, N, d,
                         amax_part);
    else
      hipLaunchKernelGGL((rmsnorm_bwd_kernel<bf16_t, false>), g, b, 0, st, dy, x, rstd, dres, dx, (bf16_t*)dxa, N, d,
                         amax_part);
  } else {
    if (y)
      hipLaunchKernelGGL((rmsnorm_bwd_kernel<float, true>), g, b, 0, st, dy, y, rstd, dres, dx, (float*)dxa, N, d,
                         amax_part);
    else
      hipLaunchKernelGGL((rmsnorm_bwd_kernel<float, false>), g, b, 0, st, dy, x, rstd, dres, dx, (float*)dxa, N, d,
                         amax_part);
  }
  return amax_part ? N : 0;
}

void launch_rope_table(float* cs, int T, int hd, float base, hipStream_t st) {
  const int n = T * (hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, cs, T, hd, base);
}

template <int HD>
static void rope_fwd_vec(bf16_t* qkv, const float* cs, float* rq, float* rk, int N, int T, int H, int Hkv, float eps,
                         hipStream_t st) {
  const long threads = (long)N * (H + Hkv) * (HD / 16);
  hipLaunchKernelGGL(rope_qknorm_fwd_vec_kernel<HD>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, qkv, cs,
                     rq, rk, N, T, H, Hkv, eps);
}

template <int HD>
static int rope_bwd_vec(bf16_t* dqkv, const bf16_t* qkv, const float* cs, const float* rq, const float* rk, int N,
                        int T, int H, int Hkv, hipStream_t st, float* amax_part, long amax_cap) {
  const long threads = (long)N * (H + Hkv) * (HD / 16);
  const long blocks = (threads + 255) / 256;
  if (!amax_part || 4 * blocks > amax_cap) amax_part = nullptr;
  hipLaunchKernelGGL(rope_qknorm_bwd_vec_kernel<HD>, dim3((unsigned)blocks), dim3(256), 0, st, dqkv, qkv, cs, rq, rk,
                     N, T, H, Hkv, amax_part);
  return amax_part ? (int)(4 * blocks) : 0;
}

void launch_rope_qknorm_fwd(void* qkv, int at, const float* cs, float* rq, float* rk, int B, int T, int H, int Hkv,
                            int hd, float eps, hipStream_t st) {
  const int N = B * T;
  if (at == ACT_BF16 && (hd == 128 || hd == 64 || hd == 32)) {
    if (hd == 128) rope_fwd_vec<128>((bf16_t*)qkv, cs, rq, rk, N, T, H, Hkv, eps, st);
    else if (hd == 64) rope_fwd_vec<64>((bf16_t*)qkv, cs, rq, rk, N, T, H, Hkv, eps, st);
    else rope_fwd_vec<32>((bf16_t*)qkv, cs, rq, rk, N, T, H, Hkv, eps, st);
    return;
  }
  dim3 g((N * (H + Hkv) + 3) / 4), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(rope_qknorm_fwd_kernel<bf16_t>, g, b, 0, st, (bf16_t*)qkv, cs, rq, rk, N, T, H, Hkv, hd, eps);
  else
    hipLaunchKernelGGL(rope_qknorm_fwd_kernel<float>, g, b, 0, st, (float*)qkv, cs, rq, rk, N, T, H, Hkv, hd, eps);
}

int launch_rope_qknorm_bwd(void* dqkv, const void* qkv, int at, const float* cs, const float* rq, const float* rk,
                           int B, int T, int H, int Hkv, int hd, hipStream_t st, float* amax_part, long amax_cap) {
  const int N = B * T;
  if (at == ACT_BF16 && (hd == 128 || hd == 64 || hd == 32)) {
    if (hd == 128)
      return rope_bwd_vec<128>((bf16_t*)dqkv, (const bf16_t*)qkv, cs, rq, rk, N, T, H, Hkv, st, amax_part, amax_cap);
    if (hd == 64)
      return rope_bwd_vec<64>((bf16_t*)dqkv, (const bf16_t*)qkv, cs, rq, rk, N, T, H, Hkv, st, amax_part, amax_cap);
    return rope_bwd_vec<32>((bf16_t*)dqkv, (const bf16_t*)qkv, cs, rq, rk, N, T, H, Hkv, st, amax_part, amax_cap);
  }
  dim3 g((N * (H + Hkv) + 3) / 4), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(rope_qknorm_bwd_kernel<bf16_t>, g, b, 0, st, (bf16_t*)dqkv, (const bf16_t*)qkv, cs, rq, rk, N,
                       T, H, Hkv, hd);
  else
    hipLaunchKernelGGL(rope_qknorm_bwd_kernel<float>, g, b, 0, st, (float*)dqkv, (const float*)qkv, cs, rq, rk, N, T,
                       H, Hkv, hd);
  return 0;
}

void launch_mix_rmsnorm_fwd(const float* x, const float* z, const float* pa, float ma, const float* pb, float mb,
                            float* m, void* y, int yt, float* rstd, int N, int d, float eps, hipStream_t st) {
  dim3 g((N + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK), b(256);
  if (yt == ACT_BF16)
    hipLaunchKernelGGL(mix_rmsnorm_fwd_kernel<bf16_t>, g, b, 0, st, x, z, pa, ma, pb, mb, m, (bf16_t*)y, rstd, N, d,
                       eps);
  else
    hipLaunchKernelGGL(mix_rmsnorm_fwd_kernel<float>, g, b, 0, st, x, z, pa, ma, pb, mb, m, (float*)y, rstd, N, d,
                       eps);
}

void launch_rmsnorm_mix_bwd(const float* dy, const float* m, const float* rstd, const float* dres, const float* pa,
                            float ma, const float* pb, float mb, bool b_to_out, const float* add1, const float* add2,
                            float* acc, const float* xa, float* dots_a, float sa, const float* xb, float* dots_b,
                            float sb, float* out, void* outa, int at, int N, int d, hipStream_t st) {
  dim3 g((N + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(rmsnorm_mix_bwd_kernel<bf16_t>, g, b, 0, st, dy, m, rstd, dres, pa, ma, pb, mb, (int)b_to_out,
                       add1, add2, acc, xa, dots_a, sa, xb, dots_b, sb, out, (bf16_t*)outa, N, d);
  else
    hipLaunchKernelGGL(rmsnorm_mix_bwd_kernel<float>, g, b, 0, st, dy, m, rstd, dres, pa, ma, pb, mb, (int)b_to_out,
                       add1, add2, acc, xa, dots_a, sa, xb, dots_b, sb, out, (float*)outa, N, d);
}

void launch_smear_fwd(const float* e, const float* pls, const float* ws, float* x, int N, int T, int d,
                      hipStream_t st) {
  hipLaunchKernelGGL(smear_fwd_kernel, dim3((N + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK), dim3(256), 0, st, e, pls, ws,
                     x, N, T, d);
}

void launch_smear_bwd(const float* dx, const float* e, const float* pls, const float* ws, float* de, float* part_ls,
                      float* part_ws, int N, int T, int d, hipStream_t st) {
  hipLaunchKernelGGL(smear_bwd_kernel, dim3((N + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK), dim3(256), 0, st, dx, e, pls,
                     ws, de, part_ls, part_ws, N, T, d);
}

void launch_extras_reduce(const float* part, int N, int L, int mask, float* dS, bool accumulate, hipStream_t st) {
  hipLaunchKernelGGL(extras_reduce_kernel, dim3(2 * L + 2 + SMEAR_CH), dim3(256), 0, st, part, N, L, mask, dS,
                     (int)accumulate);
}

void launch_extras_init(float* S, int L, hipStream_t st) {
  const int n = 2 * L + 2 + SMEAR_CH;
  hipLaunchKernelGGL(extras_init_kernel, dim3((n + 255) / 256), dim3(256), 0, st, S, L, n);
}

void launch_ve_fwd(void* qkv, int at, const void* a, const int32_t* tok, const float* ve, const float* wg,
                   float* vg, int N, int V, int H, int Hkv, int hd, int d, hipStream_t st) {
  const dim3 g((unsigned)(((long)N * Hkv + 3) / 4)), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(ve_fwd_kernel<bf16_t>, g, b, 0, st, (bf16_t*)qkv, (const bf16_t*)a, tok, ve, wg, vg, N, V, H,
                       Hkv, hd, d);
  else
    hipLaunchKernelGGL(ve_fwd_kernel<float>, g, b, 0, st, (float*)qkv, (const float*)a, tok, ve, wg, vg, N, V, H, Hkv,
                       hd, d);
}

void launch_ve_bwd(const void* dqkv, int at, const void* a, const int32_t* tok, const float* ve, const float* vg,
                   float* dve, float* dz, float* part, int N, int V, int H, int Hkv, int hd, int d,
                   hipStream_t st) {
  const dim3 g((unsigned)(((long)N * Hkv + 3) / 4)), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(ve_bwd_kernel<bf16_t>, g, b, 0, st, (const bf16_t*)dqkv, (const bf16_t*)a, tok, ve, vg, dve,
                       dz, part, N, V, H, Hkv, hd, d);
  else
    hipLaunchKernelGGL(ve_bwd_kernel<float>, g, b, 0, st, (const float*)dqkv, (const float*)a, tok, ve, vg, dve, dz,
                       part, N, V, H, Hkv, hd, d);
}

void launch_ve_da(float* da, const float* dz, const float* wg, int N, int Hkv, int d, hipStream_t st) {
  hipLaunchKernelGGL(ve_da_kernel, dim3((unsigned)(((long)N * VE_CH + 255) / 256)), dim3(256), 0, st, da, dz, wg, N,
                     Hkv, d);
}

size_t colsum_ws_bytes(int R) { return (size_t)CS_CHUNKS * R * 8; }

void launch_colsum(const float* part, int N, int R, void* ws, float* out, bool accumulate, hipStream_t st) {
  if (R <= 0) return;
  hipLaunchKernelGGL(colsum_chunk_kernel, dim3((R + 63) / 64, CS_CHUNKS), dim3(256), 0, st, part, N, R, (double*)ws);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((R + 255) / 256), dim3(256), 0, st, (const double*)ws, R, out,
                     (int)accumulate);
}

// cross-entropy kernel for V a multiple of 16384: 0 = two-pass streaming (ce_stream_kernel),
// 1 = the row held in registers (ce_kernel); both give the same argmax and, up to the
// order of the exponential sums, the same loss and dz
int g_ce_variant = 0;

template <typename T>
static void ce_dispatch(const float* z, const int32_t* tgt, T* dz, float* rl, int32_t* am, int N, int V, float inv_n,
                        int* err, hipStream_t st, float* pt) {
  dim3 g(N), b(256);
  if (g_ce_variant == 0 && V % (1024 * CE_G) == 0) {
    hipLaunchKernelGGL(ce_stream_kernel<T>, g, b, CE_LDS_RESERVE, st, z, tgt, dz, rl, am, V, inv_n, err, pt);
    return;
  }
  switch (V % 1024 == 0 ? V / 1024 : -1) {
    case 1: hipLaunchKernelGGL((ce_kernel<T, 1>), g, b, 0, st, z, tgt, dz, rl, am, V, inv_n, err, pt); break;
    case 2: hipLaunchKernelGGL((ce_kernel<T, 2>), g, b, 0, st, z, tgt, dz, rl, am, V, inv_n, err, pt); break;
    case 4: hipLaunchKernelGGL((ce_kernel<T, 4>), g, b, 0, st, z, tgt, dz, rl, am, V, inv_n, err, pt); break;
    case 8: hipLaunchKernelGGL((ce_kernel<T, 8>), g, b, 0, st, z, tgt, dz, rl, am, V, inv_n, err, pt); break;
    case 16: hipLaunchKernelGGL((ce_kernel<T, 16>), g, b, 0, st, z, tgt, dz, rl, am, V, inv_n, err, pt); break;
    case 32: hipLaunchKernelGGL((ce_kernel<T, 32>), g, b, 0, st, z, tgt, dz, rl, am, V, inv_n, err, pt); break;
    default: hipLaunchKernelGGL(ce_generic_kernel<T>, g, b, 0, st, z, tgt, dz, rl, am, V, inv_n, err, pt); break;
  }
}

void set_ce_variant(int v) { g_ce_variant = v; }

int launch_cross_entropy(const float* z, const int32_t* tgt, void* dz, int at, float* rl, int32_t* am, int N, int V,
                         float inv_n, int* err, hipStream_t st, float* dz_part, long part_cap) {
  if (N <= 0) return 0;
  if (!dz_part || 4L * N > part_cap) dz_part = nullptr;
  if (at == ACT_BF16)
    ce_dispatch<bf16_t>(z, tgt, (bf16_t*)dz, rl, am, N, V, inv_n, err, st, dz_part);
  else
    ce_dispatch<float>(z, tgt, (float*)dz, rl, am, N, V, inv_n, err, st, dz_part);
  return dz_part ? 4 * N : 0;
}

void launch_sum_rows(const float* x, int n, double* out, hipStream_t st) {
  hipLaunchKernelGGL(sum_rows_kernel, dim3(1), dim3(256), 0, st, x, n, out);
}

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t embed_ws_bytes(int N, int V, int d) {
  const size_t P = (N + SC_CHUNK - 1) / SC_CHUNK;
  return al256(P * (size_t)V * 4) + al256((size_t)V * 4) + al256(((size_t)V + 1) * 4) + al256((size_t)N * 4) +
         al256((size_t)N * d * 4);
}

// the sort of the token ids (counts per id, their offsets, positions grouped by id in
// increasing order) in ws; launch_embed_scatter_sorted reuses it for any row width
void launch_embed_sort(const int32_t* tok, int N, int V, void* ws, hipStream_t st) {
  const int P = (N + SC_CHUNK - 1) / SC_CHUNK;
  char* w = (char*)ws;
  int* table = (int*)w; w += al256((size_t)P * V * 4);
  int* counts = (int*)w; w += al256((size_t)V * 4);
  int* offsets = (int*)w; w += al256(((size_t)V + 1) * 4);
  int* sorted = (int*)w;
  launch_zero(table, (size_t)P * V * 4, st);
  if (N > 0) hipLaunchKernelGGL(sc_hist_kernel, dim3(P), dim3(SC_CHUNK), 0, st, tok, N, V, table);
  hipLaunchKernelGGL(sc_colscan_kernel, dim3((V + 255) / 256), dim3(256), 0, st, table, P, V, counts);
  hipLaunchKernelGGL(sc_vscan_kernel, dim3(1), dim3(1024), 0, st, counts, V, offsets);
  // every valid position gets a slot; out-of-range ids were flagged by the gather
  if (N > 0) hipLaunchKernelGGL(sc_fill_kernel, dim3(P), dim3(SC_CHUNK), 0, st, tok, N, V, table, offsets, sorted);
}

void launch_embed_scatter_sorted(const int32_t* tok, const float* dh, float* dE, int N, int V, int d, void* ws,
                                 hipStream_t st, bool accumulate) {
  const int P = (N + SC_CHUNK - 1) / SC_CHUNK;
  char* w = (char*)ws;
  w += al256((size_t)P * V * 4) + al256((size_t)V * 4);
  int* offsets = (int*)w; w += al256(((size_t)V + 1) * 4);
  int* sorted = (int*)w; w += al256((size_t)N * 4);
  float* partial = (float*)w;
  if (N > 0)
    hipLaunchKernelGGL(sc_segsum_kernel, dim3((N + SC_SEG - 1) / SC_SEG, (d + 255) / 256), dim3(64), 0, st, tok,
                       sorted, offsets + V, dh, d, partial);
  hipLaunchKernelGGL(sc_combine_kernel, dim3(V, (d + 255) / 256), dim3(64), 0, st, offsets, partial, d, dE,
                     (int)accumulate);
}

void launch_embed_scatter(const int32_t* tok, const float* dh, float* dE, int N, int V, int d, void* ws,
                          int32_t* sorted_out, hipStream_t st, bool accumulate) {
  launch_embed_sort(tok, N, V, ws, st);
  launch_embed_scatter_sorted(tok, dh, dE, N, V, d, ws, st, accumulate);
  if (sorted_out && N > 0) {
    const int P = (N + SC_CHUNK - 1) / SC_CHUNK;
    const char* w = (const char*)ws + al256((size_t)P * V * 4) + al256((size_t)V * 4) + al256(((size_t)V + 1) * 4);
    (void)hipMemcpyAsync(sorted_out, w, (size_t)N * 4, hipMemcpyDeviceToDevice, st);
  }
}

void launch_cast_f32_to_act(const float* x, void* y, int at, size_t n, hipStream_t st) {
  if (at == ACT_BF16)
    hipLaunchKernelGGL(cast_kernel<bf16_t>, dim3(grid_for(n)), dim3(256), 0, st, x, (bf16_t*)y, n);
  else
    hipLaunchKernelGGL(cast_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, x, (float*)y, n);
}

void launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;  // callers pass multiples of 4 bytes
  if (n) hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n)), dim3(256), 0, st, (uint32_t*)p, n);
}

void launch_fill_normal(float* w, size_t n, uint64_t seed, uint64_t sid, float stddev, hipStream_t st) {
  hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(n)), dim3(256), 0, st, w, n, seed, sid, stddev);
}


void launch_momentum_sumsq(float* m, const float* g, float mu, const long* offs, const long* sizes, int nmat,
                           double* partial, int parts, double* out, hipStream_t st) {
  hipLaunchKernelGGL(momentum_sumsq_kernel, dim3(parts, nmat), dim3(256), 0, st, m, g, mu, offs, sizes, parts,
                     partial);
  hipLaunchKernelGGL(sumsq_final_kernel, dim3((nmat + 63) / 64), dim3(64), 0, st, partial, parts, nmat, out);
}


void launch_ns_normalize(const float* src, const double* sumsq, int mat, float eps, int rows, int cols, bool tr,
                         float* xf, void* xa, void* xlo, int at, hipStream_t st) {
  const long n = (long)rows * cols;
  if (!tr && n % 4 == 0 && at != ACT_F32) {
    const long n4 = n / 4;
    const dim3 gv((unsigned)std::min<long>((n4 + 255) / 256, 4096));
    if (at == ACT_BF16)
      hipLaunchKernelGGL(ns_normalize_vec_kernel<bf16_t>, gv, dim3(256), 0, st, src, sumsq, mat, eps, n4, xf,
                         (bf16_t*)xa, (bf16_t*)xlo);
    else
      hipLaunchKernelGGL(ns_normalize_vec_kernel<f16_t>, gv, dim3(256), 0, st, src, sumsq, mat, eps, n4, xf,
                         (f16_t*)xa, (f16_t*)xlo);
    return;
  }
  const bool a16 = ((uintptr_t)src | (uintptr_t)xf) % 16 == 0 && ((uintptr_t)xa | (uintptr_t)xlo) % 8 == 0;
  if (tr && rows % 64 == 0 && cols % 64 == 0 && a16 && at != ACT_F32) {
    const dim3 gt(cols / 64, rows / 64);
    if (at == ACT_BF16)
      hipLaunchKernelGGL(ns_normalize_t64_kernel<bf16_t>, gt, dim3(256), 0, st, src, sumsq, mat, eps, rows, cols, xf,
                         (bf16_t*)xa, (bf16_t*)xlo);
    else
      hipLaunchKernelGGL(ns_normalize_t64_kernel<f16_t>, gt, dim3(256), 0, st, src, sumsq, mat, eps, rows, cols, xf,
                         (f16_t*)xa, (f16_t*)xlo);
    return;
  }
  dim3 g((cols + 31) / 32, (rows + 31) / 32), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(ns_normalize_kernel<bf16_t>, g, b, 0, st, src, sumsq, mat, eps, rows, cols, (int)tr, xf,
                       (bf16_t*)xa, (bf16_t*)xlo);
  else if (at == ACT_F16)
    hipLaunchKernelGGL(ns_normalize_kernel<f16_t>, g, b, 0, st, src, sumsq, mat, eps, rows, cols, (int)tr, xf,
                       (f16_t*)xa, (f16_t*)xlo);
  else
    hipLaunchKernelGGL(ns_normalize_kernel<float>, g, b, 0, st, src, sumsq, mat, eps, rows, cols, (int)tr, xf,
                       (float*)xa, (float*)nullptr);
}

void launch_ns_normalize_batched(const float* src, const double* sumsq, float eps, const MuonVecJob* jobs, int njobs,
                                 float* xf, void* xa, void* xlo, int at, hipStream_t st) {
  if (njobs <= 0) return;
  const dim3 g(64, njobs), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(ns_normalize_batched_kernel<bf16_t>, g, b, 0, st, src, sumsq, eps, jobs, xf, (bf16_t*)xa,
                       (bf16_t*)xlo);
  else if (at == ACT_F16)
    hipLaunchKernelGGL(ns_normalize_batched_kernel<f16_t>, g, b, 0, st, src, sumsq, eps, jobs, xf, (f16_t*)xa,
                       (f16_t*)xlo);
  else
    hipLaunchKernelGGL(ns_normalize_batched_kernel<float>, g, b, 0, st, src, sumsq, eps, jobs, xf, (float*)xa,
                       (float*)nullptr);
}

void launch_muon_apply_batched(float* w, void* wa, int at, const float* x, float lr, const MuonVecJob* jobs,
                               int njobs, const float* row_scale, hipStream_t st) {
  if (njobs <= 0) return;
  const dim3 g(64, njobs), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(muon_apply_batched_kernel<bf16_t>, g, b, 0, st, w, (bf16_t*)wa, x, lr, jobs, row_scale);
  else
    hipLaunchKernelGGL(muon_apply_batched_kernel<float>, g, b, 0, st, w, (float*)wa, x, lr, jobs, row_scale);
}

void launch_muon_apply(float* w, void* wa, int at, const float* x, float lr, int rows, int cols, bool tr,
                       hipStream_t st, const float* row_scale) {
  const long n = (long)rows * cols;
  if (!tr && cols % 4 == 0) {
    const long n4 = n / 4;
    const dim3 gv((unsigned)std::min<long>((n4 + 255) / 256, 4096));
    if (at == ACT_BF16)
      hipLaunchKernelGGL(muon_apply_vec_kernel<bf16_t>, gv, dim3(256), 0, st, w, (bf16_t*)wa, x, lr, n4, row_scale,
                         cols);
    else
      hipLaunchKernelGGL(muon_apply_vec_kernel<float>, gv, dim3(256), 0, st, w, (float*)wa, x, lr, n4, row_scale,
                         cols);
    return;
  }
  const bool a16 = ((uintptr_t)w | (uintptr_t)x) % 16 == 0 && (uintptr_t)wa % 16 == 0;
  if (tr && rows % 64 == 0 && cols % 64 == 0 && a16) {
    const dim3 gt(cols / 64, rows / 64);
    if (at == ACT_BF16)
      hipLaunchKernelGGL(muon_apply_t64_kernel<bf16_t>, gt, dim3(256), 0, st, w, (bf16_t*)wa, x, lr, rows, cols,
                         row_scale);
    else
      hipLaunchKernelGGL(muon_apply_t64_kernel<float>, gt, dim3(256), 0, st, w, (float*)wa, x, lr, rows, cols,
                         row_scale);
    return;
  }
  dim3 g((cols + 31) / 32, (rows + 31) / 32), b(256);
  if (at == ACT_BF16)
    hipLaunchKernelGGL(muon_apply_kernel<bf16_t>, g, b, 0, st, w, (bf16_t*)wa, x, lr, rows, cols, (int)tr, row_scale);
  else
    hipLaunchKernelGGL(muon_apply_kernel<float>, g, b, 0, st, w, (float*)wa, x, lr, rows, cols, (int)tr, row_scale);
}

// NorMuon.  Mean square of each output row of one matrix's update X ([rows][cols], or
// stored [cols][rows] when transposed).  Untransposed: a wave per row.  Transposed: a
// block covers 64 rows (one per lane) and one of NM_CHUNKS column ranges (its 4 waves
// interleaved), writing partial sums that a second pass adds in chunk order.
constexpr int NM_CHUNKS = 16;
__global__ void __launch_bounds__(256) normuon_colsq_kernel(const float* __restrict__ x, int rows, int cols,
                                                            float* __restrict__ part) {
  __shared__ float sm[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * 64 + lane, ch = blockIdx.y;
  const int per = (cols + NM_CHUNKS - 1) / NM_CHUNKS, c0 = ch * per, c1 = min(cols, c0 + per);
  float s = 0.f;
  if (r < rows)
    for (int c = c0 + wave; c < c1; c += 4) {
      const float v = x[(long)c * rows + r];
      s += v * v;
    }
  sm[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && r < rows) part[(long)ch * rows + r] = (sm[0][lane] + sm[1][lane]) + (sm[2][lane] + sm[3][lane]);
}

__global__ void __launch_bounds__(256) normuon_colsq_final_kernel(const float* __restrict__ part, int rows, int cols,
                                                                  float* __restrict__ vmean) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float s = 0.f;
  for (int ch = 0; ch < NM_CHUNKS; ++ch) s += part[(long)ch * rows + r];
  vmean[r] = s / (float)cols;
}

__global__ void __launch_bounds__(256) normuon_rowstats_kernel(const float* __restrict__ x, int rows, int cols,
                                                               float* __restrict__ vmean) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= rows) return;
  float s = 0.f;
  for (int c = lane; c < cols; c += 64) {
    const float v = x[(long)r * cols + c];
    s += v * v;
  }
  s = wave_sum(s);
  if (lane == 0) vmean[r] = s / (float)cols;
}

// one block per matrix (rows roff[m] .. roff[m+1] of the stacked row vectors):
// V = b2 V + (1 - b2) vmean, step = 1 / sqrt(max(V, 1e-10)), and the row scales
// step * sqrt(sum vmean) / max(sqrt(sum vmean step^2), 1e-10) (fixed-order fp64 sums)
__global__ void __launch_bounds__(256) normuon_scale_kernel(const float* __restrict__ vmean, float* __restrict__ V,
                                                            const long* __restrict__ roff, float b2,
                                                            float* __restrict__ scale) {
  __shared__ double red[2][256];
  const long r0 = roff[blockIdx.x], r1 = roff[blockIdx.x + 1];
  double s1 = 0.0, s2 = 0.0;
  for (long r = r0 + threadIdx.x; r < r1; r += 256) {
    const float v = b2 * V[r] + (1.f - b2) * vmean[r];
    V[r] = v;
    const float step = 1.f / sqrtf(fmaxf(v, 1e-10f));
    scale[r] = step;
    s1 += (double)vmean[r];
    s2 += (double)vmean[r] * step * step;
  }
  red[0][threadIdx.x] = s1;
  red[1][threadIdx.x] = s2;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
    }
    __syncthreads();
  }
  const float f = (float)(sqrt(red[0][0]) / fmax(sqrt(red[1][0]), 1e-10));
  for (long r = r0 + threadIdx.x; r < r1; r += 256) scale[r] *= f;
}

size_t normuon_ws_bytes(int max_rows) { return (size_t)NM_CHUNKS * max_rows * 4; }

void launch_normuon_rowstats(const float* x, int rows, int cols, bool transposed, float* vmean, void* ws,
                             hipStream_t st) {
  if (transposed) {
    hipLaunchKernelGGL(normuon_colsq_kernel, dim3((rows + 63) / 64, NM_CHUNKS), dim3(256), 0, st, x, rows, cols,
                       (float*)ws);
    hipLaunchKernelGGL(normuon_colsq_final_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, (const float*)ws, rows,
                       cols, vmean);
  } else {
    hipLaunchKernelGGL(normuon_rowstats_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, x, rows, cols, vmean);
  }
}

void launch_normuon_scale(const float* vmean, float* V, const long* roff, int nmat, float beta2, float* scale,
                          hipStream_t st) {
  hipLaunchKernelGGL(normuon_scale_kernel, dim3(nmat), dim3(256), 0, st, vmean, V, roff, beta2, scale);
}

void launch_adamw(float* w, const float* g, float* m, float* v, void* w_act, int act_type, size_t n, float lr,
                  float b1, float b2, float eps, float wd, float rbc1, float rbc2, hipStream_t st) {
  if (n == 0) return;
  const dim3 grid(grid_for((n + 3) / 4)), block(256);
  if (act_type == ACT_BF16)
    hipLaunchKernelGGL(adamw_kernel<bf16_t>, grid, block, 0, st, w, g, m, v, (bf16_t*)w_act, n, lr, b1, b2, eps, wd,
                       rbc1, rbc2);
  else
    hipLaunchKernelGGL(adamw_kernel<float>, grid, block, 0, st, w, g, m, v, (float*)w_act, n, lr, b1, b2, eps, wd,
                       rbc1, rbc2);
}

void launch_amax(const void* x, int it, long rows, long cols, long ld, unsigned* amax_bits, hipStream_t st,
                 float* partials) {
  const long n = rows * cols;
  if (n <= 0) return;
  if (partials && cols % 8 == 0 && ld % 8 == 0 && ((uintptr_t)x % 16) == 0) {
    const long n8 = n / 8;
    const int g = (int)std::min<long>((n8 + 256L * 8 - 1) / (256L * 8), kAmaxParts);
    if (it == ACT_BF16)
      hipLaunchKernelGGL(amax_part_kernel<bf16_t>, dim3(g), dim3(256), 0, st, (const bf16_t*)x, rows, cols / 8, ld,
                         partials);
    else
      hipLaunchKernelGGL(amax_part_kernel<float>, dim3(g), dim3(256), 0, st, (const float*)x, rows, cols / 8, ld,
                         partials);
    hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(1024), 0, st, partials, g, amax_bits);
    return;
  }
  if (cols % 8 == 0 && ld % 8 == 0 && ((uintptr_t)x % 16) == 0) {
    const long n8 = n / 8;
    const int g8 = (int)std::min<long>((n8 + 255) / 256, 2048);
    if (it == ACT_BF16)
      hipLaunchKernelGGL(amax_vec_kernel<bf16_t>, dim3(g8), dim3(256), 0, st, (const bf16_t*)x, rows, cols / 8, ld,
                         amax_bits);
    else
      hipLaunchKernelGGL(amax_vec_kernel<float>, dim3(g8), dim3(256), 0, st, (const float*)x, rows, cols / 8, ld,
                         amax_bits);
    return;
  }
  const int g = (int)std::min<long>((n + 255) / 256, 2048);
  if (it == ACT_BF16)
    hipLaunchKernelGGL(amax_kernel<bf16_t>, dim3(g), dim3(256), 0, st, (const bf16_t*)x, rows, cols, ld, amax_bits);
  else
    hipLaunchKernelGGL(amax_kernel<float>, dim3(g), dim3(256), 0, st, (const float*)x, rows, cols, ld, amax_bits);
}

void launch_amax_fold(const float* partials, int n, unsigned* amax_bits, hipStream_t st) {
  if (n <= 0) return;
  const int blocks = std::min(64, (n + 2047) / 2048);
  hipLaunchKernelGGL(amax_fold_kernel, dim3(blocks), dim3(256), 0, st, partials, n, amax_bits);
}

void launch_quant_e4m3(const void* x, int it, int rows, int cols, long ld, const unsigned* amax_bits, uint8_t* q,
                       long ldq, uint8_t* qt, long ldqt, float* inv_scale, hipStream_t st) {
  dim3 g((cols + 63) / 64, (rows + 63) / 64), b(256);
  if (rows <= 0 || cols <= 0) return;
  if (cols % 8 == 0 && ld % 8 == 0 && ((uintptr_t)x % 16) == 0 && (!q || (ldq % 8 == 0 && (uintptr_t)q % 8 == 0)) &&
      rows >= 128 && cols >= 128) {
    const dim3 g2((cols + 127) / 128, (rows + 127) / 128);
    const bool full = rows % 128 == 0 && cols % 128 == 0 && (!qt || (ldqt % 16 == 0 && (uintptr_t)qt % 16 == 0));
    if (it == ACT_BF16) {
      if (full)
        hipLaunchKernelGGL((quant_e4m3_t128_kernel<bf16_t, true>), g2, b, 0, st, (const bf16_t*)x, rows, cols, ld,
                           amax_bits, q, ldq, qt, ldqt, inv_scale);
      else
        hipLaunchKernelGGL((quant_e4m3_t128_kernel<bf16_t, false>), g2, b, 0, st, (const bf16_t*)x, rows, cols, ld,
                           amax_bits, q, ldq, qt, ldqt, inv_scale);
    } else {
      if (full)
        hipLaunchKernelGGL((quant_e4m3_t128_kernel<float, true>), g2, b, 0, st, (const float*)x, rows, cols, ld,
                           amax_bits, q, ldq, qt, ldqt, inv_scale);
      else
        hipLaunchKernelGGL((quant_e4m3_t128_kernel<float, false>), g2, b, 0, st, (const float*)x, rows, cols, ld,
                           amax_bits, q, ldq, qt, ldqt, inv_scale);
    }
    return;
  }
  if (cols % 8 == 0 && ld % 8 == 0 && ((uintptr_t)x % 16) == 0 && (!q || (ldq % 8 == 0 && (uintptr_t)q % 8 == 0))) {
    if (it == ACT_BF16)
      hipLaunchKernelGGL(quant_e4m3_vec_kernel<bf16_t>, g, b, 0, st, (const bf16_t*)x, rows, cols, ld, amax_bits, q,
                         ldq, qt, ldqt, inv_scale);
    else
      hipLaunchKernelGGL(quant_e4m3_vec_kernel<float>, g, b, 0, st, (const float*)x, rows, cols, ld, amax_bits, q,
                         ldq, qt, ldqt, inv_scale);
    return;
  }
  if (it == ACT_BF16)
    hipLaunchKernelGGL(quant_e4m3_kernel<bf16_t>, g, b, 0, st, (const bf16_t*)x, rows, cols, ld, amax_bits, q, ldq,
                       qt, ldqt, inv_scale);
  else
    hipLaunchKernelGGL(quant_e4m3_kernel<float>, g, b, 0, st, (const float*)x, rows, cols, ld, amax_bits, q, ldq, qt,
                       ldqt, inv_scale);
}
