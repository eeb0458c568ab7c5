// GEMMs of the GPT step on gfx950.
//
// bf16, large problems (gemm_bf16_dma_kernel): 256x256 tiles, 8 waves, operand
// tiles copied global -> LDS by the buffer-load DMA path, transposed operands read
// with the LDS transpose instruction (see the kernel's comment).
//
// bf16, small problems (gemm_bf16_kernel, 128x128): v_mfma_f32_32x32x16_bf16 with
// LDS double buffering.  Both operands are staged in LDS as [rows][k] (k contiguous,
// rows padded by 16 bytes).  An operand whose reduction index is its slow (row)
// index in memory is transposed on the way in: each thread loads an 8x8 block
// (8 k-rows of 16 bytes), swaps it in registers and stores 8 k-contiguous rows.
//
// Both serve the forward (X W^T), data-gradient (dY W) and weight-gradient
// (dY^T X) products and the Newton-Schulz products.
//
// fp32 path: a plain LDS-tiled SIMT kernel (the all-fp32 configuration).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

typedef unsigned int u32x8_t __attribute__((ext_vector_type(8)));
constexpr int BK = 64;        // bf16 elements of k per LDS stage
constexpr int LDSS = BK + 8;  // LDS row stride in elements (16-byte pad)

// Buffer resource over one operand matrix: raw buffer loads return zeros for
// byte offsets at or past `bytes`, which covers the row tail; the k tail and the
// column tail of transposed operands are mapped to an out-of-range offset.
constexpr uint32_t OOB = 0xFFFFFFF0u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int R, bool KMAJ, int NT>
struct TileLoader {
  static constexpr int NUNIT = KMAJ ? R * (BK / 8) : (R / 8) * (BK / 8);
  static constexpr int UPT = (NUNIT + NT - 1) / NT;  // units per thread
  static constexpr int NREG = KMAJ ? UPT : UPT * 8;
  uint4 regs[NREG];

  // element (row, k) lives at base[row*ld + k] (KMAJ) or base[k*ld + row]
  __device__ inline void load(__amdgpu_buffer_rsrc_t rs, long ld, int row0, int rows, int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (KMAJ) {
        const int r = u >> 3, kc = u & 7;
        const int gk = k0 + kc * 8;
        const bool ok = u < NUNIT && gk < kend && row0 + r < rows;
        regs[i] = buf_load16(rs, ok ? (uint32_t)(((long)(row0 + r) * ld + gk) * 2) : OOB);
      } else {
        const int kb = u & 7, rb = u >> 3;
        const int grow = row0 + rb * 8;
        const bool okr = u < NUNIT && grow < rows;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gk = k0 + kb * 8 + j;
          regs[i * 8 + j] = buf_load16(rs, (okr && gk < kend) ? (uint32_t)(((long)gk * ld + grow) * 2) : OOB);
        }
      }
    }
  }

  __device__ inline void store(bf16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (NUNIT % NT != 0 && u >= NUNIT) continue;
      if (KMAJ) {
        const int r = u >> 3, kc = u & 7;
        *reinterpret_cast<uint4*>(lds + r * LDSS + kc * 8) = regs[i];
      } else {
        const int kb = u & 7, rb = u >> 3;
        uint4 in[8], out[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) in[j] = regs[i * 8 + j];
        transpose8x8_b16(in, out);
#pragma unroll
        for (int r = 0; r < 8; ++r) *reinterpret_cast<uint4*>(lds + (rb * 8 + r) * LDSS + kb * 8) = out[r];
      }
    }
  }
};

// map a linear workgroup id onto (tile_m, tile_n): XCD-contiguous ranges, grouped rows
// (groups of 4 tile rows: the d24 step ran 1.5% faster than with 8, 2% faster than 16)
__device__ inline void tile_coords(int lin, int tilesM, int tilesN, int& tm, int& tn, bool xcd = true) {
  const int total = tilesM * tilesN;
  int id = lin;
  if (xcd && (total & 7) == 0) id = (lin & 7) * (total >> 3) + (lin >> 3);
  constexpr int G = 4;
  const int per_group = G * tilesN;
  const int group = id / per_group;
  const int first = group * G;
  const int gsz = min(tilesM - first, G);
  const int in = id - group * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

template <typename OutT>
__device__ inline void store_act(OutT* p, float v);
template <>
__device__ inline void store_act<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }
template <>
__device__ inline void store_act<float>(float* p, float v) { *p = v; }

template <typename OutT>
__device__ inline float load_act(const OutT* p);
template <>
__device__ inline float load_act<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <>
__device__ inline float load_act<float>(const float* p) { return *p; }

// the epilogue for one output element (row, col) of batch bz
template <typename OutT>
__device__ inline void epilogue_elem(const GemmArgs& p, int bz, int row, int col, float acc) {
  float v = p.alpha * acc;
  if (p.epi == EPI_LINEAR) {
    if (p.Cin) v += p.beta * p.Cin[bz * p.strideCin + (long)row * p.ldcin + col];
    if (p.outF) p.outF[bz * p.strideO + (long)row * p.ldo + col] = v;
    if (p.outA) {
      const long o = bz * p.strideOA + (long)row * p.ldoa + col;
      if (std::is_same<OutT, bf16_t>::value && p.dtype == ACT_F16) {
        _Float16* q = reinterpret_cast<_Float16*>(p.outA) + o;
        *q = (_Float16)v;
        if (p.outA_lo) reinterpret_cast<_Float16*>(p.outA_lo)[o] = (_Float16)(v - (float)*q);
      } else {
        store_act<OutT>(reinterpret_cast<OutT*>(p.outA) + o, v);
        if (p.outA_lo) store_act<OutT>(reinterpret_cast<OutT*>(p.outA_lo) + o, v - load_act<OutT>(reinterpret_cast<OutT*>(p.outA) + o));
      }
    }
  } else if (p.epi == EPI_RELU2) {
    const long o = bz * p.strideOA + (long)row * p.ldoa + col;
    const float r = fmaxf(v, 0.f);
    store_act<OutT>(reinterpret_cast<OutT*>(p.out2) + o, r * r);
  } else {  // EPI_DRELU2: aux holds g = relu(u)^2, whose root is relu(u) (the hardware square
           // root, within an ulp of fp32, far below the bf16 rounding of g itself)
    const long o = bz * p.strideOA + (long)row * p.ldoa + col;
    const float g = load_act<OutT>(reinterpret_cast<const OutT*>(p.aux) + o);
    store_act<OutT>(reinterpret_cast<OutT*>(p.outA) + o, v * 2.f * __builtin_amdgcn_sqrtf(fmaxf(g, 0.f)));
  }
}

// four consecutive columns (col % 4 == 0, col + 3 < N, every leading dimension a
// multiple of 4): one vector load/store per operand instead of four scalar ones.
// 16-bit act outputs are bf16, or fp16 when h (GemmArgs::dtype == ACT_F16)
__device__ inline void st4_act(bf16_t* q, const float (&v)[4], bool h = false) {
  if (h) {
    typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));
    const f16x4v x = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<f16x4v*>(q) = x;
    return;
  }
  typedef unsigned int u2v __attribute__((ext_vector_type(2)));
  u2v x = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  __builtin_nontemporal_store(x, reinterpret_cast<u2v*>(q));
}
__device__ inline void ld4_act(const bf16_t* q, float (&v)[4], bool h = false) {
  if (h) {
    typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));
    const f16x4v x = *reinterpret_cast<const f16x4v*>(q);
    v[0] = (float)x[0]; v[1] = (float)x[1]; v[2] = (float)x[2]; v[3] = (float)x[3];
    return;
  }
  const uint2 u = *reinterpret_cast<const uint2*>(q);
  v[0] = bf2f((bf16_t)(u.x & 0xffff)); v[1] = bf2f((bf16_t)(u.x >> 16));
  v[2] = bf2f((bf16_t)(u.y & 0xffff)); v[3] = bf2f((bf16_t)(u.y >> 16));
}

// Outputs leave with nontemporal stores: written once per launch, they need not
// displace the operands' lines (the epilogue's cost per tile fell 8-13%).
// element t of a float4 by selects (a runtime index into a local array would live in scratch)
__device__ inline float pick4(const float4& a, int t) { return t == 0 ? a.x : t == 1 ? a.y : t == 2 ? a.z : a.w; }
__device__ inline long o_act(const GemmArgs& p, int bz, int row, int col) {
  return bz * p.strideOA + (long)row * p.ldoa + col;
}

// HALF: the fp16-operand instantiations (the Newton-Schulz products), the only ones that read
// CinA
template <bool HALF = false>
__device__ inline bool epi_has_in(const GemmArgs& p) {
  return p.epi == EPI_DRELU2 || (p.epi == EPI_LINEAR && (p.Cin || (HALF && p.CinA)));
}

// the element-wise input of four consecutive outputs: beta * Cin (or CinA), or the EPI_DRELU2
// aux values; zeros where the epilogue has none
template <bool HALF = false>
__device__ inline float4 epi_in4(const GemmArgs& p, int bz, int row, int col) {
  if (p.epi == EPI_DRELU2) {
    float g[4];
    ld4_act(reinterpret_cast<const bf16_t*>(p.aux) + bz * p.strideOA + (long)row * p.ldoa + col, g);
    return make_float4(g[0], g[1], g[2], g[3]);
  }
  if (p.epi == EPI_LINEAR) {
    if (p.Cin) {
      const float4 c = *reinterpret_cast<const float4*>(p.Cin + bz * p.strideCin + (long)row * p.ldcin + col);
      return make_float4(p.beta * c.x, p.beta * c.y, p.beta * c.z, p.beta * c.w);
    }
    if constexpr (HALF) {
      if (p.CinA) {
        float c[4];
        ld4_act(reinterpret_cast<const bf16_t*>(p.CinA) + bz * p.strideCin + (long)row * p.ldcin + col, c, true);
        return make_float4(p.beta * c[0], p.beta * c[1], p.beta * c[2], p.beta * c[3]);
      }
    }
  }
  return make_float4(0.f, 0.f, 0.f, 0.f);
}

// the epilogue of four consecutive outputs a (accumulators) with their input in (epi_in4;
// used when has_in)
template <bool HALF = false>
__device__ inline void epilogue_vec4(const GemmArgs& p, int bz, int row, int col, float4 a, float4 in, bool has_in,
                                     float& mx) {  // mx: running max |stored value| of the RELU2 / DRELU2 outputs
  float v[4] = {p.alpha * a.x, p.alpha * a.y, p.alpha * a.z, p.alpha * a.w};
  if (p.epi == EPI_LINEAR) {
    if (has_in) { v[0] += in.x; v[1] += in.y; v[2] += in.z; v[3] += in.w; }
    if (p.outF) {
      typedef float f4v __attribute__((ext_vector_type(4)));
      f4v x = {v[0], v[1], v[2], v[3]};
      __builtin_nontemporal_store(x, reinterpret_cast<f4v*>(p.outF + bz * p.strideO + (long)row * p.ldo + col));
    }
    if (p.outA) {
      const bool f16 = p.dtype == ACT_F16;
      const long o = bz * p.strideOA + (long)row * p.ldoa + col;
      bf16_t* q = reinterpret_cast<bf16_t*>(p.outA) + o;
      st4_act(q, v, f16);
      if (p.outA_lo) {
        float h[4], l[4];
        ld4_act(q, h, f16);
        _Pragma("unroll") for (int t = 0; t < 4; ++t) l[t] = v[t] - h[t];
        st4_act(reinterpret_cast<bf16_t*>(p.outA_lo) + o, l, f16);
      }
    }
  } else if (p.epi == EPI_RELU2) {
    const long o = bz * p.strideOA + (long)row * p.ldoa + col;
    float g[4];
    _Pragma("unroll") for (int t = 0; t < 4; ++t) { const float r = fmaxf(v[t], 0.f); g[t] = r * r; mx = fmaxf(mx, g[t]); }
    st4_act(reinterpret_cast<bf16_t*>(p.out2) + o, g);
  } else {  // EPI_DRELU2: the input is g = relu(u)^2, whose root is relu(u)
    const float g[4] = {in.x, in.y, in.z, in.w};
    _Pragma("unroll") for (int t = 0; t < 4; ++t) {
      v[t] *= 2.f * __builtin_amdgcn_sqrtf(fmaxf(g[t], 0.f));
      mx = fmaxf(mx, fabsf(v[t]));
    }
    st4_act(reinterpret_cast<bf16_t*>(p.outA) + o_act(p, bz, row, col), v);
  }
}

// The element-wise input of the vector epilogue (uniform): 1 = fp32 Cin, 2 = bf16 aux of
// EPI_DRELU2, 3 = fp16 CinA, 0 = none
template <bool HALF>
__device__ inline int epi_kind(const GemmArgs& p) {
  return p.epi == EPI_DRELU2 ? 2 : p.epi != EPI_LINEAR ? 0 : p.Cin ? 1 : (HALF && p.CinA) ? 3 : 0;
}

// Loads the raw element-wise inputs of one 32-row block for a lane (columns col..col+3 of
// rows row0 + lrow + i RPI): one uniform branch around all the loads and clamped rows (a
// row past M loads row M-1, unused) keep them back to back; per-row branches made the
// compiler wait for each.
template <int NR, int RPI>
__device__ inline void epi_load(const GemmArgs& p, int kind, int bz, int row0, int col, int lrow, uint4 (&raw)[NR]) {
  if (kind == 1) {
    const float* b = p.Cin + bz * p.strideCin + col;
#pragma unroll
    for (int i = 0; i < NR; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(b + (long)min(row0 + lrow + i * RPI, p.M - 1) * p.ldcin);
  } else if (kind != 0) {
    const bf16_t* b = (kind == 2 ? reinterpret_cast<const bf16_t*>(p.aux) + bz * p.strideOA
                                 : reinterpret_cast<const bf16_t*>(p.CinA) + bz * p.strideCin) + col;
    const long ld = kind == 2 ? p.ldoa : p.ldcin;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const uint2 u = *reinterpret_cast<const uint2*>(b + (long)min(row0 + lrow + i * RPI, p.M - 1) * ld);
      raw[i] = make_uint4(u.x, u.y, 0u, 0u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i) raw[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// the input values of one row from its raw words (beta applied to Cin / CinA)
__device__ inline float4 epi_decode(const GemmArgs& p, int kind, const uint4& r) {
  if (kind == 1)
    return make_float4(p.beta * __uint_as_float(r.x), p.beta * __uint_as_float(r.y), p.beta * __uint_as_float(r.z),
                       p.beta * __uint_as_float(r.w));
  if (kind == 2)
    return make_float4(bf2f((bf16_t)(r.x & 0xffff)), bf2f((bf16_t)(r.x >> 16)), bf2f((bf16_t)(r.y & 0xffff)),
                       bf2f((bf16_t)(r.y >> 16)));
  typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));
  const f16x4v h = __builtin_bit_cast(f16x4v, make_uint2(r.x, r.y));
  return make_float4(p.beta * (float)h[0], p.beta * (float)h[1], p.beta * (float)h[2], p.beta * (float)h[3]);
}

// Writes back one 32-row block of a wave's 128x64 tile staged in LDS (stage: 32 rows of CS
// floats; the lane owns columns col..col+3 of rows lrow, lrow + RPI, ...): split-K partials
// to ws_blk (this launch slice's M x N plane), else the epilogue, with the block's
// element-wise inputs in raw (epi_load; the vector path only).
template <bool HALF, int CS, int RPI>
__device__ inline void write_block(const GemmArgs& p, int bz, int row0, int col, int lrow, int lc, bool vec,
                                   const float* stage, float* ws_blk, int kind, const uint4 (&raw)[32 / RPI],
                                   float& mx) {
  constexpr int NR = 32 / RPI;
  if (p.splits > 1) {
#pragma unroll 2
    for (int rr = lrow; rr < 32; rr += RPI) {
      const int row = row0 + rr;
      if (row >= p.M) break;
      const float4 a = *reinterpret_cast<const float4*>(stage + rr * CS + lc);
      float* w = ws_blk + (long)row * p.N + col;
      if (vec && col + 3 < p.N) {
        typedef float f4v __attribute__((ext_vector_type(4)));
        f4v x_ = {a.x, a.y, a.z, a.w};
        __builtin_nontemporal_store(x_, reinterpret_cast<f4v*>(w));
      } else {
#pragma unroll 1
        for (int t = 0; t < 4; ++t)
          if (col + t < p.N) w[t] = pick4(a, t);
      }
    }
  } else if (vec && col + 3 < p.N) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int rr = lrow + i * RPI, row = row0 + rr;
      if (row >= p.M) break;
      epilogue_vec4<HALF>(p, bz, row, col, *reinterpret_cast<const float4*>(stage + rr * CS + lc),
                          kind ? epi_decode(p, kind, raw[i]) : make_float4(0.f, 0.f, 0.f, 0.f), kind != 0, mx);
    }
  } else {
#pragma unroll 1
    for (int rr = lrow; rr < 32; rr += RPI) {
      const int row = row0 + rr;
      if (row >= p.M) break;
      const float4 a = *reinterpret_cast<const float4*>(stage + rr * CS + lc);
#pragma unroll 1
      for (int t = 0; t < 4; ++t)
        if (col + t < p.N) epilogue_elem<bf16_t>(p, bz, row, col + t, pick4(a, t));
    }
  }
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool SPLIT>
__global__ void __launch_bounds__(WM* WN * 64) gemm_bf16_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * LDSS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tilesM = (p.M + BM - 1) / BM, tilesN = (p.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tilesM, tilesN, tm, tn);
  const int bz = blockIdx.y / p.splits, sk = blockIdx.y % p.splits;
  const int m0 = tm * BM, n0 = tn * BN;

  const int kper = ((p.K + p.splits - 1) / p.splits + BK - 1) / BK * BK;
  const int kbeg = sk * kper;
  const int kend = min(p.K, kbeg + kper);
  const int nks = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;  // k tiles per segment
  const int nseg = SPLIT ? 3 : 1;                                   // hi*hi, hi*lo, lo*hi
  const int nk = nks * nseg;

  const bf16_t* Ah = reinterpret_cast<const bf16_t*>(p.A) + bz * p.strideA;
  const bf16_t* Bh = reinterpret_cast<const bf16_t*>(p.B) + bz * p.strideB;
  const bf16_t* Al = SPLIT ? reinterpret_cast<const bf16_t*>(p.A_lo) + bz * p.strideA : Ah;
  const bf16_t* Bl = SPLIT ? reinterpret_cast<const bf16_t*>(p.B_lo) + bz * p.strideB : Bh;
  // operand extents in bytes (the launcher guarantees they fit 32-bit offsets)
  const uint32_t abytes = (uint32_t)((long)(AK ? p.M : p.K) * p.lda * 2);
  const uint32_t bbytes = (uint32_t)((long)(BKM ? p.N : p.K) * p.ldb * 2);
  const __amdgpu_buffer_rsrc_t rAh = make_rsrc(Ah, abytes), rAl = make_rsrc(Al, abytes);
  const __amdgpu_buffer_rsrc_t rBh = make_rsrc(Bh, bbytes), rBl = make_rsrc(Bl, bbytes);
  // k tile t: segment t / nks selects the operand planes (hi*hi, hi*lo, lo*hi), t % nks the offset

  // two register stages: the global loads of tile t+2 are issued while tile t is
  // multiplied, so each load has two k-tiles of MFMA work to arrive
  TileLoader<BM, AK, NT> la0, la1;
  TileLoader<BN, BKM, NT> lb0, lb1;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lr = lane & 31, lk = (lane >> 5) * 8;

#define GEMM_LOAD(LA, LB, T)                                                              \
  do {                                                                                    \
    const int t_ = (T), sg_ = t_ < nk ? t_ / nks : 0;                                     \
    const int k_ = t_ < nk ? kbeg + (t_ % nks) * BK : kend; /* padding tile: all zeros */ \
    LA.load(sg_ == 2 ? rAl : rAh, p.lda, m0, p.M, k_, kend, tid);                         \
    LB.load(sg_ == 1 ? rBl : rBh, p.ldb, n0, p.N, k_, kend, tid);                         \
  } while (0)

#define GEMM_COMPUTE(BUF)                                                                 \
  do {                                                                                    \
    const bf16_t* as_ = smem + (BUF) * (BM * LDSS) + (wm * TM + lr) * LDSS + lk;          \
    const bf16_t* bs_ = smem + 2 * BM * LDSS + (BUF) * (BN * LDSS) + (wn * TN + lr) * LDSS + lk; \
    bf16x8_t af_[2][FM], bf_[2][FN];                                                      \
    _Pragma("unroll") for (int i = 0; i < FM; ++i)                                         \
      af_[0][i] = *reinterpret_cast<const bf16x8_t*>(as_ + i * 32 * LDSS);                \
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                         \
      bf_[0][j] = *reinterpret_cast<const bf16x8_t*>(bs_ + j * 32 * LDSS);                \
    _Pragma("unroll") for (int kk = 0; kk < BK / 16; ++kk) {                               \
      const int c_ = kk & 1;                                                              \
      if (kk + 1 < BK / 16) {                                                             \
        _Pragma("unroll") for (int i = 0; i < FM; ++i)                                     \
          af_[c_ ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(as_ + i * 32 * LDSS + (kk + 1) * 16); \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                     \
          bf_[c_ ^ 1][j] = *reinterpret_cast<const bf16x8_t*>(bs_ + j * 32 * LDSS + (kk + 1) * 16); \
      }                                                                                   \
      __builtin_amdgcn_sched_barrier(0);                                                  \
      _Pragma("unroll") for (int i = 0; i < FM; ++i)                                       \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                     \
          acc[i][j] = mfma32x32x16_bf16(af_[c_][i], bf_[c_][j], acc[i][j]);              \
      __builtin_amdgcn_sched_barrier(0);                                                  \
    }                                                                                     \
  } while (0)

  // an odd tile count is padded with one all-zero tile so the loop runs in pairs
  const int nk2 = (nk + 1) & ~1;
  if (nk2 > 0) {
    GEMM_LOAD(la0, lb0, 0);
    la0.store(smem, tid);
    lb0.store(smem + 2 * BM * LDSS, tid);
    GEMM_LOAD(la1, lb1, 1);
  }
  __syncthreads();
  // tile t sits in LDS buffer t&1 and register stage t&1; unrolled by two so the
  // stage registers are addressed statically
  for (int it = 0; it < nk2; it += 2) {
    if (it + 2 < nk2) GEMM_LOAD(la0, lb0, it + 2);
    GEMM_COMPUTE(0);
    la1.store(smem + BM * LDSS, tid);
    lb1.store(smem + 2 * BM * LDSS + BN * LDSS, tid);
    __syncthreads();
    if (it + 3 < nk2) GEMM_LOAD(la1, lb1, it + 3);
    GEMM_COMPUTE(1);
    if (it + 2 < nk2) {
      la0.store(smem, tid);
      lb0.store(smem + 2 * BM * LDSS, tid);
    }
    __syncthreads();
  }
#undef GEMM_LOAD
#undef GEMM_COMPUTE

  // epilogue through LDS, one 32-row block of every wave at a time: the accumulator
  // fragments go to LDS with constant register indices, then each wave reads its
  // 32 x TN block back by rows, four adjacent columns per lane, for vector stores
  constexpr int CS = TN + 4;  // fp32 row stride of the staging block
  static_assert(WM * WN * 32 * CS * 4 <= 2 * (BM + BN) * LDSS * 2, "staging block must fit in LDS");
  static_assert(TN % 4 == 0 && 64 % (TN / 4) == 0, "epilogue lane mapping");
  constexpr int LPR = TN / 4;        // lanes per row
  constexpr int RPI = 64 / LPR;      // rows per wave instruction
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * CS;
  const bool vec = (p.N % 4 == 0) && (p.ldo % 4 == 0) && (p.ldoa % 4 == 0) && (p.ldcin % 4 == 0) &&
                   (p.strideO % 4 == 0) && (p.strideOA % 4 == 0) && (p.strideCin % 4 == 0);
  const int lc = (lane % LPR) * 4, lrow = lane / LPR;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[acc_row(lane, r) * CS + j * 32 + lr] = acc[i][j][r];
    __syncthreads();
    const int row0 = m0 + wm * TM + i * 32;
    const int col = n0 + wn * TN + lc;
    for (int rr = lrow; rr < 32; rr += RPI) {
      const int row = row0 + rr;
      if (row >= p.M) break;
      const float4 a = *reinterpret_cast<const float4*>(stage + rr * CS + lc);
      if (p.splits > 1) {
        float* w = p.ws + ((long)blockIdx.y * p.M + row) * p.N + col;
        if (vec && col + 3 < p.N) {
          *reinterpret_cast<float4*>(w) = a;
        } else {
          const float e[4] = {a.x, a.y, a.z, a.w};
          for (int t = 0; t < 4; ++t)
            if (col + t < p.N) w[t] = e[t];
        }
      } else if (vec && col + 3 < p.N) {
        float mx_ = 0.f;
        epilogue_vec4(p, bz, row, col, a, epi_in4(p, bz, row, col), epi_has_in(p), mx_);
      } else {
        const float e[4] = {a.x, a.y, a.z, a.w};
        for (int t = 0; t < 4; ++t)
          if (col + t < p.N) epilogue_elem<bf16_t>(p, bz, row, col + t, e[t]);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bf16 GEMM for large problems: 256x256 output tile, 8 waves (two per SIMD) of
// 128x64, k tiles of BK in S LDS stages that are filled straight from global
// memory by buffer_load_dwordx4 ... lds (16 bytes per lane, lane l at M0 + 16 l;
// an offset past the buffer end writes zeros).  The tile for step t + S - 1 is
// issued when step t starts, so a load has S - 1 steps of MFMA work to land.
//
// LDS operand tiles hold 16-byte chunks XOR-swizzled so that every fragment read
// is bank-conflict free:
//   K-major operand: [256 rows][BK], chunk c of row r at c ^ kswz(r); fragments
//     are ds_read_b128 of one chunk of 32 rows.
//   MN-major operand: [BK k-rows][256], chunk c of k-row r at c ^ 4(r%4);
//     fragments are two LDS transpose reads (k = 8h..8h+3, then 8h+4..8h+7).

typedef unsigned int u32x4v_t __attribute__((ext_vector_type(4)));

__device__ inline u32x4v_t res_words(const void* base, uint32_t bytes) {
  u32x4v_t r;
  r.x = (uint32_t)(uintptr_t)base;
  r.y = (uint32_t)((uintptr_t)base >> 32) & 0xFFFFu;
  r.z = bytes;
  r.w = 0x00020000u;
  return r;
}

// written in assembly so that the compiler, which cannot tell the LDS stages
// apart, does not wait for every outstanding DMA before each LDS read; the
// pipeline's own waits are the explicit vmcnt waits below.  No VGPR is written.
__device__ inline void lds_dma16(const u32x4v_t& rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// vmcnt(N) and (LGKM) lgkmcnt(0), then a workgroup barrier (no memory fence: the
// DMA stages are ordered by the waits).  Without LGKM the wave's own LDS reads may
// still be in flight: the compiler waits for each before its first use.
template <int N, bool LGKM = true>
__device__ inline void dma_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (LGKM ? 0 : 15 << 8));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <bool KMAJ, int BK, int NTH = 512>
struct DmaOperand {
  static constexpr int CPR = KMAJ ? BK / 8 : 32;  // 16-byte chunks per LDS row
  static constexpr int ROWS = KMAJ ? 256 : BK;
  static constexpr int CHUNKS = CPR * ROWS;
  static constexpr int PER = CHUNKS / NTH;        // DMA instructions per thread per k tile
  static constexpr int BYTES = CHUNKS * 16;
  static_assert(CHUNKS % NTH == 0, "tile must split into whole wave DMAs");
  __device__ static inline int swz(int r) {
    if constexpr (KMAJ) return (r / (16 / CPR)) % CPR;
    else return 4 * (r & 3);
  }
};

// one 32x32x16 MFMA on 16-bit operands held as raw bits: bf16, or fp16 when F16
template <bool F16>
__device__ inline f32x16_t mma16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  if constexpr (F16)
    return mfma32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c);
  else
    return mfma32x32x16_bf16(a, b, c);
}

template <bool AK, bool BKM, bool SPLIT, int BK, int S, bool F16 = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_bf16_dma_kernel(GemmArgs p) {
  constexpr int WN = 4, TM = 128, TN = 64, FM = TM / 32, FN = TN / 32, NKK = BK / 16;
  using OA = DmaOperand<AK, BK>;
  using OB = DmaOperand<BKM, BK>;
  constexpr int ABASE = 0, BBASE = S * OA::BYTES;  // all A stages, then all B stages
  constexpr int LPT = OA::PER + OB::PER;
  static_assert(S >= 2 && (S - 2) * LPT < 64, "pipeline depth / vmcnt range");
  static_assert(NKK % 2 == 0, "slice 0 of every k tile uses fragment buffer 0");
  static_assert((S - 1) * OA::BYTES < 65536 && (S - 1) * OB::BYTES < 65536, "stage offsets must be immediates");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * (OA::BYTES + OB::BYTES)];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int tilesM = (p.M + 255) / 256, tilesN = (p.N + 255) / 256;
  const bool sym = p.sym && p.splits == 1 && p.M == p.N;
  // Workgroups reach the 8 XCDs round-robin in launch order.  A batched or split
  // launch maps its linear id XCD-contiguously over the whole grid, so that one XCD
  // works through whole matrices (splits) in turn and their panels stay in its L2.
  int tl = blockIdx.x, yy = blockIdx.y;
  const int nall = gridDim.x * gridDim.y;
  const bool grid_xcd = gridDim.y > 1 && (nall & 7) == 0;
  if (grid_xcd) {
    const int lin = blockIdx.y * gridDim.x + blockIdx.x;
    const int id = (lin & 7) * (nall >> 3) + (lin >> 3);
    yy = id / gridDim.x;
    tl = id - yy * gridDim.x;
  }
  int tm, tn;
  if (sym) {  // upper-triangular tiles, row by row
    int id = tl;
    tm = 0;
    while (id >= tilesM - tm) { id -= tilesM - tm; ++tm; }
    tn = tm + id;
  } else {
    tile_coords(tl, tilesM, tilesN, tm, tn, !grid_xcd);
  }
  const int bz = yy / p.splits, sk = yy % p.splits;
  const int m0 = tm * 256, n0 = tn * 256;
  const int kper = ((p.K + p.splits - 1) / p.splits + BK - 1) / BK * BK;
  const int kbeg = sk * kper;
  const int kend = min(p.K, kbeg + kper);
  const int nks = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int nk = nks * (SPLIT ? 3 : 1);
  const int nkp = (nk + S - 1) / S * S;  // padded with all-zero tiles to whole unrolled rounds

  const bf16_t* Ah = reinterpret_cast<const bf16_t*>(p.A) + bz * p.strideA;
  const bf16_t* Bh = reinterpret_cast<const bf16_t*>(p.B) + bz * p.strideB;
  const uint32_t abytes = (uint32_t)((long)(AK ? p.M : p.K) * p.lda * 2);
  const uint32_t bbytes = (uint32_t)((long)(BKM ? p.N : p.K) * p.ldb * 2);
  const u32x4v_t rAh = res_words(Ah, abytes), rBh = res_words(Bh, bbytes);
  const u32x4v_t rAl = SPLIT ? res_words(reinterpret_cast<const bf16_t*>(p.A_lo) + bz * p.strideA, abytes) : rAh;
  const u32x4v_t rBl = SPLIT ? res_words(reinterpret_cast<const bf16_t*>(p.B_lo) + bz * p.strideB, bbytes) : rBh;

  // per DMA instruction j: the chunk this lane fetches, as (byte offset without the
  // k-tile origin, row validity, position along k inside the tile)
  uint32_t aoff[OA::PER], boff[OB::PER];
  int ak_in[OA::PER], bk_in[OB::PER];
  bool aok[OA::PER], bok[OB::PER];
#pragma unroll
  for (int j = 0; j < OA::PER; ++j) {
    const int P = (j * 8 + wave) * 64 + lane, row = P / OA::CPR, lc = (P % OA::CPR) ^ OA::swz(row);
    if constexpr (AK) {
      aok[j] = m0 + row < p.M; ak_in[j] = lc * 8;
      aoff[j] = (uint32_t)(((long)(m0 + row) * p.lda + lc * 8) * 2);
    } else {
      aok[j] = m0 + lc * 8 < p.M; ak_in[j] = row;
      aoff[j] = (uint32_t)(((long)row * p.lda + m0 + lc * 8) * 2);
    }
  }
#pragma unroll
  for (int j = 0; j < OB::PER; ++j) {
    const int P = (j * 8 + wave) * 64 + lane, row = P / OB::CPR, lc = (P % OB::CPR) ^ OB::swz(row);
    if constexpr (BKM) {
      bok[j] = n0 + row < p.N; bk_in[j] = lc * 8;
      boff[j] = (uint32_t)(((long)(n0 + row) * p.ldb + lc * 8) * 2);
    } else {
      bok[j] = n0 + lc * 8 < p.N; bk_in[j] = row;
      boff[j] = (uint32_t)(((long)row * p.ldb + n0 + lc * 8) * 2);
    }
  }

  // the next k tile to issue: its index, segment (split planes) and k origin,
  // advanced incrementally (no division in the loop)
  int it_t = 0, it_sg = 0, it_k0 = kbeg;
  auto issue = [&](int st) {
    const bool live = it_t < nk;
    const u32x4v_t ra = (SPLIT && it_sg == 2) ? rAl : rAh;
    const u32x4v_t rb = (SPLIT && it_sg == 1) ? rBl : rBh;
    const bool full = it_k0 + BK <= kend;  // no k tail inside this tile
    const uint32_t ka = (uint32_t)(AK ? it_k0 * 2 : (long)it_k0 * p.lda * 2);
    const uint32_t kb = (uint32_t)(BKM ? it_k0 * 2 : (long)it_k0 * p.ldb * 2);
    if (live && full) {
      // the whole k tile is in range (a wave-uniform test, so no per-lane branches):
      // a row past M (N) starts past the end of its buffer and reads zeros, and an
      // MN-major chunk past M (N) only feeds outputs that are never stored
#pragma unroll
      for (int j = 0; j < OA::PER; ++j)
        lds_dma16(ra, lds0 + ABASE + st * OA::BYTES + (j * 8 + wave) * 1024, aoff[j] + ka);
#pragma unroll
      for (int j = 0; j < OB::PER; ++j)
        lds_dma16(rb, lds0 + BBASE + st * OB::BYTES + (j * 8 + wave) * 1024, boff[j] + kb);
    } else {
#pragma unroll
      for (int j = 0; j < OA::PER; ++j) {
        const bool ok = live && aok[j] && (full || it_k0 + ak_in[j] < kend);
        lds_dma16(ra, lds0 + ABASE + st * OA::BYTES + (j * 8 + wave) * 1024, ok ? aoff[j] + ka : OOB);
      }
#pragma unroll
      for (int j = 0; j < OB::PER; ++j) {
        const bool ok = live && bok[j] && (full || it_k0 + bk_in[j] < kend);
        lds_dma16(rb, lds0 + BBASE + st * OB::BYTES + (j * 8 + wave) * 1024, ok ? boff[j] + kb : OOB);
      }
    }
    ++it_t;
    it_k0 += BK;
    if (it_k0 >= kbeg + nks * BK) { it_k0 = kbeg; ++it_sg; }
  };

  // fragment offsets inside stage 0 of each operand region (bytes)
  const int lr = lane & 31, hl = lane >> 5, i16 = lane & 15;
  int afo[FM][NKK], bfo[FN][NKK];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if constexpr (AK) {
        const int row = wm * TM + f * 32 + lr;
        afo[f][kk] = ABASE + row * (BK * 2) + (((2 * kk + hl) ^ OA::swz(row)) << 4);
      } else {
        const int r = kk * 16 + 8 * hl + (i16 >> 2);
        const int m = wm * TM + f * 32 + ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
        afo[f][kk] = ABASE + r * 512 + (((m >> 3) ^ OA::swz(r)) << 4) + (m & 7) * 2;
      }
    }
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if constexpr (BKM) {
        const int row = wn * TN + f * 32 + lr;
        bfo[f][kk] = BBASE + row * (BK * 2) + (((2 * kk + hl) ^ OB::swz(row)) << 4);
      } else {
        const int r = kk * 16 + 8 * hl + (i16 >> 2);
        const int n = wn * TN + f * 32 + ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
        bfo[f][kk] = BBASE + r * 512 + (((n >> 3) ^ OB::swz(r)) << 4) + (n & 7) * 2;
      }
    }

  // fragment at byte offset off of stage st (st, and so the stage term, compile-time)
  auto frag = [&](int off, int stage_bytes, int st, bool kmaj) -> bf16x8_t {
    const uint8_t* base = smem + off + st * stage_bytes;
    if (kmaj) return *reinterpret_cast<const bf16x8_t*>(base);
    const i16x4_t lo = lds_read_tr16(reinterpret_cast<const bf16_t*>(base));
    const i16x4_t hi = lds_read_tr16(reinterpret_cast<const bf16_t*>(base + 4 * 512));
    typedef short i16x8_t __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8_t af[2][FM], bf[2][FN];
  if constexpr (S == 2) {
    // two stages, two tiles in flight: before the last k slice of tile t the block
    // syncs (tile t+1 has landed, and every wave holds tile t's last fragments in
    // registers, so tile t's stage is free), issues tile t+2 into that stage and loads
    // tile t+1's first fragments under the last slice's MFMAs
    issue(0);
    issue(1);
    dma_sync<LPT>();
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = frag(afo[i][0], OA::BYTES, 0, AK);
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[0][j] = frag(bfo[j][0], OB::BYTES, 0, BKM);
    for (int t0 = 0; t0 < nkp; t0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int c = kk & 1;
          if (kk + 1 < NKK) {
#pragma unroll
            for (int i = 0; i < FM; ++i) af[c ^ 1][i] = frag(afo[i][kk + 1], OA::BYTES, u, AK);
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[c ^ 1][j] = frag(bfo[j][kk + 1], OB::BYTES, u, BKM);
          } else {
            dma_sync<0>();
            issue(u);
#pragma unroll
            for (int i = 0; i < FM; ++i) af[c ^ 1][i] = frag(afo[i][0], OA::BYTES, u ^ 1, AK);
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[c ^ 1][j] = frag(bfo[j][0], OB::BYTES, u ^ 1, BKM);
          }
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mma16<F16>(af[c][i], bf[c][j], acc[i][j]);
          // one fragment read after each of the first MFMAs (0.5% per d24 step over
          // issuing all reads ahead of the MFMAs)
#pragma unroll
          for (int q = 0; q < FM + FN; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  } else {
  // prologue: tiles 0..S-2 in flight; wait for tile 0 and fetch its first fragments
#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st);
  dma_sync<(S - 2) * LPT>();
#pragma unroll
  for (int i = 0; i < FM; ++i) af[0][i] = frag(afo[i][0], OA::BYTES, 0, AK);
#pragma unroll
  for (int j = 0; j < FN; ++j) bf[0][j] = frag(bfo[j][0], OB::BYTES, 0, BKM);

  // k step t uses stage t % S.  Within it, the fragments of k slice kk+1 load under
  // the MFMAs of slice kk; before the last slice the block syncs (tile t+1 has
  // landed, every wave is past tile t-1), issues tile t+S-1 into the stage tile t-1
  // used, and loads the first fragments of tile t+1 under the last slice's MFMAs.
  for (int t0 = 0; t0 < nkp; t0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int c = kk & 1;  // NKK even: slice 0 of every tile sits in buffer 0
        if (kk + 1 < NKK) {
#pragma unroll
          for (int i = 0; i < FM; ++i) af[c ^ 1][i] = frag(afo[i][kk + 1], OA::BYTES, u, AK);
#pragma unroll
          for (int j = 0; j < FN; ++j) bf[c ^ 1][j] = frag(bfo[j][kk + 1], OB::BYTES, u, BKM);
        } else {
          dma_sync<(S - 3) * LPT>();
          issue((u + S - 1) % S);
#pragma unroll
          for (int i = 0; i < FM; ++i) af[c ^ 1][i] = frag(afo[i][0], OA::BYTES, (u + 1) % S, AK);
#pragma unroll
          for (int j = 0; j < FN; ++j) bf[c ^ 1][j] = frag(bfo[j][0], OB::BYTES, (u + 1) % S, BKM);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mma16<F16>(af[c][i], bf[c][j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  }
  // every DMA, including the zero tail, must land before the workgroup's LDS is released
  dma_sync<0>();

  // epilogue: each wave stages one 32-row block of its 128x64 tile in its own LDS
  // area (constant register indices) and writes it back by rows, four adjacent
  // columns per lane, sixteen lanes per row
  constexpr int CS = TN + 4;
  constexpr int LPR = TN / 4, RPI = 64 / LPR;
  static_assert(8 * 32 * CS * 4 <= S * (OA::BYTES + OB::BYTES), "staging must fit");
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * CS;
  const bool vec = (p.N % 4 == 0) && (p.ldo % 4 == 0) && (p.ldoa % 4 == 0) && (p.ldcin % 4 == 0) &&
                   (p.strideO % 4 == 0) && (p.strideOA % 4 == 0) && (p.strideCin % 4 == 0);
  const int lc = (lane % LPR) * 4, lrow = lane / LPR;
  // Stage one 32-row block of the wave tile (a literal block index per case keeps every
  // accumulator access static), then write it back from LDS with one rolled copy of the
  // store code for all four blocks: the epilogue stays a few hundred instructions, so
  // the k loop of the next tile still finds its code in the instruction cache (the
  // unrolled form was ~20k instructions per kernel and measurably slowed the k loop).
  static_assert(FM == 4, "one case per 32-row block");
  // the element-wise inputs of the vector path, one row block ahead: the loads of block
  // ib + 1 are in flight while block ib is written
  constexpr int NR = 32 / RPI;
  const int ekind = p.splits == 1 && vec && n0 + wn * TN + lc + 3 < p.N ? epi_kind<F16>(p) : 0;
  uint4 rin[NR];
  epi_load<NR, RPI>(p, ekind, bz, m0 + wm * TM, n0 + wn * TN + lc, lrow, rin);
  float emx = 0.f;  // max |stored output| of the lane (amax_part)
#pragma unroll 1
  for (int ib = 0; ib < FM; ++ib) {
#define GEMM_STAGE(I_)                                                                          \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) _Pragma("unroll") for (int r = 0; r < 16; ++r) \
      stage[acc_row(lane, r) * CS + j * 32 + lr] = acc[I_][j][r];
    switch (ib) {
      case 0: GEMM_STAGE(0) break;
      case 1: GEMM_STAGE(1) break;
      case 2: GEMM_STAGE(2) break;
      default: GEMM_STAGE(3) break;
    }
#undef GEMM_STAGE
    const int row0 = m0 + wm * TM + ib * 32;
    const int col = n0 + wn * TN + lc;
    uint4 rnext[NR];
    epi_load<NR, RPI>(p, ib + 1 < FM ? ekind : 0, bz, row0 + 32, col, lrow, rnext);
    write_block<F16, CS, RPI>(p, bz, row0, col, lrow, lc, vec, stage,
                                     p.splits > 1 ? p.ws + (long)yy * p.M * p.N : nullptr, ekind, rin, emx);
#pragma unroll
    for (int i = 0; i < NR; ++i) rin[i] = rnext[i];
    if (sym && tm != tn) {
      // mirror: element (row0 + r, n) also lands at (n, row0 + r); read the staged block
      // by columns so each mirrored row gets 4-wide stores (8 lanes per 32-wide row)
      const int r4 = (lane & 7) * 4;
#pragma unroll 2
      for (int q = 0; q < TN / 8; ++q) {
        const int cc = q * 8 + (lane >> 3);
        const int n = n0 + wn * TN + cc, m = row0 + r4;
        if (n >= p.M || m >= p.M) continue;
        const float4 a = make_float4(stage[(r4 + 0) * CS + cc], stage[(r4 + 1) * CS + cc], stage[(r4 + 2) * CS + cc],
                                     stage[(r4 + 3) * CS + cc]);
        if (vec && m + 3 < p.M) {
          float mx_ = 0.f;
          epilogue_vec4<F16>(p, bz, n, m, a, epi_in4<F16>(p, bz, n, m), epi_has_in<F16>(p),
                                    mx_);
        } else {
#pragma unroll 1
          for (int t = 0; t < 4; ++t)
            if (m + t < p.M) epilogue_elem<bf16_t>(p, bz, n, m + t, pick4(a, t));
        }
      }
    }
  }
  if (p.amax_part) {  // one entry per wave (single-matrix, unsplit launches: blockIdx.x is the tile)
    emx = wave_max(emx);
    if (lane == 0) p.amax_part[blockIdx.x * 8 + wave] = bf16_round(emx);
  }
}


// ---------------------------------------------------------------------------
// fp8 (e4m3) GEMM operands: 32 bytes of k per lane for v_mfma_f32_32x32x64_f8f6f4
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// fp8 GEMM on the DMA path: the 256x256 tile of the bf16 kernel with 8 waves of 128x64,
// both operands e4m3 with the reduction index contiguous, k tiles of BKB bytes in S
// LDS stages (a 64-byte tile has the byte layout of a 32-deep bf16 K-major tile, a
// 128-byte one that of a 64-deep tile: 16-byte chunk c of row r at c ^ kswz(r)).  With
// S >= 3 tile t + S - 1 is issued before the last k slice of tile t, into the stage
// tile t - 1 used; with S = 2 (128-byte tiles: every row of a tile is one whole
// 128-byte line, half the DMA requests of 64-byte tiles) tile t + 2 goes into tile t's
// own stage, after the block has waited for tile t + 1 and for its own LDS reads of
// tile t, whose last slice is then in registers.  A lane's fragment for one v_mfma_scale_f32_32x32x64_f8f6f4 is 32 bytes:
// lane half h holds k bytes 32h..32h+31 of its row (any k mapping shared by A and B
// gives the same sum).  The k slices of all tiles form one sequence: the B fragments
// of the next slice load under the current slice's MFMAs, and each A fragment is
// reloaded for the next slice as soon as its own MFMAs have issued.  The product is
// multiplied by (*dq_a) * (*dq_b) as it is staged for the epilogue.
template <int BKB, int S>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_fp8_dma_kernel(GemmArgs p) {
  constexpr int WN = 4, TM = 128, TN = 64, FM = TM / 32, FN = TN / 32, NKK = BKB / 64;
  using OP = DmaOperand<true, BKB / 2>;  // byte tile [256][BKB] = bf16 tile [256][BKB/2]
  constexpr int OBYTES = OP::BYTES, PER = OP::PER, LPT = 2 * PER;
  constexpr int ABASE = 0, BBASE = S * OBYTES;
  static_assert(NKK >= 1 && BKB % 64 == 0, "whole 64-byte MFMA k steps per tile");
  static_assert(S >= 2 && (S - 2) * LPT < 64 && LPT < 64, "pipeline depth / vmcnt range");
  static_assert((S - 1) * OBYTES < 65536, "stage offsets must be immediates");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * S * OBYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int tilesM = (p.M + 255) / 256, tilesN = (p.N + 255) / 256;
  int tm, tn;
  tile_coords(blockIdx.x, tilesM, tilesN, tm, tn);
  const int bz = blockIdx.y / p.splits, sk = blockIdx.y % p.splits;
  const int m0 = tm * 256, n0 = tn * 256;
  const int kper = ((p.K + p.splits - 1) / p.splits + BKB - 1) / BKB * BKB;
  const int kbeg = sk * kper;
  const int kend = min(p.K, kbeg + kper);
  const int nk = kend > kbeg ? (kend - kbeg + BKB - 1) / BKB : 0;
  const int nkp = (nk + S - 1) / S * S;  // padded with all-zero tiles to whole unrolled rounds
  const uint8_t* A = reinterpret_cast<const uint8_t*>(p.A) + bz * p.strideA;
  const uint8_t* B = reinterpret_cast<const uint8_t*>(p.B) + bz * p.strideB;
  const u32x4v_t rA = res_words(A, (uint32_t)((long)p.M * p.lda)), rB = res_words(B, (uint32_t)((long)p.N * p.ldb));
  const float dq = p.dq_a[0] * p.dq_b[0];

  uint32_t aoff[PER], boff[PER];
  int kin[PER];
  bool aok[PER], bok[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int P = (j * 8 + wave) * 64 + lane, row = P / OP::CPR, lc = (P % OP::CPR) ^ OP::swz(row);
    kin[j] = lc * 16;
    aok[j] = m0 + row < p.M;
    bok[j] = n0 + row < p.N;
    aoff[j] = (uint32_t)((long)(m0 + row) * p.lda + lc * 16);
    boff[j] = (uint32_t)((long)(n0 + row) * p.ldb + lc * 16);
  }
  int it_t = 0, it_k0 = kbeg;
  auto issue = [&](int st) {
    const bool live = it_t < nk, full = it_k0 + BKB <= kend;
    if (live && full) {  // whole k tile: rows past M (N) start past their buffer's end
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        lds_dma16(rA, lds0 + ABASE + st * OBYTES + (j * 8 + wave) * 1024, aoff[j] + it_k0);
        lds_dma16(rB, lds0 + BBASE + st * OBYTES + (j * 8 + wave) * 1024, boff[j] + it_k0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const bool kok = live && (full || it_k0 + kin[j] < kend);
        lds_dma16(rA, lds0 + ABASE + st * OBYTES + (j * 8 + wave) * 1024, kok && aok[j] ? aoff[j] + it_k0 : OOB);
        lds_dma16(rB, lds0 + BBASE + st * OBYTES + (j * 8 + wave) * 1024, kok && bok[j] ? boff[j] + it_k0 : OOB);
      }
    }
    ++it_t;
    it_k0 += BKB;
  };

  // kswz(row) depends on row only through (row / 4) % 4 or (row / 2) % 8, which every
  // 32-row fragment of a lane shares: the chunk positions are per-lane constants and
  // the fragment rows are immediate offsets from one base
  const int lr = lane & 31, hl = lane >> 5, sw = OP::swz(lr);
  static_assert(32 % (16 / OP::CPR) == 0 && (32 / (16 / OP::CPR)) % OP::CPR == 0, "swizzle repeats every 32 rows");
  int cofs[NKK][2];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) cofs[kk][h] = ((4 * kk + 2 * hl + h) ^ sw) << 4;
  const uint8_t* abase = smem + ABASE + (wm * TM + lr) * BKB;
  const uint8_t* bbase = smem + BBASE + (wn * TN + lr) * BKB;
  auto frag = [&](const uint8_t* rowp, int kk) -> i32x8_t {
    const uint4 a = *reinterpret_cast<const uint4*>(rowp + cofs[kk][0]);
    const uint4 b = *reinterpret_cast<const uint4*>(rowp + cofs[kk][1]);
    u32x8_t v;
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    return __builtin_bit_cast(i32x8_t, v);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // prologue: tiles 0..S-2 in flight (0 and 1 for S = 2); wait for tile 0 and fetch its
  // first fragments
  if constexpr (S == 2) {
    issue(0);
    issue(1);
    dma_sync<LPT>();
  } else {
#pragma unroll
    for (int st = 0; st < S - 1; ++st) issue(st);
    dma_sync<(S - 2) * LPT>();
  }
  i32x8_t af[FM], bf[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) af[i] = frag(abase + i * 32 * BKB, 0);
#pragma unroll
  for (int j = 0; j < FN; ++j) bf[j] = frag(bbase + j * 32 * BKB, 0);

  for (int t0 = 0; t0 < nkp; t0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bool last = kk == NKK - 1;
        const int nst = last ? (u + 1) % S : u, nkk = last ? 0 : kk + 1;
        if (last) {
          if constexpr (S == 2) {
            // tile t+1 landed and every wave's reads of tile t are done: tile t+2 into its stage
            dma_sync<0>();
            issue(u);
          } else {
            // tile t+1 landed; every wave is past tile t-1, whose stage was last read
            // (into registers the MFMAs of tile t-1 consumed) one tile earlier
            dma_sync<(S > 2 ? (S - 3) * LPT : 0), false>();
            issue((u + S - 1) % S);
          }
        }
        i32x8_t bn[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) bn[j] = frag(bbase + nst * OBYTES + j * 32 * BKB, nkk);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
          af[i] = frag(abase + nst * OBYTES + i * 32 * BKB, nkk);
        }
        // one MFMA, then two fragment reads for the next slice, so that the reads
        // spread over the slice instead of gathering before the next barrier
        static_assert(FM * FN >= FM + FN, "a read pair per MFMA");
#pragma unroll
        for (int g = 0; g < FM + FN; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN), 0);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = bn[j];
      }
    }
  }
  // every DMA, including the zero tail, must land before the workgroup's LDS is released
  dma_sync<0>();

  constexpr int CS = TN + 4;
  constexpr int LPR = TN / 4, RPI = 64 / LPR;
  static_assert(8 * 32 * CS * 4 <= 2 * S * OBYTES, "staging must fit");
  float* stage = reinterpret_cast<float*>(smem) + wave * 32 * CS;
  const bool vec = (p.N % 4 == 0) && (p.ldo % 4 == 0) && (p.ldoa % 4 == 0) && (p.ldcin % 4 == 0) &&
                   (p.strideO % 4 == 0) && (p.strideOA % 4 == 0) && (p.strideCin % 4 == 0);
  const int lc = (lane % LPR) * 4, lrow = lane / LPR;
  // staging by a literal block index, stores by one rolled copy (as in the bf16 kernel)
  static_assert(FM == 4, "one case per 32-row block");
  constexpr int NR = 32 / RPI;  // inputs one row block ahead, as in the bf16 kernel
  const int ekind = p.splits == 1 && vec && n0 + wn * TN + lc + 3 < p.N ? epi_kind<false>(p) : 0;
  uint4 rin[NR];
  epi_load<NR, RPI>(p, ekind, bz, m0 + wm * TM, n0 + wn * TN + lc, lrow, rin);
  float emx = 0.f;
#pragma unroll 1
  for (int ib = 0; ib < FM; ++ib) {
#define FP8_STAGE(I_)                                                                           \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) _Pragma("unroll") for (int r = 0; r < 16; ++r) \
      stage[acc_row(lane, r) * CS + j * 32 + lr] = acc[I_][j][r] * dq;
    switch (ib) {
      case 0: FP8_STAGE(0) break;
      case 1: FP8_STAGE(1) break;
      case 2: FP8_STAGE(2) break;
      default: FP8_STAGE(3) break;
    }
#undef FP8_STAGE
    const int row0 = m0 + wm * TM + ib * 32;
    const int col = n0 + wn * TN + lc;
    uint4 rnext[NR];
    epi_load<NR, RPI>(p, ib + 1 < FM ? ekind : 0, bz, row0 + 32, col, lrow, rnext);
    write_block<false, CS, RPI>(p, bz, row0, col, lrow, lc, vec, stage,
                               p.splits > 1 ? p.ws + (long)blockIdx.y * p.M * p.N : nullptr, ekind, rin, emx);
#pragma unroll
    for (int i = 0; i < NR; ++i) rin[i] = rnext[i];
  }
  if (p.amax_part) {
    emx = wave_max(emx);
    if (lane == 0) p.amax_part[blockIdx.x * 8 + wave] = bf16_round(emx);
  }
}

// ---------------------------------------------------------------------------
// fp32 SIMT GEMM: 64x64 tile, 256 threads, 4x4 outputs per thread

template <bool AK, bool BKM>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs p) {
  constexpr int T = 64, KB = 16;
  __shared__ float As[KB][T + 1];
  __shared__ float Bs[KB][T + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tilesM = (p.M + T - 1) / T, tilesN = (p.N + T - 1) / T;
  int tm, tn;
  tile_coords(blockIdx.x, tilesM, tilesN, tm, tn);
  const int bz = blockIdx.y / p.splits, sk = blockIdx.y % p.splits;
  const int m0 = tm * T, n0 = tn * T;
  const int kper = ((p.K + p.splits - 1) / p.splits + KB - 1) / KB * KB;
  const int kbeg = sk * kper, kend = min(p.K, kbeg + kper);
  const float* A = reinterpret_cast<const float*>(p.A) + bz * p.strideA;
  const float* B = reinterpret_cast<const float*>(p.B) + bz * p.strideB;
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += KB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      int r, k;
      if (AK) { r = e / KB; k = e % KB; } else { r = e % T; k = e / T; }
      const int gr = m0 + r, gk = k0 + k;
      float v = 0.f;
      if (gr < p.M && gk < kend) v = AK ? A[(long)gr * p.lda + gk] : A[(long)gk * p.lda + gr];
      As[k][r] = v;
      if (BKM) { r = e / KB; k = e % KB; } else { r = e % T; k = e / T; }
      const int gc = n0 + r, gk2 = k0 + k;
      float w = 0.f;
      if (gc < p.N && gk2 < kend) w = BKM ? B[(long)gc * p.ldb + gk2] : B[(long)gk2 * p.ldb + gc];
      Bs[k][r] = w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row < p.M && col < p.N) {
        if (p.splits > 1)
          p.ws[((long)blockIdx.y * p.M + row) * p.N + col] = acc[i][j];
        else
          epilogue_elem<float>(p, bz, row, col, acc[i][j]);
      }
    }
}

// sum the split-K partials in split order, then apply the linear epilogue
template <typename OutT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs p) {
  const long MN = (long)p.M * p.N;
  const long total = MN * p.batch;
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    const int bz = (int)(e / MN);
    const long rc = e - (long)bz * MN;
    const int row = (int)(rc / p.N), col = (int)(rc % p.N);
    float s = 0.f;
    for (int k = 0; k < p.splits; ++k) s += p.ws[((long)bz * p.splits + k) * MN + rc];
    epilogue_elem<OutT>(p, bz, row, col, s);
  }
}

// the same with four adjacent columns per thread (N and every leading dimension and
// stride of the outputs a multiple of 4): one row per grid row, batch along z, so no
// index division; float4 partial loads and the vectorised epilogue
__global__ void __launch_bounds__(128) splitk_reduce_vec_kernel(GemmArgs p) {
  const int c4 = blockIdx.x * 128 + threadIdx.x;
  if (c4 >= p.N / 4) return;
  const int row = blockIdx.y, bz = blockIdx.z;
  const long MN = (long)p.M * p.N;
  const float* w = p.ws + (long)bz * p.splits * MN + (long)row * p.N + 4 * c4;
  const float4 in = epi_in4(p, bz, row, 4 * c4);  // issued ahead of the partial sums
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < p.splits; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(w + k * MN);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  float mx_ = 0.f;
  epilogue_vec4(p, bz, row, 4 * c4, s, in, epi_has_in(p), mx_);
}

template <int BM, int BN, int WM, int WN, bool SPLIT>
void launch_bf16_s(const GemmArgs& p, hipStream_t st) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  dim3 grid(tiles, p.batch * p.splits), block(WM * WN * 64);
  if (p.a_kmaj && p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, true, true, SPLIT>), grid, block, 0, st, p);
  else if (p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, true, false, SPLIT>), grid, block, 0, st, p);
  else if (!p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, false, false, SPLIT>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, false, true, SPLIT>), grid, block, 0, st, p);
}

template <int BM, int BN, int WM, int WN>
void launch_bf16(const GemmArgs& p, hipStream_t st) {
  if (p.split)
    launch_bf16_s<BM, BN, WM, WN, true>(p, st);
  else
    launch_bf16_s<BM, BN, WM, WN, false>(p, st);
}

template <bool SPLIT, int BK, int S>
void launch_dma_s(const GemmArgs& p, hipStream_t st) {
  const int tM = (p.M + 255) / 256;
  const int tiles = (p.sym && p.splits == 1 && p.M == p.N) ? tM * (tM + 1) / 2 : tM * ((p.N + 255) / 256);
  dim3 grid(tiles, p.batch * p.splits), block(512);
  if (p.a_kmaj && p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<true, true, SPLIT, BK, S>), grid, block, 0, st, p);
  else if (p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<true, false, SPLIT, BK, S>), grid, block, 0, st, p);
  else if (!p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<false, false, SPLIT, BK, S>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<false, true, SPLIT, BK, S>), grid, block, 0, st, p);
}

void launch_dma_f16(const GemmArgs& p, hipStream_t st) {
  const int tM = (p.M + 255) / 256;
  const int tiles = (p.sym && p.M == p.N) ? tM * (tM + 1) / 2 : tM * ((p.N + 255) / 256);
  dim3 grid(tiles, p.batch), block(512);
  if (p.a_kmaj && p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<true, true, false, 64, 2, true>), grid, block, 0, st, p);
  else if (p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<true, false, false, 64, 2, true>), grid, block, 0, st, p);
  else if (!p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<false, false, false, 64, 2, true>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<false, true, false, 64, 2, true>), grid, block, 0, st, p);
}

template <int BK, int S>
void launch_dma(const GemmArgs& p, hipStream_t st) {
  if (p.split)
    launch_dma_s<true, BK, S>(p, st);
  else
    launch_dma_s<false, BK, S>(p, st);
}

void launch_f32(const GemmArgs& p, hipStream_t st) {
  const int tiles = ((p.M + 63) / 64) * ((p.N + 63) / 64);
  dim3 grid(tiles, p.batch * p.splits), block(256);
  if (p.a_kmaj && p.b_kmaj)
    hipLaunchKernelGGL((gemm_f32_kernel<true, true>), grid, block, 0, st, p);
  else if (p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_f32_kernel<true, false>), grid, block, 0, st, p);
  else if (!p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_f32_kernel<false, false>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<false, true>), grid, block, 0, st, p);
}

// split-K factor for a tm x tn tiling: aim for >= 512 workgroups while every split
// keeps >= 1024 of K
int splits_for(const GemmArgs& p, int tm, int tn) {
  if (p.epi != EPI_LINEAR) return 1;
  const long tiles = (long)((p.M + tm - 1) / tm) * ((p.N + tn - 1) / tn) * p.batch;
  int s = 1;
  while (tiles * s < 512 && (long)p.K / (s * 2) >= 1024 && s < 32) s *= 2;
  return s;
}

// Split-K factor for the 256x256 kernels (one workgroup per CU, 256 CUs): the one
// that minimises rounds of 256 workgroups times the k extent of a split, plus the cost
// of the splits' fp32 partials, with at least 1024 of K per split; ties go to fewer
// splits.  A last round that is almost empty costs as much as a full one, so e.g. 36
// tiles take 7 splits (one round), not 16 (three rounds).  The partials (written by
// the GEMM with nontemporal stores, read back by the reduction) cost about 1.04e-4 of
// a k step of a bf16 tile round per output element and split, twice that against the
// faster fp8 k step: the coefficient that ran the d24 step fastest (factors 2, 7, 5, 5
// for the bf16 weight gradients; 2, 7, 3, 3 for e4m3), against 0.5x and 1.5x of it.
int splits_256(const GemmArgs& p) {
  if (p.epi != EPI_LINEAR) return 1;
  constexpr long CUS = 256, KQ = 64;  // k extents are rounded to whole k tiles (<= 64)
  const long tiles = (long)((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
  const double part = (p.fp8 ? 2.0 : 1.0) * 1.04e-4 * (double)p.M * p.N * p.batch;
  double best = -1;
  int bs = 1;
  for (int s = 1; s <= 32; ++s) {
    if (s > 1 && (long)p.K / s < 1024) break;
    const long kper = ((p.K + s - 1) / s + KQ - 1) / KQ * KQ;
    const double cost = (double)((tiles * s + CUS - 1) / CUS * kper) + (s > 1 ? s * part : 0.0);
    if (best < 0 || cost < best) {
      best = cost;
      bs = s;
    }
  }
  return bs;
}

// 1: a 256x256 kernel, 2: the 128x128 kernel.  The 256 tile is used when the
// problem has >= 128 such tiles, or when split-K over them reaches >= 256
// workgroups (the long-reduction weight gradients); a pure function of the shape,
// so the split factor and the kernel always agree.
int pick_tile(const GemmArgs& p) {
  if (p.tile) return p.tile == 2 ? 2 : 1;  // 1, 3, 4: 256x256 variants
  const long big = (long)((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
  if (big >= 128) return 1;
  return big * splits_for(p, 256, 256) >= 256 ? 1 : 2;
}

}  // namespace

int gemm_amax_parts(const GemmArgs& p) {
  if (p.epi != EPI_RELU2 && p.epi != EPI_DRELU2) return 0;
  if (p.batch != 1 || p.splits > 1 || p.sym || p.split || p.dtype != ACT_BF16) return 0;
  if (p.N % 4 || p.ldo % 4 || p.ldoa % 4 || p.ldcin % 4 || p.strideO % 4 || p.strideOA % 4 || p.strideCin % 4)
    return 0;  // the vector epilogue (which tracks the maximum) must take every output
  if (!p.fp8 && (pick_tile(p) != 1 || p.tile == 4)) return 0;  // the DMA kernels only
  const long n = (long)((p.M + 255) / 256) * ((p.N + 255) / 256) * 8;
  return n <= (1L << 30) ? (int)n : 0;
}

int gemm_auto_splits(const GemmArgs& p) {
  if (p.dtype == ACT_F32) return splits_for(p, 64, 64);
  if (p.fp8 || pick_tile(p) != 2) return splits_256(p);
  return splits_for(p, 128, 128);
}

// one name per kernel instantiation: tile and operand layouts (N = reduction index
// contiguous, T = transposed on load), as "gemm_bf16_dma_kernel<256,256,NT>"
const char* gemm_kernel_name(const GemmArgs& p) {
  static const char* names[3][4] = {
      {"gemm_f32_kernel<NT>", "gemm_f32_kernel<NN>", "gemm_f32_kernel<TN>", "gemm_f32_kernel<TT>"},
      {"gemm_bf16_dma_kernel<256,256,NT>", "gemm_bf16_dma_kernel<256,256,NN>", "gemm_bf16_dma_kernel<256,256,TN>",
       "gemm_bf16_dma_kernel<256,256,TT>"},
      {"gemm_bf16_kernel<128,128,NT>", "gemm_bf16_kernel<128,128,NN>", "gemm_bf16_kernel<128,128,TN>",
       "gemm_bf16_kernel<128,128,TT>"}};
  static const char* split_names[3][4] = {
      {"", "", "", ""},
      {"gemm_bf16x3_dma_kernel<256,256,NT>", "gemm_bf16x3_dma_kernel<256,256,NN>",
       "gemm_bf16x3_dma_kernel<256,256,TN>", "gemm_bf16x3_dma_kernel<256,256,TT>"},
      {"gemm_bf16x3_kernel<128,128,NT>", "gemm_bf16x3_kernel<128,128,NN>", "gemm_bf16x3_kernel<128,128,TN>",
       "gemm_bf16x3_kernel<128,128,TT>"}};
  static const char* f16_names[4] = {"gemm_f16_dma_kernel<256,256,NT>", "gemm_f16_dma_kernel<256,256,NN>",
                                     "gemm_f16_dma_kernel<256,256,TN>", "gemm_f16_dma_kernel<256,256,TT>"};
  if (p.fp8) return "gemm_fp8_dma_kernel<256,256,NT>";
  const int lay = p.a_kmaj ? (p.b_kmaj ? 0 : 1) : (p.b_kmaj ? 3 : 2);
  if (p.dtype == ACT_F16) return f16_names[lay];
  const int t = p.dtype == ACT_F32 ? 0 : (pick_tile(p) == 2 ? 2 : 1);
  if (p.split && t) return split_names[t][lay];
  return names[t][lay];
}

int launch_gemm(const GemmArgs& p0, hipStream_t st) {
  GemmArgs p = p0;
  if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return 0;
  if (p.K < 0 || !p.A || !p.B) return 1;
  if (p.splits < 1) p.splits = 1;
  if (p.splits > 1) {
    if (p.epi != EPI_LINEAR || !p.ws) return 1;
    if ((size_t)p.splits * p.batch * p.M * p.N * sizeof(float) > p.ws_bytes) return 1;
  }
  if (p.split && (p.dtype != ACT_BF16 || p.splits != 1 || !p.A_lo || !p.B_lo)) return 1;
  // CinA is read by the vectorised epilogue of the fp16 NT and NN kernels only: every row
  // and column in groups of four
  if (p.CinA && (p.dtype != ACT_F16 || !p.a_kmaj || p.Cin || p.M % 4 || p.N % 4 || p.ldcin % 4 ||
                 p.strideCin % 4 ||
                 p.ldo % 4 || p.ldoa % 4 || p.strideO % 4 || p.strideOA % 4))
    return 1;
  if (p.dtype == ACT_F16 && (p.splits != 1 || p.epi != EPI_LINEAR)) return 1;
  if (p.amax_part && gemm_amax_parts(p) == 0) return 1;
  if (p.fp8) {
    if (!p.a_kmaj || !p.b_kmaj || p.split || !p.dq_a || !p.dq_b) return 1;
    if (p.K % 16 || p.lda % 16 || p.ldb % 16) return 2;
    if ((long)p.M * p.lda >= (long)0xFFFFFFF0u || (long)p.N * p.ldb >= (long)0xFFFFFFF0u) return 2;
    const int tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
    if (p.tile == 6)  // 64-byte k tiles in four stages (the form before 128-byte tiles)
      hipLaunchKernelGGL((gemm_fp8_dma_kernel<64, 4>), dim3(tiles, p.batch * p.splits), dim3(512), 0, st, p);
    else
      hipLaunchKernelGGL((gemm_fp8_dma_kernel<128, 2>), dim3(tiles, p.batch * p.splits), dim3(512), 0, st, p);
  } else
  if (p.dtype == ACT_BF16 || p.dtype == ACT_F16) {
    // buffer loads address each operand matrix with 32-bit byte offsets
    const long abytes = (long)(p.a_kmaj ? p.M : p.K) * p.lda * 2, bbytes = (long)(p.b_kmaj ? p.N : p.K) * p.ldb * 2;
    if (abytes >= (long)0xFFFFFFF0u || bbytes >= (long)0xFFFFFFF0u) return 2;
    // 16-byte vector loads: k (K-major operands) or rows (transposed operands) in multiples of 8
    if (p.K % 8) return 2;
    if (!p.a_kmaj && (p.M % 8 || p.lda % 8)) return 2;
    if (!p.b_kmaj && (p.N % 8 || p.ldb % 8)) return 2;
    if ((p.a_kmaj && p.lda % 8) || (p.b_kmaj && p.ldb % 8)) return 2;
    if (p.dtype == ACT_F16)  // every size on the 256x256 kernel (ragged tiles read zeros)
      launch_dma_f16(p, st);
    else if (pick_tile(p) == 2)
      launch_bf16<128, 128, 2, 2>(p, st);
    else if (p.tile == 4)
      launch_bf16<256, 256, 2, 2>(p, st);
    else if (p.tile == 3)
      launch_dma<32, 3>(p, st);
    else if (p.tile == 5)
      launch_dma<32, 4>(p, st);
    else
      launch_dma<64, 2>(p, st);
  } else {
    launch_f32(p, st);
  }
  if (p.splits > 1) {
    const long total = (long)p.M * p.N * p.batch;
    const int blocks = (int)std::min<long>((total + 255) / 256, 65536);
    const bool vec = (p.N % 4 == 0) && (p.ldo % 4 == 0) && (p.ldoa % 4 == 0) && (p.ldcin % 4 == 0) &&
                     (p.strideO % 4 == 0) && (p.strideOA % 4 == 0) && (p.strideCin % 4 == 0) && p.M <= 65535 &&
                     p.batch <= 65535 && p.dtype == ACT_BF16;
    if (vec)
      hipLaunchKernelGGL(splitk_reduce_vec_kernel, dim3((p.N / 4 + 127) / 128, p.M, p.batch), dim3(128), 0, st, p);
    else if (p.dtype == ACT_BF16)
      hipLaunchKernelGGL(splitk_reduce_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3(blocks), dim3(256), 0, st, p);
  }
  return 0;
}
