// Causal multi-head attention of the GPT step (flash form) on gfx950.
//
// Layouts: qkv [B*T][3*H*hd] (q at column h*hd, k at H*hd + h*hd, v at 2*H*hd + h*hd,
// as the QKV projection writes it), o and dO [B*T][H*hd], lse and D [B][H][T] fp32.
// lse is the natural-log log-sum-exp of the scaled scores q.k/sqrt(hd).
//
// Forward: a workgroup owns 128 queries (4 waves x 32) and streams 64-key tiles
// through LDS (K as [key][d], V transposed to [d][key]).  Each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so a lane owns one query and the
// softmax statistics are lane-local (plus one exchange with lane^32).  The
// probabilities then feed O^T += V^T P^T straight from registers: the k index of
// that product is a permutation of the 16 keys that matches the accumulator
// layout, and V^T is read from LDS in the same permuted order.
//
// Backward, without atomics: D = rowsum(dO*O); a dQ kernel per query block
// (recomputing P and dP) and a dK/dV kernel per key block (over query blocks).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ inline bf16x8_t pack8(const float* v) {
  u32x4_t u;
  u.x = pack_bf2(v[0], v[1]);
  u.y = pack_bf2(v[2], v[3]);
  u.z = pack_bf2(v[4], v[5]);
  u.w = pack_bf2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

// two 4-element (8-byte) pieces at p and p+8 -> one 8-element operand
__device__ inline bf16x8_t ld_split8(const bf16_t* p) {
  const u32x2_t a = *reinterpret_cast<const u32x2_t*>(p);
  const u32x2_t b = *reinterpret_cast<const u32x2_t*>(p + 8);
  u32x4_t u;
  u.x = a.x; u.y = a.y; u.z = b.x; u.w = b.y;
  return __builtin_bit_cast(bf16x8_t, u);
}

template <int HD>
struct Tile {
  static constexpr int R = 64;       // rows (keys or queries) per LDS tile
  static constexpr int KS = HD + 8;  // [row][d] stride, elements
  static constexpr int TS = R + 8;   // [d][row] stride, elements
};

// [64 rows][HD] tile -> LDS [row][d]
template <int HD>
struct RowStager {
  static constexpr int NCH = 64 * HD / 8;
  static constexpr int PER = NCH / 256;
  uint4 r[PER];
  __device__ inline void load(const bf16_t* base, long ld, int row0, int T, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * 256, row = c / (HD / 8), cc = c % (HD / 8);
      r[i] = (row0 + row < T) ? *reinterpret_cast<const uint4*>(base + (long)(row0 + row) * ld + cc * 8)
                              : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ inline void store(bf16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * 256, row = c / (HD / 8), cc = c % (HD / 8);
      *reinterpret_cast<uint4*>(lds + row * Tile<HD>::KS + cc * 8) = r[i];
    }
  }
};

// [64 rows][HD] tile -> LDS [d][row] through 8x8 register transposes
template <int HD>
struct TrStager {
  static constexpr int NBLK = (64 / 8) * (HD / 8);
  static constexpr int PER = (NBLK + 255) / 256;
  uint4 r[PER * 8];
  __device__ inline void load(const bf16_t* base, long ld, int row0, int T, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bb = tid + i * 256, db = bb % (HD / 8), rb = bb / (HD / 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = row0 + rb * 8 + j;
        r[i * 8 + j] = (bb < NBLK && row < T) ? *reinterpret_cast<const uint4*>(base + (long)row * ld + db * 8)
                                              : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ inline void store(bf16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bb = tid + i * 256, db = bb % (HD / 8), rb = bb / (HD / 8);
      if (bb >= NBLK) continue;
      uint4 in[8], out[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) in[j] = r[i * 8 + j];
      transpose8x8_b16(in, out);
#pragma unroll
      for (int k = 0; k < 8; ++k) *reinterpret_cast<uint4*>(lds + (db * 8 + k) * Tile<HD>::TS + rb * 8) = out[k];
    }
  }
};

// ---------------------------------------------------------------------------
// forward

template <int HD>
__global__ void __launch_bounds__(256) attn_fwd_bf16_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ out,
                                                            float* __restrict__ lse, int T, int H) {
  constexpr int BQ = 128, BKV = 64, KS = Tile<HD>::KS, TS = Tile<HD>::TS, NDB = HD / 32, NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][BKV * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[2][HD * TS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, hl = lane >> 5;
  const int nqb = (T + BQ - 1) / BQ;
  const int qb = nqb - 1 - (int)blockIdx.x;  // longest causal rows first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const long ld = 3L * H * HD;
  const bf16_t* Q = qkv + (long)b * T * ld + h * HD;
  const bf16_t* K = Q + (long)H * HD;
  const bf16_t* V = Q + 2L * H * HD;
  const int q0 = qb * BQ + wave * 32;
  const int myq = q0 + lq;

  bf16x8_t qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (myq < T) u = *reinterpret_cast<const uint4*>(Q + (long)myq * ld + kk * 16 + hl * 8);
    qf[kk] = __builtin_bit_cast(bf16x8_t, u);
  }
  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float sl2 = LOG2E / sqrtf((float)HD);
  const int kv_end = min(T, (qb + 1) * BQ);
  const int nkv = (kv_end + BKV - 1) / BKV;

  RowStager<HD> ks;
  TrStager<HD> vs;
  ks.load(K, ld, 0, T, tid);
  vs.load(V, ld, 0, T, tid);
  ks.store(Ks[0], tid);
  vs.store(Vt[0], tid);
  __syncthreads();

  for (int it = 0; it < nkv; ++it) {
    const int cur = it & 1, k0 = it * BKV;
    if (it + 1 < nkv) {
      ks.load(K, ld, k0 + BKV, T, tid);
      vs.load(V, ld, k0 + BKV, T, tid);
    }
    if (k0 <= q0 + 31 && q0 < T) {
      f32x16_t s[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb2][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(Ks[cur] + (kb2 * 32 + lq) * KS + kk * 16 + hl * 8);
          s[kb2] = mfma32x32x16_bf16(ka, qf[kk], s[kb2]);
        }
      }
      float bmax = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb2 * 32 + acc_row(lane, r);
          float v = s[kb2][r] * sl2;
          if (key > myq || key >= T) v = -INFINITY;
          s[kb2][r] = v;
          bmax = fmaxf(bmax, v);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
      const float mnew = fmaxf(m, bmax);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = exp2f(m - muse);
      float rs = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[kb2][r] - muse);
          s[kb2][r] = p;
          rs += p;
        }
      rs += __shfl_xor(rs, 32, 64);
      l = l * alpha + rs;
      m = mnew;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          float pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pv[j] = s[kb2][8 * s_ + j];
          const bf16x8_t pb = pack8(pv);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8_t va = ld_split8(Vt[cur] + (db * 32 + lq) * TS + kb2 * 32 + 16 * s_ + hl * 4);
            oacc[db] = mfma32x32x16_bf16(va, pb, oacc[db]);
          }
        }
    }
    if (it + 1 < nkv) {
      ks.store(Ks[cur ^ 1], tid);
      vs.store(Vt[cur ^ 1], tid);
    }
    __syncthreads();
  }
  if (myq < T) {
    const float inv = 1.f / l;
    bf16_t* op = out + ((long)b * T + myq) * ((long)H * HD) + h * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hl * 4;
        uint2 u = make_uint2(pack_bf2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                             pack_bf2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(op + d) = u;
      }
    if (hl == 0) lse[(long)bh * T + myq] = (m + log2f(l)) * LN2;
  }
}

// ---------------------------------------------------------------------------
// backward: D = rowsum(dO * O)

template <typename T>
__device__ inline float ldv(const T* p);
template <>
__device__ inline float ldv<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <>
__device__ inline float ldv<float>(const float* p) { return *p; }

template <typename T>
__global__ void __launch_bounds__(256) attn_bwd_prep_kernel(const T* __restrict__ o, const T* __restrict__ dO,
                                                            float* __restrict__ D, int N, int T_, int H, int hd) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= N * H) return;
  const int n = w / H, h = w % H;
  const long off = (long)n * H * hd + h * hd;
  float s = 0.f;
  for (int i = lane; i < hd; i += 64) s += ldv<T>(o + off + i) * ldv<T>(dO + off + i);
  s = wave_sum(s);
  if (lane == 0) {
    const int b = n / T_, t = n % T_;
    D[((long)b * H + h) * T_ + t] = s;
  }
}

// dQ: per 128-query block, over key tiles up to the diagonal
template <int HD>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dO,
                                                          const float* __restrict__ lse, const float* __restrict__ Dv,
                                                          bf16_t* __restrict__ dqkv, int T, int H) {
  constexpr int BQ = 128, BKV = 64, KS = Tile<HD>::KS, TS = Tile<HD>::TS, NDB = HD / 32, NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[BKV * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[BKV * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Kt[HD * TS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, hl = lane >> 5;
  const int nqb = (T + BQ - 1) / BQ;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const long ld = 3L * H * HD, ldo = (long)H * HD;
  const bf16_t* Q = qkv + (long)b * T * ld + h * HD;
  const bf16_t* K = Q + (long)H * HD;
  const bf16_t* V = Q + 2L * H * HD;
  const bf16_t* G = dO + (long)b * T * ldo + h * HD;
  const int q0 = qb * BQ + wave * 32, myq = q0 + lq;

  bf16x8_t qf[NKK], gf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0), w = u;
    if (myq < T) {
      u = *reinterpret_cast<const uint4*>(Q + (long)myq * ld + kk * 16 + hl * 8);
      w = *reinterpret_cast<const uint4*>(G + (long)myq * ldo + kk * 16 + hl * 8);
    }
    qf[kk] = __builtin_bit_cast(bf16x8_t, u);
    gf[kk] = __builtin_bit_cast(bf16x8_t, w);
  }
  const float sl2 = LOG2E / sqrtf((float)HD);
  const float lse2 = myq < T ? lse[(long)bh * T + myq] * LOG2E : 0.f;
  const float Dq = myq < T ? Dv[(long)bh * T + myq] : 0.f;
  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  const int kv_end = min(T, (qb + 1) * BQ);
  const int nkv = (kv_end + BKV - 1) / BKV;
  RowStager<HD> sk, sv;
  TrStager<HD> st;
  for (int it = 0; it < nkv; ++it) {
    const int k0 = it * BKV;
    sk.load(K, ld, k0, T, tid);
    sv.load(V, ld, k0, T, tid);
    st.load(K, ld, k0, T, tid);
    sk.store(Ks, tid);
    sv.store(Vs, tid);
    st.store(Kt, tid);
    __syncthreads();
    if (k0 <= q0 + 31 && q0 < T) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x16_t s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int o = (kb2 * 32 + lq) * KS + kk * 16 + hl * 8;
          s = mfma32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(Ks + o), qf[kk], s);
          dp = mfma32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(Vs + o), gf[kk], dp);
        }
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb2 * 32 + acc_row(lane, r);
          const float p = (key <= myq && key < T && myq < T) ? exp2f(s[r] * sl2 - lse2) : 0.f;
          ds[r] = p * (dp[r] - Dq);
        }
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          const bf16x8_t db8 = pack8(ds + 8 * s_);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8_t ka = ld_split8(Kt + (db * 32 + lq) * TS + kb2 * 32 + 16 * s_ + hl * 4);
            acc[db] = mfma32x32x16_bf16(ka, db8, acc[db]);
          }
        }
      }
    }
    __syncthreads();
  }
  if (myq < T) {
    const float sc = 1.f / sqrtf((float)HD);
    bf16_t* op = dqkv + ((long)b * T + myq) * ld + h * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hl * 4;
        uint2 u = make_uint2(pack_bf2(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc),
                             pack_bf2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc));
        *reinterpret_cast<uint2*>(op + d) = u;
      }
  }
}

// dK, dV: per 128-key block (4 waves x 32 keys), over 64-query tiles from the diagonal on
template <int HD>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_kernel(const bf16_t* __restrict__ qkv,
                                                            const bf16_t* __restrict__ dO, const float* __restrict__ lse,
                                                            const float* __restrict__ Dv, bf16_t* __restrict__ dqkv,
                                                            int T, int H) {
  constexpr int BKEY = 128, BQT = 64, KS = Tile<HD>::KS, TS = Tile<HD>::TS, NDB = HD / 32, NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[BQT * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Qt[HD * TS];
  __shared__ __attribute__((aligned(16))) bf16_t Gs[BQT * KS];
  __shared__ __attribute__((aligned(16))) bf16_t Gt[HD * TS];
  __shared__ float L2s[BQT], Ds[BQT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lq = lane & 31, hl = lane >> 5;
  const int kb = blockIdx.x;  // lowest key blocks carry the most query tiles: launched first
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const long ld = 3L * H * HD, ldo = (long)H * HD;
  const bf16_t* Q = qkv + (long)b * T * ld + h * HD;
  const bf16_t* K = Q + (long)H * HD;
  const bf16_t* V = Q + 2L * H * HD;
  const bf16_t* G = dO + (long)b * T * ldo + h * HD;
  const int key0 = kb * BKEY + wave * 32, mykey = key0 + lq;

  bf16x8_t kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0), w = u;
    if (mykey < T) {
      u = *reinterpret_cast<const uint4*>(K + (long)mykey * ld + kk * 16 + hl * 8);
      w = *reinterpret_cast<const uint4*>(V + (long)mykey * ld + kk * 16 + hl * 8);
    }
    kf[kk] = __builtin_bit_cast(bf16x8_t, u);
    vf[kk] = __builtin_bit_cast(bf16x8_t, w);
  }
  const float sl2 = LOG2E / sqrtf((float)HD);
  f32x16_t dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[i][r] = 0.f; dv[i][r] = 0.f; }

  const int nqt = (T + BQT - 1) / BQT;
  RowStager<HD> sq, sg;
  TrStager<HD> tq, tg;
  for (int qt = (kb * BKEY) / BQT; qt < nqt; ++qt) {
    const int qb0 = qt * BQT;
    sq.load(Q, ld, qb0, T, tid);
    sg.load(G, ldo, qb0, T, tid);
    tq.load(Q, ld, qb0, T, tid);
    tg.load(G, ldo, qb0, T, tid);
    sq.store(Qs, tid);
    sg.store(Gs, tid);
    tq.store(Qt, tid);
    tg.store(Gt, tid);
    if (tid < BQT) {
      const int q = qb0 + tid;
      L2s[tid] = q < T ? lse[(long)bh * T + q] * LOG2E : 0.f;
      Ds[tid] = q < T ? Dv[(long)bh * T + q] : 0.f;
    }
    __syncthreads();
    if (qb0 + BQT - 1 >= key0 && key0 < T) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        if (qb0 + qs * 32 + 31 < key0) continue;
        f32x16_t s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int o = (qs * 32 + lq) * KS + kk * 16 + hl * 8;
          s = mfma32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(Qs + o), kf[kk], s);
          dp = mfma32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(Gs + o), vf[kk], dp);
        }
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qs * 32 + acc_row(lane, r);
          const int q = qb0 + ql;
          const bool ok = (q >= mykey && q < T && mykey < T);
          p[r] = ok ? exp2f(s[r] * sl2 - L2s[ql]) : 0.f;
          ds[r] = p[r] * (dp[r] - Ds[ql]);
        }
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          const bf16x8_t pa = pack8(p + 8 * s_);
          const bf16x8_t da = pack8(ds + 8 * s_);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int o = (db * 32 + lq) * TS + qs * 32 + 16 * s_ + hl * 4;
            dv[db] = mfma32x32x16_bf16(pa, ld_split8(Gt + o), dv[db]);
            dk[db] = mfma32x32x16_bf16(da, ld_split8(Qt + o), dk[db]);
          }
        }
      }
    }
    __syncthreads();
  }
  const float sc = 1.f / sqrtf((float)HD);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + acc_row(lane, r);
      if (key < T) {
        bf16_t* rowp = dqkv + ((long)b * T + key) * ld + h * HD + db * 32 + lq;
        rowp[(long)H * HD] = f2bf(dk[db][r] * sc);
        rowp[2L * H * HD] = f2bf(dv[db][r]);
      }
    }
}

// ---------------------------------------------------------------------------
// fp32 attention (plain per-row loops; used by the all-fp32 configuration)

template <int HD>
__global__ void __launch_bounds__(64) attn_fwd_f32_kernel(const float* __restrict__ qkv, float* __restrict__ out,
                                                          float* __restrict__ lse, int T, int H) {
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= T) return;
  const long ld = 3L * H * HD;
  const float* Q = qkv + (long)b * T * ld + h * HD;
  const float* K = Q + (long)H * HD;
  const float* V = Q + 2L * H * HD;
  const float sc = 1.f / sqrtf((float)HD);
  float q[HD], o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) { q[d] = Q[(long)i * ld + d]; o[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= i; ++j) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) s = fmaf(q[d], K[(long)j * ld + d], s);
    s *= sc;
    const float mn = fmaxf(m, s), a = expf(m - mn), p = expf(s - mn);
    l = l * a + p;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] = o[d] * a + p * V[(long)j * ld + d];
    m = mn;
  }
  float* op = out + ((long)b * T + i) * ((long)H * HD) + h * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) op[d] = o[d] / l;
  lse[(long)bh * T + i] = m + logf(l);
}

template <int HD>
__global__ void __launch_bounds__(64) attn_bwd_dq_f32_kernel(const float* __restrict__ qkv, const float* __restrict__ dO,
                                                             const float* __restrict__ lse, const float* __restrict__ Dv,
                                                             float* __restrict__ dqkv, int T, int H) {
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= T) return;
  const long ld = 3L * H * HD, ldo = (long)H * HD;
  const float* Q = qkv + (long)b * T * ld + h * HD;
  const float* K = Q + (long)H * HD;
  const float* V = Q + 2L * H * HD;
  const float* G = dO + (long)b * T * ldo + h * HD;
  const float sc = 1.f / sqrtf((float)HD);
  float q[HD], g[HD], dq[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) { q[d] = Q[(long)i * ld + d]; g[d] = G[(long)i * ldo + d]; dq[d] = 0.f; }
  const float L = lse[(long)bh * T + i], D = Dv[(long)bh * T + i];
  for (int j = 0; j <= i; ++j) {
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      s = fmaf(q[d], K[(long)j * ld + d], s);
      dp = fmaf(g[d], V[(long)j * ld + d], dp);
    }
    const float p = expf(s * sc - L), ds = p * (dp - D);
#pragma unroll
    for (int d = 0; d < HD; ++d) dq[d] = fmaf(ds, K[(long)j * ld + d], dq[d]);
  }
  float* op = dqkv + ((long)b * T + i) * ld + h * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) op[d] = dq[d] * sc;
}

template <int HD>
__global__ void __launch_bounds__(64) attn_bwd_dkdv_f32_kernel(const float* __restrict__ qkv,
                                                               const float* __restrict__ dO,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ Dv, float* __restrict__ dqkv,
                                                               int T, int H) {
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int j = blockIdx.x * 64 + threadIdx.x;
  if (j >= T) return;
  const long ld = 3L * H * HD, ldo = (long)H * HD;
  const float* Q = qkv + (long)b * T * ld + h * HD;
  const float* K = Q + (long)H * HD;
  const float* V = Q + 2L * H * HD;
  const float* G = dO + (long)b * T * ldo + h * HD;
  const float sc = 1.f / sqrtf((float)HD);
  float k[HD], v[HD], dk[HD], dv[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    k[d] = K[(long)j * ld + d]; v[d] = V[(long)j * ld + d]; dk[d] = 0.f; dv[d] = 0.f;
  }
  for (int i = j; i < T; ++i) {
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      s = fmaf(Q[(long)i * ld + d], k[d], s);
      dp = fmaf(G[(long)i * ldo + d], v[d], dp);
    }
    const float p = expf(s * sc - lse[(long)bh * T + i]);
    const float ds = p * (dp - Dv[(long)bh * T + i]);
#pragma unroll
    for (int d = 0; d < HD; ++d) {
      dv[d] = fmaf(p, G[(long)i * ldo + d], dv[d]);
      dk[d] = fmaf(ds, Q[(long)i * ld + d], dk[d]);
    }
  }
  float* rowp = dqkv + ((long)b * T + j) * ld + h * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    rowp[(long)H * HD + d] = dk[d] * sc;
    rowp[2L * H * HD + d] = dv[d];
  }
}

template <int HD>
void fwd_dispatch(const void* qkv, void* o, float* lse, int at, int B, int T, int H, hipStream_t st) {
  if (at == ACT_BF16)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<HD>, dim3((T + 127) / 128, B * H), dim3(256), 0, st,
                       (const bf16_t*)qkv, (bf16_t*)o, lse, T, H);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<HD>, dim3((T + 63) / 64, B * H), dim3(64), 0, st, (const float*)qkv,
                       (float*)o, lse, T, H);
}

template <int HD>
void bwd_dispatch(const void* qkv, const void* dO, const float* lse, const float* D, void* dqkv, int at, int B, int T,
                  int H, hipStream_t st) {
  if (at == ACT_BF16) {
    hipLaunchKernelGGL(attn_bwd_dq_kernel<HD>, dim3((T + 127) / 128, B * H), dim3(256), 0, st, (const bf16_t*)qkv,
                       (const bf16_t*)dO, lse, D, (bf16_t*)dqkv, T, H);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<HD>, dim3((T + 127) / 128, B * H), dim3(256), 0, st,
                       (const bf16_t*)qkv, (const bf16_t*)dO, lse, D, (bf16_t*)dqkv, T, H);
  } else {
    hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<HD>, dim3((T + 63) / 64, B * H), dim3(64), 0, st, (const float*)qkv,
                       (const float*)dO, lse, D, (float*)dqkv, T, H);
    hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<HD>, dim3((T + 63) / 64, B * H), dim3(64), 0, st,
                       (const float*)qkv, (const float*)dO, lse, D, (float*)dqkv, T, H);
  }
}

}  // namespace

void launch_attn_fwd(const void* qkv, void* o, float* lse, int at, int B, int T, int H, int hd, hipStream_t st) {
  if (B * T * H == 0) return;
  if (hd == 128) fwd_dispatch<128>(qkv, o, lse, at, B, T, H, st);
  else if (hd == 64) fwd_dispatch<64>(qkv, o, lse, at, B, T, H, st);
  else if (hd == 32) fwd_dispatch<32>(qkv, o, lse, at, B, T, H, st);
}

void launch_attn_bwd(const void* qkv, const void* o, const void* dO, const float* lse, float* D, void* dqkv, int at,
                     int B, int T, int H, int hd, hipStream_t st) {
  if (B * T * H == 0) return;
  const int N = B * T;
  if (at == ACT_BF16)
    hipLaunchKernelGGL(attn_bwd_prep_kernel<bf16_t>, dim3((N * H + 3) / 4), dim3(256), 0, st, (const bf16_t*)o,
                       (const bf16_t*)dO, D, N, T, H, hd);
  else
    hipLaunchKernelGGL(attn_bwd_prep_kernel<float>, dim3((N * H + 3) / 4), dim3(256), 0, st, (const float*)o,
                       (const float*)dO, D, N, T, H, hd);
  if (hd == 128) bwd_dispatch<128>(qkv, dO, lse, D, dqkv, at, B, T, H, st);
  else if (hd == 64) bwd_dispatch<64>(qkv, dO, lse, D, dqkv, at, B, T, H, st);
  else if (hd == 32) bwd_dispatch<32>(qkv, dO, lse, D, dqkv, at, B, T, H, st);
}
