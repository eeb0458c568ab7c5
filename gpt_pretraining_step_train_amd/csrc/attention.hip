// Causal multi-head attention of the GPT step (flash form) on gfx950.
//
// Layouts: qkv [B*T][(H + 2 Hkv) hd] (query head h at column h hd, key head j at
// H hd + j hd, value head j at (H + Hkv) hd + j hd, as the QKV projection writes it),
// o and dO [B*T][H*hd], lse and D [B][H][T] fp32.  Query head h reads key/value head
// h / G, G = H / Hkv (grouped-query attention; Hkv = H is multi-head attention).
// lse is the natural-log log-sum-exp of the scaled scores q.k/sqrt(hd).
//
// All three bf16 kernels stage 64-row tiles row-major in LDS (double-buffered,
// the next tile prefetched into registers during the current one).  Products
// that reduce over the head dimension read rows with ds_read_b128; products that
// reduce over keys or queries read columns with the gfx950 LDS transpose read
// (tr_operand), so no tile is ever transposed in registers.
//
// Forward: a workgroup owns 128 queries (4 waves x 32).  Each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so a lane owns one query and its
// softmax statistics are lane-local (plus one exchange with lane^32).  The
// probabilities feed O^T += V^T P^T straight from registers.  The running
// maximum is only raised when a tile's maximum exceeds it by more than 2^8 in
// probability (exponents stay <= 8), so the accumulator rescale is rare.
//
// Backward, without atomics: a dQ kernel per query block (recomputing P and dP; it
// also forms D = rowsum(dO*O) for its queries) and then a dK/dV kernel per key block
// (over query tiles, and over the G query heads of its key/value head) whose dK and
// dV accumulators live in different waves.  Blocks of one sequence-head run on one
// XCD, and so do the G query heads sharing a key/value head, so the tiles they
// stream stay in its L2.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_LOG2 = 8.f;  // lazy-rescale threshold of the forward (log2 units)
// waves (of 32 queries) per forward block: 4 (8 stage each K/V tile for twice the
// queries but measured 17% slower at d24: longer causal blocks, fewer rounds)
constexpr int kFwdWaves = 4;

__device__ inline bf16x8_t pack8(const float* v) {
  uint4 u;
  u.x = pack_bf2(v[0], v[1]);
  u.y = pack_bf2(v[2], v[3]);
  u.z = pack_bf2(v[4], v[5]);
  u.w = pack_bf2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS tile of 64 rows x HD bf16.  For HD = 128 rows are unpadded and the 16-byte
// chunk c of row r sits at chunk c ^ swz(r), swz(r) = (r%4)*4 + (r/4)%4: sixteen
// consecutive rows read at one chunk (ds_read_b128) and four consecutive rows read
// across four chunks (the transpose read) both land on distinct banks.  Other head
// sizes use rows padded by 16 bytes.
template <int HD>
struct Tile {
  static constexpr int RS = HD == 128 ? 128 : HD + 8;  // row stride (elements)
  static constexpr int ELEMS = 64 * RS;
  __device__ static inline int off(int r, int d) {
    if constexpr (HD == 128) {
      const int swz = ((r & 3) << 2) | ((r >> 2) & 3);
      return r * 128 + ((((d >> 3) ^ swz)) << 3) + (d & 7);
    } else {
      return r * (HD + 8) + d;
    }
  }
};

// tr_operand over a Tile: lane l receives column c0 + l%32 at rows
// r0 + 4hl + {0..3} and r0 + 8 + 4hl + {0..3} (hl = l/32)
template <int HD>
__device__ inline bf16x8_t tile_tr_operand(const bf16_t* T, int r0, int c0, int lane) {
  const int i = lane & 15;
  const int r = r0 + 4 * (lane >> 5) + (i >> 2), c = c0 + ((lane >> 4) & 1) * 16 + 4 * (i & 3);
  const i16x4_t a = lds_read_tr16(T + Tile<HD>::off(r, c));
  const i16x4_t b = lds_read_tr16(T + Tile<HD>::off(r + 8, c));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// [64 rows][HD] bf16 tile: global -> registers -> LDS [row][d]
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
      *reinterpret_cast<uint4*>(lds + Tile<HD>::off(row, cc * 8)) = r[i];
    }
  }
};

__device__ inline bf16x8_t lds_row8(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// transpose-read operand from two precomputed LDS addresses (rows r and r + 8 of
// the tile_tr_operand layout)
__device__ inline bf16x8_t lds_tr_pair(const bf16_t* lo, const bf16_t* hi) {
  const i16x4_t a = lds_read_tr16(lo);
  const i16x4_t b = lds_read_tr16(hi);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Block coordinates (bx within a sequence-head, by = sequence-head) such that all
// blocks of one sequence-head run on one XCD, one after another: workgroups go to the
// 8 XCDs round-robin in linear launch order, so the K/V (or Q/dO) tiles every block of
// a head streams stay in that XCD's L2.  With G > 1 the G consecutive sequence-heads
// that share one key/value head also follow each other on one XCD (when gridDim.y is
// a multiple of 8 G).  Plain coordinates when gridDim.y % 8 != 0.
__device__ inline void head_major_coords(int& bx, int& by, int G = 1) {
  const int nx = gridDim.x, ny = gridDim.y;
  if (ny % 8 != 0) {
    bx = blockIdx.x;
    by = blockIdx.y;
    return;
  }
  const int lin = blockIdx.y * nx + blockIdx.x, j = lin >> 3, r = j / nx, x = lin & 7;
  by = ny % (8 * G) == 0 ? ((r / G) * 8 + x) * G + r % G : r * 8 + x;
  bx = j % nx;
}

__device__ inline f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// Buffer descriptor over rows [row0, T) of a row-major [T][ld] bf16 matrix of which
// HD columns are read: a 16-byte load of a row at or past T returns zeros.
__device__ inline __amdgpu_buffer_rsrc_t rows_rsrc(const bf16_t* base, long ld, int row0, int T, int HD) {
  const uint32_t bytes = row0 < T ? (uint32_t)(((long)(T - row0 - 1) * ld + HD) * 2) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base + (long)row0 * ld), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ inline uint4 buf16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// two [64 rows][HD] bf16 tiles staged global -> registers -> LDS by NT threads; the
// per-thread global byte offsets (from the tile's first row) and LDS offsets are
// loop-invariant, each tile's rows come from a buffer descriptor that starts there
template <int HD, int NT>
struct PairStager {
  static constexpr int CPR = HD / 8, NCH = 64 * CPR, PER = (NCH + NT - 1) / NT;
  uint32_t voa[PER], vob[PER];
  int lo[PER];
  uint4 a[PER], b[PER];
  __device__ inline void init(long lda, long ldb, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = min(tid + i * NT, NCH - 1), row = c / CPR, cc = c % CPR;
      voa[i] = (uint32_t)(((long)row * lda + cc * 8) * 2);
      vob[i] = (uint32_t)(((long)row * ldb + cc * 8) * 2);
      lo[i] = Tile<HD>::off(row, cc * 8);
    }
  }
  __device__ inline void load(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (NCH % NT != 0 && tid + i * NT >= NCH) continue;
      a[i] = buf16(ra, voa[i]);
      b[i] = buf16(rb, vob[i]);
    }
  }
  __device__ inline void store(bf16_t* ta, bf16_t* tb, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (NCH % NT != 0 && tid + i * NT >= NCH) continue;
      *reinterpret_cast<uint4*>(ta + lo[i]) = a[i];
      *reinterpret_cast<uint4*>(tb + lo[i]) = b[i];
    }
  }
};

// Buffer-load DMA of 16-byte chunks straight into LDS (no registers): lane l of one
// instruction writes LDS bytes M0 + 16 l .. + 15.  Written in assembly (as in the GEMM)
// so that the compiler does not wait for every DMA before each LDS read; the waits are
// explicit (dma_wait_sync).
typedef unsigned int u32x4w_t __attribute__((ext_vector_type(4)));
__device__ inline u32x4w_t rows_words(const bf16_t* base, long ld, int row0, int T, int HD) {
  const uint32_t bytes = row0 < T ? (uint32_t)(((long)(T - row0 - 1) * ld + HD) * 2) : 0u;
  const uintptr_t a = (uintptr_t)(base + (long)row0 * ld);
  u32x4w_t r;
  r.x = (uint32_t)a;
  r.y = (uint32_t)(a >> 32) & 0xFFFFu;
  r.z = bytes;
  r.w = 0x00020000u;
  return r;
}
__device__ inline void attn_dma16(const u32x4w_t& rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// every DMA of this wave landed (vmcnt 0) and its LDS reads done, then a workgroup barrier
__device__ inline void dma_wait_sync() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((0 & 15) | (0 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// K and V tiles [64 rows][128] (Tile<128> layout) by DMA from NT threads: instruction j
// of thread tid fills LDS chunk p = j NT + tid, i.e. row p / 16 and physical chunk p % 16,
// which holds logical chunk (p % 16) ^ swz(row).  Rows at or past T read zeros (the
// descriptor ends at the sequence's last row).
template <int NT>
struct DmaTilePair {
  static constexpr int PER = 64 * 16 / NT;
  uint32_t voff[PER];
  __device__ inline void init(long ld, int tid) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int pch = j * NT + tid, row = pch >> 4, c = (pch & 15) ^ (((row & 3) << 2) | ((row >> 2) & 3));
      voff[j] = (uint32_t)(((long)row * ld + c * 8) * 2);
    }
  }
  __device__ inline void issue(const u32x4w_t& rk, const u32x4w_t& rv, const bf16_t* ks, const bf16_t* vs, int wave) {
    const uint32_t kl = (uint32_t)(uintptr_t)ks, vl = (uint32_t)(uintptr_t)vs;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      attn_dma16(rk, kl + (j * NT + wave * 64) * 16, voff[j]);
      attn_dma16(rv, vl + (j * NT + wave * 64) * 16, voff[j]);
    }
  }
};

// ---------------------------------------------------------------------------
// forward

// NW waves of 32 queries per block: every K/V tile staged in LDS serves 32 NW queries
// QKN: q and k are RMS-normalised per head (the step's QK-norm), so |q.k| <= hd (up to
// their bf16 rounding) and every scaled score s = q.k log2(e) / sqrt(hd) lies within
// +-sqrt(hd) log2(e) (16.3 for hd 128).  exp2(s - m) with the fixed reference m =
// sqrt(hd) log2(e) then lies in [2^-33, ~1]: no overflow, no underflow, and the same
// relative precision as with the running maximum, which this form neither computes nor
// rescales to.
template <int HD, int NW, bool QKN>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_bf16_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ out, float* __restrict__ lse, int T, int H,
                     int Hkv, int W, float* __restrict__ amax_part) {
  constexpr int BQ = 32 * NW, BKV = 64, TE = Tile<HD>::ELEMS, RS = Tile<HD>::RS, NDB = HD / 32, NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][TE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][TE];
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int nqb = (T + BQ - 1) / BQ;
  const int G = H / Hkv;
  int bx, bh;
  head_major_coords(bx, bh, G);
  const int qb = nqb - 1 - bx;  // longest causal rows first
  const int b = bh / H, h = bh % H;
  const long ld = (long)(H + 2 * Hkv) * HD;
  const bf16_t* Q = qkv + (long)b * T * ld + h * HD;
  const bf16_t* K = qkv + (long)b * T * ld + (long)(H + h / G) * HD;
  const bf16_t* V = K + (long)Hkv * HD;
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
  for (int i = 0; i < NDB; ++i) oacc[i] = zero16();
  // reference (log2 units) and sum: the running maximum, which starts finite so that a
  // lane whose keys in a tile are all masked (sliding window) gets p = 0, not NaN; or,
  // for QK-normalised inputs, the fixed bound of the scores
  float m = QKN ? sqrtf((float)HD) * LOG2E : -1e30f, l = 0.f;
  const float sl2 = LOG2E / sqrtf((float)HD);
  const int Wn = W > 0 ? W : T;  // keys a query sees, itself included
  const int kv_end = min(T, (qb + 1) * BQ);
  const int nkv = (kv_end + BKV - 1) / BKV;
  const int it0 = max(0, qb * BQ - Wn + 1) / BKV;  // first tile any query of the block sees

  // Per-lane LDS element offsets, loop-invariant: every fragment's tile row origin is
  // a multiple of 16, where the swizzle repeats, so it enters as an immediate.
  int kro[NKK];  // K rows for S^T: row lq, columns kk*16 + 8hl ...
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kro[kk] = Tile<HD>::off(lq, kk * 16 + hl * 8);
  const int i16 = lane & 15;
  const int trr = 4 * hl + (i16 >> 2), trc = ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
  int vro[NDB][2];  // V^T by transpose reads: rows trr and trr + 8 of a 16-row block
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    vro[db][0] = Tile<HD>::off(trr, db * 32 + trc);
    vro[db][1] = Tile<HD>::off(trr + 8, db * 32 + trc);
  }

  // K/V tiles: head_dim 128 by buffer-load DMA straight into LDS, other sizes through registers
  PairStager<HD == 128 ? 8 : HD, NW * 64> stg;  // unused for head_dim 128
  DmaTilePair<NW * 64> dma;
  if constexpr (HD == 128) {
    dma.init(ld, tid);
    dma.issue(rows_words(K, ld, it0 * BKV, T, HD), rows_words(V, ld, it0 * BKV, T, HD), Ks[0], Vs[0], wave);
    dma_wait_sync();
  } else {
    stg.init(ld, ld, tid);
    stg.load(rows_rsrc(K, ld, it0 * BKV, T, HD), rows_rsrc(V, ld, it0 * BKV, T, HD), tid);
    stg.store(Ks[0], Vs[0], tid);
    __syncthreads();
  }

  // one KV tile; the LDS buffer index is a compile-time constant (loop unrolled by 2)
  auto body = [&](auto cur_c, int it) {
    constexpr int cur = decltype(cur_c)::value;
    const int k0 = it * BKV;
    if (it + 1 < nkv) {  // the other buffer was last read in the previous tile, before its barrier
      if constexpr (HD == 128)
        dma.issue(rows_words(K, ld, k0 + BKV, T, HD), rows_words(V, ld, k0 + BKV, T, HD), Ks[cur ^ 1], Vs[cur ^ 1],
                  wave);
      else
        stg.load(rows_rsrc(K, ld, k0 + BKV, T, HD), rows_rsrc(V, ld, k0 + BKV, T, HD), tid);
    }
    // the wave's 32 queries see keys q0 - Wn + 1 .. q0 + 31
    if (k0 <= q0 + 31 && k0 + BKV - 1 >= q0 - Wn + 1 && q0 < T) {
      f32x16_t s[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16_t* kp = Ks[cur] + kb2 * 32 * RS;
        s[kb2] = mfma32x32x16_bf16(lds_row8(kp + kro[0]), qf[0], zero16());
#pragma unroll
        for (int kk = 1; kk < NKK; ++kk) s[kb2] = mfma32x32x16_bf16(lds_row8(kp + kro[kk]), qf[kk], s[kb2]);
      }
      if (k0 + BKV - 1 > q0 || k0 + BKV > T || k0 <= q0 + 31 - Wn) {  // diagonal, ragged or window edge
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb2 * 32 + acc_row(lane, r);
            if (key > myq || key >= T || key <= myq - Wn) s[kb2][r] = -INFINITY;
          }
      }
      if constexpr (!QKN) {
        float bmax = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[kb2][r]);
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64)) * sl2;
        const bool raise = bmax > m + RESCALE_LOG2;
        if (__builtin_amdgcn_ballot_w64(raise)) {
          const float mnew = raise ? bmax : m;
          const float alpha = fast_exp2(m - mnew);  // 0 on the first raise (m = -1e30)
          l *= alpha;
#pragma unroll
          for (int i = 0; i < NDB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
          m = mnew;
        }
      }
      float rs = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kb2][r], sl2, -m));
          s[kb2][r] = p;
          rs += p;
        }
      l += rs + __shfl_xor(rs, 32, 64);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          float pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pv[j] = s[kb2][8 * s_ + j];
          const bf16x8_t pb = pack8(pv);
          const bf16_t* vp = Vs[cur] + (kb2 * 32 + 16 * s_) * RS;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            oacc[db] = mfma32x32x16_bf16(lds_tr_pair(vp + vro[db][0], vp + vro[db][1]), pb, oacc[db]);
        }
    }
    if constexpr (HD == 128) {
      dma_wait_sync();
    } else {
      if (it + 1 < nkv) stg.store(Ks[cur ^ 1], Vs[cur ^ 1], tid);
      __syncthreads();
    }
  };
  for (int it = it0; it < nkv; it += 2) {
    body(std::integral_constant<int, 0>{}, it);
    if (it + 1 < nkv) body(std::integral_constant<int, 1>{}, it + 1);
  }
  float mo = 0.f;  // max |o| of the lane as stored (amax_part)
  // The wave's 32 queries x HD go through LDS so that they leave as whole rows, 16 bytes
  // per lane (a lane holds four dimensions of one query per store otherwise).  Every wave
  // is past the last tile's barrier, so the K / V buffers are free: the first half of the
  // waves stage in Ks, the others in Vs (padded rows).
  {
    constexpr int SR = HD + 8, LPR = HD / 8, RPI = 64 / LPR, NH = NW / 2;
    static_assert(NW % 2 == 0 && NH * 32 * SR <= 2 * TE, "staging fits the tile buffers");
    bf16_t* sb = (wave < NH ? &Ks[0][0] : &Vs[0][0]) + (wave % NH) * 32 * SR;
    const float inv = myq < T ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + hl * 4;
        float ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = oacc[db][4 * g + e] * inv;
          mo = fmaxf(mo, fabsf(ov[e]));
        }
        *reinterpret_cast<uint2*>(sb + lq * SR + d) = make_uint2(pack_bf2(ov[0], ov[1]), pack_bf2(ov[2], ov[3]));
      }
    if (myq < T && hl == 0) lse[(long)bh * T + myq] = (m + log2f(l)) * LN2;
    __syncthreads();
    const int c8 = (lane % LPR) * 8, rl = lane / LPR;
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPI) {
      const int q = q0 + r0 + rl;
      if (q < T)
        *reinterpret_cast<uint4*>(out + ((long)b * T + q) * ((long)H * HD) + h * HD + c8) =
            *reinterpret_cast<const uint4*>(sb + (r0 + rl) * SR + c8);
    }
  }
  if (amax_part) {  // one entry per wave
    mo = wave_max(mo);
    if (lane == 0) amax_part[((long)blockIdx.y * gridDim.x + blockIdx.x) * NW + wave] = bf16_round(mo);
  }
}

// Forward with 64 queries per wave (two 32-query column blocks): every K and V
// fragment read from LDS feeds two MFMAs, half the LDS traffic per flop of the 32-query
// form.  The state (O^T 2 x 4 accumulators, two S^T tiles, Q fragments of 64 queries)
// needs one wave per SIMD: 4 waves, 256 queries per block.  Same tile staging, masking,
// lazy rescale and output as attn_fwd_bf16_kernel.
template <int HD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_q64_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ out, float* __restrict__ lse, int T, int H,
                    int Hkv, int W) {
  constexpr int NW = 4, BQ = 64 * NW, BKV = 64, TE = Tile<HD>::ELEMS, RS = Tile<HD>::RS, NDB = HD / 32,
                NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][TE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][TE];
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (T + BQ - 1) / BQ;
  const int G = H / Hkv;
  int bx, bh;
  head_major_coords(bx, bh, G);
  const int qb = nqb - 1 - bx;  // longest causal rows first
  const int b = bh / H, h = bh % H;
  const long ld = (long)(H + 2 * Hkv) * HD;
  const bf16_t* Q = qkv + (long)b * T * ld + h * HD;
  const bf16_t* K = qkv + (long)b * T * ld + (long)(H + h / G) * HD;
  const bf16_t* V = K + (long)Hkv * HD;
  const int q0 = qb * BQ + wave * 64;  // the wave's queries q0 .. q0 + 63, column block c: q0 + 32c + lq

  bf16x8_t qf[2][NKK];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int q = q0 + 32 * c + lq;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (q < T) u = *reinterpret_cast<const uint4*>(Q + (long)q * ld + kk * 16 + hl * 8);
      qf[c][kk] = __builtin_bit_cast(bf16x8_t, u);
    }
  f32x16_t oacc[2][NDB];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[c][i] = zero16();
  float m[2] = {-1e30f, -1e30f}, l[2] = {0.f, 0.f};
  const float sl2 = LOG2E / sqrtf((float)HD);
  const int Wn = W > 0 ? W : T;
  const int kv_end = min(T, (qb + 1) * BQ);
  const int nkv = (kv_end + BKV - 1) / BKV;
  const int it0 = max(0, qb * BQ - Wn + 1) / BKV;

  int kro[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kro[kk] = Tile<HD>::off(lq, kk * 16 + hl * 8);
  const int i16 = lane & 15;
  const int trr = 4 * hl + (i16 >> 2), trc = ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
  int vro[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    vro[db][0] = Tile<HD>::off(trr, db * 32 + trc);
    vro[db][1] = Tile<HD>::off(trr + 8, db * 32 + trc);
  }

  static_assert(HD == 128, "DMA tile layout is Tile<128>");
  DmaTilePair<NW * 64> dma;
  dma.init(ld, tid);
  dma.issue(rows_words(K, ld, it0 * BKV, T, HD), rows_words(V, ld, it0 * BKV, T, HD), Ks[0], Vs[0], wave);
  dma_wait_sync();

  auto body = [&](auto cur_c, int it) {
    constexpr int cur = decltype(cur_c)::value;
    const int k0 = it * BKV;
    // the next tile into the other stage, which every wave finished reading before the
    // barrier that ended the previous tile
    if (it + 1 < nkv)
      dma.issue(rows_words(K, ld, k0 + BKV, T, HD), rows_words(V, ld, k0 + BKV, T, HD), Ks[cur ^ 1], Vs[cur ^ 1],
                wave);
    // the wave's 64 queries see keys q0 - Wn + 1 .. q0 + 63
    if (k0 <= q0 + 63 && k0 + BKV - 1 >= q0 - Wn + 1 && q0 < T) {
      f32x16_t s[2][2];  // [key block][query column block]
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16_t* kp = Ks[cur] + kb2 * 32 * RS;
        bf16x8_t kf = lds_row8(kp + kro[0]);
        s[kb2][0] = mfma32x32x16_bf16(kf, qf[0][0], zero16());
        s[kb2][1] = mfma32x32x16_bf16(kf, qf[1][0], zero16());
#pragma unroll
        for (int kk = 1; kk < NKK; ++kk) {
          kf = lds_row8(kp + kro[kk]);
          s[kb2][0] = mfma32x32x16_bf16(kf, qf[0][kk], s[kb2][0]);
          s[kb2][1] = mfma32x32x16_bf16(kf, qf[1][kk], s[kb2][1]);
        }
      }
      if (k0 + BKV - 1 > q0 || k0 + BKV > T || k0 <= q0 + 63 - Wn) {  // diagonal, ragged or window edge
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int myq = q0 + 32 * c + lq;
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb2 * 32 + acc_row(lane, r);
              if (key > myq || key >= T || key <= myq - Wn) s[kb2][c][r] = -INFINITY;
            }
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float bmax = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[kb2][c][r]);
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64)) * sl2;
        const bool raise = bmax > m[c] + RESCALE_LOG2;
        if (__builtin_amdgcn_ballot_w64(raise)) {
          const float mnew = raise ? bmax : m[c];
          const float alpha = fast_exp2(m[c] - mnew);
          l[c] *= alpha;
#pragma unroll
          for (int i = 0; i < NDB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[c][i][r] *= alpha;
          m[c] = mnew;
        }
        float rs = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = fast_exp2(fmaf(s[kb2][c][r], sl2, -m[c]));
            s[kb2][c][r] = pr;
            rs += pr;
          }
        l[c] += rs + __shfl_xor(rs, 32, 64);
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          bf16x8_t pb[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            float pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pv[j] = s[kb2][c][8 * s_ + j];
            pb[c] = pack8(pv);
          }
          const bf16_t* vp = Vs[cur] + (kb2 * 32 + 16 * s_) * RS;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8_t vf = lds_tr_pair(vp + vro[db][0], vp + vro[db][1]);
            oacc[0][db] = mfma32x32x16_bf16(vf, pb[0], oacc[0][db]);
            oacc[1][db] = mfma32x32x16_bf16(vf, pb[1], oacc[1][db]);
          }
        }
    }
    dma_wait_sync();
  };
  for (int it = it0; it < nkv; it += 2) {
    body(std::integral_constant<int, 0>{}, it);
    if (it + 1 < nkv) body(std::integral_constant<int, 1>{}, it + 1);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int myq = q0 + 32 * c + lq;
    if (myq < T) {
      const float inv = 1.f / l[c];
      bf16_t* op = out + ((long)b * T + myq) * ((long)H * HD) + h * HD;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + g * 8 + hl * 4;
          uint2 u = make_uint2(pack_bf2(oacc[c][db][4 * g] * inv, oacc[c][db][4 * g + 1] * inv),
                               pack_bf2(oacc[c][db][4 * g + 2] * inv, oacc[c][db][4 * g + 3] * inv));
          *reinterpret_cast<uint2*>(op + d) = u;
        }
      if (hl == 0) lse[(long)bh * T + myq] = (m[c] + log2f(l[c])) * LN2;
    }
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

// dQ: per 128-query block (4 waves x 32 queries, a lane owns a query), over key
// tiles up to the diagonal.  dQ^T += K^T dS^T with K^T read by transpose.
template <int HD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ o, const bf16_t* __restrict__ dO,
                   const float* __restrict__ lse, float* __restrict__ Dv, bf16_t* __restrict__ dqkv, int T, int H,
                   int Hkv, int W) {
  constexpr int BQ = 128, BKV = 64, TE = Tile<HD>::ELEMS, RS = Tile<HD>::RS, NDB = HD / 32, NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][TE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][TE];
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int nqb = (T + BQ - 1) / BQ;
  const int Gq = H / Hkv;
  int bx, bh;
  head_major_coords(bx, bh, Gq);
  const int qb = nqb - 1 - bx;
  const int b = bh / H, h = bh % H;
  const long ld = (long)(H + 2 * Hkv) * HD, ldo = (long)H * HD;
  const bf16_t* Q = qkv + (long)b * T * ld + h * HD;
  const bf16_t* K = qkv + (long)b * T * ld + (long)(H + h / Gq) * HD;
  const bf16_t* V = K + (long)Hkv * HD;
  const bf16_t* G = dO + (long)b * T * ldo + h * HD;
  const int q0 = qb * BQ + wave * 32, myq = q0 + lq;

  // the query's q and dO rows (lane half hl holds 8-element chunks 2kk + hl), and
  // D = rowsum(dO * O), which this kernel also writes for the dK/dV kernel
  const bf16_t* O = o + (long)b * T * ldo + h * HD;
  bf16x8_t qf[NKK], gf[NKK];
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0), w = u, x = u;
    if (myq < T) {
      u = *reinterpret_cast<const uint4*>(Q + (long)myq * ld + kk * 16 + hl * 8);
      w = *reinterpret_cast<const uint4*>(G + (long)myq * ldo + kk * 16 + hl * 8);
      x = *reinterpret_cast<const uint4*>(O + (long)myq * ldo + kk * 16 + hl * 8);
    }
    qf[kk] = __builtin_bit_cast(bf16x8_t, u);
    gf[kk] = __builtin_bit_cast(bf16x8_t, w);
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w}, xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dsum += __uint_as_float(wv[e] << 16) * __uint_as_float(xv[e] << 16) +
              __uint_as_float(wv[e] & 0xFFFF0000u) * __uint_as_float(xv[e] & 0xFFFF0000u);
  }
  const float Dq = dsum + __shfl_xor(dsum, 32, 64);
  if (hl == 0 && myq < T) Dv[(long)bh * T + myq] = Dq;
  const float sl2 = LOG2E / sqrtf((float)HD);
  const float lse2 = myq < T ? lse[(long)bh * T + myq] * LOG2E : 0.f;
  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  // per-lane LDS element offsets, loop-invariant (row origins are multiples of 16)
  int kro[NKK];  // K and V rows for S^T and dP^T
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kro[kk] = Tile<HD>::off(lq, kk * 16 + hl * 8);
  const int i16 = lane & 15;
  const int trr = 4 * hl + (i16 >> 2), trc = ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
  int ktr[NDB][2];  // K^T by transpose reads
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    ktr[db][0] = Tile<HD>::off(trr, db * 32 + trc);
    ktr[db][1] = Tile<HD>::off(trr + 8, db * 32 + trc);
  }

  const int Wn = W > 0 ? W : T;  // keys a query sees, itself included
  const int kv_end = min(T, (qb + 1) * BQ);
  const int nkv = (kv_end + BKV - 1) / BKV;
  const int it0 = max(0, qb * BQ - Wn + 1) / BKV;  // first tile any query of the block sees
  // K/V tiles: head_dim 128 by buffer-load DMA straight into LDS (no registers held
  // across the tile), other sizes through registers
  PairStager<HD == 128 ? 8 : HD, 256> stg;  // unused for head_dim 128
  DmaTilePair<256> dma;
  if constexpr (HD == 128) {
    dma.init(ld, tid);
    dma.issue(rows_words(K, ld, it0 * BKV, T, HD), rows_words(V, ld, it0 * BKV, T, HD), Ks[0], Vs[0], wave);
    dma_wait_sync();
  } else {
    stg.init(ld, ld, tid);
    stg.load(rows_rsrc(K, ld, it0 * BKV, T, HD), rows_rsrc(V, ld, it0 * BKV, T, HD), tid);
    stg.store(Ks[0], Vs[0], tid);
    __syncthreads();
  }
  auto body = [&](auto cur_c, int it) {
    constexpr int cur = decltype(cur_c)::value;
    const int k0 = it * BKV;
    if (it + 1 < nkv) {  // the other buffer was last read in the previous tile, before its barrier
      if constexpr (HD == 128)
        dma.issue(rows_words(K, ld, k0 + BKV, T, HD), rows_words(V, ld, k0 + BKV, T, HD), Ks[cur ^ 1], Vs[cur ^ 1],
                  wave);
      else
        stg.load(rows_rsrc(K, ld, k0 + BKV, T, HD), rows_rsrc(V, ld, k0 + BKV, T, HD), tid);
    }
    if (k0 <= q0 + 31 && k0 + BKV - 1 >= q0 - Wn + 1 && q0 < T) {
      const bool mask = k0 + BKV - 1 > q0 || k0 + BKV > T || k0 <= q0 + 31 - Wn;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16_t* kp = Ks[cur] + kb2 * 32 * RS;
        const bf16_t* vp = Vs[cur] + kb2 * 32 * RS;
        f32x16_t s = mfma32x32x16_bf16(lds_row8(kp + kro[0]), qf[0], zero16());
        f32x16_t dp = mfma32x32x16_bf16(lds_row8(vp + kro[0]), gf[0], zero16());
#pragma unroll
        for (int kk = 1; kk < NKK; ++kk) {
          s = mfma32x32x16_bf16(lds_row8(kp + kro[kk]), qf[kk], s);
          dp = mfma32x32x16_bf16(lds_row8(vp + kro[kk]), gf[kk], dp);
        }
        if (mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb2 * 32 + acc_row(lane, r);
            if (key > myq || key >= T || key <= myq - Wn) s[r] = -INFINITY;
          }
        }
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(fmaf(s[r], sl2, -lse2)) * (dp[r] - Dq);
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          const bf16x8_t db8 = pack8(ds + 8 * s_);
          const bf16_t* tp = kp + 16 * s_ * RS;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = mfma32x32x16_bf16(lds_tr_pair(tp + ktr[db][0], tp + ktr[db][1]), db8, acc[db]);
        }
      }
    }
    if constexpr (HD == 128) {
      dma_wait_sync();
    } else {
      if (it + 1 < nkv) stg.store(Ks[cur ^ 1], Vs[cur ^ 1], tid);
      __syncthreads();
    }
  };
  for (int it = it0; it < nkv; it += 2) {
    body(std::integral_constant<int, 0>{}, it);
    if (it + 1 < nkv) body(std::integral_constant<int, 1>{}, it + 1);
  }
  const float sc = 1.f / sqrtf((float)HD);
  // The wave's 32 queries x HD go through LDS so that they leave as whole rows, 16 bytes
  // per lane (a lane holds four dimensions of one query per store otherwise).  Every
  // wave is past the last tile's barrier, so the K / V buffers are free: waves 0, 1
  // stage in Ks, waves 2, 3 in Vs (padded rows).
  constexpr int SR = HD + 8, LPR = HD / 8, RPI = 64 / LPR;
  static_assert(2 * 32 * SR <= 2 * TE, "staging fits the tile buffers");
  bf16_t* sb = (wave < 2 ? &Ks[0][0] : &Vs[0][0]) + (wave & 1) * 32 * SR;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + hl * 4;
      *reinterpret_cast<uint2*>(sb + lq * SR + d) =
          make_uint2(pack_bf2(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc),
                     pack_bf2(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc));
    }
  __syncthreads();
  const int c8 = (lane % LPR) * 8, rl = lane / LPR;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int q = q0 + r0 + rl;
    if (q < T)
      *reinterpret_cast<uint4*>(dqkv + ((long)b * T + q) * ld + h * HD + c8) =
          *reinterpret_cast<const uint4*>(sb + (r0 + rl) * SR + c8);
  }
}

// dQ with 64 queries per wave (two 32-query column blocks), one wave per SIMD, 256
// queries per block: every K, V and K^T fragment read from LDS feeds two MFMAs.  K/V
// tiles by buffer-load DMA, double-buffered.  Also writes D = rowsum(dO * O).
template <int HD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bwd_dq_q64_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ o, const bf16_t* __restrict__ dO,
                       const float* __restrict__ lse, float* __restrict__ Dv, bf16_t* __restrict__ dqkv, int T, int H,
                       int Hkv, int W) {
  static_assert(HD == 128, "DMA tile layout is Tile<128>");
  constexpr int NW = 4, BQ = 64 * NW, BKV = 64, TE = Tile<HD>::ELEMS, RS = Tile<HD>::RS, NDB = HD / 32,
                NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][TE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][TE];
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (T + BQ - 1) / BQ;
  const int Gq = H / Hkv;
  int bx, bh;
  head_major_coords(bx, bh, Gq);
  const int qb = nqb - 1 - bx;
  const int b = bh / H, h = bh % H;
  const long ld = (long)(H + 2 * Hkv) * HD, ldo = (long)H * HD;
  const bf16_t* Q = qkv + (long)b * T * ld + h * HD;
  const bf16_t* K = qkv + (long)b * T * ld + (long)(H + h / Gq) * HD;
  const bf16_t* V = K + (long)Hkv * HD;
  const bf16_t* G = dO + (long)b * T * ldo + h * HD;
  const bf16_t* O = o + (long)b * T * ldo + h * HD;
  const int q0 = qb * BQ + wave * 64;  // the wave's queries: column block c holds q0 + 32c + lq

  bf16x8_t qf[2][NKK], gf[2][NKK];
  float Dq[2], lse2[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int myq = q0 + 32 * c + lq;
    float dsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0), w = u, x = u;
      if (myq < T) {
        u = *reinterpret_cast<const uint4*>(Q + (long)myq * ld + kk * 16 + hl * 8);
        w = *reinterpret_cast<const uint4*>(G + (long)myq * ldo + kk * 16 + hl * 8);
        x = *reinterpret_cast<const uint4*>(O + (long)myq * ldo + kk * 16 + hl * 8);
      }
      qf[c][kk] = __builtin_bit_cast(bf16x8_t, u);
      gf[c][kk] = __builtin_bit_cast(bf16x8_t, w);
      const uint32_t wv[4] = {w.x, w.y, w.z, w.w}, xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dsum += __uint_as_float(wv[e] << 16) * __uint_as_float(xv[e] << 16) +
                __uint_as_float(wv[e] & 0xFFFF0000u) * __uint_as_float(xv[e] & 0xFFFF0000u);
    }
    Dq[c] = dsum + __shfl_xor(dsum, 32, 64);
    if (hl == 0 && myq < T) Dv[(long)bh * T + myq] = Dq[c];
    lse2[c] = myq < T ? lse[(long)bh * T + myq] * LOG2E : 0.f;
  }
  const float sl2 = LOG2E / sqrtf((float)HD);
  f32x16_t acc[2][NDB];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[c][i] = zero16();
  int kro[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kro[kk] = Tile<HD>::off(lq, kk * 16 + hl * 8);
  const int i16 = lane & 15;
  const int trr = 4 * hl + (i16 >> 2), trc = ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
  int ktr[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    ktr[db][0] = Tile<HD>::off(trr, db * 32 + trc);
    ktr[db][1] = Tile<HD>::off(trr + 8, db * 32 + trc);
  }
  const int Wn = W > 0 ? W : T;
  const int kv_end = min(T, (qb + 1) * BQ);
  const int nkv = (kv_end + BKV - 1) / BKV;
  const int it0 = max(0, qb * BQ - Wn + 1) / BKV;
  DmaTilePair<NW * 64> dma;
  dma.init(ld, tid);
  dma.issue(rows_words(K, ld, it0 * BKV, T, HD), rows_words(V, ld, it0 * BKV, T, HD), Ks[0], Vs[0], wave);
  dma_wait_sync();
  auto body = [&](auto cur_c, int it) {
    constexpr int cur = decltype(cur_c)::value;
    const int k0 = it * BKV;
    if (it + 1 < nkv)
      dma.issue(rows_words(K, ld, k0 + BKV, T, HD), rows_words(V, ld, k0 + BKV, T, HD), Ks[cur ^ 1], Vs[cur ^ 1],
                wave);
    if (k0 <= q0 + 63 && k0 + BKV - 1 >= q0 - Wn + 1 && q0 < T) {
      const bool mask = k0 + BKV - 1 > q0 || k0 + BKV > T || k0 <= q0 + 63 - Wn;
#pragma unroll 1
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16_t* kp = Ks[cur] + kb2 * 32 * RS;
        const bf16_t* vp = Vs[cur] + kb2 * 32 * RS;
        f32x16_t sv[2], dp[2];  // [query column block]: S^T and dP^T [key rows][query = lane]
        {
          bf16x8_t ka = lds_row8(kp + kro[0]), va = lds_row8(vp + kro[0]);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            sv[c] = mfma32x32x16_bf16(ka, qf[c][0], zero16());
            dp[c] = mfma32x32x16_bf16(va, gf[c][0], zero16());
          }
#pragma unroll
          for (int kk = 1; kk < NKK; ++kk) {
            ka = lds_row8(kp + kro[kk]);
            va = lds_row8(vp + kro[kk]);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              sv[c] = mfma32x32x16_bf16(ka, qf[c][kk], sv[c]);
              dp[c] = mfma32x32x16_bf16(va, gf[c][kk], dp[c]);
            }
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int myq = q0 + 32 * c + lq;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = sv[c][r];
            if (mask) {
              const int key = k0 + kb2 * 32 + acc_row(lane, r);
              if (key > myq || key >= T || key <= myq - Wn) x = -INFINITY;
            }
            dp[c][r] = fast_exp2(fmaf(x, sl2, -lse2[c])) * (dp[c][r] - Dq[c]);  // dS
          }
        }
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          bf16x8_t da[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            float w8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w8[j] = dp[c][8 * s_ + j];
            da[c] = pack8(w8);
          }
          const bf16_t* tp = kp + 16 * s_ * RS;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8_t kt = lds_tr_pair(tp + ktr[db][0], tp + ktr[db][1]);
            acc[0][db] = mfma32x32x16_bf16(kt, da[0], acc[0][db]);
            acc[1][db] = mfma32x32x16_bf16(kt, da[1], acc[1][db]);
          }
        }
      }
    }
    dma_wait_sync();
  };
  for (int it = it0; it < nkv; it += 2) {
    body(std::integral_constant<int, 0>{}, it);
    if (it + 1 < nkv) body(std::integral_constant<int, 1>{}, it + 1);
  }
  const float sc = 1.f / sqrtf((float)HD);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int myq = q0 + 32 * c + lq;
    if (myq < T) {
      bf16_t* op = dqkv + ((long)b * T + myq) * ld + h * HD;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + g * 8 + hl * 4;
          uint2 u = make_uint2(pack_bf2(acc[c][db][4 * g] * sc, acc[c][db][4 * g + 1] * sc),
                               pack_bf2(acc[c][db][4 * g + 2] * sc, acc[c][db][4 * g + 3] * sc));
          *reinterpret_cast<uint2*>(op + d) = u;
        }
    }
  }
}

// dK, dV with the two accumulations in different waves: 8 waves per 128-key block,
// waves 0-3 accumulate dV (S -> P, dV += P^T dO) and waves 4-7 dK (dP, P -> dS,
// dK += dS^T Q) for the same 32 keys, each role 32 MFMAs per 64-query tile.  P
// passes from the dV waves to the dK waves through LDS in bf16 (the precision the dV
// waves' own MFMA takes it in); each wave holds one 32x128
// accumulator, so two waves fit on every SIMD; the Q and dO tiles are staged once
// for all eight.  A lane owns a key.  A block serves one key/value head: it walks the
// query tiles of each of the G query heads that read it, one head after another,
// into the same accumulators.
template <int HD>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_split_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dO,
                           const float* __restrict__ lse, const float* __restrict__ Dv, bf16_t* __restrict__ dqkv,
                           int T, int H, int Hkv, int W, float* __restrict__ amax_part) {
  constexpr int BKEY = 128, BQT = 64, TE = Tile<HD>::ELEMS, RS = Tile<HD>::RS, NDB = HD / 32, NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][TE];
  __shared__ __attribute__((aligned(16))) bf16_t Gs[2][TE];
  __shared__ __attribute__((aligned(16))) float L2s[2][BQT], Ds[2][BQT];
  __shared__ __attribute__((aligned(16))) uint2 Ps[2][4][4][64];  // bf16 P: [half][key wave][reg/4][lane] x 4
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const bool dk_role = wave >= 4;
  const int kw = wave & 3;
  int kb, bk;
  head_major_coords(kb, bk);  // lowest key blocks carry the most query tiles: launched first
  const int G = H / Hkv, b = bk / Hkv, hk = bk % Hkv;
  const long ld = (long)(H + 2 * Hkv) * HD, ldo = (long)H * HD;
  const bf16_t* Qb = qkv + (long)b * T * ld;  // query head qh at column qh * HD
  const bf16_t* K = Qb + (long)(H + hk) * HD;
  const bf16_t* V = K + (long)Hkv * HD;
  const bf16_t* Gb = dO + (long)b * T * ldo;
  const long lrow = (long)b * H * T;  // lse / D of query head qh at lrow + qh * T
  const int key0 = kb * BKEY + kw * 32, mykey = key0 + lq;

  bf16x8_t kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0), w = u;
    if (mykey < T) {
      u = *reinterpret_cast<const uint4*>(K + (long)mykey * ld + kk * 16 + hl * 8);
      if (dk_role) w = *reinterpret_cast<const uint4*>(V + (long)mykey * ld + kk * 16 + hl * 8);
    }
    kf[kk] = __builtin_bit_cast(bf16x8_t, u);
    vf[kk] = __builtin_bit_cast(bf16x8_t, w);
  }
  const float sl2 = LOG2E / sqrtf((float)HD);
  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  // per-lane LDS element offsets, loop-invariant (row origins are multiples of 16)
  int qro[NKK];  // Q and dO rows for S^T and dP^T
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qro[kk] = Tile<HD>::off(lq, kk * 16 + hl * 8);
  const int i16 = lane & 15;
  const int trr = 4 * hl + (i16 >> 2), trc = ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
  int tro[NDB][2];  // dO (dV waves) or Q (dK waves) by transpose reads
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    tro[db][0] = Tile<HD>::off(trr, db * 32 + trc);
    tro[db][1] = Tile<HD>::off(trr + 8, db * 32 + trc);
  }

  const int Wn = W > 0 ? W : T;  // keys a query sees, itself included
  // query tiles from the block's first key to the last query that sees its last key
  const int nqt = min((T + BQT - 1) / BQT, (kb * BKEY + BKEY - 1 + Wn - 1) / BQT + 1);
  const int qt0 = (kb * BKEY) / BQT;
  // G (nqt - qt0) steps: the query tiles qt0 .. nqt-1 of query head hk G, then of the
  // next query head of the group, ...
  const int nsteps = G * (nqt - qt0);
  // 64-row Q and dO tiles and their lse / D values, prefetched one step ahead
  PairStager<HD, 512> stg;
  stg.init(ld, ldo, tid);
  float pl = 0.f, pd = 0.f;
  int ld_h = hk * G, ld_t = qt0;  // (query head, query tile) of the step the next load fetches
  int cur_t = qt0;                // query tile of the step being computed
  auto load = [&]() {
    const int q0 = ld_t * BQT;
    stg.load(rows_rsrc(Qb + ld_h * HD, ld, q0, T, HD), rows_rsrc(Gb + ld_h * HD, ldo, q0, T, HD), tid);
    if (tid < BQT) {
      const int q = q0 + tid;
      const long r = lrow + (long)ld_h * T + q;
      pl = q < T ? lse[r] * LOG2E : 0.f;
      pd = q < T ? Dv[r] : 0.f;
    }
    if (++ld_t == nqt) {
      ld_t = qt0;
      ++ld_h;
    }
  };
  auto store = [&](int buf) {
    stg.store(Qs[buf], Gs[buf], tid);
    if (tid < BQT) {
      L2s[buf][tid] = pl;
      Ds[buf][tid] = pd;
    }
  };
  if (nsteps > 0) {
    load();
    store(0);
  }
  __syncthreads();
  // Per query tile, phase 1: the dV waves form S and P = exp(S - lse) for both
  // 32-query halves and publish P (fp32, lane for lane: both roles hold the same keys
  // and queries in the same accumulator layout) while the dK waves form dP; phase 2,
  // after a barrier: dV += P^T dO, and dK += dS^T Q with dS = P (dP - D).
  auto body = [&](auto cur_c, int sp) {
    constexpr int cur = decltype(cur_c)::value;
    const int qb0 = cur_t * BQT;
    if (sp + 1 < nsteps) load();
    // the same for both roles: the tile holds a query that sees one of the wave's keys
    const bool live = qb0 + BQT - 1 >= key0 && qb0 <= key0 + 31 + Wn - 1 && key0 < T;
    f32x16_t pd[2];  // P (dV waves) or dP (dK waves) of each 32-query half
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      if (!live || qb0 + qs * 32 + 31 < key0 || qb0 + qs * 32 > key0 + 31 + Wn - 1) continue;
      const bf16_t* rp = (dk_role ? Gs[cur] : Qs[cur]) + qs * 32 * RS;
      const bf16x8_t* kv = dk_role ? vf : kf;
      f32x16_t a = mfma32x32x16_bf16(lds_row8(rp + qro[0]), kv[0], zero16());
#pragma unroll
      for (int kk = 1; kk < NKK; ++kk) a = mfma32x32x16_bf16(lds_row8(rp + qro[kk]), kv[kk], a);
      if (!dk_role) {
        // diagonal block (queries before the key) or window edge (queries too far after)
        if (qb0 + qs * 32 < key0 + 31 || qb0 + qs * 32 + 31 - key0 >= Wn) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int q = qb0 + qs * 32 + acc_row(lane, r);
            if (q < mykey || q - mykey >= Wn) a[r] = -INFINITY;
          }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {  // registers 4g..4g+3 hold query rows qs*32 + 8g + 4hl + 0..3
          const float4 l4 = *reinterpret_cast<const float4*>(&L2s[cur][qs * 32 + 8 * g + 4 * hl]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) a[4 * g + j] = fast_exp2(fmaf(a[4 * g + j], sl2, -lv[j]));
          // bf16, as the dV waves' own MFMA takes P
          Ps[qs][kw][g][lane] = make_uint2(pack_bf2(a[4 * g], a[4 * g + 1]), pack_bf2(a[4 * g + 2], a[4 * g + 3]));
        }
      }
      pd[qs] = a;
    }
    __syncthreads();  // P published
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      if (!live || qb0 + qs * 32 + 31 < key0 || qb0 + qs * 32 > key0 + 31 + Wn - 1) continue;
      float w[16];
      if (dk_role) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint2 p2 = Ps[qs][kw][g][lane];
          const float4 d4 = *reinterpret_cast<const float4*>(&Ds[cur][qs * 32 + 8 * g + 4 * hl]);
          const float pv[4] = {bf2f((bf16_t)(p2.x & 0xffff)), bf2f((bf16_t)(p2.x >> 16)), bf2f((bf16_t)(p2.y & 0xffff)),
                               bf2f((bf16_t)(p2.y >> 16))};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) w[4 * g + j] = pv[j] * (pd[qs][4 * g + j] - dv4[j]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) w[r] = pd[qs][r];
      }
      // dV += P^T dO (dV waves) or dK += dS^T Q (dK waves), the second operand read
      // by transpose from its row-major tile
      const bf16_t* src = (dk_role ? Qs[cur] : Gs[cur]) + qs * 32 * RS;
#pragma unroll
      for (int s_ = 0; s_ < 2; ++s_) {
        const bf16x8_t wa = pack8(w + 8 * s_);
        const bf16_t* tp = src + 16 * s_ * RS;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma32x32x16_bf16(wa, lds_tr_pair(tp + tro[db][0], tp + tro[db][1]), acc[db]);
      }
    }
    if (sp + 1 < nsteps) store(cur ^ 1);
    __syncthreads();
    cur_t = cur_t + 1 == nqt ? qt0 : cur_t + 1;
  };
  for (int sp = 0; sp < nsteps; sp += 2) {
    body(std::integral_constant<int, 0>{}, sp);
    if (sp + 1 < nsteps) body(std::integral_constant<int, 1>{}, sp + 1);
  }
  const float scale = dk_role ? 1.f / sqrtf((float)HD) : 1.f;
  const long col = (long)(dk_role ? H + hk : H + Hkv + hk) * HD;
  float mo = 0.f;  // max |dv| of the lane as stored (amax_part; dK is rewritten later, by the rope backward)
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + acc_row(lane, r);
      if (key < T) {
        const float v = acc[db][r] * scale;
        dqkv[((long)b * T + key) * ld + col + db * 32 + lq] = f2bf(v);
        if (!dk_role) mo = fmaxf(mo, fabsf(v));
      }
    }
  if (amax_part) {  // one entry per wave (0 from the dK waves)
    mo = wave_max(mo);
    if (lane == 0) amax_part[((long)blockIdx.y * gridDim.x + blockIdx.x) * 8 + wave] = bf16_round(mo);
  }
}

// The dK/dV kernel above, software-pipelined: in the split form every 64-query step
// runs S -> P on the dV waves, a barrier, then dS on the dK waves (which wait for P) and
// the two accumulations, so each role idles for part of every step.  Here the dV waves
// form P of step t + 1 while the dK waves turn step t's P into dS: step t publishes
// P[t + 1] (bf16, double-buffered) and accumulates dV += P[t]^T dO[t] from the P it
// formed one step earlier (read back from LDS, as the dK waves read it), while the dK waves form dP[t], read
// P[t] and accumulate dK += dS[t]^T Q[t].  Each step needs the Q / dO tiles of t and
// t + 1, so the tiles are triple-buffered (the one for t + 2 is staged during step t
// into the buffer of t - 1; head_dim 128 by buffer-load DMA, other sizes through
// registers), and one barrier per step orders everything.
template <int HD>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_pipe_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dO,
                          const float* __restrict__ lse, const float* __restrict__ Dv, bf16_t* __restrict__ dqkv,
                          int T, int H, int Hkv, int W, float* __restrict__ amax_part) {
  constexpr int BKEY = 128, BQT = 64, TE = Tile<HD>::ELEMS, RS = Tile<HD>::RS, NDB = HD / 32, NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[3][TE];
  __shared__ __attribute__((aligned(16))) bf16_t Gs[3][TE];
  __shared__ __attribute__((aligned(16))) float L2s[3][BQT], Ds[3][BQT];
  __shared__ __attribute__((aligned(16))) uint2 Ps[2][2][4][4][64];  // [step%2][half][key wave][reg/4][lane]
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool dk_role = wave >= 4;
  const int kw = wave & 3;
  int kb, bk;
  head_major_coords(kb, bk);
  const int G = H / Hkv, b = bk / Hkv, hk = bk % Hkv;
  const long ld = (long)(H + 2 * Hkv) * HD, ldo = (long)H * HD;
  const bf16_t* Qb = qkv + (long)b * T * ld;
  const bf16_t* K = Qb + (long)(H + hk) * HD;
  const bf16_t* V = K + (long)Hkv * HD;
  const bf16_t* Gb = dO + (long)b * T * ldo;
  const long lrow = (long)b * H * T;
  const int key0 = kb * BKEY + kw * 32, mykey = key0 + lq;

  // the dV waves hold K (for S), the dK waves V (for dP)
  bf16x8_t kvf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (mykey < T) u = *reinterpret_cast<const uint4*>((dk_role ? V : K) + (long)mykey * ld + kk * 16 + hl * 8);
    kvf[kk] = __builtin_bit_cast(bf16x8_t, u);
  }
  const float sl2 = LOG2E / sqrtf((float)HD);
  f32x16_t acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = zero16();

  int qro[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qro[kk] = Tile<HD>::off(lq, kk * 16 + hl * 8);
  const int i16 = lane & 15;
  const int trr = 4 * hl + (i16 >> 2), trc = ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
  int tro[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    tro[db][0] = Tile<HD>::off(trr, db * 32 + trc);
    tro[db][1] = Tile<HD>::off(trr + 8, db * 32 + trc);
  }

  const int Wn = W > 0 ? W : T;
  const int nqt = min((T + BQT - 1) / BQT, (kb * BKEY + BKEY - 1 + Wn - 1) / BQT + 1);
  const int qt0 = (kb * BKEY) / BQT;
  const int ntile = nqt - qt0;
  const int nsteps = G * ntile;
  // step sp covers query tile qt0 + sp % ntile of query head hk G + sp / ntile
  auto step_q0 = [&](int sp) { return (qt0 + sp % ntile) * BQT; };
  auto step_h = [&](int sp) { return hk * G + sp / ntile; };
  // whether 32-query half qs of step sp holds a query that sees one of the wave's keys
  auto half_live = [&](int sp, int qs) {
    const int q0 = step_q0(sp) + qs * 32;
    return key0 < T && q0 + 31 >= key0 && q0 <= key0 + 31 + Wn - 1;
  };

  // staging of step sp's tiles into buffer buf: load (DMA straight into LDS for head_dim
  // 128, else into registers) early, store (registers -> LDS, and lse / D) late
  PairStager<HD == 128 ? 8 : HD, 512> stg;  // unused for head_dim 128
  DmaTilePair<512> dma, dmo;                 // chunk maps of Q rows (stride ld) and dO rows (stride ldo)
  if constexpr (HD == 128) {
    dma.init(ld, tid);
    dmo.init(ldo, tid);
  } else {
    stg.init(ld, ldo, tid);
  }
  float pl = 0.f, pd = 0.f;
  auto load = [&](int sp, int buf) {
    const int q0 = step_q0(sp), h = step_h(sp);
    if constexpr (HD == 128) {
      const u32x4w_t rq = rows_words(Qb + h * HD, ld, q0, T, HD), rg = rows_words(Gb + h * HD, ldo, q0, T, HD);
      const uint32_t ql = (uint32_t)(uintptr_t)Qs[buf], gl = (uint32_t)(uintptr_t)Gs[buf];
#pragma unroll
      for (int j = 0; j < DmaTilePair<512>::PER; ++j) {
        attn_dma16(rq, ql + (j * 512 + wave * 64) * 16, dma.voff[j]);
        attn_dma16(rg, gl + (j * 512 + wave * 64) * 16, dmo.voff[j]);
      }
    } else {
      stg.load(rows_rsrc(Qb + h * HD, ld, q0, T, HD), rows_rsrc(Gb + h * HD, ldo, q0, T, HD), tid);
    }
    if (tid < BQT) {
      const int q = q0 + tid;
      const long r = lrow + (long)h * T + q;
      pl = q < T ? lse[r] * LOG2E : 0.f;
      pd = q < T ? Dv[r] : 0.f;
    }
  };
  auto store = [&](int buf) {
    if constexpr (HD != 128) stg.store(Qs[buf], Gs[buf], tid);
    if (tid < BQT) {
      L2s[buf][tid] = pl;
      Ds[buf][tid] = pd;
    }
  };
  // every wave's DMA and LDS reads done, then the block barrier
  auto step_sync = [&]() {
    if constexpr (HD == 128) dma_wait_sync();
    else __syncthreads();
  };
  // dV waves: S^T = K Q^T of step sp (buffer qb) -> P, published to Ps[sp & 1] (bf16,
  // the dV MFMA's operand)
  auto form_p = [&](auto par_c, int sp, int qb) {  // par_c: sp & 1 as a compile-time constant
    constexpr int par = decltype(par_c)::value;
    const int qb0 = step_q0(sp);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      if (!half_live(sp, qs)) continue;
      const bf16_t* rp = Qs[qb] + qs * 32 * RS;
      f32x16_t a = mfma32x32x16_bf16(lds_row8(rp + qro[0]), kvf[0], zero16());
#pragma unroll
      for (int kk = 1; kk < NKK; ++kk) a = mfma32x32x16_bf16(lds_row8(rp + qro[kk]), kvf[kk], a);
      if (qb0 + qs * 32 < key0 + 31 || qb0 + qs * 32 + 31 - key0 >= Wn) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb0 + qs * 32 + acc_row(lane, r);
          if (q < mykey || q - mykey >= Wn) a[r] = -INFINITY;
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = *reinterpret_cast<const float4*>(&L2s[qb][qs * 32 + 8 * g + 4 * hl]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = fast_exp2(fmaf(a[4 * g + j], sl2, -lv[j]));
        Ps[par][qs][kw][g][lane] = make_uint2(pack_bf2(e[0], e[1]), pack_bf2(e[2], e[3]));
      }
      __builtin_amdgcn_sched_barrier(0);  // one half at a time (registers)
    }
  };

  if (nsteps > 0) {
    load(0, 0);
    store(0);
    if (nsteps > 1) {
      load(1, 1);
      store(1);
    }
  }
  step_sync();
  if (!dk_role && nsteps > 0) form_p(std::integral_constant<int, 0>{}, 0, 0);
  step_sync();  // P of step 0 published

  // one step; par_c = sp & 1 at compile time (the loop is unrolled by two)
  auto step = [&](auto par_c, int sp) {
    constexpr int par = decltype(par_c)::value;
    const int cb = sp % 3, nb = (sp + 1) % 3;
    if (sp + 2 < nsteps) load(sp + 2, (sp + 2) % 3);  // into the buffer of step sp - 1
    if (!dk_role) {
      if (sp + 1 < nsteps) form_p(std::integral_constant<int, par ^ 1>{}, sp + 1, nb);
      __builtin_amdgcn_sched_barrier(0);  // keep the two parts' registers apart
      // dV += P^T dO of step sp
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        if (!half_live(sp, qs)) continue;
        const bf16_t* tp0 = Gs[cb] + qs * 32 * RS;
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          const uint2 lo = Ps[par][qs][kw][2 * s_][lane], hi = Ps[par][qs][kw][2 * s_ + 1][lane];
          const bf16x8_t wa = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          const bf16_t* tp = tp0 + 16 * s_ * RS;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = mfma32x32x16_bf16(wa, lds_tr_pair(tp + tro[db][0], tp + tro[db][1]), acc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        if (!half_live(sp, qs)) continue;
        // dP^T = V dO^T of step sp
        const bf16_t* rp = Gs[cb] + qs * 32 * RS;
        f32x16_t a = mfma32x32x16_bf16(lds_row8(rp + qro[0]), kvf[0], zero16());
#pragma unroll
        for (int kk = 1; kk < NKK; ++kk) a = mfma32x32x16_bf16(lds_row8(rp + qro[kk]), kvf[kk], a);
        // dS = P (dP - D), then dK += dS^T Q
        float w[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint2 p2 = Ps[par][qs][kw][g][lane];
          const float4 d4 = *reinterpret_cast<const float4*>(&Ds[cb][qs * 32 + 8 * g + 4 * hl]);
          const float pv[4] = {bf2f((bf16_t)(p2.x & 0xffff)), bf2f((bf16_t)(p2.x >> 16)),
                               bf2f((bf16_t)(p2.y & 0xffff)), bf2f((bf16_t)(p2.y >> 16))};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) w[4 * g + j] = pv[j] * (a[4 * g + j] - dv4[j]);
        }
        const bf16_t* tp0 = Qs[cb] + qs * 32 * RS;
#pragma unroll
        for (int s_ = 0; s_ < 2; ++s_) {
          const bf16x8_t wa = pack8(w + 8 * s_);
          const bf16_t* tp = tp0 + 16 * s_ * RS;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = mfma32x32x16_bf16(wa, lds_tr_pair(tp + tro[db][0], tp + tro[db][1]), acc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (sp + 2 < nsteps) store((sp + 2) % 3);
    step_sync();
  };
  for (int sp = 0; sp < nsteps; sp += 2) {
    step(std::integral_constant<int, 0>{}, sp);
    if (sp + 1 < nsteps) step(std::integral_constant<int, 1>{}, sp + 1);
  }
  const float scale = dk_role ? 1.f / sqrtf((float)HD) : 1.f;
  const long col = (long)(dk_role ? H + hk : H + Hkv + hk) * HD;
  float mo = 0.f;  // max |dv| of the lane as stored (amax_part)
  // The wave's 32 x HD result goes through LDS so that it leaves as whole rows, 16 bytes
  // per lane (a lane holds one column of the accumulator, which would make 2-byte
  // stores).  Every wave is past the last step's barrier, so the Q / dO tile buffers are
  // free: the dV waves stage in Qs, the dK waves in Gs (4 x 32 padded rows each).
  constexpr int SR = HD + 8, LPR = HD / 8, RPI = 64 / LPR;
  bf16_t* sb = (dk_role ? &Gs[0][0] : &Qs[0][0]) + kw * 32 * SR;
  static_assert(4 * 32 * SR <= 3 * TE, "staging fits the tile buffers");
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = acc_row(lane, r);
      const float v = acc[db][r] * scale;
      sb[kr * SR + db * 32 + lq] = f2bf(v);
      if (!dk_role && key0 + kr < T) mo = fmaxf(mo, fabsf(v));
    }
  __syncthreads();
  const int c8 = (lane % LPR) * 8, rl = lane / LPR;
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int kr = r0 + rl, key = key0 + kr;
    if (key < T)
      *reinterpret_cast<uint4*>(dqkv + ((long)b * T + key) * ld + col + c8) =
          *reinterpret_cast<const uint4*>(sb + kr * SR + c8);
  }
  if (amax_part) {
    mo = wave_max(mo);
    if (lane == 0) amax_part[((long)blockIdx.y * gridDim.x + blockIdx.x) * 8 + wave] = bf16_round(mo);
  }
}

// dK and dV with 64 keys per wave (two 32-key blocks), one wave per SIMD: a wave forms
// S, P, dP and dS for its own keys and accumulates both dK and dV (2 x 4 accumulators
// each, 256 registers), so P never leaves registers and every Q / dO fragment read from
// LDS feeds two MFMAs.  4 waves, 256 keys per block; the 64-query Q and dO tiles arrive
// by buffer-load DMA, double-buffered, with their lse / D values.  A block serves one
// key/value head and walks the query tiles of each of its G query heads in turn.
template <int HD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bwd_dkdv_k64_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dO,
                         const float* __restrict__ lse, const float* __restrict__ Dv, bf16_t* __restrict__ dqkv,
                         int T, int H, int Hkv, int W) {
  static_assert(HD == 128, "DMA tile layout is Tile<128>");
  constexpr int NW = 4, BKEY = 64 * NW, BQT = 64, TE = Tile<HD>::ELEMS, RS = Tile<HD>::RS, NDB = HD / 32,
                NKK = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][TE];
  __shared__ __attribute__((aligned(16))) bf16_t Gs[2][TE];
  __shared__ __attribute__((aligned(16))) float L2s[2][BQT], Ds[2][BQT];
  __shared__ __attribute__((aligned(16))) bf16_t Vk[NW * TE];  // V rows of the block's keys, Tile<128> layout
  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int kb, bk;
  head_major_coords(kb, bk);
  const int G = H / Hkv, b = bk / Hkv, hk = bk % Hkv;
  const long ld = (long)(H + 2 * Hkv) * HD, ldo = (long)H * HD;
  const bf16_t* Qb = qkv + (long)b * T * ld;
  const bf16_t* K = Qb + (long)(H + hk) * HD;
  const bf16_t* V = K + (long)Hkv * HD;
  const bf16_t* Gb = dO + (long)b * T * ldo;
  const long lrow = (long)b * H * T;
  const int key0 = kb * BKEY + wave * 64;  // the wave's keys key0 + 32 kb2 + lq

  bf16x8_t kf[2][NKK];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int key = key0 + 32 * k2 + lq;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (key < T) u = *reinterpret_cast<const uint4*>(K + (long)key * ld + kk * 16 + hl * 8);
      kf[k2][kk] = __builtin_bit_cast(bf16x8_t, u);
    }
  const float sl2 = LOG2E / sqrtf((float)HD);
  f32x16_t dva[2][NDB], dka[2][NDB];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      dva[k2][i] = zero16();
      dka[k2][i] = zero16();
    }
  int qro[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qro[kk] = Tile<HD>::off(lq, kk * 16 + hl * 8);
  const int i16 = lane & 15;
  const int trr = 4 * hl + (i16 >> 2), trc = ((lane >> 4) & 1) * 16 + 4 * (i16 & 3);
  int tro[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    tro[db][0] = Tile<HD>::off(trr, db * 32 + trc);
    tro[db][1] = Tile<HD>::off(trr + 8, db * 32 + trc);
  }

  const int Wn = W > 0 ? W : T;
  const int nqt = min((T + BQT - 1) / BQT, (kb * BKEY + BKEY - 1 + Wn - 1) / BQT + 1);
  const int qt0 = (kb * BKEY) / BQT;
  const int nsteps = G * max(0, nqt - qt0);
  DmaTilePair<NW * 64> dma;  // chunk maps of Q rows (stride ld) and dO rows (stride ldo)
  DmaTilePair<NW * 64> dmo;
  dma.init(ld, tid);
  dmo.init(ldo, tid);
  // the block's V rows, 64 per wave: each wave fetches its own four 1 KB row groups per
  // 64-row tile (the chunk map of Q, whose row stride is also ld)
#pragma unroll
  for (int t4 = 0; t4 < NW; ++t4) {
    const u32x4w_t rv = rows_words(V, ld, min(kb * BKEY + 64 * t4, T - 1), T, HD);
    const uint32_t vl = (uint32_t)(uintptr_t)(Vk + t4 * TE);
    if (kb * BKEY + 64 * t4 < T) {
#pragma unroll
      for (int j = 0; j < DmaTilePair<NW * 64>::PER; ++j) attn_dma16(rv, vl + (j * NW * 64 + wave * 64) * 16, dma.voff[j]);
    }
  }
  int vko[2][NKK];  // this lane's V row (key) fragments in Vk
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) vko[k2][kk] = wave * TE + Tile<HD>::off(32 * k2 + lq, kk * 16 + hl * 8);
  float pl = 0.f, pd = 0.f;
  int ld_h = hk * G, ld_t = qt0, cur_t = qt0;
  auto load = [&](int buf) {
    const int q0 = ld_t * BQT;
    const u32x4w_t rq = rows_words(Qb + ld_h * HD, ld, q0, T, HD), rg = rows_words(Gb + ld_h * HD, ldo, q0, T, HD);
    const uint32_t ql = (uint32_t)(uintptr_t)Qs[buf], gl = (uint32_t)(uintptr_t)Gs[buf];
#pragma unroll
    for (int j = 0; j < DmaTilePair<NW * 64>::PER; ++j) {
      attn_dma16(rq, ql + (j * NW * 64 + wave * 64) * 16, dma.voff[j]);
      attn_dma16(rg, gl + (j * NW * 64 + wave * 64) * 16, dmo.voff[j]);
    }
    if (tid < BQT) {
      const int q = q0 + tid;
      const long r = lrow + (long)ld_h * T + q;
      pl = q < T ? lse[r] * LOG2E : 0.f;
      pd = q < T ? Dv[r] : 0.f;
    }
    if (++ld_t == nqt) {
      ld_t = qt0;
      ++ld_h;
    }
  };
  auto store_ld = [&](int buf) {
    if (tid < BQT) {
      L2s[buf][tid] = pl;
      Ds[buf][tid] = pd;
    }
  };
  if (nsteps > 0) {
    load(0);
    store_ld(0);
  }
  dma_wait_sync();
  auto body = [&](auto cur_c, int sp) {
    constexpr int cur = decltype(cur_c)::value;
    const int qb0 = cur_t * BQT;
    if (sp + 1 < nsteps) load(cur ^ 1);
    const bool live = qb0 + BQT - 1 >= key0 && qb0 <= key0 + 63 + Wn - 1 && key0 < T;
#pragma unroll 1
    for (int qs = 0; qs < 2; ++qs) {
      const int qh0 = qb0 + qs * 32;  // the half's queries qh0 .. qh0 + 31
      if (!live || qh0 + 31 < key0 || qh0 > key0 + 63 + Wn - 1) continue;
      const bf16_t* qp = Qs[cur] + qs * 32 * RS;
      const bf16_t* gp = Gs[cur] + qs * 32 * RS;
      f32x16_t sa[2], dp[2];  // [key block]: S and dP [query rows][key column = lane]
      {
        bf16x8_t qa = lds_row8(qp + qro[0]), ga = lds_row8(gp + qro[0]);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          sa[k2] = mfma32x32x16_bf16(qa, kf[k2][0], zero16());
          dp[k2] = mfma32x32x16_bf16(ga, lds_row8(Vk + vko[k2][0]), zero16());
        }
#pragma unroll
        for (int kk = 1; kk < NKK; ++kk) {
          qa = lds_row8(qp + qro[kk]);
          ga = lds_row8(gp + qro[kk]);
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            sa[k2] = mfma32x32x16_bf16(qa, kf[k2][kk], sa[k2]);
            dp[k2] = mfma32x32x16_bf16(ga, lds_row8(Vk + vko[k2][kk]), dp[k2]);
          }
        }
      }
      const bool edge = qh0 < key0 + 63 || qh0 + 31 - key0 >= Wn;  // diagonal or window edge
#pragma unroll
      for (int g = 0; g < 4; ++g) {  // registers 4g..4g+3 hold query rows 8g + 4hl + 0..3 of the half
        const float4 l4 = *reinterpret_cast<const float4*>(&L2s[cur][qs * 32 + 8 * g + 4 * hl]);
        const float4 d4 = *reinterpret_cast<const float4*>(&Ds[cur][qs * 32 + 8 * g + 4 * hl]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float sv = sa[k2][4 * g + j];
            if (edge) {
              const int q = qh0 + 8 * g + 4 * hl + j, key = key0 + 32 * k2 + lq;
              if (q < key || q - key >= Wn) sv = -INFINITY;
            }
            const float pr = fast_exp2(fmaf(sv, sl2, -lv[j]));
            sa[k2][4 * g + j] = pr;                                   // P
            dp[k2][4 * g + j] = pr * (dp[k2][4 * g + j] - dv4[j]);   // dS
          }
      }
      // dV += P^T dO and dK += dS^T Q: the dO / Q fragment (read by transpose) is shared
      // by both key blocks
#pragma unroll
      for (int s_ = 0; s_ < 2; ++s_) {
        bf16x8_t pa[2], da[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          float pv[8], dsv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pv[j] = sa[k2][8 * s_ + j];
            dsv[j] = dp[k2][8 * s_ + j];
          }
          pa[k2] = pack8(pv);
          da[k2] = pack8(dsv);
        }
        const bf16_t* gt = gp + 16 * s_ * RS;
        const bf16_t* qt = qp + 16 * s_ * RS;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8_t gfr = lds_tr_pair(gt + tro[db][0], gt + tro[db][1]);
          const bf16x8_t qfr = lds_tr_pair(qt + tro[db][0], qt + tro[db][1]);
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            dva[k2][db] = mfma32x32x16_bf16(pa[k2], gfr, dva[k2][db]);
            dka[k2][db] = mfma32x32x16_bf16(da[k2], qfr, dka[k2][db]);
          }
        }
      }
    }
    if (sp + 1 < nsteps) store_ld(cur ^ 1);
    dma_wait_sync();
    cur_t = cur_t + 1 == nqt ? qt0 : cur_t + 1;
  };
  for (int sp = 0; sp < nsteps; sp += 2) {
    body(std::integral_constant<int, 0>{}, sp);
    if (sp + 1 < nsteps) body(std::integral_constant<int, 1>{}, sp + 1);
  }
  const float scale = 1.f / sqrtf((float)HD);
  const long ck = (long)(H + hk) * HD, cv = (long)(H + Hkv + hk) * HD;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * k2 + acc_row(lane, r);
        if (key < T) {
          bf16_t* rowp = dqkv + ((long)b * T + key) * ld;
          rowp[ck + db * 32 + lq] = f2bf(dka[k2][db][r] * scale);
          rowp[cv + db * 32 + lq] = f2bf(dva[k2][db][r]);
        }
      }
}

// ---------------------------------------------------------------------------
// fp32 attention (plain per-row loops; used by the all-fp32 configuration)

template <int HD>
__global__ void __launch_bounds__(64) attn_fwd_f32_kernel(const float* __restrict__ qkv, float* __restrict__ out,
                                                          float* __restrict__ lse, int T, int H, int Hkv, int W) {
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= T) return;
  const long ld = (long)(H + 2 * Hkv) * HD;
  const float* Q = qkv + (long)b * T * ld + h * HD;
  const float* K = qkv + (long)b * T * ld + (long)(H + h / (H / Hkv)) * HD;
  const float* V = K + (long)Hkv * HD;
  const float sc = 1.f / sqrtf((float)HD);
  float q[HD], o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) { q[d] = Q[(long)i * ld + d]; o[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int j = W > 0 ? max(0, i - W + 1) : 0; j <= i; ++j) {
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
                                                             float* __restrict__ dqkv, int T, int H, int Hkv, int W) {
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= T) return;
  const long ld = (long)(H + 2 * Hkv) * HD, ldo = (long)H * HD;
  const float* Q = qkv + (long)b * T * ld + h * HD;
  const float* K = qkv + (long)b * T * ld + (long)(H + h / (H / Hkv)) * HD;
  const float* V = K + (long)Hkv * HD;
  const float* G = dO + (long)b * T * ldo + h * HD;
  const float sc = 1.f / sqrtf((float)HD);
  float q[HD], g[HD], dq[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) { q[d] = Q[(long)i * ld + d]; g[d] = G[(long)i * ldo + d]; dq[d] = 0.f; }
  const float L = lse[(long)bh * T + i], D = Dv[(long)bh * T + i];
  for (int j = W > 0 ? max(0, i - W + 1) : 0; j <= i; ++j) {
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

// one key per thread; the sums over queries run over the G query heads that read its
// key/value head, one head after another
template <int HD>
__global__ void __launch_bounds__(64) attn_bwd_dkdv_f32_kernel(const float* __restrict__ qkv,
                                                               const float* __restrict__ dO,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ Dv, float* __restrict__ dqkv,
                                                               int T, int H, int Hkv, int W) {
  const int bk = blockIdx.y, b = bk / Hkv, hk = bk % Hkv, G = H / Hkv;
  const int j = blockIdx.x * 64 + threadIdx.x;
  if (j >= T) return;
  const long ld = (long)(H + 2 * Hkv) * HD, ldo = (long)H * HD;
  const float* K = qkv + (long)b * T * ld + (long)(H + hk) * HD;
  const float* V = K + (long)Hkv * HD;
  const float sc = 1.f / sqrtf((float)HD);
  float k[HD], v[HD], dk[HD], dv[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    k[d] = K[(long)j * ld + d]; v[d] = V[(long)j * ld + d]; dk[d] = 0.f; dv[d] = 0.f;
  }
  const int iend = W > 0 ? min(T, j + W) : T;  // queries that see key j
  for (int g = 0; g < G; ++g) {
    const int qh = hk * G + g;
    const float* Q = qkv + (long)b * T * ld + qh * HD;
    const float* Gr = dO + (long)b * T * ldo + qh * HD;
    const long lrow = ((long)b * H + qh) * T;
    for (int i = j; i < iend; ++i) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) {
        s = fmaf(Q[(long)i * ld + d], k[d], s);
        dp = fmaf(Gr[(long)i * ldo + d], v[d], dp);
      }
      const float p = expf(s * sc - lse[lrow + i]);
      const float ds = p * (dp - Dv[lrow + i]);
#pragma unroll
      for (int d = 0; d < HD; ++d) {
        dv[d] = fmaf(p, Gr[(long)i * ldo + d], dv[d]);
        dk[d] = fmaf(ds, Q[(long)i * ld + d], dk[d]);
      }
    }
  }
  float* rowp = dqkv + ((long)b * T + j) * ld;
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    rowp[(long)(H + hk) * HD + d] = dk[d] * sc;
    rowp[(long)(H + Hkv + hk) * HD + d] = dv[d];
  }
}

// forward kernel variant for bf16, hd 128: 0 = 32 queries per wave (4 waves of 32, two
// waves per SIMD), 1 = 64 queries per wave (4 waves of 64, one wave per SIMD)
int g_attn_fwd_variant = 0;
// backward (bf16, hd 128): 0 = dQ by 4 waves of 32 queries and dK/dV by 8 waves of 32
// keys (dV and dK in different waves), 1 = dQ by 4 waves of 64 queries and dK/dV by 4
// waves of 64 keys (both in one wave)
int g_attn_bwd_variant = 0;

// returns the number of amax partials written (0: none)
template <int HD>
int fwd_dispatch(const void* qkv, void* o, float* lse, int at, int B, int T, int H, int Hkv, int W, hipStream_t st,
                 float* amax_part, long amax_cap, bool qk_normed) {
  constexpr int NW = kFwdWaves;
  if constexpr (HD == 128) {
    if (at == ACT_BF16 && g_attn_fwd_variant == 1) {
      hipLaunchKernelGGL((attn_fwd_q64_kernel<HD>), dim3((T + 255) / 256, B * H), dim3(256), 0, st,
                         (const bf16_t*)qkv, (bf16_t*)o, lse, T, H, Hkv, W);
      return 0;
    }
  }
  if (at == ACT_BF16) {
    const dim3 g((T + 32 * NW - 1) / (32 * NW), B * H);
    const long parts = (long)g.x * g.y * NW;
    if (!amax_part || parts > amax_cap) amax_part = nullptr;
    if (qk_normed)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<HD, NW, true>), g, dim3(NW * 64), 0, st, (const bf16_t*)qkv,
                         (bf16_t*)o, lse, T, H, Hkv, W, amax_part);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<HD, NW, false>), g, dim3(NW * 64), 0, st, (const bf16_t*)qkv,
                         (bf16_t*)o, lse, T, H, Hkv, W, amax_part);
    return amax_part ? (int)parts : 0;
  }
  hipLaunchKernelGGL(attn_fwd_f32_kernel<HD>, dim3((T + 63) / 64, B * H), dim3(64), 0, st, (const float*)qkv,
                     (float*)o, lse, T, H, Hkv, W);
  return 0;
}

template <int HD>
int bwd_dispatch(const void* qkv, const void* o, const void* dO, const float* lse, float* D, void* dqkv, int at,
                 int B, int T, int H, int Hkv, int W, hipStream_t st, float* amax_part, long amax_cap) {
  int parts = 0;
  if (at == ACT_BF16) {
    // the dQ kernel also writes D = rowsum(dO * O) for the dK/dV kernel
    bool done_q = false;
    if constexpr (HD == 128) {
      if (g_attn_bwd_variant == 1) {
        hipLaunchKernelGGL(attn_bwd_dq_q64_kernel<HD>, dim3((T + 255) / 256, B * H), dim3(256), 0, st,
                           (const bf16_t*)qkv, (const bf16_t*)o, (const bf16_t*)dO, lse, D, (bf16_t*)dqkv, T, H, Hkv,
                           W);
        done_q = true;
      }
    }
    if (!done_q)
      hipLaunchKernelGGL(attn_bwd_dq_kernel<HD>, dim3((T + 127) / 128, B * H), dim3(256), 0, st, (const bf16_t*)qkv,
                         (const bf16_t*)o, (const bf16_t*)dO, lse, D, (bf16_t*)dqkv, T, H, Hkv, W);
    bool done = false;
    if constexpr (HD == 128) {
      if (g_attn_bwd_variant == 1) {
        hipLaunchKernelGGL(attn_bwd_dkdv_k64_kernel<HD>, dim3((T + 255) / 256, B * Hkv), dim3(256), 0, st,
                           (const bf16_t*)qkv, (const bf16_t*)dO, lse, D, (bf16_t*)dqkv, T, H, Hkv, W);
        done = true;
      }
    }
    if (!done) {
      const dim3 g((T + 127) / 128, B * Hkv);
      const long np = (long)g.x * g.y * 8;
      if (!amax_part || np > amax_cap) amax_part = nullptr;
      if (g_attn_bwd_variant == 2)
        hipLaunchKernelGGL(attn_bwd_dkdv_split_kernel<HD>, g, dim3(512), 0, st, (const bf16_t*)qkv,
                           (const bf16_t*)dO, lse, D, (bf16_t*)dqkv, T, H, Hkv, W, amax_part);
      else
        hipLaunchKernelGGL(attn_bwd_dkdv_pipe_kernel<HD>, g, dim3(512), 0, st, (const bf16_t*)qkv,
                           (const bf16_t*)dO, lse, D, (bf16_t*)dqkv, T, H, Hkv, W, amax_part);
      parts = amax_part ? (int)np : 0;
    }
  } else {
    hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<HD>, dim3((T + 63) / 64, B * H), dim3(64), 0, st, (const float*)qkv,
                       (const float*)dO, lse, D, (float*)dqkv, T, H, Hkv, W);
    hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<HD>, dim3((T + 63) / 64, B * Hkv), dim3(64), 0, st,
                       (const float*)qkv, (const float*)dO, lse, D, (float*)dqkv, T, H, Hkv, W);
  }
  return parts;
}

}  // namespace

void set_attn_fwd_variant(int v) { g_attn_fwd_variant = v; }
void set_attn_bwd_variant(int v) { g_attn_bwd_variant = v; }

// Hkv must divide H (the callers validate it)
int launch_attn_fwd(const void* qkv, void* o, float* lse, int at, int B, int T, int H, int Hkv, int hd, int window,
                    hipStream_t st, float* amax_part, long amax_cap, bool qk_normed) {
  if (B * T * H == 0) return 0;
  if (hd == 128) return fwd_dispatch<128>(qkv, o, lse, at, B, T, H, Hkv, window, st, amax_part, amax_cap, qk_normed);
  if (hd == 64) return fwd_dispatch<64>(qkv, o, lse, at, B, T, H, Hkv, window, st, amax_part, amax_cap, qk_normed);
  if (hd == 32) return fwd_dispatch<32>(qkv, o, lse, at, B, T, H, Hkv, window, st, amax_part, amax_cap, qk_normed);
  return 0;
}

int launch_attn_bwd(const void* qkv, const void* o, const void* dO, const float* lse, float* D, void* dqkv, int at,
                    int B, int T, int H, int Hkv, int hd, int window, hipStream_t st, float* amax_part,
                    long amax_cap) {
  if (B * T * H == 0) return 0;
  const int N = B * T;
  if (at != ACT_BF16)  // the bf16 dQ kernel forms D itself
    hipLaunchKernelGGL(attn_bwd_prep_kernel<float>, dim3((N * H + 3) / 4), dim3(256), 0, st, (const float*)o,
                       (const float*)dO, D, N, T, H, hd);
  if (hd == 128) return bwd_dispatch<128>(qkv, o, dO, lse, D, dqkv, at, B, T, H, Hkv, window, st, amax_part, amax_cap);
  if (hd == 64) return bwd_dispatch<64>(qkv, o, dO, lse, D, dqkv, at, B, T, H, Hkv, window, st, amax_part, amax_cap);
  if (hd == 32) return bwd_dispatch<32>(qkv, o, dO, lse, D, dqkv, at, B, T, H, Hkv, window, st, amax_part, amax_cap);
  return 0;
}
