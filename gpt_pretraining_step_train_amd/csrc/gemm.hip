// GEMMs of the GPT step on gfx950.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 with LDS double buffering.  Both operands
// are staged in LDS as [rows][k] (k contiguous, rows padded by 16 bytes).  An
// operand whose reduction index is its slow (row) index in memory is transposed
// on the way in: each thread loads an 8x8 block (8 k-rows of 16 bytes), swaps it
// in registers and stores 8 k-contiguous rows.  This serves the forward
// (X W^T), data-gradient (dY W) and weight-gradient (dY^T X) products and the
// Newton-Schulz products with one kernel.
//
// fp32 path: a plain LDS-tiled SIMT kernel (the all-fp32 configuration).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int BK = 64;        // bf16 elements of k per LDS stage
constexpr int LDSS = BK + 8;  // LDS row stride in elements (16-byte pad)

template <int R, bool KMAJ, int NT>
struct TileLoader {
  static constexpr int NUNIT = KMAJ ? R * (BK / 8) : (R / 8) * (BK / 8);
  static constexpr int UPT = (NUNIT + NT - 1) / NT;  // units per thread
  static constexpr int NREG = KMAJ ? UPT : UPT * 8;
  uint4 regs[NREG];

  // element (row, k) lives at base[row*ld + k] (KMAJ) or base[k*ld + row]
  __device__ inline void load(const bf16_t* __restrict__ base, long ld, int row0, int rows, int k0, int kend,
                              int tid) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (KMAJ) {
        const int r = u >> 3, kc = u & 7;
        const int grow = row0 + r, gk = k0 + kc * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (u < NUNIT && grow < rows && gk < kend) v = *reinterpret_cast<const uint4*>(base + (long)grow * ld + gk);
        regs[i] = v;
      } else {
        const int kb = u & 7, rb = u >> 3;
        const int grow = row0 + rb * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gk = k0 + kb * 8 + j;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (u < NUNIT && grow < rows && gk < kend) v = *reinterpret_cast<const uint4*>(base + (long)gk * ld + grow);
          regs[i * 8 + j] = v;
        }
      }
    }
  }

  __device__ inline void store(bf16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (u >= NUNIT) continue;
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
__device__ inline void tile_coords(int lin, int tilesM, int tilesN, int& tm, int& tn) {
  const int total = tilesM * tilesN;
  int id = lin;
  if ((total & 7) == 0) id = (lin & 7) * (total >> 3) + (lin >> 3);
  constexpr int G = 8;
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
      store_act<OutT>(reinterpret_cast<OutT*>(p.outA) + o, v);
      if (p.outA_lo) store_act<OutT>(reinterpret_cast<OutT*>(p.outA_lo) + o, v - load_act<OutT>(reinterpret_cast<OutT*>(p.outA) + o));
    }
  } else if (p.epi == EPI_RELU2) {
    const long o = bz * p.strideOA + (long)row * p.ldoa + col;
    store_act<OutT>(reinterpret_cast<OutT*>(p.outA) + o, v);
    const float r = fmaxf(v, 0.f);
    store_act<OutT>(reinterpret_cast<OutT*>(p.out2) + o, r * r);
  } else {  // EPI_DRELU2
    const long o = bz * p.strideOA + (long)row * p.ldoa + col;
    const float u = load_act<OutT>(reinterpret_cast<const OutT*>(p.aux) + o);
    store_act<OutT>(reinterpret_cast<OutT*>(p.outA) + o, v * 2.f * fmaxf(u, 0.f));
  }
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM>
__global__ void __launch_bounds__(WM* WN * 64) gemm_bf16_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDSS];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDSS];

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
  const int nseg = p.split ? 3 : 1;                                 // hi*hi, hi*lo, lo*hi
  const int nk = nks * nseg;

  const bf16_t* Ah = reinterpret_cast<const bf16_t*>(p.A) + bz * p.strideA;
  const bf16_t* Bh = reinterpret_cast<const bf16_t*>(p.B) + bz * p.strideB;
  const bf16_t* Al = p.split ? reinterpret_cast<const bf16_t*>(p.A_lo) + bz * p.strideA : Ah;
  const bf16_t* Bl = p.split ? reinterpret_cast<const bf16_t*>(p.B_lo) + bz * p.strideB : Bh;
  // k tile t: segment t / nks selects the operand planes, (t % nks) the k offset
  auto seg_a = [&](int t) { return t / nks == 2 ? Al : Ah; };
  auto seg_b = [&](int t) { return t / nks == 1 ? Bl : Bh; };
  auto seg_k = [&](int t) { return kbeg + (t % nks) * BK; };

  TileLoader<BM, AK, NT> la;
  TileLoader<BN, BKM, NT> lb;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    la.load(seg_a(0), p.lda, m0, p.M, seg_k(0), kend, tid);
    lb.load(seg_b(0), p.ldb, n0, p.N, seg_k(0), kend, tid);
    la.store(As[0], tid);
    lb.store(Bs[0], tid);
  }
  __syncthreads();

  const int lr = lane & 31, lk = (lane >> 5) * 8;
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) {
      la.load(seg_a(it + 1), p.lda, m0, p.M, seg_k(it + 1), kend, tid);
      lb.load(seg_b(it + 1), p.ldb, n0, p.N, seg_k(it + 1), kend, tid);
    }
    const bf16_t* as = As[cur] + (wm * TM + lr) * LDSS + lk;
    const bf16_t* bs = Bs[cur] + (wn * TN + lr) * LDSS + lk;
    // fragments double-buffered across the 16-wide k steps so LDS reads overlap MFMAs
    bf16x8_t af[2][FM], bfv[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = *reinterpret_cast<const bf16x8_t*>(as + i * 32 * LDSS);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfv[0][j] = *reinterpret_cast<const bf16x8_t*>(bs + j * 32 * LDSS);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[c ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(as + i * 32 * LDSS + (kk + 1) * 16);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfv[c ^ 1][j] = *reinterpret_cast<const bf16x8_t*>(bs + j * 32 * LDSS + (kk + 1) * 16);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the next step's LDS reads ahead of these MFMAs
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16_bf16(af[c][i], bfv[c][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (it + 1 < nk) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // epilogue through LDS, one 32-row block of every wave at a time: the accumulator
  // fragments go to LDS with constant register indices, then each wave reads its
  // 32 x TN block back row by row (two adjacent columns per lane) for coalesced stores
  constexpr int CS = TN + 4;  // fp32 row stride of the staging block
  static_assert(WM * WN * 32 * CS * 4 <= 2 * BM * LDSS * 2, "staging block must fit in As");
  static_assert(TN == 64 || TN % 128 == 0, "epilogue column mapping");
  float* stage = reinterpret_cast<float*>(&As[0][0]) + wave * 32 * CS;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) stage[acc_row(lane, r) * CS + j * 32 + lr] = acc[i][j][r];
    __syncthreads();
    const int row0 = m0 + wm * TM + i * 32;
    for (int rr = 0; rr < 32; ++rr) {
      const int row = row0 + rr;
      if (row >= p.M) break;
#pragma unroll
      for (int cc = 0; cc < TN / 128; ++cc) {
        const int lc = cc * 128 + lane * 2;
        const int col = n0 + wn * TN + lc;
        const float v0 = stage[rr * CS + lc], v1 = stage[rr * CS + lc + 1];
        if (p.splits > 1) {
          float* w = p.ws + ((long)blockIdx.y * p.M + row) * p.N + col;
          if (col < p.N) w[0] = v0;
          if (col + 1 < p.N) w[1] = v1;
        } else {
          if (col < p.N) epilogue_elem<bf16_t>(p, bz, row, col, v0);
          if (col + 1 < p.N) epilogue_elem<bf16_t>(p, bz, row, col + 1, v1);
        }
      }
      if (TN % 128) {  // TN = 64: lanes 0..31 cover the row
        const int lc = lane * 2;
        const int col = n0 + wn * TN + lc;
        if (lc < TN) {
          const float v0 = stage[rr * CS + lc], v1 = stage[rr * CS + lc + 1];
          if (p.splits > 1) {
            float* w = p.ws + ((long)blockIdx.y * p.M + row) * p.N + col;
            if (col < p.N) w[0] = v0;
            if (col + 1 < p.N) w[1] = v1;
          } else {
            if (col < p.N) epilogue_elem<bf16_t>(p, bz, row, col, v0);
            if (col + 1 < p.N) epilogue_elem<bf16_t>(p, bz, row, col + 1, v1);
          }
        }
      }
    }
    __syncthreads();
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

template <int BM, int BN, int WM, int WN>
void launch_bf16(const GemmArgs& p, hipStream_t st) {
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  dim3 grid(tiles, p.batch * p.splits), block(WM * WN * 64);
  if (p.a_kmaj && p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, true, true>), grid, block, 0, st, p);
  else if (p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, true, false>), grid, block, 0, st, p);
  else if (!p.a_kmaj && !p.b_kmaj)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, false, false>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, false, true>), grid, block, 0, st, p);
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

int pick_tile(const GemmArgs& p) {
  if (p.tile) return p.tile;
  const long big = (long)((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
  return big >= 128 ? 1 : 2;
}

}  // namespace

int gemm_auto_splits(const GemmArgs& p) {
  if (p.epi != EPI_LINEAR) return 1;
  int tm, tn;
  if (p.dtype == ACT_F32) {
    tm = 64; tn = 64;
  } else if (pick_tile(p) == 1) {
    tm = 256; tn = 256;
  } else {
    tm = 128; tn = 128;
  }
  const long tiles = (long)((p.M + tm - 1) / tm) * ((p.N + tn - 1) / tn) * p.batch;
  const int kstep = p.dtype == ACT_F32 ? 16 : BK;
  int s = 1;
  // aim for >= 512 workgroups while every split keeps >= 1024 of K
  while (tiles * s < 512 && (long)p.K / (s * 2) >= 1024 && s < 32) s *= 2;
  (void)kstep;
  return s;
}

// one name per kernel instantiation: tile and operand layouts (N = reduction index
// contiguous, T = transposed on load), as "gemm_bf16_kernel<256,256,NT>"
const char* gemm_kernel_name(const GemmArgs& p) {
  static const char* names[3][4] = {
      {"gemm_f32_kernel<NT>", "gemm_f32_kernel<NN>", "gemm_f32_kernel<TN>", "gemm_f32_kernel<TT>"},
      {"gemm_bf16_kernel<256,256,NT>", "gemm_bf16_kernel<256,256,NN>", "gemm_bf16_kernel<256,256,TN>",
       "gemm_bf16_kernel<256,256,TT>"},
      {"gemm_bf16_kernel<128,128,NT>", "gemm_bf16_kernel<128,128,NN>", "gemm_bf16_kernel<128,128,TN>",
       "gemm_bf16_kernel<128,128,TT>"}};
  const int lay = p.a_kmaj ? (p.b_kmaj ? 0 : 1) : (p.b_kmaj ? 3 : 2);
  const int t = p.dtype == ACT_F32 ? 0 : pick_tile(p);
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
  if (p.dtype == ACT_BF16) {
    // 16-byte vector loads: k (K-major operands) or rows (transposed operands) in multiples of 8
    if (p.K % 8) return 2;
    if (!p.a_kmaj && (p.M % 8 || p.lda % 8)) return 2;
    if (!p.b_kmaj && (p.N % 8 || p.ldb % 8)) return 2;
    if ((p.a_kmaj && p.lda % 8) || (p.b_kmaj && p.ldb % 8)) return 2;
    if (pick_tile(p) == 1)
      launch_bf16<256, 256, 2, 2>(p, st);
    else
      launch_bf16<128, 128, 2, 2>(p, st);
  } else {
    launch_f32(p, st);
  }
  if (p.splits > 1) {
    const long total = (long)p.M * p.N * p.batch;
    const int blocks = (int)std::min<long>((total + 255) / 256, 65536);
    if (p.dtype == ACT_BF16)
      hipLaunchKernelGGL(splitk_reduce_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3(blocks), dim3(256), 0, st, p);
  }
  return 0;
}
