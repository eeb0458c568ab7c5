// Internal launcher interface of the HIP kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ACT_F16 (fp16 operands and act outputs) is used by the Newton-Schulz products only
enum ActType { ACT_F32 = 0, ACT_BF16 = 1, ACT_F16 = 2 };

enum GemmEpi {
  EPI_LINEAR = 0,  // v = alpha*acc + beta*Cin -> outF (fp32) and/or outA (act type)
  EPI_RELU2 = 1,   // g = max(alpha*acc, 0)^2 -> out2 (ld / stride of outA); the pre-activation is not kept
  EPI_DRELU2 = 2,  // v = alpha*acc * 2*sqrt(max(aux,0)) -> outA, aux = g = max(u,0)^2 (so the root is max(u,0))
};

// C[M,N] = sum_k A(m,k) B(n,k), batched over `batch` with element strides.
//   a_kmaj: A(m,k) = A[m*lda + k]  else A(m,k) = A[k*lda + m]
//   b_kmaj: B(n,k) = B[n*ldb + k]  else B(n,k) = B[k*ldb + n]
struct GemmArgs {
  int M = 0, N = 0, K = 0, batch = 1;
  const void* A = nullptr; long lda = 0, strideA = 0;
  const void* B = nullptr; long ldb = 0, strideB = 0;
  bool a_kmaj = true, b_kmaj = true;
  int dtype = ACT_BF16;           // operand type (and outA type); ACT_F16: 256x256 kernel, no split
  int epi = EPI_LINEAR;
  float alpha = 1.f, beta = 0.f;
  const float* Cin = nullptr; long ldcin = 0, strideCin = 0;
  const void* CinA = nullptr;     // fp16 NT / NN kernels only: Cin as fp16 instead (Cin null; same ld/stride; M, N and
                                  // every leading dimension / stride multiples of 4, else launch_gemm fails)
  float* outF = nullptr; long ldo = 0, strideO = 0;
  void* outA = nullptr; long ldoa = 0, strideOA = 0;
  void* out2 = nullptr;           // EPI_RELU2 output (ld / stride: ldoa, strideOA)
  const void* aux = nullptr;      // EPI_DRELU2 input (same ld/stride as outA)
  int splits = 1;                 // split-K factor; >1 needs ws
  float* ws = nullptr; size_t ws_bytes = 0;
  int tile = 0;                   // 0 = auto, 1 = 256x256, 2 = 128x128
  // split: A and B come as two bf16 planes each, hi (A, B) and lo (A_lo, B_lo = the
  // rounding residual of fp32 values); the product runs as three K segments
  // hi*hi + hi*lo + lo*hi on bf16 MFMA (~16 significant bits per operand)
  bool split = false;
  const void* A_lo = nullptr;
  const void* B_lo = nullptr;
  void* outA_lo = nullptr;        // optional lo plane of outA (v - bf16(v)), same ld/stride
  // fp8: A and B are e4m3 bytes (both with the reduction index contiguous); the
  // accumulator is multiplied by (*dq_a) * (*dq_b) (device scalars) before the epilogue
  bool fp8 = false;
  const float* dq_a = nullptr;
  const float* dq_b = nullptr;
  // sym: the caller guarantees C is symmetric (M == N, A and B giving C[m][n] = C[n][m]);
  // the 256x256 kernel then computes the upper tiles only and mirrors them (the
  // epilogue of element (n, m) runs with its own Cin/aux entries).  A hint: kernels
  // that do not use it compute every tile.
  bool sym = false;
  // amax_part (or null): per-wave maxima of |stored output| of an EPI_RELU2 / EPI_DRELU2
  // launch, gemm_amax_parts(args) entries (launch_gemm fails where that is 0)
  float* amax_part = nullptr;
};

// returns 0 on success, else an error code (argument/shape problems)
int launch_gemm(const GemmArgs& p, hipStream_t st);
// split-K factor the launcher would use for these arguments (for workspace sizing)
int gemm_auto_splits(const GemmArgs& p);
// number of amax_part entries this launch writes when given the buffer (0: not supported)
int gemm_amax_parts(const GemmArgs& p);
const char* gemm_kernel_name(const GemmArgs& p);

// ---------------------------------------------------------------------------
// elementwise / reduction kernels
void launch_embed_gather(const int32_t* tok, const float* E, float* h, int N, int d, int V,
                         int* err_flag, hipStream_t st);
// Producers of tensors an fp8 step quantises take amax_part (scratch of amax_cap floats, or
// null) and return how many entries they wrote there (0: none, the buffer being null, too
// small or the path unsupported): per-wave maxima of |value| as stored, whose maximum
// (launch_amax_fold) is the tensor's amax without a pass of its own.
int launch_rmsnorm_fwd(const float* x, void* y, int ytype, float* rstd, int N, int d, float eps,
                       hipStream_t st, float* amax_part = nullptr, long amax_cap = 0);
// y (or null): the forward's stored output x * rstd (act type), read instead of x
int launch_rmsnorm_bwd(const float* dy, const float* x, const float* rstd, const float* dres,
                       float* dx, void* dx_act, int act_type, int N, int d, float eps, hipStream_t st,
                       float* amax_part = nullptr, long amax_cap = 0,  // partials of dx_act
                       const void* y = nullptr);
// extras (per-layer residual scaling, smear, backout).  A coefficient is mul * (*p), or mul
// when p is null; p points into the parameter vector on the device.
// m = a x + b z (fp32, z null: b = 0), y = m / rms(m), rstd as for launch_rmsnorm_fwd
void launch_mix_rmsnorm_fwd(const float* x, const float* z, const float* pa, float ma, const float* pb, float mb,
                            float* m, void* y, int yt, float* rstd, int N, int d, float eps, hipStream_t st);
// g = dres + (norm backward of m); out = a g + add1 + add2 (+ b g if b_to_out) with its act copy;
// acc += b g otherwise (if acc); dots_a[row] = sa g.xa, dots_b[row] = sb g.xb (if xa / xb)
void launch_rmsnorm_mix_bwd(const float* dy, const float* m, const float* rstd, const float* dres, const float* pa,
                            float ma, const float* pb, float mb, bool b_to_out, const float* add1, const float* add2,
                            float* acc, const float* xa, float* dots_a, float sa, const float* xb, float* dots_b,
                            float sb, float* out, void* outa, int at, int N, int d, hipStream_t st);
// x[n] = e[n] + ls sigmoid(ws . e[n,:24]) e[n-1] within sequences of T rows (d >= 24)
void launch_smear_fwd(const float* e, const float* pls, const float* ws, float* x, int N, int T, int d,
                      hipStream_t st);
// de from dx; part_ls [N] and part_ws [24][N] hold the per-row terms of dls and dws
void launch_smear_bwd(const float* dx, const float* e, const float* pls, const float* ws, float* de, float* part_ls,
                      float* part_ws, int N, int T, int d, hipStream_t st);
// dS[j] (+)= sum_n part[j][n] for j < 2L + 26 (entries of extras not in mask: 0)
void launch_extras_reduce(const float* part, int N, int L, int mask, float* dS, bool accumulate, hipStream_t st);
void launch_extras_init(float* S, int L, hipStream_t st);
// value embeddings (qkv rows [q | k | v] as for the attention launchers; a is the block's
// normed input [N][d]; ve the layer's table [V][Hkv hd]; wg its gate weights [Hkv][24]):
// v += 3 sigmoid(wg . a[:24]) ve[tok] per head, the gate values to vg [N][Hkv]
void launch_ve_fwd(void* qkv, int at, const void* a, const int32_t* tok, const float* ve, const float* wg,
                   float* vg, int N, int V, int H, int Hkv, int hd, int d, hipStream_t st);
// dve [N][Hkv hd] = g dv, dz [N][Hkv], part [N][Hkv*24] (rows of d wg) from dqkv's v part
void launch_ve_bwd(const void* dqkv, int at, const void* a, const int32_t* tok, const float* ve, const float* vg,
                   float* dve, float* dz, float* part, int N, int V, int H, int Hkv, int hd, int d, hipStream_t st);
// da[:, :24] += dz wg
void launch_ve_da(float* da, const float* dz, const float* wg, int N, int Hkv, int d, hipStream_t st);
// out[j] (+)= sum_n part[n][j] for j < R, fixed order (fp64); ws holds colsum_ws_bytes(R)
size_t colsum_ws_bytes(int R);
void launch_colsum(const float* part, int N, int R, void* ws, float* out, bool accumulate, hipStream_t st);
void launch_rope_table(float* cs, int T, int hd, float base, hipStream_t st);
// qkv rows are [H q heads | Hkv k heads | Hkv v heads] x hd; rstd_q is [B*T][H], rstd_k [B*T][Hkv]
void launch_rope_qknorm_fwd(void* qkv, int act_type, const float* cs, float* rstd_q, float* rstd_k,
                            int B, int T, int H, int Hkv, int hd, float eps, hipStream_t st);
int launch_rope_qknorm_bwd(void* dqkv, const void* qkv, int act_type, const float* cs,
                           const float* rstd_q, const float* rstd_k, int B, int T, int H, int Hkv, int hd,
                           hipStream_t st, float* amax_part = nullptr, long amax_cap = 0);  // partials of dq, dk
int launch_cross_entropy(const float* logits, const int32_t* targets, void* dlogits, int act_type,
                         float* row_loss, int32_t* argmax, int N, int V, float inv_n, int* err_flag,
                         hipStream_t st, float* dlogits_part = nullptr, long part_cap = 0);
void launch_sum_rows(const float* x, int n, double* out, hipStream_t st);
// deterministic embedding backward: dE[v] = sum over positions n with tok[n]==v of dh[n], summed in
// increasing n (accumulate: added to dE's previous value).  ws must hold embed_ws_bytes(N, V, d).
size_t embed_ws_bytes(int N, int V, int d);
void launch_embed_scatter(const int32_t* tok, const float* dh, float* dE, int N, int V, int d,
                          void* ws, int32_t* sorted_out, hipStream_t st, bool accumulate = false);
// the same in two parts: the sort of the ids (once per token batch), then any number of
// scatters of rows of any width <= d (the ws of embed_ws_bytes(N, V, d) keeps the sort)
void launch_embed_sort(const int32_t* tok, int N, int V, void* ws, hipStream_t st);
void launch_embed_scatter_sorted(const int32_t* tok, const float* dh, float* dE, int N, int V, int d, void* ws,
                                 hipStream_t st, bool accumulate);
void launch_cast_f32_to_act(const float* x, void* y, int act_type, size_t n, hipStream_t st);
void launch_fill_normal(float* w, size_t n, uint64_t seed, uint64_t stream_id, float stddev,
                        hipStream_t st);
void launch_zero(void* p, size_t bytes, hipStream_t st);

// Muon pieces
// AdamW on n fp32 weights with fp32 moments (rbc1/rbc2: reciprocal bias corrections);
// w_act (optional, act_type) receives the updated weights
void launch_adamw(float* w, const float* g, float* m, float* v, void* w_act, int act_type, size_t n, float lr,
                  float b1, float b2, float eps, float wd, float rbc1, float rbc2, hipStream_t st);
// m = mu m + g on every listed matrix (matrix i occupies [offs[i], offs[i]+sizes[i]), offsets
// multiples of 4) and the per-matrix sums of squares of the new m, in one pass
// one matrix of the batched Muon elementwise passes (normalise, apply): element offsets of
// its source (momentum / fp32 master) and destination (NS workspace) in their regions and
// of its act-typed weight copy, its size (a multiple of 4), its sum-of-squares index, its
// columns and the first of its NorMuon row scales
struct MuonVecJob {
  long src, dst, wact, n;
  long srow;
  int mat, cols;
};
// X0 = src / (sqrt(sumsq[mat]) + eps) for every job (no transposes): xf fp32, xa (and xlo)
// act typed (at: ACT_BF16 or ACT_F16)
void launch_ns_normalize_batched(const float* src, const double* sumsq, float eps, const MuonVecJob* jobs, int njobs,
                                 float* xf, void* xa, void* xlo, int at, hipStream_t st);
// W -= lr (s[row]) X for every job (no transposes), act copy refreshed when wa
void launch_muon_apply_batched(float* w, void* wa, int at, const float* x, float lr, const MuonVecJob* jobs,
                               int njobs, const float* row_scale, hipStream_t st);
void launch_momentum_sumsq(float* m, const float* g, float mu, const long* offs, const long* sizes, int nmat,
                           double* partial, int parts, double* out, hipStream_t st);
// X = src / (norm + eps) written (optionally transposed) into fp32 and act copies
void launch_ns_normalize(const float* src, const double* sumsq, int mat, float eps, int rows, int cols,
                         bool transpose, float* xf, void* xa, void* xa_lo, int act_type, hipStream_t st);
// W -= lr * s[r] * X, s an optional per-row scale (NorMuon)
void launch_muon_apply(float* w, void* w_act, int act_type, const float* x, float lr, int rows,
                       int cols, bool transposed, hipStream_t st, const float* row_scale = nullptr);
// NorMuon: mean square of each output row of X (stored [cols][rows] when transposed), then
// per matrix (rows roff[m] .. roff[m+1] of the stacked vectors) V = b2 V + (1-b2) vmean
// and the row scales that divide by sqrt(V) and keep the update's Frobenius norm
// (ws: normuon_ws_bytes(rows) bytes, used for transposed stores)
size_t normuon_ws_bytes(int max_rows);
void launch_normuon_rowstats(const float* x, int rows, int cols, bool transposed, float* vmean, void* ws,
                             hipStream_t st);
void launch_normuon_scale(const float* vmean, float* V, const long* roff, int nmat, float beta2, float* scale,
                          hipStream_t st);

// fp8 (OCP e4m3fn) per-tensor current scaling.  amax slot: one uint32 holding the bits of
// max|x| (non-negative floats order as integers); must be zeroed before launch_amax.
// partials (kAmaxParts floats of scratch, or null): the two-stage form, one atomic in all.
constexpr int kAmaxParts = 1024;
void launch_amax(const void* x, int in_type, long rows, long cols, long ld, unsigned* amax_bits, hipStream_t st,
                 float* partials = nullptr);
// the slot (zeroed) receives the maximum of n producer partials
void launch_amax_fold(const float* partials, int n, unsigned* amax_bits, hipStream_t st);
// q[r][c] = e4m3(x[r][c] * s) and (optionally) qt[c][r] = the same byte, s = 448/amax
// (1 when amax = 0); inv_scale[0] = 1/s.  in_type: ACT_F32 or ACT_BF16.
void launch_quant_e4m3(const void* x, int in_type, int rows, int cols, long ld, const unsigned* amax_bits,
                       uint8_t* q, long ldq, uint8_t* qt, long ldqt, float* inv_scale, hipStream_t st);

// attention (window > 0: query i sees keys i - window < j <= i; 0: all j <= i).  qkv rows are
// [H q heads | Hkv k heads | Hkv v heads] x hd; query head h reads key/value head h / (H / Hkv).
// process-wide choice of the bf16 hd-128 attention kernels (see gptk_attn_variant)
void set_attn_fwd_variant(int v);
void set_attn_bwd_variant(int v);
void set_ce_variant(int v);
// qk_normed: every q and k row is RMS-normalised per head (as the step's QK-norm leaves
// them), which bounds the scores, so the forward skips its running maximum
int launch_attn_fwd(const void* qkv, void* o, float* lse, int act_type, int B, int T, int H, int Hkv, int hd,
                    int window, hipStream_t st, float* amax_part = nullptr, long amax_cap = 0,  // partials of o
                    bool qk_normed = false);
int launch_attn_bwd(const void* qkv, const void* o, const void* dO, const float* lse, float* Dbuf,
                    void* dqkv, int act_type, int B, int T, int H, int Hkv, int hd, int window, hipStream_t st,
                    float* amax_part = nullptr, long amax_cap = 0);  // partials of dv
