/* gpt.h -- C ABI of a single-GPU GPT pretraining step on MI355X (gfx950).
 *
 * One training step on one GPU's micro-batch of the nanochat-style GPT that the
 * dev.to article "ChatGPT'nizi 50 Dolara Nasil Egitirsiniz?" (and its Arabic
 * translation) describes in "nanochat Nasil Calisir? / 1. GPT Modeli":
 * token-embedding lookup (untied from the LM head), pre-norm decoder blocks with
 * RoPE and QK-normalised causal multi-head attention and a ReLU^2 MLP, a final
 * norm, the LM head and the softmax cross-entropy over the 32,768-token
 * vocabulary; forward and backward; then the Muon update of section
 * "2. Muon Optimize Edici" (momentum, then Newton-Schulz orthogonalisation of
 * every 2-D block matrix with the Polar Express coefficient table).
 *
 * Conventions
 *  - Every pointer named d_* is device memory; h_* is host memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *    work is stream-ordered; only gpt_step, gpt_grads, gpt_get_* synchronise.
 *  - Matrices are row-major [rows][cols] float32 in the [out][in] convention of
 *    the article's Linear layer (F.linear with no bias).
 *  - Tensor ids (gpt_tensor_shape): 0 = E [V][d]; for layer l, ids 1+6l .. 6+6l
 *    are Wq [d][d], Wk [dkv][d], Wv [dkv][d], Wo [d][d], W1 [F][d], W2 [d][F]
 *    (dkv = n_kv_head * head_dim); id 1+6L = U [V][d] (LM head).  With any
 *    extras switched on, id 2+6L = S [1][2L+26]: the L residual scales, the L x0
 *    scales, the smear scale, the backout scale and the 24 smear-gate weights.
 *    With value embeddings, ids 3+6L .. 2+7L = VE_l [V][dkv] (one table per
 *    layer) and id 3+7L = G [L*Hkv][24] (gate weights, layer-major).
 *    Count = 2 + 6L (+1 with extras, +L+1 with value embeddings).
 *  - Ownership: the caller owns the arena, the token buffers and the stream and
 *    keeps them alive until the stream's work completes.  The library never
 *    allocates device memory; gpt_free releases host bookkeeping only.
 *  - Errors: functions return a gpt_status; gpt_step returns NaN on error and
 *    records the status (gpt_last_status).  No C++ exception crosses the ABI.
 *  - A model is used by one host thread at a time.
 */
#ifndef GPT_H
#define GPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT_OK = 0,
  GPT_ERR_ARG = 1,          /* bad argument, arena too small, id out of range */
  GPT_ERR_SHAPE = 2,        /* cfg inconsistent, or differs from the model's */
  GPT_ERR_TOKEN_RANGE = 3,  /* a token or target id outside [0, vocab) */
  GPT_ERR_NONFINITE = 4,    /* a non-finite logit */
  GPT_ERR_HIP = 5,          /* a HIP runtime call failed */
  GPT_ERR_UNSUPPORTED = 6   /* a precision/shape this build does not support */
} gpt_status;

typedef enum { GPT_FP32 = 0, GPT_BF16 = 1, GPT_FP8 = 2 } gpt_precision;

/* Model + step configuration (precision GPT_FP8: the Linear GEMMs -- QKV, output
 * projection, MLP and LM head, forward and both backward products -- take e4m3
 * operands with per-tensor current scaling and fp32 accumulation; everything else as
 * GPT_BF16).  depth is the one dial of the article's
 * "Felsefe" section: gpt_cfg_from_depth derives the rest. */
typedef struct gpt_cfg {
  int32_t depth;      /* L: decoder blocks */
  int32_t d_model;    /* d: residual width (multiple of 8) */
  int32_t n_head;     /* H: attention heads (n_head * head_dim == d_model) */
  int32_t head_dim;   /* hd: 32, 64 or 128 */
  int32_t d_ff;       /* F: MLP hidden width */
  int32_t vocab;      /* V */
  int32_t seq_len;    /* T */
  int32_t batch;      /* B: sequences in the micro-batch */
  int32_t precision;  /* gpt_precision: FP32 = all fp32; BF16 = fp32 master weights and
                         residual stream, bf16 GEMM/attention operands, fp32 accumulate */
  float init_std;     /* 0.02; Wo and W2 use init_std / sqrt(2 depth) */
  float rope_base;    /* 10000 */
  float norm_eps;     /* 1e-6, inside the square root of every RMSNorm */
  float muon_momentum;/* 0.95 */
  int32_t ns_steps;   /* Newton-Schulz iterations, 0..5 */
  float ns_coeffs[5][3]; /* (a, b, c) per iteration */
  int64_t num_steps;  /* informational: steps at a tokens:params ratio of 8 with 2^20-token batches */
  int32_t ns_split_steps; /* 16-bit precisions: 0 (the default) runs every Newton-Schulz
                             product on fp16 operands (fp32 accumulate, X carried in fp32);
                             n > 0 runs them on bf16 operands instead, the first n
                             iterations forming A A and B X from fp32 operands split into
                             bf16 hi + lo parts (3 MFMA products; X X^T stays plain bf16) */
  int32_t fp8_gemms;  /* precision GPT_FP8: which Linear GEMMs take per-tensor scaled e4m3
                         operands, a mask of GPT_FP8_FWD (Y = X W^T), GPT_FP8_WGRAD
                         (dW = dY^T X) and GPT_FP8_DGRAD (dX = dY W); default all three.
                         Other bits: GPT_ERR_ARG. Ignored for the other precisions. */
  int32_t attn_window;  /* sliding-window attention: query i sees keys i - attn_window < j <= i
                           (flash-attention's window_size = (attn_window - 1, 0)); 0 (the
                           default) = every earlier key; negative: GPT_ERR_ARG */
  int32_t n_kv_head;  /* grouped-query attention: key/value heads, each shared by n_head /
                         n_kv_head query heads (query head h uses key/value head
                         h / (n_head / n_kv_head)); Wk, Wv are (n_kv_head * head_dim) x d.
                         0 (the default) = n_head; must divide n_head, else GPT_ERR_SHAPE */
  int32_t extras;     /* a mask of the efficiency tricks printed under the GPT model section
                         of the nanochat articles, with their parameters in tensor S:
                         GPT_EXTRA_RESID: layer i reads lr[i] x + l0[i] x0 (x the stream
                           reaching it, x0 the stream entering layer 0);
                         GPT_EXTRA_SMEAR: after the embedding, x[t] += ls sigmoid(ws .
                           x[t, 0:24]) x[t-1] within each sequence (d >= 24);
                         GPT_EXTRA_BACKOUT: the final norm reads x_L - lb x_mid, x_mid the
                           stream entering layer L/2;
                         GPT_EXTRA_VALUE_EMB: after the QKV projection of layer i, v[t, h] +=
                           3 sigmoid(Wg_i[h] . a[t, 0:24]) VE_i[token t, h], a the block's
                           normed input (tensors VE_i and G).
                         S starts at the identity (lr = 1, the rest 0), VE and G at 0; AdamW
                         updates all of them.
                         GPT_EXTRA_NORMUON: muon_update scales each output row of a matrix's
                           orthogonalised update by 1/sqrt(V), V its running mean square
                           (decay normuon_beta2, starts at 0), and rescales the update to its
                           Frobenius norm (no parameters of its own).
                         0 (the default) = none; other bits: GPT_ERR_ARG */
  float normuon_beta2;  /* NorMuon's second-moment decay in [0, 1) (else GPT_ERR_ARG when
                           GPT_EXTRA_NORMUON is set); default 0.95 */
} gpt_cfg;

enum { GPT_FP8_FWD = 1, GPT_FP8_WGRAD = 2, GPT_FP8_DGRAD = 4 };
enum { GPT_EXTRA_RESID = 1, GPT_EXTRA_SMEAR = 2, GPT_EXTRA_BACKOUT = 4, GPT_EXTRA_VALUE_EMB = 8, GPT_EXTRA_NORMUON = 16 };

typedef struct gpt_model gpt_model; /* opaque */

/* Fill *out from depth: d = 64*depth (rounded up to a multiple of 128), hd = 128,
 * H = d/128, F = 4d, V = 32768, T = 2048, B = 16, bf16, the default Newton-Schulz
 * table.  Returns GPT_ERR_ARG for depth < 1 or out == NULL. */
int gpt_cfg_from_depth(int32_t depth, gpt_cfg* out);

/* CPU-only consistency check of a configuration. */
int gpt_cfg_validate(const gpt_cfg* cfg);

/* sizeof(gpt_cfg) as compiled into the library (for bindings that mirror it). */
size_t gpt_cfg_bytes(void);

/* Bytes of device memory the model needs (parameters, gradients, momentum,
 * saved activations and workspaces); 0 when cfg is invalid. */
size_t gpt_state_bytes(const gpt_cfg* cfg);

/* Carve the caller's arena (>= gpt_state_bytes, 256-byte aligned), draw the
 * initial weights on the device from a counter-based generator keyed by seed
 * (N(0, init_std^2), output projections scaled), zero the momentum. */
int gpt_init(const gpt_cfg* cfg, uint64_t seed, void* d_arena, size_t arena_bytes, void* stream,
             gpt_model** out);

/* One forward + backward pass over the micro-batch d_tokens/d_targets (int32,
 * row-major [batch][seq_len]).  Overwrites every gradient.  Returns the mean
 * cross-entropy over the batch*seq_len positions, or NaN on error.  cfg must
 * match the model's configuration. */
float gpt_step(gpt_model* m, const int32_t* d_tokens, const int32_t* d_targets, const gpt_cfg* cfg, void* stream);

/* gpt_step for gradient accumulation over micro-batches (the single-GPU mode of the
 * nanochat articles, which run the optimizer once per total batch): every gradient
 * of this micro-batch's mean loss is multiplied by grad_scale (1/number of
 * micro-batches gives the mean over the total batch) and, when accumulate != 0,
 * added to the stored gradients instead of replacing them.  The scale enters at
 * the loss gradient, which the whole backward is linear in.  Returns the
 * micro-batch's own mean loss; NaN and GPT_ERR_ARG for a non-finite grad_scale.
 * After an error the stored gradients are undefined.
 * gpt_step(m, t, y, cfg, s) is gpt_step_accumulate(m, t, y, cfg, 0, 1, s). */
float gpt_step_accumulate(gpt_model* m, const int32_t* d_tokens, const int32_t* d_targets, const gpt_cfg* cfg,
                          int32_t accumulate, float grad_scale, void* stream);

/* gpt_step_accumulate in two halves, for callers that enqueue several steps before
 * reading a loss, or record the step (with muon_update) into a HIP graph:
 * gpt_step_async enqueues the forward and backward on the stream and returns at once
 * (argument and launch errors as a gpt_status; no synchronisation, no device memory
 * allocated, no memset node: every buffer the step clears is cleared by a kernel);
 * gpt_step_result synchronises the stream and returns the mean loss of the last
 * enqueued step, or NaN with gpt_last_status set (token range, non-finite logits).
 * In a graph, the loss and error flags of the last replay stay on the device until
 * gpt_step_result reads them.  A graph records the host-side choices made while it is
 * captured: the e4m3 weight refresh of an fp8 step is recorded only when the weights
 * changed before the capture (capture muon_update and the next step together), and
 * adamw_update's step counter is fixed at capture, so AdamW does not belong in a
 * replayed graph. */
int gpt_step_async(gpt_model* m, const int32_t* d_tokens, const int32_t* d_targets, const gpt_cfg* cfg,
                   int32_t accumulate, float grad_scale, void* stream);
float gpt_step_result(gpt_model* m, void* stream);

/* Copy the fp32 gradient of tensor `tensor_id` (n elements) to host memory. */
int gpt_grads(gpt_model* m, int32_t tensor_id, float* h_out, size_t n, void* stream);

/* Muon on every block matrix (Wq, Wk, Wv, Wo, W1, W2 of every layer, each
 * separately): B <- mu B + G; X = B / (|B|_F + 1e-7); ns_steps iterations of
 * A = X X^T, X <- a X + (b A + c A^2) X on the wide orientation; W <- W - lr X.
 * E and U are not touched.  Stream-ordered, no synchronisation. */
int muon_update(gpt_model* m, float lr, void* stream);

/* AdamW on the token embedding E, the LM head U, the extras' scalars S and the
 * value-embedding tables and gate weights (the
 * tensors Muon leaves to it, per the parameter-type table of "2. Muon Optimize
 * Edici" in the nanochat articles; they print no formula or hyperparameters, so
 * Adam's bias-corrected moments with decoupled weight decay are used).  For the t-th call on this model,
 * with g the gradient of the last gpt_step:
 *   m <- beta1 m + (1-beta1) g;  v <- beta2 v + (1-beta2) g^2;
 *   w <- w - lr wd w - lr (m / (1-beta1^t)) / (sqrt(v / (1-beta2^t)) + eps)
 * on the fp32 masters (bf16 copies refreshed).  Moments live in the arena, zero
 * after gpt_init.  GPT_ERR_ARG for a beta outside [0, 1), negative or non-finite
 * eps, or non-finite lr / weight_decay (the step counter is not advanced then).
 * Stream-ordered, no synchronisation. */
int adamw_update(gpt_model* m, float lr, float beta1, float beta2, float eps, float weight_decay, void* stream);

/* Device copy of the argmax over the vocabulary of every position's logits of the
 * last gpt_step (lowest index among equal maxima), int32 [batch*seq_len]. */
int gpt_argmax(gpt_model* m, int32_t* d_out, void* stream);

/* Device copy of the per-position cross-entropy of the last gpt_step, fp32. */
int gpt_row_loss(gpt_model* m, float* d_out, void* stream);

/* Host copies in and out of parameters, gradients and Muon momentum (fp32).
 * Setting a parameter refreshes its low-precision copy. */
int gpt_get_params(gpt_model* m, int32_t tensor_id, float* h_out, size_t n, void* stream);
int gpt_set_params(gpt_model* m, int32_t tensor_id, const float* h_in, size_t n, void* stream);
int gpt_set_grads(gpt_model* m, int32_t tensor_id, const float* h_in, size_t n, void* stream);
int gpt_get_momentum(gpt_model* m, int32_t tensor_id, float* h_out, size_t n, void* stream);
int gpt_set_momentum(gpt_model* m, int32_t tensor_id, const float* h_in, size_t n, void* stream);

int gpt_tensor_count(const gpt_cfg* cfg);
int gpt_tensor_shape(const gpt_cfg* cfg, int32_t tensor_id, int32_t* rows, int32_t* cols);

int gpt_last_status(const gpt_model* m);
const char* gpt_status_str(int status);
void gpt_free(gpt_model* m);

/* Optional per-launch timing of one GEMM kernel class inside gpt_step and
 * muon_update: events are recorded around each launch whose kernel name
 * (gpt_gemm_kernel_name) equals `name`; NULL disables.  gpt_prof_read returns
 * the launch count, the summed milliseconds and the summed algorithmic FLOPs. */
int gpt_prof_enable(gpt_model* m, const char* name);
int gpt_prof_read(gpt_model* m, int64_t* launches, double* ms, double* flops);

/* Operand capture for stage-isolated checks of the Linear products (the QKV, output,
 * fc and proj projections of a block, each Y = X W^T with dW = dY^T X and dX = dY W,
 * and the LM head).  With d_buf non-NULL (device memory, 256-byte aligned, at least
 * gpt_capture_bytes(cfg, layer) bytes, owned by the caller and kept alive while set),
 * every later gpt_step copies what layer `layer` (0 <= layer < depth) or, with layer ==
 * depth, the LM head feeds to and gets from its GEMMs into d_buf, each item starting
 * on a 256-byte boundary in this order ("act" = the step's activation type, bf16 or
 * fp32; N = batch*seq_len, QD = d + 2 n_kv_head head_dim):
 *   block layer: a [N][d] act (QKV input), qkv [N][QD] act (QKV output, before RoPE /
 *     QK-norm / value embeddings), x [N][d] fp32 (the residual stream the layer adds to),
 *     o [N][d] act (output-projection input), h1 [N][d] fp32 (= x + o Wo^T), m [N][d] act,
 *     g [N][F] act (= relu(u)^2 with u = m W1^T; u itself is not kept), h2 [N][d] fp32
 *     (= h1 + g W2^T);
 *     backward: dh [N][d] act (proj output gradient), du [N][F] act (= (dh W2) 2 relu(u),
 *     with relu(u) taken as sqrt(g)),
 *     dm [N][d] fp32 (= du W1), dh1 [N][d] act (output-projection output gradient),
 *     do [N][d] act (= dh1 Wo), dqkv [N][QD] act (QKV output gradient), da [N][d] fp32
 *     (= dqkv [Wq; Wk; Wv]);
 *   LM head: r [N][d] act, logits [N][V] fp32, dlogits [N][V] act, dr [N][d] fp32.
 * The weight gradients are the ones gpt_grads returns.  d_buf == NULL switches the
 * capture off.  GPT_ERR_ARG for a layer out of range, a short or misaligned buffer.
 * gpt_capture_bytes returns 0 for an invalid cfg or layer. */
size_t gpt_capture_bytes(const gpt_cfg* cfg, int32_t layer);
int gpt_capture(gpt_model* m, int32_t layer, void* d_buf, size_t bytes);

/* ------------------------------------------------------------------------
 * Kernel-level entry points for stage-isolated checks.  All pointers are
 * device pointers owned by the caller; `dtype` is GPT_FP32 or GPT_BF16 and
 * gives the element type of the activation-typed buffers (act); every call is
 * stream-ordered and returns a gpt_status.
 */

/* C[b][m][n] (fp32) = sum_k A(m,k) B(n,k) for b < batch, where A(m,k) =
 * A[m*lda+k] if a_kmaj else A[k*lda+m], and likewise B.  Element strides
 * between batches sA, sB, sC.  tile (bf16): 0 auto, 1 = 256x256 (k tiles of 64
 * in two LDS stages), 3 = 256x256 (k tiles of 32, three stages), 5 = 256x256 (k
 * tiles of 32, four stages), 4 = 256x256 register-staged, 2 = 128x128;
 * adding 16 declares C symmetric (M == N and A, B such that C[m][n] = C[n][m]):
 * the 256x256 kernels then compute the upper tiles and mirror them.
 * splits > 1 splits K and needs ws of splits*batch*M*N*4 bytes; splits < 0 takes the
 * factor gpt_step's launches choose for this shape (gptk_gemm_auto_splits).
 * GPT_ERR_ARG when lda (ldb) is below the stored row length (K for a k-major operand,
 * else M (N)), ldc < N, a batch stride is negative, an input stride is neither 0 (one
 * matrix shared by the batch) nor at least one whole matrix, the output stride is
 * below M*ldc with batch > 1, or batch*splits > 65535; the workspace is too small; or a
 * shape/alignment the kernels do not take (GPT_ERR_SHAPE).  Checks run before any
 * launch. */
int gptk_gemm(int dtype, int a_kmaj, int b_kmaj, int M, int N, int K, int batch, const void* A, long lda,
              long sA, const void* B, long ldb, long sB, float* C, long ldc, long sC, int tile, int splits,
              void* ws, size_t ws_bytes, void* stream);

/* the split-K factor gptk_gemm with splits < 0 (and gpt_step) uses for this shape */
int gptk_gemm_auto_splits(int dtype, int a_kmaj, int b_kmaj, int M, int N, int K, int batch);

/* as gptk_gemm (bf16) with each operand given as two bf16 planes, a high part
 * (Ah, Bh) and the residual of an fp32 value (Al, Bl), same layout and strides:
 * C = Ah*Bh + Ah*Bl + Al*Bh on bf16 MFMA with fp32 accumulation -- the product
 * Muon's Newton-Schulz uses in its leading iterations. */
int gptk_gemm_split(int a_kmaj, int b_kmaj, int M, int N, int K, int batch, const void* Ah, const void* Al, long lda,
                    long sA, const void* Bh, const void* Bl, long ldb, long sB, float* C, long ldc, long sC,
                    void* stream);

/* Muon's orthogonalisation of one matrix, exactly as muon_update runs it on every
 * block matrix ("2. Muon Optimize Edici": X0 = G / (|G|_F + 1e-7), then `steps` (<= 5)
 * Polar-Express iterations with the table coeffs = [a0 b0 c0 a1 b1 c1 ...]): on the wide
 * orientation (a tall G is orthogonalised as G^T and transposed back), A = X X^T,
 * B = b A + c A A, X <- a X + B X, every product on MFMA with fp32 accumulation and X
 * carried in fp32; dtype GPT_BF16 = the 16-bit schedule (fp16 operands), GPT_FP32 = fp32
 * operands.  G, X fp32 [rows][cols] (rows, cols multiples of 8, else GPT_ERR_SHAPE), ws
 * device scratch of gptk_ns_ws_bytes(rows, cols) bytes, 256-byte aligned. */
size_t gptk_ns_ws_bytes(int rows, int cols);
int gptk_newton_schulz(int dtype, const float* G, int rows, int cols, const float* coeffs, int steps, float* X,
                       void* ws, size_t ws_bytes, void* stream);

/* fp8 (OCP e4m3fn) per-tensor current scaling of x [rows][cols] (row stride ld, fp32 or
 * bf16 by dtype): s = 448 / max|x| (1 when x is all zero); q [rows][cols] and/or qt
 * [cols][rows] receive e4m3(x * s) (round to nearest even, saturating at +-448);
 * inv_scale[0] = 1/s.  amax_slot is one uint32 of scratch. */
int gptk_quant_e4m3(int dtype, const void* x, int rows, int cols, long ld, uint32_t* amax_slot, uint8_t* q,
                    uint8_t* qt, float* inv_scale, void* stream);

/* C [M][N] fp32 = dq_a[0] * dq_b[0] * sum_k A[m][k] B[n][k] with e4m3 A [M][K], B [N][K]
 * (reduction index contiguous, K, lda, ldb multiples of 16), on fp8 MFMA.  splits > 1
 * divides the reduction into that many parts (multiples of 64) whose fp32 partial
 * products go to ws (splits*M*N floats, else GPT_ERR_ARG) and are then summed. */
int gptk_gemm_fp8(int M, int N, int K, const uint8_t* A, long lda, const uint8_t* B, long ldb, const float* dq_a,
                  const float* dq_b, float* C, long ldc, int splits, void* ws, size_t ws_bytes, void* stream);

/* name of the GEMM kernel instantiation gptk_gemm / gpt_step launch for these
 * layouts and sizes, e.g. "gemm_bf16_dma_kernel<256,256,NT>" (NT: both operands have
 * the reduction index contiguous; NN: B transposed on load; TN: both) */
const char* gpt_gemm_kernel_name(int dtype, int a_kmaj, int b_kmaj, int M, int N, int K, int batch);

/* causal attention over qkv act [B*T][(H + 2*Hkv)*hd] (H query heads, then Hkv key
 * heads, then Hkv value heads, hd columns each) -> o act [B*T][H*hd], lse fp32
 * [B][H][T] (natural log of the sum of exp of q.k/sqrt(hd)). hd in {32,64,128}.
 * Query head h attends with key/value head h / (H / Hkv): Hkv = H is multi-head
 * attention, Hkv < H grouped-query attention (H % Hkv != 0, Hkv < 1 or Hkv > H:
 * GPT_ERR_ARG).  window > 0: query i attends to keys i - window < j <= i (sliding
 * window); 0: all j <= i; negative: GPT_ERR_ARG. */
int gptk_attn_fwd(int dtype, const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv, int hd, int window,
                  void* stream);
/* gptk_attn_fwd for inputs whose every q and k row is RMS-normalised per head, as the
 * article's QK-norm ("1. GPT Modeli") leaves them and as gpt_step runs it: |q.k| is then at
 * most hd (up to bf16 rounding), so the bf16 kernel exponentiates against a fixed
 * reference sqrt(hd) log2(e) instead of a running row maximum (same arguments, layout and
 * errors; same result up to rounding).  Inputs that are not normalised can overflow the
 * exponentials: the caller guarantees the normalisation.  fp32 uses gptk_attn_fwd's
 * kernel. */
int gptk_attn_fwd_qknorm(int dtype, const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv, int hd,
                         int window, void* stream);
/* Process-wide choice among the bf16 head_dim-128 attention kernels, for A/B
 * measurements (every variant computes the same result; the default is the fastest
 * measured).  pass 0 = forward: variant 0 = 32 queries per wave (two waves per SIMD),
 * 1 = 64 queries per wave (one wave per SIMD); pass 1 = backward: variant 0 = dQ by
 * waves of 32 queries and dK/dV by 8 waves of 32 keys (dV and dK accumulated by different
 * waves), software-pipelined (P of the next query tile formed while the current one's
 * dS is), 1 = dQ by waves of 64 queries and dK/dV by 4 waves of 64 keys (one wave
 * accumulates both), 2 = variant 0 without the pipelining (S -> P, a barrier, then
 * dS within each query tile).  GPT_ERR_ARG for another pass/variant.
 * Not thread-safe against concurrent launches. */
int gptk_attn_variant(int pass, int variant);

/* Which cross-entropy kernel later steps and gptk_ce take when V is a multiple of 16384
 * (the article's "1. GPT Modeli": the loss over the 32,768-entry vocabulary).  variant 0 (the
 * default) = two passes over each row with few registers, two rows in flight per CU;
 * 1 = the row held in registers, one row per CU.  Both give the same argmax (lowest index
 * among equal maxima) and, up to the order of the exponential sums, the same loss and
 * gradient.  GPT_ERR_ARG for another variant.  Process-wide, not thread-safe against
 * concurrent launches. */
int gptk_ce_variant(int variant);

/* Process-wide choice of where fp8 steps take the per-tensor amax of the activations and
 * output gradients they quantise ("3. Hassasiyet Yönetimi", the --fp8 recipe: per-tensor
 * scales from the current max|x|): on = 1 (the default), the kernels that produce each
 * such tensor (RMSNorm, attention, the fc and dReLU^2 GEMM epilogues, the RoPE backward,
 * the cross-entropy gradient) also write per-wave maxima of the values as they store
 * them, which one small launch folds into the tensor's slot; off = 0, a separate pass
 * reads the stored tensor.  Both give the same amax bit for bit (bf16 rounding is
 * monotonic), so the same codes and results.  Configurations with extras, or with some
 * Linears outside fp8, always take the separate pass.  on < 0 only queries.  Returns the
 * previous setting.  Not thread-safe against concurrent steps. */
int gptk_fp8_fused_amax(int on);

/* Where the backward's weight-gradient products run (the article's "2. Muon Optimize Edici": the
 * gradients of one step feed one optimizer update, so each dW = dY^T X only has to exist
 * by the end of the step).  On the side stream: a second stream the model owns, beside
 * the data-gradient chain, with events so that each dY buffer is rewritten only after its
 * weight-gradient product has read it and the caller's stream waits for all of them before
 * gpt_step returns (or, for gpt_step_async, before any later work on that stream); the LM
 * head's products, and those of e4m3 steps whose weight gradients quantise their own
 * inputs (fp8_gemms without the forward bit), always stay on the caller's stream.  on = 1 (the
 * default): the side stream for models whose data-gradient products ([B*T][d], [B*T][F])
 * leave part of a round of 256x256 tiles on the device's CUs idle, which the weight
 * gradients then fill; 2: the side stream for every model; 0: every product on the
 * caller's stream.  All give the same results bit for bit (each product is computed the
 * same way, only its start time moves).  on < 0 only queries.  Returns the previous
 * setting.  Process-wide, not thread-safe against concurrent steps. */
int gptk_side_stream(int on);

/* backward: dqkv act [B*T][(H + 2*Hkv)*hd] from qkv, o, dO act [B*T][H*hd] and lse,
 * with the forward's Hkv and window (dK and dV of a shared head sum over its query
 * heads); D is fp32 scratch [B][H][T] (receives rowsum(dO*O)). */
int gptk_attn_bwd(int dtype, const void* qkv, const void* o, const void* dO, const float* lse, float* D,
                  void* dqkv, int B, int T, int H, int Hkv, int hd, int window, void* stream);

/* gptk_attn_bwd without the D argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight loops, harnesses that forbid hipMalloc): the
 * rowsum(dO*O) scratch is a file-scope device array of the library, 4 MiB per GPU
 * (B*H*T <= 1048576, else GPT_ERR_ARG), held until the process ends; its device address
 * is looked up once per device on the first call there (GPT_ERR_HIP if that fails).
 * Calls on one GPU share that array and keep what the last one left in it, so calls
 * that overlap on one GPU (different streams or threads) race; calls ordered on one
 * stream do not.  No hipMalloc, hipFree or allocating library call is made.  Other
 * arguments, results and errors as gptk_attn_bwd. */
int gptk_attn_bwd_noalloc(int dtype, const void* qkv, const void* o, const void* dO, const float* lse, void* dqkv,
                          int B, int T, int H, int Hkv, int hd, int window, void* stream);

/* y act = x / sqrt(mean(x^2) + eps) per row of x fp32 [N][d]; rstd fp32 [N] */
int gptk_rmsnorm_fwd(int dtype, const float* x, void* y, float* rstd, int N, int d, float eps, void* stream);
/* dx fp32 (and act copy if dx_act) = dres + rstd*(dy - y*mean(dy*y)), y = x*rstd;
 * dres may be NULL */
int gptk_rmsnorm_bwd(int dtype, const float* dy, const float* x, const float* rstd, const float* dres, float* dx,
                     void* dx_act, int N, int d, void* stream);

/* in place on the H query and Hkv key head vectors of qkv act [B*T][(H + 2*Hkv)*hd]
 * (layout as for gptk_attn_fwd): rotate half-split pairs by t*base^(-2i/hd) then
 * RMS-normalise each head vector; rstd_q fp32 [B*T][H], rstd_k fp32 [B*T][Hkv].  cs
 * is fp32 scratch of T*hd floats (the rotation table). */
int gptk_rope_qknorm_fwd(int dtype, void* qkv, float* cs, float* rstd_q, float* rstd_k, int B, int T, int H, int Hkv,
                         int hd, float base, float eps, void* stream);
/* in place on the q and k parts of dqkv: gradient through the norm and rotation */
int gptk_rope_qknorm_bwd(int dtype, void* dqkv, const void* qkv, float* cs, const float* rstd_q,
                         const float* rstd_k, int B, int T, int H, int Hkv, int hd, float base, void* stream);

/* fused softmax cross-entropy over logits fp32 [N][V]: row_loss fp32 [N],
 * dlogits act [N][V] = (softmax - onehot(target)) * inv_n, argmax int32 [N]
 * (lowest index among equal maxima); err int32 [1] gets bit 1 for a target out
 * of range and bit 2 for a non-finite logit. */
int gptk_cross_entropy(int dtype, const float* logits, const int32_t* targets, void* dlogits, float* row_loss,
                       int32_t* argmax, int N, int V, float inv_n, int32_t* err, void* stream);

/* h fp32 [N][d] = E fp32 [V][d] rows of tokens; err bit 1 on an id outside [0,V) */
int gptk_embed_gather(const int32_t* tokens, const float* E, float* h, int N, int d, int V, int32_t* err,
                      void* stream);
/* dE fp32 [V][d] = sum over positions n with tokens[n]==v of dh[n] (in increasing
 * n, deterministic); sorted int32 [N] receives the stable order of positions by
 * token; ws must hold gptk_embed_ws_bytes(N, V, d) bytes. */
size_t gptk_embed_ws_bytes(int N, int V, int d);
int gptk_embed_scatter(const int32_t* tokens, const float* dh, float* dE, int N, int V, int d, void* ws,
                       int32_t* sorted, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GPT_H */
