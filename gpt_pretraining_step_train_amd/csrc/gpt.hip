// C ABI of the GPT training step: configuration, arena carving, the forward /
// backward launch sequence of gpt_step, Muon, and the kernel-level entry points.
#include <math.h>
#include <string.h>

#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/gpt.h"
#include "common.h"
#include "kernels.h"

// Polar Express table: the first two (a, b, c) are the ones the nanochat article
// prints (section "2. Muon Optimize Edici"); the last three are this library's
// reading of the elided rows: each is the odd quintic minimising max|1 - p(x)| on
// the interval the singular values occupy after the previous steps, starting from
// [1e-3, 1] (images [0.033,1.966] -> [0.131,1.869] -> [0.432,1.568] -> [0.871,1.129]).
static const float kNsCoeffs[5][3] = {
    {8.156f, -22.483f, 15.879f},
    {4.043f, -2.809f, 0.500f},
    {3.982259f, -2.970419f, 0.565428f},
    {3.335152f, -2.500954f, 0.511463f},
    {2.315355f, -1.682066f, 0.420231f},
};

namespace {

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

#ifndef GPT_SLICE_ALIGN
#define GPT_SLICE_ALIGN 256
#endif
struct Plan {
  size_t total = 0;
  size_t add(size_t bytes) {
    // slices of 2 MiB and more start on a GPT_SLICE_ALIGN boundary (relative to the arena)
    if (bytes >= ((size_t)2 << 20)) total = (total + GPT_SLICE_ALIGN - 1) / GPT_SLICE_ALIGN * GPT_SLICE_ALIGN;
    const size_t o = total;
    total += al256(bytes);
    return o;
  }
};

// key/value heads and the rows of Wk and Wv (grouped-query attention; n_kv_head = 0
// means one key/value head per query head)
inline int kv_heads(const gpt_cfg& c) { return c.n_kv_head > 0 ? c.n_kv_head : c.n_head; }
inline size_t kv_dim(const gpt_cfg& c) { return (size_t)kv_heads(c) * c.head_dim; }
// columns of the fused QKV projection output: q (d), k and v (kv_dim each)
inline size_t qkv_dim(const gpt_cfg& c) { return (size_t)c.d_model + 2 * kv_dim(c); }
// the extras' parameter vector S (when any extra is on): residual scales lr[L], x0
// scales l0[L], the smear scale ls, the backout scale lb, the smear-gate weights ws[24]
constexpr int kSmearCh = 24;
constexpr int kModelExtras = GPT_EXTRA_RESID | GPT_EXTRA_SMEAR | GPT_EXTRA_BACKOUT | GPT_EXTRA_VALUE_EMB;
inline size_t n_extras(const gpt_cfg& c) { return c.extras & kModelExtras ? (size_t)2 * c.depth + 2 + kSmearCh : 0; }
inline int s_lr(const gpt_cfg&, int l) { return l; }
inline int s_l0(const gpt_cfg& c, int l) { return c.depth + l; }
inline int s_ls(const gpt_cfg& c) { return 2 * c.depth; }
inline int s_lb(const gpt_cfg& c) { return 2 * c.depth + 1; }
inline int s_ws(const gpt_cfg& c) { return 2 * c.depth + 2; }
// S's region in the parameter vector, padded to whole float4s so that the value-embedding
// tables (per layer [V][kv_dim], then the gate weights [L Hkv][24]) that follow are aligned
constexpr int kVeCh = 24;
inline size_t s_region(const gpt_cfg& c) { return (n_extras(c) + 3) / 4 * 4; }
inline size_t n_ve(const gpt_cfg& c) {
  return c.extras & GPT_EXTRA_VALUE_EMB ? (size_t)c.depth * c.vocab * kv_dim(c) : 0;
}
inline size_t n_vg(const gpt_cfg& c) {
  return c.extras & GPT_EXTRA_VALUE_EMB ? (size_t)c.depth * kv_heads(c) * kVeCh : 0;
}
// parameters after U: S (padded), the value-embedding tables and their gate weights
inline size_t n_tail(const gpt_cfg& c) { return s_region(c) + n_ve(c) + n_vg(c); }

// element offsets of the six block matrices inside one layer's slice
struct LayerOffs {
  size_t q, k, v, o, w1, w2, stride;
};
inline LayerOffs layer_offs(const gpt_cfg& c) {
  const size_t d = c.d_model, F = c.d_ff, dk = kv_dim(c);
  LayerOffs L;
  L.q = 0; L.k = d * d; L.v = d * d + dk * d; L.o = d * d + 2 * dk * d; L.w1 = L.o + d * d; L.w2 = L.w1 + F * d;
  L.stride = L.w2 + d * F;
  return L;
}

struct Offsets {
  size_t params, grads, mom, adam_m, adam_v, wact, uact, hs, a, rstd_a, qkv, rq, rk, o, lse, m, rstd_m, g, r, rstd_f, logits,
      dlogits, row_loss, argmax, dh0, dh1, dh_act, dtmp, dbig, dqkv, do_act, Dbuf, splitws, embws, xf, xa0, xa1, xl0,
      xl1, Af, Aa, Ba, Al, Bl, ss_part, ss, mat_off, mat_size, mv_jobs, rope, loss, err, wq8, wtq8, wscale, q8a, q8b, q8b2, q8c,
      xq8t, amax, qinv, amax_part, amax_fuse, hx, hfin, emb, dx0, dmid, xpart, vg, dve, vdz, vpart, vred, nm_v, nm_mean, nm_scale,
      nm_roff, nm_ws;
  size_t splitws_bytes;
};

constexpr int kSumsqParts = 64;
// quantisation events of one fp8 step: weights (4 per layer + head), forward inputs
// (4 per layer + head), backward output gradients and inputs (8 per layer + 2)
inline size_t kQuantSlots(const gpt_cfg& c) { return 16 * (size_t)c.depth + 8; }
// process-wide: fp8 steps take the amax of their quantised activations and gradients from
// the producing kernels (gptk_fp8_fused_amax)
static int g_fp8_fused_amax = 1;
// backward weight gradients on the model's side stream (gptk_side_stream): 0 never, 1 where
// the model's data-gradient launches leave part of a round of tiles idle, 2 always
static int g_side_stream = 1;
// capacity (floats) for the per-wave amax partials the producers of a quantised tensor
// write: the loss gradient's 4 per row, the dV and RoPE waves of dqkv, the fc / dReLU2
// GEMMs' 8 per tile (a producer that would need more falls back to the amax pass)
inline size_t kFuseParts(const gpt_cfg& c) {
  const size_t N = (size_t)c.batch * c.seq_len;
  return 4 * N + N * qkv_dim(c) / 512 + 65536;
}
// the forward's quantisation of each Linear input also serves its weight gradient
inline bool keeps_xt(const gpt_cfg& c) {
  return c.precision == GPT_FP8 && (c.fp8_gemms & GPT_FP8_FWD) && (c.fp8_gemms & GPT_FP8_WGRAD);
}

int act_of(const gpt_cfg& c) { return c.precision == GPT_FP32 ? ACT_F32 : ACT_BF16; }

size_t wgrad_ws_bytes(const gpt_cfg& c) {
  const int N = c.batch * c.seq_len, d = c.d_model, F = c.d_ff, V = c.vocab;
  const int shapes[5][2] = {{d, F}, {F, d}, {d, d}, {(int)qkv_dim(c), d}, {V, d}};
  size_t best = 0;
  for (auto& s : shapes) {
    GemmArgs p;
    p.M = s[0]; p.N = s[1]; p.K = N; p.dtype = act_of(c); p.a_kmaj = false; p.b_kmaj = false;
    const int sp = gemm_auto_splits(p);
    if (sp > 1) best = std::max(best, (size_t)sp * s[0] * s[1] * 4);
  }
  if (V >= 8192) {  // the LM head's data gradient (dr = dz U, reduction over the vocabulary)
    GemmArgs p;
    p.M = N; p.N = d; p.K = V; p.dtype = act_of(c); p.b_kmaj = false;
    const int sp = gemm_auto_splits(p);
    if (sp > 1) best = std::max(best, (size_t)sp * N * d * 4);
  }
  return best;
}

// elements of the Gram-sized Newton-Schulz workspace of the first (d x d) batch: Wq, Wk, Wv,
// Wo of every layer, or Wq, Wo when grouped-query attention gives Wk, Wv their own shape
static size_t ns_first_elems(const gpt_cfg& c) {
  return (size_t)(kv_dim(c) == (size_t)c.d_model ? 4 : 2) * c.depth * c.d_model * c.d_model;
}

Offsets plan(const gpt_cfg& c, size_t* total) {
  Plan P;
  Offsets O;
  const size_t N = (size_t)c.batch * c.seq_len, d = c.d_model, F = c.d_ff, V = c.vocab, L = c.depth;
  const size_t H = c.n_head, T = c.seq_len, B = c.batch;
  const size_t es = act_of(c) == ACT_BF16 ? 2 : 4;
  const size_t nE = V * d, nU = V * d, nBlk = L * layer_offs(c).stride;
  const size_t s = std::min(d, F), l = std::max(d, F);
  const size_t nS = n_extras(c), nT = n_tail(c);
  O.params = P.add((nE + nBlk + nU + nT) * 4);  // E, blocks, U, S, value embeddings
  O.grads = P.add((nE + nBlk + nU + nT) * 4);
  O.mom = P.add(nBlk * 4);
  O.adam_m = P.add((nE + nU + nT) * 4);  // AdamW moments of E, U, then the tail
  O.adam_v = P.add((nE + nU + nT) * 4);
  // extras: mixed layer inputs, the final norm's input, the raw embedding, the gradient
  // sums flowing to x0 and x_mid, and the per-row terms of dS
  O.hx = c.extras & GPT_EXTRA_RESID ? P.add(L * N * d * 4) : 0;
  O.dx0 = c.extras & GPT_EXTRA_RESID ? P.add(N * d * 4) : 0;
  O.hfin = c.extras & GPT_EXTRA_BACKOUT ? P.add(N * d * 4) : 0;
  O.dmid = c.extras & GPT_EXTRA_BACKOUT ? P.add(N * d * 4) : 0;
  O.emb = c.extras & GPT_EXTRA_SMEAR ? P.add(N * d * 4) : 0;
  O.xpart = nS ? P.add(nS * N * 4) : 0;
  // value embeddings: gate values per layer, and the backward's rows of dVE, dz and d(gate)
  const bool ve = c.extras & GPT_EXTRA_VALUE_EMB;
  O.vg = ve ? P.add(L * N * kv_heads(c) * 4) : 0;
  O.dve = ve ? P.add(N * kv_dim(c) * 4) : 0;
  O.vdz = ve ? P.add(N * kv_heads(c) * 4) : 0;
  O.vpart = ve ? P.add((size_t)kv_heads(c) * kVeCh * N * 4) : 0;
  O.vred = ve ? P.add(colsum_ws_bytes(kv_heads(c) * kVeCh)) : 0;
  // NorMuon: per output row of every block matrix, its running second moment, this
  // update's mean square and scale; the row offsets of the matrices
  const bool nm = c.extras & GPT_EXTRA_NORMUON;
  const size_t nrows = L * (3 * d + 2 * kv_dim(c) + F);
  O.nm_v = nm ? P.add(nrows * 4) : 0;
  O.nm_mean = nm ? P.add(nrows * 4) : 0;
  O.nm_scale = nm ? P.add(nrows * 4) : 0;
  O.nm_roff = nm ? P.add((6 * L + 1) * 8) : 0;
  O.nm_ws = nm ? P.add(normuon_ws_bytes((int)std::max(d, F))) : 0;
  O.wact = es == 2 ? P.add(nBlk * es) : 0;
  O.uact = es == 2 ? P.add(nU * es) : 0;
  O.hs = P.add((2 * L + 1) * N * d * 4);
  O.a = P.add(L * N * d * es);
  O.rstd_a = P.add(L * N * 4);
  O.qkv = P.add(L * N * qkv_dim(c) * es);
  O.rq = P.add(L * N * H * 4);
  O.rk = P.add(L * N * kv_heads(c) * 4);
  O.o = P.add(L * N * d * es);
  O.lse = P.add(L * B * H * T * 4);
  O.m = P.add(L * N * d * es);
  O.rstd_m = P.add(L * N * 4);
  O.g = P.add(L * N * F * es);
  O.r = P.add(N * d * es);
  O.rstd_f = P.add(N * 4);
  O.logits = P.add(N * V * 4);
  O.dlogits = P.add(N * V * es);
  O.row_loss = P.add(N * 4);
  O.argmax = P.add(N * 4);
  O.dh0 = P.add(N * d * 4);
  O.dh1 = P.add(N * d * 4);
  O.dh_act = P.add(N * d * es);
  O.dtmp = P.add(N * d * 4);
  O.dbig = P.add(N * F * es);
  O.dqkv = P.add(N * qkv_dim(c) * es);
  O.do_act = P.add(N * d * es);
  O.Dbuf = P.add(B * H * T * 4);
  O.splitws_bytes = wgrad_ws_bytes(c);
  O.splitws = P.add(std::max<size_t>(O.splitws_bytes, 256));
  O.embws = P.add(embed_ws_bytes((int)N, (int)V, (int)d));
  O.xf = P.add(nBlk * 4);
  O.xa0 = P.add(nBlk * es);
  O.xa1 = P.add(nBlk * es);
  O.xl0 = P.add(nBlk * es);
  O.xl1 = P.add(nBlk * es);
  // Newton-Schulz Gram-sized workspaces: the d x d batch first, then room for the other
  // batches (the (kv x d) and (s x lw) matrices, run one after the other), so that the
  // first batch can run beside the others on the side stream
  const size_t kvd = kv_dim(c);
  const size_t nsA = ns_first_elems(c) + 2 * L * std::max(s * s, kvd * kvd);
  O.Af = P.add(nsA * 4);
  O.Aa = P.add(nsA * es);
  O.Ba = P.add(nsA * es);
  O.Al = P.add(nsA * es);
  O.Bl = P.add(nsA * es);
  (void)l;
  O.ss_part = P.add(6 * L * kSumsqParts * 8);
  O.ss = P.add(6 * L * 8);
  O.mat_off = P.add(6 * L * 8);
  O.mat_size = P.add(6 * L * 8);
  O.mv_jobs = P.add(6 * L * sizeof(MuonVecJob));
  if (c.precision == GPT_FP8) {
    const size_t wide = std::max(std::max(qkv_dim(c), F), V);
    O.q8c = O.xq8t = 0;
    O.wq8 = P.add(nBlk + nU);
    O.wtq8 = P.add(nBlk + nU);
    O.wscale = P.add((4 * L + 1) * 4);
    O.q8a = P.add(N * wide);
    O.q8b = P.add(N * wide);
    // e4m3 codes of every Linear input, transposed, written by the forward's quantisation
    // pass and read by the weight-gradient GEMM (same tensor, same scale): per layer
    // a, o, m [d][N] and g [F][N], then the head input r [d][N]
    if (keeps_xt(c)) {
      O.xq8t = P.add(L * N * (3 * d + F) + N * d);
      // a second buffer for the block Linears' transposed dY codes: the weight gradient on
      // the backward's side stream reads one while the next Linear's dY is quantised into
      // the other
      O.q8b2 = P.add(N * std::max(qkv_dim(c), F));
    } else {
      O.q8c = P.add(N * std::max(d, F));
    }
    O.amax = P.add(kQuantSlots(c) * 4);
    O.qinv = P.add(kQuantSlots(c) * 4);
    O.amax_part = P.add(kAmaxParts * 4);  // per-block maxima of the amax pass (reused, stream-ordered)
    O.amax_fuse = P.add(kFuseParts(c) * 4);  // the producers' per-wave maxima (reused, stream-ordered)
  } else {
    O.wq8 = O.wtq8 = O.wscale = O.q8a = O.q8b = O.q8b2 = O.q8c = O.xq8t = O.amax = O.qinv = O.amax_part =
        O.amax_fuse = 0;
  }
  O.rope = P.add(T * (c.head_dim / 2) * 2 * 4);
  O.loss = P.add(8);
  O.err = P.add(16);
  *total = P.total;
  return O;
}

// Newton-Schulz workspace layout: every block matrix in its wide orientation, one batch
// per shape: the d x d squares (q, k, v, o of each layer; only q and o when grouped-query
// attention makes Wk, Wv kv x d, which then form their own batch), then the d x F pairs
struct NsLayout {
  int d, F, kv, s, lw;
  bool kvsq;
  size_t nsq, nkv;
  explicit NsLayout(const gpt_cfg& c)
      : d(c.d_model), F(c.d_ff), kv((int)kv_dim(c)), s(std::min(c.d_model, c.d_ff)), lw(std::max(c.d_model, c.d_ff)) {
    kvsq = kv == d;
    nsq = (size_t)(kvsq ? 4 : 2) * c.depth * d * d;
    nkv = kvsq ? 0 : (size_t)2 * c.depth * kv * d;
  }
  size_t xdst(int l, int j) const {
    if (j < 4 && kvsq) return (size_t)(4 * l + j) * d * d;
    if (j == 0 || j == 3) return (size_t)(2 * l + (j == 3)) * d * d;
    if (j < 4) return nsq + (size_t)(2 * l + (j - 1)) * kv * d;
    return nsq + nkv + (size_t)(2 * l + (j - 4)) * s * lw;
  }
  int mrows(int j) const { return j == 4 ? F : (j == 1 || j == 2) ? kv : d; }
  int mcols(int j) const { return j == 5 ? F : d; }
  bool transposed(int j) const { return (j == 4 && F > d) || (j == 5 && d > F); }  // kv <= d: k, v are wide
};

// Operand capture (gpt_capture): the slots of one block layer's four Linear products,
// or of the LM head, in byte sizes; each slot starts 256-byte aligned in the buffer.
enum {
  CAP_A, CAP_QKV, CAP_HIN, CAP_O, CAP_H1, CAP_M, CAP_G, CAP_H2,   // forward
  CAP_DY2, CAP_DU, CAP_DM, CAP_DYO, CAP_DO, CAP_DQKV, CAP_DA,           // backward
  CAP_BLOCK_SLOTS
};
enum { CAP_R, CAP_LOGITS, CAP_DLOGITS, CAP_DR, CAP_HEAD_SLOTS };
std::vector<size_t> capture_sizes(const gpt_cfg& c, int layer) {
  const size_t N = (size_t)c.batch * c.seq_len, d = c.d_model, F = c.d_ff, V = c.vocab, QD = qkv_dim(c);
  const size_t es = act_of(c) == ACT_BF16 ? 2 : 4;
  if (layer == c.depth) return {N * d * es, N * V * 4, N * V * es, N * d * 4};
  return {N * d * es, N * QD * es, N * d * 4, N * d * es, N * d * 4, N * d * es, N * F * es, N * d * 4,
          N * d * es, N * F * es, N * d * 4, N * d * es, N * d * es, N * QD * es, N * d * 4};
}
size_t capture_offset(const gpt_cfg& c, int layer, int slot, size_t* total = nullptr) {
  const std::vector<size_t> sz = capture_sizes(c, layer);
  size_t o = 0, at = 0;
  for (size_t i = 0; i < sz.size(); ++i) {
    if ((int)i == slot) at = o;
    o += al256(sz[i]);
  }
  if (total) *total = o;
  return at;
}

}  // namespace

struct gpt_model {
  gpt_cfg cfg;
  Offsets off;
  char* base = nullptr;
  size_t bytes = 0;
  int at = ACT_BF16;
  size_t es = 2;
  int N = 0;
  size_t nE = 0, nBlk = 0, nU = 0, nS = 0, nT = 0;  // nT: S (padded) and value embeddings
  LayerOffs lo;
  int last_status = GPT_OK;
  bool stepped = false;
  bool fp8 = false;
  bool wq_dirty = true;  // fp8 weight copies must be refreshed before the next step
  int qslot = 0;         // next quantisation slot of the current step
  int gemm_parts = 0;    // amax partials written by the last GEMM launched with amax_part
  long adam_t = 0;       // AdamW steps taken (bias corrections use the next one)
  bool acc_grads = false;  // the current step adds its gradients to the stored ones
  std::vector<int> xslot;  // per weight: quantisation slot of its input in this step's forward
  // operand capture of one layer's Linear products for stage-isolated checks (gpt_capture)
  char* cap_buf = nullptr;
  int cap_layer = -1;
  // matrix table for Muon, in layer order (q, k, v, o, w1, w2); the first row of each
  // matrix in the stacked per-row NorMuon vectors (6L + 1 entries)
  std::vector<long> moff, msize, nm_roff;
  std::vector<MuonVecJob> mv_jobs;  // batched normalise / apply jobs (uploaded by gpt_init)
  // A second stream for the backward's weight-gradient products (dW = dY^T X): each
  // only has to finish before its dY buffer is overwritten and before the step ends, so
  // it runs beside the data-gradient chain and fills that chain's idle CUs (launch
  // tails, bandwidth-bound kernels).  Events order the two streams: fork (the main stream
  // has produced dY), one per dY buffer (its last reader on the side stream) and join.
  hipStream_t side = nullptr;
  hipEvent_t sev_fork = nullptr, sev_join = nullptr, sev_rd[5] = {};
  bool sev_pending[5] = {};
  int q8b_cur = 0;  // fp8: the transposed-dY code buffer the next side-stream weight gradient reads
  bool use_side = false;  // this step puts weight gradients on the side stream
  // the data-gradient launches leave part of a round of 256x256 tiles on the device's CUs
  // idle (set by gpt_init); only then does the side stream gain: a GEMM workgroup holds a
  // whole CU, so two GEMMs over whole rounds only share the same CUs
  bool side_pays = false;
  // profiling
  std::string prof_name;
  std::vector<hipEvent_t> ev;
  std::vector<double> evflops;
  size_t ev_used = 0;

  template <typename T>
  T* at_off(size_t o) { return reinterpret_cast<T*>(base + o); }
  float* params() { return at_off<float>(off.params); }
  float* grads() { return at_off<float>(off.grads); }
  float* blk(float* region) { return region + nE; }
  char* act(size_t o, size_t elems) { return base + o + elems * es; }
  // act-typed copies of the block matrices and of U (the fp32 masters in fp32 mode)
  void* wact(size_t elem) {
    return at == ACT_BF16 ? (void*)(base + off.wact + elem * 2) : (void*)(blk(params()) + elem);
  }
  void* uact() { return at == ACT_BF16 ? (void*)(base + off.uact) : (void*)(params() + nE + nBlk); }
};

namespace {

int run_gemm(gpt_model* M, GemmArgs p, hipStream_t st, bool allow_split) {
  if (p.dtype != ACT_F16) p.dtype = M->at;  // fp16 is chosen per product (Newton-Schulz)
  if (allow_split) {
    p.splits = gemm_auto_splits(p);
    p.ws = M->at_off<float>(M->off.splitws);
    p.ws_bytes = M->off.splitws_bytes;
    if ((size_t)p.splits * p.batch * p.M * p.N * 4 > p.ws_bytes) p.splits = 1;
  } else {
    p.splits = 1;
  }
  if (p.amax_part) {  // the output's amax partials, where this launch can write them
    const int n = gemm_amax_parts(p);
    if (n == 0 || (size_t)n > kFuseParts(M->cfg)) p.amax_part = nullptr;
    M->gemm_parts = p.amax_part ? n : 0;
  }
  const bool prof = !M->prof_name.empty() && M->prof_name == gemm_kernel_name(p);
  if (prof) {
    if (M->ev_used + 2 > M->ev.size()) {
      for (int i = 0; i < 64; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return GPT_ERR_HIP;
        M->ev.push_back(e);
      }
      M->evflops.resize(M->ev.size() / 2 + 1);
    }
    (void)hipEventRecord(M->ev[M->ev_used], st);
  }
  const int rc = launch_gemm(p, st);
  if (prof) {
    (void)hipEventRecord(M->ev[M->ev_used + 1], st);
    M->evflops[M->ev_used / 2] = 2.0 * p.M * p.N * (double)p.K * p.batch;
    M->ev_used += 2;
  }
  return rc ? GPT_ERR_SHAPE : GPT_OK;
}

bool same_shape(const gpt_cfg& a, const gpt_cfg& b) {
  return a.depth == b.depth && a.d_model == b.d_model && a.n_head == b.n_head && a.head_dim == b.head_dim &&
         a.d_ff == b.d_ff && a.vocab == b.vocab && a.seq_len == b.seq_len && a.batch == b.batch &&
         a.precision == b.precision && a.attn_window == b.attn_window && kv_heads(a) == kv_heads(b) &&
         a.extras == b.extras;
}

// element offset of tensor id inside the parameter/gradient vector, and its shape
bool tensor_loc(const gpt_cfg& c, int id, size_t* off, int* rows, int* cols) {
  const size_t d = c.d_model, F = c.d_ff, V = c.vocab, L = c.depth;
  const LayerOffs lo = layer_offs(c);
  if (id == 0) { *off = 0; *rows = (int)V; *cols = (int)d; return true; }
  if (id == (int)(1 + 6 * L)) { *off = V * d + L * lo.stride; *rows = (int)V; *cols = (int)d; return true; }
  if (id == (int)(2 + 6 * L) && (c.extras & kModelExtras)) {
    *off = 2 * V * d + L * lo.stride;
    *rows = 1;
    *cols = (int)n_extras(c);
    return true;
  }
  if ((c.extras & GPT_EXTRA_VALUE_EMB) && id >= (int)(3 + 6 * L) && id <= (int)(3 + 7 * L)) {
    const size_t base = 2 * V * d + L * lo.stride + s_region(c);
    if (id < (int)(3 + 7 * L)) {
      *off = base + (size_t)(id - 3 - 6 * L) * V * kv_dim(c);
      *rows = (int)V;
      *cols = (int)kv_dim(c);
    } else {
      *off = base + n_ve(c);
      *rows = (int)(L * kv_heads(c));
      *cols = kVeCh;
    }
    return true;
  }
  if (id < 1 || id > (int)(6 * L)) return false;
  const int l = (id - 1) / 6, j = (id - 1) % 6;
  const size_t b = V * d + l * lo.stride;
  const size_t o6[6] = {lo.q, lo.k, lo.v, lo.o, lo.w1, lo.w2};
  *off = b + o6[j];
  *rows = j == 4 ? (int)F : (j == 1 || j == 2) ? (int)kv_dim(c) : (int)d;
  *cols = j == 5 ? (int)F : (int)d;
  return true;
}

}  // namespace

extern "C" {

int gpt_cfg_from_depth(int32_t depth, gpt_cfg* out) {
  if (!out || depth < 1 || depth > 64) return GPT_ERR_ARG;
  memset(out, 0, sizeof(*out));
  int d = 64 * depth;
  d = (d + 127) / 128 * 128;
  out->depth = depth;
  out->d_model = d;
  out->head_dim = 128;
  out->n_head = d / 128;
  out->d_ff = 4 * d;
  out->vocab = 32768;
  out->seq_len = 2048;
  out->batch = 16;
  out->precision = GPT_BF16;
  out->init_std = 0.02f;
  out->rope_base = 10000.f;
  out->norm_eps = 1e-6f;
  out->muon_momentum = 0.95f;
  out->ns_steps = 5;
  out->ns_split_steps = 0;
  out->fp8_gemms = GPT_FP8_FWD | GPT_FP8_WGRAD | GPT_FP8_DGRAD;
  out->attn_window = 0;
  out->n_kv_head = 0;
  out->extras = 0;
  out->normuon_beta2 = 0.95f;
  memcpy(out->ns_coeffs, kNsCoeffs, sizeof(kNsCoeffs));
  const double nparams = 2.0 * out->vocab * d + (double)depth * (4.0 * d * d + 2.0 * d * out->d_ff);
  out->num_steps = (int64_t)llround(8.0 * nparams / 1048576.0);
  return GPT_OK;
}

int gpt_cfg_validate(const gpt_cfg* c) {
  if (!c) return GPT_ERR_ARG;
  if (c->depth < 1 || c->d_model < 8 || c->n_head < 1 || c->d_ff < 8 || c->vocab < 8 || c->seq_len < 1 ||
      c->batch < 1)
    return GPT_ERR_SHAPE;
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return GPT_ERR_UNSUPPORTED;
  if (c->n_head * c->head_dim != c->d_model) return GPT_ERR_SHAPE;
  if (c->d_model % 8 || c->d_ff % 8 || c->vocab % 8) return GPT_ERR_SHAPE;
  if (c->d_model > 2048) return GPT_ERR_UNSUPPORTED;
  if (((long)c->batch * c->seq_len) % 8) return GPT_ERR_SHAPE;
  if ((long)c->batch * c->seq_len > (1L << 30) / 4) return GPT_ERR_UNSUPPORTED;
  if (c->precision != GPT_FP32 && c->precision != GPT_BF16 && c->precision != GPT_FP8) return GPT_ERR_UNSUPPORTED;
  if (c->precision == GPT_FP8 && (c->d_model % 16 || c->d_ff % 16 || c->vocab % 16 ||
                                  ((long)c->batch * c->seq_len) % 16))
    return GPT_ERR_SHAPE;
  if (c->ns_steps < 0 || c->ns_steps > 5 || c->ns_split_steps < 0) return GPT_ERR_ARG;
  if (c->fp8_gemms & ~(GPT_FP8_FWD | GPT_FP8_WGRAD | GPT_FP8_DGRAD)) return GPT_ERR_ARG;
  if (c->attn_window < 0) return GPT_ERR_ARG;
  if (c->n_kv_head < 0 || c->n_kv_head > c->n_head || c->n_head % kv_heads(*c) != 0) return GPT_ERR_SHAPE;
  if (c->extras & ~(kModelExtras | GPT_EXTRA_NORMUON)) return GPT_ERR_ARG;
  if ((c->extras & GPT_EXTRA_NORMUON) && !(c->normuon_beta2 >= 0.f && c->normuon_beta2 < 1.f)) return GPT_ERR_ARG;
  if ((c->extras & GPT_EXTRA_SMEAR) && c->d_model < kSmearCh) return GPT_ERR_SHAPE;
  if (!(c->norm_eps >= 0.f) || !(c->rope_base > 0.f) || !(c->init_std >= 0.f)) return GPT_ERR_ARG;
  return GPT_OK;
}

size_t gpt_state_bytes(const gpt_cfg* c) {
  if (gpt_cfg_validate(c) != GPT_OK) return 0;
  size_t total = 0;
  plan(*c, &total);
  return total;
}

size_t gpt_cfg_bytes(void) { return sizeof(gpt_cfg); }

int gpt_tensor_count(const gpt_cfg* c) {
  if (!c) return 0;
  return 2 + 6 * c->depth + (c->extras & kModelExtras ? 1 : 0) + (c->extras & GPT_EXTRA_VALUE_EMB ? c->depth + 1 : 0);
}

int gpt_tensor_shape(const gpt_cfg* c, int32_t id, int32_t* rows, int32_t* cols) {
  if (!c || !rows || !cols) return GPT_ERR_ARG;
  size_t off;
  int r, k;
  if (!tensor_loc(*c, id, &off, &r, &k)) return GPT_ERR_ARG;
  *rows = r;
  *cols = k;
  return GPT_OK;
}

const char* gpt_status_str(int s) {
  switch (s) {
    case GPT_OK: return "ok";
    case GPT_ERR_ARG: return "invalid argument";
    case GPT_ERR_SHAPE: return "shape mismatch";
    case GPT_ERR_TOKEN_RANGE: return "token id out of range";
    case GPT_ERR_NONFINITE: return "non-finite logits";
    case GPT_ERR_HIP: return "HIP runtime error";
    case GPT_ERR_UNSUPPORTED: return "unsupported configuration";
    default: return "unknown status";
  }
}

int gpt_last_status(const gpt_model* m) { return m ? m->last_status : GPT_ERR_ARG; }

static void refresh_act(gpt_model* M, hipStream_t st) {
  if (M->at != ACT_BF16) return;
  launch_cast_f32_to_act(M->blk(M->params()), M->wact(0), M->at, M->nBlk, st);
  launch_cast_f32_to_act(M->params() + M->nE + M->nBlk, M->uact(), M->at, M->nU, st);
}

static void free_side(gpt_model* M) {
  for (hipEvent_t* e : {&M->sev_fork, &M->sev_join, &M->sev_rd[0], &M->sev_rd[1], &M->sev_rd[2], &M->sev_rd[3],
                        &M->sev_rd[4]})
    if (*e) { (void)hipEventDestroy(*e); *e = nullptr; }
  if (M->side) { (void)hipStreamDestroy(M->side); M->side = nullptr; }
}

int gpt_init(const gpt_cfg* cfg, uint64_t seed, void* arena, size_t arena_bytes, void* stream, gpt_model** out) {
  if (!out) return GPT_ERR_ARG;
  *out = nullptr;
  int rc = gpt_cfg_validate(cfg);
  if (rc) return rc;
  if (!arena || ((uintptr_t)arena & 255)) return GPT_ERR_ARG;
  size_t need = 0;
  Offsets O = plan(*cfg, &need);
  if (arena_bytes < need) return GPT_ERR_ARG;
  gpt_model* M = new (std::nothrow) gpt_model();
  if (!M) return GPT_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  M->cfg = *cfg;
  M->off = O;
  M->base = (char*)arena;
  M->bytes = arena_bytes;
  M->at = act_of(*cfg);
  M->es = M->at == ACT_BF16 ? 2 : 4;
  M->fp8 = cfg->precision == GPT_FP8;
  M->xslot.assign(4 * cfg->depth + 1, -1);
  M->N = cfg->batch * cfg->seq_len;
  M->lo = layer_offs(*cfg);
  M->nE = (size_t)cfg->vocab * cfg->d_model;
  M->nU = M->nE;
  M->nBlk = (size_t)cfg->depth * M->lo.stride;
  M->nS = n_extras(*cfg);
  M->nT = n_tail(*cfg);
  const int L = cfg->depth, d = cfg->d_model, F = cfg->d_ff;
  for (int l = 0; l < L; ++l) {
    const size_t b = (size_t)l * M->lo.stride;
    const size_t o6[6] = {M->lo.q, M->lo.k, M->lo.v, M->lo.o, M->lo.w1, M->lo.w2};
    for (int j = 0; j < 6; ++j) {
      M->moff.push_back((long)(b + o6[j]));
      M->msize.push_back(j == 1 || j == 2 ? (long)kv_dim(*cfg) * d : j < 4 ? (long)d * d : (long)d * F);
      if (M->nm_roff.empty()) M->nm_roff.push_back(0);
      const long rows = j == 4 ? F : (j == 1 || j == 2) ? (long)kv_dim(*cfg) : d;  // output rows
      M->nm_roff.push_back(M->nm_roff.back() + rows);
    }
  }
  // weights: one counter-based stream per tensor id
  const int nt = 2 + 6 * L;
  for (int id = 0; id < nt; ++id) {
    size_t off;
    int r, c;
    tensor_loc(*cfg, id, &off, &r, &c);
    const int j = (id >= 1 && id <= 6 * L) ? (id - 1) % 6 : -1;
    const float sd = cfg->init_std * ((j == 3 || j == 5) ? 1.f / sqrtf(2.f * L) : 1.f);
    launch_fill_normal(M->params() + off, (size_t)r * c, seed, (uint64_t)id, sd, st);
  }
  if (M->nT) {  // S at the identity, value-embedding tables and gates at 0
    launch_zero(M->params() + M->nE + M->nBlk + M->nU, M->nT * 4, st);
    launch_extras_init(M->params() + M->nE + M->nBlk + M->nU, L, st);
  }
  launch_zero(M->at_off<float>(O.mom), M->nBlk * 4, st);
  launch_zero(M->at_off<float>(O.adam_m), (M->nE + M->nU + M->nT) * 4, st);
  launch_zero(M->at_off<float>(O.adam_v), (M->nE + M->nU + M->nT) * 4, st);
  launch_zero(M->at_off<float>(O.grads), (M->nE + M->nBlk + M->nU + M->nT) * 4, st);
  refresh_act(M, st);
  launch_rope_table(M->at_off<float>(O.rope), cfg->seq_len, cfg->head_dim, cfg->rope_base, st);
  if (cfg->extras & GPT_EXTRA_NORMUON) {
    launch_zero(M->at_off<float>(O.nm_v), (size_t)M->nm_roff.back() * 4, st);
    if (hipMemcpyAsync(M->at_off<long>(O.nm_roff), M->nm_roff.data(), M->nm_roff.size() * 8, hipMemcpyHostToDevice,
                       st) != hipSuccess) {
      delete M;
      return GPT_ERR_HIP;
    }
  }
  {
    const NsLayout nsl(*cfg);
    for (int l = 0; l < L; ++l)
      for (int j = 0; j < 6; ++j)
        if (!nsl.transposed(j)) {
          MuonVecJob jb;
          jb.src = M->moff[6 * l + j];
          jb.dst = (long)nsl.xdst(l, j);
          jb.wact = M->moff[6 * l + j];
          jb.n = (long)nsl.mrows(j) * nsl.mcols(j);
          jb.srow = M->nm_roff[6 * l + j];
          jb.mat = 6 * l + j;
          jb.cols = nsl.mcols(j);
          M->mv_jobs.push_back(jb);
        }
  }
  if (hipMemcpyAsync(M->at_off<MuonVecJob>(O.mv_jobs), M->mv_jobs.data(), M->mv_jobs.size() * sizeof(MuonVecJob),
                     hipMemcpyHostToDevice, st) != hipSuccess ||
      hipMemcpyAsync(M->at_off<long>(O.mat_off), M->moff.data(), M->moff.size() * 8, hipMemcpyHostToDevice, st) !=
          hipSuccess ||
      hipMemcpyAsync(M->at_off<long>(O.mat_size), M->msize.data(), M->msize.size() * 8, hipMemcpyHostToDevice,
                     st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    delete M;
    return GPT_ERR_HIP;
  }
  if (hipGetLastError() != hipSuccess) {
    delete M;
    return GPT_ERR_HIP;
  }
  // the side stream (default priority) and its events; without them every product stays on
  // the caller's stream
  bool side_ok = hipStreamCreateWithFlags(&M->side, hipStreamNonBlocking) == hipSuccess;
  for (hipEvent_t* e : {&M->sev_fork, &M->sev_join, &M->sev_rd[0], &M->sev_rd[1], &M->sev_rd[2], &M->sev_rd[3],
                        &M->sev_rd[4]})
    side_ok = side_ok && hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess;
  if (!side_ok) {
    (void)hipGetLastError();
    free_side(M);
  }
  {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
      auto tiles = [](long m, long n) { return ((m + 255) / 256) * ((n + 255) / 256); };
      const long Nt = M->N;  // the data gradients' rows: [N][d] (dm, do, da) and [N][F] (du)
      M->side_pays = tiles(Nt, cfg->d_model) % cus != 0 || tiles(Nt, cfg->d_ff) % cus != 0;
    } else {
      (void)hipGetLastError();
    }
  }
  *out = M;
  return GPT_OK;
}

void gpt_free(gpt_model* M) {
  if (!M) return;
  for (auto e : M->ev) (void)hipEventDestroy(e);
  free_side(M);
  delete M;
}

// Linear weights as GEMM operands: index w = 4l + {0: Wqkv [d + 2 kv_dim][d], 1: Wo, 2: W1, 3: W2}, w = 4L: U.
struct WInfo {
  size_t off;  // element offset inside the (blocks | U) part of the tensor table
  int rows, cols;
};
static WInfo winfo(const gpt_model* M, int w) {
  const gpt_cfg& c = M->cfg;
  if (w == 4 * c.depth) return {M->nBlk, c.vocab, c.d_model};
  const int l = w / 4, j = w % 4, d = c.d_model, F = c.d_ff;
  const size_t b = (size_t)l * M->lo.stride;
  switch (j) {
    case 0: return {b + M->lo.q, (int)qkv_dim(c), d};
    case 1: return {b + M->lo.o, d, d};
    case 2: return {b + M->lo.w1, F, d};
    default: return {b + M->lo.w2, d, F};
  }
}

// e4m3 copies (row-major and transposed) of every Linear weight with its own
// per-tensor scale, from the fp32 masters
static void quant_weights(gpt_model* M, hipStream_t st) {
  const Offsets& O = M->off;
  unsigned* amax = M->at_off<unsigned>(O.amax);
  float* wscale = M->at_off<float>(O.wscale);
  const float* master = M->params() + M->nE;  // blocks | U
  for (int w = 0; w <= 4 * M->cfg.depth; ++w) {
    const WInfo wi = winfo(M, w);
    const int slot = M->qslot++;
    launch_amax(master + wi.off, ACT_F32, wi.rows, wi.cols, wi.cols, amax + slot, st, M->at_off<float>(O.amax_part));
    launch_quant_e4m3(master + wi.off, ACT_F32, wi.rows, wi.cols, wi.cols, amax + slot,
                      M->at_off<uint8_t>(O.wq8) + wi.off, wi.cols, M->at_off<uint8_t>(O.wtq8) + wi.off, wi.rows,
                      wscale + w, st);
  }
  M->wq_dirty = false;
}

// quantise an activation-typed [rows][cols] tensor: q row-major and/or qt transposed
// the kept transposed e4m3 input of weight w (per layer a, o, m [d][N], g [F][N]; head r [d][N])
static uint8_t* xq8t_of(gpt_model* M, int w) {
  const size_t N = M->N, d = M->cfg.d_model, F = M->cfg.d_ff;
  const size_t l = w / 4, j = w % 4;
  return M->at_off<uint8_t>(M->off.xq8t) + l * N * (3 * d + F) + j * N * d;
}

// (slot >= 0: the tensor's amax is already in that slot, folded from its producer's partials)
static int quant_act(gpt_model* M, const void* x, int rows, int cols, long ldx, uint8_t* q, uint8_t* qt,
                     hipStream_t st, int slot = -1) {
  unsigned* amax = M->at_off<unsigned>(M->off.amax);
  if (slot < 0) {
    slot = M->qslot++;
    launch_amax(x, ACT_BF16, rows, cols, ldx, amax + slot, st, M->at_off<float>(M->off.amax_part));
  }
  launch_quant_e4m3(x, ACT_BF16, rows, cols, ldx, amax + slot, q, cols, qt, rows,
                    M->at_off<float>(M->off.qinv) + slot, st);
  return slot;
}

// Y = X W^T through weight w; p carries M, N (= rows of W), K, A/lda (X) and the epilogue
// (xslot >= 0: the quantisation slot already holding X's amax)
static int lin_fwd(gpt_model* M, GemmArgs p, int w, hipStream_t st, int xslot = -1) {
  const WInfo wi = winfo(M, w);
  if (!M->fp8 || !(M->cfg.fp8_gemms & GPT_FP8_FWD)) {
    p.B = w == 4 * M->cfg.depth ? M->uact() : M->wact(wi.off);
    p.ldb = wi.cols;
    return run_gemm(M, p, st, false);
  }
  uint8_t* q8a = M->at_off<uint8_t>(M->off.q8a);
  uint8_t* xt = keeps_xt(M->cfg) ? xq8t_of(M, w) : nullptr;
  const int sx = quant_act(M, p.A, p.M, p.K, p.lda, q8a, xt, st, xslot);
  M->xslot[w] = xt ? sx : -1;
  p.A = q8a; p.lda = p.K;
  p.B = M->at_off<uint8_t>(M->off.wq8) + wi.off; p.ldb = wi.cols;
  p.fp8 = true;
  p.dq_a = M->at_off<float>(M->off.qinv) + sx;
  p.dq_b = M->at_off<float>(M->off.wscale) + w;
  return run_gemm(M, p, st, false);
}

// buffers of the backward that weight-gradient products on the side stream read: the dY
// buffers (bf16 products) and the two transposed-dY code buffers (e4m3 products)
enum { RD_DH = 0, RD_DBIG = 1, RD_DQKV = 2, RD_Q8B = 3 };

// the main stream waits for the side stream's last reader of dY buffer rd (before it
// overwrites that buffer)
static int side_wait(gpt_model* M, int rd, hipStream_t st) {
  if (rd < 0 || !M->sev_pending[rd]) return GPT_OK;
  M->sev_pending[rd] = false;
  return hipStreamWaitEvent(st, M->sev_rd[rd], 0) == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

// backward of Y = X W^T: dW = dY^T X into dW (ld = cols of W) and dX = dY W with the
// epilogue in pd (M = tokens, N = cols of W, K = rows of W, outputs set by the caller).
// rd >= 0: dY is that buffer and dW goes to the side stream (when the step uses it); wr >= 0:
// dX overwrites that buffer, so the side stream's last reader of it must be done first
static int lin_bwd(gpt_model* M, const void* dY, long ldy, const void* X, long ldx, int w, float* dW, GemmArgs pd,
                   hipStream_t st, int yslot = -1, int rd = -1, int wr = -1) {
  const WInfo wi = winfo(M, w);
  const int N = M->N, nout = wi.rows, kin = wi.cols;
  int rc;
  GemmArgs pw;
  pw.M = nout; pw.N = kin; pw.K = N;
  pw.outF = dW; pw.ldo = kin;
  if (M->acc_grads) { pw.Cin = dW; pw.ldcin = kin; pw.beta = 1.f; }  // dW += dY^T X (same thread reads and writes)
  const bool f8w = M->fp8 && (M->cfg.fp8_gemms & GPT_FP8_WGRAD);
  const bool f8d = M->fp8 && (M->cfg.fp8_gemms & GPT_FP8_DGRAD);
  uint8_t* q8a = M->at_off<uint8_t>(M->off.q8a);
  uint8_t* q8b = M->at_off<uint8_t>(M->off.q8b);
  uint8_t* q8c = M->at_off<uint8_t>(M->off.q8c);
  const float* qinv = M->at_off<float>(M->off.qinv);
  const bool side = rd >= 0 && M->use_side;
  // the buffer the side stream's weight gradient reads: its transposed dY codes (e4m3),
  // alternating between two buffers, else dY itself
  int rbuf = rd;
  if (side && f8w) {
    rbuf = RD_Q8B + M->q8b_cur;
    if (M->q8b_cur) q8b = M->at_off<uint8_t>(M->off.q8b2);
    M->q8b_cur ^= 1;
    if ((rc = side_wait(M, rbuf, st))) return rc;  // its previous reader is done
  }
  const int sy =
      (f8w || f8d) ? quant_act(M, dY, N, nout, ldy, f8d ? q8a : nullptr, f8w ? q8b : nullptr, st, yslot) : 0;
  if (f8w) {
    // X^T: kept from the forward (the same tensor, so the same scale and codes), else quantised here
    const bool kept = M->xslot[w] >= 0;
    if (keeps_xt(M->cfg) && !kept) return GPT_ERR_ARG;  // the forward of this step did not run
    uint8_t* xt = kept ? xq8t_of(M, w) : q8c;
    const int sx = kept ? M->xslot[w] : quant_act(M, X, N, kin, ldx, nullptr, q8c, st);
    pw.A = q8b; pw.lda = N; pw.B = xt; pw.ldb = N;  // dY^T and X^T, reduction over tokens
    pw.fp8 = true; pw.dq_a = qinv + sy; pw.dq_b = qinv + sx;
  } else {
    pw.A = dY; pw.lda = ldy; pw.a_kmaj = false;
    pw.B = X; pw.ldb = ldx; pw.b_kmaj = false;
  }
  if (side) {  // dY (or its codes) and X are ready on the main stream
    if (hipEventRecord(M->sev_fork, st) != hipSuccess || hipStreamWaitEvent(M->side, M->sev_fork, 0) != hipSuccess)
      return GPT_ERR_HIP;
    if ((rc = run_gemm(M, pw, M->side, true))) return rc;
    if (hipEventRecord(M->sev_rd[rbuf], M->side) != hipSuccess) return GPT_ERR_HIP;
    M->sev_pending[rbuf] = true;
  } else if ((rc = run_gemm(M, pw, st, true))) {
    return rc;
  }
  if ((rc = side_wait(M, wr, st))) return rc;
  if (f8d) {
    pd.A = q8a; pd.lda = nout;
    pd.B = M->at_off<uint8_t>(M->off.wtq8) + wi.off; pd.ldb = nout;
    pd.fp8 = true; pd.dq_a = qinv + sy; pd.dq_b = M->at_off<float>(M->off.wscale) + w;
  } else {
    pd.A = dY; pd.lda = ldy;
    pd.B = w == 4 * M->cfg.depth ? M->uact() : M->wact(wi.off); pd.ldb = kin; pd.b_kmaj = false;
  }
  // split-K where the reduction is long (the LM head's, over the vocabulary): at d = 768 its
  // 384 output tiles are 1.5 rounds of 256 workgroups, two splits make them 3 rounds of half
  // the length.  Short reductions never gain enough to pay for the extra reduction launch.
  return run_gemm(M, pd, st, pd.K >= 8192);
}

static int forward_backward_on(gpt_model* M, const int32_t* tok, const int32_t* tgt, float grad_scale,
                               hipStream_t st) {
  const gpt_cfg& c = M->cfg;
  const int N = M->N, d = c.d_model, F = c.d_ff, V = c.vocab, L = c.depth, H = c.n_head, hd = c.head_dim;
  const int Hkv = kv_heads(c), QD = (int)qkv_dim(c);  // key/value heads, fused QKV width
  const int B = c.batch, T = c.seq_len;
  const int at = M->at;
  const size_t es = M->es;
  const Offsets& O = M->off;
  float* hs = M->at_off<float>(O.hs);
  float* grads = M->grads();
  float* gblk = M->blk(grads);
  int* err = M->at_off<int>(O.err);
  const float eps = c.norm_eps;
  auto actp = [&](size_t o, size_t elems) -> void* { return M->base + o + elems * es; };
  auto hsl = [&](int i) { return hs + (size_t)i * N * d; };
  int rc;
  // extras: S on the device, and the buffers they need
  const bool ex_resid = c.extras & GPT_EXTRA_RESID, ex_smear = c.extras & GPT_EXTRA_SMEAR,
             ex_back = c.extras & GPT_EXTRA_BACKOUT, ex_ve = c.extras & GPT_EXTRA_VALUE_EMB;
  // value embeddings: layer l's table and gate weights (parameters) and gate values
  const size_t ve_base = M->nE + M->nBlk + M->nU + s_region(c), kvd = kv_dim(c);
  auto ve_tab = [&](float* region, int l) { return region + ve_base + (size_t)l * V * kvd; };
  auto ve_gate = [&](float* region, int l) { return region + ve_base + n_ve(c) + (size_t)l * Hkv * kVeCh; };
  auto ve_g = [&](int l) { return M->at_off<float>(O.vg) + (size_t)l * N * Hkv; };
  const float* S = M->params() + M->nE + M->nBlk + M->nU;
  const int Lb = L / 2;  // backout reads the stream entering this layer
  float* xpart = M->at_off<float>(O.xpart);  // [2L+26][N] per-row terms of dS
  // the stream layer l adds its blocks to (its mixed input under residual scaling)
  auto xres = [&](int l) { return ex_resid ? M->at_off<float>(O.hx) + (size_t)l * N * d : hsl(2 * l); };
  // gpt_capture: copies of one layer's Linear operands and results, for stage-isolated checks
  bool cap_failed = false;
  auto cap = [&](int layer, int slot, const void* src) {
    if (!M->cap_buf || layer != M->cap_layer) return;
    const size_t bytes = capture_sizes(c, layer)[slot];
    if (hipMemcpyAsync(M->cap_buf + capture_offset(c, layer, slot), src, bytes, hipMemcpyDeviceToDevice, st) !=
        hipSuccess)
      cap_failed = true;
  };

  // fp8: the producers of quantised tensors write per-wave amax partials (fpart), folded
  // into the tensor's quantisation slot, so that its quantisation reads it only once
  const bool fuse = M->fp8 && g_fp8_fused_amax && c.extras == 0 && (c.fp8_gemms & GPT_FP8_FWD) &&
                    (c.fp8_gemms & GPT_FP8_DGRAD) && (c.fp8_gemms & GPT_FP8_WGRAD);
  float* fpart = fuse ? M->at_off<float>(O.amax_fuse) : nullptr;
  const long fcap = fuse ? (long)kFuseParts(c) : 0;
  auto fold = [&](int n) -> int {  // the slot of a tensor whose producer wrote n partials; -1: none
    if (n <= 0) return -1;
    const int slot = M->qslot++;
    launch_amax_fold(fpart, n, M->at_off<unsigned>(O.amax) + slot, st);
    return slot;
  };

  launch_zero(err, 16, st);
  if (M->fp8) {
    M->qslot = 0;
    launch_zero(M->base + O.amax, kQuantSlots(c) * 4, st);
    if (M->wq_dirty) quant_weights(M, st);
    else M->qslot = 4 * L + 1;
  }
  if (ex_smear) {
    float* emb = M->at_off<float>(O.emb);
    launch_embed_gather(tok, M->params(), emb, N, d, V, err, st);
    launch_smear_fwd(emb, S + s_ls(c), S + s_ws(c), hsl(0), N, T, d, st);
  } else {
    launch_embed_gather(tok, M->params(), hsl(0), N, d, V, err, st);
  }
  for (int l = 0; l < L; ++l) {
    void* a = actp(O.a, (size_t)l * N * d);
    void* qkv = actp(O.qkv, (size_t)l * N * QD);
    void* o = actp(O.o, (size_t)l * N * d);
    void* m = actp(O.m, (size_t)l * N * d);
    void* g = actp(O.g, (size_t)l * N * F);
    float* rq = M->at_off<float>(O.rq) + (size_t)l * N * H;
    float* rk = M->at_off<float>(O.rk) + (size_t)l * N * Hkv;
    float* lse = M->at_off<float>(O.lse) + (size_t)l * B * H * T;
    int sa = -1;     // quantisation slots with the amax already folded (fp8 steps), else -1
    if (ex_resid)  // layer input lr x + l0 x0
      launch_mix_rmsnorm_fwd(hsl(2 * l), hsl(0), S + s_lr(c, l), 1.f, S + s_l0(c, l), 1.f, xres(l), a, at,
                             M->at_off<float>(O.rstd_a) + (size_t)l * N, N, d, eps, st);
    else
      sa = fold(launch_rmsnorm_fwd(hsl(2 * l), a, at, M->at_off<float>(O.rstd_a) + (size_t)l * N, N, d, eps, st,
                                   fpart, fcap));
    cap(l, CAP_A, a);
    cap(l, CAP_HIN, xres(l));
    {
      GemmArgs p;  // qkv = a Wqkv^T
      p.M = N; p.N = QD; p.K = d; p.A = a; p.lda = d;
      p.outA = qkv; p.ldoa = QD;
      if ((rc = lin_fwd(M, p, 4 * l + 0, st, sa))) return rc;
    }
    cap(l, CAP_QKV, qkv);
    if (ex_ve)  // v += 3 sigmoid(gate) VE[token]
      launch_ve_fwd(qkv, at, a, tok, ve_tab(M->params(), l), ve_gate(M->params(), l), ve_g(l), N, V, H, Hkv, hd, d,
                    st);
    launch_rope_qknorm_fwd(qkv, at, M->at_off<float>(O.rope), rq, rk, B, T, H, Hkv, hd, eps, st);
    // q and k leave the QK-norm RMS-normalised per head: the forward takes its fixed reference
    const int so = fold(launch_attn_fwd(qkv, o, lse, at, B, T, H, Hkv, hd, c.attn_window, st, fpart, fcap, true));
    cap(l, CAP_O, o);
    {
      GemmArgs p;  // h' = h + o Wo^T
      p.M = N; p.N = d; p.K = d; p.A = o; p.lda = d;
      p.Cin = xres(l); p.ldcin = d; p.beta = 1.f;
      p.outF = hsl(2 * l + 1); p.ldo = d;
      if ((rc = lin_fwd(M, p, 4 * l + 1, st, so))) return rc;
    }
    cap(l, CAP_H1, hsl(2 * l + 1));
    const int sm = fold(launch_rmsnorm_fwd(hsl(2 * l + 1), m, at, M->at_off<float>(O.rstd_m) + (size_t)l * N, N, d,
                                           eps, st, fpart, fcap));
    cap(l, CAP_M, m);
    {
      GemmArgs p;  // g = relu(m W1^T)^2 (the pre-activation itself is not kept: relu(u) = sqrt(g))
      p.M = N; p.N = F; p.K = d; p.A = m; p.lda = d;
      p.epi = EPI_RELU2; p.out2 = g; p.ldoa = F;
      p.amax_part = fpart;
      M->gemm_parts = 0;
      if ((rc = lin_fwd(M, p, 4 * l + 2, st, sm))) return rc;
    }
    const int sg = fold(M->gemm_parts);
    cap(l, CAP_G, g);
    {
      GemmArgs p;  // h'' = h' + g W2^T
      p.M = N; p.N = d; p.K = F; p.A = g; p.lda = F;
      p.Cin = hsl(2 * l + 1); p.ldcin = d; p.beta = 1.f;
      p.outF = hsl(2 * l + 2); p.ldo = d;
      if ((rc = lin_fwd(M, p, 4 * l + 3, st, sg))) return rc;
    }
    cap(l, CAP_H2, hsl(2 * l + 2));
  }
  void* r = M->base + O.r;
  int sr = -1;
  if (ex_back)  // the final norm reads x_L - lb x_mid
    launch_mix_rmsnorm_fwd(hsl(2 * L), hsl(2 * Lb), nullptr, 1.f, S + s_lb(c), -1.f, M->at_off<float>(O.hfin), r, at,
                           M->at_off<float>(O.rstd_f), N, d, eps, st);
  else
    sr = fold(launch_rmsnorm_fwd(hsl(2 * L), r, at, M->at_off<float>(O.rstd_f), N, d, eps, st, fpart, fcap));
  cap(L, CAP_R, r);
  float* logits = M->at_off<float>(O.logits);
  void* dlogits = M->base + O.dlogits;
  {
    GemmArgs p;  // logits = r U^T
    p.M = N; p.N = V; p.K = d; p.A = r; p.lda = d;
    p.outF = logits; p.ldo = V;
    if ((rc = lin_fwd(M, p, 4 * L, st, sr))) return rc;
  }
  cap(L, CAP_LOGITS, logits);
  // the whole backward is linear in dlogits: grad_scale / N there scales every gradient
  const int sz = fold(launch_cross_entropy(logits, tgt, dlogits, at, M->at_off<float>(O.row_loss),
                                           M->at_off<int32_t>(O.argmax), N, V, grad_scale / (float)N, err, st, fpart,
                                           fcap));
  launch_sum_rows(M->at_off<float>(O.row_loss), N, M->at_off<double>(O.loss), st);
  cap(L, CAP_DLOGITS, dlogits);

  // ---------------- backward
  float* dtmp = M->at_off<float>(O.dtmp);
  float* dh[2] = {M->at_off<float>(O.dh0), M->at_off<float>(O.dh1)};
  void* dh_act = M->base + O.dh_act;
  void* dbig = M->base + O.dbig;
  void* dqkv = M->base + O.dqkv;
  void* do_act = M->base + O.do_act;
  {
    GemmArgs pd;  // dU = dz^T r ; dr = dz U
    pd.M = N; pd.N = d; pd.K = V;
    pd.outF = dtmp; pd.ldo = d;
    if ((rc = lin_bwd(M, dlogits, V, r, d, 4 * L, grads + M->nE + M->nBlk, pd, st, sz))) return rc;
  }
  cap(L, CAP_DR, dtmp);
  float* dmid = M->at_off<float>(O.dmid);  // d loss / d x_mid through the backout term
  float* dx0 = M->at_off<float>(O.dx0);    // d loss / d x0 through the l0 terms of layers 1..L-1
  if (ex_back) {
    launch_zero(dmid, (size_t)N * d * 4, st);
    launch_rmsnorm_mix_bwd(dtmp, M->at_off<float>(O.hfin), M->at_off<float>(O.rstd_f), nullptr, nullptr, 1.f,
                           S + s_lb(c), -1.f, false, nullptr, nullptr, dmid, hsl(2 * Lb),
                           xpart + (size_t)s_lb(c) * N, -1.f, nullptr, nullptr, 0.f, dh[0], dh_act, at, N, d, st);
  }
  int sdh = -1;  // slot of the output gradient entering the next block's W2 (dh_act)
  if (!ex_back)
    sdh = fold(launch_rmsnorm_bwd(dtmp, hsl(2 * L), M->at_off<float>(O.rstd_f), nullptr, dh[0], dh_act, at, N, d, eps,
                                  st, fpart, fcap, r));  // the norm's stored output r stands in for x rstd
  if (ex_resid) launch_zero(dx0, (size_t)N * d * 4, st);
  if (ex_ve) launch_embed_sort(tok, N, V, M->base + O.embws, st);  // shared by every scatter below
  int cur = 0;
  for (int l = L - 1; l >= 0; --l) {
    const size_t wl = (size_t)l * M->lo.stride;
    void* a = actp(O.a, (size_t)l * N * d);
    void* qkv = actp(O.qkv, (size_t)l * N * QD);
    void* o = actp(O.o, (size_t)l * N * d);
    void* m = actp(O.m, (size_t)l * N * d);
    void* g = actp(O.g, (size_t)l * N * F);
    float* rq = M->at_off<float>(O.rq) + (size_t)l * N * H;
    float* rk = M->at_off<float>(O.rk) + (size_t)l * N * Hkv;
    float* lse = M->at_off<float>(O.lse) + (size_t)l * B * H * T;
    cap(l, CAP_DY2, dh_act);
    {
      GemmArgs pd;  // dW2 = dY^T g ; du = (dY W2) * 2 relu(u), relu(u) = sqrt(g)
      pd.M = N; pd.N = F; pd.K = d;
      pd.epi = EPI_DRELU2; pd.aux = g; pd.outA = dbig; pd.ldoa = F;
      pd.amax_part = fpart;
      M->gemm_parts = 0;
      if ((rc = lin_bwd(M, dh_act, d, g, F, 4 * l + 3, gblk + wl + M->lo.w2, pd, st, sdh, RD_DH, RD_DBIG))) return rc;
    }
    const int su = fold(M->gemm_parts);
    cap(l, CAP_DU, dbig);
    {
      GemmArgs pd;  // dW1 = du^T m ; dm = du W1
      pd.M = N; pd.N = d; pd.K = F;
      pd.outF = dtmp; pd.ldo = d;
      if ((rc = lin_bwd(M, dbig, F, m, d, 4 * l + 2, gblk + wl + M->lo.w1, pd, st, su, RD_DBIG))) return rc;
    }
    cap(l, CAP_DM, dtmp);
    if ((rc = side_wait(M, RD_DH, st))) return rc;  // dh_act is rewritten here
    const int sdo = fold(launch_rmsnorm_bwd(dtmp, hsl(2 * l + 1), M->at_off<float>(O.rstd_m) + (size_t)l * N, dh[cur],
                                            dh[cur ^ 1], dh_act, at, N, d, eps, st, fpart, fcap, m));
    cur ^= 1;
    cap(l, CAP_DYO, dh_act);
    {
      GemmArgs pd;  // dWo = dY^T o ; do = dY Wo
      pd.M = N; pd.N = d; pd.K = d;
      pd.outA = do_act; pd.ldoa = d;
      if ((rc = lin_bwd(M, dh_act, d, o, d, 4 * l + 1, gblk + wl + M->lo.o, pd, st, sdo, RD_DH))) return rc;
    }
    cap(l, CAP_DO, do_act);
    // dqkv's partials: the dV waves first, then the RoPE backward's (dQ, dK)
    if ((rc = side_wait(M, RD_DQKV, st))) return rc;  // dqkv is rewritten here
    const int nq1 = launch_attn_bwd(qkv, o, do_act, lse, M->at_off<float>(O.Dbuf), dqkv, at, B, T, H, Hkv, hd,
                                    c.attn_window, st, fpart, fcap);
    if (ex_ve)  // dVE rows, the gate's dz and the rows of d(gate weights), from dv
      launch_ve_bwd(dqkv, at, a, tok, ve_tab(M->params(), l), ve_g(l), M->at_off<float>(O.dve),
                    M->at_off<float>(O.vdz), M->at_off<float>(O.vpart), N, V, H, Hkv, hd, d, st);
    const int nq2 = launch_rope_qknorm_bwd(dqkv, qkv, at, M->at_off<float>(O.rope), rq, rk, B, T, H, Hkv, hd, st,
                                           nq1 > 0 ? fpart + nq1 : nullptr, fcap - nq1);
    const int sq = nq1 > 0 && nq2 > 0 ? fold(nq1 + nq2) : -1;
    cap(l, CAP_DQKV, dqkv);
    {
      GemmArgs pd;  // dWqkv = dqkv^T a ; da = dqkv Wqkv
      pd.M = N; pd.N = d; pd.K = QD;
      pd.outF = dtmp; pd.ldo = d;
      if ((rc = lin_bwd(M, dqkv, QD, a, d, 4 * l + 0, gblk + wl + M->lo.q, pd, st, sq, RD_DQKV))) return rc;
    }
    cap(l, CAP_DA, dtmp);
    if ((rc = side_wait(M, RD_DH, st))) return rc;  // the layer's input gradient rewrites dh_act below
    if (ex_ve) {  // the gate's path into the block input; the table's and gates' gradients
      launch_ve_da(dtmp, M->at_off<float>(O.vdz), ve_gate(M->params(), l), N, Hkv, d, st);
      launch_embed_scatter_sorted(tok, M->at_off<float>(O.dve), ve_tab(grads, l), N, V, (int)kvd, M->base + O.embws,
                                  st, M->acc_grads);
      launch_colsum(M->at_off<float>(O.vpart), N, Hkv * kVeCh, M->base + O.vred, ve_gate(grads, l), M->acc_grads, st);
    }
    if (ex_resid || (ex_back && l == Lb)) {
      // g = d loss / d (layer input); the stream reaching the layer gets lr g (plus the
      // backout's x_mid term at layer L/2), x0 collects l0 g (layer 0: added to its own
      // stream, which is x0, together with the other layers' sum)
      launch_rmsnorm_mix_bwd(dtmp, xres(l), M->at_off<float>(O.rstd_a) + (size_t)l * N, dh[cur],
                             ex_resid ? S + s_lr(c, l) : nullptr, 1.f, ex_resid ? S + s_l0(c, l) : nullptr,
                             ex_resid ? 1.f : 0.f, l == 0, ex_back && l == Lb ? dmid : nullptr,
                             ex_resid && l == 0 ? dx0 : nullptr, ex_resid && l > 0 ? dx0 : nullptr,
                             ex_resid ? hsl(2 * l) : nullptr, xpart + (size_t)s_lr(c, l) * N, 1.f,
                             ex_resid ? hsl(0) : nullptr, xpart + (size_t)s_l0(c, l) * N, 1.f, dh[cur ^ 1], dh_act,
                             at, N, d, st);
      sdh = -1;
    } else {  // (layer 0's output feeds the embedding, no Linear: no partials)
      sdh = fold(launch_rmsnorm_bwd(dtmp, hsl(2 * l), M->at_off<float>(O.rstd_a) + (size_t)l * N, dh[cur],
                                    dh[cur ^ 1], dh_act, at, N, d, eps, st, l > 0 ? fpart : nullptr, fcap, a));
    }
    cur ^= 1;
  }
  if (ex_smear) {  // back through x = e + gate * previous e
    launch_smear_bwd(dh[cur], M->at_off<float>(O.emb), S + s_ls(c), S + s_ws(c), dh[cur ^ 1],
                     xpart + (size_t)s_ls(c) * N, xpart + (size_t)s_ws(c) * N, N, T, d, st);
    cur ^= 1;
  }
  if (ex_ve)
    launch_embed_scatter_sorted(tok, dh[cur], grads, N, V, d, M->base + O.embws, st, M->acc_grads);
  else
    launch_embed_scatter(tok, dh[cur], grads, N, V, d, M->base + O.embws, nullptr, st, M->acc_grads);
  if (c.extras)
    launch_extras_reduce(xpart, N, L, c.extras, grads + M->nE + M->nBlk + M->nU, M->acc_grads, st);
  return cap_failed ? GPT_ERR_HIP : GPT_OK;
}

// one forward + backward on stream st; the side stream (weight gradients) joins st before
// this returns, on every path
static int forward_backward(gpt_model* M, const int32_t* tok, const int32_t* tgt, float grad_scale, hipStream_t st) {
  // fp8 steps whose weight gradients quantise X themselves share that scratch (q8c) between
  // Linears: one stream for them
  M->use_side = g_side_stream && M->side && (!M->fp8 || keeps_xt(M->cfg)) && (M->side_pays || g_side_stream == 2);
  M->q8b_cur = 0;
  for (bool& b : M->sev_pending) b = false;
  int rc = forward_backward_on(M, tok, tgt, grad_scale, st);
  if (M->use_side) {
    if (hipEventRecord(M->sev_join, M->side) != hipSuccess || hipStreamWaitEvent(st, M->sev_join, 0) != hipSuccess)
      rc = rc ? rc : GPT_ERR_HIP;
    for (bool& b : M->sev_pending) b = false;
  }
  return rc;
}

float gpt_step(gpt_model* M, const int32_t* tok, const int32_t* tgt, const gpt_cfg* cfg, void* stream) {
  return gpt_step_accumulate(M, tok, tgt, cfg, 0, 1.f, stream);
}

int gpt_step_async(gpt_model* M, const int32_t* tok, const int32_t* tgt, const gpt_cfg* cfg, int32_t accumulate,
                   float grad_scale, void* stream) {
  if (!M) return GPT_ERR_ARG;
  if (!tok || !tgt || !std::isfinite(grad_scale)) return M->last_status = GPT_ERR_ARG;
  if (cfg && !same_shape(*cfg, M->cfg)) return M->last_status = GPT_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;
  M->acc_grads = accumulate != 0;
  int rc = forward_backward(M, tok, tgt, grad_scale, st);
  M->acc_grads = false;
  if (!rc && hipGetLastError() != hipSuccess) rc = GPT_ERR_HIP;
  if (rc) return M->last_status = rc;
  M->stepped = true;
  return M->last_status = GPT_OK;
}

float gpt_step_result(gpt_model* M, void* stream) {
  if (!M) return NAN;
  if (!M->stepped) { M->last_status = GPT_ERR_ARG; return NAN; }
  hipStream_t st = (hipStream_t)stream;
  struct { double loss; int err[4]; } h;
  if (hipMemcpyAsync(&h.loss, M->base + M->off.loss, 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(h.err, M->base + M->off.err, 16, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    M->last_status = GPT_ERR_HIP;
    return NAN;
  }
  if (h.err[0] & 1) { M->last_status = GPT_ERR_TOKEN_RANGE; return NAN; }
  if (h.err[0] & 2) { M->last_status = GPT_ERR_NONFINITE; return NAN; }
  M->last_status = GPT_OK;
  return (float)(h.loss / (double)M->N);
}

float gpt_step_accumulate(gpt_model* M, const int32_t* tok, const int32_t* tgt, const gpt_cfg* cfg,
                          int32_t accumulate, float grad_scale, void* stream) {
  if (!M) return NAN;
  if (gpt_step_async(M, tok, tgt, cfg, accumulate, grad_scale, stream) != GPT_OK) return NAN;
  return gpt_step_result(M, stream);
}

int adamw_update(gpt_model* M, float lr, float beta1, float beta2, float eps, float weight_decay, void* stream) {
  if (!M) return GPT_ERR_ARG;
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) || !(eps >= 0.f) || !std::isfinite(eps) ||
      !std::isfinite(lr) || !std::isfinite(weight_decay))
    return GPT_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  const long t = ++M->adam_t;
  const float rbc1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)t)));
  const float rbc2 = (float)(1.0 / (1.0 - std::pow((double)beta2, (double)t)));
  float* m = M->at_off<float>(M->off.adam_m);
  float* v = M->at_off<float>(M->off.adam_v);
  const size_t uo = M->nE + M->nBlk;  // U's offset in the parameter and gradient tables
  launch_adamw(M->params(), M->grads(), m, v, nullptr, M->at, M->nE, lr, beta1, beta2, eps, weight_decay, rbc1, rbc2,
               st);
  launch_adamw(M->params() + uo, M->grads() + uo, m + M->nE, v + M->nE, M->at == ACT_BF16 ? M->uact() : nullptr, M->at,
               M->nU, lr, beta1, beta2, eps, weight_decay, rbc1, rbc2, st);
  if (M->nT)  // the extras' scalars and value embeddings follow U in every table
    launch_adamw(M->params() + uo + M->nU, M->grads() + uo + M->nU, m + M->nE + M->nU, v + M->nE + M->nU, nullptr,
                 ACT_F32, M->nT, lr, beta1, beta2, eps, weight_decay, rbc1, rbc2, st);
  M->wq_dirty = true;  // the e4m3 copies of U follow the master weights
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

extern "C++" {
// The Newton-Schulz iterations on a batch of nb matrices X [s][l] (wide orientation)
// stored one after another from element offset off: A = X X^T, B = b A + c A A, X <- a X
// + B X, every product on MFMA with operands of type nat (fp16 by default; bf16 with hi /
// lo planes in the first nsplit iterations; fp32 for the all-fp32 configuration) and fp32
// accumulation, X carried in fp32 (xf; with fp16 operands only through the first
// kNsF32Carry iterations and for the result) and as operand planes (xa, xl, ping-ponged).
struct NsBuffers {
  float* xf;
  char* xa[2];
  char* xl[2];
  size_t es;
  float* Af;
  void *Aa, *Ba, *Alo, *Blo;
};
// Iterations that carry X in fp32 for the a X term before the fp16-operand schedule carries
// it in X's fp16 plane.  The first iterations' large a (the pages' Polar-Express
// coefficients start near 8) lifts the small singular directions of a low-rank-plus-noise
// momentum from magnitudes where fp16 loses them; an fp16 carry from the first iteration
// on moved such a case 3.6e-2 (relative L2, 1536 x 1536, in a numpy model of the
// iteration), from the third on 2.2e-3 against 1.2e-3 for fp32 throughout, and Gaussian
// momenta not at all (1.3e-3 against 1.7e-3).
constexpr int kNsF32Carry = 2;

template <typename Run>
static int ns_iterate(int nat, int nsplit, int steps, const float (*coeffs)[3], int s, int l, int nb_, size_t off,
                      const NsBuffers& nb, Run&& run) {
  int cur = 0, rc;
  const long ss = (long)s * s, sl = (long)s * l;
  const size_t es = nb.es;
  for (int it = 0; it < steps; ++it) {
    const float a = coeffs[it][0], b = coeffs[it][1], cc = coeffs[it][2];
    const bool sp = it < nsplit;           // this iteration multiplies hi/lo planes
    const bool next_sp = it + 1 < nsplit;  // the next one needs X's lo plane
    const void* xh = nb.xa[cur] + off * es;
    const void* xlo = nb.xl[cur] ? nb.xl[cur] + off * es : nullptr;
    {
      GemmArgs p;  // A = X X^T
      p.sym = true;
      p.dtype = nat;
      p.M = s; p.N = s; p.K = l; p.batch = nb_;
      p.A = xh; p.lda = l; p.strideA = sl;
      p.B = xh; p.ldb = l; p.strideB = sl;
      if (nat != ACT_F16) { p.outF = nb.Af; p.ldo = s; p.strideO = ss; }  // fp16: the b A term reads Aa
      p.outA = nb.Aa; p.ldoa = s; p.strideOA = ss;
      if (sp) p.outA_lo = nb.Alo;
      if ((rc = run(p))) return rc;
    }
    {
      GemmArgs p;  // Bm = b A + c A A   (A symmetric)
      p.sym = true;
      p.dtype = nat;
      p.split = sp; p.A_lo = nb.Alo; p.B_lo = nb.Alo;
      p.M = s; p.N = s; p.K = s; p.batch = nb_;
      p.A = nb.Aa; p.lda = s; p.strideA = ss;
      p.B = nb.Aa; p.ldb = s; p.strideB = ss;
      p.alpha = cc; p.beta = b; p.ldcin = s; p.strideCin = ss;
      if (nat == ACT_F16) p.CinA = nb.Aa;
      else p.Cin = nb.Af;
      p.outA = nb.Ba; p.ldoa = s; p.strideOA = ss;
      if (sp) p.outA_lo = nb.Blo;
      if ((rc = run(p))) return rc;
    }
    {
      GemmArgs p;  // X <- a X + Bm X   (fp32 X read and written by the same thread)
      p.dtype = nat;
      p.split = sp; p.A_lo = nb.Blo; p.B_lo = xlo;
      p.M = s; p.N = l; p.K = s; p.batch = nb_;
      p.A = nb.Ba; p.lda = s; p.strideA = ss;
      p.B = xh; p.ldb = l; p.strideB = sl; p.b_kmaj = false;
      p.beta = a; p.ldcin = l; p.strideCin = sl;
      // the a X term: X in fp32 through the first kNsF32Carry iterations, then (fp16
      // operands) from X's fp16 plane, which the product reads anyway
      const bool f16carry = nat == ACT_F16 && it >= kNsF32Carry;
      const bool next_f16carry = nat == ACT_F16 && it + 1 >= kNsF32Carry;
      if (f16carry) p.CinA = xh;
      else p.Cin = nb.xf + off;
      // the fp32 X only where it is read: by the next iteration's a X term, or as the result
      if (it + 1 == steps || !next_f16carry) { p.outF = nb.xf + off; p.ldo = l; p.strideO = sl; }
      if (it + 1 < steps) {  // the operand planes of the next iteration (the last X is read in fp32 only)
        p.outA = nb.xa[cur ^ 1] + off * es; p.ldoa = l; p.strideOA = sl;
        if (next_sp) p.outA_lo = nb.xl[cur ^ 1] + off * es;
      }
      if ((rc = run(p))) return rc;
    }
    cur ^= 1;
  }
  return GPT_OK;
}
}  // extern "C++"

int muon_update(gpt_model* M, float lr, void* stream) {
  if (!M) return GPT_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  const gpt_cfg& c = M->cfg;
  const Offsets& O = M->off;
  const int L = c.depth, d = c.d_model, F = c.d_ff;
  const int s = std::min(d, F), lw = std::max(d, F);
  float* mom = M->at_off<float>(O.mom);
  float* xf = M->at_off<float>(O.xf);
  char* xa[2] = {M->base + O.xa0, M->base + O.xa1};
  char* xl[2] = {M->base + O.xl0, M->base + O.xl1};
  // 16-bit precisions: by default every product takes fp16 operands (11 significant
  // bits, the bf16 MFMA rate; X, A and B stay well inside fp16's range), with X carried
  // in fp32 for the a X term of the first kNsF32Carry iterations (an fp16 carry from the
  // start loses the small entries of low-rank-plus-noise momenta to fp16's subnormals),
  // from its fp16 plane after them, and the b A term read from A's fp16 plane (as accurate
  // as an fp32 A in a numpy model of the iteration, and 4 bytes per element less).  With ns_split_steps > 0 the products run on bf16 MFMA
  // instead, and the leading iterations multiply A A and B X with operands carried as
  // bf16 hi + lo planes (three MFMA products each): rounding errors of the early
  // iterations are amplified by the later ones along small singular directions, those
  // of the last are not.  The Gram product X X^T then stays plain bf16 in every
  // iteration (its fp32 result still feeds the split A A as hi + lo planes)
  const int nsplit = M->at == ACT_BF16 ? std::min(c.ns_split_steps, c.ns_steps) : 0;
  const int nat = M->at == ACT_BF16 && c.ns_split_steps == 0 ? ACT_F16 : M->at;  // NS operand type
  const size_t es = M->es;
  // the matrix table covers the blocks region, so this is the momentum of every block
  // matrix; offsets relative to the region (mom, and the gradients' blocks)
  launch_momentum_sumsq(mom, M->blk(M->grads()), c.muon_momentum, M->at_off<long>(O.mat_off),
                        M->at_off<long>(O.mat_size), 6 * L, M->at_off<double>(O.ss_part), kSumsqParts,
                        M->at_off<double>(O.ss), st);
  // X0 into the NS workspace, every matrix in its wide orientation, one batch per
  // shape: the d x d squares (q, k, v, o of each layer; only q and o when grouped-query
  // attention makes Wk, Wv kv x d, which then form their own batch), then the d x F
  // pairs
  const NsLayout nsl(c);
  const int kv = nsl.kv;
  const bool kvsq = nsl.kvsq;  // k and v join the squares
  const size_t nsq = nsl.nsq, nkv = nsl.nkv;
  auto xdst = [&](int l, int j) { return nsl.xdst(l, j); };
  auto mrows = [&](int j) { return nsl.mrows(j); };
  auto transposed = [&](int j) { return nsl.transposed(j); };
  // the untransposed matrices (all but W1 when F > d) in one launch per pass, from the job
  // table gpt_init uploaded; the transposed ones one by one
  const MuonVecJob* jobs = M->at_off<MuonVecJob>(O.mv_jobs);
  const int njobs = (int)M->mv_jobs.size();
  launch_ns_normalize_batched(mom, M->at_off<double>(O.ss), 1e-7f, jobs, njobs, xf, xa[0],
                              nsplit > 0 ? xl[0] : nullptr, nat, st);
  for (int l = 0; l < L; ++l)
    for (int j = 0; j < 6; ++j) {
      if (!transposed(j)) continue;
      const int rows = mrows(j), cols = j == 5 ? F : d;
      const size_t dst = xdst(l, j);
      launch_ns_normalize(mom + M->moff[6 * l + j], M->at_off<double>(O.ss), 6 * l + j, 1e-7f, rows, cols,
                          true, xf + dst, xa[0] + dst * es, nsplit > 0 ? xl[0] + dst * es : nullptr, nat, st);
    }
  struct Batch { int s, l, nb; size_t off; };
  const Batch all_batches[3] = {{d, d, (kvsq ? 4 : 2) * L, 0}, {kv, d, 2 * L, nsq}, {s, lw, 2 * L, nsq + nkv}};
  std::vector<Batch> batches = {all_batches[0]};
  if (!kvsq) batches.push_back(all_batches[1]);
  batches.push_back(all_batches[2]);
  float* Af = M->at_off<float>(O.Af);
  void* Aa = M->base + O.Aa;
  void* Ba = M->base + O.Ba;
  void* Alo = M->base + O.Al;
  void* Blo = M->base + O.Bl;
  int rc;
  // the d x d batch on the caller's stream; the others one after another in the second
  // part of the Gram-sized workspaces, on the side stream beside it when the model's
  // launches leave CUs idle (gptk_side_stream), joined before the update is applied
  const size_t a1 = ns_first_elems(c);
  const NsBuffers nb0{xf, {xa[0], xa[1]}, {xl[0], xl[1]}, es, Af, Aa, Ba, Alo, Blo};
  const NsBuffers nb1{xf, {xa[0], xa[1]}, {xl[0], xl[1]}, es, Af + a1, (char*)Aa + a1 * es, (char*)Ba + a1 * es,
                      (char*)Alo + a1 * es, (char*)Blo + a1 * es};
  const bool ns_side = g_side_stream && M->side && (M->side_pays || g_side_stream == 2) && batches.size() > 1;
  hipStream_t st1 = ns_side ? M->side : st;
  if (ns_side &&
      (hipEventRecord(M->sev_fork, st) != hipSuccess || hipStreamWaitEvent(st1, M->sev_fork, 0) != hipSuccess))
    return GPT_ERR_HIP;
  auto run0 = [&](const GemmArgs& p) { return run_gemm(M, p, st, false); };
  auto run1 = [&](const GemmArgs& p) { return run_gemm(M, p, st1, false); };
  rc = ns_iterate(nat, nsplit, c.ns_steps, c.ns_coeffs, batches[0].s, batches[0].l, batches[0].nb, batches[0].off, nb0,
                  run0);
  for (size_t i = 1; i < batches.size() && !rc; ++i)
    rc = ns_iterate(nat, nsplit, c.ns_steps, c.ns_coeffs, batches[i].s, batches[i].l, batches[i].nb, batches[i].off,
                    nb1, run1);
  if (ns_side &&
      (hipEventRecord(M->sev_join, st1) != hipSuccess || hipStreamWaitEvent(st, M->sev_join, 0) != hipSuccess))
    rc = rc ? rc : GPT_ERR_HIP;
  if (rc) return rc;
  // NorMuon: per output row, the running second moment of the update; rows scaled by its
  // inverse root, the update's Frobenius norm kept
  const bool nm = c.extras & GPT_EXTRA_NORMUON;
  float* nm_scale = M->at_off<float>(O.nm_scale);
  if (nm) {
    for (int l = 0; l < L; ++l)
      for (int j = 0; j < 6; ++j)
        launch_normuon_rowstats(xf + xdst(l, j), mrows(j), j == 5 ? F : d, transposed(j),
                                M->at_off<float>(O.nm_mean) + M->nm_roff[6 * l + j], M->base + O.nm_ws, st);
    launch_normuon_scale(M->at_off<float>(O.nm_mean), M->at_off<float>(O.nm_v), M->at_off<long>(O.nm_roff), 6 * L,
                         c.normuon_beta2, nm_scale, st);
  }
  float* wblk = M->blk(M->params());
  launch_muon_apply_batched(wblk, M->at == ACT_BF16 ? M->wact(0) : nullptr, M->at, xf, lr, jobs, njobs,
                            nm ? nm_scale : nullptr, st);
  for (int l = 0; l < L; ++l)
    for (int j = 0; j < 6; ++j) {
      if (!transposed(j)) continue;
      const int rows = mrows(j), cols = j == 5 ? F : d;
      const size_t mo = M->moff[6 * l + j];
      launch_muon_apply(wblk + mo, M->at == ACT_BF16 ? M->wact(mo) : nullptr, M->at, xf + xdst(l, j), lr, rows, cols,
                        true, st, nm ? nm_scale + M->nm_roff[6 * l + j] : nullptr);
    }
  M->wq_dirty = true;
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

static int copy_tensor(gpt_model* M, int id, float* region, bool to_host, float* h, size_t n, hipStream_t st,
                       bool blocks_only) {
  size_t off;
  int r, c;
  if (!M || !h || !tensor_loc(M->cfg, id, &off, &r, &c)) return GPT_ERR_ARG;
  if (n != (size_t)r * c) return GPT_ERR_ARG;
  if (blocks_only) {
    if (id == 0 || id >= 1 + 6 * M->cfg.depth) return GPT_ERR_ARG;
    off -= M->nE;
  }
  float* p = region + off;
  if (hipStreamSynchronize(st) != hipSuccess) return GPT_ERR_HIP;
  if (hipMemcpy(to_host ? (void*)h : (void*)p, to_host ? (const void*)p : (const void*)h, n * 4,
                to_host ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice) != hipSuccess)
    return GPT_ERR_HIP;
  return GPT_OK;
}

int gpt_grads(gpt_model* M, int32_t id, float* h, size_t n, void* s) {
  return M ? copy_tensor(M, id, M->grads(), true, h, n, (hipStream_t)s, false) : GPT_ERR_ARG;
}
int gpt_get_params(gpt_model* M, int32_t id, float* h, size_t n, void* s) {
  return M ? copy_tensor(M, id, M->params(), true, h, n, (hipStream_t)s, false) : GPT_ERR_ARG;
}
int gpt_set_grads(gpt_model* M, int32_t id, const float* h, size_t n, void* s) {
  return M ? copy_tensor(M, id, M->grads(), false, const_cast<float*>(h), n, (hipStream_t)s, false) : GPT_ERR_ARG;
}
int gpt_get_momentum(gpt_model* M, int32_t id, float* h, size_t n, void* s) {
  return M ? copy_tensor(M, id, M->at_off<float>(M->off.mom), true, h, n, (hipStream_t)s, true) : GPT_ERR_ARG;
}
int gpt_set_momentum(gpt_model* M, int32_t id, const float* h, size_t n, void* s) {
  return M ? copy_tensor(M, id, M->at_off<float>(M->off.mom), false, const_cast<float*>(h), n, (hipStream_t)s, true)
           : GPT_ERR_ARG;
}
int gpt_set_params(gpt_model* M, int32_t id, const float* h, size_t n, void* s) {
  if (!M) return GPT_ERR_ARG;
  hipStream_t st = (hipStream_t)s;
  int rc = copy_tensor(M, id, M->params(), false, const_cast<float*>(h), n, st, false);
  if (rc) return rc;
  M->wq_dirty = true;
  if (M->at == ACT_BF16) {
    size_t off;
    int r, c;
    tensor_loc(M->cfg, id, &off, &r, &c);
    if (id == 1 + 6 * M->cfg.depth)
      launch_cast_f32_to_act(M->params() + off, M->uact(), M->at, n, st);
    else if (id >= 1 && id <= 6 * M->cfg.depth)  // only the block matrices have act copies
      launch_cast_f32_to_act(M->params() + off, M->wact(off - M->nE), M->at, n, st);
  }
  return hipStreamSynchronize(st) == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gpt_argmax(gpt_model* M, int32_t* d_out, void* s) {
  if (!M || !d_out || !M->stepped) return GPT_ERR_ARG;
  return hipMemcpyAsync(d_out, M->base + M->off.argmax, (size_t)M->N * 4, hipMemcpyDeviceToDevice,
                        (hipStream_t)s) == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gpt_row_loss(gpt_model* M, float* d_out, void* s) {
  if (!M || !d_out || !M->stepped) return GPT_ERR_ARG;
  return hipMemcpyAsync(d_out, M->base + M->off.row_loss, (size_t)M->N * 4, hipMemcpyDeviceToDevice,
                        (hipStream_t)s) == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gpt_prof_enable(gpt_model* M, const char* name) {
  if (!M) return GPT_ERR_ARG;
  M->prof_name = name ? name : "";
  M->ev_used = 0;
  return GPT_OK;
}

int gpt_prof_read(gpt_model* M, int64_t* launches, double* ms, double* flops) {
  if (!M || !launches || !ms || !flops) return GPT_ERR_ARG;
  double t = 0, f = 0;
  for (size_t i = 0; i + 1 < M->ev_used; i += 2) {
    if (hipEventSynchronize(M->ev[i + 1]) != hipSuccess) return GPT_ERR_HIP;
    float e = 0;
    if (hipEventElapsedTime(&e, M->ev[i], M->ev[i + 1]) != hipSuccess) return GPT_ERR_HIP;
    t += e;
    f += M->evflops[i / 2];
  }
  *launches = (int64_t)(M->ev_used / 2);
  *ms = t;
  *flops = f;
  return GPT_OK;
}

size_t gpt_capture_bytes(const gpt_cfg* c, int32_t layer) {
  if (gpt_cfg_validate(c) != GPT_OK || layer < 0 || layer > c->depth) return 0;
  size_t total = 0;
  capture_offset(*c, layer, -1, &total);
  return total;
}

int gpt_capture(gpt_model* M, int32_t layer, void* d_buf, size_t bytes) {
  if (!M) return GPT_ERR_ARG;
  if (!d_buf) {
    M->cap_buf = nullptr;
    M->cap_layer = -1;
    return GPT_OK;
  }
  if (layer < 0 || layer > M->cfg.depth || bytes < gpt_capture_bytes(&M->cfg, layer) || ((uintptr_t)d_buf & 255))
    return GPT_ERR_ARG;
  M->cap_buf = (char*)d_buf;
  M->cap_layer = layer;
  return GPT_OK;
}

// ---------------------------------------------------------------------------
// kernel-level entry points

static int act_type(int dtype) { return dtype == GPT_FP32 ? ACT_F32 : dtype == GPT_BF16 ? ACT_BF16 : -1; }

// Leading dimensions cover one row of each stored matrix (A(m,k) = A[m lda + k] when
// k-major, A[k lda + m] otherwise), and batch strides are non-negative and cover one
// whole matrix (0 shares an operand between the batch entries; never the output's).
static bool gemm_layout_ok(int a_kmaj, int b_kmaj, int M, int N, int K, int batch, long lda, long sA, long ldb,
                           long sB, long ldc, long sC) {
  if (M == 0 || N == 0 || batch == 0) return true;  // nothing is read or written
  if (lda < (a_kmaj ? K : M) || lda < 1 || ldb < (b_kmaj ? K : N) || ldb < 1 || ldc < N) return false;
  if (batch > 1) {
    const long ea = (long)(a_kmaj ? M : K) * lda, eb = (long)(b_kmaj ? N : K) * ldb, ec = (long)M * ldc;
    if (sA < 0 || sB < 0 || (sA && sA < ea) || (sB && sB < eb) || sC < ec) return false;
  }
  return true;
}

int gptk_gemm_auto_splits(int dtype, int a_kmaj, int b_kmaj, int M, int N, int K, int batch) {
  const int at = act_type(dtype);
  if (at < 0 || M < 0 || N < 0 || K < 0 || batch < 0) return 0;
  GemmArgs p;
  p.M = M; p.N = N; p.K = K; p.batch = batch; p.dtype = at;
  p.a_kmaj = a_kmaj != 0; p.b_kmaj = b_kmaj != 0;
  return gemm_auto_splits(p);
}

int gptk_gemm(int dtype, int a_kmaj, int b_kmaj, int M, int N, int K, int batch, const void* A, long lda, long sA,
              const void* B, long ldb, long sB, float* C, long ldc, long sC, int tile, int splits, void* ws,
              size_t ws_bytes, void* stream) {
  const int at = act_type(dtype);
  if (at < 0) return GPT_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || batch < 0 || !C) return GPT_ERR_ARG;
  if (!gemm_layout_ok(a_kmaj, b_kmaj, M, N, K, batch, lda, sA, ldb, sB, ldc, sC)) return GPT_ERR_ARG;
  GemmArgs p;
  p.M = M; p.N = N; p.K = K; p.batch = batch;
  p.A = A; p.lda = lda; p.strideA = sA; p.a_kmaj = a_kmaj != 0;
  p.B = B; p.ldb = ldb; p.strideB = sB; p.b_kmaj = b_kmaj != 0;
  p.dtype = at; p.outF = C; p.ldo = ldc; p.strideO = sC;
  p.tile = tile & 15; p.sym = (tile & 16) != 0;
  p.splits = splits < 0 ? gemm_auto_splits(p) : splits < 1 ? 1 : splits;
  p.ws = (float*)ws; p.ws_bytes = ws_bytes;
  if ((long)p.batch * p.splits > 65535) return GPT_ERR_ARG;  // grid rows
  const int rc = launch_gemm(p, (hipStream_t)stream);
  if (rc == 1) return GPT_ERR_ARG;
  if (rc == 2) return GPT_ERR_SHAPE;
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_gemm_split(int a_kmaj, int b_kmaj, int M, int N, int K, int batch, const void* Ah, const void* Al, long lda,
                    long sA, const void* Bh, const void* Bl, long ldb, long sB, float* C, long ldc, long sC,
                    void* stream) {
  if (M < 0 || N < 0 || K < 0 || batch < 0 || !C || !Ah || !Al || !Bh || !Bl) return GPT_ERR_ARG;
  if (!gemm_layout_ok(a_kmaj, b_kmaj, M, N, K, batch, lda, sA, ldb, sB, ldc, sC) || batch > 65535) return GPT_ERR_ARG;
  GemmArgs p;
  p.M = M; p.N = N; p.K = K; p.batch = batch; p.split = true; p.dtype = ACT_BF16;
  p.A = Ah; p.A_lo = Al; p.lda = lda; p.strideA = sA; p.a_kmaj = a_kmaj != 0;
  p.B = Bh; p.B_lo = Bl; p.ldb = ldb; p.strideB = sB; p.b_kmaj = b_kmaj != 0;
  p.outF = C; p.ldo = ldc; p.strideO = sC;
  const int rc = launch_gemm(p, (hipStream_t)stream);
  if (rc) return rc == 1 ? GPT_ERR_ARG : GPT_ERR_SHAPE;
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

// workspace of gptk_newton_schulz: the copy whose Frobenius norm is taken, the fp32
// carried X, two operand planes of X, A and B (fp32 A too for the fp32 path), the
// sum-of-squares partials and the one-matrix table
static size_t ns_ws_layout(int rows, int cols, size_t* o) {
  const size_t n = (size_t)rows * cols, s = std::min(rows, cols);
  Plan P;
  o[0] = P.add(n * 4);                // copy of G
  o[1] = P.add(n * 4);                // xf
  o[2] = P.add(n * 4);                // xa0 (fp32 path: 4 bytes per element)
  o[3] = P.add(n * 4);                // xa1
  o[4] = P.add(s * s * 4);            // Af
  o[5] = P.add(s * s * 4);            // Aa
  o[6] = P.add(s * s * 4);            // Ba
  o[7] = P.add(kSumsqParts * 8 + 8);  // sum-of-squares partials and total
  o[8] = P.add(16);                   // offset and size of the one matrix
  return P.total;
}

size_t gptk_ns_ws_bytes(int rows, int cols) {
  if (rows < 1 || cols < 1) return 0;
  size_t o[9];
  return ns_ws_layout(rows, cols, o);
}

int gptk_newton_schulz(int dtype, const float* G, int rows, int cols, const float* coeffs, int steps, float* X,
                       void* ws, size_t ws_bytes, void* stream) {
  const int at = act_type(dtype);
  if (at < 0) return GPT_ERR_UNSUPPORTED;
  if (!G || !X || !coeffs || !ws || rows < 1 || cols < 1 || steps < 0 || steps > 5 || ((uintptr_t)ws & 255))
    return GPT_ERR_ARG;
  if (rows % 8 || cols % 8) return GPT_ERR_SHAPE;  // the 16-bit operand planes take 8-element rows
  size_t o[9];
  if (ws_bytes < ns_ws_layout(rows, cols, o)) return GPT_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  const bool tr = rows > cols;  // a tall G is orthogonalised as G^T
  const int s = std::min(rows, cols), l = std::max(rows, cols);
  const int nat = at == ACT_BF16 ? ACT_F16 : ACT_F32;
  const size_t es = nat == ACT_F16 ? 2 : 4;
  float* copy = (float*)(w + o[0]);
  float* xf = (float*)(w + o[1]);
  double* part = (double*)(w + o[7]);
  double* ss = part + kSumsqParts;
  const long table[2] = {0, (long)rows * cols};  // pageable: copied before hipMemcpyAsync returns
  if (hipMemcpyAsync(w + o[8], table, sizeof(table), hipMemcpyHostToDevice, st) != hipSuccess) return GPT_ERR_HIP;
  // copy = 0 * copy + G (a momentum update with mu = 0), and its sum of squares
  launch_zero(copy, (size_t)rows * cols * 4, st);
  launch_momentum_sumsq(copy, G, 0.f, (const long*)(w + o[8]), (const long*)(w + o[8]) + 1, 1, part, kSumsqParts, ss,
                        st);
  launch_ns_normalize(copy, ss, 0, 1e-7f, rows, cols, tr, xf, w + o[2], nullptr, nat, st);
  float cf[5][3];
  for (int i = 0; i < steps; ++i)
    for (int j = 0; j < 3; ++j) cf[i][j] = coeffs[3 * i + j];
  const NsBuffers nb{xf, {w + o[2], w + o[3]}, {nullptr, nullptr}, es, (float*)(w + o[4]), w + o[5], w + o[6], nullptr,
                     nullptr};
  auto run = [&](const GemmArgs& p0) {
    GemmArgs p = p0;
    p.splits = 1;
    return launch_gemm(p, st) ? GPT_ERR_SHAPE : GPT_OK;
  };
  int rc = ns_iterate(nat, 0, steps, cf, s, l, 1, 0, nb, run);
  if (rc) return rc;
  // X = the result in G's orientation: X = 0 - (-1) xf (transposed back for a tall G)
  launch_zero(X, (size_t)rows * cols * 4, st);
  launch_muon_apply(X, nullptr, ACT_F32, xf, -1.f, rows, cols, tr, st, nullptr);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_quant_e4m3(int dtype, const void* x, int rows, int cols, long ld, uint32_t* amax_slot, uint8_t* q, uint8_t* qt,
                    float* inv_scale, void* stream) {
  const int at = act_type(dtype);
  if (at < 0) return GPT_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || ld < cols || !x || !amax_slot || !inv_scale || (!q && !qt)) return GPT_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  launch_zero(amax_slot, 4, st);
  launch_amax(x, at, rows, cols, ld, amax_slot, st);
  launch_quant_e4m3(x, at, rows, cols, ld, amax_slot, q, cols, qt, rows, inv_scale, st);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_gemm_fp8(int M, int N, int K, const uint8_t* A, long lda, const uint8_t* B, long ldb, const float* dq_a,
                  const float* dq_b, float* C, long ldc, int splits, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || N < 0 || K < 0 || !A || !B || !dq_a || !dq_b || !C) return GPT_ERR_ARG;
  if (!gemm_layout_ok(1, 1, M, N, K, 1, lda, 0, ldb, 0, ldc, 0) || splits > 65535) return GPT_ERR_ARG;
  GemmArgs p;
  p.M = M; p.N = N; p.K = K; p.fp8 = true; p.dtype = ACT_BF16;
  p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.dq_a = dq_a; p.dq_b = dq_b;
  p.outF = C; p.ldo = ldc;
  p.splits = splits < 1 ? 1 : splits; p.ws = (float*)ws; p.ws_bytes = ws_bytes;
  const int rc = launch_gemm(p, (hipStream_t)stream);
  if (rc) return rc == 1 ? GPT_ERR_ARG : GPT_ERR_SHAPE;
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

const char* gpt_gemm_kernel_name(int dtype, int a_kmaj, int b_kmaj, int M, int N, int K, int batch) {
  GemmArgs p;
  p.M = M; p.N = N; p.K = K; p.batch = batch; p.dtype = act_type(dtype) < 0 ? ACT_BF16 : act_type(dtype);
  p.a_kmaj = a_kmaj != 0; p.b_kmaj = b_kmaj != 0;
  return gemm_kernel_name(p);
}

static int attn_ok(int dtype, int hd) {
  if (act_type(dtype) < 0) return GPT_ERR_UNSUPPORTED;
  if (hd != 32 && hd != 64 && hd != 128) return GPT_ERR_UNSUPPORTED;
  return GPT_OK;
}

// key/value heads: 1 <= Hkv <= H with H % Hkv == 0 (any Hkv when H = 0)
static bool kv_heads_ok(int H, int Hkv) { return H == 0 ? Hkv >= 0 : (Hkv >= 1 && Hkv <= H && H % Hkv == 0); }

int gptk_ce_variant(int variant) {
  if (variant < 0 || variant > 1) return GPT_ERR_ARG;
  set_ce_variant(variant);
  return GPT_OK;
}

int gptk_side_stream(int on) {
  const int prev = g_side_stream;
  if (on >= 0) g_side_stream = on > 2 ? 2 : on;
  return prev;
}

int gptk_fp8_fused_amax(int on) {
  const int prev = g_fp8_fused_amax;
  if (on >= 0) g_fp8_fused_amax = on ? 1 : 0;
  return prev;
}

int gptk_attn_variant(int pass, int variant) {
  if (pass < 0 || pass > 1 || variant < 0 || variant > (pass == 1 ? 2 : 1)) return GPT_ERR_ARG;
  if (pass == 0) set_attn_fwd_variant(variant);
  else set_attn_bwd_variant(variant);
  return GPT_OK;
}

static int attn_fwd_entry(int dtype, const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv, int hd,
                          int window, void* stream, bool qk_normed) {
  int rc = attn_ok(dtype, hd);
  if (rc) return rc;
  if (B < 0 || T < 0 || H < 0 || !kv_heads_ok(H, Hkv) || window < 0 || !qkv || !o || !lse) return GPT_ERR_ARG;
  launch_attn_fwd(qkv, o, lse, act_type(dtype), B, T, H, Hkv, hd, window, (hipStream_t)stream, nullptr, 0, qk_normed);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_attn_fwd(int dtype, const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv, int hd, int window,
                  void* stream) {
  return attn_fwd_entry(dtype, qkv, o, lse, B, T, H, Hkv, hd, window, stream, false);
}

int gptk_attn_fwd_qknorm(int dtype, const void* qkv, void* o, float* lse, int B, int T, int H, int Hkv, int hd,
                         int window, void* stream) {
  return attn_fwd_entry(dtype, qkv, o, lse, B, T, H, Hkv, hd, window, stream, true);
}

int gptk_attn_bwd(int dtype, const void* qkv, const void* o, const void* dO, const float* lse, float* D, void* dqkv,
                  int B, int T, int H, int Hkv, int hd, int window, void* stream) {
  int rc = attn_ok(dtype, hd);
  if (rc) return rc;
  if (B < 0 || T < 0 || H < 0 || !kv_heads_ok(H, Hkv) || window < 0 || !qkv || !o || !dO || !lse || !D || !dqkv)
    return GPT_ERR_ARG;
  launch_attn_bwd(qkv, o, dO, lse, D, dqkv, act_type(dtype), B, T, H, Hkv, hd, window, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

// Allocation-free attention backward: the rowsum(dO * O) scratch that gptk_attn_bwd
// takes as an argument lives here in a file-scope device array instead (each GPU holds
// its own copy until the process ends).  Host code never passes the array's name to a
// kernel: it resolves the device address once per device with hipGetSymbolAddress and
// uses that pointer.
constexpr size_t kAttnScratchFloats = (size_t)1 << 20;  // 4 MiB: B * H * T <= 1,048,576
constexpr int kMaxDevices = 64;
static __device__ __align__(256) float scratch[kAttnScratchFloats];
static std::mutex g_scratch_mu;
static float* g_scratch_ptr[kMaxDevices] = {};

static int scratch_of_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GPT_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GPT_ERR_HIP;
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return GPT_OK;
}

int gptk_attn_bwd_noalloc(int dtype, const void* qkv, const void* o, const void* dO, const float* lse, void* dqkv,
                          int B, int T, int H, int Hkv, int hd, int window, void* stream) {
  int rc = attn_ok(dtype, hd);
  if (rc) return rc;
  if (B < 0 || T < 0 || H < 0 || !kv_heads_ok(H, Hkv) || window < 0 || !qkv || !o || !dO || !lse || !dqkv)
    return GPT_ERR_ARG;
  if ((double)B * H * T > (double)kAttnScratchFloats) return GPT_ERR_ARG;
  float* D = nullptr;
  if ((rc = scratch_of_current_device(&D))) return rc;
  // every (b, h, t) of D is written by the backward before it is read: nothing to clear
  launch_attn_bwd(qkv, o, dO, lse, D, dqkv, act_type(dtype), B, T, H, Hkv, hd, window, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_rmsnorm_fwd(int dtype, const float* x, void* y, float* rstd, int N, int d, float eps, void* stream) {
  if (act_type(dtype) < 0) return GPT_ERR_UNSUPPORTED;
  if (N < 0 || d < 4 || d % 4 || d > 2048 || !x || !y || !rstd) return GPT_ERR_ARG;
  launch_rmsnorm_fwd(x, y, act_type(dtype), rstd, N, d, eps, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_rmsnorm_bwd(int dtype, const float* dy, const float* x, const float* rstd, const float* dres, float* dx,
                     void* dxa, int N, int d, void* stream) {
  if (act_type(dtype) < 0) return GPT_ERR_UNSUPPORTED;
  if (N < 0 || d < 4 || d % 4 || d > 2048 || !dy || !x || !rstd || !dx) return GPT_ERR_ARG;
  launch_rmsnorm_bwd(dy, x, rstd, dres, dx, dxa, act_type(dtype), N, d, 0.f, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_rope_qknorm_fwd(int dtype, void* qkv, float* cs, float* rq, float* rk, int B, int T, int H, int Hkv, int hd,
                         float base, float eps, void* stream) {
  int rc = attn_ok(dtype, hd);
  if (rc) return rc;
  if (!qkv || !cs || !rq || !rk || B < 0 || T < 0 || H < 0 || !kv_heads_ok(H, Hkv)) return GPT_ERR_ARG;
  launch_rope_table(cs, T, hd, base, (hipStream_t)stream);
  launch_rope_qknorm_fwd(qkv, act_type(dtype), cs, rq, rk, B, T, H, Hkv, hd, eps, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_rope_qknorm_bwd(int dtype, void* dqkv, const void* qkv, float* cs, const float* rq, const float* rk, int B,
                         int T, int H, int Hkv, int hd, float base, void* stream) {
  int rc = attn_ok(dtype, hd);
  if (rc) return rc;
  if (!dqkv || !qkv || !cs || !rq || !rk || B < 0 || T < 0 || H < 0 || !kv_heads_ok(H, Hkv)) return GPT_ERR_ARG;
  launch_rope_table(cs, T, hd, base, (hipStream_t)stream);
  launch_rope_qknorm_bwd(dqkv, qkv, act_type(dtype), cs, rq, rk, B, T, H, Hkv, hd, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_cross_entropy(int dtype, const float* z, const int32_t* tgt, void* dz, float* rl, int32_t* am, int N, int V,
                       float inv_n, int32_t* err, void* stream) {
  if (act_type(dtype) < 0) return GPT_ERR_UNSUPPORTED;
  if (N < 0 || V < 1 || !z || !tgt || !dz || !rl || !am || !err) return GPT_ERR_ARG;
  launch_cross_entropy(z, tgt, dz, act_type(dtype), rl, am, N, V, inv_n, err, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

int gptk_embed_gather(const int32_t* tok, const float* E, float* h, int N, int d, int V, int32_t* err, void* stream) {
  if (N < 0 || d < 4 || d % 4 || V < 1 || !tok || !E || !h || !err) return GPT_ERR_ARG;
  launch_embed_gather(tok, E, h, N, d, V, err, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

size_t gptk_embed_ws_bytes(int N, int V, int d) { return embed_ws_bytes(N, V, d); }

int gptk_embed_scatter(const int32_t* tok, const float* dh, float* dE, int N, int V, int d, void* ws, int32_t* sorted,
                       void* stream) {
  if (N < 0 || d < 4 || d % 4 || V < 1 || !tok || !dh || !dE || !ws) return GPT_ERR_ARG;
  launch_embed_scatter(tok, dh, dE, N, V, d, ws, sorted, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_HIP;
}

}  // extern "C"
