"""Stage-isolated parity of each HIP kernel against the fp64 oracle pieces.

Inputs are seeded and rounded to the kernel's operand type on the host, so the
oracle sees exactly the values the kernel reads; the remaining differences are
accumulation order/precision and the kernel's own roundings.
"""
import numpy as np
import pytest
import torch

from gpt_pretraining_step_train_amd import binding as B
from oracle import gpt_oracle as O
from tests.gpu_util import bf16_round, from_dev, rel_l2, say, to_dev

pytestmark = pytest.mark.gpu
DT = {"bf16": B.GPT_BF16, "fp32": B.GPT_FP32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    torch.cuda.set_device(0)


def _round(x, dtype):
    return bf16_round(x) if dtype == "bf16" else x.astype(np.float32)


# ----------------------------------------------------------------------------- GEMM

GEMM_CASES = [
    # dtype, a_kmaj, b_kmaj, M, N, K, batch, tile, splits
    ("bf16", 1, 1, 300, 200, 136, 1, 0, 1),
    ("bf16", 1, 1, 520, 264, 200, 1, 1, 1),
    ("bf16", 1, 0, 296, 264, 136, 1, 2, 1),
    ("bf16", 1, 0, 512, 520, 256, 1, 1, 1),
    ("bf16", 0, 0, 296, 200, 264, 1, 2, 1),
    ("bf16", 0, 0, 264, 528, 520, 1, 1, 1),
    ("bf16", 0, 1, 136, 300, 72, 1, 2, 1),
    ("bf16", 1, 1, 256, 384, 128, 3, 2, 1),
    ("bf16", 0, 0, 136, 200, 1032, 1, 2, 3),
    # 256x256 direct-to-LDS kernel (tile 1: k tiles of 64 in 2 stages, tile 3: k tiles of
    # 32 in 3 stages, tile 5: k tiles of 32 in 4 stages)
    # and the register-staged 256x256 kernel (tile 4)
    ("bf16", 1, 1, 520, 264, 200, 1, 3, 1),
    ("bf16", 1, 0, 512, 520, 256, 1, 3, 1),
    ("bf16", 0, 0, 264, 528, 520, 1, 3, 1),
    ("bf16", 0, 1, 264, 300, 72, 1, 1, 1),
    ("bf16", 0, 1, 264, 300, 72, 1, 3, 1),
    ("bf16", 1, 1, 256, 384, 128, 3, 1, 1),
    ("bf16", 0, 0, 136, 200, 1032, 1, 1, 3),
    ("bf16", 1, 0, 1000, 776, 1000, 1, 1, 1),
    ("bf16", 1, 1, 520, 264, 200, 1, 5, 1),
    ("bf16", 1, 0, 512, 520, 256, 1, 5, 1),
    ("bf16", 0, 0, 264, 528, 520, 1, 5, 1),
    ("bf16", 0, 1, 264, 300, 72, 1, 5, 1),
    ("bf16", 1, 1, 256, 384, 128, 3, 5, 1),
    ("bf16", 0, 0, 136, 200, 1032, 1, 5, 3),
    ("bf16", 1, 1, 520, 264, 200, 1, 4, 1),
    ("bf16", 0, 0, 264, 528, 520, 1, 4, 1),
    # batched / split-K launches of a multiple of 8 workgroups: the grid-wide XCD order
    # (6 tiles x batch 4, x 4 splits with a ragged last split, x batch 2 x 2 splits)
    ("bf16", 1, 1, 520, 264, 200, 4, 1, 1),
    ("bf16", 0, 0, 264, 528, 2080, 1, 1, 4),
    ("bf16", 1, 0, 264, 528, 1040, 2, 1, 2),
    ("fp32", 1, 1, 100, 70, 33, 1, 0, 1),
    ("fp32", 1, 0, 96, 72, 40, 2, 0, 1),
    ("fp32", 0, 0, 72, 96, 200, 1, 0, 2),
]


@pytest.mark.parametrize("case", GEMM_CASES)
def test_gemm_layouts_tails_batch_split(case):
    dtype, ak, bk, M, N, K, batch, tile, splits = case
    say("gemm", case)
    rng = np.random.default_rng(M * 7 + N)
    a_shape = (batch, M, K) if ak else (batch, K, M)
    b_shape = (batch, N, K) if bk else (batch, K, N)
    A = _round(rng.standard_normal(a_shape), dtype)
    Bm = _round(rng.standard_normal(b_shape), dtype)
    Am = A if ak else A.transpose(0, 2, 1)
    Bn = Bm if bk else Bm.transpose(0, 2, 1)
    ref = np.einsum("zmk,znk->zmn", Am.astype(np.float64), Bn.astype(np.float64))
    dA, dB = to_dev(A, dtype), to_dev(Bm, dtype)
    C = torch.full((batch, M, N), float("nan"), device="cuda")
    ws = torch.empty(splits * batch * M * N, device="cuda") if splits > 1 else None
    B.gemm(DT[dtype], ak, bk, M, N, K, dA, K if ak else M, dB, K if bk else N, C, N, batch=batch,
           sA=A[0].size, sB=Bm[0].size, sC=M * N, tile=tile, splits=splits, ws=ws)
    torch.cuda.synchronize()
    got = from_dev(C)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert np.isfinite(got).all()
    assert err < (1e-5 if dtype == "bf16" else 1e-5), err


SYM_CASES = [  # a_kmaj, M, K, batch, tile (+16: symmetric hint), splits
    (1, 520, 200, 2, 17, 1), (0, 264, 136, 1, 17, 1), (1, 1000, 64, 1, 19, 1), (1, 1002, 96, 1, 17, 1),
    (1, 520, 2048, 1, 17, 2), (1, 300, 72, 3, 18, 1), (1, 520, 200, 2, 21, 1), (0, 264, 136, 1, 21, 1),
    (1, 520, 200, 4, 17, 1), (0, 264, 136, 8, 17, 1),  # 24 upper tiles in all: grid-wide XCD order
]


@pytest.mark.parametrize("case", SYM_CASES)
def test_gemm_symmetric_hint(case):
    """C = A A^T (or A^T A) with the symmetric hint: upper tiles computed, mirrored;
    every element of both triangles against fp64 (split-K and the 128 kernel ignore it)."""
    ak, M, K, batch, tile, splits = case
    say("gemm sym", case)
    rng = np.random.default_rng(M + K)
    A = _round(rng.standard_normal((batch, M, K) if ak else (batch, K, M)), "bf16")
    Am = A if ak else A.transpose(0, 2, 1)
    ref = np.einsum("zmk,znk->zmn", Am.astype(np.float64), Am.astype(np.float64))
    dA = to_dev(A, "bf16")
    C = torch.full((batch, M, M), float("nan"), device="cuda")
    ws = torch.empty(splits * batch * M * M, device="cuda") if splits > 1 else None
    B.gemm(DT["bf16"], ak, ak, M, M, K, dA, K if ak else M, dA, K if ak else M, C, M, batch=batch,
           sA=A[0].size, sB=A[0].size, sC=M * M, tile=tile, splits=splits, ws=ws)
    torch.cuda.synchronize()
    got = from_dev(C)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() / np.abs(ref).max() < 1e-5


SPLIT_CASES = [(1, 1, 300, 200, 136, 1), (1, 0, 296, 264, 264, 2), (0, 0, 136, 200, 1032, 1), (0, 1, 128, 72, 72, 1),
               # batches large enough for the 256x256 kernel
               (1, 1, 520, 264, 200, 64), (1, 0, 264, 520, 136, 64), (0, 0, 264, 264, 264, 128)]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_gemm_split_precision(case):
    """fp32 operands carried as bf16 hi + lo planes: ~16-bit operands, far tighter than bf16."""
    ak, bk, M, N, K, batch = case
    rng = np.random.default_rng(K + M)
    A = rng.standard_normal((batch, M, K) if ak else (batch, K, M)).astype(np.float32)
    Bm = rng.standard_normal((batch, N, K) if bk else (batch, K, N)).astype(np.float32)
    Am = A if ak else A.transpose(0, 2, 1)
    Bn = Bm if bk else Bm.transpose(0, 2, 1)
    ref = np.einsum("zmk,znk->zmn", Am.astype(np.float64), Bn.astype(np.float64))

    def planes(x):
        hi = torch.from_numpy(x).bfloat16()
        lo = (torch.from_numpy(x) - hi.float()).bfloat16()
        return hi.cuda(), lo.cuda()

    Ah, Al = planes(A)
    Bh, Bl = planes(Bm)
    C = torch.full((batch, M, N), float("nan"), device="cuda")
    B.gemm_split(ak, bk, M, N, K, Ah, Al, K if ak else M, Bh, Bl, K if bk else N, C, N, batch=batch,
                 sA=A[0].size, sB=Bm[0].size, sC=M * N)
    torch.cuda.synchronize()
    got = from_dev(C)
    assert np.abs(got - ref).max() / np.abs(ref).max() < 5e-5


def test_gemm_full_size_sampled():
    """d24 MLP up-projection shape [32768 x 6144 x 1536] in the launch configuration of
    the step; 4096 sampled outputs recomputed one by one in fp64."""
    M, N, K = 32768, 6144, 1536
    g = torch.Generator(device="cuda").manual_seed(0)
    A = torch.randn(M, K, device="cuda", generator=g).bfloat16()
    Bw = torch.randn(N, K, device="cuda", generator=g).bfloat16()
    C = torch.empty(M, N, device="cuda")
    B.gemm(B.GPT_BF16, 1, 1, M, N, K, A, K, Bw, K, C, N)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = rng.integers(0, M, 4096)
    cols = rng.integers(0, N, 4096)
    rows[:2], cols[:2] = [0, M - 1], [0, N - 1]
    a = A[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    b = Bw[torch.from_numpy(cols).cuda()].float().cpu().numpy().astype(np.float64)
    ref = np.sum(a * b, axis=1)
    got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    assert np.abs(got - ref).max() < 1e-4 * np.sqrt(K) * 4


# d24 weight-gradient products dW = dY^T X over the 32768 tokens of a B = 16, T = 2048
# micro-batch (both operands token-major, so both are transposed on load): (rows of W,
# cols of W) for the stacked QKV weight, Wo, W1, W2 and the LM head
D24_WGRAD = [(4608, 1536), (1536, 1536), (6144, 1536), (1536, 6144), (32768, 1536)]


@pytest.mark.parametrize("nout,kin", D24_WGRAD, ids=[f"{a}x{b}" for a, b in D24_WGRAD])
def test_gemm_d24_weight_gradients_with_the_steps_split(nout, kin):
    """The launcher's own split-K factor (gptk_gemm with splits < 0, the factor gpt_step
    picks for these shapes) over K = 32768: 2048 sampled outputs recomputed one by one
    in fp64 from the same bf16 operands, the first and last rows and columns included."""
    K = 32768
    splits = B.gemm_auto_splits(B.GPT_BF16, nout, kin, K, 1, 0, 0)
    say(f"  d24 weight gradient {nout}x{kin}x{K}: {splits} splits, kernel "
        f"{B.gemm_kernel_name(B.GPT_BF16, nout, kin, K, 1, 0, 0)}")
    g = torch.Generator(device="cuda").manual_seed(nout + kin)
    dY = torch.randn(K, nout, device="cuda", generator=g).bfloat16()
    X = torch.randn(K, kin, device="cuda", generator=g).bfloat16()
    C = torch.empty(nout, kin, device="cuda")
    ws = torch.empty(max(splits, 1) * nout * kin if splits > 1 else 64, device="cuda")
    B.gemm(B.GPT_BF16, 0, 0, nout, kin, K, dY, nout, X, kin, C, kin, splits=-1, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(nout)
    rows = rng.integers(0, nout, 2048)
    cols = rng.integers(0, kin, 2048)
    rows[:4], cols[:4] = [0, nout - 1, 0, nout - 1], [0, kin - 1, kin - 1, 0]
    a = dY[:, torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    b = X[:, torch.from_numpy(cols).cuda()].float().cpu().numpy().astype(np.float64)
    ref = np.sum(a * b, axis=0)
    scale = np.sum(np.abs(a * b), axis=0)  # fp32 accumulation error grows with the sum of |terms|
    got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    err = np.abs(got - ref) / scale
    say(f"    max |err| / sum|a b| = {err.max():.2e}")
    assert err.max() < 1e-5


@pytest.mark.parametrize("d", [768, 1664])
def test_gemm_lm_head_data_gradient_with_the_steps_split(d):
    """dr = dz U of the LM head at the full step size (32768 tokens, vocabulary 32768,
    d = 768 as in d12 and 1664 as in d26): dz token-major (K-major), U [V][d] read
    transposed, with the launcher's own split-K factor (gpt_step lets this long-reduction
    data gradient split).  Sampled outputs recomputed one by one in fp64."""
    M, N, K = 32768, d, 32768
    splits = B.gemm_auto_splits(B.GPT_BF16, M, N, K, 1, 1, 0)
    say(f"  LM-head data gradient {M}x{N}x{K}: {splits} splits")
    assert splits > 1  # the 1.5- and 3.5-round tilings are the ones the split is for
    g = torch.Generator(device="cuda").manual_seed(d)
    dz = (torch.randn(M, K, device="cuda", generator=g) * 1e-3).bfloat16()
    U = torch.randn(K, N, device="cuda", generator=g).bfloat16()
    C = torch.empty(M, N, device="cuda")
    ws = torch.empty(splits * M * N, device="cuda")
    B.gemm(B.GPT_BF16, 1, 0, M, N, K, dz, K, U, N, C, N, splits=-1, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(d)
    rows = rng.integers(0, M, 512)
    cols = rng.integers(0, N, 512)
    rows[:4], cols[:4] = [0, M - 1, 0, M - 1], [0, N - 1, N - 1, 0]
    a = dz[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    b = U[:, torch.from_numpy(cols).cuda()].float().cpu().numpy().astype(np.float64).T
    ref = np.sum(a * b, axis=1)
    scale = np.sum(np.abs(a * b), axis=1)
    got = C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy()
    err = np.abs(got - ref) / scale
    say(f"    max |err| / sum|a b| = {err.max():.2e}")
    assert err.max() < 1e-5


# ----------------------------------------------------------------------------- attention


def _qkv(Bn, T, H, hd, seed, dtype, Hkv=None):
    """Fused qkv rows [q: H heads | k: Hkv heads | v: Hkv heads] and the fp64 q, k, v."""
    Hkv = H if Hkv is None else Hkv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Bn, T, H, hd))
    k = rng.standard_normal((Bn, T, Hkv, hd))
    v = rng.standard_normal((Bn, T, Hkv, hd))
    q, _ = O.rms_norm(q, 1e-6)          # unit-RMS heads, as after QK-norm
    k, _ = O.rms_norm(k, 1e-6)
    qkv = np.concatenate([q.reshape(Bn, T, -1), k.reshape(Bn, T, -1), v.reshape(Bn, T, -1)], -1)
    qkv = _round(qkv, dtype)
    d, dkv = H * hd, Hkv * hd
    q = qkv[..., :d].reshape(Bn, T, H, hd).astype(np.float64)
    k = qkv[..., d:d + dkv].reshape(Bn, T, Hkv, hd).astype(np.float64)
    v = qkv[..., d + dkv:].reshape(Bn, T, Hkv, hd).astype(np.float64)
    return qkv, q, k, v


# (dtype, B, T, H, hd, window[, Hkv]): window > 0 is sliding-window attention (query i
# sees keys i - window < j <= i): one key, windows at and across a 64-key tile edge, and
# windows spanning several 128-query blocks.  Hkv < H is grouped-query attention (H / Hkv
# query heads per key/value head): groups of 2, 4 and 6 (one key/value head), sequence-
# head counts that do and do not fill the XCD-aware block order (multiples of 8 G).
ATTN_CASES = [("bf16", 2, 300, 3, 128, 0), ("bf16", 1, 256, 2, 64, 0), ("bf16", 2, 130, 2, 32, 0),
              ("bf16", 1, 1, 1, 128, 0), ("fp32", 2, 128, 4, 32, 0), ("fp32", 1, 77, 2, 64, 0),
              ("bf16", 2, 300, 3, 128, 1), ("bf16", 2, 300, 3, 128, 100), ("bf16", 1, 256, 2, 64, 64),
              ("bf16", 1, 256, 2, 64, 65), ("bf16", 2, 130, 2, 32, 37), ("bf16", 1, 700, 2, 128, 200),
              ("bf16", 1, 1024, 1, 128, 129), ("fp32", 2, 128, 4, 32, 17), ("fp32", 1, 77, 2, 64, 5),
              ("bf16", 2, 300, 4, 128, 0, 2), ("bf16", 2, 256, 8, 64, 0, 2), ("bf16", 1, 300, 6, 128, 100, 1),
              ("bf16", 4, 130, 4, 32, 0, 1), ("bf16", 2, 512, 16, 64, 0, 4), ("bf16", 1, 1, 4, 128, 0, 2),
              ("fp32", 2, 128, 4, 32, 0, 2), ("fp32", 1, 77, 4, 64, 9, 1)]


@pytest.mark.parametrize("case", ATTN_CASES)
def test_attention_fwd_bwd(case):
    dtype, Bn, T, H, hd, win = case[:6]
    Hkv = case[6] if len(case) > 6 else H
    G = H // Hkv
    say("attention", case)
    qkv, q, k, v = _qkv(Bn, T, H, hd, 11, dtype, Hkv)
    # query head h reads key/value head h // G
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    o_ref, P = O.causal_attention(q, kr, vr, window=win)
    # lse from the oracle's probabilities: the diagonal key is always visible, and
    # P_ii = exp(S_ii - lse_i)
    S_ii = np.einsum("bihd,bihd->bhi", q, kr) / np.sqrt(hd)
    lse_ref = S_ii - np.log(np.diagonal(P, axis1=2, axis2=3))   # [B,H,T]
    d, dkv = H * hd, Hkv * hd
    dq = to_dev(qkv, dtype)
    o = torch.zeros(Bn * T, d, device="cuda", dtype=dq.dtype)
    lse = torch.zeros(Bn * H * T, device="cuda")
    B.attn_fwd(DT[dtype], dq, o, lse, Bn, T, H, hd, win, n_kv=Hkv)
    torch.cuda.synchronize()
    o_got = from_dev(o).reshape(Bn, T, H, hd)
    tol = 1e-2 if dtype == "bf16" else 1e-5
    assert rel_l2(o_got, o_ref) < tol
    assert np.abs(from_dev(lse).reshape(Bn, H, T) - lse_ref).max() < (2e-3 if dtype == "bf16" else 1e-5)
    # the forward the step runs: q and k are RMS-normalised per head (as _qkv makes them), so
    # it exponentiates against a fixed reference instead of a running maximum
    o2 = torch.zeros_like(o)
    lse2 = torch.zeros_like(lse)
    B.attn_fwd_qknorm(DT[dtype], dq, o2, lse2, Bn, T, H, hd, win, n_kv=Hkv)
    torch.cuda.synchronize()
    assert rel_l2(from_dev(o2).reshape(Bn, T, H, hd), o_ref) < tol
    assert np.abs(from_dev(lse2).reshape(Bn, H, T) - lse_ref).max() < (2e-3 if dtype == "bf16" else 1e-5)
    # backward, from the kernel's own forward output (as in the step)
    rng = np.random.default_rng(12)
    dO = _round(rng.standard_normal((Bn, T, H, hd)), dtype)
    o_in = o_got
    dq_ref, dk_ref, dv_ref = O.causal_attention_bwd(dO.astype(np.float64), q, kr, vr, o_in, window=win)
    # a shared key/value head's gradient sums over its G query heads
    dk_ref = dk_ref.reshape(Bn, T, Hkv, G, hd).sum(axis=3)
    dv_ref = dv_ref.reshape(Bn, T, Hkv, G, hd).sum(axis=3)
    ddo = to_dev(dO.reshape(Bn * T, d), dtype)
    D = torch.zeros(Bn * H * T, device="cuda")
    dqkv = torch.full((Bn * T, d + 2 * dkv), float("nan"), device="cuda", dtype=dq.dtype)
    B.attn_bwd(DT[dtype], dq, o, ddo, lse, D, dqkv, Bn, T, H, hd, win, n_kv=Hkv)
    torch.cuda.synchronize()
    g = from_dev(dqkv).reshape(Bn, T, d + 2 * dkv)
    got = (g[..., :d].reshape(Bn, T, H, hd), g[..., d:d + dkv].reshape(Bn, T, Hkv, hd),
           g[..., d + dkv:].reshape(Bn, T, Hkv, hd))
    gtol = 2e-2 if dtype == "bf16" else 1e-4
    # relative to the largest of the three references: at T = 1 dq and dk are exactly 0
    scale = max(np.linalg.norm(r) for r in (dq_ref, dk_ref, dv_ref))
    for i, ref in enumerate((dq_ref, dk_ref, dv_ref)):
        e = np.linalg.norm(got[i] - ref) / max(np.linalg.norm(ref), 1e-3 * scale)
        assert e < gtol, (i, e)


# the backward's kernel variants (gptk_attn_variant pass 1): the pipelined dK/dV kernel
# (0, the default) and the unpipelined one (2) take the same steps in the same order, so
# their results must be bit-identical; the 64-key form (1, head_dim 128 only; run here on
# whole 256-query blocks of causal multi-head attention) is held to the kernel tolerance
BWD_VARIANT_CASES = [("bf16", 2, 300, 3, 128, 0), ("bf16", 1, 256, 2, 64, 0), ("bf16", 2, 130, 2, 32, 37),
                     ("bf16", 1, 700, 2, 128, 200), ("bf16", 2, 300, 4, 128, 0, 2), ("bf16", 1, 300, 6, 128, 100, 1),
                     ("bf16", 1, 1, 4, 128, 0, 2), ("bf16", 1, 64, 2, 128, 0), ("bf16", 1, 2048, 2, 128, 0)]


@pytest.mark.parametrize("case", BWD_VARIANT_CASES)
def test_attention_bwd_variants_agree(case):
    dtype, Bn, T, H, hd, win = case[:6]
    Hkv = case[6] if len(case) > 6 else H
    qkv, _, _, _ = _qkv(Bn, T, H, hd, 13, dtype, Hkv)
    d, dkv = H * hd, Hkv * hd
    dq = to_dev(qkv, dtype)
    o = torch.zeros(Bn * T, d, device="cuda", dtype=dq.dtype)
    lse = torch.zeros(Bn * H * T, device="cuda")
    B.attn_fwd(DT[dtype], dq, o, lse, Bn, T, H, hd, win, n_kv=Hkv)
    rng = np.random.default_rng(14)
    ddo = to_dev(_round(rng.standard_normal((Bn * T, d)), dtype), dtype)
    out = {}
    try:
        for var in ([0, 2, 1] if hd == 128 and T % 256 == 0 and win == 0 and Hkv == H else [0, 2]):
            B.attn_variant(1, var)
            D = torch.zeros(Bn * H * T, device="cuda")
            dqkv = torch.full((Bn * T, d + 2 * dkv), float("nan"), device="cuda", dtype=dq.dtype)
            B.attn_bwd(DT[dtype], dq, o, ddo, lse, D, dqkv, Bn, T, H, hd, win, n_kv=Hkv)
            torch.cuda.synchronize()
            out[var] = from_dev(dqkv)
    finally:
        B.attn_variant(1, 0)
    np.testing.assert_array_equal(out[0], out[2])
    assert np.isfinite(out[0]).all()
    if 1 in out:
        assert rel_l2(out[1], out[0]) < 1e-2


def test_attention_rejects_bad_kv_heads():
    t = torch.zeros(16, device="cuda")
    for H, Hkv in [(4, 3), (4, 0), (4, 8), (3, -1)]:
        with pytest.raises(B.GptError, match="argument"):
            B.attn_fwd(B.GPT_BF16, t, t, t, 1, 1, H, 128, 0, n_kv=Hkv)
        with pytest.raises(B.GptError, match="argument"):
            B.rope_qknorm_fwd(B.GPT_BF16, t, t, t, t, 1, 1, H, 128, 10000.0, 1e-6, n_kv=Hkv)


def test_attention_full_size_sampled_heads():
    """d24 shape (B=16, T=2048, 12 heads of 128) in the step's launch configuration;
    the oracle recomputes two (sequence, head) pairs."""
    Bn, T, H, hd = 16, 2048, 12, 128
    g = torch.Generator(device="cuda").manual_seed(3)
    qkv = torch.randn(Bn * T, 3 * H * hd, device="cuda", generator=g)
    qkv = qkv.bfloat16()
    o = torch.empty(Bn * T, H * hd, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(Bn * H * T, device="cuda")
    B.attn_fwd(B.GPT_BF16, qkv, o, lse, Bn, T, H, hd)
    torch.cuda.synchronize()
    x = qkv.float().cpu().numpy().astype(np.float64).reshape(Bn, T, 3, H, hd)
    og = o.float().cpu().numpy().reshape(Bn, T, H, hd)
    for (b, h) in [(0, 0), (Bn - 1, H - 1)]:
        q, k, v = (x[b:b + 1, :, i, h:h + 1] for i in range(3))
        ref, _ = O.causal_attention(q, k, v)
        assert rel_l2(og[b:b + 1, :, h:h + 1], ref) < 1e-2


# ----------------------------------------------------------------------------- norms


@pytest.mark.parametrize("dtype,N,d", [("bf16", 37, 1536), ("bf16", 64, 192), ("fp32", 29, 128),
                                       ("bf16", 5, 1664), ("fp32", 3, 2048)])
def test_rmsnorm_fwd_bwd(dtype, N, d):
    rng = np.random.default_rng(d + N)
    x = (rng.standard_normal((N, d)) * 2.5).astype(np.float32)
    dy = rng.standard_normal((N, d)).astype(np.float32)
    dres = rng.standard_normal((N, d)).astype(np.float32)
    y_ref, r_ref = O.rms_norm(x.astype(np.float64), 1e-6)
    dx_ref = O.rms_norm_bwd(dy.astype(np.float64), y_ref, r_ref) + dres
    tx, tdy, tres = (torch.from_numpy(a).cuda() for a in (x, dy, dres))
    y = torch.empty(N, d, device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    rstd = torch.empty(N, device="cuda")
    B.rmsnorm_fwd(DT[dtype], tx, y, rstd, N, d, 1e-6)
    dx = torch.empty(N, d, device="cuda")
    dxa = torch.empty_like(y)
    B.rmsnorm_bwd(DT[dtype], tdy, tx, rstd, tres, dx, dxa, N, d)
    torch.cuda.synchronize()
    assert rel_l2(from_dev(y), y_ref) < (4e-3 if dtype == "bf16" else 1e-6)
    assert np.abs(rstd.cpu().numpy() - r_ref[:, 0]).max() / r_ref.max() < 1e-6
    assert rel_l2(dx.cpu().numpy(), dx_ref) < 1e-5
    assert rel_l2(from_dev(dxa), dx_ref) < (4e-3 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("dtype,Bn,T,H,hd,Hkv", [("bf16", 2, 100, 3, 128, 3), ("bf16", 1, 64, 2, 64, 2),
                                                 ("fp32", 2, 40, 4, 32, 4), ("bf16", 1, 2048, 1, 128, 1),
                                                 ("bf16", 3, 37, 5, 32, 5), ("bf16", 1, 33, 7, 64, 7),
                                                 ("bf16", 2, 100, 6, 128, 2), ("bf16", 3, 37, 4, 32, 1),
                                                 ("bf16", 1, 33, 4, 64, 2), ("fp32", 2, 40, 4, 32, 1),
                                                 ("fp32", 1, 19, 6, 64, 3)])
def test_rope_qknorm_fwd_bwd(dtype, Bn, T, H, hd, Hkv):
    """Rows [q: H heads | k: Hkv heads | v: Hkv heads]; q and k are rotated and
    normalised head by head, v is left as it is."""
    rng = np.random.default_rng(T + Hkv)
    d, dkv = H * hd, Hkv * hd
    W = d + 2 * dkv
    qkv = _round(rng.standard_normal((Bn, T, W)) * 0.7, dtype)
    dqkv = _round(rng.standard_normal((Bn, T, W)), dtype)
    ang = O.rope_angles(T, hd, 10000.0)
    x = qkv.astype(np.float64)
    spans = [(0, d, H), (d, d + dkv, Hkv)]  # q, k
    outs = []
    for a, b, nh in spans:
        y, r = O.rms_norm(O.rope(x[..., a:b].reshape(Bn, T, nh, hd), ang), 1e-6)
        outs.append((y, r))
    tq = to_dev(qkv.reshape(Bn * T, W), dtype)
    cs = torch.empty(T * hd, device="cuda")
    rq = torch.empty(Bn * T * H, device="cuda")
    rk = torch.empty(Bn * T * Hkv, device="cuda")
    B.rope_qknorm_fwd(DT[dtype], tq, cs, rq, rk, Bn, T, H, hd, 10000.0, 1e-6, n_kv=Hkv)
    torch.cuda.synchronize()
    got = from_dev(tq).reshape(Bn, T, W)
    tol = 5e-3 if dtype == "bf16" else 2e-6
    for (a, b, nh), (y, r) in zip(spans, outs):
        assert rel_l2(got[..., a:b].reshape(Bn, T, nh, hd), y) < tol
    np.testing.assert_array_equal(got[..., d + dkv:], qkv[..., d + dkv:].astype(np.float64))   # v untouched
    for rt, (y, r), nh in ((rq, outs[0], H), (rk, outs[1], Hkv)):
        assert np.abs(rt.cpu().numpy().reshape(Bn, T, nh) - r[..., 0]).max() / r.max() < 1e-5
    # backward uses the kernel's normalised q, k as y (what the step saves)
    ddq = to_dev(dqkv.reshape(Bn * T, W), dtype)
    B.rope_qknorm_bwd(DT[dtype], ddq, tq, cs, rq, rk, Bn, T, H, hd, 10000.0, n_kv=Hkv)
    torch.cuda.synchronize()
    gg = from_dev(ddq).reshape(Bn, T, W)
    for (a, b, nh), (y, r) in zip(spans, outs):
        dy = dqkv[..., a:b].reshape(Bn, T, nh, hd).astype(np.float64)
        ref = O.rope(O.rms_norm_bwd(dy, y, r), ang, inverse=True)
        assert rel_l2(gg[..., a:b].reshape(Bn, T, nh, hd), ref) < (1e-2 if dtype == "bf16" else 1e-5)
    np.testing.assert_array_equal(gg[..., d + dkv:], dqkv[..., d + dkv:].astype(np.float64))


# ----------------------------------------------------------------------------- cross-entropy


# variant 0 takes the two-pass streaming kernel for V a multiple of 16384 (one or more
# groups of 16 float4 per thread; a later group raising the maximum rescales the sum),
# variant 1 the register-resident kernel
@pytest.mark.parametrize("dtype,N,V,variant", [("bf16", 40, 4096, 0), ("fp32", 33, 4096, 0), ("bf16", 9, 32768, 0),
                                               ("bf16", 9, 32768, 1), ("fp32", 9, 16384, 0), ("fp32", 9, 65536, 0),
                                               ("fp32", 7, 1000, 0)])
def test_cross_entropy_and_argmax(dtype, N, V, variant):
    rng = np.random.default_rng(V + N)
    z = (rng.standard_normal((N, V)) * 3).astype(np.float32)
    z[0, :] = 1.25                       # all tied -> index 0
    z[1, [7, 300, 901]] = 50.0           # tie among three -> 7
    z[2, V - 1] = 60.0                   # max at the last index
    z[6, [V // 2 + 5, V - 3]] = 40.0     # tie across the halves of the row -> the first
    y = rng.integers(0, V, N).astype(np.int32)
    y[3] = V - 1
    per_ref = O.loss_from_logits(z.astype(np.float64), y)[1]
    dz_ref = O.cross_entropy_grad(z.astype(np.float64), y)
    am_ref = O.argmax_lowest(z)
    tz, ty = torch.from_numpy(z).cuda(), torch.from_numpy(y).cuda()
    dz = torch.empty(N, V, device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    rl = torch.empty(N, device="cuda")
    am = torch.empty(N, device="cuda", dtype=torch.int32)
    err = torch.zeros(4, device="cuda", dtype=torch.int32)
    B.ce_variant(variant)
    try:
        B.cross_entropy(DT[dtype], tz, ty, dz, rl, am, N, V, 1.0 / N, err)
    finally:
        B.ce_variant(0)
    torch.cuda.synchronize()
    assert err.cpu().numpy()[0] == 0
    np.testing.assert_array_equal(am.cpu().numpy(), am_ref)
    assert np.abs(rl.cpu().numpy() - per_ref).max() < 1e-5 * np.abs(per_ref).max()
    assert rel_l2(from_dev(dz), dz_ref) < (4e-3 if dtype == "bf16" else 1e-6)
    # error flags: a target out of range, a non-finite logit
    y2 = y.copy(); y2[4] = V
    z2 = z.copy(); z2[5, 3] = np.inf
    B.cross_entropy(DT[dtype], torch.from_numpy(z2).cuda(), torch.from_numpy(y2).cuda(), dz, rl, am, N, V,
                    1.0 / N, err)
    torch.cuda.synchronize()
    assert err.cpu().numpy()[0] == 3


# ----------------------------------------------------------------------------- embedding


@pytest.mark.parametrize("N,V,d,dist", [(512, 4096, 128, "uniform"), (8192, 4096, 192, "zipf"),
                                        (2056, 32768, 1664, "zipf"), (32768, 32768, 1536, "zipf")])
def test_embedding_gather_scatter(N, V, d, dist):
    from gpt_pretraining_step_train_amd import inputs
    say("embedding", N, V, d, dist)
    tok, _ = inputs.token_batch(1, N, V, dist=dist, seed=5)
    tok = tok.reshape(-1)
    rng = np.random.default_rng(6)
    E = rng.standard_normal((V, d)).astype(np.float32)
    dh = rng.standard_normal((N, d)).astype(np.float32)
    tt = torch.from_numpy(tok).cuda()
    tE = torch.from_numpy(E).cuda()
    h = torch.empty(N, d, device="cuda")
    err = torch.zeros(4, device="cuda", dtype=torch.int32)
    B.embed_gather(tt, tE, h, N, d, V, err)
    ws = torch.empty(B.embed_ws_bytes(N, V, d), device="cuda", dtype=torch.uint8)
    dE = torch.full((V, d), float("nan"), device="cuda")
    srt = torch.empty(N, device="cuda", dtype=torch.int32)
    B.embed_scatter(tt, torch.from_numpy(dh).cuda(), dE, N, V, d, ws, srt)
    torch.cuda.synchronize()
    assert err.cpu().numpy()[0] == 0
    np.testing.assert_array_equal(h.cpu().numpy(), E[tok])                       # bit-exact copy
    np.testing.assert_array_equal(srt.cpu().numpy(), np.argsort(tok, kind="stable"))
    ref = np.zeros((V, d))
    np.add.at(ref, tok, dh.astype(np.float64))
    got = dE.cpu().numpy()
    absent = np.bincount(tok, minlength=V) == 0
    assert np.all(got[absent] == 0.0)
    assert np.abs(got - ref).max() < 1e-4 * max(1.0, np.sqrt(np.bincount(tok).max()))
    # determinism
    dE2 = torch.empty_like(dE)
    B.embed_scatter(tt, torch.from_numpy(dh).cuda(), dE2, N, V, d, ws, srt)
    torch.cuda.synchronize()
    assert torch.equal(dE, dE2)
    bad = tok.copy(); bad[7] = V
    B.embed_gather(torch.from_numpy(bad).cuda(), tE, h, N, d, V, err)
    torch.cuda.synchronize()
    assert err.cpu().numpy()[0] == 1


# ----------------------------------------------------------------------------- fp8 (e4m3)


def _e4m3_table():
    """Values of all 256 OCP e4m3fn codes (NaN for 0x7F / 0xFF), from the format's fields."""
    vals = np.empty(256)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            v = np.nan
        elif e == 0:
            v = m / 8 * 2.0 ** -6
        else:
            v = (1 + m / 8) * 2.0 ** (e - 7)
        vals[code] = -v if s else v
    return vals


def _e4m3_encode_ref(x):
    """Nearest representable value, ties to the even code (mantissa lsb 0), saturating at 448."""
    tab = _e4m3_table()
    pos = [c for c in range(128) if np.isfinite(tab[c])]
    pv = tab[pos]
    out = np.empty(x.shape, dtype=np.uint8)
    for idx, v in np.ndenumerate(x):
        a = min(abs(v), 448.0)
        dist = np.abs(pv - a)
        best = np.flatnonzero(dist == dist.min())
        code = pos[best[0]] if len(best) == 1 else [pos[b] for b in best if pos[b] % 2 == 0][0]
        out[idx] = code | (0x80 if v < 0 or (v == 0 and np.signbit(v)) else 0)
    return out


def _check_quant(x, dtype, pad=0, sample=None):
    """Quantise x (rows x cols, rows pad elements apart beyond cols, the padding holding
    values far above max|x| that must not enter the scale) through the library and
    compare every byte (or `sample` random bytes) with the format's round-to-nearest-even,
    saturating encode of x * (448 / amax) in fp32."""
    rows, cols = x.shape
    xr = bf16_round(x).astype(np.float32) if dtype == "bf16" else x.astype(np.float32)
    amax = np.abs(xr).max()
    s = np.float32(448.0) / np.float32(amax)
    full = np.full((rows, cols + pad), 1e30, dtype=np.float32)
    full[:, :cols] = xr
    tx = to_dev(full, dtype)
    slot = torch.zeros(1, dtype=torch.int32, device="cuda")
    inv = torch.zeros(1, device="cuda")
    q = torch.zeros(rows, cols, dtype=torch.uint8, device="cuda")
    qt = torch.zeros(cols, rows, dtype=torch.uint8, device="cuda")
    B.quant_e4m3(DT[dtype], tx, rows, cols, cols + pad, slot, q, qt, inv)
    torch.cuda.synchronize()
    assert inv.item() == pytest.approx(1.0 / s, rel=1e-6)
    got = q.cpu().numpy()
    np.testing.assert_array_equal(qt.cpu().numpy(), got.T)
    if sample is not None:
        idx = np.random.default_rng(0).integers(0, rows * cols, sample)
        xr, got = xr.reshape(-1)[idx], got.reshape(-1)[idx]
    want = _e4m3_encode_ref((xr * s).astype(np.float32))
    nz = want & 0x7F != 0          # signed zero: either sign of the zero code is accepted
    np.testing.assert_array_equal(got[nz], want[nz])
    assert np.all(got[~nz] & 0x7F == 0)


@pytest.mark.parametrize("dtype,rows,cols,pad", [("fp32", 67, 129, 0), ("fp32", 67, 136, 0), ("bf16", 130, 200, 0),
                                                 ("bf16", 64, 64, 0), ("bf16", 1, 8, 0), ("bf16", 300, 128, 8),
                                                 ("fp32", 70, 64, 16), ("bf16", 33, 72, 3), ("bf16", 129, 136, 0),
                                                 ("fp32", 256, 384, 0)])
def test_quant_e4m3_matches_format(dtype, rows, cols, pad):
    rng = np.random.default_rng(21 + cols)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-6, 4, (rows, cols)))
    x.flat[:3] = [0.0, -0.0, 1e-12][: x.size]
    _check_quant(x, dtype, pad)


@pytest.mark.parametrize("dtype,rows,cols,pad", [("bf16", 5000, 3200, 0), ("bf16", 2048, 6144, 0),
                                                 ("fp32", 4100, 1544, 0), ("bf16", 3000, 1536, 64)])
def test_quant_e4m3_large(dtype, rows, cols, pad):
    """Sizes where the amax pass runs whole grid-stride rounds plus a remainder (up to
    16M elements), the largest magnitude placed near the end; the scale is exact and
    sampled codes match the format."""
    rng = np.random.default_rng(rows)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[rows - 1, cols - 5] = -37.5
    _check_quant(x, dtype, pad, sample=3000)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_quant_e4m3_ties_and_subnormals(dtype):
    """amax = 448 makes the scale exactly 1: every midpoint between adjacent e4m3 values
    (normal and subnormal) is an exact tie that must round to the even code."""
    tab = _e4m3_table()
    pos = np.sort(tab[np.isfinite(tab) & (tab >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([[448.0], mids, -mids, pos, -pos, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    if dtype == "bf16":  # keep only values bf16 holds exactly (ties survive the input rounding)
        vals = vals[bf16_round(vals) == vals]
    n = (len(vals) + 7) // 8 * 8
    x = np.zeros(n)
    x[: len(vals)] = vals
    _check_quant(x.reshape(n // 8, 8), dtype)


FP8_GEMM_CASES = [(300, 200, 160, 1), (512, 768, 1024, 1), (1, 1, 16, 1), (257, 513, 48, 1), (768, 520, 4096, 3),
                  (264, 1040, 2064, 2), (256, 256, 208, 1)]


def _gemm_fp8(A, Bq, M, N, K, splits, dqa=0.5, dqb=0.25):
    C = torch.full((M, N), float("nan"), device="cuda")
    ws = torch.empty(splits * M * N, device="cuda") if splits > 1 else None
    B.gemm_fp8(M, N, K, torch.from_numpy(A).cuda(), K, torch.from_numpy(Bq).cuda(), K,
               torch.tensor([dqa], device="cuda"), torch.tensor([dqb], device="cuda"), C, N, splits, ws)
    torch.cuda.synchronize()
    return C.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K,splits", FP8_GEMM_CASES)
def test_gemm_fp8_exact_on_integers(M, N, K, splits):
    """Integer e4m3 values up to 16 in magnitude: every product is an integer of at
    most 256 and every partial sum an integer below 2^24, which the instruction's
    adder and fp32 hold exactly, so the result must be bit-exact.  Any tile, swizzle,
    k-tail or split-K mistake moves some output by a whole product."""
    tab = _e4m3_table()
    rng = np.random.default_rng(K)
    ints = np.array([c for c in range(256) if np.isfinite(tab[c]) and tab[c] == np.round(tab[c]) and abs(tab[c]) <= 16],
                    dtype=np.uint8)
    A = rng.choice(ints, size=(M, K))
    Bq = rng.choice(ints, size=(N, K))
    got = _gemm_fp8(A, Bq, M, N, K, splits, 0.5, 0.25)
    np.testing.assert_array_equal(got, tab[A] @ tab[Bq].T * 0.125)


@pytest.mark.parametrize("M,N,K,splits", FP8_GEMM_CASES)
def test_gemm_fp8_on_e4m3_values(M, N, K, splits):
    """Full-range e4m3 inputs decode exactly and every product of two e4m3 values is
    exact, so the only error is the accumulation.  The fp8 matrix instruction does not
    add its 64 products in full fp32: measured on random e4m3 operands, its error stays
    below 2^-10.9 of the largest |product| of each 64-wide k block.  The bound is 2^-10
    of the sum over blocks of that maximum, plus fp32 rounding of the block sums."""
    tab = _e4m3_table()
    rng = np.random.default_rng(M)
    finite = np.array([c for c in range(256) if np.isfinite(tab[c]) and abs(tab[c]) < 64], dtype=np.uint8)
    A = rng.choice(finite, size=(M, K))
    Bq = rng.choice(finite, size=(N, K))
    a, b = tab[A], tab[Bq]
    ref = a @ b.T * 0.125
    got = _gemm_fp8(A, Bq, M, N, K, splits, 0.5, 0.25)
    blockmax = np.zeros((M, N))
    for k0 in range(0, K, 64):
        pa = np.abs(a[:, k0:k0 + 64]).astype(np.float32)
        pb = np.abs(b[:, k0:k0 + 64]).astype(np.float32)
        blockmax += (pa[:, None, :] * pb[None, :, :]).max(-1)
    mag = np.abs(a) @ np.abs(b).T
    bound = (2.0 ** -10 * blockmax + 2.0 ** -20 * mag) * 0.125
    err = np.abs(got - ref)
    assert np.all(err <= bound)
    say(f"  fp8 accumulation error max {err.max():.3g} (max err/bound {np.max(err / bound):.2f}) of max|C| "
        f"{np.abs(ref).max():.3g}")


# ----------------------------------------------------------------------------- Newton-Schulz

# (dtype, rows, cols, kind): the d24 square, grouped-query Wk (wide), W1 (tall: run as its
# transpose) and W2 shapes, small ragged ones, and a low-rank-plus-noise momentum (the
# case whose small singular directions the fp32-carried X must keep)
NS_CASES = [("bf16", 1536, 1536, "gauss"), ("bf16", 512, 1536, "gauss"), ("bf16", 6144, 1536, "gauss"),
            ("bf16", 1536, 6144, "lowrank"), ("bf16", 136, 264, "gauss"), ("bf16", 264, 136, "lowrank"),
            ("fp32", 128, 512, "gauss"), ("fp32", 512, 128, "lowrank")]


@pytest.mark.parametrize("case", NS_CASES)
def test_newton_schulz_matches_the_oracle(case):
    """gptk_newton_schulz (the orthogonalisation muon_update runs on every block matrix)
    against the oracle's normalisation + Polar-Express iterations on the same matrix."""
    from oracle import polar_express as PE
    dtype, rows, cols, kind = case
    rng = np.random.default_rng(rows + 7 * cols)
    if kind == "gauss":
        G = rng.standard_normal((rows, cols))
    else:
        G = rng.standard_normal((rows, 16)) @ rng.standard_normal((16, cols)) + 0.05 * rng.standard_normal((rows, cols))
    G = G.astype(np.float32)
    table, _ = PE.coefficients()
    X = torch.empty(rows, cols, device="cuda")
    B.newton_schulz(DT[dtype], torch.from_numpy(G).cuda(), rows, cols, table, 5, X)
    ref, _ = O.muon_matrix(G, np.zeros_like(G, dtype=np.float64), table, mu=0.0)
    e = rel_l2(from_dev(X), ref)
    say(f"  NS {case}: rel L2 {e:.2e}")
    assert e < (1e-4 if dtype == "fp32" else 2e-2)
