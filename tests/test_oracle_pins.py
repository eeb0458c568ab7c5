"""Pins of the fp64 oracle against facts it does not itself define.

Each test checks the oracle against finite differences, closed forms,
library routines (torch CPU fp64, scipy, LAPACK SVD), invariants or brute
force, chosen so that a dropped term, a wrong sign or index or a transposed
operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import gpt_oracle as O
from oracle import polar_express as PE
from gpt_pretraining_step_train_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")

MICRO = dict(depth=1, d_model=16, n_head=2, head_dim=8, d_ff=64, vocab=64, seq_len=8,
             batch=2, norm_eps=1e-6, rope_base=10000.0, init_std=0.02)
MICRO2 = dict(MICRO, depth=2)
MICRO_W = dict(MICRO2, attn_window=3)  # sliding window: each query sees 3 keys
MICRO_G = dict(MICRO2, n_head=4, head_dim=4, n_kv_head=2)  # grouped-query attention, 2 heads per group
# residual scaling + smear + backout + value embeddings; the gates read 24 channels,
# so d = 32
MICRO_X1 = dict(MICRO, d_model=32, head_dim=16, extras=15)  # one layer: backout reads x0
MICRO_X = dict(MICRO_X1, depth=2)                           # backout reads layer 1's input
TINY = dict(depth=2, d_model=128, n_head=4, head_dim=32, d_ff=512, vocab=4096, seq_len=128,
            batch=4, norm_eps=1e-6, rope_base=10000.0, init_std=0.02)


def _params(cfg, seed=0, std=None, random_s=True):
    """Weights of the tensor table; the extras' tensors (when present) get random values
    instead of their inert start (S and the gate weights around 0.5, the value-embedding
    tables N(0, 0.5^2)), so that every extra acts."""
    c = dict(cfg)
    if std is not None:
        c["init_std"] = std
    ws = [w.astype(np.float64) for w in inputs.init_weights(c, seed)]
    if cfg.get("extras", 0) & 15 and random_s:
        rng = np.random.default_rng(seed + 1000)
        for i, (name, shape) in enumerate(inputs.tensor_shapes(cfg)):
            if name in ("S", "G"):
                ws[i] = 0.5 + 0.3 * rng.standard_normal(shape)
            elif name.endswith(".VE"):
                ws[i] = 0.5 * rng.standard_normal(shape)
    return ws


def _tokens(cfg, seed=0, dist="uniform"):
    return inputs.token_batch(cfg["batch"], cfg["seq_len"], cfg["vocab"], dist=dist, seed=seed)


# --------------------------------------------------------------------------
# P1: the whole backward against centred finite differences


@pytest.mark.parametrize("cfg", [MICRO, MICRO2, MICRO_W, MICRO_G, MICRO_X1, MICRO_X])
def test_fd_gradient_every_element(cfg):
    params = _params(cfg, seed=1, std=0.5)          # large weights: non-linear regime
    tok, tgt = _tokens(cfg, seed=2)
    tok[0, 3] = tok[0, 5] = tok[1, 0]               # repeated ids exercise the scatter-add
    loss, grads, _, _ = O.loss_and_grads(params, tok, tgt, cfg)
    h = 1e-5
    for ti, (w, g) in enumerate(zip(params, grads)):
        fd = np.zeros_like(w)
        it = np.nditer(w, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = w[idx]
            w[idx] = old + h
            lp = O.loss_only(params, tok, tgt, cfg)
            w[idx] = old - h
            lm = O.loss_only(params, tok, tgt, cfg)
            w[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        rel = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-300)
        assert rel <= 1e-6, (ti, rel)


def test_fd_gradient_directions_tiny():
    cfg = TINY
    params = _params(cfg, seed=3, std=0.1)
    tok, tgt = _tokens(cfg, seed=4)
    loss, grads, _, _ = O.loss_and_grads(params, tok, tgt, cfg)
    rng = np.random.default_rng(5)
    h = 1e-5
    for ti in range(len(params)):
        gn = np.linalg.norm(grads[ti])
        for j in range(3):
            # the gradient direction itself, then random directions; the error is
            # measured against |grad| (the largest directional derivative)
            v = grads[ti] / gn if j == 0 else rng.standard_normal(params[ti].shape)
            v = v / np.linalg.norm(v)
            w0 = params[ti]
            params[ti] = w0 + h * v
            lp = O.loss_only(params, tok, tgt, cfg)
            params[ti] = w0 - h * v
            lm = O.loss_only(params, tok, tgt, cfg)
            params[ti] = w0
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(grads[ti] * v))
            assert abs(fd - an) <= 1e-6 * gn, (ti, j, fd, an, gn)


# --------------------------------------------------------------------------
# P2: zero LM head => uniform prediction


def test_zero_head_gives_ln_vocab_and_closed_form_grads():
    gold = json.load(open(os.path.join(GOLD, "vocab_and_uniform_loss.json")))
    cfg = dict(TINY)
    params = _params(cfg, seed=7, std=0.05)
    params[-1][:] = 0.0
    tok, tgt = _tokens(cfg, seed=8)
    loss, grads, am, _ = O.loss_and_grads(params, tok, tgt, cfg)
    assert loss == pytest.approx(gold["small_uniform_loss"], abs=1e-12)
    assert math.log(cfg["vocab"]) == pytest.approx(gold["small_uniform_loss"], abs=1e-12)
    for g in grads[:-1]:
        assert np.all(g == 0.0)
    assert np.all(am == 0)                  # all logits tie -> lowest index
    # dU = (1/N) sum_n (1/V - e_{y_n}) r_n^T, r_n = final-norm output
    z, cache = O.forward(params, tok, cfg)
    N = tok.size
    r = cache["r"].reshape(N, -1)
    want = np.tile(r.sum(0) / cfg["vocab"], (cfg["vocab"], 1))
    np.subtract.at(want, tgt.reshape(-1), r)
    want /= N
    np.testing.assert_allclose(grads[-1], want, rtol=1e-12, atol=1e-15)


def test_zero_head_at_32768_vocab():
    gold = json.load(open(os.path.join(GOLD, "vocab_and_uniform_loss.json")))
    cfg = dict(MICRO, vocab=gold["vocab"])
    params = _params(cfg, seed=9)
    params[-1][:] = 0.0
    tok, tgt = _tokens(cfg, seed=10, dist="zipf")
    z, _ = O.forward(params, tok, cfg)
    assert O.loss_from_logits(z, tgt)[0] == pytest.approx(gold["uniform_loss"], abs=1e-12)


# --------------------------------------------------------------------------
# P3: initial loss near ln V + s^2/2 (logits ~ N(0, 0.02^2 d), unit-RMS final norm)


def test_initial_loss_statistics():
    cfg = TINY
    params = _params(cfg, seed=0)
    tok, tgt = _tokens(cfg, seed=0)
    z, _ = O.forward(params, tok, cfg)
    loss = O.loss_from_logits(z, tgt)[0]
    want = math.log(cfg["vocab"]) + 0.5 * 0.02 ** 2 * cfg["d_model"]
    assert abs(loss - want) < 0.03, (loss, want)


# --------------------------------------------------------------------------
# P4: causality


@pytest.mark.parametrize("extras", [0, 15])
def test_causality_exact(extras):
    """Changing token t+1 leaves every logit up to position t unchanged (with the
    extras: the smear mixes only the previous position into the current one)."""
    cfg = dict(TINY, extras=extras)
    params = _params(cfg, seed=11, std=0.2)
    tok, _ = _tokens(cfg, seed=12)
    z0, _ = O.forward(params, tok, cfg, keep=False)
    t = 57
    tok2 = tok.copy()
    tok2[:, t + 1] = (tok2[:, t + 1] + 17) % cfg["vocab"]
    z1, _ = O.forward(params, tok2, cfg, keep=False)
    assert np.array_equal(z0[:, : t + 1], z1[:, : t + 1])
    assert not np.array_equal(z0[:, t + 1], z1[:, t + 1])


# --------------------------------------------------------------------------
# P5: attention special cases and a library routine


def test_attention_special_cases_and_sdpa():
    rng = np.random.default_rng(0)
    B, T, H, hd = 2, 9, 3, 8
    q, k, v = (rng.standard_normal((B, T, H, hd)) for _ in range(3))
    o, _ = O.causal_attention(q[:, :1], k[:, :1], v[:, :1])
    np.testing.assert_array_equal(o, v[:, :1])                    # T = 1 -> o = v
    o, _ = O.causal_attention(np.zeros_like(q), k, v)               # q = 0 -> running mean
    want = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-14)
    o, _ = O.causal_attention(q, k, v)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-13)
    # brute force on one (b, h, i)
    b, h, i = 1, 2, 6
    s = np.array([np.dot(q[b, i, h], k[b, j, h]) / math.sqrt(hd) for j in range(i + 1)])
    w = np.exp(s - s.max())
    w /= w.sum()
    np.testing.assert_allclose(o[b, i, h], sum(w[j] * v[b, j, h] for j in range(i + 1)),
                               rtol=1e-12)


def test_sliding_window_attention_pins():
    """window = 1: every query sees only itself (o = v); window >= T: plain causal
    attention; and the window edge is exact: a key just outside query i's window
    (j = i - window) leaves o_i unchanged, a key just inside (j = i - window + 1)
    changes it."""
    rng = np.random.default_rng(4)
    B, T, H, hd = 2, 11, 2, 8
    q, k, v = (rng.standard_normal((B, T, H, hd)) for _ in range(3))
    o1, _ = O.causal_attention(q, k, v, window=1)
    np.testing.assert_allclose(o1, v, rtol=1e-14, atol=1e-15)
    full, _ = O.causal_attention(q, k, v)
    for w in (T, T + 5):
        ow, _ = O.causal_attention(q, k, v, window=w)
        np.testing.assert_array_equal(ow, full)
    W, i = 4, 8
    base, _ = O.causal_attention(q, k, v, window=W)
    for j, moves in ((i - W, False), (i - W + 1, True)):
        k2, v2 = k.copy(), v.copy()
        k2[:, j] += 1.0
        v2[:, j] += 1.0
        o2, _ = O.causal_attention(q, k2, v2, window=W)
        changed = not np.array_equal(o2[:, i], base[:, i])
        assert changed == moves, (j, changed)
    assert not np.array_equal(base, full)  # the window binds at T = 11


@pytest.mark.parametrize("n_kv", [1, 2])
def test_grouped_query_attention_is_mha_with_shared_heads(n_kv):
    """A model with n_kv key/value heads computes what the multi-head model computes
    when each of its Wk/Wv head blocks is copied to the n_head / n_kv query heads
    that share it; its Wk/Wv gradients are the sums of those copies' gradients and
    every other gradient is the same."""
    cfg = dict(MICRO2, n_head=4, head_dim=4, n_kv_head=n_kv)
    mha = dict(cfg, n_kv_head=0)
    H, hd, d, G = 4, 4, 16, 4 // n_kv
    params = _params(cfg, seed=7, std=0.3)
    tok, tgt = _tokens(cfg, seed=8)
    widen = lambda W: np.repeat(W.reshape(n_kv, hd, d), G, axis=0).reshape(H * hd, d)
    wide = [widen(w) if (i - 1) % 6 in (1, 2) and 0 < i < len(params) - 1 else w for i, w in enumerate(params)]
    assert wide[2].shape == (H * hd, d) and params[2].shape == (n_kv * hd, d)
    loss, grads, _, _ = O.loss_and_grads(params, tok, tgt, cfg)
    loss_m, grads_m, _, _ = O.loss_and_grads(wide, tok, tgt, mha)
    assert loss == pytest.approx(loss_m, rel=1e-13)
    for i, (g, gm) in enumerate(zip(grads, grads_m)):
        if 0 < i < len(params) - 1 and (i - 1) % 6 in (1, 2):
            gm = gm.reshape(n_kv, G, hd, d).sum(axis=1).reshape(n_kv * hd, d)
        np.testing.assert_allclose(g, gm, rtol=1e-11, atol=1e-14, err_msg=f"tensor {i}")


def test_attention_backward_vs_autograd():
    rng = np.random.default_rng(1)
    B, T, H, hd = 2, 7, 2, 4
    q, k, v, do = (rng.standard_normal((B, T, H, hd)) for _ in range(4))
    o, _ = O.causal_attention(q, k, v)
    dq, dk, dv = O.causal_attention_bwd(do, q, k, v, o)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    ref.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# P6: RMSNorm, RoPE, QK-norm invariants


def test_rmsnorm_library_and_closed_form():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 33)) * 3
    y, r = O.rms_norm(x, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), np.sqrt(ms / (ms + 1e-6)), rtol=1e-13)
    # backward against autograd
    tx = torch.from_numpy(x).requires_grad_()
    dy = rng.standard_normal(x.shape)
    torch.nn.functional.rms_norm(tx, (33,), eps=1e-6).backward(torch.from_numpy(dy))
    np.testing.assert_allclose(O.rms_norm_bwd(dy, y, r), tx.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_rope_pairing_frequencies_and_relative_property():
    T, hd, base = 11, 8, 10000.0
    ang = O.rope_angles(T, hd, base)
    x = np.zeros((1, T, 1, hd))
    x[..., 0] = 1.0          # unit vector on the first pair (frequency base^0 = 1)
    y = O.rope(x, ang)
    t = np.arange(T)
    np.testing.assert_allclose(y[0, :, 0, 0], np.cos(t), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(y[0, :, 0, hd // 2], np.sin(t), rtol=1e-14, atol=1e-15)
    x = np.zeros((1, T, 1, hd))
    x[..., hd // 2 + 1] = 1.0  # second element of pair 1 (frequency base^(-2/hd))
    y = O.rope(x, ang)
    f1 = base ** (-2.0 / hd)
    np.testing.assert_allclose(y[0, :, 0, 1], -np.sin(t * f1), atol=1e-15)
    np.testing.assert_allclose(y[0, :, 0, hd // 2 + 1], np.cos(t * f1), atol=1e-15)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, T, 1, hd))
    np.testing.assert_array_equal(O.rope(q, ang)[0, 0], q[0, 0])      # position 0: identity
    np.testing.assert_allclose(O.rope(O.rope(q, ang), ang, inverse=True), q, rtol=1e-13, atol=1e-14)
    k = rng.standard_normal((1, T, 1, hd))
    qq = np.repeat(q[:, :1], T, axis=1)
    kk = np.repeat(k[:, :1], T, axis=1)
    rq, rk = O.rope(qq, ang), O.rope(kk, ang)
    dots = np.einsum("btd,bsd->ts", rq[:, :, 0], rk[:, :, 0])
    for dlt in range(-3, 4):
        dd = np.diagonal(dots, offset=dlt)
        np.testing.assert_allclose(dd, dd[0], rtol=1e-12, atol=1e-13)   # depends on m - n only
    # norm commutes with the rotation
    a, _ = O.rms_norm(O.rope(q, ang), 1e-6)
    b = O.rope(O.rms_norm(q, 1e-6)[0], ang)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# P7: cross-entropy against library routines


def test_cross_entropy_library():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((3, 5, 97)) * 4
    y = rng.integers(0, 97, (3, 5))
    loss, per = O.loss_from_logits(z, y)
    ref = scipy.special.logsumexp(z, axis=-1) - np.take_along_axis(z, y[..., None], -1)[..., 0]
    np.testing.assert_allclose(per, ref, rtol=1e-14)
    tl = torch.nn.functional.cross_entropy(torch.from_numpy(z.reshape(-1, 97)),
                                           torch.from_numpy(y.reshape(-1)))
    assert loss == pytest.approx(float(tl), rel=1e-14)


def test_argmax_lowest_index():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [0.0, -1.0, 0.5, 0.5]])
    assert O.argmax_lowest(z).tolist() == [1, 0, 2]


# --------------------------------------------------------------------------
# P8: Newton-Schulz


def _composed(coeffs, s):
    for abc in coeffs:
        s = PE.quintic(s, abc)
    return s


def test_polar_express_table_printed_prefix_and_band():
    gold = json.load(open(os.path.join(GOLD, "ns_printed_coeffs.json")))
    table, iv = PE.coefficients(gold["ns_steps"])
    assert [list(t) for t in table[:2]] == gold["printed"]
    lo, hi = iv[-1]
    assert 0.85 < lo < 0.9 and 1.1 < hi < 1.15
    # each derived step is minimax: the error equioscillates (max |1-p| reached >= 4 times)
    for k in range(2, 5):
        l0, h0 = iv[k]
        x = np.geomspace(l0, h0, 20001)
        e = 1 - PE.quintic(x, table[k])
        emax = np.abs(e).max()
        peaks = np.sum((np.abs(e[1:-1]) >= np.abs(e[:-2])) & (np.abs(e[1:-1]) >= np.abs(e[2:]))
                       & (np.abs(e[1:-1]) > 0.999 * emax)) + (abs(e[0]) > 0.999 * emax) + (abs(e[-1]) > 0.999 * emax)
        assert peaks >= 4, (k, peaks)


def test_newton_schulz_closed_form_band_and_symmetries():
    table, _ = PE.coefficients()
    rng = np.random.default_rng(6)
    G = rng.standard_normal((24, 40))
    X0 = G / np.linalg.norm(G)
    X = O.newton_schulz(X0, table)
    U, S, Vt = np.linalg.svd(X0, full_matrices=False)
    np.testing.assert_allclose(X, (U * _composed(table, S)) @ Vt, rtol=1e-11, atol=1e-12)
    sv = np.linalg.svd(X, compute_uv=False)
    keep = S >= 1e-3
    assert np.all(sv[keep] > 0.85) and np.all(sv[keep] < 1.15)
    # scale invariance of the normalised direction, transpose and orthogonal equivariance
    Xa, _ = O.muon_matrix(3.7 * G, np.zeros_like(G), table, mu=0.95)
    Xb, _ = O.muon_matrix(G, np.zeros_like(G), table, mu=0.95)
    np.testing.assert_allclose(Xa, Xb, rtol=0, atol=1e-7)   # up to eps=1e-7 in the normaliser
    Xt, _ = O.muon_matrix(G.T, np.zeros_like(G.T), table)
    np.testing.assert_allclose(Xt, Xb.T, rtol=1e-10, atol=1e-11)
    P, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    Q, _ = np.linalg.qr(rng.standard_normal((40, 40)))
    Xpq, _ = O.muon_matrix(P @ G @ Q, np.zeros_like(G), table)
    np.testing.assert_allclose(Xpq, P @ Xb @ Q, rtol=1e-9, atol=1e-10)
    # the two Gram orientations agree
    Y = X0.copy()
    for (a, b, c) in table:
        A = Y @ Y.T
        Y = a * Y + (b * A + c * A @ A) @ Y
    np.testing.assert_allclose(Y, X, rtol=1e-11, atol=1e-12)


def test_newton_schulz_textbook_quintic():
    # with the fixed quintic (15x - 10x^3 + 3x^5)/8 repeated, NS converges to the polar factor
    rng = np.random.default_rng(8)
    G = rng.standard_normal((6, 9)) + 3 * np.eye(6, 9)
    X0 = G / np.linalg.norm(G, 2)     # spectral normalisation -> sigma in (0, 1]
    X = O.newton_schulz(X0, [(15 / 8, -10 / 8, 3 / 8)] * 60)
    U, _, Vt = np.linalg.svd(G, full_matrices=False)
    np.testing.assert_allclose(X, U @ Vt, atol=1e-10)


# --------------------------------------------------------------------------
# P9: momentum


def test_momentum_heavy_ball():
    table, _ = PE.coefficients()
    rng = np.random.default_rng(9)
    G1, G2 = rng.standard_normal((2, 8, 12))
    _, B1 = O.muon_matrix(G1, np.zeros_like(G1), table, mu=0.95)
    np.testing.assert_array_equal(B1, G1)
    X2, B2 = O.muon_matrix(G2, B1, table, mu=0.95)
    np.testing.assert_allclose(B2, 0.95 * G1 + G2, rtol=1e-15)
    # EMA form B <- mu B + (1-mu) G gives the same direction (normalisation is scale-free;
    # eps = 0 removes the only scale-dependent term)
    Xe, _ = O.muon_matrix(0.05 * G2, 0.05 * B1, table, mu=0.95, eps=0.0)
    Xh, _ = O.muon_matrix(G2, B1, table, mu=0.95, eps=0.0)
    np.testing.assert_allclose(Xe, Xh, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Xh, X2, rtol=0, atol=1e-5)


def test_muon_update_touches_only_block_matrices():
    cfg = MICRO2
    table, _ = PE.coefficients()
    params = _params(cfg, seed=3)
    rng = np.random.default_rng(1)
    grads = [rng.standard_normal(w.shape) for w in params]
    moms = [np.zeros_like(w) for w in params]
    newp, newm, dirs = O.muon_update(params, grads, moms, cfg, 0.02, table)
    np.testing.assert_array_equal(newp[0], params[0])
    np.testing.assert_array_equal(newp[-1], params[-1])
    for i in range(1, len(params) - 1):
        np.testing.assert_allclose(newp[i], params[i] - 0.02 * dirs[i], rtol=1e-15)
        np.testing.assert_array_equal(newm[i], grads[i])


# --------------------------------------------------------------------------
# P11: whole-model gradient against torch fp64 autograd; structural special cases


def _torch_loss(params, tok, tgt, cfg):
    """An independent torch formulation using library ops (rms_norm, SDPA, cross_entropy)."""
    E, U = params[0], params[-1]
    L, H, hd, d = cfg["depth"], cfg["n_head"], cfg["head_dim"], cfg["d_model"]
    B, T = tok.shape
    eps = cfg["norm_eps"]
    pos = torch.arange(T, dtype=torch.float64)
    inv = cfg["rope_base"] ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = pos[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[None, :, None, :]
    sin = torch.cat([ang.sin(), ang.sin()], -1)[None, :, None, :]

    def rot(x):
        x1, x2 = x[..., : hd // 2], x[..., hd // 2:]
        return x * cos + torch.cat([-x2, x1], -1) * sin

    rms = lambda x: torch.nn.functional.rms_norm(x, (x.shape[-1],), eps=eps)
    ex = cfg.get("extras", 0)
    if ex:
        U, S = params[1 + 6 * L], params[2 + 6 * L][0]
        lam_r, lam_0, lam_s, lam_b, w_s = S[:L], S[L:2 * L], S[2 * L], S[2 * L + 1], S[2 * L + 2:]
    if ex & 8:
        ve_tabs, gates = params[3 + 6 * L: 3 + 7 * L], params[3 + 7 * L].view(L, H, 24)
    x = E[torch.from_numpy(tok).long()]
    if ex & 2:   # previous position's embedding, zero-padded at the start of each sequence
        shifted = torch.nn.functional.pad(x, (0, 0, 1, 0))[:, :-1]
        x = x + lam_s * torch.sigmoid(x[..., :24] @ w_s)[..., None] * shifted
    x0 = x
    for l in range(L):
        Wq, Wk, Wv, Wo, W1, W2 = params[1 + 6 * l: 7 + 6 * l]
        if ex & 4 and l == L // 2:
            x_mid = x
        if ex & 1:
            x = lam_r[l] * x + lam_0[l] * x0
        a = rms(x)
        q = rms(rot((a @ Wq.T).view(B, T, H, hd)))
        k = rms(rot((a @ Wk.T).view(B, T, H, hd)))
        v = (a @ Wv.T).view(B, T, H, hd)
        if ex & 8:  # torch.nn.functional.embedding lookup and a sigmoid gate per head
            ve = torch.nn.functional.embedding(torch.from_numpy(tok).long(), ve_tabs[l]).view(B, T, H, hd)
            v = v + (3 * torch.sigmoid(a[..., :24] @ gates[l].T)).unsqueeze(-1) * ve
        o = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=True)
        x = x + o.transpose(1, 2).reshape(B, T, d) @ Wo.T
        x = x + torch.relu(rms(x) @ W1.T).square() @ W2.T
    if ex & 4:
        x = x - lam_b * x_mid
    z = rms(x) @ U.T
    return torch.nn.functional.cross_entropy(z.reshape(B * T, -1),
                                             torch.from_numpy(tgt).long().reshape(-1))


@pytest.mark.parametrize("extras", [0, 15])
def test_full_gradient_vs_torch_autograd(extras):
    cfg = dict(TINY, extras=extras)
    params = _params(cfg, seed=21, std=0.1)
    tok, tgt = _tokens(cfg, seed=22, dist="zipf")
    loss, grads, _, _ = O.loss_and_grads(params, tok, tgt, cfg)
    tp = [torch.from_numpy(w.copy()).requires_grad_() for w in params]
    tl = _torch_loss(tp, tok, tgt, cfg)
    tl.backward()
    assert loss == pytest.approx(tl.item(), rel=1e-12)
    for g, t in zip(grads, tp):
        rel = np.linalg.norm(g - t.grad.numpy()) / np.linalg.norm(t.grad.numpy())
        assert rel < 1e-10


def test_identity_blocks_reduce_to_embedding_head():
    cfg = TINY
    params = _params(cfg, seed=23, std=0.3)
    for l in range(cfg["depth"]):
        params[1 + 6 * l + 3][:] = 0.0     # Wo
        params[1 + 6 * l + 5][:] = 0.0     # W2
    tok, tgt = _tokens(cfg, seed=24)
    z, _ = O.forward(params, tok, cfg)
    x = params[0][tok]
    r = x / np.sqrt(np.mean(x * x, -1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(z, r @ params[-1].T, rtol=1e-12, atol=1e-13)
    per = scipy.special.logsumexp(z, -1) - np.take_along_axis(z, tgt[..., None], -1)[..., 0]
    assert O.loss_from_logits(z, tgt)[0] == pytest.approx(per.mean(), rel=1e-14)


# --------------------------------------------------------------------------
# extras: residual scaling, smear, backout


def test_extras_at_their_start_values_are_the_plain_model():
    """S at its identity start (residual scales 1, the rest 0): loss and every
    other gradient equal the plain model's bit for bit, whichever extras are on."""
    base = dict(MICRO_X, extras=0)
    pb = _params(base, seed=3, std=0.4)
    tok, tgt = _tokens(base, seed=4)
    lb, gb, _, _ = O.loss_and_grads(pb, tok, tgt, base)
    for ex in (1, 2, 4, 7, 8, 15):
        cfg = dict(MICRO_X, extras=ex)
        p = _params(cfg, seed=3, std=0.4, random_s=False)
        l, g, _, _ = O.loss_and_grads(p, tok, tgt, cfg)
        assert l == lb
        for x, y in zip(g, gb):  # the plain model's tensors lead the table
            np.testing.assert_array_equal(x, y)


def test_residual_scaling_can_skip_a_layer():
    """lr = (1, 0), l0 = (0, 1): the second layer reads x0 alone and the first
    layer's output is dropped, so the two-layer model is the one-layer plain model
    built from the second layer's weights."""
    cfg = dict(MICRO_X, extras=1)
    p = _params(cfg, seed=5, std=0.4)
    L = 2
    S = np.zeros(2 * L + 26)
    S[:L] = (1.0, 0.0)
    S[L:2 * L] = (0.0, 1.0)
    p[-1] = S[None, :]
    one = dict(MICRO_X, depth=1, extras=0)
    p1 = [p[0]] + p[7:13] + [p[13]]
    tok, tgt = _tokens(cfg, seed=6)
    z, _ = O.forward(p, tok, cfg)
    z1, _ = O.forward(p1, tok, one)
    np.testing.assert_allclose(z, z1, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("depth", [1, 2, 3])
def test_backout_subtracts_the_middle_stream(depth):
    """lb = 1: the final norm reads x_L - x_mid, x_mid the stream entering layer
    L // 2, both taken from the plain model's own forward."""
    base = dict(MICRO_X, depth=depth, extras=0)
    cfg = dict(base, extras=4)
    p = _params(cfg, seed=7, std=0.4, random_s=False)
    p[-1][0, 2 * depth + 1] = 1.0                     # backout scale
    tok, tgt = _tokens(cfg, seed=8)
    z, _ = O.forward(p, tok, cfg)
    _, cache = O.forward(p[:-1], tok, base)
    mid = cache["layers"][depth // 2]["h"]
    x = cache["hL"] - mid
    r = x / np.sqrt(np.mean(x * x, -1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(z, r @ p[-2].T, rtol=1e-12, atol=1e-14)


def test_value_embedding_reproduces_the_first_layers_values():
    """Layer 0 (no residual scaling, no smear) reads a = rms(E[token]), a function of the
    token alone, so its values a Wv^T are a table lookup: with Wv = 0, gate weights 0
    (gate 3 sigmoid(0) = 1.5) and VE_0 = rms(E) Wv^T / 1.5 (other layers' tables 0),
    the value-embedding model computes the plain model's logits."""
    base = dict(MICRO_X, extras=0)
    cfg = dict(MICRO_X, extras=8)
    p = _params(base, seed=11, std=0.4)
    tok, tgt = _tokens(cfg, seed=12)
    z, _ = O.forward(p, tok, base)
    q = [w.copy() for w in _params(cfg, seed=11, std=0.4, random_s=False)]
    E, Wv = p[0], p[3]
    L = cfg["depth"]
    r = E / np.sqrt(np.mean(E * E, -1, keepdims=True) + 1e-6)
    q[3] = np.zeros_like(Wv)
    q[3 + 6 * L] = (r @ Wv.T) / 1.5
    z2, _ = O.forward(q, tok, cfg)
    np.testing.assert_allclose(z2, z, rtol=1e-12, atol=1e-14)


def test_smear_with_a_constant_gate_is_a_bigram_embedding():
    """Smear gate weights 0 (sigmoid = 1/2) and scale 2: position t reads
    E[x_t] + E[x_(t-1)], which is the plain model on the pair ids x_(t-1) V + x_t
    with the pair table E2[a V + b] = E[a] + E[b], and V^2 + x_0 for the first
    position (E2 row E[x_0])."""
    cfg = dict(MICRO_X, extras=2)
    V, d = cfg["vocab"], cfg["d_model"]
    p = _params(cfg, seed=9, std=0.4, random_s=False)
    p[-1][0, 2 * cfg["depth"]] = 2.0                  # smear scale; gate weights stay 0
    tok, tgt = _tokens(cfg, seed=10)
    E = p[0]
    E2 = np.concatenate([(E[:, None, :] + E[None, :, :]).reshape(V * V, d), E])
    pair = np.empty_like(tok)
    pair[:, 1:] = tok[:, :-1] * V + tok[:, 1:]
    pair[:, 0] = V * V + tok[:, 0]
    big = dict(cfg, extras=0, vocab=V * V + V)
    z, _ = O.forward(p, tok, cfg)
    z2, _ = O.forward([E2] + p[1:-1], pair, big)
    np.testing.assert_allclose(z, z2, rtol=1e-13, atol=1e-15)


def test_normuon_closed_forms():
    """NorMuon keeps the Frobenius norm for any buffer and decay; with decay 0 every
    row of the result has the same norm; a single row, or rows of equal mean square
    with a buffer proportional to them, pass unchanged; and a frozen buffer (decay 1)
    scales row i by 1/sqrt(V_i) up to the common factor that keeps the norm."""
    rng = np.random.default_rng(41)
    X = rng.standard_normal((9, 13)) * rng.uniform(0.05, 4.0, (9, 1))
    for b2, V in ((0.0, np.zeros(9)), (0.9, rng.uniform(0, 3, 9)), (0.5, np.zeros(9))):
        Y, _ = O.normuon(X, V, b2)
        assert np.linalg.norm(Y) == pytest.approx(np.linalg.norm(X), rel=1e-13)
    Y, V1 = O.normuon(X, np.zeros(9), 0.0)
    np.testing.assert_allclose(np.linalg.norm(Y, axis=1), np.linalg.norm(X) / 3.0, rtol=1e-13)
    np.testing.assert_allclose(V1, np.mean(X * X, axis=1), rtol=1e-15)
    row = X[:1]
    np.testing.assert_allclose(O.normuon(row, np.zeros(1), 0.3)[0], row, rtol=1e-13)
    U = rng.standard_normal((6, 8))
    U /= np.linalg.norm(U, axis=1, keepdims=True)                # equal mean squares
    np.testing.assert_allclose(O.normuon(U, np.full(6, 0.7), 0.6)[0], U, rtol=1e-13)
    V0 = rng.uniform(0.5, 2.0, 9)
    Y, V2 = O.normuon(X, V0, 1.0)
    np.testing.assert_array_equal(V2, V0)
    Z = X / np.sqrt(V0)[:, None]
    np.testing.assert_allclose(Y, Z * np.linalg.norm(X) / np.linalg.norm(Z), rtol=1e-13)


# --------------------------------------------------------------------------
# P12: batch symmetry


def test_batch_row_swap_symmetry():
    cfg = TINY
    params = _params(cfg, seed=31, std=0.1)
    tok, tgt = _tokens(cfg, seed=32)
    l0, g0, a0, p0 = O.loss_and_grads(params, tok, tgt, cfg)
    perm = [2, 0, 3, 1]
    l1, g1, a1, p1 = O.loss_and_grads(params, tok[perm], tgt[perm], cfg)
    assert l1 == pytest.approx(l0, rel=1e-13)
    np.testing.assert_array_equal(a1, a0[perm])
    np.testing.assert_allclose(p1, p0[perm], rtol=1e-13)
    for x, y in zip(g0, g1):
        np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-14)


# --------------------------------------------------------------------------
# fp8: the e4m3 model and the fp8 oracle step


def _e4m3_code_values():
    """Decode all 126 non-negative finite e4m3fn codes from the bit fields
    (bias 7, 3 fraction bits, exponent field 0 subnormal, code 0x7F NaN)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def test_e4m3_round_matches_torch_cast():
    from oracle.e4m3 import e4m3_round
    grid = _e4m3_code_values()
    assert grid[-1] == 448.0 and grid[1] == 2.0 ** -9 and np.all(np.diff(grid) > 0)
    np.testing.assert_array_equal(e4m3_round(grid), grid)                # every value is a fixed point
    np.testing.assert_array_equal(e4m3_round(-grid), -grid)
    mids = (grid[:-1] + grid[1:]) / 2                                    # exact ties
    rng = np.random.default_rng(5)
    x = np.concatenate([mids, -mids, rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2, 20000)])
    x = np.clip(x, -440.0, 440.0).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x).float().to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(e4m3_round(x), want)
    even = e4m3_round(mids)                                              # ties go to the even code
    codes = np.searchsorted(grid, even)
    assert np.all(codes % 2 == 0)


def test_e4m3_saturation_and_quantise_invariants():
    from oracle.e4m3 import e4m3_round, quantise
    np.testing.assert_array_equal(e4m3_round(np.array([448.0, 463.9, 464.0, 1e6, -500.0])),
                                  [448.0, 448.0, 448.0, 448.0, -448.0])
    rng = np.random.default_rng(6)
    t = rng.standard_normal((64, 48)) * 0.02
    q = quantise(t)
    i = np.unravel_index(np.argmax(np.abs(t)), t.shape)
    assert q[i] == pytest.approx(t[i], rel=1e-15)                         # amax lands on 448 exactly
    big = np.abs(t) >= np.abs(t[i]) * 2.0 ** -6 / 448                     # normal range after scaling
    assert np.all(np.abs(q - t)[big] <= np.abs(t)[big] * 2.0 ** -4 + 1e-18)
    np.testing.assert_array_equal(quantise(t * 2.0 ** 7), q * 2.0 ** 7)  # per-tensor scale invariance
    np.testing.assert_array_equal(quantise(np.zeros((3, 4))), np.zeros((3, 4)))
    assert len(np.unique(np.round(quantise(t) * 448 / np.abs(t[i]), 9))) <= 253


def _tq(t, store):
    """Per-tensor e4m3 quantise-dequantise with torch's own bfloat16 and float8
    casts: the operand as stored (bf16 or fp32), s = 448/amax and t*s in fp32."""
    x = t.to(torch.bfloat16).float() if store == "bf16" else t.float()
    amax = x.abs().max()
    s = torch.full((), 448.0) / amax if amax > 0 else torch.ones(())   # one rounded fp32 division
    return (x * s).clamp(-448, 448).to(torch.float8_e4m3fn).to(t.dtype) / s.double()


class _F8Linear(torch.autograd.Function):
    """Y = X W^T with the straight-through fp8 rule: the GEMMs the mask selects
    (1 forward, 2 weight gradient, 4 input gradient) see quantised operands."""

    @staticmethod
    def forward(ctx, x, w, mask):
        ctx.save_for_backward(x, w)
        ctx.mask = mask
        on = bool(mask & 1)
        return (_tq(x, "bf16") if on else x) @ (_tq(w, "fp32") if on else w).T

    @staticmethod
    def backward(ctx, gy):
        x, w = ctx.saved_tensors
        g2, x2 = gy.reshape(-1, gy.shape[-1]), x.reshape(-1, x.shape[-1])
        a = lambda t, bit: _tq(t, "bf16") if ctx.mask & bit else t  # noqa: E731
        dw = a(g2, 2).T @ a(x2, 2)
        dx = a(g2, 4) @ (_tq(w, "fp32") if ctx.mask & 4 else w)
        return dx.reshape(x.shape), dw, None


def _torch_fp8_loss(params, tok, tgt, cfg, mask):
    E, U = params[0], params[-1]
    L, H, hd, d = cfg["depth"], cfg["n_head"], cfg["head_dim"], cfg["d_model"]
    B, T = tok.shape
    eps = cfg["norm_eps"]
    lin = lambda x, w: _F8Linear.apply(x, w, mask)  # noqa: E731
    pos = torch.arange(T, dtype=torch.float64)
    inv = cfg["rope_base"] ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = pos[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[None, :, None, :]
    sin = torch.cat([ang.sin(), ang.sin()], -1)[None, :, None, :]

    def rot(x):
        x1, x2 = x[..., : hd // 2], x[..., hd // 2:]
        return x * cos + torch.cat([-x2, x1], -1) * sin

    rms = lambda x: torch.nn.functional.rms_norm(x, (x.shape[-1],), eps=eps)  # noqa: E731
    x = E[torch.from_numpy(tok).long()]
    for l in range(L):
        Wq, Wk, Wv, Wo, W1, W2 = params[1 + 6 * l: 7 + 6 * l]
        qkv = lin(rms(x), torch.cat([Wq, Wk, Wv]))
        q = rms(rot(qkv[..., :d].reshape(B, T, H, hd)))
        k = rms(rot(qkv[..., d:2 * d].reshape(B, T, H, hd)))
        v = qkv[..., 2 * d:].reshape(B, T, H, hd)
        o = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=True)
        x = x + lin(o.transpose(1, 2).reshape(B, T, d), Wo)
        x = x + lin(torch.relu(lin(rms(x), W1)).square(), W2)
    z = lin(rms(x), U)
    return torch.nn.functional.cross_entropy(z.reshape(B * T, -1), torch.from_numpy(tgt).long().reshape(-1))


@pytest.mark.parametrize("mask", [1, 2, 4, 7])
def test_fp8_step_vs_torch_float8_autograd(mask):
    """Each fp8 flag and all three together against torch autograd over torch's
    own bfloat16 and float8 casts."""
    cfg = dict(TINY, precision="fp8", fp8_gemms=mask, batch=2, seq_len=64)
    params = _params(cfg, seed=41, std=0.1)
    tok, tgt = _tokens(cfg, seed=42, dist="zipf")
    loss, grads, _, _ = O.loss_and_grads(params, tok, tgt, cfg)
    tp = [torch.from_numpy(w.copy()).requires_grad_() for w in params]
    tl = _torch_fp8_loss(tp, tok, tgt, cfg, mask)
    tl.backward()
    assert loss == pytest.approx(float(tl.detach()), rel=1e-12)
    for g, t in zip(grads, tp):
        rel = np.linalg.norm(g - t.grad.numpy()) / np.linalg.norm(t.grad.numpy())
        assert rel < 1e-9


def test_fp8_flags_reach_their_gemms():
    base = dict(TINY, batch=2, seq_len=64)
    params = _params(base, seed=43, std=0.1)
    tok, tgt = _tokens(base, seed=44)
    l0, g0, _, _ = O.loss_and_grads(params, tok, tgt, base)
    res = {m: O.loss_and_grads(params, tok, tgt, dict(base, precision="fp8", fp8_gemms=m)) for m in (0, 1, 2, 4)}
    assert res[0][0] == l0 and all(np.array_equal(a, b) for a, b in zip(res[0][1], g0))
    for m in (2, 4):                      # backward-only flags leave the forward exact
        assert res[m][0] == l0
    assert 0 < abs(res[1][0] - l0) / l0 < 1e-2
    for m in (1, 2, 4):
        errs = [np.linalg.norm(a - b) / np.linalg.norm(b) for a, b in zip(res[m][1], g0)]
        assert min(errs[1:-1]) > 1e-3 and max(errs) < 0.3, (m, errs)
    # the input-gradient flag cannot touch the head's weight gradient, the weight-gradient one can
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)  # noqa: E731
    assert rel(res[4][1][-1], g0[-1]) == 0 and rel(res[2][1][-1], g0[-1]) > 1e-3
    # and only the weight-gradient flag leaves the embedding gradient exact
    assert rel(res[2][1][0], g0[0]) == 0 and rel(res[4][1][0], g0[0]) > 1e-3


# ---------------------------------------------------------------------------
# AdamW (E and U)

from oracle import adamw as AW  # noqa: E402


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_adamw_matches_torch_adamw(wd):
    """Four steps against torch.optim.AdamW in fp64 (a library routine), with
    gradients of mixed magnitude, some exactly zero."""
    rng = np.random.default_rng(5)
    w0 = rng.standard_normal((7, 11))
    grads = [rng.standard_normal((7, 11)) * np.exp(rng.uniform(-8, 2, (7, 11))) for _ in range(4)]
    grads[1][2] = 0.0
    hp = dict(lr=3e-3, betas=(0.8, 0.95), eps=1e-10, weight_decay=wd)
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.AdamW([p], **hp, foreach=False)
    w, m, v = w0, np.zeros_like(w0), np.zeros_like(w0)
    for t, g in enumerate(grads, 1):
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        w, m, v = AW.adamw_step(w, g, m, v, t, hp["lr"], *hp["betas"], hp["eps"], wd)
        np.testing.assert_allclose(w, p.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_adamw_closed_forms():
    """From zero moments the first step is w - lr wd w - lr g / (|g| + eps); a zero
    gradient leaves the moments at zero and only decays the weight; the bias
    corrections make a constant gradient give the same step at every t."""
    rng = np.random.default_rng(6)
    w = rng.standard_normal(50)
    g = rng.standard_normal(50)
    lr, b1, b2, eps, wd = 1e-2, 0.9, 0.99, 1e-8, 0.05
    w1, m1, v1 = AW.adamw_step(w, g, 0 * w, 0 * w, 1, lr, b1, b2, eps, wd)
    np.testing.assert_allclose(w1, w - lr * wd * w - lr * g / (np.abs(g) + eps), rtol=1e-14)
    np.testing.assert_allclose(m1, (1 - b1) * g, rtol=1e-15)
    np.testing.assert_allclose(v1, (1 - b2) * g * g, rtol=1e-15)
    w0, m0, v0 = AW.adamw_step(w, 0 * g, 0 * w, 0 * w, 1, lr, b1, b2, eps, wd)
    np.testing.assert_array_equal(m0, 0 * w)
    np.testing.assert_array_equal(v0, 0 * w)
    np.testing.assert_allclose(w0, w * (1 - lr * wd), rtol=1e-15)
    # constant gradient, no decay: m_hat = g and v_hat = g^2 at every t
    wt, m, v = w.copy(), 0 * w, 0 * w
    for t in range(1, 6):
        prev = wt
        wt, m, v = AW.adamw_step(wt, g, m, v, t, lr, b1, b2, eps, 0.0)
        np.testing.assert_allclose(prev - wt, lr * g / (np.abs(g) + eps), rtol=1e-9)
