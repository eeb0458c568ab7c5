"""fp64 CPU oracle of one nanochat-style GPT pretraining step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
run this module; only the tests, the smoke check and the benchmark's CPU
baseline do.  It shares no code with the HIP library.

What it computes (plain definitions, no blocking or fusion):

* Forward of the pre-norm decoder GPT that the nanochat articles describe
  ("nanochat Nasil Calisir? / 1. GPT Modeli" on the dev.to page in Turkish and
  the same section of its Arabic translation): token-embedding lookup with an
  untied LM head, rotary position embeddings and QK normalisation on queries
  and keys, causal multi-head attention, a ReLU^2 MLP, bias-free linears
  (the article's ``Linear`` casts its weight and calls ``F.linear`` with no
  bias, section "3. Hassasiyet Yonetimi"), a final norm, then the mean
  softmax cross-entropy over the vocabulary.
* Its exact gradient, by a hand-written reverse pass.
* The Muon update of every block matrix: heavy-ball momentum, Frobenius
  normalisation, then the Newton-Schulz / Polar Express loop exactly in the
  form the article prints (section "2. Muon Optimize Edici": A = X^T X,
  B = b A + c A^2, X = a X + X B for each (a, b, c) of the table).

Readings where the pages are silent (all parameter-free norms, eps = 1e-6 inside
the square root, RoPE base 10000 with half-split pairs, QK-norm as a per-head
RMSNorm applied after the rotation, MHA with scale 1/sqrt(head_dim), loss =
mean over all B*T positions, heavy-ball momentum, X0 = B/(|B|_F + 1e-7),
W <- W - lr X) are listed with the design notes of this repository.

Parity pins: every function here is pinned by a test under tests/ that does not
re-type its formula (finite differences, closed forms, library routines,
invariants).

fp8 (cfg precision "fp8"): the Linear GEMMs named by the cfg's fp8_gemms mask
(1 forward, 2 weight gradient, 4 input gradient) take per-tensor e4m3
quantised operands (oracle/e4m3.py).  The backward then uses the quantised
operands as if quantisation were the identity (the straight-through rule every
fp8 training recipe uses), so the fp8 gradients are not the derivative of the
fp8 loss.  Q, K and V form one Linear with the concatenated weight [Wq; Wk; Wv],
so they share one weight scale and one gradient scale.  The e4m3 code of each
element is a rounding decision; it is taken on the operand as stored (weights
fp32, activations and output gradients bf16, the scale and the scaled value in
fp32), so that both implementations decide it from the same number.

Extras (cfg "extras", a bitmask; the efficiency tricks printed under "Verimlilik
Puf Noktalari" in "1. GPT Modeli" of the Turkish page and its Arabic
translation).  Their parameters form one more tensor S at the end of the table
(the page's optimizer table puts scalar parameters with AdamW), laid out as in
``extras_layout``:

* 1, per-layer residual scaling: layer i's input is lr[i] x + l0[i] x0, where
  x is the residual stream reaching the layer and x0 the stream entering the
  first layer (after the embedding and the smear).
* 2, smear: after the embedding lookup, x[t] += ls sigmoid(ws . x[t, :24]) x[t-1]
  within each sequence (nothing is added at t = 0): the gate reads the first 24
  channels of the current position, the added term is the previous position's
  embedding before smearing.
* 4, backout: the final norm reads x_L - lb x_mid, x_mid the residual stream
  entering layer L // 2 (before that layer's residual scaling).
* 16, NorMuon: the Muon update of every block matrix goes through normuon()
  (section "2. Muon Optimize Edici"); it adds no model parameters.
* 8, value embeddings (the ResFormer snippet of the same section): every layer i
  has its own table VE_i [V, Hkv hd] and gate weights Wg_i [Hkv, 24]; after the
  QKV projection, v[t, h] += 3 sigmoid(Wg_i[h] . a[t, :24]) VE_i[token t, h], a the
  attention block's normed input.  The tables follow S in the tensor table, then
  one tensor G [L Hkv, 24] of the gate weights.
"""
from __future__ import annotations

import numpy as np

from oracle.e4m3 import quantise

# ---------------------------------------------------------------------------
# configuration / parameter table


EXTRA_RESID, EXTRA_SMEAR, EXTRA_BACKOUT, EXTRA_VALUE_EMB = 1, 2, 4, 8
EXTRA_NORMUON = 16     # an optimizer option (normuon() below): no parameters of its own
MODEL_EXTRAS = 15      # the bits that add the parameter tensor S
SMEAR_CHANNELS = 24  # channels of the current position the smear gate reads
VE_GATE_CHANNELS = 24  # channels of the block's normed input the value-embedding gate reads


def extras_layout(L):
    """Index of each extra parameter inside S (a flat vector of 2L + 2 + 24 values)."""
    return dict(lr=np.arange(0, L), l0=np.arange(L, 2 * L), ls=2 * L, lb=2 * L + 1,
                ws=np.arange(2 * L + 2, 2 * L + 2 + SMEAR_CHANNELS), size=2 * L + 2 + SMEAR_CHANNELS)


def unpack(params, cfg):
    """Split the flat tensor table [E, (Wq,Wk,Wv,Wo,W1,W2)*L, U(, S)(, VE_0..VE_L-1, G)]
    into (E, layers, U, S, VE, G); S (flattened) is None when no extra is switched on,
    VE (a list) and G ([L, Hkv, 24]) are None without value embeddings."""
    L = cfg["depth"]
    ex = cfg.get("extras", 0)
    has_s, has_ve = bool(ex & MODEL_EXTRAS), bool(ex & EXTRA_VALUE_EMB)
    assert len(params) == 2 + 6 * L + has_s + (L + 1) * has_ve
    E = params[0]
    layers = [tuple(params[1 + 6 * l: 7 + 6 * l]) for l in range(L)]
    U = params[1 + 6 * L]
    S = np.asarray(params[2 + 6 * L], dtype=np.float64).reshape(-1) if has_s else None
    VE = G = None
    if has_ve:
        VE = [np.asarray(w, dtype=np.float64) for w in params[3 + 6 * L: 3 + 7 * L]]
        G = np.asarray(params[3 + 7 * L], dtype=np.float64).reshape(L, -1, VE_GATE_CHANNELS)
    return E, layers, U, S, VE, G


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


# ---------------------------------------------------------------------------
# building blocks


def rms_norm(x, eps):
    """Parameter-free RMSNorm over the last axis: y = x / sqrt(mean(x^2) + eps).

    Returns (y, r) with r = 1/sqrt(mean(x^2) + eps) kept for the backward.
    """
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r, r


def rms_norm_bwd(dy, y, r):
    """Gradient of rms_norm: dx = r * (dy - y * mean(dy * y))."""
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rope_angles(T, hd, base):
    """angle[t, i] = t * base^(-2i/hd) for i < hd/2 (positions 0..T-1)."""
    i = np.arange(hd // 2, dtype=np.float64)
    freq = base ** (-2.0 * i / hd)
    t = np.arange(T, dtype=np.float64)
    return t[:, None] * freq[None, :]


def rope(x, ang, inverse=False):
    """Rotate half-split pairs (i, i + hd/2) of x [..., T, H, hd] by angle [T, hd/2].

    forward:  x'_i = x_i cos - x_{i+h} sin ;  x'_{i+h} = x_i sin + x_{i+h} cos.
    inverse=True rotates by -angle (this is also the backward of the rotation).
    """
    h = x.shape[-1] // 2
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    if inverse:
        s = -s
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def causal_attention(q, k, v, window=0):
    """o[b,i,h] = sum_{j<=i} softmax_j(q_i . k_j / sqrt(hd)) v_j ; q,k,v [B,T,H,hd].

    window > 0 restricts query i to the keys i - window < j <= i (sliding-window
    attention: the articles list it among the model's features and pass a
    window_size to the flash-attention call, "5. Flash Dikkat Mekanizmasi
    Birlesimi", without a value; window counts the keys a query sees, itself
    included, i.e. flash-attention's window_size = (window - 1, 0))."""
    B, T, H, hd = q.shape
    qh, kh, vh = (x.transpose(0, 2, 1, 3) for x in (q, k, v))      # [B,H,T,hd]
    S = (qh @ kh.transpose(0, 1, 3, 2)) / np.sqrt(hd)             # [B,H,T,T]
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    if window > 0:
        mask |= np.tril(np.ones((T, T), dtype=bool), -window)
    S = np.where(mask, -np.inf, S)
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=-1, keepdims=True)
    o = (P @ vh).transpose(0, 2, 1, 3)
    return o, P


def causal_attention_bwd(do, q, k, v, o, P=None, window=0):
    """Backward of causal_attention.

    dP = dO v^T ; dS = P * (dP - rowsum(dO * O)) ; dq = dS k / sqrt(hd);
    dk = dS^T q / sqrt(hd) ; dv = P^T dO.
    """
    B, T, H, hd = q.shape
    if P is None:
        _, P = causal_attention(q, k, v, window)
    qh, kh, vh, doh, oh = (x.transpose(0, 2, 1, 3) for x in (q, k, v, do, o))
    dv = P.transpose(0, 1, 3, 2) @ doh
    dP = doh @ vh.transpose(0, 1, 3, 2)
    D = np.sum(doh * oh, axis=-1, keepdims=True)
    dS = P * (dP - D)
    sc = 1.0 / np.sqrt(hd)
    dq = (dS @ kh) * sc
    dk = (dS.transpose(0, 1, 3, 2) @ qh) * sc
    return tuple(x.transpose(0, 2, 1, 3) for x in (dq, dk, dv))


def logsumexp(z):
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


def argmax_lowest(z):
    """Index of the maximum along the last axis, lowest index among exact ties."""
    return np.argmax(z, axis=-1).astype(np.int32)  # numpy returns the first maximum


# ---------------------------------------------------------------------------
# forward / backward


def _fp8_quantisers(cfg):
    """Operand maps (activation or output gradient, weight) of the forward, the
    weight-gradient and the input-gradient GEMMs: per-tensor e4m3
    quantise-dequantise where the fp8 mask selects that GEMM, identity otherwise."""
    ident = lambda t: t  # noqa: E731
    act = lambda t: quantise(t, "bf16")  # noqa: E731
    wgt = lambda t: quantise(t, "fp32")  # noqa: E731
    on = cfg.get("precision") == "fp8"
    mask = cfg.get("fp8_gemms", 7)
    return tuple((act, wgt) if on and mask & bit else (ident, ident) for bit in (1, 2, 4))


def forward(params, tokens, cfg, keep=True):
    """Forward pass.  Returns (logits [B,T,V], cache for backward)."""
    p = [np.asarray(w, dtype=np.float64) for w in params]
    qf, qfw = _fp8_quantisers(cfg)[0]
    E, layers, U, S, VE, G = unpack(p, cfg)
    eps = cfg.get("norm_eps", 1e-6)
    H, hd = cfg["n_head"], cfg["head_dim"]
    Hkv = int(cfg.get("n_kv_head") or H)
    B, T = tokens.shape
    d, dkv = cfg["d_model"], Hkv * hd
    ang = rope_angles(T, hd, cfg.get("rope_base", 10000.0))
    ex = cfg.get("extras", 0)
    X = extras_layout(len(layers))
    Lb = len(layers) // 2                                 # backout: stream entering this layer

    h = E[tokens]                                         # [B,T,d]
    cache = {"tokens": tokens, "ang": ang, "layers": [], "p": p}
    if ex & EXTRA_SMEAR:
        prev = np.zeros_like(h)
        prev[:, 1:] = h[:, :-1]                           # previous position, same sequence
        zs = h[..., :SMEAR_CHANNELS] @ S[X["ws"]]         # [B,T]
        cache.update(emb=h, prev=prev, zs=zs)
        h = h + (S[X["ls"]] * sigmoid(zs))[..., None] * prev
    x0 = h
    cache["x0"] = x0
    for li, (Wq, Wk, Wv, Wo, W1, W2) in enumerate(layers):
        if ex & EXTRA_BACKOUT and li == Lb:
            cache["x_mid"] = h
        x_in = h
        if ex & EXTRA_RESID:
            h = S[X["lr"][li]] * h + S[X["l0"][li]] * x0
        a, ra = rms_norm(h, eps)
        qkv = qf(a) @ qfw(np.concatenate([Wq, Wk, Wv])).T
        q = qkv[..., :d].reshape(B, T, H, hd)
        k = qkv[..., d:d + dkv].reshape(B, T, Hkv, hd)
        v = qkv[..., d + dkv:].reshape(B, T, Hkv, hd)
        if ex & EXTRA_VALUE_EMB:                          # v += 3 sigmoid(gate) * VE[token]
            ve = VE[li][tokens].reshape(B, T, Hkv, hd)
            vg = 3.0 * sigmoid(a[..., :VE_GATE_CHANNELS] @ G[li].T)   # [B,T,Hkv]
            v = v + vg[..., None] * ve
        qn, rq = rms_norm(rope(q, ang), eps)
        kn, rk = rms_norm(rope(k, ang), eps)
        # grouped-query attention: query head h uses key/value head h // (H / Hkv)
        o, _ = causal_attention(qn, np.repeat(kn, H // Hkv, axis=2), np.repeat(v, H // Hkv, axis=2),
                                cfg.get("attn_window", 0))
        o2 = o.reshape(B, T, d)
        h1 = h + qf(o2) @ qfw(Wo).T
        m, rm = rms_norm(h1, eps)
        u = qf(m) @ qfw(W1).T
        g = np.maximum(u, 0.0) ** 2
        h2 = h1 + qf(g) @ qfw(W2).T
        if keep:
            cache["layers"].append(dict(h=h, x_in=x_in, a=a, ra=ra, qn=qn, rq=rq, kn=kn, rk=rk,
                                        v=v, o=o, h1=h1, m=m, rm=rm, u=u, g=g,
                                        ve=ve if ex & EXTRA_VALUE_EMB else None,
                                        vg=vg if ex & EXTRA_VALUE_EMB else None))
        h = h2
    if ex & EXTRA_BACKOUT:
        h = h - S[X["lb"]] * cache["x_mid"]
    r, rf = rms_norm(h, eps)
    z = qf(r) @ qfw(U).T
    cache.update(hL=h, r=r, rf=rf)
    return z, cache


def loss_from_logits(z, targets):
    """Mean over positions of logsumexp(z) - z[target]."""
    lse = logsumexp(z)
    zy = np.take_along_axis(z, targets[..., None].astype(np.int64), axis=-1)[..., 0]
    return float(np.mean(lse - zy)), lse - zy


def cross_entropy_grad(z, targets):
    """d(mean cross-entropy)/dz = (softmax(z) - onehot(y)) / (number of positions)."""
    n = targets.size
    P = np.exp(z - z.max(axis=-1, keepdims=True))
    P /= P.sum(axis=-1, keepdims=True)
    idx = targets[..., None].astype(np.int64)
    np.put_along_axis(P, idx, np.take_along_axis(P, idx, -1) - 1.0, -1)
    return P / n


def backward(z, targets, cache, cfg):
    """Exact gradient of the mean cross-entropy w.r.t. every tensor of the table."""
    p = cache["p"]
    E, layers, U, S, VE, Gv = unpack(p, cfg)                # Gv: value-embedding gate weights
    ex = cfg.get("extras", 0)
    X = extras_layout(len(layers))
    Lb = len(layers) // 2
    dS = np.zeros(X["size"]) if S is not None else None
    H, hd = cfg["n_head"], cfg["head_dim"]
    B, T, V = z.shape
    d = cfg["d_model"]
    Hkv = int(cfg.get("n_kv_head") or H)
    G, dkv = H // Hkv, Hkv * hd
    N = B * T
    ang = cache["ang"]
    tokens = cache["tokens"]

    dz = cross_entropy_grad(z, targets)
    _, (qw, _), (qd, qdw) = _fp8_quantisers(cfg)

    def lin_bwd(dy, x, W):
        """Y = X W^T: (dW = dY^T X, dX = dY W) on the flattened token axis."""
        dy2 = dy.reshape(N, -1)
        return qw(dy2).T @ qw(x.reshape(N, -1)), qd(dy2) @ qdw(W)

    r = cache["r"]
    dU, dr = lin_bwd(dz, r, U)
    dh = rms_norm_bwd(dr.reshape(B, T, d), r, cache["rf"])
    if ex & EXTRA_BACKOUT:                                # final input x_L - lb x_mid
        d_mid = -S[X["lb"]] * dh
        dS[X["lb"]] = -np.sum(dh * cache["x_mid"])
    dx0 = np.zeros_like(dh)                               # through the l0 terms
    dVE = [np.zeros_like(t) for t in VE] if VE is not None else None
    dG = np.zeros_like(Gv) if Gv is not None else None

    grads_layers = []
    for li, (Wq, Wk, Wv, Wo, W1, W2), c in zip(reversed(range(len(layers))), reversed(layers),
                                                reversed(cache["layers"])):
        # MLP block: h2 = h1 + g W2^T, g = relu(u)^2, u = m W1^T, m = rms(h1)
        dW2, dg = lin_bwd(dh, c["g"], W2)
        du = dg.reshape(c["u"].shape) * 2.0 * np.maximum(c["u"], 0.0)
        dW1, dm = lin_bwd(du, c["m"], W1)
        dh1 = dh + rms_norm_bwd(dm.reshape(B, T, d), c["m"], c["rm"])
        # attention block: h1 = h + o Wo^T
        dWo, do = lin_bwd(dh1, c["o"], Wo)
        do = do.reshape(B, T, H, hd)
        dqn, dkn, dv = causal_attention_bwd(do, c["qn"], np.repeat(c["kn"], G, axis=2), np.repeat(c["v"], G, axis=2),
                                            c["o"], window=cfg.get("attn_window", 0))
        # a key/value head's gradient is the sum over the G query heads sharing it
        dkn = dkn.reshape(B, T, Hkv, G, hd).sum(axis=3)
        dv = dv.reshape(B, T, Hkv, G, hd).sum(axis=3)
        da_ve = 0.0
        if ex & EXTRA_VALUE_EMB:                          # v' = v + vg ve, vg = 3 sigmoid(z)
            np.add.at(dVE[li], tokens.reshape(-1), (c["vg"][..., None] * dv).reshape(N, dkv))
            dz = np.sum(dv * c["ve"], axis=-1) * c["vg"] * (1.0 - c["vg"] / 3.0)   # [B,T,Hkv]
            dG[li] = np.einsum("bth,btc->hc", dz, c["a"][..., :VE_GATE_CHANNELS])
            da_ve = np.zeros((B, T, d))
            da_ve[..., :VE_GATE_CHANNELS] = dz @ Gv[li]
        dq = rope(rms_norm_bwd(dqn, c["qn"], c["rq"]), ang, inverse=True).reshape(B, T, d)
        dk = rope(rms_norm_bwd(dkn, c["kn"], c["rk"]), ang, inverse=True).reshape(B, T, dkv)
        dv = dv.reshape(B, T, dkv)
        # one Linear with weight [Wq; Wk; Wv]: dY = [dq | dk | dv]
        dWqkv, da = lin_bwd(np.concatenate([dq, dk, dv], axis=-1), c["a"], np.concatenate([Wq, Wk, Wv]))
        dWq, dWk, dWv = dWqkv[:d], dWqkv[d:d + dkv], dWqkv[d + dkv:]
        dh = dh1 + rms_norm_bwd(da.reshape(B, T, d) + da_ve, c["a"], c["ra"])
        if ex & EXTRA_RESID:                              # layer input lr x_in + l0 x0
            dS[X["lr"][li]] = np.sum(dh * c["x_in"])
            dS[X["l0"][li]] = np.sum(dh * cache["x0"])
            dx0 += S[X["l0"][li]] * dh
            dh = S[X["lr"][li]] * dh
        if ex & EXTRA_BACKOUT and li == Lb:
            dh = dh + d_mid
        grads_layers.append((dWq, dWk, dWv, dWo, dW1, dW2))
    grads_layers.reverse()
    dh = dh + dx0                                         # x0 is also the first layer's input
    if ex & EXTRA_SMEAR:                                  # x = e + ls sigmoid(zs) prev(e)
        sg = sigmoid(cache["zs"])
        demb = dh.copy()
        demb[:, :-1] += (S[X["ls"]] * sg)[:, 1:, None] * dh[:, 1:]
        dgate = np.sum(dh * cache["prev"], axis=-1)       # d loss / d (ls sigmoid(zs))
        dS[X["ls"]] = np.sum(dgate * sg)
        dzs = dgate * S[X["ls"]] * sg * (1.0 - sg)
        dS[X["ws"]] = np.einsum("bt,btc->c", dzs, cache["emb"][..., :SMEAR_CHANNELS])
        demb[..., :SMEAR_CHANNELS] += dzs[..., None] * S[X["ws"]]
        dh = demb

    dE = np.zeros_like(E)
    np.add.at(dE, tokens.reshape(-1), dh.reshape(N, d))
    grads = [dE]
    for gl in grads_layers:
        grads.extend(gl)
    grads.append(dU)
    if dS is not None:
        grads.append(dS.reshape(np.shape(p[2 + 6 * len(layers)])))
    if dVE is not None:
        grads.extend(dVE)
        grads.append(dG.reshape(np.shape(p[3 + 7 * len(layers)])))
    return grads


def loss_and_grads(params, tokens, targets, cfg):
    """(loss, grads in tensor-table order, argmax [B,T], per-position loss [B,T])."""
    z, cache = forward(params, tokens, cfg)
    loss, per_pos = loss_from_logits(z, targets)
    grads = backward(z, targets, cache, cfg)
    return loss, grads, argmax_lowest(z), per_pos


def loss_only(params, tokens, targets, cfg):
    z, _ = forward(params, tokens, cfg, keep=False)
    return loss_from_logits(z, targets)[0]


# ---------------------------------------------------------------------------
# Muon


def newton_schulz(X, coeffs):
    """The article's orthogonalisation loop, verbatim in form:

    for (a, b, c): A = X^T X ; B = b A + c A A ; X = a X + X B.
    """
    X = np.asarray(X, dtype=np.float64)
    for (a, b, c) in coeffs:
        A = X.T @ X
        Bm = b * A + c * (A @ A)
        X = a * X + X @ Bm
    return X


def muon_matrix(G, Bm, coeffs, mu=0.95, eps=1e-7):
    """One Muon direction for one matrix.

    Bm <- mu Bm + G (heavy ball, starts at zero); X0 = Bm / (|Bm|_F + eps);
    returns (X_ns, Bm_new).
    """
    Bm = mu * np.asarray(Bm, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    X0 = Bm / (np.linalg.norm(Bm) + eps)
    return newton_schulz(X0, coeffs), Bm


def normuon(X, V, beta2, eps=1e-10):
    """NorMuon's per-neuron normalisation of one matrix's orthogonalised update X
    [out, in] (the nanochat articles print its last four lines under "NorMuon Varyans
    Azaltma" in "2. Muon Optimize Edici"; the rest follows the published method, Li et
    al. 2025, "NorMuon: Making Muon more efficient and scalable"):

        v_mean[i] = mean_j X[i, j]^2              one statistic per output neuron
        V <- beta2 V + (1 - beta2) v_mean          running second moment (starts at 0)
        step[i] = 1 / sqrt(max(V[i], eps))
        v_norm = sqrt(sum_i v_mean[i]),  v_norm_new = sqrt(sum_i v_mean[i] step[i]^2)
        X'[i, :] = X[i, :] step[i] v_norm / max(v_norm_new, eps)

    so rows are rescaled by the inverse root of their running second moment while the
    Frobenius norm of X is kept.  Returns (X', V')."""
    X = np.asarray(X, dtype=np.float64)
    v_mean = np.mean(X * X, axis=1)
    V = beta2 * np.asarray(V, dtype=np.float64) + (1.0 - beta2) * v_mean
    step = 1.0 / np.sqrt(np.maximum(V, eps))
    v_norm = np.sqrt(np.sum(v_mean))
    v_norm_new = np.sqrt(np.sum(v_mean * step * step))
    return X * (step * v_norm / max(v_norm_new, eps))[:, None], V


def muon_update(params, grads, moms, cfg, lr, coeffs):
    """Muon step on every block matrix (Wq, Wk, Wv, Wo, W1, W2 of each layer,
    each separately).  E and U are left untouched (their AdamW group is not part
    of this step).  Returns (new_params, new_moms, directions) as lists in
    tensor-table order (None for E and U)."""
    L = cfg["depth"]
    mu = cfg.get("muon_momentum", 0.95)
    newp = [np.asarray(w, dtype=np.float64).copy() for w in params]
    newm = [None] * len(params)
    dirs = [None] * len(params)
    for i in range(1, 1 + 6 * L):
        X, Bm = muon_matrix(grads[i], moms[i], coeffs, mu)
        newp[i] = newp[i] - lr * X
        newm[i] = Bm
        dirs[i] = X
    return newp, newm, dirs
