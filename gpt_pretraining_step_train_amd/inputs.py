"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds no arithmetic of the training step itself: it only draws
token ids and initial weights.  Both sides receive the same arrays.

* Token ids: i.i.d. uniform over the vocabulary, or Zipf(s) with
  P(id = k) proportional to (k+1)^-s for k in [0, V) (id 0 most frequent,
  no permutation), drawn by inverse-CDF lookup of seeded uniforms.  Each row
  draws T+1 ids; tokens are the first T, targets the last T ("targets are
  tokens shifted by one").  These stand in for the tokenised web text the
  nanochat articles train on, which is not available here.
* Weights: every matrix ~ N(0, init_std^2) in float32, with the two output
  projections (attention W_o and MLP W_2) scaled by 1/sqrt(2*depth).

Tensor table order (the C ABI's tensor ids): 0 = E [V,d]; for layer l the
ids 1+6l .. 1+6l+5 are Wq [d,d], Wk [dkv,d], Wv [dkv,d], Wo [d,d], W1 [F,d],
W2 [d,F]; id 1+6L is the LM head U [V,d].  When the cfg switches on any of the
extras, id 2+6L is S [1, 2L+26]: L per-layer residual scales, L per-layer x0
scales, the smear scale, the backout scale and the 24 smear-gate weights.  S
starts as the identity (residual scales 1, everything else 0), where the
extras leave the model unchanged.  With value embeddings (extras bit 8) the
ids 3+6L .. 2+7L are the per-layer tables VE_l [V, dkv] and id 3+7L is G
[L*Hkv, 24], the gate weights (layer-major); both start at 0.
"""
from __future__ import annotations

import numpy as np


def tensor_shapes(cfg: dict) -> list[tuple[str, tuple[int, int]]]:
    d, F, V, L = cfg["d_model"], cfg["d_ff"], cfg["vocab"], cfg["depth"]
    dkv = int(cfg.get("n_kv_head") or cfg["n_head"]) * cfg["head_dim"]  # key/value rows
    out = [("E", (V, d))]
    for l in range(L):
        out += [(f"l{l}.Wq", (d, d)), (f"l{l}.Wk", (dkv, d)), (f"l{l}.Wv", (dkv, d)),
                (f"l{l}.Wo", (d, d)), (f"l{l}.W1", (F, d)), (f"l{l}.W2", (d, F))]
    out.append(("U", (V, d)))
    if cfg.get("extras", 0) & 15:  # bit 16 (NorMuon) is an optimizer option without parameters
        out.append(("S", (1, 2 * L + 26)))
    if cfg.get("extras", 0) & 8:
        out += [(f"l{l}.VE", (V, dkv)) for l in range(L)]
        out.append(("G", (L * int(cfg.get("n_kv_head") or cfg["n_head"]), 24)))
    return out


def init_weights(cfg: dict, seed: int = 0) -> list[np.ndarray]:
    """float32 weights in tensor-table order, N(0, std^2), output projections scaled."""
    rng = np.random.Generator(np.random.PCG64(seed))
    std = float(cfg.get("init_std", 0.02))
    out_scale = 1.0 / np.sqrt(2.0 * cfg["depth"])
    ws = []
    for name, shape in tensor_shapes(cfg):
        if name == "S":
            w = np.zeros(shape, dtype=np.float32)
            w[0, :cfg["depth"]] = 1.0
            ws.append(w)
            continue
        if name == "G" or name.endswith(".VE"):
            ws.append(np.zeros(shape, dtype=np.float32))
            continue
        s = std * (out_scale if name.endswith(".Wo") or name.endswith(".W2") else 1.0)
        w = rng.standard_normal(shape, dtype=np.float32)
        w *= np.float32(s)
        ws.append(w)
    return ws


def zipf_cdf(vocab: int, s: float) -> np.ndarray:
    p = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def token_batch(batch: int, seq_len: int, vocab: int, dist: str = "zipf",
                s: float = 1.1, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """(tokens, targets), both int32 [batch, seq_len]; targets = tokens shifted by one."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if dist == "uniform":
        ids = rng.integers(0, vocab, size=(batch, seq_len + 1), dtype=np.int64)
    elif dist == "zipf":
        u = rng.random((batch, seq_len + 1))
        ids = np.searchsorted(zipf_cdf(vocab, s), u, side="right")
        ids = np.minimum(ids, vocab - 1)
    else:
        raise ValueError(f"unknown token distribution {dist!r}")
    ids = ids.astype(np.int32)
    return np.ascontiguousarray(ids[:, :-1]), np.ascontiguousarray(ids[:, 1:])


def gaussian(shape, seed: int, scale: float = 1.0, dtype=np.float32) -> np.ndarray:
    """Plain seeded N(0, scale^2) array, used for stage-isolated kernel inputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(shape) * scale).astype(dtype)
