"""The five named model/step configurations (shapes only).

depth sets the rest on the nanochat pages ("one dial"); the shapes here are
the tiny, laptop-scale, d12, d24 and d26 GPTs with vocab 2^15 = 32768 for the
depth-dialled ones and 4096 for the two small ones, sequence length 2048 and
device batch 16 for the depth-dialled ones.
"""
from __future__ import annotations

PRECISION = {"fp32": 0, "bf16": 1, "fp8": 2}

CONFIGS = {
    "tiny": dict(depth=2, d_model=128, n_head=4, head_dim=32, d_ff=512, vocab=4096,
                 seq_len=128, batch=4, precision="fp32", tokens="uniform"),
    "laptop": dict(depth=3, d_model=192, n_head=3, head_dim=64, d_ff=768, vocab=4096,
                   seq_len=256, batch=32, precision="bf16", tokens="zipf"),
    "d12": dict(depth=12, d_model=768, n_head=6, head_dim=128, d_ff=3072, vocab=32768,
                seq_len=2048, batch=16, precision="bf16", tokens="zipf"),
    "d24": dict(depth=24, d_model=1536, n_head=12, head_dim=128, d_ff=6144, vocab=32768,
                seq_len=2048, batch=16, precision="bf16", tokens="zipf"),
    "d26": dict(depth=26, d_model=1664, n_head=13, head_dim=128, d_ff=6656, vocab=32768,
                seq_len=2048, batch=16, precision="fp8", tokens="zipf"),
}

DEFAULTS = dict(init_std=0.02, rope_base=10000.0, norm_eps=1e-6, muon_momentum=0.95,
                ns_steps=5, fp8_gemms=7,   # fp8: forward, weight- and input-gradient GEMMs
                attn_window=0,             # sliding-window attention off (every earlier key)
                n_kv_head=0,               # key/value heads; 0 = n_head (multi-head attention)
                extras=0,                  # mask: 1 residual scaling, 2 smear, 4 backout, 8 value embeddings,
                                           # 16 NorMuon
                normuon_beta2=0.95)        # NorMuon's second-moment decay


def kv_heads(cfg: dict) -> int:
    """Key/value heads: n_kv_head, or n_head when it is 0 / absent (grouped-query
    attention shares each key/value head among n_head / n_kv_head query heads)."""
    return int(cfg.get("n_kv_head") or cfg["n_head"])


def get(name: str, **over) -> dict:
    c = dict(DEFAULTS)
    c.update(CONFIGS[name])
    c.update(over)
    c["name"] = name
    return c


def n_params(cfg: dict) -> int:
    d, F, V, L = cfg["d_model"], cfg["d_ff"], cfg["vocab"], cfg["depth"]
    dkv = kv_heads(cfg) * cfg["head_dim"] if cfg.get("n_kv_head") else d  # Wk, Wv rows
    n_s = 2 * L + 26 if cfg.get("extras", 0) & 15 else 0  # the extras' scalars
    if cfg.get("extras", 0) & 8:  # value-embedding tables and gate weights
        n_s += L * V * kv_heads(cfg) * cfg["head_dim"] + L * kv_heads(cfg) * 24
    return 2 * V * d + L * (2 * d * d + 2 * dkv * d + 2 * F * d) + n_s


def step_flops(cfg: dict) -> dict:
    """Algorithmic FLOPs of one step: dense GEMMs, exact causal attention, Newton-Schulz.

    fwd+bwd = 6 N (12 L d^2 + d V) when F = 4d (generally 6 N (4 L d^2 + 2 L d F + d V);
    with grouped-query attention Wk, Wv are dkv x d, dkv = n_kv_head * head_dim), plus
    causal attention 12 L B d S, S = the (query, key) pairs of one sequence: T (T+1) / 2
    for full causal attention (fwd 4 d S per sequence and layer, bwd 2x); a sliding
    window W < T leaves W (W+1) / 2 + (T - W) W of them.
    Muon = ns_steps * sum over block matrices of (4 s^2 l + 2 s^3), s = min dim, l = max dim.
    """
    d, F, V, L = cfg["d_model"], cfg["d_ff"], cfg["vocab"], cfg["depth"]
    dkv = kv_heads(cfg) * cfg["head_dim"]
    B, T = cfg["batch"], cfg["seq_len"]
    N = B * T
    linear = 6 * N * (2 * L * d * d + 2 * L * dkv * d + 2 * L * d * F)
    head = 6 * N * d * V
    W = cfg.get("attn_window", 0)
    pairs = T * (T + 1) // 2 if not W or W >= T else W * (W + 1) // 2 + (T - W) * W
    attn = 12 * L * B * d * pairs
    k = cfg.get("ns_steps", 5)
    mats = [(d, d), (dkv, d), (dkv, d), (d, d), (F, d), (d, F)]
    muon = 0
    for (r, c) in mats:
        s, l = min(r, c), max(r, c)
        muon += k * (4 * s * s * l + 2 * s ** 3)
    muon *= L
    return dict(linear=linear, head=head, attn=attn, muon=muon,
                total=linear + head + attn + muon)
