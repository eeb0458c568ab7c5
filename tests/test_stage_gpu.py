"""Stage-isolated parity of every Linear product inside gpt_step.

gpt_capture copies what one layer's GEMMs received and produced during a real step
(the QKV, output, fc and proj projections of a block, or the LM head), so each
product is checked on exactly its own operands, with nothing upstream able to move
them.  For a Linear Y = X W^T the oracle computes

    forward            Y  = q(X) q(W)^T
    weight gradient    dW = q(dY)^T q(X)
    input gradient     dX = q(dY) q(W)

with q the oracle's per-tensor e4m3 quantise-dequantise (fp8 steps: activations and
output gradients as stored in bf16, weights from the fp32 masters) or, for bf16
steps, the identity with W rounded to bf16 as the kernels read it.  The fused
epilogues are part of the products: the residual adds (Y = h1 - x, h2 - h1), ReLU^2
(g = relu(u)^2), dReLU^2 (du = (dY W2) 2 relu(u), with relu(u) read back as sqrt(g):
the step keeps g, not u) and the cross-entropy
gradient of the head (dlogits from the captured logits).  Each product is held to
the step's per-tensor bar (2e-2 bf16, 6e-2 fp8); the errors printed are what is left
after the operands are pinned: accumulation order and the outputs' own rounding.
"""
import numpy as np
import pytest
import torch

from gpt_pretraining_step_train_amd import binding, configs, inputs
from oracle import gpt_oracle as O
from oracle.e4m3 import quantise, to_bf16
from tests.gpu_util import rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    torch.cuda.set_device(0)


def _quantisers(cfg):
    if cfg["precision"] == "fp8":
        return (lambda t: quantise(t, "bf16")), (lambda w: quantise(w, "fp32"))
    return (lambda t: t), (lambda w: to_bf16(w))


def _check(name, got, ref, bar, worst):
    e = rel_l2(got, ref)
    say(f"    {name:<28s} rel L2 {e:.2e}")
    assert e <= bar, (name, e)
    worst[0] = max(worst[0], e)


def _check_block(cap, W, grads, cfg, bar, worst):
    """W, grads: dict of fp64 matrices by name (qkv stacked, o, 1, 2)."""
    qa, qw = _quantisers(cfg)
    relu = lambda t: np.maximum(t, 0.0)  # noqa: E731
    # forward
    _check("qkv = a Wqkv^T", cap["qkv"], qa(cap["a"]) @ qw(W["qkv"]).T, bar, worst)
    _check("h1 - x = o Wo^T", cap["h1"] - cap["x"], qa(cap["o"]) @ qw(W["o"]).T, bar, worst)
    _check("g = relu(m W1^T)^2", cap["g"], relu(qa(cap["m"]) @ qw(W["1"]).T) ** 2, bar, worst)
    _check("h2 - h1 = g W2^T", cap["h2"] - cap["h1"], qa(cap["g"]) @ qw(W["2"]).T, bar, worst)
    # backward, last product first
    _check("dW2 = dh^T g", grads["2"], qa(cap["dh"]).T @ qa(cap["g"]), bar, worst)
    _check("du = (dh W2) 2 relu(u)", cap["du"], (qa(cap["dh"]) @ qw(W["2"])) * 2.0 * np.sqrt(cap["g"]), bar, worst)
    _check("dW1 = du^T m", grads["1"], qa(cap["du"]).T @ qa(cap["m"]), bar, worst)
    _check("dm = du W1", cap["dm"], qa(cap["du"]) @ qw(W["1"]), bar, worst)
    _check("dWo = dh1^T o", grads["o"], qa(cap["dh1"]).T @ qa(cap["o"]), bar, worst)
    _check("do = dh1 Wo", cap["do"], qa(cap["dh1"]) @ qw(W["o"]), bar, worst)
    _check("dWqkv = dqkv^T a", grads["qkv"], qa(cap["dqkv"]).T @ qa(cap["a"]), bar, worst)
    _check("da = dqkv Wqkv", cap["da"], qa(cap["dqkv"]) @ qw(W["qkv"]), bar, worst)


def _check_head(cap, U, dU, tgt, cfg, bar, worst):
    qa, qw = _quantisers(cfg)
    _check("logits = r U^T", cap["logits"], qa(cap["r"]) @ qw(U).T, bar, worst)
    dz = O.cross_entropy_grad(cap["logits"], tgt.reshape(-1))
    _check("dlogits = (softmax - 1_y)/N", cap["dlogits"], dz, bar, worst)
    _check("dU = dlogits^T r", dU, qa(cap["dlogits"]).T @ qa(cap["r"]), bar, worst)
    _check("dr = dlogits U", cap["dr"], qa(cap["dlogits"]) @ qw(U), bar, worst)


# (config, overrides, layers to capture; "head" = the LM head)
STAGE_CASES = [
    ("laptop", {"precision": "fp8"}, [0, 2, "head"]),
    ("d26", {"batch": 1, "depth": 2}, [0, 1, "head"]),
    ("d26", {"batch": 1}, [0, 13, 25, "head"]),
    ("d24", {"batch": 1}, [0, 23, "head"]),
    ("d24", {"batch": 1, "precision": "fp8"}, [0, 23, "head"]),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,over,layers", STAGE_CASES,
                         ids=[f"{c[0]}_{c[1].get('precision', configs.get(c[0])['precision'])}"
                              f"_L{c[1].get('depth', configs.get(c[0])['depth'])}" for c in STAGE_CASES])
def test_linear_products_on_captured_operands(name, over, layers):
    cfg = configs.get(name, **over)
    say("stage-isolated Linear products", name, over)
    model = binding.Model(cfg, seed=0)
    params = inputs.init_weights(cfg, 0)
    model.set_all_params(params)
    tok, tgt = inputs.token_batch(cfg["batch"], cfg["seq_len"], cfg["vocab"], dist=cfg["tokens"], seed=0)
    dtok, dtgt = torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()
    bar = 6e-2 if cfg["precision"] == "fp8" else 2e-2
    L = cfg["depth"]
    worst = [0.0]
    for layer in layers:
        li = L if layer == "head" else layer
        loss, cap = model.capture_step(li, dtok, dtgt)
        say(f"  layer {layer} (loss {loss:.5f})")
        if layer == "head":
            _check_head(cap, params[1 + 6 * L].astype(np.float64), model.grads(1 + 6 * L).astype(np.float64), tgt,
                        cfg, bar, worst)
            continue
        ids = [1 + 6 * li + j for j in range(6)]
        p = [params[i].astype(np.float64) for i in ids]
        g = [model.grads(i).astype(np.float64) for i in ids]
        W = {"qkv": np.concatenate(p[:3]), "o": p[3], "1": p[4], "2": p[5]}
        G = {"qkv": np.concatenate(g[:3]), "o": g[3], "1": g[4], "2": g[5]}
        _check_block(cap, W, G, cfg, bar, worst)
    say(f"  worst product rel L2 {worst[0]:.2e} (bar {bar:g})")
