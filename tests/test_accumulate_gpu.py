"""Gradient accumulation over micro-batches (gpt_step_accumulate) through the C ABI.

* grad_scale is exact: a power-of-two scale commutes with every rounding of the
  backward (bf16 and fp32 stores, and the per-tensor e4m3 scales, which move by
  the same power of two), so 0.5 gives exactly half of every gradient.
* n micro-batches accumulated with grad_scale 1/n give the gradient of the mean
  loss over their concatenation.  For bf16 and fp32 the oracle computes that
  gradient directly on the concatenated batch, with the step's own bars
  (gradients 2e-2, fp32 1e-4).  Under fp8 each micro-batch has its own e4m3 scales,
  so the oracle's per-micro-batch fp8 gradients are averaged instead (bar 6e-2).
"""
import numpy as np
import pytest
import torch

from gpt_pretraining_step_train_amd import binding, configs, inputs
from oracle import gpt_oracle as O
from tests.gpu_util import random_extras, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    torch.cuda.set_device(0)


def _model(name, **over):
    cfg = configs.get(name, **over)
    model = binding.Model(cfg, seed=0)
    params = random_extras(inputs.init_weights(cfg, 0), cfg, 0)
    model.set_all_params(params)
    return cfg, model, params


def _batch(cfg, seed):
    tok, tgt = inputs.token_batch(cfg["batch"], cfg["seq_len"], cfg["vocab"], dist=cfg["tokens"], seed=seed)
    return tok, tgt, torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()


@pytest.mark.parametrize("name,over", [("tiny", {}), ("laptop", {"batch": 8}),
                                       ("laptop", {"batch": 8, "precision": "fp8"}),
                                       ("laptop", {"batch": 8, "extras": 15})], ids=["fp32", "bf16", "fp8", "extras"])
def test_grad_scale_is_exact(name, over):
    cfg, model, params = _model(name, **over)
    _, _, dt, dg = _batch(cfg, 3)
    l1 = model.step(dt, dg)
    g1 = [model.grads(i) for i in range(len(params))]
    l2 = model.step(dt, dg, grad_scale=0.5)
    torch.cuda.synchronize()
    assert l1 == l2
    for i, g in enumerate(g1):
        np.testing.assert_array_equal(model.grads(i), 0.5 * g, err_msg=f"tensor {i}")


@pytest.mark.parametrize("name,over", [("tiny", {}), ("laptop", {"batch": 8}),
                                       ("laptop", {"batch": 8, "precision": "fp8"}),
                                       ("laptop", {"batch": 8, "extras": 15})], ids=["fp32", "bf16", "fp8", "extras"])
def test_accumulated_gradient_is_the_total_batch_gradient(name, over):
    cfg, model, params = _model(name, **over)
    n = 3
    parts = [_batch(cfg, 10 + k) for k in range(n)]
    losses = [model.step(dt, dg, accumulate=k > 0, grad_scale=1.0 / n) for k, (_, _, dt, dg) in enumerate(parts)]
    torch.cuda.synchronize()
    fp32, fp8 = cfg["precision"] == "fp32", cfg["precision"] == "fp8"
    if fp8:
        refs = [O.loss_and_grads(params, tok, tgt, cfg) for tok, tgt, _, _ in parts]
        ref_grads = [sum(r[1][i] for r in refs) / n for i in range(len(params))]
        ref_losses = [r[0] for r in refs]
    else:
        tok = np.concatenate([p[0] for p in parts])
        tgt = np.concatenate([p[1] for p in parts])
        ref_loss, ref_grads, _, _ = O.loss_and_grads(params, tok, tgt, dict(cfg, batch=n * cfg["batch"]))
        ref_losses = [O.loss_only(params, p[0], p[1], cfg) for p in parts]
        assert abs(np.mean(losses) - ref_loss) / ref_loss <= (1e-5 if fp32 else 1e-3)
    for l, r in zip(losses, ref_losses):
        assert abs(l - r) / r <= (1e-5 if fp32 else 1e-2 if fp8 else 1e-3)
    worst = 0.0
    for i, ref in enumerate(ref_grads):
        e = rel_l2(model.grads(i), ref)
        worst = max(worst, e)
        assert e <= (1e-4 if fp32 else 6e-2 if fp8 else 2e-2), (i, e)
    say(f"  {name} {over}: {n} micro-batches, worst grad rel L2 {worst:.2e}")
