"""AdamW on E and U through the C ABI (adamw_update) against the fp64 oracle.

Bars: the updates are fp32 elementwise arithmetic, so the weights after three
steps must agree with the oracle to four fp32 ulps of the weight (each step rounds
w once) plus 1e-6 of the step: |w_gpu - w_ref| <= max(3e-8, 4 ulp(|w|)) +
1e-6 |w_ref - w0| (3e-8 is 4 ulps at |w| = 0.1, the largest E and U entries; the
extras' scales sit near 1).
The next gpt_step must see the new U through its bf16 (and e4m3) copies: its
loss is held to the step's own bar against the oracle on the updated weights.
"""
import numpy as np
import pytest
import torch

from gpt_pretraining_step_train_amd import binding, configs, inputs
from oracle import adamw as AW
from oracle import gpt_oracle as O
from tests.gpu_util import random_extras, rel_l2, say

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.8, beta2=0.95, eps=1e-8, weight_decay=0.1)


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


def _adamw_chain(w0, grads, hp):
    w, m, v = np.asarray(w0, dtype=np.float64), 0.0, 0.0
    for t, g in enumerate(grads, 1):
        w, m, v = AW.adamw_step(w, g, m, v, t, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    return w


@pytest.mark.parametrize("name,over", [("tiny", {}), ("laptop", {}), ("laptop", {"extras": 15})],
                         ids=["tiny", "laptop", "laptop_extras"])
def test_adamw_matches_oracle(name, over):
    cfg, model, params = _model(name, **over)
    say("adamw parity", name, over)
    L = cfg["depth"]
    ids = [0, 1 + 6 * L]  # E, U, and the extras' S, a value-embedding table and the gate weights
    if cfg.get("extras"):
        ids += [2 + 6 * L, 3 + 6 * L, 3 + 7 * L]
    rng = np.random.default_rng(7)
    grads = {i: [] for i in ids}
    for step in range(3):
        for i in ids:
            g = (rng.standard_normal(params[i].shape) * np.exp(rng.uniform(-6, 1, params[i].shape))).astype(np.float32)
            g[rng.random(g.shape[0]) < 0.3] = 0.0  # rows no token touched
            grads[i].append(g)
            model.set_grads(i, g)
        model.adamw_update(**HP)
    torch.cuda.synchronize()
    for i in ids:
        ref = _adamw_chain(params[i], grads[i], HP)
        got = model.get_params(i).astype(np.float64)
        err = np.abs(got - ref)
        mag = np.maximum(np.abs(ref), np.abs(params[i])).astype(np.float32)
        bound = np.maximum(3e-8, 4 * np.spacing(mag).astype(np.float64)) + 1e-6 * np.abs(ref - params[i])
        say(f"  tensor {i} {params[i].shape}: max err {err.max():.2e}, update rel L2 "
            f"{rel_l2(got - params[i], ref - params[i]):.2e}")
        assert np.all(err <= bound)
    np.testing.assert_array_equal(model.get_params(1), params[1])  # Muon's tensors untouched


@pytest.mark.parametrize("name,over", [("laptop", {}), ("laptop", {"precision": "fp8"})], ids=["bf16", "fp8"])
def test_next_step_sees_the_new_head(name, over):
    """After AdamW, the next gpt_step multiplies by the new U (bf16 copy, and the e4m3
    copy under fp8): its loss matches the oracle on the updated weights, five times
    closer than the loss on the old weights is."""
    cfg, model, params = _model(name, **over)
    tok, tgt = inputs.token_batch(cfg["batch"], cfg["seq_len"], cfg["vocab"], dist=cfg["tokens"], seed=1)
    dt, dg = torch.from_numpy(tok).cuda(), torch.from_numpy(tgt).cuda()
    model.step(dt, dg)
    model.adamw_update(lr=1e-2, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.0)
    loss = model.step(dt, dg)
    torch.cuda.synchronize()
    new = [params[i] if 0 < i < len(params) - 1 else model.get_params(i) for i in range(len(params))]
    ref = O.loss_only(new, tok, tgt, cfg)
    old = O.loss_only(params, tok, tgt, cfg)
    bar = 1e-2 if cfg["precision"] == "fp8" else 1e-3
    say(f"  {over or 'bf16'}: loss {loss:.6f} oracle(new) {ref:.6f} oracle(old) {old:.6f}")
    assert abs(loss - ref) / ref <= bar
    assert abs(loss - ref) < 0.2 * abs(old - ref)


def test_adamw_rejects_bad_arguments_without_counting_them():
    cfg, model, params = _model("tiny")
    U = len(params) - 1
    g = np.random.default_rng(8).standard_normal(params[U].shape).astype(np.float32)
    model.set_grads(U, g)
    for bad in (dict(HP, beta1=1.0), dict(HP, beta2=-0.1), dict(HP, eps=-1e-8), dict(HP, lr=float("nan")),
                dict(HP, weight_decay=float("inf"))):
        with pytest.raises(binding.GptError, match="argument"):
            model.adamw_update(**bad)
    model.adamw_update(**HP)  # the first valid call is step t = 1
    torch.cuda.synchronize()
    ref = _adamw_chain(params[U], [g], HP)
    np.testing.assert_allclose(model.get_params(U), ref, rtol=0, atol=3e-8 + 1e-6 * np.abs(ref - params[U]).max())
